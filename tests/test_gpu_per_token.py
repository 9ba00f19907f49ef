"""GPU parity of per-token dynamic activation scales against the CPU oracle.

Each token row of x is calibrated on its own amax (g_t = amax_t / 2688) and
quantized with 1 / g_t; the gate_up GEMM then scales token t's row by
fl(g_w * g_t). Quantize results (codes, scale bytes, g_t) are bit-exact;
GEMM/MLP outputs meet the fp32 tolerance; the fused re-quantized h meets the
one-step tie rule against the pure oracle.
"""
import numpy as np
import pytest
import torch

import nvfp4_synth as synth
import oracle
from gpu_helpers import (gemm_close, mlp_weights, packed_weights, requant_check, scalar, to_dev,
                         to_host)

pytestmark = pytest.mark.gpu

nv = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global nv
    import nvfp4_quantized_dense_amd as _nv
    nv = _nv
    nv.lib()
    assert torch.cuda.is_available()
    yield
    nv.set_path(nv.PATH_AUTO)


PATHS = {"gemv": 1, "stream": 2, "tiled": 3, "tiled64": 4, "mid": 5}


@pytest.fixture(params=list(PATHS))
def path(request):
    prev = nv.set_path(PATHS[request.param])
    yield request.param
    nv.set_path(prev)


def skewed_tokens(seed, M, H, outliers=False):
    """bf16 activations whose rows differ in magnitude by orders of ten (the
    case per-token scales are for): N(0,1) rows times exp(2 N(0,1))."""
    x = synth.bf16_bits_to_f32(synth.activations(seed, M, H, outliers=outliers))
    mult = np.exp(2.0 * np.random.default_rng(seed + 17).standard_normal((M, 1))).astype(np.float32)
    return synth.f32_to_bf16_bits(x * mult)


def _edge_rows(K, rng):
    """A zero row, a row of -0 and 0, a saturating row, a tiny row, a row of
    E2M1 ties, and a row whose g is a subnormal float (amax 1.5e-35)."""
    tie = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, 6, -0.25, -2.5, 0.5, 1, 1.5, 2, 3, 4],
                   np.float32)
    z = np.zeros(K, np.float32)
    z[::16] = -0.0
    sub = (rng.standard_normal(K) * 1e-36).astype(np.float32)
    sub[0] = 1.5e-35
    sub = np.clip(sub, -1.5e-35, 1.5e-35)
    return np.stack([np.zeros(K, np.float32), z,
                     np.full(K, 3.0e4, np.float32) * np.sign(rng.standard_normal(K)).astype(np.float32),
                     (rng.standard_normal(K) * 1e-30).astype(np.float32),
                     np.tile(tie, K // 16), sub])


@pytest.mark.parametrize("M,K", [(1, 16), (3, 256), (64, 5120), (257, 7168), (5, 18432)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_per_token_bit_exact(M, K, dtype):
    rng = np.random.default_rng(M * 11 + K)
    x = (rng.standard_normal((M, K)) * np.exp(3 * rng.standard_normal((M, 1)))).astype(np.float32)
    x = np.concatenate([x, _edge_rows(K, rng)])
    xo = synth.f32_to_bf16_bits(x) if dtype == "bf16" else x
    c, s, g = nv.nvfp4_quantize_per_token(to_dev(xo))
    oc, os_, og = oracle.quantize_per_token(xo)
    assert np.array_equal(to_host(g).view(np.uint32), og.view(np.uint32)), "row g differs"
    assert np.array_equal(to_host(s), os_), "scales differ"
    assert np.array_equal(to_host(c), oc), "codes differ"
    assert np.all(to_host(g)[M:M + 2] == 0) and not np.any(to_host(c)[M:M + 2] & 0x77)


def _rowscale_case(M, K, seed):
    x = skewed_tokens(seed, M, K)
    if M > 2:
        x[M // 2] = 0  # a zero token: g = 0, its output row must be exactly zero
    return oracle.quantize_per_token(x)


@pytest.mark.parametrize("M", [1, 2, 3, 5, 16, 17, 40, 64, 130])
def test_gemm_rowscale(path, M):
    rng = np.random.default_rng(300 + M)
    N, K = 272, 768
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    ws = rng.integers(0x28, 0x48, (N, K // 16), dtype=np.uint8)
    p = nv.nvfp4_repack_weight(0, to_dev(wc), to_dev(ws))
    g_w = np.float32(0.0173)
    ac, as_, g = _rowscale_case(M, K, M)
    alpha_rows = np.array([oracle.alpha(gt, g_w) for gt in g], np.float32)
    ref = oracle.gemm_w4a4_rows(ac, as_, wc, ws, alpha_rows)
    y = nv.nvfp4_gemm_rowscale(to_dev(ac), to_dev(as_), to_dev(g), p, N, K, scalar(g_w))
    yh = to_host(y)
    gemm_close(yh, ref, f"{path} rowscale M={M}")
    if M > 2:
        assert np.all(yh[M // 2] == 0)
    # the per-token scale is applied per row: each row within tolerance of its own reference
    for t in range(M):
        if g[t] != 0:
            gemm_close(yh[t:t + 1], ref[t:t + 1], f"{path} rowscale M={M} row {t}")
    yb = nv.nvfp4_gemm_rowscale(to_dev(ac), to_dev(as_), to_dev(g), p, N, K, scalar(g_w),
                                out_dtype=torch.bfloat16)
    assert np.array_equal(to_host(yb), synth.f32_to_bf16_bits(yh))


@pytest.mark.parametrize("M", [1, 3, 16, 40, 129])
def test_swiglu_rowscale_requant(path, M):
    H, I = 512, 256
    w = mlp_weights(H, I, 1)
    p_gu, _ = packed_weights(H, I, 1)
    xq, xs, g = _rowscale_case(M, H, 40 + M)
    alpha_rows = np.array([oracle.alpha(gt, w["g_gu"]) for gt in g], np.float32)
    h_ref = oracle.swiglu(oracle.gemm_w4a4_rows(xq, xs, w["c_gu"], w["s_gu"], alpha_rows))
    _, g2_inv = oracle.global_scale(h_ref)
    hc, hs = nv.gemm_swiglu_nvfp4_quant_rowscale(to_dev(xq), to_dev(xs), to_dev(g), p_gu, I, H,
                                                 scalar(w["g_gu"]), scalar(g2_inv))
    requant_check(to_host(hc), to_host(hs), h_ref, g2_inv)


def _g2_for(x, w):
    """h's static global scale as a calibration pass over x would set it."""
    xq, xs, g = oracle.quantize_per_token(x)
    alpha_rows = np.array([oracle.alpha(gt, w["g_gu"]) for gt in g], np.float32)
    h = oracle.swiglu(oracle.gemm_w4a4_rows(xq, xs, w["c_gu"], w["s_gu"], alpha_rows))
    g2, g2_inv = oracle.global_scale(h)
    return g2_inv, oracle.alpha(g2, w["g_d"])


def _check_mlp_per_token(M, H, I, seed=0, rows=None, outliers=False, calib_rows=64):
    w = mlp_weights(H, I, 0)
    p_gu, p_d = packed_weights(H, I, 0)
    x = skewed_tokens(seed, M, H, outliers=outliers)
    g2_inv, a_d = _g2_for(x[:min(M, calib_rows)], w)
    y = to_host(nv.mlp_forward(nv.MODE_W4A4_DYN, to_dev(x), p_gu, scalar(w["g_gu"]), p_d, scalar(a_d), I,
                               g2_inv=scalar(g2_inv)))
    sel = np.arange(M) if rows is None else rows
    r = oracle.mlp_w4a4_per_token(x[sel], w["c_gu"], w["s_gu"], w["g_gu"], w["c_d"], w["s_d"], a_d, g2_inv)
    gemm_close(y[sel], r["out"], f"mlp per-token M={M} H={H} I={I}")
    return y


def test_mlp_per_token_tiny(path):
    _check_mlp_per_token(4, 256, 512)


@pytest.mark.parametrize("M", [1, 7, 64, 200])
def test_mlp_per_token_auto(M):
    nv.set_path(nv.PATH_AUTO)
    _check_mlp_per_token(M, 512, 768, seed=M)


@pytest.mark.parametrize("M,H,I", [(64, 2048, 6400), (300, 7168, 4096)])
def test_mlp_per_token_split_down(M, H, I):
    """The per-token scales through the K-split down projection of the
    mid-size kernels: 64-token tiles split 3 ways (64 tokens), 128-token
    tiles split 2 ways (300 tokens, hidden 7168; 48 sampled rows)."""
    nv.set_path(nv.PATH_AUTO)
    rows = None if M <= 64 else np.unique(np.concatenate([np.arange(16), np.arange(M - 16, M),
                                                           np.random.default_rng(M).choice(M, 16, replace=False)]))
    _check_mlp_per_token(M, H, I, seed=M + 1, rows=rows, calib_rows=16)


@pytest.mark.parametrize("M", [1, 16])
def test_mlp_per_token_decode_full_size(M):
    """Hidden 5120, intermediate 17408 (with outliers), through the GEMV path."""
    nv.set_path(nv.PATH_AUTO)
    _check_mlp_per_token(M, 5120, 17408, seed=5 + M, outliers=True)


def test_mlp_per_token_prefill_full_size_sampled_rows():
    """M=8192, hidden 7168, intermediate 18432 on the GPU; 32 seeded rows by the oracle."""
    nv.set_path(nv.PATH_AUTO)
    rows = np.sort(np.random.default_rng(8193).choice(8192, 32, replace=False))
    _check_mlp_per_token(8192, 7168, 18432, rows=rows, calib_rows=16)


def test_mlp_per_token_matches_static_for_one_token():
    """At one token the per-token scale is the static scale calibrated on
    that token, so both modes give the same output bit for bit (the
    two-launch W4A4 path; the per-token mode never takes the single launch)."""
    H, I = 1024, 2304
    w = mlp_weights(H, I, 0)
    p_gu, p_d = packed_weights(H, I, 0)
    x = skewed_tokens(3, 1, H)
    g2_inv, a_d = _g2_for(x, w)
    g1, g1_inv = oracle.global_scale(x)
    prev = nv.set_path(nv.PATH_GEMV)
    try:
        yd = nv.mlp_forward(nv.MODE_W4A4_DYN, to_dev(x), p_gu, scalar(w["g_gu"]), p_d, scalar(a_d), I,
                            g2_inv=scalar(g2_inv))
        ys = nv.mlp_forward(nv.MODE_W4A4, to_dev(x), p_gu, scalar(oracle.alpha(g1, w["g_gu"])), p_d,
                            scalar(a_d), I, g1_inv=scalar(g1_inv), g2_inv=scalar(g2_inv))
        assert np.array_equal(to_host(yd), to_host(ys))
    finally:
        nv.set_path(prev)
