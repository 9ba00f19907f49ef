"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bit-exact where the result is integer/byte work (quantize codes and scale
bytes, calibration, repack); within the fp32 tolerance for GEMM/MLP outputs;
the one-step tie rule for re-quantized codes against the pure oracle, and
bit-exact against the oracle's quantization of the kernel's own fp32 h.
"""
import numpy as np
import pytest
import torch

import nvfp4_synth as synth
import oracle
from gpu_helpers import (calibrate_activation_scales, dev, gemm_close, mlp_weights, packed_weights,
                         requant_check, scalar, to_dev, to_host)

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


# "tiled64" forces the 64-bit-addressed tiled kernel, which the other paths
# run only for operands of 2^31 bytes or more.
PATHS = {"gemv": 1, "stream": 2, "tiled": 3, "tiled64": 4, "mid": 5}


@pytest.fixture(params=list(PATHS))
def path(request):
    prev = nv.set_path(PATHS[request.param])
    yield request.param
    nv.set_path(prev)


def rand_nvfp4(rng, R, K, lo=0x28, hi=0x48):
    return (rng.integers(0, 256, (R, K // 2), dtype=np.uint8),
            rng.integers(lo, hi, (R, K // 16), dtype=np.uint8))


# -- quantize / calibrate / repack (bit-exact) -------------------------------

def _edge_rows(K, rng):
    """Rows that hit ties, saturation, subnormal scales, zero blocks, -0."""
    rows = []
    tie = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, 6, -0.25, -2.5, 0.5, 1, 1.5, 2, 3, 4],
                   np.float32)
    rows.append(np.tile(tie, K // 16))
    rows.append(np.zeros(K, np.float32))
    z = np.zeros(K, np.float32); z[::16] = -0.0; z[1::16] = -1e-38
    rows.append(z)
    rows.append(np.full(K, 3.0e4, np.float32) * np.sign(rng.standard_normal(K)).astype(np.float32))
    rows.append((rng.standard_normal(K) * 1e-30).astype(np.float32))
    return np.stack(rows)


@pytest.mark.parametrize("M,K", [(1, 16), (3, 256), (64, 5120), (257, 7168), (5, 18432)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_bit_exact(M, K, dtype):
    rng = np.random.default_rng(M * 7 + K)
    x = (rng.standard_normal((M, K)) * np.exp(2 * rng.standard_normal((M, 1)))).astype(np.float32)
    x = np.concatenate([x, _edge_rows(K, rng)])
    xb = synth.f32_to_bf16_bits(x)
    for gi in [np.float32(1.0), np.float32(0.37), np.float32(2.0e3)]:
        if dtype == "bf16":
            xin, xo = to_dev(xb), xb
        else:
            xin, xo = to_dev(x), x
        c, s = nv.nvfp4_quantize(xin, scalar(gi))
        oc, os_ = oracle.quantize(xo, gi)
        assert np.array_equal(to_host(s), os_), f"scales differ (g_inv={gi})"
        assert np.array_equal(to_host(c), oc), f"codes differ (g_inv={gi})"


def test_quantize_exhaustive_bf16_slot():
    """Every finite bf16 value beside a block max of 6 (s = 1, r = 1)."""
    vals = synth.bf16_bits_to_f32(np.arange(65536, dtype=np.uint16))
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 6)]
    x = np.zeros((vals.size, 16), np.float32)
    x[:, 0] = 6.0
    x[:, 5] = vals
    xb = synth.f32_to_bf16_bits(x)
    c, s = nv.nvfp4_quantize(to_dev(xb), scalar(1.0))
    oc, os_ = oracle.quantize(xb, np.float32(1.0))
    assert np.array_equal(to_host(c), oc) and np.array_equal(to_host(s), os_)


def _e4m3_grid():
    """The 127 finite non-negative E4M3 values (bytes 0x00..0x7E), from the
    format's definition: subnormals m/8 * 2^-6, normals (1 + m/8) * 2^(e-7)."""
    b = np.arange(0x7F)
    e, m = b >> 3, b & 7
    return np.where(e == 0, m / 8 * 2.0 ** -6, (1 + m / 8) * 2.0 ** (e - 7))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_e4m3_scale_sweep(dtype):
    """The block-scale encoder at every E4M3 value, every midpoint between
    neighbours (ties to the even mantissa), one fp32 ulp either side of each,
    the saturation edge above 448, the underflow range below the smallest
    subnormal, and 200k log-uniform scales: with g_inv = 1 a block whose max
    is fl(6 sv) gives exactly sv before rounding. The other 15 elements are
    uniform below the max, so the element encoder runs under every scale."""
    rng = np.random.default_rng(23)
    v = _e4m3_grid()
    mid = (v[:-1] + v[1:]) / 2
    sat = np.array([448.0, 456.0, 464.0, 472.0, 480.0, 1e4])
    base = np.concatenate([v, mid, sat]).astype(np.float32)
    sv = np.concatenate([base, np.nextafter(base, np.float32(np.inf)),
                         np.nextafter(base, np.float32(0)),
                         np.exp2(rng.uniform(-13, 10, 200_000)).astype(np.float32)])
    sv = sv[sv > 0]
    amax = sv * np.float32(6)
    n = amax.size
    x = (rng.uniform(-1, 1, (n, 16)) * amax[:, None].astype(np.float64)).astype(np.float32)
    x[np.arange(n), rng.integers(0, 16, n)] = amax * rng.choice(np.float32([-1, 1]), n)
    if dtype == "bf16":
        xo = synth.f32_to_bf16_bits(x)
    else:
        xo = x
    for gi in [np.float32(1.0), np.float32(0.37), np.float32(2.0e3)]:
        c, s = nv.nvfp4_quantize(to_dev(xo), scalar(gi))
        oc, os_ = oracle.quantize(xo, gi)
        assert np.array_equal(to_host(s), os_), f"scale bytes differ (g_inv={gi})"
        assert np.array_equal(to_host(c), oc), f"codes differ (g_inv={gi})"


@pytest.mark.parametrize("n,dtype", [(1, "bf16"), (4097, "bf16"), (1 << 20, "f32")])
def test_calibrate_bit_exact(n, dtype):
    rng = np.random.default_rng(n)
    x = (rng.standard_normal(n) * 3).astype(np.float32)
    xo = synth.f32_to_bf16_bits(x) if dtype == "bf16" else x
    g, gi = nv.nvfp4_calibrate(to_dev(xo))
    og, ogi = oracle.global_scale(xo)
    assert to_host(g)[0] == og and to_host(gi)[0] == ogi


def test_calibrate_golden_non_power_of_two():
    """g and g_inv at the hand-worked amax values (tests/golden), on the GPU."""
    from golden_fixtures import global_scale_examples
    for amax, g_ref, gi_ref, _ in global_scale_examples():
        x = np.array([0.25, -amax, 1.0, 2.0], np.float32)
        for xo in (x, synth.f32_to_bf16_bits(x)):
            g, gi = nv.nvfp4_calibrate(to_dev(xo))
            assert to_host(g)[0] == g_ref and to_host(gi)[0] == gi_ref, amax


@pytest.mark.parametrize("kind,R,C", [(0, 16, 256), (0, 5120, 512), (1, 32, 256), (1, 1024, 768)])
def test_repack_round_trip(kind, R, C):
    rng = np.random.default_rng(R + C)
    c, s = rand_nvfp4(rng, R, C, 0, 256)
    p = nv.nvfp4_repack_weight(kind, to_dev(c), to_dev(s))
    assert p.numel() == R * C * 9 // 16
    c2, s2 = nv.nvfp4_unpack_weight(kind, p, R, C)
    assert np.array_equal(to_host(c2), c) and np.array_equal(to_host(s2), s)
    # the packed buffer is a permutation of the input bytes
    assert np.array_equal(np.sort(to_host(p)), np.sort(np.concatenate([c.ravel(), s.ravel()])))


# -- GEMM ---------------------------------------------------------------------

@pytest.mark.parametrize("M", [1, 2, 3, 5, 16, 17, 40, 64, 130])
@pytest.mark.parametrize("mode", ["w4a4", "w4a16"])
def test_gemm_matches_oracle(path, M, mode):
    rng = np.random.default_rng(M)
    N, K = 272, 768  # 17 row groups, 3 K tiles: ragged against every tile shape
    wc, ws = rand_nvfp4(rng, N, K)
    p = nv.nvfp4_repack_weight(0, to_dev(wc), to_dev(ws))
    alpha = np.float32(0.0173)
    if mode == "w4a4":
        ac, as_ = rand_nvfp4(rng, M, K)
        ref = oracle.gemm_w4a4(ac, as_, wc, ws, alpha)
        y = nv.nvfp4_gemm(0, to_dev(ac), to_dev(as_), p, N, K, scalar(alpha))
    else:
        x = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
        ref = oracle.gemm_w4a16(x, wc, ws, alpha)
        y = nv.nvfp4_gemm(1, to_dev(x), None, p, N, K, scalar(alpha))
    gemm_close(to_host(y), ref, f"{path} {mode} M={M}")
    yb = nv.nvfp4_gemm(0 if mode == "w4a4" else 1, to_dev(ac if mode == "w4a4" else x),
                       to_dev(as_) if mode == "w4a4" else None, p, N, K, scalar(alpha),
                       out_dtype=torch.bfloat16)
    assert np.array_equal(to_host(yb), synth.f32_to_bf16_bits(to_host(y)))


def _full_range_scales(rng, R, K, which):
    """Scale bytes over the finite E4M3 range: 'all' draws 0x00..0x7E
    uniformly (zero, the subnormals 0x01..0x07 and the saturated 0x7E among
    them); 'low' keeps to 0x00..0x0F (zero, subnormals, the smallest
    normals); 'high' to 0x70..0x7E. Each kind also holds its edge bytes."""
    lo, hi, edge = {"all": (0, 0x7F, [0x00, 0x01, 0x07, 0x08, 0x7E]),
                    "low": (0, 0x10, [0x00, 0x01, 0x07, 0x0F]),
                    "high": (0x70, 0x7F, [0x70, 0x7E])}[which]
    s = rng.integers(lo, hi, (R, K // 16), dtype=np.uint8)
    s.flat[:len(edge)] = edge
    return s


@pytest.mark.parametrize("M", [1, 2, 5, 17, 130])
@pytest.mark.parametrize("mode", ["w4a4", "w4a16"])
def test_gemm_full_scale_byte_range(path, M, mode):
    """Scale bytes over 0x00..0x7E on both operands: uniform over the range,
    and low weight scales (subnormal) against high activation scales and the
    reverse, so that blocks with subnormal scales carry as much of the sum as
    any other."""
    rng = np.random.default_rng(900 + M)
    N, K = 272, 768
    for wk, ak in [("all", "all"), ("low", "high"), ("high", "low")]:
        wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
        ws = _full_range_scales(rng, N, K, wk)
        p = nv.nvfp4_repack_weight(0, to_dev(wc), to_dev(ws))
        alpha = np.float32(0.0173)
        if mode == "w4a4":
            ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
            as_ = _full_range_scales(rng, M, K, ak)
            ref = oracle.gemm_w4a4(ac, as_, wc, ws, alpha)
            y = nv.nvfp4_gemm(0, to_dev(ac), to_dev(as_), p, N, K, scalar(alpha))
        else:
            x = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
            ref = oracle.gemm_w4a16(x, wc, ws, alpha)
            y = nv.nvfp4_gemm(1, to_dev(x), None, p, N, K, scalar(alpha))
        gemm_close(to_host(y), ref, f"{path} {mode} M={M} scales w={wk} a={ak}")


@pytest.mark.parametrize("M", [1, 4, 33])
def test_gemm_power_of_two_scales_bit_exact(path, M):
    """All partial sums exactly representable: every path must be bit-exact."""
    rng = np.random.default_rng(100 + M)
    N, K = 64, 1024
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    pw = np.array([0x30, 0x38, 0x40], np.uint8)
    as_, ws = rng.choice(pw, (M, K // 16)), rng.choice(pw, (N, K // 16))
    p = nv.nvfp4_repack_weight(0, to_dev(wc), to_dev(ws))
    y = nv.nvfp4_gemm(0, to_dev(ac), to_dev(as_), p, N, K, scalar(0.25))
    assert np.array_equal(to_host(y), oracle.gemm_w4a4(ac, as_, wc, ws, np.float32(0.25)))
    # W4A16 with bf16 activations that are small multiples of powers of two
    x = synth.f32_to_bf16_bits((rng.integers(-8, 9, (M, K)) * 0.25).astype(np.float32))
    y = nv.nvfp4_gemm(1, to_dev(x), None, p, N, K, scalar(0.5))
    assert np.array_equal(to_host(y), oracle.gemm_w4a16(x, wc, ws, np.float32(0.5)))


def test_gemm_deterministic_and_guarded(path):
    rng = np.random.default_rng(5)
    M, N, K = 37, 128, 512
    wc, ws = rand_nvfp4(rng, N, K)
    ac, as_ = rand_nvfp4(rng, M, K)
    p = nv.nvfp4_repack_weight(0, to_dev(wc), to_dev(ws))
    guard = torch.full((M * N + 64,), 12345.0, dtype=torch.float32, device=dev())
    out = guard[16:16 + M * N].view(M, N)
    nv.nvfp4_gemm(0, to_dev(ac), to_dev(as_), p, N, K, scalar(1.0), out=out)
    y1 = to_host(out).copy()
    nv.nvfp4_gemm(0, to_dev(ac), to_dev(as_), p, N, K, scalar(1.0), out=out)
    assert np.array_equal(y1, to_host(out))
    g = to_host(guard)
    assert np.all(g[:16] == 12345.0) and np.all(g[16 + M * N:] == 12345.0)


# -- W4A16 prefill kernel: 128-row x 256-token workgroup tiles ------------------
#
# Several token tiles (ragged past 256 and 512), a last row tile that is
# partly past N (21 row groups = 2 full tiles of 8 and one of 5; for SwiGLU
# 42 groups = 5 full tiles and one of 2), 5 K tiles (10 staged halves).

@pytest.mark.parametrize("M", [256, 257, 600])
def test_w4a16_prefill_tiles(M):
    prev = nv.set_path(PATHS["tiled"])
    try:
        rng = np.random.default_rng(700 + M)
        N, K = 16 * 21, 1280
        wc, ws = rand_nvfp4(rng, N, K)
        p = nv.nvfp4_repack_weight(0, to_dev(wc), to_dev(ws))
        x = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
        alpha = np.float32(0.031)
        y = nv.nvfp4_gemm(1, to_dev(x), None, p, N, K, scalar(alpha))
        gemm_close(to_host(y), oracle.gemm_w4a16(x, wc, ws, alpha), f"w4a16 prefill gemm M={M}")
        yb = nv.nvfp4_gemm(1, to_dev(x), None, p, N, K, scalar(alpha), out_dtype=torch.bfloat16)
        assert np.array_equal(to_host(yb), synth.f32_to_bf16_bits(to_host(y)))
        H, I = 768, 336
        w = mlp_weights(H, I, 2)
        p_gu = nv.nvfp4_repack_weight(nv.REPACK_SWIGLU, to_dev(w["c_gu"]), to_dev(w["s_gu"]))
        xh = synth.activations(M, M, H)
        a_gu = np.float32(w["g_gu"])
        h32 = nv.gemm_swiglu(1, to_dev(xh), None, p_gu, I, H, scalar(a_gu), h_dtype=torch.float32)
        h_ref = oracle.swiglu(oracle.gemm_w4a16(xh, w["c_gu"], w["s_gu"], a_gu))
        gemm_close(to_host(h32), h_ref, f"w4a16 prefill swiglu M={M}")
        hb = nv.gemm_swiglu(1, to_dev(xh), None, p_gu, I, H, scalar(a_gu), h_dtype=torch.bfloat16)
        assert np.array_equal(to_host(hb), synth.f32_to_bf16_bits(to_host(h32)))
    finally:
        nv.set_path(prev)


# -- fused gate_up + SwiGLU (+ NVFP4) ------------------------------------------

@pytest.mark.parametrize("M", [1, 3, 16, 24, 40, 129])
def test_swiglu_fused_requant(path, M):
    H, I = 512, 256
    w = mlp_weights(H, I, 1)
    p_gu, _ = packed_weights(H, I, 1)
    x = synth.activations(3, M, H)
    sc = calibrate_activation_scales(x, w)
    xq, xs = oracle.quantize(x, sc["g1_inv"])
    dxq, dxs = to_dev(xq), to_dev(xs)
    # dense h in f32 against the oracle
    h32 = nv.gemm_swiglu(0, dxq, dxs, p_gu, I, H, scalar(sc["a_gu"]), h_dtype=torch.float32)
    gu = oracle.gemm_w4a4(xq, xs, w["c_gu"], w["s_gu"], sc["a_gu"])
    h_ref = oracle.swiglu(gu)
    gemm_close(to_host(h32), h_ref, f"{path} h M={M}")
    # fused NVFP4: bit-exact against the oracle's quantization of the kernel's h
    hc, hs = nv.gemm_swiglu_nvfp4_quant(dxq, dxs, p_gu, I, H, scalar(sc["a_gu"]), scalar(sc["g2_inv"]))
    oc, os_ = oracle.quantize(to_host(h32), sc["g2_inv"])
    assert np.array_equal(to_host(hs), os_) and np.array_equal(to_host(hc), oc)
    # and within the tie rule against the pure oracle
    requant_check(to_host(hc), to_host(hs), h_ref, sc["g2_inv"])
    # bf16 h (W4A16 chain epilogue) is the rounding of the f32 one
    hb = nv.gemm_swiglu(0, dxq, dxs, p_gu, I, H, scalar(sc["a_gu"]), h_dtype=torch.bfloat16)
    assert np.array_equal(to_host(hb), synth.f32_to_bf16_bits(to_host(h32)))


# -- MLP ------------------------------------------------------------------------

def _run_mlp(mode, x, w, sc, p_gu, p_d):
    if mode == "w4a4":
        return nv.mlp_forward(0, to_dev(x), p_gu, scalar(sc["a_gu"]), p_d, scalar(sc["a_d"]), w["I"],
                              g1_inv=scalar(sc["g1_inv"]), g2_inv=scalar(sc["g2_inv"]))
    return nv.mlp_forward(1, to_dev(x), p_gu, scalar(w["g_gu"]), p_d, scalar(w["g_d"]), w["I"])


def _check_mlp(mode, M, H, I, seed=0, outliers=False, rows=None):
    w = mlp_weights(H, I, 0)
    p_gu, p_d = packed_weights(H, I, 0)
    x = synth.activations(seed, M, H, outliers=outliers)
    sc = calibrate_activation_scales(x[:min(M, 64)], w) if mode == "w4a4" else None
    y = to_host(_run_mlp(mode, x, w, sc, p_gu, p_d))
    torch.cuda.synchronize()
    sel = np.arange(M) if rows is None else rows
    xs_ = x[sel]
    if mode == "w4a4":
        r = oracle.mlp_w4a4(xs_, w["c_gu"], w["s_gu"], sc["a_gu"], w["c_d"], w["s_d"], sc["a_d"],
                            sc["g1_inv"], sc["g2_inv"])
    else:
        r = oracle.mlp_w4a16(xs_, w["c_gu"], w["s_gu"], w["g_gu"], w["c_d"], w["s_d"], w["g_d"])
    gemm_close(y[sel], r["out"], f"mlp {mode} M={M} H={H} I={I}")
    return y


@pytest.mark.parametrize("mode", ["w4a4", "w4a16"])
def test_mlp_tiny_workload(path, mode):
    """M=4, hidden 256, intermediate 512, seed 0 (the tiny NVFP4 MLP)."""
    _check_mlp(mode, 4, 256, 512)


@pytest.mark.parametrize("M", [1, 7, 24, 32, 33, 48, 56, 63, 64, 96, 97, 100, 128, 129, 144, 192, 193, 200, 512,
                               513])
def test_mlp_auto_dispatch(M):
    """Token counts on both sides of each automatic switch: W4A4 streams up
    to 128 tokens, W4A16 up to 32 (SwiGLU) and 96 (dense), the gate_up from
    33 tokens on the mid-size kernel (48-token tiles up to 48 tokens,
    64-token tiles above; W4A16 up to 64 tokens, W4A4 up to 512); the tiled
    kernels take over above. (At hidden 512, intermediate 768 the down
    projection has too few K tiles to split, so the split mid-size down
    projection is covered by test_mlp_auto_split_down.)"""
    nv.set_path(nv.PATH_AUTO)
    _check_mlp("w4a4", M, 512, 768, seed=M)
    _check_mlp("w4a16", M, 512, 768, seed=M)


# Shapes where the automatic path takes the workspace-split down projection
# of the mid-size kernel (W4A4 from 17 tokens, W4A16 from 65 to 192, where
# hidden / 128 x token tiles <= 256 and K splits into parts of at least 8 K
# tiles: intermediate 6400 gives 3 splits of 9, 9 and 7 K tiles, 4096 two
# of 8), and where the W4A16 down projection streams through 5 or 7 row
# groups per workgroup (hidden 5120 / 7168 at 49-64 tokens: 4 groups would
# overfill one round of workgroups).
@pytest.mark.parametrize("mode,M,H,I", [("w4a4", 17, 2048, 6400), ("w4a4", 48, 2048, 6400),
                                        ("w4a4", 100, 2048, 6400), ("w4a4", 200, 1024, 6400),
                                        ("w4a4", 256, 1024, 4096), ("w4a4", 300, 1024, 4096),
                                        ("w4a4", 400, 2048, 6400), ("w4a4", 300, 7168, 4096),
                                        ("w4a16", 80, 1024, 4096),
                                        ("w4a16", 150, 1024, 6400), ("w4a16", 56, 5120, 512),
                                        ("w4a16", 64, 7168, 512)])
def test_mlp_auto_split_down(mode, M, H, I):
    """(At hidden 7168 and 300 tokens the 64-token grid of the W4A4 down
    projection has 280 tiles, so it takes 128-token tiles, split 2 ways;
    above 256 tokens the oracle checks 48 sampled rows, the ragged last
    tile among them.)"""
    nv.set_path(nv.PATH_AUTO)
    rows = None if M <= 256 else np.unique(np.concatenate([np.arange(16), np.arange(M - 16, M),
                                                           np.random.default_rng(M).choice(M, 16, replace=False)]))
    _check_mlp(mode, M, H, I, seed=M + H, rows=rows)


def test_gemm_w4a4_mid_128_token_tiles():
    """A one-expert dense W4A4 GEMM under NVFP4_PATH_MID whose 64-token grid
    would exceed 256 tiles (7168 rows, 300 tokens) runs the 128-token
    kernel, unsplit (the standalone entry has no workspace)."""
    prev = nv.set_path(PATHS["mid"])
    try:
        rng = np.random.default_rng(300)
        M, N, K = 300, 7168, 512
        wc, ws = rand_nvfp4(rng, N, K)
        p = nv.nvfp4_repack_weight(0, to_dev(wc), to_dev(ws))
        alpha = np.float32(0.0173)
        ac, as_ = rand_nvfp4(rng, M, K)
        y = nv.nvfp4_gemm(0, to_dev(ac), to_dev(as_), p, N, K, scalar(alpha))
        gemm_close(to_host(y), oracle.gemm_w4a4(ac, as_, wc, ws, alpha), "mid 128-token tiles")
    finally:
        nv.set_path(prev)


@pytest.mark.parametrize("N,M", [(5120, 56), (5120, 80), (7168, 40), (7168, 64)])
def test_gemm_w4a16_one_round_groups(N, M):
    """W4A16 dense GEMMs whose streaming grid takes 5, 8, 7 and 7 row groups
    per workgroup (one round of at most 256 workgroups)."""
    nv.set_path(nv.PATH_AUTO)
    rng = np.random.default_rng(N + M)
    K = 512
    wc, ws = rand_nvfp4(rng, N, K)
    p = nv.nvfp4_repack_weight(0, to_dev(wc), to_dev(ws))
    alpha = np.float32(0.0173)
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    y = nv.nvfp4_gemm(1, to_dev(x), None, p, N, K, scalar(alpha))
    gemm_close(to_host(y), oracle.gemm_w4a16(x, wc, ws, alpha), f"w4a16 one-round N={N} M={M}")


def test_mlp_decode_full_size():
    """Decode W4A4: M=1, hidden 5120, intermediate 17408, outliers; every 50th
    of the 1000 seeded inputs the decode benchmark cycles through, and the
    last (the static g1 and g2 stay those calibrated on seed 0)."""
    nv.set_path(nv.PATH_AUTO)
    H, I = 5120, 17408
    w = mlp_weights(H, I, 0)
    p_gu, p_d = packed_weights(H, I, 0)
    sc = calibrate_activation_scales(synth.activations(0, 1, H, outliers=True), w)
    ws = torch.zeros(nv.mlp_workspace_bytes(0, 1, H, I), dtype=torch.uint8, device=dev())
    n_diff = 0
    for seed in list(range(0, 1000, 50)) + [1, 999]:
        x = synth.activations(seed, 1, H, outliers=True)
        y = to_host(nv.mlp_forward(0, to_dev(x), p_gu, scalar(sc["a_gu"]), p_d, scalar(sc["a_d"]), I,
                                   g1_inv=scalar(sc["g1_inv"]), g2_inv=scalar(sc["g2_inv"]), ws=ws))
        torch.cuda.synchronize()
        r = oracle.mlp_w4a4(x, w["c_gu"], w["s_gu"], sc["a_gu"], w["c_d"], w["s_d"], sc["a_d"],
                            sc["g1_inv"], sc["g2_inv"])
        gemm_close(y, r["out"], f"decode W4A4 seed {seed}")
        # the single launch's NVFP4 h (left in the workspace) against the
        # pure oracle's pre-quant h, under the tie rule
        hc, hs = _ws_h(ws, H, I)
        n_diff += requant_check(hc.reshape(1, I // 2), hs.reshape(1, I // 16), r["h"], sc["g2_inv"])[0]
    print(f"decode h: {n_diff} re-quantized elements differ over 22 inputs")
    assert to_host(nv.mlp_workspace_status(ws))[0] == 0


@pytest.mark.parametrize("M", [1, 4, 16, 64, 128, 300])
def test_mlp_small_batch_full_size(M):
    """Fused W4A4 MLP, hidden 7168, intermediate 18432."""
    nv.set_path(nv.PATH_AUTO)
    _check_mlp("w4a4", M, 7168, 18432, rows=np.arange(min(M, 16)))


# -- mlp_forward workspace use: split-K of the down projection (weight-
# streaming, mid-size and W4A16 tiled kernels) and the decode GEMV's
# in-kernel activation quantization
#
# Hidden 512 leaves 32 output row groups, so the streaming kernel splits
# the down projection's K (intermediate) over several workgroups: 27 tiles
# (6912) split unevenly, 32 tiles (8192) evenly. At 200 tokens the W4A16
# tiled kernel has 4 output tiles and splits K 7 ways (6912) or 8 (8192). The workspace starts as
# 0xFF bytes (the counters must be cleared by the gate_up launch) and is
# reused by a call on another input and then on the first input again,
# which must give bit-identical output (counts reset, no stale partials).
# The GEMV cases run the W4A4 gate_up with the quantization of x fused.

@pytest.mark.parametrize("I", [6912, 8192])
@pytest.mark.parametrize("kpath,M,H", [("gemv", 1, 512), ("gemv", 2, 512), ("stream", 3, 512), ("stream", 16, 512),
                                       ("stream", 40, 512), ("tiled", 200, 512), ("mid", 64, 512),
                                       ("mid", 100, 512), ("mid", 64, 2048), ("mid", 200, 2048),
                                       ("mid", 300, 512)])
@pytest.mark.parametrize("mode", ["w4a4", "w4a16"])
def test_mlp_split_k(mode, kpath, M, H, I):
    """(The mid-size kernels split K for the dense down projection only: 3
    or 4 ways at these shapes, unevenly at 6912, on 128-token tiles at 300
    tokens in W4A4; the gate_up runs unsplit.)"""
    prev = nv.set_path(PATHS[kpath])
    try:
        w = mlp_weights(H, I, 0)
        p_gu, p_d = packed_weights(H, I, 0)
        x = synth.activations(M + I, M, H)
        xd = to_dev(x)
        nws = nv.mlp_workspace_bytes(0 if mode == "w4a4" else 1, M, H, I)
        ws = torch.full((nws,), 0xFF, dtype=torch.uint8, device=dev())
        if mode == "w4a4":
            sc = calibrate_activation_scales(x, w)
            args = (0, xd, p_gu, scalar(sc["a_gu"]), p_d, scalar(sc["a_d"]), I)
            kw = dict(g1_inv=scalar(sc["g1_inv"]), g2_inv=scalar(sc["g2_inv"]), ws=ws)
            r = oracle.mlp_w4a4(x, w["c_gu"], w["s_gu"], sc["a_gu"], w["c_d"], w["s_d"], sc["a_d"],
                                sc["g1_inv"], sc["g2_inv"])
        else:
            args = (1, xd, p_gu, scalar(w["g_gu"]), p_d, scalar(w["g_d"]), I)
            kw = dict(ws=ws)
            r = oracle.mlp_w4a16(x, w["c_gu"], w["s_gu"], w["g_gu"], w["c_d"], w["s_d"], w["g_d"])
        y1 = to_host(nv.mlp_forward(*args, **kw))
        # another input through the same workspace, then the first again:
        # partials or counts left from one call must not leak into the next
        xb = to_dev(synth.activations(M + I + 1, M, H))
        nv.mlp_forward(args[0], xb, *args[2:], **kw)
        y2 = to_host(nv.mlp_forward(*args, **kw))
        torch.cuda.synchronize()
        gemm_close(y1, r["out"], f"split-K mlp {mode} {kpath} M={M} I={I}")
        assert np.array_equal(y1, y2), "the same input through a reused workspace differs"
    finally:
        nv.set_path(prev)


# -- single-launch W4A4 decode (M = 1 under the automatic path) ----------------
#
# The gate_up workgroups hand h to the down workgroups, and those their
# partial sums to the last K split, as records tagged with a per-launch
# epoch; the down projection's K is split over 1 to 5 workgroups per row
# group over these shapes (ragged where the tiles do not divide). The
# workspace starts zero-filled and is reused by a launch on another input,
# so records left by an earlier launch would show. h (NVFP4, in the
# workspace) must equal the two-launch GEMV path's byte for byte: the same
# arithmetic produces it.

def _ws_h(ws, H, I, mode=0):
    """h inside an M = 1 mlp_forward workspace: W4A4 (codes, scale bytes)
    after x's NVFP4; W4A16 bf16 h [I] at the start."""
    b = to_host(ws)
    if mode == 1:
        return (b[:2 * I].copy(),)
    a256 = lambda v: (v + 255) // 256 * 256
    o = a256(H // 2) + a256(H // 16)
    return b[o:o + I // 2].copy(), b[o + a256(I // 2):o + a256(I // 2) + I // 16].copy()


def _decode_call(mode, x, w, sc, p_gu, p_d, I):
    if mode == 0:
        return (0, to_dev(x), p_gu, scalar(sc["a_gu"]), p_d, scalar(sc["a_d"]), I), \
            dict(g1_inv=scalar(sc["g1_inv"]), g2_inv=scalar(sc["g2_inv"]))
    return (1, to_dev(x), p_gu, scalar(w["g_gu"]), p_d, scalar(w["g_d"]), I), {}


def _decode_ref(mode, x, w, sc):
    if mode == 0:
        return oracle.mlp_w4a4(x, w["c_gu"], w["s_gu"], sc["a_gu"], w["c_d"], w["s_d"], sc["a_d"],
                               sc["g1_inv"], sc["g2_inv"])
    return oracle.mlp_w4a16(x, w["c_gu"], w["s_gu"], w["g_gu"], w["c_d"], w["s_d"], w["g_d"])


@pytest.mark.parametrize("H,I", [(256, 256), (256, 4096), (512, 4352), (1024, 2304), (2048, 6912),
                                 (256, 18432)])
@pytest.mark.parametrize("mode", [0, 1])
def test_mlp_decode_single_launch(mode, H, I):
    nv.set_path(nv.PATH_AUTO)
    w = mlp_weights(H, I, 0)
    p_gu, p_d = packed_weights(H, I, 0)
    x = synth.activations(H + I, 1, H)
    sc = calibrate_activation_scales(x, w) if mode == 0 else None
    args, gkw = _decode_call(mode, x, w, sc, p_gu, p_d, I)
    nws = nv.mlp_workspace_bytes(mode, 1, H, I)
    ws = torch.zeros((nws,), dtype=torch.uint8, device=dev())
    y1 = to_host(nv.mlp_forward(*args, ws=ws, **gkw))
    h1 = _ws_h(ws, H, I, mode)
    nv.mlp_forward(mode, to_dev(synth.activations(H + I + 1, 1, H)), *args[2:], ws=ws, **gkw)
    y2 = to_host(nv.mlp_forward(*args, ws=ws, **gkw))
    yb = to_host(nv.mlp_forward(*args, ws=ws, out_dtype=torch.bfloat16, **gkw))
    prev = nv.set_path(PATHS["gemv"])
    try:
        ws2 = torch.full((nws,), 0xFF, dtype=torch.uint8, device=dev())
        y3 = to_host(nv.mlp_forward(*args, ws=ws2, **gkw))
        h3 = _ws_h(ws2, H, I, mode)
    finally:
        nv.set_path(prev)
    torch.cuda.synchronize()
    r = _decode_ref(mode, x, w, sc)
    gemm_close(y1, r["out"], f"decode mode {mode} H={H} I={I}")
    gemm_close(y3, r["out"], f"two-launch decode mode {mode} H={H} I={I}")
    assert np.array_equal(y1, y2), "the same input through a reused workspace differs"
    assert np.array_equal(yb, synth.f32_to_bf16_bits(y1)), "bf16 output is not the f32 output rounded"
    for a, b in zip(h1, h3):
        assert np.array_equal(a, b), "h differs from the two-launch path"
    assert to_host(nv.mlp_workspace_status(ws))[0] == 0


def test_mlp_workspace_shared_across_token_counts():
    """One workspace sized for 16 tokens serves W4A4 at 16 tokens, W4A16 at
    16, per-token W4A4 at 16 and the single-launch W4A4 decode at 1 token,
    in turns. The decode's records lie in the workspace's tail, which no
    other call writes: the tail bytes the decode leaves are still there
    after the other calls, and every output equals a fresh workspace's."""
    nv.set_path(nv.PATH_AUTO)
    H, I = 512, 4352
    w = mlp_weights(H, I, 0)
    p_gu, p_d = packed_weights(H, I, 0)
    nws = max(nv.mlp_workspace_bytes(m, 16, H, I) for m in (0, 1, 2))
    ws = torch.zeros(nws, dtype=torch.uint8, device=dev())
    tail = 4 << 20  # the workspace tail: status word and decode records
    x16 = synth.activations(5, 16, H)
    x1 = synth.activations(6, 1, H)
    sc = calibrate_activation_scales(x16, w)
    a_gu, a_d, g1i, g2i = scalar(sc["a_gu"]), scalar(sc["a_d"]), scalar(sc["g1_inv"]), scalar(sc["g2_inv"])
    calls = {
        "w4a4 M=16": lambda ws_: nv.mlp_forward(0, to_dev(x16), p_gu, a_gu, p_d, a_d, I, g1_inv=g1i, g2_inv=g2i,
                                                ws=ws_),
        "w4a16 M=16": lambda ws_: nv.mlp_forward(1, to_dev(x16), p_gu, scalar(w["g_gu"]), p_d, scalar(w["g_d"]), I,
                                                 ws=ws_),
        "dyn M=16": lambda ws_: nv.mlp_forward(2, to_dev(x16), p_gu, scalar(w["g_gu"]), p_d, a_d, I, g2_inv=g2i,
                                               ws=ws_),
        "w4a4 M=1": lambda ws_: nv.mlp_forward(0, to_dev(x1), p_gu, a_gu, p_d, a_d, I, g1_inv=g1i, g2_inv=g2i,
                                               ws=ws_),
        "w4a16 M=1": lambda ws_: nv.mlp_forward(1, to_dev(x1), p_gu, scalar(w["g_gu"]), p_d, scalar(w["g_d"]), I,
                                                ws=ws_),
    }
    fresh = {k: to_host(f(torch.zeros(nws, dtype=torch.uint8, device=dev()))) for k, f in calls.items()}
    after_decode = None
    for rnd in range(3):
        for k, f in calls.items():
            y = to_host(f(ws))
            torch.cuda.synchronize()
            assert np.array_equal(y, fresh[k]), f"{k} in round {rnd} differs from a fresh workspace"
            t = to_host(ws)[-tail:].copy()
            if k.endswith("M=1"):
                after_decode = t
            elif after_decode is not None:
                assert np.array_equal(t, after_decode), f"{k} wrote the decode's tail"
    r = oracle.mlp_w4a4(x1, w["c_gu"], w["s_gu"], sc["a_gu"], w["c_d"], w["s_d"], sc["a_d"], sc["g1_inv"],
                        sc["g2_inv"])
    gemm_close(fresh["w4a4 M=1"], r["out"], "decode through a shared workspace")
    assert to_host(nv.mlp_workspace_status(ws))[0] == 0


@pytest.mark.parametrize("mode", [0, 1])
def test_mlp_decode_expired_wait_reports(mode):
    """The single-launch decode's bounded waits, made to give up from the
    host: the test hook has its workgroups tag their records with a number
    the waiting ones never look for and bounds each wait at 64 polls. Every
    workgroup still exits; the output is NaN and the workspace's status word
    says so. The next call without the hook is correct and leaves the status
    alone."""
    nv.set_path(nv.PATH_AUTO)
    H, I = 512, 4352
    w = mlp_weights(H, I, 0)
    p_gu, p_d = packed_weights(H, I, 0)
    x = synth.activations(9, 1, H)
    sc = calibrate_activation_scales(x, w) if mode == 0 else None
    ws = torch.zeros(nv.mlp_workspace_bytes(mode, 1, H, I), dtype=torch.uint8, device=dev())
    status = nv.mlp_workspace_status(ws)
    args, gkw = _decode_call(mode, x, w, sc, p_gu, p_d, I)
    run = lambda: nv.mlp_forward(*args, ws=ws, **gkw)
    nv.set_decode_wait_test(True, 64)
    try:
        y = to_host(run())
    finally:
        nv.set_decode_wait_test(False)
    torch.cuda.synchronize()
    assert to_host(status)[0] == nv.STATUS_DECODE_WAIT_EXPIRED
    assert np.all(np.isnan(y))
    status.zero_()
    y = to_host(run())
    torch.cuda.synchronize()
    assert to_host(status)[0] == 0
    gemm_close(y, _decode_ref(mode, x, w, sc)["out"], f"decode mode {mode} after an expired launch")


@pytest.mark.parametrize("mode", [0, 1])
def test_mlp_decode_graph_capture(mode):
    """Under stream capture mlp_forward records the two-launch path (the
    single launch needs a new epoch per run); replays match eager results."""
    nv.set_path(nv.PATH_AUTO)
    H, I = 512, 4352
    w = mlp_weights(H, I, 0)
    p_gu, p_d = packed_weights(H, I, 0)
    xs = [synth.activations(7 + k, 1, H) for k in range(3)]
    sc = calibrate_activation_scales(xs[0], w) if mode == 0 else None
    args, gkw = _decode_call(mode, xs[0], w, sc, p_gu, p_d, I)
    xd = args[1]
    nws = nv.mlp_workspace_bytes(mode, 1, H, I)
    ws = torch.zeros((nws,), dtype=torch.uint8, device=dev())
    out = torch.empty((1, H), dtype=torch.float32, device=dev())
    call = lambda: nv.mlp_forward(*args, ws=ws, out=out, **gkw)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for x in xs + xs[:1]:
        xd.copy_(to_dev(x))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        y_graph = to_host(out)
        eager = to_host(nv.mlp_forward(*args, ws=torch.zeros_like(ws), **gkw))
        torch.cuda.synchronize()
        r = _decode_ref(mode, x, w, sc)
        gemm_close(y_graph, r["out"], f"graph replay mode {mode}")
        gemm_close(eager, r["out"], f"eager mode {mode}")


@pytest.mark.parametrize("mode,M", [(0, 64), (0, 128), (1, 100)])
def test_mlp_split_down_graph_replay(mode, M):
    """The forward with its down projection K-split on the mid-size kernel
    (hidden 2048, intermediate 6400: 3 splits), captured in a graph and
    replayed on three inputs, eager forwards between the replays: every
    replay equals the eager forward bit for bit (the split counters are
    cleared by the gate_up launch and left at zero, no memset in the graph)."""
    nv.set_path(nv.PATH_AUTO)
    H, I = 2048, 6400
    w = mlp_weights(H, I, 0)
    p_gu, p_d = packed_weights(H, I, 0)
    xs = [synth.activations(11 + k, M, H) for k in range(3)]
    if mode == 0:
        sc = calibrate_activation_scales(xs[0], w)
        args = (0, to_dev(xs[0]), p_gu, scalar(sc["a_gu"]), p_d, scalar(sc["a_d"]), I)
        gkw = dict(g1_inv=scalar(sc["g1_inv"]), g2_inv=scalar(sc["g2_inv"]))
    else:
        sc = None
        args = (1, to_dev(xs[0]), p_gu, scalar(w["g_gu"]), p_d, scalar(w["g_d"]), I)
        gkw = {}
    xd = args[1]
    nws = nv.mlp_workspace_bytes(mode, M, H, I)
    ws = torch.full((nws,), 0xFF, dtype=torch.uint8, device=dev())
    out = torch.empty((M, H), dtype=torch.float32, device=dev())
    call = lambda: nv.mlp_forward(*args, ws=ws, out=out, **gkw)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for k, x in enumerate(xs + xs[:1]):
        xd.copy_(to_dev(x))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        y_graph = to_host(out)
        eager = to_host(nv.mlp_forward(*args, ws=torch.full_like(ws, 0xFF), **gkw))
        torch.cuda.synchronize()
        assert np.array_equal(y_graph, eager), f"replay {k} differs from the eager forward"
        if k == 0:
            r = _decode_ref(mode, x, w, sc)
            gemm_close(y_graph, r["out"], f"split-down graph mode {mode} M={M}")


def test_swiglu_fused_requant_prefill_sampled_rows():
    """The fused gate_up + SwiGLU + NVFP4 kernel at the prefill shape (8192
    tokens, hidden 7168, intermediate 18432: the tiled kernel) against the
    pure oracle's h on 16 seeded rows, under the tie rule."""
    nv.set_path(nv.PATH_AUTO)
    M, H, I = 8192, 7168, 18432
    w = mlp_weights(H, I, 0)
    p_gu, _ = packed_weights(H, I, 0)
    x = synth.activations(0, M, H)
    sc = calibrate_activation_scales(x[:64], w)
    xq, xs = oracle.quantize(x, sc["g1_inv"])
    hc, hs = nv.gemm_swiglu_nvfp4_quant(to_dev(xq), to_dev(xs), p_gu, I, H, scalar(sc["a_gu"]),
                                        scalar(sc["g2_inv"]))
    rows = np.sort(np.random.default_rng(18432).choice(M, 16, replace=False))
    h_ref = oracle.swiglu(oracle.gemm_w4a4(xq[rows], xs[rows], w["c_gu"], w["s_gu"], sc["a_gu"]))
    n, total = requant_check(to_host(hc)[rows], to_host(hs)[rows], h_ref, sc["g2_inv"])
    print(f"prefill h: {n} of {total} re-quantized elements differ")


def test_mlp_prefill_full_size_sampled_rows():
    """Prefill W4A4: M=8192 on the GPU, 64 seeded rows checked by the oracle."""
    nv.set_path(nv.PATH_AUTO)
    rows = np.sort(np.random.default_rng(8192).choice(8192, 64, replace=False))
    _check_mlp("w4a4", 8192, 7168, 18432, rows=rows)


def test_mlp_prefill_tail_split():
    """W4A4 prefill whose down projection ends in a part-filled round of
    tiles: hidden 4096 (16 weight tiles) x 4352 tokens (17 token tiles) is
    272 output tiles, 16 past one per CU, so those 16 are K-split (3 ways at
    intermediate 6144). Sampled rows (all but the first 256 tokens cross the
    split tiles) against the oracle; a second call on the same workspace
    (counters left at zero by the first) gives the same bytes."""
    nv.set_path(nv.PATH_AUTO)
    M, H, I = 4352, 4096, 6144
    rows = np.unique(np.concatenate([np.random.default_rng(4352).choice(M, 24, replace=False), [0, 300, M - 1]]))
    y = _check_mlp("w4a4", M, H, I, rows=rows)
    w = mlp_weights(H, I, 0)
    p_gu, p_d = packed_weights(H, I, 0)
    x = synth.activations(0, M, H)
    sc = calibrate_activation_scales(x[:64], w)
    ws = torch.zeros(nv.mlp_workspace_bytes(0, M, H, I), dtype=torch.uint8, device=dev())
    outs = []
    for _ in range(2):
        outs.append(to_host(nv.mlp_forward(0, to_dev(x), p_gu, scalar(sc["a_gu"]), p_d, scalar(sc["a_d"]), I,
                                           g1_inv=scalar(sc["g1_inv"]), g2_inv=scalar(sc["g2_inv"]), ws=ws)))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], y)


@pytest.mark.parametrize("mode", ["w4a4", "w4a16"])
@pytest.mark.parametrize("M", [128, 200])
def test_mlp_tiled_small_grid_split(mode, M):
    """Tiled kernels, down projection of fewer tiles than CUs (hidden 1024:
    4 weight tiles x 1-2 token tiles), K split to fill one round
    (intermediate 4096: 16 K tiles). The workspace starts as 0xFF bytes and
    a second call on it gives the same bytes."""
    nv.set_path(nv.PATH_AUTO)
    H, I = 1024, 4096
    w = mlp_weights(H, I, 0)
    p_gu, p_d = packed_weights(H, I, 0)
    x = synth.activations(M, M, H)
    qm = 0 if mode == "w4a4" else 1
    ws = torch.full((nv.mlp_workspace_bytes(qm, M, H, I),), 0xFF, dtype=torch.uint8, device=dev())
    if mode == "w4a4":
        sc = calibrate_activation_scales(x[:64], w)
        run = lambda: nv.mlp_forward(0, to_dev(x), p_gu, scalar(sc["a_gu"]), p_d, scalar(sc["a_d"]), I,
                                     g1_inv=scalar(sc["g1_inv"]), g2_inv=scalar(sc["g2_inv"]), ws=ws)
    else:
        run = lambda: nv.mlp_forward(1, to_dev(x), p_gu, scalar(w["g_gu"]), p_d, scalar(w["g_d"]), I, ws=ws)
    ys = [to_host(run()) for _ in range(2)]
    if mode == "w4a4":
        r = oracle.mlp_w4a4(x, w["c_gu"], w["s_gu"], sc["a_gu"], w["c_d"], w["s_d"], sc["a_d"], sc["g1_inv"],
                            sc["g2_inv"])
    else:
        r = oracle.mlp_w4a16(x, w["c_gu"], w["s_gu"], w["g_gu"], w["c_d"], w["s_d"], w["g_d"])
    gemm_close(ys[0], r["out"], f"{mode} small-grid split M={M}")
    assert np.array_equal(ys[0], ys[1])


def test_mlp_w4a16_gate_up_tail_split():
    """W4A16 at 256 tokens, intermediate 17408: the gate_up GEMM has 272
    tiles, 16 past one round, whose K is split (its SwiGLU epilogue runs on
    the combined sums). Hidden 512 keeps the oracle cheap. The workspace
    starts as 0xFF bytes (the gate_up's first launch clears every split
    counter) and a second call on it gives the same bytes."""
    nv.set_path(nv.PATH_AUTO)
    M, H, I = 256, 512, 17408
    w = mlp_weights(H, I, 0)
    p_gu, p_d = packed_weights(H, I, 0)
    x = synth.activations(11, M, H)
    ws = torch.full((nv.mlp_workspace_bytes(1, M, H, I),), 0xFF, dtype=torch.uint8, device=dev())
    ys = [to_host(nv.mlp_forward(1, to_dev(x), p_gu, scalar(w["g_gu"]), p_d, scalar(w["g_d"]), I, ws=ws))
          for _ in range(2)]
    rows = np.arange(120, 256, 3)  # the split tiles hold tokens 128..255
    r = oracle.mlp_w4a16(x[rows], w["c_gu"], w["s_gu"], w["g_gu"], w["c_d"], w["s_d"], w["g_d"])
    gemm_close(ys[0][rows], r["out"], "w4a16 gate_up tail split")
    assert np.array_equal(ys[0], ys[1])


@pytest.mark.parametrize("M", [1, 16, 256, 4096])
def test_mlp_w4a16_full_size(M):
    nv.set_path(nv.PATH_AUTO)
    rows = np.arange(M) if M <= 16 else np.sort(np.random.default_rng(M).choice(M, 32, replace=False))
    _check_mlp("w4a16", M, 5120, 17408, rows=rows)


# -- every kernel instantiation: waves per workgroup (16, 8, 4) x token tiles --

# 17, 513 and 1025 row groups select 16-, 8- and 4-wave workgroups.
WAVE_N = [272, 8208, 16400]
M_FOR = {"gemv": [1, 2, 3], "stream": [5, 12, 16, 20, 40, 60]}


@pytest.mark.parametrize("kpath", ["gemv", "stream"])
@pytest.mark.parametrize("N", WAVE_N)
@pytest.mark.parametrize("mode", ["w4a4", "w4a16"])
def test_gemm_wave_variants(kpath, N, mode):
    prev = nv.set_path(PATHS[kpath])
    try:
        rng = np.random.default_rng(N)
        K = 512
        wc, ws = rand_nvfp4(rng, N, K)
        p = nv.nvfp4_repack_weight(0, to_dev(wc), to_dev(ws))
        for M in M_FOR[kpath]:
            if mode == "w4a4":
                ac, as_ = rand_nvfp4(rng, M, K)
                ref = oracle.gemm_w4a4(ac, as_, wc, ws, np.float32(0.5))
                y = nv.nvfp4_gemm(0, to_dev(ac), to_dev(as_), p, N, K, scalar(0.5))
            else:
                x = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
                ref = oracle.gemm_w4a16(x, wc, ws, np.float32(0.5))
                y = nv.nvfp4_gemm(1, to_dev(x), None, p, N, K, scalar(0.5))
            gemm_close(to_host(y), ref, f"{kpath} {mode} N={N} M={M}")
    finally:
        nv.set_path(prev)


@pytest.mark.parametrize("kpath", ["gemv", "stream"])
@pytest.mark.parametrize("I", [256, 8208, 16400])
def test_swiglu_wave_variants(kpath, I):
    """SwiGLU epilogues (f32, bf16, NVFP4) at 16-, 8- and 4-wave workgroups."""
    prev = nv.set_path(PATHS[kpath])
    try:
        rng = np.random.default_rng(I)
        H = 512
        wc, ws = rand_nvfp4(rng, 2 * I, H)
        p = nv.nvfp4_repack_weight(1, to_dev(wc), to_dev(ws))
        for M in M_FOR[kpath]:
            ac, as_ = rand_nvfp4(rng, M, H)
            alpha = np.float32(0.01)
            h_ref = oracle.swiglu(oracle.gemm_w4a4(ac, as_, wc, ws, alpha))
            h32 = nv.gemm_swiglu(0, to_dev(ac), to_dev(as_), p, I, H, scalar(alpha), h_dtype=torch.float32)
            gemm_close(to_host(h32), h_ref, f"{kpath} swiglu I={I} M={M}")
            _, g2_inv = oracle.global_scale(h_ref)
            hc, hs = nv.gemm_swiglu_nvfp4_quant(to_dev(ac), to_dev(as_), p, I, H, scalar(alpha), scalar(g2_inv))
            oc, os_ = oracle.quantize(to_host(h32), g2_inv)
            assert np.array_equal(to_host(hc), oc) and np.array_equal(to_host(hs), os_)
            hb = nv.gemm_swiglu(0, to_dev(ac), to_dev(as_), p, I, H, scalar(alpha), h_dtype=torch.bfloat16)
            assert np.array_equal(to_host(hb), synth.f32_to_bf16_bits(to_host(h32)))
            # W4A16 with the same weights
            x = synth.f32_to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
            h_ref16 = oracle.swiglu(oracle.gemm_w4a16(x, wc, ws, alpha))
            for dt in (torch.float32, torch.bfloat16):
                hh = nv.gemm_swiglu(1, to_dev(x), None, p, I, H, scalar(alpha), h_dtype=dt)
                gemm_close(to_host(hh).astype(np.float32) if dt == torch.float32 else
                           synth.bf16_bits_to_f32(to_host(hh)), h_ref16, f"{kpath} w4a16 swiglu I={I} M={M}")
    finally:
        nv.set_path(prev)
