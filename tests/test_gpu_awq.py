"""GPU parity of the W4A16 AWQ pre-quant scales against the CPU oracle: the
bf16 pre-scale bit for bit, the MLP forward with scales on both GEMM inputs
within the fp32 tolerance on every kernel path (x' before the gate_up GEMM,
h' in its epilogue), and AWQ's identity on the GPU path."""
import numpy as np
import pytest
import torch

import nvfp4_synth as synth
import oracle
from gpu_helpers import dev, gemm_close, mlp_weights, packed_weights, scalar, to_dev, to_host

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


def awq_scales(seed, n):
    """Per-channel pre-quant scales of AWQ's typical spread (about 0.3 to 3)."""
    rng = np.random.default_rng(seed)
    return synth.f32_to_bf16_bits(np.exp(0.6 * rng.standard_normal(n)).astype(np.float32))


@pytest.mark.parametrize("M,K", [(1, 8), (3, 256), (64, 5120), (257, 17408)])
def test_prescale_bit_exact(M, K):
    x = synth.activations(M + K, M, K)
    s = awq_scales(K, K)
    y = nv.nvfp4_prescale_bf16(to_dev(x), to_dev(s))
    assert np.array_equal(to_host(y), oracle.prescale_bf16(x, s))
    xi = to_dev(x)  # in place
    nv.nvfp4_prescale_bf16(xi, to_dev(s), out=xi)
    assert np.array_equal(to_host(xi), oracle.prescale_bf16(x, s))


def _check_awq(M, H, I, seed=0, rows=None):
    w = mlp_weights(H, I, 0)
    p_gu, p_d = packed_weights(H, I, 0)
    x = synth.activations(seed, M, H)
    s_gu, s_d = awq_scales(1 + seed, H), awq_scales(2 + seed, I)
    y = to_host(nv.mlp_forward_w4a16_awq(to_dev(x), p_gu, scalar(w["g_gu"]), to_dev(s_gu), p_d, scalar(w["g_d"]),
                                         to_dev(s_d), I))
    sel = np.arange(M) if rows is None else rows
    r = oracle.mlp_w4a16_awq(x[sel], w["c_gu"], w["s_gu"], w["g_gu"], s_gu, w["c_d"], w["s_d"], w["g_d"], s_d)
    gemm_close(y[sel], r["out"], f"awq M={M} H={H} I={I}")
    return y


@pytest.mark.parametrize("kpath", list(PATHS))
@pytest.mark.parametrize("M", [1, 5, 40])
def test_awq_mlp_every_path(kpath, M):
    prev = nv.set_path(PATHS[kpath])
    try:
        _check_awq(M, 512, 768, seed=M)
    finally:
        nv.set_path(prev)


@pytest.mark.parametrize("M", [1, 16, 256])
def test_awq_mlp_full_size(M):
    """Hidden 5120, intermediate 17408 (at 256 tokens the gate_up GEMM splits
    its tail tiles and applies s_d after combining)."""
    nv.set_path(nv.PATH_AUTO)
    rows = np.arange(M) if M <= 16 else np.sort(np.random.default_rng(M).choice(M, 24, replace=False))
    _check_awq(M, 5120, 17408, seed=3, rows=rows)


def test_awq_identity_on_the_gpu():
    """Power-of-two scales constant over each 16-block, with the weights'
    block scales moved the opposite way, reproduce the plain W4A16 forward of
    the GPU bit for bit (every path). Weight scale bytes are drawn from
    normal E4M3 values two exponent steps from either end, so every shifted
    byte is still a normal value."""
    H, I, M = 512, 768, 7
    rng = np.random.default_rng(9)
    c_gu = rng.integers(0, 256, (2 * I, H // 2), dtype=np.uint8)
    s_gu_w = rng.integers(0x28, 0x48, (2 * I, H // 16), dtype=np.uint8)
    c_d = rng.integers(0, 256, (H, I // 2), dtype=np.uint8)
    s_d_w = rng.integers(0x28, 0x48, (H, I // 16), dtype=np.uint8)
    g_gu, g_d = np.float32(0.01), np.float32(0.02)
    eg, ed = rng.integers(-1, 2, H // 16), rng.integers(-1, 2, I // 16)
    s_gu = synth.f32_to_bf16_bits(np.repeat(2.0 ** eg, 16).astype(np.float32))
    s_d = synth.f32_to_bf16_bits(np.repeat(2.0 ** ed, 16).astype(np.float32))
    pack = lambda kind, c, sc: nv.nvfp4_repack_weight(kind, to_dev(c), to_dev(sc))
    p_gu, p_d = pack(nv.REPACK_SWIGLU, c_gu, s_gu_w), pack(nv.REPACK_PLAIN, c_d, s_d_w)
    q_gu = pack(nv.REPACK_SWIGLU, c_gu, (s_gu_w.astype(np.int64) - 8 * eg[None, :]).astype(np.uint8))
    q_d = pack(nv.REPACK_PLAIN, c_d, (s_d_w.astype(np.int64) - 8 * ed[None, :]).astype(np.uint8))
    x = synth.activations(4, M, H)
    for kpath in PATHS.values():
        prev = nv.set_path(kpath)
        try:
            a = nv.mlp_forward_w4a16_awq(to_dev(x), q_gu, scalar(g_gu), to_dev(s_gu), q_d, scalar(g_d), to_dev(s_d), I)
            b = nv.mlp_forward(1, to_dev(x), p_gu, scalar(g_gu), p_d, scalar(g_d), I)
            assert np.array_equal(to_host(a), to_host(b)), kpath
        finally:
            nv.set_path(prev)
