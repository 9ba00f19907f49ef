"""GPU parity of the grouped (expert) NVFP4 GEMM with masked_m against the
CPU oracle, W4A4 and W4A16, on the weight-streaming, mid-size (W4A4) and
tiled kernels (every expert in one launch): rows past
masked_m keep the sentinel the output held, valid rows
meet the fp32 tolerance, and each expert matches the plain GEMM entry."""
import numpy as np
import pytest
import torch

import nvfp4_synth as synth
import oracle
from gpu_helpers import dev, gemm_close, scalar, to_dev, to_host

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


def _case(seed, E, M, N, K):
    rng = np.random.default_rng(seed)
    ac = rng.integers(0, 256, (E, M, K // 2), dtype=np.uint8)
    asc = rng.integers(0x28, 0x48, (E, M, K // 16), dtype=np.uint8)
    xb = synth.activations(seed, E * M, K).reshape(E, M, K)
    wc = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    ws = rng.integers(0x28, 0x48, (E, N, K // 16), dtype=np.uint8)
    al = (0.01 * np.exp(rng.standard_normal(E))).astype(np.float32)
    return ac, asc, xb, wc, ws, al


def _packed(wc, ws):
    return torch.cat([nv.nvfp4_repack_weight(nv.REPACK_PLAIN, to_dev(wc[e]), to_dev(ws[e]))
                      for e in range(wc.shape[0])])


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("E,M,N,K,mm", [
    (3, 1, 272, 768, [1, 0, 1]), (4, 5, 272, 768, [5, 2, 0, 9]), (2, 40, 512, 1024, [40, 17]),
    (3, 300, 288, 512, [300, 1, 129]), (2, 64, 256, 256, None),
    (20, 16, 256, 512, [16, 0, 3, 16, 9, 0, 1, 12, 16, 5, 7, 0, 16, 2, 11, 16, 4, 8, 0, 15]),
    (4, 200, 256, 512, [200, 77, 0, 130])])
@pytest.mark.parametrize("kpath", ["auto", "tiled", "stream", "mid"])
def test_grouped_gemm_matches_oracle(kpath, mode, E, M, N, K, mm):
    """Every expert runs in one launch: under the automatic path W4A4 on the
    mid-size kernel from 64 to 512 tokens per expert, otherwise on the
    weight-streaming kernel up to 256 tokens and on the tiled kernel above;
    the overrides force a kernel at any size (W4A16 has no mid-size kernel:
    its override runs the streaming one)."""
    prev = nv.set_path({"tiled": nv.PATH_TILED, "stream": nv.PATH_STREAM, "mid": nv.PATH_MID}.get(kpath, nv.PATH_AUTO))
    try:
        _grouped_vs_oracle(mode, E, M, N, K, mm)
    finally:
        nv.set_path(prev)


def _grouped_vs_oracle(mode, E, M, N, K, mm):
    ac, asc, xb, wc, ws, al = _case(E * 100 + M, E, M, N, K)
    a, sc = (ac, asc) if mode == 0 else (xb, None)
    mmv = None if mm is None else np.array(mm, np.int32)
    out = torch.full((E, M, N), float("nan"), dtype=torch.float32, device=dev())
    y = nv.nvfp4_grouped_gemm(mode, to_dev(a), None if sc is None else to_dev(sc), _packed(wc, ws), N, K,
                              to_dev(al), None if mmv is None else to_dev(mmv), out=out)
    yh = to_host(y)
    ref = oracle.grouped_gemm(mode, a, sc, wc, ws, np.full(E, M, np.int32) if mmv is None else mmv, al)
    for e in range(E):
        rows = M if mmv is None else max(0, min(M, int(mmv[e])))
        assert np.all(np.isnan(yh[e, rows:])), f"expert {e}: rows past masked_m written"
        if rows:
            gemm_close(yh[e, :rows], ref[e, :rows], f"mode {mode} expert {e}")


def test_grouped_gemm_equals_plain_gemm_per_expert():
    """With every row valid, each expert's output is the plain GEMM entry's
    on that expert's operands, bit for bit (same kernel, same M)."""
    E, M, N, K = 3, 24, 272, 768
    ac, asc, xb, wc, ws, al = _case(7, E, M, N, K)
    prev = nv.set_path(nv.PATH_STREAM)
    try:
        y = to_host(nv.nvfp4_grouped_gemm(0, to_dev(ac), to_dev(asc), _packed(wc, ws), N, K, to_dev(al)))
        for e in range(E):
            p = nv.nvfp4_repack_weight(nv.REPACK_PLAIN, to_dev(wc[e]), to_dev(ws[e]))
            ye = to_host(nv.nvfp4_gemm(0, to_dev(ac[e]), to_dev(asc[e]), p, N, K, scalar(al[e])))
            assert np.array_equal(y[e], ye), e
    finally:
        nv.set_path(prev)


@pytest.mark.parametrize("M", [16, 300])
def test_grouped_gemm_bf16_output(M):
    """bf16 output is the f32 output rounded to nearest even, on the
    streaming (16 tokens) and tiled (300) launches, masked rows untouched."""
    E, N, K = 3, 256, 512
    ac, asc, xb, wc, ws, al = _case(11 + M, E, M, N, K)
    mmv = to_dev(np.array([M, M // 3, 0], np.int32))
    args = (0, to_dev(ac), to_dev(asc), _packed(wc, ws), N, K, to_dev(al))
    y32 = to_host(nv.nvfp4_grouped_gemm(*args, masked_m=mmv))
    sentinel = torch.full((E, M, N), 0x7FC1, dtype=torch.int16, device=dev()).view(torch.bfloat16)
    y16 = nv.nvfp4_grouped_gemm(*args, masked_m=mmv, out=sentinel)
    b = to_host(y16.view(torch.int16)).view(np.uint16)
    for e, rows in enumerate([M, M // 3, 0]):
        assert np.array_equal(b[e, :rows], synth.f32_to_bf16_bits(y32[e, :rows])), e
        assert np.all(b[e, rows:] == 0x7FC1), f"expert {e}: rows past masked_m written"
