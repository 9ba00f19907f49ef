"""GPU parity of the standalone SiLU(gate) * up + NVFP4 quantize (bf16
gate_up batched by expert with masked_m) against the CPU oracle.

Rows past masked_m keep the sentinel bytes the outputs held; written rows
meet the one-step tie rule against the oracle's quantization of its own h
(the kernel evaluates SiLU in fp32, the oracle in double)."""
import numpy as np
import pytest
import torch

import nvfp4_synth as synth
import oracle
from gpu_helpers import dev, requant_check, to_dev, to_host

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


def _inputs(seed, E, M, I, scale=2.0):
    x = synth.bf16_bits_to_f32(synth.activations(seed, E * M, 2 * I)) * np.float32(scale)
    return synth.f32_to_bf16_bits(x).reshape(E, M, 2 * I)


def _g_inv(gu, mm):
    """Per-expert inverse global scales calibrated on the oracle's h."""
    E, M = gu.shape[:2]
    _, _, h = oracle.silu_mul_quant_experts(gu, np.full(E, M, np.int32), np.ones(E, np.float32))
    out = []
    for e in range(E):
        rows = max(1, min(M, int(mm[e]))) if mm is not None else M
        out.append(oracle.global_scale(h[e, :rows])[1])
    return np.array(out, np.float32)


def _check(gu, mm, gi, kc, ks, sentinel=0xAB):
    E, M = gu.shape[:2]
    oc, os_, h = oracle.silu_mul_quant_experts(gu, np.full(E, M, np.int32) if mm is None else mm, gi)
    for e in range(E):
        rows = M if mm is None else max(0, min(M, int(mm[e])))
        assert np.all(kc[e, rows:] == sentinel) and np.all(ks[e, rows:] == sentinel), f"expert {e}: masked rows written"
        if rows:
            requant_check(kc[e, :rows], ks[e, :rows], h[e, :rows], gi[e])


@pytest.mark.parametrize("E,M,I,mm", [
    (1, 1, 256, [1]), (1, 5, 512, [5]), (1, 64, 18432, [64]), (4, 33, 4096, [0, 1, 17, 33]),
    (3, 7, 2064, [7, 50, -1]), (2, 130, 768, None)])
def test_silu_quant_matches_oracle(E, M, I, mm):
    gu = _inputs(E * 1000 + M, E, M, I)
    mmv = None if mm is None else np.array(mm, np.int32)
    gi = _g_inv(gu, mmv)
    kc = torch.full((E, M, I // 2), 0xAB, dtype=torch.uint8, device=dev())
    ks = torch.full((E, M, I // 16), 0xAB, dtype=torch.uint8, device=dev())
    nv.silu_mul_nvfp4_quant(to_dev(gu), to_dev(gi), None if mmv is None else to_dev(mmv), codes=kc, scales=ks)
    _check(gu, mmv, gi, to_host(kc), to_host(ks))


def test_silu_quant_matches_fused_epilogue_codes():
    """On h that is exactly representable in bf16 halves (gate 30, so
    SiLU(g) * u rounds to 30 u in both fp32 and double), the kernel's codes
    equal the oracle's bit for bit."""
    I, M = 1024, 9
    rng = np.random.default_rng(5)
    u = synth.f32_to_bf16_bits(rng.standard_normal((M, I)).astype(np.float32))
    g = synth.f32_to_bf16_bits(np.full((M, I), 30.0, np.float32))
    gu = np.concatenate([g, u], axis=1)[None]
    gi = np.array([0.37], np.float32)
    kc, ks = nv.silu_mul_nvfp4_quant(to_dev(gu), to_dev(gi))
    oc, os_, _ = oracle.silu_mul_quant_experts(gu, np.array([M], np.int32), gi)
    assert np.array_equal(to_host(kc), oc) and np.array_equal(to_host(ks), os_)


def test_silu_quant_prefill_shape_sampled_rows():
    """8192 rows of an intermediate of 18432 (the prefill h), one expert;
    24 seeded rows checked against the oracle."""
    E, M, I = 1, 8192, 18432
    gu = _inputs(77, E, M, I, scale=1.0)
    rows = np.sort(np.random.default_rng(78).choice(M, 24, replace=False))
    sub = np.ascontiguousarray(gu[:, rows])
    gi = _g_inv(sub, None)
    kc, ks = nv.silu_mul_nvfp4_quant(to_dev(gu), to_dev(gi), to_dev(np.array([M], np.int32)))
    kc, ks = to_host(kc)[:, rows], to_host(ks)[:, rows]
    oc, os_, h = oracle.silu_mul_quant_experts(sub, np.array([len(rows)], np.int32), gi)
    requant_check(kc[0], ks[0], h[0], gi[0])
