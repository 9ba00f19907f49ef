"""Exhaustive sweeps of the GPU's two encoders, through the quantize entry.

E2M1 element encoder: with a block maximum of 6 and g_inv = 1 the block
scale is exactly 1 (byte 0x38) and its per-element multiplier is 1, so the
code of every other element is the encoder applied to that element itself.
Every fp32 bit pattern with |x| <= 6, both signs (about 2.2e9 values), goes
through the kernel.

E4M3 block-scale encoder: with g_inv = 1 a block whose only non-zero element
is a gives the scale byte of fl(a / 6). Every fp32 pattern a from 2^-11
(scale rounds to 0) to 4096 (scale saturates at 448) goes through the kernel.

Both encoders are nondecreasing step functions of the input's magnitude
(each is a chain of correctly rounded, monotone operations: the multiply by
g_inv, the divide by 6, round-to-nearest onto a fixed grid), and a positive
fp32 pattern orders like its value. So the oracle's whole map over a range
is fixed by the first pattern at which each output level is reached; those
are found by bisection over the oracle, and every GPU output is checked
against them. A random sample is also compared with the oracle directly,
which does not lean on monotonicity.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import dev, scalar, to_dev, to_host

pytestmark = pytest.mark.gpu

nv = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global nv
    import nvfp4_quantized_dense_amd as _nv
    nv = _nv
    nv.lib()
    assert torch.cuda.is_available()


def _f32(bits: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(bits.astype(np.uint32)).view(np.float32)


def _oracle_e2m1(bits: np.ndarray) -> np.ndarray:
    """Oracle code of each value in a block [6, x, 0, ...] under g_inv = 1."""
    x = np.zeros((bits.size, 16), np.float32)
    x[:, 0] = 6.0
    x[:, 1] = _f32(bits)
    c, s = oracle.quantize(x, np.float32(1.0))
    assert np.all(s[:, 0] == 0x38)
    return (c[:, 0] >> 4).astype(np.int64)


def _oracle_e4m3(bits: np.ndarray) -> np.ndarray:
    """Oracle scale byte of a block [a, 0, ...] under g_inv = 1."""
    x = np.zeros((bits.size, 16), np.float32)
    x[:, 0] = _f32(bits)
    _, s = oracle.quantize(x, np.float32(1.0))
    return s[:, 0].astype(np.int64)


def _first_reaching(fn, lo: int, hi: int, levels: np.ndarray) -> np.ndarray:
    """For a nondecreasing map fn over patterns [lo, hi] with fn(lo) below every
    level and fn(hi) at or above it: the smallest pattern reaching each level
    (one vectorised bisection, one oracle call per halving)."""
    a = np.full(levels.size, lo, np.int64)
    b = np.full(levels.size, hi, np.int64)
    assert np.all(fn(a) < levels) and np.all(fn(b) >= levels)
    while np.any(b - a > 1):
        m = (a + b) // 2
        up = fn(m) >= levels
        b = np.where(up, m, b)
        a = np.where(up, a, m)
    return b


def _bounds_tensor(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(b.astype(np.int32)).to(dev())


E2M1_HI = 0x40C00000        # 6.0
E4M3_LO = 0x3A000000        # 2^-11: fl(a / 6) is below half the smallest subnormal scale
E4M3_HI = 0x45800000        # 4096: fl(a / 6) is above 448


def test_e2m1_encoder_every_fp32_up_to_6():
    levels = np.arange(1, 8)
    bounds = _first_reaching(_oracle_e2m1, 0, E2M1_HI, levels)
    assert _oracle_e2m1(np.array([E2M1_HI]))[0] == 7
    bt = _bounds_tensor(bounds)
    one = scalar(1.0)
    n_all = E2M1_HI + 1
    chunk = 15 << 24
    for start in range(0, n_all, chunk):
        n = min(chunk, n_all - start)
        nb = -(-n // 15)
        bits = torch.arange(start, start + nb * 15, dtype=torch.int32, device=dev())
        bits.clamp_(max=E2M1_HI)  # the tail of the last chunk repeats 6.0
        expect = torch.bucketize(bits, bt, right=True, out_int32=True).to(torch.uint8)
        x = torch.empty((nb, 16), dtype=torch.float32, device=dev())
        x[:, 0] = 6.0
        x[:, 1:] = bits.view(torch.float32).view(nb, 15)
        for sign in (1.0, -1.0):
            xs = x if sign > 0 else -x
            c, s = nv.nvfp4_quantize(xs, one)
            assert bool((s == 0x38).all()), f"scale byte not 0x38 in chunk at {start:#x}"
            nib = torch.stack([c & 15, c >> 4], dim=2).view(nb, 16)[:, 1:].reshape(-1)
            want = expect if sign > 0 else expect | 8
            bad = (nib != want).nonzero()
            assert bad.numel() == 0, (f"sign {sign:+}: first mismatch at pattern "
                                      f"{int(bits[bad[0, 0]]):#010x}: {int(nib[bad[0, 0]])} vs "
                                      f"{int(want[bad[0, 0]])}")
            del c, s, nib
        del x, bits, expect
    torch.cuda.synchronize()


def test_e2m1_encoder_random_sample_direct():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, E2M1_HI + 1, 15 * 100_000, dtype=np.int64).astype(np.uint32)
    bits |= rng.integers(0, 2, bits.size, dtype=np.uint32) << 31
    x = np.empty((100_000, 16), np.float32)
    x[:, 0] = 6.0
    x[:, 1:] = _f32(bits).reshape(-1, 15)
    c, s = nv.nvfp4_quantize(to_dev(x), scalar(1.0))
    oc, os_ = oracle.quantize(x, np.float32(1.0))
    assert np.array_equal(to_host(s), os_) and np.array_equal(to_host(c), oc)


def test_e4m3_encoder_every_fp32_amax():
    lo_byte = _oracle_e4m3(np.array([E4M3_LO]))[0]
    hi_byte = _oracle_e4m3(np.array([E4M3_HI]))[0]
    assert lo_byte == 0 and hi_byte == 0x7E
    levels = np.arange(1, 0x7F)
    bounds = _first_reaching(_oracle_e4m3, E4M3_LO, E4M3_HI, levels)
    bt = _bounds_tensor(bounds)
    one = scalar(1.0)
    chunk = 1 << 24
    for start in range(E4M3_LO, E4M3_HI + 1, chunk):
        n = min(chunk, E4M3_HI + 1 - start)
        bits = torch.arange(start, start + n, dtype=torch.int32, device=dev())
        x = torch.zeros((n, 16), dtype=torch.float32, device=dev())
        x[:, 0] = bits.view(torch.float32)
        _, s = nv.nvfp4_quantize(x, one)
        want = torch.bucketize(bits, bt, right=True, out_int32=True).to(torch.uint8)
        bad = (s[:, 0] != want).nonzero()
        assert bad.numel() == 0, (f"first mismatch at amax pattern {int(bits[bad[0, 0]]):#010x}: "
                                  f"{int(s[bad[0, 0], 0])} vs {int(want[bad[0, 0]])}")
        del x, s, bits, want
    torch.cuda.synchronize()


def test_e4m3_encoder_random_sample_direct():
    rng = np.random.default_rng(6)
    n = 400_000
    x = np.zeros((n, 16), np.float32)
    x[:, 0] = _f32(rng.integers(E4M3_LO, E4M3_HI + 1, n, dtype=np.int64))
    x[:, 1:] = x[:, :1] * rng.uniform(-1, 1, (n, 15)).astype(np.float32)
    for gi in [np.float32(1.0), np.float32(0.6180339), np.float32(3.0)]:
        c, s = nv.nvfp4_quantize(to_dev(x), scalar(gi))
        oc, os_ = oracle.quantize(x, gi)
        assert np.array_equal(to_host(s), os_), f"scale bytes differ (g_inv={gi})"
        assert np.array_equal(to_host(c), oc), f"codes differ (g_inv={gi})"


def test_bf16_every_block_max_under_many_global_scales():
    """The activation path (bf16 input): every positive finite bf16 value as a
    block maximum, with a random sign and slot, the other 15 elements random
    below it, under 48 global scales from 2^-40 to 2^40 (including ones whose
    amax * g_inv overflows fp32: the scale saturates at 448)."""
    import nvfp4_synth as synth
    rng = np.random.default_rng(9)
    amax = synth.bf16_bits_to_f32(np.arange(1, 0x7F80, dtype=np.uint16))
    n = amax.size
    x = (rng.uniform(-1, 1, (n, 16)) * amax[:, None].astype(np.float64)).astype(np.float32)
    x[np.arange(n), rng.integers(0, 16, n)] = amax * rng.choice(np.float32([-1, 1]), n)
    xb = synth.f32_to_bf16_bits(x)
    xd = to_dev(xb)
    g_invs = np.concatenate([np.float32([1.0, 0.5, 3.0, 2688.0, 1.0 / 2688.0]),
                             np.exp2(rng.uniform(-40, 40, 43)).astype(np.float32)])
    for gi in g_invs:
        c, s = nv.nvfp4_quantize(xd, scalar(gi))
        oc, os_ = oracle.quantize(xb, gi)
        assert np.array_equal(to_host(s), os_), f"scale bytes differ (g_inv={gi!r})"
        assert np.array_equal(to_host(c), oc), f"codes differ (g_inv={gi!r})"
