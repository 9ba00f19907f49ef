"""Pins of the CPU oracle against facts fixed outside it.

Each test ties the oracle to something it does not itself compute: the
E2M1 grid, torch's independent float8_e4m3fn and bfloat16 conversions,
hand-worked examples (tests/golden/quant_examples.txt), brute-force nearest
searches, closed forms, numpy float64 matmuls of independently decoded
operands, and invariants of the encoding.
"""
import math
import os
import subprocess

import numpy as np
import pytest
import torch

import nvfp4_synth as synth
from golden_fixtures import global_scale_examples

HERE = os.path.dirname(os.path.abspath(__file__))
GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


# -- independent decoders used by the pins (not the oracle's) ---------------

def ref_e4m3(byte_arr):
    """E4M3FN bytes -> float64 via torch's float8_e4m3fn."""
    t = torch.from_numpy(np.ascontiguousarray(byte_arr, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def ref_e2m1(codes4):
    c = np.asarray(codes4)
    mag = np.array(GRID)[c & 7]
    return np.where(c & 8, -mag, mag)


def ref_dequant(codes, scales):
    lo = codes & 15
    hi = codes >> 4
    q = np.empty((codes.shape[0], codes.shape[1] * 2), np.float64)
    q[:, 0::2] = ref_e2m1(lo)
    q[:, 1::2] = ref_e2m1(hi)
    s = np.repeat(ref_e4m3(scales), 16, axis=1)
    return q * s


def nibbles(codes):
    out = np.empty((codes.shape[0], codes.shape[1] * 2), np.uint8)
    out[:, 0::2] = codes & 15
    out[:, 1::2] = codes >> 4
    return out


# -- formats ----------------------------------------------------------------

def test_e2m1_decode_is_the_grid(orc):
    for c in range(8):
        assert orc.e2m1_value(c) == GRID[c]
        v = orc.e2m1_value(c | 8)
        assert v == -GRID[c] and math.copysign(1.0, v) == -1.0


def test_e4m3_decode_matches_torch_float8_e4m3fn(orc):
    ref = ref_e4m3(np.arange(256, dtype=np.uint8))
    for b in range(256):
        v = orc.e4m3_value(b)
        if math.isnan(ref[b]):
            assert math.isnan(v), b
        else:
            assert v == ref[b], (b, v, ref[b])
    assert orc.e4m3_value(0x7E) == 448.0
    assert orc.e4m3_value(0x08) == 2.0 ** -6
    assert orc.e4m3_value(0x01) == 2.0 ** -9
    assert math.isnan(orc.e4m3_value(0x7F))


def test_e4m3_encode_matches_torch_rne_below_448(orc):
    # every finite non-negative E4M3 value, every midpoint, and 3 ulps around each
    vals = np.sort(ref_e4m3(np.arange(127, dtype=np.uint8)))
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids, [448.0]]).astype(np.float32)
    u = pts.view(np.uint32).astype(np.int64)
    near = np.concatenate([u + d for d in range(-3, 4)])
    near = near[(near >= 0) & (near < 0x43E00000)].astype(np.uint32).view(np.float32)
    rng = np.random.default_rng(1)
    rand = (rng.random(200000) * 448).astype(np.float32)
    xs = np.unique(np.concatenate([near, rand]))
    xs = xs[(xs >= 0) & (xs <= 448)]
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(float(x)) for x in xs], np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (xs[bad[:5]], got[bad[:5]], ref[bad[:5]])
    # satfinite above the largest finite value (torch gives NaN or 448 there)
    for x in [448.0, 449.0, 463.99, 464.0, 500.0, 1e6, 3.0e38]:
        assert orc.e4m3_encode(x) == 0x7E


def test_encoders_exhaustive_against_brute_force(tmp_path):
    """Every fp32 pattern in the binades where codes change, strided elsewhere."""
    import oracle
    oracle._lib()
    from oracle import build as ob
    exe = str(tmp_path / "exh")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "exhaustive_encoders.c"), "-L", os.path.dirname(ob.LIB),
                    "-loracle_nvfp4", "-Wl,-rpath," + os.path.dirname(ob.LIB), "-lm",
                    "-lpthread"], check=True)
    r = subprocess.run([exe, str(min(8, os.cpu_count() or 1)), "fast"], capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0 and "OK" in r.stdout, r.stdout + r.stderr


def test_e2m1_encode_ties_and_signed_zero(orc):
    mids = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for y, c in mids.items():
        assert orc.e2m1_encode(y) == c
        assert orc.e2m1_encode(-y) == c | 8
    assert orc.e2m1_encode(-0.0) == 8
    assert orc.e2m1_encode(-1e-30) == 8
    assert orc.e2m1_encode(6.9) == 7 and orc.e2m1_encode(1e30) == 7


def test_bf16_round_trip_matches_torch(orc):
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e-38).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 65504.0, 3.0e38], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.f32_to_bf16(x), ref)
    assert np.array_equal(synth.f32_to_bf16_bits(x), ref)
    assert np.array_equal(orc.bf16_to_f32(ref), torch.from_numpy(ref.view(np.int16)).view(
        torch.bfloat16).float().numpy())


# -- quantize -----------------------------------------------------------------

def load_golden():
    rows = []
    with open(os.path.join(HERE, "golden", "quant_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, gi, xs, sb, codes, packed = [p.strip() for p in line.split("|")]
            rows.append((name, float(gi), [float(v) for v in xs.split()], int(sb, 16),
                         [int(c, 16) for c in codes.split()],
                         [int(b, 16) for b in packed.split()]))
    return rows


@pytest.mark.parametrize("ex", load_golden(), ids=lambda e: e[0])
def test_quantize_golden_examples(orc, ex):
    name, gi, xs, sb, codes, packed = ex
    c, s = orc.quantize(np.array([xs], np.float32), np.float32(gi))
    assert s[0, 0] == sb
    assert list(nibbles(c)[0]) == codes
    assert list(c[0]) == packed


def test_quantize_block_max_maps_to_six_and_error_bound(orc):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.standard_normal((64, 1)))).astype(np.float32)
    g, gi = orc.global_scale(x)
    c, s = orc.quantize(x, gi)
    deq = ref_dequant(c, s)               # q * s, independently decoded
    sv = ref_e4m3(s)
    xb = x.reshape(64, 16, 16).astype(np.float64)
    amax_idx = np.abs(xb).argmax(axis=2)
    nib = nibbles(c).reshape(64, 16, 16)
    for i in range(64):
        for b in range(16):
            if sv[i, b] >= 2.0 ** -6:      # normal scales: the block max element is +-6
                assert nib[i, b, amax_idx[i, b]] & 7 == 7
    # element error: |x*g_inv - q*s| <= half the E2M1 spacing at |y|, times s
    y = xb * np.float64(gi)
    spacing = np.where(np.abs(y / np.repeat(sv, 16, 1).reshape(64, 16, 16)) < 2, 0.5, 1.0)
    spacing = np.where(np.abs(y / np.repeat(sv, 16, 1).reshape(64, 16, 16)) >= 4, 2.0, spacing)
    err = np.abs(y - deq.reshape(64, 16, 16))
    bound = 0.5 * spacing * np.repeat(sv, 16, 1).reshape(64, 16, 16) * (1 + 1e-6) + 1e-30
    # r = g_inv/s is rounded to fp32, so allow its relative error as well
    assert np.all(err <= bound + np.abs(y) * 2.0 ** -22)


def test_quantize_idempotent_for_power_of_two_global(orc):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((8, 512)).astype(np.float32)
    for gi in [1.0, 4.0, 0.25]:
        c, s = orc.quantize(x, np.float32(gi))
        xd = (ref_dequant(c, s) / gi).astype(np.float32)   # exact: powers of two
        c2, s2 = orc.quantize(xd, np.float32(gi))
        assert np.array_equal(s, s2)
        # codes agree up to the sign of zero
        n1, n2 = nibbles(c), nibbles(c2)
        assert np.array_equal(np.where(n1 & 7, n1, 0), np.where(n2 & 7, n2, 0))


def test_quantize_single_slot_exhaustive_bf16(orc):
    """Slot 0 holds 6 (so s = 1, r = 1 at g_inv = 1); slot 1 walks every finite
    bf16 value with |v| <= 6: its code must be the brute-force nearest."""
    vals = np.arange(65536, dtype=np.uint16)
    f = synth.bf16_bits_to_f32(vals)
    keep = np.isfinite(f) & (np.abs(f) <= 6.0)
    f = f[keep]
    x = np.zeros((f.size, 16), np.float32)
    x[:, 0] = 6.0
    x[:, 1] = f
    c, s = orc.quantize(x, np.float32(1.0))
    assert np.all(s == 0x38)
    got = nibbles(c)[:, 1]
    a = np.abs(f.astype(np.float64))[:, None]
    d = np.abs(a - np.array(GRID)[None, :])
    best = np.argmin(d, axis=1)
    # ties: the even index
    dmin = d[np.arange(f.size), best]
    tie_hi = (best + 1 < 8) & np.isclose(d[np.arange(f.size), np.minimum(best + 1, 7)], dmin,
                                          rtol=0, atol=0)
    best = np.where(tie_hi & (best % 2 == 1), best + 1, best)
    exp = best | np.where(np.signbit(f), 8, 0)
    assert np.array_equal(got, exp)


def test_global_scale_golden_non_power_of_two(orc):
    """g and g_inv at amax 3, 6, 11, 25 from the hand-worked fixture: g_inv is
    the reciprocal of the rounded g, not fl(2688 / amax)."""
    ex = global_scale_examples()
    assert len(ex) == 4
    for amax, g_ref, gi_ref, alt in ex:
        x = np.array([[0.5, -amax, 1.0]], np.float32)
        g, gi = orc.global_scale(x)
        assert g == g_ref, (amax, g, g_ref)
        assert gi == gi_ref, (amax, gi, gi_ref)
        assert gi != alt


def test_global_scale_and_alpha(orc):
    x = np.array([[1.0, -2688.0, 3.0]], np.float32)
    g, gi = orc.global_scale(x)
    assert g == np.float32(1.0) and gi == np.float32(1.0)
    x = np.array([[448.0 * 6 * 0.5]], np.float32)
    g, gi = orc.global_scale(x)
    assert g == np.float32(0.5) and gi == np.float32(2.0)
    assert orc.alpha(np.float32(0.5), np.float32(0.25)) == np.float32(0.125)
    # bf16 input is widened exactly
    xb = synth.f32_to_bf16_bits(np.array([[-2688.0, 1.0]], np.float32))
    assert orc.global_scale(xb)[0] == np.float32(1.0)


# -- GEMMs --------------------------------------------------------------------

def rand_nvfp4(rng, R, K, scale_lo=0x30, scale_hi=0x48):
    codes = rng.integers(0, 256, (R, K // 2), dtype=np.uint8)
    scales = rng.integers(scale_lo, scale_hi, (R, K // 16), dtype=np.uint8)
    return codes, scales


def test_gemm_closed_form_all_sixes(orc):
    K = 256
    a = np.full((3, K // 2), 0x77, np.uint8)     # +6 +6
    w = np.full((5, K // 2), 0x77, np.uint8)
    w[1] = 0xFF                                   # -6 -6
    ones = lambda r: np.full((r, K // 16), 0x38, np.uint8)
    y = orc.gemm_w4a4(a, ones(3), w, ones(5), np.float32(0.5))
    assert np.all(y[:, 0] == 36 * K * 0.5) and np.all(y[:, 1] == -36 * K * 0.5)
    y = orc.gemm_w4a4(a, ones(3), w, ones(5), np.float32(0.5), dense=True)
    assert np.all(y[:, 0] == 36 * K * 0.5)


def test_gemm_worked_example_block_a(orc):
    # block A of the golden file against w = 16 x 1.0 with scale byte 0x40 (2.0)
    x = np.array([[0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, 6, -0.25, -2.5, 0.5, 1, 1.5, 2, 3, 4]],
                 np.float32)
    ac, as_ = orc.quantize(x, np.float32(1.0))
    wc = np.full((1, 8), 0x22, np.uint8)
    ws = np.array([[0x40]], np.uint8)
    assert orc.gemm_w4a4(ac, as_, wc, ws, np.float32(1.0))[0, 0] == 60.0


@pytest.mark.parametrize("M,N,K", [(1, 16, 64), (3, 5, 128), (7, 33, 256), (16, 48, 512)])
def test_gemm_w4a4_against_numpy_matmul(orc, M, N, K):
    rng = np.random.default_rng(M * 1000 + N)
    ac, as_ = rand_nvfp4(rng, M, K)
    wc, ws = rand_nvfp4(rng, N, K)
    alpha = np.float32(0.0123)
    ref = (np.float64(alpha) * (ref_dequant(ac, as_) @ ref_dequant(wc, ws).T)).astype(np.float32)
    y1 = orc.gemm_w4a4(ac, as_, wc, ws, alpha)
    y2 = orc.gemm_w4a4(ac, as_, wc, ws, alpha, dense=True)
    assert y1.shape == (M, N)
    # both formulations are the exact sum rounded once, up to double rounding
    ulp = np.spacing(np.abs(ref)).astype(np.float64)
    assert np.all(np.abs(y1.astype(np.float64) - ref) <= ulp)
    assert np.all(np.abs(y2.astype(np.float64) - ref) <= ulp)


@pytest.mark.parametrize("M,N,K", [(1, 16, 64), (5, 9, 256)])
def test_gemm_w4a16_against_numpy_matmul(orc, M, N, K):
    rng = np.random.default_rng(7 + M)
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    wc, ws = rand_nvfp4(rng, N, K)
    alpha = np.float32(0.02)
    ref = (np.float64(alpha) * (synth.bf16_bits_to_f32(x).astype(np.float64)
                                @ ref_dequant(wc, ws).T)).astype(np.float32)
    ulp = np.spacing(np.abs(ref)).astype(np.float64)
    for dense in (False, True):
        y = orc.gemm_w4a16(x, wc, ws, alpha, dense=dense)
        assert np.all(np.abs(y.astype(np.float64) - ref) <= ulp)


def test_gemm_power_of_two_scales_exact(orc):
    """With power-of-two scales every partial sum is an exactly representable
    fp32 for these sizes, so the result is exact (the GPU must match bit for bit)."""
    rng = np.random.default_rng(9)
    M, N, K = 4, 32, 1024
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    as_ = rng.choice(np.array([0x30, 0x38, 0x40], np.uint8), (M, K // 16))
    ws = rng.choice(np.array([0x30, 0x38, 0x40], np.uint8), (N, K // 16))
    y = orc.gemm_w4a4(ac, as_, wc, ws, np.float32(0.25))
    ref = 0.25 * (ref_dequant(ac, as_) @ ref_dequant(wc, ws).T)
    assert np.array_equal(y.astype(np.float64), ref)


# -- SwiGLU and the MLP -------------------------------------------------------

def test_swiglu_closed_form(orc):
    from scipy.special import expit
    rng = np.random.default_rng(11)
    gu = (rng.standard_normal((6, 64)) * 4).astype(np.float32)
    gu[0, 0] = 0.0
    gu[0, 1] = -100.0
    gu[0, 2] = 100.0
    h = orc.swiglu(gu)
    g, u = gu[:, :32].astype(np.float64), gu[:, 32:].astype(np.float64)
    ref = (g * expit(g) * u).astype(np.float32)
    assert np.all(np.abs(h - ref) <= np.spacing(np.abs(ref)))
    assert h[0, 0] == 0.0
    assert abs(h[0, 1]) < 1e-40
    assert h[0, 2] == np.float32(100.0 * np.float64(gu[0, 34]))


def _tiny_mlp_inputs(orc, M=4, H=256, I=512):
    x = synth.activations(0, M, H)
    wgu = synth.weights(0, 2 * I, H, synth.TENSOR_W_GATE_UP)
    wd = synth.weights(0, H, I, synth.TENSOR_W_DOWN)
    ggu, ggu_inv = orc.global_scale(wgu)
    gd, gd_inv = orc.global_scale(wd)
    wguc, wgus = orc.quantize(wgu, ggu_inv)
    wdc, wds = orc.quantize(wd, gd_inv)
    g1, g1_inv = orc.global_scale(x)
    return x, wgu, wd, (ggu, wguc, wgus), (gd, wdc, wds), (g1, g1_inv)


def test_mlp_w4a4_stages_compose(orc):
    x, wgu, wd, (ggu, wguc, wgus), (gd, wdc, wds), (g1, g1_inv) = _tiny_mlp_inputs(orc)
    a_gu = orc.alpha(g1, ggu)
    # g2 calibrated on this input's h
    gu = orc.gemm_w4a4(*orc.quantize(x, g1_inv), wguc, wgus, a_gu)
    h = orc.swiglu(gu)
    g2, g2_inv = orc.global_scale(h)
    a_d = orc.alpha(g2, gd)
    r = orc.mlp_w4a4(x, wguc, wgus, a_gu, wdc, wds, a_d, g1_inv, g2_inv)
    assert np.array_equal(r["gu"], gu) and np.array_equal(r["h"], h)
    hq, hs = orc.quantize(h, g2_inv)
    assert np.array_equal(r["hq"], hq) and np.array_equal(r["hs"], hs)
    assert np.array_equal(r["out"], orc.gemm_w4a4(hq, hs, wdc, wds, a_d))
    # the NVFP4 MLP tracks the fp64 MLP of the unquantized weights
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    gu64 = xf @ wgu.T.astype(np.float64)
    g64, u64 = gu64[:, :512], gu64[:, 512:]
    out64 = (g64 / (1 + np.exp(-g64)) * u64) @ wd.T.astype(np.float64)
    rel = np.linalg.norm(r["out"] - out64) / np.linalg.norm(out64)
    assert rel < 0.25, rel


def test_mlp_w4a16_stages_compose(orc):
    x, wgu, wd, (ggu, wguc, wgus), (gd, wdc, wds), _ = _tiny_mlp_inputs(orc)
    r = orc.mlp_w4a16(x, wguc, wgus, ggu, wdc, wds, gd)
    gu = orc.gemm_w4a16(x, wguc, wgus, ggu)
    assert np.array_equal(r["gu"], gu)
    hb = orc.f32_to_bf16(orc.swiglu(gu)).reshape(r["h"].shape)
    assert np.array_equal(r["h"], hb)
    assert np.array_equal(r["out"], orc.gemm_w4a16(hb, wdc, wds, gd))


def test_mlp_uses_gate_as_first_half(orc):
    """Swapping the gate and up halves of W_gate_up must change h (a mistaken
    half assignment would pass the composition test but fail this one)."""
    x, wgu, wd, (ggu, wguc, wgus), (gd, wdc, wds), (g1, g1_inv) = _tiny_mlp_inputs(orc)
    gu = orc.gemm_w4a4(*orc.quantize(x, g1_inv), wguc, wgus, orc.alpha(g1, ggu))
    h = orc.swiglu(gu)
    g, u = gu[:, :512].astype(np.float64), gu[:, 512:].astype(np.float64)
    assert np.allclose(h, g / (1 + np.exp(-g)) * u, rtol=1e-6, atol=1e-30)
    assert not np.allclose(h, u / (1 + np.exp(-u)) * g, rtol=1e-3)


# -- per-token dynamic activation scales ------------------------------------

@pytest.mark.parametrize("v", [3.0, -0.015625, 1.0e-3, -1234.5, 2688.0])
def test_per_token_single_element_row(orc, v):
    """A row whose only nonzero is v: g = fl(|v| / 2688); v's block takes the
    largest scale (E4M3 448 = 0x7E) and v the largest code (6, signed);
    every other block is zero."""
    K = 64
    x = np.zeros((1, K), np.float32)
    x[0, 21] = v
    c, s, g = orc.quantize_per_token(x)
    assert g[0] == np.float32(np.float32(abs(v)) / np.float32(2688.0))
    assert s[0, 1] == 0x7E and ref_e4m3(s[0, 1]) == 448.0
    n = nibbles(c)[0]
    assert n[21] == (0xF if v < 0 else 0x7)
    assert np.all(np.delete(n, 21) & 7 == 0) and np.all(np.delete(s[0], 1) == 0)
    # dequantized back: q * s * g reproduces v to the E2M1/E4M3 rounding
    assert abs(6 * 448 * float(g[0]) - abs(v)) <= 1e-6 * abs(v)


def test_per_token_power_of_two_rows(orc):
    """Rows that are one row times powers of two quantize to the same codes
    and scales, with g scaled by exactly that power (amax, the division by
    2688 and g_inv all scale exactly)."""
    base = np.random.default_rng(11).standard_normal(256).astype(np.float32)
    ks = [-3, -1, 0, 2, 5]
    x = np.stack([base * np.float32(2.0 ** k) for k in ks])
    c, s, g = orc.quantize_per_token(x)
    for i in range(1, len(ks)):
        assert np.array_equal(c[i], c[0]) and np.array_equal(s[i], s[0])
        assert g[i] == np.float32(g[0] * np.float32(2.0 ** (ks[i] - ks[0])))


def test_per_token_zero_row_and_mixed_magnitudes(orc):
    """A zero row gets g = 0, zero codes and scales; the other rows are
    quantized as each alone with the per-tensor calibration (rows of very
    different magnitude share nothing)."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal((4, 128)).astype(np.float32)
    x[1] = 0.0
    x[2] *= np.float32(1e-4)
    x[3] *= np.float32(300.0)
    c, s, g = orc.quantize_per_token(x)
    assert g[1] == 0 and not c[1].any() and not s[1].any()
    for i in (0, 2, 3):
        gi, gi_inv = orc.global_scale(x[i:i + 1])
        assert g[i] == gi
        ci, si = orc.quantize(x[i:i + 1], gi_inv)
        assert np.array_equal(c[i:i + 1], ci) and np.array_equal(s[i:i + 1], si)


def test_gemm_rows_scale_each_row(orc):
    """Per-row alphas scale output rows exactly where they differ by powers of
    two, and each row equals numpy's float64 matmul of the decoded operands
    times its own alpha."""
    rng = np.random.default_rng(13)
    M, N, K = 3, 20, 256
    wc, ws = rand_nvfp4(rng, N, K)
    ac1, as1 = rand_nvfp4(rng, 1, K)
    ac, as_ = np.repeat(ac1, M, axis=0), np.repeat(as1, M, axis=0)
    a = np.array([0.0625, 0.125, 0.5], np.float32)
    y = orc.gemm_w4a4_rows(ac, as_, wc, ws, a)
    assert np.array_equal(y[1], 2 * y[0]) and np.array_equal(y[2], 8 * y[0])
    ref = ref_dequant(ac, as_) @ ref_dequant(wc, ws).T
    assert np.allclose(y, (ref * a[:, None].astype(np.float64)).astype(np.float32), rtol=1e-6, atol=0)


def test_mlp_per_token_single_row_equals_static(orc):
    """On one token the per-token forward is the static one with that token's
    own calibration (g1 = its g, alpha_gu = fl(g1 * g_wgu)); on several tokens
    each row equals its own single-token forward."""
    x, wgu, wd, (ggu, wguc, wgus), (gd, wdc, wds), _ = _tiny_mlp_inputs(orc, M=3)
    a_d, g2_inv = np.float32(0.002), np.float32(50.0)
    r = orc.mlp_w4a4_per_token(x, wguc, wgus, ggu, wdc, wds, a_d, g2_inv)
    for t in range(3):
        g1, g1_inv = orc.global_scale(x[t:t + 1])
        assert r["g"][t] == g1
        s = orc.mlp_w4a4(x[t:t + 1], wguc, wgus, orc.alpha(g1, ggu), wdc, wds, a_d, g1_inv, g2_inv)
        assert np.array_equal(r["out"][t:t + 1], s["out"])
        assert np.array_equal(r["xq"][t:t + 1], s["xq"]) and np.array_equal(r["hq"][t:t + 1], s["hq"])


# -- standalone SiLU(gate) * up + NVFP4 quantize by expert (masked_m) --------

def _bf16(a):
    return synth.f32_to_bf16_bits(np.asarray(a, np.float32))


def test_silu_quant_rows_past_masked_m_untouched(orc):
    """Rows t >= masked_m[e] keep what the outputs held (masked_m clamped to
    [0, M]); the other rows are written."""
    rng = np.random.default_rng(21)
    E, M, I = 4, 6, 64
    gu = _bf16(rng.standard_normal((E, M, 2 * I)) * 2)
    mm = np.array([0, 3, 9, -2], np.int32)
    sc = np.full((E, M, I // 2), 0xAB, np.uint8)
    ss = np.full((E, M, I // 16), 0xAB, np.uint8)
    c, s, h = orc.silu_mul_quant_experts(gu, mm, np.ones(E, np.float32), sc, ss)
    for e, rows in enumerate([0, 3, 6, 0]):
        assert np.all(c[e, rows:] == 0xAB) and np.all(s[e, rows:] == 0xAB)
        assert np.all(np.isnan(h[e, rows:])) and not np.any(np.isnan(h[e, :rows]))
        assert not np.all(s[e, :rows] == 0xAB) if rows else True


def test_silu_mul_closed_forms(orc):
    """SiLU(g) * u against closed forms: g = 0 or u = 0 gives 0; g = 30 gives
    30 u (sigmoid(30) = 1 - 9.4e-14, below half an ulp of the exact 30 u);
    the gate is the first half of the row (swapping halves breaks the 30 u
    case); h(g, u) - h(-g, u) = g u up to the two fp32 roundings."""
    rng = np.random.default_rng(22)
    I = 64
    u = _bf16(rng.standard_normal(I))
    g = _bf16(rng.standard_normal(I) * 3)
    uf, gf = synth.bf16_bits_to_f32(u), synth.bf16_bits_to_f32(g)
    rows = np.stack([
        np.concatenate([_bf16(np.zeros(I)), u]),       # g = 0
        np.concatenate([g, _bf16(np.zeros(I))]),       # u = 0
        np.concatenate([_bf16(np.full(I, 30.0)), u]),  # g = 30
        np.concatenate([g, u]),
        np.concatenate([g ^ np.uint16(0x8000), u]),    # -g
    ])[None]
    _, _, h = orc.silu_mul_quant_experts(rows, np.array([5], np.int32), np.ones(1, np.float32))
    h = h[0].astype(np.float64)
    assert np.all(h[0] == 0) and np.all(h[1] == 0)
    assert np.array_equal(h[2], (30.0 * uf).astype(np.float32).astype(np.float64))
    ulp = np.spacing(np.abs(h[3]).astype(np.float32)).astype(np.float64) + \
        np.spacing(np.abs(h[4]).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(h[3] - h[4] - gf.astype(np.float64) * uf) <= ulp)


def test_silu_quant_expert_scale_power_of_two(orc):
    """The same rows under g_inv and 2 g_inv: identical codes, and every
    normal, non-saturating scale byte one exponent step (+8) higher: each
    expert uses its own g_inv."""
    rng = np.random.default_rng(23)
    M, I = 8, 256
    gu1 = _bf16(rng.standard_normal((1, M, 2 * I)) * 4)
    gu = np.concatenate([gu1, gu1])
    c, s, h = orc.silu_mul_quant_experts(gu, np.array([M, M], np.int32), np.array([0.75, 1.5], np.float32))
    assert np.array_equal(c[0], c[1]) and np.array_equal(h[0], h[1])
    exp0 = (s[0] >> 3) & 15
    ok = (exp0 >= 1) & (s[0] <= 0x76)
    assert ok.sum() > 100
    assert np.array_equal(s[1][ok], s[0][ok] + 8)


def test_silu_quant_codes_are_the_quantizer_of_h(orc):
    """Each written row's codes and scales are the quantizer's output for
    that row's h with its expert's g_inv."""
    rng = np.random.default_rng(24)
    E, M, I = 2, 3, 128
    gu = _bf16(rng.standard_normal((E, M, 2 * I)) * 2)
    gi = np.array([0.5, 3.0], np.float32)
    c, s, h = orc.silu_mul_quant_experts(gu, np.array([M, 2], np.int32), gi)
    for e, rows in enumerate([M, 2]):
        qc, qs = orc.quantize(h[e, :rows], gi[e])
        assert np.array_equal(c[e, :rows], qc) and np.array_equal(s[e, :rows], qs)


# -- W4A16 AWQ pre-quant scales -------------------------------------------------

def test_prescale_rounds_to_nearest_even_bf16(orc):
    """bf16(x * s): a product below half an ulp rounds down, an exact tie
    goes to the even mantissa, a product past the tie rounds up, s = 1 is the
    identity and a power of two scales exactly."""
    f = lambda v: int(synth.f32_to_bf16_bits(np.array([v], np.float32))[0])
    x = np.array([[f(3.0), f(1.0625), f(1.0625), f(-2.5), f(1.0078125)]], np.uint16)
    s = np.array([f(0.333984375), f(1.0625), f(1.0703125), f(1.0), f(0.25)], np.uint16)
    y = synth.bf16_bits_to_f32(orc.prescale_bf16(x, s))[0]
    # 3 * 0.333984375 = 1.001953125 -> 1.0; 1.0625^2 = 1.12890625 is the tie
    # between 1.125 (even) and 1.1328125; 1.0625 * 1.0703125 = 1.13720703125
    # -> 1.140625; identity; exact quarter.
    assert list(y) == [1.0, 1.125, 1.140625, -2.5, 0.251953125]


def _awq_case(orc, M=3, H=256, I=512, seed=31):
    rng = np.random.default_rng(seed)
    x = synth.activations(seed, M, H)
    wguc = rng.integers(0, 256, (2 * I, H // 2), dtype=np.uint8)
    wgus = rng.integers(0x28, 0x48, (2 * I, H // 16), dtype=np.uint8)
    wdc = rng.integers(0, 256, (H, I // 2), dtype=np.uint8)
    wds = rng.integers(0x28, 0x48, (H, I // 16), dtype=np.uint8)
    return rng, x, wguc, wgus, wdc, wds


def test_awq_unit_scales_are_the_plain_w4a16_forward(orc):
    rng, x, wguc, wgus, wdc, wds = _awq_case(orc)
    one = lambda n: synth.f32_to_bf16_bits(np.ones(n, np.float32))
    a = orc.mlp_w4a16_awq(x, wguc, wgus, np.float32(0.01), one(256), wdc, wds, np.float32(0.02), one(512))
    b = orc.mlp_w4a16(x, wguc, wgus, np.float32(0.01), wdc, wds, np.float32(0.02))
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["xs"], x) and np.array_equal(a["hs"], b["h"])


def test_awq_invariance_with_compensated_weight_scales(orc):
    """AWQ's identity x W^T = (x diag(s)) (W diag(1/s))^T, exact for
    power-of-two s constant over each 16-block: the weight's E4M3 block scale
    moves by the opposite exponent steps (8 per step) and the codes stay, so
    the pre-scaled forward equals the plain one bit for bit."""
    rng, x, wguc, wgus, wdc, wds = _awq_case(orc)
    H, I = 256, 512
    eg = rng.integers(-1, 2, H // 16)   # exponent per block of x's channels
    ed = rng.integers(-1, 2, I // 16)   # per block of h's channels
    s_gu = synth.f32_to_bf16_bits(np.repeat(2.0 ** eg, 16).astype(np.float32))
    s_d = synth.f32_to_bf16_bits(np.repeat(2.0 ** ed, 16).astype(np.float32))
    wgus2 = (wgus.astype(np.int64) - 8 * eg[None, :]).astype(np.uint8)
    wds2 = (wds.astype(np.int64) - 8 * ed[None, :]).astype(np.uint8)
    a = orc.mlp_w4a16_awq(x, wguc, wgus2, np.float32(0.01), s_gu, wdc, wds2, np.float32(0.02), s_d)
    b = orc.mlp_w4a16(x, wguc, wgus, np.float32(0.01), wdc, wds, np.float32(0.02))
    assert np.array_equal(a["out"], b["out"])
    assert not np.array_equal(a["xs"], x)


# -- grouped (expert) GEMM with masked_m --------------------------------------

def _grouped_case(rng, E, M, N, K):
    ac = rng.integers(0, 256, (E, M, K // 2), dtype=np.uint8)
    asc = rng.integers(0x28, 0x48, (E, M, K // 16), dtype=np.uint8)
    xb = synth.f32_to_bf16_bits(rng.standard_normal((E, M, K)).astype(np.float32))
    wc = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    ws = rng.integers(0x28, 0x48, (E, N, K // 16), dtype=np.uint8)
    return ac, asc, xb, wc, ws


@pytest.mark.parametrize("mode", [0, 1])
def test_grouped_gemm_masking_and_expert_independence(orc, mode):
    """Rows past masked_m[e] (clamped to [0, M]) keep their contents; each
    expert's rows depend only on its own activations, weight and alpha:
    swapping two experts swaps their outputs, and a power-of-two alpha
    scales an expert's rows exactly."""
    rng = np.random.default_rng(41 + mode)
    E, M, N, K = 3, 5, 32, 256
    ac, asc, xb, wc, ws = _grouped_case(rng, E, M, N, K)
    a, sc = (ac, asc) if mode == 0 else (xb, None)
    mm = np.array([5, 2, 0], np.int32)
    al = np.array([0.5, 0.25, 1.0], np.float32)
    y = orc.grouped_gemm(mode, a, sc, wc, ws, mm, al)
    assert np.all(np.isnan(y[1, 2:])) and np.all(np.isnan(y[2])) and not np.any(np.isnan(y[0]))
    perm = [1, 0, 2]
    yp = orc.grouped_gemm(mode, a[perm], None if sc is None else sc[perm], wc[perm], ws[perm], mm[perm], al[perm])
    assert np.array_equal(yp[0, :2], y[1, :2]) and np.array_equal(yp[1], y[0])
    y2 = orc.grouped_gemm(mode, a, sc, wc, ws, np.array([5, 9, -1], np.int32), np.array([0.5, 1.0, 1.0], np.float32))
    assert np.array_equal(y2[1, :2], 4 * y[1, :2]) and np.all(np.isnan(y2[2]))


def test_grouped_gemm_rows_are_plain_gemms(orc):
    """Each expert's valid rows equal the float64 product of its decoded
    operands times its alpha (W4A4), within the oracle's final fp32 rounding."""
    rng = np.random.default_rng(43)
    E, M, N, K = 2, 4, 16, 512
    ac, asc, _, wc, ws = _grouped_case(rng, E, M, N, K)
    al = np.array([0.125, 0.0625], np.float32)
    y = orc.grouped_gemm(0, ac, asc, wc, ws, np.array([4, 3], np.int32), al)
    for e, rows in enumerate([4, 3]):
        ref = ref_dequant(ac[e, :rows], asc[e, :rows]) @ ref_dequant(wc[e], ws[e]).T * float(al[e])
        assert np.allclose(y[e, :rows], ref, rtol=1e-6, atol=0)
