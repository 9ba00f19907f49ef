"""Helpers of the GPU parity tests: device transfer, the tolerance rules and
oracle-side construction of seeded workloads (weights quantized by the
oracle, global scales calibrated by the oracle)."""
import functools

import numpy as np
import torch

import nvfp4_synth as synth
import oracle

# GEMM / MLP fp32 outputs: max |y - ref| / max |ref| and relative L2 error.
MAX_REL_ERR = 1e-2
REL_L2_ERR = 2e-3
# Fused re-quantized codes: at most this share of elements may differ, each by
# one E2M1 step, and only where the oracle's pre-quant value is within
# TIE_WINDOW (relative) of a rounding boundary.
REQUANT_BUDGET = 1e-3
TIE_WINDOW = 1e-5

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MIDS = (E2M1_GRID[:-1] + E2M1_GRID[1:]) / 2


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:  # bf16 bits
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev())
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def scalar(v) -> torch.Tensor:
    return torch.tensor([np.float32(v)], dtype=torch.float32, device=dev())


def gemm_close(y: np.ndarray, ref: np.ndarray, what: str = ""):
    """The fp32 output tolerance: max abs err / max |ref| and relative L2."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    den = np.max(np.abs(ref))
    if den == 0:
        assert np.max(np.abs(y)) == 0, what
        return 0.0, 0.0
    mre = np.max(np.abs(y - ref)) / den
    rl2 = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert mre <= MAX_REL_ERR and rl2 <= REL_L2_ERR, f"{what}: max rel {mre:.3e}, rel L2 {rl2:.3e}"
    return mre, rl2


def nibbles(codes: np.ndarray) -> np.ndarray:
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = codes & 15
    out[..., 1::2] = codes >> 4
    return out


def _e4m3_value(b):
    return torch.from_numpy(np.ascontiguousarray(b, np.uint8)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def requant_check(kc, ks, h_ref, g2_inv):
    """Check kernel NVFP4 codes/scales of h against the oracle's quantization
    of its own h (fp32). Returns (differing elements, total)."""
    h = np.ascontiguousarray(h_ref, np.float32)
    oc, os_ = oracle.quantize(h, g2_inv)
    M, I = h.shape
    kn, on = nibbles(kc).reshape(M, I // 16, 16), nibbles(oc).reshape(M, I // 16, 16)
    kmag, omag = kn & 7, on & 7
    # scale bytes: one E4M3 step, only where sv sits at the midpoint within the window
    ks = ks.reshape(M, I // 16)
    os_ = os_.reshape(M, I // 16)
    hb = h.reshape(M, I // 16, 16)
    gi = np.float32(g2_inv)
    amax = np.abs(hb).max(axis=2)
    sv = (amax * gi).astype(np.float32) / np.float32(6.0)
    bad_scale = ks != os_
    if np.any(bad_scale):
        ii = np.nonzero(bad_scale)
        d = np.abs(ks[ii].astype(int) - os_[ii].astype(int))
        assert np.all(d == 1), "scale bytes differ by more than one E4M3 step"
        mid = (_e4m3_value(ks[ii]) + _e4m3_value(os_[ii])) / 2
        assert np.all(np.abs(sv[ii] - mid) <= TIE_WINDOW * mid), "scale differs away from a tie"
    # pre-quant values of the oracle with the kernel's scale byte per block
    s_k = _e4m3_value(ks).astype(np.float32)
    with np.errstate(divide="ignore"):
        r = np.where(s_k != 0, gi / s_k, np.float32(0)).astype(np.float32)
    y = (hb * r[:, :, None]).astype(np.float32)
    # reference codes: the oracle's where scales agree; where the scale byte
    # differs (at a tie), the oracle's E2M1 encoding of y under the kernel's scale
    if np.any(bad_scale):
        for a, b in zip(*np.nonzero(bad_scale)):
            omag[a, b] = [oracle.e2m1_encode(float(v)) & 7 for v in y[a, b]]
            on[a, b] = [oracle.e2m1_encode(float(v)) for v in y[a, b]]
    diff = kmag != omag
    n_diff = int(diff.sum()) + int(bad_scale.sum()) * 16
    if np.any(diff):
        step = np.abs(kmag.astype(int) - omag.astype(int))
        assert np.all(step[diff] == 1), "a code differs by more than one E2M1 step"
        ya = np.abs(y[diff].astype(np.float64))
        lo = np.minimum(kmag[diff], omag[diff])
        bnd = E2M1_MIDS[lo]
        assert np.all(np.abs(ya - bnd) <= TIE_WINDOW * bnd), "a code differs away from a boundary"
        # signs must agree where the magnitude is non-zero on both sides
    nz = (kmag != 0) & (omag != 0)
    assert np.array_equal((kn & 8)[nz], (on & 8)[nz]), "sign mismatch"
    total = M * I
    assert n_diff <= REQUANT_BUDGET * total, f"{n_diff} of {total} re-quantized elements differ"
    return n_diff, total


@functools.lru_cache(maxsize=8)
def mlp_weights(H: int, I: int, seed: int = 0):
    """Oracle-quantized gate_up [2I, H] (rows [gate; up]) and down [H, I]."""
    wgu = synth.weights(seed, 2 * I, H, synth.TENSOR_W_GATE_UP)
    g_gu, gi_gu = oracle.global_scale(wgu)
    c_gu, s_gu = oracle.quantize(wgu, gi_gu)
    del wgu
    wd = synth.weights(seed, H, I, synth.TENSOR_W_DOWN)
    g_d, gi_d = oracle.global_scale(wd)
    c_d, s_d = oracle.quantize(wd, gi_d)
    del wd
    return dict(H=H, I=I, g_gu=g_gu, c_gu=c_gu, s_gu=s_gu, g_d=g_d, c_d=c_d, s_d=s_d)


@functools.lru_cache(maxsize=8)
def packed_weights(H: int, I: int, seed: int = 0):
    import nvfp4_quantized_dense_amd as nv
    w = mlp_weights(H, I, seed)
    p_gu = nv.nvfp4_repack_weight(nv.REPACK_SWIGLU, to_dev(w["c_gu"]), to_dev(w["s_gu"]))
    p_d = nv.nvfp4_repack_weight(nv.REPACK_PLAIN, to_dev(w["c_d"]), to_dev(w["s_d"]))
    torch.cuda.synchronize()
    return p_gu, p_d


def calibrate_activation_scales(x_bf16: np.ndarray, w: dict):
    """Static scales as a calibration pass would set them: g1 from x, g2 from
    the oracle's h for that x (W4A4)."""
    g1, g1_inv = oracle.global_scale(x_bf16)
    a_gu = oracle.alpha(g1, w["g_gu"])
    gu = oracle.gemm_w4a4(*oracle.quantize(x_bf16, g1_inv), w["c_gu"], w["s_gu"], a_gu)
    h = oracle.swiglu(gu)
    g2, g2_inv = oracle.global_scale(h)
    a_d = oracle.alpha(g2, w["g_d"])
    return dict(g1=g1, g1_inv=g1_inv, g2=g2, g2_inv=g2_inv, a_gu=a_gu, a_d=a_d)
