"""CPU oracle for the NVFP4 dense MLP -- TEST INFRASTRUCTURE.

A ctypes binding of ``nvfp4_oracle.c``. It is what the GPU library is
checked against; only the tests, the smoke check of the entry module and the
CPU-baseline leg of the benchmark may import it. It shares no code with the
HIP library and never calls it.

Arrays are numpy; codes are uint8 [rows, K/2] (element 2i in the low nibble),
scales uint8 [rows, K/16] (E4M3FN), bf16 values are carried as uint16 bits.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64 = ctypes.c_int64
_f32 = ctypes.c_float


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB) or (
                os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        sig = {
            "orc_e2m1_value": (ctypes.c_double, [ctypes.c_uint32]),
            "orc_e4m3_value": (ctypes.c_double, [ctypes.c_uint32]),
            "orc_e4m3_encode": (ctypes.c_uint32, [_f32]),
            "orc_e2m1_encode": (ctypes.c_uint32, [_f32]),
            "orc_bf16_to_f32": (_f32, [ctypes.c_uint16]),
            "orc_f32_to_bf16": (ctypes.c_uint16, [_f32]),
            "orc_global_scale": (None, [_f32p, _i64, _f32p, _f32p]),
            "orc_alpha": (_f32, [_f32, _f32]),
            "orc_quantize": (None, [_f32p, _i64, _i64, _f32, _u8p, _u8p]),
            "orc_dequantize": (None, [_u8p, _u8p, _i64, _i64, _f64p]),
            "orc_gemm_w4a4": (None, [_u8p, _u8p, _u8p, _u8p, _i64, _i64, _i64, _f32, _f32p]),
            "orc_gemm_w4a4_dense": (None, [_u8p, _u8p, _u8p, _u8p, _i64, _i64, _i64, _f32, _f32p]),
            "orc_gemm_w4a16": (None, [_u16p, _u8p, _u8p, _i64, _i64, _i64, _f32, _f32p]),
            "orc_gemm_w4a16_dense": (None, [_u16p, _u8p, _u8p, _i64, _i64, _i64, _f32, _f32p]),
            "orc_swiglu": (None, [_f32p, _i64, _i64, _f32p]),
            "orc_mlp_w4a4": (None, [_u16p, _i64, _i64, _i64, _u8p, _u8p, _f32, _u8p, _u8p, _f32,
                                    _f32, _f32, _f32p, _u8p, _u8p, _f32p, _f32p, _u8p, _u8p]),
            "orc_mlp_w4a16": (None, [_u16p, _i64, _i64, _i64, _u8p, _u8p, _f32, _u8p, _u8p, _f32,
                                     _f32p, _f32p, _u16p]),
            "orc_quantize_per_token": (None, [_f32p, _i64, _i64, _u8p, _u8p, _f32p]),
            "orc_gemm_w4a4_rows": (None, [_u8p, _u8p, _u8p, _u8p, _i64, _i64, _i64, _f32p, _f32p]),
            "orc_mlp_w4a4_per_token": (None, [_u16p, _i64, _i64, _i64, _u8p, _u8p, _f32, _u8p, _u8p,
                                              _f32, _f32, _f32p, _u8p, _u8p, _f32p, _f32p, _f32p,
                                              _u8p, _u8p]),
            "orc_silu_mul_quant_experts": (None, [_u16p, _i64, _i64, _i64, _i32p, _f32p, _u8p, _u8p,
                                                  _f32p]),
            "orc_prescale_bf16": (None, [_u16p, _u16p, _i64, _i64, _u16p]),
            "orc_mlp_w4a16_awq": (None, [_u16p, _i64, _i64, _i64, _u8p, _u8p, _f32, _u16p, _u8p, _u8p, _f32,
                                         _u16p, _f32p, _u16p, _u16p]),
            "orc_grouped_gemm": (None, [ctypes.c_int, _u8p, _u8p, _u16p, _u8p, _u8p, _i64, _i64, _i64, _i64,
                                        _i32p, _f32p, _f32p]),
            "orc_num_threads": (ctypes.c_int, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def _p(a, t):
    return a.ctypes.data_as(t)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_lib().orc_num_threads())


# -- formats ---------------------------------------------------------------

def e2m1_value(code: int) -> float:
    return _lib().orc_e2m1_value(int(code))


def e4m3_value(byte: int) -> float:
    return _lib().orc_e4m3_value(int(byte))


def e4m3_encode(v: float) -> int:
    return int(_lib().orc_e4m3_encode(float(v)))


def e2m1_encode(y: float) -> int:
    return int(_lib().orc_e2m1_encode(float(y)))


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    h = _c(h, np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    lib = _lib()
    x = _c(x, np.float32).ravel()
    out = np.empty(x.shape, np.uint16)
    for i in range(x.size):
        out[i] = lib.orc_f32_to_bf16(float(x[i]))
    return out


# -- scales and quantize ---------------------------------------------------

def global_scale(x: np.ndarray):
    """(g, g_inv) as np.float32 for the tensor x (bf16 as uint16 or fp32)."""
    x = bf16_to_f32(x) if x.dtype == np.uint16 else _c(x, np.float32)
    x = np.ascontiguousarray(x).ravel()
    g = _f32()
    gi = _f32()
    _lib().orc_global_scale(_p(x, _f32p), x.size, ctypes.byref(g), ctypes.byref(gi))
    return np.float32(g.value), np.float32(gi.value)


def alpha(g_a, g_w) -> np.float32:
    return np.float32(_lib().orc_alpha(float(g_a), float(g_w)))


def quantize(x: np.ndarray, g_inv):
    """x: [M, K] fp32, or bf16 bits as uint16 (widened exactly)."""
    x = bf16_to_f32(x) if x.dtype == np.uint16 else _c(x, np.float32)
    x = np.ascontiguousarray(x)
    M, K = x.shape
    assert K % 16 == 0
    codes = np.empty((M, K // 2), np.uint8)
    scales = np.empty((M, K // 16), np.uint8)
    _lib().orc_quantize(_p(x, _f32p), M, K, float(g_inv), _p(codes, _u8p), _p(scales, _u8p))
    return codes, scales


def quantize_per_token(x: np.ndarray):
    """Per-token dynamic quantization of x [M, K] (fp32, or bf16 bits as
    uint16): returns (codes, scales, g) with g [M] fp32, each row's own
    global scale."""
    x = bf16_to_f32(x) if x.dtype == np.uint16 else _c(x, np.float32)
    x = np.ascontiguousarray(x)
    M, K = x.shape
    assert K % 16 == 0
    codes = np.empty((M, K // 2), np.uint8)
    scales = np.empty((M, K // 16), np.uint8)
    g = np.empty(M, np.float32)
    _lib().orc_quantize_per_token(_p(x, _f32p), M, K, _p(codes, _u8p), _p(scales, _u8p), _p(g, _f32p))
    return codes, scales, g


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    M, K = codes.shape[0], codes.shape[1] * 2
    out = np.empty((M, K), np.float64)
    _lib().orc_dequantize(_p(codes, _u8p), _p(scales, _u8p), M, K, _p(out, _f64p))
    return out


# -- GEMMs -----------------------------------------------------------------

def gemm_w4a4(a_codes, a_scales, w_codes, w_scales, alpha_, dense=False) -> np.ndarray:
    a_codes, a_scales = _c(a_codes, np.uint8), _c(a_scales, np.uint8)
    w_codes, w_scales = _c(w_codes, np.uint8), _c(w_scales, np.uint8)
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = w_codes.shape[0]
    assert w_codes.shape[1] * 2 == K
    out = np.empty((M, N), np.float32)
    fn = _lib().orc_gemm_w4a4_dense if dense else _lib().orc_gemm_w4a4
    fn(_p(a_codes, _u8p), _p(a_scales, _u8p), _p(w_codes, _u8p), _p(w_scales, _u8p),
       M, N, K, float(alpha_), _p(out, _f32p))
    return out


def gemm_w4a16(x_bf16, w_codes, w_scales, alpha_, dense=False) -> np.ndarray:
    x = _c(x_bf16, np.uint16)
    w_codes, w_scales = _c(w_codes, np.uint8), _c(w_scales, np.uint8)
    M, K = x.shape
    N = w_codes.shape[0]
    assert w_codes.shape[1] * 2 == K
    out = np.empty((M, N), np.float32)
    fn = _lib().orc_gemm_w4a16_dense if dense else _lib().orc_gemm_w4a16
    fn(_p(x, _u16p), _p(w_codes, _u8p), _p(w_scales, _u8p), M, N, K, float(alpha_),
       _p(out, _f32p))
    return out


def swiglu(gu: np.ndarray) -> np.ndarray:
    gu = _c(gu, np.float32)
    M, I2 = gu.shape
    I = I2 // 2
    h = np.empty((M, I), np.float32)
    _lib().orc_swiglu(_p(gu, _f32p), M, I, _p(h, _f32p))
    return h


def silu_mul_quant_experts(gate_up_bf16, masked_m, g_inv, codes=None, scales=None):
    """Standalone SiLU(gate) * up + NVFP4 quantization of a bf16 gate_up
    [E, M, 2I] by expert: rows t < masked_m[e] of expert e quantized with
    g_inv[e]. Returns (codes [E, M, I/2], scales [E, M, I/16], h [E, M, I]);
    rows past masked_m keep what codes/scales held (zeros if not given) and
    their h is NaN."""
    gu = _c(gate_up_bf16, np.uint16)
    E, M, I2 = gu.shape
    I = I2 // 2
    assert I % 16 == 0
    mm = _c(masked_m, np.int32)
    gi = _c(g_inv, np.float32)
    assert mm.shape == (E,) and gi.shape == (E,)
    codes = np.zeros((E, M, I // 2), np.uint8) if codes is None else _c(codes, np.uint8).copy()
    scales = np.zeros((E, M, I // 16), np.uint8) if scales is None else _c(scales, np.uint8).copy()
    h = np.full((E, M, I), np.nan, np.float32)
    _lib().orc_silu_mul_quant_experts(_p(gu, _u16p), E, M, I, _p(mm, _i32p), _p(gi, _f32p), _p(codes, _u8p),
                                      _p(scales, _u8p), _p(h, _f32p))
    return codes, scales, h


# -- MLP -------------------------------------------------------------------

def gemm_w4a4_rows(a_codes, a_scales, w_codes, w_scales, alpha_rows) -> np.ndarray:
    """W4A4 GEMM whose output row i is scaled by alpha_rows[i]."""
    a_codes, a_scales = _c(a_codes, np.uint8), _c(a_scales, np.uint8)
    w_codes, w_scales = _c(w_codes, np.uint8), _c(w_scales, np.uint8)
    alpha_rows = _c(alpha_rows, np.float32)
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = w_codes.shape[0]
    out = np.empty((M, N), np.float32)
    _lib().orc_gemm_w4a4_rows(_p(a_codes, _u8p), _p(a_scales, _u8p), _p(w_codes, _u8p),
                              _p(w_scales, _u8p), M, N, K, _p(alpha_rows, _f32p), _p(out, _f32p))
    return out


def mlp_w4a4_per_token(x_bf16, wgu_codes, wgu_scales, g_wgu, wd_codes, wd_scales, alpha_d,
                       g2_inv) -> dict:
    """W4A4 forward with per-token dynamic scales for x; every stage."""
    x = _c(x_bf16, np.uint16)
    M, H = x.shape
    I = wd_codes.shape[1] * 2
    assert wgu_codes.shape == (2 * I, H // 2) and wd_codes.shape == (H, I // 2)
    wgu_codes, wgu_scales = _c(wgu_codes, np.uint8), _c(wgu_scales, np.uint8)
    wd_codes, wd_scales = _c(wd_codes, np.uint8), _c(wd_scales, np.uint8)
    r = {
        "out": np.empty((M, H), np.float32),
        "xq": np.empty((M, H // 2), np.uint8), "xs": np.empty((M, H // 16), np.uint8),
        "g": np.empty(M, np.float32),
        "gu": np.empty((M, 2 * I), np.float32), "h": np.empty((M, I), np.float32),
        "hq": np.empty((M, I // 2), np.uint8), "hs": np.empty((M, I // 16), np.uint8),
    }
    _lib().orc_mlp_w4a4_per_token(_p(x, _u16p), M, H, I, _p(wgu_codes, _u8p), _p(wgu_scales, _u8p),
                                  float(g_wgu), _p(wd_codes, _u8p), _p(wd_scales, _u8p),
                                  float(alpha_d), float(g2_inv), _p(r["out"], _f32p),
                                  _p(r["xq"], _u8p), _p(r["xs"], _u8p), _p(r["g"], _f32p),
                                  _p(r["gu"], _f32p), _p(r["h"], _f32p), _p(r["hq"], _u8p),
                                  _p(r["hs"], _u8p))
    return r


def mlp_w4a4(x_bf16, wgu_codes, wgu_scales, alpha_gu, wd_codes, wd_scales, alpha_d,
             g1_inv, g2_inv) -> dict:
    """Full W4A4 forward; returns every stage: xq, xs, gu, h, hq, hs, out."""
    x = _c(x_bf16, np.uint16)
    M, H = x.shape
    I = wd_codes.shape[1] * 2
    assert wgu_codes.shape == (2 * I, H // 2) and wd_codes.shape == (H, I // 2)
    wgu_codes, wgu_scales = _c(wgu_codes, np.uint8), _c(wgu_scales, np.uint8)
    wd_codes, wd_scales = _c(wd_codes, np.uint8), _c(wd_scales, np.uint8)
    r = {
        "out": np.empty((M, H), np.float32),
        "xq": np.empty((M, H // 2), np.uint8), "xs": np.empty((M, H // 16), np.uint8),
        "gu": np.empty((M, 2 * I), np.float32), "h": np.empty((M, I), np.float32),
        "hq": np.empty((M, I // 2), np.uint8), "hs": np.empty((M, I // 16), np.uint8),
    }
    _lib().orc_mlp_w4a4(_p(x, _u16p), M, H, I, _p(wgu_codes, _u8p), _p(wgu_scales, _u8p),
                        float(alpha_gu), _p(wd_codes, _u8p), _p(wd_scales, _u8p),
                        float(alpha_d), float(g1_inv), float(g2_inv), _p(r["out"], _f32p),
                        _p(r["xq"], _u8p), _p(r["xs"], _u8p), _p(r["gu"], _f32p),
                        _p(r["h"], _f32p), _p(r["hq"], _u8p), _p(r["hs"], _u8p))
    return r


def mlp_w4a16(x_bf16, wgu_codes, wgu_scales, alpha_gu, wd_codes, wd_scales, alpha_d) -> dict:
    """Full W4A16 forward; returns gu (fp32), h (bf16 bits), out (fp32)."""
    x = _c(x_bf16, np.uint16)
    M, H = x.shape
    I = wd_codes.shape[1] * 2
    assert wgu_codes.shape == (2 * I, H // 2) and wd_codes.shape == (H, I // 2)
    wgu_codes, wgu_scales = _c(wgu_codes, np.uint8), _c(wgu_scales, np.uint8)
    wd_codes, wd_scales = _c(wd_codes, np.uint8), _c(wd_scales, np.uint8)
    r = {"out": np.empty((M, H), np.float32), "gu": np.empty((M, 2 * I), np.float32),
         "h": np.empty((M, I), np.uint16)}
    _lib().orc_mlp_w4a16(_p(x, _u16p), M, H, I, _p(wgu_codes, _u8p), _p(wgu_scales, _u8p),
                         float(alpha_gu), _p(wd_codes, _u8p), _p(wd_scales, _u8p),
                         float(alpha_d), _p(r["out"], _f32p), _p(r["gu"], _f32p),
                         _p(r["h"], _u16p))
    return r


def prescale_bf16(x_bf16, s_bf16) -> np.ndarray:
    """AWQ pre-quant scaling: bf16(x * s) per input channel (bf16 bits in and out)."""
    x = _c(x_bf16, np.uint16)
    sv = _c(s_bf16, np.uint16)
    M, K = x.shape
    assert sv.shape == (K,)
    out = np.empty((M, K), np.uint16)
    _lib().orc_prescale_bf16(_p(x, _u16p), _p(sv, _u16p), M, K, _p(out, _u16p))
    return out


def mlp_w4a16_awq(x_bf16, wgu_codes, wgu_scales, alpha_gu, s_gu, wd_codes, wd_scales, alpha_d, s_d) -> dict:
    """W4A16 forward with AWQ pre-quant scales s_gu [H] and s_d [I] (bf16 bits)
    on the inputs of the two GEMMs; returns out (fp32), xs and hs (the scaled
    GEMM inputs, bf16 bits)."""
    x = _c(x_bf16, np.uint16)
    M, H = x.shape
    I = wd_codes.shape[1] * 2
    assert wgu_codes.shape == (2 * I, H // 2) and wd_codes.shape == (H, I // 2)
    sg, sd = _c(s_gu, np.uint16), _c(s_d, np.uint16)
    assert sg.shape == (H,) and sd.shape == (I,)
    wgu_codes, wgu_scales = _c(wgu_codes, np.uint8), _c(wgu_scales, np.uint8)
    wd_codes, wd_scales = _c(wd_codes, np.uint8), _c(wd_scales, np.uint8)
    r = {"out": np.empty((M, H), np.float32), "xs": np.empty((M, H), np.uint16),
         "hs": np.empty((M, I), np.uint16)}
    _lib().orc_mlp_w4a16_awq(_p(x, _u16p), M, H, I, _p(wgu_codes, _u8p), _p(wgu_scales, _u8p), float(alpha_gu),
                             _p(sg, _u16p), _p(wd_codes, _u8p), _p(wd_scales, _u8p), float(alpha_d),
                             _p(sd, _u16p), _p(r["out"], _f32p), _p(r["xs"], _u16p), _p(r["hs"], _u16p))
    return r


def grouped_gemm(mode, a, a_scales, w_codes, w_scales, masked_m, alpha, out=None) -> np.ndarray:
    """Grouped (expert) GEMM: expert e's first masked_m[e] rows of a[e]
    against its own weight (w_codes[e], w_scales[e]) with alpha[e]. mode 0:
    a = codes [E, M, K/2] + a_scales; mode 1: a = bf16 bits [E, M, K].
    Rows past masked_m keep what out held (NaN if not given)."""
    w_codes, w_scales = _c(w_codes, np.uint8), _c(w_scales, np.uint8)
    E, N, K2 = w_codes.shape
    K = K2 * 2
    if mode == 0:
        ac, asc, ab = _c(a, np.uint8), _c(a_scales, np.uint8), np.zeros(1, np.uint16)
        M = ac.shape[1]
    else:
        ab, ac, asc = _c(a, np.uint16), np.zeros(1, np.uint8), np.zeros(1, np.uint8)
        M = ab.shape[1]
    mm, al = _c(masked_m, np.int32), _c(alpha, np.float32)
    assert mm.shape == (E,) and al.shape == (E,)
    o = np.full((E, M, N), np.nan, np.float32) if out is None else _c(out, np.float32).copy()
    _lib().orc_grouped_gemm(int(mode), _p(ac, _u8p), _p(asc, _u8p), _p(ab, _u16p), _p(w_codes, _u8p),
                            _p(w_scales, _u8p), E, M, N, K, _p(mm, _i32p), _p(al, _f32p), _p(o, _f32p))
    return o
