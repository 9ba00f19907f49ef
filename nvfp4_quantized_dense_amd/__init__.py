"""MI355X-native NVFP4 dense MLP: Python binding of libnvfp4_mi355x.so.

Argument marshalling only: every step of the path runs in the HIP library
(include/nvfp4.h). PyTorch supplies device memory (tensors) and the stream
(the current torch stream unless one is given). The library must have been
built (``python -m nvfp4_quantized_dense_amd.build``); importing this module
without it fails loudly, there is no other implementation.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4_mi355x.so")

NVFP4_OK = 0
NVFP4_ERR_INVALID_ARG = -1
NVFP4_ERR_UNSUPPORTED = -2
NVFP4_ERR_HIP = -3
DTYPE_BF16, DTYPE_F32 = 0, 1
MODE_W4A4, MODE_W4A16, MODE_W4A4_DYN, MODE_W4A16_AWQ = 0, 1, 2, 3
REPACK_PLAIN, REPACK_SWIGLU = 0, 1
PATH_AUTO, PATH_GEMV, PATH_STREAM, PATH_TILED, PATH_TILED64, PATH_MID = 0, 1, 2, 3, 4, 5

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_sz = ctypes.c_size_t

# name -> (restype, argtypes); the exported C ABI.
SIGNATURES = {
    "nvfp4_last_error": (ctypes.c_char_p, []),
    "nvfp4_set_path": (_int, [_int]),
    "nvfp4_calibrate": (_int, [_vp, _int, _i64, _vp, _vp, _vp]),
    "nvfp4_quantize": (_int, [_vp, _int, _i64, _i64, _vp, _vp, _vp, _vp]),
    "nvfp4_quantize_per_token": (_int, [_vp, _int, _i64, _i64, _vp, _vp, _vp, _vp]),
    "nvfp4_repack_bytes": (_sz, [_int, _i64, _i64]),
    "nvfp4_packed_bytes": (_sz, [_int, _i64, _i64]),
    "nvfp4_repack_weight": (_int, [_int, _vp, _vp, _i64, _i64, _vp, _vp]),
    "nvfp4_unpack_weight": (_int, [_int, _vp, _i64, _i64, _vp, _vp, _vp]),
    "nvfp4_gemm": (_int, [_int, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _int, _vp]),
    "gemm_swiglu_nvfp4_quant": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "nvfp4_gemm_rowscale": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _int, _vp]),
    "gemm_swiglu_nvfp4_quant_rowscale": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp,
                                                _vp, _vp]),
    "gemm_swiglu": (_int, [_int, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _int, _vp]),
    "silu_mul_nvfp4_quant": (_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "nvfp4_prescale_bf16": (_int, [_vp, _vp, _i64, _i64, _vp, _vp]),
    "mlp_forward_w4a16_awq": (_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _int,
                                     _vp]),
    "nvfp4_grouped_gemm": (_int, [_int, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _int, _vp]),
    "mlp_workspace_bytes": (_sz, [_int, _i64, _i64, _i64]),
    "mlp_workspace_status": (_vp, [_vp, _sz]),
    "nvfp4_set_decode_wait_test": (_int, [_int, _int]),
    "mlp_forward": (_int, [_int, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                           _vp, _int, _vp]),
    "mlp_forward_noalloc": (_int, [_int, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _vp]),
}

_LIB = None


def lib():
    """The loaded C library (ctypes.CDLL) with typed entry points."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m nvfp4_quantized_dense_amd.build); there is no fallback path")
        cdll = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(cdll, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = cdll
    return _LIB


class Nvfp4Error(RuntimeError):
    def __init__(self, name, code, msg):
        super().__init__(f"{name} failed ({code}): {msg}")
        self.code = code


def _check(name, code):
    if code != NVFP4_OK:
        raise Nvfp4Error(name, code, lib().nvfp4_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        if torch.cuda.is_available():
            return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        return None
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return DTYPE_BF16
    if dt == torch.float32:
        return DTYPE_F32
    raise ValueError(f"unsupported dtype {dt}")


def _dense(t, name):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def set_path(path: int) -> int:
    prev = lib().nvfp4_set_path(int(path))
    if prev < 0:
        _check("nvfp4_set_path", prev)
    return prev


def nvfp4_calibrate(x, g=None, g_inv=None, stream=None):
    """(g, g_inv): 1-element fp32 device tensors with g = amax(|x|)/2688."""
    _dense(x, "x")
    g = torch.empty(1, dtype=torch.float32, device=x.device) if g is None else g
    g_inv = torch.empty(1, dtype=torch.float32, device=x.device) if g_inv is None else g_inv
    _check("nvfp4_calibrate", lib().nvfp4_calibrate(_ptr(x), _dtype_code(x.dtype), x.numel(),
                                                    _ptr(g), _ptr(g_inv), _stream(stream)))
    return g, g_inv


def nvfp4_quantize(x, g_inv, codes=None, scales=None, stream=None):
    """x [M, K] bf16/f32 -> (codes uint8 [M, K/2], scales uint8 [M, K/16])."""
    _dense(x, "x")
    M, K = x.shape
    if codes is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M, K // 16), dtype=torch.uint8, device=x.device)
    _check("nvfp4_quantize", lib().nvfp4_quantize(_ptr(x), _dtype_code(x.dtype), M, K, _ptr(g_inv),
                                                  _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def nvfp4_quantize_per_token(x, codes=None, scales=None, row_g=None, stream=None):
    """x [M, K] bf16/f32 -> (codes [M, K/2], scales [M, K/16], row_g fp32 [M]), each row
    quantized with its own global scale row_g[t] = amax(|x[t]|)/2688."""
    _dense(x, "x")
    M, K = x.shape
    if codes is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M, K // 16), dtype=torch.uint8, device=x.device)
    if row_g is None:
        row_g = torch.empty(M, dtype=torch.float32, device=x.device)
    _check("nvfp4_quantize_per_token",
           lib().nvfp4_quantize_per_token(_ptr(x), _dtype_code(x.dtype), M, K, _ptr(codes), _ptr(scales),
                                          _ptr(row_g), _stream(stream)))
    return codes, scales, row_g


def nvfp4_repack_bytes(kind, R, C) -> int:
    return int(lib().nvfp4_repack_bytes(int(kind), int(R), int(C)))


nvfp4_packed_bytes = nvfp4_repack_bytes


def nvfp4_repack_weight(kind, codes, scales, packed=None, stream=None):
    """Canonical NVFP4 weight (codes [R, C/2], scales [R, C/16]) -> packed uint8."""
    _dense(codes, "codes"); _dense(scales, "scales")
    R, C = codes.shape[0], codes.shape[1] * 2
    nbytes = nvfp4_repack_bytes(kind, R, C)
    if packed is None:
        packed = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=codes.device)
    _check("nvfp4_repack_weight", lib().nvfp4_repack_weight(int(kind), _ptr(codes), _ptr(scales), R, C,
                                                            _ptr(packed), _stream(stream)))
    return packed


def nvfp4_unpack_weight(kind, packed, R, C, stream=None):
    codes = torch.empty((R, C // 2), dtype=torch.uint8, device=packed.device)
    scales = torch.empty((R, C // 16), dtype=torch.uint8, device=packed.device)
    _check("nvfp4_unpack_weight", lib().nvfp4_unpack_weight(int(kind), _ptr(packed), R, C, _ptr(codes),
                                                            _ptr(scales), _stream(stream)))
    return codes, scales


def nvfp4_gemm(mode, a, a_scales, w_packed, N, K, alpha, out=None, out_dtype=torch.float32,
               stream=None):
    """out [M, N] = alpha * A @ W^T. W4A4: a = codes [M, K/2] + a_scales; W4A16: a = bf16 [M, K]."""
    _dense(a, "a")
    M = a.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _check("nvfp4_gemm", lib().nvfp4_gemm(int(mode), _ptr(a), _ptr(a_scales), _ptr(w_packed), M, N, K,
                                          _ptr(alpha), _ptr(out), _dtype_code(out.dtype),
                                          _stream(stream)))
    return out


def gemm_swiglu_nvfp4_quant(a_codes, a_scales, w_gu_packed, I, K, alpha, g2_inv, h_codes=None,
                            h_scales=None, stream=None):
    """Fused gate_up GEMM + SiLU(gate)*up + NVFP4 quantize -> (h_codes, h_scales)."""
    _dense(a_codes, "a_codes")
    M = a_codes.shape[0]
    if h_codes is None:
        h_codes = torch.empty((M, I // 2), dtype=torch.uint8, device=a_codes.device)
    if h_scales is None:
        h_scales = torch.empty((M, I // 16), dtype=torch.uint8, device=a_codes.device)
    _check("gemm_swiglu_nvfp4_quant",
           lib().gemm_swiglu_nvfp4_quant(_ptr(a_codes), _ptr(a_scales), _ptr(w_gu_packed), M, I, K,
                                         _ptr(alpha), _ptr(g2_inv), _ptr(h_codes), _ptr(h_scales),
                                         _stream(stream)))
    return h_codes, h_scales


def nvfp4_gemm_rowscale(a_codes, a_scales, row_g, w_packed, N, K, g_w, out=None,
                        out_dtype=torch.float32, stream=None):
    """W4A4 out [M, N] = g_w * row_g[t] * (A @ W^T) with per-token activation scales."""
    _dense(a_codes, "a_codes")
    M = a_codes.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_codes.device)
    _check("nvfp4_gemm_rowscale",
           lib().nvfp4_gemm_rowscale(_ptr(a_codes), _ptr(a_scales), _ptr(row_g), _ptr(w_packed), M, N, K,
                                     _ptr(g_w), _ptr(out), _dtype_code(out.dtype), _stream(stream)))
    return out


def gemm_swiglu_nvfp4_quant_rowscale(a_codes, a_scales, row_g, w_gu_packed, I, K, g_w, g2_inv,
                                     h_codes=None, h_scales=None, stream=None):
    """gemm_swiglu_nvfp4_quant with per-token activation scales row_g."""
    _dense(a_codes, "a_codes")
    M = a_codes.shape[0]
    if h_codes is None:
        h_codes = torch.empty((M, I // 2), dtype=torch.uint8, device=a_codes.device)
    if h_scales is None:
        h_scales = torch.empty((M, I // 16), dtype=torch.uint8, device=a_codes.device)
    _check("gemm_swiglu_nvfp4_quant_rowscale",
           lib().gemm_swiglu_nvfp4_quant_rowscale(_ptr(a_codes), _ptr(a_scales), _ptr(row_g), _ptr(w_gu_packed),
                                                  M, I, K, _ptr(g_w), _ptr(g2_inv), _ptr(h_codes),
                                                  _ptr(h_scales), _stream(stream)))
    return h_codes, h_scales


def gemm_swiglu(mode, a, a_scales, w_gu_packed, I, K, alpha, h=None, h_dtype=torch.bfloat16,
                stream=None):
    """gate_up GEMM + SiLU(gate)*up -> h [M, I] (bf16 or f32)."""
    _dense(a, "a")
    M = a.shape[0]
    if h is None:
        h = torch.empty((M, I), dtype=h_dtype, device=a.device)
    _check("gemm_swiglu", lib().gemm_swiglu(int(mode), _ptr(a), _ptr(a_scales), _ptr(w_gu_packed), M, I, K,
                                            _ptr(alpha), _ptr(h), _dtype_code(h.dtype), _stream(stream)))
    return h


def silu_mul_nvfp4_quant(gate_up, g_inv, masked_m=None, codes=None, scales=None, stream=None):
    """gate_up bf16 [E, M, 2I] (or [M, 2I] as one expert) -> (codes [E, M, I/2],
    scales [E, M, I/16]) of SiLU(gate) * up, expert e quantized with g_inv[e];
    rows t >= masked_m[e] (int32 device tensor [E]) are not written."""
    _dense(gate_up, "gate_up")
    gu = gate_up if gate_up.dim() == 3 else gate_up.unsqueeze(0)
    E, M, I2 = gu.shape
    I = I2 // 2
    if codes is None:
        codes = torch.zeros((E, M, I // 2), dtype=torch.uint8, device=gu.device)
    if scales is None:
        scales = torch.zeros((E, M, I // 16), dtype=torch.uint8, device=gu.device)
    _check("silu_mul_nvfp4_quant",
           lib().silu_mul_nvfp4_quant(_ptr(gu), E, M, I, _ptr(masked_m), _ptr(g_inv), _ptr(codes), _ptr(scales),
                                      _stream(stream)))
    return codes, scales


def mlp_workspace_bytes(mode, M, H, I) -> int:
    return int(lib().mlp_workspace_bytes(int(mode), int(M), int(H), int(I)))


STATUS_DECODE_WAIT_EXPIRED = 1


def mlp_workspace_status(ws):
    """The workspace's status word as a 1-element int32 view of ws (its last
    4 bytes, the address the library computes)."""
    n = ws.numel() * ws.element_size()
    addr = lib().mlp_workspace_status(_ptr(ws), n)
    if not addr:
        raise ValueError("workspace too small for a status word")
    off = addr - ws.data_ptr()
    return ws.view(torch.uint8)[off:off + 4].view(torch.int32)


def set_decode_wait_test(withhold: bool, spin_limit: int = 0):
    """Test hook: the calling thread's single-launch decodes withhold their
    records, so every bounded wait gives up after spin_limit polls."""
    _check("nvfp4_set_decode_wait_test", lib().nvfp4_set_decode_wait_test(int(bool(withhold)), int(spin_limit)))


def mlp_forward(mode, x, w_gu_packed, alpha_gu, w_d_packed, alpha_d, I, g1_inv=None, g2_inv=None,
                ws=None, out=None, out_dtype=torch.float32, stream=None):
    """Dense MLP forward: x bf16 [M, H] -> out [M, H]."""
    _dense(x, "x")
    M, H = x.shape
    nws = mlp_workspace_bytes(mode, M, H, I)
    if ws is None:
        ws = torch.zeros(max(nws, 1), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((M, H), dtype=out_dtype, device=x.device)
    _check("mlp_forward", lib().mlp_forward(int(mode), _ptr(x), M, H, I, _ptr(w_gu_packed), _ptr(alpha_gu),
                                            _ptr(w_d_packed), _ptr(alpha_d), _ptr(g1_inv), _ptr(g2_inv),
                                            _ptr(ws), ws.numel() * ws.element_size(), _ptr(out),
                                            _dtype_code(out.dtype), _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20


def mlp_forward_noalloc(mode, x, w_gu_packed, alpha_gu, w_d_packed, alpha_d, I, g1_inv=None, g2_inv=None,
                        out=None, out_dtype=torch.float32, stream=None):
    """mlp_forward on the library's own per-GPU scratch (no workspace
    argument; the library allocates nothing). Pass `out` to allocate nothing
    here either. Calls that overlap on one GPU race."""
    _dense(x, "x")
    M, H = x.shape
    if out is None:
        out = torch.empty((M, H), dtype=out_dtype, device=x.device)
    _check("mlp_forward_noalloc",
           lib().mlp_forward_noalloc(int(mode), _ptr(x), M, H, I, _ptr(w_gu_packed), _ptr(alpha_gu), _ptr(w_d_packed),
                                     _ptr(alpha_d), _ptr(g1_inv), _ptr(g2_inv), _ptr(out), _dtype_code(out.dtype),
                                     _stream(stream)))
    return out


def nvfp4_prescale_bf16(x, s, out=None, stream=None):
    """AWQ pre-quant scaling: bf16(x * s) per input channel; x bf16 [M, K], s bf16 [K]."""
    _dense(x, "x"); _dense(s, "s")
    M, K = x.shape
    if out is None:
        out = torch.empty_like(x)
    _check("nvfp4_prescale_bf16", lib().nvfp4_prescale_bf16(_ptr(x), _ptr(s), M, K, _ptr(out), _stream(stream)))
    return out


def mlp_forward_w4a16_awq(x, w_gu_packed, g_gu, s_gu, w_d_packed, g_d, s_d, I, ws=None, out=None,
                          out_dtype=torch.float32, stream=None):
    """W4A16 MLP forward with AWQ pre-quant scales s_gu [H] and s_d [I] (bf16)."""
    _dense(x, "x")
    M, H = x.shape
    nws = mlp_workspace_bytes(MODE_W4A16_AWQ, M, H, I)
    if ws is None:
        ws = torch.zeros(max(nws, 1), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((M, H), dtype=out_dtype, device=x.device)
    _check("mlp_forward_w4a16_awq",
           lib().mlp_forward_w4a16_awq(_ptr(x), M, H, I, _ptr(w_gu_packed), _ptr(g_gu), _ptr(s_gu), _ptr(w_d_packed),
                                       _ptr(g_d), _ptr(s_d), _ptr(ws), ws.numel() * ws.element_size(), _ptr(out),
                                       _dtype_code(out.dtype), _stream(stream)))
    return out


def nvfp4_grouped_gemm(mode, a, a_scales, w_packed, N, K, alpha, masked_m=None, out=None, out_dtype=torch.float32,
                       stream=None):
    """Grouped (expert) GEMM: a [E, M, K/2] codes (+ a_scales [E, M, K/16]) or
    bf16 [E, M, K]; w_packed: E packed [N, K] weights back to back; alpha [E];
    masked_m int32 [E] or None. Returns out [E, M, N] (rows past masked_m
    keep what out held)."""
    _dense(a, "a")
    E, M = a.shape[0], a.shape[1]
    if out is None:
        out = torch.empty((E, M, N), dtype=out_dtype, device=a.device)
    _check("nvfp4_grouped_gemm",
           lib().nvfp4_grouped_gemm(int(mode), _ptr(a), _ptr(a_scales), _ptr(w_packed), E, M, N, K, _ptr(masked_m),
                                    _ptr(alpha), _ptr(out), _dtype_code(out.dtype), _stream(stream)))
    return out
