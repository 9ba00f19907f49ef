"""The C-ABI library on the CPU: it loads, exports every function that
include/nvfp4.h declares, and rejects bad arguments before any HIP call
(these calls never reach a device, so they run without a GPU)."""
import ctypes
import os
import re

import pytest

import nvfp4_quantized_dense_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "nvfp4.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|size_t|uint32_t|char\s*\*|const char\s*\*)\s*\**\s*"
                                 r"([a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["nvfp4_quantize", "nvfp4_gemm", "gemm_swiglu_nvfp4_quant", "mlp_forward",
              "nvfp4_repack_weight", "nvfp4_repack_bytes", "nvfp4_packed_bytes", "nvfp4_last_error",
              "mlp_workspace_bytes", "mlp_workspace_status"]:
        assert n in names, names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(nv.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(declared_functions()) == set(nv.SIGNATURES)


def test_packed_and_workspace_sizes():
    assert nv.nvfp4_packed_bytes(nv.REPACK_PLAIN, 5120, 17408) == 5120 * 17408 * 9 // 16
    assert nv.nvfp4_packed_bytes(nv.REPACK_SWIGLU, 2 * 17408, 5120) == 2 * 17408 * 5120 * 9 // 16
    assert nv.nvfp4_packed_bytes(nv.REPACK_PLAIN, 24, 256) == 0       # rows % 16
    assert nv.nvfp4_packed_bytes(nv.REPACK_PLAIN, 16, 128) == 0       # cols % 256
    assert nv.nvfp4_packed_bytes(nv.REPACK_SWIGLU, 48, 256) == 0      # half not % 16
    assert nv.nvfp4_packed_bytes(7, 16, 256) == 0
    assert nv.nvfp4_repack_bytes(nv.REPACK_PLAIN, 5120, 17408) == 5120 * 17408 * 9 // 16

    def tail(H, I):
        # the same 4 MiB for every shape: the status word and the
        # single-launch decode's records (3 words per 16 elements of h, 8
        # splits x 16-row partials: 354 KB at hidden 5120)
        words = 3 * I // 16 + 8 * H
        assert 512 + words * 8 <= 4 << 20
        return 4 << 20

    w = nv.mlp_workspace_bytes(nv.MODE_W4A4, 1, 5120, 17408)
    # x 2560 + 320 -> 512, h 8704 -> 8960, 1088 -> 1280, then the largest
    # split-K plan over the paths, then the tail
    assert w >= 2560 + 512 + 8960 + 1280 + tail(5120, 17408) and w % 256 == 0
    assert nv.mlp_workspace_bytes(nv.MODE_W4A16, 4, 256, 512) == 4 * 512 * 2 + tail(256, 512)
    assert nv.mlp_workspace_bytes(9, 1, 256, 512) == 0
    # W4A4_DYN: the W4A4 activations, then one fp32 g per token
    # x codes 512, x scales 64 -> 256, h codes 1024, h scales 128 -> 256, g 16 -> 256
    assert nv.mlp_workspace_bytes(nv.MODE_W4A4_DYN, 4, 256, 512) == 512 + 256 + 1024 + 256 + 256 + tail(256, 512)
    assert nv.mlp_workspace_bytes(nv.MODE_W4A4_DYN, 1000, 256, 512) >= \
        nv.mlp_workspace_bytes(nv.MODE_W4A4, 1000, 256, 512) + 4000
    # the tail comes after everything a call of any token count writes, so a
    # buffer sized for many tokens holds the same tail at its end
    for M in (1, 16, 256, 4096):
        for mode in (nv.MODE_W4A4, nv.MODE_W4A16, nv.MODE_W4A4_DYN, nv.MODE_W4A16_AWQ):
            assert nv.mlp_workspace_bytes(mode, M, 7168, 18432) >= tail(7168, 18432) + M * 7168 // 2


def test_workspace_holds_split_down_partials():
    """The forward's workspace holds the K-split partial tiles and counters of
    its down projection on the mid-size kernels (host sizing only). Restated
    plan: tiles of 128 rows x 48, 64 or (one-expert W4A4 dense grids of more
    than 256 such tiles) 128 tokens; splits = min(8, 512 / tiles), reduced
    until every split is non-empty and at least 8 K tiles long; a partial
    tile is 256 threads x 2 row groups x TG token groups x 4 floats."""
    def a256(v):
        return (v + 255) // 256 * 256

    def split_bytes(mode, M, H, I):
        tg = 3 if (M + 47) // 48 * 48 <= (M + 63) // 64 * 64 else 4
        rows = (H // 16 + 7) // 8
        if mode == nv.MODE_W4A4 and rows * -(-M // (16 * tg)) > 256:
            tg = 8
        units, T = rows * -(-M // (16 * tg)), I // 256
        ks = min(2 * 256 // units, 8)
        while ks > 1 and ((ks - 1) * -(-T // ks) >= T or -(-T // ks) < 8):
            ks -= 1
        return 0 if ks < 2 else a256(units * ks * 2048 * tg * 4) + a256(units * 4)

    for mode in (nv.MODE_W4A4, nv.MODE_W4A16):
        for M, H, I in [(17, 7168, 18432), (64, 7168, 18432), (128, 5120, 17408), (300, 7168, 18432),
                        (384, 5120, 17408), (100, 2048, 6400)]:
            act = (a256(M * H // 2) + a256(M * H // 16) + a256(M * I // 2) + a256(M * I // 16)
                   if mode == nv.MODE_W4A4 else a256(M * I * 2))
            need = act + split_bytes(mode, M, H, I) + (4 << 20)
            assert nv.mlp_workspace_bytes(mode, M, H, I) >= need, (mode, M, H, I)
    # the 8-way split of 56 tiles at 64 tokens, hidden 7168: 14.7 MB of partials
    assert split_bytes(nv.MODE_W4A4, 64, 7168, 18432) == a256(56 * 8 * 8192 * 4) + a256(56 * 4)


def test_workspace_status_address():
    lib = nv.lib()
    base = 0x7F0000000000
    for n in (512, 4096, 4099, 1 << 20):
        a = lib.mlp_workspace_status(ctypes.c_void_p(base), n)
        assert a == (base + n - 4) & ~3
    assert lib.mlp_workspace_status(ctypes.c_void_p(base), 511) is None
    assert lib.mlp_workspace_status(None, 4096) is None


def test_noalloc_rejects_on_the_host():
    """The allocation-free forward checks its arguments and its size limit
    before any HIP call."""
    lib = nv.lib()
    P = ctypes.c_void_p(0x100000)
    N = None
    INV = nv.NVFP4_ERR_INVALID_ARG
    # prefill at hidden 7168 needs far more than the 64 MiB scratch
    assert lib.mlp_forward_noalloc(0, P, 8192, 7168, 18432, P, P, P, P, P, P, P, 1, N) == INV
    assert b"scratch" in lib.nvfp4_last_error()
    assert lib.mlp_forward_noalloc(1, P, 4096, 5120, 17408, P, P, P, P, N, N, P, 1, N) == INV
    assert lib.mlp_forward_noalloc(0, N, 1, 256, 512, P, P, P, P, P, P, P, 1, N) == INV   # null x
    assert lib.mlp_forward_noalloc(3, P, 1, 256, 512, P, P, P, P, N, N, P, 1, N) == INV   # AWQ
    assert lib.mlp_forward_noalloc(0, P, 1, 250, 512, P, P, P, P, P, P, P, 1, N) == INV   # H % 256
    assert lib.mlp_forward_noalloc(0, P, 0, 256, 512, N, N, N, N, N, N, N, 1, N) == nv.NVFP4_OK  # empty


def test_decode_wait_test_hook_arguments():
    lib = nv.lib()
    assert lib.nvfp4_set_decode_wait_test(1, 0) == nv.NVFP4_ERR_INVALID_ARG
    assert lib.nvfp4_set_decode_wait_test(1, 16) == nv.NVFP4_OK
    assert lib.nvfp4_set_decode_wait_test(0, 0) == nv.NVFP4_OK


def test_path_override_is_per_thread():
    import threading
    assert nv.set_path(nv.PATH_TILED64) == nv.PATH_AUTO
    seen = []
    t = threading.Thread(target=lambda: seen.append(nv.set_path(nv.PATH_AUTO)))
    t.start()
    t.join()
    assert seen == [nv.PATH_AUTO]           # another thread starts at AUTO
    assert nv.set_path(nv.PATH_AUTO) == nv.PATH_TILED64
    assert nv.lib().nvfp4_set_path(6) == nv.NVFP4_ERR_INVALID_ARG


def _code(fn, *args):
    return fn(*args)


def test_invalid_arguments_are_rejected_on_the_host():
    lib = nv.lib()
    P = ctypes.c_void_p(0x100000)  # 16-byte aligned, never dereferenced
    U = ctypes.c_void_p(0x100001)  # misaligned
    N = None
    INV = nv.NVFP4_ERR_INVALID_ARG
    assert lib.nvfp4_quantize(P, 7, 4, 256, P, P, P, N) == INV                 # dtype
    assert lib.nvfp4_quantize(P, 0, 4, 250, P, P, P, N) == INV                 # K % 16
    assert lib.nvfp4_quantize(N, 0, 4, 256, P, P, P, N) == INV                 # null x
    assert lib.nvfp4_quantize(U, 0, 4, 256, P, P, P, N) == INV                 # misaligned
    assert b"aligned" in lib.nvfp4_last_error()
    assert lib.nvfp4_quantize(N, 0, 0, 256, N, N, N, N) == nv.NVFP4_OK         # empty: no-op
    assert lib.nvfp4_quantize(P, 0, (1 << 24) + 1, 16, P, P, P, N) == INV      # M > 2^24
    assert b"2^24" in lib.nvfp4_last_error()
    assert lib.nvfp4_quantize(P, 0, 1, (1 << 30) + 16, P, P, P, N) == INV     # K > 2^30
    assert lib.nvfp4_gemm(3, P, P, P, 4, 16, 256, P, P, 1, N) == INV           # mode
    assert b"mode" in lib.nvfp4_last_error()
    assert lib.nvfp4_gemm(0, P, P, P, 4, 16, 200, P, P, 1, N) == INV           # K % 256
    assert lib.nvfp4_gemm(0, P, P, P, 4, 24, 256, P, P, 1, N) == INV           # N % 16
    assert lib.nvfp4_gemm(0, P, N, P, 4, 16, 256, P, P, 1, N) == INV           # W4A4 needs scales
    assert lib.nvfp4_gemm(1, P, P, P, 4, 16, 256, P, P, 1, N) == INV           # W4A16 takes none
    assert lib.nvfp4_gemm(0, P, P, P, 4, 16, 256, P, P, 5, N) == INV           # out dtype
    assert lib.nvfp4_gemm(0, P, P, P, -1, 16, 256, P, P, 1, N) == INV          # negative M
    assert lib.nvfp4_gemm(0, P, P, P, 0, 16, 256, P, P, 1, N) == nv.NVFP4_OK   # M = 0: no-op
    assert lib.gemm_swiglu_nvfp4_quant(P, P, P, 4, 24, 256, P, P, P, P, N) == INV  # I % 16
    assert lib.gemm_swiglu_nvfp4_quant(P, P, P, 4, 32, 256, P, N, P, P, N) == INV  # null g2_inv
    assert lib.gemm_swiglu(0, P, P, P, 4, 32, 256, P, P, 3, N) == INV          # h dtype
    assert lib.nvfp4_repack_weight(0, P, P, 17, 256, P, N) == INV              # rows
    assert lib.nvfp4_unpack_weight(1, P, 48, 256, P, P, N) == INV              # swiglu half
    assert lib.nvfp4_calibrate(P, 0, 0, P, P, N) == INV                        # n
    assert lib.nvfp4_calibrate(P, 0, 16, P, P, N) == INV                       # g == g_inv
    ws = ctypes.c_size_t(1 << 20)
    assert lib.mlp_forward(0, P, 4, 256, 500, P, P, P, P, P, P, P, ws, P, 1, N) == INV  # I % 256
    assert lib.mlp_forward(1, P, 4, 256, 512, P, P, P, P, P, N, P, ws, P, 1, N) == INV  # W4A16 + g1
    assert lib.mlp_forward(0, P, 4, 256, 512, P, P, P, P, N, P, P, ws, P, 1, N) == INV  # W4A4 no g1
    assert lib.mlp_forward(0, P, 4, 256, 512, P, P, P, P, P, P, P, ctypes.c_size_t(16), P, 1, N) == INV
    assert b"workspace" in lib.nvfp4_last_error()
    # per-token dynamic scales
    assert lib.nvfp4_quantize_per_token(P, 0, 4, 250, P, P, P, N) == INV       # K % 16
    assert lib.nvfp4_quantize_per_token(P, 0, 4, 256, P, P, N, N) == INV       # null row_g
    assert lib.nvfp4_quantize_per_token(P, 0, 4, 256, P, P, ctypes.c_void_p(0x100002), N) == INV
    assert lib.nvfp4_quantize_per_token(N, 0, 0, 256, N, N, N, N) == nv.NVFP4_OK  # empty
    assert lib.nvfp4_gemm_rowscale(P, P, N, P, 4, 16, 256, P, P, 1, N) == INV   # null row_g
    assert lib.nvfp4_gemm_rowscale(P, P, P, P, 4, 16, 200, P, P, 1, N) == INV   # K % 256
    assert lib.nvfp4_gemm_rowscale(N, N, N, P, 0, 16, 256, P, P, 1, N) == nv.NVFP4_OK
    assert lib.gemm_swiglu_nvfp4_quant_rowscale(P, P, N, P, 4, 32, 256, P, P, P, P, N) == INV
    assert lib.gemm_swiglu_nvfp4_quant_rowscale(P, P, P, P, 4, 24, 256, P, P, P, P, N) == INV
    assert lib.mlp_forward(2, P, 4, 256, 512, P, P, P, P, P, P, P, ws, P, 1, N) == INV  # DYN + g1
    assert b"per token" in lib.nvfp4_last_error()
    assert lib.mlp_forward(2, P, 4, 256, 512, P, P, P, P, N, N, P, ws, P, 1, N) == INV  # DYN no g2
    # standalone SiLU * mul + NVFP4 quantize
    assert lib.silu_mul_nvfp4_quant(P, 1, 4, 24, N, P, P, P, N) == INV        # I % 16
    assert lib.silu_mul_nvfp4_quant(P, 1, 70000, 32, N, P, P, P, N) == INV    # M too large
    assert lib.silu_mul_nvfp4_quant(P, 1, 4, 32, N, N, P, P, N) == INV        # null g_inv
    assert lib.silu_mul_nvfp4_quant(U, 1, 4, 32, N, P, P, P, N) == INV        # misaligned gate_up
    assert lib.silu_mul_nvfp4_quant(N, 0, 4, 32, N, N, N, N, N) == nv.NVFP4_OK  # empty
    # AWQ pre-quant scales
    assert lib.nvfp4_prescale_bf16(P, P, 4, 12, P, N) == INV                  # K % 8
    assert lib.nvfp4_prescale_bf16(P, N, 4, 16, P, N) == INV                  # null s
    assert lib.nvfp4_prescale_bf16(P, U, 4, 16, P, N) == INV                  # misaligned s
    assert lib.nvfp4_prescale_bf16(N, N, 0, 16, N, N) == nv.NVFP4_OK          # empty
    assert lib.mlp_forward_w4a16_awq(P, 4, 256, 512, P, P, N, P, P, P, P, ws, P, 1, N) == INV  # null s_gu
    assert lib.mlp_forward_w4a16_awq(P, 4, 256, 512, P, P, P, P, P, U, P, ws, P, 1, N) == INV  # misaligned s_d
    assert lib.mlp_forward(3, P, 4, 256, 512, P, P, P, P, N, N, P, ws, P, 1, N) == INV  # AWQ through mlp_forward
    assert nv.mlp_workspace_bytes(nv.MODE_W4A16_AWQ, 4, 256, 512) == \
        nv.mlp_workspace_bytes(nv.MODE_W4A16, 4, 256, 512) + 4 * 256 * 2
    # grouped GEMM
    assert lib.nvfp4_grouped_gemm(0, P, P, P, 2, 4, 24, 256, N, P, P, 1, N) == INV   # N % 16
    assert lib.nvfp4_grouped_gemm(0, P, N, P, 2, 4, 32, 256, N, P, P, 1, N) == INV   # W4A4 needs scales
    assert lib.nvfp4_grouped_gemm(1, P, N, P, 2, 4, 32, 256, U, P, P, 1, N) == INV   # misaligned masked_m
    assert lib.nvfp4_grouped_gemm(0, P, P, P, -1, 4, 32, 256, N, P, P, 1, N) == INV  # E < 0
    assert lib.nvfp4_grouped_gemm(0, P, P, P, 65536, 4, 32, 256, N, P, P, 1, N) == INV  # E > 65535 (grid limit)
    assert lib.nvfp4_grouped_gemm(0, N, N, N, 0, 4, 32, 256, N, N, N, 1, N) == nv.NVFP4_OK  # no experts
    assert lib.nvfp4_set_path(9) == INV


def test_set_path_round_trip():
    prev = nv.set_path(nv.PATH_TILED)
    assert nv.set_path(prev) == nv.PATH_TILED


def test_python_binding_raises_with_the_message():
    import torch
    x = torch.zeros((4, 250), dtype=torch.bfloat16)
    with pytest.raises(nv.Nvfp4Error, match="multiple of 16"):
        nv.nvfp4_quantize(x, torch.ones(1))
