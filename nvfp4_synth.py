"""Seeded synthetic inputs for the NVFP4 dense MLP (shared by tests and bench).

This module only draws numbers; it holds none of the quantization or GEMM
arithmetic. Both the CPU oracle and the GPU library receive its outputs
byte for byte.

Generator (all counter-based, so any slice can be drawn on its own):
  * SplitMix64 (Steele, Lea & Flood, 2014): output i of stream `key` is
    mix(key + (i + 1) * 0x9E3779B97F4A7C15) with the usual two xor-shift-
    multiply rounds and a final xor-shift.
  * key = seed * 2**32 + tensor_id.
  * Uniforms u = (z >> 11) * 2**-53; a normal takes outputs 2n and 2n + 1:
    sqrt(-2 ln(1 - u1)) * cos(2 pi u2) (Box-Muller, cosine branch), in double.
  * Activations: N(0, 1) in double -> fp32 (round to nearest even) -> bf16
    (round to nearest even). With outliers, round(0.001 * M * H) positions,
    chosen as the smallest SplitMix64 keys of an outlier stream, are scaled by
    20 before rounding.
  * Weights: N(0, std) in double -> fp32 (round to nearest even).
"""
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)

TENSOR_X = 1
TENSOR_W_GATE_UP = 2
TENSOR_W_DOWN = 3
TENSOR_OUTLIERS = 4

_CHUNK = 1 << 22


def _key(seed: int, tensor_id: int) -> np.uint64:
    return np.uint64(((int(seed) << 32) + int(tensor_id)) & 0xFFFFFFFFFFFFFFFF)


def splitmix64(key: np.uint64, start: int, count: int) -> np.ndarray:
    """Outputs start .. start+count-1 of the stream `key` (uint64)."""
    with np.errstate(over="ignore"):
        i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = key + i * GOLDEN
        z = (z ^ (z >> np.uint64(30))) * M1
        z = (z ^ (z >> np.uint64(27))) * M2
        return z ^ (z >> np.uint64(31))


def _normals_chunk(key, start, count):
    z = splitmix64(key, 2 * start, 2 * count)
    u = (z >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
    u1 = 1.0 - u[0::2]
    u2 = u[1::2]
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def normals(key: np.uint64, n: int, threads: int = 0) -> np.ndarray:
    """n standard normals (float64) of stream `key`, drawn in chunks."""
    out = np.empty(n, np.float64)
    starts = list(range(0, n, _CHUNK))

    def work(s):
        c = min(_CHUNK, n - s)
        out[s:s + c] = _normals_chunk(key, s, c)

    threads = threads or min(8, os.cpu_count() or 1)
    if len(starts) > 1 and threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, starts))
    else:
        for s in starts:
            work(s)
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even (finite values)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def activations(seed: int, M: int, H: int, outliers: bool = False) -> np.ndarray:
    """bf16 activations [M, H] as uint16 bits, N(0,1) (+0.1% outliers x20)."""
    x = normals(_key(seed, TENSOR_X), M * H)
    if outliers:
        n_out = int(round(0.001 * M * H))
        if n_out:
            keys = splitmix64(_key(seed, TENSOR_OUTLIERS), 0, M * H)
            pos = np.argsort(keys, kind="stable")[:n_out]
            x[pos] *= 20.0
    return f32_to_bf16_bits(x.astype(np.float32)).reshape(M, H)


def weights(seed: int, R: int, C: int, tensor_id: int, std: float = 0.02) -> np.ndarray:
    """fp32 weights [R, C] ~ N(0, std)."""
    w = normals(_key(seed, tensor_id), R * C)
    w *= std
    return w.astype(np.float32).reshape(R, C)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


# Workload shapes: (name, M values, hidden H, intermediate I, mode, outliers).
WORKLOADS = {
    "tiny_w4a4": dict(M=[4], H=256, I=512, mode="w4a4", outliers=False),
    "decode_w4a4": dict(M=[1], H=5120, I=17408, mode="w4a4", outliers=True),
    "smallbatch_w4a4": dict(M=[1, 4, 16, 64], H=7168, I=18432, mode="w4a4", outliers=False),
    "prefill_w4a4": dict(M=[8192], H=7168, I=18432, mode="w4a4", outliers=False),
    "w4a16": dict(M=[1, 16, 256, 4096], H=5120, I=17408, mode="w4a16", outliers=False),
}
