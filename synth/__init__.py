"""Seeded synthetic inputs for the tests and the benchmark.

Both the CPU oracle and the GPU library receive tensors made here; this package holds
none of their arithmetic.  Values come from ``synth_gen.h`` (integer-only, identical on
the host and on the device), so any slice of a workload can be regenerated on the CPU
for the oracle while the full workload is generated on the GPU.

Workload recipe (Llama-3.1-8B and Qwen2.5-7B shaped caches):
  * K, V, q: Irwin-Hall(12) approximations of N(0, 1), bf16 (round to nearest even) or
    binary32, one stream per (seed, tensor kind, layer).
  * outlier key channels: a seeded partial Fisher-Yates picks ``n_outliers`` of the 128
    channels per (layer, KV head); those channels are multiplied by 10 before rounding.
  * ragged lengths: L_i = lo + mix64(...) mod (hi - lo + 1).
  * paged layout: a seeded Fisher-Yates permutation of the physical page ids.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
CPU_LIB = os.path.join(_HERE, "libkvq_synth_cpu.so")
HIP_LIB = os.path.join(_HERE, "libkvq_synth_hip.so")

KIND_K, KIND_V, KIND_Q, KIND_K_NEW, KIND_V_NEW = 1, 2, 3, 4, 5
HEAD_DIM = 128
_M64 = (1 << 64) - 1
_GOLDEN = 0x9E3779B97F4A7C15


def build(hip: bool = True) -> None:
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", CPU_LIB + ".tmp",
                    os.path.join(_HERE, "synth_cpu.c")], check=True)
    os.replace(CPU_LIB + ".tmp", CPU_LIB)
    if hip:
        subprocess.run(["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-o", HIP_LIB + ".tmp", os.path.join(_HERE, "synth_hip.hip")],
                       check=True, stderr=subprocess.DEVNULL)
        os.replace(HIP_LIB + ".tmp", HIP_LIB)


_cpu = None
_hip = None


def _cpu_lib():
    global _cpu
    if _cpu is None:
        if not os.path.exists(CPU_LIB):
            build(hip=False)
        _cpu = ctypes.CDLL(CPU_LIB)
        _cpu.sg_fill_cpu.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32] + \
            [ctypes.c_int] * 7 + [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        _cpu.sg_fill_cpu.restype = ctypes.c_int
    return _cpu


def _hip_lib():
    global _hip
    if _hip is None:
        if not os.path.exists(HIP_LIB):
            raise RuntimeError(f"{HIP_LIB} is not built; run __graft_entry__.build()")
        _hip = ctypes.CDLL(HIP_LIB)
        _hip.sg_fill_hip.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32] + \
            [ctypes.c_int] * 7 + [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        _hip.sg_fill_hip.restype = ctypes.c_int
    return _hip


def mix64(z: int) -> int:
    z &= _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def _key(seed: int, kind: int, layer: int) -> int:
    return mix64(seed ^ mix64(((kind & 0xFFFFFFFF) << 32) | (layer & 0xFFFFFFFF)))


def outlier_channels(seed: int, layer: int, head: int, n_outliers: int, head_dim: int = HEAD_DIM):
    """Seeded partial Fisher-Yates: the first n_outliers entries of a shuffled channel list."""
    key = _key(seed, 0x0071, layer * 4096 + head)
    perm = list(range(head_dim))
    for i in range(n_outliers):
        j = i + mix64(key + i * _GOLDEN) % (head_dim - i)
        perm[i], perm[j] = perm[j], perm[i]
    return sorted(perm[:n_outliers])


def outlier_mult(seed: int, layer: int, n_heads: int, n_outliers: int, factor: float = 10.0,
                 head_dim: int = HEAD_DIM) -> np.ndarray:
    m = np.ones((n_heads, head_dim), dtype=np.float32)
    for h in range(n_heads):
        m[h, outlier_channels(seed, layer, h, n_outliers, head_dim)] = factor
    return m


def seq_lens(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    key = _key(seed, 0x0051, 0)
    return np.array([lo + mix64(key + i * _GOLDEN) % (hi - lo + 1) for i in range(batch)],
                    dtype=np.int32)


def permutation(seed: int, n: int) -> np.ndarray:
    key = _key(seed, 0x0052, 0)
    p = np.arange(n, dtype=np.int32)
    for i in range(n - 1, 0, -1):
        j = mix64(key + i * _GOLDEN) % (i + 1)
        p[i], p[j] = p[j], p[i]
    return p


def fill(seed: int, kind: int, layer: int, nB: int, nT: int, nH: int, *, b0: int = 0, t0: int = 0,
         h0: int = 0, chan_mult=None, dtype: str = "bf16", device="cpu", out=None):
    """Tensor [nB][nT][nH][128] of elements (b0+ib, t0+it, h0+ih, c).

    dtype "bf16" returns torch.bfloat16, "f32" torch.float32.  device "cpu" runs the host
    generator; a CUDA device runs the HIP generator on the current stream.  chan_mult is a
    numpy [H][128] multiplier (outlier channels) or None."""
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = torch.device(device)
    if out is None:
        out = torch.empty((nB, nT, nH, HEAD_DIM), dtype=tdt, device=dev)
    assert out.is_contiguous() and out.dtype == tdt and tuple(out.shape) == (nB, nT, nH, HEAD_DIM)
    if out.numel() == 0:
        return out
    if dev.type == "cpu":
        cm = None if chan_mult is None else np.ascontiguousarray(chan_mult, dtype=np.float32)
        rc = _cpu_lib().sg_fill_cpu(seed, kind, layer, nB, nT, nH, HEAD_DIM, b0, t0, h0,
                                    None if cm is None else cm.ctypes.data,
                                    int(dtype == "bf16"), out.data_ptr())
    else:
        cm = None if chan_mult is None else torch.from_numpy(
            np.ascontiguousarray(chan_mult, dtype=np.float32)).to(dev)
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = _hip_lib().sg_fill_hip(seed, kind, layer, nB, nT, nH, HEAD_DIM, b0, t0, h0,
                                    None if cm is None else cm.data_ptr(), int(dtype == "bf16"),
                                    out.data_ptr(), stream)
        if cm is not None:
            # keep the multiplier alive until the kernel has read it
            torch.cuda.current_stream(dev).synchronize()
    if rc != 0:
        raise RuntimeError(f"synthetic generator failed (code {rc})")
    return out
