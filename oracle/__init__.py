"""CPU reference ("oracle") for layer-wise mixed-precision KV-cache quantization.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` import this package.  The GPU library
(``layer_wise_mixed_kvq_amd``) never imports it, and the two share no code.

Two parts:

* ``kvq_oracle.c`` (loaded through ctypes): the group codec, the packed page
  layout, prefill packing, decode-time append and binary64 decode attention.
* the closed forms below: equivalent bit-width, page and cache byte accounting,
  and the throughput definition.  Each one says which passage it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from fractions import Fraction
from typing import Iterable, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB = os.path.join(_HERE, "libkvq_oracle.so")

HEAD_DIM = 128
GROUP = 32

# --------------------------------------------------------------------------------------
# build / load
# --------------------------------------------------------------------------------------


def build() -> str:
    """Compile the oracle with gcc: binary32 evaluation, no contraction, no fast-math."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
           "-fno-fast-math", "-fPIC", "-shared", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        i32p = ctypes.POINTER(ctypes.c_int32)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        vp = ctypes.c_void_p
        ci = ctypes.c_int
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f32.restype = ctypes.c_float
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_quant_group.argtypes = [f32p, ci, ci, u16p, u16p, u8p]
        L.orc_quant_group.restype = ci
        L.orc_head_page_bytes.argtypes = [ci, ci]
        L.orc_head_page_bytes.restype = ctypes.c_size_t
        L.orc_fp8_to_f32.argtypes = [ctypes.c_uint8]
        L.orc_fp8_to_f32.restype = ctypes.c_float
        L.orc_f32_to_fp8.argtypes = [ctypes.c_float]
        L.orc_f32_to_fp8.restype = ctypes.c_uint8
        L.orc_head_page_bytes_x.argtypes = [ci, ci, ci]
        L.orc_head_page_bytes_x.restype = ctypes.c_size_t
        L.orc_pack_page_x.argtypes = [f32p, f32p, ci, ci, ci, ci, ctypes.c_float, ctypes.c_float, u8p]
        L.orc_pack_page_x.restype = ci
        L.orc_dequant_page_x.argtypes = [u8p, ci, ci, ci, ctypes.c_float, ctypes.c_float, f64p, f64p]
        L.orc_dequant_page_x.restype = ci
        L.orc_pack_x.argtypes = [ci, ci, ci, f32p, ci, ci, ci, ci, vp, vp, i32p, i32p, ci, u8p, u16p, u16p]
        L.orc_pack_x.restype = ci
        L.orc_append_x.argtypes = [ci, ci, ci, f32p, ci, ci, u16p, u16p, i32p, i32p, ci, u8p, u16p, u16p]
        L.orc_append_x.restype = ci
        L.orc_decode_attn_x.argtypes = [ci, ci, ci, f32p, ci, ci, ci, ci, vp, i32p, i32p, ci, u8p, u16p, u16p,
                                        f64p, f64p]
        L.orc_decode_attn_x.restype = ci
        L.orc_pack_page_m.argtypes = [f32p, f32p, ci, ci, ci, ci, u8p]
        L.orc_pack_page_m.restype = ci
        L.orc_dequant_page_m.argtypes = [u8p, ci, ci, ci, f64p, f64p]
        L.orc_dequant_page_m.restype = ci
        L.orc_pack_m.argtypes = [ci, ci, ci, ci, ci, ci, ci, vp, vp, i32p, i32p, ci, u8p, u16p, u16p]
        L.orc_pack_m.restype = ci
        L.orc_append_m.argtypes = [ci, ci, ci, ci, ci, u16p, u16p, i32p, i32p, ci, u8p, u16p, u16p]
        L.orc_append_m.restype = ci
        L.orc_decode_attn_m.argtypes = [ci, ci, ci, ci, ci, ci, ci, vp, i32p, i32p, ci, u8p, u16p, u16p,
                                        f64p, f64p]
        L.orc_decode_attn_m.restype = ci
        _lib = L
    return _lib


def _ptr(a: np.ndarray, ctype):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


# --------------------------------------------------------------------------------------
# scalar conversions and the group codec
# --------------------------------------------------------------------------------------


def f32_to_f16_bits(x: float) -> int:
    return int(lib().orc_f32_to_f16(float(np.float32(x))))


def f16_bits_to_f32(h: int) -> float:
    return float(lib().orc_f16_to_f32(int(h)))


def f32_to_bf16_bits(x: float) -> int:
    return int(lib().orc_f32_to_bf16(float(np.float32(x))))


def bf16_bits_to_f32(b: int) -> float:
    return float(lib().orc_bf16_to_f32(int(b)))


def quant_group(x: Sequence[float], bits: int):
    """One 32-element group -> (s16 bits, z16 bits, codes[32] uint8)."""
    xs = np.ascontiguousarray(np.asarray(x, dtype=np.float32).reshape(GROUP))
    s16 = ctypes.c_uint16()
    z16 = ctypes.c_uint16()
    codes = np.zeros(GROUP, dtype=np.uint8)
    _check(lib().orc_quant_group(_ptr(xs, ctypes.c_float), 1, bits, ctypes.byref(s16),
                                 ctypes.byref(z16), _ptr(codes, ctypes.c_uint8)), "quant_group")
    return int(s16.value), int(z16.value), codes


def head_page_bytes(kb: int, vb: int) -> int:
    return int(lib().orc_head_page_bytes(kb, vb))


# layer formats: integer codes with per-channel keys / per-token keys, OCP FP8 E4M3 with
# per-head scales (kb = vb = 8), BF16 (kb = vb = 16)
KMODE_CHANNEL, KMODE_TOKEN, FMT_FP8, FMT_BF16 = 0, 1, 2, 3


def fp8_to_f32(b: int) -> float:
    return float(lib().orc_fp8_to_f32(b))


def f32_to_fp8(x: float) -> int:
    return int(lib().orc_f32_to_fp8(x))


def head_page_bytes_fmt(kb: int, vb: int, fmt: int) -> int:
    return int(lib().orc_head_page_bytes_x(kb, vb, fmt))


def pack_page(k_tile: np.ndarray, v_tile: np.ndarray, kb: int, vb: int, kmode: int = KMODE_CHANNEL,
              ks: float = 1.0, vs: float = 1.0) -> np.ndarray:
    """Quantize one 32x128 fp32 K tile and V tile into one packed page (uint8); kmode is
    the layer format (KMODE_* / FMT_*), ks / vs the FP8 scales."""
    k = np.ascontiguousarray(k_tile, dtype=np.float32).reshape(GROUP, HEAD_DIM)
    v = np.ascontiguousarray(v_tile, dtype=np.float32).reshape(GROUP, HEAD_DIM)
    out = np.zeros(head_page_bytes_fmt(kb, vb, kmode), dtype=np.uint8)
    _check(lib().orc_pack_page_x(_ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float), HEAD_DIM, kb, vb, kmode,
                                 ks, vs, _ptr(out, ctypes.c_uint8)), "pack_page")
    return out


def dequant_page(page: np.ndarray, kb: int, vb: int, kmode: int = KMODE_CHANNEL, ks: float = 1.0,
                 vs: float = 1.0):
    """Packed page -> (K, V) float64 [32][128]."""
    p = np.ascontiguousarray(page, dtype=np.uint8)
    k = np.zeros((GROUP, HEAD_DIM), dtype=np.float64)
    v = np.zeros((GROUP, HEAD_DIM), dtype=np.float64)
    _check(lib().orc_dequant_page_x(_ptr(p, ctypes.c_uint8), kb, vb, kmode, ks, vs, _ptr(k, ctypes.c_double),
                                    _ptr(v, ctypes.c_double)), "dequant_page")
    return k, v


def _scales_ptr(scales, H):
    if scales is None:
        return None, None
    a = np.ascontiguousarray(scales, dtype=np.float32).reshape(H, 2)
    return a, _ptr(a, ctypes.c_float)


# --------------------------------------------------------------------------------------
# layer-level operations (host numpy arrays in the library's layouts)
# --------------------------------------------------------------------------------------


def _src_kind(a: np.ndarray) -> int:
    """1 for raw bf16 bit patterns (uint16), 0 for float32."""
    if a.dtype == np.uint16:
        return 1
    if a.dtype == np.float32:
        return 0
    raise TypeError("sources are bf16 bit patterns (uint16) or float32")


def pack(kb: int, vb: int, k_src: np.ndarray, v_src: np.ndarray, seq_len, block_table,
         pages: np.ndarray, resid_k: np.ndarray, resid_v: np.ndarray, kmode: int = KMODE_CHANNEL,
         scales=None) -> None:
    """Prefill quantize-on-write; k_src, v_src are [B][T][H][128]; updates in place.
    kmode is the layer format; scales (FP8) is [H][2] (K, V), None for all 1."""
    B, T, H, D = k_src.shape
    assert D == HEAD_DIM and v_src.shape == k_src.shape and v_src.dtype == k_src.dtype
    kind = _src_kind(k_src)
    k_src = np.ascontiguousarray(k_src)
    v_src = np.ascontiguousarray(v_src)
    sl = np.ascontiguousarray(seq_len, dtype=np.int32)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    keep, sp = _scales_ptr(scales, H)
    _check(lib().orc_pack_x(kb, vb, kmode, sp, H, B, T, kind, k_src.ctypes.data, v_src.ctypes.data,
                          _ptr(sl, ctypes.c_int32), _ptr(bt, ctypes.c_int32), bt.shape[1],
                          _ptr(pages, ctypes.c_uint8), _ptr(resid_k, ctypes.c_uint16),
                          _ptr(resid_v, ctypes.c_uint16)), "pack")


def append(kb: int, vb: int, k_new: np.ndarray, v_new: np.ndarray, pos, block_table,
           pages: np.ndarray, resid_k: np.ndarray, resid_v: np.ndarray, kmode: int = KMODE_CHANNEL,
           scales=None) -> None:
    """Decode-time write of one bf16 token per sequence ([B][H][128] uint16); in place."""
    B, H, D = k_new.shape
    assert D == HEAD_DIM and k_new.dtype == np.uint16 and v_new.dtype == np.uint16
    kn = np.ascontiguousarray(k_new)
    vn = np.ascontiguousarray(v_new)
    p = np.ascontiguousarray(pos, dtype=np.int32)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    keep, sp = _scales_ptr(scales, H)
    _check(lib().orc_append_x(kb, vb, kmode, sp, H, B, _ptr(kn, ctypes.c_uint16), _ptr(vn, ctypes.c_uint16),
                            _ptr(p, ctypes.c_int32), _ptr(bt, ctypes.c_int32), bt.shape[1],
                            _ptr(pages, ctypes.c_uint8), _ptr(resid_k, ctypes.c_uint16),
                            _ptr(resid_v, ctypes.c_uint16)), "append")


def decode_attn(kb: int, vb: int, n_kv_heads: int, q: np.ndarray, seq_len, block_table,
                pages: np.ndarray, resid_k: np.ndarray, resid_v: np.ndarray, kmode: int = KMODE_CHANNEL,
                scales=None):
    """binary64 decode attention; q is [B][Hq][128] (bf16 bits as uint16, or float32).
    Returns (out float64 [B][Hq][128], lse float64 [B][Hq])."""
    B, Hq, D = q.shape
    assert D == HEAD_DIM
    kind = _src_kind(q)
    q = np.ascontiguousarray(q)
    sl = np.ascontiguousarray(seq_len, dtype=np.int32)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    lse = np.zeros((B, Hq), dtype=np.float64)
    keep, sp = _scales_ptr(scales, n_kv_heads)
    _check(lib().orc_decode_attn_x(kb, vb, kmode, sp, Hq, n_kv_heads, B, kind, q.ctypes.data,
                                 _ptr(sl, ctypes.c_int32), _ptr(bt, ctypes.c_int32), bt.shape[1],
                                 _ptr(pages, ctypes.c_uint8), _ptr(resid_k, ctypes.c_uint16),
                                 _ptr(resid_v, ctypes.c_uint16), _ptr(out, ctypes.c_double),
                                 _ptr(lse, ctypes.c_double)), "decode_attn")
    return out, lse


def new_cache(kb: int, vb: int, n_kv_heads: int, batch: int, n_phys_pages: int, fmt: int = KMODE_CHANNEL):
    """Zeroed host cache: (pages [P][H][page bytes], resid_k, resid_v [B][H][32][128])."""
    pages = np.zeros((n_phys_pages, n_kv_heads, head_page_bytes_fmt(kb, vb, fmt)), dtype=np.uint8)
    rk = np.zeros((batch, n_kv_heads, GROUP, HEAD_DIM), dtype=np.uint16)
    rv = np.zeros((batch, n_kv_heads, GROUP, HEAD_DIM), dtype=np.uint16)
    return pages, rk, rv


# --------------------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------------------


def equiv_bits(pairs: Iterable[tuple[int, int]]) -> Fraction:
    """Equivalent KV bit-width of a per-layer table: the mean over layers of
    (key bits + value bits) / 2, counting code bits only.  A uniform pair K8V4 is "C6",
    K8V2 "C5", K4V2 "C3".
    [KVTuner OpenReview discussion, reply to reviewer 1, section 2 "Comparison with KIVI"]
    [KVTuner, Abstract: 3.25-bit Llama-3.1-8B-Instruct, 4.0-bit Qwen2.5-7B-Instruct]"""
    pairs = list(pairs)
    return sum((Fraction(k + v, 2) for k, v in pairs), Fraction(0)) / len(pairs)


def effective_bits(pairs: Iterable[tuple[int, int]]) -> Fraction:
    """Stored bits per KV element including the fp16 scale/zero metadata: every 32 codes
    carry one 32-bit (scale, zero) word, i.e. one extra bit per element."""
    return equiv_bits(pairs) + 1


def page_bytes(n_kv_heads: int, kb: int, vb: int, head_dim: int = HEAD_DIM) -> int:
    """Bytes of one 32-token page of one layer for all KV heads: per head, 32*head_dim codes
    of kb and of vb bits, plus head_dim key (s,z) words and 32*head_dim/32 value words."""
    codes = GROUP * head_dim * (kb + vb) // 8
    sz = 4 * head_dim + 4 * GROUP * (head_dim // GROUP)
    return n_kv_heads * (codes + sz)


def kv_bytes_per_token(n_layers: int, n_kv_heads: int, head_dim: int, bytes_per_elem: float) -> float:
    """Unquantized K+V cache bytes per token: 2 (K and V) * layers * heads * head_dim * width."""
    return 2 * n_layers * n_kv_heads * head_dim * bytes_per_elem


def idealized_layer_mix_bytes(layer_bytes_bf16: float, widths_bits: Sequence[int]) -> float:
    """Idealized cache size when each layer stores its K/V at the given bit width, scaling a
    bf16 layer size linearly and ignoring scales and metadata.
    [When should you use mixed-precision KV caching to preserve accuracy in sensitive
     Transformer layers? (machinoai.in), section 2 "Beginner-friendly numerical example"]"""
    return float(sum(layer_bytes_bf16 * w / 16 for w in widths_bits))


def relative_saving(base: float, new: float) -> float:
    """(base - new) / base, the reduction convention of the pages (memory saving vs a
    baseline).  [KVTuner OpenReview discussion, reply to reviewer 1, section 2]"""
    return (base - new) / base


def tokens_per_second(batch: int, step_ms: float) -> float:
    """Throughput = generated tokens per second = batch * 1000 / step time in ms.
    [KVTuner OpenReview discussion, reply to reviewer 2, section 1, "Throughput definition"]"""
    return batch * 1000.0 / step_ms
