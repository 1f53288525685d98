"""Layer-wise mixed-precision KV-cache quantization on MI355X (gfx950).

A thin binding over the C ABI in ``include/kvq.h`` (``libkvq.so``): the functions below
carry the C names, check tensor shapes and dtypes, and pass raw device pointers plus the
current HIP stream.  Every step of the path runs in the library's kernels; PyTorch only
provides device memory and streams.

    model = Model([(4, 8)] * 3 + [(4, 2)] * 24 + [(2, 2)] * 4 + [(4, 8)], n_q_heads=32, n_kv_heads=8)
    cache = LayerCache(model, layer, batch, max_pages)         # one per layer
    kvq_pack(model, layer, cache, k_src, v_src, seq_len)        # prefill quantize-on-write
    kvq_append(model, layer, cache, k_new, v_new, pos)          # decode quantize-on-write
    out, lse = kvq_decode_attn(model, layer, cache, q, seq_len, max_seq_len)
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

from . import _native
from ._native import (KVQ_BF16, KVQ_F32, KVQ_LAYER_BF16, KVQ_LAYER_FP8, KVQ_LAYER_INT, KvqError, KvqLayerCache,
                      KvqModel, check, lib)

HEAD_DIM = 128
GROUP = 32

__all__ = ["Model", "KEYS_PER_CHANNEL", "KEYS_PER_TOKEN", "LAYER_INT", "LAYER_FP8", "LAYER_BF16", "LayerCache", "KvqError", "kvq_pack", "kvq_append", "kvq_dequant", "kvq_decode_attn", "kvq_append_decode_attn", "kvq_append_decode_attn_noalloc", "kvq_noalloc_scratch_bytes",
           "kvq_decode_workspace_bytes", "kvq_workspace_init", "kvq_head_page_bytes",
           "kvq_page_bytes", "kvq_equiv_bits", "kvq_format_version", "lib"]


KEYS_PER_CHANNEL, KEYS_PER_TOKEN = 0, 1
LAYER_INT, LAYER_FP8, LAYER_BF16 = KVQ_LAYER_INT, KVQ_LAYER_FP8, KVQ_LAYER_BF16


class Model:
    """Per-layer table plus the attention shape (kvq_model).  Each entry of `pairs` is
    (key bits, value bits) for integer codes with per-channel keys, (key bits, value bits,
    key mode) with key mode "channel" / "token" (or KEYS_PER_CHANNEL / KEYS_PER_TOKEN), or
    "fp8" / "bf16" for a layer stored as FP8 E4M3 (scaled per KV head) or BF16."""

    def __init__(self, pairs: Sequence, n_q_heads: int, n_kv_heads: int, head_dim: int = HEAD_DIM):
        modes = {"channel": KEYS_PER_CHANNEL, "token": KEYS_PER_TOKEN, KEYS_PER_CHANNEL: KEYS_PER_CHANNEL,
                 KEYS_PER_TOKEN: KEYS_PER_TOKEN}
        floats = {"fp8": (8, 8, LAYER_FP8), "bf16": (16, 16, LAYER_BF16)}
        self.pairs, self.k_modes, self.formats = [], [], []
        for e in pairs:
            if isinstance(e, str):
                kb, vb, fmt = floats[e]
                self.pairs.append((kb, vb))
                self.k_modes.append(KEYS_PER_CHANNEL)
                self.formats.append(fmt)
            else:
                self.pairs.append((int(e[0]), int(e[1])))
                self.k_modes.append(modes[e[2]] if len(e) > 2 else KEYS_PER_CHANNEL)
                self.formats.append(LAYER_INT)
        n = len(self.pairs)
        self._kb = (ctypes.c_uint8 * max(n, 1))(*[k for k, _ in self.pairs])
        self._vb = (ctypes.c_uint8 * max(n, 1))(*[v for _, v in self.pairs])
        self._km = (ctypes.c_uint8 * max(n, 1))(*self.k_modes)
        self._fmt = (ctypes.c_uint8 * max(n, 1))(*self.formats)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        self.c = KvqModel(n, n_q_heads, n_kv_heads, head_dim, ctypes.cast(self._kb, u8p),
                          ctypes.cast(self._vb, u8p), ctypes.cast(self._km, u8p), ctypes.cast(self._fmt, u8p))
        self.n_layers, self.n_q_heads, self.n_kv_heads, self.head_dim = n, n_q_heads, n_kv_heads, head_dim

    @property
    def G(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def validate(self) -> None:
        check(lib().kvq_validate_model(ctypes.byref(self.c)), "kvq_validate_model")


def kvq_format_version() -> int:
    return int(lib().kvq_format_version())


def kvq_head_page_bytes(k_bits: int, v_bits: int) -> int:
    return int(lib().kvq_head_page_bytes(k_bits, v_bits))


def kvq_page_bytes(model: Model, layer: int) -> int:
    return int(lib().kvq_page_bytes(ctypes.byref(model.c), layer))


def kvq_equiv_bits(model: Model) -> float:
    return float(lib().kvq_equiv_bits(ctypes.byref(model.c)))


class LayerCache:
    """Device buffers of one layer (kvq_layer_cache).

    pages       uint8 [n_pages][n_kv_heads][head page bytes of this layer's format]
    resid_k/v   bfloat16 [batch][n_kv_heads][32][128]
    block_table int32 [batch][max_pages]; pass one tensor to every layer to share it.
    fp8_scales  FP8 layers: float32 [n_kv_heads][2] (K scale, V scale) on the device, or
                None for 1.0; ignored by the other formats.
    """

    def __init__(self, model: Model, layer: int, batch: int, max_pages: int,
                 n_pages: Optional[int] = None, block_table=None, device="cuda", fp8_scales=None):
        import torch
        self.layer = layer
        self.batch, self.max_pages = batch, max_pages
        self.n_pages = batch * max_pages if n_pages is None else n_pages
        hp = kvq_page_bytes(model, layer) // model.n_kv_heads
        if hp == 0:
            raise KvqError(_native.KVQ_ERR_UNSUPPORTED, f"layer {layer} of the model")
        if fp8_scales is not None:
            if fp8_scales.dtype != torch.float32 or tuple(fp8_scales.shape) != (model.n_kv_heads, 2):
                raise ValueError("fp8_scales must be float32 [n_kv_heads][2]")
            _dev(fp8_scales, "fp8_scales")
        self.fp8_scales = fp8_scales
        self.pages = torch.zeros((self.n_pages, model.n_kv_heads, hp), dtype=torch.uint8, device=device)
        self.resid_k = torch.zeros((batch, model.n_kv_heads, GROUP, HEAD_DIM), dtype=torch.bfloat16, device=device)
        self.resid_v = torch.zeros_like(self.resid_k)
        if block_table is None:
            block_table = torch.arange(batch * max_pages, dtype=torch.int32, device=device).view(batch, max_pages)
        assert block_table.dtype == torch.int32 and tuple(block_table.shape) == (batch, max_pages)
        assert block_table.is_contiguous()
        self.block_table = block_table

    def sub_batch(self, b0: int, b1: int) -> "LayerCache":
        """View of sequences b0 .. b1-1: the same page pool, their residual pages and
        block-table rows.  Calls on the view touch only those sequences."""
        assert 0 <= b0 < b1 <= self.batch
        v = object.__new__(LayerCache)
        v.layer, v.batch, v.max_pages, v.n_pages = self.layer, b1 - b0, self.max_pages, self.n_pages
        v.pages = self.pages
        v.resid_k, v.resid_v = self.resid_k[b0:b1], self.resid_v[b0:b1]
        v.block_table = self.block_table[b0:b1]
        v.fp8_scales = self.fp8_scales
        return v

    def c_struct(self) -> KvqLayerCache:
        return KvqLayerCache(self.pages.data_ptr(), self.n_pages, self.resid_k.data_ptr(),
                             self.resid_v.data_ptr(), self.block_table.data_ptr(), self.batch,
                             self.max_pages, self.fp8_scales.data_ptr() if self.fp8_scales is not None else None)


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return KVQ_BF16
    if t.dtype == torch.float32:
        return KVQ_F32
    raise TypeError(f"expected bfloat16 or float32, got {t.dtype}")


def _dev(t, name):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")


def kvq_pack(model: Model, layer: int, cache: LayerCache, k_src, v_src, seq_len, stream=None) -> None:
    """Prefill quantize-on-write: k_src, v_src [batch][max_tokens][n_kv_heads][128]."""
    import torch
    for t, n in ((k_src, "k_src"), (v_src, "v_src"), (seq_len, "seq_len")):
        _dev(t, n)
    if k_src.shape != v_src.shape or k_src.dtype != v_src.dtype or k_src.dim() != 4:
        raise ValueError("k_src and v_src must have the same [batch][tokens][heads][128] shape and dtype")
    if k_src.shape[0] != cache.batch or k_src.shape[2] != model.n_kv_heads or k_src.shape[3] != HEAD_DIM:
        raise ValueError(f"source shape {tuple(k_src.shape)} does not match the model and cache")
    if seq_len.dtype != torch.int32 or seq_len.numel() != cache.batch:
        raise ValueError("seq_len must be int32 [batch]")
    cs = cache.c_struct()
    check(lib().kvq_pack(ctypes.byref(model.c), layer, ctypes.byref(cs), _dtype_code(k_src),
                         k_src.data_ptr(), v_src.data_ptr(), k_src.shape[1], seq_len.data_ptr(),
                         _stream(stream)), "kvq_pack")


def kvq_dequant(model: Model, layer: int, cache: LayerCache, seq_len, max_tokens: int, k_out=None, v_out=None,
                stream=None):
    """One layer's cache back to fp32 K, V [batch][max_tokens][n_kv_heads][128] (tokens past
    seq_len[b] keep what k_out / v_out held; new tensors start at zero).  Returns (k, v)."""
    import torch
    _dev(seq_len, "seq_len")
    if seq_len.dtype != torch.int32 or seq_len.numel() != cache.batch:
        raise ValueError("seq_len must be int32 [batch]")
    shape = (cache.batch, int(max_tokens), model.n_kv_heads, HEAD_DIM)
    outs = []
    for t, n in ((k_out, "k_out"), (v_out, "v_out")):
        if t is None:
            t = torch.zeros(shape, dtype=torch.float32, device=seq_len.device)
        _dev(t, n)
        if tuple(t.shape) != shape or t.dtype != torch.float32:
            raise ValueError(f"{n} must be float32 {shape}")
        outs.append(t)
    cs = cache.c_struct()
    check(lib().kvq_dequant(ctypes.byref(model.c), layer, ctypes.byref(cs), int(max_tokens), seq_len.data_ptr(),
                            outs[0].data_ptr(), outs[1].data_ptr(), _stream(stream)), "kvq_dequant")
    return outs[0], outs[1]


def kvq_append(model: Model, layer: int, cache: LayerCache, k_new, v_new, pos, stream=None) -> None:
    """Decode-time quantize-on-write of one bf16 token per sequence ([batch][n_kv_heads][128])."""
    import torch
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (pos, "pos")):
        _dev(t, n)
    shape = (cache.batch, model.n_kv_heads, HEAD_DIM)
    if tuple(k_new.shape) != shape or tuple(v_new.shape) != shape:
        raise ValueError(f"k_new / v_new must be {shape}")
    if k_new.dtype != torch.bfloat16 or v_new.dtype != torch.bfloat16:
        raise TypeError("k_new / v_new must be bfloat16")
    if pos.dtype != torch.int32 or pos.numel() != cache.batch:
        raise ValueError("pos must be int32 [batch]")
    cs = cache.c_struct()
    check(lib().kvq_append(ctypes.byref(model.c), layer, ctypes.byref(cs), k_new.data_ptr(),
                           v_new.data_ptr(), pos.data_ptr(), _stream(stream)), "kvq_append")


def kvq_decode_workspace_bytes(model: Model, batch: int, max_seq_len: int, pages_per_split: int = 0) -> int:
    n = int(lib().kvq_decode_workspace_bytes(ctypes.byref(model.c), batch, max_seq_len, pages_per_split))
    if n == 0:
        raise KvqError(_native.KVQ_ERR_INVALID_ARG, "kvq_decode_workspace_bytes")
    return n


def kvq_workspace_init(workspace, stream=None) -> None:
    _dev(workspace, "workspace")
    check(lib().kvq_workspace_init(workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                   _stream(stream)), "kvq_workspace_init")


def new_workspace(model: Model, batch: int, max_seq_len: int, pages_per_split: int = 0, device="cuda"):
    """A zeroed workspace tensor for kvq_decode_attn."""
    import torch
    n = kvq_decode_workspace_bytes(model, batch, max_seq_len, pages_per_split)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def kvq_decode_attn(model: Model, layer: int, cache: LayerCache, q, seq_len, max_seq_len: int,
                    pages_per_split: int = 0, out=None, lse=None, workspace=None, stream=None):
    """Single-token decode attention; q is [batch][n_q_heads][128] (bf16 or fp32).
    Returns (out fp32 [batch][n_q_heads][128], lse fp32 [batch][n_q_heads])."""
    import torch
    _dev(q, "q")
    _dev(seq_len, "seq_len")
    if tuple(q.shape) != (cache.batch, model.n_q_heads, HEAD_DIM):
        raise ValueError(f"q must be [{cache.batch}][{model.n_q_heads}][128]")
    if seq_len.dtype != torch.int32 or seq_len.numel() != cache.batch:
        raise ValueError("seq_len must be int32 [batch]")
    if out is None:
        out = torch.empty((cache.batch, model.n_q_heads, HEAD_DIM), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((cache.batch, model.n_q_heads), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = new_workspace(model, cache.batch, max_seq_len, pages_per_split, q.device)
    cs = cache.c_struct()
    check(lib().kvq_decode_attn(ctypes.byref(model.c), layer, ctypes.byref(cs), _dtype_code(q),
                                q.data_ptr(), seq_len.data_ptr(), max_seq_len, pages_per_split,
                                out.data_ptr(), lse.data_ptr() if lse is not False else None,
                                workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                _stream(stream)), "kvq_decode_attn")
    return out, lse


def kvq_append_decode_attn(model: Model, layer: int, cache: LayerCache, k_new, v_new, pos, q, max_seq_len: int,
                           pages_per_split: int = 0, out=None, lse=None, workspace=None, stream=None):
    """kvq_append of one bf16 token per sequence followed by decode attention over pos + 1
    tokens, in one launch.  Returns (out, lse) as kvq_decode_attn."""
    import torch
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (pos, "pos"), (q, "q")):
        _dev(t, n)
    shape = (cache.batch, model.n_kv_heads, HEAD_DIM)
    if tuple(k_new.shape) != shape or tuple(v_new.shape) != shape:
        raise ValueError(f"k_new / v_new must be {shape}")
    if k_new.dtype != torch.bfloat16 or v_new.dtype != torch.bfloat16:
        raise TypeError("k_new / v_new must be bfloat16")
    if pos.dtype != torch.int32 or pos.numel() != cache.batch:
        raise ValueError("pos must be int32 [batch]")
    if tuple(q.shape) != (cache.batch, model.n_q_heads, HEAD_DIM):
        raise ValueError(f"q must be [{cache.batch}][{model.n_q_heads}][128]")
    if out is None:
        out = torch.empty((cache.batch, model.n_q_heads, HEAD_DIM), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((cache.batch, model.n_q_heads), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = new_workspace(model, cache.batch, max_seq_len, pages_per_split, q.device)
    cs = cache.c_struct()
    check(lib().kvq_append_decode_attn(ctypes.byref(model.c), layer, ctypes.byref(cs), k_new.data_ptr(),
                                       v_new.data_ptr(), pos.data_ptr(), _dtype_code(q), q.data_ptr(),
                                       max_seq_len, pages_per_split, out.data_ptr(),
                                       lse.data_ptr() if lse is not False else None, workspace.data_ptr(),
                                       workspace.numel() * workspace.element_size(), _stream(stream)),
          "kvq_append_decode_attn")
    return out, lse


def kvq_append_decode_attn_noalloc(model: Model, layer: int, cache: LayerCache, k_new, v_new, pos, q,
                                   max_seq_len: int, out, lse, pages_per_split: int = 0, stream=None):
    """kvq_append_decode_attn with the library's own per-GPU scratch instead of a workspace:
    the C call allocates nothing (the caller passes out [batch][n_q_heads][128] fp32 and lse
    [batch][n_q_heads] fp32, or lse=False).  Calls that overlap on one GPU race."""
    import torch
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (pos, "pos"), (q, "q"), (out, "out")):
        _dev(t, n)
    shape = (cache.batch, model.n_kv_heads, HEAD_DIM)
    if tuple(k_new.shape) != shape or tuple(v_new.shape) != shape:
        raise ValueError(f"k_new / v_new must be {shape}")
    if k_new.dtype != torch.bfloat16 or v_new.dtype != torch.bfloat16:
        raise TypeError("k_new / v_new must be bfloat16")
    if pos.dtype != torch.int32 or pos.numel() != cache.batch:
        raise ValueError("pos must be int32 [batch]")
    if tuple(q.shape) != (cache.batch, model.n_q_heads, HEAD_DIM):
        raise ValueError(f"q must be [{cache.batch}][{model.n_q_heads}][128]")
    if tuple(out.shape) != (cache.batch, model.n_q_heads, HEAD_DIM) or out.dtype != torch.float32:
        raise ValueError("out must be float32 [batch][n_q_heads][128]")
    if lse is not False:
        _dev(lse, "lse")
        if tuple(lse.shape) != (cache.batch, model.n_q_heads) or lse.dtype != torch.float32:
            raise ValueError("lse must be float32 [batch][n_q_heads]")
    cs = cache.c_struct()
    check(lib().kvq_append_decode_attn_noalloc(ctypes.byref(model.c), layer, ctypes.byref(cs), k_new.data_ptr(),
                                               v_new.data_ptr(), pos.data_ptr(), _dtype_code(q), q.data_ptr(),
                                               max_seq_len, pages_per_split, out.data_ptr(),
                                               lse.data_ptr() if lse is not False else None, _stream(stream)),
          "kvq_append_decode_attn_noalloc")
    return out, lse


def kvq_noalloc_scratch_bytes(model: Model, batch: int, max_seq_len: int, pages_per_split: int = 0) -> int:
    return int(lib().kvq_noalloc_scratch_bytes(ctypes.byref(model.c), batch, max_seq_len, pages_per_split))
