"""Host-side checks of the C ABI (CPU only, nothing is launched on a GPU):
  * libkvq.so loads and exports every function include/kvq.h declares,
  * accounting helpers agree with the format's closed forms,
  * invalid arguments are rejected before any HIP call, with the documented status.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


@pytest.fixture(scope="module")
def kvq():
    import layer_wise_mixed_kvq_amd as k
    k.lib()
    return k


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_0-9]+)\s*\(", text)))


def test_header_symbols_exported(kvq):
    names = declared_functions()
    assert len(names) >= 10
    from layer_wise_mixed_kvq_amd import _native
    assert set(names) == set(_native.EXPORTED)
    for n in names:
        assert hasattr(kvq.lib(), n), n


def test_format_constants(kvq):
    assert kvq.kvq_format_version() == 2
    for kb in (2, 4, 8):
        for vb in (2, 4, 8):
            assert kvq.kvq_head_page_bytes(kb, vb) == 512 * (kb + vb + 2)
    assert kvq.kvq_head_page_bytes(3, 4) == 0
    assert kvq.kvq_head_page_bytes(4, 16) == 0


LLAMA = [(4, 8)] * 3 + [(4, 2)] * 24 + [(2, 2)] * 4 + [(4, 8)]
QWEN = [(8, 4)] * 4 + [(4, 4)] * 4 + [(4, 2)] * 16 + [(8, 4)] * 4


def test_equiv_bits_and_page_bytes(kvq):
    m = kvq.Model(LLAMA, 32, 8)
    assert kvq.kvq_equiv_bits(m) == 3.25
    assert kvq.kvq_equiv_bits(kvq.Model(QWEN, 28, 4)) == 4.0
    assert kvq.kvq_page_bytes(m, 0) == 8 * 512 * 14
    assert kvq.kvq_page_bytes(m, 5) == 8 * 512 * 8
    assert kvq.kvq_page_bytes(m, 28) == 8 * 512 * 6
    assert kvq.kvq_page_bytes(m, 32) == 0


def test_float_layer_formats(kvq):
    """FP8 / BF16 layers: page bytes 8192 / 16384 per KV head, equivalent bits 8 / 16, the
    machinoai page's 8 BF16 + 24 FP8 example at 10 bits, and width checks per format."""
    from layer_wise_mixed_kvq_amd import _native as N
    mix = kvq.Model(["bf16"] * 8 + ["fp8"] * 24, 32, 8)
    assert kvq.lib().kvq_validate_model(ctypes.byref(mix.c)) == N.KVQ_OK
    assert kvq.kvq_page_bytes(mix, 0) == 8 * 16384
    assert kvq.kvq_page_bytes(mix, 8) == 8 * 8192
    assert kvq.kvq_equiv_bits(mix) == (8 * 16 + 24 * 8) / 32
    # integer and float layers side by side
    m = kvq.Model([(4, 2), "fp8", (2, 2, "token"), "bf16"], 8, 2)
    assert [kvq.kvq_page_bytes(m, l) for l in range(4)] == [2 * 512 * 8, 2 * 8192, 2 * 512 * 6, 2 * 16384]
    # FP8 needs 8 / 8 and BF16 16 / 16; unknown format codes are rejected
    for fmt, kb, vb in [(N.KVQ_LAYER_FP8, 4, 8), (N.KVQ_LAYER_FP8, 16, 16), (N.KVQ_LAYER_BF16, 8, 8),
                        (N.KVQ_LAYER_INT, 16, 16), (3, 4, 4)]:
        bad = kvq.Model([(kb, vb)], 4, 1)
        bad._fmt[0] = fmt
        assert kvq.lib().kvq_validate_model(ctypes.byref(bad.c)) == N.KVQ_ERR_UNSUPPORTED, (fmt, kb, vb)
        assert kvq.kvq_page_bytes(bad, 0) == 0


def _status(kvq, fn, *args):
    return fn(*args)


def test_model_validation(kvq):
    from layer_wise_mixed_kvq_amd import _native as N
    ok = kvq.Model(LLAMA, 32, 8)
    assert kvq.lib().kvq_validate_model(ctypes.byref(ok.c)) == N.KVQ_OK
    assert kvq.lib().kvq_validate_model(None) == N.KVQ_ERR_INVALID_ARG
    for bad, want in [(kvq.Model([(3, 4)], 4, 1), N.KVQ_ERR_UNSUPPORTED),
                      (kvq.Model([(4, 4)], 4, 1, head_dim=64), N.KVQ_ERR_UNSUPPORTED),
                      (kvq.Model([(4, 4)], 6, 4), N.KVQ_ERR_UNSUPPORTED),
                      (kvq.Model([(4, 4)], 0, 1), N.KVQ_ERR_INVALID_ARG),
                      (kvq.Model([], 4, 1), N.KVQ_ERR_INVALID_ARG)]:
        assert kvq.lib().kvq_validate_model(ctypes.byref(bad.c)) == want
    assert kvq.kvq_equiv_bits(kvq.Model([(3, 4)], 4, 1)) == -1.0
    with pytest.raises(kvq.KvqError):
        kvq.Model([(4, 4)], 6, 4).validate()


def _fake_cache(kvq, **over):
    f = dict(pages=0x10000, n_pages=4, resid_k=0x20000, resid_v=0x30000, block_table=0x40000,
             batch=2, max_pages=2)
    f.update(over)
    return kvq.KvqLayerCache(f["pages"], f["n_pages"], f["resid_k"], f["resid_v"], f["block_table"],
                             f["batch"], f["max_pages"])


def test_entry_points_reject_before_launch(kvq):
    """Every case below fails validation on the host, so no HIP call is made."""
    from layer_wise_mixed_kvq_amd import _native as N
    L = kvq.lib()
    m = kvq.Model([(4, 2), (8, 8)], 8, 2)
    mp = ctypes.byref(m.c)
    good = _fake_cache(kvq)
    A = 0x50000   # 16-byte aligned stand-in pointers; never dereferenced on the host
    # pack
    assert L.kvq_pack(mp, 2, ctypes.byref(good), N.KVQ_BF16, A, A, 64, A, None) == N.KVQ_ERR_INVALID_ARG
    assert L.kvq_pack(mp, -1, ctypes.byref(good), N.KVQ_BF16, A, A, 64, A, None) == N.KVQ_ERR_INVALID_ARG
    assert L.kvq_pack(mp, 0, None, N.KVQ_BF16, A, A, 64, A, None) == N.KVQ_ERR_INVALID_ARG
    assert L.kvq_pack(mp, 0, ctypes.byref(good), N.KVQ_BF16, None, A, 64, A, None) == N.KVQ_ERR_INVALID_ARG
    assert L.kvq_pack(mp, 0, ctypes.byref(good), 7, A, A, 64, A, None) == N.KVQ_ERR_UNSUPPORTED
    assert L.kvq_pack(mp, 0, ctypes.byref(good), N.KVQ_BF16, A + 2, A, 64, A, None) == N.KVQ_ERR_ALIGNMENT
    assert L.kvq_pack(mp, 0, ctypes.byref(_fake_cache(kvq, pages=0x10008)), N.KVQ_BF16, A, A, 64, A,
                      None) == N.KVQ_ERR_ALIGNMENT
    assert L.kvq_pack(mp, 0, ctypes.byref(_fake_cache(kvq, batch=0)), N.KVQ_BF16, A, A, 64, A,
                      None) == N.KVQ_ERR_INVALID_ARG
    assert L.kvq_pack(mp, 0, ctypes.byref(_fake_cache(kvq, n_pages=0)), N.KVQ_BF16, A, A, 64, A,
                      None) == N.KVQ_ERR_INVALID_ARG
    assert L.kvq_pack(mp, 0, ctypes.byref(good), N.KVQ_BF16, A, A, -1, A, None) == N.KVQ_ERR_INVALID_ARG
    # zero tokens is a valid no-op that launches nothing
    assert L.kvq_pack(mp, 0, ctypes.byref(good), N.KVQ_BF16, A, A, 0, A, None) == N.KVQ_OK
    # append
    assert L.kvq_append(mp, 0, ctypes.byref(good), None, A, A, None) == N.KVQ_ERR_INVALID_ARG
    assert L.kvq_append(mp, 0, ctypes.byref(good), A + 4, A, A, None) == N.KVQ_ERR_ALIGNMENT
    assert L.kvq_append(mp, 9, ctypes.byref(good), A, A, A, None) == N.KVQ_ERR_INVALID_ARG
    # dequant
    assert L.kvq_dequant(mp, 0, ctypes.byref(good), 64, None, A, A, None) == N.KVQ_ERR_INVALID_ARG
    assert L.kvq_dequant(mp, 0, ctypes.byref(good), 64, A, None, A, None) == N.KVQ_ERR_INVALID_ARG
    assert L.kvq_dequant(mp, 0, ctypes.byref(good), -1, A, A, A, None) == N.KVQ_ERR_INVALID_ARG
    assert L.kvq_dequant(mp, 0, ctypes.byref(good), 64, A, A + 4, A, None) == N.KVQ_ERR_ALIGNMENT
    assert L.kvq_dequant(mp, 2, ctypes.byref(good), 64, A, A, A, None) == N.KVQ_ERR_INVALID_ARG
    assert L.kvq_dequant(mp, 0, ctypes.byref(good), 0, A, A, A, None) == N.KVQ_OK
    # decode
    need = L.kvq_decode_workspace_bytes(mp, 2, 64, 0)
    assert need > 0
    assert L.kvq_decode_attn(mp, 0, ctypes.byref(good), N.KVQ_BF16, A, A, 64, 0, A, A, A, need - 1,
                             None) == N.KVQ_ERR_WORKSPACE
    assert L.kvq_decode_attn(mp, 0, ctypes.byref(good), N.KVQ_BF16, A, A, 64, 0, A, A, None, need,
                             None) == N.KVQ_ERR_WORKSPACE
    assert L.kvq_decode_attn(mp, 0, ctypes.byref(good), N.KVQ_BF16, None, A, 64, 0, A, A, A, need,
                             None) == N.KVQ_ERR_INVALID_ARG
    assert L.kvq_decode_attn(mp, 0, ctypes.byref(good), N.KVQ_BF16, A, A, -5, 0, A, A, A, need,
                             None) == N.KVQ_ERR_INVALID_ARG
    assert L.kvq_decode_attn(mp, 0, ctypes.byref(good), N.KVQ_BF16, A + 8, A, 64, 0, A, A, A, need,
                             None) == N.KVQ_ERR_ALIGNMENT
    assert L.kvq_decode_attn(mp, 0, ctypes.byref(good), 3, A, A, 64, 0, A, A, A, need,
                             None) == N.KVQ_ERR_UNSUPPORTED
    bad = kvq.Model([(4, 5)], 8, 2)
    assert L.kvq_decode_attn(ctypes.byref(bad.c), 0, ctypes.byref(good), N.KVQ_BF16, A, A, 64, 0, A, A,
                             A, need, None) == N.KVQ_ERR_UNSUPPORTED
    assert L.kvq_workspace_init(None, 16, None) == N.KVQ_ERR_INVALID_ARG
    assert L.kvq_workspace_init(A + 4, 16, None) == N.KVQ_ERR_ALIGNMENT
    # the scratch-backed fused entry point: argument errors, and shapes beyond its fixed
    # maximum (more than KVQ_NOALLOC_MAX_COUNTERS (sequence, KV head) pairs, or more than
    # KVQ_NOALLOC_MAX_PARTIAL_BYTES of partials), all before any HIP call
    na = L.kvq_append_decode_attn_noalloc
    assert na(mp, 0, ctypes.byref(good), None, A, A, N.KVQ_BF16, A, 64, 0, A, A, None) == N.KVQ_ERR_INVALID_ARG
    assert na(mp, 0, ctypes.byref(good), A + 2, A, A, N.KVQ_BF16, A, 64, 0, A, A, None) == N.KVQ_ERR_ALIGNMENT
    assert na(mp, 0, ctypes.byref(good), A, A, A, N.KVQ_BF16, A, 64, 0, None, A, None) == N.KVQ_ERR_INVALID_ARG
    assert na(mp, 0, ctypes.byref(good), A, A, A, 3, A, 64, 0, A, A, None) == N.KVQ_ERR_UNSUPPORTED
    wide = _fake_cache(kvq, batch=65535)           # 65535 * 2 KV heads > 65536 counters
    assert na(mp, 0, ctypes.byref(wide), A, A, A, N.KVQ_BF16, A, 64, 0, A, A, None) == N.KVQ_ERR_WORKSPACE
    long_ = _fake_cache(kvq, batch=64)            # 64 * 2 heads * 2**20 tokens: partials far beyond 32 MiB
    assert na(mp, 0, ctypes.byref(long_), A, A, A, N.KVQ_BF16, A, 1 << 20, 1, A, A, None) == N.KVQ_ERR_WORKSPACE
    assert L.kvq_noalloc_scratch_bytes(mp, 64, 1 << 20, 1) > (32 << 20)
    assert 0 < L.kvq_noalloc_scratch_bytes(mp, 2, 64, 0) <= (32 << 20)


def test_workspace_grows_with_splits(kvq):
    m = kvq.Model([(4, 2)], 32, 8)
    a = kvq.kvq_decode_workspace_bytes(m, 16, 4097, 16)
    b = kvq.kvq_decode_workspace_bytes(m, 16, 4097, 1)
    assert b > a > 0
    assert a % 256 == 0


def test_status_strings(kvq):
    from layer_wise_mixed_kvq_amd import _native as N
    assert N.status_str(N.KVQ_ERR_WORKSPACE) == "KVQ_ERR_WORKSPACE"
    assert N.status_str(N.KVQ_OK) == "KVQ_OK"
