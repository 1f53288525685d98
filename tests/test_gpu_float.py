"""GPU parity of the floating-point layer formats: FP8 E4M3 with one K and one V scale per
KV head, and BF16 (the per-layer BF16 / FP8 mix of the machinoai page).

Pages and live residual slots bit-exact against the oracle (FP8 encode is round to nearest
even with saturation, computed from x / scale in binary32 on both sides); attention within
2e-4 (max abs) and 1e-4 (relative lse) of the oracle's binary64 result for several query
group sizes and split sizes; the fused append (including flushes) against the oracle and
the two-launch path; a model that mixes integer, FP8 and BF16 layers.
"""
import math

import numpy as np
import pytest

from kvq_cases import Case, assert_attention_close, host_array, live_resid_equal, log
import synth

pytestmark = pytest.mark.gpu

FP8, BF16 = 2, 3
BITS = {FP8: 8, BF16: 16}


@pytest.fixture(scope="module")
def kvq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import layer_wise_mixed_kvq_amd as k
    k.lib()
    return k


def calibrated_scales(c):
    """Per KV head: max |x| / 448 over the case's K and V (binary32), the usual E4M3 scaling."""
    k = host_array(c.k.float()).reshape(c.B, c.T, c.H, 128)
    v = host_array(c.v.float()).reshape(c.B, c.T, c.H, 128)
    ks = np.abs(k).max(axis=(0, 1, 3)).astype(np.float32) / np.float32(448.0)
    vs = np.abs(v).max(axis=(0, 1, 3)).astype(np.float32) / np.float32(448.0)
    return np.stack([ks, vs], axis=1)


def make_case(fmt, scaled, **kw):
    bits = BITS[fmt]
    c = Case(bits, bits, kmode=fmt, **kw)
    if fmt == FP8 and scaled:
        c = Case(bits, bits, kmode=fmt, scales=calibrated_scales(c), **kw)
    return c


VARIANTS = [(FP8, False), (FP8, True), (BF16, False)]
IDS = ["fp8-unit", "fp8-scaled", "bf16"]


@pytest.mark.parametrize("fmt,scaled", VARIANTS, ids=IDS)
@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_float_pack_bit_exact(kvq, orc, fmt, scaled, src):
    c = make_case(fmt, scaled, H=2, G=1, lens=[77, 64, 5, 0, 200], seed=fmt * 5 + scaled, src=src)
    log(f"float pack fmt={fmt} scaled={scaled} src={src}")
    c.oracle_pack(orc)
    c.device_setup(kvq)
    c.device_pack(kvq)
    assert np.array_equal(c.cache.pages.cpu().numpy(), c.o_pages), "packed pages differ"
    assert live_resid_equal(host_array(c.cache.resid_k), c.o_rk, c.lens)
    assert live_resid_equal(host_array(c.cache.resid_v), c.o_rv, c.lens)


def test_fp8_saturation_and_signed_zero(kvq, orc):
    """Values beyond 448 * scale saturate to +-448 and -0 keeps its sign bit, as in the oracle."""
    import torch
    c = Case(8, 8, H=1, G=1, lens=[64], seed=3, kmode=FP8, scales=[[0.01, 0.02]], src="f32")
    k = c.k.clone()
    k[0, 0, 0, :8] = torch.tensor([5.0, -5.0, 4.48, 4.4801, -0.0, 0.0, 1e-7, -1e-7])
    c.k = k
    c.oracle_pack(orc)
    c.device_setup(kvq)
    c.device_pack(kvq)
    pages = c.cache.pages.cpu().numpy()
    assert np.array_equal(pages, c.o_pages)
    phys = c.bt[0, 0]
    assert list(pages[phys, 0, :6]) == [0x7E, 0xFE, 0x7E, 0x7E, 0x80, 0x00]


@pytest.mark.parametrize("fmt,scaled", VARIANTS, ids=IDS)
@pytest.mark.parametrize("G", [1, 4, 7, 16])
def test_float_decode_parity(kvq, orc, fmt, scaled, G):
    c = make_case(fmt, scaled, H=2, G=G, lens=[1, 31, 32, 33, 200, 517], seed=fmt * 101 + G + 7 * scaled)
    log(f"float decode fmt={fmt} scaled={scaled} G={G}")
    c.oracle_pack(orc)
    c.device_setup(kvq)
    c.device_pack(kvq)
    o_ref, l_ref = c.oracle_decode(orc)
    for pps in (0, 2, 1):
        out, lse = c.device_decode(kvq, pages_per_split=pps)
        assert_attention_close(out, lse, o_ref, l_ref, f"fmt={fmt} scaled={scaled} G={G} pps={pps}")


@pytest.mark.parametrize("fmt,scaled,G", [(FP8, True, 4), (FP8, False, 1), (BF16, False, 4), (BF16, False, 7)])
def test_float_fused_append(kvq, orc, fmt, scaled, G):
    """Fused append + attention; steps cover flushes (starting lengths 29, 62, 0).  After
    each step the cache equals the oracle's and a twin cache driven by kvq_append."""
    import torch
    L0 = np.array([29, 62, 0], dtype=np.int32)
    steps, H = 4, 2
    c = make_case(fmt, scaled, H=H, G=G, lens=list(L0 + steps), seed=fmt + 3 * G + scaled)
    c.o_pages, c.o_rk, c.o_rv = orc.new_cache(c.kb, c.vb, H, c.B, c.n_phys, fmt)
    orc.pack(c.kb, c.vb, host_array(c.k), host_array(c.v), L0, c.bt, c.o_pages, c.o_rk, c.o_rv, kmode=fmt,
             scales=c.scales)
    c.device_setup(kvq)
    twin = kvq.LayerCache(c.model, 0, c.B, c.maxp, n_pages=c.n_phys, block_table=c.bt_d, device=c.dev,
                          fp8_scales=c.scales_d)
    l0 = torch.from_numpy(L0).to(c.dev)
    for cache in (c.cache, twin):
        kvq.kvq_pack(c.model, 0, cache, c.k.to(c.dev), c.v.to(c.dev), l0)
    q = c.q.to(c.dev)
    msl = c.maxp * 32
    for s in range(steps):
        pos = L0 + s
        kn = synth.fill(c.seed, synth.KIND_K_NEW, 0, c.B, 1, H, t0=s).view(c.B, H, 128)
        vn = synth.fill(c.seed, synth.KIND_V_NEW, 0, c.B, 1, H, t0=s).view(c.B, H, 128)
        log(f"float fused fmt={fmt} scaled={scaled} G={G} step {s}")
        orc.append(c.kb, c.vb, host_array(kn), host_array(vn), pos, c.bt, c.o_pages, c.o_rk, c.o_rv, kmode=fmt,
                   scales=c.scales)
        o_ref, l_ref = orc.decode_attn(c.kb, c.vb, H, host_array(c.q), pos + 1, c.bt, c.o_pages, c.o_rk, c.o_rv,
                                       kmode=fmt, scales=c.scales)
        pos_d = torch.from_numpy(pos).to(c.dev)
        knd, vnd = kn.to(c.dev), vn.to(c.dev)
        pps = [0, 1, 2, 0][s]
        out, lse = kvq.kvq_append_decode_attn(c.model, 0, c.cache, knd, vnd, pos_d, q, msl, pages_per_split=pps)
        kvq.kvq_append(c.model, 0, twin, knd, vnd, pos_d)
        out2, lse2 = kvq.kvq_decode_attn(c.model, 0, twin, q, pos_d + 1, msl, pages_per_split=pps)
        torch.cuda.synchronize()
        pages = c.cache.pages.cpu().numpy()
        assert np.array_equal(pages, c.o_pages), f"step {s}: pages differ from the oracle"
        assert np.array_equal(twin.pages.cpu().numpy(), c.o_pages), f"step {s}: kvq_append pages differ"
        assert live_resid_equal(host_array(c.cache.resid_k), c.o_rk, pos + 1), f"step {s}: residual"
        assert live_resid_equal(host_array(c.cache.resid_v), c.o_rv, pos + 1), f"step {s}: residual"
        assert_attention_close(out.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"fused step {s}")
        assert_attention_close(out2.cpu().numpy(), lse2.cpu().numpy(), o_ref, l_ref, f"two-launch step {s}")


def test_mixed_integer_fp8_bf16_model(kvq, orc):
    """Four layers -- BF16, FP8 (scaled), integer K4V2, integer per-token K2V2 -- in one model;
    each layer's pages and attention match the oracle run in that layer's format."""
    import torch
    H, G, lens = 2, 4, [95, 40, 129]
    specs = [(BF16, 16, 16, False), (FP8, 8, 8, True), (0, 4, 2, False), (1, 2, 2, False)]
    cases = []
    for l, (fmt, kb, vb, scaled) in enumerate(specs):
        c = Case(kb, vb, H=H, G=G, lens=lens, seed=60 + l, layer=l, kmode=fmt)
        if scaled:
            c = Case(kb, vb, H=H, G=G, lens=lens, seed=60 + l, layer=l, kmode=fmt, scales=calibrated_scales(c))
        cases.append(c)
    model = kvq.Model([c.layer_entry() for c in cases], H * G, H)
    for l, c in enumerate(cases):
        log(f"mixed model layer {l} fmt={c.kmode}")
        c.oracle_pack(orc)
        c.device_setup(kvq)
        cache = kvq.LayerCache(model, l, c.B, c.maxp, n_pages=c.n_phys, block_table=c.bt_d, device=c.dev,
                               fp8_scales=c.scales_d)
        kvq.kvq_pack(model, l, cache, c.k.to(c.dev), c.v.to(c.dev), c.lens_d)
        out, lse = kvq.kvq_decode_attn(model, l, cache, c.q.to(c.dev), c.lens_d, c.maxp * 32)
        torch.cuda.synchronize()
        assert np.array_equal(cache.pages.cpu().numpy(), c.o_pages), f"layer {l}: pages"
        o_ref, l_ref = c.oracle_decode(orc)
        assert_attention_close(out.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"layer {l}")


def _e4m3_values_and_ties():
    """Every finite E4M3 value, every midpoint between neighbours (exact ties), both signs,
    plus signed zeros, tiny values and values past the largest finite 448."""
    vals = []
    for b in range(128):
        e, m = (b >> 3) & 15, b & 7
        if e == 15 and m == 7:
            continue
        v = math.ldexp(8 + m, e - 10) if e else math.ldexp(m, -9)
        nxt = math.ldexp(16, e - 10) if m == 7 else (math.ldexp(9 + m, e - 10) if e else math.ldexp(m + 1, -9))
        vals += [v, -v, (v + nxt) / 2, -(v + nxt) / 2]
    vals += [0.0, -0.0, 1e-30, -1e-30, 448.5, 463.9, 464.0, 465.0, 480.0, 1e6, -1e6]
    return np.array(vals, dtype=np.float32)


@pytest.mark.parametrize("scale", [1.0, 0.03125, 0.7])
def test_fp8_encode_every_value_and_tie(kvq, orc, scale):
    """Pages of K and V tiles holding every E4M3 value and tie (times the scale) are
    bit-exact with the oracle's encoder (round to nearest even, saturation at 448)."""
    import torch
    vals = _e4m3_values_and_ties() * np.float32(scale)
    c = Case(8, 8, H=1, G=1, lens=[64], seed=11, kmode=FP8, scales=[[scale, scale]], src="f32")
    k = c.k.clone()
    v = c.v.clone()
    flat = np.resize(vals, 64 * 128).reshape(1, 64, 1, 128)
    k[:] = torch.from_numpy(flat)
    v[:] = torch.from_numpy(np.ascontiguousarray(flat[:, ::-1]))
    c.k, c.v = k, v
    log(f"fp8 every value scale={scale}")
    c.oracle_pack(orc)
    c.device_setup(kvq)
    c.device_pack(kvq)
    assert np.array_equal(c.cache.pages.cpu().numpy(), c.o_pages)
