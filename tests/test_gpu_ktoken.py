"""GPU parity of the per-token key mode (keys quantized per token over 32-channel groups).

Pages and live residual slots bit-exact against the oracle for every pair; attention within
2e-4 (max abs) and 1e-4 (relative lse) for every pair and query-group size, over several
split sizes; the fused append (including flushes) in this mode; and a model whose layers
mix the two key modes.
"""
import numpy as np
import pytest

from kvq_cases import Case, assert_attention_close, host_array, live_resid_equal, log
import synth

pytestmark = pytest.mark.gpu

PAIRS = [(k, v) for k in (2, 4, 8) for v in (2, 4, 8)]
KT = 1


@pytest.fixture(scope="module")
def kvq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import layer_wise_mixed_kvq_amd as k
    k.lib()
    return k


@pytest.mark.parametrize("kb,vb", PAIRS)
def test_ktoken_pack_bit_exact(kvq, orc, kb, vb):
    c = Case(kb, vb, H=2, G=1, lens=[77, 64, 5, 0, 200], seed=kb * 13 + vb, kmode=KT)
    log(f"per-token pack kb={kb} vb={vb}")
    c.oracle_pack(orc)
    c.device_setup(kvq)
    c.device_pack(kvq)
    assert np.array_equal(c.cache.pages.cpu().numpy(), c.o_pages), "packed pages differ"
    assert live_resid_equal(host_array(c.cache.resid_k), c.o_rk, c.lens)


@pytest.mark.parametrize("kb,vb", PAIRS)
@pytest.mark.parametrize("G", [1, 4, 7, 16])
def test_ktoken_decode_parity(kvq, orc, kb, vb, G):
    c = Case(kb, vb, H=2, G=G, lens=[1, 31, 32, 33, 200, 517], seed=kb * 101 + vb * 11 + G, kmode=KT)
    log(f"per-token decode kb={kb} vb={vb} G={G}")
    c.oracle_pack(orc)
    c.device_setup(kvq)
    c.device_pack(kvq)
    o_ref, l_ref = c.oracle_decode(orc)
    for pps in (0, 2):
        out, lse = c.device_decode(kvq, pages_per_split=pps)
        assert_attention_close(out, lse, o_ref, l_ref, f"kb={kb} vb={vb} G={G} pps={pps}")


@pytest.mark.parametrize("kb,vb,G", [(4, 2, 4), (8, 8, 7), (2, 4, 1)])
def test_ktoken_fused_append(kvq, orc, kb, vb, G):
    """Fused append + attention in the per-token mode; steps cover flushes."""
    import torch
    L0 = np.array([29, 62, 0], dtype=np.int32)
    steps, H = 4, 2
    c = Case(kb, vb, H=H, G=G, lens=list(L0 + steps), seed=kb + 3 * vb + G, kmode=KT)
    c.o_pages, c.o_rk, c.o_rv = orc.new_cache(kb, vb, H, c.B, c.n_phys)
    orc.pack(kb, vb, host_array(c.k), host_array(c.v), L0, c.bt, c.o_pages, c.o_rk, c.o_rv, kmode=KT)
    c.device_setup(kvq)
    kvq.kvq_pack(c.model, 0, c.cache, c.k.to(c.dev), c.v.to(c.dev), torch.from_numpy(L0).to(c.dev))
    q = c.q.to(c.dev)
    msl = c.maxp * 32
    for s in range(steps):
        pos = L0 + s
        kn = synth.fill(c.seed, synth.KIND_K_NEW, 0, c.B, 1, H, t0=s).view(c.B, H, 128)
        vn = synth.fill(c.seed, synth.KIND_V_NEW, 0, c.B, 1, H, t0=s).view(c.B, H, 128)
        log(f"per-token fused kb={kb} vb={vb} G={G} step {s}")
        orc.append(kb, vb, host_array(kn), host_array(vn), pos, c.bt, c.o_pages, c.o_rk, c.o_rv, kmode=KT)
        o_ref, l_ref = orc.decode_attn(kb, vb, H, host_array(c.q), pos + 1, c.bt, c.o_pages, c.o_rk, c.o_rv,
                                       kmode=KT)
        out, lse = kvq.kvq_append_decode_attn(c.model, 0, c.cache, kn.to(c.dev), vn.to(c.dev),
                                              torch.from_numpy(pos).to(c.dev), q, msl,
                                              pages_per_split=[0, 1, 2, 0][s])
        torch.cuda.synchronize()
        assert np.array_equal(c.cache.pages.cpu().numpy(), c.o_pages), f"step {s}: pages"
        assert live_resid_equal(host_array(c.cache.resid_k), c.o_rk, pos + 1), f"step {s}: residual"
        assert_attention_close(out.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"step {s}")


def test_mixed_key_modes_per_layer(kvq, orc):
    """A 3-layer model: per-channel, per-token, per-channel keys; each layer's pages and
    attention match the oracle run in that layer's mode."""
    import torch
    layers = [(4, 2, 0), (4, 2, 1), (8, 4, 0)]
    H, G, lens = 2, 4, [95, 40, 129]
    model = kvq.Model(layers, H * G, H)
    for l, (kb, vb, km) in enumerate(layers):
        c = Case(kb, vb, H=H, G=G, lens=lens, seed=50 + l, layer=l, kmode=km)
        c.oracle_pack(orc)
        c.device_setup(kvq)
        cache = kvq.LayerCache(model, l, c.B, c.maxp, n_pages=c.n_phys, block_table=c.bt_d, device=c.dev)
        kvq.kvq_pack(model, l, cache, c.k.to(c.dev), c.v.to(c.dev), c.lens_d)
        out, lse = kvq.kvq_decode_attn(model, l, cache, c.q.to(c.dev), c.lens_d, c.maxp * 32)
        torch.cuda.synchronize()
        assert np.array_equal(cache.pages.cpu().numpy(), c.o_pages), f"layer {l}: pages"
        o_ref, l_ref = c.oracle_decode(orc)
        assert_attention_close(out.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"layer {l}")
