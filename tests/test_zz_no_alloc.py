"""kvq_append_decode_attn_noalloc (the library's own per-GPU scratch, no workspace argument)
against kvq_append_decode_attn (the caller's workspace) through the C ABI.

Two calls in a row, the second with a smaller input (fewer sequences, fewer heads, one split
plan the library picks), each on a cache of its own with a twin cache for the workspace entry
point: out and lse bit-identical between the two entry points (the same kernel; the split
combine merges partials in a fixed order), pages and live residual slots bit-identical to the
oracle's after its append, attention within 2e-4 / 1e-4 (relative lse) of the binary64 oracle.
The first call's lengths include one whose appended token completes a page (95)."""
import numpy as np
import pytest

from kvq_cases import Case, assert_attention_close, host_array, live_resid_equal, log
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import layer_wise_mixed_kvq_amd as k
    k.lib()
    return k


def _one(kvq, orc, kb, vb, H, G, lens, seed, pps):
    import torch
    L0 = np.asarray(lens, dtype=np.int32)
    c = Case(kb, vb, H=H, G=G, lens=list(L0 + 1), seed=seed)
    c.o_pages, c.o_rk, c.o_rv = orc.new_cache(kb, vb, H, c.B, c.n_phys)
    orc.pack(kb, vb, host_array(c.k), host_array(c.v), L0, c.bt, c.o_pages, c.o_rk, c.o_rv)
    c.device_setup(kvq)
    mine = c.cache
    twin = kvq.LayerCache(c.model, 0, c.B, c.maxp, n_pages=c.n_phys, block_table=c.bt_d, device=c.dev)
    l0 = torch.from_numpy(L0).to(c.dev)
    kd, vd = c.k.to(c.dev), c.v.to(c.dev)
    kvq.kvq_pack(c.model, 0, mine, kd, vd, l0)
    kvq.kvq_pack(c.model, 0, twin, kd, vd, l0)
    kn = synth.fill(seed, synth.KIND_K_NEW, 0, c.B, 1, H).view(c.B, H, 128)
    vn = synth.fill(seed, synth.KIND_V_NEW, 0, c.B, 1, H).view(c.B, H, 128)
    orc.append(kb, vb, host_array(kn), host_array(vn), L0, c.bt, c.o_pages, c.o_rk, c.o_rv)
    o_ref, l_ref = orc.decode_attn(kb, vb, H, host_array(c.q), L0 + 1, c.bt, c.o_pages, c.o_rk, c.o_rv)
    knd, vnd, q = kn.to(c.dev), vn.to(c.dev), c.q.to(c.dev)
    msl = c.maxp * 32
    out_a = torch.full((c.B, H * G, 128), 7.0, dtype=torch.float32, device=c.dev)
    lse_a = torch.full((c.B, H * G), 7.0, dtype=torch.float32, device=c.dev)
    kvq.kvq_append_decode_attn_noalloc(c.model, 0, mine, knd, vnd, l0, q, msl, out_a, lse_a, pages_per_split=pps)
    out_b, lse_b = kvq.kvq_append_decode_attn(c.model, 0, twin, knd, vnd, l0, q, msl, pages_per_split=pps)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b), "no-alloc and workspace results differ"
    pages = mine.pages.cpu().numpy()
    assert np.array_equal(pages, c.o_pages), "pages differ from the oracle"
    assert np.array_equal(pages, twin.pages.cpu().numpy()), "pages differ between the entry points"
    rk, rv = host_array(mine.resid_k), host_array(mine.resid_v)
    assert live_resid_equal(rk, c.o_rk, L0 + 1) and live_resid_equal(rv, c.o_rv, L0 + 1), "residual slots"
    assert_attention_close(out_a.cpu().numpy(), lse_a.cpu().numpy(), o_ref, l_ref, "no-alloc")


def test_noalloc_matches_workspace_entry_point(kvq, orc):
    log("no-alloc call 1: K4V2, H=4, G=4, lengths 300, 95 (page completes), 1000, 64; 4 pages per split")
    _one(kvq, orc, 4, 2, 4, 4, [300, 95, 1000, 64], 41, 4)
    log("no-alloc call 2 (smaller): K8V4, H=1, G=7, length 40; library split plan")
    _one(kvq, orc, 8, 4, 1, 7, [40], 43, 0)
