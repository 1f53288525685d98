"""GPU parity of kvq_append_decode_attn (append fused into the decode launch).

Each step appends one token per sequence and attends over pos + 1 tokens.  After every
step the cache (pages and live residual slots) must be bit-identical to the oracle's after
its append and to a twin device cache driven by kvq_append + kvq_decode_attn, and the
attention must be within 2e-4 / 1e-4 (relative lse) of the oracle's binary64 result.
Starting lengths 29, 62, 0 make the steps cover a flush whose page is the sequence's first
(no pool pages attended), a flush after one pool page, the very first token, and plain
residual appends; split sizes vary between steps.
"""
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


def _prefill(kvq, orc, c, L0):
    """Oracle and two device caches holding the first L0[b] tokens of each sequence."""
    import torch
    c.o_pages, c.o_rk, c.o_rv = orc.new_cache(c.kb, c.vb, c.H, c.B, c.n_phys)
    kh, vh = host_array(c.k), host_array(c.v)
    orc.pack(c.kb, c.vb, kh, vh, L0, c.bt, c.o_pages, c.o_rk, c.o_rv)
    c.device_setup(kvq)
    fused = c.cache
    twin = kvq.LayerCache(c.model, 0, c.B, c.maxp, n_pages=c.n_phys, block_table=c.bt_d, device=c.dev)
    l0 = torch.from_numpy(np.asarray(L0, np.int32)).to(c.dev)
    kd, vd = c.k.to(c.dev), c.v.to(c.dev)
    kvq.kvq_pack(c.model, 0, fused, kd, vd, l0)
    kvq.kvq_pack(c.model, 0, twin, kd, vd, l0)
    return fused, twin


@pytest.mark.parametrize("kb,vb,G", [(4, 2, 4), (8, 8, 4), (2, 4, 7), (8, 4, 1), (4, 8, 16)])
def test_fused_steps_match_oracle_and_two_launch_path(kvq, orc, kb, vb, G):
    import torch
    L0 = np.array([29, 62, 0], dtype=np.int32)
    steps, H = 4, 2
    c = Case(kb, vb, H=H, G=G, lens=list(L0 + steps), seed=kb * 7 + vb + G)
    fused, twin = _prefill(kvq, orc, c, L0)
    q = c.q.to(c.dev)
    msl = c.maxp * 32
    for s in range(steps):
        pos = L0 + s
        kn = synth.fill(c.seed, synth.KIND_K_NEW, 0, c.B, 1, H, t0=s).view(c.B, H, 128)
        vn = synth.fill(c.seed, synth.KIND_V_NEW, 0, c.B, 1, H, t0=s).view(c.B, H, 128)
        log(f"fused kb={kb} vb={vb} G={G} step {s} pos={pos.tolist()}")
        orc.append(kb, vb, host_array(kn), host_array(vn), pos, c.bt, c.o_pages, c.o_rk, c.o_rv)
        o_ref, l_ref = orc.decode_attn(kb, vb, H, host_array(c.q), pos + 1, c.bt, c.o_pages, c.o_rk, c.o_rv)
        pos_d = torch.from_numpy(pos).to(c.dev)
        knd, vnd = kn.to(c.dev), vn.to(c.dev)
        pps = [0, 1, 2, 0][s]
        out, lse = kvq.kvq_append_decode_attn(c.model, 0, fused, knd, vnd, pos_d, q, msl, pages_per_split=pps)
        kvq.kvq_append(c.model, 0, twin, knd, vnd, pos_d)
        out2, lse2 = kvq.kvq_decode_attn(c.model, 0, twin, q, pos_d + 1, msl, pages_per_split=pps)
        torch.cuda.synchronize()
        pages = fused.pages.cpu().numpy()
        assert np.array_equal(pages, c.o_pages), f"step {s}: pages differ from the oracle"
        assert np.array_equal(pages, twin.pages.cpu().numpy()), f"step {s}: pages differ from append + decode"
        lens = pos + 1
        rk, rv = host_array(fused.resid_k), host_array(fused.resid_v)
        assert live_resid_equal(rk, c.o_rk, lens) and live_resid_equal(rv, c.o_rv, lens), f"step {s}: residual"
        assert live_resid_equal(rk, host_array(twin.resid_k), lens), f"step {s}: residual vs append"
        assert_attention_close(out.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"fused step {s}")
        assert_attention_close(out2.cpu().numpy(), lse2.cpu().numpy(), o_ref, l_ref, f"two-launch step {s}")


def test_fused_bad_positions_are_nan_others_unaffected(kvq, orc):
    """pos + 1 beyond max_seq_len, or pos < 0, gives NaN for that sequence and writes
    nothing for it; the other sequences are unaffected."""
    import torch
    L0 = np.array([40, 10, 33], dtype=np.int32)
    H, kb, vb = 2, 4, 4
    c = Case(kb, vb, H=H, G=2, lens=list(L0 + 1), seed=5)
    fused, _ = _prefill(kvq, orc, c, L0)
    kn = synth.fill(c.seed, synth.KIND_K_NEW, 0, c.B, 1, H).view(c.B, H, 128)
    vn = synth.fill(c.seed, synth.KIND_V_NEW, 0, c.B, 1, H).view(c.B, H, 128)
    pos = np.array([40, -1, 33], dtype=np.int32)          # max_seq_len 40: sequence 0 attends 41
    rk_before = host_array(fused.resid_k).copy()
    out, lse = kvq.kvq_append_decode_attn(c.model, 0, fused, kn.to(c.dev), vn.to(c.dev),
                                          torch.from_numpy(pos).to(c.dev), c.q.to(c.dev), 40)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for b in (0, 1):
        assert np.all(np.isnan(out[b])) and np.all(np.isnan(lse[b])), f"sequence {b} not NaN"
        assert np.array_equal(host_array(fused.resid_k)[b], rk_before[b]), f"sequence {b} written"
    # sequence 2 alone through the oracle
    rk2, rv2 = c.o_rk[[2]].copy(), c.o_rv[[2]].copy()
    bt2 = np.ascontiguousarray(c.bt[[2]])
    orc.append(kb, vb, host_array(kn)[[2]], host_array(vn)[[2]], pos[[2]], bt2, c.o_pages, rk2, rv2)
    o_ref, l_ref = orc.decode_attn(kb, vb, H, host_array(c.q)[[2]], pos[[2]] + 1, bt2, c.o_pages, rk2, rv2)
    assert_attention_close(out[2:], lse[2:], o_ref, l_ref, "valid sequence")


def test_fused_graph_replay_matches_eager(kvq, orc):
    """The fused step captured in a HIP graph: every replay (same pos, so idempotent) equals
    the eager result bit for bit, with eager work and synchronizations between replays."""
    import torch
    L0 = np.array([63, 40, 31], dtype=np.int32)
    c = Case(4, 2, H=2, G=4, lens=list(L0 + 1), seed=33)
    fused, _ = _prefill(kvq, orc, c, L0)
    kn = synth.fill(c.seed, synth.KIND_K_NEW, 0, c.B, 1, 2).view(c.B, 2, 128).to(c.dev)
    vn = synth.fill(c.seed, synth.KIND_V_NEW, 0, c.B, 1, 2).view(c.B, 2, 128).to(c.dev)
    pos = torch.from_numpy(L0).to(c.dev)
    q = c.q.to(c.dev)
    msl = c.maxp * 32
    ws = kvq.new_workspace(c.model, c.B, msl)
    out = torch.empty((c.B, 8, 128), dtype=torch.float32, device=c.dev)
    lse = torch.empty((c.B, 8), dtype=torch.float32, device=c.dev)

    def step():
        kvq.kvq_append_decode_attn(c.model, 0, fused, kn, vn, pos, q, msl, out=out, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    ref_pages = fused.pages.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {i} differs"
        assert torch.equal(fused.pages, ref_pages), f"replay {i}: pages changed"
