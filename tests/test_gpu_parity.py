"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Packed codes, scales, zeros and live residual slots must be bit-exact; attention must be
within 2e-4 (max abs) of the oracle's binary64 result, with |d lse| <= 1e-4 * max(1, |lse|).
Sizes span several pages, several split-K work items and ragged tails.
"""
import numpy as np
import pytest

from kvq_cases import Case, assert_attention_close, host_array, live_resid_equal, log

pytestmark = pytest.mark.gpu

PAIRS = [(k, v) for k in (2, 4, 8) for v in (2, 4, 8)]


@pytest.fixture(scope="module")
def kvq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import layer_wise_mixed_kvq_amd as k
    k.lib()
    return k


def test_pack_long_source_grid(kvq, orc):
    """Sources longer than 65,535 pages per sequence: the pack launches its page-fastest grid
    (the heads-fastest one would exceed a grid's y extent). The two short sequences in them
    are packed bit-exact against the oracle."""
    import torch
    c = Case(4, 2, H=2, G=1, lens=[100, 70], seed=77)
    log(f"pack from a {65536 * 32 + 32}-token source buffer, lens={c.lens.tolist()}")
    c.oracle_pack(orc)
    c.device_setup(kvq)
    t_long = 65536 * 32 + 32
    k = torch.zeros((c.B, t_long, c.H, 128), dtype=torch.bfloat16, device=c.dev)
    v = torch.zeros_like(k)
    k[:, :c.T] = c.k.to(c.dev)
    v[:, :c.T] = c.v.to(c.dev)
    kvq.kvq_pack(c.model, 0, c.cache, k, v, c.lens_d)
    torch.cuda.synchronize()
    assert np.array_equal(c.cache.pages.cpu().numpy(), c.o_pages)
    assert live_resid_equal(host_array(c.cache.resid_k), c.o_rk, c.lens)
    assert live_resid_equal(host_array(c.cache.resid_v), c.o_rv, c.lens)
    del k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kb,vb", PAIRS)
def test_pack_bit_exact(kvq, orc, kb, vb):
    c = Case(kb, vb, H=2, G=1, lens=[77, 64, 5, 0, 200], seed=kb * 10 + vb)
    log(f"pack kb={kb} vb={vb} lens={c.lens.tolist()}")
    c.oracle_pack(orc)
    c.device_setup(kvq)
    c.device_pack(kvq)
    pages = c.cache.pages.cpu().numpy()
    assert np.array_equal(pages, c.o_pages), "packed pages differ"
    assert live_resid_equal(host_array(c.cache.resid_k), c.o_rk, c.lens)
    assert live_resid_equal(host_array(c.cache.resid_v), c.o_rv, c.lens)


@pytest.mark.parametrize("kb,vb", [(8, 4), (4, 2), (2, 8)])
def test_pack_fp32_source_bit_exact(kvq, orc, kb, vb):
    c = Case(kb, vb, H=3, G=1, lens=[96, 45, 130], seed=5, src="f32")
    log(f"pack fp32 kb={kb} vb={vb}")
    c.oracle_pack(orc)
    c.device_setup(kvq)
    c.device_pack(kvq)
    assert np.array_equal(c.cache.pages.cpu().numpy(), c.o_pages)
    assert live_resid_equal(host_array(c.cache.resid_k), c.o_rk, c.lens)
    assert live_resid_equal(host_array(c.cache.resid_v), c.o_rv, c.lens)


def test_config_single_layer_k8v4_fp32(kvq, orc):
    """One layer, batch 1, 1 KV head with 4 query heads, head_dim 128, 512 tokens, K8V4,
    fp32 K, V and q, 4 of 128 key channels x10."""
    c = Case(8, 4, H=1, G=4, lens=[512], seed=2024, src="f32", q_dtype="f32", n_outliers=4, shuffle=False,
             extra_pages=0)
    log("single-layer K8V4 fp32 L=512")
    c.oracle_pack(orc)
    c.device_setup(kvq)
    c.device_pack(kvq)
    assert np.array_equal(c.cache.pages.cpu().numpy(), c.o_pages)
    o_ref, l_ref = c.oracle_decode(orc)
    for pps in (0, 1, 16):
        out, lse = c.device_decode(kvq, pages_per_split=pps)
        assert_attention_close(out, lse, o_ref, l_ref, f"pps={pps}")


@pytest.mark.parametrize("kb,vb", PAIRS)
@pytest.mark.parametrize("G", [1, 4, 7, 12, 16])
def test_decode_parity(kvq, orc, kb, vb, G):
    c = Case(kb, vb, H=2, G=G, lens=[1, 31, 32, 33, 200, 517], seed=kb * 100 + vb * 10 + G)
    log(f"decode kb={kb} vb={vb} G={G}")
    c.oracle_pack(orc)
    c.device_setup(kvq)
    c.device_pack(kvq)
    o_ref, l_ref = c.oracle_decode(orc)
    out, lse = c.device_decode(kvq, pages_per_split=2)
    assert_attention_close(out, lse, o_ref, l_ref, f"kb={kb} vb={vb} G={G}")


@pytest.mark.parametrize("G", [4, 7])
def test_decode_four_wave_workgroups(kvq, orc, G):
    """More than 256 (sequence, KV head) pairs with G <= 8: the launch takes four-wave
    workgroups (two per CU) instead of eight; plain decode and the fused append, several
    split sizes, lengths with no full page, a ragged tail or a page about to complete."""
    import torch
    import synth
    H, B = 8, 36
    rng = np.random.default_rng(G)
    L0 = rng.integers(1, 200, B).astype(np.int32)
    L0[:4] = [1, 31, 63, 95]
    c = Case(4, 2, H=H, G=G, lens=list(L0 + 1), seed=300 + G)
    log(f"four-wave workgroups: B={B} H={H} G={G}")
    c.o_pages, c.o_rk, c.o_rv = orc.new_cache(4, 2, H, B, c.n_phys)
    orc.pack(4, 2, host_array(c.k), host_array(c.v), L0, c.bt, c.o_pages, c.o_rk, c.o_rv)
    c.device_setup(kvq)
    l0 = torch.from_numpy(L0).to(c.dev)
    kvq.kvq_pack(c.model, 0, c.cache, c.k.to(c.dev), c.v.to(c.dev), l0)
    q = c.q.to(c.dev)
    msl = c.maxp * 32
    o_ref, l_ref = orc.decode_attn(4, 2, H, host_array(c.q), L0, c.bt, c.o_pages, c.o_rk, c.o_rv)
    for pps in (0, 1, 3):
        out, lse = kvq.kvq_decode_attn(c.model, 0, c.cache, q, l0, msl, pages_per_split=pps)
        assert_attention_close(out.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"decode pps={pps}")
    kn = synth.fill(c.seed, synth.KIND_K_NEW, 0, B, 1, H).view(B, H, 128)
    vn = synth.fill(c.seed, synth.KIND_V_NEW, 0, B, 1, H).view(B, H, 128)
    orc.append(4, 2, host_array(kn), host_array(vn), L0, c.bt, c.o_pages, c.o_rk, c.o_rv)
    o_ref, l_ref = orc.decode_attn(4, 2, H, host_array(c.q), L0 + 1, c.bt, c.o_pages, c.o_rk, c.o_rv)
    out, lse = kvq.kvq_append_decode_attn(c.model, 0, c.cache, kn.to(c.dev), vn.to(c.dev), l0, q, msl,
                                          pages_per_split=2)
    torch.cuda.synchronize()
    assert np.array_equal(c.cache.pages.cpu().numpy(), c.o_pages), "pages after the fused append differ"
    assert_attention_close(out.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "fused")


@pytest.mark.parametrize("q_dtype", ["bf16", "f32"])
def test_decode_q_dtypes(kvq, orc, q_dtype):
    c = Case(4, 2, H=2, G=4, lens=[300, 64], seed=77, q_dtype=q_dtype)
    c.oracle_pack(orc)
    c.device_setup(kvq)
    c.device_pack(kvq)
    o_ref, l_ref = c.oracle_decode(orc)
    out, lse = c.device_decode(kvq)
    assert_attention_close(out, lse, o_ref, l_ref, q_dtype)


def test_split_invariance_and_determinism(kvq, orc):
    c = Case(4, 2, H=2, G=4, lens=[1000, 640, 33], seed=9)
    c.oracle_pack(orc)
    c.device_setup(kvq)
    c.device_pack(kvq)
    ref = None
    for pps in (1, 2, 7, 32, 1000):
        out, lse = c.device_decode(kvq, pages_per_split=pps)
        out2, lse2 = c.device_decode(kvq, pages_per_split=pps)
        assert np.array_equal(out, out2) and np.array_equal(lse, lse2), "not run-to-run deterministic"
        if ref is None:
            ref = (out, lse)
        else:
            assert np.abs(out - ref[0]).max() <= 1e-5
            assert np.abs(lse - ref[1]).max() <= 1e-5


def test_equal_queries_give_equal_heads(kvq, orc):
    import torch
    c = Case(2, 4, H=2, G=4, lens=[150, 90], seed=12)
    c.q = c.q[:, ::4].repeat_interleave(4, dim=1).contiguous()
    c.device_setup(kvq)
    c.device_pack(kvq)
    out, lse = c.device_decode(kvq)
    for g in range(1, 4):
        assert np.array_equal(out[:, g::4], out[:, 0::4])
        assert np.array_equal(lse[:, g::4], lse[:, 0::4])
    del torch


def test_empty_sequence_and_bounds_checks(kvq, orc):
    """Length 0 gives out = 0 and lse = -inf.  A length above max_seq_len, or a block-table
    entry outside the pool, is caught by the kernel's own bounds checks and yields NaN for
    that sequence only; the other sequences are unaffected."""
    import torch
    c = Case(4, 4, H=2, G=2, lens=[0, 70, 64], seed=3)
    c.oracle_pack(orc)
    c.device_setup(kvq)
    c.device_pack(kvq)
    out, lse = c.device_decode(kvq)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    o_ref, l_ref = c.oracle_decode(orc, lens=[1, 70, 64])
    assert_attention_close(out[1:], lse[1:], o_ref[1:], l_ref[1:], "others")
    # sequence 1 claims more tokens than max_seq_len
    out, lse = c.device_decode(kvq, lens=[0, 200, 64], max_seq_len=96)
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(lse[1]))
    assert_attention_close(out[2:], lse[2:], o_ref[2:], l_ref[2:], "others")
    # sequence 2 points at a physical page outside the pool
    bt = c.bt.copy()
    bt[2, 1] = c.n_phys
    c.cache.block_table.copy_(torch.from_numpy(bt))
    out, lse = c.device_decode(kvq)
    assert np.all(np.isnan(out[2])) and np.isnan(lse[2]).all()
    assert_attention_close(out[1:2], lse[1:2], o_ref[1:2], l_ref[1:2], "others")


@pytest.mark.parametrize("kb,vb", [(4, 2), (8, 8), (2, 4)])
def test_append_parity_and_prefix_invariance(kvq, orc, kb, vb):
    """Prefill 58 tokens, then append 12 one at a time (the append at position 63 flushes
    page 1).  Pages and live residual slots must equal the oracle's after the same calls,
    and equal a one-shot prefill of all 70 tokens."""
    import torch
    B, H, G, L0, L1 = 3, 2, 4, 58, 70
    c = Case(kb, vb, H=H, G=G, lens=[L1] * B, seed=kb + 5 * vb)
    full_dev_pages = None
    # one-shot reference on the device
    c.device_setup(kvq)
    c.device_pack(kvq)
    full_dev_pages = c.cache.pages.cpu().numpy().copy()
    full_rk = host_array(c.cache.resid_k).copy()
    # incremental, oracle and device side by side
    c.o_pages, c.o_rk, c.o_rv = orc.new_cache(kb, vb, H, B, c.n_phys)
    kh, vh = host_array(c.k), host_array(c.v)
    orc.pack(kb, vb, np.ascontiguousarray(kh[:, :L0]), np.ascontiguousarray(vh[:, :L0]), [L0] * B, c.bt,
             c.o_pages, c.o_rk, c.o_rv)
    c.device_setup(kvq)
    kd, vd = c.k.to(c.dev), c.v.to(c.dev)
    kvq.kvq_pack(c.model, 0, c.cache, kd[:, :L0].contiguous(), vd[:, :L0].contiguous(),
                 torch.full((B,), L0, dtype=torch.int32, device=c.dev))
    for t in range(L0, L1):
        log(f"append kb={kb} vb={vb} pos={t}")
        orc.append(kb, vb, np.ascontiguousarray(kh[:, t]), np.ascontiguousarray(vh[:, t]), [t] * B, c.bt,
                   c.o_pages, c.o_rk, c.o_rv)
        pos = torch.full((B,), t, dtype=torch.int32, device=c.dev)
        kvq.kvq_append(c.model, 0, c.cache, kd[:, t].contiguous(), vd[:, t].contiguous(), pos)
        # idempotent: repeating the same append changes nothing
        kvq.kvq_append(c.model, 0, c.cache, kd[:, t].contiguous(), vd[:, t].contiguous(), pos)
    torch.cuda.synchronize()
    pages = c.cache.pages.cpu().numpy()
    assert np.array_equal(pages, c.o_pages), "append pages differ from the oracle"
    assert np.array_equal(pages, full_dev_pages), "prefill != prefix prefill + appends"
    lens = [L1] * B
    assert live_resid_equal(host_array(c.cache.resid_k), c.o_rk, lens)
    assert live_resid_equal(host_array(c.cache.resid_v), c.o_rv, lens)
    assert live_resid_equal(host_array(c.cache.resid_k), full_rk, lens)
    o_ref, l_ref = c.oracle_decode(orc)
    out, lse = c.device_decode(kvq)
    assert_attention_close(out, lse, o_ref, l_ref, "after appends")


def test_graph_replay_matches_eager(kvq, orc):
    """append + decode captured in a HIP graph: every replay, with eager work and
    synchronizations in between, equals the eager result bit for bit."""
    import torch
    c = Case(4, 2, H=2, G=4, lens=[130, 64], seed=21)
    c.device_setup(kvq)
    c.device_pack(kvq)
    kn = torch.zeros((c.B, c.H, 128), dtype=torch.bfloat16, device=c.dev) + 0.5
    vn = torch.zeros_like(kn) - 0.25
    pos = c.lens_d.clone()
    lens1 = c.lens_d + 1
    q = c.q.to(c.dev)
    ws = kvq.new_workspace(c.model, c.B, c.maxp * 32)
    out = torch.empty((c.B, c.H * c.G, 128), dtype=torch.float32, device=c.dev)
    lse = torch.empty((c.B, c.H * c.G), dtype=torch.float32, device=c.dev)

    def step():
        kvq.kvq_append(c.model, 0, c.cache, kn, vn, pos)
        kvq.kvq_decode_attn(c.model, 0, c.cache, q, lens1, c.maxp * 32, out=out, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        out.zero_()
        lse.zero_()
        kvq.kvq_decode_attn(c.model, 0, c.cache, q, lens1, c.maxp * 32, workspace=ws)   # eager work between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {i} differs"


def _tie_tile(bits, T, H, seed):
    """fp32 source whose groups get min 0 and max (2^bits - 1) * S with S = 1434/2048 (an
    fp16 value, so the stored scale is exactly S and the zero 0), every other value being
    fl((k + 0.5) * S) moved by -2 .. +2 ulps: quotients at and beside half-integers, where
    any departure from one correctly rounded binary32 division changes the code."""
    L = (1 << bits) - 1
    S = np.float32(1434.0 / 2048.0)
    rng = np.random.default_rng(seed)
    x = ((rng.integers(0, L, (1, T, H, 128)).astype(np.float32) + np.float32(0.5)) * S).astype(np.float32)
    steps = rng.integers(-2, 3, x.shape)
    for _ in range(2):
        x = np.where(steps > 0, np.nextafter(x, np.float32(np.inf)), np.where(steps < 0, np.nextafter(x, np.float32(0)), x))
        steps = steps - np.sign(steps)
    return x.astype(np.float32), np.float32(L) * S


@pytest.mark.parametrize("kb,vb,kmode", [(2, 2, 0), (4, 4, 0), (8, 8, 0), (4, 2, 0), (4, 4, 1), (2, 8, 1)])
def test_pack_rounding_ties_bit_exact(kvq, orc, kb, vb, kmode):
    """Quotients at and beside half-integers (rounding ties of the code rule) pack
    bit-exactly as the oracle does, in both key modes."""
    import torch
    T, H = 64, 2
    c = Case(kb, vb, H=H, G=1, lens=[T], seed=kb * 7 + vb + kmode, src="f32", kmode=kmode)
    kt, Lk = _tie_tile(kb, T, H, 1 + kb)
    vt, Lv = _tie_tile(vb, T, H, 2 + vb)
    # group extremes: per-channel keys over each page's 32 tokens, per-token groups over
    # 32 channels (values, and keys in the per-token mode)
    if kmode == 0:
        kt[:, 0::32], kt[:, 1::32] = 0.0, Lk
    else:
        kt[..., 0::32], kt[..., 1::32] = 0.0, Lk
    vt[..., 0::32], vt[..., 1::32] = 0.0, Lv
    c.k, c.v = torch.from_numpy(kt), torch.from_numpy(vt)
    log(f"rounding ties kb={kb} vb={vb} kmode={kmode}")
    c.oracle_pack(orc)
    c.device_setup(kvq)
    c.device_pack(kvq)
    assert np.array_equal(c.cache.pages.cpu().numpy(), c.o_pages)
