"""GPU parity at the benchmark's full sizes, in the launch configuration bench.py times.

The device builds the whole cache exactly as the benchmark does and runs one full step
(append + decode attention for every layer, library-chosen split plan).  The oracle then
recomputes (layer, sequence) pairs one at a time from the same seeded inputs, regenerated on
the host, in a thread pool (the oracle and the generator are C called through ctypes, which
releases the interpreter lock):
  * packed pages (reached through the shared, possibly shuffled block table) and the live
    residual slots after the append: bit-exact;
  * out and lse of that sequence: within 2e-4 / 1e-4 (relative) of the binary64 oracle.
The Llama step is compared at every (layer, sequence) pair, the Qwen step at every layer for
eight sequences; two more steps start one token short of a page boundary (contexts 4095 and
8191), so that every sequence's append completes and quantizes a page inside the fused launch.
The prefill pack workload is checked on sampled pages.
"""
import numpy as np
import pytest

from kvq_cases import assert_attention_close, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import layer_wise_mixed_kvq_amd as k
    k.lib()
    return k


def _bits(t):
    import torch
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _oracle_sequence(orc, cfg, l, b, C):
    """Oracle cache and attention of sequence b, layer l: pack C tokens, append token C,
    attend over C + 1 tokens."""
    import synth
    seed, H, Hq = cfg["seed"], cfg["n_kv_heads"], cfg["n_q_heads"]
    kb, vb = cfg["pairs"][l]
    cm = synth.outlier_mult(seed, l, H, cfg["n_outliers"])
    maxp = (C + 1 + 31) // 32
    bt = np.arange(maxp, dtype=np.int32).reshape(1, maxp)
    k = synth.fill(seed, synth.KIND_K, l, 1, C, H, b0=b, chan_mult=cm)
    v = synth.fill(seed, synth.KIND_V, l, 1, C, H, b0=b)
    kn = synth.fill(seed, synth.KIND_K_NEW, l, 1, 1, H, b0=b, chan_mult=cm).view(1, H, 128)
    vn = synth.fill(seed, synth.KIND_V_NEW, l, 1, 1, H, b0=b).view(1, H, 128)
    q = synth.fill(seed, synth.KIND_Q, l, 1, 1, Hq, b0=b).view(1, Hq, 128)
    pages, rk, rv = orc.new_cache(kb, vb, H, 1, maxp)
    orc.pack(kb, vb, _bits(k), _bits(v), [C], bt, pages, rk, rv)
    orc.append(kb, vb, _bits(kn), _bits(vn), [C], bt, pages, rk, rv)
    out, lse = orc.decode_attn(kb, vb, H, _bits(q), [C + 1], bt, pages, rk, rv)
    return pages, rk, rv, out, lse


def _workers():
    import os
    return max(1, min(16, os.cpu_count() or 1))


def _check_samples(orc, stack, samples, what):
    """Every (layer, sequence) pair of `samples`, the oracle's side computed in a thread pool."""
    from concurrent.futures import ThreadPoolExecutor
    import synth
    import torch
    cfg = stack.cfg
    synth.fill(0, synth.KIND_K, 0, 1, 1, 1)          # load the host generator before the threads start
    log(f"{what}: {len(samples)} (layer, sequence) pairs, {_workers()} oracle threads")
    with ThreadPoolExecutor(_workers()) as ex:
        futs = [ex.submit(_oracle_sequence, orc, cfg, l, b, int(stack.lens[b])) for l, b in samples]
        for (l, b), fut in zip(samples, futs):
            C = int(stack.lens[b])
            pages_o, rk_o, rv_o, out_o, lse_o = fut.result()
            n_full = (C + 1) // 32
            ids = torch.from_numpy(stack.block_table_host[b, :n_full].astype(np.int64)).to(stack.caches[l].pages.device)
            dev_pages = stack.caches[l].pages.index_select(0, ids).cpu().numpy()
            assert np.array_equal(dev_pages, pages_o[:n_full]), f"{what}: layer {l} seq {b}: packed pages differ"
            n_live = (C + 1) % 32
            rk_d = _bits(stack.caches[l].resid_k[b].cpu())
            rv_d = _bits(stack.caches[l].resid_v[b].cpu())
            assert np.array_equal(rk_d[:, :n_live], rk_o[0][:, :n_live]), f"{what}: layer {l} seq {b}: resid K"
            assert np.array_equal(rv_d[:, :n_live], rv_o[0][:, :n_live]), f"{what}: layer {l} seq {b}: resid V"
            out_d = stack.out[l][b:b + 1].cpu().numpy()
            lse_d = stack.lse[l][b:b + 1].cpu().numpy()
            assert_attention_close(out_d, lse_d, out_o, lse_o, f"{what}: layer {l} seq {b}")
    log(f"{what}: all {len(samples)} pairs match")


def _full_step(name, **override):
    import torch
    import bench
    stack = bench.DecodeStack(dict(bench.CONFIGS[name], **override), torch.device("cuda:0"))
    stack.step(with_append=True)
    torch.cuda.synchronize()
    return stack


def _release():
    import gc
    import torch
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_llama_c325_full_size(kvq, orc):
    """32 layers, 32/8 heads, batch 16, 4096 cached + 1 appended token, C3.25 table: every
    (layer, sequence) pair."""
    stack = _full_step("llama")
    _check_samples(orc, stack, [(l, b) for l in range(32) for b in range(16)], "llama")
    del stack
    _release()


def test_llama_c325_full_size_flushing_step(kvq, orc):
    """As above with 4095 cached tokens: every sequence's appended token completes page 127,
    which the fused launch quantizes and attends over; every (layer, sequence) pair."""
    stack = _full_step("llama", context=4095)
    _check_samples(orc, stack, [(l, b) for l in range(32) for b in range(16)], "llama flush")
    del stack
    _release()


QWEN_SEQS = [0, 9, 18, 27, 36, 45, 54, 63]


def test_qwen_c40_full_size(kvq, orc):
    """28 layers, 28/4 heads (G = 7), batch 64, 8192 cached + 1 appended token, C4.0 table:
    every layer, eight sequences."""
    stack = _full_step("qwen")
    _check_samples(orc, stack, [(l, b) for l in range(28) for b in QWEN_SEQS], "qwen")
    del stack
    _release()


def test_qwen_c40_full_size_flushing_step(kvq, orc):
    """8191 cached tokens: every append completes page 255 inside the fused launch; every
    layer, four sequences."""
    stack = _full_step("qwen", context=8191)
    _check_samples(orc, stack, [(l, b) for l in range(28) for b in QWEN_SEQS[::2]], "qwen flush")
    del stack
    _release()


def test_ragged_paged_full_size(kvq, orc):
    """Batch 256, lengths U{1024..32768}, physical pages a seeded permutation shared by all
    layers.  Samples: the shortest and the longest sequence, one whose append flushes a
    page (length mod 32 == 31), one more; every third layer."""
    stack = _full_step("ragged")
    lens = stack.lens
    flush = int(np.nonzero(lens % 32 == 31)[0][0]) if np.any(lens % 32 == 31) else 1
    seqs = [int(np.argmin(lens)), int(np.argmax(lens)), flush, 100]
    samples = [(l, b) for l in range(0, 32, 3) for b in seqs]
    _check_samples(orc, stack, samples, "ragged")
    del stack
    _release()


def test_prefill_pack_full_size(kvq, orc):
    """kvq_pack of 32768 bf16 tokens (batch 1) for all 32 layers of the C3.25 table, as the
    pack benchmark calls it; sampled pages of sampled layers are bit-exact."""
    import torch
    import bench
    import synth
    cfg = bench.CONFIGS["pack"]
    dev = torch.device("cuda:0")
    B, H, T = cfg["batch"], cfg["n_kv_heads"], cfg["context"]
    model = kvq.Model(cfg["pairs"], cfg["n_q_heads"], H)
    maxp = T // 32
    bt = torch.arange(B * maxp, dtype=torch.int32, device=dev).view(B, maxp)
    seq = torch.full((B,), T, dtype=torch.int32, device=dev)
    for l in [0, 4, 27, 31]:
        kb, vb = cfg["pairs"][l]
        cache = kvq.LayerCache(model, l, B, maxp, block_table=bt, device=dev)
        cm = synth.outlier_mult(cfg["seed"], l, H, cfg["n_outliers"])
        k = synth.fill(cfg["seed"], synth.KIND_K, l, B, T, H, chan_mult=cm, device=dev)
        v = synth.fill(cfg["seed"], synth.KIND_V, l, B, T, H, device=dev)
        kvq.kvq_pack(model, l, cache, k, v, seq)
        torch.cuda.synchronize()
        del k, v
        for g in [0, 1, 500, maxp - 1]:
            log(f"pack: layer {l} {(kb, vb)} page {g}")
            kh = synth.fill(cfg["seed"], synth.KIND_K, l, 1, 32, H, t0=32 * g, chan_mult=cm)
            vh = synth.fill(cfg["seed"], synth.KIND_V, l, 1, 32, H, t0=32 * g)
            po, rko, rvo = orc.new_cache(kb, vb, H, 1, 1)
            orc.pack(kb, vb, _bits(kh), _bits(vh), [32], np.zeros((1, 1), dtype=np.int32), po, rko, rvo)
            assert np.array_equal(cache.pages[g].cpu().numpy(), po[0]), f"pack layer {l} page {g} differs"
        del cache
    torch.cuda.empty_cache()
