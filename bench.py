#!/usr/bin/env python3
"""Benchmark of the mixed-precision KV decode hot path on one MI355X.

Default workload (the headline): a Llama-3.1-8B-shaped stack -- 32 layers, 32 query heads,
8 KV heads, head_dim 128 -- with the 3.25-bit per-layer table (layers 0-2 and 31 K4V8, 24
layers K4V2, 4 layers K2V2), batch 16, 4096 cached tokens per sequence.  One step is one
decode step of the whole stack: for every layer, kvq_append of the new token (position
4096) and kvq_decode_attn over the 4097 tokens.  Throughput follows the pages' definition:
generated tokens per second = batch / step time
[KVTuner OpenReview discussion (paperhub.cn/paper/zDwipF6h06), reply to reviewer 2,
section 1, "Throughput definition"].

Inputs are seeded synthetic tensors (synth/), generated on the device; the timed region
starts with the packed cache resident in HBM.  The step is captured once as a HIP graph and
replayed (no allocation or host work inside the timed region).

Prints ONE JSON line.  Other workloads: --config qwen | pack | single | copy (a plain
streaming kernel of known size: the measured bandwidth ceiling, and the calibration of the
HBM byte counters).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, vendor figure
LLAMA_C325 = [(4, 8)] * 3 + [(4, 2)] * 24 + [(2, 2)] * 4 + [(4, 8)]
QWEN_C40 = [(8, 4)] * 4 + [(4, 4)] * 4 + [(4, 2)] * 16 + [(8, 4)] * 4
# the machinoai page's 32-layer example: 8 sensitive layers kept in BF16, 24 in FP8; the
# sensitive ones here are the boundary layers (first four and last four)
BF16_FP8_MIX = ["bf16"] * 4 + ["fp8"] * 24 + ["bf16"] * 4
# FP8 scales per (layer, KV head): the synthetic data's bound over 448 (K: |x| < 60 with the
# x10 outlier channels, V: |x| < 6)
FP8_SCALES = (60.0 / 448.0, 6.0 / 448.0)


def layer_spec(entry, k_mode=0):
    """(key bits, value bits, oracle format code, head-page bytes) of one table entry:
    (kb, vb) integer codes, "fp8" or "bf16"."""
    if entry == "fp8":
        return 8, 8, 2, 8192
    if entry == "bf16":
        return 16, 16, 3, 16384
    kb, vb = entry
    return kb, vb, k_mode, 512 * (kb + vb + 2)

CONFIGS = {
    "llama": dict(workload="llama3.1-8b-shape C3.25 decode step (append + attention, 32 layers)",
                  pairs=LLAMA_C325, n_q_heads=32, n_kv_heads=8, batch=16, context=4096, n_outliers=3,
                  seed=20250204),
    "qwen": dict(workload="qwen2.5-7b-shape C4.0 decode step (append + attention, 28 layers)",
                 pairs=QWEN_C40, n_q_heads=28, n_kv_heads=4, batch=64, context=8192, n_outliers=3,
                 seed=20250205),
    "single": dict(workload="single layer K8V4, GQA 4, 512 tokens, fp32 K/V/q (attention only)",
                   pairs=[(8, 4)], n_q_heads=4, n_kv_heads=1, batch=1, context=512, n_outliers=4,
                   seed=2024, f32=True, append=False),
    "ragged": dict(workload="llama3.1-8b-shape C3.25 paged decode step, batch 256, lengths U{1024..32768}, "
                            "shuffled page pool (append + attention, 32 layers)",
                   pairs=LLAMA_C325, n_q_heads=32, n_kv_heads=8, batch=256, ragged=(1024, 32768), shuffle=True,
                   n_outliers=3, seed=20250207),
    "pack": dict(workload="prefill pack, llama3.1-8b shape C3.25, 32768 tokens, batch 1 (32 layers)",
                 pairs=LLAMA_C325, n_q_heads=32, n_kv_heads=8, batch=1, context=32768, n_outliers=3,
                 seed=20250206),
    "ktoken": dict(workload="llama3.1-8b-shape C3.25 decode step with per-token keys in every layer "
                            "(append + attention, 32 layers)",
                   pairs=LLAMA_C325, n_q_heads=32, n_kv_heads=8, batch=16, context=4096, n_outliers=3,
                   seed=20250204, k_mode=1),
    "bf16fp8": dict(workload="llama3.1-8b-shape BF16/FP8 per-layer mix (layers 0-3 and 28-31 BF16, 4-27 FP8 "
                             "E4M3 with per-head scales) decode step (append + attention, 32 layers)",
                    pairs=BF16_FP8_MIX, n_q_heads=32, n_kv_heads=8, batch=16, context=4096, n_outliers=3,
                    seed=20250208),
    "formats": dict(workload="llama3.1-8b shape, B=16, 4096 cached tokens, 32 layers: decode step tokens/s of "
                             "all-BF16, calibrated all-FP8, the 8 BF16 + 24 FP8 mix and the C3.25 integer table"),
    "copy": dict(workload="streaming copy: 1 GiB int32 read + 1 GiB written (torch bitwise_not)"),
    "sweep": dict(workload="uniform-pair sweep, llama3.1-8b shape, 32 layers: decode step tokens/s per table "
                           "relative to KV8 at the (batch, input length) points of the pages' throughput table "
                           "and at (16, 4096)"),
}

# per-layer tables of the sweep: uniform pairs of the pages' throughput comparison and the
# mixed 3.25-bit table
SWEEP_TABLES = {"KV8": [(8, 8)] * 32, "K8V4": [(8, 4)] * 32, "KV4": [(4, 4)] * 32, "K4V2": [(4, 2)] * 32,
                "C3.25": LLAMA_C325}
SWEEP_SHAPES = [(64, 128), (16, 512), (8, 1024), (16, 4096)]


# sources the decode kernel is built from: a stored HBM-traffic measurement is reported only
# while they are unchanged
DECODE_SOURCES = ["layer_wise_mixed_kvq_amd/csrc/kvq_decode.hip", "layer_wise_mixed_kvq_amd/csrc/kvq_device.h",
                  "layer_wise_mixed_kvq_amd/csrc/kvq_internal.h", "layer_wise_mixed_kvq_amd/csrc/kvq_codec.h"]
PACK_SOURCES = ["layer_wise_mixed_kvq_amd/csrc/kvq_quant.hip", "layer_wise_mixed_kvq_amd/csrc/kvq_device.h",
                "layer_wise_mixed_kvq_amd/csrc/kvq_internal.h", "layer_wise_mixed_kvq_amd/csrc/kvq_codec.h"]
COPY_BYTES = 1 << 30


def measured_traffic(config, kernel="decode_kernel", sources=DECODE_SOURCES):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE / WRITE_SIZE measurement
    of this workload, or None when there is none or the kernel changed since it was taken."""
    from layer_wise_mixed_kvq_amd.profiling import source_hash
    path = os.path.join(ROOT, "profiles", f"{kernel}_{config}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_hash([os.path.join(ROOT, x) for x in sources]):
        return None
    return rec["traffic_bytes_per_launch"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def decode_alg_bytes(kb, vb, batch, H, Hq, L):
    """Bytes one decode-attention launch must move when every sequence attends over L
    tokens: the pages covering the attended tokens (codes + fp16 scale/zero), the live bf16
    residual tokens (K and V), q (bf16), out (fp32) and lse (fp32)."""
    return ragged_decode_alg_bytes(kb, vb, [L] * batch, H, Hq)


def ragged_decode_alg_bytes(kb, vb, lens, H, Hq, head_page=None):
    """As decode_alg_bytes, for sequences attending over lens[b] tokens each (head_page:
    bytes of one page of one KV head, default the integer layout of (kb, vb))."""
    hp = 512 * (kb + vb + 2) if head_page is None else head_page
    tot = 0
    for L in lens:
        full, nres = int(L) // 32, int(L) % 32
        tot += H * full * hp + H * nres * 128 * 2 * 2
    return tot + len(lens) * Hq * 128 * (2 + 4) + len(lens) * Hq * 4


def append_alg_bytes(batch, H):
    """Read of the new K/V token and its write into the residual slot (no flush)."""
    return 2 * (batch * H * 128 * 2) * 2


class DecodeStack:
    """Packed per-layer caches of a decode workload, resident on the device.

    Sequence b holds lens[b] tokens (C for every sequence, or seeded ragged lengths); its
    logical pages 0 .. ceil((lens[b]+1)/32)-1 map to physical pages through one block table
    shared by all layers (identity order, or a seeded permutation of the pool).  Sources are
    generated on the device and packed in chunks of sequences, never materialized whole."""

    CHUNK_BYTES = 2 << 30

    def __init__(self, cfg, device):
        import numpy as np
        import torch
        import synth
        import layer_wise_mixed_kvq_amd as kvq
        self.cfg = cfg
        self.kvq = kvq
        pairs = cfg["pairs"]
        self.k_mode = cfg.get("k_mode", 0)       # 0: per-channel keys, 1: per-token keys
        self.specs = [layer_spec(e, self.k_mode) for e in pairs]
        self.model = kvq.Model([e if isinstance(e, str) else (e[0], e[1], self.k_mode) for e in pairs],
                               cfg["n_q_heads"], cfg["n_kv_heads"])
        B, H = cfg["batch"], cfg["n_kv_heads"]
        seed = cfg["seed"]
        if "ragged" in cfg:
            lens = synth.seq_lens(seed, B, *cfg["ragged"]).astype(np.int64)
        else:
            lens = np.full(B, cfg["context"], dtype=np.int64)
        self.lens = lens
        self.B, self.H, self.Hq, self.C = B, H, cfg["n_q_heads"], int(lens.max())
        # a decode step appends token C and attends over C + 1 tokens; the single-layer
        # workload attends over exactly its C given tokens
        self.extra = 1 if cfg.get("append", True) else 0
        self.L = self.C + self.extra
        n_log = (lens + 1 + 31) // 32                      # pages incl. room for the appended token
        self.max_pages = int(n_log.max())
        n_phys = int(n_log.sum())
        perm = synth.permutation(seed, n_phys) if cfg.get("shuffle") else np.arange(n_phys, dtype=np.int32)
        bt = np.zeros((B, self.max_pages), dtype=np.int32)
        off = 0
        for b in range(B):
            bt[b, :n_log[b]] = perm[off:off + n_log[b]]
            off += int(n_log[b])
        self.block_table_host = bt
        self.block_table = torch.from_numpy(bt).to(device)
        self.caches, self.q, self.k_new, self.v_new, self.out, self.lse = [], [], [], [], [], []
        src_dtype = "f32" if cfg.get("f32") else "bf16"
        self.src_dtype = src_dtype
        # sequences per pack chunk: bounded source bytes (K and V)
        per_tok = H * 128 * (4 if src_dtype == "f32" else 2) * 2
        order = np.arange(B)
        fp8_scales = torch.tensor([FP8_SCALES] * H, dtype=torch.float32, device=device)
        for l, _ in enumerate(pairs):
            cache = kvq.LayerCache(self.model, l, B, self.max_pages, n_pages=n_phys, block_table=self.block_table,
                                   device=device, fp8_scales=fp8_scales if self.specs[l][2] == 2 else None)
            cm = synth.outlier_mult(seed, l, H, cfg["n_outliers"])
            b0 = 0
            while b0 < B:
                b1 = b0 + 1
                while b1 < B and (b1 + 1 - b0) * int(lens[b0:b1 + 1].max()) * per_tok <= self.CHUNK_BYTES:
                    b1 += 1
                T = int(lens[b0:b1].max())
                k = synth.fill(seed, synth.KIND_K, l, b1 - b0, T, H, b0=b0, chan_mult=cm, dtype=src_dtype, device=device)
                v = synth.fill(seed, synth.KIND_V, l, b1 - b0, T, H, b0=b0, dtype=src_dtype, device=device)
                sl = torch.from_numpy(lens[b0:b1].astype(np.int32)).to(device)
                kvq.kvq_pack(self.model, l, cache.sub_batch(b0, b1), k, v, sl)
                del k, v
                b0 = b1
            self.caches.append(cache)
            self.k_new.append(synth.fill(seed, synth.KIND_K_NEW, l, B, 1, H, chan_mult=cm, device=device).view(B, H, 128))
            self.v_new.append(synth.fill(seed, synth.KIND_V_NEW, l, B, 1, H, device=device).view(B, H, 128))
            qd = "f32" if src_dtype == "f32" else "bf16"
            self.q.append(synth.fill(seed, synth.KIND_Q, l, B, 1, self.Hq, dtype=qd, device=device).view(B, self.Hq, 128))
            self.out.append(torch.empty((B, self.Hq, 128), dtype=torch.float32, device=device))
            self.lse.append(torch.empty((B, self.Hq), dtype=torch.float32, device=device))
        torch.cuda.synchronize()
        del order
        self.pos = torch.from_numpy(lens.astype(np.int32)).to(device)
        self.attend = lens + self.extra
        self.seq_len = torch.from_numpy(self.attend.astype(np.int32)).to(device)
        self.workspace = kvq.new_workspace(self.model, B, self.L, 0, device)

    def decode_layer(self, l):
        self.kvq.kvq_decode_attn(self.model, l, self.caches[l], self.q[l], self.seq_len, self.L,
                                 out=self.out[l], lse=self.lse[l], workspace=self.workspace)

    def step(self, with_append=True, fused=True):
        """One decode step over every layer: the new token's append (fused into the attention
        launch, or as its own kvq_append launch) and attention over C + 1 tokens."""
        for l in range(len(self.caches)):
            if with_append and fused:
                self.kvq.kvq_append_decode_attn(self.model, l, self.caches[l], self.k_new[l], self.v_new[l],
                                                self.pos, self.q[l], self.L, out=self.out[l], lse=self.lse[l],
                                                workspace=self.workspace)
                continue
            if with_append:
                self.kvq.kvq_append(self.model, l, self.caches[l], self.k_new[l], self.v_new[l], self.pos)
            self.decode_layer(l)

    def alg_bytes(self, with_append=True):
        tot = sum(self.decode_bytes())
        if with_append:
            tot += len(self.cfg["pairs"]) * append_alg_bytes(self.B, self.H)
        return tot

    def decode_bytes(self):
        return [ragged_decode_alg_bytes(kb, vb, self.attend, self.H, self.Hq, hp) for kb, vb, _, hp in self.specs]


def capture(fn):
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


# After the requested warmup replays, untimed replays continue until the GPU has been busy
# for this long: the GPU raises its clocks over the first tens of milliseconds of sustained
# work, and a timed region that starts earlier measures the ramp (measured on the Llama
# step: 0.685 ms per step after 5 warmup replays, 0.648 ms after 300; single replays after
# the timed region take 0.651 ms either way).  The timed region is still exactly `steps`
# replays.
SETTLE_S = 0.25


def time_graph(g, steps, warmup):
    import torch
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < SETTLE_S:
        for _ in range(8):
            g.replay()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def replay_stats(g, reps):
    """Median and minimum of `reps` single replays, each between its own event pair (after
    the timed region; context for the mean over the timed steps)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in evs:
        e0.record()
        g.replay()
        e1.record()
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    return [t[len(t) // 2], t[0]]


def per_launch_durations(launch, n_items, reps):
    """Event pairs around every launch, on the stream the kernels run on; a GPU-side sleep
    first lets the host queue every launch ahead of the GPU so only kernel time is seen."""
    import torch
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_items)]
           for _ in range(reps)]
    torch.cuda.synchronize()
    torch.cuda._sleep(40_000_000)
    for r in range(reps):
        for i in range(n_items):
            evs[r][i][0].record()
            launch(i)
            evs[r][i][1].record()
    torch.cuda.synchronize()
    return [sum(evs[r][i][0].elapsed_time(evs[r][i][1]) for r in range(reps)) / reps for i in range(n_items)]


def quality_report(stack, n_seq=4):
    """Quantization error of each distinct layer format, on the GPU, for the first n_seq
    sequences (reported, not a pass/fail criterion): relative RMS error of the decoded K and
    V (kvq_dequant) against the bf16 / fp32 source, and of the decode attention output
    against plain fp32 attention over the unquantized tokens (the source plus the appended
    token).  Runs after the timed region."""
    import numpy as np
    import torch
    import synth
    kvq = stack.kvq
    cfg = stack.cfg
    nb = min(n_seq, stack.B)
    H, Hq, G = stack.H, stack.Hq, stack.Hq // stack.H
    T = int(stack.lens[:nb].max())
    L = T + 1
    lens_d = torch.from_numpy(stack.attend[:nb].astype(np.int32)).to(stack.seq_len.device)
    seen, rep = set(), {}
    for l, spec in enumerate(stack.specs):
        name = {2: "FP8", 3: "BF16"}.get(spec[2], f"K{spec[0]}V{spec[1]}" + ("-tok" if spec[2] == 1 else ""))
        if name in seen:
            continue
        seen.add(name)
        dev = stack.seq_len.device
        cm = synth.outlier_mult(cfg["seed"], l, H, cfg["n_outliers"])
        src = {}
        for kind, key in ((synth.KIND_K, "k"), (synth.KIND_V, "v")):
            x = synth.fill(cfg["seed"], kind, l, nb, T, H, chan_mult=cm if key == "k" else None,
                           dtype=stack.src_dtype, device=dev).float()
            new = (stack.k_new if key == "k" else stack.v_new)[l][:nb].float().view(nb, 1, H, 128)
            full = torch.cat([x, new], dim=1)                     # [nb][L][H][128]
            for b in range(nb):                                   # the new token sits at position lens[b]
                lb = int(stack.lens[b])
                full[b, lb] = new[b, 0]
                full[b, lb + 1:] = 0.0
            src[key] = full
        cache = stack.caches[l].sub_batch(0, nb)
        kd, vd = kvq.kvq_dequant(stack.model, l, cache, lens_d, L)
        mask = (torch.arange(L, device=dev).view(1, L) < lens_d.view(nb, 1)).view(nb, L, 1, 1).float()
        rel = {}
        for key, d in (("k", kd), ("v", vd)):
            err = (d - src[key]) * mask
            rel[key] = float(err.square().sum().sqrt() / (src[key] * mask).square().sum().sqrt())
        # fp32 attention over the unquantized tokens, every sequence at its own length
        q = stack.q[l][:nb].float().view(nb, H, G, 128)
        worst, num, den = 0.0, 0.0, 0.0
        for b in range(nb):
            lb = int(stack.attend[b])
            kk = src["k"][b, :lb].permute(1, 2, 0).contiguous()      # [H][128][lb]
            vv = src["v"][b, :lb].permute(1, 0, 2).contiguous()      # [H][lb][128]
            s_ = torch.matmul(q[b], kk) * (1.0 / math.sqrt(128.0))   # [H][G][lb]
            ref = torch.matmul(torch.softmax(s_, dim=-1), vv).view(Hq, 128)
            got = stack.out[l][b]
            worst = max(worst, float((got - ref).abs().max()))
            num += float((got - ref).square().sum())
            den += float(ref.square().sum())
        rep[name] = {"layer": l, "k_rel_rms": rel["k"], "v_rel_rms": rel["v"],
                     "attn_max_abs_vs_fp32": worst, "attn_rel_rms_vs_fp32": math.sqrt(num / den)}
    return {"sequences": nb, "reference": "fp32 attention over the unquantized source tokens", "layers": rep}


def host_info():
    """nproc and the CPU model string of the host the oracle runs on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


class OneCore:
    """While the oracle is timed, the calling thread runs on one core only (the lowest-numbered
    core it may use); the previous affinity is restored afterwards."""

    def __enter__(self):
        self.saved = os.sched_getaffinity(0)
        self.core = min(self.saved)
        os.sched_setaffinity(0, {self.core})
        return self

    def __exit__(self, *exc):
        os.sched_setaffinity(0, self.saved)


def _bits16(t):
    import numpy as np
    import torch
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def oracle_decode_seq(cfg, l, b, C, append=True):
    """Seconds the oracle takes for sequence b of layer l at C cached tokens: the append of the
    new token (when `append`) and binary64 attention over C (+1) tokens; packing the sequence
    beforehand is not timed."""
    import numpy as np
    import oracle as orc
    import synth
    seed, H, Hq = cfg["seed"], cfg["n_kv_heads"], cfg["n_q_heads"]
    kb, vb, km, _ = layer_spec(cfg["pairs"][l], cfg.get("k_mode", 0))
    scales = np.array([FP8_SCALES] * H, dtype=np.float32) if km == 2 else None
    cm = synth.outlier_mult(seed, l, H, cfg["n_outliers"])
    f32 = cfg.get("f32", False)
    dt = "f32" if f32 else "bf16"
    conv = (lambda t: t.contiguous().numpy()) if f32 else _bits16
    maxp = (C + 1 + 31) // 32
    bt = np.arange(maxp, dtype=np.int32).reshape(1, maxp)
    k = synth.fill(seed, synth.KIND_K, l, 1, C, H, b0=b, chan_mult=cm, dtype=dt)
    v = synth.fill(seed, synth.KIND_V, l, 1, C, H, b0=b, dtype=dt)
    q = synth.fill(seed, synth.KIND_Q, l, 1, 1, Hq, b0=b, dtype=dt).view(1, Hq, 128)
    pages, rk, rv = orc.new_cache(kb, vb, H, 1, maxp, km)
    orc.pack(kb, vb, conv(k), conv(v), [C], bt, pages, rk, rv, kmode=km, scales=scales)
    if append:
        kn = synth.fill(seed, synth.KIND_K_NEW, l, 1, 1, H, b0=b, chan_mult=cm).view(1, H, 128)
        vn = synth.fill(seed, synth.KIND_V_NEW, l, 1, 1, H, b0=b).view(1, H, 128)
    t0 = time.perf_counter()
    if append:
        orc.append(kb, vb, _bits16(kn), _bits16(vn), [C], bt, pages, rk, rv, kmode=km, scales=scales)
    orc.decode_attn(kb, vb, H, conv(q), [C + (1 if append else 0)], bt, pages, rk, rv, kmode=km, scales=scales)
    return time.perf_counter() - t0


def cpu_baseline_decode(cfg, lens, seqs, layers=None, append=True):
    """The CPU oracle as it stands, on one core: append + attention of sequences `seqs` for
    `layers` (default: every layer).  Returns {layer: [seconds per sequence]}."""
    layers = range(len(cfg["pairs"])) if layers is None else layers
    out = {}
    with OneCore():
        for l in layers:
            out[l] = [oracle_decode_seq(cfg, l, b, int(lens[b]), append) for b in seqs]
    return out


def cpu_record(value, unit, sample, extrapolated=False):
    return dict({"value": value, "unit": unit, "cores": 1, "kind": "oracle", "sample": sample,
                 "extrapolated": extrapolated}, **host_info())


def cpu_baseline_for(name, cfg, stack):
    """The oracle's rate on a bounded sample of workload `name` (about 10-30 s of one core)."""
    import numpy as np
    lens = stack.lens
    n_layers = len(cfg["pairs"])
    if name == "single":
        t = cpu_baseline_decode(cfg, lens, [0], append=False)
        secs = sum(v[0] for v in t.values())
        return cpu_record(1.0 / secs, "tokens/s", "the whole workload: binary64 attention of the one query over "
                          "its 512 tokens (packing not timed)")
    if name in ("llama", "ktoken", "bf16fp8"):
        # two sequences: about 10 s of timed oracle work (the untimed packing of the sample
        # takes four times that)
        seqs = list(range(min(2, stack.B)))
        t = cpu_baseline_decode(cfg, lens, seqs)
        secs = sum(sum(v) for v in t.values())
        return cpu_record(len(seqs) / secs, "tokens/s",
                          f"{len(seqs)} of {stack.B} sequences, all {n_layers} layers: append + binary64 attention "
                          "(packing of the sample not timed)")
    if name == "qwen":
        t = cpu_baseline_decode(cfg, lens, [0])
        secs = sum(v[0] for v in t.values())
        return cpu_record(1.0 / secs, "tokens/s",
                          f"1 of {stack.B} sequences, all {n_layers} layers: append + binary64 attention "
                          "(packing of the sample not timed)")
    if name == "ragged":
        # the shortest and the longest sequence, one whose append flushes a page, one more; one
        # layer of each distinct pair; seconds per attended token of each pair, extrapolated to
        # every sequence and layer by attended tokens
        flush = int(np.nonzero(lens % 32 == 31)[0][0]) if np.any(lens % 32 == 31) else 1
        seqs = [int(np.argmin(lens)), int(np.argmax(lens)), flush, 100 % stack.B]
        first = {}
        for l, e in enumerate(cfg["pairs"]):
            first.setdefault(tuple(e) if not isinstance(e, str) else e, l)
        t = cpu_baseline_decode(cfg, lens, seqs, layers=sorted(first.values()))
        attended = sum(int(lens[b]) + 1 for b in seqs)
        per_tok = {l: sum(v) / attended for l, v in t.items()}
        total_tok = int((lens + 1).sum())
        est = sum(per_tok[first[tuple(e) if not isinstance(e, str) else e]] * total_tok for e in cfg["pairs"])
        return cpu_record(stack.B / est, "tokens/s",
                          f"sequences {seqs} (shortest, longest, one that flushes, one more) at layers "
                          f"{sorted(first.values())} (one per distinct pair); step time extrapolated to all "
                          f"{stack.B} sequences and {n_layers} layers by attended tokens ({est:.1f} s per step)",
                          extrapolated=True)
    return None


def decode_workload(name, args, dev, flush_step=False):
    """Time one decode workload as the headline does: the fused append + attention step over
    every layer, captured as a graph.  Returns the record (not printed)."""
    import torch
    import layer_wise_mixed_kvq_amd as kvq
    cfg = CONFIGS[name]
    log(f"[bench] building {name} cache ...")
    t0 = time.perf_counter()
    stack = DecodeStack(cfg, dev)
    torch.cuda.synchronize()
    build_s = time.perf_counter() - t0
    log(f"[bench] cache built in {build_s:.1f} s")
    with_append = cfg.get("append", True)
    step_fn = (lambda: stack.step(with_append, fused=not args.unfused))
    if args.no_graph:
        for _ in range(args.warmup):
            step_fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(args.steps):
            step_fn()
        e1.record()
        torch.cuda.synchronize()
        ms, wall = e0.elapsed_time(e1) / args.steps, time.perf_counter() - t0
        step_stats = None
    else:
        g = capture(step_fn)
        log("[bench] graph captured; timing")
        ms, wall = time_graph(g, args.steps, args.warmup)
        step_stats = replay_stats(g, 20)
        del g
    # attention-only step, and the step with the append as its own launch (context)
    g_attn = capture(lambda: stack.step(False))
    ms_attn, _ = time_graph(g_attn, args.steps, 2)
    del g_attn
    ms_unfused = None
    if with_append and not args.unfused:
        g_unf = capture(lambda: stack.step(True, fused=False))
        ms_unfused, _ = time_graph(g_unf, args.steps, 2)
        del g_unf
    log(f"[bench] {name}: step {ms:.4f} ms (attention only {ms_attn:.4f} ms, append as its own launch "
        f"{ms_unfused} ms)")
    # the dominant kernel (decode attention): its average launch duration is the
    # attention-only step (one launch per layer, replayed as a graph on the stream the kernels
    # run on, timed with events over the whole timed region) divided by the layer count;
    # event pairs around single eager launches are reported beside it (they add a few us of
    # marker overhead per launch)
    n_layers = len(cfg["pairs"])
    dbytes = stack.decode_bytes()
    launch_us = ms_attn * 1e3 / n_layers
    achieved = sum(dbytes) / (ms_attn * 1e-3) / 1e9
    durs = per_launch_durations(stack.decode_layer, n_layers, args.roofline_reps)
    log(f"[bench] {name}: decode kernel avg {launch_us:.2f} us/launch (graph), "
        f"{sum(durs) / n_layers * 1e3:.2f} us (eager, event pairs); {achieved:.1f} GB/s")
    step_bytes = stack.alg_bytes(with_append)
    quality = quality_report(stack) if (with_append and args.quality) else None
    if quality:
        for qn, r in quality["layers"].items():
            log(f"[bench] {qn} (layer {r['layer']}): K rel RMS {r['k_rel_rms']:.4f}, V {r['v_rel_rms']:.4f}; "
                f"attention vs fp32 max abs {r['attn_max_abs_vs_fp32']:.2e}, rel RMS {r['attn_rel_rms_vs_fp32']:.4f}")
    flush = None
    if flush_step and with_append:
        flush = flush_step_timing(cfg, args, dev, ms, stack)
    lens = stack.lens
    B = stack.B
    rec = {
        "metric": "mixed-precision KV decode-attn tokens/s + packed-KV GB/s (% HBM peak), 1 GPU",
        "value": B * 1000.0 / ms,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle_s": SETTLE_S if not args.no_graph else None,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": stack_dtype(stack),
        "data": "synthetic (seeded Irwin-Hall N(0,1) K/V/q, outlier key channels x10 per layer and head)",
        "config": {"workload": cfg["workload"], "batch": B, "context": stack.C,
                   "attended_tokens": stack.L, "mean_attended_tokens": float(stack.attend.mean()), "layers": n_layers,
                   "n_q_heads": stack.Hq, "n_kv_heads": stack.H, "head_dim": 128,
                   "equiv_bits": kvq.kvq_equiv_bits(stack.model), "graph": not args.no_graph,
                   "fused_append": with_append and not args.unfused,
                   "keys": "per-token" if stack.k_mode else "per-channel"},
        "packed_kv_gbps": step_bytes / (ms * 1e-3) / 1e9,
        "packed_kv_frac_of_peak": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "step_alg_bytes": step_bytes,
        "attention_only_ms_per_step": ms_attn,
        "unfused_append_ms_per_step": ms_unfused,
        "wall_s_timed": wall,
        "step_ms_median_min": step_stats,
        "cache_build_s": build_s,
        "flush_step": flush,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": measured_traffic(name),
                     "kernel": "decode_kernel (kvq_decode_attn)",
                     "avg_launch_us": launch_us,
                     "avg_launch_us_eager_events": sum(durs) / n_layers * 1e3,
                     "alg_bytes_per_launch": sum(dbytes) / n_layers},
        "cpu_baseline": None,
        "quantization_error": quality,
    }
    del stack
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if args.cpu_baseline:
        log(f"[bench] {name}: CPU oracle baseline ...")
        t0 = time.perf_counter()
        rec["cpu_baseline"] = cpu_baseline_for(name, cfg, _LensOnly(lens, B))
        log(f"[bench] {name}: CPU oracle {rec['cpu_baseline']['value']:.4g} {rec['cpu_baseline']['unit']} "
            f"({time.perf_counter() - t0:.1f} s)")
    return rec


class _LensOnly:
    """The sequence lengths and batch of a workload (what the oracle sample needs)."""

    def __init__(self, lens, B):
        self.lens, self.B = lens, B


def flush_step_timing(cfg, args, dev, ms_steady, stack_steady):
    """A decode step in which every sequence's appended token completes a page (one token
    short of a page boundary): the fused launch quantizes that page and attends over it.  One
    step in 32 is such a step, so the amortized rate is batch * 32 / (31 * steady + flush)."""
    import torch
    C = int(stack_steady.lens.max())
    ctx = (C // 32) * 32 - 1
    fstack = DecodeStack(dict(cfg, context=ctx), dev)
    g = capture(lambda: fstack.step(True))
    ms_flush, _ = time_graph(g, args.steps, args.warmup)
    del g
    g_attn = capture(lambda: fstack.step(False))
    ms_flush_attn, _ = time_graph(g_attn, args.steps, 2)
    del g_attn
    B, n_layers = fstack.B, len(cfg["pairs"])
    del fstack
    torch.cuda.empty_cache()
    amort = B * 32 * 1000.0 / (31 * ms_steady + ms_flush)
    log(f"[bench] flush step ({ctx} cached tokens, every append completes a page): {ms_flush:.4f} ms "
        f"(attention only {ms_flush_attn:.4f} ms); 32-step amortized {amort:.0f} tokens/s")
    return {"context": ctx, "ms_per_step": ms_flush, "attention_only_ms_per_step": ms_flush_attn,
            "flush_cost_us_per_launch": (ms_flush - ms_flush_attn) * 1e3 / n_layers,
            "tokens_per_s_flush_step": B * 1000.0 / ms_flush,
            "tokens_per_s_32_step_amortized": amort}


def pack_workload(args, dev):
    return bench_pack(CONFIGS["pack"], args, emit=False)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="llama", choices=sorted(CONFIGS))
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false",
                    help="skip the oracle's CPU baseline legs")
    ap.add_argument("--no-quality", dest="quality", action="store_false",
                    help="skip the quantization-error report")
    ap.add_argument("--headline-only", action="store_true",
                    help="with the default workload: skip the nested records of the other workloads")
    ap.add_argument("--roofline-reps", type=int, default=5)
    ap.add_argument("--unfused", action="store_true", help="append as its own launch before each attention launch")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU: --gpus {args.gpus} (WORLD_SIZE {world}) is not supported; "
              "this decode path has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch
    import layer_wise_mixed_kvq_amd as kvq
    kvq.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = CONFIGS[args.config]
    if args.config == "pack":
        return bench_pack(cfg, args)
    if args.config == "copy":
        return bench_copy(args)
    if args.config == "sweep":
        return bench_sweep(args)
    if args.config == "formats":
        return bench_formats(args)

    headline = args.config == "llama"
    rec = decode_workload(args.config, args, dev, flush_step=headline)
    if headline and not args.headline_only:
        # the other four workloads, each timed and roofline-measured like the headline, with
        # its own CPU baseline leg: nested records of the same JSON line
        others = {}
        for name in ("single", "qwen", "ragged"):
            sub = argparse.Namespace(**vars(args))
            sub.steps, sub.warmup = min(args.steps, 20), min(args.warmup, 3)
            sub.quality = False
            others[name] = decode_workload(name, sub, dev)
        sub = argparse.Namespace(**vars(args))
        sub.steps, sub.warmup = min(args.steps, 20), min(args.warmup, 3)
        others["pack"] = pack_workload(sub, dev)
        rec["workloads"] = others
    print(json.dumps(rec), flush=True)


def stack_dtype(stack):
    kinds = sorted({("fp8 e4m3" if s[2] == 2 else "bf16" if s[2] == 3 else "int2/4/8 codes") for s in stack.specs})
    return "bf16-in/fp32-acc, " + " + ".join(kinds)


FORMAT_TABLES = {"BF16": ["bf16"] * 32, "FP8": ["fp8"] * 32, "BF16/FP8 mix": BF16_FP8_MIX, "C3.25": LLAMA_C325}


def bench_formats(args):
    """The machinoai page's comparison at kernel level: all-BF16, calibrated all-FP8 and the
    8 BF16 + 24 FP8 mix (plus the C3.25 integer table) on one shape: decode step tokens/s,
    KV bytes per step and the decode kernel's GB/s."""
    import torch
    dev = torch.device("cuda:0")
    res = {}
    for name, pairs in FORMAT_TABLES.items():
        cfg = dict(CONFIGS["bf16fp8"], pairs=pairs)
        stack = DecodeStack(cfg, dev)
        g = capture(lambda: stack.step(True))
        ms, _ = time_graph(g, args.steps, args.warmup)
        g_attn = capture(lambda: stack.step(False))
        ms_attn, _ = time_graph(g_attn, args.steps, 2)
        kv = sum(stack.decode_bytes())
        res[name] = {"tokens_per_s": stack.B * 1000.0 / ms, "ms_per_step": ms, "decode_bytes_per_step": kv,
                     "decode_gbps": kv / (ms_attn * 1e-3) / 1e9, "equiv_bits": stack.kvq.kvq_equiv_bits(stack.model)}
        log(f"[bench] formats {name}: {ms:.4f} ms/step, {res[name]['tokens_per_s']:.0f} tok/s, "
            f"decode {res[name]['decode_gbps']:.0f} GB/s, {kv / 2**20:.0f} MiB/step")
        del g, g_attn, stack
        torch.cuda.empty_cache()
    base = res["BF16"]["tokens_per_s"]
    for r in res.values():
        r["relative_to_BF16"] = r["tokens_per_s"] / base
    mix = res["BF16/FP8 mix"]
    rec = {"metric": "decode step tokens/s of the 8 BF16 + 24 FP8 layer mix (llama3.1-8b shape, B=16, 4096 cached "
                     "tokens), 1 GPU",
           "value": mix["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": mix["ms_per_step"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16-in/fp32-acc, fp8 e4m3 + bf16 pages", "data": "synthetic",
           "config": {"workload": CONFIGS["formats"]["workload"], "tables": list(FORMAT_TABLES)},
           "formats": res, "roofline": None, "cpu_baseline": None}
    print(json.dumps(rec), flush=True)


def bench_pack(cfg, args, emit=True):
    """Prefill pack of 32768 bf16 tokens per layer for all 32 layers; source GB/s."""
    import torch
    import synth
    import layer_wise_mixed_kvq_amd as kvq
    dev = torch.device("cuda:0")
    B, H, T = cfg["batch"], cfg["n_kv_heads"], cfg["context"]
    model = kvq.Model(cfg["pairs"], cfg["n_q_heads"], H)
    maxp = T // 32
    bt = torch.arange(B * maxp, dtype=torch.int32, device=dev).view(B, maxp)
    seq = torch.full((B,), T, dtype=torch.int32, device=dev)
    caches, ks, vs = [], [], []
    log("[bench] generating 32 layers of bf16 sources ...")
    for l in range(len(cfg["pairs"])):
        caches.append(kvq.LayerCache(model, l, B, maxp, block_table=bt, device=dev))
        cm = synth.outlier_mult(cfg["seed"], l, H, cfg["n_outliers"])
        ks.append(synth.fill(cfg["seed"], synth.KIND_K, l, B, T, H, chan_mult=cm, device=dev))
        vs.append(synth.fill(cfg["seed"], synth.KIND_V, l, B, T, H, device=dev))
    torch.cuda.synchronize()

    def step():
        for l in range(len(caches)):
            kvq.kvq_pack(model, l, caches[l], ks[l], vs[l], seq)

    g = capture(step)
    ms, wall = time_graph(g, args.steps, args.warmup)
    src_bytes = 2 * B * T * H * 128 * 2 * len(caches)
    page_bytes = sum(B * maxp * H * 512 * (kb + vb + 2) for kb, vb in cfg["pairs"])
    # average launch duration: the graph of one pack launch per layer, timed over the whole
    # timed region, divided by the layer count
    launch_us = ms * 1e3 / len(caches)
    achieved = (src_bytes + page_bytes) / (ms * 1e-3) / 1e9
    rec = {
        "metric": "mixed-precision KV prefill pack source GB/s (% HBM peak), 1 GPU",
        "value": src_bytes / (ms * 1e-3) / 1e9, "unit": "GB/s (bf16 source)", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "clock_settle_s": SETTLE_S, "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16-in, int2/4/8 codes", "data": "synthetic",
        "config": {"workload": cfg["workload"], "tokens": T, "layers": len(caches)},
        "total_gbps": (src_bytes + page_bytes) / (ms * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": measured_traffic("pack", "pack_kernel", PACK_SOURCES),
                     "kernel": "pack_kernel (kvq_pack)",
                     "avg_launch_us": launch_us, "alg_bytes_per_launch": (src_bytes + page_bytes) / len(caches)},
        "cpu_baseline": None,
    }
    del g, ks, vs, caches
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log(f"[bench] pack: {ms:.4f} ms per 32-layer step, {rec['value']:.0f} GB/s of bf16 source, "
        f"{launch_us:.2f} us per launch, frac {achieved / HBM_PEAK_GBPS:.3f}")
    if getattr(args, "cpu_baseline", True):
        rec["cpu_baseline"] = cpu_baseline_pack(cfg)
        log(f"[bench] pack: CPU oracle {rec['cpu_baseline']['value']:.4g} GB/s of source")
    if emit:
        print(json.dumps(rec), flush=True)
    return rec


def cpu_baseline_pack(cfg, pages_per_layer=64):
    """The oracle's quantize-on-write of the first `pages_per_layer` 32-token pages of every
    layer (one core), extrapolated by pages to the whole prefill; bf16 source GB/s."""
    import numpy as np
    import oracle as orc
    import synth
    H, T = cfg["n_kv_heads"], cfg["context"]
    n = pages_per_layer * 32
    secs = 0.0
    with OneCore():
        for l, (kb, vb) in enumerate(cfg["pairs"]):
            cm = synth.outlier_mult(cfg["seed"], l, H, cfg["n_outliers"])
            k = _bits16(synth.fill(cfg["seed"], synth.KIND_K, l, 1, n, H, chan_mult=cm))
            v = _bits16(synth.fill(cfg["seed"], synth.KIND_V, l, 1, n, H))
            bt = np.arange(pages_per_layer, dtype=np.int32).reshape(1, pages_per_layer)
            pages, rk, rv = orc.new_cache(kb, vb, H, 1, pages_per_layer)
            t0 = time.perf_counter()
            orc.pack(kb, vb, k, v, [n], bt, pages, rk, rv)
            secs += time.perf_counter() - t0
    est = secs * (T / n)
    src_bytes = 2 * T * H * 128 * 2 * len(cfg["pairs"])
    return cpu_record(src_bytes / est / 1e9, "GB/s (bf16 source)",
                      f"the first {pages_per_layer} of {T // 32} pages of every layer; step time extrapolated by "
                      f"pages ({est:.1f} s per 32-layer prefill)", extrapolated=True)


def bench_sweep(args):
    """Decode step (append + attention, 32 layers, Llama-3.1-8B heads) for each table of
    SWEEP_TABLES at each (batch, cached tokens) of SWEEP_SHAPES; tokens/s and the ratio to
    the uniform 8-bit table, the shape of the pages' throughput comparison at kernel level."""
    import torch
    dev = torch.device("cuda:0")
    rows = []
    for batch, ctx in SWEEP_SHAPES:
        row = {"batch": batch, "input_len": ctx, "tokens_per_s": {}, "ms_per_step": {}, "decode_gbps": {}}
        for name, pairs in SWEEP_TABLES.items():
            cfg = dict(CONFIGS["llama"], pairs=pairs, batch=batch, context=ctx)
            stack = DecodeStack(cfg, dev)
            g = capture(lambda: stack.step(True))
            ms, _ = time_graph(g, args.steps, args.warmup)
            g_attn = capture(lambda: stack.step(False))
            ms_attn, _ = time_graph(g_attn, args.steps, 2)
            row["tokens_per_s"][name] = batch * 1000.0 / ms
            row["ms_per_step"][name] = ms
            row["decode_gbps"][name] = sum(stack.decode_bytes()) / (ms_attn * 1e-3) / 1e9
            log(f"[bench] sweep B={batch} L={ctx} {name}: {ms:.4f} ms/step, {row['tokens_per_s'][name]:.0f} tok/s, "
                f"decode {row['decode_gbps'][name]:.0f} GB/s")
            del g, g_attn, stack
            torch.cuda.empty_cache()
        base = row["tokens_per_s"]["KV8"]
        row["relative_to_KV8"] = {k: v / base for k, v in row["tokens_per_s"].items()}
        rows.append(row)
    head = rows[-1]
    rec = {"metric": "decode step tokens/s of the C3.25 table relative to uniform KV8 (llama3.1-8b shape, B=16, "
                     "4096 cached tokens), 1 GPU",
           "value": head["relative_to_KV8"]["C3.25"], "unit": "x (ratio)", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": head["ms_per_step"]["C3.25"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16-in/fp32-acc, int2/4/8 codes", "data": "synthetic",
           "config": {"workload": CONFIGS["sweep"]["workload"], "tables": list(SWEEP_TABLES),
                      "shapes": SWEEP_SHAPES},
           "sweep": rows, "roofline": None, "cpu_baseline": None}
    print(json.dumps(rec), flush=True)


def bench_copy(args):
    """A plain streaming kernel of known size (torch's elementwise bitwise_not over 1 GiB of
    int32 into another 1 GiB): the bandwidth a simple kernel reaches on this GPU, and the
    reference against which the HBM byte counters are scaled."""
    import torch
    dev = torch.device("cuda:0")
    n = COPY_BYTES // 4
    src = torch.arange(n, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        torch.bitwise_not(src, out=dst)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    assert int(dst[12345].item()) == ~12345
    gbps = 2 * COPY_BYTES / (ms * 1e-3) / 1e9
    rec = {"metric": "streaming copy GB/s (read + write), 1 GPU", "value": gbps, "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "int32", "data": "synthetic",
           "config": {"workload": CONFIGS["copy"]["workload"], "bytes_read": COPY_BYTES,
                      "bytes_written": COPY_BYTES},
           "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": gbps / HBM_PEAK_GBPS, "traffic": None, "kernel": "torch bitwise_not"},
           "cpu_baseline": None}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
