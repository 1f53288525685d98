"""Shared builders for the GPU parity tests: the same seeded synthetic inputs go to the
oracle (host numpy) and to the HIP library (device tensors)."""
from __future__ import annotations

import math

import numpy as np

import synth

ATOL = 2e-4          # max abs error of attention outputs vs the binary64 oracle
LSE_RTOL = 1e-4      # |d lse| <= 1e-4 * max(1, |lse|)

LLAMA_C325 = [(4, 8)] * 3 + [(4, 2)] * 24 + [(2, 2)] * 4 + [(4, 8)]
QWEN_C40 = [(8, 4)] * 4 + [(4, 4)] * 4 + [(4, 2)] * 16 + [(8, 4)] * 4


def bits_of(t):
    """torch bf16 tensor -> numpy uint16 bit patterns (host)."""
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host_array(t):
    """torch tensor -> numpy array in the oracle's convention (bf16 as uint16 bits)."""
    import torch
    if t.dtype == torch.bfloat16:
        return bits_of(t)
    return t.detach().cpu().contiguous().numpy()


class Case:
    """One layer's seeded inputs plus its oracle cache and its device cache."""

    def __init__(self, kb, vb, H, G, lens, *, seed=1, layer=0, src="bf16", q_dtype="bf16", shuffle=True,
                 extra_pages=3, n_outliers=3, spare_pages_per_seq=0, kmode=0, scales=None):
        import torch
        self.kb, self.vb, self.H, self.G = kb, vb, H, G
        # the oracle's layer format: 0 / 1 integer codes with per-channel / per-token keys,
        # 2 FP8 E4M3 (kb = vb = 8, scales [H][2] or None for 1.0), 3 BF16 (kb = vb = 16)
        self.kmode = kmode
        self.scales = None if scales is None else np.ascontiguousarray(scales, dtype=np.float32).reshape(H, 2)
        self.lens = np.array(lens, dtype=np.int32)
        self.B = len(lens)
        self.T = max(1, int(self.lens.max()))
        self.maxp = (self.T + 31) // 32 + spare_pages_per_seq
        self.n_phys = self.B * self.maxp + extra_pages
        self.seed, self.layer = seed, layer
        cm = synth.outlier_mult(seed, layer, H, n_outliers) if n_outliers else None
        self.k = synth.fill(seed, synth.KIND_K, layer, self.B, self.T, H, chan_mult=cm, dtype=src)
        self.v = synth.fill(seed, synth.KIND_V, layer, self.B, self.T, H, dtype=src)
        self.q = synth.fill(seed, synth.KIND_Q, layer, self.B, 1, H * G, dtype=q_dtype).view(self.B, H * G, 128)
        perm = synth.permutation(seed + 17, self.n_phys) if shuffle else np.arange(self.n_phys, dtype=np.int32)
        self.bt = np.ascontiguousarray(perm[: self.B * self.maxp].reshape(self.B, self.maxp))
        self.dev = torch.device("cuda") if torch.cuda.is_available() else None

    # ---- oracle side -------------------------------------------------------------
    def oracle_pack(self, orc):
        self.o_pages, self.o_rk, self.o_rv = orc.new_cache(self.kb, self.vb, self.H, self.B, self.n_phys,
                                                           self.kmode)
        orc.pack(self.kb, self.vb, host_array(self.k), host_array(self.v), self.lens, self.bt,
                 self.o_pages, self.o_rk, self.o_rv, kmode=self.kmode, scales=self.scales)

    def oracle_decode(self, orc, lens=None):
        lens = self.lens if lens is None else np.asarray(lens, dtype=np.int32)
        return orc.decode_attn(self.kb, self.vb, self.H, host_array(self.q), lens, self.bt, self.o_pages,
                               self.o_rk, self.o_rv, kmode=self.kmode, scales=self.scales)

    def layer_entry(self):
        """This layer's entry in a device Model table."""
        return {2: "fp8", 3: "bf16"}.get(self.kmode, (self.kb, self.vb, self.kmode))

    # ---- device side -------------------------------------------------------------
    def device_setup(self, kvq):
        import torch
        self.model = kvq.Model([self.layer_entry()], self.H * self.G, self.H)
        self.bt_d = torch.from_numpy(self.bt).to(self.dev)
        self.scales_d = None if self.scales is None else torch.from_numpy(self.scales).to(self.dev)
        self.cache = kvq.LayerCache(self.model, 0, self.B, self.maxp, n_pages=self.n_phys,
                                    block_table=self.bt_d, device=self.dev, fp8_scales=self.scales_d)
        self.lens_d = torch.from_numpy(self.lens).to(self.dev)

    def device_pack(self, kvq):
        kvq.kvq_pack(self.model, 0, self.cache, self.k.to(self.dev), self.v.to(self.dev), self.lens_d)

    def device_decode(self, kvq, lens=None, pages_per_split=0, max_seq_len=None):
        import torch
        lens_d = self.lens_d if lens is None else torch.as_tensor(np.asarray(lens, np.int32)).to(self.dev)
        msl = int(self.maxp * 32) if max_seq_len is None else max_seq_len
        out, lse = kvq.kvq_decode_attn(self.model, 0, self.cache, self.q.to(self.dev), lens_d, msl,
                                       pages_per_split=pages_per_split)
        torch.cuda.synchronize()
        return out.cpu().numpy(), lse.cpu().numpy()


def assert_attention_close(out, lse, o_ref, l_ref, what=""):
    err = np.abs(out.astype(np.float64) - o_ref)
    assert np.all(np.isfinite(out)), f"{what}: non-finite outputs"
    assert err.max() <= ATOL, f"{what}: max abs err {err.max():.3e} > {ATOL}"
    lerr = np.abs(lse.astype(np.float64) - l_ref) / np.maximum(1.0, np.abs(l_ref))
    assert lerr.max() <= LSE_RTOL, f"{what}: lse rel err {lerr.max():.3e} > {LSE_RTOL}"
    return float(err.max()), float(lerr.max())


def live_resid_equal(a, b, lens):
    """Compare residual slots 0 .. L mod 32 - 1 of every sequence."""
    for i, L in enumerate(lens):
        n = int(L) % 32
        if not np.array_equal(a[i, :, :n], b[i, :, :n]):
            return False
    return True


def ceil_div(a, b):
    return -(-a // b)


def log(msg):
    print(msg, flush=True)


__all__ = ["Case", "assert_attention_close", "live_resid_equal", "bits_of", "host_array", "ATOL",
           "LSE_RTOL", "LLAMA_C325", "QWEN_C40", "ceil_div", "log", "math"]
