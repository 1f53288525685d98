"""The code quotient over every fp16 scale, through kvq_pack, bit-exact against the oracle.

The codec rule codes each element as clamp(rne(fl32(fl32(x - z) / s)), 0, 2^b - 1) with the
fp16-rounded scale s and zero z widened to binary32, the division being one correctly rounded
binary32 division (readings R2-R4; keys per channel or per token, values per token, with fp16
scale/zero pairs [Mixed-precision KV-cache quantization per-layer sensitivity
(llms-explorer.com), Facts]).  The GPU reaches that quotient without a division instruction, so
this test packs groups that realize every positive finite fp16 scale S the input domain
(|x| <= 65504) allows at each code width b = 2, 4, 8 -- subnormal scales included -- with
quotients at every half-integer k + 1/2 (k = 0 .. 2^b - 2) and at -2 .. +2 binary32 ulps
beside it, where any departure from the correctly rounded quotient changes a code.  Packed
pages are compared with the oracle byte for byte, for keys per channel and per token and for
values.

Group construction (binary32, all exact): minimum m (an fp16 value: 0, or minus the least fp16
value >= L*S - 65504 when L*S exceeds 65504, L = 2^b - 1), maximum m + L*S, so the stored
scale is exactly S and the stored zero exactly m; the other 30 elements are m + (k + 1/2)*S
moved by the ulp steps.
"""
from __future__ import annotations

import numpy as np
import pytest

from kvq_cases import log


@pytest.fixture(scope="module")
def kvq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import layer_wise_mixed_kvq_amd as k
    k.lib()
    return k


def scale_groups(bits: int) -> np.ndarray:
    """[n_groups][32] binary32 groups covering every in-domain fp16 scale (see the module
    docstring); element 0 is the minimum, element 1 the maximum."""
    L = (1 << bits) - 1
    S = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    LS = S * L
    S, LS = S[LS <= 2 * 65504.0], LS[LS <= 2 * 65504.0]
    need = np.maximum(LS - 65504.0, 0.0)
    m = need.astype(np.float16).astype(np.float64)                 # round to nearest fp16 ...
    up = m < need                                                  # ... then up to >= need
    m[up] = np.nextafter(m[up].astype(np.float16), np.float16(np.inf)).astype(np.float64)
    mn = -m
    mx = mn + LS
    assert np.all(mx.astype(np.float32).astype(np.float64) == mx) and np.all(np.abs(mx) <= 65504)
    # test values: (scale, k, ulp step)
    k = np.arange(L, dtype=np.float64) + 0.5
    steps = np.arange(-2, 3)
    base = mn[:, None] + k[None, :] * S[:, None]                  # [nS][L], exact in binary32
    b32 = base.astype(np.float32)
    assert np.all(b32.astype(np.float64) == base)
    vals = np.repeat(b32[:, :, None], len(steps), axis=2)          # [nS][L][5]
    for d in (1, 2):
        up1 = vals[:, :, 2 + d]
        dn1 = vals[:, :, 2 - d]
        for _ in range(d):
            up1 = np.nextafter(up1, np.float32(np.inf))
            dn1 = np.nextafter(dn1, np.float32(-np.inf))
        vals[:, :, 2 + d] = up1
        vals[:, :, 2 - d] = dn1
    per_s = vals.reshape(len(S), -1)                               # [nS][5L]
    n_per = -(-per_s.shape[1] // 30)
    pad = n_per * 30 - per_s.shape[1]
    if pad:
        per_s = np.concatenate([per_s, per_s[:, :pad]], axis=1)
    groups = np.empty((len(S), n_per, 32), dtype=np.float32)
    groups[:, :, 0] = mn[:, None].astype(np.float32)
    groups[:, :, 1] = mx[:, None].astype(np.float32)
    groups[:, :, 2:] = per_s.reshape(len(S), n_per, 30)
    return groups.reshape(-1, 32)


def test_scale_groups_construction(orc):
    """Host-side check of the construction on a sample: the oracle's group quantizer stores
    exactly S and m (so the GPU comparison below exercises the quotient at every scale)."""
    for bits in (2, 4, 8):
        g = scale_groups(bits)
        idx = np.linspace(0, len(g) - 1, 400).astype(np.int64)
        L = (1 << bits) - 1
        for i in idx:
            s16, z16, _ = orc.quant_group(g[i], bits)
            S = float(np.uint16(s16).view(np.float16))
            assert np.float64(g[i][1]) - np.float64(g[i][0]) == S * L
            assert float(np.uint16(z16).view(np.float16)) == float(g[i][0])


def _tiles(groups: np.ndarray, along_tokens: bool) -> np.ndarray:
    """Lay groups out in a [T][128] binary32 tile: along tokens (one channel of 32 tokens per
    group: per-channel keys) or along channels (32 channels of one token: values, per-token
    keys)."""
    n = len(groups)
    if along_tokens:
        n_pages = -(-n // 128)
        g = np.concatenate([groups, groups[: n_pages * 128 - n]]) if n_pages * 128 > n else groups
        return np.ascontiguousarray(g.reshape(n_pages, 128, 32).transpose(0, 2, 1).reshape(n_pages * 32, 128))
    T = -(-n // 4)
    T = -(-T // 32) * 32
    g = np.concatenate([groups, np.resize(groups, (T * 4 - n, 32))]) if T * 4 > n else groups
    return np.ascontiguousarray(g.reshape(T, 128))


@pytest.mark.gpu
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("kmode", [0, 1])
def test_every_fp16_scale_bit_exact(kvq, orc, bits, kmode):
    import torch
    groups = scale_groups(bits)
    kt = _tiles(groups, along_tokens=(kmode == 0))
    vt = _tiles(groups, along_tokens=False)
    T = max(len(kt), len(vt))
    k = np.zeros((1, T, 1, 128), dtype=np.float32)
    v = np.zeros((1, T, 1, 128), dtype=np.float32)
    k[0, :len(kt), 0] = kt
    v[0, :len(vt), 0] = vt
    if len(kt) < T:
        k[0, len(kt):, 0] = kt[: T - len(kt)]
    if len(vt) < T:
        v[0, len(vt):, 0] = vt[: T - len(vt)]
    log(f"every fp16 scale: bits={bits} kmode={kmode}: {len(groups)} groups, {T} tokens")
    n_pages = T // 32
    bt = np.arange(n_pages, dtype=np.int32).reshape(1, n_pages)
    pages, rk, rv = orc.new_cache(bits, bits, 1, 1, n_pages, kmode)
    orc.pack(bits, bits, k, v, [T], bt, pages, rk, rv, kmode=kmode)
    model = kvq.Model([(bits, bits, kmode)], 1, 1)
    dev = torch.device("cuda")
    cache = kvq.LayerCache(model, 0, 1, n_pages, n_pages=n_pages, block_table=torch.from_numpy(bt).to(dev),
                           device=dev)
    kvq.kvq_pack(model, 0, cache, torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev),
                 torch.tensor([T], dtype=torch.int32, device=dev))
    got = cache.pages.cpu().numpy().reshape(pages.shape)
    if not np.array_equal(got, pages):
        bad = np.argwhere(got != pages)
        raise AssertionError(f"{len(bad)} bytes differ, first at {bad[0].tolist()}")
