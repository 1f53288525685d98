"""Pins of the oracle's per-token key mode (keys quantized per token over 32-channel groups,
the other key mode the pages compare; the per-channel mode is pinned in test_oracle_pins).

  * symmetry: per-token key groups follow exactly the value rule, so a tile packed as
    per-token keys dequantizes to what the same tile gives as values;
  * layout: found by packing one-hot tiles (not by restating the slot formula): every
    channel has its own slot, each 4*kb-byte chunk a of a row holds channels
    32J + 8a .. 32J + 8a + 7 of every group J, and channels 32J + 8a + 2i, + 1 sit 16 bits
    apart inside one 32-bit word;
  * tokens on a per-(token, group) grid dequantize exactly;
  * attention equals a textbook evaluation over the dequantized keys;
  * prefill of L tokens == prefill of a prefix + single-token appends.
"""
import math

import numpy as np
import pytest


PAIRS = [(k, v) for k in (2, 4, 8) for v in (2, 4, 8)]


def _bf16_bits(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _bf16_val(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("kb,vb", PAIRS)
def test_per_token_keys_follow_the_value_rule(orc, kb, vb):
    rng = np.random.default_rng(kb * 31 + vb)
    x = rng.standard_normal((32, 128)).astype(np.float32)
    x[:, 5] *= 10
    other = rng.standard_normal((32, 128)).astype(np.float32)
    kd, _ = orc.dequant_page(orc.pack_page(x, other, kb, vb, orc.KMODE_TOKEN), kb, vb, orc.KMODE_TOKEN)
    _, vd = orc.dequant_page(orc.pack_page(other, x, vb, kb, orc.KMODE_CHANNEL), vb, kb, orc.KMODE_CHANNEL)
    assert np.array_equal(kd, vd)
    # and it differs from the per-channel key mode on the same data
    kc, _ = orc.dequant_page(orc.pack_page(x, other, kb, vb, orc.KMODE_CHANNEL), kb, vb, orc.KMODE_CHANNEL)
    assert not np.array_equal(kd, kc)


@pytest.mark.parametrize("kb", [2, 4, 8])
def test_per_token_key_row_layout(orc, kb):
    """Token 0's row, one channel at a time: the only nonzero code marks the channel's slot."""
    vb = 2
    v = np.zeros((32, 128), np.float32)
    where = {}
    for c in range(128):
        k = np.zeros((32, 128), np.float32)
        k[0, c] = 1.0                      # group of c: min 0, max 1 -> code 2^kb - 1 at c, 0 elsewhere
        page = orc.pack_page(k, v, kb, vb, orc.KMODE_TOKEN)
        row = page[: 16 * kb]
        bits = np.unpackbits(row, bitorder="little")
        on = np.nonzero(bits)[0]
        assert len(on) == kb and on[-1] - on[0] == kb - 1 and on[0] % kb == 0, f"channel {c}: {on}"
        where[c] = int(on[0])              # bit offset in the row
    offs = sorted(where.values())
    assert offs == [kb * i for i in range(128)], "channels do not fill the row one slot each"
    chunk_bits = 32 * kb
    for c, off in where.items():
        J, rest = divmod(c, 32)
        a = rest // 8
        assert off // chunk_bits == a, f"channel {c} not in chunk {a}"
    for J in range(4):
        for a in range(4):
            for i in range(4):
                c0 = 32 * J + 8 * a + 2 * i
                o0, o1 = where[c0], where[c0 + 1]
                assert o0 // 32 == o1 // 32, f"channels {c0}, {c0 + 1} not in one 32-bit word"
                assert o1 - o0 == 16, f"channels {c0}, {c0 + 1} not 16 bits apart"
    # the slot order the format states (n = 16/kb, hh = (s/n)%2, k = (s/(2n))*n + s%n,
    # channel 32*(k/4) + 8*a + 2*(k%4) + hh), written out by hand for the first 16 slots
    # of chunk 0 and checked for every slot of every chunk
    by_slot = {off // kb: c for c, off in where.items()}
    first16 = {2: [0, 2, 4, 6, 32, 34, 36, 38, 1, 3, 5, 7, 33, 35, 37, 39],
               4: [0, 2, 4, 6, 1, 3, 5, 7, 32, 34, 36, 38, 33, 35, 37, 39],
               8: [0, 2, 1, 3, 4, 6, 5, 7, 32, 34, 33, 35, 36, 38, 37, 39]}[kb]
    assert [by_slot[s] for s in range(16)] == first16, f"kb={kb}: slot order of chunk 0"
    n = 16 // kb
    for a in range(4):
        for s in range(32):
            hh, k = (s // n) % 2, (s // (2 * n)) * n + s % n
            assert by_slot[32 * a + s] == 32 * (k // 4) + 8 * a + 2 * (k % 4) + hh, f"kb={kb} chunk {a} slot {s}"


@pytest.mark.parametrize("kb,vb", PAIRS)
def test_per_token_keys_on_grid_are_exact(orc, kb, vb):
    rng = np.random.default_rng(kb * 10 + vb + 7)
    s = np.exp2(rng.integers(-8, 0, (32, 4))).astype(np.float64)
    z = rng.integers(-64, 64, (32, 4)) / 16.0
    codes = rng.integers(0, 2**kb, (32, 128))
    codes[:, 0::32], codes[:, 1::32] = 0, 2**kb - 1
    k = (np.repeat(z, 32, axis=1) + codes * np.repeat(s, 32, axis=1)).astype(np.float32)
    v = rng.standard_normal((32, 128)).astype(np.float32)
    kd, _ = orc.dequant_page(orc.pack_page(k, v, kb, vb, orc.KMODE_TOKEN), kb, vb, orc.KMODE_TOKEN)
    assert np.array_equal(kd, k.astype(np.float64))


def _textbook(q, K, V):
    sc = (q @ K.T) / math.sqrt(128)
    m = sc.max()
    p = np.exp(sc - m)
    return (p @ V) / p.sum(), m + math.log(p.sum())


@pytest.mark.parametrize("kb,vb,G", [(4, 2, 4), (8, 8, 1), (2, 4, 7)])
def test_per_token_attention_brute_force(orc, kb, vb, G):
    rng = np.random.default_rng(kb + 5 * vb + G)
    B, H, L = 2, 2, [45, 70]
    T, maxp = 70, 3
    k = _bf16_bits(rng.standard_normal((B, T, H, 128)))
    v = _bf16_bits(rng.standard_normal((B, T, H, 128)))
    ids = np.arange(B * maxp + 2, dtype=np.int32)
    rng.shuffle(ids)
    bt = ids[: B * maxp].reshape(B, maxp).copy()
    pages, rk, rv = orc.new_cache(kb, vb, H, B, B * maxp + 2)
    orc.pack(kb, vb, k, v, L, bt, pages, rk, rv, kmode=orc.KMODE_TOKEN)
    q = _bf16_bits(rng.standard_normal((B, H * G, 128)))
    out, lse = orc.decode_attn(kb, vb, H, q, L, bt, pages, rk, rv, kmode=orc.KMODE_TOKEN)
    for b in range(B):
        for h in range(H):
            Kd = np.zeros((L[b], 128))
            Vd = np.zeros((L[b], 128))
            for g in range(L[b] // 32):
                Kd[32 * g:32 * g + 32], Vd[32 * g:32 * g + 32] = orc.dequant_page(pages[bt[b, g], h], kb, vb,
                                                                                  orc.KMODE_TOKEN)
            for t in range(32 * (L[b] // 32), L[b]):
                Kd[t], Vd[t] = _bf16_val(rk[b, h, t % 32]), _bf16_val(rv[b, h, t % 32])
            for gq in range(G):
                hq = h * G + gq
                o, l = _textbook(_bf16_val(q[b, hq]).astype(np.float64), Kd, Vd)
                assert np.allclose(out[b, hq], o, rtol=0, atol=1e-12)
                assert abs(lse[b, hq] - l) < 1e-12


@pytest.mark.parametrize("kb,vb", [(4, 2), (8, 4)])
def test_per_token_prefill_equals_prefix_plus_appends(orc, kb, vb):
    rng = np.random.default_rng(kb * 3 + vb)
    B, H, L, k0, maxp = 2, 2, 70, 25, 3
    k = _bf16_bits(rng.standard_normal((B, L, H, 128)))
    v = _bf16_bits(rng.standard_normal((B, L, H, 128)))
    bt = np.arange(B * maxp, dtype=np.int32).reshape(B, maxp)
    full = orc.new_cache(kb, vb, H, B, B * maxp)
    orc.pack(kb, vb, k, v, [L] * B, bt, *full, kmode=orc.KMODE_TOKEN)
    inc = orc.new_cache(kb, vb, H, B, B * maxp)
    orc.pack(kb, vb, np.ascontiguousarray(k[:, :k0]), np.ascontiguousarray(v[:, :k0]), [k0] * B, bt, *inc,
             kmode=orc.KMODE_TOKEN)
    for t in range(k0, L):
        orc.append(kb, vb, np.ascontiguousarray(k[:, t]), np.ascontiguousarray(v[:, t]), [t] * B, bt, *inc,
                   kmode=orc.KMODE_TOKEN)
    assert np.array_equal(full[0], inc[0])
    live = slice(0, L % 32)
    assert np.array_equal(full[1][:, :, live], inc[1][:, :, live])
    assert np.array_equal(full[2][:, :, live], inc[2][:, :, live])
