"""Pins of the CPU oracle to things other than itself.

Every test here runs on the CPU.  The oracle is checked against:
  * numbers the pages print (closed forms, tests/golden/pages_closed_forms.json),
  * library routines for the special cases that reduce to them (numpy's IEEE binary16
    conversion, torch's bfloat16 conversion, a numpy textbook softmax attention),
  * exactness on inputs that already lie on the quantization grid,
  * hand-derived codes, scales and packed bytes for tiny groups,
  * invariants (round-trip bound, nearest-grid-point codes, GQA head mapping, block-table
    indirection, prefill == prefix prefill + appends).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_closed_forms.json")
BITS = (2, 4, 8)
PAIRS = [(k, v) for k in BITS for v in BITS]


@pytest.fixture(scope="module")
def gold():
    with open(GOLDEN) as f:
        return json.load(f)


# ------------------------------------------------------------------------------------
# closed forms printed by the pages
# ------------------------------------------------------------------------------------

LLAMA_C325 = [(4, 8)] * 3 + [(4, 2)] * 24 + [(2, 2)] * 4 + [(4, 8)]       # 32 layers
QWEN_C40 = [(8, 4)] * 4 + [(4, 4)] * 4 + [(4, 2)] * 16 + [(8, 4)] * 4       # 28 layers


def test_equivalent_bits_tables(orc, gold):
    g = gold["equivalent_bits"]
    assert len(LLAMA_C325) == 32 and len(QWEN_C40) == 28
    assert [LLAMA_C325[i] for i in (0, 1, 2, 31)] == [(4, 8)] * 4
    assert orc.equiv_bits(LLAMA_C325) == Fraction(g["llama31_8b_c325"]).limit_denominator()
    assert orc.equiv_bits(QWEN_C40) == Fraction(g["qwen25_7b_c40"]).limit_denominator()
    names = {"K8V4": (8, 4), "K8V2": (8, 2), "K4V2": (4, 2), "KV8": (8, 8), "KV4": (4, 4)}
    for name, c in g["uniform"].items():
        assert orc.equiv_bits([names[name]] * 7) == c
    # a plausible slip (counting only key bits, or summing instead of averaging) fails:
    assert orc.equiv_bits([(8, 2)]) != 8 and orc.equiv_bits([(8, 2)]) != 10


def test_memory_reduction_convention(orc, gold):
    g = gold["memory_reduction_c344_vs_kivi4"]
    assert orc.relative_saving(g["base_bits"], g["new_bits"]) == pytest.approx(g["reduction"], abs=1e-12)


def test_idealized_bf16_fp8_mix(orc, gold):
    g = gold["idealized_bf16_fp8_mix"]
    L, mib = g["layers"], g["bf16_layer_mib"]
    all_bf16 = orc.idealized_layer_mix_bytes(mib, [16] * L)
    all_fp8 = orc.idealized_layer_mix_bytes(mib, [8] * L)
    mixed = orc.idealized_layer_mix_bytes(mib, [16] * 8 + [8] * 24)
    assert all_bf16 == g["all_bf16_mib"]
    assert all_fp8 == g["all_fp8_mib"]
    assert mixed == g["mixed_8bf16_24fp8_mib"]
    assert orc.relative_saving(all_bf16, mixed) == g["saving_vs_bf16"]
    assert mixed - all_fp8 == g["extra_vs_fp8_mib"]


def test_fp16_cache_bytes_batch4_8k(orc, gold):
    g = gold["fp16_cache_4x8k"]
    per_tok = orc.kv_bytes_per_token(n_layers=32, n_kv_heads=8, head_dim=128, bytes_per_elem=2)
    assert per_tok == 131072
    total = per_tok * g["batch"] * g["tokens"]
    assert total == 4 * 2**30
    assert abs(total - g["approx_bytes"]) / g["approx_bytes"] < 0.08


def test_throughput_definition(orc, gold):
    g = gold["throughput_definition"]
    assert orc.tokens_per_second(g["batch"], g["step_ms"]) == g["tokens_per_s"]


def test_table7_gains(orc, gold):
    g = gold["table7_tokens_per_s"]
    cols = g["columns"]
    for row in g["rows"].values():
        tps = dict(zip(cols, row["tokens_per_s"]))
        for name, pct in row["gain_pct"].items():
            gain = -orc.relative_saving(tps["KV8"], tps[name]) * 100
            # the printed percentages were rounded from unrounded throughputs
            assert abs(gain - pct) < 0.1, (name, gain, pct)


def test_page_bytes_closed_form(orc):
    for kb, vb in PAIRS:
        assert orc.head_page_bytes(kb, vb) == 512 * (kb + vb + 2)
        assert orc.page_bytes(1, kb, vb) == orc.head_page_bytes(kb, vb)
    # C3.25 on the Llama shape: 136 bytes per (token, KV head, layer) on average
    per_tok = sum(orc.page_bytes(8, k, v) for k, v in LLAMA_C325) / 32
    assert per_tok / 8 / 32 == 136
    assert orc.effective_bits(LLAMA_C325) == Fraction(17, 4)


# ------------------------------------------------------------------------------------
# binary16 / bfloat16 conversions against library routines
# ------------------------------------------------------------------------------------

def _special_f32():
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.996, 65520.0, 70000.0, 2.0**-14, 2.0**-24,
            2.0**-25, 3 * 2.0**-26, 2.0**-26, 1.5 * 2.0**-24, 2.5 * 2.0**-24, 1e-30, 3e38,
            1 + 2.0**-11, 1 + 3 * 2.0**-11, 1 + 2.0**-8, 1 + 3 * 2.0**-8, 0.1, 1 / 3, 2 / 3,
            1 / 15, 4 / 255, 6.103515625e-05]
    return np.array(vals + [-v for v in vals], dtype=np.float32)


def test_f16_conversion_matches_numpy(orc):
    rng = np.random.default_rng(1)
    mags = rng.uniform(-30, 17, 20000)
    xs = (np.sign(rng.standard_normal(20000)) * np.exp2(mags)).astype(np.float32)
    # exact ties between neighbouring binary16 values
    e = rng.integers(-24, 15, 4000)
    m = rng.integers(0, 2048, 4000)
    ties = ((2 * m + 1) * np.exp2(e.astype(np.float64) - 11)).astype(np.float32)
    allx = np.concatenate([xs, ties, _special_f32()])
    want = allx.astype(np.float16).view(np.uint16)
    got = np.array([orc.lib().orc_f32_to_f16(float(x)) for x in allx], dtype=np.uint16)
    assert np.array_equal(got, want)
    # every binary16 pattern (other than NaN) widens exactly
    bits = np.arange(65536, dtype=np.uint16)
    f = bits.view(np.float16)
    ok = ~np.isnan(f)
    widened = np.array([orc.lib().orc_f16_to_f32(int(b)) for b in bits[ok]], dtype=np.float32)
    assert np.array_equal(widened.view(np.uint32), f[ok].astype(np.float32).view(np.uint32))


def test_bf16_conversion_matches_torch(orc):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(2)
    xs = (rng.standard_normal(20000) * np.exp2(rng.uniform(-130, 120, 20000))).astype(np.float32)
    e = rng.integers(-133, 120, 4000)
    m = rng.integers(0, 256, 4000)
    ties = ((2 * m + 1) * np.exp2(e.astype(np.float64) - 8)).astype(np.float32)
    allx = np.concatenate([xs, ties, _special_f32()])
    want = torch.from_numpy(allx).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.lib().orc_f32_to_bf16(float(x)) for x in allx], dtype=np.uint16)
    assert np.array_equal(got, want)
    bits = np.arange(65536, dtype=np.uint16)
    tb = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    ok = ~np.isnan(tb)
    widened = np.array([orc.lib().orc_bf16_to_f32(int(b)) for b in bits[ok]], dtype=np.float32)
    assert np.array_equal(widened.view(np.uint32), tb[ok].view(np.uint32))


# ------------------------------------------------------------------------------------
# the group codec
# ------------------------------------------------------------------------------------

def f16(x):
    return int(np.float16(x).view(np.uint16))


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("scale_exp,zero", [(-6, -2.0), (-3, 0.5), (0, -7.0), (-10, 0.0)])
def test_grid_exactness(orc, bits, scale_exp, zero):
    """Inputs already on the grid {z + k s}, with k spanning 0 .. 2^b-1, come back exactly:
    the stored scale is s, the stored zero is z and the codes are k."""
    rng = np.random.default_rng(bits * 100 + scale_exp)
    s = 2.0**scale_exp
    top = 2**bits - 1
    for _ in range(20):
        k = rng.integers(0, top + 1, 32)
        k[0], k[1] = 0, top
        rng.shuffle(k)
        x = (zero + k * s).astype(np.float32)
        assert np.array_equal(x.astype(np.float64), zero + k * s)   # exact in fp32
        s16, z16, codes = orc.quant_group(x, bits)
        assert s16 == f16(s) and z16 == f16(zero)
        assert np.array_equal(codes, k)
        page_val = codes * np.float64(np.float16(s)) + np.float64(np.float16(zero))
        assert np.array_equal(page_val, x.astype(np.float64))


@pytest.mark.parametrize("bits", BITS)
def test_constant_group(orc, bits):
    x = np.full(32, 1.2345, dtype=np.float32)
    s16, z16, codes = orc.quant_group(x, bits)
    assert s16 == 0 and z16 == f16(np.float32(1.2345)) and not codes.any()


def test_tiny_scale_underflows_to_zero(orc):
    # range 2^-33 over 3 levels: scale < 2^-25 rounds to fp16 zero -> all codes 0
    x = np.full(32, 2.0**-10, dtype=np.float32)
    x[5] = np.float32(2.0**-10 + 2.0**-33)
    s16, z16, codes = orc.quant_group(x, 2)
    assert s16 == 0 and z16 == f16(2.0**-10) and not codes.any()
    # range 2^-23 over 3 levels is above 2^-25: it rounds up to the smallest subnormal
    x = np.full(32, 1.0, dtype=np.float32)
    x[5] = np.float32(1.0 + 2.0**-23)
    s16, z16, codes = orc.quant_group(x, 2)
    assert s16 == 1 and z16 == f16(1.0)
    # (x - 1) / 2^-24 = 2 -> code 2 for the larger element, 0 elsewhere
    assert codes[5] == 2 and codes.sum() == 2


def test_hand_computed_groups(orc):
    # 2-bit, values 0..3 on the unit grid plus the ties 0.5, 1.5, 2.5: round half to even
    x = np.zeros(32, dtype=np.float32)
    x[:7] = [0, 1, 2, 3, 0.5, 1.5, 2.5]
    s16, z16, codes = orc.quant_group(x, 2)
    assert (s16, z16) == (0x3C00, 0x0000)
    assert list(codes[:7]) == [0, 1, 2, 3, 0, 2, 2]
    # 4-bit, range [0, 1]: s32 = 1/15 -> binary16 1092 * 2^-14 = 0x2C44 (by hand)
    x = np.zeros(32, dtype=np.float32)
    x[1] = 1.0
    x[2] = 0.5
    s16, z16, codes = orc.quant_group(x, 4)
    assert s16 == 0x2C44 and z16 == 0
    # 0.5 / 0.066650390625 = 7.5018... -> 8 ; 1.0 / 0.06665... = 15.0037 -> 15
    assert (codes[1], codes[2], codes[0]) == (15, 8, 0)
    # negative zero is read as +0: the stored zero is +0, not -0
    x = np.zeros(32, dtype=np.float32)
    x[0] = -0.0
    x[3] = 3.0
    s16, z16, _ = orc.quant_group(x, 2)
    assert z16 == 0x0000 and s16 == 0x3C00
    # a shifted group: min -1.5, max 1.5, 2 bits -> s = 1, z = -1.5 (0xBE00)
    x = np.full(32, -1.5, dtype=np.float32)
    x[4], x[9], x[11] = 1.5, 0.0, -1.0
    s16, z16, codes = orc.quant_group(x, 2)
    assert (s16, z16) == (0x3C00, 0xBE00)
    # 0 - (-1.5) = 1.5 -> tie -> 2 ; -1 + 1.5 = 0.5 -> tie -> 0
    assert (codes[4], codes[9], codes[11], codes[0]) == (3, 2, 0, 0)


def _groups(rng, n):
    base = rng.standard_normal((n, 32)).astype(np.float32)
    base[n // 2:] *= 10.0                                    # outlier-scale groups
    base[: n // 8] = np.float32(3.0) + base[: n // 8] * 1e-3  # narrow groups away from zero
    return base


@pytest.mark.parametrize("bits", BITS)
def test_round_trip_bound_and_nearest_code(orc, bits):
    rng = np.random.default_rng(bits)
    top = 2**bits - 1
    for x in _groups(rng, 400):
        s16, z16, codes = orc.quant_group(x, bits)
        s = float(np.float16(np.uint16(s16).view(np.float16)))
        z = float(np.uint16(z16).view(np.float16))
        xd = x.astype(np.float64)
        mn, mx = xd.min(), xd.max()
        s32 = float(np.float32(np.float32(mx - mn) / np.float32(top)))
        deq = codes * s + z
        err = np.abs(xd - deq)
        bound = s / 2 + abs(z - mn) + top * max(0.0, s32 - s) + 2.0**-22 * np.maximum(np.abs(xd), abs(z))
        assert np.all(err <= bound), (bits, err.max(), bound.min())
        # each code is a nearest grid point among the representable codes
        for dc in (-1, 1):
            alt = np.clip(codes.astype(np.int64) + dc, 0, top)
            alt_err = np.abs(xd - (alt * s + z))
            assert np.all(err <= alt_err + 2.0**-20 * np.maximum(np.abs(xd), 1.0))


# ------------------------------------------------------------------------------------
# packed page layout
# ------------------------------------------------------------------------------------

def test_packed_bytes_hand_derived(orc):
    """Spec check of the byte layout with codes chosen so each byte is predictable."""
    # keys 2-bit: channel c of every token has code c % 4 -> each row byte is 0b11100100
    t_idx = np.arange(32)[:, None].astype(np.float32)
    c_idx = np.arange(128)[None, :].astype(np.float32)
    k = np.broadcast_to(c_idx % 4, (32, 128)).astype(np.float32).copy()
    k[:, :] += 0 * t_idx
    # make every channel group span the full grid so s = 1, z = 0: token 0 -> 0, token 1 -> 3
    k[0, :] = 0.0
    k[1, :] = 3.0
    v = np.zeros((32, 128), dtype=np.float32)
    v[:, 0] = 3.0                         # every value group j=0 spans [0, 3]
    v[:, 32] = 3.0
    v[:, 64] = 3.0
    v[:, 96] = 3.0
    page = orc.pack_page(k, v, 2, 2)
    kc = page[0:1024].reshape(32, 32)
    assert kc[0].tolist() == [0] * 32 and kc[1].tolist() == [0xFF] * 32
    assert all(kc[t].tolist() == [0xE4] * 32 for t in range(2, 32))
    ksz = page[1024:1536].view(np.uint32)
    assert np.all(ksz == 0x3C00)            # s = 1.0 (0x3C00) in the low half, z = +0 above
    # V codes, 2-bit: channels 0, 32, 64, 96 (r = 0, nb = 0, 2, 4, 6) have code 3 for every
    # token.  They sit in chunks 0, 16, 32, 48 (one per token octet, 16 bytes each); with
    # n = 8 codes per half-word, k = 4*nb + j -> word nb/2, bits 2j (tokens 8q..8q+3) and
    # 16 + 2j (tokens 8q+4..8q+7): words 0..3 of those chunks are 0x00FF00FF.
    vc = page[1536:2560]
    want = np.zeros(1024, dtype=np.uint8)
    for q in range(4):
        for w in range(4):
            want[16 * q * 16 + 4 * w + 0] = 0xFF
            want[16 * q * 16 + 4 * w + 2] = 0xFF
    assert np.array_equal(vc, want)
    vsz = page[2560:3072].view(np.uint32).reshape(32, 4)
    assert np.all(vsz == 0x3C00)
    # 4-bit keys: nibble order inside a byte is LSB-first
    k4 = np.zeros((32, 128), dtype=np.float32)
    k4[0, :] = 15.0                         # scale 1, zero 0 for every channel
    k4[5, 0], k4[5, 1], k4[5, 2] = 1.0, 2.0, 15.0
    page = orc.pack_page(k4, v, 4, 2)
    row5 = page[5 * 64:(5 + 1) * 64]
    assert row5[0] == 0x21 and row5[1] == 0x0F and not row5[2:].any()
    # 8-bit values: (token 7, channel 3): q = 0, r = 3 -> chunk 3 (64 bytes at offset 192);
    # i = 7 -> j = 3, half 1; k = 3 -> word 1, bit 16 + 8 = 24 -> byte 4 + 3 = 7: offset 199.
    # Channel 31 (r = 15, nb = 1) is 255 for every token: chunks 15, 31, 47, 63, k = 4..7
    # -> words 2 and 3 of each chunk are all ones.
    v8 = np.zeros((32, 128), dtype=np.float32)
    v8[:, 31] = 255.0                       # channel 31 pins s = 1 for group 0 of every token
    v8[7, 3] = 200.0
    page = orc.pack_page(k4, v8, 4, 8)
    vc8 = page[4 * 512 + 512: 4 * 512 + 512 + 4096]
    want = np.zeros(4096, dtype=np.uint8)
    want[199] = 200
    for q in range(4):
        base = (16 * q + 15) * 64
        want[base + 8: base + 16] = 255
    assert np.array_equal(vc8, want)


def _value_code_bits(orc, vb, cells):
    """Bit offset, inside the V code section, of the code of each (token, channel) cell,
    found by packing a tile whose only nonzero value is that cell (its group then spans
    [0, 1]: the cell gets code 2^vb - 1, every other code is 0)."""
    k = np.zeros((32, 128), dtype=np.float32)
    base = 512 * 2 + 512
    out = {}
    for t, c in cells:
        v = np.zeros((32, 128), dtype=np.float32)
        v[t, c] = 1.0
        page = orc.pack_page(k, v, 2, vb)
        bits = np.unpackbits(page[base:base + 512 * vb], bitorder="little")
        on = np.nonzero(bits)[0]
        assert len(on) == vb and on[-1] - on[0] == vb - 1 and on[0] % vb == 0, f"vb={vb} ({t}, {c}): {on}"
        out[(t, c)] = int(on[0])
    return out


@pytest.mark.parametrize("vb", BITS)
def test_value_code_layout_one_hot(orc, vb):
    """Every (token, channel) code sits where the format says: chunk 16*(t/8) + c%16 of
    8*vb bytes; inside it, with i = t%8, j = i%4, k = 4*(c/16) + j, n = 16/vb, at bit
    32*(k/n) + 16*(i/4) + vb*(k%n).  A few offsets are worked out by hand first."""
    hand = {2: {(0, 0): 0, (5, 17): 154, (12, 100): 2672},
            4: {(31, 127): 16380, (0, 16): 32, (9, 1): 17 * 256 + 4},
            8: {(7, 3): 1592, (0, 0): 0, (8, 0): 16 * 512}}[vb]
    got = _value_code_bits(orc, vb, list(hand))
    assert got == hand, f"vb={vb}: {got} != {hand}"
    cells = [(t, c) for t in range(32) for c in range(128)]
    got = _value_code_bits(orc, vb, cells)
    n = 16 // vb
    for (t, c), off in got.items():
        i, j = t % 8, t % 4
        k = 4 * (c // 16) + j
        want = (16 * (t // 8) + c % 16) * 64 * vb + 32 * (k // n) + 16 * (i // 4) + vb * (k % n)
        assert off == want, f"vb={vb} ({t}, {c}): bit {off}, format says {want}"
    assert sorted(got.values()) == [vb * x for x in range(4096)]


@pytest.mark.parametrize("kb,vb", PAIRS)
def test_page_round_trip_on_grid(orc, kb, vb):
    rng = np.random.default_rng(kb * 10 + vb)
    # keys: per channel a grid z_c + k s_c ; values: per (token, group) a grid
    sk = np.exp2(rng.integers(-8, 0, 128)).astype(np.float64)
    zk = rng.integers(-64, 64, 128) / 16.0
    kc = rng.integers(0, 2**kb, (32, 128))
    kc[0], kc[1] = 0, 2**kb - 1
    k = (zk[None, :] + kc * sk[None, :]).astype(np.float32)
    sv = np.exp2(rng.integers(-8, 0, (32, 4))).astype(np.float64)
    zv = rng.integers(-64, 64, (32, 4)) / 16.0
    vc = rng.integers(0, 2**vb, (32, 128))
    vc[:, 0::32], vc[:, 1::32] = 0, 2**vb - 1
    v = (np.repeat(zv, 32, axis=1) + vc * np.repeat(sv, 32, axis=1)).astype(np.float32)
    page = orc.pack_page(k, v, kb, vb)
    assert page.size == 512 * (kb + vb + 2)
    kd, vd = orc.dequant_page(page, kb, vb)
    assert np.array_equal(kd, k.astype(np.float64))
    assert np.array_equal(vd, v.astype(np.float64))


# ------------------------------------------------------------------------------------
# attention
# ------------------------------------------------------------------------------------

def _bf16_bits(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _bf16_val(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _build(orc, kb, vb, B, H, L, rng, src_dtype=np.uint16, shuffle=False, extra_pages=0):
    T = max(L)
    maxp = (T + 31) // 32
    n_phys = B * maxp + extra_pages
    k = rng.standard_normal((B, T, H, 128)).astype(np.float32)
    v = rng.standard_normal((B, T, H, 128)).astype(np.float32)
    k[..., 7] *= 10
    if src_dtype == np.uint16:
        ks, vs = _bf16_bits(k), _bf16_bits(v)
    else:
        ks, vs = k, v
    ids = np.arange(n_phys, dtype=np.int32)
    if shuffle:
        rng.shuffle(ids)
    bt = ids[: B * maxp].reshape(B, maxp).copy()
    pages, rk, rv = orc.new_cache(kb, vb, H, B, n_phys)
    orc.pack(kb, vb, ks, vs, np.array(L, dtype=np.int32), bt, pages, rk, rv)
    return ks, vs, bt, pages, rk, rv


def _textbook(q, K, V):
    s = (q @ K.T) / math.sqrt(128)
    m = s.max(axis=-1, keepdims=True)
    p = np.exp(s - m)
    return (p @ V) / p.sum(-1, keepdims=True), (m[..., 0] + np.log(p.sum(-1)))


def _dequant_seq(orc, kb, vb, pages, rk, rv, bt, b, h, L):
    K = np.zeros((L, 128))
    V = np.zeros((L, 128))
    for g in range(L // 32):
        kd, vd = orc.dequant_page(pages[bt[b, g], h], kb, vb)
        K[32 * g:32 * g + 32], V[32 * g:32 * g + 32] = kd, vd
    for t in range(32 * (L // 32), L):
        K[t] = _bf16_val(rk[b, h, t % 32])
        V[t] = _bf16_val(rv[b, h, t % 32])
    return K, V


@pytest.mark.parametrize("kb,vb,G", [(4, 2, 4), (8, 4, 1), (2, 2, 7), (4, 8, 4), (8, 8, 2)])
def test_attention_brute_force(orc, kb, vb, G):
    rng = np.random.default_rng(kb * 7 + vb * 3 + G)
    B, H = 2, 2
    L = [45, 64]
    ks, vs, bt, pages, rk, rv = _build(orc, kb, vb, B, H, L, rng, shuffle=True, extra_pages=3)
    q = _bf16_bits(rng.standard_normal((B, H * G, 128)))
    out, lse = orc.decode_attn(kb, vb, H, q, L, bt, pages, rk, rv)
    for b in range(B):
        for hq in range(H * G):
            K, V = _dequant_seq(orc, kb, vb, pages, rk, rv, bt, b, hq // G, L[b])
            o, l = _textbook(_bf16_val(q[b, hq]).astype(np.float64), K, V)
            assert np.allclose(out[b, hq], o, rtol=0, atol=1e-12)
            assert abs(lse[b, hq] - l) < 1e-12


def test_attention_single_token(orc):
    rng = np.random.default_rng(5)
    ks, vs, bt, pages, rk, rv = _build(orc, 4, 2, 1, 1, [1], rng)
    q = _bf16_bits(rng.standard_normal((1, 4, 128)))
    out, lse = orc.decode_attn(4, 2, 1, q, [1], bt, pages, rk, rv)
    v0 = _bf16_val(rv[0, 0, 0]).astype(np.float64)
    k0 = _bf16_val(rk[0, 0, 0]).astype(np.float64)
    for hq in range(4):
        assert np.array_equal(out[0, hq], v0)
        s0 = float(_bf16_val(q[0, hq]).astype(np.float64) @ k0) / math.sqrt(128)
        assert abs(lse[0, hq] - s0) < 1e-12


@pytest.mark.parametrize("L", [32, 77, 256])
def test_attention_equal_keys(orc, L):
    """All keys equal -> uniform weights: out = mean of the values, lse = s + ln L."""
    rng = np.random.default_rng(L)
    B, H, kb, vb = 1, 1, 4, 4
    kvec = _bf16_val(_bf16_bits(rng.standard_normal(128))).astype(np.float32)
    k = np.broadcast_to(kvec, (B, L, H, 128)).astype(np.float32)
    v = rng.standard_normal((B, L, H, 128)).astype(np.float32)
    ks, vs = _bf16_bits(k), _bf16_bits(v)
    maxp = (L + 31) // 32
    bt = np.arange(maxp, dtype=np.int32).reshape(1, maxp)
    pages, rk, rv = orc.new_cache(kb, vb, H, B, maxp)
    orc.pack(kb, vb, ks, vs, [L], bt, pages, rk, rv)
    q = _bf16_bits(rng.standard_normal((1, 2, 128)))
    out, lse = orc.decode_attn(kb, vb, H, q, [L], bt, pages, rk, rv)
    K, V = _dequant_seq(orc, kb, vb, pages, rk, rv, bt, 0, 0, L)
    assert np.all(K == K[0])                      # constant keys stay constant after the codec
    for hq in range(2):
        s = float(_bf16_val(q[0, hq]).astype(np.float64) @ K[0]) / math.sqrt(128)
        assert np.allclose(out[0, hq], V.mean(0), rtol=0, atol=1e-12)
        assert abs(lse[0, hq] - (s + math.log(L))) < 1e-12


def test_attention_on_grid_equals_unquantized(orc):
    """8-bit on-grid sources survive the codec exactly, so attention over the packed cache
    equals textbook attention over the sources."""
    rng = np.random.default_rng(11)
    L, kb, vb = 96, 8, 8
    kc = rng.integers(0, 256, (L, 128))
    kc[::32] = 0
    kc[1::32] = 255
    k = (-2.0 + kc / 64.0).astype(np.float32)
    vc = rng.integers(0, 256, (L, 128))
    vc[:, ::32] = 0
    vc[:, 1::32] = 255
    v = (-1.0 + vc / 128.0).astype(np.float32)
    bt = np.arange(3, dtype=np.int32).reshape(1, 3)
    pages, rk, rv = orc.new_cache(kb, vb, 1, 1, 3)
    orc.pack(kb, vb, k[None, :, None], v[None, :, None], [L], bt, pages, rk, rv)
    q = rng.standard_normal((1, 3, 128)).astype(np.float32)
    out, lse = orc.decode_attn(kb, vb, 1, q, [L], bt, pages, rk, rv)
    o, l = _textbook(q[0].astype(np.float64), k.astype(np.float64), v.astype(np.float64))
    assert np.allclose(out[0], o, rtol=0, atol=1e-12)
    assert np.allclose(lse[0], l, rtol=0, atol=1e-12)


def test_gqa_head_mapping(orc):
    """Query head hq reads KV head hq // G: give every KV head constant values equal to its
    index and check each query head's output."""
    H, G, L = 3, 4, 40
    v = np.zeros((1, L, H, 128), dtype=np.float32)
    for h in range(H):
        v[0, :, h, :] = h + 1
    rng = np.random.default_rng(3)
    k = rng.standard_normal((1, L, H, 128)).astype(np.float32)
    bt = np.arange(2, dtype=np.int32).reshape(1, 2)
    pages, rk, rv = orc.new_cache(2, 2, H, 1, 2)
    orc.pack(2, 2, _bf16_bits(k), _bf16_bits(v), [L], bt, pages, rk, rv)
    q = _bf16_bits(rng.standard_normal((1, H * G, 128)))
    out, _ = orc.decode_attn(2, 2, H, q, [L], bt, pages, rk, rv)
    for hq in range(H * G):
        assert np.allclose(out[0, hq], hq // G + 1, atol=1e-12)


def test_block_table_indirection(orc):
    rng = np.random.default_rng(9)
    L = [100, 33]
    ks, vs, bt, pages, rk, rv = _build(orc, 4, 2, 2, 2, L, rng, shuffle=False)
    q = _bf16_bits(rng.standard_normal((2, 8, 128)))
    out_a, lse_a = orc.decode_attn(4, 2, 2, q, L, bt, pages, rk, rv)
    perm = rng.permutation(pages.shape[0] + 5).astype(np.int32)
    pages2 = np.zeros((pages.shape[0] + 5,) + pages.shape[1:], dtype=np.uint8)
    bt2 = perm[: bt.size].reshape(bt.shape)
    pages2b, rk2, rv2 = orc.new_cache(4, 2, 2, 2, pages2.shape[0])
    orc.pack(4, 2, ks, vs, L, bt2, pages2b, rk2, rv2)
    for b in range(2):
        for g in range(L[b] // 32):
            assert np.array_equal(pages2b[bt2[b, g]], pages[bt[b, g]])
    out_b, lse_b = orc.decode_attn(4, 2, 2, q, L, bt2, pages2b, rk2, rv2)
    assert np.array_equal(out_a, out_b) and np.array_equal(lse_a, lse_b)


@pytest.mark.parametrize("L", [63, 64, 70])
@pytest.mark.parametrize("kb,vb", [(4, 2), (2, 8)])
def test_prefill_equals_prefix_plus_appends(orc, kb, vb, L):
    rng = np.random.default_rng(kb + vb + L)
    B, H, k0 = 2, 2, 25
    maxp = 3
    k = _bf16_bits(rng.standard_normal((B, L, H, 128)))
    v = _bf16_bits(rng.standard_normal((B, L, H, 128)))
    bt = np.arange(B * maxp, dtype=np.int32).reshape(B, maxp)
    full = orc.new_cache(kb, vb, H, B, B * maxp)
    orc.pack(kb, vb, k, v, [L] * B, bt, *full)
    inc = orc.new_cache(kb, vb, H, B, B * maxp)
    orc.pack(kb, vb, np.ascontiguousarray(k[:, :k0]), np.ascontiguousarray(v[:, :k0]),
             [k0] * B, bt, *inc)
    for t in range(k0, L):
        orc.append(kb, vb, np.ascontiguousarray(k[:, t]), np.ascontiguousarray(v[:, t]),
                   [t] * B, bt, *inc)
    assert np.array_equal(full[0], inc[0])
    live = slice(0, L % 32)
    assert np.array_equal(full[1][:, :, live], inc[1][:, :, live])
    assert np.array_equal(full[2][:, :, live], inc[2][:, :, live])


def test_fp32_source_residual_is_rne_bf16(orc):
    rng = np.random.default_rng(4)
    L = 40
    k = rng.standard_normal((1, L, 1, 128)).astype(np.float32)
    v = rng.standard_normal((1, L, 1, 128)).astype(np.float32)
    bt = np.arange(2, dtype=np.int32).reshape(1, 2)
    pages, rk, rv = orc.new_cache(8, 4, 1, 1, 2)
    orc.pack(8, 4, k, v, [L], bt, pages, rk, rv)
    assert np.array_equal(rk[0, 0, :8], _bf16_bits(k[0, 32:, 0]))
    assert np.array_equal(rv[0, 0, :8], _bf16_bits(v[0, 32:, 0]))


def test_oracle_rejects_bad_arguments(orc):
    with pytest.raises(ValueError):
        orc.quant_group(np.zeros(32, np.float32), 3)
    pages, rk, rv = orc.new_cache(4, 2, 1, 1, 1)
    with pytest.raises(ValueError):
        orc.decode_attn(4, 2, 1, np.zeros((1, 1, 128), np.float32), [64], np.zeros((1, 1), np.int32),
                        pages, rk, rv)


def test_oracle_calls_from_several_threads_agree(orc):
    """The full-size parity tests call the oracle from a thread pool: pack, append and decode
    keep no state between calls, so concurrent calls give the single-threaded results."""
    from concurrent.futures import ThreadPoolExecutor
    rng = np.random.default_rng(11)
    B, H, L = 2, 2, 200
    k = rng.standard_normal((B, L, H, 128)).astype(np.float32)
    v = rng.standard_normal((B, L, H, 128)).astype(np.float32)
    kn = rng.standard_normal((B, H, 128)).astype(np.float32)
    q = rng.standard_normal((B, 4 * H, 128)).astype(np.float32)
    bt = np.arange(B * 8, dtype=np.int32).reshape(B, 8)
    kn16 = _bf16_bits(kn).reshape(B, H, 128)

    def run(_):
        pages, rk, rv = orc.new_cache(4, 2, H, B, B * 8)
        orc.pack(4, 2, k, v, [L - 9, L], bt, pages, rk, rv)
        orc.append(4, 2, kn16, kn16, [L - 9, L], bt, pages, rk, rv)
        out, lse = orc.decode_attn(4, 2, H, q, [L - 8, L + 1], bt, pages, rk, rv)
        return pages, out, lse

    ref = run(0)
    with ThreadPoolExecutor(8) as ex:
        for got in ex.map(run, range(16)):
            assert all(np.array_equal(a, b) for a, b in zip(ref, got))
