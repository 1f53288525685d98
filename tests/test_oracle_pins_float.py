"""Pins of the oracle's floating-point layer formats (OCP FP8 E4M3 with per-head scales,
and BF16), the per-layer BF16/FP8 mix the machinoai page describes.

  * E4M3 decode of all 256 bit patterns equals torch's float8_e4m3fn;
  * E4M3 encode of in-range values (including exact rounding ties) equals torch's
    round-to-nearest-even cast; beyond 448 it saturates (the reading this library takes:
    the format has no infinity and S.1111.111 is NaN);
  * BF16 pages round-trip bf16 inputs exactly; FP8 pages dequantize to
    fp8(x / scale) * scale with the scale division in binary32;
  * head-page layout found by one-hot tiles: K token-major, V channel-major;
  * page bytes reproduce the page's 32-layer example (8 BF16 + 24 FP8 = 2000 of 3200 MiB);
  * attention equals a textbook evaluation over the dequantized pages;
  * prefill == prefix + appends in the FP8 format.
"""
import json
import math
import os

import numpy as np
import pytest


@pytest.fixture(scope="module")
def gold():
    with open(os.path.join(os.path.dirname(__file__), "golden", "pages_closed_forms.json")) as f:
        return json.load(f)


def _bf16_bits(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _bf16_val(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _torch_fp8(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def _torch_fp8_val(b):
    import torch
    return torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def test_fp8_decode_all_patterns(orc):
    ours = np.array([orc.fp8_to_f32(b) for b in range(256)], dtype=np.float32)
    ref = _torch_fp8_val(np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[~np.isnan(ours)], ref[~np.isnan(ref)])


def test_fp8_encode_round_to_nearest_even(orc):
    rng = np.random.default_rng(3)
    finite = np.array([orc.fp8_to_f32(b) for b in range(256) if (b & 0x7f) != 0x7f], dtype=np.float64)
    pos = np.unique(finite[finite >= 0])
    mids = (pos[:-1] + pos[1:]) / 2            # exact ties between neighbouring values
    xs = np.concatenate([rng.standard_normal(4000) * 30, rng.standard_normal(1000) * 0.01, mids, -mids,
                         [0.0, 448.0, -448.0, 2.0**-9, 2.0**-10, 1.5 * 2.0**-9]]).astype(np.float32)
    xs = xs[np.abs(xs) <= 448]
    ours = np.array([orc.f32_to_fp8(float(x)) for x in xs], dtype=np.uint8)
    assert np.array_equal(ours, _torch_fp8(xs))
    for x, want in [(448.5, 0x7e), (464.0, 0x7e), (480.0, 0x7e), (1e9, 0x7e), (-500.0, 0xfe)]:
        assert orc.f32_to_fp8(x) == want


def test_bf16_page_round_trip(orc):
    rng = np.random.default_rng(4)
    k = _bf16_val(_bf16_bits(rng.standard_normal((32, 128)) * 10))
    v = _bf16_val(_bf16_bits(rng.standard_normal((32, 128))))
    page = orc.pack_page(k, v, 16, 16, orc.FMT_BF16)
    assert page.size == 32 * 128 * 4
    kd, vd = orc.dequant_page(page, 16, 16, orc.FMT_BF16)
    assert np.array_equal(kd, k.astype(np.float64)) and np.array_equal(vd, v.astype(np.float64))


@pytest.mark.parametrize("ks,vs", [(1.0, 1.0), (0.0625, 3.0), (0.7, 0.013)])
def test_fp8_page_values(orc, ks, vs):
    rng = np.random.default_rng(5)
    k = (rng.standard_normal((32, 128)) * 10).astype(np.float32)
    v = rng.standard_normal((32, 128)).astype(np.float32)
    page = orc.pack_page(k, v, 8, 8, orc.FMT_FP8, ks, vs)
    assert page.size == 32 * 128 * 2
    kd, vd = orc.dequant_page(page, 8, 8, orc.FMT_FP8, ks, vs)
    kq = (k / np.float32(ks)).astype(np.float32)
    vq = (v / np.float32(vs)).astype(np.float32)
    kref = _torch_fp8_val(_torch_fp8(np.clip(kq, -448, 448))).astype(np.float64) * np.float64(np.float32(ks))
    vref = _torch_fp8_val(_torch_fp8(np.clip(vq, -448, 448))).astype(np.float64) * np.float64(np.float32(vs))
    assert np.array_equal(kd, kref) and np.array_equal(vd, vref)


@pytest.mark.parametrize("fmt,bits,esz", [(3, 16, 2), (2, 8, 1)])
def test_float_page_layout(orc, fmt, bits, esz):
    for t, c in [(0, 0), (0, 1), (1, 0), (5, 77), (31, 127), (17, 32)]:
        k = np.zeros((32, 128), np.float32)
        v = np.zeros((32, 128), np.float32)
        k[t, c] = 1.0
        v[t, c] = 1.0
        page = orc.pack_page(k, v, bits, bits, fmt)
        nz = np.nonzero(page)[0]
        kpos = (t * 128 + c) * esz
        vpos = 32 * 128 * esz + (c * 32 + t) * esz
        assert set(nz.tolist()) <= set(range(kpos, kpos + esz)) | set(range(vpos, vpos + esz)), (t, c, nz)
        assert any(kpos <= i < kpos + esz for i in nz) and any(vpos <= i < vpos + esz for i in nz)


def test_bf16_fp8_mix_bytes_match_the_pages_example(orc, gold):
    g = gold["idealized_bf16_fp8_mix"]
    bf16 = orc.head_page_bytes_fmt(16, 16, orc.FMT_BF16)
    fp8 = orc.head_page_bytes_fmt(8, 8, orc.FMT_FP8)
    unit = g["bf16_layer_mib"] / bf16               # MiB per byte of head page, any fixed shape
    assert g["layers"] * bf16 * unit == g["all_bf16_mib"]
    assert g["layers"] * fp8 * unit == g["all_fp8_mib"]
    mixed = (8 * bf16 + 24 * fp8) * unit
    assert mixed == g["mixed_8bf16_24fp8_mib"]
    assert (g["all_bf16_mib"] - mixed) / g["all_bf16_mib"] == g["saving_vs_bf16"]
    assert mixed - g["all_fp8_mib"] == g["extra_vs_fp8_mib"]


def _textbook(q, K, V):
    s = (q @ K.T) / math.sqrt(128)
    m = s.max()
    p = np.exp(s - m)
    return (p @ V) / p.sum(), m + math.log(p.sum())


@pytest.mark.parametrize("fmt,bits", [(2, 8), (3, 16)])
def test_float_attention_brute_force(orc, fmt, bits):
    rng = np.random.default_rng(6 + fmt)
    B, H, G, L, T, maxp = 2, 2, 4, [45, 70], 70, 3
    k = _bf16_bits(rng.standard_normal((B, T, H, 128)) * 3)
    v = _bf16_bits(rng.standard_normal((B, T, H, 128)))
    scales = np.array([[0.05, 0.01], [0.02, 0.004]], np.float32) if fmt == 2 else None
    bt = np.arange(B * maxp, dtype=np.int32).reshape(B, maxp)
    pages, rk, rv = orc.new_cache(bits, bits, H, B, B * maxp, fmt)
    orc.pack(bits, bits, k, v, L, bt, pages, rk, rv, kmode=fmt, scales=scales)
    q = _bf16_bits(rng.standard_normal((B, H * G, 128)))
    out, lse = orc.decode_attn(bits, bits, H, q, L, bt, pages, rk, rv, kmode=fmt, scales=scales)
    for b in range(B):
        for h in range(H):
            ks, vs = (scales[h] if scales is not None else (1.0, 1.0))
            K = np.zeros((L[b], 128))
            V = np.zeros((L[b], 128))
            for g in range(L[b] // 32):
                K[32 * g:32 * g + 32], V[32 * g:32 * g + 32] = orc.dequant_page(pages[bt[b, g], h], bits, bits, fmt,
                                                                                ks, vs)
            for t in range(32 * (L[b] // 32), L[b]):
                K[t], V[t] = _bf16_val(rk[b, h, t % 32]), _bf16_val(rv[b, h, t % 32])
            for gq in range(G):
                o, l = _textbook(_bf16_val(q[b, h * G + gq]).astype(np.float64), K, V)
                assert np.allclose(out[b, h * G + gq], o, rtol=0, atol=1e-12)
                assert abs(lse[b, h * G + gq] - l) < 1e-12


def test_fp8_prefill_equals_prefix_plus_appends(orc):
    rng = np.random.default_rng(7)
    B, H, L, k0, maxp = 2, 2, 70, 25, 3
    k = _bf16_bits(rng.standard_normal((B, L, H, 128)) * 4)
    v = _bf16_bits(rng.standard_normal((B, L, H, 128)))
    scales = np.array([[0.03, 0.01], [0.05, 0.008]], np.float32)
    bt = np.arange(B * maxp, dtype=np.int32).reshape(B, maxp)
    full = orc.new_cache(8, 8, H, B, B * maxp, orc.FMT_FP8)
    orc.pack(8, 8, k, v, [L] * B, bt, *full, kmode=orc.FMT_FP8, scales=scales)
    inc = orc.new_cache(8, 8, H, B, B * maxp, orc.FMT_FP8)
    orc.pack(8, 8, np.ascontiguousarray(k[:, :k0]), np.ascontiguousarray(v[:, :k0]), [k0] * B, bt, *inc,
             kmode=orc.FMT_FP8, scales=scales)
    for t in range(k0, L):
        orc.append(8, 8, np.ascontiguousarray(k[:, t]), np.ascontiguousarray(v[:, t]), [t] * B, bt, *inc,
                   kmode=orc.FMT_FP8, scales=scales)
    assert np.array_equal(full[0], inc[0])
    live = slice(0, L % 32)
    assert np.array_equal(full[1][:, :, live], inc[1][:, :, live])
