/*
 * kvq_oracle.c -- plain, slow CPU reference ("oracle") for layer-wise mixed-precision
 * KV-cache quantization and for single-token decode attention over the packed cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load this library.  The GPU library neither links nor calls it, and the
 * two share no source, header, table or helper.
 *
 * What it computes, and where that comes from:
 *   - Keys are quantized per channel (asymmetric, min/max over a group of tokens) because
 *     keys carry channel-wise outliers; values are quantized per token (asymmetric, min/max
 *     over a group of channels).
 *       [Mixed-precision KV-cache quantization per-layer sensitivity (llms-explorer.com),
 *        Facts: per-channel vs per-token keys]
 *       [KVTuner OpenReview discussion (paperhub.cn/paper/zDwipF6h06), reply to reviewer 1,
 *        section 4 "Per-channel vs. per-token quantization"; reply to reviewer 2, section 2
 *        "Discussion of conflicting literature" (per-channel keys, per-token values)]
 *   - Each layer carries its own (key bits, value bits) pair from an offline table; online,
 *     only the newly generated token is quantized, at that layer's pair.
 *       [KVTuner (mlsanity.com/paper/2502.04420), Abstract]
 *       [KVTuner OpenReview discussion, reply to reviewer 3, section 1 "Computational cost"]
 *   - Decode attention runs over the dequantized cache (FlashAttention-compatible method).
 *       [KVTuner OpenReview discussion, reply to reviewer 2, section 1 "Efficiency evaluation
 *        clarifications"]
 *   - Format of this library: groups of 32 (32 tokens per key group, 32 channels per value
 *     group), scale and zero stored as IEEE binary16, head_dim 128, bit widths {2,4,8}, and
 *     the tokens that do not yet fill a 32-token group kept unquantized as bfloat16.
 *
 * Arithmetic: the codec runs in IEEE binary32 exactly as written below (every operation
 * rounds to nearest-even; no contraction, no fast-math; SSE2 on x86-64), the attention runs
 * in IEEE binary64.  The fp16 and bf16 conversions are written from the formats'
 * definitions using exact binary64 arithmetic.
 */
#include <float.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if !defined(FLT_EVAL_METHOD) || FLT_EVAL_METHOD != 0
#error "the oracle needs binary32 evaluation of float expressions (x86-64 SSE2)"
#endif

#define ORC_D 128     /* head dimension */
#define ORC_G 32      /* tokens per key group == channels per value group == tokens per page */

/* ------------------------------------------------------------------------------------ */
/* binary16 / bfloat16 conversions                                                      */
/* ------------------------------------------------------------------------------------ */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Normal: (1024 + m) * 2^(e - 25); subnormal (e == 0): m * 2^-24. */
float orc_f16_to_f32(uint16_t h)
{
    int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return (float)(sign ? -v : v);
}

/* Round a binary32 value to the nearest binary16 value, ties to even. */
uint16_t orc_f32_to_f16(float xf)
{
    double x = xf;
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sign | 0x7e00u);
    double a = fabs(x);
    if (isinf(a)) return (uint16_t)(sign | 0x7c00u);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);               /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;
    if (E < -14) E = -14;        /* subnormals share the spacing of the lowest normal binade */
    double quantum = ldexp(1.0, E - 10);
    double n = nearbyint(a / quantum);   /* exact quotient, rounded to integer, ties to even */
    if (n == 0.0) return sign;
    if (n >= 2048.0) { n /= 2.0; E += 1; }
    if (E > 15) return (uint16_t)(sign | 0x7c00u);
    if (n < 1024.0) return (uint16_t)(sign | (uint16_t)n);            /* subnormal */
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(n - 1024.0));
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.
 * Normal: (128 + m) * 2^(e - 134); subnormal: m * 2^-133. */
float orc_bf16_to_f32(uint16_t b)
{
    int sign = b >> 15, e = (b >> 7) & 255, m = b & 127;
    double v;
    if (e == 0)
        v = ldexp((double)m, -133);
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + m), e - 134);
    return (float)(sign ? -v : v);
}

/* Round a binary32 value to the nearest bfloat16 value, ties to even. */
uint16_t orc_f32_to_bf16(float xf)
{
    double x = xf;
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sign | 0x7fc0u);
    double a = fabs(x);
    if (isinf(a)) return (uint16_t)(sign | 0x7f80u);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);
    int E = e2 - 1;
    if (E < -126) E = -126;
    double quantum = ldexp(1.0, E - 7);
    double n = nearbyint(a / quantum);
    if (n == 0.0) return sign;
    if (n >= 256.0) { n /= 2.0; E += 1; }
    if (E > 127) return (uint16_t)(sign | 0x7f80u);
    if (n < 128.0) return (uint16_t)(sign | (uint16_t)n);
    return (uint16_t)(sign | (uint16_t)((E + 127) << 7) | (uint16_t)(n - 128.0));
}

/* OCP FP8 E4M3 (the "fn" variant): 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits;
 * no infinities, S.1111.111 is NaN, the largest finite value is 448 = 1.75 * 2^8.
 * Normal (e >= 1): (8 + m) * 2^(e - 10); subnormal (e == 0): m * 2^-9. */
float orc_fp8_to_f32(uint8_t b)
{
    int sign = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 10);
    return (float)(sign ? -v : v);
}

/* Round a binary32 value to the nearest E4M3 value, ties to even; finite values beyond
 * the largest finite E4M3 value saturate to +-448 (the format has no infinity). */
uint8_t orc_f32_to_fp8(float xf)
{
    double x = xf;
    uint8_t sign = signbit(x) ? 0x80u : 0u;
    if (isnan(x)) return (uint8_t)(sign | 0x7fu);
    double a = fabs(x);
    if (a == 0.0) return sign;
    if (isinf(a)) return (uint8_t)(sign | 0x7eu);
    int e2;
    frexp(a, &e2);
    int E = e2 - 1;
    if (E < -6) E = -6;          /* subnormals share the spacing of the lowest normal binade */
    double quantum = ldexp(1.0, E - 3);
    double n = nearbyint(a / quantum);
    if (n == 0.0) return sign;
    if (n >= 16.0) { n /= 2.0; E += 1; }
    if (E > 8 || (E == 8 && n > 14.0)) return (uint8_t)(sign | 0x7eu);   /* saturate to 448 */
    if (n < 8.0) return (uint8_t)(sign | (uint8_t)n);
    return (uint8_t)(sign | (uint8_t)((E + 7) << 3) | (uint8_t)(n - 8.0));
}

/* ------------------------------------------------------------------------------------ */
/* the group codec                                                                      */
/* ------------------------------------------------------------------------------------ */

static int valid_bits(int b) { return b == 2 || b == 4 || b == 8; }

/* Quantize one group of 32 values x[0], x[stride], ... to `bits`-bit unsigned codes.
 *   mn, mx   : minimum and maximum of the group (binary32, exact)
 *   s32      : (mx - mn) / (2^bits - 1), one binary32 subtraction and one binary32 division
 *   s16, z16 : binary16 round-to-nearest-even of s32 and of mn  (the stored scale and zero)
 *   code_i   : clamp(round_half_even((x_i - z) / s), 0, 2^bits - 1), with s, z the stored
 *              binary16 values widened to binary32; every code is 0 when s == 0.
 * Dequantization is code * s + z.  -0 inputs are read as +0 so the stored zero never
 * depends on the order of a min over signed zeros. */
int orc_quant_group(const float *x, int stride, int bits,
                    uint16_t *s16_out, uint16_t *z16_out, uint8_t *codes)
{
    if (!valid_bits(bits)) return 1;
    float v[ORC_G];
    for (int i = 0; i < ORC_G; ++i) v[i] = x[(ptrdiff_t)i * stride] + 0.0f;
    float mn = v[0], mx = v[0];
    for (int i = 1; i < ORC_G; ++i) {
        if (v[i] < mn) mn = v[i];
        if (v[i] > mx) mx = v[i];
    }
    const float levels = (float)((1 << bits) - 1);
    float range = mx - mn;
    float s32 = range / levels;
    uint16_t s16 = orc_f32_to_f16(s32);
    uint16_t z16 = orc_f32_to_f16(mn);
    float s = orc_f16_to_f32(s16);
    float z = orc_f16_to_f32(z16);
    for (int i = 0; i < ORC_G; ++i) {
        if (s == 0.0f) { codes[i] = 0; continue; }
        float d = v[i] - z;
        float q = d / s;
        float r = rintf(q);
        if (r < 0.0f) r = 0.0f;
        if (r > levels) r = levels;
        codes[i] = (uint8_t)r;
    }
    *s16_out = s16;
    *z16_out = z16;
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* packed page layout (one page = 32 tokens of one KV head of one layer)                */
/*                                                                                      */
/*   offset 0            K codes, token-major: 32 rows of 16*kb bytes; token t, channel  */
/*                       c sits at bit c*kb of row t (LSB-first, little-endian bytes)    */
/*   offset 512*kb       K scale/zero: 128 words of 32 bits; word c = s16 | z16 << 16,   */
/*                       the group of channel c over the page's 32 tokens                */
/*   offset 512*kb+512   V codes, 64 chunks of 8*vb bytes; see vcode_bit() for the bit   */
/*                       of (token t, channel c)                                         */
/*   offset 512*(kb+vb)+512  V scale/zero: 32 tokens x 4 groups of 32-bit words;         */
/*                       word 4*t + j = s16 | z16 << 16 for channels 32j .. 32j+31       */
/*   total 512*(kb+vb+2) bytes                                                           */
/*                                                                                      */
/* A layer's pool is [physical page][KV head][page bytes]; block_table[b][i] names the   */
/* physical page that holds tokens 32i .. 32i+31 of sequence b.                         */
/* ------------------------------------------------------------------------------------ */

size_t orc_head_page_bytes(int kb, int vb) { return (size_t)512 * (size_t)(kb + vb + 2); }

static size_t off_kcodes(int kb, int vb) { (void)kb; (void)vb; return 0; }
static size_t off_ksz(int kb, int vb) { (void)vb; return (size_t)512 * kb; }
static size_t off_vcodes(int kb, int vb) { (void)vb; return (size_t)512 * kb + 512; }
static size_t off_vsz(int kb, int vb) { return (size_t)512 * (kb + vb) + 512; }

/* Bit offset of the value code of (token t, channel c) inside the V code section.
 * The section is 64 chunks of 8*vb bytes.  Chunk 16*q + r holds the 64 codes of tokens
 * 8q .. 8q+7 and channels r, r+16, ..., r+112.  Inside a chunk, with i = t mod 8,
 * j = i mod 4, hh = i / 4, nb = c / 16, k = 4*nb + j and n = 16 / vb codes per 16-bit
 * half-word, the code sits at bit 32*(k / n) + 16*hh + vb*(k mod n).
 * (Each 16-bit half of a 32-bit word then holds codes of consecutive k for one half of
 * the token octet, so one shift and one mask extract a pair of codes of one channel for
 * tokens 8q+j and 8q+j+4.) */
static size_t vcode_bit(int t, int c, int vb)
{
    int q = t / 8, i = t % 8, r = c % 16, nb = c / 16;
    int j = i % 4, hh = i / 4;
    int k = 4 * nb + j;
    int n = 16 / vb;
    size_t chunk_bits = (size_t)(16 * q + r) * 8 * vb * 8;
    return chunk_bits + 32 * (size_t)(k / n) + 16 * (size_t)hh + (size_t)vb * (k % n);
}

/* Key modes.  KMODE_CHANNEL: one key group per channel over the page's 32 tokens; token
 * row t holds channel c at bit c*kb; K s/z word c.  KMODE_TOKEN: one key group per
 * (token, 32 consecutive channels), like the values; K s/z word 4t + j for channels
 * 32j .. 32j+31, and the row's channels are permuted as follows.
 *   [When should you use mixed-precision KV caching ... (machinoai.in); KVTuner OpenReview
 *    discussion, reply to reviewer 1, section 4 (per-token asymmetric keys)]
 * Per-token key row layout: the row's 16*kb bytes are four chunks of 4*kb bytes; slot s of
 * chunk a (bits s*kb .. s*kb + kb-1 of the chunk) holds channel
 *     32*(k / 4) + 8*a + 2*(k % 4) + hh,   with n = 16/kb, x = s / (2n),
 *     hh = (s / n) mod 2, p = s mod n, k = x*n + p.
 * So chunk a holds channels 32J + 8a .. 32J + 8a + 7 of every key group J, and the two
 * channels 32J + 8a + 2i and 32J + 8a + 2i + 1 sit at the same position of the two 16-bit
 * halves of one 32-bit word. */
enum { KMODE_CHANNEL = 0, KMODE_TOKEN = 1 };

static int kslot_channel(int a, int slot, int kb)
{
    int n = 16 / kb;
    int x = slot / (2 * n), hh = (slot / n) % 2, p = slot % n;
    int k = x * n + p;
    return 32 * (k / 4) + 8 * a + 2 * (k % 4) + hh;
}

/* bit offset, inside a per-token key row, of channel c */
static size_t ktok_bit(int c, int kb)
{
    for (int a = 0; a < 4; ++a)
        for (int slot = 0; slot < 32; ++slot)
            if (kslot_channel(a, slot, kb) == c) return (size_t)(a * 32 + slot) * kb;
    return (size_t)-1;
}

static void put_code_at(uint8_t *base, size_t bit, unsigned code)
{
    base[bit / 8] |= (uint8_t)(code << (bit % 8));
}

static unsigned get_code_at(const uint8_t *base, size_t bit, int bits)
{
    return (base[bit / 8] >> (bit % 8)) & ((1u << bits) - 1u);
}

static void put_code(uint8_t *row, int idx, int bits, unsigned code)
{
    size_t bit = (size_t)idx * bits;
    row[bit / 8] |= (uint8_t)(code << (bit % 8));
}

static unsigned get_code(const uint8_t *row, int idx, int bits)
{
    size_t bit = (size_t)idx * bits;
    return (row[bit / 8] >> (bit % 8)) & ((1u << bits) - 1u);
}

static void put_u32(uint8_t *p, uint32_t w)
{
    p[0] = (uint8_t)w; p[1] = (uint8_t)(w >> 8); p[2] = (uint8_t)(w >> 16); p[3] = (uint8_t)(w >> 24);
}

static uint32_t get_u32(const uint8_t *p)
{
    return (uint32_t)p[0] | (uint32_t)p[1] << 8 | (uint32_t)p[2] << 16 | (uint32_t)p[3] << 24;
}

/* Quantize one page: k and v point at token 0, channel 0 of a 32 x 128 fp32 tile whose
 * consecutive tokens are `tok_stride` floats apart. */
int orc_pack_page_m(const float *k, const float *v, int tok_stride, int kb, int vb, int kmode, uint8_t *dst)
{
    if (!valid_bits(kb) || !valid_bits(vb) || (kmode != KMODE_CHANNEL && kmode != KMODE_TOKEN)) return 1;
    memset(dst, 0, orc_head_page_bytes(kb, vb));
    uint8_t codes[ORC_G];
    uint16_t s16, z16;
    if (kmode == KMODE_CHANNEL) {
        /* keys: one group per channel, over the page's 32 tokens */
        for (int c = 0; c < ORC_D; ++c) {
            orc_quant_group(k + c, tok_stride, kb, &s16, &z16, codes);
            for (int t = 0; t < ORC_G; ++t)
                put_code(dst + off_kcodes(kb, vb) + (size_t)t * 16 * kb, c, kb, codes[t]);
            put_u32(dst + off_ksz(kb, vb) + 4 * (size_t)c, (uint32_t)s16 | (uint32_t)z16 << 16);
        }
    } else {
        /* keys: one group per (token, 32 consecutive channels) */
        for (int t = 0; t < ORC_G; ++t)
            for (int j = 0; j < ORC_D / ORC_G; ++j) {
                orc_quant_group(k + (size_t)t * tok_stride + 32 * j, 1, kb, &s16, &z16, codes);
                for (int i = 0; i < ORC_G; ++i)
                    put_code_at(dst + off_kcodes(kb, vb) + (size_t)t * 16 * kb, ktok_bit(32 * j + i, kb), codes[i]);
                put_u32(dst + off_ksz(kb, vb) + 4 * (size_t)(4 * t + j), (uint32_t)s16 | (uint32_t)z16 << 16);
            }
    }
    /* values: one group per (token, 32 consecutive channels) */
    for (int t = 0; t < ORC_G; ++t) {
        for (int j = 0; j < ORC_D / ORC_G; ++j) {
            orc_quant_group(v + (size_t)t * tok_stride + 32 * j, 1, vb, &s16, &z16, codes);
            for (int i = 0; i < ORC_G; ++i)
                put_code_at(dst + off_vcodes(kb, vb), vcode_bit(t, 32 * j + i, vb), codes[i]);
            put_u32(dst + off_vsz(kb, vb) + 4 * (size_t)(4 * t + j),
                    (uint32_t)s16 | (uint32_t)z16 << 16);
        }
    }
    return 0;
}

int orc_pack_page(const float *k, const float *v, int tok_stride, int kb, int vb, uint8_t *dst)
{
    return orc_pack_page_m(k, v, tok_stride, kb, vb, KMODE_CHANNEL, dst);
}

/* Floating-point layer formats (a layer stores its K and V in one of them instead of the
 * integer codes): FMT_FP8 keeps x / scale as OCP E4M3 with one K scale and one V scale per
 * (layer, KV head); FMT_BF16 keeps x as bfloat16.  [When should you use mixed-precision
 * KV caching to preserve accuracy in sensitive transformer layers (machinoai.in),
 * sections 1-2: sensitive layers in BF16, the rest in FP8, per-head calibration scales]
 * Head page: K token-major [32][128] elements at +0, then V channel-major [128][32]
 * (element (t, c) at c*32 + t), 1 byte (FP8) or 2 bytes (BF16) per element.  The division
 * x / scale is one IEEE binary32 division, then rounding to E4M3. */
enum { FMT_INT_CHANNEL = 0, FMT_INT_TOKEN = 1, FMT_FP8 = 2, FMT_BF16 = 3 };

int orc_dequant_page_m(const uint8_t *src, int kb, int vb, int kmode, double *k, double *v);

static int valid_format(int kb, int vb, int fmt)
{
    if (fmt == FMT_INT_CHANNEL || fmt == FMT_INT_TOKEN) return valid_bits(kb) && valid_bits(vb);
    if (fmt == FMT_FP8) return kb == 8 && vb == 8;
    if (fmt == FMT_BF16) return kb == 16 && vb == 16;
    return 0;
}

size_t orc_head_page_bytes_x(int kb, int vb, int fmt)
{
    if (!valid_format(kb, vb, fmt)) return 0;
    if (fmt == FMT_FP8) return (size_t)ORC_G * ORC_D * 2;
    if (fmt == FMT_BF16) return (size_t)ORC_G * ORC_D * 4;
    return orc_head_page_bytes(kb, vb);
}

static void pack_page_float(const float *k, const float *v, int tok_stride, int fmt, float ks, float vs,
                            uint8_t *dst)
{
    const size_t esz = fmt == FMT_FP8 ? 1 : 2;
    uint8_t *vdst = dst + (size_t)ORC_G * ORC_D * esz;
    for (int t = 0; t < ORC_G; ++t)
        for (int c = 0; c < ORC_D; ++c) {
            float kx = k[(size_t)t * tok_stride + c], vx = v[(size_t)t * tok_stride + c];
            size_t ki = (size_t)t * ORC_D + c, vi = (size_t)c * ORC_G + t;
            if (fmt == FMT_FP8) {
                dst[ki] = orc_f32_to_fp8(kx / ks);
                vdst[vi] = orc_f32_to_fp8(vx / vs);
            } else {
                uint16_t kb16 = orc_f32_to_bf16(kx), vb16 = orc_f32_to_bf16(vx);
                dst[2 * ki] = (uint8_t)kb16; dst[2 * ki + 1] = (uint8_t)(kb16 >> 8);
                vdst[2 * vi] = (uint8_t)vb16; vdst[2 * vi + 1] = (uint8_t)(vb16 >> 8);
            }
        }
}

/* binary64 values; E4M3 value times a binary32 scale is exact in binary64 */
static void dequant_page_float(const uint8_t *src, int fmt, float ks, float vs, double *k, double *v)
{
    const size_t esz = fmt == FMT_FP8 ? 1 : 2;
    const uint8_t *vsrc = src + (size_t)ORC_G * ORC_D * esz;
    for (int t = 0; t < ORC_G; ++t)
        for (int c = 0; c < ORC_D; ++c) {
            size_t ki = (size_t)t * ORC_D + c, vi = (size_t)c * ORC_G + t;
            if (fmt == FMT_FP8) {
                k[ki] = (double)orc_fp8_to_f32(src[ki]) * (double)ks;
                v[ki] = (double)orc_fp8_to_f32(vsrc[vi]) * (double)vs;
            } else {
                k[ki] = orc_bf16_to_f32((uint16_t)(src[2 * ki] | src[2 * ki + 1] << 8));
                v[ki] = orc_bf16_to_f32((uint16_t)(vsrc[2 * vi] | vsrc[2 * vi + 1] << 8));
            }
        }
}

int orc_pack_page_x(const float *k, const float *v, int tok_stride, int kb, int vb, int fmt, float ks, float vs,
                    uint8_t *dst)
{
    if (!valid_format(kb, vb, fmt)) return 1;
    if (fmt == FMT_FP8 || fmt == FMT_BF16) {
        pack_page_float(k, v, tok_stride, fmt, ks, vs, dst);
        return 0;
    }
    return orc_pack_page_m(k, v, tok_stride, kb, vb, fmt, dst);
}

int orc_dequant_page_x(const uint8_t *src, int kb, int vb, int fmt, float ks, float vs, double *k, double *v)
{
    if (!valid_format(kb, vb, fmt)) return 1;
    if (fmt == FMT_FP8 || fmt == FMT_BF16) {
        dequant_page_float(src, fmt, ks, vs, k, v);
        return 0;
    }
    return orc_dequant_page_m(src, kb, vb, fmt, k, v);
}

/* Decode one page into binary64 K and V tiles [32][128].  code * s + z is exact in
 * binary64 (an 8-bit integer times a binary16 value plus a binary16 value). */
int orc_dequant_page_m(const uint8_t *src, int kb, int vb, int kmode, double *k, double *v)
{
    if (!valid_bits(kb) || !valid_bits(vb) || (kmode != KMODE_CHANNEL && kmode != KMODE_TOKEN)) return 1;
    for (int t = 0; t < ORC_G; ++t) {
        const uint8_t *row = src + off_kcodes(kb, vb) + (size_t)t * 16 * kb;
        for (int c = 0; c < ORC_D; ++c) {
            size_t widx = kmode == KMODE_CHANNEL ? (size_t)c : (size_t)(4 * t + c / 32);
            uint32_t w = get_u32(src + off_ksz(kb, vb) + 4 * widx);
            double s = orc_f16_to_f32((uint16_t)(w & 0xffffu));
            double z = orc_f16_to_f32((uint16_t)(w >> 16));
            unsigned code = kmode == KMODE_CHANNEL ? get_code(row, c, kb) : get_code_at(row, ktok_bit(c, kb), kb);
            k[t * ORC_D + c] = (double)code * s + z;
        }
    }
    for (int t = 0; t < ORC_G; ++t) {
        for (int c = 0; c < ORC_D; ++c) {
            uint32_t w = get_u32(src + off_vsz(kb, vb) + 4 * (size_t)(4 * t + c / 32));
            double s = orc_f16_to_f32((uint16_t)(w & 0xffffu));
            double z = orc_f16_to_f32((uint16_t)(w >> 16));
            unsigned code = get_code_at(src + off_vcodes(kb, vb), vcode_bit(t, c, vb), vb);
            v[t * ORC_D + c] = (double)code * s + z;
        }
    }
    return 0;
}

int orc_dequant_page(const uint8_t *src, int kb, int vb, double *k, double *v)
{
    return orc_dequant_page_m(src, kb, vb, KMODE_CHANNEL, k, v);
}

/* ------------------------------------------------------------------------------------ */
/* layer-level operations                                                               */
/* ------------------------------------------------------------------------------------ */

static float src_elem(const void *src, int is_bf16, size_t i)
{
    return is_bf16 ? orc_bf16_to_f32(((const uint16_t *)src)[i]) : ((const float *)src)[i];
}

static uint16_t src_to_bf16(const void *src, int is_bf16, size_t i)
{
    return is_bf16 ? ((const uint16_t *)src)[i] : orc_f32_to_bf16(((const float *)src)[i]);
}

/* Prefill: quantize-on-write of sequences of length seq_len[b] taken from
 * k_src / v_src [batch][max_tokens][H][128] (bf16 or fp32).  Full 32-token groups go to
 * the pages named by the block table; the last seq_len mod 32 tokens go, as bf16, to
 * residual slot t mod 32 of resid_k / resid_v [batch][H][32][128]. */
/* Layer-level operations take a format code fmt (FMT_*; for the integer formats it is the
 * key mode) and, for FP8, scales[2*h] / scales[2*h + 1] = K / V scale of KV head h (NULL:
 * every scale 1). */
static float scale_of(const float *scales, int h, int which) { return scales ? scales[2 * h + which] : 1.0f; }

int orc_pack_x(int kb, int vb, int fmt, const float *scales, int H, int batch, int max_tokens, int src_is_bf16,
               const void *k_src, const void *v_src, const int32_t *seq_len,
               const int32_t *block_table, int max_pages,
               uint8_t *pages, uint16_t *resid_k, uint16_t *resid_v)
{
    if (!valid_format(kb, vb, fmt)) return 1;
    const size_t hp = orc_head_page_bytes_x(kb, vb, fmt);
    float tk[ORC_G * ORC_D], tv[ORC_G * ORC_D];   /* per call: the oracle is called from several threads */
    for (int b = 0; b < batch; ++b) {
        int L = seq_len[b];
        if (L < 0 || L > max_tokens || L > 32 * max_pages) return 2;
        int full = L / ORC_G;
        for (int h = 0; h < H; ++h) {
            for (int g = 0; g < full; ++g) {
                for (int t = 0; t < ORC_G; ++t)
                    for (int c = 0; c < ORC_D; ++c) {
                        size_t i = (((size_t)b * max_tokens + (size_t)(g * ORC_G + t)) * H + h) * ORC_D + c;
                        tk[t * ORC_D + c] = src_elem(k_src, src_is_bf16, i);
                        tv[t * ORC_D + c] = src_elem(v_src, src_is_bf16, i);
                    }
                int32_t phys = block_table[(size_t)b * max_pages + g];
                orc_pack_page_x(tk, tv, ORC_D, kb, vb, fmt, scale_of(scales, h, 0), scale_of(scales, h, 1),
                                pages + ((size_t)phys * H + h) * hp);
            }
            for (int t = full * ORC_G; t < L; ++t)
                for (int c = 0; c < ORC_D; ++c) {
                    size_t i = (((size_t)b * max_tokens + (size_t)t) * H + h) * ORC_D + c;
                    size_t r = (((size_t)b * H + h) * ORC_G + (size_t)(t % ORC_G)) * ORC_D + c;
                    resid_k[r] = src_to_bf16(k_src, src_is_bf16, i);
                    resid_v[r] = src_to_bf16(v_src, src_is_bf16, i);
                }
        }
    }
    return 0;
}

/* Decode-time write of one new token per sequence, at position pos[b] (the length before
 * the write).  The token goes to residual slot pos mod 32; when that slot is 31 the 32
 * residual tokens form a full group and are quantized into page pos / 32.
 * k_new / v_new are bf16 [batch][H][128]. */
int orc_append_x(int kb, int vb, int fmt, const float *scales, int H, int batch, const uint16_t *k_new,
                 const uint16_t *v_new, const int32_t *pos, const int32_t *block_table, int max_pages,
                 uint8_t *pages, uint16_t *resid_k, uint16_t *resid_v)
{
    if (!valid_format(kb, vb, fmt)) return 1;
    const size_t hp = orc_head_page_bytes_x(kb, vb, fmt);
    float tk[ORC_G * ORC_D], tv[ORC_G * ORC_D];   /* per call: the oracle is called from several threads */
    for (int b = 0; b < batch; ++b) {
        int p = pos[b];
        if (p < 0 || p >= 32 * max_pages) return 2;
        int slot = p % ORC_G;
        for (int h = 0; h < H; ++h) {
            uint16_t *rk = resid_k + ((size_t)b * H + h) * ORC_G * ORC_D;
            uint16_t *rv = resid_v + ((size_t)b * H + h) * ORC_G * ORC_D;
            for (int c = 0; c < ORC_D; ++c) {
                rk[slot * ORC_D + c] = k_new[((size_t)b * H + h) * ORC_D + c];
                rv[slot * ORC_D + c] = v_new[((size_t)b * H + h) * ORC_D + c];
            }
            if (slot == ORC_G - 1) {
                for (int i = 0; i < ORC_G * ORC_D; ++i) {
                    tk[i] = orc_bf16_to_f32(rk[i]);
                    tv[i] = orc_bf16_to_f32(rv[i]);
                }
                int32_t phys = block_table[(size_t)b * max_pages + p / ORC_G];
                orc_pack_page_x(tk, tv, ORC_D, kb, vb, fmt, scale_of(scales, h, 0), scale_of(scales, h, 1),
                                pages + ((size_t)phys * H + h) * hp);
            }
        }
    }
    return 0;
}

/* Single-token decode attention of every query head over the seq_len[b] cached tokens:
 * full pages 0 .. seq_len/32 - 1 (dequantized) and the seq_len mod 32 residual tokens
 * (exact bf16).  Query head hq reads KV head hq / (Hq / H).  In binary64:
 *   s_j = (sum_c q_c k_jc) / sqrt(128),  m = max_j s_j,  l = sum_j exp(s_j - m),
 *   lse = m + ln l,  out_c = sum_j exp(s_j - m) v_jc / l.
 * q is [batch][Hq][128] (bf16 or fp32); out is [batch][Hq][128]; lse is [batch][Hq]
 * (may be NULL). */
int orc_decode_attn_x(int kb, int vb, int fmt, const float *scales, int Hq, int H, int batch, int q_is_bf16,
                      const void *q, const int32_t *seq_len, const int32_t *block_table, int max_pages,
                      const uint8_t *pages, const uint16_t *resid_k, const uint16_t *resid_v,
                      double *out, double *lse)
{
    if (!valid_format(kb, vb, fmt)) return 1;
    if (H <= 0 || Hq % H != 0) return 3;
    const int G = Hq / H;
    const size_t hp = orc_head_page_bytes_x(kb, vb, fmt);
    for (int b = 0; b < batch; ++b) {
        int L = seq_len[b];
        if (L <= 0 || L > 32 * max_pages) return 2;
        int full = L / ORC_G;
        double *K = (double *)malloc(sizeof(double) * (size_t)L * ORC_D);
        double *V = (double *)malloc(sizeof(double) * (size_t)L * ORC_D);
        double *s = (double *)malloc(sizeof(double) * (size_t)L);
        if (!K || !V || !s) { free(K); free(V); free(s); return 4; }
        for (int h = 0; h < H; ++h) {
            /* this head's keys and values for all L tokens, as exact binary64 */
            for (int g = 0; g < full; ++g) {
                int32_t phys = block_table[(size_t)b * max_pages + g];
                orc_dequant_page_x(pages + ((size_t)phys * H + h) * hp, kb, vb, fmt, scale_of(scales, h, 0),
                                   scale_of(scales, h, 1), K + (size_t)g * ORC_G * ORC_D,
                                   V + (size_t)g * ORC_G * ORC_D);
            }
            const uint16_t *rk = resid_k + ((size_t)b * H + h) * ORC_G * ORC_D;
            const uint16_t *rv = resid_v + ((size_t)b * H + h) * ORC_G * ORC_D;
            for (int t = full * ORC_G; t < L; ++t)
                for (int c = 0; c < ORC_D; ++c) {
                    K[(size_t)t * ORC_D + c] = orc_bf16_to_f32(rk[(t % ORC_G) * ORC_D + c]);
                    V[(size_t)t * ORC_D + c] = orc_bf16_to_f32(rv[(t % ORC_G) * ORC_D + c]);
                }
            for (int gq = 0; gq < G; ++gq) {
                int hq = h * G + gq;
                double qd[ORC_D];
                for (int c = 0; c < ORC_D; ++c)
                    qd[c] = src_elem(q, q_is_bf16, ((size_t)b * Hq + hq) * ORC_D + c);
                double m = -INFINITY;
                for (int t = 0; t < L; ++t) {
                    double dot = 0.0;
                    for (int c = 0; c < ORC_D; ++c) dot += qd[c] * K[(size_t)t * ORC_D + c];
                    s[t] = dot / sqrt((double)ORC_D);
                    if (s[t] > m) m = s[t];
                }
                double l = 0.0, acc[ORC_D];
                for (int c = 0; c < ORC_D; ++c) acc[c] = 0.0;
                for (int t = 0; t < L; ++t) {
                    double p = exp(s[t] - m);
                    l += p;
                    for (int c = 0; c < ORC_D; ++c) acc[c] += p * V[(size_t)t * ORC_D + c];
                }
                for (int c = 0; c < ORC_D; ++c) out[((size_t)b * Hq + hq) * ORC_D + c] = acc[c] / l;
                if (lse) lse[(size_t)b * Hq + hq] = m + log(l);
            }
        }
        free(K); free(V); free(s);
    }
    return 0;
}

/* integer formats with a key mode */
int orc_pack_m(int kb, int vb, int kmode, int H, int batch, int max_tokens, int src_is_bf16,
               const void *k_src, const void *v_src, const int32_t *seq_len,
               const int32_t *block_table, int max_pages,
               uint8_t *pages, uint16_t *resid_k, uint16_t *resid_v)
{
    if (kmode != KMODE_CHANNEL && kmode != KMODE_TOKEN) return 1;
    return orc_pack_x(kb, vb, kmode, NULL, H, batch, max_tokens, src_is_bf16, k_src, v_src, seq_len, block_table,
                      max_pages, pages, resid_k, resid_v);
}

int orc_append_m(int kb, int vb, int kmode, int H, int batch, const uint16_t *k_new, const uint16_t *v_new,
                 const int32_t *pos, const int32_t *block_table, int max_pages,
                 uint8_t *pages, uint16_t *resid_k, uint16_t *resid_v)
{
    if (kmode != KMODE_CHANNEL && kmode != KMODE_TOKEN) return 1;
    return orc_append_x(kb, vb, kmode, NULL, H, batch, k_new, v_new, pos, block_table, max_pages, pages, resid_k,
                        resid_v);
}

int orc_decode_attn_m(int kb, int vb, int kmode, int Hq, int H, int batch, int q_is_bf16, const void *q,
                      const int32_t *seq_len, const int32_t *block_table, int max_pages,
                      const uint8_t *pages, const uint16_t *resid_k, const uint16_t *resid_v,
                      double *out, double *lse)
{
    if (kmode != KMODE_CHANNEL && kmode != KMODE_TOKEN) return 1;
    return orc_decode_attn_x(kb, vb, kmode, NULL, Hq, H, batch, q_is_bf16, q, seq_len, block_table, max_pages,
                             pages, resid_k, resid_v, out, lse);
}

/* per-channel-key entry points (the library's default key mode) */
int orc_pack(int kb, int vb, int H, int batch, int max_tokens, int src_is_bf16,
             const void *k_src, const void *v_src, const int32_t *seq_len,
             const int32_t *block_table, int max_pages,
             uint8_t *pages, uint16_t *resid_k, uint16_t *resid_v)
{
    return orc_pack_m(kb, vb, KMODE_CHANNEL, H, batch, max_tokens, src_is_bf16, k_src, v_src, seq_len,
                      block_table, max_pages, pages, resid_k, resid_v);
}

int orc_append(int kb, int vb, int H, int batch, const uint16_t *k_new, const uint16_t *v_new,
               const int32_t *pos, const int32_t *block_table, int max_pages,
               uint8_t *pages, uint16_t *resid_k, uint16_t *resid_v)
{
    return orc_append_m(kb, vb, KMODE_CHANNEL, H, batch, k_new, v_new, pos, block_table, max_pages,
                        pages, resid_k, resid_v);
}

int orc_decode_attn(int kb, int vb, int Hq, int H, int batch, int q_is_bf16, const void *q,
                    const int32_t *seq_len, const int32_t *block_table, int max_pages,
                    const uint8_t *pages, const uint16_t *resid_k, const uint16_t *resid_v,
                    double *out, double *lse)
{
    return orc_decode_attn_m(kb, vb, KMODE_CHANNEL, Hq, H, batch, q_is_bf16, q, seq_len, block_table, max_pages,
                             pages, resid_k, resid_v, out, lse);
}
