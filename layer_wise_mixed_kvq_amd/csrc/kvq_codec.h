// kvq_codec.h -- the page codec shared by the quantize-on-write kernels (prefill pack,
// append + flush) and by the decode kernel's fused append: one 32-token page of one KV
// head, staged in LDS (as binary32, or as the bfloat16 values themselves), quantized by one
// workgroup of 256 threads.
//
// Keys are quantized per channel over the page's 32 tokens, values per token over groups
// of 32 channels, each group with an fp16 scale (max - min) / (2^bits - 1) and an fp16
// zero (the group minimum); codes round half to even and clamp.
//   [Mixed-precision KV-cache quantization per-layer sensitivity (llms-explorer.com), Facts]
//   [KVTuner OpenReview discussion (paperhub.cn/paper/zDwipF6h06), reply to reviewer 1,
//    section 4; reply to reviewer 2, section 2]
//
// Keys are per channel by default; in the per-token key mode they are grouped like the
// values (one group per token and 32 consecutive channels).
//   1. threads 0..127 each reduce one key group (a channel over the 32 tokens, or in the
//      per-token mode one (token, 32-channel group)), threads 128..255 each reduce one
//      (token, 32-channel group) of the values -- every thread owns exactly one group, so
//      the min/max needs no cross-thread reduction;
//   2. each thread encodes its own 32 values (binary32 subtract, the correctly rounded
//      quotient by the scale, round half to even, clamp) and writes the codes as bytes to
//      LDS;
//   3. all 256 threads pack the code bytes into the bit layout and store whole dwords.
#ifndef KVQ_CODEC_H
#define KVQ_CODEC_H

#include "kvq_device.h"

namespace kvq {

constexpr int kCodecThreads = 256;

// Element type of a staged tile: binary32, or the bits of a bfloat16 source staged as they
// are (every bfloat16 value is exactly a binary32 value, so the codec computes the same
// thing from either; the bfloat16 tile takes half the LDS, so twice as many workgroups fit
// on a CU).
template <typename T>
struct TileElem;

template <>
struct TileElem<float> {
    static constexpr int kStride = kHeadDim + 1;   // padded row: column walks hit distinct banks
    __device__ static float get(const float *p) { return *p; }
};

template <>
struct TileElem<uint16_t> {
    static constexpr int kStride = kHeadDim + 8;   // 272-byte rows: 16-byte aligned, 4 banks apart
    __device__ static float get(const uint16_t *p) { return __uint_as_float(static_cast<uint32_t>(*p) << 16); }
};

template <typename T>
struct QuantSmemT;

// binary32 tiles: with DEQUANT they are rewritten after the codes, so the codes keep their
// own space
template <>
struct QuantSmemT<float> {
    static constexpr int kStride = TileElem<float>::kStride;
    static constexpr bool kCodesOverTiles = false;
    float k[kGroup * kStride];               // [token][channel]
    float v[kGroup * kStride];
    uint8_t kcode[kGroup * kHeadDim];        // [token][channel]
    uint8_t vcode[kHeadDim * kGroup];        // [channel][token]
};

// bfloat16 tiles: every thread reads its group into registers before any code is written
// (a barrier apart), so the codes reuse the tiles' space
template <>
struct QuantSmemT<uint16_t> {
    static constexpr int kStride = TileElem<uint16_t>::kStride;
    static constexpr bool kCodesOverTiles = true;
    union {
        struct {
            alignas(16) uint16_t k[kGroup * kStride];
            alignas(16) uint16_t v[kGroup * kStride];
        };
        struct {
            uint8_t kcode[kGroup * kHeadDim];
            uint8_t vcode[kHeadDim * kGroup];
        };
    };
};

using QuantSmem = QuantSmemT<float>;
constexpr int kTileStride = QuantSmem::kStride;

// The 32 values of one group, `stride` elements apart, as binary32.
template <typename T>
__device__ __forceinline__ void load_group(const T *x, int stride, float (&v)[kGroup])
{
    if constexpr (sizeof(T) == 2) {
        if (stride == 1) {   // a row segment: four 16-byte reads
#pragma unroll
            for (int q = 0; q < kGroup / 8; ++q) {
                const uint4 u = *reinterpret_cast<const uint4 *>(__builtin_assume_aligned(x + 8 * q, 16));
                const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[8 * q + 2 * e] = __uint_as_float(w[e] << 16);
                    v[8 * q + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
                }
            }
            return;
        }
    }
#pragma unroll
    for (int i = 0; i < kGroup; ++i) v[i] = TileElem<T>::get(x + i * stride);
}

// Codec of one 32-value group held by one thread (its values v, read by load_group).
// Strict IEEE binary32: the compiler must not contract or reassociate anything in here.
// With DEQUANT the group's tile values x are replaced by their dequantized values
// code * s + z (binary32, one rounding).
template <int BITS, bool DEQUANT, typename T>
__device__ __forceinline__ void encode_group(const float (&v)[kGroup], T *x, int stride, uint32_t &sz_word,
                                             uint8_t *codes, int code_stride)
{
#pragma clang fp contract(off)
    static_assert(!DEQUANT || sizeof(T) == 4, "dequantized values are written back as binary32");
    // the values are finite, so the hardware min / max (v_min3 / v_max3 after contraction)
    // give the comparison-based extremes up to the sign of a zero; + 0 makes -0 into +0
    // (and that is all a -0 value changes: v - z and the codes are the same for +-0)
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int i = 1; i < kGroup; ++i) {
        mn = __builtin_fminf(mn, v[i]);
        mx = __builtin_fmaxf(mx, v[i]);
    }
    mn = mn + 0.0f;
    mx = mx + 0.0f;
    constexpr float levels = static_cast<float>((1 << BITS) - 1);
    const float s32 = (mx - mn) / levels;
    const uint16_t s16 = float_to_half_bits(s32);
    const uint16_t z16 = float_to_half_bits(mn);
    const float s = half_bits_to_float(s16);
    const float z = half_bits_to_float(z16);
    // The code is rne(q), q = (v - z) / s correctly rounded, clamped to [0, levels]; a zero
    // scale gives code 0.  For the finite scales of an fp16 word q comes from the
    // reciprocal: y = RN(1/s) is the hardware reciprocal (within 1 ulp) after one Newton
    // step (this holds for every significand that is not all ones, so for every fp16
    // value), q0 = RN(d y), and two corrections q <- q + (d - s q) y with exact residuals
    // make it RN(d / s) (Markstein's theorem for the second; the first only has to make q
    // faithful): five operations instead of the eleven of the general division, which
    // remains for non-finite s or z (outside the input domain).  With s = 0, y = 0 makes
    // every q 0.  tests/test_gpu_codec_scales.py packs groups at every finite fp16 scale,
    // with quotients at each half-integer and two ulps either side, at 2, 4 and 8 bits, and
    // matches the oracle's correctly rounded division byte for byte.
    float q[kGroup];
    if (__builtin_isfinite(s) && __builtin_isfinite(z)) {
        const float y0 = __builtin_amdgcn_rcpf(s);
        const float y = s != 0.0f ? __builtin_fmaf(__builtin_fmaf(-s, y0, 1.0f), y0, y0) : 0.0f;
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            const float d = v[i] - z;
            const float q0 = d * y;
            const float q1 = __builtin_fmaf(__builtin_fmaf(-s, q0, d), y, q0);
            q[i] = __builtin_fmaf(__builtin_fmaf(-s, q1, d), y, q1);
        }
    } else {
#pragma unroll
        for (int i = 0; i < kGroup; ++i) q[i] = s != 0.0f ? (v[i] - z) / s : 0.0f;
    }
    // rne and clamp in one add and one v_med3_f32: q + 2^23 rounds to the nearest integer
    // (ties to even) for 0 <= q < 2^23, anything below 2^23 clamps to code 0, and the code
    // is then the low bits of the result
    constexpr float kMagic = 8388608.0f;
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
        const float f = __builtin_amdgcn_fmed3f(q[i] + kMagic, kMagic, kMagic + levels);
        codes[i * code_stride] = static_cast<uint8_t>(__float_as_uint(f));
        if constexpr (DEQUANT) x[i * stride] = __builtin_fmaf(f - kMagic, s, z);
    }
    sz_word = static_cast<uint32_t>(s16) | (static_cast<uint32_t>(z16) << 16);
}

// Channel held by slot `slot` of chunk `a` (4*KB bytes) of a token row in the per-token
// key mode: each chunk holds channels 32J + 8a .. 32J + 8a + 7 of every key group J, the
// pair 32J + 8a + 2i, + 1 at the same position of the two 16-bit halves of one word --
// the order in which the decode kernel's matrix-core operands consume them.
template <int KB>
__device__ __forceinline__ int ktok_slot_channel(int a, int slot)
{
    constexpr int n = 16 / KB;
    const int x = slot / (2 * n), hh = (slot / n) % 2, p = slot % n;
    const int k = x * n + p;
    return 32 * (k / 4) + 8 * a + 2 * (k % 4) + hh;
}

// Quantize the staged tiles of one page-head into `dst` (global).  Every thread of the
// workgroup calls it (at least 256: threads 256 and up only take part in the barriers);
// with DEQUANT the tiles hold the dequantized values afterwards (valid after the
// workgroup's next barrier).  KTOK selects the per-token key mode.
template <int KB, int VB, bool DEQUANT = false, bool KTOK = false, typename T>
__device__ void quantize_page(QuantSmemT<T> &sm, uint8_t *__restrict__ dst)
{
    using P = PageLayout<KB, VB>;
    constexpr int kTileStride = QuantSmemT<T>::kStride;
    const int tid = threadIdx.x;
    uint32_t *dst32 = reinterpret_cast<uint32_t *>(dst);
    // the thread's group: threads 0..127 a key group (channel tid, or in the per-token mode
    // token tid % 32 and channels 32 (tid / 32) ..), threads 128..255 the value group of
    // token (tid - 128) % 32 and channels 32 ((tid - 128) / 32) ..
    const bool act = tid < kCodecThreads;
    const bool is_k = tid < kHeadDim;
    const int t = tid & (kGroup - 1), j = (tid & (kHeadDim - 1)) >> 5;
    float v[kGroup];
    if (!act) {
    } else if (is_k) {
        if constexpr (KTOK)
            load_group(&sm.k[t * kTileStride + kGroup * j], 1, v);
        else
            load_group(&sm.k[tid], kTileStride, v);
    } else {
        load_group(&sm.v[t * kTileStride + kGroup * j], 1, v);
    }
    if constexpr (QuantSmemT<T>::kCodesOverTiles) __syncthreads();   // the codes overwrite the tiles
    uint32_t w;
    if (!act) {
    } else if (is_k) {
        if constexpr (KTOK) {
            encode_group<KB, DEQUANT>(v, &sm.k[t * kTileStride + kGroup * j], 1, w, &sm.kcode[t * kHeadDim + kGroup * j], 1);
            dst32[P::kKSz / 4 + kValueGroups * t + j] = w;
        } else {
            encode_group<KB, DEQUANT>(v, &sm.k[tid], kTileStride, w, &sm.kcode[tid], kHeadDim);
            dst32[P::kKSz / 4 + tid] = w;
        }
    } else {
        encode_group<VB, DEQUANT>(v, &sm.v[t * kTileStride + kGroup * j], 1, w, &sm.vcode[(kGroup * j) * kGroup + t],
                                  kGroup);
        dst32[P::kVSz / 4 + kValueGroups * t + j] = w;
    }
    __syncthreads();
    // K codes: dword d of the section holds 32/KB slots of one token row (consecutive
    // channels, or in the per-token mode the channels of ktok_slot_channel)
    constexpr int kPerWord = 32 / KB;
    for (int d = tid; act && d < 128 * KB; d += kCodecThreads) {
        const int t = d / (4 * KB), dr = d % (4 * KB);
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < kPerWord; ++i) {
            int c;
            if constexpr (KTOK)
                c = ktok_slot_channel<KB>(dr / KB, (dr % KB) * kPerWord + i);
            else
                c = dr * kPerWord + i;
            w |= static_cast<uint32_t>(sm.kcode[t * kHeadDim + c]) << (i * KB);
        }
        dst32[P::kKCodes / 4 + d] = w;
    }
    // V codes: 64 chunks of 2*VB words; chunk 16q + r holds tokens 8q..8q+7 of channels
    // r, r+16, ..., r+112.  Word dw of a chunk holds, in each 16-bit half hh, the codes of
    // k = dw*n .. dw*n + n-1 (n = 16/VB), k = 4*(c/16) + (t%4), token t = 8q + (t%4) + 4hh.
    constexpr int n = 16 / VB;
    for (int d = tid; act && d < 128 * VB; d += kCodecThreads) {
        const int u = d / (2 * VB), dw = d % (2 * VB);
        const int q = u >> 4, r = u & 15;
        uint32_t w = 0;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
            for (int kk = 0; kk < n; ++kk) {
                const int k = dw * n + kk;
                const int t = 8 * q + (k & 3) + 4 * hh, c = 16 * (k >> 2) + r;
                w |= static_cast<uint32_t>(sm.vcode[c * kGroup + t]) << (16 * hh + VB * kk);
            }
        }
        dst32[P::kVCodes / 4 + d] = w;
    }
}

// ------------------------------------------------------------------------------------
// floating-point layer formats: FP8 (OCP E4M3) and BF16
// ------------------------------------------------------------------------------------
// A layer may store K and V as x / scale in E4M3 (one K and one V scale per KV head) or as
// bfloat16, instead of integer codes.  [When should you use mixed-precision KV caching to
// preserve accuracy in sensitive transformer layers (machinoai.in), sections 1-2]
// Head page: K token-major [32][128] elements, then V channel-major [128][32].
// Layer codes: how one layer's pages are stored.
constexpr int kLayerKeysPerChannel = 0, kLayerKeysPerToken = 1;   // integer codes, key mode
constexpr int kLayerFp8 = 2, kLayerBf16 = 3;                       // floating point

constexpr bool is_float_layer(int km) { return km == kLayerFp8 || km == kLayerBf16; }

template <int FMT>
struct FloatLayout {
    static constexpr int kElem = FMT == kLayerFp8 ? 1 : 2;            // bytes per element
    static constexpr int kV = kGroup * kHeadDim * kElem;              // V section offset
    static constexpr int kBytes = 2 * kV;
};

// bytes of one head page of a layer with bit widths (KB, VB) and layer code KM
template <int KB, int VB, int KM>
constexpr int layer_page_bytes()
{
    if constexpr (is_float_layer(KM))
        return FloatLayout<KM>::kBytes;
    else
        return PageLayout<KB, VB>::kBytes;
}

// E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits; no infinities; S.1111.111
// is NaN; largest finite 448.  Round to nearest even; finite values beyond 448 saturate.
// The hardware conversion (v_cvt_scalef32_pk_fp8_f32, scale 1) of the value clamped to
// [-448, 448] is exactly that rule -- checked against a direct implementation of the
// definition on every E4M3 value, every tie between neighbours, the saturation boundary,
// signed zeros and millions of random inputs -- so only NaN needs its own code.  Two
// values per call, as bytes 0 and 1 of the result.
typedef short kvq_short2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t e4m3_pair(float a, float b)
{
    const kvq_short2 zero = {0, 0};
    const uint32_t w = __builtin_bit_cast(
        uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(zero, fminf(fmaxf(a, -448.0f), 448.0f),
                                                           fminf(fmaxf(b, -448.0f), 448.0f), 1.0f, false));
    uint32_t lo = w & 0xFFu, hi = (w >> 8) & 0xFFu;
    if (a != a) lo = ((__float_as_uint(a) >> 24) & 0x80u) | 0x7Fu;
    if (b != b) hi = ((__float_as_uint(b) >> 24) & 0x80u) | 0x7Fu;
    return lo | (hi << 8);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t b)
{
    const int e = (b >> 3) & 15, m = b & 7;
    const float v = e ? ldexpf(static_cast<float>(8 + m), e - 10) : ldexpf(static_cast<float>(m), -9);
    return (b & 0x80u) ? -v : v;
}

// Convert the staged tiles of one page-head into `dst` (global) in format FMT.  Every thread
// calls it (threads 256 and up do nothing); every output dword is built from tile elements no other thread reads,
// so with DEQUANT the tiles are overwritten in place with the values the page stores
// (E4M3 value * scale, binary32), valid after the workgroup's next barrier.
template <int FMT, bool DEQUANT = false, typename T>
__device__ void quantize_page_float(QuantSmemT<T> &sm, uint8_t *__restrict__ dst, float ks, float vs)
{
#pragma clang fp contract(off)
    static_assert(!DEQUANT || sizeof(T) == 4, "dequantized values are written back as binary32");
    using FL = FloatLayout<FMT>;
    using E = TileElem<T>;
    constexpr int kTileStride = QuantSmemT<T>::kStride;
    const int tid = threadIdx.x;
    uint32_t *k32 = reinterpret_cast<uint32_t *>(dst);
    uint32_t *v32 = reinterpret_cast<uint32_t *>(dst + FL::kV);
    constexpr int kPer = 4 / FL::kElem;                                // elements per dword
    constexpr int kWords = kGroup * kHeadDim / kPer;
    for (int d = tid; tid < kCodecThreads && d < kWords; d += kCodecThreads) {
        // K: token-major
        {
            const int t = d / (kHeadDim / kPer), c0 = (d % (kHeadDim / kPer)) * kPer;
            T *x = &sm.k[t * kTileStride + c0];
            uint32_t w = 0;
            if constexpr (FMT == kLayerFp8) {
                w = e4m3_pair(E::get(x) / ks, E::get(x + 1) / ks) | (e4m3_pair(E::get(x + 2) / ks, E::get(x + 3) / ks) << 16);
                if constexpr (DEQUANT) {
#pragma unroll
                    for (int i = 0; i < kPer; ++i) x[i] = e4m3_to_f32((w >> (8 * i)) & 0xFFu) * ks;
                }
            } else {
#pragma unroll
                for (int i = 0; i < kPer; ++i) {
                    const uint32_t b = float_to_bf16_bits(E::get(x + i));
                    w |= b << (16 * i);
                    if constexpr (DEQUANT) x[i] = bf16_bits_to_float(static_cast<uint16_t>(b));
                }
            }
            k32[d] = w;
        }
        // V: channel-major
        {
            const int c = d / (kGroup / kPer), t0 = (d % (kGroup / kPer)) * kPer;
            T *x0 = &sm.v[t0 * kTileStride + c];
            uint32_t w = 0;
            if constexpr (FMT == kLayerFp8) {
                w = e4m3_pair(E::get(x0) / vs, E::get(x0 + kTileStride) / vs) |
                    (e4m3_pair(E::get(x0 + 2 * kTileStride) / vs, E::get(x0 + 3 * kTileStride) / vs) << 16);
                if constexpr (DEQUANT) {
#pragma unroll
                    for (int i = 0; i < kPer; ++i) x0[i * kTileStride] = e4m3_to_f32((w >> (8 * i)) & 0xFFu) * vs;
                }
            } else {
#pragma unroll
                for (int i = 0; i < kPer; ++i) {
                    const uint32_t b = float_to_bf16_bits(E::get(x0 + i * kTileStride));
                    w |= b << (16 * i);
                    if constexpr (DEQUANT) x0[i * kTileStride] = bf16_bits_to_float(static_cast<uint16_t>(b));
                }
            }
            v32[d] = w;
        }
    }
}

}  // namespace kvq

#endif  // KVQ_CODEC_H
