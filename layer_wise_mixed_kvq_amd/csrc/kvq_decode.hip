// kvq_decode.hip -- single-token decode attention over the packed mixed-precision cache
// for gfx950: both dot products on MFMA (v_mfma_f32_16x16x32_f16), split-K over 32-token
// pages with an online-softmax combine.
//
// Method: attention over the dequantized cache, FlashAttention-compatible (online
// softmax), with GQA (query head hq reads KV head hq / G); attention is memory-bound, so
// time follows the KV bytes moved.
//   [KVTuner OpenReview discussion (paperhub.cn/paper/zDwipF6h06), reply to reviewer 2,
//    section 1 "Efficiency evaluation clarifications"; reply to reviewer 3, section 2
//    "Latency experiment"; reply to reviewer 3, section 6 "MHA"]
//
// Dequantization is never done element by element.  The per-channel key scale is folded
// into q and the per-token value scale into the softmax weights, so the matrix cores see
// the raw integer codes:
//   score(t) = sum_c q_c (k_tc s_c + z_c) = sum_c (q_c s_c) k_tc + sum_c q_c z_c
//   out(c)   = sum_t p_t (v_tc s_tg + z_tg) = sum_t (p_t s_tg) v_tc + sum_t p_t z_tg
// Codes are unpacked into exact normal fp16 integers: 2- and 4-bit codes by the FP4 / FP8
// conversion instructions (one instruction per pair), 8-bit codes by a bit-insert into
// 1024.0 and a packed subtract.  The matrix cores accumulate subnormal fp16 operands
// several bits less accurately, which the scores (a small difference of two large sums)
// and the value sums do not tolerate.  The folded operands (q s and p s) are split into
// fp16 hi + lo parts (22 significant bits) and both parts meet the same code operand (in
// one MFMA, as different rows, when the head slots leave room).  Both are scaled by powers
// of two so their largest values sit just below
// 2^15: q s per page (from the page's largest key scale), p s per wave (from the largest
// value scale seen so far, p <= 1).  That keeps the lo parts in the normal fp16 range, where
// the matrix cores accumulate at full binary32 accuracy.
//
// Work decomposition.  One workgroup of NW waves (eight when the launch fits one workgroup
// per CU, else four) per (split, KV head, sequence).  Split s covers pages
// [s*P, min((s+1)*P, full)), dealt to its waves in weighted rounds (split_page).  A wave
// keeps its own online-softmax state; the waves are merged in LDS, and every split writes
// (m, l, o[128]) per query head to the workspace.  Split 0 also attends over the residual
// tokens (wave 0, from registers, before its page loop).  The last split of a (sequence,
// KV head) to finish -- a device-scope counter -- merges everything:
//   m = max m_s, l = sum 2^(m_s - m) l_s, out = sum 2^(m_s - m) o_s / l, lse = (m + log2 l) ln 2
// and resets the counter for the next call.  Scores are in log2 units (q carries
// log2(e)/sqrt(128)).
//
// MFMA roles (16x16x32, wave64).  Row r of an A operand / D tile holds query head
// 4*(r % 4) + r / 4, so head h sits in lane group h % 4 (lanes 16*(h%4) ..) and element
// h / 4 of the accumulator: with G <= 4 every lane holds exactly one head per token.
//   scores:  D[head][token]   = A(q s hi|lo, from LDS)    x B(key codes, token-major rows)
//   values:  D[head][channel] = A(p s hi|lo, from LDS)    x B(value codes, chunk layout)
// With G <= 8 the hi and lo parts occupy different rows of one A operand (parts x head
// slots <= 16), so one MFMA per B operand forms both and the parts are summed afterwards.
// Integer layers: score column r of blocks 0 and 1 holds not tokens r and 16 + r but the
// two tokens (t0, t1) whose products lane r of each lane group packs into one A-operand
// word of the values, so a lane folds its own softmax weights into all four value groups'
// A operands and only that write goes through LDS.
//
// Floating-point layers (FP8 E4M3 with one K and one V scale per KV head, or BF16) hold
// the values themselves, so nothing is folded per page: the scales multiply the scores
// and the output once.  FP8 bytes convert exactly to normal fp16 values (v_cvt_scalef32_
// pk_f16_fp8 at scale 1) and meet the same fp16 hi|lo A operands; BF16 pages go to the
// bf16 matrix-core instruction with A split into three bf16 parts (24 significant bits).
// The contraction order inside one MFMA is free, so each lane takes 32 consecutive
// channels of a token row (one or two 16-byte loads) and A is laid out to match.
//   [When should you use mixed-precision KV caching to preserve accuracy in sensitive
//    transformer layers (machinoai.in), sections 1-2]
#include "kvq_codec.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

// Waves per workgroup (NW): eight, one workgroup filling a CU, so that the CU's waves all
// work on one split of one (sequence, KV head) and run out of pages together, when every
// workgroup of the launch is resident at once (at most one per CU) and two waves per SIMD
// fit (G <= 8); four otherwise, two workgroups per CU, so that one's merge and combine
// overlap the other's pages.  decode_waves_for() is the host's choice.
constexpr int kMaxWaves = 8;
[[maybe_unused]] constexpr int kMaxGS = 4;                   // head slots per lane group: G <= 16
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kScoreScale = 1.4426950408889634f * 0.08838834764831845f;   // log2(e)/sqrt(128)

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float4_t mfma(const uint4 &a, const uint4 &b, const float4_t &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float4_t mfma_bf16(const uint4 &a, const uint4 &b, const float4_t &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
}

// Eight E4M3 bytes (two words, byte i = element i) as eight fp16 values: exact, since every
// E4M3 value is zero or a normal fp16 value.
__device__ __forceinline__ uint4 fp8x8_to_f16(uint32_t w0, uint32_t w1)
{
    const half2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
    const half2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
    const half2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
    const half2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
    return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
                      __builtin_bit_cast(uint32_t, d));
}

// hi / lo split of two products x0*y0, x1*y1 into packed fp16 pairs with hi + lo equal to
// the exact products to about 22 bits.  The residual is formed from the very bits stored
// as hi (one fma of the exact product minus hi), so the two halves can never disagree on
// how a rounding tie went: an inline-asm barrier keeps the compiler from recomputing hi
// with a differently rounded fused instruction for the residual.
__device__ __forceinline__ uint32_t split_hi(float a0, float a1)
{
    uint32_t h = __builtin_bit_cast(uint32_t, half2_t{static_cast<_Float16>(a0), static_cast<_Float16>(a1)});
    __asm__ volatile("" : "+v"(h));
    return h;
}

__device__ __forceinline__ uint32_t split_lo(float x0, float y0, float x1, float y1, uint32_t hi)
{
    const float r0 = fmaf(x0, y0, -half_bits_to_float(hi & 0xFFFFu));
    const float r1 = fmaf(x1, y1, -half_bits_to_float(hi >> 16));
    return __builtin_bit_cast(uint32_t, half2_t{static_cast<_Float16>(r0), static_cast<_Float16>(r1)});
}

// Two values as a packed bf16 pair (round to nearest even) and the residuals x - bf16(x),
// exact in binary32.  Three such steps give hi + mid + lo equal to x to 24 bits.
__device__ __forceinline__ uint32_t bf16_pair(float x0, float x1, float &r0, float &r1)
{
    uint32_t h = __builtin_bit_cast(uint32_t, bf16x2_t{static_cast<__bf16>(x0), static_cast<__bf16>(x1)});
    __asm__ volatile("" : "+v"(h));
    r0 = x0 - __uint_as_float(h << 16);
    r1 = x1 - __uint_as_float(h & 0xFFFF0000u);
    return h;
}

__device__ __forceinline__ void split3_bf16(float x0, float x1, uint32_t &hi, uint32_t &mid, uint32_t &lo)
{
    float r0, r1, e0, e1;
    hi = bf16_pair(x0, x1, r0, r1);
    mid = bf16_pair(r0, r1, e0, e1);
    lo = bf16_pair(e0, e1, r0, r1);
}

// hi / lo split of two products a0 * s0, a1 * s1 with s0, s1 the fp16 in the low halves of
// w0, w1: each product is formed from the fp16 operand directly by a mixed-precision
// multiply-add (no conversion of s, no separate product), and lo from the very bits stored
// as hi, as in split_hi / split_lo.
__device__ __forceinline__ _Float16 lo_half(uint32_t w) { return __builtin_bit_cast(half2_t, w)[0]; }
__device__ __forceinline__ _Float16 hi_half(uint32_t w) { return __builtin_bit_cast(half2_t, w)[1]; }

__device__ __forceinline__ uint32_t fold_hi(float a0, float a1, uint32_t w0, uint32_t w1)
{
    const _Float16 x0 = static_cast<_Float16>(__builtin_fmaf(a0, static_cast<float>(lo_half(w0)), 0.0f));
    const _Float16 x1 = static_cast<_Float16>(__builtin_fmaf(a1, static_cast<float>(lo_half(w1)), 0.0f));
    uint32_t h = __builtin_bit_cast(uint32_t, half2_t{x0, x1});
    __asm__ volatile("" : "+v"(h));
    return h;
}

__device__ __forceinline__ uint32_t fold_lo(float a0, float a1, uint32_t w0, uint32_t w1, uint32_t hi)
{
    const float r0 = __builtin_fmaf(a0, static_cast<float>(lo_half(w0)), -static_cast<float>(lo_half(hi)));
    const float r1 = __builtin_fmaf(a1, static_cast<float>(lo_half(w1)), -static_cast<float>(hi_half(hi)));
    return __builtin_bit_cast(uint32_t, half2_t{static_cast<_Float16>(r0), static_cast<_Float16>(r1)});
}

// fp16 bits of 2^k, clamped to [smallest subnormal, infinity]: a threshold for fp16 scale
// words (non-negative, so they order as unsigned integers)
__device__ __forceinline__ uint32_t fp16_pow2_bits(int k)
{
    if (k > 15) return 0x7C00u;
    if (k >= -14) return static_cast<uint32_t>(k + 15) << 10;
    if (k >= -24) return 1u << (k + 24);
    return 1u;
}

// LDS ordering inside one wave: the LDS executes one wave's DS instructions in issue
// order, so a read issued after a write of the same wave returns the written data without
// waiting for the write to complete.  Only the compiler must keep the order: the barrier
// stops it from moving LDS accesses across this point (the normal waits on read results
// are still inserted where the data is used).
__device__ __forceinline__ void wave_lds_sync()
{
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_wave_barrier();
}

// Reductions over the 16 lanes of a lane group with DPP (no LDS round trip): xor 1 and
// xor 2 via quad permutes, then row_half_mirror and row_mirror fold the quads and the two
// halves; every lane of the group ends with the result.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v)
{
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xF, 0xF, true));
}
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kRowHalfMirror = 0x141, kRowMirror = 0x140;

__device__ __forceinline__ float fdpp1(float v) { return __uint_as_float(dpp<kQuadXor1>(__float_as_uint(v))); }
__device__ __forceinline__ float fdpp2(float v) { return __uint_as_float(dpp<kQuadXor2>(__float_as_uint(v))); }
__device__ __forceinline__ float fdpp3(float v) { return __uint_as_float(dpp<kRowHalfMirror>(__float_as_uint(v))); }
__device__ __forceinline__ float fdpp4(float v) { return __uint_as_float(dpp<kRowMirror>(__float_as_uint(v))); }

__device__ __forceinline__ float row_max(float v)
{
    v = fmaxf(v, fdpp1(v));
    v = fmaxf(v, fdpp2(v));
    v = fmaxf(v, fdpp3(v));
    return fmaxf(v, fdpp4(v));
}

__device__ __forceinline__ float row_sum(float v)
{
    v += fdpp1(v);
    v += fdpp2(v);
    v += fdpp3(v);
    return v + fdpp4(v);
}

__device__ __forceinline__ uint32_t row_max_u32(uint32_t v)
{
    v = max(v, dpp<kQuadXor1>(v));
    v = max(v, dpp<kQuadXor2>(v));
    v = max(v, dpp<kRowHalfMirror>(v));
    return max(v, dpp<kRowMirror>(v));
}

template <typename QT>
__device__ __forceinline__ float load_q(const void *q, long long i);
template <>
__device__ __forceinline__ float load_q<uint16_t>(const void *q, long long i)
{
    return bf16_bits_to_float(static_cast<const uint16_t *>(q)[i]);
}
template <>
__device__ __forceinline__ float load_q<float>(const void *q, long long i)
{
    return static_cast<const float *>(q)[i];
}

// eight consecutive q elements from element i (a multiple of 8): one 16-byte load for bf16,
// two for binary32
template <typename QT>
__device__ __forceinline__ void load_q8(const void *q, long long i, float (&out)[8]);
template <>
__device__ __forceinline__ void load_q8<uint16_t>(const void *q, long long i, float (&out)[8])
{
    const uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(q) + i);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        out[2 * k] = __uint_as_float(u[k] << 16);
        out[2 * k + 1] = __uint_as_float(u[k] & 0xFFFF0000u);
    }
}
template <>
__device__ __forceinline__ void load_q8<float>(const void *q, long long i, float (&out)[8])
{
    const float4 x = *reinterpret_cast<const float4 *>(static_cast<const float *>(q) + i);
    const float4 y = *reinterpret_cast<const float4 *>(static_cast<const float *>(q) + i + 4);
    out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
    out[4] = y.x; out[5] = y.y; out[6] = y.z; out[7] = y.w;
}

// 1024.0 in both fp16 halves, opaque to the optimizer so that the unpack below stays one
// bit-field insert (v_bfi_b32) instead of a constant-folded and + or.  The empty asm emits
// no instruction: the register is written by an ordinary compiler-generated move.
__device__ __forceinline__ uint32_t fp16x2_1024()
{
    uint32_t m = 0x64006400u;
    __asm__ volatile("" : "+v"(m));
    return m;
}

// Pair j (0..3) of operand `op` from a lane's packed codes, as exact normal fp16 values:
// with n = 16/BITS codes per 16-bit half, k = 4*op + j sits in word k / n at position
// p = k % n in both halves.  The m = 8/BITS positions of a half's low byte are inserted
// in place into 1024.0 (0x6400: spacing 1, low ten bits zero); those of the high byte after
// one shift by 8 (shared by every pair of the word).  After one packed subtract of 1024 the
// pair is code * 2^unpack_shift<BITS>(j), exact; the power of two is divided out of the
// matching A-operand element.  The matrix cores keep full binary32 accuracy only for normal
// fp16 inputs: subnormal operands lose about four bits in the accumulation.
// No inline asm writes a register here: the hazard recognizer does not see registers an
// asm statement writes, and a register that is dead in an MFMA result can be reused while
// that MFMA is still in flight, which has to wait until the MFMA retires.
template <int BITS>
__device__ __forceinline__ constexpr int unpack_shift(int j)
{
    if constexpr (BITS != 8)
        return 0;     // 2- and 4-bit codes unpack exactly (below); not a code width (float layers)
    else
        return BITS * (j % (8 / BITS));
}

template <int BITS>
__device__ __forceinline__ uint4 unpack_codes(const uint32_t *w, int op, uint32_t magic)
{
    constexpr int n = 16 / BITS, m = 8 / BITS;
    constexpr uint32_t M = ((1u << BITS) - 1u) * 0x00010001u;
    const half2_t bias = {static_cast<_Float16>(-1024.0f), static_cast<_Float16>(-1024.0f)};
    uint32_t r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int k = 4 * op + j, p = k % n;
        const uint32_t x = p >= m ? w[k / n] >> 8 : w[k / n];
        const uint32_t Mp = M << (BITS * (p % m));
        const uint32_t y = (x & Mp) | (magic & ~Mp);
        r[j] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, y) + bias);
    }
    return make_uint4(r[0], r[1], r[2], r[3]);
}

// 2- and 4-bit codes through the hardware's small-float conversions.  A 4-bit code alone
// in a byte is the E4M3 value c * 2^-9 (subnormal below 8, normal from 8), and a 2-bit code
// alone in a nibble is the E2M1 value c / 2; a power-of-two scale of 2^9 or 2 turns either
// back into the integer c exactly (a normal fp16 value, or 0).  Two masks per word leave
// one code per byte (or nibble), and each conversion yields one fp16 pair.
//   4-bit, operand op = word op:    pairs (c0, c2), (c1, c3), (c4, c6), (c5, c7)
//   2-bit, operand op = word op/2, bytes b = op%2 and b + 2 of its two masked copies:
//                                   pairs (c[4b], c[4b+2]), (c[4b+1], c[4b+3]), then b + 2
// where c[i] is the code at bit BITS*i of the word.
template <int BITS>
__device__ __forceinline__ uint4 unpack_cvt(const uint32_t *w, int op)
{
    half2_t r[4];
    if constexpr (BITS == 4) {
        const uint32_t x = w[op];
        const uint32_t m0 = x & 0x0F0F0F0Fu, m1 = (x >> 4) & 0x0F0F0F0Fu;
        r[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(m0, 512.0f, false);
        r[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(m1, 512.0f, false);
        r[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(m0, 512.0f, true);
        r[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(m1, 512.0f, true);
    } else {
        static_assert(BITS == 2, "2- or 4-bit codes");
        const uint32_t x = w[op >> 1];
        const uint32_t m0 = x & 0x33333333u, m1 = (x >> 2) & 0x33333333u;
        if (op & 1) {
            r[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m0, 2.0f, 1);
            r[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m1, 2.0f, 1);
            r[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m0, 2.0f, 3);
            r[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m1, 2.0f, 3);
        } else {
            r[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m0, 2.0f, 0);
            r[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m1, 2.0f, 0);
            r[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m0, 2.0f, 2);
            r[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m1, 2.0f, 2);
        }
    }
    return make_uint4(__builtin_bit_cast(uint32_t, r[0]), __builtin_bit_cast(uint32_t, r[1]),
                      __builtin_bit_cast(uint32_t, r[2]), __builtin_bit_cast(uint32_t, r[3]));
}

// B operand `op` of a lane's packed codes: conversions for 2 and 4 bits, the 1024.0 insert
// for 8 bits
template <int BITS>
__device__ __forceinline__ uint4 unpack_b(const uint32_t *w, int op, uint32_t magic)
{
    if constexpr (BITS == 8)
        return unpack_codes<BITS>(w, op, magic);
    else
        return unpack_cvt<BITS>(w, op);
}

// Channel (within a lane's 32-channel k-group) of the first code of pair j of key operand
// jj (per-channel keys); the second code is key_pair_step<KB>() channels further.
template <int KB>
__device__ __forceinline__ int key_pair_channel(int jj, int j)
{
    if constexpr (KB == 4) {
        return 8 * jj + 4 * (j >> 1) + (j & 1);
    } else if constexpr (KB == 2) {
        return 16 * (jj >> 1) + 4 * (jj & 1) + 8 * (j >> 1) + (j & 1);
    } else {
        constexpr int n = 16 / KB, nd = 32 / KB;
        const int k = 4 * jj + j;
        return nd * (k / n) + (k % n);
    }
}

template <int KB>
__device__ __forceinline__ constexpr int key_pair_step()
{
    return KB == 8 ? 16 / KB : 2;
}

// A-operand parts: fp16 hi | lo, or bf16 hi | mid | lo for BF16 layers
constexpr int a_parts(int km) { return km == kLayerBf16 ? 3 : 2; }

template <int GS, int KM>
struct WaveLds {
    static constexpr int NP = a_parts(KM);
    static constexpr int PG = is_float_layer(KM) ? 1 : 4;   // value groups with their own scales
    // rows padded by 4 words so that the 128-bit A-operand reads of different head rows
    // fall into different LDS banks
    alignas(16) uint32_t qp[NP][4 * GS + 1][68];     // (q s) parts: [part][head, + zero row][pair]
    // (p s) parts, one block per value group: [part][head, + zero row][pair]
    static constexpr int kPPBlock = NP * (4 * GS + 1) * 20;
    alignas(16) uint32_t pp[PG][kPPBlock];
    alignas(16) float p[4 * GS][48];                 // FP8 / BF16 layers: the page's softmax weights, [head][token];
                                                     // before the page loop: the residual tokens' weights
    float bv[4][4 * GS];                             // value zero terms at the end: [group][head]
    __device__ uint32_t *pp_row(int g, int part, int row) { return &pp[g][(part * (4 * GS + 1) + row) * 20]; }
};

template <int GS, int NW>
struct MergeLds {
    float o[NW][4 * GS][kHeadDim + 16];   // head rows 16 mod 64 words apart: the lane groups' writes miss each other's banks
    float m[NW][4 * GS];
    float l[NW][4 * GS];
};

template <int GS>
struct ResidualLds {              // staging of the residual tokens (page-codec layout)
    QuantSmem q;
    float s[4 * GS][kGroup];
};

template <int GS>
struct ResidualOut {              // (m, l, o) of the residual tokens, kept for the merge
    alignas(16) float o[4 * GS][kHeadDim];
    float m[4 * GS];
    float l[4 * GS];
};

template <int GS, int KM, int NW>
struct DecodeSmem {
    alignas(16) float qs[4 * GS][kHeadDim];   // q * log2(e)/sqrt(128), for the residual tokens
    ResidualOut<GS> ro;
    union {
        WaveLds<GS, KM> w[NW];
        MergeLds<GS, NW> merge;
        ResidualLds<GS> res;
    } u;
    int last;
    int early;
    int bad;                      // some wave saw a page id outside the pool
};

#if defined(KVQ_PHASE_TIMERS)
// Profiling build only: lane 0 of each wave records the 100 MHz real-time counter at the
// kernel's phase boundaries (record layout beside kPhaseStamps in kvq_internal.h).
__device__ __forceinline__ void phase_stamp(const DecodeParams &p, int k)
{
    if (p.phase_ts && (threadIdx.x & 63) == 0) {
        const long long wg = blockIdx.x + static_cast<long long>(gridDim.x) * (blockIdx.y + static_cast<long long>(gridDim.y) * blockIdx.z);
        unsigned long long *r = p.phase_ts + (wg * kMaxWaves + (threadIdx.x >> 6)) * kPhaseStamps;
        r[k] = __builtin_amdgcn_s_memrealtime();
        if (k == 0) {
            // HW_REG_HW_ID (id 4) and HW_REG_XCC_ID (id 20), all 32 bits
            const unsigned hw = static_cast<unsigned>(__builtin_amdgcn_s_getreg(4 | (31 << 11)));
            const unsigned xcc = static_cast<unsigned>(__builtin_amdgcn_s_getreg(20 | (31 << 11)));
            r[6] = (static_cast<unsigned long long>(xcc & 0xFu) << 32) | hw;
            r[7] = static_cast<unsigned long long>(blockIdx.x) | (static_cast<unsigned long long>(blockIdx.y) << 20) |
                   (static_cast<unsigned long long>(blockIdx.z) << 40);
        }
    }
}
#define KVQ_STAMP(k) phase_stamp(p, k)
#else
#define KVQ_STAMP(k) ((void)0)
#endif

__device__ __forceinline__ uint4 lds_read16(const uint32_t *p)
{
    return *reinterpret_cast<const uint4 *>(__builtin_assume_aligned(p, 16));
}

// Split partials cross workgroups (and XCDs, whose L2s are not coherent with each other),
// so they are written and read with device-scope relaxed atomics (sc1 stores / loads,
// coherent without flushing any cache); each thread waits for its stores to land before
// the workgroup bumps the counter.
__device__ __forceinline__ void store_dev(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_dev(const float *p)
{
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Position of channel c inside a head's 128 split-partial outputs: (c % 4) * 32 + c / 4,
// so that a thread's 4 consecutive channels go out as 4 stores of consecutive addresses.
__device__ __forceinline__ int part_slot(int c)
{
    return (c % 4) * (kHeadDim / 4) + c / 4;
}

__device__ __forceinline__ void wait_stores()
{
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ------------------------------------------------------------------------------------
// residual tokens (bf16): (m, l, o) per head into LDS
// ------------------------------------------------------------------------------------
// With a flush split 0's workgroup attends them after its page loop.  The whole 32 x 128
// tile is requested right after the first page, in 16-byte chunks, chunk i = tid, tid + NT,
// ... (token i / 16, channels 8 (i % 16) .. +7), and with the fused append the chunk of the
// new token at the same channels.
template <int NT>
__device__ __forceinline__ void load_residual(const DecodeParams &p, long long bh, bool append,
                                              uint4 (&kv)[4 * (512 / NT)])
{
    constexpr int KC = 512 / NT;
    const uint4 *rk = reinterpret_cast<const uint4 *>(p.resid_k + bh * kGroup * kHeadDim);
    const uint4 *rv = reinterpret_cast<const uint4 *>(p.resid_v + bh * kGroup * kHeadDim);
    const uint4 *nk = reinterpret_cast<const uint4 *>((append ? p.k_new : p.resid_k) + bh * kHeadDim);
    const uint4 *nv = reinterpret_cast<const uint4 *>((append ? p.v_new : p.resid_v) + bh * kHeadDim);
#pragma unroll
    for (int k = 0; k < KC; ++k) {
        const int i = threadIdx.x + k * NT, col = i % (kHeadDim / 8);
        kv[k] = rk[i];
        kv[KC + k] = rv[i];
        kv[2 * KC + k] = nk[col];
        kv[3 * KC + k] = nv[col];
    }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Without a flush (at most 31 tokens) wave 0 of split 0 attends the residual tokens before
// its page loop, from registers, with no barrier.  Lane roles:
//   keys:   token t = lane % 32, channels 64 (lane / 32) .. +63 (eight 16-byte loads)
//   values: channels 2 lane, 2 lane + 1 of every token (one 4-byte load per token)
// Rows past nres - 1 reload row nres - 1 (the same addresses: cache hits) and are masked.
// With the fused append the last row (nres - 1) is the new token, read from k_new / v_new.
struct ResidualWaveRegs {
    uint4 k[8];
    uint32_t v[kGroup];
};

__device__ __forceinline__ void load_residual_wave(const DecodeParams &p, long long bh, int nres, bool append,
                                                   ResidualWaveRegs &r)
{
    const int lane = threadIdx.x & 63;
    const int t = min(lane & 31, nres - 1), half = lane >> 5;
    const uint16_t *krow = append && t == nres - 1 ? p.k_new + bh * kHeadDim
                                                   : p.resid_k + (bh * kGroup + t) * kHeadDim;
    const uint4 *k4 = reinterpret_cast<const uint4 *>(krow + 64 * half);
#pragma unroll
    for (int i = 0; i < 8; ++i) r.k[i] = k4[i];
#pragma unroll
    for (int tt = 0; tt < kGroup; ++tt) {
        const int row = min(tt, nres - 1);
        const uint16_t *vrow = append && row == nres - 1 ? p.v_new + bh * kHeadDim
                                                         : p.resid_v + (bh * kGroup + row) * kHeadDim;
        r.v[tt] = reinterpret_cast<const uint32_t *>(vrow)[lane];
    }
}

// The wave's residual attention into sm.ro: scores against q~ (sm.qs, which this wave
// wrote), softmax over the nres tokens, values weighted through the wave's own WaveLds::p;
// the fused append also stores the new token into its residual slot.
template <int GS, int KM, int NW>
__device__ void residual_wave(const DecodeParams &p, DecodeSmem<GS, KM, NW> &sm, WaveLds<GS, KM> &W,
                              const ResidualWaveRegs &r, int nres, int G, long long bh, bool append)
{
    constexpr int HS = 4 * GS;
    const int lane = threadIdx.x & 63, t = lane & 31, half = lane >> 5;
    KVQ_STAMP(12);
    if (append) {
        const long long row = (bh * kGroup + (nres - 1)) * kHeadDim;
        if (t == nres - 1) {
            uint4 *dk = reinterpret_cast<uint4 *>(p.resid_k + row + 64 * half);
#pragma unroll
            for (int i = 0; i < 8; ++i) dk[i] = r.k[i];
        }
#pragma unroll
        for (int tt = 0; tt < kGroup; ++tt)
            if (tt == nres - 1) reinterpret_cast<uint32_t *>(p.resid_v + row)[lane] = r.v[tt];
    }
    const bool live = t < nres;
    // scores of every head (independent chains): each 8-channel chunk of the key row is
    // widened once and used by every head, then the softmax of each head
    float sc[HS];
#pragma unroll
    for (int h = 0; h < HS; ++h) sc[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint4 kw = r.k[i];
        const float kf[8] = {bf16_lo(kw.x), bf16_hi(kw.x), bf16_lo(kw.y), bf16_hi(kw.y),
                             bf16_lo(kw.z), bf16_hi(kw.z), bf16_lo(kw.w), bf16_hi(kw.w)};
#pragma unroll
        for (int h = 0; h < HS; ++h) {
            if (h >= G) break;
            const float4 *qrow = reinterpret_cast<const float4 *>(&sm.qs[h][64 * half + 8 * i]);
            const float4 qa = qrow[0], qb = qrow[1];
            float acc = sc[h];
            acc = fmaf(qa.x, kf[0], acc);
            acc = fmaf(qa.y, kf[1], acc);
            acc = fmaf(qa.z, kf[2], acc);
            acc = fmaf(qa.w, kf[3], acc);
            acc = fmaf(qb.x, kf[4], acc);
            acc = fmaf(qb.y, kf[5], acc);
            acc = fmaf(qb.z, kf[6], acc);
            acc = fmaf(qb.w, kf[7], acc);
            sc[h] = acc;
        }
    }
#pragma unroll
    for (int h = 0; h < HS; ++h) {
        if (h >= G) continue;
        const float acc = sc[h] + __shfl_xor(sc[h], 32);
        const float x = live ? acc : -INFINITY;
        // tokens 0-15 are lane group 0, tokens 16-31 lane group 1 (groups 2, 3 repeat them)
        const float mr = row_max(x);
        const float m = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(mr), 0)),
                              __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mr), 16)));
        const float e = live ? __builtin_amdgcn_exp2f(x - m) : 0.0f;
        const float er = row_sum(e);
        const float l = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(er), 0)) +
                        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(er), 16));
        if (half == 0) W.p[h][t] = e;
        if (lane == 0) {
            sm.ro.m[h] = m;
            sm.ro.l[h] = l;
        }
    }
    wave_lds_sync();
#pragma unroll
    for (int h = 0; h < HS; ++h) {
        if (h >= G) continue;
        const float4 *ep = reinterpret_cast<const float4 *>(&W.p[h][0]);
        float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
        for (int q4 = 0; q4 < kGroup / 4; ++q4) {
            const float4 e4 = ep[q4];
            const float ev[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t v = r.v[4 * q4 + u];
                o0 = fmaf(ev[u], bf16_lo(v), o0);
                o1 = fmaf(ev[u], bf16_hi(v), o1);
            }
        }
        *reinterpret_cast<float2 *>(&sm.ro.o[h][2 * lane]) = make_float2(o0, o1);
    }
    KVQ_STAMP(13);
}

// The residual tokens' attention by the whole workgroup (every thread calls it; used when
// the fused append completes a group, and written for a tile without a flush as well):
//   1. V (and, with a flush, K) staged in LDS as binary32; the fused append's new token
//      stored into its residual slot;
//   2. flush: the 32 rows quantized into their page `flush_page` (same codec and bytes as
//      kvq_append) and the tiles replaced by their dequantized values;
//   3. scores: thread (token i / 16, channels 8 (i % 16) ..) against q~ (sm.qs), summed over
//      the token's 16 lanes;
//   4. softmax: one wave per head;
//   5. values: thread (head, channel), a sum over the tokens in token order.
// Returns false if the flush page id is outside the pool.
template <int KB, int VB, int GS, int KM, int NW, int NT = 64 * NW>
__device__ bool residual_wg(const DecodeParams &p, DecodeSmem<GS, KM, NW> &sm, const uint4 (&kv_in)[4 * (512 / NT)],
                            int nres, int G, long long bh, bool append, bool flush, int flush_page)
{
    constexpr int KC = 512 / NT;
    ResidualLds<GS> &R = sm.u.res;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    KVQ_STAMP(12);
    // the chunks of the attended tokens: the new token's in row nres - 1 (fused append)
    uint4 kv[2 * KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
        const int row = (tid + k * NT) / (kHeadDim / 8);
        const bool fresh = append && row == nres - 1;
        kv[k] = fresh ? kv_in[2 * KC + k] : kv_in[k];
        kv[KC + k] = fresh ? kv_in[3 * KC + k] : kv_in[KC + k];
    }
#pragma unroll
    for (int k = 0; k < KC; ++k) {
        const int i = tid + k * NT, row = i / (kHeadDim / 8), col = 8 * (i % (kHeadDim / 8));
        const uint32_t kw[4] = {kv[k].x, kv[k].y, kv[k].z, kv[k].w};
        const uint32_t vw[4] = {kv[KC + k].x, kv[KC + k].y, kv[KC + k].z, kv[KC + k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (flush) {
                R.q.k[row * kTileStride + col + 2 * e] = bf16_lo(kw[e]);
                R.q.k[row * kTileStride + col + 2 * e + 1] = bf16_hi(kw[e]);
            }
            R.q.v[row * kTileStride + col + 2 * e] = bf16_lo(vw[e]);
            R.q.v[row * kTileStride + col + 2 * e + 1] = bf16_hi(vw[e]);
        }
        if (append && row == nres - 1) {
            reinterpret_cast<uint4 *>(p.resid_k + bh * kGroup * kHeadDim)[i] = kv[k];
            reinterpret_cast<uint4 *>(p.resid_v + bh * kGroup * kHeadDim)[i] = kv[KC + k];
        }
    }
    __syncthreads();
    bool ok = true;
    if (flush) {
        const int b = static_cast<int>(bh / p.H), h = static_cast<int>(bh % p.H);
        const int phys = p.block_table[static_cast<long long>(b) * p.max_pages + flush_page];
        ok = phys >= 0 && phys < p.n_pages;
        if (ok) {
            uint8_t *dst = static_cast<uint8_t *>(p.pages) +
                           (static_cast<long long>(phys) * p.H + h) * layer_page_bytes<KB, VB, KM>();
            if constexpr (is_float_layer(KM))
                quantize_page_float<KM, true>(R.q, dst, p.scales ? p.scales[2 * h] : 1.0f,
                                              p.scales ? p.scales[2 * h + 1] : 1.0f);
            else
                quantize_page<KB, VB, true, KM == kLayerKeysPerToken>(R.q, dst);
        }
        __syncthreads();
    }
    // scores
#pragma unroll
    for (int k = 0; k < KC; ++k) {
        const int i = tid + k * NT, t = i / (kHeadDim / 8), part = i % (kHeadDim / 8);
        float kf[8];
        if (flush) {
#pragma unroll
            for (int e = 0; e < 8; ++e) kf[e] = R.q.k[t * kTileStride + 8 * part + e];
        } else {
            const uint32_t kw[4] = {kv[k].x, kv[k].y, kv[k].z, kv[k].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kf[2 * e] = bf16_lo(kw[e]);
                kf[2 * e + 1] = bf16_hi(kw[e]);
            }
        }
        for (int h = 0; h < G; ++h) {
            const float4 qa = *reinterpret_cast<const float4 *>(&sm.qs[h][8 * part]);
            const float4 qb = *reinterpret_cast<const float4 *>(&sm.qs[h][8 * part + 4]);
            float s = qa.x * kf[0];
            s = fmaf(qa.y, kf[1], s);
            s = fmaf(qa.z, kf[2], s);
            s = fmaf(qa.w, kf[3], s);
            s = fmaf(qb.x, kf[4], s);
            s = fmaf(qb.y, kf[5], s);
            s = fmaf(qb.z, kf[6], s);
            s = fmaf(qb.w, kf[7], s);
            s = row_sum(s);                       // the token's 16 lanes
            if (part == 0) R.s[h][t] = t < nres ? s : -INFINITY;
        }
    }
    __syncthreads();
    // softmax over the tokens, one wave per head: lane t < 32 holds token t
    for (int h = wave; h < G; h += NW) {
        const float x = lane < kGroup ? R.s[h][lane] : -INFINITY;
        const float mr = row_max(x);
        const float m = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(mr), 0)),
                              __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mr), 16)));
        const float e = lane < nres ? __builtin_amdgcn_exp2f(x - m) : 0.0f;
        const float er = row_sum(e);
        const float l = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(er), 0)) +
                        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(er), 16));
        if (lane < kGroup) R.s[h][lane] = e;
        if (lane == 0) {
            sm.ro.m[h] = m;
            sm.ro.l[h] = l;
        }
    }
    __syncthreads();
    for (int idx = tid; idx < G * kHeadDim; idx += NT) {
        const int h = idx / kHeadDim, c = idx % kHeadDim;
        float o = 0.0f;
        for (int t = 0; t < nres; ++t) o = fmaf(R.s[h][t], R.q.v[t * kTileStride + c], o);
        sm.ro.o[h][c] = o;
    }
    __syncthreads();     // the page loop reuses the space
    KVQ_STAMP(13);
    return ok;
}

// ------------------------------------------------------------------------------------
// the page work of one wave
// ------------------------------------------------------------------------------------
template <int KB, int VB>
struct PageRegs {
    uint32_t kc[2][KB];      // key codes of token t0 (blk 0) / t1 (blk 1) of the lane's value
                             // pair, k-group lane / 16
    uint32_t vc[2 * VB];     // value code chunk `lane`
    uint32_t kszw[2];        // key (s, z) of the two channels this lane folds into q
    uint32_t kszb[8];        // key (s, z) of channels 8*(lane%16) .. +7 (zero terms, page max);
                             // per-token keys: (s, z) of groups 0..3 of tokens t0, t1
    uint32_t vszq[2][4];     // value (s, z) of groups 0..3 of tokens t0, t1
};

// Floating-point layers: kc[blk] holds channels 32a .. 32a+31 of token 16*blk + r16 (one
// element per byte for FP8, two per word for BF16) and vc holds, for each channel block nb,
// tokens 8a .. 8a+7 of channel 16*nb + r16 (vc[2nb..] for FP8, vc[4nb..] for BF16).
template <int KM, int NK, int NV>
__device__ __forceinline__ void load_page_float(uint32_t (&kc)[2][NK], uint32_t (&vc)[NV], const uint8_t *base,
                                                int lane)
{
    using FL = FloatLayout<KM>;
    constexpr int E = FL::kElem;
    const int a = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const uint4 *src = reinterpret_cast<const uint4 *>(base + (16 * blk + r16) * kHeadDim * E + 32 * a * E);
#pragma unroll
        for (int i = 0; i < 2 * E; ++i) {
            const uint4 x = src[i];
            kc[blk][4 * i] = x.x; kc[blk][4 * i + 1] = x.y; kc[blk][4 * i + 2] = x.z; kc[blk][4 * i + 3] = x.w;
        }
    }
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
        const uint8_t *src = base + FL::kV + (16 * nb + r16) * kGroup * E + 8 * a * E;
        if constexpr (E == 1) {
            const uint2 x = *reinterpret_cast<const uint2 *>(src);
            vc[2 * nb] = x.x; vc[2 * nb + 1] = x.y;
        } else {
            const uint4 x = *reinterpret_cast<const uint4 *>(src);
            vc[4 * nb] = x.x; vc[4 * nb + 1] = x.y; vc[4 * nb + 2] = x.z; vc[4 * nb + 3] = x.w;
        }
    }
}

template <int KB, int VB, int KM>
__device__ __forceinline__ void load_page(PageRegs<KB, VB> &r, const uint8_t *base, int lane, int ch0, int ch1,
                                          int t0, int t1)
{
    if constexpr (is_float_layer(KM)) {
        load_page_float<KM>(r.kc, r.vc, base, lane);
        return;
    } else {
    constexpr bool KT = KM == kLayerKeysPerToken;
    using PL = PageLayout<KB, VB>;
    const int a = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const uint32_t *src = reinterpret_cast<const uint32_t *>(base + PL::kKCodes + (blk == 0 ? t0 : t1) * PL::kKRowBytes + a * 4 * KB);
        if constexpr (KB == 2) {
            const uint2 x = *reinterpret_cast<const uint2 *>(src);
            r.kc[blk][0] = x.x; r.kc[blk][1] = x.y;
        } else {
#pragma unroll
            for (int i = 0; i < KB; i += 4) {
                const uint4 x = *reinterpret_cast<const uint4 *>(src + i);
                r.kc[blk][i] = x.x; r.kc[blk][i + 1] = x.y; r.kc[blk][i + 2] = x.z; r.kc[blk][i + 3] = x.w;
            }
        }
    }
    const uint32_t *vsrc = reinterpret_cast<const uint32_t *>(base + PL::kVCodes + lane * 8 * VB);
#pragma unroll
    for (int i = 0; i < 2 * VB; i += 4) {
        const uint4 x = *reinterpret_cast<const uint4 *>(vsrc + i);
        r.vc[i] = x.x; r.vc[i + 1] = x.y; r.vc[i + 2] = x.z; r.vc[i + 3] = x.w;
    }
    const uint32_t *ksz = reinterpret_cast<const uint32_t *>(base + PL::kKSz);
    if constexpr (!KT) {
        r.kszw[0] = ksz[ch0];
        r.kszw[1] = ksz[ch1];
    }
    const uint4 b0 = *reinterpret_cast<const uint4 *>(ksz + (KT ? kValueGroups * t0 : 8 * r16));
    const uint4 b1 = *reinterpret_cast<const uint4 *>(ksz + (KT ? kValueGroups * t1 : 8 * r16 + 4));
    r.kszb[0] = b0.x; r.kszb[1] = b0.y; r.kszb[2] = b0.z; r.kszb[3] = b0.w;
    r.kszb[4] = b1.x; r.kszb[5] = b1.y; r.kszb[6] = b1.z; r.kszb[7] = b1.w;
    const uint32_t *vsz = reinterpret_cast<const uint32_t *>(base + PL::kVSz);
    const uint4 w0 = *reinterpret_cast<const uint4 *>(vsz + kValueGroups * t0);
    const uint4 w1 = *reinterpret_cast<const uint4 *>(vsz + kValueGroups * t1);
    r.vszq[0][0] = w0.x; r.vszq[0][1] = w0.y; r.vszq[0][2] = w0.z; r.vszq[0][3] = w0.w;
    r.vszq[1][0] = w1.x; r.vszq[1][1] = w1.y; r.vszq[1][2] = w1.z; r.vszq[1][3] = w1.w;
    }
}

// Pages of a split among its waves.  Four-wave workgroups (two per CU) and every split but
// split 0 deal them round robin.  On split 0 of an eight-wave workgroup, wave 0 also attends
// the residual tokens, which costs it about as long as four pages: the first 4 * 7 pages go
// round robin to waves 1-7, the rest round robin to waves 1-7 and then 0 (a split of 64
// pages: 4, 9, 9, 9, 9, 8, 8, 8; of 256: 28, then 33 or 32).  Returns the split-relative
// index of the wave's page `j` (increasing in j).
constexpr int kResidualPages = 4;

template <int NW>
__device__ __forceinline__ int split_page(int wave, int j, int split)
{
    if constexpr (NW != 8) return NW * j + wave;
    if (split != 0) return 8 * j + wave;
    constexpr int head = kResidualPages * 7;
    if (wave == 0) return head + 8 * j + 7;
    if (j < kResidualPages) return 7 * j + wave - 1;
    return head + 8 * (j - kResidualPages) + wave - 1;
}

// KM: the layer code -- integer codes with per-channel or per-token keys (one key group per
// token and 32 channels), or FP8 / BF16 values
// two waves per SIMD (two workgroups per CU) whenever G <= 8: at most 256 registers per lane
template <int KB, int VB, int GS, typename QT, int KM, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(GS <= 2 ? 2 : 1)))
void decode_kernel(const int32_t *len_src, const int32_t *block_table, const void *q_in, const uint8_t *pool,
                   int batch, int max_pages, int P, int H, int G, int fused, DecodeParams p)
{
    constexpr int NT = 64 * NW;
    constexpr bool KT = KM == kLayerKeysPerToken;
    constexpr bool FLT = is_float_layer(KM);
    constexpr int kPageBytes = layer_page_bytes<KB, VB, KM>();
    constexpr int HS = 4 * GS;                 // head slots
    __shared__ DecodeSmem<GS, KM, NW> sm;
    // grid (H, batch, splits): the split index varies slowest, so every (sequence, KV head)
    // has its split 0 dispatched first
    const int h = blockIdx.x, b = blockIdx.y, split = blockIdx.z;
    const int tid = threadIdx.x;
    KVQ_STAMP(0);
    const long long bh = static_cast<long long>(b) * H + h;
    float *out_bh = p.out + bh * G * kHeadDim;
    float *lse_bh = p.lse ? p.lse + bh * G : nullptr;
    const bool append = fused != 0;            // fused append: attend over pos + 1 tokens
    // ---- the length, this wave's block-table ids (every page the split could hold) and q
    // are requested together, before any of them is waited for.  The length is read as a
    // lane-indexed vector load (lane i: sequence 64*(b/64) + i) and taken from lane b % 64: a
    // uniform scalar load would be waited for (with the kernel arguments) before the other
    // requests could go out -------------------------------------------------------------
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int a = lane >> 4, r16 = lane & 15;
    const int pg_lim = min(max_pages, (split + 1) * P);    // >= 1
    // the split-relative index of this lane's page (lane j: the wave's j-th page)
    const int pg_rel = split_page<NW>(wave, lane, split);
    // lane roles in the page loop
    const int kq = lane >> 4, kjj = (lane >> 2) & 3, kj = lane & 3;   // key pair this lane folds
    // per-channel keys: any channel pair of the lane's 32-channel group; per-token keys: the
    // pair 32*kjj + 8*kq + 2*kj, + 1, so that matrix-core block kjj is exactly key group kjj
    // floating-point layers: the natural pair 2*lane, 2*lane + 1
    // (per-token keys with 2- or 4-bit codes: the pair holds slots 4 apart in one half-word,
    // channels 32*kjj + 8*kq + 2*(kj%2) + kj/2 and 4 further)
    const int ch0 = FLT                 ? 2 * lane
                    : KT && KB == 8     ? 32 * kjj + 8 * kq + 2 * kj
                    : KT                ? 32 * kjj + 8 * kq + 2 * (kj & 1) + (kj >> 1)
                                        : 32 * kq + key_pair_channel<KB>(kjj, kj);
    const int ch1 = FLT || (KT && KB == 8) ? ch0 + 1 : KT ? ch0 + 4 : ch0 + key_pair_step<KB>();
    // (unconditional loads at clamped indices, in one basic block, none waited for before the
    // last is issued; the length first, so that waiting for it leaves the others in flight)
    const int len_lane = len_src[min((b & ~63) + lane, batch - 1)];
    const int bt_i = split * P + pg_rel;
    int my_phys = block_table[static_cast<long long>(b) * max_pages + min(bt_i, pg_lim - 1)];
    // q straight from memory in the layouts the lane uses: 8 channels 8*r16 .. +7 of heads
    // 4i + a (the zero terms; their maxima give the per-head exponents) and channels ch0, ch1
    // of every head (the folded key pair); per-token keys also take channels 32J + 2*r16, +1
    const long long q0 = bh * G * kHeadDim;
    float qbl[GS][8], qwl[HS][2], qtl[KT ? GS : 1][4][2];
#pragma unroll
    for (int i = 0; i < GS; ++i) {
        const long long qi = q0 + min(4 * i + a, G - 1) * kHeadDim + 8 * r16;
        load_q8<QT>(q_in, qi, qbl[i]);
    }
#pragma unroll
    for (int hh = 0; hh < HS; ++hh) {
        const long long qh = q0 + min(hh, G - 1) * kHeadDim;
        qwl[hh][0] = load_q<QT>(q_in, qh + ch0);
        qwl[hh][1] = load_q<QT>(q_in, qh + ch1);
    }
    if constexpr (KT) {
#pragma unroll
        for (int i = 0; i < GS; ++i)
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                const long long qi = q0 + min(4 * i + a, G - 1) * kHeadDim + 32 * J + 2 * r16;
                qtl[i][J][0] = load_q<QT>(q_in, qi);
                qtl[i][J][1] = load_q<QT>(q_in, qi + 1);
            }
    }
    if (bt_i >= pg_lim) my_phys = 0;
    const int L = __builtin_amdgcn_readlane(len_lane, b & 63) + (append ? 1 : 0);
    KVQ_STAMP(8);

    const bool bad_len = (append ? L <= 0 : L < 0) || L > p.max_seq_len || L > kGroup * max_pages;
    if (bad_len || L == 0) {
        if (split == 0) {
            const float o = bad_len ? NAN : 0.0f;
            for (int i = tid; i < G * kHeadDim; i += NT) out_bh[i] = o;
            if (lse_bh && tid < G) lse_bh[tid] = bad_len ? NAN : -INFINITY;
        }
        KVQ_STAMP(5);
        return;
    }
    // a fused append that completes a group quantizes that page itself (split 0) and attends
    // over it from LDS: the pool supplies only the pages that existed before this call
    const bool flush = append && L % kGroup == 0;
    const int full = L / kGroup - (flush ? 1 : 0);      // pages read from the pool
    const int nres = flush ? kGroup : L % kGroup;       // tokens attended from the residual tile
    const int n_ps = (full + P - 1) / P;               // splits with pages
    const int n_work = n_ps > 0 ? n_ps : 1;             // workgroups of this (sequence, KV head)
    if (split >= n_work) {
        KVQ_STAMP(5);
        return;
    }
    // the residual tokens belong to split 0: the first workgroups dispatched absorb the extra
    // work while the last ones are still starting
    const bool has_res = nres > 0 && split == 0;

    const int pg_end = min(full, (split + 1) * P);
    const int n_my = __builtin_popcountll(__ballot(bt_i < pg_end));
    // value pair this lane folds (group a): tokens (w, w+4) of its octet for 8-bit codes,
    // (w%2 + 4*(w/2), +2) for 2- and 4-bit codes, w = r16 % 4 -- the order their B operand
    // pairs take
    const int vw = r16 & 3;
    const int t0 = 8 * (r16 >> 2) + (VB == 8 ? vw : (vw & 1) + 4 * (vw >> 1));
    const int t1 = t0 + (VB == 8 ? 4 : 2);
    // powers of two the code unpack leaves on this lane's key channels / value tokens
    const int kshift = unpack_shift<KB>(kj), vshift = unpack_shift<VB>(r16 & 3);
    // Without a flush, wave 0 of split 0 attends the residual tokens before its page loop:
    // their rows are requested as soon as the length is known.  With a flush the workgroup
    // quantizes and attends them after its page loop (rows requested after the first page).
    const bool res_wave = has_res && !flush && wave == 0;
    ResidualWaveRegs rw;
    if (res_wave) load_residual_wave(p, bh, nres, append, rw);
    // The first page is requested as soon as the block-table ids are in: q, requested before
    // it, is waited for afterwards (the memory counter completes in order), which leaves the
    // page in flight during the q setup below.
    // page ids outside the pool mark the sequence bad (NaN outputs) and are read as page 0
    const bool id_bad = lane < n_my && (my_phys < 0 || my_phys >= p.n_pages);
    bool bad_page = __any(id_bad);
    if (id_bad) my_phys = 0;
    auto page_base = [&](int j) -> const uint8_t * {
        const int phys = __builtin_amdgcn_readlane(my_phys, j);
        return pool + (static_cast<long long>(phys) * H + h) * kPageBytes;
    };
    PageRegs<KB, VB> cur, nxt;
    if (n_my > 0) load_page<KB, VB, KM>(cur, page_base(0), lane, ch0, ch1, t0, t1);
    uint4 res_kv[4 * (512 / NT)];
    if (has_res && flush) load_residual<NT>(p, bh, append, res_kv);
    KVQ_STAMP(9);
    // q~ = q log2(e)/sqrt(128); the residual tokens (split 0) read it from LDS, written here by
    // wave 0
    if (wave == 0) {
#pragma unroll
        for (int i = 0; i < GS; ++i) {
            if (4 * i + a < G) {
#pragma unroll
                for (int x = 0; x < 8; ++x) sm.qs[4 * i + a][8 * r16 + x] = qbl[i][x] * kScoreScale;
            }
        }
    }
    // per-head normalization exponent eq: |q~ * 2^eq| in [1, 2) -- the maximum over a head's
    // 128 channels is a 16-lane row maximum of the zero-term layout; every lane of group a
    // holds it for heads 4i + a, and lane 16*(hh % 4) gives it for any head hh
    int eqv[GS];
#pragma unroll
    for (int i = 0; i < GS; ++i) {
        float mx = 0.0f;
#pragma unroll
        for (int x = 0; x < 8; ++x) mx = fmaxf(mx, fabsf(qbl[i][x]));
        mx = row_max(mx) * kScoreScale;
        int e = 0;
        if (mx > 0.0f) frexpf(mx, &e);
        eqv[i] = 1 - e;
    }
    KVQ_STAMP(10);
    if (res_wave) {
        // (the highest issue priority while the other waves wait for their first pages)
        if (NW == 8) __builtin_amdgcn_s_setprio(3);
        wave_lds_sync();
        residual_wave<GS, KM, NW>(p, sm, sm.u.w[0], rw, nres, G, bh, append);
    }

    const long long slot0 = bh * p.n_splits;
    int early_cnt = -1;
    // ---- the split combine's batches of partials (splits s0 .. s0+kCB-1 of this (sequence,
    // KV head)): one thread per 4 consecutive channels of a head, kMI such items per thread
    constexpr int kVec = 4, kPerHead = kHeadDim / kVec;
    constexpr int kMI = (HS * kPerHead + NT - 1) / NT;                 // items per thread
    constexpr int kCB = 4;
    float cmv[kMI][kCB], clv[kMI][kCB];
    float4 cov[kMI][kCB];
    auto load_batch = [&](int k, int s0) {
        const int it = tid + k * NT;
        const int hh = min(it / kPerHead, G - 1), c = (it % kPerHead) * kVec;
        const float *ml_base = p.part_ml + (slot0 * G + hh) * 2;            // split s at + s * G * 2
        const float *o_base = p.part_o + (slot0 * G + hh) * kHeadDim;       // split s at + s * G * 128
#pragma unroll
        for (int jb = 0; jb < kCB; ++jb) {
            const int s_ = s0 + jb;
            cmv[k][jb] = -INFINITY;
            clv[k][jb] = 0.0f;
            cov[k][jb] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (s_ != split && s_ < n_work) {       // this split's own partial comes from registers
                const float *ml = ml_base + static_cast<long long>(s_) * G * 2;
                const float *po = o_base + static_cast<long long>(s_) * G * kHeadDim;
                cmv[k][jb] = load_dev(ml);
                clv[k][jb] = load_dev(ml + 1);
                cov[k][jb] = make_float4(load_dev(po + part_slot(c)), load_dev(po + part_slot(c + 1)),
                                         load_dev(po + part_slot(c + 2)), load_dev(po + part_slot(c + 3)));
            }
        }
    };
    if (tid == 0) {
        sm.early = 0;
        sm.bad = 0;
    }
    if (n_ps > 0) {
        WaveLds<GS, KM> &W = sm.u.w[wave];
        constexpr int NP = WaveLds<GS, KM>::NP, PG = WaveLds<GS, KM>::PG;
#pragma unroll
        for (int part = 0; part < NP; ++part) {     // zero rows: A operands of absent heads
            W.qp[part][HS][lane] = 0u;
            if (lane < 16 * PG) W.pp_row(lane / 16, part, HS)[lane % 16] = 0u;
        }
        const int hr = 4 * (r16 & 3) + (r16 >> 2);             // head of A row r16
        // With few head slots the A-operand parts (hi / lo, or hi / mid / lo) share one
        // matrix: part p of head slot hh is row slot p*HS + hh, so one MFMA forms every part
        // and D element p*GS + i holds part p of head 4i + a (summed after the MFMA).
        constexpr bool RS = NP * HS <= 16;
        const int arow = RS ? ((hr < NP * HS && hr % HS < G) ? hr % HS : HS) : (hr < G ? hr : HS);
        const int apart = RS && hr < NP * HS ? hr / HS : 0;
        // element i of an MFMA result with its parts summed
        auto dsum = [&](const float4_t &v, int i) -> float {
            float x = v[i];
            if constexpr (RS) {
#pragma unroll
                for (int part = 1; part < NP; ++part) x += v[part * GS + i];
            }
            return x;
        };
        // q~ of the folded key pair, every head; per-channel integer keys keep it times
        // 2^(KE - kshift), KE the wave's current key exponent (see the page work)
        float qw[HS][2];
        float qb[GS][8];                                        // q~ of the zero-term channels
        float inv_eq[GS];                                       // 2^-eq of the lane's heads
#pragma unroll
        for (int hh = 0; hh < HS; ++hh) {
            const int e = __builtin_amdgcn_readlane(eqv[hh / 4], 16 * (hh % 4));
            qw[hh][0] = hh < G ? ldexpf(qwl[hh][0] * kScoreScale, e) : 0.0f;
            qw[hh][1] = hh < G ? ldexpf(qwl[hh][1] * kScoreScale, e) : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < GS; ++i) {
            const int hh = 4 * i + a;
#pragma unroll
            for (int x = 0; x < 8; ++x) qb[i][x] = hh < G ? ldexpf(qbl[i][x] * kScoreScale, eqv[i]) : 0.0f;
            inv_eq[i] = hh < G ? ldexpf(1.0f, -eqv[i]) : 0.0f;
        }
        // per-token keys: the A operand is q~ itself (page-invariant), folded once; the zero
        // terms need q~ summed over each key group: qsum[i][J] for head 4i + a
        float qsum[GS][4];
        if constexpr (KT) {
            const float f = ldexpf(1.0f, -kshift);
#pragma unroll
            for (int hh = 0; hh < HS; ++hh) {
                const uint32_t hi = split_hi(qw[hh][0] * f, qw[hh][1] * f);
                W.qp[0][hh][lane] = hi;
                W.qp[1][hh][lane] = split_lo(qw[hh][0], f, qw[hh][1], f, hi);
            }
#pragma unroll
            for (int i = 0; i < GS; ++i) {
                const int hh = 4 * i + a;
#pragma unroll
                for (int J = 0; J < 4; ++J) {
                    const float x = hh < G ? ldexpf(qtl[i][J][0] * kScoreScale + qtl[i][J][1] * kScoreScale, eqv[i])
                                           : 0.0f;
                    qsum[i][J] = row_sum(x);
                }
            }
            wave_lds_sync();
        }
        // floating-point layers: A = q~ (FP8: times 2^14, fp16 hi | lo; BF16: three bf16
        // parts) for the pair 2*lane, 2*lane + 1, folded once; the scores take the K scale
        const float ks = FLT && p.scales ? p.scales[2 * h] : 1.0f;
        const float vs = FLT && p.scales ? p.scales[2 * h + 1] : 1.0f;
        float ksc[GS];                                          // score factor per head slot
        if constexpr (FLT) {
#pragma unroll
            for (int hh = 0; hh < HS; ++hh) {
                if constexpr (KM == kLayerFp8) {
                    const uint32_t hi = split_hi(qw[hh][0] * 16384.0f, qw[hh][1] * 16384.0f);
                    W.qp[0][hh][lane] = hi;
                    W.qp[1][hh][lane] = split_lo(qw[hh][0], 16384.0f, qw[hh][1], 16384.0f, hi);
                } else {
                    split3_bf16(qw[hh][0], qw[hh][1], W.qp[0][hh][lane], W.qp[1][hh][lane], W.qp[2][hh][lane]);
                }
            }
#pragma unroll
            for (int i = 0; i < GS; ++i) ksc[i] = KM == kLayerFp8 ? inv_eq[i] * (ks * (1.0f / 16384.0f)) : inv_eq[i];
            wave_lds_sync();
        }

        // per-channel integer keys: |q~ s 2^KE| < 2^15 for every channel of every page; KE is
        // set from the first page and recomputed only for a page whose largest scale reaches
        // 2^(14 - KE) or stays below 2^(6 - KE) (thresholds ke_hi / ke_lo, 0 before the first
        // page), where sck = 2^-KE / 2^eq undoes it in the scores
        int KE = 0;
        uint32_t ke_hi = 0u, ke_lo = 0u;
        float sck[GS];
#pragma unroll
        for (int i = 0; i < GS; ++i) sck[i] = inv_eq[i];
        if constexpr (!KT && !FLT) {
#pragma unroll
            for (int hh = 0; hh < HS; ++hh) {
                qw[hh][0] = ldexpf(qw[hh][0], -kshift);
                qw[hh][1] = ldexpf(qw[hh][1], -kshift);
            }
        }
        const uint32_t magic = fp16x2_1024();
        float4_t acc[8];
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) acc[nb] = float4_t{0.f, 0.f, 0.f, 0.f};
        float m_run[GS], l_part[GS];
#pragma unroll
        for (int i = 0; i < GS; ++i) {
            m_run[i] = -INFINITY;
            l_part[i] = 0.0f;
        }
        float zb[GS][4];                                        // value zero terms: head 4i + a, group j
#pragma unroll
        for (int i = 0; i < GS; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) zb[i][j] = 0.0f;
        // The value accumulators hold sum_t (p s 2^ev) v: ev keeps the folded
        // weights in the normal fp16 range (|p s 2^ev| < 2^15); it only decreases, rescaling
        // acc when it does -- exactly when a page holds a scale >= 2^(14 - ev) (threshold
        // ev_thr); fv = 2^(ev - vshift) scales this lane's weights before the fold.
        int ev = 127;
        uint32_t ev_thr = 1u;
        float fv = ldexpf(1.0f, ev - vshift);

        auto process_page = [&](const PageRegs<KB, VB> &cur) {
          float s2[2][GS];
          if constexpr (FLT) {
            // ---- floating-point keys: q~ against the stored values, then the K scale ------
            float4_t sacc[2];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                uint4 av[NP];
#pragma unroll
                for (int part = 0; part < (RS ? 1 : NP); ++part)
                    av[part] = lds_read16(&W.qp[RS ? apart : part][arow][16 * a + 4 * jj]);
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) {
                    float4_t c = jj == 0 ? float4_t{0.f, 0.f, 0.f, 0.f} : sacc[blk];
                    if constexpr (KM == kLayerFp8) {
                        const uint4 bk = fp8x8_to_f16(cur.kc[blk][2 * jj], cur.kc[blk][2 * jj + 1]);
#pragma unroll
                        for (int part = 0; part < (RS ? 1 : NP); ++part) c = mfma(av[part], bk, c);
                    } else {
                        const uint4 bk = make_uint4(cur.kc[blk][4 * jj], cur.kc[blk][4 * jj + 1], cur.kc[blk][4 * jj + 2],
                                                    cur.kc[blk][4 * jj + 3]);
#pragma unroll
                        for (int part = 0; part < (RS ? 1 : NP); ++part) c = mfma_bf16(av[part], bk, c);
                    }
                    sacc[blk] = c;
                }
            }
#pragma unroll
            for (int i = 0; i < GS; ++i)
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) s2[blk][i] = dsum(sacc[blk], i) * ksc[i];
          } else if constexpr (!KT) {
            // ---- key exponent: every lane checks the two scales it folds; the exact page
            // exponent (the largest scale of the page) only when one is out of range ---------
            {
                // (the barrier keeps the compiler from moving the masks up to the loads, where
                // they would wait for a page just requested)
                uint32_t kw0 = cur.kszw[0], kw1 = cur.kszw[1];
                __asm__ volatile("" : "+v"(kw0), "+v"(kw1));
                const uint32_t u = max(kw0 & 0xFFFFu, kw1 & 0xFFFFu);
                if (__any(u >= ke_hi) || !__any(u >= ke_lo)) {
                    uint32_t smax = 0;
#pragma unroll
                    for (int x = 0; x < 8; ++x) smax = max(smax, cur.kszb[x] & 0x7FFFu);
                    smax = row_max_u32(smax);
                    int E = 0;
                    if (smax != 0u) {
                        int e;
                        frexpf(half_bits_to_float(smax), &e);
                        E = 14 - e;
                    }
#pragma unroll
                    for (int hh = 0; hh < HS; ++hh) {
                        qw[hh][0] = ldexpf(qw[hh][0], E - KE);
                        qw[hh][1] = ldexpf(qw[hh][1], E - KE);
                    }
#pragma unroll
                    for (int i = 0; i < GS; ++i) sck[i] = ldexpf(inv_eq[i], -E);
                    KE = E;
                    ke_hi = fp16_pow2_bits(14 - KE);
                    ke_lo = 14 - KE - 8 < -24 ? 0u : fp16_pow2_bits(14 - KE - 8);
                }
            }
            // ---- fold key scales into q: two channels x every head slot, hi/lo ---------
#pragma unroll
            for (int hh = 0; hh < HS; ++hh) {
                const uint32_t hi = fold_hi(qw[hh][0], qw[hh][1], cur.kszw[0], cur.kszw[1]);
                W.qp[0][hh][lane] = hi;
                W.qp[1][hh][lane] = fold_lo(qw[hh][0], qw[hh][1], cur.kszw[0], cur.kszw[1], hi);
            }
            // ---- key zero terms: sum_c q~_c z_c per head, lane group a holds heads a+4i
            float bias[GS];
#pragma unroll
            for (int i = 0; i < GS; ++i) {
                float s = 0.0f;
#pragma unroll
                for (int x = 0; x < 8; ++x) s = fmaf(qb[i][x], half_bits_to_float(cur.kszb[x] >> 16), s);
                bias[i] = row_sum(s);
            }
            wave_lds_sync();
            // ---- scores on MFMA ------------------------------------------------------
            float4_t sacc[2];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const uint4 ahi = lds_read16(&W.qp[RS ? apart : 0][arow][16 * a + 4 * jj]);
                const uint4 alo = RS ? ahi : lds_read16(&W.qp[1][arow][16 * a + 4 * jj]);
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) {
                    const uint4 bk = unpack_b<KB>(cur.kc[blk], jj, magic);
                    sacc[blk] = mfma(ahi, bk, jj == 0 ? float4_t{0.f, 0.f, 0.f, 0.f} : sacc[blk]);
                    if constexpr (!RS) sacc[blk] = mfma(alo, bk, sacc[blk]);
                }
            }
#pragma unroll
            for (int i = 0; i < GS; ++i) {
                const float bc = bias[i] * inv_eq[i];
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) s2[blk][i] = fmaf(dsum(sacc[blk], i), sck[i], bc);
            }
          } else {
            // ---- per-token keys: one accumulator per key group, then the token's scales --
            float4_t sk[4][2];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const uint4 ahi = lds_read16(&W.qp[RS ? apart : 0][arow][16 * a + 4 * jj]);
                const uint4 alo = RS ? ahi : lds_read16(&W.qp[1][arow][16 * a + 4 * jj]);
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) {
                    const uint4 bk = unpack_b<KB>(cur.kc[blk], jj, magic);
                    sk[jj][blk] = mfma(ahi, bk, float4_t{0.f, 0.f, 0.f, 0.f});
                    if constexpr (!RS) sk[jj][blk] = mfma(alo, bk, sk[jj][blk]);
                }
            }
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
                for (int i = 0; i < GS; ++i) {
                    float raw = 0.0f;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const uint32_t w = cur.kszb[4 * blk + jj];
                        raw = fmaf(half_bits_to_float(w & 0xFFFFu), dsum(sk[jj][blk], i), raw);
                        raw = fmaf(half_bits_to_float(w >> 16), qsum[i][jj], raw);
                    }
                    s2[blk][i] = raw * inv_eq[i];
                }
            }
          }
            // ---- online softmax ------------------------------------------------------
            bool grow = false;
#pragma unroll
            for (int i = 0; i < GS; ++i) {
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) grow |= (4 * i + a < G) && s2[blk][i] > m_run[i];
            }
            if (__any(grow)) {
                float alpha[GS];
#pragma unroll
                for (int i = 0; i < GS; ++i) {
                    const float mp = row_max(fmaxf(s2[0][i], s2[1][i]));
                    const float mn = fmaxf(m_run[i], mp);
                    alpha[i] = exp2f(m_run[i] - mn);
                    m_run[i] = mn;
                    l_part[i] *= alpha[i];
#pragma unroll
                    for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
                        for (int part = 0; part < (RS ? NP : 1); ++part) acc[nb][part * GS + i] *= alpha[i];
                    }
                    if constexpr (!FLT) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) zb[i][j] *= alpha[i];
                    }
                }
            }
            // integer layers: blk 0 / 1 of this lane are tokens t0 / t1, the value pair it folds
            float pw[2][GS];
#pragma unroll
            for (int i = 0; i < GS; ++i) {
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) {
                    const float pv = __builtin_amdgcn_exp2f(s2[blk][i] - m_run[i]);
                    l_part[i] += pv;
                    pw[blk][i] = pv;
                    if constexpr (FLT) W.p[4 * i + a][16 * blk + r16] = pv;
                }
            }
          if constexpr (FLT) {
            // ---- floating-point values: A = p (FP8: times 2^14, fp16 hi | lo; BF16: three
            // bf16 parts) for token pair r16 of the lane's heads; the V scale comes at the end
            wave_lds_sync();
#pragma unroll
            for (int i = 0; i < GS; ++i) {
                const int hh = 4 * i + a;
                const float p0 = W.p[hh][2 * r16], p1 = W.p[hh][2 * r16 + 1];
                if constexpr (KM == kLayerFp8) {
                    const uint32_t hi = split_hi(p0 * 16384.0f, p1 * 16384.0f);
                    W.pp_row(0, 0, hh)[r16] = hi;
                    W.pp_row(0, 1, hh)[r16] = split_lo(p0, 16384.0f, p1, 16384.0f, hi);
                } else {
                    split3_bf16(p0, p1, W.pp_row(0, 0, hh)[r16], W.pp_row(0, 1, hh)[r16], W.pp_row(0, 2, hh)[r16]);
                }
            }
            wave_lds_sync();
            uint4 av[NP];
#pragma unroll
            for (int part = 0; part < (RS ? 1 : NP); ++part) av[part] = lds_read16(&W.pp_row(0, RS ? apart : part, arow)[4 * a]);
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                if constexpr (KM == kLayerFp8) {
                    const uint4 bv = fp8x8_to_f16(cur.vc[2 * nb], cur.vc[2 * nb + 1]);
#pragma unroll
                    for (int part = 0; part < (RS ? 1 : NP); ++part) acc[nb] = mfma(av[part], bv, acc[nb]);
                } else {
                    const uint4 bv = make_uint4(cur.vc[4 * nb], cur.vc[4 * nb + 1], cur.vc[4 * nb + 2], cur.vc[4 * nb + 3]);
#pragma unroll
                    for (int part = 0; part < (RS ? 1 : NP); ++part) acc[nb] = mfma_bf16(av[part], bv, acc[nb]);
                }
            }
          } else {
            // ---- value-scale exponent: ev decreases when a page holds a scale >= 2^(14 - ev)
            // (a check of the lane's own eight scales); the page's exact exponent only then
            {
                uint32_t vw[2][4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    vw[0][j] = cur.vszq[0][j];
                    vw[1][j] = cur.vszq[1][j];
                }
                __asm__ volatile("" : "+v"(vw[0][0]), "+v"(vw[0][1]), "+v"(vw[0][2]), "+v"(vw[0][3]),
                                      "+v"(vw[1][0]), "+v"(vw[1][1]), "+v"(vw[1][2]), "+v"(vw[1][3]));
                uint32_t u = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) u = max(u, max(vw[0][j] & 0xFFFFu, vw[1][j] & 0xFFFFu));
                if (__any(u >= ev_thr)) {
                    // every row of lanes holds all 32 tokens and all four groups
                    uint32_t vmax = 0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) vmax = max(vmax, max(cur.vszq[0][j] & 0x7FFFu, cur.vszq[1][j] & 0x7FFFu));
                    vmax = row_max_u32(vmax);
                    if (vmax != 0u) {
                        int e;
                        frexpf(half_bits_to_float(vmax), &e);
                        const int ev_page = 14 - e;
                        if (ev_page < ev) {
                            const float f = ldexpf(1.0f, ev_page - ev);
#pragma unroll
                            for (int nb = 0; nb < 8; ++nb) acc[nb] *= f;
                            ev = ev_page;
                            ev_thr = fp16_pow2_bits(14 - ev);
                            fv = ldexpf(1.0f, ev - vshift);
                        }
                    }
                }
            }
            // ---- fold value scales into p: the lane's own weights of tokens t0, t1 x every
            // value group, hi/lo (no exchange: the scores put this lane's pair in its registers)
            float ps[2][GS];
#pragma unroll
            for (int i = 0; i < GS; ++i) {
                ps[0][i] = pw[0][i] * fv;
                ps[1][i] = pw[1][i] * fv;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t w0 = cur.vszq[0][j], w1 = cur.vszq[1][j];
#pragma unroll
                for (int i = 0; i < GS; ++i) {
                    const uint32_t hi = fold_hi(ps[0][i], ps[1][i], w0, w1);
                    W.pp_row(j, 0, 4 * i + a)[r16] = hi;
                    W.pp_row(j, 1, 4 * i + a)[r16] = fold_lo(ps[0][i], ps[1][i], w0, w1, hi);
                    zb[i][j] = fmaf(pw[0][i], static_cast<float>(hi_half(w0)),
                                    fmaf(pw[1][i], static_cast<float>(hi_half(w1)), zb[i][j]));
                }
            }
            wave_lds_sync();
            // ---- values on MFMA ------------------------------------------------------
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const uint4 ahi = lds_read16(&W.pp_row(g, RS ? apart : 0, arow)[4 * a]);
                const uint4 alo = RS ? ahi : lds_read16(&W.pp_row(g, 1, arow)[4 * a]);
#pragma unroll
                for (int nb = 2 * g; nb < 2 * g + 2; ++nb) {
                    const uint4 bv = unpack_b<VB>(cur.vc, nb, magic);
                    acc[nb] = mfma(ahi, bv, acc[nb]);
                    if constexpr (!RS) acc[nb] = mfma(alo, bv, acc[nb]);
                }
            }
          }
        };
        // two page buffers in fixed roles: page j+1 is in flight while page j is processed.
        // Every prefetch is unconditional (past the wave's last page it reloads that page,
        // an L2 hit), so the compiler's wait counts see one path and wait only for the page
        // about to be used, never for the one just requested.
        auto prefetch = [&](PageRegs<KB, VB> &dst, int j) {
            load_page<KB, VB, KM>(dst, page_base(min(j, n_my - 1)), lane, ch0, ch1, t0, t1);
        };
        // The two waves of a SIMD share its issue arbiter, which favours the higher priority and
        // then the older wave: each wave's priority follows the pages it has left, so the wave
        // that is behind is served first and the two run out of pages together.
        auto set_prio = [&](int left) {
            if (NW != 8) return;
            if (left > 6) __builtin_amdgcn_s_setprio(3);
            else if (left > 4) __builtin_amdgcn_s_setprio(2);
            else if (left > 2) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
        };
        KVQ_STAMP(1);
        int j = 0;
        for (; j + 1 < n_my; j += 2) {
            prefetch(nxt, j + 1);
            set_prio(n_my - j);
            process_page(cur);
            if (j == 0) KVQ_STAMP(11);
            prefetch(cur, j + 2);
            set_prio(n_my - j - 1);
            process_page(nxt);
        }
        if (j < n_my) {
            set_prio(1);
            process_page(cur);
        }
        if (NW == 8) __builtin_amdgcn_s_setprio(0);
        KVQ_STAMP(2);
        // the split counter, read right after the page loop and used after the merge (see below)
        if (tid == 0 && n_work > 1) early_cnt = __hip_atomic_load(p.counters + bh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

        // ---- this wave's state: l per head, value zero terms, unnormalized output -------
        float lw[GS];
#pragma unroll
        for (int i = 0; i < GS; ++i) lw[i] = row_sum(l_part[i]);
        if constexpr (!FLT) {
#pragma unroll
            for (int i = 0; i < GS; ++i) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float v = row_sum(zb[i][j]);    // the 16 lanes' pairs cover all 32 tokens once
                    if (r16 == 0) W.bv[j][4 * i + a] = v;
                }
            }
            wave_lds_sync();
        }
        float o_out[8][GS];
        if constexpr (FLT) {
            const float unscale = KM == kLayerFp8 ? vs * (1.0f / 16384.0f) : 1.0f;
#pragma unroll
            for (int nb = 0; nb < 8; ++nb)
#pragma unroll
                for (int i = 0; i < GS; ++i) o_out[nb][i] = dsum(acc[nb], i) * unscale;
        } else {
            const float unscale = ldexpf(1.0f, -ev);
#pragma unroll
            for (int nb = 0; nb < 8; ++nb)
#pragma unroll
                for (int i = 0; i < GS; ++i) o_out[nb][i] = fmaf(dsum(acc[nb], i), unscale, W.bv[nb >> 1][4 * i + a]);
        }
        __syncthreads();     // every wave is done with its WaveLds: reuse the space
        KVQ_STAMP(14);
        if (has_res && flush)
            bad_page |= !residual_wg<KB, VB, GS, KM, NW>(p, sm, res_kv, nres, G, bh, append, flush, full);
        MergeLds<GS, NW> &M = sm.u.merge;
#pragma unroll
        for (int i = 0; i < GS; ++i) {
            const int hh = 4 * i + a;
            if (hh < G) {
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) M.o[wave][hh][16 * nb + r16] = o_out[nb][i];
                if (r16 == 0) {
                    M.m[wave][hh] = m_run[i];
                    M.l[wave][hh] = lw[i];
                }
            }
        }
    } else if (has_res && flush) {
        bad_page |= !residual_wg<KB, VB, GS, KM, NW>(p, sm, res_kv, nres, G, bh, append, flush, full);
    }

    // ---- this workgroup's merge: its waves' page states and, on split 0, the residual ----
    // (bad_page is uniform in each wave: any wave that has it set marks the workgroup; one
    // barrier, where a block-wide OR would take three)
    if (bad_page && lane == 0) sm.bad = 1;
    __syncthreads();
    const bool bad = sm.bad != 0;
    KVQ_STAMP(15);
    const bool single = n_work == 1;
    // one thread per 4 consecutive channels of a head: the head's weights once, then 16-byte
    // reads of the waves' partial outputs (exponents <= 0: the raw exp2)
    float om[kMI], ol[kMI];
    float4 oo[kMI];
    {
        const MergeLds<GS, NW> &M = sm.u.merge;
#pragma unroll
        for (int k = 0; k < kMI; ++k) {
            const int it = tid + k * NT;
            om[k] = -INFINITY;
            ol[k] = 0.0f;
            oo[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (it >= G * kPerHead) continue;
            const int hh = it / kPerHead, c = (it % kPerHead) * kVec;
            float m = has_res ? sm.ro.m[hh] : -INFINITY;
            if (n_ps > 0) {
#pragma unroll
                for (int w = 0; w < NW; ++w) m = fmaxf(m, M.m[w][hh]);
            }
            float l = 0.0f;
            float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (has_res) {
                const float wt = __builtin_amdgcn_exp2f(sm.ro.m[hh] - m);
                const float4 r = *reinterpret_cast<const float4 *>(&sm.ro.o[hh][c]);
                l = wt * sm.ro.l[hh];
                o = make_float4(wt * r.x, wt * r.y, wt * r.z, wt * r.w);
            }
            if (n_ps > 0) {
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    const float wt = M.m[w][hh] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M.m[w][hh] - m);
                    const float4 r = *reinterpret_cast<const float4 *>(&M.o[w][hh][c]);
                    l = fmaf(wt, M.l[w][hh], l);
                    o = make_float4(fmaf(wt, r.x, o.x), fmaf(wt, r.y, o.y), fmaf(wt, r.z, o.z), fmaf(wt, r.w, o.w));
                }
            }
            // a bad sequence: NaN outputs (and a running max that keeps the others' weights finite)
            om[k] = bad ? 0.0f : m;
            ol[k] = bad ? NAN : l;
            oo[k] = bad ? make_float4(NAN, NAN, NAN, NAN) : o;
        }
    }
    if (single) {
#pragma unroll
        for (int k = 0; k < kMI; ++k) {
            const int it = tid + k * NT;
            if (it >= G * kPerHead) continue;
            const int hh = it / kPerHead, c = (it % kPerHead) * kVec;
            const float inv = 1.0f / ol[k];
            *reinterpret_cast<float4 *>(&out_bh[hh * kHeadDim + c]) =
                make_float4(oo[k].x * inv, oo[k].y * inv, oo[k].z * inv, oo[k].w * inv);
            if (lse_bh && c == 0) lse_bh[hh] = (om[k] + log2f(ol[k])) * kLn2;
        }
        KVQ_STAMP(3);
        KVQ_STAMP(5);
        return;
    }
    // Thread 0 read the split counter right after its page loop (early_cnt, used only now: its
    // latency passes under the merge).  When every other split of this (sequence, KV head)
    // had published its partial by then, this workgroup combines at once, with its own state
    // from registers, and publishes nothing.
    if (tid == 0 && early_cnt >= 0) sm.early = early_cnt == n_work - 1;
    __syncthreads();
    const bool early = sm.early != 0;
    if (!early) {
        // publish (m, l, o) with device-scope stores, wait until they are complete, then count
        // this split in; the workgroup that completes the count combines
#pragma unroll
        for (int k = 0; k < kMI; ++k) {
            const int it = tid + k * NT;
            if (it >= G * kPerHead) continue;
            const int hh = it / kPerHead, c = (it % kPerHead) * kVec;
            float *po = p.part_o + ((slot0 + split) * G + hh) * kHeadDim;
            store_dev(po + part_slot(c), oo[k].x);
            store_dev(po + part_slot(c + 1), oo[k].y);
            store_dev(po + part_slot(c + 2), oo[k].z);
            store_dev(po + part_slot(c + 3), oo[k].w);
            if (c == 0) {
                float *pml = p.part_ml + ((slot0 + split) * G + hh) * 2;
                store_dev(pml, om[k]);
                store_dev(pml + 1, ol[k]);
            }
        }
        KVQ_STAMP(3);
        wait_stores();
        __syncthreads();
        if (tid == 0)
            sm.last = __hip_atomic_fetch_add(p.counters + bh, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n_work - 1;
        __syncthreads();
        KVQ_STAMP(4);
        if (!sm.last) {
            KVQ_STAMP(5);
            return;
        }
    } else {
        KVQ_STAMP(3);
        KVQ_STAMP(4);
    }

    // ---- combine every split of this (sequence, KV head): the maximum over all running maxima,
    // then the weighted sums in split order, so the result does not depend on which workgroup
    // combines.  Other splits' partials are read with device-scope loads issued in batches of
    // kCB splits (a dependent chain would cost one memory round trip per split); this split's
    // own partial comes from registers.
#pragma unroll
    for (int k = 0; k < kMI; ++k) {
        const int it = tid + k * NT;
        if (it >= G * kPerHead) continue;
        const int hh = it / kPerHead, c = (it % kPerHead) * kVec;
        const float *ml_base = p.part_ml + (slot0 * G + hh) * 2;
        load_batch(k, 0);
        // (slot by slot with constant indices: an index computed at run time would put the
        // batch arrays in scratch memory)
        auto own = [&](int s0) {
#pragma unroll
            for (int jb = 0; jb < kCB; ++jb) {
                if (s0 + jb == split) {
                    cmv[k][jb] = om[k];
                    clv[k][jb] = ol[k];
                    cov[k][jb] = oo[k];
                }
            }
        };
        own(0);
        float mx = -INFINITY;
#pragma unroll
        for (int jb = 0; jb < kCB; ++jb) mx = fmaxf(mx, cmv[k][jb]);
        for (int s_ = kCB; s_ < n_work; ++s_)
            mx = fmaxf(mx, s_ == split ? om[k] : load_dev(ml_base + static_cast<long long>(s_) * G * 2));
        float l = 0.0f;
        float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        for (int s0 = 0;;) {
#pragma unroll
            for (int jb = 0; jb < kCB; ++jb) {
                if (s0 + jb < n_work) {
                    const float w = cmv[k][jb] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(cmv[k][jb] - mx);
                    l = fmaf(w, clv[k][jb], l);
                    o = make_float4(fmaf(w, cov[k][jb].x, o.x), fmaf(w, cov[k][jb].y, o.y), fmaf(w, cov[k][jb].z, o.z),
                                    fmaf(w, cov[k][jb].w, o.w));
                }
            }
            s0 += kCB;
            if (s0 >= n_work) break;
            load_batch(k, s0);
            own(s0);
        }
        const float inv = 1.0f / l;
        *reinterpret_cast<float4 *>(&out_bh[hh * kHeadDim + c]) = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
        if (lse_bh && c == 0) lse_bh[hh] = (mx + log2f(l)) * kLn2;
    }
    // the count is complete (or was, for an early combine): reset it for the next call
    if (tid == 0) __hip_atomic_store(p.counters + bh, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    KVQ_STAMP(5);
}

#if defined(KVQ_DECODE_COMMON)
__global__ void zero_fill_kernel(uint32_t *p, size_t n_words)
{
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n_words;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        p[i] = 0u;
}
#endif

template <int KB, int VB, int GS, int KM, int NW>
hipError_t launch_decode_g(const DecodeParams &p, bool q_f32, hipStream_t s)
{
    dim3 grid(p.H, p.batch, p.n_splits);
    // the fields the prologue needs first lead as scalar arguments, which the dispatch
    // preloads into scalar registers (no wait for a kernel-argument load before the first
    // memory requests); the rest stay in the parameter block
    const int32_t *len_src = p.pos ? p.pos : p.seq_len;
    const uint8_t *pool = static_cast<const uint8_t *>(p.pages);
    if (q_f32)
        hipLaunchKernelGGL((decode_kernel<KB, VB, GS, float, KM, NW>), grid, dim3(64 * NW), 0, s, len_src, p.block_table,
                           p.q, pool, p.batch, p.max_pages, p.pages_per_split, p.H, p.G, p.pos != nullptr, p);
    else
        hipLaunchKernelGGL((decode_kernel<KB, VB, GS, uint16_t, KM, NW>), grid, dim3(64 * NW), 0, s, len_src,
                           p.block_table, p.q, pool, p.batch, p.max_pages, p.pages_per_split, p.H, p.G, p.pos != nullptr, p);
    return hipGetLastError();
}

template <int KB, int VB, int KM>
hipError_t launch_decode_k(const DecodeParams &p, bool q_f32, hipStream_t s)
{
    const bool w8 = p.waves == 8;
    if (p.G <= 4) return w8 ? launch_decode_g<KB, VB, 1, KM, 8>(p, q_f32, s) : launch_decode_g<KB, VB, 1, KM, 4>(p, q_f32, s);
    if (p.G <= 8) return w8 ? launch_decode_g<KB, VB, 2, KM, 8>(p, q_f32, s) : launch_decode_g<KB, VB, 2, KM, 4>(p, q_f32, s);
    return launch_decode_g<KB, VB, 4, KM, 4>(p, q_f32, s);
}

// integer layers: key mode 0 / 1
template <int KB, int VB>
hipError_t launch_decode_t(int kmode, const DecodeParams &p, bool q_f32, hipStream_t s)
{
    if (kmode == kLayerKeysPerChannel) return launch_decode_k<KB, VB, kLayerKeysPerChannel>(p, q_f32, s);
    if (kmode == kLayerKeysPerToken) return launch_decode_k<KB, VB, kLayerKeysPerToken>(p, q_f32, s);
    return hipErrorInvalidValue;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

// This source is compiled once per key bit width (KVQ_DECODE_KB = 2, 4, 8: the kernels of
// that width, FP8 with 8; 16: BF16) and once with KVQ_DECODE_COMMON (host helpers and the dispatch), so that the
// kernel instantiations build in parallel.
#if defined(KVQ_DECODE_KB)
#define KVQ_LAUNCH_KB_NAME_(KBV) launch_decode_kb##KBV
#define KVQ_LAUNCH_KB_NAME(KBV) KVQ_LAUNCH_KB_NAME_(KBV)
hipError_t KVQ_LAUNCH_KB_NAME(KVQ_DECODE_KB)(int vb, int kmode, const DecodeParams &p, bool q_f32, hipStream_t s)
{
#if KVQ_DECODE_KB == 16
    if (vb == 16 && kmode == kLayerBf16) return launch_decode_k<16, 16, kLayerBf16>(p, q_f32, s);
#else
#if KVQ_DECODE_KB == 8
    if (vb == 8 && kmode == kLayerFp8) return launch_decode_k<8, 8, kLayerFp8>(p, q_f32, s);
#endif
    if (vb == 2) return launch_decode_t<KVQ_DECODE_KB, 2>(kmode, p, q_f32, s);
    if (vb == 4) return launch_decode_t<KVQ_DECODE_KB, 4>(kmode, p, q_f32, s);
    if (vb == 8) return launch_decode_t<KVQ_DECODE_KB, 8>(kmode, p, q_f32, s);
#endif
    return hipErrorInvalidValue;
}
#endif

#if defined(KVQ_DECODE_COMMON)
DecodeWorkspace decode_workspace_layout(int batch, int H, int G, int n_splits)
{
    DecodeWorkspace w;
    const size_t slots = static_cast<size_t>(batch) * H * n_splits * G;
    w.part_o_off = 0;
    w.part_ml_off = align256(slots * kHeadDim * sizeof(float));
    w.counters_off = w.part_ml_off + align256(slots * 2 * sizeof(float));
    w.bytes = w.counters_off + align256(static_cast<size_t>(batch) * H * sizeof(int));
    return w;
}

int decode_waves_for(int batch, int H, int G)
{
    return G <= 8 && static_cast<long long>(batch) * H <= 256 ? 8 : 4;
}

int decode_default_pages_per_split(int batch, int H, int G, int max_full_pages)
{
    // about 2048 waves for the longest sequences (eight per CU, all resident at once), at
    // least four pages per wave, at most 256 pages per split (32 or 64 per wave: block-table
    // ids are held one per lane)
    const int nw = decode_waves_for(batch, H, G);
    const long long wgs = 2048 / nw;
    const long long work = static_cast<long long>(batch) * H * (max_full_pages > 0 ? max_full_pages : 1);
    long long pps = (work + wgs - 1) / wgs;
    pps = (pps + nw - 1) / nw * nw;
    if (pps < 4 * nw) pps = 4 * nw;
    if (pps > 256) pps = 256;
    return static_cast<int>(pps);
}

int decode_max_g() { return 4 * kMaxGS; }

hipError_t launch_decode(int kb, int vb, int kmode, const DecodeParams &p, bool q_f32, hipStream_t s)
{
    if (kb == 2) return launch_decode_kb2(vb, kmode, p, q_f32, s);
    if (kb == 4) return launch_decode_kb4(vb, kmode, p, q_f32, s);
    if (kb == 8) return launch_decode_kb8(vb, kmode, p, q_f32, s);
    if (kb == 16) return launch_decode_kb16(vb, kmode, p, q_f32, s);
    return hipErrorInvalidValue;
}

hipError_t launch_zero_fill(void *ptr, size_t bytes, hipStream_t s)
{
    const size_t words = bytes / 4;
    if (words == 0) return hipSuccess;
    size_t blocks = (words + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(zero_fill_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<uint32_t *>(ptr), words);
    return hipGetLastError();
}
#endif  // KVQ_DECODE_COMMON

}  // namespace kvq
