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
// Codes are unpacked with one shift, one mask-and-or and one packed subtract per pair into
// exact fp16 integers (OR into 1024.0, subtract 1024).  The folded operands (q s and p s) are split into
// fp16 hi + lo parts (22 significant bits) and both parts are fed to the MFMA with the same
// code operand.  Both are scaled by powers of two so their largest values sit just below
// 2^15: q s per page (from the page's largest key scale), p s per wave (from the largest
// value scale seen so far, p <= 1).  That keeps the lo parts in the normal fp16 range, where
// the matrix cores accumulate at full binary32 accuracy.
//
// Work decomposition.  One workgroup of four waves per (split, KV head, sequence).  Split
// s < n_ps covers pages [s*P, min((s+1)*P, full)), each wave taking every fourth page;
// split n_ps (when L mod 32 > 0) attends over the bf16 residual.  A wave keeps its own
// online-softmax state; the four are merged in LDS, and every split writes (m, l, o[128])
// per query head to the workspace.  The last split of a (sequence, KV head) to finish --
// a device-scope counter -- merges the splits:
//   m = max m_s, l = sum 2^(m_s - m) l_s, out = sum 2^(m_s - m) o_s / l, lse = (m + log2 l) ln 2
// and resets the counter for the next call.  Scores are in log2 units (q carries
// log2(e)/sqrt(128)).
//
// MFMA roles (16x16x32, wave64).  Row r of an A operand / D tile holds query head
// 4*(r % 4) + r / 4, so head h sits in lane group h % 4 (lanes 16*(h%4) ..) and element
// h / 4 of the accumulator: with G <= 4 every lane holds exactly one head per token.
//   scores:  D[head][token]   = A(q s hi|lo, from LDS)    x B(key codes, token-major rows)
//   values:  D[head][channel] = A(p s hi|lo, from LDS)    x B(value codes, chunk layout)
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxGS = 4;                     // head slots per lane group: G <= 16
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kScoreScale = 1.4426950408889634f * 0.08838834764831845f;   // log2(e)/sqrt(128)

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4_t mfma(const uint4 &a, const uint4 &b, const float4_t &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c, 0, 0, 0);
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

// LDS ordering inside one wave: every lane's earlier LDS stores are visible to the
// wave's later LDS loads.
__device__ __forceinline__ void wave_lds_sync()
{
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ float row_max(float v)   // over the 16 lanes of a lane group
{
    v = fmaxf(v, __shfl_xor(v, 1));
    v = fmaxf(v, __shfl_xor(v, 2));
    v = fmaxf(v, __shfl_xor(v, 4));
    v = fmaxf(v, __shfl_xor(v, 8));
    return v;
}

__device__ __forceinline__ float row_sum(float v)
{
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    return v;
}

__device__ __forceinline__ uint32_t row_max_u32(uint32_t v)
{
    v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 1)));
    v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 2)));
    v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 4)));
    v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 8)));
    return v;
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

// Pair j (0..3) of operand `op` from a lane's packed codes, as exact small integers in the
// normal fp16 range: with n = 16/BITS codes per 16-bit half, k = 4*op + j sits in word
// k / n at shift BITS*(k % n) in both halves; OR into 1024.0 (0x6400, whose spacing is 1),
// then subtract 1024 with one packed add.  The matrix cores keep full binary32 accuracy
// only for normal fp16 inputs (subnormal operands lose about four bits in the
// accumulation).
template <int BITS>
__device__ __forceinline__ uint4 unpack_operand_normal(const uint32_t *w, int op)
{
    constexpr int n = 16 / BITS;
    constexpr uint32_t M = ((1u << BITS) - 1u) * 0x00010001u;
    const half2_t bias = {static_cast<_Float16>(-1024.0f), static_cast<_Float16>(-1024.0f)};
    uint32_t r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int k = 4 * op + j;
        const uint32_t x = ((w[k / n] >> (BITS * (k % n))) & M) | 0x64006400u;
        r[j] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, x) + bias);
    }
    return make_uint4(r[0], r[1], r[2], r[3]);
}

// Channel (within a lane's 32-channel k-group) of the low half of pair j of key operand jj.
template <int KB>
__device__ __forceinline__ int key_pair_channel(int jj, int j)
{
    constexpr int n = 16 / KB, nd = 32 / KB;
    const int k = 4 * jj + j;
    return nd * (k / n) + (k % n);
}

template <int GS>
struct WaveLds {
    uint32_t qp[2][4 * GS + 1][64];      // (q s) hi / lo pairs: [part][head, + zero row][pair]
    float p[32][4 * GS];                 // softmax weights of the page: [token][head]
    uint32_t pp[2][4][4 * GS + 1][16];   // (p s) hi / lo pairs: [part][value group][head][pair]
    float alpha[4 * GS];
    float bv[4][4 * GS];                 // value zero terms at the end: [group][head]
};

template <int GS>
struct MergeLds {
    float o[kWaves][4 * GS][kHeadDim];
    float m[kWaves][4 * GS];
    float l[kWaves][4 * GS];
};

template <int GS>
struct DecodeSmem {
    float qs[4 * GS][kHeadDim];   // q * log2(e)/sqrt(128) * 2^eq[h], |.| in [1, 2) per head
    int eq[4 * GS];
    union {
        WaveLds<GS> w[kWaves];
        MergeLds<GS> merge;
        struct {
            float k[kGroup][kHeadDim];
            float v[kGroup][kHeadDim];
            float s[4 * GS][kGroup];
        } res;
    } u;
    int last;
};

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

__device__ __forceinline__ void wait_stores()
{
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ------------------------------------------------------------------------------------
// split-K combine (last split of a (sequence, KV head))
// ------------------------------------------------------------------------------------
__device__ void combine_splits(const DecodeParams &p, long long bh, int expected, int G, float *out_bh, float *lse_bh)
{
    const long long slot0 = bh * p.n_splits;
    for (int idx = threadIdx.x; idx < G * kHeadDim; idx += kThreads) {
        const int g = idx / kHeadDim, c = idx % kHeadDim;
        float m = -INFINITY;
        for (int s = 0; s < expected; ++s) m = fmaxf(m, load_dev(&p.part_ml[((slot0 + s) * G + g) * 2]));
        float l = 0.0f, o = 0.0f;
        for (int s = 0; s < expected; ++s) {
            const float ms = load_dev(&p.part_ml[((slot0 + s) * G + g) * 2]);
            const float ls = load_dev(&p.part_ml[((slot0 + s) * G + g) * 2 + 1]);
            const float w = exp2f(ms - m);
            l = fmaf(w, ls, l);
            o = fmaf(w, load_dev(&p.part_o[((slot0 + s) * G + g) * kHeadDim + c]), o);
        }
        out_bh[g * kHeadDim + c] = o / l;
        if (lse_bh && c == 0) lse_bh[g] = (m + log2f(l)) * kLn2;
    }
}

// ------------------------------------------------------------------------------------
// residual split: up to 31 bf16 tokens, plain VALU
// ------------------------------------------------------------------------------------
template <int GS>
__device__ void residual_split(const DecodeParams &p, DecodeSmem<GS> &sm, long long bh, int nres, int G,
                               long long slot)
{
    const int tid = threadIdx.x;
    const uint16_t *rk = p.resid_k + bh * kGroup * kHeadDim;
    const uint16_t *rv = p.resid_v + bh * kGroup * kHeadDim;
    for (int i = tid; i < nres * kHeadDim; i += kThreads) {
        sm.u.res.k[i / kHeadDim][i % kHeadDim] = bf16_bits_to_float(rk[i]);
        sm.u.res.v[i / kHeadDim][i % kHeadDim] = bf16_bits_to_float(rv[i]);
    }
    __syncthreads();
    // scores: thread (t, part) covers channels 16*part .. 16*part+15 of token t
    {
        const int t = tid >> 3, part = tid & 7;
        for (int h = 0; h < G; ++h) {
            float s = 0.0f;
            if (t < nres) {
#pragma unroll
                for (int x = 0; x < 16; ++x) s = fmaf(sm.qs[h][16 * part + x], sm.u.res.k[t][16 * part + x], s);
            }
            s += __shfl_xor(s, 1);
            s += __shfl_xor(s, 2);
            s += __shfl_xor(s, 4);
            if (part == 0) sm.u.res.s[h][t] = t < nres ? ldexpf(s, -sm.eq[h]) : -INFINITY;
        }
    }
    __syncthreads();
    float *part_ml = p.part_ml + slot * G * 2;
    if (tid < G) {
        const int h = tid;
        float m = -INFINITY;
        for (int t = 0; t < nres; ++t) m = fmaxf(m, sm.u.res.s[h][t]);
        float l = 0.0f;
        for (int t = 0; t < kGroup; ++t) {
            const float e = t < nres ? exp2f(sm.u.res.s[h][t] - m) : 0.0f;
            sm.u.res.s[h][t] = e;
            l += e;
        }
        store_dev(&part_ml[2 * h], m);
        store_dev(&part_ml[2 * h + 1], l);
    }
    __syncthreads();
    float *part_o = p.part_o + slot * G * kHeadDim;
    for (int idx = tid; idx < G * kHeadDim; idx += kThreads) {
        const int h = idx / kHeadDim, c = idx % kHeadDim;
        float o = 0.0f;
        for (int t = 0; t < nres; ++t) o = fmaf(sm.u.res.s[h][t], sm.u.res.v[t][c], o);
        store_dev(&part_o[idx], o);
    }
}

// ------------------------------------------------------------------------------------
// the page splits
// ------------------------------------------------------------------------------------
template <int KB, int VB>
struct PageRegs {
    uint32_t kc[2][KB];      // key codes of tokens 16*blk + (lane % 16), k-group lane / 16
    uint32_t vc[2 * VB];     // value code chunk `lane`
    uint32_t kszw[2];        // key (s, z) of the two channels this lane folds into q
    uint32_t kszb[8];        // key (s, z) of channels 8*(lane%16) .. +7 (zero terms, page max)
    uint32_t vszw[2];        // value (s, z) of the two tokens this lane folds into p
};

template <int KB, int VB>
__device__ __forceinline__ void load_page(PageRegs<KB, VB> &r, const uint8_t *base, int lane, int ch0, int ch1,
                                          int t0, int t1)
{
    using PL = PageLayout<KB, VB>;
    const int a = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const uint32_t *src = reinterpret_cast<const uint32_t *>(base + PL::kKCodes + (16 * blk + r16) * PL::kKRowBytes + a * 4 * KB);
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
    r.kszw[0] = ksz[ch0];
    r.kszw[1] = ksz[ch1];
    const uint4 b0 = *reinterpret_cast<const uint4 *>(ksz + 8 * r16);
    const uint4 b1 = *reinterpret_cast<const uint4 *>(ksz + 8 * r16 + 4);
    r.kszb[0] = b0.x; r.kszb[1] = b0.y; r.kszb[2] = b0.z; r.kszb[3] = b0.w;
    r.kszb[4] = b1.x; r.kszb[5] = b1.y; r.kszb[6] = b1.z; r.kszb[7] = b1.w;
    const uint32_t *vsz = reinterpret_cast<const uint32_t *>(base + PL::kVSz);
    r.vszw[0] = vsz[kValueGroups * t0 + a];
    r.vszw[1] = vsz[kValueGroups * t1 + a];
}

template <int KB, int VB, int GS, typename QT>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeParams p)
{
    using PL = PageLayout<KB, VB>;
    __shared__ DecodeSmem<GS> sm;
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int G = p.G;
    const long long bh = static_cast<long long>(b) * p.H + h;
    float *out_bh = p.out + bh * G * kHeadDim;
    float *lse_bh = p.lse ? p.lse + bh * G : nullptr;
    const int L = p.seq_len[b];

    const bool bad_len = L < 0 || L > p.max_seq_len || L > kGroup * p.max_pages;
    if (bad_len || L == 0) {
        if (split == 0) {
            const float o = bad_len ? NAN : 0.0f;
            for (int i = tid; i < G * kHeadDim; i += kThreads) out_bh[i] = o;
            if (lse_bh && tid < G) lse_bh[tid] = bad_len ? NAN : -INFINITY;
        }
        return;
    }
    const int full = L / kGroup, nres = L % kGroup;
    const int P = p.pages_per_split;
    const int n_ps = (full + P - 1) / P;
    const int expected = n_ps + (nres > 0 ? 1 : 0);
    if (split >= expected) return;
    const long long slot = bh * p.n_splits + split;

    // q, scaled to log2 units and normalized per head to |q~| in [1, 2)
    for (int i = tid; i < G * kHeadDim; i += kThreads)
        sm.qs[i / kHeadDim][i % kHeadDim] = load_q<QT>(p.q, bh * G * kHeadDim + i) * kScoreScale;
    __syncthreads();
    if (tid < G) {
        float mx = 0.0f;
        for (int c = 0; c < kHeadDim; ++c) mx = fmaxf(mx, fabsf(sm.qs[tid][c]));
        int e = 0;
        if (mx > 0.0f) frexpf(mx, &e);
        sm.eq[tid] = 1 - e;
    }
    __syncthreads();
    for (int i = tid; i < G * kHeadDim; i += kThreads)
        sm.qs[i / kHeadDim][i % kHeadDim] = ldexpf(sm.qs[i / kHeadDim][i % kHeadDim], sm.eq[i / kHeadDim]);
    __syncthreads();

    if (split == n_ps) {
        residual_split<GS>(p, sm, bh, nres, G, slot);
    } else {
        const int wave = tid >> 6, lane = tid & 63;
        const int a = lane >> 4, r16 = lane & 15;
        WaveLds<GS> &W = sm.u.w[wave];
        // zero rows (A operands of rows whose head is >= G)
        for (int i = lane; i < 64; i += 64) {
            W.qp[0][4 * GS][i] = 0u;
            W.qp[1][4 * GS][i] = 0u;
        }
        for (int i = lane; i < 4 * 16; i += 64) {
            W.pp[0][i / 16][4 * GS][i % 16] = 0u;
            W.pp[1][i / 16][4 * GS][i % 16] = 0u;
        }
        // lane roles
        const int hr = 4 * (r16 & 3) + (r16 >> 2);             // head of A row r16
        const int arow = hr < G ? hr : 4 * GS;                  // zero row when absent
        const int kq = lane >> 4, kjj = (lane >> 2) & 3, kj = lane & 3;   // key pair this lane folds
        const int ch0 = 32 * kq + key_pair_channel<KB>(kjj, kj);
        const int ch1 = ch0 + 16 / KB;
        const int t0 = 8 * (r16 >> 2) + (r16 & 3), t1 = t0 + 4;   // value pair this lane folds (group a)
        float qw[4 * GS][2];                                      // q~ of the folded key pair, every head
#pragma unroll
        for (int hh = 0; hh < 4 * GS; ++hh) {
            qw[hh][0] = hh < G ? sm.qs[hh][ch0] : 0.0f;
            qw[hh][1] = hh < G ? sm.qs[hh][ch1] : 0.0f;
        }
        float qb[GS][8];                                          // q~ of the zero-term channels
        float eqs[GS];
#pragma unroll
        for (int i = 0; i < GS; ++i) {
            const int hh = 4 * i + a;
#pragma unroll
            for (int x = 0; x < 8; ++x) qb[i][x] = hh < G ? sm.qs[hh][8 * r16 + x] : 0.0f;
            eqs[i] = hh < G ? static_cast<float>(sm.eq[hh]) : 0.0f;
        }

        float4_t acc[8];
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) acc[nb] = float4_t{0.f, 0.f, 0.f, 0.f};
        float m_run[GS], l_part[GS];
#pragma unroll
        for (int i = 0; i < GS; ++i) {
            m_run[i] = -INFINITY;
            l_part[i] = 0.0f;
        }
        float zb[4 * GS];
#pragma unroll
        for (int hh = 0; hh < 4 * GS; ++hh) zb[hh] = 0.0f;
        // The value accumulators hold sum_t (p s 2^ev) v: ev keeps the folded weights in the
        // normal fp16 range (|p s 2^ev| < 2^15); it only decreases, rescaling acc when it does.
        int ev = 127;
        bool bad_page = false;

        const int pg_begin = split * P + wave;
        const int pg_end = min(full, (split + 1) * P);
        const uint8_t *pool = static_cast<const uint8_t *>(p.pages);
        // physical ids of this wave's pages (pg_begin + 4j, j < 64), one per lane
        const int n_my = pg_begin < pg_end ? (pg_end - pg_begin + kWaves - 1) / kWaves : 0;
        int my_phys = 0;
        if (lane < n_my) my_phys = p.block_table[static_cast<long long>(b) * p.max_pages + pg_begin + kWaves * lane];
        auto page_base = [&](int j, bool &ok) -> const uint8_t * {
            const int phys = __builtin_amdgcn_readlane(my_phys, j);
            ok = phys >= 0 && phys < p.n_pages;
            return pool + (static_cast<long long>(ok ? phys : 0) * p.H + h) * PL::kBytes;
        };

        PageRegs<KB, VB> cur, nxt;
        if (n_my > 0) {
            bool ok;
            const uint8_t *base = page_base(0, ok);
            bad_page |= !ok;
            load_page<KB, VB>(cur, base, lane, ch0, ch1, t0, t1);
        }
        for (int j = 0; j < n_my; ++j) {
            if (j + 1 < n_my) {
                bool ok;
                const uint8_t *base = page_base(j + 1, ok);
                bad_page |= !ok;
                load_page<KB, VB>(nxt, base, lane, ch0, ch1, t0, t1);
            }
            // ---- page exponent: |q~ s 2^E| < 2^15 for every channel ---------------
            uint32_t smax = 0;
#pragma unroll
            for (int x = 0; x < 8; ++x) smax = max(smax, cur.kszb[x] & 0x7FFFu);
            smax = row_max_u32(smax);
            int E = 0;
            {
                const float sm_f = half_bits_to_float(smax);
                if (sm_f > 0.0f) {
                    int e;
                    frexpf(sm_f, &e);
                    E = 14 - e;
                }
            }
            // ---- fold key scales into q: two channels x every head, hi/lo ------------
            {
                const float s0 = ldexpf(half_bits_to_float(cur.kszw[0] & 0xFFFFu), E);
                const float s1 = ldexpf(half_bits_to_float(cur.kszw[1] & 0xFFFFu), E);
#pragma unroll
                for (int hh = 0; hh < 4 * GS; ++hh) {
                    if (hh < G) {
                        const uint32_t hi = split_hi(qw[hh][0] * s0, qw[hh][1] * s1);
                        W.qp[0][hh][lane] = hi;
                        W.qp[1][hh][lane] = split_lo(qw[hh][0], s0, qw[hh][1], s1, hi);
                    }
                }
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
            float4_t sacc[2] = {float4_t{0.f, 0.f, 0.f, 0.f}, float4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const uint4 ahi = *reinterpret_cast<const uint4 *>(&W.qp[0][arow][16 * a + 4 * jj]);
                const uint4 alo = *reinterpret_cast<const uint4 *>(&W.qp[1][arow][16 * a + 4 * jj]);
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) {
                    const uint4 bk = unpack_operand_normal<KB>(cur.kc[blk], jj);
                    sacc[blk] = mfma(ahi, bk, sacc[blk]);
                    sacc[blk] = mfma(alo, bk, sacc[blk]);
                }
            }
            // ---- online softmax ------------------------------------------------------
            float s2[2][GS];
            bool grow = false;
#pragma unroll
            for (int i = 0; i < GS; ++i) {
                const float sc = ldexpf(1.0f, -E) * exp2f(-eqs[i]);
                const float bc = bias[i] * exp2f(-eqs[i]);
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) {
                    s2[blk][i] = fmaf(sacc[blk][i], sc, bc);
                    grow |= (4 * i + a < G) && s2[blk][i] > m_run[i];
                }
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
                    for (int nb = 0; nb < 8; ++nb) acc[nb][i] *= alpha[i];
                    if (r16 == 0 && 4 * i + a < G) W.alpha[4 * i + a] = alpha[i];
                }
                wave_lds_sync();
#pragma unroll
                for (int hh = 0; hh < 4 * GS; ++hh)
                    if (hh < G) zb[hh] *= W.alpha[hh];
            }
#pragma unroll
            for (int i = 0; i < GS; ++i) {
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) {
                    const float pv = __builtin_amdgcn_exp2f(s2[blk][i] - m_run[i]);
                    l_part[i] += pv;
                    if (4 * i + a < G) W.p[16 * blk + r16][4 * i + a] = pv;
                }
            }
            wave_lds_sync();
            // ---- value-scale exponent of this page -----------------------------------
            {
                uint32_t vmax = max(cur.vszw[0] & 0x7FFFu, cur.vszw[1] & 0x7FFFu);
                vmax = row_max_u32(vmax);
                vmax = max(vmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(vmax), 16)));
                vmax = max(vmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(vmax), 32)));
                if (vmax != 0u) {
                    int e;
                    frexpf(half_bits_to_float(vmax), &e);
                    const int ev_page = 14 - e;
                    if (ev_page < ev) {
                        const float f = ldexpf(1.0f, ev_page - ev);
#pragma unroll
                        for (int nb = 0; nb < 8; ++nb) acc[nb] *= f;
                        ev = ev_page;
                    }
                }
            }
            // ---- fold value scales into p: two tokens x every head, hi/lo --------------
            {
                const float sv0 = ldexpf(half_bits_to_float(cur.vszw[0] & 0xFFFFu), ev);
                const float sv1 = ldexpf(half_bits_to_float(cur.vszw[1] & 0xFFFFu), ev);
                const float zv0 = half_bits_to_float(cur.vszw[0] >> 16);
                const float zv1 = half_bits_to_float(cur.vszw[1] >> 16);
#pragma unroll
                for (int hh = 0; hh < 4 * GS; ++hh) {
                    if (hh < G) {
                        const float p0 = W.p[t0][hh], p1 = W.p[t1][hh];
                        const uint32_t hi = split_hi(p0 * sv0, p1 * sv1);
                        W.pp[0][a][hh][r16] = hi;
                        W.pp[1][a][hh][r16] = split_lo(p0, sv0, p1, sv1, hi);
                        zb[hh] = fmaf(p0, zv0, fmaf(p1, zv1, zb[hh]));
                    }
                }
            }
            wave_lds_sync();
            // ---- values on MFMA ------------------------------------------------------
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const uint4 ahi = *reinterpret_cast<const uint4 *>(&W.pp[0][g][arow][4 * a]);
                const uint4 alo = *reinterpret_cast<const uint4 *>(&W.pp[1][g][arow][4 * a]);
#pragma unroll
                for (int nb = 2 * g; nb < 2 * g + 2; ++nb) {
                    const uint4 bv = unpack_operand_normal<VB>(cur.vc, nb);
                    acc[nb] = mfma(ahi, bv, acc[nb]);
                    acc[nb] = mfma(alo, bv, acc[nb]);
                }
            }
            cur = nxt;
        }

        // ---- this wave's state: l per head, value zero terms, unnormalized output -------
        float lw[GS];
#pragma unroll
        for (int i = 0; i < GS; ++i) lw[i] = row_sum(l_part[i]);
#pragma unroll
        for (int hh = 0; hh < 4 * GS; ++hh) {
            if (hh < G) {
                const float v = row_sum(zb[hh]);    // lanes of group a cover all 32 tokens once
                if (r16 == 0) W.bv[a][hh] = v;
            }
        }
        wave_lds_sync();
        float o_out[8][GS];
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
#pragma unroll
            for (int i = 0; i < GS; ++i) {
                const int hh = 4 * i + a;
                o_out[nb][i] = hh < G ? fmaf(acc[nb][i], ldexpf(1.0f, -ev), W.bv[nb >> 1][hh]) : 0.0f;
            }
        __syncthreads();     // every wave is done with its WaveLds: reuse the space to merge
        MergeLds<GS> &M = sm.u.merge;
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
        __syncthreads();
        float *part_o = p.part_o + slot * G * kHeadDim;
        float *part_ml = p.part_ml + slot * G * 2;
        const bool bad = __syncthreads_or(bad_page);
        for (int idx = tid; idx < G * kHeadDim; idx += kThreads) {
            const int hh = idx / kHeadDim, c = idx % kHeadDim;
            float m = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) m = fmaxf(m, M.m[w][hh]);
            float l = 0.0f, o = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float wt = M.m[w][hh] == -INFINITY ? 0.0f : exp2f(M.m[w][hh] - m);
                l = fmaf(wt, M.l[w][hh], l);
                o = fmaf(wt, M.o[w][hh][c], o);
            }
            store_dev(&part_o[idx], bad ? NAN : o);
            if (c == 0) {
                store_dev(&part_ml[2 * hh], bad ? 0.0f : m);
                store_dev(&part_ml[2 * hh + 1], bad ? NAN : l);
            }
        }
    }

    wait_stores();
    __syncthreads();
    if (tid == 0)
        sm.last = __hip_atomic_fetch_add(p.counters + bh, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == expected - 1;
    __syncthreads();
    if (!sm.last) return;
    combine_splits(p, bh, expected, G, out_bh, lse_bh);
    if (tid == 0) __hip_atomic_store(p.counters + bh, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void zero_fill_kernel(uint32_t *p, size_t n_words)
{
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n_words;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        p[i] = 0u;
}

template <int KB, int VB, int GS>
hipError_t launch_decode_g(const DecodeParams &p, bool q_f32, hipStream_t s)
{
    dim3 grid(p.n_splits, p.H, p.batch);
    if (q_f32)
        hipLaunchKernelGGL((decode_kernel<KB, VB, GS, float>), grid, dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((decode_kernel<KB, VB, GS, uint16_t>), grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <int KB, int VB>
hipError_t launch_decode_t(const DecodeParams &p, bool q_f32, hipStream_t s)
{
    if (p.G <= 4) return launch_decode_g<KB, VB, 1>(p, q_f32, s);
    if (p.G <= 8) return launch_decode_g<KB, VB, 2>(p, q_f32, s);
    return launch_decode_g<KB, VB, 4>(p, q_f32, s);
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

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

int decode_default_pages_per_split(int batch, int H, int max_full_pages)
{
    // about 1024 workgroups of four waves for the longest sequences, at least four pages
    // per wave, at most 128 pages per split
    const long long work = static_cast<long long>(batch) * H * (max_full_pages > 0 ? max_full_pages : 1);
    long long pps = (work + 1023) / 1024;
    pps = (pps + kWaves - 1) / kWaves * kWaves;
    if (pps < 4 * kWaves) pps = 4 * kWaves;
    if (pps > 128) pps = 128;   // at most 32 pages per wave (block-table ids held one per lane)
    return static_cast<int>(pps);
}

int decode_max_g() { return 4 * kMaxGS; }

hipError_t launch_decode(int kb, int vb, const DecodeParams &p, bool q_f32, hipStream_t s)
{
#define KVQ_P(KBV, VBV) if (kb == KBV && vb == VBV) return launch_decode_t<KBV, VBV>(p, q_f32, s)
    KVQ_P(2, 2); KVQ_P(2, 4); KVQ_P(2, 8);
    KVQ_P(4, 2); KVQ_P(4, 4); KVQ_P(4, 8);
    KVQ_P(8, 2); KVQ_P(8, 4); KVQ_P(8, 8);
#undef KVQ_P
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

}  // namespace kvq
