// kvq_decode.hip -- single-token decode attention over the packed mixed-precision cache
// (gfx950), split-K over 32-token pages with an online-softmax combine.
//
// Method: attention over the dequantized cache, FlashAttention-compatible (online softmax),
// with GQA (query head hq reads KV head hq / G); attention is memory-bound, so time follows
// the KV bytes moved.
//   [KVTuner OpenReview discussion (paperhub.cn/paper/zDwipF6h06), reply to reviewer 2,
//    section 1 "Efficiency evaluation clarifications"; reply to reviewer 3, section 2
//    "Latency experiment"; reply to reviewer 3, section 6 "MHA"]
//
// Work decomposition: one workgroup per (split, KV head, sequence).  Split s < n_ps covers
// pages [s*P, min((s+1)*P, full)); split n_ps (when L mod 32 > 0) covers the bf16 residual.
// Every split writes (m, l, o[128]) per query head to the workspace; the last split of a
// (sequence, KV head) to finish -- a device-scope counter -- merges them:
//   m = max m_s, l = sum 2^(m_s - m) l_s, out = sum 2^(m_s - m) o_s / l, lse = (m + log2 l) ln 2
// and resets the counter to zero for the next call.  Scores are kept in log2 units
// (q is pre-scaled by log2(e)/sqrt(128)).
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kMaxG = 8;
constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kScoreScale = kLog2e * 0.08838834764831845f;   // log2(e) / sqrt(128)

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
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

struct DecodeSmem {
    float q[kMaxG][kHeadDim];
    float2 ksz[kHeadDim];
    float2 vsz[kGroup][kValueGroups];
    float p[kMaxG][kGroup];
    int last;
};

struct SoftmaxState {
    float m[kMaxG];
    float l[kMaxG];
    float acc[kMaxG][2];
};

// Online-softmax update for one block of 32 tokens held two lanes per token (lane 2t and
// 2t+1 hold the same score of token t).  Writes the block's weights to sm.p and rescales
// the running accumulators.
__device__ __forceinline__ void softmax_block(SoftmaxState &st, const float (&s)[kMaxG], bool valid, int G,
                                              DecodeSmem &sm)
{
    const int lane = threadIdx.x;
#pragma unroll
    for (int g = 0; g < kMaxG; ++g) {
        if (g >= G) break;
        const float sv = valid ? s[g] : -INFINITY;
        const float mp = wave_max(sv);
        const float m_new = fmaxf(st.m[g], mp);
        const float alpha = exp2f(st.m[g] - m_new);
        const float pv = valid ? exp2f(sv - m_new) : 0.0f;
        const float psum = wave_sum((lane & 1) ? 0.0f : pv);
        st.l[g] = st.l[g] * alpha + psum;
        st.m[g] = m_new;
        st.acc[g][0] *= alpha;
        st.acc[g][1] *= alpha;
        if (!(lane & 1)) sm.p[g][lane >> 1] = pv;
    }
}

template <int KB, int VB, typename QT>
__global__ __launch_bounds__(kWave) void decode_kernel(DecodeParams p)
{
    using PL = PageLayout<KB, VB>;
    __shared__ DecodeSmem sm;
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    const int G = p.G;
    const long long bh = static_cast<long long>(b) * p.H + h;
    float *out_bh = p.out + bh * G * kHeadDim;
    float *lse_bh = p.lse ? p.lse + bh * G : nullptr;
    const int L = p.seq_len[b];

    const bool bad_len = L < 0 || L > p.max_seq_len || L > kGroup * p.max_pages;
    if (bad_len || L == 0) {
        if (split == 0) {
            const float o = bad_len ? NAN : 0.0f;
            for (int i = lane; i < G * kHeadDim; i += kWave) out_bh[i] = o;
            if (lse_bh && lane < G) lse_bh[lane] = bad_len ? NAN : -INFINITY;
        }
        return;
    }
    const int full = L / kGroup, nres = L % kGroup;
    const int P = p.pages_per_split;
    const int n_ps = (full + P - 1) / P;
    const int expected = n_ps + (nres > 0 ? 1 : 0);
    if (split >= expected) return;
    const bool is_resid = split == n_ps;

    for (int i = lane; i < G * kHeadDim; i += kWave)
        sm.q[i / kHeadDim][i % kHeadDim] = load_q<QT>(p.q, bh * G * kHeadDim + i) * kScoreScale;
    __syncthreads();

    SoftmaxState st;
#pragma unroll
    for (int g = 0; g < kMaxG; ++g) {
        st.m[g] = -INFINITY;
        st.l[g] = 0.0f;
        st.acc[g][0] = st.acc[g][1] = 0.0f;
    }
    bool bad_page = false;
    const int t = lane >> 1, hf = lane & 1;
    const int c0 = 2 * lane;

    if (!is_resid) {
        const int pg_end = min(full, (split + 1) * P);
        for (int pg = split * P; pg < pg_end; ++pg) {
            const int phys = p.block_table[static_cast<long long>(b) * p.max_pages + pg];
            if (phys < 0 || phys >= p.n_pages) {
                bad_page = true;
                break;
            }
            const uint8_t *base = static_cast<const uint8_t *>(p.pages) +
                                  (static_cast<long long>(phys) * p.H + h) * PL::kBytes;
            const uint32_t *ksz = reinterpret_cast<const uint32_t *>(base + PL::kKSz);
            const uint32_t *vsz = reinterpret_cast<const uint32_t *>(base + PL::kVSz);
            for (int i = lane; i < kHeadDim; i += kWave) {
                const uint32_t w = ksz[i];
                sm.ksz[i] = make_float2(half_bits_to_float(w & 0xFFFFu), half_bits_to_float(w >> 16));
                const uint32_t u = vsz[i];
                sm.vsz[i / kValueGroups][i % kValueGroups] =
                    make_float2(half_bits_to_float(u & 0xFFFFu), half_bits_to_float(u >> 16));
            }
            __syncthreads();
            // scores: lane (t, hf) covers channels 64*hf .. 64*hf+63 of token t
            uint32_t kw[2 * KB];
            const uint32_t *krow = reinterpret_cast<const uint32_t *>(base + PL::kKCodes + t * PL::kKRowBytes) + hf * 2 * KB;
#pragma unroll
            for (int i = 0; i < 2 * KB; ++i) kw[i] = krow[i];
            float s[kMaxG];
#pragma unroll
            for (int g = 0; g < kMaxG; ++g) s[g] = 0.0f;
#pragma unroll 8
            for (int c = 0; c < 64; ++c) {
                const int cc = hf * 64 + c;
                const uint32_t code = (kw[(c * KB) >> 5] >> ((c * KB) & 31)) & ((1u << KB) - 1u);
                const float2 sz = sm.ksz[cc];
                const float kv = fmaf(static_cast<float>(code), sz.x, sz.y);
#pragma unroll
                for (int g = 0; g < kMaxG; ++g)
                    if (g < G) s[g] = fmaf(sm.q[g][cc], kv, s[g]);
            }
#pragma unroll
            for (int g = 0; g < kMaxG; ++g)
                if (g < G) s[g] += __shfl_xor(s[g], 1);
            softmax_block(st, s, true, G, sm);
            __syncthreads();
            // values: lane owns channels c0, c0 + 1 (rows c0, c0+1 of the channel-major codes)
            uint32_t vw[2 * VB];
            const uint32_t *vrow = reinterpret_cast<const uint32_t *>(base + PL::kVCodes + c0 * PL::kVRowBytes);
#pragma unroll
            for (int i = 0; i < 2 * VB; ++i) vw[i] = vrow[i];
            const int j = c0 / kGroup;
#pragma unroll 4
            for (int tt = 0; tt < kGroup; ++tt) {
                const float2 sz = sm.vsz[tt][j];
                const uint32_t mask = (1u << VB) - 1u;
                const uint32_t code0 = (vw[(tt * VB) >> 5] >> ((tt * VB) & 31)) & mask;
                const uint32_t code1 = (vw[VB + ((tt * VB) >> 5)] >> ((tt * VB) & 31)) & mask;
                const float v0 = fmaf(static_cast<float>(code0), sz.x, sz.y);
                const float v1 = fmaf(static_cast<float>(code1), sz.x, sz.y);
#pragma unroll
                for (int g = 0; g < kMaxG; ++g) {
                    if (g < G) {
                        const float pw = sm.p[g][tt];
                        st.acc[g][0] = fmaf(pw, v0, st.acc[g][0]);
                        st.acc[g][1] = fmaf(pw, v1, st.acc[g][1]);
                    }
                }
            }
            __syncthreads();
        }
    } else {
        const uint16_t *rk = p.resid_k + bh * kGroup * kHeadDim;
        const uint16_t *rv = p.resid_v + bh * kGroup * kHeadDim;
        float s[kMaxG];
#pragma unroll
        for (int g = 0; g < kMaxG; ++g) s[g] = 0.0f;
        const bool valid = t < nres;
        if (valid) {
            for (int c = 0; c < 64; ++c) {
                const int cc = hf * 64 + c;
                const float kv = bf16_bits_to_float(rk[t * kHeadDim + cc]);
#pragma unroll
                for (int g = 0; g < kMaxG; ++g)
                    if (g < G) s[g] = fmaf(sm.q[g][cc], kv, s[g]);
            }
        }
#pragma unroll
        for (int g = 0; g < kMaxG; ++g)
            if (g < G) s[g] += __shfl_xor(s[g], 1);
        softmax_block(st, s, valid, G, sm);
        __syncthreads();
        for (int tt = 0; tt < nres; ++tt) {
            const uint32_t w = *reinterpret_cast<const uint32_t *>(rv + tt * kHeadDim + c0);
            const float v0 = __uint_as_float(w << 16), v1 = __uint_as_float(w & 0xFFFF0000u);
#pragma unroll
            for (int g = 0; g < kMaxG; ++g) {
                if (g < G) {
                    const float pw = sm.p[g][tt];
                    st.acc[g][0] = fmaf(pw, v0, st.acc[g][0]);
                    st.acc[g][1] = fmaf(pw, v1, st.acc[g][1]);
                }
            }
        }
    }

    // this split's partial
    const long long slot = bh * p.n_splits + split;
#pragma unroll
    for (int g = 0; g < kMaxG; ++g) {
        if (g >= G) break;
        float2 o = make_float2(st.acc[g][0], st.acc[g][1]);
        if (bad_page) o = make_float2(NAN, NAN);
        *reinterpret_cast<float2 *>(p.part_o + (slot * G + g) * kHeadDim + c0) = o;
        if (lane == 0) {
            p.part_ml[(slot * G + g) * 2 + 0] = bad_page ? 0.0f : st.m[g];
            p.part_ml[(slot * G + g) * 2 + 1] = bad_page ? NAN : st.l[g];
        }
    }
    __threadfence();
    __syncthreads();
    if (lane == 0) sm.last = atomicAdd(p.counters + bh, 1) == expected - 1;
    __syncthreads();
    if (!sm.last) return;
    __threadfence();

    // last split of this (sequence, KV head): merge the partials
    const long long slot0 = bh * p.n_splits;
    for (int g = 0; g < G; ++g) {
        float m = -INFINITY;
        for (int sidx = 0; sidx < expected; ++sidx) m = fmaxf(m, p.part_ml[((slot0 + sidx) * G + g) * 2]);
        float l = 0.0f, o0 = 0.0f, o1 = 0.0f;
        for (int sidx = 0; sidx < expected; ++sidx) {
            const float ms = p.part_ml[((slot0 + sidx) * G + g) * 2];
            const float ls = p.part_ml[((slot0 + sidx) * G + g) * 2 + 1];
            const float w = exp2f(ms - m);
            const float2 os = *reinterpret_cast<const float2 *>(p.part_o + ((slot0 + sidx) * G + g) * kHeadDim + c0);
            l = fmaf(w, ls, l);
            o0 = fmaf(w, os.x, o0);
            o1 = fmaf(w, os.y, o1);
        }
        const float inv = 1.0f / l;
        *reinterpret_cast<float2 *>(out_bh + g * kHeadDim + c0) = make_float2(o0 * inv, o1 * inv);
        if (lse_bh && lane == 0) lse_bh[g] = (m + log2f(l)) * kLn2;
    }
    if (lane == 0) p.counters[bh] = 0;
}

__global__ void zero_fill_kernel(uint32_t *p, size_t n_words)
{
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n_words;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        p[i] = 0u;
}

template <int KB, int VB>
hipError_t launch_decode_t(const DecodeParams &p, bool q_f32, hipStream_t s)
{
    dim3 grid(p.n_splits, p.H, p.batch);
    if (q_f32)
        hipLaunchKernelGGL((decode_kernel<KB, VB, float>), grid, dim3(kWave), 0, s, p);
    else
        hipLaunchKernelGGL((decode_kernel<KB, VB, uint16_t>), grid, dim3(kWave), 0, s, p);
    return hipGetLastError();
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
    const long long work = static_cast<long long>(batch) * H * (max_full_pages > 0 ? max_full_pages : 1);
    long long pps = (work + 2047) / 2048;
    if (pps < 1) pps = 1;
    if (pps > 4096) pps = 4096;
    return static_cast<int>(pps);
}

int decode_max_g() { return kMaxG; }

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
