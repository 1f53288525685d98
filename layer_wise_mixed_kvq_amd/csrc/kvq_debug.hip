// kvq_debug.hip -- the KVQ_DEBUG checks: with the environment variable KVQ_DEBUG set (to
// anything but "" or "0") every entry point first checks what only the device holds --
// lengths and positions against the block table, block-table ids against the pool, and
// input values against the domain (finite, |x| <= 65504 for K / V, finite q, positive
// finite FP8 scales) -- and returns KVQ_ERR_INVALID_ARG without launching its kernel when
// a check fails.  The checks copy the lengths and block table to the host and count
// out-of-domain values on the device into one counter per GPU, so a checked call waits
// for its stream; it must not be captured into a graph, and checked calls on several
// streams of one GPU at once share that counter.  Without KVQ_DEBUG nothing here runs.
#include <stdint.h>
#include <stdlib.h>

#include <vector>

#include "kvq_debug.h"

namespace kvq {
namespace {

constexpr float kMaxAbs = 65504.0f;   // fp16 range: scales and zeros stay finite

__device__ unsigned long long g_out_of_domain;

__device__ __forceinline__ float elem(const void *p, long long i, bool f32)
{
    if (f32) return static_cast<const float *>(p)[i];
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(p)[i]) << 16);
}

__device__ __forceinline__ bool in_domain(float x, bool limit) { return limit ? fabsf(x) <= kMaxAbs : x - x == 0.0f; }

// rows [0, rows(b)) of x[b] ([batch][row_stride_rows][row_elems]), rows(b) = lens[b] + len_add
// (all max_rows when lens is null); counts values outside the domain
__global__ void count_kernel(const void *x, bool f32, const int32_t *lens, int len_add, int max_rows,
                             long long row_elems, bool limit)
{
    const int b = blockIdx.y;
    const int rows = lens ? min(lens[b] + len_add, max_rows) : max_rows;
    const long long n = static_cast<long long>(rows) * row_elems;
    const long long base = static_cast<long long>(b) * max_rows * row_elems;
    unsigned long long bad = 0;
    for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<long long>(gridDim.x) * blockDim.x)
        bad += in_domain(elem(x, base + i, f32), limit) ? 0u : 1u;
    if (bad) atomicAdd(&g_out_of_domain, bad);
}

bool hip_ok(hipError_t e) { return e == hipSuccess; }

// counts over every listed region, then waits for the stream; -1 on a HIP error
struct Counter {
    hipStream_t s;
    bool ok;
    explicit Counter(hipStream_t st) : s(st), ok(true)
    {
        static const unsigned long long zero = 0;   // outlives the asynchronous copy
        ok = hip_ok(hipMemcpyToSymbolAsync(HIP_SYMBOL(g_out_of_domain), &zero, sizeof(zero), 0,
                                           hipMemcpyHostToDevice, s));
    }
    void add(const void *x, bool f32, const int32_t *lens, int len_add, int batch, int max_rows, long long row_elems,
             bool limit)
    {
        if (!ok || batch <= 0 || max_rows <= 0) return;
        const long long total = static_cast<long long>(max_rows) * row_elems;
        const int gx = static_cast<int>(min(1024LL, (total + 255) / 256));
        hipLaunchKernelGGL(count_kernel, dim3(gx, batch), dim3(256), 0, s, x, f32, lens, len_add, max_rows, row_elems,
                           limit);
        ok = hip_ok(hipGetLastError());
    }
    long long finish()
    {
        unsigned long long n = 0;
        if (ok) ok = hip_ok(hipMemcpyFromSymbolAsync(&n, HIP_SYMBOL(g_out_of_domain), sizeof(n), 0,
                                                     hipMemcpyDeviceToHost, s));
        if (ok) ok = hip_ok(hipStreamSynchronize(s));
        return ok ? static_cast<long long>(n) : -1;
    }
};

template <typename T>
bool fetch(std::vector<T> &dst, const T *src, size_t n, hipStream_t s)
{
    dst.resize(n);
    if (n == 0) return true;
    return hip_ok(hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, s)) &&
           hip_ok(hipStreamSynchronize(s));
}

// block-table ids of pages [0, n_used) of every sequence inside [0, n_pages)
bool ids_ok(const std::vector<int32_t> &bt, int b, int n_used, int max_pages, long long n_pages)
{
    for (int i = 0; i < n_used; ++i) {
        const int32_t id = bt[static_cast<size_t>(b) * max_pages + i];
        if (id < 0 || id >= n_pages) return false;
    }
    return true;
}

kvq_status scales_ok(const float *scales, int H, hipStream_t s)
{
    if (!scales) return KVQ_OK;
    std::vector<float> sc;
    if (!fetch(sc, scales, static_cast<size_t>(2) * H, s)) return KVQ_ERR_HIP;
    for (float x : sc)
        if (!(x > 0.0f) || x - x != 0.0f) return KVQ_ERR_INVALID_ARG;
    return KVQ_OK;
}

kvq_status from_count(long long n)
{
    if (n < 0) return KVQ_ERR_HIP;
    return n == 0 ? KVQ_OK : KVQ_ERR_INVALID_ARG;
}

}  // namespace

bool debug_checks_enabled()
{
    const char *v = getenv("KVQ_DEBUG");
    return v && v[0] != '\0' && !(v[0] == '0' && v[1] == '\0');
}

kvq_status debug_check_pack(const PackParams &p, bool src_f32, hipStream_t s)
{
    std::vector<int32_t> len, bt;
    if (!fetch(len, p.seq_len, static_cast<size_t>(p.batch), s)) return KVQ_ERR_HIP;
    if (!fetch(bt, p.block_table, static_cast<size_t>(p.batch) * p.max_pages, s)) return KVQ_ERR_HIP;
    for (int b = 0; b < p.batch; ++b) {
        const int L = len[b];
        if (L < 0 || L > p.max_tokens || L > kGroupTokens * p.max_pages) return KVQ_ERR_INVALID_ARG;
        if (!ids_ok(bt, b, L / kGroupTokens, p.max_pages, p.n_pages)) return KVQ_ERR_INVALID_ARG;
    }
    const kvq_status sc = scales_ok(p.scales, p.H, s);
    if (sc != KVQ_OK) return sc;
    Counter c(s);
    const long long row = static_cast<long long>(p.H) * kHeadDimElems;
    c.add(p.k_src, src_f32, p.seq_len, 0, p.batch, p.max_tokens, row, true);
    c.add(p.v_src, src_f32, p.seq_len, 0, p.batch, p.max_tokens, row, true);
    return from_count(c.finish());
}

kvq_status debug_check_append(const AppendParams &p, hipStream_t s)
{
    std::vector<int32_t> pos, bt;
    if (!fetch(pos, p.pos, static_cast<size_t>(p.batch), s)) return KVQ_ERR_HIP;
    if (!fetch(bt, p.block_table, static_cast<size_t>(p.batch) * p.max_pages, s)) return KVQ_ERR_HIP;
    for (int b = 0; b < p.batch; ++b) {
        const int t = pos[b];
        if (t < 0 || t >= kGroupTokens * p.max_pages) return KVQ_ERR_INVALID_ARG;
        // a flush writes page t / 32
        if (t % kGroupTokens == kGroupTokens - 1 && !ids_ok(bt, b, t / kGroupTokens + 1, p.max_pages, p.n_pages))
            return KVQ_ERR_INVALID_ARG;
    }
    const kvq_status sc = scales_ok(p.scales, p.H, s);
    if (sc != KVQ_OK) return sc;
    Counter c(s);
    const long long row = static_cast<long long>(p.H) * kHeadDimElems;
    c.add(p.k_new, false, nullptr, 0, p.batch, 1, row, true);
    c.add(p.v_new, false, nullptr, 0, p.batch, 1, row, true);
    return from_count(c.finish());
}

kvq_status debug_check_decode(const DecodeParams &p, bool q_f32, hipStream_t s)
{
    const bool fused = p.pos != nullptr;
    std::vector<int32_t> len, bt;
    if (!fetch(len, fused ? p.pos : p.seq_len, static_cast<size_t>(p.batch), s)) return KVQ_ERR_HIP;
    if (!fetch(bt, p.block_table, static_cast<size_t>(p.batch) * p.max_pages, s)) return KVQ_ERR_HIP;
    for (int b = 0; b < p.batch; ++b) {
        const long long L = fused ? static_cast<long long>(len[b]) + 1 : len[b];
        if ((fused ? L <= 0 : L < 0) || L > p.max_seq_len || L > static_cast<long long>(kGroupTokens) * p.max_pages)
            return KVQ_ERR_INVALID_ARG;
        // pages read (and, for a fused flush, the page written): 0 .. L/32 - 1
        if (!ids_ok(bt, b, static_cast<int>(L / kGroupTokens), p.max_pages, p.n_pages)) return KVQ_ERR_INVALID_ARG;
    }
    const kvq_status sc = scales_ok(p.scales, p.H, s);
    if (sc != KVQ_OK) return sc;
    Counter c(s);
    c.add(p.q, q_f32, nullptr, 0, p.batch, 1, static_cast<long long>(p.H) * p.G * kHeadDimElems, false);
    if (fused) {
        const long long row = static_cast<long long>(p.H) * kHeadDimElems;
        c.add(p.k_new, false, nullptr, 0, p.batch, 1, row, true);
        c.add(p.v_new, false, nullptr, 0, p.batch, 1, row, true);
    }
    return from_count(c.finish());
}

kvq_status debug_check_dequant(const DequantParams &p, hipStream_t s)
{
    std::vector<int32_t> len, bt;
    if (!fetch(len, p.seq_len, static_cast<size_t>(p.batch), s)) return KVQ_ERR_HIP;
    if (!fetch(bt, p.block_table, static_cast<size_t>(p.batch) * p.max_pages, s)) return KVQ_ERR_HIP;
    for (int b = 0; b < p.batch; ++b) {
        const int L = len[b];
        if (L < 0 || L > p.max_tokens || L > kGroupTokens * p.max_pages) return KVQ_ERR_INVALID_ARG;
        if (!ids_ok(bt, b, L / kGroupTokens, p.max_pages, p.n_pages)) return KVQ_ERR_INVALID_ARG;
    }
    return scales_ok(p.scales, p.H, s);
}

}  // namespace kvq
