// kvq_quant.hip -- quantize-on-write kernels for gfx950: prefill pack and decode-time
// append (+ page flush).
//
// Method: keys are quantized per channel over 32-token groups, values per token over
// 32-channel groups, each group with an fp16 scale and an fp16 zero (asymmetric min/max);
// only newly generated tokens are quantized online, at their layer's pair.
//   [Mixed-precision KV-cache quantization per-layer sensitivity (llms-explorer.com), Facts]
//   [KVTuner OpenReview discussion (paperhub.cn/paper/zDwipF6h06), reply to reviewer 1,
//    section 4; reply to reviewer 2, section 2; reply to reviewer 3, section 1]
//
// One workgroup of 256 threads quantizes one page of one KV head: the 32 x 128 K and V
// tiles are staged in LDS (coalesced 16-byte loads; a bfloat16 source is staged as it is, an
// fp32 source as binary32), then the page codec of kvq_codec.h encodes and packs them.  Layers kept in
// FP8 (E4M3 of x / scale, one K and one V scale per KV head) or BF16 go through the
// floating-point page codec instead.
//   [When should you use mixed-precision KV caching to preserve accuracy in sensitive
//    transformer layers (machinoai.in), sections 1-2]
#include "kvq_codec.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = kCodecThreads;

// bf16 residual value of a source element (round to nearest even from fp32)
template <typename SrcT>
struct Src;

template <>
struct Src<uint16_t> {   // bf16 bit patterns
    __device__ static uint16_t to_bf16(uint16_t x) { return x; }
};

template <>
struct Src<float> {
    __device__ static uint16_t to_bf16(float x) { return float_to_bf16_bits(x); }
};

// Stage a 32-token tile whose token rows are `row_stride` elements apart, in the source's
// own element type (16-byte chunks, 16 or 32 threads per token row).
template <typename SrcT>
__device__ void stage_tile(const SrcT *__restrict__ src, long long row_stride, SrcT *tile)
{
    constexpr int V = 16 / sizeof(SrcT);
    constexpr int kChunks = kGroup * kHeadDim / V;
    constexpr int kStride = QuantSmemT<SrcT>::kStride;
    for (int i = threadIdx.x; i < kChunks; i += kThreads) {
        const int t = i / (kHeadDim / V);
        const int c = (i % (kHeadDim / V)) * V;
        const uint4 x = *reinterpret_cast<const uint4 *>(src + t * row_stride + c);
        if constexpr (sizeof(SrcT) == 2) {
            *reinterpret_cast<uint4 *>(&tile[t * kStride + c]) = x;
        } else {   // padded binary32 rows are not 16-byte aligned
            tile[t * kStride + c] = __uint_as_float(x.x);
            tile[t * kStride + c + 1] = __uint_as_float(x.y);
            tile[t * kStride + c + 2] = __uint_as_float(x.z);
            tile[t * kStride + c + 3] = __uint_as_float(x.w);
        }
    }
}

// One page-head from the staged tiles, in the layer's format (KM: layer code).
template <int KB, int VB, int KM, typename T>
__device__ __forceinline__ void encode_page(QuantSmemT<T> &sm, uint8_t *pages, const float *scales, int phys, int H, int h)
{
    uint8_t *dst = pages + (static_cast<long long>(phys) * H + h) * layer_page_bytes<KB, VB, KM>();
    if constexpr (is_float_layer(KM))
        quantize_page_float<KM>(sm, dst, scales ? scales[2 * h] : 1.0f, scales ? scales[2 * h + 1] : 1.0f);
    else
        quantize_page<KB, VB, false, KM == kLayerKeysPerToken>(sm, dst);
}

// grid: (n_kv_heads, pages covering max_tokens, batch), heads fastest, so that neighbouring
// workgroups read the H head slices of the same token rows; with more pages than a grid's y
// extent allows, (pages, n_kv_heads, batch)
template <int KB, int VB, int KM, typename SrcT>
__global__ __launch_bounds__(kThreads) void pack_kernel(PackParams p)
{
    __shared__ QuantSmemT<SrcT> sm;
    const int g = p.heads_fastest ? blockIdx.y : blockIdx.x, h = p.heads_fastest ? blockIdx.x : blockIdx.y;
    const int b = blockIdx.z;
    const int L = p.seq_len[b];
    if (L < 0 || L > p.max_tokens || L > kGroup * p.max_pages) return;
    const int full = L / kGroup;
    const SrcT *ks = static_cast<const SrcT *>(p.k_src);
    const SrcT *vs = static_cast<const SrcT *>(p.v_src);
    const long long row_stride = static_cast<long long>(p.H) * kHeadDim;
    const long long base = ((static_cast<long long>(b) * p.max_tokens + static_cast<long long>(g) * kGroup) * p.H + h) *
                           kHeadDim;
    if (g < full) {
        const int phys = p.block_table[static_cast<long long>(b) * p.max_pages + g];
        if (phys < 0 || phys >= p.n_pages) return;
        stage_tile<SrcT>(ks + base, row_stride, sm.k);
        stage_tile<SrcT>(vs + base, row_stride, sm.v);
        __syncthreads();
        encode_page<KB, VB, KM>(sm, static_cast<uint8_t *>(p.pages), p.scales, phys, p.H, h);
    } else if (g == full) {
        // trailing L mod 32 tokens -> bf16 residual slots 0 .. L mod 32 - 1
        const int nres = L - full * kGroup;
        const long long rbase = (static_cast<long long>(b) * p.H + h) * kGroup * kHeadDim;
        for (int i = threadIdx.x; i < nres * kHeadDim; i += kThreads) {
            const int t = i / kHeadDim, c = i % kHeadDim;
            const long long si = base + t * row_stride + c;
            p.resid_k[rbase + i] = Src<SrcT>::to_bf16(ks[si]);
            p.resid_v[rbase + i] = Src<SrcT>::to_bf16(vs[si]);
        }
    }
}

// grid: (n_kv_heads, batch)
template <int KB, int VB, int KM>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendParams p)
{
    __shared__ QuantSmemT<uint16_t> sm;
    const int h = blockIdx.x, b = blockIdx.y;
    const int pos = p.pos[b];
    if (pos < 0 || pos >= kGroup * p.max_pages) return;
    const int slot = pos % kGroup;
    const long long nb = (static_cast<long long>(b) * p.H + h) * kHeadDim;
    const long long rbase = (static_cast<long long>(b) * p.H + h) * kGroup * kHeadDim;
    const int tid = threadIdx.x;
    // the new token into its residual slot (threads 0..127: K, 128..255: V)
    if (tid < kHeadDim)
        p.resid_k[rbase + slot * kHeadDim + tid] = p.k_new[nb + tid];
    else
        p.resid_v[rbase + slot * kHeadDim + tid - kHeadDim] = p.v_new[nb + tid - kHeadDim];
    if (slot != kGroup - 1) return;
    // the group is complete: quantize the 31 older residual tokens plus the new one
    const int phys = p.block_table[static_cast<long long>(b) * p.max_pages + pos / kGroup];
    if (phys < 0 || phys >= p.n_pages) return;
    constexpr int kStride = QuantSmemT<uint16_t>::kStride;
    for (int i = tid; i < kGroup * kHeadDim; i += kThreads) {
        const int t = i / kHeadDim, c = i % kHeadDim;
        sm.k[t * kStride + c] = (t == kGroup - 1) ? p.k_new[nb + c] : p.resid_k[rbase + i];
        sm.v[t * kStride + c] = (t == kGroup - 1) ? p.v_new[nb + c] : p.resid_v[rbase + i];
    }
    __syncthreads();
    encode_page<KB, VB, KM>(sm, static_cast<uint8_t *>(p.pages), p.scales, phys, p.H, h);
}

template <int KB, int VB, int KM>
hipError_t launch_pack_m(const PackParams &p, bool src_f32, hipStream_t s)
{
    const int gx = (p.max_tokens + kGroup - 1) / kGroup;
    if (gx == 0) return hipSuccess;
    PackParams q = p;
    q.heads_fastest = gx <= 65535;
    const dim3 grid = q.heads_fastest ? dim3(p.H, gx, p.batch) : dim3(gx, p.H, p.batch);
    if (src_f32)
        hipLaunchKernelGGL((pack_kernel<KB, VB, KM, float>), grid, dim3(kThreads), 0, s, q);
    else
        hipLaunchKernelGGL((pack_kernel<KB, VB, KM, uint16_t>), grid, dim3(kThreads), 0, s, q);
    return hipGetLastError();
}

template <int KB, int VB, int KM>
hipError_t launch_append_m(const AppendParams &p, hipStream_t s)
{
    hipLaunchKernelGGL((append_kernel<KB, VB, KM>), dim3(p.H, p.batch), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <int KB, int VB>
hipError_t launch_pack_t(int kmode, const PackParams &p, bool src_f32, hipStream_t s)
{
    if (kmode == kLayerKeysPerChannel) return launch_pack_m<KB, VB, kLayerKeysPerChannel>(p, src_f32, s);
    if (kmode == kLayerKeysPerToken) return launch_pack_m<KB, VB, kLayerKeysPerToken>(p, src_f32, s);
    return hipErrorInvalidValue;
}

template <int KB, int VB>
hipError_t launch_append_t(int kmode, const AppendParams &p, hipStream_t s)
{
    if (kmode == kLayerKeysPerChannel) return launch_append_m<KB, VB, kLayerKeysPerChannel>(p, s);
    if (kmode == kLayerKeysPerToken) return launch_append_m<KB, VB, kLayerKeysPerToken>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_pack(int kb, int vb, int kmode, const PackParams &p, bool src_f32, hipStream_t s)
{
    if (kb == 8 && vb == 8 && kmode == kLayerFp8) return launch_pack_m<8, 8, kLayerFp8>(p, src_f32, s);
    if (kb == 16 && vb == 16 && kmode == kLayerBf16) return launch_pack_m<16, 16, kLayerBf16>(p, src_f32, s);
#define KVQ_P(KBV, VBV) if (kb == KBV && vb == VBV) return launch_pack_t<KBV, VBV>(kmode, p, src_f32, s)
    KVQ_P(2, 2); KVQ_P(2, 4); KVQ_P(2, 8);
    KVQ_P(4, 2); KVQ_P(4, 4); KVQ_P(4, 8);
    KVQ_P(8, 2); KVQ_P(8, 4); KVQ_P(8, 8);
#undef KVQ_P
    return hipErrorInvalidValue;
}

hipError_t launch_append(int kb, int vb, int kmode, const AppendParams &p, hipStream_t s)
{
    if (kb == 8 && vb == 8 && kmode == kLayerFp8) return launch_append_m<8, 8, kLayerFp8>(p, s);
    if (kb == 16 && vb == 16 && kmode == kLayerBf16) return launch_append_m<16, 16, kLayerBf16>(p, s);
#define KVQ_P(KBV, VBV) if (kb == KBV && vb == VBV) return launch_append_t<KBV, VBV>(kmode, p, s)
    KVQ_P(2, 2); KVQ_P(2, 4); KVQ_P(2, 8);
    KVQ_P(4, 2); KVQ_P(4, 4); KVQ_P(4, 8);
    KVQ_P(8, 2); KVQ_P(8, 4); KVQ_P(8, 8);
#undef KVQ_P
    return hipErrorInvalidValue;
}

}  // namespace kvq
