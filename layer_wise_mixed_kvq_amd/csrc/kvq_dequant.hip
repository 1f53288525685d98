// kvq_dequant.hip -- the inverse of the pack: a layer's cache back to binary32 K and V.
//
// Every stored value is what the decode attention attends: code * s + z for integer codes
// (one binary32 rounding of the exact value, which has at most 19 significant bits before
// the add), the E4M3 value times the KV head's scale for FP8 pages, the bf16 value for
// BF16 pages and for the bf16 residual tokens.  A caller uses it to inspect a cache, to
// hand it to code that wants plain tensors, or to measure each layer's quantization error
// against its source.
//   [Mixed-precision KV-cache quantization per-layer sensitivity (llms-explorer.com), Facts]
//   [When should you use mixed-precision KV caching to preserve accuracy in sensitive
//    transformer layers (machinoai.in), sections 1-2]
//
// One workgroup of 256 threads decodes one page-head (or the residual tokens of one
// sequence and head): thread i writes token i / 8, channels 16 (i % 8) .. + 15 of K and V,
// reading each code from the dword that holds it (codes never straddle dwords).
#include "kvq_codec.h"
#include "kvq_dequant.h"
#include "kvq_device.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = kGroup * kHeadDim / kThreads;   // 16 channels of one token

__device__ __forceinline__ float half_to_f32(uint32_t h) { return half_bits_to_float(static_cast<uint16_t>(h)); }

__device__ __forceinline__ float apply_sz(uint32_t code, uint32_t sz)
{
    return __builtin_fmaf(static_cast<float>(code), half_to_f32(sz & 0xFFFFu), half_to_f32(sz >> 16));
}

__device__ __forceinline__ uint32_t code_at(const uint32_t *words, int bit, int bits)
{
    return (words[bit >> 5] >> (bit & 31)) & ((1u << bits) - 1u);
}

// bit of channel c inside a per-token-mode key row: chunk a = (c % 32) / 8 of 4*KB bytes,
// slot s with c = 32 (k / 4) + 8 a + 2 (k % 4) + hh, s = (k / n) 2n + hh n + k % n, n = 16 / KB
template <int KB>
__device__ __forceinline__ int ktok_bit(int c)
{
    constexpr int n = 16 / KB;
    const int a = (c % 32) / 8, hh = c % 2, k = 4 * (c / 32) + (c % 8) / 2;
    const int s = (k / n) * 2 * n + hh * n + k % n;
    return a * 32 * KB + s * KB;
}

// bit of (token t, channel c) inside the value code section (chunk 16 q + r holds tokens
// 8q .. 8q+7 of channels r, r+16, ..; word k / n of the chunk, half (t % 8) / 4)
template <int VB>
__device__ __forceinline__ int vcode_bit(int t, int c)
{
    constexpr int n = 16 / VB;
    const int chunk = 16 * (t / 8) + c % 16, i = t % 8, k = 4 * (c / 16) + i % 4;
    return chunk * 64 * VB + 32 * (k / n) + 16 * (i / 4) + VB * (k % n);
}

template <int KB, int VB, int KM>
__device__ void decode_page(const uint8_t *src, const float *scales, int h, int t, int c0, float *ko, float *vo)
{
    if constexpr (is_float_layer(KM)) {
        using FL = FloatLayout<KM>;
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const int c = c0 + i;
            if constexpr (KM == kLayerFp8) {
                const float ks = scales ? scales[2 * h] : 1.0f, vs = scales ? scales[2 * h + 1] : 1.0f;
                ko[i] = e4m3_to_f32(src[t * kHeadDim + c]) * ks;
                vo[i] = e4m3_to_f32(src[FL::kV + c * kGroup + t]) * vs;
            } else {
                const uint16_t *s16 = reinterpret_cast<const uint16_t *>(src);
                ko[i] = bf16_bits_to_float(s16[t * kHeadDim + c]);
                vo[i] = bf16_bits_to_float(s16[FL::kV / 2 + c * kGroup + t]);
            }
        }
    } else {
        using P = PageLayout<KB, VB>;
        const uint32_t *kw = reinterpret_cast<const uint32_t *>(src + P::kKCodes + t * P::kKRowBytes);
        const uint32_t *ksz = reinterpret_cast<const uint32_t *>(src + P::kKSz);
        const uint32_t *vw = reinterpret_cast<const uint32_t *>(src + P::kVCodes);
        const uint32_t *vsz = reinterpret_cast<const uint32_t *>(src + P::kVSz);
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const int c = c0 + i;
            if constexpr (KM == kLayerKeysPerToken)
                ko[i] = apply_sz(code_at(kw, ktok_bit<KB>(c), KB), ksz[kValueGroups * t + c / kGroup]);
            else
                ko[i] = apply_sz(code_at(kw, c * KB, KB), ksz[c]);
            vo[i] = apply_sz(code_at(vw, vcode_bit<VB>(t, c), VB), vsz[kValueGroups * t + c / kGroup]);
        }
    }
}

// grid: (pages covering max_tokens, n_kv_heads, batch)
template <int KB, int VB, int KM>
__global__ __launch_bounds__(kThreads) void dequant_kernel(DequantParams p)
{
    const int g = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int L = p.seq_len[b];
    if (L < 0 || L > p.max_tokens || L > kGroup * p.max_pages) return;
    const int full = L / kGroup;
    const int t = threadIdx.x / 8, c0 = kPerThread * (threadIdx.x % 8);
    const int tok = g * kGroup + t;
    if (tok >= L) return;
    float ko[kPerThread], vo[kPerThread];
    if (g < full) {
        const int phys = p.block_table[static_cast<long long>(b) * p.max_pages + g];
        if (phys < 0 || phys >= p.n_pages) return;
        const uint8_t *src =
            static_cast<const uint8_t *>(p.pages) + (static_cast<long long>(phys) * p.H + h) * layer_page_bytes<KB, VB, KM>();
        decode_page<KB, VB, KM>(src, p.scales, h, t, c0, ko, vo);
    } else {
        const long long r = ((static_cast<long long>(b) * p.H + h) * kGroup + t) * kHeadDim + c0;
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            ko[i] = bf16_bits_to_float(p.resid_k[r + i]);
            vo[i] = bf16_bits_to_float(p.resid_v[r + i]);
        }
    }
    const long long o = ((static_cast<long long>(b) * p.max_tokens + tok) * p.H + h) * kHeadDim + c0;
#pragma unroll
    for (int i = 0; i < kPerThread; i += 4) {
        *reinterpret_cast<float4 *>(p.k_out + o + i) = make_float4(ko[i], ko[i + 1], ko[i + 2], ko[i + 3]);
        *reinterpret_cast<float4 *>(p.v_out + o + i) = make_float4(vo[i], vo[i + 1], vo[i + 2], vo[i + 3]);
    }
}

template <int KB, int VB, int KM>
hipError_t launch_m(const DequantParams &p, hipStream_t s)
{
    const int gx = (p.max_tokens + kGroup - 1) / kGroup;
    if (gx == 0) return hipSuccess;
    hipLaunchKernelGGL((dequant_kernel<KB, VB, KM>), dim3(gx, p.H, p.batch), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <int KB, int VB>
hipError_t launch_t(int kmode, const DequantParams &p, hipStream_t s)
{
    if (kmode == kLayerKeysPerChannel) return launch_m<KB, VB, kLayerKeysPerChannel>(p, s);
    if (kmode == kLayerKeysPerToken) return launch_m<KB, VB, kLayerKeysPerToken>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_dequant(int kb, int vb, int kmode, const DequantParams &p, hipStream_t s)
{
    if (kb == 8 && vb == 8 && kmode == kLayerFp8) return launch_m<8, 8, kLayerFp8>(p, s);
    if (kb == 16 && vb == 16 && kmode == kLayerBf16) return launch_m<16, 16, kLayerBf16>(p, s);
#define KVQ_P(KBV, VBV) if (kb == KBV && vb == VBV) return launch_t<KBV, VBV>(kmode, p, s)
    KVQ_P(2, 2); KVQ_P(2, 4); KVQ_P(2, 8);
    KVQ_P(4, 2); KVQ_P(4, 4); KVQ_P(4, 8);
    KVQ_P(8, 2); KVQ_P(8, 4); KVQ_P(8, 8);
#undef KVQ_P
    return hipErrorInvalidValue;
}

}  // namespace kvq
