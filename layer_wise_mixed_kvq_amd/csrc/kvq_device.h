// kvq_device.h -- device-side definitions shared by the quantize-on-write kernels and the
// decode-attention kernels of the gfx950 library: the packed page layout and the number
// conversions both sides must agree on.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kHeadDim = 128;   // channels per head
constexpr int kGroup = 32;      // tokens per page / per key group, channels per value group
constexpr int kValueGroups = kHeadDim / kGroup;

// Byte offsets of the four sections of one KV head's page (all multiples of 512).
template <int KB, int VB>
struct PageLayout {
    static constexpr int kKCodes = 0;                       // 32 rows x 16*KB bytes
    static constexpr int kKRowBytes = 16 * KB;
    static constexpr int kKSz = 512 * KB;                   // 128 x u32 (s16 | z16 << 16)
    static constexpr int kVCodes = 512 * KB + 512;          // 512*VB bytes in MFMA chunk order: lane l's
                                                            // 8*VB bytes at 8*VB*l
    static constexpr int kVSz = 512 * (KB + VB) + 512;      // 32 tokens x 4 groups x u32
    static constexpr int kBytes = 512 * (KB + VB + 2);
};

__host__ __device__ constexpr int head_page_bytes(int kb, int vb) { return 512 * (kb + vb + 2); }

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b)
{
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// bf16 bits of a finite binary32 value, round to nearest even.
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// fp16 bits of a binary32 value, round to nearest even (v_cvt_f16_f32 under the default
// rounding mode; fp16 denormals are kept).
__device__ __forceinline__ uint16_t float_to_half_bits(float f)
{
    _Float16 h = static_cast<_Float16>(f);
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

}  // namespace kvq
