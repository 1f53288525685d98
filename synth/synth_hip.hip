/* Device build of the synthetic input generator (see synth_gen.h): one thread per
 * element, bit-identical to the host build. */
#include <hip/hip_runtime.h>
#include "synth_gen.h"

__global__ void sg_fill_kernel(uint64_t key, long long n, int nT, int nH, int D, int b0, int t0,
                               int h0, const float *chan_mult, int out_bf16, void *out)
{
    long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long stride = (long long)gridDim.x * blockDim.x;
    for (; i < n; i += stride) {
        int c = (int)(i % D);
        long long r = i / D;
        int ih = (int)(r % nH);
        int it = (int)((r / nH) % nT);
        int ib = (int)(r / ((long long)nH * nT));
        float x = sg_value(key, (uint32_t)(b0 + ib), (uint32_t)(t0 + it), (uint32_t)(h0 + ih),
                           (uint32_t)c, chan_mult, D);
        if (out_bf16)
            ((uint16_t *)out)[i] = sg_to_bf16(x);
        else
            ((float *)out)[i] = x;
    }
}

/* Same contract as sg_fill_cpu; out and chan_mult are device pointers, the call is
 * asynchronous on `stream` (a hipStream_t, NULL for the default stream). */
extern "C" int sg_fill_hip(uint64_t seed, uint32_t kind, uint32_t layer, int nB, int nT, int nH,
                           int D, int b0, int t0, int h0, const float *chan_mult, int out_bf16,
                           void *out, void *stream)
{
    if (nB < 0 || nT < 0 || nH < 0 || D <= 0 || D > 256) return 1;
    const long long n = (long long)nB * nT * nH * D;
    if (n == 0) return 0;
    long long blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(sg_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       sg_stream_key(seed, kind, layer), n, nT, nH, D, b0, t0, h0, chan_mult,
                       out_bf16, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
