/* Host build of the synthetic input generator (see synth_gen.h). */
#include <stddef.h>
#include "synth_gen.h"

/* Fill out[nB][nT][nH][D] with elements (b0 + ib, t0 + it, h0 + ih, c) of stream
 * (seed, kind, layer); bf16 bits (out_bf16 != 0) or binary32.  chan_mult is [H][D] or
 * NULL, indexed with the absolute head h0 + ih. */
int sg_fill_cpu(uint64_t seed, uint32_t kind, uint32_t layer, int nB, int nT, int nH, int D,
                int b0, int t0, int h0, const float *chan_mult, int out_bf16, void *out)
{
    if (nB < 0 || nT < 0 || nH < 0 || D <= 0 || D > 256) return 1;
    const uint64_t key = sg_stream_key(seed, kind, layer);
    const long long rows = (long long)nB * nT * nH;
#pragma omp parallel for schedule(static)
    for (long long r = 0; r < rows; ++r) {
        int ih = (int)(r % nH);
        int it = (int)((r / nH) % nT);
        int ib = (int)(r / ((long long)nH * nT));
        for (int c = 0; c < D; ++c) {
            float x = sg_value(key, (uint32_t)(b0 + ib), (uint32_t)(t0 + it), (uint32_t)(h0 + ih),
                               (uint32_t)c, chan_mult, D);
            size_t i = (size_t)r * D + c;
            if (out_bf16)
                ((uint16_t *)out)[i] = sg_to_bf16(x);
            else
                ((float *)out)[i] = x;
        }
    }
    return 0;
}
