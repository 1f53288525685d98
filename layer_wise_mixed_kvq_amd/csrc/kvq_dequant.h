// kvq_dequant.h -- launch parameters of kvq_dequant (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

struct DequantParams {
    const int32_t *seq_len;
    const int32_t *block_table;
    const void *pages;
    const uint16_t *resid_k;
    const uint16_t *resid_v;
    const float *scales;  // FP8 layers: [H][2] K / V scale, or null (1.0)
    float *k_out;         // [batch][max_tokens][H][128]
    float *v_out;
    long long n_pages;
    int H;
    int batch;
    int max_tokens;
    int max_pages;
};

// kmode: the layer code (as for launch_pack)
hipError_t launch_dequant(int kb, int vb, int kmode, const DequantParams &p, hipStream_t s);

}  // namespace kvq
