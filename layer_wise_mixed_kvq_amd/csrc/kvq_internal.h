// kvq_internal.h -- launch parameters and launchers behind the C ABI (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

struct PackParams {
    const void *k_src;
    const void *v_src;
    const int32_t *seq_len;
    const int32_t *block_table;
    void *pages;
    uint16_t *resid_k;
    uint16_t *resid_v;
    const float *scales;  // FP8 layers: [H][2] K / V scale, or null (1.0)
    long long n_pages;
    int H;
    int batch;
    int max_tokens;
    int max_pages;
    int heads_fastest;    // set by the launcher: grid (H, pages, batch) rather than (pages, H, batch)
};

struct AppendParams {
    const uint16_t *k_new;
    const uint16_t *v_new;
    const int32_t *pos;
    const int32_t *block_table;
    void *pages;
    uint16_t *resid_k;
    uint16_t *resid_v;
    const float *scales;  // FP8 layers: [H][2] K / V scale, or null (1.0)
    long long n_pages;
    int H;
    int batch;
    int max_pages;
};

struct DecodeParams {
    const void *q;
    const int32_t *seq_len;      // tokens attended (decode only; null with the fused append)
    const int32_t *pos;          // fused append: position of the new token (attends pos + 1)
    const uint16_t *k_new;       // fused append: bf16 [batch][H][128]
    const uint16_t *v_new;
    const int32_t *block_table;
    void *pages;                 // written only by the fused append's page flush
    uint16_t *resid_k;           // written only by the fused append (the new token's slot)
    uint16_t *resid_v;
    const float *scales;         // FP8 layers: [H][2] K / V scale, or null (1.0)
    float *out;
    float *lse;
    float *part_o;        // [batch][H][n_splits][G][128], channel c at (c % 4) * 32 + c / 4
    float *part_ml;       // [batch][H][n_splits][G][2]  (running max in log2 units, sum)
    int *counters;        // [batch][H]
    long long n_pages;
    int H;
    int G;
    int batch;
    int max_pages;
    int max_seq_len;
    int pages_per_split;
    int n_splits;         // page splits per (b, h)
    int waves;            // waves per workgroup: 8 or 4 (decode_waves_for)
    // profiling build only (KVQ_PHASE_TIMERS): per wave, [kPhaseStamps] u64 real-time
    // stamps at the kernel's phase boundaries; null otherwise
    unsigned long long *phase_ts;
};

// Phase-timer record per wave (KVQ_PHASE_TIMERS builds): stamps 0-5 are the 100 MHz
// real-time counter at entry, page loop start, page loop end, partials stored, split
// counter known, exit; stamps 8-13 at finer points: length known, first page requested, q
// setup done, first page done, residual tokens start and end; 14 and 15 after the two
// barriers of the workgroup's merge (0 where a wave did not reach the point).  Stamp 6 holds the hardware XCC id (bits 32-35) and
// HW_ID register (bits 0-31); stamp 7 the work item as h | b << 20 | split << 40.
constexpr int kPhaseStamps = 16;
#if defined(KVQ_PHASE_TIMERS)
extern unsigned long long *g_phase_buf;   // set by kvq_profile_set_phase_buffer (profiling build)
extern size_t g_phase_bytes;
#endif

// Workspace layout of kvq_decode_attn for (batch, H, G, n_splits).
struct DecodeWorkspace {
    size_t part_o_off, part_ml_off, counters_off, bytes;
};
DecodeWorkspace decode_workspace_layout(int batch, int H, int G, int n_splits);
int decode_waves_for(int batch, int H, int G);
int decode_default_pages_per_split(int batch, int H, int G, int max_full_pages);

// kmode: the layer code -- 0 = integer codes with per-channel keys, 1 = integer codes with
// per-token keys, 2 = FP8 E4M3 (kb = vb = 8), 3 = BF16 (kb = vb = 16)
hipError_t launch_pack(int kb, int vb, int kmode, const PackParams &p, bool src_f32, hipStream_t s);
hipError_t launch_append(int kb, int vb, int kmode, const AppendParams &p, hipStream_t s);
hipError_t launch_decode(int kb, int vb, int kmode, const DecodeParams &p, bool q_f32, hipStream_t s);
// the kernels of one key bit width (each built in its own translation unit)
hipError_t launch_decode_kb2(int vb, int kmode, const DecodeParams &p, bool q_f32, hipStream_t s);
hipError_t launch_decode_kb4(int vb, int kmode, const DecodeParams &p, bool q_f32, hipStream_t s);
hipError_t launch_decode_kb8(int vb, int kmode, const DecodeParams &p, bool q_f32, hipStream_t s);
hipError_t launch_decode_kb16(int vb, int kmode, const DecodeParams &p, bool q_f32, hipStream_t s);
hipError_t launch_zero_fill(void *ptr, size_t bytes, hipStream_t s);

}  // namespace kvq

#if defined(KVQ_PHASE_TIMERS)
// Profiling build only (libkvq_phases.so): every later decode launch whose per-wave
// records ([H][batch][splits][8 wave slots][kPhaseStamps] u64) fit in `bytes` writes them to
// the device buffer `buf`; null turns the recording off.
extern "C" void kvq_profile_set_phase_buffer(void *buf, size_t bytes);
#endif
