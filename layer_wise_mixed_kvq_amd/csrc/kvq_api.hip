// kvq_api.hip -- the C ABI declared in include/kvq.h: host-side validation, split planning
// and workspace sizing, then one kernel launch per call on the caller's stream.
#include <stdint.h>

#include <mutex>

#include "../../include/kvq.h"
#include "kvq_codec.h"
#include "kvq_debug.h"
#include "kvq_dequant.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
int decode_max_g();
}

#if defined(KVQ_PHASE_TIMERS)
namespace kvq {
unsigned long long *g_phase_buf = nullptr;
size_t g_phase_bytes = 0;
}
extern "C" void kvq_profile_set_phase_buffer(void *buf, size_t bytes)
{
    kvq::g_phase_buf = static_cast<unsigned long long *>(buf);
    kvq::g_phase_bytes = buf ? bytes : 0;
}
#endif

namespace {

bool valid_bits(int b) { return b == 2 || b == 4 || b == 8; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

kvq_status check_model(const kvq_model *m)
{
    if (!m || !m->k_bits || !m->v_bits) return KVQ_ERR_INVALID_ARG;
    if (m->n_layers <= 0 || m->n_q_heads <= 0 || m->n_kv_heads <= 0) return KVQ_ERR_INVALID_ARG;
    if (m->head_dim != KVQ_HEAD_DIM) return KVQ_ERR_UNSUPPORTED;
    if (m->n_q_heads % m->n_kv_heads != 0) return KVQ_ERR_UNSUPPORTED;
    if (m->n_q_heads / m->n_kv_heads > kvq::decode_max_g()) return KVQ_ERR_UNSUPPORTED;
    if (m->n_kv_heads > 65535) return KVQ_ERR_UNSUPPORTED;
    for (int l = 0; l < m->n_layers; ++l) {
        const int fmt = m->layer_format ? m->layer_format[l] : KVQ_LAYER_INT;
        if (fmt == KVQ_LAYER_FP8) {
            if (m->k_bits[l] != 8 || m->v_bits[l] != 8) return KVQ_ERR_UNSUPPORTED;
        } else if (fmt == KVQ_LAYER_BF16) {
            if (m->k_bits[l] != 16 || m->v_bits[l] != 16) return KVQ_ERR_UNSUPPORTED;
        } else if (fmt == KVQ_LAYER_INT) {
            if (!valid_bits(m->k_bits[l]) || !valid_bits(m->v_bits[l])) return KVQ_ERR_UNSUPPORTED;
            if (m->k_mode && m->k_mode[l] != KVQ_KEYS_PER_CHANNEL && m->k_mode[l] != KVQ_KEYS_PER_TOKEN)
                return KVQ_ERR_UNSUPPORTED;
        } else {
            return KVQ_ERR_UNSUPPORTED;
        }
    }
    return KVQ_OK;
}

int layer_format(const kvq_model *m, int layer) { return m->layer_format ? m->layer_format[layer] : KVQ_LAYER_INT; }

// the kernels' layer code: integer key mode 0 / 1, FP8 2, BF16 3
int layer_code(const kvq_model *m, int layer)
{
    const int fmt = layer_format(m, layer);
    if (fmt == KVQ_LAYER_FP8) return kvq::kLayerFp8;
    if (fmt == KVQ_LAYER_BF16) return kvq::kLayerBf16;
    return m->k_mode ? m->k_mode[layer] : KVQ_KEYS_PER_CHANNEL;
}

size_t head_page_bytes_of(const kvq_model *m, int layer)
{
    const int fmt = layer_format(m, layer);
    if (fmt == KVQ_LAYER_FP8) return static_cast<size_t>(kvq::FloatLayout<kvq::kLayerFp8>::kBytes);
    if (fmt == KVQ_LAYER_BF16) return static_cast<size_t>(kvq::FloatLayout<kvq::kLayerBf16>::kBytes);
    return static_cast<size_t>(kvq::head_page_bytes(m->k_bits[layer], m->v_bits[layer]));
}

// the FP8 scales the kernels read for this layer (null: 1.0, and for every other format)
const float *scales_of(const kvq_model *m, int layer, const kvq_layer_cache *c)
{
    return layer_format(m, layer) == KVQ_LAYER_FP8 ? c->fp8_scales : nullptr;
}

kvq_status check_layer(const kvq_model *m, int32_t layer, const kvq_layer_cache *c)
{
    kvq_status s = check_model(m);
    if (s != KVQ_OK) return s;
    if (layer < 0 || layer >= m->n_layers) return KVQ_ERR_INVALID_ARG;
    if (!c || !c->pages || !c->resid_k || !c->resid_v || !c->block_table) return KVQ_ERR_INVALID_ARG;
    if (c->batch <= 0 || c->batch > 65535 || c->max_pages <= 0 || c->n_pages <= 0) return KVQ_ERR_INVALID_ARG;
    if (c->n_pages > (int64_t)INT32_MAX) return KVQ_ERR_UNSUPPORTED;
    if (!aligned16(c->pages) || !aligned16(c->resid_k) || !aligned16(c->resid_v)) return KVQ_ERR_ALIGNMENT;
    if (c->fp8_scales && (reinterpret_cast<uintptr_t>(c->fp8_scales) & 3u)) return KVQ_ERR_ALIGNMENT;
    return KVQ_OK;
}

kvq_status hip_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP; }

// page splits of the longest sequence (at least one workgroup per (sequence, KV head))
int n_splits_for(int max_seq_len, int pps)
{
    const int n = (max_seq_len / KVQ_GROUP + pps - 1) / pps;
    return n > 0 ? n : 1;
}

// pages per split-K work item: the caller's value (at most 256: a workgroup's waves hold
// at most 64 page ids each), or the library's choice for 0
int plan_pages_per_split(int requested, int batch, int H, int G, int max_seq_len)
{
    if (requested > 256) return 256;
    if (requested > 0) return requested;
    return kvq::decode_default_pages_per_split(batch, H, G, max_seq_len / KVQ_GROUP);
}

}  // namespace

extern "C" {

const char *kvq_status_str(kvq_status s)
{
    switch (s) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_ERR_INVALID_ARG: return "KVQ_ERR_INVALID_ARG";
    case KVQ_ERR_UNSUPPORTED: return "KVQ_ERR_UNSUPPORTED";
    case KVQ_ERR_ALIGNMENT: return "KVQ_ERR_ALIGNMENT";
    case KVQ_ERR_WORKSPACE: return "KVQ_ERR_WORKSPACE";
    case KVQ_ERR_HIP: return "KVQ_ERR_HIP";
    }
    return "KVQ_ERR_UNKNOWN";
}

int32_t kvq_format_version(void) { return KVQ_FORMAT_VERSION; }

size_t kvq_head_page_bytes(int32_t k_bits, int32_t v_bits)
{
    if (!valid_bits(k_bits) || !valid_bits(v_bits)) return 0;
    return static_cast<size_t>(kvq::head_page_bytes(k_bits, v_bits));
}

size_t kvq_page_bytes(const kvq_model *model, int32_t layer)
{
    if (check_model(model) != KVQ_OK || layer < 0 || layer >= model->n_layers) return 0;
    return static_cast<size_t>(model->n_kv_heads) * head_page_bytes_of(model, layer);
}

double kvq_equiv_bits(const kvq_model *model)
{
    if (check_model(model) != KVQ_OK) return -1.0;
    long long sum = 0;
    for (int l = 0; l < model->n_layers; ++l) sum += model->k_bits[l] + model->v_bits[l];
    return static_cast<double>(sum) / (2.0 * model->n_layers);
}

kvq_status kvq_validate_model(const kvq_model *model) { return check_model(model); }

kvq_status kvq_pack(const kvq_model *model, int32_t layer, const kvq_layer_cache *cache,
                    kvq_dtype src_dtype, const void *k_src, const void *v_src, int32_t max_tokens,
                    const int32_t *seq_len, void *stream)
{
    kvq_status s = check_layer(model, layer, cache);
    if (s != KVQ_OK) return s;
    if (!k_src || !v_src || !seq_len || max_tokens < 0) return KVQ_ERR_INVALID_ARG;
    if (src_dtype != KVQ_BF16 && src_dtype != KVQ_F32) return KVQ_ERR_UNSUPPORTED;
    if (!aligned16(k_src) || !aligned16(v_src)) return KVQ_ERR_ALIGNMENT;
    if ((max_tokens + KVQ_GROUP - 1) / KVQ_GROUP > 2147483647) return KVQ_ERR_UNSUPPORTED;
    if (max_tokens == 0) return KVQ_OK;
    kvq::PackParams p;
    p.k_src = k_src;
    p.v_src = v_src;
    p.seq_len = seq_len;
    p.block_table = cache->block_table;
    p.pages = cache->pages;
    p.resid_k = cache->resid_k;
    p.resid_v = cache->resid_v;
    p.scales = scales_of(model, layer, cache);
    p.n_pages = cache->n_pages;
    p.H = model->n_kv_heads;
    p.batch = cache->batch;
    p.max_tokens = max_tokens;
    p.max_pages = cache->max_pages;
    if (kvq::debug_checks_enabled()) {
        s = kvq::debug_check_pack(p, src_dtype == KVQ_F32, static_cast<hipStream_t>(stream));
        if (s != KVQ_OK) return s;
    }
    return hip_status(kvq::launch_pack(model->k_bits[layer], model->v_bits[layer], layer_code(model, layer), p,
                                       src_dtype == KVQ_F32, static_cast<hipStream_t>(stream)));
}

kvq_status kvq_append(const kvq_model *model, int32_t layer, const kvq_layer_cache *cache,
                      const uint16_t *k_new, const uint16_t *v_new, const int32_t *pos, void *stream)
{
    kvq_status s = check_layer(model, layer, cache);
    if (s != KVQ_OK) return s;
    if (!k_new || !v_new || !pos) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(k_new) || !aligned16(v_new)) return KVQ_ERR_ALIGNMENT;
    kvq::AppendParams p;
    p.k_new = k_new;
    p.v_new = v_new;
    p.pos = pos;
    p.block_table = cache->block_table;
    p.pages = cache->pages;
    p.resid_k = cache->resid_k;
    p.resid_v = cache->resid_v;
    p.scales = scales_of(model, layer, cache);
    p.n_pages = cache->n_pages;
    p.H = model->n_kv_heads;
    p.batch = cache->batch;
    p.max_pages = cache->max_pages;
    if (kvq::debug_checks_enabled()) {
        s = kvq::debug_check_append(p, static_cast<hipStream_t>(stream));
        if (s != KVQ_OK) return s;
    }
    return hip_status(kvq::launch_append(model->k_bits[layer], model->v_bits[layer], layer_code(model, layer), p,
                                         static_cast<hipStream_t>(stream)));
}

kvq_status kvq_dequant(const kvq_model *model, int32_t layer, const kvq_layer_cache *cache, int32_t max_tokens,
                       const int32_t *seq_len, float *k_out, float *v_out, void *stream)
{
    kvq_status s = check_layer(model, layer, cache);
    if (s != KVQ_OK) return s;
    if (!seq_len || !k_out || !v_out || max_tokens < 0) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(k_out) || !aligned16(v_out)) return KVQ_ERR_ALIGNMENT;
    if (max_tokens == 0) return KVQ_OK;
    kvq::DequantParams p;
    p.seq_len = seq_len;
    p.block_table = cache->block_table;
    p.pages = cache->pages;
    p.resid_k = cache->resid_k;
    p.resid_v = cache->resid_v;
    p.scales = scales_of(model, layer, cache);
    p.k_out = k_out;
    p.v_out = v_out;
    p.n_pages = cache->n_pages;
    p.H = model->n_kv_heads;
    p.batch = cache->batch;
    p.max_tokens = max_tokens;
    p.max_pages = cache->max_pages;
    if (kvq::debug_checks_enabled()) {
        s = kvq::debug_check_dequant(p, static_cast<hipStream_t>(stream));
        if (s != KVQ_OK) return s;
    }
    return hip_status(kvq::launch_dequant(model->k_bits[layer], model->v_bits[layer], layer_code(model, layer), p,
                                          static_cast<hipStream_t>(stream)));
}

size_t kvq_decode_workspace_bytes(const kvq_model *model, int32_t batch, int32_t max_seq_len,
                                  int32_t pages_per_split)
{
    if (check_model(model) != KVQ_OK || batch <= 0 || max_seq_len < 0 || pages_per_split < 0) return 0;
    const int H = model->n_kv_heads, G = model->n_q_heads / model->n_kv_heads;
    const int pps = plan_pages_per_split(pages_per_split, batch, H, G, max_seq_len);
    return kvq::decode_workspace_layout(batch, H, G, n_splits_for(max_seq_len, pps)).bytes;
}

kvq_status kvq_workspace_init(void *workspace, size_t workspace_bytes, void *stream)
{
    if (!workspace) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(workspace)) return KVQ_ERR_ALIGNMENT;
    return hip_status(kvq::launch_zero_fill(workspace, workspace_bytes, static_cast<hipStream_t>(stream)));
}

namespace {

// Where a decode call keeps its split partials and split counters.
struct DecodeScratch {
    float *part_o;
    float *part_ml;
    int *counters;
};

kvq_status decode_checks(const kvq_model *model, int32_t layer, const kvq_layer_cache *cache, kvq_dtype q_dtype,
                         const void *q, const float *out, const float *lse, int32_t max_seq_len,
                         int32_t pages_per_split)
{
    kvq_status s = check_layer(model, layer, cache);
    if (s != KVQ_OK) return s;
    if (!q || !out || max_seq_len < 0 || pages_per_split < 0) return KVQ_ERR_INVALID_ARG;
    if (q_dtype != KVQ_BF16 && q_dtype != KVQ_F32) return KVQ_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(out) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
        return KVQ_ERR_ALIGNMENT;
    return KVQ_OK;
}

kvq_status decode_launch(const kvq_model *model, int32_t layer, const kvq_layer_cache *cache, kvq_dtype q_dtype,
                         const void *q, const int32_t *seq_len, const uint16_t *k_new, const uint16_t *v_new,
                         const int32_t *pos, int32_t max_seq_len, int pps, int n_splits, float *out, float *lse,
                         const DecodeScratch &w, bool debug_checks, void *stream)
{
    const int H = model->n_kv_heads, G = model->n_q_heads / model->n_kv_heads;
    kvq::DecodeParams p;
    p.q = q;
    p.seq_len = seq_len;
    p.pos = pos;
    p.k_new = k_new;
    p.v_new = v_new;
    p.block_table = cache->block_table;
    p.pages = cache->pages;
    p.resid_k = cache->resid_k;
    p.resid_v = cache->resid_v;
    p.scales = scales_of(model, layer, cache);
    p.out = out;
    p.lse = lse;
    p.part_o = w.part_o;
    p.part_ml = w.part_ml;
    p.counters = w.counters;
    p.n_pages = cache->n_pages;
    p.H = H;
    p.G = G;
    p.batch = cache->batch;
    p.max_pages = cache->max_pages;
    p.max_seq_len = max_seq_len;
    p.pages_per_split = pps;
    p.n_splits = n_splits;
    p.waves = kvq::decode_waves_for(cache->batch, H, G);
    p.phase_ts = nullptr;
#if defined(KVQ_PHASE_TIMERS)
    {
        const size_t need = static_cast<size_t>(H) * cache->batch * n_splits * 8 * kvq::kPhaseStamps * 8;
        if (kvq::g_phase_buf && kvq::g_phase_bytes >= need) p.phase_ts = kvq::g_phase_buf;
    }
#endif
    if (debug_checks && kvq::debug_checks_enabled()) {
        const kvq_status s = kvq::debug_check_decode(p, q_dtype == KVQ_F32, static_cast<hipStream_t>(stream));
        if (s != KVQ_OK) return s;
    }
    return hip_status(kvq::launch_decode(model->k_bits[layer], model->v_bits[layer], layer_code(model, layer), p,
                                         q_dtype == KVQ_F32, static_cast<hipStream_t>(stream)));
}

kvq_status decode_common(const kvq_model *model, int32_t layer, const kvq_layer_cache *cache, kvq_dtype q_dtype,
                         const void *q, const int32_t *seq_len, const uint16_t *k_new, const uint16_t *v_new,
                         const int32_t *pos, int32_t max_seq_len, int32_t pages_per_split, float *out, float *lse,
                         void *workspace, size_t workspace_bytes, void *stream)
{
    kvq_status s = decode_checks(model, layer, cache, q_dtype, q, out, lse, max_seq_len, pages_per_split);
    if (s != KVQ_OK) return s;
    const int H = model->n_kv_heads, G = model->n_q_heads / model->n_kv_heads;
    const int pps = plan_pages_per_split(pages_per_split, cache->batch, H, G, max_seq_len);
    const int n_splits = n_splits_for(max_seq_len, pps);
    if (n_splits > 65535) return KVQ_ERR_UNSUPPORTED;
    const kvq::DecodeWorkspace ws = kvq::decode_workspace_layout(cache->batch, H, G, n_splits);
    if (!workspace || workspace_bytes < ws.bytes) return KVQ_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KVQ_ERR_ALIGNMENT;
    char *w = static_cast<char *>(workspace);
    const DecodeScratch sc = {reinterpret_cast<float *>(w + ws.part_o_off), reinterpret_cast<float *>(w + ws.part_ml_off),
                              reinterpret_cast<int *>(w + ws.counters_off)};
    return decode_launch(model, layer, cache, q_dtype, q, seq_len, k_new, v_new, pos, max_seq_len, pps, n_splits, out,
                         lse, sc, true, stream);
}

// ---- the library's own decode scratch, for kvq_append_decode_attn_noalloc --------------
// One file-scope device array per GPU: split counters at a fixed offset (so every call finds
// them at zero, whatever its shape), then the split partials.  Host code uses the device
// address hipGetSymbolAddress returns for the current device, never the array's name.
constexpr size_t kScratchCounterBytes = static_cast<size_t>(KVQ_NOALLOC_MAX_COUNTERS) * sizeof(int);
constexpr size_t kScratchBytes = kScratchCounterBytes + KVQ_NOALLOC_MAX_PARTIAL_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};
static ScratchSlot g_scratch[kMaxDevices];

// The scratch's device address on the current device; the first call on a device also zeroes
// its counters (a fill kernel on `stream`).
static kvq_status scratch_for_current_device(void **ptr, hipStream_t stream)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVQ_ERR_HIP;
    ScratchSlot &slot = g_scratch[dev];
    std::call_once(slot.once, [&] {
        void *p = nullptr;
        slot.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (slot.err == hipSuccess) slot.err = kvq::launch_zero_fill(p, kScratchCounterBytes, stream);
        if (slot.err == hipSuccess) slot.ptr = p;
    });
    if (slot.err != hipSuccess || !slot.ptr) return KVQ_ERR_HIP;
    *ptr = slot.ptr;
    return KVQ_OK;
}

}  // namespace

kvq_status kvq_decode_attn(const kvq_model *model, int32_t layer, const kvq_layer_cache *cache,
                           kvq_dtype q_dtype, const void *q, const int32_t *seq_len, int32_t max_seq_len,
                           int32_t pages_per_split, float *out, float *lse, void *workspace,
                           size_t workspace_bytes, void *stream)
{
    if (!seq_len) return KVQ_ERR_INVALID_ARG;
    return decode_common(model, layer, cache, q_dtype, q, seq_len, nullptr, nullptr, nullptr, max_seq_len,
                         pages_per_split, out, lse, workspace, workspace_bytes, stream);
}

kvq_status kvq_append_decode_attn(const kvq_model *model, int32_t layer, const kvq_layer_cache *cache,
                                  const uint16_t *k_new, const uint16_t *v_new, const int32_t *pos,
                                  kvq_dtype q_dtype, const void *q, int32_t max_seq_len, int32_t pages_per_split,
                                  float *out, float *lse, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!k_new || !v_new || !pos) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(k_new) || !aligned16(v_new)) return KVQ_ERR_ALIGNMENT;
    return decode_common(model, layer, cache, q_dtype, q, nullptr, k_new, v_new, pos, max_seq_len,
                         pages_per_split, out, lse, workspace, workspace_bytes, stream);
}

kvq_status kvq_append_decode_attn_noalloc(const kvq_model *model, int32_t layer, const kvq_layer_cache *cache,
                                          const uint16_t *k_new, const uint16_t *v_new, const int32_t *pos,
                                          kvq_dtype q_dtype, const void *q, int32_t max_seq_len,
                                          int32_t pages_per_split, float *out, float *lse, void *stream)
{
    if (!k_new || !v_new || !pos) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(k_new) || !aligned16(v_new)) return KVQ_ERR_ALIGNMENT;
    kvq_status s = decode_checks(model, layer, cache, q_dtype, q, out, lse, max_seq_len, pages_per_split);
    if (s != KVQ_OK) return s;
    const int H = model->n_kv_heads, G = model->n_q_heads / model->n_kv_heads;
    const int pps = plan_pages_per_split(pages_per_split, cache->batch, H, G, max_seq_len);
    const int n_splits = n_splits_for(max_seq_len, pps);
    if (n_splits > 65535) return KVQ_ERR_UNSUPPORTED;
    const kvq::DecodeWorkspace ws = kvq::decode_workspace_layout(cache->batch, H, G, n_splits);
    // the partials take everything before the workspace layout's counters
    if (static_cast<long long>(cache->batch) * H > KVQ_NOALLOC_MAX_COUNTERS ||
        ws.counters_off > static_cast<size_t>(KVQ_NOALLOC_MAX_PARTIAL_BYTES))
        return KVQ_ERR_WORKSPACE;
    void *base = nullptr;
    s = scratch_for_current_device(&base, static_cast<hipStream_t>(stream));
    if (s != KVQ_OK) return s;
    char *part = static_cast<char *>(base) + kScratchCounterBytes;
    const DecodeScratch sc = {reinterpret_cast<float *>(part + ws.part_o_off),
                              reinterpret_cast<float *>(part + ws.part_ml_off), static_cast<int *>(base)};
    return decode_launch(model, layer, cache, q_dtype, q, nullptr, k_new, v_new, pos, max_seq_len, pps, n_splits,
                         out, lse, sc, false, stream);
}

size_t kvq_noalloc_scratch_bytes(const kvq_model *model, int32_t batch, int32_t max_seq_len, int32_t pages_per_split)
{
    if (check_model(model) != KVQ_OK || batch <= 0 || max_seq_len < 0 || pages_per_split < 0) return 0;
    const int H = model->n_kv_heads, G = model->n_q_heads / model->n_kv_heads;
    const int pps = plan_pages_per_split(pages_per_split, batch, H, G, max_seq_len);
    return kvq::decode_workspace_layout(batch, H, G, n_splits_for(max_seq_len, pps)).counters_off;
}

}  // extern "C"
