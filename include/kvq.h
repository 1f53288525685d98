/*
 * kvq.h -- C ABI of the MI355X (gfx950) library for layer-wise mixed-precision KV-cache
 * quantization: quantize-on-write of K and V into per-layer (key bits, value bits) pairs,
 * and single-token decode attention that reads the packed low-bit cache and dequantizes
 * it inside the kernel.
 *
 * Method.
 *   - Every layer has its own precision pair, taken from an offline-searched table and
 *     applied online with no per-token decision; online, only the newly generated token is
 *     quantized, at its layer's pair.
 *       [KVTuner (mlsanity.com/paper/2502.04420), Abstract]
 *       [Mixed-precision KV-cache quantization per-layer sensitivity (llms-explorer.com), Facts]
 *       [KVTuner OpenReview discussion (paperhub.cn/paper/zDwipF6h06), reply to reviewer 3,
 *        section 1 "Computational cost"]
 *   - Keys are quantized per channel (asymmetric min/max over a group of tokens; keys carry
 *     channel-wise outliers), values per token (asymmetric min/max over a group of channels).
 *       [llms-explorer.com page above, Facts]
 *       [KVTuner OpenReview discussion, reply to reviewer 1, section 4; reply to reviewer 2,
 *        section 2]
 *   - Decode attention works on the dequantized cache and is FlashAttention-compatible
 *     (online softmax).  [KVTuner OpenReview discussion, reply to reviewer 2, section 1]
 *   - Prefill and decode must agree on every layer's format, scales and layout, and
 *     per-layer page sizes differ.  [When should you use mixed-precision KV caching to
 *     preserve accuracy in sensitive Transformer layers? (machinoai.in), section 5]
 *
 * Packed format, version KVQ_FORMAT_VERSION (the contract shared by pack, append and
 * decode; head_dim is 128, bit widths are 2, 4 or 8):
 *
 *   Group quantizer over 32 values x_i (binary32):
 *     mn = min x_i, mx = max x_i (-0 read as +0)
 *     s16 = fp16_rne((mx - mn) / (2^b - 1))     binary32 subtract, binary32 divide
 *     z16 = fp16_rne(mn)
 *     s, z = s16, z16 widened to binary32
 *     code_i = clamp(round_half_even((x_i - z) / s), 0, 2^b - 1), all 0 when s == 0
 *     dequantized value = code * s + z
 *   Keys, per-channel mode: one group per (page, KV head, channel) over the page's 32
 *   tokens.  Keys, per-token mode: one group per (token, KV head, 32 consecutive channels).
 *   Values: one group per (token, KV head, 32 consecutive channels).
 *
 *   One page = 32 consecutive tokens of one sequence for all KV heads of one layer.
 *   A layer's pool is [physical page][KV head][head_page], head_page = 512*(kb+vb+2) bytes:
 *     +0              K codes, token-major: row t (16*kb bytes).  Per-channel mode:
 *                     channel c at bit c*kb.  Per-token mode: the row is four chunks of
 *                     4*kb bytes and slot s of chunk a (bit s*kb of the chunk) holds
 *                     channel 32*(k/4) + 8*a + 2*(k%4) + hh, where n = 16/kb,
 *                     hh = (s/n)%2, k = (s/(2n))*n + s%n
 *     +512*kb         K scale/zero: 128 x u32 = s16 | z16 << 16; per-channel mode word c,
 *                     per-token mode word 4*t + j (channels 32j..32j+31)
 *     +512*kb+512     V codes: 64 chunks of 8*vb bytes; chunk 16*q + r holds tokens
 *                     8q..8q+7 of channels r, r+16, ..., r+112; inside it, with
 *                     i = t%8, j = i%4, k = 4*(c/16) + j, n = 16/vb, the code of
 *                     (t, c) is at bit 32*(k/n) + 16*(i/4) + vb*(k%n)
 *     +512*(kb+vb)+512 V scale/zero: 128 x u32, word 4*t + j (channels 32j..32j+31)
 *   Codes are little-endian, LSB-first.  block_table[b][i] names the physical page that
 *   holds tokens 32i..32i+31 of sequence b; one block table serves every layer, each
 *   layer has its own pool sized by its pair.
 *   Residual: tokens 32*floor(L/32) .. L-1 of a sequence of length L are kept unquantized
 *   as bf16 in slot t mod 32 of resid_k / resid_v [batch][n_kv_heads][32][128].
 *
 *   Floating-point layers (layer_format, below) store the values themselves, in the same
 *   pages, block table and residual:
 *     KVQ_LAYER_FP8:  head_page = 8192 bytes.  +0: K token-major [32][128] bytes,
 *                     +4096: V channel-major [128][32] bytes.  Each byte is the OCP FP8
 *                     E4M3 encoding of x / scale (binary32 divide; round to nearest even;
 *                     finite values beyond 448 saturate to +-448), with one K scale and one
 *                     V scale per KV head (fp8_scales); the stored value is byte * scale.
 *     KVQ_LAYER_BF16: head_page = 16384 bytes.  +0: K token-major [32][128] bf16,
 *                     +8192: V channel-major [128][32] bf16 (round to nearest even).
 *   The pages keep precision-sensitive layers in BF16 and the rest in FP8 with per-layer
 *   scaling.  [When should you use mixed-precision KV caching to preserve accuracy in
 *   sensitive transformer layers (machinoai.in), sections 1-2]
 *
 * Conventions.
 *   - Every device pointer is owned by the caller.  The library never allocates device
 *     memory, keeps no pointer after returning and has no mutable global state (apart from
 *     the KVQ_DEBUG counter below).
 *   - Every entry point is asynchronous on `stream` (a hipStream_t; NULL is the default
 *     stream).  Arguments are validated on the host before anything is launched; a
 *     nonzero status means nothing was launched.
 *   - Device-side preconditions that the host cannot see (contents of seq_len, pos and
 *     block_table) are bounds-checked in the kernels: a sequence with an invalid length or
 *     page id is skipped by pack/append and yields NaN outputs in decode attention; the
 *     kernels never read or write outside the buffers the caller described.
 *   - Input values must be finite with |x| <= 65504 (fp16 range) so that scales and zeros
 *     are finite.
 *   - KVQ_DEBUG: with this environment variable set to anything but "" or "0", every entry
 *     point also checks, before its launch, what only the device holds: each length or
 *     position against max_tokens / max_seq_len and the block table's capacity, the
 *     block-table ids of the pages the call reads or writes against the pool, K / V values
 *     of the live tokens and of the new token (finite, |x| <= 65504), q (finite) and the
 *     FP8 scales (positive, finite).  A failed check returns KVQ_ERR_INVALID_ARG and
 *     launches nothing.  The checks copy lengths and block table to the host and count
 *     out-of-domain values in one device counter per GPU, so a checked call waits for its
 *     stream, must not be captured into a graph, and checked calls on several streams of
 *     one GPU at once share that counter.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_FORMAT_VERSION 2
#define KVQ_HEAD_DIM 128
#define KVQ_GROUP 32

typedef enum kvq_status {
    KVQ_OK = 0,
    KVQ_ERR_INVALID_ARG = 1,  /* null pointer, layer out of range, non-positive sizes,
                                 a failed KVQ_DEBUG check                               */
    KVQ_ERR_UNSUPPORTED = 2,  /* bits not in {2,4,8}, head_dim != 128, Hq % H != 0, ...   */
    KVQ_ERR_ALIGNMENT = 3,    /* a device pointer is not 16-byte aligned                  */
    KVQ_ERR_WORKSPACE = 4,    /* decode workspace missing or smaller than required        */
    KVQ_ERR_HIP = 5           /* the HIP runtime reported an error at launch              */
} kvq_status;

typedef enum kvq_dtype { KVQ_BF16 = 0, KVQ_F32 = 1 } kvq_dtype;

/* Key quantization modes.  KVQ_KEYS_PER_CHANNEL (the default): one key group per channel
 * over a page's 32 tokens -- keys carry channel-wise outliers.  KVQ_KEYS_PER_TOKEN: one
 * key group per (token, 32 consecutive channels), the rule the values use.  The pages
 * compare the two modes and find different Pareto-optimal pairs for each.
 *   [Mixed-precision KV-cache quantization per-layer sensitivity (llms-explorer.com), Facts]
 *   [KVTuner OpenReview discussion, reply to reviewer 1, section 4] */
#define KVQ_KEYS_PER_CHANNEL 0
#define KVQ_KEYS_PER_TOKEN 1

/* Layer formats.  KVQ_LAYER_INT: integer codes at (k_bits, v_bits) in {2, 4, 8} with the
 * layer's key mode.  KVQ_LAYER_FP8: E4M3 with per-head scales, k_bits = v_bits = 8.
 * KVQ_LAYER_BF16: bfloat16, k_bits = v_bits = 16.  (Key modes apply to integer layers only.) */
#define KVQ_LAYER_INT 0
#define KVQ_LAYER_FP8 1
#define KVQ_LAYER_BF16 2

/* The per-layer precision table and the attention shape.  k_bits / v_bits are HOST
 * arrays of n_layers entries: 2, 4 or 8 for integer layers, 8 / 8 for FP8 layers and
 * 16 / 16 for BF16 layers.  k_mode is a HOST array of n_layers key modes
 * (KVQ_KEYS_PER_CHANNEL / KVQ_KEYS_PER_TOKEN), or NULL for per-channel keys in every layer.
 * layer_format is a HOST array of n_layers KVQ_LAYER_* values, or NULL for integer codes in
 * every layer. */
typedef struct kvq_model {
    int32_t n_layers;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;          /* must be 128 */
    const uint8_t *k_bits;
    const uint8_t *v_bits;
    const uint8_t *k_mode;     /* optional, see above */
    const uint8_t *layer_format; /* optional, see above */
} kvq_model;

/* One layer's cache (all device pointers). */
typedef struct kvq_layer_cache {
    void *pages;               /* [n_pages][n_kv_heads][kvq_head_page_bytes(kb, vb)]       */
    int64_t n_pages;           /* physical pages in this layer's pool                      */
    uint16_t *resid_k;         /* bf16 [batch][n_kv_heads][32][128]                         */
    uint16_t *resid_v;         /* bf16 [batch][n_kv_heads][32][128]                         */
    const int32_t *block_table;/* int32 [batch][max_pages]                                  */
    int32_t batch;
    int32_t max_pages;
    const float *fp8_scales;   /* FP8 layers: fp32 [n_kv_heads][2] = (K scale, V scale) of
                                  each KV head, positive, finite and normal; NULL = all 1.0.
                                  Ignored by the other formats.                             */
} kvq_layer_cache;

/* Status name, e.g. "KVQ_ERR_WORKSPACE". */
const char *kvq_status_str(kvq_status s);

/* KVQ_FORMAT_VERSION of the built library. */
int32_t kvq_format_version(void);

/* Bytes of one page of one KV head of an integer layer: 512 * (kb + vb + 2); 0 for
 * unsupported widths. */
size_t kvq_head_page_bytes(int32_t k_bits, int32_t v_bits);

/* Bytes of one page of layer `layer` for all KV heads, in the layer's format (integer,
 * FP8: 8192 per head, BF16: 16384 per head); 0 on invalid arguments. */
size_t kvq_page_bytes(const kvq_model *model, int32_t layer);

/* Equivalent bit-width of the table: mean over layers of (k_bits + v_bits) / 2, counting
 * code bits only (K8V4 is 6, the Llama table with layers 0-2 and 31 at K4V8 is 3.25; FP8
 * layers count 8, BF16 layers 16).
 * [KVTuner OpenReview discussion, reply to reviewer 1, section 2]  Returns -1 on invalid
 * arguments. */
double kvq_equiv_bits(const kvq_model *model);

/* Checks the table and the shape; KVQ_OK or the reason it is rejected. */
kvq_status kvq_validate_model(const kvq_model *model);

/* Prefill quantize-on-write of one layer.
 *   k_src, v_src: device [batch][max_tokens][n_kv_heads][128], bf16 or fp32 (src_dtype)
 *   seq_len:      device int32 [batch]; sequence b has seq_len[b] tokens (0 allowed)
 * Writes pages 0 .. seq_len/32 - 1 of every sequence through the block table and copies the
 * seq_len mod 32 trailing tokens into the residual (fp32 sources are rounded to bf16,
 * nearest even).  Residual slots past the live tokens are left unspecified. */
kvq_status kvq_pack(const kvq_model *model, int32_t layer, const kvq_layer_cache *cache,
                    kvq_dtype src_dtype, const void *k_src, const void *v_src,
                    int32_t max_tokens, const int32_t *seq_len, void *stream);

/* The inverse of the pack: one layer's cache back to binary32 K and V.
 *   k_out, v_out: device fp32 [batch][max_tokens][n_kv_heads][128], 16-byte aligned
 *   seq_len:      device int32 [batch]; tokens 0 .. seq_len[b] - 1 are written, the rest
 *                 of k_out / v_out is left as it was
 * Each value is what decode attention attends: code * s + z rounded once to binary32 for
 * integer pages, E4M3 value * scale for FP8 pages, the bf16 value for BF16 pages and for
 * the residual tokens.  A sequence whose length or page ids are invalid is skipped.
 * For inspecting a cache, handing it to code that wants plain tensors, or measuring each
 * layer's quantization error against its source.  [Mixed-precision KV-cache quantization
 * per-layer sensitivity (llms-explorer.com), Facts] */
kvq_status kvq_dequant(const kvq_model *model, int32_t layer, const kvq_layer_cache *cache,
                       int32_t max_tokens, const int32_t *seq_len, float *k_out, float *v_out,
                       void *stream);

/* Decode-time quantize-on-write of one new token per sequence for one layer.
 *   k_new, v_new: device bf16 [batch][n_kv_heads][128]
 *   pos:          device int32 [batch], the sequence length BEFORE this token
 * The token goes to residual slot pos mod 32; when that slot is 31 the 32 residual tokens
 * are quantized into page pos / 32 (its block-table entry must be set).  pos is not
 * advanced: the caller advances its lengths once after every layer has appended, so
 * repeating a call with the same pos is idempotent. */
kvq_status kvq_append(const kvq_model *model, int32_t layer, const kvq_layer_cache *cache,
                      const uint16_t *k_new, const uint16_t *v_new, const int32_t *pos,
                      void *stream);

/* Workspace bytes kvq_decode_attn needs for this batch, longest sequence and split size
 * (pages_per_split 0 = the library's choice, values above 256 act as 256). */
size_t kvq_decode_workspace_bytes(const kvq_model *model, int32_t batch, int32_t max_seq_len,
                                  int32_t pages_per_split);

/* Zeroes a decode workspace (a fill kernel on `stream`; no memset node, so it can be
 * captured in a graph).  A workspace must be zeroed once before its first use; every
 * decode call leaves it ready for the next. */
kvq_status kvq_workspace_init(void *workspace, size_t workspace_bytes, void *stream);

/* Single-token decode attention of one layer.
 *   q:        device [batch][n_q_heads][128], bf16 or fp32 (q_dtype); query head hq reads
 *             KV head hq / (n_q_heads / n_kv_heads)
 *   seq_len:  device int32 [batch]; attends over tokens 0 .. seq_len[b]-1 (full pages, then
 *             the residual); seq_len[b] must not exceed max_seq_len
 *   out:      device fp32 [batch][n_q_heads][128] = softmax(q K^T / sqrt(128)) V
 *   lse:      device fp32 [batch][n_q_heads], natural-log log-sum-exp of the scaled
 *             scores, or NULL
 *   A sequence of length 0 yields out = 0 and lse = -inf.
 *   pages_per_split: pages per split-K work item (0 = the library's choice; values above
 *   256 act as 256); the result depends on it only through floating-point rounding.
 *   workspace: device memory of at least kvq_decode_workspace_bytes(...) bytes, zeroed once
 *   before first use (kvq_workspace_init).  Calls that share a workspace must not overlap. */
kvq_status kvq_decode_attn(const kvq_model *model, int32_t layer, const kvq_layer_cache *cache,
                           kvq_dtype q_dtype, const void *q, const int32_t *seq_len,
                           int32_t max_seq_len, int32_t pages_per_split, float *out, float *lse,
                           void *workspace, size_t workspace_bytes, void *stream);

/* kvq_append followed by kvq_decode_attn over pos[b] + 1 tokens, in one launch.
 * Only the new token is quantized online, inside the attention step.
 *   [KVTuner OpenReview discussion, reply to reviewer 3, section 1 "Computational cost"]
 *   [KVTuner OpenReview discussion, reply to reviewer 2, section 1, "Throughput
 *    definition" (quantization overhead counts in throughput)]
 * Arguments as for kvq_append (k_new, v_new, pos) and kvq_decode_attn (the rest); there is
 * no seq_len: sequence b attends over pos[b] + 1 tokens, which must not exceed max_seq_len.
 * Afterwards the cache holds exactly what kvq_append leaves (same bytes): the token in
 * residual slot pos mod 32 and, when that slot is 31, the 32 residual tokens quantized into
 * page pos / 32 (its block-table entry must be set).  That page is attended as quantized.
 * The outputs equal kvq_decode_attn's after kvq_append up to floating-point rounding.  The
 * workspace is the one kvq_decode_workspace_bytes sizes for (batch, max_seq_len).  pos is
 * not advanced, so a repeated call with the same pos is idempotent.  pos[b] < 0 or
 * pos[b] + 1 > max_seq_len yields NaN outputs for that sequence. */
kvq_status kvq_append_decode_attn(const kvq_model *model, int32_t layer, const kvq_layer_cache *cache,
                                  const uint16_t *k_new, const uint16_t *v_new, const int32_t *pos,
                                  kvq_dtype q_dtype, const void *q, int32_t max_seq_len,
                                  int32_t pages_per_split, float *out, float *lse, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): kvq_append_decode_attn without a
 * workspace argument.  The split partials and split counters live in a device array of the
 * library (one per GPU, held until the process ends): KVQ_NOALLOC_MAX_COUNTERS counters at a
 * fixed place, which every call leaves at zero, then at most KVQ_NOALLOC_MAX_PARTIAL_BYTES of
 * partials.  The first call on a GPU zeroes that GPU's counters with a fill kernel on
 * `stream`.  Nothing is allocated: no hipMalloc, hipFree or allocating library routine.
 *   Arguments and results as for kvq_append_decode_attn.
 *   Returns KVQ_ERR_WORKSPACE when batch * n_kv_heads exceeds KVQ_NOALLOC_MAX_COUNTERS or
 *   the partials exceed KVQ_NOALLOC_MAX_PARTIAL_BYTES (kvq_noalloc_scratch_bytes gives their
 *   size), before anything is launched.  The KVQ_DEBUG checks (which wait for the stream)
 *   are not run.
 *   All calls on one GPU share the array: calls that overlap in time on one GPU (on
 *   different streams, or from different threads without ordering) race. */
#define KVQ_NOALLOC_MAX_COUNTERS 65536
#define KVQ_NOALLOC_MAX_PARTIAL_BYTES (32u << 20)
kvq_status kvq_append_decode_attn_noalloc(const kvq_model *model, int32_t layer, const kvq_layer_cache *cache,
                                          const uint16_t *k_new, const uint16_t *v_new, const int32_t *pos,
                                          kvq_dtype q_dtype, const void *q, int32_t max_seq_len,
                                          int32_t pages_per_split, float *out, float *lse, void *stream);

/* Partial bytes a kvq_append_decode_attn_noalloc call of this shape uses (compare with
 * KVQ_NOALLOC_MAX_PARTIAL_BYTES); 0 for an invalid model or shape. */
size_t kvq_noalloc_scratch_bytes(const kvq_model *model, int32_t batch, int32_t max_seq_len,
                                 int32_t pages_per_split);

#ifdef __cplusplus
}
#endif

#endif
