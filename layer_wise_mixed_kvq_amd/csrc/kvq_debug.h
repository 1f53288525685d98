// kvq_debug.h -- the KVQ_DEBUG checks run by the C ABI before a launch (host side).
#pragma once

#include "../../include/kvq.h"
#include "kvq_dequant.h"
#include "kvq_internal.h"

namespace kvq {

constexpr int kGroupTokens = KVQ_GROUP;
constexpr int kHeadDimElems = KVQ_HEAD_DIM;

// KVQ_DEBUG is set to anything but "" or "0"
bool debug_checks_enabled();
// KVQ_OK, KVQ_ERR_INVALID_ARG (a device-side precondition fails) or KVQ_ERR_HIP; each
// waits for `s`
kvq_status debug_check_pack(const PackParams &p, bool src_f32, hipStream_t s);
kvq_status debug_check_append(const AppendParams &p, hipStream_t s);
kvq_status debug_check_decode(const DecodeParams &p, bool q_f32, hipStream_t s);
kvq_status debug_check_dequant(const DequantParams &p, hipStream_t s);

}  // namespace kvq
