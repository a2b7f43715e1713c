// Internal to the fp8kv library (not part of the C ABI).
#pragma once
#include <stdint.h>

namespace fp8kv_detail {
// records the hipError_t returned by fp8kv_last_hip_error() on this thread
void record_hip_error(int32_t e);
extern thread_local int32_t g_last_hip_error;
}  // namespace fp8kv_detail
