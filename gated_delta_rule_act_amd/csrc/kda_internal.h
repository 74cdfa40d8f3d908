// Host helpers shared by the forward and backward sources of libkda: the
// thread-local error string, parameter validation and workspace geometry.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda.h"

namespace kda_internal {

extern thread_local char g_last_error[512];
// Records a formatted message for kda_last_error() and returns s.
kda_status fail(kda_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// The parameter predicates shared by every entry point (shapes, gate mode,
// flags, lower bound, scale, state dtypes, segments).
kda_status check_params(const kda_fwd_params* p, bool packed);
// Upper bound on the 64-token chunks of the whole batch.
int64_t max_chunks_of(const kda_fwd_params* p, bool packed);
// Bytes of the workspace header (the int32 chunk map), padded to 256.
size_t header_bytes(const kda_fwd_params* p);
bool aligned16(const void* ptr);
// chunk_off[n] = first global chunk of packed sequence n, on the device.
void launch_chunk_map(const int64_t* cu, int N, int* chunk_off, hipStream_t st);
// KDA_ERR_LAUNCH if the runtime reports a launch error since the last check.
kda_status launch_status();

}  // namespace kda_internal
