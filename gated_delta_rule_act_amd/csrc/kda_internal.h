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
// Time segments per state chain (dense input only; 1 = no split) and chunks
// per segment, from params->segments (0 = automatic).
constexpr int kMaxSegments = 256;
// Launch sizes: a dispatch dimension holds fewer than 2^32 work-items.  Chunk
// launches put one 256-thread workgroup per chunk along x (fewer than
// kMaxChunks chunks); state launches 4 per job, a job being a (sequence,
// head) pair or one of its segments (at most kMaxChains jobs); the segment
// combine 16 per pair (it runs with 3 segments or more).
constexpr int64_t kMaxChunks = (int64_t)1 << 24;
constexpr int64_t kMaxChains = (int64_t)1 << 21;
int seg_plan(const kda_fwd_params* p, bool packed, int* seg_len);
// Bytes of segment scratch for nseg segments (0 when nseg == 1).
size_t seg_scratch_bytes(const kda_fwd_params* p, int nseg);

}  // namespace kda_internal
