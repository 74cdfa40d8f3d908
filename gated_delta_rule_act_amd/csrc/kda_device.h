// Device helpers shared by the forward and backward sources of libkda.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda_device {
namespace {

// Raw buffer resource over [base, base + bytes): loads beyond the range return
// zero and stores beyond it are dropped by the hardware range check, so tail
// rows need no branches (and no branch-dependent wait counts).
// Every caller passes workgroup-uniform values; they are read from the first
// lane so the descriptor is built in scalar registers even where a uniform
// value was computed by a vector instruction (a clamp has no scalar form), as
// a descriptor in vector registers turns each load into a loop over lanes.
constexpr int kBufferWord3 = 0x00020000;  // gfx9-family raw buffer descriptor
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint64_t bu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)b);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(bu), (short)0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), kBufferWord3);
}

}  // namespace
}  // namespace kda_device
