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


typedef uint32_t kd_u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t kd_u32x4 __attribute__((ext_vector_type(4)));

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes
// the 16 addresses are read as a 16 x 4 block M[s][e] of 16-bit values (4 at
// each address) and lane i receives M[4e + (i >> 2)][i & 3], e = 0..3.
template <typename T>
__device__ __forceinline__ kd_u32x2 lds_read_tr16(const T* p) {
  static_assert(sizeof(T) == 2, "16-bit elements");
  typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 fp16x4_t;
  auto lp = (__attribute__((address_space(3))) fp16x4_t*)(p);
  return __builtin_bit_cast(kd_u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4f16(lp));
}

// One 16 x 32 MFMA operand fragment with the contraction index contiguous per
// lane, read from a row-major [k][n] tile of 16-bit values whose rows are kept
// in groups of 8 (row stride ld within a group, group stride gs; k0 a
// multiple of 8): lane (i, g) receives column n0 + i, rows k0 + 8g .. k0 +
// 8g + 7.  Source lane s of a group points at row k0 + 8g + (s >> 2),
// columns n0 + 4 (s & 3).
template <typename T>
__device__ __forceinline__ kd_u32x4 lds_frag_tr_grouped(const T* tile, int ld, int gs, int k0, int n0, int lane) {
  const int i = lane & 15, g = lane >> 4;
  const T* p = tile + (k0 / 8 + g) * gs + (i >> 2) * ld + n0 + 4 * (i & 3);
  const kd_u32x2 a = lds_read_tr16(p), b = lds_read_tr16(p + 4 * ld);
  return kd_u32x4{a[0], a[1], b[0], b[1]};
}

}  // namespace
}  // namespace kda_device
