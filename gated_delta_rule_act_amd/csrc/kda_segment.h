// Time segments of a state chain, shared by the forward and backward sources
// of libkda.  A chain of chunks whose state update is affine, X' = X M_c + B_c,
// is cut into segments that run in parallel: each segment's carry F[r] (the
// recurrence from zero) and map P[r] (from the identity with zero inputs)
// give the entry states S_in[r + 1] = S_in[r] P[r] + F[r].  Segments are
// numbered in the order the chain is processed (for a reverse recurrence,
// from its end).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace kda_segment {
namespace {

constexpr int SD = 128;  // the carried matrix is SD x SD

// What a state workgroup computes over its chunk range: the full pass (its
// per-chunk results and the state), the carry (the state only), or the map
// (the recurrence with its inputs set to zero, started from the identity).
constexpr int ST_FULL = 0, ST_CARRY = 1, ST_TRANS = 2;

// Segment scratch: fp32 [SD][SD] matrices, one per (chain, segment), in three
// planes: entry states, carries from zero, segment maps.
constexpr int SEG_SIN = 0, SEG_F = 1, SEG_P = 2;
__device__ __forceinline__ float* seg_mat(float* seg, int chains, int nseg, int plane, int chain, int r) {
  return seg + (((size_t)plane * chains + chain) * nseg + r) * (size_t)(SD * SD);
}

// Entry states S_in[r + 1] = S_in[r] P[r] + F[r] for r = 1..nseg-2 (S_in[1]
// is the first segment's exit state).  One workgroup per (chain, 8 rows);
// P[r] is staged in LDS, the 8 rows of S_in stay in LDS from step to step.
constexpr int CMB_ROWS = 8;
constexpr int CMB_XS = SD + 4;  // sX row stride: the two rows a wave reads sit on different banks
__global__ void __launch_bounds__(256)
kda_segment_combine_kernel(float* __restrict__ seg, int chains, int nseg) {
  __shared__ __attribute__((aligned(16))) float sP[SD * SD];
  __shared__ __attribute__((aligned(16))) float sX[CMB_ROWS * CMB_XS];
  const int chain = blockIdx.x / (SD / CMB_ROWS), rb = blockIdx.x % (SD / CMB_ROWS);
  if (chain >= chains) return;
  const int tid = threadIdx.x, row = tid >> 5, c0 = 4 * (tid & 31);
  const size_t off = (size_t)(rb * CMB_ROWS + row) * SD + c0;
  *reinterpret_cast<float4*>(&sX[row * CMB_XS + c0]) =
      *reinterpret_cast<const float4*>(seg_mat(seg, chains, nseg, SEG_SIN, chain, 1) + off);
  for (int r = 1; r + 1 < nseg; ++r) {
    const float* P = seg_mat(seg, chains, nseg, SEG_P, chain, r);
#pragma unroll
    for (int i = 0; i < SD * SD / 4 / 256; ++i) {
      const int e = tid + 256 * i;
      *reinterpret_cast<float4*>(&sP[4 * e]) = *reinterpret_cast<const float4*>(P + 4 * e);
    }
    float4 acc = *reinterpret_cast<const float4*>(seg_mat(seg, chains, nseg, SEG_F, chain, r) + off);
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < SD; ++k) {
      const float xk = sX[row * CMB_XS + k];
      const float4 pk = *reinterpret_cast<const float4*>(&sP[k * SD + c0]);
      acc.x += xk * pk.x; acc.y += xk * pk.y; acc.z += xk * pk.z; acc.w += xk * pk.w;
    }
    __syncthreads();  // every read of sX and sP of this step is done
    *reinterpret_cast<float4*>(&sX[row * CMB_XS + c0]) = acc;
    *reinterpret_cast<float4*>(seg_mat(seg, chains, nseg, SEG_SIN, chain, r + 1) + off) = acc;
  }
}

}  // namespace
}  // namespace kda_segment
