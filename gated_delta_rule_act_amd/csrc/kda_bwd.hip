// Chunked Kimi Delta Attention backward for MI355X (gfx950, CDNA4).
//
// Gradients of the forward in include/kda.h with respect to q, k, v, g, beta,
// A_log, dt_bias and the initial state, given the gradients of out and of the
// final state.  The fla-kda SKILL.md lists backward passes in its "Code map"
// and asks for forward, final-state and gradient coverage in "Validation";
// the pages do not print the backward, so it is derived here from the chunked
// forward (64-token chunks, per chunk with entry state S):
//     Akk = diag(b) (K K^T . E) strictly lower,  Aqk = (Q K^T . E) lower,
//     E_ij = e^(G_i - G_j) per key channel,  T = (I + Akk)^-1,  M = T diag(b),
//     W = M (K . e^G),  Ubar = M V,  U = Ubar - W S^T,
//     O = (Q . e^G) S^T + Aqk U,  S' = S Diag(e^G_last) + U^T (K . e^(G_last - G))
// (Q carries the output scale).  Reverse mode, with dO and dS' given:
//     dU  = Aqk^T dO + Kd dS'^T            dS  = dS' Diag(gn) + dO^T Qg - dU^T W
//     dQg = dO S      dKd = U dS'          dgn = colsum(dS' . S)
//     dAqk = dO U^T (lower)                dW  = -dU S
//     dM  = dU V^T + dW Kg^T               dV  = M^T dU      dKg = M^T dW
//     dT  = dM diag(b), db += colsum(dM . T),  dAkk = -(T^T dT T^T) (strictly lower)
// and the pairwise terms of Akk and Aqk into dK, dQ and dG, then dG to the
// per-token decay by a reverse cumulative sum, through the gate activation,
// the L2 norms and the beta sigmoid to the raw inputs.
//
// Six kernels (plus the chunk map for packed input, and the carry, map and
// combine launches of segmented state passes).  Values are fp32; the
// contractions over LDS operands run on the bf16 MFMA with each operand split
// into bf16 hi + lo (three products), or on the fp32 MFMA.  Every kernel but
// the reductions holds most of a CU's LDS, so each runs 8 waves (two per
// SIMD) in one workgroup:
//   kda_bwd_prep_kernel    per (chunk, v-head): norms, G, Akk and Aqk from
//                          factors e^(G_i - G_j) (pairs in different 16-row
//                          blocks factored through a reference row onto the
//                          MFMA; diagonal blocks through the block midpoint
//                          when the decay is bounded, else pair by pair with
//                          every exponent <= 0), T by blocked substitution,
//                          W, Ubar, Kd, Qg, Kg, gn -> workspace.
//   kda_bwd_fstate_kernel  per (sequence, v-head, 32-row V slice), forward
//                          over chunks: stores each chunk's entry state S and U.
//   kda_bwd_bstate_kernel  per (sequence, v-head, V slice), backward over
//                          chunks: stores dS' and dU, writes dS of the initial state.
//                          Both state passes may cut a long chain into time
//                          segments (carry, map and combine launches first).
//   kda_bwd_dense_kernel   per (chunk, v-head): the dense products above.
//   kda_bwd_pair_kernel    per (chunk, v-head): the pairwise terms, the
//                          elementwise factors, the decay cumulative sum, gate,
//                          norm and beta derivatives -> dq, dk, dv, dg, dbeta
//                          and per-chunk partials of dA_log and ddt_bias.
//   kda_bwd_reduce_kernel  sums q/k gradients over grouped v-heads and the
//                          per-chunk gate-parameter partials.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "kda.h"
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_segment.h"

namespace {
using namespace kda_internal;
using namespace kda_segment;
using namespace kda_device;

constexpr int CH = 64;
constexpr int DK = 128;
constexpr int DV = 128;
constexpr int RS = 132;  // LDS row stride of 128-wide fp32 tiles (rows 4 banks apart)
constexpr int QS = 68;   // LDS row stride of 64-wide fp32 tiles
constexpr int BV = 32;   // V rows per state workgroup
constexpr int BNS = DV / BV;
constexpr int64_t kBwdCUs = 256;   // compute units of an MI355X (persistent grids)
constexpr int PREP_THREADS = 512;  // 8 waves: two per SIMD beside the prep kernel's 157 KB of LDS
constexpr int PAIR_THREADS = 512;  // the same for the pair kernel (147 KB)
constexpr int DENSE_THREADS = 512;  // and for the dense kernel (152 KB)
constexpr int STATE_THREADS = 512;  // and for the state passes (94 and 154 KB)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kL2Eps = 1e-6f;
constexpr float kMinLog2Decay = -1.0e4f;

// Workspace, per (v-head, chunk) "chunk-head", all fp32 row-major:
// prep block (written by prep)
constexpr int PB_T = 0;                // T = (I + Akk)^-1       [64][64]
constexpr int PB_AQK = PB_T + 4096;    // Aqk (lower)            [64][64]
constexpr int PB_W = PB_AQK + 4096;    // W = M Kg               [64][128]
constexpr int PB_UB = PB_W + 8192;     // Ubar = M V             [64][128]
constexpr int PB_KD = PB_UB + 8192;    // Kd = K . e^(G_last-G)  [64][128]
constexpr int PB_QG = PB_KD + 8192;    // Qg = Q . e^G           [64][128]
constexpr int PB_KG = PB_QG + 8192;    // Kg = K . e^G           [64][128]
constexpr int PB_GN = PB_KG + 8192;    // gn = e^G_last          [128]
constexpr int PB_FLOATS = PB_GN + 128;
// state block (written by the two state passes)
constexpr int SB_H = 0;                // S entering the chunk   [128 v][128 k]
constexpr int SB_DH = SB_H + 16384;    // dS' after the chunk    [128][128]
constexpr int SB_U = SB_DH + 16384;    // U                      [64 t][128 v]
constexpr int SB_DU = SB_U + 8192;     // dU                     [64][128]
constexpr int SB_FLOATS = SB_DU + 8192;
// gradient block (written by dense, read by pair)
constexpr int GB_DQG = 0;              // dQg                    [64][128]
constexpr int GB_DKG = GB_DQG + 8192;  // dKg
constexpr int GB_DKD = GB_DKG + 8192;  // dKd
constexpr int GB_DAQK = GB_DKD + 8192; // dAqk (lower)           [64][64]
constexpr int GB_DAKK = GB_DAQK + 4096;// dAkk (strictly lower)  [64][64]
constexpr int GB_DGN = GB_DAKK + 4096; // dgn                    [128]
constexpr int GB_DB = GB_DGN + 128;    // db from dM . T         [64]
constexpr int GB_FLOATS = GB_DB + 64;
constexpr int GP_FLOATS = 192;         // gate partials per chunk-head: ddt_bias [128], dA_log [1], pad
constexpr size_t CHUNK_HEAD_FLOATS = (size_t)PB_FLOATS + SB_FLOATS + GB_FLOATS + GP_FLOATS;
static_assert(CHUNK_HEAD_FLOATS % 64 == 0, "chunk-head block alignment");

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float sigm(float x) { return 1.0f / (1.0f + __expf(-x)); }
__device__ __forceinline__ float softplus(float x) { return fmaxf(x, 0.0f) + log1pf(__expf(-fabsf(x))); }

// Gate activation a (natural log) and its derivatives d a / d x and
// d a / d A_log, for x = g + dt_bias.
template <int MODE>
__device__ __forceinline__ void gate_fwd_bwd(float x, float A_exp, float lb, float& a, float& dadx, float& dadA) {
  if constexpr (MODE == KDA_GATE_SOFTPLUS) {
    a = -A_exp * softplus(x);
    dadx = -A_exp * sigm(x);
    dadA = a;
  } else if constexpr (MODE == KDA_GATE_SAFE_SIGMOID) {
    const float z = A_exp * x, s = sigm(z);
    a = lb * s;
    dadx = lb * s * (1.0f - s) * A_exp;
    dadA = lb * s * (1.0f - s) * z;
  } else {
    a = x;
    dadx = 1.0f;
    dadA = 0.0f;
  }
}

struct ChunkLoc {
  int n;        // sequence
  int64_t row0; // first token row (b*T + t, or packed offset)
  int len;      // valid tokens (0 if the chunk index is past the last chunk)
};

// Global chunk x -> (sequence, first row, length).  Packed input: chunk_off
// holds each sequence's first global chunk (binary search).
__device__ __forceinline__ ChunkLoc chunk_loc(int x, const int64_t* cu, const int* chunk_off, int T, int N) {
  ChunkLoc L;
  if (cu == nullptr) {
    const int ncs = (T + CH - 1) / CH;
    L.n = ncs > 0 ? x / ncs : 0;
    const int c = ncs > 0 ? x % ncs : 0;
    L.row0 = (int64_t)L.n * T + (int64_t)c * CH;
    L.len = (L.n < N && ncs > 0) ? min(CH, T - c * CH) : 0;
  } else {
    if (x >= chunk_off[N]) { L.n = 0; L.row0 = 0; L.len = 0; return L; }
    int lo = 0, hi = N - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (chunk_off[mid] <= x) lo = mid; else hi = mid - 1;
    }
    L.n = lo;
    const int c = x - chunk_off[lo];
    L.row0 = cu[lo] + (int64_t)c * CH;
    L.len = (int)min((int64_t)CH, cu[lo + 1] - L.row0);
  }
  return L;
}

// 64 x 128 fp32 global tile (row stride gs floats) -> LDS rows of stride RS.
template <int NTH = 256>
__device__ __forceinline__ void load_tile128(float* s, const float* g, int gs, int tid) {
#pragma unroll
  for (int i = 0; i < 2048 / NTH; ++i) {
    const int e = tid + NTH * i, r = e >> 5, c = 4 * (e & 31);
    *reinterpret_cast<float4*>(s + r * RS + c) = *reinterpret_cast<const float4*>(g + (size_t)r * gs + c);
  }
}
// The same tile in two steps, so that the global loads can be issued ahead of
// the products that run before the tile's LDS space is free: fetch into
// registers, then put into LDS.  (Native vector types: with HIP's float4 and
// uint4 classes the compiler keeps such arrays in scratch memory.)
typedef float stage_f4 __attribute__((ext_vector_type(4)));
typedef uint32_t stage_u4 __attribute__((ext_vector_type(4)));
template <int NTH>
__device__ __forceinline__ void fetch_tile128(stage_f4 (&r4)[2048 / NTH], const float* g, int gs, int tid) {
#pragma unroll
  for (int i = 0; i < 2048 / NTH; ++i) {
    const int e = tid + NTH * i, r = e >> 5, c = 4 * (e & 31);
    r4[i] = *reinterpret_cast<const stage_f4*>(g + (size_t)r * gs + c);
  }
}
template <int NTH>
__device__ __forceinline__ void put_tile128(float* s, const stage_f4 (&r4)[2048 / NTH], int tid) {
#pragma unroll
  for (int i = 0; i < 2048 / NTH; ++i) {
    const int e = tid + NTH * i, r = e >> 5, c = 4 * (e & 31);
    *reinterpret_cast<stage_f4*>(s + r * RS + c) = r4[i];
  }
}
// 64 x 64 fp32 global tile (dense, stride 64) -> LDS rows of stride QS.
template <int NTH = 256>
__device__ __forceinline__ void load_tile64(float* s, const float* g, int tid) {
#pragma unroll
  for (int i = 0; i < 1024 / NTH; ++i) {
    const int e = tid + NTH * i, r = e >> 4, c = 4 * (e & 15);
    *reinterpret_cast<float4*>(s + r * QS + c) = *reinterpret_cast<const float4*>(g + r * 64 + c);
  }
}
template <int NTH>
__device__ __forceinline__ void fetch_tile64(stage_f4 (&r4)[1024 / NTH], const float* g, int tid) {
#pragma unroll
  for (int i = 0; i < 1024 / NTH; ++i) {
    const int e = tid + NTH * i, r = e >> 4, c = 4 * (e & 15);
    r4[i] = *reinterpret_cast<const stage_f4*>(g + r * 64 + c);
  }
}
template <int NTH>
__device__ __forceinline__ void put_tile64(float* s, const stage_f4 (&r4)[1024 / NTH], int tid) {
#pragma unroll
  for (int i = 0; i < 1024 / NTH; ++i) {
    const int e = tid + NTH * i, r = e >> 4, c = 4 * (e & 15);
    *reinterpret_cast<stage_f4*>(s + r * QS + c) = r4[i];
  }
}
// 64 rows x 128 bf16 (row stride gs elements; rows >= len read as zero) -> fp32 LDS.
// (range-checked buffer loads: rows >= len read as zero with no branch)
template <int NTH = 256>
__device__ __forceinline__ void load_bf16_tile128(float* s, const uint16_t* g, size_t gs, int len, int tid) {
  const __amdgpu_buffer_rsrc_t rg = buffer_rsrc(g, (uint32_t)((size_t)len * gs * 2));
#pragma unroll
  for (int i = 0; i < 1024 / NTH; ++i) {
    const int e = tid + NTH * i, r = e >> 4, c = 8 * (e & 15);
    const uint4 u = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rg, (uint32_t)(r * gs + c) * 2, 0, 0));
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    float* d = s + r * RS + c;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      d[2 * q] = __uint_as_float(w[q] << 16);
      d[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
    }
  }
}

// the same in two steps (fetch the raw bf16 into registers, put into LDS)
template <int NTH>
__device__ __forceinline__ void fetch_bf16_tile128(stage_u4 (&u4)[1024 / NTH], const uint16_t* g, size_t gs, int len,
                                                   int tid) {
  const __amdgpu_buffer_rsrc_t rg = buffer_rsrc(g, (uint32_t)((size_t)len * gs * 2));
#pragma unroll
  for (int i = 0; i < 1024 / NTH; ++i) {
    const int e = tid + NTH * i, r = e >> 4, c = 8 * (e & 15);
    u4[i] = __builtin_bit_cast(stage_u4, __builtin_amdgcn_raw_buffer_load_b128(rg, (uint32_t)(r * gs + c) * 2, 0, 0));
  }
}
template <int NTH>
__device__ __forceinline__ void put_bf16_tile128(float* s, const stage_u4 (&u4)[1024 / NTH], int tid) {
#pragma unroll
  for (int i = 0; i < 1024 / NTH; ++i) {
    const int e = tid + NTH * i, r = e >> 4, c = 8 * (e & 15);
    const uint32_t w[4] = {u4[i][0], u4[i][1], u4[i][2], u4[i][3]};
    float* d = s + r * RS + c;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      d[2 * q] = __uint_as_float(w[q] << 16);
      d[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
    }
  }
}

// Per chunk: q, k normalised (the output scale is applied by the callers),
// beta, and the chunk's cumulative log2-decay G, kept as a 16-row block-local
// inclusive sum sG plus the four block totals sBt[4][128]: every exponent is
// then composed from sums of nearby decays, never formed as the difference of
// two large cumulative values.  Rows past the sequence end: zero inputs,
// beta 0, zero decay.  Thread t: row t >> 2, channels 32 (t & 3) .. +31.
// Lane sums by DPP moves (no LDS): lanes paired by quad_perm [1,0,3,2] and
// [2,3,0,1], then the 4-lane halves of each 8 by row_half_mirror, then the
// 8-lane halves of each 16-lane row by row_mirror.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float sum8(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0x141>(x);
  return x;
}
__device__ __forceinline__ float sum16(float x) {
  x = sum8(x);
  return x + dpp_f<0x140>(x);
}

// The raw inputs of one chunk for thread t (row t / TPR, CPT channels): the
// global loads, kept apart from their processing so that a persistent
// kernel can issue the next chunk's loads while it works on the current one.
template <int NTH>
struct ChunkRaw {
  static constexpr int TPR = NTH / CH, CPT = DK / TPR;  // threads per row, channels per thread
  stage_u4 q[CPT / 8], k[CPT / 8], g[CPT / 8];
  stage_f4 db[CPT / 4];  // dt_bias of the thread's channels (zero when absent)
  uint32_t b;  // beta of the row (bf16 bits)
};
template <int NTH>
__device__ __forceinline__ void fetch_chunk_raw(ChunkRaw<NTH>& raw, const uint16_t* q, const uint16_t* k,
                                                const uint16_t* g, const uint16_t* beta, const float* dt_bias, int Hqk,
                                                int Hv, int h, int hq, int64_t row0, int len, int tid) {
  constexpr int TPR = ChunkRaw<NTH>::TPR, CPT = ChunkRaw<NTH>::CPT;
  const int r = tid / TPR, c0 = CPT * (tid % TPR);
  // range-checked buffer loads over the chunk's rows: rows >= len read as
  // zero, with no branch around the loads
  const __amdgpu_buffer_rsrc_t bq = buffer_rsrc(q + ((size_t)row0 * Hqk + hq) * DK, (uint32_t)len * Hqk * DK * 2);
  const __amdgpu_buffer_rsrc_t bk = buffer_rsrc(k + ((size_t)row0 * Hqk + hq) * DK, (uint32_t)len * Hqk * DK * 2);
  const __amdgpu_buffer_rsrc_t bg = buffer_rsrc(g + ((size_t)row0 * Hv + h) * DK, (uint32_t)len * Hv * DK * 2);
  const __amdgpu_buffer_rsrc_t bb = buffer_rsrc(beta + (size_t)row0 * Hv + h, (uint32_t)len * Hv * 2);
#pragma unroll
  for (int i = 0; i < CPT; i += 8) {
    const uint32_t oqk = (uint32_t)(r * Hqk * DK + c0 + i) * 2, og = (uint32_t)(r * Hv * DK + c0 + i) * 2;
    raw.q[i / 8] = __builtin_bit_cast(stage_u4, __builtin_amdgcn_raw_buffer_load_b128(bq, oqk, 0, 0));
    raw.k[i / 8] = __builtin_bit_cast(stage_u4, __builtin_amdgcn_raw_buffer_load_b128(bk, oqk, 0, 0));
    raw.g[i / 8] = __builtin_bit_cast(stage_u4, __builtin_amdgcn_raw_buffer_load_b128(bg, og, 0, 0));
  }
  raw.b = (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(bb, (uint32_t)(r * Hv) * 2, 0, 0);
  // dt_bias through a buffer of size 0 when absent: zeros, and no branch (a
  // conditional load became a branch with a full wait after it, per load)
  const __amdgpu_buffer_rsrc_t bd =
      buffer_rsrc(dt_bias ? dt_bias + (size_t)h * DK : dt_bias, dt_bias ? (uint32_t)DK * 4 : 0u);
#pragma unroll
  for (int i = 0; i < CPT; i += 4)
    raw.db[i / 4] = __builtin_bit_cast(stage_f4, __builtin_amdgcn_raw_buffer_load_b128(bd, (uint32_t)(c0 + i) * 4, 0, 0));
}

template <int MODE, int NTH>
__device__ __forceinline__ void process_chunk_inputs(const ChunkRaw<NTH>& raw, float* sK, float* sQ, float* sG,
                                                     float* sBt, float* sB, const float* A_log, int h, int len,
                                                     float lb, int flags, int tid, float* rq_out, float* rk_out) {
  constexpr int TPR = ChunkRaw<NTH>::TPR, CPT = ChunkRaw<NTH>::CPT;
  const int r = tid / TPR, c0 = CPT * (tid % TPR);
  const bool ok = r < len;
  float qv[CPT], kv[CPT], gv[CPT];
#pragma unroll
  for (int i = 0; i < CPT; i += 8) {
    const stage_u4 uq = raw.q[i / 8], uk = raw.k[i / 8], ug = raw.g[i / 8];
    const uint32_t wq[4] = {uq[0], uq[1], uq[2], uq[3]}, wk[4] = {uk[0], uk[1], uk[2], uk[3]}, wg[4] = {ug[0], ug[1], ug[2], ug[3]};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qv[i + 2 * j] = __uint_as_float(wq[j] << 16); qv[i + 2 * j + 1] = __uint_as_float(wq[j] & 0xffff0000u);
      kv[i + 2 * j] = __uint_as_float(wk[j] << 16); kv[i + 2 * j + 1] = __uint_as_float(wk[j] & 0xffff0000u);
      gv[i + 2 * j] = __uint_as_float(wg[j] << 16); gv[i + 2 * j + 1] = __uint_as_float(wg[j] & 0xffff0000u);
    }
  }
  float sq = 0.0f, sk = 0.0f;
#pragma unroll
  for (int i = 0; i < CPT; ++i) { sq += qv[i] * qv[i]; sk += kv[i] * kv[i]; }
  if constexpr (TPR == 8) {
    sq = sum8(sq);
    sk = sum8(sk);
  } else {
#pragma unroll
    for (int m = 1; m < TPR; m *= 2) { sq += __shfl_xor(sq, m); sk += __shfl_xor(sk, m); }
  }
  const bool norm = flags & KDA_FLAG_QK_L2NORM;
  const float rq = norm ? rsqrtf(sq + kL2Eps) : 1.0f, rk = norm ? rsqrtf(sk + kL2Eps) : 1.0f;
  if (rq_out) { rq_out[0] = rq; rk_out[0] = rk; }
  const float A_exp = (MODE == KDA_GATE_PREGATED || A_log == nullptr) ? 1.0f : __expf(A_log[h]);
#pragma unroll
  for (int i = 0; i < CPT; i += 4) {
    float g4[4];
    const float db[4] = {raw.db[i / 4][0], raw.db[i / 4][1], raw.db[i / 4][2], raw.db[i / 4][3]};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // every row's gate (zero inputs past the end, finite), then the select:
      // a branch around each element's exponentials costs more
      float a, d1, d2;
      gate_fwd_bwd<MODE>(gv[i + e] + db[e], A_exp, lb, a, d1, d2);
      g4[e] = fmaxf((ok ? a : 0.0f) * kLog2e, kMinLog2Decay);
    }
    *reinterpret_cast<float4*>(sQ + r * RS + c0 + i) =
        make_float4(qv[i] * rq, qv[i + 1] * rq, qv[i + 2] * rq, qv[i + 3] * rq);
    *reinterpret_cast<float4*>(sK + r * RS + c0 + i) =
        make_float4(kv[i] * rk, kv[i + 1] * rk, kv[i + 2] * rk, kv[i + 3] * rk);
    *reinterpret_cast<float4*>(sG + r * RS + c0 + i) = make_float4(g4[0], g4[1], g4[2], g4[3]);
  }
  if (tid % TPR == 0) {
    const float braw = bf2f((uint16_t)raw.b);
    const float bp = (flags & KDA_FLAG_BETA_IS_PROB) ? braw : sigm(braw);
    sB[r] = ok ? bp : 0.0f;
  }
  __syncthreads();
  // block-local inclusive sums: thread t owns channel t & 127 and BPT of the
  // four 16-row blocks; all 16 rows read first, summed in registers, written back
  {
    constexpr int BPT = 4 * DK / NTH;
    const int c = tid & 127;
#pragma unroll
    for (int B = BPT * (tid >> 7); B < BPT * (tid >> 7) + BPT; ++B) {
      float x[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) x[rr] = sG[(16 * B + rr) * RS + c];
#pragma unroll
      for (int rr = 1; rr < 16; ++rr) x[rr] += x[rr - 1];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sG[(16 * B + rr) * RS + c] = x[rr];
      sBt[B * DK + c] = x[15];
    }
  }
  __syncthreads();
}

// fetch and process in one go
template <int MODE, int NTH = 256>
__device__ __forceinline__ void load_chunk_inputs(float* sK, float* sQ, float* sG, float* sBt, float* sB, const uint16_t* q,
                                                  const uint16_t* k, const uint16_t* g, const uint16_t* beta,
                                                  const float* A_log, const float* dt_bias, int Hqk, int Hv, int h,
                                                  int hq, int64_t row0, int len, float lb, int flags,
                                                  int tid, float* rq_out, float* rk_out) {
  ChunkRaw<NTH> raw;
  fetch_chunk_raw<NTH>(raw, q, k, g, beta, dt_bias, Hqk, Hv, h, hq, row0, len, tid);
  process_chunk_inputs<MODE, NTH>(raw, sK, sQ, sG, sBt, sB, A_log, h, len, lb, flags, tid, rq_out, rk_out);
}

// Exponents from the block-local form (log2 units):
//   G_i (from the chunk start) and G_last - G_i
__device__ __forceinline__ float gabs(const float* sG, const float* sBt, int i, int c) {
  float d = sG[i * RS + c];
  for (int B = 0; B < (i >> 4); ++B) d += sBt[B * DK + c];
  return d;
}
__device__ __forceinline__ float gtail(const float* sG, const float* sBt, int i, int c) {
  const int I = i >> 4;
  float d = sBt[I * DK + c] - sG[i * RS + c];
  for (int B = I + 1; B < 4; ++B) d += sBt[B * DK + c];
  return d;
}

// ---------------------------------------------------------------------------
// fp32 MFMA (16x16x4) blocks with operands in LDS.  Lane (li = lane & 15,
// lg = lane >> 4) feeds A[li][k + lg] and B[k + lg][li] and receives
// C[4 lg + r][li] (r < 4) of each 16 x 16 tile.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// acc[m][n] += the (16 m, 16 n) tile of A B over k < kdim (a multiple of
// 32), operands fp32 in LDS:
//   A(r, k) = AT ? sA[k * lda + r] : sA[r * lda + k]
//   B(k, c) = BT ? sB[c * ldb + k] : sB[k * ldb + c]
// on the bf16 MFMA (16x16x32) with each operand split as x = hi + lo (both
// bf16, round to nearest even) and three products hi.hi + hi.lo + lo.hi:
// fp32-level accuracy (relative ~2^-16 per product) at the bf16 matrix rate.
// Lane (li, g = lane >> 4) feeds A[li][8 g .. 8 g + 7] and B[8 g .. +7][li].
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void split8(const float (&x)[8], bf16x8_t& hi, bf16x8_t& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = (__bf16)x[e];
    hi[e] = h;
    lo[e] = (__bf16)(x[e] - (float)h);
  }
}

// Which 8 of a 32-wide k step lane group g feeds is a free choice as long as
// A and B agree.  When both operands are read along rows (A(r, k) with k
// contiguous, B^T likewise) the group takes 8 consecutive k, two 16-byte LDS
// reads per operand; otherwise it takes k = 4 e + g, so that the strided reads
// of the four groups fall on different banks.
template <bool AT, bool BT, int MT, int NT>
__device__ __forceinline__ void mfma_block(f32x4 (&acc)[MT][NT], const float* sA, int lda, const float* sB, int ldb,
                                           int row0, int col0, int kdim, int lane) {
  constexpr bool kContig = !AT && BT;
  const int li = lane & 15, g = lane >> 4;
#pragma unroll 2
  for (int k0 = 0; k0 < kdim; k0 += 32) {
    bf16x8_t ah[MT], al[MT], bh[NT], bl[NT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int r = row0 + 16 * m + li;
      float x[8];
      if constexpr (kContig) {
        const float4 u0 = *reinterpret_cast<const float4*>(sA + r * lda + k0 + 8 * g);
        const float4 u1 = *reinterpret_cast<const float4*>(sA + r * lda + k0 + 8 * g + 4);
        x[0] = u0.x; x[1] = u0.y; x[2] = u0.z; x[3] = u0.w; x[4] = u1.x; x[5] = u1.y; x[6] = u1.z; x[7] = u1.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int k = k0 + 4 * e + g;
          x[e] = AT ? sA[k * lda + r] : sA[r * lda + k];
        }
      }
      split8(x, ah[m], al[m]);
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int c = col0 + 16 * n + li;
      float x[8];
      if constexpr (kContig) {
        const float4 u0 = *reinterpret_cast<const float4*>(sB + c * ldb + k0 + 8 * g);
        const float4 u1 = *reinterpret_cast<const float4*>(sB + c * ldb + k0 + 8 * g + 4);
        x[0] = u0.x; x[1] = u0.y; x[2] = u0.z; x[3] = u0.w; x[4] = u1.x; x[5] = u1.y; x[6] = u1.z; x[7] = u1.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int k = k0 + 4 * e + g;
          x[e] = BT ? sB[c * ldb + k] : sB[k * ldb + c];
        }
      }
      split8(x, bh[n], bl[n]);
    }
    // one product over all tiles at a time, so consecutive MFMAs write
    // different accumulators and none waits on the previous one's result
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[m], bh[n], acc[m][n], 0, 0, 0);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[m], bl[n], acc[m][n], 0, 0, 0);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[m], bh[n], acc[m][n], 0, 0, 0);
  }
}

// Pre-split operands.  A tile that several waves read as split-bf16 MFMA
// operands is stored once as two bf16 tiles, hi = bf16(x) and lo = bf16(x -
// hi) (the split of mfma_block), so that no reader splits it again.  Rows are
// kept in groups of 8 (row stride ld, group stride gs, in elements).  A tile
// read down its columns (the transposing LDS read) takes ld = 144 (or 48 for
// 32 columns) and a 64-element gap between groups, so that the lane groups of
// one read fall on different banks; a tile read only along its rows takes
// ld = 136 and no gap.
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
struct PsTile {
  __bf16* hi;
  __bf16* lo;
  int ld, gs;
  __device__ __forceinline__ int row(int r) const { return (r & 7) * ld + (r >> 3) * gs; }
};
constexpr int PS_ROW_LD = 136;                    // tiles read along rows
constexpr int PS_COL_LD = 144, PS_COL_GS = 8 * PS_COL_LD + 64;  // 128-column tiles read down columns
constexpr int PS_C32_LD = 48, PS_C32_GS = 8 * PS_C32_LD + 64;   // 32-column tiles read down columns
constexpr int PS_C64_LD = 80, PS_C64_GS = 8 * PS_C64_LD + 64;   // 64-column tiles read down columns
// 32-column tiles read down columns, unpadded: the four rows of a lane group
// lie 16 banks apart and the next group of rows 8 banks further (64 banks)
constexpr int PS_N32_LD = 32, PS_N32_GS = 8 * PS_N32_LD + 16;

__device__ __forceinline__ void ps_put1(const PsTile& t, int r, int c, float x) {
  const __bf16 h = (__bf16)x;
  t.hi[t.row(r) + c] = h;
  t.lo[t.row(r) + c] = (__bf16)(x - (float)h);
}
// four consecutive values of row r from column c (a multiple of 4)
__device__ __forceinline__ void ps_put4(const PsTile& t, int r, int c, const stage_f4& x) {
  bf16x4_t h, l;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = (__bf16)x[e];
    l[e] = (__bf16)(x[e] - (float)h[e]);
  }
  *reinterpret_cast<bf16x4_t*>(t.hi + t.row(r) + c) = h;
  *reinterpret_cast<bf16x4_t*>(t.lo + t.row(r) + c) = l;
}
// a fetched 64 x 128 fp32 tile (fetch_tile128's thread layout) into a split tile
template <int NTH>
__device__ __forceinline__ void put_ps_tile128(const PsTile& t, const stage_f4 (&r4)[2048 / NTH], int tid) {
#pragma unroll
  for (int i = 0; i < 2048 / NTH; ++i) {
    const int e = tid + NTH * i;
    ps_put4(t, e >> 5, 4 * (e & 31), r4[i]);
  }
}

// a 64 x 128 fp32 global tile (row stride gs floats) straight into a split tile
template <int NTH>
__device__ __forceinline__ void load_ps_tile128(const PsTile& t, const float* g, int gs, int tid) {
#pragma unroll
  for (int i = 0; i < 2048 / NTH; ++i) {
    const int e = tid + NTH * i, r = e >> 5, c = 4 * (e & 31);
    ps_put4(t, r, c, *reinterpret_cast<const stage_f4*>(g + (size_t)r * gs + c));
  }
}
// 64 rows x 128 bf16 (row stride gs elements; rows >= len read as zero) into a
// split tile: the values are bf16 already, so hi is the value and lo zero
template <int NTH>
__device__ __forceinline__ void load_ps_bf16_tile128(const PsTile& t, const uint16_t* g, size_t gs, int len, int tid) {
  const __amdgpu_buffer_rsrc_t rg = buffer_rsrc(g, (uint32_t)((size_t)len * gs * 2));
#pragma unroll
  for (int i = 0; i < 1024 / NTH; ++i) {
    const int e = tid + NTH * i, r = e >> 4, c = 8 * (e & 15);
    const stage_u4 u = __builtin_bit_cast(stage_u4, __builtin_amdgcn_raw_buffer_load_b128(rg, (uint32_t)(r * gs + c) * 2, 0, 0));
    *reinterpret_cast<stage_u4*>(t.hi + t.row(r) + c) = u;
    *reinterpret_cast<stage_u4*>(t.lo + t.row(r) + c) = stage_u4{0u, 0u, 0u, 0u};
  }
}

// a fetched 64 x 64 fp32 tile (fetch_tile64's thread layout) into a split tile
template <int NTH>
__device__ __forceinline__ void put_ps_tile64(const PsTile& t, const stage_f4 (&r4)[1024 / NTH], int tid) {
#pragma unroll
  for (int i = 0; i < 1024 / NTH; ++i) {
    const int e = tid + NTH * i;
    ps_put4(t, e >> 4, 4 * (e & 15), r4[i]);
  }
}

// acc[m][n] += the (16 m, 16 n) tile of A B over k < kdim (a multiple of 32)
// from split tiles, A(r, k) = AT ? tA[k][r] : tA[r][k] and B(k, c) = BT ?
// tB[c][k] : tB[k][c]: lane (li, g) feeds A[li][8 g .. +7] and B[8 g .. +7][li],
// read along a row (16 bytes per half) or down a column (transposing reads),
// and the three products of mfma_block.
template <bool AT, bool BT, int MT, int NT>
__device__ __forceinline__ void mfma_block_ps(f32x4 (&acc)[MT][NT], const PsTile& A, const PsTile& B, int row0,
                                              int col0, int kdim, int lane) {
  const int li = lane & 15, g = lane >> 4;
#pragma unroll 2
  for (int k0 = 0; k0 < kdim; k0 += 32) {
    bf16x8_t ah[MT], al[MT], bh[NT], bl[NT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if constexpr (AT) {
        ah[m] = __builtin_bit_cast(bf16x8_t, lds_frag_tr_grouped(A.hi, A.ld, A.gs, k0, row0 + 16 * m, lane));
        al[m] = __builtin_bit_cast(bf16x8_t, lds_frag_tr_grouped(A.lo, A.ld, A.gs, k0, row0 + 16 * m, lane));
      } else {
        const int o = A.row(row0 + 16 * m + li) + k0 + 8 * g;
        ah[m] = *reinterpret_cast<const bf16x8_t*>(A.hi + o);
        al[m] = *reinterpret_cast<const bf16x8_t*>(A.lo + o);
      }
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      if constexpr (BT) {
        const int o = B.row(col0 + 16 * n + li) + k0 + 8 * g;
        bh[n] = *reinterpret_cast<const bf16x8_t*>(B.hi + o);
        bl[n] = *reinterpret_cast<const bf16x8_t*>(B.lo + o);
      } else {
        bh[n] = __builtin_bit_cast(bf16x8_t, lds_frag_tr_grouped(B.hi, B.ld, B.gs, k0, col0 + 16 * n, lane));
        bl[n] = __builtin_bit_cast(bf16x8_t, lds_frag_tr_grouped(B.lo, B.ld, B.gs, k0, col0 + 16 * n, lane));
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[m], bh[n], acc[m][n], 0, 0, 0);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[m], bl[n], acc[m][n], 0, 0, 0);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[m], bh[n], acc[m][n], 0, 0, 0);
  }
}

// Products with one operand pre-split and the other in fp32 (split as it is
// read).  Every operand reader gives lane (li, g) the 8 consecutive k from
// k0 + 8 g, so the two sides agree.  F32Tile: fp32 rows of stride ld.
struct F32Tile {
  const float* s;
  int ld;
};
// A(r, k) or B^T(c, k) along a row (T = false) / down a column (T = true) of
// the tile: the fragment for index x0 + li (row for T = false, column for T = true)
template <bool T>
__device__ __forceinline__ void opnd_frag(const F32Tile& t, int x0, int k0, int lane, bf16x8_t& hi, bf16x8_t& lo) {
  const int li = lane & 15, g = lane >> 4;
  float x[8];
  if constexpr (!T) {
    const float4 u0 = *reinterpret_cast<const float4*>(t.s + (x0 + li) * t.ld + k0 + 8 * g);
    const float4 u1 = *reinterpret_cast<const float4*>(t.s + (x0 + li) * t.ld + k0 + 8 * g + 4);
    x[0] = u0.x; x[1] = u0.y; x[2] = u0.z; x[3] = u0.w; x[4] = u1.x; x[5] = u1.y; x[6] = u1.z; x[7] = u1.w;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = t.s[(k0 + 8 * g + e) * t.ld + x0 + li];
  }
  split8(x, hi, lo);
}
template <bool T>
__device__ __forceinline__ void opnd_frag(const PsTile& t, int x0, int k0, int lane, bf16x8_t& hi, bf16x8_t& lo) {
  if constexpr (!T) {
    const int o = t.row(x0 + (lane & 15)) + k0 + 8 * (lane >> 4);
    hi = *reinterpret_cast<const bf16x8_t*>(t.hi + o);
    lo = *reinterpret_cast<const bf16x8_t*>(t.lo + o);
  } else {
    hi = __builtin_bit_cast(bf16x8_t, lds_frag_tr_grouped(t.hi, t.ld, t.gs, k0, x0, lane));
    lo = __builtin_bit_cast(bf16x8_t, lds_frag_tr_grouped(t.lo, t.ld, t.gs, k0, x0, lane));
  }
}
// acc[m][n] += the (16 m, 16 n) tile of A B over k < kdim (a multiple of 32):
// A(r, k) = AT ? tA[k][r] : tA[r][k], B(k, c) = BT ? tB[c][k] : tB[k][c], each
// tile fp32 (F32Tile) or pre-split (PsTile); the three products of mfma_block.
template <bool AT, bool BT, int MT, int NT, class TA, class TB>
__device__ __forceinline__ void mfma_block_mix(f32x4 (&acc)[MT][NT], const TA& A, const TB& B, int row0, int col0,
                                               int kdim, int lane) {
#pragma unroll 2
  for (int k0 = 0; k0 < kdim; k0 += 32) {
    bf16x8_t ah[MT], al[MT], bh[NT], bl[NT];
#pragma unroll
    for (int m = 0; m < MT; ++m) opnd_frag<AT>(A, row0 + 16 * m, k0, lane, ah[m], al[m]);
#pragma unroll
    for (int n = 0; n < NT; ++n) opnd_frag<!BT>(B, col0 + 16 * n, k0, lane, bh[n], bl[n]);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[m], bh[n], acc[m][n], 0, 0, 0);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[m], bl[n], acc[m][n], 0, 0, 0);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[m], bh[n], acc[m][n], 0, 0, 0);
  }
}

// The same product on the fp32 MFMA (16x16x4): lane (li, lg) feeds
// A[li][k + lg] and B[k + lg][li] for each 4-wide k step.  Used where the
// operands are read across rows only and the chain of products is short.
template <bool AT, bool BT, int MT, int NT>
__device__ __forceinline__ void mfma_block_f32(f32x4 (&acc)[MT][NT], const float* sA, int lda, const float* sB,
                                               int ldb, int row0, int col0, int kdim, int lane) {
  const int li = lane & 15, lg = lane >> 4;
#pragma unroll 8
  for (int k = 0; k < kdim; k += 4) {
    const int kk = k + lg;
    float a[MT], b[NT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int r = row0 + 16 * m + li;
      a[m] = AT ? sA[kk * lda + r] : sA[r * lda + kk];
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int c = col0 + 16 * n + li;
      b[n] = BT ? sB[c * ldb + kk] : sB[kk * ldb + c];
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m], b[n], acc[m][n], 0, 0, 0);
  }
}

template <int MT, int NT>
__device__ __forceinline__ void zero_block(f32x4 (&acc)[MT][NT]) {
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// element (row, col) of block tile (m, n, r): the lane's layout above
#define BLK_ROW(row0, m, r) ((row0) + 16 * (m) + 4 * lg + (r))
#define BLK_COL(col0, n) ((col0) + 16 * (n) + li)

// ---------------------------------------------------------------------------
// prep: per (chunk, v-head) forward quantities in fp32
template <int MODE>
__global__ void __launch_bounds__(PREP_THREADS)
kda_bwd_prep_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                    const uint16_t* __restrict__ g, const uint16_t* __restrict__ beta, const float* __restrict__ A_log,
                    const float* __restrict__ dt_bias, const int64_t* __restrict__ cu, const int* __restrict__ chunk_off,
                    int T, int N, int Hqk, int Hv, int mc, float scale, float lb, int flags, float* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) float sK[CH * RS];
  __shared__ __attribute__((aligned(16))) float sQ[CH * RS];
  __shared__ __attribute__((aligned(16))) float sG[CH * RS];
  __shared__ __attribute__((aligned(16))) float sA[CH * QS];
  __shared__ __attribute__((aligned(16))) float sAq[CH * QS];
  __shared__ __attribute__((aligned(16))) float sT[CH * QS];
  __shared__ float sB[CH];
  __shared__ float sX[2 * 16 * 17];
  __shared__ __attribute__((aligned(16))) float sBt[4 * DK];
  // Persistent: workgroup b takes the chunk-heads b, b + gridDim.x, ...
  // (chunk-head id = v-head * mc + chunk), and the raw inputs of the next one
  // are fetched into registers while the current one runs, so that their
  // latency is not exposed at one workgroup per CU.
  const int tid0 = threadIdx.x, total = mc * Hv;
  ChunkRaw<PREP_THREADS> raw;
  stage_u4 rawv[1024 / PREP_THREADS];  // the chunk's V tile (bf16)
  auto fetch = [&](int id) {
    const int x2 = id % mc, h2 = id / mc;
    const ChunkLoc L2 = chunk_loc(x2, cu, chunk_off, T, N);
    fetch_chunk_raw<PREP_THREADS>(raw, q, k, g, beta, dt_bias, Hqk, Hv, h2, h2 / (Hv / Hqk), L2.row0, L2.len, tid0);
    fetch_bf16_tile128<PREP_THREADS>(rawv, v + ((size_t)L2.row0 * Hv + h2) * DV, (size_t)Hv * DV, L2.len, tid0);
  };
  if ((int)blockIdx.x < total) fetch(blockIdx.x);
  for (int id = blockIdx.x; id < total; id += gridDim.x) {
  // the thread index is renewed opaquely every chunk-head, so the compiler
  // does not hoist the body's index arithmetic out of the loop and hold it in
  // registers across the whole body
  int tid = tid0;
  asm volatile("" : "+v"(tid));
  const int x = id % mc, h = id / mc;
  const ChunkLoc L = chunk_loc(x, cu, chunk_off, T, N);
  const int nxt = id + (int)gridDim.x;
  if (L.len == 0) {
    if (nxt < total) fetch(nxt);
    continue;
  }
  const int hq = h / (Hv / Hqk);
  float* pb = ws + ((size_t)h * mc + x) * CHUNK_HEAD_FLOATS;

  for (int e = tid; e < CH * QS; e += PREP_THREADS) { sA[e] = 0.0f; sAq[e] = 0.0f; sT[e] = 0.0f; }
  process_chunk_inputs<MODE, PREP_THREADS>(raw, sK, sQ, sG, sBt, sB, A_log, h, L.len, lb, flags, tid, nullptr,
                                           nullptr);
  stage_u4 vcur[1024 / PREP_THREADS];  // this chunk's V, kept until it goes to LDS
#pragma unroll
  for (int i = 0; i < 1024 / PREP_THREADS; ++i) vcur[i] = rawv[i];
  if (nxt < total) fetch(nxt);

  // Akk and Aqk.  Each off-diagonal block (I, J), J < I, is formed in two
  // halves over the channels, twelve tasks in all; waves 0..3 also sum the
  // diagonal block w.  With the safe gate a diagonal block costs about half
  // an off-diagonal one, so waves 0..3 take one half-block each and waves
  // 4..7 two; with unbounded decays the pairwise diagonal is the heavy part,
  // and waves 4..7 take three half-blocks each.  Waves w and w + 4 share a
  // SIMD, so either way every SIMD gets about the same work.  An off-diagonal
  // block factors through the row before block I:
  // e^(G_i - G_j) = e^(sG_i) e^(Bt_J - sG_j + sum_{J<B<I} Bt_B), both
  // exponents <= 0, so it is one fp32 MFMA product over the channels (A = K
  // or Q times the row factor, B = K times the column factor).  The first
  // half goes to sA / sAq, the second to sT (Akk part below the diagonal,
  // Aqk part transposed above it, both unused until the solve), and waves
  // 4..7 add the two while waves 0..3 solve the diagonal blocks.
  {
    // (the wave index through readfirstlane: the compiler then knows it is
    // uniform, and tests and loops on it are scalar branches, not exec masks)
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), li = lane & 15, lg = lane >> 4;
    constexpr bool kSafe = MODE == KDA_GATE_SAFE_SIGMOID;
    const int t0 = kSafe ? (w < 4 ? w : 4 + 2 * (w - 4)) : 3 * (w - 4);
    const int ntask = kSafe ? (w < 4 ? 1 : 2) : (w < 4 ? 0 : 3);
    for (int task = t0; task < t0 + ntask; ++task) {
      // blocks (1,0) (2,0) (2,1) (3,0) (3,1) (3,2), two channel halves each
      const int blk = task >> 1, hc = task & 1;
      const int I = blk == 0 ? 1 : blk < 3 ? 2 : 3;
      const int J = blk == 0 ? 0 : blk < 3 ? blk - 1 : blk - 3;
      f32x4 akk = f32x4{0.f, 0.f, 0.f, 0.f}, aqk = akk;
      const int i = 16 * I + li, j = 16 * J + li;
#pragma unroll 4
      for (int kc = 64 * hc; kc < 64 * hc + 64; kc += 4) {
        const int c = kc + lg;
        const float fr = ex2(sG[i * RS + c]);
        float mid = sBt[J * DK + c];
        for (int B = J + 1; B < I; ++B) mid += sBt[B * DK + c];
        const float zb = sK[j * RS + c] * ex2(mid - sG[j * RS + c]);
        akk = __builtin_amdgcn_mfma_f32_16x16x4f32(sK[i * RS + c] * fr, zb, akk, 0, 0, 0);
        aqk = __builtin_amdgcn_mfma_f32_16x16x4f32(sQ[i * RS + c] * fr, zb, aqk, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ii = 16 * I + 4 * lg + r, jj = 16 * J + li;
        if (hc == 0) {
          sA[ii * QS + jj] = sB[ii] * akk[r];
          sAq[ii * QS + jj] = scale * aqk[r];
        } else {
          sT[ii * QS + jj] = sB[ii] * akk[r];
          sT[jj * QS + ii] = scale * aqk[r];
        }
      }
    }
    if (w >= 4) {
      // waves 4..7: off-diagonal half-blocks only
    } else if constexpr (MODE == KDA_GATE_SAFE_SIGMOID) {
      // diagonal block, bounded decay: e^(G_i - G_j) = e^(sG_i - sG_m) e^(sG_m - sG_j)
      // with m the block's row 8, each factor within 2^(8 |lb| log2 e) of one:
      // one fp32 MFMA product over the channels, masked on store
      f32x4 akk = f32x4{0.f, 0.f, 0.f, 0.f}, aqk = akk;
      const int i = 16 * w + li, m = 16 * w + 8;
#pragma unroll 4
      for (int kc = 0; kc < DK; kc += 4) {
        const int c = kc + lg;
        const float gm = sG[m * RS + c], gi = sG[i * RS + c];
        const float fr = ex2(gi - gm), fc = ex2(gm - gi);  // row i and column i of the block
        const float zb = sK[i * RS + c] * fc;
        akk = __builtin_amdgcn_mfma_f32_16x16x4f32(sK[i * RS + c] * fr, zb, akk, 0, 0, 0);
        aqk = __builtin_amdgcn_mfma_f32_16x16x4f32(sQ[i * RS + c] * fr, zb, aqk, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ii = 16 * w + 4 * lg + r, jj = 16 * w + li;
        sA[ii * QS + jj] = jj < ii ? sB[ii] * akk[r] : 0.0f;
        sAq[ii * QS + jj] = jj <= ii ? scale * aqk[r] : 0.0f;
      }
    } else {
      // diagonal block: the 136 pairs i >= j of block w, two or three per lane
      for (int pr = lane; pr < 136; pr += 64) {
        int ii = (int)((sqrtf(8.0f * pr + 1.0f) - 1.0f) * 0.5f);
        while ((ii + 1) * (ii + 2) / 2 <= pr) ++ii;
        while (ii * (ii + 1) / 2 > pr) --ii;
        const int jj = pr - ii * (ii + 1) / 2;
        const int i = 16 * w + ii, j = 16 * w + jj;
        float akk = 0.0f, aqk = 0.0f;
#pragma unroll 4
        for (int c = 0; c < DK; c += 4) {
          const float4 ki = *reinterpret_cast<const float4*>(sK + i * RS + c);
          const float4 qi = *reinterpret_cast<const float4*>(sQ + i * RS + c);
          const float4 gi = *reinterpret_cast<const float4*>(sG + i * RS + c);
          const float4 kj = *reinterpret_cast<const float4*>(sK + j * RS + c);
          const float4 gj = *reinterpret_cast<const float4*>(sG + j * RS + c);
          const float e0 = kj.x * ex2(fminf(gi.x - gj.x, 0.0f)), e1 = kj.y * ex2(fminf(gi.y - gj.y, 0.0f));
          const float e2 = kj.z * ex2(fminf(gi.z - gj.z, 0.0f)), e3 = kj.w * ex2(fminf(gi.w - gj.w, 0.0f));
          akk += ki.x * e0 + ki.y * e1 + ki.z * e2 + ki.w * e3;
          aqk += qi.x * e0 + qi.y * e1 + qi.z * e2 + qi.w * e3;
        }
        sA[i * QS + j] = jj < ii ? sB[i] * akk : 0.0f;
        sAq[i * QS + j] = scale * aqk;
      }
    }
  }
  __syncthreads();

  // T = (I + Akk)^-1: the four 16 x 16 diagonal blocks by forward
  // substitution (one wave each, lane = column), then block rows 1..3
  {
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    if (w >= 4) {
      // the second channel halves of the off-diagonal blocks, out of sT
      const int e = tid - 256;
#pragma unroll
      for (int blk = 0; blk < 6; ++blk) {
        const int I = blk == 0 ? 1 : blk < 3 ? 2 : 3;
        const int J = blk == 0 ? 0 : blk < 3 ? blk - 1 : blk - 3;
        const int ii = 16 * I + (e >> 4), jj = 16 * J + (e & 15);
        sA[ii * QS + jj] += sT[ii * QS + jj];
        sAq[ii * QS + jj] += sT[jj * QS + ii];
        sT[ii * QS + jj] = 0.0f;
        sT[jj * QS + ii] = 0.0f;
      }
    }
    if (w < 4 && lane < 16) {
      // the lane's column of the block stays in registers (zero above the
      // diagonal: those rows only ever subtract products with zeros)
      const int base = 16 * w, cc = lane;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = i == cc ? 1.0f : 0.0f;
#pragma unroll
        for (int j = 0; j < i; ++j) acc -= sA[(base + i) * QS + base + j] * x[j];
        x[i] = i >= cc ? acc : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sT[(base + i) * QS + base + cc] = x[i];
    }
  }
  __syncthreads();
  {
    // block row I: the blocks J < I are independent given rows < I, so up
    // to two are formed at once, 256 threads each (element (r, c))
    const int r = (tid >> 4) & 15, c = tid & 15, half = tid >> 8;
    float* sXh = sX + half * (16 * 17);
    for (int I = 1; I < 4; ++I)
      for (int J0 = 0; J0 < I; J0 += 2) {
        const int J = J0 + half;
        const bool act = J < I;
        // X = sum_{K=J}^{I-1} A_IK T_KJ;  T_IJ = -T_II X
        if (act) {
          float xacc = 0.0f;
          for (int kk = 16 * J; kk < 16 * I; ++kk) xacc += sA[(16 * I + r) * QS + kk] * sT[kk * QS + 16 * J + c];
          sXh[r * 17 + c] = xacc;
        }
        __syncthreads();
        if (act) {
          float t = 0.0f;
#pragma unroll
          for (int m = 0; m < 16; ++m) t += sT[(16 * I + r) * QS + 16 * I + m] * sXh[m * 17 + c];
          sT[(16 * I + r) * QS + 16 * J + c] = -t;
        }
        __syncthreads();
      }
  }

  // store T and Aqk
#pragma unroll
  for (int i = 0; i < 1024 / PREP_THREADS; ++i) {
    const int e = tid + PREP_THREADS * i, r = e >> 4, c = 4 * (e & 15);
    *reinterpret_cast<float4*>(pb + PB_T + r * 64 + c) = *reinterpret_cast<const float4*>(sT + r * QS + c);
    *reinterpret_cast<float4*>(pb + PB_AQK + r * 64 + c) = *reinterpret_cast<const float4*>(sAq + r * QS + c);
  }
  // Kd, Qg, Kg, gn: element e = tid + PREP_THREADS i is row e >> 5, channels 4 (e & 31)
  // .. +3, so the 32 lanes of a row store 512 contiguous bytes
  __syncthreads();  // Kg overwrites sK rows that other threads still read above
  constexpr int KIT = 2048 / PREP_THREADS;
  float4 kgv[KIT];
#pragma unroll
  for (int it = 0; it < KIT; ++it) {
    const int e = tid + PREP_THREADS * it, r = e >> 5, c = 4 * (e & 31);
    const float4 kk = *reinterpret_cast<const float4*>(sK + r * RS + c);
    const float4 qq = *reinterpret_cast<const float4*>(sQ + r * RS + c);
    float eg[4], ed[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) { eg[u] = ex2(gabs(sG, sBt, r, c + u)); ed[u] = ex2(gtail(sG, sBt, r, c + u)); }
    *reinterpret_cast<float4*>(pb + PB_KD + r * DK + c) =
        make_float4(kk.x * ed[0], kk.y * ed[1], kk.z * ed[2], kk.w * ed[3]);
    *reinterpret_cast<float4*>(pb + PB_QG + r * DK + c) =
        make_float4(scale * qq.x * eg[0], scale * qq.y * eg[1], scale * qq.z * eg[2], scale * qq.w * eg[3]);
    kgv[it] = make_float4(kk.x * eg[0], kk.y * eg[1], kk.z * eg[2], kk.w * eg[3]);
    *reinterpret_cast<float4*>(pb + PB_KG + r * DK + c) = kgv[it];
  }
  if (tid < 32)
    *reinterpret_cast<float4*>(pb + PB_GN + 4 * tid) =
        make_float4(ex2(gabs(sG, sBt, 63, 4 * tid)), ex2(gabs(sG, sBt, 63, 4 * tid + 1)),
                    ex2(gabs(sG, sBt, 63, 4 * tid + 2)), ex2(gabs(sG, sBt, 63, 4 * tid + 3)));
  __syncthreads();
#pragma unroll
  for (int it = 0; it < KIT; ++it) {  // sK now holds Kg
    const int e = tid + PREP_THREADS * it, r = e >> 5, c = 4 * (e & 31);
    *reinterpret_cast<float4*>(sK + r * RS + c) = kgv[it];
  }
  __syncthreads();
  // sQ <- V (fetched with the chunk's other inputs); sT <- M = T diag(b)
  put_bf16_tile128<PREP_THREADS>(sQ, vcur, tid);
  for (int e = tid; e < CH * CH; e += PREP_THREADS) {
    const int r = e >> 6, c = e & 63;
    sT[r * QS + c] *= sB[c];
  }
  __syncthreads();
  // W = M Kg, Ubar = M V (split-bf16 MFMA; wave w: rows 32 (w >> 2) .., columns 32 (w & 3) ..)
  {
    const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6), li = lane & 15, lg = lane >> 4;
    const int R0 = 32 * (wv >> 2), C0 = 32 * (wv & 3);
    f32x4 w[2][2], u[2][2];
    zero_block(w);
    zero_block(u);
    mfma_block<false, false, 2, 2>(w, sT, QS, sK, RS, R0, C0, CH, lane);
    mfma_block<false, false, 2, 2>(u, sT, QS, sQ, RS, R0, C0, CH, lane);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = R0 + 16 * m + 4 * lg + r, c = C0 + 16 * n + li;
          pb[PB_W + t * DK + c] = w[m][n][r];
          pb[PB_UB + t * DV + c] = u[m][n][r];
        }
  }
  __syncthreads();  // the next chunk-head rewrites every LDS array
  }
}

// ---------------------------------------------------------------------------
// state passes: one workgroup per (sequence, v-head, 32-row V slice).  The
// 32 x 128 slice of the state (or of its gradient) lives in MFMA accumulator
// layout: wave w (of 8) holds key columns 16 w .. +15 for all 32 rows,
// element (v = 16 m + 4 lg + r, k = 16 w + li) in acc[m][0][r].

__device__ __forceinline__ void chain_chunks(int n, const int* chunk_off, const int64_t* cu, int T, int& x0, int& nc,
                                             int64_t& bos) {
  if (cu == nullptr) {
    const int ncs = (T + CH - 1) / CH;
    x0 = n * ncs; nc = ncs; bos = (int64_t)n * T;
  } else {
    x0 = chunk_off[n]; nc = chunk_off[n + 1] - x0; bos = cu[n];
  }
}

// slice <-> [128][128] fp32 matrix g (rows v0 ..), and <-> LDS [32][RS]
__device__ __forceinline__ void slice_to_global(const f32x4 (&S)[2][1], float* g, int v0, int w, int li, int lg) {
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) g[(size_t)(v0 + 16 * m + 4 * lg + r) * DK + 16 * w + li] = S[m][0][r];
}

// XCD-aware decode: the BNS slices of one chain share (id mod 8), so they run
// on one XCD and read the chain's chunk operands through its L2.
__device__ __forceinline__ void chain_slice(int id, int& chain, int& slice) {
  chain = (id / (8 * BNS)) * 8 + (id & 7);
  slice = (id >> 3) % BNS;
}

// Both state passes are affine in the carried matrix X (rows v, columns k):
//   forward   S   -> S (Diag(gn) - W^T Kd) + Ubar^T Kd
//   backward  dS' -> dS' (Diag(gn) - Kd^T W) + dO^T (Qg - Aqk W)
// so a long chain is cut into time segments as in the forward state launch:
// carries from zero, maps from the identity with zero inputs, a combine, then
// the full pass of every segment from its true entry.  Segments are numbered
// in processing order (the backward pass starts at the end of the sequence).
// Jobs (chain, r), BNS workgroups per job:
//   ST_FULL  r = 0..nseg-1 with the per-chunk stores, from the true entry
//            (nseg == 1) or from S_in[r];
//   ST_CARRY r = 0..nseg-2: r = 0 from the true entry (also copied to S_in[0])
//            into S_in[1], r >= 1 from zero into F[r];
//   ST_TRANS r = 1..nseg-2: from the identity into P[r].
template <int KIND>
__device__ __forceinline__ int jobs_per_chain(int nseg) {
  return KIND == ST_FULL ? nseg : KIND == ST_CARRY ? nseg - 1 : nseg - 2;
}

struct StateJob {
  int chain, r, n, h, v0;
  int x0, c0, c1;  // workspace index of the chain's first chunk; this job's chunks c0 .. c1-1
  int64_t bos;
};

// false: the workgroup has no job.  With `reverse`, processing segment r
// covers time segment nseg-1-r.
template <int KIND>
__device__ __forceinline__ bool state_job(int id, const int64_t* cu, const int* chunk_off, int T, int N, int Hv,
                                          int nseg, int seg_len, bool reverse, StateJob& j) {
  const int jpc = jobs_per_chain<KIND>(nseg);
  int job, slice;
  chain_slice(id, job, slice);
  if (job >= N * Hv * jpc) return false;
  j.chain = job / jpc;
  j.r = job % jpc + (KIND == ST_TRANS ? 1 : 0);
  j.n = j.chain / Hv;
  j.h = j.chain % Hv;
  j.v0 = BV * slice;
  int nc;
  chain_chunks(j.n, chunk_off, cu, T, j.x0, nc, j.bos);
  j.c0 = 0;
  j.c1 = nc;
  if (nseg > 1) {
    const int ts = reverse ? nseg - 1 - j.r : j.r;
    j.c0 = min(nc, ts * seg_len);
    j.c1 = min(nc, j.c0 + seg_len);
  }
  return true;
}

__device__ __forceinline__ void slice_identity(f32x4 (&S)[2][1], int v0, int w, int li, int lg) {
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) S[m][0][r] = v0 + 16 * m + 4 * lg + r == 16 * w + li ? 1.0f : 0.0f;
}

// the slice of a [128][128] matrix: fp32, bf16, or zero (KDA_STATE_NONE / NULL).
// Range-checked loads under one branch on the (uniform) dtype: an absent
// matrix is a buffer of size 0 and reads zeros (conditional loads per element
// became a branch with a full wait after each)
__device__ __forceinline__ void slice_from_global(f32x4 (&S)[2][1], const void* g, int dtype, int v0, int w, int li,
                                                  int lg) {
  const bool f32 = g != nullptr && dtype == KDA_STATE_F32, b16 = g != nullptr && dtype == KDA_STATE_BF16;
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(g, f32 ? (uint32_t)DV * DK * 4 : b16 ? (uint32_t)DV * DK * 2 : 0u);
  if (b16) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t e = (uint32_t)(v0 + 16 * m + 4 * lg + r) * DK + 16 * w + li;
        S[m][0][r] = bf2f((uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rs, e * 2, 0, 0));
      }
  } else {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t e = (uint32_t)(v0 + 16 * m + 4 * lg + r) * DK + 16 * w + li;
        S[m][0][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, e * 4, 0, 0));
      }
  }
}

// Entry slice of a job; `entry` is the chain's true entry matrix.
template <int KIND>
__device__ __forceinline__ void job_entry(f32x4 (&S)[2][1], const StateJob& j, const void* entry, int dtype,
                                          float* seg, int chains, int nseg, int w, int li, int lg) {
  if (KIND == ST_TRANS) {
    slice_identity(S, j.v0, w, li, lg);
  } else if (KIND == ST_FULL && nseg > 1) {
    slice_from_global(S, seg_mat(seg, chains, nseg, SEG_SIN, j.chain, j.r), KDA_STATE_F32, j.v0, w, li, lg);
  } else if (KIND == ST_CARRY && j.r > 0) {
    slice_from_global(S, nullptr, KDA_STATE_NONE, j.v0, w, li, lg);
  } else {
    slice_from_global(S, entry, dtype, j.v0, w, li, lg);
    if (KIND == ST_CARRY) slice_to_global(S, seg_mat(seg, chains, nseg, SEG_SIN, j.chain, 0), j.v0, w, li, lg);
  }
}

// where a carry or map job leaves its matrix
template <int KIND>
__device__ __forceinline__ float* job_exit(float* seg, int chains, int nseg, const StateJob& j) {
  return KIND == ST_TRANS ? seg_mat(seg, chains, nseg, SEG_P, j.chain, j.r)
         : j.r == 0       ? seg_mat(seg, chains, nseg, SEG_SIN, j.chain, 1)
                          : seg_mat(seg, chains, nseg, SEG_F, j.chain, j.r);
}

// Register staging of a chunk's operands: the backward state pass fetches
// the next chunk's tiles into registers while the current chunk's products
// run, and moves them to LDS after the chunk's last barrier.
constexpr int ST128 = 2048 / STATE_THREADS, ST64 = 1024 / STATE_THREADS;  // 16-byte pieces per thread
__device__ __forceinline__ void fetch_tile128(f32x4 (&r)[ST128], const float* g, int tid) {
#pragma unroll
  for (int i = 0; i < ST128; ++i) {
    const int e = tid + STATE_THREADS * i;
    r[i] = *reinterpret_cast<const f32x4*>(g + (size_t)(e >> 5) * DK + 4 * (e & 31));
  }
}
__device__ __forceinline__ void put_tile128(float* s, const f32x4 (&r)[ST128], int tid) {
#pragma unroll
  for (int i = 0; i < ST128; ++i) {
    const int e = tid + STATE_THREADS * i;
    *reinterpret_cast<f32x4*>(s + (e >> 5) * RS + 4 * (e & 31)) = r[i];
  }
}
__device__ __forceinline__ void fetch_tile64(f32x4 (&r)[ST64], const float* g, int tid) {
#pragma unroll
  for (int i = 0; i < ST64; ++i) {
    const int e = tid + STATE_THREADS * i;
    r[i] = *reinterpret_cast<const f32x4*>(g + (e >> 4) * 64 + 4 * (e & 15));
  }
}
__device__ __forceinline__ void put_tile64(float* s, const f32x4 (&r)[ST64], int tid) {
#pragma unroll
  for (int i = 0; i < ST64; ++i) {
    const int e = tid + STATE_THREADS * i;
    *reinterpret_cast<f32x4*>(s + (e >> 4) * QS + 4 * (e & 15)) = r[i];
  }
}

template <int KIND>
__global__ void __launch_bounds__(STATE_THREADS)
kda_bwd_fstate_kernel(const int64_t* __restrict__ cu, const int* __restrict__ chunk_off, const void* __restrict__ h0,
                      int init_dtype, int T, int N, int Hv, int mc, float* __restrict__ ws, float* __restrict__ seg,
                      int nseg, int seg_len) {
  // pre-split operand tiles: W and the state slice read along rows, U and Kd
  // down columns
  __shared__ __attribute__((aligned(16))) __bf16 sWh[CH * PS_ROW_LD], sWl[CH * PS_ROW_LD];
  __shared__ __attribute__((aligned(16))) __bf16 sKdh[CH / 8 * PS_COL_GS], sKdl[CH / 8 * PS_COL_GS];
  __shared__ __attribute__((aligned(16))) __bf16 sUh[CH / 8 * PS_C32_GS], sUl[CH / 8 * PS_C32_GS];
  __shared__ __attribute__((aligned(16))) __bf16 sSh[BV * PS_ROW_LD], sSl[BV * PS_ROW_LD];
  const PsTile tW{sWh, sWl, PS_ROW_LD, 8 * PS_ROW_LD}, tKd{sKdh, sKdl, PS_COL_LD, PS_COL_GS};
  const PsTile tU{sUh, sUl, PS_C32_LD, PS_C32_GS}, tS{sSh, sSl, PS_ROW_LD, 8 * PS_ROW_LD};
  StateJob j;
  if (!state_job<KIND>(blockIdx.x, cu, chunk_off, T, N, Hv, nseg, seg_len, false, j)) return;
  const int chains = N * Hv, h = j.h, v0 = j.v0, tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), li = lane & 15, lg = lane >> 4;
  // wave w: state columns 16 w .. +15; U rows 16 (w & 3) .., columns 16 (w >> 2) ..
  const int ut = 16 * (w & 3), uv = 16 * (w >> 2);
  f32x4 S[2][1];
  job_entry<KIND>(S, j, h0 == nullptr ? nullptr : reinterpret_cast<const char*>(h0) +
                                                      (size_t)j.chain * DV * DK * (init_dtype == KDA_STATE_BF16 ? 2 : 4),
                  init_dtype, seg, chains, nseg, w, li, lg);
  // every global operand of a chunk (W, Kd, the Ubar tile and gn) is fetched
  // into registers one chunk ahead, so a chunk step waits on memory only for
  // loads issued a whole step earlier
  f32x4 fW[ST128], fKd[ST128];
  f32x4 fUb = f32x4{0.f, 0.f, 0.f, 0.f};
  float fgn = 0.0f;
  auto fetch = [&](int c) {
    const float* pb = ws + ((size_t)h * mc + j.x0 + c) * CHUNK_HEAD_FLOATS;
    fetch_tile128(fW, pb + PB_W, tid);
    fetch_tile128(fKd, pb + PB_KD, tid);
    // U rows 16 w .. +15 start from -Ubar (lane layout of the product below);
    // a map job has no inputs, Ubar = 0
    if constexpr (KIND != ST_TRANS) {
#pragma unroll
      for (int r = 0; r < 4; ++r) fUb[r] = pb[PB_UB + (ut + 4 * lg + r) * DV + v0 + uv + li];
    }
    fgn = pb[PB_GN + 16 * w + li];
  };
  if (j.c0 < j.c1) fetch(j.c0);
  for (int c = j.c0; c < j.c1; ++c) {
    const float* pb = ws + ((size_t)h * mc + j.x0 + c) * CHUNK_HEAD_FLOATS;
    float* sb = const_cast<float*>(pb) + PB_FLOATS;
    if constexpr (KIND == ST_FULL) slice_to_global(S, sb + SB_H, v0, w, li, lg);
    // the state slice S[v][k] (v = 16 m + 4 lg + r, k = 16 w + li)
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) ps_put1(tS, 16 * m + 4 * lg + r, 16 * w + li, S[m][0][r]);
    put_ps_tile128<STATE_THREADS>(tW, fW, tid);
    put_ps_tile128<STATE_THREADS>(tKd, fKd, tid);
    f32x4 U[1][1];
    U[0][0] = -fUb;
    const float gn = fgn;
    fetch(min(c + 1, j.c1 - 1));
    __syncthreads();
    // -U = W S^T - Ubar:  A(t, k) = W[t][k],  B(k, v) = S[v][k]
    mfma_block_ps<false, true, 1, 1>(U, tW, tS, ut, uv, DK, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = ut + 4 * lg + r, vv = uv + li;
      const float u = -U[0][0][r];
      ps_put1(tU, t, vv, u);
      if constexpr (KIND == ST_FULL) sb[SB_U + t * DV + v0 + vv] = u;
    }
    __syncthreads();
    // S <- S Diag(gn) + U^T Kd:  A(v, t) = U[t][v],  B(t, k) = Kd[t][k]
#pragma unroll
    for (int m = 0; m < 2; ++m) S[m][0] *= gn;
    mfma_block_ps<true, false, 2, 1>(S, tU, tKd, 0, 16 * w, CH, lane);
    __syncthreads();
  }
  if constexpr (KIND != ST_FULL) slice_to_global(S, job_exit<KIND>(seg, chains, nseg, j), v0, w, li, lg);
}

// (native vector types: staging arrays of them stay in registers)
struct BStage {
  f32x4 kd[ST128], w[ST128], qg[ST128], aq[ST64];
  u32x2 dO;  // bf16: token tid >> 3, columns v0 + 4 (tid & 7) .. +3
  float gn;
};

template <int KIND>
__device__ __forceinline__ void bstate_fetch(BStage& b, const float* pb, const uint16_t* d_out, int64_t row0, int len,
                                             int Hv, int h, int v0, int tid, int w, int li) {
  fetch_tile128(b.kd, pb + PB_KD, tid);
  fetch_tile128(b.w, pb + PB_W, tid);
  if constexpr (KIND != ST_TRANS) {
    fetch_tile128(b.qg, pb + PB_QG, tid);
    fetch_tile64(b.aq, pb + PB_AQK, tid);
    const int t = tid >> 3;
    b.dO = u32x2{0u, 0u};
    if (t < len) b.dO = *reinterpret_cast<const u32x2*>(d_out + ((size_t)(row0 + t) * Hv + h) * DV + v0 + 4 * (tid & 7));
  }
  b.gn = pb[PB_GN + 16 * w + li];
}

template <int KIND>
__global__ void __launch_bounds__(STATE_THREADS)
kda_bwd_bstate_kernel(const uint16_t* __restrict__ d_out, const float* __restrict__ dhT, float* __restrict__ dh0,
                      const int64_t* __restrict__ cu, const int* __restrict__ chunk_off, int T, int N, int Hv, int mc,
                      float* __restrict__ ws, float* __restrict__ seg, int nseg, int seg_len) {
  __shared__ __attribute__((aligned(16))) float sQg[CH * RS];
  __shared__ __attribute__((aligned(16))) float sW[CH * RS];
  // pre-split: dO and dU (every wave reads all of both), the dS' slice (four
  // waves read each part), Kd and Aqk (two); Qg and W (one wave each) stay
  // fp32, as the CU's LDS holds no more
  __shared__ __attribute__((aligned(16))) __bf16 sdOh[CH / 8 * PS_N32_GS], sdOl[CH / 8 * PS_N32_GS];
  __shared__ __attribute__((aligned(16))) __bf16 sdUh[CH / 8 * PS_N32_GS], sdUl[CH / 8 * PS_N32_GS];
  __shared__ __attribute__((aligned(16))) __bf16 sdhh[BV * PS_ROW_LD], sdhl[BV * PS_ROW_LD];
  __shared__ __attribute__((aligned(16))) __bf16 sKdh[CH * PS_ROW_LD], sKdl[CH * PS_ROW_LD];
  __shared__ __attribute__((aligned(16))) __bf16 sAqh[CH / 8 * PS_C64_GS], sAql[CH / 8 * PS_C64_GS];
  const PsTile tdO{sdOh, sdOl, PS_N32_LD, PS_N32_GS}, tdU{sdUh, sdUl, PS_N32_LD, PS_N32_GS};
  const PsTile tdh{sdhh, sdhl, PS_ROW_LD, 8 * PS_ROW_LD}, tKd{sKdh, sKdl, PS_ROW_LD, 8 * PS_ROW_LD};
  const PsTile tAq{sAqh, sAql, PS_C64_LD, PS_C64_GS};
  const F32Tile tQg{sQg, RS}, tW{sW, RS};
  StateJob j;
  if (!state_job<KIND>(blockIdx.x, cu, chunk_off, T, N, Hv, nseg, seg_len, true, j)) return;
  const int chains = N * Hv, h = j.h, v0 = j.v0, tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), li = lane & 15, lg = lane >> 4;
  const int64_t seqlen = cu == nullptr ? (int64_t)T : cu[j.n + 1] - cu[j.n];
  const size_t sbase = (size_t)j.chain * DV * DK;
  // wave w: gradient columns 16 w .. +15; dU rows 16 (w & 3) .., columns 16 (w >> 2) ..
  const int ut = 16 * (w & 3), uv = 16 * (w >> 2);
  f32x4 D[2][1];
  job_entry<KIND>(D, j, dhT == nullptr ? nullptr : dhT + sbase, KDA_STATE_F32, seg, chains, nseg, w, li, lg);
  const float* pb0 = ws + ((size_t)h * mc + j.x0) * CHUNK_HEAD_FLOATS;
  auto chunk_len = [&](int c) { return (int)min((int64_t)CH, seqlen - (int64_t)c * CH); };
  BStage b;
  if (j.c0 < j.c1) {
    const int c = j.c1 - 1;
    bstate_fetch<KIND>(b, pb0 + (size_t)c * CHUNK_HEAD_FLOATS, d_out, j.bos + (int64_t)c * CH, chunk_len(c), Hv, h,
                       v0, tid, w, li);
  }
  for (int c = j.c1 - 1; c >= j.c0; --c) {
    float* sb = const_cast<float*>(pb0) + (size_t)c * CHUNK_HEAD_FLOATS + PB_FLOATS;
    if constexpr (KIND == ST_FULL) slice_to_global(D, sb + SB_DH, v0, w, li, lg);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) ps_put1(tdh, 16 * m + 4 * lg + r, 16 * w + li, D[m][0][r]);
    put_ps_tile128<STATE_THREADS>(tKd, b.kd, tid);
    put_tile128(sW, b.w, tid);
    if constexpr (KIND != ST_TRANS) {
      put_tile128(sQg, b.qg, tid);
      put_ps_tile64<STATE_THREADS>(tAq, b.aq, tid);
      const int t = tid >> 3, jj = 4 * (tid & 7);
      ps_put4(tdO, t, jj,
              stage_f4{__uint_as_float(b.dO[0] << 16), __uint_as_float(b.dO[0] & 0xffff0000u),
                       __uint_as_float(b.dO[1] << 16), __uint_as_float(b.dO[1] & 0xffff0000u)});
    }
    const float gn = b.gn;
    __syncthreads();
    if (c - 1 >= j.c0)
      bstate_fetch<KIND>(b, pb0 + (size_t)(c - 1) * CHUNK_HEAD_FLOATS, d_out, j.bos + (int64_t)(c - 1) * CH,
                         chunk_len(c - 1), Hv, h, v0, tid, w, li);
    // dU rows 16 w .. +15:  Aqk^T dO  +  Kd dS'^T  (a map job has dO = 0)
    f32x4 dU[1][1];
    zero_block(dU);
    if constexpr (KIND != ST_TRANS) mfma_block_mix<true, false, 1, 1>(dU, tAq, tdO, ut, uv, CH, lane);
    mfma_block_mix<false, true, 1, 1>(dU, tKd, tdh, ut, uv, DK, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = ut + 4 * lg + r, vv = uv + li;
      ps_put1(tdU, t, vv, -dU[0][0][r]);
      if constexpr (KIND == ST_FULL) sb[SB_DU + t * DV + v0 + vv] = dU[0][0][r];
    }
    __syncthreads();
    // dS = dS' Diag(gn) + dO^T Qg - dU^T W:  A(v, t) = dO[t][v] (then -dU[t][v])
#pragma unroll
    for (int m = 0; m < 2; ++m) D[m][0] *= gn;
    if constexpr (KIND != ST_TRANS) mfma_block_mix<true, false, 2, 1>(D, tdO, tQg, 0, 16 * w, CH, lane);
    mfma_block_mix<true, false, 2, 1>(D, tdU, tW, 0, 16 * w, CH, lane);
    __syncthreads();
  }
  if constexpr (KIND == ST_FULL) {
    if (dh0 && j.r == nseg - 1) slice_to_global(D, dh0 + sbase, v0, w, li, lg);
  } else {
    slice_to_global(D, job_exit<KIND>(seg, chains, nseg, j), v0, w, li, lg);
  }
}

// ---------------------------------------------------------------------------
// dense products per (chunk, v-head), on the split-bf16 MFMA.  Lane
// (li = lane & 15, lg = lane >> 4) receives C[4 lg + r][li] (r < 4) of each
// 16 x 16 tile.  Wave w (of 8) computes rows 32 (w >> 2) .. +31 of every
// product: columns 32 (w & 3) .. +31 of the 128-wide ones, 16 (w & 3) .. +15
// of the 64-wide ones.
__global__ void __launch_bounds__(DENSE_THREADS)
kda_bwd_dense_kernel(const uint16_t* __restrict__ v, const uint16_t* __restrict__ d_out,
                     const uint16_t* __restrict__ beta, const int64_t* __restrict__ cu,
                     const int* __restrict__ chunk_off, int T, int N, int Hv, int mc, int flags,
                     float* __restrict__ dv, float* __restrict__ ws) {
  // B0 (dO, then dS', then Kg), B1 (dU) and B3 (S, then dW) are read by the
  // most waves and products: they are kept pre-split; B2 and T stay fp32
  // (all five pre-split would not fit a CU's LDS)
  __shared__ __attribute__((aligned(16))) __bf16 B0h[CH * PS_ROW_LD], B0l[CH * PS_ROW_LD];
  __shared__ __attribute__((aligned(16))) __bf16 B1h[CH * PS_ROW_LD], B1l[CH * PS_ROW_LD];
  __shared__ __attribute__((aligned(16))) float B2[CH * RS];
  __shared__ __attribute__((aligned(16))) __bf16 B3h[CH * PS_ROW_LD], B3l[CH * PS_ROW_LD];
  __shared__ __attribute__((aligned(16))) float sT[CH * QS];
  __shared__ float sB[CH];
  const PsTile tB0{B0h, B0l, PS_ROW_LD, 8 * PS_ROW_LD}, tB1{B1h, B1l, PS_ROW_LD, 8 * PS_ROW_LD};
  const PsTile tB0v{B0h + 64, B0l + 64, PS_ROW_LD, 8 * PS_ROW_LD}, tB1v{B1h + 64, B1l + 64, PS_ROW_LD, 8 * PS_ROW_LD};
  const PsTile tB3{B3h, B3l, PS_ROW_LD, 8 * PS_ROW_LD};
  const F32Tile fB2{B2, RS}, fB2v{B2 + 64, RS}, fT{sT, QS};
  const int x = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const ChunkLoc L = chunk_loc(x, cu, chunk_off, T, N);
  if (L.len == 0) return;
  float* pb = ws + ((size_t)h * mc + x) * CHUNK_HEAD_FLOATS;
  float* sb = pb + PB_FLOATS;
  float* gb = sb + SB_FLOATS;
  // wave w: rows 32 (w >> 2) .. of every output, columns 32 (w & 3) .. of the
  // 128-wide ones and 16 (w & 3) .. of the 64-wide ones
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), li = lane & 15, lg = lane >> 4;
  const int R0 = 32 * (w >> 2), C0 = 32 * (w & 3), Q0 = 16 * (w & 3);
  constexpr int NTH = DENSE_THREADS;

  // 1. dO, dU, U and the first half of S (rows v < 64)
  load_ps_bf16_tile128<NTH>(tB0, d_out + ((size_t)L.row0 * Hv + h) * DV, (size_t)Hv * DV, L.len, tid);
  load_ps_tile128<NTH>(tB1, sb + SB_DU, DV, tid);
  load_tile128<NTH>(B2, sb + SB_U, DV, tid);
  // the first half of S also stays in registers, for step 4's column sums
  // (rows (tid >> 5) + 16 i, channels 4 (tid & 31): the put's layout)
  stage_f4 s1[2048 / NTH];
  fetch_tile128<NTH>(s1, sb + SB_H, DK, tid);
  put_ps_tile128<NTH>(tB3, s1, tid);
  // Each later single-tile reload is fetched into registers one phase early
  // and put into LDS once its space is free, so its latency hides behind the
  // products in between: pf holds the second half of S now, then the two
  // halves of dS' (second half first), then Kg (with pv = V and pt = T) for
  // step 5.
  stage_f4 pf[2048 / NTH];
  fetch_tile128<NTH>(pf, sb + SB_H + 64 * DK, DK, tid);
  __syncthreads();
  // 2. dQg = dO S and dW = -dU S, contracting over v in two halves
  f32x4 dqg[2][2], dw[2][2];
  zero_block(dqg);
  zero_block(dw);
  mfma_block_mix<false, false, 2, 2>(dqg, tB0, tB3, R0, C0, 64, lane);
  mfma_block_mix<false, false, 2, 2>(dw, tB1, tB3, R0, C0, 64, lane);
  __syncthreads();
  // the second half of S stays in registers too, for step 4's column sums
  // (rows (tid >> 5) + 16 i, channels 4 (tid & 31): the put's layout)
  stage_f4 s2[2048 / NTH];
#pragma unroll
  for (int i = 0; i < 2048 / NTH; ++i) s2[i] = pf[i];
  put_ps_tile128<NTH>(tB3, pf, tid);
  fetch_tile128<NTH>(pf, sb + SB_DH + 64 * DK, DK, tid);  // dS' rows 64 .. 127, first in step 4
  __syncthreads();
  mfma_block_mix<false, false, 2, 2>(dqg, tB0v, tB3, R0, C0, 64, lane);
  mfma_block_mix<false, false, 2, 2>(dw, tB1v, tB3, R0, C0, 64, lane);
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) gb[GB_DQG + BLK_ROW(R0, m, r) * DK + BLK_COL(C0, n)] = dqg[m][n][r];
  // 3. dAqk = dO U^T, lower triangle including the diagonal
  {
    f32x4 a[2][1];
    zero_block(a);
    mfma_block_mix<false, true, 2, 1>(a, tB0, fB2, R0, Q0, DV, lane);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = BLK_ROW(R0, m, r), j = BLK_COL(Q0, 0);
        gb[GB_DAQK + i * 64 + j] = j <= i ? a[m][0][r] : 0.0f;
      }
  }
  __syncthreads();
  // 4. dKd = U dS', contracting over v in two halves; dgn = colsum(dS' . S).
  //    B0 is free since step 3, so dS' goes to B0, second half first.  The
  //    column sums take dS' from the registers it is put from (B0 holds it
  //    split): thread (rows rb + 16 i, channels c4) pairs each half with
  //    the half of S it kept in registers when S went to LDS.
  stage_u4 pv[1024 / NTH];
  stage_f4 pt[1024 / NTH];
  {
    const int rb = tid >> 5, c4 = 4 * (tid & 31);
    f32x4 dkd[2][2];
    zero_block(dkd);
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += pf[i] * s2[i];
    put_ps_tile128<NTH>(tB0, pf, tid);  // dS' rows 64 .. 127
    fetch_tile128<NTH>(pf, sb + SB_DH, DK, tid);
    __syncthreads();
    mfma_block_mix<false, false, 2, 2>(dkd, fB2v, tB0, R0, C0, 64, lane);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += pf[i] * s1[i];
    put_ps_tile128<NTH>(tB0, pf, tid);  // dS' rows 0 .. 63
    fetch_tile128<NTH>(pf, pb + PB_KG, DK, tid);
    fetch_bf16_tile128<NTH>(pv, v + ((size_t)L.row0 * Hv + h) * DV, (size_t)Hv * DV, L.len, tid);
    fetch_tile64<NTH>(pt, pb + PB_T, tid);
    __syncthreads();
    mfma_block_mix<false, false, 2, 2>(dkd, fB2, tB0, R0, C0, 64, lane);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) gb[GB_DKD + BLK_ROW(R0, m, r) * DK + BLK_COL(C0, n)] = dkd[m][n][r];
    // the 16 row groups meet in sT, free until step 5
    *reinterpret_cast<f32x4*>(sT + rb * DK + c4) = acc;
  }
  __syncthreads();
  if (tid < DK) {
    float sum = 0.0f;
#pragma unroll
    for (int g8 = 0; g8 < 16; ++g8) sum += sT[g8 * DK + tid];
    gb[GB_DGN + tid] = sum;
  }
  __syncthreads();  // B0, B2, B3 and sT are refilled below
  // 5. B3 <- dW, B0 <- Kg, B2 <- V, sT <- T, sB <- beta
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) ps_put1(tB3, BLK_ROW(R0, m, r), BLK_COL(C0, n), -dw[m][n][r]);
  put_ps_tile128<NTH>(tB0, pf, tid);
  put_bf16_tile128<NTH>(B2, pv, tid);
  put_tile64<NTH>(sT, pt, tid);
  if (tid < CH) {
    const __amdgpu_buffer_rsrc_t bb = buffer_rsrc(beta + (size_t)L.row0 * Hv + h, (uint32_t)L.len * Hv * 2);
    const float braw = bf2f((uint16_t)__builtin_amdgcn_raw_buffer_load_b16(bb, (uint32_t)(tid * Hv) * 2, 0, 0));
    const float bp = (flags & KDA_FLAG_BETA_IS_PROB) ? braw : sigm(braw);
    sB[tid] = tid < L.len ? bp : 0.0f;
  }
  __syncthreads();
  // 6. dM = dU V^T + dW Kg^T;  dV = M^T dU;  dKg = M^T dW  (M = T diag(b))
  f32x4 dm[2][1];
  zero_block(dm);
  mfma_block_mix<false, true, 2, 1>(dm, tB1, fB2, R0, Q0, DV, lane);
  mfma_block_mix<false, true, 2, 1>(dm, tB3, tB0, R0, Q0, DK, lane);
  {
    f32x4 a[2][2];
    zero_block(a);
    mfma_block_mix<true, false, 2, 2>(a, fT, tB1, R0, C0, CH, lane);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = BLK_ROW(R0, m, r);
        if (t < L.len) {
          float* d = dv + ((size_t)(L.row0 + t) * Hv + h) * DV;
#pragma unroll
          for (int n = 0; n < 2; ++n) d[BLK_COL(C0, n)] = sB[t] * a[m][n][r];
        }
      }
    zero_block(a);
    mfma_block_mix<true, false, 2, 2>(a, fT, tB3, R0, C0, CH, lane);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = BLK_ROW(R0, m, r);
          gb[GB_DKG + t * DK + BLK_COL(C0, n)] = sB[t] * a[m][n][r];
        }
  }
  __syncthreads();
  // 7. db_j = sum_i dM[i][j] T[i][j];  dT = dM diag(b);  dAkk = -(T^T dT T^T) strictly lower
  float* sDM = reinterpret_cast<float*>(B0h);  // [64][QS] (B0's hi tile is dead: same 17,408 bytes)
  static_assert(CH * QS * sizeof(float) <= CH * PS_ROW_LD * sizeof(__bf16), "sDM fits B0's hi tile");
  float* sDT = B2;  // [64][QS]
  float* sX = reinterpret_cast<float*>(B3h);  // [64][QS] (B3's hi tile, dead by now)
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = BLK_ROW(R0, m, r), j = BLK_COL(Q0, 0);
      sDM[i * QS + j] = dm[m][0][r];
      sDT[i * QS + j] = dm[m][0][r] * sB[j];
    }
  __syncthreads();
  if (tid < CH) {
    float acc = 0.0f;
    for (int i = 0; i < CH; ++i) acc += sDM[i * QS + tid] * sT[i * QS + tid];
    gb[GB_DB + tid] = acc;
  }
  {
    f32x4 a[2][1];
    zero_block(a);
    mfma_block<true, false, 2, 1>(a, sT, QS, sDT, QS, R0, Q0, CH, lane);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) sX[BLK_ROW(R0, m, r) * QS + BLK_COL(Q0, 0)] = a[m][0][r];
    __syncthreads();
    zero_block(a);
    mfma_block<false, true, 2, 1>(a, sX, QS, sT, QS, R0, Q0, CH, lane);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = BLK_ROW(R0, m, r), j = BLK_COL(Q0, 0);
        gb[GB_DAKK + i * 64 + j] = j < i ? -a[m][0][r] : 0.0f;
      }
  }
}

// ---------------------------------------------------------------------------
// pairwise terms, elementwise factors, decay sum, gate, norms and beta.
// Wave (w, half) owns row block w (rows 16 w .. +15) and half of the channels
// in MFMA accumulator layout: element (row 16 w + 4 lg + r, channel 16 (nb +
// n) + li) in acc[n][r], nb = 4 half.  With
// a = dAkk, b = dAqk (masked), E_ij = e^(G_i - G_j) per channel:
//   R1_i = sum_j a_ij K_j E_ij,   R2_i = sum_j b_ij K_j E_ij      (row side)
//   C_j  = sum_i (beta_i a_ij K_i + b_ij scale Q_i) E_ij           (column side)
//   dK = beta R1 + C,  d(scale Q) = R2,  dG = beta K R1 + scale Q R2 - K C,
//   dbeta_i (from Akk) = sum_c K_ic R1_ic.
// Pairs in different 16-row blocks I > J factor through p = 16 I - 1, the
// row before block I: E_ij = e^(G_i - G_p) e^(G_p - G_j), both exponents <= 0,
// so those sums are fp32 MFMA products with one factor on each operand.
// Pairs inside a block use the block's row 8 as the reference when the decay
// is bounded (safe gate), and are summed directly otherwise.

template <int MODE>
__global__ void __launch_bounds__(PAIR_THREADS)
kda_bwd_pair_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ g,
                    const uint16_t* __restrict__ beta, const float* __restrict__ A_log,
                    const float* __restrict__ dt_bias, const int64_t* __restrict__ cu,
                    const int* __restrict__ chunk_off, int T, int N, int Hqk, int Hv, int mc, float scale, float lb,
                    int flags, float* __restrict__ dq, float* __restrict__ dk, int qk_heads_out,
                    float* __restrict__ dg, float* __restrict__ dbeta, float* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) float sK[CH * RS];
  __shared__ __attribute__((aligned(16))) float sQ[CH * RS];
  __shared__ __attribute__((aligned(16))) float sG[CH * RS];
  __shared__ __attribute__((aligned(16))) float sDA[CH * QS];  // dAkk
  __shared__ __attribute__((aligned(16))) float sDQ[CH * QS];  // dAqk
  __shared__ float sB[CH];
  __shared__ float sRq[CH], sRk[CH];
  __shared__ float sCol[16 * DK];
  __shared__ float sRed[8];
  __shared__ float sRow[3][2][CH];  // per-row partial sums of the two channel halves
  __shared__ __attribute__((aligned(16))) float sBt[4 * DK];
  const int x = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const ChunkLoc L = chunk_loc(x, cu, chunk_off, T, N);
  float* pb = ws + ((size_t)h * mc + x) * CHUNK_HEAD_FLOATS;
  float* gb = pb + PB_FLOATS + SB_FLOATS;
  float* gp = gb + GB_FLOATS;
  if (L.len == 0) {  // past the last chunk: zero gate partials
    if (tid < GP_FLOATS) gp[tid] = 0.0f;
    return;
  }
  const int hq = h / (Hv / Hqk);
  // dAkk and dAqk first: their loads overlap the chunk inputs' (the loader's
  // barriers order the LDS writes before any read)
  load_tile64<PAIR_THREADS>(sDA, gb + GB_DAKK, tid);
  load_tile64<PAIR_THREADS>(sDQ, gb + GB_DAQK, tid);
  float rq, rk;
  load_chunk_inputs<MODE, PAIR_THREADS>(sK, sQ, sG, sBt, sB, q, k, g, beta, A_log, dt_bias, Hqk, Hv, h, hq, L.row0,
                                        L.len, lb, flags, tid, &rq, &rk);
  constexpr int TPR = PAIR_THREADS / CH;
  if (tid % TPR == 0) { sRq[tid / TPR] = rq; sRk[tid / TPR] = rk; }
  __syncthreads();

  // wave (w, half): row block w = wave & 3, channel columns 16 (nb + n) + li,
  // n < 4, nb = 4 (wave >> 2)
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), w = wave & 3, half = wave >> 2, nb = 4 * half;
  const int li = lane & 15, lg = lane >> 4;
  const int rbase = 16 * w + 4 * lg;  // own rows rbase + r
  // the raw gate inputs of the gate phase, loaded now so their latency hides
  // behind the pairwise sums (bf16 bits; zero past the chunk's end)
  // (range-checked buffer loads: a conditional load was compiled into a
  // branch that waited for each load in turn)
  uint16_t graw[4][4];
  // db from dM . T of the own rows (dense kernel), for the dbeta stores at the end
  float dbw[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) dbw[r] = gb[GB_DB + rbase + r];
  {
    const __amdgpu_buffer_rsrc_t bg = buffer_rsrc(g + ((size_t)L.row0 * Hv + h) * DK, (uint32_t)L.len * Hv * DK * 2);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int n = 0; n < 4; ++n)
        graw[n][r] = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(
            bg, (uint32_t)((rbase + r) * Hv * DK + 16 * (nb + n) + li) * 2, 0, 0);
  }
  float Ko[4][4], Qo[4][4], Go[4][4];
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = (rbase + r) * RS + 16 * (nb + n) + li;
      Ko[n][r] = sK[e];
      Qo[n][r] = sQ[e];
      Go[n][r] = sG[e];
    }

  // ---- row side: R1, R2 for own rows
  f32x4 R1[4], R2[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) { R1[n] = f32x4{0.f, 0.f, 0.f, 0.f}; R2[n] = R1[n]; }
  if (w > 0) {
    // p = 16 w - 1: G_i - G_p = sG_i;  G_p - G_j = Bt_J - sG_j + sum_{J<B<w} Bt_B
    for (int J = 0; J < w; ++J) {
      float mid[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        float o = sBt[J * DK + 16 * (nb + n) + li];
        for (int B = J + 1; B < w; ++B) o += sBt[B * DK + 16 * (nb + n) + li];
        mid[n] = o;
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int j = 16 * J + 4 * kk + lg;
        const float a = sDA[(16 * w + li) * QS + j], b = sDQ[(16 * w + li) * QS + j];
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const int c = 16 * (nb + n) + li;
          const float z = sK[j * RS + c] * ex2(mid[n] - sG[j * RS + c]);
          R1[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, z, R1[n], 0, 0, 0);
          R2[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(b, z, R2[n], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float f = ex2(Go[n][r]);
        R1[n][r] *= f;
        R2[n][r] *= f;
      }
  }
  // the midpoint decay of the own block, per channel (safe gate only)
  float Gm[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) Gm[n] = sG[(16 * w + 8) * RS + 16 * (nb + n) + li];
  if constexpr (MODE == KDA_GATE_SAFE_SIGMOID) {
    // Diagonal block, bounded decay: e^(G_i - G_j) = e^(sG_i - sG_m) e^(sG_m - sG_j)
    // with m the block's row 8, each factor within 2^(8 |lb| log2 e) of one.
    // The masked dAkk / dAqk blocks (zero above the diagonal) make it one
    // fp32 MFMA product per term.
    f32x4 D1[4], D2[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) { D1[n] = f32x4{0.f, 0.f, 0.f, 0.f}; D2[n] = D1[n]; }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int j = 16 * w + 4 * kk + lg;
      const float a = sDA[(16 * w + li) * QS + j], b = sDQ[(16 * w + li) * QS + j];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int c = 16 * (nb + n) + li;
        const float z = sK[j * RS + c] * ex2(Gm[n] - sG[j * RS + c]);
        D1[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, z, D1[n], 0, 0, 0);
        D2[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(b, z, D2[n], 0, 0, 0);
      }
    }
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float f = ex2(Go[n][r] - Gm[n]);
        R1[n][r] += f * D1[n][r];
        R2[n][r] += f * D2[n][r];
      }
  } else {
    // unbounded decay: pair by pair, every exponent <= 0
    for (int jj = 0; jj < 16; ++jj) {
      const int j = 16 * w + jj;
      float a[4], b[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) { a[r] = sDA[(rbase + r) * QS + j]; b[r] = sDQ[(rbase + r) * QS + j]; }
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int c = 16 * (nb + n) + li;
        const float kj = sK[j * RS + c], gj = sG[j * RS + c];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = kj * ex2(fminf(Go[n][r] - gj, 0.0f));
          R1[n][r] += a[r] * e;
          R2[n][r] += b[r] * e;
        }
      }
    }
  }

  // ---- column side: C for own rows (as j)
  f32x4 Cc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) Cc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int I = w + 1; I < 4; ++I) {
    f32x4 X[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) X[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int i = 16 * I + 4 * kk + lg;
      const float a = sB[i] * sDA[i * QS + 16 * w + li], b = sDQ[i * QS + 16 * w + li];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int c = 16 * (nb + n) + li;
        const float f = ex2(sG[i * RS + c]);
        X[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sK[i * RS + c] * f, X[n], 0, 0, 0);
        X[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(b, scale * sQ[i * RS + c] * f, X[n], 0, 0, 0);
      }
    }
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      float mid = sBt[w * DK + 16 * (nb + n) + li];
      for (int B = w + 1; B < I; ++B) mid += sBt[B * DK + 16 * (nb + n) + li];
#pragma unroll
      for (int r = 0; r < 4; ++r) Cc[n][r] += X[n][r] * ex2(mid - Go[n][r]);
    }
  }
  // the workspace gradients of the elementwise factors, issued here so their
  // latency hides behind the column-side products
  float eq[4][4], egk[4][4], ed4[4][4];
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int o = (rbase + r) * DK + 16 * (nb + n) + li;
      eq[n][r] = gb[GB_DQG + o];
      egk[n][r] = gb[GB_DKG + o];
      ed4[n][r] = gb[GB_DKD + o];
    }
  if constexpr (MODE == KDA_GATE_SAFE_SIGMOID) {
    // diagonal block through the midpoint, as on the row side
    f32x4 X[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) X[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int i = 16 * w + 4 * kk + lg;
      const float a = sB[i] * sDA[i * QS + 16 * w + li], b = sDQ[i * QS + 16 * w + li];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int c = 16 * (nb + n) + li;
        const float f = ex2(sG[i * RS + c] - Gm[n]);
        X[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sK[i * RS + c] * f, X[n], 0, 0, 0);
        X[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(b, scale * sQ[i * RS + c] * f, X[n], 0, 0, 0);
      }
    }
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) Cc[n][r] += X[n][r] * ex2(Gm[n] - Go[n][r]);
  } else {
    for (int ii = 0; ii < 16; ++ii) {
      const int i = 16 * w + ii;
      const float bi = sB[i];
      float a[4], b[4];
  #pragma unroll
      for (int r = 0; r < 4; ++r) { a[r] = bi * sDA[i * QS + rbase + r]; b[r] = sDQ[i * QS + rbase + r]; }
  #pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int c = 16 * (nb + n) + li;
        const float ki = sK[i * RS + c], qi = scale * sQ[i * RS + c], gi = sG[i * RS + c];
  #pragma unroll
        for (int r = 0; r < 4; ++r) Cc[n][r] += (a[r] * ki + b[r] * qi) * ex2(fminf(gi - Go[n][r], 0.0f));
      }
    }
  }

  // ---- combine: dK, dQ (w.r.t. scale q_hat), dG; dbeta from Akk
  float dK[4][4], dQ[4][4], dG[4][4], dbk[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) dbk[r] = 0.0f;
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float bo = sB[rbase + r];
      dK[n][r] = bo * R1[n][r] + Cc[n][r];
      dQ[n][r] = R2[n][r];
      dG[n][r] = bo * Ko[n][r] * R1[n][r] + scale * Qo[n][r] * R2[n][r] - Ko[n][r] * Cc[n][r];
      dbk[r] += Ko[n][r] * R1[n][r];
    }

  // ---- elementwise factors: Qg = scale Q e^G, Kg = K e^G, Kd = K e^(G_last - G), gn = e^G_last
  // The own rows all lie in block w, so the block totals before it (Pa) and
  // from it on (Pt) are per channel: G_abs = Go + Pa, G_last - G_abs = Pt - Go.
  float colKd[4], Pa[4], Pt[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int c = 16 * (nb + n) + li;
    float a = 0.0f, t = 0.0f;
    for (int B = 0; B < 4; ++B) {
      const float bt = sBt[B * DK + c];
      if (B < w) a += bt; else t += bt;
    }
    Pa[n] = a;
    Pt[n] = t;
    colKd[n] = 0.0f;
  }
#pragma unroll
  for (int n = 0; n < 4; ++n) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float vq = eq[n][r], vg = egk[n][r], vd = ed4[n][r];
      const float eg = ex2(Go[n][r] + Pa[n]), ed = ex2(Pt[n] - Go[n][r]);
      dQ[n][r] += vq * eg;
      dK[n][r] += vg * eg + vd * ed;
      const float kd = vd * Ko[n][r] * ed;
      dG[n][r] += (vq * scale * Qo[n][r] + vg * Ko[n][r]) * eg - kd;
      colKd[n] += kd;
    }
  }
  // dG of the chunk's last row gains sum_t dKd . Kd and dgn . gn
#pragma unroll
  for (int n = 0; n < 4; ++n) sCol[(4 * w + lg) * DK + 16 * (nb + n) + li] = colKd[n];
  __syncthreads();  // also: every read of sQ above is done
  // dG -> sQ, then the reverse cumulative sum over rows gives d a per token
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) sQ[(rbase + r) * RS + 16 * (nb + n) + li] = dG[n][r];
  __syncthreads();
  if (tid < DK) {
    float sum = gb[GB_DGN + tid] * ex2(gabs(sG, sBt, 63, tid));
    for (int rg = 0; rg < 16; ++rg) sum += sCol[rg * DK + tid];
    sQ[63 * RS + tid] += sum;
  }
  __syncthreads();
  {
    // thread (c, qr): suffix sums over rows 16 qr .. 16 qr + 15, then the
    // totals of the later row quarters are added
    const int c = tid & 127, qr = tid >> 7;
    float x[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) x[rr] = sQ[(16 * qr + rr) * RS + c];
#pragma unroll
    for (int rr = 14; rr >= 0; --rr) x[rr] += x[rr + 1];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) sQ[(16 * qr + rr) * RS + c] = x[rr];
    __syncthreads();
    float base = 0.0f;
    for (int q2 = 3; q2 > qr; --q2) base += sQ[(16 * q2) * RS + c];
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) sQ[(16 * qr + rr) * RS + c] = x[rr] + base;
  }
  __syncthreads();

  // ---- gate: a = f(x), x = g + dt_bias;  norms;  beta
  const float A_exp = (MODE == KDA_GATE_PREGATED || A_log == nullptr) ? 1.0f : __expf(A_log[h]);
  const bool norm = flags & KDA_FLAG_QK_L2NORM;
  float colDt[4], dA = 0.0f;
#pragma unroll
  for (int n = 0; n < 4; ++n) colDt[n] = 0.0f;
  float dtb[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) dtb[n] = dt_bias ? dt_bias[(size_t)h * DK + 16 * (nb + n) + li] : 0.0f;
  float dgo[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = rbase + r;
    const bool ok = row < L.len;  // uniform over the 16 lanes of the row
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int c = 16 * (nb + n) + li;
      const float da = sQ[row * RS + c];
      const float gv = bf2f(graw[n][r]);
      float a, dadx, dadA;
      gate_fwd_bwd<MODE>(gv + dtb[n], A_exp, lb, a, dadx, dadA);
      // below the decay floor the factor e^a is exactly zero in fp32
      if (a * kLog2e < kMinLog2Decay) dadx = dadA = 0.0f;
      dgo[n][r] = ok ? da * dadx : 0.0f;
      colDt[n] += dgo[n][r];
      if (ok) dA += da * dadA;
    }
    // this half's share of the row sums y . dy (q and k) and of dbeta
    float yq = 0.0f, yk = 0.0f;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      yq += Qo[n][r] * (scale * dQ[n][r]);
      yk += Ko[n][r] * dK[n][r];
    }
    yq = sum16(yq);
    yk = sum16(yk);
    const float dbs = sum16(dbk[r]);
    if (li == 0) { sRow[0][half][row] = yq; sRow[1][half][row] = yk; sRow[2][half][row] = dbs; }
  }
  __syncthreads();
  // dq, dk and dg go through LDS (sK, sQ and sG are free now), so that every
  // thread stores whole 64-byte row segments instead of 48 scattered floats
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = rbase + r;
    // y = q/|q| (the operand is scale y): dq = r (dy - y (y . dy)), dy = scale dQ
    const float yq = norm ? sRow[0][0][row] + sRow[0][1][row] : 0.0f;
    const float yk = norm ? sRow[1][0][row] + sRow[1][1][row] : 0.0f;
    const float rqi = sRq[row], rki = sRk[row];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int e = row * RS + 16 * (nb + n) + li;
      sK[e] = rqi * (scale * dQ[n][r] - Qo[n][r] * yq);
      sQ[e] = rki * (dK[n][r] - Ko[n][r] * yk);
      sG[e] = dgo[n][r];
    }
    if (li == 0 && half == 0 && row < L.len) {
      const float db = dbw[r] + (sRow[2][0][row] + sRow[2][1][row]);
      const float b = sB[row];
      dbeta[(size_t)(L.row0 + row) * Hv + h] = (flags & KDA_FLAG_BETA_IS_PROB) ? db : db * b * (1.0f - b);
    }
  }
  // per-chunk partials of ddt_bias (column sums) and dA_log
#pragma unroll
  for (int n = 0; n < 4; ++n) sCol[(4 * w + lg) * DK + 16 * (nb + n) + li] = colDt[n];
  dA = sum16(dA);
  dA += __shfl_xor(dA, 16); dA += __shfl_xor(dA, 32);
  if (lane == 0) sRed[wave] = dA;
  __syncthreads();
  {
    // thread t: channels 4 (t & 31) .. +3 of rows (t >> 5) + 16 i, so the 32
    // lanes of a row store its 512 bytes in order
    const int c4 = 4 * (tid & 31);
    const int hh = qk_heads_out == Hqk ? hq : h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (tid >> 5) + 16 * i;
      if (row < L.len) {
        const size_t trow = (size_t)(L.row0 + row);
        *reinterpret_cast<f32x4*>(dq + (trow * qk_heads_out + hh) * DK + c4) =
            *reinterpret_cast<const f32x4*>(sK + row * RS + c4);
        *reinterpret_cast<f32x4*>(dk + (trow * qk_heads_out + hh) * DK + c4) =
            *reinterpret_cast<const f32x4*>(sQ + row * RS + c4);
        *reinterpret_cast<f32x4*>(dg + (trow * Hv + h) * DK + c4) = *reinterpret_cast<const f32x4*>(sG + row * RS + c4);
      }
    }
  }
  if (tid < DK) {
    float sum = 0.0f;
    for (int rg = 0; rg < 16; ++rg) sum += sCol[rg * DK + tid];
    gp[tid] = sum;
  }
  if (tid == 0) gp[DK] = ((sRed[0] + sRed[1]) + (sRed[2] + sRed[3])) + ((sRed[4] + sRed[5]) + (sRed[6] + sRed[7]));
}

// q/k gradients summed over the v-heads sharing a q/k head; gate-parameter
// partials summed over chunks.
// one float4 of (row, q/k head hq): the sum over its G v-heads
__device__ __forceinline__ void reduce_qk_one(const float* __restrict__ dqv, const float* __restrict__ dkv,
                                              float* __restrict__ dq, float* __restrict__ dk, int64_t e, int Hqk,
                                              int G) {
  const int c4 = (int)(e % (DK / 4));
  const int64_t rh = e / (DK / 4);
  const int hq = (int)(rh % Hqk);
  const int64_t row = rh / Hqk;
  float4 sq = make_float4(0.f, 0.f, 0.f, 0.f), sk = sq;
  for (int j = 0; j < G; ++j) {
    const size_t o = ((size_t)row * Hqk * G + (size_t)hq * G + j) * DK + 4 * c4;
    const float4 a = *reinterpret_cast<const float4*>(dqv + o), b = *reinterpret_cast<const float4*>(dkv + o);
    sq.x += a.x; sq.y += a.y; sq.z += a.z; sq.w += a.w;
    sk.x += b.x; sk.y += b.y; sk.z += b.z; sk.w += b.w;
  }
  *reinterpret_cast<float4*>(dq + ((size_t)row * Hqk + hq) * DK + 4 * c4) = sq;
  *reinterpret_cast<float4*>(dk + ((size_t)row * Hqk + hq) * DK + 4 * c4) = sk;
}

// grid-stride over the float4s of dq and dk
__global__ void __launch_bounds__(256)
kda_bwd_reduce_qk_kernel(const float* __restrict__ dqv, const float* __restrict__ dkv, float* __restrict__ dq,
                         float* __restrict__ dk, int64_t rows, int Hqk, int G) {
  const int64_t total = rows * Hqk * (DK / 4);
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256)
    reduce_qk_one(dqv, dkv, dq, dk, e, Hqk, G);
}

// Gate-parameter partials of a (chunk, v-head): ddt_bias [128], dA_log [1].
constexpr int GATE_GROUP = 16;  // chunks summed by one workgroup of the first stage
__device__ __forceinline__ float* gate_partials(float* ws, int h, int mc, int x) {
  return ws + ((size_t)h * mc + x) * CHUNK_HEAD_FLOATS + PB_FLOATS + SB_FLOATS + GB_FLOATS;
}

// First stage, per (group of GATE_GROUP chunks, v-head): the group's sum
// replaces the partials of its first chunk.  Two halves of 128 threads take
// alternate chunks, with all their loads in flight at once.
__global__ void __launch_bounds__(256)
kda_bwd_reduce_gate_groups_kernel(float* __restrict__ ws, int mc) {
  __shared__ float sPart[DK + 1];
  const int x0 = GATE_GROUP * blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int c = tid & 127, half = tid >> 7;
  float v[GATE_GROUP / 2], a[GATE_GROUP / 2];
#pragma unroll
  for (int i = 0; i < GATE_GROUP / 2; ++i) {
    const int x = x0 + 2 * i + half;
    v[i] = 0.0f;
    a[i] = 0.0f;
    if (x < mc) {
      const float* gp = gate_partials(ws, h, mc, x);
      v[i] = gp[c];
      if (c == 0) a[i] = gp[DK];
    }
  }
  float sum = 0.0f, sa = 0.0f;
#pragma unroll
  for (int i = 0; i < GATE_GROUP / 2; ++i) {
    sum += v[i];
    sa += a[i];
  }
  if (half == 1) {
    sPart[c] = sum;
    if (c == 0) sPart[DK] = sa;
  }
  __syncthreads();
  if (half == 0) {
    // only this thread read these two entries of chunk x0
    float* gp = gate_partials(ws, h, mc, x0);
    gp[c] = sum + sPart[c];
    if (c == 0) gp[DK] = sa + sPart[DK];
  }
}

// Second stage, per v-head: the sums of the groups (at chunks 0, GATE_GROUP, ...).
__global__ void __launch_bounds__(256)
kda_bwd_reduce_gate_kernel(float* __restrict__ ws, int mc, float* __restrict__ dA_log,
                           float* __restrict__ ddt_bias) {
  __shared__ float sPart[2][DK + 1];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int c = tid & 127, half = tid >> 7;
  constexpr int U = 8;  // loads in flight per thread
  float sum = 0.0f, sa = 0.0f;
  for (int x = GATE_GROUP * half; x < mc; x += 2 * GATE_GROUP * U) {
    float v[U], a[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int xi = x + 2 * GATE_GROUP * i;
      v[i] = 0.0f;
      a[i] = 0.0f;
      if (xi < mc) {
        const float* gp = gate_partials(ws, h, mc, xi);
        v[i] = gp[c];
        if (c == 0) a[i] = gp[DK];
      }
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
      sum += v[i];
      sa += a[i];
    }
  }
  sPart[half][c] = sum;
  if (c == 0) sPart[half][DK] = sa;
  __syncthreads();
  if (tid < DK && ddt_bias) ddt_bias[(size_t)h * DK + tid] = sPart[0][tid] + sPart[1][tid];
  if (tid == 0 && dA_log) dA_log[h] = sPart[0][DK] + sPart[1][DK];
}

}  // namespace

// ---------------------------------------------------------------------------
// host side
namespace {

// header | per-chunk blocks | q/k gradients per v-head (grouped heads only) |
// segment scratch (nseg > 1)
size_t gqa_floats(const kda_fwd_params* p) {
  return p->H_v != p->H_qk ? 2 * (size_t)p->B * (size_t)p->T * p->H_v * DK : 0;
}
size_t bwd_bytes(const kda_fwd_params* p, int64_t mc, int nseg) {
  return header_bytes(p) + ((size_t)p->H_v * (size_t)mc * CHUNK_HEAD_FLOATS + gqa_floats(p)) * sizeof(float) +
         seg_scratch_bytes(p, nseg);
}

template <int MODE>
void launch_bwd(const kda_fwd_params* p, const void* q, const void* k, const void* v, const void* g, const void* beta,
                const float* A_log, const float* dt_bias, const int64_t* cu, const void* h0, const void* d_out,
                const float* dhT, float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dA_log,
                float* ddt_bias, float* dh0, void* workspace, hipStream_t st) {
  const bool packed = cu != nullptr;
  const int64_t mc = max_chunks_of(p, packed);
  uint8_t* wsb = reinterpret_cast<uint8_t*>(workspace);
  int* chunk_off = reinterpret_cast<int*>(wsb);
  float* ws = reinterpret_cast<float*>(wsb + header_bytes(p));
  const int G = p->H_v / p->H_qk;
  float* dqv = dq;
  float* dkv = dk;
  if (G > 1) {
    dqv = ws + (size_t)p->H_v * mc * CHUNK_HEAD_FLOATS;
    dkv = dqv + (size_t)p->B * p->T * p->H_v * DK;
  }
  const int chains = p->num_seqs * p->H_v;
  const uint16_t* qq = (const uint16_t*)q;
  const uint16_t* kk = (const uint16_t*)k;
  const uint16_t* vv = (const uint16_t*)v;
  const uint16_t* gg = (const uint16_t*)g;
  const uint16_t* bb = (const uint16_t*)beta;
  const uint16_t* dd = (const uint16_t*)d_out;
  if (packed) launch_chunk_map(cu, p->num_seqs, chunk_off, st);
  const dim3 cg((unsigned)mc, (unsigned)p->H_v);
  // the prep kernel is persistent: one workgroup per CU (its LDS allows no
  // more), each looping over chunk-heads
  const dim3 pg((unsigned)std::min<int64_t>(mc * p->H_v, kBwdCUs));
  if (mc > 0)
    hipLaunchKernelGGL(kda_bwd_prep_kernel<MODE>, pg, dim3(PREP_THREADS), 0, st, qq, kk, vv, gg, bb, A_log, dt_bias, cu,
                       chunk_off, p->T, p->num_seqs, p->H_qk, p->H_v, (int)mc, p->scale, p->lower_bound, p->flags, ws);
  if (chains > 0) {
    float* seg = ws + (size_t)p->H_v * mc * CHUNK_HEAD_FLOATS + gqa_floats(p);
    int seg_len;
    const int nseg = seg_plan(p, packed, &seg_len);
    // grid of a launch with `jobs` jobs: groups of 8 jobs, BNS slices each
    auto grid = [](int64_t jobs) { return dim3((unsigned)(((jobs + 7) / 8) * 8 * BNS)); };
    const dim3 cmb((unsigned)(chains * (SD / CMB_ROWS)));
    const int N = p->num_seqs, H = p->H_v, T = p->T, idt = p->init_state_dtype;
    if (nseg > 1) {
      hipLaunchKernelGGL(kda_bwd_fstate_kernel<ST_CARRY>, grid((int64_t)chains * (nseg - 1)), dim3(STATE_THREADS), 0, st, cu,
                         chunk_off, h0, idt, T, N, H, (int)mc, ws, seg, nseg, seg_len);
      if (nseg > 2) {
        hipLaunchKernelGGL(kda_bwd_fstate_kernel<ST_TRANS>, grid((int64_t)chains * (nseg - 2)), dim3(STATE_THREADS), 0, st, cu,
                           chunk_off, h0, idt, T, N, H, (int)mc, ws, seg, nseg, seg_len);
        hipLaunchKernelGGL(kda_segment_combine_kernel, cmb, dim3(256), 0, st, seg, chains, nseg);
      }
    }
    hipLaunchKernelGGL(kda_bwd_fstate_kernel<ST_FULL>, grid((int64_t)chains * nseg), dim3(STATE_THREADS), 0, st, cu, chunk_off,
                       h0, idt, T, N, H, (int)mc, ws, seg, nseg, seg_len);
    // the backward pass reuses the scratch once the forward pass is done with it
    if (nseg > 1) {
      hipLaunchKernelGGL(kda_bwd_bstate_kernel<ST_CARRY>, grid((int64_t)chains * (nseg - 1)), dim3(STATE_THREADS), 0, st, dd,
                         dhT, dh0, cu, chunk_off, T, N, H, (int)mc, ws, seg, nseg, seg_len);
      if (nseg > 2) {
        hipLaunchKernelGGL(kda_bwd_bstate_kernel<ST_TRANS>, grid((int64_t)chains * (nseg - 2)), dim3(STATE_THREADS), 0, st, dd,
                           dhT, dh0, cu, chunk_off, T, N, H, (int)mc, ws, seg, nseg, seg_len);
        hipLaunchKernelGGL(kda_segment_combine_kernel, cmb, dim3(256), 0, st, seg, chains, nseg);
      }
    }
    hipLaunchKernelGGL(kda_bwd_bstate_kernel<ST_FULL>, grid((int64_t)chains * nseg), dim3(STATE_THREADS), 0, st, dd, dhT, dh0,
                       cu, chunk_off, T, N, H, (int)mc, ws, seg, nseg, seg_len);
  }
  if (mc > 0) {
    hipLaunchKernelGGL(kda_bwd_dense_kernel, cg, dim3(DENSE_THREADS), 0, st, vv, dd, bb, cu, chunk_off, p->T, p->num_seqs,
                       p->H_v, (int)mc, p->flags, dv, ws);
    hipLaunchKernelGGL(kda_bwd_pair_kernel<MODE>, cg, dim3(PAIR_THREADS), 0, st, qq, kk, gg, bb, A_log, dt_bias, cu, chunk_off,
                       p->T, p->num_seqs, p->H_qk, p->H_v, (int)mc, p->scale, p->lower_bound, p->flags, dqv, dkv,
                       G > 1 ? p->H_v : p->H_qk, dg, dbeta, ws);
    if (G > 1) {
      const int64_t rows = (int64_t)p->B * p->T;
      const int64_t n4 = rows * p->H_qk * (DK / 4);
      hipLaunchKernelGGL(kda_bwd_reduce_qk_kernel, dim3((unsigned)std::min<int64_t>((n4 + 255) / 256, 1 << 20)),
                         dim3(256), 0, st, dqv, dkv, dq, dk, rows, p->H_qk, G);
    }
  }
  if (dA_log || ddt_bias) {
    if (mc > 0)
      hipLaunchKernelGGL(kda_bwd_reduce_gate_groups_kernel,
                         dim3((unsigned)((mc + GATE_GROUP - 1) / GATE_GROUP), (unsigned)p->H_v), dim3(256), 0, st, ws,
                         (int)mc);
    hipLaunchKernelGGL(kda_bwd_reduce_gate_kernel, dim3((unsigned)p->H_v), dim3(256), 0, st, ws, (int)mc, dA_log,
                       ddt_bias);
  }
}

}  // namespace

extern "C" {

size_t kda_bwd_workspace_size(const kda_fwd_params* p) {
  if (!p) return 0;
  // packed or dense cannot be told from params alone; size for the larger
  // chunk count (packed when it can be) and the larger segment count (dense)
  const bool packed = p->B == 1 && p->num_seqs >= 1;
  const bool dense_ok = check_params(p, false) == KDA_OK;
  if (!dense_ok && check_params(p, true) != KDA_OK) return 0;
  int len, nseg = 1;
  if (dense_ok) nseg = seg_plan(p, false, &len);
  return bwd_bytes(p, max_chunks_of(p, packed), nseg);
}

kda_status kda_bwd(const kda_fwd_params* p, const void* q, const void* k, const void* v, const void* g,
                   const void* beta, const float* A_log, const float* dt_bias, const int64_t* cu_seqlens,
                   const void* initial_state, const void* d_out, const float* d_final_state, float* dq, float* dk,
                   float* dv, float* dg, float* dbeta, float* dA_log, float* ddt_bias, float* d_initial_state,
                   void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  const bool packed = cu_seqlens != nullptr;
  kda_status s = check_params(p, packed);
  if (s != KDA_OK) return s;
  if (p->gate_mode == KDA_GATE_PREGATED && (dt_bias || ddt_bias || dA_log))
    return fail(KDA_ERR_UNSUPPORTED, "dt_bias, ddt_bias and dA_log must be NULL with pre-gated decay");
  if (p->gate_mode == KDA_GATE_SOFTPLUS && !A_log)
    return fail(KDA_ERR_NULL, "A_log is NULL (required by the softplus gate)");
  if (dA_log && !A_log) return fail(KDA_ERR_UNSUPPORTED, "dA_log needs A_log");
  if ((int64_t)p->B * p->T > 0) {
    const void* req[] = {q, k, v, g, beta, d_out, dq, dk, dv, dg, dbeta};
    const char* names[] = {"q", "k", "v", "g", "beta", "d_out", "dq", "dk", "dv", "dg", "dbeta"};
    for (int i = 0; i < 11; ++i)
      if (!req[i]) return fail(KDA_ERR_NULL, "%s is NULL", names[i]);
    const void* al[] = {q, k, v, g, d_out, dq, dk, dv, dg};
    const char* aln[] = {"q", "k", "v", "g", "d_out", "dq", "dk", "dv", "dg"};
    for (int i = 0; i < 9; ++i)
      if (!aligned16(al[i])) return fail(KDA_ERR_ALIGN, "%s is not 16-byte aligned", aln[i]);
    if (dt_bias && !aligned16(dt_bias)) return fail(KDA_ERR_ALIGN, "dt_bias is not 16-byte aligned");
    if (ddt_bias && !aligned16(ddt_bias)) return fail(KDA_ERR_ALIGN, "ddt_bias is not 16-byte aligned");
  }
  if (p->init_state_dtype != KDA_STATE_NONE) {
    if (!initial_state) return fail(KDA_ERR_NULL, "initial_state is NULL but init_state_dtype is set");
    if (!aligned16(initial_state)) return fail(KDA_ERR_ALIGN, "initial_state is not 16-byte aligned");
  }
  if (d_final_state && !aligned16(d_final_state)) return fail(KDA_ERR_ALIGN, "d_final_state is not 16-byte aligned");
  if (d_initial_state && !aligned16(d_initial_state))
    return fail(KDA_ERR_ALIGN, "d_initial_state is not 16-byte aligned");
  const size_t need = kda_bwd_workspace_size(p);
  if (!workspace || workspace_bytes < need)
    return fail(KDA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", NULL");
  if (((uintptr_t)workspace & 255u) != 0) return fail(KDA_ERR_ALIGN, "workspace is not 256-byte aligned");

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  auto run = p->gate_mode == KDA_GATE_SAFE_SIGMOID ? launch_bwd<KDA_GATE_SAFE_SIGMOID>
             : p->gate_mode == KDA_GATE_PREGATED   ? launch_bwd<KDA_GATE_PREGATED>
                                                   : launch_bwd<KDA_GATE_SOFTPLUS>;
  run(p, q, k, v, g, beta, A_log, dt_bias, cu_seqlens, initial_state, d_out, d_final_state, dq, dk, dv, dg, dbeta,
      dA_log, ddt_bias, d_initial_state, workspace, st);
  return launch_status();
}

}  // extern "C"
