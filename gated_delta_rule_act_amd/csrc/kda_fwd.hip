// Chunked Kimi Delta Attention forward for MI355X (gfx950, CDNA4).
//
// What is computed (contract in include/kda.h): per sequence and v-head, the
// per-key-channel gated delta rule with state S in R^{V x K}
//     S <- S Diag(e^{a_t});  S <- S + b_t (v_t - S k_t) k_t^T;  o_t = scale S q_t
// with the in-kernel gate activations of the fla-kda SKILL.md ("Gate
// contracts") and the tensor layout of the FlashKDA page ("Tensor shapes and
// dtypes").  It is evaluated in the chunked WY form: 64-token chunks made of
// 16-token sub-chunks, as the fla-kda SKILL.md "Numerical invariants" and
// "Code map" sections describe the intra / inter split.
//
// Two launches (plus a tiny chunk-map launch for packed sequences):
//   kda_intra_kernel  one workgroup per (chunk, v-head), fully parallel.
//       gate activation + chunk-local cumulative log2-decay Gamma;
//       Akk = diag(b) (K Kt . 2^(Gi-Gj)) strictly lower and
//       Aqk = (Q Kt . 2^(Gi-Gj)) lower incl. diagonal, on 16x16 sub-chunk
//       blocks: off-diagonal blocks factor through the last row before the
//       row block (both exponents <= 0); diagonal blocks either through the
//       sub-chunk midpoint (safe gate: exponent span bounded by 8*|lb|) or by
//       binary levels with a reference row per level (unbounded decays);
//       T = (I + Akk)^-1 by 16x16 forward substitution plus fp32-MFMA block
//       merges; WY factors W = T diag(b) (K . 2^G) and T diag(b) for u.
//   kda_state_kernel  one workgroup per (sequence, v-head, 32-wide V slice),
//       sequential over that sequence's chunks with the fp32 state slice in
//       registers:  U = T diag(b) V - W S^T,  O = (Q . 2^G) S^T + Aqk U,
//       S <- S Diag(2^G_last) + U^T (K . 2^(G_last - G)).
//
// Precision: 16-bit MFMA operands with fp32 accumulation.  The contraction
// that writes the state (U^T Kd) uses a 3-product hi/lo split (U and Kd in
// fp16 hi/lo, the low part of Kd kept in e4m3 with a 2^18 scale), T diag(b)
// enters U as bf16 hi/lo against exact bf16 V, the midpoint diagonal blocks
// (factors up to 2^58) take both sides as bf16 hi/lo (three products), and T
// is computed in fp32.  The
// exp2 operands are always differences of Gamma values, never ratios of
// exponentials.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "kda.h"
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_segment.h"

// Device memory of kda_fwd_noalloc: the workspace of its calls, one array per
// GPU, allocated with the code object and held until the process ends.  Host
// code must not use this name as an address: it takes the address the
// runtime reports for the current device (noalloc_scratch below).
static __device__ __align__(256) uint8_t scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {
using namespace kda_internal;
using namespace kda_segment;
using namespace kda_device;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int CH = 64;      // chunk length
constexpr int DK = 128;     // key dim
constexpr int DV = 128;     // value dim
// V slice per state workgroup: 16 NVT columns (NVT = 2 or 4 V tiles)
constexpr int NVT_NARROW = 2, NVT_WIDE = 4;
constexpr int NSLICE = DV / (16 * NVT_NARROW);  // narrow slices per (sequence, head)
constexpr int64_t kGpuCUs = 256;                 // compute units of an MI355X
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kL2Eps = 1e-6f;
// Per-token log2 decay floor.  Any decay below 2^-1e4 is already exactly zero
// in fp32; the floor only keeps Gamma finite so differences never form inf-inf.
constexpr float kMinLog2Decay = -1.0e4f;

// Per (v-head, chunk) workspace block, written by the intra kernel and read by
// the state kernel: 75 fragments of 1 KB.  A fragment is one 16 x 32 tile of
// a 16-bit MFMA operand in lane order -- lane l = (i = l & 15, g = l >> 4)
// holds row i and contraction columns 8g..8g+7 (16 bytes) -- so every
// fragment moves as one contiguous 1 KB load, store or LDS access.
constexpr int FRAG = 1024;
constexpr int F_WN = 0;       // -W             (ta 0..3, kb 0..3) fp16  rows t, columns k
constexpr int F_QG = 16;      // Q . 2^G        (ta, kb)           fp16  raw q
// The token-by-token operands are lower triangular: their token block 1
// (columns 32..63) is zero for token tiles 0 and 1, and those two fragments
// are neither stored nor loaded (tri_frag numbers the other six).
constexpr int F_TBH = 32;     // T diag(b) hi   (ta, kb 0..1)      bf16  rows t, columns s
constexpr int F_TBL = 38;     //           lo
constexpr int F_AQK = 44;     // scale (Q K^T . 2^(G_t - G_s)), lower incl. diagonal (ta, kb 0..1) fp16
constexpr int F_VEC = 50;     // 2^G_last f32[128] (the rest of the fragment is unused)
constexpr int F_KD = 51;      // (K . 2^(G_last - G))^T hi (km 0..7, kb 0..1) fp16 rows k, columns t
constexpr int F_KDL = 67;     // its low part, e4m3 of (Kd - hi) 2^18, 8 B per lane and fragment;
                              // the two token blocks of key tile km share fragment F_KDL + km,
                              // lane l holding kb 0 at 16 l and kb 1 at 16 l + 8 (one 16-byte load)
                              // (fragments 0..50 are shared by all V slices of a chain)
constexpr int NFRAG = 75;
// Q and K here are the normalised q and k (with the L2 norm on, every element
// is at most 1 in size), so no operand depends on the scale of the raw inputs.
// Kd = hi + lo with hi = fp16(Kd) and |lo| <= ulp(hi) / 2 <= 2^-12 for |Kd| <= 1.
// lo is kept as e4m3 of lo 2^18 (3 mantissa bits), within +-64 for |Kd| <= 1
// and clamped to the e4m3 range (+-448) beyond that (only without the L2 norm):
// Kd to about 2^-15 relative, for half the bytes of an fp16 lo.  The scale
// keeps typical lo (|Kd| near 0.01) in the normal e4m3 range; the state kernel
// decodes it exactly to fp16 and scales its product back by 2^-18 in fp32.
constexpr float kKdLoScale = 262144.0f, kKdLoUnscale = 1.0f / 262144.0f, kE4m3Max = 448.0f;
constexpr int NTRI = 6;       // stored fragments of a lower-triangular token-by-token operand
// fragment (ta, kb) of a lower-triangular operand, kb <= ta / 2
__host__ __device__ constexpr int tri_frag(int ta, int kb) { return ta < 2 ? ta : 2 * ta - 2 + kb; }
// and back: the stored fragment f = 0..5 is (tri_ta(f), tri_kb(f))
__host__ __device__ constexpr int tri_ta(int f) { return f < 2 ? f : (f + 2) >> 1; }
__host__ __device__ constexpr int tri_kb(int f) { return f < 2 ? 0 : f & 1; }
static_assert(tri_frag(tri_ta(5), tri_kb(5)) == 5 && tri_frag(tri_ta(2), tri_kb(2)) == 2 &&
              tri_frag(tri_ta(3), tri_kb(3)) == 3 && tri_frag(3, 1) == 5 && tri_frag(1, 0) == 1, "tri_frag");
constexpr size_t BLOCK = (size_t)NFRAG * FRAG;
static_assert(BLOCK % 256 == 0, "workspace block alignment");

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// One 1 KB workspace fragment from a wave (16 bytes per lane).  Non-temporal:
// the workspace is written once and read by the next launch; the state
// kernel measured 5 % faster reading blocks stored this way.
__device__ __forceinline__ void st_frag(uint8_t* blk, int fr, int lane, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(blk + fr * FRAG + lane * 16));
}
// 8 bytes per lane at a 16-byte lane stride (two such halves share a fragment)
__device__ __forceinline__ void st_half_frag(uint8_t* blk, int off, int lane, u32x2 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(blk + off + lane * 16));
}
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef short short2v __attribute__((ext_vector_type(2)));
// eight fp16 -> eight e4m3 bytes (rounded to nearest; the caller has clamped
// the values to the e4m3 range), in the same element order
__device__ __forceinline__ u32x2 pack_e4m3(u32x4 f) {
  u32x2 r;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    // (copied to scalars first: this compiler's __builtin_bit_cast of a vector
    // element reads element 0 whatever the index)
    const uint32_t e0 = f[2 * i], e1 = f[2 * i + 1];
    short2v w = {0, 0};
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(w, __builtin_bit_cast(half2v, e0), 1.0f, false);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(w, __builtin_bit_cast(half2v, e1), 1.0f, true);
    r[i] = __builtin_bit_cast(uint32_t, w);
  }
  return r;
}
// and back: every e4m3 value is exact in fp16
__device__ __forceinline__ half8 unpack_e4m3(u32x2 v) {
  half8 h;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)v[i], 1.0f, false);
    const half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)v[i], 1.0f, true);
    h[4 * i] = a[0]; h[4 * i + 1] = a[1]; h[4 * i + 2] = b[0]; h[4 * i + 3] = b[1];
  }
  return h;
}

__device__ __forceinline__ void unpack_bf16x8(const uint4& u, float* f) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

struct ChunkPos {
  int n;          // sequence
  int c;          // chunk index within the sequence
  int64_t row0;   // first token row (row = b*T + t, or packed offset)
  int len;        // valid tokens in this chunk (1..64)
};

// ---------------------------------------------------------------------------
// chunk map for packed sequences: chunk_off[n] = sum_{m<n} ceil(L_m / 64)
__global__ void kda_chunk_map_kernel(const int64_t* __restrict__ cu, int N, int* __restrict__ chunk_off) {
  const int lane = threadIdx.x;  // one wave of 64
  int carry = 0;
  if (lane == 0) chunk_off[0] = 0;
  for (int base = 0; base < N; base += 64) {
    int n = base + lane;
    int cnt = 0;
    if (n < N) {
      int64_t L = cu[n + 1] - cu[n];
      cnt = (int)((L + CH - 1) / CH);
    }
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      int o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    if (n < N) chunk_off[n + 1] = carry + incl;
    carry += __shfl(incl, 63);
  }
}

__device__ __forceinline__ bool chunk_pos(int x, int B, int T, int N, const int64_t* cu,
                                          const int* chunk_off, ChunkPos& cp) {
  if (cu == nullptr) {
    const int nc = (T + CH - 1) / CH;
    if (x >= B * nc) return false;
    cp.n = x / nc;
    cp.c = x % nc;
    cp.row0 = (int64_t)cp.n * T + (int64_t)cp.c * CH;
    cp.len = min(CH, T - cp.c * CH);
    return true;
  }
  if (x >= chunk_off[N]) return false;
  int lo = 0, hi = N;  // find n: chunk_off[n] <= x < chunk_off[n+1]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (chunk_off[mid] <= x) lo = mid; else hi = mid;
  }
  cp.n = lo;
  cp.c = x - chunk_off[lo];
  cp.row0 = cu[lo] + (int64_t)cp.c * CH;
  cp.len = (int)min((int64_t)CH, cu[lo + 1] - cp.row0);
  return true;
}

// ---------------------------------------------------------------------------
// intra-chunk kernel
//
// Register layout: wave w owns the 16-row sub-chunk I = w (rows 16I..16I+15);
// lane l = (i = l & 15, g = l >> 4) holds row r = 16I + i and the 32 channels
// c = 32*kb + 8*g + e (kb = 0..3, e = 0..7).  This is exactly the operand
// layout of v_mfma_*_16x16x32 (A: row i, B: column-row i, slots 8g..8g+7 of
// each 32-channel k-block), so every per-element factor is formed in
// registers and fed to the MFMA without moving it.
//
// Exponent safety.  With p = last row of sub-chunk I-1 (Gamma_p = 0 for I = 0)
// and e = last row of sub-chunk I, every element needs only
//     R = 2^(Gamma_r - Gamma_p) <= 1   and   C = 2^(Gamma_e - Gamma_r) <= 1.
// All other factors are per-channel vectors, computed once per chunk:
//     P_I  = 2^Gamma_p            (Q . 2^Gamma = qR P_I, K . 2^Gamma = kR P_I)
//     L_I  = 2^(Gamma_63 - Gamma_e)   (K . 2^(Gamma_63 - Gamma) = kC L_I)
//     D_IJ = 2^(Gamma_p(I) - Gamma_e(J)), I >= J + 2 (off-diagonal columns)
//     Mr_I = 2^(Gamma_p - Gamma_m), Mc_I = 2^(Gamma_m - Gamma_e), m = 16I + 8
// Off-diagonal block (I, J < I): rows qR, kR against columns kC D_IJ -- all
// factors <= 1, fp16 MFMA (kC is posted once in fp16; the reader multiplies
// it by D_IJ, also in fp16).  Diagonal block, safe gate: rows kR Mr against
// columns kC Mc, i.e. both sides offset by the sub-chunk midpoint, with
// exponents within 8 * |lower_bound| * log2(e) of zero (at most 2^58), as
// bf16 hi/lo products.  Diagonal block, unbounded decays (softplus gate,
// pre-gated decay): the same midpoint form where a sub-chunk's decay span
// allows it, else binary levels, one fp16 product per level (diag_level).
constexpr int AS = 68;      // fp32 row stride of Akk / T
constexpr int AQS = 72;     // fp16 row stride of Aqk
constexpr int KER = 144;    // fp16 row stride of the row-major [t][k] K . 2^G and Kd tiles
constexpr int WTS = 80;     // fp16 row stride of the [k][t] W staging tile
// Tiles read by lds_frag_tr_grouped keep their rows in groups of 8 with a 64-element
// gap after each group: the four rows of a lane group fall on different
// banks through the row stride, and the gap shifts the next group of rows
// (the other lane group served in the same pass) by half the banks.
constexpr int KEG = 8 * KER + 64;  // group stride of the K . 2^G / Kd tiles
constexpr int WG8 = 8 * WTS + 64;  // group stride of the W staging tile
__device__ __forceinline__ int ke_row(int t) { return (t & 7) * KER + (t >> 3) * KEG; }
__device__ __forceinline__ int w_row(int k) { return (k & 7) * WTS + (k >> 3) * WG8; }
constexpr int NVEC = 16;    // per-channel fp32 vectors: P0..3, L0..3, Mr0..3, Mc0..3
constexpr int V_P = 0, V_L = 4, V_MR = 8, V_MC = 12;
constexpr int NDH = 4;      // per-channel fp16 vectors D20, D30, D31 and ones (read by the off-diagonal blocks)

// LDS plan (bytes).  Region X is reused: mailbox (phases 3-4), Kd staging
// (phase 4b), then Akk fp32 / W staging (phases 5-7).  Region T holds the
// sub-chunk totals, midpoints and per-channel vectors until phase 4, then T.
constexpr int MB_BYTES = 3 * 4 * 64 * 16;               // column sub-chunks J = 0..2 x 4 k-blocks x 64 lanes x 16 B
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int X_BYTES = cmax(cmax(MB_BYTES, 64 * AS * 4), cmax(16 * WG8 * 2, 8 * KEG * 2));
constexpr int L_X = 0;
constexpr int L_T = L_X + X_BYTES;
constexpr int T_BYTES = 64 * AS * 4;
constexpr int L_TOT = L_T;                              // [4][128] f32, inside region T
constexpr int L_MID = L_TOT + 4 * 128 * 4;              // [4][128] f32
constexpr int L_VEC = L_MID + 4 * 128 * 4;              // [NVEC][128] f32
constexpr int L_DH = L_VEC + NVEC * 128 * 4;            // [NDH][128] fp16
constexpr int L_KE = L_T + T_BYTES;
constexpr int L_AQ = L_KE + 8 * KEG * 2;
constexpr int L_BETA = L_AQ + 64 * AQS * 2;
constexpr int L_QD = L_BETA + 64 * 4;  // unbounded decays: q_i . k_i per row [64] f32
constexpr int L_END = L_QD + 64 * 4;
static_assert(L_DH + NDH * 128 * 2 <= L_T + T_BYTES, "vectors fit in region T");

template <int CTRL>
__device__ __forceinline__ float dpp_row_shr(float x) {
  // lane i of each 16-lane row reads lane i - k of the same row; lanes with
  // no source keep `old` = 0
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Magnitudes are compared as the bit patterns of |x|: for non-negative floats
// the unsigned integer order is the numeric order, and integer maxima need
// none of the NaN canonicalisation a float maximum of loaded values does.
__device__ __forceinline__ uint32_t abs_bits(float x) { return __builtin_bit_cast(uint32_t, x) & 0x7fffffffu; }

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t x) {
  // lanes outside ROWS, and lanes with no source, take 0 (the identity of an
  // unsigned maximum) and so keep their own value; with that identity the
  // compiler fuses the move into the maximum (one DPP instruction per step)
  return max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, 0xf, true));
}

// Largest value over a wave (as |x| bit patterns): row maxima by DPP shifts,
// then rows 0+1 and 2+3 and all four by row broadcasts; lane 63 holds it.
__device__ __forceinline__ uint32_t wave_max_bits(uint32_t x) {
  x = dpp_max_u32<0x111, 0xf>(x);  // row_shr:1
  x = dpp_max_u32<0x112, 0xf>(x);  // row_shr:2
  x = dpp_max_u32<0x114, 0xf>(x);  // row_shr:4
  x = dpp_max_u32<0x118, 0xf>(x);  // row_shr:8: lane 15 of each row holds its row
  x = dpp_max_u32<0x142, 0xa>(x);  // row_bcast:15 into rows 1, 3
  x = dpp_max_u32<0x143, 0xc>(x);  // row_bcast:31 into rows 2, 3
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// log2-domain gate activation of x = g + dt_bias (A_exp = exp(A_log)); with a
// pre-gated decay, x = g is the natural-log decay itself.
template <int MODE>
__device__ __forceinline__ float gate2(float x, float A_exp, float lb_log2e) {
  if (MODE == KDA_GATE_PREGATED) {
    return fmaxf(kLog2e * x, kMinLog2Decay);
  } else if (MODE == KDA_GATE_SAFE_SIGMOID) {
    // lb * sigmoid(A x) * log2(e)
    return lb_log2e * fast_rcp(1.0f + fast_exp2(-(A_exp * kLog2e) * x));
  } else {
    // -A * softplus(x) * log2(e), softplus(x) = max(x, 0) + log1p(e^-|x|)
    // (both forms are evaluated and one is selected: the choice differs from
    // lane to lane, and a branch would run both sides anyway)
    const float ex = fast_exp2(-kLog2e * fabsf(x));
    const float l1p_series = ex * (1.0f - ex * (0.5f - ex * (1.0f / 3.0f)));
    const float l1p_log = fast_log2(1.0f + ex) * 0.6931471805599453f;
    const float l1p = (ex < 0.0078125f) ? l1p_series : l1p_log;
    const float a2 = -(A_exp * kLog2e) * (fmaxf(x, 0.0f) + l1p);
    return fmaxf(a2, kMinLog2Decay);
  }
}

__device__ __forceinline__ half8 to_half8(const float* v) {
  half8 h;
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = (_Float16)v[e];
  return h;
}

// Diagonal block for unbounded decays (softplus gate, pre-gated decay): the
// per-token decay has no bound, so no single
// reference row keeps both factors of every pair in range.  Instead the block
// is split by levels: at level L the rows form blocks of 2^(4-L) with halves
// of 2^(3-L); every pair i > j lies in exactly one (lower half, upper half)
// rectangle -- the level of the highest bit where i and j differ -- and with
// the reference p = last row of the upper half both factors
// 2^(Gamma_i - Gamma_p) and 2^(Gamma_p - Gamma_j) are <= 1.  Each row is in
// the lower half (a row operand) or the upper half (a column operand) of its
// level block, so one factor 2^-|Gamma_r - Gamma_p| per element and level
// suffices, and a level is one fp16 product over the channels; products of
// rows and columns from different level blocks are discarded afterwards.
// The reference value sits in another lane of the same 16-lane row.
template <int L>
__device__ __forceinline__ float level_ref(float x) {
  const int xi = __builtin_bit_cast(int, x);
  int r;
  if constexpr (L == 0) {
    r = __builtin_amdgcn_ds_swizzle(xi, 0xF0);  // lane (i & 0x10) | 7 of each 32: row 7
  } else if constexpr (L == 1) {
    const int t = __builtin_amdgcn_update_dpp(0, xi, 0xFF, 0xf, 0xf, false);  // quad_perm 3,3,3,3
    r = __builtin_amdgcn_update_dpp(t, t, 0x114, 0xf, 0xA, false);            // row_shr:4 into lanes 4-7, 12-15
  } else if constexpr (L == 2) {
    r = __builtin_amdgcn_update_dpp(0, xi, 0x55, 0xf, 0xf, false);  // quad_perm 1,1,1,1
  } else {
    r = __builtin_amdgcn_update_dpp(0, xi, 0xA0, 0xf, 0xf, false);  // quad_perm 0,0,2,2
  }
  return __builtin_bit_cast(float, r);
}

template <int L>
__device__ __forceinline__ void diag_level(const float (&Gk)[8], const float (&kf)[8], const float (&qf)[8], int li,
                                           f32x4& akk, f32x4& aqk) {
  const bool lower = (li >> (3 - L)) & 1;
  float a[8], aq[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float F = fast_exp2(-fabsf(Gk[e] - level_ref<L>(Gk[e])));
    a[e] = kf[e] * F;
    aq[e] = qf[e] * F;
  }
  const half8 ha = to_half8(a), hq = to_half8(aq), z = {};
  const half8 A = lower ? ha : z, Aq = lower ? hq : z, Bc = lower ? z : ha;
  akk = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bc, akk, 0, 0, 0);
  aqk = __builtin_amdgcn_mfma_f32_16x16x32_f16(Aq, Bc, aqk, 0, 0, 0);
}

// (lds_read_tr16 and lds_frag_tr_grouped, the transposing LDS reads, are in kda_device.h)

template <int MODE>
__global__ void __launch_bounds__(256, 2)
kda_intra_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                 const uint16_t* __restrict__ g, const uint16_t* __restrict__ beta,
                 const float* __restrict__ A_log, const float* __restrict__ dt_bias,
                 const int64_t* __restrict__ cu, const int* __restrict__ chunk_off,
                 int B, int T, int N, int Hqk, int Hv, int max_chunks,
                 float scale, float lower_bound, int flags, uint8_t* __restrict__ ws) {
  constexpr int LDS = L_END;
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS];
  uint8_t* sX = smem + L_X;                                          // mailbox / Kd staging / Akk / W staging
  float* sA = reinterpret_cast<float*>(smem + L_X);
  _Float16* sW = reinterpret_cast<_Float16*>(smem + L_X);
  _Float16* sKd = reinterpret_cast<_Float16*>(smem + L_X);
  float* sT = reinterpret_cast<float*>(smem + L_T);
  _Float16* sKE = reinterpret_cast<_Float16*>(smem + L_KE);
  _Float16* sAq = reinterpret_cast<_Float16*>(smem + L_AQ);
  float* sTot = reinterpret_cast<float*>(smem + L_TOT);
  float* sMid = reinterpret_cast<float*>(smem + L_MID);
  float* sVec = reinterpret_cast<float*>(smem + L_VEC);
  _Float16* sDh = reinterpret_cast<_Float16*>(smem + L_DH);
  float* sBeta = reinterpret_cast<float*>(smem + L_BETA);
  float* sQd = reinterpret_cast<float*>(smem + L_QD);

  const int x = blockIdx.x, h = blockIdx.y;
  ChunkPos cp;
  if (!chunk_pos(x, B, T, N, cu, chunk_off, cp)) return;
  const int hq = h / (Hv / Hqk);
  // the wave index is uniform: keeping it in a scalar register turns every
  // test on the sub-chunk index into a scalar branch
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int I = wave;
  const int r = 16 * I + li;
  const bool valid = r < cp.len;
  uint8_t* blk = ws + ((size_t)h * max_chunks + x) * BLOCK;

  // ---- phase 1: loads, gate, norms, beta, in-register 16-row scan
  // G holds the scan local to the sub-chunk: G = Gamma_r - Gamma_p.  rq, rk
  // are the L2-norm factors of this lane's row (1 with the norm off): q and k
  // are scaled by them as soon as they are unpacked, before any rounding to
  // 16 bits, so no 16-bit operand depends on the size of the raw inputs.
  float G[4][8];
  uint4 qraw[4], kraw[4];
  float rq, rk;
  {
    // a missing A_log means a multiplier of one (unused for pre-gated decay)
    const float A_exp = (MODE == KDA_GATE_PREGATED || A_log == nullptr) ? 1.0f : expf(A_log[h]);
    const float lb_log2e = lower_bound * kLog2e;
    // All input loads are issued before any use, as range-checked buffer loads:
    // rows at or beyond the chunk length read as zero, so no branch (and no
    // exposed latency per k-block) is needed.
    const uint32_t vrow = (uint32_t)li;
    const __amdgpu_buffer_rsrc_t rg = buffer_rsrc(g + ((size_t)(cp.row0 + 16 * I) * Hv + h) * DK,
                                                  (uint32_t)max(0, min(16, cp.len - 16 * I)) * Hv * DK * 2);
    const __amdgpu_buffer_rsrc_t bq = buffer_rsrc(q + ((size_t)(cp.row0 + 16 * I) * Hqk + hq) * DK,
                                                  (uint32_t)max(0, min(16, cp.len - 16 * I)) * Hqk * DK * 2);
    const __amdgpu_buffer_rsrc_t bk = buffer_rsrc(k + ((size_t)(cp.row0 + 16 * I) * Hqk + hq) * DK,
                                                  (uint32_t)max(0, min(16, cp.len - 16 * I)) * Hqk * DK * 2);
    // beta, then g (and dt_bias) first: loads complete in order, so the gate
    // and the scan below, which need only those, run while q and k are in
    // flight (beta is used only after the scan; a range-checked load, since a
    // conditional one became a branch with a full wait after it)
    const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(beta + (size_t)cp.row0 * Hv + h, (uint32_t)max(0, cp.len) * Hv * 2);
    const float blogit = bf2f((uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rb, (uint32_t)(r * Hv) * 2, 0, 0));
    uint4 graw[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      graw[kb] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(rg, (vrow * Hv * DK + 32 * kb + 8 * lg) * 2, 0, 0));
    float4 dtb4[8];
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) dtb4[kb] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (dt_bias != nullptr) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        dtb4[2 * kb] = *reinterpret_cast<const float4*>(dt_bias + (size_t)h * DK + 32 * kb + 8 * lg);
        dtb4[2 * kb + 1] = *reinterpret_cast<const float4*>(dt_bias + (size_t)h * DK + 32 * kb + 8 * lg + 4);
      }
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const uint32_t c0 = 32 * kb + 8 * lg;
      qraw[kb] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(bq, (vrow * Hqk * DK + c0) * 2, 0, 0));
      kraw[kb] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(bk, (vrow * Hqk * DK + c0) * 2, 0, 0));
    }
    // (kept here: the scheduler would otherwise sink the q and k loads below
    // the gate's first wait)
    __builtin_amdgcn_sched_barrier(0);
    const float vmask = valid ? 1.0f : 0.0f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      unpack_bf16x8(graw[kb], G[kb]);
      const float dtb[8] = {dtb4[2 * kb].x, dtb4[2 * kb].y, dtb4[2 * kb].z, dtb4[2 * kb].w,
                            dtb4[2 * kb + 1].x, dtb4[2 * kb + 1].y, dtb4[2 * kb + 1].z, dtb4[2 * kb + 1].w};
#pragma unroll
      // the gate of a row past the chunk end (zero inputs, finite) times 0:
      // a product, where a select had the compiler branch around each
      // element's exponential
      for (int e = 0; e < 8; ++e) G[kb][e] = gate2<MODE>(G[kb][e] + dtb[e], A_exp, lb_log2e) * vmask;
    }
    // the 32 scans of a lane advance together, one shift at a time: each DPP
    // step then reads a value written many instructions earlier (no hazard wait)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) G[kb][e] += dpp_row_shr<0x111>(G[kb][e]);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) G[kb][e] += dpp_row_shr<0x112>(G[kb][e]);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) G[kb][e] += dpp_row_shr<0x114>(G[kb][e]);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) G[kb][e] += dpp_row_shr<0x118>(G[kb][e]);
    // the L2-norm factors, once q and k have arrived
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float qf[8], kf[8];
      unpack_bf16x8(qraw[kb], qf);
      unpack_bf16x8(kraw[kb], kf);
#pragma unroll
      for (int e = 0; e < 8; ++e) { sq += qf[e] * qf[e]; sk += kf[e] * kf[e]; }
    }
    sq += __shfl_xor(sq, 16); sq += __shfl_xor(sq, 32);
    sk += __shfl_xor(sk, 16); sk += __shfl_xor(sk, 32);
    const bool norm = flags & KDA_FLAG_QK_L2NORM;
    rq = norm ? rsqrtf(sq + kL2Eps) : 1.0f;
    rk = norm ? rsqrtf(sk + kL2Eps) : 1.0f;
    if (lg == 0) {
      const float bp = (flags & KDA_FLAG_BETA_IS_PROB) ? blogit : fast_rcp(1.0f + fast_exp2(-kLog2e * blogit));
      sBeta[r] = valid ? bp : 0.0f;
    }
    // sub-chunk totals (row 15) and midpoint values (row 8), both local
    if (li == 15 || li == 8) {
      float* dst = (li == 15 ? sTot : sMid) + I * 128;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        float4* p4 = reinterpret_cast<float4*>(dst + 32 * kb + 8 * lg);
        p4[0] = make_float4(G[kb][0], G[kb][1], G[kb][2], G[kb][3]);
        p4[1] = make_float4(G[kb][4], G[kb][5], G[kb][6], G[kb][7]);
      }
    }
  }
  // The diagonal block: through the sub-chunk midpoint (phase 3) when the
  // sub-chunk's decay spans at most 2^100 in every channel, so that every
  // offset factor times a q or k element (below 2^15) is a normal bf16 --
  // always with the safe gate, whose decay per token is bounded (a span of
  // at most 2^58) -- else by binary levels (below).  G is non-increasing down
  // the rows, so its largest size is the sub-chunk total.
  bool mid_ok = true;
  if constexpr (MODE != KDA_GATE_SAFE_SIGMOID) {
    float mg = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) mg = fmaxf(mg, -G[kb][e]);
    mid_ok = (int)wave_max_bits(abs_bits(mg)) <= __builtin_bit_cast(int, 100.0f);
  }
  // four partial accumulators of the diagonal block (midpoint form), or one
  // per level (level form)
  f32x4 dkkp[4], dqkp[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) { dkkp[j] = f32x4{0, 0, 0, 0}; dqkp[j] = f32x4{0, 0, 0, 0}; }
  float qkd = 0.0f;
  if (MODE != KDA_GATE_SAFE_SIGMOID && !mid_ok) {
    // diagonal block by levels (see diag_level); its diagonal is q_i . k_i
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float qf[8], kf[8];
      unpack_bf16x8(qraw[kb], qf);
      unpack_bf16x8(kraw[kb], kf);
#pragma unroll
      for (int e = 0; e < 8; ++e) { qf[e] *= rq; kf[e] *= rk; qkd += qf[e] * kf[e]; }
      // one level at a time keeps the temporaries of only one level live
      diag_level<0>(G[kb], kf, qf, li, dkkp[0], dqkp[0]);
      __builtin_amdgcn_sched_barrier(0);
      diag_level<1>(G[kb], kf, qf, li, dkkp[1], dqkp[1]);
      __builtin_amdgcn_sched_barrier(0);
      diag_level<2>(G[kb], kf, qf, li, dkkp[2], dqkp[2]);
      __builtin_amdgcn_sched_barrier(0);
      diag_level<3>(G[kb], kf, qf, li, dkkp[3], dqkp[3]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (MODE != KDA_GATE_SAFE_SIGMOID && !mid_ok) {
    qkd += __shfl_xor(qkd, 16);
    qkd += __shfl_xor(qkd, 32);
    if (lg == 0) sQd[r] = qkd;
  }
  __syncthreads();

  // ---- phase 2: per-channel vectors from the sub-chunk totals T_J and local
  // midpoints M_J (every exponent is a sum of totals, so none is a difference
  // of large cumulative values):
  //   P_I = 2^(T_0+..+T_{I-1}), L_I = 2^(T_{I+1}+..+T_3), D_IJ = 2^(T_{J+1}+..+T_{I-1}),
  //   Mr_I = 2^(-M_I), Mc_I = 2^(M_I - T_I), 2^Gamma_63 = 2^(T_0+..+T_3)
  {
    const int c = tid & 127, half = tid >> 7;
    const float T0 = sTot[c], T1 = sTot[128 + c], T2 = sTot[256 + c], T3 = sTot[384 + c];
    if (half == 0) {
      sVec[(V_P + 0) * 128 + c] = 1.0f;
      sVec[(V_P + 1) * 128 + c] = fast_exp2(T0);
      sVec[(V_P + 2) * 128 + c] = fast_exp2(T0 + T1);
      sVec[(V_P + 3) * 128 + c] = fast_exp2((T0 + T1) + T2);
      reinterpret_cast<float*>(blk + F_VEC * FRAG)[c] = fast_exp2(((T0 + T1) + T2) + T3);
      sDh[0 * 128 + c] = (_Float16)fast_exp2(T1);
      sDh[1 * 128 + c] = (_Float16)fast_exp2(T1 + T2);
      sDh[2 * 128 + c] = (_Float16)fast_exp2(T2);
      sDh[3 * 128 + c] = (_Float16)1.0f;  // adjacent sub-chunks: no factor
    } else {
      sVec[(V_L + 0) * 128 + c] = fast_exp2((T1 + T2) + T3);
      sVec[(V_L + 1) * 128 + c] = fast_exp2(T2 + T3);
      sVec[(V_L + 2) * 128 + c] = fast_exp2(T3);
      sVec[(V_L + 3) * 128 + c] = 1.0f;
      const float Tj[4] = {T0, T1, T2, T3};
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        const float m = sMid[J * 128 + c];
        sVec[(V_MR + J) * 128 + c] = fast_exp2(-m);
        sVec[(V_MC + J) * 128 + c] = fast_exp2(m - Tj[J]);
      }
    }
  }
  __syncthreads();

  // ---- phase 3: per-element factors R = 2^G, C = 2^(T_I - G); outputs that
  // need no other row; column operands for the later row blocks
  // accumulators: the diagonal block, and off-diagonal blocks J = 0..2 (J < I);
  // all register arrays are indexed by compile-time values only
  f32x4 dkk = f32x4{0, 0, 0, 0}, dqk = f32x4{0, 0, 0, 0};
  f32x4 okk[3], oqk[3];
#pragma unroll
  for (int J = 0; J < 3; ++J) { okk[J] = f32x4{0, 0, 0, 0}; oqk[J] = f32x4{0, 0, 0, 0}; }
  half8 aK[4], aQ[4], kdh[4], kdl[4];
  {
    const float* vP = sVec + (V_P + I) * 128;
    const float* vL = sVec + (V_L + I) * 128;
    const float* vMr = sVec + (V_MR + I) * 128;
    const float* vMc = sVec + (V_MC + I) * 128;
    const float* vT = sTot + I * 128;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int c0 = 32 * kb + 8 * lg;
      float kR[8], qR[8], kC[8];
      {
        float qf[8], kf[8];
        unpack_bf16x8(qraw[kb], qf);
        unpack_bf16x8(kraw[kb], kf);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          qf[e] *= rq;
          kf[e] *= rk;
          const float R = fast_exp2(G[kb][e]);
          const float C = fast_exp2(vT[c0 + e] - G[kb][e]);
          kR[e] = kf[e] * R;
          qR[e] = qf[e] * R;
          kC[e] = kf[e] * C;
        }
      }
      aK[kb] = to_half8(kR);
      aQ[kb] = to_half8(qR);
      {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = qR[e] * vP[c0 + e];
        st_frag(blk, F_QG + I * 4 + kb, lane, __builtin_bit_cast(u32x4, to_half8(o)));
      }
      {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = kR[e] * vP[c0 + e];
        *reinterpret_cast<half8*>(sKE + ke_row(r) + c0) = to_half8(o);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float kd = kC[e] * vL[c0 + e];
        const _Float16 hh = (_Float16)kd;
        kdh[kb][e] = hh;
        kdl[kb][e] = (_Float16)__builtin_amdgcn_fmed3f((kd - (float)hh) * kKdLoScale, -kE4m3Max, kE4m3Max);
      }
      // the column operand of the off-diagonal blocks (I', I), I' > I; the
      // blocks with I' >= I + 2 scale it by D_(I'I) as they read it, so every
      // posting wave does the same work
      if (I < 3) *reinterpret_cast<half8*>(sX + ((I * 4 + kb) * 64 + lane) * 16) = to_half8(kC);
      if (mid_ok) {
        // diagonal block, both sides offset by the midpoint.  The factors span
        // up to 2^+-58, within bf16's exponent range but not fp16's: each
        // operand is split into bf16 hi + lo, and three products (hi hi, hi
        // lo, lo hi) on the bf16 MFMA give the block to about 2^-16 of its
        // terms, for an eighth of the fp32 MFMA's issue time.  One
        // accumulator per channel block keeps the chains short.
        bf16x8 ah, al, qh, ql, bh, bl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a = kR[e] * vMr[c0 + e], aq = qR[e] * vMr[c0 + e], b = kC[e] * vMc[c0 + e];
          ah[e] = (__bf16)a;
          al[e] = (__bf16)(a - (float)ah[e]);
          qh[e] = (__bf16)aq;
          ql[e] = (__bf16)(aq - (float)qh[e]);
          bh[e] = (__bf16)b;
          bl[e] = (__bf16)(b - (float)bh[e]);
        }
        dkkp[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, dkkp[kb], 0, 0, 0);
        dqkp[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, bh, dqkp[kb], 0, 0, 0);
        dkkp[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, dkkp[kb], 0, 0, 0);
        dqkp[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, bl, dqkp[kb], 0, 0, 0);
        dkkp[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, dkkp[kb], 0, 0, 0);
        dqkp[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql, bh, dqkp[kb], 0, 0, 0);
      }
    }
  }
  if (mid_ok) {
    dkk = (dkkp[0] + dkkp[1]) + (dkkp[2] + dkkp[3]);
    dqk = (dqkp[0] + dqkp[1]) + (dqkp[2] + dqkp[3]);
  }
  __syncthreads();

  // ---- phase 4: off-diagonal blocks from the mailbox; diagonal levels combined
  {
#pragma unroll
    for (int J = 0; J < 3; ++J) {
      if (J >= I) continue;
      // D_IJ in fp16 (D20, D30, D31; ones for I = J + 1): every block
      // multiplies, so no branch separates the reads from their use
      const _Float16* dh = sDh + (I == J + 1 ? 3 : I == 2 ? 0 : J == 0 ? 1 : 2) * 128;
      half8 bs[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        bs[kb] = *reinterpret_cast<const half8*>(sX + ((J * 4 + kb) * 64 + lane) * 16) *
                 *reinterpret_cast<const half8*>(dh + 32 * kb + 8 * lg);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const half8 b = bs[kb];
        okk[J] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aK[kb], b, okk[J], 0, 0, 0);
        oqk[J] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aQ[kb], b, oqk[J], 0, 0, 0);
      }
    }
    if (MODE != KDA_GATE_SAFE_SIGMOID && !mid_ok) {
      // pair (i, j), i > j, of the diagonal block belongs to the level of the
      // highest bit in which i and j differ
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        // (a chain of selects on scalars: nested conditionals on the vector
        // elements were compiled into branches)
        const int xd = (4 * lg + rr) ^ li;
        const float k0 = dkkp[0][rr], k1 = dkkp[1][rr], k2 = dkkp[2][rr], k3 = dkkp[3][rr];
        const float q0 = dqkp[0][rr], q1 = dqkp[1][rr], q2 = dqkp[2][rr], q3 = dqkp[3][rr];
        float vk = xd >= 2 ? k2 : k3, vq = xd >= 2 ? q2 : q3;
        vk = xd >= 4 ? k1 : vk; vq = xd >= 4 ? q1 : vq;
        vk = xd >= 8 ? k0 : vk; vq = xd >= 8 ? q0 : vq;
        const float qd = sQd[16 * I + 4 * lg + rr];  // read by every lane: no branch around the load
        dkk[rr] = vk;
        dqk[rr] = xd == 0 ? qd : vq;
      }
    }
  }
  __syncthreads();  // mailbox is dead

  // ---- phase 4b: (K . 2^(G_63 - G))^T hi then lo to global: staged row-major
  // [t][k] in LDS and read back transposed into fragment (key tile, token block)
  for (int part = 0; part < 2; ++part) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      *reinterpret_cast<half8*>(sKd + ke_row(r) + 32 * kb + 8 * lg) = part == 0 ? kdh[kb] : kdl[kb];
    __syncthreads();
    for (int it = 0; it < 4; ++it) {
      const int fr = wave + 4 * it;  // fragment (km = fr >> 1, kb = fr & 1)
      const u32x4 f = lds_frag_tr_grouped(sKd, KER, KEG, 32 * (fr & 1), 16 * (fr >> 1), lane);
      if (part == 0) st_frag(blk, F_KD + fr, lane, f);
      else st_half_frag(blk, (F_KDL + (fr >> 1)) * FRAG + 8 * (fr & 1), lane, pack_e4m3(f));
    }
    __syncthreads();
  }

  // ---- phase 5: Akk (fp32) and Aqk (fp16) into LDS with masks, beta and scale.
  // Blocks above the diagonal: Aqk is written as zero (it is copied out whole);
  // Akk is never read there, and the blocks of T above the diagonal are never
  // written: every reader of T masks them.
  {
    float fk[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) fk[rr] = sBeta[16 * I + 4 * lg + rr];
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      if (J > I) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) sAq[(16 * I + 4 * lg + rr) * AQS + 16 * J + li] = (_Float16)0.0f;
        continue;
      }
      f32x4 vk, vq;
      if (J == I) { vk = dkk; vq = dqk; }
      else { vk = okk[J < 3 ? J : 0]; vq = oqk[J < 3 ? J : 0]; }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int row = 16 * I + 4 * lg + rr, col = 16 * J + li;
        float akk = vk[rr] * fk[rr];
        float aqk = vq[rr] * scale;
        if (J == I) {
          akk = (4 * lg + rr > li) ? akk : 0.0f;
          aqk = (4 * lg + rr >= li) ? aqk : 0.0f;
        }
        sA[row * AS + col] = akk;
        sAq[row * AQS + col] = (_Float16)aqk;
      }
    }
  }
  __syncthreads();

  // ---- phase 6: T = (I + Akk)^-1
  if (lane < 16) {
    const int j = lane, o = 16 * wave;
    float xcol[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = (i == j) ? 1.0f : 0.0f;
#pragma unroll
      for (int m = 0; m < i; ++m) s -= sA[(o + i) * AS + o + m] * xcol[m];
      xcol[i] = s;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sT[(o + i) * AS + o + j] = xcol[i];
  }
  __syncthreads();
  for (int d = 1; d < 4; ++d) {
    if (wave < 4 - d) {
      const int Ib = wave + d, Jb = wave;
      f32x4 z = f32x4{0, 0, 0, 0};
      for (int Kb = Jb; Kb < Ib; ++Kb) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const float a = sA[(16 * Ib + li) * AS + 16 * Kb + 4 * kb + lg];
          const float b = sT[(16 * Kb + 4 * kb + lg) * AS + 16 * Jb + li];
          z = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, z, 0, 0, 0);
        }
      }
      f32x4 y = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float a = sT[(16 * Ib + li) * AS + 16 * Ib + 4 * lg + rr];
        y = __builtin_amdgcn_mfma_f32_16x16x4f32(a, z[rr], y, 0, 0, 0);
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) sT[(16 * Ib + 4 * lg + rr) * AS + 16 * Jb + li] = -y[rr];
    }
    __syncthreads();
  }

  // ---- phase 7: W = T diag(b) (K . 2^G); T diag(b) hi/lo; Aqk
  {
    f32x4 accw[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) accw[nt] = f32x4{0, 0, 0, 0};
    const int t = 16 * wave + li;
    const int nkb = (wave >= 2) ? 2 : 1;
    for (int kb = 0; kb < nkb; ++kb) {
      const int s0 = 32 * kb + 8 * lg;
      // column block 2 kb + (lg >> 1) above the diagonal block I is zero
      const bool keep = 2 * kb + (lg >> 1) <= I;
      half8 a;
#pragma unroll
      // every lane reads (T above the diagonal holds stale values, dropped by
      // the select): a load under the lane-dependent condition is a branch
      for (int e = 0; e < 8; ++e) {
        const float tb = sT[t * AS + s0 + e] * sBeta[s0 + e];
        a[e] = keep ? (_Float16)tb : (_Float16)0.0f;
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const half8 b = __builtin_bit_cast(half8, lds_frag_tr_grouped(sKE, KER, KEG, 32 * kb, 16 * nt, lane));
        accw[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, accw[nt], 0, 0, 0);
      }
    }
    for (int it = 0; it < 2; ++it) {
      const int item = tid + 256 * it;  // stored fragment x lane
      if (item >= NTRI * 64) break;     // (waves 2, 3 in the second pass)
      const int fr = item >> 6, ln = item & 63;
      const int ta = tri_ta(fr), kb = tri_kb(fr);
      const int row = 16 * ta + (ln & 15), c0 = 32 * kb + 8 * (ln >> 4);
      bf16x8 th, tl;
      const bool keep = 2 * kb + (ln >> 5) <= ta;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float tb = sT[row * AS + c0 + e] * sBeta[c0 + e];
        const float v = keep ? tb : 0.0f;
        const __bf16 hv = (__bf16)v;
        th[e] = hv;
        tl[e] = (__bf16)(v - (float)hv);
      }
      st_frag(blk, F_TBH + fr, ln, __builtin_bit_cast(u32x4, th));
      st_frag(blk, F_TBL + fr, ln, __builtin_bit_cast(u32x4, tl));
      st_frag(blk, F_AQK + fr, ln, *reinterpret_cast<const u32x4*>(sAq + row * AQS + c0));
    }
    // sA (region X) is dead after the solve: stage -W there
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      typedef _Float16 half4 __attribute__((ext_vector_type(4)));
      const half4 hv = {(_Float16)(-accw[nt][0]), (_Float16)(-accw[nt][1]), (_Float16)(-accw[nt][2]),
                        (_Float16)(-accw[nt][3])};
      *reinterpret_cast<half4*>(sW + w_row(16 * nt + li) + 16 * wave + 4 * lg) = hv;
    }
    __syncthreads();
    for (int it = 0; it < 4; ++it) {
      const int fr = wave + 4 * it;  // fragment (ta = fr >> 2, kb = fr & 3)
      st_frag(blk, F_WN + fr, lane, lds_frag_tr_grouped(sW, WTS, WG8, 32 * (fr & 3), 16 * (fr >> 2), lane));
    }
  }
}

// ---------------------------------------------------------------------------
// inter-chunk state kernel
//
// One workgroup of 4 waves (one per SIMD) per (sequence, v-head, 32-wide V
// slice), sequential over the sequence's chunks with the fp32 state slice
// S^T[k][v] in registers.  Wave w owns key rows 32w..32w+31 (key tiles 2w and
// 2w+1) of the state, for both 16-wide V tiles, and token tile w of U and O.
// Per chunk:
//     U = T diag(b) V - W S^T
//     O = scale (Q . 2^G) S^T + Aqk U
//     S <- S Diag(2^G_last) + U^T (K . 2^(G_last - G))
// Every wave contracts over the full key (or token) range itself, so the only
// exchanges are the state (fp16, for W S^T and Q S^T) and U (hi/lo, for the
// state update): two barriers per chunk.
//
// Range.  S and U reach the 16-bit operands as fp16, whose range is about
// 2^-14 .. 2^16, while v and the states may hold any bf16 / fp32 value.  The
// workgroup therefore keeps them in units of 2^E: chunk c converts S_c 2^-E_c
// and U_c 2^-E_(c+1), with one integer E per chunk shared by all the waves.
// Before the first barrier of chunk c each wave posts to LDS the largest
// magnitude of its S_c, its U_(c-1) and its token tile of T diag(b) V_c (in
// units of 2^E_c); after the barrier every wave reads the four values and
// sets E_(c+1) so that the largest lies in [1, 2).  T diag(b) V_c is formed
// at the start of chunk c for that purpose, from the V slice that chunk c - 1
// put in LDS (two V buffers alternate), so the scale follows what is written
// into the state this chunk, not the size of v: a chunk whose v is far larger
// than the state's stays in range, and writes with tiny beta keep their
// precision instead of flushing to zero.  The shift is applied with
// no branch: U, the state's decay factors and the output factor of the chunk
// carry 2^(E_c - E_(c+1)), so the update lands in units of E_(c+1).  Within
// one chunk S and U grow by far less than the 2^14 headroom this leaves under
// the fp16 limit.  Because E follows the magnitudes exactly, scaling v and
// the initial state by any power of two shifts E and changes nothing else:
// the results scale exactly, bit for bit.  Each operand fragment of a chunk is
// loaded by exactly one wave, straight into registers: the token-tile
// operands (W, Q . 2^G, T diag(b), Aqk) two chunks ahead, the key-tile
// operands (Kd) one chunk ahead -- they are needed only after the second
// barrier.  The loads are issued in groups between the MFMA products of each
// half of the step rather than in one burst before a barrier: a wave whose
// loads find the memory queue full stalls at issue, and before a barrier that
// holds up all four.  The V slices of one chain run on one XCD and share its L2.
constexpr int SWAVES = 4;
// What one state workgroup computes over its range of chunks:
//   ST_FULL   outputs and the state (the whole chain, or one segment of it
//             from that segment's true entry state);
//   ST_CARRY  the state only, no outputs (a segment carried from zero, or
//             the first segment from the initial state);
//   ST_TRANS  the segment's linear map P: the same recurrence with v = 0
//             started from the identity, on key rows instead of value rows.
constexpr int SSS = 136;  // sS row stride (fp16): state slice stored as [v][k]
constexpr int SUS = 72;   // sU row stride (fp16): U' stored as [v][t]
// sV: the V slice row-major [t][v] (16-bit), rows in groups of 8 with a
// 64-element gap after each group.  A transposed operand read takes rows
// r0 + 8 g + (0..3) (g = lane >> 4): the row stride puts the four rows of
// one lane group on different banks, and the gap shifts the next group by
// half the banks, so the two lane groups served together do not collide.
template <int NVT> constexpr int svs() { return NVT == 2 ? 48 : 80; }
template <int NVT> constexpr int svg() { return 8 * svs<NVT>() + 64; }
template <int NVT> __device__ __forceinline__ int sv_row(int t) { return (t & 7) * svs<NVT>() + (t >> 3) * svg<NVT>(); }
// one V buffer; two alternate by chunk parity
template <int NVT> constexpr int SV_HALFS = (CH / 8) * svg<NVT>();

struct ChunkRegs {
  // arrays indexed only by compile-time values (fully unrolled loops)
  u32x4 wn[4], qg[4];        // -W, Q . 2^G: token tile w, key blocks 0..3
  u32x4 tbh[2], tbl[2];      // T diag(b) hi/lo: token tile w, token blocks 0, 1
  u32x4 aq[2];               // Aqk: token tile w, token blocks 0, 1
  u32x4 vec;                 // bytes 256 w + 16 (lane & 15) of the vector fragment
  u32x4 vraw[2];             // V slice: row tid >> 2, columns 32 i + 8 (tid & 3) .. (i < NVT / 2)
  u32x4 kd[2][2];            // Kd^T hi: key tile 2w + j, token block b
  u32x2 kdl[2][2];           // and its e4m3 low part
};

// (a buffer load over the chunk-head block: the scalar base and immediate
// offsets take less address arithmetic than a flat pointer, measured 3 % faster)
__device__ __forceinline__ u32x4 ld_frag(const uint8_t* blk, int fr, int lane) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(buffer_rsrc(blk, (uint32_t)BLOCK),
                                                                          fr * FRAG + lane * 16, 0, 0));
}

// The V slice of one chunk: row tid >> 2, columns 32 i + 8 (tid & 3) ..;
// rows s >= len lie beyond the buffer range and read as zero.
template <int NVT>
__device__ __forceinline__ void load_v(ChunkRegs& o, const uint16_t* __restrict__ v, int64_t row0, int len, int Hv,
                                       int h, int v0, int tid) {
  const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(v + ((size_t)row0 * Hv + h) * DV + v0, (uint32_t)len * Hv * DV * 2);
#pragma unroll
  for (int i = 0; i < NVT / 2; ++i)
    o.vraw[i] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, ((tid >> 2) * Hv * DV + 32 * i + 8 * (tid & 3)) * 2, 0, 0));
}

// PART 0: token-tile operands, vectors and (narrow slices) V, issued two
// chunks ahead (wide slices: one chunk ahead, V two chunks ahead on its own),
// also in groups: PART 2 the W fragments, PART 4 the Q fragments, PART 3 the
// rest (PART 5 its vectors alone, PART 6 the rest without them, PART 7 that
// without V); PART 1: key-tile operands (issued one chunk ahead).
// Operands a kind does not use are neither loaded nor kept.
template <int PART, int KIND, int NVT>
__device__ __forceinline__ void load_chunk_part(ChunkRegs& o, const uint8_t* blk, int wave, int lane,
                                                const uint16_t* __restrict__ v, int64_t row0, int len, int Hv, int h,
                                                int v0, int tid) {
  if constexpr (PART == 0 || PART == 2) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) o.wn[kb] = ld_frag(blk, F_WN + wave * 4 + kb, lane);
  }
  if constexpr ((PART == 0 || PART == 4) && KIND == ST_FULL) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) o.qg[kb] = ld_frag(blk, F_QG + wave * 4 + kb, lane);
  }
  if constexpr (PART == 0 || PART == 3 || PART == 6 || PART == 7) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // token block 1 of token tiles 0, 1 is not stored: a fragment index past
      // the block reads zeros through the buffer range check, with no memory access
      const int tf = (kb == 1 && wave < 2) ? NFRAG : tri_frag(wave, kb);
      if constexpr (KIND != ST_TRANS) {
        o.tbh[kb] = ld_frag(blk, tf == NFRAG ? NFRAG : F_TBH + tf, lane);
        o.tbl[kb] = ld_frag(blk, tf == NFRAG ? NFRAG : F_TBL + tf, lane);
      }
      if constexpr (KIND == ST_FULL) o.aq[kb] = ld_frag(blk, tf == NFRAG ? NFRAG : F_AQK + tf, lane);
    }
  }
  if constexpr (PART == 0 || PART == 3 || PART == 5) o.vec = ld_frag(blk, F_VEC, 16 * wave + (lane & 15));
  if constexpr ((PART == 0 || PART == 3 || PART == 6) && KIND != ST_TRANS && NVT == NVT_NARROW)
    load_v<NVT>(o, v, row0, len, Hv, h, v0, tid);
  if constexpr (PART == 1) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int b = 0; b < 2; ++b) o.kd[j][b] = ld_frag(blk, F_KD + (2 * wave + j) * 2 + b, lane);
      // both token blocks' low parts in one load
      const u32x4 lo = ld_frag(blk, F_KDL + 2 * wave + j, lane);
      o.kdl[j][0] = u32x2{lo[0], lo[1]};
      o.kdl[j][1] = u32x2{lo[2], lo[3]};
    }
  }
}

struct StateCtx {
  const uint16_t* __restrict__ v;
  uint16_t* __restrict__ out;
  const uint8_t* wsh;
  int64_t bos, seqlen;
  int x0, nc, Hv, h, v0, tid, wave, lane, li, lg;
  float scale;
  uint32_t* sMx;  // [SWAVES] largest magnitude posted by each wave (|x| bit patterns)
  float* sVec;
  _Float16* sS;
  _Float16* sUh;
  _Float16* sUl;
  _Float16* sV;
};

// Output tiles of a finished chunk, held in registers and stored at the start
// of the next chunk, before that chunk's prefetch: stores count in vmcnt like
// loads, so a store queued behind a prefetch would lengthen the operand wait.
template <int NVT>
struct PendingOut {
  uint16_t o[NVT][4];
  int64_t row0;
  int len;
};

// wave w stores the output tiles of token tile w, V tiles 0 .. NVT-1
template <int NVT>
__device__ __forceinline__ void store_pending(const PendingOut<NVT>& pd, uint16_t* __restrict__ out, int Hv, int h,
                                              int v0, int wave, int li, int lg) {
  // rows t >= len fall outside the buffer range and are dropped
  const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(out + ((size_t)pd.row0 * Hv + h) * DV + v0, (uint32_t)pd.len * Hv * DV * 2);
#pragma unroll
  for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int t = 16 * wave + 4 * lg + rr;
      __builtin_amdgcn_raw_buffer_store_b16((short)pd.o[vt][rr], ro, (t * Hv * DV + 16 * vt + li) * 2, 0, 0);
    }
}

__device__ __forceinline__ int chunk_len(const StateCtx& x, int c) {
  return (int)min((int64_t)CH, x.seqlen - (int64_t)c * CH);
}

__device__ __forceinline__ half8 as_half8(const u32x4& u) { return __builtin_bit_cast(half8, u); }
__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& u) { return __builtin_bit_cast(bf16x8, u); }

// An empty use that forces the registers to be loaded here: issued once before
// the chunk loop, it completes the initial state and first chunk's loads
// there, so the loop is entered with nothing of them outstanding (otherwise
// the wait inserted at the loop head for that path is a full drain, paid on
// every iteration).
__device__ __forceinline__ void settle(const u32x4& a) { asm volatile("" ::"v"(a)); }
__device__ __forceinline__ void settle(const u32x2& a) { asm volatile("" ::"v"(a)); }
__device__ __forceinline__ void settle(const f32x4& a) { asm volatile("" ::"v"(a)); }
template <int KIND, int NVT>
__device__ __forceinline__ void settle(const ChunkRegs& r) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    settle(r.wn[kb]);
    if constexpr (KIND == ST_FULL) settle(r.qg[kb]);
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    if constexpr (KIND != ST_TRANS) { settle(r.tbh[kb]); settle(r.tbl[kb]); }
    if constexpr (KIND == ST_FULL) settle(r.aq[kb]);
  }
  settle(r.vec);
  if constexpr (KIND != ST_TRANS)
#pragma unroll
    for (int i = 0; i < NVT / 2; ++i) settle(r.vraw[i]);
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int b = 0; b < 2; ++b) { settle(r.kd[j][b]); settle(r.kdl[j][b]); }
}

// largest |value| of eight bf16 values packed in four dwords, as the bit
// pattern of that value in fp32
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x8_absmax_bits(const u32x4& w) {
  const u16x2 a = __builtin_bit_cast(u16x2, w[0] & 0x7fff7fffu), b = __builtin_bit_cast(u16x2, w[1] & 0x7fff7fffu);
  const u16x2 c = __builtin_bit_cast(u16x2, w[2] & 0x7fff7fffu), d = __builtin_bit_cast(u16x2, w[3] & 0x7fff7fffu);
  const u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  return (uint32_t)max(m[0], m[1]) << 16;
}

// The scale exponent is kept within [-kMaxExp, kMaxExp] and moves by at most
// kMaxStep per chunk, so that 2^E, 2^-E and the per-chunk factor 2^-d are
// normal floats and scale 2^-d stays finite.
constexpr int kMaxExp = 126, kMaxStep = 64;
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }

// floor(log2 m) for a normal m > 0, from its bit pattern (m >= 0)
__device__ __forceinline__ int ilog2_bits(int mi) { return (mi >> 23) - 127; }

// The shift d = E_(c+1) - E_c that brings the largest of the four posted
// maxima (units of 2^E_c) into [1, 2); 0 when all are zero.  Every wave reads
// the same four values, so d is uniform across the workgroup.
__device__ __forceinline__ int scale_shift(const uint32_t* sMx, int E) {
  const u32x4 m4 = *reinterpret_cast<const u32x4*>(sMx);
  const int mi = __builtin_amdgcn_readfirstlane((int)max(max(m4[0], m4[1]), max(m4[2], m4[3])));
  if (mi == 0) return 0;
  const int d = min(max(ilog2_bits(mi), -kMaxStep), kMaxStep);
  return min(max(E + d, -kMaxExp), kMaxExp) - E;
}

// ub tile vt = T diag(b) V (real units) of token tile w, from a chunk's
// T diag(b) fragments in `r` and its V slice in LDS at sVb
template <int KIND, int NVT>
__device__ __forceinline__ void ub_one(f32x4& u, const _Float16* sVb, const ChunkRegs& r, int vt, int lane) {
  u = f32x4{0, 0, 0, 0};
  if constexpr (KIND != ST_TRANS) {
    const bf16x8 vb0 = __builtin_bit_cast(bf16x8, lds_frag_tr_grouped(sVb, svs<NVT>(), svg<NVT>(), 0, 16 * vt, lane));
    const bf16x8 vb1 = __builtin_bit_cast(bf16x8, lds_frag_tr_grouped(sVb, svs<NVT>(), svg<NVT>(), 32, 16 * vt, lane));
    u = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(r.tbh[0]), vb0, u, 0, 0, 0);
    u = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(r.tbl[0]), vb0, u, 0, 0, 0);
    u = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(r.tbh[1]), vb1, u, 0, 0, 0);
    u = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(r.tbl[1]), vb1, u, 0, 0, 0);
  }
}
template <int KIND, int NVT>
__device__ __forceinline__ void ub_tile(f32x4 (&u)[NVT], const _Float16* sVb, const ChunkRegs& r, int lane) {
#pragma unroll
  for (int vt = 0; vt < NVT; ++vt) ub_one<KIND, NVT>(u[vt], sVb, r, vt, lane);
}

// Entry tiles S^T[k][v] (k = 32 wave + 16 j + 4 lg + rr, v = v0 + 16 vt + li)
// of a [V][K] state matrix at `src` + `base` elements: fp32, bf16, or zero
// (KDA_STATE_NONE).  Range-checked loads under one branch on the uniform
// dtype, where a conditional load per tile became a branch with a full memory
// wait after each.
template <int NVT>
__device__ __forceinline__ void load_entry_tiles(f32x4 (&S)[2][NVT], const void* src, int dtype, size_t base, int wave,
                                                 int v0, int li, int lg) {
  const bool f32 = dtype == KDA_STATE_F32, b16 = dtype == KDA_STATE_BF16;
  const void* b = f32 ? (const void*)(reinterpret_cast<const float*>(src) + base)
                      : b16 ? (const void*)(reinterpret_cast<const uint16_t*>(src) + base) : nullptr;
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(b, f32 ? (uint32_t)DV * DK * 4 : b16 ? (uint32_t)DV * DK * 2 : 0u);
  if (b16) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        const uint32_t e = (uint32_t)(v0 + 16 * vt + li) * DK + 32 * wave + 16 * j + 4 * lg;
        const u32x2 u = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, e * 2, 0, 0));
        S[j][vt] = f32x4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u), __uint_as_float(u[1] << 16),
                         __uint_as_float(u[1] & 0xffff0000u)};
      }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        const uint32_t e = (uint32_t)(v0 + 16 * vt + li) * DK + 32 * wave + 16 * j + 4 * lg;
        S[j][vt] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, e * 4, 0, 0));
      }
  }
}

// One chunk of the state chain: `cur` holds chunk c, `n1` receives the key-tile
// operands of chunk c+1, `n2` the token-tile operands of chunk c+2.  The wide
// slices (NVT = 4) have no registers for that depth: their token-tile
// operands of chunk c+1 go to `n1` too (`n2` unused), and their V of chunk
// c+2 goes to `cur`, whose own V is in LDS by then.  On entry S holds S_c in
// units of 2^E (E = E_c) and mu this wave's largest |U_(c-1)| in the same
// units; on exit S holds S_(c+1), E = E_(c+1) and mu the largest |U_c|.
template <int KIND, int NVT>
__device__ __forceinline__ void state_chunk(const StateCtx& x, f32x4 (&S)[2][NVT], ChunkRegs& cur, ChunkRegs& n1,
                                            ChunkRegs& n2, const int c, PendingOut<NVT>& pd, int& E, uint32_t& mu,
                                            f32x4 (&ub)[NVT]) {
  // no fused multiply-adds the source does not spell out: each instantiation
  // then rounds every element the same way, whatever its schedule
#pragma clang fp contract(off)
  const int wave = x.wave, lane = x.lane, li = x.li, lg = x.lg, tid = x.tid;
  const int64_t row0 = x.bos + (int64_t)c * CH;
  typedef _Float16 half4 __attribute__((ext_vector_type(4)));
  // 0. ub = T diag(b) V_c of token tile w (real units), from the V slice the
  //    previous chunk step put in LDS, so that its magnitude can set the
  //    scale of U_c below.  The narrow slices formed it in the previous
  //    chunk step already (their T diag(b) of chunk c+1 is in registers one
  //    chunk early), between the barriers where it fills MFMA idle cycles.
  if constexpr (NVT != NVT_NARROW) ub_tile<KIND, NVT>(ub, x.sV + (c & 1) * SV_HALFS<NVT>, cur, lane);
  // 1. publish the chunk's vectors, the next chunk's V slice and the current
  //    state, and this wave's largest magnitude of S_c, U_(c-1) and Ub.
  //    Every reader of these buffers in the previous chunk was before its B2
  //    (the other V buffer: before B1 of the previous chunk).
  // (one lane per address: four lanes writing one address stall the LDS)
  if (lane < 16) reinterpret_cast<u32x4*>(x.sVec)[16 * wave + lane] = cur.vec;
  if constexpr (KIND != ST_TRANS) {
    _Float16* const sVn = x.sV + ((c + 1) & 1) * SV_HALFS<NVT>;
#pragma unroll
    for (int i = 0; i < NVT / 2; ++i)
      *reinterpret_cast<u32x4*>(sVn + sv_row<NVT>(tid >> 2) + 32 * i + 8 * (tid & 3)) = n1.vraw[i];
  }
  float ms = 0.0f;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) {
      const half4 hv = {(_Float16)S[j][vt][0], (_Float16)S[j][vt][1], (_Float16)S[j][vt][2], (_Float16)S[j][vt][3]};
      *reinterpret_cast<half4*>(x.sS + (16 * vt + li) * SSS + 32 * wave + 16 * j + 4 * lg) = hv;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) ms = fmaxf(ms, fabsf(S[j][vt][rr]));
    }
  uint32_t mx = max(mu, abs_bits(ms));
  if constexpr (KIND != ST_TRANS) {
    float mb = 0.0f;
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) mb = fmaxf(mb, fabsf(ub[vt][rr]));
    mx = max(mx, abs_bits(mb * pow2f(-E)));
  }
  mx = wave_max_bits(mx);
  if (lane == 0) x.sMx[wave] = mx;
  // 2. the previous chunk's outputs (none before the first chunk: len 0); the
  //    prefetches are issued between the MFMA groups below, a few loads at a
  //    time, so no wave stalls on a full memory queue before a barrier.
  //    Prefetch indices are clamped, so every chunk queues the same operations.
  if constexpr (KIND == ST_FULL) store_pending(pd, x.out, x.Hv, x.h, x.v0, wave, li, lg);
  constexpr int AHEAD = NVT == NVT_NARROW ? 2 : 1;
  ChunkRegs& nt = AHEAD == 2 ? n2 : n1;  // receives the token-tile operands of chunk c + AHEAD
  const int ct = min(c + AHEAD, x.nc - 1);
  const uint8_t* blk_t = x.wsh + (size_t)(x.x0 + ct) * BLOCK;
  __syncthreads();  // B1
  // the scale of the chunk's results: E_(c+1) = E_c + d
  const int d = scale_shift(x.sMx, E);
  const float f = pow2f(-d);
  const int En = E + d;
  // 3. U and O of token tile w for all V tiles, full contractions, in units
  //    of 2^E_(c+1):
  //    U = 2^-E_(c+1) (T diag(b) V) - 2^-d W (S 2^-E_c)^T,
  //    O = 2^-d scale (Q . 2^G) (S 2^-E_c)^T
  const float scn = pow2f(-En), sf = x.scale * f;
  const f32x4 gn0 = *reinterpret_cast<const f32x4*>(x.sVec + 32 * wave + 4 * lg) * f;
  const f32x4 gn1 = *reinterpret_cast<const f32x4*>(x.sVec + 32 * wave + 16 + 4 * lg) * f;
  f32x4 U[NVT], O[NVT], ubn[NVT];
#pragma unroll
  for (int vt = 0; vt < NVT; ++vt) {
    // the next chunk's ub (narrow slices): its V slice went to LDS before B1
    if constexpr (NVT == NVT_NARROW) ub_one<KIND, NVT>(ubn[vt], x.sV + ((c + 1) & 1) * SV_HALFS<NVT>, n1, vt, lane);
    half8 sb[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sb[kb] = *reinterpret_cast<const half8*>(x.sS + (16 * vt + li) * SSS + 32 * kb + 8 * lg);
    f32x4 uw = f32x4{0, 0, 0, 0}, o0 = f32x4{0, 0, 0, 0}, o1 = f32x4{0, 0, 0, 0};
    if constexpr (KIND != ST_TRANS) {
      uw = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.wn[0]), sb[0], uw, 0, 0, 0);
      if constexpr (KIND == ST_FULL) {
        o0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.qg[0]), sb[0], o0, 0, 0, 0);
        o1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.qg[1]), sb[1], o1, 0, 0, 0);
      }
      uw = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.wn[1]), sb[1], uw, 0, 0, 0);
      if constexpr (KIND == ST_FULL) {
        o0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.qg[2]), sb[2], o0, 0, 0, 0);
        o1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.qg[3]), sb[3], o1, 0, 0, 0);
      }
      uw = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.wn[2]), sb[2], uw, 0, 0, 0);
      uw = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.wn[3]), sb[3], uw, 0, 0, 0);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) U[vt][rr] = __builtin_fmaf(ub[vt][rr], scn, uw[rr] * f);
    } else {
      f32x4 uw2 = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int kb = 0; kb < 4; kb += 2) {
        uw = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.wn[kb]), sb[kb], uw, 0, 0, 0);
        uw2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.wn[kb + 1]), sb[kb + 1], uw2, 0, 0, 0);
      }
      U[vt] = (uw + uw2) * f;
    }
    if constexpr (KIND == ST_FULL) O[vt] = (o0 + o1) * sf;
    // 4. the token-tile prefetch: the W and Q fragments after the first V
    //    tile's products, the rest after the second
    if (vt < 2) {
      __builtin_amdgcn_sched_barrier(0);
      if (vt == 0) {
        load_chunk_part<2, KIND, NVT>(nt, blk_t, wave, lane, x.v, 0, 0, x.Hv, x.h, x.v0, tid);
        load_chunk_part<4, KIND, NVT>(nt, blk_t, wave, lane, x.v, 0, 0, x.Hv, x.h, x.v0, tid);
      } else {
        load_chunk_part<3, KIND, NVT>(nt, blk_t, wave, lane, x.v, x.bos + (int64_t)ct * CH, chunk_len(x, ct), x.Hv,
                                      x.h, x.v0, tid);
        if constexpr (KIND != ST_TRANS && NVT != NVT_NARROW) {
          const int cv = min(c + 2, x.nc - 1);
          load_v<NVT>(cur, x.v, x.bos + (int64_t)cv * CH, chunk_len(x, cv), x.Hv, x.h, x.v0, tid);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // 5. U -> LDS hi/lo, transposed [v][t]
  float mu_n = 0.0f;  // this wave's largest |U|
#pragma unroll
  for (int vt = 0; vt < NVT; ++vt) {
    half4 hi, lo;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float up = U[vt][rr];
      const _Float16 hh = (_Float16)up;
      hi[rr] = hh;
      lo[rr] = (_Float16)(up - (float)hh);
      mu_n = fmaxf(mu_n, fabsf(up));
    }
    const int vv = 16 * vt + li, tt = 16 * wave + 4 * lg;
    *reinterpret_cast<half4*>(x.sUh + vv * SUS + tt) = hi;
    *reinterpret_cast<half4*>(x.sUl + vv * SUS + tt) = lo;
  }
  __syncthreads();  // B2
  // 6. S <- S Diag(2^G_last) + U^T Kd ;  O += Aqk U  (Aqk of token tiles 0,
  //    1 is zero in token block 1, so that product adds nothing there)
  half8 kdlo[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int b = 0; b < 2; ++b) kdlo[j][b] = unpack_e4m3(cur.kdl[j][b]);
#pragma unroll
  for (int vt = 0; vt < NVT; ++vt) {
    const half8 uh0 = *reinterpret_cast<const half8*>(x.sUh + (16 * vt + li) * SUS + 8 * lg);
    const half8 uh1 = *reinterpret_cast<const half8*>(x.sUh + (16 * vt + li) * SUS + 32 + 8 * lg);
    const half8 ul0 = *reinterpret_cast<const half8*>(x.sUl + (16 * vt + li) * SUS + 8 * lg);
    const half8 ul1 = *reinterpret_cast<const half8*>(x.sUl + (16 * vt + li) * SUS + 32 + 8 * lg);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // one chain for the fp16 parts, one for the scaled low part of Kd
      f32x4 sa = S[j][vt] * (j == 0 ? gn0 : gn1), sl = f32x4{0, 0, 0, 0};
      sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.kd[j][0]), uh0, sa, 0, 0, 0);
      sl = __builtin_amdgcn_mfma_f32_16x16x32_f16(kdlo[j][0], uh0, sl, 0, 0, 0);
      sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.kd[j][1]), uh1, sa, 0, 0, 0);
      sl = __builtin_amdgcn_mfma_f32_16x16x32_f16(kdlo[j][1], uh1, sl, 0, 0, 0);
      sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.kd[j][0]), ul0, sa, 0, 0, 0);
      sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.kd[j][1]), ul1, sa, 0, 0, 0);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) S[j][vt][rr] = __builtin_fmaf(sl[rr], kKdLoUnscale, sa[rr]);
    }
    if constexpr (KIND == ST_FULL) {
      O[vt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.aq[0]), uh0, O[vt], 0, 0, 0);
      O[vt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.aq[1]), uh1, O[vt], 0, 0, 0);
    }
    // 7. the key-tile prefetch of chunk c+1, after the first V tile's update products
    if (vt == 0) {
      __builtin_amdgcn_sched_barrier(0);
      const int cp = min(c + 1, x.nc - 1);
      load_chunk_part<1, KIND, NVT>(n1, x.wsh + (size_t)(x.x0 + cp) * BLOCK, wave, lane, x.v, 0, 0, x.Hv, x.h, x.v0,
                                    tid);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if constexpr (KIND == ST_FULL) {
    const float se = pow2f(En);
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) pd.o[vt][rr] = __builtin_bit_cast(uint16_t, (__bf16)(O[vt][rr] * se));
    pd.row0 = row0;
    pd.len = chunk_len(x, c);
  }
  E = En;
  mu = abs_bits(mu_n);
  if constexpr (NVT == NVT_NARROW)
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) ub[vt] = ubn[vt];
}

// One workgroup per (job, V slice).  A job is a whole chain (nseg == 1) or one
// segment of it; seg_len chunks per segment (dense input only).
//   ST_FULL  jobs (chain, r), r = 0..nseg-1: entry state h0 (nseg == 1) or
//            S_in[r]; outputs; the final state from the last segment.
//   ST_CARRY jobs (chain, r), r = 0..nseg-2: r = 0 copies h0 to S_in[0] and
//            carries it into S_in[1], r >= 1 carries zero into F[r].
// With segments, h0 is read only by the carry launch and the final state is
// written only by the full launch, so the two may share one buffer.
//   ST_TRANS jobs (chain, r), r = 1..nseg-2: from the identity into P[r];
//            the "V slice" is then a range of key rows.
template <int KIND, int NVT>
__global__ void __launch_bounds__(64 * SWAVES, 1)
kda_state_kernel(const uint16_t* __restrict__ v, const int64_t* __restrict__ cu,
                 const int* __restrict__ chunk_off, const void* __restrict__ h0, void* __restrict__ hT,
                 uint16_t* __restrict__ out, const uint8_t* __restrict__ ws, float* __restrict__ seg,
                 int T, int N, int Hv, int max_chunks, int init_dtype, int final_dtype, int nseg,
                 int seg_len, float scale) {
  __shared__ __attribute__((aligned(16))) float sVec[256];
  __shared__ __attribute__((aligned(16))) uint32_t sMx[SWAVES];
  constexpr int VS = 16 * NVT, NSL = DV / VS;
  __shared__ __attribute__((aligned(16))) _Float16 sS[VS * SSS];
  __shared__ __attribute__((aligned(16))) _Float16 sUh[VS * SUS];
  __shared__ __attribute__((aligned(16))) _Float16 sUl[VS * SUS];
  __shared__ __attribute__((aligned(16))) _Float16 sV[2 * SV_HALFS<NVT>];

  // XCD-aware decode: the NSL slices of one job share (id mod 8), so they
  // are dispatched to the same XCD and share its L2 for the job's operands.
  const int jpc = KIND == ST_FULL ? nseg : KIND == ST_CARRY ? nseg - 1 : nseg - 2;  // jobs per chain
  const int chains = N * Hv;
  const int id = blockIdx.x;
  const int job = (id / (8 * NSL)) * 8 + (id & 7);
  const int slice = (id >> 3) % NSL;
  if (job >= chains * jpc) return;
  const int chain = job / jpc, r = job % jpc + (KIND == ST_TRANS ? 1 : 0);
  const int n = chain / Hv, h = chain % Hv;
  const int v0 = VS * slice;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;

  int64_t bos, seqlen;
  int x0, nc;
  if (cu == nullptr) {
    const int ncs = (T + CH - 1) / CH;
    const int cs = r * seg_len;
    bos = (int64_t)n * T + (int64_t)cs * CH; seqlen = (int64_t)T - (int64_t)cs * CH;
    x0 = n * ncs + cs; nc = max(0, min(seg_len, ncs - cs));
  } else {
    bos = cu[n]; seqlen = cu[n + 1] - cu[n];
    x0 = chunk_off[n]; nc = chunk_off[n + 1] - x0;
  }

  // entry state: tiles S^T[k][v]: k = 32 wave + 16 j + 4 lg + rr, v = v0 + 16 vt + li
  const void* src = nullptr;
  int src_dtype = KDA_STATE_NONE;
  size_t src_base = 0;
  if ((KIND == ST_CARRY && r == 0) || (KIND == ST_FULL && nseg == 1)) {
    src = h0; src_dtype = init_dtype; src_base = ((size_t)n * Hv + h) * DV * DK;
  } else if (KIND == ST_FULL) {
    src = seg_mat(seg, chains, nseg, SEG_SIN, chain, r); src_dtype = KDA_STATE_F32;
  }
  f32x4 S[2][NVT];
  if constexpr (KIND != ST_TRANS) load_entry_tiles<NVT>(S, src, src_dtype, src_base, wave, v0, li, lg);
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) {
      const int kk = 32 * wave + 16 * j + 4 * lg, vv = v0 + 16 * vt + li;
      if constexpr (KIND == ST_TRANS) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) S[j][vt][rr] = kk + rr == vv ? 1.0f : 0.0f;
      }
      if (KIND == ST_CARRY && r == 0)
        *reinterpret_cast<f32x4*>(seg_mat(seg, chains, nseg, SEG_SIN, chain, 0) + (size_t)vv * DK + kk) = S[j][vt];
    }

  const uint8_t* wsh = ws + (size_t)h * max_chunks * BLOCK;
  StateCtx ctx{v, out, wsh, bos, seqlen, x0, nc, Hv, h, v0, tid, wave, lane, li, lg, scale, sMx, sVec, sS, sUh, sUl, sV};
  ChunkRegs rA, rB, rC;
  if (nc > 0) {
    load_chunk_part<0, KIND, NVT>(rA, wsh + (size_t)x0 * BLOCK, wave, lane, v, bos, chunk_len(ctx, 0), Hv, h, v0,
                                  tid);
    load_chunk_part<1, KIND, NVT>(rA, wsh + (size_t)x0 * BLOCK, wave, lane, v, 0, 0, Hv, h, v0, tid);
  }
  if (nc > 0 && NVT == NVT_NARROW) {
    const int c1 = min(1, nc - 1);
    load_chunk_part<0, KIND, NVT>(rB, wsh + (size_t)(x0 + c1) * BLOCK, wave, lane, v, bos + (int64_t)c1 * CH,
                             chunk_len(ctx, c1), Hv, h, v0, tid);
  }
  if (KIND != ST_TRANS && nc > 0 && NVT != NVT_NARROW) {
    // wide slices: V runs two chunks ahead on its own
    const int c1 = min(1, nc - 1);
    load_v<NVT>(rA, v, bos, chunk_len(ctx, 0), Hv, h, v0, tid);
    load_v<NVT>(rB, v, bos + (int64_t)c1 * CH, chunk_len(ctx, c1), Hv, h, v0, tid);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) settle(S[j][vt]);
  settle<KIND, NVT>(rA);
  // the first chunk's V slice into V buffer 0 (visible after the barrier below)
  if (KIND != ST_TRANS && nc > 0)
#pragma unroll
    for (int i = 0; i < NVT / 2; ++i)
      *reinterpret_cast<u32x4*>(sV + sv_row<NVT>(tid >> 2) + 32 * i + 8 * (tid & 3)) = rA.vraw[i];
  // the entry scale: the largest magnitude of the entry state and the first
  // chunk's V brought into [1, 2)
  int E = 0;
  if (nc > 0) {
    uint32_t mx = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) mx = max(mx, abs_bits(S[j][vt][rr]));
    if constexpr (KIND != ST_TRANS)
#pragma unroll
      for (int i = 0; i < NVT / 2; ++i) mx = max(mx, bf16x8_absmax_bits(rA.vraw[i]));
    mx = wave_max_bits(mx);
    if (lane == 0) sMx[wave] = mx;
    __syncthreads();
    const int mi = __builtin_amdgcn_readfirstlane((int)max(max(sMx[0], sMx[1]), max(sMx[2], sMx[3])));
    E = mi == 0 ? 0 : min(max(ilog2_bits(mi), -kMaxExp), kMaxExp);
    // every wave has read the entry maxima before any wave posts again
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) S[j][vt][rr] = __builtin_amdgcn_ldexpf(S[j][vt][rr], -E);
  }
  __syncthreads();
  // the first chunk's ub (the narrow slices carry it from one chunk step to the next)
  f32x4 ub[NVT];
  if (NVT == NVT_NARROW && nc > 0) ub_tile<KIND, NVT>(ub, sV, rA, lane);
  uint32_t mu = 0;  // no U before the first chunk
  PendingOut<NVT> pd;
  pd.row0 = bos;
  pd.len = 0;
  int c = 0;
  if constexpr (NVT == NVT_NARROW) {
    for (; c + 3 <= nc; c += 3) {
      state_chunk<KIND, NVT>(ctx, S, rA, rB, rC, c, pd, E, mu, ub);
      state_chunk<KIND, NVT>(ctx, S, rB, rC, rA, c + 1, pd, E, mu, ub);
      state_chunk<KIND, NVT>(ctx, S, rC, rA, rB, c + 2, pd, E, mu, ub);
    }
    if (c < nc) state_chunk<KIND, NVT>(ctx, S, rA, rB, rC, c, pd, E, mu, ub);
    if (c + 1 < nc) state_chunk<KIND, NVT>(ctx, S, rB, rC, rA, c + 1, pd, E, mu, ub);
  } else {
    for (; c + 2 <= nc; c += 2) {
      state_chunk<KIND, NVT>(ctx, S, rA, rB, rB, c, pd, E, mu, ub);
      state_chunk<KIND, NVT>(ctx, S, rB, rA, rA, c + 1, pd, E, mu, ub);
    }
    if (c < nc) state_chunk<KIND, NVT>(ctx, S, rA, rB, rB, c, pd, E, mu, ub);
  }
  if constexpr (KIND == ST_FULL) store_pending(pd, out, Hv, h, v0, wave, li, lg);
  // back to the state's own units
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) S[j][vt][rr] = __builtin_amdgcn_ldexpf(S[j][vt][rr], E);

  // exit state
  void* dst = nullptr;
  int dst_dtype = KDA_STATE_NONE;
  size_t dst_base = 0;
  if constexpr (KIND == ST_FULL) {
    if (r == nseg - 1) { dst = hT; dst_dtype = final_dtype; dst_base = ((size_t)n * Hv + h) * DV * DK; }
  } else {
    dst = KIND == ST_TRANS ? seg_mat(seg, chains, nseg, SEG_P, chain, r)
          : r == 0         ? seg_mat(seg, chains, nseg, SEG_SIN, chain, 1)
                           : seg_mat(seg, chains, nseg, SEG_F, chain, r);
    dst_dtype = KDA_STATE_F32;
  }
  if (dst_dtype != KDA_STATE_NONE) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        const int kk = 32 * wave + 16 * j + 4 * lg, vv = v0 + 16 * vt + li;
        if (dst_dtype == KDA_STATE_F32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(dst) + dst_base + (size_t)vv * DK + kk) = S[j][vt];
        } else {
          uint2 u;
          u.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)S[j][vt][0]) |
                ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)S[j][vt][1]) << 16);
          u.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)S[j][vt][2]) |
                ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)S[j][vt][3]) << 16);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(dst) + dst_base + (size_t)vv * DK + kk) = u;
        }
      }
  }
}

// ---------------------------------------------------------------------------
// The same chain on 32-column slices for full outputs (ST_FULL) or the state
// alone (ST_CARRY), with each chunk step split over two roles of four waves,
// two waves per SIMD:
//   chain waves (0..3), wave w: the recurrence itself -- S_c to LDS, U of
//     token tile w = 2^-E_(c+1) Ub - 2^-d W (S 2^-E_c)^T to LDS, then its key
//     rows of S <- S Diag(2^G_last) + U^T Kd; operands W, the vectors, Kd;
//   helper waves (4..7), wave 4 + w: everything off that path for token tile
//     w -- Ub = T diag(b) V of the next chunk and (ST_FULL) O = scale
//     (Q . 2^G) S^T + Aqk U, its bf16 rounding and stores; operands
//     T diag(b), V and (ST_FULL) Q . 2^G, Aqk.
// With one wave per SIMD the step's serial instruction stream was the bound:
// here the helper issues while the chain wave waits on an MFMA result, an LDS
// read or a barrier.  The barriers, LDS buffers and scale rule are those of
// kda_state_kernel (the helper posts the largest |Ub|, the chain wave those
// of S and U, and the scale takes the largest of the eight), and every
// product and rounding is the same, so the results are bit-identical to it.
// Each role runs its own loop over the chunks, so the registers of the one
// role's operands are free for the other's.
constexpr int SPWAVES = 8;

// the scale shift from the eight posted maxima (chain waves 0..3, helpers 4..7)
__device__ __forceinline__ int scale_shift8(const uint32_t* sMx, int E) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(sMx), b = *reinterpret_cast<const u32x4*>(sMx + 4);
  const int mi = __builtin_amdgcn_readfirstlane(
      (int)max(max(max(a[0], a[1]), max(a[2], a[3])), max(max(b[0], b[1]), max(b[2], b[3]))));
  if (mi == 0) return 0;
  const int d = min(max(ilog2_bits(mi), -kMaxStep), kMaxStep);
  return min(max(E + d, -kMaxExp), kMaxExp) - E;
}

// chain wave, chunk c: `cur` holds W, the vectors and Kd of chunk c, `n1`
// receives Kd of chunk c+1, `n2` W and the vectors of chunk c+2.  On entry S
// holds S_c in units of 2^E and mu this wave's largest |U_(c-1)|.
template <int KIND>
__device__ __forceinline__ void chain_step(const StateCtx& x, f32x4 (&S)[2][NVT_NARROW], ChunkRegs& cur,
                                           ChunkRegs& n1, ChunkRegs& n2, const int c, int& E, uint32_t& mu,
                                           const f32x4* sUb) {
#pragma clang fp contract(off)
  constexpr int NVT = NVT_NARROW;
  const int wave = x.wave, lane = x.lane, li = x.li, lg = x.lg, tid = x.tid;
  typedef _Float16 half4 __attribute__((ext_vector_type(4)));
  if (lane < 16) reinterpret_cast<u32x4*>(x.sVec)[16 * wave + lane] = cur.vec;
  float ms = 0.0f;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) {
      const half4 hv = {(_Float16)S[j][vt][0], (_Float16)S[j][vt][1], (_Float16)S[j][vt][2], (_Float16)S[j][vt][3]};
      *reinterpret_cast<half4*>(x.sS + (16 * vt + li) * SSS + 32 * wave + 16 * j + 4 * lg) = hv;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) ms = fmaxf(ms, fabsf(S[j][vt][rr]));
    }
  uint32_t mx = wave_max_bits(max(mu, abs_bits(ms)));
  if (lane == 0) x.sMx[wave] = mx;
  const int ct = min(c + 2, x.nc - 1);
  const uint8_t* blk_t = x.wsh + (size_t)(x.x0 + ct) * BLOCK;
  __syncthreads();  // B1
  const int d = scale_shift8(x.sMx, E);
  const float f = pow2f(-d);
  const int En = E + d;
  const float scn = pow2f(-En);
  const f32x4 gn0 = *reinterpret_cast<const f32x4*>(x.sVec + 32 * wave + 4 * lg) * f;
  const f32x4 gn1 = *reinterpret_cast<const f32x4*>(x.sVec + 32 * wave + 16 + 4 * lg) * f;
  f32x4 U[NVT];
#pragma unroll
  for (int vt = 0; vt < NVT; ++vt) {
    const f32x4 ub = sUb[(wave * NVT + vt) * 64 + lane];
    half8 sb[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sb[kb] = *reinterpret_cast<const half8*>(x.sS + (16 * vt + li) * SSS + 32 * kb + 8 * lg);
    f32x4 uw = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) uw = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.wn[kb]), sb[kb], uw, 0, 0, 0);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) U[vt][rr] = __builtin_fmaf(ub[rr], scn, uw[rr] * f);
    __builtin_amdgcn_sched_barrier(0);
    if (vt == 0) load_chunk_part<2, KIND, NVT>(n2, blk_t, wave, lane, x.v, 0, 0, x.Hv, x.h, x.v0, tid);
    else load_chunk_part<5, KIND, NVT>(n2, blk_t, wave, lane, x.v, 0, 0, x.Hv, x.h, x.v0, tid);
    __builtin_amdgcn_sched_barrier(0);
  }
  float mu_n = 0.0f;
#pragma unroll
  for (int vt = 0; vt < NVT; ++vt) {
    half4 hi, lo;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float up = U[vt][rr];
      const _Float16 hh = (_Float16)up;
      hi[rr] = hh;
      lo[rr] = (_Float16)(up - (float)hh);
      mu_n = fmaxf(mu_n, fabsf(up));
    }
    const int vv = 16 * vt + li, tt = 16 * wave + 4 * lg;
    *reinterpret_cast<half4*>(x.sUh + vv * SUS + tt) = hi;
    *reinterpret_cast<half4*>(x.sUl + vv * SUS + tt) = lo;
  }
  __syncthreads();  // B2
  half8 kdlo[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int b = 0; b < 2; ++b) kdlo[j][b] = unpack_e4m3(cur.kdl[j][b]);
#pragma unroll
  for (int vt = 0; vt < NVT; ++vt) {
    const half8 uh0 = *reinterpret_cast<const half8*>(x.sUh + (16 * vt + li) * SUS + 8 * lg);
    const half8 uh1 = *reinterpret_cast<const half8*>(x.sUh + (16 * vt + li) * SUS + 32 + 8 * lg);
    const half8 ul0 = *reinterpret_cast<const half8*>(x.sUl + (16 * vt + li) * SUS + 8 * lg);
    const half8 ul1 = *reinterpret_cast<const half8*>(x.sUl + (16 * vt + li) * SUS + 32 + 8 * lg);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f32x4 sa = S[j][vt] * (j == 0 ? gn0 : gn1), sl = f32x4{0, 0, 0, 0};
      sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.kd[j][0]), uh0, sa, 0, 0, 0);
      sl = __builtin_amdgcn_mfma_f32_16x16x32_f16(kdlo[j][0], uh0, sl, 0, 0, 0);
      sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.kd[j][1]), uh1, sa, 0, 0, 0);
      sl = __builtin_amdgcn_mfma_f32_16x16x32_f16(kdlo[j][1], uh1, sl, 0, 0, 0);
      sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.kd[j][0]), ul0, sa, 0, 0, 0);
      sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.kd[j][1]), ul1, sa, 0, 0, 0);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) S[j][vt][rr] = __builtin_fmaf(sl[rr], kKdLoUnscale, sa[rr]);
    }
    if (vt == 0) {
      __builtin_amdgcn_sched_barrier(0);
      const int cp = min(c + 1, x.nc - 1);
      load_chunk_part<1, KIND, NVT>(n1, x.wsh + (size_t)(x.x0 + cp) * BLOCK, wave, lane, x.v, 0, 0, x.Hv, x.h,
                                       x.v0, tid);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  E = En;
  mu = abs_bits(mu_n);
}

// helper wave, chunk c: `cur` holds Q . 2^G and Aqk of chunk c (ST_FULL; its
// V is in LDS already, and the register set receives V of chunk c+3), `n1`
// holds T diag(b) and V of chunk c+1, `n2` receives the helper operands of
// chunk c+2.  On entry ub holds T diag(b) V_c of token tile w (real units); the
// outputs of chunk c-1 are in pd.  V of chunk c+1 goes to LDS between the
// barriers and T diag(b) V_(c+1) is formed after the second: so those
// operands are consumed a step and a half after their loads are issued (loads
// complete in order, so a wait for a young load waits for all the older ones).
template <int KIND>
__device__ __forceinline__ void helper_step(const StateCtx& x, ChunkRegs& cur, ChunkRegs& n1, ChunkRegs& n2,
                                            const int c, PendingOut<NVT_NARROW>& pd, int& E,
                                            f32x4 (&ub)[NVT_NARROW], f32x4* sUb) {
#pragma clang fp contract(off)
  constexpr int NVT = NVT_NARROW;
  const int wave = x.wave, lane = x.lane, li = x.li, lg = x.lg, tid = x.tid;
  const int64_t row0 = x.bos + (int64_t)c * CH;
  // this chunk's Ub for the chain waves, and its magnitude
  float mb = 0.0f;
#pragma unroll
  for (int vt = 0; vt < NVT; ++vt) {
    sUb[(wave * NVT + vt) * 64 + lane] = ub[vt];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) mb = fmaxf(mb, fabsf(ub[vt][rr]));
  }
  const uint32_t mx = wave_max_bits(abs_bits(mb * pow2f(-E)));
  if (lane == 0) x.sMx[SWAVES + wave] = mx;
  if constexpr (KIND == ST_FULL) store_pending(pd, x.out, x.Hv, x.h, x.v0, wave, li, lg);
  const int ct = min(c + 2, x.nc - 1), cv = min(c + 3, x.nc - 1);
  const uint8_t* blk_t = x.wsh + (size_t)(x.x0 + ct) * BLOCK;
  __syncthreads();  // B1
  const int d = scale_shift8(x.sMx, E);
  const int En = E + d;
  const float sf = x.scale * pow2f(-d);
  f32x4 O[NVT];
#pragma unroll
  for (int vt = 0; vt < NVT; ++vt) {
    if constexpr (KIND == ST_FULL) {
      half8 sb[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        sb[kb] = *reinterpret_cast<const half8*>(x.sS + (16 * vt + li) * SSS + 32 * kb + 8 * lg);
      f32x4 o0 = f32x4{0, 0, 0, 0}, o1 = f32x4{0, 0, 0, 0};
      o0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.qg[0]), sb[0], o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.qg[1]), sb[1], o1, 0, 0, 0);
      o0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.qg[2]), sb[2], o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.qg[3]), sb[3], o1, 0, 0, 0);
      O[vt] = (o0 + o1) * sf;
    }
    __builtin_amdgcn_sched_barrier(0);
    if (vt == 0) {
      load_chunk_part<4, KIND, NVT>(n2, blk_t, wave, lane, x.v, 0, 0, x.Hv, x.h, x.v0, tid);
    } else {
      load_chunk_part<7, KIND, NVT>(n2, blk_t, wave, lane, x.v, 0, 0, x.Hv, x.h, x.v0, tid);
      load_v<NVT>(cur, x.v, x.bos + (int64_t)cv * CH, chunk_len(x, cv), x.Hv, x.h, x.v0, tid);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // V of chunk c+1 into the V buffer of its parity (last read before B2 of
  // the previous chunk step but one)
  _Float16* const sVn = x.sV + ((c + 1) & 1) * SV_HALFS<NVT>;
  *reinterpret_cast<u32x4*>(sVn + sv_row<NVT>(tid >> 2) + 8 * (tid & 3)) = n1.vraw[0];
  __syncthreads();  // B2
  if constexpr (KIND == ST_FULL) {
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) {
      const half8 uh0 = *reinterpret_cast<const half8*>(x.sUh + (16 * vt + li) * SUS + 8 * lg);
      const half8 uh1 = *reinterpret_cast<const half8*>(x.sUh + (16 * vt + li) * SUS + 32 + 8 * lg);
      O[vt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.aq[0]), uh0, O[vt], 0, 0, 0);
      O[vt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(cur.aq[1]), uh1, O[vt], 0, 0, 0);
    }
    const float se = pow2f(En);
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) pd.o[vt][rr] = __builtin_bit_cast(uint16_t, (__bf16)(O[vt][rr] * se));
    pd.row0 = row0;
    pd.len = chunk_len(x, c);
  }
  E = En;
  // the next chunk's Ub
#pragma unroll
  for (int vt = 0; vt < NVT; ++vt) ub_one<KIND, NVT>(ub[vt], sVn, n1, vt, lane);
}

// One workgroup of 8 waves per (job, 32-column V slice); jobs, their entry
// and exit states and the XCD-aware decode as in kda_state_kernel.
template <int KIND>
__global__ void __launch_bounds__(64 * SPWAVES, 1)
kda_state_split_kernel(const uint16_t* __restrict__ v, const int64_t* __restrict__ cu,
                       const int* __restrict__ chunk_off, const void* __restrict__ h0, void* __restrict__ hT,
                       uint16_t* __restrict__ out, const uint8_t* __restrict__ ws, float* __restrict__ seg,
                       int T, int N, int Hv, int max_chunks, int init_dtype, int final_dtype, int nseg,
                       int seg_len, float scale) {
  constexpr int NVT = NVT_NARROW;
  __shared__ __attribute__((aligned(16))) float sVec[256];
  __shared__ __attribute__((aligned(16))) uint32_t sMx[SPWAVES];
  constexpr int VS = 16 * NVT, NSL = DV / VS;
  __shared__ __attribute__((aligned(16))) _Float16 sS[VS * SSS];
  __shared__ __attribute__((aligned(16))) _Float16 sUh[VS * SUS];
  __shared__ __attribute__((aligned(16))) _Float16 sUl[VS * SUS];
  __shared__ __attribute__((aligned(16))) _Float16 sV[2 * SV_HALFS<NVT>];
  __shared__ __attribute__((aligned(16))) f32x4 sUb[SWAVES * NVT * 64];  // Ub of each token tile, lane order

  static_assert(KIND == ST_FULL || KIND == ST_CARRY, "the split kernel runs full and carry jobs");
  const int jpc = KIND == ST_FULL ? nseg : nseg - 1;  // jobs per chain
  const int chains = N * Hv;
  const int id = blockIdx.x;
  const int job = (id / (8 * NSL)) * 8 + (id & 7);
  const int slice = (id >> 3) % NSL;
  if (job >= chains * jpc) return;
  const int chain = job / jpc, r = job % jpc;
  const int n = chain / Hv, h = chain % Hv;
  const int v0 = VS * slice;
  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const bool helper = wv >= SWAVES;
  // the role's own wave index and thread index (0..255)
  const int wave = helper ? wv - SWAVES : wv, tid = (int)threadIdx.x & (64 * SWAVES - 1), lane = tid & 63;
  const int li = lane & 15, lg = lane >> 4;

  int64_t bos, seqlen;
  int x0, nc;
  if (cu == nullptr) {
    const int ncs = (T + CH - 1) / CH;
    const int cs = r * seg_len;
    bos = (int64_t)n * T + (int64_t)cs * CH; seqlen = (int64_t)T - (int64_t)cs * CH;
    x0 = n * ncs + cs; nc = max(0, min(seg_len, ncs - cs));
  } else {
    bos = cu[n]; seqlen = cu[n + 1] - cu[n];
    x0 = chunk_off[n]; nc = chunk_off[n + 1] - x0;
  }
  const uint8_t* wsh = ws + (size_t)h * max_chunks * BLOCK;
  StateCtx ctx{v, out, wsh, bos, seqlen, x0, nc, Hv, h, v0, tid, wave, lane, li, lg, scale, sMx, sVec, sS, sUh, sUl, sV};

  if (!helper) {
    // entry state: tiles S^T[k][v]: k = 32 wave + 16 j + 4 lg + rr, v = v0 + 16 vt + li
    const void* src = nullptr;
    int src_dtype = KDA_STATE_NONE;
    size_t src_base = 0;
    if ((KIND == ST_CARRY && r == 0) || (KIND == ST_FULL && nseg == 1)) {
      src = h0; src_dtype = init_dtype; src_base = ((size_t)n * Hv + h) * DV * DK;
    } else if (KIND == ST_FULL) {
      src = seg_mat(seg, chains, nseg, SEG_SIN, chain, r); src_dtype = KDA_STATE_F32;
    }
    f32x4 S[2][NVT];
    load_entry_tiles<NVT>(S, src, src_dtype, src_base, wave, v0, li, lg);
    if (KIND == ST_CARRY && r == 0)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) {
          const int kk = 32 * wave + 16 * j + 4 * lg, vv = v0 + 16 * vt + li;
          *reinterpret_cast<f32x4*>(seg_mat(seg, chains, nseg, SEG_SIN, chain, 0) + (size_t)vv * DK + kk) = S[j][vt];
        }
    ChunkRegs rA, rB, rC;
    if (nc > 0) {
      const uint8_t* b0 = wsh + (size_t)x0 * BLOCK;
      load_chunk_part<2, KIND, NVT>(rA, b0, wave, lane, v, 0, 0, Hv, h, v0, tid);
      load_chunk_part<5, KIND, NVT>(rA, b0, wave, lane, v, 0, 0, Hv, h, v0, tid);
      load_chunk_part<1, KIND, NVT>(rA, b0, wave, lane, v, 0, 0, Hv, h, v0, tid);
      const uint8_t* b1 = wsh + (size_t)(x0 + min(1, nc - 1)) * BLOCK;
      load_chunk_part<2, KIND, NVT>(rB, b1, wave, lane, v, 0, 0, Hv, h, v0, tid);
      load_chunk_part<5, KIND, NVT>(rB, b1, wave, lane, v, 0, 0, Hv, h, v0, tid);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) settle(S[j][vt]);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) settle(rA.wn[kb]);
    settle(rA.vec);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int b = 0; b < 2; ++b) { settle(rA.kd[j][b]); settle(rA.kdl[j][b]); }
    // the entry scale: the largest magnitude of the entry state (chain waves)
    // and of the first chunk's V (helpers) brought into [1, 2)
    int E = 0;
    if (nc > 0) {
      uint32_t mx = 0;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) mx = max(mx, abs_bits(S[j][vt][rr]));
      mx = wave_max_bits(mx);
      if (lane == 0) sMx[wave] = mx;
      __syncthreads();
      const u32x4 a = *reinterpret_cast<const u32x4*>(sMx), b = *reinterpret_cast<const u32x4*>(sMx + 4);
      const int mi = __builtin_amdgcn_readfirstlane(
          (int)max(max(max(a[0], a[1]), max(a[2], a[3])), max(max(b[0], b[1]), max(b[2], b[3]))));
      E = mi == 0 ? 0 : min(max(ilog2_bits(mi), -kMaxExp), kMaxExp);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) S[j][vt][rr] = __builtin_amdgcn_ldexpf(S[j][vt][rr], -E);
    }
    __syncthreads();  // every wave has read the entry maxima before any posts again
    uint32_t mu = 0;
    int c = 0;
    for (; c + 3 <= nc; c += 3) {
      chain_step<KIND>(ctx, S, rA, rB, rC, c, E, mu, sUb);
      chain_step<KIND>(ctx, S, rB, rC, rA, c + 1, E, mu, sUb);
      chain_step<KIND>(ctx, S, rC, rA, rB, c + 2, E, mu, sUb);
    }
    if (c < nc) chain_step<KIND>(ctx, S, rA, rB, rC, c, E, mu, sUb);
    if (c + 1 < nc) chain_step<KIND>(ctx, S, rB, rC, rA, c + 1, E, mu, sUb);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) S[j][vt][rr] = __builtin_amdgcn_ldexpf(S[j][vt][rr], E);
    // exit state: the chain's final state from the last full job; a carry
    // job's state into the segment scratch
    void* dst = nullptr;
    int dst_dtype = KDA_STATE_NONE;
    size_t dst_base = 0;
    if constexpr (KIND == ST_FULL) {
      if (r == nseg - 1) { dst = hT; dst_dtype = final_dtype; dst_base = ((size_t)n * Hv + h) * DV * DK; }
    } else {
      dst = r == 0 ? seg_mat(seg, chains, nseg, SEG_SIN, chain, 1) : seg_mat(seg, chains, nseg, SEG_F, chain, r);
      dst_dtype = KDA_STATE_F32;
    }
    if (dst_dtype != KDA_STATE_NONE) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) {
          const int kk = 32 * wave + 16 * j + 4 * lg, vv = v0 + 16 * vt + li;
          if (dst_dtype == KDA_STATE_F32) {
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(dst) + dst_base + (size_t)vv * DK + kk) = S[j][vt];
          } else {
            uint2 u;
            u.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)S[j][vt][0]) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)S[j][vt][1]) << 16);
            u.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)S[j][vt][2]) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)S[j][vt][3]) << 16);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(dst) + dst_base + (size_t)vv * DK + kk) = u;
          }
        }
    }
  } else {
    ChunkRegs rA, rB, rC;
    if (nc > 0) {
      const uint8_t* b0 = wsh + (size_t)x0 * BLOCK;
      load_chunk_part<4, KIND, NVT>(rA, b0, wave, lane, v, 0, 0, Hv, h, v0, tid);
      load_chunk_part<6, KIND, NVT>(rA, b0, wave, lane, v, bos, chunk_len(ctx, 0), Hv, h, v0, tid);
      const int c1 = min(1, nc - 1), c2 = min(2, nc - 1);
      const uint8_t* b1 = wsh + (size_t)(x0 + c1) * BLOCK;
      load_chunk_part<4, KIND, NVT>(rB, b1, wave, lane, v, 0, 0, Hv, h, v0, tid);
      load_chunk_part<6, KIND, NVT>(rB, b1, wave, lane, v, bos + (int64_t)c1 * CH, chunk_len(ctx, c1), Hv, h, v0,
                                    tid);
      // V runs three chunks ahead: chunk 2's goes to the third register set now
      load_v<NVT>(rC, v, bos + (int64_t)c2 * CH, chunk_len(ctx, c2), Hv, h, v0, tid);
    }
    if constexpr (KIND == ST_FULL)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) settle(rA.qg[kb]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      settle(rA.tbh[kb]);
      settle(rA.tbl[kb]);
      if constexpr (KIND == ST_FULL) settle(rA.aq[kb]);
    }
    settle(rA.vraw[0]);
    // the first chunk's V slice into V buffer 0 (visible after the barrier below)
    if (nc > 0) *reinterpret_cast<u32x4*>(sV + sv_row<NVT>(tid >> 2) + 8 * (tid & 3)) = rA.vraw[0];
    int E = 0;
    if (nc > 0) {
      const uint32_t mx = wave_max_bits(bf16x8_absmax_bits(rA.vraw[0]));
      if (lane == 0) sMx[SWAVES + wave] = mx;
      __syncthreads();
      const u32x4 a = *reinterpret_cast<const u32x4*>(sMx), b = *reinterpret_cast<const u32x4*>(sMx + 4);
      const int mi = __builtin_amdgcn_readfirstlane(
          (int)max(max(max(a[0], a[1]), max(a[2], a[3])), max(max(b[0], b[1]), max(b[2], b[3]))));
      E = mi == 0 ? 0 : min(max(ilog2_bits(mi), -kMaxExp), kMaxExp);
    }
    __syncthreads();
    f32x4 ub[NVT];
    if (nc > 0) ub_tile<KIND, NVT>(ub, sV, rA, lane);
    PendingOut<NVT> pd;
    pd.row0 = bos;
    pd.len = 0;
    int c = 0;
    for (; c + 3 <= nc; c += 3) {
      helper_step<KIND>(ctx, rA, rB, rC, c, pd, E, ub, sUb);
      helper_step<KIND>(ctx, rB, rC, rA, c + 1, pd, E, ub, sUb);
      helper_step<KIND>(ctx, rC, rA, rB, c + 2, pd, E, ub, sUb);
    }
    if (c < nc) helper_step<KIND>(ctx, rA, rB, rC, c, pd, E, ub, sUb);
    if (c + 1 < nc) helper_step<KIND>(ctx, rB, rC, rA, c + 1, pd, E, ub, sUb);
    if constexpr (KIND == ST_FULL) store_pending(pd, out, Hv, h, v0, wave, li, lg);
  }
}

// ---------------------------------------------------------------------------
// token-recurrent forward (decode and short sequences)
//
// One workgroup of 256 threads per (sequence, v-head, 32-row V slice): thread
// t owns state row v0 + (t >> 3) and the key columns 32 m + 4 (t & 7) + i
// (m, i = 0..3), as 16 fp32 values in registers, so that each 16-byte load or
// store instruction of a wave covers whole 128-byte row segments.  Tokens go
// in blocks of RTB.  The inputs of a block are fetched into registers one
// block ahead; wave w then prepares tokens w, w + 4, ... of the block (lane l
// holds channels 2l, 2l + 1, so a token's norms are one wave reduction) and
// writes scale q/|q|, k/|k| and the per-channel decay factor exp(a) to a
// double-buffered LDS slot.  After one barrier the tokens of the block run
// with no further barrier -- every state row is independent: decay its
// columns, r = S k (an 8-lane reduction), the delta write, o = S q.
constexpr int RSLICE = 32;                 // V rows per workgroup
constexpr int RNSLICE = DV / RSLICE;
// Tokens per block: RTB for sequences, 1 for decode steps (one token each).
constexpr int RTB = 8;

template <int TB>
struct RecurrentIn {
  static constexpr int TPW = (TB + 3) / 4;  // tokens per wave
  uint32_t q[TPW], k[TPW], g[TPW];          // bf16 pairs: token wave + 4 i, channels 2 lane, 2 lane + 1
  float vv;                                 // v: token tid >> 5, row tid & 31
  float braw;                               // beta of token tid (tid < TB)
};

// Issue the loads of the block starting at token s0 (tokens >= len read
// nothing; the conditions are uniform per wave).
template <int TB>
__device__ __forceinline__ void recurrent_load(RecurrentIn<TB>& in, int64_t s0, int64_t len, int64_t bos,
                                               const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                               const uint16_t* g, const uint16_t* beta, int Hqk, int Hv, int h,
                                               int hq, int v0, int tid, int wave) {
  const int c = 2 * (tid & 63);
#pragma unroll
  for (int i = 0; i < RecurrentIn<TB>::TPW; ++i) {
    const int tk = wave + 4 * i;
    in.q[i] = in.k[i] = in.g[i] = 0u;
    if (tk < TB && s0 + tk < len) {
      const size_t tok = (size_t)(bos + s0 + tk);
      in.q[i] = *reinterpret_cast<const uint32_t*>(q + (tok * Hqk + hq) * DK + c);
      in.k[i] = *reinterpret_cast<const uint32_t*>(k + (tok * Hqk + hq) * DK + c);
      in.g[i] = *reinterpret_cast<const uint32_t*>(g + (tok * Hv + h) * DK + c);
    }
  }
  in.vv = 0.0f;
  if ((tid >> 5) < TB && s0 + (tid >> 5) < len)
    in.vv = bf2f(v[((size_t)(bos + s0 + (tid >> 5)) * Hv + h) * DV + v0 + (tid & 31)]);
  in.braw = 0.0f;
  if (tid < TB && s0 + tid < len) in.braw = bf2f(beta[(size_t)(bos + s0 + tid) * Hv + h]);
}

// Sums by DPP moves within a 16-lane row (no LDS permute round trips): lanes
// paired by quad_perm [1,0,3,2] and [2,3,0,1], then the 4-lane halves of each
// 8 by row_half_mirror, then the 8-lane halves of the row by row_mirror.
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
// Sum over the 64 lanes of a wave, in a fixed order: row sums, then rows 0..3.
__device__ __forceinline__ float sum64(float x) {
  x = sum8(x);
  x += dpp_f<0x140>(x);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
  return ((r0 + r1) + r2) + r3;
}

template <int MODE, int TB>
__global__ void __launch_bounds__(256)
kda_recurrent_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                     const uint16_t* __restrict__ v, const uint16_t* __restrict__ g,
                     const uint16_t* __restrict__ beta, const float* __restrict__ A_log,
                     const float* __restrict__ dt_bias, const int64_t* __restrict__ cu,
                     const void* h0, void* hT, uint16_t* __restrict__ out,
                     int T, int N, int Hqk, int Hv, float scale, float lower_bound, int flags,
                     int init_dtype, int final_dtype) {
  __shared__ __attribute__((aligned(16))) float sK[2][TB][DK];
  __shared__ __attribute__((aligned(16))) float sQ[2][TB][DK];
  __shared__ __attribute__((aligned(16))) float sD[2][TB][DK];
  __shared__ __attribute__((aligned(16))) float sVv[2][TB][RSLICE];
  __shared__ float sB[2][TB];

  const int chain = blockIdx.x / RNSLICE, slice = blockIdx.x % RNSLICE;
  if (chain >= N * Hv) return;
  const int n = chain / Hv, h = chain % Hv, hq = h / (Hv / Hqk);
  const int v0 = RSLICE * slice;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = tid >> 3, kc = 4 * (tid & 7);
  int64_t bos, len;
  if (cu == nullptr) { bos = (int64_t)n * T; len = T; }
  else { bos = cu[n]; len = cu[n + 1] - cu[n]; }

  // state row v0 + row, columns kc + 32 m + i (m, i = 0..3)
  float S[16];
  const size_t sidx = (((size_t)n * Hv + h) * DV + v0 + row) * DK + kc;
#pragma unroll
  for (int j = 0; j < 16; j += 4) {
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (init_dtype == KDA_STATE_F32) {
      x = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(h0) + sidx + 8 * j);
    } else if (init_dtype == KDA_STATE_BF16) {
      const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(h0) + sidx + 8 * j);
      x = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                      __uint_as_float(u.y & 0xffff0000u));
    }
    S[j] = x.x; S[j + 1] = x.y; S[j + 2] = x.z; S[j + 3] = x.w;
  }

  const float A_exp = (MODE == KDA_GATE_PREGATED || A_log == nullptr) ? 1.0f : expf(A_log[h]);
  const float lb_log2e = lower_bound * kLog2e;
  const float2 dtb = dt_bias != nullptr ? *reinterpret_cast<const float2*>(dt_bias + (size_t)h * DK + 2 * (tid & 63))
                                        : make_float2(0.0f, 0.0f);
  const bool norm = flags & KDA_FLAG_QK_L2NORM;
  const bool beta_prob = flags & KDA_FLAG_BETA_IS_PROB;

  RecurrentIn<TB> cur;
  recurrent_load<TB>(cur, 0, len, bos, q, k, v, g, beta, Hqk, Hv, h, hq, v0, tid, wave);
  for (int64_t s0 = 0; s0 < len; s0 += TB) {
    const int buf = (int)((s0 / TB) & 1);
    const int nb = (int)min((int64_t)TB, len - s0);
    RecurrentIn<TB> nxt;
    recurrent_load<TB>(nxt, s0 + TB, len, bos, q, k, v, g, beta, Hqk, Hv, h, hq, v0, tid, wave);
    // 1. the block into LDS: scale q/|q|, k/|k| and the decay factors of
    //    wave w's tokens; v of the slice rows; beta.  This buffer was last read
    //    two blocks ago, before the previous block's barrier.  A token's norms
    //    are one reduction over its wave in a fixed order, so any split of a
    //    sequence into calls gives bit-identical results.
    const int c = 2 * (tid & 63);
#pragma unroll
    for (int i = 0; i < RecurrentIn<TB>::TPW; ++i) {
      const int tk = wave + 4 * i;
      if (tk < TB) {  // uniform per wave
        const float q0 = __uint_as_float(cur.q[i] << 16), q1 = __uint_as_float(cur.q[i] & 0xffff0000u);
        const float k0 = __uint_as_float(cur.k[i] << 16), k1 = __uint_as_float(cur.k[i] & 0xffff0000u);
        const float g0 = __uint_as_float(cur.g[i] << 16), g1 = __uint_as_float(cur.g[i] & 0xffff0000u);
        float rq = scale, rk = 1.0f;
        if (norm) {
          rq *= rsqrtf(sum64(q0 * q0 + q1 * q1) + kL2Eps);
          rk = rsqrtf(sum64(k0 * k0 + k1 * k1) + kL2Eps);
        }
        *reinterpret_cast<float2*>(&sQ[buf][tk][c]) = make_float2(q0 * rq, q1 * rq);
        *reinterpret_cast<float2*>(&sK[buf][tk][c]) = make_float2(k0 * rk, k1 * rk);
        *reinterpret_cast<float2*>(&sD[buf][tk][c]) =
            make_float2(fast_exp2(gate2<MODE>(g0 + dtb.x, A_exp, lb_log2e)),
                        fast_exp2(gate2<MODE>(g1 + dtb.y, A_exp, lb_log2e)));
      }
    }
    if ((tid >> 5) < TB) sVv[buf][tid >> 5][tid & 31] = cur.vv;
    if (tid < TB) sB[buf][tid] = beta_prob ? cur.braw : fast_rcp(1.0f + fast_exp2(-kLog2e * cur.braw));
    __syncthreads();
    // 3. the block's tokens, in order, with no barrier
    for (int j = 0; j < nb; ++j) {
      const float b = sB[buf][j];
      const float vv = sVv[buf][j][row];
      float Kc[16], Qc[16], Dc[16];
#pragma unroll
      for (int jj = 0; jj < 16; jj += 4) {
        const float4 kk = *reinterpret_cast<const float4*>(&sK[buf][j][kc + 8 * jj]);
        const float4 qq = *reinterpret_cast<const float4*>(&sQ[buf][j][kc + 8 * jj]);
        const float4 dd = *reinterpret_cast<const float4*>(&sD[buf][j][kc + 8 * jj]);
        Kc[jj] = kk.x; Kc[jj + 1] = kk.y; Kc[jj + 2] = kk.z; Kc[jj + 3] = kk.w;
        Qc[jj] = qq.x; Qc[jj + 1] = qq.y; Qc[jj + 2] = qq.z; Qc[jj + 3] = qq.w;
        Dc[jj] = dd.x; Dc[jj + 1] = dd.y; Dc[jj + 2] = dd.z; Dc[jj + 3] = dd.w;
      }
      float r = 0.f;
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) { S[jj] *= Dc[jj]; r += S[jj] * Kc[jj]; }
      r = sum8(r);
      const float coef = b * (vv - r);
      float o = 0.f;
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) { S[jj] += coef * Kc[jj]; o += S[jj] * Qc[jj]; }
      o = sum8(o);
      if ((tid & 7) == 0)
        out[((size_t)(bos + s0 + j) * Hv + h) * DV + v0 + row] = __builtin_bit_cast(uint16_t, (__bf16)o);
    }
    cur = nxt;
  }

  if (final_dtype == KDA_STATE_F32) {
#pragma unroll
    for (int j = 0; j < 16; j += 4)
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(hT) + sidx + 8 * j) =
          make_float4(S[j], S[j + 1], S[j + 2], S[j + 3]);
  } else if (final_dtype == KDA_STATE_BF16) {
#pragma unroll
    for (int j = 0; j < 16; j += 4) {
      uint2 u;
      u.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)S[j]) |
            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)S[j + 1]) << 16);
      u.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)S[j + 2]) |
            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)S[j + 3]) << 16);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(hT) + sidx + 8 * j) = u;
    }
  }
}

// ---------------------------------------------------------------------------
// host side
}  // namespace

namespace kda_internal {

thread_local char g_last_error[512] = "";

kda_status fail(kda_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

int64_t max_chunks_of(const kda_fwd_params* p, bool packed) {
  const int64_t nc = ((int64_t)p->T + CH - 1) / CH;
  return packed ? nc + p->num_seqs : (int64_t)p->B * nc;
}

size_t header_bytes(const kda_fwd_params* p) {
  size_t b = (size_t)(p->num_seqs + 1) * sizeof(int);
  return (b + 255) & ~(size_t)255;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

void launch_chunk_map(const int64_t* cu, int N, int* chunk_off, hipStream_t st) {
  hipLaunchKernelGGL(kda_chunk_map_kernel, dim3(1), dim3(64), 0, st, cu, N, chunk_off);
}

kda_status launch_status() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KDA_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return KDA_OK;
}

}  // namespace kda_internal

namespace kda_internal {

// Time segments per state chain (dense input only) and chunks per segment.
// Automatic (segments == 0): split only when the state launch has at most
// half as many workgroups as the GPU has CUs (one state workgroup fills a
// CU), into up to 256 / workgroups segments of at least 16 chunks each.
int seg_plan(const kda_fwd_params* p, bool packed, int* seg_len) {
  const int ncs = (int)(((int64_t)p->T + CH - 1) / CH);
  int nseg = 1;
  if (!packed && ncs > 1) {
    if (p->segments >= 2) {
      nseg = p->segments;
    } else if (p->segments == 0) {
      const int64_t wgs = (int64_t)p->num_seqs * p->H_v * NSLICE;
      if (wgs <= 128) nseg = (int)std::min<int64_t>(256 / wgs, ncs / 16);
    }
    nseg = std::min(nseg, std::min(ncs, kMaxSegments));
    // at most kMaxChains jobs per launch (the combine runs only for nseg >= 3)
    nseg = std::max(1, std::min<int>(nseg, (int)(kMaxChains / std::max<int64_t>(1, (int64_t)p->num_seqs * p->H_v))));
  }
  const int len = ncs > 0 ? (ncs + nseg - 1) / nseg : 0;
  *seg_len = len;
  return len > 0 ? (ncs + len - 1) / len : 1;
}

size_t seg_scratch_bytes(const kda_fwd_params* p, int nseg) {
  return nseg > 1 ? (size_t)3 * p->num_seqs * p->H_v * nseg * DV * DK * sizeof(float) : 0;
}

kda_status check_params(const kda_fwd_params* p, bool packed) {
  if (!p) return fail(KDA_ERR_NULL, "params is NULL");
  if (p->K != DK || p->V != DV) return fail(KDA_ERR_SHAPE, "K and V must both be 128 (got K=%d, V=%d)", p->K, p->V);
  if (p->B <= 0 || p->T < 0 || p->H_qk <= 0 || p->H_v <= 0)
    return fail(KDA_ERR_SHAPE, "need B > 0, T >= 0, H_qk > 0, H_v > 0");
  if (p->H_v % p->H_qk != 0) return fail(KDA_ERR_SHAPE, "H_v (%d) must be a multiple of H_qk (%d)", p->H_v, p->H_qk);
  if (packed) {
    if (p->B != 1) return fail(KDA_ERR_SHAPE, "with cu_seqlens, B must be 1 (got %d)", p->B);
    if (p->num_seqs <= 0) return fail(KDA_ERR_SHAPE, "with cu_seqlens, num_seqs must be > 0");
  } else if (p->num_seqs != p->B) {
    return fail(KDA_ERR_SHAPE, "without cu_seqlens, num_seqs (%d) must equal B (%d)", p->num_seqs, p->B);
  }
  if ((int64_t)p->B * p->T * (int64_t)p->H_v > ((int64_t)1 << 40))
    return fail(KDA_ERR_SHAPE, "B*T*H_v too large");
  // a dispatch dimension holds fewer than 2^32 work-items: one 256-thread
  // workgroup per chunk (grid x) and 4 per (sequence, head) pair
  if (max_chunks_of(p, packed) >= kMaxChunks || max_chunks_of(p, packed) * (int64_t)p->H_v > ((int64_t)1 << 30))
    return fail(KDA_ERR_SHAPE, "too many chunks");
  if ((int64_t)p->num_seqs * p->H_v > kMaxChains)
    return fail(KDA_ERR_SHAPE, "too many (sequence, head) pairs");
  if (p->H_v > 65535) return fail(KDA_ERR_SHAPE, "H_v must be at most 65535 (the y extent of a launch)");
  if (p->gate_mode != KDA_GATE_SOFTPLUS && p->gate_mode != KDA_GATE_SAFE_SIGMOID &&
      p->gate_mode != KDA_GATE_PREGATED)
    return fail(KDA_ERR_UNSUPPORTED, "unknown gate_mode %d", p->gate_mode);
  if (p->flags & ~(KDA_FLAG_QK_L2NORM | KDA_FLAG_BETA_IS_PROB))
    return fail(KDA_ERR_UNSUPPORTED, "unknown flag bits in %d", p->flags);
  if (p->gate_mode == KDA_GATE_SAFE_SIGMOID && !(p->lower_bound >= -5.0f && p->lower_bound < 0.0f))
    return fail(KDA_ERR_RANGE, "safe gate needs -5 <= lower_bound < 0 (got %g)", (double)p->lower_bound);
  if (!(p->scale == p->scale) || p->scale > 3.0e38f || p->scale < -3.0e38f)
    return fail(KDA_ERR_RANGE, "scale must be finite");
  const int sd[2] = {p->init_state_dtype, p->final_state_dtype};
  for (int i = 0; i < 2; ++i)
    if (sd[i] != KDA_STATE_NONE && sd[i] != KDA_STATE_F32 && sd[i] != KDA_STATE_BF16)
      return fail(KDA_ERR_DTYPE, "unknown state dtype code %d", sd[i]);
  if (p->init_state_dtype != KDA_STATE_NONE && p->final_state_dtype != KDA_STATE_NONE &&
      p->init_state_dtype != p->final_state_dtype)
    return fail(KDA_ERR_DTYPE, "initial_state and final_state dtypes must match when both are given");
  if (p->segments < 0 || p->segments > kMaxSegments)
    return fail(KDA_ERR_RANGE, "segments must be in [0, %d] (got %d)", kMaxSegments, p->segments);
  return KDA_OK;
}

}  // namespace kda_internal

extern "C" {

size_t kda_fwd_workspace_size(const kda_fwd_params* p) {
  if (!p) return 0;
  // packed or dense cannot be told from params alone; size for the larger
  const bool packed = p->B == 1 && p->num_seqs >= 1;
  if (check_params(p, false) != KDA_OK && check_params(p, true) != KDA_OK) return 0;
  const int64_t mc = max_chunks_of(p, packed);
  size_t seg = 0;
  if (check_params(p, false) == KDA_OK) {
    int len;
    seg = seg_scratch_bytes(p, seg_plan(p, false, &len));
  }
  return header_bytes(p) + (size_t)p->H_v * (size_t)mc * BLOCK + seg;
}

int kda_fwd_segments(const kda_fwd_params* p, int packed) {
  if (!p || check_params(p, packed != 0) != KDA_OK) return 0;
  int len;
  return seg_plan(p, packed != 0, &len);
}

}  // extern "C"

namespace {
// The predicates of kda_fwd_check; the workspace ones only when it is used.
kda_status check_call(const kda_fwd_params* p, const void* q, const void* k, const void* v, const void* g,
                      const void* beta, const float* A_log, const float* dt_bias, const int64_t* cu_seqlens,
                      const void* initial_state, const void* final_state, const void* out,
                      const void* workspace, size_t workspace_bytes, bool uses_workspace) {
  g_last_error[0] = 0;
  const bool packed = cu_seqlens != nullptr;
  kda_status s = check_params(p, packed);
  if (s != KDA_OK) return s;
  if (p->gate_mode == KDA_GATE_PREGATED && dt_bias)
    return fail(KDA_ERR_UNSUPPORTED, "dt_bias must be NULL with pre-gated decay");
  const bool empty = (int64_t)p->B * p->T == 0;
  if (!empty) {
    const void* req[] = {q, k, v, g, beta, out};
    const char* names[] = {"q", "k", "v", "g", "beta", "out"};
    for (int i = 0; i < 6; ++i)
      if (!req[i]) return fail(KDA_ERR_NULL, "%s is NULL", names[i]);
    if (p->gate_mode == KDA_GATE_SOFTPLUS && !A_log)
      return fail(KDA_ERR_NULL, "A_log is NULL (required by the softplus gate)");
    const void* al[] = {q, k, v, g, out};
    const char* aln[] = {"q", "k", "v", "g", "out"};
    for (int i = 0; i < 5; ++i)
      if (!aligned16(al[i])) return fail(KDA_ERR_ALIGN, "%s is not 16-byte aligned", aln[i]);
    if (dt_bias && !aligned16(dt_bias)) return fail(KDA_ERR_ALIGN, "dt_bias is not 16-byte aligned");
  }
  if (p->init_state_dtype != KDA_STATE_NONE) {
    if (!initial_state) return fail(KDA_ERR_NULL, "initial_state is NULL but init_state_dtype is set");
    if (!aligned16(initial_state)) return fail(KDA_ERR_ALIGN, "initial_state is not 16-byte aligned");
  }
  if (p->final_state_dtype != KDA_STATE_NONE) {
    if (!final_state) return fail(KDA_ERR_NULL, "final_state is NULL but final_state_dtype is set");
    if (!aligned16(final_state)) return fail(KDA_ERR_ALIGN, "final_state is not 16-byte aligned");
  }
  if (!uses_workspace) return KDA_OK;
  const size_t need = kda_fwd_workspace_size(p);
  if (!workspace || workspace_bytes < need)
    return fail(KDA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", NULL");
  if (((uintptr_t)workspace & 255u) != 0) return fail(KDA_ERR_ALIGN, "workspace is not 256-byte aligned");
  return KDA_OK;
}
}  // namespace

extern "C" {

kda_status kda_fwd_check(const kda_fwd_params* p, const void* q, const void* k, const void* v,
                         const void* g, const void* beta, const float* A_log, const float* dt_bias,
                         const int64_t* cu_seqlens, const void* initial_state, const void* final_state,
                         const void* out, const void* workspace, size_t workspace_bytes) {
  return check_call(p, q, k, v, g, beta, A_log, dt_bias, cu_seqlens, initial_state, final_state, out, workspace,
                    workspace_bytes, true);
}

}  // extern "C"

namespace {

kda_status launch_intra(const kda_fwd_params* p, const void* q, const void* k, const void* g, const void* beta,
                        const float* A_log, const float* dt_bias, const int64_t* cu_seqlens, void* workspace,
                        hipStream_t st) {
  const bool packed = cu_seqlens != nullptr;
  const int64_t mc = max_chunks_of(p, packed);
  uint8_t* wsb = reinterpret_cast<uint8_t*>(workspace);
  int* chunk_off = reinterpret_cast<int*>(wsb);
  uint8_t* blocks = wsb + header_bytes(p);
  if (packed) launch_chunk_map(cu_seqlens, p->num_seqs, chunk_off, st);
  if (mc > 0) {
    auto kern = p->gate_mode == KDA_GATE_SAFE_SIGMOID ? kda_intra_kernel<KDA_GATE_SAFE_SIGMOID>
                : p->gate_mode == KDA_GATE_PREGATED   ? kda_intra_kernel<KDA_GATE_PREGATED>
                                                      : kda_intra_kernel<KDA_GATE_SOFTPLUS>;
    hipLaunchKernelGGL(kern, dim3((unsigned)mc, (unsigned)p->H_v), dim3(256), 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)g, (const uint16_t*)beta,
                       A_log, dt_bias, cu_seqlens, chunk_off, p->B, p->T, p->num_seqs, p->H_qk, p->H_v,
                       (int)mc, p->scale, p->lower_bound, p->flags, blocks);
  }
  return KDA_OK;
}

struct StateArgs {
  const uint16_t* v;
  const int64_t* cu;
  const int* chunk_off;
  const void* h0;
  void* hT;
  uint16_t* out;
  const uint8_t* ws;
  float* seg;
  int T, N, Hv, mc, init_dtype, final_dtype, nseg, seg_len;
  float scale;
};

// One state launch of `jobs` jobs: groups of 8 jobs, one workgroup (one per
// CU) per V slice.  A chunk step of a 64-column slice takes about 1.85 times
// that of a 32-column one (measured on the varlen workload), and each job
// needs half as many of them; so the launch takes the width whose rounds of
// 256 workgroups, weighted by step time, cost less (narrow up to 64 jobs,
// wide for 65..128; with many jobs the two alternate, wide saving up to 7 %).
constexpr int64_t kWideStepPct = 185;
template <int KIND>
void launch_state_kind(const StateArgs& a, int64_t jobs, hipStream_t st) {
  const int64_t narrow_rounds = (jobs * NSLICE + kGpuCUs - 1) / kGpuCUs;
  const int64_t wide_rounds = (jobs * (NSLICE / 2) + kGpuCUs - 1) / kGpuCUs;
  if (wide_rounds * kWideStepPct >= narrow_rounds * 100) {
    if constexpr (KIND == ST_FULL || KIND == ST_CARRY)
      hipLaunchKernelGGL(kda_state_split_kernel<KIND>, dim3((unsigned)(((jobs + 7) / 8) * 8 * NSLICE)),
                         dim3(64 * SPWAVES), 0, st, a.v, a.cu, a.chunk_off, a.h0, a.hT, a.out, a.ws, a.seg, a.T, a.N,
                         a.Hv, a.mc, a.init_dtype, a.final_dtype, a.nseg, a.seg_len, a.scale);
    else
      hipLaunchKernelGGL((kda_state_kernel<KIND, NVT_NARROW>), dim3((unsigned)(((jobs + 7) / 8) * 8 * NSLICE)),
                         dim3(64 * SWAVES), 0, st, a.v, a.cu, a.chunk_off, a.h0, a.hT, a.out, a.ws, a.seg, a.T, a.N,
                         a.Hv, a.mc, a.init_dtype, a.final_dtype, a.nseg, a.seg_len, a.scale);
  } else {
    constexpr int nsl = DV / (16 * NVT_WIDE);
    hipLaunchKernelGGL((kda_state_kernel<KIND, NVT_WIDE>), dim3((unsigned)(((jobs + 7) / 8) * 8 * nsl)),
                       dim3(64 * SWAVES), 0, st, a.v, a.cu, a.chunk_off, a.h0, a.hT, a.out, a.ws, a.seg, a.T, a.N,
                       a.Hv, a.mc, a.init_dtype, a.final_dtype, a.nseg, a.seg_len, a.scale);
  }
}

kda_status launch_state(const kda_fwd_params* p, const void* v, const int64_t* cu_seqlens,
                        const void* initial_state, void* final_state, void* out, void* workspace, hipStream_t st) {
  const bool packed = cu_seqlens != nullptr;
  const int64_t mc = max_chunks_of(p, packed);
  uint8_t* wsb = reinterpret_cast<uint8_t*>(workspace);
  const int* chunk_off = reinterpret_cast<const int*>(wsb);
  const uint8_t* blocks = wsb + header_bytes(p);
  float* seg = reinterpret_cast<float*>(wsb + header_bytes(p) + (size_t)p->H_v * (size_t)mc * BLOCK);
  const int chains = p->num_seqs * p->H_v;
  int seg_len;
  const int nseg = seg_plan(p, packed, &seg_len);
  const StateArgs a{(const uint16_t*)v, cu_seqlens, chunk_off, initial_state, final_state, (uint16_t*)out, blocks,
                    seg, p->T, p->num_seqs, p->H_v, (int)mc, p->init_state_dtype, p->final_state_dtype, nseg, seg_len,
                    p->scale};
  if (nseg > 1) {
    // entry states of the segments from their zero-state carries and maps
    launch_state_kind<ST_CARRY>(a, (int64_t)chains * (nseg - 1), st);
    if (nseg > 2) {
      launch_state_kind<ST_TRANS>(a, (int64_t)chains * (nseg - 2), st);
      hipLaunchKernelGGL(kda_segment_combine_kernel, dim3((unsigned)(chains * (DV / CMB_ROWS))), dim3(256), 0, st,
                         seg, chains, nseg);
    }
  }
  launch_state_kind<ST_FULL>(a, (int64_t)chains * nseg, st);
  return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_fwd(const kda_fwd_params* p, const void* q, const void* k, const void* v, const void* g,
                   const void* beta, const float* A_log, const float* dt_bias, const int64_t* cu_seqlens,
                   const void* initial_state, void* final_state, void* out, void* workspace,
                   size_t workspace_bytes, void* stream) {
  kda_status s = kda_fwd_check(p, q, k, v, g, beta, A_log, dt_bias, cu_seqlens, initial_state, final_state,
                               out, workspace, workspace_bytes);
  if (s != KDA_OK) return s;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if ((s = launch_intra(p, q, k, g, beta, A_log, dt_bias, cu_seqlens, workspace, st)) != KDA_OK) return s;
  if ((s = launch_state(p, v, cu_seqlens, initial_state, final_state, out, workspace, st)) != KDA_OK) return s;
  return launch_status();
}

kda_status kda_fwd_intra(const kda_fwd_params* p, const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* A_log, const float* dt_bias, const int64_t* cu_seqlens,
                         const void* initial_state, void* final_state, void* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  kda_status s = kda_fwd_check(p, q, k, v, g, beta, A_log, dt_bias, cu_seqlens, initial_state, final_state,
                               out, workspace, workspace_bytes);
  if (s != KDA_OK) return s;
  (void)hipGetLastError();
  launch_intra(p, q, k, g, beta, A_log, dt_bias, cu_seqlens, workspace, reinterpret_cast<hipStream_t>(stream));
  return launch_status();
}

kda_status kda_fwd_state(const kda_fwd_params* p, const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* A_log, const float* dt_bias, const int64_t* cu_seqlens,
                         const void* initial_state, void* final_state, void* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  kda_status s = kda_fwd_check(p, q, k, v, g, beta, A_log, dt_bias, cu_seqlens, initial_state, final_state,
                               out, workspace, workspace_bytes);
  if (s != KDA_OK) return s;
  (void)hipGetLastError();
  launch_state(p, v, cu_seqlens, initial_state, final_state, out, workspace, reinterpret_cast<hipStream_t>(stream));
  return launch_status();
}

}  // extern "C"

namespace {
// The address of `scratch` on each device, looked up once per device with that
// device current (every GPU holds its own copy of the array).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

kda_status noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KDA_ERR_LAUNCH, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(KDA_ERR_UNSUPPORTED, "device index %d is beyond the %d this library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(KDA_ERR_LAUNCH, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KDA_OK;
}
}  // namespace

extern "C" {

kda_status kda_fwd_noalloc(const kda_fwd_params* p, const void* q, const void* k, const void* v, const void* g,
                           const void* beta, const float* A_log, const float* dt_bias, const int64_t* cu_seqlens,
                           const void* initial_state, void* final_state, void* out, void* stream) {
  kda_status s = check_call(p, q, k, v, g, beta, A_log, dt_bias, cu_seqlens, initial_state, final_state, out,
                            nullptr, 0, false);
  if (s != KDA_OK) return s;
  const size_t need = kda_fwd_workspace_size(p);
  if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES)
    return fail(KDA_ERR_WORKSPACE, "kda_fwd_noalloc handles calls whose workspace fits %zu bytes; this one needs %zu "
                "(use kda_fwd with a caller workspace)", (size_t)KDA_NOALLOC_SCRATCH_BYTES, need);
  void* ws = nullptr;
  if ((s = noalloc_scratch(&ws)) != KDA_OK) return s;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  // the same launches as kda_fwd, on the device array; nothing in the
  // workspace needs to start at zero (every block is written before it is read)
  if ((s = launch_intra(p, q, k, g, beta, A_log, dt_bias, cu_seqlens, ws, st)) != KDA_OK) return s;
  if ((s = launch_state(p, v, cu_seqlens, initial_state, final_state, out, ws, st)) != KDA_OK) return s;
  return launch_status();
}

kda_status kda_fused_recurrent_fwd(const kda_fwd_params* p, const void* q, const void* k, const void* v,
                                   const void* g, const void* beta, const float* A_log, const float* dt_bias,
                                   const int64_t* cu_seqlens, const void* initial_state, void* final_state,
                                   void* out, void* stream) {
  kda_status s = check_call(p, q, k, v, g, beta, A_log, dt_bias, cu_seqlens, initial_state, final_state, out,
                            nullptr, 0, false);
  if (s != KDA_OK) return s;
  const int64_t chains = (int64_t)p->num_seqs * p->H_v;
  if (chains == 0) return KDA_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  // decode steps (at most one token per sequence): one-token blocks
  const bool decode = (int64_t)p->B * p->T <= (int64_t)p->num_seqs;
  auto kern = decode ? (p->gate_mode == KDA_GATE_SAFE_SIGMOID ? kda_recurrent_kernel<KDA_GATE_SAFE_SIGMOID, 1>
                        : p->gate_mode == KDA_GATE_PREGATED   ? kda_recurrent_kernel<KDA_GATE_PREGATED, 1>
                                                              : kda_recurrent_kernel<KDA_GATE_SOFTPLUS, 1>)
                     : (p->gate_mode == KDA_GATE_SAFE_SIGMOID ? kda_recurrent_kernel<KDA_GATE_SAFE_SIGMOID, RTB>
                        : p->gate_mode == KDA_GATE_PREGATED   ? kda_recurrent_kernel<KDA_GATE_PREGATED, RTB>
                                                              : kda_recurrent_kernel<KDA_GATE_SOFTPLUS, RTB>);
  hipLaunchKernelGGL(kern, dim3((unsigned)(chains * RNSLICE)), dim3(256), 0, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)g, (const uint16_t*)beta, A_log,
                     dt_bias, cu_seqlens, initial_state, final_state, (uint16_t*)out, p->T, p->num_seqs, p->H_qk,
                     p->H_v, p->scale, p->lower_bound, p->flags, p->init_state_dtype, p->final_state_dtype);
  return launch_status();
}

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_NULL: return "KDA_ERR_NULL";
    case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE";
    case KDA_ERR_DTYPE: return "KDA_ERR_DTYPE";
    case KDA_ERR_RANGE: return "KDA_ERR_RANGE";
    case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
    case KDA_ERR_LAUNCH: return "KDA_ERR_LAUNCH";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
  }
  return "KDA_ERR_UNKNOWN";
}

const char* kda_last_error(void) { return g_last_error; }

}  // extern "C"
