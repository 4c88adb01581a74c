// Shared device/host helpers for the MoE layer kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_WAVE 64

namespace moe {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// ---- element types -------------------------------------------------------
// Every type moves through memory in 16-byte vectors (uint4); VEC elements each.
struct DtF32 {
  using T = float;
  static constexpr int VEC = 4;
  __device__ static inline float to_f(T v) { return v; }
  __device__ static inline T from_f(float v) { return v; }
};
struct DtF16 {
  using T = _Float16;
  static constexpr int VEC = 8;
  __device__ static inline float to_f(T v) { return (float)v; }
  __device__ static inline T from_f(float v) { return (T)v; }   // round to nearest even
};
struct DtBF16 {
  using T = __bf16;
  static constexpr int VEC = 8;
  __device__ static inline float to_f(T v) { return (float)v; }
  __device__ static inline T from_f(float v) { return (T)v; }   // round to nearest even
};

// Unpack a 16-byte vector into VEC floats.
template <typename DT>
__device__ inline void unpack16(const uint4& v, float* out) {
  const typename DT::T* e = reinterpret_cast<const typename DT::T*>(&v);
#pragma unroll
  for (int i = 0; i < DT::VEC; ++i) out[i] = DT::to_f(e[i]);
}

// Dot product of two 16-byte vectors (VEC elements), fp32 accumulate.
template <typename DT>
__device__ inline float dot16(const uint4& a, const uint4& b, float acc) {
  const typename DT::T* ea = reinterpret_cast<const typename DT::T*>(&a);
  const typename DT::T* eb = reinterpret_cast<const typename DT::T*>(&b);
#pragma unroll
  for (int i = 0; i < DT::VEC; ++i) acc = fmaf(DT::to_f(ea[i]), DT::to_f(eb[i]), acc);
  return acc;
}

// Dot of a 16-byte vector with VEC floats.
template <typename DT>
__device__ inline float dot16f(const uint4& a, const float* b, float acc) {
  const typename DT::T* ea = reinterpret_cast<const typename DT::T*>(&a);
#pragma unroll
  for (int i = 0; i < DT::VEC; ++i) acc = fmaf(DT::to_f(ea[i]), b[i], acc);
  return acc;
}

// Exact GeLU u * Phi(u) = 0.5 u (1 + erf(u / sqrt 2)), with the device erff.
__device__ inline float gelu_erf(float u) { return 0.5f * u * (1.0f + erff(u * 0.70710678118654752f)); }

// Wave-wide sum (all lanes get the result).
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
  return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, MOE_WAVE));
  return v;
}

__device__ inline int lane_id() { return threadIdx.x & (MOE_WAVE - 1); }

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load marked non-temporal: data streamed once (expert weights) should
// not displace reused lines from the caches.
__device__ inline uint4 ld_nt16(const void* ptr) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(ptr));
  return __builtin_bit_cast(uint4, v);
}

}  // namespace moe

// ---------------------------------------------------------------------------
// Launch descriptors shared by the host code and the kernel files.

namespace moe {

enum Dtype { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

// Grouped GEMM  C[r, n] = epi( sum_k A[arow(r), k] * B_s[n, k] + bias_s[n] )
// for every row r of every segment s, where segments are row ranges
// [seg_off[s], seg_off[s+1]) of a shared row space (or one segment [0, M)).
struct GemmParams {
  const void* A;          // activations, row-major [*, K]
  const int* a_rows;      // optional row map: row r of the row space reads A row a_rows[r]
  const int* seg_off;     // [nseg + 1] or null (single segment of M rows)
  int nseg;
  int M;                  // rows of the single segment when seg_off == null
  int N, K;
  const void* B;          // weights [nseg][N][K]
  long long b_stride;     // elements between consecutive segments' weights
  const void* bias;       // [nseg][N] or null
  long long bias_stride;
  void* C;                // output rows of the row space, ldc = N
  const int2* tiles;      // tile list (seg, nt<<16 | mt) or null (single segment)
  const int* tile_count;  // number of m-tiles in the list (device)
  int n_ntiles;
};

// Fused small-M expert FFN: each work-group handles one active segment and one
// BF-wide slice of the FFN width, writing partial outputs part[slice][row][H].
struct DecodeParams {
  const void* x;          // activations [*, H]
  const int* a_rows;      // row map (slot -> token) or null (dense: rows [0, M))
  const int* seg_off;     // [nseg + 1] or null
  int nseg;
  int M;                  // rows when seg_off == null
  int H, F;
  const void* w1; const void* b1; const void* w2; const void* b2;  // [nseg][F][H] ...
  float* part;            // [F / BF][row_space][H]
  long long row_space;
};

}  // namespace moe
