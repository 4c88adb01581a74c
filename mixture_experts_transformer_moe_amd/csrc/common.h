// Shared device/host helpers for the MoE layer kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_WAVE 64

// Launch; when either event is given they are recorded by the dispatch itself
// (kernel start / end timestamps, no extra queue packets).
#define MOE_LAUNCH(kernel, grid, block, lds, stream, ev0, ev1, ...)                                  \
  do {                                                                                              \
    if ((ev0) || (ev1))                                                                             \
      hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, ev0, ev1, 0, __VA_ARGS__);            \
    else                                                                                            \
      hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);                            \
  } while (0)

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

// Pin a value to an fp32 register so the compiler cannot fold the following
// conversion to a narrower type into the operation that produced it (e.g. an
// fp32 multiply + fp16 conversion into one mixed-precision FMA with a single
// rounding). Every result is rounded to fp32 first, then to the I/O dtype, the
// same way on every path.
__device__ inline float pin_f32(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Exact GeLU u * Phi(u) = 0.5 u (1 + erf(u / sqrt 2)), with the device erff.
__device__ inline float gelu_erf(float u) { return 0.5f * u * (1.0f + erff(u * 0.70710678118654752f)); }

// Lane moves inside rows of 16 lanes through DPP (an operand modifier of the
// VALU instruction, no LDS round trip as a bpermute shuffle takes): xor 1 and
// xor 2 inside each quad, then the mirrors that pair lane i with lane 7 - i in
// each half row and with 15 - i in each row. Once the two quad steps have given
// every lane of a quad the same value, the mirrors pair quads and half rows as
// xor 4 and xor 8 would, so four steps leave a row's result in all its lanes.
// Every lane of the wave must be active.
#define MOE_DPP_XOR1 0xB1      // quad_perm [1, 0, 3, 2]
#define MOE_DPP_XOR2 0x4E      // quad_perm [2, 3, 0, 1]
#define MOE_DPP_HMIRROR 0x141  // row_half_mirror
#define MOE_DPP_MIRROR 0x140   // row_mirror
template <int CTRL>
__device__ inline int dpp_mov(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ inline float dpp_mov(float v) {
  return __builtin_bit_cast(float, dpp_mov<CTRL>(__builtin_bit_cast(int, v)));
}
__device__ inline float readlane_f(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Wave-wide sum (all lanes get the result): rows reduced by DPP, then the four
// row sums added as (r0 + r1) + (r2 + r3).
__device__ inline float wave_sum(float v) {
  v += dpp_mov<MOE_DPP_XOR1>(v);
  v += dpp_mov<MOE_DPP_XOR2>(v);
  v += dpp_mov<MOE_DPP_HMIRROR>(v);
  v += dpp_mov<MOE_DPP_MIRROR>(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}
__device__ inline float wave_max(float v) {
  v = fmaxf(v, dpp_mov<MOE_DPP_XOR1>(v));
  v = fmaxf(v, dpp_mov<MOE_DPP_XOR2>(v));
  v = fmaxf(v, dpp_mov<MOE_DPP_HMIRROR>(v));
  v = fmaxf(v, dpp_mov<MOE_DPP_MIRROR>(v));
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

__device__ inline int lane_id() { return threadIdx.x & (MOE_WAVE - 1); }

// v of lane (lane ^ O): DPP moves inside rows of 16 lanes for O < 16 (xor 1 and
// 2 by quad permutes, xor 8 by a rotate of the row by 8, xor 4 by a rotate by 12
// (lanes with bit 2 clear, taking lane + 4) or by 4 (the others, lane - 4));
// gfx950's lane-swap instructions for 16 and 32 (a swap of v with itself leaves
// each lane's partner value in one of its two results). The same values as
// __shfl_xor, with no LDS round trip. Every lane of the wave must be active.
template <int O>
__device__ inline float shfl_xor_wave(float v, int lane) {
  if constexpr (O == 1) {
    return dpp_mov<MOE_DPP_XOR1>(v);
  } else if constexpr (O == 2) {
    return dpp_mov<MOE_DPP_XOR2>(v);
  } else if constexpr (O == 4) {
    const float up = dpp_mov<0x12C>(v);   // row_ror:12: lane i takes lane (i + 4) mod 16
    const float dn = dpp_mov<0x124>(v);   // row_ror:4: lane i takes lane (i - 4) mod 16
    return (lane & 4) ? dn : up;
  } else if constexpr (O == 8) {
    return dpp_mov<0x128>(v);             // row_ror:8: lane i takes lane i ^ 8
  } else if constexpr (O == 16) {
    // [0]: lanes 16-31 / 48-63 hold lanes 0-15 / 32-47; [1]: lanes 0-15 / 32-47 hold 16-31 / 48-63
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __builtin_bit_cast(float, (lane & 16) ? r[0] : r[1]);
  } else {
    static_assert(O == 32, "xor 1, 2, 4, 8, 16 or 32");
    // [0]: lanes 32-63 hold lanes 0-31; [1]: lanes 0-31 hold lanes 32-63
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (lane & 32) ? r[0] : r[1]);
  }
}

// Inclusive sum of v over lanes 0 .. lane (integers, so exact in any order):
// DPP row shifts by 1, 2, 4 and 8 scan each row of 16 lanes (a lane with no
// source adds 0), then the row broadcasts add lane 15's total to rows 1 and 3
// and lane 31's to rows 2 and 3. Every lane of the wave must be active.
__device__ inline int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15, rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31, rows 2 and 3
  return v;
}

// Reduce N per-lane values over the whole wave at once (N a power of two, <= 64).
// Transpose steps: at offset O each lane pair swaps half of its values, so after
// log2(N) steps lane l holds one index, l >> (6 - log2 N), summed over the lanes
// sharing its low bits; plain xor steps over those low bits finish the sum.
// 63 shuffles for N = 64 instead of 6 N. Every step is unrolled at compile time
// so the values stay in registers.
template <int N, int O>
struct WaveTranspose {
  __device__ static inline void run(float* v, int lane) {
    constexpr int h = N / 2;
    const bool hi = (lane & O) != 0;
#pragma unroll
    for (int j = 0; j < h; ++j) {
      const float send = hi ? v[j] : v[j + h];
      const float keep = hi ? v[j + h] : v[j];
      v[j] = keep + shfl_xor_wave<O>(send, lane);
    }
    WaveTranspose<h, O / 2>::run(v, lane);
  }
};
template <int O>
struct WaveTranspose<1, O> {
  __device__ static inline void run(float*, int) {}
};

// Returns the wave-wide total of index (lane >> (6 - log2 N)) in every lane.
template <int N>
__device__ inline float wave_reduce_multi(float (&v)[N]) {
  static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "N must be a power of two <= 64");
  const int lane = threadIdx.x & 63;
  WaveTranspose<N, 32>::run(v, lane);
  float r = v[0];
  if constexpr (32 / N >= 32) r += shfl_xor_wave<32>(r, lane);
  if constexpr (32 / N >= 16) r += shfl_xor_wave<16>(r, lane);
  if constexpr (32 / N >= 8) r += shfl_xor_wave<8>(r, lane);
  if constexpr (32 / N >= 4) r += shfl_xor_wave<4>(r, lane);
  if constexpr (32 / N >= 2) r += shfl_xor_wave<2>(r, lane);
  if constexpr (32 / N >= 1) r += shfl_xor_wave<1>(r, lane);
  return r;
}

// All-ones if cond else zero, to mask loaded data without a branch.
__device__ inline uint4 mask16(const uint4& v, bool cond) {
  const unsigned m = cond ? 0xffffffffu : 0u;
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load marked non-temporal: data streamed once (expert weights) should
// not displace reused lines from the caches.
// global address space stated so the load is a global_load, never a flat one
// (a flat load also counts against lgkmcnt, so LDS waits would wait for it)
__device__ inline uint4 ld_nt16(const void* ptr) {
  typedef const __attribute__((address_space(1))) u32x4_t* gptr_t;
  const u32x4_t v = __builtin_nontemporal_load((gptr_t)ptr);
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
  const void* const* Bp;     // optional: segment s's weights [N][K] at Bp[s] (replaces B, b_stride)
  const void* const* biasp;  // optional: segment s's bias [N] at biasp[s] (replaces bias, bias_stride)
  void* C;                // output rows of the row space, ldc = N
  const int2* tiles;      // tile list (seg, nt<<16 | mt) or null (single segment)
  const int* tile_count;  // number of m-tiles in the list (device)
  int n_ntiles;
  // optional extra segment (id nseg) with its own operands: rows [0, M2) of A2
  // (no row map), weights B2 [N][K], bias2 [N], output C2 [M2][N]; M2 = 0: none
  const void* A2;
  const void* B2;
  const void* bias2;
  void* C2;
  int M2;
  // split over K (fp32 output, float bias): grid.y = ksplit slices of K, slice s
  // writes its partial sums to C + s * c_split (bias in slice 0 only); 0 or 1: none
  int ksplit;
  long long c_split;
  // optional top-1 combine folded into an fp32 epilogue: row r of the row space
  // is token fold_token[r], and the epilogue writes fold_y[token] =
  // round(fold_w[token] * value) in the I/O dtype (zero_esz bytes) instead of C.
  // null: none
  void* fold_y;
  const int* fold_token;
  const float* fold_w;
  // optional: after their K loops the launch's work-groups also zero the zero_T
  // rows of zero_y (zero_N elements of zero_esz bytes each), row t by work-group
  // t mod (gridDim.x * gridDim.y). null: none
  void* zero_y;
  int zero_T, zero_esz, zero_N;
  // optional: the launch's work-groups also zero zero_n16 16-byte words at
  // zero_ws (spread over them the same way). null: none
  void* zero_ws;
  int zero_n16;
  // host only: every expert weight tile is read by at most two work-groups
  // (segments of at most two row tiles), so the launch picks the variant that
  // streams the expert weights with non-temporal loads
  int stream_w;
  // host only: every operand (A, A2 and each segment's weights) spans less than
  // 4 GB, so byte offsets from its base fit 32 bits (buffer-load addressing)
  int off32;
};

// Expert FFN for segments of at most MAXM rows: each work-group takes one
// non-empty segment (or, with seg_off == null, the single segment [0, M)) and
// a block of weight rows.
struct DecodeParams {
  const void* x;          // activations [*, H]
  const int* a_rows;      // row map (row -> token) or null (rows index x directly)
  const int* seg_off;     // [nseg + 1] or null
  int nseg;
  int M;                  // rows when seg_off == null
  int H, F;
  const void* w1; const void* b1; const void* w2; const void* b2;  // [nseg][F][H], [nseg][F], ...
  // optional per-segment placement: segment s's W1 [F][H] at w1p[s], ... (device
  // arrays of nseg pointers, device or pinned host memory); null: the arrays above
  const void* const* w1p; const void* const* b1p; const void* const* w2p; const void* const* b2p;
  void* h;                // hidden activation [rows][F], I/O dtype (written by up, read by down)
  void* out;              // down: fp32 [rows][H], or the layer output [T][H] when the combine is folded in
  const int* slot_token;  // folded combine: token of each row
  const float* topk_w;    // folded combine: top-1 weight of each token
  // optional dense segment, the residual MLP over rows [0, dM) of x (dM <= 8),
  // served by work-groups after those of the ngroups expert segment groups:
  // weights dw1 [F][H], db1 [F], dw2 [H][F], db2 [H]; hidden dh [dM][F] (I/O
  // dtype); output dout fp32 [dM][H]. dM = 0: none
  int dM;
  int ngroups;            // expert segment groups of the launch (set by the launcher)
  const void* dw1; const void* db1; const void* dw2; const void* db2;
  void* dh;
  float* dout;
};

// Routing of a decode-sized batch done inside the first expert kernel: every
// work-group computes softmax / top-k and the dispatch of all k*T <= 256
// assignments in LDS from the gate logits z; work-group 0 also writes them out.
struct RouteParams {
  const float* z;          // [T][E] gate logits
  int T, k, E, e_lo, E_loc, C, R_max, renorm;
  int* idx;                // [T][k]
  float* w;                // [T][k]
  int* demand;             // [E]
  int* offsets;            // [E_loc + 1]
  int* slot_token;         // [R_max]
  int* token_slot;         // [T][k]
  void* y_zero;            // output rows of tokens with nothing kept are zeroed (folded top-1 combine) or null
  int y_esz;
};

}  // namespace moe
