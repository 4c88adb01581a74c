// Grouped GEMM over variable-length expert segments on the CDNA4 matrix cores.
//
//   C[r, n] = epi( sum_k A[arow(r), k] * B_s[n, k] + bias_s[n] )   for r in segment s
//
// Both operands are K-contiguous (nn.Linear weights, row-major activations), so
// every lane moves 16-byte vectors along K. The MFMA "A" operand is the weight
// tile (its rows become output columns n) and the "B" operand the activation
// tile (rows m), so each lane of a 16x16 accumulator holds four consecutive n of
// one output row: the epilogue stores 4 contiguous values per lane.
//
// grouped_gemm_kernel: a work-group computes a BM x BN output tile (BN <= 128)
// with 4 waves; K advances 128 bytes per stage through double-buffered LDS. In
// LDS each row keeps its 128 bytes as eight 16-byte columns, column c of row r
// at position c ^ (r & 7): the row-wise stores and the fragment reads (16 rows
// at one column) then hit distinct banks, where a padded row pitch leaves every
// fragment read with bank conflicts. Global loads are full 128-byte lines (8
// lanes per row), which HBM serves faster than the 64-byte row pieces the MFMA
// operand layout would need if loaded directly. Tiles of <= 64 rows (bound by
// weight bandwidth) keep two stages of loads in flight in a register ping-pong,
// 128 x 128 tiles one.
//
// grouped_gemm_pp_kernel: the eight-wave 128 x 256 tiles of long segments and
// the dense MLP. With all eight waves in the same phase of a K step, the LDS
// reads and the MFMAs of a step ran one after the other; there the two halves
// of the work-group run half a step apart, and the K steps reach three LDS
// buffers (same swizzled layout) by direct-to-LDS buffer loads.
// grouped_gemm_pp2_kernel: the same schedule on 256 x 256 and 320 x 256 tiles
// (one per segment of 129..320 rows) with 64 / 80 x 128 wave blocks, two LDS
// stages and sub-steps of 32 K.
//
// Epilogues: bias + exact GeLU rounded to the I/O dtype (first expert GEMM), or
// bias in fp32 (second GEMM and gate logits); the ping-pong tiles stage their
// output rows through LDS.
//
// Tiles come from a device tile list built on the device from the kept rows of
// each segment, by the dispatch kernel that fills the segments or by the plan
// kernel from segment offsets (no host sync). Order: segment, column tile,
// m-tile, so the m-tiles that share a weight tile are adjacent, with the extra
// segment's tiles spread evenly among them; the block index is remapped so
// adjacent tiles land on the same XCD (work-groups are dealt round-robin over the
// 8 XCDs) and share its L2.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "tile_plan.h"

namespace moe {

#define GEMM_THREADS 256
#define LDS_ROW 128      // bytes per LDS row: 128 bytes of K, 16-byte columns XOR-swizzled by row

template <typename DT>
struct Mfma;

template <>
struct Mfma<DtF16> {
  __device__ static inline float4_t op(const uint4& a, const uint4& b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b),
                                                   c, 0, 0, 0);
  }
};
template <>
struct Mfma<DtBF16> {
  __device__ static inline float4_t op(const uint4& a, const uint4& b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                    __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <>
struct Mfma<DtF32> {
  // four K=4 steps; element i of every lane's vector is the same K position
  // for both operands, so the products pair up correctly
  __device__ static inline float4_t op(const uint4& a, const uint4& b, float4_t c) {
    const float4 fa = __builtin_bit_cast(float4, a);
    const float4 fb = __builtin_bit_cast(float4, b);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.x, fb.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.y, fb.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.z, fb.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.w, fb.w, c, 0, 0, 0);
    return c;
  }
};


// Buffer descriptor over [base, base + 4 GB): raw (stride 0) dword access.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1 /* num_records: 4 GB */,
                                           0x00020000 /* dword format word of gfx9 */);
}
#define MOE_CPOL_NT 2   // cache policy bits of a buffer load: non-temporal

// Bijection on [0, total) placing consecutive tiles on one XCD.
__device__ inline int xcd_remap(int i, int total) {
  const int NX = 8;
  const int xcd = i % NX, slot = i / NX;
  const int q = total / NX, r = total % NX;
  return xcd * q + min(xcd, r) + slot;
}

template <typename BiasT>
__device__ inline float load_bias(const BiasT* b, int n);
// (global address space stated: the bias may come from a per-segment pointer table)
template <>
__device__ inline float load_bias<float>(const float* b, int n) {
  return ((const __attribute__((address_space(1))) float*)b)[n];
}
template <>
__device__ inline float load_bias<_Float16>(const _Float16* b, int n) {
  return (float)((const __attribute__((address_space(1))) _Float16*)b)[n];
}
template <>
__device__ inline float load_bias<__bf16>(const __bf16* b, int n) {
  return (float)((const __attribute__((address_space(1))) __bf16*)b)[n];
}

// Epilogue of a wave's TN x TM accumulator tiles: lane holds
// D[n = n0 + 16 i + 4 (lane / 16) + q][m = m0 + 16 j + lane % 16], q = 0..3;
// rows at or past r1 are not stored.
// With the combine folded in (p.fold_y): ftok[j] / fw[j] are the token and gate
// weight of this lane's row m0 + 16 j + lane % 16 (fold_prefetch).
template <typename DT, int EPI, typename BiasT, int TN, int TM>
__device__ inline void gemm_epilogue(const GemmParams& p, const float4_t (&acc)[TN][TM], int seg, int n0, int m0,
                                     int r1, int lane, const int (&ftok)[TM], const float (&fw)[TM]) {
  using T = typename DT::T;
  const bool extra = seg == p.nseg;
  void* Cout = extra ? p.C2 : p.C;
  const BiasT* bias = extra     ? reinterpret_cast<const BiasT*>(p.bias2)
                      : p.biasp ? reinterpret_cast<const BiasT*>(p.biasp[seg])
                      : p.bias  ? reinterpret_cast<const BiasT*>(p.bias) + (long long)seg * p.bias_stride
                                : nullptr;
#pragma unroll
  for (int i = 0; i < TN; ++i) {
    const int n = n0 + i * 16 + (lane >> 4) * 4;
    float bv[4] = {0.f, 0.f, 0.f, 0.f};
    if (bias) {
#pragma unroll
      for (int q = 0; q < 4; ++q) bv[q] = load_bias<BiasT>(bias, n + q);
    }
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int r = m0 + j * 16 + (lane & 15);
      if (r >= r1) continue;
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = acc[i][j][q] + bv[q];
      if constexpr (EPI == EPI_GELU) {
        T o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = DT::from_f(pin_f32(gelu_erf(v[q])));
        T* dst = reinterpret_cast<T*>(Cout) + (long long)r * p.N + n;
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<uint2*>(dst) = __builtin_bit_cast(uint2, o);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) dst[q] = o[q];
        }
      } else if (p.fold_y && !extra) {
        // top-1 combine: this row is one token's only kept choice; the same
        // fp32 product with the gate weight, rounded once, as the combine kernel
        const int t = ftok[j];
        const float wt = fw[j];
        T o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = DT::from_f(pin_f32(fmaf(wt, v[q], 0.f)));
        T* dst = reinterpret_cast<T*>(p.fold_y) + (long long)t * p.N + n;
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<uint2*>(dst) = __builtin_bit_cast(uint2, o);
        } else {
          *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
        }
      } else {
        float* dst = reinterpret_cast<float*>(Cout) + (long long)r * p.N + n;
        *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  }
}

// Token and gate weight of each of this lane's rows m0 + 16 j + lane % 16 for
// the folded combine, loaded before the K loop so that the epilogue does not
// wait for them (rows past r1 read nothing).
template <int TM>
__device__ inline void fold_prefetch(const GemmParams& p, bool fold, int m0, int r1, int lane, int (&ftok)[TM],
                                     float (&fw)[TM]) {
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int r = m0 + j * 16 + (lane & 15);
    ftok[j] = (fold && r < r1) ? p.fold_token[r] : 0;
  }
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int r = m0 + j * 16 + (lane & 15);
    fw[j] = (fold && r < r1) ? p.fold_w[ftok[j]] : 0.f;
  }
}

// Zeroing of p.zero_y (the layer output, before a folded combine writes its
// kept rows) and of p.zero_ws (words a later launch publishes into): work-group
// b of the launch (b = x + y * gridDim.x, over every K slice) zeroes rows b,
// b + nb, ... and its share of the words before its K loop, in 16-byte stores
// that drain while the loop waits on its loads (prefill gate 14.5 -> 13.8 us
// against zeroing after the loop).
__device__ inline void zero_rows_share(const GemmParams& p) {
  const int nb = gridDim.x * gridDim.y, b = blockIdx.y * gridDim.x + blockIdx.x;
  if (p.zero_y) {
    const int vecs = p.zero_N * p.zero_esz / 16;   // 16-byte vectors per row (N % 8 == 0)
    for (int t = b; t < p.zero_T; t += nb) {
      uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<char*>(p.zero_y) + (long long)t * p.zero_N * p.zero_esz);
      for (int c = threadIdx.x; c < vecs; c += blockDim.x) dst[c] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  if (p.zero_ws) {
    uint4* dst = reinterpret_cast<uint4*>(p.zero_ws);
    for (int c = b * blockDim.x + threadIdx.x; c < p.zero_n16; c += nb * blockDim.x) dst[c] = make_uint4(0u, 0u, 0u, 0u);
  }
}

// Epilogue through LDS for 64-column wave blocks (the ping-pong tiles): the same
// values as gemm_epilogue, but the wave first writes 128 bytes of each of its
// 16 TM rows to its own LDS area (the 16-byte columns XOR-swizzled by row) and
// then stores whole 128-byte row pieces, eight rows per store instruction,
// where the register layout of the accumulators gives 32-byte (2-byte outputs)
// or 64-byte (fp32) pieces of sixteen rows per instruction. 2-byte GeLU outputs
// take one pass (64 columns), fp32 outputs two (32 columns each). The caller
// guarantees that no wave still reads the LDS the area overlaps.
template <typename DT, int EPI, typename BiasT, int TM>
__device__ inline void gemm_epilogue_lds(const GemmParams& p, const float4_t (&acc)[4][TM], int seg, int n0, int m0,
                                         int r1, int lane, char* area) {
  using T = typename DT::T;
  constexpr bool GELU = EPI == EPI_GELU;
  static_assert(!GELU || sizeof(T) == 2, "GeLU outputs of 2 bytes");
  constexpr int ESZ = GELU ? 2 : 4;
  constexpr int CPP = 128 / ESZ;              // columns per pass: one 128-byte row piece
  constexpr int NP = 64 / CPP;
  const bool extra = seg == p.nseg;
  char* Cout = reinterpret_cast<char*>(extra ? p.C2 : p.C);
  const BiasT* bias = extra     ? reinterpret_cast<const BiasT*>(p.bias2)
                      : p.biasp ? reinterpret_cast<const BiasT*>(p.biasp[seg])
                      : p.bias  ? reinterpret_cast<const BiasT*>(p.bias) + (long long)seg * p.bias_stride
                                : nullptr;
  const int quad = lane >> 4;
#pragma unroll
  for (int ps = 0; ps < NP; ++ps) {
#pragma unroll
    for (int ii = 0; ii < 4 / NP; ++ii) {
      const int i = ps * (4 / NP) + ii;
      const int n = i * 16 + quad * 4;        // column within the wave's block
      const int byte = (n - ps * CPP) * ESZ;  // within this pass's row piece
      float bv[4] = {0.f, 0.f, 0.f, 0.f};
      if (bias) {
#pragma unroll
        for (int q = 0; q < 4; ++q) bv[q] = load_bias<BiasT>(bias, n0 + n + q);
      }
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int m = j * 16 + (lane & 15);
        char* dst = area + m * 128 + ((((byte >> 4) ^ (m & 7))) << 4) + (byte & 15);
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = acc[i][j][q] + bv[q];
        if constexpr (GELU) {
          T o[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = DT::from_f(pin_f32(gelu_erf(v[q])));
          *reinterpret_cast<uint2*>(dst) = __builtin_bit_cast(uint2, o);
        } else {
          *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
    // LDS executes a wave's accesses in order: the reads below see every lane's
    // writes above, and the next pass's writes follow these reads
#pragma unroll
    for (int r = 0; r < TM * 2; ++r) {
      const int m = r * 8 + (lane >> 3);
      const int c = lane & 7;
      const uint4 v = *reinterpret_cast<const uint4*>(area + m * 128 + ((c ^ (m & 7)) << 4));
      if (m0 + m < r1)
        *reinterpret_cast<uint4*>(Cout + ((long long)(m0 + m) * p.N + n0 + ps * CPP) * ESZ + c * 16) = v;
    }
  }
}

// Entry L of the tile list: (segment, column tile, row tile) and the segment's
// row range. False for an entry that names no tile with rows (a segment or
// column tile out of range, or rows past the segment's end), which the caller
// skips: the lists the dispatch writes hold none, and with this check no entry
// can send a work-group outside its operands.
__device__ inline bool tile_entry(const GemmParams& p, int BM, int L, int& seg, int& nt, int& mt, int& r0, int& r1) {
  const int2 d = p.tiles[L];
  seg = d.x;
  nt = d.y >> 16;
  mt = d.y & 0xffff;
  if ((unsigned)seg > (unsigned)p.nseg || nt >= p.n_ntiles) return false;
  if (seg == p.nseg) {       // the extra segment
    r0 = 0;
    r1 = p.M2;
  } else {
    r0 = p.seg_off[seg];
    r1 = p.seg_off[seg + 1];
  }
  return r0 >= 0 && r0 + mt * BM < r1;
}

// Which output tile a work-group computes: (segment, column tile, row tile) and
// the segment's row range. Returns false past the end of the tile list (or for
// an entry tile_entry rejects).
__device__ inline bool gemm_tile(const GemmParams& p, int BM, int& seg, int& nt, int& mt, int& r0, int& r1) {
  const int nmt = p.tiles ? *p.tile_count : (p.M + BM - 1) / BM;
  const int total = nmt * p.n_ntiles;
  if ((int)blockIdx.x >= total) return false;
  const int L = xcd_remap(blockIdx.x, total);
  if (p.tiles) {
    if (!tile_entry(p, BM, L, seg, nt, mt, r0, r1)) return false;
  } else {
    seg = 0;
    nt = L / nmt;
    mt = L - nt * nmt;
    r0 = 0;
    r1 = p.M;
  }
  return true;
}

// NTH threads (4 or 8 waves, laid out WM x WN over the tile); DEPTH stages of
// global loads in flight; the launch bound asks for two waves per SIMD when the
// registers of two stages or of eight waves must fit. WNT: the expert tiles load
// their weights non-temporally (the host sets it when every weight tile is read
// by at most two row tiles). PERS: a grid of resident work-groups walks the
// tile list, work-group (x, j) on XCD x (x = blockIdx % 8) taking tiles j,
// j + gridDim / 8, ... of XCD x's contiguous share of the list (the order
// xcd_remap gives one tile per work-group); the residual layer's second GEMM,
// whose list mixes the dense MLP's tiles with the experts', runs 443 -> 429 us
// so, the other weight-streaming launches measured unchanged.
template <typename DT, int BM, int BN, int EPI, typename BiasT, int DEPTH, int NTH, bool WNT, bool PERS = false>
__global__ __launch_bounds__(NTH, (DEPTH > 1 || NTH > 256) ? 2 : 1) void grouped_gemm_kernel(GemmParams p) {
  using T = typename DT::T;
  constexpr int NW = NTH / 64;
  constexpr int WM = (BM >= 64) ? 2 : 1;
  constexpr int WN = NW / WM;
  constexpr int TN = BN / WN / 16;
  constexpr int TM = BM / WM / 16;
  static_assert(TN >= 1 && TM >= 1 && TN * WN * 16 == BN && TM * WM * 16 == BM, "tile does not split over the waves");
  constexpr int ACH = (BM * 8 + NTH - 1) / NTH;   // 16-byte chunks per thread
  constexpr int BCH = (BN * 8) / NTH;
  static_assert(BCH >= 1 && BCH * NTH == BN * 8, "BN does not split over the threads");
  constexpr int STAGE = (BN + BM) * LDS_ROW;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  int it_L = 0, it_end = 0, it_step = 1;   // PERS: this work-group's tiles it_L, it_L + it_step, ... < it_end
  if constexpr (PERS) {
    const int total = *p.tile_count * p.n_ntiles;
    const int xcd = blockIdx.x & 7, g8 = gridDim.x >> 3;   // (the host launches a multiple of 8)
    const int q = total >> 3, rr = total & 7;
    const int start = xcd * q + min(xcd, rr);
    it_L = start + (int)(blockIdx.x >> 3);
    it_end = start + q + (xcd < rr ? 1 : 0);
    it_step = g8;
  }
  for (;;) {
  // ---- which tile
  int seg, nt, mt, r0, r1;
  if constexpr (PERS) {
    if (it_L >= it_end) return;
    if (!tile_entry(p, BM, it_L, seg, nt, mt, r0, r1)) {
      it_L += it_step;
      continue;
    }
  } else {
    if (!gemm_tile(p, BM, seg, nt, mt, r0, r1)) {
      if (p.zero_y || p.zero_ws) zero_rows_share(p);
      return;
    }
  }
  const int m0 = r0 + mt * BM;        // first row-space row of the tile
  const bool extra = seg == p.nseg;   // the extra segment: its own operands, rows index A2 directly

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_n = wave % WN;
  const int wave_m = wave / WN;
  int ftok[TM];
  float fw[TM];
  fold_prefetch<TM>(p, EPI == EPI_F32 && p.fold_y && !extra, m0 + wave_m * TM * 16, r1, lane, ftok, fw);

  // ---- per-thread global source rows. LDS layout: row r of a stage holds its 128
  // bytes of K as eight 16-byte columns, column c stored at position c ^ (r & 7),
  // so both the row-wise stores (8 lanes per row) and the fragment reads (16 rows
  // at one column) spread over all banks. When BM * 8 is not a multiple of the
  // thread count, the threads past the tile load a valid duplicate and skip the
  // LDS store, so every load is unconditional and all stay in flight together.
  const char* a_src[ACH];
  int a_dst[ACH];
  bool a_own[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    a_own[i] = tid + i * NTH < BM * 8;
    const int c = min(tid + i * NTH, BM * 8 - 1);
    const int row = c >> 3, col = c & 7;
    int r = m0 + row;
    if (r >= r1) r = r1 - 1;
    const long long arow = (p.a_rows && !extra) ? (long long)p.a_rows[r] : (long long)r;
    a_src[i] = reinterpret_cast<const char*>(extra ? p.A2 : p.A) + (arow * p.K) * (long long)sizeof(T) + col * 16;
    a_dst[i] = BN * LDS_ROW + row * LDS_ROW + ((col ^ (row & 7)) * 16);
  }
  const char* b_src[BCH];
  int b_dst[BCH];
  const char* bbase = extra    ? reinterpret_cast<const char*>(p.B2)
                      : p.Bp ? reinterpret_cast<const char*>(p.Bp[seg])
                             : reinterpret_cast<const char*>(p.B) + (long long)seg * p.b_stride * (long long)sizeof(T);
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int c = tid + i * NTH;
    const int row = c >> 3, col = c & 7;
    const long long n = (long long)nt * BN + row;
    b_src[i] = bbase + n * p.K * (long long)sizeof(T) + col * 16;
    b_dst[i] = row * LDS_ROW + ((col ^ (row & 7)) * 16);
  }

  float4_t acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  if constexpr (!PERS) {
    if (p.zero_y || p.zero_ws) zero_rows_share(p);
  }
  int nk = (int)(((long long)p.K * sizeof(T)) / 128);
  if constexpr (std::is_same<BiasT, float>::value) {
    if (p.ksplit > 1) {   // this work-group's slice of K (the host makes nk divisible)
      nk /= p.ksplit;
      const long long k0 = (long long)blockIdx.y * nk * 128;
#pragma unroll
      for (int i = 0; i < ACH; ++i) a_src[i] += k0;
#pragma unroll
      for (int i = 0; i < BCH; ++i) b_src[i] += k0;
    }
  }
  const int frag_row = lane & 15;
  // 16-byte column of the lane's fragment in k-block kb (0 or 1), swizzled for its row
  const int frag_c0 = (((lane >> 4)) ^ (frag_row & 7)) * 16;
  const int frag_c1 = ((4 + (lane >> 4)) ^ (frag_row & 7)) * 16;

// global -> registers RA/RB for stage KS (all loads of the stage in flight together).
// The operands are global memory: said so, the loads are global_load (a flat
// load would also count against lgkmcnt, and every LDS wait would then wait for
// the stage in flight too). W_: the weights are loaded non-temporally.
#define GEMM_GLOAD(RA, RB, KS)                                                           \
  {                                                                                      \
    const long long off_ = (long long)(KS) * 128;                                        \
    _Pragma("unroll") for (int i = 0; i < ACH; ++i) RA[i] =                              \
        *(const __attribute__((address_space(1))) u32x4_t*)(a_src[i] + off_);           \
    _Pragma("unroll") for (int i = 0; i < BCH; ++i) {                                    \
      const __attribute__((address_space(1))) u32x4_t* q_ =                              \
          (const __attribute__((address_space(1))) u32x4_t*)(b_src[i] + off_);           \
      if constexpr (W_) RB[i] = __builtin_nontemporal_load(q_);                          \
      else RB[i] = *q_;                                                                  \
    }                                                                                    \
  }
// registers RA/RB -> LDS buffer BUF
#define GEMM_LSTORE(RA, RB, BUF)                                                         \
  {                                                                                      \
    char* base_ = smem + (BUF) * STAGE;                                                  \
    _Pragma("unroll") for (int i = 0; i < ACH; ++i) if (a_own[i])                        \
        *reinterpret_cast<u32x4_t*>(base_ + a_dst[i]) = RA[i];                           \
    _Pragma("unroll") for (int i = 0; i < BCH; ++i)                                      \
        *reinterpret_cast<u32x4_t*>(base_ + b_dst[i]) = RB[i];                           \
  }
// MFMAs over the stage in LDS buffer BUF
#define GEMM_MATH(BUF)                                                                   \
  {                                                                                      \
    const char* sb = smem + (BUF) * STAGE;                                               \
    const char* sa = sb + BN * LDS_ROW;                                                  \
    _Pragma("unroll") for (int kb = 0; kb < 2; ++kb) {                                   \
      uint4 fa[TN], fb[TM];                                                              \
      _Pragma("unroll") for (int i = 0; i < TN; ++i)                                     \
        fa[i] = *reinterpret_cast<const uint4*>(sb + (wave_n * TN * 16 + i * 16 + frag_row) * LDS_ROW + \
                                                (kb ? frag_c1 : frag_c0));               \
      _Pragma("unroll") for (int j = 0; j < TM; ++j)                                     \
        fb[j] = *reinterpret_cast<const uint4*>(sa + (wave_m * TM * 16 + j * 16 + frag_row) * LDS_ROW + \
                                                (kb ? frag_c1 : frag_c0));               \
      _Pragma("unroll") for (int i = 0; i < TN; ++i)                                     \
        _Pragma("unroll") for (int j = 0; j < TM; ++j) acc[i][j] = Mfma<DT>::op(fa[i], fb[j], acc[i][j]); \
    }                                                                                    \
  }
#define GEMM_SB __builtin_amdgcn_sched_barrier(0)

  // The K loop, with or without non-temporal weight loads. With WNT the expert
  // tiles stream their weights (each weight tile is read by one or two row tiles)
  // and the extra segment's tiles, which all read the same dense weights, keep
  // them cached: two copies of the loop, one per choice.
  auto k_loop = [&](auto stream_tag) {
    constexpr bool W_ = decltype(stream_tag)::value;
    if constexpr (DEPTH == 1) {
      // one stage in flight: stage ks + 1 loads while stage ks is multiplied
      u32x4_t ra[ACH], rb[BCH];
      GEMM_GLOAD(ra, rb, 0);
      GEMM_LSTORE(ra, rb, 0);
      __syncthreads();
      for (int ks = 0; ks < nk; ++ks) {
        const int buf = ks & 1;
        if (ks + 1 < nk) GEMM_GLOAD(ra, rb, ks + 1);
        GEMM_MATH(buf);
        if (ks + 1 < nk) GEMM_LSTORE(ra, rb, buf ^ 1);
        __syncthreads();
      }
    } else {
      // two stages in flight (register ping-pong): while stage c is multiplied from
      // LDS, stages c + 1 and c + 2 are loading. Stage c sits in LDS buffer c & 1;
      // stage c + 1 in register set (c + 1) & 1. The steady loop's loads are
      // unconditional so the wait for one register set leaves the other in flight.
      u32x4_t ra0[ACH], rb0[BCH], ra1[ACH], rb1[BCH];
      GEMM_GLOAD(ra0, rb0, 0);
      GEMM_SB;
      if (nk > 1) GEMM_GLOAD(ra1, rb1, 1);
      GEMM_SB;
      GEMM_LSTORE(ra0, rb0, 0);
      if (nk > 2) GEMM_GLOAD(ra0, rb0, 2);
      GEMM_SB;
      __syncthreads();
      int c = 0;
      for (; c + 4 < nk; c += 2) {   // LDS buf 0 = stage c, set 1 = stage c + 1, set 0 = stage c + 2
        GEMM_MATH(0);
        GEMM_LSTORE(ra1, rb1, 1);
        GEMM_GLOAD(ra1, rb1, c + 3);
        GEMM_SB;
        __syncthreads();
        GEMM_MATH(1);
        GEMM_LSTORE(ra0, rb0, 0);
        GEMM_GLOAD(ra0, rb0, c + 4);
        GEMM_SB;
        __syncthreads();
      }
      for (; c < nk; ++c) {          // the last (at most four) stages
        if ((c & 1) == 0) {
          GEMM_MATH(0);
          if (c + 1 < nk) {
            GEMM_LSTORE(ra1, rb1, 1);
            if (c + 3 < nk) GEMM_GLOAD(ra1, rb1, c + 3);
          }
        } else {
          GEMM_MATH(1);
          if (c + 1 < nk) {
            GEMM_LSTORE(ra0, rb0, 0);
            if (c + 3 < nk) GEMM_GLOAD(ra0, rb0, c + 3);
          }
        }
        __syncthreads();
      }
    }
  };
  if constexpr (WNT) {
    if (extra) k_loop(std::false_type{});
    else k_loop(std::true_type{});
  } else {
    k_loop(std::false_type{});
  }
#undef GEMM_GLOAD
#undef GEMM_LSTORE
#undef GEMM_MATH
#undef GEMM_SB

  if constexpr (std::is_same<BiasT, float>::value) {
    if (p.ksplit > 1) {   // partial sums of this slice; the bias goes with slice 0
      GemmParams q = p;
      q.C = reinterpret_cast<float*>(p.C) + (long long)blockIdx.y * p.c_split;
      if (blockIdx.y != 0) q.bias = nullptr;
      gemm_epilogue<DT, EPI, BiasT, TN, TM>(q, acc, seg, nt * BN + wave_n * TN * 16, m0 + wave_m * TM * 16, r1, lane,
                                            ftok, fw);
      return;
    }
  }
  gemm_epilogue<DT, EPI, BiasT, TN, TM>(p, acc, seg, nt * BN + wave_n * TN * 16, m0 + wave_m * TM * 16, r1, lane, ftok,
                                        fw);
  if constexpr (!PERS) return;
  it_L += it_step;
  __syncthreads();   // (every wave's last fragment reads are done before the next tile's LDS stores)
  }
}


// s_waitcnt immediates (gfx9 layout: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8): wait for vmcnt <= n only, and for lgkmcnt == 0 only
#define MOE_VMCNT(n) ((((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8)))
#define MOE_LGKM0 0xC07F

// Eight-wave 128 x 256 tiles for segments of 65..256 rows and the dense MLP,
// where the matrix cores set the pace. Ping-pong schedule: waves 0-3 (the
// tile's upper rows) and waves 4-7 (lower rows) run half a K step apart, so on
// every SIMD one wave multiplies while the other reads its fragments of the next
// step from LDS. The K steps reach LDS by direct-to-LDS buffer loads (no
// registers, no LDS store instructions) into three buffers, issued two steps
// ahead. Every wave passes 2 nk + 2 barriers. Measured on the 24B-share expert
// GEMMs (16 experts, H = 8192, F = 32768) with this kernel at 160 x 256 (two
// tiles per 320-row segment, before the 320 x 256 kernel took those): 2.74 /
// 2.67 ms per launch; 2.91 / 2.74 ms with the steps staged through registers
// and LDS stores, 3.39 / 3.37 ms with all eight waves in the same phase.
template <typename DT, int BM, int EPI, typename BiasT, bool WNT>
__global__ __launch_bounds__(512, 2) void grouped_gemm_pp_kernel(GemmParams p) {
  using T = typename DT::T;
  constexpr int BN = 256, WN = 4;
  constexpr int TN = 4, TM = BM / 32;
  constexpr int HB = BM / 2;
  constexpr int NCG = 16 + HB / 8;            // 8-row chunks of one group's half of a K step
  constexpr int NCH = NCG / 4;                // chunks per wave
  static_assert(NCH * 4 == NCG, "a group's chunks split evenly over its four waves");
  constexpr int STAGE = (BN + BM) * LDS_ROW;
  __shared__ __attribute__((aligned(16))) char smem[3 * STAGE];

  int seg, nt, mt, r0, r1;
  if (!gemm_tile(p, BM, seg, nt, mt, r0, r1)) return;
  const int m0 = r0 + mt * BM;
  const bool extra = seg == p.nseg;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_n = wave % WN;
  const int g = wave / WN;
  const bool fold = EPI == EPI_F32 && p.fold_y && !extra;
  int ftok[TM];
  float fw[TM];
  fold_prefetch<TM>(p, fold, m0 + g * TM * 16, r1, lane, ftok, fw);

  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(extra ? p.A2 : p.A);
  const char* bbase = extra    ? reinterpret_cast<const char*>(p.B2)
                      : p.Bp ? reinterpret_cast<const char*>(p.Bp[seg])
                             : reinterpret_cast<const char*>(p.B) + (long long)seg * p.b_stride * (long long)sizeof(T);
  const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(bbase + (long long)nt * BN * p.K * (long long)sizeof(T));
  // chunk i of this wave: c = wave_n + 4 i; c < 16 weight rows 128 g + 8 c, else
  // activation rows HB g + 8 (c - 16). A wave's LDS DMA writes
  // 64 x 16 bytes contiguously: lane l lands in row l / 8 of the chunk, 16-byte
  // slot l % 8, so it loads column (l % 8) ^ (l / 8) (the XOR swizzle).
  const int col = ((lane & 7) ^ (lane >> 3)) * 16;
  unsigned voff[NCH];
  int ldst[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = wave_n + 4 * i;
    if (i < 4) {
      const int row = g * 128 + c * 8 + (lane >> 3);
      voff[i] = (unsigned)(row * p.K * (int)sizeof(T)) + col;
      ldst[i] = (g * 128 + c * 8) * LDS_ROW;
    } else {
      int r = m0 + g * HB + (c - 16) * 8 + (lane >> 3);
      if (r >= r1) r = r1 - 1;
      const long long arow = (p.a_rows && !extra) ? (long long)p.a_rows[r] : (long long)r;
      voff[i] = (unsigned)(arow * p.K * (long long)sizeof(T)) + col;
      ldst[i] = BN * LDS_ROW + (g * HB + (c - 16) * 8) * LDS_ROW;
    }
  }

  float4_t acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = (int)(((long long)p.K * sizeof(T)) / 128);
  const int frag_row = lane & 15;
  const int frag_c0 = (((lane >> 4)) ^ (frag_row & 7)) * 16;
  const int frag_c1 = ((4 + (lane >> 4)) ^ (frag_row & 7)) * 16;

#define DM_ISSUE(KS, BUF)                                                                \
  {                                                                                      \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                        \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc,                                   \
          (__attribute__((address_space(3))) void*)(smem + (BUF) * STAGE + ldst[i]), 16,  \
          (int)voff[i], (KS) * 128, 0, W_ ? MOE_CPOL_NT : 0);                            \
    _Pragma("unroll") for (int i = 4; i < NCH; ++i)                                      \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc,                                   \
          (__attribute__((address_space(3))) void*)(smem + (BUF) * STAGE + ldst[i]), 16,  \
          (int)voff[i], (KS) * 128, 0, 0);                                               \
  }
#define DM_FRAGS(BUF)                                                                    \
  {                                                                                      \
    const char* sb = smem + (BUF) * STAGE;                                               \
    const char* sa = sb + BN * LDS_ROW;                                                  \
    _Pragma("unroll") for (int kb = 0; kb < 2; ++kb) {                                   \
      _Pragma("unroll") for (int i = 0; i < TN; ++i)                                     \
        fa[kb][i] = *reinterpret_cast<const uint4*>(sb + (wave_n * TN * 16 + i * 16 + frag_row) * LDS_ROW + \
                                                    (kb ? frag_c1 : frag_c0));           \
      _Pragma("unroll") for (int j = 0; j < TM; ++j)                                     \
        fb[kb][j] = *reinterpret_cast<const uint4*>(sa + (g * TM * 16 + j * 16 + frag_row) * LDS_ROW + \
                                                    (kb ? frag_c1 : frag_c0));           \
    }                                                                                    \
  }
#define DM_MATH                                                                          \
  {                                                                                      \
    _Pragma("unroll") for (int kb = 0; kb < 2; ++kb)                                     \
      _Pragma("unroll") for (int i = 0; i < TN; ++i)                                     \
        _Pragma("unroll") for (int j = 0; j < TM; ++j)                                   \
          acc[i][j] = Mfma<DT>::op(fa[kb][i], fb[kb][j], acc[i][j]);                     \
  }
// A barrier nothing moves across. The waits that make a K step's direct-to-LDS
// loads visible are explicit (s_waitcnt vmcnt before the barrier); the compiler
// adds its own vmcnt(0) before the fragment reads while any such load is in
// flight, which only shortens the lead of the loads to one multiply phase.
#define DM_BAR                                                                           \
  {                                                                                      \
    __builtin_amdgcn_sched_barrier(0);                                                   \
    asm volatile("" ::: "memory");                                                       \
    __builtin_amdgcn_s_barrier();                                                        \
    asm volatile("" ::: "memory");                                                       \
    __builtin_amdgcn_sched_barrier(0);                                                   \
  }

  auto k_loop = [&](auto stream_tag) {
    constexpr bool W_ = decltype(stream_tag)::value;
    uint4 fa[2][TN], fb[2][TM];
    // steps 0 and 1 into LDS buffers 0 and 1; step 0 complete before the barrier
    DM_ISSUE(0, 0);
    if (nk > 1) {
      DM_ISSUE(1, 1);
      __builtin_amdgcn_s_waitcnt(MOE_VMCNT(NCH));
    } else {
      __builtin_amdgcn_s_waitcnt(MOE_VMCNT(0));
    }
    DM_BAR;
    // Group 1 passes one extra barrier first and group 0 one extra at the end:
    // barrier n of a wave then pairs with barrier n of the other group, so one
    // group's memory phase runs beside the other's multiply phase. Step s lives
    // in buffer s % 3. Memory phase of step s: fragments of step s, then the DMA
    // of step s + 2 into buffer (s + 2) % 3 (both groups finished reading step
    // s - 1 there before the previous barrier), then wait until this wave's DMA
    // of step s + 1 has landed; a reader of step s + 1 passes a barrier after
    // both groups' waits.
    if (g == 1) DM_BAR;
    for (int s = 0; s < nk; ++s) {
      DM_FRAGS(s % 3);
      if (s + 2 < nk) {
        DM_ISSUE(s + 2, (s + 2) % 3);
        __builtin_amdgcn_s_waitcnt(MOE_VMCNT(NCH));
      } else {
        __builtin_amdgcn_s_waitcnt(MOE_VMCNT(0));
      }
      __builtin_amdgcn_s_waitcnt(MOE_LGKM0);
      DM_BAR;
      DM_MATH;
      DM_BAR;
    }
    if (g == 0) DM_BAR;
  };
  if constexpr (WNT) {
    if (extra) k_loop(std::false_type{});
    else k_loop(std::true_type{});
  } else {
    k_loop(std::false_type{});
  }
#undef DM_ISSUE
#undef DM_FRAGS
#undef DM_MATH
#undef DM_BAR
  if (fold) {
    gemm_epilogue<DT, EPI, BiasT, TN, TM>(p, acc, seg, nt * BN + wave_n * TN * 16, m0 + g * TM * 16, r1, lane, ftok,
                                          fw);
  } else if constexpr (EPI != EPI_GELU || sizeof(T) == 2) {
    // every wave is past its last fragment read of the K loop's buffers before
    // any wave overwrites them with its output rows (8 x 16 TM rows of 128 B)
    static_assert(8 * TM * 16 * 128 <= 3 * STAGE, "output blocks fit the K-step buffers");
    __syncthreads();
    gemm_epilogue_lds<DT, EPI, BiasT, TM>(p, acc, seg, nt * BN + wave_n * TN * 16, m0 + g * TM * 16, r1, lane,
                                          smem + wave * (TM * 16 * 128));
  } else {
    gemm_epilogue<DT, EPI, BiasT, TN, TM>(p, acc, seg, nt * BN + wave_n * TN * 16, m0 + g * TM * 16, r1, lane, ftok,
                                          fw);
  }
}

// Eight-wave BM x 256 tiles, BM = 256 or 320, for segments of 129..320 rows
// (the expert GEMMs of a capacity-256 or -320 share): one work-group covers a
// whole segment, so each weight tile is read once, and each wave holds a
// BM / 4 x 128 block (at BM = 320: 160 accumulator VGPRs), which at BM = 320
// reads 28 % fewer LDS fragment bytes per multiply than the 80 x 64 blocks of
// 160 x 256 tiles. Two LDS stages (256 weight rows and BM activation rows of
// 128 bytes of K, same swizzle; 73.7 KB at BM = 320) in two separate
// arrays, so that the compiler sees which stage a direct-to-LDS load writes and
// which one a fragment read reads, and adds no wait of its own between them.
// Waves 0-3 (rows 0 .. BM / 2 - 1) and 4-7 (the rest) run half a phase apart on
// sub-steps of 32 K (one sub-step's fragments, 48 / 52 VGPRs at BM = 256 / 320,
// fit beside the accumulators): on every SIMD one wave multiplies while the other reads its
// fragments. Each group loads its half of a stage (its BM / 2 activation rows
// and 128 of the weight rows) in its memory phase of sub-step 2 s, after the
// barrier that frees the buffer, and waits for its loads (vmcnt 0) right before
// the barrier after which stage s + 1 is first read: group 0 at the end of its
// multiply phase of sub-step 2 s + 1, group 1 at the end of its memory phase
// of that sub-step (3.5 and 2.5 phases after the issue). No load is then in
// flight at the loop's back edge, where the compiler waits for all of them.
template <typename DT, int BM, int EPI, typename BiasT, bool WNT>
__global__ __launch_bounds__(512, 2) void grouped_gemm_pp2_kernel(GemmParams p) {
  using T = typename DT::T;
  static_assert(BM == 256 || BM == 320, "256- or 320-row tiles");
  constexpr int BN = 256;
  constexpr int HB = BM / 2, WB = BM / 4;      // rows of a group, of a wave's block
  constexpr int TN = 8, TM = WB / 16;
  constexpr int NCH = (16 + HB / 8) / 4;       // 8-row chunks per wave per stage: 16 weight + HB / 8 activation per group
  constexpr int STAGE = (BN + BM) * LDS_ROW;
  __shared__ __attribute__((aligned(16))) char lds0[STAGE];
  __shared__ __attribute__((aligned(16))) char lds1[STAGE];

  int seg, nt, mt, r0, r1;
  if (!gemm_tile(p, BM, seg, nt, mt, r0, r1)) return;
  const int m0 = r0 + mt * BM;
  const bool extra = seg == p.nseg;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave >> 2;          // row half: activation rows HB g ..
  const int wm = (wave >> 1) & 1;   // WB-row block within the half
  const int wn = wave & 1;          // 128-column block
  const int wl = wave & 3;          // wave within its group (load chunks)
  const int mw = m0 + g * HB + wm * WB;   // first row of this wave's block
  const bool fold = EPI == EPI_F32 && p.fold_y && !extra;
  int ftok[TM];
  float fw[TM];
  fold_prefetch<TM>(p, fold, mw, r1, lane, ftok, fw);

  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(extra ? p.A2 : p.A);
  const char* bbase = extra    ? reinterpret_cast<const char*>(p.B2)
                      : p.Bp ? reinterpret_cast<const char*>(p.Bp[seg])
                             : reinterpret_cast<const char*>(p.B) + (long long)seg * p.b_stride * (long long)sizeof(T);
  const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(bbase + (long long)nt * BN * p.K * (long long)sizeof(T));
  // chunk i of this wave: c = wl + 4 i; c < 16: weight rows 128 g + 8 c; else
  // activation rows HB g + 8 (c - 16) (clamped into the segment). Lane l lands
  // in row l / 8 of the chunk, 16-byte slot l % 8, so it loads column
  // (l % 8) ^ (l / 8) (the XOR swizzle).
  const int col = ((lane & 7) ^ (lane >> 3)) * 16;
  unsigned voff[NCH];
  int ldst[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = wl + 4 * i;
    if (i < 4) {
      const int row = g * 128 + c * 8 + (lane >> 3);
      voff[i] = (unsigned)(row * p.K * (int)sizeof(T)) + col;
      ldst[i] = (g * 128 + c * 8) * LDS_ROW;
    } else {
      int r = m0 + g * HB + (c - 16) * 8 + (lane >> 3);
      if (r >= r1) r = r1 - 1;
      const long long arow = (p.a_rows && !extra) ? (long long)p.a_rows[r] : (long long)r;
      voff[i] = (unsigned)(arow * p.K * (long long)sizeof(T)) + col;
      ldst[i] = BN * LDS_ROW + (g * HB + (c - 16) * 8) * LDS_ROW;
    }
  }

  float4_t acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = (int)(((long long)p.K * sizeof(T)) / 128);
  const int frag_row = lane & 15;
  const int frag_c0 = (((lane >> 4)) ^ (frag_row & 7)) * 16;
  const int frag_c1 = ((4 + (lane >> 4)) ^ (frag_row & 7)) * 16;

#define P3_ISSUE(KS, BUF)                                                                \
  {                                                                                      \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                        \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc,                                   \
          (__attribute__((address_space(3))) void*)((BUF) + ldst[i]), 16, (int)voff[i],  \
          (KS) * 128, 0, W_ ? MOE_CPOL_NT : 0);                                          \
    _Pragma("unroll") for (int i = 4; i < NCH; ++i)                                      \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc,                                   \
          (__attribute__((address_space(3))) void*)((BUF) + ldst[i]), 16, (int)voff[i],  \
          (KS) * 128, 0, 0);                                                             \
  }
#define P3_FRAGS(BUF, KB)                                                                \
  {                                                                                      \
    const int fc_ = (KB) ? frag_c1 : frag_c0;                                            \
    _Pragma("unroll") for (int i = 0; i < TN; ++i)                                       \
      fa[i] = *reinterpret_cast<const uint4*>((BUF) + (wn * 128 + i * 16 + frag_row) * LDS_ROW + fc_); \
    _Pragma("unroll") for (int j = 0; j < TM; ++j)                                       \
      fb[j] = *reinterpret_cast<const uint4*>((BUF) + (BN + g * HB + wm * WB + j * 16 + frag_row) * LDS_ROW + fc_); \
  }
#define P3_MATH                                                                          \
  {                                                                                      \
    _Pragma("unroll") for (int i = 0; i < TN; ++i)                                       \
      _Pragma("unroll") for (int j = 0; j < TM; ++j)                                     \
        acc[i][j] = Mfma<DT>::op(fa[i], fb[j], acc[i][j]);                               \
  }
#define P3_BAR                                                                           \
  {                                                                                      \
    __builtin_amdgcn_sched_barrier(0);                                                   \
    asm volatile("" ::: "memory");                                                       \
    __builtin_amdgcn_s_barrier();                                                        \
    asm volatile("" ::: "memory");                                                       \
    __builtin_amdgcn_sched_barrier(0);                                                   \
  }
// one sub-step (stage S, K half KB) read from BUF; NBUF is the other stage
#define P3_SUB(S, KB, BUF, NBUF)                                                         \
  {                                                                                      \
    P3_FRAGS(BUF, KB);                                                                   \
    if ((KB) == 0 && (S) + 1 < nk) P3_ISSUE((S) + 1, NBUF);                              \
    if (g == 1 && (KB) == 1 && (S) + 1 < nk) __builtin_amdgcn_s_waitcnt(MOE_VMCNT(0));   \
    __builtin_amdgcn_s_waitcnt(MOE_LGKM0);                                               \
    P3_BAR;                                                                              \
    P3_MATH;                                                                             \
    if (g == 0 && (KB) == 1 && (S) + 1 < nk) __builtin_amdgcn_s_waitcnt(MOE_VMCNT(0));   \
    P3_BAR;                                                                              \
  }

  auto k_loop = [&](auto stream_tag) {
    constexpr bool W_ = decltype(stream_tag)::value;
    uint4 fa[TN], fb[TM];
    // stage 0 (both groups' halves) complete before the first barrier
    P3_ISSUE(0, lds0);
    __builtin_amdgcn_s_waitcnt(MOE_VMCNT(0));
    P3_BAR;
    if (g == 1) P3_BAR;
    for (int s = 0; s < nk; s += 2) {
      P3_SUB(s, 0, lds0, lds1);
      P3_SUB(s, 1, lds0, lds1);
      if (s + 1 < nk) {
        P3_SUB(s + 1, 0, lds1, lds0);
        P3_SUB(s + 1, 1, lds1, lds0);
      }
    }
    if (g == 0) P3_BAR;
  };
  if constexpr (WNT) {
    if (extra) k_loop(std::false_type{});
    else k_loop(std::true_type{});
  } else {
    k_loop(std::false_type{});
  }
#undef P3_ISSUE
#undef P3_FRAGS
#undef P3_MATH
#undef P3_BAR
#undef P3_SUB
  const int n0 = nt * BN + wn * 128;
  if (fold) {
    gemm_epilogue<DT, EPI, BiasT, TN, TM>(p, acc, seg, n0, mw, r1, lane, ftok, fw);
  } else if constexpr (EPI != EPI_GELU || sizeof(T) == 2) {
    // every wave is past its last fragment read before any wave overwrites the
    // stages with its output rows (waves 0-3 in the first array, 4-7 in the
    // second, 16 TM rows of 128 bytes each), 64 columns at a time
    static_assert(4 * TM * 16 * 128 <= STAGE, "output blocks fit a stage");
    __syncthreads();
    char* area = (g == 0 ? lds0 : lds1) + wl * (TM * 16 * 128);
    gemm_epilogue_lds<DT, EPI, BiasT, TM>(p, reinterpret_cast<const float4_t(&)[4][TM]>(acc[0]), seg, n0, mw, r1,
                                          lane, area);
    gemm_epilogue_lds<DT, EPI, BiasT, TM>(p, reinterpret_cast<const float4_t(&)[4][TM]>(acc[4]), seg, n0 + 64, mw,
                                          r1, lane, area);
  } else {
    gemm_epilogue<DT, EPI, BiasT, TN, TM>(p, acc, seg, n0, mw, r1, lane, ftok, fw);
  }
}

// ---------------------------------------------------------------- plan kernel
// Tile lists of the two expert GEMMs from the segment offsets (one block; the
// layer forward builds them inside its dispatch kernel instead).
__global__ __launch_bounds__(1024) void gemm_plan_kernel(const int* __restrict__ seg_off, int nseg, TilePlanArgs a) {
  __shared__ int lds[tile_plan_lds_ints(1024)];
  const int tid = threadIdx.x;
  const int rows = (tid < nseg) ? seg_off[tid + 1] - seg_off[tid] : 0;
  tile_plan_body<1024>(rows, nseg, a, lds);
}

hipError_t launch_gemm_plan(const int* seg_off, int nseg, const TilePlanArgs& a, hipStream_t s) {
  if (nseg > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_plan_kernel, dim3(1), dim3(1024), 0, s, seg_off, nseg, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- dispatch on shape
struct LaunchEv {
  hipEvent_t start, stop;
};

// Work-groups of a kernel resident on the whole device at once, from its
// registers and LDS and gfx950's limits (512 registers per lane of a SIMD in
// granules of 8, at most 8 waves per SIMD, 4 SIMDs and 160 KB of LDS per CU),
// rounded down to a multiple of 8; cached per kernel and device; 0 if unknown.
template <auto KERNEL>
static int resident_workgroups(int nth) {
  static int cache[64];   // per device (one array per kernel: KERNEL is a template argument)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    hipFuncAttributes fa;
    int cus = 0;
    if (hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(KERNEL)) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || fa.numRegs <= 0 ||
        cus < 1)
      return 0;
    const int regs = (fa.numRegs + 7) / 8 * 8;
    const int waves_simd = std::min(8, 512 / regs);
    const int by_waves = waves_simd * 4 / ((nth + 63) / 64);
    const int by_lds = fa.sharedSizeBytes > 0 ? (int)((160 * 1024) / fa.sharedSizeBytes) : 64;
    const int per_cu = std::min(by_waves, by_lds);
    if (per_cu < 1) return 0;
    cache[dev] = per_cu * cus / 8 * 8;
  }
  return cache[dev];
}

template <typename DT, int BM, int BN, int EPI, typename BiasT>
static void launch_t(const GemmParams& p, int grid, hipStream_t s, LaunchEv ev) {
  constexpr int NTH = BN == 256 ? 512 : GEMM_THREADS;
  constexpr int DEPTH = BM <= 64 ? 2 : 1;
  const dim3 g(grid, p.ksplit > 1 ? p.ksplit : 1);
  if constexpr (BN == 256) {
    // (launch_grouped_gemm refuses float-bias 256-column tiles and operands
    // beyond 32-bit offsets before getting here)
    if constexpr (!std::is_same<BiasT, float>::value) {
      if constexpr (BM == 256 || BM == 320) {
        if (p.stream_w)
          MOE_LAUNCH((grouped_gemm_pp2_kernel<DT, BM, EPI, BiasT, true>), g, dim3(NTH), 0, s, ev.start, ev.stop, p);
        else
          MOE_LAUNCH((grouped_gemm_pp2_kernel<DT, BM, EPI, BiasT, false>), g, dim3(NTH), 0, s, ev.start, ev.stop, p);
      } else {
        if (p.stream_w)
          MOE_LAUNCH((grouped_gemm_pp_kernel<DT, BM, EPI, BiasT, true>), g, dim3(NTH), 0, s, ev.start, ev.stop, p);
        else
          MOE_LAUNCH((grouped_gemm_pp_kernel<DT, BM, EPI, BiasT, false>), g, dim3(NTH), 0, s, ev.start, ev.stop, p);
      }
    }
  } else {
    // (float bias: the gate's logits, whose weight tile every token tile reads)
    if constexpr (!std::is_same<BiasT, float>::value) {
      if (p.stream_w) {   // expert weights read by one or two row tiles each
        if constexpr (DEPTH == 2 && NTH == 256) {
          if (p.tiles && p.ksplit <= 1) {   // resident work-groups walking the tile list
            constexpr auto kern = grouped_gemm_kernel<DT, BM, BN, EPI, BiasT, DEPTH, NTH, true, true>;
            const int slots = resident_workgroups<kern>(NTH);
            if (slots >= 8) {
              const int gp = grid < slots ? (grid + 7) / 8 * 8 : slots;
              MOE_LAUNCH(kern, dim3(gp), dim3(NTH), 0, s, ev.start, ev.stop, p);
              return;
            }
          }
        }
        MOE_LAUNCH((grouped_gemm_kernel<DT, BM, BN, EPI, BiasT, DEPTH, NTH, true>), g, dim3(NTH), 0, s, ev.start,
                   ev.stop, p);
        return;
      }
    }
    MOE_LAUNCH((grouped_gemm_kernel<DT, BM, BN, EPI, BiasT, DEPTH, NTH, false>), g, dim3(NTH), 0, s, ev.start,
               ev.stop, p);
  }
}

template <typename DT, int BM, int BN>
static void launch_epi(int epi, bool bias_f32, const GemmParams& p, int grid, hipStream_t s, LaunchEv ev) {
  using T = typename DT::T;
  if (epi == EPI_GELU) launch_t<DT, BM, BN, EPI_GELU, T>(p, grid, s, ev);
  else if (bias_f32) launch_t<DT, BM, BN, EPI_F32, float>(p, grid, s, ev);
  else launch_t<DT, BM, BN, EPI_F32, T>(p, grid, s, ev);
}

template <typename DT, int BN>
static bool launch_bm(int BM, int epi, bool bias_f32, const GemmParams& p, int grid, hipStream_t s, LaunchEv ev) {
  switch (BM) {
    case 16: launch_epi<DT, 16, BN>(epi, bias_f32, p, grid, s, ev); return true;
    case 32: launch_epi<DT, 32, BN>(epi, bias_f32, p, grid, s, ev); return true;
    case 64: launch_epi<DT, 64, BN>(epi, bias_f32, p, grid, s, ev); return true;
    case 128: launch_epi<DT, 128, BN>(epi, bias_f32, p, grid, s, ev); return true;
  }
  return false;
}

// 128 x 256, 256 x 256 and 320 x 256 tiles, eight waves: segments of 65..320 rows and the dense MLP
template <typename DT>
static bool launch_big(int BM, int epi, bool bias_f32, const GemmParams& p, int grid, hipStream_t s, LaunchEv ev) {
  switch (BM) {
    case 128: launch_epi<DT, 128, 256>(epi, bias_f32, p, grid, s, ev); return true;
    case 256: launch_epi<DT, 256, 256>(epi, bias_f32, p, grid, s, ev); return true;
    case 320: launch_epi<DT, 320, 256>(epi, bias_f32, p, grid, s, ev); return true;
  }
  return false;
}

template <typename DT>
static bool launch_bn(int BM, int BN, int epi, bool bias_f32, const GemmParams& p, int grid, hipStream_t s,
                      LaunchEv ev) {
  if constexpr (sizeof(typename DT::T) == 2) {
    if (BN == 256) return launch_big<DT>(BM, epi, bias_f32, p, grid, s, ev);
  }
  if (BN == 128) return launch_bm<DT, 128>(BM, epi, bias_f32, p, grid, s, ev);
  if (BN == 64) return launch_bm<DT, 64>(BM, epi, bias_f32, p, grid, s, ev);
  return false;
}

hipError_t launch_grouped_gemm(int dtype, int epi, bool bias_f32, int BM, int BN, const GemmParams& p, int grid,
                               hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  if (grid <= 0) return hipSuccess;
  if (BN == 256 && (bias_f32 || !p.off32)) return hipErrorInvalidValue;   // the ping-pong kernel's limits
  if (p.ksplit > 1) {   // fp32 partial outputs with a float bias only, and whole 128-byte steps per slice
    const long long steps = (long long)p.K * (dtype == DT_F32 ? 4 : 2) / 128;
    if (!bias_f32 || epi != EPI_F32 || p.tiles || steps % p.ksplit != 0 || p.ksplit > 65535)
      return hipErrorInvalidValue;
  }
  bool ok;
  const LaunchEv ev{ev0, ev1};
  switch (dtype) {
    case DT_F32: ok = launch_bn<DtF32>(BM, BN, epi, bias_f32, p, grid, s, ev); break;
    case DT_F16: ok = launch_bn<DtF16>(BM, BN, epi, bias_f32, p, grid, s, ev); break;
    default: ok = launch_bn<DtBF16>(BM, BN, epi, bias_f32, p, grid, s, ev); break;
  }
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace moe
