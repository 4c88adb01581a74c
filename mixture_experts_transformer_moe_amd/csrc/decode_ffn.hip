// Fused expert FFN for segments of at most MAXM rows (decode-sized batches).
//
// With a handful of rows per expert the layer is a stream over the active
// experts' weights: there is nothing for the matrix cores to reuse, so this
// kernel reads each weight byte once with 16-byte vector loads and does the
// arithmetic on the vector ALUs. Work-group (g, c) takes the g-th non-empty
// segment and the c-th 64-wide slice of the FFN width:
//
//   phase 1  h[m, f] = GeLU(x_m . W1[f, :] + b1[f])  for the slice's 64 f
//            (a contiguous 64 x H block of W1; one wave per row, rounded to
//            the I/O dtype like the GEMM path's hidden activation)
//   phase 2  part[c][m, j] = sum_{f in slice} h[m, f] W2[j, f] (+ b2[j] in slice 0)
//            (each W2 row contributes one 128-byte run; 8 lanes per row)
//
// The F/64 slice partials are summed in slice order by the combine (or by the
// reduce kernel), so results do not depend on scheduling.
#include "common.h"
#include "kernels.h"

namespace moe {

#define DEC_BF 64
#define DEC_RU 8     // W1 rows in flight per wave
#define DEC_U 8      // W2 row groups in flight per wave

template <typename DT, int MAXM>
__global__ __launch_bounds__(256) void decode_ffn_kernel(DecodeParams p) {
  using T = typename DT::T;
  extern __shared__ __attribute__((aligned(16))) char dsm[];
  T* xs = reinterpret_cast<T*>(dsm);                                       // [MAXM][H]
  float* hs = reinterpret_cast<float*>(dsm + (size_t)MAXM * p.H * sizeof(T));  // [MAXM][BF]
  __shared__ int s_info[3];

  const int nslice = p.F / DEC_BF;
  const int slice = blockIdx.x % nslice;
  const int g = blockIdx.x / nslice;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // ---- the g-th non-empty segment
  if (wave == 0) {
    if (p.seg_off) {
      int base = 0;
      bool done = false;
      for (int s0 = 0; s0 < p.nseg && !done; s0 += 64) {
        const int s = s0 + lane;
        const bool ne = (s < p.nseg) && (p.seg_off[s + 1] > p.seg_off[s]);
        const uint64_t bal = __ballot(ne);
        const int cnt = __popcll(bal);
        if (g < base + cnt) {
          const uint64_t below = lane ? (bal & ((~0ull) >> (64 - lane))) : 0ull;
          if (ne && __popcll(below) == g - base) {
            s_info[0] = s;
            s_info[1] = p.seg_off[s];
            s_info[2] = p.seg_off[s + 1];
          }
          done = true;
        }
        base += cnt;
      }
      if (!done && lane == 0) s_info[0] = -1;
    } else if (lane == 0) {
      s_info[0] = (g == 0) ? 0 : -1;
      s_info[1] = 0;
      s_info[2] = p.M;
    }
  }
  __syncthreads();
  const int seg = s_info[0];
  if (seg < 0) return;
  const int r0 = s_info[1];
  const int M = min(s_info[2] - r0, MAXM);
  const int H = p.H;
  const long long F = p.F;
  const int f0 = slice * DEC_BF;

  // ---- stage the segment's x rows in LDS (zeros past M)
  const int nvec = H / DT::VEC;
  for (int i = tid; i < MAXM * nvec; i += 256) {
    const int m = i / nvec, c = i - m * nvec;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (m < M) {
      const long long row = p.a_rows ? (long long)p.a_rows[r0 + m] : (long long)(r0 + m);
      v = reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(p.x) + row * H)[c];
    }
    reinterpret_cast<uint4*>(xs)[i] = v;
  }
  __syncthreads();

  // ---- phase 1: 16 rows of the slice per wave
  const T* w1 = reinterpret_cast<const T*>(p.w1) + (long long)seg * F * H;
  const T* b1 = reinterpret_cast<const T*>(p.b1) + (long long)seg * F;
  for (int rg = 0; rg < DEC_BF / 4; rg += DEC_RU) {
    const int fr = f0 + wave * (DEC_BF / 4) + rg;
    float acc[DEC_RU][MAXM];
#pragma unroll
    for (int u = 0; u < DEC_RU; ++u)
#pragma unroll
      for (int m = 0; m < MAXM; ++m) acc[u][m] = 0.f;
    for (int c = lane; c < nvec; c += 64) {
      uint4 wv[DEC_RU];
#pragma unroll
      for (int u = 0; u < DEC_RU; ++u)
        wv[u] = ld_nt16(reinterpret_cast<const uint4*>(w1 + (long long)(fr + u) * H) + c);
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {
        const uint4 xv = reinterpret_cast<const uint4*>(xs + (long long)m * H)[c];
        float xf[DT::VEC];
        unpack16<DT>(xv, xf);
#pragma unroll
        for (int u = 0; u < DEC_RU; ++u) acc[u][m] = dot16f<DT>(wv[u], xf, acc[u][m]);
      }
    }
#pragma unroll
    for (int u = 0; u < DEC_RU; ++u) {
      const float bb = DT::to_f(b1[fr + u]);
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {
        const float s = wave_sum(acc[u][m]);
        if (lane == 0) hs[m * DEC_BF + (fr + u - f0)] = DT::to_f(DT::from_f(gelu_erf(s + bb)));
      }
    }
  }
  __syncthreads();

  // ---- phase 2: every output j, 8 lanes per W2 row (64 f = 8 x 16 bytes)
  const int sub = lane & 7;
  const int rsub = lane >> 3;
  float hv[MAXM][8];
#pragma unroll
  for (int m = 0; m < MAXM; ++m)
#pragma unroll
    for (int i = 0; i < 8; ++i) hv[m][i] = hs[m * DEC_BF + sub * 8 + i];
  const T* w2 = reinterpret_cast<const T*>(p.w2) + (long long)seg * F * H + f0 + sub * 8;
  const T* b2 = reinterpret_cast<const T*>(p.b2) + (long long)seg * H;
  float* part = p.part + (long long)slice * p.row_space * H;
  const int rows_per_wave = H / 4;
  const int jw = wave * rows_per_wave;
  for (int it = 0; it < rows_per_wave; it += 8 * DEC_U) {
    uint4 wv[DEC_U];
#pragma unroll
    for (int u = 0; u < DEC_U; ++u) {
      const int j = jw + it + u * 8 + rsub;
      wv[u] = ld_nt16(w2 + (long long)j * F);
    }
#pragma unroll
    for (int u = 0; u < DEC_U; ++u) {
      const int j = jw + it + u * 8 + rsub;
      const float bj = (slice == 0) ? DT::to_f(b2[j]) : 0.f;
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {
        float v = dot16f<DT>(wv[u], hv[m], 0.f);
        v += __shfl_xor(v, 1, 64);
        v += __shfl_xor(v, 2, 64);
        v += __shfl_xor(v, 4, 64);
        if (sub == 0 && m < M) part[(long long)(r0 + m) * H + j] = v + bj;
      }
    }
  }
}

size_t decode_ffn_lds(int dtype, int maxm, int H) {
  const size_t esz = (dtype == DT_F32) ? 4 : 2;
  return (size_t)maxm * H * esz + (size_t)maxm * DEC_BF * sizeof(float);
}

template <typename DT>
static bool launch_m(int maxm, const DecodeParams& p, int grid, size_t lds, hipStream_t s) {
  switch (maxm) {
    case 1: hipLaunchKernelGGL((decode_ffn_kernel<DT, 1>), dim3(grid), dim3(256), lds, s, p); return true;
    case 2: hipLaunchKernelGGL((decode_ffn_kernel<DT, 2>), dim3(grid), dim3(256), lds, s, p); return true;
    case 4: hipLaunchKernelGGL((decode_ffn_kernel<DT, 4>), dim3(grid), dim3(256), lds, s, p); return true;
    case 8: hipLaunchKernelGGL((decode_ffn_kernel<DT, 8>), dim3(grid), dim3(256), lds, s, p); return true;
  }
  return false;
}

hipError_t launch_decode_ffn(int dtype, int maxm, const DecodeParams& p, int grid_segs, hipStream_t s) {
  const int grid = grid_segs * (p.F / DEC_BF);
  if (grid <= 0) return hipSuccess;
  const size_t lds = decode_ffn_lds(dtype, maxm, p.H);
  bool ok = (dtype == DT_F16) ? launch_m<DtF16>(maxm, p, grid, lds, s)
          : (dtype == DT_BF16) ? launch_m<DtBF16>(maxm, p, grid, lds, s) : false;
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace moe
