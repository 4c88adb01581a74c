// Expert FFN for segments of at most MAXM rows (decode-sized batches).
//
// With a handful of rows per expert the FFN is a stream over the active
// experts' weights: there is nothing for the matrix cores to reuse, so these
// kernels read each weight byte once with 16-byte non-temporal vector loads and
// do the arithmetic on the vector ALUs. Two launches, no barriers inside:
//
//   up    h[r, f] = GeLU(x_r . W1[f, :] + b1[f]), rounded to the I/O dtype
//   down  y[r, j] = h_r . W2[j, :] + b2[j]   (fp32), or, for a top-1 layer
//         without the dense MLP, the combine folded in: out[t, j] =
//         round(w_t * y[r, j]) with t the token of row r
//
// A wave owns RPW weight rows. Each lane loads its NQ 16-byte vectors of every
// row up front (all loads in flight at once), multiplies them with the
// segment's activation rows and a single multi-value wave reduction sums the
// RPW x MAXM dot products. Work-group g x c takes the g-th non-empty segment
// (found by each wave on its own from the offsets) and the c-th block of rows.
#include "common.h"
#include "kernels.h"

namespace moe {

// The g-th non-empty segment of seg_off[0..nseg] (nseg <= 512), per wave. All
// offsets are loaded at once (clamped addresses, masked values, no branches).
__device__ inline bool find_active(const int* __restrict__ seg_off, int nseg, int g, int& seg, int& r0, int& r1) {
  const int lane = threadIdx.x & 63;
  int lo[8], hi[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int s = min(i * 64 + lane, nseg - 1);
    lo[i] = seg_off[s];
    hi[i] = seg_off[s + 1];
  }
  int base = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool ne = (i * 64 + lane < nseg) && hi[i] > lo[i];
    const uint64_t bal = __ballot(ne);
    const int cnt = __popcll(bal);
    if (g < base + cnt) {
      const uint64_t below = lane ? (bal & ((~0ull) >> (64 - lane))) : 0ull;
      const uint64_t pick = __ballot(ne && __popcll(below) == g - base);
      const int src = __ffsll((unsigned long long)pick) - 1;
      seg = i * 64 + src;
      r0 = __shfl(lo[i], src, 64);
      r1 = __shfl(hi[i], src, 64);
      return true;
    }
    base += cnt;
  }
  return false;
}

template <int NQ, int MAXM>
struct DecRows {
  static constexpr int by_regs = (16 / NQ) > 0 ? 16 / NQ : 1;
  static constexpr int by_red = 64 / MAXM;
  static constexpr int RPW = by_regs < by_red ? by_regs : by_red;    // weight rows per wave
};

__host__ __device__ constexpr int ilog2(int n) { return n <= 1 ? 0 : 1 + ilog2(n / 2); }

// Issue every weight load of the wave: RPW rows of length K, NQ 16-byte vectors per lane.
template <typename DT, int NQ, int RPW>
__device__ inline void load_rows(uint4 (&wv)[RPW][NQ], const typename DT::T* __restrict__ wrow0, long long K) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      wv[i][q] = ld_nt16(wrow0 + (long long)i * K + (long long)(lane + 64 * q) * DT::VEC);
}

// Dot the wave's rows with MAXM activation rows and reduce: returns, in each
// lane, the sum for value v = lane >> (6 - log2(RPW * MAXM)) (row v / MAXM,
// activation v % MAXM).
template <typename DT, int MAXM, int NQ, int RPW>
__device__ inline float dot_rows(const uint4 (&wv)[RPW][NQ], const typename DT::T* const (&act)[MAXM]) {
  const int lane = threadIdx.x & 63;
  float acc[RPW * MAXM];
#pragma unroll
  for (int i = 0; i < RPW * MAXM; ++i) acc[i] = 0.f;
  if constexpr (MAXM * NQ <= 16) {
    // few activation vectors: load them all at once
    uint4 av[MAXM][NQ];
#pragma unroll
    for (int m = 0; m < MAXM; ++m)
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        av[m][q] = *reinterpret_cast<const uint4*>(act[m] + (long long)(lane + 64 * q) * DT::VEC);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {
        float af[DT::VEC];
        unpack16<DT>(av[m][q], af);
#pragma unroll
        for (int i = 0; i < RPW; ++i) acc[i * MAXM + m] = dot16f<DT>(wv[i][q], af, acc[i * MAXM + m]);
      }
    }
  } else {
    // many: one vector column q at a time
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      uint4 av[MAXM];
#pragma unroll
      for (int m = 0; m < MAXM; ++m)
        av[m] = *reinterpret_cast<const uint4*>(act[m] + (long long)(lane + 64 * q) * DT::VEC);
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {
        float af[DT::VEC];
        unpack16<DT>(av[m], af);
#pragma unroll
        for (int i = 0; i < RPW; ++i) acc[i * MAXM + m] = dot16f<DT>(wv[i][q], af, acc[i * MAXM + m]);
      }
    }
  }
  return wave_reduce_multi<RPW * MAXM>(acc);
}

template <typename DT, int MAXM, int NQ>
__global__ __launch_bounds__(256) void decode_up_kernel(DecodeParams p) {
  using T = typename DT::T;
  constexpr int RPW = DecRows<NQ, MAXM>::RPW;
  constexpr int N = RPW * MAXM;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nchunk = p.F / (4 * RPW);
  const int g = blockIdx.x / nchunk;
  const int chunk = blockIdx.x - g * nchunk;
  int seg = 0, r0 = 0, r1 = p.M;
  if (p.seg_off) {
    if (!find_active(p.seg_off, p.nseg, g, seg, r0, r1)) return;
  } else if (g > 0) {
    return;
  }
  const long long H = p.H, F = p.F;
  const int f0 = chunk * 4 * RPW + wave * RPW;
  uint4 wv[RPW][NQ];
  load_rows<DT, NQ, RPW>(wv, reinterpret_cast<const T*>(p.w1) + (long long)seg * F * H + (long long)f0 * H, H);
  __builtin_amdgcn_sched_barrier(0);   // every weight load is in flight before anything else
  const int M = min(r1 - r0, MAXM);
  const T* x = reinterpret_cast<const T*>(p.x);
  const T* act[MAXM];
#pragma unroll
  for (int m = 0; m < MAXM; ++m) {
    const int r = r0 + (m < M ? m : 0);
    const long long row = p.a_rows ? (long long)p.a_rows[r] : (long long)r;
    act[m] = x + row * H;
  }
  const float s = dot_rows<DT, MAXM, NQ, RPW>(wv, act);
  constexpr int SH = 6 - ilog2(N);
  const int v = lane >> SH;
  const int i = v / MAXM, m = v - (v / MAXM) * MAXM;
  if ((lane & ((1 << SH) - 1)) == 0 && m < M) {
    const T* b1 = reinterpret_cast<const T*>(p.b1) + (long long)seg * F;
    const float u = s + DT::to_f(b1[f0 + i]);
    reinterpret_cast<T*>(p.h)[(long long)(r0 + m) * F + f0 + i] = DT::from_f(pin_f32(gelu_erf(u)));
  }
}

template <typename DT, int MAXM, int NQ, bool FUSE>
__global__ __launch_bounds__(256) void decode_down_kernel(DecodeParams p) {
  using T = typename DT::T;
  constexpr int RPW = DecRows<NQ, MAXM>::RPW;
  constexpr int N = RPW * MAXM;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nchunk = p.H / (4 * RPW);
  const int g = blockIdx.x / nchunk;
  const int chunk = blockIdx.x - g * nchunk;
  int seg = 0, r0 = 0, r1 = p.M;
  if (p.seg_off) {
    if (!find_active(p.seg_off, p.nseg, g, seg, r0, r1)) return;
  } else if (g > 0) {
    return;
  }
  const long long H = p.H, F = p.F;
  const int j0 = chunk * 4 * RPW + wave * RPW;
  uint4 wv[RPW][NQ];
  load_rows<DT, NQ, RPW>(wv, reinterpret_cast<const T*>(p.w2) + (long long)seg * H * F + (long long)j0 * F, F);
  __builtin_amdgcn_sched_barrier(0);
  const int M = min(r1 - r0, MAXM);
  const T* h = reinterpret_cast<const T*>(p.h);
  const T* act[MAXM];
#pragma unroll
  for (int m = 0; m < MAXM; ++m) act[m] = h + (long long)(r0 + (m < M ? m : 0)) * F;
  const float s = dot_rows<DT, MAXM, NQ, RPW>(wv, act);
  constexpr int SH = 6 - ilog2(N);
  const int v = lane >> SH;
  const int i = v / MAXM, m = v - (v / MAXM) * MAXM;
  if ((lane & ((1 << SH) - 1)) == 0 && m < M) {
    const T* b2 = reinterpret_cast<const T*>(p.b2) + (long long)seg * H;
    const float yv = s + DT::to_f(b2[j0 + i]);
    if (FUSE) {
      const int t = p.slot_token[r0 + m];
      const float wt = p.topk_w[t];
      reinterpret_cast<T*>(p.out)[(long long)t * H + j0 + i] = DT::from_f(pin_f32(fmaf(wt, yv, 0.f)));
    } else {
      reinterpret_cast<float*>(p.out)[(long long)(r0 + m) * H + j0 + i] = yv;
    }
  }
}

// ---------------------------------------------------------------- launchers
static int nq_of(int K, int vec) { return K / (64 * vec); }

template <typename DT, int MAXM, int NQ>
static hipError_t launch_up_t(const DecodeParams& p, int grid_segs, hipStream_t s) {
  constexpr int RPW = DecRows<NQ, MAXM>::RPW;
  const int grid = grid_segs * (p.F / (4 * RPW));
  hipLaunchKernelGGL((decode_up_kernel<DT, MAXM, NQ>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename DT, int MAXM, int NQ>
static hipError_t launch_down_t(const DecodeParams& p, int grid_segs, bool fuse, hipStream_t s) {
  constexpr int RPW = DecRows<NQ, MAXM>::RPW;
  const int grid = grid_segs * (p.H / (4 * RPW));
  if (fuse) hipLaunchKernelGGL((decode_down_kernel<DT, MAXM, NQ, true>), dim3(grid), dim3(256), 0, s, p);
  else hipLaunchKernelGGL((decode_down_kernel<DT, MAXM, NQ, false>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename DT, int MAXM>
static hipError_t launch_m(bool up, const DecodeParams& p, int grid_segs, bool fuse, hipStream_t s) {
  const int nq = up ? nq_of(p.H, DT::VEC) : nq_of(p.F, DT::VEC);
  switch (nq) {
#define CASE(Q)                                                                              \
  case Q:                                                                                    \
    return up ? launch_up_t<DT, MAXM, Q>(p, grid_segs, s) : launch_down_t<DT, MAXM, Q>(p, grid_segs, fuse, s);
    CASE(1) CASE(2) CASE(4) CASE(8) CASE(16)
#undef CASE
  }
  return hipErrorInvalidValue;
}

template <typename DT>
static hipError_t launch_dt(bool up, int maxm, const DecodeParams& p, int grid_segs, bool fuse, hipStream_t s) {
  switch (maxm) {
    case 1: return launch_m<DT, 1>(up, p, grid_segs, fuse, s);
    case 2: return launch_m<DT, 2>(up, p, grid_segs, fuse, s);
    case 4: return launch_m<DT, 4>(up, p, grid_segs, fuse, s);
    case 8: return launch_m<DT, 8>(up, p, grid_segs, fuse, s);
  }
  return hipErrorInvalidValue;
}

bool decode_supported(int dtype, int H, int F) {
  if (dtype == DT_F32) return false;
  auto ok = [](int K) {
    if (K % 512) return false;
    const int q = K / 512;
    return q == 1 || q == 2 || q == 4 || q == 8 || q == 16;
  };
  return ok(H) && ok(F);
}

hipError_t launch_decode_up(int dtype, int maxm, const DecodeParams& p, int grid_segs, hipStream_t s) {
  if (grid_segs <= 0) return hipSuccess;
  return dtype == DT_F16 ? launch_dt<DtF16>(true, maxm, p, grid_segs, false, s)
                         : launch_dt<DtBF16>(true, maxm, p, grid_segs, false, s);
}

hipError_t launch_decode_down(int dtype, int maxm, const DecodeParams& p, int grid_segs, bool fuse_combine,
                              hipStream_t s) {
  if (grid_segs <= 0) return hipSuccess;
  return dtype == DT_F16 ? launch_dt<DtF16>(false, maxm, p, grid_segs, fuse_combine, s)
                         : launch_dt<DtBF16>(false, maxm, p, grid_segs, fuse_combine, s);
}

}  // namespace moe
