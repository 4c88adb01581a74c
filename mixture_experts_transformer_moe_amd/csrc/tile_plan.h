// Work lists of the two expert GEMMs, built by one block from the rows each
// segment holds. Shared by the plan kernel (segment offsets given) and the
// dispatch kernels, which end with every segment's kept rows in hand and so
// build the lists without a launch of their own.
#pragma once

#include "common.h"

namespace moe {

struct TilePlanArgs {
  int2* list1;      // first GEMM's tiles (segment, nt << 16 | mt); null: not built
  int2* list2;      // second GEMM's tiles; null: not built
  int* count;       // count[0] = number of row tiles (the extra segment's included)
  int BM;           // rows per tile
  int n_nt1, n_nt2; // column tiles of the two GEMMs
  int mt_extra;     // row tiles of the extra segment (id nseg), listed first
};

// ints of LDS tile_plan_body<NTH> needs
__host__ __device__ constexpr int tile_plan_lds_ints(int nth) { return 2 * nth + nth / 64 + 2; }

// Thread s < nseg (nseg <= NTH) passes the rows of segment s. Order: the extra
// segment's tiles first (so they run alongside the expert tiles), then segment
// by segment, column tile, then row tile, so the row tiles that share a weight
// tile are adjacent. Every thread of the block must call it.
template <int NTH>
__device__ inline void tile_plan_body(int rows, int nseg, const TilePlanArgs& a, int* lds) {
  constexpr int NW = NTH / 64;
  int* P = lds;              // [NTH + 1] first row tile of each segment
  int* C = P + NTH + 1;      // [NTH] row tiles of each segment
  int* wsum = C + NTH;       // [NW + 1]
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int c = (tid < nseg) ? (rows + a.BM - 1) / a.BM : 0;
  C[tid] = c;
  int incl = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < NW; ++i) {
      const int t = wsum[i];
      wsum[i] = run;
      run += t;
    }
    wsum[NW] = run;
  }
  __syncthreads();
  P[tid] = wsum[w] + incl - c;
  if (tid == 0) P[nseg] = wsum[NW];
  __syncthreads();
  const int total = wsum[NW];
  if (tid == 0) a.count[0] = total + a.mt_extra;
  for (int g = 0; g < 2; ++g) {
    const int n_nt = g ? a.n_nt2 : a.n_nt1;
    int2* list = g ? a.list2 : a.list1;
    if (!list) continue;
    const int n_extra = a.mt_extra * n_nt;
    for (int L = tid; L < n_extra; L += NTH) {
      const int nt = L / a.mt_extra, mt = L - nt * a.mt_extra;
      list[L] = make_int2(nseg, (nt << 16) | mt);
    }
    for (int L = tid; L < total * n_nt; L += NTH) {
      const int v = L / n_nt;
      int lo = 0, hi = nseg;               // largest s with P[s] <= v and P[s+1] > v
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (P[mid] <= v) lo = mid; else hi = mid;
      }
      const int s = lo;
      const int q = L - P[s] * n_nt;
      const int cs = C[s];
      const int nt = q / cs, mt = q - (q / cs) * cs;
      list[n_extra + L] = make_int2(s, (nt << 16) | mt);
    }
  }
}

}  // namespace moe
