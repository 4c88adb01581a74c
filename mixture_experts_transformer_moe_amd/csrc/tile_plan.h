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
  int mt_extra;     // row tiles of the extra segment (id nseg), spread over the list
  int parts;        // blocks that build the lists in the multi-block dispatch (>= 1)
};

// ints of LDS tile_plan_body<NTH> needs
__host__ __device__ constexpr int tile_plan_lds_ints(int nth) { return 2 * nth + nth / 64 + 2; }

// Thread s < nseg (nseg <= NTH) passes the rows of segment s. Expert tiles go
// segment by segment, column tile, then row tile, so the row tiles that share a
// weight tile are adjacent; the extra segment's tiles are spread evenly among
// them. Every thread of the block must call it. With nparts blocks calling it,
// block `part` writes list entries part * NTH + tid, ... (stride nparts * NTH)
// and block 0 the count.
template <int NTH>
__device__ inline void tile_plan_body(int rows, int nseg, const TilePlanArgs& a, int* lds, int part = 0,
                                      int nparts = 1) {
  constexpr int NW = NTH / 64;
  int* P = lds;              // [NTH + 1] first row tile of each segment
  int* C = P + NTH + 1;      // [NTH] row tiles of each segment
  int* wsum = C + NTH;       // [NW + 1]
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int c = (tid < nseg) ? (rows + a.BM - 1) / a.BM : 0;
  C[tid] = c;
  const int incl = wave_incl_scan(c);
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  if (tid == 0) {
    int t[NW];   // every wave's total read before the first write
#pragma unroll
    for (int i = 0; i < NW; ++i) t[i] = wsum[i];
    int run = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      wsum[i] = run;
      run += t[i];
    }
    wsum[NW] = run;
  }
  __syncthreads();
  P[tid] = wsum[w] + incl - c;
  if (tid == 0) P[nseg] = wsum[NW];
  __syncthreads();
  const int total = wsum[NW];
  if (tid == 0 && part == 0) a.count[0] = total + a.mt_extra;
  for (int g = 0; g < 2; ++g) {
    const int n_nt = g ? a.n_nt2 : a.n_nt1;
    int2* list = g ? a.list2 : a.list1;
    if (!list) continue;
    // The extra segment's n_x tiles are spread evenly over the N entries: the
    // number of them among entries [0, L] is ceil((L + 1) n_x / N), so entry L
    // holds one iff that count steps at L. Each stretch of the list, and so each
    // XCD's share at any moment, mixes the extra segment's tiles (compute-bound
    // when its weights stay cached) with the expert tiles (weight streaming).
    const long long n_x = (long long)a.mt_extra * n_nt;
    const long long N = n_x + (long long)total * n_nt;
    for (int L = part * NTH + tid; L < N; L += nparts * NTH) {   // (N < 2^31: checked by the plan)
      const long long cx = n_x ? ((long long)(L + 1) * n_x + N - 1) / N : 0;
      const long long cp = n_x ? ((long long)L * n_x + N - 1) / N : 0;
      if (cx > cp) {              // the extra segment's tile cx - 1: column tile major, then row tile
        const int i = (int)(cx - 1);
        const int nt = i / a.mt_extra, mt = i - nt * a.mt_extra;
        list[L] = make_int2(nseg, (nt << 16) | mt);
        continue;
      }
      const int j = (int)(L - cx);   // expert tile j
      const int v = j / n_nt;
      int lo = 0, hi = nseg;               // largest s with P[s] <= v and P[s+1] > v
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (P[mid] <= v) lo = mid; else hi = mid;
      }
      const int s = lo;
      const int q = j - P[s] * n_nt;
      const int cs = C[s];
      const int nt = q / cs, mt = q - (q / cs) * cs;
      list[L] = make_int2(s, (nt << 16) | mt);
    }
  }
}

}  // namespace moe
