// C ABI of the MoE layer library: argument checks, capacity, workspace layout
// and the launch sequence. Everything here runs on the host; every step of the
// layer itself runs in the kernels of the other files.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "moe.h"
#include "common.h"
#include "kernels.h"
#include "api_internal.h"

using namespace moe;

namespace {

thread_local char g_err[512] = "";

moe_status_t fail(moe_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status_t fail(moe_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

moe_status_t hip_fail(hipError_t e, const char* where) {
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

#define ST_TRY(expr)                 \
  do {                               \
    moe_status_t _s = (expr);        \
    if (_s != MOE_OK) return _s;     \
  } while (0)

#define HIP_TRY(expr, where)                   \
  do {                                         \
    hipError_t _e = (expr);                    \
    if (_e != hipSuccess) return hip_fail(_e, where); \
  } while (0)

constexpr int kMaxExperts = 512;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int64_t kMaxAssignments = (int64_t)1 << 30;   // T * k

// Exact ceil(k*T*cf / E) for a finite cf > 0 (cf = mant * 2^e2 exactly).
// Needs 1 <= E <= 512 and 0 <= T * k <= 2^30 (the callers check both), which
// keeps every shift below inside 128 bits: A < 2^83 before a left shift of at
// most 40, and E * 2^s < 2^10 * 2^115.
int64_t capacity_exact(int64_t T, int32_t E, int32_t k, double cf) {
  if (T == 0) return 0;
  int ex;
  const double f = frexp(cf, &ex);                       // cf = f * 2^ex, f in [0.5, 1)
  const unsigned long long mant = (unsigned long long)ldexp(f, 53);
  const int e2 = ex - 53;
  const __int128 N = (__int128)T * k;
  __int128 A = N * (__int128)mant;                       // < 2^32 * 2^53
  if (e2 >= 0) {
    if (e2 > 40) return INT64_MAX;
    A <<= e2;
    const __int128 q = (A + E - 1) / E;
    return q > (__int128)INT64_MAX ? INT64_MAX : (int64_t)q;
  }
  const int s = -e2;
  if (s + 11 >= 126) return A > 0 ? 1 : 0;               // E * 2^s exceeds A
  const __int128 B = (__int128)E << s;
  const __int128 q = (A + B - 1) / B;
  return (int64_t)q;
}

int pow2_at_least(int64_t v) {
  int m = 1;
  while (m < v) m <<= 1;
  return m;
}

int gemm_bm_for_rows(int64_t rows) {
  if (rows <= 16) return 16;
  if (rows <= 32) return 32;
  if (rows <= 64) return 64;
  return 128;
}

struct Plan {
  int64_t T, C, R_max;
  int H, F, E, e_lo, E_loc, k;
  int dtype;
  size_t esz;
  bool residual, renorm;
  // gate
  bool gate_mfma;
  bool stream_w;       // first expert GEMM: each weight tile read by <= 2 work-groups (non-temporal weight loads)
  bool stream_w2;      // second expert GEMM: each weight tile read by one work-group
  bool off32;          // GEMM operands each span < 4 GB (32-bit byte offsets; 256-column tiles need it)
  int gate_BM, gate_BN;
  int gate_ksplit;     // matrix-core gate: slices of K, each writing fp32 partial logits
  // dispatch
  bool disp_small;
  int nblk;
  bool route_fused;  // softmax / top-k and the multi-block dispatch in one launch (words zeroed by the gate)
  // experts
  bool exp_decode;   // streaming kernels for segments of <= 8 rows, else grouped MFMA GEMM
  bool fold_combine; // top-1 standard layer: the second expert kernel (decode or grouped GEMM) writes y
  bool zero_in_gate; // with fold_combine: the matrix-core gate zeroes y first
  bool route_in_up;  // decode path with a tiny batch: the first expert kernel does the dispatch
  bool fused_decode; // ... and both expert products run in one launch (h marked unwritten by the gate)
  int exp_maxm;
  int BM, BN1, BN2, mt_bound;
  // dense MLP
  bool dense_decode;
  bool dense_in_experts;  // residual MLP as an extra segment of the expert GEMM launches
  bool dense_in_decode;   // residual MLP as extra work-groups of the two decode expert launches
  int mt_extra;           // its row tiles
  int dBM, dBN1, dBN2;
  // workspace offsets (bytes)
  size_t o_z, o_idx, o_w, o_rank, o_blk, o_demand, o_off, o_slot_token, o_token_slot;
  size_t o_h, o_ydisp, o_list1, o_list2, o_count;
  size_t o_dh, o_dense;
  size_t total;
};

moe_status_t validate_uncached(const moe_layer_desc_t* d, Plan* pl);

// The plan of the last descriptor this thread validated: a decode loop calls the
// layer with the same descriptor every step, and the plan is a pure function of
// it (byte-equal descriptors have equal fields).
moe_status_t validate(const moe_layer_desc_t* d, Plan* pl) {
  thread_local moe_layer_desc_t last_d;
  thread_local Plan last_p;
  thread_local bool have = false;
  if (d && have && memcmp(d, &last_d, sizeof(*d)) == 0) {
    *pl = last_p;
    return MOE_OK;
  }
  const moe_status_t st = validate_uncached(d, pl);
  if (st == MOE_OK) {
    memcpy(&last_d, d, sizeof(*d));
    last_p = *pl;
    have = true;
  }
  return st;
}

moe_status_t validate_uncached(const moe_layer_desc_t* d, Plan* pl) {
  if (!d) return fail(MOE_ERR_INVALID_ARGUMENT, "descriptor is NULL");
  if (d->num_tokens < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "num_tokens < 0");
  if (d->hidden <= 0 || d->ffn <= 0) return fail(MOE_ERR_INVALID_ARGUMENT, "hidden and ffn must be > 0");
  if (d->num_experts < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "num_experts must be >= 1");
  if (d->top_k != 1 && d->top_k != 2) return fail(MOE_ERR_INVALID_ARGUMENT, "top_k must be 1 or 2");
  if (d->top_k > d->num_experts) return fail(MOE_ERR_INVALID_ARGUMENT, "top_k > num_experts");
  if (d->first_local_expert < 0 || d->first_local_expert >= d->num_experts)
    return fail(MOE_ERR_INVALID_ARGUMENT, "first_local_expert out of [0, E)");
  if (d->num_local_experts < 1 || (int64_t)d->first_local_expert + d->num_local_experts > d->num_experts)
    return fail(MOE_ERR_INVALID_ARGUMENT, "local expert range not inside [0, E)");
  if (!(d->capacity_factor > 0.0) || !isfinite(d->capacity_factor))
    return fail(MOE_ERR_INVALID_ARGUMENT, "capacity_factor must be finite and > 0");
  if (d->mlp_type != MOE_MLP_STANDARD && d->mlp_type != MOE_MLP_RESIDUAL)
    return fail(MOE_ERR_INVALID_ARGUMENT, "unknown mlp_type");
  if (d->mlp_type == MOE_MLP_RESIDUAL && d->top_k != 1)
    return fail(MOE_ERR_INVALID_ARGUMENT, "residual mode routes one expert per token (top_k must be 1)");
  if (d->dtype != MOE_DTYPE_F32 && d->dtype != MOE_DTYPE_F16 && d->dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_INVALID_ARGUMENT, "unknown dtype");
  if (d->flags & ~(MOE_FLAG_RENORM_TOPK | MOE_FLAG_DECODE_ONE_LAUNCH))
    return fail(MOE_ERR_INVALID_ARGUMENT, "unknown flag bits");
  if (d->hidden % 64 || d->ffn % 64) return fail(MOE_ERR_UNSUPPORTED, "hidden and ffn must be multiples of 64");
  if (d->num_experts > kMaxExperts) return fail(MOE_ERR_UNSUPPORTED, "num_experts > %d", kMaxExperts);
  if (d->num_tokens * (int64_t)d->top_k > kMaxAssignments)
    return fail(MOE_ERR_UNSUPPORTED, "num_tokens * top_k > 2^30");
  if (d->ffn > (1 << 20) || d->hidden > (1 << 20)) return fail(MOE_ERR_UNSUPPORTED, "hidden / ffn > 2^20");

  Plan& p = *pl;
  memset(&p, 0, sizeof(p));
  p.T = d->num_tokens;
  p.H = d->hidden;
  p.F = d->ffn;
  p.E = d->num_experts;
  p.e_lo = d->first_local_expert;
  p.E_loc = d->num_local_experts;
  p.k = d->top_k;
  p.dtype = (int)d->dtype;
  p.esz = d->dtype == MOE_DTYPE_F32 ? 4 : 2;
  p.residual = d->mlp_type == MOE_MLP_RESIDUAL;
  p.renorm = (d->flags & MOE_FLAG_RENORM_TOPK) != 0;
  p.C = capacity_exact(p.T, p.E, p.k, d->capacity_factor);
  const int64_t kT = p.T * p.k;
  p.R_max = (p.C >= kT) ? kT : std::min<int64_t>((int64_t)p.E_loc * p.C, kT);
  if ((int64_t)p.R_max * std::max(p.H, p.F) > ((int64_t)1 << 40))
    return fail(MOE_ERR_UNSUPPORTED, "dispatched buffers too large");

  // dispatch: one block when every assignment fits in it
  p.disp_small = kT <= dispatch_block_size();
  p.nblk = dispatch_num_blocks(kT);
  // gate: matrix cores when the batch fills tiles; else 4x8 wave blocks on the ALUs
  p.gate_mfma = p.T >= 64 && (p.E % 64) == 0;
  // experts: streaming kernels for tiny segments, grouped MFMA GEMM otherwise
  const int64_t seg_rows = std::min<int64_t>(p.C, kT);
  p.exp_maxm = pow2_at_least(std::max<int64_t>(seg_rows, 1));
  p.exp_decode = seg_rows <= 8 && decode_supported(p.dtype, p.H, p.F);
  if (p.exp_decode) {
    // the streaming kernels give every segment group (every assignment when
    // they route the batch themselves) a work-group per block of weight rows,
    // and each routed work-group first routes the whole batch: past about 8192
    // work-groups per launch the grouped GEMM, whose tile list holds only the
    // active experts' tiles, is faster (decode at 8 tokens: 350M 30 vs 54 us,
    // 6.7B top-1 339 vs 371 us with <= 8192; 6.7B and 24B one-GPU shares with
    // top-2 472 vs 304 and 1857 vs 1123 us with 16 k and 64 k work-groups)
    const int64_t segs = std::min<int64_t>(p.E_loc, p.R_max);
    const int64_t up_groups = route_in_decode_supported((int)p.T, p.k, p.E, p.E_loc) ? kT : segs;
    if (decode_max_workgroups(p.dtype, p.H, p.F, p.exp_maxm, up_groups, segs) > 8192) p.exp_decode = false;
  }
  // top-1 standard layers: the second expert kernel writes y itself (the decode
  // kernel or the second grouped GEMM's epilogue)
  p.fold_combine = p.k == 1 && !p.residual && p.R_max > 0;
  // ... and the rows of tokens without a kept choice are zeroed: by the
  // matrix-core gate's work-groups (all of y, before the dispatch) on the
  // grouped-GEMM path, else by the routing (its dispatch or the decode kernel)
  p.zero_in_gate = p.fold_combine && !p.exp_decode && p.gate_mfma;
  p.route_in_up = p.exp_decode && route_in_decode_supported((int)p.T, p.k, p.E, p.E_loc);
  // one launch for both expert products: the vector-ALU gate kernel marks its h rows unwritten
  p.fused_decode = (d->flags & MOE_FLAG_DECODE_ONE_LAUNCH) && p.route_in_up && !p.gate_mfma &&
                   decode_fused_supported(p.dtype, p.H, p.F, p.exp_maxm);
  // softmax / top-k and the whole multi-block dispatch in one launch, whose
  // published words (keys, block counts) and slot_token the matrix-core gate zeroes
  p.route_fused = !p.disp_small && !p.route_in_up && p.gate_mfma && route_dispatch_supported(kT);
  // matrix-core gate: each K step of a work-group waits on its loads, so a
  // short tile over all of K is latency-bound. Column tiles of 128 experts (x
  // read once per token tile); the tallest row tile and the fewest slices of K
  // (at least 8 steps each) that give 512 work-groups. Slices leave fp32 partial
  // logits that the softmax / top-k adds in a fixed order. The routing inside
  // the first decode expert kernel reads plain logits: no slices there.
  p.gate_BN = (p.E % 128 == 0) ? 128 : 64;
  p.gate_BM = 16;
  p.gate_ksplit = 1;
  if (p.gate_mfma) {
    const int64_t steps = (int64_t)p.H * p.esz / 128;
    bool found = false;
    for (int bm : {64, 32, 16}) {
      const int64_t tiles = ((p.T + bm - 1) / bm) * (p.E / p.gate_BN);
      for (int s : {1, 2, 4, 8}) {
        if (s > 1 && (p.route_in_up || steps % s != 0 || steps / s < 8)) break;
        if (tiles * s >= 512) { p.gate_BM = bm; p.gate_ksplit = s; found = true; break; }
      }
      if (found) break;
    }
    if (!found) {   // small batch: the most slices allowed
      p.gate_BM = 16;
      for (int s : {2, 4, 8})
        if (!p.route_in_up && steps % s == 0 && steps / s >= 8) p.gate_ksplit = s;
    }
  }
  p.BM = gemm_bm_for_rows(seg_rows);
  p.BN1 = (p.F % 128 == 0) ? 128 : 64;
  p.BN2 = (p.H % 128 == 0) ? 128 : 64;
  // segments of more than 64 rows: eight-wave 128 x 256 or 160 x 256 tiles
  // (256 / 320 when one tile covers a segment that would need two / three
  // 128-row tiles: each weight tile is then read once, by a work-group of
  // 64 / 80 x 128 wave blocks)
  // (they address their operands with 32-bit byte offsets: activations x,
  // x_disp and h, at most max(T, R_max) rows of max(H, F), and one expert's or
  // the MLP's weights, H x F, must each stay below 4 GB)
  p.off32 = std::max<int64_t>(p.T, p.R_max) * std::max(p.H, p.F) * (int64_t)p.esz < ((int64_t)1 << 32) &&
            (int64_t)p.H * p.F * (int64_t)p.esz < ((int64_t)1 << 32);
  const bool big_ok = p.dtype != MOE_DTYPE_F32 && p.F % 256 == 0 && p.H % 256 == 0 && p.off32;
  if (p.BM == 128 && big_ok) {
    p.BN1 = p.BN2 = 256;
    if (seg_rows > 128 && seg_rows <= 256) p.BM = 256;
    if (seg_rows > 256 && seg_rows <= 320) p.BM = 320;
  }
  {
    const int64_t segs = std::min<int64_t>(p.E_loc, p.R_max);
    const int64_t mtb = (p.R_max + (int64_t)(p.BM - 1) * segs) / p.BM;
    if (!p.exp_decode && mtb >= 65536) return fail(MOE_ERR_UNSUPPORTED, "too many row tiles");
    p.mt_bound = (int)mtb;
    if (p.F / p.BN1 >= 65536 || p.H / p.BN2 >= 65536) return fail(MOE_ERR_UNSUPPORTED, "too many column tiles");
  }
  p.dense_decode = p.T <= 8 && decode_supported(p.dtype, p.H, p.F);
  // GEMM path with 64-row expert tiles: the dense MLP's tiles join the expert
  // GEMM launches (its L2-resident weights overlap the experts' weight
  // streaming). With smaller expert tiles the MLP would run on tiles too thin
  // for its T rows (measured slower), so it keeps its own launches.
  p.dense_in_experts = p.residual && !p.exp_decode && !p.dense_decode && p.BM >= 64;
  // decode path: the dense MLP's work-groups join the two expert launches (not
  // the one-launch kernel, set below)
  p.dense_in_decode = p.residual && p.exp_decode && p.dense_decode && !p.fused_decode;
  // weight-streaming tiles (<= 64 rows) of a second GEMM with long weight rows:
  // 64-column tiles halve each work-group's share of the weights (F = 8192,
  // fp16: 1 MB instead of 2 MB), so the work-groups left over when the tile
  // count is just past a multiple of the resident ones (33 experts x 16 tiles =
  // 528 against 512) finish sooner: prefill layer 425 -> 417 us. Not with the
  // dense MLP's tiles in the launch, which lose more on 64-column tiles than
  // the experts gain (residual layer 955 -> 1010 us).
  if (!p.exp_decode && p.BM <= 64 && p.BN2 == 128 && !p.dense_in_experts && (int64_t)p.F * p.esz > 8192) p.BN2 = 64;
  // segments of at most two row tiles: each expert weight tile is read by one
  // or two work-groups, so the first GEMM streams the expert weights with
  // non-temporal loads (the dense MLP's tiles in the same launches, read by
  // every token tile, keep their weights cached)
  p.stream_w = !p.exp_decode && seg_rows <= 2 * (int64_t)p.BM;
  // The second GEMM streams its weights only when every segment fits one row
  // tile: its weight tiles are long (K = F), and the two row tiles of a segment
  // read each of them side by side, the second finding it in L2 when cached
  // (24B share, 160 x 256 tiles: 2.58 ms cached against 2.73 ms streamed). The
  // first GEMM keeps streaming them, leaving L2 to the activation rows that all
  // of its column tiles re-read (2.85 ms streamed against 2.92 ms cached).
  p.stream_w2 = !p.exp_decode && seg_rows <= (int64_t)p.BM;
  if (p.dense_in_experts) {
    const int64_t mte = (p.T + p.BM - 1) / p.BM;
    if (mte >= 65536) return fail(MOE_ERR_UNSUPPORTED, "too many row tiles");
    p.mt_extra = (int)mte;
    p.mt_bound += p.mt_extra;
  }
  if (!p.exp_decode && (int64_t)p.mt_bound * std::max(p.F / p.BN1, p.H / p.BN2) >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "too many tiles");
  p.dBM = gemm_bm_for_rows(p.T);
  {
    // 256-wide tiles only where they still give every CU two work-groups
    const int64_t dmt = (p.T + p.dBM - 1) / p.dBM;
    const bool big1 = p.dBM == 128 && big_ok && dmt * (p.F / 256) >= 512;
    const bool big2 = p.dBM == 128 && big_ok && dmt * (p.H / 256) >= 512;
    p.dBN1 = big1 ? 256 : ((p.F % 128 == 0) ? 128 : 64);
    p.dBN2 = big2 ? 256 : ((p.H % 128 == 0) ? 128 : 64);
  }

  // workspace layout
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  const size_t T = (size_t)p.T, H = (size_t)p.H, F = (size_t)p.F, R = (size_t)p.R_max;
  p.o_z = take(T * p.E * 4 * (size_t)p.gate_ksplit);
  p.o_idx = take(T * p.k * 4);
  p.o_w = take(T * p.k * 4);
  p.o_rank = take(p.disp_small ? 0 : T * p.k * 4);
  p.o_blk = take(p.disp_small ? 0 : (size_t)p.nblk * p.E * 4);
  p.o_demand = take((size_t)p.E * 4);
  p.o_off = take((size_t)(p.E_loc + 1) * 4);
  p.o_slot_token = take(R * 4);
  p.o_token_slot = take(T * p.k * 4);
  p.o_h = take(R * F * p.esz);
  p.o_ydisp = take(R * H * 4);
  if (!p.exp_decode) {
    p.o_list1 = take((size_t)p.mt_bound * (F / p.BN1) * sizeof(int2));
    p.o_list2 = take((size_t)p.mt_bound * (H / p.BN2) * sizeof(int2));
    p.o_count = take(4);
  }
  if (p.residual) {
    p.o_dh = take(T * F * p.esz);
    p.o_dense = take(T * H * 4);
  }
  p.total = o;
  return MOE_OK;
}

template <typename Tp>
Tp* wsp(void* ws, size_t off) {
  return reinterpret_cast<Tp*>(reinterpret_cast<char*>(ws) + off);
}

moe_status_t check_ptr(const void* p, const char* name) {
  if (!p) return fail(MOE_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned16(p)) return fail(MOE_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
  return MOE_OK;
}

#define PTR_TRY(p, name)                          \
  do {                                            \
    moe_status_t _s = check_ptr((p), (name));     \
    if (_s != MOE_OK) return _s;                  \
  } while (0)

moe_status_t check_weights(const Plan& p, const moe_layer_weights_t* w, bool experts, bool dense) {
  if (!w) return fail(MOE_ERR_INVALID_ARGUMENT, "weights is NULL");
  if (experts) {
    const int tables = (w->w1_experts != nullptr) + (w->b1_experts != nullptr) + (w->w2_experts != nullptr) +
                       (w->b2_experts != nullptr);
    if (tables == 4) {
      PTR_TRY(w->w1_experts, "w1_experts");
      PTR_TRY(w->b1_experts, "b1_experts");
      PTR_TRY(w->w2_experts, "w2_experts");
      PTR_TRY(w->b2_experts, "b2_experts");
    } else if (tables != 0) {
      return fail(MOE_ERR_INVALID_ARGUMENT, "set all four per-expert pointer tables or none");
    } else {
      PTR_TRY(w->w1, "w1");
      PTR_TRY(w->b1, "b1");
      PTR_TRY(w->w2, "w2");
      PTR_TRY(w->b2, "b2");
    }
  }
  if (dense) {
    PTR_TRY(w->mlp_w1, "mlp_w1");
    PTR_TRY(w->mlp_b1, "mlp_b1");
    PTR_TRY(w->mlp_w2, "mlp_w2");
    PTR_TRY(w->mlp_b2, "mlp_b2");
  }
  (void)p;
  return MOE_OK;
}

// ---------------------------------------------------------------- launch steps
// y_zero (matrix-core gate only): the layer output, zeroed by the gate's
// work-groups before a folded top-1 combine writes its kept rows.
moe_status_t run_gate_logits(const Plan& p, const void* x, const void* gate_w, const float* gate_b, float* z,
                             hipStream_t s, unsigned* fill = nullptr, int nfill = 0, void* y_zero = nullptr,
                             void* ws_zero = nullptr, int ws_zero16 = 0) {
  if (p.gate_mfma) {
    GemmParams g{};
    if (y_zero) {
      g.zero_y = y_zero;
      g.zero_T = (int)p.T;
      g.zero_esz = (int)p.esz;
      g.zero_N = p.H;
    }
    if (ws_zero && ws_zero16 > 0) {
      g.zero_ws = ws_zero;
      g.zero_n16 = ws_zero16;
    }
    g.A = x;
    g.M = (int)p.T;
    g.nseg = 1;
    g.N = p.E;
    g.K = p.H;
    g.B = gate_w;
    g.bias = gate_b;
    g.C = z;
    g.n_ntiles = p.E / p.gate_BN;
    g.ksplit = p.gate_ksplit;
    g.c_split = (long long)p.T * p.E;
    const int grid = (int)((p.T + p.gate_BM - 1) / p.gate_BM) * g.n_ntiles;
    HIP_TRY(launch_grouped_gemm(p.dtype, EPI_F32, true, p.gate_BM, p.gate_BN, g, grid, s), "gate logits (mfma)");
  } else {
    HIP_TRY(launch_gate_logits_fma(p.dtype, x, gate_w, gate_b, z, (int)p.T, p.H, p.E, s, fill, nfill),
            "gate logits");
  }
  return MOE_OK;
}

// plan (nullable): the dispatch kernel that computes the segment offsets also
// writes the expert GEMMs' tile lists.
moe_status_t run_dispatch(const Plan& p, bool fuse_topk, const float* z, float* probs, float* topk_w, int* idx,
                          int* demand, int* offsets, int* slot_token, int* token_slot, void* y_zero, void* ws,
                          hipStream_t s, const TilePlanArgs* plan = nullptr) {
  const int C = (int)std::min<int64_t>(p.C, INT32_MAX);
  if (p.disp_small) {
    HIP_TRY(launch_dispatch_small(fuse_topk, z, p.renorm ? 1 : 0, probs, topk_w, idx, (int)p.T, p.k, p.E, p.e_lo,
                                  p.E_loc, C, (int)p.R_max, demand, offsets, slot_token, token_slot, y_zero,
                                  (int)p.esz, p.H, plan, p.gate_ksplit, s),
            "dispatch (one block)");
    return MOE_OK;
  }
  if (fuse_topk)
    HIP_TRY(launch_softmax_topk(z, (int)p.T, p.E, p.k, p.renorm ? 1 : 0, idx, topk_w, probs, s, p.gate_ksplit),
            "softmax/top-k");
  HIP_TRY(launch_dispatch_multi(idx, (int)p.T, p.k, p.E, p.e_lo, p.E_loc, C, (int)p.R_max, wsp<int>(ws, p.o_rank),
                                wsp<int>(ws, p.o_blk), demand, offsets, slot_token, token_slot, y_zero,
                                (int)p.esz, p.H, plan, s),
          "dispatch");
  return MOE_OK;
}

// The expert GEMMs' tile lists in the workspace (with the extra segment's row
// tiles when the dense MLP runs inside the expert GEMMs).
TilePlanArgs tile_plan_args(const Plan& p, void* ws, bool with_dense) {
  TilePlanArgs a{};
  a.list1 = wsp<int2>(ws, p.o_list1);
  a.list2 = wsp<int2>(ws, p.o_list2);
  a.count = wsp<int>(ws, p.o_count);
  a.BM = p.BM;
  a.n_nt1 = p.F / p.BN1;
  a.n_nt2 = p.H / p.BN2;
  a.mt_extra = (with_dense && p.dense_in_experts) ? p.mt_extra : 0;
  // the multi-block dispatch builds the lists in blocks of about 2048 entries
  // (their length bound: row tiles x column tiles of both GEMMs), at most 16
  const int64_t bound = (int64_t)p.mt_bound * (a.n_nt1 + a.n_nt2);
  a.parts = (int)std::min<int64_t>(16, std::max<int64_t>(1, (bound + 2047) / 2048));
  return a;
}

// Expert FFN. x rows come from x via slot_token (a_rows != null) or from
// x_disp directly. Decode path leaves partials in ws; GEMM path writes ydisp.
moe_status_t record(hipEvent_t ev, hipStream_t s);

moe_status_t run_experts(const Plan& p, const void* x, const int* a_rows, const int* offsets,
                         const moe_layer_weights_t* w, float* ydisp, void* ws, hipStream_t s,
                         void* y_fold = nullptr, const int* slot_token = nullptr, const float* topk_w = nullptr,
                         const moe_phase_events_t* ev = nullptr, const RouteParams* route = nullptr,
                         bool with_dense = false, bool plan_ready = false) {
  const moe_phase_events_t none{};
  const moe_phase_events_t& e = ev ? *ev : none;
  hipEvent_t split = e.ffn_split;
  if (p.exp_decode) {
    DecodeParams d{};
    d.x = x;
    d.a_rows = a_rows;
    d.seg_off = offsets;
    d.nseg = p.E_loc;
    d.H = p.H;
    d.F = p.F;
    d.w1 = w->w1;
    d.b1 = w->b1;
    d.w2 = w->w2;
    d.b2 = w->b2;
    d.w1p = w->w1_experts;
    d.b1p = w->b1_experts;
    d.w2p = w->w2_experts;
    d.b2p = w->b2_experts;
    d.h = wsp<void>(ws, p.o_h);
    d.out = y_fold ? y_fold : (void*)ydisp;
    d.slot_token = slot_token;
    d.topk_w = topk_w;
    if (with_dense && p.dense_in_decode) {   // the residual MLP's work-groups in the same two launches
      d.dM = (int)p.T;
      d.dw1 = w->mlp_w1;
      d.db1 = w->mlp_b1;
      d.dw2 = w->mlp_w2;
      d.db2 = w->mlp_b2;
      d.dh = wsp<void>(ws, p.o_dh);
      d.dout = wsp<float>(ws, p.o_dense);
    }
    const int gsegs = (int)std::min<int64_t>(p.E_loc, p.R_max);
    // routed in the kernel: one group of work-groups per assignment (see route_phase1)
    const int gsegs_up = route ? (int)(p.T * p.k) : gsegs;
    if (route && p.fused_decode) {
      HIP_TRY(launch_decode_fused(p.dtype, p.exp_maxm, d, *route, gsegs_up, y_fold != nullptr, s, e.up_start,
                                  e.up_stop),
              "expert ffn (decode, one launch)");
      ST_TRY(record(split, s));
      return MOE_OK;
    }
    HIP_TRY(launch_decode_up(p.dtype, p.exp_maxm, d, gsegs_up, s, e.up_start, e.up_stop, route),
            "expert ffn up (decode)");
    ST_TRY(record(split, s));
    HIP_TRY(launch_decode_down(p.dtype, p.exp_maxm, d, gsegs, y_fold != nullptr, s, e.down_start, e.down_stop),
            "expert ffn down (decode)");
    return MOE_OK;
  }
  int2* l1 = wsp<int2>(ws, p.o_list1);
  int2* l2 = wsp<int2>(ws, p.o_list2);
  int* cnt = wsp<int>(ws, p.o_count);
  const int nt1 = p.F / p.BN1, nt2 = p.H / p.BN2;
  const bool dense = with_dense && p.dense_in_experts;
  if (!plan_ready) HIP_TRY(launch_gemm_plan(offsets, p.E_loc, tile_plan_args(p, ws, with_dense), s), "gemm plan");
  void* h = wsp<void>(ws, p.o_h);
  GemmParams g1{};
  g1.A = x;
  g1.a_rows = a_rows;
  g1.seg_off = offsets;
  g1.nseg = p.E_loc;
  g1.N = p.F;
  g1.K = p.H;
  g1.B = w->w1;
  g1.Bp = w->w1_experts;
  g1.biasp = w->b1_experts;
  g1.b_stride = (long long)p.F * p.H;
  g1.bias = w->b1;
  g1.bias_stride = p.F;
  g1.C = h;
  g1.tiles = l1;
  g1.tile_count = cnt;
  g1.n_ntiles = nt1;
  g1.stream_w = p.stream_w ? 1 : 0;
  g1.off32 = p.off32 ? 1 : 0;
  if (dense) {   // the residual MLP over all T tokens: h_dense = GeLU(x W1_mlp^T + b1_mlp)
    g1.A2 = x;
    g1.B2 = w->mlp_w1;
    g1.bias2 = w->mlp_b1;
    g1.C2 = wsp<void>(ws, p.o_dh);
    g1.M2 = (int)p.T;
  }
  HIP_TRY(launch_grouped_gemm(p.dtype, EPI_GELU, false, p.BM, p.BN1, g1, p.mt_bound * nt1, s, e.up_start, e.up_stop),
          "expert gemm 1");
  ST_TRY(record(split, s));
  GemmParams g2{};
  g2.A = h;
  g2.seg_off = offsets;
  g2.nseg = p.E_loc;
  g2.N = p.H;
  g2.K = p.F;
  g2.B = w->w2;
  g2.Bp = w->w2_experts;
  g2.biasp = w->b2_experts;
  g2.b_stride = (long long)p.H * p.F;
  g2.bias = w->b2;
  g2.bias_stride = p.H;
  g2.C = ydisp;
  g2.tiles = l2;
  g2.tile_count = cnt;
  g2.n_ntiles = nt2;
  g2.stream_w = p.stream_w2 ? 1 : 0;
  g2.off32 = p.off32 ? 1 : 0;
  if (y_fold) {   // top-1 combine in the epilogue
    g2.fold_y = y_fold;
    g2.fold_token = slot_token;
    g2.fold_w = topk_w;
  }
  if (dense) {   // m = h_dense W2_mlp^T + b2_mlp, fp32
    g2.A2 = wsp<void>(ws, p.o_dh);
    g2.B2 = w->mlp_w2;
    g2.bias2 = w->mlp_b2;
    g2.C2 = wsp<void>(ws, p.o_dense);
    g2.M2 = (int)p.T;
  }
  HIP_TRY(launch_grouped_gemm(p.dtype, EPI_F32, false, p.BM, p.BN2, g2, p.mt_bound * nt2, s, e.down_start,
                              e.down_stop),
          "expert gemm 2");
  return MOE_OK;
}

// Dense MLP (residual mode) over all T rows into out [T, H] fp32.
moe_status_t run_dense(const Plan& p, const void* x, const moe_layer_weights_t* w, float* out, void* ws,
                       hipStream_t s) {
  if (p.dense_decode) {
    // the decode kernels' dense work-groups alone (no expert groups): the same
    // code and arithmetic as when they join the expert launches
    DecodeParams d{};
    d.x = x;
    d.H = p.H;
    d.F = p.F;
    d.dM = (int)p.T;
    d.dw1 = w->mlp_w1;
    d.db1 = w->mlp_b1;
    d.dw2 = w->mlp_w2;
    d.db2 = w->mlp_b2;
    d.dh = wsp<void>(ws, p.o_dh);
    d.dout = out;
    HIP_TRY(launch_decode_up(p.dtype, 1, d, 0, s), "dense mlp up (decode)");
    HIP_TRY(launch_decode_down(p.dtype, 1, d, 0, false, s), "dense mlp down (decode)");
    return MOE_OK;
  }
  void* h = wsp<void>(ws, p.o_dh);
  GemmParams g1{};
  g1.A = x;
  g1.M = (int)p.T;
  g1.nseg = 1;
  g1.N = p.F;
  g1.K = p.H;
  g1.B = w->mlp_w1;
  g1.bias = w->mlp_b1;
  g1.C = h;
  g1.n_ntiles = p.F / p.dBN1;
  g1.off32 = p.off32 ? 1 : 0;
  const int mt = (int)((p.T + p.dBM - 1) / p.dBM);
  HIP_TRY(launch_grouped_gemm(p.dtype, EPI_GELU, false, p.dBM, p.dBN1, g1, mt * g1.n_ntiles, s), "dense gemm 1");
  GemmParams g2{};
  g2.A = h;
  g2.M = (int)p.T;
  g2.nseg = 1;
  g2.N = p.H;
  g2.K = p.F;
  g2.B = w->mlp_w2;
  g2.bias = w->mlp_b2;
  g2.C = out;
  g2.n_ntiles = p.H / p.dBN2;
  g2.off32 = p.off32 ? 1 : 0;
  HIP_TRY(launch_grouped_gemm(p.dtype, EPI_F32, false, p.dBM, p.dBN2, g2, mt * g2.n_ntiles, s), "dense gemm 2");
  return MOE_OK;
}

moe_status_t record(hipEvent_t ev, hipStream_t s) {
  if (ev) HIP_TRY(hipEventRecord(ev, s), "hipEventRecord");
  return MOE_OK;
}


moe_status_t check_ws(const void* ws, size_t have, size_t need) {
  if (have < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", have, need);
  if (need > 0) PTR_TRY(ws, "workspace");
  return MOE_OK;
}

}  // namespace

namespace moe {
moe_status_t api_error(moe_status_t st, const char* msg) { return fail(st, "%s", msg); }
}  // namespace moe

// ================================================================ C ABI
extern "C" {

int64_t moe_capacity(int64_t T, int32_t E, int32_t k, double cf) {
  if (T < 0 || E < 1 || k < 1 || !(cf > 0.0) || !isfinite(cf)) return -1;
  // the limits a layer descriptor has (beyond them the exact arithmetic would overflow)
  if (E > kMaxExperts || k > 2 || T > kMaxAssignments / k) return -1;
  return capacity_exact(T, E, k, cf);
}

int64_t moe_max_rows(const moe_layer_desc_t* d) {
  Plan p;
  if (validate(d, &p) != MOE_OK) return -1;
  return p.R_max;
}

moe_status_t moe_workspace_size(const moe_layer_desc_t* d, size_t* bytes) {
  if (!bytes) return fail(MOE_ERR_INVALID_ARGUMENT, "bytes is NULL");
  Plan p;
  ST_TRY(validate(d, &p));
  *bytes = p.total;
  return MOE_OK;
}

moe_status_t moe_layer_plan(const moe_layer_desc_t* d, moe_layer_plan_t* out) {
  if (!out) return fail(MOE_ERR_INVALID_ARGUMENT, "out is NULL");
  Plan p;
  ST_TRY(validate(d, &p));
  out->capacity = p.C;
  out->max_rows = p.R_max;
  out->workspace_bytes = p.total;
  out->gate_path = p.gate_mfma ? MOE_GATE_MATRIX : MOE_GATE_VECTOR;
  out->expert_path = p.exp_decode ? MOE_EXPERTS_STREAM : MOE_EXPERTS_GROUPED_GEMM;
  out->dispatch_in_expert_kernel = p.route_in_up ? 1 : 0;
  out->combine_in_expert_kernel = p.fold_combine ? 1 : 0;
  out->dense_in_expert_kernels = (p.dense_in_experts || p.dense_in_decode) ? 1 : 0;
  out->tile_rows = p.exp_decode ? 0 : p.BM;
  out->tile_cols_w1 = p.exp_decode ? 0 : p.BN1;
  out->tile_cols_w2 = p.exp_decode ? 0 : p.BN2;
  // gate; dispatch (one block, one launch of many blocks, or softmax/top-k +
  // count, scan, scatter); two
  // expert kernels (the GEMMs' tile lists come from the dispatch); the dense
  // MLP's two unless inside the expert GEMMs; combine
  out->experts_one_launch = p.fused_decode ? 1 : 0;
  out->launches = 1 + (p.route_in_up ? 0 : ((p.disp_small || p.route_fused) ? 1 : 4)) + (p.fused_decode ? 1 : 2) +
                  ((p.residual && !p.dense_in_experts && !p.dense_in_decode) ? 2 : 0) + (p.fold_combine ? 0 : 1);
  return MOE_OK;
}

moe_status_t moe_gate(const moe_layer_desc_t* d, const void* x, const void* gate_w, const float* gate_b,
                      int32_t* topk_idx, float* topk_w, float* probs, void* ws, size_t ws_bytes, hipStream_t stream) {
  Plan p;
  ST_TRY(validate(d, &p));
  if (p.T == 0) return MOE_OK;
  PTR_TRY(x, "x");
  PTR_TRY(gate_w, "gate_w");
  PTR_TRY(topk_idx, "topk_idx");
  PTR_TRY(topk_w, "topk_w");
  if (gate_b && !aligned16(gate_b)) return fail(MOE_ERR_INVALID_ARGUMENT, "gate_b is not 16-byte aligned");
  if (probs && !aligned16(probs)) return fail(MOE_ERR_INVALID_ARGUMENT, "probs is not 16-byte aligned");
  ST_TRY(check_ws(ws, ws_bytes, align_up(p.T * p.E * 4 * (size_t)p.gate_ksplit)));
  float* z = wsp<float>(ws, 0);
  ST_TRY(run_gate_logits(p, x, gate_w, gate_b, z, stream));
  HIP_TRY(launch_softmax_topk(z, (int)p.T, p.E, p.k, p.renorm ? 1 : 0, topk_idx, topk_w, probs, stream,
                              p.gate_ksplit),
          "softmax/top-k");
  return MOE_OK;
}

moe_status_t moe_dispatch(const moe_layer_desc_t* d, const int32_t* topk_idx, const void* x, int32_t* expert_demand,
                          int32_t* expert_offsets, int32_t* slot_token, int32_t* token_slot, void* x_disp, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  Plan p;
  ST_TRY(validate(d, &p));
  PTR_TRY(expert_demand, "expert_demand");
  PTR_TRY(expert_offsets, "expert_offsets");
  // with T == 0 only demand (all zero) and offsets (all zero) are written
  if (p.T > 0) {
    PTR_TRY(topk_idx, "topk_idx");
    PTR_TRY(slot_token, "slot_token");
    PTR_TRY(token_slot, "token_slot");
  }
  if (x_disp && p.T > 0) {
    PTR_TRY(x, "x");
    PTR_TRY(x_disp, "x_disp");
  }
  // the multi-block path keeps ranks and block histograms at the layer's offsets
  const size_t need = p.disp_small ? 0 : p.o_blk + (size_t)p.nblk * p.E * 4;
  ST_TRY(check_ws(ws, ws_bytes, need));
  ST_TRY(run_dispatch(p, false, nullptr, nullptr, nullptr, (int*)topk_idx, expert_demand, expert_offsets, slot_token,
                      token_slot, nullptr, ws, stream));
  if (x_disp && p.T > 0) HIP_TRY(launch_gather_rows(p.dtype, x, slot_token, (int)p.R_max, p.H, x_disp, stream), "gather");
  return MOE_OK;
}

moe_status_t moe_expert_ffn(const moe_layer_desc_t* d, const void* x_disp, const int32_t* expert_offsets,
                            const moe_layer_weights_t* w, float* y_disp, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  Plan p;
  ST_TRY(validate(d, &p));
  if (p.T == 0 || p.R_max == 0) return MOE_OK;
  PTR_TRY(x_disp, "x_disp");
  PTR_TRY(expert_offsets, "expert_offsets");
  PTR_TRY(y_disp, "y_disp");
  ST_TRY(check_weights(p, w, true, false));
  ST_TRY(check_ws(ws, ws_bytes, p.total));
  ST_TRY(run_experts(p, x_disp, nullptr, expert_offsets, w, y_disp, ws, stream));
  return MOE_OK;
}

moe_status_t moe_dense_ffn(const moe_layer_desc_t* d, const void* x, const moe_layer_weights_t* w, float* out,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  Plan p;
  ST_TRY(validate(d, &p));
  if (!p.residual) return fail(MOE_ERR_INVALID_ARGUMENT, "dense MLP needs mlp_type RESIDUAL");
  if (p.T == 0) return MOE_OK;
  PTR_TRY(x, "x");
  PTR_TRY(out, "out");
  ST_TRY(check_weights(p, w, false, true));
  ST_TRY(check_ws(ws, ws_bytes, p.total));
  ST_TRY(run_dense(p, x, w, out, ws, stream));
  return MOE_OK;
}

moe_status_t moe_combine(const moe_layer_desc_t* d, const float* y_disp, const int32_t* token_slot,
                         const float* topk_w, const float* dense_out, void* y, hipStream_t stream) {
  Plan p;
  ST_TRY(validate(d, &p));
  if (p.T == 0) return MOE_OK;
  PTR_TRY(token_slot, "token_slot");
  PTR_TRY(topk_w, "topk_w");
  PTR_TRY(y, "y");
  if (p.R_max > 0) PTR_TRY(y_disp, "y_disp");
  if (dense_out && !aligned16(dense_out)) return fail(MOE_ERR_INVALID_ARGUMENT, "dense_out is not 16-byte aligned");
  HIP_TRY(launch_combine(p.dtype, y_disp, token_slot, topk_w, p.k, dense_out, y, (int)p.T, p.H, stream),
          "combine");
  return MOE_OK;
}

moe_status_t moe_layer_forward_ex(const moe_layer_desc_t* d, const moe_layer_weights_t* w, const void* x, void* y,
                                  void* ws, size_t ws_bytes, hipStream_t stream, const moe_phase_events_t* ev) {
  Plan p;
  ST_TRY(validate(d, &p));
  if (p.T == 0) return MOE_OK;
  PTR_TRY(x, "x");
  PTR_TRY(y, "y");
  if (!w) return fail(MOE_ERR_INVALID_ARGUMENT, "weights is NULL");
  PTR_TRY(w->gate_w, "gate_w");
  if (w->gate_b && !aligned16(w->gate_b)) return fail(MOE_ERR_INVALID_ARGUMENT, "gate_b is not 16-byte aligned");
  ST_TRY(check_weights(p, w, true, p.residual));
  ST_TRY(check_ws(ws, ws_bytes, p.total));
  const moe_phase_events_t none{};
  const moe_phase_events_t& e = ev ? *ev : none;

  float* z = wsp<float>(ws, p.o_z);
  int* idx = wsp<int>(ws, p.o_idx);
  float* tw = wsp<float>(ws, p.o_w);
  int* demand = wsp<int>(ws, p.o_demand);
  int* offsets = wsp<int>(ws, p.o_off);
  int* slot_token = wsp<int>(ws, p.o_slot_token);
  int* token_slot = wsp<int>(ws, p.o_token_slot);

  void* y_fold = p.fold_combine ? y : nullptr;
  ST_TRY(record(e.gate_begin, stream));
  // the one-launch decode kernel finds its hidden rows marked unwritten (0xFFFF);
  // the one-launch dispatch its keys, block counts and slot_token zeroed (one
  // range: they lie back to back in the workspace, its end rounded up to 16
  // bytes inside the alignment gap after slot_token)
  const int zero16 =
      p.route_fused ? (int)((p.o_slot_token + (size_t)p.R_max * 4 - p.o_rank + 15) / 16) : 0;
  ST_TRY(run_gate_logits(p, x, w->gate_w, w->gate_b, z, stream, p.fused_decode ? wsp<unsigned>(ws, p.o_h) : nullptr,
                         p.fused_decode ? (int)(p.R_max * p.F * (int64_t)p.esz / 4) : 0,
                         p.zero_in_gate ? y : nullptr, p.route_fused ? wsp<char>(ws, p.o_rank) : nullptr, zero16));
  ST_TRY(record(e.gate_end, stream));
  ST_TRY(record(e.dispatch_begin, stream));
  RouteParams rp{};
  if (p.route_in_up) {
    // the first expert kernel routes the batch itself (every work-group in LDS)
    rp.z = z;
    rp.T = (int)p.T;
    rp.k = p.k;
    rp.E = p.E;
    rp.e_lo = p.e_lo;
    rp.E_loc = p.E_loc;
    rp.C = (int)std::min<int64_t>(p.C, INT32_MAX);
    rp.R_max = (int)p.R_max;
    rp.renorm = p.renorm ? 1 : 0;
    rp.idx = idx;
    rp.w = tw;
    rp.demand = demand;
    rp.offsets = offsets;
    rp.slot_token = slot_token;
    rp.token_slot = token_slot;
    rp.y_zero = y_fold;
    rp.y_esz = (int)p.esz;
  } else {
    // the GEMM path's tile lists come out of the dispatch kernel that finds the offsets
    const TilePlanArgs tp = tile_plan_args(p, ws, true);
    if (p.route_fused) {
      RouteDispatchArgs ra{};
      ra.z = z;
      ra.zsplit = p.gate_ksplit;
      ra.renorm = p.renorm ? 1 : 0;
      ra.probs = nullptr;
      ra.topk_w = tw;
      ra.idx = idx;
      ra.T = (int)p.T;
      ra.k = p.k;
      ra.E = p.E;
      ra.e_lo = p.e_lo;
      ra.E_loc = p.E_loc;
      ra.C = (int)std::min<int64_t>(p.C, INT32_MAX);
      ra.R_max = (int)p.R_max;
      ra.H = p.H;
      ra.y_esz = (int)p.esz;
      ra.keys = wsp<int>(ws, p.o_rank);
      ra.hist = wsp<int>(ws, p.o_blk);
      ra.demand = demand;
      ra.offsets = offsets;
      ra.slot_token = slot_token;
      ra.token_slot = token_slot;
      ra.y_zero = p.zero_in_gate ? nullptr : y_fold;
      HIP_TRY(launch_route_dispatch(ra, p.exp_decode ? nullptr : &tp, stream), "softmax/top-k + dispatch");
    } else {
      ST_TRY(run_dispatch(p, true, z, nullptr, tw, idx, demand, offsets, slot_token, token_slot,
                          p.zero_in_gate ? nullptr : y_fold, ws, stream, p.exp_decode ? nullptr : &tp));
    }
  }
  ST_TRY(record(e.dispatch_end, stream));
  ST_TRY(record(e.ffn_begin, stream));
  float* ydisp = wsp<float>(ws, p.o_ydisp);
  if (p.R_max > 0 || p.dense_in_experts || p.dense_in_decode)
    ST_TRY(run_experts(p, x, slot_token, offsets, w, ydisp, ws, stream, y_fold, slot_token, tw, ev,
                       p.route_in_up ? &rp : nullptr, true, true));
  float* dense = nullptr;
  if (p.residual) {
    dense = wsp<float>(ws, p.o_dense);
    if (!p.dense_in_experts && !p.dense_in_decode) ST_TRY(run_dense(p, x, w, dense, ws, stream));
  }
  ST_TRY(record(e.ffn_end, stream));
  ST_TRY(record(e.combine_begin, stream));
  if (!p.fold_combine)
    HIP_TRY(launch_combine(p.dtype, ydisp, token_slot, tw, p.k, dense, y, (int)p.T, p.H, stream),
            "combine");
  ST_TRY(record(e.combine_end, stream));
  return MOE_OK;
}

moe_status_t moe_layer_forward(const moe_layer_desc_t* d, const moe_layer_weights_t* w, const void* x, void* y,
                               void* ws, size_t ws_bytes, hipStream_t stream) {
  return moe_layer_forward_ex(d, w, x, y, ws, ws_bytes, stream, nullptr);
}

const char* moe_status_str(moe_status_t st) {
  switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_err; }

}  // extern "C"
