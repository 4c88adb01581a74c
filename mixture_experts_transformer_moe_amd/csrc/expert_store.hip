// Host-resident experts fetched by routing, with a device cache of hot experts.
//
// The review page's PR-MoE / MoS sections name the weights of many experts as
// the memory cost of MoE inference, and the MoE-MPMC summary keeps most experts
// off the GPU and brings in the ones the routing needs. Here every local
// expert's weights live in pinned host memory owned by the store; `slots`
// device slots hold copies of the experts the routing asks for most. The layer
// reads each expert through per-expert pointer tables (moe_layer_weights_t),
// so an expert in a slot is read from HBM and any other expert is read by the
// expert kernels straight from pinned host memory over the host link, only
// when the routing selects it.
//
// Residency follows an exponentially decayed demand count per expert: each
// moe_expert_store_update() folds in the demand the caller observed (e.g. the
// expert_demand output of moe_dispatch) and keeps the `slots` highest-scoring
// experts resident. Everything an update changes is enqueued on one stream in
// this order: (1) the pointers of experts leaving the cache switch back to host
// memory, (2) the newly cached experts are copied into their slots, (3) their
// pointers switch to the slots. Work enqueued earlier on the stream still reads
// the old placement; work enqueued later sees the new one.
//
// moe_expert_store_update_async() puts step (2) on a copy stream that first
// waits for step (1) on the compute stream, so the copies overlap with the
// layers enqueued meanwhile (which read the incoming experts from host memory,
// as before); moe_expert_store_commit() later makes the compute stream wait for
// the copies and enqueues step (3). A freed slot is only written after every
// read of it enqueued before step (1), and only read after step (3).
#include <math.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

#include "moe.h"
#include "api_internal.h"
#include "common.h"

using namespace moe;

namespace {

constexpr int kTableUpdates = 64;   // pointer updates carried by one launch (by value)

struct TableUpdate {
  int n;
  int idx[kTableUpdates];
  const void* ptr[kTableUpdates];
};

__global__ __launch_bounds__(64) void store_set_pointers(const void** tables, TableUpdate u) {
  const int i = threadIdx.x;
  if (i < u.n) tables[u.idx[i]] = u.ptr[i];
}

size_t round256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

struct moe_expert_store {
  int H = 0, F = 0, E = 0, e_lo = 0, E_loc = 0, esz = 0, slots = 0;
  size_t off_b1 = 0, off_w2 = 0, off_b2 = 0, expert_bytes = 0;   // layout of one expert (host and slot)
  size_t w1_bytes = 0, b1_bytes = 0, w2_bytes = 0, b2_bytes = 0;
  char* host = nullptr;          // pinned host memory, E_loc experts
  char* dev = nullptr;           // device slots
  const void** tables = nullptr; // device: w1, b1, w2, b2 pointer arrays of E_loc entries each
  std::vector<const void*> shadow;   // host copy of the tables as last enqueued
  std::vector<int> slot_of;          // local expert -> slot, -1 = host
  std::vector<int> expert_in;        // slot -> local expert, -1 = free
  std::vector<double> score;         // decayed demand
  double decay = 0.5;
  hipEvent_t evicted = nullptr;      // recorded on the compute stream after step (1)
  hipEvent_t copied = nullptr;       // recorded on the copy stream after step (2)
  bool pending = false;              // an asynchronous update awaits its commit
  std::vector<std::pair<int, const void*>> pending_place;
};

namespace {

const char* expert_part(const moe_expert_store* s, bool on_device, int e_or_slot, int part) {
  const char* base = on_device ? s->dev : s->host;
  const size_t off[4] = {0, s->off_b1, s->off_w2, s->off_b2};
  return base + (size_t)e_or_slot * s->expert_bytes + off[part];
}

// Enqueue pointer updates for (table part, expert, pointer) triples.
moe_status_t push_updates(moe_expert_store* s, const std::vector<std::pair<int, const void*>>& upd,
                          hipStream_t stream) {
  for (size_t i = 0; i < upd.size(); i += kTableUpdates) {
    TableUpdate u{};
    u.n = (int)std::min<size_t>(kTableUpdates, upd.size() - i);
    for (int j = 0; j < u.n; ++j) {
      u.idx[j] = upd[i + j].first;
      u.ptr[j] = upd[i + j].second;
      s->shadow[upd[i + j].first] = upd[i + j].second;
    }
    hipLaunchKernelGGL(store_set_pointers, dim3(1), dim3(64), 0, stream, s->tables, u);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return api_error(MOE_ERR_HIP, hipGetErrorString(e));
  }
  return MOE_OK;
}

void placement_updates(const moe_expert_store* s, int e, bool on_device, int slot,
                       std::vector<std::pair<int, const void*>>& upd) {
  for (int part = 0; part < 4; ++part)
    upd.emplace_back(part * s->E_loc + e, expert_part(s, on_device, on_device ? slot : e, part));
}

void release(moe_expert_store* s) {
  if (s->evicted) (void)hipEventDestroy(s->evicted);
  if (s->copied) (void)hipEventDestroy(s->copied);
  if (s->tables) (void)hipFree((void*)s->tables);
  if (s->dev) (void)hipFree(s->dev);
  if (s->host) (void)hipHostFree(s->host);
  delete s;
}

}  // namespace

extern "C" {

moe_status_t moe_expert_store_create(const moe_layer_desc_t* d, int32_t slots, moe_expert_store_t* out) {
  if (!out) return api_error(MOE_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  size_t ws = 0;
  const moe_status_t st = moe_workspace_size(d, &ws);   // validates the descriptor
  if (st != MOE_OK) return st;
  if (slots < 0 || slots > d->num_local_experts)
    return api_error(MOE_ERR_INVALID_ARGUMENT, "slots must be in [0, num_local_experts]");
  moe_expert_store* s = new (std::nothrow) moe_expert_store;
  if (!s) return api_error(MOE_ERR_HIP, "host allocation failed");
  s->H = d->hidden;
  s->F = d->ffn;
  s->E = d->num_experts;
  s->e_lo = d->first_local_expert;
  s->E_loc = d->num_local_experts;
  s->esz = d->dtype == MOE_DTYPE_F32 ? 4 : 2;
  s->slots = slots;
  s->w1_bytes = (size_t)s->F * s->H * s->esz;
  s->b1_bytes = (size_t)s->F * s->esz;
  s->w2_bytes = (size_t)s->H * s->F * s->esz;
  s->b2_bytes = (size_t)s->H * s->esz;
  s->off_b1 = round256(s->w1_bytes);
  s->off_w2 = s->off_b1 + round256(s->b1_bytes);
  s->off_b2 = s->off_w2 + round256(s->w2_bytes);
  s->expert_bytes = s->off_b2 + round256(s->b2_bytes);
  s->shadow.assign(4 * (size_t)s->E_loc, nullptr);
  s->slot_of.assign(s->E_loc, -1);
  s->expert_in.assign(slots, -1);
  s->score.assign(s->E_loc, 0.0);

  hipError_t e = hipHostMalloc((void**)&s->host, s->expert_bytes * s->E_loc, hipHostMallocDefault);
  if (e != hipSuccess) { release(s); return api_error(MOE_ERR_HIP, hipGetErrorString(e)); }
  memset(s->host, 0, s->expert_bytes * s->E_loc);
  if (slots > 0) {
    e = hipMalloc((void**)&s->dev, s->expert_bytes * slots);
    if (e != hipSuccess) { release(s); return api_error(MOE_ERR_HIP, hipGetErrorString(e)); }
  }
  e = hipMalloc((void**)&s->tables, sizeof(void*) * 4 * s->E_loc);
  if (e != hipSuccess) { release(s); return api_error(MOE_ERR_HIP, hipGetErrorString(e)); }
  e = hipEventCreateWithFlags(&s->evicted, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&s->copied, hipEventDisableTiming);
  if (e != hipSuccess) { release(s); return api_error(MOE_ERR_HIP, hipGetErrorString(e)); }
  for (int i = 0; i < s->E_loc; ++i)
    for (int part = 0; part < 4; ++part) s->shadow[part * s->E_loc + i] = expert_part(s, false, i, part);
  e = hipMemcpy((void*)s->tables, s->shadow.data(), sizeof(void*) * 4 * s->E_loc, hipMemcpyHostToDevice);
  if (e != hipSuccess) { release(s); return api_error(MOE_ERR_HIP, hipGetErrorString(e)); }
  *out = s;
  return MOE_OK;
}

moe_status_t moe_expert_store_destroy(moe_expert_store_t s) {
  if (!s) return MOE_OK;
  const hipError_t e = hipDeviceSynchronize();
  release(s);
  if (e != hipSuccess) return api_error(MOE_ERR_HIP, hipGetErrorString(e));
  return MOE_OK;
}

moe_status_t moe_expert_store_set_expert(moe_expert_store_t s, int32_t e, const void* w1, const void* b1,
                                         const void* w2, const void* b2) {
  if (!s) return api_error(MOE_ERR_INVALID_ARGUMENT, "store is NULL");
  if (e < 0 || e >= s->E_loc) return api_error(MOE_ERR_INVALID_ARGUMENT, "expert out of [0, num_local_experts)");
  if (!w1 || !b1 || !w2 || !b2) return api_error(MOE_ERR_INVALID_ARGUMENT, "expert weights are NULL");
  // no copy of the old contents may still be pending
  hipError_t err = hipDeviceSynchronize();
  if (err != hipSuccess) return api_error(MOE_ERR_HIP, hipGetErrorString(err));
  const void* src[4] = {w1, b1, w2, b2};
  const size_t bytes[4] = {s->w1_bytes, s->b1_bytes, s->w2_bytes, s->b2_bytes};
  for (int part = 0; part < 4; ++part) memcpy((void*)expert_part(s, false, e, part), src[part], bytes[part]);
  if (s->slot_of[e] >= 0) {
    for (int part = 0; part < 4; ++part) {
      err = hipMemcpy((void*)expert_part(s, true, s->slot_of[e], part), src[part], bytes[part],
                      hipMemcpyHostToDevice);
      if (err != hipSuccess) return api_error(MOE_ERR_HIP, hipGetErrorString(err));
    }
  }
  return MOE_OK;
}

moe_status_t moe_expert_store_weights(moe_expert_store_t s, moe_layer_weights_t* w) {
  if (!s || !w) return api_error(MOE_ERR_INVALID_ARGUMENT, "store or weights is NULL");
  w->w1 = w->b1 = w->w2 = w->b2 = nullptr;
  w->w1_experts = s->tables;
  w->b1_experts = s->tables + s->E_loc;
  w->w2_experts = s->tables + 2 * (size_t)s->E_loc;
  w->b2_experts = s->tables + 3 * (size_t)s->E_loc;
  return MOE_OK;
}

}  // extern "C"

namespace {

// Folds demand into the scores and moves the placement to the `slots` best
// experts (host bookkeeping only): evict gets the pointer updates of leaving
// experts, moves the (expert, slot) pairs to copy, place their pointer updates.
moe_status_t choose(moe_expert_store* s, const int32_t* demand, std::vector<std::pair<int, const void*>>& evict,
                    std::vector<std::pair<int, int>>& moves, std::vector<std::pair<int, const void*>>& place) {
  for (int i = 0; i < s->E_loc; ++i)
    if (demand[s->e_lo + i] < 0) return api_error(MOE_ERR_INVALID_ARGUMENT, "negative demand");
  for (int i = 0; i < s->E_loc; ++i) s->score[i] = s->decay * s->score[i] + demand[s->e_lo + i];
  // the `slots` highest scores (ties to the lower expert), demanded at least once
  std::vector<int> order(s->E_loc);
  for (int i = 0; i < s->E_loc; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return s->score[a] > s->score[b]; });
  std::vector<char> want(s->E_loc, 0);
  for (int r = 0; r < s->slots && r < s->E_loc; ++r)
    if (s->score[order[r]] > 0) want[order[r]] = 1;
  for (int sl = 0; sl < s->slots; ++sl) {
    const int e = s->expert_in[sl];
    if (e >= 0 && !want[e]) {
      placement_updates(s, e, false, -1, evict);
      s->slot_of[e] = -1;
      s->expert_in[sl] = -1;
    }
  }
  int sl = 0;
  for (int e = 0; e < s->E_loc; ++e) {
    if (!want[e] || s->slot_of[e] >= 0) continue;
    while (sl < s->slots && s->expert_in[sl] >= 0) ++sl;
    if (sl >= s->slots) break;
    s->expert_in[sl] = e;
    s->slot_of[e] = sl;
    moves.emplace_back(e, sl);
    placement_updates(s, e, true, sl, place);
  }
  return MOE_OK;
}

moe_status_t copy_in(moe_expert_store* s, const std::vector<std::pair<int, int>>& moves, hipStream_t stream) {
  for (const auto& m : moves) {
    const hipError_t err = hipMemcpyAsync((void*)expert_part(s, true, m.second, 0), expert_part(s, false, m.first, 0),
                                          s->expert_bytes, hipMemcpyHostToDevice, stream);
    if (err != hipSuccess) return api_error(MOE_ERR_HIP, hipGetErrorString(err));
  }
  return MOE_OK;
}

moe_status_t commit(moe_expert_store* s, hipStream_t stream) {
  if (!s->pending) return MOE_OK;
  const hipError_t err = hipStreamWaitEvent(stream, s->copied, 0);
  if (err != hipSuccess) return api_error(MOE_ERR_HIP, hipGetErrorString(err));
  s->pending = false;
  return push_updates(s, s->pending_place, stream);
}

}  // namespace

extern "C" {

moe_status_t moe_expert_store_update(moe_expert_store_t s, const int32_t* demand, hipStream_t stream,
                                     int32_t* copied) {
  if (!s || !demand) return api_error(MOE_ERR_INVALID_ARGUMENT, "store or demand is NULL");
  MOE_RETURN_IF_ERROR(commit(s, stream));
  std::vector<std::pair<int, const void*>> evict, place;
  std::vector<std::pair<int, int>> moves;
  MOE_RETURN_IF_ERROR(choose(s, demand, evict, moves, place));
  MOE_RETURN_IF_ERROR(push_updates(s, evict, stream));   // (1) leaving experts read from host memory from here on
  MOE_RETURN_IF_ERROR(copy_in(s, moves, stream));        // (2) after every earlier use of the freed slots (stream order)
  MOE_RETURN_IF_ERROR(push_updates(s, place, stream));   // (3) the copied experts read from their slots from here on
  if (copied) *copied = (int32_t)moves.size();
  return MOE_OK;
}

moe_status_t moe_expert_store_update_async(moe_expert_store_t s, const int32_t* demand, hipStream_t stream,
                                           hipStream_t copy_stream, int32_t* copied) {
  if (!s || !demand) return api_error(MOE_ERR_INVALID_ARGUMENT, "store or demand is NULL");
  if (copy_stream == stream) return api_error(MOE_ERR_INVALID_ARGUMENT, "copy_stream must differ from stream");
  MOE_RETURN_IF_ERROR(commit(s, stream));
  std::vector<std::pair<int, const void*>> evict, place;
  std::vector<std::pair<int, int>> moves;
  MOE_RETURN_IF_ERROR(choose(s, demand, evict, moves, place));
  MOE_RETURN_IF_ERROR(push_updates(s, evict, stream));   // (1) on the compute stream
  hipError_t err = hipEventRecord(s->evicted, stream);
  if (err == hipSuccess) err = hipStreamWaitEvent(copy_stream, s->evicted, 0);
  if (err != hipSuccess) return api_error(MOE_ERR_HIP, hipGetErrorString(err));
  MOE_RETURN_IF_ERROR(copy_in(s, moves, copy_stream));  // (2) on the copy stream, after (1)
  err = hipEventRecord(s->copied, copy_stream);
  if (err != hipSuccess) return api_error(MOE_ERR_HIP, hipGetErrorString(err));
  s->pending_place = place;                 // (3) at the commit
  s->pending = true;
  if (copied) *copied = (int32_t)moves.size();
  return MOE_OK;
}

moe_status_t moe_expert_store_commit(moe_expert_store_t s, hipStream_t stream) {
  if (!s) return api_error(MOE_ERR_INVALID_ARGUMENT, "store is NULL");
  return commit(s, stream);
}

moe_status_t moe_expert_store_residency(moe_expert_store_t s, int32_t* slot_of) {
  if (!s || !slot_of) return api_error(MOE_ERR_INVALID_ARGUMENT, "store or slot_of is NULL");
  for (int i = 0; i < s->E_loc; ++i) slot_of[i] = s->slot_of[i];
  return MOE_OK;
}

}  // extern "C"
