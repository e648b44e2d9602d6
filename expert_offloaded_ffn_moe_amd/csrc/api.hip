// C ABI of the MoE offload library: plans, residency pools, forward dispatch and
// the expert cache. See include/moe_offload.h for the contract of each call.
//
// Memory: per layer, one pinned device-mapped host pool holding every expert in
// the internal layout (page "我在 32GB 单卡上跑两万四千专家的 MoE:分层放置实测与三个坑",
// section "二、跑起来靠的是分层,不是激活": all experts pinned in host RAM), and
// hbm_slots HBM slots holding copies of the resident experts. A per-layer device
// table gives each expert's blob pointer: its HBM slot, or its host copy read in
// place over the host link (page "763B MoE 塞进两张 96GB 显卡：闲置专家丢进主机内存",
// sections "显存缺口从哪里来" and "同一个思路，vLLM 原生方案反而跑不通").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "host_logic.h"
#include "kernels.h"
#include "moe_offload.h"

using namespace moe;

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

#define HIP_TRY(expr)                                                                            \
  do {                                                                                           \
    hipError_t _e = (expr);                                                                      \
    if (_e != hipSuccess)                                                                        \
      return fail(MOE_E_HIP, std::string(#expr) + ": " + hipGetErrorString(_e));                 \
  } while (0)

struct Layer {
  uint8_t* host_pool = nullptr;      // E * L.bytes, pinned, host VA
  uint8_t* host_pool_dev = nullptr;  // device VA of host_pool
  uint8_t* hbm = nullptr;            // hbm_slots * L.bytes
  const uint8_t** d_wptr = nullptr;  // [E]
  int32_t* d_is_host = nullptr;      // [E]
  void* d_router_w = nullptr;        // [E][H]
  float* d_router_b = nullptr;       // [E]
  int64_t* d_counts_acc = nullptr;   // [E] since last cache update
  int64_t* d_stats = nullptr;        // [ST_COUNT]
  uint64_t* h_wptr_stage = nullptr;  // pinned [E] staging of the pointer table
  int32_t* h_ishost_stage = nullptr; // pinned [E]
  int64_t* h_counts_stage = nullptr; // pinned [E]
  std::vector<int32_t> slot_of;      // host mirror (a pending promotion already holds its slot)
  std::vector<double> score;
  std::vector<Promotion> pending;    // pipelined update: copies in flight, table still reads host
  bool loaded = false;
  int64_t bytes_copied = 0, promotions = 0, evictions = 0;
};

struct Workspace {
  float* logits = nullptr;   // [Tmax][E]
  float* xsum = nullptr;     // [Tmax][H/G]
  int32_t* ids = nullptr;    // [Tmax*k]
  float* wts = nullptr;      // [Tmax*k]
  int32_t* counts = nullptr; // [E]
  int32_t* offsets = nullptr;// [E+1]
  int32_t* sorted = nullptr; // [Tmax*k]
  int32_t* inv = nullptr;    // [Tmax*k]
  int32_t* active = nullptr; // [E]
  int32_t* n_active = nullptr;
  void* h = nullptr;         // [Tmax*k][I] act dtype
  float* hpart = nullptr;    // [Tmax*k][I/32]
  float* o = nullptr;        // [Tmax*k][H]
  int2* tiles = nullptr;     // [Tmax*k/64 + E] prefill GEMM row tiles
  WorkDesc* work = nullptr;  // [E] GEMV work descriptors
  const uint8_t** aptr = nullptr;  // [Tmax*k] expert blob per assignment (fused down + combine)
  int32_t* hist = nullptr;   // [ceil(Tmax/16)][E] block counts / bases of the multi-block grouping
  int32_t* act_pos = nullptr;  // [E]
  int32_t* n_tiles = nullptr;
  unsigned* route_cnt = nullptr;  // [64] arrival counters: [0] fused decode routing, [16] multi-block grouping
  uint8_t* stage = nullptr;       // [prefill_stage_slots][blob bytes] prefill staging slots
  const uint8_t** gptr = nullptr; // [E] blob table of a staged prefill forward
};

}  // namespace

struct moe_plan {
  moe_config cfg{};
  Layout L{};
  int device = 0;
  size_t act_size = 2;
  std::vector<Layer> layers;
  Workspace ws{};
  bool profiling = false;
  struct Rec {
    int kind;
    hipEvent_t a, b;
  };
  std::vector<Rec> recs;           // recorded launches
  std::vector<hipEvent_t> spare;   // reusable events
  std::vector<void*> dev_allocs;   // freed with hipFree
  std::vector<void*> host_allocs;  // freed with hipHostFree
  // Per-layer counters and pointer tables live in [layers][E] arrays, so that a
  // pipelined cache update moves all layers' counts and tables with one copy each.
  int64_t* d_counts_all = nullptr;
  const uint8_t** d_wptr_all = nullptr;
  int32_t* d_ishost_all = nullptr;
  // pipelined cache updates: pinned staging used by alternate updates, a copy
  // stream for the promotions, and the events that order them
  int64_t* h_counts_all[2] = {nullptr, nullptr};
  uint64_t* h_wptr_all[2] = {nullptr, nullptr};
  int32_t* h_ishost_all[2] = {nullptr, nullptr};
  std::vector<char> counts_staged[2];  // per layer: that staging set holds counts not yet used
  hipStream_t copy_stream = nullptr;
  hipEvent_t ev_counts[2] = {nullptr, nullptr}, ev_table[2] = {nullptr, nullptr}, ev_copy = nullptr;
  bool counts_recorded[2] = {false, false}, table_recorded[2] = {false, false}, copy_pending = false;
  unsigned update_seq = 0;
};

namespace {

moe_status dev_alloc(moe_plan* p, void** out, size_t bytes) {
  *out = nullptr;
  if (bytes == 0) bytes = 256;
  hipError_t e = hipMalloc(out, bytes);
  if (e != hipSuccess) {
    *out = nullptr;
    (void)hipGetLastError();
    return fail(MOE_E_NOMEM, "hipMalloc of " + std::to_string(bytes) + " bytes failed: " + hipGetErrorString(e));
  }
  p->dev_allocs.push_back(*out);
  return MOE_OK;
}

moe_status host_alloc(moe_plan* p, void** out, size_t bytes, unsigned flags) {
  *out = nullptr;
  if (bytes == 0) bytes = 256;
  hipError_t e = hipHostMalloc(out, bytes, flags);
  if (e != hipSuccess) {
    *out = nullptr;
    (void)hipGetLastError();
    return fail(MOE_E_HOST_NOMEM,
                "hipHostMalloc of " + std::to_string(bytes) + " bytes failed: " + hipGetErrorString(e));
  }
  p->host_allocs.push_back(*out);
  return MOE_OK;
}

void free_plan(moe_plan* p) {
  if (!p) return;
  (void)hipSetDevice(p->device);
  (void)hipDeviceSynchronize();
  for (auto& r : p->recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  for (hipEvent_t e : p->spare) (void)hipEventDestroy(e);
  for (hipEvent_t e : {p->ev_counts[0], p->ev_counts[1], p->ev_table[0], p->ev_table[1], p->ev_copy})
    if (e) (void)hipEventDestroy(e);
  if (p->copy_stream) (void)hipStreamDestroy(p->copy_stream);
  for (void* q : p->dev_allocs) (void)hipFree(q);
  for (void* q : p->host_allocs) (void)hipHostFree(q);
  delete p;
}

template <typename T>
moe_status alloc_as(moe_plan* p, T** out, size_t count) {
  void* v = nullptr;
  moe_status s = dev_alloc(p, &v, count * sizeof(T));
  *out = static_cast<T*>(v);
  return s;
}

hipEvent_t take_event(moe_plan* p) {
  if (!p->spare.empty()) {
    hipEvent_t e = p->spare.back();
    p->spare.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Event pair stamped by the dispatch of one kernel class when profiling is on;
// the record is kept when the timer goes out of scope.
struct KernelTimer {
  moe_plan* p;
  int kind;
  Timing tm;
  KernelTimer(moe_plan* p_, int kind_) : p(p_), kind(kind_) {
    if (!p->profiling) return;
    tm.start = take_event(p);
    tm.stop = take_event(p);
    if (!tm.start || !tm.stop) tm = Timing{};
  }
  ~KernelTimer() {
    if (tm.start && tm.stop) p->recs.push_back({kind, tm.start, tm.stop});
  }
};

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

// Upload the pointer table and host flags of a layer from its slot table.
moe_status push_tables(moe_plan* p, Layer& ly, hipStream_t s) {
  const int E = p->cfg.num_experts;
  for (int e = 0; e < E; ++e) {
    const int slot = ly.slot_of[e];
    const uint8_t* ptr = slot >= 0 ? ly.hbm + (size_t)slot * p->L.bytes : ly.host_pool_dev + (size_t)e * p->L.bytes;
    ly.h_wptr_stage[e] = reinterpret_cast<uint64_t>(ptr);
    ly.h_ishost_stage[e] = slot >= 0 ? 0 : 1;
  }
  HIP_TRY(hipMemcpyAsync(ly.d_wptr, ly.h_wptr_stage, sizeof(uint64_t) * E, hipMemcpyHostToDevice, s));
  HIP_TRY(hipMemcpyAsync(ly.d_is_host, ly.h_ishost_stage, sizeof(int32_t) * E, hipMemcpyHostToDevice, s));
  return MOE_OK;
}

// Wait for the promotion copies of a pipelined update and drop what it staged
// for layers [l0, l1): afterwards slot_of is exactly what push_tables uploads.
moe_status settle_pipelined(moe_plan* p, int l0, int l1) {
  if (p->copy_pending) {
    HIP_TRY(hipStreamSynchronize(p->copy_stream));
    p->copy_pending = false;
  }
  for (int l = l0; l < l1; ++l) p->layers[l].pending.clear();
  return MOE_OK;
}

// Pipelined cache update of layers [l0, l1) (see moe_cache_update): the policy
// reads the counts the previous update staged, so the host never waits for the
// step just enqueued; promotions are copied on the plan's copy stream and become
// visible at the next update.
moe_status cache_update_pipelined(moe_plan* p, int l0, int l1, double decay, int maxp, hipStream_t s) {
  const int E = p->cfg.num_experts, S = p->cfg.hbm_slots;
  const int cur = (int)(p->update_seq & 1u), prev = cur ^ 1;
  ++p->update_seq;
  const size_t off = (size_t)l0 * E, n = (size_t)(l1 - l0) * E;
  // (a) the previous update's promotions: forwards after this table upload read
  // them from HBM, so the upload waits for their copies (a device-side wait)
  if (p->copy_pending) {
    HIP_TRY(hipStreamWaitEvent(s, p->ev_copy, 0));
    p->copy_pending = false;
  }
  // (b) the counts of the forwards enqueued since the last update, for the next update
  if (p->counts_recorded[cur]) HIP_TRY(hipEventSynchronize(p->ev_counts[cur]));
  HIP_TRY(hipMemcpyAsync(p->h_counts_all[cur] + off, p->d_counts_all + off, sizeof(int64_t) * n,
                         hipMemcpyDeviceToHost, s));
  HIP_TRY(hipMemsetAsync(p->d_counts_all + off, 0, sizeof(int64_t) * n, s));
  HIP_TRY(hipEventRecord(p->ev_counts[cur], s));
  p->counts_recorded[cur] = true;
  // (c) the policy on the counts staged by the previous update (complete by now:
  // a whole step has been enqueued since)
  if (p->counts_recorded[prev]) HIP_TRY(hipEventSynchronize(p->ev_counts[prev]));
  if (p->table_recorded[cur]) HIP_TRY(hipEventSynchronize(p->ev_table[cur]));  // staging set free again
  std::vector<Promotion> promoted;
  std::vector<int32_t> evicted;
  bool copies = false;
  for (int l = l0; l < l1; ++l) {
    Layer& ly = p->layers[l];
    ly.pending.clear();
    if (p->counts_staged[prev][l]) {
      cache_policy_step(E, S, decay, maxp, p->h_counts_all[prev] + (size_t)l * E, ly.score.data(),
                        ly.slot_of.data(), &promoted, &evicted);
      ly.pending = promoted;
      ly.promotions += (int64_t)promoted.size();
      ly.evictions += (int64_t)evicted.size();
      ly.bytes_copied += (int64_t)promoted.size() * p->L.canonical_bytes;
      copies |= !promoted.empty();
    }
    p->counts_staged[prev][l] = 0;
    p->counts_staged[cur][l] = 1;
    // (d) the table: resident experts read HBM, except the promotions whose
    // copies are only being enqueued now
    uint64_t* wp = p->h_wptr_all[cur] + (size_t)l * E;
    int32_t* ih = p->h_ishost_all[cur] + (size_t)l * E;
    for (int e = 0; e < E; ++e) {
      const int slot = ly.slot_of[e];
      const uint8_t* ptr = slot >= 0 ? ly.hbm + (size_t)slot * p->L.bytes : ly.host_pool_dev + (size_t)e * p->L.bytes;
      wp[e] = reinterpret_cast<uint64_t>(ptr);
      ih[e] = slot >= 0 ? 0 : 1;
    }
    for (const Promotion& pr : ly.pending) {
      wp[pr.expert] = reinterpret_cast<uint64_t>(ly.host_pool_dev + (size_t)pr.expert * p->L.bytes);
      ih[pr.expert] = 1;
    }
  }
  HIP_TRY(hipMemcpyAsync(p->d_wptr_all + off, p->h_wptr_all[cur] + off, sizeof(uint64_t) * n,
                         hipMemcpyHostToDevice, s));
  HIP_TRY(hipMemcpyAsync(p->d_ishost_all + off, p->h_ishost_all[cur] + off, sizeof(int32_t) * n,
                         hipMemcpyHostToDevice, s));
  HIP_TRY(hipEventRecord(p->ev_table[cur], s));
  p->table_recorded[cur] = true;
  // (e) the copies: after the upload above, no forward enqueued later reads the
  // evicted experts' slots, and the ones enqueued before it have finished
  if (copies) {
    HIP_TRY(hipStreamWaitEvent(p->copy_stream, p->ev_table[cur], 0));
    for (int l = l0; l < l1; ++l) {
      Layer& ly = p->layers[l];
      for (const Promotion& pr : ly.pending)
        HIP_TRY(hipMemcpyAsync(ly.hbm + (size_t)pr.slot * p->L.bytes, ly.host_pool + (size_t)pr.expert * p->L.bytes,
                               p->L.bytes, hipMemcpyHostToDevice, p->copy_stream));
    }
    HIP_TRY(hipEventRecord(p->ev_copy, p->copy_stream));
    p->copy_pending = true;
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_E_INVALID: return "MOE_E_INVALID";
    case MOE_E_NOMEM: return "MOE_E_NOMEM";
    case MOE_E_HOST_NOMEM: return "MOE_E_HOST_NOMEM";
    case MOE_E_HIP: return "MOE_E_HIP";
    case MOE_E_UNSUPPORTED: return "MOE_E_UNSUPPORTED";
    case MOE_E_STATE: return "MOE_E_STATE";
  }
  return "MOE_E_UNKNOWN";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_expert_bytes(const moe_config* cfg, size_t* out) {
  if (!cfg || !out) return fail(MOE_E_INVALID, "null argument");
  const std::string why = check_config(*cfg);
  if (!why.empty()) return fail(MOE_E_INVALID, why);
  *out = (size_t)make_layout(cfg->hidden, cfg->inter, cfg->group_size).canonical_bytes;
  return MOE_OK;
}

moe_status moe_plan_create(const moe_config* cfg, moe_stream stream, moe_plan** out) {
  if (!out) return fail(MOE_E_INVALID, "out is null");
  *out = nullptr;
  if (!cfg) return fail(MOE_E_INVALID, "cfg is null");
  const std::string why = check_config(*cfg);
  if (!why.empty()) return fail(MOE_E_INVALID, why);
  (void)stream;

  moe_plan* p = new moe_plan();
  p->cfg = *cfg;
  if (p->cfg.gemm_min_tokens == 0) p->cfg.gemm_min_tokens = kGemmMinTokensDefault;
  p->L = make_layout(cfg->hidden, cfg->inter, cfg->group_size);
  p->act_size = cfg->act_dtype == MOE_ACT_BF16 ? 2 : 4;
  if (hipGetDevice(&p->device) != hipSuccess) {
    delete p;
    return fail(MOE_E_HIP, "hipGetDevice failed");
  }
  const int E = cfg->num_experts, H = cfg->hidden, I = cfg->inter, k = cfg->top_k, G = cfg->group_size;
  const size_t Tm = (size_t)cfg->max_tokens, A = Tm * k;
  moe_status st = MOE_OK;
#define TRY(x)          \
  do {                  \
    st = (x);           \
    if (st != MOE_OK) { \
      free_plan(p);     \
      return st;        \
    }                   \
  } while (0)
  p->layers.resize(cfg->num_layers);
  const size_t LE = (size_t)cfg->num_layers * E;
  TRY(alloc_as(p, &p->d_counts_all, LE));
  {
    void* v;
    TRY(dev_alloc(p, &v, sizeof(uint64_t) * LE));
    p->d_wptr_all = static_cast<const uint8_t**>(v);
    for (int b = 0; b < 2; ++b) {
      TRY(host_alloc(p, &v, sizeof(int64_t) * LE, 0));
      p->h_counts_all[b] = static_cast<int64_t*>(v);
      TRY(host_alloc(p, &v, sizeof(uint64_t) * LE, 0));
      p->h_wptr_all[b] = static_cast<uint64_t*>(v);
      TRY(host_alloc(p, &v, sizeof(int32_t) * LE, 0));
      p->h_ishost_all[b] = static_cast<int32_t*>(v);
      p->counts_staged[b].assign(cfg->num_layers, 0);
    }
  }
  TRY(alloc_as(p, &p->d_ishost_all, LE));
  if (hipStreamCreateWithFlags(&p->copy_stream, hipStreamNonBlocking) != hipSuccess) {
    free_plan(p);
    return fail(MOE_E_HIP, "creating the copy stream failed");
  }
  for (hipEvent_t* e : {&p->ev_counts[0], &p->ev_counts[1], &p->ev_table[0], &p->ev_table[1], &p->ev_copy})
    if (hipEventCreateWithFlags(e, hipEventDisableTiming) != hipSuccess) {
      free_plan(p);
      return fail(MOE_E_HIP, "creating cache-update events failed");
    }
  for (size_t li = 0; li < p->layers.size(); ++li) {
    Layer& ly = p->layers[li];
    void* v;
    TRY(host_alloc(p, &v, (size_t)E * p->L.bytes, hipHostMallocMapped | hipHostMallocNonCoherent));
    ly.host_pool = static_cast<uint8_t*>(v);
    void* dv = nullptr;
    if (hipHostGetDevicePointer(&dv, ly.host_pool, 0) != hipSuccess) {
      free_plan(p);
      return fail(MOE_E_HIP, "hipHostGetDevicePointer failed");
    }
    ly.host_pool_dev = static_cast<uint8_t*>(dv);
    if (cfg->hbm_slots > 0) {
      TRY(dev_alloc(p, &v, (size_t)cfg->hbm_slots * p->L.bytes));
      ly.hbm = static_cast<uint8_t*>(v);
    }
    ly.d_wptr = p->d_wptr_all + li * E;
    ly.d_is_host = p->d_ishost_all + li * E;
    TRY(dev_alloc(p, &ly.d_router_w, (size_t)E * H * p->act_size));
    TRY(alloc_as(p, &ly.d_router_b, E));
    ly.d_counts_acc = p->d_counts_all + li * E;
    TRY(alloc_as(p, &ly.d_stats, ST_COUNT));
    TRY(host_alloc(p, &v, sizeof(uint64_t) * E, 0));
    ly.h_wptr_stage = static_cast<uint64_t*>(v);
    TRY(host_alloc(p, &v, sizeof(int32_t) * E, 0));
    ly.h_ishost_stage = static_cast<int32_t*>(v);
    TRY(host_alloc(p, &v, sizeof(int64_t) * E, 0));
    ly.h_counts_stage = static_cast<int64_t*>(v);
    ly.slot_of.assign(E, -1);
    ly.score.assign(E, 0.0);
  }
  Workspace& w = p->ws;
  TRY(alloc_as(p, &w.logits, Tm * E));
  TRY(alloc_as(p, &w.xsum, Tm * (H / G)));
  TRY(alloc_as(p, &w.ids, A));
  TRY(alloc_as(p, &w.wts, A));
  TRY(alloc_as(p, &w.counts, E));
  TRY(alloc_as(p, &w.offsets, E + 1));
  TRY(alloc_as(p, &w.sorted, A));
  TRY(alloc_as(p, &w.inv, A));
  TRY(alloc_as(p, &w.active, E));
  TRY(alloc_as(p, &w.n_active, 64));
  TRY(dev_alloc(p, &w.h, A * I * p->act_size));
  TRY(alloc_as(p, &w.hpart, A * (I / 32)));
  TRY(alloc_as(p, &w.o, A * H));
  TRY(alloc_as(p, &w.route_cnt, 64));
  TRY(alloc_as(p, &w.tiles, A / kGemmRows + E + 1));
  TRY(alloc_as(p, &w.work, E));
  TRY(alloc_as(p, &w.aptr, A));
  TRY(alloc_as(p, &w.hist, (size_t)((Tm + kGroupTokens - 1) / kGroupTokens) * E));
  TRY(alloc_as(p, &w.act_pos, E));
  TRY(alloc_as(p, &w.n_tiles, 64));
  if (cfg->prefill_stage_slots > 0) {
    void* v = nullptr;
    TRY(dev_alloc(p, &v, (size_t)cfg->prefill_stage_slots * p->L.bytes));
    w.stage = static_cast<uint8_t*>(v);
    TRY(alloc_as(p, &w.gptr, E));
  }
#undef TRY
  if (hipMemset(w.route_cnt, 0, 64 * sizeof(unsigned)) != hipSuccess) {
    free_plan(p);
    return fail(MOE_E_HIP, "clearing arrival counters failed");
  }
  if (hipDeviceSynchronize() != hipSuccess) {
    free_plan(p);
    return fail(MOE_E_HIP, "device synchronize after allocation failed");
  }
  *out = p;
  return MOE_OK;
}

moe_status moe_plan_load_layer(moe_plan* p, int32_t layer, const moe_layer_weights* w, moe_stream stream) {
  if (!p || !w) return fail(MOE_E_INVALID, "null argument");
  if (layer < 0 || layer >= p->cfg.num_layers) return fail(MOE_E_INVALID, "layer out of range");
  if (!w->router_w || !w->experts) return fail(MOE_E_INVALID, "router_w and experts are required");
  const int E = p->cfg.num_experts, H = p->cfg.hidden, S = p->cfg.hbm_slots;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Layer& ly = p->layers[layer];

  std::vector<int32_t> slot_of(E, -1);
  int used = 0;
  for (int e = 0; e < E; ++e) {
    const bool res = w->resident ? (w->resident[e] != 0) : (e < S);
    if (res) {
      if (used >= S) return fail(MOE_E_INVALID, "more resident experts than hbm_slots");
      slot_of[e] = used++;
    }
  }
  HIP_TRY(hipSetDevice(p->device));
  HIP_TRY(hipStreamSynchronize(s));  // no queued work may still read this layer
  {
    moe_status st = settle_pipelined(p, layer, layer + 1);  // nor copy into it
    if (st != MOE_OK) return st;
    p->counts_staged[0][layer] = p->counts_staged[1][layer] = 0;
  }

  // repack every expert into the host pool, threads over experts
  const Layout L = p->L;
  const size_t cb = (size_t)L.canonical_bytes;
  unsigned nth = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  std::vector<std::thread> th;
  for (unsigned t = 0; t < nth; ++t)
    th.emplace_back([&, t] {
      for (int e = (int)t; e < E; e += (int)nth)
        repack_expert(L, w->experts + (size_t)e * cb, ly.host_pool + (size_t)e * L.bytes);
    });
  for (auto& x : th) x.join();

  for (int e = 0; e < E; ++e)
    if (slot_of[e] >= 0)
      HIP_TRY(hipMemcpyAsync(ly.hbm + (size_t)slot_of[e] * L.bytes, ly.host_pool + (size_t)e * L.bytes, L.bytes,
                             hipMemcpyHostToDevice, s));
  ly.slot_of = slot_of;
  ly.score.assign(E, 0.0);
  moe_status st = push_tables(p, ly, s);
  if (st != MOE_OK) return st;
  HIP_TRY(hipMemcpyAsync(ly.d_router_w, w->router_w, (size_t)E * H * p->act_size, hipMemcpyHostToDevice, s));
  if (w->router_b)
    HIP_TRY(hipMemcpyAsync(ly.d_router_b, w->router_b, sizeof(float) * E, hipMemcpyHostToDevice, s));
  else
    HIP_TRY(hipMemsetAsync(ly.d_router_b, 0, sizeof(float) * E, s));
  HIP_TRY(hipMemsetAsync(ly.d_counts_acc, 0, sizeof(int64_t) * E, s));
  HIP_TRY(hipMemsetAsync(ly.d_stats, 0, sizeof(int64_t) * ST_COUNT, s));
  HIP_TRY(hipStreamSynchronize(s));
  ly.bytes_copied = ly.promotions = ly.evictions = 0;
  ly.loaded = true;
  return MOE_OK;
}

moe_status moe_layer_forward(moe_plan* p, int32_t layer, int32_t T, const void* x, const float* logits_in, float* y,
                             const moe_routing* ro, moe_stream stream) {
  if (!p) return fail(MOE_E_INVALID, "plan is null");
  if (layer < 0 || layer >= p->cfg.num_layers) return fail(MOE_E_INVALID, "layer out of range");
  if (T < 0 || T > p->cfg.max_tokens) return fail(MOE_E_INVALID, "T out of range 0..max_tokens");
  if (T == 0) return MOE_OK;
  if (!x || !y) return fail(MOE_E_INVALID, "x and y are required");
  if (!aligned16(x) || !aligned16(y) || (logits_in && !aligned16(logits_in)))
    return fail(MOE_E_INVALID, "x, y and logits_in must be 16-byte aligned");
  Layer& ly = p->layers[layer];
  if (!ly.loaded) return fail(MOE_E_INVALID, "layer not loaded");
  const moe_config& c = p->cfg;
  const int E = c.num_experts, H = c.hidden, I = c.inter, k = c.top_k, G = c.group_size;
  const int bf16 = c.act_dtype == MOE_ACT_BF16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Workspace& w = p->ws;
  const int A = T * k;

  RouterArgs ra{};
  ra.x = x;
  ra.w = ly.d_router_w;
  ra.b = ly.d_router_b;
  ra.logits = w.logits;
  ra.xsum = bf16 ? w.xsum : nullptr;
  ra.T = T;
  ra.H = H;
  ra.E = E;
  ra.G = G;
  const float* logits = logits_in ? logits_in : w.logits;

  RouteArgs rt{};
  rt.logits = logits;
  rt.ids = w.ids;
  rt.wts = w.wts;
  rt.counts = w.counts;
  rt.offsets = w.offsets;
  rt.sorted = w.sorted;
  rt.inv = w.inv;
  rt.active = w.active;
  rt.n_active = w.n_active;
  rt.is_host = ly.d_is_host;
  rt.counts_acc = ly.d_counts_acc;
  rt.stats = ly.d_stats;
  rt.expert_bytes = p->L.canonical_bytes;
  rt.T = T;
  rt.E = E;
  rt.k = k;
  rt.wptr = ly.d_wptr;
  rt.hist = w.hist;
  rt.act_pos = w.act_pos;

  // one-launch routing for small batches (its router walks the tokens one by one;
  // past a few bf16 tokens the MFMA router and the multi-block grouping are faster)
  const bool decode = T <= (bf16 ? kRouteDecodeMaxTokensBf16 : kRouteSmallMaxTokens) && A <= kRouteSmallMaxAssign;
  const bool prefill = bf16 && c.gemm_min_tokens > 0 && T >= c.gemm_min_tokens && !decode;
  rt.work = prefill ? nullptr : w.work;
  // a few tokens: down projection and combine in one launch (K split over the free
  // waves), when its (H/64) x T workgroups still keep the CUs streaming; below that
  // the per-expert down GEMV spreads the same bytes over more workgroups
  const int down_splits = std::max(1, std::min(16 / k, (int)p->L.dn_groups));
  const bool fuse_small = bf16 && decode && T <= kDownCombMaxTokens && k <= 16;
  const bool fuse_down = fuse_small && (H / 64) * T >= kDownCombMinGroups;
  // fewer 64-row tiles than that: the same fusion on 16-row tiles of H, with the
  // K chunks of each wave spread over its four 16-lane quarters
  // (the token's k rows of h staged in LDS); K split over as many waves per slot
  // as still keep every workgroup resident in one round
  const bool fuse_narrow = fuse_small && !fuse_down && down_combine16_lds(k, I) <= kDownComb16MaxLds;
  int narrow_splits = std::max(1, std::min(16 / k, (int)p->L.dn_chunks / 4));
  while (narrow_splits > 1 && (int64_t)(H / 16) * T > 256LL * (kDownComb16WavesPerCU / (k * narrow_splits)))
    --narrow_splits;
  rt.aptr = (fuse_down || fuse_narrow) ? w.aptr : nullptr;
  if (prefill) {
    {
      RouterArgs rp = ra;  // logits only: the GEMMs take no group sums
      rp.router_blocks = 1;
      rp.xsum = nullptr;
      KernelTimer kt(p, MOE_K_ROUTER);
      if (!logits_in) launch_router_mfma(rp, kt.tm, s);
    }
    rt.tiles = w.tiles;
    rt.n_tiles = w.n_tiles;
    {
      KernelTimer kt(p, MOE_K_ROUTE);
      launch_topk_group(rt, w.route_cnt + 16, kt.tm, s);
    }
    // offloaded experts of this batch into the staging slots (when the plan has
    // them and the layer has offloaded experts); the GEMMs read the table it writes
    const uint8_t* const* gemm_wptr = ly.d_wptr;
    if (c.prefill_stage_slots > 0 && c.hbm_slots < E) {
      StageArgs sa{};
      sa.wptr = ly.d_wptr;
      sa.is_host = ly.d_is_host;
      sa.counts = w.counts;
      sa.act_pos = w.act_pos;
      sa.active = w.active;
      sa.n_active = w.n_active;
      sa.stage = w.stage;
      sa.gptr = w.gptr;
      sa.bytes = p->L.bytes;
      sa.E = E;
      sa.n_slots = c.prefill_stage_slots;
      KernelTimer kt(p, MOE_K_STAGE);
      launch_stage(sa, kt.tm, s);
      gemm_wptr = w.gptr;
    }
    GemmArgs gg{};
    gg.wptr = gemm_wptr;
    gg.tiles = w.tiles;
    gg.n_tiles = w.n_tiles;
    gg.offsets = w.offsets;
    gg.sorted = w.sorted;
    gg.a_src = static_cast<const uint16_t*>(x);
    gg.out = w.h;
    gg.off_codes = p->L.off_gu_codes;
    gg.off_scales = p->L.off_gu_scales;
    gg.chunks = (int)p->L.gu_chunks;
    gg.groups = (int)p->L.gu_groups;
    gg.ntiles_n = (int)p->L.gu_tiles;
    gg.K = H;
    gg.out_ld = I;
    gg.k = k;
    gg.G = G;
    gg.max_tiles = A / kGemmRows + std::min(E, A);
    {
      KernelTimer kt(p, MOE_K_GEMM_GATEUP);
      launch_gemm_gateup(gg, kt.tm, s);
    }
    GemmArgs gd = gg;
    gd.a_src = static_cast<const uint16_t*>(w.h);
    gd.out = w.o;
    gd.off_codes = p->L.off_dn_codes;
    gd.off_scales = p->L.off_dn_scales;
    gd.chunks = (int)p->L.dn_chunks;
    gd.groups = (int)p->L.dn_groups;
    gd.ntiles_n = (int)p->L.dn_tiles;
    gd.K = I;
    gd.out_ld = H;
    {
      KernelTimer kt(p, MOE_K_GEMM_DOWN);
      launch_gemm_down(gd, kt.tm, s);
    }
    CombineArgs ca{};
    ca.o = w.o;
    ca.wts = w.wts;
    ca.inv = w.inv;
    ca.y = y;
    ca.T = T;
    ca.H = H;
    ca.k = k;
    {
      KernelTimer kt(p, MOE_K_COMBINE);
      launch_combine(ca, kt.tm, s);
    }
    HIP_TRY(hipGetLastError());
  } else if (decode) {
    // router + group sums + top-k + grouping in one launch (8 expert rows per block)
    ra.router_blocks = logits_in ? 0 : (E + 7) / 8;
    KernelTimer kt(p, MOE_K_ROUTE);
    launch_route_decode(rt, ra, bf16, w.route_cnt, kt.tm, s);
  } else {
    {
      KernelTimer kt(p, MOE_K_ROUTER);
      if (bf16) {  // MFMA logits tiles (unless given) and the group sums, one launch
        ra.router_blocks = logits_in ? 0 : 1;
        launch_router_mfma(ra, kt.tm, s);
      } else {
        ra.router_blocks = logits_in ? 0 : (E + 3) / 4;
        launch_router(ra, bf16, kt.tm, s);
      }
    }
    KernelTimer kt(p, MOE_K_ROUTE);
    launch_topk_group(rt, w.route_cnt + 16, kt.tm, s);
  }

  if (!prefill) {  // decode / small-batch path: dequant-GEMVs over the active experts
    const int max_act = std::min(E, A);
    GemvArgs ga{};
    ga.work = w.work;
    ga.sorted = w.sorted;
    ga.in = x;
    ga.insum = w.xsum;
    ga.out = w.h;
    ga.outpart = w.hpart;
    ga.off_codes = p->L.off_gu_codes;
    ga.off_scales = p->L.off_gu_scales;
    ga.chunks = (int)p->L.gu_chunks;
    ga.groups = (int)p->L.gu_groups;
    ga.tiles = (int)p->L.gu_tiles;
    ga.H = H;
    ga.I = I;
    ga.G = G;
    ga.k = k;
    ga.T = T;
    {
      KernelTimer kt(p, MOE_K_GATEUP);
      launch_gateup(ga, bf16, std::min(T, 8), max_act * ga.tiles, kt.tm, s);
    }

    GemvArgs da = ga;
    da.in = w.h;
    da.insum = w.hpart;
    da.out = w.o;
    da.outpart = nullptr;
    da.off_codes = p->L.off_dn_codes;
    da.off_scales = p->L.off_dn_scales;
    da.chunks = (int)p->L.dn_chunks;
    da.groups = (int)p->L.dn_groups;
    da.tiles = (int)p->L.dn_tiles;
    if (fuse_down || fuse_narrow) {
      DownCombArgs dc{};
      dc.aptr = w.aptr;
      dc.inv = w.inv;
      dc.wts = w.wts;
      dc.h = w.h;
      dc.hpart = w.hpart;
      dc.y = y;
      dc.off_codes = p->L.off_dn_codes;
      dc.off_scales = p->L.off_dn_scales;
      dc.chunks = (int)p->L.dn_chunks;
      dc.groups = (int)p->L.dn_groups;
      dc.G = G;
      dc.H = H;
      dc.I = I;
      dc.k = k;
      dc.T = T;
      dc.splits = fuse_down ? down_splits : narrow_splits;
      KernelTimer kt(p, MOE_K_DOWN);
      if (fuse_down)
        launch_down_combine(dc, kt.tm, s);
      else
        launch_down_combine16(dc, kt.tm, s);
    } else {
      {
        KernelTimer kt(p, MOE_K_DOWN);
        launch_down(da, bf16, std::min(T, 8), max_act * da.tiles, kt.tm, s);
      }
      CombineArgs ca{};
      ca.o = w.o;
      ca.wts = w.wts;
      ca.inv = w.inv;
      ca.y = y;
      ca.T = T;
      ca.H = H;
      ca.k = k;
      KernelTimer kt(p, MOE_K_COMBINE);
      launch_combine(ca, kt.tm, s);
    }
    HIP_TRY(hipGetLastError());
  }

  if (ro) {
    if (ro->logits) HIP_TRY(hipMemcpyAsync(ro->logits, logits, sizeof(float) * T * E, hipMemcpyDeviceToDevice, s));
    if (ro->topk_ids) HIP_TRY(hipMemcpyAsync(ro->topk_ids, w.ids, sizeof(int32_t) * A, hipMemcpyDeviceToDevice, s));
    if (ro->topk_w) HIP_TRY(hipMemcpyAsync(ro->topk_w, w.wts, sizeof(float) * A, hipMemcpyDeviceToDevice, s));
    if (ro->counts) HIP_TRY(hipMemcpyAsync(ro->counts, w.counts, sizeof(int32_t) * E, hipMemcpyDeviceToDevice, s));
    if (ro->offsets)
      HIP_TRY(hipMemcpyAsync(ro->offsets, w.offsets, sizeof(int32_t) * (E + 1), hipMemcpyDeviceToDevice, s));
    if (ro->sorted) HIP_TRY(hipMemcpyAsync(ro->sorted, w.sorted, sizeof(int32_t) * A, hipMemcpyDeviceToDevice, s));
    if (ro->inv) HIP_TRY(hipMemcpyAsync(ro->inv, w.inv, sizeof(int32_t) * A, hipMemcpyDeviceToDevice, s));
  }
  return MOE_OK;
}

moe_status moe_cache_update(moe_plan* p, int32_t layer, const moe_cache_policy* pol, moe_stream stream) {
  if (!p) return fail(MOE_E_INVALID, "plan is null");
  if (layer < -1 || layer >= p->cfg.num_layers) return fail(MOE_E_INVALID, "layer out of range");
  if (p->cfg.hbm_slots == 0) return fail(MOE_E_STATE, "plan has no HBM slots to cache experts in");
  const double decay = pol ? pol->decay : 0.9;
  const int maxp = pol ? pol->max_promotions : 8;
  if (!(decay >= 0.0 && decay <= 1.0) || maxp < 0) return fail(MOE_E_INVALID, "bad policy");
  const int l0 = layer < 0 ? 0 : layer, l1 = layer < 0 ? p->cfg.num_layers : layer + 1;
  for (int l = l0; l < l1; ++l)
    if (!p->layers[l].loaded) return fail(MOE_E_INVALID, "layer not loaded");
  const int E = p->cfg.num_experts;
  hipStream_t s = static_cast<hipStream_t>(stream);
  HIP_TRY(hipSetDevice(p->device));
  if (pol && pol->overlap) return cache_update_pipelined(p, l0, l1, decay, maxp, s);
  for (int l = l0; l < l1; ++l) {
    Layer& ly = p->layers[l];
    HIP_TRY(hipMemcpyAsync(ly.h_counts_stage, ly.d_counts_acc, sizeof(int64_t) * E, hipMemcpyDeviceToHost, s));
    HIP_TRY(hipMemsetAsync(ly.d_counts_acc, 0, sizeof(int64_t) * E, s));
  }
  HIP_TRY(hipStreamSynchronize(s));
  std::vector<char> settled(p->cfg.num_layers, 0);  // layers whose pipelined promotions become visible now
  for (int l = l0; l < l1; ++l) settled[l] = !p->layers[l].pending.empty();
  {  // after pipelined updates: their copies done, their staged counts not lost
    moe_status st = settle_pipelined(p, l0, l1);
    if (st != MOE_OK) return st;
    for (int b = 0; b < 2; ++b)
      for (int l = l0; l < l1; ++l) {
        if (!p->counts_staged[b][l]) continue;
        HIP_TRY(hipEventSynchronize(p->ev_counts[b]));
        for (int e = 0; e < E; ++e) p->layers[l].h_counts_stage[e] += p->h_counts_all[b][(size_t)l * E + e];
        p->counts_staged[b][l] = 0;
      }
  }
  std::vector<Promotion> promoted;
  std::vector<int32_t> evicted;
  for (int l = l0; l < l1; ++l) {
    Layer& ly = p->layers[l];
    cache_policy_step(E, p->cfg.hbm_slots, decay, maxp, ly.h_counts_stage, ly.score.data(), ly.slot_of.data(),
                      &promoted, &evicted);
    if (promoted.empty()) {
      if (settled[l]) {
        moe_status st = push_tables(p, ly, s);
        if (st != MOE_OK) return st;
      }
      continue;
    }
    for (const Promotion& pr : promoted) {
      HIP_TRY(hipMemcpyAsync(ly.hbm + (size_t)pr.slot * p->L.bytes, ly.host_pool + (size_t)pr.expert * p->L.bytes,
                             p->L.bytes, hipMemcpyHostToDevice, s));
      ly.bytes_copied += p->L.canonical_bytes;
    }
    ly.promotions += (int64_t)promoted.size();
    ly.evictions += (int64_t)evicted.size();
    moe_status st = push_tables(p, ly, s);
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

moe_status moe_plan_stats(moe_plan* p, int32_t layer, moe_stats* out) {
  if (!p || !out) return fail(MOE_E_INVALID, "null argument");
  if (layer < -1 || layer >= p->cfg.num_layers) return fail(MOE_E_INVALID, "layer out of range");
  HIP_TRY(hipSetDevice(p->device));
  HIP_TRY(hipDeviceSynchronize());
  std::memset(out, 0, sizeof(*out));
  const int l0 = layer < 0 ? 0 : layer, l1 = layer < 0 ? p->cfg.num_layers : layer + 1;
  for (int l = l0; l < l1; ++l) {
    Layer& ly = p->layers[l];
    int64_t st[ST_COUNT];
    HIP_TRY(hipMemcpy(st, ly.d_stats, sizeof(st), hipMemcpyDeviceToHost));
    out->forwards += st[ST_FORWARDS];
    out->tokens += st[ST_TOKENS];
    out->hits += st[ST_HITS];
    out->misses += st[ST_MISSES];
    out->bytes_hbm += st[ST_BYTES_HBM];
    out->bytes_host += st[ST_BYTES_HOST];
    out->bytes_copied += ly.bytes_copied;
    out->promotions += ly.promotions;
    out->evictions += ly.evictions;
  }
  return MOE_OK;
}

moe_status moe_plan_reset_stats(moe_plan* p) {
  if (!p) return fail(MOE_E_INVALID, "plan is null");
  HIP_TRY(hipSetDevice(p->device));
  HIP_TRY(hipDeviceSynchronize());
  for (Layer& ly : p->layers) {
    HIP_TRY(hipMemset(ly.d_stats, 0, sizeof(int64_t) * ST_COUNT));
    ly.bytes_copied = ly.promotions = ly.evictions = 0;
  }
  HIP_TRY(hipDeviceSynchronize());
  return MOE_OK;
}

moe_status moe_plan_residency(moe_plan* p, int32_t layer, int32_t* slot_of) {
  if (!p || !slot_of) return fail(MOE_E_INVALID, "null argument");
  if (layer < 0 || layer >= p->cfg.num_layers) return fail(MOE_E_INVALID, "layer out of range");
  const Layer& ly = p->layers[layer];
  std::copy(ly.slot_of.begin(), ly.slot_of.end(), slot_of);
  for (const Promotion& pr : ly.pending) slot_of[pr.expert] = -1;  // copy in flight: still read from host
  return MOE_OK;
}

moe_status moe_plan_profile(moe_plan* p, int32_t enable) {
  if (!p) return fail(MOE_E_INVALID, "plan is null");
  if (enable) {
    HIP_TRY(hipDeviceSynchronize());
    for (auto& r : p->recs) {
      p->spare.push_back(r.a);
      p->spare.push_back(r.b);
    }
    p->recs.clear();
  }
  p->profiling = enable != 0;
  return MOE_OK;
}

moe_status moe_plan_kernel_times(moe_plan* p, moe_kernel_times* out) {
  if (!p || !out) return fail(MOE_E_INVALID, "null argument");
  std::memset(out, 0, sizeof(*out));
  HIP_TRY(hipSetDevice(p->device));
  HIP_TRY(hipDeviceSynchronize());
  for (auto& r : p->recs) {
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, r.a, r.b));
    if (r.kind >= 0 && r.kind < MOE_K_COUNT) {
      out->launches[r.kind] += 1;
      out->total_ms[r.kind] += ms;
    }
  }
  return MOE_OK;
}

void moe_plan_destroy(moe_plan* p) { free_plan(p); }

}  // extern "C"
