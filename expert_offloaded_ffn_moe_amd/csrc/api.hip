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

#include <linux/mempolicy.h>
#include <sched.h>
#include <sys/syscall.h>
#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>
#include <type_traits>
#include <vector>

#include "host_ffn.h"
#include "host_logic.h"
#include "kernels.h"
#include "moe_offload.h"

using namespace moe;

namespace {

thread_local std::string g_last_error;

// The workspace of moe_layer_forward_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends. Host code never passes its name to a
// kernel (on the host the name is only a stand-in): each device's address comes
// from hipGetSymbolAddress, taken once with that device current, and only that
// address is used.
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};

// moe_debug_fail_alloc: countdown to the device (0) / pinned host (1) allocation that fails
std::atomic<int> g_fail_alloc[2] = {{0}, {0}};
// allocations currently held: device (0), pinned host (1)
std::atomic<int64_t> g_live[2] = {{0}, {0}};

bool injected_failure(int kind) {
  int v = g_fail_alloc[kind].load();
  while (v > 0)
    if (g_fail_alloc[kind].compare_exchange_weak(v, v - 1)) return v == 1;
  return false;
}

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
  int host_mode = MOE_HOST_COMPUTE_NONE;  // moe_plan_set_host_compute
  int64_t host_computed = 0;             // unique experts computed by the host cores, summed over forwards
  // predictive prefetch (moe_prefetch): slots, their occupants and the copy list on
  // the device; the prefetch's completion as an event
  uint8_t* pf_slots = nullptr;   // [prefetch_slots][L.bytes]
  int32_t* d_pf_occ = nullptr;   // [prefetch_slots] expert per slot, -1 none
  int32_t* d_pf_list = nullptr;  // [prefetch_slots + 1] slots to fill, then their count
  hipEvent_t ev_prefetch = nullptr;
  bool pf_pending = false;
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
  int debug_ws = 0;                // MOE_DEBUG_WORKSPACE: 1 = poison the float workspace at create, 2 = and per forward
  int gpu_node = -1, pool_node = -1, numa_bound = 0;
  int64_t host_pool_bytes = 0, hbm_slot_bytes = 0, workspace_bytes = 0, dev_bytes = 0;
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
  // host computation of experts: worker pool, pinned staging of the routing results,
  // the activations and the host-computed o rows, and host scratch for packed rows
  HostPool* host_pool = nullptr;
  int32_t* hs_route = nullptr;  // n_active[2] | active[E] | offsets[E+1] | sorted[Tmax*k]; mapped, coherent
  void* hs_x = nullptr;         // [Tmax][H] act dtype; mapped, coherent
  int32_t* hs_route_dev = nullptr;  // device addresses of the two
  void* hs_x_dev = nullptr;
  float* hs_o = nullptr;        // [Tmax*k][H]
  std::vector<float> hx, hh;    // packed x rows [Tmax*k][H], h rows [Tmax*k][I]
  hipEvent_t ev_route = nullptr;  // the routing results and x are in the host staging
  hipEvent_t ev_host_o = nullptr; // the last host part's o copies have read hs_o
  bool host_o_pending = false;
  // predictive prefetch: its stream, router logits and arrival counter (prefetches of
  // all layers run in order on the one stream), and the caller's point it starts after
  hipStream_t pf_stream = nullptr;
  float* pf_logits = nullptr;       // [Tmax][E]
  unsigned* pf_counter = nullptr;   // [1]
  hipEvent_t ev_caller = nullptr;
};

namespace {

moe_status dev_alloc(moe_plan* p, void** out, size_t bytes) {
  *out = nullptr;
  if (bytes == 0) bytes = 256;
  if (injected_failure(0)) return fail(MOE_E_NOMEM, "hipMalloc of " + std::to_string(bytes) + " bytes failed (injected)");
  hipError_t e = hipMalloc(out, bytes);
  if (e != hipSuccess) {
    *out = nullptr;
    (void)hipGetLastError();
    return fail(MOE_E_NOMEM, "hipMalloc of " + std::to_string(bytes) + " bytes failed: " + hipGetErrorString(e));
  }
  p->dev_allocs.push_back(*out);
  ++g_live[0];
  p->dev_bytes += (int64_t)bytes;
  return MOE_OK;
}

moe_status host_alloc(moe_plan* p, void** out, size_t bytes, unsigned flags) {
  *out = nullptr;
  if (bytes == 0) bytes = 256;
  if (injected_failure(1))
    return fail(MOE_E_HOST_NOMEM, "hipHostMalloc of " + std::to_string(bytes) + " bytes failed (injected)");
  hipError_t e = hipHostMalloc(out, bytes, flags);
  if (e != hipSuccess) {
    *out = nullptr;
    (void)hipGetLastError();
    return fail(MOE_E_HOST_NOMEM,
                "hipHostMalloc of " + std::to_string(bytes) + " bytes failed: " + hipGetErrorString(e));
  }
  p->host_allocs.push_back(*out);
  ++g_live[1];
  return MOE_OK;
}

// Host NUMA node closest to `device` (-1 if not reported). A failed query leaves
// no error state behind for the caller's next HIP call.
int gpu_numa_node(int device) {
  int node = -1;
  if (hipDeviceGetAttribute(&node, hipDeviceAttributeHostNumaId, device) != hipSuccess) {
    (void)hipGetLastError();
    return -1;
  }
  return node;
}

// NUMA node of the page at `addr` (-1 if the system does not say).
int page_node(const void* addr) {
  int node = -1;
  if (syscall(SYS_get_mempolicy, &node, nullptr, 0, const_cast<void*>(addr), MPOL_F_NODE | MPOL_F_ADDR) != 0)
    return -1;
  return node;
}

// A host pool on the GPU's NUMA node (page "763B MoE 塞进两张 96GB 显卡：闲置专家丢进
// 主机内存", section "PCIe 拓扑：容易被忽略的性能变量": host memory on a remote node
// slowed the host link). When the device reports its closest node, the calling
// thread's memory policy prefers that node while the pool is allocated and pinned
// (hipHostMallocNumaUser makes HIP follow the thread's policy), and is restored after.
moe_status host_alloc_numa(moe_plan* p, void** out, size_t bytes, unsigned flags) {
  if (p->gpu_node < 0 || p->gpu_node >= 1024) return host_alloc(p, out, bytes, flags);
  constexpr unsigned long kMaxNode = 1024 + 1;  // bits of the masks below, plus one (the kernel's convention)
  unsigned long old_mask[16] = {0}, mask[16] = {0};
  int old_mode = MPOL_DEFAULT;
  if (syscall(SYS_get_mempolicy, &old_mode, old_mask, kMaxNode, nullptr, 0) != 0)
    return host_alloc(p, out, bytes, flags);
  mask[p->gpu_node / 64] = 1ul << (p->gpu_node % 64);
  if (syscall(SYS_set_mempolicy, MPOL_PREFERRED, mask, kMaxNode) != 0) return host_alloc(p, out, bytes, flags);
  void* q = nullptr;
  const bool injected = injected_failure(1);
  hipError_t e = injected ? hipErrorOutOfMemory : hipHostMalloc(&q, bytes, flags | hipHostMallocNumaUser);
  (void)syscall(SYS_set_mempolicy, old_mode, old_mode == MPOL_DEFAULT ? nullptr : old_mask, kMaxNode);
  if (injected)
    return fail(MOE_E_HOST_NOMEM, "hipHostMalloc of " + std::to_string(bytes) + " bytes failed (injected)");
  if (e != hipSuccess) {  // this allocation path refused: the plain one decides
    (void)hipGetLastError();
    return host_alloc(p, out, bytes, flags);
  }
  p->host_allocs.push_back(q);
  ++g_live[1];
  *out = q;
  p->numa_bound = 1;
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
  if (p->ev_route) (void)hipEventDestroy(p->ev_route);
  if (p->ev_host_o) (void)hipEventDestroy(p->ev_host_o);
  if (p->pf_stream) (void)hipStreamDestroy(p->pf_stream);
  if (p->ev_caller) (void)hipEventDestroy(p->ev_caller);
  for (Layer& ly : p->layers)
    if (ly.ev_prefetch) (void)hipEventDestroy(ly.ev_prefetch);
  delete p->host_pool;
  for (void* q : p->dev_allocs) (void)hipFree(q);
  for (void* q : p->host_allocs) (void)hipHostFree(q);
  g_live[0] -= (int64_t)p->dev_allocs.size();
  g_live[1] -= (int64_t)p->host_allocs.size();
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

// Work on `s` that reads or rewrites a layer's table, or its prefetch slots, waits
// on the device for the layer's pending prefetch.
moe_status wait_prefetch(moe_plan* p, Layer& ly, hipStream_t s) {
  if (ly.pf_pending) {
    HIP_TRY(hipStreamWaitEvent(s, ly.ev_prefetch, 0));
    ly.pf_pending = false;
  }
  (void)p;
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
  for (int l = l0; l < l1; ++l) {
    moe_status st = wait_prefetch(p, p->layers[l], s);
    if (st != MOE_OK) return st;
  }
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

// The device address of `scratch` on the current device `dev`, taken (and its
// arrival counters cleared) on the first call for that device. nullptr on failure.
uint8_t* scratch_on(int dev, std::string* why) {
  if (dev < 0 || dev >= kMaxDevices) {
    *why = "device index out of range for the static workspace";
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev]) return g_scratch_ptr[dev];
  void* ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr) {
    (void)hipGetLastError();
    *why = std::string("hipGetSymbolAddress of the static workspace failed: ") + hipGetErrorString(e);
    return nullptr;
  }
  // the routing kernels' arrival counters (the first 256 bytes) start at zero; each
  // launch leaves them at zero again when its last block finishes
  launch_fill32(ptr, 0u, 64, nullptr);
  e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    *why = std::string("clearing the static workspace failed: ") + hipGetErrorString(e);
    return nullptr;
  }
  g_scratch_ptr[dev] = static_cast<uint8_t*>(ptr);
  return g_scratch_ptr[dev];
}

// A forward workspace for T tokens laid out from `base` in 256-byte aligned pieces,
// arrival counters first; returns its size (base == nullptr: the size only). The
// prefill staging slots stay the plan's own.
size_t carve_workspace(const moe_plan* p, int T, uint8_t* base, Workspace* w) {
  const moe_config& c = p->cfg;
  const size_t E = c.num_experts, A = (size_t)T * c.top_k;
  size_t off = 0;
  auto take = [&](auto** ptr, size_t bytes) {
    using Ptr = std::remove_pointer_t<decltype(ptr)>;
    *ptr = base ? reinterpret_cast<Ptr>(base + off) : nullptr;
    off += (bytes + 255) / 256 * 256;
  };
  take(&w->route_cnt, 64 * sizeof(unsigned));
  take(&w->n_active, 64 * sizeof(int32_t));
  take(&w->n_tiles, 64 * sizeof(int32_t));
  take(&w->logits, (size_t)T * E * sizeof(float));
  take(&w->xsum, (size_t)T * (c.hidden / c.group_size) * sizeof(float));
  take(&w->ids, A * sizeof(int32_t));
  take(&w->wts, A * sizeof(float));
  take(&w->counts, E * sizeof(int32_t));
  take(&w->offsets, (E + 1) * sizeof(int32_t));
  take(&w->sorted, A * sizeof(int32_t));
  take(&w->inv, A * sizeof(int32_t));
  take(&w->active, E * sizeof(int32_t));
  take(&w->act_pos, E * sizeof(int32_t));
  take(&w->work, E * sizeof(WorkDesc));
  take(&w->aptr, A * sizeof(uint8_t*));
  take(&w->tiles, (A / kGemmRows + E + 1) * sizeof(int2));
  take(&w->hist, (size_t)((T + kGroupTokens - 1) / kGroupTokens) * E * sizeof(int32_t));
  take(&w->hpart, A * (c.inter / 32) * sizeof(float));
  take(&w->o, A * c.hidden * sizeof(float));
  uint8_t* h = nullptr;
  take(&h, A * c.inter * p->act_size);
  w->h = h;
  w->stage = p->ws.stage;
  w->gptr = p->ws.gptr;
  return off;
}

// Arguments of one layer's weights: router and experts given, initial HBM set within the slots.
moe_status check_layer_args(const moe_config& c, const moe_layer_weights* w, const int32_t* initial_hbm) {
  if (!w || !w->router_w || !w->experts) return fail(MOE_E_INVALID, "router_w and experts are required");
  if (initial_hbm) {
    int n = 0;
    for (int e = 0; e < c.num_experts; ++e) n += initial_hbm[e] != 0;
    if (n > c.hbm_slots) return fail(MOE_E_INVALID, "more initially resident experts than hbm_slots");
  }
  return MOE_OK;
}

// Debug mode: the float workspace buffers (logits, group sums, h, its chunk sums, o)
// filled with a pattern that is a quiet NaN both as fp32 and as each of its bf16
// halves, so that a kernel reading values no launch of the current forward wrote
// turns the output into NaN. The index buffers are never filled.
void poison_workspace(moe_plan* p, hipStream_t s) {
  const moe_config& c = p->cfg;
  const size_t Tm = (size_t)c.max_tokens, A = Tm * c.top_k;
  const uint32_t nan2 = 0x7FC07FC0u;
  Workspace& w = p->ws;
  launch_fill32(w.logits, nan2, Tm * c.num_experts, s);
  launch_fill32(w.xsum, nan2, Tm * (c.hidden / c.group_size), s);
  launch_fill32(w.h, nan2, A * c.inter * p->act_size / 4, s);
  launch_fill32(w.hpart, nan2, A * (c.inter / 32), s);
  launch_fill32(w.o, nan2, A * c.hidden, s);
}

moe_status load_layer_impl(moe_plan* p, int layer, const moe_layer_weights* w, const int32_t* initial_hbm,
                           hipStream_t s) {
  const int E = p->cfg.num_experts, H = p->cfg.hidden, S = p->cfg.hbm_slots;
  Layer& ly = p->layers[layer];
  std::vector<int32_t> slot_of(E, -1);
  int used = 0;
  for (int e = 0; e < E; ++e)
    if (initial_hbm ? (initial_hbm[e] != 0) : (e < S)) slot_of[e] = used++;
  HIP_TRY(hipSetDevice(p->device));
  HIP_TRY(hipStreamSynchronize(s));  // no queued work may still read this layer
  if (p->pf_stream) HIP_TRY(hipStreamSynchronize(p->pf_stream));  // nor a prefetch copy from it
  ly.pf_pending = false;
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
  {
    moe_status st = push_tables(p, ly, s);
    if (st != MOE_OK) return st;
  }
  HIP_TRY(hipMemcpyAsync(ly.d_router_w, w->router_w, (size_t)E * H * p->act_size, hipMemcpyHostToDevice, s));
  if (w->router_b)
    HIP_TRY(hipMemcpyAsync(ly.d_router_b, w->router_b, sizeof(float) * E, hipMemcpyHostToDevice, s));
  else
    HIP_TRY(hipMemsetAsync(ly.d_router_b, 0, sizeof(float) * E, s));
  HIP_TRY(hipMemsetAsync(ly.d_counts_acc, 0, sizeof(int64_t) * E, s));
  HIP_TRY(hipMemsetAsync(ly.d_stats, 0, sizeof(int64_t) * ST_COUNT, s));
  if (ly.d_pf_occ) launch_fill32(ly.d_pf_occ, 0xFFFFFFFFu, (size_t)p->cfg.prefetch_slots, s);
  HIP_TRY(hipStreamSynchronize(s));
  ly.bytes_copied = ly.promotions = ly.evictions = 0;
  ly.loaded = true;
  return MOE_OK;
}


// Workspace buffers of a forward. Every launch of moe_layer_forward names the
// buffers it reads and writes; a read of a buffer that no earlier launch of the
// same forward wrote would take whatever an earlier forward (or the allocator's
// previous owner of the memory) left there, so the dispatch refuses to enqueue it.
// A launch that writes a buffer and reads it back itself (the routing kernels'
// last blocks reading the logits their router blocks wrote) lists it as written.
// Partial writes are documented at the kernels: a writer covers the range its
// readers use (the GEMV work slots up to min(E, T*k), act_pos where counts > 0).
enum : uint32_t {
  WB_LOGITS = 1u << 0, WB_XSUM = 1u << 1, WB_IDS = 1u << 2, WB_WTS = 1u << 3, WB_COUNTS = 1u << 4,
  WB_OFFSETS = 1u << 5, WB_SORTED = 1u << 6, WB_INV = 1u << 7, WB_ACTIVE = 1u << 8, WB_NACTIVE = 1u << 9,
  WB_H = 1u << 10, WB_HPART = 1u << 11, WB_O = 1u << 12, WB_TILES = 1u << 13, WB_NTILES = 1u << 14,
  WB_WORK = 1u << 15, WB_APTR = 1u << 16, WB_HIST = 1u << 17, WB_ACTPOS = 1u << 18, WB_STAGE = 1u << 19,
  WB_GPTR = 1u << 20, WB_COUNT_ = 21
};

const char* const kWbNames[WB_COUNT_] = {"logits", "xsum",   "ids",   "wts",     "counts", "offsets", "sorted",
                                         "inv",    "active", "n_active", "h",     "hpart",  "o",       "tiles",
                                         "n_tiles", "work",  "aptr",  "hist",    "act_pos", "stage",  "gptr"};

struct WsTrack {
  uint32_t written = 0;
  std::string err;
  bool launch(const char* kernel, uint32_t reads, uint32_t writes) {
    const uint32_t missing = reads & ~written;
    written |= writes;
    if (!missing) return true;
    err = std::string(kernel) + " reads";
    for (int b = 0; b < WB_COUNT_; ++b)
      if (missing & (1u << b)) err += std::string(" ") + kWbNames[b];
    err += " before this forward writes it";
    return false;
  }
};

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
  *out = (size_t)make_layout(cfg->hidden, cfg->inter, cfg->group_size, cfg_bits(*cfg)).canonical_bytes;
  return MOE_OK;
}

moe_status moe_plan_create(const moe_config* cfg, const moe_layer_weights* layers, const int32_t* initial_hbm,
                           moe_stream stream, moe_plan** out) {
  if (!out) return fail(MOE_E_INVALID, "out is null");
  *out = nullptr;
  if (!cfg) return fail(MOE_E_INVALID, "cfg is null");
  const std::string why = check_config(*cfg);
  if (!why.empty()) return fail(MOE_E_INVALID, why);
  if (layers) {
    for (int l = 0; l < cfg->num_layers; ++l) {
      moe_status st = check_layer_args(*cfg, &layers[l], initial_hbm ? initial_hbm + (size_t)l * cfg->num_experts
                                                                     : nullptr);
      if (st != MOE_OK) return st;
    }
  }

  moe_plan* p = new moe_plan();
  p->cfg = *cfg;
  if (p->cfg.gemm_min_tokens == 0) p->cfg.gemm_min_tokens = kGemmMinTokensDefault;
  p->L = make_layout(cfg->hidden, cfg->inter, cfg->group_size, cfg_bits(*cfg));
  p->act_size = cfg->act_dtype == MOE_ACT_BF16 ? 2 : 4;
  if (hipGetDevice(&p->device) != hipSuccess) {
    delete p;
    return fail(MOE_E_HIP, "hipGetDevice failed");
  }
  p->gpu_node = gpu_numa_node(p->device);
  {
    const char* dbg = std::getenv("MOE_DEBUG_WORKSPACE");
    p->debug_ws = dbg ? std::atoi(dbg) : 0;
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
    TRY(host_alloc_numa(p, &v, (size_t)E * p->L.bytes, hipHostMallocMapped | hipHostMallocNonCoherent));
    ly.host_pool = static_cast<uint8_t*>(v);
    p->host_pool_bytes += (int64_t)E * p->L.bytes;
    void* dv = nullptr;
    if (hipHostGetDevicePointer(&dv, ly.host_pool, 0) != hipSuccess) {
      free_plan(p);
      return fail(MOE_E_HIP, "hipHostGetDevicePointer failed");
    }
    ly.host_pool_dev = static_cast<uint8_t*>(dv);
    if (cfg->hbm_slots > 0) {
      TRY(dev_alloc(p, &v, (size_t)cfg->hbm_slots * p->L.bytes));
      ly.hbm = static_cast<uint8_t*>(v);
      p->hbm_slot_bytes += (int64_t)cfg->hbm_slots * p->L.bytes;
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
    if (cfg->prefetch_slots > 0) {
      TRY(dev_alloc(p, &v, (size_t)cfg->prefetch_slots * p->L.bytes));
      ly.pf_slots = static_cast<uint8_t*>(v);
      p->hbm_slot_bytes += (int64_t)cfg->prefetch_slots * p->L.bytes;
      TRY(alloc_as(p, &ly.d_pf_occ, (size_t)cfg->prefetch_slots));
      TRY(alloc_as(p, &ly.d_pf_list, (size_t)cfg->prefetch_slots + 1));
      launch_fill32(ly.d_pf_occ, 0xFFFFFFFFu, (size_t)cfg->prefetch_slots, nullptr);
      if (hipEventCreateWithFlags(&ly.ev_prefetch, hipEventDisableTiming) != hipSuccess) {
        free_plan(p);
        return fail(MOE_E_HIP, "creating prefetch events failed");
      }
    }
  }
  if (cfg->prefetch_slots > 0) {
    TRY(alloc_as(p, &p->pf_logits, Tm * E));
    TRY(alloc_as(p, &p->pf_counter, 64));
    if (hipMemset(p->pf_counter, 0, 64 * sizeof(unsigned)) != hipSuccess ||
        hipStreamCreateWithFlags(&p->pf_stream, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&p->ev_caller, hipEventDisableTiming) != hipSuccess) {
      free_plan(p);
      return fail(MOE_E_HIP, "setting up the prefetch stream failed");
    }
  }
  Workspace& w = p->ws;
  const int64_t dev_before_ws = p->dev_bytes;
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
  p->workspace_bytes = p->dev_bytes - dev_before_ws;
  if (hipMemset(w.route_cnt, 0, 64 * sizeof(unsigned)) != hipSuccess) {
    free_plan(p);
    return fail(MOE_E_HIP, "clearing arrival counters failed");
  }
  if (p->debug_ws > 0) poison_workspace(p, nullptr);
  if (hipDeviceSynchronize() != hipSuccess) {
    free_plan(p);
    return fail(MOE_E_HIP, "device synchronize after allocation failed");
  }
  p->pool_node = page_node(p->layers[0].host_pool);
  {  // the static workspace of moe_layer_forward_noalloc on this device
    std::string why;
    if (!scratch_on(p->device, &why)) {
      free_plan(p);
      return fail(MOE_E_HIP, why);
    }
  }
  if (layers)
    for (int l = 0; l < cfg->num_layers; ++l)
      TRY(load_layer_impl(p, l, &layers[l], initial_hbm ? initial_hbm + (size_t)l * E : nullptr,
                          static_cast<hipStream_t>(stream)));
#undef TRY
  *out = p;
  return MOE_OK;
}

moe_status moe_plan_load_layer(moe_plan* p, int32_t layer, const moe_layer_weights* w, const int32_t* initial_hbm,
                               moe_stream stream) {
  if (!p || !w) return fail(MOE_E_INVALID, "null argument");
  if (layer < 0 || layer >= p->cfg.num_layers) return fail(MOE_E_INVALID, "layer out of range");
  moe_status st = check_layer_args(p->cfg, w, initial_hbm);
  if (st != MOE_OK) return st;
  return load_layer_impl(p, layer, w, initial_hbm, static_cast<hipStream_t>(stream));
}

moe_status moe_plan_get_info(moe_plan* p, moe_plan_info* out) {
  if (!p || !out) return fail(MOE_E_INVALID, "null argument");
  std::memset(out, 0, sizeof(*out));
  out->device = p->device;
  out->gpu_numa_node = p->gpu_node;
  out->host_pool_node = p->pool_node;
  out->numa_bound = p->numa_bound;
  out->internal_expert_bytes = p->L.bytes;
  out->host_pool_bytes = p->host_pool_bytes;
  out->hbm_slot_bytes = p->hbm_slot_bytes;
  out->workspace_bytes = p->workspace_bytes;
  return MOE_OK;
}
}  // extern "C"

namespace {

// The host part of a forward on a host-compute layer: wait for the routing results,
// compute the experts the GPU skipped (the host-read ones, or all) from their host
// copies, and copy their o rows into the workspace at their sorted positions (each
// expert's rows are contiguous there), on `s` after the GEMVs, before the combine.
moe_status host_part(moe_plan* p, Layer& ly, int T, Workspace& w, hipStream_t s) {
  const moe_config& c = p->cfg;
  const int E = c.num_experts, H = c.hidden, k = c.top_k;
  HIP_TRY(hipEventSynchronize(p->ev_route));
  const int32_t* hr = p->hs_route;
  const int n_act = hr[0], n_host = hr[1];
  const int32_t* active = hr + 2;
  const int32_t* offsets = hr + 2 + E;
  const int32_t* sorted = hr + 3 + 2 * E;
  const int n = ly.host_mode == MOE_HOST_COMPUTE_LAYER ? n_act : n_host;
  if (n <= 0) return MOE_OK;
  // the previous host part's copies out of hs_o (maybe on another stream) are done
  if (p->host_o_pending) {
    HIP_TRY(hipEventSynchronize(p->ev_host_o));
    p->host_o_pending = false;
  }
  std::vector<const uint8_t*> blobs(n);
  std::vector<int> M(n), xoff(n);
  int rows = 0;
  const bool bf16 = c.act_dtype == MOE_ACT_BF16;
  for (int i = 0; i < n; ++i) {
    const int e = active[i];
    blobs[i] = ly.host_pool + (size_t)e * p->L.bytes;
    M[i] = offsets[e + 1] - offsets[e];
    xoff[i] = rows;
    for (int r = 0; r < M[i]; ++r) {  // token rows of the expert, in sorted order, as fp32
      const int t = sorted[offsets[e] + r] / k;
      float* dst = p->hx.data() + (size_t)(rows + r) * H;
      if (bf16) {
        const uint16_t* src = static_cast<const uint16_t*>(p->hs_x) + (size_t)t * H;
        for (int j = 0; j < H; ++j) {
          const uint32_t u = (uint32_t)src[j] << 16;
          std::memcpy(dst + j, &u, 4);
        }
      } else {
        std::memcpy(dst, static_cast<const float*>(p->hs_x) + (size_t)t * H, sizeof(float) * H);
      }
    }
    rows += M[i];
  }
  host_experts_ffn(p->L, n, blobs.data(), M.data(), xoff.data(), p->hx.data(), p->hh.data(), p->hs_o, bf16,
                   *p->host_pool);
  for (int i = 0; i < n; ++i)
    HIP_TRY(hipMemcpyAsync(w.o + (size_t)offsets[active[i]] * H, p->hs_o + (size_t)xoff[i] * H,
                           sizeof(float) * M[i] * H, hipMemcpyHostToDevice, s));
  HIP_TRY(hipEventRecord(p->ev_host_o, s));
  p->host_o_pending = true;
  ly.host_computed += n;
  (void)T;
  return MOE_OK;
}

// The forward of moe_layer_forward on the workspace `w` (the plan's, or one carved
// from the static scratch array for moe_layer_forward_noalloc).
moe_status forward_impl(moe_plan* p, int32_t layer, int32_t T, const void* x, const float* logits_in, float* y,
                        void* x_out, const moe_routing* ro, hipStream_t s, Workspace& w, bool own_ws) {
  Layer& ly = p->layers[layer];
  const moe_config& c = p->cfg;
  const int E = c.num_experts, H = c.hidden, I = c.inter, k = c.top_k, G = c.group_size;
  const int bf16 = c.act_dtype == MOE_ACT_BF16;
  const int A = T * k;
  if (own_ws && p->debug_ws >= 2) poison_workspace(p, s);
  WsTrack trk;
#define LAUNCH_USES(kernel, reads, writes) \
  if (!trk.launch(kernel, reads, writes)) return fail(MOE_E_STATE, "internal dispatch error: " + trk.err)

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
  ra.rw = router_split(H, bf16, E);
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
  rt.skip_host = ly.host_mode;

  // one-launch routing for small batches (its router walks the tokens one by one;
  // past a few bf16 tokens the MFMA router and the multi-block grouping are faster)
  const bool decode = T <= (bf16 ? kRouteDecodeMaxTokensBf16 : kRouteSmallMaxTokens) && A <= kRouteSmallMaxAssign;
  // the grouped MFMA GEMMs and the fused down + combine kernels take 4-bit codes only;
  // 2- and 3-bit layers run every batch on the dequant-GEMVs
  const bool int4 = p->L.bits == 4;
  // layers whose experts the host cores compute (some or all) run on the GEMVs with the
  // down projection and the combine apart, so the combine can merge the host's rows
  const int hmode = ly.host_mode;
  const bool prefill =
      bf16 && int4 && hmode == MOE_HOST_COMPUTE_NONE && c.gemm_min_tokens > 0 && T >= c.gemm_min_tokens && !decode;
  rt.work = prefill ? nullptr : w.work;
  // the MFMA router takes one workgroup per 32 x 32 logits tile: with few tiles (a
  // few tokens) the row-split router's many workgroups are faster (7168-wide,
  // 384-expert layer, 16 tokens: 12 MFMA workgroups took 29.7 us)
  const bool mfma_router = (int64_t)((T + 31) / 32) * ((E + 31) / 32) >= kMfmaRouterMinTiles;
  // a few tokens: down projection and combine in one launch (K split over the free
  // waves), when its (H/64) x T workgroups still keep the CUs streaming; below that
  // the per-expert down GEMV spreads the same bytes over more workgroups
  const int down_splits = std::max(1, std::min(16 / k, (int)p->L.dn_groups));
  const bool fuse_small = bf16 && int4 && hmode == MOE_HOST_COMPUTE_NONE && decode && T <= kDownCombMaxTokens && k <= 16;
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
      rp.xsum = nullptr;
      if (!logits_in) {
        LAUNCH_USES(mfma_router ? "k_router_mfma" : "k_router", 0, WB_LOGITS);
        KernelTimer kt(p, MOE_K_ROUTER);
        if (mfma_router) {
          rp.router_blocks = 1;
          launch_router_mfma(rp, kt.tm, s);
        } else {
          rp.router_blocks = router_blocks_for(H, bf16, E);
          launch_router(rp, bf16, kt.tm, s);
        }
      }
    }
    rt.tiles = w.tiles;
    rt.n_tiles = w.n_tiles;
    {
      LAUNCH_USES("k_topk_count + k_scatter", logits_in ? 0 : WB_LOGITS,
                  WB_IDS | WB_WTS | WB_COUNTS | WB_OFFSETS | WB_SORTED | WB_INV | WB_ACTIVE | WB_NACTIVE | WB_HIST |
                      WB_ACTPOS | WB_TILES | WB_NTILES);
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
      LAUNCH_USES("k_stage", WB_COUNTS | WB_ACTPOS | WB_ACTIVE | WB_NACTIVE, WB_STAGE | WB_GPTR);
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
    const uint32_t staged = gemm_wptr == w.gptr ? WB_GPTR | WB_STAGE : 0;
    {
      LAUNCH_USES("k_gemm gate/up", staged | WB_TILES | WB_NTILES | WB_OFFSETS | WB_SORTED, WB_H);
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
      LAUNCH_USES("k_gemm down", staged | WB_TILES | WB_NTILES | WB_OFFSETS | WB_H, WB_O);
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
    ca.xres = x_out ? x : nullptr;
    ca.xout = x_out;
    ca.act_bf16 = bf16;
    {
      LAUNCH_USES("k_combine", WB_O | WB_WTS | WB_INV, 0);
      KernelTimer kt(p, MOE_K_COMBINE);
      launch_combine(ca, kt.tm, s);
    }
    HIP_TRY(hipGetLastError());
  } else if (decode) {
    // router + group sums + top-k + grouping in one launch
    ra.router_blocks = logits_in ? 0 : router_blocks_for(H, bf16, E);
    LAUNCH_USES("k_route_decode", 0,
                (logits_in ? 0 : WB_LOGITS) | (bf16 ? WB_XSUM : 0) | WB_IDS | WB_WTS | WB_COUNTS | WB_OFFSETS |
                    WB_SORTED | WB_INV | WB_ACTIVE | WB_NACTIVE | WB_WORK | (rt.aptr ? WB_APTR : 0));
    KernelTimer kt(p, MOE_K_ROUTE);
    launch_route_decode(rt, ra, bf16, w.route_cnt, kt.tm, s);
  } else {
    {
      LAUNCH_USES(bf16 && mfma_router ? "k_router_mfma" : "k_router", 0,
                  (logits_in ? 0 : WB_LOGITS) | (bf16 ? WB_XSUM : 0));
      KernelTimer kt(p, MOE_K_ROUTER);
      if (bf16 && mfma_router) {  // MFMA logits tiles (unless given) and the group sums, one launch
        ra.router_blocks = logits_in ? 0 : 1;
        launch_router_mfma(ra, kt.tm, s);
      } else {
        ra.router_blocks = logits_in ? 0 : router_blocks_for(H, bf16, E);
        launch_router(ra, bf16, kt.tm, s);
      }
    }
    LAUNCH_USES("k_topk_count + k_scatter", logits_in ? 0 : WB_LOGITS,
                WB_IDS | WB_WTS | WB_COUNTS | WB_OFFSETS | WB_SORTED | WB_INV | WB_ACTIVE | WB_NACTIVE | WB_HIST |
                    WB_ACTPOS | WB_WORK);
    KernelTimer kt(p, MOE_K_ROUTE);
    launch_topk_group(rt, w.route_cnt + 16, kt.tm, s);
  }

  if (hmode != MOE_HOST_COMPUTE_NONE) {
    // the routing results and x for the host part, written by one small kernel into
    // mapped, coherent pinned memory right after the routing (the GEMVs follow it);
    // the host part waits for the event, and the call returns only after it has read
    // the staging, so the next forward cannot overwrite it while it is read
    LAUNCH_USES("k_export_route", WB_NACTIVE | WB_ACTIVE | WB_OFFSETS | WB_SORTED, 0);
    launch_export_route(w.n_active, w.active, w.offsets, w.sorted, x, p->act_size * T * H, p->hs_route_dev,
                        p->hs_x_dev, E, A, s);
    HIP_TRY(hipEventRecord(p->ev_route, s));
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
    ga.off_hi = p->L.off_gu_hi;
    ga.off_scales = p->L.off_gu_scales;
    ga.bits = (int)p->L.bits;
    ga.chunks = (int)p->L.gu_chunks;
    ga.groups = (int)p->L.gu_groups;
    ga.tiles = (int)p->L.gu_tiles;
    ga.H = H;
    ga.I = I;
    ga.G = G;
    ga.k = k;
    ga.T = T;
    {
      LAUNCH_USES("k_gateup", WB_WORK | WB_SORTED | (bf16 ? WB_XSUM : 0), WB_H | (bf16 ? WB_HPART : 0));
      KernelTimer kt(p, MOE_K_GATEUP);
      launch_gateup(ga, bf16, std::min(T, 8), max_act * ga.tiles, kt.tm, s);
    }

    GemvArgs da = ga;
    da.in = w.h;
    da.insum = w.hpart;
    da.out = w.o;
    da.outpart = nullptr;
    da.off_codes = p->L.off_dn_codes;
    da.off_hi = p->L.off_dn_hi;
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
      dc.xres = x_out ? static_cast<const uint16_t*>(x) : nullptr;
      dc.xout = static_cast<uint16_t*>(x_out);
      LAUNCH_USES(fuse_down ? "k_down_comb" : "k_down_comb16", WB_APTR | WB_INV | WB_WTS | WB_H | WB_HPART, 0);
      KernelTimer kt(p, MOE_K_DOWN);
      if (fuse_down)
        launch_down_combine(dc, kt.tm, s);
      else
        launch_down_combine16(dc, kt.tm, s);
    } else {
      {
        LAUNCH_USES("k_down", WB_WORK | WB_H | (bf16 ? WB_HPART : 0), WB_O);
        KernelTimer kt(p, MOE_K_DOWN);
        launch_down(da, bf16, std::min(T, 8), max_act * da.tiles, kt.tm, s);
      }
      if (hmode != MOE_HOST_COMPUTE_NONE) {
        moe_status st = host_part(p, ly, T, w, s);
        if (st != MOE_OK) return st;
      }
      CombineArgs ca{};
      ca.o = w.o;
      ca.wts = w.wts;
      ca.inv = w.inv;
      ca.y = y;
      ca.T = T;
      ca.H = H;
      ca.k = k;
    ca.xres = x_out ? x : nullptr;
    ca.xout = x_out;
    ca.act_bf16 = bf16;
      LAUNCH_USES("k_combine", WB_O | WB_WTS | WB_INV, 0);
      KernelTimer kt(p, MOE_K_COMBINE);
      launch_combine(ca, kt.tm, s);
    }
    HIP_TRY(hipGetLastError());
  }
#undef LAUNCH_USES

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

moe_status cache_update_sync(moe_plan* p, int l0, int l1, double decay, int maxp, const int32_t* want,
                             hipStream_t s);

// Arguments shared by both forward entry points.
moe_status check_forward_args(moe_plan* p, int32_t layer, int32_t T, const void* x, const float* logits_in,
                              const float* y) {
  if (!p) return fail(MOE_E_INVALID, "plan is null");
  if (layer < 0 || layer >= p->cfg.num_layers) return fail(MOE_E_INVALID, "layer out of range");
  if (T < 0 || T > p->cfg.max_tokens) return fail(MOE_E_INVALID, "T out of range 0..max_tokens");
  if (T == 0) return MOE_OK;
  if (!x || !y) return fail(MOE_E_INVALID, "x and y are required");
  if (!aligned16(x) || !aligned16(y) || (logits_in && !aligned16(logits_in)))
    return fail(MOE_E_INVALID, "x, y and logits_in must be 16-byte aligned");
  if (!p->layers[layer].loaded) return fail(MOE_E_INVALID, "layer not loaded");
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_layer_forward(moe_plan* p, int32_t layer, int32_t T, const void* x, const float* logits_in, float* y,
                             const moe_routing* ro, moe_stream stream) {
  moe_status st = check_forward_args(p, layer, T, x, logits_in, y);
  if (st != MOE_OK || T == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = wait_prefetch(p, p->layers[layer], s);
  if (st == MOE_OK) st = forward_impl(p, layer, T, x, logits_in, y, nullptr, ro, s, p->ws, true);
  return st;
}

moe_status moe_layer_forward_residual(moe_plan* p, int32_t layer, int32_t T, const void* x, const float* logits_in,
                                      float* y, void* x_out, const moe_routing* ro, moe_stream stream) {
  moe_status st = check_forward_args(p, layer, T, x, logits_in, y);
  if (st != MOE_OK || T == 0) return st;
  if (!x_out || !aligned16(x_out)) return fail(MOE_E_INVALID, "x_out is required and must be 16-byte aligned");
  const size_t xb = (size_t)T * p->cfg.hidden * p->act_size;
  const char *xa = static_cast<const char*>(x), *oa = static_cast<const char*>(x_out);
  if (oa < xa + xb && xa < oa + xb) return fail(MOE_E_INVALID, "x_out overlaps x");
  const char* ya = reinterpret_cast<const char*>(y);
  const size_t yb = (size_t)T * p->cfg.hidden * sizeof(float);
  if (oa < ya + yb && ya < oa + xb) return fail(MOE_E_INVALID, "x_out overlaps y");
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = wait_prefetch(p, p->layers[layer], s);
  if (st == MOE_OK) st = forward_impl(p, layer, T, x, logits_in, y, x_out, ro, s, p->ws, true);
  return st;
}

moe_status moe_layer_forward_noalloc(moe_plan* p, int32_t layer, int32_t T, const void* x, const float* logits_in,
                                     float* y, const moe_routing* ro, moe_stream stream) {
  moe_status st = check_forward_args(p, layer, T, x, logits_in, y);
  if (st != MOE_OK || T == 0) return st;
  Workspace w{};
  const size_t need = carve_workspace(p, T, nullptr, &w);
  if (need > kScratchBytes)
    return fail(MOE_E_INVALID, "the workspace of this forward needs " + std::to_string(need) +
                                   " bytes, more than the static workspace's " + std::to_string(kScratchBytes));
  std::string why;
  uint8_t* base = scratch_on(p->device, &why);  // set up by moe_plan_create on this device
  if (!base) return fail(MOE_E_HIP, why);
  carve_workspace(p, T, base, &w);
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = wait_prefetch(p, p->layers[layer], s);
  if (st == MOE_OK) st = forward_impl(p, layer, T, x, logits_in, y, nullptr, ro, s, w, false);
  return st;
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
  const int32_t* want = pol ? pol->want_resident : nullptr;
  if (want)
    for (int l = l0; l < l1; ++l) {
      int n = 0;
      for (int e = 0; e < E; ++e) n += want[(size_t)(l - l0) * E + e] != 0;
      if (n > p->cfg.hbm_slots) return fail(MOE_E_INVALID, "want_resident names more experts than hbm_slots");
    }
  hipStream_t s = static_cast<hipStream_t>(stream);
  HIP_TRY(hipSetDevice(p->device));
  return pol && pol->overlap && !want ? cache_update_pipelined(p, l0, l1, decay, maxp, s)
                                      : cache_update_sync(p, l0, l1, decay, maxp, want, s);
}

moe_status moe_prefetch(moe_plan* p, int32_t layer, int32_t T, const void* x, const float* logits_in,
                        int32_t candidates, int32_t* predicted_out, moe_stream stream) {
  if (!p) return fail(MOE_E_INVALID, "plan is null");
  if (layer < 0 || layer >= p->cfg.num_layers) return fail(MOE_E_INVALID, "layer out of range");
  if (p->cfg.prefetch_slots == 0) return fail(MOE_E_STATE, "plan has no prefetch slots");
  const int E = p->cfg.num_experts;
  if (T < 1 || T > p->cfg.max_tokens) return fail(MOE_E_INVALID, "T out of range 1..max_tokens");
  const int kp = candidates == 0 ? p->cfg.top_k : candidates;
  if (kp < 1 || kp > 64 || kp > E) return fail(MOE_E_INVALID, "candidates must be in 0..min(64, num_experts)");
  if ((int64_t)T * kp > kPrefetchMaxCand) return fail(MOE_E_INVALID, "T * candidates must be <= 2048");
  if (!logits_in && !x) return fail(MOE_E_INVALID, "x or logits_in is required");
  if ((x && !logits_in && !aligned16(x)) || (logits_in && !aligned16(logits_in)))
    return fail(MOE_E_INVALID, "x and logits_in must be 16-byte aligned");
  Layer& ly = p->layers[layer];
  if (!ly.loaded) return fail(MOE_E_INVALID, "layer not loaded");
  hipStream_t s = static_cast<hipStream_t>(stream);
  HIP_TRY(hipSetDevice(p->device));
  HIP_TRY(hipEventRecord(p->ev_caller, s));
  HIP_TRY(hipStreamWaitEvent(p->pf_stream, p->ev_caller, 0));
  RouterArgs r{};
  r.x = x;
  r.w = ly.d_router_w;
  r.b = ly.d_router_b;
  r.logits = p->pf_logits;
  r.T = T;
  r.H = p->cfg.hidden;
  r.E = E;
  r.G = p->cfg.group_size;
  r.router_blocks = logits_in ? 0 : router_blocks_for(p->cfg.hidden, p->cfg.act_dtype == MOE_ACT_BF16, E);
  r.rw = router_split(p->cfg.hidden, p->cfg.act_dtype == MOE_ACT_BF16, E);
  PrefetchArgs a{};
  a.wptr = ly.d_wptr;
  a.is_host = ly.d_is_host;
  a.host_pool = ly.host_pool_dev;
  a.slots = ly.pf_slots;
  a.occ = ly.d_pf_occ;
  a.list = ly.d_pf_list;
  a.predicted_out = predicted_out;
  a.stats = ly.d_stats;
  a.logits = logits_in ? logits_in : p->pf_logits;
  a.bytes = p->L.bytes;
  a.E = E;
  a.P = p->cfg.prefetch_slots;
  a.kp = kp;
  a.T = T;
  launch_prefetch(a, r, p->cfg.act_dtype == MOE_ACT_BF16, p->pf_counter, p->pf_stream);
  HIP_TRY(hipGetLastError());
  HIP_TRY(hipEventRecord(ly.ev_prefetch, p->pf_stream));
  ly.pf_pending = true;
  return MOE_OK;
}

moe_status moe_plan_prefetch_slots(moe_plan* p, int32_t layer, int32_t* slot_expert) {
  if (!p || !slot_expert) return fail(MOE_E_INVALID, "null argument");
  if (layer < 0 || layer >= p->cfg.num_layers) return fail(MOE_E_INVALID, "layer out of range");
  if (p->cfg.prefetch_slots == 0) return fail(MOE_E_STATE, "plan has no prefetch slots");
  HIP_TRY(hipSetDevice(p->device));
  HIP_TRY(hipStreamSynchronize(p->pf_stream));
  HIP_TRY(hipMemcpy(slot_expert, p->layers[layer].d_pf_occ, sizeof(int32_t) * p->cfg.prefetch_slots,
                    hipMemcpyDeviceToHost));
  return MOE_OK;
}

}  // extern "C"

namespace {

// Synchronous cache update of layers [l0, l1) (see moe_cache_update).
moe_status cache_update_sync(moe_plan* p, int l0, int l1, double decay, int maxp, const int32_t* want,
                             hipStream_t s) {
  const int E = p->cfg.num_experts;
  for (int l = l0; l < l1; ++l) {
    moe_status st = wait_prefetch(p, p->layers[l], s);
    if (st != MOE_OK) return st;
  }
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
    if (want)
      cache_set_resident(E, p->cfg.hbm_slots, decay, ly.h_counts_stage, want + (size_t)(l - l0) * E, ly.score.data(),
                         ly.slot_of.data(), &promoted, &evicted);
    else
      cache_policy_step(E, p->cfg.hbm_slots, decay, maxp, ly.h_counts_stage, ly.score.data(), ly.slot_of.data(),
                        &promoted, &evicted);
    if (promoted.empty() && !evicted.empty()) {  // evictions only: the table still changes
      ly.evictions += (int64_t)evicted.size();
      moe_status st = push_tables(p, ly, s);
      if (st != MOE_OK) return st;
      continue;
    }
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

}  // namespace

extern "C" {

moe_status moe_plan_set_host_compute(moe_plan* p, int32_t layer, int32_t mode, int32_t threads) {
  if (!p) return fail(MOE_E_INVALID, "plan is null");
  if (layer < -1 || layer >= p->cfg.num_layers) return fail(MOE_E_INVALID, "layer out of range");
  if (mode < MOE_HOST_COMPUTE_NONE || mode > MOE_HOST_COMPUTE_LAYER) return fail(MOE_E_INVALID, "bad mode");
  const int l0 = layer < 0 ? 0 : layer, l1 = layer < 0 ? p->cfg.num_layers : layer + 1;
  if (mode != MOE_HOST_COMPUTE_NONE) {
    if (p->L.bits != 4) return fail(MOE_E_UNSUPPORTED, "host computation takes 4-bit codes only");
    if (!host_ffn_supported()) return fail(MOE_E_UNSUPPORTED, "host computation needs AVX-512 (F, BW, VL) and F16C");
    if (!p->host_pool) {  // pinned staging and the worker pool, once per plan
      const moe_config& c = p->cfg;
      const size_t Tm = (size_t)c.max_tokens, A = Tm * c.top_k, E = c.num_experts;
      void* v = nullptr;
      const unsigned mapped = hipHostMallocMapped | hipHostMallocCoherent;
      moe_status st = host_alloc(p, &v, sizeof(int32_t) * (3 + 2 * E + A), mapped);
      if (st != MOE_OK) return st;
      p->hs_route = static_cast<int32_t*>(v);
      st = host_alloc(p, &p->hs_x, p->act_size * Tm * c.hidden, mapped);
      if (st != MOE_OK) return st;
      void *d1 = nullptr, *d2 = nullptr;
      if (hipHostGetDevicePointer(&d1, p->hs_route, 0) != hipSuccess ||
          hipHostGetDevicePointer(&d2, p->hs_x, 0) != hipSuccess) {
        (void)hipGetLastError();
        return fail(MOE_E_HIP, "hipHostGetDevicePointer of the host-part staging failed");
      }
      p->hs_route_dev = static_cast<int32_t*>(d1);
      p->hs_x_dev = d2;
      st = host_alloc(p, &v, sizeof(float) * A * c.hidden, 0);
      if (st != MOE_OK) return st;
      p->hs_o = static_cast<float*>(v);
      if ((!p->ev_route && hipEventCreateWithFlags(&p->ev_route, hipEventDisableTiming) != hipSuccess) ||
          (!p->ev_host_o && hipEventCreateWithFlags(&p->ev_host_o, hipEventDisableTiming) != hipSuccess)) {
        (void)hipGetLastError();
        return fail(MOE_E_HIP, "creating the host-part events failed");
      }
      try {
        p->hx.assign(A * c.hidden, 0.f);
        p->hh.assign(A * c.inter, 0.f);
      } catch (const std::bad_alloc&) {
        return fail(MOE_E_HOST_NOMEM, "host scratch for the host computation");
      }
      int n = threads;
      if (n <= 0) {
        cpu_set_t set;
        n = sched_getaffinity(0, sizeof(set), &set) == 0 ? CPU_COUNT(&set) : (int)std::thread::hardware_concurrency();
      }
      p->host_pool = new HostPool(std::max(1, n));
    }
  }
  for (int l = l0; l < l1; ++l) p->layers[l].host_mode = mode;
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
    out->host_computed += ly.host_computed;
    out->prefetched += st[ST_PREFETCHED];
  }
  return MOE_OK;
}

moe_status moe_plan_reset_stats(moe_plan* p) {
  if (!p) return fail(MOE_E_INVALID, "plan is null");
  HIP_TRY(hipSetDevice(p->device));
  HIP_TRY(hipDeviceSynchronize());
  for (Layer& ly : p->layers) {
    HIP_TRY(hipMemset(ly.d_stats, 0, sizeof(int64_t) * ST_COUNT));
    ly.bytes_copied = ly.promotions = ly.evictions = ly.host_computed = 0;
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

moe_status moe_measure_link_ceilings(size_t hbm_bytes, size_t host_bytes, int32_t iters, moe_stream stream,
                                     moe_link_ceilings* out) {
  if (!out) return fail(MOE_E_INVALID, "out is null");
  std::memset(out, 0, sizeof(*out));
  if (hbm_bytes < (1u << 20) || host_bytes < (1u << 20) || hbm_bytes % 4096 || host_bytes % 4096 || iters < 1)
    return fail(MOE_E_INVALID, "sizes must be >= 1 MiB and multiples of 4 KiB, iters >= 1");
  hipStream_t s = static_cast<hipStream_t>(stream);
  // a plan-less holder for the buffers, freed on every exit
  moe_plan tmp;
  if (hipGetDevice(&tmp.device) != hipSuccess) return fail(MOE_E_HIP, "hipGetDevice failed");
  tmp.gpu_node = gpu_numa_node(tmp.device);
  struct Release {
    moe_plan* p;
    ~Release() {
      (void)hipDeviceSynchronize();
      for (void* q : p->dev_allocs) (void)hipFree(q);
      for (void* q : p->host_allocs) (void)hipHostFree(q);
      g_live[0] -= (int64_t)p->dev_allocs.size();
      g_live[1] -= (int64_t)p->host_allocs.size();
    }
  } release{&tmp};
  void *dbuf = nullptr, *hbuf = nullptr, *hdst = nullptr, *sink = nullptr, *hdev = nullptr;
  moe_status st = dev_alloc(&tmp, &dbuf, hbm_bytes);
  if (st == MOE_OK) st = dev_alloc(&tmp, &hdst, host_bytes);
  if (st == MOE_OK) st = dev_alloc(&tmp, &sink, sizeof(uint32_t) * stream_read_blocks());
  if (st == MOE_OK) st = host_alloc_numa(&tmp, &hbuf, host_bytes, hipHostMallocMapped | hipHostMallocNonCoherent);
  if (st != MOE_OK) return st;
  HIP_TRY(hipHostGetDevicePointer(&hdev, hbuf, 0));
  std::memset(hbuf, 0, host_bytes);
  HIP_TRY(hipMemsetAsync(dbuf, 0, hbm_bytes, s));
  hipEvent_t e0 = nullptr, e1 = nullptr;
  HIP_TRY(hipEventCreate(&e0));
  HIP_TRY(hipEventCreate(&e1));
  auto best_gbps = [&](auto&& run, size_t bytes, double* outv) -> moe_status {
    double best = 0.0;
    for (int i = 0; i <= iters; ++i) {  // run 0 is untimed
      HIP_TRY(hipEventRecord(e0, s));
      run();
      HIP_TRY(hipEventRecord(e1, s));
      HIP_TRY(hipEventSynchronize(e1));
      float ms = 0.f;
      HIP_TRY(hipEventElapsedTime(&ms, e0, e1));
      if (i > 0 && ms > 0.f) best = std::max(best, (double)bytes / (ms * 1e-3) / 1e9);
    }
    *outv = best;
    return MOE_OK;
  };
  uint32_t* sk = static_cast<uint32_t*>(sink);
  st = best_gbps([&] { launch_stream_read(dbuf, hbm_bytes, sk, s); }, hbm_bytes, &out->hbm_read_gbps);
  if (st == MOE_OK)
    st = best_gbps([&] { launch_stream_read(hdev, host_bytes, sk, s); }, host_bytes, &out->host_read_gbps);
  if (st == MOE_OK)
    st = best_gbps([&] { (void)hipMemcpyAsync(hdst, hbuf, host_bytes, hipMemcpyHostToDevice, s); }, host_bytes,
                   &out->h2d_copy_gbps);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (st != MOE_OK) return st;
  HIP_TRY(hipGetLastError());
  return MOE_OK;
}

moe_status moe_debug_fail_alloc(int32_t kind, int32_t n) {
  if (kind < 0 || kind > 1 || n < 0) return fail(MOE_E_INVALID, "kind must be 0 or 1 and n >= 0");
  g_fail_alloc[kind].store(n);
  return MOE_OK;
}

moe_status moe_debug_live_allocs(int64_t* device, int64_t* host) {
  if (!device || !host) return fail(MOE_E_INVALID, "null argument");
  *device = g_live[0].load();
  *host = g_live[1].load();
  return MOE_OK;
}

void moe_plan_destroy(moe_plan* p) { free_plan(p); }

}  // extern "C"
