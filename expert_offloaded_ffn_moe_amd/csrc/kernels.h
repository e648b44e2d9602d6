// Internal kernel interface of the MoE offload library (gfx950 only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

namespace moe {

// Device counters per layer, int64 each.
enum StatIndex { ST_FORWARDS = 0, ST_TOKENS, ST_HITS, ST_MISSES, ST_BYTES_HBM, ST_BYTES_HOST, ST_PREFETCHED, ST_COUNT };

// Optional events stamped by the dispatch itself at kernel start and end.
struct Timing {
  hipEvent_t start = nullptr, stop = nullptr;
};

template <typename F, typename... Args>
inline void launch_timed(F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t s, const Timing& tm,
                         Args... args) {
  if (tm.start || tm.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, tm.start, tm.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
}

struct RouterArgs {
  const void* x;         // [T][H] act dtype
  const void* w;         // [E][H] act dtype
  const float* b;        // [E] or null
  float* logits;         // [T][E]
  float* xsum;           // [T][H/G] sums of x over each group (bf16 path), or null
  int T, H, E, G;
  int router_blocks;     // blocks computing logits (the rest compute xsum); MFMA router: > 0 = logits wanted
  int rw;                // waves per router row (router_split)
};

// Router rows: kRouterWaves waves per workgroup, rw of them per row. rw (1, 2, 4
// or 8) is the smallest that keeps a wave's part of a row within 8 x 64 chunks of
// 16 bytes (the routing launch of a 7168-wide layer, together with the fence-free
// arrival of route_dev.h: batch 1 13.3 -> 12.2 us, batch 4 18.8 -> 14.7 us against
// one wave per row; splitting further, to fill more workgroups, gained less).
constexpr int kRouterWaves = 8;
constexpr int kMfmaRouterMinTiles = 64;  // logits tiles (32 x 32) from which the MFMA router is used
inline int router_split(int H, int act_bf16, int E) {
  const int nchunk = H * (act_bf16 ? 2 : 4) / 16;
  int rw = 1;
  while (rw < 8 && (nchunk + rw - 1) / rw > 8 * 64) rw *= 2;
  return rw;
}
inline int router_blocks_for(int H, int act_bf16, int E) {
  return (E * router_split(H, act_bf16, E) + kRouterWaves - 1) / kRouterWaves;
}

// One GEMV work item: an active expert of the current forward, written by the
// grouping step so that the weight kernels reach both the expert's weights and
// its first tokens' activations after a single dependent load.
constexpr int kDescTok = 8;
struct alignas(64) WorkDesc {
  const uint8_t* w;        // internal blob (HBM slot or host-mapped copy)
  int32_t p0, M;           // first sorted position of the expert's rows, number of rows
  int32_t tok[kDescTok];   // token of each of the first min(M, kDescTok) rows
};

struct RouteArgs {
  const float* logits;      // [T][E]
  int32_t* ids;             // [T*k]
  float* wts;               // [T*k]
  int32_t* counts;          // [E]
  int32_t* offsets;         // [E+1]
  int32_t* sorted;          // [T*k]
  int32_t* inv;             // [T*k]
  int32_t* active;          // [E] experts with counts > 0: host-read ones first, then ascending id
  int32_t* n_active;        // [2]: active experts, of which host-read (the first entries of `active`)
  const int32_t* is_host;   // [E] 1 = expert read from host memory
  int64_t* counts_acc;      // [E] per-layer assignment counts since the last cache update
  int64_t* stats;           // [ST_COUNT]
  int64_t expert_bytes;     // canonical bytes per expert (stats)
  int T, E, k;
  int2* tiles;              // prefill: (expert, first row) of each 64-row tile, or null
  int32_t* n_tiles;         // [1]
  const uint8_t* const* wptr;  // [E] expert blob table (for the work descriptors)
  WorkDesc* work;           // [E] one per active expert, in active-list order, or null
  const uint8_t** aptr;     // [T*k] blob of each assignment's expert (decode), or null
  int32_t* hist;            // [ceil(T/16)][E] per-block counts, then bases (multi-block grouping)
  int32_t* act_pos;         // [E] active-list position of each expert (multi-block grouping)
  int skip_host;            // GEMV descriptors with zero rows for: 0 none, 1 host-read experts, 2 all experts
};

struct GemvArgs {
  const WorkDesc* work;        // [min(E, T*k)] active experts (blob, rows, first tokens), then M = 0
  const int32_t* sorted;       // [T*k]
  const void* in;              // gate/up: x [T][H]; down: h [T*k][I] (rows by sorted position)
  const float* insum;          // gate/up: xsum [T][H/G]; down: hpart [T*k][I/32] (bf16 path)
  void* out;                   // gate/up: h [T*k][I] act dtype; down: o [T*k][H] fp32
  float* outpart;              // gate/up: hpart [T*k][I/32] (bf16 path); down: unused
  int64_t off_codes, off_hi, off_scales;  // code words, 3-bit high planes, scales (offsets in the blob)
  int chunks, groups;          // 16-byte lane words of K and quantisation groups per row
  int tiles;                   // tiles per expert
  int H, I, G, k, T;
  int bits;                    // bits per weight code: 4, 3 or 2
};

struct GemmArgs {
  const uint8_t* const* wptr;  // [E] internal expert blobs
  const int2* tiles;           // (expert, first row) per 64-row tile
  const int32_t* n_tiles;      // [1]
  const int32_t* offsets;      // [E+1]
  const int32_t* sorted;       // [T*k]
  const uint16_t* a_src;       // gate/up: x [T][H]; down: h [T*k][I] by sorted position
  void* out;                   // gate/up: h [T*k][I] bf16; down: o [T*k][H] fp32
  int64_t off_codes, off_scales;
  int chunks, groups;          // per weight row
  int ntiles_n;                // 64-row weight tiles (gate/up: I/32, down: H/64)
  int K, out_ld, k, G;
  int max_tiles;               // launch bound on the number of row tiles
};

// Down projection fused with the combine, one workgroup per (64-row tile of H,
// token): y[t] rows = sum over the token's slots j, in order, of w_j * (Wd_e h).
struct DownCombArgs {
  const uint8_t* const* aptr;  // [T*k] blob of each assignment's expert
  const int32_t* inv;          // [T*k] sorted position of each assignment (its h row)
  const float* wts;            // [T*k]
  const void* h;               // [T*k][I] bf16 by sorted position
  const float* hpart;          // [T*k][I/32]
  float* y;                    // [T][H]
  const uint16_t* xres;        // [T][H] bf16 x, with xout: xout = bf16(x + y), or null
  uint16_t* xout;
  int64_t off_codes, off_scales;
  int chunks, groups, G, H, I, k, T;
  int splits;                  // waves per slot (K split)
};

// Prefill staging of offloaded experts (see k_stage.hip).
struct StageArgs {
  const uint8_t* const* wptr;  // [E] layer blob table (HBM slot or host-mapped copy)
  const int32_t* is_host;      // [E]
  const int32_t* counts;       // [E] rows per expert of this forward
  const int32_t* act_pos;      // [E] active-list position (valid where counts > 0)
  const int32_t* active;       // [E] active experts, host-read ones first
  const int32_t* n_active;     // [1]
  uint8_t* stage;              // [n_slots][bytes] staging slots in HBM
  const uint8_t** gptr;        // [E] out: blob table for the GEMMs
  int64_t bytes;               // internal blob bytes (multiple of 16)
  int E, n_slots;
  int table_blocks, blocks_per_expert;  // set by launch_stage
};

// Predictive prefetch of one layer's experts into its prefetch slots (k_route.hip).
struct PrefetchArgs {
  const uint8_t** wptr;        // [E] the layer's blob table (read and written)
  int32_t* is_host;            // [E]
  const uint8_t* host_pool;    // device address of the layer's host copies (expert e at e * bytes)
  uint8_t* slots;              // [P][bytes] the layer's prefetch slots
  int32_t* occ;                // [P] expert each slot holds, -1 none
  int32_t* list;               // [P] slots to fill this time, then [P] their count
  int32_t* predicted_out;      // [P] or null: the predicted experts in order, -1 past their count
  int64_t* stats;              // [ST_COUNT] the layer's counters (ST_PREFETCHED)
  const float* logits;         // [T][E] logits the prediction takes (the router's, or given)
  int64_t bytes;               // internal blob bytes (multiple of 16)
  int E, P, kp, T;             // kp: candidates per token
  int blocks_per_expert;       // set by launch_prefetch
};

struct CombineArgs {
  const float* o;       // [T*k][H]
  const float* wts;     // [T*k]
  const int32_t* inv;   // [T*k]
  float* y;             // [T][H]
  const void* xres;     // [T][H] x in the act dtype, with xout: xout = act(x + y), or null
  void* xout;
  int T, H, k, act_bf16;
};

// The residual epilogue of the combines: act(x + y), the sum formed in fp32 and
// rounded to bf16 (nearest, ties to even) for bf16 activations.
__device__ __forceinline__ uint16_t residual_bf16(uint16_t x, float y) {
  const float r = __uint_as_float((uint32_t)x << 16) + y;
  uint32_t u = __float_as_uint(r);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x0040u);  // NaN stays NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

constexpr int kRouteSmallMaxAssign = 256;   // T*k handled by launch_route_decode
constexpr int kRouteSmallMaxTokens = 64;
constexpr int kRouteDecodeMaxTokensBf16 = 4;  // bf16 batches routed by the one-launch decode routing
constexpr int kDownCombMaxTokens = 4;     // decode batches whose down projection and combine fuse
constexpr int kDownCombMinGroups = 256;   // ... if (H/64) * T workgroups reach this (else 16-row tiles)

void launch_router(const RouterArgs& a, int act_bf16, const Timing& tm, hipStream_t s);
void launch_route_decode(const RouteArgs& a, const RouterArgs& r, int act_bf16, unsigned* counter,
                         const Timing& tm, hipStream_t s);
// top-k and grouping over ceil(T/16) blocks (any T*k), counter: a zeroed device word
void launch_topk_group(const RouteArgs& a, unsigned* counter, const Timing& tm, hipStream_t s);
constexpr int kGroupTokens = 16;  // tokens per block of the multi-block grouping
void launch_gateup(const GemvArgs& a, int act_bf16, int max_tok, int grid, const Timing& tm, hipStream_t s);
void launch_down(const GemvArgs& a, int act_bf16, int max_tok, int grid, const Timing& tm, hipStream_t s);
void launch_combine(const CombineArgs& a, const Timing& tm, hipStream_t s);
void launch_down_combine(const DownCombArgs& a, const Timing& tm, hipStream_t s);  // bf16, k * splits <= 16
// the same on 16-row tiles of H (grid H/16 x T), for batches with few 64-row tiles
void launch_down_combine16(const DownCombArgs& a, const Timing& tm, hipStream_t s);  // bf16, k * splits <= 16
size_t down_combine16_lds(int k, int I);  // dynamic LDS bytes of launch_down_combine16
constexpr size_t kDownComb16MaxLds = 48 * 1024;
constexpr int kDownComb16WavesPerCU = 24;  // resident waves per CU at its register count (20-32 by variant)
void launch_stage(StageArgs a, const Timing& tm, hipStream_t s);
// router (unless r.router_blocks == 0) + prediction, then the copies and the table entries
void launch_prefetch(PrefetchArgs a, const RouterArgs& r, int act_bf16, unsigned* counter, hipStream_t s);
constexpr int kPrefetchMaxCand = 2048;  // T * kp of one prediction
constexpr int kPrefetchMaxE = 1024;     // experts per layer
constexpr int kPrefetchMaxSlots = 64;   // prefetch slots per layer
void launch_router_mfma(const RouterArgs& a, const Timing& tm, hipStream_t s);
void launch_gemm_gateup(const GemmArgs& a, const Timing& tm, hipStream_t s);
void launch_gemm_down(const GemmArgs& a, const Timing& tm, hipStream_t s);
constexpr int kGemmRows = 64;  // token rows per prefill GEMM tile
// Default of moe_config.gemm_min_tokens. From batches of about 6 tokens on, the
// experts that several tokens share make the GEMVs' per-token dot products cost
// more than the grouped MFMA GEMM's padded 64-row tiles (measured on H2048/E128
// and H7168/E384 layers: equal at 5-6 tokens, the GEMM 13% ahead at 8, 2x at 32).
constexpr int kGemmMinTokensDefault = 6;

// k_util.hip
void launch_fill32(void* p, uint32_t v, size_t n_words, hipStream_t s);
int stream_read_blocks();  // workgroups of launch_stream_read (one sink word each)
void launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s);  // bytes % 16 == 0
// routing results and x (x_bytes % 4 == 0) into host staging reached through its device address
void launch_export_route(const int32_t* n_active, const int32_t* active, const int32_t* offsets,
                         const int32_t* sorted, const void* x, size_t x_bytes, int32_t* dst, void* xdst, int E, int A,
                         hipStream_t s);


}  // namespace moe
