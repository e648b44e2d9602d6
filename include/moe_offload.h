/*
 * moe_offload.h — forward pass of a routed Mixture-of-Experts FFN layer on one
 * AMD MI355X (gfx950), under a per-expert residency plan.
 *
 * What is computed (per layer, per token t of x[T][H]):
 *   logits[t][e] = sum_h x[t][h] * Wr[e][h] + b[e]                  (fp32 accumulation)
 *   ids[t][0..k)  = the k largest logits, ties to the lower expert id,
 *                   slot order (logit descending, id ascending)
 *   w[t][j]       = softmax of the k selected logits (renormalised to sum 1)
 *   y[t]          = sum_j w[t][j] * Wd_e . rho( silu(Wg_e x[t]) * (Wu_e x[t]) ),  e = ids[t][j]
 * with W = q * s (int4 code times fp16 group scale) and rho rounding the
 * intermediate to the activation dtype; y is fp32.
 *
 * The pages describe the problem; the numerics above are the plain reading of
 * them. Page titles are abbreviated below as
 *   [763B]  "763B MoE 塞进两张 96GB 显卡：闲置专家丢进主机内存"
 *   [125B]  "125B 稀疏模型塞进一张 32GB 消费卡"
 *   [24K]   "我在 32GB 单卡上跑两万四千专家的 MoE:分层放置实测与三个坑"
 * and each call below names the section that defines what it does.
 *
 * Residency. Every expert of every layer has a copy in pinned, device-mapped
 * host memory (hipHostMalloc, on the host NUMA node closest to the GPU when the
 * system reports one). A layer has `hbm_slots` HBM slots; an expert in a slot
 * is read from HBM, every other expert is read by the kernels directly from its
 * host copy over the host link. moe_cache_update moves experts between the two.
 *
 * Canonical expert blob (the weight format of this ABI), per expert, for b =
 * weight_bits bits per code:
 *   q_gate[I][H*b/8] | q_up[I][H*b/8] | q_down[H][I*b/8] | s_gate[I][H/G] | s_up[I][H/G] | s_down[H][I/G]
 * K is contiguous. Code i of a row is the unsigned n at bits [b*i, b*i+b) of the
 * row's little-endian bit string (bit j = bit j % 8 of byte j / 8); for b = 4
 * that is byte j = (q[2j] & 0xF) | (q[2j+1] & 0xF) << 4. The weight code q:
 *   b = 4: two's complement, q = n - 16 * (n >= 8), -8..7;
 *   b = 3, 2: odd symmetric levels, q = 2n - (2^b - 1): -7, -5, ..., 7 / -3, -1, 1, 3.
 * Scales are IEEE fp16; s[n][g] covers k in [g*G, (g+1)*G); the weight is q * s.
 * The library repacks blobs into its own layout.
 *
 * Conventions for every call:
 *  - Return a moe_status; nothing is thrown across the ABI. moe_last_error()
 *    gives a message for the last failure on the calling thread.
 *  - Arguments are validated before any work is enqueued.
 *  - "device" pointers are GPU-visible memory (hipMalloc, or torch CUDA tensors),
 *    "host" pointers are ordinary CPU memory.
 *  - `stream` is a hipStream_t (NULL = the null stream). Forward and cache update
 *    are stream-ordered; kernel faults surface as MOE_E_HIP at the next call
 *    that synchronises (moe_plan_stats, moe_cache_update, moe_plan_destroy).
 *  - A plan is externally synchronised: no two calls on one plan at once.
 */
#ifndef MOE_OFFLOAD_H
#define MOE_OFFLOAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_plan moe_plan; /* opaque, owned by the library */
typedef void* moe_stream;         /* a hipStream_t */

typedef enum {
  MOE_OK = 0,
  MOE_E_INVALID = 1,     /* bad argument, shape or state of an argument */
  MOE_E_NOMEM = 2,       /* device (HBM) allocation failed */
  MOE_E_HOST_NOMEM = 3,  /* pinned host allocation failed */
  MOE_E_HIP = 4,         /* a HIP runtime call failed, or an earlier kernel faulted */
  MOE_E_UNSUPPORTED = 5, /* valid request this build does not handle */
  MOE_E_STATE = 6        /* call not allowed in the plan's current state */
} moe_status;

typedef enum { MOE_ACT_F32 = 0, MOE_ACT_BF16 = 1 } moe_act_dtype;

typedef struct {
  int32_t hidden;          /* H; multiple of 64 and of group_size */
  int32_t inter;           /* I; multiple of 32 and of group_size */
  int32_t num_experts;     /* E; 1..1024 */
  int32_t top_k;           /* k; 1..min(E, 32) */
  int32_t group_size;      /* G; 32, 64, 128 or 256 */
  int32_t num_layers;      /* L >= 1 */
  int32_t act_dtype;       /* moe_act_dtype of x, router weights and the intermediate h */
  int32_t max_tokens;      /* largest T of any forward; sizes the workspace */
  int32_t hbm_slots;       /* HBM expert slots per layer, 0..E */
  int32_t gemm_min_tokens; /* forwards with T >= this use the grouped MFMA GEMM path
                              (bf16 only; never for T <= 4, which take the one-launch
                              decode routing and the GEMVs); 0 = library default (6:
                              from about 6 tokens, experts shared by several tokens
                              make the GEMM faster than the GEMVs), < 0 = never */
  int32_t prefill_stage_slots; /* 0..E HBM slots, shared by all layers, into which a
                              GEMM-path forward first copies the offloaded experts its
                              routing touches (one read of each over the host link, by
                              a copy kernel, before the GEMMs; those then re-read HBM
                              once per 64-row tile). Active offloaded experts beyond
                              this count are read in place. 0 = none: the GEMMs read
                              every offloaded expert in place. [24K] section 二 keeps
                              the experts in use in VRAM slots; [125B] section
                              "真正卡死容量的是一块计算缓冲" sizes prefill micro-batches
                              at 1024/2048 tokens, which makes in-place re-reads large */
  int32_t weight_bits;     /* bits per weight code: 4 (0 = 4), 3 or 2. [763B] section "显存缺口从
                              哪里来" packs the experts at 3 bits, [24K] section 二 at about 2
                              bits; neither layout is given, so the library defines its own (see
                              the canonical blob below). 2 and 3 bits need bf16 activations,
                              group_size >= 64 and inter a multiple of 64; their forwards run
                              on the dequant-GEMVs for every batch size (no MFMA path) */
  int32_t prefetch_slots;  /* 0..min(E, 64) extra HBM slots per layer that moe_prefetch fills with
                              the experts it predicts; 0 = no prefetch */
} moe_config;

typedef struct {
  const void* router_w;    /* host [E][H], act dtype (fp32 or bf16 bits) */
  const float* router_b;   /* host [E] fp32, or NULL for zeros */
  const uint8_t* experts;  /* host [E][expert_bytes] canonical blobs */
} moe_layer_weights;

typedef struct {          /* optional routing outputs, device pointers, each may be NULL */
  float* logits;          /* [T][E] fp32 (the router's, or a copy of logits_in) */
  int32_t* topk_ids;      /* [T][k] */
  float* topk_w;          /* [T][k] */
  int32_t* counts;        /* [E]   assignments per expert */
  int32_t* offsets;       /* [E+1] exclusive prefix sum of counts */
  int32_t* sorted;        /* [T*k] assignments a = t*k + j grouped by expert, ascending a within */
  int32_t* inv;           /* [T*k] inv[sorted[p]] = p */
} moe_routing;

typedef struct {
  int64_t forwards;       /* moe_layer_forward calls with T > 0 */
  int64_t tokens;         /* sum of T */
  int64_t hits;           /* assignments whose expert was in HBM */
  int64_t misses;         /* assignments whose expert was read from host memory */
  int64_t bytes_hbm;      /* canonical expert bytes of unique HBM experts touched, per forward */
  int64_t bytes_host;     /* canonical expert bytes of unique host experts touched, per forward */
  int64_t bytes_copied;   /* host -> HBM bytes copied by cache updates */
  int64_t promotions;     /* experts moved into HBM slots by cache updates */
  int64_t evictions;      /* experts sent back to their host copy by cache updates */
  int64_t host_computed;  /* unique experts whose FFN the host cores computed, per forward, summed
                             (moe_plan_set_host_compute); their bytes are read from host memory by
                             the CPU, not over the host link, though bytes_host still counts them
                             when they are offloaded */
  int64_t prefetched;     /* experts copied host -> prefetch slot by moe_prefetch */
} moe_stats;

/* Where the experts of a layer are computed (moe_plan_set_host_compute). */
typedef enum {
  MOE_HOST_COMPUTE_NONE = 0,    /* the GPU computes every expert; offloaded ones read in place over the host link */
  MOE_HOST_COMPUTE_MISSES = 1,  /* the host cores compute the experts read from host memory, the GPU the rest */
  MOE_HOST_COMPUTE_LAYER = 2    /* the host cores compute every expert of the layer; the GPU routes and combines */
} moe_host_compute;

typedef struct {
  double decay;           /* score_e <- decay * score_e + count_e; default 0.9 */
  int32_t max_promotions; /* per layer per update; default 8 */
  int32_t overlap;        /* 0: synchronous update; 1: pipelined update (see moe_cache_update) */
  const int32_t* want_resident; /* NULL: the frequency policy. Else host [E] (one layer) or
                              [L][E] (layer = -1): 1 = the expert must read from HBM after
                              the update, 0 = from its host copy; at most hbm_slots ones per
                              layer. The update evicts every resident expert not wanted,
                              then copies every wanted non-resident into the lowest free
                              slots in ascending expert id (max_promotions does not apply);
                              scores still take the counts. Always synchronous. */
} moe_cache_policy;

/* Kernel classes timed by the profiling hooks. */
typedef enum {
  MOE_K_ROUTER = 0,      /* router logits and per-group activation sums */
  MOE_K_ROUTE = 1,       /* top-k, counts, offsets, permutation, active list */
  MOE_K_GATEUP = 2,      /* gate/up dequant-GEMV + SwiGLU (decode path) */
  MOE_K_DOWN = 3,        /* down dequant-GEMV (decode path) */
  MOE_K_COMBINE = 4,     /* gate-weighted combine */
  MOE_K_GEMM_GATEUP = 5, /* gate/up grouped MFMA GEMM + SwiGLU (prefill path) */
  MOE_K_GEMM_DOWN = 6,   /* down grouped MFMA GEMM (prefill path) */
  MOE_K_STAGE = 7,       /* copy of offloaded experts into prefill staging slots */
  MOE_K_COUNT = 8
} moe_kernel;

typedef struct {
  int64_t launches[MOE_K_COUNT]; /* launches recorded per kernel class */
  double total_ms[MOE_K_COUNT];  /* summed GPU time between the events around them */
} moe_kernel_times;

typedef struct {
  int32_t device;           /* HIP device of the plan */
  int32_t gpu_numa_node;    /* host NUMA node closest to the GPU, -1 if not reported */
  int32_t host_pool_node;   /* NUMA node of the host pool's first page, -1 if unknown */
  int32_t numa_bound;       /* 1 = the host pool was allocated under a policy preferring gpu_numa_node */
  int64_t internal_expert_bytes; /* bytes of one expert in the library's layout */
  int64_t host_pool_bytes;  /* pinned host bytes of all layers' host copies */
  int64_t hbm_slot_bytes;   /* device bytes of all layers' HBM slots */
  int64_t workspace_bytes;  /* device bytes of the forward workspace */
} moe_plan_info;

typedef struct {
  double hbm_read_gbps;     /* streaming-read kernel over a device buffer */
  double host_read_gbps;    /* the same kernel over pinned, device-mapped host memory */
  double h2d_copy_gbps;     /* hipMemcpyAsync host -> device from pinned host memory */
} moe_link_ceilings;

/* Canonical bytes of one expert for cfg: 3*H*I*b/8 + 6*H*I/G (b = weight_bits).
 * Errors: MOE_E_INVALID (cfg). */
moe_status moe_expert_bytes(const moe_config* cfg, size_t* out);

/* Create a plan: HBM slots for every layer, the pinned device-mapped host pool
 * (every expert of every layer), router weights and the workspace for
 * max_tokens, then (when `layers` is given) load every layer's weights as
 * moe_plan_load_layer does.
 *   layers:      host [L] weights, or NULL to load layers later one by one.
 *   initial_hbm: host [L][E], 1 = the expert starts in an HBM slot (at most
 *                hbm_slots ones per layer), or NULL: experts 0..hbm_slots-1.
 *                Ignored when layers is NULL.
 * [763B] section "同一个思路，vLLM 原生方案反而跑不通": residency and read path
 * are decided for each expert individually; [763B] section "显存缺口从哪里来":
 * the experts left out of VRAM are read by GPU kernels from host memory in
 * place; [24K] section 二: every expert pinned in host RAM, free VRAM a cache.
 * The caller's host buffers may be freed when the call returns.
 * On failure *out is NULL and nothing stays allocated.
 * Errors: MOE_E_INVALID (cfg, weights, initial_hbm), MOE_E_NOMEM,
 * MOE_E_HOST_NOMEM, MOE_E_HIP. */
moe_status moe_plan_create(const moe_config* cfg, const moe_layer_weights* layers, const int32_t* initial_hbm,
                           moe_stream stream, moe_plan** out);

/* Copy one layer's weights into the plan: repack every expert into the host
 * pool, copy the initially resident ones into HBM slots, router weights to the
 * device; reset that layer's counters and cache scores. Same sources as
 * moe_plan_create.
 *   initial_hbm: host [E] (1 = start in an HBM slot, at most hbm_slots ones) or
 *                NULL: experts 0..hbm_slots-1.
 * Synchronises `stream`; the host buffers may be freed when the call returns.
 * Errors: MOE_E_INVALID, MOE_E_HIP. */
moe_status moe_plan_load_layer(moe_plan* plan, int32_t layer, const moe_layer_weights* w,
                               const int32_t* initial_hbm, moe_stream stream);

/* Forward of one layer for T tokens, enqueued on `stream`: router logits, top-k
 * gate choice, grouping of the token-expert assignments by expert, each touched
 * expert's SwiGLU FFN read from its HBM slot or in place from host memory, and
 * the gate-weighted combine. [763B] section "显存缺口从哪里来": each token, in
 * each layer, uses a few routed experts (6 of 384), and experts outside VRAM
 * are read over PCIe by the GPU kernels; [24K] section "一、第一个坑:MoE 省算力,
 * 不省内存": the gate picks them at run time.
 * x: device [T][H] act dtype. y: device [T][H] fp32 (written, not accumulated).
 * logits_in: device [T][E] fp32 or NULL; when given, routing uses it and the
 *   router is skipped (the ids then do not depend on the router's rounding).
 * route_out: NULL or device buffers for the routing results.
 * T == 0 is a no-op. Errors: MOE_E_INVALID (T > max_tokens, unloaded layer,
 * misaligned pointer), MOE_E_HIP (launch failure). */
moe_status moe_layer_forward(moe_plan* plan, int32_t layer, int32_t T, const void* x,
                             const float* logits_in, float* y, const moe_routing* route_out,
                             moe_stream stream);

/* The forward, and the residual stream's next value with it: y as moe_layer_forward,
 * and x_out[t][h] = act(x[t][h] + y[t][h]) (the sum formed in fp32, rounded to bf16,
 * nearest even, for bf16 activations), written by the same kernel that writes y. The
 * pages place the MoE FFN inside a transformer's layers ([125B] and [24K]: the
 * experts of each layer), whose output adds to the residual stream; fusing that add
 * saves a launch and a round trip of y per layer. x_out: device [T][H] act dtype,
 * 16-byte aligned, overlapping neither x nor y. Errors: as moe_layer_forward. */
moe_status moe_layer_forward_residual(moe_plan* plan, int32_t layer, int32_t T, const void* x,
                                      const float* logits_in, float* y, void* x_out,
                                      const moe_routing* route_out, moe_stream stream);

/* moe_layer_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation. The
 * same kernels and results (bitwise), with the forward's workspace (logits,
 * routing tables, work descriptors, the intermediate h and the down outputs)
 * carved from a static device array of the library instead of the plan's
 * workspace; the call allocates nothing. The array holds 8 MiB per device
 * (held until the process ends), which covers decode batches (a
 * H7168/I2048/E384/k6 layer: about 200 KiB per token). One array serves every
 * plan on a device and keeps the last call's contents: calls on one GPU that
 * overlap in time (different streams, or host threads) race, so order them.
 * The plan itself (weights, tables, counters) is created as usual.
 * Errors: as moe_layer_forward; MOE_E_INVALID also when this forward's workspace
 * exceeds 8 MiB (the message gives the bytes needed). */
moe_status moe_layer_forward_noalloc(moe_plan* plan, int32_t layer, int32_t T, const void* x,
                                     const float* logits_in, float* y, const moe_routing* route_out,
                                     moe_stream stream);

/* Predictive prefetch of one layer ([24K] section 二: while the current layer is
 * computed, the next layer's experts are already streaming over the link into
 * VRAM). The pages do not say how the experts are chosen; the plain reading taken
 * is the layer's own router applied to the activations at hand, normally the
 * current layer's input x (or the given logits_in [T][E] fp32), since the residual
 * stream changes little from one layer to the next:
 *   candidates = each token's `candidates` best experts (0 = top_k; at most 64 and
 *                E), in the routing's order, tokens in order, T * candidates <= 2048;
 *   predicted  = the first prefetch_slots distinct candidates whose weights are read
 *                from host memory without a prefetch (their host copy, or a prefetch
 *                slot of this layer);
 *   the layer's prefetch slots: a slot whose expert is predicted again keeps it;
 *                every other slot gives its expert back to its host copy; each
 *                predicted expert not in a slot is copied into the lowest free slot.
 * Until the next moe_prefetch of the layer, forwards read the slotted experts from
 * HBM (hits). The work (router rows, prediction, copies) runs on a stream of the
 * plan, after the work enqueued on `stream` before this call: x must be ready there,
 * and the layer's earlier forwards and the plan's cache updates must be ordered
 * before that point (enqueued on `stream`, or joined to it by the caller's events).
 * The layer's next forward, cache update or load waits for the prefetch on the
 * device, on whatever stream it runs. So a prefetch of layer l+1 issued just before
 * the forward of layer l overlaps that forward. Both calls may be captured into a
 * HIP graph (the prefetch stream forks from and joins the capturing stream).
 * x [T][H] act dtype device (unused when logits_in is given); predicted_out: device
 * int32 [prefetch_slots] or NULL, the predicted experts in order, -1 after the last.
 * Cache updates rewrite whole tables and so give prefetched experts back to their
 * host copies (or HBM slots). Errors: MOE_E_INVALID (arguments, T out of
 * 1..max_tokens, layer not loaded), MOE_E_STATE (prefetch_slots == 0), MOE_E_HIP. */
moe_status moe_prefetch(moe_plan* plan, int32_t layer, int32_t T, const void* x, const float* logits_in,
                        int32_t candidates, int32_t* predicted_out, moe_stream stream);

/* Host [prefetch_slots] slot table of a layer's prefetch: slot_expert[i] = the
 * expert prefetch slot i holds, -1 none (a slot whose table entry a cache update
 * has since rewritten still lists its expert until the next prefetch frees it).
 * Waits for the layer's prefetch work. Errors: MOE_E_INVALID, MOE_E_STATE, MOE_E_HIP. */
moe_status moe_plan_prefetch_slots(moe_plan* plan, int32_t layer, int32_t* slot_expert);

/* Expert-cache update of one layer (or all, layer = -1). [24K] section 二: free
 * VRAM holds the most used experts, and the cache adapts the longer it runs; the
 * pages give no policy, so the plain frequency reading is taken:
 * scores decay and accumulate the assignment counts since the last update; the
 * hbm_slots highest-scored experts are wanted in HBM; up to max_promotions
 * wanted experts per layer are copied host -> HBM slot (DMA on `stream`),
 * each into an empty slot or the slot of the lowest-scored resident no longer
 * wanted, which goes back to being read from its host copy. The pointer-table
 * switch is enqueued after the copies on `stream`, so forwards enqueued later
 * on the same stream see it and earlier ones finish on the old table; other
 * streams must order themselves with events. Synchronises `stream` first to
 * read the counts. policy NULL = defaults. policy->want_resident replaces the
 * frequency choice by the caller's set (see moe_cache_policy).
 * Pipelined form (policy->overlap = 1), for decode loops that update after every
 * step: the host does not wait for the step just enqueued. The counts of the
 * forwards since the last update are staged (one copy for all the layers) and
 * used by the next update; this update's policy uses the counts the previous
 * update staged, so decisions lag one update behind. The new pointer tables
 * (evictions now, promotions not yet) are uploaded on `stream` with one copy;
 * the promotion copies then run on a copy stream of the plan, after that upload,
 * overlapping the forwards enqueued next, and the promoted experts are switched
 * to HBM by the next update's table upload, which waits for the copies on the
 * device. moe_plan_residency reports the table the kernels read (a promotion in
 * flight reads as -1). A synchronous update after pipelined ones first waits for
 * their copies and adds the counts they staged.
 * Errors: MOE_E_INVALID, MOE_E_STATE (hbm_slots == 0), MOE_E_HIP. */
moe_status moe_cache_update(moe_plan* plan, int32_t layer, const moe_cache_policy* policy,
                            moe_stream stream);

/* Where a layer's experts are computed (one layer, or all for layer = -1), for plans
 * with 4-bit codes on a host with AVX-512. [24K] section 二 computes the experts that
 * are not in VRAM on the CPU; [125B] sections "先说结论" and "排除法" keep whole
 * layers' experts on the CPU (ncmoe), where the serialisation between GPU and CPU
 * was the measured cost. With a host mode, a forward on the layer enqueues the routing
 * and copies the routing results and x to pinned host memory; the GPU's GEMVs skip the
 * experts the host computes; the call then waits for the routing (the GPU meanwhile
 * computes its experts), computes those experts on `threads` host threads (<= 0: the
 * cores this process may use) from the host pool, copies their rows into the
 * forward's workspace and enqueues the gate-weighted combine, which merges all rows in
 * slot order. So the call returns after the host part is done. Host-computed rows are
 * fp32 sums in another order than the GPU's: results match the oracle's tolerance,
 * not the GPU path bit for bit. Batches of a host-mode layer run on the GEMV path.
 * Errors: MOE_E_INVALID (layer, mode), MOE_E_UNSUPPORTED (codes other than 4-bit, no
 * AVX-512), MOE_E_HOST_NOMEM (pinned staging), MOE_E_HIP. */
moe_status moe_plan_set_host_compute(moe_plan* plan, int32_t layer, int32_t mode, int32_t threads);

/* Counters of one layer, or summed over layers for layer = -1: hits and misses
 * per assignment and expert bytes per link, the quantities [763B] section
 * "显存缺口从哪里来" weighs (how often an offloaded expert is needed, and the
 * PCIe bytes it costs). Synchronises the device. Errors: MOE_E_INVALID, MOE_E_HIP. */
moe_status moe_plan_stats(moe_plan* plan, int32_t layer, moe_stats* out);

/* Zero the counters of every layer (not the cache scores). Synchronises the device. */
moe_status moe_plan_reset_stats(moe_plan* plan);

/* Host [E] slot table of a layer: slot_of[e] = HBM slot, or -1 when read from
 * host memory (the per-expert plan of [763B] section "同一个思路，vLLM 原生方案
 * 反而跑不通"). Does not synchronise. Errors: MOE_E_INVALID. */
moe_status moe_plan_residency(moe_plan* plan, int32_t layer, int32_t* slot_of);

/* Sizes and host-memory placement of a plan. [763B] section "PCIe 拓扑：容易被
 * 忽略的性能变量": host memory on the GPU's NUMA node matters for the host link.
 * Errors: MOE_E_INVALID. */
moe_status moe_plan_get_info(moe_plan* plan, moe_plan_info* out);

/* Profiling: enable != 0 starts recording a HIP event pair around every kernel
 * launch of moe_layer_forward on its stream (and drops earlier records);
 * enable == 0 stops. Recording adds event packets between kernels, so time
 * end-to-end throughput with it off. Errors: MOE_E_INVALID. */
moe_status moe_plan_profile(moe_plan* plan, int32_t enable);

/* Per-class launch counts and summed durations of the recorded launches.
 * Synchronises the device. Errors: MOE_E_INVALID, MOE_E_HIP. */
moe_status moe_plan_kernel_times(moe_plan* plan, moe_kernel_times* out);

/* Measured ceilings of the two links the experts are read over, on the current
 * device ([763B] section "显存缺口从哪里来" gives PCIe 5.0 x16 at about 64 GB/s
 * per direction against on-card memory; section "PCIe 拓扑" found the placement
 * of host memory to matter): a streaming-read kernel over hbm_bytes of device
 * memory and over host_bytes of pinned device-mapped host memory (on the GPU's
 * NUMA node when reported), and hipMemcpyAsync of host_bytes host -> device.
 * Each figure is the best of `iters` timed runs after one untimed run. The call
 * allocates and frees its own buffers and synchronises `stream`.
 * Errors: MOE_E_INVALID (sizes < 1 MiB or not multiples of 4 KiB, iters < 1),
 * MOE_E_NOMEM, MOE_E_HOST_NOMEM, MOE_E_HIP. */
moe_status moe_measure_link_ceilings(size_t hbm_bytes, size_t host_bytes, int32_t iters, moe_stream stream,
                                     moe_link_ceilings* out);

/* Free everything the plan owns (synchronises the device first). NULL is a no-op. */
void moe_plan_destroy(moe_plan* plan);

const char* moe_status_str(moe_status s);

/* Message of the last failed call on this thread ("" if none). */
const char* moe_last_error(void);

/* Test hook for the allocation-failure paths: after this call, the n-th next
 * device allocation (kind 0) or pinned host allocation (kind 1) made by this
 * library on any thread fails as if out of memory (n >= 1; n = 0 disarms).
 * The failing call then returns MOE_E_NOMEM / MOE_E_HOST_NOMEM and frees what
 * it had allocated. Errors: MOE_E_INVALID (kind or n out of range). */
moe_status moe_debug_fail_alloc(int32_t kind, int32_t n);

/* Test hook: the device and pinned host allocations this library currently holds
 * (over all plans). Errors: MOE_E_INVALID (null argument). */
moe_status moe_debug_live_allocs(int64_t* device, int64_t* host);

#ifdef __cplusplus
}
#endif

#endif /* MOE_OFFLOAD_H */
