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
 * Sources (the pages describe the problem; the numerics above are the plain
 * reading of it):
 *  - "763B MoE 塞进两张 96GB 显卡：闲置专家丢进主机内存", section "显存缺口从哪里来":
 *    a few routed experts per token per layer (6 of 384); idle experts moved
 *    to host memory and read by GPU kernels in place over PCIe through
 *    unified addressing, without explicit copies.
 *  - same page, section "同一个思路，vLLM 原生方案反而跑不通": a per-expert plan,
 *    residency and read path decided for each expert individually.
 *  - same page, section "PCIe 拓扑：容易被忽略的性能变量": keep host-resident
 *    experts on the GPU's NUMA node.
 *  - "我在 32GB 单卡上跑两万四千专家的 MoE:分层放置实测与三个坑", section
 *    "二、跑起来靠的是分层,不是激活": all experts pinned in host RAM, free VRAM
 *    turned into an expert cache of the most used experts that adapts with use.
 *
 * Residency. Every expert of every layer has a copy in pinned, device-mapped
 * host memory (hipHostMalloc). A layer has `hbm_slots` HBM slots; an expert in
 * a slot is read from HBM, every other expert is read by the kernels directly
 * from its host copy over the host link. moe_cache_update moves experts
 * between the two.
 *
 * Canonical expert blob (the weight format of this ABI), per expert:
 *   q_gate[I][H/2] | q_up[I][H/2] | q_down[H][I/2] | s_gate[I][H/G] | s_up[I][H/G] | s_down[H][I/G]
 * K is contiguous. Byte j of a row = (q[2j] & 0xF) | (q[2j+1] & 0xF) << 4;
 * nibbles are two's complement (-8..7). Scales are IEEE fp16; s[n][g] covers
 * k in [g*G, (g+1)*G). The library repacks blobs into its own layout.
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
  int32_t group_size;      /* G; multiple of 32 */
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
                              every offloaded expert in place. Page "我在 32GB 单卡上
                              跑两万四千专家的 MoE", section 二, has the VRAM cache
                              keep slots for the experts a batch needs; P2's prefill
                              micro-batches (ub 1024/2048) make the re-reads large */
} moe_config;

typedef struct {
  const void* router_w;    /* host [E][H], act dtype (fp32 or bf16 bits) */
  const float* router_b;   /* host [E] fp32, or NULL for zeros */
  const uint8_t* experts;  /* host [E][expert_bytes] canonical blobs */
  const int32_t* resident; /* host [E], 1 = start in an HBM slot; at most hbm_slots ones.
                              NULL = experts 0..hbm_slots-1 */
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
} moe_stats;

typedef struct {
  double decay;           /* score_e <- decay * score_e + count_e; default 0.9 */
  int32_t max_promotions; /* per layer per update; default 8 */
  int32_t overlap;        /* 0: synchronous update; 1: pipelined update (see moe_cache_update) */
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

/* Canonical bytes of one expert for cfg: 3*H*I/2 + 6*H*I/G. */
moe_status moe_expert_bytes(const moe_config* cfg, size_t* out);

/* Validate cfg and allocate a plan: HBM slots for every layer, the pinned
 * device-mapped host pool (all experts of all layers), router weights and
 * the workspace for max_tokens. Weights are loaded by moe_plan_load_layer.
 * On failure *out is NULL and nothing stays allocated.
 * Errors: MOE_E_INVALID (cfg), MOE_E_NOMEM, MOE_E_HOST_NOMEM, MOE_E_HIP. */
moe_status moe_plan_create(const moe_config* cfg, moe_stream stream, moe_plan** out);

/* Copy one layer's weights into the plan (host pool for every expert, HBM slots
 * for the resident ones, router weights to the device) and reset that layer's
 * counters. The host buffers may be freed when the call returns (it
 * synchronises `stream`). Errors: MOE_E_INVALID, MOE_E_HIP. */
moe_status moe_plan_load_layer(moe_plan* plan, int32_t layer, const moe_layer_weights* w,
                               moe_stream stream);

/* Forward of one layer for T tokens, enqueued on `stream`.
 * x: device [T][H] act dtype. y: device [T][H] fp32 (written, not accumulated).
 * logits_in: device [T][E] fp32 or NULL; when given, routing uses it and the
 *   router is skipped (the ids then do not depend on the router's rounding).
 * route_out: NULL or device buffers for the routing results.
 * T == 0 is a no-op. Errors: MOE_E_INVALID (T > max_tokens, unloaded layer,
 * misaligned pointer), MOE_E_HIP (launch failure). */
moe_status moe_layer_forward(moe_plan* plan, int32_t layer, int32_t T, const void* x,
                             const float* logits_in, float* y, const moe_routing* route_out,
                             moe_stream stream);

/* Expert-cache update of one layer (or all, layer = -1) from the assignment
 * counts since the last update: frequency scores decay and accumulate; the
 * hbm_slots highest-scored experts are wanted in HBM; up to max_promotions
 * wanted experts per layer are copied host -> HBM slot (DMA on `stream`),
 * each into an empty slot or the slot of the lowest-scored resident no longer
 * wanted, which goes back to being read from its host copy. The pointer-table
 * switch is enqueued after the copies on `stream`, so forwards enqueued later
 * on the same stream see it and earlier ones finish on the old table; other
 * streams must order themselves with events. Synchronises `stream` first to
 * read the counts. policy NULL = defaults.
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

/* Counters of one layer, or summed over layers for layer = -1. Synchronises the device. */
moe_status moe_plan_stats(moe_plan* plan, int32_t layer, moe_stats* out);

/* Zero the counters of every layer (not the cache scores). Synchronises the device. */
moe_status moe_plan_reset_stats(moe_plan* plan);

/* Host [E] slot table of a layer: slot_of[e] = HBM slot, or -1 when read from host memory. */
moe_status moe_plan_residency(moe_plan* plan, int32_t layer, int32_t* slot_of);

/* Profiling: enable != 0 starts recording a HIP event pair around every kernel
 * launch of moe_layer_forward on its stream (and drops earlier records);
 * enable == 0 stops. Recording adds event packets between kernels, so time
 * end-to-end throughput with it off. Errors: MOE_E_INVALID. */
moe_status moe_plan_profile(moe_plan* plan, int32_t enable);

/* Per-class launch counts and summed durations of the recorded launches.
 * Synchronises the device. Errors: MOE_E_INVALID, MOE_E_HIP. */
moe_status moe_plan_kernel_times(moe_plan* plan, moe_kernel_times* out);

/* Free everything the plan owns (synchronises the device first). NULL is a no-op. */
void moe_plan_destroy(moe_plan* plan);

const char* moe_status_str(moe_status s);

/* Message of the last failed call on this thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_OFFLOAD_H */
