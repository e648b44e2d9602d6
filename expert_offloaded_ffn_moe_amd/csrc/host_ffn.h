// Host (CPU) computation of expert FFNs, for layers whose offloaded experts are
// computed by the host cores instead of being read over the host link by the GPU
// (page "我在 32GB 单卡上跑两万四千专家的 MoE:分层放置实测与三个坑", section
// "二、跑起来靠的是分层,不是激活": experts missing from VRAM are computed by the
// CPU; page "125B 稀疏模型塞进一张 32GB 消费卡", section "先说结论": whole layers'
// experts on the CPU, where serialisation was the measured cost).
//
// The expert is read from the host pool in the library's internal layout (4-bit
// codes only). Per output row: g = sum_k q s x over K in fp32 (int codes exact,
// the group scale multiplying the group's sum), h = silu(g) * u (rounded to bf16 for
// bf16 layers), o = the down row's sum over h in fp32. Needs AVX-512 (F, BW, VL) and
// F16C; host_ffn_supported() says whether this CPU has them.
#pragma once

#include <cstdint>
#include <functional>

#include "host_logic.h"

namespace moe {

bool host_ffn_supported();

// A persistent pool of worker threads for the host FFN (created once per plan).
class HostPool {
 public:
  explicit HostPool(int threads);
  ~HostPool();
  int threads() const;
  // fn(item) for item in [0, n), spread over the workers and the calling thread; returns when all are done
  void run(int n, const std::function<void(int)>& fn);

 private:
  struct Impl;
  Impl* impl_;
};

// One expert (internal blob `blob`) on M tokens: x [M][H] fp32 -> o [M][H] fp32.
// h [M][I] fp32 is caller scratch, rounded to bf16 when h_bf16 (the activation dtype
// of the layer), else kept fp32. Work is spread over the pool (tiles of rows).
void host_expert_ffn(const Layout& L, const uint8_t* blob, const float* x, int M, float* h, float* o, bool h_bf16,
                     HostPool& pool);

// Several experts at once (both phases spread over the pool across experts):
// expert i has blob[i], M[i] tokens with rows x_i = x + x_off[i] * H, h_i = h + x_off[i] * I,
// o_i = o + x_off[i] * H.
void host_experts_ffn(const Layout& L, int n_experts, const uint8_t* const* blob, const int* M, const int* x_off,
                      const float* x, float* h, float* o, bool h_bf16, HostPool& pool);

}  // namespace moe
