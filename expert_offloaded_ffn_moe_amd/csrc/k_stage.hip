// Prefill staging of offloaded experts: before the grouped GEMMs of a large
// batch, one kernel copies every offloaded expert that the batch's routing
// touched from its pinned, device-mapped host copy into a reserved HBM slot,
// and writes the per-forward blob table the GEMMs read. Each such expert then
// crosses the host link once, in long coalesced reads with many loads in
// flight, instead of once per 64-row tile of its routed rows.
//
// Page "我在 32GB 单卡上跑两万四千专家的 MoE…", section 二, keeps the experts a
// batch needs in VRAM slots and reads the rest from host memory; page "125B
// 稀疏模型塞进一张 32GB 消费卡" runs prefill in micro-batches of 1024 and 2048
// tokens, where an expert carries about a hundred rows and in-place reads would
// repeat per row tile.
#include <hip/hip_runtime.h>

#include "copy_dev.h"
#include "kernels.h"

namespace moe {

// Blocks [0, table_blocks): the blob table, one thread per expert. Then
// n_slots * blocks_per_expert copy blocks: block (s, part) copies part `part`
// of the expert at active-list position s, if that expert is read from host
// memory (host-read experts lead the active list, so positions below n_slots
// that hold one are exactly the staged experts).
__global__ __launch_bounds__(kCopyThreads) void k_stage(StageArgs a) {
  const int tb = a.table_blocks;
  if ((int)blockIdx.x < tb) {
    const int e = blockIdx.x * kCopyThreads + threadIdx.x;
    if (e < a.E) {
      const int pos = a.act_pos[e];
      const bool staged = a.counts[e] > 0 && a.is_host[e] != 0 && pos >= 0 && pos < a.n_slots;
      a.gptr[e] = staged ? a.stage + (size_t)pos * a.bytes : a.wptr[e];
    }
    return;
  }
  const int b = blockIdx.x - tb;
  const int s = b / a.blocks_per_expert, part = b % a.blocks_per_expert;
  if (s >= *a.n_active) return;
  const int e = a.active[s];
  if (a.is_host[e] == 0) return;
  const int64_t n16 = a.bytes / 16;
  const int64_t u0 = (int64_t)part * kCopyUnits, u1 = u0 + kCopyUnits < n16 ? u0 + kCopyUnits : n16;
  copy_units(a.wptr[e], a.stage + (size_t)s * a.bytes, u0, u1);
}

void launch_stage(StageArgs a, const Timing& tm, hipStream_t s) {
  a.table_blocks = (a.E + kCopyThreads - 1) / kCopyThreads;
  a.blocks_per_expert = (int)((a.bytes / 16 + kCopyUnits - 1) / kCopyUnits);
  const int grid = a.table_blocks + a.n_slots * a.blocks_per_expert;
  launch_timed(k_stage, dim3(grid), dim3(kCopyThreads), 0, s, tm, a);
}

}  // namespace moe
