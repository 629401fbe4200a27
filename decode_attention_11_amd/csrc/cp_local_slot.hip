// Rank-local KV slot mapping under decode context parallelism, gfx950.
//
// Follows the cp_local_slot definition on the PR #52188 page (key source
// snippets): positions fall into virtual blocks of block_size*cp_world
// (the DFlash input preparation's block index, same page, implementation
// breakdown); inside a virtual block, segments of cp_interleave positions are
// dealt to ranks in turn; an owned position's local offset counts whole
// rounds of segments and then its offset inside the segment; positions of
// other ranks, the rejected suffix (index >= num_valid[b]), negative
// positions and virtual blocks past the table width get the pad slot.
// The block-table lookup is fused.  All arithmetic is int64 and exact.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "mla_decode.h"
#include "mla_device.h"

namespace {

using mla::floordiv;

struct SlotArgs {
  const int64_t* pos;
  const int32_t* num_valid;
  const int32_t* bt;
  int64_t total;
  int n, max_blocks;
  int64_t bs, W, rank, I;
  int64_t* slots;
};

__global__ __launch_bounds__(256) void slot_kernel(SlotArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= a.total) return;
  const int64_t b = floordiv(idx, a.n);
  const int64_t i = idx - b * a.n;
  const int64_t pos = a.pos[idx];
  int64_t slot = MLA_PAD_SLOT_ID;
  const bool valid = (a.num_valid == nullptr || i < (int64_t)a.num_valid[b]) && pos >= 0;
  if (valid) {
    const int64_t span = a.bs * a.W;
    const int64_t v = floordiv(pos, span);
    const int64_t off = pos - v * span;
    if (v < a.max_blocks) {
      const int64_t base = (int64_t)a.bt[b * a.max_blocks + v] * a.bs;
      if (a.W == 1) {
        slot = base + off;
      } else {
        // segment of I positions inside the virtual block, its owner, and
        // the rounds of W segments before it
        const int64_t seg = floordiv(off, a.I);
        const int64_t round = floordiv(seg, a.W);
        if (seg - round * a.W == a.rank) slot = base + round * a.I + (off - seg * a.I);
      }
    }
  }
  a.slots[idx] = slot;
}

}  // namespace

extern "C" int cp_local_slot(const int64_t* positions, const int32_t* num_valid, int B, int n,
                             const int32_t* block_table, int max_blocks, int block_size,
                             int cp_world, int cp_rank, int cp_interleave, int64_t* slots,
                             hipStream_t stream) {
  if (B < 0 || n < 0 || max_blocks < 1 || block_size < 1 || cp_world < 1 || cp_rank < 0 ||
      cp_rank >= cp_world || cp_interleave < 1 || block_size % cp_interleave != 0)
    return MLA_ERR_INVALID_ARG;
  const int64_t total = (int64_t)B * n;
  if (total == 0) return MLA_OK;
  if (!positions || !block_table || !slots) return MLA_ERR_INVALID_ARG;
  SlotArgs a{positions, num_valid, block_table, total, n, max_blocks,
             block_size, cp_world, cp_rank, cp_interleave, slots};
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7FFFFFFF) return MLA_ERR_INVALID_ARG;
  if (mla::launch(slot_kernel, dim3((unsigned)blocks), dim3(256), stream, a) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}
