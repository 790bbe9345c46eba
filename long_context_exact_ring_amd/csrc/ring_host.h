// Internal host-side declarations of the ring-attention library.
#pragma once

#include <stddef.h>

#include <vector>

namespace ra {

struct Shape {
  int n_blocks = 0, block_len = 0, heads = 0, kv_heads = 0, head_dim = 0;
  int causal = 0, rank = 0;
  int elem_bytes = 2;  // 2 = bf16 inputs, 4 = fp32 inputs
  int zigzag = 0;      // block j holds sequence chunks j and 2D-1-j (half a block each)
  // blocks the ring visits: with the zig-zag layout every block holds work for every rank
  int schedule_causal() const { return causal && !zigzag; }
  size_t q_bytes() const { return (size_t)block_len * heads * head_dim * elem_bytes; }
  size_t kv_bytes() const { return (size_t)block_len * kv_heads * head_dim * elem_bytes; }
  size_t kv_f32_bytes() const { return (size_t)block_len * kv_heads * head_dim * 4; }
  size_t out_bytes() const { return (size_t)block_len * heads * head_dim * 4; }
  size_t lse_bytes() const { return (size_t)block_len * heads * 4; }
};

// Sequence-block ids in ring order for one rank: round s uses (rank - s) mod D;
// causal drops rounds with a block id greater than the rank.
std::vector<int> ring_schedule(int rank, int n_blocks, int causal);

}  // namespace ra
