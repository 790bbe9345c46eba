// Internal host-side declarations of the ring-attention library.
#pragma once

#include <stddef.h>

#include <vector>

namespace ra {

struct Shape {
  int n_blocks = 0, block_len = 0, heads = 0, kv_heads = 0, head_dim = 0;
  int causal = 0, rank = 0;
  int elem_bytes = 2;  // 2 = bf16 inputs, 4 = fp32 inputs
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
