// Host-visible launch interface of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

namespace ra {

// One forward ring step: queries [len][hq][D] against one K/V block [len][hkv][D].
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  float* out;   // [len][hq][D] running output (overwritten when first != 0)
  float* lse;   // [hq][len] running log-sum-exp (natural log)
  int len;      // query rows
  int klen;     // keys (K/V rows); equal to len whenever diag is set
  int hq, hkv;
  int group;    // hq / hkv
  int hpw;      // query heads sharing one workgroup (divides group and the wave count)
  int hsub;     // group / hpw
  int diag;     // causal diagonal block: key j visible to query i iff j <= i
  int first;    // first round of the ring: write instead of merge
  float scale_log2;  // log2(e) / sqrt(D)
  int ls;       // elements between heads in lse (len, or more when rows are a slice of a longer block)
};

// Up to two independent sub-problems share one launch along gridDim.y (the
// zig-zag layout's two query chunks for the forward and dQ, or two key chunks
// for dK/dV); the bf16 path has a pair variant of each kernel, in which every
// workgroup runs the sub-problem of its blockIdx.y.
template <typename A> struct ArgPair { A s[2]; };

hipError_t launch_fwd_step(const FwdArgs* a, int nsub, int elem_bytes, int head_dim, hipStream_t st);
// waves per forward workgroup for an element size (the host packs heads by it)
int fwd_waves_per_block(int elem_bytes);

// Backward: Delta = rowsum(dout * out) per (head, row); for bf16 inputs also
// the half (IEEE fp16) copies of q and dout that the bf16 backward contracts.
struct BwdPreArgs {
  const void* dout;  // [len][hq][D] bf16 or fp32
  const float* out;  // [len][hq][D]
  const float* lse;  // [hq][len]
  float* delta;      // [hq][len]  Delta = rowsum(dout * out)
  float* lse2;       // [hq][len]  lse * log2(e)
  int len, hq;
  int ls;            // elements between heads in lse / delta / lse2
  const void* q;     // bf16 only: [len][hq][D] bf16
  void* q16;         // bf16 only: [len][hq][D] half copy of q
  void* do16;        // bf16 only: [len][hq][D] half copy of dout
};
hipError_t launch_bwd_pre(const BwdPreArgs& a, int elem_bytes, int head_dim, hipStream_t st);

// Backward ring step against one K/V block.  bf16 path: q and dout are the
// half copies; the dK/dV kernel reads k/v as bf16 and writes their half copies
// to k16/v16, which the dQ kernel then reads as its k/v.
struct BwdArgs {
  const void* q;     // [len][hq][D]
  const void* k;     // [klen][hkv][D]
  const void* v;
  const void* dout;  // [len][hq][D]
  void* k16;         // bf16 dK/dV kernel: [klen][hkv][D] half copy of k (written)
  void* v16;         // bf16 dK/dV kernel: [klen][hkv][D] half copy of v (written)
  const float* lse;  // [hq][len]
  const float* delta;  // [hq][len]
  const float* lse2;   // [hq][len] lse * log2(e)
  float* dq;         // [len][hq][D]   (overwrite when first != 0, else accumulate)
  float* dk;         // [klen][hkv][D] (accumulate)
  float* dv;         // [klen][hkv][D] (accumulate)
  int len;           // query rows
  int klen;          // keys; equal to len whenever diag is set
  int hq, hkv, group;
  int hpw, hsub;     // dQ kernel: query heads per workgroup (as FwdArgs)
  int diag;
  int first;
  float scale;       // 1/sqrt(D)
  float scale_log2;  // log2(e)/sqrt(D)
  int ls;            // elements between heads in lse / delta / lse2
};
hipError_t launch_bwd_dkdv(const BwdArgs* a, int nsub, int elem_bytes, int head_dim, hipStream_t st);
hipError_t launch_bwd_dq(const BwdArgs* a, int nsub, int elem_bytes, int head_dim, hipStream_t st);
int bwd_dq_waves_per_block();
// bf16 fast paths (LDS-DMA staging, transposed operand reads)
hipError_t launch_bwd_dkdv_bf16(const BwdArgs* a, int nsub, int head_dim, hipStream_t st);
hipError_t launch_bwd_dq_bf16(const BwdArgs* a, int nsub, int head_dim, hipStream_t st);
int bwd_bf16_waves_per_block();

// Pairwise merge of two normalised partials.
struct MergeArgs {
  const float* out_a;
  const float* lse_a;
  const float* out_b;
  const float* lse_b;
  float* out;
  float* lse;
  int rows, heads, head_dim;
};
hipError_t launch_merge(const MergeArgs& a, hipStream_t st);

// Decode: q_len query rows against every K/V block, split over key chunks
// (one wave each), then merged.  Partials: [hkv][n_parts][group*q_len][D]
// and [hkv][n_parts][group*q_len], n_parts = n_blocks * n_chunks.
constexpr int kDecodeMaxBlocks = 64;
struct DecodeArgs {
  const void* q;                        // [q_len][hq][D] bf16
  const void* kblk[kDecodeMaxBlocks];   // block j: [len][hkv][D] bf16
  const void* vblk[kDecodeMaxBlocks];
  float* out;                           // [q_len][hq][D]
  float* lse;                           // [hq][ls] (this call's rows 0..q_len-1 of each head's row)
  float* part_o;
  float* part_lse;
  long long q_pos0;                     // global position of query row 0
  int n_blocks, len, q_len, hq, hkv, group;
  int chunk, n_chunks, n_parts;         // keys per wave, chunks per block, partials per row
  float scale_log2;
  int ls = 0;                           // elements between heads in lse (0: q_len)
};
hipError_t launch_decode_partial(const DecodeArgs& a, int head_dim, hipStream_t st);

// C[m][n] = sum_k A[m][k] B[n][k] (+ bias[n]); bf16 A and B (k contiguous), fp32 accumulation.
// gelu_bf16_out: C = bf16(GELU(.)) else C = fp32.  n % 128 == 0, k % 64 == 0.
struct GemmArgs {
  const void* a;      // [m][lda] bf16
  const void* b;      // [n][ldb] bf16
  void* c;            // [m][ldc] bf16 or fp32
  const float* bias;  // [n] or nullptr
  int m, n, k, lda, ldb, ldc;
  int group = 0;      // row tiles per band of the workgroup order (set by launch_gemm_bt)
};
hipError_t launch_gemm_bt(const GemmArgs& a, bool gelu_bf16_out, hipStream_t st);
int gemm_tile_n();
int gemm_tile_k();
hipError_t launch_decode_merge(const DecodeArgs& a, int head_dim, hipStream_t st);
// Device address and size of the fixed decode scratch on the current device (the
// partials of the no-allocation entry point); looked up once per device.
hipError_t decode_scratch(float** ptr, size_t* bytes);

// Pipeline diagnostics: NaN-fill two staging buffers; spin for a bounded number of cycles.
hipError_t launch_fill_nan(void* a, void* b, size_t bytes, hipStream_t st);
hipError_t launch_spin(long long cycles, hipStream_t st);
// `blocks` workgroups of 8 waves; sink receives one float per workgroup
hipError_t launch_mfma_rate(int iters, float* sink, int blocks, hipStream_t st);

}  // namespace ra
