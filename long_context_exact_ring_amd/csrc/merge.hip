// Elementwise kernels: pairwise partial merge and the backward preprocess.
//
// Merge (close-reading notes on "Ring Attention with Blockwise Transformers for
// Near-Infinite Context", §3.1: per-block statistics are combined by
// rescaling): a normalised partial is (o, lse) over a key subset; two partials
// over disjoint subsets combine as lse = log(e^lse_a + e^lse_b) and
// o = e^(lse_a - lse) o_a + e^(lse_b - lse) o_b.  HBM-bound, VALU only.
//
// Backward preprocess: Delta_i = sum_d dout_i * out_i for every (head, row),
// the row term of dS = P * (dP - Delta), and lse in log2 units (the exponent
// offset the backward kernels use); for bf16 inputs also the half copies of q
// and dout that the bf16 backward kernels contract.  One wavefront per (row, head).
#include "kcommon.h"
#include "kernels.h"

namespace ra {

__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  // A group of 16 lanes of one wavefront owns a (row, head) pair: every lane
  // reads that pair's lse values before any lane of the wave writes the merged
  // one, which keeps the in-place form (lse aliasing lse_a or lse_b) safe.
  const long groups = (long)a.rows * a.heads;
  const int sub = threadIdx.x & 15;
  for (long rh = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 4; rh < groups;
       rh += ((long)gridDim.x * blockDim.x) >> 4) {
    const int h = (int)(rh % a.heads);
    const int r = (int)(rh / a.heads);
    const float la = a.lse_a[(long)h * a.rows + r];
    const float lb = a.lse_b[(long)h * a.rows + r];
    const float mx = fmaxf(la, lb);
    float wa = 0.f, wb = 0.f, l = kNegInf;
    if (mx != kNegInf) {
      const float ea = expf(la - mx), eb = expf(lb - mx);
      const float z = ea + eb;
      l = mx + logf(z);
      wa = ea / z;
      wb = eb / z;
    }
    const long base = rh * a.head_dim;
    for (int c = sub; c < a.head_dim; c += 16) {
      // an empty partial contributes nothing, even if its out holds garbage
      const float xa = (wa != 0.f) ? wa * a.out_a[base + c] : 0.f;
      const float xb = (wb != 0.f) ? wb * a.out_b[base + c] : 0.f;
      a.out[base + c] = xa + xb;
    }
    if (sub == 0) a.lse[(long)h * a.rows + r] = l;
  }
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t st) {
  const long total = (long)a.rows * a.heads * 16;
  if (total == 0) return hipSuccess;
  long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------- Delta = rowsum(dO * O)
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdPreArgs a) {
  // one wave per (row, head); each lane covers D/64 consecutive columns
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  const long rh = wave;
  if (rh >= (long)a.len * a.hq) return;
  const int h = (int)(rh % a.hq);
  const int r = (int)(rh / a.hq);
  constexpr int PER = D / 64;
  const T* dp = reinterpret_cast<const T*>(a.dout) + rh * D + lane * PER;
  const float* op = a.out + rh * D + lane * PER;
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    float dv;
    if constexpr (sizeof(T) == 2) {
      dv = __uint_as_float((uint32_t)dp[j] << 16);
    } else {
      dv = dp[j];
    }
    acc = __builtin_fmaf(dv, op[j], acc);
  }
  if constexpr (sizeof(T) == 2) {  // half copies of q and dout (exact for |x| in [2^-14, 65504])
    static_assert(PER == 1 || PER == 2, "one 32-bit word per lane and tensor");
    const T* qp = reinterpret_cast<const T*>(a.q) + rh * D + lane * PER;
    T* q16 = reinterpret_cast<T*>(a.q16) + rh * D + lane * PER;
    T* d16 = reinterpret_cast<T*>(a.do16) + rh * D + lane * PER;
    if constexpr (PER == 2) {
      const uint32_t qw = *reinterpret_cast<const uint32_t*>(qp);
      const uint32_t dw = *reinterpret_cast<const uint32_t*>(dp);
      *reinterpret_cast<uint32_t*>(q16) = bf16x2_to_f16x2(qw);
      *reinterpret_cast<uint32_t*>(d16) = bf16x2_to_f16x2(dw);
    } else {
      q16[0] = (T)bf16x2_to_f16x2((uint32_t)qp[0]);
      d16[0] = (T)bf16x2_to_f16x2((uint32_t)dp[0]);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) {
    a.delta[(long)h * a.ls + r] = acc;
    a.lse2[(long)h * a.ls + r] = a.lse[(long)h * a.ls + r] * kLog2e;
  }
}

hipError_t launch_bwd_pre(const BwdPreArgs& a, int elem_bytes, int head_dim, hipStream_t st) {
  const long waves = (long)a.len * a.hq;
  if (waves == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((waves + 3) / 4);
  if (elem_bytes == 2) {
    if (head_dim == 64) hipLaunchKernelGGL((bwd_pre_kernel<bf16_storage, 64>), dim3(blocks), dim3(256), 0, st, a);
    else if (head_dim == 128) hipLaunchKernelGGL((bwd_pre_kernel<bf16_storage, 128>), dim3(blocks), dim3(256), 0, st, a);
    else return hipErrorInvalidValue;
  } else {
    if (head_dim == 64) hipLaunchKernelGGL((bwd_pre_kernel<float, 64>), dim3(blocks), dim3(256), 0, st, a);
    else if (head_dim == 128) hipLaunchKernelGGL((bwd_pre_kernel<float, 128>), dim3(blocks), dim3(256), 0, st, a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------- pipeline diagnostics
__global__ __launch_bounds__(256) void fill_nan_kernel(uint32_t* a, uint32_t* b, size_t words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (size_t)gridDim.x * blockDim.x) {
    a[i] = 0xffffffffu;  // NaN as bf16 pairs and as fp32
    b[i] = 0xffffffffu;
  }
}

hipError_t launch_fill_nan(void* a, void* b, size_t bytes, hipStream_t st) {
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  size_t blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_nan_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (uint32_t*)a, (uint32_t*)b,
                     words);
  return hipGetLastError();
}

__global__ void spin_kernel(long long cycles) {
  // bounded busy wait on the shader clock: always terminates after `cycles`
  const long long t0 = clock64();
  while (clock64() - t0 < cycles) {
  }
}

hipError_t launch_spin(long long cycles, hipStream_t st) {
  hipLaunchKernelGGL(spin_kernel, dim3(1), dim3(1), 0, st, cycles);
  return hipGetLastError();
}

}  // namespace ra
