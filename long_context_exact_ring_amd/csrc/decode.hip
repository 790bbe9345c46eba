// Long-context decode: a few new query rows against every K/V block of the
// ring ("Ring Attention with Blockwise Transformers for Near-Infinite
// Context", §3.1 blockwise attention and the log-sum-exp combination of
// per-block statistics; the method serves inference as well as training).
//
// In decode the query block is tiny (q_len tokens) and the K/V blocks are the
// long context, so the roles of the ring flip: each host keeps its K/V block
// and only the few query rows (and their partial results) travel.  The work
// is therefore HBM-bound: every K/V byte is read once for q_len x group rows
// of dot products.
//
// Kernel 1 (decode_partial_kernel): one wavefront per (K/V block, K/V head,
// key chunk).  The wave streams its chunk through a private double-buffered
// LDS region (LDS DMA, no barriers: a wave only reads what it copied) and
// keeps the rows of its K/V head's query group -- group * q_len <= 32 rows in
// one launch (the host runs a longer query block as several such passes), one
// per lane of the 32x32 MFMA accumulator -- with the same transposed
// score / online-softmax / P-fed-back layout as the forward step.  It writes
// a normalised partial (o, lse) per row.
// Kernel 2 (decode_merge_kernel): one workgroup per (K/V head, row) folds the
// partials of all chunks and blocks with the log-sum-exp merge.
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/ring_attn.h"
#include "kcommon.h"
#include "kernels.h"

namespace ra {

namespace {

constexpr float kDecRescale = 8.0f;  // lazy-rescale threshold, log2 units

#ifndef RA_DEC_NB
#define RA_DEC_NB 2  // LDS stages per wave (K+V tiles of 32 keys); more stages cost occupancy
#endif

template <int D>
__device__ __forceinline__ void dec_dma_tile(const bf16_storage* base, size_t stride, int t0, int len,
                                             unsigned char* tile, int lane) {
  // 32 rows of one head, [32][D] bf16, swizzled like the forward tiles; rows
  // past the end re-read the last row (masked by position below)
  constexpr int ROWB = D * 2, RPI = 1024 / ROWB, CPR = ROWB / 16, NI = 32 / RPI;
#pragma unroll
  for (int q = 0; q < NI; ++q) {
    const int r = q * RPI + lane / CPR, slot = lane % CPR;
    const int row = min(t0 + r, len - 1);
    lds_dma16(base + (size_t)row * stride + ((slot ^ swz<D>(r)) * 8),
              __builtin_amdgcn_readfirstlane(lds_addr(tile + q * 1024)));
  }
}

}  // namespace

template <int N>
__device__ __forceinline__ void dec_wait_vmcnt() {  // all but the newest N vector-memory operations done
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int D, int NB>
__global__ __launch_bounds__(64) void decode_partial_kernel(DecodeArgs a) {
  constexpr int ROWB = D * 2, TILEB = 32 * ROWB, STAGE = 2 * TILEB;
  constexpr int DPT = 2 * (TILEB / 1024);  // LDS DMA instructions per K/V tile
  __shared__ __attribute__((aligned(1024))) unsigned char smem[NB * STAGE];
  const int lane = threadIdx.x, n = lane & 31, hf = lane >> 5;

  // block id -> (chunk, K/V head, K/V block)
  int id = blockIdx.x;
  const int c = id % a.n_chunks;
  id /= a.n_chunks;
  const int g = id % a.hkv;
  const int j = id / a.hkv;
  const int k0 = c * a.chunk, k1 = min(k0 + a.chunk, a.len);
  const int ntiles = (k1 - k0 + 31) / 32;

  // this lane's query row r = hh * q_len + i (head g * group + hh, query i)
  const int rows = a.group * a.q_len;
  const int r = min(n, rows - 1);
  const int hh = r / a.q_len, qi = r % a.q_len;
  const int head = g * a.group + hh;
  const long long qpos = a.q_pos0 + qi;
  const long long kpos0 = (long long)j * a.len;  // global position of this block's first key
  const size_t qstride = (size_t)a.hq * D, kvstride = (size_t)a.hkv * D;

  Frag<bf16_storage> qf[D / 16];
  {
    const bf16_storage* qp =
        reinterpret_cast<const bf16_storage*>(a.q) + (size_t)qi * qstride + (size_t)head * D + hf * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = frag_load<bf16_storage>(qp + ks * 16);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q settled before the tile stream

  const bf16_storage* kbase = reinterpret_cast<const bf16_storage*>(a.kblk[j]) + (size_t)g * D;
  const bf16_storage* vbase = reinterpret_cast<const bf16_storage*>(a.vblk[j]) + (size_t)g * D;
  auto issue = [&](int t, unsigned char* st) {
    dec_dma_tile<D>(kbase, kvstride, k0 + t * 32, a.len, st, lane);
    dec_dma_tile<D>(vbase, kvstride, k0 + t * 32, a.len, st + TILEB, lane);
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x16_t o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16_t{};

  // NB-stage ring: tiles t+1 .. t+NB-2 stay in flight while tile t is used;
  // tiles past the end are clamped re-reads of the last one (never used)
  for (int u = 0; u < NB - 1; ++u) issue(min(u, max(ntiles - 1, 0)), smem + u * STAGE);
  int sc = 0;  // stage of tile t
  for (int t = 0; t < ntiles; ++t) {
    dec_wait_vmcnt<(NB - 2) * DPT>();  // tile t (this wave's own copy) has landed
    const int sn = sc == 0 ? NB - 1 : sc - 1;  // stage of tile t + NB - 1 (= that of tile t - 1)
    issue(min(t + NB - 1, ntiles - 1), smem + sn * STAGE);
    const unsigned char* kt = smem + sc * STAGE;
    const unsigned char* vt = kt + TILEB;
    f32x16_t s = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) mma(s, row_frag<D>(kt, n, ks, hf), qf[ks]);
    // visible: local key index < k1 (inside the chunk and the block) and key position <= query position
    const int t0 = k0 + t * 32;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kl = t0 + crow(i, hf);
      if (kl >= k1 || kpos0 + kl > qpos) s[i] = kNegInf;
    }
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[i], s[i + 1]));
    const float mxh = mx * a.scale_log2;
    if (__builtin_amdgcn_ballot_w64(mxh > m_run + kDecRescale) != 0) {
      const float m_new = fmaxf(m_run, fmaxf(mxh, swap_halves(mxh)));
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    Frag<bf16_storage> pf[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = fast_exp2(__builtin_fmaf(s[kc * 8 + e], a.scale_log2, -m_use));
        l_run += p[e];
      }
      pf[kc] = frag_from_f32<bf16_storage>(p);
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) mma(o[dt], tr_frag<D>(vt, dt * 32, kc, lane), pf[kc]);
    sc = sc + 1 == NB ? 0 : sc + 1;
  }
  dec_wait_vmcnt<0>();  // no copy into LDS may outlive the wave

  // normalised partial of this (block, head, chunk): o / l and lse = ln(l) + m ln 2
  const float l_tot = l_run + swap_halves(l_run);
  if (n >= rows) return;
  const int p = j * a.n_chunks + c;
  const size_t prow = ((size_t)g * a.n_parts + p) * rows + n;
  float* po = a.part_o + prow * D;
  const float w = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float4 v = make_float4(o[dt][4 * q4] * w, o[dt][4 * q4 + 1] * w, o[dt][4 * q4 + 2] * w, o[dt][4 * q4 + 3] * w);
      *reinterpret_cast<float4*>(po + dt * 32 + q4 * 8 + hf * 4) = v;
    }
  if (hf == 0) a.part_lse[prow] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : kNegInf;
}

// One workgroup of 4 waves per (K/V head, row): lse = log sum_p e^(lse_p) and
// out = sum_p e^(lse_p - lse) o_p over the n_parts partials.  The partials of
// a row are spread over the 256 threads for the two scalar reductions, and
// over the 4 waves (lanes along head_dim) for the weighted sum, so the loads
// of many partials are in flight at once.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  __shared__ float red[4][D];
  __shared__ float part[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rows = a.group * a.q_len;
  const int g = blockIdx.x / rows, r = blockIdx.x % rows;
  const int hh = r / a.q_len, qi = r % a.q_len;
  const int head = g * a.group + hh;
  const float* pl = a.part_lse + (size_t)g * a.n_parts * rows + r;
  float* orow = a.out + ((size_t)qi * a.hq + head) * D;

  float mx = kNegInf;
  for (int p = tid; p < a.n_parts; p += 256) mx = fmaxf(mx, pl[(size_t)p * rows]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if (lane == 0) part[w] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
  __syncthreads();
  if (mx == kNegInf) {  // no visible key for this row (uniform over the workgroup)
    for (int d = tid; d < D; d += 256) orow[d] = 0.f;
    if (tid == 0) a.lse[(size_t)head * (a.ls ? a.ls : a.q_len) + qi] = kNegInf;
    return;
  }
  float z = 0.f;
  for (int p = tid; p < a.n_parts; p += 256) z += expf(pl[(size_t)p * rows] - mx);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off, 64);
  if (lane == 0) part[w] = z;
  __syncthreads();
  const float lse = mx + logf(part[0] + part[1] + part[2] + part[3]);

  float acc[D / 64];
#pragma unroll
  for (int u = 0; u < D / 64; ++u) acc[u] = 0.f;
  const size_t pstride = (size_t)rows * D;  // floats between consecutive partials of a row
  const float* po = a.part_o + ((size_t)g * a.n_parts * rows + r) * D + lane;
#pragma unroll 4
  for (int p = w; p < a.n_parts; p += 4) {
    const float lp = pl[(size_t)p * rows];
    const float wgt = lp == kNegInf ? 0.f : expf(lp - lse);  // empty partials hold o = 0
#pragma unroll
    for (int u = 0; u < D / 64; ++u) acc[u] += wgt * po[p * pstride + 64 * u];
  }
#pragma unroll
  for (int u = 0; u < D / 64; ++u) red[w][lane + 64 * u] = acc[u];
  __syncthreads();
  for (int d = tid; d < D; d += 256) orow[d] = red[0][d] + red[1][d] + red[2][d] + red[3][d];
  if (tid == 0) a.lse[(size_t)head * (a.ls ? a.ls : a.q_len) + qi] = lse;
}

static bool decode_args_ok(const DecodeArgs& a) {
  return a.group * a.q_len <= 32 && a.n_blocks <= kDecodeMaxBlocks && a.n_parts == a.n_blocks * a.n_chunks;
}

hipError_t launch_decode_partial(const DecodeArgs& a, int head_dim, hipStream_t st) {
  if (!decode_args_ok(a)) return hipErrorInvalidValue;
  const long nwaves = (long)a.n_blocks * a.hkv * a.n_chunks;
  if (nwaves == 0) return hipSuccess;
  if (head_dim == 64)
    hipLaunchKernelGGL((decode_partial_kernel<64, RA_DEC_NB>), dim3((unsigned)nwaves), dim3(64), 0, st, a);
  else if (head_dim == 128)
    hipLaunchKernelGGL((decode_partial_kernel<128, RA_DEC_NB>), dim3((unsigned)nwaves), dim3(64), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeArgs& a, int head_dim, hipStream_t st) {
  if (!decode_args_ok(a)) return hipErrorInvalidValue;
  const unsigned nrows = (unsigned)(a.hkv * a.group * a.q_len);
  if (head_dim == 64)
    hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(nrows), dim3(256), 0, st, a);
  else if (head_dim == 128)
    hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(nrows), dim3(256), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ------------------------------------------------------------------ fixed scratch
// The partials of the entry point that allocates nothing live in this
// file-scope device array: one copy per GPU, held until the process ends,
// shared by every such call on that GPU.  In host code the name `scratch` is
// only a stand-in for the symbol (passing it to a kernel would hand the GPU a
// host address); its device address comes from hipGetSymbolAddress, looked up
// once per device with that device current, and only that address is used.
constexpr size_t kDecodeScratchBytes = RA_DECODE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

hipError_t decode_scratch(float** ptr, size_t* bytes) {
  static std::mutex mu;
  static std::vector<std::pair<int, float*>> addr;  // (device, address of its copy)
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  for (const auto& da : addr)
    if (da.first == dev) {
      *ptr = da.second;
      *bytes = kDecodeScratchBytes;
      return hipSuccess;
    }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  addr.emplace_back(dev, static_cast<float*>(p));
  *ptr = static_cast<float*>(p);
  *bytes = kDecodeScratchBytes;
  return hipSuccess;
}

}  // namespace ra
