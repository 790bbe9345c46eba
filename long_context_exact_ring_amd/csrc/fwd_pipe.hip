// bf16 forward ring-step kernel, software-pipelined over two row groups per
// wave ("Ring Attention with Blockwise Transformers for Near-Infinite
// Context", §3.1 blockwise attention with online softmax; same mathematics as
// fwd_bf16_kernel in fwd_step.hip).
//
// Why a second schedule: with 32 query rows per wave every 32x32x16 MFMA needs
// one 1 KB operand read from LDS, which is the whole LDS bandwidth of a CU
// when all four matrix cores are busy, and the softmax VALU work of a tile is
// nearly as long as its MFMA work.  Here a wave owns 64 rows (two groups of
// 32, g0 and g1) and keeps every K and V fragment it reads in registers long
// enough to feed both groups, which halves the LDS bytes per MFMA.  One wave
// per SIMD (512 registers) holds the two accumulators, the two Q blocks and
// two generations of K/V fragments.  With no second wave on the SIMD to hide
// the softmax, the wave overlaps it with its own MFMAs: group g1 runs half a
// tile behind g0, so that each half-iteration issues 16 MFMAs that do not
// depend on the softmax it computes in between:
//
//   A(t): read V(t)          MFMA  O_g1 += V(t-1)^T P_g1(t-1), S_g1(t) = K(t) Q_g1^T
//                            VALU  softmax of S_g0(t) -> P_g0(t)
//   B(t): barrier, K(t+1)    MFMA  O_g0 += V(t)^T P_g0(t), S_g0(t+1) = K(t+1) Q_g0^T
//                            VALU  softmax of S_g1(t) -> P_g1(t)
//
// K(t) feeds S_g0(t) at the end of B(t-1) and S_g1(t) in A(t); V(t) feeds
// PV_g0(t) in B(t) and PV_g1(t) in A(t+1).  K/V tiles of 32 keys rotate
// through four LDS stages; the LDS DMA for tile t+3 is issued in B(t), after
// the barrier that retires tile t-1.  Tile indices past the end are clamped
// (the copies land in stages nobody reads), which keeps the loop free of
// branches on the tile count.
#include <type_traits>

#include "fwd_common.h"
#include "kcommon.h"
#include "kernels.h"

namespace ra {

namespace {

#ifndef RA_PIPE_IL
#define RA_PIPE_IL 4  // VALU instructions scheduled after each MFMA (0: compiler's choice)
#endif

#ifndef RA_PIPE_FENCE_ON
#define RA_PIPE_FENCE_ON 0
#endif
// keeps the V(t) reads behind the MFMAs that still read V(t-1) from the same registers
#define RA_PIPE_FENCE()                                       \
  do {                                                        \
    if constexpr (RA_PIPE_FENCE_ON) __builtin_amdgcn_sched_barrier(0); \
  } while (0)

constexpr float kPipeRescale = 8.0f;  // log2 units, as in the other bf16 forward

using BF = Frag<bf16_storage>;

// Operand reads from a K or V tile at `base`; the per-lane byte offsets of
// every read are computed once (they only depend on the lane), so a read is a
// single ds_read with the stage base folded into its immediate offset.
template <int D>
__device__ __forceinline__ void pipe_kfrags(const unsigned char* base, const uint32_t (&koff)[D / 16],
                                            BF (&kf)[D / 16]) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) kf[ks] = BF{*reinterpret_cast<const uint4*>(base + koff[ks])};
}

template <int D>
__device__ __forceinline__ void pipe_vfrags(const unsigned char* base, const uint32_t (&voff)[D / 32][2][2],
                                            BF (&vf)[D / 32][2]) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const uint2 lo = ds_read_tr16(base + voff[dt][kc][0]);
      const uint2 hi = ds_read_tr16(base + voff[dt][kc][1]);
      vf[dt][kc] = BF{make_uint4(lo.x, lo.y, hi.x, hi.y)};
    }
}

template <int D>
__device__ __forceinline__ void pipe_scores(f32x16_t& s, const BF (&kf)[D / 16], const BF (&qf)[D / 16]) {
  s = f32x16_t{};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) mma(s, kf[ks], qf[ks]);
}

template <int D>
__device__ __forceinline__ void pipe_pv(f32x16_t (&o)[D / 32], const BF (&vf)[D / 32][2], const BF (&pf)[2]) {
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) mma(o[dt], vf[dt][kc], pf[kc]);
}

// Masking and the running-max update of one group's 32x32 score tile (keys on
// accumulator rows, one query per lane).  Each half of the wave compares its
// own 16 keys with the shared reference; the halves exchange maxima only when
// some row has to move it (rare), then O and l are rescaled.
template <int D, bool MASKED>
__device__ __forceinline__ void pipe_max(f32x16_t& s, f32x16_t (&o)[D / 32], float& m_run, float& l_run,
                                         float scale_log2, int lim, int hf) {
  if constexpr (MASKED) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (crow(i, hf) > lim) s[i] = kNegInf;
  }
  float mx = kNegInf;
#pragma unroll
  for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[i], s[i + 1]));
  const float mxh = mx * scale_log2;
  if (__builtin_amdgcn_ballot_w64(mxh > m_run + kPipeRescale) != 0) {
    const float m_new = fmaxf(m_run, fmaxf(mxh, swap_halves(mxh)));
    const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
    l_run *= alpha;
    // one 16-register accumulator at a time (they may live in AGPRs)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
      __builtin_amdgcn_sched_barrier(0);
    }
    m_run = m_new;
  }
}

// P^T = exp2(S^T * scale - m) as two bf16 B fragments; the row sum uses the
// fp32 values (the lse the backward reuses is not perturbed by bf16 rounding).
__device__ __forceinline__ void pipe_exp(const f32x16_t& s, float m_run, float& l_run, BF (&pf)[2],
                                         float scale_log2) {
  const float m_use = (m_run == kNegInf) ? 0.f : m_run;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = fast_exp2(__builtin_fmaf(s[kc * 8 + e], scale_log2, -m_use));
      l_run += p[e];
    }
    pf[kc] = frag_from_f32<bf16_storage>(p);
  }
}

// Pins a value to this point of the program: the compiler may not sink the
// instructions that produce it past here (it would otherwise move a
// half-iteration's softmax next to the MFMAs that consume it, leaving the
// other half-iteration without VALU work to overlap).
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void pipe_anchor(const BF (&pf)[2]) {
  asm volatile("" ::"v"(__builtin_bit_cast(u32x4_t, pf[0].v)), "v"(__builtin_bit_cast(u32x4_t, pf[1].v)));
}

// Scheduling patterns for the two MFMA/VALU regions of an iteration (one
// MFMA, then V VALU instructions; in A the V(t) fragment reads go between the
// MFMAs that still read V(t-1) and those that do not).
template <int V>
__device__ __forceinline__ void pipe_pattern_a() {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);  // VALU
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);  // DS reads
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
  }
}
template <int V>
__device__ __forceinline__ void pipe_pattern_b() {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
  }
}

}  // namespace

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1))) void fwd_pipe_kernel(FwdArgs a) {
  constexpr int BC = 32, NB = 4;
  constexpr int ROWB = D * 2, TILEB = BC * ROWB, STAGE = 2 * TILEB;
  constexpr int NI = BC * ROWB / 1024;  // 1 KB DMA instructions per tensor tile
  static_assert(NI % NW == 0, "tile DMA must split evenly over the waves");
  constexpr int DPT = 2 * (NI / NW);    // DMA instructions per wave per K/V tile
  static_assert(DPT == 2 || DPT == 4, "wait counts below");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[NB * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int n = lane & 31, hf = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int R = NW * 64 / a.hpw;  // query rows per head in this workgroup
  const int nrt = (a.len + R - 1) / R;
  int rt = logical % nrt;
  const int rest = logical / nrt;
  const int hs = rest % a.hsub;
  const int g = rest / a.hsub;
  if (a.diag) rt = nrt - 1 - rt;  // longest row tiles first
  const int wpr = NW / a.hpw;
  const int head = g * a.group + hs * a.hpw + wu / wpr;
  const int row0 = rt * R + (wu % wpr) * 64;
  const int qi[2] = {row0 + n, row0 + 32 + n};
  const int wg_first_row = rt * R;
  const int wg_last_row = min(rt * R + R, a.len) - 1;
  int T = (a.len + BC - 1) / BC;
  if (a.diag) T = min(T, wg_last_row / BC + 1);
  // tiles [0, nfull) need no mask for any row of the workgroup
  const int nfull = min(T, a.diag ? (wg_first_row + 1) / BC : a.len / BC);
  // visible local keys of each group's query (before subtracting the tile's first key)
  const int lim[2] = {a.diag ? min(qi[0], a.len - 1) : a.len - 1, a.diag ? min(qi[1], a.len - 1) : a.len - 1};

  const size_t qstride = (size_t)a.hq * D, kvstride = (size_t)a.hkv * D;
  const bf16_storage* kbase = reinterpret_cast<const bf16_storage*>(a.k) + (size_t)g * D;
  const bf16_storage* vbase = reinterpret_cast<const bf16_storage*>(a.v) + (size_t)g * D;

  BF qf[2][D / 16];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const bf16_storage* qp = reinterpret_cast<const bf16_storage*>(a.q) + (size_t)min(qi[r], a.len - 1) * qstride +
                             (size_t)head * D + hf * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[r][ks] = frag_load<bf16_storage>(qp + ks * 16);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no Q load left pending inside the loop

  // ---- per-lane constants: LDS operand offsets and global DMA offsets
  uint32_t koff[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) koff[ks] = n * ROWB + (((ks * 2 + hf) ^ swz<D>(n)) * 16);
  uint32_t voff[D / 32][2][2];  // the two transposed reads of tr_frag(dt * 32, kc)
  {
    const int gq = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int dcol = dt * 32 + (gq & 1) * 16 + 4 * (i16 & 3);
          const int r = kc * 16 + u * 8 + (gq >> 1) * 4 + (i16 >> 2);
          voff[dt][kc][u] = TILEB + r * ROWB + (((dcol >> 3) ^ swz<D>(r)) * 16) + (dcol & 7) * 2;
        }
  }
  constexpr int RPI = 1024 / ROWB, CPR = ROWB / 16, IPW = NI / NW;
  uint32_t goff[IPW];  // byte offset of this lane's 16-byte chunk from a tile's first row
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int r = (wu * IPW + j) * RPI + lane / CPR, slot = lane % CPR;
    goff[j] = (uint32_t)(r * kvstride + (slot ^ swz<D>(r)) * 8) * 2;
  }

  // K/V tile t (clamped to the last one) into stage t % NB.  Whole tiles take a
  // uniform base plus the fixed lane offsets; a ragged last tile re-reads its
  // last row for the rows past the end (they are masked).
  auto issue = [&](int t) {
    const int tc = min(t, T - 1);
    unsigned char* st = smem + (t % NB) * STAGE;
    if ((tc + 1) * BC <= a.len) {
      const size_t tb = (size_t)tc * BC * kvstride * 2;
      const unsigned char* kb = reinterpret_cast<const unsigned char*>(kbase) + tb;
      const unsigned char* vb = reinterpret_cast<const unsigned char*>(vbase) + tb;
#pragma unroll
      for (int j = 0; j < IPW; ++j) {
        const uint32_t q = (uint32_t)(wu * IPW + j) * 1024;
        lds_dma16_off(kb, goff[j], __builtin_amdgcn_readfirstlane(lds_addr(st + q)));
        lds_dma16_off(vb, goff[j], __builtin_amdgcn_readfirstlane(lds_addr(st + TILEB + q)));
      }
    } else {
      dma_rows<D, BC, NW>(kbase, kvstride, tc * BC, a.len, st, wu, lane);
      dma_rows<D, BC, NW>(vbase, kvstride, tc * BC, a.len, st + TILEB, wu, lane);
    }
  };

  f32x16_t o[2][D / 32];
  float m_run[2] = {kNegInf, kNegInf}, l_run[2] = {0.f, 0.f};
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[r][dt] = f32x16_t{};
  f32x16_t s0, s1;
  BF p0[2], p1[2];
  BF kf[D / 16];     // K(t) until S_g1(t) is issued, then K(t+1)
  BF vf[D / 32][2];  // V(t-1) until PV_g1(t-1) is issued, then V(t)
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) p1[kc] = frag_zero<bf16_storage>();
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) vf[dt][kc] = frag_zero<bf16_storage>();  // "V(-1)": PV_g1(-1) adds 0

  issue(0);
  issue(1);
  issue(2);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  pipe_kfrags<D>(smem, koff, kf);
  pipe_scores<D>(s0, kf, qf[0]);

  // Each fragment set is overwritten right after the MFMAs that last read it
  // are issued, so only one K and one V generation occupy registers.  SG is the
  // stage of tile t when known at compile time (the unrolled steady loop: the
  // stage bases become immediate offsets of the LDS reads), else -1.
  auto body = [&](int t, auto masked_tag, auto stage_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr int SG = decltype(stage_tag)::value;
    const int t0 = t * BC;
    const unsigned char* cur = smem + (SG >= 0 ? SG : (t % NB)) * STAGE;
    const unsigned char* nxt = smem + (SG >= 0 ? (SG + 1) % NB : ((t + 1) % NB)) * STAGE;
    // ---- A(t)
    pipe_max<D, MASKED>(s0, o[0], m_run[0], l_run[0], a.scale_log2, lim[0] - t0, hf);
    pipe_pv<D>(o[1], vf, p1);  // O_g1 += V(t-1)^T P_g1(t-1)
    RA_PIPE_FENCE();
    pipe_vfrags<D>(cur, voff, vf);
    pipe_scores<D>(s1, kf, qf[1]);
    pipe_exp(s0, m_run[0], l_run[0], p0, a.scale_log2);
    if constexpr (RA_PIPE_IL > 0) pipe_pattern_a<RA_PIPE_IL>();
    pipe_anchor(p0);
    // ---- B(t)
    if constexpr (DPT == 4)
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");  // tile t+1 (issued two barriers ago) has landed
    else
      asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    __syncthreads();  // ... for every wave; stage (t-1) % NB is no longer read
    issue(t + 3);
    pipe_kfrags<D>(nxt, koff, kf);
    pipe_max<D, MASKED>(s1, o[1], m_run[1], l_run[1], a.scale_log2, lim[1] - t0, hf);
    pipe_pv<D>(o[0], vf, p0);  // O_g0 += V(t)^T P_g0(t)
    pipe_scores<D>(s0, kf, qf[0]);  // S_g0(t+1)
    pipe_exp(s1, m_run[1], l_run[1], p1, a.scale_log2);
    if constexpr (RA_PIPE_IL > 0) pipe_pattern_b<RA_PIPE_IL>();
    pipe_anchor(p1);
  };

  using Open = std::false_type;
  using Masked = std::true_type;
  int t = 0;
  for (; t + 3 < nfull; t += 4) {  // t % NB == 0 here
    body(t, Open{}, std::integral_constant<int, 0>{});
    body(t + 1, Open{}, std::integral_constant<int, 1>{});
    body(t + 2, Open{}, std::integral_constant<int, 2>{});
    body(t + 3, Open{}, std::integral_constant<int, 3>{});
  }
  for (; t < nfull; ++t) body(t, Open{}, std::integral_constant<int, -1>{});
  for (; t < T; ++t) body(t, Masked{}, std::integral_constant<int, -1>{});
  pipe_pv<D>(o[1], vf, p1);  // drain: O_g1 += V(T-1)^T P_g1(T-1)
  // the clamped copies issued for tiles past the end are still in flight: no
  // copy into this workgroup's LDS may outlive it
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

#pragma unroll
  for (int r = 0; r < 2; ++r) fwd_epilogue<D>(a, o[r], m_run[r], l_run[r], head, qi[r], hf);
}

template <int D, int NW>
hipError_t launch_fwd_pipe_t(const FwdArgs& a, hipStream_t st) {
  if (a.hpw < 1 || a.hsub < 1 || NW % a.hpw != 0) return hipErrorInvalidValue;
  const int R = NW * 64 / a.hpw;
  const int nblk = ((a.len + R - 1) / R) * a.hsub * a.hkv;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_pipe_kernel<D, NW>), dim3(nblk), dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

constexpr int kPipeWaves = 4;

hipError_t launch_fwd_pipe_bf16(const FwdArgs& a, int head_dim, hipStream_t st) {
  if (head_dim == 64) return launch_fwd_pipe_t<64, kPipeWaves>(a, st);
  if (head_dim == 128) return launch_fwd_pipe_t<128, kPipeWaves>(a, st);
  return hipErrorInvalidValue;
}

int fwd_pipe_waves_per_block() { return kPipeWaves; }

}  // namespace ra
