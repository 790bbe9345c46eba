// Forward ring-step kernel for gfx950: one rank's query block against one K/V block.
//
// What it computes (close-reading notes on "Ring Attention with Blockwise
// Transformers for Near-Infinite Context", §2.1 and §3.1; "Ring Attention 与序列并行",
// "Ring Attention 核心机制"): blockwise attention of the local queries over the
// keys of one block with a running row max and row sum (online softmax), never
// writing the score matrix to HBM; the block's normalised partial is then folded
// into the running (out, lse) with the log-sum-exp rescaling that lets blocks
// arrive in any order.
//
// Design (MI355X-first):
//  * A workgroup of NW wavefronts shares one K/V head.  Each wave owns 32 query
//    rows of one query head; with grouped heads the waves of a workgroup take
//    different query heads of the same K/V head, so each K/V tile staged in LDS
//    serves NW*32 query rows.
//  * Scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16.
//    The accumulator then keeps one query per lane (16 keys per lane, the other
//    16 in lane l^32), so the row max needs at most one cross-half exchange and
//    the row sum none until the end.  Q lives in registers as the B operand.
//  * The exponentiated tile P^T is fed back unchanged as the B operand of
//    O^T += V^T P^T.  To make that legal the V operand takes its keys in the
//    order in which the accumulator holds them (the contraction over keys is
//    order-free): the fp32 path stages V^T in LDS with the keys of every
//    16-key chunk permuted (perm_pos); the bf16 path keeps V in its natural
//    layout and reads it transposed in that order.
//  * K/V tiles are double-buffered in LDS with one barrier per tile: the bf16
//    path copies the next tile global -> LDS by LDS DMA while the current one
//    is computed; the fp32 path stages it through registers.
//  * Causal (diagonal block): tiles wholly above a wave's rows are skipped, the
//    straddling tile is masked; heavy row tiles are dispatched first.
//  * Epilogue: normalise, then overwrite (first round) or merge into the running
//    (out, lse) in HBM.
#include "kcommon.h"
#include <type_traits>

#include "fwd_common.h"
#include "kernels.h"
#include "tile_stage.h"

namespace ra {

template <typename T, int D, int BC, int NW>
struct FwdCfg {
  static constexpr int NT = NW * 64;
  static constexpr int ES = sizeof(T);
  static constexpr int CH = 16 / ES;            // elements per 16-byte chunk
  static constexpr int KROW = D * ES + 16;      // bytes per K row in LDS (16-byte pad)
  static constexpr int VROW = BC * ES + 16;     // bytes per V^T row in LDS
  static constexpr int KBYTES = BC * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int LDS = 2 * STAGE;
  static_assert(BC % 32 == 0 && D % 32 == 0, "32x32 MFMA tiles");
};


#ifndef RA_FWD_WAVES
#define RA_FWD_WAVES 8
#endif
#ifndef RA_FWD_BC
#define RA_FWD_BC 64
#endif
#ifdef RA_FWD_WPE
#define RA_FWD_OCC __attribute__((amdgpu_waves_per_eu(RA_FWD_WPE)))
#else
#define RA_FWD_OCC
#endif

template <typename T, int D, int BC, int NW>
__global__ __launch_bounds__(NW * 64) RA_FWD_OCC void fwd_step_kernel(FwdArgs a) {
  using C = FwdCfg<T, D, BC, NW>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, hf = lane >> 5;

  // ------------------------------------------------ work decomposition
  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int R = NW * 32 / a.hpw;  // query rows per head in this workgroup
  const int nrt = (a.len + R - 1) / R;
  int rt = logical % nrt;
  const int rest = logical / nrt;
  const int hs = rest % a.hsub;
  const int g = rest / a.hsub;
  if (a.diag) rt = nrt - 1 - rt;  // longest row tiles first
  const int wpr = NW / a.hpw;
  const int head = g * a.group + hs * a.hpw + w / wpr;
  const int row0 = rt * R + (w % wpr) * 32;
  const int wg_last_row = min(rt * R + R, a.len) - 1;
  int ntiles = (a.klen + BC - 1) / BC;
  if (a.diag) ntiles = min(ntiles, wg_last_row / BC + 1);

  const size_t qstride = (size_t)a.hq * D;   // elements between query rows
  const size_t kvstride = (size_t)a.hkv * D; // elements between key rows
  const T* kbase = reinterpret_cast<const T*>(a.k) + (size_t)g * D;
  const T* vbase = reinterpret_cast<const T*>(a.v) + (size_t)g * D;

  // ------------------------------------------------ Q fragments (B operand)
  Frag<T> qf[D / 16];
  {
    const int qrow = row0 + n;
    const T* qp = reinterpret_cast<const T*>(a.q) + (size_t)qrow * qstride + (size_t)head * D + hf * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      qf[ks] = (qrow < a.len) ? frag_load<T>(qp + ks * 16) : frag_zero<T>();
  }

  // ------------------------------------------------ K/V staging (natural K, permuted V^T)
  using St = TileStager<T, BC, D, C::NT>;
  static_assert(St::NROW == C::KROW && St::TROW == C::VROW, "LDS pitches");
  St kst, vst;
  auto gload = [&](int t0) {
    kst.load(kbase, kvstride, t0, a.klen, tid);
    vst.load(vbase, kvstride, t0, a.klen, tid);
  };
  auto lstore = [&](int buf) {
    unsigned char* ks = smem + buf * C::STAGE;
    kst.store(ks, nullptr, tid);
    vst.store(nullptr, ks + C::KBYTES, tid);
  };

  // ------------------------------------------------ running state (one query per lane)
  float m_run = kNegInf;  // running max of scaled scores, log2 units
  float l_run = 0.f;      // this lane's share of the running row sum
  f32x16_t o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16_t{};

  gload(0);
  lstore(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int t0 = t * BC;
    if (t + 1 < ntiles) gload(t0 + BC);
    const unsigned char* ks = smem + (t & 1) * C::STAGE;
    const unsigned char* vs = ks + C::KBYTES;

    const bool active = !(a.diag && t0 > row0 + 31);
    if (active) {
      // S^T = K Q^T for BC keys (BC/32 accumulator tiles)
      f32x16_t s[BC / 32];
#pragma unroll
      for (int kt = 0; kt < BC / 32; ++kt) {
        s[kt] = f32x16_t{};
        const T* krow = reinterpret_cast<const T*>(ks + (kt * 32 + n) * C::KROW) + hf * 8;
#pragma unroll
        for (int ks_ = 0; ks_ < D / 16; ++ks_) mma(s[kt], frag_load<T>(krow + ks_ * 16), qf[ks_]);
      }
      // masking: diagonal block (key > query) and ragged tail (key >= klen)
      const int qi = row0 + n;
      if ((a.diag && t0 + BC - 1 > row0) || (t0 + BC > a.klen)) {
#pragma unroll
        for (int kt = 0; kt < BC / 32; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = t0 + kt * 32 + crow(i, hf);
            if (key >= a.klen || (a.diag && key > qi)) s[kt][i] = kNegInf;
          }
      }
      // online softmax (log2 domain)
      float mx = kNegInf;
#pragma unroll
      for (int kt = 0; kt < BC / 32; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
      mx = fmaxf(mx, swap_halves(mx));
      const float m_new = fmaxf(m_run, mx * a.scale_log2);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float rs = 0.f;
#pragma unroll
      for (int kt = 0; kt < BC / 32; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(__builtin_fmaf(s[kt][i], a.scale_log2, -m_use));
          s[kt][i] = p;
          rs += p;
        }
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;

      // O^T += V^T P^T
      Frag<T> pf[BC / 16];
#pragma unroll
      for (int kc = 0; kc < BC / 16; ++kc) {
        float tmp[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) tmp[e] = s[kc >> 1][(kc & 1) * 8 + e];
        pf[kc] = frag_from_f32<T>(tmp);
      }
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const T* vrow = reinterpret_cast<const T*>(vs + (dt * 32 + n) * C::VROW) + hf * 8;
#pragma unroll
        for (int kc = 0; kc < BC / 16; ++kc) mma(o[dt], frag_load<T>(vrow + kc * 16), pf[kc]);
      }
    }
    if (t + 1 < ntiles) lstore((t + 1) & 1);
    __syncthreads();
  }

  fwd_epilogue<D>(a, o, m_run, l_run, head, row0 + n, hf);
}


// ============================================================================
// bf16 path.  Same mathematics as fwd_step_kernel, arranged for the VALU
// budget of gfx950 (the softmax instructions, not the MFMAs, set the pace):
//  * K and V tiles are copied global -> LDS by the load unit itself
//    (global_load_lds_dwordx4: no staging registers, no VALU), 1 KB per wave
//    instruction, rows unpadded with an XOR swizzle of the 16-byte chunks so
//    that the MFMA operand reads are bank-conflict free.
//  * V stays in its natural [key][d] layout; the transposed A operand of
//    O^T += V^T P^T is read with ds_read_b64_tr_b16 (four keys of one column
//    per read), keys ordered to match the accumulator-fed P^T fragments.
//  * The hot path carries no masking; diagonal / ragged tiles take a separate
//    instantiation.
//  * Lazy rescaling: the running max used as exponent reference only moves
//    when a row's new max exceeds it by more than 2^8 (probabilities stay
//    below 256, far from fp32/bf16 range limits), so the O rescale is skipped
//    on almost every tile.  Results are exact either way: the reference max
//    cancels in the final normalisation.
// ============================================================================
constexpr float kRescaleThreshold = 8.0f;  // log2 units

template <int D, int BC, int NW, int RG, bool MASKED>
__device__ __forceinline__ void fwd_bf16_tile(const FwdArgs& a, const unsigned char* stage_lds,
                                              const LdsOperandOffsets<D>& lo,
                                              const Frag<bf16_storage> (&qf)[RG][D / 16],
                                              f32x16_t (&o)[RG][D / 32], float (&m_run)[RG], float (&l_run)[RG],
                                              int t0, int qi0, int n, int hf, int lane) {
  // S^T = K Q^T; every K fragment read from LDS feeds the RG row groups of this wave
  f32x16_t s[RG][BC / 32];
#pragma unroll
  for (int kt = 0; kt < BC / 32; ++kt) {
#pragma unroll
    for (int r = 0; r < RG; ++r) s[r][kt] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const Frag<bf16_storage> kf{*reinterpret_cast<const uint4*>(stage_lds + kt * 32 * (D * 2) + lo.k[ks])};
#pragma unroll
      for (int r = 0; r < RG; ++r) mma(s[r][kt], kf, qf[r][ks]);
    }
  }
  Frag<bf16_storage> pf[RG][BC / 16];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    if constexpr (MASKED) {
      // visible keys of this lane's query: local key index <= lim
      const int lim = (a.diag ? min(qi0 + 32 * r, a.klen - 1) : a.klen - 1) - t0;
#pragma unroll
      for (int kt = 0; kt < BC / 32; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kt * 32 + crow(i, hf) > lim) s[r][kt][i] = kNegInf;
    }
    // row max over this lane's 16*BC/32 keys
    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < BC / 32; ++kt)
#pragma unroll
      for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[r][kt][i], s[r][kt][i + 1]));
    // Each half of the wave checks its own 16 keys per row against the shared
    // reference; only when some row must move it (rare) are the halves'
    // maxima exchanged, so the common path has no cross-lane traffic.
    const float mxh = mx * a.scale_log2;
    if (__builtin_amdgcn_ballot_w64(mxh > m_run[r] + kRescaleThreshold) != 0) {
      const float m_new = fmaxf(m_run[r], fmaxf(mxh, swap_halves(mxh)));
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run[r] - m_new);
      l_run[r] *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[r][dt][i] *= alpha;
      m_run[r] = m_new;
    }
    const float m_use = (m_run[r] == kNegInf) ? 0.f : m_run[r];
    // P^T = exp2(S^T * scale - m) as bf16 fragments; the row sum is taken on the
    // fp32 values so that lse (reused by the backward) is not perturbed by the
    // bf16 rounding of P.
#pragma unroll
    for (int kc = 0; kc < BC / 16; ++kc) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = fast_exp2(__builtin_fmaf(s[r][kc >> 1][(kc & 1) * 8 + e], a.scale_log2, -m_use));
        l_run[r] += p[e];
      }
      pf[r][kc] = frag_from_f32<bf16_storage>(p);
    }
  }
  // O^T += V^T P^T; A fragment = 2 transposed reads of 4 keys x 16 columns, shared by the row groups
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int kc = 0; kc < BC / 16; ++kc) {
      const uint2 v0 = ds_read_tr16(stage_lds + kc * 16 * (D * 2) + lo.v[dt][0]);
      const uint2 v1 = ds_read_tr16(stage_lds + kc * 16 * (D * 2) + lo.v[dt][1]);
      const Frag<bf16_storage> vf{make_uint4(v0.x, v0.y, v1.x, v1.y)};
#pragma unroll
      for (int r = 0; r < RG; ++r) mma(o[r][dt], vf, pf[r][kc]);
    }
}

// The arguments of this workgroup's sub-problem: a single argument set, or the
// blockIdx.y entry of a pair (the kernel is instantiated for both; unlike the
// backward's body-plus-wrapper kernels, this form keeps the single-argument
// forward's code exactly as fast as a plain FwdArgs kernel -- measured).
__device__ __forceinline__ const FwdArgs& fwd_sub_args(const FwdArgs& a) { return a; }
__device__ __forceinline__ FwdArgs fwd_sub_args(const ArgPair<FwdArgs>& p) { return p.s[blockIdx.y]; }

template <int D, int BC, int NW, int RG, typename ARG>
__global__ __launch_bounds__(NW * 64) void fwd_bf16_kernel(ARG arg) {
  const FwdArgs a = fwd_sub_args(arg);  // ARG: FwdArgs, or a pair of them along gridDim.y
  constexpr int ROWB = D * 2;
  constexpr int TILEB = BC * ROWB;
  constexpr int STAGE = 2 * TILEB;
  constexpr int RPI = 1024 / ROWB;  // rows per 1 KB load instruction
  constexpr int CPR = ROWB / 16;    // 16-byte chunks per row
  constexpr int IPW = BC / RPI / NW;  // load instructions per wave per tensor
  static_assert(IPW >= 1 && (BC / RPI) % NW == 0, "tile rows must split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, hf = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);

  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int R = NW * 32 * RG / a.hpw;  // query rows per head in this workgroup
  const int nrt = (a.len + R - 1) / R;
  int rt = logical % nrt;
  const int rest = logical / nrt;
  const int hs = rest % a.hsub;
  const int g = rest / a.hsub;
  if (a.diag) rt = nrt - 1 - rt;
  const int wpr = NW / a.hpw;
  const int head = g * a.group + hs * a.hpw + wu / wpr;
  const int row0 = rt * R + (wu % wpr) * 32 * RG;  // this wave's first row (RG groups of 32)
  const int qi = row0 + n;
  const int wg_last_row = min(rt * R + R, a.len) - 1;
  int ntiles = (a.klen + BC - 1) / BC;
  if (a.diag) ntiles = min(ntiles, wg_last_row / BC + 1);

  const size_t qstride = (size_t)a.hq * D, kvstride = (size_t)a.hkv * D;
  const bf16_storage* kbase = reinterpret_cast<const bf16_storage*>(a.k) + (size_t)g * D;
  const bf16_storage* vbase = reinterpret_cast<const bf16_storage*>(a.v) + (size_t)g * D;

  Frag<bf16_storage> qf[RG][D / 16];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int qr = qi + 32 * r;
    const bf16_storage* qp =
        reinterpret_cast<const bf16_storage*>(a.q) + (size_t)min(qr, a.len - 1) * qstride + (size_t)head * D + hf * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[r][ks] = frag_load<bf16_storage>(qp + ks * 16);
  }
  // Settle the Q loads here (vmcnt(0), other counters untouched), so that no
  // wait for them is left inside the loop where it would also stall on the
  // tile prefetch in flight.
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // every lane fetches one 16-byte chunk per instruction: row q*RPI + lane/CPR,
  // LDS chunk slot lane%CPR, holding logical chunk slot ^ swizzle(row)
  const int lrow = lane / CPR, slot = lane % CPR;
  uint32_t koff[IPW];  // byte offsets of this lane's chunks from the tile's first row
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int r = (wu * IPW + j) * RPI + lrow;
    koff[j] = (uint32_t)(r * kvstride + (slot ^ swz<D>(r)) * 8) * 2;
  }
  const unsigned char* kbytes = reinterpret_cast<const unsigned char*>(kbase);
  const unsigned char* vbytes = reinterpret_cast<const unsigned char*>(vbase);
  auto issue = [&](int t0, unsigned char* kd) {  // kd: K tile, V tile follows
    unsigned char* vd = kd + TILEB;
    const size_t tb = (size_t)t0 * kvstride * 2;
    if (t0 + BC <= a.klen) {
#pragma unroll
      for (int j = 0; j < IPW; ++j) {
        const int q = wu * IPW + j;
        lds_dma16_off(kbytes + tb, koff[j], __builtin_amdgcn_readfirstlane(lds_addr(kd + q * 1024)));
        lds_dma16_off(vbytes + tb, koff[j], __builtin_amdgcn_readfirstlane(lds_addr(vd + q * 1024)));
      }
    } else {  // ragged tail: rows past the end re-read the last row (masked later)
#pragma unroll
      for (int j = 0; j < IPW; ++j) {
        const int q = wu * IPW + j;
        const int r = q * RPI + lrow;
        const int row = min(t0 + r, a.klen - 1);
        const bf16_storage* ks = kbase + (size_t)row * kvstride + ((slot ^ swz<D>(r)) * 8);
        const bf16_storage* vs = vbase + (size_t)row * kvstride + ((slot ^ swz<D>(r)) * 8);
        lds_dma16(ks, __builtin_amdgcn_readfirstlane(lds_addr(kd + q * 1024)));
        lds_dma16(vs, __builtin_amdgcn_readfirstlane(lds_addr(vd + q * 1024)));
      }
    }
  };

  float m_run[RG], l_run[RG];
  f32x16_t o[RG][D / 32];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    m_run[r] = kNegInf;
    l_run[r] = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[r][dt] = f32x16_t{};
  }

  // tiles [0, nfull) need no mask for any wave of this workgroup; the rest
  // (diagonal band, ragged tail) take the masked instantiation
  const int wg_first_row = rt * R;
  const int nfull = min(ntiles, a.diag ? (wg_first_row + 1) / BC : a.klen / BC);
  const LdsOperandOffsets<D> lo(lane, TILEB);
  // one unmasked tile; ST is its stage when known at compile time (then every
  // LDS read address is an offset register plus an immediate), else -1
  auto open_step = [&](int t, auto stage_tag) {
    constexpr int ST = decltype(stage_tag)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's part of tile t has landed
    __syncthreads();                                     // ... and everyone's; the other buffer is free
    const int sc = ST >= 0 ? ST : (t & 1);
    if (t + 1 < ntiles) issue((t + 1) * BC, smem + (ST >= 0 ? 1 - ST : 1 - sc) * STAGE);
    fwd_bf16_tile<D, BC, NW, RG, false>(a, smem + sc * STAGE, lo, qf, o, m_run, l_run, t * BC, qi, n, hf, lane);
  };
  issue(0, smem);
  int t = 0;
  for (; t + 1 < nfull; t += 2) {
    open_step(t, std::integral_constant<int, 0>{});
    open_step(t + 1, std::integral_constant<int, 1>{});
  }
  if (t < nfull) {
    open_step(t, std::integral_constant<int, 0>{});
    ++t;
  }
  for (; t < ntiles; ++t) {
    const int t0 = t * BC;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t + 1 < ntiles) issue(t0 + BC, smem + ((t + 1) & 1) * STAGE);
    if (a.diag && t0 > row0 + 32 * RG - 1) continue;  // wholly above this wave's rows (uniform)
    fwd_bf16_tile<D, BC, NW, RG, true>(a, smem + (t & 1) * STAGE, lo, qf, o, m_run, l_run, t0, qi, n, hf, lane);
  }
#pragma unroll
  for (int r = 0; r < RG; ++r) fwd_epilogue<D>(a, o[r], m_run[r], l_run[r], head, qi + 32 * r, hf);
}


template <typename T, int D, int BC, int NW>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st) {
  if (a.hpw < 1 || a.hsub < 1 || NW % a.hpw != 0) return hipErrorInvalidValue;
  const int R = NW * 32 / a.hpw;
  const int nrt = (a.len + R - 1) / R;
  const int nblk = nrt * a.hsub * a.hkv;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_step_kernel<T, D, BC, NW>), dim3(nblk), dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

constexpr int kFwdWaves = RA_FWD_WAVES;
// Both paths must share the wave count: the host derives the head packing from it.
constexpr int kF32Waves = kFwdWaves;

#ifndef RA_FWD_RG
#define RA_FWD_RG 1  // 32-row query groups per wave (2: 64 rows at one wave per SIMD)
#endif

// sub-problems of one launch must agree on the grid: same lengths and head layout.
// A causal diagonal block pairs query row i with key i, so it needs as many keys as rows.
template <typename A> static bool same_grid(const A* a, int nsub) {
  for (int i = 0; i < nsub; ++i)
    if (a[i].len != a[0].len || a[i].klen != a[0].klen || a[i].hq != a[0].hq || a[i].hkv != a[0].hkv ||
        a[i].hpw != a[0].hpw || a[i].hsub != a[0].hsub || (a[i].diag && a[i].klen != a[i].len))
      return false;
  return true;
}

template <int D, int BC, int NW>
static hipError_t launch_fwd_bf16(const FwdArgs* a, int nsub, hipStream_t st) {
  if (a[0].hpw < 1 || a[0].hsub < 1 || NW % a[0].hpw != 0) return hipErrorInvalidValue;
  const int R = NW * 32 * RA_FWD_RG / a[0].hpw;
  const int nblk = ((a[0].len + R - 1) / R) * a[0].hsub * a[0].hkv;
  if (nblk == 0) return hipSuccess;
  ArgPair<FwdArgs> pair{};
  for (int i = 0; i < nsub; ++i) pair.s[i] = a[i];
  if (nsub == 1)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, BC, NW, RA_FWD_RG, FwdArgs>), dim3(nblk), dim3(NW * 64), 0, st, a[0]);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, BC, NW, RA_FWD_RG, ArgPair<FwdArgs>>), dim3(nblk, nsub), dim3(NW * 64), 0,
                       st, pair);
  return hipGetLastError();
}

hipError_t launch_fwd_step(const FwdArgs* a, int nsub, int elem_bytes, int head_dim, hipStream_t st) {
  if (nsub < 1 || nsub > 2 || !same_grid(a, nsub)) return hipErrorInvalidValue;
  if (elem_bytes == 2) {
    if (head_dim == 64) return launch_fwd_bf16<64, RA_FWD_BC, kFwdWaves>(a, nsub, st);
    if (head_dim == 128) return launch_fwd_bf16<128, RA_FWD_BC, kFwdWaves>(a, nsub, st);
  } else {
    if (nsub != 1) return hipErrorInvalidValue;  // the fp32 path runs one sub-problem per launch
    if (head_dim == 64) return launch_fwd_t<float, 64, 64, kF32Waves>(a[0], st);
    if (head_dim == 128) return launch_fwd_t<float, 128, 32, kF32Waves>(a[0], st);
  }
  return hipErrorInvalidValue;
}

int fwd_waves_per_block(int) { return kFwdWaves; }

}  // namespace ra
