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
//    16 in lane l^32), so the row max needs a single cross-half exchange and the
//    row sum none until the end.  Q lives in registers as the B operand.
//  * The exponentiated tile P^T is fed back unchanged as the B operand of
//    O^T += V^T P^T.  To make that legal V^T is staged in LDS with its keys
//    permuted inside every 16-key chunk to the order in which the accumulator
//    holds them (perm_pos); the contraction over keys is order-free.
//  * K/V tiles are double-buffered in LDS: the next tile's global loads are in
//    flight in registers while the current tile is computed; one barrier per tile.
//  * Causal (diagonal block): tiles wholly above a wave's rows are skipped, the
//    straddling tile is masked; heavy row tiles are dispatched first.
//  * Epilogue: normalise, then overwrite (first round) or merge into the running
//    (out, lse) in HBM.
#include "kcommon.h"
#include "kernels.h"

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
  static constexpr int KCH = BC * (D / CH);     // 16-byte K chunks per tile
  static constexpr int KIT = KCH / NT;
  static constexpr int VCH = (BC / 2) * (D / CH);  // (key pair, 16-byte chunk) items per tile
  static constexpr int VIT = VCH / NT;
  static_assert(KCH % NT == 0 && VCH % NT == 0, "tile not divisible among threads");
  static_assert((D / CH) % 4 == 0, "V staging groups 4 chunks");
  static_assert(BC % 32 == 0 && D % 32 == 0, "32x32 MFMA tiles");
};

template <typename T, int D, int BC, int NW>
__global__ __launch_bounds__(NW * 64) void fwd_step_kernel(FwdArgs a) {
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
  int ntiles = (a.len + BC - 1) / BC;
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

  // ------------------------------------------------ K/V staging
  uint4 kreg[C::KIT];
  uint4 vreg[C::VIT][2];
  auto gload = [&](int t0) {
#pragma unroll
    for (int it = 0; it < C::KIT; ++it) {
      const int id = it * C::NT + tid;
      const int r = id / (D / C::CH), ch = id % (D / C::CH);
      const int key = t0 + r;
      kreg[it] = (key < a.len) ? ld16(kbase + (size_t)key * kvstride + ch * C::CH) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int it = 0; it < C::VIT; ++it) {
      const int id = it * C::NT + tid;
      const int dc = ((id >> 2) / (BC / 2)) * 4 + (id & 3);
      const int kp = (id >> 2) % (BC / 2);
      const int key = t0 + 2 * kp;
      const T* p = vbase + (size_t)key * kvstride + dc * C::CH;
      vreg[it][0] = (key < a.len) ? ld16(p) : make_uint4(0, 0, 0, 0);
      vreg[it][1] = (key + 1 < a.len) ? ld16(p + kvstride) : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
    unsigned char* ks = smem + buf * C::STAGE;
    unsigned char* vs = ks + C::KBYTES;
#pragma unroll
    for (int it = 0; it < C::KIT; ++it) {
      const int id = it * C::NT + tid;
      const int r = id / (D / C::CH), ch = id % (D / C::CH);
      st16(ks + r * C::KROW + ch * 16, kreg[it]);
    }
#pragma unroll
    for (int it = 0; it < C::VIT; ++it) {
      const int id = it * C::NT + tid;
      const int dc = ((id >> 2) / (BC / 2)) * 4 + (id & 3);
      const int kp = (id >> 2) % (BC / 2);
      const int pos = perm_pos(2 * kp);  // keys 2kp, 2kp+1 stay adjacent
      const uint32_t* a0 = reinterpret_cast<const uint32_t*>(&vreg[it][0]);
      const uint32_t* a1 = reinterpret_cast<const uint32_t*>(&vreg[it][1]);
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t lo = (a0[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
          const uint32_t hi = (a1[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
          *reinterpret_cast<uint32_t*>(vs + (dc * 8 + e) * C::VROW + pos * 2) = lo | (hi << 16);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          *reinterpret_cast<uint2*>(vs + (dc * 4 + e) * C::VROW + pos * 4) = make_uint2(a0[e], a1[e]);
        }
      }
    }
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
      // masking: diagonal block (key > query) and ragged tail (key >= len)
      const int qi = row0 + n;
      if ((a.diag && t0 + BC - 1 > row0) || (t0 + BC > a.len)) {
#pragma unroll
        for (int kt = 0; kt < BC / 32; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = t0 + kt * 32 + crow(i, hf);
            if (key >= a.len || (a.diag && key > qi)) s[kt][i] = kNegInf;
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

  // ------------------------------------------------ epilogue: normalise and merge
  const int qi = row0 + n;
  if (qi >= a.len) return;
  const float l_tot = l_run + swap_halves(l_run);
  float* orow = a.out + (size_t)qi * qstride + (size_t)head * D;
  float* lsep = a.lse + (size_t)head * a.len + qi;
  float lse_cur, w_cur, w_old = 0.f;
  if (l_tot > 0.f) {
    lse_cur = (m_run + log2f(l_tot)) * kLn2;
    w_cur = 1.f / l_tot;
  } else {
    lse_cur = kNegInf;
    w_cur = 0.f;
  }
  float lse_new = lse_cur;
  if (!a.first) {
    const float lse_old = *lsep;
    const float mxl = fmaxf(lse_old, lse_cur);
    if (mxl == kNegInf) {
      lse_new = kNegInf;
      w_old = 0.f;
      w_cur = 0.f;
    } else {
      const float eo = expf(lse_old - mxl), ec = expf(lse_cur - mxl);
      const float z = eo + ec;
      lse_new = mxl + logf(z);
      w_old = eo / z;
      w_cur *= ec / z;
    }
  }
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float4* dst = reinterpret_cast<float4*>(orow + dt * 32 + j * 8 + hf * 4);
      float4 r = make_float4(o[dt][4 * j] * w_cur, o[dt][4 * j + 1] * w_cur, o[dt][4 * j + 2] * w_cur,
                             o[dt][4 * j + 3] * w_cur);
      if (!a.first) {
        const float4 old = *dst;
        r.x += w_old * old.x;
        r.y += w_old * old.y;
        r.z += w_old * old.z;
        r.w += w_old * old.w;
      }
      *dst = r;
    }
  if (hf == 0) *lsep = lse_new;
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

constexpr int kFwdWaves = 4;

hipError_t launch_fwd_step(const FwdArgs& a, int elem_bytes, int head_dim, hipStream_t st) {
  if (elem_bytes == 2) {
    if (head_dim == 64) return launch_fwd_t<bf16_storage, 64, 64, kFwdWaves>(a, st);
    if (head_dim == 128) return launch_fwd_t<bf16_storage, 128, 64, kFwdWaves>(a, st);
  } else {
    if (head_dim == 64) return launch_fwd_t<float, 64, 64, kFwdWaves>(a, st);
    if (head_dim == 128) return launch_fwd_t<float, 128, 32, kFwdWaves>(a, st);
  }
  return hipErrorInvalidValue;
}

int fwd_waves_per_block() { return kFwdWaves; }

}  // namespace ra
