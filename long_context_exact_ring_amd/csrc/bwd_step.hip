// Backward ring-step kernels for gfx950: gradients of one rank's share with
// respect to Q and to one K/V block, recomputing the attention probabilities
// from the forward's saved log-sum-exp (no score matrix is stored).
//
// With S = Q K^T / sqrt(d), P = exp(S - lse), dP = dO V^T, Delta = rowsum(dO * O),
// dS = P * (dP - Delta):   dQ += dS K / sqrt(d),  dK += dS^T Q / sqrt(d),  dV += P^T dO.
// (Gradients of exact attention; the training use is named on the close-reading
// notes on "Ring Attention with Blockwise Transformers for Near-Infinite
// Context", abstract and §3.5, where the ring runs inside every layer.)
//
// Two kernels per ring round, neither uses atomics:
//  * dK/dV kernel, key-tile-major: a wave owns 32 keys of one K/V head with K and
//    V in registers as B operands; it walks every query tile of every query head
//    of the group, computing S and dP with keys on lanes (C layout: one key per
//    lane), so P and dS feed dV^T += dO^T P and dK^T += Q^T dS directly as B
//    operands against row-permuted transposed Q/dO tiles in LDS.
//  * dQ kernel, query-tile-major (the forward's structure): a wave owns 32
//    query rows with Q and dO in registers, computes S^T and dP^T with queries on
//    lanes, so lse and Delta are per-lane scalars, and accumulates
//    dQ^T += K^T dS^T against a row-permuted transposed K tile in LDS.
//  This recomputes S and dP in both kernels (7 contractions instead of 5) in
//  exchange for deterministic, contention-free accumulation.
#include "kcommon.h"
#include "kernels.h"
#include "tile_stage.h"

namespace ra {

// =================================================================== dK / dV
template <typename T, int D, int BR, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int NT = NW * 64;
  using St = TileStager<T, BR, D, NT>;
  constexpr int STAGE = 2 * St::NBYTES + 2 * St::TBYTES + 2 * BR * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, hf = lane >> 5;

  const int KW = NW * 32;  // keys per workgroup
  const int nkt = (a.len + KW - 1) / KW;
  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int kt = logical % nkt;  // ascending: with a causal diagonal, low key tiles are heaviest
  const int g = logical / nkt;
  const int kb0 = kt * KW;
  const int key0 = kb0 + w * 32;  // this wave's first key
  const int key = key0 + n;       // this lane's key

  const size_t qstride = (size_t)a.hq * D, kvstride = (size_t)a.hkv * D;

  // K and V of this lane's key as B operands (k = head_dim)
  Frag<T> kf[D / 16], vf[D / 16];
  {
    const T* kp = reinterpret_cast<const T*>(a.k) + (size_t)key * kvstride + (size_t)g * D + hf * 8;
    const T* vp = reinterpret_cast<const T*>(a.v) + (size_t)key * kvstride + (size_t)g * D + hf * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      kf[ks] = (key < a.len) ? frag_load<T>(kp + ks * 16) : frag_zero<T>();
      vf[ks] = (key < a.len) ? frag_load<T>(vp + ks * 16) : frag_zero<T>();
    }
  }
  f32x16_t dkT[D / 32], dvT[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    dkT[dt] = f32x16_t{};
    dvT[dt] = f32x16_t{};
  }

  const int nqt = (a.len + BR - 1) / BR;
  const int qt0 = a.diag ? kb0 / BR : 0;  // query tiles wholly above the diagonal are skipped
  const int per_head = nqt - qt0;
  const int iters = per_head * a.group;

  St qs, ds;
  auto gload = [&](int itn) {
    const int hh = itn / per_head, qt = qt0 + itn % per_head;
    const int head = g * a.group + hh;
    const int r0 = qt * BR;
    qs.load(reinterpret_cast<const T*>(a.q) + (size_t)head * D, qstride, r0, a.len, tid);
    ds.load(reinterpret_cast<const T*>(a.dout) + (size_t)head * D, qstride, r0, a.len, tid);
  };
  float lse_r = 0.f, del_r = 0.f;  // one row term per thread (tid < BR)
  auto gload_rows = [&](int itn) {
    const int hh = itn / per_head, qt = qt0 + itn % per_head;
    const int head = g * a.group + hh;
    const int r = qt * BR + tid;
    if (tid < BR) {
      lse_r = (r < a.len) ? a.lse[(size_t)head * a.ls + r] * kLog2e : 0.f;
      del_r = (r < a.len) ? a.delta[(size_t)head * a.ls + r] : 0.f;
    }
  };
  auto lstore = [&](int buf) {
    unsigned char* b = smem + buf * STAGE;
    qs.store(b, b + 2 * St::NBYTES, tid);
    ds.store(b + St::NBYTES, b + 2 * St::NBYTES + St::TBYTES, tid);
    float* rows = reinterpret_cast<float*>(b + 2 * St::NBYTES + 2 * St::TBYTES);
    if (tid < BR) {
      rows[tid] = lse_r;
      rows[BR + tid] = del_r;
    }
  };

  if (iters > 0) {
    gload(0);
    gload_rows(0);
    lstore(0);
  }
  __syncthreads();
  for (int it = 0; it < iters; ++it) {
    const int qt = qt0 + it % per_head;
    if (it + 1 < iters) {
      gload(it + 1);
      gload_rows(it + 1);
    }
    const unsigned char* b = smem + (it & 1) * STAGE;
    const unsigned char* qn = b;
    const unsigned char* dn = b + St::NBYTES;
    const unsigned char* qT = b + 2 * St::NBYTES;
    const unsigned char* dT = qT + St::TBYTES;
    const float* lse2 = reinterpret_cast<const float*>(dT + St::TBYTES);
    const float* dlt = lse2 + BR;
    const int r0 = qt * BR;
    // a wave whose keys all lie after the tile's last row sees only masked entries
    const bool active = !(a.diag && key0 > r0 + BR - 1) && key0 < a.len;
    if (active) {
#pragma unroll
      for (int qsub = 0; qsub < BR / 32; ++qsub) {
        f32x16_t s = f32x16_t{}, dp = f32x16_t{};
        const T* qrow = reinterpret_cast<const T*>(qn + (qsub * 32 + n) * St::NROW) + hf * 8;
        const T* drow = reinterpret_cast<const T*>(dn + (qsub * 32 + n) * St::NROW) + hf * 8;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          mma(s, frag_load<T>(qrow + ks * 16), kf[ks]);
          mma(dp, frag_load<T>(drow + ks * 16), vf[ks]);
        }
        // rows of this lane's 16 accumulator entries: qsub*32 + crow(i, hf)
        float p[16], dsv[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 l4 = *reinterpret_cast<const float4*>(lse2 + qsub * 32 + j * 8 + hf * 4);
          const float4 d4 = *reinterpret_cast<const float4*>(dlt + qsub * 32 + j * 8 + hf * 4);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * j + e;
            const int row = r0 + qsub * 32 + crow(i, hf);
            float pv = fast_exp2(__builtin_fmaf(s[i], a.scale_log2, -lv[e]));
            if (row >= a.len || key >= a.len || (a.diag && key > row)) pv = 0.f;
            p[i] = pv;
            dsv[i] = pv * (dp[i] - dv[e]);
          }
        }
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const Frag<T> pf = frag_from_f32<T>(p + c2 * 8);
          const Frag<T> sf = frag_from_f32<T>(dsv + c2 * 8);
          const int kcol = qsub * 32 + c2 * 16 + hf * 8;  // logical k offset within the tile
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
            const T* dtr = reinterpret_cast<const T*>(dT + (dt * 32 + n) * St::TROW) + kcol;
            const T* qtr = reinterpret_cast<const T*>(qT + (dt * 32 + n) * St::TROW) + kcol;
            mma(dvT[dt], frag_load<T>(dtr), pf);
            mma(dkT[dt], frag_load<T>(qtr), sf);
          }
        }
      }
    }
    if (it + 1 < iters) lstore((it + 1) & 1);
    __syncthreads();
  }

  if (key >= a.len) return;
  float* dkp = a.dk + (size_t)key * kvstride + (size_t)g * D;
  float* dvp = a.dv + (size_t)key * kvstride + (size_t)g * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = dt * 32 + j * 8 + hf * 4;
      float4* pk = reinterpret_cast<float4*>(dkp + d0);
      float4* pv = reinterpret_cast<float4*>(dvp + d0);
      float4 ok = *pk, ov = *pv;
      ok.x += a.scale * dkT[dt][4 * j];
      ok.y += a.scale * dkT[dt][4 * j + 1];
      ok.z += a.scale * dkT[dt][4 * j + 2];
      ok.w += a.scale * dkT[dt][4 * j + 3];
      ov.x += dvT[dt][4 * j];
      ov.y += dvT[dt][4 * j + 1];
      ov.z += dvT[dt][4 * j + 2];
      ov.w += dvT[dt][4 * j + 3];
      *pk = ok;
      *pv = ov;
    }
}

// =================================================================== dQ
template <typename T, int D, int BC, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dq_kernel(BwdArgs a) {
  constexpr int NT = NW * 64;
  using StK = TileStager<T, BC, D, NT>;
  constexpr int STAGE = 2 * StK::NBYTES + StK::TBYTES;  // K natural, V natural, K transposed
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, hf = lane >> 5;

  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int R = NW * 32 / a.hpw;
  const int nrt = (a.len + R - 1) / R;
  int rt = logical % nrt;
  const int rest = logical / nrt;
  const int hs = rest % a.hsub;
  const int g = rest / a.hsub;
  if (a.diag) rt = nrt - 1 - rt;
  const int wpr = NW / a.hpw;
  const int head = g * a.group + hs * a.hpw + w / wpr;
  const int row0 = rt * R + (w % wpr) * 32;
  const int qi = row0 + n;
  const int wg_last_row = min(rt * R + R, a.len) - 1;
  int ntiles = (a.len + BC - 1) / BC;
  if (a.diag) ntiles = min(ntiles, wg_last_row / BC + 1);

  const size_t qstride = (size_t)a.hq * D, kvstride = (size_t)a.hkv * D;

  Frag<T> qf[D / 16], of[D / 16];
  {
    const T* qp = reinterpret_cast<const T*>(a.q) + (size_t)qi * qstride + (size_t)head * D + hf * 8;
    const T* op = reinterpret_cast<const T*>(a.dout) + (size_t)qi * qstride + (size_t)head * D + hf * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      qf[ks] = (qi < a.len) ? frag_load<T>(qp + ks * 16) : frag_zero<T>();
      of[ks] = (qi < a.len) ? frag_load<T>(op + ks * 16) : frag_zero<T>();
    }
  }
  const float lse2 = (qi < a.len) ? a.lse[(size_t)head * a.ls + qi] * kLog2e : 0.f;
  const float dlt = (qi < a.len) ? a.delta[(size_t)head * a.ls + qi] : 0.f;

  f32x16_t dqT[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) dqT[dt] = f32x16_t{};

  const T* kbase = reinterpret_cast<const T*>(a.k) + (size_t)g * D;
  const T* vbase = reinterpret_cast<const T*>(a.v) + (size_t)g * D;
  StK kst, vst;
  auto gload = [&](int t0) {
    kst.load(kbase, kvstride, t0, a.len, tid);
    vst.load(vbase, kvstride, t0, a.len, tid);
  };
  auto lstore = [&](int buf) {
    unsigned char* b = smem + buf * STAGE;
    kst.store(b, b + 2 * StK::NBYTES, tid);
    vst.store(b + StK::NBYTES, nullptr, tid);
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int t0 = t * BC;
    if (t + 1 < ntiles) gload(t0 + BC);
    const unsigned char* b = smem + (t & 1) * STAGE;
    const unsigned char* kn = b;
    const unsigned char* vn = b + StK::NBYTES;
    const unsigned char* kT = b + 2 * StK::NBYTES;
    const bool active = !(a.diag && t0 > row0 + 31);
    if (active) {
      f32x16_t s[BC / 32], dp[BC / 32];
#pragma unroll
      for (int kt = 0; kt < BC / 32; ++kt) {
        s[kt] = f32x16_t{};
        dp[kt] = f32x16_t{};
        const T* krow = reinterpret_cast<const T*>(kn + (kt * 32 + n) * StK::NROW) + hf * 8;
        const T* vrow = reinterpret_cast<const T*>(vn + (kt * 32 + n) * StK::NROW) + hf * 8;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          mma(s[kt], frag_load<T>(krow + ks * 16), qf[ks]);
          mma(dp[kt], frag_load<T>(vrow + ks * 16), of[ks]);
        }
      }
      const bool need_mask = (a.diag && t0 + BC - 1 > row0) || (t0 + BC > a.len);
      float dsv[BC / 32][16];
#pragma unroll
      for (int kt = 0; kt < BC / 32; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float pv = fast_exp2(__builtin_fmaf(s[kt][i], a.scale_log2, -lse2));
          if (need_mask) {
            const int key = t0 + kt * 32 + crow(i, hf);
            if (key >= a.len || (a.diag && key > qi)) pv = 0.f;
          }
          dsv[kt][i] = pv * (dp[kt][i] - dlt);
        }
#pragma unroll
      for (int kc = 0; kc < BC / 16; ++kc) {
        const Frag<T> sf = frag_from_f32<T>(&dsv[kc >> 1][(kc & 1) * 8]);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const T* ktr = reinterpret_cast<const T*>(kT + (dt * 32 + n) * StK::TROW) + kc * 16 + hf * 8;
          mma(dqT[dt], frag_load<T>(ktr), sf);
        }
      }
    }
    if (t + 1 < ntiles) lstore((t + 1) & 1);
    __syncthreads();
  }

  if (qi >= a.len) return;
  float* dqp = a.dq + (size_t)qi * qstride + (size_t)head * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float4* p = reinterpret_cast<float4*>(dqp + dt * 32 + j * 8 + hf * 4);
      float4 r = make_float4(a.scale * dqT[dt][4 * j], a.scale * dqT[dt][4 * j + 1],
                             a.scale * dqT[dt][4 * j + 2], a.scale * dqT[dt][4 * j + 3]);
      if (!a.first) {
        const float4 o = *p;
        r.x += o.x;
        r.y += o.y;
        r.z += o.z;
        r.w += o.w;
      }
      *p = r;
    }
}

#ifndef RA_DQ_WAVES
#define RA_DQ_WAVES 8
#endif
#ifndef RA_KV_WAVES
#define RA_KV_WAVES 8
#endif
constexpr int kBwdWaves = RA_DQ_WAVES;
constexpr int kKvWaves = RA_KV_WAVES;

template <typename T, int D, int BR>
static hipError_t launch_dkdv_t(const BwdArgs& a, hipStream_t st) {
  const int KW = kKvWaves * 32;
  const int nblk = ((a.len + KW - 1) / KW) * a.hkv;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, BR, kKvWaves>), dim3(nblk), dim3(kKvWaves * 64), 0, st, a);
  return hipGetLastError();
}

template <typename T, int D, int BC>
static hipError_t launch_dq_t(const BwdArgs& a, hipStream_t st) {
  if (a.hpw < 1 || a.hsub < 1 || kBwdWaves % a.hpw != 0) return hipErrorInvalidValue;
  const int R = kBwdWaves * 32 / a.hpw;
  const int nblk = ((a.len + R - 1) / R) * a.hsub * a.hkv;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_dq_kernel<T, D, BC, kBwdWaves>), dim3(nblk), dim3(kBwdWaves * 64), 0, st, a);
  return hipGetLastError();
}

// sub-problems of one launch must agree on the grid: same lengths and head layout.
// A causal diagonal block pairs query row i with key i, so it needs as many keys as rows.
static bool same_bwd_grid(const BwdArgs* a, int nsub) {
  for (int i = 0; i < nsub; ++i)
    if (a[i].len != a[0].len || a[i].klen != a[0].klen || a[i].hq != a[0].hq || a[i].hkv != a[0].hkv ||
        a[i].hpw != a[0].hpw || a[i].hsub != a[0].hsub || (a[i].diag && a[i].klen != a[i].len))
      return false;
  return true;
}

hipError_t launch_bwd_dkdv(const BwdArgs* ap, int nsub, int elem_bytes, int head_dim, hipStream_t st) {
  if (nsub < 1 || nsub > 2 || !same_bwd_grid(ap, nsub)) return hipErrorInvalidValue;
  if (elem_bytes == 2) return launch_bwd_dkdv_bf16(ap, nsub, head_dim, st);
  // fp32: one sub-problem per launch, as many keys as query rows
  if (nsub != 1 || elem_bytes != 4 || ap[0].klen != ap[0].len) return hipErrorInvalidValue;
  const BwdArgs& a = ap[0];
  if (head_dim == 64) return launch_dkdv_t<float, 64, 32>(a, st);
  if (head_dim == 128) return launch_dkdv_t<float, 128, 32>(a, st);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq(const BwdArgs* ap, int nsub, int elem_bytes, int head_dim, hipStream_t st) {
  if (nsub < 1 || nsub > 2 || !same_bwd_grid(ap, nsub)) return hipErrorInvalidValue;
  if (elem_bytes == 2) return launch_bwd_dq_bf16(ap, nsub, head_dim, st);
  if (nsub != 1 || elem_bytes != 4 || ap[0].klen != ap[0].len) return hipErrorInvalidValue;
  const BwdArgs& a = ap[0];
  if (head_dim == 64) return launch_dq_t<float, 64, 32>(a, st);
  if (head_dim == 128) return launch_dq_t<float, 128, 32>(a, st);
  return hipErrorInvalidValue;
}

int bwd_dq_waves_per_block() { return kBwdWaves; }

}  // namespace ra
