// Forward epilogue shared by the forward kernels: normalise a lane's query
// row and overwrite the output, or fold it into the running (out, lse) of
// earlier ring rounds (close-reading notes on "Ring Attention with Blockwise
// Transformers for Near-Infinite Context", §3.1: partial results over disjoint
// key sets combine exactly through their log-sum-exp).
#pragma once

#include "kcommon.h"
#include "kernels.h"

namespace ra {

// Normalise this lane's query row and write it, or merge it into the running
// (out, lse) of earlier rounds: lse' = log(e^lse + e^lse_blk),
// out' = e^(lse - lse') out + e^(lse_blk - lse') O_blk.  m_run is the reference
// max (log2 units) the block's exponentials were taken against; l_run is this
// lane's half of the row sum (the other half sits in lane ^ 32).
template <int D>
__device__ __forceinline__ void fwd_epilogue(const FwdArgs& a, const f32x16_t (&o)[D / 32], float m_run,
                                             float l_run, int head, int qi, int hf) {
  const float l_tot = l_run + swap_halves(l_run);
  if (qi >= a.len) return;
  const size_t qstride = (size_t)a.hq * D;
  float* orow = a.out + (size_t)qi * qstride + (size_t)head * D;
  float* lsep = a.lse + (size_t)head * a.ls + qi;
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

}  // namespace ra
