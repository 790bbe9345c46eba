// bf16 backward ring-step kernels for gfx950 (the fp32 twins live in bwd_step.hip).
//
// Gradients of exact attention over one K/V block, recomputing the
// probabilities from the forward's log-sum-exp: with S = Q K^T / sqrt(d),
// P = exp(S - lse), dP = dO V^T, dS = P * (dP - Delta):
//   dQ += dS K / sqrt(d),   dK += dS^T Q / sqrt(d),   dV += P^T dO.
// (The ring runs in every layer of training -- close-reading notes on "Ring
// Attention with Blockwise Transformers for Near-Infinite Context", §3.5 --
// so the same rotated K/V blocks drive the backward.)
//
// Operand precision: the inputs are bf16, but every contraction here runs on
// fp16 MFMA.  Q and dO reach these kernels as half copies made by the
// preprocess kernel, the dK/dV kernel converts its K and V rows when it loads
// them (and writes the half K/V rows out for the dQ kernel of the same round).
// The conversion is exact for the inputs' values, so S and dP are the same
// products as in bf16; what changes is the rounding of P and dS, the operands
// the kernels produce themselves: 11 significant bits instead of 8, an eighth
// of the error in dV, dK and dQ.  Inputs must stay below 65504 in magnitude
// (the half range); below 2^-14 a half keeps an absolute step of 2^-24.
//
// Same building blocks as the bf16 forward: streamed tiles are copied
// global -> LDS by LDS DMA into unpadded, XOR-swizzled rows; operands whose
// contraction index runs along the tile rows are read with transposed LDS
// reads (tr_frag) instead of being stored twice; diagonal-band and ragged
// tiles run in separate (masked) loops so the hot loop carries no masking.
//
//  * dK/dV kernel: a wave owns 32 keys (B operands with keys on lanes: V in
//    registers, the wave's K rows written to LDS once) and walks the query
//    tiles of every query head of its group, two tiles per barrier.  S and dP
//    come out with keys on lanes, so P and dS are B operands of
//    dV^T += dO^T P and dK^T += Q^T dS, whose A operands are transposed reads
//    of the streamed Q and dO tiles.  The row terms (lse, Delta) of a tile
//    ride along in LDS.
//  * dQ kernel: a wave owns 32 query rows (Q, dO in registers, queries on
//    lanes, lse and Delta per-lane scalars) and walks the K/V tiles; dQ^T +=
//    K^T dS^T reads K transposed from the same K tile used for S^T.
#include <type_traits>

#include "kcommon.h"
#include "kernels.h"

namespace ra {

namespace {

#ifndef RA_BWD_NW
#define RA_BWD_NW 8
#endif
#ifndef RA_KV_NW
#define RA_KV_NW 8
#endif
constexpr int kBwdNW = RA_BWD_NW;  // dQ kernel: waves per workgroup (2 per SIMD)
constexpr int kKvNW = RA_KV_NW;    // dK/dV kernel: waves per workgroup (2 per SIMD; K rows read from LDS)

}  // namespace

// =================================================================== dK / dV
template <int D, int BR, int NW>
__device__ __forceinline__ void dkdv_body(const BwdArgs& a) {
  constexpr int ROWB = D * 2;
  constexpr int TILEB = BR * ROWB;
  constexpr int STAGE = 2 * TILEB + 2 * BR * 4;  // Q tile, dO tile, lse2[BR], Delta[BR]
  // Four LDS stages: one barrier per two query tiles, the DMA of the next two
  // tiles issued right after it.
  constexpr int NB = 4;
  constexpr int KTB = NW * 32 * ROWB;  // the workgroup's K rows (half), read from LDS
  static_assert(BR % 32 == 0 && (BR == 32 || BR % 64 == 0), "row-term DMA covers 64 dwords per wave");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[NB * STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char ktile[KTB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int n = lane & 31, hf = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int KW = NW * 32;
  const int nkt = (a.klen + KW - 1) / KW;
  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int kt = logical % nkt;  // ascending: with a causal diagonal, low key tiles are heaviest
  const int g = logical / nkt;
  const int kb0 = kt * KW;
  const int key0 = kb0 + wu * 32;
  const int key = key0 + n;
  const size_t qstride = (size_t)a.hq * D, kvstride = (size_t)a.hkv * D;

  // K and V become half operands here.  The workgroup's K rows are copied to
  // LDS by DMA (each wave moves exactly its own 32 rows), converted in place by
  // that wave, and written back out as halves with whole-row stores; this
  // lane's V row is loaded and converted in registers (B operands with keys
  // on lanes) and written out too.  The half copies feed the dQ kernel of the
  // same round: every key of every K/V head belongs to exactly one workgroup.
  dma_rows<D, NW * 32, NW>(reinterpret_cast<const bf16_storage*>(a.k) + (size_t)g * D, kvstride, kb0, a.klen,
                           ktile, wu, lane);
  Frag<bf16_storage> vf[D / 16];
  {
    const int kr = min(key, a.klen - 1);  // lanes past the end compute garbage that is never stored
    const size_t off = (size_t)kr * kvstride + (size_t)g * D + hf * 8;
    const bf16_storage* vp = reinterpret_cast<const bf16_storage*>(a.v) + off;
    bf16_storage* v16 = reinterpret_cast<bf16_storage*>(a.v16) + off;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) vf[ks].v = bf16x8_to_f16x8(ld16(vp + ks * 16));
    if (key < a.klen)
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) st16(v16 + ks * 16, vf[ks].v);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's K rows have landed
  {
    constexpr int CPR = ROWB / 16, RPI = 64 / CPR;  // 16-byte chunks per row, rows per pass
    bf16_storage* k16 = reinterpret_cast<bf16_storage*>(a.k16) + (size_t)g * D;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = wu * 32 + i * RPI + lane / CPR, slot = lane % CPR;
      uint4* p = reinterpret_cast<uint4*>(ktile + r * ROWB + slot * 16);
      const uint4 kh = bf16x8_to_f16x8(*p);
      *p = kh;
      if (kb0 + r < a.klen) st16(k16 + (size_t)(kb0 + r) * kvstride + ((slot ^ swz<D>(r)) * 8), kh);
    }
  }
  __syncthreads();  // the half K rows are in LDS

  f32x16_t dkT[D / 32], dvT[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    dkT[dt] = f32x16_t{};
    dvT[dt] = f32x16_t{};
  }

  const int nqt = (a.len + BR - 1) / BR;
  const int qt_lo = a.diag ? kb0 / BR : 0;                        // earlier tiles: every key is in their future
  const int qt_nb = a.diag ? min(nqt, (kb0 + KW - 1 + BR - 1) / BR) : qt_lo;  // end of the diagonal band
  const int qt_full = max(qt_nb, a.len / BR);                     // ragged tail from here
  const int per_head = nqt - qt_lo;
  const int iters = per_head * a.group;

  // a.q / a.dout hold the half copies of the query block and its output gradient
  auto issue = [&](int it, unsigned char* st) {
    const int hh = it / per_head, qt = qt_lo + it % per_head;
    const int head = g * a.group + hh;
    const int r0 = qt * BR;
    dma_rows<D, BR, NW>(reinterpret_cast<const bf16_storage*>(a.q) + (size_t)head * D, qstride, r0, a.len, st, wu, lane);
    dma_rows<D, BR, NW>(reinterpret_cast<const bf16_storage*>(a.dout) + (size_t)head * D, qstride, r0, a.len,
                        st + TILEB, wu, lane);
    // row terms [lse2(BR) | Delta(BR)]: the last waves move 64 dwords each
    constexpr int NRW = (2 * BR + 63) / 64;
    static_assert(NRW <= NW, "row terms need more waves than the workgroup has");
    const int k = wu - (NW - NRW);
    if (k >= 0) {  // uniform
      const int e = k * 64 + lane;
      const int r = min(r0 + (e % BR), a.len - 1);
      const float* src = (e < BR ? a.lse2 : a.delta) + (size_t)head * a.ls + r;
      lds_dma4(src, __builtin_amdgcn_readfirstlane(lds_addr(st + 2 * TILEB + k * 256)));
    }
  };

  // part12: S = Q K^T and dP = dO V^T of one query tile, then P and dS as half
  // B fragments; false if every row of the tile precedes this wave's keys.
  // part3: dV^T += dO^T P and dK^T += Q^T dS with the tile's Q/dO read transposed.
  using BF = Frag<bf16_storage>;
  auto part12 = [&](int it, const unsigned char* st, auto masked_tag, BF(&pf)[BR / 32][2],
                    BF(&sf)[BR / 32][2]) -> bool {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int qt = qt_lo + it % per_head;
    const int r0 = qt * BR;
    const unsigned char* qn = st;
    const unsigned char* dn = st + TILEB;
    const float* rt = reinterpret_cast<const float*>(st + 2 * TILEB);
    if (MASKED && a.diag && key0 > r0 + BR - 1) return false;  // every row precedes this wave's keys
#pragma unroll
    for (int qs = 0; qs < BR / 32; ++qs) {
      f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        mma_h(s, row_frag<D>(qn, qs * 32 + n, ks, hf), row_frag<D>(ktile, wu * 32 + n, ks, hf));
        mma_h(dp, row_frag<D>(dn, qs * 32 + n, ks, hf), vf[ks]);
      }
      float p[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 l4 = *reinterpret_cast<const float4*>(rt + qs * 32 + j * 8 + hf * 4);
        const float4 d4 = *reinterpret_cast<const float4*>(rt + BR + qs * 32 + j * 8 + hf * 4);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * j + e;
          float pv = fast_exp2(__builtin_fmaf(s[i], a.scale_log2, -lv[e]));
          if constexpr (MASKED) {
            const int row = r0 + qs * 32 + crow(i, hf);
            if (row >= a.len || (a.diag && key > row)) pv = 0.f;
          }
          p[i] = pv;
          dp[i] = pv * (dp[i] - dv[e]);  // dS
        }
      }
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        float ds8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) ds8[e] = dp[c2 * 8 + e];
        pf[qs][c2] = frag_h_from_f32(p + c2 * 8);
        sf[qs][c2] = frag_h_from_f32(ds8);
      }
    }
    return true;
  };
  auto part3 = [&](const unsigned char* st, const BF(&pf)[BR / 32][2], const BF(&sf)[BR / 32][2]) {
    const unsigned char* qn = st;
    const unsigned char* dn = st + TILEB;
#pragma unroll
    for (int qs = 0; qs < BR / 32; ++qs)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const int kc = qs * 2 + c2;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          mma_h(dvT[dt], tr_frag<D>(dn, dt * 32, kc, lane), pf[qs][c2]);
          mma_h(dkT[dt], tr_frag<D>(qn, dt * 32, kc, lane), sf[qs][c2]);
        }
      }
  };

  int cur = 0;  // stage of tile it
  auto step = [&](int it, auto masked_tag) {
    if ((it & 1) == 0) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's DMA for tiles it and it+1 has landed
      __syncthreads();  // ... everyone's; every wave is past tile it-1, so the stages of tiles it-2, it-1 are free
      if (it + 2 < iters) issue(it + 2, smem + (it + 2) % NB * STAGE);
      if (it + 3 < iters) issue(it + 3, smem + (it + 3) % NB * STAGE);
    }
    BF pf[BR / 32][2], sf[BR / 32][2];
    if (part12(it, smem + cur * STAGE, masked_tag, pf, sf)) part3(smem + cur * STAGE, pf, sf);
    cur = cur + 1 == NB ? 0 : cur + 1;
  };
  if (iters > 0) issue(0, smem);
  if (iters > 1) issue(1, smem + STAGE);
  int it = 0;
  for (int hh = 0; hh < a.group; ++hh) {
    const int base = hh * per_head - qt_lo;  // it = base + qt
    for (; it < base + qt_nb; ++it) step(it, std::true_type{});
    for (; it < base + qt_full; ++it) step(it, std::false_type{});
    for (; it < base + nqt; ++it) step(it, std::true_type{});
  }

  if (key >= a.klen) return;
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

template <int D, int BR, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dkdv_bf16_kernel(BwdArgs a) {
  dkdv_body<D, BR, NW>(a);
}
// Two independent dK/dV sub-problems of one launch (blockIdx.y selects), e.g. the
// zig-zag layout's two key chunks of a block against the same query chunk.
template <int D, int BR, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dkdv_bf16_pair_kernel(ArgPair<BwdArgs> pair) {
  const BwdArgs a = pair.s[blockIdx.y];
  dkdv_body<D, BR, NW>(a);
}

// =================================================================== dQ
template <int D, int BC, int NW>
__device__ __forceinline__ void dq_body(const BwdArgs& a) {
  constexpr int ROWB = D * 2;
  constexpr int TILEB = BC * ROWB;
  constexpr int STAGE = 2 * TILEB;  // K tile, V tile
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int n = lane & 31, hf = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int R = NW * 32 / a.hpw;
  const int nrt = (a.len + R - 1) / R;
  int rt = logical % nrt;
  const int rest = logical / nrt;
  const int hs = rest % a.hsub;
  const int g = rest / a.hsub;
  if (a.diag) rt = nrt - 1 - rt;  // longest row tiles first
  const int wpr = NW / a.hpw;
  const int head = g * a.group + hs * a.hpw + wu / wpr;
  const int row0 = rt * R + (wu % wpr) * 32;
  const int qi = row0 + n;
  const int wg_first_row = rt * R;
  const int wg_last_row = min(rt * R + R, a.len) - 1;
  int ntiles = (a.klen + BC - 1) / BC;
  if (a.diag) ntiles = min(ntiles, wg_last_row / BC + 1);
  const int nfull = min(ntiles, a.diag ? (wg_first_row + 1) / BC : a.klen / BC);

  const size_t qstride = (size_t)a.hq * D, kvstride = (size_t)a.hkv * D;
  Frag<bf16_storage> qf[D / 16], of[D / 16];
  {
    const int qr = min(qi, a.len - 1);
    const bf16_storage* qp = reinterpret_cast<const bf16_storage*>(a.q) + (size_t)qr * qstride + (size_t)head * D + hf * 8;
    const bf16_storage* op = reinterpret_cast<const bf16_storage*>(a.dout) + (size_t)qr * qstride + (size_t)head * D + hf * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      qf[ks] = frag_load<bf16_storage>(qp + ks * 16);
      of[ks] = frag_load<bf16_storage>(op + ks * 16);
    }
  }
  const float lse2 = a.lse2[(size_t)head * a.ls + min(qi, a.len - 1)];
  const float dlt = a.delta[(size_t)head * a.ls + min(qi, a.len - 1)];
  __builtin_amdgcn_s_waitcnt(0x0F70);

  f32x16_t dqT[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) dqT[dt] = f32x16_t{};

  const bf16_storage* kbase = reinterpret_cast<const bf16_storage*>(a.k) + (size_t)g * D;
  const bf16_storage* vbase = reinterpret_cast<const bf16_storage*>(a.v) + (size_t)g * D;
  // whole tiles: a uniform base plus fixed per-lane offsets; the ragged last
  // tile re-reads its last row for the rows past the end (masked)
  constexpr int RPI = 1024 / ROWB, CPR = ROWB / 16, NI = BC / RPI;
  constexpr int IPW = (NI + NW - 1) / NW;
  uint32_t goff[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int r = (wu * IPW + j) * RPI + lane / CPR, slot = lane % CPR;
    goff[j] = (uint32_t)(r * kvstride + (slot ^ swz<D>(r)) * 8) * 2;
  }
  auto issue = [&](int t, unsigned char* st) {
    if ((t + 1) * BC <= a.klen) {
      const size_t tb = (size_t)t * BC * kvstride * 2;
      const unsigned char* kb = reinterpret_cast<const unsigned char*>(kbase) + tb;
      const unsigned char* vb = reinterpret_cast<const unsigned char*>(vbase) + tb;
#pragma unroll
      for (int j = 0; j < IPW; ++j) {
        const int q = wu * IPW + j;
        if (NI % NW != 0 && q >= NI) break;  // uniform
        lds_dma16_off(kb, goff[j], __builtin_amdgcn_readfirstlane(lds_addr(st + q * 1024)));
        lds_dma16_off(vb, goff[j], __builtin_amdgcn_readfirstlane(lds_addr(st + TILEB + q * 1024)));
      }
    } else {
      dma_rows<D, BC, NW>(kbase, kvstride, t * BC, a.klen, st, wu, lane);
      dma_rows<D, BC, NW>(vbase, kvstride, t * BC, a.klen, st + TILEB, wu, lane);
    }
  };
  const LdsOperandOffsets<D> lo(lane, 0);  // row reads of K and V, transposed reads of K

  auto tile = [&](int t, const unsigned char* st, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int t0 = t * BC;
    if (MASKED && a.diag && t0 > row0 + 31) return;  // wholly in this wave's future
    f32x16_t s[BC / 32], dp[BC / 32];
#pragma unroll
    for (int kt = 0; kt < BC / 32; ++kt) {
      s[kt] = f32x16_t{};
      dp[kt] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const Frag<bf16_storage> kf{*reinterpret_cast<const uint4*>(st + kt * 32 * ROWB + lo.k[ks])};
        const Frag<bf16_storage> vf{*reinterpret_cast<const uint4*>(st + TILEB + kt * 32 * ROWB + lo.k[ks])};
        mma_h(s[kt], kf, qf[ks]);
        mma_h(dp[kt], vf, of[ks]);
      }
    }
    const int lim = (a.diag ? min(qi, a.klen - 1) : a.klen - 1) - t0;  // visible local keys: <= lim
#pragma unroll
    for (int kt = 0; kt < BC / 32; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float pv = fast_exp2(__builtin_fmaf(s[kt][i], a.scale_log2, -lse2));
        if constexpr (MASKED) {
          if (kt * 32 + crow(i, hf) > lim) pv = 0.f;
        }
        dp[kt][i] = pv * (dp[kt][i] - dlt);  // dS^T
      }
#pragma unroll
    for (int kc = 0; kc < BC / 16; ++kc) {
      float ds8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ds8[e] = dp[kc >> 1][(kc & 1) * 8 + e];
      const Frag<bf16_storage> sf = frag_h_from_f32(ds8);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const uint2 v0 = ds_read_tr16(st + kc * 16 * ROWB + lo.v[dt][0]);
        const uint2 v1 = ds_read_tr16(st + kc * 16 * ROWB + lo.v[dt][1]);
        mma_h(dqT[dt], Frag<bf16_storage>{make_uint4(v0.x, v0.y, v1.x, v1.y)}, sf);
      }
    }
  };

  // ST: the stage of tile t when known at compile time (immediate LDS offsets), else -1
  auto step = [&](int t, auto masked_tag, auto stage_tag) {
    constexpr int ST = decltype(stage_tag)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int sc = ST >= 0 ? ST : (t & 1);
    if (t + 1 < ntiles) issue(t + 1, smem + (1 - sc) * STAGE);
    tile(t, smem + sc * STAGE, masked_tag);
  };

  issue(0, smem);
  int t = 0;
  for (; t + 1 < nfull; t += 2) {
    step(t, std::false_type{}, std::integral_constant<int, 0>{});
    step(t + 1, std::false_type{}, std::integral_constant<int, 1>{});
  }
  for (; t < nfull; ++t) step(t, std::false_type{}, std::integral_constant<int, -1>{});
  for (; t < ntiles; ++t) step(t, std::true_type{}, std::integral_constant<int, -1>{});

  if (qi >= a.len) return;
  float* dqp = a.dq + (size_t)qi * qstride + (size_t)head * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float4* p = reinterpret_cast<float4*>(dqp + dt * 32 + j * 8 + hf * 4);
      float4 r = make_float4(a.scale * dqT[dt][4 * j], a.scale * dqT[dt][4 * j + 1], a.scale * dqT[dt][4 * j + 2],
                             a.scale * dqT[dt][4 * j + 3]);
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

template <int D, int BC, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dq_bf16_kernel(BwdArgs a) {
  dq_body<D, BC, NW>(a);
}
// Two independent dQ sub-problems of one launch (blockIdx.y selects), e.g. the
// zig-zag layout's two query chunks against the same key chunk of a block.
template <int D, int BC, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dq_bf16_pair_kernel(ArgPair<BwdArgs> pair) {
  const BwdArgs a = pair.s[blockIdx.y];
  dq_body<D, BC, NW>(a);
}

#ifndef RA_BWD_BR
#define RA_BWD_BR 32
#endif
#ifndef RA_BWD_BC
#define RA_BWD_BC 64  // dQ kernel: keys per tile (64 measured 5% faster than 32)
#endif

template <int D>
static hipError_t launch_dkdv_bf16_t(const BwdArgs* a, int nsub, hipStream_t st) {
  const int KW = kKvNW * 32;
  const int nblk = ((a[0].klen + KW - 1) / KW) * a[0].hkv;
  if (nblk == 0) return hipSuccess;
  ArgPair<BwdArgs> pair{};
  for (int i = 0; i < nsub; ++i) pair.s[i] = a[i];
  if (nsub == 1)
    hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, RA_BWD_BR, kKvNW>), dim3(nblk), dim3(kKvNW * 64), 0, st, a[0]);
  else
    hipLaunchKernelGGL((bwd_dkdv_bf16_pair_kernel<D, RA_BWD_BR, kKvNW>), dim3(nblk, nsub), dim3(kKvNW * 64), 0, st,
                       pair);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_dq_bf16_t(const BwdArgs* a, int nsub, hipStream_t st) {
  if (a[0].hpw < 1 || a[0].hsub < 1 || kBwdNW % a[0].hpw != 0) return hipErrorInvalidValue;
  const int R = kBwdNW * 32 / a[0].hpw;
  const int nblk = ((a[0].len + R - 1) / R) * a[0].hsub * a[0].hkv;
  if (nblk == 0) return hipSuccess;
  ArgPair<BwdArgs> pair{};
  for (int i = 0; i < nsub; ++i) pair.s[i] = a[i];
  if (nsub == 1)
    hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, RA_BWD_BC, kBwdNW>), dim3(nblk), dim3(kBwdNW * 64), 0, st, a[0]);
  else
    hipLaunchKernelGGL((bwd_dq_bf16_pair_kernel<D, RA_BWD_BC, kBwdNW>), dim3(nblk, nsub), dim3(kBwdNW * 64), 0, st,
                       pair);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_bf16(const BwdArgs* a, int nsub, int head_dim, hipStream_t st) {
  if (head_dim == 64) return launch_dkdv_bf16_t<64>(a, nsub, st);
  if (head_dim == 128) return launch_dkdv_bf16_t<128>(a, nsub, st);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq_bf16(const BwdArgs* a, int nsub, int head_dim, hipStream_t st) {
  if (head_dim == 64) return launch_dq_bf16_t<64>(a, nsub, st);
  if (head_dim == 128) return launch_dq_bf16_t<128>(a, nsub, st);
  return hipErrorInvalidValue;
}

int bwd_bf16_waves_per_block() { return kBwdNW; }

}  // namespace ra
