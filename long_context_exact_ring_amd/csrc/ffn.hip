// Blockwise feedforward for gfx950 (the feedforward half of a blockwise
// transformer layer: "Ring Attention with Blockwise Transformers for
// Near-Infinite Context" close-reading notes, §2.2 -- computing the
// feedforward block by block caps its largest activation at the size of one
// block of the 4h-wide intermediate instead of the whole sequence's).
//
//   Y = GELU(X W1^T + b1) W2^T + b2      X [rows][hidden], W1 [ffn][hidden],
//                                        W2 [hidden][ffn] (weights [out][in])
//
// computed over row chunks: per chunk, one GEMM writes the bf16 intermediate
// H = GELU(X W1^T + b1) of that chunk only, a second GEMM reads it back.
//
// GEMM kernel (gemm_bt_kernel): C[m][n] = sum_k A[m][k] B[n][k] with both
// operands k-contiguous.  A 256x256 workgroup tile of eight 64x128 waves
// (0.75 KB of LDS reads per MFMA) where the shape fills the chip with it,
// else 128x128 with four 64x64 waves; a k-step of 64 staged global -> LDS by
// LDS DMA into swizzled 128-byte rows (double-buffered, one barrier per
// k-step).  The MFMA computes the tile
// transposed (weights as the A operand, activation rows as B), so a lane ends
// up holding four consecutive output columns of one row: bias, GELU and the
// bf16 / fp32 stores work on contiguous 8- or 16-byte pieces.
#include "kcommon.h"
#include "kernels.h"

namespace ra {

namespace {

constexpr int kGemmBM = 128, kGemmBN = 128, kGemmBK = 64;

// exact GELU, x * Phi(x), with the error function of the device math library
__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.f + erff(x * 0.70710678118654752f)); }

}  // namespace

// A wave computes TM x TN transposed 32x32 tiles (TM along the activation
// rows, TN along the weight rows); the workgroup is WGM x WGN waves.
template <int TM, int TN, int WGM, int WGN, bool GELU_BF16_OUT>
__global__ __launch_bounds__(WGM * WGN * 64) void gemm_bt_kernel(GemmArgs a) {
  constexpr int NW = WGM * WGN;
  constexpr int BM = WGM * TM * 32, BN = WGN * TN * 32;
  constexpr int ROWB = kGemmBK * 2;              // 128 bytes per tile row
  constexpr int ATILE = BM * ROWB, BTILE = BN * ROWB;
  constexpr int STAGE = ATILE + BTILE;           // activation tile, weight tile
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int n = lane & 31, hf = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wu % WGM, wn = wu / WGM;  // this wave's (TM*32) x (TN*32) piece

  // workgroup -> (row tile, column tile).  Consecutive workgroups (one XCD's
  // share, one L2) cover a band of up to a.group row tiles across successive
  // column tiles, so the tiles one XCD holds in flight form a block of the
  // output and each operand tile it reads from HBM serves several of them.
  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int ntn = a.n / BN, ntm = (a.m + BM - 1) / BM;
  const int band = logical / (a.group * ntn), first_m = band * a.group;
  const int gm = min(ntm - first_m, a.group), in_band = logical - band * a.group * ntn;
  const int tm = first_m + in_band % gm, tn = in_band / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  // DMA lane offsets: a 1 KB instruction moves 8 rows of 128 bytes
  constexpr int RPI = 1024 / ROWB, CPR = ROWB / 16;  // 8 rows, 8 chunks per row
  constexpr int NIA = BM / RPI, NIB = BN / RPI;      // instructions per operand tile
  static_assert(NIA % NW == 0 && NIB % NW == 0, "tile DMA must split evenly over the waves");
  constexpr int IPA = NIA / NW, IPB = NIB / NW;
  uint32_t aoff[IPA], boff[IPB];
#pragma unroll
  for (int j = 0; j < IPA; ++j) {
    const int r = (wu * IPA + j) * RPI + lane / CPR, slot = lane % CPR;
    const int mr = min(m0 + r, a.m - 1);  // rows past the end re-read the last row (never stored)
    aoff[j] = (uint32_t)(((size_t)mr * a.lda + (slot ^ swz<64>(r)) * 8) * 2);
  }
#pragma unroll
  for (int j = 0; j < IPB; ++j) {
    const int r = (wu * IPB + j) * RPI + lane / CPR, slot = lane % CPR;
    boff[j] = (uint32_t)(((size_t)(n0 + r) * a.ldb + (slot ^ swz<64>(r)) * 8) * 2);
  }
  const unsigned char* abase = reinterpret_cast<const unsigned char*>(a.a);
  const unsigned char* bbase = reinterpret_cast<const unsigned char*>(a.b);
  auto issue = [&](int ks, unsigned char* st) {
    const size_t kb = (size_t)ks * kGemmBK * 2;
#pragma unroll
    for (int j = 0; j < IPA; ++j)
      lds_dma16_off(abase + kb, aoff[j],
                    __builtin_amdgcn_readfirstlane(lds_addr(st + (uint32_t)(wu * IPA + j) * 1024)));
#pragma unroll
    for (int j = 0; j < IPB; ++j)
      lds_dma16_off(bbase + kb, boff[j],
                    __builtin_amdgcn_readfirstlane(lds_addr(st + ATILE + (uint32_t)(wu * IPB + j) * 1024)));
  };

  f32x16_t acc[TN][TM];  // [weight-row tile][activation-row tile], transposed 32x32 tiles
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = f32x16_t{};

  const int nk = a.k / kGemmBK;
  issue(0, smem);
  for (int ks = 0; ks < nk; ++ks) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's part of k-step ks has landed
    __syncthreads();                                     // ... everyone's; the other stage is free
    if (ks + 1 < nk) issue(ks + 1, smem + ((ks + 1) & 1) * STAGE);
    const unsigned char* at = smem + (ks & 1) * STAGE;  // activation rows
    const unsigned char* bt = at + ATILE;               // weight rows
#pragma unroll
    for (int kk = 0; kk < kGemmBK / 16; ++kk) {
      Frag<bf16_storage> wf[TN], xf[TM];
#pragma unroll
      for (int i = 0; i < TN; ++i) wf[i] = row_frag<64>(bt, (wn * TN + i) * 32 + n, kk, hf);
#pragma unroll
      for (int j = 0; j < TM; ++j) xf[j] = row_frag<64>(at, (wm * TM + j) * 32 + n, kk, hf);
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) mma(acc[i][j], wf[i], xf[j]);
    }
  }

  // epilogue: lane holds output row m = m0 + (wm*TM + j)*32 + n and columns
  // n0 + (wn*TN + i)*32 + crow(r, hf) for the 16 accumulator registers r
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int m = m0 + (wm * TM + j) * 32 + n;
    if (m >= a.m) continue;
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c0 = n0 + (wn * TN + i) * 32 + q4 * 8 + hf * 4;  // four consecutive columns
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = acc[i][j][4 * q4 + e];
          if (a.bias) v[e] += a.bias[c0 + e];
        }
        if constexpr (GELU_BF16_OUT) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = gelu_erf(v[e]);
          f32x2_t lo = {v[0], v[1]}, hi = {v[2], v[3]};
          const uint2 packed = make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2_t)),
                                          __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2_t)));
          *reinterpret_cast<uint2*>(reinterpret_cast<bf16_storage*>(a.c) + (size_t)m * a.ldc + c0) = packed;
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.c) + (size_t)m * a.ldc + c0) =
              make_float4(v[0], v[1], v[2], v[3]);
        }
      }
  }
}

#ifndef RA_GEMM_BIG
#define RA_GEMM_BIG 1  // 0: always the 128x128 tile; 1: 256-wide tiles where the shape allows
#endif

template <int TM, int TN, int WGM, int WGN>
static hipError_t launch_gemm_cfg(const GemmArgs& a, bool gelu_bf16_out, hipStream_t st) {
  constexpr int BM = WGM * TM * 32, BN = WGN * TN * 32;
  const long nblk = (long)((a.m + BM - 1) / BM) * (a.n / BN);
  if (gelu_bf16_out)
    hipLaunchKernelGGL((gemm_bt_kernel<TM, TN, WGM, WGN, true>), dim3((unsigned)nblk), dim3(WGM * WGN * 64), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_bt_kernel<TM, TN, WGM, WGN, false>), dim3((unsigned)nblk), dim3(WGM * WGN * 64), 0, st,
                       a);
  return hipGetLastError();
}

hipError_t launch_gemm_bt(const GemmArgs& args, bool gelu_bf16_out, hipStream_t st) {
  if (args.m < 1 || args.n % kGemmBN != 0 || args.k % kGemmBK != 0 || args.n < kGemmBN || args.k < kGemmBK)
    return hipErrorInvalidValue;
  // bands of 4 row tiles for short contractions, 8 for long ones (measured on
  // the 8192 x 4096 x 16384 feedforward block: the hidden -> ffn product
  // gains ~8% with 4, the ffn -> hidden product ~2% with 8)
  GemmArgs a = args;
  a.group = a.k <= 8192 ? 4 : 8;
  // 256x256 tiles (8 waves of 64x128) when the columns allow it and the grid still fills the chip
  if (RA_GEMM_BIG && a.n % 256 == 0 && (long)((a.m + 255) / 256) * (a.n / 256) >= 256)
    return launch_gemm_cfg<2, 4, 4, 2>(a, gelu_bf16_out, st);
  // 128x256 tiles (four 64x128 waves) for shorter row blocks
  if (RA_GEMM_BIG >= 2 && a.n % 256 == 0 && (long)((a.m + 127) / 128) * (a.n / 256) >= 256)
    return launch_gemm_cfg<2, 4, 2, 2>(a, gelu_bf16_out, st);
  return launch_gemm_cfg<2, 2, 2, 2>(a, gelu_bf16_out, st);
}

int gemm_tile_n() { return kGemmBN; }
int gemm_tile_k() { return kGemmBK; }

}  // namespace ra
