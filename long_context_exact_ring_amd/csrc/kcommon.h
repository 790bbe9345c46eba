// Device-side building blocks shared by the gfx950 ring-attention kernels.
//
// Matrix core: v_mfma_f32_32x32x16_bf16 (bf16 path) and v_mfma_f32_32x32x2_f32
// (fp32 path).  Both use the same 32x32 fp32 accumulator layout, so one
// kernel body serves both element types:
//
//   A operand (32 rows x 16 k): lane l supplies row l%32, k = (l/32)*8 + e, e=0..7
//   B operand (16 k x 32 cols): lane l supplies col l%32, k = (l/32)*8 + e
//   C (32x32 fp32, 16 regs):    lane l holds col l%32, rows (i/4)*8 + (l/32)*4 + i%4
//
// A bf16 "fragment" is the 8 k-values of one lane (16 bytes); the fp32 path
// keeps 8 fp32 values per lane and issues eight k=2 MFMAs, the e-th of which
// contracts element e of every lane.  Because a contraction may visit its k
// index in any order, a fragment only has to hold the same logical k values
// in the A and B operands; the kernels exploit this to feed an accumulator
// straight back in as the next product's B operand (see key_of_creg).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

typedef uint16_t bf16_storage;  // bf16 values travel as raw 16-bit patterns

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- fragments
template <typename T> struct Frag;
template <> struct Frag<bf16_storage> { uint4 v; };
template <> struct Frag<float> { float4 lo, hi; };

template <typename T> __device__ __forceinline__ Frag<T> frag_zero();
template <> __device__ __forceinline__ Frag<bf16_storage> frag_zero<bf16_storage>() {
  return Frag<bf16_storage>{make_uint4(0, 0, 0, 0)};
}
template <> __device__ __forceinline__ Frag<float> frag_zero<float>() {
  return Frag<float>{make_float4(0, 0, 0, 0), make_float4(0, 0, 0, 0)};
}

// 8 consecutive elements from (global or LDS) memory, 16-byte aligned
template <typename T> __device__ __forceinline__ Frag<T> frag_load(const T* p);
template <> __device__ __forceinline__ Frag<bf16_storage> frag_load(const bf16_storage* p) {
  return Frag<bf16_storage>{*reinterpret_cast<const uint4*>(p)};
}
template <> __device__ __forceinline__ Frag<float> frag_load(const float* p) {
  const float4* q = reinterpret_cast<const float4*>(p);
  return Frag<float>{q[0], q[1]};
}

// 8 fp32 values -> fragment (bf16: round to nearest even via v_cvt_pk_bf16_f32)
template <typename T> __device__ __forceinline__ Frag<T> frag_from_f32(const float* x);
template <> __device__ __forceinline__ Frag<bf16_storage> frag_from_f32(const float* x) {
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f32x2_t a = {x[2 * j], x[2 * j + 1]};
    bf16x2_t b = __builtin_convertvector(a, bf16x2_t);
    w[j] = __builtin_bit_cast(uint32_t, b);
  }
  return Frag<bf16_storage>{make_uint4(w[0], w[1], w[2], w[3])};
}
template <> __device__ __forceinline__ Frag<float> frag_from_f32(const float* x) {
  return Frag<float>{make_float4(x[0], x[1], x[2], x[3]), make_float4(x[4], x[5], x[6], x[7])};
}

// fp16 operands.  The bf16 backward converts its inputs to IEEE half once
// (exact: a bf16 value has 8 significant bits, a half 11, and every bf16 of
// magnitude in [2^-14, 65504] is a normal half) and then runs its contractions
// on fp16 MFMA, so the probabilities and dS it rounds for the matrix core keep
// 11 bits instead of 8.  Half fragments travel in the same 16-byte Frag
// storage as bf16 ones.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// c += A * B over one 16-wide k slice, both fragments holding IEEE half bits
__device__ __forceinline__ void mma_h(f32x16_t& c, const Frag<bf16_storage>& a, const Frag<bf16_storage>& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a.v), __builtin_bit_cast(f16x8_t, b.v), c,
                                             0, 0, 0);
}

// 8 fp32 values -> half fragment (round to nearest even, v_cvt_pk_f16_f32)
__device__ __forceinline__ Frag<bf16_storage> frag_h_from_f32(const float* x) {
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f32x2_t a = {x[2 * j], x[2 * j + 1]};
    f16x2_t b = __builtin_convertvector(a, f16x2_t);
    w[j] = __builtin_bit_cast(uint32_t, b);
  }
  return Frag<bf16_storage>{make_uint4(w[0], w[1], w[2], w[3])};
}

// Two bf16 values (one 32-bit word) -> two halves, in place.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  f32x2_t a = {__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(a, f16x2_t));
}
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 v) {
  return make_uint4(bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z), bf16x2_to_f16x2(v.w));
}

// c += A * B over one 16-wide k slice
__device__ __forceinline__ void mma(f32x16_t& c, const Frag<bf16_storage>& a,
                                    const Frag<bf16_storage>& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a.v),
                                              __builtin_bit_cast(bf16x8_t, b.v), c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16_t& c, const Frag<float>& a, const Frag<float>& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.x, b.lo.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.y, b.lo.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.z, b.lo.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.w, b.lo.w, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.x, b.hi.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.y, b.hi.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.z, b.hi.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.w, b.hi.w, c, 0, 0, 0);
}

// Row (within a 32-row C tile) held by accumulator register i of a lane in half hf.
__device__ __forceinline__ constexpr int crow(int i, int hf) {
  return ((i >> 2) << 3) + (hf << 2) + (i & 3);
}

// The accumulator of a 32x32 C tile, read as B operands: registers
// (kc%2)*8 .. +7 of C tile kc/2 hold rows {crow(i, hf)}, i.e. for 16-row
// chunk kc the lane in half hf holds rows kc*16 + (e/4)*8 + hf*4 + e%4.
// The matching A operand must therefore list its k values in that order.
// perm16(r) gives, for row r of a 16-row chunk, the position at which a
// lane-contiguous A fragment stores it: half hf = (r/4)%2, element e.
__device__ __forceinline__ constexpr int perm16(int r) {
  return (((r >> 2) & 1) << 3) + ((r >> 3) << 2) + (r & 3);
}
__device__ __forceinline__ constexpr int perm_pos(int r) {  // any row index
  return (r & ~15) + perm16(r & 15);
}

// cross-half exchange: value of lane l ^ 32
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte global load / store helpers
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// Global -> LDS copy of 16 bytes per lane by the load unit (LDS DMA): lane i's
// 16 bytes land at LDS byte address lds_base + 16*i.  Written as inline asm on
// purpose: with the compiler's intrinsic, the wait-count pass cannot tell which
// LDS bytes the copy writes and stalls every later LDS read until the copy
// completes, which serialises the prefetch of the next tile against the reads
// of the current one.  The asm has no register outputs; callers make the data
// visible with `s_waitcnt vmcnt(0)` followed by a workgroup barrier.  The LDS
// base goes in through the M0 register as an operand ("{m0}"), so the compiler
// writes M0 itself and knows what it holds; the asm never modifies it.
__device__ __forceinline__ void lds_dma16(const void* gaddr, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(gaddr), "{m0}"(lds_base) : "memory");
}

// Same, with a uniform 64-bit base in SGPRs and a 32-bit per-lane byte offset
// (no per-lane address arithmetic when only the base moves).
__device__ __forceinline__ void lds_dma16_off(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "{m0}"(lds_base) : "memory");
}

// Same, 4 bytes per lane (lane i's dword lands at lds_base + 4*i).
__device__ __forceinline__ void lds_dma4(const void* gaddr, uint32_t lds_base) {
  asm volatile("global_load_lds_dword %0, off" : : "v"(gaddr), "{m0}"(lds_base) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// XOR swizzle of the 16-byte chunks of an unpadded [rows][D] bf16 tile in LDS
// (row r stores logical chunk c at chunk slot c ^ swz(r)).  Chosen so that both
// ways the kernels read such a tile are bank-conflict free on the 64 x 4-byte
// LDS banks:
//  * ds_read_b128 of one chunk by 16 consecutive rows (MFMA operand with k = D)
//    -- swz is a bijection on every 16 consecutive rows (D=128) or on every 8
//    row pairs (D=64, two 128-byte rows per bank sweep);
//  * ds_read_b64_tr_b16 of 4 (x2) consecutive rows by 4 consecutive chunks
//    (transposed operand) -- the high bits of swz spread such row quads over
//    different 64-byte bank groups.
template <int D> __device__ __forceinline__ constexpr int swz(int r);
template <> __device__ __forceinline__ constexpr int swz<128>(int r) {
  return ((r & 3) << 2) | ((r >> 2) & 3);
}
template <> __device__ __forceinline__ constexpr int swz<64>(int r) {
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));

// Transposed LDS read (ds_read_b64_tr_b16).  Within each 16-lane group, lane j
// receives element k (k = 0..3) = the 16-bit value at byte (address of lane
// 4k + j/4) + 2*(j%4).  With lane i pointing at row base+i/4, column
// c0 + 4*(i%4) of a row-major bf16 tile, lane j thus gets rows base..base+3 of
// column c0 + j: four consecutive k values of one operand row.
__device__ __forceinline__ uint2 ds_read_tr16(const unsigned char* p) {
  v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)(p));
  return __builtin_bit_cast(uint2, r);
}

// A operand (rows = tile column, k = 16 tile rows) of a 32x32x16 MFMA read
// transposed from a swizzled [rows][D] bf16 tile: lane l covers operand row
// (column of the tile) col0 + l%32 and tile rows kc*16 + {h*4..h*4+3,
// 8+h*4..8+h*4+3} (h = l/32), the order in which a 32x32 accumulator hands
// its rows to a B operand (see perm16).
template <int D>
__device__ __forceinline__ Frag<bf16_storage> tr_frag(const unsigned char* tile, int col0, int kc, int lane) {
  const int g = lane >> 4, i16 = lane & 15;
  const int dcol = col0 + (g & 1) * 16 + 4 * (i16 & 3);
  uint2 part[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = kc * 16 + u * 8 + (g >> 1) * 4 + (i16 >> 2);
    const int c = (dcol >> 3) ^ swz<D>(r);
    part[u] = ds_read_tr16(tile + r * (D * 2) + c * 16 + (dcol & 7) * 2);
  }
  return Frag<bf16_storage>{make_uint4(part[0].x, part[0].y, part[1].x, part[1].y)};
}

// B or A operand with k = D from a swizzled [rows][D] bf16 tile: row r, k slice ks.
template <int D>
__device__ __forceinline__ Frag<bf16_storage> row_frag(const unsigned char* tile, int r, int ks, int hf) {
  const int c = (ks * 2 + hf) ^ swz<D>(r);
  return Frag<bf16_storage>{*reinterpret_cast<const uint4*>(tile + r * (D * 2) + c * 16)};
}

// Per-lane byte offsets of the operand reads of a stage holding swizzled
// [rows][D] bf16 tiles: `k` for row_frag(n, ks, hf) reads of a tile at the
// stage start, `v` for the transposed tr_frag(dt * 32, kc = 0) reads of a
// tile `tileb` bytes in.  A swizzled row's chunk order repeats every 16 rows,
// so reads of other 32-row (row_frag) or 16-row (tr_frag) slices differ from
// these by immediates, and with the stage known at compile time every read is
// one ds_read with no address arithmetic.
template <int D>
struct LdsOperandOffsets {
  uint32_t k[D / 16];     // row_frag(n, ks, hf) of the tile at the stage start
  uint32_t v[D / 32][2];  // the two transposed reads of tr_frag(dt * 32, kc = 0) of the tile at tileb
  __device__ __forceinline__ LdsOperandOffsets(int lane, int tileb) {
    const int n = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) k[ks] = n * (D * 2) + (((ks * 2 + hf) ^ swz<D>(n)) * 16);
    const int gq = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int dcol = dt * 32 + (gq & 1) * 16 + 4 * (i16 & 3);
        const int r = u * 8 + (gq >> 1) * 4 + (i16 >> 2);
        v[dt][u] = tileb + r * (D * 2) + (((dcol >> 3) ^ swz<D>(r)) * 16) + (dcol & 7) * 2;
      }
  }
};

// LDS DMA of rows [t0, t0 + ROWS) of a token-major [len][heads][D] bf16 tensor
// (head offset already applied, `stride` elements between rows) into a
// swizzled [ROWS][D] tile.  The NW waves of the workgroup split the 1 KB
// instructions; rows past `len` re-read row len-1 (callers mask them).
template <int D, int ROWS, int NW>
__device__ __forceinline__ void dma_rows(const bf16_storage* base, size_t stride, int t0, int len,
                                         unsigned char* tile, int wu, int lane) {
  constexpr int ROWB = D * 2, RPI = 1024 / ROWB, CPR = ROWB / 16;
  constexpr int NI = ROWS / RPI;  // 1 KB instructions per tile
  static_assert(NI % NW == 0 || NI < NW, "tile instructions must spread over the waves");
  constexpr int IPW = (NI + NW - 1) / NW;
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int q = wu * IPW + j;
    if (NI % NW != 0 && q >= NI) break;  // uniform
    const int r = q * RPI + lane / CPR, slot = lane % CPR;
    const int row = min(t0 + r, len - 1);
    const bf16_storage* src = base + (size_t)row * stride + ((slot ^ swz<D>(r)) * 8);
    lds_dma16(src, __builtin_amdgcn_readfirstlane(lds_addr(tile + q * 1024)));
  }
}

// XCD-aware work order: the dispatcher deals workgroups round-robin over the
// 8 XCDs, so consecutive logical tiles (which share K/V) are remapped onto
// one XCD and its L2.
__device__ __forceinline__ int xcd_logical_block(int bid, int nblocks) {
  if (nblocks % 8 != 0) return bid;
  return (bid % 8) * (nblocks / 8) + bid / 8;
}

}  // namespace ra
