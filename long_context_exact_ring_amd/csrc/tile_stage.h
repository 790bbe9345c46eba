// Global -> LDS staging of a [ROWS][D] tile (token-major rows, 16-byte chunks),
// optionally in two layouts at once from the same global loads:
//   natural    [ROWS][D], row pitch D*ES + 16 bytes (MFMA operand with k = D)
//   transposed [D][ROWS], row pitch ROWS*ES + 16 bytes, rows permuted inside
//              every 16-row chunk by perm_pos (MFMA A operand with k = rows,
//              matched to accumulator-fed B operands, see kcommon.h)
// Each thread owns (row pair, chunk) items so that the transposed store can
// pack the two rows' values of one column into one 32-bit (bf16) or 64-bit
// (fp32) LDS write.  Rows at or beyond `valid` are zero-filled.
#pragma once

#include "kcommon.h"

namespace ra {

template <typename T, int ROWS, int D, int NT>
struct TileStager {
  static constexpr int ES = sizeof(T);
  static constexpr int CH = 16 / ES;
  static constexpr int NROW = D * ES + 16;     // natural pitch (bytes)
  static constexpr int TROW = ROWS * ES + 16;  // transposed pitch (bytes)
  static constexpr int NBYTES = ROWS * NROW;
  static constexpr int TBYTES = D * TROW;
  static constexpr int ITEMS = (ROWS / 2) * (D / CH);
  static constexpr int IT = (ITEMS + NT - 1) / NT;
  static_assert((D / CH) % 4 == 0, "chunks are grouped by four");
  static_assert(ROWS % 16 == 0, "row permutation works on 16-row chunks");

  uint4 reg[IT][2];

  __device__ __forceinline__ static void item(int id, int& dc, int& rp) {
    dc = ((id >> 2) / (ROWS / 2)) * 4 + (id & 3);
    rp = (id >> 2) % (ROWS / 2);
  }

  // base points at row 0 column 0 of the tile's head; stride = elements between rows
  __device__ __forceinline__ void load(const T* base, size_t stride, int row0, int valid, int tid) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int id = it * NT + tid;
      if (ITEMS % NT != 0 && id >= ITEMS) continue;
      int dc, rp;
      item(id, dc, rp);
      const int r = row0 + 2 * rp;
      const T* p = base + (size_t)r * stride + dc * CH;
      reg[it][0] = (r < valid) ? ld16(p) : make_uint4(0, 0, 0, 0);
      reg[it][1] = (r + 1 < valid) ? ld16(p + stride) : make_uint4(0, 0, 0, 0);
    }
  }

  __device__ __forceinline__ void store(unsigned char* nat, unsigned char* trn, int tid) const {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int id = it * NT + tid;
      if (ITEMS % NT != 0 && id >= ITEMS) continue;
      int dc, rp;
      item(id, dc, rp);
      if (nat) {
        st16(nat + (2 * rp) * NROW + dc * 16, reg[it][0]);
        st16(nat + (2 * rp + 1) * NROW + dc * 16, reg[it][1]);
      }
      if (trn) {
        const int pos = perm_pos(2 * rp);  // rows 2rp and 2rp+1 stay adjacent
        const uint32_t* a0 = reinterpret_cast<const uint32_t*>(&reg[it][0]);
        const uint32_t* a1 = reinterpret_cast<const uint32_t*>(&reg[it][1]);
        if constexpr (ES == 2) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t lo = (a0[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
            const uint32_t hi = (a1[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
            *reinterpret_cast<uint32_t*>(trn + (dc * 8 + e) * TROW + pos * 2) = lo | (hi << 16);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            *reinterpret_cast<uint2*>(trn + (dc * 4 + e) * TROW + pos * 4) = make_uint2(a0[e], a1[e]);
        }
      }
    }
  }
};

}  // namespace ra
