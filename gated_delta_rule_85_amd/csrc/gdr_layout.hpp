// LDS images shared by gdr_chunk_prep (writer) and gdr_scan_output (reader).
//
// Tiles in LDS are row-major with their 16-byte chunks XOR-swizzled by row:
// physical chunk p of row r holds logical chunk p ^ (r mod S), S = min(16,
// chunks per row).  Sixteen consecutive rows read at one column (the MFMA
// operand pattern) then fall into different banks, and a wave's direct
// global->LDS copy (64 lanes x 16 bytes, lane l -> base + 16 l) can still
// fill whole rows in order.
//
// Per (chunk, v head), gdr_chunk_prep writes one "T block", the exact LDS
// image the scan copies in:
//   bf16 inputs: T_hi[64][64] bf16, T_lo[64][64] bf16  (T = T_hi + T_lo)
//   fp32 inputs: T[64][64] fp32
//   then gam[64], e^gam[64], e^(gam_last - gam)[64], beta[64] (fp32)
// with rows/entries past the chunk end zero (gam: the last value repeated).
#pragma once

#include "gdr_device.hpp"

namespace gdr {

template <int ROWB> struct Swz {
    static constexpr int CPR = ROWB / 16;
    static constexpr int S = CPR < 16 ? CPR : 16;
    // byte offset of (row, byte-in-row) in the swizzled tile
    static __device__ __forceinline__ int off(int row, int byte) {
        return row * ROWB + ((((byte >> 4) ^ (row & (S - 1)))) << 4) + (byte & 15);
    }
    // logical chunk held by physical chunk p of row r (an involution)
    static __device__ __forceinline__ int chunk(int row, int p) { return p ^ (row & (S - 1)); }
};

template <typename In> struct TBlock {
    static constexpr bool BF = sizeof(In) == 2;
    static constexpr int ROWB = CH * (BF ? 2 : 4);  // bytes per plane row
    static constexpr int PLANE = CH * ROWB;
    static constexpr int NPL = BF ? 2 : 1;
    static constexpr int SC = NPL * PLANE;          // scalars
    static constexpr int BYTES = SC + 4 * CH * 4;
    static_assert(BYTES % 1024 == 0, "block copied in 1 KB wave transfers");
};

}  // namespace gdr
