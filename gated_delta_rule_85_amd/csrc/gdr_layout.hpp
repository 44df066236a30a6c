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

// Write one T block from an fp32 row-major T (row r, column i at T[r * ld + i])
// and the chunk's 64 gate values (gam padded with its last value, bet zero
// past the chunk end); rows r >= n are written as zero.  All threads of the
// workgroup take part; gam/bet/T are read, never written.
template <typename In>
__device__ __forceinline__ void write_tblock(char *blk, const float *T, int ld, const float *gam,
                                             const float *bet, int n, int tid, int nthr) {
    using TB = TBlock<In>;
    using SW = Swz<TB::ROWB>;
    constexpr int EPC = 16 / (TB::BF ? 2 : 4);  // elements per 16-byte chunk
    for (int idx = tid; idx < CH * SW::CPR; idx += nthr) {
        const int r = idx / SW::CPR, pc = idx % SW::CPR, lc = SW::chunk(r, pc);
        f32x4 x0 = zero4(), x1 = zero4();
        if (r < n) {
#pragma unroll
            for (int e = 0; e < 4; ++e) x0[e] = T[r * ld + EPC * lc + e];
            if constexpr (TB::BF) {
#pragma unroll
                for (int e = 0; e < 4; ++e) x1[e] = T[r * ld + EPC * lc + 4 + e];
            }
        }
        if constexpr (TB::BF) {
            bf16x4 h0, l0, h1, l1;
            split4(x0, h0, l0);
            split4(x1, h1, l1);
            *reinterpret_cast<bf16x8 *>(blk + r * TB::ROWB + 16 * pc) = cat(h0, h1);
            *reinterpret_cast<bf16x8 *>(blk + TB::PLANE + r * TB::ROWB + 16 * pc) = cat(l0, l1);
        } else {
            *reinterpret_cast<f32x4 *>(blk + r * TB::ROWB + 16 * pc) = x0;
        }
    }
    if (tid < CH) {
        float *sc = reinterpret_cast<float *>(blk + TB::SC);
        const float gl = gam[n - 1];
        sc[tid] = gam[tid];
        sc[CH + tid] = fast_exp(gam[tid]);
        sc[2 * CH + tid] = fast_exp(gl - gam[tid]);
        sc[3 * CH + tid] = bet[tid];
    }
}

}  // namespace gdr
