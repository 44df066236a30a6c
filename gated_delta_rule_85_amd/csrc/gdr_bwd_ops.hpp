// Helpers shared by the bf16 backward kernels (gdr_bwd_scan.hip,
// gdr_bwd_mfma.hip): split-plane operand reads, tile copies, the
// transposed decayed scores and lane sums.
#pragma once

#include "gdr_kernels.hpp"
#include "gdr_lds.hpp"

namespace gdr {
namespace bwd {


// split operands from the hi plane at `hi` and the lo plane `plane` bytes after it,
// in layout L (L::off(row, byte): a swizzled tile, or the compact T block)
template <typename L>
__device__ __forceinline__ OpS frag_s_in(const char *hi, int plane, int row, int byte) {
    const int o0 = L::off(row, byte), o1 = L::off(row, byte + 32);
    OpS r;
    r.h0 = *reinterpret_cast<const bf16x4 *>(hi + o0);
    r.h1 = *reinterpret_cast<const bf16x4 *>(hi + o1);
    r.l0 = *reinterpret_cast<const bf16x4 *>(hi + plane + o0);
    r.l1 = *reinterpret_cast<const bf16x4 *>(hi + plane + o1);
    return r;
}
template <int ROWB>
__device__ __forceinline__ OpS frag_s(const char *hi, int plane, int row, int byte) {
    return frag_s_in<Swz<ROWB>>(hi, plane, row, byte);
}
// A operand of M^T (rows = columns c0 + lane16 of M, k = its rows 32 ip ..), layout L
template <typename L>
__device__ __forceinline__ OpX kt_in(const char *M, int c0, int ip) {
    const int n = ln16(), g = lg4();
    const int row = 32 * ip + 4 * g + (n >> 2), byte = 2 * (c0 + 4 * (n & 3));
    OpX r;
    r.b0 = lds_tr4(M + L::off(row, byte));
    r.b1 = lds_tr4(M + L::off(row + 16, byte));
    return r;
}
template <typename L>
__device__ __forceinline__ OpS kt_s_in(const char *hi, int plane, int c0, int ip) {
    const OpX a = kt_in<L>(hi, c0, ip), b = kt_in<L>(hi + plane, c0, ip);
    OpS r;
    r.h0 = a.b0;
    r.h1 = a.b1;
    r.l0 = b.b0;
    r.l1 = b.b1;
    return r;
}
template <int ROWB>
__device__ __forceinline__ OpS kt_s(const char *hi, int plane, int c0, int ip) {
    return kt_s_in<Swz<ROWB>>(hi, plane, c0, ip);
}

template <int ROWB, typename KEY = typename DefaultKey<ROWB>::type>
__device__ __forceinline__ void copy_tile(char *dst, const char *src, int stride, int nm1, int w) {
    copy_rows<ROWB, KEY>(dst, src, stride, nm1, w, NTHR / 64);
}
__device__ __forceinline__ void copy_flat(char *dst, const char *src, int bytes, int w) {
    copy_bytes(dst, src, bytes, w, NTHR / 64);
}

// upper-triangle 16x16 tiles (tr <= ti) of a 64 x 64 matrix, t = 0..9
__device__ __forceinline__ void upper_tile(int t, int &tr, int &ti) {
    tr = t < 4 ? 0 : t < 7 ? 1 : t < 9 ? 2 : 3;
    ti = t - (tr == 0 ? 0 : tr == 1 ? 3 : tr == 2 ? 5 : 6);
}

// P^T[r'][i] = (Q K^T)[i][r'] exp(gam_i - gam_r') for r' <= i < n into split
// planes (upper tiles only; wave w forms tiles w, w + 4, w + 8 of the ten)
template <int KD>
__device__ __forceinline__ void scores_t(char *Pt, const char *Qs, const char *Ks, const float *gam, int n,
                                         int w) {
    constexpr int KROW = KD * 2, PROW = 128, PPLANE = CH * PROW, DP = KD / 32;
    using SP = Swz<PROW>;
    const int n16 = ln16(), g = lg4();
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int t = w + 4 * k;
        if (t >= 10) break;
        int tr, ti;
        upper_tile(t, tr, ti);
        f32x4 acc = zero4();
#pragma unroll
        for (int dp = 0; dp < DP; ++dp)
            acc = mma(acc, frag<bf16, KROW, KeyBK>(Qs, 16 * ti + n16, (32 * dp + 4 * g) * 2),
                      frag<bf16, KROW, KeyBK>(Ks, 16 * tr + n16, (32 * dp + 4 * g) * 2));
        const int r = 16 * tr + n16;
        const float gr = gam[r];
        f32x4 v;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int i = 16 * ti + 4 * g + jj;
            v[jj] = (r <= i && i < n) ? acc[jj] * fast_exp(gam[i] - gr) : 0.f;
        }
        bf16x4 hi, lo;
        split4(v, hi, lo);
        const int off = SP::off(r, 2 * (16 * ti + 4 * g));
        *reinterpret_cast<bf16x4 *>(Pt + off) = hi;
        *reinterpret_cast<bf16x4 *>(Pt + PPLANE + off) = lo;
    }
}

// P^T tiles (1,0) and (3,2) below the diagonal are read as zero and never written
__device__ __forceinline__ void zero_lower_pt(char *Pt) {
    constexpr int PROW = 128, PPLANE = CH * PROW;
    using SP = Swz<PROW>;
    for (int idx = threadIdx.x; idx < 2 * 16 * 16; idx += NTHR) {
        const int t = idx >> 8, r = 16 + 32 * t + ((idx >> 4) & 15), i = 32 * t + (idx & 15);
        const int off = SP::off(r, 2 * i);
        *reinterpret_cast<bf16 *>(Pt + off) = bf16(0.f);
        *reinterpret_cast<bf16 *>(Pt + PPLANE + off) = bf16(0.f);
    }
}

// the same, by the threads of an eight-wave workgroup
__device__ __forceinline__ void zero_lower_pt2(char *Pt) {
    constexpr int PROW = 128, PPLANE = CH * PROW;
    using SP = Swz<PROW>;
    for (int idx = threadIdx.x; idx < 2 * 16 * 16; idx += 2 * NTHR) {
        const int t = idx >> 8, r = 16 + 32 * t + ((idx >> 4) & 15), i = 32 * t + (idx & 15);
        const int off = SP::off(r, 2 * i);
        *reinterpret_cast<bf16 *>(Pt + off) = bf16(0.f);
        *reinterpret_cast<bf16 *>(Pt + PPLANE + off) = bf16(0.f);
    }
}

// sum over the 4 lane groups
__device__ __forceinline__ float sum_groups(float v) {
    v += __shfl_xor(v, 16, 64);
    return v + __shfl_xor(v, 32, 64);
}
__device__ __forceinline__ float sum_wave(float v) { return sum_groups(row_sum16(v)); }

// four consecutive fp32 values (columns col .. col + 3 of one row) as hi/lo rows of
// split planes with 64 columns
__device__ __forceinline__ void put4_s(char *hi, int plane, int row, int col, f32x4 v) {
    const int off = Swz<128>::off(row, 2 * col);
    bf16x4 h, l;
    split4(v, h, l);
    *reinterpret_cast<bf16x4 *>(hi + off) = h;
    *reinterpret_cast<bf16x4 *>(hi + plane + off) = l;
}

}  // namespace bwd
}  // namespace gdr
