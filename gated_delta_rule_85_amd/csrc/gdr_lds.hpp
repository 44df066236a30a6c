// LDS data movement and MFMA operand reads shared by the gfx950 kernels.
//
// Tiles live in LDS row-major with XOR-swizzled 16-byte chunks (Swz in
// gdr_layout.hpp).  In the accumulator-order convention of gdr_device.hpp
// every operand of a row-major tile M is one of two reads:
//   frag(M, row, byte)     A operand of M (rows of M, k = its columns), which
//                          is also the B operand of M^T;
//   kt_operand(M, c0, ip)  A operand of M^T (rows = columns c0.. of M, k = its
//                          rows 32 ip ..), which is also the B operand of M,
//                          read with the gfx950 transposing LDS read.
#pragma once

#include "gdr_device.hpp"
#include "gdr_layout.hpp"

namespace gdr {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// wave-wide copy of 64 x 16 bytes: lane l's source -> lds_base + 16 l.  The
// LDS address is taken from the low 32 bits of the generic pointer (its
// offset in the LDS aperture) rather than by a pointer cast, whose null check
// the compiler cannot always select.
__device__ __forceinline__ void dma16(const void *src, char *lds_base) {
    lds_void *d = (lds_void *)(uintptr_t)(uint32_t)(uintptr_t)lds_base;
    __builtin_amdgcn_global_load_lds((glb_void *)src, d, 16, 0, 0);
}
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)

// Workgroup barrier that orders LDS accesses only: __syncthreads() also waits
// for every global load and store the wave has in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// gfx950 transposing LDS read: within each 16-lane group, lane i receives
// element i%4 of the 8-byte chunks read by source lanes i/4 + 4j, j = 0..3.
__device__ __forceinline__ bf16x4 lds_tr4(const char *p) {
    v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p));
    return __builtin_bit_cast(bf16x4, v);
}

// Copy the 64 rows of a row-major global tile (row r at src + r * stride,
// ROWB bytes each) into a swizzled LDS tile, rows past nm1 repeating row nm1.
// The 1 KB pieces are spread over nw waves; this wave is number wi of them.
template <int ROWB, typename KEY = typename DefaultKey<ROWB>::type>
__device__ __forceinline__ void copy_rows(char *dst, const char *src, int stride, int nm1, int wi, int nw) {
    using S = Swz<ROWB, KEY>;
    constexpr int PIECES = CH * ROWB / 1024;
    const int l = lane_id();
    for (int i = wi; i < PIECES; i += nw) {
        const int b = i * 1024 + 16 * l, r = b / ROWB, pc = (b % ROWB) / 16;
        dma16(src + (uint32_t)(min(r, nm1) * stride + 16 * S::chunk(r, pc)), dst + i * 1024);
    }
}
// Copy `bytes` (a multiple of 1 KB) verbatim, pieces spread as above.
__device__ __forceinline__ void copy_bytes(char *dst, const char *src, int bytes, int wi, int nw) {
    const int l = lane_id();
    for (int i = wi; i < bytes / 1024; i += nw) dma16(src + i * 1024 + 16 * l, dst + i * 1024);
}

// A-operand fragment rows (row0 + lane16, bytes off..off+7 and off+32..) of a swizzled tile
template <typename In, int ROWB, typename KEY = typename DefaultKey<ROWB>::type>
__device__ __forceinline__ typename Ops<In>::X frag(const char *tile, int row, int byte) {
    using S = Swz<ROWB, KEY>;
    return Ops<In>::load(reinterpret_cast<const In *>(tile + S::off(row, byte)),
                         reinterpret_cast<const In *>(tile + S::off(row, byte + 16 * sizeof(In))));
}

// 4 consecutive rows r0+4g..r0+4g+3 of column c0+lane16, as the B operand of
// an accumulator-ordered tile expects
template <typename In, int ROWB>
__device__ __forceinline__ f32x4 rows4(const char *tile, int r0, int c0) {
    using S = Swz<ROWB>;
    const int n = ln16(), g = lg4();
    if constexpr (sizeof(In) == 2) {
        const bf16x4 v = lds_tr4(tile + S::off(r0 + 4 * g + (n >> 2), 2 * (c0 + 4 * (n & 3))));
        return __builtin_convertvector(v, f32x4);
    } else {
        f32x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            r[j] = *reinterpret_cast<const float *>(tile + S::off(r0 + 4 * g + j, 4 * (c0 + n)));
        return r;
    }
}

// A operand of K^T: rows = key dims d0 + lane16, k = tokens 32 ip .. 32 ip + 31
template <typename In, int ROWB, typename KEY = typename DefaultKey<ROWB>::type>
__device__ __forceinline__ typename Ops<In>::X kt_operand(const char *Ks, int d0, int ip) {
    typename Ops<In>::X r;
    if constexpr (sizeof(In) == 2) {
        using S = Swz<ROWB, KEY>;
        const int n = ln16(), g = lg4();
        const int row = 32 * ip + 4 * g + (n >> 2), byte = 2 * (d0 + 4 * (n & 3));
        r.b0 = lds_tr4(Ks + S::off(row, byte));
        r.b1 = lds_tr4(Ks + S::off(row + 16, byte));
    } else {
        r.b0 = rows4<In, ROWB>(Ks, 32 * ip, d0);
        r.b1 = rows4<In, ROWB>(Ks, 32 * ip + 16, d0);
    }
    return r;
}

// ------------------------------------------------- contiguous-slot operands
// The slot -> k map of an operand may be any map shared by A and B.  With
// "slot j (0..7) of lane group g is k = 8g + j" inside each 32-deep k block,
// a lane's operand is 8 consecutive elements of a row: one 16-byte LDS read
// (bf16).  A pair of accumulator tiles (t0, t0+1) used as such an operand has
// to hold k = 8g + i in tile t0 and 8g + 4 + i in tile t0+1 at row 4g + i, so
// the rows of tile t of a 64-row block are taken in the order
//   row 4g + i of tile t  <->  index slot_base(t, g) + i.
__host__ __device__ __forceinline__ int slot_base(int t, int g) { return 32 * (t >> 1) + 4 * (t & 1) + 8 * g; }
// index held by A-operand row n (0..15) of tile t in that order
__host__ __device__ __forceinline__ int slot_row(int t, int n) { return slot_base(t, n >> 2) + (n & 3); }

// A operand (row `row`, k = 8 consecutive elements from byte `byte`, which is
// a multiple of 16) of a row-major tile with swizzle S
template <typename In, typename S>
__device__ __forceinline__ typename Ops<In>::X frag8(const char *tile, int row, int byte) {
    typename Ops<In>::X r;
    if constexpr (sizeof(In) == 2) {
        const bf16x8 v = *reinterpret_cast<const bf16x8 *>(tile + S::off(row, byte));
        r.b0 = __builtin_shufflevector(v, v, 0, 1, 2, 3);
        r.b1 = __builtin_shufflevector(v, v, 4, 5, 6, 7);
    } else {
        r.b0 = *reinterpret_cast<const f32x4 *>(tile + S::off(row, byte));
        r.b1 = *reinterpret_cast<const f32x4 *>(tile + S::off(row, byte + 16));
    }
    return r;
}

// rows rb + j (j = 0..3; rb may differ per lane group) of column c0 + lane16,
// as the B operand of an accumulator tile expects
template <typename In, typename S>
__device__ __forceinline__ f32x4 rows4b(const char *tile, int rb, int c0) {
    const int n = ln16();
    if constexpr (sizeof(In) == 2) {
        const bf16x4 v = lds_tr4(tile + S::off(rb + (n >> 2), 2 * (c0 + 4 * (n & 3))));
        return __builtin_convertvector(v, f32x4);
    } else {
        f32x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = *reinterpret_cast<const float *>(tile + S::off(rb + j, 4 * (c0 + n)));
        return r;
    }
}

// A operand of M^T in contiguous slots: row n of the 16-row tile is column
// c0 + cstep * (n / 4) + n % 4 of M, k = rows r0 + 8g + j (j = 0..7) of M.
template <typename In, typename S>
__device__ __forceinline__ typename Ops<In>::X kt8(const char *M, int r0, int c0, int cstep) {
    typename Ops<In>::X r;
    const int n = ln16(), g = lg4();
    if constexpr (sizeof(In) == 2) {
        const int row = r0 + 8 * g + (n >> 2), byte = 2 * (c0 + cstep * (n & 3));
        r.b0 = lds_tr4(M + S::off(row, byte));
        r.b1 = lds_tr4(M + S::off(row + 4, byte));
    } else {
        const int col = c0 + cstep * (n >> 2) + (n & 3);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            r.b0[j] = *reinterpret_cast<const float *>(M + S::off(r0 + 8 * g + j, 4 * col));
            r.b1[j] = *reinterpret_cast<const float *>(M + S::off(r0 + 8 * g + 4 + j, 4 * col));
        }
    }
    return r;
}

}  // namespace gdr
