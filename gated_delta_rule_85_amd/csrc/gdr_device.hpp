// Device helpers shared by the gfx950 gated delta rule kernels.
//
// MFMA operand convention ("accumulator order").  A 16x16 output tile of a
// v_mfma_f32_16x16x* instruction lives in lane l as rows 4*(l>>4)+j, j=0..3,
// of column l&15.  Every operand here uses the same shape for its k index:
// inside each 16-deep k block, lane l holds the 4 consecutive k values
// 4*(l>>4) .. 4*(l>>4)+3 of row (A) or column (B) l&15.  Because A and B use
// the same lane/slot -> k mapping, any such mapping gives the same product,
// and with this one an accumulator tile of X is, unchanged, the B operand of
// X (k = X's rows) and the A operand of X^T.  That is what lets the state h,
// the corrected values U~ and the decayed scores stay in registers between
// products.
//
// Precision.  Inputs q, k, v are exact bf16 values.  fp32 intermediates that
// feed a product are split into hi = bf16(x) and lo = bf16(x - hi); a product
// of a split operand with an exact one takes two MFMAs, split x split takes
// three (hi*hi + hi*lo + lo*hi), which keeps about 16 significant bits.  For
// fp32 inputs every operand is fp32 and the products use
// v_mfma_f32_16x16x4_f32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;    // chunk length
constexpr int NTHR = 256; // threads per workgroup (4 waves)

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
__device__ __forceinline__ int ln16() { return threadIdx.x & 15; }
__device__ __forceinline__ int lg4() { return (threadIdx.x >> 4) & 3; }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------- operands
struct OpX { bf16x4 b0, b1; };                    // exact bf16, k blocks 0 and 1
struct OpS { bf16x4 h0, h1, l0, l1; };            // split fp32, k blocks 0 and 1
struct OpF { f32x4 b0, b1; };                     // fp32 path

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x4 mfma_bf16(bf16x4 a0, bf16x4 a1, bf16x4 b0, bf16x4 b1, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(cat(a0, a1), cat(b0, b1), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma(f32x4 c, const OpX &a, const OpX &b) {
    return mfma_bf16(a.b0, a.b1, b.b0, b.b1, c);
}
__device__ __forceinline__ f32x4 mma(f32x4 c, const OpS &a, const OpX &b) {
    c = mfma_bf16(a.l0, a.l1, b.b0, b.b1, c);
    return mfma_bf16(a.h0, a.h1, b.b0, b.b1, c);
}
__device__ __forceinline__ f32x4 mma(f32x4 c, const OpX &a, const OpS &b) {
    c = mfma_bf16(a.b0, a.b1, b.l0, b.l1, c);
    return mfma_bf16(a.b0, a.b1, b.h0, b.h1, c);
}
__device__ __forceinline__ f32x4 mma(f32x4 c, const OpS &a, const OpS &b) {
    c = mfma_bf16(a.l0, a.l1, b.h0, b.h1, c);
    c = mfma_bf16(a.h0, a.h1, b.l0, b.l1, c);
    return mfma_bf16(a.h0, a.h1, b.h0, b.h1, c);
}
__device__ __forceinline__ f32x4 mma(f32x4 c, const OpF &a, const OpF &b) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b0[j], b.b0[j], c, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b1[j], b.b1[j], c, 0, 0, 0);
    return c;
}

// fp32 -> (hi, lo) bf16 pair, round to nearest even
// (each hi pair is one packed conversion; the fp32 value of its halves is a
// shift and a mask of that word)
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split4(f32x4 x, bf16x4 &hi, bf16x4 &lo) {
    const uint32_t a = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[0], x[1]}, bf16x2));
    const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[2], x[3]}, bf16x2));
    const f32x4 hf = {__builtin_bit_cast(float, a << 16), __builtin_bit_cast(float, a & 0xffff0000u),
                      __builtin_bit_cast(float, b << 16), __builtin_bit_cast(float, b & 0xffff0000u)};
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    hi = __builtin_bit_cast(bf16x4, (u32x2{a, b}));
    lo = __builtin_convertvector(x - hf, bf16x4);
}

// Per-input-type operand policy.
template <typename In> struct Ops;

template <> struct Ops<bf16> {
    using X = OpX;  // operand built from input values
    using S = OpS;  // operand built from fp32 intermediates
    // 4 consecutive inputs at p0 (k block 0) and p1 (k block 1)
    static __device__ __forceinline__ X load(const bf16 *p0, const bf16 *p1) {
        X r;
        r.b0 = *reinterpret_cast<const bf16x4 *>(p0);
        r.b1 = *reinterpret_cast<const bf16x4 *>(p1);
        return r;
    }
    static __device__ __forceinline__ S split(f32x4 x0, f32x4 x1) {
        S r;
        split4(x0, r.h0, r.l0);
        split4(x1, r.h1, r.l1);
        return r;
    }
};

template <> struct Ops<float> {
    using X = OpF;
    using S = OpF;
    static __device__ __forceinline__ X load(const float *p0, const float *p1) {
        X r;
        r.b0 = *reinterpret_cast<const f32x4 *>(p0);
        r.b1 = *reinterpret_cast<const f32x4 *>(p1);
        return r;
    }
    static __device__ __forceinline__ S split(f32x4 x0, f32x4 x1) { return S{x0, x1}; }
};

// split-operand storage in LDS for an fp32 matrix that is read as an A
// operand (row r, 4 consecutive k).  bf16 path: two bf16 planes; fp32 path:
// one fp32 plane.
template <typename In> struct SplitPlaneT { typedef bf16 type; };
template <> struct SplitPlaneT<float> { typedef float type; };

template <typename In> struct SplitPlane;
template <> struct SplitPlane<bf16> {
    bf16 *hi, *lo;
    // operand from byte offsets of k block 0 and k block 1 in both planes
    __device__ __forceinline__ OpS get_bytes(int b0, int b1) const {
        const char *H = reinterpret_cast<const char *>(hi), *Lo = reinterpret_cast<const char *>(lo);
        OpS r;
        r.h0 = *reinterpret_cast<const bf16x4 *>(H + b0);
        r.h1 = *reinterpret_cast<const bf16x4 *>(H + b1);
        r.l0 = *reinterpret_cast<const bf16x4 *>(Lo + b0);
        r.l1 = *reinterpret_cast<const bf16x4 *>(Lo + b1);
        return r;
    }
    // operand of 8 consecutive elements at byte o0 (16-byte aligned) of both planes
    __device__ __forceinline__ OpS get8(int o0, int) const {
        const bf16x8 h = *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const char *>(hi) + o0);
        const bf16x8 l = *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const char *>(lo) + o0);
        OpS r;
        r.h0 = __builtin_shufflevector(h, h, 0, 1, 2, 3);
        r.h1 = __builtin_shufflevector(h, h, 4, 5, 6, 7);
        r.l0 = __builtin_shufflevector(l, l, 0, 1, 2, 3);
        r.l1 = __builtin_shufflevector(l, l, 4, 5, 6, 7);
        return r;
    }
    __device__ __forceinline__ void put4(int off, f32x4 x) const {
        bf16x4 h, l;
        split4(x, h, l);
        *reinterpret_cast<bf16x4 *>(hi + off) = h;
        *reinterpret_cast<bf16x4 *>(lo + off) = l;
    }
    __device__ __forceinline__ OpS get(int off0, int off1) const {
        OpS r;
        r.h0 = *reinterpret_cast<const bf16x4 *>(hi + off0);
        r.h1 = *reinterpret_cast<const bf16x4 *>(hi + off1);
        r.l0 = *reinterpret_cast<const bf16x4 *>(lo + off0);
        r.l1 = *reinterpret_cast<const bf16x4 *>(lo + off1);
        return r;
    }
};
template <> struct SplitPlane<float> {
    float *hi, *lo;  // lo unused
    __device__ __forceinline__ OpF get_bytes(int b0, int b1) const {
        const char *H = reinterpret_cast<const char *>(hi);
        OpF r;
        r.b0 = *reinterpret_cast<const f32x4 *>(H + b0);
        r.b1 = *reinterpret_cast<const f32x4 *>(H + b1);
        return r;
    }
    // operand of 8 consecutive elements: bytes o0 .. o0+15 and o1 .. o1+15
    __device__ __forceinline__ OpF get8(int o0, int o1) const { return get_bytes(o0, o1); }
    __device__ __forceinline__ void put4(int off, f32x4 x) const {
        *reinterpret_cast<f32x4 *>(hi + off) = x;
    }
    __device__ __forceinline__ OpF get(int off0, int off1) const {
        OpF r;
        r.b0 = *reinterpret_cast<const f32x4 *>(hi + off0);
        r.b1 = *reinterpret_cast<const f32x4 *>(hi + off1);
        return r;
    }
};

template <typename T> __device__ __forceinline__ float to_f32(T x) { return static_cast<float>(x); }

// 16-byte vector of inputs
template <typename In> struct Vec16;
template <> struct Vec16<bf16> { typedef bf16x8 type; static constexpr int n = 8; };
template <> struct Vec16<float> { typedef f32x4 type; static constexpr int n = 4; };

// ---------------------------------------------------------------- sequences
// Packed-token view of a batch.  Without cu_seqlens, sequence j is tokens
// [j*T, (j+1)*T) and its chunks are j*ceil(T/64) ...; with cu_seqlens the
// chunk offsets come from a table built on the device (gdr_chunk_offsets).
struct SeqMap {
    const int32_t *cu;        // [n_seq+1] or null
    const int32_t *chunk_off; // [n_seq+1] or null (with cu)
    const int32_t *order;     // [n_seq] sequences by decreasing length, or null (with cu)
    int64_t T;                // tokens per sequence without cu
    int32_t n_seq;
    int32_t nct;              // chunks per sequence without cu

    __device__ __forceinline__ void bounds(int j, int64_t &bos, int64_t &eos) const {
        if (cu) {
            bos = cu[j];
            eos = cu[j + 1];
        } else {
            bos = (int64_t)j * T;
            eos = bos + T;
        }
    }
    __device__ __forceinline__ int chunk_base(int j) const { return cu ? chunk_off[j] : j * nct; }
    // global chunk id -> (sequence, chunk in sequence); false past the end
    __device__ __forceinline__ bool locate(int gid, int &j, int &c) const {
        if (!cu) {
            j = gid / nct;
            c = gid - j * nct;
            return j < n_seq;
        }
        if (gid >= chunk_off[n_seq]) return false;
        int lo = 0, hi = n_seq - 1;  // largest j with chunk_off[j] <= gid
        while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if (chunk_off[mid] <= gid) lo = mid; else hi = mid - 1;
        }
        j = lo;
        c = gid - chunk_off[j];
        return true;
    }
};

// Workgroup id -> logical work index such that consecutive logical indices
// run on the same XCD (the hardware deals workgroups to the 8 XCDs round
// robin, each XCD with its own L2).
__device__ __forceinline__ int xcd_remap(int id, int nb) {
    const int xcd = id & 7, pos = id >> 3, per = nb >> 3, rem = nb & 7;
    return xcd < rem ? xcd * (per + 1) + pos : rem * (per + 1) + (xcd - rem) * per + pos;
}

// Longest-first dealing of the (sequence, v head, value block) items of a scan
// launch over packed sequences of different lengths.  Items are grouped by
// (sequence, q/k head): the n_vt * (Hv / Hq) items of a group share K and Q.
// Group rank r (0 = a group of the longest sequence) goes to XCD r % 8 at the
// r / 8-th place of its queue, so that the first workgroups dispatched on every
// XCD hold the longest sequences and a group's items share one L2.  The grid
// has lpt_blocks() workgroups; false: this workgroup has no item.
__host__ __device__ inline int lpt_blocks(int n_seq, int Hq, int Hv, int n_vt) {
    return 8 * ((n_seq * Hq + 7) / 8) * n_vt * (Hv / Hq);
}
__device__ __forceinline__ bool lpt_item(const SeqMap &sm, int Hq, int Hv, int n_vt, int &vt, int &unit) {
    const int G = Hv / Hq, members = n_vt * G;
    const int b = blockIdx.x, x = b & 7, pp = b >> 3;
    const int q = pp / members, m = pp - q * members;
    const int r = q * 8 + x;
    if (r >= sm.n_seq * Hq) return false;
    const int j = sm.order[r / Hq], hq = r % Hq;
    vt = m % n_vt;
    unit = j * Hv + hq * G + m / n_vt;
    return true;
}

__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }

// ------------------------------------------------------------ lane sums
// DPP lane moves within a row of 16 lanes (VALU, no LDS round trip)
template <int CTRL> __device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL, int ROWS> __device__ __forceinline__ float dpp_mov_rows(float v) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xF, false));
}
// inclusive prefix sum over the 64 lanes: row_shr 1, 2, 4, 8 within each row of
// 16 (lanes without a source add 0), then row_bcast15 into rows 1 and 3 and
// row_bcast31 into rows 2 and 3
__device__ __forceinline__ float wave_prefix_sum(float x) {
    x += dpp_mov<0x111>(x);
    x += dpp_mov<0x112>(x);
    x += dpp_mov<0x114>(x);
    x += dpp_mov<0x118>(x);
    x += dpp_mov_rows<0x142, 0xA>(x);
    x += dpp_mov_rows<0x143, 0xC>(x);
    return x;
}
// sum over the 16 lanes of each row: quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp_mov<0xB1>(v);
    v += dpp_mov<0x4E>(v);
    v += dpp_mov<0x141>(v);
    v += dpp_mov<0x140>(v);
    return v;
}

}  // namespace gdr
