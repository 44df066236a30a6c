// Reverse state scan of the backward for bf16 inputs on bf16 MFMA.
//
// Part of the backward described in gdr_bwd_mfma.hip (the same split-bf16
// arithmetic); it sits in a file of its own because it is compiled with a
// scheduler of its own (the default one; the chain waves' operand reads are
// pipelined by hand, a stage ahead of their products).
#include <type_traits>

#include "gdr_bwd_ops.hpp"

namespace gdr {

namespace {

using namespace bwd;

// ------------------------------------------------------------- reverse scan
// One workgroup per (sequence, v head, 64 value columns); chain wave w owns
// columns 16 w .. 16 w + 15 and keeps its K x 16 slice of dh in registers
// (dh[dt] = keys slot_base(dt, g) + i, column 16 w + lane16).
// Per chunk, from the end: the transposed decayed scores P^T (upper
// triangular, shared split planes), then per chain wave
//   dU~ = diag(r) K dh' + s P^T dO,  dX = T^T dU~,
//   dh  = e_last dh' + Q^T diag(s e) dO - K^T diag(beta e) dX.
// A operand of M^T for a K x V tile in the contiguous-slot key order: row n is
// key c0 + 8 (n / 4) + n % 4, k = tokens 32 ip + 4g + j and 32 ip + 16 + 4g + j
// (the accumulator order of the token tiles it multiplies).  M is a K or Q tile
// of this kernel, swizzled with KeyBK (gdr_layout.hpp)
template <int ROWB>
__device__ __forceinline__ OpX kt_keys(const char *M, int c0, int ip) {
    using S = Swz<ROWB, KeyBK>;
    const int n = ln16(), g = lg4();
    const int row = 32 * ip + 4 * g + (n >> 2), byte = 2 * (c0 + 8 * (n & 3));
    OpX r;
    r.b0 = lds_tr4(M + S::off(row, byte));
    r.b1 = lds_tr4(M + S::off(row + 16, byte));
    return r;
}

// Eight waves, two per SIMD, in three roles: waves 0-3 ("chain") keep dh and
// form each chunk's products, plus one of the ten score tiles each; waves 4-5
// copy the next chunk (in reverse order) into LDS; waves 6-7 form the other six
// score tiles.  Per chunk two barriers, both ordering LDS only: after the score
// tiles (P^T dO needs all of them) and at the end (the copy waves wait for
// their copies first).
template <int KD>
__device__ __forceinline__ void score_tile_t(int t, char *Pt, const char *Qs, const char *Ks, const float *gam,
                                             int n) {
    constexpr int KROW = KD * 2, PROW = 128, PPLANE = CH * PROW, DP = KD / 32;
    using SP = Swz<PROW>;
    const int n16 = ln16(), g = lg4();
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

template <int KD>
__global__ __launch_bounds__(2 * NTHR) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_scan_roles_bf16(
    const BwdParams p, int n_units) {
    constexpr int KROW = KD * 2, DROW = 64 * 2, PROW = 64 * 2, PPLANE = CH * PROW;
    constexpr int DT = KD / 16, DP = KD / 32;
    constexpr int NCP = 2;  // copy waves
    using TB = TBlockF<bf16>;
    __shared__ __attribute__((aligned(16))) char Ks0[CH * KROW], Ks1[CH * KROW];
    __shared__ __attribute__((aligned(16))) char Qs0[CH * KROW], Qs1[CH * KROW];
    __shared__ __attribute__((aligned(16))) char Ds0[CH * DROW], Ds1[CH * DROW];
    __shared__ __attribute__((aligned(16))) char Tb0[TB::BYTES], Tb1[TB::BYTES];
    __shared__ __attribute__((aligned(16))) char Pt[2 * PPLANE];

    const int nvt = p.V / 64;
    int vt, unit, seg = 0;
    if (p.sm.order && p.n_seg == 1) {  // packed sequences: longest first
        if (!lpt_item(p.sm, p.Hq, p.Hv, nvt, vt, unit)) return;
    } else {
        const int wid = xcd_remap(blockIdx.x, gridDim.x);
        vt = wid % nvt;
        unit = (wid / nvt) % n_units;
        seg = wid / nvt / n_units;
        if (seg >= p.n_seg) return;
    }
    const int j = unit / p.Hv, hv = unit % p.Hv, hq = hv / (p.Hv / p.Hq);
    const int wv = __builtin_amdgcn_readfirstlane(wave_id()), n16 = ln16(), g = lg4();
    int64_t bos, eos;
    p.sm.bounds(j, bos, eos);
    const int N = (int)((eos - bos + CH - 1) / CH);
    const int c_begin = seg * p.seg_chunks;
    if (c_begin >= N && !(N == 0 && seg == 0)) return;
    const int c_end = min(N, c_begin + p.seg_chunks);
    const int cb = p.sm.chunk_base(j);
    const int64_t KV = (int64_t)KD * p.V;
    zero_lower_pt2(Pt);

    if (wv < 4) {
        // ------------------------------------------------------------ chain waves
        const int w = wv, col = vt * 64 + 16 * w + n16;
        const float *dh_start = c_end == N ? (p.dht ? p.dht + unit * KV : nullptr)
                                : p.d_seg ? nullptr
                                          : p.dh_seg + ((int64_t)unit * p.n_seg + seg) * KV;
        f32x4 dh[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dh[dt][i] = dh_start ? dh_start[(slot_base(dt, g) + i) * p.V + col] : 0.f;
        auto body = [&](auto cur, int c) {
            constexpr bool ONE = decltype(cur)::value == 1;
            const char *Ks = ONE ? Ks1 : Ks0, *Qs = ONE ? Qs1 : Qs0, *Ds = ONE ? Ds1 : Ds0, *Tb = ONE ? Tb1 : Tb0;
            const float *sc = reinterpret_cast<const float *>(Tb + TB::SC);
            const float *eg = sc + CH, *rr = sc + 2 * CH, *bet = sc + 3 * CH;
            const int64_t ts = bos + (int64_t)c * CH;
            const int n = (int)min<int64_t>(CH, eos - ts);
            score_tile_t<KD>(w, Pt, Qs, Ks, sc, n);
            // dU~ = diag(r) K dh' + s P^T dO  (rows = tokens, this wave's columns)
            f32x4 du[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) du[rt] = zero4();
            // (operands read a stage ahead of their products, fenced so that the
            // scheduler keeps them there)
            {
                OpX kf[2][4];
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) kf[0][rt] = frag8<bf16, Swz<KROW, KeyBK>>(Ks, 16 * rt + n16, 8 * g * 2);
#pragma unroll
                for (int dp = 0; dp < DP; ++dp) {
                    if (dp + 1 < DP)
#pragma unroll
                        for (int rt = 0; rt < 4; ++rt)
                            kf[(dp + 1) & 1][rt] = frag8<bf16, Swz<KROW, KeyBK>>(Ks, 16 * rt + n16, (32 * (dp + 1) + 8 * g) * 2);
                    __builtin_amdgcn_sched_barrier(0);
                    const OpS hb = Ops<bf16>::split(dh[2 * dp], dh[2 * dp + 1]);
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt) du[rt] = mma(du[rt], kf[dp & 1][rt], hb);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            const OpX dob0 = kt_operand<bf16, DROW>(Ds, 16 * w, 0), dob1 = kt_operand<bf16, DROW>(Ds, 16 * w, 1);
            lds_barrier();  // score planes complete
            // gradient of this chunk's end state, for the chunk-local stage: hi, lo planes
            // of dh'^T (stored after the barrier: before it the copy waves use the memory path)
            if (!p.d_seg) {
                char *o = reinterpret_cast<char *>(p.dhs + ((int64_t)(cb + c) * p.Hv + hv) * KV);
                const int plane = KD * p.V * 2;
#pragma unroll
                for (int dp = 0; dp < DP; ++dp) {
                    bf16x4 hi0, lo0, hi1, lo1;
                    split4(dh[2 * dp], hi0, lo0);
                    split4(dh[2 * dp + 1], hi1, lo1);
                    const uint32_t off = (uint32_t)((col * KD + slot_base(2 * dp, g)) * 2);
                    *reinterpret_cast<bf16x8 *>(o + off) = cat(hi0, hi1);
                    *reinterpret_cast<bf16x8 *>(o + plane + off) = cat(lo0, lo1);
                }
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 pd = zero4();
#pragma unroll
                for (int ip = rt / 2; ip < 2; ++ip)
                    pd = mma(pd, frag_s<PROW>(Pt, PPLANE, 16 * rt + n16, (32 * ip + 4 * g) * 2), ip == 0 ? dob0 : dob1);
                const f32x4 r4 = *reinterpret_cast<const f32x4 *>(rr + 16 * rt + 4 * g);
                du[rt] = r4 * du[rt] + p.scale * pd;
            }
            // dX = T^T dU~ (T^T upper triangular)
            const OpS dus0 = Ops<bf16>::split(du[0], du[1]), dus1 = Ops<bf16>::split(du[2], du[3]);
            f32x4 dx[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                dx[rt] = zero4();
#pragma unroll
                for (int ip = rt / 2; ip < 2; ++ip)
                    dx[rt] = mma(dx[rt], kt_s_in<TB>(Tb, TB::PLANE, 16 * rt, ip), ip == 0 ? dus0 : dus1);
            }
            // dh = e_last dh' + Q^T diag(s e) dO - K^T diag(beta e) dX
            OpS edo[2], bdx[2];
            {
                f32x4 y[4], z[4];
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const int r0 = 16 * rt + 4 * g;
                    const f32x4 e4 = *reinterpret_cast<const f32x4 *>(eg + r0);
                    const f32x4 b4 = *reinterpret_cast<const f32x4 *>(bet + r0);
                    const f32x4 d4 = rows4<bf16, DROW>(Ds, 16 * rt, 16 * w);
#pragma unroll
                    for (int i = 0; i < 4; ++i) y[rt][i] = r0 + i < n ? p.scale * e4[i] * d4[i] : 0.f;
                    z[rt] = -(b4 * e4) * dx[rt];
                }
                edo[0] = Ops<bf16>::split(y[0], y[1]);
                edo[1] = Ops<bf16>::split(y[2], y[3]);
                bdx[0] = Ops<bf16>::split(z[0], z[1]);
                bdx[1] = Ops<bf16>::split(z[2], z[3]);
            }
            const float el = eg[CH - 1];
            {
                OpX qk[2][2][2];  // [stage][Q, K][ip]
                auto keys = [&](int dt, OpX (&d)[2][2]) {
                    const int c0 = 32 * (dt >> 1) + 4 * (dt & 1);
#pragma unroll
                    for (int ip = 0; ip < 2; ++ip) {
                        d[0][ip] = kt_keys<KROW>(Qs, c0, ip);
                        d[1][ip] = kt_keys<KROW>(Ks, c0, ip);
                    }
                };
                keys(0, qk[0]);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    if (dt + 1 < DT) keys(dt + 1, qk[(dt + 1) & 1]);
                    __builtin_amdgcn_sched_barrier(0);
                    dh[dt] *= el;
#pragma unroll
                    for (int ip = 0; ip < 2; ++ip) {
                        dh[dt] = mma(dh[dt], qk[dt & 1][0][ip], edo[ip]);
                        dh[dt] = mma(dh[dt], qk[dt & 1][1][ip], bdx[ip]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            lds_barrier();  // chunk c done with its tiles and the score planes; c - 1 landed
        };
        __syncthreads();  // first chunk landed
        for (int c = c_end - 1; c >= c_begin; c -= 2) {
            body(std::integral_constant<int, 0>{}, c);
            if (c - 1 >= c_begin) body(std::integral_constant<int, 1>{}, c - 1);
        }
        float *dh_out = p.d_seg ? p.d_seg + ((int64_t)unit * p.n_seg + seg) * KV
                        : c_begin == 0 && p.dh0 ? p.dh0 + unit * KV : nullptr;
        if (dh_out) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) dh_out[(slot_base(dt, g) + i) * p.V + col] = dh[dt][i];
        }
    } else if (wv < 4 + NCP) {
        // ------------------------------------------------------------- copy waves
        const int iw = wv - 4;
        const char *kp = reinterpret_cast<const char *>(p.k), *qp = reinterpret_cast<const char *>(p.q);
        const char *dop = reinterpret_cast<const char *>(p.dout);
        // the K tile of a chunk (part 0), then its Q and dO tiles and T block (part 1)
        auto issue = [&](int part, int c, char *K_, char *Q_, char *D_, char *T_) {
            const int64_t ts = bos + (int64_t)c * CH;
            const int n = (int)min<int64_t>(CH, eos - ts);
            if (part == 0) {
                copy_rows<KROW, KeyBK>(K_, kp + (ts * p.Hq + hq) * KROW, p.Hq * KROW, n - 1, iw, NCP);
            } else {
                copy_rows<KROW, KeyBK>(Q_, qp + (ts * p.Hq + hq) * KROW, p.Hq * KROW, n - 1, iw, NCP);
                copy_rows<DROW>(D_, dop + ((ts * p.Hv + hv) * p.V + vt * 64) * 2, p.Hv * p.V * 2, n - 1, iw, NCP);
                copy_bytes(T_, p.tblk + ((int64_t)(cb + c) * p.Hv + hv) * TB::BYTES, TB::BYTES, iw, NCP);
            }
        };
        // the next chunk's K tile is issued before the mid-chunk barrier and the rest
        // after it, so that these waves reach it as early as the others
        auto body = [&](auto cur, int c) {
            constexpr bool ONE = decltype(cur)::value == 1;
            const bool more = c - 1 >= c_begin;
            if (more) {
                if constexpr (ONE)
                    issue(0, c - 1, Ks0, Qs0, Ds0, Tb0);
                else
                    issue(0, c - 1, Ks1, Qs1, Ds1, Tb1);
            }
            lds_barrier();  // score planes complete
            if (more) {
                if constexpr (ONE)
                    issue(1, c - 1, Ks0, Qs0, Ds0, Tb0);
                else
                    issue(1, c - 1, Ks1, Qs1, Ds1, Tb1);
            }
            wait_dma();
            lds_barrier();  // chunk c done with its tiles and the score planes; c - 1 landed
        };
        if (c_end > c_begin) {
            issue(0, c_end - 1, Ks0, Qs0, Ds0, Tb0);
            issue(1, c_end - 1, Ks0, Qs0, Ds0, Tb0);
        }
        wait_dma();
        __syncthreads();  // first chunk landed
        for (int c = c_end - 1; c >= c_begin; c -= 2) {
            body(std::integral_constant<int, 0>{}, c);
            if (c - 1 >= c_begin) body(std::integral_constant<int, 1>{}, c - 1);
        }
    } else {
        // ------------------------------------------------------------ score waves
        const int iw = wv - 4 - NCP;  // tiles 4 + iw, 6 + iw, 8 + iw
        auto body = [&](auto cur, int c) {
            constexpr bool ONE = decltype(cur)::value == 1;
            const char *Ks = ONE ? Ks1 : Ks0, *Qs = ONE ? Qs1 : Qs0, *Tb = ONE ? Tb1 : Tb0;
            const float *sc = reinterpret_cast<const float *>(Tb + TB::SC);
            const int64_t ts = bos + (int64_t)c * CH;
            const int n = (int)min<int64_t>(CH, eos - ts);
#pragma unroll
            for (int k = 0; k < 3; ++k) score_tile_t<KD>(4 + iw + 2 * k, Pt, Qs, Ks, sc, n);
            lds_barrier();  // score planes complete
            lds_barrier();  // chunk c done with its tiles and the score planes; c - 1 landed
        };
        __syncthreads();  // first chunk landed
        for (int c = c_end - 1; c >= c_begin; c -= 2) {
            body(std::integral_constant<int, 0>{}, c);
            if (c - 1 >= c_begin) body(std::integral_constant<int, 1>{}, c - 1);
        }
    }
}

}  // namespace

hipError_t launch_bwd_scan_bf16(int K, const BwdParams &p, int n_units, hipStream_t s) {
    const dim3 grid(p.sm.order && p.n_seg == 1 ? lpt_blocks(p.sm.n_seq, p.Hq, p.Hv, p.V / 64)
                                               : n_units * (p.V / 64) * p.n_seg);
    if (K == 128)
        launch_k((bwd_scan_roles_bf16<128>), grid, dim3(2 * NTHR), 0, s, p, n_units);
    else
        launch_k((bwd_scan_roles_bf16<64>), grid, dim3(2 * NTHR), 0, s, p, n_units);
    return hipGetLastError();
}


}  // namespace gdr
