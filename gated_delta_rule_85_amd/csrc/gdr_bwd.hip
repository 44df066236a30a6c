// Backward of the chunked gated delta rule: gradients of <dout, o> +
// <dht, final_state> with respect to q, k, v, beta, g and the initial state
// (the low-level chunk_gated_delta_rule_bwd of the PyPI README, "Usage").
//
// Per chunk, with gam the in-chunk cumulative log-gate, e = exp(gam),
// r = exp(gam_last - gam), Gam[r][i] = exp(gam_r - gam_i), T = (I + A)^{-1},
// the forward is
//   X  = diag(beta) (V - diag(e) K h),   U~ = T X
//   P  = (Q K^T * Gam) on i <= r,        O  = s (diag(e) Q h + P U~)
//   h' = e_last h + K^T diag(r) U~
// so, given dO and the end-state gradient dh',
//   dU~ = diag(r) K dh' + s P^T dO,      dX = T^T dU~
//   dh  = e_last dh' + s Q^T diag(e) dO - K^T diag(beta e) dX
// runs backwards over chunks (the reverse scan), and the chunk-local terms are
//   dP = s dO U~^T,  dT = dU~ X^T,  dA = -(T^T dT T^T) on i < r,  dS = diag(beta)(dA * Gam)
//   dq = s diag(e) dO h^T + (dP * Gam) K
//   dk = diag(r) U~ dh'^T + (dP * Gam)^T Q + (dS + dS^T) K - diag(beta e) dX h^T
//   dv = diag(beta) dX
//   dbeta = rowsum(dA * K K^T * Gam) + rowsum(dX * (V - diag(e) K h))
//   dgam  = e (s rowsum(dO * Q h) - beta rowsum(dX * K h)) + rowsum(Z) - colsum(Z)
//           - r rowsum(U~ * K dh'),  Z = dP * P + dA * A,
//           and on the last row also e_last <dh', h> + sum_i r_i rowsum(U~ * K dh')_i
//   dg  = in-chunk reverse running sum of dgam.
//
// Stages: the T blocks are rebuilt from A, the forward scan re-creates the
// chunk-start states (its states-only mode), bwd_scan_kernel runs the
// reverse scan per (sequence, v head, 64 value columns) with dh in registers
// and stores every chunk's end-state gradient, and bwd_local_kernel forms
// the chunk-local gradients per (chunk, q/k head), summing dq and dk over
// the head's v heads in registers.  Products use fp32 MFMA
// (v_mfma_f32_16x16x4_f32) on LDS-resident matrices.
#include "gdr_kernels.hpp"

namespace gdr {

namespace {

// acc (16x16 tile at (m0, n0)) += sum_k a(m0+i, k) b(k, n0+j), k < kd (multiple of 16).
// Output in accumulator order: lane (n, g) holds rows m0+4g+i, column n0+n.
template <class FA, class FB>
__device__ __forceinline__ f32x4 tile_f32(f32x4 acc, const FA &a, const FB &b, int m0, int n0, int kd) {
    const int n = ln16(), g = lg4();
#pragma unroll 1
    for (int k0 = 0; k0 < kd; k0 += 16) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a(m0 + n, k0 + 4 * g + j), b(k0 + 4 * g + j, n0 + n),
                                                       acc, 0, 0, 0);
    }
    return acc;
}

// acc += a(m0 + i, k) B(k, :) with B held in registers as accumulator tiles:
// b[kb] holds rows 16 kb .. 16 kb + 15 of B in this lane's column
template <class FA, int NK>
__device__ __forceinline__ f32x4 tile_rb(f32x4 acc, const FA &a, int m0, const f32x4 (&b)[NK]) {
    const int n = ln16(), g = lg4();
#pragma unroll
    for (int kb = 0; kb < NK; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a(m0 + n, 16 * kb + 4 * g + j), b[kb][j], acc, 0, 0, 0);
    return acc;
}

// LDS matrix views
struct RowF {  // row-major fp32
    const float *p;
    int ld;
    __device__ __forceinline__ float operator()(int r, int c) const { return p[r * ld + c]; }
};
struct ColF {  // transposed view of a row-major fp32 matrix
    const float *p;
    int ld;
    __device__ __forceinline__ float operator()(int r, int c) const { return p[c * ld + r]; }
};
template <typename In> struct RowI {
    const In *p;
    int ld;
    __device__ __forceinline__ float operator()(int r, int c) const { return to_f32(p[r * ld + c]); }
};
template <typename In> struct ColI {
    const In *p;
    int ld;
    __device__ __forceinline__ float operator()(int r, int c) const { return to_f32(p[c * ld + r]); }
};

__device__ __forceinline__ void put_tile(float *C, int ld, int m0, int n0, f32x4 acc) {
    const int n = ln16(), g = lg4();
#pragma unroll
    for (int i = 0; i < 4; ++i) C[(m0 + 4 * g + i) * ld + n0 + n] = acc[i];
}

template <typename In> __device__ __forceinline__ In from_f32(float x) { return static_cast<In>(x); }

constexpr int LF = 65;  // fp32 rows of 64 (+1 against bank conflicts)

// gate scalars of one (chunk, v head): gam (padded with its last value), e, r, beta (0 past the end)
__device__ __forceinline__ void load_gates(const BwdParams &p, int64_t ts, int n, int hv, float *gam, float *eg,
                                           float *rr, float *bet) {
    const int t = threadIdx.x;
    if (t < CH) {
        const float gr = p.g_cum[(ts + min(t, n - 1)) * p.Hv + hv];
        const float gl = p.g_cum[(ts + n - 1) * p.Hv + hv];
        gam[t] = gr;
        eg[t] = fast_exp(gr);
        rr[t] = fast_exp(gl - gr);
        bet[t] = t < n ? p.beta[(ts + t) * p.Hv + hv] : 0.f;
    }
}

// T rows of one (chunk, v head), zero past the chunk end.  Every load is
// issued before the first LDS write (rows past the end read the last row and
// are zeroed), so the tile costs one memory round trip.
__device__ __forceinline__ void load_T(const BwdParams &p, int64_t ts, int n, int hv, float *Tf) {
    constexpr int PER = CH * CH / 4 / NTHR;
    static_assert(CH * CH / 4 % NTHR == 0, "16-byte pieces spread evenly");
    f32x4 v[PER];
#pragma unroll
    for (int it = 0; it < PER; ++it) {
        const int idx = threadIdx.x + it * NTHR, r = idx >> 4, c4 = idx & 15;
        v[it] = *reinterpret_cast<const f32x4 *>(p.A + ((ts + min(r, n - 1)) * p.Hv + hv) * CH + 4 * c4);
    }
#pragma unroll
    for (int it = 0; it < PER; ++it) {
        const int idx = threadIdx.x + it * NTHR, r = idx >> 4, c4 = idx & 15;
        const f32x4 x = r < n ? v[it] : zero4();
#pragma unroll
        for (int e = 0; e < 4; ++e) Tf[r * LF + 4 * c4 + e] = x[e];  // (odd pitch: scalar LDS writes)
    }
}

// ------------------------------------------------------------------ T blocks
// The T blocks, rebuilt from the forward's A rows and g_cum: the compact form the
// forward writes for bf16 inputs, full rows for the fp32 kernels.
template <typename In>
__global__ __launch_bounds__(NTHR) void tblock_kernel(const BwdParams p) {
    __shared__ float Tf[CH * LF];
    __shared__ float gam[CH], eg[CH], rr[CH], bet[CH];
    const int gid = blockIdx.x, hv = blockIdx.y;
    int j, c;
    if (!p.sm.locate(gid, j, c)) return;
    int64_t bos, eos;
    p.sm.bounds(j, bos, eos);
    const int64_t ts = bos + (int64_t)c * CH;
    const int n = (int)min<int64_t>(CH, eos - ts);
    load_T(p, ts, n, hv, Tf);
    load_gates(p, ts, n, hv, gam, eg, rr, bet);
    __syncthreads();
    if constexpr (sizeof(In) == 2)  // the compact block the bf16 kernels read
        write_tblock_f<In>(p.tblk + ((int64_t)gid * p.Hv + hv) * TBlockF<In>::BYTES, Tf, LF, gam, bet, n,
                           threadIdx.x, NTHR);
    else
        write_tblock<In>(p.tblk + ((int64_t)gid * p.Hv + hv) * TBlock<In>::BYTES, Tf, LF, gam, bet, n,
                         threadIdx.x, NTHR);
}

// ------------------------------------------------------------- reverse scan
// One workgroup per (sequence, v head, 64 value columns); wave w owns columns
// 16 w .. 16 w + 15 of the tile and keeps its K x 16 slice of dh in registers.
template <typename In, int KD>
__global__ __launch_bounds__(NTHR) void bwd_scan_kernel(const BwdParams p, int n_units) {
    constexpr int LK = KD + 2;
    constexpr int NK = KD / 16;
    __shared__ In Ks[CH * LK], Qs[CH * LK];
    __shared__ float Tf[CH * LF], Pf[CH * LF], DOs[CH * LF];
    __shared__ float gam[CH], eg[CH], rr[CH], bet[CH];

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
    const int w = wave_id(), nn = ln16(), g = lg4();
    const int col = vt * 64 + 16 * w + nn;  // this lane's value column
    int64_t bos, eos;
    p.sm.bounds(j, bos, eos);
    const int N = (int)((eos - bos + CH - 1) / CH);
    // this workgroup's segment of chunks (the whole sequence without a split)
    const int c_begin = seg * p.seg_chunks;
    if (c_begin >= N && !(N == 0 && seg == 0)) return;
    const int c_end = min(N, c_begin + p.seg_chunks);
    const int cb = p.sm.chunk_base(j);
    const int64_t KV = (int64_t)KD * p.V;
    const float *dh_start = c_end == N ? (p.dht ? p.dht + unit * KV : nullptr)
                            : p.d_seg ? nullptr
                                      : p.dh_seg + ((int64_t)unit * p.n_seg + seg) * KV;
    const In *qp = reinterpret_cast<const In *>(p.q), *kp = reinterpret_cast<const In *>(p.k);
    const In *dop = reinterpret_cast<const In *>(p.dout);

    f32x4 dh[NK];  // rows 16 kb + 4 g + i of dh, column col
#pragma unroll
    for (int kb = 0; kb < NK; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dh[kb][i] = dh_start ? dh_start[(16 * kb + 4 * g + i) * p.V + col] : 0.f;

    for (int c = c_end - 1; c >= c_begin; --c) {
        const int64_t ts = bos + (int64_t)c * CH;
        const int n = (int)min<int64_t>(CH, eos - ts);
        __syncthreads();  // previous chunk done with the LDS tiles
        for (int idx = threadIdx.x; idx < CH * KD; idx += NTHR) {
            const int r = idx / KD, d = idx % KD;
            const bool ok = r < n;
            Ks[r * LK + d] = ok ? kp[((ts + r) * p.Hq + hq) * KD + d] : In(0.f);
            Qs[r * LK + d] = ok ? qp[((ts + r) * p.Hq + hq) * KD + d] : In(0.f);
        }
        for (int idx = threadIdx.x; idx < CH * 64; idx += NTHR) {
            const int r = idx >> 6, cc = idx & 63;
            DOs[r * LF + cc] = r < n ? to_f32(dop[((ts + r) * p.Hv + hv) * p.V + vt * 64 + cc]) : 0.f;
        }
        load_T(p, ts, n, hv, Tf);
        load_gates(p, ts, n, hv, gam, eg, rr, bet);
        if (!p.d_seg) {  // gradient of this chunk's end state, for the chunk-local stage
            float *o = p.dhs + ((int64_t)(cb + c) * p.Hv + hv) * KV;
#pragma unroll
            for (int kb = 0; kb < NK; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[(16 * kb + 4 * g + i) * p.V + col] = dh[kb][i];
        }
        __syncthreads();
        // P = (Q K^T * Gam) on i <= r: tiles w, w+4, w+8, w+12
        for (int t = w; t < 16; t += 4) {
            const int m0 = 16 * (t >> 2), n0 = 16 * (t & 3);
            const f32x4 acc = tile_f32(zero4(), RowI<In>{Qs, LK}, ColI<In>{Ks, LK}, m0, n0, KD);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = m0 + 4 * g + i, ci = n0 + nn;
                Pf[r * LF + ci] = ci <= r ? acc[i] * fast_exp(gam[r] - gam[ci]) : 0.f;
            }
        }
        __syncthreads();
        // dU~ = diag(r) K dh' + s P^T dO ;  dX = T^T dU~
        f32x4 du[4], dx[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const f32x4 kdh = tile_rb(zero4(), RowI<In>{Ks, LK}, 16 * rt, dh);
            const f32x4 pdo = tile_f32(zero4(), ColF{Pf, LF}, RowF{DOs, LF}, 16 * rt, 16 * w, CH);
#pragma unroll
            for (int i = 0; i < 4; ++i) du[rt][i] = rr[16 * rt + 4 * g + i] * kdh[i] + p.scale * pdo[i];
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) dx[rt] = tile_rb(zero4(), ColF{Tf, LF}, 16 * rt, du);
        // dh = e_last dh' + s Q^T diag(e) dO - K^T diag(beta e) dX
        f32x4 bedx[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * rt + 4 * g + i;
                bedx[rt][i] = -bet[r] * eg[r] * dx[rt][i];
            }
        struct EDO {
            const float *d, *e;
            __device__ float operator()(int r, int c) const { return e[r] * d[r * LF + c]; }
        };
        const float el = eg[CH - 1];
#pragma unroll
        for (int kb = 0; kb < NK; ++kb) {
            const f32x4 a = tile_f32(zero4(), ColI<In>{Qs, LK}, EDO{DOs, eg}, 16 * kb, 16 * w, CH);
            const f32x4 nd = el * dh[kb] + p.scale * a;
            dh[kb] = tile_rb(nd, ColI<In>{Ks, LK}, 16 * kb, bedx);
        }
    }
    float *dh_out = p.d_seg ? p.d_seg + ((int64_t)unit * p.n_seg + seg) * KV
                    : c_begin == 0 && p.dh0 ? p.dh0 + unit * KV : nullptr;
    if (dh_out) {
#pragma unroll
        for (int kb = 0; kb < NK; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) dh_out[(16 * kb + 4 * g + i) * p.V + col] = dh[kb][i];
    }
}

// ------------------------------------------------------- chunk-local terms
// One workgroup per (chunk, q/k head); its v heads in turn, the value
// dimension in blocks of 16 columns.
template <typename In, typename Gt, int KD>
__global__ __launch_bounds__(NTHR) void bwd_local_kernel(const BwdParams p) {
    constexpr int LK = KD + 2;
    constexpr int VB = 16, LB = VB + 1;
    constexpr int NKT = KD / 16;  // column tiles of a 64 x KD matrix
    constexpr int PW = NKT;       // of its 4 NKT tiles, per wave
    constexpr int BLK0 = 2 * KD * LB + 9 * CH * LB, BLK = BLK0 > 3 * CH * LF ? BLK0 : 3 * CH * LF;
    __shared__ In Ks[CH * LK], Qs[CH * LK];
    __shared__ float Tf[CH * LF], Pf[CH * LF];
    __shared__ float blk[BLK];  // per value block; three 64 x 64 matrices afterwards
    __shared__ float gam[CH], eg[CH], rr[CH], bet[CH], dea[CH], deb[CH], drr[CH], dbx[CH], dgm[CH];
    __shared__ float red[NTHR / 64];

    const int gid = blockIdx.x, hq = blockIdx.y, tid = threadIdx.x, w = wave_id();
    int j, c;
    if (!p.sm.locate(gid, j, c)) return;
    int64_t bos, eos;
    p.sm.bounds(j, bos, eos);
    const int64_t ts = bos + (int64_t)c * CH;
    const int n = (int)min<int64_t>(CH, eos - ts);
    const int G = p.Hv / p.Hq;
    const int64_t KV = (int64_t)KD * p.V;
    const In *qp = reinterpret_cast<const In *>(p.q), *kp = reinterpret_cast<const In *>(p.k);
    const In *vp = reinterpret_cast<const In *>(p.v), *dop = reinterpret_cast<const In *>(p.dout);
    Gt *dvp = reinterpret_cast<Gt *>(p.dv);
    const int nn = ln16(), g = lg4();

    float *Hb = blk, *DHb = Hb + KD * LB, *Vb = DHb + KD * LB, *DOb = Vb + CH * LB, *Khb = DOb + CH * LB;
    float *Yb = Khb + CH * LB, *Qhb = Yb + CH * LB, *Ub = Qhb + CH * LB, *Kdhb = Ub + CH * LB;
    float *DUb = Kdhb + CH * LB, *DXb = DUb + CH * LB;
    float *W1 = blk, *W2 = W1 + CH * LF, *W3 = W2 + CH * LF;

    for (int idx = tid; idx < CH * KD; idx += NTHR) {
        const int r = idx / KD, d = idx % KD;
        const bool ok = r < n;
        Ks[r * LK + d] = ok ? kp[((ts + r) * p.Hq + hq) * KD + d] : In(0.f);
        Qs[r * LK + d] = ok ? qp[((ts + r) * p.Hq + hq) * KD + d] : In(0.f);
    }
    // dq, dk of this q/k head, summed over its v heads (tile t = w + 4 s)
    f32x4 dqa[PW], dka[PW];
#pragma unroll
    for (int s = 0; s < PW; ++s) dqa[s] = dka[s] = zero4();

    for (int gi = 0; gi < G; ++gi) {
        const int hv = hq * G + gi;
        __syncthreads();  // previous v head done with every LDS array
        load_T(p, ts, n, hv, Tf);
        load_gates(p, ts, n, hv, gam, eg, rr, bet);
        if (tid < CH) dea[tid] = deb[tid] = drr[tid] = dbx[tid] = 0.f;
        __syncthreads();
        for (int t = w; t < 16; t += 4) {  // P = (Q K^T * Gam) on i <= r
            const int m0 = 16 * (t >> 2), n0 = 16 * (t & 3);
            const f32x4 acc = tile_f32(zero4(), RowI<In>{Qs, LK}, ColI<In>{Ks, LK}, m0, n0, KD);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = m0 + 4 * g + i, ci = n0 + nn;
                Pf[r * LF + ci] = ci <= r ? acc[i] * fast_exp(gam[r] - gam[ci]) : 0.f;
            }
        }
        // products contracted over the value dimension
        f32x4 aP[4], aT[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) aP[s] = aT[s] = zero4();
        float dec = 0.f;  // this thread's share of <dh', h>
        const int64_t hoff = ((int64_t)gid * p.Hv + hv) * KV;

        for (int vb = 0; vb < p.V; vb += VB) {
            __syncthreads();
            for (int idx = tid; idx < KD * VB; idx += NTHR) {
                const int d = idx / VB, cc = idx % VB;
                const float hx = p.hs[hoff + d * p.V + vb + cc], dhx = p.dhs[hoff + d * p.V + vb + cc];
                Hb[d * LB + cc] = hx;
                DHb[d * LB + cc] = dhx;
                dec += hx * dhx;
            }
            for (int idx = tid; idx < CH * VB; idx += NTHR) {
                const int r = idx / VB, cc = idx % VB;
                const bool ok = r < n;
                Vb[r * LB + cc] = ok ? to_f32(vp[((ts + r) * p.Hv + hv) * p.V + vb + cc]) : 0.f;
                DOb[r * LB + cc] = ok ? to_f32(dop[((ts + r) * p.Hv + hv) * p.V + vb + cc]) : 0.f;
            }
            __syncthreads();
            const int m0 = 16 * w;  // this wave's 16 token rows
            {  // K h, Q h, K dh'
                const f32x4 kh = tile_f32(zero4(), RowI<In>{Ks, LK}, RowF{Hb, LB}, m0, 0, KD);
                const f32x4 qh = tile_f32(zero4(), RowI<In>{Qs, LK}, RowF{Hb, LB}, m0, 0, KD);
                const f32x4 kd = tile_f32(zero4(), RowI<In>{Ks, LK}, RowF{DHb, LB}, m0, 0, KD);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = m0 + 4 * g + i;
                    Khb[r * LB + nn] = kh[i];
                    Yb[r * LB + nn] = Vb[r * LB + nn] - eg[r] * kh[i];
                    Qhb[r * LB + nn] = qh[i];
                    Kdhb[r * LB + nn] = kd[i];
                }
            }
            __syncthreads();
            struct BY {  // X = diag(beta) Y
                const float *y, *b;
                __device__ float operator()(int r, int c) const { return b[r] * y[r * LB + c]; }
            };
            put_tile(Ub, LB, m0, 0, tile_f32(zero4(), RowF{Tf, LF}, BY{Yb, bet}, m0, 0, CH));
            {  // dU~ = diag(r) K dh' + s P^T dO on this wave's rows
                const f32x4 a2 = tile_f32(zero4(), ColF{Pf, LF}, RowF{DOb, LB}, m0, 0, CH);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = m0 + 4 * g + i;
                    DUb[r * LB + nn] = rr[r] * Kdhb[r * LB + nn] + p.scale * a2[i];
                }
            }
            __syncthreads();
            {  // dX = T^T dU~ ; dv = diag(beta) dX
                const f32x4 dx = tile_f32(zero4(), ColF{Tf, LF}, RowF{DUb, LB}, m0, 0, CH);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = m0 + 4 * g + i;
                    DXb[r * LB + nn] = dx[i];
                    if (r < n) dvp[((ts + r) * p.Hv + hv) * p.V + vb + nn] = from_f32<Gt>(bet[r] * dx[i]);
                }
            }
            __syncthreads();
            struct BYT {  // X^T
                const float *y, *b;
                __device__ float operator()(int r, int c) const { return b[c] * y[c * LB + r]; }
            };
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int t = w + 4 * s, r0 = 16 * (t >> 2), c0 = 16 * (t & 3);
                aP[s] = tile_f32(aP[s], RowF{DOb, LB}, ColF{Ub, LB}, r0, c0, VB);
                aT[s] = tile_f32(aT[s], RowF{DUb, LB}, BYT{Yb, bet}, r0, c0, VB);
            }
            // dq += s diag(e) dO h^T ;  dk += diag(r) U~ dh'^T - diag(beta e) dX h^T
            struct Scaled {
                const float *m, *a, *b;
                float c;
                __device__ float operator()(int r, int k) const { return c * a[r] * (b ? b[r] : 1.f) * m[r * LB + k]; }
            };
#pragma unroll
            for (int s = 0; s < PW; ++s) {
                const int t = w + 4 * s, r0 = 16 * (t / NKT), c0 = 16 * (t % NKT);
                dqa[s] = tile_f32(dqa[s], Scaled{DOb, eg, nullptr, p.scale}, ColF{Hb, LB}, r0, c0, VB);
                dka[s] = tile_f32(dka[s], Scaled{Ub, rr, nullptr, 1.f}, ColF{DHb, LB}, r0, c0, VB);
                dka[s] = tile_f32(dka[s], Scaled{DXb, bet, eg, -1.f}, ColF{Hb, LB}, r0, c0, VB);
            }
            if (tid < CH) {
                const int r = tid;
                float s1 = 0.f, s2 = 0.f, s3 = 0.f, s4 = 0.f;
#pragma unroll
                for (int cc = 0; cc < VB; ++cc) {
                    s1 += DOb[r * LB + cc] * Qhb[r * LB + cc];
                    s2 += DXb[r * LB + cc] * Khb[r * LB + cc];
                    s3 += Ub[r * LB + cc] * Kdhb[r * LB + cc];
                    s4 += DXb[r * LB + cc] * Yb[r * LB + cc];
                }
                dea[r] += s1;
                deb[r] -= bet[r] * s2;
                drr[r] += s3;
                dbx[r] += s4;
            }
        }
        // <dh', h> over the workgroup
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) dec += __shfl_xor(dec, off, 64);
        if (lane_id() == 0) red[w] = dec;
        __syncthreads();
        const float deC = red[0] + red[1] + red[2] + red[3];
        // W1 = dP * Gam on i <= r;  Pf <- dP * P;  W2 = dT
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int t = w + 4 * s, r0 = 16 * (t >> 2), c0 = 16 * (t & 3);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = r0 + 4 * g + i, ci = c0 + nn;
                const float dP = p.scale * aP[s][i];
                W1[r * LF + ci] = ci <= r ? dP * fast_exp(gam[r] - gam[ci]) : 0.f;
                Pf[r * LF + ci] *= dP;
                W2[r * LF + ci] = aT[s][i];
            }
        }
        __syncthreads();
        for (int t = w; t < 16; t += 4) {  // W3 = T^T dT
            const int r0 = 16 * (t >> 2), c0 = 16 * (t & 3);
            put_tile(W3, LF, r0, c0, tile_f32(zero4(), ColF{Tf, LF}, RowF{W2, LF}, r0, c0, CH));
        }
        __syncthreads();
        for (int t = w; t < 16; t += 4) {  // W2 = dA = -(T^T dT T^T) on i < r
            const int r0 = 16 * (t >> 2), c0 = 16 * (t & 3);
            const f32x4 acc = tile_f32(zero4(), RowF{W3, LF}, ColF{Tf, LF}, r0, c0, CH);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = r0 + 4 * g + i, ci = c0 + nn;
                W2[r * LF + ci] = ci < r ? -acc[i] : 0.f;
            }
        }
        __syncthreads();
        for (int t = w; t < 16; t += 4) {  // W3 = S = K K^T
            const int r0 = 16 * (t >> 2), c0 = 16 * (t & 3);
            put_tile(W3, LF, r0, c0, tile_f32(zero4(), RowI<In>{Ks, LK}, ColI<In>{Ks, LK}, r0, c0, KD));
        }
        __syncthreads();
        if (tid < CH) {
            // row and column sums of Z = dP * P + dA * A (A = diag(beta) S * Gam); dbeta through A
            const int r = tid;
            float zr = 0.f, zc = 0.f, dba = 0.f;
            for (int i = 0; i < CH; ++i) {
                zr += Pf[r * LF + i];
                zc += Pf[i * LF + r];
                if (i < r) dba += W2[r * LF + i] * W3[r * LF + i] * fast_exp(gam[r] - gam[i]);
                if (i > r) zc += W2[i * LF + r] * bet[i] * W3[i * LF + r] * fast_exp(gam[i] - gam[r]);
            }
            zr += bet[r] * dba;
            dgm[r] = zr - zc;
            dbx[r] += dba;
        }
        __syncthreads();
        for (int idx = tid; idx < CH * CH; idx += NTHR) {  // W2 <- dS = diag(beta) (dA * Gam)
            const int r = idx >> 6, i = idx & 63;
            W2[r * LF + i] = i < r ? bet[r] * W2[r * LF + i] * fast_exp(gam[r] - gam[i]) : 0.f;
        }
        __syncthreads();
        struct SymS {  // dS + dS^T
            const float *d;
            __device__ float operator()(int r, int c) const { return d[r * LF + c] + d[c * LF + r]; }
        };
#pragma unroll
        for (int s = 0; s < PW; ++s) {
            const int t = w + 4 * s, r0 = 16 * (t / NKT), c0 = 16 * (t % NKT);
            const f32x4 dqc = tile_f32(zero4(), RowF{W1, LF}, RowI<In>{Ks, LK}, r0, c0, CH);
            const f32x4 dkc = tile_f32(zero4(), ColF{W1, LF}, RowI<In>{Qs, LK}, r0, c0, CH);
            const f32x4 dks = tile_f32(zero4(), SymS{W2}, RowI<In>{Ks, LK}, r0, c0, CH);
            dqa[s] += dqc;
            dka[s] += dkc + dks;
        }
        // dgam -> dg (reverse running sum over the chunk), dbeta
        if (w == 0) {
            const int r = lane_id();
            float x = 0.f;
            if (r < n) {
                x = eg[r] * (p.scale * dea[r] + deb[r]) + dgm[r] - rr[r] * drr[r];
                if (r == n - 1) {
                    float srd = 0.f;
                    for (int i = 0; i < n; ++i) srd += rr[i] * drr[i];
                    x += eg[r] * deC + srd;
                }
            }
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_down(x, off, 64);
                if (r + off < 64) x += y;
            }
            if (r < n) {
                p.dg[(ts + r) * p.Hv + hv] = x;
                p.dbeta[(ts + r) * p.Hv + hv] = dbx[r];
            }
        }
    }
    Gt *dq = reinterpret_cast<Gt *>(p.dq), *dk = reinterpret_cast<Gt *>(p.dk);
#pragma unroll
    for (int s = 0; s < PW; ++s) {
        const int t = w + 4 * s, r0 = 16 * (t / NKT), c0 = 16 * (t % NKT);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = r0 + 4 * g + i;
            if (r < n) {
                const int64_t o = ((ts + r) * p.Hq + hq) * KD + c0 + nn;
                dq[o] = from_f32<Gt>(dqa[s][i]);
                dk[o] = from_f32<Gt>(dka[s][i]);
            }
        }
    }
}

template <typename In, typename Gt, int KD>
hipError_t launch_bwd_t(const BwdParams &p, int n_chunks_ub, int n_units, const hipEvent_t *ev, hipStream_t s) {
    hipError_t e;
    if constexpr (sizeof(In) == 2) {
        e = launch_bwd_scan_bf16(KD, p, n_units, s);
    } else {
        launch_k((bwd_scan_kernel<In, KD>),
                           dim3(p.sm.order && p.n_seg == 1 ? lpt_blocks(p.sm.n_seq, p.Hq, p.Hv, p.V / 64)
                                                           : n_units * (p.V / 64) * p.n_seg),
                           dim3(NTHR), 0, s, p, n_units);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    if ((e = close_stage(s)) != hipSuccess) return e;  // the reverse scan's stage
    open_stage(ev ? ev[0] : nullptr, ev ? ev[1] : nullptr);
    if (n_chunks_ub > 0) {
        if constexpr (sizeof(In) == 2) {
            e = launch_bwd_local_bf16(sizeof(Gt) == 2 ? Dt::BF16 : Dt::F32, KD, p, n_chunks_ub, s);
        } else {
            launch_k((bwd_local_kernel<In, Gt, KD>), dim3(n_chunks_ub, p.Hq), dim3(NTHR), 0, s, p);
            e = hipGetLastError();
        }
        if (e != hipSuccess) return e;
    }
    return close_stage(s);
}

template <typename In, typename Gt>
hipError_t launch_bwd_k(int K, const BwdParams &p, int n_chunks_ub, int n_units, const hipEvent_t *ev,
                        hipStream_t s) {
    return K == 128 ? launch_bwd_t<In, Gt, 128>(p, n_chunks_ub, n_units, ev, s)
                    : launch_bwd_t<In, Gt, 64>(p, n_chunks_ub, n_units, ev, s);
}

}  // namespace

hipError_t launch_tblocks(Dt dt, const BwdParams &p, int n_chunks_ub, hipStream_t s) {
    const dim3 grid(n_chunks_ub, p.Hv);
    if (dt == Dt::BF16)
        launch_k(tblock_kernel<bf16>, grid, dim3(NTHR), 0, s, p);
    else
        launch_k(tblock_kernel<float>, grid, dim3(NTHR), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_bwd_reverse(Dt dt, int K, const BwdParams &p, int n_units, hipStream_t s) {
    if (dt == Dt::BF16) return launch_bwd_scan_bf16(K, p, n_units, s);
    const dim3 grid(p.sm.order && p.n_seg == 1 ? lpt_blocks(p.sm.n_seq, p.Hq, p.Hv, p.V / 64)
                                               : n_units * (p.V / 64) * p.n_seg);
    if (K == 128)
        launch_k((bwd_scan_kernel<float, 128>), grid, dim3(NTHR), 0, s, p, n_units);
    else
        launch_k((bwd_scan_kernel<float, 64>), grid, dim3(NTHR), 0, s, p, n_units);
    return hipGetLastError();
}

hipError_t launch_bwd(Dt dt, Dt gt, int K, const BwdParams &p, int n_chunks_ub, int n_units,
                      const hipEvent_t *ev, hipStream_t s) {
    if (dt == Dt::BF16)
        return gt == Dt::BF16 ? launch_bwd_k<bf16, bf16>(K, p, n_chunks_ub, n_units, ev, s)
                              : launch_bwd_k<bf16, float>(K, p, n_chunks_ub, n_units, ev, s);
    return gt == Dt::BF16 ? launch_bwd_k<float, bf16>(K, p, n_chunks_ub, n_units, ev, s)
                          : launch_bwd_k<float, float>(K, p, n_chunks_ub, n_units, ev, s);
}

}  // namespace gdr
