// Backward kernels for bf16 inputs on bf16 MFMA (v_mfma_f32_16x16x32_bf16).
//
// The same adjoint as gdr_bwd.hip (which holds the fp32-input kernels and
// the derivation), arranged for the matrix cores: q, k, v, do are exact
// bf16 operands; fp32 intermediates (T, the decayed scores, dh, dU~, dX,
// ...) are split into bf16 hi/lo pairs (gdr_device.hpp), so a product costs
// 2 MFMAs against an exact operand and 3 between split operands, keeping
// about 16 significant bits; accumulation is fp32.  Tiles sit in LDS
// row-major with swizzled rows (gdr_lds.hpp), fp32 matrices as two bf16
// planes.
#include "gdr_kernels.hpp"
#include "gdr_lds.hpp"

namespace gdr {

namespace {

// split operands from the hi plane at `hi` and the lo plane `plane` bytes after it
template <int ROWB>
__device__ __forceinline__ OpS frag_s(const char *hi, int plane, int row, int byte) {
    using S = Swz<ROWB>;
    const int o0 = S::off(row, byte), o1 = S::off(row, byte + 32);
    OpS r;
    r.h0 = *reinterpret_cast<const bf16x4 *>(hi + o0);
    r.h1 = *reinterpret_cast<const bf16x4 *>(hi + o1);
    r.l0 = *reinterpret_cast<const bf16x4 *>(hi + plane + o0);
    r.l1 = *reinterpret_cast<const bf16x4 *>(hi + plane + o1);
    return r;
}
template <int ROWB>
__device__ __forceinline__ OpS kt_s(const char *hi, int plane, int c0, int ip) {
    const OpX a = kt_operand<bf16, ROWB>(hi, c0, ip), b = kt_operand<bf16, ROWB>(hi + plane, c0, ip);
    OpS r;
    r.h0 = a.b0;
    r.h1 = a.b1;
    r.l0 = b.b0;
    r.l1 = b.b1;
    return r;
}

// copy the 64 rows of a row-major global tile (row r at src + r * stride,
// ROWB bytes each) into a swizzled LDS tile, rows past nm1 repeating row nm1;
// 1 KB pieces spread over the waves
template <int ROWB>
__device__ __forceinline__ void copy_tile(char *dst, const char *src, int64_t stride, int nm1, int w) {
    using S = Swz<ROWB>;
    constexpr int PIECES = CH * ROWB / 1024;
    const int l = lane_id();
    for (int i = w; i < PIECES; i += NTHR / 64) {
        const int b = i * 1024 + 16 * l, r = b / ROWB, pc = (b % ROWB) / 16;
        dma16(src + min(r, nm1) * stride + 16 * S::chunk(r, pc), dst + i * 1024);
    }
}
__device__ __forceinline__ void copy_flat(char *dst, const char *src, int bytes, int w) {
    const int l = lane_id();
    for (int i = w; i < bytes / 1024; i += NTHR / 64) dma16(src + i * 1024 + 16 * l, dst + i * 1024);
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
            acc = mma(acc, frag<bf16, KROW>(Qs, 16 * ti + n16, (32 * dp + 4 * g) * 2),
                      frag<bf16, KROW>(Ks, 16 * tr + n16, (32 * dp + 4 * g) * 2));
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

// Sums over the 16 lanes of each lane group of the 4 values of an
// accumulator-ordered tile: lane (n, g) returns the sum for row 4 g + ((n >> 2) & 3).
__device__ __forceinline__ float rowsum16(f32x4 v) {
    const int n = ln16();
    const bool b3 = (n >> 3) & 1, b2 = (n >> 2) & 1;
    float k0 = b3 ? v[2] : v[0], k1 = b3 ? v[3] : v[1];
    const float s0 = b3 ? v[0] : v[2], s1 = b3 ? v[1] : v[3];
    k0 += __shfl_xor(s0, 8, 64);
    k1 += __shfl_xor(s1, 8, 64);
    float k = b2 ? k1 : k0;
    k += __shfl_xor(b2 ? k0 : k1, 4, 64);
    k += __shfl_xor(k, 2, 64);
    k += __shfl_xor(k, 1, 64);
    return k;
}
// sum over the 4 lane groups
__device__ __forceinline__ float sum_groups(float v) {
    v += __shfl_xor(v, 16, 64);
    return v + __shfl_xor(v, 32, 64);
}
__device__ __forceinline__ float sum_wave(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// one fp32 value as a hi/lo pair at (row, col) of split planes with 64 columns
__device__ __forceinline__ void put_s(char *hi, int plane, int row, int col, float v) {
    const int off = Swz<128>::off(row, 2 * col);
    const bf16 h = bf16(v);
    *reinterpret_cast<bf16 *>(hi + off) = h;
    *reinterpret_cast<bf16 *>(hi + plane + off) = bf16(v - float(h));
}
__device__ __forceinline__ float get_s(const char *hi, int plane, int row, int col) {
    const int off = Swz<128>::off(row, 2 * col);
    return float(*reinterpret_cast<const bf16 *>(hi + off)) + float(*reinterpret_cast<const bf16 *>(hi + plane + off));
}

// ------------------------------------------------------------- reverse scan
// One workgroup per (sequence, v head, 64 value columns); wave w owns
// columns 16 w .. 16 w + 15 and keeps its K x 16 slice of dh in registers
// (accumulator order: dh[dt] = rows 16 dt + 4 g + i, column 16 w + lane16).
// Per chunk, from the end: the transposed decayed scores P^T (upper
// triangular, shared split planes), then per wave
//   dU~ = diag(r) K dh' + s P^T dO,  dX = T^T dU~,
//   dh  = e_last dh' + Q^T diag(s e) dO - K^T diag(beta e) dX.
template <int KD>
__global__ __launch_bounds__(NTHR) void bwd_scan_bf16(const BwdParams p, int n_units) {
    constexpr int KROW = KD * 2, DROW = 64 * 2, PROW = 64 * 2, PPLANE = CH * PROW;
    constexpr int DT = KD / 16, DP = KD / 32;
    using TB = TBlock<bf16>;
    using SP = Swz<PROW>;
    __shared__ __attribute__((aligned(16))) char Ks[CH * KROW];
    __shared__ __attribute__((aligned(16))) char Qs[CH * KROW];
    __shared__ __attribute__((aligned(16))) char Ds[CH * DROW];
    __shared__ __attribute__((aligned(16))) char Tb[TB::BYTES];
    __shared__ __attribute__((aligned(16))) char Pt[2 * PPLANE];

    const int nvt = p.V / 64;
    const int wid = xcd_remap(blockIdx.x, gridDim.x);
    const int vt = wid % nvt, unit = wid / nvt;
    if (unit >= n_units) return;
    const int j = unit / p.Hv, hv = unit % p.Hv, hq = hv / (p.Hv / p.Hq);
    const int w = __builtin_amdgcn_readfirstlane(wave_id()), n16 = ln16(), g = lg4();
    const int col = vt * 64 + 16 * w + n16;
    int64_t bos, eos;
    p.sm.bounds(j, bos, eos);
    const int N = (int)((eos - bos + CH - 1) / CH);
    const int cb = p.sm.chunk_base(j);
    const int64_t KV = (int64_t)KD * p.V;
    const char *kp = reinterpret_cast<const char *>(p.k), *qp = reinterpret_cast<const char *>(p.q);
    const char *dop = reinterpret_cast<const char *>(p.dout);
    const float *sc = reinterpret_cast<const float *>(Tb + TB::SC);
    const float *eg = sc + CH, *rr = sc + 2 * CH, *bet = sc + 3 * CH;

    f32x4 dh[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dh[dt][i] = p.dht ? p.dht[unit * KV + (16 * dt + 4 * g + i) * p.V + col] : 0.f;
    zero_lower_pt(Pt);

    for (int c = N - 1; c >= 0; --c) {
        const int64_t ts = bos + (int64_t)c * CH;
        const int n = (int)min<int64_t>(CH, eos - ts);
        __syncthreads();  // the previous chunk is done with every tile
        copy_tile<KROW>(Ks, kp + (ts * p.Hq + hq) * KROW, (int64_t)p.Hq * KROW, n - 1, w);
        copy_tile<KROW>(Qs, qp + (ts * p.Hq + hq) * KROW, (int64_t)p.Hq * KROW, n - 1, w);
        copy_tile<DROW>(Ds, dop + ((ts * p.Hv + hv) * p.V + vt * 64) * 2, (int64_t)p.Hv * p.V * 2, n - 1, w);
        copy_flat(Tb, p.tblk + ((int64_t)(cb + c) * p.Hv + hv) * TB::BYTES, TB::BYTES, w);
        {  // gradient of this chunk's end state, for the chunk-local stage
            float *o = p.dhs + ((int64_t)(cb + c) * p.Hv + hv) * KV;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[(16 * dt + 4 * g + i) * p.V + col] = dh[dt][i];
        }
        wait_dma();
        __syncthreads();
        scores_t<KD>(Pt, Qs, Ks, sc, n, w);
        __syncthreads();
        // dU~ = diag(r) K dh' + s P^T dO  (rows = tokens, this wave's columns)
        f32x4 du[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) du[rt] = zero4();
#pragma unroll
        for (int dp = 0; dp < DP; ++dp) {
            const OpS hb = Ops<bf16>::split(dh[2 * dp], dh[2 * dp + 1]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
                du[rt] = mma(du[rt], frag<bf16, KROW>(Ks, 16 * rt + n16, (32 * dp + 4 * g) * 2), hb);
        }
        const OpX dob0 = kt_operand<bf16, DROW>(Ds, 16 * w, 0), dob1 = kt_operand<bf16, DROW>(Ds, 16 * w, 1);
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
                dx[rt] = mma(dx[rt], kt_s<TB::ROWB>(Tb, TB::PLANE, 16 * rt, ip), ip == 0 ? dus0 : dus1);
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
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            dh[dt] *= el;
#pragma unroll
            for (int ip = 0; ip < 2; ++ip) {
                dh[dt] = mma(dh[dt], kt_operand<bf16, KROW>(Qs, 16 * dt, ip), edo[ip]);
                dh[dt] = mma(dh[dt], kt_operand<bf16, KROW>(Ks, 16 * dt, ip), bdx[ip]);
            }
        }
    }
    if (p.dh0) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) p.dh0[unit * KV + (16 * dt + 4 * g + i) * p.V + col] = dh[dt][i];
    }
}

// ------------------------------------------------------- chunk-local terms
// One workgroup per (chunk, q/k head); its v heads in turn, the value
// dimension in blocks of 64 columns.  In a block, wave w first works on
// columns 16 w .. 16 w + 15 with tokens on the rows (K h, Q h, K dh', X,
// U~ = T X, dU~, dX = T^T dU~, dv), then writes U~, dU~, X and
// -diag(beta e) dX to LDS as split planes; the products over the value
// dimension (dP, dT and the value parts of dq, dk) are then accumulated on
// the tiles each wave owns: column strip w of the 64 x 64 matrices and key
// tiles w, w + 4 of the 64 x K ones.  After the value blocks, the 64 x 64
// stage forms dP * Gam, T^T dT T^T, dA, dS and the gate-gradient sums, and
// dq, dk take their score and K K^T terms; dq, dk add up over the v heads.
template <typename Gt, int KD>
__global__ __launch_bounds__(NTHR) void bwd_local_bf16(const BwdParams p) {
    constexpr int KROW = KD * 2, VROW = 128, PROW = 128, PPL = CH * PROW;
    constexpr int DP = KD / 32, TD = KD / 64;
    constexpr int NQ = 7;  // row sums: dO.Qh, dX.Kh, U~.Kdh', dX.Y, of dP*P, of dA*A, dbeta through A
    using TB = TBlock<bf16>;
    __shared__ __attribute__((aligned(16))) char Ks[CH * KROW];
    __shared__ __attribute__((aligned(16))) char Qs[CH * KROW];
    __shared__ __attribute__((aligned(16))) char Tb[TB::BYTES];
    __shared__ __attribute__((aligned(16))) char Pt[2 * PPL];
    __shared__ __attribute__((aligned(16))) char Ds[CH * VROW];
    __shared__ __attribute__((aligned(16))) char Wm[4][2 * PPL];
    __shared__ float rs[NQ][4][CH];
    __shared__ float cs[2][CH];
    __shared__ float red[4];

    const int gid = blockIdx.x, hq = blockIdx.y;
    int j, c;
    if (!p.sm.locate(gid, j, c)) return;
    int64_t bos, eos;
    p.sm.bounds(j, bos, eos);
    const int64_t ts = bos + (int64_t)c * CH;
    const int n = (int)min<int64_t>(CH, eos - ts);
    const int G = p.Hv / p.Hq;
    const int w = __builtin_amdgcn_readfirstlane(wave_id()), n16 = ln16(), g = lg4();
    const int V = p.V;
    const int64_t KV = (int64_t)KD * V;
    const char *kp = reinterpret_cast<const char *>(p.k), *qp = reinterpret_cast<const char *>(p.q);
    const bf16 *vp = reinterpret_cast<const bf16 *>(p.v);
    const char *dop = reinterpret_cast<const char *>(p.dout);
    Gt *dvp = reinterpret_cast<Gt *>(p.dv);
    const float *sc = reinterpret_cast<const float *>(Tb + TB::SC);
    const float *gam = sc, *eg = sc + CH, *rr = sc + 2 * CH, *bet = sc + 3 * CH;

    copy_tile<KROW>(Ks, kp + (ts * p.Hq + hq) * KROW, (int64_t)p.Hq * KROW, n - 1, w);
    copy_tile<KROW>(Qs, qp + (ts * p.Hq + hq) * KROW, (int64_t)p.Hq * KROW, n - 1, w);
    zero_lower_pt(Pt);
    f32x4 dqt[TD][4], dkt[TD][4];  // dq, dk tiles (key tile w + 4 s, token tile tr)
#pragma unroll
    for (int s = 0; s < TD; ++s)
#pragma unroll
        for (int tr = 0; tr < 4; ++tr) dqt[s][tr] = dkt[s][tr] = zero4();

    for (int gi = 0; gi < G; ++gi) {
        const int hv = hq * G + gi;
        __syncthreads();  // the previous v head is done with every LDS array
        copy_flat(Tb, p.tblk + ((int64_t)gid * p.Hv + hv) * TB::BYTES, TB::BYTES, w);
        wait_dma();
        __syncthreads();
        scores_t<KD>(Pt, Qs, Ks, gam, n, w);

        f32x4 dPa[4], dTa[4];
#pragma unroll
        for (int tr = 0; tr < 4; ++tr) dPa[tr] = dTa[tr] = zero4();
        float rsum[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) rsum[q][rt] = 0.f;
        float dec = 0.f;
        const int64_t hoff = ((int64_t)gid * p.Hv + hv) * KV;

        for (int vb = 0; vb < V; vb += 64) {
            __syncthreads();  // the previous block is done with Ds and Wm; scores complete
            copy_tile<VROW>(Ds, dop + ((ts * p.Hv + hv) * V + vb) * 2, (int64_t)p.Hv * V * 2, n - 1, w);
            const int colg = vb + 16 * w + n16;
            // K h, K dh' for this wave's columns (h, dh' in accumulator order from HBM)
            f32x4 kh[4], kd[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) kh[rt] = kd[rt] = zero4();
#pragma unroll 1
            for (int dp = 0; dp < DP; ++dp) {
                f32x4 h0, h1, d0, d1;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t o0 = hoff + (int64_t)(32 * dp + 4 * g + i) * V + colg, o1 = o0 + 16 * V;
                    h0[i] = p.hs[o0];
                    h1[i] = p.hs[o1];
                    d0[i] = p.dhs[o0];
                    d1[i] = p.dhs[o1];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) dec += h0[i] * d0[i] + h1[i] * d1[i];
                const OpS hb = Ops<bf16>::split(h0, h1), db = Ops<bf16>::split(d0, d1);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const OpX kf = frag<bf16, KROW>(Ks, 16 * rt + n16, (32 * dp + 4 * g) * 2);
                    kh[rt] = mma(kh[rt], kf, hb);
                    kd[rt] = mma(kd[rt], kf, db);
                }
            }
            // Y = V - diag(e) K h, X = diag(beta) Y
            f32x4 y[4], x[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int r0 = 16 * rt + 4 * g;
                const f32x4 e4 = *reinterpret_cast<const f32x4 *>(eg + r0);
                const f32x4 b4 = *reinterpret_cast<const f32x4 *>(bet + r0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tok = r0 + i;
                    const float vv = tok < n ? float(vp[((ts + tok) * p.Hv + hv) * V + colg]) : 0.f;
                    y[rt][i] = vv - e4[i] * kh[rt][i];
                }
                x[rt] = b4 * y[rt];
            }
            wait_dma();
            __syncthreads();  // dO block landed
            const OpS xs0 = Ops<bf16>::split(x[0], x[1]), xs1 = Ops<bf16>::split(x[2], x[3]);
            // U~ = T X (T lower triangular)
            f32x4 u[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                u[rt] = zero4();
#pragma unroll
                for (int ip = 0; ip <= rt / 2; ++ip)
                    u[rt] = mma(u[rt], frag_s<TB::ROWB>(Tb, TB::PLANE, 16 * rt + n16, (32 * ip + 4 * g) * 2),
                                ip == 0 ? xs0 : xs1);
            }
            // dU~ = diag(r) K dh' + s P^T dO
            const OpX dob0 = kt_operand<bf16, VROW>(Ds, 16 * w, 0), dob1 = kt_operand<bf16, VROW>(Ds, 16 * w, 1);
            f32x4 du[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 pd = zero4();
#pragma unroll
                for (int ip = rt / 2; ip < 2; ++ip)
                    pd = mma(pd, frag_s<PROW>(Pt, PPL, 16 * rt + n16, (32 * ip + 4 * g) * 2), ip == 0 ? dob0 : dob1);
                const f32x4 r4 = *reinterpret_cast<const f32x4 *>(rr + 16 * rt + 4 * g);
                du[rt] = r4 * kd[rt] + p.scale * pd;
            }
            // dX = T^T dU~
            const OpS dus0 = Ops<bf16>::split(du[0], du[1]), dus1 = Ops<bf16>::split(du[2], du[3]);
            f32x4 dx[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                dx[rt] = zero4();
#pragma unroll
                for (int ip = rt / 2; ip < 2; ++ip)
                    dx[rt] = mma(dx[rt], kt_s<TB::ROWB>(Tb, TB::PLANE, 16 * rt, ip), ip == 0 ? dus0 : dus1);
            }
            // dv = diag(beta) dX; row sums; U~, dU~, X, -diag(beta e) dX to LDS
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int r0 = 16 * rt + 4 * g;
                const f32x4 e4 = *reinterpret_cast<const f32x4 *>(eg + r0);
                const f32x4 b4 = *reinterpret_cast<const f32x4 *>(bet + r0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tok = r0 + i;
                    if (tok < n) dvp[((ts + tok) * p.Hv + hv) * V + colg] = Gt(b4[i] * dx[rt][i]);
                }
                rsum[1][rt] += rowsum16(dx[rt] * kh[rt]);
                rsum[3][rt] += rowsum16(dx[rt] * y[rt]);
                const f32x4 sdx = -(b4 * e4) * dx[rt];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    put_s(Wm[0], PPL, r0 + i, 16 * w + n16, u[rt][i]);
                    put_s(Wm[1], PPL, r0 + i, 16 * w + n16, du[rt][i]);
                    put_s(Wm[2], PPL, r0 + i, 16 * w + n16, x[rt][i]);
                    put_s(Wm[3], PPL, r0 + i, 16 * w + n16, sdx[i]);
                }
            }
            __syncthreads();
            // products over this block's 64 value columns (two k blocks of 32)
#pragma unroll 1
            for (int kb = 0; kb < 2; ++kb) {
                const int kbyte = (32 * kb + 4 * g) * 2;
                const OpS ub = frag_s<PROW>(Wm[0], PPL, 16 * w + n16, kbyte);  // U~^T, tokens of strip w
                const OpS xb = frag_s<PROW>(Wm[2], PPL, 16 * w + n16, kbyte);  // X^T
#pragma unroll
                for (int tr = 0; tr < 4; ++tr) {
                    dPa[tr] = mma(dPa[tr], frag<bf16, VROW>(Ds, 16 * tr + n16, kbyte), ub);
                    dTa[tr] = mma(dTa[tr], frag_s<PROW>(Wm[1], PPL, 16 * tr + n16, kbyte), xb);
                }
            }
            // value parts of dq, dk: s diag(e) dO h^T and diag(r) U~ dh'^T (row scales applied
            // per block), - diag(beta e) dX h^T (scale already in the plane).  The row sums
            // of dO * (Q h) and U~ * (K dh') are those of Q * (dO h^T) and K * (U~ dh'^T).
            f32x4 sq[4], sk[4];
#pragma unroll
            for (int tr = 0; tr < 4; ++tr) sq[tr] = sk[tr] = zero4();
#pragma unroll
            for (int s = 0; s < TD; ++s) {
                const int td = w + 4 * s;
                f32x4 aQ[4], aKa[4];
#pragma unroll
                for (int tr = 0; tr < 4; ++tr) aQ[tr] = aKa[tr] = zero4();
#pragma unroll 1
                for (int kb = 0; kb < 2; ++kb) {
                    const int kbyte = (32 * kb + 4 * g) * 2;
                    // h^T, dh'^T: rows d = 16 td + lane16, value columns vb + 32 kb + 4 g ..
                    const int64_t o = hoff + (int64_t)(16 * td + n16) * V + vb + 32 * kb + 4 * g;
                    const OpS hT = Ops<bf16>::split(*reinterpret_cast<const f32x4 *>(p.hs + o),
                                                    *reinterpret_cast<const f32x4 *>(p.hs + o + 16));
                    const OpS dhT = Ops<bf16>::split(*reinterpret_cast<const f32x4 *>(p.dhs + o),
                                                     *reinterpret_cast<const f32x4 *>(p.dhs + o + 16));
#pragma unroll
                    for (int tr = 0; tr < 4; ++tr) {
                        aQ[tr] = mma(aQ[tr], frag<bf16, VROW>(Ds, 16 * tr + n16, kbyte), hT);
                        aKa[tr] = mma(aKa[tr], frag_s<PROW>(Wm[0], PPL, 16 * tr + n16, kbyte), dhT);
                        dkt[s][tr] = mma(dkt[s][tr], frag_s<PROW>(Wm[3], PPL, 16 * tr + n16, kbyte), hT);
                    }
                }
#pragma unroll
                for (int tr = 0; tr < 4; ++tr) {
                    const f32x4 e4 = *reinterpret_cast<const f32x4 *>(eg + 16 * tr + 4 * g);
                    const f32x4 r4 = *reinterpret_cast<const f32x4 *>(rr + 16 * tr + 4 * g);
                    dqt[s][tr] += (p.scale * e4) * aQ[tr];
                    dkt[s][tr] += r4 * aKa[tr];
                    sq[tr] += rows4<bf16, KROW>(Qs, 16 * tr, 16 * td) * aQ[tr];
                    sk[tr] += rows4<bf16, KROW>(Ks, 16 * tr, 16 * td) * aKa[tr];
                }
            }
#pragma unroll
            for (int tr = 0; tr < 4; ++tr) {
                rsum[0][tr] += rowsum16(sq[tr]);
                rsum[2][tr] += rowsum16(sk[tr]);
            }
        }
        const int rtok = 4 * g + (n16 >> 2);  // token (within a 16-row tile) of this lane's row sums
        if ((n16 & 3) == 0) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) rs[q][w][16 * rt + rtok] = rsum[q][rt];
        }
        dec = sum_wave(dec);
        if (lane_id() == 0) red[w] = dec;
        __syncthreads();  // every wave is done with the block planes
        // W1 = dP * Gam on i <= r < n (Wm[0]); sums of dP * P; M1 = T^T dT (Wm[1]); S = K K^T strip
        const int ci = 16 * w + n16;  // this lane's column of the strips
        float zac = 0.f, zar[4];
#pragma unroll
        for (int tr = 0; tr < 4; ++tr) {
            f32x4 za;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * tr + 4 * g + i;
                const float dpv = p.scale * dPa[tr][i];
                const float w1 = (ci <= r && r < n) ? dpv * fast_exp(gam[r] - gam[ci]) : 0.f;
                put_s(Wm[0], PPL, r, ci, w1);
                za[i] = ci <= r ? dpv * get_s(Pt, PPL, ci, r) : 0.f;  // P^T below its diagonal is not stored
                zac += za[i];
            }
            zar[tr] = rowsum16(za);
        }
        zac = sum_groups(zac);
        {
            const OpS dts0 = Ops<bf16>::split(dTa[0], dTa[1]), dts1 = Ops<bf16>::split(dTa[2], dTa[3]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 m = zero4();
#pragma unroll
                for (int ip = rt / 2; ip < 2; ++ip)
                    m = mma(m, kt_s<TB::ROWB>(Tb, TB::PLANE, 16 * rt, ip), ip == 0 ? dts0 : dts1);
#pragma unroll
                for (int i = 0; i < 4; ++i) put_s(Wm[1], PPL, 16 * rt + 4 * g + i, ci, m[i]);
            }
        }
        f32x4 sS[4];
#pragma unroll
        for (int tr = 0; tr < 4; ++tr) {
            sS[tr] = zero4();
#pragma unroll
            for (int dp = 0; dp < DP; ++dp)
                sS[tr] = mma(sS[tr], frag<bf16, KROW>(Ks, 16 * tr + n16, (32 * dp + 4 * g) * 2),
                             frag<bf16, KROW>(Ks, 16 * w + n16, (32 * dp + 4 * g) * 2));
        }
        __syncthreads();
        // dA = -(M1 T^T) on i < r; dS = diag(beta) (dA * Gam) (Wm[2]); sums of dA * A; dbeta through A
        float zbc = 0.f, zbr[4], dbr[4];
#pragma unroll
        for (int tr = 0; tr < 4; ++tr) {
            f32x4 a = zero4();
#pragma unroll
            for (int ip = 0; ip <= w / 2; ++ip)
                a = mma(a, frag_s<PROW>(Wm[1], PPL, 16 * tr + n16, (32 * ip + 4 * g) * 2),
                        frag_s<TB::ROWB>(Tb, TB::PLANE, ci, (32 * ip + 4 * g) * 2));
            f32x4 zb, dbv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * tr + 4 * g + i;
                float dsv = 0.f;
                zb[i] = dbv[i] = 0.f;
                if (ci < r) {
                    const float G_ = fast_exp(gam[r] - gam[ci]);
                    const float da = -a[i];
                    dbv[i] = da * sS[tr][i] * G_;
                    zb[i] = bet[r] * dbv[i];
                    dsv = bet[r] * da * G_;
                }
                put_s(Wm[2], PPL, r, ci, dsv);
                zbc += zb[i];
            }
            zbr[tr] = rowsum16(zb);
            dbr[tr] = rowsum16(dbv);
        }
        zbc = sum_groups(zbc);
        if ((n16 & 3) == 0) {
#pragma unroll
            for (int tr = 0; tr < 4; ++tr) {
                rs[4][w][16 * tr + rtok] = zar[tr];
                rs[5][w][16 * tr + rtok] = zbr[tr];
                rs[6][w][16 * tr + rtok] = dbr[tr];
            }
        }
        if (g == 0) {
            cs[0][ci] = zac;
            cs[1][ci] = zbc;
        }
        __syncthreads();
        // dq += W1 K ;  dk += W1^T Q + dS K + dS^T K
#pragma unroll
        for (int s = 0; s < TD; ++s) {
            const int td = w + 4 * s;
            const OpX k0 = kt_operand<bf16, KROW>(Ks, 16 * td, 0), k1 = kt_operand<bf16, KROW>(Ks, 16 * td, 1);
            const OpX q0 = kt_operand<bf16, KROW>(Qs, 16 * td, 0), q1 = kt_operand<bf16, KROW>(Qs, 16 * td, 1);
#pragma unroll
            for (int tr = 0; tr < 4; ++tr) {
#pragma unroll
                for (int ip = 0; ip < 2; ++ip) {
                    const OpX &kb = ip == 0 ? k0 : k1;
                    if (ip <= tr / 2) {
                        const int kbyte = (32 * ip + 4 * g) * 2;
                        dqt[s][tr] = mma(dqt[s][tr], frag_s<PROW>(Wm[0], PPL, 16 * tr + n16, kbyte), kb);
                        dkt[s][tr] = mma(dkt[s][tr], frag_s<PROW>(Wm[2], PPL, 16 * tr + n16, kbyte), kb);
                    }
                    if (ip >= tr / 2) {
                        dkt[s][tr] = mma(dkt[s][tr], kt_s<PROW>(Wm[0], PPL, 16 * tr, ip), ip == 0 ? q0 : q1);
                        dkt[s][tr] = mma(dkt[s][tr], kt_s<PROW>(Wm[2], PPL, 16 * tr, ip), kb);
                    }
                }
            }
        }
        // dgam -> dg (reverse running sum over the chunk), dbeta
        if (w == 0) {
            const int r = lane_id();
            float x = 0.f, rd = 0.f;
            if (r < n) {
                float dea = 0.f, dkh = 0.f, drv = 0.f, dbx = 0.f, zr = 0.f, zb = 0.f, dba = 0.f;
#pragma unroll
                for (int ww = 0; ww < 4; ++ww) {
                    dea += rs[0][ww][r];
                    dkh += rs[1][ww][r];
                    drv += rs[2][ww][r];
                    dbx += rs[3][ww][r];
                    zr += rs[4][ww][r];
                    zb += rs[5][ww][r];
                    dba += rs[6][ww][r];
                }
                rd = rr[r] * drv;
                x = eg[r] * (p.scale * dea - bet[r] * dkh) + (zr - cs[0][r]) + (zb - cs[1][r]) - rd;
                p.dbeta[(ts + r) * p.Hv + hv] = dbx + dba;
            }
            const float tot = sum_wave(rd);
            if (r == n - 1) x += eg[r] * (red[0] + red[1] + red[2] + red[3]) + tot;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float yv = __shfl_down(x, off, 64);
                if (r + off < 64) x += yv;
            }
            if (r < n) p.dg[(ts + r) * p.Hv + hv] = x;
        }
    }
    Gt *dq = reinterpret_cast<Gt *>(p.dq), *dk = reinterpret_cast<Gt *>(p.dk);
#pragma unroll
    for (int s = 0; s < TD; ++s)
#pragma unroll
        for (int tr = 0; tr < 4; ++tr)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = 16 * tr + 4 * g + i;
                if (tok < n) {
                    const int64_t o = ((ts + tok) * p.Hq + hq) * KD + 16 * (w + 4 * s) + n16;
                    dq[o] = Gt(dqt[s][tr][i]);
                    dk[o] = Gt(dkt[s][tr][i]);
                }
            }
}

}  // namespace

hipError_t launch_bwd_local_bf16(Dt gt, int K, const BwdParams &p, int n_chunks_ub, hipStream_t s) {
    const dim3 grid(n_chunks_ub, p.Hq);
    if (gt == Dt::BF16) {
        if (K == 128)
            hipLaunchKernelGGL((bwd_local_bf16<bf16, 128>), grid, dim3(NTHR), 0, s, p);
        else
            hipLaunchKernelGGL((bwd_local_bf16<bf16, 64>), grid, dim3(NTHR), 0, s, p);
    } else {
        if (K == 128)
            hipLaunchKernelGGL((bwd_local_bf16<float, 128>), grid, dim3(NTHR), 0, s, p);
        else
            hipLaunchKernelGGL((bwd_local_bf16<float, 64>), grid, dim3(NTHR), 0, s, p);
    }
    return hipGetLastError();
}

hipError_t launch_bwd_scan_bf16(int K, const BwdParams &p, int n_units, hipStream_t s) {
    const dim3 grid(n_units * (p.V / 64));
    if (K == 128)
        hipLaunchKernelGGL((bwd_scan_bf16<128>), grid, dim3(NTHR), 0, s, p, n_units);
    else
        hipLaunchKernelGGL((bwd_scan_bf16<64>), grid, dim3(NTHR), 0, s, p, n_units);
    return hipGetLastError();
}

}  // namespace gdr
