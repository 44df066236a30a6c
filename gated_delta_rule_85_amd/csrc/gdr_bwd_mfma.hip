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
    // P^T tiles (1,0) and (3,2) below the diagonal are read as zero and never written
    for (int idx = threadIdx.x; idx < 2 * 16 * 16; idx += NTHR) {
        const int t = idx >> 8, r = 16 + 32 * t + ((idx >> 4) & 15), i = 32 * t + (idx & 15);
        const int off = SP::off(r, 2 * i);
        *reinterpret_cast<bf16 *>(Pt + off) = bf16(0.f);
        *reinterpret_cast<bf16 *>(Pt + PPLANE + off) = bf16(0.f);
    }

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
        // P^T[r'][i] = (Q K^T)[i][r'] exp(gam_i - gam_r') for r' <= i < n
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
            const float gr = sc[r];
            f32x4 v;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int i = 16 * ti + 4 * g + jj;
                v[jj] = (r <= i && i < n) ? acc[jj] * fast_exp(sc[i] - gr) : 0.f;
            }
            bf16x4 hi, lo;
            split4(v, hi, lo);
            const int off = SP::off(r, 2 * (16 * ti + 4 * g));
            *reinterpret_cast<bf16x4 *>(Pt + off) = hi;
            *reinterpret_cast<bf16x4 *>(Pt + PPLANE + off) = lo;
        }
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

}  // namespace

hipError_t launch_bwd_scan_bf16(int K, const BwdParams &p, int n_units, hipStream_t s) {
    const dim3 grid(n_units * (p.V / 64));
    if (K == 128)
        hipLaunchKernelGGL((bwd_scan_bf16<128>), grid, dim3(NTHR), 0, s, p, n_units);
    else
        hipLaunchKernelGGL((bwd_scan_bf16<64>), grid, dim3(NTHR), 0, s, p, n_units);
    return hipGetLastError();
}

}  // namespace gdr
