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

#include "gdr_bwd_ops.hpp"

namespace gdr {

namespace {

using namespace bwd;

// ------------------------------------------------------- chunk-local terms
// One workgroup per (chunk, q/k head); its v heads in turn, the value
// dimension in blocks of 64 columns.  In a block, wave w first works on
// columns 16 w .. 16 w + 15 with tokens on the rows: K h and K dh' (h, dh'
// staged through LDS in 64-row halves as split planes), X, U~ = T X,
// dU~ = diag(r) K dh' + s P^T dO, dX = T^T dU~ and dv; it writes U~ and dX
// to LDS as split planes.  Then the products over the value dimension are
// accumulated on the tiles each wave owns: column strip w of
// dP = s dO U~^T and dA = -dX U~^T (= -T^T dT T^T with dT = dU~ X^T), and
// key tiles w, w + 4 of dO h^T, U~ dh'^T, dX h^T for dq and dk.  Row sums
// over the value dimension come from the same tiles where possible
// (sum_c dO.(Q h) = sum_d Q.(dO h^T) and alike).  After the value blocks
// the 64 x 64 stage forms dP * Gam and dS = diag(beta)(dA * Gam) with the
// gate-gradient sums, and dq, dk take their score and K K^T terms; dq, dk
// add up over the v heads of the q/k head.
template <typename Gt, int KD>
__global__ __launch_bounds__(NTHR) void bwd_local_bf16(const BwdParams p) {
    constexpr int KROW = KD * 2, VROW = 128, PROW = 128, PPL = CH * PROW;
    constexpr int DP = KD / 32, TD = KD / 64, NH = KD / 64;  // 64-row halves of h
    constexpr int NQ = 7;
    // row sums: 0 Q.(dO h^T), 1 K.(dX h^T), 2 K.(U~ dh'^T), 3 dX.V, 4 dP*P, 5 dA*A, 6 dbeta via A
    using TB = TBlockF<bf16>;  // compact T blocks: rows 0-31 stored in their first 32 columns
    using S128 = Swz<128>;
    __shared__ __attribute__((aligned(16))) char Ks[CH * KROW];
    __shared__ __attribute__((aligned(16))) char Qs[CH * KROW];
    __shared__ __attribute__((aligned(16))) char Tb[TB::BYTES];
    __shared__ __attribute__((aligned(16))) char Pt[2 * PPL];
    __shared__ __attribute__((aligned(16))) char Ds[CH * VROW];
    __shared__ __attribute__((aligned(16))) char Vs[CH * VROW];
    __shared__ __attribute__((aligned(16))) char Wm[2][2 * PPL];  // U~, dX; later dP * Gam, dS
    __shared__ __attribute__((aligned(16))) char Hs[2][2 * PPL];  // h, dh' rows of one half
    __shared__ float rs[NQ][4][CH];
    __shared__ float cs[2][CH];
    __shared__ float red[4];

    // Workgroup b runs on XCD b % 8.  The chunks are dealt to the XCDs in turn, so that
    // the rows of dbeta and dg that a chunk's q/k heads all write meet in one L2; within
    // an XCD the q/k head runs fastest (neighbours read adjacent pieces of the same q,
    // k, v and dO rows).  Chunks past the last (the grid rounds them up to a multiple
    // of 8) have no work.
    const int slot = blockIdx.x >> 3;
    const int hq = slot % p.Hq, gid = (slot / p.Hq) * 8 + (blockIdx.x & 7);
    int j, c;
    if (!p.sm.locate(gid, j, c)) return;
    int64_t bos, eos;
    p.sm.bounds(j, bos, eos);
    const int64_t ts = bos + (int64_t)c * CH;
    const int n = (int)min<int64_t>(CH, eos - ts);
    const int G = p.Hv / p.Hq;
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(wave_id()), n16 = ln16(), g = lg4();
    const int V = p.V;
    const int64_t KV = (int64_t)KD * V;
    const char *kp = reinterpret_cast<const char *>(p.k), *qp = reinterpret_cast<const char *>(p.q);
    const char *vpc = reinterpret_cast<const char *>(p.v), *dop = reinterpret_cast<const char *>(p.dout);
    Gt *dvp = reinterpret_cast<Gt *>(p.dv);
    const float *sc = reinterpret_cast<const float *>(Tb + TB::SC);
    const float *gam = sc, *eg = sc + CH, *rr = sc + 2 * CH, *bet = sc + 3 * CH;
    const int ci = 16 * w + n16;  // this lane's column in a 64-wide strip

    copy_tile<KROW, KeyBK>(Ks, kp + (ts * p.Hq + hq) * KROW, p.Hq * KROW, n - 1, w);
    copy_tile<KROW, KeyBK>(Qs, qp + (ts * p.Hq + hq) * KROW, p.Hq * KROW, n - 1, w);
    zero_lower_pt(Pt);
    f32x4 dqt[TD][4], dkt[TD][4];  // dq, dk tiles (key tile w + 4 s, token tile tr)
#pragma unroll
    for (int s = 0; s < TD; ++s)
#pragma unroll
        for (int tr = 0; tr < 4; ++tr) dqt[s][tr] = dkt[s][tr] = zero4();

    for (int gi = 0; gi < G; ++gi) {
        const int hv = hq * G + gi;
        const int64_t hoff = ((int64_t)gid * p.Hv + hv) * KV;
        // this (chunk, v head)'s states and end-state gradients: hi, lo planes of h^T, dh'^T [V][K]
        const char *hsb = reinterpret_cast<const char *>(p.hs + hoff);
        const char *dhsb = reinterpret_cast<const char *>(p.dhs + hoff);
        const int splane = KD * V * 2;
        Gt *dvb = dvp + (ts * p.Hv + hv) * V;                      // row tok at tok * Hv * V
        float dec = 0.f;
        // stage keys [64 hf, 64 hf + 64) of the value block vb of h^T and dh'^T (split planes,
        // rows = value columns) into B (Hs, or Wm while it is free) by direct copies ...
        auto stage = [&](char (*B)[2 * PPL], int hf, int vb) {
            const int src = (vb * KD + 64 * hf) * 2;
            copy_rows<128>(B[0], hsb + src, KD * 2, 63, w, 4);
            copy_rows<128>(B[0] + PPL, hsb + splane + src, KD * 2, 63, w, 4);
            copy_rows<128>(B[1], dhsb + src, KD * 2, 63, w, 4);
            copy_rows<128>(B[1] + PPL, dhsb + splane + src, KD * 2, 63, w, 4);
        };
        // ... wait for them; with `dot`, add this thread's share of <dh', h>
        auto land = [&](char (*B)[2 * PPL], bool dot) {
            wait_dma();
            __syncthreads();
            if (dot) {
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const int idx = tid + NTHR * it, row = idx >> 4, c4 = idx & 15;
                    const int off = S128::off(row, 8 * c4);
                    auto ld = [&](const char *pl) {
                        return __builtin_convertvector(*reinterpret_cast<const bf16x4 *>(pl + off), f32x4);
                    };
                    const f32x4 hx = ld(B[0]) + ld(B[0] + PPL), dx = ld(B[1]) + ld(B[1] + PPL);
                    dec += hx[0] * dx[0] + hx[1] * dx[1] + hx[2] * dx[2] + hx[3] * dx[3];
                }
            }
        };

        __syncthreads();  // the previous v head is done with every LDS array
        copy_flat(Tb, p.tblk + ((int64_t)gid * p.Hv + hv) * TB::BYTES, TB::BYTES, w);
        wait_dma();
        __syncthreads();
        // the first value block's dO, V and first key half are copied while the scores form
        copy_tile<VROW>(Ds, dop + (ts * p.Hv + hv) * V * 2, p.Hv * V * 2, n - 1, w);
        copy_tile<VROW>(Vs, vpc + (ts * p.Hv + hv) * V * 2, p.Hv * V * 2, n - 1, w);
        stage(NH == 2 ? Wm : Hs, 0, 0);
        scores_t<KD>(Pt, Qs, Ks, gam, n, w);

        f32x4 dPa[4], dAa[4];
#pragma unroll
        for (int tr = 0; tr < 4; ++tr) dPa[tr] = dAa[tr] = zero4();
        float rsum[3][4];  // partial row sums over this lane's 4 keys (token 16 rt + lane16)
        float rs3[4];      // dX.V partial over this lane's 4 columns (token 16 rt + lane16)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) rsum[0][rt] = rsum[1][rt] = rsum[2][rt] = rs3[rt] = 0.f;

        for (int vb = 0; vb < V; vb += 64) {
            __syncthreads();  // the previous block is done with Ds, Vs, Wm, Hs; scores complete
            if (vb > 0) {  // (the first block's were issued before the scores)
                copy_tile<VROW>(Ds, dop + ((ts * p.Hv + hv) * V + vb) * 2, p.Hv * V * 2, n - 1, w);
                copy_tile<VROW>(Vs, vpc + ((ts * p.Hv + hv) * V + vb) * 2, p.Hv * V * 2, n - 1, w);
            }
            // K h, K dh' for this wave's columns, over the halves of the key dimension
            f32x4 kh[4], kd[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) kh[rt] = kd[rt] = zero4();
            // the first of two halves goes to Wm (free until U~ and dX are formed), the
            // second to Hs, copied while the first half's products run; Hs then holds the
            // last half, which the dq, dk pass below starts from
#pragma unroll 1
            for (int hf = 0; hf < NH; ++hf) {
                char (*B)[2 * PPL] = NH == 2 && hf == 0 ? Wm : Hs;
                if (hf == 0 && vb > 0) stage(B, 0, vb);
                land(B, true);
                if (hf + 1 < NH) stage(Hs, hf + 1, vb);
#pragma unroll
                for (int ip = 0; ip < 2; ++ip) {
                    // B operands of h, dh' (k = keys 64 hf + 32 ip .., column 16 w + lane16)
                    const OpS hb = frag_s<128>(B[0], PPL, 16 * w + n16, (32 * ip + 4 * g) * 2);
                    const OpS db = frag_s<128>(B[1], PPL, 16 * w + n16, (32 * ip + 4 * g) * 2);
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt) {
                        const OpX kf = frag<bf16, KROW, KeyBK>(Ks, 16 * rt + n16, (64 * hf + 32 * ip + 4 * g) * 2);
                        kh[rt] = mma(kh[rt], kf, hb);
                        kd[rt] = mma(kd[rt], kf, db);
                    }
                }
            }
            wait_dma();
            __syncthreads();  // dO and V blocks landed
            // X = diag(beta) (V - diag(e) K h)
            f32x4 x[4], vv[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int r0 = 16 * rt + 4 * g;
                const f32x4 e4 = *reinterpret_cast<const f32x4 *>(eg + r0);
                const f32x4 b4 = *reinterpret_cast<const f32x4 *>(bet + r0);
                vv[rt] = rows4<bf16, VROW>(Vs, 16 * rt, 16 * w);
                x[rt] = b4 * (vv[rt] - e4 * kh[rt]);
            }
            const OpS xs0 = Ops<bf16>::split(x[0], x[1]), xs1 = Ops<bf16>::split(x[2], x[3]);
            // U~ and dX transposed (rows = this wave's 16 value columns, columns = tokens):
            // lane (token 16 rt + lane16, g) then holds columns 16 w + 4 g .. + 3 of its token,
            // which it writes as one row piece.  U~^T = X^T T^T (T lower triangular).
            const OpX dob0 = kt_operand<bf16, VROW>(Ds, 16 * w, 0), dob1 = kt_operand<bf16, VROW>(Ds, 16 * w, 1);
            f32x4 du[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {  // dU~ = diag(r) K dh' + s P^T dO (tokens on the rows)
                f32x4 pd = zero4();
#pragma unroll
                for (int ip = rt / 2; ip < 2; ++ip)
                    pd = mma(pd, frag_s<PROW>(Pt, PPL, 16 * rt + n16, (32 * ip + 4 * g) * 2), ip == 0 ? dob0 : dob1);
                const f32x4 r4 = *reinterpret_cast<const f32x4 *>(rr + 16 * rt + 4 * g);
                du[rt] = r4 * kd[rt] + p.scale * pd;
            }
            const OpS dus0 = Ops<bf16>::split(du[0], du[1]), dus1 = Ops<bf16>::split(du[2], du[3]);
            const int c4 = 16 * w + 4 * g;  // first of this lane's 4 value columns in the block
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int tok = 16 * rt + n16;
                f32x4 ut = zero4(), dxt = zero4();
#pragma unroll
                for (int ip = 0; ip <= rt / 2; ++ip)
                    ut = mma(ut, ip == 0 ? xs0 : xs1, frag_s_in<TB>(Tb, TB::PLANE, tok, (32 * ip + 4 * g) * 2));
#pragma unroll
                for (int ip = rt / 2; ip < 2; ++ip)  // dX^T = dU~^T T (T^T upper triangular)
                    dxt = mma(dxt, ip == 0 ? dus0 : dus1, kt_s_in<TB>(Tb, TB::PLANE, 16 * rt, ip));
                put4_s(Wm[0], PPL, tok, c4, ut);
                put4_s(Wm[1], PPL, tok, c4, dxt);
                if (tok < n) {
                    const f32x4 dvv = bet[tok] * dxt;
                    Gt *o = dvb + (uint32_t)(tok * p.Hv * V + vb + c4);
                    if constexpr (sizeof(Gt) == 2)
                        *reinterpret_cast<bf16x4 *>(o) = __builtin_convertvector(dvv, bf16x4);
                    else
                        *reinterpret_cast<f32x4 *>(o) = dvv;
                }
                const f32x4 v4 = __builtin_convertvector(
                    *reinterpret_cast<const bf16x4 *>(Vs + Swz<VROW>::off(tok, 2 * c4)), f32x4);
                rs3[rt] += dxt[0] * v4[0] + dxt[1] * v4[1] + dxt[2] * v4[2] + dxt[3] * v4[3];
            }
            __syncthreads();  // U~, dX planes complete; Hs holds the last half
            // dP += dO U~^T, dA -= dX U~^T on strip w (two k blocks of 32 value columns)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int kbyte = (32 * kb + 4 * g) * 2;
                const OpS ub = frag_s<PROW>(Wm[0], PPL, ci, kbyte);  // U~^T for the tokens of strip w
#pragma unroll
                for (int tr = 0; tr < 4; ++tr) {
                    // transposed: lane (token 16 tr + lane16, g) holds tokens i = 16 w + 4 g ..
                    dPa[tr] = mma(dPa[tr], ub, frag<bf16, VROW>(Ds, 16 * tr + n16, kbyte));
                    dAa[tr] = mma(dAa[tr], ub, frag_s<PROW>(Wm[1], PPL, 16 * tr + n16, kbyte));
                }
            }
            // value parts of dq, dk on key tiles w + 4 s (the half holding them, last half first)
#pragma unroll
            for (int s = TD - 1; s >= 0; --s) {
                if (s != NH - 1) {
                    __syncthreads();  // every wave is done with the staged half
                    stage(Hs, s, vb);
                    land(Hs, false);
                }
                // transposed tiles: lane (token 16 tr + lane16, g) holds keys 16 td + 4 g .. + 3
                f32x4 aQ[4], aKa[4], aKe[4];
#pragma unroll
                for (int tr = 0; tr < 4; ++tr) aQ[tr] = aKa[tr] = aKe[tr] = zero4();
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int kbyte = (32 * kb + 4 * g) * 2;
                    // A operands of h, dh' (rows = keys 64 s + 16 w + lane16, k = value columns 32 kb ..)
                    const OpS hT = kt_s<128>(Hs[0], PPL, 16 * w, kb);
                    const OpS dhT = kt_s<128>(Hs[1], PPL, 16 * w, kb);
#pragma unroll
                    for (int tr = 0; tr < 4; ++tr) {
                        aQ[tr] = mma(aQ[tr], hT, frag<bf16, VROW>(Ds, 16 * tr + n16, kbyte));
                        aKa[tr] = mma(aKa[tr], dhT, frag_s<PROW>(Wm[0], PPL, 16 * tr + n16, kbyte));
                        aKe[tr] = mma(aKe[tr], hT, frag_s<PROW>(Wm[1], PPL, 16 * tr + n16, kbyte));
                    }
                }
                const int td = w + 4 * s;
#pragma unroll
                for (int tr = 0; tr < 4; ++tr) {
                    const int r = 16 * tr + n16;
                    const float er = eg[r];
                    dqt[s][tr] += (p.scale * er) * aQ[tr];
                    dkt[s][tr] += rr[r] * aKa[tr] - (bet[r] * er) * aKe[tr];
                    const f32x4 q4 = __builtin_convertvector(
                        *reinterpret_cast<const bf16x4 *>(Qs + Swz<KROW, KeyBK>::off(r, 2 * (16 * td + 4 * g))), f32x4);
                    const f32x4 k4 = __builtin_convertvector(
                        *reinterpret_cast<const bf16x4 *>(Ks + Swz<KROW, KeyBK>::off(r, 2 * (16 * td + 4 * g))), f32x4);
                    const f32x4 a = q4 * aQ[tr], b = k4 * aKe[tr], cc = k4 * aKa[tr];
                    rsum[0][tr] += a[0] + a[1] + a[2] + a[3];
                    rsum[1][tr] += b[0] + b[1] + b[2] + b[3];
                    rsum[2][tr] += cc[0] + cc[1] + cc[2] + cc[3];
                }
            }
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const float t0 = sum_groups(rsum[0][rt]), t1 = sum_groups(rsum[1][rt]);
            const float t2 = sum_groups(rsum[2][rt]), t3 = sum_groups(rs3[rt]);
            if (g == 0) {
                rs[0][w][16 * rt + n16] = t0;
                rs[1][w][16 * rt + n16] = t1;
                rs[2][w][16 * rt + n16] = t2;
                rs[3][w][16 * rt + n16] = t3;
            }
        }
        dec = sum_wave(dec);
        if (lane_id() == 0) red[w] = dec;
        __syncthreads();  // every wave is done with the block planes
        // dP * Gam on i <= r < n (Wm[0]) and sums of dP * P; dS = diag(beta) (dA * Gam) on i < r
        // (Wm[1]) and sums of dA * A, with A = diag(beta) (K K^T * Gam).  Lane (token
        // r = 16 tr + lane16, g) holds columns i = 16 w + 4 g .. + 3 of row r.
        const int i0 = 16 * w + 4 * g;
        f32x4 zac = zero4(), zbc = zero4();  // column sums, summed over the token tiles
#pragma unroll
        for (int tr = 0; tr < 4; ++tr) {
            const int r = 16 * tr + n16;
            f32x4 sS = zero4();  // S[r][i] (S = K K^T is symmetric)
#pragma unroll
            for (int dp = 0; dp < DP; ++dp)
                sS = mma(sS, frag<bf16, KROW, KeyBK>(Ks, 16 * w + n16, (32 * dp + 4 * g) * 2),
                         frag<bf16, KROW, KeyBK>(Ks, r, (32 * dp + 4 * g) * 2));
            // P[r][i] = P^T[i][r]: four rows of P^T at column r (only i <= r is stored)
            const f32x4 pr = rows4<bf16, 128>(Pt, 16 * w, 16 * tr) + rows4<bf16, 128>(Pt + PPL, 16 * w, 16 * tr);
            const float gr = gam[r], br = bet[r];
            const f32x4 gi = *reinterpret_cast<const f32x4 *>(gam + i0);
            f32x4 w1, ds, za, zb;
            float dba = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = i0 + j;
                const float dpv = p.scale * dPa[tr][j];
                const float G_ = i <= r ? fast_exp(gr - gi[j]) : 0.f;
                w1[j] = r < n ? dpv * G_ : 0.f;
                za[j] = i <= r ? dpv * pr[j] : 0.f;
                const float da = i < r ? -dAa[tr][j] : 0.f;
                const float dbv = da * sS[j] * G_;
                dba += dbv;
                zb[j] = br * dbv;
                ds[j] = br * da * G_;
            }
            put4_s(Wm[0], PPL, r, i0, w1);
            put4_s(Wm[1], PPL, r, i0, ds);
            zac += za;
            zbc += zb;
            const float zrow = sum_groups(za[0] + za[1] + za[2] + za[3]);
            const float zbrow = sum_groups(zb[0] + zb[1] + zb[2] + zb[3]);
            dba = sum_groups(dba);
            if (g == 0) {
                rs[4][w][r] = zrow;
                rs[5][w][r] = zbrow;
                rs[6][w][r] = dba;
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float za_c = row_sum16(zac[j]), zb_c = row_sum16(zbc[j]);
            if (n16 == 0) {
                cs[0][i0 + j] = za_c;
                cs[1][i0 + j] = zb_c;
            }
        }
        __syncthreads();
        // dq += (dP * Gam) K ;  dk += (dP * Gam)^T Q + dS K + dS^T K
#pragma unroll
        for (int s = 0; s < TD; ++s) {
            const int td = w + 4 * s;
            const OpX k0 = kt_operand<bf16, KROW, KeyBK>(Ks, 16 * td, 0), k1 = kt_operand<bf16, KROW, KeyBK>(Ks, 16 * td, 1);
            const OpX q0 = kt_operand<bf16, KROW, KeyBK>(Qs, 16 * td, 0), q1 = kt_operand<bf16, KROW, KeyBK>(Qs, 16 * td, 1);
#pragma unroll
            for (int tr = 0; tr < 4; ++tr) {
#pragma unroll
                for (int ip = 0; ip < 2; ++ip) {
                    const OpX &kb = ip == 0 ? k0 : k1;
                    // transposed: K^T, Q^T as the A operands
                    if (ip <= tr / 2) {
                        const int kbyte = (32 * ip + 4 * g) * 2;
                        dqt[s][tr] = mma(dqt[s][tr], kb, frag_s<PROW>(Wm[0], PPL, 16 * tr + n16, kbyte));
                        dkt[s][tr] = mma(dkt[s][tr], kb, frag_s<PROW>(Wm[1], PPL, 16 * tr + n16, kbyte));
                    }
                    if (ip >= tr / 2) {
                        dkt[s][tr] = mma(dkt[s][tr], ip == 0 ? q0 : q1, kt_s<PROW>(Wm[0], PPL, 16 * tr, ip));
                        dkt[s][tr] = mma(dkt[s][tr], kb, kt_s<PROW>(Wm[1], PPL, 16 * tr, ip));
                    }
                }
            }
        }
        // dgam -> dg (reverse running sum over the chunk), dbeta
        if (w == 0) {
            const int r = lane_id();
            float x = 0.f, rd = 0.f;
            if (r < n) {
                float q[NQ];
#pragma unroll
                for (int k = 0; k < NQ; ++k) q[k] = rs[k][0][r] + rs[k][1][r] + rs[k][2][r] + rs[k][3][r];
                rd = rr[r] * q[2];
                x = eg[r] * (p.scale * q[0] - bet[r] * q[1]) + (q[4] - cs[0][r]) + (q[5] - cs[1][r]) - rd;
                p.dbeta[ts * p.Hv + (uint32_t)(r * p.Hv + hv)] = q[3] - eg[r] * q[1] + q[6];
            }
            const float tot = sum_wave(rd);
            if (r == n - 1) x += eg[r] * (red[0] + red[1] + red[2] + red[3]) + tot;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float yv = __shfl_down(x, off, 64);
                if (r + off < 64) x += yv;
            }
            if (r < n) p.dg[ts * p.Hv + (uint32_t)(r * p.Hv + hv)] = x;
        }
    }
    Gt *dq = reinterpret_cast<Gt *>(p.dq) + (ts * p.Hq + hq) * KD;
    Gt *dk = reinterpret_cast<Gt *>(p.dk) + (ts * p.Hq + hq) * KD;
#pragma unroll
    for (int s = 0; s < TD; ++s)
#pragma unroll
        for (int tr = 0; tr < 4; ++tr) {
            const int tok = 16 * tr + n16;
            if (tok < n) {  // keys 16 (w + 4 s) + 4 g .. + 3 of the token
                const uint32_t o = (uint32_t)(tok * p.Hq * KD + 16 * (w + 4 * s) + 4 * g);
                if constexpr (sizeof(Gt) == 2) {
                    *reinterpret_cast<bf16x4 *>(dq + o) = __builtin_convertvector(dqt[s][tr], bf16x4);
                    *reinterpret_cast<bf16x4 *>(dk + o) = __builtin_convertvector(dkt[s][tr], bf16x4);
                } else {
                    *reinterpret_cast<f32x4 *>(dq + o) = dqt[s][tr];
                    *reinterpret_cast<f32x4 *>(dk + o) = dkt[s][tr];
                }
            }
        }
}


}  // namespace

hipError_t launch_bwd_local_bf16(Dt gt, int K, const BwdParams &p, int n_chunks_ub, hipStream_t s) {
    const dim3 grid((n_chunks_ub + 7) / 8 * 8 * p.Hq);  // (chunk, q/k head)
    if (gt == Dt::BF16) {
        if (K == 128)
            launch_k((bwd_local_bf16<bf16, 128>), grid, dim3(NTHR), 0, s, p);
        else
            launch_k((bwd_local_bf16<bf16, 64>), grid, dim3(NTHR), 0, s, p);
    } else {
        if (K == 128)
            launch_k((bwd_local_bf16<float, 128>), grid, dim3(NTHR), 0, s, p);
        else
            launch_k((bwd_local_bf16<float, 64>), grid, dim3(NTHR), 0, s, p);
    }
    return hipGetLastError();
}


}  // namespace gdr
