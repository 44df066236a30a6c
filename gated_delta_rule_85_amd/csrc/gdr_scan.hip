// gdr_scan_output — the serial inter-chunk scan fused with the output.
//
// One workgroup owns one (sequence, v-head, block of BV value columns) and
// walks the chunks of its segment in order, keeping the K x BV slice of the
// state h in registers (fp32, accumulator order; wave w holds columns
// [16*NCT*w, 16*NCT*(w+1)) of the block).  For a chunk of n tokens with
// start state h (the chunked form of the gated delta rule):
//
//   X  = beta * (V - diag(e^gam) K h)          (delta-rule target before the
//                                                in-chunk correction)
//   U~ = T X            = U - W h              (the "V correction": with
//                                                U = T diag(beta) V and
//                                                W = T diag(beta e^gam) K)
//   O  = scale (diag(e^gam) Q h + P U~),  P = tril(Q K^T) * exp(gam_r - gam_i)
//   h' = e^{gam_last} h + K^T (exp(gam_last - gam) * U~)
//
// T comes from gdr_chunk_prep.  Columns of h evolve independently, so the
// value dimension is split across workgroups.  Products with fp32 operands
// use split-bf16 MFMA (see gdr_device.hpp); accumulation is fp32.
//
// Sequence split (the pages' AutoCP with its sliding-window warm-up): with
// seg_chunks smaller than the sequence, segment s > 0 starts from a zero
// state warm_chunks chunks before its first chunk (from the true initial
// state when that window reaches chunk 0) and runs the scan without output
// over the window before its own chunks.
#include "gdr_kernels.hpp"

namespace gdr {

namespace {

template <typename In> struct PlaneT { typedef bf16 type; static constexpr int planes = 2; };
template <> struct PlaneT<float> { typedef float type; static constexpr int planes = 1; };

template <typename In, int KD, int NCT> struct ScanLayout {
    static constexpr int BV = 64 * NCT;
    static constexpr int EV = Vec16<In>::n;
    static constexpr int LDK = KD + EV;   // K, Q rows
    static constexpr int LDV = BV + EV;   // V rows
    typedef typename PlaneT<In>::type P;
    static constexpr int LDT = CH + 16 / (int)sizeof(P);  // T, P planes
    static constexpr size_t ks = 0;
    static constexpr size_t qs = ks + sizeof(In) * CH * LDK;
    static constexpr size_t vs = qs + sizeof(In) * CH * LDK;
    static constexpr size_t tp = vs + sizeof(In) * CH * LDV;
    static constexpr size_t pp = tp + sizeof(P) * CH * LDT * PlaneT<In>::planes;
    static constexpr size_t sc = pp + sizeof(P) * CH * LDT * PlaneT<In>::planes;
    static constexpr size_t bytes = sc + sizeof(float) * 4 * CH;
    // per-thread prefetch counts
    static constexpr int NK = CH * (KD / EV) / NTHR;
    static constexpr int NV = CH * (BV / EV) / NTHR;
    static constexpr int NT = CH * 16 / NTHR;
    static_assert(NK * NTHR == CH * (KD / EV), "K tiling");
    static_assert(NV * NTHR == CH * (BV / EV), "V tiling");
};

template <typename In> __device__ __forceinline__ SplitPlane<In> plane(char *base, int ldt) {
    typedef typename PlaneT<In>::type P;
    SplitPlane<In> sp;
    sp.hi = reinterpret_cast<P *>(base);
    sp.lo = reinterpret_cast<P *>(base) + CH * ldt;
    return sp;
}

// A operand of K^T (rows = key dims d0 + lane, k = tokens 32*ip ..), gathered
// from the token-major K tile.
template <typename In>
__device__ __forceinline__ typename Ops<In>::X gather_kt(const In *Ks, int ldk, int d, int ip) {
    const int g = lg4();
    const In *b0 = Ks + (32 * ip + 4 * g) * ldk + d;
    const In *b1 = b0 + 16 * ldk;
    typename Ops<In>::X r;
    if constexpr (sizeof(In) == 2) {
        r.b0 = bf16x4{b0[0], b0[ldk], b0[2 * ldk], b0[3 * ldk]};
        r.b1 = bf16x4{b1[0], b1[ldk], b1[2 * ldk], b1[3 * ldk]};
    } else {
        r.b0 = f32x4{b0[0], b0[ldk], b0[2 * ldk], b0[3 * ldk]};
        r.b1 = f32x4{b1[0], b1[ldk], b1[2 * ldk], b1[3 * ldk]};
    }
    return r;
}

template <typename T> __device__ __forceinline__ void store_out(T *p, float x);
template <> __device__ __forceinline__ void store_out<float>(float *p, float x) { *p = x; }
template <> __device__ __forceinline__ void store_out<bf16>(bf16 *p, float x) { *p = static_cast<bf16>(x); }

template <typename In, typename Out, int KD, int NCT>
__global__ __launch_bounds__(NTHR) void scan_output_kernel(const ScanParams p) {
    using L = ScanLayout<In, KD, NCT>;
    using O = Ops<In>;
    using XT = typename O::X;
    using ST = typename O::S;
    using V16 = typename Vec16<In>::type;
    constexpr int EV = L::EV, LDK = L::LDK, LDV = L::LDV, LDT = L::LDT, BV = L::BV;
    constexpr int DT = KD / 16;  // row tiles of the state
    extern __shared__ __attribute__((aligned(16))) char smem[];
    In *Ks = reinterpret_cast<In *>(smem + L::ks);
    In *Qs = reinterpret_cast<In *>(smem + L::qs);
    In *Vs = reinterpret_cast<In *>(smem + L::vs);
    const SplitPlane<In> Tp = plane<In>(smem + L::tp, LDT);
    const SplitPlane<In> Pp = plane<In>(smem + L::pp, LDT);
    float *gam = reinterpret_cast<float *>(smem + L::sc);
    float *eg = gam + CH, *rr = eg + CH, *bet = rr + CH;

    // ---- work item: (v tile, v head, sequence, segment), XCD-grouped
    const int wid = xcd_remap(blockIdx.x, gridDim.x);
    const int vt = wid % p.n_vt;
    const int rest = wid / p.n_vt;
    const int unit = rest % p.n_units, seg = rest / p.n_units;
    const int j = unit / p.Hv, hv = unit % p.Hv;
    const int G = p.Hv / p.Hq, hq = hv / G;
    int64_t bos, eos;
    p.sm.bounds(j, bos, eos);
    const int N = (int)((eos - bos + CH - 1) / CH);
    const int c_begin = seg * p.seg_chunks;
    if (c_begin >= N && !(N == 0 && seg == 0)) return;
    const int c_end = min(N, c_begin + p.seg_chunks);
    const int w_begin = seg == 0 ? 0 : max(0, c_begin - p.warm_chunks);

    const int tid = threadIdx.x, w = wave_id(), n16 = ln16(), g = lg4();
    const In *qp = reinterpret_cast<const In *>(p.q);
    const In *kp = reinterpret_cast<const In *>(p.k);
    const In *vp = reinterpret_cast<const In *>(p.v);
    const int64_t KV = (int64_t)KD * p.V;
    const int colw = vt * BV + w * 16 * NCT;  // first value column of this wave

    // ---- state slice in accumulator order: h[dt][ct] = rows 16dt+4g+i, column colw+16ct+n16
    f32x4 h[DT][NCT];
    {
        const bool from_h0 = (w_begin == 0) && p.h0 != nullptr;
        const float *h0 = from_h0 ? p.h0 + (int64_t)unit * KV : nullptr;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    h[dt][ct][i] = from_h0 ? h0[(16 * dt + 4 * g + i) * p.V + colw + 16 * ct + n16] : 0.f;
    }
    // never-written tiles of P above the diagonal pairs
    {
        typedef typename PlaneT<In>::type PT;
        for (int idx = tid; idx < 2 * 16 * 16; idx += NTHR) {
            const int t = idx >> 8, r = (idx >> 4) & 15, i = idx & 15;
            const int off = (32 * t + r) * LDT + 32 * t + 16 + i;
            Pp.hi[off] = PT(0.f);
            if constexpr (PlaneT<In>::planes == 2) Pp.lo[off] = PT(0.f);
        }
    }

    // ---- prefetch registers (next chunk)
    V16 kr[L::NK], qr[L::NK], vr[L::NV];
    f32x4 tr[L::NT];
    float gr = 0.f, glast = 0.f, br = 0.f;
    int pf_n = 0;
    auto prefetch = [&](int c) {
        const int64_t ts = bos + (int64_t)c * CH;
        const int n = (int)min<int64_t>(CH, eos - ts);
        pf_n = n;
#pragma unroll
        for (int s = 0; s < L::NK; ++s) {
            const int idx = tid + NTHR * s, r = idx / (KD / EV), cv = idx % (KD / EV);
            kr[s] = V16{};
            qr[s] = V16{};
            if (r < n) {
                kr[s] = *reinterpret_cast<const V16 *>(kp + ((ts + r) * p.Hq + hq) * KD + cv * EV);
                qr[s] = *reinterpret_cast<const V16 *>(qp + ((ts + r) * p.Hq + hq) * KD + cv * EV);
            }
        }
#pragma unroll
        for (int s = 0; s < L::NV; ++s) {
            const int idx = tid + NTHR * s, r = idx / (BV / EV), cv = idx % (BV / EV);
            vr[s] = V16{};
            if (r < n) vr[s] = *reinterpret_cast<const V16 *>(vp + ((ts + r) * p.Hv + hv) * p.V + vt * BV + cv * EV);
        }
#pragma unroll
        for (int s = 0; s < L::NT; ++s) {
            const int idx = tid + NTHR * s, r = idx >> 4, c4 = idx & 15;
            tr[s] = zero4();
            if (r < n) tr[s] = *reinterpret_cast<const f32x4 *>(p.Tm + ((ts + r) * p.Hv + hv) * CH + 4 * c4);
        }
        if (tid < CH) {
            const int r = min(tid, n - 1);
            gr = p.g_cum[(ts + r) * p.Hv + hv];
            glast = p.g_cum[(ts + n - 1) * p.Hv + hv];
            br = tid < n ? p.beta[(ts + tid) * p.Hv + hv] : 0.f;
        }
    };
    auto commit = [&]() {
#pragma unroll
        for (int s = 0; s < L::NK; ++s) {
            const int idx = tid + NTHR * s, r = idx / (KD / EV), cv = idx % (KD / EV);
            *reinterpret_cast<V16 *>(Ks + r * LDK + cv * EV) = kr[s];
            *reinterpret_cast<V16 *>(Qs + r * LDK + cv * EV) = qr[s];
        }
#pragma unroll
        for (int s = 0; s < L::NV; ++s) {
            const int idx = tid + NTHR * s, r = idx / (BV / EV), cv = idx % (BV / EV);
            *reinterpret_cast<V16 *>(Vs + r * LDV + cv * EV) = vr[s];
        }
#pragma unroll
        for (int s = 0; s < L::NT; ++s) {
            const int idx = tid + NTHR * s, r = idx >> 4, c4 = idx & 15;
            Tp.put4(r * LDT + 4 * c4, tr[s]);
        }
        if (tid < CH) {
            gam[tid] = gr;
            eg[tid] = fast_exp(gr);
            rr[tid] = fast_exp(glast - gr);
            bet[tid] = br;
        }
    };

    if (w_begin < c_end) prefetch(w_begin);
    const int cb = p.sm.chunk_base(j);
    for (int c = w_begin; c < c_end; ++c) {
        const bool emit = c >= c_begin;
        const int64_t ts = bos + (int64_t)c * CH;
        __syncthreads();  // previous chunk done with LDS
        commit();
        const int n = pf_n;
        if (c + 1 < c_end) prefetch(c + 1);
        __syncthreads();

        if (emit && p.hsnap) {
            float *hs = p.hsnap + ((int64_t)(cb + c) * p.Hv + hv) * KV;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        hs[(16 * dt + 4 * g + i) * p.V + colw + 16 * ct + n16] = h[dt][ct][i];
        }
        // P = tril(Q K^T) * exp(gam_r - gam_i): ten tiles spread over the waves
        if (emit) {
            const int t0 = w == 0 ? 0 : w == 1 ? 3 : w == 2 ? 6 : 8;
            const int t1 = w == 0 ? 3 : w == 1 ? 6 : w == 2 ? 8 : 10;
            for (int t = t0; t < t1; ++t) {
                int trow = 0;
                while ((trow + 1) * (trow + 2) / 2 <= t) ++trow;
                const int ti = t - trow * (trow + 1) / 2;
                f32x4 acc = zero4();
#pragma unroll
                for (int dp = 0; dp < KD / 32; ++dp) {
                    const In *ar = Ks + (16 * ti + n16) * LDK + 32 * dp + 4 * g;
                    const In *brw = Qs + (16 * trow + n16) * LDK + 32 * dp + 4 * g;
                    acc = mma(acc, O::load(ar, ar + 16), O::load(brw, brw + 16));
                }
                // acc[jj] = (K Q^T)[i][r] = P[r][i], i = 16ti+4g+jj, r = 16trow+n16
                const int r = 16 * trow + n16;
                f32x4 pv;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int i = 16 * ti + 4 * g + jj;
                    pv[jj] = i <= r ? acc[jj] * fast_exp(gam[r] - gam[i]) : 0.f;
                }
                Pp.put4(r * LDT + 16 * ti + 4 * g, pv);
            }
        }

        // split state as B operand (k = key dims)
        ST hsb[DT / 2][NCT];
#pragma unroll
        for (int dp = 0; dp < DT / 2; ++dp)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) hsb[dp][ct] = O::split(h[2 * dp][ct], h[2 * dp + 1][ct]);

        // K h and Q h over the chunk's 64 rows
        f32x4 kh[4][NCT], qh[4][NCT];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                kh[rt][ct] = zero4();
                qh[rt][ct] = zero4();
            }
#pragma unroll
            for (int dp = 0; dp < DT / 2; ++dp) {
                const In *ar = Ks + (16 * rt + n16) * LDK + 32 * dp + 4 * g;
                const XT a = O::load(ar, ar + 16);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) kh[rt][ct] = mma(kh[rt][ct], a, hsb[dp][ct]);
                if (emit) {
                    const In *aq = Qs + (16 * rt + n16) * LDK + 32 * dp + 4 * g;
                    const XT b = O::load(aq, aq + 16);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) qh[rt][ct] = mma(qh[rt][ct], b, hsb[dp][ct]);
                }
            }
        }
        // X = beta (V - e^gam K h), split as B operand (k = tokens)
        ST xs[2][NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int col = w * 16 * NCT + 16 * ct + n16;
            f32x4 x[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * rt + 4 * g + i;
                    x[rt][i] = bet[row] * (to_f32(Vs[row * LDV + col]) - eg[row] * kh[rt][ct][i]);
                }
            xs[0][ct] = O::split(x[0], x[1]);
            xs[1][ct] = O::split(x[2], x[3]);
        }
        // U~ = T X  (T unit lower triangular: row tile rt uses k pairs <= rt/2)
        f32x4 ut[4][NCT];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) ut[rt][ct] = zero4();
#pragma unroll
            for (int ip = 0; ip <= rt / 2; ++ip) {
                const int off = (16 * rt + n16) * LDT + 32 * ip + 4 * g;
                const ST a = Tp.get(off, off + 16);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) ut[rt][ct] = mma(ut[rt][ct], a, xs[ip][ct]);
            }
        }
        __syncthreads();  // P tiles visible
        if (emit) {
            ST us[2][NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                us[0][ct] = O::split(ut[0][ct], ut[1][ct]);
                us[1][ct] = O::split(ut[2][ct], ut[3][ct]);
            }
            Out *op = reinterpret_cast<Out *>(p.o);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 acc[NCT];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[ct][i] = eg[16 * rt + 4 * g + i] * qh[rt][ct][i];
#pragma unroll
                for (int ip = 0; ip <= rt / 2; ++ip) {
                    const int off = (16 * rt + n16) * LDT + 32 * ip + 4 * g;
                    const ST a = Pp.get(off, off + 16);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) acc[ct] = mma(acc[ct], a, us[ip][ct]);
                }
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 16 * rt + 4 * g + i;
                        if (row < n)
                            store_out(op + ((ts + row) * p.Hv + hv) * p.V + colw + 16 * ct + n16,
                                      p.scale * acc[ct][i]);
                    }
            }
        }
        // h' = e^{gam_last} h + K^T (exp(gam_last - gam) U~)
        {
            ST rus[2][NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                f32x4 y[4];
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) y[rt][i] = rr[16 * rt + 4 * g + i] * ut[rt][ct][i];
                rus[0][ct] = O::split(y[0], y[1]);
                rus[1][ct] = O::split(y[2], y[3]);
            }
            const float ec = eg[CH - 1];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) h[dt][ct] *= ec;
#pragma unroll
                for (int ip = 0; ip < 2; ++ip) {
                    const XT a = gather_kt<In>(Ks, LDK, 16 * dt + n16, ip);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) h[dt][ct] = mma(h[dt][ct], a, rus[ip][ct]);
                }
            }
        }
    }
    if (c_end == N && p.hT) {
        float *hT = p.hT + (int64_t)unit * KV;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    hT[(16 * dt + 4 * g + i) * p.V + colw + 16 * ct + n16] = h[dt][ct][i];
    }
}

template <typename In, typename Out, int KD, int NCT>
hipError_t launch_scan_t(const ScanParams &p, hipStream_t s) {
    using L = ScanLayout<In, KD, NCT>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&scan_output_kernel<In, Out, KD, NCT>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
    (void)attr;  // a refusal shows up as a launch error below
    const int nb = p.n_vt * p.n_units * p.n_seg;
    hipLaunchKernelGGL((scan_output_kernel<In, Out, KD, NCT>), dim3(nb), dim3(NTHR), L::bytes, s, p);
    return hipGetLastError();
}

template <typename In, typename Out>
hipError_t launch_scan_k(int K, const ScanParams &p, hipStream_t s) {
    if (K == 128) return launch_scan_t<In, Out, 128, 1>(p, s);
    return launch_scan_t<In, Out, 64, 1>(p, s);
}

}  // namespace

int scan_vtile(Dt, int, int V) { return V < 64 ? V : 64; }

hipError_t launch_scan_output(Dt dt, Dt out, int K, int V, const ScanParams &p, hipStream_t s) {
    (void)V;
    if (dt == Dt::BF16)
        return out == Dt::F32 ? launch_scan_k<bf16, float>(K, p, s) : launch_scan_k<bf16, bf16>(K, p, s);
    return out == Dt::F32 ? launch_scan_k<float, float>(K, p, s) : launch_scan_k<float, bf16>(K, p, s);
}

}  // namespace gdr
