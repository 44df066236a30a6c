// gdr_scan_output — the serial inter-chunk scan fused with the output.
//
// One workgroup owns one (sequence, v-head, block of 64 value columns) and
// walks the chunks of its segment in order.  Wave w keeps columns
// [16w, 16w+16) of the block of the K x V state h in registers (fp32,
// accumulator order).  For a chunk of n tokens with start state h (the
// chunked form of the gated delta rule):
//
//   X  = beta * (V - diag(e^gam) K h)          (delta-rule target before the
//                                                in-chunk correction)
//   U~ = T X            = U - W h              (the "V correction": with
//                                                U = T diag(beta) V and
//                                                W = T diag(beta e^gam) K)
//   O  = scale (diag(e^gam) Q h + P U~),  P = tril(Q K^T) * exp(gam_r - gam_i)
//   h' = e^{gam_last} h + K^T (exp(gam_last - gam) * U~)
//
// T (split into bf16 hi/lo planes) and the gate scalars come from
// gdr_chunk_prep as one LDS image per (chunk, v head).  Columns of h evolve
// independently, so waves never exchange state; the waves share the decayed
// scores P through LDS, formed as ten 16x16 K Q^T tiles, whose accumulator
// layout is P's A operand.  Two forms: scan_output_kernel (four waves, each
// owning 16 state columns; waves 2 and 3 form the score tiles while waves 0
// and 1 issue the next chunk's copies) serves fp32 inputs and the states
// pass, and scan_output_roles_kernel (eight waves, the role split below)
// serves the bf16 forward.  Products with fp32 operands use split-bf16 MFMA
// (gdr_device.hpp); accumulation is fp32.
//
// Data movement: K, Q, the V columns and the T block of the next chunk are
// copied global -> LDS by the waves' direct-to-LDS loads while the current
// chunk computes (two LDS buffers, bf16 inputs), into XOR-swizzled rows
// (gdr_layout.hpp).  The K^T operand of the state update and the V columns
// are read with the gfx950 transposing LDS read.  In the four-wave form each
// wave keeps its output tiles in registers and stores them (16 bytes per lane
// and row) at the start of the next chunk.
//
// Sequence split (the pages' AutoCP with its sliding-window warm-up): with
// seg_chunks smaller than the sequence, segment s > 0 starts from a zero
// state warm_chunks chunks before its first chunk (from the true initial
// state when that window reaches chunk 0) and runs the scan without output
// over the window before its own chunks.  With warm_gated the window is
// chosen from the gates instead (gated_window_start): the shortest one whose
// decay makes the zero start as good as the true state in fp32, or the whole
// prefix when the gates do not decay that much.  For the exact split a segment can
// instead start from a given state (h0_seg) or from the identity over a
// shared zero row of values (its end state is then the segment's transition
// matrix), and hand its end state to hT_seg; carry_kernel below chains them.
#include <type_traits>

#include "gdr_kernels.hpp"
#include "gdr_lds.hpp"

namespace gdr {

namespace {

constexpr int BV = 64;  // value columns per workgroup (16 per wave)

// FULLT: the backward's T blocks (the states pass), else the forward's
template <typename In, int KD, bool FULLT = false> struct Cfg {
    static constexpr bool BF = sizeof(In) == 2;
    static constexpr int NB = BF ? 2 : 1;          // LDS buffers
    static constexpr int ES = sizeof(In);
    static constexpr int EV = 16 / ES;             // elements per 16-byte chunk
    static constexpr int KROW = KD * ES, VROW = BV * ES;
    static constexpr int KT = CH * KROW, VT = CH * VROW;
    using TB = typename std::conditional<FULLT && !BF, TBlock<In>, TBlockF<In>>::type;
    static constexpr int OFF_K = 0, OFF_Q = KT, OFF_V = 2 * KT, OFF_T = 2 * KT + VT;
    static constexpr int BUF = OFF_T + TB::BYTES;
    static constexpr int PROW = CH * (BF ? 2 : 4);  // score plane row bytes
    static constexpr int PBYTES = CH * PROW * (BF ? 2 : 1);
    static constexpr int NKI = KT / 1024, NVI = VT / 1024, NTI = TB::BYTES / 1024;
    static_assert(NKI % 2 == 0 && NVI % 2 == 0, "tile copies spread over 2 waves");
    static constexpr int DT = KD / 16, DP = KD / 32;
};

// o is written with nontemporal stores: nothing in the kernel reads it back, and
// lines streamed past L2 leave less to write back when the kernel ends
template <typename T> struct OutVec;
template <> struct OutVec<float> {
    static __device__ __forceinline__ void put(float *p, f32x4 x) {
        __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>(p));
    }
};
template <> struct OutVec<bf16> {
    static __device__ __forceinline__ void put(bf16 *p, f32x4 x) {
        __builtin_nontemporal_store(__builtin_convertvector(x, bf16x4), reinterpret_cast<bf16x4 *>(p));
    }
};

// STATES: the backward's states pass, which reads the backward's T blocks
template <typename In, typename Out, int KD, bool STATES> struct Scan {
    using C = Cfg<In, KD, STATES>;
    using O = Ops<In>;
    using XT = typename O::X;
    using ST = typename O::S;
    using TB = typename C::TB;
    using SK = Swz<C::KROW, KeyKQ>;
    using SV = Swz<C::VROW, KeyVP>;
    using SP = Swz<C::PROW, typename std::conditional<C::BF, KeyP, KeyVP>::type>;

    const ScanParams &p;
    char *buf[2];
    char *pplane;  // shared score planes (hi, lo)
    // work item
    int vt, unit, j, hv, hq, cb;
    int64_t bos, eos;
    int tid, w, n16, g, colw;
    const In *qp, *kp, *vp;
    Out *op;
    // state slice: h[dt][i] = key slot_base(dt, g) + i, column colw + n16, so that a
    // tile pair is a contiguous-slot operand (gdr_lds.hpp); the K h, X and U~ tiles
    // take their tokens in the same order, the score and output tiles in natural order
    f32x4 h[C::DT];
    // pending output bookkeeping
    int64_t pend_ts;
    int pend_n;

    __device__ __forceinline__ Scan(const ScanParams &p_) : p(p_) {}

    // Waves 0-1 issue the chunk copies (spreading them keeps each copy wave's
    // vmcnt wait short); every wave stores its own output columns.
    static constexpr int NCW = 2;  // copy waves
    // per-lane parts of the copies (fixed for the whole scan): row of the tile
    // this lane fills in each of its copies and the byte offset of its 16-byte
    // chunk inside that row
    int krow[C::NKI / NCW], kchk[C::NKI / NCW], vrow[C::NVI / NCW], vchk[C::NVI / NCW];

    __device__ __forceinline__ void setup_copies() {
        const int l = lane_id();
        const int cw = w < NCW ? w : 0;
#pragma unroll
        for (int s = 0; s < C::NKI / NCW; ++s) {
            const int byte = (cw + NCW * s) * 1024 + 16 * l, r = byte / C::KROW;
            krow[s] = r;
            kchk[s] = 16 * SK::chunk(r, (byte % C::KROW) / 16);
        }
#pragma unroll
        for (int s = 0; s < C::NVI / NCW; ++s) {
            const int byte = (cw + NCW * s) * 1024 + 16 * l, r = byte / C::VROW;
            vrow[s] = r;
            vchk[s] = 16 * SV::chunk(r, (byte % C::VROW) / 16);
        }
    }

    // copy chunk c into LDS buffer b (rows past the chunk end repeat its last row)
    __device__ __forceinline__ void issue(int c, char *b) {
        if (w >= NCW) return;
        const int64_t ts = bos + (int64_t)c * CH;
        const int nm1 = (int)min<int64_t>(CH, eos - ts) - 1;
        const int l = lane_id();
        const int krs = p.Hq * KD * C::ES, vrs = (int)(p.v_tok * C::ES);  // row strides (bytes)
        const char *kb = reinterpret_cast<const char *>(kp + (ts * p.Hq + hq) * KD);
        const char *qb = reinterpret_cast<const char *>(qp + (ts * p.Hq + hq) * KD);
        const char *vb = reinterpret_cast<const char *>(vp + ts * p.v_tok + hv * p.v_head + vt * BV);
#pragma unroll
        for (int s = 0; s < C::NKI / NCW; ++s) {
            const uint32_t off = (uint32_t)(min(krow[s], nm1) * krs + kchk[s]);
            const int i = w + NCW * s;
            dma16(kb + off, b + C::OFF_K + i * 1024);
            dma16(qb + off, b + C::OFF_Q + i * 1024);
        }
#pragma unroll
        for (int s = 0; s < C::NVI / NCW; ++s) {
            const uint32_t off = (uint32_t)(min(vrow[s], nm1) * vrs + vchk[s]);
            dma16(vb + off, b + C::OFF_V + (w + NCW * s) * 1024);
        }
        const char *blk = p.tblk + ((int64_t)(cb + c) * p.Hv + hv) * TB::BYTES;
        for (int i = w; i < C::NTI; i += NCW) dma16(blk + i * 1024 + 16 * l, b + C::OFF_T + i * 1024);
    }

    // output of the previous chunk, held in registers as O^T tiles: pend_o[rt]
    // holds o[token 16 rt + lane16][columns colw + 4g .. colw + 4g + 3]
    f32x4 pend_o[4];

    __device__ __forceinline__ void store_pending() {
        if (pend_ts < 0) return;
        Out *ob = op + (pend_ts * p.Hv + hv) * p.V + colw + 4 * g;
        const int rstride = p.Hv * p.V;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const int tok = 16 * rt + n16;
            if (tok < pend_n) OutVec<Out>::put(ob + (uint32_t)(tok * rstride), pend_o[rt]);
        }
        pend_ts = -1;
    }

    // one chunk; LDS buffer `b` holds it and every wave has passed the barrier after it landed
    template <bool EMIT, bool SNAP>
    __device__ __forceinline__ void step(int c, const char *b) {
        const char *Ks = b + C::OFF_K, *Qs = b + C::OFF_Q, *Vs = b + C::OFF_V, *Tb = b + C::OFF_T;
        const float *sc = reinterpret_cast<const float *>(Tb + TB::SC);
        const float *gam = sc, *eg = sc + CH, *rr = sc + 2 * CH, *bet = sc + 3 * CH;
        const int64_t ts = bos + (int64_t)c * CH;
        const int n = (int)min<int64_t>(CH, eos - ts);

        // decayed causal scores: this wave's share of the ten tiles (tr >= ti)
        if constexpr (EMIT) {
            // the ten tiles go to waves 2 and 3, five each: waves 0 and 1 issue the
            // copies of the next chunk meanwhile
#pragma unroll
            for (int k = 0; k < 5; ++k) {
                if (w < NCW) break;
                const int t = 2 * k + (w - NCW);
                const int tr = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
                const int ti = t - tr * (tr + 1) / 2;
                f32x4 acc = zero4();
#pragma unroll
                for (int dp = 0; dp < C::DP; ++dp)
                    acc = mma(acc, frag8<In, SK>(Ks, 16 * ti + n16, (32 * dp + 8 * g) * C::ES),
                              frag8<In, SK>(Qs, 16 * tr + n16, (32 * dp + 8 * g) * C::ES));
                // acc[jj] = P[r][i], r = 16 tr + n16, i = 16 ti + 4g + jj
                const int r = 16 * tr + n16;
                const float gr = gam[r];
                const f32x4 gi = *reinterpret_cast<const f32x4 *>(gam + 16 * ti + 4 * g);
                f32x4 v;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    v[jj] = (ti < tr || 4 * g + jj <= n16) ? acc[jj] * fast_exp(gr - gi[jj]) : 0.f;
                const int off = SP::off(r, (16 * ti + 4 * g) * (C::BF ? 2 : 4));
                if constexpr (C::BF) {
                    bf16x4 hi, lo;
                    split4(v, hi, lo);
                    *reinterpret_cast<bf16x4 *>(pplane + off) = hi;
                    *reinterpret_cast<bf16x4 *>(pplane + CH * C::PROW + off) = lo;
                } else {
                    *reinterpret_cast<f32x4 *>(pplane + off) = v;
                }
            }
        }
        if constexpr (SNAP) {
            if (p.hsnap) {
                float *hs = p.hsnap + ((int64_t)(cb + c) * p.Hv + hv) * (int64_t)KD * p.V;
                if (C::BF && p.hsnap_split) {  // hi, lo planes of h^T: this lane's 8 keys at its column
                    char *hb = reinterpret_cast<char *>(hs);
                    const int plane = KD * p.V * 2;
#pragma unroll
                    for (int dp = 0; dp < C::DP; ++dp) {  // tiles 2dp, 2dp + 1 hold keys 32dp + 8g .. + 7
                        bf16x4 hi0, lo0, hi1, lo1;
                        split4(h[2 * dp], hi0, lo0);
                        split4(h[2 * dp + 1], hi1, lo1);
                        const uint32_t off = (uint32_t)(((colw + n16) * KD + slot_base(2 * dp, g)) * 2);
                        *reinterpret_cast<bf16x8 *>(hb + off) = cat(hi0, hi1);
                        *reinterpret_cast<bf16x8 *>(hb + plane + off) = cat(lo0, lo1);
                    }
                } else {
                    // row stride made opaque per chunk: otherwise the 32 per-lane
                    // addresses are hoisted out of the chunk loop and held in registers
                    int rs = p.V;
                    asm volatile("" : "+s"(rs));
                    float *hl = hs + 8 * g * rs + colw + n16;
#pragma unroll
                    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            hl[(uint32_t)((32 * (dt >> 1) + 4 * (dt & 1) + i) * rs)] = h[dt][i];
                }
            }
        }

        // K h (chain) and Q h (output) for this wave's columns
        f32x4 kh[4], qh[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) kh[rt] = qh[rt] = zero4();
#pragma unroll
        for (int dp = 0; dp < C::DP; ++dp) {
            const ST hb = O::split(h[2 * dp], h[2 * dp + 1]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                kh[rt] = mma(kh[rt], frag8<In, SK>(Ks, slot_row(rt, n16), (32 * dp + 8 * g) * C::ES), hb);
                if constexpr (EMIT)  // (Q h)^T tile: lane (token, g) holds 4 output columns
                    qh[rt] = mma(qh[rt], hb, frag8<In, SK>(Qs, 16 * rt + n16, (32 * dp + 8 * g) * C::ES));
            }
        }
        // X = beta (V - e^gam K h), as the split B operand (k = tokens)
        ST xs0, xs1;
        {
            f32x4 x[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int tb = slot_base(rt, g);
                const f32x4 vv = rows4b<In, SV>(Vs, tb, w * 16);
                const f32x4 b4 = *reinterpret_cast<const f32x4 *>(bet + tb);
                const f32x4 e4 = *reinterpret_cast<const f32x4 *>(eg + tb);
                x[rt] = b4 * (vv - e4 * kh[rt]);
            }
            xs0 = O::split(x[0], x[1]);
            xs1 = O::split(x[2], x[3]);
        }
        // U~ = T X  (T unit lower triangular, zero rows past the chunk end)
        f32x4 ut[4];
        {
            SplitPlane<In> tp;
            tp.hi = reinterpret_cast<typename SplitPlaneT<In>::type *>(const_cast<char *>(Tb));
            tp.lo = reinterpret_cast<typename SplitPlaneT<In>::type *>(const_cast<char *>(Tb) + TB::PLANE);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                ut[rt] = zero4();
#pragma unroll
                for (int ip = 0; ip <= rt / 2; ++ip) {
                    const int row = slot_row(rt, n16), byte = (32 * ip + 8 * g) * (C::BF ? 2 : 4);
                    const int o0 = TB::off(row, byte), o1 = TB::off(row, byte + 16);
                    ut[rt] = mma(ut[rt], tp.get8(o0, o1), ip == 0 ? xs0 : xs1);
                }
            }
        }
        // h' = e^{gam_last} h + K^T (exp(gam_last - gam) U~)
        {
            f32x4 y[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) y[rt] = *reinterpret_cast<const f32x4 *>(rr + slot_base(rt, g)) * ut[rt];
            const ST rus0 = O::split(y[0], y[1]);
            const ST rus1 = O::split(y[2], y[3]);
            const float ec = eg[CH - 1];
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt) {
                h[dt] *= ec;
                const int c0 = 32 * (dt >> 1) + 4 * (dt & 1);
                h[dt] = mma(h[dt], kt8<In, SK>(Ks, 0, c0, 8), rus0);
                h[dt] = mma(h[dt], kt8<In, SK>(Ks, 32, c0, 8), rus1);
            }
        }
        ST us0, us1;
        f32x4 oq[4];
        if constexpr (EMIT) {
            us0 = O::split(ut[0], ut[1]);
            us1 = O::split(ut[2], ut[3]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) oq[rt] = eg[16 * rt + n16] * qh[rt];
        }
        __syncthreads();  // score planes complete
        if constexpr (EMIT) {
            // O^T = (Q h)^T diag(e^gam) + U~^T P^T; the split U~ serves as the A operand of U~^T
            // and the P fragments as the B operand of P^T
            SplitPlane<In> pp;
            pp.hi = reinterpret_cast<typename SplitPlaneT<In>::type *>(pplane);
            pp.lo = reinterpret_cast<typename SplitPlaneT<In>::type *>(pplane + CH * C::PROW);
            const int EB = C::BF ? 2 : 4;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 acc = oq[rt];
#pragma unroll
                for (int ip = 0; ip <= rt / 2; ++ip) {
                    const int row = 16 * rt + n16, byte = (32 * ip + 8 * g) * EB;
                    acc = mma(acc, ip == 0 ? us0 : us1, pp.get8(SP::off(row, byte), SP::off(row, byte + 16)));
                }
                pend_o[rt] = p.scale * acc;
            }
            pend_ts = ts;
            pend_n = n;
        }
    }

    // chunk c from buffer `cur`; chunk c+1 (if any) copied into `nxt` meanwhile
    template <int CUR>
    __device__ __forceinline__ void run(int c, int c_begin, int c_end) {
        char *cur = buf[C::NB == 2 ? CUR : 0];
        char *nxt = buf[C::NB == 2 ? 1 - CUR : 0];
        if constexpr (C::NB == 1) {
            issue(c, cur);
            store_pending();
            if (w < NCW) wait_dma();
            __syncthreads();
        } else {
            if (c + 1 < c_end) issue(c + 1, nxt);
            store_pending();
        }
        if constexpr (STATES)
            step<false, true>(c, cur);
        else if (c >= c_begin && p.o)
            step<true, true>(c, cur);
        else
            step<false, false>(c, cur);
        if (C::NB == 2 && w < NCW) wait_dma();
        __syncthreads();  // chunk c done with `cur`, chunk c+1 landed
    }
};

// First chunk of the gate-driven warm-up window of a segment that starts at
// chunk c_begin of its sequence: the latest chunk w such that the log-gates of
// chunks [w, c_begin) sum to -24 ln 2 or less, so that the zero-state start at
// w differs from the true state at c_begin by at most 2^-24 of the state at w
// (each token maps the state error e to e^g (I - beta k k^T) e, of norm at most
// e^g |e| for a unit key and 0 <= beta <= 2); 0 (the sequence start, from the
// true initial state, exact) when the gates of the whole prefix decay less.
// Each chunk's total log-gate is the last entry of its T block's running sum.
// Wave-uniform result; all lanes take part.
template <int TBYTES>
__device__ int gated_window_start(const char *tblk, int64_t cb, int Hv, int hv, int c_begin, int sc_off) {
    constexpr float LOG_2M24 = -16.6355323f;  // -24 ln 2
    const int l = lane_id();
    float acc = 0.f;
    int c = c_begin;
    while (c > 0) {
        const int cnt = min(c, 64);
        float x = 0.f;
        if (l < cnt)
            x = *reinterpret_cast<const float *>(tblk + ((cb + c - 1 - l) * Hv + hv) * (int64_t)TBYTES + sc_off +
                                                 4 * (CH - 1));
        const float ps = acc + wave_prefix_sum(x);  // chunks c-1 .. c-1-l
        const uint64_t hit = __ballot(l < cnt && ps <= LOG_2M24);
        if (hit) return c - 1 - __builtin_ctzll(hit);
        acc = __shfl(ps, cnt - 1);
        c -= cnt;
    }
    return 0;
}

// STATES: chunk-start states only (no scores, no output), for the backward
template <typename In, typename Out, int KD, bool STATES>
__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(1, 1))) void scan_output_kernel(const ScanParams p) {
    using C = Cfg<In, KD, STATES>;
    __shared__ __attribute__((aligned(16))) char buf0[C::BUF];
    __shared__ __attribute__((aligned(16))) char buf1[C::NB == 2 ? C::BUF : 16];
    __shared__ __attribute__((aligned(16))) char pplane[C::PBYTES];

    Scan<In, Out, KD, STATES> S(p);
    S.buf[0] = buf0;
    S.buf[1] = buf1;
    S.pplane = pplane;

    // work item: (v tile, v head, sequence, segment), XCD-grouped; packed sequences
    // of different lengths longest first
    int seg = 0;
    if (p.sm.order && p.n_seg == 1) {
        if (!lpt_item(p.sm, p.Hq, p.Hv, p.n_vt, S.vt, S.unit)) return;
    } else {
        const int wid = xcd_remap(blockIdx.x, gridDim.x);
        S.vt = wid % p.n_vt;
        const int rest = wid / p.n_vt;
        S.unit = rest % p.n_units;
        seg = rest / p.n_units;
    }
    S.j = S.unit / p.Hv;
    S.hv = S.unit % p.Hv;
    S.hq = S.hv / (p.Hv / p.Hq);
    p.sm.bounds(S.j, S.bos, S.eos);
    const int N = (int)((S.eos - S.bos + CH - 1) / CH);
    const int c_begin = seg * p.seg_chunks;
    if (c_begin >= N && !(N == 0 && seg == 0)) return;
    const int c_end = min(N, c_begin + p.seg_chunks);
    S.cb = p.sm.chunk_base(S.j);
    int w_begin = seg == 0 ? 0 : max(0, c_begin - p.warm_chunks);
    if (seg > 0 && p.warm_gated)
        w_begin = __builtin_amdgcn_readfirstlane(gated_window_start<C::TB::BYTES>(
            p.tblk, S.cb, p.Hv, S.hv, c_begin, C::TB::SC));

    S.tid = threadIdx.x;
    S.w = __builtin_amdgcn_readfirstlane(wave_id());
    S.n16 = ln16();
    S.g = lg4();
    S.colw = S.vt * BV + S.w * 16;
    S.qp = reinterpret_cast<const In *>(p.q);
    S.kp = reinterpret_cast<const In *>(p.k);
    S.vp = reinterpret_cast<const In *>(p.v);
    S.op = reinterpret_cast<Out *>(p.o);
    S.pend_ts = -1;
    S.pend_n = 0;
    S.setup_copies();
    const int64_t KV = (int64_t)KD * p.V;
    {
        const bool from_seg = seg > 0 && p.h0_seg != nullptr;
        const bool from_h0 = !from_seg && (w_begin == 0) && p.h0 != nullptr;
        const float *h0 = from_seg ? p.h0_seg + ((int64_t)S.unit * p.n_seg + seg) * KV
                          : from_h0 ? p.h0 + (int64_t)S.unit * KV : nullptr;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = slot_base(dt, S.g) + i;
                S.h[dt][i] = p.eye_h0 ? (key == S.colw + S.n16 ? 1.f : 0.f)
                             : h0 ? h0[key * p.V + S.colw + S.n16] : 0.f;
            }
    }
    // score-plane tiles above the diagonal pairs, (0,1) and (2,3), are read as zero and never written
    {
        using SP = typename Scan<In, Out, KD, STATES>::SP;
        constexpr int EB = C::BF ? 2 : 4;
        for (int idx = threadIdx.x; idx < 2 * 16 * 16; idx += NTHR) {
            const int t = idx >> 8, r = 32 * t + ((idx >> 4) & 15), i = 32 * t + 16 + (idx & 15);
            const int off = SP::off(r, i * EB);
            if constexpr (C::BF) {
                *reinterpret_cast<bf16 *>(pplane + off) = bf16(0.f);
                *reinterpret_cast<bf16 *>(pplane + CH * C::PROW + off) = bf16(0.f);
            } else {
                *reinterpret_cast<float *>(pplane + off) = 0.f;
            }
        }
    }
    wait_dma();  // initial-state loads done before the copy engine counts start
    if constexpr (C::NB == 2) {
        if (w_begin < c_end) S.issue(w_begin, buf0);
        wait_dma();
        __syncthreads();
    }
    for (int c = w_begin; c < c_end; c += 2) {
        S.template run<0>(c, c_begin, c_end);
        if (c + 1 < c_end) S.template run<1>(c + 1, c_begin, c_end);
    }
    S.store_pending();
    if (p.hT_seg) {
        float *hs = p.hT_seg + ((int64_t)S.unit * p.n_seg + seg) * KV;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) hs[(slot_base(dt, S.g) + i) * p.V + S.colw + S.n16] = S.h[dt][i];
    }
    if (c_end == N && p.hT) {
        float *hT = p.hT + (int64_t)S.unit * KV;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) hT[(slot_base(dt, S.g) + i) * p.V + S.colw + S.n16] = S.h[dt][i];
    }
}

// ------------------------------------------------------------------ role split
// The bf16 forward with eight waves, two per SIMD: waves 0-3 ("chain") own the
// state columns [16w, 16w+16) of the block and form K h, Q h, X, U~, h' and the
// output tiles, with no global memory traffic inside the chunk loop.  Waves 4-7
// ("io") serve them: waves 4-5 ("copy") issue the next chunk's direct-to-LDS
// copies and store each chunk's output, which the chain waves leave in an LDS
// plane, one chunk later as whole 256-byte token rows; waves 6-7 ("score") form
// the ten decayed score tiles.  Same work items, chunk order and split
// products as scan_output_kernel: the states are bit-identical to it, the
// output within a few fp32 ulps (the compiler contracts the score exponent
// differently in the two kernels).
template <typename In, typename Out, int KD> struct ScanRS {
    using C = Cfg<In, KD, false>;
    using O = Ops<In>;
    using ST = typename O::S;
    using TB = typename C::TB;
    using SK = Swz<C::KROW, KeyKQ>;
    using SV = Swz<C::VROW, KeyVP>;
    using SP = Swz<C::PROW, KeyP>;
    using SO = Swz<BV * 4>;  // fp32 output plane, 256-byte token rows
    static constexpr int NIO = 4;  // io waves
    static constexpr int NCP = 2;  // of which copy waves
    static_assert(C::BF, "bf16 inputs only");
};

template <typename In, typename Out, int KD>
__global__ __launch_bounds__(2 * NTHR) __attribute__((amdgpu_waves_per_eu(2, 2))) void scan_output_roles_kernel(
    const ScanParams p) {
    using R = ScanRS<In, Out, KD>;
    using C = typename R::C;
    using O = typename R::O;
    using ST = typename R::ST;
    using TB = typename R::TB;
    using SK = typename R::SK;
    using SV = typename R::SV;
    using SP = typename R::SP;
    using SO = typename R::SO;
    __shared__ __attribute__((aligned(16))) char buf0[C::BUF];
    __shared__ __attribute__((aligned(16))) char buf1[C::BUF];
    __shared__ __attribute__((aligned(16))) char pplane[C::PBYTES];
    __shared__ __attribute__((aligned(16))) char oplane[CH * BV * 4];

    int vt, unit, seg = 0;
    if (p.sm.order && p.n_seg == 1) {
        if (!lpt_item(p.sm, p.Hq, p.Hv, p.n_vt, vt, unit)) return;
    } else {
        const int wid = xcd_remap(blockIdx.x, gridDim.x);
        vt = wid % p.n_vt;
        const int rest = wid / p.n_vt;
        unit = rest % p.n_units;
        seg = rest / p.n_units;
    }
    const int j = unit / p.Hv, hv = unit % p.Hv, hq = hv / (p.Hv / p.Hq);
    int64_t bos, eos;
    p.sm.bounds(j, bos, eos);
    const int N = (int)((eos - bos + CH - 1) / CH);
    const int c_begin = seg * p.seg_chunks;
    if (c_begin >= N && !(N == 0 && seg == 0)) return;
    const int c_end = min(N, c_begin + p.seg_chunks);
    const int cb = p.sm.chunk_base(j);
    int w_begin = seg == 0 ? 0 : max(0, c_begin - p.warm_chunks);
    if (seg > 0 && p.warm_gated)
        w_begin = __builtin_amdgcn_readfirstlane(
            gated_window_start<C::TB::BYTES>(p.tblk, cb, p.Hv, hv, c_begin, C::TB::SC));
    const int wv = __builtin_amdgcn_readfirstlane(wave_id());
    const int n16 = ln16(), g = lg4(), l = lane_id();
    const int64_t KV = (int64_t)KD * p.V;
    const bool emit_any = p.o != nullptr;

    if (wv < 4) {
        // ------------------------------------------------------------ chain waves
        const int colw = vt * BV + wv * 16;
        f32x4 h[C::DT];
        {
            const bool from_seg = seg > 0 && p.h0_seg != nullptr;
            const bool from_h0 = !from_seg && (w_begin == 0) && p.h0 != nullptr;
            const float *h0 = from_seg ? p.h0_seg + ((int64_t)unit * p.n_seg + seg) * KV
                              : from_h0 ? p.h0 + (int64_t)unit * KV : nullptr;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = slot_base(dt, g) + i;
                    h[dt][i] = p.eye_h0 ? (key == colw + n16 ? 1.f : 0.f) : h0 ? h0[key * p.V + colw + n16] : 0.f;
                }
        }
        __syncthreads();  // first chunk landed
        for (int c = w_begin; c < c_end; ++c) {
            const char *b = ((c - w_begin) & 1) ? buf1 : buf0;
            const bool emit = emit_any && c >= c_begin;
            const char *Ks = b + C::OFF_K, *Qs = b + C::OFF_Q, *Vs = b + C::OFF_V, *Tb = b + C::OFF_T;
            const float *sc = reinterpret_cast<const float *>(Tb + TB::SC);
            const float *eg = sc + CH, *rr = sc + 2 * CH, *bet = sc + 3 * CH;
            if (p.hsnap && c >= c_begin) {  // the segment's own chunks (not its warm-up window)
                float *hs = p.hsnap + ((int64_t)(cb + c) * p.Hv + hv) * KV;
                if (p.hsnap_split) {
                    char *hb = reinterpret_cast<char *>(hs);
                    const int plane = KD * p.V * 2;
#pragma unroll
                    for (int dp = 0; dp < C::DP; ++dp) {
                        bf16x4 hi0, lo0, hi1, lo1;
                        split4(h[2 * dp], hi0, lo0);
                        split4(h[2 * dp + 1], hi1, lo1);
                        const uint32_t off = (uint32_t)(((colw + n16) * KD + slot_base(2 * dp, g)) * 2);
                        // streamed past L2: nothing reads them before the backward
                        __builtin_nontemporal_store(cat(hi0, hi1), reinterpret_cast<bf16x8 *>(hb + off));
                        __builtin_nontemporal_store(cat(lo0, lo1), reinterpret_cast<bf16x8 *>(hb + plane + off));
                    }
                } else {
                    int rs = p.V;
                    asm volatile("" : "+s"(rs));
                    float *hl = hs + 8 * g * rs + colw + n16;
#pragma unroll
                    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            hl[(uint32_t)((32 * (dt >> 1) + 4 * (dt & 1) + i) * rs)] = h[dt][i];
                }
            }
            f32x4 kh[4], qh[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) kh[rt] = qh[rt] = zero4();
            // K h first, on the chain; Q h (also for warm-up chunks, whose output is
            // dropped: one straight-line block for the scheduler) queues behind it on
            // the matrix unit while X is formed
            ST hb[C::DP];
#pragma unroll
            for (int dp = 0; dp < C::DP; ++dp) {
                hb[dp] = O::split(h[2 * dp], h[2 * dp + 1]);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
                    kh[rt] = mma(kh[rt], frag8<In, SK>(Ks, slot_row(rt, n16), (32 * dp + 8 * g) * C::ES), hb[dp]);
            }
#pragma unroll
            for (int dp = 0; dp < C::DP; ++dp)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
                    qh[rt] = mma(qh[rt], hb[dp], frag8<In, SK>(Qs, 16 * rt + n16, (32 * dp + 8 * g) * C::ES));
            ST xs0, xs1;
            {
                f32x4 x[4];
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const int tb = slot_base(rt, g);
                    const f32x4 vv = rows4b<In, SV>(Vs, tb, wv * 16);
                    const f32x4 b4 = *reinterpret_cast<const f32x4 *>(bet + tb);
                    const f32x4 e4 = *reinterpret_cast<const f32x4 *>(eg + tb);
                    x[rt] = b4 * (vv - e4 * kh[rt]);
                }
                xs0 = O::split(x[0], x[1]);
                xs1 = O::split(x[2], x[3]);
            }
            f32x4 ut[4];
            {
                SplitPlane<In> tp;
                tp.hi = reinterpret_cast<bf16 *>(const_cast<char *>(Tb));
                tp.lo = reinterpret_cast<bf16 *>(const_cast<char *>(Tb) + TB::PLANE);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    ut[rt] = zero4();
#pragma unroll
                    for (int ip = 0; ip <= rt / 2; ++ip) {
                        const int row = slot_row(rt, n16), byte = (32 * ip + 8 * g) * 2;
                        ut[rt] = mma(ut[rt], tp.get8(TB::off(row, byte), 0), ip == 0 ? xs0 : xs1);
                    }
                }
            }
            {
                f32x4 y[4];
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) y[rt] = *reinterpret_cast<const f32x4 *>(rr + slot_base(rt, g)) * ut[rt];
                const ST rus0 = O::split(y[0], y[1]);
                const ST rus1 = O::split(y[2], y[3]);
                const float ec = eg[CH - 1];
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt) {
                    h[dt] *= ec;
                    const int c0 = 32 * (dt >> 1) + 4 * (dt & 1);
                    h[dt] = mma(h[dt], kt8<In, SK>(Ks, 0, c0, 8), rus0);
                    h[dt] = mma(h[dt], kt8<In, SK>(Ks, 32, c0, 8), rus1);
                }
            }
            if (emit) {
                const ST us0 = O::split(ut[0], ut[1]);
                const ST us1 = O::split(ut[2], ut[3]);
                f32x4 oq[4];
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) oq[rt] = eg[16 * rt + n16] * qh[rt];
                lds_barrier();  // score planes complete, output plane free
                SplitPlane<In> pp;
                pp.hi = reinterpret_cast<bf16 *>(pplane);
                pp.lo = reinterpret_cast<bf16 *>(pplane + CH * C::PROW);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    f32x4 acc = oq[rt];
#pragma unroll
                    for (int ip = 0; ip <= rt / 2; ++ip) {
                        const int row = 16 * rt + n16, byte = (32 * ip + 8 * g) * 2;
                        acc = mma(acc, ip == 0 ? us0 : us1, pp.get8(SP::off(row, byte), 0));
                    }
                    *reinterpret_cast<f32x4 *>(oplane + SO::off(16 * rt + n16, (wv * 16 + 4 * g) * 4)) = p.scale * acc;
                }
            }
            lds_barrier();  // chunk done with its buffer, the next one landed, output plane written
        }
        if (p.hT_seg) {
            float *hs = p.hT_seg + ((int64_t)unit * p.n_seg + seg) * KV;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) hs[(slot_base(dt, g) + i) * p.V + colw + n16] = h[dt][i];
        }
        if (c_end == N && p.hT) {
            float *hT = p.hT + (int64_t)unit * KV;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) hT[(slot_base(dt, g) + i) * p.V + colw + n16] = h[dt][i];
        }
    } else {
        // --------------------------------------------------------------- io waves
        // waves 4-5 copy the next chunk and store the output, waves 6-7 form the
        // decayed score tiles (five each)
        const int iw = wv - 4;
        const In *qp = reinterpret_cast<const In *>(p.q), *kp = reinterpret_cast<const In *>(p.k);
        const In *vp = reinterpret_cast<const In *>(p.v);
        // score-plane tiles above the diagonal pairs, (0,1) and (2,3), are read as zero and never written
        for (int idx = threadIdx.x - 4 * 64; idx < 2 * 16 * 16; idx += R::NIO * 64) {
            const int t = idx >> 8, r = 32 * t + ((idx >> 4) & 15), i = 32 * t + 16 + (idx & 15);
            const int off = SP::off(r, i * 2);
            *reinterpret_cast<bf16 *>(pplane + off) = bf16(0.f);
            *reinterpret_cast<bf16 *>(pplane + CH * C::PROW + off) = bf16(0.f);
        }
        if (iw < R::NCP) {
            // copy pieces of this wave (fixed for the whole scan)
            constexpr int NK = C::NKI / R::NCP, NV = C::NVI / R::NCP;
            static_assert(C::NKI % R::NCP == 0 && C::NVI % R::NCP == 0, "copies spread over the copy waves");
            int krow[NK], kchk[NK], vrow[NV], vchk[NV];
#pragma unroll
            for (int s = 0; s < NK; ++s) {
                const int byte = (iw + R::NCP * s) * 1024 + 16 * l, r = byte / C::KROW;
                krow[s] = r;
                kchk[s] = 16 * SK::chunk(r, (byte % C::KROW) / 16);
            }
#pragma unroll
            for (int s = 0; s < NV; ++s) {
                const int byte = (iw + R::NCP * s) * 1024 + 16 * l, r = byte / C::VROW;
                vrow[s] = r;
                vchk[s] = 16 * SV::chunk(r, (byte % C::VROW) / 16);
            }
            auto issue = [&](int c, char *b) {
                const int64_t ts = bos + (int64_t)c * CH;
                const int nm1 = (int)min<int64_t>(CH, eos - ts) - 1;
                const int krs = p.Hq * KD * C::ES, vrs = (int)(p.v_tok * C::ES);
                const char *kb = reinterpret_cast<const char *>(kp + (ts * p.Hq + hq) * KD);
                const char *qb = reinterpret_cast<const char *>(qp + (ts * p.Hq + hq) * KD);
                const char *vb = reinterpret_cast<const char *>(vp + ts * p.v_tok + hv * p.v_head + vt * BV);
#pragma unroll
                for (int s = 0; s < NK; ++s) {
                    const uint32_t off = (uint32_t)(min(krow[s], nm1) * krs + kchk[s]);
                    const int i = iw + R::NCP * s;
                    dma16(kb + off, b + C::OFF_K + i * 1024);
                    dma16(qb + off, b + C::OFF_Q + i * 1024);
                }
#pragma unroll
                for (int s = 0; s < NV; ++s) {
                    const uint32_t off = (uint32_t)(min(vrow[s], nm1) * vrs + vchk[s]);
                    dma16(vb + off, b + C::OFF_V + (iw + R::NCP * s) * 1024);
                }
                const char *blk = p.tblk + ((int64_t)(cb + c) * p.Hv + hv) * TB::BYTES;
                for (int i = iw; i < C::NTI; i += R::NCP) dma16(blk + i * 1024 + 16 * l, b + C::OFF_T + i * 1024);
            };
            // output of chunk c from the output plane: this wave's 32 token rows, 4
            // rows per instruction
            auto store_out = [&](int c) {
                const int64_t ts = bos + (int64_t)c * CH;
                const int n = (int)min<int64_t>(CH, eos - ts);
                Out *ob = reinterpret_cast<Out *>(p.o) + (ts * p.Hv + hv) * p.V + vt * BV + 4 * n16;
                const int rstride = p.Hv * p.V;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int tok = 32 * iw + 4 * k + g;
                    const f32x4 x = *reinterpret_cast<const f32x4 *>(oplane + SO::off(tok, 16 * n16));
                    if (tok < n) OutVec<Out>::put(ob + (uint32_t)(tok * rstride), x);
                }
            };
            if (w_begin < c_end) issue(w_begin, buf0);
            wait_dma();
            __syncthreads();  // first chunk landed
            int pend = -1;
            for (int c = w_begin; c < c_end; ++c) {
                char *nb = ((c - w_begin) & 1) ? buf0 : buf1;
                const bool emit = emit_any && c >= c_begin;
                if (c + 1 < c_end) issue(c + 1, nb);
                if (pend >= 0) store_out(pend);
                pend = -1;
                if (emit) {
                    lds_barrier();  // score planes complete, output plane free
                    pend = c;
                }
                wait_dma();
                lds_barrier();  // chunk done with its buffer, the next one landed, output plane written
            }
            if (pend >= 0) store_out(pend);
        } else {
            // tiles t = PAR, PAR + 2, ... of the ten on or below the diagonal (t -> (tr, ti)
            // row-major), every operand read issued before the first product
            auto tiles = [&](auto par_tag, const char *b) {
                constexpr int PAR = decltype(par_tag)::value;
                const char *Ks = b + C::OFF_K, *Qs = b + C::OFF_Q;
                const float *gam = reinterpret_cast<const float *>(b + C::OFF_T + TB::SC);
                typename O::X kf[5][C::DP], qf[5][C::DP];
#pragma unroll
                for (int k = 0; k < 5; ++k) {
                    const int t = PAR + 2 * k;
                    const int tr = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
                    const int ti = t - tr * (tr + 1) / 2;
#pragma unroll
                    for (int dp = 0; dp < C::DP; ++dp) {
                        kf[k][dp] = frag8<In, SK>(Ks, 16 * ti + n16, (32 * dp + 8 * g) * 2);
                        qf[k][dp] = frag8<In, SK>(Qs, 16 * tr + n16, (32 * dp + 8 * g) * 2);
                    }
                }
#pragma unroll
                for (int k = 0; k < 5; ++k) {
                    const int t = PAR + 2 * k;
                    const int tr = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
                    const int ti = t - tr * (tr + 1) / 2;
                    f32x4 acc = zero4();
#pragma unroll
                    for (int dp = 0; dp < C::DP; ++dp) acc = mma(acc, kf[k][dp], qf[k][dp]);
                    // acc[jj] = P[r][i], r = 16 tr + n16, i = 16 ti + 4g + jj
                    const int r = 16 * tr + n16;
                    const float gr = gam[r];
                    const f32x4 gi = *reinterpret_cast<const f32x4 *>(gam + 16 * ti + 4 * g);
                    f32x4 v;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const float e = acc[jj] * fast_exp(gr - gi[jj]);
                        v[jj] = (ti < tr || 4 * g + jj <= n16) ? e : 0.f;
                    }
                    const int off = SP::off(r, (16 * ti + 4 * g) * 2);
                    bf16x4 hi, lo;
                    split4(v, hi, lo);
                    *reinterpret_cast<bf16x4 *>(pplane + off) = hi;
                    *reinterpret_cast<bf16x4 *>(pplane + CH * C::PROW + off) = lo;
                }
            };
            __syncthreads();  // first chunk landed
            for (int c = w_begin; c < c_end; ++c) {
                const char *b = ((c - w_begin) & 1) ? buf1 : buf0;
                if (emit_any && c >= c_begin) {
                    if (iw == R::NCP)
                        tiles(std::integral_constant<int, 0>{}, b);
                    else
                        tiles(std::integral_constant<int, 1>{}, b);
                    lds_barrier();  // score planes complete, output plane free
                }
                lds_barrier();  // chunk done with its buffer, the next one landed, output plane written
            }
        }
    }
}

template <typename In, typename Out, int KD, bool STATES>
hipError_t launch_scan_t(const ScanParams &p, hipStream_t s) {
    const int nb = p.sm.order && p.n_seg == 1 ? lpt_blocks(p.sm.n_seq, p.Hq, p.Hv, p.n_vt)
                                              : p.n_vt * p.n_units * p.n_seg;
    if constexpr (sizeof(In) == 2 && !STATES)
        launch_k((scan_output_roles_kernel<In, Out, KD>), dim3(nb), dim3(2 * NTHR), 0, s, p);
    else
        launch_k((scan_output_kernel<In, Out, KD, STATES>), dim3(nb), dim3(NTHR), 0, s, p);
    return hipGetLastError();
}

template <typename In, typename Out, bool STATES = false>
hipError_t launch_scan_k(int K, const ScanParams &p, hipStream_t s) {
    if (K == 128) return launch_scan_t<In, Out, 128, STATES>(p, s);
    return launch_scan_t<In, Out, 64, STATES>(p, s);
}

// Carry of the exact sequence split, one workgroup per (unit, 16 value
// columns): start(1) = b(0), start(s + 1) = M(s) start(s) + b(s).  The 16
// columns of start(s) stay in LDS; wave w forms the row tiles 2w, 2w + 1 of the
// next start on fp32 MFMA, with the rows of M(s) read from memory as A operands
// (k = 16 dt + 4 g + j in instruction j, the B operand's rows in the same order).
// The reverse carry (rev) runs the segments backwards with M(s)^T.  Each step's
// operands from memory (its rows of M and b) are loaded during the step before.
template <int KD>
__global__ __launch_bounds__(NTHR) void carry_kernel(const CarryParams p) {
    constexpr int MT = KD / 16;
    __shared__ float hs[KD * 16];
    const int unit = blockIdx.x, c0 = blockIdx.y * 16;
    int64_t bos, eos;
    p.sm.bounds(unit / p.Hv, bos, eos);
    const int N = (int)((eos - bos + CH - 1) / CH);
    const int nseg = (N + p.seg_chunks - 1) / p.seg_chunks;
    if (nseg < 2) return;
    const int V = p.V;
    const int w = wave_id(), n16 = ln16(), g = lg4();
    const int64_t KV = (int64_t)KD * V, KK = (int64_t)KD * KD, base = (int64_t)unit * p.n_seg;
    // first carried segment: forward start(1) = b(0); reverse end(n-2) = b(n-1)
    const int first_src = p.rev ? nseg - 1 : 0, first_dst = p.rev ? nseg - 2 : 1;
    for (int idx = threadIdx.x; idx < KD * 16; idx += NTHR) {
        const int r = idx >> 4, c = idx & 15;
        const float v = p.b[(base + first_src) * KV + r * V + c0 + c];
        hs[r * 16 + c] = v;
        p.h0_seg[(base + first_dst) * KV + r * V + c0 + c] = v;
    }
    // this wave's row tiles: 2w, 2w + 1 (K = 128) or w (K = 64)
    constexpr int NT = MT >= 8 ? 2 : 1;
    const bool active = (MT >= 8 ? 2 * w : w) < MT;
    f32x4 a[NT][MT], bt[NT];
    auto load = [&](int s) {
        const float *Ms = p.M + (base + s) * KK;
        const float *bs = p.b + (base + s) * KV;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int mt = (MT >= 8 ? 2 * w : w) + t;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) bt[t][jj] = bs[(16 * mt + 4 * g + jj) * V + c0 + n16];
#pragma unroll
            for (int dt = 0; dt < MT; ++dt) {
                if (p.rev) {  // rows of M^T: columns of M
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) a[t][dt][jj] = Ms[(16 * dt + 4 * g + jj) * KD + 16 * mt + n16];
                } else {
                    a[t][dt] = *reinterpret_cast<const f32x4 *>(Ms + (16 * mt + n16) * KD + 16 * dt + 4 * g);
                }
            }
        }
    };
    auto seg_of = [&](int step) { return p.rev ? nseg - 1 - step : step; };
    if (active && nseg > 2) load(seg_of(1));
    __syncthreads();
    for (int step = 1; step + 1 < nseg; ++step) {
        const int s = seg_of(step), dst = p.rev ? s - 1 : s + 1;
        f32x4 acc[NT];
        if (active) {
            f32x4 y[MT];  // B operands: rows 16 dt + 4 g + j of start(s), read up front
#pragma unroll
            for (int dt = 0; dt < MT; ++dt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) y[dt][jj] = hs[(16 * dt + 4 * g + jj) * 16 + n16];
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[t] = bt[t];
#pragma unroll
            for (int dt = 0; dt < MT; ++dt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t][dt][jj], y[dt][jj], acc[t], 0, 0, 0);
            if (step + 2 < nseg) load(seg_of(step + 1));  // the next step's operands
        }
        // barriers that wait for LDS only: the stores of the carried states and the
        // loads of the next step's operands stay in flight
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // start(s) read by every wave
        if (active) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int mt = (MT >= 8 ? 2 * w : w) + t;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int r = 16 * mt + 4 * g + jj;
                    hs[r * 16 + n16] = acc[t][jj];
                    p.h0_seg[(base + dst) * KV + r * V + c0 + n16] = acc[t][jj];
                }
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
}

__global__ void fill_zero_kernel(uint32_t *p, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0;
}

}  // namespace

hipError_t launch_carry(const CarryParams &p, int n_units, hipStream_t s) {
    if (p.K == 128)
        launch_k(carry_kernel<128>, dim3(n_units, p.V / 16), dim3(NTHR), 0, s, p);
    else
        launch_k(carry_kernel<64>, dim3(n_units, p.V / 16), dim3(NTHR), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s) {
    launch_k(fill_zero_kernel, dim3(1), dim3(256), 0, s, static_cast<uint32_t *>(p), bytes / 4);
    return hipGetLastError();
}

int scan_vtile(Dt, int, int) { return BV; }

hipError_t launch_scan_output(Dt dt, Dt out, int K, int V, const ScanParams &p, hipStream_t s) {
    (void)V;
    if (dt == Dt::BF16)
        return out == Dt::F32 ? launch_scan_k<bf16, float>(K, p, s) : launch_scan_k<bf16, bf16>(K, p, s);
    return out == Dt::F32 ? launch_scan_k<float, float>(K, p, s) : launch_scan_k<float, bf16>(K, p, s);
}

hipError_t launch_scan_states(Dt dt, int K, const ScanParams &p, hipStream_t s) {
    if (dt == Dt::BF16) return launch_scan_k<bf16, float, true>(K, p, s);
    return launch_scan_k<float, float, true>(K, p, s);
}

}  // namespace gdr
