// Host side of the libgdr C ABI: argument validation, workspace sizing, the
// sequence-split decision and kernel launches.  Declarations and the
// contract of every entry point are in include/gdr.h.
#include <math.h>
#include <string.h>

#include <algorithm>

#include "../../include/gdr.h"
#include "gdr_kernels.hpp"

using namespace gdr;

namespace gdr {
StageEvents &stage_events() {
    static thread_local StageEvents e = {nullptr, nullptr, false};
    return e;
}
}  // namespace gdr

namespace {

// leaves no timing stage open on this thread when an entry point returns
struct StageGuard {
    ~StageGuard() { stage_events() = {nullptr, nullptr, false}; }
};

constexpr size_t ALIGN = 256;
size_t up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }
bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
// Packed sequences up to this count are scanned longest first (their order is
// computed on the device with one thread per sequence, O(n_seq^2) work).
constexpr int64_t LPT_MAX_SEQ = 8192;
bool use_lpt(bool varlen, int64_t n_seq) { return varlen && n_seq <= LPT_MAX_SEQ; }
// varlen bookkeeping: chunk offsets [n_seq + 1], the clamped sequence bounds
// [n_seq + 1] that every kernel reads, then the length order [n_seq]
size_t seq_table_bytes(bool varlen, int64_t n_seq) {
    if (!varlen) return 0;
    return up(sizeof(int32_t) * (size_t)(2 * (n_seq + 1) + (use_lpt(varlen, n_seq) ? n_seq : 0)));
}
// the table's parts, from its base (the chunk offsets)
int32_t *seq_bounds(int32_t *chunk_off, int64_t n_seq) { return chunk_off + n_seq + 1; }
int32_t *seq_order(int32_t *chunk_off, int64_t n_seq) { return chunk_off + 2 * (n_seq + 1); }

struct FwdPlan {
    int64_t n_seq, tokens, nct, nt_ub;  // nct: chunks per sequence bound
    size_t off_chunk, off_tblk, total;
    size_t tblk_bytes;  // the scan's T blocks in the workspace
    size_t tblk_bwd_bytes;  // their copy in the backward's layout (tblk_bwd)
    // exact split: segment transitions, zero-start end states, true start states, a zero row
    size_t off_M, off_b, off_hseg, off_zero;
    int seg_chunks, warm_chunks, n_seg;
    bool split, exact, gated;  // gated: gate-driven warm-up windows (GDR_CP_AUTO)
};

int check_dims(int64_t B, int64_t T, int64_t Hq, int64_t Hv, int64_t K, int64_t V, int64_t n_seq,
               bool varlen, int32_t dtype) {
    if (B < 1 || T < 0 || Hq < 1 || Hv < 1) return GDR_EINVAL;
    if (Hv % Hq != 0) return GDR_EINVAL;
    if (varlen && (B != 1 || n_seq < 1)) return GDR_EINVAL;
    if (dtype != GDR_BF16 && dtype != GDR_F32) return GDR_ENOTSUP;
    if ((K != 64 && K != 128) || (V != 64 && V != 128)) return GDR_ENOTSUP;
    // 32-bit limits of the chunk bookkeeping
    if (B * T >= (int64_t)1 << 31 || (varlen ? n_seq : B) * Hv > (int64_t)1 << 30) return GDR_EINVAL;
    return GDR_OK;
}

// Segment length of the sequence split when the caller leaves it open.  The
// scan runs one workgroup per compute unit, so a launch of W workgroups per
// segment index takes ceil(W S / slots) rounds, each as long as the longest
// segment: choose the segment count S >= min_seg that minimises, in chunk steps,
//   warm-up split:  rounds x (L + wm)
//   exact split:    rounds x 3 L + (S - 1)   (transitions, zero-start states and
//                   output passes, one carry step per segment)
// with L = ceil(N / S) (ties: fewer segments); one segment costs rounds x N.
// Segment counts beyond eight rounds of the device are not considered.
// Returns N + 1 (no split) when one segment is best.
int64_t split_chunks(int64_t N, int64_t W, int64_t slots, int64_t wm, int64_t min_seg, bool exact = false) {
    int64_t best_t = -1, best_L = N + 1;
    const int64_t s_max = std::min(N, 8 * cdiv(slots, std::max<int64_t>(W, 1)));
    for (int64_t S = min_seg; S <= s_max; ++S) {
        const int64_t L = cdiv(N, S), Sx = cdiv(N, L);
        if (Sx != S) continue;  // same L as a smaller S
        const int64_t rounds = cdiv(W * S, slots);
        const int64_t t = S == 1 ? rounds * N : exact ? rounds * 3 * L + (S - 1) : rounds * (L + wm);
        if (best_t < 0 || t < best_t) {
            best_t = t;
            best_L = S > 1 ? L : N + 1;
        }
    }
    return best_L;
}

// Compute units assumed when no device can be queried (an MI355X has 256).
constexpr int64_t DEFAULT_SLOTS = 256;

// slots: workgroups the device runs at once (its compute units); 0 = unknown
int plan_fwd(const gdr_fwd_args *a, FwdPlan &pl, int64_t slots = 0) {
    if (!a) return GDR_EINVAL;
    const bool varlen = a->cu_seqlens != nullptr;
    int rc = check_dims(a->B, a->T, a->H_q, a->H_v, a->K, a->V, a->n_seq, varlen, a->dtype);
    if (rc) return rc;
    if (a->out_dtype != GDR_BF16 && a->out_dtype != GDR_F32) return GDR_ENOTSUP;
    if (a->cp_mode < GDR_CP_AUTO || a->cp_mode > GDR_CP_AUTO_PAGES) return GDR_EINVAL;
    if (a->cp_segment_chunks < 0 || a->cp_warmup_chunks < 0) return GDR_EINVAL;
    // the backward's states must be exact: no fixed warm-up window, and AUTO splits as AUTO_EXACT
    if (a->h_bwd && (a->h || a->cp_mode == GDR_CP_WARMUP || a->cp_mode == GDR_CP_AUTO_PAGES)) return GDR_EINVAL;
    const int32_t cp_mode = a->h_bwd && a->cp_mode == GDR_CP_AUTO ? GDR_CP_AUTO_EXACT : a->cp_mode;
    pl.n_seq = varlen ? a->n_seq : a->B;
    pl.tokens = a->B * a->T;
    pl.nct = cdiv(a->T, GDR_CHUNK);
    pl.nt_ub = varlen ? pl.nct + pl.n_seq : a->B * pl.nct;
    // the chunk-parallel kernels run one-dimensional grids of (chunk, q/k head)
    // workgroups of 256 threads (the chunks rounded up to a multiple of 8), at most
    // 2^32 work-items
    if ((pl.nt_ub + 7) * a->H_q >= (int64_t)1 << 24) return GDR_EINVAL;
    size_t off = 0;
    pl.off_chunk = off;
    off += seq_table_bytes(varlen, pl.n_seq);
    pl.off_tblk = off;
    const Dt pdt = a->dtype == GDR_BF16 ? Dt::BF16 : Dt::F32;
    pl.tblk_bwd_bytes = up(tblock_bytes(pdt) * (size_t)(pl.nt_ub * a->H_v));
    // bf16: the forward's T blocks are the backward's, so with tblk_bwd they are written
    // there and take no workspace
    pl.tblk_bytes = a->tblk_bwd && pdt == Dt::BF16 ? 0 : up(tblock_bytes_fwd(pdt) * (size_t)(pl.nt_ub * a->H_v));
    off += pl.tblk_bytes;
    pl.total = off;
    // sequence split ("AutoCP")
    const int64_t bh = pl.n_seq * a->H_v;
    // GDR_CP_AUTO: the device model decides, segments warm up over a gate-driven
    // window; GDR_CP_AUTO_EXACT: the device model decides, exact carry;
    // GDR_CP_AUTO_PAGES: the pages' trigger on batch x heads and length, fixed window
    const bool autom = cp_mode == GDR_CP_AUTO || cp_mode == GDR_CP_AUTO_EXACT || cp_mode == GDR_CP_AUTO_PAGES;
    const bool exact_mode = cp_mode == GDR_CP_EXACT || cp_mode == GDR_CP_AUTO_EXACT;
    const bool gated = cp_mode == GDR_CP_AUTO;
    bool split = cp_mode == GDR_CP_WARMUP || exact_mode || gated ||
                 (cp_mode == GDR_CP_AUTO_PAGES && (bh <= 40 || (bh <= 56 && a->T >= 8192)));
    pl.warm_chunks = a->cp_warmup_chunks > 0 ? a->cp_warmup_chunks : 8;
    const int64_t n_vt = a->V / scan_vtile(a->dtype == GDR_BF16 ? Dt::BF16 : Dt::F32, (int)a->K, (int)a->V);
    // the gate-driven window is priced at one chunk (gates that decay as the
    // workloads' do need one; a head whose gates do not decay costs its segments
    // up to the whole prefix, no more than rounds x N)
    int64_t L = a->cp_segment_chunks > 0
                    ? a->cp_segment_chunks
                    : split_chunks(pl.nct, bh * n_vt, slots > 0 ? slots : DEFAULT_SLOTS,
                                   gated ? 1 : pl.warm_chunks, autom ? 1 : 2, exact_mode);
    if (L < 1) L = 1;
    if (!split || L >= pl.nct) {
        split = false;
        L = pl.nct + 1;
    }
    pl.split = split;
    pl.exact = split && exact_mode;
    pl.gated = split && gated;
    if (pl.exact || pl.gated) pl.warm_chunks = 0;
    pl.seg_chunks = (int)L;
    // segments x units bounds the scan grids (x 2 column blocks) and the split's
    // workspace sizes; a caller's short segment length can otherwise overflow them
    if (split && cdiv(pl.nct, L) * bh > ((int64_t)1 << 30)) return GDR_EINVAL;
    pl.n_seg = split ? (int)cdiv(pl.nct, L) : 1;
    pl.off_M = pl.off_b = pl.off_hseg = pl.off_zero = 0;
    if (pl.exact) {
        const size_t per = (size_t)bh * pl.n_seg * (size_t)a->K * sizeof(float);
        pl.off_M = pl.total;
        pl.off_b = pl.off_M + up(per * (size_t)a->K);
        pl.off_hseg = pl.off_b + up(per * (size_t)a->V);
        pl.off_zero = pl.off_hseg + up(per * (size_t)a->V);
        pl.total = pl.off_zero + up(512);
    }
    return GDR_OK;
}

// compute units of a device: the scan's concurrent workgroups (one per unit); 0 on failure
int64_t device_slots(int dev) {
    int cus = 0;
    return hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0 ? cus
                                                                                                          : 0;
}

struct BwdPlan {
    int64_t n_seq, tokens, nct, nt_ub;
    size_t off_chunk, off_tblk, off_hs, off_dhs, total;
    // exact split: transitions, zero-start end states, true start states, zero-end
    // start gradients, true end gradients, a zero row
    size_t off_M, off_b, off_hseg, off_d, off_gseg, off_zero;
    int seg_chunks, n_seg;
    bool split;
};

// workspace: [chunk offsets] | T blocks | chunk-start states | chunk-end state
// gradients (T blocks and states only where the forward's are not given)
int plan_bwd(const gdr_bwd_args *a, BwdPlan &pl, int64_t slots = 0) {
    if (!a) return GDR_EINVAL;
    const bool varlen = a->cu_seqlens != nullptr;
    int rc = check_dims(a->B, a->T, a->H_q, a->H_v, a->K, a->V, a->n_seq, varlen, a->dtype);
    if (rc) return rc;
    if (a->grad_dtype != GDR_BF16 && a->grad_dtype != GDR_F32) return GDR_ENOTSUP;
    if (a->cp_mode != GDR_CP_AUTO && a->cp_mode != GDR_CP_OFF && a->cp_mode != GDR_CP_EXACT &&
        a->cp_mode != GDR_CP_AUTO_EXACT)
        return GDR_EINVAL;
    if (a->cp_segment_chunks < 0) return GDR_EINVAL;
    pl.n_seq = varlen ? a->n_seq : a->B;
    pl.tokens = a->B * a->T;
    pl.nct = cdiv(a->T, GDR_CHUNK);
    pl.nt_ub = varlen ? pl.nct + pl.n_seq : a->B * pl.nct;
    // the chunk-parallel kernels run one-dimensional grids of (chunk, q/k head)
    // workgroups of 256 threads (the chunks rounded up to a multiple of 8), at most
    // 2^32 work-items
    if ((pl.nt_ub + 7) * a->H_q >= (int64_t)1 << 24) return GDR_EINVAL;
    const size_t nb = (size_t)(pl.nt_ub * a->H_v);
    size_t off = 0;
    pl.off_chunk = off;
    off += seq_table_bytes(varlen, pl.n_seq);
    pl.off_tblk = off;
    if (!a->tblk_bwd) off += up(tblock_bytes(a->dtype == GDR_BF16 ? Dt::BF16 : Dt::F32) * nb);  // else the forward's
    pl.off_hs = off;
    if (!a->h_bwd) off += up(sizeof(float) * nb * (size_t)(a->K * a->V));  // else the forward's
    pl.off_dhs = off;
    off += up(sizeof(float) * nb * (size_t)(a->K * a->V));
    pl.total = pl.tokens > 0 ? off : pl.off_tblk;
    // exact sequence split of the state scan and the reverse scan: the device model
    // chooses whether and how long (AUTO), or how long (EXACT)
    const int64_t bh = pl.n_seq * a->H_v;
    // the device model decides for AUTO and AUTO_EXACT (the split is exact here)
    const bool autom = a->cp_mode == GDR_CP_AUTO || a->cp_mode == GDR_CP_AUTO_EXACT;
    bool split = a->cp_mode == GDR_CP_EXACT || autom;
    const int64_t n_vt = a->V / 64;
    int64_t L = a->cp_segment_chunks > 0 ? a->cp_segment_chunks
                                          : split_chunks(pl.nct, bh * n_vt, slots > 0 ? slots : DEFAULT_SLOTS, 8,
                                                         autom ? 1 : 2, true);
    if (L < 1) L = 1;
    if (!split || L >= pl.nct || pl.tokens == 0) {
        split = false;
        L = pl.nct + 1;
    }
    pl.split = split;
    pl.seg_chunks = (int)L;
    if (split && cdiv(pl.nct, L) * bh > ((int64_t)1 << 30)) return GDR_EINVAL;  // as in plan_fwd
    pl.n_seg = split ? (int)cdiv(pl.nct, L) : 1;
    pl.off_M = pl.off_b = pl.off_hseg = pl.off_d = pl.off_gseg = pl.off_zero = 0;
    if (split) {
        const size_t per = (size_t)bh * pl.n_seg * (size_t)a->K * sizeof(float);
        pl.off_M = pl.total;
        pl.off_b = pl.off_M + up(per * (size_t)a->K);
        pl.off_hseg = pl.off_b + up(per * (size_t)a->V);
        pl.off_d = pl.off_hseg + up(per * (size_t)a->V);
        pl.off_gseg = pl.off_d + up(per * (size_t)a->V);
        pl.off_zero = pl.off_gseg + up(per * (size_t)a->V);
        pl.total = pl.off_zero + up(512);
    }
    return GDR_OK;
}

// sequence view of a launch; with packed sequences the kernels read the clamped
// bounds written by launch_chunk_offsets, never the caller's cu_seqlens
SeqMap make_map(bool varlen, int64_t T, int64_t n_seq, int64_t nct, int32_t *chunk_off) {
    SeqMap m;
    m.cu = varlen ? seq_bounds(chunk_off, n_seq) : nullptr;
    m.chunk_off = chunk_off;
    m.order = use_lpt(varlen, n_seq) ? seq_order(chunk_off, n_seq) : nullptr;
    m.T = T;
    m.n_seq = (int32_t)n_seq;
    m.nct = (int32_t)nct;
    return m;
}

}  // namespace

extern "C" {

int gdr_abi_version(void) { return GDR_ABI_VERSION; }

const char *gdr_strerror(int code) {
    switch (code) {
        case GDR_OK: return "ok";
        case GDR_EINVAL: return "invalid argument";
        case GDR_ENOTSUP: return "unsupported size or dtype";
        case GDR_EWORKSPACE: return "workspace too small";
        case GDR_ELAUNCH: return "kernel launch failed";
        case GDR_ESCRATCH: return "problem needs more than the library's static scratch buffer";
        default: return "unknown error";
    }
}

int gdr_fwd_workspace(const gdr_fwd_args *a, size_t *bytes) {
    if (!bytes) return GDR_EINVAL;
    // the split's segment length, and with it the exact split's workspace, follows
    // the compute units of the current device (without one: 256)
    int dev = 0;
    const int64_t slots = hipGetDevice(&dev) == hipSuccess ? device_slots(dev) : 0;
    FwdPlan pl;
    int rc = plan_fwd(a, pl, slots);
    if (rc) return rc;
    *bytes = pl.total;
    return GDR_OK;
}

int gdr_tblocks_bytes(const gdr_fwd_args *a, size_t *bytes) {
    if (!bytes) return GDR_EINVAL;
    FwdPlan pl;
    int rc = plan_fwd(a, pl, DEFAULT_SLOTS);
    if (rc) return rc;
    *bytes = pl.tokens > 0 ? pl.tblk_bwd_bytes : 0;
    return GDR_OK;
}

int gdr_fwd(const gdr_fwd_args *a, hipStream_t stream) { return gdr::fwd_impl(a, stream, nullptr, 0); }

}  // extern "C"

// The forward on the caller's workspace (scratch_for null) or, for the
// allocation-free entry point, on the library's per-device scratch buffer of
// scratch_bytes bytes, whose device address scratch_for(device) returns (null
// when it cannot be had).  Every host-side check runs before the scratch is
// looked up or anything is launched.
int gdr::fwd_impl(const gdr_fwd_args *a, hipStream_t stream, void *(*scratch_for)(int), size_t scratch_bytes) {
    // host-side checks come first; the device query is needed only to launch
    int dev = 0;
    const int64_t slots = hipStreamGetDevice(stream, &dev) == hipSuccess ? device_slots(dev) : 0;
    FwdPlan pl;
    int rc = plan_fwd(a, pl, slots);
    if (rc) return rc;
    if (pl.tokens > 0) {
        if (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->o) return GDR_EINVAL;
        if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->v, 16) || !aligned(a->o, 16) ||
            !aligned(a->g, 4) || !aligned(a->beta, 4))
            return GDR_EINVAL;
    }
    if ((a->A && !aligned(a->A, 16)) || (a->g_cum && !aligned(a->g_cum, 4)) ||
        (a->h && !aligned(a->h, 16)) || (a->final_state && !aligned(a->final_state, 16)) ||
        (a->initial_state && !aligned(a->initial_state, 16)) || (a->w_out && !aligned(a->w_out, 16)) ||
        (a->u_out && !aligned(a->u_out, 16)) || (a->h_bwd && !aligned(a->h_bwd, 16)) ||
        (a->tblk_bwd && !aligned(a->tblk_bwd, 16)))
        return GDR_EINVAL;
    char *ws;
    if (scratch_for) {
        if (pl.total > scratch_bytes) return GDR_ESCRATCH;
        if (slots == 0) return GDR_ELAUNCH;
        ws = static_cast<char *>(scratch_for(dev));
        if (!ws) return GDR_ELAUNCH;
    } else {
        if (a->workspace_bytes < pl.total || (pl.total > 0 && !a->workspace)) return GDR_EWORKSPACE;
        if (pl.total > 0 && !aligned(a->workspace, 16)) return GDR_EINVAL;
        if (slots == 0) return GDR_ELAUNCH;
        ws = static_cast<char *>(a->workspace);
    }
    int32_t *chunk_off = a->cu_seqlens ? reinterpret_cast<int32_t *>(ws + pl.off_chunk) : nullptr;
    // T blocks: the caller's tblk_bwd for bf16 inputs when given (the backward reads the
    // same blocks), else the workspace
    char *tblk = a->tblk_bwd && a->dtype == GDR_BF16 ? static_cast<char *>(a->tblk_bwd) : ws + pl.off_tblk;
    const Dt dt = a->dtype == GDR_BF16 ? Dt::BF16 : Dt::F32;
    const Dt ot = a->out_dtype == GDR_BF16 ? Dt::BF16 : Dt::F32;
    const SeqMap sm = make_map(a->cu_seqlens != nullptr, a->T, pl.n_seq, pl.nct, chunk_off);

    auto ev = [&](int i) { return a->events ? a->events[i] : nullptr; };
    StageGuard stage_guard;
    if (a->cu_seqlens && launch_chunk_offsets(a->cu_seqlens, const_cast<int32_t *>(sm.cu), chunk_off,
                                              const_cast<int32_t *>(sm.order), (int)pl.n_seq, a->T,
                                              stream) != hipSuccess)
        return GDR_ELAUNCH;
    open_stage(ev(0), ev(1));
    if (pl.tokens > 0) {
        PrepParams pp;
        pp.k = a->k;
        pp.g = a->g;
        pp.beta = a->beta;
        pp.g_cum = a->g_cum;
        pp.Tm = a->A;
        pp.tblk = tblk;
        pp.tblk_bwd = dt == Dt::F32 ? static_cast<char *>(a->tblk_bwd) : nullptr;
        pp.sm = sm;
        pp.Hq = (int)a->H_q;
        pp.Hv = (int)a->H_v;
        if (launch_prep(dt, (int)a->K, pp, (int)pl.nt_ub, stream) != hipSuccess) return GDR_ELAUNCH;
    }
    if (close_stage(stream) != hipSuccess) return GDR_ELAUNCH;
    open_stage(ev(2), ev(3));
    ScanParams sp;
    sp.q = a->q;
    sp.k = a->k;
    sp.v = a->v;
    sp.v_tok = a->H_v * a->V;
    sp.v_head = a->V;
    sp.h0_seg = nullptr;
    sp.hT_seg = nullptr;
    sp.eye_h0 = 0;
    sp.tblk = tblk;
    sp.h0 = a->initial_state;
    sp.o = a->o;
    sp.hT = a->final_state;
    // chunk-start states: h, or h_bwd in the backward's layout (bf16: split planes of h^T)
    sp.hsnap = a->h_bwd ? static_cast<float *>(a->h_bwd) : a->h;
    sp.hsnap_split = a->h_bwd && dt == Dt::BF16;
    sp.sm = sm;
    sp.Hq = (int)a->H_q;
    sp.Hv = (int)a->H_v;
    sp.V = (int)a->V;
    sp.scale = a->scale;
    sp.seg_chunks = pl.seg_chunks;
    sp.warm_chunks = pl.warm_chunks;
    sp.warm_gated = pl.gated;
    sp.n_vt = (int)(a->V / scan_vtile(dt, (int)a->K, (int)a->V));
    sp.n_units = (int)(pl.n_seq * a->H_v);
    sp.n_seg = pl.n_seg;
    if (pl.exact && pl.tokens > 0) {
        // segment transitions: the scan from the identity over zero values (V = K) ...
        float *Mb = reinterpret_cast<float *>(ws + pl.off_M), *bb = reinterpret_cast<float *>(ws + pl.off_b);
        float *hseg = reinterpret_cast<float *>(ws + pl.off_hseg);
        if (launch_fill_zero(ws + pl.off_zero, 512, stream) != hipSuccess) return GDR_ELAUNCH;
        ScanParams tp = sp;
        tp.v = ws + pl.off_zero;
        tp.v_tok = tp.v_head = 0;
        tp.V = (int)a->K;
        tp.n_vt = (int)(a->K / scan_vtile(dt, (int)a->K, (int)a->K));
        tp.eye_h0 = 1;
        tp.h0 = nullptr;
        tp.o = nullptr;
        tp.hT = nullptr;
        tp.hsnap = nullptr;
        tp.hT_seg = Mb;
        if (launch_scan_output(dt, ot, (int)a->K, (int)a->K, tp, stream) != hipSuccess) return GDR_ELAUNCH;
        // ... the end states from a zero start (the first segment from the initial state) ...
        ScanParams bp = sp;
        bp.o = nullptr;
        bp.hT = nullptr;
        bp.hsnap = nullptr;
        bp.hT_seg = bb;
        if (launch_scan_output(dt, ot, (int)a->K, (int)a->V, bp, stream) != hipSuccess) return GDR_ELAUNCH;
        // ... the serial carry over the segments, then the segments again from their true starts
        CarryParams cp;
        cp.M = Mb;
        cp.b = bb;
        cp.h0_seg = hseg;
        cp.sm = sm;
        cp.Hv = (int)a->H_v;
        cp.K = (int)a->K;
        cp.V = (int)a->V;
        cp.seg_chunks = pl.seg_chunks;
        cp.n_seg = pl.n_seg;
        cp.rev = 0;
        if (launch_carry(cp, (int)(pl.n_seq * a->H_v), stream) != hipSuccess) return GDR_ELAUNCH;
        sp.h0_seg = hseg;
    }
    if (launch_scan_output(dt, ot, (int)a->K, (int)a->V, sp, stream) != hipSuccess) return GDR_ELAUNCH;
    if (close_stage(stream) != hipSuccess) return GDR_ELAUNCH;
    open_stage(ev(4), ev(5));
    if ((a->w_out || a->u_out) && pl.tokens > 0) {
        if (!a->w_out || !a->u_out) return GDR_EINVAL;
        WUParams wp;
        wp.k = a->k;
        wp.v = a->v;
        wp.tblk = tblk;
        wp.beta = a->beta;
        wp.w = a->w_out;
        wp.u = a->u_out;
        wp.sm = sm;
        wp.Hq = (int)a->H_q;
        wp.Hv = (int)a->H_v;
        wp.K = (int)a->K;
        wp.V = (int)a->V;
        if (launch_wu(dt, wp, (int)pl.nt_ub, stream) != hipSuccess) return GDR_ELAUNCH;
    }
    if (close_stage(stream) != hipSuccess) return GDR_ELAUNCH;
    return GDR_OK;
}

extern "C" {

int gdr_bwd_workspace(const gdr_bwd_args *a, size_t *bytes) {
    if (!bytes) return GDR_EINVAL;
    int dev = 0;
    const int64_t slots = hipGetDevice(&dev) == hipSuccess ? device_slots(dev) : 0;
    BwdPlan pl;
    int rc = plan_bwd(a, pl, slots);
    if (rc) return rc;
    *bytes = pl.total;
    return GDR_OK;
}

int gdr_bwd(const gdr_bwd_args *a, hipStream_t stream) {
    int dev = 0;
    const int64_t slots = hipStreamGetDevice(stream, &dev) == hipSuccess ? device_slots(dev) : 0;
    BwdPlan pl;
    int rc = plan_bwd(a, pl, slots);
    if (rc) return rc;
    if (pl.tokens > 0) {
        // the bf16 kernels read A and g_cum only to rebuild the T blocks
        const bool need_ga = !a->tblk_bwd || a->dtype != GDR_BF16;
        if (!a->q || !a->k || !a->v || (need_ga && (!a->g_cum || !a->A)) || !a->beta || !a->dout || !a->dq ||
            !a->dk || !a->dv || !a->dbeta || !a->dg)
            return GDR_EINVAL;
        if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->v, 16) || !aligned(a->dout, 16) ||
            !aligned(a->A, 16) || !aligned(a->dq, 16) || !aligned(a->dk, 16) || !aligned(a->dv, 16) ||
            !aligned(a->g_cum, 4) || !aligned(a->beta, 4) || !aligned(a->dbeta, 4) || !aligned(a->dg, 4) ||
            !aligned(a->tblk_bwd, 16))
            return GDR_EINVAL;
    }
    if ((a->dht && !aligned(a->dht, 16)) || (a->initial_state && !aligned(a->initial_state, 16)) ||
        (a->dh0 && !aligned(a->dh0, 16)) || (a->h_bwd && !aligned(a->h_bwd, 16)))
        return GDR_EINVAL;
    if (a->workspace_bytes < pl.total || (pl.total > 0 && !a->workspace)) return GDR_EWORKSPACE;
    if (pl.total > 0 && !aligned(a->workspace, 16)) return GDR_EINVAL;
    if (slots == 0) return GDR_ELAUNCH;

    char *ws = static_cast<char *>(a->workspace);
    int32_t *chunk_off = a->cu_seqlens ? reinterpret_cast<int32_t *>(ws + pl.off_chunk) : nullptr;
    const Dt dt = a->dtype == GDR_BF16 ? Dt::BF16 : Dt::F32;
    const SeqMap sm = make_map(a->cu_seqlens != nullptr, a->T, pl.n_seq, pl.nct, chunk_off);
    const int n_units = (int)(pl.n_seq * a->H_v);

    BwdParams bp;
    bp.q = a->q;
    bp.k = a->k;
    bp.v = a->v;
    bp.dout = a->dout;
    bp.g_cum = a->g_cum;
    bp.beta = a->beta;
    bp.A = a->A;
    bp.dht = a->dht;
    bp.tblk = a->tblk_bwd ? static_cast<char *>(const_cast<void *>(a->tblk_bwd)) : ws + pl.off_tblk;
    bp.hs = a->h_bwd ? static_cast<const float *>(a->h_bwd) : reinterpret_cast<float *>(ws + pl.off_hs);
    bp.dhs = reinterpret_cast<float *>(ws + pl.off_dhs);
    bp.dq = a->dq;
    bp.dk = a->dk;
    bp.dv = a->dv;
    bp.dbeta = a->dbeta;
    bp.dg = a->dg;
    bp.dh0 = a->dh0;
    bp.sm = sm;
    bp.Hq = (int)a->H_q;
    bp.Hv = (int)a->H_v;
    bp.V = (int)a->V;
    bp.scale = a->scale;
    bp.seg_chunks = pl.seg_chunks;
    bp.n_seg = pl.n_seg;
    bp.dh_seg = nullptr;
    bp.d_seg = nullptr;

    auto ev = [&](int i) { return a->events ? a->events[i] : nullptr; };
    StageGuard stage_guard;
    if (a->cu_seqlens && launch_chunk_offsets(a->cu_seqlens, const_cast<int32_t *>(sm.cu), chunk_off,
                                              const_cast<int32_t *>(sm.order), (int)pl.n_seq, a->T,
                                              stream) != hipSuccess)
        return GDR_ELAUNCH;
    open_stage(ev(0), ev(1));
    if (pl.tokens > 0 && !a->tblk_bwd && launch_tblocks(dt, bp, (int)pl.nt_ub, stream) != hipSuccess)
        return GDR_ELAUNCH;
    if (close_stage(stream) != hipSuccess) return GDR_ELAUNCH;
    open_stage(ev(2), ev(3));
    if (pl.tokens > 0 && !a->h_bwd) {
        // chunk-start states: the exact forward scan without its output
        ScanParams sp;
        sp.q = a->q;
        sp.k = a->k;
        sp.v = a->v;
        sp.v_tok = a->H_v * a->V;
        sp.v_head = a->V;
        sp.h0_seg = nullptr;
        sp.hT_seg = nullptr;
        sp.eye_h0 = 0;
        sp.tblk = bp.tblk;
        sp.h0 = a->initial_state;
        sp.o = nullptr;
        sp.hT = nullptr;
        sp.hsnap = reinterpret_cast<float *>(ws + pl.off_hs);
        sp.hsnap_split = dt == Dt::BF16;  // the bf16 backward kernels copy split planes straight to LDS
        sp.sm = sm;
        sp.Hq = (int)a->H_q;
        sp.Hv = (int)a->H_v;
        sp.V = (int)a->V;
        sp.scale = a->scale;
        sp.seg_chunks = pl.seg_chunks;
        sp.warm_chunks = 0;
        sp.warm_gated = 0;
        sp.n_vt = (int)(a->V / scan_vtile(dt, (int)a->K, (int)a->V));
        sp.n_units = n_units;
        sp.n_seg = pl.n_seg;
        if (pl.split) {
            // the forward's exact split on the rebuilt T blocks: segment transitions from
            // the identity over a zero row, zero-start end states, the carry; the states
            // pass below then starts every segment from its true state
            if (launch_fill_zero(ws + pl.off_zero, 512, stream) != hipSuccess) return GDR_ELAUNCH;
            ScanParams tp = sp;
            tp.v = ws + pl.off_zero;
            tp.v_tok = tp.v_head = 0;
            tp.V = (int)a->K;
            tp.n_vt = (int)(a->K / scan_vtile(dt, (int)a->K, (int)a->K));
            tp.eye_h0 = 1;
            tp.h0 = nullptr;
            tp.hsnap = nullptr;
            tp.hT_seg = reinterpret_cast<float *>(ws + pl.off_M);
            if (launch_scan_states(dt, (int)a->K, tp, stream) != hipSuccess) return GDR_ELAUNCH;
            ScanParams zp = sp;
            zp.hsnap = nullptr;
            zp.hT_seg = reinterpret_cast<float *>(ws + pl.off_b);
            if (launch_scan_states(dt, (int)a->K, zp, stream) != hipSuccess) return GDR_ELAUNCH;
            CarryParams cp;
            cp.M = reinterpret_cast<float *>(ws + pl.off_M);
            cp.b = reinterpret_cast<float *>(ws + pl.off_b);
            cp.h0_seg = reinterpret_cast<float *>(ws + pl.off_hseg);
            cp.sm = sm;
            cp.Hv = (int)a->H_v;
            cp.K = (int)a->K;
            cp.V = (int)a->V;
            cp.seg_chunks = pl.seg_chunks;
            cp.n_seg = pl.n_seg;
            cp.rev = 0;
            if (launch_carry(cp, n_units, stream) != hipSuccess) return GDR_ELAUNCH;
            sp.h0_seg = cp.h0_seg;
        }
        if (launch_scan_states(dt, (int)a->K, sp, stream) != hipSuccess) return GDR_ELAUNCH;
    } else if (pl.tokens > 0 && pl.split) {
        // states from the forward: the reverse carry still needs the segment transitions
        ScanParams tp;
        tp.q = a->q;
        tp.k = a->k;
        tp.v = ws + pl.off_zero;
        tp.v_tok = tp.v_head = 0;
        tp.h0_seg = nullptr;
        tp.hT_seg = reinterpret_cast<float *>(ws + pl.off_M);
        tp.eye_h0 = 1;
        tp.tblk = bp.tblk;
        tp.h0 = nullptr;
        tp.o = nullptr;
        tp.hT = nullptr;
        tp.hsnap = nullptr;
        tp.hsnap_split = 0;
        tp.sm = sm;
        tp.Hq = (int)a->H_q;
        tp.Hv = (int)a->H_v;
        tp.V = (int)a->K;
        tp.scale = a->scale;
        tp.seg_chunks = pl.seg_chunks;
        tp.warm_chunks = 0;
        tp.warm_gated = 0;
        tp.n_vt = (int)(a->K / scan_vtile(dt, (int)a->K, (int)a->K));
        tp.n_units = n_units;
        tp.n_seg = pl.n_seg;
        if (launch_fill_zero(ws + pl.off_zero, 512, stream) != hipSuccess) return GDR_ELAUNCH;
        if (launch_scan_states(dt, (int)a->K, tp, stream) != hipSuccess) return GDR_ELAUNCH;
    }
    if (close_stage(stream) != hipSuccess) return GDR_ELAUNCH;
    open_stage(ev(4), ev(5));  // closed by launch_bwd after the reverse scan
    if (pl.split) {
        // reverse scan: every segment's start gradient from a zero end gradient (the last
        // segment from dht), the reverse carry with the transposed transitions, then the
        // scan below from every segment's true end gradient
        BwdParams dp = bp;
        dp.d_seg = reinterpret_cast<float *>(ws + pl.off_d);
        if (launch_bwd_reverse(dt, (int)a->K, dp, n_units, stream) != hipSuccess) return GDR_ELAUNCH;
        CarryParams cp;
        cp.M = reinterpret_cast<float *>(ws + pl.off_M);
        cp.b = dp.d_seg;
        cp.h0_seg = reinterpret_cast<float *>(ws + pl.off_gseg);
        cp.sm = sm;
        cp.Hv = (int)a->H_v;
        cp.K = (int)a->K;
        cp.V = (int)a->V;
        cp.seg_chunks = pl.seg_chunks;
        cp.n_seg = pl.n_seg;
        cp.rev = 1;
        if (launch_carry(cp, n_units, stream) != hipSuccess) return GDR_ELAUNCH;
        bp.dh_seg = cp.h0_seg;
    }
    const Dt gt = a->grad_dtype == GDR_BF16 ? Dt::BF16 : Dt::F32;
    const hipEvent_t *lev = a->events ? a->events + 6 : nullptr;  // the chunk-local stage
    if (launch_bwd(dt, gt, (int)a->K, bp, pl.tokens > 0 ? (int)pl.nt_ub : 0, n_units, lev, stream) != hipSuccess)
        return GDR_ELAUNCH;
    return GDR_OK;
}

}  // extern "C"
