// Kernel parameter blocks and host-side launchers of libgdr (internal).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdr.h"
#include "gdr_device.hpp"
#include "gdr_layout.hpp"

namespace gdr {

enum class Dt : int { BF16 = 0, F32 = 1 };

// Stage timing for the callers' event hooks.  The events of a stage are bound
// to its kernel launches (hipExtLaunchKernel), so they carry the kernels' own
// start and end times, with no marker packets on the stream between kernels:
// the stage's first launch takes the start event, and every launch takes the
// stop event, so the last launch's end stands.  A stage that launches nothing
// records both events at once when it closes.  One open stage per host thread.
struct StageEvents {
    hipEvent_t start, stop;
    bool launched;
};
StageEvents &stage_events();  // this thread's (gdr_api.hip)
inline void open_stage(hipEvent_t start, hipEvent_t stop) { stage_events() = {start, stop, false}; }
inline hipError_t close_stage(hipStream_t s) {
    StageEvents &e = stage_events();
    hipError_t r = hipSuccess;
    if (!e.launched) {
        if (e.start) r = hipEventRecord(e.start, s);
        if (r == hipSuccess && e.stop) r = hipEventRecord(e.stop, s);
    }
    e = {nullptr, nullptr, false};
    return r;
}
// every kernel of the library is launched through this (errors: hipGetLastError)
template <typename F, typename... Args>
inline void launch_k(F kernel, dim3 grid, dim3 block, uint32_t smem, hipStream_t s, Args... args) {
    StageEvents &e = stage_events();
    hipExtLaunchKernelGGL(kernel, grid, block, smem, s, e.launched ? nullptr : e.start, e.stop, 0, args...);
    e.launched = true;
}

// gdr_chunk_prep: per (chunk, q/k head): in-chunk cumulative log-gate,
// decayed strictly lower beta K K^T, T = (I + A)^{-1}.
struct PrepParams {
    const void *k;
    const float *g, *beta;
    float *g_cum;  // [tokens, H_v] or null
    float *Tm;     // [tokens, H_v, 64] or null
    char *tblk;    // [chunks, H_v] T blocks (gdr_layout.hpp), the compact form the scan reads
    char *tblk_bwd;  // fp32 inputs: null, or the same blocks with full rows for the backward
    SeqMap sm;
    int Hq, Hv;
};

// gdr_scan_output: per (sequence, v-head, V tile, segment): serial scan over
// chunks with the output of each chunk.
struct ScanParams {
    const void *q, *k, *v;
    int64_t v_tok, v_head;  // element strides of v between tokens and between v heads
                            // (both 0: every row is the same, a zero row for transitions)
    const char *tblk;  // [chunks, H_v] T blocks from gdr_chunk_prep
    const float *h0;  // [N, H_v, K, V] or null
    void *o;          // [tokens, H_v, V]
    float *hT;        // [N, H_v, K, V] or null
    float *hsnap;     // [NT, H_v, K, V] or null
    int hsnap_split;  // bf16 inputs only: hsnap holds, per (chunk, v head), bf16 hi then lo
                      // planes of the transposed state [V][K] (4 bytes per element)
    SeqMap sm;
    int Hq, Hv, V;
    float scale;
    int seg_chunks;   // chunks per segment
    int warm_chunks;  // warm-up window of segments after the first
    // gate-driven warm-up (instead of warm_chunks): a segment after the first starts
    // from a zero state at the latest chunk from which the gates decay the state by
    // at least 2^-24 up to the segment's start, or from the sequence start
    int warm_gated;
    int n_vt, n_units, n_seg;
    // exact sequence split: segments after the first start from h0_seg (or, eye_h0,
    // from the identity, V = K, which makes the segment's end state its transition
    // matrix); hT_seg receives every segment's end state.  [n_units][n_seg][K][V]
    const float *h0_seg;
    float *hT_seg;
    int eye_h0;
};

// carry of the exact sequence split: for segments s = 1 .. of each unit,
// start(s) = M(s-1) start(s-1) + b(s-1), start(1) = b(0), written to h0_seg
// With rev (the backward's reverse scan): for s = n-2 down to 0,
// end(s) = M(s+1)^T end(s+1) + b(s+1), end(n-2) = b(n-1), written to h0_seg[s]
// (b: each segment's start gradient from a zero end gradient, the last from dht).
struct CarryParams {
    const float *M;    // [n_units][n_seg][K][K] segment transitions
    const float *b;    // [n_units][n_seg][K][V] segment end states from a zero start (s = 0: from h0)
    float *h0_seg;     // [n_units][n_seg][K][V]
    SeqMap sm;
    int Hv, K, V, seg_chunks, n_seg;
    int rev;
};

// optional materialisation of W = T diag(beta e^gam) K and U = T diag(beta) V
struct WUParams {
    const void *k, *v;
    const char *tblk;
    const float *beta;
    float *w, *u;
    SeqMap sm;
    int Hq, Hv, K, V;
};

// backward: per (chunk, q/k head) local gradients after a reverse scan over
// chunks per (sequence, v head, 64 value columns)
struct BwdParams {
    const void *q, *k, *v, *dout;
    const float *g_cum, *beta, *A;
    const float *dht;  // [N, H_v, K, V] or null
    char *tblk;        // [chunks, H_v] T blocks rebuilt from A
    const float *hs;   // [NT, H_v, K, V] chunk-start states (bf16 inputs: split planes, as hsnap_split)
    float *dhs;        // [NT, H_v, K, V] gradient of each chunk's end state (same layout as hs)
    void *dq, *dk, *dv;
    float *dbeta, *dg;
    float *dh0;        // [N, H_v, K, V] or null
    SeqMap sm;
    int Hq, Hv, V;
    float scale;
    // exact sequence split of the reverse scan: segments of seg_chunks chunks (n_seg = 1:
    // none).  A segment other than the last starts from dh_seg (its end gradient) or,
    // with d_seg set, from zero, and then writes its start gradient to d_seg and no
    // chunk-end gradients.  [n_units][n_seg][K][V]
    int seg_chunks, n_seg;
    const float *dh_seg;
    float *d_seg;
};

// clamped bounds (cuc) and chunk offsets of packed sequences and (order non-null)
// their longest-first order; every kernel reads the bounds from cuc
hipError_t launch_chunk_offsets(const int32_t *cu, int32_t *cuc, int32_t *chunk_off, int32_t *order, int n_seq,
                               int64_t T, hipStream_t s);
hipError_t launch_prep(Dt dt, int K, const PrepParams &p, int n_chunks_ub, hipStream_t s);
hipError_t launch_scan_output(Dt dt, Dt out, int K, int V, const ScanParams &p, hipStream_t s);
hipError_t launch_wu(Dt dt, const WUParams &p, int n_chunks_ub, hipStream_t s);
hipError_t launch_scan_states(Dt dt, int K, const ScanParams &p, hipStream_t s);
hipError_t launch_carry(const CarryParams &p, int n_units, hipStream_t s);
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s);
hipError_t launch_tblocks(Dt dt, const BwdParams &p, int n_chunks_ub, hipStream_t s);
// the reverse scan alone (the exact split's pass from zero end gradients)
hipError_t launch_bwd_reverse(Dt dt, int K, const BwdParams &p, int n_units, hipStream_t s);
// Closes the timing stage open on this thread (the reverse scan, opened by the
// caller) after the reverse scan; ev: null or 2 events, the start and stop of
// the chunk-local stage.
hipError_t launch_bwd(Dt dt, Dt gt, int K, const BwdParams &p, int n_chunks_ub, int n_units,
                      const hipEvent_t *ev, hipStream_t s);
hipError_t launch_bwd_scan_bf16(int K, const BwdParams &p, int n_units, hipStream_t s);
hipError_t launch_bwd_local_bf16(Dt gt, int K, const BwdParams &p, int n_chunks_ub, hipStream_t s);
size_t tblock_bytes(Dt dt);      // the backward's T blocks (bf16: the forward's compact ones)
size_t tblock_bytes_fwd(Dt dt);  // the forward's T blocks, read by the scan
// Body of gdr_fwd (gdr_api.hip): on the caller's workspace (scratch_for null), or
// on a library-owned buffer of scratch_bytes bytes whose device address
// scratch_for(device) returns (null: not available), as gdr_fwd_noalloc does.
int fwd_impl(const gdr_fwd_args *a, hipStream_t stream, void *(*scratch_for)(int), size_t scratch_bytes);
int scan_vtile(Dt dt, int K, int V);  // V columns per scan workgroup

}  // namespace gdr
