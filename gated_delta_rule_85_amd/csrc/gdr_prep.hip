// gdr_chunk_prep — the chunk-parallel part of the chunked forward.
//
// For one chunk of one q/k head (and each of the v heads sharing it, two at a
// time):
//   gam = in-chunk running sum of the log-gate g          (returned as g_cum)
//   A   = strictly lower part of diag(beta) (K K^T) * exp(gam_r - gam_i)
//   T   = (I + A)^{-1}                                     (returned as A)
// These are the first steps the efeozkan blog lists under "2. Hardware-
// Friendly Algebraic Reformulation" (computing the A matrix, then W and U);
// W = T diag(beta e^gam) K and U = T diag(beta) V are not stored: the scan
// kernel applies T to V - diag(e^gam) K h directly (U - W h in one product).
// For the scan it writes one T block per (chunk, v head), the LDS image the
// scan copies in (gdr_layout.hpp): T split into bf16 hi/lo planes (fp32 for
// fp32 inputs) with swizzled rows, and the chunk's gate scalars.
//
// K K^T depends only on the q/k head, so it is formed once per workgroup on
// MFMA and reused by the H_v/H_q v heads.  The inverse of the unit lower
// triangular 64x64 matrix is blocked in 16x16 tiles: the four diagonal tiles
// by forward substitution (one wave per head, one lane per column), the
// off-diagonal tiles by T_ab = -D_a sum_{m=b}^{a-1} A_am T_mb on fp32 MFMA, block
// column by block column.  The v heads are taken two at a time so that the
// one-wave phases (the gates' prefix sum, the substitution) run for both heads
// at once.
#include "gdr_kernels.hpp"
#include "gdr_lds.hpp"

namespace gdr {

namespace {

constexpr int LDF = 68;  // fp32 64x64 tiles in LDS: row pitch (floats)
static_assert(LDF % 4 == 0, "rows of the tiles are read as 16-byte vectors");

// Each v head's 64 x 64 matrices share one LDS tile M: T (lower triangular) in
// its lower part with the diagonal, A (strictly lower) transposed in its
// strict upper part, M[i][r] = A[r][i] for i < r.  The diagonal blocks of A
// are read only by the substitution, which then overwrites the upper part of
// each diagonal block with the zeros of T; T's blocks above the diagonal are
// never stored (they are zero) and readers mask them.

// acc += A_am T_mb (block rows of A from the transposed store, T block rows)
__device__ __forceinline__ f32x4 blk_mm_at(f32x4 acc, const float *M, int a, int m, int b) {
    const int n = ln16(), g = lg4();
#pragma unroll
    for (int j = 0; j < 4; ++j)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(M[(16 * m + 4 * g + j) * LDF + 16 * a + n],
                                                   M[(16 * m + 4 * g + j) * LDF + 16 * b + n], acc, 0, 0, 0);
    return acc;
}
// acc += T_aa * Y where Y is an accumulator tile in registers
__device__ __forceinline__ f32x4 blk_mm_reg(f32x4 acc, const float *X, f32x4 y) {
    const int n = ln16(), g = lg4();
    const f32x4 a = *reinterpret_cast<const f32x4 *>(X + n * LDF + 4 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], y[j], acc, 0, 0, 0);
    return acc;
}

// T_ab (a > b) = -T_aa sum_{m=b}^{a-1} A_am T_mb, from the diagonal inverses and
// the lower blocks already done
__device__ __forceinline__ void offdiag_tile(float *M, int a, int b) {
    f32x4 P = zero4();
    for (int m = b; m < a; ++m) P = blk_mm_at(P, M, a, m, b);
    const f32x4 R = blk_mm_reg(zero4(), M + 16 * a * LDF + 16 * a, P);
    const int n = ln16(), g = lg4();
#pragma unroll
    for (int j = 0; j < 4; ++j) M[(16 * a + 4 * g + j) * LDF + 16 * b + n] = -R[j];
}

// The v heads of the q/k head are taken two at a time, in step: every phase
// below serves both heads of a pair, so a pair costs the phases of one head.
template <typename In, int KD>
__global__ __launch_bounds__(NTHR) void prep_kernel(const PrepParams p) {
    using O = Ops<In>;
    using V16 = typename Vec16<In>::type;
    constexpr int EV = Vec16<In>::n;
    constexpr int LDK = KD + EV;  // 16-byte row padding
    // K (until S = K K^T is in registers), then the first head's tile, share the first region
    constexpr int KBYTES = sizeof(In) * CH * LDK, MBYTES = sizeof(float) * CH * LDF;
    constexpr int R0 = KBYTES > MBYTES ? KBYTES : MBYTES;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    In *Ks = reinterpret_cast<In *>(smem);
    float *const M0 = reinterpret_cast<float *>(smem), *const M1 = reinterpret_cast<float *>(smem + R0);
    auto tile = [&](int h) { return h ? M1 : M0; };  // head h of the pair
    float *gb = reinterpret_cast<float *>(smem + R0 + MBYTES);  // gam, bet of the two heads
    auto gam_of = [&](int h) { return gb + 2 * CH * h; };
    auto bet_of = [&](int h) { return gb + 2 * CH * h + CH; };

    // Workgroup b runs on XCD b % 8.  The chunks are dealt to the XCDs in turn, so that
    // the log-gate and beta rows of a chunk, which all its q/k heads read, are fetched
    // into one L2; within an XCD the q/k head runs fastest, so that neighbours read
    // adjacent 256-byte pieces of the same key rows and write adjacent T blocks.
    // Chunks past the last (the grid rounds them up to a multiple of 8) have no work.
    const int slot = blockIdx.x >> 3;
    const int hq = slot % p.Hq, gid = (slot / p.Hq) * 8 + (blockIdx.x & 7);
    int j, c;
    if (!p.sm.locate(gid, j, c)) return;
    int64_t bos, eos;
    p.sm.bounds(j, bos, eos);
    const int64_t ts = bos + (int64_t)c * CH;
    const int n = (int)min<int64_t>(CH, eos - ts);
    const int tid = threadIdx.x, w = wave_id(), l = lane_id();
    const int G = p.Hv / p.Hq;

    // waves 0 and 1 hold the log-gate and beta of the pair's two v heads, one token
    // per lane; each pair's are loaded one pair ahead, the first before the K tile,
    // so their latency overlaps other work
    float g_nx = 0.f, b_nx = 0.f;
    if (w < 2 && w < G && l < n) {
        g_nx = p.g[(ts + l) * p.Hv + hq * G + w];
        b_nx = p.beta[(ts + l) * p.Hv + hq * G + w];
    }

    // K rows of the chunk (zero past its end)
    const In *kp = reinterpret_cast<const In *>(p.k);
    {
        // all of this thread's loads first, then the LDS writes (one memory round trip)
        constexpr int PER = CH * (KD / EV) / NTHR;
        static_assert(CH * (KD / EV) % NTHR == 0, "K tile pieces spread evenly");
        V16 val[PER];
#pragma unroll
        for (int it = 0; it < PER; ++it) {
            const int idx = tid + it * NTHR, r = idx / (KD / EV), cv = idx % (KD / EV);
            // rows past the chunk end read its last row (no branch around the
            // load, which would make the compiler wait on it) and are zeroed
            const int rr = min(r, n - 1);
            val[it] = *reinterpret_cast<const V16 *>(kp + ((ts + rr) * p.Hq + hq) * KD + cv * EV);
        }
#pragma unroll
        for (int it = 0; it < PER; ++it)
            if ((tid + it * NTHR) / (KD / EV) >= n) val[it] = V16{};
#pragma unroll
        for (int it = 0; it < PER; ++it) {
            const int idx = tid + it * NTHR, r = idx / (KD / EV), cv = idx % (KD / EV);
            *reinterpret_cast<V16 *>(Ks + r * LDK + cv * EV) = val[it];
        }
    }
    __syncthreads();

    // S = K K^T, the ten tiles (str, sti) on or below the diagonal, kept in
    // registers as their transposes (S is symmetric: the product with the operands
    // swapped), so that lane (n16, g) holds S[16 str + n16][16 sti + 4 g + jj]:
    // one row r per lane, the layout in which A^T is stored without bank
    // conflicts.  Wave w holds tiles w, w + 4 and (waves 0, 1) w + 8
    const int n16 = ln16(), g = lg4();
    f32x4 sS[3];
    int str[3], sti[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int t = w + 4 * k;
        str[k] = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
        sti[k] = t - str[k] * (str[k] + 1) / 2;
        sS[k] = zero4();
        if (t < 10) {
            // operand slot j of lane group g is k = 8 g + j in each 32-deep block (both
            // operands alike): 8 consecutive elements of a row per lane
#pragma unroll
            for (int dp = 0; dp < KD / 32; ++dp) {
                const In *ar = Ks + (16 * sti[k] + n16) * LDK + 32 * dp + 8 * g;
                const In *br = Ks + (16 * str[k] + n16) * LDK + 32 * dp + 8 * g;
                sS[k] = mma(sS[k], O::load(ar, ar + 4), O::load(br, br + 4));
            }
        }
    }
    __syncthreads();  // K is no longer read: its region becomes the first head's tile

    for (int r0 = 0; r0 < G; r0 += 2) {
        const int np = min(2, G - r0);  // heads in this pair
        if (w < np) {
            // inclusive running sum of g over the chunk (zero past its end)
            const int hv = hq * G + r0 + w;
            const float x = wave_prefix_sum(g_nx);
            gam_of(w)[l] = x;
            bet_of(w)[l] = b_nx;
            if (l < n && p.g_cum) p.g_cum[(ts + l) * p.Hv + hv] = x;
            if (r0 + 2 + w < G && l < n) {
                g_nx = p.g[(ts + l) * p.Hv + hv + 2];
                b_nx = p.beta[(ts + l) * p.Hv + hv + 2];
            }
        }
        __syncthreads();
        // A = diag(beta) S * exp(gam_r - gam_i) below the diagonal, from the S tiles in
        // registers, stored transposed: M[i][r] = A[r][i], i < r
#pragma unroll 1
        for (int h = 0; h < np; ++h) {
            float *M = tile(h);
            const float *gam = gam_of(h), *bet = bet_of(h);
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                if (w + 4 * k >= 10) break;
                const int r = 16 * str[k] + n16, i0 = 16 * sti[k] + 4 * g;
                const float br = bet[r], gr = gam[r];
                const f32x4 gi = *reinterpret_cast<const f32x4 *>(gam + i0);
                // no branch: in a diagonal tile the entries i >= r land in the lower
                // part of the block, which the substitution overwrites with T
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) M[(i0 + jj) * LDF + r] = br * fast_exp(gr - gi[jj]) * sS[k][jj];
            }
        }
        __syncthreads();
        if (w < np) {
            // diagonal tiles of head w: lane = (tile b, column cc); forward substitution,
            // then column cc of T_bb over the (no longer needed) block of A
            // (right-looking: once x_i is final, row i of the transposed store, A's
            // column i, is read as 16-byte vectors and taken off the rows below)
            float *M = tile(w);
            const int b = l >> 4, cc = l & 15;
            float *Mb = M + 16 * b * LDF + 16 * b;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = (r == cc) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < 15; ++i) {
#pragma unroll
                for (int q = (i + 1) / 4; q < 4; ++q) {
                    const f32x4 a = *reinterpret_cast<const f32x4 *>(Mb + i * LDF + 4 * q);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * q + e > i) x[4 * q + e] -= a[e] * x[i];
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) Mb[r * LDF + cc] = x[r];
        }
        __syncthreads();
        // off-diagonal blocks by block column, with no barrier inside a column: T_ab
        // needs the diagonal inverses and the blocks T_mb above it in its own column
        // only.  Wave w takes head w & 1: column 0 (waves 0, 1) or columns 1 and 2
        // (waves 2, 3); each wave reads back the blocks it wrote (LDS keeps a wave's
        // accesses in order)
        if ((w & 1) < np) {
            float *M = tile(w & 1);
            if (w < 2) {
                offdiag_tile(M, 1, 0);
                offdiag_tile(M, 2, 0);
                offdiag_tile(M, 3, 0);
            } else {
                offdiag_tile(M, 2, 1);
                offdiag_tile(M, 3, 1);
                offdiag_tile(M, 3, 2);
            }
        }
        __syncthreads();
        if constexpr (sizeof(In) == 2) {
            // the T blocks of the pair's heads as one list of pieces (an even share per
            // thread), then the scalars, 64 threads per head
            char *blk0 = p.tblk + ((int64_t)gid * p.Hv + hq * G + r0) * TBlockF<In>::BYTES;
            for (int idx = tid; idx < np * TBF_PIECES; idx += NTHR) {
                const int h = idx >= TBF_PIECES;
                write_tblock_f_piece<true>(blk0 + h * TBlockF<In>::BYTES, tile(h), LDF, n, idx - h * TBF_PIECES);
            }
            if (tid < np * CH) {
                const int h = tid >> 6;
                write_tblock_scalars<TBlockF<In>>(blk0 + h * TBlockF<In>::BYTES, gam_of(h), bet_of(h), n, tid & 63);
            }
        }
#pragma unroll 1
        for (int h = 0; h < np; ++h) {
            const int hv = hq * G + r0 + h;
            const float *T = tile(h);
            if (p.Tm) {
                for (int idx = tid; idx < CH * 16; idx += NTHR) {
                    const int r = idx >> 4, c4 = idx & 15;
                    if (r < n)
                        *reinterpret_cast<f32x4 *>(p.Tm + ((ts + r) * p.Hv + hv) * CH + 4 * c4) =
                            (c4 >> 2) > (r >> 4) ? zero4() : *reinterpret_cast<const f32x4 *>(T + r * LDF + 4 * c4);
                }
            }
            if constexpr (sizeof(In) == 4) {
                // T block for the scan: fp32 rows, swizzled (rows past the chunk end zero)
                // + scalars, and for the backward of fp32 inputs the same in the layout its
                // kernels copy (plain 16-byte-chunk order); the bf16 backward reads the
                // blocks written above
                write_tblock_f<In>(p.tblk + ((int64_t)gid * p.Hv + hv) * TBlockF<In>::BYTES, T, LDF, gam_of(h),
                                   bet_of(h), n, tid, NTHR);
                if (p.tblk_bwd)
                    write_tblock<In>(p.tblk_bwd + ((int64_t)gid * p.Hv + hv) * TBlock<In>::BYTES, T, LDF,
                                     gam_of(h), bet_of(h), n, tid, NTHR);
            }
        }
        lds_barrier();  // the tiles and gates free again; the blocks' stores drain meanwhile
    }
}

template <typename In, int KD>
size_t prep_smem() {
    const size_t kb = sizeof(In) * CH * (KD + Vec16<In>::n), mb = sizeof(float) * CH * LDF;
    return (kb > mb ? kb : mb) + mb + sizeof(float) * 4 * CH;
}

template <typename In, int KD>
hipError_t launch_prep_t(const PrepParams &p, int n_chunks_ub, hipStream_t s) {
    const size_t smem = prep_smem<In, KD>();
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&prep_kernel<In, KD>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    (void)attr;  // a refusal shows up as a launch error below
    dim3 grid((n_chunks_ub + 7) / 8 * 8 * p.Hq);  // (chunk, q/k head)
    launch_k((prep_kernel<In, KD>), grid, dim3(NTHR), smem, s, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------- W, U
// Materialises W = T diag(beta e^gam) K and U = T diag(beta) V in fp32 (a
// check of the algebra; not used by the forward itself).
// entry (r, i), i <= r, of the T of a forward T block
template <typename In>
__device__ __forceinline__ float tblock_T(const char *blk, int r, int i) {
    using TB = TBlockF<In>;
    const int byte = i * (TB::BF ? 2 : 4);
    if constexpr (TB::BF)
        return to_f32(*reinterpret_cast<const bf16 *>(blk + TB::off(r, byte))) +
               to_f32(*reinterpret_cast<const bf16 *>(blk + TB::PLANE + TB::off(r, byte)));
    else
        return *reinterpret_cast<const float *>(blk + TB::off(r, byte));
}

template <typename In>
__global__ __launch_bounds__(NTHR) void wu_kernel(const WUParams p) {
    const int gid = blockIdx.x, hv = blockIdx.y;
    int j, c;
    if (!p.sm.locate(gid, j, c)) return;
    int64_t bos, eos;
    p.sm.bounds(j, bos, eos);
    const int64_t ts = bos + (int64_t)c * CH;
    const int n = (int)min<int64_t>(CH, eos - ts);
    const int hq = hv / (p.Hv / p.Hq);
    const In *kp = reinterpret_cast<const In *>(p.k);
    const In *vp = reinterpret_cast<const In *>(p.v);
    const char *blk = p.tblk + ((int64_t)gid * p.Hv + hv) * TBlockF<In>::BYTES;
    const float *sc = reinterpret_cast<const float *>(blk + TBlockF<In>::SC);
    for (int idx = threadIdx.x; idx < n * (p.K + p.V); idx += NTHR) {
        const int r = idx / (p.K + p.V), col = idx % (p.K + p.V);
        const bool isw = col < p.K;
        float acc = 0.f;
        for (int i = 0; i <= r; ++i) {
            const float t = tblock_T<In>(blk, r, i);
            const float b = sc[3 * CH + i];
            if (isw)
                acc += t * b * sc[CH + i] * to_f32(kp[((ts + i) * p.Hq + hq) * p.K + col]);
            else
                acc += t * b * to_f32(vp[((ts + i) * p.Hv + hv) * p.V + col - p.K]);
        }
        if (isw)
            p.w[((ts + r) * p.Hv + hv) * p.K + col] = acc;
        else
            p.u[((ts + r) * p.Hv + hv) * p.V + col - p.K] = acc;
    }
}

// Sequence bounds of packed sequences, clamped so that no kernel can index
// past the packed tokens whatever the caller's offsets hold: cuc[0] =
// clamp(cu[0], 0, T), cuc[j] = clamp(cu[j], cuc[j-1], T) (non-decreasing, at
// most T), and chunk_off[j] = sum_{i<j} ceil((cuc[i+1] - cuc[i]) / 64).  For
// valid offsets (cu[0] = 0, non-decreasing, cu[n] = T) cuc equals cu.
__global__ void chunk_offsets_kernel(const int32_t *cu, int32_t *cuc, int32_t *off, int n_seq, int32_t T) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        int32_t acc = 0;
        int32_t prev = min(max(cu[0], 0), T);
        cuc[0] = prev;
        for (int j = 0; j < n_seq; ++j) {
            const int32_t nx = min(max(cu[j + 1], prev), T);
            cuc[j + 1] = nx;
            off[j] = acc;
            acc += (nx - prev + CH - 1) / CH;
            prev = nx;
        }
        off[n_seq] = acc;
    }
}

// order[rank] = j: sequences by decreasing length, ties by index (one thread per
// sequence counts the sequences ahead of it); cu is the clamped table
__global__ void seq_order_kernel(const int32_t *cu, int32_t *order, int n_seq) {
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= n_seq) return;
    const int lj = cu[j + 1] - cu[j];
    int rank = 0;
    for (int i = 0; i < n_seq; ++i) {
        const int li = cu[i + 1] - cu[i];
        rank += (li > lj) || (li == lj && i < j);
    }
    order[rank] = j;
}

}  // namespace

hipError_t launch_chunk_offsets(const int32_t *cu, int32_t *cuc, int32_t *chunk_off, int32_t *order, int n_seq,
                               int64_t T, hipStream_t s) {
    launch_k(chunk_offsets_kernel, dim3(1), dim3(64), 0, s, cu, cuc, chunk_off, n_seq, (int32_t)T);
    if (order) launch_k(seq_order_kernel, dim3((n_seq + 255) / 256), dim3(256), 0, s, cuc, order, n_seq);
    return hipGetLastError();
}

hipError_t launch_prep(Dt dt, int K, const PrepParams &p, int n_chunks_ub, hipStream_t s) {
    if (dt == Dt::BF16)
        return K == 128 ? launch_prep_t<bf16, 128>(p, n_chunks_ub, s) : launch_prep_t<bf16, 64>(p, n_chunks_ub, s);
    return K == 128 ? launch_prep_t<float, 128>(p, n_chunks_ub, s) : launch_prep_t<float, 64>(p, n_chunks_ub, s);
}

size_t tblock_bytes(Dt dt) { return dt == Dt::BF16 ? TBlockF<bf16>::BYTES : TBlock<float>::BYTES; }
size_t tblock_bytes_fwd(Dt dt) { return dt == Dt::BF16 ? TBlockF<bf16>::BYTES : TBlockF<float>::BYTES; }

hipError_t launch_wu(Dt dt, const WUParams &p, int n_chunks_ub, hipStream_t s) {
    dim3 grid(n_chunks_ub, p.Hv);
    if (dt == Dt::BF16)
        launch_k(wu_kernel<bf16>, grid, dim3(NTHR), 0, s, p);
    else
        launch_k(wu_kernel<float>, grid, dim3(NTHR), 0, s, p);
    return hipGetLastError();
}

}  // namespace gdr
