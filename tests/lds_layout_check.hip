// Host-side check of the kernels' LDS layouts (built with --cuda-host-only and
// run on the CPU by test_lds_layout.py).  For each operand read the kernels
// make of a swizzled tile, it forms the byte address of every lane with the
// layout functions the kernels use (gdr_layout.hpp, gdr_lds.hpp) and prices it
// with the bank model measured on gfx950 (64 banks of 4 bytes):
//   16-byte reads: 4 passes of 16 lanes; pass p takes lanes 0-3 and 12-15 of
//     16-lane group p and lanes 4-11 of group p ^ 1;
//   8-byte reads (plain and transposing) and writes: 2 passes of 32 lanes.
// A pass costs the largest number of distinct addresses that fall on one bank
// slot (16 bytes wide for 16-byte reads, 8 bytes for 8-byte accesses); an
// instruction's cost is its passes' mean, 1 when conflict-free.  Prints one
// line "name cost" per access pattern (the worst over the pattern's
// instructions), then "bijective ok|FAIL" for the chunk permutations.
#include <stdio.h>
#include <set>
#include <map>
#include <vector>

#include "gdr_lds.hpp"

using namespace gdr;

static double cost16(const std::vector<int> &a) {
    double t = 0;
    for (int p = 0; p < 4; ++p) {
        std::map<int, std::set<int>> b;
        for (int m = 0; m < 16; ++m) {
            const int l = m + 16 * (p ^ (((m >> 2) ^ (m >> 3)) & 1));
            b[(a[l] >> 4) & 15].insert(a[l] >> 4);
        }
        size_t mx = 0;
        for (auto &kv : b) mx = kv.second.size() > mx ? kv.second.size() : mx;
        t += (double)mx;
    }
    return t / 4;
}
static double cost8(const std::vector<int> &a) {
    double t = 0;
    for (int p = 0; p < 2; ++p) {
        std::map<int, std::set<int>> b;
        for (int l = 32 * p; l < 32 * p + 32; ++l) b[(a[l] >> 3) & 31].insert(a[l] >> 3);
        size_t mx = 0;
        for (auto &kv : b) mx = kv.second.size() > mx ? kv.second.size() : mx;
        t += (double)mx;
    }
    return t / 2;
}

template <typename F> static double worst(int n_inst, bool b16, F addr) {
    double w = 0;
    for (int i = 0; i < n_inst; ++i) {
        std::vector<int> a(64);
        for (int l = 0; l < 64; ++l) a[l] = addr(i, l & 15, l >> 4);
        const double c = b16 ? cost16(a) : cost8(a);
        w = c > w ? c : w;
    }
    return w;
}

int main() {
    // ---- forward scan (bf16, K = 128, 64 value columns per workgroup)
    using SK = Swz<256, KeyKQ>;
    using SV = Swz<128, KeyVP>;
    using SP = Swz<128, KeyP>;
    using TF = TBlockF<bf16>;
    // K h: K rows in slot order, 8 keys from 32 dp + 8 g
    printf("fwd_Kh %.2f\n", worst(16, true, [](int i, int n, int g) {
               return SK::off(slot_row(i & 3, n), (32 * (i >> 2) + 8 * g) * 2); }));
    // scores and Q h: K or Q rows 16 t + n
    printf("fwd_KQ_rows %.2f\n", worst(16, true, [](int i, int n, int g) {
               return SK::off(16 * (i & 3) + n, (32 * (i >> 2) + 8 * g) * 2); }));
    // T operand: slot rows, k block ip <= rt / 2
    printf("fwd_T %.2f\n", worst(8, true, [](int i, int n, int g) {
               const int rt = i & 3, ip = (i >> 2) <= rt / 2 ? (i >> 2) : 0;
               return TF::off(slot_row(rt, n), (32 * ip + 8 * g) * 2); }));
    // score planes: operand reads of rows 16 rt + n and the tiles' 8-byte writes
    printf("fwd_P_read %.2f\n", worst(8, true, [](int i, int n, int g) {
               const int rt = i & 3, ip = (i >> 2) <= rt / 2 ? (i >> 2) : 0;
               return SP::off(16 * rt + n, (32 * ip + 8 * g) * 2); }));
    printf("fwd_P_write %.2f\n", worst(16, false, [](int i, int n, int g) {
               return SP::off(16 * (i & 3) + n, (16 * (i >> 2) + 4 * g) * 2); }));
    // V columns, transposing reads: rows slot_base(rt, g) + n / 4, columns 16 w + 4 (n % 4)
    printf("fwd_V_tr %.2f\n", worst(16, false, [](int i, int n, int g) {
               return SV::off(slot_base(i & 3, g) + (n >> 2), 2 * (16 * (i >> 2) + 4 * (n & 3))); }));
    // K^T, transposing reads (one half of each 16-byte column per pass: 2-way by construction)
    printf("fwd_KT_tr %.2f\n", worst(32, false, [](int i, int n, int g) {
               const int dt = i & 7, r0 = (i >> 3) & 1 ? 32 : 0, d = (i >> 4) & 1 ? 4 : 0;
               const int c0 = 32 * (dt >> 1) + 4 * (dt & 1);
               return SK::off(r0 + 8 * g + (n >> 2) + d, 2 * (c0 + 8 * (n & 3))); }));

    // ---- backward (bf16): tiles with 128-byte rows under the default key
    using S128 = Swz<128>;
    // split-plane operand reads of 16 consecutive rows: bytes 64 ip + 8 g and 32 more
    printf("bwd_rows_b64 %.2f\n", worst(16, false, [](int i, int n, int g) {
               return S128::off(16 * (i & 3) + n, 64 * ((i >> 2) & 1) + 8 * g + ((i >> 3) & 1) * 32); }));
    // transposing reads: rows r0 + 4 g + n / 4, columns d0 + 4 (n % 4)
    printf("bwd_tr %.2f\n", worst(16, false, [](int i, int n, int g) {
               return S128::off(16 * (i & 3) + 4 * g + (n >> 2), 2 * (16 * (i >> 2) + 4 * (n & 3))); }));
    // 8-byte writes of rows 16 rt + n at columns 16 w + 4 g
    printf("bwd_put4 %.2f\n", worst(16, false, [](int i, int n, int g) {
               return S128::off(16 * (i & 3) + n, 2 * (16 * (i >> 2) + 4 * g)); }));
    // the compact T block as the backward reads it: 8-byte reads of rows 16 rt + n
    // (k block ip <= rt / 2, bytes 64 ip + 8 g and 32 more) and transposing reads of
    // rows 32 ip + 4 g + n / 4 (+16) at columns 16 rt + 4 (n % 4), ip >= rt / 2
    printf("bwd_T_rows %.2f\n", worst(16, false, [](int i, int n, int g) {
               const int rt = i & 3, ip = ((i >> 2) & 1) <= rt / 2 ? ((i >> 2) & 1) : 0;
               return TF::off(16 * rt + n, 64 * ip + 8 * g + ((i >> 3) & 1) * 32); }));
    printf("bwd_T_tr %.2f\n", worst(16, false, [](int i, int n, int g) {
               const int rt = i & 3, ip = ((i >> 2) & 1) >= rt / 2 ? ((i >> 2) & 1) : 1;
               return TF::off(32 * ip + 4 * g + (n >> 2) + ((i >> 3) & 1) * 16, 2 * (16 * rt + 4 * (n & 3))); }));
    // the states pass's 16-byte T reads of fp32-free blocks: the compact block, slot rows
    printf("bwd_states_T %.2f\n", worst(8, true, [](int i, int n, int g) {
               const int rt = i & 3, ip = (i >> 2) <= rt / 2 ? (i >> 2) : 0;
               return TF::off(slot_row(rt, n), (32 * ip + 8 * g) * 2); }));

    // ---- reverse scan (bf16, K = 128): K and Q tiles under KeyBK
    using SB = Swz<256, KeyBK>;
    // transposing reads of K^T, Q^T: rows 32 ip + 4 g + n / 4 (+16), keys c0 + 8 (n % 4)
    // (all lanes in one 8-byte half of their 16-byte column: 2-way at best)
    printf("bwd_KT_tr %.2f\n", worst(32, false, [](int i, int n, int g) {
               const int dt = i & 7, ip = (i >> 3) & 1, h = (i >> 4) & 1;
               const int c0 = 32 * (dt >> 1) + 4 * (dt & 1);
               return SB::off(32 * ip + 4 * g + (n >> 2) + 16 * h, 2 * (c0 + 8 * (n & 3))); }));
    printf("bwd_KT_tr_rowkey %.2f\n", worst(32, false, [](int i, int n, int g) {
               const int dt = i & 7, ip = (i >> 3) & 1, h = (i >> 4) & 1;
               const int c0 = 32 * (dt >> 1) + 4 * (dt & 1);
               return Swz<256>::off(32 * ip + 4 * g + (n >> 2) + 16 * h, 2 * (c0 + 8 * (n & 3))); }));
    // K rows for K dh': 16-byte reads of rows 16 rt + n at keys 32 dp + 8 g
    printf("bwd_K_rows16 %.2f\n", worst(16, true, [](int i, int n, int g) {
               return SB::off(16 * (i & 3) + n, 2 * (32 * (i >> 2) + 8 * g)); }));
    // score tiles: 8-byte reads of rows 16 t + n at keys 32 dp + 4 g and 16 more
    printf("bwd_KQ_rows8 %.2f\n", worst(32, false, [](int i, int n, int g) {
               return SB::off(16 * (i & 3) + n, 2 * (32 * ((i >> 2) & 3) + 4 * g) + 32 * ((i >> 4) & 1)); }));

    // chunk-local backward: transposing reads of K^T, Q^T at rows 32 ip + 4 g + n / 4
    // (+16), keys 16 td + 4 (n % 4), and 8-byte reads of rows 16 tr + n at keys 16 td + 4 g
    printf("bwd_local_KT_tr %.2f\n", worst(32, false, [](int i, int n, int g) {
               const int td = i & 7, ip = (i >> 3) & 1, h = (i >> 4) & 1;
               return SB::off(32 * ip + 4 * g + (n >> 2) + 16 * h, 2 * (16 * td + 4 * (n & 3))); }));
    printf("bwd_local_KQ_rows4 %.2f\n", worst(32, false, [](int i, int n, int g) {
               return SB::off(16 * (i & 3) + n, 2 * (16 * (i >> 2) + 4 * g)); }));

    // ---- every row's chunk map is a permutation (no two logical chunks share a slot)
    bool ok = true;
    auto perm = [&](auto S, int rows) {
        using SS = decltype(S);
        for (int r = 0; r < rows; ++r) {
            std::set<int> seen;
            for (int c = 0; c < SS::S; ++c) seen.insert(SS::chunk(r, c));
            ok = ok && (int)seen.size() == SS::S;
        }
    };
    perm(SK{}, 64);
    perm(SV{}, 64);
    perm(SP{}, 64);
    perm(S128{}, 64);
    perm(Swz<256>{}, 64);
    perm(SB{}, 64);
    {
        std::set<int> seen;  // compact T block: every (row, column chunk) at its own 16 bytes, inside a plane
        for (int r = 0; r < 64; ++r)
            for (int c = 0; c < (r < 32 ? 4 : 8); ++c) {
                const int o = TF::off(r, 16 * c);
                ok = ok && o >= 0 && o + 16 <= TF::PLANE && (o & 15) == 0;
                seen.insert(o);
            }
        ok = ok && (int)seen.size() == 32 * 4 + 32 * 8;
    }
    printf("bijective %s\n", ok ? "ok" : "FAIL");
    return 0;
}
