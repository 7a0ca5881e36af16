// Backward of the layer (the training side): grouped GEMMs on bf16 MFMA with
// fp32 accumulation, gfx950.
//
// Given the upstream gradient dO = dLoss/dout and the state a training
// forward saved (routing, permutation, the gate/up pre-activations
// Z = [W1 x | W3 x] of every row), per row r of group g (token t, gate g_r;
// g_r = 1 for a shared expert), with A = W1 x, B = W3 x:
//
//   dH'  = dO[t] . W2_g                    (dH GEMM, K = d)
//   dgate_r = <dH', silu(A) * B>           (= <dO, y>: Y is never needed,
//                                          the SonicMoE note's dH-kernel idea)
//   dH   = g_r dH',  dA = dH * B * silu'(A),  dB = dH * silu(A)
//   dX_r = [dA | dB] . [W1_g ; W3_g]       (dX GEMM, K = 2 inter)
//   dW2_g  = sum_r dO[t_r] (x) g_r H_r     (dW2 GEMM, K = rows of g)
//   dW1_g | dW3_g = sum_r [dA | dB]_r (x) x[t_r]   (dW13 GEMM, K = rows of g)
//
// and for the router, with dL the affinity gradients of every token (from
// the gate gradients through the softmax / sigmoid, and the expert-level
// balance term — "DeepSeekMoE 深度解读报告", sections 2.5 / 3.2):
//
//   dx_router = dL . C,   dC = dL^T . x
//
// Every one of these products has its second operand stored with the
// reduction index as the slow one ("K-major": W2 [d][I] read along d, W1 /
// W3 [I][d] along I, C [E][d] along E, and the activations [rows][..]
// along rows in the weight-gradient GEMMs).  gfx950's LDS transpose read
// (ds_read_b64_tr_b16) turns such a tile into MFMA fragments directly: in
// each group of 16 lanes, lane 4e + q reads 4 consecutive elements of row
// k0 + e at column 4q, and lane j receives the 4 elements of column j, rows
// k0..k0+3.  Two such reads give a lane the 8 consecutive k of its column
// that one v_mfma_f32_32x32x16_bf16 operand needs.  So the K-major tiles
// load as whole 512-byte row pieces, straight to LDS, with no transposed
// copy of any weight or activation.
//
// Tile: 256 x 256 outputs, eight waves (2 along M, 4 along N) of 128 x 64,
// BK = 64, a ring of five 32 KB LDS slots holding one operand half (the A or
// the B part of a slice) each, direct-to-LDS buffer loads, one barrier per
// slice.  Layouts in LDS:
//   K-contiguous operand: [256 rows][64 k], 16-byte chunk c of row r at
//     position c ^ ((r / 2) mod 8) (conflict-free ds_read_b128 fragments)
//   K-major operand: [64 k][256 cols], 16-byte chunk c of row k at
//     position c ^ 4 (k mod 4), so that the 32 lanes one transpose read
//     serves (4 rows x 64 bytes) hit 64 distinct banks.
#include "common.h"

namespace moe {
namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) bf16_t lds_bf16_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));

constexpr int kBT = 256;                  // tile rows = tile columns
constexpr int kBK = 64;                   // k per slice
constexpr int kNW = 8;                    // waves: 2 along M x 4 along N
constexpr int kHalf = kBT * kBK;          // elements of one operand slice (32 KB)
constexpr int kSlots = 5;                 // LDS ring of operand halves (32 KB each)
constexpr int kLdsBytes = kSlots * kHalf * 2;
constexpr int kLoads = kHalf * 2 / 1024 / kNW; // 1 KB load instructions per wave per operand slice
static_assert(kLoads == 4, "four loads per wave per operand slice");

// The six products (see the header).
enum Kind { K_DH = 0, K_DX = 1, K_DXR = 2, K_DW2 = 3, K_DW13 = 4, K_DC = 5 };

// A operand K-contiguous (A[m][k]) for the products whose M runs over rows.
__host__ __device__ constexpr bool a_kcontig(int kind) { return kind <= K_DXR; }

struct BwdParams {
    // grouping
    const int32_t* goff;       // [G + 1] first row of each group
    const int32_t* tok_of;     // [rows] token of each row
    const Tile* tiles;         // NN products: work list
    const int32_t* ntiles;     //   and its length
    const int32_t* gorder;     // TN products: groups, most rows first
    int ngt;                   //   and how many of them get tiles
    int E, Ks, T, K, d, I, Is, Epad;
    uint32_t flags;
    // inputs
    const bf16_t* x;           // [T, d]
    const bf16_t* dO;          // [T, d]
    const bf16_t* C;           // [E, d]
    const bf16_t *w1, *w3, *w2, *ws1, *ws3, *ws2;
    const bf16_t* Z;           // saved pre-activations: routed [T K, 2 I], shared [T Ks, 2 Is]
    const bf16_t* H;           // saved SwiGLU outputs:  routed [T K, I], shared [T Ks, Is]
    const float* row_gate;     // [T K] gate of each routed row
    // intermediates
    bf16_t* dZ;                // like Z
    bf16_t* gH;                // routed [T K, I]: g_r * H_r
    float* dgp;                // [rows, ceil(max(I, Is) / 256)] dgate partials
    const bf16_t* dL;          // [T, Epad] affinity gradients
    float* R32;                // [T, d] dO (residual) + dL . C
    bf16_t* dXr;               // [rows, d]
    // outputs
    bf16_t *dw1, *dw3, *dw2, *dws1, *dws3, *dws2;
    float* dC;                 // [E, d]
};

__device__ __forceinline__ float silu_f(float a) { return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }

template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

// LDS transpose reads (ds_read_b64_tr_b16, byte addresses), issued together
// and waited for in the same statement.  Written out because the compiler
// puts a wait for every direct-to-LDS load in flight (vmcnt(0)) in front of
// each transpose-read builtin, which would stall the operand ring at every
// fragment read; an ordinary LDS read gets no such wait.  These run after
// the MFMAs of the previous k16 step have been issued, under them.
__device__ __forceinline__ void tr_reads4(u32x2v (&r)[4], const uint32_t (&a)[4]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %5\n\t"
        "ds_read_b64_tr_b16 %2, %6\n\t"
        "ds_read_b64_tr_b16 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
}
__device__ __forceinline__ void tr_reads12(u32x2v (&r)[12], const uint32_t (&a)[12]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %12\n\t"
        "ds_read_b64_tr_b16 %1, %13\n\t"
        "ds_read_b64_tr_b16 %2, %14\n\t"
        "ds_read_b64_tr_b16 %3, %15\n\t"
        "ds_read_b64_tr_b16 %4, %16\n\t"
        "ds_read_b64_tr_b16 %5, %17\n\t"
        "ds_read_b64_tr_b16 %6, %18\n\t"
        "ds_read_b64_tr_b16 %7, %19\n\t"
        "ds_read_b64_tr_b16 %8, %20\n\t"
        "ds_read_b64_tr_b16 %9, %21\n\t"
        "ds_read_b64_tr_b16 %10, %22\n\t"
        "ds_read_b64_tr_b16 %11, %23\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
          "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
          "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11])
        : "memory");
}

__device__ __forceinline__ uint32_t kmajor_pos(int k, int chunk) {   // byte offset in a K-major slice
    return (uint32_t)(k * (kBT * 2) + ((chunk ^ (4 * (k & 3))) << 4));
}

// Tile coordinates and operand sources, resolved once per tile.
struct TileCtx {
    int g;            // group
    bool shared;
    int m0, n0;       // first output row / column of the tile
    int mrows, ncols; // valid output rows / columns of the tile
    int kdim;         // reduction length (a multiple of 64 for the NN products)
    int row0;         // first row of the group (global row space)
};

// ---------------------------------------------------------------------------
// The kernel.  One tile per workgroup.
// ---------------------------------------------------------------------------
template <int KIND>
__global__ __launch_bounds__(64 * kNW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_gemm_kernel(BwdParams P) {
    __shared__ __attribute__((aligned(1024))) bf16_t smem[kLdsBytes / 2];
    constexpr bool ACONT = a_kcontig(KIND);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;

    // ---- which tile ----
    TileCtx tc;
    if (ACONT) {
        // NN products: a work-list entry (group, m0 over the group's rows, n0)
        if (KIND == K_DXR) {
            const int nt = (P.d + kBT - 1) / kBT;
            const int b = blockIdx.x;
            tc.g = 0;
            tc.shared = false;
            tc.m0 = (b / nt) * kBT;
            tc.n0 = (b % nt) * kBT;
            if (tc.m0 >= P.T) return;
            tc.mrows = min(kBT, P.T - tc.m0);
            tc.ncols = min(kBT, P.d - tc.n0);
            tc.kdim = P.Epad;
            tc.row0 = 0;
        } else {
            if ((int)blockIdx.x >= *P.ntiles) return;
            const Tile t = P.tiles[blockIdx.x];
            tc.g = t.group;
            tc.shared = t.group >= P.E;
            tc.m0 = t.m0;
            tc.n0 = t.n0;
            tc.mrows = t.nrows;
            tc.row0 = P.goff[t.group];
            const int inter = tc.shared ? P.Is : P.I;
            if (KIND == K_DH) {
                tc.ncols = min(kBT, inter - t.n0);
                tc.kdim = P.d;
            } else {
                tc.ncols = min(kBT, P.d - t.n0);
                tc.kdim = 2 * inter;
            }
        }
    } else {
        // TN products: blockIdx -> (group in size order, m tile, n tile);
        // K runs over the group's rows
        int mt, nt, gi, rem;
        if (KIND == K_DC) {
            mt = P.Epad / kBT + (P.Epad % kBT != 0);
            nt = (P.d + kBT - 1) / kBT;
            gi = 0;
            rem = blockIdx.x;
            if (rem >= mt * nt) return;
            tc.g = 0;
            tc.shared = false;
            tc.row0 = 0;
            tc.kdim = P.T;
            tc.m0 = (rem / nt) * kBT;
            tc.n0 = (rem % nt) * kBT;
            tc.mrows = min(kBT, P.E - tc.m0);
            tc.ncols = min(kBT, P.d - tc.n0);
            if (tc.mrows <= 0) return;
        } else {
            // every group gets the routed tile grid (the larger of routed /
            // shared inter sizes); tiles past a group's own extent exit
            const int inter_max = P.I > P.Is ? P.I : P.Is;
            const int M = KIND == K_DW2 ? P.d : 2 * inter_max;
            const int N = KIND == K_DW2 ? inter_max : P.d;
            mt = (M + kBT - 1) / kBT;
            nt = (N + kBT - 1) / kBT;
            gi = blockIdx.x / (mt * nt);
            rem = blockIdx.x - gi * (mt * nt);
            if (gi >= P.ngt) return;
            tc.g = P.gorder[gi];
            tc.shared = tc.g >= P.E;
            const int inter = tc.shared ? P.Is : P.I;
            const int Mg = KIND == K_DW2 ? P.d : 2 * inter;
            const int Ng = KIND == K_DW2 ? inter : P.d;
            tc.m0 = (rem / nt) * kBT;
            tc.n0 = (rem % nt) * kBT;
            if (tc.m0 >= Mg || tc.n0 >= Ng) return;
            tc.mrows = min(kBT, Mg - tc.m0);
            tc.ncols = min(kBT, Ng - tc.n0);
            tc.row0 = P.goff[tc.g];
            tc.kdim = P.goff[tc.g + 1] - tc.row0;
        }
    }
    const int TK = P.T * P.K;
    const int inter = tc.shared ? P.Is : P.I;
    const int rrow0 = tc.shared ? tc.row0 - TK : tc.row0;   // first row within its region
    const int sidx = tc.g - P.E;                             // shared expert index

    // bf16 outputs (dX rows, dW2, dW1 | dW3): the start of output row m of
    // the tile (column n0); every output width is a multiple of 64, so a
    // tile row is whole 16-byte pieces
    constexpr bool STAGED = KIND == K_DX || KIND == K_DW2 || KIND == K_DW13;
    auto out_row = [&](int m) -> bf16_t* {
        const int row = tc.m0 + m;
        if (KIND == K_DX) return P.dXr + (size_t)(tc.row0 + row) * P.d + tc.n0;
        if (KIND == K_DW2) {
            bf16_t* o = tc.shared ? P.dws2 + (size_t)sidx * P.d * P.Is : P.dw2 + (size_t)tc.g * P.d * P.I;
            return o + (size_t)row * inter + tc.n0;
        }
        const bool up = row >= inter;                          // K_DW13
        bf16_t* o = tc.shared ? (up ? P.dws3 : P.dws1) + (size_t)sidx * P.Is * P.d
                              : (up ? P.dw3 : P.dw1) + (size_t)tc.g * P.I * P.d;
        return o + (size_t)(up ? row - inter : row) * P.d + tc.n0;
    };
    // an expert no row chose: its weight gradients are zero, written as
    // whole rows (32 lanes per 512-byte tile row), nothing else to do
    if ((KIND == K_DW2 || KIND == K_DW13) && tc.kdim == 0) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        const int cpr = tc.ncols >> 3;
        for (int idx = tid; idx < tc.mrows * 32; idx += 64 * kNW) {
            const int m = idx >> 5, c = idx & 31;
            if (c < cpr) __builtin_nontemporal_store(z, reinterpret_cast<u32x4*>(out_row(m) + 8 * c));
        }
        return;
    }

    // ---- operand A ----
    // K-contiguous (NN): rows of the tile; the slice's k offset in the scalar offset.
    // K-major (TN): rows are k (the group's rows), columns m0 .. m0 + 255.
    __amdgpu_buffer_rsrc_t ra;
    uint32_t a_off[kLoads];                 // K-contig: per-load row byte offsets
    int a_ld = 0;                           // K-major: row pitch in elements
    if (KIND == K_DH) {                     // dO rows of the tile's tokens
        ra = make_rsrc(P.dO, (uint32_t)((size_t)P.T * P.d * 2));
    } else if (KIND == K_DX) {              // dZ rows
        const bf16_t* base = tc.shared ? P.dZ + (size_t)TK * 2 * P.I : P.dZ;
        const size_t nrow = tc.shared ? (size_t)P.T * P.Ks : (size_t)TK;
        ra = make_rsrc(base, (uint32_t)(nrow * 2 * inter * 2));
    } else if (KIND == K_DXR) {             // dL rows
        ra = make_rsrc(P.dL, (uint32_t)((size_t)P.T * P.Epad * 2));
    } else if (KIND == K_DW2) {             // dO, rows gathered
        ra = make_rsrc(P.dO, (uint32_t)((size_t)P.T * P.d * 2));
        a_ld = P.d;
    } else if (KIND == K_DW13) {            // dZ rows in place
        const bf16_t* base = tc.shared ? P.dZ + (size_t)TK * 2 * P.I : P.dZ;
        const size_t nrow = tc.shared ? (size_t)P.T * P.Ks : (size_t)TK;
        ra = make_rsrc(base, (uint32_t)(nrow * 2 * inter * 2));
        a_ld = 2 * inter;
    } else {                                // K_DC: dL rows = tokens
        ra = make_rsrc(P.dL, (uint32_t)((size_t)P.T * P.Epad * 2));
        a_ld = P.Epad;
    }
    if (ACONT) {
        // load q of this wave fills rows 8 (wave + 8 q) .. + 7; lane l the
        // position l % 8 of row 8 (wave + 8 q) + l / 8
#pragma unroll
        for (int q = 0; q < kLoads; ++q) {
            const int row = 8 * (wave + kNW * q) + (lane >> 3);
            const int rr = row < tc.mrows ? row : 0;
            const uint32_t cb = (uint32_t)(((lane & 7) ^ ((row >> 1) & 7)) << 4);
            uint32_t grow;
            const int kd = KIND == K_DH ? P.d : (KIND == K_DX ? 2 * inter : P.Epad);
            if (KIND == K_DH) grow = (uint32_t)P.tok_of[tc.row0 + tc.m0 + rr];
            else if (KIND == K_DX) grow = (uint32_t)(rrow0 + tc.m0 + rr);
            else grow = (uint32_t)(tc.m0 + rr);
            a_off[q] = grow * (uint32_t)kd * 2u + cb;
        }
    }

    // ---- operand B (always K-major) ----
    // rows k of the slice: NN products — weight rows (two matrices for dX);
    // TN products — the group's rows (gathered for x).
    __amdgpu_buffer_rsrc_t rb1, rb2;
    int b_ld, b_split;                      // row pitch (elements); dX: rows >= b_split from rb2
    if (KIND == K_DH) {
        const bf16_t* w = tc.shared ? P.ws2 + (size_t)sidx * P.d * P.Is : P.w2 + (size_t)tc.g * P.d * P.I;
        rb1 = rb2 = make_rsrc(w, (uint32_t)((size_t)P.d * inter * 2));
        b_ld = inter;
        b_split = 1 << 30;
    } else if (KIND == K_DX) {
        const size_t o = tc.shared ? (size_t)sidx * P.Is * P.d : (size_t)tc.g * P.I * P.d;
        rb1 = make_rsrc((tc.shared ? P.ws1 : P.w1) + o, (uint32_t)((size_t)inter * P.d * 2));
        rb2 = make_rsrc((tc.shared ? P.ws3 : P.w3) + o, (uint32_t)((size_t)inter * P.d * 2));
        b_ld = P.d;
        b_split = inter;
    } else if (KIND == K_DXR) {
        rb1 = rb2 = make_rsrc(P.C, (uint32_t)((size_t)P.E * P.d * 2));   // rows >= E read 0
        b_ld = P.d;
        b_split = 1 << 30;
    } else if (KIND == K_DW2) {             // g H (routed) or H (shared)
        const bf16_t* base = tc.shared ? P.H + (size_t)TK * P.I : P.gH;
        const size_t nrow = tc.shared ? (size_t)P.T * P.Ks : (size_t)TK;
        rb1 = rb2 = make_rsrc(base, (uint32_t)(nrow * inter * 2));
        b_ld = inter;
        b_split = 1 << 30;
    } else {                                // dW13, dC: x rows
        rb1 = rb2 = make_rsrc(P.x, (uint32_t)((size_t)P.T * P.d * 2));
        b_ld = P.d;
        b_split = 1 << 30;
    }

    // ---- loads ----
    // LDS is a ring of five 32 KB slots, one operand half each: A of slice
    // s in slot 2s mod 5, B in slot 2s + 1 mod 5.  Iteration kt loads A of
    // slice kt + 2 over its first three k16 steps (into the slot B of slice
    // kt - 1 left) and B of slice kt + 2 after the barrier that ends the
    // reads of slice kt (into A of slice kt's slot), so every load has at
    // least one slice of MFMA time to land and half of them nearly two.
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem + (uint32_t)(wave * 1024));
    auto slot_of = [](int h) { return h % kSlots; };
    // K-major slices: load q of this wave fills rows 2 (wave + 8 q) + l / 32
    // (two 512-byte rows per instruction); lane l fills physical chunk l % 32.
    auto kmajor_row = [&](int q) { return 2 * (wave + kNW * q) + (lane >> 5); };
    const int kchunk = lane & 31;
    // TN products: the token of each gathered k row (dO rows for dW2, x
    // rows for dW13), two sets by the parity of the slice, looked up three
    // slices ahead of the slice's first load and first used there (a use
    // right after the lookup would wait for every load in flight).  The
    // lookup is made for every lane (row clamped), so each fetch issues the
    // same loads.
    // gcur: the slice whose loads go out this iteration; gnext: the one
    // after, rotated in at the top of each iteration (by then its lookups
    // have had a whole iteration to land)
    constexpr bool GATHER = KIND == K_DW2 || KIND == K_DW13;
    int gcur[kLoads], gnext[kLoads];
    auto fetch_rows = [&](int (&g)[kLoads], int s) {
        if (!GATHER) return;
#pragma unroll
        for (int q = 0; q < kLoads; ++q) {
            const int kr = min(s * kBK + kmajor_row(q), tc.kdim - 1);
            g[q] = P.tok_of[tc.row0 + kr];
        }
    };
    // global row (element index of its first column) of the k row of load q
    // of slice s (TN, its lookups in gcur), -1 past the group (read as 0)
    auto tn_row = [&](int s, int q, bool for_a) -> int {
        const int kr = s * kBK + kmajor_row(q);
        if (kr >= tc.kdim) return -1;
        if (KIND == K_DC) return kr;
        const int own = tc.shared ? tc.row0 + kr - TK : tc.row0 + kr;   // row in its region
        const int tok = GATHER ? gcur[q] : 0;
        if (KIND == K_DW2) return for_a ? tok : own;
        return for_a ? own : tok;                                        // K_DW13
    };
    auto issue_a = [&](int s, int q) {
        const uint32_t dst = lds0 + (uint32_t)(slot_of(2 * s) * kHalf * 2) + (uint32_t)(kNW * q * 1024);
        if (ACONT) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(uintptr_t)dst, 16, (int)a_off[q],
                                                     s * kBK * 2, 0, 0);
        } else {
            const int row = tn_row(s, q, true);
            const int k = kmajor_row(q);
            const uint32_t c = (uint32_t)(kchunk ^ (4 * (k & 3)));
            const uint32_t off = row < 0 ? 0x80000000u
                                         : ((uint32_t)row * (uint32_t)a_ld + (uint32_t)tc.m0) * 2u + c * 16u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(uintptr_t)dst, 16, (int)off, 0, 0, 0);
        }
    };
    auto issue_b = [&](int s, int q) {
        const uint32_t dst = lds0 + (uint32_t)(slot_of(2 * s + 1) * kHalf * 2) + (uint32_t)(kNW * q * 1024);
        const int k = kmajor_row(q);
        const uint32_t c = (uint32_t)(kchunk ^ (4 * (k & 3)));
        int row;
        if (ACONT) row = s * kBK + k;              // weight row (dXR: rows >= E are past the resource)
        else row = tn_row(s, q, false);
        const bool second = ACONT && row >= b_split;
        const int wr = second ? row - b_split : row;
        const uint32_t off = row < 0 ? 0x80000000u
                                     : ((uint32_t)wr * (uint32_t)b_ld + (uint32_t)tc.n0) * 2u + c * 16u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(second ? rb2 : rb1, (lds_ptr_t)(uintptr_t)dst, 16,
                                                 (int)off, 0, 0, 0);
    };

    // ---- fragments ----
    // acc[i][j]: m block i (32 rows of the wave's 128), n block j (32 of its
    // 64); the weight / second operand is the MFMA's first operand, so lane l
    // holds output row m = wm*128 + 32 i + (l & 31) and columns
    // n = wn*64 + 32 j + 8 (r / 4) + 4 (l / 32) + r % 4.
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    const int lrow = lane & 31;
    const int g16 = lane >> 4, i16 = lane & 15;
    // transpose read of a K-major slice: 4 k of column block cb for step st, half h
    // byte address of transpose read h (k 4h .. 4h + 3 of the lane's 8) of
    // the fragment of column block cb, step st: lane 4e + q of each 16-lane
    // group reads row k0 + e at columns 4q .. 4q + 3
    auto tr_addr = [&](const lds_bf16_t* base, int cb, int st, int h) -> uint32_t {
        const int k = 16 * st + 8 * (g16 >> 1) + 4 * h + (i16 >> 2);
        const int c = (cb >> 3) + 2 * (g16 & 1) + ((i16 & 3) >> 1);
        return (uint32_t)(uintptr_t)base + kmajor_pos(k, c) + 8u * (uint32_t)(i16 & 1);
    };
    auto frag_of = [](u32x2v lo, u32x2v hi) -> bf16x8 {
        const u32x4 v = {lo.x, lo.y, hi.x, hi.y};
        return __builtin_bit_cast(bf16x8, v);
    };
    auto frag_kcontig = [&](const lds_bf16_t* base, int row, int st) -> bf16x8 {
        const int chunk = 2 * st + (lane >> 5);
        return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
            base + row * kBK + ((chunk ^ ((row >> 1) & 7)) << 3));
    };
    // fragments of step st of slice s into register set `set`; the MFMAs of a set
    bf16x8 fa[2][4], fb[2][2];
    // NA: this wave's 32-row blocks of A that hold rows of the tile (NN
    // products; a compile-time constant per main-loop instance): a ragged
    // tile skips the reads and MFMAs of its padding blocks
    auto read_frags = [&](auto na_c, auto set_c, int s, int st) {
        constexpr int NA = decltype(na_c)::value;
        constexpr int SET = decltype(set_c)::value;
        const lds_bf16_t* sa = (const lds_bf16_t*)smem + slot_of(2 * s) * kHalf;
        const lds_bf16_t* sb = (const lds_bf16_t*)smem + slot_of(2 * s + 1) * kHalf;
        if (ACONT) {
            if (NA == 0) return;
#pragma unroll
            for (int i = 0; i < NA; ++i) fa[SET][i] = frag_kcontig(sa, wm * 128 + 32 * i + lrow, st);
            uint32_t ad[4];
            u32x2v r[4];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                ad[2 * j] = tr_addr(sb, wn * 64 + 32 * j, st, 0);
                ad[2 * j + 1] = tr_addr(sb, wn * 64 + 32 * j, st, 1);
            }
            tr_reads4(r, ad);
#pragma unroll
            for (int j = 0; j < 2; ++j) fb[SET][j] = frag_of(r[2 * j], r[2 * j + 1]);
        } else {
            uint32_t ad[12];
            u32x2v r[12];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                ad[2 * j] = tr_addr(sb, wn * 64 + 32 * j, st, 0);
                ad[2 * j + 1] = tr_addr(sb, wn * 64 + 32 * j, st, 1);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ad[4 + 2 * i] = tr_addr(sa, wm * 128 + 32 * i, st, 0);
                ad[5 + 2 * i] = tr_addr(sa, wm * 128 + 32 * i, st, 1);
            }
            tr_reads12(r, ad);
#pragma unroll
            for (int j = 0; j < 2; ++j) fb[SET][j] = frag_of(r[2 * j], r[2 * j + 1]);
#pragma unroll
            for (int i = 0; i < 4; ++i) fa[SET][i] = frag_of(r[4 + 2 * i], r[5 + 2 * i]);
        }
    };
    auto mfmas = [&](auto na_c, auto set_c) {
        constexpr int NA = decltype(na_c)::value;
        constexpr int SET = decltype(set_c)::value;
#pragma unroll
        for (int i = 0; i < NA; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[SET][j], fa[SET][i], acc[i][j], 0, 0, 0);
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;

    // ---- main loop over the ring ----
    // Order of this wave's vector-memory instructions (they complete in
    // order for the waits): the row lookups of slice kt + 3 (TN), then A of
    // slice kt + 2 over steps 0-2; the wait before the barrier lets only
    // those A loads stay in flight, so slice kt + 1 has landed.
    const int nk = (tc.kdim + kBK - 1) / kBK;
    auto main_loop = [&](auto na_c) {
        if (nk <= 0) return;
        fetch_rows(gcur, 0);
#pragma unroll
        for (int q = 0; q < kLoads; ++q) issue_a(0, q);
#pragma unroll
        for (int q = 0; q < kLoads; ++q) issue_b(0, q);
        if (nk > 1) {
            fetch_rows(gcur, 1);
            fetch_rows(gnext, 2);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < kLoads; ++q) issue_a(1, q);
#pragma unroll
            for (int q = 0; q < kLoads; ++q) issue_b(1, q);
            wait_vm<2 * kLoads>();                     // slice 0 landed
        } else {
            wait_vm<0>();
        }
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        read_frags(na_c, S0{}, 0, 0);
        for (int kt = 0; kt < nk; ++kt) {
            const bool more = kt + 2 < nk;
            if (GATHER) {                              // (unconditional: rows past the group clamp)
#pragma unroll
                for (int q = 0; q < kLoads; ++q) gcur[q] = gnext[q];   // slice kt + 2
                fetch_rows(gnext, kt + 3);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int st = 0; st < 3; ++st) {
                if (st & 1) {                          // the MFMAs first: the reads wait under them
                    mfmas(na_c, S1{});
                    read_frags(na_c, S0{}, kt, st + 1);
                } else {
                    mfmas(na_c, S0{});
                    read_frags(na_c, S1{}, kt, st + 1);
                }
                if (more)
#pragma unroll
                    for (int q = st * kLoads / 3; q < (st + 1) * kLoads / 3; ++q) issue_a(kt + 2, q);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (kt + 1 < nk) {
                if (more) wait_vm<kLoads>();           // slice kt + 1 landed (A of kt + 2 may not)
                else wait_vm<0>();
            }
            // this wave's reads of slice kt have returned before the barrier
            // after which A of slice kt's slot is refilled
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            mfmas(na_c, S1{});                         // step 3
            if (more)
#pragma unroll
                for (int q = 0; q < kLoads; ++q) issue_b(kt + 2, q);
            if (kt + 1 < nk) read_frags(na_c, S0{}, kt + 1, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if constexpr (!ACONT) {
        main_loop(std::integral_constant<int, 4>{});
    } else {
        // the instance for this wave's live blocks (wave-uniform)
        const int na = (tc.mrows - wm * 128 + 31) >> 5;
        if (na >= 4) main_loop(std::integral_constant<int, 4>{});
        else if (na == 3) main_loop(std::integral_constant<int, 3>{});
        else if (na == 2) main_loop(std::integral_constant<int, 2>{});
        else if (na == 1) main_loop(std::integral_constant<int, 1>{});
        else main_loop(std::integral_constant<int, 0>{});
    }

    // ---- epilogues ----
    const int mbase = wm * 128 + lrow;                  // + 32 i
    const int nbase = wn * 64 + 4 * (lane >> 5);         // + 32 j + 8 r4 (+ e)
    if (KIND == K_DH) {
        // C = dH' for rows r of the group, columns i of inter.  With A, B
        // from Z: H = silu(A) B, dgate partial = sum_i C * H over the tile's
        // columns; dH = g C, dA = dH B silu'(A), dB = dH silu(A).
        const size_t zld = 2 * (size_t)inter;
        const bf16_t* zb = tc.shared ? P.Z + (size_t)TK * 2 * P.I : P.Z;
        bf16_t* dzb = tc.shared ? P.dZ + (size_t)TK * 2 * P.I : P.dZ;
        float rowsum[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = mbase + 32 * i;
            const bool mv = m < tc.mrows;
            const int r = rrow0 + tc.m0 + (mv ? m : 0);   // row within its region
            const float g = tc.shared ? 1.0f : P.row_gate[mv ? tc.row0 + tc.m0 + m : tc.row0];
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int n = nbase + 32 * j + 8 * r4;
                    const int col = tc.n0 + n;
                    if (!mv || col >= inter) continue;            // inter % 64 == 0: whole runs
                    const u32x2 za = *reinterpret_cast<const u32x2*>(zb + (size_t)r * zld + col);
                    const u32x2 zbv = *reinterpret_cast<const u32x2*>(zb + (size_t)r * zld + inter + col);
                    const float av[4] = {bf16_to_f32((bf16_t)(za.x & 0xffff)), bf16_to_f32((bf16_t)(za.x >> 16)),
                                         bf16_to_f32((bf16_t)(za.y & 0xffff)), bf16_to_f32((bf16_t)(za.y >> 16))};
                    const float bv[4] = {bf16_to_f32((bf16_t)(zbv.x & 0xffff)), bf16_to_f32((bf16_t)(zbv.x >> 16)),
                                         bf16_to_f32((bf16_t)(zbv.y & 0xffff)), bf16_to_f32((bf16_t)(zbv.y >> 16))};
                    float da[4], db[4], gh[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float c = acc[i][j][4 * r4 + e];
                        const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-av[e]));
                        const float sl = av[e] * sg;
                        const float h = sl * bv[e];
                        s += c * h;
                        const float dh = g * c;
                        da[e] = dh * bv[e] * (sg * (1.0f + av[e] * (1.0f - sg)));
                        db[e] = dh * sl;
                        gh[e] = g * h;
                    }
                    *reinterpret_cast<u32x2*>(dzb + (size_t)r * zld + col) =
                        u32x2{pack_bf16x2(da[0], da[1]), pack_bf16x2(da[2], da[3])};
                    *reinterpret_cast<u32x2*>(dzb + (size_t)r * zld + inter + col) =
                        u32x2{pack_bf16x2(db[0], db[1]), pack_bf16x2(db[2], db[3])};
                    if (!tc.shared)
                        *reinterpret_cast<u32x2*>(P.gH + (size_t)r * P.I + col) =
                            u32x2{pack_bf16x2(gh[0], gh[1]), pack_bf16x2(gh[2], gh[3])};
                }
            // the wave's 64 columns: this lane's 32 and its partner's (lane ^ 32)
            s += __shfl_xor(s, 32, 64);
            rowsum[i] = s;
        }
        // the four waves along N, in order, through LDS (the stages are free)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __syncthreads();
        float* red = reinterpret_cast<float*>(smem);      // [4 wn][256 rows]
        if (lane < 32)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wn * kBT + wm * 128 + 32 * i + lane] = rowsum[i];
        __syncthreads();
        if (tid < kBT && tid < tc.mrows) {
            const float v = ((red[tid] + red[kBT + tid]) + red[2 * kBT + tid]) + red[3 * kBT + tid];
            const int ntile = (P.I > P.Is ? P.I : P.Is) / kBT + ((P.I > P.Is ? P.I : P.Is) % kBT != 0);
            P.dgp[(size_t)(tc.row0 + tc.m0 + tid) * ntile + tc.n0 / kBT] = v;
        }
        return;
    }
    if (STAGED) {
        // the tile (256 x 256 bf16, 128 KB) through the free ring: 16-byte
        // chunk c of row r at position c ^ (r mod 32), then out as whole rows
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __syncthreads();
        lds_bf16_t* stile = (lds_bf16_t*)smem;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int m = mbase + 32 * i;
                    const int n = nbase + 32 * j + 8 * r4;
                    const int off = m * kBT + (((n >> 3) ^ (m & 31)) << 3) + (n & 4);
                    *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(stile + off) =
                        u32x2{pack_bf16x2(acc[i][j][4 * r4], acc[i][j][4 * r4 + 1]),
                              pack_bf16x2(acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3])};
                }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __syncthreads();
        const int cpr = tc.ncols >> 3;
        for (int idx = tid; idx < tc.mrows * 32; idx += 64 * kNW) {
            const int m = idx >> 5, c = idx & 31;
            if (c < cpr) {
                const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                    stile + m * kBT + ((c ^ (m & 31)) << 3));
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out_row(m) + 8 * c));
            }
        }
        return;
    }
    // plain stores: 4 consecutive columns per (i, j, r4)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = mbase + 32 * i;
        if (m >= tc.mrows) continue;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int n = nbase + 32 * j + 8 * r4;
                if (n >= tc.ncols) continue;             // every width here is a multiple of 4
                const float v[4] = {acc[i][j][4 * r4], acc[i][j][4 * r4 + 1], acc[i][j][4 * r4 + 2],
                                    acc[i][j][4 * r4 + 3]};
                const int col = tc.n0 + n;
                const int row = tc.m0 + m;
                if (KIND == K_DX) {
                    *reinterpret_cast<u32x2*>(P.dXr + (size_t)(tc.row0 + row) * P.d + col) =
                        u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                } else if (KIND == K_DXR) {
                    f32x4 o = {v[0], v[1], v[2], v[3]};
                    if (!(P.flags & 1u)) {                // residual: dx gets dO itself
                        const u32x2 r = *reinterpret_cast<const u32x2*>(P.dO + (size_t)row * P.d + col);
                        o[0] += bf16_to_f32((bf16_t)(r.x & 0xffff));
                        o[1] += bf16_to_f32((bf16_t)(r.x >> 16));
                        o[2] += bf16_to_f32((bf16_t)(r.y & 0xffff));
                        o[3] += bf16_to_f32((bf16_t)(r.y >> 16));
                    }
                    *reinterpret_cast<f32x4*>(P.R32 + (size_t)row * P.d + col) = o;
                } else if (KIND == K_DW2) {
                    bf16_t* o = tc.shared ? P.dws2 + (size_t)sidx * P.d * P.Is : P.dw2 + (size_t)tc.g * P.d * P.I;
                    *reinterpret_cast<u32x2*>(o + (size_t)row * inter + col) =
                        u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                } else if (KIND == K_DW13) {
                    const bool up = row >= inter;
                    bf16_t* o = tc.shared ? (up ? P.dws3 : P.dws1) + (size_t)sidx * P.Is * P.d
                                          : (up ? P.dw3 : P.dw1) + (size_t)tc.g * P.I * P.d;
                    *reinterpret_cast<u32x2*>(o + (size_t)(up ? row - inter : row) * P.d + col) =
                        u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                } else {                                  // K_DC
                    *reinterpret_cast<f32x4*>(P.dC + (size_t)row * P.d + col) = f32x4{v[0], v[1], v[2], v[3]};
                }
            }
    }
}

// ---------------------------------------------------------------------------
// Work lists of the two products whose M runs over a group's rows (dH: N =
// the group's inter-dim; dX: N = d), in blocks of 4 M-tiles x all N-tiles
// (consecutive entries share A rows or weight rows), and the groups in
// descending row count (ties: lower id) for the weight-gradient products, so
// the longest reductions start first, with the groups no row chose spread
// among them (routed layers).  One workgroup.
// ---------------------------------------------------------------------------
constexpr int kListThreads = 1024;
constexpr int kMaxGroups = 256 + 16;

__device__ int scan_excl(int v, int* swave, int* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) swave[w] = x;
    __syncthreads();
    int base = 0, tot = 0;
    for (int i = 0; i < kListThreads / 64; ++i) {
        base += i < w ? swave[i] : 0;
        tot += swave[i];
    }
    __syncthreads();
    *total = tot;
    return base + x - v;
}

__device__ void emit_tiles(Tile* out, int total, const int* s_off, const int* s_cnt, int G, int E,
                           int ncols_r, int ncols_s) {
    for (int i = threadIdx.x; i < total; i += kListThreads) {
        int lo = 0, hi = G - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_off[mid] <= i) lo = mid;
            else hi = mid - 1;
        }
        const int g = lo, n = s_cnt[g];
        const int mt = (n + kBT - 1) / kBT;
        const int nt = ((g < E ? ncols_r : ncols_s) + kBT - 1) / kBT;
        const int j = i - s_off[g];
        const int b = j / (4 * nt);
        const int jj = j - b * 4 * nt;
        const int gm = min(4, mt - 4 * b);
        const int nn = jj / gm;
        const int m = 4 * b + (jj - nn * gm);
        Tile t;
        t.group = g;
        t.m0 = m * kBT;
        t.n0 = nn * kBT;
        t.nrows = min(kBT, n - m * kBT);
        out[i] = t;
    }
}

__global__ __launch_bounds__(kListThreads) void bwd_lists_kernel(const int32_t* goff, int E, int G,
                                                                 int I, int Is, int d, Tile* tdh,
                                                                 Tile* tdx, int32_t* ntiles,
                                                                 int32_t* gorder, int spread) {
    __shared__ int s_cnt[kMaxGroups], s_o1[kMaxGroups], s_o2[kMaxGroups], s_rows[kMaxGroups];
    __shared__ long long s_cum[kMaxGroups + 1];
    __shared__ int swave[kListThreads / 64];
    const int tid = threadIdx.x;
    int cnt = 0, t1 = 0, t2 = 0;
    if (tid < G) {
        cnt = goff[tid + 1] - goff[tid];
        const int mt = (cnt + kBT - 1) / kBT;
        t1 = mt * (((tid < E ? I : Is) + kBT - 1) / kBT);
        t2 = mt * ((d + kBT - 1) / kBT);
        s_cnt[tid] = cnt;
    }
    int tot1, tot2;
    const int o1 = scan_excl(t1, swave, &tot1);
    const int o2 = scan_excl(t2, swave, &tot2);
    if (tid < G) {
        s_o1[tid] = o1;
        s_o2[tid] = o2;
    }
    if (tid == 0) {
        ntiles[0] = tot1;
        ntiles[1] = tot2;
    }
    __syncthreads();
    // Groups with rows take ranks 0 .. nc - 1 (most rows first); the nz
    // empty ones (zero gradients: stores only) are spread among them in
    // proportion to the rows before them, so that their stores run while
    // other CUs still compute: empty group j goes right after the last group
    // whose rows start at or before (j + 1) / (nz + 1) of all rows.  Every
    // group with rows keeps its rank order, so the positions form a
    // bijection onto 0 .. G - 1.
    int rank = 0, nc = 0;
    if (tid < G) {
        for (int h = 0; h < G; ++h) {
            const int c = s_cnt[h];
            rank += (c > cnt) || (c == cnt && h < tid);
            nc += c > 0;
        }
        if (cnt > 0) s_rows[rank] = cnt;
    }
    __syncthreads();
    if (tid == 0) {                                     // rows before each rank
        long long a = 0;
        for (int i = 0; i < nc; ++i) {
            const long long v = s_rows[i];
            s_cum[i] = a;
            a += v;
        }
        s_cum[nc] = a;
    }
    __syncthreads();
    if (tid < G) {
        const int nz = G - nc;
        int pos = rank;
        if (spread && nc > 0 && nz > 0) {
            const long long total = s_cum[nc];
            if (cnt > 0) {                              // + empty groups placed before it
                const long long S = s_cum[rank] * (nz + 1);
                pos = rank + (int)(S == 0 ? 0 : min((long long)nz, (S - 1) / total));
            } else {
                const int j = rank - nc;
                const long long thr = ((long long)(j + 1) * total) / (nz + 1);
                int lo = 0, hi = nc - 1;                // last group starting at or before thr
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (s_cum[mid] <= thr) lo = mid;
                    else hi = mid - 1;
                }
                pos = lo + 1 + j;
            }
        }
        gorder[pos] = tid;
    }
    emit_tiles(tdh, tot1, s_o1, s_cnt, G, E, I, Is);
    emit_tiles(tdx, tot2, s_o2, s_cnt, G, E, d, d);
}

// ---------------------------------------------------------------------------
// Router backward, one wavefront per token (16 per workgroup): the gate
// gradients (the dH GEMM's per-tile partials summed in tile order), then
// gate -> score (renormalised: through the division by the kept scores'
// sum), plus the balance term alpha f_e / T on every score, then score ->
// affinity (softmax: s (ds - <s, ds>); sigmoid: s (1 - s) ds).  Lane l holds
// experts l + 64 j.  Writes dgate [T, K] (fp32) and dL [T, Epad] (bf16, the
// dx_router / dC GEMM operand; 0 past E).
// ---------------------------------------------------------------------------
constexpr int kRbWaves = 16;

__device__ __forceinline__ float wsum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__global__ __launch_bounds__(64 * kRbWaves) void router_bwd_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ idx, const float* __restrict__ gate,
    const int32_t* __restrict__ slot_of, const int32_t* __restrict__ goff, const float* __restrict__ dgp,
    int ndh, int nrt, float alpha, int T, int E, int Epad, int K, uint32_t flags,
    float* __restrict__ dgate, bf16_t* __restrict__ dL) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * kRbWaves + (threadIdx.x >> 6);
    if (t >= T) return;
    const bool sig = (flags & kGateSigmoid) != 0, ren = (flags & kGateRenorm) != 0;
    float sc[4], ds[4];
    const float bal = alpha * (float)E / ((float)K * (float)T * (float)T);   // alpha f_e / T per row of e
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
        sc[j] = e < Epad ? scores[(size_t)t * Epad + e] : 0.f;
        ds[j] = e < E ? bal * (float)(goff[e + 1] - goff[e]) : 0.f;
    }
    // gate gradients: lane k holds dg_k (k < 64), taken in dH tile order —
    // the nrt partials of a routed row (its N tiles over I; the row stride
    // ndh is the larger of the routed and shared counts, and a routed row's
    // entries past nrt are never written)
    float dgl[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int k = lane + 64 * j;
        if (k < K) {
            const float* pp = dgp + (size_t)slot_of[(size_t)t * K + k] * ndh;
            float a = 0.f;
            for (int n = 0; n < nrt; ++n) a += pp[n];
            dgl[j] = a;
            dgate[(size_t)t * K + k] = a;
        }
    }
    float sg = 0.f, z = 0.f;
    if (ren) {
        float ps = 0.f, pz = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k = lane + 64 * j;
            if (k < K) {
                ps += dgl[j] * gate[(size_t)t * K + k];
                pz += scores[(size_t)t * Epad + idx[(size_t)t * K + k]];
            }
        }
        sg = wsum(ps);
        z = wsum(pz);
    }
    // scatter d score of the kept experts to their lanes, in k order
    for (int k = 0; k < K; ++k) {
        const float dg = __shfl(dgl[k >> 6], k & 63, 64);
        const int e = idx[(size_t)t * K + k];
        const float v = ren ? (dg - sg) / z : dg;
        if ((e & 63) == lane) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (j == (e >> 6)) ds[j] += v;
        }
    }
    float dl[4];
    if (sig) {
#pragma unroll
        for (int j = 0; j < 4; ++j) dl[j] = sc[j] * (1.f - sc[j]) * ds[j];
    } else {
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) m += sc[j] * ds[j];
        m = wsum(m);
#pragma unroll
        for (int j = 0; j < 4; ++j) dl[j] = sc[j] * (ds[j] - m);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
        if (e < Epad) dL[(size_t)t * Epad + e] = f32_to_bf16(e < E ? dl[j] : 0.f);
    }
}

// ---------------------------------------------------------------------------
// dx[t] = R32[t] (or dO[t] / 0 without a router) + the token's shared-expert
// rows + its K routed rows of dX, in that fixed order, fp32, one RNE
// rounding.  One workgroup per token, 8 columns per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dx_combine_kernel(const float* __restrict__ R32,
                                                         const bf16_t* __restrict__ dO,
                                                         const bf16_t* __restrict__ dXr,
                                                         const int32_t* __restrict__ slot_of, int T,
                                                         int d, int K, int Ks, uint32_t flags,
                                                         bf16_t* __restrict__ dx) {
    const int t = blockIdx.x;
    const int TK = T * K;
    for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
        float a[8];
        if (R32) {
            const f32x4 u = *reinterpret_cast<const f32x4*>(R32 + (size_t)t * d + c);
            const f32x4 v = *reinterpret_cast<const f32x4*>(R32 + (size_t)t * d + c + 4);
            for (int e = 0; e < 4; ++e) {
                a[e] = u[e];
                a[4 + e] = v[e];
            }
        } else if (!(flags & 1u)) {
            const u32x4 r = *reinterpret_cast<const u32x4*>(dO + (size_t)t * d + c);
            for (int e = 0; e < 4; ++e) {
                a[2 * e] = bf16_to_f32((bf16_t)(r[e] & 0xffff));
                a[2 * e + 1] = bf16_to_f32((bf16_t)(r[e] >> 16));
            }
        } else {
            for (int e = 0; e < 8; ++e) a[e] = 0.f;
        }
        auto add_row = [&](size_t row) {
            const u32x4 r = *reinterpret_cast<const u32x4*>(dXr + row * d + c);
            for (int e = 0; e < 4; ++e) {
                a[2 * e] += bf16_to_f32((bf16_t)(r[e] & 0xffff));
                a[2 * e + 1] += bf16_to_f32((bf16_t)(r[e] >> 16));
            }
        };
        for (int s = 0; s < Ks; ++s) add_row((size_t)TK + (size_t)s * T + t);
        for (int k = 0; k < K; ++k) add_row((size_t)slot_of[(size_t)t * K + k]);
        u32x4 o;
        for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(a[2 * e], a[2 * e + 1]);
        *reinterpret_cast<u32x4*>(dx + (size_t)t * d + c) = o;
    }
}

// ---------------------------------------------------------------------------
// Balance statistics of a training forward ("DeepSeekMoE 深度解读报告",
// sections 2.5 / 3.2): per expert the hit rate f_e = E n_e / (K T) and the
// mean score P_e = (1/T) sum_t s_{t,e}, and L_bal = sum_e f_e P_e.  The
// score sums come per 16-token workgroup of the router and are added in
// order; L_bal sums experts in order.  One workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void balance_stats_kernel(const int32_t* goff, const float* score_part,
                                                           int nparts, int E, int Epad, int K, int T,
                                                           float* stats) {
    __shared__ float sl[256];
    const int e = threadIdx.x;
    float l = 0.f;
    if (e < E) {
        float ps = 0.f;
        for (int p = 0; p < nparts; ++p) ps += score_part[(size_t)p * Epad + e];
        const float P = ps / (float)T;
        const float f = (float)E * (float)(goff[e + 1] - goff[e]) / ((float)K * (float)T);
        stats[e] = f;
        stats[E + e] = P;
        l = f * P;
    }
    sl[e] = l;
    __syncthreads();
    if (e == 0) {
        float tot = 0.f;
        for (int i = 0; i < E; ++i) tot += sl[i];
        stats[2 * E] = tot;
    }
}

}  // namespace

hipError_t launch_balance_stats(const Plan& p, float* stats, hipStream_t st) {
    balance_stats_kernel<<<1, 256, 0, st>>>(p.goff, p.score_part, p.nchunk * 4, p.E, p.Epad, p.K,
                                            p.T, stats);
    return hipGetLastError();
}

hipError_t launch_backward(const Plan& p, const BwdPlan& b, const BwdArgs& a, hipStream_t st,
                           void (*mark)(int slot, int end, hipStream_t s)) {
    BwdParams P{};
    P.goff = p.goff;
    P.tok_of = p.tok_of;
    P.E = p.E;
    P.Ks = p.Ks;
    P.T = p.T;
    P.K = p.K;
    P.d = p.d;
    P.I = p.I;
    P.Is = p.Is;
    P.Epad = p.Epad;
    P.flags = p.flags;
    P.x = a.x;
    P.dO = a.dout;
    P.C = a.C;
    P.w1 = a.w1;
    P.w3 = a.w3;
    P.w2 = a.w2;
    P.ws1 = a.ws1;
    P.ws3 = a.ws3;
    P.ws2 = a.ws2;
    P.Z = p.Z;
    P.H = p.H;
    P.row_gate = p.row_gate;
    P.dZ = b.dZ;
    P.gH = b.gH;
    P.dgp = b.dgp;
    P.dL = b.dL;
    P.R32 = b.R32;
    P.dXr = b.dXr;
    P.dw1 = a.dw1;
    P.dw3 = a.dw3;
    P.dw2 = a.dw2;
    P.dws1 = a.dws1;
    P.dws3 = a.dws3;
    P.dws2 = a.dws2;
    P.dC = a.dC;
    P.gorder = b.gorder;
    hipError_t e = hipSuccess;
    auto step = [&](int slot, auto&& launch) {
        if (e != hipSuccess) return;
        mark(slot, 0, st);
        launch();
        e = hipGetLastError();
        mark(slot, 1, st);
    };
    const int G = p.E + p.Ks;
    const bool routed = p.K > 0;
    float* dgate = a.dgate ? a.dgate : b.dgate;
    step(0, [&] {
        bwd_lists_kernel<<<1, kListThreads, 0, st>>>(p.goff, p.E, G, p.I, p.Is, p.d, b.tiles_dh,
                                                     b.tiles_dx, b.ntiles, b.gorder, routed ? 1 : 0);
    });
    P.tiles = b.tiles_dh;
    P.ntiles = b.ntiles;
    step(1, [&] { bwd_gemm_kernel<K_DH><<<b.max_tiles_dh, 64 * kNW, 0, st>>>(P); });
    if (routed) {
        step(2, [&] {
            router_bwd_kernel<<<(p.T + kRbWaves - 1) / kRbWaves, 64 * kRbWaves, 0, st>>>(
                p.scores, p.idx, p.gate, p.slot_of, p.goff, b.dgp, b.ndh, (p.I + kBT - 1) / kBT, a.alpha,
                p.T, p.E, p.Epad,
                p.K, p.flags, dgate, b.dL);
        });
        const int g3 = ((p.T + kBT - 1) / kBT) * ((p.d + kBT - 1) / kBT);
        step(3, [&] { bwd_gemm_kernel<K_DXR><<<g3, 64 * kNW, 0, st>>>(P); });
    }
    P.tiles = b.tiles_dx;
    P.ntiles = b.ntiles + 1;
    step(4, [&] { bwd_gemm_kernel<K_DX><<<b.max_tiles_dx, 64 * kNW, 0, st>>>(P); });
    step(5, [&] {
        dx_combine_kernel<<<p.T, 256, 0, st>>>(routed ? b.R32 : nullptr, a.dout, b.dXr, p.slot_of, p.T,
                                               p.d, p.K, p.Ks, p.flags, a.dx);
    });
    // weight gradients: without a router only the shared groups (every
    // routed group is empty then, so they sort last)
    P.ngt = routed ? G : p.Ks;
    const int imax = p.I > p.Is ? p.I : p.Is;
    const int g6 = P.ngt * ((p.d + kBT - 1) / kBT) * ((imax + kBT - 1) / kBT);
    step(6, [&] { bwd_gemm_kernel<K_DW2><<<g6, 64 * kNW, 0, st>>>(P); });
    const int g7 = P.ngt * ((2 * imax + kBT - 1) / kBT) * ((p.d + kBT - 1) / kBT);
    step(7, [&] { bwd_gemm_kernel<K_DW13><<<g7, 64 * kNW, 0, st>>>(P); });
    if (routed) {
        const int g8 = ((p.Epad + kBT - 1) / kBT) * ((p.d + kBT - 1) / kBT);
        step(8, [&] { bwd_gemm_kernel<K_DC><<<g8, 64 * kNW, 0, st>>>(P); });
    }
    return e;
}

}  // namespace moe
