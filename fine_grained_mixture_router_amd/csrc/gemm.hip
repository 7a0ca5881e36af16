// Grouped expert GEMMs on bf16 MFMA (gfx950), fp32 accumulation.
//
//   G1 (gate/up):  H[r,:] = silu(X[tok(r)] . W1_g^T) * (X[tok(r)] . W3_g^T)
//   G2 (down):     Y[r,:] = H[r,:] . W2_g^T
//
// for every row r of group g (a routed expert or a shared expert) — the
// Expert module w2(silu(w1 x) * w3 x) of the youleyou page, applied to the
// rows the permutation grouped per expert.  W1 and W3 share one pass: a tile
// holds matching rows of both, so each wave owns the w1 and w3 accumulators
// of the same outputs and applies silu(a)*b in registers before the single
// bf16 store (the gather-in-mainloop and activation-in-epilogue ideas the
// SonicMoE note describes, re-done for CDNA4).
//
// One kernel template serves both: a work-list entry (group, m0, n0, nrows)
// names the tile; A rows are gathered through tok_of (G1) or read in place
// (G2).  Tiles are BM x BN with BK = 64, staged through LDS in XOR-swizzled
// 16-byte chunks (a double buffer in the few-rows tile, a ring of five
// operand slots in the many-rows tile) and consumed by
// v_mfma_f32_32x32x16_bf16.
// The grid is the work-list bound; workgroups past the device-side count
// exit at once.  Workgroup ids are dealt round-robin over the 8 XCDs; the
// many-rows kernels (and the 8-bit few-rows one) remap them so that each
// XCD takes runs of consecutive work-list tiles, whose A rows and weight
// rows its L2 then shares.
#include "common.h"

#include <type_traits>

// Phase timestamps (built only with -DMOE_PHASE_STAMPS, by
// `build.py --phase`; the library itself carries none of this): per
// workgroup of the many-rows GEMM tiles, the shader clock (s_memtime) at the
// tile's start, after its first slice has landed, after its main loop and
// after its epilogue's stores have been issued, and the hardware id of the
// wave.  Four regions of kPhaseWgs workgroups: bf16 gate/up, bf16 down, FP8
// gate/up, FP8 down; a later launch of the same kind overwrites.
#ifdef MOE_PHASE_STAMPS
constexpr int kPhaseWgs = 32768;
__device__ unsigned long long g_phase[4 * kPhaseWgs * 5];
extern "C" __attribute__((visibility("default"))) int moe_phase_read(unsigned long long* host, int n) {
    if (n < 0 || n > 4 * kPhaseWgs * 5) return 1;
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_phase), (size_t)n * 8, 0, hipMemcpyDeviceToHost);
}
extern "C" __attribute__((visibility("default"))) int moe_phase_slots() { return 4 * kPhaseWgs * 5; }
#define PHASE_STAMP(kind, k)                                                                   \
    do {                                                                                       \
        if (threadIdx.x == 0 && blockIdx.x < (unsigned)kPhaseWgs) {                            \
            const size_t at_ = ((size_t)(kind) * kPhaseWgs + blockIdx.x) * 5;                  \
            g_phase[at_ + (k)] = __builtin_amdgcn_s_memtime();                                 \
            if ((k) == 0) {                                                                    \
                unsigned hw_;                                                                  \
                asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw_));              \
                g_phase[at_ + 4] = hw_;                                                        \
            }                                                                                  \
        }                                                                                      \
    } while (0)
#else
#define PHASE_STAMP(kind, k) \
    do {                     \
    } while (0)
#endif

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;
// Runs of consecutive work-list tiles per XCD (see fetch_tile).
constexpr int kXcdChunk = 16;


__device__ __forceinline__ int swz(int row, int chunk) {
    return row * kBK + ((chunk ^ (row & 7)) << 3);
}

struct GemmParams {
    const Tile* tiles;
    const int32_t* ntiles;
    const int32_t* goff;
    const int32_t* tok_of;   // G1 only
    const bf16_t* A_r;       // routed A base (G1: x, G2: H routed)
    const bf16_t* A_s;       // shared A base (G1: x, G2: H shared)
    const bf16_t* Ba_r;      // routed weights (G1: W1, G2: W2)
    const bf16_t* Bb_r;      // routed W3 (G1 only)
    const bf16_t* Ba_s;      // shared weights
    const bf16_t* Bb_s;
    const uint8_t* Qa_r;     // 8-bit routed weights (G1: W1, G2: W2), or null
    const uint8_t* Qb_r;     // 8-bit routed W3 (G1 only)
    const float* Sa_r;       // their per-row scales [E, n_r]
    const float* Sb_r;
    const uint8_t* Xq;       // 8-bit activations: codes of the routed A rows (G1: x [T, d],
                             //   G2: h [T*K, I]), or null
    const int32_t* Xe;       //   their per-row scale exponents
    bf16_t* O_r;             // routed output base (G1: H routed, G2: Y)
    bf16_t* O_s;             // shared output base (G1: H shared, G2: Y)
    bf16_t* Z_r;             // G1 of a training forward: pre-activations [W1 x | W3 x]
    bf16_t* Z_s;             //   of routed / shared rows (null otherwise)
    int kdim_r, kdim_s;      // reduction length
    int n_r, n_s;            // output columns
    int E, TK;               // routed experts, routed rows (T*K)
    uint32_t abytes_r, abytes_s;  // sizes of the A regions in bytes
};

// silu(a) = a / (1 + e^-a), the reciprocal from the hardware's v_rcp_f32
// (1 ulp), far below the bf16 rounding of the output: a full IEEE division
// made the SwiGLU epilogue of a 256 x 256 tile about 4 % of its time.
__device__ __forceinline__ float silu(float a) { return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }

// Two packed bf16 from the two 8-bit E4M3 codes in the low (HI = false) or
// high (HI = true) half of `w`, the lower byte in the lower half.  Every
// E4M3 value is exact in bf16; the scale operand 1.0 leaves it unscaled.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, v);
}

// BM x BN tile, WM x WN waves.  SWIGLU: the BN B-rows are BN/2 rows of W1
// followed by the same BN/2 rows of W3, and the output has BN/2 columns.
//
// bf16 weights: each BK slice is loaded into registers two iterations ahead
// (two register sets), stored to the LDS double buffer, and multiplied.
//
// Q8: the tile's weights are 8-bit E4M3 codes with one float scale per
// weight row (a routed expert's matrices in moe_forward_fp8).  Codes are
// loaded a slice pair at a time — 128 codes, one whole 128-byte line, per
// row — so that they can stream with the nontemporal policy; they stay
// 8-bit in LDS and are widened exactly to bf16 after each fragment read.
// The scale multiplies the fp32 accumulator of its output column in the
// epilogue (the scale is per output channel, so it factors out of the
// reduction).
template <int BM, int BN, int WM, int WN, bool SWIGLU, bool Q8>
__device__ __forceinline__ void thin_tile(const GemmParams& P, const Tile& tl, bf16_t* sA,
                                          bf16_t* sB) {
    static_assert(WM * WN == 4, "four waves");
    constexpr int WROWS = BM / WM;                 // rows per wave
    constexpr int WCOLS = BN / WN;                 // B-rows per wave
    constexpr int MB = WROWS / 32;
    constexpr int NB = WCOLS / 32;
    static_assert(MB >= 1 && NB >= 1 && (!SWIGLU || NB % 2 == 0), "tile shape");
    constexpr int AL = BM / 32;                    // A chunks per thread per slice
    constexpr int BL = BN / 32;                    // B chunks per thread per slice (bf16) or pair (8-bit)
    static_assert(!Q8 || AL == 1, "the 8-bit path loads one A chunk per thread per slice");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    const bool shared = tl.group >= P.E;
    const int s = tl.group - P.E;
    const int kdim = shared ? P.kdim_s : P.kdim_r;
    const int ncols = shared ? P.n_s : P.n_r;
    const int grow = P.goff[tl.group] + tl.m0;      // first global row of the tile
    const int rrow = shared ? grow - P.TK : grow;   // first row within its region

    // Raw buffer loads: resource (base, size) in scalar registers, a 32-bit
    // byte offset per lane, the k position in the scalar offset.  Rows past
    // the tile's end are clamped to its first row and weight rows past the
    // output width to the last one, so every access stays inside its tensor
    // (those rows are never stored); loads past a resource's end return 0.
    const int ch = tid & 7;
    const __amdgpu_buffer_rsrc_t ra_src =
        make_rsrc(shared ? P.A_s : P.A_r, shared ? P.abytes_s : P.abytes_r);
    constexpr uint32_t WB = Q8 ? 1u : 2u;          // bytes per weight
    const uint32_t wbytes = (uint32_t)ncols * (uint32_t)kdim * WB;
    const size_t wofs = (size_t)(shared ? s : tl.group) * ncols * kdim;
    const void* wa;
    const void* wb;
    if (Q8) {
        wa = P.Qa_r + wofs;
        wb = SWIGLU ? P.Qb_r + wofs : wa;
    } else {
        wa = (shared ? P.Ba_s : P.Ba_r) + wofs;
        wb = SWIGLU ? (shared ? P.Bb_s : P.Bb_r) + wofs : wa;
    }
    const __amdgpu_buffer_rsrc_t rw1 = make_rsrc(wa, wbytes);
    const __amdgpu_buffer_rsrc_t rw3 = make_rsrc(wb, wbytes);
    uint32_t aoff[AL];
    uint32_t boff[BL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
        const int r = (tid >> 3) + 32 * i;
        const int rr = r < tl.nrows ? r : 0;
        uint32_t arow;
        if (SWIGLU) arow = (uint32_t)P.tok_of[grow + rr];
        else arow = (uint32_t)(rrow + rr);
        aoff[i] = (arow * (uint32_t)kdim + ch * 8) * 2u;
    }
    // B: thread moves 16-byte piece ch of rows (tid >> 3) + 32 i — for bf16
    // the 8 weights 8 ch .. 8 ch + 7 of a slice, for 8-bit the 16 codes
    // 16 ch .. 16 ch + 15 of a slice pair (slice 2p when ch < 4, else 2p+1).
    // i < BL/2 <=> the row is in the W1 half.
#pragma unroll
    for (int i = 0; i < BL; ++i) {
        const int r = (tid >> 3) + 32 * i;
        int n = tl.n0 + ((SWIGLU && r >= BN / 2) ? r - BN / 2 : r);
        n = n < ncols ? n : ncols - 1;
        boff[i] = Q8 ? (uint32_t)n * (uint32_t)kdim + ch * 16u : ((uint32_t)n * (uint32_t)kdim + ch * 8) * 2u;
    }

    f32x16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f32x16{};

    // LDS addressing.  Every row index used below is (multiple of 8) + the
    // lane's own (lane & 7) or (tid >> 3) & 7, so the swizzled chunk
    // position of a lane is fixed per k16 step and the rest is a
    // compile-time or wave-uniform row offset.
    const int srow = tid >> 3;
    const int sx = (ch ^ (srow & 7)) << 3;
    bf16_t* const a_st = sA + srow * kBK + sx;
    bf16_t* const b_st = sB + srow * kBK + sx;
    const int lrow = lane & 31;
    int cx[kBK / 16];
#pragma unroll
    for (int st = 0; st < kBK / 16; ++st) cx[st] = ((2 * st + (lane >> 5)) ^ (lane & 7)) << 3;
    const bf16_t* const a_ld = sA + (wm * WROWS + lrow) * kBK;
    const bf16_t* const b_ld = sB + lrow * kBK;

    auto compute = [&](int buf) {
        const bf16_t* a_b = a_ld + buf * (BM * kBK);
        const bf16_t* b_b = b_ld + buf * (BN * kBK);
#pragma unroll
        for (int st = 0; st < kBK / 16; ++st) {
            bf16x8 af[MB], bfr[NB];
#pragma unroll
            for (int i = 0; i < MB; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(a_b + i * 32 * kBK + cx[st]);
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                int bro;
                if (SWIGLU) {
                    constexpr int half = NB / 2;
                    bro = (j < half ? 0 : BN / 2) + wn * (WCOLS / 2) + (j < half ? j : j - half) * 32;
                } else {
                    bro = wn * WCOLS + j * 32;
                }
                bfr[j] = *reinterpret_cast<const bf16x8*>(b_b + bro * kBK + cx[st]);
            }
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    };
    // Barrier after this wave's LDS stores, without __syncthreads()'s wait
    // for every outstanding global load (which would drain the prefetch).
    auto bar = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
    auto store_a = [&](int buf, const u32x4 (&ra)[AL]) {
#pragma unroll
        for (int i = 0; i < AL; ++i) *reinterpret_cast<u32x4*>(a_st + buf * (BM * kBK) + 32 * i * kBK) = ra[i];
    };
    const int nk = kdim / kBK;

    if constexpr (!Q8) {
        // Two register sets: iteration kt loads slice kt + 2 into the free
        // set, multiplies slice kt out of LDS and stores slice kt + 1 (loaded
        // one iteration earlier) to the other LDS buffer — two iterations of
        // MFMA work hide each load's latency.
        u32x4 ra0[AL], rb0[BL], ra1[AL], rb1[BL];
        auto gload = [&](int kt, u32x4 (&ra)[AL], u32x4 (&rb)[BL]) {
            const uint32_t kb = (uint32_t)kt * kBK * 2u;
#pragma unroll
            for (int i = 0; i < AL; ++i) ra[i] = buf_load16(ra_src, aoff[i], kb);
#pragma unroll
            for (int i = 0; i < BL; ++i)            // weights: read once, streamed
                rb[i] = buf_load16_nt((SWIGLU && i >= BL / 2) ? rw3 : rw1, boff[i], kb);
        };
        auto sstore = [&](int buf, const u32x4 (&ra)[AL], const u32x4 (&rb)[BL]) {
            store_a(buf, ra);
#pragma unroll
            for (int i = 0; i < BL; ++i)
                *reinterpret_cast<u32x4*>(b_st + buf * (BN * kBK) + 32 * i * kBK) = rb[i];
        };
        auto iter = [&](int kt, bool load, bool store, u32x4 (&ca)[AL], u32x4 (&cb)[BL],
                        u32x4 (&na)[AL], u32x4 (&nb)[BL]) {
            if (load) gload(kt + 2, ca, cb);
            __builtin_amdgcn_sched_barrier(0);       // the prefetch leaves before the MFMAs
            compute(kt & 1);
            if (store) sstore((kt + 1) & 1, na, nb);
            bar();
        };
        gload(0, ra0, rb0);
        if (nk > 1) gload(1, ra1, rb1);
        sstore(0, ra0, rb0);
        bar();
        // Steady state, two iterations at a time (the register sets swap
        // roles): every iteration loads and stores, so the loop body has no
        // branch and each wait covers just the older slice.  The last one to
        // three iterations run in the tail.
        int kt = 0;
        for (; kt + 3 < nk; kt += 2) {
            iter(kt, true, true, ra0, rb0, ra1, rb1);
            iter(kt + 1, true, true, ra1, rb1, ra0, rb0);
        }
        if (kt < nk) {
            iter(kt, kt + 2 < nk, kt + 1 < nk, ra0, rb0, ra1, rb1);
            if (kt + 1 < nk) {
                iter(kt + 1, kt + 3 < nk, kt + 2 < nk, ra1, rb1, ra0, rb0);
                if (kt + 2 < nk) iter(kt + 2, false, false, ra0, rb0, ra1, rb1);
            }
        }
    } else {
        // Slice pairs: an iteration covers 128 k.  Register set p & 1 holds
        // pair p — its codes (one whole 128-byte line per weight row,
        // streamed) and the two 128-byte A pieces of each row — and goes to
        // the LDS buffer p & 1 as is: codes stay 8-bit in LDS and are widened
        // after the fragment read, so a pair costs one barrier, half the LDS
        // traffic of widened weights, and widening work for every lane.
        //
        // k order of a pair: in k16 step t (0..7) lanes 0-31 take the pair's
        // k 8t .. 8t+7 and lanes 32-63 take k 64 + 8t .. 64 + 8t + 7, for the
        // activations and the codes alike (the products pair up as in any
        // order).  One 16-byte code read then serves steps 2u and 2u + 1,
        // and an activation read is one 16-byte chunk of the row.
        //
        // LDS: A rows of 256 bytes (the pair's 128 bf16), chunk c at c ^
        // (row & 15); code rows of 128 bytes, chunk c at c ^ ((row >> 1) & 7).
        // Either way the 16 lanes of one LDS service group read 16 rows at
        // one logical chunk and hit 16 distinct bank groups.
        static_assert(MB == 1, "one 32-row activation block per wave");
        constexpr int QAB = BM * 256;                // bytes of one A buffer
        constexpr int QBB = BN * 128;                // bytes of one code buffer
        uint8_t* const qa_lds = reinterpret_cast<uint8_t*>(sA);
        uint8_t* const qb_lds = reinterpret_cast<uint8_t*>(sB);
        const int np = (nk + 1) / 2;                 // an odd nk leaves the last pair half-used
        u32x4 qa0[2], qb0[BL], qa1[2], qb1[BL];
        auto gload = [&](int p, u32x4 (&qa)[2], u32x4 (&qb)[BL]) {
            const uint32_t kb = (uint32_t)p * (2 * kBK * 2u);   // A: bytes of two bf16 slices
            qa[0] = buf_load16(ra_src, aoff[0], kb);
            qa[1] = buf_load16(ra_src, aoff[0], kb + kBK * 2u);
#pragma unroll
            for (int i = 0; i < BL; ++i)            // codes: whole 128-byte lines, streamed
                qb[i] = buf_load16_nt((SWIGLU && i >= BL / 2) ? rw3 : rw1, boff[i], kb / 2);
        };
        // thread (row srow + 32 i, piece ch): A chunks ch and 8 + ch, code chunk ch
        const int qa_st0 = srow * 256 + ((ch ^ (srow & 15)) << 4);
        const int qa_st1 = srow * 256 + (((8 + ch) ^ (srow & 15)) << 4);
        auto sstore = [&](int buf, const u32x4 (&qa)[2], const u32x4 (&qb)[BL]) {
            *reinterpret_cast<u32x4*>(qa_lds + buf * QAB + qa_st0) = qa[0];
            *reinterpret_cast<u32x4*>(qa_lds + buf * QAB + qa_st1) = qa[1];
#pragma unroll
            for (int i = 0; i < BL; ++i) {
                const int r = srow + 32 * i;
                *reinterpret_cast<u32x4*>(qb_lds + buf * QBB + r * 128 + ((ch ^ ((r >> 1) & 7)) << 4)) = qb[i];
            }
        };
        // fragment addressing: lane (row lrow, half h)
        const int h = lane >> 5;
        int qbrow[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            int bro;
            if (SWIGLU) {
                constexpr int half = NB / 2;
                bro = (j < half ? 0 : BN / 2) + wn * (WCOLS / 2) + (j < half ? j : j - half) * 32;
            } else {
                bro = wn * WCOLS + j * 32;
            }
            qbrow[j] = (bro + lrow) * 128;
        }
        const int qaro = lrow * 256;
        auto compute_q = [&](int buf, bool half_pair) {
            const uint8_t* ab = qa_lds + buf * QAB + qaro;
            const uint8_t* bb = qb_lds + buf * QBB;
            // the second 64 k of a half-used pair lie past the row: lanes
            // 32-63 multiply zeros there
            const bool zero_hi = half_pair && h;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c0 = 8 * h + 2 * u;        // A chunks of steps 2u, 2u + 1
                const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(ab + ((c0 ^ (lrow & 15)) << 4));
                const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(ab + (((c0 + 1) ^ (lrow & 15)) << 4));
                bf16x8 b0[NB], b1[NB];
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int r = (qbrow[j] >> 7);
                    const u32x4 w = *reinterpret_cast<const u32x4*>(bb + qbrow[j] + (((4 * h + u) ^ ((r >> 1) & 7)) << 4));
                    u32x4 lo = {e4m3x2_to_bf16x2<false>(w.x), e4m3x2_to_bf16x2<true>(w.x),
                                e4m3x2_to_bf16x2<false>(w.y), e4m3x2_to_bf16x2<true>(w.y)};
                    u32x4 hi = {e4m3x2_to_bf16x2<false>(w.z), e4m3x2_to_bf16x2<true>(w.z),
                                e4m3x2_to_bf16x2<false>(w.w), e4m3x2_to_bf16x2<true>(w.w)};
                    if (zero_hi) lo = hi = u32x4{0u, 0u, 0u, 0u};
                    b0[j] = __builtin_bit_cast(bf16x8, lo);
                    b1[j] = __builtin_bit_cast(bf16x8, hi);
                }
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[0][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0[j], acc[0][j], 0, 0, 0);
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[0][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1[j], acc[0][j], 0, 0, 0);
            }
        };
        // Iteration p: load pair p + 2 into the free register set, multiply
        // pair p out of LDS, store pair p + 1 (loaded an iteration earlier)
        // to the other buffer — as the bf16 path does with slices.
        auto iter = [&](int p, bool load, bool store, u32x4 (&ca)[2], u32x4 (&cb)[BL],
                        u32x4 (&na)[2], u32x4 (&nb)[BL]) {
            if (load) gload(p + 2, ca, cb);
            __builtin_amdgcn_sched_barrier(0);       // the prefetch leaves before the MFMAs
            compute_q(p & 1, 2 * p + 1 == nk);
            if (store) sstore((p + 1) & 1, na, nb);
            bar();
        };
        gload(0, qa0, qb0);
        if (np > 1) gload(1, qa1, qb1);
        sstore(0, qa0, qb0);
        bar();
        int p = 0;
        for (; p + 3 < np; p += 2) {                 // steady state: no branch, constant waits
            iter(p, true, true, qa0, qb0, qa1, qb1);
            iter(p + 1, true, true, qa1, qb1, qa0, qb0);
        }
        if (p < np) {
            iter(p, p + 2 < np, p + 1 < np, qa0, qb0, qa1, qb1);
            if (p + 1 < np) {
                iter(p + 1, p + 3 < np, p + 2 < np, qa1, qb1, qa0, qb0);
                if (p + 2 < np) iter(p + 2, false, false, qa0, qb0, qa1, qb1);
            }
        }
    }

    // Epilogue.  32x32 accumulator layout: lane holds column (lane & 31) and
    // rows 8*(r/4) + 4*(lane/32) + (r%4), r = 0..15.  The outputs go through
    // LDS (free: every wave passed the main loop's last barrier after its
    // last fragment read) and leave as whole 16-byte pieces of each row.
    // Stored straight from the accumulators, each store instruction wrote
    // 2-byte values to two 64-byte row pieces; on the decode down GEMM those
    // stores cost 8 % of its time (measured without them).
    bf16_t* obase = shared ? P.O_s : P.O_r;
    const int orow0 = SWIGLU ? rrow : grow;
    const float* sca = Q8 ? P.Sa_r + (size_t)tl.group * ncols : nullptr;
    const float* scb = Q8 && SWIGLU ? P.Sb_r + (size_t)tl.group * ncols : nullptr;
    constexpr int OC = SWIGLU ? BN / 2 : BN;       // output columns of the tile
    static_assert(BM * OC <= 2 * BN * kBK, "the output tile fits the B buffers");
    bf16_t* const stage = sB;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
#pragma unroll
        for (int j = 0; j < (SWIGLU ? NB / 2 : NB); ++j) {
            const int lcol = (SWIGLU ? wn * (WCOLS / 2) : wn * WCOLS) + j * 32 + (lane & 31);
            const int col = tl.n0 + lcol;
            float fa = 1.f, fb = 1.f;
            if (Q8 && col < ncols) {
                fa = sca[col];
                if (SWIGLU) fb = scb[col];
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * WROWS + i * 32 + ((r >> 2) << 3) + ((lane >> 5) << 2) + (r & 3);
                float v;
                if (SWIGLU) v = silu(Q8 ? acc[i][j][r] * fa : acc[i][j][r]) *
                                (Q8 ? acc[i][j + NB / 2][r] * fb : acc[i][j + NB / 2][r]);
                else v = Q8 ? acc[i][j][r] * fa : acc[i][j][r];
                stage[row * OC + lcol] = f32_to_bf16(v);
                if (SWIGLU && !Q8 && P.Z_r && row < tl.nrows && col < ncols) {
                    bf16_t* z = (shared ? P.Z_s : P.Z_r) + (size_t)(orow0 + row) * 2 * ncols + col;
                    z[0] = f32_to_bf16(acc[i][j][r]);
                    z[ncols] = f32_to_bf16(acc[i][j + NB / 2][r]);
                }
            }
        }
    }
    bar();
    for (int idx = tid; idx < BM * (OC / 8); idx += kThreads) {
        const int row = idx / (OC / 8);
        const int c = idx - row * (OC / 8);
        const int col = tl.n0 + c * 8;                // ncols is a multiple of 8: whole pieces
        if (row < tl.nrows && col < ncols)                // streaming stores: 4 % faster decode down
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(stage + row * OC + c * 8),
                                        reinterpret_cast<u32x4*>(obase + (size_t)(orow0 + row) * ncols + col));
    }
}

// Few-rows-per-expert tiles.  Q8: routed experts' weights are 8-bit codes
// with per-row scales; shared experts' tiles always take the bf16 path.
template <int BM, int BN, int WM, int WN, bool SWIGLU, bool Q8>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(GemmParams P) {
    // the 8-bit path's A buffers hold slice pairs (twice the bf16 slice)
    __shared__ __attribute__((aligned(16))) bf16_t sA[2 * BM * kBK * (Q8 ? 2 : 1)];
    __shared__ __attribute__((aligned(16))) bf16_t sB[2 * BN * kBK];

    // Workgroup ids are dealt round-robin over the 8 XCDs.  bf16 weights:
    // XCD x takes the x-th contiguous eighth of the work list (every tile
    // streams the same bytes; measured 1-3 % faster than dealing runs).
    // 8-bit weights: the shared-expert tiles (bf16, twice a routed tile's
    // bytes; listed last) would all fall in the last XCD's eighth and
    // finish last, so runs of kXcdChunk tiles are dealt to the XCDs in turn
    // and the list is taken from its end: the shared tiles go first, spread
    // over the XCDs, and the last tiles to run are short ones.
    const int nt = *P.ntiles;
    const int wg = blockIdx.x;
    int lt;
    if (!Q8) {
        const int nr = (nt + 7) & ~7;
        if (wg >= nr) return;
        lt = (wg & 7) * (nr >> 3) + (wg >> 3);
        if (lt >= nt) return;
    } else {
        const int nr = (nt + 8 * kXcdChunk - 1) / (8 * kXcdChunk) * (8 * kXcdChunk);
        if (wg >= nr) return;
        const int jx = wg >> 3;
        const int lt0 = (jx / kXcdChunk) * (8 * kXcdChunk) + (wg & 7) * kXcdChunk + jx % kXcdChunk;
        if (lt0 >= nt) return;
        lt = nt - 1 - lt0;
    }
    const Tile tl = P.tiles[lt];
    if (Q8 && tl.group < P.E) thin_tile<BM, BN, WM, WN, SWIGLU, true>(P, tl, sA, sB);
    else thin_tile<BM, BN, WM, WN, SWIGLU, false>(P, tl, sA, sB);
}

// ---------------------------------------------------------------------------
// 256 x 256 tile for many rows per expert (MFMA-bound).  Eight waves, two
// per SIMD, each 128 rows x 64 B-rows (4 x 2 blocks of 32x32x16 MFMAs, 128
// fp32 accumulators per lane: with two waves per SIMD that is the register
// budget, which is what bounds the tile).
//
// Global -> LDS with direct-to-LDS buffer loads: one wave instruction moves
// 1 KB = (1024 / row bytes) rows of one BK slice into LDS, lane l filling
// the 16-byte position l, so staging costs no VGPRs and no ds_write.  The
// vector-memory path moves about 31 B/clk/CU when each row segment is 64
// bytes, 43 with 128-byte segments and 72 for 1 KB contiguous (measured on
// MI355X with L2-resident data), and this tile needs about 22 B/clk/CU at
// 1.5 PFLOP/s — so the slice width BK = 64 (128-byte segments) is kept and
// the load latency is hidden by a ring of operand slots (big_tile).
//
// LDS layout of one operand tile: rows of BK bf16; a row's logical 16-byte
// chunk c sits at position c ^ f(row), f(row) = (row / R) mod (BK / 8) with
// R = 256 / (2 * BK) rows per 256 bytes.  A fragment read of the 32x32x16
// MFMA puts 16 consecutive lanes on 16 consecutive rows at one logical
// chunk; those 16 reads then cover the 256 bytes of LDS banks exactly once
// (row mod R picks the row's slot, f the chunk within it): no bank conflicts.
//
// Within a slice the fragments of k16 step s + 1 are read under the MFMAs
// of step s; the barrier sits before the last step, so the first fragments
// of the next slice are read, and the slice's slots are refilled, under the
// slice's last MFMAs.  The order is pinned with scheduling fences.
// ---------------------------------------------------------------------------
constexpr int kBig = 256;
// Configuration of the many-rows tile (measured on MI355X, V3-shape prefill):
// BK = 64 (128-byte row segments) in a ring of five 32 KB operand slots,
// 8 waves (two per SIMD, so one issues MFMAs while its sibling waits on
// loads or LDS), and
// runs of 16 consecutive tiles per XCD (kXcdChunk: 3 % faster than the list
// dealt tile by tile, which shares fewer panels in each L2, and than one
// contiguous slice per XCD, which leaves the XCDs unevenly loaded at the end).
#ifndef MOE_BIG_WAVES
#define MOE_BIG_WAVES 8
#endif
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) bf16_t lds_bf16_t;   // bf16 in LDS

// Workgroup barrier without the memory fence of __syncthreads(), whose
// release semantics would wait for every outstanding load (vmcnt(0)) and
// drain the multi-stage pipeline.  Ordering is kept explicitly: each wave
// waits for its own stage loads first (vmcnt), and for its own LDS fragment
// reads of a stage (lgkmcnt(0)) before the barrier that precedes the refill
// of that stage.  The "memory" clobber keeps the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

// Work-list tile of workgroup blockIdx.x for the many-rows kernels; false
// when the workgroup has none.  XCD-aware order: workgroup ids are dealt
// round-robin over the 8 XCDs, so the j-th workgroup of XCD x is id 8 j + x;
// it takes tile (j / kXcdChunk) * 8 kXcdChunk + x * kXcdChunk + j % kXcdChunk.
// Each XCD thus works through runs of kXcdChunk consecutive work-list tiles
// (sharing A and weight panels in its own L2), and the runs are dealt out in
// turn, so every XCD keeps drawing from the whole list.
__device__ __forceinline__ bool fetch_tile(const GemmParams& P, Tile& tl) {
    const int nt = *P.ntiles;
    const int wg = blockIdx.x;
    const int nr = (nt + 8 * kXcdChunk - 1) / (8 * kXcdChunk) * (8 * kXcdChunk);
    if (wg >= nr) return false;
    const int jx = wg >> 3;
    const int lt = (jx / kXcdChunk) * (8 * kXcdChunk) + (wg & 7) * kXcdChunk + jx % kXcdChunk;
    if (lt >= nt) return false;
    tl = P.tiles[lt];
    return true;
}

// One 256 x 256 tile, bf16 weights (or, Q8, 8-bit routed weights).
//
// LDS is a ring of five 32 KB slots, each holding one operand half — the
// A or the B part of one BK = 64 slice; half h (A of slice s: h = 2s, B:
// h = 2s + 1) lives in slot h mod 5.  Four slots hold the slice being read
// and the next one; the fifth lets the A half of the slice after that load
// a whole slice earlier: iteration kt issues A of slice kt + 2 from its
// start, spread over steps 0-2 (its slot held B of slice kt - 1, free since
// the previous barrier), and B of slice kt + 2 after the barrier that ends
// the reads of slice kt, over step 3 (into A of slice kt's slot).  Fewer
// loads then leave at once, and half of them have nearly two slices of MFMA
// time to land.  (Measured on the V3-shape prefill: gate/up 6.82 -> 6.47 ms
// and down 3.63 -> 3.57 ms against two 64 KB stages; running several tiles
// per workgroup, with the next tile's first slice loading under the
// epilogue, measured slower than one tile per workgroup with this ring.)
// SAVEZ (gate/up of a training forward): the tile's pre-activations W1 x and
// W3 x also go out, as bf16, to Z.
template <bool SWIGLU, int NW, bool Q8 = false, bool SAVEZ = false>
__device__ __forceinline__ void big_tile(const GemmParams& P, const Tile& tl, lds_bf16_t* smem) {
    constexpr int BK = 64;
    constexpr int OPER = kBig * BK;                // elements of one operand half (32 KB)
    constexpr int NSLOT = 5;
    constexpr int CH = BK / 8;                     // 16-byte chunks per row
    constexpr int RI = 1024 / (2 * BK);            // rows per load instruction
    constexpr int R = 256 / (2 * BK);              // rows per 256 bytes of LDS
    constexpr int NI = kBig / RI;                  // load instructions per half
    constexpr int QI = NI / NW;                    // ... per wave
    // 8-bit B: a half is 64 codes per weight row (16 KB of its slot), one
    // instruction moving 16 rows x 64 B
    constexpr int QB = Q8 ? (kBig / 16) / NW : QI; // B load instructions per wave per half
    constexpr int SPS = BK / 16;                   // k16 steps per slice
    constexpr int WN = NW / 2;                     // waves along the B rows (2 along M)
    constexpr int WCOLS = kBig / WN;               // B-rows per wave
    constexpr int NB = WCOLS / 32;                 // 32-wide B blocks per wave
    constexpr int HB = NB / 2;                     // SwiGLU: W1 blocks (then as many W3)
    static_assert(NW == 4 || NW == 8, "waves per workgroup");
    static_assert(SPS == 4, "four k16 steps per slice");
    static_assert(2 * QI <= 63, "vmcnt range");
    static_assert(QI >= 2 && QI % 2 == 0 && QB >= 2 && QB % 2 == 0, "W1 / W3 halves of the load list");

    const int tid = threadIdx.x;
    constexpr int kPhaseKind = SWIGLU ? 0 : 1;
    PHASE_STAMP(kPhaseKind, 0);
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const int wm = wave / WN, wn = wave % WN;

    // Load assignment: wave w issues instructions j = w + NW q, q < QI, of
    // each half; instruction j fills rows RI*j .. RI*j + RI - 1.  Lane l
    // fills position l % CH of row RI*j + l / CH, i.e. logical chunk
    // (l % CH) ^ f(row).  SwiGLU: B rows 0..127 (q < QI/2) come from W1,
    // 128..255 from W3.
    const bool shared = tl.group >= P.E;
    const int s = tl.group - P.E;
    const int kdim = shared ? P.kdim_s : P.kdim_r;
    const int ncols = shared ? P.n_s : P.n_r;
    const int grow = P.goff[tl.group] + tl.m0;
    const int rrow = shared ? grow - P.TK : grow;
    const void* wa;
    const void* wb;
    if (Q8) {                                      // routed tiles only
        wa = P.Qa_r + (size_t)tl.group * ncols * kdim;
        wb = SWIGLU ? P.Qb_r + (size_t)tl.group * ncols * kdim : wa;
    } else {
        wa = shared ? P.Ba_s + (size_t)s * ncols * kdim : P.Ba_r + (size_t)tl.group * ncols * kdim;
        wb = wa;
        if (SWIGLU)
            wb = shared ? P.Bb_s + (size_t)s * ncols * kdim : P.Bb_r + (size_t)tl.group * ncols * kdim;
    }
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(shared ? P.A_s : P.A_r, shared ? P.abytes_s : P.abytes_r);
    const uint32_t wbytes = (uint32_t)ncols * (uint32_t)kdim * (Q8 ? 1u : 2u);
    const __amdgpu_buffer_rsrc_t rw1 = make_rsrc(wa, wbytes);
    const __amdgpu_buffer_rsrc_t rw3 = make_rsrc(wb, wbytes);
    uint32_t aoff[QI], boff[QB];
#pragma unroll
    for (int q = 0; q < QI; ++q) {
        const int row = RI * (wave + NW * q) + lane / CH;
        const uint32_t cbytes = (uint32_t)(((lane % CH) ^ ((row / R) % CH)) * 16);
        const int rr = row < tl.nrows ? row : 0;
        const uint32_t arow = SWIGLU ? (uint32_t)P.tok_of[grow + rr] : (uint32_t)(rrow + rr);
        aoff[q] = arow * (uint32_t)kdim * 2u + cbytes;
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
        // bf16: as A; 8-bit: lane l fills chunk l % 4 of row 16 j + l / 4,
        // at position (l % 4) ^ ((row >> 2) & 3)
        const int row = Q8 ? 16 * (wave + NW * q) + lane / 4 : RI * (wave + NW * q) + lane / CH;
        const uint32_t cbytes = Q8 ? (uint32_t)(((lane & 3) ^ ((row >> 2) & 3)) * 16)
                                   : (uint32_t)(((lane % CH) ^ ((row / R) % CH)) * 16);
        int n = tl.n0 + ((SWIGLU && q >= QB / 2) ? row - kBig / 2 : row);
        n = n < ncols ? n : ncols - 1;
        boff[q] = (uint32_t)n * (uint32_t)kdim * (Q8 ? 1u : 2u) + cbytes;
    }

    // LDS destinations are wave-uniform: computed from a scalar base so the
    // M0 value of every load is a scalar add (no VGPR -> SGPR round trip).
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)smem + (uint32_t)(wave * RI * BK * 2));
    auto slot = [](int h) { return h % NSLOT; };
    // Load q of half h: the A rows of slice h / 2 for even h, else its B
    // rows.  The slice's k offset goes in the scalar offset, so the lane
    // offsets stay fixed over the main loop.
    auto load_one = [&](int h, int q) {
        const uint32_t sa = lds_base + (uint32_t)(slot(h) * OPER * 2) + (uint32_t)(NW * q * 1024);
        if ((h & 1) == 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(uintptr_t)sa, 16, (int)aoff[q],
                                                     (h >> 1) * (BK * 2), 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds((SWIGLU && q >= QB / 2) ? rw3 : rw1,
                                                     (lds_ptr_t)(uintptr_t)sa, 16, (int)boff[q],
                                                     (h >> 1) * (BK * (Q8 ? 1 : 2)), 0, 0);
    };
    auto load_half = [&](int h) {
#pragma unroll
        for (int q = 0; q < ((h & 1) ? QB : QI); ++q) load_one(h, q);
    };

    f32x16 acc[4][NB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f32x16{};

    // Fragment addressing (elements): this lane's row base and the swizzled
    // chunk of k16 step st (rows differ from lane & 31 by multiples of 32).
    // SwiGLU: blocks j < HB are W1 rows, j >= HB the same rows of W3.
    const int lrow = lane & 31;
    const int a_row0 = (wm * 128 + lrow) * BK;
    int b_row0[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int br = SWIGLU ? ((j < HB ? 0 : kBig / 2) + wn * (WCOLS / 2) + (j % HB) * 32)
                              : (wn * WCOLS + j * 32);
        b_row0[j] = (br + lrow) * BK;
    }
    // 8-bit: the order of k inside a slice is permuted alike for both
    // operands — step st = 2u + s, lane half h and element e stand for k =
    // 32 u + 16 h + 8 s + e — so a lane's 16 codes for steps 2u and 2u + 1
    // are one 16-byte chunk (codes 32 u + 16 h .. + 15), read once and
    // widened exactly to two bf16 fragments, and its A fragment of step st
    // is the 8-element chunk 4 u + 2 h + s.
    const int h = lane >> 5;
    int cx[SPS];
#pragma unroll
    for (int st = 0; st < SPS; ++st) {
        const int chunk = Q8 ? 4 * (st >> 1) + 2 * h + (st & 1) : 2 * st + h;
        cx[st] = (chunk ^ ((lrow / R) % CH)) << 3;
    }
    int qb_row[NB];                                 // 8-bit: byte offset of the lane's code row
    uint32_t cq[2];                                 // 8-bit: code chunk of step pair u
#pragma unroll
    for (int j = 0; j < NB; ++j) qb_row[j] = (b_row0[j] / BK) * 64;
#pragma unroll
    for (int u = 0; u < 2; ++u) cq[u] = (uint32_t)(((2 * u + h) ^ ((lrow >> 2) & 3)) << 4);

    // The fragment reads and MFMAs take the number of this wave's 32-row
    // activation blocks that hold rows of the tile (NA, a compile-time
    // constant per main-loop instance): a ragged last tile of a group skips
    // the products (and fragment reads) of its padding blocks.  The waves of
    // one SIMD are one from each half of the tile's rows, so the skipped
    // work shortens every SIMD's share alike.
    bf16x8 fa[2][4], fb[2][NB];
    u32x4 codes[NB];                                // 8-bit: codes of the next step pair
    // Fragment read r of step st of slice kt: the A fragments fa[0..NA) and
    // the B fragments fb[0..NB) (bf16) or, 8-bit and st even, the codes of
    // the B blocks for steps st and st + 1.  Down: A first.  Gate/up: B
    // first, so that the first MFMAs of the step have their operands
    // earliest (measured 0.7 % faster there, 1.4 % slower on down).
    auto read_one = [&](auto na_c, int set, int kt, int st, int r) {
        constexpr int NA = decltype(na_c)::value;
        const int nbr = (!Q8 || (st & 1) == 0) ? NB : 0;   // B reads of step st
        const bool is_a = SWIGLU ? r >= nbr : r < NA;
        const int ra = SWIGLU ? r - nbr : r;
        const int rb = SWIGLU ? r : r - NA;
        if (is_a) {
            const lds_bf16_t* sa = smem + slot(2 * kt) * OPER;
            fa[set][ra] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(sa + a_row0 + ra * 32 * BK + cx[st]);
        } else if (!Q8) {
            const lds_bf16_t* sb = smem + slot(2 * kt + 1) * OPER;
            fb[set][rb] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(sb + b_row0[rb] + cx[st]);
        } else {
            const __attribute__((address_space(3))) uint8_t* sb =
                reinterpret_cast<const __attribute__((address_space(3))) uint8_t*>(smem + slot(2 * kt + 1) * OPER);
            codes[rb] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(sb + qb_row[rb] + cq[st >> 1]);
        }
    };
    // reads of step st: the A fragments, and the B fragments (bf16) or the
    // codes of the step pair starting at st (8-bit)
    auto reads_of = [](int na, int st) {
        return na > 0 ? na + ((!Q8 || (st & 1) == 0) ? NB : 0) : 0;
    };
    // 8-bit: the codes of a step pair to the B fragments of its two steps
    auto widen = [&]() {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const u32x4 w = codes[j];
            const u32x4 lo = {e4m3x2_to_bf16x2<false>(w.x), e4m3x2_to_bf16x2<true>(w.x),
                              e4m3x2_to_bf16x2<false>(w.y), e4m3x2_to_bf16x2<true>(w.y)};
            const u32x4 hi = {e4m3x2_to_bf16x2<false>(w.z), e4m3x2_to_bf16x2<true>(w.z),
                              e4m3x2_to_bf16x2<false>(w.w), e4m3x2_to_bf16x2<true>(w.w)};
            fb[0][j] = __builtin_bit_cast(bf16x8, lo);
            fb[1][j] = __builtin_bit_cast(bf16x8, hi);
        }
    };
    // The weight fragment is the MFMA's first operand, the activation
    // fragment its second, so the accumulator is the transposed block: lane
    // l holds activation row (l & 31) and output columns 8i + 4(l >> 5) + j
    // (i, j = 0..3) — four runs of four consecutive columns, which the
    // epilogue writes as 8-byte pieces.
    auto mfma_one = [&](int set, int m) {
        const int i = m / NB, j = m % NB;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[set][j], fa[set][i], acc[i][j], 0, 0, 0);
    };

    // Main loop (nk slices), slices 0 and 1 issued and slice 0 landed.  Each k16 step is a sequence of fenced groups — one MFMA of
    // the step, one fragment read of the next step and the group's share of
    // the loads — so that the reads and loads issue under running MFMAs
    // (left to the scheduler, loads leave in one burst and the MFMAs wait
    // behind them).  Before step 3 of slice kt: wait for slice kt + 1 and
    // for this wave's reads of slice kt, then the barrier after which slice
    // kt's slots are free.
    auto main_loop = [&](auto na_c, int nk) {
        constexpr int NA = decltype(na_c)::value;
        constexpr int MF = NA * NB;
        constexpr int RD = NA > 0 ? NA + NB : 0;     // most reads of one step
        constexpr int G = MF > RD ? MF : (RD > 0 ? RD : 1);
        // The next step's fragment reads go out RPG per group.  Two per group
        // (all of them in the step's first half, more time to land before the
        // wait ahead of the barrier) measured 3 % faster on the down GEMM and
        // 1 % slower on gate/up, so gate/up keeps one per group.
        constexpr int RPG = SWIGLU ? 1 : 2;
#pragma unroll
        for (int r = 0; r < RD; ++r) read_one(na_c, 0, 0, 0, r);
        int kt = 0;
        for (; kt + 2 < nk; ++kt) {                  // steady state: slice kt + 2 to issue
#pragma unroll
            for (int st = 0; st + 1 < SPS; ++st) {
                if (Q8 && NA > 0 && (st & 1) == 0) widen();
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    if (g < MF) mfma_one(st & 1, g);
#pragma unroll
                    for (int r = RPG * g; r < RPG * g + RPG; ++r)
                        if (r < reads_of(NA, st + 1)) read_one(na_c, (st + 1) & 1, kt, st + 1, r);
                    const int t = st * G + g;        // A of slice kt + 2 over steps 0-2
#pragma unroll
                    for (int q = t * QI / (3 * G); q < (t + 1) * QI / (3 * G); ++q)
                        load_one(2 * (kt + 2), q);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            wait_vm<QI>();                           // slice kt + 1 landed (A of kt + 2 may not)
            // this wave's reads of slice kt (the last step's fragments) have
            // returned before the barrier after which its slots are refilled
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            stage_barrier();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int g = 0; g < G; ++g) {            // step 3, B of slice kt + 2, slice kt + 1's first reads
                if (g < MF) mfma_one((SPS - 1) & 1, g);
#pragma unroll
                for (int q = g * QB / G; q < (g + 1) * QB / G; ++q) load_one(2 * (kt + 2) + 1, q);
                if (g < RD) read_one(na_c, 0, kt + 1, 0, g);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        for (; kt < nk; ++kt) {                      // tail: nothing left to issue
#pragma unroll
            for (int st = 0; st + 1 < SPS; ++st) {
                if (Q8 && NA > 0 && (st & 1) == 0) widen();
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    if (g < MF) mfma_one(st & 1, g);
#pragma unroll
                    for (int r = RPG * g; r < RPG * g + RPG; ++r)
                        if (r < reads_of(NA, st + 1)) read_one(na_c, (st + 1) & 1, kt, st + 1, r);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            wait_vm<0>();
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            stage_barrier();
            __builtin_amdgcn_sched_barrier(0);
            const bool more_k = kt + 1 < nk;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (g < MF) mfma_one((SPS - 1) & 1, g);
                if (g < RD && more_k) read_one(na_c, 0, kt + 1, 0, g);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    const int nk = kdim / BK;
    load_half(0);
    load_half(1);
    if (nk > 1) {
        load_half(2);
        load_half(3);
        wait_vm<QI + QB>();                          // slice 0 landed
    } else {
        wait_vm<0>();
    }
    stage_barrier();
    PHASE_STAMP(kPhaseKind, 1);
    // the instance for this wave's share of the tile's rows (wave-uniform)
    {
        const int na = (tl.nrows - wm * 128 + 31) >> 5;
        if (na >= 4) main_loop(std::integral_constant<int, 4>{}, nk);
        else if (na == 3) main_loop(std::integral_constant<int, 3>{}, nk);
        else if (na == 2) main_loop(std::integral_constant<int, 2>{}, nk);
        else if (na == 1) main_loop(std::integral_constant<int, 1>{}, nk);
        else main_loop(std::integral_constant<int, 0>{}, nk);
    }
    PHASE_STAMP(kPhaseKind, 2);

    // Epilogue: the tile's outputs (bf16; SwiGLU applied in registers) go
    // through LDS — now free — and leave as whole 16-byte row pieces.
    // Gate/up (128 output columns per tile, 32 per wave): the workgroup
    // stages the whole tile, one row segment of OC * 2 bytes per CPR lanes.
    // Down (256 columns, WCOLS = 64 per wave): each wave stages its own
    // 128 x WCOLS block in a private region and stores it as whole 128-byte
    // row segments, with no second barrier (waves that finish early store
    // early).  In LDS, 16-byte chunk c of row r sits at position c ^ (r mod
    // chunks per row), so the 32 rows one write instruction touches spread
    // over the banks.
    constexpr int OC = SWIGLU ? kBig / 2 : kBig;     // output columns of the tile
    constexpr int CPR = OC / 8;                      // 16-byte chunks per row
    constexpr int RC = WCOLS / 8;                    // down: chunks per region row
    static_assert(kBig * OC <= NSLOT * OPER, "output tile fits the slots");
    // No barrier before the staging: the main loop's last barrier comes
    // after every wave's last fragment read and after the last load into
    // the slots has landed; only MFMAs on registers follow it.
    {
        const int ocol_l = (SWIGLU ? wn * (WCOLS / 2) : wn * WCOLS) + 4 * (lane >> 5);   // + 32 j + 8 r4
        // 8-bit: each output column's accumulators times its weight rows' scales
        const float* sca = Q8 ? P.Sa_r + (size_t)tl.group * ncols : nullptr;
        const float* scb = Q8 && SWIGLU ? P.Sb_r + (size_t)tl.group * ncols : nullptr;
#pragma unroll
        for (int j = 0; j < (SWIGLU ? HB : NB); ++j) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                float fa4[4] = {1.f, 1.f, 1.f, 1.f}, fb4[4] = {1.f, 1.f, 1.f, 1.f};
                if (Q8) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int n = tl.n0 + ocol_l + 32 * j + 8 * r4 + e;
                        fa4[e] = n < ncols ? sca[n] : 0.f;
                        if (SWIGLU) fb4[e] = n < ncols ? scb[n] : 0.f;
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * r4 + e;
                        const float a = Q8 ? acc[i][j][r] * fa4[e] : acc[i][j][r];
                        v[e] = SWIGLU ? silu(a) * (Q8 ? acc[i][j + HB][r] * fb4[e] : acc[i][j + HB][r]) : a;
                    }
                    const uint32_t lo = pack_bf16x2(v[0], v[1]);
                    const uint32_t hi = pack_bf16x2(v[2], v[3]);
                    const int orow = wm * 128 + 32 * i + lrow;
                    const int ocol = ocol_l + 32 * j + 8 * r4;      // multiple of 4
                    if (SAVEZ && SWIGLU && orow < tl.nrows && tl.n0 + ocol < ncols) {
                        bf16_t* z = (shared ? P.Z_s : P.Z_r) + (size_t)(rrow + orow) * 2 * ncols + tl.n0 + ocol;
                        const int r0 = 4 * r4;
                        *reinterpret_cast<u32x2*>(z) =
                            u32x2{pack_bf16x2(acc[i][j][r0], acc[i][j][r0 + 1]),
                                  pack_bf16x2(acc[i][j][r0 + 2], acc[i][j][r0 + 3])};
                        *reinterpret_cast<u32x2*>(z + ncols) =
                            u32x2{pack_bf16x2(acc[i][j + HB][r0], acc[i][j + HB][r0 + 1]),
                                  pack_bf16x2(acc[i][j + HB][r0 + 2], acc[i][j + HB][r0 + 3])};
                    }
                    int off;
                    if (SWIGLU) {
                        off = orow * OC + (((ocol >> 3) ^ (orow % CPR)) << 3) + (ocol & 4);
                    } else {
                        const int lr = 32 * i + lrow, lc = ocol - wn * WCOLS;
                        off = wave * (128 * WCOLS) + lr * WCOLS + (((lc >> 3) ^ (lr % RC)) << 3) + (lc & 4);
                    }
                    *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(smem + off) = u32x2{lo, hi};
                }
            }
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    bf16_t* obase = shared ? P.O_s : P.O_r;
    if (SWIGLU) {
        stage_barrier();
        for (int c = tid; c < kBig * CPR; c += 64 * NW) {
            const int row = c / CPR;
            const int cc = c - row * CPR;
            const int col = tl.n0 + cc * 8;
            if (row < tl.nrows && col < ncols) {
                const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(smem + row * OC + ((cc ^ (row % CPR)) << 3));
                *reinterpret_cast<u32x4*>(obase + (size_t)(rrow + row) * ncols + col) = v;
            }
        }
    } else {
        // this wave's own writes have landed (LDS operations of one wave
        // complete in order, and lgkmcnt(0) above waited for them)
        const int c0 = tl.n0 + wn * WCOLS;
#pragma unroll 4
        for (int it = 0; it < 128 * RC / 64; ++it) {
            const int idx = it * 64 + lane;
            const int lr = idx / RC, c = idx % RC;
            const int row = wm * 128 + lr, col = c0 + c * 8;
            if (row < tl.nrows && col < ncols) {
                const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                    smem + wave * (128 * WCOLS) + lr * WCOLS + ((c ^ (lr % RC)) << 3));
                *reinterpret_cast<u32x4*>(obase + (size_t)(grow + row) * ncols + col) = v;
            }
        }
    }
    PHASE_STAMP(kPhaseKind, 3);
}

// One 256 x 256 tile of a routed expert with 8-bit activations and 8-bit
// weights (MOE_FLAG_ACT8), on the FP8 matrix cores: v_mfma_f32_32x32x64_f8f6f4
// (E4M3 x E4M3, fp32 accumulation), twice the bf16 rate per k.  Gate/up
// (SWIGLU): A = codes of the gathered token rows, B = 128 rows of W1 then the
// same 128 rows of W3.  Down: A = codes of the tile's rows of h (contiguous),
// B = 256 rows of W2.  A slice is 128 codes of k, so an operand half (256
// rows x 128 bytes, 32 KB) loads exactly like a bf16 half of 64 values: the
// same ring of five slots, load assignment and swizzle as big_tile, with two
// k64 MFMA steps per slice instead of four k16 steps.  Fragment of a 32-row
// block: lane l holds row l % 32 and the 32 codes k = 32 (l / 32) .. + 31 of
// the step (two 16-byte LDS reads); on this instruction a lane's half
// (l / 32) and byte position pair A and B codes of equal k, and lane l
// addresses row / column l % 32 of the operand (measured on MI355X).
// Each wave owns 128 rows x 64 B-rows (gate/up: 32 of W1 and the same 32 of
// W3).  As in big_tile, each step is a sequence of fenced groups — one MFMA,
// one fragment read of the next step into the other register set, a share of
// the loads — so reads and loads issue under running MFMAs.  The epilogue
// scales each output by 2^e of its activation row and its weight row's scale
// (the exact power-of-two step first), then gate/up applies SwiGLU.
template <bool SWIGLU>
__device__ __forceinline__ void f8_tile(const GemmParams& P, const Tile& tl, lds_bf16_t* smem) {
    constexpr int BKB = 128;                       // codes (bytes) of k per slice
    constexpr int OPER = kBig * BKB / 2;           // bf16-sized elements of one operand half
    constexpr int NSLOT = 5;
    constexpr int NW = 8;
    constexpr int CH = BKB / 16;                   // 16-byte chunks per row
    constexpr int RI = 1024 / BKB;                 // rows per load instruction
    constexpr int R = 256 / BKB;                   // rows per 256 bytes of LDS
    constexpr int QI = kBig / RI / NW;             // load instructions per wave per half
    constexpr int WN = NW / 2;                     // waves along the B rows (2 along M)
    constexpr int WCOLS = kBig / WN;               // B-rows per wave
    constexpr int MF = 8;                          // MFMAs per step: 4 row blocks x 2 B blocks
    constexpr int RD = 6;                          // fragment reads per step: 2 B, then 4 A
    typedef int i32x8 __attribute__((ext_vector_type(8)));
    static_assert(QI == 4, "four load instructions per wave per half");

    const int tid = threadIdx.x;
    constexpr int kPhaseKind = SWIGLU ? 2 : 3;
    PHASE_STAMP(kPhaseKind, 0);
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int kdim = P.kdim_r;                     // codes per activation / weight row
    const int ncols = P.n_r;
    const int grow = P.goff[tl.group] + tl.m0;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(P.Xq, P.abytes_r / 2);   // codes: half the bf16 bytes
    const uint32_t wbytes = (uint32_t)ncols * (uint32_t)kdim;
    const __amdgpu_buffer_rsrc_t rw1 = make_rsrc(P.Qa_r + (size_t)tl.group * wbytes, wbytes);
    const __amdgpu_buffer_rsrc_t rw3 =
        SWIGLU ? make_rsrc(P.Qb_r + (size_t)tl.group * wbytes, wbytes) : rw1;
    uint32_t aoff[QI], boff[QI];
#pragma unroll
    for (int q = 0; q < QI; ++q) {
        const int row = RI * (wave + NW * q) + lane / CH;
        const uint32_t cbytes = (uint32_t)(((lane % CH) ^ ((row / R) % CH)) * 16);
        const int rr = row < tl.nrows ? row : 0;
        const uint32_t arow = SWIGLU ? (uint32_t)P.tok_of[grow + rr] : (uint32_t)(grow + rr);
        aoff[q] = arow * (uint32_t)kdim + cbytes;
        int n = tl.n0 + ((SWIGLU && q >= QI / 2) ? row - kBig / 2 : row);   // gate/up: W1 rows, then W3
        n = n < ncols ? n : ncols - 1;
        boff[q] = (uint32_t)n * (uint32_t)kdim + cbytes;
    }
    const int lrow = lane & 31, hh = lane >> 5;
    // the scale exponents of this lane's four output rows, for the epilogue
    // (gate/up: two dependent loads through tok_of, issued under the last
    // slice's MFMAs)
    int ex[4];
    auto fetch_ex = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = wm * 128 + 32 * i + lrow;
            ex[i] = m < tl.nrows ? P.Xe[SWIGLU ? P.tok_of[grow + m] : grow + m] : 0;
        }
    };
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)smem + (uint32_t)(wave * RI * BKB));
    auto slot = [](int h) { return h % NSLOT; };
    auto load_one = [&](int h, int q) {            // half h: A (even) or B (odd) of slice h / 2
        const uint32_t sa = lds_base + (uint32_t)(slot(h) * OPER * 2) + (uint32_t)(NW * q * 1024);
        if ((h & 1) == 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(uintptr_t)sa, 16, (int)aoff[q],
                                                     (h >> 1) * BKB, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds((SWIGLU && q >= QI / 2) ? rw3 : rw1,
                                                     (lds_ptr_t)(uintptr_t)sa, 16, (int)boff[q],
                                                     (h >> 1) * BKB, 0, 0);
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    int b_row[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
        b_row[j] = SWIGLU ? (j == 0 ? 0 : kBig / 2) + wn * (WCOLS / 2) + lrow : wn * WCOLS + 32 * j + lrow;
    i32x8 fa[2][4], fb[2][2];
    // fragment read r of step st of slice kt into register set `set`: the
    // two B fragments first, then the four A fragments (chunks 4 st + 2 hh
    // and + 1 of the row)
    auto read_one = [&](int set, int kt, int st, int r) {
        const bool is_b = r < 2;
        const lds_bf16_t* base = smem + slot(2 * kt + (is_b ? 1 : 0)) * OPER;
        const int row = is_b ? b_row[r] : wm * 128 + 32 * (r - 2) + lrow;
        const int c0 = 4 * st + 2 * hh, f = (row / R) % CH;
        const u32x4 lo = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
            base + row * (BKB / 2) + ((c0 ^ f) << 3));
        const u32x4 hi = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
            base + row * (BKB / 2) + (((c0 + 1) ^ f) << 3));
        const i32x8 v = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        if (is_b) fb[set][r] = v;
        else fa[set][r - 2] = v;
    };
    // The weight fragment is the first operand, so lane l of the
    // accumulator holds activation row l % 32 (as in big_tile)
    auto mfma_one = [&](int set, int m) {
        const int i = m / 2, j = m % 2;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[set][j], fa[set][i], acc[i][j], 0, 0, 0,
                                                                    0, 0, 0);
    };

    const int nk = kdim / BKB;
#pragma unroll
    for (int q = 0; q < QI; ++q) load_one(0, q);
#pragma unroll
    for (int q = 0; q < QI; ++q) load_one(1, q);
    if (nk > 1) {
#pragma unroll
        for (int q = 0; q < QI; ++q) load_one(2, q);
#pragma unroll
        for (int q = 0; q < QI; ++q) load_one(3, q);
        wait_vm<2 * QI>();                         // slice 0 landed
    } else {
        wait_vm<0>();
    }
    stage_barrier();
    PHASE_STAMP(kPhaseKind, 1);
#pragma unroll
    for (int r = 0; r < RD; ++r) read_one(0, 0, 0, r);
    int kt = 0;
    for (; kt + 2 < nk; ++kt) {                    // steady state: slice kt + 2 to issue
#pragma unroll
        for (int g = 0; g < MF; ++g) {             // step 0, step 1's reads, A of slice kt + 2
            mfma_one(0, g);
            if (g < RD) read_one(1, kt, 1, g);
            if (g % 2 == 1) load_one(2 * (kt + 2), g / 2);
            __builtin_amdgcn_sched_barrier(0);
        }
        wait_vm<QI>();                             // slice kt + 1 landed (A of kt + 2 may not)
        // this wave's reads of slice kt have returned before the barrier after
        // which slice kt's A slot is refilled
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        stage_barrier();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int g = 0; g < MF; ++g) {             // step 1, B of slice kt + 2, slice kt + 1's first reads
            mfma_one(1, g);
            if (g % 2 == 1) load_one(2 * (kt + 2) + 1, g / 2);
            if (g < RD) read_one(0, kt + 1, 0, g);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    for (; kt < nk; ++kt) {                        // tail: nothing left to issue
#pragma unroll
        for (int g = 0; g < MF; ++g) {
            mfma_one(0, g);
            if (g < RD) read_one(1, kt, 1, g);
        }
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<0>();
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        stage_barrier();
        __builtin_amdgcn_sched_barrier(0);
        const bool more_k = kt + 1 < nk;
        if constexpr (SWIGLU)
            if (!more_k) fetch_ex();
#pragma unroll
        for (int g = 0; g < MF; ++g) {
            mfma_one(1, g);
            if (g < RD && more_k) read_one(0, kt + 1, 0, g);
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    PHASE_STAMP(kPhaseKind, 2);
    // Epilogue: each output times 2^e of its activation row and its weight
    // row's scale; gate/up applies SwiGLU and stages the whole 256 x 128
    // tile in LDS, down stages each wave's 128 x 64 block in a region of its
    // own (as big_tile); both leave as 16-byte row pieces.  No barrier before
    // the staging: after the main loop's last barrier no wave reads the
    // slots again and no load into them is in flight.
    constexpr int OC = SWIGLU ? kBig / 2 : kBig;   // output columns of the tile
    constexpr int CPR = OC / 8;
    constexpr int RC = WCOLS / 8;                  // down: chunks per region row
    constexpr int NJ = SWIGLU ? 1 : 2;
    typedef float f32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
    {
        const int ocol_l = (SWIGLU ? wn * (WCOLS / 2) : wn * WCOLS) + 4 * hh;
        const float* sca = P.Sa_r + (size_t)tl.group * ncols;
        const float* scb = SWIGLU ? P.Sb_r + (size_t)tl.group * ncols : sca;
        // the weight-row scales of the lane's output columns, all loads
        // issued before any is used: runs of four consecutive columns (ncols
        // and the run starts are multiples of 4, so a run is wholly inside
        // or wholly past the matrix)
        f32x4 sa4[NJ][4], sb4[4];
        if constexpr (!SWIGLU) fetch_ex();
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int n = tl.n0 + ocol_l + 32 * j + 8 * r4;
                sa4[j][r4] = n < ncols ? (f32x4)*reinterpret_cast<const f32x4a4*>(sca + n) : f32x4{};
                if (SWIGLU) sb4[r4] = n < ncols ? (f32x4)*reinterpret_cast<const f32x4a4*>(scb + n) : f32x4{};
            }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                float fa4[4], fb4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    fa4[e] = sa4[j][r4][e];
                    fb4[e] = SWIGLU ? sb4[r4][e] : 0.f;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * r4 + e;
                        const float a = ldexpf(acc[i][j][r], ex[i]) * fa4[e];
                        v[e] = SWIGLU ? silu(a) * (ldexpf(acc[i][1][r], ex[i]) * fb4[e]) : a;
                    }
                    const int orow = wm * 128 + 32 * i + lrow;
                    const int ocol = ocol_l + 32 * j + 8 * r4;      // multiple of 4
                    int off;
                    if (SWIGLU) {
                        off = orow * OC + (((ocol >> 3) ^ (orow % CPR)) << 3) + (ocol & 4);
                    } else {
                        const int lr = 32 * i + lrow, lc = ocol - wn * WCOLS;
                        off = wave * (128 * WCOLS) + lr * WCOLS + (((lc >> 3) ^ (lr % RC)) << 3) + (lc & 4);
                    }
                    *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(smem + off) =
                        u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                }
            }
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (SWIGLU) {
        stage_barrier();
        for (int c = tid; c < kBig * CPR; c += 64 * NW) {
            const int row = c / CPR;
            const int cc = c - row * CPR;
            const int col = tl.n0 + cc * 8;
            if (row < tl.nrows && col < ncols) {
                const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                    smem + row * OC + ((cc ^ (row % CPR)) << 3));
                *reinterpret_cast<u32x4*>(P.O_r + (size_t)(grow + row) * ncols + col) = v;
            }
        }
    } else {
        // this wave's own writes have landed (LDS operations of one wave
        // complete in order, and lgkmcnt(0) above waited for them)
        const int c0 = tl.n0 + wn * WCOLS;
#pragma unroll 4
        for (int it = 0; it < 128 * RC / 64; ++it) {
            const int idx = it * 64 + lane;
            const int lr = idx / RC, c = idx % RC;
            const int row = wm * 128 + lr, col = c0 + c * 8;
            if (row < tl.nrows && col < ncols) {
                const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                    smem + wave * (128 * WCOLS) + lr * WCOLS + ((c ^ (lr % RC)) << 3));
                *reinterpret_cast<u32x4*>(P.O_r + (size_t)(grow + row) * ncols + col) = v;
            }
        }
    }
    PHASE_STAMP(kPhaseKind, 3);
}

// LDS of the many-rows tile: five 32 KB operand slots (160 KB).
constexpr int kBigLdsBytes = 5 * kBig * 64 * 2;

// Many rows per expert with 8-bit routed weights: routed tiles take the
// 8-bit tile (A8: with 8-bit activations, the FP8 tile), shared-expert tiles
// (bf16 weights) the bf16 one.
template <bool SWIGLU, bool A8>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_big_q8_kernel(GemmParams P) {
    __shared__ __attribute__((aligned(1024))) bf16_t smem[kBigLdsBytes / 2];
    Tile tl;
    if (!fetch_tile(P, tl)) return;
    if (tl.group < P.E) {
        if constexpr (A8) f8_tile<SWIGLU>(P, tl, (lds_bf16_t*)smem);
        else big_tile<SWIGLU, 8, true>(P, tl, (lds_bf16_t*)smem);
    } else {
        big_tile<SWIGLU, 8, false>(P, tl, (lds_bf16_t*)smem);
    }
}

template <bool SWIGLU, int NW, bool SAVEZ = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void gemm_big_kernel(GemmParams P) {
    __shared__ __attribute__((aligned(1024))) bf16_t smem[kBigLdsBytes / 2];
    Tile tl;
    if (!fetch_tile(P, tl)) return;
    big_tile<SWIGLU, NW, false, SAVEZ>(P, tl, (lds_bf16_t*)smem);
}


// One workgroup per work-list tile (the bound; the XCD runs need whole
// rounds of 8 kXcdChunk).
int tile_grid(int max_tiles) {
    return (max_tiles + 8 * kXcdChunk - 1) / (8 * kXcdChunk) * (8 * kXcdChunk);
}

template <int BM, int BN, int WM, int WN, bool SWIGLU>
hipError_t launch_cfg(const GemmParams& gp, int max_tiles, hipStream_t st) {
    if (max_tiles == 0) return hipSuccess;
    if (gp.Qa_r)
        grouped_gemm_kernel<BM, BN, WM, WN, SWIGLU, true><<<tile_grid(max_tiles), kThreads, 0, st>>>(gp);
    else
        grouped_gemm_kernel<BM, BN, WM, WN, SWIGLU, false><<<(max_tiles + 7) & ~7, kThreads, 0, st>>>(gp);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_gate_up(const Plan& p, const bf16_t* x, const bf16_t* w1,
                               const bf16_t* w3, const bf16_t* ws1, const bf16_t* ws3,
                               const RoutedQ8* q8, hipStream_t st) {
    GemmParams gp{};
    if (q8) {
        gp.Qa_r = q8->q1;
        gp.Qb_r = q8->q3;
        gp.Sa_r = q8->s1;
        gp.Sb_r = q8->s3;
    }
    gp.tiles = p.tiles1;
    gp.ntiles = p.ntiles;
    gp.goff = p.goff;
    gp.tok_of = p.tok_of;
    gp.A_r = p.xd ? p.xd : x;                       // 8-bit activations off the FP8 tile: dequantised rows
    if (q8 && p.xq && !p.xd) {
        gp.Xq = p.xq;
        gp.Xe = p.xe;
    }
    gp.A_s = x;
    gp.Ba_r = w1;
    gp.Bb_r = w3;
    gp.Ba_s = ws1;
    gp.Bb_s = ws3;
    gp.O_r = p.H;
    gp.O_s = p.H + (size_t)p.T * p.K * p.I;
    gp.kdim_r = p.d;
    gp.kdim_s = p.d;
    gp.n_r = p.I;
    gp.n_s = p.Is;
    gp.E = p.E;
    gp.TK = p.T * p.K;
    gp.abytes_r = (uint32_t)((size_t)p.T * p.d * 2);
    gp.abytes_s = gp.abytes_r;
    if (p.Z && !q8) {
        gp.Z_r = p.Z;
        gp.Z_s = p.Z + (size_t)p.T * p.K * 2 * p.I;
    }
    if (p.g1.bm == 256) {
        if (q8 && gp.Xq)
            gemm_big_q8_kernel<true, true><<<tile_grid(p.max_tiles1), 512, 0, st>>>(gp);
        else if (q8)
            gemm_big_q8_kernel<true, false><<<tile_grid(p.max_tiles1), 512, 0, st>>>(gp);
        else if (gp.Z_r)
            gemm_big_kernel<true, MOE_BIG_WAVES, true>
                <<<tile_grid(p.max_tiles1), 64 * MOE_BIG_WAVES, 0, st>>>(gp);
        else
            gemm_big_kernel<true, MOE_BIG_WAVES>
                <<<tile_grid(p.max_tiles1), 64 * MOE_BIG_WAVES, 0, st>>>(gp);
        return hipGetLastError();
    }
    return launch_cfg<32, 256, 1, 4, true>(gp, p.max_tiles1, st);
}

hipError_t launch_gemm_down(const Plan& p, const bf16_t* w2, const bf16_t* ws2,
                            const RoutedQ8* q8, hipStream_t st) {
    GemmParams gp{};
    if (q8) {
        gp.Qa_r = q8->q2;
        gp.Sa_r = q8->s2;
    }
    gp.tiles = p.tiles2;
    gp.ntiles = p.ntiles + 1;
    gp.goff = p.goff;
    gp.tok_of = nullptr;
    gp.A_r = p.H;
    gp.A_s = p.H + (size_t)p.T * p.K * p.I;
    gp.Ba_r = w2;
    gp.Bb_r = nullptr;
    gp.Ba_s = ws2;
    gp.Bb_s = nullptr;
    if (q8 && p.hq) {                               // 8-bit activations on the FP8 tile
        gp.Xq = p.hq;
        gp.Xe = p.he;
    }
    gp.O_r = p.Y;
    gp.O_s = p.Y;
    gp.kdim_r = p.I;
    gp.kdim_s = p.Is;
    gp.n_r = p.d;
    gp.n_s = p.d;
    gp.E = p.E;
    gp.TK = p.T * p.K;
    gp.abytes_r = (uint32_t)((size_t)p.T * p.K * p.I * 2);
    gp.abytes_s = (uint32_t)((size_t)p.T * p.Ks * p.Is * 2);
    if (p.g2.bm == 256) {
        if (q8 && gp.Xq)
            gemm_big_q8_kernel<false, true><<<tile_grid(p.max_tiles2), 512, 0, st>>>(gp);
        else if (q8)
            gemm_big_q8_kernel<false, false><<<tile_grid(p.max_tiles2), 512, 0, st>>>(gp);
        else
            gemm_big_kernel<false, MOE_BIG_WAVES>
                <<<tile_grid(p.max_tiles2), 64 * MOE_BIG_WAVES, 0, st>>>(gp);
        return hipGetLastError();
    }
    return launch_cfg<32, 256, 1, 4, false>(gp, p.max_tiles2, st);
}

}  // namespace moe
