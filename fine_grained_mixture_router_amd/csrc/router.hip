// Router: token-to-centroid affinities, the gate, top-K selection and the
// per-chunk expert masks, in one kernel.
//
// Definition: the generic top-K gate of "DeepSeekMoE 深度解读报告" section 3.1
// (softmax over the inner products of the token with every expert centroid,
// keep the K largest scores, zero the rest, no renormalisation), plus an
// optional fixed per-expert logit bias.  Variants: gates renormalised over
// the K selected (the eliteato DeepSeek-V2 explainer's routing code, section
// 3.1: softmax over the top-K logits), and sigmoid affinities whose bias only
// steers the selection (the youleyou page's auxiliary-loss-free remark; the
// V3 line in the report's closing notes).
//
// One workgroup owns a tile of BT tokens and every expert (E <= 256):
//   1. affinities x . C^T on bf16 MFMA (fp32 accumulation), BK = 64 slices
//      of d streamed by direct-to-LDS loads through three LDS stages;
//   2. fp32 gate per token, one wavefront per token: softmax of logit + bias
//      (default) or sigmoid of the affinity with the bias in the selection
//      key only; K rounds of a wavefront arg-max (DPP within rows of 16
//      lanes, scalar across rows) over the E keys, ceil(E / 64) per lane,
//      ties to the lower expert id; optional renormalisation;
//   3. the tile's bits of every expert's 64-token chunk mask, from which the
//      permutation ranks tokens per expert without atomics.
// Large batches (the plan's split S = 1) keep the whole reduction over d in
// the workgroup: the affinities go from the accumulators to LDS and never to
// memory.  Small batches (decode) cannot fill the chip that way, so the d
// range is split S ways: each workgroup writes its fp32 partial affinities,
// takes a ticket (one atomic per workgroup), and the workgroup that takes
// the last ticket of its tile sums the S partials in split order — a fixed
// order whatever order the workgroups finish in — and does steps 2-3.  The
// tickets are cleared by a one-workgroup kernel launched just before.
//
// Tiles: 64 tokens (32x32x16 MFMA blocks, one chunk per tile) for large
// batches; 16 tokens (16x16x32 blocks, a quarter chunk per tile) for small
// ones, where a 64-token tile's S partials would be too many bytes for the
// one workgroup that sums them.  Workgroups of 16 waves (see the kernel).
#include "common.h"

namespace moe {
namespace {

constexpr int kRThreads = 1024;  // 16 waves
constexpr int kRWaves = kRThreads / 64;

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) bf16_t lds_bf16_t;
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Rows of 64 bf16 (one BK slice), 16-byte chunk c of row r at position
// c ^ ((r >> 1) & 7): a fragment read puts 16 lanes on 16 consecutive rows
// at one logical chunk, and those land in 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row, int chunk) {
    return row * 64 + ((chunk ^ ((row >> 1) & 7)) << 3);
}


// Order-preserving unsigned image of a float (-0 taken as +0, so equal
// values have equal keys); real keys are all above 0, which marks "none".
__device__ __forceinline__ uint32_t key_of(float v) {
    const uint32_t b = __float_as_uint(v + 0.f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float float_of_key(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

template <int NE>
__device__ __forceinline__ uint32_t lane_max(const uint32_t (&u)[NE]) {
    uint32_t m = u[0];
#pragma unroll
    for (int j = 1; j < NE; ++j) m = max(m, u[j]);
    return m;
}

// Maximum over the wavefront, returned to every lane: DPP within each row
// of 16 lanes (pair swap, quad swap, half-row mirror, row mirror leave the
// row's maximum in all 16 lanes), then the four rows through scalar reads.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // [1,0,3,2]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // [2,3,0,1]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // half mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row mirror
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(a, b), max(c, d));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the wavefront, the same in every lane: the four DPP steps above
// within each row of 16, then the row sums added in row order.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    v += dpp_f<0x140>(v);
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return ((a + b) + c) + d;
}

struct RouterArgs {
    const bf16_t* x;
    const bf16_t* C;
    const float* bias;
    int T, d, E, Epad, K, S, kps;   // S splits of the d range, kps slices each
    uint32_t flags;
    float* part;                    // [S, T, Epad] partial affinities (S > 1)
    int32_t* tickets;               // [tiles] (S > 1), zero at launch
    int32_t* idx;                   // [T, K]
    float* gate;                    // [T, K]
    uint64_t* masks;                // [nchunk, Epad]
    float* scores;                  // [T, Epad] or null (training forward)
    float* score_part;              // [nchunk * 4, Epad] or null
};

template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

template <int BT, int NE>
struct RouterLds {
    static constexpr int ROWS = BT + 64 * NE;            // x rows, then centroid rows
    static constexpr int STAGE = ROWS * 64 * 2;          // bytes of one stage
    // stages: as many as about 150 KB hold, 3 to 8 (slices in flight: one
    // fewer); each workgroup's products are bound by load latency, so the
    // depth sets their rate
    static constexpr int SG0 = (150 * 1024) / STAGE;
    static constexpr int SG = SG0 < 3 ? 3 : (SG0 > 8 ? 8 : SG0);
    static constexpr int GEMM = SG * STAGE;
    static constexpr int LOGITS = BT * 64 * NE * 4;      // fp32 [BT][Epad]
    static constexpr int BYTES = GEMM > LOGITS ? GEMM : LOGITS;
};

// BT tokens x (64 NE) experts per workgroup, 16 waves.  The products run on
// waves 0-3, one per SIMD.  With BT = 64 and NE >= 3 wave w takes all 64
// tokens by experts 64 w .. + 63 (four 32x32 blocks); with NE <= 2 wave w
// takes tokens 32 (w / NE) .. + 31 by experts 64 (w % NE) .. + 63 (two
// blocks).  With BT = 16 wave w takes the 16 tokens by experts 64 w .. + 63
// (four 16x16 blocks).  Every operand passes through LDS (written once by
// the loads, read by each wave that needs it), and LDS bandwidth, not the
// MFMA rate, bounds this phase: large per-wave tiles keep the reads down
// (64 KB of reads and 40 KB of writes per 64-deep slice at BT = 64,
// E = 256, about 800 cycles against 512 of MFMA work per SIMD).  Every wave
// issues loads and every wave selects (4 tokens each for BT = 64, one for
// BT = 16): the top-K is a chain of dependent cross-lane steps, and 16
// waves overlap 16 tokens' chains.
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) float lds_float_t;

template <int BT, int NE>
__device__ __forceinline__ void router_tile(const RouterArgs& a, lds_char_t* smem, unsigned* smask,
                                            int& s_last) {
    typedef RouterLds<BT, NE> L;
    constexpr int EP = 64 * NE;
    constexpr int NI = L::ROWS / 8;             // 1 KB load instructions per slice
    constexpr int NQ = (NI + kRWaves - 1) / kRWaves;   // ... per wave, at most
    constexpr int LMIN = NI / kRWaves;                 // ... per wave, at least
    constexpr int SG = L::SG;
    constexpr int P = SG - 1;                          // slices in flight
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = blockIdx.x;
    const int z = blockIdx.y;
    const int t0 = tile * BT;
    const int nk = a.d >> 6;
    const int kb = z * a.kps;
    const int nloc = min(nk, kb + a.kps) - kb;

    for (int i = tid; i < 2 * EP; i += kRThreads) smask[i] = 0u;
    // the bias, one value per lane and block of 64 experts, fetched now so
    // that its latency hides behind the products
    float bj[NE];
#pragma unroll
    for (int j = 0; j < NE; ++j) {
        const int e = lane + 64 * j;
        bj[j] = (a.bias && e < a.E) ? a.bias[e] : 0.f;
    }

    // ---- 1. affinities ----
    // load instruction i = wave + 16 q fills LDS rows 8 i .. 8 i + 7 of a
    // stage (x rows first, then centroid rows); lane l fills position l % 8
    // of row 8 i + l / 8.  Rows past T or E are clamped (never read back).
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)a.T * (uint32_t)a.d * 2u);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.C, (uint32_t)a.E * (uint32_t)a.d * 2u);
    uint32_t off[NQ];
    bool isx[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int i = wave + kRWaves * q;
        const int row = 8 * i + (lane >> 3);
        const uint32_t cb = (uint32_t)(((lane & 7) ^ ((row >> 1) & 7)) * 16);
        isx[q] = i < BT / 8;          // whole instruction: wave-uniform, one resource per load
        const int src = isx[q] ? min(t0 + row, a.T - 1) : min(row - BT, a.E - 1);
        off[q] = (uint32_t)src * (uint32_t)a.d * 2u + cb;
    }
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);
    auto issue = [&](int kt, int stage) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int i = wave + kRWaves * q;
            if (i < NI)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    isx[q] ? rx : rc, (lds_ptr_t)(uintptr_t)(lds0 + stage * L::STAGE + i * 1024), 16,
                    (int)off[q], kt * 128, 0, 0);
        }
    };

    // this wave's share of the products: token blocks tb0 .. tb0 + TBW - 1
    // of 32, expert group eg of 64; waves 0-3, one per SIMD
    constexpr int TBW = (BT == 64 && NE >= 3) ? 2 : 1;
    const int eg = (BT == 64 && TBW == 1) ? wave % NE : wave;
    const int tb0 = (BT == 64 && TBW == 1) ? wave / NE : 0;
    const bool active = BT == 64 ? (TBW == 2 ? wave < NE : wave < 2 * NE) : wave < NE;
    const int lrow32 = lane & 31, lrow16 = lane & 15;
    // BT 64: acc32[b][j] 32x32 blocks (tokens 32 (tb0 + b).., experts 64 eg + 32 j..)
    // BT 16: acc16[j] 16x16 blocks (tokens 0..15, experts 64 eg + 16 j..)
    f32x16 acc32[TBW][2];
    f32x4_t acc16[4];
#pragma unroll
    for (int b = 0; b < TBW; ++b)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc32[b][j] = f32x16{};
#pragma unroll
    for (int j = 0; j < 4; ++j) acc16[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int stage) {
        const lds_bf16_t* sx = (const lds_bf16_t*)smem + stage * (L::STAGE / 2);
        const lds_bf16_t* sc = sx + BT * 64;
        if (BT == 64) {
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int c = 2 * st + (lane >> 5);
                bf16x8 fa[TBW], fb[2];
#pragma unroll
                for (int b = 0; b < TBW; ++b)
                    fa[b] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
                        sx + swz(32 * (tb0 + b) + lrow32, c));
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    fb[j] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
                        sc + swz(64 * eg + 32 * j + lrow32, c));
#pragma unroll
                for (int b = 0; b < TBW; ++b)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc32[b][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[b], fb[j], acc32[b][j], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int c = 4 * kk + (lane >> 4);
                const bf16x8 fa = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
                    sx + swz(lrow16, c));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bf16x8 fb = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
                        sc + swz(64 * eg + 16 * j + lrow16, c));
                    acc16[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, acc16[j], 0, 0, 0);
                }
            }
        }
    };

    // this wave's loads of slice kt have landed once no more than those of
    // the `ahead` later slices in flight remain outstanding (loads count
    // down in issue order)
    const bool more = wave < NI % kRWaves;             // LMIN + 1 loads per slice
    auto wait_slice = [&](int ahead) {
        switch (ahead) {
            case 0: wait_vm<0>(); break;
#define MOE_WAIT_AHEAD(A) \
    case A: if (A < P) { if (more) wait_vm<(A < P ? A : 0) * NQ>(); else wait_vm<(A < P ? A : 0) * LMIN>(); } break;
            MOE_WAIT_AHEAD(1) MOE_WAIT_AHEAD(2) MOE_WAIT_AHEAD(3)
            MOE_WAIT_AHEAD(4) MOE_WAIT_AHEAD(5) MOE_WAIT_AHEAD(6)
#undef MOE_WAIT_AHEAD
            default: break;
        }
    };
    if (nloc > 0) {
        for (int s2 = 0; s2 < P && s2 < nloc; ++s2) issue(kb + s2, s2);
        for (int kt = 0; kt < nloc; ++kt) {
            wait_slice(min(P - 1, nloc - 1 - kt));
            // every wave's loads of slice kt landed; every wave is done with slice kt - 1
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            if (kt + P < nloc) issue(kb + kt + P, (kt + P) % SG);
            if (active) compute(kt % SG);
        }
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();

    // the tile's affinities: lane layout of the accumulators
    lds_float_t* lg = (lds_float_t*)smem;              // [BT][EP], reusing the stages
    auto for_each_acc = [&](auto&& f) {               // f(token in tile, expert, value)
        if (!active) return;
        if (BT == 64) {
#pragma unroll
            for (int b = 0; b < TBW; ++b)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        f(32 * (tb0 + b) + ((r >> 2) << 3) + ((lane >> 5) << 2) + (r & 3),
                          64 * eg + 32 * j + lrow32, acc32[b][j][r]);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) f(4 * (lane >> 4) + r, 64 * eg + 16 * j + lrow16, acc16[j][r]);
        }
    };
    if (a.S == 1) {
        for_each_acc([&](int tl, int e, float v) { lg[tl * EP + e] = v; });
    } else {
        // Partial of split z; the last workgroup of the tile to finish sums
        // them.  The partials pass between workgroups (and XCDs, each with
        // its own L2) as device-scope relaxed atomic stores and loads, which
        // the hardware writes through to, and reads from, the device-coherent
        // level: a fence would write back and invalidate the whole L2 of the
        // XCD instead, evicting the centroids every other workgroup there is
        // streaming.  Order: every store of this workgroup has completed
        // (vmcnt 0, then the barrier) before its ticket is taken, and the
        // last workgroup reads only after its ticket returned.
        float* pz = a.part + (size_t)z * a.T * a.Epad;
        for_each_acc([&](int tl, int e, float v) {
            if (t0 + tl < a.T)
                __hip_atomic_store(&pz[(size_t)(t0 + tl) * a.Epad + e], v, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        });
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0)
            s_last = __hip_atomic_fetch_add(&a.tickets[tile], 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) == a.S - 1;
        __syncthreads();
        if (!s_last) return;
        // 16-byte loads with the device-coherent policy (sc1, what a
        // device-scope relaxed atomic load uses), eight splits in flight at a
        // time, summed in split order whoever finished last
        const __amdgpu_buffer_rsrc_t rp =
            make_rsrc(a.part, (uint32_t)((size_t)a.S * a.T * a.Epad * 4));
        const uint32_t zstride = (uint32_t)a.T * (uint32_t)a.Epad * 4u;
        for (int i = tid; i < BT * EP / 4; i += kRThreads) {
            const int tl = i / (EP / 4), e = (i % (EP / 4)) * 4;
            f32x4_t s = {0.f, 0.f, 0.f, 0.f};
            if (t0 + tl < a.T) {
                const uint32_t base = ((uint32_t)(t0 + tl) * (uint32_t)a.Epad + (uint32_t)e) * 4u;
                for (int z0 = 0; z0 < a.S; z0 += 8) {
                    f32x4_t pz[8];
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        pz[q] = __builtin_bit_cast(
                            f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                         rp, (int)(base + (uint32_t)min(z0 + q, a.S - 1) * zstride), 0, 16));
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        if (z0 + q < a.S) s += pz[q];
                }
            }
            *reinterpret_cast<__attribute__((address_space(3))) f32x4_t*>(&lg[tl * EP + e]) = s;
        }
    }
    __syncthreads();

    // ---- 2. gate and top-K, one wavefront per token ----
    const bool sig = (a.flags & kGateSigmoid) != 0;
    const bool ren = (a.flags & kGateRenorm) != 0;
    const float NEG = -INFINITY;
    for (int tl = wave; tl < BT; tl += kRWaves) {
        const int t = t0 + tl;
        if (t >= a.T) {
            if (a.scores)                                 // rows past T add nothing to the sums
                for (int e = lane; e < EP; e += 64) lg[tl * EP + e] = 0.f;
            continue;
        }
        float v[NE], sc[NE];
        uint32_t u[NE];                 // selection keys, 0 once taken or past E
#pragma unroll
        for (int j = 0; j < NE; ++j) {
            const int e = lane + 64 * j;
            const float aff = lg[tl * EP + e];
            sc[j] = sig ? __builtin_amdgcn_rcpf(1.0f + __expf(-aff)) : 0.f;
            v[j] = e < a.E ? (sig ? sc[j] + bj[j] : aff + bj[j]) : NEG;
            u[j] = e < a.E ? max(key_of(v[j]), 1u) : 0u;   // (a NaN could map to 0)
        }
        // the largest key: the softmax shift (and the first pick)
        uint32_t m = wave_max_u32(lane_max(u));
        float g[NE];
        if (!sig) {                                      // softmax over the routed experts
            const float vmax = float_of_key(m);
            float ps = 0.f;
#pragma unroll
            for (int j = 0; j < NE; ++j) {
                g[j] = (lane + 64 * j < a.E) ? __expf(v[j] - vmax) : 0.f;
                ps += g[j];
            }
            const float rs = 1.0f / wave_sum(ps);
#pragma unroll
            for (int j = 0; j < NE; ++j) g[j] *= rs;
        } else {
#pragma unroll
            for (int j = 0; j < NE; ++j) g[j] = sc[j];
        }
        if (a.scores) {
#pragma unroll
            for (int j = 0; j < NE; ++j) {
                const int e = lane + 64 * j;
                const float sv = e < a.E ? g[j] : 0.f;
                a.scores[(size_t)t * a.Epad + e] = sv;
                lg[tl * EP + e] = sv;                     // this wave's row only
            }
        }
        // K rounds of a wavefront arg-max: round r takes the largest key
        // left (ties: the lowest expert id, the lowest block j first, then
        // the lowest lane) and gives it rank r.  The K gates are summed in
        // rank order for the renormalisation.
        int rank[NE];
#pragma unroll
        for (int j = 0; j < NE; ++j) rank[j] = -1;
        float zs = 0.f;
        for (int r = 0; r < a.K; ++r) {
            if (r > 0) m = wave_max_u32(lane_max(u));
            int js = -1, l = 0;
#pragma unroll
            for (int j = 0; j < NE; ++j) {
                const uint64_t b = __ballot(u[j] == m);
                if (js < 0 && b) { js = j; l = (int)__builtin_ctzll(b); }
            }
#pragma unroll
            for (int j = 0; j < NE; ++j) {
                if (j == js) {
                    zs += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g[j]), l));
                    if (lane == l) { rank[j] = r; u[j] = 0u; }
                }
            }
        }
        const float rz = ren ? 1.0f / zs : 1.0f;
#pragma unroll
        for (int j = 0; j < NE; ++j) {
            if (rank[j] >= 0) {
                const int e = lane + 64 * j;
                a.idx[(size_t)t * a.K + rank[j]] = e;
                a.gate[(size_t)t * a.K + rank[j]] = g[j] * rz;
                if (BT == 64) atomicOr(&smask[2 * e + (tl >> 5)], 1u << (tl & 31));
                else atomicOr(&smask[e], 1u << tl);
            }
        }
    }
    __syncthreads();

    // ---- 3. chunk masks (and, training, the score sums per 16 tokens) ----
    if (BT == 64) {
        for (int e = tid; e < EP; e += kRThreads)
            a.masks[(size_t)tile * a.Epad + e] = ((uint64_t)smask[2 * e + 1] << 32) | smask[2 * e];
    } else {
        uint16_t* m16 = reinterpret_cast<uint16_t*>(a.masks);
        for (int e = tid; e < EP; e += kRThreads)
            m16[((size_t)(tile >> 2) * a.Epad + e) * 4 + (tile & 3)] = (uint16_t)smask[e];
    }
    if (a.score_part) {
        for (int i = tid; i < (BT / 16) * EP; i += kRThreads) {
            const int q = i / EP, e = i % EP;
            float s = 0.f;
            for (int r = 0; r < 16; ++r) s += lg[(16 * q + r) * EP + e];
            a.score_part[((size_t)tile * (BT / 16) + q) * a.Epad + e] = s;
        }
    }
}

// (the body lives in a device function: kept in the kernel itself, with its
// lambdas and shared arrays, the host pass emitted no launch stub for it)
template <int BT, int NE>
__global__ __launch_bounds__(kRThreads) void router_fused_kernel(RouterArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[RouterLds<BT, NE>::BYTES];
    __shared__ unsigned smask[2 * 64 * NE];
    __shared__ int s_last;
    router_tile<BT, NE>(a, (lds_char_t*)smem, smask, s_last);
}

__global__ void clear_tickets_kernel(int32_t* t, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) t[i] = 0;
}

template <int BT>
hipError_t launch_bt(const RouterArgs& a, int tiles, hipStream_t st) {
    const dim3 grid(tiles, a.S);
    switch (a.Epad / 64) {
        case 1: router_fused_kernel<BT, 1><<<grid, kRThreads, 0, st>>>(a); break;
        case 2: router_fused_kernel<BT, 2><<<grid, kRThreads, 0, st>>>(a); break;
        case 3: router_fused_kernel<BT, 3><<<grid, kRThreads, 0, st>>>(a); break;
        default: router_fused_kernel<BT, 4><<<grid, kRThreads, 0, st>>>(a); break;
    }
    return hipGetLastError();
}

}  // namespace

int router_tiles(const Plan& p) {
    // 16-token tiles cover every quarter chunk (the permutation reads all four
    // quarters of every chunk mask)
    return p.router_bt == 64 ? p.nchunk : p.nchunk * 4;
}

hipError_t launch_router_tickets(const Plan& p, hipStream_t st) {
    if (p.split <= 1) return hipSuccess;
    clear_tickets_kernel<<<1, 256, 0, st>>>(p.tickets, router_tiles(p));
    return hipGetLastError();
}

hipError_t launch_router(const Plan& p, const bf16_t* x, const bf16_t* C, const float* bias,
                         hipStream_t st) {
    RouterArgs a;
    a.x = x;
    a.C = C;
    a.bias = bias;
    a.T = p.T;
    a.d = p.d;
    a.E = p.E;
    a.Epad = p.Epad;
    a.K = p.K;
    a.S = p.split;
    a.kps = p.kps;
    a.flags = p.flags;
    a.part = p.logits;
    a.tickets = p.tickets;
    a.idx = p.idx;
    a.gate = p.gate;
    a.masks = p.masks;
    a.scores = p.scores;
    a.score_part = p.score_part;
    return p.router_bt == 64 ? launch_bt<64>(a, router_tiles(p), st)
                             : launch_bt<16>(a, router_tiles(p), st);
}

}  // namespace moe
