// Shared definitions of the gfx950 MoE kernels: bf16 / MFMA vector types,
// the per-call plan (shape-derived sizes and the workspace carve-up) and the
// launchers each kernel file exports to the C-ABI dispatcher.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;                                   // bf16 bit pattern
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Buffer resource over [base, base + bytes) for the raw buffer loads: the
// base and size live in scalar registers and each lane supplies a 32-bit
// byte offset.  0x00020000 is the gfx9-family dword-3 value for untyped
// 32-bit data.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
}
// The same with the nontemporal (streaming) cache policy, for data read
// once: measured on MI355X, a pure stream reads HBM at about 7.1 TB/s this
// way against 6.3 TB/s with the default policy.
__device__ __forceinline__ u32x4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 2);
}

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even (gfx950's v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(bf16_t, (__bf16)f);
}

// Two fp32 -> two bf16 in one word, the first in the low half: one
// conversion instruction for the pair.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Tokens per routing chunk: one 64-bit lane mask per (chunk, expert).
constexpr int kChunk = 64;
constexpr uint32_t kGateRenorm = 2u;    // shape flag bits of the gating variants
constexpr uint32_t kGateSigmoid = 4u;
constexpr uint32_t kAct8 = 8u;         // 8-bit activations for the routed products
// Router: experts padded to a multiple of 64 (a wavefront's share).
constexpr int kRouterBE = 64;

// One entry of a grouped-GEMM work list.
struct Tile {
    int32_t group;   // 0..E-1 routed expert, E..E+Ks-1 shared expert
    int32_t m0;      // first row of the group covered by the tile
    int32_t n0;      // first output column
    int32_t nrows;   // rows of the group in this tile (<= BM)
};

// Grouped-GEMM tile configuration chosen per call.
struct GemmCfg {
    int bm, bn;      // rows, B-rows (output cols; for SwiGLU half W1, half W3)
};

// Everything a call needs, derived on the host from the shape.  Device
// pointers point into the caller's workspace.
struct Plan {
    int T, d, E, I, K, Ks, Is;
    uint32_t flags;
    int Epad;        // E rounded up to the router tile
    int nchunk;      // ceil(T / kChunk)
    int router_bt;   // router tile: 64 tokens (large batches) or 16
    int split;       // router: d range split this many ways (1: no partials)
    int kps;         //   slices of 64 per split
    int rows;        // T*K routed rows + T*Ks shared rows
    GemmCfg g1, g2;
    int max_tiles1, max_tiles2;

    // workspace carve-up (byte offsets while planning, then pointers)
    float* logits;       // [split, T, Epad] partial affinities (split > 1)
    int32_t* tickets;    // [router tiles] (split > 1)
    int32_t* idx;        // [T, K]
    float* gate;         // [T, K]
    uint64_t* masks;     // [nchunk, Epad]
    int32_t* chunk_base; // [nchunk, Epad]
    int32_t* goff;       // [E + Ks + 1] row offset of each group
    int32_t* toff;       // [2 (E + Ks + 1)] first work-list entry of each group, G1 then G2
    int32_t* tok_of;     // [rows] token of each permuted row
    int32_t* slot_of;    // [T, K] permuted row of each (token, k)
    Tile* tiles1;        // [max_tiles1]
    Tile* tiles2;        // [max_tiles2]
    int32_t* ntiles;     // [2]
    uint8_t* xq;         // 8-bit activations (MOE_FLAG_ACT8): codes [T, d]
    int32_t* xe;         //   their scale exponents [T]
    bf16_t* xd;          //   the dequantised rows [T, d] (batches off the FP8 tile only)
    uint8_t* hq;         // 8-bit activations of the routed rows of H: codes [T*K, I] and
    int32_t* he;         //   exponents [T*K] (FP8 down tiles only; else H is dequantised in place)
    bf16_t* H;           // routed [T*K, I] then shared [Ks*T, Is]
    bf16_t* Y;           // [rows, d]

    // training forward only (null otherwise): what the backward reads
    float* scores;       // [T, Epad] every expert's score (softmax / sigmoid), 0 past E
    float* score_part;   // [nchunk * 4, Epad] score sums of each 16-token quarter chunk
    float* row_gate;     // [T*K] gate of each routed row
    bf16_t* Z;           // pre-activations [W1 x | W3 x]: routed [T*K, 2I], shared [Ks*T, 2Is]
};

// 8-bit routed weights: E4M3 codes with one float scale per output row
// (q1, q3 [E, I, d] with s1, s3 [E, I]; q2 [E, d, I] with s2 [E, d]).
struct RoutedQ8 {
    const uint8_t *q1, *q3, *q2;
    const float *s1, *s3, *s2;
};

// Launchers (each enqueues on `st`; return the launch status).  q8 != null:
// the routed weights are 8-bit (the plan then uses the thin tiles).
int router_tiles(const Plan& p);
hipError_t launch_router_tickets(const Plan& p, hipStream_t st);
hipError_t launch_router(const Plan& p, const bf16_t* x, const bf16_t* C, const float* bias,
                         hipStream_t st);
hipError_t launch_perm_scan(const Plan& p, hipStream_t st);
hipError_t launch_perm_scatter(const Plan& p, hipStream_t st);
hipError_t launch_gemm_gate_up(const Plan& p, const bf16_t* x, const bf16_t* w1,
                               const bf16_t* w3, const bf16_t* ws1, const bf16_t* ws3,
                               const RoutedQ8* q8, hipStream_t st);
hipError_t launch_gemm_down(const Plan& p, const bf16_t* w2, const bf16_t* ws2,
                            const RoutedQ8* q8, hipStream_t st);
hipError_t launch_combine(const Plan& p, const bf16_t* x, bf16_t* out, hipStream_t st);
// MOE_FLAG_ACT8: the 8-bit activations of `rows` bf16 rows of width d
// (d a multiple of 8): codes [rows, d] and exponents [rows] (each may be
// null) and the dequantised rows (deq, may be null or equal to x)
hipError_t launch_act8_quant(const bf16_t* x, int rows, int d, uint8_t* codes, int32_t* exps,
                             bf16_t* deq, hipStream_t st);
// the FP8 tiles: 256-row tiles and a reduction length of whole 128-deep slices
inline bool f8_gate_up(const Plan& p) { return p.g1.bm == 256 && p.d % 128 == 0; }
inline bool f8_down(const Plan& p) { return p.g2.bm == 256 && p.I % 128 == 0; }
// training forward: balance statistics [2E + 1] = (f_e, P_e, L_bal) from the
// group offsets and the score sums
hipError_t launch_balance_stats(const Plan& p, float* stats, hipStream_t st);

// Backward (backward.hip).  The workspace carve-up of one backward call.
struct BwdPlan {
    int max_tiles_dh, max_tiles_dx;   // work-list bounds (256 x 256 tiles)
    int ndh;                          // dgate partials per row (N tiles of the dH GEMM)
    bf16_t* dZ;       // like Plan::Z
    bf16_t* gH;       // [T*K, I]
    float* dgp;       // [rows, ndh]
    bf16_t* dL;       // [T, Epad]
    float* R32;       // [T, d]
    bf16_t* dXr;      // [rows, d]
    Tile* tiles_dh;
    Tile* tiles_dx;
    int32_t* ntiles;  // [2]
    int32_t* gorder;  // [E + Ks]
    float* dgate;     // [T, K] when the caller passes none
};
struct BwdArgs {
    const bf16_t *x, *C, *w1, *w3, *w2, *ws1, *ws3, *ws2, *dout;
    float alpha;
    bf16_t *dx, *dw1, *dw3, *dw2, *dws1, *dws3, *dws2;
    float *dC, *dgate;
};
hipError_t launch_backward(const Plan& p, const BwdPlan& b, const BwdArgs& a, hipStream_t st,
                           void (*mark)(int slot, int end, hipStream_t s));
hipError_t launch_stream_read(const void* buf, size_t bytes, hipStream_t st);

}  // namespace moe
