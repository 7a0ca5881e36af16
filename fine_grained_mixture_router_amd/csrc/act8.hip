// 8-bit activations for the routed products (MOE_FLAG_ACT8): the token rows
// x before W1 / W3, the routed rows of h (bf16) before W2.
//
// Each row gets the scale 2^e, e the smallest integer with
// max_j |x_j| <= 448 * 2^e (448: the largest finite E4M3 value; e = 0 for an
// all-zero row), and the codes are the nearest E4M3 values of x * 2^-e, ties
// to the even code.  The pages only advise low-bit routed experts with
// per-channel or per-group scales (eliteato DeepSeek-V2 explainer, section
// 5.5); a power-of-two per-row scale makes x * 2^-e exact, so the codes
// depend on nothing but round-to-nearest-even, which the hardware conversion
// (v_cvt_pk_fp8_f32) performs.
//
// e from the row maximum a = f * 2^E2, f in [0.5, 1) (frexp, exact):
// a <= 448 * 2^e = 0.875 * 2^(9 + e) holds for e = E2 - 9 when f <= 0.875 and
// needs e = E2 - 8 otherwise; one less never holds (f >= 0.5 > 0.4375).
//
// One wave per row: the row maximum over 16-byte pieces (a wavefront
// reduction), then the codes, eight per 64-bit store, and where the FP8
// tiles do not apply (decode-size tiles, or a reduction length that is not
// a multiple of their 128-deep slices) the dequantised row in bf16 (exact:
// an E4M3 value times a power of two fits bf16's 8-bit significand).  The dequantised row may overwrite the input:
// each lane writes only the pieces it has itself read, after the wave-wide
// maximum (and so every read of the first pass) is complete.
#include "common.h"

namespace moe {
namespace {

constexpr int kQThreads = 256;

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// One wave per row, kQRows rows per workgroup; a lane keeps up to kQHold of
// its row's 16-byte pieces in registers between the two passes, so rows of
// up to 64 * kQHold * 8 values are read from memory once.
constexpr int kQRows = kQThreads / 64;
constexpr int kQHold = 8;

__device__ __forceinline__ float piece_max(const u32x4 p, float m) {
    const uint32_t u[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(u[i])), fabsf(bf16_hi(u[i]))));
    return m;
}

__device__ __forceinline__ void quant_piece(const u32x4 p, int e, uint32_t* qrow, u32x4* drow, int v) {
    const uint32_t u[4] = {p.x, p.y, p.z, p.w};
    float y[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        y[2 * i] = ldexpf(bf16_lo(u[i]), -e);       // exact: a power-of-two rescale
        y[2 * i + 1] = ldexpf(bf16_hi(u[i]), -e);
    }
    uint32_t c[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * h], y[4 * h + 1], 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * h + 2], y[4 * h + 3], w, true);
        c[h] = (uint32_t)w;
    }
    if (qrow) *reinterpret_cast<u32x2*>(qrow + 2 * v) = u32x2{c[0], c[1]};
    if (drow) {
        uint32_t o[4];
        typedef float f32x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // two codes at a time -> two floats (exact), times 2^e, to bf16 (exact)
            const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[h], false);
            const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[h], true);
            o[2 * h] = pack_bf16x2(ldexpf(lo.x, e), ldexpf(lo.y, e));
            o[2 * h + 1] = pack_bf16x2(ldexpf(hi.x, e), ldexpf(hi.y, e));
        }
        drow[v] = u32x4{o[0], o[1], o[2], o[3]};
    }
}

__global__ __launch_bounds__(kQThreads) void act8_quant_kernel(const bf16_t* x, int rows, int d,
                                                               uint8_t* __restrict__ xq,
                                                               int32_t* __restrict__ xe,
                                                               bf16_t* xd) {
    const int t = blockIdx.x * kQRows + (int)(threadIdx.x >> 6);   // wave-uniform
    if (t >= rows) return;
    const int lane = threadIdx.x & 63;
    const u32x4* row = reinterpret_cast<const u32x4*>(x + (size_t)t * d);
    const int nv = d >> 3;                          // 16-byte pieces (8 values)
    u32x4 held[kQHold];
#pragma unroll
    for (int j = 0; j < kQHold; ++j) {
        const int v = lane + 64 * j;
        held[j] = v < nv ? row[v] : u32x4{0u, 0u, 0u, 0u};
    }
    float amax = 0.f;
    for (int v = lane + 64 * kQHold; v < nv; v += 64) amax = piece_max(row[v], amax);
#pragma unroll
    for (int j = 0; j < kQHold; ++j) amax = piece_max(held[j], amax);
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    int e = 0;
    if (amax > 0.f) {
        int e2;
        const float f = frexpf(amax, &e2);
        e = e2 - 9 + (f > 0.875f ? 1 : 0);
    }
    if (xe && lane == 0) xe[t] = e;
    uint32_t* qrow = xq ? reinterpret_cast<uint32_t*>(xq + (size_t)t * d) : nullptr;
    u32x4* drow = xd ? reinterpret_cast<u32x4*>(xd + (size_t)t * d) : nullptr;
#pragma unroll
    for (int j = 0; j < kQHold; ++j) {
        const int v = lane + 64 * j;
        if (v < nv) quant_piece(held[j], e, qrow, drow, v);
    }
    for (int v = lane + 64 * kQHold; v < nv; v += 64) quant_piece(row[v], e, qrow, drow, v);
}

}  // namespace

hipError_t launch_act8_quant(const bf16_t* x, int rows, int d, uint8_t* codes, int32_t* exps,
                             bf16_t* deq, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    if (d % 8) return hipErrorInvalidValue;
    act8_quant_kernel<<<(rows + kQRows - 1) / kQRows, kQThreads, 0, st>>>(x, rows, d, codes, exps, deq);
    return hipGetLastError();
}

}  // namespace moe
