// Router: token-to-centroid affinities, softmax and top-K selection.
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
// Two kernels:
//   router_logits  bf16 MFMA GEMM x[T,d] . C[E,d]^T -> fp32 partial logits.
//                  Tiles of 64 tokens x 64 experts; for small T the d range is
//                  split so that the launch still covers the chip, and the
//                  partials are summed in a fixed order by the next kernel.
//   router_select  one wavefront per token (16 per workgroup): sum partials,
//                  then the gate — softmax of logit + bias (default), or
//                  sigmoid of the affinity with the bias added to the
//                  selection key only — and K rounds of a wavefront arg-max
//                  over the E<=256 keys (4 per lane; ties go to the lower
//                  expert id); optionally the K gates are renormalised to sum
//                  to one.  Per expert it also records the 64-bit
//                  mask of the tokens of each 64-token chunk that chose that
//                  expert; the permutation step turns those masks into a
//                  stable, atomics-free grouping of tokens by expert.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// 64 rows x 64 bf16 of a row-major tile, one 16-byte chunk per (row, c),
// stored at chunk position c ^ ((row >> 1) & 7).  LDS serves 16 lanes x 16
// bytes per cycle; an MFMA fragment read puts 16 lanes on 16 consecutive
// rows at one logical chunk, and with 128-byte rows those 16 reads then
// land in 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row, int chunk) {
    return row * 64 + ((chunk ^ ((row >> 1) & 7)) << 3);
}

__global__ __launch_bounds__(kThreads) void router_logits_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ C, float* __restrict__ logits,
    int T, int d, int E, int Epad, int ksteps_per_split) {
    __shared__ __attribute__((aligned(16))) bf16_t sA[2][kRouterBT * 64];
    __shared__ __attribute__((aligned(16))) bf16_t sB[2][kRouterBE * 64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int t0 = blockIdx.x * kRouterBT;
    const int e0 = blockIdx.y * kRouterBE;
    const int split = blockIdx.z;
    const int nk = d >> 6;
    const int k_begin = split * ksteps_per_split;
    const int k_end = min(nk, k_begin + ksteps_per_split);

    // each thread moves 2 chunks of A and 2 of B per 64-wide k step
    const int ch = tid & 7;
    const bf16_t* pa[2];
    const bf16_t* pb[2];
    bool bvalid[2];
    int rrow[2];
    for (int i = 0; i < 2; ++i) {
        const int r = (tid >> 3) + 32 * i;
        rrow[i] = r;
        const int t = min(t0 + r, T - 1);
        pa[i] = x + (size_t)t * d + ch * 8;
        const int e = e0 + r;
        bvalid[i] = e < E;
        pb[i] = C + (size_t)(bvalid[i] ? e : 0) * d + ch * 8;
    }

    f32x16 acc = {};
    u32x4 ra[2], rb[2];
    auto gload = [&](int kt) {
        for (int i = 0; i < 2; ++i) {
            ra[i] = *reinterpret_cast<const u32x4*>(pa[i] + (size_t)kt * 64);
            rb[i] = bvalid[i] ? *reinterpret_cast<const u32x4*>(pb[i] + (size_t)kt * 64)
                              : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto sstore = [&](int buf) {
        for (int i = 0; i < 2; ++i) {
            *reinterpret_cast<u32x4*>(&sA[buf][swz(rrow[i], ch)]) = ra[i];
            *reinterpret_cast<u32x4*>(&sB[buf][swz(rrow[i], ch)]) = rb[i];
        }
    };

    if (k_begin < k_end) {
        gload(k_begin);
        sstore(0);
        __syncthreads();
        for (int kt = k_begin; kt < k_end; ++kt) {
            const int buf = (kt - k_begin) & 1;
            if (kt + 1 < k_end) gload(kt + 1);
            const int arow = wm * 32 + (lane & 31);
            const int brow = wn * 32 + (lane & 31);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int c = 2 * s + (lane >> 5);
                bf16x8 a = *reinterpret_cast<const bf16x8*>(&sA[buf][swz(arow, c)]);
                bf16x8 b = *reinterpret_cast<const bf16x8*>(&sB[buf][swz(brow, c)]);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
            }
            if (kt + 1 < k_end) sstore(buf ^ 1);
            __syncthreads();
        }
    }

    // 32x32 accumulator: lane holds column (lane & 31), rows
    // 8*(r/4) + 4*(lane/32) + (r%4) for r = 0..15.
    const int col = e0 + wn * 32 + (lane & 31);
    float* outp = logits + (size_t)split * T * Epad;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = t0 + wm * 32 + ((r >> 2) << 3) + ((lane >> 5) << 2) + (r & 3);
        if (row < T) outp[(size_t)row * Epad + col] = acc[r];
    }
}

__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// One wavefront per token: a workgroup of 16 waves takes 16 consecutive
// tokens, a quarter of a 64-token chunk, and writes that quarter's 16 bits
// of every expert's chunk mask (a 16-bit store into the 64-bit word, so the
// four workgroups of a chunk write disjoint bytes and no mask needs clearing
// first; quarters past T write zeros).
constexpr int kSelectWaves = 16;
constexpr int kSelectThreads = 64 * kSelectWaves;
constexpr int kSubChunks = kChunk / kSelectWaves;
static_assert(kSubChunks == 4, "16-bit quarters of the 64-bit chunk mask");
constexpr int kPartBatch = 8;       // partial logits loaded ahead of their adds

__device__ __forceinline__ float pick4(const float (&a)[4], int j) {
    return j == 0 ? a[0] : j == 1 ? a[1] : j == 2 ? a[2] : a[3];
}

__global__ __launch_bounds__(kSelectThreads) void router_select_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int32_t* __restrict__ idx,
    float* __restrict__ gate, uint64_t* __restrict__ masks, int T, int E, int Epad, int K,
    int split, uint32_t flags) {
    __shared__ unsigned smask[256];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c = blockIdx.x / kSubChunks;
    const int q = blockIdx.x % kSubChunks;
    const bool sig = (flags & kGateSigmoid) != 0;
    const bool ren = (flags & kGateRenorm) != 0;
    for (int e = tid; e < Epad; e += kSelectThreads) smask[e] = 0u;
    __syncthreads();

    const int tl = q * kSelectWaves + wave;          // token within the chunk
    const int t = c * kChunk + tl;
    if (t < T) {
        const float NEG = -INFINITY;
        // affinities of experts lane + 64 j: the split-K partials summed in
        // order z = 0, 1, ..., loaded kPartBatch at a time
        float v[4];
        int taken = 0;                               // bit j: expert lane + 64j is out
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[j] = 0.f;
            if (lane + 64 * j >= E) taken |= 1 << j;
        }
        const float* lp = logits + (size_t)t * Epad + lane;
        const size_t zstride = (size_t)T * Epad;
        for (int z0 = 0; z0 < split; z0 += kPartBatch) {
            float pv[kPartBatch][4];
#pragma unroll
            for (int b = 0; b < kPartBatch; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    pv[b][j] = (z0 + b < split && !((taken >> j) & 1))
                                   ? lp[(size_t)(z0 + b) * zstride + 64 * j] : 0.f;
#pragma unroll
            for (int b = 0; b < kPartBatch; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (z0 + b < split) v[j] += pv[b][j];
        }
        // selection keys: softmax gate -> logit + bias (the softmax is
        // monotone in it); sigmoid gate -> sigmoid(affinity) + bias, the bias
        // steering the choice only
        float sc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = lane + 64 * j;
            const float b = (bias && e < E) ? bias[e] : 0.f;
            sc[j] = sig ? 1.0f / (1.0f + expf(-v[j])) : 0.f;
            v[j] = e < E ? (sig ? sc[j] + b : v[j] + b) : NEG;
        }
        float mx = 0.f, sum = 1.f;
        if (!sig) {
            mx = wave_max(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
            float ps = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) ps += (lane + 64 * j < E) ? expf(v[j] - mx) : 0.f;
            sum = wave_sum(ps);
        }

        float gk[4] = {0.f, 0.f, 0.f, 0.f};          // renormalised: gate k kept by lane k % 64
        float zsum = 0.f;
        for (int k = 0; k < K; ++k) {
            // local best: strictly greater wins, so the lower j (lower e) keeps ties
            float bv = NEG;
            int be = 0x7fffffff;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (!((taken >> j) & 1) && (be == 0x7fffffff || v[j] > bv)) {
                    bv = v[j];
                    be = lane + 64 * j;
                }
            for (int o = 32; o > 0; o >>= 1) {
                const float ov = __shfl_xor(bv, o, 64);
                const int oe = __shfl_xor(be, o, 64);
                if (ov > bv || (ov == bv && oe < be)) {
                    bv = ov;
                    be = oe;
                }
            }
            if ((be & 63) == lane) taken |= 1 << (be >> 6);
            const float g = sig ? __shfl(pick4(sc, be >> 6), be & 63, 64) : expf(bv - mx) / sum;
            if (ren) {
                zsum += g;                           // every lane, in selection order
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if ((k & 63) == lane && (k >> 6) == j) gk[j] = g;
            }
            if (lane == 0) {
                idx[(size_t)t * K + k] = be;
                if (!ren) gate[(size_t)t * K + k] = g;
                atomicOr(&smask[be], 1u << wave);
            }
        }
        if (ren) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int k = 64 * j + lane;
                if (k < K) gate[(size_t)t * K + k] = gk[j] / zsum;
            }
        }
    }
    __syncthreads();
    uint16_t* m16 = reinterpret_cast<uint16_t*>(masks);
    for (int e = tid; e < Epad; e += kSelectThreads)
        m16[((size_t)c * Epad + e) * kSubChunks + q] = (uint16_t)smask[e];
}

}  // namespace

hipError_t launch_router_logits(const Plan& p, const bf16_t* x, const bf16_t* C, hipStream_t st) {
    const int nk = p.d / 64;
    const int kps = (nk + p.split - 1) / p.split;
    dim3 grid((p.T + kRouterBT - 1) / kRouterBT, p.Epad / kRouterBE, p.split);
    router_logits_kernel<<<grid, kThreads, 0, st>>>(x, C, p.logits, p.T, p.d, p.E, p.Epad, kps);
    return hipGetLastError();
}

hipError_t launch_router_select(const Plan& p, const float* bias, hipStream_t st) {
    router_select_kernel<<<p.nchunk * kSubChunks, kSelectThreads, 0, st>>>(
        p.logits, bias, p.idx, p.gate, p.masks, p.T, p.E, p.Epad, p.K, p.split, p.flags);
    return hipGetLastError();
}

}  // namespace moe
