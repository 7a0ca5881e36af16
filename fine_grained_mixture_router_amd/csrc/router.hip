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
//                  Tiles of 64 tokens x all experts; for small T the d range
//                  is split so that the launch still covers the chip, and the
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

// Rows of 64 bf16 (one BK = 64 slice), one 16-byte chunk per (row, c),
// chunk c stored at position c ^ ((row >> 1) & 7).  LDS serves 16 lanes x
// 16 bytes per cycle; an MFMA fragment read puts 16 lanes on 16 consecutive
// rows at one logical chunk, and with 128-byte rows those 16 reads then
// land in 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row, int chunk) {
    return row * 64 + ((chunk ^ ((row >> 1) & 7)) << 3);
}

// Affinities x . C^T for a tile of kRouterBT = 64 tokens and all Epad (<= 256)
// experts, over the d range of split blockIdx.y, written as fp32 partials
// [split, T, Epad].  A tile reads its token rows once and the centroids from
// L2 (at most 3.7 MB, shared by every tile).  Four waves; wave w computes
// experts 64 w .. 64 w + 63 for all 64 tokens (2 x 2 MFMA 32x32x16 blocks).
// Slices of BK = 64 are staged through registers into a double buffer.
constexpr int kRouterThreads = 256;
constexpr int kRouterMaxE = 256;

__global__ __launch_bounds__(kRouterThreads) void router_logits_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ C, float* __restrict__ logits,
    int T, int d, int E, int Epad, int ksteps_per_split) {
    __shared__ __attribute__((aligned(16))) bf16_t sA[2][kRouterBT * 64];
    __shared__ __attribute__((aligned(16))) bf16_t sB[2][kRouterMaxE * 64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int t0 = blockIdx.x * kRouterBT;
    const int split = blockIdx.y;
    const int nk = d >> 6;
    const int k_begin = split * ksteps_per_split;
    const int k_end = min(nk, k_begin + ksteps_per_split);
    const int nbl = Epad / 32;                     // B chunks per thread per slice (<= 8)
    const bool active = 64 * wave < Epad;          // this wave's experts exist

    // loads: thread moves chunk ch of token rows srow + 32 i and of centroid
    // rows srow + 32 i; rows past T or E are clamped to the last one (their
    // results are never read)
    const int ch = tid & 7;
    const int srow = tid >> 3;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)T * (uint32_t)d * 2u);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(C, (uint32_t)E * (uint32_t)d * 2u);
    uint32_t aoff[2], boff[8];
#pragma unroll
    for (int i = 0; i < 2; ++i)
        aoff[i] = ((uint32_t)min(t0 + srow + 32 * i, T - 1) * (uint32_t)d + ch * 8) * 2u;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        boff[i] = ((uint32_t)min(srow + 32 * i, E - 1) * (uint32_t)d + ch * 8) * 2u;
    const int sx = swz(srow, ch);                  // rows srow + 32 i share the swizzle

    u32x4 ra[2], rb[8];
    auto gload = [&](int kt) {
        const uint32_t kb = (uint32_t)kt * 128u;
#pragma unroll
        for (int i = 0; i < 2; ++i) ra[i] = buf_load16(rx, aoff[i], kb);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < nbl) rb[i] = buf_load16(rc, boff[i], kb);
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4*>(&sA[buf][sx + 32 * i * 64]) = ra[i];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < nbl) *reinterpret_cast<u32x4*>(&sB[buf][sx + 32 * i * 64]) = rb[i];
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    const int lrow = lane & 31;
    if (k_begin < k_end) {
        gload(k_begin);
        sstore(0);
        __syncthreads();
        for (int kt = k_begin; kt < k_end; ++kt) {
            const int buf = (kt - k_begin) & 1;
            const bool more = kt + 1 < k_end;
            if (more) gload(kt + 1);
            if (active) {
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    const int c = 2 * st + (lane >> 5);
                    bf16x8 a[2], b[2];
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        a[i] = *reinterpret_cast<const bf16x8*>(&sA[buf][swz(32 * i + lrow, c)]);
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        b[j] = *reinterpret_cast<const bf16x8*>(&sB[buf][swz(64 * wave + 32 * j + lrow, c)]);
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int j = 0; j < 2; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
                }
            }
            if (more) sstore(buf ^ 1);
            __syncthreads();
        }
    }

    // 32x32 accumulator: lane holds column (lane & 31) = expert, rows (tokens)
    // 8*(r/4) + 4*(lane/32) + (r%4) for r = 0..15.
    if (!active) return;
    float* outp = logits + (size_t)split * T * Epad;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = 64 * wave + 32 * j + lrow;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = t0 + 32 * i + ((r >> 2) << 3) + ((lane >> 5) << 2) + (r & 3);
                if (row < T) outp[(size_t)row * Epad + col] = acc[i][j][r];
            }
        }
}

// The same affinities for large batches: tiles of kRouterWideT = 256 tokens
// by all Epad (<= 256) experts, so the centroids are re-read once per 256
// tokens rather than per 64 (with 64-token tiles the loads, not the MFMAs,
// bound the kernel: 40 KB of operands per 512 MFMA cycles of a workgroup).
// Eight waves, wave (wm, wn) computing tokens 128 wm .. + 127 by experts
// 64 wn .. + 63 (4 x 2 MFMA 32x32x16 blocks); BK = 64 slices come in by
// direct-to-LDS buffer loads (one wave instruction fills 8 rows x 128 B)
// into two LDS stages, swizzled as in swz(); the refill of a stage is
// issued right after the barrier that ends its reads, a whole stage ahead
// of its use.
constexpr int kRouterWideThreads = 512;

__global__ __launch_bounds__(kRouterWideThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void router_logits_wide_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ C,
                               float* __restrict__ logits, int T, int d, int E, int Epad,
                               int ksteps_per_split) {
    constexpr int OPER = kRouterWideT * 64;        // elements of one operand slice
    constexpr int QI = 4;                          // load instructions per wave per operand
    __shared__ __attribute__((aligned(1024))) bf16_t smem[2 * 2 * OPER];
    typedef __attribute__((address_space(3))) void* lds_ptr_t;
    typedef __attribute__((address_space(3))) bf16_t lds_bf16_t;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int t0 = blockIdx.x * kRouterWideT;
    const int nk = d >> 6;
    const int k_begin = blockIdx.y * ksteps_per_split;
    const int k_end = min(nk, k_begin + ksteps_per_split);
    const bool active = 64 * wn < Epad;            // this wave's experts exist

    // Load instruction j = wave + 8 q fills rows 8 j .. 8 j + 7 of a slice;
    // lane l fills chunk position l % 8 of row 8 j + l / 8.  Rows past T or
    // E are clamped to the last one (their results are never read).
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)T * (uint32_t)d * 2u);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(C, (uint32_t)E * (uint32_t)d * 2u);
    uint32_t aoff[QI], boff[QI];
#pragma unroll
    for (int q = 0; q < QI; ++q) {
        const int row = 8 * (wave + 8 * q) + (lane >> 3);
        const uint32_t cb = (uint32_t)(((lane & 7) ^ ((row >> 1) & 7)) * 16);
        aoff[q] = (uint32_t)min(t0 + row, T - 1) * (uint32_t)d * 2u + cb;
        boff[q] = (uint32_t)min(row, E - 1) * (uint32_t)d * 2u + cb;
    }
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem + (uint32_t)(wave * 1024));
    auto issue = [&](int kt, int buf) {
        const uint32_t sa = lds_base + (uint32_t)(buf * 2 * OPER * 2);
        const int kb = kt * 128;
#pragma unroll
        for (int q = 0; q < QI; ++q) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)(uintptr_t)(sa + q * 8 * 1024), 16,
                                                     (int)aoff[q], kb, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (lds_ptr_t)(uintptr_t)(sa + OPER * 2 + q * 8 * 1024),
                                                     16, (int)boff[q], kb, 0, 0);
        }
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    const int lrow = lane & 31;
    const lds_bf16_t* lsm = (const lds_bf16_t*)smem;
    if (k_begin < k_end) {
        issue(k_begin, 0);
        if (k_begin + 1 < k_end) {
            issue(k_begin + 1, 1);
            asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        asm volatile("s_barrier" ::: "memory");
        for (int kt = k_begin; kt < k_end; ++kt) {
            const int buf = (kt - k_begin) & 1;
            const lds_bf16_t* sa = lsm + buf * 2 * OPER;
            const lds_bf16_t* sb = sa + OPER;
            if (active) {
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    const int c = 2 * st + (lane >> 5);
                    bf16x8 a[4], b[2];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        a[i] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(sa + swz(128 * wm + 32 * i + lrow, c));
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        b[j] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(sb + swz(64 * wn + 32 * j + lrow, c));
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 2; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
                }
            }
            // the next slice landed; every wave is done reading this one
            if (kt + 1 < k_end) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            if (kt + 2 < k_end) issue(kt + 2, buf);
        }
    }

    // 32x32 accumulator: lane holds column (lane & 31) = expert, rows (tokens)
    // 8*(r/4) + 4*(lane/32) + (r%4) for r = 0..15.
    if (!active) return;
    float* outp = logits + (size_t)blockIdx.y * T * Epad;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = 64 * wn + 32 * j + lrow;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = t0 + 128 * wm + 32 * i + ((r >> 2) << 3) + ((lane >> 5) << 2) + (r & 3);
                if (row < T && col < Epad) outp[(size_t)row * Epad + col] = acc[i][j][r];
            }
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

// scores / score_part (training forward only, else null): every expert's
// score of every token, and the sums of those scores over each workgroup's
// 16 tokens, taken in token order (the mean-score statistic of the
// expert-level balance loss is their sum over workgroups, in order).
__global__ __launch_bounds__(kSelectThreads) void router_select_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int32_t* __restrict__ idx,
    float* __restrict__ gate, uint64_t* __restrict__ masks, int T, int E, int Epad, int K,
    int split, uint32_t flags, float* __restrict__ scores, float* __restrict__ score_part) {
    __shared__ unsigned smask[256];
    __shared__ float sscore[kSelectWaves][256];
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
        if (scores) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = lane + 64 * j;
                if (e < Epad) {
                    const float sv = e < E ? (sig ? sc[j] : expf(v[j] - mx) / sum) : 0.f;
                    scores[(size_t)t * Epad + e] = sv;
                    sscore[wave][e] = sv;
                }
            }
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
    if (scores && t >= T)
        for (int e = lane; e < Epad; e += 64) sscore[wave][e] = 0.f;
    __syncthreads();
    if (score_part)
        for (int e = tid; e < Epad; e += kSelectThreads) {
            float acc = 0.f;
            for (int w = 0; w < kSelectWaves; ++w) acc += sscore[w][e];
            score_part[(size_t)blockIdx.x * Epad + e] = acc;
        }
    uint16_t* m16 = reinterpret_cast<uint16_t*>(masks);
    for (int e = tid; e < Epad; e += kSelectThreads)
        m16[((size_t)c * Epad + e) * kSubChunks + q] = (uint16_t)smask[e];
}

}  // namespace

hipError_t launch_router_logits(const Plan& p, const bf16_t* x, const bf16_t* C, hipStream_t st) {
    const int nk = p.d / 64;
    const int kps = (nk + p.split - 1) / p.split;
    if (p.router_wide) {
        dim3 grid((p.T + kRouterWideT - 1) / kRouterWideT, p.split);
        router_logits_wide_kernel<<<grid, kRouterWideThreads, 0, st>>>(x, C, p.logits, p.T, p.d, p.E,
                                                                       p.Epad, kps);
    } else {
        dim3 grid((p.T + kRouterBT - 1) / kRouterBT, p.split);
        router_logits_kernel<<<grid, kRouterThreads, 0, st>>>(x, C, p.logits, p.T, p.d, p.E, p.Epad, kps);
    }
    return hipGetLastError();
}

hipError_t launch_router_select(const Plan& p, const float* bias, hipStream_t st) {
    router_select_kernel<<<p.nchunk * kSubChunks, kSelectThreads, 0, st>>>(
        p.logits, bias, p.idx, p.gate, p.masks, p.T, p.E, p.Epad, p.K, p.split, p.flags,
        p.scores, p.score_part);
    return hipGetLastError();
}

}  // namespace moe
