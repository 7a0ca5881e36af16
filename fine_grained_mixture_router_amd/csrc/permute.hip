// Permutation: group the (token, k) assignments by expert, in token order,
// and build the work lists of the two grouped GEMMs.
//
// The pages' remark that a real implementation gathers tokens per expert
// after the top-K instead of looping over every expert (eliteato.com
// DeepSeek-V2 explainer, section 3.1) is what this step does.  It is exact
// integer work and deterministic: ranks come from popcounts of the per-chunk
// lane masks the router wrote, never from the order of atomics.
//
// Row space of the grouped GEMMs ("groups"):
//   groups 0..E-1      routed experts, n_e rows each, stable by token
//   groups E..E+Ks-1   shared experts, T rows each, row r is token r
// goff[g] is the first row of group g; routed rows total T*K.
#include "common.h"

namespace moe {
namespace {

constexpr int kScanThreads = 512;   // >= E + Ks (E <= 256, Ks <= 16)
constexpr int kGroupM = 4;          // M-tiles per N sweep in the work-list order

__device__ int block_exclusive_scan(int v, int* sbuf, int* total) {
    const int tid = threadIdx.x;
    sbuf[tid] = v;
    __syncthreads();
    for (int o = 1; o < kScanThreads; o <<= 1) {
        int add = tid >= o ? sbuf[tid - o] : 0;
        __syncthreads();
        sbuf[tid] += add;
        __syncthreads();
    }
    const int incl = sbuf[tid];
    *total = sbuf[kScanThreads - 1];
    __syncthreads();
    return incl - v;
}

// Writes the tiles of one group in "kGroupM M-tiles x all N-tiles" blocks:
// consecutive entries share either the A rows or the weight rows, which is
// what keeps the L2 of one XCD warm (each XCD takes a contiguous slice of
// the list, see the GEMM kernel).
__device__ void emit_tiles(Tile* out, int base, int g, int nrows_g, int bm, int ncols, int bn_out,
                           int tid, int nthr) {
    const int mt = (nrows_g + bm - 1) / bm;
    const int nt = (ncols + bn_out - 1) / bn_out;
    const int total = mt * nt;
    for (int i = tid; i < total; i += nthr) {
        const int b = i / (kGroupM * nt);
        const int j = i - b * kGroupM * nt;
        const int gm = min(kGroupM, mt - b * kGroupM);
        const int n = j / gm;
        const int m = b * kGroupM + (j - n * gm);
        Tile t;
        t.group = g;
        t.m0 = m * bm;
        t.n0 = n * bn_out;
        t.nrows = min(bm, nrows_g - m * bm);
        out[base + i] = t;
    }
}

__global__ __launch_bounds__(kScanThreads) void perm_scan_kernel(Plan p, int routed) {
    __shared__ int sbuf[kScanThreads];
    __shared__ int s_cnt[kScanThreads];
    __shared__ int s_t1[kScanThreads];
    __shared__ int s_t2[kScanThreads];
    const int tid = threadIdx.x;
    const int G = p.E + p.Ks;

    // rows per group
    int cnt = 0;
    if (tid < p.E && routed) {
        for (int c = 0; c < p.nchunk; ++c) cnt += __popcll(p.masks[(size_t)c * p.Epad + tid]);
    } else if (tid >= p.E && tid < G) {
        cnt = p.T;
    }
    int total;
    const int off = block_exclusive_scan(cnt, sbuf, &total);
    if (tid < G) {
        p.goff[tid] = off;
        s_cnt[tid] = cnt;
    }
    if (tid == 0) p.goff[G] = total;

    // per-(chunk, expert) first row
    if (tid < p.E && routed) {
        int run = off;
        for (int c = 0; c < p.nchunk; ++c) {
            p.chunk_base[(size_t)c * p.Epad + tid] = run;
            run += __popcll(p.masks[(size_t)c * p.Epad + tid]);
        }
    }

    // work-list sizes
    const int bn1 = p.g1.bn / 2;   // SwiGLU tile: half W1 rows, half W3 rows
    int t1 = 0, t2 = 0;
    if (tid < G) {
        const int n1 = tid < p.E ? p.I : p.Is;
        t1 = ((cnt + p.g1.bm - 1) / p.g1.bm) * ((n1 + bn1 - 1) / bn1);
        t2 = ((cnt + p.g2.bm - 1) / p.g2.bm) * ((p.d + p.g2.bn - 1) / p.g2.bn);
    }
    int tot1, tot2;
    const int o1 = block_exclusive_scan(t1, sbuf, &tot1);
    const int o2 = block_exclusive_scan(t2, sbuf, &tot2);
    if (tid < G) {
        s_t1[tid] = o1;
        s_t2[tid] = o2;
    }
    if (tid == 0) {
        p.ntiles[0] = tot1;
        p.ntiles[1] = tot2;
    }
    __syncthreads();

    for (int g = 0; g < G; ++g) {
        const int n = s_cnt[g];
        if (n == 0) continue;
        emit_tiles(p.tiles1, s_t1[g], g, n, p.g1.bm, g < p.E ? p.I : p.Is, bn1, tid, kScanThreads);
        emit_tiles(p.tiles2, s_t2[g], g, n, p.g2.bm, p.d, p.g2.bn, tid, kScanThreads);
    }
}

// One workgroup per 64-token chunk: slot of every (token, k) and the token of
// every permuted row (routed rows by expert, then the shared rows).
__global__ __launch_bounds__(256) void perm_scatter_kernel(Plan p, int routed) {
    const int c = blockIdx.x;
    const int t0 = c * kChunk;
    const int nt = min(kChunk, p.T - t0);
    if (routed) {
        for (int i = threadIdx.x; i < nt * p.K; i += blockDim.x) {
            const int tl = i / p.K;
            const int t = t0 + tl;
            const int e = p.idx[(size_t)t * p.K + (i - tl * p.K)];
            const uint64_t m = p.masks[(size_t)c * p.Epad + e];
            const uint64_t below = tl ? (m & ((1ull << tl) - 1ull)) : 0ull;
            const int slot = p.chunk_base[(size_t)c * p.Epad + e] + __popcll(below);
            p.slot_of[(size_t)t * p.K + (i - tl * p.K)] = slot;
            p.tok_of[slot] = t;
        }
    }
    const int tk = p.T * p.K;
    for (int i = threadIdx.x; i < nt * p.Ks; i += blockDim.x) {
        const int s = i / nt;
        const int t = t0 + (i - s * nt);
        p.tok_of[(size_t)tk + (size_t)s * p.T + t] = t;
    }
}

}  // namespace

hipError_t launch_permute(const Plan& p, hipStream_t st) {
    const int routed = p.K > 0 ? 1 : 0;
    perm_scan_kernel<<<1, kScanThreads, 0, st>>>(p, routed);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    perm_scatter_kernel<<<p.nchunk, 256, 0, st>>>(p, routed);
    return hipGetLastError();
}

}  // namespace moe
