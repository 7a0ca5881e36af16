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

constexpr int kScanThreads = 1024;
constexpr int kQuarters = 4;        // threads per expert when counting chunk masks
#ifndef MOE_GROUP_M
#define MOE_GROUP_M 4
#endif
constexpr int kGroupM = MOE_GROUP_M;  // M-tiles per N sweep in the work-list order
static_assert(kScanThreads >= 256 * kQuarters, "one thread per (expert, quarter)");

constexpr int kScanWaves = kScanThreads / 64;
constexpr int kMaskBatch = 8;       // chunk masks loaded ahead of their use

// Exclusive prefix sum over the workgroup, in thread order: a shuffle scan
// within each wavefront, then the wavefront totals.  Two barriers; `swave`
// (kScanWaves ints of LDS) is free again on return.
__device__ int block_exclusive_scan(int v, int* swave, int* total) {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) swave[w] = x;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kScanWaves; ++i) {
        const int si = swave[i];
        base += i < w ? si : 0;
        tot += si;
    }
    __syncthreads();
    *total = tot;
    return base + x - v;
}

// Work-list entry i of a group with mt M-tiles and nt N-tiles, in
// "kGroupM M-tiles x all N-tiles" blocks: consecutive entries share either
// the A rows or the weight rows, which keeps the L2 of one XCD warm (each XCD
// takes runs of consecutive entries, see the GEMM kernels).
__device__ Tile tile_at(int i, int g, int nrows_g, int bm, int bn_out, int mt, int nt) {
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
    return t;
}

// Fill entries first, first + stride, ... of a work list: entry i belongs to
// the last group whose first entry is <= i (binary search over the exclusive
// tile offsets s_off[0..G)).
__device__ void emit_list(Tile* out, int total, int first, int stride, const int* s_off,
                          const int* s_cnt, int G, int bm, int bn_out, int ncols_r, int ncols_s,
                          int E) {
    for (int i = first; i < total; i += stride) {
        int lo = 0, hi = G - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_off[mid] <= i) lo = mid;
            else hi = mid - 1;
        }
        const int g = lo;
        const int n = s_cnt[g];
        const int mt = (n + bm - 1) / bm;
        const int ncols = g < E ? ncols_r : ncols_s;
        const int nt = (ncols + bn_out - 1) / bn_out;
        out[i] = tile_at(i - s_off[g], g, n, bm, bn_out, mt, nt);
    }
}

__global__ __launch_bounds__(kScanThreads) void perm_scan_kernel(Plan p, int routed) {
    __shared__ int sbuf[kScanWaves];
    __shared__ int s_part[kQuarters][256];
    __shared__ int s_cnt[kScanThreads];
    const int tid = threadIdx.x;
    const int G = p.E + p.Ks;
    const int e = tid & 255;
    const int q = tid >> 8;
    const int cq = (p.nchunk + kQuarters - 1) / kQuarters;
    const int c0 = min(p.nchunk, q * cq), c1 = min(p.nchunk, c0 + cq);

    // rows of expert e in chunk quarter q
    int part = 0;
    if (routed && e < p.E && q < kQuarters)
        for (int c = c0; c < c1; c += kMaskBatch) {
            uint64_t m[kMaskBatch];
#pragma unroll
            for (int b = 0; b < kMaskBatch; ++b)
                m[b] = c + b < c1 ? p.masks[(size_t)(c + b) * p.Epad + e] : 0ull;
#pragma unroll
            for (int b = 0; b < kMaskBatch; ++b) part += __popcll(m[b]);
        }
    if (q < kQuarters) s_part[q][e] = part;
    __syncthreads();

    // rows per group, then group offsets
    int cnt = 0;
    if (tid < p.E && routed) {
        for (int k = 0; k < kQuarters; ++k) cnt += s_part[k][tid];
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
    __syncthreads();

    // per-(chunk, expert) first row
    if (routed && e < p.E && q < kQuarters) {
        int run = p.goff[e];
        for (int k = 0; k < q; ++k) run += s_part[k][e];
        for (int c = c0; c < c1; c += kMaskBatch) {
            uint64_t m[kMaskBatch];
#pragma unroll
            for (int b = 0; b < kMaskBatch; ++b)
                m[b] = c + b < c1 ? p.masks[(size_t)(c + b) * p.Epad + e] : 0ull;
#pragma unroll
            for (int b = 0; b < kMaskBatch; ++b) {
                if (c + b < c1) p.chunk_base[(size_t)(c + b) * p.Epad + e] = run;
                run += __popcll(m[b]);
            }
        }
    }

    // work lists
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
        p.toff[tid] = o1;                           // the lists themselves are filled by
        p.toff[G + 1 + tid] = o2;                   // every workgroup of perm_scatter
    }
    if (tid == 0) {
        p.toff[G] = tot1;
        p.toff[2 * G + 1] = tot2;
        p.ntiles[0] = tot1;
        p.ntiles[1] = tot2;
    }
}

// One workgroup per 64-token chunk: slot of every (token, k) and the token of
// every permuted row (routed rows by expert, then the shared rows).  Every
// workgroup (at least kEmitGroups of them) also fills a strided share of the
// two GEMM work lists from the group offsets and tile offsets perm_scan left.
constexpr int kEmitGroups = 64;
constexpr int kScatterThreads = 256;

__global__ __launch_bounds__(kScatterThreads) void perm_scatter_kernel(Plan p, int routed) {
    __shared__ int s_cnt[256 + 16];
    __shared__ int s_t1[256 + 16];
    __shared__ int s_t2[256 + 16];
    const int G = p.E + p.Ks;
    for (int g = threadIdx.x; g < G; g += kScatterThreads) {
        s_cnt[g] = p.goff[g + 1] - p.goff[g];
        s_t1[g] = p.toff[g];
        s_t2[g] = p.toff[G + 1 + g];
    }
    const int tot1 = p.toff[G], tot2 = p.toff[2 * G + 1];
    __syncthreads();
    const int first = blockIdx.x * kScatterThreads + threadIdx.x;
    const int stride = gridDim.x * kScatterThreads;
    emit_list(p.tiles1, tot1, first, stride, s_t1, s_cnt, G, p.g1.bm, p.g1.bn / 2, p.I, p.Is, p.E);
    emit_list(p.tiles2, tot2, first, stride, s_t2, s_cnt, G, p.g2.bm, p.g2.bn, p.d, p.d, p.E);

    const int c = blockIdx.x;
    if (c >= p.nchunk) return;
    const int t0 = c * kChunk;
    const int nt = min(kChunk, p.T - t0);
    if (routed) {
        for (int i = threadIdx.x; i < nt * p.K; i += kScatterThreads) {
            const int tl = i / p.K;
            const int t = t0 + tl;
            const int e = p.idx[(size_t)t * p.K + (i - tl * p.K)];
            const uint64_t m = p.masks[(size_t)c * p.Epad + e];
            const uint64_t below = tl ? (m & ((1ull << tl) - 1ull)) : 0ull;
            const int slot = p.chunk_base[(size_t)c * p.Epad + e] + __popcll(below);
            p.slot_of[(size_t)t * p.K + (i - tl * p.K)] = slot;
            p.tok_of[slot] = t;
            if (p.row_gate) p.row_gate[slot] = p.gate[(size_t)t * p.K + (i - tl * p.K)];
        }
    }
    const int tk = p.T * p.K;
    for (int i = threadIdx.x; i < nt * p.Ks; i += kScatterThreads) {
        const int s = i / nt;
        const int t = t0 + (i - s * nt);
        p.tok_of[(size_t)tk + (size_t)s * p.T + t] = t;
    }
}

}  // namespace

hipError_t launch_perm_scan(const Plan& p, hipStream_t st) {
    perm_scan_kernel<<<1, kScanThreads, 0, st>>>(p, p.K > 0 ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_perm_scatter(const Plan& p, hipStream_t st) {
    const int grid = p.nchunk > kEmitGroups ? p.nchunk : kEmitGroups;
    perm_scatter_kernel<<<grid, kScatterThreads, 0, st>>>(p, p.K > 0 ? 1 : 0);
    return hipGetLastError();
}

}  // namespace moe
