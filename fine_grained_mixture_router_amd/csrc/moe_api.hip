// C-ABI dispatcher: validation, per-call plan and workspace carve-up, and the
// launch sequence router -> permutation -> G1 -> G2 -> combine, all enqueued
// on the caller's stream with no host synchronisation and no allocation.
#include <atomic>
#include <string.h>

#include "../../include/moe.h"
#include "common.h"

using namespace moe;

#ifndef MOE_ROUTER_WGS
#define MOE_ROUTER_WGS 512
#endif
#ifndef MOE_ROUTER_WIDE_T
#define MOE_ROUTER_WIDE_T 8192
#endif
#ifndef MOE_ROUTER_MINK
#define MOE_ROUTER_MINK 4
#endif

static_assert(kGateRenorm == MOE_FLAG_RENORM && kGateSigmoid == MOE_FLAG_SIGMOID,
              "gating flag bits");

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

bool shape_ok(const moe_shape_t* s) {
    if (!s) return false;
    if (s->T < 1 || s->T > (1 << 24)) return false;
    if (s->d < 64 || s->d > 65536 || s->d % 64) return false;
    if (s->E < 1 || s->E > 256) return false;
    if (s->K < 0 || s->K > s->E) return false;
    if (s->I < 64 || s->I > 65536 || s->I % 64) return false;
    if (s->Ks < 0 || s->Ks > 16) return false;
    if (s->Ks > 0 && (s->Is < 64 || s->Is > 65536 || s->Is % 64)) return false;
    if (s->flags & ~(MOE_FLAG_NO_RESIDUAL | MOE_FLAG_RENORM | MOE_FLAG_SIGMOID)) return false;
    const long long rows = (long long)s->T * (s->K + s->Ks);
    if (rows > (1LL << 30)) return false;
    // The GEMM kernels address x, H and one expert's weights with 32-bit
    // byte offsets: keep each of those below 2^31 bytes.
    const long long lim = 1LL << 31;
    const long long Is = s->Ks > 0 ? s->Is : 0;
    if ((long long)s->T * s->d * 2 >= lim) return false;
    if ((long long)s->T * s->K * s->I * 2 >= lim) return false;
    if ((long long)s->T * s->Ks * Is * 2 >= lim) return false;
    if ((long long)s->I * s->d * 2 >= lim || Is * s->d * 2 >= lim) return false;
    return true;
}

// Fill the shape-derived part of the plan and the workspace offsets (as byte
// offsets from 0); returns the total workspace size.  q8: the routed weights
// are 8-bit (the same tile sizes; each has an 8-bit kernel).
size_t make_plan(const moe_shape_t* s, Plan* p, bool q8) {
    (void)q8;
    memset(p, 0, sizeof(*p));
    p->T = s->T;
    p->d = s->d;
    p->E = s->E;
    p->I = s->I;
    p->K = s->K;
    p->Ks = s->Ks;
    p->Is = s->Ks > 0 ? s->Is : 64;
    p->flags = s->flags;
    p->Epad = (s->E + kRouterBE - 1) / kRouterBE * kRouterBE;
    p->nchunk = (s->T + kChunk - 1) / kChunk;
    const int nk = s->d / 64;
    // Router: a tile covers 64 tokens and every expert; the d range is split
    // so that the launch has about kRouterWGs workgroups (two per CU, which
    // its 80 KB of LDS allows), each split keeping at least kRouterMinK
    // slices of 64.
    // Batches of MOE_ROUTER_WIDE_T tokens or more take 256-token tiles (one
    // workgroup per CU, so about half as many workgroups are aimed at).  On
    // the V3-shape prefill batch (16 384 tokens) that takes the affinities
    // from 120 to 86 us; at 4 096 tokens the larger split's extra partials
    // cost the selection what the tiles save.
    p->router_wide = s->T >= MOE_ROUTER_WIDE_T ? 1 : 0;
    const int bt = p->router_wide ? kRouterWideT : kRouterBT;
    const int target = p->router_wide ? MOE_ROUTER_WGS / 2 : MOE_ROUTER_WGS;
    const int rtiles = (s->T + bt - 1) / bt;
    const int kmax = nk / MOE_ROUTER_MINK > 0 ? nk / MOE_ROUTER_MINK : 1;
    int split = (target + rtiles - 1) / rtiles;
    split = split < 1 ? 1 : (split > kmax ? kmax : split);
    const int kps = (nk + split - 1) / split;
    p->split = (nk + kps - 1) / kps;
    const long long TK = (long long)s->T * s->K;
    p->rows = (int)(TK + (long long)s->T * s->Ks);

    // Few rows per expert (decode-sized batches): thin tiles that stream each
    // weight once; otherwise 256x256 MFMA tiles.
    const bool thin = TK < 64LL * s->E;
    p->g1.bm = thin ? 32 : 256;
    p->g1.bn = 256;
    p->g2.bm = thin ? 32 : 256;
    p->g2.bn = 256;
    const long long busy = TK < s->E ? TK : s->E;
    const long long n1r = (s->I + p->g1.bn / 2 - 1) / (p->g1.bn / 2);
    const long long n1s = (p->Is + p->g1.bn / 2 - 1) / (p->g1.bn / 2);
    const long long n2 = (s->d + p->g2.bn - 1) / p->g2.bn;
    const long long m1s = (s->T + p->g1.bm - 1) / p->g1.bm;
    const long long m2s = (s->T + p->g2.bm - 1) / p->g2.bm;
    const long long t1 = (TK / p->g1.bm + busy) * n1r + (long long)s->Ks * m1s * n1s;
    const long long t2 = (TK / p->g2.bm + busy) * n2 + (long long)s->Ks * m2s * n2;
    p->max_tiles1 = (int)t1;
    p->max_tiles2 = (int)t2;

    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    p->logits = (float*)take(s->K > 0 ? (size_t)p->split * s->T * p->Epad * 4 : 0);
    p->idx = (int32_t*)take((size_t)TK * 4);
    p->gate = (float*)take((size_t)TK * 4);
    p->masks = (uint64_t*)take((size_t)p->nchunk * p->Epad * 8);
    p->chunk_base = (int32_t*)take((size_t)p->nchunk * p->Epad * 4);
    p->goff = (int32_t*)take((size_t)(s->E + s->Ks + 1) * 4);
    p->toff = (int32_t*)take((size_t)2 * (s->E + s->Ks + 1) * 4);
    p->tok_of = (int32_t*)take((size_t)p->rows * 4);
    p->slot_of = (int32_t*)take((size_t)TK * 4);
    p->tiles1 = (Tile*)take((size_t)p->max_tiles1 * sizeof(Tile));
    p->tiles2 = (Tile*)take((size_t)p->max_tiles2 * sizeof(Tile));
    p->ntiles = (int32_t*)take(16);
    p->H = (bf16_t*)take(((size_t)TK * s->I + (size_t)s->T * s->Ks * p->Is) * 2);
    p->Y = (bf16_t*)take((size_t)p->rows * s->d * 2);
    return off;
}

template <class T>
T* rebase(T* off, char* base) {
    return reinterpret_cast<T*>(base + reinterpret_cast<size_t>(off));
}

void place(Plan* p, void* ws) {
    char* b = static_cast<char*>(ws);
    p->logits = rebase(p->logits, b);
    p->idx = rebase(p->idx, b);
    p->gate = rebase(p->gate, b);
    p->masks = rebase(p->masks, b);
    p->chunk_base = rebase(p->chunk_base, b);
    p->goff = rebase(p->goff, b);
    p->toff = rebase(p->toff, b);
    p->tok_of = rebase(p->tok_of, b);
    p->slot_of = rebase(p->slot_of, b);
    p->tiles1 = rebase(p->tiles1, b);
    p->tiles2 = rebase(p->tiles2, b);
    p->ntiles = rebase(p->ntiles, b);
    p->H = rebase(p->H, b);
    p->Y = rebase(p->Y, b);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// 0 unknown, 1 gfx950, 2 other architecture
std::atomic<int> g_arch[64];

moe_status_t device_ok() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return MOE_ERR_NO_DEVICE;
    }
    int known = dev < 64 ? g_arch[dev].load(std::memory_order_relaxed) : 0;
    if (known == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return MOE_ERR_NO_DEVICE;
        }
        known = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        if (dev < 64) g_arch[dev].store(known, std::memory_order_relaxed);
    }
    return known == 1 ? MOE_OK : MOE_ERR_DEVICE_ARCH;
}

// Benchmark instrumentation: HIP events recorded around every kernel of the
// next moe_forward calls, on the call's stream.  One global recorder; not
// thread-safe (documented in moe.h).
constexpr int kSlots = 7;
const char* const kSlotNames[kSlots] = {"router_logits", "router_select", "perm_scan",
                                        "perm_scatter",  "gemm_gate_up",  "gemm_down",
                                        "combine"};
struct Recorder {
    bool on = false;
    int max_calls = 0;
    int calls = 0;
    hipEvent_t* ev = nullptr;   // [max_calls][kSlots][2]
    uint32_t mask = 0;          // kernel slots recorded
    bool used[kSlots] = {};
} g_rec;

void rec_mark(int slot, int end, hipStream_t s) {
    if (!g_rec.on || g_rec.calls >= g_rec.max_calls || !((g_rec.mask >> slot) & 1u)) return;
    (void)hipEventRecord(g_rec.ev[(g_rec.calls * kSlots + slot) * 2 + end], s);
}

void rec_free() {
    if (g_rec.ev) {
        for (int i = 0; i < g_rec.max_calls * kSlots * 2; ++i) (void)hipEventDestroy(g_rec.ev[i]);
        delete[] g_rec.ev;
    }
    g_rec = Recorder{};
}

moe_status_t check_common(const moe_shape_t* shape, const void* x, const void* centroids,
                          const float* bias, void* ws, size_t ws_bytes, Plan* plan,
                          bool q8 = false) {
    if (!shape) return MOE_ERR_NULL;
    if (!shape_ok(shape)) return MOE_ERR_SHAPE;
    if (!x || !ws) return MOE_ERR_NULL;
    if (shape->K > 0 && !centroids) return MOE_ERR_NULL;
    if (!aligned(x, 16) || (centroids && !aligned(centroids, 16))) return MOE_ERR_ALIGN;
    if (bias && !aligned(bias, 4)) return MOE_ERR_ALIGN;
    if (!aligned(ws, kAlign)) return MOE_ERR_ALIGN;
    const size_t need = make_plan(shape, plan, q8);
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) size_t moe_workspace_size(const moe_shape_t* shape) {
    if (!shape_ok(shape)) return 0;
    Plan p;
    const size_t a = make_plan(shape, &p, false);
    const size_t b = make_plan(shape, &p, true);   // moe_forward_fp8's plan
    return a > b ? a : b;
}

__attribute__((visibility("default"))) const char* moe_status_string(moe_status_t st) {
    switch (st) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
        case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: shape outside the supported limits or bad flags";
        case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: a pointer is misaligned";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace smaller than moe_workspace_size()";
        case MOE_ERR_NO_DEVICE: return "MOE_ERR_NO_DEVICE: no HIP device is available";
        case MOE_ERR_DEVICE_ARCH: return "MOE_ERR_DEVICE_ARCH: the current device is not gfx950";
        case MOE_ERR_HIP: return "MOE_ERR_HIP: a kernel launch failed";
    }
    return "unknown moe_status_t";
}

}  // extern "C"

namespace {

// The forward of both entry points: w1/w3/w2 are bf16 (q8 == null) or
// ignored in favour of the 8-bit routed weights q8.
moe_status_t run_forward(const moe_shape_t* shape, const void* x, const void* centroids,
                         const float* expert_bias, const void* w1, const void* w3,
                         const void* w2, const RoutedQ8* q8, const void* ws1, const void* ws3,
                         const void* ws2, void* out, int32_t* topk_idx, float* topk_gate,
                         void* workspace, size_t workspace_bytes, void* stream) {
    Plan p;
    moe_status_t st = check_common(shape, x, centroids, expert_bias, workspace, workspace_bytes,
                                   &p, q8 != nullptr);
    if (st != MOE_OK) return st;
    if (!out) return MOE_ERR_NULL;
    if (shape->K > 0) {
        if (q8 ? (!q8->q1 || !q8->q3 || !q8->q2 || !q8->s1 || !q8->s3 || !q8->s2)
               : (!w1 || !w3 || !w2))
            return MOE_ERR_NULL;
    }
    if (shape->Ks > 0 && (!ws1 || !ws3 || !ws2)) return MOE_ERR_NULL;
    const bool rk = shape->K > 0, sk = shape->Ks > 0;
    const void* a16[] = {out, rk && !q8 ? w1 : nullptr, rk && !q8 ? w3 : nullptr,
                         rk && !q8 ? w2 : nullptr, sk ? ws1 : nullptr, sk ? ws3 : nullptr,
                         sk ? ws2 : nullptr, rk && q8 ? q8->q1 : nullptr,
                         rk && q8 ? q8->q3 : nullptr, rk && q8 ? q8->q2 : nullptr};
    for (const void* a : a16)
        if (a && !aligned(a, 16)) return MOE_ERR_ALIGN;
    const void* a4[] = {topk_idx, topk_gate, rk && q8 ? q8->s1 : nullptr,
                        rk && q8 ? q8->s3 : nullptr, rk && q8 ? q8->s2 : nullptr};
    for (const void* a : a4)
        if (a && !aligned(a, 4)) return MOE_ERR_ALIGN;
    st = device_ok();
    if (st != MOE_OK) return st;

    place(&p, workspace);
    if (topk_idx) p.idx = topk_idx;
    if (topk_gate) p.gate = topk_gate;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const bf16_t* w1b = static_cast<const bf16_t*>(w1);
    const bf16_t* w3b = static_cast<const bf16_t*>(w3);
    const bf16_t* w2b = static_cast<const bf16_t*>(w2);
    const bf16_t* ws1b = static_cast<const bf16_t*>(ws1);
    const bf16_t* ws3b = static_cast<const bf16_t*>(ws3);
    const bf16_t* ws2b = static_cast<const bf16_t*>(ws2);
    const RoutedQ8* q = rk ? q8 : nullptr;
    hipError_t e = hipSuccess;
    auto step = [&](int slot, auto&& launch) {
        if (e != hipSuccess) return;
        rec_mark(slot, 0, s);
        e = launch();
        rec_mark(slot, 1, s);
    };
    if (p.K > 0) {
        step(0, [&] { return launch_router_logits(p, xb, static_cast<const bf16_t*>(centroids), s); });
        step(1, [&] { return launch_router_select(p, expert_bias, s); });
    }
    step(2, [&] { return launch_perm_scan(p, s); });
    step(3, [&] { return launch_perm_scatter(p, s); });
    step(4, [&] { return launch_gemm_gate_up(p, xb, w1b, w3b, ws1b, ws3b, q, s); });
    step(5, [&] { return launch_gemm_down(p, w2b, ws2b, q, s); });
    step(6, [&] { return launch_combine(p, xb, static_cast<bf16_t*>(out), s); });
    if (g_rec.on && g_rec.calls < g_rec.max_calls) {
        for (int k = 0; k < kSlots; ++k)
            if ((k >= 2 || p.K > 0) && ((g_rec.mask >> k) & 1u)) g_rec.used[k] = true;
        ++g_rec.calls;
    }
    if (e != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) moe_status_t moe_forward(
    const moe_shape_t* shape, const void* x, const void* centroids, const float* expert_bias,
    const void* w1, const void* w3, const void* w2, const void* ws1, const void* ws3,
    const void* ws2, void* out, int32_t* topk_idx, float* topk_gate, void* workspace,
    size_t workspace_bytes, void* stream) {
    return run_forward(shape, x, centroids, expert_bias, w1, w3, w2, nullptr, ws1, ws3, ws2, out,
                       topk_idx, topk_gate, workspace, workspace_bytes, stream);
}

__attribute__((visibility("default"))) moe_status_t moe_forward_fp8(
    const moe_shape_t* shape, const void* x, const void* centroids, const float* expert_bias,
    const void* w1q, const float* w1_scale, const void* w3q, const float* w3_scale,
    const void* w2q, const float* w2_scale, const void* ws1, const void* ws3, const void* ws2,
    void* out, int32_t* topk_idx, float* topk_gate, void* workspace, size_t workspace_bytes,
    void* stream) {
    const RoutedQ8 q8{static_cast<const uint8_t*>(w1q), static_cast<const uint8_t*>(w3q),
                      static_cast<const uint8_t*>(w2q), w1_scale, w3_scale, w2_scale};
    return run_forward(shape, x, centroids, expert_bias, nullptr, nullptr, nullptr, &q8, ws1, ws3,
                       ws2, out, topk_idx, topk_gate, workspace, workspace_bytes, stream);
}

__attribute__((visibility("default"))) moe_status_t moe_route(
    const moe_shape_t* shape, const void* x, const void* centroids, const float* expert_bias,
    int32_t* topk_idx, float* topk_gate, void* workspace, size_t workspace_bytes, void* stream) {
    Plan p;
    moe_status_t st = check_common(shape, x, centroids, expert_bias, workspace, workspace_bytes, &p);
    if (st != MOE_OK) return st;
    if (shape->K < 1) return MOE_ERR_SHAPE;
    if (!topk_idx || !topk_gate) return MOE_ERR_NULL;
    if (!aligned(topk_idx, 4) || !aligned(topk_gate, 4)) return MOE_ERR_ALIGN;
    st = device_ok();
    if (st != MOE_OK) return st;
    place(&p, workspace);
    p.idx = topk_idx;
    p.gate = topk_gate;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (launch_router_logits(p, static_cast<const bf16_t*>(x),
                             static_cast<const bf16_t*>(centroids), s) != hipSuccess ||
        launch_router_select(p, expert_bias, s) != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

__attribute__((visibility("default"))) moe_status_t moe_profile_begin_slots(int32_t max_calls,
                                                                            uint32_t slot_mask) {
    if (max_calls < 1 || max_calls > 100000) return MOE_ERR_SHAPE;
    if (slot_mask == 0 || (slot_mask >> kSlots) != 0) return MOE_ERR_SHAPE;
    moe_status_t st = device_ok();
    if (st != MOE_OK) return st;
    rec_free();
    g_rec.ev = new hipEvent_t[(size_t)max_calls * kSlots * 2];
    for (int i = 0; i < max_calls * kSlots * 2; ++i) {
        if (hipEventCreate(&g_rec.ev[i]) != hipSuccess) {
            for (int j = 0; j < i; ++j) (void)hipEventDestroy(g_rec.ev[j]);
            delete[] g_rec.ev;
            g_rec = Recorder{};
            return MOE_ERR_HIP;
        }
    }
    g_rec.max_calls = max_calls;
    g_rec.mask = slot_mask;
    g_rec.on = true;
    return MOE_OK;
}

__attribute__((visibility("default"))) moe_status_t moe_profile_begin(int32_t max_calls) {
    return moe_profile_begin_slots(max_calls, (1u << kSlots) - 1u);
}

__attribute__((visibility("default"))) moe_status_t moe_profile_end(float* ms, int32_t* launches,
                                                                    int32_t n_slots) {
    if (!g_rec.on) return MOE_ERR_NULL;
    moe_status_t st = MOE_OK;
    for (int k = 0; k < n_slots && k < kSlots; ++k) {
        float tot = 0.f;
        int n = 0;
        if (g_rec.used[k]) {
            for (int c = 0; c < g_rec.calls; ++c) {
                hipEvent_t b = g_rec.ev[(c * kSlots + k) * 2], en = g_rec.ev[(c * kSlots + k) * 2 + 1];
                float t = 0.f;
                if (hipEventSynchronize(en) != hipSuccess || hipEventElapsedTime(&t, b, en) != hipSuccess) {
                    st = MOE_ERR_HIP;
                    continue;
                }
                tot += t;
                ++n;
            }
        }
        if (ms) ms[k] = tot;
        if (launches) launches[k] = n;
    }
    for (int k = kSlots; k < n_slots; ++k) {
        if (ms) ms[k] = 0.f;
        if (launches) launches[k] = 0;
    }
    rec_free();
    return st;
}

__attribute__((visibility("default"))) const char* moe_profile_slot_name(int32_t slot) {
    return (slot >= 0 && slot < kSlots) ? kSlotNames[slot] : "";
}

__attribute__((visibility("default"))) moe_status_t moe_profile_stream_read(const void* buf,
                                                                            size_t bytes,
                                                                            void* stream) {
    if (!buf) return MOE_ERR_NULL;
    if (bytes == 0 || bytes % 32768) return MOE_ERR_SHAPE;
    if ((uintptr_t)buf % 16) return MOE_ERR_ALIGN;
    moe_status_t st = device_ok();
    if (st != MOE_OK) return st;
    return launch_stream_read(buf, bytes, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
