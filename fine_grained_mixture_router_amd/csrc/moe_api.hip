// C-ABI dispatcher: validation, per-call plan and workspace carve-up, and the
// launch sequence router -> permutation -> G1 -> G2 -> combine, all enqueued
// on the caller's stream with no host synchronisation and no allocation.
#include <atomic>
#include <mutex>
#include <string.h>

#include "../../include/moe.h"
#include "common.h"

using namespace moe;

// Router tiles: batches of MOE_ROUTER_BIG_T tokens or more keep the whole d
// range in one workgroup (no partials leave it), on 16-token tiles while
// those leave a workgroup per CU or more and re-read the centroids no more
// than MOE_ROUTER_CBYTES in all, else on 64-token tiles; smaller batches
// take 16-token tiles with d split to about one workgroup per CU.
#ifndef MOE_ROUTER_BIG_T
#define MOE_ROUTER_BIG_T 4096
#endif
#ifndef MOE_ROUTER_WGS
#define MOE_ROUTER_WGS 256
#endif
#ifndef MOE_ROUTER_CBYTES
#define MOE_ROUTER_CBYTES (256LL << 20)
#endif

static_assert(kGateRenorm == MOE_FLAG_RENORM && kGateSigmoid == MOE_FLAG_SIGMOID &&
                  kAct8 == MOE_FLAG_ACT8,
              "flag bits");
static_assert(sizeof(Tile) == sizeof(moe_tile_t) && offsetof(Tile, group) == offsetof(moe_tile_t, group) &&
                  offsetof(Tile, m0) == offsetof(moe_tile_t, m0) && offsetof(Tile, n0) == offsetof(moe_tile_t, n0) &&
                  offsetof(Tile, nrows) == offsetof(moe_tile_t, nrows),
              "work-list entries as the header describes them");

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
    if (s->flags & ~(MOE_FLAG_NO_RESIDUAL | MOE_FLAG_RENORM | MOE_FLAG_SIGMOID | MOE_FLAG_ACT8))
        return false;
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
// are 8-bit (the same tile sizes; each has an 8-bit kernel).  route_only:
// carve only what routing needs (affinity partials and the chunk masks; the
// caller passes idx and gate), for moe_route.
size_t make_plan(const moe_shape_t* s, Plan* p, bool q8, bool route_only = false,
                 bool train = false) {
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
    if (s->T >= MOE_ROUTER_BIG_T) {
        const long long reread = (long long)s->E * s->d * 2 * (p->nchunk * 4);
        p->router_bt = (p->nchunk >= MOE_ROUTER_WGS || reread > MOE_ROUTER_CBYTES) ? 64 : 16;
        p->split = 1;
        p->kps = nk;
    } else {
        p->router_bt = 16;
        const int tiles = p->nchunk * 4;
        const int kmax = nk / 2 > 1 ? nk / 2 : 1;          // at least two slices per split
        int split = (MOE_ROUTER_WGS + tiles - 1) / tiles;
        split = split < 1 ? 1 : (split > kmax ? kmax : split);
        p->kps = (nk + split - 1) / split;
        p->split = (nk + p->kps - 1) / p->kps;
    }
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
    const bool part = s->K > 0 && p->split > 1;
    p->logits = (float*)take(part ? (size_t)p->split * s->T * p->Epad * 4 : 0);
    p->tickets = (int32_t*)take(part ? (size_t)router_tiles(*p) * 4 : 0);
    if (route_only) {
        p->masks = (uint64_t*)take((size_t)p->nchunk * p->Epad * 8);
        return off;
    }
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
    const bool act8 = (s->flags & MOE_FLAG_ACT8) && s->K > 0;
    p->xq = (uint8_t*)take(act8 ? (size_t)s->T * s->d : 0);
    p->xe = (int32_t*)take(act8 ? (size_t)s->T * 4 : 0);
    // the FP8 tile takes 256-row tiles with d a multiple of its 128-deep
    // slices; other batches feed the dequantised rows to the 8-bit-weight tiles
    p->xd = (bf16_t*)take(act8 && !f8_gate_up(*p) ? (size_t)s->T * s->d * 2 : 0);
    p->hq = (uint8_t*)take(act8 && f8_down(*p) ? (size_t)TK * s->I : 0);
    p->he = (int32_t*)take(act8 && f8_down(*p) ? (size_t)TK * 4 : 0);
    p->H = (bf16_t*)take(((size_t)TK * s->I + (size_t)s->T * s->Ks * p->Is) * 2);
    p->Y = (bf16_t*)take((size_t)p->rows * s->d * 2);
    if (train) {
        p->scores = (float*)take(s->K > 0 ? (size_t)s->T * p->Epad * 4 : 0);
        p->score_part = (float*)take(s->K > 0 ? (size_t)p->nchunk * 4 * p->Epad * 4 : 0);
        p->row_gate = (float*)take((size_t)TK * 4);
        p->Z = (bf16_t*)take(((size_t)TK * s->I + (size_t)s->T * s->Ks * p->Is) * 2 * 2);
    }
    return off;
}

// The backward's own workspace: offsets from 0, returns the total size.
size_t make_bwd_plan(const moe_shape_t* s, const Plan& p, BwdPlan* b) {
    memset(b, 0, sizeof(*b));
    const size_t TK = (size_t)s->T * s->K;
    const int imax = s->I > p.Is ? s->I : p.Is;
    b->ndh = (imax + 255) / 256;
    // 256-row tiles: sum over groups of ceil(n_g / 256) <= rows / 256 + groups
    const long long mt = (long long)p.rows / 256 + s->E + s->Ks;
    b->max_tiles_dh = (int)(mt * b->ndh);
    b->max_tiles_dx = (int)(mt * ((s->d + 255) / 256));
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    b->dZ = (bf16_t*)take((TK * s->I + (size_t)s->T * s->Ks * p.Is) * 2 * 2);
    b->gH = (bf16_t*)take(TK * s->I * 2);
    b->dgp = (float*)take((size_t)p.rows * b->ndh * 4);
    b->dL = (bf16_t*)take(s->K > 0 ? (size_t)s->T * p.Epad * 2 : 0);
    b->R32 = (float*)take(s->K > 0 ? (size_t)s->T * s->d * 4 : 0);
    b->dXr = (bf16_t*)take((size_t)p.rows * s->d * 2);
    b->tiles_dh = (Tile*)take((size_t)b->max_tiles_dh * sizeof(Tile));
    b->tiles_dx = (Tile*)take((size_t)b->max_tiles_dx * sizeof(Tile));
    b->ntiles = (int32_t*)take(16);
    b->gorder = (int32_t*)take((size_t)(s->E + s->Ks) * 4);
    b->dgate = (float*)take(TK * 4);
    return off;
}

template <class T>
T* rebase(T* off, char* base) {
    return reinterpret_cast<T*>(base + reinterpret_cast<size_t>(off));
}

// Route-only plan: the two pieces make_plan(route_only) carved.
void place_bwd(BwdPlan* q, void* ws) {
    char* b = static_cast<char*>(ws);
    q->dZ = rebase(q->dZ, b);
    q->gH = rebase(q->gH, b);
    q->dgp = rebase(q->dgp, b);
    q->dL = rebase(q->dL, b);
    q->R32 = rebase(q->R32, b);
    q->dXr = rebase(q->dXr, b);
    q->tiles_dh = rebase(q->tiles_dh, b);
    q->tiles_dx = rebase(q->tiles_dx, b);
    q->ntiles = rebase(q->ntiles, b);
    q->gorder = rebase(q->gorder, b);
    q->dgate = rebase(q->dgate, b);
}

void place_route(Plan* p, void* ws) {
    char* b = static_cast<char*>(ws);
    p->logits = rebase(p->logits, b);
    p->tickets = rebase(p->tickets, b);
    p->masks = rebase(p->masks, b);
}

void place(Plan* p, void* ws) {
    char* b = static_cast<char*>(ws);
    p->tickets = rebase(p->tickets, b);
    if (p->Z) {                                     // a training plan
        p->scores = rebase(p->scores, b);
        p->score_part = rebase(p->score_part, b);
        p->row_gate = rebase(p->row_gate, b);
        p->Z = rebase(p->Z, b);
    }
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
    const bool act8 = (p->flags & kAct8) && p->K > 0;
    p->xq = act8 ? rebase(p->xq, b) : nullptr;
    p->xe = act8 ? rebase(p->xe, b) : nullptr;
    p->xd = act8 && !f8_gate_up(*p) ? rebase(p->xd, b) : nullptr;
    p->hq = act8 && f8_down(*p) ? rebase(p->hq, b) : nullptr;
    p->he = act8 && f8_down(*p) ? rebase(p->he, b) : nullptr;
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
constexpr int kSlots = 18;
constexpr int kBwdSlot0 = 7;                 // backward kernels: slots 7..15
constexpr int kAct8Slot0 = 16;               // 8-bit activations: quantisation of x, of h
const char* const kSlotNames[kSlots] = {"router",        "router_tickets", "perm_scan",
                                        "perm_scatter",  "gemm_gate_up",  "gemm_down",
                                        "combine",       "bwd_lists",     "bwd_dh",
                                        "bwd_router",    "bwd_dx_router", "bwd_dx",
                                        "bwd_dx_combine", "bwd_dw2",      "bwd_dw13",
                                        "bwd_dc",         "act8_x",       "act8_h"};
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

void rec_mark_bwd(int slot, int end, hipStream_t s) { rec_mark(kBwdSlot0 + slot, end, s); }

void rec_free() {
    if (g_rec.ev) {
        for (int i = 0; i < g_rec.max_calls * kSlots * 2; ++i) (void)hipEventDestroy(g_rec.ev[i]);
        delete[] g_rec.ev;
    }
    g_rec = Recorder{};
}

moe_status_t check_common(const moe_shape_t* shape, const void* x, const void* centroids,
                          const float* bias, void* ws, size_t ws_bytes, Plan* plan,
                          bool q8 = false, bool route_only = false, bool train = false) {
    if (!shape) return MOE_ERR_NULL;
    if (!shape_ok(shape)) return MOE_ERR_SHAPE;
    if (!x || !ws) return MOE_ERR_NULL;
    if (shape->K > 0 && !centroids) return MOE_ERR_NULL;
    if (!aligned(x, 16) || (centroids && !aligned(centroids, 16))) return MOE_ERR_ALIGN;
    if (bias && !aligned(bias, 4)) return MOE_ERR_ALIGN;
    if (!aligned(ws, kAlign)) return MOE_ERR_ALIGN;
    const size_t need = make_plan(shape, plan, q8, route_only, train);
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) moe_status_t moe_workspace_layout(const moe_shape_t* shape,
                                                                          moe_layout_t* layout) {
    if (!layout || !shape) return MOE_ERR_NULL;
    if (!shape_ok(shape)) return MOE_ERR_SHAPE;
    Plan p;
    make_plan(shape, &p, false);
    auto at = [](const void* off) { return reinterpret_cast<size_t>(off); };
    layout->idx = at(p.idx);
    layout->gate = at(p.gate);
    layout->goff = at(p.goff);
    layout->tok_of = at(p.tok_of);
    layout->slot_of = at(p.slot_of);
    layout->tiles_gate_up = at(p.tiles1);
    layout->tiles_down = at(p.tiles2);
    layout->ntiles = at(p.ntiles);
    const bool act8 = (shape->flags & MOE_FLAG_ACT8) && shape->K > 0;
    layout->act8_codes = act8 ? at(p.xq) : 0;
    layout->act8_exps = act8 ? at(p.xe) : 0;
    layout->h = at(p.H);
    layout->act8_h_codes = act8 && f8_down(p) ? at(p.hq) : 0;
    layout->act8_h_exps = act8 && f8_down(p) ? at(p.he) : 0;
    layout->rows = p.rows;
    layout->max_tiles_gate_up = p.max_tiles1;
    layout->max_tiles_down = p.max_tiles2;
    layout->tile_rows_gate_up = p.g1.bm;
    layout->tile_cols_gate_up = p.g1.bn / 2;
    layout->tile_rows_down = p.g2.bm;
    layout->tile_cols_down = p.g2.bn;
    return MOE_OK;
}

__attribute__((visibility("default"))) size_t moe_workspace_size(const moe_shape_t* shape) {
    if (!shape_ok(shape)) return 0;
    Plan p;
    const size_t a = make_plan(shape, &p, false);
    const size_t b = make_plan(shape, &p, true);   // moe_forward_fp8's plan
    return a > b ? a : b;
}

__attribute__((visibility("default"))) size_t moe_train_state_size(const moe_shape_t* shape) {
    if (!shape_ok(shape)) return 0;
    Plan p;
    return make_plan(shape, &p, false, false, true);
}

__attribute__((visibility("default"))) size_t moe_backward_workspace_size(const moe_shape_t* shape) {
    if (!shape_ok(shape)) return 0;
    Plan p;
    make_plan(shape, &p, false, false, true);
    BwdPlan b;
    return make_bwd_plan(shape, p, &b);
}

__attribute__((visibility("default"))) size_t moe_route_workspace_size(const moe_shape_t* shape) {
    if (!shape_ok(shape) || shape->K < 1) return 0;
    Plan p;
    return make_plan(shape, &p, false, true);
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
        case MOE_ERR_SCRATCH:
            return "MOE_ERR_SCRATCH: the shape needs more scratch than moe_forward_noalloc's static "
                   "buffer holds (moe_noalloc_scratch_bytes())";
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
                         void* workspace, size_t workspace_bytes, void* stream,
                         bool train = false, float* stats = nullptr) {
    Plan p;
    moe_status_t st = check_common(shape, x, centroids, expert_bias, workspace, workspace_bytes,
                                   &p, q8 != nullptr, false, train);
    if (st != MOE_OK) return st;
    if ((shape->flags & MOE_FLAG_ACT8) && !q8) return MOE_ERR_SHAPE;   // 8-bit weights only
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
                        rk && q8 ? q8->s3 : nullptr, rk && q8 ? q8->s2 : nullptr, stats};
    for (const void* a : a4)
        if (a && !aligned(a, 4)) return MOE_ERR_ALIGN;
    st = device_ok();
    if (st != MOE_OK) return st;

    place(&p, workspace);
    // A training forward keeps the routing in its state (the backward reads
    // it there) and copies it out afterwards; otherwise the router writes
    // the caller's arrays directly.
    if (!train) {
        if (topk_idx) p.idx = topk_idx;
        if (topk_gate) p.gate = topk_gate;
    }
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
        step(1, [&] { return launch_router_tickets(p, s); });
        step(0, [&] {
            return launch_router(p, xb, static_cast<const bf16_t*>(centroids), expert_bias, s);
        });
        const size_t rb = (size_t)p.T * p.K * 4;
        if (train && topk_idx && e == hipSuccess)
            e = hipMemcpyAsync(topk_idx, p.idx, rb, hipMemcpyDeviceToDevice, s);
        if (train && topk_gate && e == hipSuccess)
            e = hipMemcpyAsync(topk_gate, p.gate, rb, hipMemcpyDeviceToDevice, s);
    }
    step(2, [&] { return launch_perm_scan(p, s); });
    step(3, [&] { return launch_perm_scatter(p, s); });
    if (stats && p.K > 0 && e == hipSuccess) e = launch_balance_stats(p, stats, s);
    // 8-bit activations: each GEMM's routed input rows (x; the routed rows
    // of H) are quantised just before it
    if (p.xq) step(kAct8Slot0, [&] { return launch_act8_quant(xb, p.T, p.d, p.xq, p.xe, p.xd, s); });
    step(4, [&] { return launch_gemm_gate_up(p, xb, w1b, w3b, ws1b, ws3b, q, s); });
    if (p.xq) {
        step(kAct8Slot0 + 1, [&] {
            return p.hq ? launch_act8_quant(p.H, p.T * p.K, p.I, p.hq, p.he, nullptr, s)
                        : launch_act8_quant(p.H, p.T * p.K, p.I, nullptr, nullptr, p.H, s);
        });
    }
    step(5, [&] { return launch_gemm_down(p, w2b, ws2b, q, s); });
    step(6, [&] { return launch_combine(p, xb, static_cast<bf16_t*>(out), s); });
    if (g_rec.on && g_rec.calls < g_rec.max_calls) {
        for (int k = 0; k < kBwdSlot0; ++k) {
            const bool ran = k >= 2 || (p.K > 0 && (k == 0 || p.split > 1));
            if (ran && ((g_rec.mask >> k) & 1u)) g_rec.used[k] = true;
        }
        for (int k = kAct8Slot0; k < kSlots; ++k)
            if (p.xq && ((g_rec.mask >> k) & 1u)) g_rec.used[k] = true;
        ++g_rec.calls;
    }
    if (e != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
}

moe_status_t run_backward(const moe_shape_t* shape, const void* x, const void* centroids,
                          const void* w1, const void* w3, const void* w2, const void* ws1,
                          const void* ws3, const void* ws2, const void* dout, float alpha,
                          const void* state, size_t state_bytes, void* dx, void* dw1, void* dw3,
                          void* dw2, void* dws1, void* dws3, void* dws2, float* dC, float* dgate,
                          void* workspace, size_t workspace_bytes, void* stream) {
    if (!shape) return MOE_ERR_NULL;
    if (!shape_ok(shape)) return MOE_ERR_SHAPE;
    if (shape->flags & ~(MOE_FLAG_NO_RESIDUAL | MOE_FLAG_RENORM | MOE_FLAG_SIGMOID)) return MOE_ERR_SHAPE;
    if (!(alpha >= 0.f) || !(alpha < 1e30f)) return MOE_ERR_SHAPE;   // also rejects NaN
    const bool rk = shape->K > 0, sk = shape->Ks > 0;
    if (!x || !dout || !state || !dx || !workspace) return MOE_ERR_NULL;
    if (rk && (!centroids || !w1 || !w3 || !w2 || !dw1 || !dw3 || !dw2 || !dC)) return MOE_ERR_NULL;
    if (sk && (!ws1 || !ws3 || !ws2 || !dws1 || !dws3 || !dws2)) return MOE_ERR_NULL;
    const void* a16[] = {x, dout, dx, rk ? centroids : nullptr, rk ? w1 : nullptr, rk ? w3 : nullptr,
                         rk ? w2 : nullptr, rk ? dw1 : nullptr, rk ? dw3 : nullptr, rk ? dw2 : nullptr,
                         sk ? ws1 : nullptr, sk ? ws3 : nullptr, sk ? ws2 : nullptr,
                         sk ? dws1 : nullptr, sk ? dws3 : nullptr, sk ? dws2 : nullptr,
                         rk ? dC : nullptr};
    for (const void* a : a16)
        if (a && !aligned(a, 16)) return MOE_ERR_ALIGN;
    if (dgate && !aligned(dgate, 4)) return MOE_ERR_ALIGN;
    if (!aligned(state, kAlign) || !aligned(workspace, kAlign)) return MOE_ERR_ALIGN;
    Plan p;
    if (state_bytes < make_plan(shape, &p, false, false, true)) return MOE_ERR_WORKSPACE;
    BwdPlan b;
    if (workspace_bytes < make_bwd_plan(shape, p, &b)) return MOE_ERR_WORKSPACE;
    moe_status_t st = device_ok();
    if (st != MOE_OK) return st;
    place(&p, const_cast<void*>(state));
    place_bwd(&b, workspace);
    BwdArgs a{};
    a.x = static_cast<const bf16_t*>(x);
    a.C = static_cast<const bf16_t*>(centroids);
    a.w1 = static_cast<const bf16_t*>(w1);
    a.w3 = static_cast<const bf16_t*>(w3);
    a.w2 = static_cast<const bf16_t*>(w2);
    a.ws1 = static_cast<const bf16_t*>(ws1);
    a.ws3 = static_cast<const bf16_t*>(ws3);
    a.ws2 = static_cast<const bf16_t*>(ws2);
    a.dout = static_cast<const bf16_t*>(dout);
    a.alpha = alpha;
    a.dx = static_cast<bf16_t*>(dx);
    a.dw1 = static_cast<bf16_t*>(dw1);
    a.dw3 = static_cast<bf16_t*>(dw3);
    a.dw2 = static_cast<bf16_t*>(dw2);
    a.dws1 = static_cast<bf16_t*>(dws1);
    a.dws3 = static_cast<bf16_t*>(dws3);
    a.dws2 = static_cast<bf16_t*>(dws2);
    a.dC = dC;
    a.dgate = dgate;
    const hipError_t e = launch_backward(p, b, a, static_cast<hipStream_t>(stream), rec_mark_bwd);
    if (g_rec.on && g_rec.calls < g_rec.max_calls) {
        for (int k = kBwdSlot0; k < kAct8Slot0; ++k) {
            const int bs = k - kBwdSlot0;
            const bool ran = rk || !(bs == 2 || bs == 3 || bs == 8);
            if (ran && ((g_rec.mask >> k) & 1u)) g_rec.used[k] = true;
        }
        ++g_rec.calls;
    }
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// Allocation-free forward: the workspace is a static device array of
// kScratchBytes (every GPU the library runs on holds its own copy until the
// process ends).  Host code never uses the array's name as an address — it
// is a host-side stand-in there — but the device address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device on the entry point's first call there.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of this device's scratch array, or null (and *err set) if
// the lookup failed.  The caller has made `dev` current.
void* scratch_address(int dev, hipError_t* err) {
    std::call_once(g_scratch_once[dev], [dev] {
        void* ptr = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
        if (g_scratch_err[dev] != hipSuccess) (void)hipGetLastError();
    });
    *err = g_scratch_err[dev];
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) moe_status_t moe_forward_noalloc(
    const moe_shape_t* shape, const void* x, const void* centroids, const float* expert_bias,
    const void* w1, const void* w3, const void* w2, const void* ws1, const void* ws3,
    const void* ws2, void* out, int32_t* topk_idx, float* topk_gate, void* stream) {
    if (!shape) return MOE_ERR_NULL;
    if (!shape_ok(shape)) return MOE_ERR_SHAPE;
    Plan probe;
    if (make_plan(shape, &probe, false) > kScratchBytes) return MOE_ERR_SCRATCH;
    moe_status_t st = device_ok();
    if (st != MOE_OK) return st;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return MOE_ERR_NO_DEVICE;
    }
    hipError_t err = hipSuccess;
    void* ws = scratch_address(dev, &err);
    if (!ws) return MOE_ERR_HIP;
    return run_forward(shape, x, centroids, expert_bias, w1, w3, w2, nullptr, ws1, ws3, ws2, out,
                       topk_idx, topk_gate, ws, kScratchBytes, stream);
}

__attribute__((visibility("default"))) size_t moe_noalloc_scratch_bytes(void) {
    return kScratchBytes;
}

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

__attribute__((visibility("default"))) moe_status_t moe_forward_train(
    const moe_shape_t* shape, const void* x, const void* centroids, const float* expert_bias,
    const void* w1, const void* w3, const void* w2, const void* ws1, const void* ws3,
    const void* ws2, void* out, int32_t* topk_idx, float* topk_gate, float* balance_stats,
    void* state, size_t state_bytes, void* stream) {
    return run_forward(shape, x, centroids, expert_bias, w1, w3, w2, nullptr, ws1, ws3, ws2, out,
                       topk_idx, topk_gate, state, state_bytes, stream, true, balance_stats);
}

__attribute__((visibility("default"))) moe_status_t moe_backward(
    const moe_shape_t* shape, const void* x, const void* centroids, const void* w1,
    const void* w3, const void* w2, const void* ws1, const void* ws3, const void* ws2,
    const void* dout, float alpha, const void* state, size_t state_bytes, void* dx, void* dw1,
    void* dw3, void* dw2, void* dws1, void* dws3, void* dws2, float* dC, float* dgate,
    void* workspace, size_t workspace_bytes, void* stream) {
    return run_backward(shape, x, centroids, w1, w3, w2, ws1, ws3, ws2, dout, alpha, state,
                        state_bytes, dx, dw1, dw3, dw2, dws1, dws3, dws2, dC, dgate, workspace,
                        workspace_bytes, stream);
}

__attribute__((visibility("default"))) moe_status_t moe_route(
    const moe_shape_t* shape, const void* x, const void* centroids, const float* expert_bias,
    int32_t* topk_idx, float* topk_gate, void* workspace, size_t workspace_bytes, void* stream) {
    Plan p;
    moe_status_t st = check_common(shape, x, centroids, expert_bias, workspace, workspace_bytes,
                                   &p, false, true);
    if (st != MOE_OK) return st;
    if (shape->K < 1) return MOE_ERR_SHAPE;
    if (!topk_idx || !topk_gate) return MOE_ERR_NULL;
    if (!aligned(topk_idx, 4) || !aligned(topk_gate, 4)) return MOE_ERR_ALIGN;
    st = device_ok();
    if (st != MOE_OK) return st;
    place_route(&p, workspace);
    p.idx = topk_idx;
    p.gate = topk_gate;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (launch_router_tickets(p, s) != hipSuccess ||
        launch_router(p, static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(centroids),
                      expert_bias, s) != hipSuccess)
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
