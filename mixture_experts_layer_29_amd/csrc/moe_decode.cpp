// moe_decode.cpp -- host side of the C ABI declared in include/moe_decode.h.
//
// A plan validates the layer shape, resolves the kernel family (small-matrix
// GEMV at batch <= 2, split-K above: the shape choice the Kimi K3 decode
// article describes in Part 1 section 1) and sizes the workspace; it touches
// no device.  The first forward allocates the workspace, a second stream and
// events, and builds a HIP graph: front (router, and by default the shared
// expert's gate/up in trailing workgroups) -> [top-k] -> routed gate/up (at
// batch <= 4 by default selecting for itself) -> down.  With shared_stream = 1 the shared expert's gate/up is a parallel
// branch on the second stream joined before the down projection instead
// (article Part 1 section 3: shared expert on its own stream, overlapped with
// routing; "What's next": per-step host work replayed as a graph).  Later
// forwards replay the graph, patching kernel arguments when the caller's
// pointers change; a forward on a capturing stream launches the kernels
// directly so they land in the caller's graph.  The eager path is also used
// for per-kernel timing.
#include "moe_decode.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "moe_args.h"

using namespace moe;

namespace {

thread_local std::string g_err;

moe_status fail(moe_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

#define HIP_TRY(call)                                                                         \
    do {                                                                                      \
        hipError_t e_ = (call);                                                               \
        if (e_ != hipSuccess)                                                                 \
            return fail(MOE_ERR_HIP, "%s failed: %s (%s:%d)", #call, hipGetErrorString(e_),   \
                        __FILE__, __LINE__);                                                  \
    } while (0)

// An expert's gate/up takes split-K MFMA tiles from this many tokens on (GEMV
// tiles below): measured on MI355X, an expert with 4 tokens streams faster as
// one-round GEMV tiles than as MFMA tiles with their atomics and last-arriver
// epilogue (batch 64, TP8 shard: 352 -> 347 us); capped by the GEMV tiles' LDS.
constexpr int kDefaultMfmaMin = 5;
// batch 5-16: experts from 3 tokens on MFMA tiles (measured 1-3 us faster at
// batch 8 / 16 than from 5; at batch 64 it is not)
constexpr int kDefaultMfmaMinSmall = 3, kMfmaMinSmallMaxBatch = 16;
constexpr int kMaxProfiledForwards = 1024;
constexpr int kSmallRouterMaxBatch = 4;
constexpr int kTopkOneGroupMaxBatch = 8;     // the top-k launch selects in one workgroup up to this batch
constexpr size_t kSelectGateupMaxTiles = 512;  // gate/up workgroups of one generation (2 per CU x 256 CUs)
constexpr size_t kSmallRouterLds = 56 * 1024;

constexpr size_t kLayerLds = 56 * 1024;  // dynamic LDS of the single launch: x staging, then h rows
constexpr size_t kDownHLds = 48 * 1024;   // output-stationary down: h fully staged in LDS up to this
constexpr int kDownOsMaxBatch = 4;        // output-stationary down up to this batch, expert-major above

enum Slot { S_FRONT = 0, S_TOPK = 1, S_GATEUP = 2, S_SHARED = 3, S_DOWN = 4, S_LAYER = 5, S_COMBINE = 6,
            S_EXPERTS = 7, S_COUNT = 8 };
const char* kSlotNames[S_COUNT] = {"front", "topk_bucket", "gateup_routed", "gateup_shared", "down_combine",
                                   "layer", "combine", "experts"};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Argument blocks and kernel picks of one forward; the pointer fields are
// refreshed when the caller's pointers change.
struct Launches {
    FrontArgs fa{};
    GateUpArgs ga{};
    TopkArgs ta{};        // top-k launch (router part refreshed per forward)
    SelGateUpArgs sga{};  // gate/up launch of the select-in-gate/up form
    DownArgs da{};        // down of the single launch / output-stationary down
    DownXArgs dx{};       // expert-major down of the staged launches
    LayerArgs la{};
    InitArgs ia{};        // per-call set-up of the allocation-free forward
    FusedArgs fb{};       // batch 1: the routed experts, shared down and combine in one launch
    FrontArgs fbf{};      // batch 1: its router launch (router rows, shared gate/up pairs, sync re-arm)
    KernelPick kf{}, kt{}, kg{}, ks{}, kd{}, kl{}, kc{}, ki{}, kb{}, kbf{};
};

struct Layout {
    size_t meta, z, zacc, topk_idx, topk_w, act_e, act_off, perm, sh_act_e, sh_act_off, sh_perm;
    size_t h, hs, g_acc, g_acc_s, tile_cnt, tile_cnt_s, s_out, part, part_s, spart, total;
    size_t sync;      // counters and flags of the batch-1 experts launch
    size_t zero_end;  // [sync, zero_end): counters, flags, split-K partials and tile counters, zero between uses
};

}  // namespace

struct moe_decode_plan_s {
    moe_decode_config cfg;
    int variant;
    int mfma_min;         // routed experts with >= this many tokens use MFMA tiles; 0 = never
    int routed_gemv_tb;   // largest token count of a routed GEMV tile
    bool shared_mfma;
    int max_act;          // min(E, B*k)
    int ksplit, kslice;
    int dks, dsteps;      // dense front (batch > 4): K splits and 32-wide steps per split
    int dks_r, dsteps_r;  // the same for its router tiles
    bool small_router;    // batch <= 4: one router launch; else MFMA router + top-k launch
    bool shared_stream;   // shared gate/up on the second stream instead of the front launch
    bool select_in_router;// batch <= 4: top-k + bucketing in the router's last workgroup
    bool select_in_gateup;// batch <= 4: every routed gate/up workgroup selects and buckets
    bool shared_in_gateup;// that form also runs the shared gate/up row pairs (one per workgroup)
    bool fused;           // the whole layer as one persistent launch (batch <= 4, on request)
    bool fused_small;     // batch 1-2: router launch + one fused experts launch (fused_experts_kernel)
    int fb_grid = 0;      // its workgroups on this device (0 until resolved)
    int sel_grid = 0;     // select-in-gate/up form: workgroups the device holds at once (0 until known)
    bool expert_major;    // staged down: expert-major tiles + combine launch (else output-stationary)
    size_t layer_lds;     // its dynamic LDS bytes
    int layer_grid = 0;   // its workgroups (set on the first forward)
    Layout L;

    // device state (first forward)
    bool ready = false;
    int device = -1;
    char* ws = nullptr;
    hipStream_t s2 = nullptr;
    hipEvent_t ev_fork = nullptr, ev_join = nullptr;

    // argument blocks over the plan's workspace (m) and over the device's
    // static scratch array (na, the allocation-free forward)
    Launches m{}, na{};
    char* na_ws = nullptr;      // the scratch the na blocks point into
    const void* na_for[7] = {};
    const char* last_ws = nullptr;  // workspace of the last forward (routing / stats read it)

    // graph
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    hipGraphNode_t n_front = nullptr, n_topk = nullptr, n_gateup = nullptr, n_shared = nullptr,
                   n_down = nullptr, n_layer = nullptr, n_combine = nullptr;
    // x, router_w, expert_w, shared_w, out, next router_w, next shared_w
    const void* args_for[7] = {};   // in the arg blocks
    const void* graph_for[7] = {};  // in the graph exec
    bool have_forward = false;
    bool m_valid = false;  // the m blocks hold the pointers in args_for
    hipStream_t last_stream = nullptr;  // the stream of the last forward

    // profiling
    bool profiling = false;
    std::vector<hipEvent_t> prof_events;  // [forward][slot][start,end]
    int prof_count = 0;
};

namespace {

bool has_shared(const moe_decode_plan_s* p) { return p->cfg.shared_inter > 0; }
// top-k and bucketing in a launch of their own (batch > 4, or topk_launch = 2)
bool topk_own_launch(const moe_decode_plan_s* p) { return !p->select_in_router && !p->select_in_gateup; }
// the shared expert's gate/up in trailing workgroups of the front launch
bool shared_in_front(const moe_decode_plan_s* p) { return has_shared(p) && !p->shared_stream; }


// The fused experts launch (batch 1-2) needs all of its workgroups resident at
// once: its grid, sized from what the occupancy allows on the current device.
// Falls back to the staged launches (fused_small = false) where it does not fit.
FusedArgs fused_shape(const moe_decode_config& c) {
    FusedArgs f{};
    f.H = c.hidden;
    f.E = c.n_experts;
    f.k = c.top_k;
    f.I = c.inter;
    f.Is = c.shared_inter;
    f.B = c.batch;
    return f;
}

moe_status resolve_fused_small(moe_decode_plan_s* p) {
    if (!p->fused_small || p->fb_grid) return MOE_OK;
    const FusedArgs f = fused_shape(p->cfg);
    KernelPick k = pick_fused_experts(f, 1 << 30);
    if (!k.func) {
        p->fused_small = false;
        return MOE_OK;
    }
    int dev = 0, per_cu = 0, cus = 0;
    HIP_TRY(hipGetDevice(&dev));
    HIP_TRY(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k.func, 256, 0));
    HIP_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    k = pick_fused_experts(f, per_cu * cus);
    if (!k.func) {
        p->fused_small = false;
        return MOE_OK;
    }
    p->fb_grid = (int)k.grid.x;
    return MOE_OK;
}

moe_status validate(const moe_decode_config* c) {
    if (!c) return fail(MOE_ERR_INVALID, "config is NULL");
    if (c->hidden < 1 || c->n_experts < 1 || c->top_k < 1 || c->inter < 1 || c->batch < 1 ||
        c->shared_inter < 0)
        return fail(MOE_ERR_INVALID, "sizes must be positive (hidden %d, experts %d, top_k %d, "
                    "inter %d, batch %d, shared_inter %d)", c->hidden, c->n_experts, c->top_k,
                    c->inter, c->batch, c->shared_inter);
    if (c->top_k > c->n_experts)
        return fail(MOE_ERR_INVALID, "top_k %d exceeds n_experts %d", c->top_k, c->n_experts);
    if (c->score_fn != MOE_SCORE_SOFTMAX && c->score_fn != MOE_SCORE_SIGMOID)
        return fail(MOE_ERR_INVALID, "score_fn %d is not a moe_score_fn", c->score_fn);
    if ((c->renormalize != 0 && c->renormalize != 1) || (c->add_residual != 0 && c->add_residual != 1))
        return fail(MOE_ERR_INVALID, "renormalize and add_residual must be 0 or 1");
    if (!std::isfinite(c->routed_scale))
        return fail(MOE_ERR_INVALID, "routed_scale must be finite");
    if (c->force_variant < MOE_VARIANT_AUTO || c->force_variant > MOE_VARIANT_SPLIT_K)
        return fail(MOE_ERR_INVALID, "force_variant %d is not a moe_variant", c->force_variant);
    if (c->mfma_min_tokens < 0)
        return fail(MOE_ERR_INVALID, "mfma_min_tokens must be >= 0");
    if (c->shared_stream != 0 && c->shared_stream != 1)
        return fail(MOE_ERR_INVALID, "shared_stream must be 0 or 1");
    if (c->topk_launch < 0 || c->topk_launch > 3)
        return fail(MOE_ERR_INVALID, "topk_launch must be 0, 1, 2 or 3");
    if (c->single_launch < 0 || c->single_launch > 2)
        return fail(MOE_ERR_INVALID, "single_launch must be 0, 1 or 2");
    if (c->router_bias && (reinterpret_cast<uintptr_t>(c->router_bias) & 3))
        return fail(MOE_ERR_INVALID, "router_bias must be 4-byte aligned");
    // shapes the kernels cover
    if (c->hidden % 64 || c->hidden > 16384)
        return fail(MOE_ERR_UNSUPPORTED, "hidden %d: need a multiple of 64 up to 16384", c->hidden);
    if (c->n_experts > kMaxExperts)
        return fail(MOE_ERR_UNSUPPORTED, "n_experts %d > %d", c->n_experts, kMaxExperts);
    if (c->top_k > kMaxTopK) return fail(MOE_ERR_UNSUPPORTED, "top_k %d > %d", c->top_k, kMaxTopK);
    if (c->batch > kMaxBatch) return fail(MOE_ERR_UNSUPPORTED, "batch %d > %d", c->batch, kMaxBatch);
    const int I = c->inter;
    const bool i_ok = (I == 64 || I == 128 || I == 256) || (I % 512 == 0 && I <= 4096);
    if (!i_ok)
        return fail(MOE_ERR_UNSUPPORTED, "inter %d: need 64, 128, 256 or a multiple of 512 up to 4096", I);
    if (c->shared_inter && (c->shared_inter % I || c->shared_inter > 8 * 4096))
        return fail(MOE_ERR_UNSUPPORTED, "shared_inter %d: need 0 or a multiple of inter %d", c->shared_inter, I);
    return MOE_OK;
}

Layout make_layout(const moe_decode_config& c, int max_act, bool split, bool fused, bool expert_major, int nzpart,
                   int nspart) {
    const size_t B = c.batch, E = c.n_experts, k = c.top_k, I = c.inter, Is = c.shared_inter;
    Layout L{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t r = o;
        o = align_up(o + bytes, 256);
        return r;
    };
    L.meta = take(M_COUNT * 4);
    L.z = take(B * E * 4);
    L.zacc = take((size_t)nzpart * B * E * 4);
    L.topk_idx = take(B * k * 4);
    L.topk_w = take(B * k * 4);
    L.act_e = take((size_t)max_act * 4);
    L.act_off = take(((size_t)max_act + 1) * 4);
    L.perm = take(B * k * 4);
    L.sh_act_e = take(4);
    L.sh_act_off = take(8);
    L.sh_perm = take(B * 4);
    L.h = take(B * k * I * 4);
    L.hs = take(B * (Is ? Is : 1) * 4);
    L.sync = take((size_t)kSyncWords * 4);
    if (split) {
        L.g_acc = take(B * k * 2 * I * 4);
        L.g_acc_s = take(B * 2 * (Is ? Is : 1) * 4);
        L.tile_cnt = take((size_t)max_act * (I / kPairsPerMfmaTile) * 4);
        L.tile_cnt_s = take((Is / kPairsPerMfmaTile + 1) * 4);
    }
    L.zero_end = o;
    if (fused && Is) L.s_out = take(B * c.hidden * 4);
    if (expert_major) {  // per-pair / per-shared-block partials of the expert-major down
        L.part = take(B * k * c.hidden * 4);
        L.part_s = take((Is / I) * B * c.hidden * 4 + 4);
    }
    if (nspart) L.spart = take((size_t)nspart * B * 2 * Is * 4);
    L.total = o;
    return L;
}

template <class T>
T* at(char* ws, size_t off) {
    return reinterpret_cast<T*>(ws + off);
}

// Fills the argument blocks whose pointers do not depend on the caller, over
// the workspace `ws` (laid out as p->L).  clear: the set-up launch also clears
// the counters and split-K partials (a workspace another plan may have used).
void fill_static_args(moe_decode_plan_s* p, char* ws, Launches& A, bool clear) {
    const moe_decode_config& c = p->cfg;
    const bool split = p->variant == MOE_VARIANT_SPLIT_K;
    A.ia = InitArgs{at<int32_t>(ws, p->L.meta), at<int32_t>(ws, p->L.sh_act_e), at<int32_t>(ws, p->L.sh_act_off),
                    at<int32_t>(ws, p->L.sh_perm), c.batch, clear ? 1 : 0,
                    clear ? at<uint32_t>(ws, p->L.sync) : nullptr,
                    clear ? (long long)((p->L.zero_end - p->L.sync) / 4) : 0};
    A.ki = pick_init(A.ia);
    RouterArgs& r = A.fa.r;
    r.bias = c.router_bias;
    r.z = at<float>(ws, p->L.z);
    r.zacc = at<float>(ws, p->L.zacc);
    r.nzpart = p->small_router ? 1 : p->dks_r;
    r.topk_idx = at<int32_t>(ws, p->L.topk_idx);
    r.topk_w = at<float>(ws, p->L.topk_w);
    r.meta = at<int32_t>(ws, p->L.meta);
    r.act_e = at<int32_t>(ws, p->L.act_e);
    r.act_off = at<int32_t>(ws, p->L.act_off);
    r.perm = at<int32_t>(ws, p->L.perm);
    r.H = c.hidden;
    r.E = c.n_experts;
    r.k = c.top_k;
    r.B = c.batch;
    r.score_fn = c.score_fn;
    r.renormalize = c.renormalize;
    r.routed_scale = c.routed_scale;
    r.mfma_min_tokens = p->mfma_min;
    r.tiles_per_expert = c.inter / kPairsPerGemvTile;
    r.mfma_tiles_per_expert = (c.inter / kPairsPerMfmaTile) * p->ksplit;

    GateUpArgs& g = A.ga;
    g.expert_stride = 2LL * c.inter * c.hidden;
    g.n_act = at<int32_t>(ws, p->L.meta) + M_NACT;
    g.act_e = r.act_e;
    g.act_off = r.act_off;
    g.perm = r.perm;
    g.pair_div = c.top_k;
    g.h = at<float>(ws, p->L.h);
    g.g_acc = split ? at<float>(ws, p->L.g_acc) : nullptr;
    g.tile_cnt = split ? at<uint32_t>(ws, p->L.tile_cnt) : nullptr;
    g.meta = r.meta;
    g.H = c.hidden;
    g.n = c.inter;
    g.n_experts = c.n_experts;
    g.max_slots = c.batch * c.top_k;
    g.tiles_per_expert = c.inter / kPairsPerGemvTile;
    g.mfma_min_tokens = p->mfma_min;
    g.ksplit = p->ksplit;
    g.kslice = p->kslice;

    if (has_shared(p)) {
        GateUpArgs& s = A.fa.s;
        s.expert_stride = 0;
        s.n_act = at<int32_t>(ws, p->L.meta) + M_SHARED_NACT;
        s.act_e = at<int32_t>(ws, p->L.sh_act_e);
        s.act_off = at<int32_t>(ws, p->L.sh_act_off);
        s.perm = at<int32_t>(ws, p->L.sh_perm);
        s.pair_div = 1;
        s.h = at<float>(ws, p->L.hs);
        s.g_acc = split ? at<float>(ws, p->L.g_acc_s) : nullptr;
        s.tile_cnt = split ? at<uint32_t>(ws, p->L.tile_cnt_s) : nullptr;
        s.meta = r.meta;
        s.H = c.hidden;
        s.n = c.shared_inter;
        s.n_experts = 1;
        s.max_slots = c.batch;
        s.tiles_per_expert = c.shared_inter / kPairsPerGemvTile;
        s.mfma_min_tokens = p->shared_mfma ? 1 : 0;
        s.ksplit = p->ksplit;
        s.kslice = p->kslice;
    }

    // The select-in-gate/up form: the front computes one router row per
    // workgroup; the shared expert's gate/up row pairs run in the gate/up
    // launch (one per workgroup, during the selection) when it has enough
    // workgroups, else in the front, one pair per workgroup.
    A.fa.router_blocks = p->select_in_gateup ? c.n_experts
                          : p->small_router     ? front_router_blocks(r)
                                                : ((c.n_experts + 15) / 16) * p->dks_r;
    const bool sh_sel = p->shared_in_gateup;
    A.sga.shared_pairs = sh_sel ? c.shared_inter : 0;
    A.fa.shared_blocks = !shared_in_front(p) || sh_sel ? 0
                          : p->select_in_gateup ? c.shared_inter
                          : p->small_router     ? c.shared_inter / kPairsPerGemvTile
                                                : (2 * c.shared_inter / 16) * p->dks;
    A.fa.dks = p->dks;
    A.fa.dsteps = p->dsteps;
    A.fa.dks_r = p->dks_r;
    A.fa.dsteps_r = p->dsteps_r;
    A.fa.spart = p->L.spart ? at<float>(ws, p->L.spart) : nullptr;
    A.ta.spart = A.fa.spart;
    A.ta.hs = at<float>(ws, p->L.hs);
    A.ta.Is = c.shared_inter;
    A.ta.nspart = p->L.spart ? p->dks : 0;
    // top-k launch: up to batch 8 (and 64 pairs, bucketed by one wave) one
    // selecting workgroup with a wave per token (no hand-off between
    // workgroups), else one workgroup per four tokens
    A.ta.sel_blocks = c.batch <= kTopkOneGroupMaxBatch && c.batch * c.top_k <= 64 ? 1 : (c.batch + 3) / 4;

    {
        FusedArgs& f = A.fb;
        f.z = at<float>(ws, p->L.z);
        f.h = at<float>(ws, p->L.h);
        f.hs = at<float>(ws, p->L.hs);
        f.sync = at<int32_t>(ws, p->L.sync);
        f.topk_idx = r.topk_idx;
        f.topk_w = r.topk_w;
        f.meta = r.meta;
        f.act_e = r.act_e;
        f.act_off = r.act_off;
        f.perm = r.perm;
        f.H = c.hidden;
        f.E = c.n_experts;
        f.k = c.top_k;
        f.I = c.inter;
        f.Is = c.shared_inter;
        f.B = c.batch;
        f.score_fn = c.score_fn;
        f.renormalize = c.renormalize;
        f.routed_scale = c.routed_scale;
        f.add_residual = c.add_residual;
        f.rows = p->fb_grid ? (c.hidden + p->fb_grid - 1) / p->fb_grid : 0;
    }

    DownArgs& d = A.da;
    d.n_act = g.n_act;
    d.act_e = r.act_e;
    d.act_off = r.act_off;
    d.perm = r.perm;
    d.topk_w = r.topk_w;
    d.h = g.h;
    d.hs = at<float>(ws, p->L.hs);
    d.H = c.hidden;
    d.I = c.inter;
    d.Is = c.shared_inter;
    d.B = c.batch;
    d.k = c.top_k;
    d.add_residual = c.add_residual;
    d.n_experts = c.n_experts;
    d.h_in_lds = down_h_lds_bytes(c.batch, c.top_k, c.inter, c.shared_inter) <= kDownHLds ? 1 : 0;
    d.s_out = (p->fused && has_shared(p)) ? at<float>(ws, p->L.s_out) : nullptr;

    DownXArgs& x = A.dx;
    x.n_act = g.n_act;
    x.act_e = r.act_e;
    x.act_off = r.act_off;
    x.perm = r.perm;
    x.topk_w = r.topk_w;
    x.h = g.h;
    x.hs = d.hs;
    x.part = p->expert_major ? at<float>(ws, p->L.part) : nullptr;
    x.part_s = p->expert_major ? at<float>(ws, p->L.part_s) : nullptr;
    x.meta = r.meta;
    x.H = c.hidden;
    x.I = c.inter;
    x.Is = c.shared_inter;
    x.B = c.batch;
    x.k = c.top_k;
    x.add_residual = c.add_residual;
    x.n_experts = c.n_experts;
    x.max_act = p->max_act;
    x.nsh = c.shared_inter / c.inter;
    x.mfma_min_tokens = p->mfma_min;

    if (p->fused) {
        LayerArgs& l = A.la;
        const int R = down_rows_per_block(c.inter);
        l.n_router = (c.n_experts + 3) / 4;
        l.n_sgu = has_shared(p) ? c.shared_inter / kPairsPerGemvTile : 0;
        l.sgu_expect = !has_shared(p) ? 0
                       : p->shared_mfma ? (c.shared_inter / kPairsPerMfmaTile) * p->ksplit
                                        : c.shared_inter / kPairsPerGemvTile;
        l.n_sdown = has_shared(p) ? c.hidden / R : 0;
        l.n_gu = p->max_act * (c.inter / kPairsPerGemvTile);
        l.n_down = c.hidden / R;
        l.shared_mfma = p->shared_mfma ? 1 : 0;
    }
}

int layer_tasks(const LayerArgs& l) { return l.n_router + l.n_sgu + l.n_sdown + l.n_gu + l.n_down; }

void set_pointers(moe_decode_plan_s* p, Launches& A, const void* x, const void* router_w, const void* expert_w,
                  const void* shared_w, void* out, const void* next_router_w = nullptr,
                  const void* next_shared_w = nullptr) {
    const moe_decode_config& c = p->cfg;
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const uint16_t* ew = static_cast<const uint16_t*>(expert_w);
    const uint16_t* sw = static_cast<const uint16_t*>(shared_w);
    A.fa.r.x = xb;
    A.fa.r.wr = static_cast<const uint16_t*>(router_w);
    A.ga.x = xb;
    A.ga.w = ew;
    A.fa.s.x = xb;
    A.fa.s.w = sw;
    A.da.x = xb;
    A.da.w2 = ew + (size_t)c.n_experts * 2 * c.inter * c.hidden;
    A.da.s2 = has_shared(p) ? sw + (size_t)2 * c.shared_inter * c.hidden : nullptr;
    A.da.out = static_cast<uint16_t*>(out);
    A.dx.x = xb;
    A.dx.w2 = A.da.w2;
    A.dx.s2 = A.da.s2;
    A.dx.out = A.da.out;
    if (p->fused_small) {
        FusedArgs& f = A.fb;
        f.x = xb;
        f.w13 = ew;
        f.w2 = A.da.w2;
        f.s2 = A.da.s2;
        f.out = A.da.out;
        f.pf_a = static_cast<const uint16_t*>(next_router_w);
        f.pf_a_units = next_router_w ? (long long)c.n_experts * c.hidden / 8 : 0;
        f.pf_b = has_shared(p) ? static_cast<const uint16_t*>(next_shared_w) : nullptr;
        f.pf_b_units = f.pf_b ? 3LL * c.shared_inter * c.hidden / 8 : 0;
        A.kb = pick_fused_experts(f, p->fb_grid);
        // its router launch: one router row per workgroup, then one shared
        // gate/up row pair per workgroup; workgroup 0 re-arms the sync block
        A.fbf = A.fa;
        A.fbf.router_blocks = c.n_experts;
        A.fbf.shared_blocks = has_shared(p) ? c.shared_inter : 0;
        A.fbf.sync_clear = f.sync;
        A.fbf.sync_words = kSyncWords;
        A.kbf = pick_front_split(A.fbf);
    }
    if (p->select_in_gateup) {
        A.sga.r = A.fa.r;
        A.sga.g = A.ga;
        A.sga.s = A.fa.s;
        A.kf = pick_front_split(A.fa);
        A.kg = pick_gateup_select(A.sga, p->max_act);
        // a grid no larger than what the device holds at once: every workgroup
        // selects once, then loops over its tiles
        if (!p->sel_grid) {
            int dev = 0, per_cu = 0, cus = 0;
            if (hipGetDevice(&dev) == hipSuccess &&
                hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, A.kg.func, 256, A.kg.lds) == hipSuccess &&
                hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
                p->sel_grid = std::max(1, per_cu * cus);
        }
        if (p->sel_grid && (int)A.kg.grid.x > p->sel_grid) A.kg.grid.x = p->sel_grid;
    } else {
        A.kf = pick_front(A.fa, p->small_router, p->select_in_router, p->shared_mfma ? 0 : c.batch);
        if (topk_own_launch(p)) {
            A.ta.r = A.fa.r;
            A.kt = pick_topk(A.ta);
        }
        A.kg = pick_gateup(A.ga, p->max_act, p->routed_gemv_tb);
    }
    if (has_shared(p) && p->shared_stream) A.ks = pick_gateup(A.fa.s, 1, p->shared_mfma ? 1 : c.batch);
    if (p->expert_major) {
        A.kd = pick_down_x(A.dx);
        A.kc = pick_combine(A.dx);
    } else {
        A.kd = pick_down_os(A.da);
        if (!A.kd.func) A.kd = pick_down(A.da);
    }
    if (p->fused) {
        A.la.f = A.fa;
        A.la.g = A.ga;
        A.la.d = A.da;
        A.kl = pick_layer(A.la, p->layer_lds);
        A.kl.grid = dim3(p->layer_grid);
    }
}

// Frees what device_init created (any subset of it).
void release_device_state(moe_decode_plan_s* p) {
    if (p->ev_fork) (void)hipEventDestroy(p->ev_fork);
    if (p->ev_join) (void)hipEventDestroy(p->ev_join);
    if (p->s2) (void)hipStreamDestroy(p->s2);
    if (p->ws) (void)hipFree(p->ws);
    p->ev_fork = p->ev_join = nullptr;
    p->s2 = nullptr;
    p->ws = nullptr;
}

moe_status device_init_once(moe_decode_plan_s* p, hipStream_t stream, int dev);

moe_status device_init(moe_decode_plan_s* p, hipStream_t stream) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    if (p->ready) {
        if (dev != p->device)
            return fail(MOE_ERR_STATE, "plan was set up on device %d, current device is %d", p->device, dev);
        return MOE_OK;
    }
    const moe_status st = device_init_once(p, stream, dev);
    if (st != MOE_OK) {
        // leave nothing behind: a later forward starts from scratch
        (void)hipStreamSynchronize(stream);
        release_device_state(p);
    }
    return st;
}

moe_status device_init_once(moe_decode_plan_s* p, hipStream_t stream, int dev) {
    hipError_t e = hipMalloc(reinterpret_cast<void**>(&p->ws), p->L.total);
    if (e != hipSuccess) {
        p->ws = nullptr;
        return fail(MOE_ERR_NOMEM, "hipMalloc of %zu workspace bytes failed: %s", p->L.total,
                    hipGetErrorString(e));
    }
    p->device = dev;
    HIP_TRY(hipStreamCreateWithFlags(&p->s2, hipStreamNonBlocking));
    HIP_TRY(hipEventCreateWithFlags(&p->ev_fork, hipEventDisableTiming));
    HIP_TRY(hipEventCreateWithFlags(&p->ev_join, hipEventDisableTiming));
    // zero once: counters re-arm themselves and split-K partials are cleared after use
    HIP_TRY(hipMemsetAsync(p->ws, 0, p->L.total, stream));
    Launches& A = p->m;
    moe_status st = resolve_fused_small(p);
    if (st) return st;
    fill_static_args(p, p->ws, A, false);
    {
        void* args[] = {&A.ia};
        HIP_TRY(hipLaunchKernel(A.ki.func, A.ki.grid, A.ki.block, args, A.ki.lds, stream));
    }
    if (p->fused) {
        // every workgroup of the single launch must be resident at once: the grid is
        // what the occupancy allows on this device, capped at the task count
        const KernelPick k = pick_layer(A.la, p->layer_lds);
        if (!k.func) return fail(MOE_ERR_UNSUPPORTED, "no single-launch kernel for this shape");
        if (p->layer_lds > 64 * 1024)
            HIP_TRY(hipFuncSetAttribute(k.func, hipFuncAttributeMaxDynamicSharedMemorySize, (int)p->layer_lds));
        int per_cu = 0, cus = 0;
        HIP_TRY(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k.func, 256, p->layer_lds));
        HIP_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
        if (per_cu < 1 || cus < 1)
            return fail(MOE_ERR_UNSUPPORTED, "single-launch kernel does not fit a compute unit (%zu B LDS)",
                        p->layer_lds);
        p->layer_grid = std::min(layer_tasks(A.la), per_cu * cus);
    }
    p->ready = true;
    return MOE_OK;
}

void* gateup_args(moe_decode_plan_s* p, Launches& A) { return p->select_in_gateup ? (void*)&A.sga : (void*)&A.ga; }

moe_status launch(const KernelPick& k, void* args, hipStream_t s) {
    void* a[] = {args};
    HIP_TRY(hipLaunchKernel(k.func, k.grid, k.block, a, k.lds, s));
    return MOE_OK;
}

// Eager launch on the caller's stream (and, in shared_stream mode, the plan's
// second stream).  ev: per-slot start/end events for timing, or null.
moe_status enqueue_eager(moe_decode_plan_s* p, Launches& A, hipStream_t stream, hipEvent_t* ev) {
    moe_status st;
    if (p->fused_small) {
        if (ev) HIP_TRY(hipEventRecord(ev[2 * S_FRONT], stream));
        if ((st = launch(A.kbf, &A.fbf, stream))) return st;
        if (ev) HIP_TRY(hipEventRecord(ev[2 * S_FRONT + 1], stream));
        if (ev) HIP_TRY(hipEventRecord(ev[2 * S_EXPERTS], stream));
        if ((st = launch(A.kb, &A.fb, stream))) return st;
        if (ev) HIP_TRY(hipEventRecord(ev[2 * S_EXPERTS + 1], stream));
        return MOE_OK;
    }
    if (p->fused) {
        if (ev) HIP_TRY(hipEventRecord(ev[2 * S_LAYER], stream));
        if ((st = launch(A.kl, &A.la, stream))) return st;
        if (ev) HIP_TRY(hipEventRecord(ev[2 * S_LAYER + 1], stream));
        return MOE_OK;
    }
    const bool side = has_shared(p) && p->shared_stream;
    if (side) {
        HIP_TRY(hipEventRecord(p->ev_fork, stream));
        HIP_TRY(hipStreamWaitEvent(p->s2, p->ev_fork, 0));
        if (ev) HIP_TRY(hipEventRecord(ev[2 * S_SHARED], p->s2));
        if ((st = launch(A.ks, &A.fa.s, p->s2))) return st;
        if (ev) HIP_TRY(hipEventRecord(ev[2 * S_SHARED + 1], p->s2));
        HIP_TRY(hipEventRecord(p->ev_join, p->s2));
    }
    if (ev) HIP_TRY(hipEventRecord(ev[2 * S_FRONT], stream));
    if ((st = launch(A.kf, &A.fa, stream))) return st;
    if (ev) HIP_TRY(hipEventRecord(ev[2 * S_FRONT + 1], stream));
    if (topk_own_launch(p)) {
        if (ev) HIP_TRY(hipEventRecord(ev[2 * S_TOPK], stream));
        if ((st = launch(A.kt, &A.ta, stream))) return st;
        if (ev) HIP_TRY(hipEventRecord(ev[2 * S_TOPK + 1], stream));
    }
    if (ev) HIP_TRY(hipEventRecord(ev[2 * S_GATEUP], stream));
    if ((st = launch(A.kg, gateup_args(p, A), stream))) return st;
    if (ev) HIP_TRY(hipEventRecord(ev[2 * S_GATEUP + 1], stream));
    if (side) HIP_TRY(hipStreamWaitEvent(stream, p->ev_join, 0));
    if (ev) HIP_TRY(hipEventRecord(ev[2 * S_DOWN], stream));
    if ((st = launch(A.kd, p->expert_major ? (void*)&A.dx : (void*)&A.da, stream))) return st;
    if (ev) HIP_TRY(hipEventRecord(ev[2 * S_DOWN + 1], stream));
    if (p->expert_major) {
        if (ev) HIP_TRY(hipEventRecord(ev[2 * S_COMBINE], stream));
        if ((st = launch(A.kc, &A.dx, stream))) return st;
        if (ev) HIP_TRY(hipEventRecord(ev[2 * S_COMBINE + 1], stream));
    }
    return MOE_OK;
}

hipKernelNodeParams node_params(const KernelPick& k, void** args) {
    hipKernelNodeParams np{};
    np.blockDim = k.block;
    np.gridDim = k.grid;
    np.func = const_cast<void*>(k.func);
    np.kernelParams = args;
    np.sharedMemBytes = (unsigned int)k.lds;
    np.extra = nullptr;
    return np;
}

moe_status build_graph(moe_decode_plan_s* p) {
    Launches& A = p->m;
    HIP_TRY(hipGraphCreate(&p->graph, 0));
    if (p->fused_small) {
        void* af[] = {&A.fbf};
        void* ae[] = {&A.fb};
        hipKernelNodeParams np = node_params(A.kbf, af);
        HIP_TRY(hipGraphAddKernelNode(&p->n_front, p->graph, nullptr, 0, &np));
        np = node_params(A.kb, ae);
        HIP_TRY(hipGraphAddKernelNode(&p->n_layer, p->graph, &p->n_front, 1, &np));
        HIP_TRY(hipGraphInstantiate(&p->exec, p->graph, nullptr, nullptr, 0));
        return MOE_OK;
    }
    if (p->fused) {
        void* al[] = {&A.la};
        hipKernelNodeParams np = node_params(A.kl, al);
        HIP_TRY(hipGraphAddKernelNode(&p->n_layer, p->graph, nullptr, 0, &np));
        HIP_TRY(hipGraphInstantiate(&p->exec, p->graph, nullptr, nullptr, 0));
        return MOE_OK;
    }
    void* af[] = {&A.fa};
    void* ar[] = {&A.ta};
    void* ag[] = {gateup_args(p, A)};
    void* as[] = {&A.fa.s};
    void* ad[] = {p->expert_major ? (void*)&A.dx : (void*)&A.da};
    void* ac[] = {&A.dx};
    hipKernelNodeParams np = node_params(A.kf, af);
    HIP_TRY(hipGraphAddKernelNode(&p->n_front, p->graph, nullptr, 0, &np));
    hipGraphNode_t route_done = p->n_front;
    if (topk_own_launch(p)) {
        np = node_params(A.kt, ar);
        HIP_TRY(hipGraphAddKernelNode(&p->n_topk, p->graph, &p->n_front, 1, &np));
        route_done = p->n_topk;
    }
    np = node_params(A.kg, ag);
    HIP_TRY(hipGraphAddKernelNode(&p->n_gateup, p->graph, &route_done, 1, &np));
    hipGraphNode_t deps[2] = {p->n_gateup, nullptr};
    int ndeps = 1;
    if (has_shared(p) && p->shared_stream) {
        np = node_params(A.ks, as);
        HIP_TRY(hipGraphAddKernelNode(&p->n_shared, p->graph, nullptr, 0, &np));
        deps[ndeps++] = p->n_shared;
    }
    np = node_params(A.kd, ad);
    HIP_TRY(hipGraphAddKernelNode(&p->n_down, p->graph, deps, ndeps, &np));
    if (p->expert_major) {
        np = node_params(A.kc, ac);
        HIP_TRY(hipGraphAddKernelNode(&p->n_combine, p->graph, &p->n_down, 1, &np));
    }
    HIP_TRY(hipGraphInstantiate(&p->exec, p->graph, nullptr, nullptr, 0));
    return MOE_OK;
}

moe_status patch_graph(moe_decode_plan_s* p) {
    Launches& A = p->m;
    if (p->fused_small) {
        void* af[] = {&A.fbf};
        void* ae[] = {&A.fb};
        hipKernelNodeParams np = node_params(A.kbf, af);
        HIP_TRY(hipGraphExecKernelNodeSetParams(p->exec, p->n_front, &np));
        np = node_params(A.kb, ae);
        HIP_TRY(hipGraphExecKernelNodeSetParams(p->exec, p->n_layer, &np));
        return MOE_OK;
    }
    if (p->fused) {
        void* al[] = {&A.la};
        hipKernelNodeParams np = node_params(A.kl, al);
        HIP_TRY(hipGraphExecKernelNodeSetParams(p->exec, p->n_layer, &np));
        return MOE_OK;
    }
    void* af[] = {&A.fa};
    void* ar[] = {&A.ta};
    void* ag[] = {gateup_args(p, A)};
    void* as[] = {&A.fa.s};
    void* ad[] = {p->expert_major ? (void*)&A.dx : (void*)&A.da};
    void* ac[] = {&A.dx};
    hipKernelNodeParams np = node_params(A.kf, af);
    HIP_TRY(hipGraphExecKernelNodeSetParams(p->exec, p->n_front, &np));
    if (topk_own_launch(p)) {
        np = node_params(A.kt, ar);
        HIP_TRY(hipGraphExecKernelNodeSetParams(p->exec, p->n_topk, &np));
    }
    np = node_params(A.kg, ag);
    HIP_TRY(hipGraphExecKernelNodeSetParams(p->exec, p->n_gateup, &np));
    if (has_shared(p) && p->shared_stream) {
        np = node_params(A.ks, as);
        HIP_TRY(hipGraphExecKernelNodeSetParams(p->exec, p->n_shared, &np));
    }
    np = node_params(A.kd, ad);
    HIP_TRY(hipGraphExecKernelNodeSetParams(p->exec, p->n_down, &np));
    if (p->expert_major) {
        np = node_params(A.kc, ac);
        HIP_TRY(hipGraphExecKernelNodeSetParams(p->exec, p->n_combine, &np));
    }
    return MOE_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const char* x = static_cast<const char*>(a);
    const char* y = static_cast<const char*>(b);
    return x < y + nb && y < x + na;
}

bool misaligned(const void* p) { return reinterpret_cast<uintptr_t>(p) & 15; }

moe_status check_forward_args(const moe_decode_plan_s* p, const void* x, const void* router_w,
                              const void* expert_w, const void* shared_w, const void* out) {
    if (!p) return fail(MOE_ERR_INVALID, "plan is NULL");
    const moe_decode_config& c = p->cfg;
    if (!x || !router_w || !expert_w || !out || (c.shared_inter > 0 && !shared_w))
        return fail(MOE_ERR_INVALID, "NULL tensor pointer");
    if (misaligned(x) || misaligned(router_w) || misaligned(expert_w) || misaligned(out) ||
        (c.shared_inter > 0 && misaligned(shared_w)))
        return fail(MOE_ERR_INVALID, "tensor pointers must be 16-byte aligned");
    const size_t act_bytes = (size_t)c.batch * c.hidden * 2;
    if (overlaps(x, act_bytes, out, act_bytes)) return fail(MOE_ERR_INVALID, "out overlaps x");
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_decode_plan(const moe_decode_config* cfg, moe_decode_plan_t* out_plan) {
    g_err.clear();
    if (!out_plan) return fail(MOE_ERR_INVALID, "out_plan is NULL");
    *out_plan = nullptr;
    moe_status st = validate(cfg);
    if (st) return st;
    moe_decode_plan_s* p = new (std::nothrow) moe_decode_plan_s();
    if (!p) return fail(MOE_ERR_NOMEM, "host allocation of the plan failed");
    p->cfg = *cfg;
    const moe_decode_config& c = p->cfg;
    // a GEMV tile stages its tokens' activations in LDS: at most this many tokens
    const int gemv_cap = (int)(kGemvLdsBytes / ((size_t)2 * c.hidden));
    // AUTO: small-matrix tiles at batch <= 2 where their activations fit the
    // LDS budget, split-K otherwise
    p->variant = c.force_variant != MOE_VARIANT_AUTO ? c.force_variant
                 : (c.batch <= 2 && c.batch <= gemv_cap ? MOE_VARIANT_SMALL_M : MOE_VARIANT_SPLIT_K);
    if (p->variant == MOE_VARIANT_SPLIT_K) {
        p->mfma_min = c.mfma_min_tokens                                          ? c.mfma_min_tokens
                      : c.batch > kSmallRouterMaxBatch && c.batch <= kMfmaMinSmallMaxBatch ? kDefaultMfmaMinSmall
                                                                                           : kDefaultMfmaMin;
        if (p->mfma_min > kMaxBatch + 1) p->mfma_min = kMaxBatch + 1;
        if (p->mfma_min > gemv_cap + 1) p->mfma_min = std::max(1, gemv_cap + 1);
        p->routed_gemv_tb = std::max(1, std::min(c.batch, p->mfma_min - 1));
        p->shared_mfma = c.batch >= p->mfma_min;
    } else {
        if (c.batch > gemv_cap) {
            delete p;
            return fail(MOE_ERR_UNSUPPORTED, "SMALL_M at batch %d needs %d bytes of LDS per workgroup "
                        "(limit %d); use SPLIT_K", c.batch, 2 * c.batch * c.hidden, kGemvLdsBytes);
        }
        p->mfma_min = 0;
        p->routed_gemv_tb = c.batch;
        p->shared_mfma = false;
    }
    p->small_router = c.batch <= kSmallRouterMaxBatch &&
                      (size_t)2 * c.batch * c.hidden <= kSmallRouterLds;
    p->shared_stream = c.shared_stream != 0;
    p->select_in_router = p->small_router && c.topk_launch != 2;
    p->max_act = std::min(c.n_experts, c.batch * c.top_k);
    // K split of an MFMA row block: the most splits <= 16 that divide H into multiples of 32
    p->ksplit = 1;
    for (int s = kSplitK; s >= 1; --s)
        if (c.hidden % (32 * s) == 0) { p->ksplit = s; break; }
    p->kslice = c.hidden / p->ksplit;
    // dense front: the fewest K splits (<= 32) that leave at most 16 steps of
    // 32 per split (one round of loads per wave), else the most splits <= 32
    {
        const int steps = c.hidden / 32;
        int d = 0;
        for (int s = 1; s <= 32 && !d; ++s)
            if (steps % s == 0 && steps / s <= 16) d = s;
        if (!d)
            for (int s = 32; s >= 1 && !d; --s)
                if (steps % s == 0) d = s;
        p->dks = d;
        p->dsteps = steps / d;
        // router tiles: the fewest splits that leave at most 32 steps (two
        // load rounds), so the top-k launch sums at most 8 partials in one round
        int dr = 0;
        for (int s = 1; s <= 32 && !dr; ++s)
            if (steps % s == 0 && steps / s <= 32) dr = s;
        if (!dr) dr = d;
        p->dks_r = dr;
        p->dsteps_r = steps / dr;
    }
    // single launch: batch <= 4, activations and every h row fit the LDS budget,
    // a down shape with an instantiation (I = 64, 128, 256 or 512..2048)
    {
        const size_t x_lds = (size_t)2 * c.batch * c.hidden;
        const size_t h_lds = down_h_lds_bytes(c.batch, c.top_k, c.inter, c.shared_inter);
        const int ur = c.inter / 8;
        const bool shape_ok = ur == 8 || ur == 16 || ur == 32 || (ur % 64 == 0 && ur / 64 <= 4);
        const char* why = nullptr;
        if (c.batch > kSmallRouterMaxBatch) why = "batch > 4";
        else if (!p->small_router) why = "activations exceed the LDS budget";
        else if (h_lds > kLayerLds) why = "the h rows exceed the LDS budget";
        else if (!shape_ok) why = "no down shape for this inter";
        else if (c.shared_stream) why = "shared_stream = 1 asks for the staged launches";
        else if (c.topk_launch == 2 || c.topk_launch == 3) why = "topk_launch = 2 or 3 asks for the staged launches";
        // measured slower than the staged launches on MI355X (one workgroup per
        // CU and a latency-inflated critical path), so only on request
        p->fused = c.single_launch == 2 && !why;
        p->layer_lds = std::max(x_lds, h_lds);
        if (c.single_launch == 2 && why) {
            delete p;
            return fail(MOE_ERR_UNSUPPORTED, "single_launch = 2: %s", why);
        }
    }
    // Batch <= 4: the selection runs in every routed gate/up workgroup
    // (topk_launch 3) by default.  That form runs every tile as a GEMV tile,
    // so with the library's MFMA threshold it turns MFMA tiles off; a
    // threshold the caller set that could reach MFMA tiles keeps the selection
    // in the router's last workgroup (topk_launch 1) unless 3 is asked for.
    // Its grid is capped at what the device holds at once and each workgroup
    // loops over its tiles, so the selection is paid once per workgroup, not
    // once per tile (a grid of one tile per workgroup, two generations at
    // batch 2, measured 61.0 us against 58.8 us selecting in the router).
    p->select_in_gateup = false;
    if (!p->fused && p->small_router && (c.topk_launch == 3 || c.topk_launch == 0)) {
        const bool gemv_only = !p->shared_mfma && (p->mfma_min == 0 || p->mfma_min > c.batch);
        if (gemv_only || c.mfma_min_tokens == 0) {
            p->select_in_gateup = true;
            p->mfma_min = 0;
            p->shared_mfma = false;
            p->routed_gemv_tb = c.batch;
            p->select_in_router = false;
        } else if (c.topk_launch == 3) {
            delete p;
            return fail(MOE_ERR_UNSUPPORTED, "topk_launch = 3 runs GEMV tiles only; mfma_min_tokens %d "
                        "reaches MFMA tiles at batch %d", c.mfma_min_tokens, c.batch);
        }
    } else if (c.topk_launch == 3 && !p->fused) {
        delete p;
        return fail(MOE_ERR_UNSUPPORTED, "topk_launch = 3 needs batch <= 4 with x in the LDS budget");
    }
    // the shared expert's row pairs ride in the first gate/up workgroups (one
    // pair each, streaming during their selection) where there are enough of
    // them: the grid is the routed tiles, capped at one generation
    p->shared_in_gateup = p->select_in_gateup && shared_in_front(p) &&
                          (size_t)c.shared_inter <= std::min((size_t)p->max_act * (c.inter / kPairsPerGemvTile),
                                                             kSelectGateupMaxTiles);
    // Batch 1-2: the router launch and one fused experts launch where the
    // shape has such a kernel (GEMV tiles only: no MFMA threshold the batch
    // reaches), unless the caller asks for another form.  Whether its grid
    // fits the device is checked at the first forward (else the staged
    // launches run).
    p->fused_small = c.batch <= 2 && !p->fused && c.single_launch == 0 && !p->shared_stream && c.topk_launch == 0 &&
                  !p->shared_mfma && (p->mfma_min == 0 || p->mfma_min > c.batch) &&
                  pick_fused_experts(fused_shape(c), 1 << 30).func != nullptr;
    p->expert_major = c.batch > kDownOsMaxBatch;
    p->L = make_layout(c, p->max_act, p->variant == MOE_VARIANT_SPLIT_K, p->fused, p->expert_major,
                       p->small_router ? 1 : p->dks_r,
                       !p->small_router && c.shared_inter > 0 && !p->shared_stream ? p->dks : 0);
    *out_plan = p;
    return MOE_OK;
}

moe_status moe_decode_forward_prefetch(moe_decode_plan_t p, const void* x, const void* router_w,
                                       const void* expert_w, const void* shared_w, void* out,
                                       const void* next_router_w, const void* next_shared_w, void* stream_) {
    g_err.clear();
    moe_status st = check_forward_args(p, x, router_w, expert_w, shared_w, out);
    if (st) return st;
    if (misaligned(next_router_w) || misaligned(next_shared_w))
        return fail(MOE_ERR_INVALID, "next-layer pointers must be 16-byte aligned");
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    HIP_TRY(hipStreamIsCapturing(stream, &cap));
    if (cap == hipStreamCaptureStatusActive && !p->ready)
        return fail(MOE_ERR_STATE, "the first forward of a plan allocates and zeroes its workspace; "
                    "run it outside stream capture");
    st = device_init(p, stream);
    if (st) return st;
    if (!has_shared(p)) shared_w = nullptr;
    if (!has_shared(p)) next_shared_w = nullptr;
    const void* tuple[7] = {x, router_w, expert_w, shared_w, out, next_router_w, next_shared_w};
    if (!p->m_valid || std::memcmp(tuple, p->args_for, sizeof tuple) != 0) {
        set_pointers(p, p->m, x, router_w, expert_w, shared_w, out, next_router_w, next_shared_w);
        std::memcpy(p->args_for, tuple, sizeof tuple);
        p->m_valid = true;
    }
    p->have_forward = true;
    p->last_stream = stream;
    p->last_ws = p->ws;

    if (cap == hipStreamCaptureStatusActive) return enqueue_eager(p, p->m, stream, nullptr);  // into the caller's graph
    if (p->profiling) {
        if (p->prof_count >= kMaxProfiledForwards)
            return fail(MOE_ERR_STATE, "profiling records at most %d forwards", kMaxProfiledForwards);
        const size_t base = (size_t)p->prof_count * S_COUNT * 2;
        while (p->prof_events.size() < base + S_COUNT * 2) {
            hipEvent_t ev;  // timing events without the system-scope fence (device-local timing)
            HIP_TRY(hipEventCreateWithFlags(&ev, hipEventDisableSystemFence));
            p->prof_events.push_back(ev);
        }
        st = enqueue_eager(p, p->m, stream, &p->prof_events[base]);
        if (st) return st;
        ++p->prof_count;
        return MOE_OK;
    }
    if (!p->exec) {
        st = build_graph(p);
        if (st) return st;
        std::memcpy(p->graph_for, tuple, sizeof tuple);
    } else if (std::memcmp(tuple, p->graph_for, sizeof tuple) != 0) {
        st = patch_graph(p);
        if (st) return st;
        std::memcpy(p->graph_for, tuple, sizeof tuple);
    }
    HIP_TRY(hipGraphLaunch(p->exec, stream));
    return MOE_OK;
}

moe_status moe_decode_forward(moe_decode_plan_t p, const void* x, const void* router_w,
                              const void* expert_w, const void* shared_w, void* out, void* stream) {
    return moe_decode_forward_prefetch(p, x, router_w, expert_w, shared_w, out, nullptr, nullptr, stream);
}

moe_status moe_decode_forward_noalloc(moe_decode_plan_t p, const void* x, const void* router_w,
                                      const void* expert_w, const void* shared_w, void* out, void* stream_) {
    g_err.clear();
    moe_status st = check_forward_args(p, x, router_w, expert_w, shared_w, out);
    if (st) return st;
    if (p->fused)
        return fail(MOE_ERR_UNSUPPORTED, "the allocation-free forward runs the staged launches; this plan "
                    "asks for the single launch (single_launch = 2)");
    if (has_shared(p) && p->shared_stream)
        return fail(MOE_ERR_UNSUPPORTED, "the allocation-free forward runs on the caller's stream only; this "
                    "plan puts the shared expert on a second stream (shared_stream = 1)");
    if ((st = resolve_fused_small(p))) return st;
    void* scratch = nullptr;
    size_t scratch_bytes = 0;
    HIP_TRY(scratch_for_current_device(&scratch, &scratch_bytes));
    if (p->L.total > scratch_bytes)
        return fail(MOE_ERR_UNSUPPORTED, "the plan needs %zu bytes of scratch; the allocation-free forward "
                    "has %zu", p->L.total, scratch_bytes);
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    if (!has_shared(p)) shared_w = nullptr;
    const void* tuple[7] = {x, router_w, expert_w, shared_w, out, nullptr, nullptr};
    char* ws = static_cast<char*>(scratch);
    if (p->na_ws != ws) {
        fill_static_args(p, ws, p->na, true);
        p->na_ws = ws;
        set_pointers(p, p->na, x, router_w, expert_w, shared_w, out);
        std::memcpy(p->na_for, tuple, sizeof tuple);
    } else if (std::memcmp(tuple, p->na_for, sizeof tuple) != 0) {
        set_pointers(p, p->na, x, router_w, expert_w, shared_w, out);
        std::memcpy(p->na_for, tuple, sizeof tuple);
    }
    // the scratch holds whatever the device's last call left: clear the
    // counters and split-K partials and write the shared expert's work list
    if ((st = launch(p->na.ki, &p->na.ia, stream))) return st;
    if ((st = enqueue_eager(p, p->na, stream, nullptr))) return st;
    p->have_forward = true;
    p->last_stream = stream;
    p->last_ws = ws;
    return MOE_OK;
}

moe_status moe_decode_routing(moe_decode_plan_t p, int32_t* topk_idx, float* topk_w, int32_t* n_unique,
                              float* logits, void* stream_) {
    g_err.clear();
    if (!p) return fail(MOE_ERR_INVALID, "plan is NULL");
    if (!p->have_forward) return fail(MOE_ERR_STATE, "no forward has run on this plan");
    hipStream_t s = static_cast<hipStream_t>(stream_);
    const size_t n = (size_t)p->cfg.batch * p->cfg.top_k;
    const char* ws = p->last_ws;
    if (topk_idx) HIP_TRY(hipMemcpyAsync(topk_idx, ws + p->L.topk_idx, n * 4, hipMemcpyDeviceToDevice, s));
    if (topk_w) HIP_TRY(hipMemcpyAsync(topk_w, ws + p->L.topk_w, n * 4, hipMemcpyDeviceToDevice, s));
    if (n_unique)
        HIP_TRY(hipMemcpyAsync(n_unique, ws + p->L.meta + 4 * M_NACT, 4, hipMemcpyDeviceToDevice, s));
    if (logits)
        HIP_TRY(hipMemcpyAsync(logits, ws + p->L.z, (size_t)p->cfg.batch * p->cfg.n_experts * 4,
                               hipMemcpyDeviceToDevice, s));
    return MOE_OK;
}

moe_status moe_decode_read_stats(moe_decode_plan_t p, moe_decode_stats* stats) {
    g_err.clear();
    if (!p || !stats) return fail(MOE_ERR_INVALID, "NULL argument");
    if (!p->have_forward) return fail(MOE_ERR_STATE, "no forward has run on this plan");
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    HIP_TRY(hipStreamIsCapturing(p->last_stream, &cap));
    if (cap != hipStreamCaptureStatusNone)
        return fail(MOE_ERR_STATE, "the last forward's stream is being captured; read the stats after replay");
    HIP_TRY(hipStreamSynchronize(p->last_stream));
    if (p->s2) HIP_TRY(hipStreamSynchronize(p->s2));
    int32_t meta[M_COUNT];
    HIP_TRY(hipMemcpy(meta, p->last_ws + p->L.meta, sizeof meta, hipMemcpyDeviceToHost));
    stats->n_unique = meta[M_NACT];
    stats->gemv_tiles = meta[M_GEMV_TILES];
    stats->mfma_tiles = meta[M_MFMA_TILES];
    stats->error_flags = meta[M_ERR];
    return MOE_OK;
}

moe_status moe_decode_plan_info(moe_decode_plan_t p, moe_decode_info* info) {
    g_err.clear();
    if (!p || !info) return fail(MOE_ERR_INVALID, "NULL argument");
    info->variant = p->variant;
    info->n_kernels = p->fused ? 1 : p->fused_small ? 2
                      : 3 + (topk_own_launch(p) ? 1 : 0) + (has_shared(p) && p->shared_stream ? 1 : 0) +
                            (p->expert_major ? 1 : 0);
    info->topk_launch = p->fused || p->fused_small ? 0 : p->select_in_gateup ? 3 : p->select_in_router ? 1 : 2;
    info->mfma_min_tokens = p->mfma_min;
    info->shared_mfma = p->shared_mfma ? 1 : 0;
    info->shared_stream = p->shared_stream ? 1 : 0;
    info->router_mfma = p->small_router ? 0 : 1;
    info->single_launch = p->fused ? 1 : p->fused_small ? 2 : 0;
    info->layer_grid = p->fused_small ? p->fb_grid : p->layer_grid;
    info->workspace_bytes = p->L.total;
    info->shared_gateup_in = !has_shared(p) ? 0 : p->fused ? 4 : p->fused_small ? 1 : p->shared_stream ? 3
                             : p->shared_in_gateup ? 2 : 1;
    return MOE_OK;
}

moe_status moe_decode_set_profiling(moe_decode_plan_t p, int32_t enable) {
    g_err.clear();
    if (!p) return fail(MOE_ERR_INVALID, "plan is NULL");
    if (p->ready) {
        HIP_TRY(hipDeviceSynchronize());
    }
    for (hipEvent_t e : p->prof_events) (void)hipEventDestroy(e);
    p->prof_events.clear();
    p->prof_count = 0;
    p->profiling = enable != 0;
    return MOE_OK;
}

moe_status moe_decode_profile_read(moe_decode_plan_t p, int32_t cap, double* total_ms, int32_t* launches,
                                   const char** names, int32_t* n) {
    g_err.clear();
    if (!p || !n || cap < 0 || (cap > 0 && (!total_ms || !launches)))
        return fail(MOE_ERR_INVALID, "bad argument");
    *n = S_COUNT;
    for (int s = 0; s < S_COUNT && s < cap; ++s) {
        total_ms[s] = 0.0;
        launches[s] = 0;
        if (names) names[s] = kSlotNames[s];
    }
    if (p->prof_count == 0) return MOE_OK;
    for (int f = 0; f < p->prof_count; ++f) {
        for (int s = 0; s < S_COUNT && s < cap; ++s) {
            const bool used = p->fused_small ? (s == S_FRONT || s == S_EXPERTS)
                              : p->fused ? s == S_LAYER
                              : !((s == S_SHARED && !(has_shared(p) && p->shared_stream)) ||
                                  (s == S_TOPK && !topk_own_launch(p)) || s == S_LAYER || s == S_EXPERTS ||
                                  (s == S_COMBINE && !p->expert_major));
            if (!used) continue;
            hipEvent_t a = p->prof_events[((size_t)f * S_COUNT + s) * 2];
            hipEvent_t b = p->prof_events[((size_t)f * S_COUNT + s) * 2 + 1];
            HIP_TRY(hipEventSynchronize(b));
            float ms = 0.0f;
            HIP_TRY(hipEventElapsedTime(&ms, a, b));
            total_ms[s] += ms;
            launches[s] += 1;
        }
    }
    return MOE_OK;
}

moe_status moe_decode_destroy(moe_decode_plan_t p) {
    g_err.clear();
    if (!p) return MOE_OK;
    moe_status st = MOE_OK;
    if (p->ready) {
        (void)hipSetDevice(p->device);
        if (hipDeviceSynchronize() != hipSuccess) st = fail(MOE_ERR_HIP, "synchronize before destroy failed");
        for (hipEvent_t e : p->prof_events) (void)hipEventDestroy(e);
        if (p->exec) (void)hipGraphExecDestroy(p->exec);
        if (p->graph) (void)hipGraphDestroy(p->graph);
        release_device_state(p);
    }
    delete p;
    return st;
}

const char* moe_decode_last_error(void) { return g_err.c_str(); }

}  // extern "C"
