// moe_kernels.hip -- gfx950 (CDNA4) kernels of the decode-time MoE layer,
// staged form (one launch per stage; the single-launch form for batch <= 4
// is in moe_layer.h).
//
// One layer is, on the main stream (batch 1-2: the router launch and the
// fused experts launch of moe_fused.hip instead):
//   front      batch 3-4: front_split -- one router row per workgroup, logits to
//              z (and, where the gate/up launch has too few workgroups for
//              them, the shared expert's gate/up row pairs); the routed gate/up
//              launch then selects and buckets in every workgroup
//              (gateup_select);
//              batch > 4: front_dense -- dense split-K MFMA tiles writing plain
//              fp32 partial logits (no atomics) and the shared expert's gate/up
//              partials -- then topk_bucket -- which sums the partials in a
//              fixed order, selects with one wave per token, and buckets (one
//              wave, or an LDS histogram) in its last workgroup;
//   gateup     grouped gate/up projection + SiLU*up over the active experts:
//              GEMV tiles (full K, VALU dot2) for experts with few tokens -- the
//              "small-matrix" form the Kimi K3 decode article uses at batch 1-2
//              -- and split-K MFMA tiles for experts with many tokens -- the
//              "split-K" form it uses at larger batches (Part 1 section 1);
//   down       down projection of every active expert and of the shared
//              expert, routing-weighted sum, residual add, bf16 output: at
//              batch 3-4 output-stationary (down_os: no atomics, fixed order);
//              above, expert-major tiles with fp32 partial rows and a combine
//              launch that sums them in a fixed order;
// or, with shared_stream = 1, the shared expert's gate/up on a second stream
// (same gateup kernel with a one-entry work list), joined before `down`
// (article Part 1 section 3: the shared expert on its own stream, overlapped
// with routing).
//
// Small-batch decode is bound by how fast weights stream from HBM (article
// Part 1 section 4).  Every weight-streaming loop therefore issues all of a
// wave's 16-byte weight loads for a batch of units before it consumes the
// first one, so a wave keeps up to 16 KiB in flight instead of waiting a
// memory round trip per unit.  Hand-offs between workgroups of one launch go
// through device-coherent stores and loads plus a counter (moe_device.h);
// hand-off data is only read after the counter was seen, and only static
// weights are loaded before that (article Part 2 section 3 reports a compiler
// hoisting activation loads above a wait as a real bug).
#include <algorithm>

#include "moe_device.h"

namespace moe {

// SELECT: the last router workgroup to arrive selects and buckets; otherwise
// the router writes raw logits to zacc and topk_bucket_kernel follows.
template <int TB, bool SH_MFMA, bool SELECT, int NS>
__global__ __launch_bounds__(256) void front_small_kernel(FrontArgs f) {
    extern __shared__ __align__(16) uint16_t s_x[];  // [B][H] activations
    const RouterArgs& a = f.r;
    if ((int)blockIdx.x >= f.router_blocks) {  // shared expert: all B tokens, weight 1
        const int local = blockIdx.x - f.router_blocks;
        if constexpr (SH_MFMA) mfma_gateup_tile<1>(f.s, f.s.w, 0, 0, a.B, local);
        else gemv_gateup_tile<TB>(f.s, f.s.w, 0, a.B, local, s_x);
        return;
    }
    __shared__ int32_t s_pair_e[4 * kMaxTopK];
    __shared__ __align__(16) int32_t s_ps[128];
    __shared__ int s_flag;

    router_rows<TB, SELECT>(a, blockIdx.x, s_x);
    if constexpr (!SELECT) return;

    // the last router workgroup to arrive selects and buckets
    if (!arrive_last(reinterpret_cast<unsigned*>(&a.meta[M_ROUTER_CNT]), f.router_blocks, &s_flag)) return;

    select_tokens<NS>(a, 0, a.z, nullptr, false, s_pair_e);
    if ((threadIdx.x >> 6) == 0) bucket_wave(a, s_pair_e, threadIdx.x & 63, s_ps);
}

// Dense split-K front (batch > 4): router tiles, then the shared expert's
// gate/up tiles (gate and up rows are independent rows here; the top-k launch
// pairs them).  Every tile is one round of loads: many small tiles keep the
// whole chip streaming the 12.8 MB of the TP8-shard shape at once.
template <int NT>
__global__ __launch_bounds__(256) void front_dense_kernel(FrontArgs f) {
    __shared__ float s_red[4 * NT * 4 * 64];
    const RouterArgs& a = f.r;
    const int b = blockIdx.x;
    if (b < f.router_blocks) {
        dense_splitk_tile<NT>(a.wr, a.E, a.x, a.B, a.H, f.dsteps_r, b / f.dks_r, b % f.dks_r, a.zacc, s_red);
    } else {
        const int l = b - f.router_blocks;
        dense_splitk_tile<NT>(f.s.w, 2 * f.s.n, a.x, a.B, a.H, f.dsteps, l / f.dks, l % f.dks, f.spart, s_red);
    }
}

// Logits = sum of the partial slices + bias, top-k, weights, bucketing.
// With one selecting workgroup (batch <= 4) everything stays in registers and
// LDS: no atomics, fences or reloads sit between reading the logits and
// writing the buckets.  With several, the last selecting workgroup to arrive
// buckets all pairs.  Workgroups from sel_blocks on reduce the shared
// expert's gate/up partials into h_s.
template <int NS>
__global__ __launch_bounds__(512) void topk_bucket_kernel(TopkArgs ta) {
    __shared__ int32_t s_pair_e[kMaxBatch * kMaxTopK];
    __shared__ int32_t s_rank[kMaxBatch * kMaxTopK];
    __shared__ int32_t s_cnt[kMaxExperts];
    __shared__ int32_t s_tmp[8];
    __shared__ int32_t s_nmfma;
    __shared__ __align__(16) int32_t s_ps[128];
    __shared__ int s_flag;
    const RouterArgs& a = ta.r;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if ((int)blockIdx.x >= ta.sel_blocks) {
        const int idx = (blockIdx.x - ta.sel_blocks) * blockDim.x + tid;
        const int Is = ta.Is, n2 = 2 * Is;
        if (idx >= a.B * Is) return;
        const int t = idx / Is, i = idx - t * Is;
        const size_t qs = (size_t)a.B * n2;
        const float* p = ta.spart + (size_t)t * n2 + i;
        float g = 0.0f, u = 0.0f;
        for (int q0 = 0; q0 < ta.nspart; q0 += 8) {
            float tg[8], tu[8];
#pragma unroll
            for (int qq = 0; qq < 8; ++qq) {
                const size_t q = (size_t)min(q0 + qq, ta.nspart - 1);
                tg[qq] = p[q * qs];
                tu[qq] = p[q * qs + Is];
            }
#pragma unroll
            for (int qq = 0; qq < 8; ++qq)
                if (q0 + qq < ta.nspart) {
                    g += tg[qq];
                    u += tu[qq];
                }
        }
        ta.hs[(size_t)t * Is + i] = silu_f(g) * u;
        return;
    }
    const int B = a.B, np = B * a.k;
    const bool single = ta.sel_blocks == 1;
    // one selecting workgroup (blockDim / 64 >= B waves, one token each: no
    // hand-off, no reload) or one per four tokens
    select_tokens<NS, false>(a, single ? 0 : blockIdx.x * 4, a.zacc, a.bias, true, single ? s_pair_e : nullptr);
    if (!single) {
        if (!arrive_last(reinterpret_cast<unsigned*>(&a.meta[M_ROUTER_CNT]), ta.sel_blocks, &s_flag)) return;
        for (int p = tid; p < np; p += 256) s_pair_e[p] = ld_dev(a.topk_idx + p);
        __syncthreads();
    }
    if (np <= 64) {
        if (wave == 0) bucket_wave(a, s_pair_e, lane, s_ps);
    } else {
        bucket_block(a, s_pair_e, s_rank, s_cnt, s_tmp, &s_nmfma);
    }
}

template <int TB, bool WITH_MFMA>
__global__ __launch_bounds__(256) void gateup_kernel(GateUpArgs a) {
    extern __shared__ __align__(16) uint16_t s_x[];  // [TB][H] (GEMV tiles)
    const int entry = blockIdx.x / a.tiles_per_expert;
    const int local = blockIdx.x % a.tiles_per_expert;
    if (entry >= *a.n_act) return;
    const int e = a.act_e[entry];
    const int off = a.act_off[entry];
    const int T = a.act_off[entry + 1] - off;
    if (e < 0 || e >= a.n_experts || off < 0 || T < 1 || off + T > a.max_slots) {
        if (threadIdx.x == 0 && local == 0) atomicOr(&a.meta[M_ERR], ERR_TILE);
        return;
    }
    const uint16_t* W = a.w + (size_t)e * (size_t)a.expert_stride;
    if (WITH_MFMA && a.mfma_min_tokens > 0 && T >= a.mfma_min_tokens) {
        if (T > kMaxBatch) {
            if (threadIdx.x == 0 && local == 0) atomicOr(&a.meta[M_ERR], ERR_TILE);
            return;
        }
        mfma_gateup_tile_lds(a, W, entry, off, T, local, s_x);
    } else {
        if (T > TB) {
            if (threadIdx.x == 0 && local == 0) atomicOr(&a.meta[M_ERR], ERR_TILE);
            return;
        }
        gemv_gateup_tile<TB>(a, W, off, T, local, s_x);
    }
}


// ---------------------------------------------------------------------------
// batch <= 4 with the selection in the gate/up launch: router_split writes
// the logits, then every routed gate/up workgroup selects and buckets for
// itself, so no workgroup waits on another's counter and the shared expert's
// gate/up streams while the routed workgroups select
// ---------------------------------------------------------------------------

// Dot products of NR weight rows with the B <= TB token rows of x ([B][H]),
// K split over the workgroup's 256 threads in interleaved 16-byte units (the
// row loads are coalesced across the workgroup; x is a few KB per token and
// stays in L2).  The wave sums meet in s_part in a fixed order; every thread
// returns the totals.
template <int TB, int NR>
__device__ __forceinline__ void wg_rows_dot(const uint16_t* const (&w)[NR], const uint16_t* x, int H, int B,
                                            float (*s_part)[NR][TB], float (&res)[NR][TB]) {
    constexpr int Q = 4;  // units per thread in flight
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int units = H >> 3;
    const u32x4 zero = u32x4{0, 0, 0, 0};
    float acc[NR][TB];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int t = 0; t < TB; ++t) acc[r][t] = 0.0f;
    for (int u0 = 0; u0 < units; u0 += 256 * Q) {
        u32x4 wv[Q][NR], xv[Q][TB];
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int u = u0 + 256 * q + tid;
#pragma unroll
            for (int r = 0; r < NR; ++r) wv[q][r] = u < units ? ld16_stream(w[r] + u * 8) : zero;
        }
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int u = u0 + 256 * q + tid;
#pragma unroll
            for (int t = 0; t < TB; ++t) xv[q][t] = (u < units && t < B) ? ld16(x + (size_t)t * H + u * 8) : zero;
        }
#pragma unroll
        for (int q = 0; q < Q; ++q)
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int t = 0; t < TB; ++t)
                    if (t < B) acc[r][t] = dot8(wv[q][r], xv[q][t], acc[r][t]);
    }
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            if (t < B) {
                const float sum = wave_sum(acc[r][t]);
                if (lane == 0) s_part[wave][r][t] = sum;
            }
        }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int t = 0; t < TB; ++t)
            res[r][t] = (s_part[0][r][t] + s_part[1][r][t]) + (s_part[2][r][t] + s_part[3][r][t]);
}

// Front launch of the select-in-gate/up form (batch <= 4): workgroups
// [0, router_blocks = E) compute one router row each (z = x . Wr[e] + bias);
// workgroups [E, E + shared_blocks) one gate/up row pair of the shared expert
// each (hs = SiLU(gate) * up).  Small workgroups, all resident at once: the
// launch is one round trip of weight loads wide.
template <int TB>
__global__ __launch_bounds__(256) void front_split_kernel(FrontArgs f) {
    const RouterArgs& a = f.r;
    const int tid = threadIdx.x;
    if (blockIdx.x == 0 && f.sync_clear)  // re-arms the next launch's counters and flags
        for (int i = tid; i < f.sync_words; i += 256) f.sync_clear[i] = 0;
    if ((int)blockIdx.x < f.router_blocks) {
        __shared__ float s_part[4][1][TB];
        const int e = blockIdx.x;
        const uint16_t* w[1] = {a.wr + (size_t)e * a.H};
        float z[1][TB];
        wg_rows_dot<TB, 1>(w, a.x, a.H, a.B, s_part, z);
        const float b = a.bias ? a.bias[e] : 0.0f;
#pragma unroll
        for (int t = 0; t < TB; ++t)
            if (tid == t && t < a.B) a.z[(size_t)t * a.E + e] = z[0][t] + b;
    } else {
        __shared__ float s_part[4][2][TB];
        const GateUpArgs& s = f.s;
        const int i = blockIdx.x - f.router_blocks;
        const uint16_t* w[2] = {s.w + (size_t)i * s.H, s.w + (size_t)(s.n + i) * s.H};
        float gu[2][TB];
        wg_rows_dot<TB, 2>(w, s.x, s.H, a.B, s_part, gu);
#pragma unroll
        for (int t = 0; t < TB; ++t)
            if (tid == t && t < a.B) s.h[(size_t)t * s.n + i] = silu_f(gu[0][t]) * gu[1][t];
    }
}

// Wave t < B selects token t's experts from z (the routing rows are written
// by workgroup 0 only), wave 0 buckets the B*k pairs into LDS lists (and, in
// workgroup 0, into the global lists the down launch reads), then the
// workgroup runs routed tiles b, b + G, ... with each entry's token ids from
// LDS.  Every workgroup derives the same lists from the same logits; the host
// keeps the grid within what the device holds at once, so each workgroup pays
// the selection once.  At
// B = 1 the k experts are distinct, so pair j is entry j in slot j.
// Workgroups b < shared_pairs also compute the shared expert's gate/up row
// pair b: its loads go out right behind the logit loads, so they stream while
// the selection runs (the weights of the routed tile are not known yet).
template <int TB, int NS>
__global__ __launch_bounds__(256) void gateup_select_kernel(SelGateUpArgs sa) {
    extern __shared__ __align__(16) uint16_t s_x[];  // [B][H]
    __shared__ int32_t s_pair_e[4 * kMaxTopK];
    __shared__ int32_t s_tok[4 * kMaxTopK];  // slot -> token
    __shared__ int32_t s_act_e[4 * kMaxTopK];
    __shared__ int32_t s_act_off[4 * kMaxTopK + 1];
    __shared__ int32_t s_nact;
    __shared__ __align__(16) int32_t s_ps[128];
    __shared__ float s_part[4][2][TB];
    const RouterArgs& a = sa.r;
    const GateUpArgs& g = sa.g;
    const GateUpArgs& sg = sa.s;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x;
    const bool out = b == 0;
    // shared row pair b: the first 1024 units of K requested during the selection
    constexpr int Q = 4;
    const bool shp = b < sa.shared_pairs;
    const int units = sg.H >> 3;
    const u32x4 zero = u32x4{0, 0, 0, 0};
    const uint16_t* srow[2] = {sg.w + (size_t)b * sg.H, sg.w + (size_t)(sg.n + b) * sg.H};
    u32x4 swv[Q][2], sxv[Q][TB];
    auto issue_shared = [&]() {
        if (!shp) return;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int u = 256 * q + tid;
#pragma unroll
            for (int r = 0; r < 2; ++r) swv[q][r] = u < units ? ld16_stream(srow[r] + u * 8) : zero;
#pragma unroll
            for (int t = 0; t < TB; ++t)
                sxv[q][t] = (u < units && t < a.B) ? ld16(sg.x + (size_t)t * sg.H + u * 8) : zero;
        }
    };
    select_tokens<NS, false>(a, 0, a.z, nullptr, false, s_pair_e, out, issue_shared);
    if (tid < 64) {
        const int np = a.B * a.k;
        const int e = lane < np ? s_pair_e[lane] : kNone;
        int nact = 0;
        if (__ballot(lane < np && (e < 0 || e >= a.E))) {  // never hand an invalid id to the experts
            if (out && lane == 0) bucket_meta(a, 0, 0, np, -1);
        } else {
            const PairSlot ps = a.B == 1 ? PairSlot{lane, lane, 1, lane < np, false} : pair_slot(e, np, lane, s_ps);
            if (lane < np) s_tok[ps.pos] = lane / a.k;
            if (ps.lead) {
                s_act_e[ps.apos] = e;
                s_act_off[ps.apos] = ps.pos;
            }
            nact = __popcll(__ballot(ps.lead));
            if (out) {
                if (lane < np) a.perm[ps.pos] = lane;
                if (ps.lead) {
                    a.act_e[ps.apos] = e;
                    a.act_off[ps.apos] = ps.pos;
                }
                if (lane == 0) bucket_meta(a, nact, 0, np, np);
            }
        }
        if (lane == 0) {
            s_nact = nact;
            s_act_off[nact] = np;
        }
    }
    __syncthreads();
    if (shp) {  // finish the shared row pair: the rest of K, then the wave sums in a fixed order
        float acc[2][TB];
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int t = 0; t < TB; ++t) acc[r][t] = 0.0f;
#pragma unroll
        for (int q = 0; q < Q; ++q)
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int t = 0; t < TB; ++t)
                    if (t < a.B) acc[r][t] = dot8(swv[q][r], sxv[q][t], acc[r][t]);
        for (int u = 256 * Q + tid; u < units; u += 256)
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const u32x4 w = ld16_stream(srow[r] + u * 8);
#pragma unroll
                for (int t = 0; t < TB; ++t)
                    if (t < a.B) acc[r][t] = dot8(w, ld16(sg.x + (size_t)t * sg.H + u * 8), acc[r][t]);
            }
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                if (t < a.B) {
                    const float sum = wave_sum(acc[r][t]);
                    if (lane == 0) s_part[wave][r][t] = sum;
                }
            }
        __syncthreads();
        if (tid < a.B) {
            float gu[2];
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                float v = 0.0f;
#pragma unroll
                for (int t = 0; t < TB; ++t)
                    if (t == tid) v = (s_part[0][r][t] + s_part[1][r][t]) + (s_part[2][r][t] + s_part[3][r][t]);
                gu[r] = v;
            }
            sg.h[(size_t)tid * sg.n + b] = silu_f(gu[0]) * gu[1];
        }
    }
    // the routed tiles, grid-strided: the grid is at most what the device
    // holds at once, so each workgroup selects once for all its tiles
    const int ntiles = uni(s_nact) * g.tiles_per_expert;
    const int gunits = g.H >> 3;
    if (((gunits + 63) >> 6) <= kMaxGemvUnits) {
        // software-pipelined: every token's x row is staged once, behind the
        // first tile's weight requests, and a tile's successor is requested
        // as soon as the tile's rows are used (no restaging, no barrier and
        // no h store between a workgroup's tiles)
        if (b >= ntiles) return;
        const int tpe = g.tiles_per_expert, H = g.H, G = gridDim.x;
        u32x4 wg[kMaxGemvUnits], wu[kMaxGemvUnits];
        auto issue = [&](int tile) {
            const int entry = tile / tpe;
            const int i = (tile - entry * tpe) * kPairsPerGemvTile + wave;
            const uint16_t* gr = g.w + (size_t)uni(s_act_e[entry]) * g.expert_stride + (size_t)i * H;
            const uint16_t* ur = gr + (size_t)g.n * H;
#pragma unroll
            for (int q = 0; q < kMaxGemvUnits; ++q) {
                const int uu = q * 64 + lane;
                const bool ok = uu < gunits;
                wg[q] = ok ? ld16_stream(gr + uu * 8) : zero;
                wu[q] = ok ? ld16_stream(ur + uu * 8) : zero;
            }
        };
        issue(b);
        const int nx = a.B * gunits;  // x is [B][H]: unit idx of token idx / units
        for (int i0 = tid; i0 < nx; i0 += 256 * 8) {
            u32x4 xr[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) xr[q] = ld16(g.x + (size_t)min(i0 + 256 * q, nx - 1) * 8);
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (i0 + 256 * q < nx) st16(s_x + (size_t)(i0 + 256 * q) * 8, xr[q]);
        }
        __syncthreads();
        for (int tile = b; tile < ntiles; tile += G) {
            const int entry = tile / tpe;
            const int i = (tile - entry * tpe) * kPairsPerGemvTile + wave;
            const int off = uni(s_act_off[entry]);
            int T = uni(s_act_off[entry + 1]) - off;
            if (T > TB) {  // an expert holds at most one pair per token, so T <= B <= TB
                if (tid == 0 && i < kPairsPerGemvTile) atomicOr(&g.meta[M_ERR], ERR_TILE);
                T = 0;
            }
            int tk[TB];
#pragma unroll
            for (int j = 0; j < TB; ++j) tk[j] = j < T ? uni(s_tok[off + j]) : 0;
            float ag[TB], au[TB];
#pragma unroll
            for (int j = 0; j < TB; ++j) { ag[j] = 0.0f; au[j] = 0.0f; }
#pragma unroll
            for (int q = 0; q < kMaxGemvUnits; ++q) {
                const int uu = q * 64 + lane;
                if (uu < gunits) {
#pragma unroll
                    for (int j = 0; j < TB; ++j) {
                        if (j < T) {
                            const u32x4 xv = ld16(s_x + (size_t)tk[j] * H + uu * 8);
                            ag[j] = dot8(wg[q], xv, ag[j]);
                            au[j] = dot8(wu[q], xv, au[j]);
                        }
                    }
                }
            }
            if (tile + G < ntiles) issue(tile + G);  // the rows are used: the next tile's go out
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                if (j < T) {
                    const float gs = wave_sum(ag[j]), us = wave_sum(au[j]);
                    if (lane == 0) st_dev(g.h + (size_t)(off + j) * g.n + i, silu_f(gs) * us);
                }
            }
        }
        return;
    }
    for (int tile = b; tile < ntiles; tile += gridDim.x) {
        const int entry = tile / g.tiles_per_expert, local = tile % g.tiles_per_expert;
        const int e = uni(s_act_e[entry]), off = uni(s_act_off[entry]);
        const int T = uni(s_act_off[entry + 1]) - off;
        if (T > TB) {  // an expert holds at most one pair per token, so T <= B <= TB
            if (tid == 0 && local == 0) atomicOr(&g.meta[M_ERR], ERR_TILE);
            continue;
        }
        gemv_gateup_tile<TB>(g, g.w + (size_t)e * (size_t)g.expert_stride, off, T, local, s_x, s_tok + off);
        __syncthreads();  // the next tile restages s_x
    }
}

// ---------------------------------------------------------------------------
// down, output-stationary (staged launches, small batches): each workgroup
// owns a block of output rows and runs every active expert and shared column
// block over them (down_rows), so the combine needs no second pass
// ---------------------------------------------------------------------------

template <int LPR, int NQ, int RP, bool HLDS>
__global__ __launch_bounds__(256) void down_combine_kernel(DownArgs a) {
    extern __shared__ __align__(16) float s_h[];
    __shared__ float s_acc[kMaxBatch * DownShape<LPR, NQ, RP>::R];
    down_rows<LPR, NQ, RP, HLDS, DOWN_ALL, false>(a, blockIdx.x, s_h, s_acc, [] {});
}

// Packs 4 floats into bf16 hi and lo parts (v ~= hi + lo to ~2^-16 relative)
// and stores them as pairs 2i, 2i+1 of s_hh and s_hl.
__device__ __forceinline__ void store_hilo4(uint32_t* s_hh, uint32_t* s_hl, int i, float4 v) {
    const uint32_t h0 = f32_to_bf16_rne(v.x), h1 = f32_to_bf16_rne(v.y);
    const uint32_t h2 = f32_to_bf16_rne(v.z), h3 = f32_to_bf16_rne(v.w);
    const uint32_t l0 = f32_to_bf16_rne(v.x - __uint_as_float(h0 << 16));
    const uint32_t l1 = f32_to_bf16_rne(v.y - __uint_as_float(h1 << 16));
    const uint32_t l2 = f32_to_bf16_rne(v.z - __uint_as_float(h2 << 16));
    const uint32_t l3 = f32_to_bf16_rne(v.w - __uint_as_float(h3 << 16));
    reinterpret_cast<uint2*>(s_hh)[i] = uint2{h0 | (h1 << 16), h2 | (h3 << 16)};
    reinterpret_cast<uint2*>(s_hl)[i] = uint2{l0 | (l1 << 16), l2 | (l3 << 16)};
}

// Output-stationary down for batch <= TB <= 4 (staged launches).  Workgroup:
// output rows [row0, row0 + R), R = 4 * 64 / LPR; wave w owns 64 / LPR of
// them, LPR lanes per row (LPR <= 16), NQ 16-byte units per lane, so
// 8 * LPR * NQ = I.  Entries: the nact active routed experts, then the shared
// expert's nsh column blocks; CE per chunk, two chunks in flight.
// Order of requests, so that the weights wait for one round trip at most:
//   the entry count and the first 2*CE expert ids together (scalar; ids past
//   the count are read but unused -- act_e is a 256-byte block);
//   every slot's and token's h row, the slots' pair ids, the pairs' routing
//   weights and the entries' slot offsets (vector, to LDS);
//   the weights of the first two chunks once the scalars are in.
// h goes to LDS as bf16 hi/lo pairs while the weights stream.  Per entry and
// token: v_dot2 of W2 with h's hi and lo parts over the lane's units, an
// LPR-lane DPP sum (every lane of the group ends with it), times the routing
// weight into a register accumulator per token; entries then tokens in a
// fixed order, so the sum is deterministic.
template <int TB, int LPR, int NQ>
__global__ __launch_bounds__(256) void down_os_kernel(DownArgs a) {
    extern __shared__ __align__(16) uint32_t s_hp[];  // hi pairs [nrow][I/2], then lo pairs
    constexpr int NP = TB * kMaxTopK;
    __shared__ int32_t s_tok[NP];   // slot -> token
    __shared__ float s_wsl[NP];     // slot -> routing weight
    __shared__ int32_t s_perm[NP];  // staging: slot -> pair
    __shared__ float s_tw[NP];      // staging: pair -> routing weight
    __shared__ int32_t s_off[NP + 1];
    __shared__ int32_t s_acte[NP];
    static_assert(LPR <= 16, "every lane of a group needs the group sum");
    constexpr int RW = 64 / LPR, R = 4 * RW;
    constexpr int CE = (16 / NQ) > 0 ? 16 / NQ : 1;  // entries per chunk
    static_assert(2 * CE <= 64, "the early ids stay inside act_e's 256-byte block");
    constexpr int HREG = 3 * TB;                     // h float4 per thread requested before the weights
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H, I = a.I, B = a.B, k = a.k;
    const int nsh = a.s2 ? a.Is / I : 0;
    const int np = B * k, maxa = min(a.n_experts, np);
    const int row = blockIdx.x * R + wave * RW + lane / LPR;
    const int c = lane % LPR;
    const size_t estride = (size_t)H * I;

    const int nact = min(uni(*a.n_act), maxa);
    int eid0[2 * CE];
#pragma unroll
    for (int i = 0; i < 2 * CE; ++i) eid0[i] = uni(a.act_e[i]);

    // vector loads that need no work list: h rows (routed slots [0, np), then
    // shared rows [np, np + B*nsh): hs is [B][nsh][I]), pair ids, weights, offsets
    const int I4 = I / 4, nh4 = np * I4, nrow = np + B * nsh, n4 = nrow * I4;
    float4 hv[HREG];
#pragma unroll
    for (int j = 0; j < HREG; ++j) {
        const int i = tid + 256 * j;
        const float* src = i < nh4 ? a.h + 4 * (size_t)i : a.hs + 4 * (size_t)(i < n4 ? i - nh4 : 0);
        hv[j] = *reinterpret_cast<const float4*>(src);
    }
    int32_t pv = 0, ov = 0, ev = 0;
    float twv = 0.0f;
    if (tid < np) {
        pv = a.perm[tid];
        twv = a.topk_w[tid];
    }
    if (tid <= maxa) ov = a.act_off[tid];
    if (tid < maxa) ev = a.act_e[tid];

    const int total = nact + nsh;
    // this lane's first unit of entry ent's row; e: the expert id when routed
    auto w_of = [&](int ent, int e) -> const uint16_t* {
        if (ent >= nact) return a.s2 + (size_t)row * a.Is + (size_t)(ent - nact) * I + 8 * c;
        if ((unsigned)e >= (unsigned)a.n_experts) e = 0;  // bucketing never publishes this
        return a.w2 + (size_t)e * estride + (size_t)row * I + 8 * c;
    };
    auto load_early = [&](int c0, u32x4 (&buf)[CE][NQ]) {  // c0 = 0 or CE
#pragma unroll
        for (int ce = 0; ce < CE; ++ce) {
            const int ent = c0 + ce;
            if (ent < total) {
                const uint16_t* w = w_of(ent, eid0[c0 + ce]);
#pragma unroll
                for (int q = 0; q < NQ; ++q) buf[ce][q] = ld16_stream(w + 8 * LPR * q);
            }
        }
    };
    auto load_later = [&](int c0, u32x4 (&buf)[CE][NQ]) {
#pragma unroll
        for (int ce = 0; ce < CE; ++ce) {
            const int ent = c0 + ce;
            if (ent < total) {
                const uint16_t* w = w_of(ent, ent < nact ? uni(s_acte[ent]) : 0);
#pragma unroll
                for (int q = 0; q < NQ; ++q) buf[ce][q] = ld16_stream(w + 8 * LPR * q);
            }
        }
    };
    u32x4 wb0[CE][NQ], wb1[CE][NQ];
    load_early(0, wb0);
    if (CE < total) load_early(CE, wb1);

    uint32_t* s_hh = s_hp;
    uint32_t* s_hl = s_hp + (size_t)nrow * I / 2;
#pragma unroll
    for (int j = 0; j < HREG; ++j) {
        const int i = tid + 256 * j;
        if (i < n4) store_hilo4(s_hh, s_hl, i, hv[j]);
    }
    for (int i = tid + 256 * HREG; i < n4; i += 256) {
        const float* src = i < nh4 ? a.h + 4 * (size_t)i : a.hs + 4 * (size_t)(i - nh4);
        store_hilo4(s_hh, s_hl, i, *reinterpret_cast<const float4*>(src));
    }
    if (tid < np) {
        s_perm[tid] = pv;
        s_tw[tid] = twv;
    }
    if (tid <= maxa) s_off[tid] = ov;
    if (tid < maxa) s_acte[tid] = ev;
    __syncthreads();
    if (tid < np) {
        const int p = s_perm[tid];
        const bool ok = p >= 0 && p < np;  // bucketing never publishes a bad pair id
        s_tok[tid] = ok ? p / k : 0;
        s_wsl[tid] = ok ? s_tw[p] : 0.0f;
    }
    __syncthreads();

    float acc[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[t] = 0.0f;
    auto dot_row = [&](const u32x4 (&w)[NQ], int hrow) {
        float d = 0.0f;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const size_t pe = (size_t)hrow * (I / 2) + 4 * (c + LPR * q);
            d = dot8_hilo(w[q], *reinterpret_cast<const u32x4*>(s_hh + pe),
                          *reinterpret_cast<const u32x4*>(s_hl + pe), d);
        }
        return d;  // this lane's part; the row's LPR lanes are summed once per token at the end
    };
    auto add = [&](int t, float v) {
#pragma unroll
        for (int tt = 0; tt < TB; ++tt)
            if (tt == t) acc[tt] += v;
    };
    auto process = [&](int c0, const u32x4 (&wa)[CE][NQ]) {
#pragma unroll
        for (int ce = 0; ce < CE; ++ce) {
            const int ent = c0 + ce;
            if (ent < nact) {
                if constexpr (TB == 1) {  // one token: entry ent is slot ent
                    acc[0] += s_wsl[ent] * dot_row(wa[ce], ent);
                } else {
                    const int off = max(uni(s_off[ent]), 0), end = min(uni(s_off[ent + 1]), np);
                    for (int sl = off; sl < end; ++sl) add(uni(s_tok[sl]), s_wsl[sl] * dot_row(wa[ce], sl));
                }
            } else if (ent < total) {
                const int v = ent - nact;
                for (int t = 0; t < B; ++t) add(t, dot_row(wa[ce], np + t * nsh + v));
            }
        }
    };
    for (int c0 = 0; c0 < total; c0 += 2 * CE) {
        process(c0, wb0);
        if (c0 + 2 * CE < total) load_later(c0 + 2 * CE, wb0);
        if (c0 + CE >= total) break;
        process(c0 + CE, wb1);
        if (c0 + 3 * CE < total) load_later(c0 + 3 * CE, wb1);
    }
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[t] = group_sum<LPR>(acc[t]);
    if (c == 0) {
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            if (t < B) {
                float v = acc[t];
                if (a.add_residual) v += __uint_as_float((uint32_t)a.x[(size_t)t * H + row] << 16);
                a.out[(size_t)t * H + row] = f32_to_bf16_rne(v);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// down, expert-major (staged launches, larger batches)
// ---------------------------------------------------------------------------

// Packs 8 floats into bf16 hi and lo parts (v ~= hi + lo to ~2^-16 relative):
// the MFMA down tile multiplies W2 by both, which keeps h at near-fp32
// precision through a bf16 matrix core.
__device__ __forceinline__ void split_bf16x8(const float4 f0, const float4 f1, u32x4& hi, u32x4& lo) {
    const float v[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
    uint32_t h[8], l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        h[i] = f32_to_bf16_rne(v[i]);
        l[i] = f32_to_bf16_rne(v[i] - __uint_as_float(h[i] << 16));
    }
    hi = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    lo = u32x4{l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16)};
}

// One workgroup: output rows [r0, r0 + kDownXRows) of one entry (a routed
// expert with T tokens, or a shared column block with all B tokens); wave w
// owns the 64-row band r0 + 64w.  Token j's h row is hsrc + j * hstride (I
// floats); its partial output row is dst + s_dsto[j] (H floats).
// Order of work, so that the weights are requested after one scalar round
// trip and everything else rides behind them (vector memory loads complete in
// issue order): work-list fields (read together with the entry count), then
// the band's weights, then h (to LDS) and the rows' output offsets, barrier,
// compute.
//  GEMV (few tokens, h in LDS): LPR lanes per row, NQ 16-byte units per lane
//    per row; the band's rows in batches of 16 units per lane, two batches in
//    flight, a batch re-requested as soon as the one before it is used.
//  MFMA (else, or when h does not fit LDS): per 32-column step, each wave
//    multiplies its four 16-row groups (A = W2 rows, all steps of a 256-column
//    chunk requested at once) by h^T (B, split into bf16 hi + lo) with
//    mfma_f32_16x16x32_bf16.
// The partials are combined by combine_kernel, the next launch.
template <int LPR, int NQ>
__global__ __launch_bounds__(256, 2) void down_x_kernel(DownXArgs a) {
    // h split into bf16 hi and lo parts when it fits: pairs [T][I/2] each
    extern __shared__ __align__(16) uint32_t s_hh[];
    __shared__ int s_dsto[kMaxBatch];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H, I = a.I, B = a.B, k = a.k;
    const int nrb = (H + kDownXRows - 1) / kDownXRows;
    // grid order: the shared expert's column blocks (all B tokens, the
    // heaviest tiles) first, then the routed entries, so that the launch's
    // tail holds light routed tiles and the entries past n_act, which exit
    const int rb = blockIdx.x % nrb, gent = blockIdx.x / nrb;
    const bool routed = gent >= a.nsh;
    const int ent = routed ? gent - a.nsh : 0;   // routed entry
    const int sblk = routed ? 0 : gent;           // shared column block
    const int r0 = rb * kDownXRows;
    const int band = r0 + 64 * wave;
    const bool band_ok = band < H;  // H is a multiple of 64
    const int ent_c = ent;  // the lists are valid memory for every grid entry
    const int nact = uni(*a.n_act);
    const int e_r = uni(a.act_e[ent_c]), off_r = uni(a.act_off[ent_c]), end_r = uni(a.act_off[ent_c + 1]);

    const uint16_t* W;
    const float* hsrc;
    float* dst;
    int ld, hstride, T;
    if (routed) {
        if (ent >= nact) return;
        T = end_r - off_r;
        if ((unsigned)e_r >= (unsigned)a.n_experts || off_r < 0 || T < 1 || off_r + T > B * k || T > kMaxBatch) {
            if (tid == 0 && rb == 0) atomicOr(&a.meta[M_ERR], ERR_TILE);
            return;
        }
        W = a.w2 + (size_t)e_r * H * I;
        ld = I;
        hsrc = a.h + (size_t)off_r * I;
        hstride = I;
        dst = a.part;
    } else {
        const int v = sblk;
        W = a.s2 + (size_t)v * I;
        ld = a.Is;
        hsrc = a.hs + (size_t)v * I;
        hstride = a.Is;
        T = B;
        dst = a.part_s;
    }
    const bool h_lds = (size_t)T * I * 4 <= (size_t)kDownXLds;
    const bool mfma = (a.mfma_min_tokens > 0 && T >= a.mfma_min_tokens) || !h_lds;
    const u32x4 zero = u32x4{0, 0, 0, 0};

    uint32_t* s_hl = s_hh + (size_t)T * I / 2;
    // h rows go to LDS as bf16 hi + lo pairs (when they fit).  A thread's
    // first float4 of h (one on GEMV tiles, two on MFMA tiles: all of h for up
    // to 4 / 8 tokens at I = 256) are requested before the weights: loads
    // complete in issue order, so they arrive first and are staged while the
    // weights stream.  The rest of a larger tile's h is requested after the
    // weights, two float4 at a time.  (More than two ahead of the MFMA tile's
    // weights exceeds its registers.)
    constexpr int kHFirst = 2;
    constexpr std::integral_constant<int, 1> kGemvFirst{};
    constexpr std::integral_constant<int, kHFirst> kMfmaFirst{};
    const int I4 = I / 4, n4 = h_lds ? T * I4 : 0;
    float4 hv[kHFirst];
    int pv = 0;
    auto h_issue = [&](auto nfirst) {
        constexpr int NF = decltype(nfirst)::value;
        // unconditional loads (clamped indices; the extra values are unused)
#pragma unroll
        for (int q = 0; q < NF; ++q) {
            const int i = max(min(tid + 256 * q, n4 - 1), 0);
            const int j = i / I4, c4 = i - j * I4;
            hv[q] = *reinterpret_cast<const float4*>(hsrc + (size_t)j * hstride + 4 * c4);
        }
    };
    // the tokens' pair ids, requested after the weights (at the join of the
    // GEMV and MFMA paths the compiler waits for every load in flight)
    auto perm_issue = [&]() {
        const int pl = a.perm[routed ? off_r + min(tid, T - 1) : 0];
        pv = routed ? pl : sblk * B + tid;
    };
    auto put = [&](int i, const float4 v) {
        const uint32_t h0 = f32_to_bf16_rne(v.x), h1 = f32_to_bf16_rne(v.y);
        const uint32_t h2 = f32_to_bf16_rne(v.z), h3 = f32_to_bf16_rne(v.w);
        const uint32_t l0 = f32_to_bf16_rne(v.x - __uint_as_float(h0 << 16));
        const uint32_t l1 = f32_to_bf16_rne(v.y - __uint_as_float(h1 << 16));
        const uint32_t l2 = f32_to_bf16_rne(v.z - __uint_as_float(h2 << 16));
        const uint32_t l3 = f32_to_bf16_rne(v.w - __uint_as_float(h3 << 16));
        reinterpret_cast<uint2*>(s_hh)[i] = uint2{h0 | (h1 << 16), h2 | (h3 << 16)};
        reinterpret_cast<uint2*>(s_hl)[i] = uint2{l0 | (l1 << 16), l2 | (l3 << 16)};
    };
    // called once the band's weights are requested
    auto stage = [&](auto nfirst) {
        constexpr int NF = decltype(nfirst)::value;
#pragma unroll
        for (int q = 0; q < NF; ++q) {
            const int i = tid + 256 * q;
            if (i < n4) put(i, hv[q]);
        }
        // keep the pair ids' store (which waits for every load) after h's
        __builtin_amdgcn_sched_barrier(0);
        if (tid < T) s_dsto[tid] = pv * H;
        for (int i0 = tid + 256 * NF; i0 < n4; i0 += 512) {
            float4 v[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int i = i0 + 256 * q;
                const int j = i / I4, c4 = i - j * I4;
                v[q] = i < n4 ? *reinterpret_cast<const float4*>(hsrc + (size_t)j * hstride + 4 * c4)
                              : float4{0.0f, 0.0f, 0.0f, 0.0f};
            }
#pragma unroll
            for (int q = 0; q < 2; ++q)
                if (i0 + 256 * q < n4) put(i0 + 256 * q, v[q]);
        }
        __syncthreads();
    };

    if (!mfma) {
        constexpr int RW = 64 / LPR, P = 64 / RW;            // rows per pass, passes per band
        constexpr int QB = (16 / NQ) < P ? 16 / NQ : P;      // passes per batch of loads
        const int rw = lane / LPR, c = lane % LPR;
        auto load = [&](int q0, u32x4 (&w)[QB][NQ]) {
#pragma unroll
            for (int q = 0; q < QB; ++q) {
                // a band past H (H not a multiple of 256) reads band 0's rows
                // and stores nothing: no load is conditional, so the waits for
                // h and for the first batch count the loads issued after them
                const int row = (band_ok ? band : 0) + (q0 + q) * RW + rw;
#pragma unroll
                for (int u = 0; u < NQ; ++u)
                    w[q][u] = q0 + q < P ? ld16_stream(W + (size_t)row * ld + 8 * (c + LPR * u)) : zero;
            }
        };
        // two register buffers; the batch loop is unrolled, so they alternate
        // without copies and each batch's loads are waited for only when used
        u32x4 wbuf[2][QB][NQ];
        h_issue(kGemvFirst);
        load(0, wbuf[0]);
        if (QB < P) load(QB, wbuf[1]);
        perm_issue();
        stage(kGemvFirst);
#pragma unroll
        for (int q0 = 0; q0 < P; q0 += QB) {
            u32x4 (&wa)[QB][NQ] = wbuf[(q0 / QB) & 1];
            if (band_ok) {
                // token-outer: a lane reads its h units of token j from LDS
                // once per batch of QB rows (row-outer re-read them per row)
                for (int j = 0; j < T; ++j) {
                    u32x4 hh[NQ], hl[NQ];
#pragma unroll
                    for (int u = 0; u < NQ; ++u) {
                        const size_t pe = ((size_t)j * I + 8 * (c + LPR * u)) / 2;  // pair index
                        hh[u] = *reinterpret_cast<const u32x4*>(s_hh + pe);
                        hl[u] = *reinterpret_cast<const u32x4*>(s_hl + pe);
                    }
                    float* drow = dst + s_dsto[j] + band + rw;
#pragma unroll
                    for (int q = 0; q < QB; ++q) {
                        if (q0 + q < P) {
                            float acc = 0.0f;
#pragma unroll
                            for (int u = 0; u < NQ; ++u) acc = dot8_hilo(wa[q][u], hh[u], hl[u], acc);
                            acc = group_sum<LPR>(acc);
                            if (c == LPR - 1) drow[(q0 + q) * RW] = acc;
                        }
                    }
                }
            }
            if (q0 + 2 * QB < P) load(q0 + 2 * QB, wa);
        }
    } else {
        const int tl = lane & 15, kq = lane >> 4;
        const int NT = (T + 15) >> 4;
        const uint16_t* arow = W + (size_t)((band_ok ? band : 0) + tl) * ld + 8 * kq;  // group g: + 16 g rows
        const float* hrow[4];
        bool hok[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int j = tt * 16 + tl;
            hok[tt] = j < T;
            hrow[tt] = hsrc + (size_t)(hok[tt] ? j : 0) * hstride + 8 * kq;
        }
        f32x4 acc[4][4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) acc[g][tt] = f32x4{0, 0, 0, 0};
        constexpr int NSC = (LPR * NQ / 4) < 8 ? LPR * NQ / 4 : 8;  // 32-column steps per chunk (I / 32, at most 8)
        u32x4 A[NSC][4];
        auto load_a = [&](int c0) {
#pragma unroll
            for (int st = 0; st < NSC; ++st)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    A[st][g] = ld16_stream(arow + (size_t)16 * g * ld + c0 + 32 * st);
        };
        auto chunk = [&](int c0) {
#pragma unroll
            for (int st = 0; st < NSC; ++st) {
                const int col = c0 + 32 * st;
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    if (tt < NT) {
                        const int j = tt * 16 + tl;
                        u32x4 bh = zero, bl = zero;
                        if (j < T) {
                            if (h_lds) {
                                const size_t pe = ((size_t)j * I + col + 8 * kq) / 2;
                                bh = *reinterpret_cast<const u32x4*>(s_hh + pe);
                                bl = *reinterpret_cast<const u32x4*>(s_hl + pe);
                            } else {
                                const float4* hp = reinterpret_cast<const float4*>(hrow[tt] + col);
                                split_bf16x8(hp[0], hp[1], bh, bl);
                            }
                        }
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const bf16x8 Aw = __builtin_bit_cast(bf16x8, A[st][g]);
                            acc[g][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                Aw, __builtin_bit_cast(bf16x8, bh), acc[g][tt], 0, 0, 0);
                            acc[g][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                Aw, __builtin_bit_cast(bf16x8, bl), acc[g][tt], 0, 0, 0);
                        }
                    }
                }
            }
        };
        // the first chunk in straight-line code: h is requested, then the
        // weights, then h is staged (inside a loop the compiler hoisted the
        // staging's conversion, and its wait for h, above the weight requests)
        h_issue(kMfmaFirst);
        load_a(0);
        perm_issue();
        stage(kMfmaFirst);
        chunk(0);
        for (int c0 = 32 * NSC; c0 < I; c0 += 32 * NSC) {
            load_a(c0);
            chunk(c0);
        }
        // D layout: lane holds rows 4*(lane/16)+r of the group, column (token) lane%16
        if (band_ok) {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const int j = tt * 16 + tl;
                if (tt < NT && j < T) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        float* dp = dst + s_dsto[j] + band + 16 * g + 4 * kq;
                        *reinterpret_cast<float4*>(dp) =
                            float4{acc[g][tt][0], acc[g][tt][1], acc[g][tt][2], acc[g][tt][3]};
                    }
                }
            }
        }
    }
}

// out[t][r] = bf16( sum_j w[t][j] * part[t*k+j][r] + sum_sb part_s[sb][t][r] (+ x) ),
// summed in that fixed order; four rows per thread.  KB >= k: the k partial
// rows of a token are requested in one round (addresses past k clamped, their
// terms skipped).
template <int KB>
__global__ __launch_bounds__(128) void combine_kernel(DownXArgs a) {
    const int H = a.H, k = a.k, B = a.B;
    const int i4 = blockIdx.x * 128 + threadIdx.x;
    if (i4 >= B * H / 4) return;
    const int t = (4 * i4) / H, r = 4 * i4 - t * H;
    float4 y[KB];
    float w[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
        const int p = t * k + (j < k ? j : k - 1);
        y[j] = *reinterpret_cast<const float4*>(a.part + (size_t)p * H + r);
        w[j] = a.topk_w[p];
    }
    uint2 xb = uint2{0, 0};
    if (a.add_residual) xb = *reinterpret_cast<const uint2*>(a.x + (size_t)t * H + r);
    float4 v = float4{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < KB; ++j) {
        if (j < k) {
            v.x += w[j] * y[j].x; v.y += w[j] * y[j].y; v.z += w[j] * y[j].z; v.w += w[j] * y[j].w;
        }
    }
    for (int sb = 0; sb < a.nsh; ++sb) {
        const float4 ys = *reinterpret_cast<const float4*>(a.part_s + ((size_t)sb * B + t) * H + r);
        v.x += ys.x; v.y += ys.y; v.z += ys.z; v.w += ys.w;
    }
    if (a.add_residual) {
        v.x += bf16_lo(xb.x); v.y += bf16_hi(xb.x); v.z += bf16_lo(xb.y); v.w += bf16_hi(xb.y);
    }
    const uint32_t o0 = f32_to_bf16_rne(v.x) | ((uint32_t)f32_to_bf16_rne(v.y) << 16);
    const uint32_t o1 = f32_to_bf16_rne(v.z) | ((uint32_t)f32_to_bf16_rne(v.w) << 16);
    *reinterpret_cast<uint2*>(a.out + (size_t)t * H + r) = uint2{o0, o1};
}

__global__ __launch_bounds__(256) void init_lists_kernel(InitArgs a) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t < a.B) a.sh_perm[t] = t;
    if (t < M_COUNT && a.zero_meta) a.meta[t] = t == M_SHARED_NACT ? 1 : 0;
    if (t == 0) {
        if (!a.zero_meta) a.meta[M_SHARED_NACT] = 1;
        a.sh_act_e[0] = 0;
        a.sh_act_off[0] = 0;
        a.sh_act_off[1] = a.B;
    }
    const long long n4 = a.zero_words / 4;
    for (long long i = t; i < n4; i += (long long)gridDim.x * blockDim.x)
        reinterpret_cast<u32x4*>(a.zero)[i] = u32x4{0, 0, 0, 0};
}

// ---------------------------------------------------------------------------
// kernel selection (the host library launches the returned function)
// ---------------------------------------------------------------------------

static int tb_bucket(int b) {
    int tb = 1;
    while (tb < b) tb <<= 1;
    return tb;
}

#define MOE_FN(f) reinterpret_cast<const void*>(&f)

KernelPick pick_init(const InitArgs& a) {
    const long long need = std::max<long long>({(long long)a.B, (long long)M_COUNT, a.zero_words / 4});
    const long long grid = std::min<long long>(1024, (need + 255) / 256);
    return {MOE_FN(init_lists_kernel), dim3((unsigned)grid), dim3(256), 0};
}

int front_router_blocks(const RouterArgs& a) { return (a.E + 3) / 4; }

// shared_tb: 0 when the shared expert runs on MFMA tiles, else its GEMV token count.
KernelPick pick_front(const FrontArgs& f, bool small_router, bool select_in_router, int shared_tb) {
    const RouterArgs& a = f.r;
    const int grid = f.router_blocks + f.shared_blocks;
    const void* fn;
    size_t lds;
    if (small_router) {
        const bool shm = f.shared_blocks > 0 && shared_tb == 0;
        const int tb = tb_bucket(a.B);
        const int ns = tb_bucket((a.E + 63) / 64);
        // NS only matters when the router selects; the plain router uses NS = 1
        const int key = (tb * 2 + (shm ? 1 : 0)) * 32 + (select_in_router ? ns : 0);
        switch (key) {
#define MOE_FS(TB, SHM, NS) case (TB * 2 + SHM) * 32 + NS: \
    fn = MOE_FN((front_small_kernel<TB, (SHM != 0), (NS != 0), (NS ? NS : 1)>)); break;
#define MOE_FS_NS(TB, SHM) MOE_FS(TB, SHM, 0) MOE_FS(TB, SHM, 1) MOE_FS(TB, SHM, 2) MOE_FS(TB, SHM, 4) \
    MOE_FS(TB, SHM, 8) MOE_FS(TB, SHM, 16)
            MOE_FS_NS(1, 0) MOE_FS_NS(1, 1) MOE_FS_NS(2, 0) MOE_FS_NS(2, 1) MOE_FS_NS(4, 0) MOE_FS_NS(4, 1)
#undef MOE_FS_NS
#undef MOE_FS
            default: fn = nullptr;
        }
        lds = (size_t)a.B * a.H * 2;
    } else {
        return pick_front_dense(f);
    }
    return {fn, dim3(grid), dim3(256), lds};
}

KernelPick pick_front_dense(const FrontArgs& f) {
    const void* fn;
    switch ((f.r.B + 15) / 16) {
        case 1: fn = MOE_FN(front_dense_kernel<1>); break;
        case 2: fn = MOE_FN(front_dense_kernel<2>); break;
        case 3: fn = MOE_FN(front_dense_kernel<3>); break;
        default: fn = MOE_FN(front_dense_kernel<4>); break;
    }
    return {fn, dim3(f.router_blocks + f.shared_blocks), dim3(256), 0};
}

KernelPick pick_topk(const TopkArgs& t) {
    const RouterArgs& a = t.r;
    const void* fn;
    switch (tb_bucket((a.E + 63) / 64)) {
        case 1: fn = MOE_FN(topk_bucket_kernel<1>); break;
        case 2: fn = MOE_FN(topk_bucket_kernel<2>); break;
        case 4: fn = MOE_FN(topk_bucket_kernel<4>); break;
        case 8: fn = MOE_FN(topk_bucket_kernel<8>); break;
        default: fn = MOE_FN(topk_bucket_kernel<16>); break;
    }
    // one selecting workgroup of one wave per token up to batch 8, else
    // 256-thread workgroups of four tokens each
    const int threads = t.sel_blocks == 1 ? std::max(256, 64 * a.B) : 256;
    const int red = t.spart ? (a.B * t.Is + threads - 1) / threads : 0;
    return {fn, dim3(t.sel_blocks + red), dim3(threads), 0};
}

KernelPick pick_front_split(const FrontArgs& f) {
    const void* fn;
    switch (tb_bucket(f.r.B)) {
        case 1: fn = MOE_FN(front_split_kernel<1>); break;
        case 2: fn = MOE_FN(front_split_kernel<2>); break;
        default: fn = MOE_FN(front_split_kernel<4>); break;
    }
    return {fn, dim3(f.router_blocks + f.shared_blocks), dim3(256), 0};
}

KernelPick pick_gateup_select(const SelGateUpArgs& a, int max_entries) {
    const int tb = tb_bucket(a.r.B), ns = tb_bucket((a.r.E + 63) / 64);
    const void* f;
    switch (tb * 32 + ns) {
#define MOE_GS(TB, NS) case TB * 32 + NS: f = MOE_FN((gateup_select_kernel<TB, NS>)); break;
#define MOE_GS_NS(TB) MOE_GS(TB, 1) MOE_GS(TB, 2) MOE_GS(TB, 4) MOE_GS(TB, 8) MOE_GS(TB, 16)
        MOE_GS_NS(1) MOE_GS_NS(2) MOE_GS_NS(4)
#undef MOE_GS_NS
#undef MOE_GS
        default: f = nullptr;
    }
    return {f, dim3(max_entries * a.g.tiles_per_expert), dim3(256), (size_t)a.r.B * a.r.H * 2};
}

// gemv_tokens: the largest token count a GEMV tile of this list may see.
KernelPick pick_gateup(const GateUpArgs& a, int max_entries, int gemv_tokens) {
    const bool mf = a.mfma_min_tokens > 0;
    const void* f;
    const int tb = tb_bucket(gemv_tokens);
#define MOE_GU(TB) f = mf ? MOE_FN((gateup_kernel<TB, true>)) : MOE_FN((gateup_kernel<TB, false>));
    switch (tb) {
        case 1: MOE_GU(1) break;
        case 2: MOE_GU(2) break;
        case 4: MOE_GU(4) break;
        case 8: MOE_GU(8) break;
        case 16: MOE_GU(16) break;
        case 32: MOE_GU(32) break;
        default: MOE_GU(64) break;
    }
#undef MOE_GU
    size_t lds = (size_t)gemv_tokens * a.H * 2;
    if (mf) lds = std::max(lds, mfma_tile_lds_bytes());  // the MFMA tiles' staged activations
    return {f, dim3(max_entries * a.tiles_per_expert), dim3(256), lds};
}

// Output rows per down row block of the single launch for intermediate size I.
int down_rows_per_block(int I) {
    const int ur = I / 8;
    if (ur == 8) return DownShape<8, 1, 1>::R;
    if (ur == 16) return DownShape<16, 1, 1>::R;
    if (ur == 32) return DownShape<32, 1, 2>::R;
    return ur / 64 <= 4 ? DownShape<64, 1, 2>::R : DownShape<64, 5, 1>::R;
}

size_t down_h_lds_bytes(int B, int k, int I, int Is) { return ((size_t)B * k * I + (size_t)B * Is) * 4; }



KernelPick pick_down(const DownArgs& a) {
    const int ur = a.I / 8;
    const bool hl = a.h_in_lds != 0;
    const void* f;
    int rows;  // output rows per workgroup of the chosen instantiation
#define MOE_DN(LPR, NQ, RP)                                                                                     \
    {                                                                                                            \
        f = hl ? MOE_FN((down_combine_kernel<LPR, NQ, RP, true>)) : MOE_FN((down_combine_kernel<LPR, NQ, RP, false>)); \
        rows = DownShape<LPR, NQ, RP>::R;                                                                        \
    }
    if (ur == 8) MOE_DN(8, 1, 1)
    else if (ur == 16) MOE_DN(16, 1, 1)
    else if (ur == 32) MOE_DN(32, 1, 2)
    else {
        switch (ur / 64) {
            case 1: MOE_DN(64, 1, 2) break;
            case 2: MOE_DN(64, 2, 2) break;
            case 3: MOE_DN(64, 3, 2) break;
            // I = 2048 (the unsharded shape at batch 1-2): 16-row workgroups,
            // 448 at H = 7168, all resident at once; 8-row ones (896) ran a
            // second, partial generation: 60.8 -> 50.5 us at batch 1
            case 4: MOE_DN(64, 4, 4) break;
            case 5: MOE_DN(64, 5, 1) break;
            case 6: MOE_DN(64, 6, 1) break;
            case 7: MOE_DN(64, 7, 1) break;
            default: MOE_DN(64, 8, 1) break;
        }
    }
#undef MOE_DN
    const size_t lds = hl ? down_h_lds_bytes(a.B, a.k, a.I, a.s2 ? a.Is : 0) : (size_t)kDownHStage;
    return {f, dim3(a.H / rows), dim3(256), lds};
}

// Output-stationary down for batch <= 4, or a null func when the shape has no
// instantiation (I in {64, 128, 256, 512, 1024}) or h exceeds kDownOsLds.
KernelPick pick_down_os(const DownArgs& a) {
    const int ur = a.I / 8, tb = tb_bucket(a.B);
    const size_t lds = down_os_lds_bytes(a.B, a.k, a.I, a.s2 ? a.Is : 0);
    const void* f = nullptr;
    int lpr = 16;
    if (a.B <= 4 && lds <= (size_t)kDownOsLds) {
#define MOE_DO(LPR, NQ) \
    f = tb == 1 ? MOE_FN((down_os_kernel<1, LPR, NQ>)) : tb == 2 ? MOE_FN((down_os_kernel<2, LPR, NQ>)) \
                                                           : MOE_FN((down_os_kernel<4, LPR, NQ>));
        switch (ur) {
            case 8: MOE_DO(8, 1) lpr = 8; break;
            case 16: MOE_DO(16, 1) break;
            case 32: MOE_DO(16, 2) break;
            case 64: MOE_DO(16, 4) break;
            case 128: MOE_DO(16, 8) break;
            default: break;
        }
#undef MOE_DO
    }
    return {f, dim3(a.H / (4 * 64 / lpr)), dim3(256), lds};
}

size_t down_os_lds_bytes(int B, int k, int I, int Is) { return ((size_t)B * k + (size_t)B * (Is / I)) * I * 4; }

KernelPick pick_combine(const DownXArgs& a) {
    const void* f;
    switch (tb_bucket(a.k)) {
        case 1: f = MOE_FN(combine_kernel<1>); break;
        case 2: f = MOE_FN(combine_kernel<2>); break;
        case 4: f = MOE_FN(combine_kernel<4>); break;
        case 8: f = MOE_FN(combine_kernel<8>); break;
        default: f = MOE_FN(combine_kernel<16>); break;
    }
    return {f, dim3((a.B * a.H / 4 + 127) / 128), dim3(128), 0};
}

KernelPick pick_down_x(const DownXArgs& a) {
    // four 16-byte units per lane per row where I allows (short reductions),
    // 64 lanes per row from I = 2048
    const int ur = a.I / 8;
    const void* f;
#define MOE_DX(LPR, NQ) f = MOE_FN((down_x_kernel<LPR, NQ>));
    if (ur == 8) MOE_DX(2, 4)
    else if (ur == 16) MOE_DX(4, 4)
    else if (ur == 32) MOE_DX(8, 4)
    else if (ur == 64) MOE_DX(16, 4)
    else if (ur == 128) MOE_DX(32, 4)
    else {
        switch (ur / 64) {
            case 1: MOE_DX(64, 1) break;
            case 2: MOE_DX(64, 2) break;
            case 3: MOE_DX(64, 3) break;
            case 4: MOE_DX(64, 4) break;
            case 5: MOE_DX(64, 5) break;
            case 6: MOE_DX(64, 6) break;
            case 7: MOE_DX(64, 7) break;
            default: MOE_DX(64, 8) break;
        }
    }
#undef MOE_DX
    const int grid = (a.max_act + a.nsh) * ((a.H + kDownXRows - 1) / kDownXRows);
    return {f, dim3(grid), dim3(256), (size_t)kDownXLds};
}

template <int TB>
const void* layer_fn(int ns, int shape);  // moe_layer_tb{1,2,4}.hip
extern template const void* layer_fn<1>(int, int);
extern template const void* layer_fn<2>(int, int);
extern template const void* layer_fn<4>(int, int);

KernelPick pick_layer(const LayerArgs& L, size_t lds_bytes) {
    const RouterArgs& a = L.f.r;
    const int tb = tb_bucket(a.B);
    int ns = tb_bucket((a.E + 63) / 64);
    if (ns < 4) ns = 4;
    const int ur = L.d.I / 8;
    const int shape = ur == 8 ? 0 : ur == 16 ? 1 : ur == 32 ? 2 : (ur % 64 == 0 && ur / 64 <= 4) ? 2 + ur / 64 : -1;
    const void* fn = nullptr;
    if (shape >= 0 && ns <= 16) {
        if (tb == 1) fn = layer_fn<1>(ns, shape);
        else if (tb == 2) fn = layer_fn<2>(ns, shape);
        else if (tb == 4) fn = layer_fn<4>(ns, shape);
    }
    return {fn, dim3(1), dim3(256), lds_bytes};
}

}  // namespace moe
