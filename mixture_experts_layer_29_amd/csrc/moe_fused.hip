// moe_fused.hip -- batch 1 and 2: routed experts, shared down and combine in
// ONE launch after the router launch (gfx950).
//
// At small batch the layer is a chain: router logits -> top-k -> the selected
// experts' gate/up rows -> their down rows.  As separate launches, the down
// projection's weights are requested only after the gate/up launch has
// ended, and its launch pays a ramp and a tail in which HBM idles.  Here, after
// the router launch (front_split_kernel: logits, the shared expert's h), one
// grid of co-resident workgroups (two per CU) does the rest.  The B k
// (token, expert) pairs are the units of work, each with one token: at batch
// 2 two tokens rarely share an expert (about one pair in a hundred at the
// TP8 shard), and a shared one is simply read twice.
//
//   select    waves t < B of every workgroup select token t's top-k from the
//             logits (the selection is not handed between workgroups);
//   gate/up   tile g = four row pairs (one per wave) of pair p = g / (I/4);
//             workgroup b computes tiles b, b + G, ..., requesting the next
//             tile's rows as soon as the current tile's are consumed, stores
//             its rows of h_p, and once its last tile is stored counts each
//             tile on its pair's counter; the tile that completes pair p
//             raises p's flag in every replica of the flag block;
//   down      workgroup b owns output rows [b*R, b*R + R).  Right after its
//             counts it requests its W2 rows of all B k pairs (its S2 rows
//             went out before the selection) -- static weights -- then takes
//             each pair as soon as that pair's flag is up (per-pair
//             readiness: pairs that finish early are staged and multiplied
//             while later ones still stream), and ends with a fixed-order sum
//             per token: the shared expert, w_p * W2_p h_p over the token's
//             pairs, the residual, rounded to bf16 (round to nearest even).
//
// This follows the small-batch fusions of the Kimi K3 decode article (Part 1
// section 2: producer and consumer fused into one kernel at small batch; the
// Hungarian summary, "Kevesebb kernel": fewer kernels per layer) and its
// validation lesson (Part 2 section 3: only static weights are loaded before a
// synchronisation wait; h is read only after its flag is seen).
//
// Hand-off cost: every counter and flag replica sits on its own 256-byte line,
// and each workgroup polls one of 16 flag replicas, so no line sees more than
// I/4 increments or 32 pollers (one line polled and incremented by every
// workgroup of the grid serialised a whole launch on MI355X; replicated
// counters, incremented by every tile without a returned value, cost 1.4 us
// more at batch 1 than one counter per pair and replicated flags).  Data
// crossing workgroups (h) is stored and loaded with device-coherent
// (agent-scope) atomic accesses and a counter is updated only after the
// stores completed (the protocol and its argument are in moe_device.h).  Every
// wait is bounded: one that runs out sets ERR_TIMEOUT in meta and the launch
// still ends, so a lost hand-off gives a flagged wrong result, never a hang.
// The counters and flags are re-armed by the next layer step's router launch.
#include <algorithm>

#include "moe_device.h"

namespace moe {

// NS: selection slots (E <= 64 NS); NU: 16-byte units per lane of a routed
// gate/up row (H <= 512 NU); UP / SP: W2 / S2 units per thread in the down
// phase (at most TB k I / 128 and Is / 128); TB: tokens (the batch).  Unused
// units load a clamped, already cached address and are masked, so every load
// is unconditional and the compiler's wait counts stay exact (the gate/up rows
// are consumed while the loads behind them are still in flight).
template <int NS, int NU, int UP, int SP, int TB>
__global__ __launch_bounds__(256, 2) void fused_experts_kernel(FusedArgs a) {
    constexpr int UX = 4;  // x units per thread and token for the LDS staging (H <= 8192)
    static_assert(TB >= 1 && TB <= 2, "one or two tokens");
    __shared__ __align__(16) uint16_t s_x[TB * 8192];
    __shared__ __align__(16) float s_h[TB * 2048];   // h rows of ready pairs at p * I (B k I <= TB * 2048)
    __shared__ __align__(16) float s_hs[TB * 512];   // shared h per token (Is <= 512)
    __shared__ int32_t s_sel_e[TB * kMaxTopK];
    __shared__ float s_sel_w[TB * kMaxTopK];
    __shared__ __align__(16) int32_t s_ps[128];      // pair_slot scratch (workgroup 0)
    __shared__ unsigned s_new;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H, E = a.E, k = a.k, I = a.I, Is = a.Is;
    const int P = TB * k;  // pairs
    const int units = H >> 3;
    const int b = blockIdx.x, G = gridDim.x;
    const u32x4 zero = u32x4{0, 0, 0, 0};

    // ------------------- x, the S2 rows and hs (static or from the router
    // launch: they stream while the selection runs), then the selection
    u32x4 xr[TB][UX];
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
        for (int q = 0; q < UX; ++q) {
            const int u = tid + 256 * q;
            xr[t][q] = ld16(a.x + (size_t)t * H + 8 * (u < units ? u : 0));
        }
    // down rows: thread -> (row rr, lane-in-row l); its units are l + 16 q of
    // the row's B k I / 8 routed units and of the row's Is / 8 shared units
    const int rr = tid / kFusedRowThreads, l = tid % kFusedRowThreads;
    const int row = b * a.rows + rr;
    const bool row_ok = rr < a.rows && row < H;
    const int rowc = row_ok ? row : 0;
    const int nsu = Is >> 3;
    u32x4 s2u[SP];
#pragma unroll
    for (int q = 0; q < SP; ++q) {
        const int c = l + kFusedRowThreads * q;
        const bool ok = row_ok && c < nsu;
        s2u[q] = (Is > 0) ? ld16_stream(a.s2 + (size_t)rowc * Is + 8 * (ok ? c : 0)) : zero;
    }
    const bool hs_mine = tid < TB * Is / 4;  // hs is [B][Is]
    const float4 hsv = *reinterpret_cast<const float4*>(a.hs + 4 * (hs_mine ? tid : 0));
    if (wave < TB) {  // wave t selects token t
        const int t = wave;
        float v[NS];
#pragma unroll
        for (int m = 0; m < NS; ++m) {
            const int e = m * 64 + lane;
            v[m] = e < E ? a.z[(size_t)t * E + e] : -INFINITY;
        }
        int my_e;
        float my_z;
        topk_wave<NS>(v, E, k, lane, my_e, my_z);
        const bool mine = lane < k;
        const float zmax = __shfl(my_z, 0, 64);
        float w;
        if (a.score_fn == 0) {
            const float ex = mine ? expf(my_z - zmax) : 0.0f;
            float den;
            if (a.renormalize) {
                den = wave_sum(ex);
            } else {
                float part = 0.0f;
#pragma unroll
                for (int m = 0; m < NS; ++m) part += m * 64 + lane < E ? expf(v[m] - zmax) : 0.0f;
                den = wave_sum(part);
            }
            w = ex / den;
        } else {
            const float sg = mine ? 1.0f / (1.0f + expf(-my_z)) : 0.0f;
            w = a.renormalize ? sg / wave_sum(sg) : sg;
        }
        const bool bad = __ballot(mine && (my_e < 0 || my_e >= E)) != 0;
        if (mine) {
            s_sel_e[t * k + lane] = bad ? 0 : my_e;
            s_sel_w[t * k + lane] = bad ? 0.0f : w * a.routed_scale;
        }
        if (b == 0) {  // the routing, for the caller
            if (mine) {
                a.topk_idx[t * k + lane] = my_e;
                a.topk_w[t * k + lane] = w * a.routed_scale;
            }
            if (bad && lane == 0) atomicOr(&a.meta[M_ERR], ERR_BUCKET);
            if (TB == 1) {  // k distinct experts: pair j is entry j in slot j
                if (mine) {
                    a.act_e[lane] = my_e;
                    a.act_off[lane] = lane;
                    a.perm[lane] = lane;
                }
                if (lane == 0) {
                    a.act_off[k] = k;
                    a.meta[M_NACT] = bad ? 0 : k;
                }
            }
            if (lane == 0 && t == 0) {
                a.meta[M_GEMV_TILES] = P * (I / kPairsPerGemvTile);
                a.meta[M_MFMA_TILES] = 0;
            }
        }
    }
    if (wave >= TB && (a.pf_a || a.pf_b)) {
        // cross-layer prefetch while the selecting waves work: the next
        // layer's router and shared weights, read with ordinary (cached)
        // loads and dropped
        constexpr int PL = 256 - 64 * TB;  // prefetching lanes per workgroup
        const long long na = a.pf_a ? a.pf_a_units : 0, n = na + (a.pf_b ? a.pf_b_units : 0);
        const long long stride = (long long)G * PL;
        const long long u0 = (long long)b * PL + (tid - 64 * TB);
        u32x4 pv[kPrefetchUnits];
#pragma unroll
        for (int q = 0; q < kPrefetchUnits; ++q) {
            const long long u = u0 + q * stride;
            pv[q] = u < na ? ld16(a.pf_a + 8 * u) : u < n ? ld16(a.pf_b + 8 * (u - na)) : zero;
        }
        uint32_t sink = 0;
#pragma unroll
        for (int q = 0; q < kPrefetchUnits; ++q) sink ^= pv[q][0] ^ pv[q][3];
        asm volatile("" ::"v"(sink));  // keeps the loads; the value is not used
    }
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
        for (int q = 0; q < UX; ++q) {
            const int u = tid + 256 * q;
            if (u < units) st16(s_x + (size_t)t * H + 8 * u, xr[t][q]);
        }
    if (hs_mine) reinterpret_cast<float4*>(s_hs)[tid] = hsv;
    __syncthreads();
    if (TB > 1 && b == 0 && wave == 0) {
        // the bucketing of the B k pairs, for the caller (distinct experts, slots)
        const int e = lane < P ? s_sel_e[lane] : kNone;
        const PairSlot ps = pair_slot(e, P, lane, s_ps);
        if (lane < P) a.perm[ps.pos] = lane;
        if (ps.lead) {
            a.act_e[ps.apos] = e;
            a.act_off[ps.apos] = ps.pos;
        }
        const int nact = __popcll(__ballot(ps.lead));
        if (lane == 0) {
            a.act_off[nact] = P;
            a.meta[M_NACT] = nact;
        }
    }

    // --------- routed gate/up tiles b, b + G, ...; h stored; counted once all
    // are stored; then the W2 rows requested.  I is a power of two from 128
    // (the host checks): pair / unit indices below are shifts, not divisions
    const int tiles_per = I / kPairsPerGemvTile, tsh = __builtin_ctz(tiles_per);
    const int ntiles = P << tsh;
    u32x4 wg[NU], wu[NU];
    // this wave's gate and up rows of `tile` (< ntiles; calls are behind
    // workgroup-uniform branches: a per-unit select on the tile's validity
    // became per-unit branches that loaded the same registers, and the waits
    // between them serialised the row's loads)
    auto issue = [&](int tile) {
        const int p = tile >> tsh;
        const int i = (tile & (tiles_per - 1)) * kPairsPerGemvTile + wave;
        const uint16_t* grow = a.w13 + ((size_t)s_sel_e[p] * 2 * I + i) * H;
        const uint16_t* urow = grow + (size_t)I * H;
#pragma unroll
        for (int q = 0; q < NU; ++q) {
            const int u = q * 64 + lane;
            const int uc = u < units ? u : 0;
            wg[q] = ld16_stream(grow + 8 * uc);
            wu[q] = ld16_stream(urow + 8 * uc);
        }
    };
    if (b < ntiles) issue(b);
    for (int tile = b; tile < ntiles; tile += G) {  // workgroup-uniform
        const int p = tile >> tsh;
        const int t = TB == 1 ? 0 : (p >= k ? 1 : 0);
        const int i = (tile & (tiles_per - 1)) * kPairsPerGemvTile + wave;
        float ag = 0.0f, au = 0.0f;
#pragma unroll
        for (int q = 0; q < NU; ++q) {
            const int u = q * 64 + lane;
            if (u < units) {
                const u32x4 xv = ld16(s_x + (size_t)t * H + 8 * u);
                ag = dot8(wg[q], xv, ag);
                au = dot8(wu[q], xv, au);
            }
        }
        const float gs = wave_sum(ag), us = wave_sum(au);
        if (tile + G < ntiles) issue(tile + G);  // the rows are consumed: the next tile's go out
        if (lane == 0) st_dev(a.h + (size_t)p * I + i, silu_f(gs) * us);
    }
    stores_done_barrier();  // every h row of this workgroup's tiles is stored
    // counted: lane m of wave 0 counts tile b + m G on its pair's counter; the
    // value is looked at once the first W2 rows are requested
    const int my_tile = b + lane * G;
    const bool counts = wave == 0 && my_tile < ntiles;
    const int my_p = counts ? my_tile >> tsh : 0;
    int arrived = 0;
    if (counts)
        arrived = __hip_atomic_fetch_add(a.sync + kSyncLineWords * my_p, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    // wave 0 takes the counts before requesting its W2 rows: a wait placed at
    // their use, behind those requests, would hold the flags back until the
    // rows arrive (loads and atomics complete in order)
    if (wave == 0) __builtin_amdgcn_s_waitcnt(0);
    // ----------------------------------------------------------------- down
    // One phase per token (the shared expert's term first in its sum): its W2
    // rows (static weights) are requested -- the first token's once this
    // workgroup's h is counted, so the hand-off runs while they stream; the
    // next token's as soon as the previous token's rows are used -- and each
    // of its pairs is taken as soon as that pair's flag is up.  I / 8 is a
    // multiple of 16, so unit q of a phase belongs to the token's pair
    // q >> qsh and column unit c = 16 (q & (qpe - 1)) + l.
    float acc[TB];
    constexpr int UPT = UP / TB;  // W2 units per thread and phase
    const int upr = I >> 3, qpe = upr / kFusedRowThreads, qsh = __builtin_ctz(qpe);
    const int nq = k * qpe;  // this thread's routed units per token
    const int* flags = a.sync + kSyncLineWords * (kMaxFusedPairs + b % kFlagReplicas);
    int spins = 0;
#pragma unroll
    for (int t = 0; t < TB; ++t) {
        const int p0 = t * k;  // the token's first pair
        u32x4 w2u[UPT];
#pragma unroll
        for (int q = 0; q < UPT; ++q) {
            const bool ok = row_ok && q < nq;
            const int p = p0 + (ok ? q >> qsh : 0), c = ok ? kFusedRowThreads * (q & (qpe - 1)) + l : 0;
            w2u[q] = ld16_stream(a.w2 + ((size_t)s_sel_e[p] * H + rowc) * I + 8 * c);
        }
        if (t == 0 && counts && arrived == tiles_per - 1) {
            // pair my_p complete: raise its flag in every replica
#pragma unroll 1
            for (int r = 0; r < kFlagReplicas; ++r) st_dev(a.sync + kSyncLineWords * (kMaxFusedPairs + r) + my_p, 1);
        }
        // the token's shared expert term (S2 rows and hs are in), behind
        // its W2 requests so that its waits do not hold them back
        acc[t] = 0.0f;
#pragma unroll
        for (int q = 0; q < SP; ++q) {
            const int c = l + kFusedRowThreads * q;
            if (c < nsu) {
                const float4* hp = reinterpret_cast<const float4*>(s_hs + (size_t)t * Is + 8 * c);
                acc[t] = dot8_f32(s2u[q], hp[0], hp[1], acc[t]);
            }
        }
        float dq[UPT];
#pragma unroll
        for (int q = 0; q < UPT; ++q) dq[q] = 0.0f;
        const unsigned all = (k >= 32 ? ~0u : (1u << k) - 1u) << p0;  // the token's pairs
        unsigned done = 0;
        while (done != all) {
            if (wave == 0) {  // poll: lane p reads pair p's flag (one line)
                const bool up = lane < P && ld_dev(flags + lane) != 0;
                const unsigned ready = (unsigned)__ballot(up) & all;
                unsigned fresh = ready & ~done;
                if (!fresh) {
                    if (++spins > kSpinLimit) {  // give up on the rest: flagged, never a hang
                        if (lane == 0) atomicOr(&a.meta[M_ERR], ERR_TIMEOUT);
                        fresh = all & ~done;
                    } else {
                        __builtin_amdgcn_s_sleep(4);
                    }
                }
                if (lane == 0) s_new = fresh;
            }
            __syncthreads();
            const unsigned fresh = (unsigned)uni((int)s_new);
            if (fresh) {
                const int i4sh = tsh;  // I / 4 float4 per pair row = tiles_per
                for (int idx = tid; idx < P * I / 4; idx += 256)
                    if ((fresh >> (idx >> i4sh)) & 1u)
                        reinterpret_cast<float4*>(s_h)[idx] = ld_dev4(a.h + 4 * (size_t)idx);
                __syncthreads();
#pragma unroll
                for (int q = 0; q < UPT; ++q) {
                    const int p = p0 + (q >> qsh);
                    if (q < nq && ((fresh >> p) & 1u)) {
                        const int c = kFusedRowThreads * (q & (qpe - 1)) + l;
                        const float4* hp = reinterpret_cast<const float4*>(s_h + (size_t)p * I + 8 * c);
                        dq[q] = dot8_f32(w2u[q], hp[0], hp[1], 0.0f);
                    }
                }
                done |= fresh;
            }
            __syncthreads();  // s_new is rewritten by the next poll
        }
        // fixed order: the token's pairs in selection order, each pair's units in q order
        float d = 0.0f;
#pragma unroll
        for (int q = 0; q < UPT; ++q) {
            if (q < nq) {
                d += dq[q];
                if ((q & (qpe - 1)) == qpe - 1) {
                    acc[t] += s_sel_w[p0 + (q >> qsh)] * d;
                    d = 0.0f;
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < TB; ++t) {
        const float v0 = group_sum<kFusedRowThreads>(acc[t]);
        if (row_ok && l == 0) {
            float v = v0;
            if (a.add_residual) v += __uint_as_float((uint32_t)a.x[(size_t)t * H + row] << 16);
            a.out[(size_t)t * H + row] = f32_to_bf16_rne(v);
        }
    }
}

#define MOE_FN(f) reinterpret_cast<const void*>(&f)

KernelPick pick_fused_experts(const FusedArgs& a, int resident_wgs) {
    const KernelPick none{nullptr, dim3(1), dim3(256), 0};
    const int H = a.H, E = a.E, k = a.k, I = a.I, Is = a.Is, B = a.B;
    // I a power of two from 128 (unit -> pair maps are shifts), Is a multiple of 128 up to 512
    if (B < 1 || B > 2 || H % 64 || H > 8192 || E > 1024 || k > kMaxTopK || B * k > kMaxFusedPairs || I < 128 ||
        (I & (I - 1)) || Is % 128 || Is > 512)
        return none;
    const int tiles = B * k * (I / kPairsPerGemvTile);
    const int nru = B * k * I / 8;
    if (nru / kFusedRowThreads > kFusedMaxUnits) return none;
    // at most 16 output rows per workgroup; every workgroup resident at once
    const int G = std::max(std::min(tiles, resident_wgs), (H + 15) / 16);
    if (G > resident_wgs || (tiles + G - 1) / G > 64) return none;  // one counting lane per tile
    const int ns = (E + 63) / 64, nu = (H / 8 + 63) / 64, up = nru / kFusedRowThreads, sp = Is / 128;
    const void* f = nullptr;
    if (B == 1) {
        if (ns <= 8 && ns > 4 && nu == 14 && up == 16 && sp == 2) f = MOE_FN((fused_experts_kernel<8, 14, 16, 2, 1>));
        else if (ns == 1 && nu == 1 && up <= 2 && sp <= 1) f = MOE_FN((fused_experts_kernel<1, 1, 2, 1, 1>));
        else if (up <= 16) f = MOE_FN((fused_experts_kernel<16, 16, 16, 4, 1>));
    } else {
        if (ns <= 8 && ns > 4 && nu == 14 && up == 32 && sp == 2) f = MOE_FN((fused_experts_kernel<8, 14, 32, 2, 2>));
        else if (ns == 1 && nu == 1 && up <= 4 && sp <= 1) f = MOE_FN((fused_experts_kernel<1, 1, 4, 1, 2>));
    }
    if (!f) return none;
    return {f, dim3(G), dim3(256), 0};
}

}  // namespace moe
