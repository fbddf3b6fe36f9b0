// moe_fused.hip -- batch 1: routed experts, shared down and combine in ONE
// launch after the router launch (gfx950).
//
// At batch 1 the layer is a chain: router logits -> top-k -> the selected
// experts' gate/up rows -> their down rows.  As separate launches, the down
// projection's weights are requested only after the gate/up launch has
// ended, and its launch pays a ramp and a tail in which HBM idles.  Here, after
// the router launch (front_split_kernel: logits, the shared expert's h), one
// grid of co-resident workgroups (two per CU) does the rest:
//
//   select    every workgroup selects the top-k from the logits itself (one
//             wave), so the selection is not handed between workgroups;
//   gate/up   workgroup b computes routed tile b: four row pairs (one per wave)
//             of selected expert j = b / (I/4), stores its rows of h_j and
//             counts them on expert j's own counter; the tile that completes
//             expert j raises j's flag in every replica of the flag block;
//   down      workgroup b owns output rows [b*R, b*R + R).  Right after the
//             selection it requests its W2 rows of all k selected experts and
//             its S2 rows -- static weights, so they stream together with the
//             gate/up rows -- then takes each expert as soon as that expert's
//             flag is up (per-expert readiness: experts that finish early are
//             staged and multiplied while later ones still stream), and ends
//             with a fixed-order sum w_j * W2_j h_j over j, the shared expert
//             and the residual, rounded to bf16 (round to nearest even).
//
// This follows the small-batch fusions of the Kimi K3 decode article (Part 1
// section 2: producer and consumer fused into one kernel at small batch; the
// Hungarian summary, "Kevesebb kernel": fewer kernels per layer) and its
// validation lesson (Part 2 section 3: only static weights are loaded before a
// synchronisation wait; h is read only after its flag is seen).
//
// Hand-off cost: every counter and flag replica sits on its own 256-byte line,
// and each workgroup polls one of 16 flag replicas, so no line sees more than
// 64 increments or 32 pollers (one line polled and incremented by every
// workgroup of the grid serialised a whole launch on MI355X).  Data crossing
// workgroups (h) is stored and loaded with device-coherent (agent-scope)
// atomic accesses and a counter is updated only after the stores completed
// (the protocol and its argument are in moe_device.h).  Every wait is bounded:
// one that runs out sets ERR_TIMEOUT in meta and the launch still ends, so a
// lost hand-off gives a flagged wrong result, never a hang.  The counters and
// flags are re-armed by the next layer step's router launch.
#include <algorithm>

#include "moe_device.h"

namespace moe {

// NS: selection slots (E <= 64 NS); NU: 16-byte units per lane of a routed
// gate/up row (H <= 512 NU); UP / SP: W2 / S2 units per thread in the down
// phase (at most k I / 128 and Is / 128).  Unused units load a clamped,
// already cached address and are masked, so every load is unconditional and
// the compiler's wait counts stay exact (the gate/up rows are consumed while
// the W2 rows behind them are still in flight).
template <int NS, int NU, int UP, int SP>
__global__ __launch_bounds__(256, 2) void fused_b1_kernel(FusedArgs a) {
    constexpr int UX = 4;  // x units per thread for the LDS staging (H <= 8192)
    __shared__ __align__(16) uint16_t s_x[8192];
    __shared__ __align__(16) float s_h[2048];   // h_j rows of ready experts at j * I (k I <= 2048)
    __shared__ __align__(16) float s_hs[512];   // shared h (Is <= 512)
    __shared__ int32_t s_sel_e[kMaxTopK];
    __shared__ float s_sel_w[kMaxTopK];
    __shared__ unsigned s_new;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H, E = a.E, k = a.k, I = a.I, Is = a.Is;
    const int units = H >> 3;
    const int b = blockIdx.x;
    const u32x4 zero = u32x4{0, 0, 0, 0};

    // ------------------- x, the S2 rows and hs (static or from the router
    // launch: they stream while the selection runs), then the selection
    u32x4 xr[UX];
#pragma unroll
    for (int q = 0; q < UX; ++q) {
        const int u = tid + 256 * q;
        xr[q] = ld16(a.x + 8 * (u < units ? u : 0));
    }
    // down rows: thread -> (row rr, lane-in-row l); its units are l + 16 q of
    // the row's k * I / 8 routed units and of the row's Is / 8 shared units
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
    const bool hs_mine = tid < Is / 4;
    const float4 hsv = *reinterpret_cast<const float4*>(a.hs + 4 * (hs_mine ? tid : 0));
    if (wave == 0) {
        float v[NS];
#pragma unroll
        for (int m = 0; m < NS; ++m) {
            const int e = m * 64 + lane;
            v[m] = e < E ? a.z[e] : -INFINITY;
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
            s_sel_e[lane] = bad ? 0 : my_e;
            s_sel_w[lane] = bad ? 0.0f : w * a.routed_scale;
        }
        if (b == 0) {  // the routing, for the caller
            if (mine) {
                a.topk_idx[lane] = my_e;
                a.topk_w[lane] = w * a.routed_scale;
                a.act_e[lane] = my_e;
                a.act_off[lane] = lane;
                a.perm[lane] = lane;
            }
            if (lane == 0) {
                a.act_off[k] = k;
                a.meta[M_NACT] = bad ? 0 : k;
                a.meta[M_GEMV_TILES] = k * (I / kPairsPerGemvTile);
                a.meta[M_MFMA_TILES] = 0;
                if (bad) atomicOr(&a.meta[M_ERR], ERR_BUCKET);
            }
        }
    }
    if (wave > 0 && (a.pf_a || a.pf_b)) {
        // cross-layer prefetch while wave 0 selects: the next layer's router
        // and shared weights, read with ordinary (cached) loads and dropped
        const long long na = a.pf_a ? a.pf_a_units : 0, n = na + (a.pf_b ? a.pf_b_units : 0);
        const long long stride = (long long)gridDim.x * 192;
        const long long u0 = (long long)b * 192 + (tid - 64);
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
    for (int q = 0; q < UX; ++q) {
        const int u = tid + 256 * q;
        if (u < units) st16(s_x + 8 * u, xr[q]);
    }
    if (hs_mine) reinterpret_cast<float4*>(s_hs)[tid] = hsv;
    __syncthreads();

    // --------- routed gate/up rows; h published; then the W2 rows requested
    // I is a power of two from 128 (the host checks): expert / unit indices
    // below are shifts, not divisions
    const int tiles_per = I / kPairsPerGemvTile, tsh = __builtin_ctz(tiles_per);
    const bool has_tile = b < k * tiles_per;  // workgroup-uniform
    const int j_t = has_tile ? b >> tsh : 0;
    const int i_t = (has_tile ? b & (tiles_per - 1) : 0) * kPairsPerGemvTile + wave;
    const uint16_t* grow = a.w13 + ((size_t)s_sel_e[j_t] * 2 * I + i_t) * H;
    const uint16_t* urow = grow + (size_t)I * H;
    u32x4 wg[NU], wu[NU];
#pragma unroll
    for (int q = 0; q < NU; ++q) {
        const int u = q * 64 + lane;
        const int uc = (has_tile && u < units) ? u : 0;
        wg[q] = ld16_stream(grow + 8 * uc);
        wu[q] = ld16_stream(urow + 8 * uc);
    }
    int32_t* cnt_j = a.sync + kSyncLineWords * j_t;
    int arrived = 0;
    if (has_tile) {
        float ag = 0.0f, au = 0.0f;
#pragma unroll
        for (int q = 0; q < NU; ++q) {
            const int u = q * 64 + lane;
            if (u < units) {
                const u32x4 xv = ld16(s_x + 8 * u);
                ag = dot8(wg[q], xv, ag);
                au = dot8(wu[q], xv, au);
            }
        }
        const float gs = wave_sum(ag), us = wave_sum(au);
        if (lane == 0) st_dev(a.h + (size_t)j_t * I + i_t, silu_f(gs) * us);
        stores_done_barrier();
        // counted now; its value is looked at once the W2 rows are requested
        if (tid == 0) arrived = __hip_atomic_fetch_add(cnt_j, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // W2 rows of the k selected experts (static weights): requested after the
    // gate/up rows are consumed and h is counted, so the hand-off below runs
    // while they stream.  I / 8 is a multiple of 16, so unit q of every thread
    // belongs to expert q >> qsh and column unit c = 16 (q & (qpe - 1)) + l.
    const int upr = I >> 3, qpe = upr / kFusedRowThreads, qsh = __builtin_ctz(qpe);
    const int nq = k * qpe;  // this thread's routed units
    u32x4 w2u[UP];
#pragma unroll
    for (int q = 0; q < UP; ++q) {
        const bool ok = row_ok && q < nq;
        const int j = ok ? q >> qsh : 0, c = ok ? kFusedRowThreads * (q & (qpe - 1)) + l : 0;
        w2u[q] = ld16_stream(a.w2 + ((size_t)s_sel_e[j] * H + rowc) * I + 8 * c);
    }
    if (has_tile && tid == 0 && arrived == tiles_per - 1) {
        // expert j complete: raise its flag in every replica
#pragma unroll 1
        for (int r = 0; r < kFlagReplicas; ++r) st_dev(a.sync + kSyncLineWords * (kMaxTopK + r) + j_t, 1);
    }

    // ----------------------------------------------------------------- down
    float acc = 0.0f;
#pragma unroll
    for (int q = 0; q < SP; ++q) {
        const int c = l + kFusedRowThreads * q;
        if (c < nsu) {
            const float4* hp = reinterpret_cast<const float4*>(s_hs + 8 * c);
            acc = dot8_f32(s2u[q], hp[0], hp[1], acc);
        }
    }
    float dq[UP];
#pragma unroll
    for (int q = 0; q < UP; ++q) dq[q] = 0.0f;
    const int* flags = a.sync + kSyncLineWords * (kMaxTopK + b % kFlagReplicas);
    const unsigned all = k >= 32 ? ~0u : (1u << k) - 1u;
    unsigned done = 0;
    int spins = 0;
    while (done != all) {
        if (wave == 0) {  // poll: lane j reads expert j's flag (one line)
            const bool up = lane < k && ld_dev(flags + lane) != 0;
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
            const int i4sh = tsh;  // I / 4 float4 per expert row = tiles_per
            for (int idx = tid; idx < k * I / 4; idx += 256)
                if ((fresh >> (idx >> i4sh)) & 1u)
                    reinterpret_cast<float4*>(s_h)[idx] = ld_dev4(a.h + 4 * (size_t)idx);
            __syncthreads();
#pragma unroll
            for (int q = 0; q < UP; ++q) {
                const int j = q >> qsh;
                if (q < nq && ((fresh >> j) & 1u)) {
                    const int c = kFusedRowThreads * (q & (qpe - 1)) + l;
                    const float4* hp = reinterpret_cast<const float4*>(s_h + (size_t)j * I + 8 * c);
                    dq[q] = dot8_f32(w2u[q], hp[0], hp[1], 0.0f);
                }
            }
            done |= fresh;
        }
        __syncthreads();  // s_new is rewritten by the next poll
    }
    // fixed order: expert 0..k-1 (units q of expert j are consecutive), each
    // expert's units in q order
    {
        float d = 0.0f;
#pragma unroll
        for (int q = 0; q < UP; ++q) {
            if (q < nq) {
                d += dq[q];
                if ((q & (qpe - 1)) == qpe - 1) {
                    acc += s_sel_w[q >> qsh] * d;
                    d = 0.0f;
                }
            }
        }
    }
    acc = group_sum<kFusedRowThreads>(acc);
    if (row_ok && l == 0) {
        float v = acc;
        if (a.add_residual) v += __uint_as_float((uint32_t)a.x[row] << 16);
        a.out[row] = f32_to_bf16_rne(v);
    }
}

#define MOE_FN(f) reinterpret_cast<const void*>(&f)

KernelPick pick_fused_b1(const FusedArgs& a, int resident_wgs) {
    const KernelPick none{nullptr, dim3(1), dim3(256), 0};
    const int H = a.H, E = a.E, k = a.k, I = a.I, Is = a.Is;
    // I a power of two from 128 (unit -> expert maps are shifts), Is a multiple of 128 up to 512
    if (H % 64 || H > 8192 || E > 1024 || k > kMaxTopK || I < 128 || (I & (I - 1)) || Is % 128 || Is > 512)
        return none;
    const int tiles = k * (I / kPairsPerGemvTile);
    const int nru = k * I / 8;
    if (nru / kFusedRowThreads > kFusedMaxUnits) return none;
    // one routed tile per workgroup and at most 16 output rows per workgroup
    const int G = std::max(tiles, (H + 15) / 16);
    if (G > resident_wgs) return none;
    const int ns = (E + 63) / 64, nu = (H / 8 + 63) / 64, up = nru / kFusedRowThreads, sp = Is / 128;
    const void* f = nullptr;
    if (ns <= 8 && ns > 4 && nu == 14 && up == 16 && sp == 2) f = MOE_FN((fused_b1_kernel<8, 14, 16, 2>));
    else if (ns == 1 && nu == 1 && up <= 2 && sp <= 1) f = MOE_FN((fused_b1_kernel<1, 1, 2, 1>));
    else f = MOE_FN((fused_b1_kernel<16, 16, 16, 4>));
    return {f, dim3(G), dim3(256), 0};
}

}  // namespace moe
