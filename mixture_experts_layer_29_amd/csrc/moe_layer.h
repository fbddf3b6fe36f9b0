// moe_layer.h -- the whole decode-time MoE layer in one persistent launch
// (batch <= 4), built from the work units in moe_device.h.  Instantiated per
// token bucket TB in moe_layer_tb{1,2,4}.hip so the variants compile in
// parallel.
#pragma once
#include "moe_device.h"

namespace moe {

// ---------------------------------------------------------------------------
// single-launch layer (batch <= 4)
// ---------------------------------------------------------------------------

// Tasks, in an order where every dependency points to a lower index:
//   router rows (the last to finish selects, buckets and publishes M_SEL),
//   shared gate/up tiles, shared down row blocks (fp32 into s_out),
//   routed gate/up tiles (after M_SEL), routed down row blocks (W2 rows are
//   requested before waiting for the gate/up tiles; finalize adds s_out and
//   the residual).  Workgroup b starts with task b; further tasks are claimed
//   in increasing order through M_NEXT, the next claim issued while the
//   current task runs.  So the lowest unfinished task is always running and
//   everything it waits for has a lower index and is done: no deadlock,
//   provided every workgroup of the grid is resident at once, which the host
//   ensures by sizing the grid from the occupancy.  Each wait is bounded all
//   the same (ERR_TIMEOUT).  The last workgroup to leave re-arms the counters.
template <int TB, int NS, int LPR, int NQ, int RP>
__global__ __launch_bounds__(256) void layer_kernel(LayerArgs L) {
    extern __shared__ __align__(16) unsigned char s_dyn[];  // x staging, then h rows of down tasks
    __shared__ int32_t s_pair_e[4 * kMaxTopK];
    __shared__ __align__(16) int32_t s_ps[128];  // pair_slot scratch

    __shared__ float s_acc[4 * DownShape<LPR, NQ, RP>::R];  // batch <= 4
    __shared__ int s_task, s_flag;
    uint16_t* s_x = reinterpret_cast<uint16_t*>(s_dyn);
    float* s_h = reinterpret_cast<float*>(s_dyn);
    const RouterArgs& a = L.f.r;
    int32_t* meta = a.meta;
    const int tid = threadIdx.x;
    const int t_sgu = L.n_router, t_sdown = t_sgu + L.n_sgu, t_gu = t_sdown + L.n_sdown;
    const int t_down = t_gu + L.n_gu, t_end = t_down + L.n_down;
    const int n_static = gridDim.x;  // the host keeps the grid <= the task count

    int t = blockIdx.x;
    while (t < t_end) {
        // claim the next task now; its value is only needed after this one
        int next = 0;
        if (tid == 0) next = n_static + atomicAdd(&meta[M_NEXT], 1);
        if (t < t_sgu) {
            router_rows<TB, true>(a, t, s_x);
            if (arrive_last(reinterpret_cast<unsigned*>(&meta[M_ROUTER_CNT]), L.n_router, &s_flag)) {
                select_tokens<NS>(a, 0, a.z, nullptr, false, s_pair_e);
                if ((tid >> 6) == 0) bucket_wave(a, s_pair_e, tid & 63, s_ps);
                publish(&meta[M_SEL]);
            }
        } else if (t < t_sdown) {
            const int local = t - t_sgu;
            bool did = true;
            if (L.shared_mfma) did = mfma_gateup_tile<1>(L.f.s, L.f.s.w, 0, 0, a.B, local);
            else gemv_gateup_tile<TB>(L.f.s, L.f.s.w, 0, a.B, local, s_x);
            if (did) publish(&meta[M_SGU_DONE]);
        } else if (t < t_gu) {
            down_rows<LPR, NQ, RP, true, DOWN_SHARED, true>(L.d, t - t_sdown, s_h, s_acc,
                                         [&] { wait_count(&meta[M_SGU_DONE], L.sgu_expect, meta); });
            publish(&meta[M_SDOWN_DONE]);
        } else if (t < t_down) {
            wait_count(&meta[M_SEL], 1, meta);
            const GateUpArgs& g = L.g;
            const int entry = (t - t_gu) / g.tiles_per_expert, local = (t - t_gu) % g.tiles_per_expert;
            if (entry < uni(ld_dev(g.n_act))) {
                const int e = uni(ld_dev(g.act_e + entry)), off = uni(ld_dev(g.act_off + entry));
                const int T = uni(ld_dev(g.act_off + entry + 1)) - off;
                const bool mfma = g.mfma_min_tokens > 0 && T >= g.mfma_min_tokens;
                // tiles the bucketing counted for this entry publish even on a bad entry,
                // so the down tasks' wait still ends (the error flag tells the caller)
                bool counted = !mfma || local < (g.n / kPairsPerMfmaTile) * g.ksplit;
                if (e < 0 || e >= g.n_experts || off < 0 || T < 1 || off + T > g.max_slots ||
                    T > (mfma ? 16 : TB)) {
                    if (tid == 0) atomicOr(&meta[M_ERR], ERR_TILE);
                } else {
                    const uint16_t* W = g.w + (size_t)e * (size_t)g.expert_stride;
                    if (mfma) counted = mfma_gateup_tile<1>(g, W, entry, off, T, local);
                    else gemv_gateup_tile<TB, true>(g, W, off, T, local, s_x);
                }
                if (counted) publish(&meta[M_GU_DONE]);
            }
        } else {
            wait_count(&meta[M_SEL], 1, meta);
            down_rows<LPR, NQ, RP, true, DOWN_ROUTED, true>(L.d, t - t_down, s_h, s_acc, [&] {
                wait_count(&meta[M_GU_DONE], ld_dev(meta + M_GEMV_TILES) + ld_dev(meta + M_MFMA_TILES), meta);
                wait_count(&meta[M_SDOWN_DONE], L.n_sdown, meta);
            });
        }
        if (tid == 0) s_task = next;
        __syncthreads();  // also: LDS is reused by the next task
        t = uni(s_task);
        __syncthreads();
    }
    // the last workgroup to leave re-arms the counters for the next launch
    if (tid == 0) {
        if (atomicAdd(&meta[M_EXIT], 1) == (int)gridDim.x - 1) {
            st_dev(meta + M_NEXT, 0);
            st_dev(meta + M_SGU_DONE, 0);
            st_dev(meta + M_SDOWN_DONE, 0);
            st_dev(meta + M_GU_DONE, 0);
            st_dev(meta + M_SEL, 0);
            st_dev(meta + M_EXIT, 0);
        }
    }
}

// The layer kernel for token bucket TB, selection slots NS (4, 8 or 16 wave
// slots of 64 experts) and down shape index `shape` (0..2 for
// I = 64, 128, 256, then 2 + I / 512 up to I = 2048); null if none.
template <int TB>
const void* layer_fn(int ns, int shape) {
#define MOE_L(NS, SH, LPR, NQ, RP) \
    if (ns == NS && shape == SH) return reinterpret_cast<const void*>(&layer_kernel<TB, NS, LPR, NQ, RP>);
#define MOE_LS(NS) MOE_L(NS, 0, 8, 1, 1) MOE_L(NS, 1, 16, 1, 1) MOE_L(NS, 2, 32, 1, 2) \
    MOE_L(NS, 3, 64, 1, 2) MOE_L(NS, 4, 64, 2, 2) MOE_L(NS, 5, 64, 3, 2) MOE_L(NS, 6, 64, 4, 2)
    MOE_LS(4) MOE_LS(8) MOE_LS(16)
#undef MOE_LS
#undef MOE_L
    return nullptr;
}

}  // namespace moe
