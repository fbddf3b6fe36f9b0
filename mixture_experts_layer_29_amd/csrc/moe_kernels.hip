// moe_kernels.hip -- gfx950 (CDNA4) kernels of the decode-time MoE layer,
// staged form (one launch per stage; the single-launch form for batch <= 4
// is in moe_layer.h).
//
// One layer is, on the main stream:
//   front      batch <= 4: front_small -- router GEMV, then the last workgroup
//              to arrive selects the top-k experts of every token, computes the
//              routing weights and buckets the (token, slot) pairs by expert;
//              batch > 4: front_mfma -- split-K MFMA router GEMM accumulating
//              fp32 logits -- then topk_bucket -- one wave per token selects
//              the top-k, the last workgroup buckets with an LDS histogram;
//              trailing workgroups of the front launch run the shared expert's
//              gate/up, which needs only x;
//   gateup     grouped gate/up projection + SiLU*up over the active experts:
//              GEMV tiles (full K, VALU dot2) for experts with few tokens -- the
//              "small-matrix" form the Kimi K3 decode article uses at batch 1-2
//              -- and split-K MFMA tiles for experts with many tokens -- the
//              "split-K" form it uses at larger batches (Part 1 section 1);
//   down       down projection of every active expert and of the shared
//              expert, routing-weighted sum, residual add, bf16 output;
//              output-stationary, so no atomics and a fixed summation order;
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
    __shared__ int32_t s_cand_e[4 * kMaxTopK];
    __shared__ float s_cand_z[4 * kMaxTopK];
    __shared__ float s_z[kMaxExperts];
    __shared__ int s_flag;

    router_rows<TB, SELECT>(a, blockIdx.x, s_x);
    if constexpr (!SELECT) return;

    // the last router workgroup to arrive selects and buckets
    if (!arrive_last(reinterpret_cast<unsigned*>(&a.meta[M_ROUTER_CNT]), f.router_blocks, &s_flag)) return;

    select_tokens<NS>(a, 0, a.z, nullptr, false, s_pair_e, s_cand_e, s_cand_z, s_z);
    __syncthreads();
    if ((threadIdx.x >> 6) == 0) bucket_wave(a, s_pair_e, threadIdx.x & 63);
}

template <int SHTB>  // 0: the shared expert runs on MFMA tiles, else its GEMV token bucket
__global__ __launch_bounds__(256) void front_mfma_kernel(FrontArgs f) {
    extern __shared__ __align__(16) uint16_t s_x[];
    if ((int)blockIdx.x >= f.router_blocks) {
        const int local = blockIdx.x - f.router_blocks;
        if constexpr (SHTB == 0) mfma_gateup_tile<4>(f.s, f.s.w, 0, 0, f.r.B, local);
        else gemv_gateup_tile<SHTB>(f.s, f.s.w, 0, f.r.B, local, s_x);
        return;
    }
    router_mfma_tile(f.r, blockIdx.x);
}

// Logits = zacc + bias (zacc re-armed to zero), top-k, weights, bucketing.
// With one workgroup (batch <= 4) everything stays in registers and LDS: no
// atomics, fences or reloads sit between reading the logits and writing the
// buckets.  With several, the last workgroup to arrive buckets all pairs.
template <int NS>
__global__ __launch_bounds__(256) void topk_bucket_kernel(RouterArgs a) {
    __shared__ int32_t s_pair_e[kMaxBatch * kMaxTopK];
    __shared__ int32_t s_rank[kMaxBatch * kMaxTopK];
    __shared__ int32_t s_cnt[kMaxExperts];
    __shared__ int32_t s_cand_e[4 * kMaxTopK];
    __shared__ float s_cand_z[4 * kMaxTopK];
    __shared__ float s_z[kMaxExperts];
    __shared__ int32_t s_tmp[8];
    __shared__ int32_t s_nmfma;
    __shared__ int s_flag;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int B = a.B, np = B * a.k;
    const bool single = gridDim.x == 1;
    select_tokens<NS>(a, blockIdx.x * 4, a.zacc, a.bias, true, single ? s_pair_e : nullptr, s_cand_e, s_cand_z,
                      s_z);
    if (!single) {
        if (!arrive_last(reinterpret_cast<unsigned*>(&a.meta[M_ROUTER_CNT]), gridDim.x, &s_flag)) return;
        for (int p = tid; p < np; p += 256) s_pair_e[p] = ld_dev(a.topk_idx + p);
        __syncthreads();
    }
    if (np <= 64) {
        if (wave == 0) bucket_wave(a, s_pair_e, lane);
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
        mfma_gateup_tile<4>(a, W, entry, off, T, local);
    } else {
        if (T > TB) {
            if (threadIdx.x == 0 && local == 0) atomicOr(&a.meta[M_ERR], ERR_TILE);
            return;
        }
        gemv_gateup_tile<TB>(a, W, off, T, local, s_x);
    }
}

template <int LPR, int NQ, int RP, bool HLDS>
__global__ __launch_bounds__(256) void down_combine_kernel(DownArgs a) {
    extern __shared__ __align__(16) float s_h[];
    __shared__ float s_acc[kMaxBatch * DownShape<LPR, NQ, RP>::R];
    down_rows<LPR, NQ, RP, HLDS, DOWN_ALL>(a, blockIdx.x, s_h, s_acc, [] {});
}

__global__ void init_lists_kernel(InitArgs a) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t < a.B) a.sh_perm[t] = t;
    if (t == 0) {
        a.meta[M_SHARED_NACT] = 1;
        a.sh_act_e[0] = 0;
        a.sh_act_off[0] = 0;
        a.sh_act_off[1] = a.B;
    }
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
    return {MOE_FN(init_lists_kernel), dim3((a.B + 63) / 64), dim3(64), 0};
}

int front_router_blocks(const RouterArgs& a, bool small_router) {
    return small_router ? (a.E + 3) / 4
                        : ((a.E + kRouterRowsPerMfmaTile - 1) / kRouterRowsPerMfmaTile) * a.ksplit;
}

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
        const int tb = f.shared_blocks > 0 && shared_tb > 0 ? tb_bucket(shared_tb) : 0;
        switch (tb) {
            case 0: fn = MOE_FN(front_mfma_kernel<0>); break;
            case 1: fn = MOE_FN(front_mfma_kernel<1>); break;
            case 2: fn = MOE_FN(front_mfma_kernel<2>); break;
            case 4: fn = MOE_FN(front_mfma_kernel<4>); break;
            case 8: fn = MOE_FN(front_mfma_kernel<8>); break;
            case 16: fn = MOE_FN(front_mfma_kernel<16>); break;
            case 32: fn = MOE_FN(front_mfma_kernel<32>); break;
            default: fn = MOE_FN(front_mfma_kernel<64>); break;
        }
        lds = tb ? (size_t)shared_tb * a.H * 2 : 0;
    }
    return {fn, dim3(grid), dim3(256), lds};
}

KernelPick pick_topk(const RouterArgs& a) {
    const void* fn;
    switch (tb_bucket((a.E + 63) / 64)) {
        case 1: fn = MOE_FN(topk_bucket_kernel<1>); break;
        case 2: fn = MOE_FN(topk_bucket_kernel<2>); break;
        case 4: fn = MOE_FN(topk_bucket_kernel<4>); break;
        case 8: fn = MOE_FN(topk_bucket_kernel<8>); break;
        default: fn = MOE_FN(topk_bucket_kernel<16>); break;
    }
    return {fn, dim3((a.B + 3) / 4), dim3(256), 0};
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
    return {f, dim3(max_entries * a.tiles_per_expert), dim3(256), (size_t)gemv_tokens * a.H * 2};
}

// Output rows per down_combine workgroup for intermediate size I (matches pick_down).
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
#define MOE_DN(LPR, NQ, RP) \
    f = hl ? MOE_FN((down_combine_kernel<LPR, NQ, RP, true>)) : MOE_FN((down_combine_kernel<LPR, NQ, RP, false>));
    if (ur == 8) MOE_DN(8, 1, 1)
    else if (ur == 16) MOE_DN(16, 1, 1)
    else if (ur == 32) MOE_DN(32, 1, 2)
    else {
        switch (ur / 64) {
            case 1: MOE_DN(64, 1, 2) break;
            case 2: MOE_DN(64, 2, 2) break;
            case 3: MOE_DN(64, 3, 2) break;
            case 4: MOE_DN(64, 4, 2) break;
            case 5: MOE_DN(64, 5, 1) break;
            case 6: MOE_DN(64, 6, 1) break;
            case 7: MOE_DN(64, 7, 1) break;
            default: MOE_DN(64, 8, 1) break;
        }
    }
#undef MOE_DN
    const size_t lds = hl ? down_h_lds_bytes(a.B, a.k, a.I, a.s2 ? a.Is : 0) : (size_t)kDownHStage;
    return {f, dim3(a.H / down_rows_per_block(a.I)), dim3(256), lds};
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
