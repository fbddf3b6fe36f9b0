// moe_kernels.hip -- gfx950 (CDNA4) kernels of the decode-time MoE layer.
//
// Three kernels make one layer on the main stream, plus one on a second
// stream for the shared expert (the Kimi K3 decode article, Part 1 section 3,
// runs the shared expert on a separate stream, overlapped with routing):
//
//   router_topk   router GEMV, then the last workgroup to arrive selects the
//                 top-k experts per token, computes the routing weights and
//                 buckets the (token, slot) pairs by expert (LDS histogram);
//   gateup        grouped gate/up projection + SiLU*up over the active
//                 experts: GEMV tiles (full K, VALU dot2) for experts with few
//                 tokens -- the "small-matrix" form the article uses at batch
//                 1-2 -- and split-K MFMA tiles for experts with many tokens
//                 -- the "split-K" form it uses at larger batches (Part 1
//                 section 1); the same kernel serves the shared expert;
//   down_combine  down projection of every active expert and the shared
//                 expert, routing-weighted sum, residual add and bf16 output;
//                 output-stationary, so no atomics and a fixed summation order.
//
// Small-batch decode is bound by how fast weights stream from HBM (article
// Part 1 section 4): each tile streams its weight rows once with 16-byte
// loads and keeps fp32 accumulators.  Cross-workgroup hand-offs use a release
// fence + counter on the writer side and an acquire fence on the reader side;
// activations, partials and h are only read after the acquire, and only
// static weights may be loaded earlier (article Part 2 section 3 reports the
// compiler hoisting activation loads above a wait as a real bug).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_args.h"

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// acc + sum_{i<8} a_i * b_i over two vectors of 8 bf16 (v_dot2_f32_bf16).
// The dword lanes are copied to scalars before the bit cast: hipcc 7.2 lowers
// __builtin_bit_cast of an ext-vector member access (v.y) as element 0.
__device__ __forceinline__ float dot8(u32x4 a, u32x4 b, float acc) {
    const uint32_t a0 = a[0], a1 = a[1], a2 = a[2], a3 = a[3];
    const uint32_t b0 = b[0], b1 = b[1], b2 = b[2], b3 = b[3];
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a0), as_bf16x2(b0), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a1), as_bf16x2(b1), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a2), as_bf16x2(b2), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a3), as_bf16x2(b3), acc, false);
    return acc;
}

// acc + sum_{i<8} w_i * h_i, w bf16, h fp32.
__device__ __forceinline__ float dot8_f32(u32x4 w, const float4 h0, const float4 h1, float acc) {
    const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3];
    acc = fmaf(bf16_lo(w0), h0.x, acc);
    acc = fmaf(bf16_hi(w0), h0.y, acc);
    acc = fmaf(bf16_lo(w1), h0.z, acc);
    acc = fmaf(bf16_hi(w1), h0.w, acc);
    acc = fmaf(bf16_lo(w2), h1.x, acc);
    acc = fmaf(bf16_hi(w2), h1.y, acc);
    acc = fmaf(bf16_lo(w3), h1.z, acc);
    acc = fmaf(bf16_hi(w3), h1.w, acc);
    return acc;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Sum over aligned groups of G lanes (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Ordered 64-bit key: larger key = larger logit, then lower expert id.
__device__ __forceinline__ uint64_t topk_key(float v, int e) {
    uint32_t b = __float_as_uint(v + 0.0f);  // -0 -> +0
    uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)ord << 32) | (uint32_t)(0xffffffffu - (uint32_t)e);
}
__device__ __forceinline__ float key_value(uint64_t key) {
    uint32_t ord = (uint32_t)(key >> 32);
    uint32_t b = (ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord;
    return __uint_as_float(b);
}
__device__ __forceinline__ int key_expert(uint64_t key) {
    return (int)(0xffffffffu - (uint32_t)key);
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
    return ((uint64_t)hi << 32) | lo;
}

// ---------------------------------------------------------------------------
// router_topk
// ---------------------------------------------------------------------------

// Top-k of one token's logits by one wave: k rounds of a wave-wide argmax
// over (logit, -index) keys; lane l holds experts l, l+64, ...
__device__ void topk_one_token(const RouterArgs& a, int t, int lane, int32_t* s_pair_e) {
    const int E = a.E, k = a.k;
    const float* zt = a.z + (size_t)t * E;
    uint64_t key[kMaxExperts / 64];
    float zl[kMaxExperts / 64];
#pragma unroll
    for (int j = 0; j < kMaxExperts / 64; ++j) {
        const int e = lane + 64 * j;
        zl[j] = (e < E) ? zt[e] : 0.0f;
        key[j] = (e < E) ? topk_key(zl[j], e) : 0ull;
    }
    int sel_e[kMaxTopK];
    float sel_z[kMaxTopK];
#pragma unroll
    for (int r = 0; r < kMaxTopK; ++r) {
        if (r < k) {
            uint64_t best = 0;
#pragma unroll
            for (int j = 0; j < kMaxExperts / 64; ++j) best = key[j] > best ? key[j] : best;
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) {
                uint64_t o = shfl_xor_u64(best, m);
                best = o > best ? o : best;
            }
            const int ew = key_expert(best);
            sel_e[r] = ew;
            sel_z[r] = key_value(best);
            if ((ew & 63) == lane) {
#pragma unroll
                for (int j = 0; j < kMaxExperts / 64; ++j)
                    if (j == (ew >> 6)) key[j] = 0ull;
            }
        } else {
            sel_e[r] = 0;
            sel_z[r] = 0.0f;
        }
    }
    // routing weights (every lane computes the same values)
    float w[kMaxTopK];
    const float m = sel_z[0];
    if (a.score_fn == 0) {
        float den = 0.0f;
        if (a.renormalize) {
#pragma unroll
            for (int r = 0; r < kMaxTopK; ++r)
                if (r < k) den += expf(sel_z[r] - m);
        } else {
            float part = 0.0f;
#pragma unroll
            for (int j = 0; j < kMaxExperts / 64; ++j)
                if (lane + 64 * j < E) part += expf(zl[j] - m);
            den = wave_sum(part);
        }
#pragma unroll
        for (int r = 0; r < kMaxTopK; ++r) w[r] = expf(sel_z[r] - m) / den;
    } else {
        float den = 0.0f;
#pragma unroll
        for (int r = 0; r < kMaxTopK; ++r) {
            w[r] = 1.0f / (1.0f + expf(-sel_z[r]));
            if (r < k) den += w[r];
        }
        if (a.renormalize) {
#pragma unroll
            for (int r = 0; r < kMaxTopK; ++r) w[r] = w[r] / den;
        }
    }
#pragma unroll
    for (int r = 0; r < kMaxTopK; ++r) {
        if (r < k && lane == r) {
            a.topk_idx[t * k + r] = sel_e[r];
            a.topk_w[t * k + r] = w[r] * a.routed_scale;
            s_pair_e[t * k + r] = sel_e[r];
        }
    }
}

// Exclusive scan over the 256 threads of the block of two counters at once.
__device__ void block_scan2(int v0, int v1, int* s_tmp, int& ex0, int& ex1, int& tot0, int& tot1) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int i0 = v0, i1 = v1;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int o0 = __shfl_up(i0, d, 64), o1 = __shfl_up(i1, d, 64);
        if (lane >= d) { i0 += o0; i1 += o1; }
    }
    if (lane == 63) { s_tmp[wave] = i0; s_tmp[4 + wave] = i1; }
    __syncthreads();
    int p0 = 0, p1 = 0;
    for (int w = 0; w < wave; ++w) { p0 += s_tmp[w]; p1 += s_tmp[4 + w]; }
    tot0 = s_tmp[0] + s_tmp[1] + s_tmp[2] + s_tmp[3];
    tot1 = s_tmp[4] + s_tmp[5] + s_tmp[6] + s_tmp[7];
    ex0 = p0 + i0 - v0;
    ex1 = p1 + i1 - v1;
    __syncthreads();
}

template <int TB>
__global__ __launch_bounds__(256) void router_topk_kernel(RouterArgs a) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H, E = a.E, B = a.B, k = a.k;
    const int units = H >> 3;

    // 1. router GEMV: one wave per expert row, all tokens
    const int e = blockIdx.x * 4 + wave;
    if (e < E) {
        float acc[TB];
#pragma unroll
        for (int t = 0; t < TB; ++t) acc[t] = 0.0f;
        const uint16_t* wrow = a.wr + (size_t)e * H;
#pragma unroll 2
        for (int u = lane; u < units; u += 64) {
            const u32x4 w = ld16(wrow + u * 8);
#pragma unroll
            for (int t = 0; t < TB; ++t)
                if (t < B) acc[t] = dot8(w, ld16(a.x + (size_t)t * H + u * 8), acc[t]);
        }
        const float b = a.bias ? a.bias[e] : 0.0f;
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            if (t < B) {
                const float s = wave_sum(acc[t]);
                if (lane == 0) a.z[(size_t)t * E + e] = s + b;
            }
        }
    }

    // 2. the last workgroup to arrive owns the selection
    __shared__ int s_last;
    __threadfence();  // release this workgroup's logits
    __syncthreads();
    if (tid == 0) {
        const unsigned ticket = atomicAdd(reinterpret_cast<unsigned*>(&a.meta[M_ROUTER_CNT]), 1u);
        s_last = (ticket == gridDim.x - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();  // acquire every workgroup's logits

    __shared__ int32_t s_pair_e[kMaxBatch * kMaxTopK];
    __shared__ int32_t s_rank[kMaxBatch * kMaxTopK];
    __shared__ int32_t s_cnt[kMaxExperts];
    __shared__ int32_t s_tmp[8];
    __shared__ int32_t s_nmfma;

    for (int t = wave; t < B; t += 4) topk_one_token(a, t, lane, s_pair_e);
    for (int i = tid; i < E; i += 256) s_cnt[i] = 0;
    if (tid == 0) s_nmfma = 0;
    __syncthreads();

    // 3. bucketing: histogram with a rank per pair, scan, scatter
    const int npairs = B * k;
    for (int p = tid; p < npairs; p += 256) s_rank[p] = atomicAdd(&s_cnt[s_pair_e[p]], 1);
    __syncthreads();

    constexpr int CH = kMaxExperts / 256;  // bins per thread
    int cnt[CH], csum = 0, fsum = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int bin = tid * CH + c;
        cnt[c] = (bin < E) ? s_cnt[bin] : 0;
        csum += cnt[c];
        fsum += cnt[c] > 0 ? 1 : 0;
    }
    int cex, fex, ctot, ftot;
    block_scan2(csum, fsum, s_tmp, cex, fex, ctot, ftot);
    int nm = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int bin = tid * CH + c;
        if (bin < E) {
            s_cnt[bin] = cex;  // becomes the bucket offset
            if (cnt[c] > 0) {
                a.act_e[fex] = bin;
                a.act_off[fex] = cex;
                if (a.mfma_min_tokens > 0 && cnt[c] >= a.mfma_min_tokens) ++nm;
                ++fex;
            }
            cex += cnt[c];
        }
    }
    if (nm) atomicAdd(&s_nmfma, nm);
    __syncthreads();
    for (int p = tid; p < npairs; p += 256) a.perm[s_cnt[s_pair_e[p]] + s_rank[p]] = p;
    if (tid == 0) {
        a.act_off[ftot] = ctot;
        a.meta[M_NACT] = ftot;
        a.meta[M_MFMA_TILES] = s_nmfma * a.mfma_tiles_per_expert;
        a.meta[M_GEMV_TILES] = (ftot - s_nmfma) * a.tiles_per_expert;
        if (ctot != npairs) atomicOr(&a.meta[M_ERR], ERR_BUCKET);
        a.meta[M_ROUTER_CNT] = 0;  // re-armed for the next launch
    }
}

// ---------------------------------------------------------------------------
// gateup
// ---------------------------------------------------------------------------

// Full-K GEMV tile: wave w computes row pair i = 4*local + w (gate row i and
// up row n+i) for the entry's T <= TB tokens.
template <int TB>
__device__ void gemv_gateup_tile(const GateUpArgs& a, const uint16_t* W, int off, int T, int local) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int H = a.H, n = a.n, units = H >> 3;
    const int i = local * kPairsPerGemvTile + wave;
    if (i >= n) return;
    int tok[TB];
#pragma unroll
    for (int j = 0; j < TB; ++j) tok[j] = (j < T) ? a.perm[off + j] / a.pair_div : 0;
    const uint16_t* g = W + (size_t)i * H;
    const uint16_t* u = W + (size_t)(n + i) * H;
    float ag[TB], au[TB];
#pragma unroll
    for (int j = 0; j < TB; ++j) { ag[j] = 0.0f; au[j] = 0.0f; }
#pragma unroll 4
    for (int q = lane; q < units; q += 64) {
        const u32x4 wg = ld16(g + q * 8);
        const u32x4 wu = ld16(u + q * 8);
#pragma unroll
        for (int j = 0; j < TB; ++j) {
            if (j < T) {
                const u32x4 xv = ld16(a.x + (size_t)tok[j] * H + q * 8);
                ag[j] = dot8(wg, xv, ag[j]);
                au[j] = dot8(wu, xv, au[j]);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < TB; ++j) {
        if (j < T) {
            const float gs = wave_sum(ag[j]);
            const float us = wave_sum(au[j]);
            if (lane == 0) a.h[(size_t)(off + j) * n + i] = silu_f(gs) * us;
        }
    }
}

// Split-K MFMA tile: 64 row pairs (16 per wave) x one K slice x T <= 64 tokens.
// A = weight rows (16 x 32), B = x^T (32 x 16 tokens); fp32 partials are
// added to g_acc; the last of the `ksplit` tiles of the row block applies
// SiLU*up, writes h and clears g_acc and its counter.
__device__ void mfma_gateup_tile(const GateUpArgs& a, const uint16_t* W, int entry, int off, int T,
                                 int local) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H, n = a.n;
    const int nrb = n / kPairsPerMfmaTile;
    const int rb = local / a.ksplit, ks = local % a.ksplit;
    if (rb >= nrb) return;
    const int i0 = rb * kPairsPerMfmaTile + wave * 16;
    const int kbeg = ks * a.kslice;
    const int kend = min(H, kbeg + a.kslice);
    const int tl = lane & 15, kq = lane >> 4;
    const int NT = (T + 15) >> 4;

    const uint16_t* xrow[4];
    bool xok[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int j = tt * 16 + tl;
        xok[tt] = j < T;
        xrow[tt] = a.x + (size_t)(xok[tt] ? a.perm[off + j] / a.pair_div : 0) * H + 8 * kq;
    }
    const uint16_t* gr = W + (size_t)(i0 + tl) * H + 8 * kq;
    const uint16_t* ur = W + (size_t)(n + i0 + tl) * H + 8 * kq;
    f32x4 cg[4], cu[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) { cg[tt] = f32x4{0, 0, 0, 0}; cu[tt] = f32x4{0, 0, 0, 0}; }
    const u32x4 zero = u32x4{0, 0, 0, 0};
    for (int k0 = kbeg; k0 < kend; k0 += 32) {
        const bf16x8 Ag = __builtin_bit_cast(bf16x8, ld16(gr + k0));
        const bf16x8 Au = __builtin_bit_cast(bf16x8, ld16(ur + k0));
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            if (tt < NT) {
                const bf16x8 Bx = __builtin_bit_cast(bf16x8, xok[tt] ? ld16(xrow[tt] + k0) : zero);
                cg[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ag, Bx, cg[tt], 0, 0, 0);
                cu[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Au, Bx, cu[tt], 0, 0, 0);
            }
        }
    }
    // D layout: lane holds rows 4*(lane/16)+r, column (token) lane%16
    const int n2 = 2 * n;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int j = tt * 16 + tl;
        if (tt < NT && j < T) {
            float* gp = a.g_acc + (size_t)(off + j) * n2 + i0 + 4 * kq;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                atomicAdd(gp + r, cg[tt][r]);
                atomicAdd(gp + n + r, cu[tt][r]);
            }
        }
    }
    __shared__ int s_last;
    __threadfence();  // release the partials
    __syncthreads();
    if (tid == 0) {
        const unsigned old = atomicAdd(&a.tile_cnt[entry * nrb + rb], 1u);
        s_last = (old == (unsigned)a.ksplit - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();  // acquire the other splits' partials
    const int rows = kPairsPerMfmaTile;
    for (int idx = tid; idx < rows * T; idx += 256) {
        const int j = idx / rows, i = rb * rows + idx % rows;
        float* gp = a.g_acc + (size_t)(off + j) * n2;
        const float g = gp[i], u = gp[n + i];
        a.h[(size_t)(off + j) * n + i] = silu_f(g) * u;
        gp[i] = 0.0f;
        gp[n + i] = 0.0f;
    }
    if (tid == 0) a.tile_cnt[entry * nrb + rb] = 0u;
}

template <int TB, bool WITH_MFMA>
__global__ __launch_bounds__(256) void gateup_kernel(GateUpArgs a) {
    const int entry = blockIdx.x / a.tiles_per_expert;
    const int local = blockIdx.x % a.tiles_per_expert;
    if (entry >= *a.n_act) return;
    const int e = a.act_e[entry];
    const int off = a.act_off[entry];
    const int T = a.act_off[entry + 1] - off;
    const uint16_t* W = a.w + (size_t)e * (size_t)a.expert_stride;
    if (WITH_MFMA && a.mfma_min_tokens > 0 && T >= a.mfma_min_tokens) {
        if (T > kMaxBatch) {
            if (threadIdx.x == 0 && local == 0) atomicOr(&a.meta[M_ERR], ERR_TILE);
            return;
        }
        mfma_gateup_tile(a, W, entry, off, T, local);
    } else {
        if (T > TB) {
            if (threadIdx.x == 0 && local == 0) atomicOr(&a.meta[M_ERR], ERR_TILE);
            return;
        }
        gemv_gateup_tile<TB>(a, W, off, T, local);
    }
}

// ---------------------------------------------------------------------------
// down_combine
// ---------------------------------------------------------------------------

// LPR lanes share one W2 row (LPR = min(I/8, 64)); each lane loads NQ 16-byte
// units per row; a wave covers 64/LPR rows per pass and RP passes; the
// workgroup covers R = RP * 4 * (64/LPR) consecutive output rows.
template <int LPR, int NQ, int RP>
struct DownShape {
    static constexpr int RW = 64 / LPR;
    static constexpr int R = RP * 4 * RW;
};

template <int LPR, int NQ, int RP>
__device__ __forceinline__ void down_load(const uint16_t* w, int ld, int row0, int wave, int lane,
                                          u32x4 (&wv)[RP][NQ]) {
    constexpr int RW = 64 / LPR;
    const int rw = lane / LPR, c = lane % LPR;
#pragma unroll
    for (int rp = 0; rp < RP; ++rp) {
        const int r = row0 + (rp * 4 + wave) * RW + rw;
#pragma unroll
        for (int q = 0; q < NQ; ++q) wv[rp][q] = ld16(w + (size_t)r * ld + 8 * (c + LPR * q));
    }
}

template <int LPR, int NQ, int RP>
__device__ __forceinline__ void down_accum(const u32x4 (&wv)[RP][NQ], const float* hrow, float wt,
                                           int t, int wave, int lane, float* s_acc) {
    constexpr int RW = 64 / LPR;
    constexpr int R = DownShape<LPR, NQ, RP>::R;
    const int rw = lane / LPR, c = lane % LPR;
    float4 h0[NQ], h1[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const float4* hp = reinterpret_cast<const float4*>(hrow + 8 * (c + LPR * q));
        h0[q] = hp[0];
        h1[q] = hp[1];
    }
#pragma unroll
    for (int rp = 0; rp < RP; ++rp) {
        float p = 0.0f;
#pragma unroll
        for (int q = 0; q < NQ; ++q) p = dot8_f32(wv[rp][q], h0[q], h1[q], p);
        p = group_sum<LPR>(p);
        if (c == 0) s_acc[t * R + (rp * 4 + wave) * RW + rw] += wt * p;
    }
}

template <int LPR, int NQ, int RP>
__global__ __launch_bounds__(256) void down_combine_kernel(DownArgs a) {
    constexpr int RW = 64 / LPR;
    constexpr int R = DownShape<LPR, NQ, RP>::R;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H, I = a.I, B = a.B, k = a.k;
    const int row0 = blockIdx.x * R;
    const int rw = lane / LPR, c = lane % LPR;
    __shared__ float s_acc[kMaxBatch * R];
    for (int i = tid; i < B * R; i += 256) s_acc[i] = 0.0f;
    __syncthreads();

    const int nact = *a.n_act;
    const size_t estride = (size_t)H * I;
    u32x4 wv[RP][NQ], wn[RP][NQ];
    if (nact > 0) down_load<LPR, NQ, RP>(a.w2 + (size_t)a.act_e[0] * estride, I, row0, wave, lane, wv);
    for (int ent = 0; ent < nact; ++ent) {
        // weights are static: the next expert's rows are requested before this one is used
        if (ent + 1 < nact)
            down_load<LPR, NQ, RP>(a.w2 + (size_t)a.act_e[ent + 1] * estride, I, row0, wave, lane, wn);
        const int off = a.act_off[ent], T = a.act_off[ent + 1] - off;
        for (int j = 0; j < T; ++j) {
            const int p = a.perm[off + j];
            down_accum<LPR, NQ, RP>(wv, a.h + (size_t)(off + j) * I, a.topk_w[p], p / k, wave, lane, s_acc);
        }
#pragma unroll
        for (int rp = 0; rp < RP; ++rp)
#pragma unroll
            for (int q = 0; q < NQ; ++q) wv[rp][q] = wn[rp][q];
    }
    // shared expert: Is/I column blocks of S2 (row stride Is), weight 1, all tokens
    if (a.s2) {
        for (int v = 0; v < a.Is / I; ++v) {
            down_load<LPR, NQ, RP>(a.s2 + (size_t)v * I, a.Is, row0, wave, lane, wv);
            for (int t = 0; t < B; ++t)
                down_accum<LPR, NQ, RP>(wv, a.hs + (size_t)t * a.Is + (size_t)v * I, 1.0f, t, wave, lane, s_acc);
        }
    }
    // the lane that accumulated (t, row) also writes it: no barrier needed
    if (c == 0) {
#pragma unroll
        for (int rp = 0; rp < RP; ++rp) {
            const int rl = (rp * 4 + wave) * RW + rw;
            const int r = row0 + rl;
            for (int t = 0; t < B; ++t) {
                float v = s_acc[t * R + rl];
                if (a.add_residual) v += __uint_as_float((uint32_t)a.x[(size_t)t * H + r] << 16);
                a.out[(size_t)t * H + r] = f32_to_bf16_rne(v);
            }
        }
    }
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

KernelPick pick_init(const InitArgs& a) {
    return {reinterpret_cast<const void*>(&init_lists_kernel), dim3((a.B + 63) / 64), dim3(64)};
}

KernelPick pick_router(const RouterArgs& a) {
    const dim3 grid((a.E + 3) / 4), block(256);
    const void* f;
    switch (tb_bucket(a.B)) {
        case 1: f = reinterpret_cast<const void*>(&router_topk_kernel<1>); break;
        case 2: f = reinterpret_cast<const void*>(&router_topk_kernel<2>); break;
        case 4: f = reinterpret_cast<const void*>(&router_topk_kernel<4>); break;
        case 8: f = reinterpret_cast<const void*>(&router_topk_kernel<8>); break;
        case 16: f = reinterpret_cast<const void*>(&router_topk_kernel<16>); break;
        case 32: f = reinterpret_cast<const void*>(&router_topk_kernel<32>); break;
        default: f = reinterpret_cast<const void*>(&router_topk_kernel<64>); break;
    }
    return {f, grid, block};
}

// gemv_tokens: the largest token count a GEMV tile of this list may see.
KernelPick pick_gateup(const GateUpArgs& a, int max_entries, int gemv_tokens) {
    const dim3 grid(max_entries * a.tiles_per_expert), block(256);
    const bool mf = a.mfma_min_tokens > 0;
    const void* f;
#define MOE_GU(TB)                                                                              \
    f = mf ? reinterpret_cast<const void*>(&gateup_kernel<TB, true>)                          \
           : reinterpret_cast<const void*>(&gateup_kernel<TB, false>);
    switch (tb_bucket(gemv_tokens)) {
        case 1: MOE_GU(1) break;
        case 2: MOE_GU(2) break;
        case 4: MOE_GU(4) break;
        case 8: MOE_GU(8) break;
        case 16: MOE_GU(16) break;
        case 32: MOE_GU(32) break;
        default: MOE_GU(64) break;
    }
#undef MOE_GU
    return {f, grid, block};
}

// Output rows per down_combine workgroup for intermediate size I (matches pick_down).
int down_rows_per_block(int I) {
    const int ur = I / 8;
    if (ur == 8) return DownShape<8, 1, 1>::R;
    if (ur == 16) return DownShape<16, 1, 1>::R;
    if (ur == 32) return DownShape<32, 1, 2>::R;
    return ur / 64 <= 4 ? DownShape<64, 1, 2>::R : DownShape<64, 5, 1>::R;
}

KernelPick pick_down(const DownArgs& a) {
    const int ur = a.I / 8;
    const void* f;
#define MOE_DN(LPR, NQ, RP) f = reinterpret_cast<const void*>(&down_combine_kernel<LPR, NQ, RP>);
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
    return {f, dim3(a.H / down_rows_per_block(a.I)), dim3(256)};
}

}  // namespace moe
