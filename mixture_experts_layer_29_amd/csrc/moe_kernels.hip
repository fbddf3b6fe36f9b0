// moe_kernels.hip -- gfx950 (CDNA4) kernels of the decode-time MoE layer.
//
// One layer is, on the main stream:
//   router     batch <= 4: router_small -- router GEMV, then the last workgroup
//              to arrive selects the top-k experts of every token, computes the
//              routing weights and buckets the (token, slot) pairs by expert
//              with an LDS histogram;
//              batch > 4: router_mfma -- split-K MFMA router GEMM accumulating
//              fp32 logits -- then topk_bucket -- one wave per token selects
//              the top-k, the last workgroup buckets;
//   gateup     grouped gate/up projection + SiLU*up over the active experts:
//              GEMV tiles (full K, VALU dot2) for experts with few tokens -- the
//              "small-matrix" form the Kimi K3 decode article uses at batch 1-2
//              -- and split-K MFMA tiles for experts with many tokens -- the
//              "split-K" form it uses at larger batches (Part 1 section 1);
//   down       down projection of every active expert and of the shared
//              expert, routing-weighted sum, residual add, bf16 output;
//              output-stationary, so no atomics and a fixed summation order;
// and on a second stream the shared expert's gate/up (same gateup kernel with
// a one-entry work list), joined before `down` (article Part 1 section 3: the
// shared expert runs on its own stream, overlapped with routing).
//
// Small-batch decode is bound by how fast weights stream from HBM (article
// Part 1 section 4).  Every weight-streaming loop therefore issues all of a
// wave's 16-byte weight loads for a batch of units before it consumes the
// first one, so a wave keeps up to 16 KiB in flight instead of waiting a
// memory round trip per unit.  Cross-workgroup hand-offs use a release fence +
// counter on the writer side and an acquire fence on the reader side;
// activations, partials and h are only read after the acquire, and only static
// weights are loaded before it (article Part 2 section 3 reports a compiler
// hoisting activation loads above a wait as a real bug).
#include <hip/hip_runtime.h>
#include <math.h>
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
__device__ __forceinline__ void st16(uint16_t* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

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

// Wave-wide reductions through DPP (quad permutes, row mirrors, row
// broadcasts 15/31); the result is read from lane 63 and is wave-uniform.
// Lanes outside a step's row mask receive `old`: 0 for sums, v for max/min.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xf, false);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i(int v) {
    return dpp_i<CTRL, ROW_MASK>(v, v);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, dpp_i<CTRL, ROW_MASK>(__builtin_bit_cast(int, v)));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f0(float v) {  // masked-off lanes read 0
    return __builtin_bit_cast(float, dpp_i<CTRL, ROW_MASK>(0, __builtin_bit_cast(int, v)));
}

// Sum over aligned groups of G lanes (G a power of two <= 64).  For G <= 16
// every lane of a group gets the sum; for G = 32 and 64 the lanes of the
// group's highest 16-lane row do (so lane G-1 of the group always has it).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (G >= 2) v += dpp_f0<0xb1, 0xf>(v);   // quad_perm [1,0,3,2]
    if constexpr (G >= 4) v += dpp_f0<0x4e, 0xf>(v);   // quad_perm [2,3,0,1]
    if constexpr (G >= 8) v += dpp_f0<0x141, 0xf>(v);  // row_half_mirror
    if constexpr (G >= 16) v += dpp_f0<0x140, 0xf>(v); // row_mirror
    if constexpr (G >= 32) v += dpp_f0<0x142, 0xa>(v); // row_bcast15 into rows 1, 3
    if constexpr (G >= 64) v += dpp_f0<0x143, 0xc>(v); // row_bcast31 into rows 2, 3
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f<0xb1, 0xf>(v));   // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp_f<0x4e, 0xf>(v));   // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp_f<0x141, 0xf>(v));  // row_half_mirror
    v = fmaxf(v, dpp_f<0x140, 0xf>(v));  // row_mirror
    v = fmaxf(v, dpp_f<0x142, 0xa>(v));  // row_bcast15
    v = fmaxf(v, dpp_f<0x143, 0xc>(v));  // row_bcast31
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ float wave_sum(float v) {
    v = group_sum<64>(v);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ int wave_min_int(int v) {
    v = min(v, dpp_i<0xb1, 0xf>(v));
    v = min(v, dpp_i<0x4e, 0xf>(v));
    v = min(v, dpp_i<0x141, 0xf>(v));
    v = min(v, dpp_i<0x140, 0xf>(v));
    v = min(v, dpp_i<0x142, 0xa>(v));
    v = min(v, dpp_i<0x143, 0xc>(v));
    return __builtin_amdgcn_readlane(v, 63);
}

// Publishes this workgroup's earlier global stores device-wide and counts its
// arrival; returns true (after an acquire) in the last of `total` workgroups
// to arrive.  One wave releases: the L2 write-back covers every wave's stores
// once they have completed, which the waitcnt + barrier ensure.
__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned total, int* s_flag) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const unsigned t = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = t == total - 1;
        if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        *s_flag = last;
    }
    __syncthreads();
    return *s_flag != 0;
}


__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// top-k selection, routing weights, bucketing
// ---------------------------------------------------------------------------

constexpr int kSlots = kMaxExperts / 64;  // logits held per lane
constexpr int kNone = 0x7fffffff;

// Top-k of one token by one wave.  Slot m of lane l holds the logit of expert
// (slot0 + m * step) * 64 + l in v[m] (slots past E hold -inf and are never
// selected).  Each round takes the wave-wide largest remaining logit (DPP
// max); equal logits go to the lower expert id (ballot, then DPP min when
// several lanes tie).  Fills sel_e / sel_z in rank order (wave-uniform);
// rounds that find nothing left give sel_e = -1.
template <int NS>
__device__ __forceinline__ void topk_wave(const float (&v)[NS], int slot0, int step, int E, int k, int lane,
                                          int (&sel_e)[kMaxTopK], float (&sel_z)[kMaxTopK]) {
    uint32_t avail = 0;
#pragma unroll
    for (int m = 0; m < NS; ++m)
        if ((slot0 + m * step) * 64 + lane < E) avail |= 1u << m;
    float bv = -INFINITY;
    int be = kNone;
    auto lane_best = [&]() {
        bv = -INFINITY;
        be = kNone;
#pragma unroll
        for (int m = 0; m < NS; ++m)
            if (((avail >> m) & 1u) && v[m] > bv) { bv = v[m]; be = (slot0 + m * step) * 64 + lane; }
    };
    lane_best();
#pragma unroll
    for (int r = 0; r < kMaxTopK; ++r) {
        sel_e[r] = -1;
        sel_z[r] = -INFINITY;
        if (r < k) {
            const float m = wave_max(bv);
            const unsigned long long bal = __ballot(be != kNone && bv == m);
            if (bal) {
                int e;
                if (__popcll(bal) == 1) e = __builtin_amdgcn_readlane(be, __ffsll(bal) - 1);
                else e = wave_min_int(((bal >> lane) & 1ull) ? be : kNone);
                sel_e[r] = e;
                sel_z[r] = m;
                if (lane == (e & 63)) {
#pragma unroll
                    for (int q = 0; q < NS; ++q)
                        if ((slot0 + q * step) * 64 + lane == e) avail &= ~(1u << q);
                    lane_best();
                }
            }
        }
    }
}

// Merges per-wave candidate lists (up to 64 (logit, expert) pairs, one per
// lane; invalid lanes hold e = kNone) into the top-k, same order and ties.
__device__ __forceinline__ void topk_merge(float cv, int ce, int k, int lane, int (&sel_e)[kMaxTopK],
                                           float (&sel_z)[kMaxTopK]) {
#pragma unroll
    for (int r = 0; r < kMaxTopK; ++r) {
        sel_e[r] = -1;
        sel_z[r] = -INFINITY;
        if (r < k) {
            const float m = wave_max(cv);
            const unsigned long long bal = __ballot(ce != kNone && cv == m);
            if (bal) {
                int e;
                if (__popcll(bal) == 1) e = __builtin_amdgcn_readlane(ce, __ffsll(bal) - 1);
                else e = wave_min_int(((bal >> lane) & 1ull) ? ce : kNone);
                sel_e[r] = e;
                sel_z[r] = m;
                if (ce == e) { cv = -INFINITY; ce = kNone; }
            }
        }
    }
}

// Routing weights of the selected logits (softmax or sigmoid, optional
// renormalisation over the selection, times routed_scale); lane r < k
// computes and writes entry r of the token's topk_idx / topk_w row (and of
// s_pair_e when given).  zrow (the token's logits, readable by this wave) is
// read only for a softmax without renormalisation, whose denominator runs
// over all E experts.
__device__ __forceinline__ void route_token(const RouterArgs& a, int t, int lane, const float* zrow,
                                            const int (&sel_e)[kMaxTopK], const float (&sel_z)[kMaxTopK],
                                            int32_t* s_pair_e) {
    const int k = a.k, E = a.E;
    float zr = -INFINITY;
    int er = -1;
#pragma unroll
    for (int r = 0; r < kMaxTopK; ++r)
        if (lane == r) { zr = sel_z[r]; er = sel_e[r]; }
    const bool mine = lane < k;
    const float m = sel_z[0];
    float w;
    if (a.score_fn == 0) {
        const float ex = mine ? expf(zr - m) : 0.0f;
        float den;
        if (a.renormalize) {
            den = wave_sum(ex);
        } else {
            float part = 0.0f;
            for (int e = lane; e < E; e += 64) part += expf(zrow[e] - m);
            den = wave_sum(part);
        }
        w = ex / den;
    } else {
        const float sg = mine ? 1.0f / (1.0f + expf(-zr)) : 0.0f;
        w = a.renormalize ? sg / wave_sum(sg) : sg;
    }
    if (mine) {
        a.topk_idx[t * k + lane] = er;
        a.topk_w[t * k + lane] = w * a.routed_scale;
        if (s_pair_e) s_pair_e[t * k + lane] = er;
    }
}

// Writes the bucketing results common to both bucketing forms.
__device__ __forceinline__ void bucket_meta(const RouterArgs& a, int nact, int nmfma, int npairs, int placed) {
    if (placed != npairs) nact = nmfma = 0;  // invalid selection: no expert work at all
    a.act_off[nact] = npairs;
    a.meta[M_NACT] = nact;
    a.meta[M_MFMA_TILES] = nmfma * a.mfma_tiles_per_expert;
    a.meta[M_GEMV_TILES] = (nact - nmfma) * a.tiles_per_expert;
    if (placed != npairs) atomicOr(&a.meta[M_ERR], ERR_BUCKET);
    a.meta[M_ROUTER_CNT] = 0;  // re-armed for the next launch
}

// Bucketing by one wave for B*k <= 64 pairs (pair p in lane p): a pair's slot
// is the number of pairs with a smaller (expert, pair) key, so slots are
// ordered by expert then token; the first pair of each expert defines the
// active-expert entry.  No barriers and no LDS atomics.
__device__ __forceinline__ void bucket_wave(const RouterArgs& a, const int32_t* s_pair_e, int lane) {
    const int np = a.B * a.k;
    const int e = lane < np ? s_pair_e[lane] : kNone;
    if (__ballot(lane < np && (e < 0 || e >= a.E))) {  // never hand an invalid id to the experts
        if (lane == 0) bucket_meta(a, 0, 0, np, -1);
        return;
    }
    int pos = 0, cnt = 0;
    bool first = true;
    for (int q = 0; q < np; ++q) {
        const int eq = __builtin_amdgcn_readlane(e, q);
        pos += (eq < e || (eq == e && q < lane)) ? 1 : 0;
        cnt += eq == e ? 1 : 0;
        if (eq == e && q < lane) first = false;
    }
    if (lane < np) a.perm[pos] = lane;
    const bool lead = lane < np && first;
    const unsigned long long fm = __ballot(lead);
    int apos = 0;
    for (int q = 0; q < np; ++q) {
        const int eq = __builtin_amdgcn_readlane(e, q);
        apos += (((fm >> q) & 1ull) && eq < e) ? 1 : 0;
    }
    if (lead) {
        a.act_e[apos] = e;
        a.act_off[apos] = pos;
    }
    const int nact = __popcll(fm);
    const int nmfma = __popcll(__ballot(lead && a.mfma_min_tokens > 0 && cnt >= a.mfma_min_tokens));
    if (lane == 0) bucket_meta(a, nact, nmfma, np, np);
}

// Exclusive scan over the 256 threads of the block of two counters at once.
__device__ __forceinline__ void block_scan2(int v0, int v1, int* s_tmp, int& ex0, int& ex1, int& tot0, int& tot1) {
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

// Bucketing by a 256-thread workgroup for up to 1024 pairs: LDS histogram
// with a rank per pair, exclusive scan, scatter.  s_pair_e must hold the
// selected ids; the order of pairs inside a bucket is unspecified.
__device__ __forceinline__ void bucket_block(const RouterArgs& a, const int32_t* s_pair_e, int32_t* s_rank, int32_t* s_cnt,
                             int32_t* s_tmp, int32_t* s_nmfma) {
    const int tid = threadIdx.x, E = a.E;
    for (int i = tid; i < E; i += 256) s_cnt[i] = 0;
    if (tid == 0) *s_nmfma = 0;
    __syncthreads();
    const int npairs = a.B * a.k;
    for (int p = tid; p < npairs; p += 256) {
        const int e = s_pair_e[p];
        s_rank[p] = (e >= 0 && e < E) ? atomicAdd(&s_cnt[e], 1) : -1;
    }
    __syncthreads();
    // (an invalid id leaves ctot < npairs; bucket_meta then publishes an empty list)

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
    if (nm) atomicAdd(s_nmfma, nm);
    __syncthreads();
    for (int p = tid; p < npairs; p += 256)
        if (s_rank[p] >= 0) a.perm[s_cnt[s_pair_e[p]] + s_rank[p]] = p;
    if (tid == 0) bucket_meta(a, ftot, *s_nmfma, npairs, ctot);
}

// Selection for tokens t0 + wave of this workgroup.
// src: per-token logit rows (E floats); with `from_acc` they are split-K
// accumulators: the bias is added, the sum stored to a.z and the accumulator
// cleared.  A single token is ranked by all four waves (each over every
// fourth slot) and merged by wave 0.  Ends with a workgroup barrier, after
// which s_pair_e (if given) holds the selected ids of the workgroup's tokens.
template <int NS>
__device__ __forceinline__ void select_tokens(const RouterArgs& a, int t0, float* src, const float* bias,
                                              bool from_acc, int32_t* s_pair_e, int32_t* s_cand_e,
                                              float* s_cand_z, float* s_z) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = a.E, B = a.B, k = a.k;
    int sel_e[kMaxTopK];
    float sel_z[kMaxTopK];
    auto fetch = [&](float* row, float* zout, int e) {
        float v = row[e];
        if (from_acc) {
            v += bias ? bias[e] : 0.0f;
            zout[e] = v;
            row[e] = 0.0f;
        }
        return v;
    };
    if (B == 1) {
        constexpr int NQ = (NS + 3) / 4;
        float v[NQ];
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
            const int e = (wave + 4 * m) * 64 + lane;
            v[m] = (e < E) ? fetch(src, a.z, e) : -INFINITY;
            if (e < E) s_z[e] = v[m];
        }
        topk_wave<NQ>(v, wave, 4, E, k, lane, sel_e, sel_z);
        if (lane < k) {
            int ce = kNone;
            float cz = -INFINITY;
#pragma unroll
            for (int r = 0; r < kMaxTopK; ++r)
                if (lane == r) { ce = sel_e[r] >= 0 ? sel_e[r] : kNone; cz = sel_z[r]; }
            s_cand_e[wave * kMaxTopK + lane] = ce;
            s_cand_z[wave * kMaxTopK + lane] = cz;
        }
        __syncthreads();
        if (wave == 0) {
            const int r = lane % kMaxTopK;
            const bool ok = r < k;
            topk_merge(ok ? s_cand_z[lane] : -INFINITY, ok ? s_cand_e[lane] : kNone, k, lane, sel_e, sel_z);
            route_token(a, 0, lane, s_z, sel_e, sel_z, s_pair_e);
        }
    } else {
        const int t = t0 + wave;
        if (t < B) {
            float* row = src + (size_t)t * E;
            float* zo = a.z + (size_t)t * E;
            float v[NS];
#pragma unroll
            for (int m = 0; m < NS; ++m) {
                const int e = m * 64 + lane;
                v[m] = (e < E) ? fetch(row, zo, e) : -INFINITY;
            }
            topk_wave<NS>(v, 0, 1, E, k, lane, sel_e, sel_z);
            // a full softmax reads the token's logits back: from_acc rows are in a.z (this wave's stores)
            route_token(a, t, lane, from_acc ? zo : row, sel_e, sel_z, s_pair_e);
        }
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// front launch, batch <= 4: router GEMV + (last workgroup) top-k and bucketing,
// plus the shared expert's gate/up in trailing workgroups
// ---------------------------------------------------------------------------

template <int TB>
__device__ __forceinline__ void gemv_gateup_tile(const GateUpArgs& a, const uint16_t* W, int off, int T, int local,
                                 uint16_t* s_x);
__device__ __forceinline__ void mfma_gateup_tile(const GateUpArgs& a, const uint16_t* W, int entry, int off, int T, int local);

// SELECT: the last router workgroup to arrive selects and buckets; otherwise
// the router writes raw logits to zacc and topk_bucket_kernel follows.
template <int TB, bool SH_MFMA, bool SELECT, int NS>
__global__ __launch_bounds__(256) void front_small_kernel(FrontArgs f) {
    extern __shared__ __align__(16) uint16_t s_x[];  // [B][H] activations
    const RouterArgs& a = f.r;
    if ((int)blockIdx.x >= f.router_blocks) {  // shared expert: all B tokens, weight 1
        const int local = blockIdx.x - f.router_blocks;
        if constexpr (SH_MFMA) mfma_gateup_tile(f.s, f.s.w, 0, 0, a.B, local);
        else gemv_gateup_tile<TB>(f.s, f.s.w, 0, a.B, local, s_x);
        return;
    }
    __shared__ int32_t s_pair_e[4 * kMaxTopK];
    __shared__ int32_t s_cand_e[4 * kMaxTopK];
    __shared__ float s_cand_z[4 * kMaxTopK];
    __shared__ float s_z[kMaxExperts];
    __shared__ int s_flag;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H, E = a.E, B = a.B;
    const int units = H >> 3, nu = (units + 63) >> 6;
    const int e = blockIdx.x * 4 + wave;
    const bool row_ok = e < E;
    const uint16_t* wrow = a.wr + (size_t)(row_ok ? e : 0) * H;
    const u32x4 zero = u32x4{0, 0, 0, 0};

    float acc[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[t] = 0.0f;
    for (int base = 0; base < nu; base += kMaxGemvUnits) {
        u32x4 w[kMaxGemvUnits];
#pragma unroll
        for (int q = 0; q < kMaxGemvUnits; ++q) {
            const int u = (base + q) * 64 + lane;
            w[q] = (row_ok && u < units) ? ld16(wrow + u * 8) : zero;
        }
        if (base == 0) {  // stage x while the weight loads are in flight
            for (int i = tid; i < B * units; i += 256) {
                const int t = i / units, u = i - t * units;
                st16(s_x + t * H + u * 8, ld16(a.x + (size_t)t * H + u * 8));
            }
            __syncthreads();
        }
#pragma unroll
        for (int q = 0; q < kMaxGemvUnits; ++q) {
            const int u = (base + q) * 64 + lane;
            if (base + q < nu && u < units) {
#pragma unroll
                for (int t = 0; t < TB; ++t)
                    if (t < B) acc[t] = dot8(w[q], ld16(s_x + t * H + u * 8), acc[t]);
            }
        }
    }
    if (row_ok) {
        const float b = a.bias ? a.bias[e] : 0.0f;
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            if (t < B) {
                const float s = wave_sum(acc[t]);
                if (lane == 0) {
                    if constexpr (SELECT) a.z[(size_t)t * E + e] = s + b;
                    else a.zacc[(size_t)t * E + e] = s;
                }
            }
        }
    }
    if constexpr (!SELECT) return;

    // the last router workgroup to arrive selects and buckets
    if (!arrive_last(reinterpret_cast<unsigned*>(&a.meta[M_ROUTER_CNT]), f.router_blocks, &s_flag)) return;

    select_tokens<NS>(a, 0, a.z, nullptr, false, s_pair_e, s_cand_e, s_cand_z, s_z);
    __syncthreads();
    if (wave == 0) bucket_wave(a, s_pair_e, lane);
}

// ---------------------------------------------------------------------------
// front launch, batch > 4: split-K MFMA router GEMM into zacc, plus the
// shared expert's gate/up in trailing workgroups; then topk_bucket
// ---------------------------------------------------------------------------

// Tile: 64 router rows (16 per wave) x one K slice x all B tokens.
// A = router rows (16 x 32), B = x^T (32 x 16 tokens), fp32 atomics into zacc.
__device__ __forceinline__ void router_mfma_tile(const RouterArgs& a, int tile) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int H = a.H, E = a.E, B = a.B;
    const int r0 = (tile / a.ksplit) * kRouterRowsPerMfmaTile + wave * 16;
    const int tl = lane & 15, kq = lane >> 4;
    const int kbeg = (tile % a.ksplit) * a.kslice;
    const int nsteps = min(a.kslice, H - kbeg) >> 5;
    const int NT = (B + 15) >> 4;
    const bool rok = r0 + tl < E;
    const uint16_t* ar = a.wr + (size_t)(rok ? r0 + tl : 0) * H + kbeg + 8 * kq;
    const uint16_t* xr[4];
    bool xok[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int t = tt * 16 + tl;
        xok[tt] = t < B;
        xr[tt] = a.x + (size_t)(xok[tt] ? t : 0) * H + kbeg + 8 * kq;
    }
    const u32x4 zero = u32x4{0, 0, 0, 0};
    f32x4 c[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) c[tt] = f32x4{0, 0, 0, 0};
    for (int s = 0; s < nsteps; s += 4) {
        u32x4 A[4], X[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool sok = s + u < nsteps;
            A[u] = (sok && rok) ? ld16(ar + 32 * (s + u)) : zero;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
                X[u][tt] = (sok && tt < NT && xok[tt]) ? ld16(xr[tt] + 32 * (s + u)) : zero;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
                if (s + u < nsteps && tt < NT)
                    c[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[u]),
                                                                    __builtin_bit_cast(bf16x8, X[u][tt]),
                                                                    c[tt], 0, 0, 0);
    }
    // D layout: lane holds rows 4*(lane/16)+r, column (token) lane%16
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int t = tt * 16 + tl;
        if (tt < NT && t < B) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = r0 + 4 * kq + r;
                if (row < E) atomicAdd(&a.zacc[(size_t)t * E + row], c[tt][r]);
            }
        }
    }
}

template <int SHTB>  // 0: the shared expert runs on MFMA tiles, else its GEMV token bucket
__global__ __launch_bounds__(256) void front_mfma_kernel(FrontArgs f) {
    extern __shared__ __align__(16) uint16_t s_x[];
    if ((int)blockIdx.x >= f.router_blocks) {
        const int local = blockIdx.x - f.router_blocks;
        if constexpr (SHTB == 0) mfma_gateup_tile(f.s, f.s.w, 0, 0, f.r.B, local);
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
        for (int p = tid; p < np; p += 256) s_pair_e[p] = a.topk_idx[p];
        __syncthreads();
    }
    if (np <= 64) {
        if (wave == 0) bucket_wave(a, s_pair_e, lane);
    } else {
        bucket_block(a, s_pair_e, s_rank, s_cnt, s_tmp, &s_nmfma);
    }
}

// ---------------------------------------------------------------------------
// gateup
// ---------------------------------------------------------------------------

// Full-K GEMV tile: wave w computes row pair i = 4*local + w (gate row i and
// up row n+i) for the entry's T <= TB tokens, whose activations the workgroup
// stages in LDS after issuing its weight loads.
template <int TB>
__device__ __forceinline__ void gemv_gateup_tile(const GateUpArgs& a, const uint16_t* W, int off, int T, int local,
                                 uint16_t* s_x) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H, n = a.n, units = H >> 3, nu = (units + 63) >> 6;
    const int i = local * kPairsPerGemvTile + wave;
    const uint16_t* g = W + (size_t)i * H;
    const uint16_t* u = W + (size_t)(n + i) * H;
    const u32x4 zero = u32x4{0, 0, 0, 0};
    float ag[TB], au[TB];
#pragma unroll
    for (int j = 0; j < TB; ++j) { ag[j] = 0.0f; au[j] = 0.0f; }
    for (int base = 0; base < nu; base += kMaxGemvUnits) {
        u32x4 wg[kMaxGemvUnits], wu[kMaxGemvUnits];
#pragma unroll
        for (int q = 0; q < kMaxGemvUnits; ++q) {
            const int uu = (base + q) * 64 + lane;
            const bool ok = uu < units;
            wg[q] = ok ? ld16(g + uu * 8) : zero;
            wu[q] = ok ? ld16(u + uu * 8) : zero;
        }
        if (base == 0) {  // stage the tokens' activations while the weights stream in
            for (int idx = tid; idx < T * units; idx += 256) {
                const int j = idx / units, uu = idx - j * units;
                const int tok = a.perm[off + j] / a.pair_div;
                st16(s_x + j * H + uu * 8, ld16(a.x + (size_t)tok * H + uu * 8));
            }
            __syncthreads();
        }
#pragma unroll
        for (int q = 0; q < kMaxGemvUnits; ++q) {
            const int uu = (base + q) * 64 + lane;
            if (base + q < nu && uu < units) {
#pragma unroll
                for (int j = 0; j < TB; ++j) {
                    if (j < T) {
                        const u32x4 xv = ld16(s_x + j * H + uu * 8);
                        ag[j] = dot8(wg[q], xv, ag[j]);
                        au[j] = dot8(wu[q], xv, au[j]);
                    }
                }
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
__device__ __forceinline__ void mfma_gateup_tile(const GateUpArgs& a, const uint16_t* W, int entry, int off, int T,
                                 int local) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H, n = a.n;
    const int nrb = n / kPairsPerMfmaTile;
    const int rb = local / a.ksplit, ks = local % a.ksplit;
    if (rb >= nrb) return;
    const int i0 = rb * kPairsPerMfmaTile + wave * 16;
    const int kbeg = ks * a.kslice;
    const int nsteps = min(a.kslice, H - kbeg) >> 5;
    const int tl = lane & 15, kq = lane >> 4;
    const int NT = (T + 15) >> 4;

    const uint16_t* xrow[4];
    bool xok[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int j = tt * 16 + tl;
        xok[tt] = j < T;
        xrow[tt] = a.x + (size_t)(xok[tt] ? a.perm[off + j] / a.pair_div : 0) * H + kbeg + 8 * kq;
    }
    const uint16_t* gr = W + (size_t)(i0 + tl) * H + kbeg + 8 * kq;
    const uint16_t* ur = W + (size_t)(n + i0 + tl) * H + kbeg + 8 * kq;
    const u32x4 zero = u32x4{0, 0, 0, 0};
    f32x4 cg[4], cu[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) { cg[tt] = f32x4{0, 0, 0, 0}; cu[tt] = f32x4{0, 0, 0, 0}; }
    for (int s = 0; s < nsteps; s += 4) {
        u32x4 Ag[4], Au[4], X[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool sok = s + u < nsteps;
            Ag[u] = sok ? ld16(gr + 32 * (s + u)) : zero;
            Au[u] = sok ? ld16(ur + 32 * (s + u)) : zero;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
                X[u][tt] = (sok && tt < NT && xok[tt]) ? ld16(xrow[tt] + 32 * (s + u)) : zero;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                if (s + u < nsteps && tt < NT) {
                    const bf16x8 Bx = __builtin_bit_cast(bf16x8, X[u][tt]);
                    cg[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, Ag[u]), Bx,
                                                                     cg[tt], 0, 0, 0);
                    cu[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, Au[u]), Bx,
                                                                     cu[tt], 0, 0, 0);
                }
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
    __shared__ int s_flag;
    if (!arrive_last(&a.tile_cnt[entry * nrb + rb], (unsigned)a.ksplit, &s_flag)) return;
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
        mfma_gateup_tile(a, W, entry, off, T, local);
    } else {
        if (T > TB) {
            if (threadIdx.x == 0 && local == 0) atomicOr(&a.meta[M_ERR], ERR_TILE);
            return;
        }
        gemv_gateup_tile<TB>(a, W, off, T, local, s_x);
    }
}

// ---------------------------------------------------------------------------
// down
// ---------------------------------------------------------------------------

// LPR lanes share one W2 row (LPR = min(I/8, 64)); each lane loads NQ 16-byte
// units per row; a wave covers 64/LPR rows per pass and RP passes; the
// workgroup covers R = RP * 4 * (64/LPR) consecutive output rows.  Entries
// (active routed experts, then Is/I column blocks of the shared expert) are
// processed CE at a time, the next chunk's weights requested before the
// current chunk is used.
template <int LPR, int NQ, int RP>
struct DownShape {
    static constexpr int RW = 64 / LPR;
    static constexpr int R = RP * 4 * RW;
    static constexpr int CE = (16 / (RP * NQ)) > 0 ? 16 / (RP * NQ) : 1;
};

template <int LPR, int NQ, int RP>
__device__ __forceinline__ void down_accum(const u32x4 (&wv)[RP][NQ], const float* hrow, float wt, int t,
                                           int wave, int lane, float* s_acc) {
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
        if (c == LPR - 1) s_acc[t * R + (rp * 4 + wave) * RW + rw] += wt * p;
    }
}

// HLDS: every h row of the step (routed slots, then the shared expert's
// rows) is copied to LDS at kernel start, overlapped with the first chunk of
// weight loads, so no h load sits on the per-expert dependency chain.
template <int LPR, int NQ, int RP, bool HLDS>
__global__ __launch_bounds__(256) void down_combine_kernel(DownArgs a) {
    using S = DownShape<LPR, NQ, RP>;
    constexpr int RW = S::RW, R = S::R, CE = S::CE;
    extern __shared__ __align__(16) float s_h[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H, I = a.I, B = a.B, k = a.k;
    const int row0 = blockIdx.x * R;
    const int rw = lane / LPR, c = lane % LPR;
    __shared__ float s_acc[kMaxBatch * R];

    const int nact = *a.n_act;
    const int nsh = a.s2 ? a.Is / I : 0;
    const int total = nact + nsh;
    const size_t estride = (size_t)H * I;

    auto load_chunk = [&](int c0, u32x4 (&buf)[CE][RP][NQ]) {
#pragma unroll
        for (int ce = 0; ce < CE; ++ce) {
            const int ent = c0 + ce;
            if (ent < total) {
                const uint16_t* w;
                int ld;
                if (ent < nact) {
                    int ee = a.act_e[ent];
                    if ((unsigned)ee >= (unsigned)a.n_experts) ee = 0;  // bucketing never publishes this
                    w = a.w2 + (size_t)ee * estride;
                    ld = I;
                }
                else { w = a.s2 + (size_t)(ent - nact) * I; ld = a.Is; }
#pragma unroll
                for (int rp = 0; rp < RP; ++rp) {
                    const int r = row0 + (rp * 4 + wave) * RW + rw;
#pragma unroll
                    for (int q = 0; q < NQ; ++q) buf[ce][rp][q] = ld16(w + (size_t)r * ld + 8 * (c + LPR * q));
                }
            }
        }
    };

    u32x4 wa[CE][RP][NQ], wb[CE][RP][NQ];
    load_chunk(0, wa);
    for (int i = tid; i < B * R; i += 256) s_acc[i] = 0.0f;
    if constexpr (HLDS) {
        const int nh = B * k * I / 4, nhs = (a.s2 ? B * a.Is : 0) / 4;
        const float4* g = reinterpret_cast<const float4*>(a.h);
        const float4* gs = reinterpret_cast<const float4*>(a.hs);
        float4* d = reinterpret_cast<float4*>(s_h);
        for (int i = tid; i < nh; i += 256) d[i] = g[i];
        for (int i = tid; i < nhs; i += 256) d[nh + i] = gs[i];
    }
    __syncthreads();

    // copies h rows [r0, r1) (row i at src + i * ld) into s_h, I floats per row
    auto stage_rows = [&](const float* src, size_t ld, int r0, int r1) {
        const int per = I / 4;
        float4* d = reinterpret_cast<float4*>(s_h);
        for (int i = tid; i < (r1 - r0) * per; i += 256) {
            const int r = i / per, c4 = i - r * per;
            d[i] = reinterpret_cast<const float4*>(src + (size_t)(r0 + r) * ld)[c4];
        }
    };
    const int PB = (kDownHStage / 4) / I;  // h rows per staged batch

    for (int c0 = 0; c0 < total; c0 += CE) {
        if (c0 + CE < total) load_chunk(c0 + CE, wb);  // static weights: requested ahead
        const int c1 = min(c0 + CE, total);
        const int r1 = min(c1, nact);
        if constexpr (HLDS) {
#pragma unroll
            for (int ce = 0; ce < CE; ++ce) {
                const int ent = c0 + ce;
                if (ent < nact) {
                    const int off = a.act_off[ent], T = a.act_off[ent + 1] - off;
                    for (int j = 0; j < T; ++j) {
                        const int p = a.perm[off + j];
                        down_accum<LPR, NQ, RP>(wa[ce], s_h + (size_t)(off + j) * I, a.topk_w[p], p / k, wave,
                                                lane, s_acc);
                    }
                } else if (ent < total) {
                    const int v = ent - nact;
                    const float* hs = s_h + (size_t)B * k * I;
                    for (int t = 0; t < B; ++t)
                        down_accum<LPR, NQ, RP>(wa[ce], hs + (size_t)t * a.Is + (size_t)v * I, 1.0f, t, wave,
                                                lane, s_acc);
                }
            }
        } else {
            // routed entries of the chunk: their h rows are consecutive slots
            if (c0 < r1) {
                const int sa = a.act_off[c0], sb = a.act_off[r1];
                for (int b0 = sa; b0 < sb; b0 += PB) {
                    const int b1 = min(sb, b0 + PB);
                    stage_rows(a.h, I, b0, b1);
                    __syncthreads();
#pragma unroll
                    for (int ce = 0; ce < CE; ++ce) {
                        const int ent = c0 + ce;
                        if (ent < r1) {
                            const int o0 = max(a.act_off[ent], b0), o1 = min(a.act_off[ent + 1], b1);
                            for (int sl = o0; sl < o1; ++sl) {
                                const int p = a.perm[sl];
                                down_accum<LPR, NQ, RP>(wa[ce], s_h + (size_t)(sl - b0) * I, a.topk_w[p], p / k,
                                                        wave, lane, s_acc);
                            }
                        }
                    }
                    __syncthreads();
                }
            }
            // shared-expert column blocks of the chunk: all B tokens each
#pragma unroll
            for (int ce = 0; ce < CE; ++ce) {
                const int ent = c0 + ce;
                if (ent >= nact && ent < c1) {
                    const int v = ent - nact;
                    for (int t0 = 0; t0 < B; t0 += PB) {
                        const int t1 = min(B, t0 + PB);
                        stage_rows(a.hs + (size_t)v * I, a.Is, t0, t1);
                        __syncthreads();
                        for (int t = t0; t < t1; ++t)
                            down_accum<LPR, NQ, RP>(wa[ce], s_h + (size_t)(t - t0) * I, 1.0f, t, wave, lane, s_acc);
                        __syncthreads();
                    }
                }
            }
        }
#pragma unroll
        for (int ce = 0; ce < CE; ++ce)
#pragma unroll
            for (int rp = 0; rp < RP; ++rp)
#pragma unroll
                for (int q = 0; q < NQ; ++q) wa[ce][rp][q] = wb[ce][rp][q];
    }
    // the lane that accumulated (t, row) also writes it: no barrier needed
    if (c == LPR - 1) {
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

}  // namespace moe
