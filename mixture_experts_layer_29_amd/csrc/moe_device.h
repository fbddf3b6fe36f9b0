// moe_device.h -- gfx950 device code shared by the launches of the decode-time
// MoE layer: load/dot/reduction helpers, top-k selection and routing weights,
// bucketing, and the router, gate/up and down work units that the kernels in
// moe_kernels.hip (one launch per stage) and moe_layer.h (the whole layer in
// one launch) are built from.
#pragma once
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
// Expert weights are read once per step: a streaming (non-temporal) load, so
// they do not displace reused data from the caches.
// (Measured on MI355X: 5-6 % faster expert streams above batch 4, and the
// partial rows of the expert-major down stay cached for the combine launch.)
__device__ __forceinline__ u32x4 ld16_stream(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
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

// acc + sum_{i<8} w_i * h_i, w bf16, h given as bf16 hi + lo parts (h ~= hi +
// lo to ~2^-16 relative): two v_dot2_f32_bf16 per weight pair, no unpacking.
__device__ __forceinline__ float dot8_hilo(u32x4 w, u32x4 hi, u32x4 lo, float acc) {
    const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3];
    const uint32_t h0 = hi[0], h1 = hi[1], h2 = hi[2], h3 = hi[3];
    const uint32_t l0 = lo[0], l1 = lo[1], l2 = lo[2], l3 = lo[3];
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w0), as_bf16x2(h0), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w0), as_bf16x2(l0), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w1), as_bf16x2(h1), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w1), as_bf16x2(l1), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w2), as_bf16x2(h2), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w2), as_bf16x2(l2), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w3), as_bf16x2(h3), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w3), as_bf16x2(l3), acc, false);
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

// Wave-wide maximum of unsigned values; masked-off lanes read 0, the identity,
// so each step is a single DPP-fused v_max_u32.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    int x = (int)v;
    x = (int)max((uint32_t)x, (uint32_t)dpp_i<0xb1, 0xf>(0, x));   // quad_perm [1,0,3,2]
    x = (int)max((uint32_t)x, (uint32_t)dpp_i<0x4e, 0xf>(0, x));   // quad_perm [2,3,0,1]
    x = (int)max((uint32_t)x, (uint32_t)dpp_i<0x141, 0xf>(0, x));  // row_half_mirror
    x = (int)max((uint32_t)x, (uint32_t)dpp_i<0x140, 0xf>(0, x));  // row_mirror
    x = (int)max((uint32_t)x, (uint32_t)dpp_i<0x142, 0xa>(0, x));  // row_bcast15
    x = (int)max((uint32_t)x, (uint32_t)dpp_i<0x143, 0xc>(0, x));  // row_bcast31
    return (uint32_t)__builtin_amdgcn_readlane(x, 63);
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

// A value every lane of the wave holds, made visibly wave-uniform (an SGPR):
// branches and loop bounds on it stay scalar instead of being linearised
// with exec masks, which would keep both sides' registers live together.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Data handed from one workgroup to another inside a launch (logits, routing,
// work lists, h, partial sums, the shared-expert output) is written and read
// only through these device-coherent accesses: relaxed agent-scope atomics,
// which gfx950 issues with the sc1 (device scope) cache policy, so they are
// performed where all 8 XCDs see them instead of in one XCD's L2.  A hand-off
// is then: coherent stores, every wave waits for its stores to complete,
// barrier, one relaxed counter update; the reader sees the counter, then
// issues coherent loads.  This avoids agent-scope release/acquire fences,
// which write back / invalidate a whole L2 and cost microseconds each when
// many workgroups hand off at once.  Static data (weights, x, bias) is read
// with ordinary cached loads.
__device__ __forceinline__ float ld_dev(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_dev(const int* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(unsigned* p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// four consecutive floats (16-byte aligned) as two coherent 64-bit loads
__device__ __forceinline__ float4 ld_dev4(const float* p) {
    const unsigned long long* q = reinterpret_cast<const unsigned long long*>(p);
    const unsigned long long a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return float4{__uint_as_float((uint32_t)a), __uint_as_float((uint32_t)(a >> 32)),
                  __uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32))};
}

// Every wave's coherent stores have completed (and the compiler keeps later
// memory operations after them); then the workgroup synchronises.
__device__ __forceinline__ void stores_done_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}

// Counts this workgroup's arrival after its coherent stores completed;
// returns true in the last of `total` workgroups to arrive, which may then
// read every arriver's coherent stores.
__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned total, int* s_flag) {
    stores_done_barrier();
    if (threadIdx.x == 0) {
        const unsigned t = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = t == total - 1;
    }
    __syncthreads();
    return uni(*s_flag) != 0;
}


constexpr int kSpinLimit = 1 << 20;  // bounded waits: a lost hand-off ends in ERR_TIMEOUT, not a hang

// Adds one to *counter once every wave's coherent stores (st_dev) have
// completed, so a workgroup that sees the count can read them with ld_dev.
__device__ __forceinline__ void publish(int32_t* counter) {
    stores_done_barrier();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Blocks the workgroup until *counter >= target (bounded wait).  Loads after
// it are issued after the counter was seen (barrier), and hand-off data is
// read with coherent loads, so no cache invalidation is needed.
__device__ __forceinline__ void wait_count(const int32_t* counter, int target, int32_t* meta) {
    if (threadIdx.x == 0) {
        int it = 0;
        while (ld_dev(counter) < target) {
            if (++it > kSpinLimit) {
                atomicOr(&meta[M_ERR], ERR_TIMEOUT);
                break;
            }
            // back off: many waiting workgroups polling one address slow the
            // memory channel it lives on
            if (it < 4) __builtin_amdgcn_s_sleep(2);
            else if (it < 16) __builtin_amdgcn_s_sleep(8);
            else __builtin_amdgcn_s_sleep(32);
        }
    }
    __syncthreads();
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

constexpr int kNone = 0x7fffffff;

// Unsigned key with the order of the float (larger key = larger value; every
// key of a number, -inf included, is > 0).  -0 and +0 get different keys;
// adding +0.0f first folds -0 into +0.
__device__ __forceinline__ uint32_t order_key(float v) {
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Top-k of one token by one wave.  Slot m of lane l holds the logit of expert
// m * 64 + l in v[m] (slots at or past E are never selected).  Each lane
// first sorts its slots (Batcher's odd-even merge network) by the 64-bit key
// (order key of the logit, then the complement of the expert id), so larger
// logits come first and equal logits go to the lower id; -0 is keyed as +0.
// Each round then takes the wave-wide largest head (DPP max over the upper
// halves; a second max over the lower halves only when several lanes hold
// that logit), and the winning lane pops its head.  Lane r < k ends with
// entry r of the selection (my_e, my_z).  A round costs one reduction and a
// register shift, no rescan of the slots, and the round loop is not unrolled,
// so the code stays small (it runs once per launch, from a cold instruction
// cache).
template <int NS>
__device__ __forceinline__ void topk_wave(const float (&v)[NS], int E, int k, int lane, int& my_e, float& my_z) {
    uint64_t K[NS];  // 0 = empty slot
#pragma unroll
    for (int m = 0; m < NS; ++m) {
        const int e = m * 64 + lane;
        const uint64_t key = ((uint64_t)order_key(v[m] + 0.0f) << 32) | (uint32_t)~e;
        K[m] = e < E ? key : 0ull;
    }
#pragma unroll
    for (int p = 1; p < NS; p <<= 1)
#pragma unroll
        for (int d = p; d >= 1; d >>= 1)
#pragma unroll
            for (int j = d % p; j + d < NS; j += 2 * d)
#pragma unroll
                for (int i = 0; i < d && i + j + d < NS; ++i)
                    if ((i + j) / (2 * p) == (i + j + d) / (2 * p)) {
                        const uint64_t x = K[i + j], y = K[i + j + d];
                        const bool sw = y > x;
                        K[i + j] = sw ? y : x;
                        K[i + j + d] = sw ? x : y;
                    }
    my_e = -1;
    my_z = -INFINITY;
#pragma unroll 1
    for (int r = 0; r < k; ++r) {
        const uint32_t hk = (uint32_t)(K[0] >> 32);
        const uint32_t mk = wave_max_u32(hk);
        if (mk == 0) break;
        unsigned long long bal = __ballot(hk == mk);
        if (__popcll(bal) != 1) {  // the same logit in several lanes: the lowest id
            const uint32_t lo = (uint32_t)K[0];
            const uint32_t ml = wave_max_u32(hk == mk ? lo : 0u);
            bal = __ballot(hk == mk && lo == ml);
        }
        const int w = __ffsll(bal) - 1;
        const int e = ~__builtin_amdgcn_readlane((int)(uint32_t)K[0], w);
        if (lane == r) {
            my_e = e;
            my_z = __uint_as_float((mk & 0x80000000u) ? (mk & 0x7fffffffu) : ~mk);
        }
        if (lane == w) {
#pragma unroll
            for (int m = 0; m + 1 < NS; ++m) K[m] = K[m + 1];
            K[NS - 1] = 0ull;
        }
    }
}

// Routing weights of the selected logits (softmax or sigmoid, optional
// renormalisation over the selection, times routed_scale).  Lane r < k holds
// entry r of the selection (expert er, logit zr); zmax is the largest
// selected logit.  Writes the token's topk_idx / topk_w row (unless
// !to_global) and its s_pair_e row when given.  zrow (the token's logits, readable by this wave) is read only
// for a softmax without renormalisation, whose denominator runs over all E.
__device__ __forceinline__ void route_one(const RouterArgs& a, int t, int lane, const float* zrow, int er, float zr,
                                          float zmax, int32_t* s_pair_e, bool to_global = true) {
    const int k = a.k, E = a.E;
    const bool mine = lane < k;
    float w;
    if (a.score_fn == 0) {
        const float ex = mine ? expf(zr - zmax) : 0.0f;
        float den;
        if (a.renormalize) {
            den = wave_sum(ex);
        } else {
            float part = 0.0f;
            for (int e = lane; e < E; e += 64) part += expf(ld_dev(zrow + e) - zmax);
            den = wave_sum(part);
        }
        w = ex / den;
    } else {
        const float sg = mine ? 1.0f / (1.0f + expf(-zr)) : 0.0f;
        w = a.renormalize ? sg / wave_sum(sg) : sg;
    }
    if (mine) {
        if (to_global) {
            st_dev(a.topk_idx + t * k + lane, er);
            st_dev(a.topk_w + t * k + lane, w * a.routed_scale);
        }
        if (s_pair_e) s_pair_e[t * k + lane] = er;
    }
}

// Writes the bucketing results common to both bucketing forms.
__device__ __forceinline__ void bucket_meta(const RouterArgs& a, int nact, int nmfma, int npairs, int placed) {
    if (placed != npairs) nact = nmfma = 0;  // invalid selection: no expert work at all
    st_dev(a.act_off + nact, npairs);
    st_dev(a.meta + M_NACT, nact);
    st_dev(a.meta + M_MFMA_TILES, nmfma * a.mfma_tiles_per_expert);
    st_dev(a.meta + M_GEMV_TILES, (nact - nmfma) * a.tiles_per_expert);
    if (placed != npairs) atomicOr(&a.meta[M_ERR], ERR_BUCKET);
    st_dev(a.meta + M_ROUTER_CNT, 0);  // re-armed for the next launch
}

// Slot of pair `lane` (expert e) among np <= 64 pairs held one per lane.
// Entries (active experts) come in two classes, experts with at least
// mfma_min pairs ("hot", only when mfma_min > 0) first, then the rest, each by
// ascending id; an entry's slots follow in the same order, by token inside an
// entry.  pos: the pair's slot; the first pair of each expert leads; apos:
// the entry's position (set for leads); cnt: the expert's pair count; hot: its
// class.
//
// Runs in one wave with 128 ints of LDS (s_ps) of its own: every lane writes
// its unique key (class, expert, lane) to LDS and counts the smaller keys from
// broadcast reads of all of them (a rank, i.e. the key's sorted position),
// then scatters its key to that position; neighbours in sorted order give the
// leads, and a ballot of the leads gives apos and the counts.  The class needs
// the counts, so a second pass ranks again when any expert is hot.  LDS
// accesses of one wave complete in issue order, so compiler-only fences are
// all the ordering this needs.  (A loop of per-lane readlanes cost ~5 us for
// 64 pairs.)
struct PairSlot {
    int pos, apos, cnt;
    bool lead, hot;
};
__device__ __forceinline__ void rank_pass(int key, bool act, int np, int lane, int32_t* s_ps, int& pos,
                                          unsigned long long& lm) {
    s_ps[lane] = key;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    pos = 0;
    const int4* k4 = reinterpret_cast<const int4*>(s_ps);
    const int nq = (np + 15) >> 4;
    for (int q = 0; q < nq; ++q) {
        int4 v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = k4[4 * q + c];
#pragma unroll
        for (int c = 0; c < 4; ++c)
            pos += (v[c].x < key ? 1 : 0) + (v[c].y < key ? 1 : 0) + (v[c].z < key ? 1 : 0) + (v[c].w < key ? 1 : 0);
    }
    if (act) s_ps[64 + pos] = key;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const int cur = act ? s_ps[64 + lane] >> 6 : -1;
    const int prev = (act && lane > 0) ? s_ps[63 + lane] >> 6 : -1;
    lm = __ballot(act && cur != prev);  // leads, by sorted position
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ PairSlot pair_slot(int e, int np, int lane, int32_t* s_ps, int mfma_min = 0) {
    constexpr int kPad = 1 << 21;  // inactive lanes: above every class and expert id (E <= 1024)
    const bool act = lane < np;
    int key = (act ? e : kPad) * 64 + lane, pos;
    unsigned long long lm;
    rank_pass(key, act, np, lane, s_ps, pos, lm);
    const int p = act ? pos : 0;
    // the pair's expert's count: from its lead (highest lead at or below p) to the next lead
    const unsigned long long below = lm & ((p < 63 ? (2ull << p) : 0ull) - 1ull);
    const unsigned long long above = p < 63 ? (lm >> (p + 1)) << (p + 1) : 0ull;
    const int lead_at = 63 - __clzll(below | 1ull);
    const int cnt = (above ? __ffsll(above) - 1 : np) - lead_at;
    const bool hot = act && mfma_min > 0 && cnt >= mfma_min;
    if (__ballot(hot)) {  // second pass: hot experts' keys first
        key = (act && !hot ? (1 << 26) : 0) + key;
        rank_pass(key, act, np, lane, s_ps, pos, lm);
    }
    PairSlot r{0, 0, 0, false, false};
    if (act) {
        r.pos = pos;
        r.lead = (lm >> pos) & 1ull;
        r.apos = __popcll(lm & ((1ull << pos) - 1ull));
        r.cnt = cnt;
        r.hot = hot;
    }
    return r;
}

// Bucketing by one wave for B*k <= 64 pairs (pair p in lane p) into the
// global work lists (see pair_slot).  No barriers and no LDS atomics.
__device__ __forceinline__ void bucket_wave(const RouterArgs& a, const int32_t* s_pair_e, int lane, int32_t* s_ps) {
    const int np = a.B * a.k;
    const int e = lane < np ? s_pair_e[lane] : kNone;
    if (__ballot(lane < np && (e < 0 || e >= a.E))) {  // never hand an invalid id to the experts
        if (lane == 0) bucket_meta(a, 0, 0, np, -1);
        return;
    }
    const PairSlot ps = pair_slot(e, np, lane, s_ps, a.mfma_min_tokens);
    if (lane < np) st_dev(a.perm + ps.pos, lane);
    if (ps.lead) {
        st_dev(a.act_e + ps.apos, e);
        st_dev(a.act_off + ps.apos, ps.pos);
    }
    const int nact = __popcll(__ballot(ps.lead));
    const int nmfma = __popcll(__ballot(ps.lead && ps.hot));
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

    // Entries (and their slot ranges) in two classes: experts with at least
    // mfma_min_tokens tokens first, then the rest, each by ascending id.  The
    // grids of the staged gate/up and down launches follow the entry order, so
    // the heavy entries are dispatched first and the launches end on light ones.
    constexpr int CH = kMaxExperts / 256;  // bins per thread
    int cnt[CH], hc = 0, hf = 0, lc = 0, lf = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int bin = tid * CH + c;
        cnt[c] = (bin < E) ? s_cnt[bin] : 0;
        const bool hot = a.mfma_min_tokens > 0 && cnt[c] >= a.mfma_min_tokens;
        hc += hot ? cnt[c] : 0;
        hf += hot ? 1 : 0;
        lc += hot ? 0 : cnt[c];
        lf += (!hot && cnt[c] > 0) ? 1 : 0;
    }
    int hcx, hfx, hct, hft, lcx, lfx, lct, lft;
    block_scan2(hc, hf, s_tmp, hcx, hfx, hct, hft);
    block_scan2(lc, lf, s_tmp, lcx, lfx, lct, lft);
    lcx += hct;  // the light entries' slots and list positions follow the heavy ones
    lfx += hft;
    const int ctot = hct + lct, ftot = hft + lft;
    int nm = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int bin = tid * CH + c;
        if (bin < E) {
            const bool hot = a.mfma_min_tokens > 0 && cnt[c] >= a.mfma_min_tokens;
            const int cex = hot ? hcx : lcx, fex = hot ? hfx : lfx;
            s_cnt[bin] = cex;  // becomes the bucket offset
            if (cnt[c] > 0) {
                st_dev(a.act_e + fex, bin);
                st_dev(a.act_off + fex, cex);
                if (hot) {
                    ++nm;
                    ++hfx;
                } else {
                    ++lfx;
                }
            }
            if (hot) hcx += cnt[c];
            else lcx += cnt[c];
        }
    }
    if (nm) atomicAdd(s_nmfma, nm);
    __syncthreads();
    for (int p = tid; p < npairs; p += 256)
        if (s_rank[p] >= 0) st_dev(a.perm + s_cnt[s_pair_e[p]] + s_rank[p], p);
    if (tid == 0) bucket_meta(a, ftot, *s_nmfma, npairs, ctot);
}

// Selection for tokens t0 + wave of this workgroup, one wave per token.
// src: per-token logit rows (E floats); with `from_acc` they are the first of
// a.nzpart split-K partial slices [nzpart][B][E] written by an earlier launch:
// they are summed, the bias is added and the logits stored to a.z.  Ends with a workgroup barrier, after which s_pair_e (if given)
// holds the selected ids of the workgroup's tokens.  !to_global: the routing
// rows (topk_idx / topk_w) are not written.  COH: src was written by other
// workgroups of this launch (coherent loads); else by an earlier launch.
// mid() runs in every wave once the logit loads are issued and before they
// are used: loads it issues complete after them.
struct NoMid {
    __device__ void operator()() const {}
};
template <int NS, bool COH = true, class Mid = NoMid>
__device__ __forceinline__ void select_tokens(const RouterArgs& a, int t0, float* src, const float* bias,
                                              bool from_acc, int32_t* s_pair_e, bool to_global = true,
                                              Mid&& mid = Mid{}) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int E = a.E, B = a.B, k = a.k;
    const int t = t0 + wave;
    float* row = src + (size_t)t * E;
    float* zo = a.z + (size_t)t * E;
    float v[NS];
    if (t < B && from_acc) {
        // partial logits [nzpart][B][E] written by the launch before, summed in
        // a fixed order; QC partials per round, every load of a round issued
        // before the first add (clamped addresses, masked adds)
        constexpr int QC = NS <= 8 ? 8 : 4;
        const int nz = a.nzpart;
        const size_t qs = (size_t)B * E;
#pragma unroll
        for (int m = 0; m < NS; ++m) v[m] = 0.0f;
        for (int q0 = 0; q0 < nz; q0 += QC) {
            float tmp[QC][NS];
#pragma unroll
            for (int qq = 0; qq < QC; ++qq) {
                const size_t q = (size_t)min(q0 + qq, nz - 1);
#pragma unroll
                for (int m = 0; m < NS; ++m) tmp[qq][m] = row[q * qs + min(m * 64 + lane, E - 1)];
            }
            // keep the adds below every load of the round: interleaved by the
            // scheduler, they made the round several dependent round trips
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int qq = 0; qq < QC; ++qq)
#pragma unroll
                for (int m = 0; m < NS; ++m)
                    if (q0 + qq < nz) v[m] += tmp[qq][m];
        }
#pragma unroll
        for (int m = 0; m < NS; ++m) {
            const int e = m * 64 + lane;
            if (e < E) {
                v[m] += bias ? bias[e] : 0.0f;
                st_dev(zo + e, v[m]);
            } else {
                v[m] = -INFINITY;
            }
        }
    } else if (t < B) {
#pragma unroll
        for (int m = 0; m < NS; ++m) {
            const int e = m * 64 + lane;
            float x = -INFINITY;
            if (e < E) {
                if constexpr (COH) x = ld_dev(row + e);
                else x = row[e];
            }
            v[m] = x;
        }
    }
    mid();
    if (t < B) {
        int my_e;
        float my_z;
        topk_wave<NS>(v, E, k, lane, my_e, my_z);
        // a full softmax (no renormalisation) reads the token's logits back:
        // from_acc rows are in a.z (this wave's stores, complete after the
        // wait).  Every other weight form needs only the selection, and
        // skips the wait for the stores' write-through.
        if (from_acc && a.score_fn == 0 && !a.renormalize) __builtin_amdgcn_s_waitcnt(0);
        route_one(a, t, lane, from_acc ? zo : row, my_e, my_z, __shfl(my_z, 0, 64), s_pair_e, to_global);
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// front launch, batch <= 4: router GEMV + (last workgroup) top-k and bucketing,
// plus the shared expert's gate/up in trailing workgroups
// ---------------------------------------------------------------------------

template <int TB, bool COH = false>
__device__ __forceinline__ void gemv_gateup_tile(const GateUpArgs& a, const uint16_t* W, int off, int T, int local,
                                 uint16_t* s_x, const int32_t* s_tok = nullptr);
template <int NTM>
__device__ __forceinline__ bool mfma_gateup_tile(const GateUpArgs& a, const uint16_t* W, int entry, int off, int T, int local);

// Router rows of block `blk` (one row per wave) for all B tokens: x staged in
// LDS while the row loads are in flight; z = x . Wr[e] (+ bias) -- or the raw
// sum into zacc when the selection runs in a later launch.
template <int TB, bool TO_Z>
__device__ __forceinline__ void router_rows(const RouterArgs& a, int blk, uint16_t* s_x) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H, E = a.E, B = a.B;
    const int units = H >> 3, nu = (units + 63) >> 6;
    const int e = blk * 4 + wave;
    const bool row_ok = e < E;
    const uint16_t* wrow = a.wr + (size_t)(row_ok ? e : 0) * H;
    const u32x4 zero = u32x4{0, 0, 0, 0};

    float acc[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[t] = 0.0f;
    // x ([B][H], contiguous) is staged in LDS: the first kXStage units per
    // thread are requested before the weights, since vector memory loads
    // complete in issue order and a store of x issued after the weights would
    // wait for them; any rest follows them.
    const int nx = B * units;
    u32x4 xr[kXStage];
#pragma unroll
    for (int q = 0; q < kXStage; ++q) {
        const int i = tid + 256 * q;
        xr[q] = ld16(a.x + (size_t)(i < nx ? i : 0) * 8);
    }
    for (int base = 0; base < nu; base += kMaxGemvUnits) {
        u32x4 w[kMaxGemvUnits];
#pragma unroll
        for (int q = 0; q < kMaxGemvUnits; ++q) {
            const int u = (base + q) * 64 + lane;
            w[q] = (row_ok && u < units) ? ld16_stream(wrow + u * 8) : zero;
        }
        if (base == 0) {
#pragma unroll
            for (int q = 0; q < kXStage; ++q)
                if (tid + 256 * q < nx) st16(s_x + (tid + 256 * q) * 8, xr[q]);
            for (int i = tid + 256 * kXStage; i < nx; i += 256) st16(s_x + i * 8, ld16(a.x + (size_t)i * 8));
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
                    if constexpr (TO_Z) st_dev(a.z + (size_t)t * E + e, s + b);
                    else st_dev(a.zacc + (size_t)t * E + e, s);
                }
            }
        }
    }
}


// ---------------------------------------------------------------------------
// front launch, batch > 4: dense split-K MFMA tiles (router logits and the
// shared expert's gate/up rows) writing fp32 partials; topk_bucket sums them
// ---------------------------------------------------------------------------

// One tile: 16 rows of W [nrows][H] x one K split of `ksteps` 32-wide steps x
// all B <= 16*NT tokens.  The four waves take interleaved steps of the split
// (wave w: steps w, w+4, ...), so a wave issues all its weight and activation
// loads of a round of four steps before its first MFMA; the waves' 16 x B
// accumulators are summed in LDS and stored as partial [ks][B][nrows] with
// plain stores: no atomics, no counters, nothing to re-arm.  The consumer (the
// next launch) sums the nks partials in a fixed order.
// MFMA 16x16x32 bf16: A = 16 weight rows x 32 K (lane: row lane%16, K group
// lane/16), B = x^T 32 K x 16 tokens (lane: token lane%16, K group lane/16);
// D: lane holds rows 4*(lane/16)+r of token lane%16.
template <int NT>
__device__ __forceinline__ void dense_splitk_tile(const uint16_t* W, int nrows, const uint16_t* x, int B, int H,
                                                  int ksteps, int rb, int ks, float* part, float* s_red) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tl = lane & 15, kq = lane >> 4;
    const int r0 = rb * 16;
    const bool rok = r0 + tl < nrows;
    const uint16_t* wr = W + (size_t)(rok ? r0 + tl : 0) * H + (size_t)ks * ksteps * 32 + 8 * kq;
    const uint16_t* xr[NT];
    bool xok[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
        const int t = tt * 16 + tl;
        xok[tt] = t < B;
        xr[tt] = x + (size_t)(xok[tt] ? t : 0) * H + (size_t)ks * ksteps * 32 + 8 * kq;
    }
    const u32x4 zero = u32x4{0, 0, 0, 0};
    f32x4 c[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) c[tt] = f32x4{0, 0, 0, 0};
    for (int base = wave; base < ksteps; base += 16) {
        u32x4 A[4], X[4][NT];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int s = base + 4 * u;
            const bool sok = s < ksteps;
            A[u] = (sok && rok) ? ld16_stream(wr + 32 * s) : zero;
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) X[u][tt] = (sok && xok[tt]) ? ld16(xr[tt] + 32 * s) : zero;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (base + 4 * u < ksteps)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt)
                    c[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[u]),
                                                                    __builtin_bit_cast(bf16x8, X[u][tt]), c[tt],
                                                                    0, 0, 0);
    }
    // s_red[wave][tt][r][lane]
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) s_red[((wave * NT + tt) * 4 + r) * 64 + lane] = c[tt][r];
    __syncthreads();
    // thread -> (token t, row 0..15), 16 consecutive rows of one token per 16 threads
    for (int idx = tid; idx < NT * 256; idx += 256) {
        const int t = idx >> 4, row = idx & 15;
        const int tt = t >> 4, src = (row >> 2) * 16 + (t & 15), r = row & 3;
        if (t < B && r0 + row < nrows) {
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < 4; ++w) v += s_red[((w * NT + tt) * 4 + r) * 64 + src];
            part[((size_t)ks * B + t) * nrows + r0 + row] = v;
        }
    }
}


// ---------------------------------------------------------------------------
// gateup
// ---------------------------------------------------------------------------

// Full-K GEMV tile: wave w computes row pair i = 4*local + w (gate row i and
// up row n+i) for the entry's T <= TB tokens, whose activations the workgroup
// stages in LDS after issuing its weight loads.  s_tok (TB <= 4, not COH): the
// entry's token ids in LDS, in slot order, instead of a.perm.
template <int TB, bool COH>
__device__ __forceinline__ void gemv_gateup_tile(const GateUpArgs& a, const uint16_t* W, int off, int T, int local,
                                 uint16_t* s_x, const int32_t* s_tok) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H, n = a.n, units = H >> 3, nu = (units + 63) >> 6;
    const int i = local * kPairsPerGemvTile + wave;
    const uint16_t* g = W + (size_t)i * H;
    const uint16_t* u = W + (size_t)(n + i) * H;
    const u32x4 zero = u32x4{0, 0, 0, 0};
    float ag[TB], au[TB];
#pragma unroll
    for (int j = 0; j < TB; ++j) { ag[j] = 0.0f; au[j] = 0.0f; }
    // The entry's token rows.  Staged launches read the work list of an
    // earlier launch with scalar loads (their counter is separate from the
    // weights'); the single launch reads it coherently, per unit.
    const int nx = T * units;
    int tk[4] = {0, 0, 0, 0};
    if constexpr (!COH && TB <= 4) {
#pragma unroll
        for (int j = 0; j < TB; ++j)
            tk[j] = j >= T ? 0 : s_tok ? uni(s_tok[j]) : uni(a.perm[off + j]) / a.pair_div;
    }
    auto xsrc = [&](int idx) {  // unit idx of the staged [T][H] activations
        const int j = idx / units, uu = idx - j * units;
        int t;
        if constexpr (!COH && TB <= 4) t = j == 0 ? tk[0] : j == 1 ? tk[1] : j == 2 ? tk[2] : tk[3];
        else t = (COH ? ld_dev(a.perm + off + j) : a.perm[off + j]) / a.pair_div;
        return a.x + (size_t)t * H + uu * 8;
    };
    for (int base = 0; base < nu; base += kMaxGemvUnits) {
        u32x4 wg[kMaxGemvUnits], wu[kMaxGemvUnits];
#pragma unroll
        for (int q = 0; q < kMaxGemvUnits; ++q) {
            const int uu = (base + q) * 64 + lane;
            const bool ok = uu < units;
            wg[q] = ok ? ld16_stream(g + uu * 8) : zero;
            wu[q] = ok ? ld16_stream(u + uu * 8) : zero;
        }
        if (base == 0) {
            // activations to LDS: all of this thread's first kXStage units are
            // requested right behind the weights and stored once they are in
            // (loads complete in issue order), so x costs no extra round trip
            u32x4 xr[kXStage];
#pragma unroll
            for (int q = 0; q < kXStage; ++q) {
                const int idx = tid + 256 * q;
                xr[q] = ld16(xsrc(idx < nx ? idx : 0));
            }
#pragma unroll
            for (int q = 0; q < kXStage; ++q)
                if (tid + 256 * q < nx) st16(s_x + (tid + 256 * q) * 8, xr[q]);
            for (int idx = tid + 256 * kXStage; idx < nx; idx += 256) st16(s_x + idx * 8, ld16(xsrc(idx)));
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
            if (lane == 0) st_dev(a.h + (size_t)(off + j) * n + i, silu_f(gs) * us);
        }
    }
}

// Last of a row block's split-K tiles: h = SiLU(gate) * up for the block's
// 64 row pairs and T tokens from the fp32 sums, which (with the block's
// counter) it clears for the next step.  A thread requests the sums of
// kFinishBatch elements at once: at 64 tokens it handles 16, and one at a
// time would be 16 coherent round trips in a row.
__device__ __forceinline__ void mfma_tile_finish(const GateUpArgs& a, int entry, int nrb, int rb, int off, int T) {
    constexpr int kFinishBatch = 8;
    const int tid = threadIdx.x, n = a.n, n2 = 2 * n;
    const int rows = kPairsPerMfmaTile, total = rows * T;
    for (int i0 = tid; i0 < total; i0 += 256 * kFinishBatch) {
        float g[kFinishBatch], u[kFinishBatch];
#pragma unroll
        for (int q = 0; q < kFinishBatch; ++q) {
            const int idx = min(i0 + 256 * q, total - 1);
            const int j = idx / rows, i = rb * rows + idx % rows;
            const float* gp = a.g_acc + (size_t)(off + j) * n2;
            g[q] = ld_dev(gp + i);
            u[q] = ld_dev(gp + n + i);
        }
#pragma unroll
        for (int q = 0; q < kFinishBatch; ++q) {
            const int idx = i0 + 256 * q;
            if (idx < total) {
                const int j = idx / rows, i = rb * rows + idx % rows;
                float* gp = a.g_acc + (size_t)(off + j) * n2;
                st_dev(a.h + (size_t)(off + j) * n + i, silu_f(g[q]) * u[q]);
                st_dev(gp + i, 0.0f);
                st_dev(gp + n + i, 0.0f);
            }
        }
    }
    if (tid == 0) st_dev(a.tile_cnt + entry * nrb + rb, 0u);
}

// Split-K MFMA tile: 64 row pairs (16 per wave) x one K slice x T <= 16*NTM
// tokens (NTM 16-token column tiles; a small NTM keeps the register budget
// small where the token count is known to be small).
// A = weight rows (16 x 32), B = x^T (32 x 16 tokens); fp32 partials are
// added to g_acc; the last of the `ksplit` tiles of the row block applies
// SiLU*up, writes h and clears g_acc and its counter.
template <int NTM>
__device__ __forceinline__ bool mfma_gateup_tile(const GateUpArgs& a, const uint16_t* W, int entry, int off, int T,
                                 int local) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H, n = a.n;
    const int nrb = n / kPairsPerMfmaTile;
    const int rb = local / a.ksplit, ks = local % a.ksplit;
    if (rb >= nrb) return false;
    const int i0 = rb * kPairsPerMfmaTile + wave * 16;
    const int kbeg = ks * a.kslice;
    const int nsteps = min(a.kslice, H - kbeg) >> 5;
    const int tl = lane & 15, kq = lane >> 4;
    const int NT = (T + 15) >> 4;

    const uint16_t* xrow[NTM];
    bool xok[NTM];
#pragma unroll
    for (int tt = 0; tt < NTM; ++tt) {
        const int j = tt * 16 + tl;
        xok[tt] = j < T;
        xrow[tt] = a.x + (size_t)(xok[tt] ? ld_dev(a.perm + off + j) / a.pair_div : 0) * H + kbeg + 8 * kq;
    }
    const uint16_t* gr = W + (size_t)(i0 + tl) * H + kbeg + 8 * kq;
    const uint16_t* ur = W + (size_t)(n + i0 + tl) * H + kbeg + 8 * kq;
    const u32x4 zero = u32x4{0, 0, 0, 0};
    f32x4 cg[NTM], cu[NTM];
#pragma unroll
    for (int tt = 0; tt < NTM; ++tt) { cg[tt] = f32x4{0, 0, 0, 0}; cu[tt] = f32x4{0, 0, 0, 0}; }
    for (int s = 0; s < nsteps; s += 4) {
        u32x4 Ag[4], Au[4], X[4][NTM];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool sok = s + u < nsteps;
            Ag[u] = sok ? ld16_stream(gr + 32 * (s + u)) : zero;
            Au[u] = sok ? ld16_stream(ur + 32 * (s + u)) : zero;
#pragma unroll
            for (int tt = 0; tt < NTM; ++tt)
                X[u][tt] = (sok && tt < NT && xok[tt]) ? ld16(xrow[tt] + 32 * (s + u)) : zero;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int tt = 0; tt < NTM; ++tt) {
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
    for (int tt = 0; tt < NTM; ++tt) {
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
    if (!arrive_last(&a.tile_cnt[entry * nrb + rb], (unsigned)a.ksplit, &s_flag)) return true;
    mfma_tile_finish(a, entry, nrb, rb, off, T);
    return true;
}


// Split-K MFMA tile of the staged gate/up launch (batch > 4): the same tile
// as mfma_gateup_tile<4> (64 row pairs x one K slice x T <= 64 tokens, fp32
// partials to g_acc, the last of the ksplit tiles applies SiLU*up), but a wave
// requests all gate and up weights of its slice (up to kMfmaChunk steps of 32)
// in one round, and the tokens' activations for the slice are staged in LDS
// (rows padded by 8 elements against bank conflicts) while the weights stream.
constexpr int kMfmaChunk = 14;                    // K steps of 32 per round (the TP8 shape's slice)
constexpr int kMfmaXLd = kMfmaChunk * 32 + 8;     // LDS row stride of staged x (elements)
__host__ __device__ constexpr size_t mfma_tile_lds_bytes() { return (size_t)kMaxBatch * kMfmaXLd * 2; }

__device__ __forceinline__ bool mfma_gateup_tile_lds(const GateUpArgs& a, const uint16_t* W, int entry, int off,
                                                     int T, int local, uint16_t* s_x) {
    __shared__ int s_tk[kMaxBatch];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H, n = a.n;
    const int nrb = n / kPairsPerMfmaTile;
    const int rb = local / a.ksplit, ks = local % a.ksplit;
    if (rb >= nrb) return false;
    const int i0 = rb * kPairsPerMfmaTile + wave * 16;
    const int kbeg = ks * a.kslice;
    const int nsteps = min(a.kslice, H - kbeg) >> 5;
    const int tl = lane & 15, kq = lane >> 4;
    const int NT = (T + 15) >> 4;
    const uint16_t* gr = W + (size_t)(i0 + tl) * H + kbeg + 8 * kq;
    const uint16_t* ur = W + (size_t)(n + i0 + tl) * H + kbeg + 8 * kq;
    const u32x4 zero = u32x4{0, 0, 0, 0};
    f32x4 cg[4], cu[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) { cg[tt] = f32x4{0, 0, 0, 0}; cu[tt] = f32x4{0, 0, 0, 0}; }
    for (int c0 = 0; c0 < nsteps; c0 += kMfmaChunk) {
        const int ns = min(kMfmaChunk, nsteps - c0);
        u32x4 Ag[kMfmaChunk], Au[kMfmaChunk];
#pragma unroll
        for (int u = 0; u < kMfmaChunk; ++u) {
            const bool ok = u < ns;
            Ag[u] = ok ? ld16_stream(gr + 32 * (c0 + u)) : zero;
            Au[u] = ok ? ld16_stream(ur + 32 * (c0 + u)) : zero;
        }
        // stage x[T][ns * 32] of this chunk: token ids first, then this
        // thread's units (at most 64 * 14 * 4 / 256 <= 16) in rounds of 8
        if (c0 == 0 && tid < T) s_tk[tid] = ld_dev(a.perm + off + tid) / a.pair_div;
        __syncthreads();  // token ids in; the previous chunk's reads of s_x done
        const int upr = ns * 4;  // 16-byte units per token row of the chunk
        for (int q0 = 0; q0 < 16; q0 += 8) {  // two rounds of 8 units: registers stay for the weights
            if (256 * q0 >= T * upr) break;
            u32x4 xv[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int idx = tid + 256 * (q0 + q);
                const int j = idx / upr, uu = idx - j * upr;
                xv[q] = idx < T * upr ? ld16(a.x + (size_t)s_tk[j < T ? j : 0] * H + kbeg + 32 * c0 + 8 * uu) : zero;
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int idx = tid + 256 * (q0 + q);
                const int j = idx / upr, uu = idx - j * upr;
                if (idx < T * upr) st16(s_x + j * kMfmaXLd + 8 * uu, xv[q]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kMfmaChunk; ++u) {
            if (u < ns) {
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    if (tt < NT) {
                        const int j = tt * 16 + tl;
                        const u32x4 xb = j < T ? ld16(s_x + j * kMfmaXLd + 32 * u + 8 * kq) : zero;
                        const bf16x8 Bx = __builtin_bit_cast(bf16x8, xb);
                        cg[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, Ag[u]), Bx,
                                                                         cg[tt], 0, 0, 0);
                        cu[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, Au[u]), Bx,
                                                                         cu[tt], 0, 0, 0);
                    }
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
    if (!arrive_last(&a.tile_cnt[entry * nrb + rb], (unsigned)a.ksplit, &s_flag)) return true;
    mfma_tile_finish(a, entry, nrb, rb, off, T);
    return true;
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

enum DownMode : int {
    DOWN_ALL = 0,     // routed experts + shared column blocks, bf16 out (+ residual)
    DOWN_SHARED = 1,  // shared column blocks only, fp32 result to s_out
    DOWN_ROUTED = 2   // routed experts only; finalize adds s_out (+ residual)
};

// Down projection of one block of R output rows (row_block), see DownShape.
// HLDS: every h row the block needs is copied to LDS once, overlapped with the
// first chunk of weight loads; otherwise h is staged chunk by chunk.
// wait() runs after the first chunk of (static) weights is requested and
// before any h is read: the single-launch layer blocks there until the gate/up
// tasks are done.  s_h: dynamic LDS; s_acc: kMaxBatch * R floats of LDS.
// COH: routing, work lists and h may come from other workgroups of this
// launch (coherent loads); otherwise from an earlier launch (cached loads).
template <int LPR, int NQ, int RP, bool HLDS, int MODE, bool COH, class Wait>
__device__ __forceinline__ void down_rows(const DownArgs& a, int row_block, float* s_h, float* s_acc, Wait&& wait) {
    constexpr int mode = MODE;
    auto ldi = [](const int* p) { if constexpr (COH) return ld_dev(p); else return *p; };
    auto ldf = [](const float* p) { if constexpr (COH) return ld_dev(p); else return *p; };
    auto ld4 = [](const float* p) {
        if constexpr (COH) return ld_dev4(p);
        else return *reinterpret_cast<const float4*>(p);
    };
    using S = DownShape<LPR, NQ, RP>;
    constexpr int RW = S::RW, R = S::R, CE = S::CE;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H, I = a.I, B = a.B, k = a.k;
    const int row0 = row_block * R;
    const int rw = lane / LPR, c = lane % LPR;

    const int nact = mode == DOWN_SHARED ? 0 : uni(ldi(a.n_act));
    const int nsh = (mode == DOWN_ROUTED || !a.s2) ? 0 : a.Is / I;
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
                    int ee = uni(ldi(a.act_e + ent));
                    if ((unsigned)ee >= (unsigned)a.n_experts) ee = 0;  // bucketing never publishes this
                    w = a.w2 + (size_t)ee * estride;
                    ld = I;
                } else {
                    w = a.s2 + (size_t)(ent - nact) * I;
                    ld = a.Is;
                }
#pragma unroll
                for (int rp = 0; rp < RP; ++rp) {
                    const int r = row0 + (rp * 4 + wave) * RW + rw;
#pragma unroll
                    for (int q = 0; q < NQ; ++q) buf[ce][rp][q] = ld16_stream(w + (size_t)r * ld + 8 * (c + LPR * q));
                }
            }
        }
    };

    // two chunk buffers used alternately (the chunk loop is unrolled by two),
    // so the next chunk's weights are in flight while this one is used and no
    // register copies force an early wait
    u32x4 wbuf0[CE][RP][NQ], wbuf1[CE][RP][NQ];
    load_chunk(0, wbuf0);
    for (int i = tid; i < B * R; i += 256) s_acc[i] = 0.0f;
    wait();
    // LDS layout when HLDS: routed h rows [B*k][I], then shared rows [B][Is]
    const size_t hs_off = (size_t)B * k * I;
    if constexpr (HLDS) {
        const int nh = nact ? B * k * I / 4 : 0, nhs = nsh ? B * a.Is / 4 : 0;
        float4* d = reinterpret_cast<float4*>(s_h);
        for (int i = tid; i < nh; i += 256) d[i] = ld4(a.h + 4 * i);
        for (int i = tid; i < nhs; i += 256) d[hs_off / 4 + i] = ld4(a.hs + 4 * i);
    }
    __syncthreads();

    // copies h rows [r0, r1) (row i at src + i * ld) into s_h, I floats per row
    auto stage_rows = [&](const float* src, size_t ld, int r0, int r1) {
        const int per = I / 4;
        float4* d = reinterpret_cast<float4*>(s_h);
        for (int i = tid; i < (r1 - r0) * per; i += 256) {
            const int r = i / per, c4 = i - r * per;
            d[i] = ld4(src + (size_t)(r0 + r) * ld + 4 * c4);
        }
    };
    const int PB = (kDownHStage / 4) / I;  // h rows per staged batch

    auto process = [&](int c0, const u32x4 (&wa)[CE][RP][NQ]) {
        const int c1 = min(c0 + CE, total);
        const int r1 = min(c1, nact);
        if constexpr (HLDS) {
#pragma unroll
            for (int ce = 0; ce < CE; ++ce) {
                const int ent = c0 + ce;
                if (ent < nact) {
                    const int off = uni(ldi(a.act_off + ent)), T = uni(ldi(a.act_off + ent + 1)) - off;
                    for (int j = 0; j < T; ++j) {
                        const int p = uni(ldi(a.perm + off + j));
                        down_accum<LPR, NQ, RP>(wa[ce], s_h + (size_t)(off + j) * I, ldf(a.topk_w + p), p / k, wave,
                                                lane, s_acc);
                    }
                } else if (ent < total) {
                    const int v = ent - nact;
                    const float* hs = s_h + hs_off;
                    for (int t = 0; t < B; ++t)
                        down_accum<LPR, NQ, RP>(wa[ce], hs + (size_t)t * a.Is + (size_t)v * I, 1.0f, t, wave,
                                                lane, s_acc);
                }
            }
        } else {
            // routed entries of the chunk: their h rows are consecutive slots
            if (c0 < r1) {
                const int sa = uni(ldi(a.act_off + c0)), sb = uni(ldi(a.act_off + r1));
                for (int b0 = sa; b0 < sb; b0 += PB) {
                    const int b1 = min(sb, b0 + PB);
                    stage_rows(a.h, I, b0, b1);
                    __syncthreads();
#pragma unroll
                    for (int ce = 0; ce < CE; ++ce) {
                        const int ent = c0 + ce;
                        if (ent < r1) {
                            const int o0 = max(uni(ldi(a.act_off + ent)), b0);
                            const int o1 = min(uni(ldi(a.act_off + ent + 1)), b1);
                            for (int sl = o0; sl < o1; ++sl) {
                                const int p = uni(ldi(a.perm + sl));
                                down_accum<LPR, NQ, RP>(wa[ce], s_h + (size_t)(sl - b0) * I, ldf(a.topk_w + p), p / k,
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
    };
    for (int c0 = 0; c0 < total; c0 += 2 * CE) {
        if (c0 + CE < total) load_chunk(c0 + CE, wbuf1);  // static weights: requested ahead
        process(c0, wbuf0);
        if (c0 + CE >= total) break;
        if (c0 + 2 * CE < total) load_chunk(c0 + 2 * CE, wbuf0);
        process(c0 + CE, wbuf1);
    }
    // the lane that accumulated (t, row) also writes it: no barrier needed
    if (c == LPR - 1) {
#pragma unroll
        for (int rp = 0; rp < RP; ++rp) {
            const int rl = (rp * 4 + wave) * RW + rw;
            const int r = row0 + rl;
            for (int t = 0; t < B; ++t) {
                float v = s_acc[t * R + rl];
                if (mode == DOWN_SHARED) {
                    st_dev(a.s_out + (size_t)t * H + r, v);
                    continue;
                }
                if (mode == DOWN_ROUTED && a.s_out) v += ld_dev(a.s_out + (size_t)t * H + r);
                if (a.add_residual) v += __uint_as_float((uint32_t)a.x[(size_t)t * H + r] << 16);
                a.out[(size_t)t * H + r] = f32_to_bf16_rne(v);
            }
        }
    }
}


}  // namespace moe
