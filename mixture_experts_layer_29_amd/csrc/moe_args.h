// moe_args.h -- kernel argument blocks and workspace layout shared by the
// host side (moe_decode.cpp) and the gfx950 kernels (moe_kernels.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Slots of the int32 `meta` block at the start of the workspace.
enum Meta : int {
    M_NACT = 0,        // |U| of the step (routed experts with >= 1 token)
    M_ROUTER_CNT = 1,  // arrival counter of the router kernel's workgroups
    M_GEMV_TILES = 2,  // routed gate/up tiles that took the GEMV path
    M_MFMA_TILES = 3,  // routed gate/up tiles that took the MFMA path
    M_ERR = 4,         // device-side error bits
    M_SHARED_NACT = 5, // constant 1: the shared expert's one-entry work list
    M_COUNT = 16
};

enum ErrBits : int { ERR_BUCKET = 1, ERR_TILE = 2 };

constexpr int kMaxBatch = 64;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;
constexpr int kSplitK = 16;        // K-splits of an MFMA gate/up tile group
constexpr int kPairsPerGemvTile = 4;
constexpr int kPairsPerMfmaTile = 64;

// Router GEMV + top-k + routing weights + bucketing (one launch).
struct RouterArgs {
    const uint16_t* x;      // bf16 [B][H]
    const uint16_t* wr;     // bf16 [E][H]
    const float* bias;      // fp32 [E] or null
    float* z;               // fp32 [B][E] logits (workspace)
    int32_t* topk_idx;      // [B][k]
    float* topk_w;          // [B][k]
    int32_t* meta;
    int32_t* act_e;         // [max_act]   active expert ids, ascending
    int32_t* act_off;       // [max_act+1] slot offsets of each active expert
    int32_t* perm;          // [B*k]       slot -> pair id (token*k + j)
    int32_t H, E, k, B;
    int32_t score_fn, renormalize;
    float routed_scale;
    int32_t mfma_min_tokens; // experts with at least this many tokens use MFMA tiles (0 = never)
    int32_t tiles_per_expert;
    int32_t mfma_tiles_per_expert;
};

// Grouped gate/up projection + SiLU*up for a list of experts.
struct GateUpArgs {
    const uint16_t* x;       // bf16 [B][H]
    const uint16_t* w;       // bf16 [n_exp][2n][H]: gate rows then up rows per expert
    long long expert_stride; // elements between consecutive experts (2n*H)
    const int32_t* n_act;    // device: number of entries in the work list
    const int32_t* act_e;    // expert id per entry
    const int32_t* act_off;  // slot range per entry
    const int32_t* perm;     // slot -> pair id
    int32_t pair_div;        // token = pair / pair_div
    float* h;                // fp32 [slots][n] output
    float* g_acc;            // fp32 [slots][2n] split-K partials (zero between uses)
    uint32_t* tile_cnt;      // per (entry, row block) arrival counters (zero between uses)
    int32_t* meta;
    int32_t H, n;
    int32_t tiles_per_expert;   // grid.x = max entries * tiles_per_expert
    int32_t mfma_min_tokens;    // 0: GEMV only
    int32_t ksplit;             // K-splits per MFMA row block
    int32_t kslice;             // K elements per split (multiple of 32)
};

// Down projection + routing-weighted combine + shared expert + residual.
struct DownArgs {
    const uint16_t* x;       // bf16 [B][H] (residual)
    const uint16_t* w2;      // bf16 [E][H][I]
    const uint16_t* s2;      // bf16 [H][Is] or null
    const int32_t* n_act;
    const int32_t* act_e;
    const int32_t* act_off;
    const int32_t* perm;
    const float* topk_w;     // [B][k] routing weight per pair
    const float* h;          // fp32 [B*k][I] routed h, slot-major
    const float* hs;         // fp32 [B][Is] shared h
    uint16_t* out;           // bf16 [B][H]
    int32_t H, I, Is, B, k;
    int32_t add_residual;
};

// Writes the shared expert's constant work list (run once per workspace).
struct InitArgs {
    int32_t* meta;
    int32_t* sh_act_e;   // [1]
    int32_t* sh_act_off; // [2]
    int32_t* sh_perm;    // [B]
    int32_t B;
};

// A kernel and its launch shape, chosen for one argument block.
struct KernelPick {
    const void* func;
    dim3 grid;
    dim3 block;
};

KernelPick pick_init(const InitArgs& a);
KernelPick pick_router(const RouterArgs& a);
KernelPick pick_gateup(const GateUpArgs& a, int max_entries, int gemv_tokens);
KernelPick pick_down(const DownArgs& a);
int down_rows_per_block(int I);

}  // namespace moe
