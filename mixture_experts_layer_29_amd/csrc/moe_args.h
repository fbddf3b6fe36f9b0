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
    // single-launch layer (all re-armed to 0 by the last workgroup to exit)
    M_NEXT = 6,        // next dynamically claimed task
    M_SGU_DONE = 7,    // shared gate/up tiles done
    M_SDOWN_DONE = 8,  // shared down row blocks done
    M_GU_DONE = 9,     // routed gate/up tiles done
    M_SEL = 10,        // routing published
    M_EXIT = 11,       // workgroups that left the task loop
    M_COUNT = 16
};

enum ErrBits : int { ERR_BUCKET = 1, ERR_TILE = 2, ERR_TIMEOUT = 4 };

constexpr int kMaxBatch = 64;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;
// K-splits of an MFMA gate/up tile group.  Measured on MI355X (Zipf-skewed
// batch 64, TP8 shard): 16 splits 305 us, 8 splits 290 us (half the fp32
// partial atomics; two load rounds per tile), 4 splits 319 us.
constexpr int kSplitK = 8;
constexpr int kPairsPerGemvTile = 4;
constexpr int kPairsPerMfmaTile = 64;
constexpr int kMaxGemvUnits = 16;  // 16-byte units per lane held in registers by a GEMV wave
constexpr int kGemvLdsBytes = 60 * 1024;  // x staging budget of a GEMV workgroup
constexpr int kXStage = 4;                 // x units per thread requested ahead of a GEMV's weights
constexpr int kDownHStage = 32 * 1024;  // LDS bytes for a staged batch of h rows in down

// Router + top-k + routing weights + bucketing.  Batches up to 4 use one
// launch (GEMV, last workgroup selects and buckets); larger batches use an
// MFMA split-K launch accumulating into zacc and a per-token top-k launch
// whose last workgroup buckets.
struct RouterArgs {
    const uint16_t* x;      // bf16 [B][H]
    const uint16_t* wr;     // bf16 [E][H]
    const float* bias;      // fp32 [E] or null
    float* z;               // fp32 [B][E] logits (workspace)
    float* zacc;            // fp32 [nzpart][B][E] partial logits for a later top-k launch
    int32_t nzpart;         // partial slices in zacc (1: full sums)
    int32_t* topk_idx;      // [B][k]
    float* topk_w;          // [B][k]
    int32_t* meta;
    int32_t* act_e;         // [max_act]   active expert ids (ascending; above batch 4 those with
                            //             >= mfma_min_tokens tokens first, each class ascending)
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
    int32_t n_experts;          // valid expert ids: [0, n_experts)
    int32_t max_slots;          // valid slots: [0, max_slots)
    int32_t tiles_per_expert;   // grid.x = max entries * tiles_per_expert
    int32_t mfma_min_tokens;    // 0: GEMV only
    int32_t ksplit;             // K-splits per MFMA row block
    int32_t kslice;             // K elements per split (multiple of 32)
};

// Down projection + routing-weighted combine + shared expert + residual,
// output-stationary (the single launch's down tasks, rows x all entries).
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
    float* s_out;            // fp32 [B][H] shared-expert output (single-launch layer)
    int32_t H, I, Is, B, k;
    int32_t add_residual;
    int32_t n_experts;
    int32_t h_in_lds;        // 1: all of h and hs are staged in LDS at kernel start
};

// Down projection, expert-major (staged launches, larger batches): one
// workgroup per (entry, block of 256 output rows), entries = active routed
// experts then the shared expert's Is/I column blocks.  Each writes fp32
// partial rows per pair (or per shared block and token); combine_kernel then
// sums them in a fixed order (routing weights, shared blocks, residual) into
// bf16.
struct DownXArgs {
    const uint16_t* x;       // bf16 [B][H] (residual)
    const uint16_t* w2;      // bf16 [E][H][I]
    const uint16_t* s2;      // bf16 [H][Is] or null
    const int32_t* n_act;
    const int32_t* act_e;
    const int32_t* act_off;
    const int32_t* perm;     // slot -> pair id
    const float* topk_w;     // [B][k]
    const float* h;          // fp32 [B*k][I] routed h, slot-major
    const float* hs;         // fp32 [B][Is] shared h
    float* part;             // fp32 [B*k][H] per-pair partial outputs
    float* part_s;           // fp32 [nsh][B][H] per-shared-block partial outputs
    int32_t* meta;
    uint16_t* out;           // bf16 [B][H]
    int32_t H, I, Is, B, k;
    int32_t add_residual;
    int32_t n_experts;
    int32_t max_act;         // routed entries of the grid
    int32_t nsh;             // shared column blocks (Is / I, 0 without a shared expert)
    int32_t mfma_min_tokens; // entries with at least this many tokens use MFMA (0: never)
};

// First launch of a layer: the router (GEMV for batch <= 4, split-K MFMA
// above) and, in its trailing workgroups, the shared expert's gate/up rows,
// which need only x and so overlap routing without a second stream.
struct FrontArgs {
    RouterArgs r;
    GateUpArgs s;           // shared expert work list (ignored when shared_blocks == 0)
    int32_t router_blocks;  // workgroups [0, router_blocks) run the router
    int32_t shared_blocks;  // workgroups [router_blocks, +shared_blocks) run the shared gate/up
    // dense split-K form (batch > 4): tiles of 16 rows x one of `dks` K splits
    // of `dsteps` 32-wide steps; router partials to r.zacc, shared gate/up
    // partials [dks][B][2 Is] to `spart`
    float* spart;
    int32_t* sync_clear;    // words zeroed by workgroup 0 (the fused experts launch's sync block) or null
    int32_t sync_words;
    int32_t dks, dsteps;
    int32_t dks_r, dsteps_r;  // the router tiles' K splits and steps (fewer partials for the top-k launch)
};

// Top-k launch (batch > 4): workgroups [0, sel_blocks) select and bucket
// (four tokens each); the rest reduce the shared expert's gate/up partials
// to h_s = silu(sum gate) * sum up, one (token, row) per thread.
struct TopkArgs {
    RouterArgs r;
    const float* spart;     // fp32 [nspart][B][2 Is] or null
    float* hs;              // fp32 [B][Is]
    int32_t Is, nspart;
    int32_t sel_blocks;
};

// Gate/up launch that selects for itself (batch <= 4; the front launch before
// it writes the logits z with the bias added): every workgroup reads z,
// selects the top-k of all B tokens (one wave per token) and buckets the
// pairs in LDS, then runs the tile of the active expert its index maps to;
// workgroups [0, shared_pairs) first compute one of the shared expert's
// gate/up row pairs, whose weights stream during the selection.  Workgroup 0 also writes the routing rows and the
// work lists for the down launch and the caller.  Every workgroup computes the
// same lists, so there is no hand-off inside the launch.
struct SelGateUpArgs {
    RouterArgs r;           // logits (r.z) and the routing / work-list outputs
    GateUpArgs g;           // routed experts
    GateUpArgs s;           // shared expert (row pairs [0, shared_pairs), one per workgroup)
    int32_t shared_pairs;   // 0: the shared gate/up runs elsewhere
};

// Whole layer in one launch (batch <= 4): tasks in dependency order
// [router rows][shared gate/up][shared down][routed gate/up][routed down];
// the first two groups are assigned by block index, the rest claimed in order.
struct LayerArgs {
    FrontArgs f;            // router (f.r) and shared gate/up list (f.s)
    GateUpArgs g;           // routed gate/up
    DownArgs d;             // down (shared part to d.s_out, then routed + finalize)
    int32_t n_router;       // router tasks: 4 rows each
    int32_t n_sgu;          // shared gate/up tasks
    int32_t sgu_expect;     // shared gate/up tasks that do work
    int32_t n_sdown;        // shared down tasks (row blocks)
    int32_t n_gu;           // routed gate/up tasks (max entries * tiles per expert)
    int32_t n_down;         // routed down tasks (row blocks)
    int32_t shared_mfma;    // shared expert on MFMA tiles
};

// Batch 1 and 2 in two launches: front_split_kernel (router logits z and the
// shared expert's h, one row / row pair per workgroup; it also clears the
// counters of the sync block below) and fused_experts_kernel, one grid of
// co-resident workgroups (the host sizes it from the occupancy):
//   select    waves t < B of every workgroup select token t's top-k from z
//             (no hand-off);
//   gate/up   the B k (token, expert) pairs are the units; workgroup b
//             computes tiles b, b + G, ... (four row pairs each, one per
//             wave), stores their h rows, then counts each tile on its pair's
//             counter; the tile that completes pair p raises p's flag in every
//             replica of the flag block;
//   down      workgroup b owns output rows [b*R, b*R + R): it requests its W2
//             rows of the B k pairs once its h is counted (its S2 rows before
//             the selection), accumulates each pair as soon as that pair's
//             flag is up (per-pair readiness), in a fixed order per token,
//             adds the shared expert and the residual and writes the rows in
//             bf16.
// Sync block (int32 words, each counter and flag replica on its own 256-byte
// line): counter of pair p at word 64 p; flag replica r at word
// 64 (kMaxFusedPairs + r), flag of pair p its word p.
constexpr int kSyncLineWords = 64;
constexpr int kFlagReplicas = 16;
constexpr int kMaxFusedPairs = 32;
constexpr int kSyncWords = (kMaxFusedPairs + kFlagReplicas) * kSyncLineWords;
struct FusedArgs {
    const uint16_t* x;       // bf16 [B][H]
    const float* z;          // fp32 [B][E] logits (bias included), from the front launch
    const float* hs;         // fp32 [B][Is] shared h, from the front launch
    const uint16_t* w13;     // bf16 [E][2I][H]
    const uint16_t* w2;      // bf16 [E][H][I]
    const uint16_t* s2;      // bf16 [H][Is] or null
    uint16_t* out;           // bf16 [B][H]
    float* h;                // fp32 [B k][I] routed h, by pair (token-major, selection rank)
    int32_t* sync;           // [kSyncWords], counters zero at launch (cleared by the front launch)
    // routing results for the caller (written by workgroup 0)
    int32_t* topk_idx;       // [B][k]
    float* topk_w;           // [B][k]
    int32_t* meta;
    int32_t* act_e;
    int32_t* act_off;
    int32_t* perm;
    int32_t H, E, k, I, Is, B;
    int32_t score_fn, renormalize;
    float routed_scale;
    int32_t add_residual;
    int32_t rows;            // R: output rows per workgroup (<= 16)
    // cross-layer prefetch: bytes read (and dropped) during the selection so
    // the next layer's launches find them in the Infinity Cache; null = none
    const uint16_t* pf_a;    // the next layer's router weight
    long long pf_a_units;    // 16-byte units
    const uint16_t* pf_b;    // the next layer's shared expert weights
    long long pf_b_units;
};
constexpr int kPrefetchUnits = 16;  // 16-byte prefetch loads per lane (the non-selecting waves)
constexpr int kFusedRowThreads = 16;   // threads per output row in the down phase
constexpr int kFusedMaxUnits = 32;     // W2 16-byte units per thread
constexpr int kFusedMaxSUnits = 4;     // S2 16-byte units per thread

// Writes the shared expert's constant work list (once per workspace, or before
// every allocation-free forward); with zero_meta it also clears the meta block
// and the words [zero, zero + zero_words) -- the split-K partials and tile
// counters, which must start at zero -- with plain stores (no memset node).
struct InitArgs {
    int32_t* meta;
    int32_t* sh_act_e;   // [1]
    int32_t* sh_act_off; // [2]
    int32_t* sh_perm;    // [B]
    int32_t B;
    int32_t zero_meta;
    uint32_t* zero;      // 16-byte aligned, or null
    long long zero_words;// a multiple of 4
};

// A kernel and its launch shape, chosen for one argument block.
struct KernelPick {
    const void* func;
    dim3 grid;
    dim3 block;
    size_t lds;  // dynamic LDS bytes
};

KernelPick pick_init(const InitArgs& a);
// Launch shape of the batch-1 single launch for this shape (grid = the
// workgroups it needs), given how many of its workgroups fit on the device at
// once; func is null where it does not apply or does not fit.
KernelPick pick_fused_experts(const FusedArgs& a, int resident_wgs);

// Device scratch of the allocation-free forward: a static array, one copy per
// GPU, held until the process ends (moe_scratch.hip).
constexpr size_t kScratchBytes = 48u << 20;
// The current device's copy (its device address, looked up once per device).
hipError_t scratch_for_current_device(void** ptr, size_t* bytes);
// Front launch: batch <= 4 (router GEMV, with top-k + bucketing in the last
// workgroup when select_in_router) or larger (router MFMA).  Otherwise top-k
// and bucketing follow in pick_topk's launch.  shared_tb: 0 when the shared
// expert uses MFMA tiles, else its GEMV token count.
KernelPick pick_front(const FrontArgs& f, bool small_router, bool select_in_router, int shared_tb);
int front_router_blocks(const RouterArgs& a);  // batch <= 4: four router rows per workgroup
KernelPick pick_topk(const TopkArgs& a);
// Dense split-K front (router + shared gate/up partials) for batch > 4.
KernelPick pick_front_dense(const FrontArgs& f);
// Front launch of the select-in-gate/up form (batch <= 4): f.router_blocks
// (= E) router rows, then f.shared_blocks (= Is or 0) shared gate/up row
// pairs, one per workgroup, K split over its four waves.
KernelPick pick_front_split(const FrontArgs& f);
// Gate/up launch that selects for itself (batch <= 4).
KernelPick pick_gateup_select(const SelGateUpArgs& a, int max_entries);
KernelPick pick_gateup(const GateUpArgs& a, int max_entries, int gemv_tokens);
constexpr int kDownXRows = 256;           // output rows per expert-major down tile
constexpr int kDownXLds = 64 * 1024;      // LDS for a down tile's staged h rows
KernelPick pick_down_x(const DownXArgs& a);
KernelPick pick_combine(const DownXArgs& a);
// Output-stationary down (down_rows over all entries) for small batches.
KernelPick pick_down(const DownArgs& a);
// Output-stationary down for batch <= 4 on v_dot2 with h in LDS as bf16 hi/lo
// pairs; func is null where it does not apply (then pick_down).
constexpr int kDownOsLds = 60 * 1024;
KernelPick pick_down_os(const DownArgs& a);
size_t down_os_lds_bytes(int B, int k, int I, int Is);
// Single-launch layer; func is null when the shape has no instantiation.
KernelPick pick_layer(const LayerArgs& L, size_t lds_bytes);
int down_rows_per_block(int I);
size_t down_h_lds_bytes(int B, int k, int I, int Is);

}  // namespace moe
