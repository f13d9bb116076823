// internal.h -- launch plans and launcher declarations shared between the
// C-ABI layer (api.cpp) and the kernel files.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/attn.h"

namespace attn {

// Tile classification codes, one byte per (workgroup query block, 64-key tile).
enum : uint8_t { TILE_SKIP = 0, TILE_MASKED = 1, TILE_OPEN = 2 };

// How one attn_prefill call is cut into workgroups.  A workgroup owns one
// batch item, one KV head, `heads_per_wg` consecutive query heads of that KV
// head and `rows_per_wg` consecutive query rows: rows_per_wg * heads_per_wg
// query slots, 32 per query wave; with head_dim 512 two waves share the 32
// slots, one per 256-column slice of the head dimension.
struct PrefillPlan {
    int head_dim, slices, slice_dim;
    int rows_per_wg, heads_per_wg, query_waves, waves;
    int row_blocks, head_groups;      // per batch item: ceil(rows/rows_per_wg), n_kv_heads * g / heads_per_wg
    int kv_tiles;                     // ceil(kv_len / 64)
    int blk_stride;                   // bytes per row of tile codes (kv_tiles rounded up to 4)
    int splits, tiles_per_split;      // KV range split across workgroups
    int wide;                         // head_dim 512 in 128-slot workgroups, each wave over the whole head dim
    int narrow;                       // head_dim <= 256 in 128-slot workgroups of eight 16-slot waves
    size_t status_offset;             // status block (ATTN_PREFILL_STATUS_BYTES) at the workspace start
    size_t blk_bytes, blk_offset;     // tile codes [batch][blk heads][row_blocks][blk_stride]
    size_t part_offset, part_bytes;   // split partials: O [splits][batch][n_heads][rows][D] f32
    size_t ml_offset, ml_bytes;       // split partials: (m, l) [splits][batch][n_heads][rows] float2
    // Paired row blocks (masked calls, no KV split): row blocks p and row_blocks-1-p
    // share two workgroups that split their unskipped tiles evenly.
    int pairing;
    size_t pair_cnt_offset, pair_cnt_bytes;    // u32 [batch][head_groups][row_blocks/2][arrivals, ready]
    size_t pair_ml_offset, pair_ml_bytes;      // float2 [pairs][2 sides][slots]
    size_t pair_part_offset, pair_part_bytes;  // f32 [pairs][2 sides][slots][D]
    size_t workspace_bytes;
};

int plan_prefill(const attn_prefill_params *p, PrefillPlan *plan);
hipError_t launch_prefill(const attn_prefill_params *p, const PrefillPlan *plan, const void *q,
                          const void *k, const void *v, const void *mask, float *o, void *ws,
                          hipStream_t stream);

struct DecodePlan {
    int head_dim, group;              // query heads per KV head
    int heads_per_wg;                 // query heads one workgroup serves
    int hgroups;                      // workgroup head groups per sequence
    int per, per_max;                 // tiles per range: at least per, at most per_max
    int max_splits;                   // pieces per unit at most
    int64_t grid;                     // workgroups (the ones the device runs at once)
    size_t part_offset, part_bytes;   // O partials [batch][n_heads][max_splits][D] f32
    size_t ml_offset, ml_bytes;       // (m, l) [batch][n_heads][max_splits] float2
    size_t workspace_bytes;
};

int plan_decode(const attn_decode_params *p, DecodePlan *plan);
// Address of this device's ATTN_DECODE_SCRATCH_BYTES scratch array (looked up once per device).
int decode_scratch(void **ptr);

// Multi-token paged attention: the decode line with up to 64 query columns
// (heads x tokens) per workgroup.
constexpr int kMultiMinTilesPerWorkgroup = 16;
constexpr int kMultiMaxTilesPerWorkgroup = 128;
constexpr int kMultiDefaultWorkgroups = 256;  // without a device query
constexpr int kMultiMaxTokens = 64;

struct MultiPlan {
    int group, heads_per_wg, qgroups, hgroups;
    int ctx_cap, target, max_splits;
    int64_t grid;
    size_t ml_offset, ml_bytes;        // (m, l) [batch][max_tokens][n_heads][max_splits] float2
    size_t part_offset, part_bytes;    // O partials [batch][max_tokens][n_heads][max_splits][head_dim] f32
    size_t npiece_offset, npiece_bytes;  // pieces per unit [batch][hgroups] i32
    size_t workspace_bytes;
};

int plan_paged_prefill(const attn_paged_prefill_params *p, MultiPlan *plan);
hipError_t launch_paged_prefill(const attn_paged_prefill_params *p, const MultiPlan *plan, const float *q,
                                const void *k_pool, const void *v_pool, const int32_t *page_table,
                                const int32_t *query_lens, const int32_t *position_starts, float *o, void *ws,
                                hipStream_t stream);
hipError_t launch_paged_decode(const attn_decode_params *p, const DecodePlan *plan, const float *q,
                               const void *k_pool, const void *v_pool, const int32_t *page_table,
                               const int32_t *context_lens, float *o, void *ws, hipStream_t stream);

// Pack-free block verify: workgroups per (split, KV head x query-head group,
// lane); the splits per lane are sized on the device from the cache lengths.
constexpr int kVerifyTileKeys = 32;          // keys per tile
constexpr int kVerifyMaxSplits = 32;          // splits per lane at most (bounds the workspace)
constexpr int kVerifyDefaultWorkgroups = 256;  // busy workgroups the split aims for without a device query
constexpr uint32_t kVerifyMaxWindow = 1u << 24;

struct VerifyPlan {
    int group, heads_per_wg, qgroups;  // query heads per KV head, per workgroup, groups per KV head
    int max_splits, target_wgs;
    size_t ml_offset, ml_bytes;        // (m, l) [lanes][q_heads][rows][max_splits] float2
    size_t part_offset, part_bytes;    // O partials [lanes][q_heads][rows][max_splits][head_dim] f32
    size_t workspace_bytes;
};

int plan_verify(const dflash_params *p, VerifyPlan *plan);
hipError_t launch_dflash_verify(const dflash_params *p, const VerifyPlan *plan, float scale,
                                const uint16_t *ring_k, const uint16_t *ring_v, const float *cur_q,
                                const float *cur_k, const float *cur_v, const uint32_t *cache_lengths,
                                const uint32_t *write_positions, float *o, void *ws, hipStream_t stream);

hipError_t launch_paged_prepare(const attn_paged_prepare_params *p, const float *q_raw, const float *k_raw,
                                const float *v_raw, const float *q_norm, const float *k_norm,
                                const int32_t *page_table, const int32_t *query_lens,
                                const int32_t *position_starts, float *q_out, void *k_pool, void *v_pool,
                                hipStream_t stream);

hipError_t launch_dflash_pack(const dflash_params *p, const uint16_t *ring_k, const uint16_t *ring_v,
                              const float *cur_q, const float *cur_k, const float *cur_v,
                              const uint32_t *cache_lengths, const uint32_t *write_positions,
                              uint16_t *packed_q, uint16_t *packed_k, uint16_t *packed_v,
                              hipStream_t stream);
hipError_t launch_dflash_mask(const dflash_params *p, const uint32_t *cache_lengths, uint16_t *mask,
                              hipStream_t stream);
hipError_t launch_dflash_commit(const dflash_params *p, const float *new_k, const float *new_v,
                                const uint32_t *commit_counts, const uint32_t *write_positions,
                                uint16_t *ring_k, uint16_t *ring_v, hipStream_t stream);
hipError_t launch_dflash_mask_rows(uint32_t lanes, uint32_t rows, uint32_t hidden,
                                   const uint16_t *mask_embedding, float *draft_input,
                                   hipStream_t stream);

}  // namespace attn
