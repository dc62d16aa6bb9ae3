// pkv_launch.h -- launchers of the gfx950 kernels, called by the C-ABI layer
// (api.hip) after it has validated the arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

struct DecodeArgs;

// Most layers one paged_kv_copy_blocks call takes (their pool pointers travel as
// kernel arguments: 2 KiB of pointers).
constexpr int kMaxCopyLayers = 128;

hipError_t launch_decode_g1(const DecodeArgs &a, int dtype, int block_size, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeArgs &a, int dtype, int block_size,
                              hipStream_t stream);
// Shared-prefix pass over n_items (query tile, KV head, prefix partition) items.
hipError_t launch_prefix_mfma(const DecodeArgs &a, int n_items, int dtype, int block_size,
                              hipStream_t stream);
// Decode over slotted segment lists (one work-group per (sequence, KV head)).
hipError_t launch_slotted_mfma(const DecodeArgs &a, int dtype, int block_size,
                               hipStream_t stream);
// Shared-prefix decode in one pass over n_items (query tile, KV head) items.  A
// tile is kPrefixHalves halves of 16 query columns, each half floor(16 / G)
// member sequences (tuning knob: 1 or 2).
#ifndef PKV_PREFIX_HALVES
#define PKV_PREFIX_HALVES 2
#endif
constexpr int kPrefixHalves = PKV_PREFIX_HALVES;
hipError_t launch_prefix_fused_mfma(const DecodeArgs &a, int n_items, int dtype, int block_size,
                                    hipStream_t stream);
// Slotted decode over n_items (query tile, KV head) items, tiles as for the
// one-pass shared-prefix kernel; a tile's sub-tile list must fit in
// kSlottedTileSubs descriptors (members x max_segments x ceil(B / 16)).
constexpr int kSlottedTileSubs = 1024;
hipError_t launch_slotted_tiled_mfma(const DecodeArgs &a, int n_items, int dtype, int block_size,
                                     hipStream_t stream);
hipError_t launch_reduce(void *out, const float *part_o, const float *part_lse,
                         const int32_t *lens, int num_seqs, int num_q_heads, int partition_size,
                         int max_partitions, int dtype, hipStream_t stream);
hipError_t launch_append(void *k_pool, void *v_pool, const void *k_new, const void *v_new,
                         const int32_t *tables, const int32_t *lens, int64_t *slot_out,
                         int num_seqs, int num_kv_heads, int block_size, int width,
                         hipStream_t stream);
hipError_t launch_append_tokens(void *k_pool, void *v_pool, const void *k_src,
                                const void *v_src, const int64_t *cu, const int32_t *start_pos,
                                const int32_t *tables, int num_runs, int64_t total_tokens,
                                int num_kv_heads, int block_size, int width, hipStream_t stream);
// Work-groups launch_append_tokens uses for total_tokens rows (and the rows per
// group it picks).
int64_t append_tokens_groups(int64_t total_tokens, int num_kv_heads, int *rows_per_group);
// Slot copies ([num_copies][5] device tuples) over every layer's K and V pools.
hipError_t launch_copy_slots(void *const *k_pools, void *const *v_pools, int num_layers,
                             const int32_t *copies, int num_copies, int num_kv_heads,
                             int block_size, hipStream_t stream);
hipError_t launch_copy_blocks(void *const *k_pools, void *const *v_pools, int num_layers,
                              const int32_t *src, const int32_t *dst, int num_pairs,
                              int64_t slab_elems, hipStream_t stream);

// Debug check of the caller contract on device data (PKV_DEBUG_CHECK=1): returns
// 0 when lens/tables are valid, a negative PKV status otherwise.  Synchronises.
int debug_check_tables(const int32_t *tables, const int32_t *lens, int num_seqs, int width,
                       int block_size, int64_t num_blocks, hipStream_t stream);
int debug_check_runs(const int64_t *cu, const int32_t *start_pos, const int32_t *tables,
                     int num_runs, int64_t total_tokens, int width, int block_size,
                     int64_t num_blocks, hipStream_t stream);
int debug_check_groups(const int32_t *group_cu, const int32_t *prefix_lens,
                       const int32_t *lens, int num_groups, int num_seqs, int extra,
                       hipStream_t stream);
int debug_check_segments(const int32_t *segs, const int32_t *nsegs, int num_seqs, int max_segs,
                         int block_size, int64_t num_blocks, hipStream_t stream);
int debug_check_copies(const int32_t *src, const int32_t *dst, int num_pairs,
                       int64_t num_blocks, hipStream_t stream);
int debug_check_slot_copies(const int32_t *copies, int num_copies, int block_size,
                            int64_t num_blocks, hipStream_t stream);
int debug_check_order(const int32_t *order, int num_seqs, hipStream_t stream);

}  // namespace pkv
