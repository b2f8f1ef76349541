// Host-side launch descriptors passed from the C ABI layer to each kernel file.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// The checked build (-DPA_CHECKED=1): kernels test the block ids, slots and context lengths
// they are handed against the pool and the tables, count a breach in a device error word
// (the kErr* bits) and go on with a safe value (block 0, a skipped row, a clipped length),
// so a broken caller contract is reported instead of reading or writing outside the pools.
// The release build compiles none of it.
#ifndef PA_CHECKED
#define PA_CHECKED 0
#endif
constexpr bool kChecked = PA_CHECKED != 0;
enum : uint32_t { kErrSlot = 1u, kErrBlock = 2u, kErrLength = 4u, kErrPair = 8u };

struct WriteArgs {
  const void* k;
  const void* v;
  const int32_t* slots;
  void* k_cache;
  void* v_cache;
  int32_t num_tokens;
  int32_t row_elems;   // H_kv * head_dim
  int32_t mode;        // 0 bf16 copy, 1 f32 copy, 2 bf16 -> e4m3, 3 f32 -> e4m3, 4 bf16 -> int8, 5 f32 -> int8
  float inv_k, inv_v;  // fp32(1 / scale) for e4m3 and int8 pools
  int64_t num_slots;   // num_blocks * block_size (checked build)
  uint32_t* err;       // device error word (checked build; nullptr otherwise)
};

// Storage formats, numbered as pa_dtype in include/pa.h.
enum Fmt : int32_t { kF32 = 0, kBf16 = 1, kE4m3 = 2, kInt8 = 3 };

struct DecodeArgs {
  const void* q;             // [B, H_q, D]
  const uint8_t* k_cache;    // [num_blocks, bs, H_kv, D]
  const uint8_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_m;               // [B, H_q, max_parts]
  float* ws_l;               // [B, H_q, max_parts]
  float* ws_o;               // [B, H_q, max_parts, D]
  void* out;                 // [B, H_q, D], q's format
  int64_t row_bytes;         // H_kv * D * elem
  int64_t block_bytes;       // bs * row_bytes
  int32_t num_seqs, num_q_heads, num_kv_heads, group, head_dim;
  int32_t block_size, log2_bs, bt_stride, max_parts, partition_tokens;
  int32_t heads_per_wg, head_groups;
  int32_t q_fmt, kv_fmt;
  float qk_scale;            // scale * log2(e) * k_scale
  float v_scale;
  int32_t dense;             // 1: workgroup ids number only existing (sequence, partition) pairs
  int32_t waves_per_head;    // matrix-core path: waves sharing one KV head's partition (1, 2 or 4)
  // Appended token (matrix-core grid kernel only; k_new == nullptr: none): bf16 rows
  // [B, H_kv, D] written, in the pool's format, at position context_lens[b] - 1.
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint8_t* k_cache_w;        // the pools, writable (same addresses as k_cache, v_cache)
  uint8_t* v_cache_w;
  float inv_k, inv_v;        // fp32(1 / scale) for one-byte pools
  int64_t num_blocks;        // checked build: the pool's block count
  uint32_t* err;             // checked build: device error word (nullptr otherwise)
};

// Launches with at most this many partitions per sequence merge with one 16-lane row per
// query head (merge_rows.hpp); longer ones use the merge kernel's partition-parallel
// schedule.
#ifndef PA_ROW_MERGE_MAX_PARTS
#define PA_ROW_MERGE_MAX_PARTS 16
#endif
constexpr int kRowMergeMaxParts = PA_ROW_MERGE_MAX_PARTS;

// Partitions longer than 256 tokens are split among several waves of one workgroup
// (matrix-core path), whose pieces are combined through LDS.
constexpr int kMaxPartitionTokens = 1024;
constexpr int kMaxWavesPerHead = 4;
constexpr int kCombineO = 4 * 64 * 8;   // floats of one wave's O registers (4 rows r, 64 lanes, up to 8 columns)
__host__ __device__ constexpr int combine_floats(int waves) { return 32 * waves + (waves - 1) * kCombineO; }

// Row of the workspace pieces of (sequence b, partition j, query head h): the
// pieces are laid out partition-major, m / l [B, J, H] and o [B, J, H, D], so the
// heads of one partition -- written together by one workgroup -- are contiguous.
__host__ __device__ inline int64_t piece_row(int b, int j, int h, int max_parts, int num_q_heads) {
  return ((int64_t)b * max_parts + j) * num_q_heads + h;
}

struct MergeArgs {
  const float* ws_m;
  const float* ws_l;
  const float* ws_o;
  const int32_t* context_lens;
  void* out;
  int32_t num_seqs, num_q_heads, head_dim, max_parts, partition_tokens, out_fmt;
};

struct CopyArgs {
  uint8_t* k_cache;
  uint8_t* v_cache;
  const int32_t* src;        // [num_pairs] physical block ids
  const int32_t* dst;
  int64_t num_blocks;
  int64_t block_bytes;       // bs * H_kv * D * elem, a multiple of 16
  int64_t chunks;            // block_bytes / 16
  int64_t layer_bytes;       // multi-layer pools: distance between layers' pools (0 for one layer)
  int32_t num_pairs;
  int32_t num_layers;
  uint32_t* err;             // checked build: device error word (nullptr otherwise)
};

struct AttnArgs {
  const void* q;             // [num_tokens, H_q, D] bf16
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;         // [B]
  const int32_t* query_start_loc;  // [B + 1]
  void* out;                 // [num_tokens, H_q, D] bf16
  int64_t row_bytes, block_bytes;
  int32_t num_tokens, num_seqs, num_q_heads, head_dim, log2_group;
  int32_t block_size, log2_bs, bt_stride, max_query_len;
  int32_t num_kv_heads, kv_fmt;
  float qk_scale, v_scale;
  int64_t num_blocks;        // checked build: the pool's block count
  uint32_t* err;             // checked build: device error word (nullptr otherwise)
};

struct SlotArgs {
  const int32_t* block_tables;
  int32_t* seq_lens;               // advanced in place when `advance` is set
  const int32_t* query_start_loc;  // NULL: one new token per sequence, row b
  int32_t* slot_mapping;
  int32_t num_seqs, num_tokens, bt_stride, block_size, log2_bs, advance;
};

hipError_t launch_write_kv(const WriteArgs& a, hipStream_t stream);
hipError_t launch_slot_mapping(const SlotArgs& a, hipStream_t stream);
hipError_t launch_attention_mfma(const AttnArgs& a, hipStream_t stream);
// new tokens of one request handled by one workgroup of the multi-query kernel
int attention_tokens_per_workgroup(int log2_group);
// the multi-query kernel with K/V tiles shared through LDS (bf16 pools, head_dim 128,
// blocks of 16 tokens or more)
bool attention_lds_supported(const AttnArgs& a);
int attention_lds_tokens_per_workgroup(int log2_group);
hipError_t launch_attention_lds(const AttnArgs& a, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_valu(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);

}  // namespace pa
