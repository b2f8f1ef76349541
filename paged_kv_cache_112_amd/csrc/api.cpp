// C ABI of the paged-KV library: argument checks, workspace sizing and kernel
// dispatch.  Every check runs on the host before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/pa.h"
#include "api_internal.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace {

constexpr int32_t kDefaultPartition = 256;
// The single-call decodes on the matrix-core path take 512-token partitions from this
// context length on (half the partial outputs; measured faster on 8192- and
// 32768-token batches, slower on batches of 3,360-token contexts).
constexpr int32_t kLongContext = 4096;
constexpr int32_t kLongPartition = 512;
constexpr float kLog2e = 1.4426950408889634f;
constexpr size_t kAlign = 256;
#ifndef PA_MAX_WG_WAVES
#define PA_MAX_WG_WAVES 4
#endif
#ifndef PA_MAX_HEADS_PER_WG
#define PA_MAX_HEADS_PER_WG 4
#endif
// multi-query attention: shapes the LDS-sharing kernel covers use it
#ifndef PA_ATTN_LDS
#define PA_ATTN_LDS 1
#endif

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int32_t log2i(int64_t x) {
  int32_t r = 0;
  while ((int64_t(1) << r) < x) ++r;
  return r;
}

int32_t elem_bytes(int32_t fmt) { return fmt == PA_F32 ? 4 : fmt == PA_BF16 ? 2 : 1; }
// one-byte pools store code * per-pool scale
bool is_scaled(int32_t fmt) { return fmt == PA_FP8_E4M3 || fmt == PA_INT8; }

bool valid_partition(int32_t p) {
  return p == 16 || p == 32 || p == 64 || p == 128 || p == 256 || p == 512 || p == 1024;
}

struct Workspace {
  size_t m_off, l_off, o_off, bytes;
  int32_t parts;
};

// Returns false for invalid sizes.
bool workspace_layout(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t max_context_len,
                      int32_t partition, Workspace* w) {
  if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0 || !valid_partition(partition))
    return false;
  const int64_t parts = max_context_len <= partition ? 1 : (max_context_len + partition - 1) / partition;
  w->parts = (int32_t)parts;
  if (parts <= 1) {
    w->m_off = w->l_off = w->o_off = w->bytes = 0;
    return true;
  }
  const size_t rows = (size_t)num_seqs * (size_t)num_q_heads * (size_t)parts;
  w->m_off = 0;
  w->l_off = w->m_off + align_up(rows * 4);
  w->o_off = w->l_off + align_up(rows * 4);
  w->bytes = w->o_off + align_up(rows * (size_t)head_dim * 4);
  return true;
}

pa_status check_cache(const pa_kv_cache* c) {
  if (!c) return PA_ERR_NULL;
  if (c->num_blocks < 1 || c->num_kv_heads < 1 || c->block_size < 1) return PA_ERR_SHAPE;
  if (c->dtype != PA_F32 && c->dtype != PA_BF16 && c->dtype != PA_FP8_E4M3 && c->dtype != PA_INT8) return PA_ERR_DTYPE;
  if (!is_pow2(c->block_size) || c->block_size > 1024) return PA_ERR_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (is_scaled(c->dtype)) {
    if (!(c->k_scale > 0.f) || !(c->v_scale > 0.f) || !std::isfinite(c->k_scale) || !std::isfinite(c->v_scale))
      return PA_ERR_SHAPE;
  }
  return PA_OK;
}

struct DecodeCall {
  pa::DecodeArgs args;
  int32_t kernel;  // resolved: PA_KERNEL_VALU or PA_KERNEL_MFMA
  Workspace ws;
};

pa_status prepare_decode(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                         const void* k_cache, const void* v_cache, const pa_kv_cache* cache,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t max_context_len, float scale, void* out,
                         void* workspace, size_t workspace_bytes, int32_t partition_tokens, int32_t kernel,
                         bool whole_call, DecodeCall* call) {
  if (!q || !k_cache || !v_cache || !cache || !block_tables || !context_lens || !out) return PA_ERR_NULL;
  if (const pa_status s = check_cache(cache); s != PA_OK) return s;
  if (num_seqs < 0 || num_q_heads < 1 || max_blocks_per_seq < 1 || max_context_len < 0) return PA_ERR_SHAPE;
  if (num_q_heads % cache->num_kv_heads != 0) return PA_ERR_SHAPE;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * cache->block_size) return PA_ERR_SHAPE;
  if (!std::isfinite(scale)) return PA_ERR_SHAPE;
  if (num_seqs > 65535) return PA_ERR_UNSUPPORTED;
  const bool f32_pair = q_dtype == PA_F32 && cache->dtype == PA_F32;
  const bool bf16_q = q_dtype == PA_BF16 && cache->dtype != PA_F32;
  if (!f32_pair && !bf16_q) return PA_ERR_DTYPE;
  const int32_t group = num_q_heads / cache->num_kv_heads;
  if (kernel < PA_KERNEL_AUTO || kernel > PA_KERNEL_MFMA) return PA_ERR_UNSUPPORTED;
  int32_t k = kernel;
  if (k == PA_KERNEL_AUTO) k = f32_pair ? PA_KERNEL_VALU : PA_KERNEL_MFMA;
  // partition_tokens = 0: the two-stage calls (whose pa_merge cannot know the kernel) and
  // the vector path take 256 tokens; a whole decode on the matrix cores takes the size
  // pa_partition_tokens_for gives
  int32_t P = partition_tokens;
  if (P == 0) P = whole_call && k == PA_KERNEL_MFMA ? pa_partition_tokens_for(max_context_len) : kDefaultPartition;
  if (!valid_partition(P)) return PA_ERR_UNSUPPORTED;
  if (k == PA_KERNEL_MFMA && (f32_pair || group > 16)) return PA_ERR_UNSUPPORTED;
  if (k == PA_KERNEL_VALU && group > 8) return PA_ERR_UNSUPPORTED;
  // partitions beyond 256 tokens: matrix-core grid kernel only (several waves per KV head)
  if (P > 256 && k != PA_KERNEL_MFMA) return PA_ERR_UNSUPPORTED;
  Workspace ws;
  if (!workspace_layout(num_seqs, num_q_heads, cache->head_dim, max_context_len, P, &ws)) return PA_ERR_SHAPE;
  if (ws.bytes > 0 && (!workspace || workspace_bytes < ws.bytes)) return PA_ERR_WORKSPACE;

  pa::DecodeArgs& a = call->args;
  const int32_t esz = elem_bytes(cache->dtype);
  a.q = q;
  a.k_cache = static_cast<const uint8_t*>(k_cache);
  a.v_cache = static_cast<const uint8_t*>(v_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  uint8_t* wsb = static_cast<uint8_t*>(workspace);
  a.ws_m = ws.parts > 1 ? reinterpret_cast<float*>(wsb + ws.m_off) : nullptr;
  a.ws_l = ws.parts > 1 ? reinterpret_cast<float*>(wsb + ws.l_off) : nullptr;
  a.ws_o = ws.parts > 1 ? reinterpret_cast<float*>(wsb + ws.o_off) : nullptr;
  a.out = out;
  a.row_bytes = (int64_t)cache->num_kv_heads * cache->head_dim * esz;
  a.block_bytes = a.row_bytes * cache->block_size;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = cache->num_kv_heads;
  a.group = group;
  a.head_dim = cache->head_dim;
  a.block_size = cache->block_size;
  a.log2_bs = log2i(cache->block_size);
  a.bt_stride = max_blocks_per_seq;
  a.max_parts = ws.parts;
  a.partition_tokens = P;
  a.waves_per_head = P > 256 ? P / 256 : 1;
  a.heads_per_wg = 1;
  for (int32_t h = PA_MAX_HEADS_PER_WG; h > 1; h /= 2)
    if (cache->num_kv_heads % h == 0 && (k == PA_KERNEL_MFMA || h <= 4) && h * a.waves_per_head <= PA_MAX_WG_WAVES) {
      a.heads_per_wg = h;
      break;
    }
  a.head_groups = cache->num_kv_heads / a.heads_per_wg;
  a.q_fmt = q_dtype;
  a.kv_fmt = cache->dtype;
  const float ks = is_scaled(cache->dtype) ? cache->k_scale : 1.0f;
  a.qk_scale = scale * kLog2e * ks;
  a.v_scale = is_scaled(cache->dtype) ? cache->v_scale : 1.0f;
  a.dense = num_seqs <= pa::kDenseMaxSeqs && (int64_t)ws.parts * a.head_groups * num_seqs < INT32_MAX;
  a.k_new = nullptr;
  a.v_new = nullptr;
  a.k_cache_w = nullptr;
  a.v_cache_w = nullptr;
  a.inv_k = a.inv_v = 1.0f;
  a.num_blocks = cache->num_blocks;
  a.err = pa::checked_error_word();
  call->kernel = k;
  call->ws = ws;
  return PA_OK;
}

pa_status run_partition(const DecodeCall& c, void* stream) {
  if (c.args.num_seqs == 0) return PA_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = c.kernel == PA_KERNEL_MFMA ? pa::launch_decode_mfma(c.args, s) : pa::launch_decode_valu(c.args, s);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}


pa_status run_merge(const DecodeCall& c, void* stream) {
  if (c.args.num_seqs == 0 || c.ws.parts <= 1) return PA_OK;
  pa::MergeArgs m;
  m.ws_m = c.args.ws_m;
  m.ws_l = c.args.ws_l;
  m.ws_o = c.args.ws_o;
  m.context_lens = c.args.context_lens;
  m.out = c.args.out;
  m.num_seqs = c.args.num_seqs;
  m.num_q_heads = c.args.num_q_heads;
  m.head_dim = c.args.head_dim;
  m.max_parts = c.ws.parts;
  m.partition_tokens = c.args.partition_tokens;
  m.out_fmt = c.args.q_fmt;
  const hipError_t e = pa::launch_merge(m, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

pa_status pa::decode_in_scratch(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                                const void* k_cache, const void* v_cache, const pa_kv_cache* cache,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t max_context_len, float scale, void* out,
                                int32_t partition_tokens, int32_t kernel, uint8_t* scratch, size_t scratch_bytes,
                                void* stream) {
  if (!scratch) return PA_ERR_SCRATCH;
  DecodeCall c;
  pa_status s = prepare_decode(q, q_dtype, num_seqs, num_q_heads, k_cache, v_cache, cache, block_tables,
                               max_blocks_per_seq, context_lens, max_context_len, scale, out, scratch, scratch_bytes,
                               partition_tokens, kernel, true, &c);
  if (s == PA_ERR_WORKSPACE) return PA_ERR_SCRATCH;
  if (s != PA_OK) return s;
  s = run_partition(c, stream);
  if (s != PA_OK) return s;
  return run_merge(c, stream);
}

extern "C" {

int32_t pa_default_partition_tokens(void) { return kDefaultPartition; }

int32_t pa_partition_tokens_for(int32_t max_context_len) {
  return max_context_len >= kLongContext ? kLongPartition : kDefaultPartition;
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t max_context_len,
                                 int32_t partition_tokens) {
  Workspace ws;
  const int32_t P = partition_tokens == 0 ? kDefaultPartition : partition_tokens;
  if (!workspace_layout(num_seqs, num_q_heads, head_dim, max_context_len, P, &ws)) return 0;
  return ws.bytes;
}

pa_status pa_write_kv(const void* k, const void* v, int32_t in_dtype, int32_t num_tokens,
                      const int32_t* slot_mapping, void* k_cache, void* v_cache, const pa_kv_cache* cache,
                      void* stream) {
  if (!k || !v || !slot_mapping || !k_cache || !v_cache || !cache) return PA_ERR_NULL;
  if (const pa_status s = check_cache(cache); s != PA_OK) return s;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (cache->num_blocks * (int64_t)cache->block_size > INT32_MAX) return PA_ERR_SHAPE;
  int32_t mode;
  if (cache->dtype == PA_BF16 && in_dtype == PA_BF16) mode = 0;
  else if (cache->dtype == PA_F32 && in_dtype == PA_F32) mode = 1;
  else if (cache->dtype == PA_FP8_E4M3 && in_dtype == PA_BF16) mode = 2;
  else if (cache->dtype == PA_FP8_E4M3 && in_dtype == PA_F32) mode = 3;
  else if (cache->dtype == PA_INT8 && in_dtype == PA_BF16) mode = 4;
  else if (cache->dtype == PA_INT8 && in_dtype == PA_F32) mode = 5;
  else return PA_ERR_DTYPE;
  if (num_tokens == 0) return PA_OK;
  pa::WriteArgs a;
  a.k = k;
  a.v = v;
  a.slots = slot_mapping;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_tokens = num_tokens;
  a.row_elems = cache->num_kv_heads * cache->head_dim;
  a.mode = mode;
  a.inv_k = is_scaled(cache->dtype) ? 1.0f / cache->k_scale : 1.0f;
  a.inv_v = is_scaled(cache->dtype) ? 1.0f / cache->v_scale : 1.0f;
  a.num_slots = cache->num_blocks * (int64_t)cache->block_size;
  a.err = pa::checked_error_word();
  return pa::launch_write_kv(a, static_cast<hipStream_t>(stream)) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const pa_kv_cache* cache, const int32_t* src,
                         const int32_t* dst, int32_t num_pairs, void* stream) {
  return pa_copy_blocks_layers(k_cache, v_cache, cache, 1, src, dst, num_pairs, stream);
}

pa_status pa_copy_blocks_layers(void* k_cache, void* v_cache, const pa_kv_cache* cache, int32_t num_layers,
                                const int32_t* src, const int32_t* dst, int32_t num_pairs, void* stream) {
  if (!k_cache || !v_cache || !cache || !src || !dst) return PA_ERR_NULL;
  if (const pa_status s = check_cache(cache); s != PA_OK) return s;
  if (num_pairs < 0 || num_pairs > 65535 || num_layers < 1 || num_layers > 65535) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  pa::CopyArgs a;
  a.k_cache = static_cast<uint8_t*>(k_cache);
  a.v_cache = static_cast<uint8_t*>(v_cache);
  a.src = src;
  a.dst = dst;
  a.num_blocks = cache->num_blocks;
  a.block_bytes = (int64_t)cache->block_size * cache->num_kv_heads * cache->head_dim * elem_bytes(cache->dtype);
  a.chunks = a.block_bytes / 16;
  a.layer_bytes = a.block_bytes * cache->num_blocks;
  a.num_pairs = num_pairs;
  a.num_layers = num_layers;
  a.err = pa::checked_error_word();
  return pa::launch_copy_blocks(a, static_cast<hipStream_t>(stream)) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_paged_attention(const void* q, int32_t q_dtype, int32_t num_tokens, int32_t num_seqs,
                             int32_t num_q_heads, const void* k_cache, const void* v_cache,
                             const pa_kv_cache* cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* seq_lens, const int32_t* query_start_loc, int32_t max_query_len,
                             float scale, void* out, void* stream) {
  if (!q || !k_cache || !v_cache || !cache || !block_tables || !seq_lens || !query_start_loc || !out)
    return PA_ERR_NULL;
  if (const pa_status s = check_cache(cache); s != PA_OK) return s;
  if (num_tokens < 0 || num_seqs < 0 || num_q_heads < 1 || max_blocks_per_seq < 1 || max_query_len < 0)
    return PA_ERR_SHAPE;
  if (num_q_heads % cache->num_kv_heads != 0 || !std::isfinite(scale)) return PA_ERR_SHAPE;
  if (q_dtype != PA_BF16 || cache->dtype == PA_F32) return PA_ERR_DTYPE;
  const int32_t group = num_q_heads / cache->num_kv_heads;
  if (group > 16 || (group & (group - 1)) != 0) return PA_ERR_UNSUPPORTED;
  if (num_seqs > 65535) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0 || num_seqs == 0 || max_query_len == 0) return PA_OK;
  pa::AttnArgs a;
  const int32_t esz = elem_bytes(cache->dtype);
  a.q = q;
  a.k_cache = static_cast<const uint8_t*>(k_cache);
  a.v_cache = static_cast<const uint8_t*>(v_cache);
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.query_start_loc = query_start_loc;
  a.out = out;
  a.row_bytes = (int64_t)cache->num_kv_heads * cache->head_dim * esz;
  a.block_bytes = a.row_bytes * cache->block_size;
  a.num_tokens = num_tokens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.head_dim = cache->head_dim;
  a.log2_group = log2i(group);
  a.block_size = cache->block_size;
  a.log2_bs = log2i(cache->block_size);
  a.bt_stride = max_blocks_per_seq;
  a.max_query_len = max_query_len;
  a.num_kv_heads = cache->num_kv_heads;
  a.kv_fmt = cache->dtype;
  const float ks = is_scaled(cache->dtype) ? cache->k_scale : 1.0f;
  a.qk_scale = scale * kLog2e * ks;
  a.v_scale = is_scaled(cache->dtype) ? cache->v_scale : 1.0f;
  a.num_blocks = cache->num_blocks;
  a.err = pa::checked_error_word();
  const bool lds = PA_ATTN_LDS && pa::attention_lds_supported(a);
  const int64_t per_wg = lds ? pa::attention_lds_tokens_per_workgroup(a.log2_group)
                             : pa::attention_tokens_per_workgroup(a.log2_group);
  if (((int64_t)max_query_len + per_wg - 1) / per_wg * a.num_kv_heads > INT32_MAX) return PA_ERR_SHAPE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return (lds ? pa::launch_attention_lds(a, s) : pa::launch_attention_mfma(a, s)) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t* seq_lens,
                          const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens, int32_t block_size,
                          int32_t advance, int32_t* slot_mapping, void* stream) {
  if (!block_tables || !seq_lens || !slot_mapping) return PA_ERR_NULL;
  if (num_seqs < 0 || num_tokens < 0 || max_blocks_per_seq < 1) return PA_ERR_SHAPE;
  if (!query_start_loc && num_tokens < num_seqs) return PA_ERR_SHAPE;
  if (block_size < 1 || block_size > 1024 || (block_size & (block_size - 1)) != 0) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  pa::SlotArgs a;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.query_start_loc = query_start_loc;
  a.slot_mapping = slot_mapping;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.bt_stride = max_blocks_per_seq;
  a.block_size = block_size;
  a.log2_bs = log2i(block_size);
  a.advance = advance != 0;
  return pa::launch_slot_mapping(a, static_cast<hipStream_t>(stream)) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_decode_partition(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                              const void* k_cache, const void* v_cache, const pa_kv_cache* cache,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t max_context_len, float scale, void* out,
                              void* workspace, size_t workspace_bytes, int32_t partition_tokens, int32_t kernel,
                              void* stream) {
  DecodeCall c;
  const pa_status s = prepare_decode(q, q_dtype, num_seqs, num_q_heads, k_cache, v_cache, cache, block_tables,
                                     max_blocks_per_seq, context_lens, max_context_len, scale, out, workspace,
                                     workspace_bytes, partition_tokens, kernel, false, &c);
  if (s != PA_OK) return s;
  return run_partition(c, stream);
}

// Decode with the step's token appended by the partition kernel itself.
static pa_status prepare_append(const void* q, int32_t q_dtype, const void* k_new, const void* v_new, int32_t in_dtype,
                                int32_t num_seqs, int32_t num_q_heads, void* k_cache, void* v_cache,
                                const pa_kv_cache* cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t max_context_len, float scale, void* out,
                                void* workspace, size_t workspace_bytes, int32_t partition_tokens, bool whole_call,
                                DecodeCall* c) {
  if (!k_new || !v_new) return PA_ERR_NULL;
  const pa_status s = prepare_decode(q, q_dtype, num_seqs, num_q_heads, k_cache, v_cache, cache, block_tables,
                                     max_blocks_per_seq, context_lens, max_context_len, scale, out, workspace,
                                     workspace_bytes, partition_tokens, PA_KERNEL_MFMA, whole_call, c);
  if (s != PA_OK) return s;
  if (in_dtype != PA_BF16) return PA_ERR_DTYPE;
  if (c->args.partition_tokens < 256) return PA_ERR_UNSUPPORTED;
  pa::DecodeArgs& a = c->args;
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.k_cache_w = static_cast<uint8_t*>(k_cache);
  a.v_cache_w = static_cast<uint8_t*>(v_cache);
  a.inv_k = is_scaled(cache->dtype) ? 1.0f / cache->k_scale : 1.0f;
  a.inv_v = is_scaled(cache->dtype) ? 1.0f / cache->v_scale : 1.0f;
  return PA_OK;
}

pa_status pa_decode_partition_append(const void* q, int32_t q_dtype, const void* k_new, const void* v_new,
                                     int32_t in_dtype, int32_t num_seqs, int32_t num_q_heads, void* k_cache,
                                     void* v_cache, const pa_kv_cache* cache, const int32_t* block_tables,
                                     int32_t max_blocks_per_seq, const int32_t* context_lens,
                                     int32_t max_context_len, float scale, void* out, void* workspace,
                                     size_t workspace_bytes, int32_t partition_tokens, void* stream) {
  DecodeCall c;
  const pa_status s = prepare_append(q, q_dtype, k_new, v_new, in_dtype, num_seqs, num_q_heads, k_cache, v_cache,
                                     cache, block_tables, max_blocks_per_seq, context_lens, max_context_len, scale,
                                     out, workspace, workspace_bytes, partition_tokens, false, &c);
  if (s != PA_OK) return s;
  return run_partition(c, stream);
}

pa_status pa_decode_append(const void* q, int32_t q_dtype, const void* k_new, const void* v_new, int32_t in_dtype,
                           int32_t num_seqs, int32_t num_q_heads, void* k_cache, void* v_cache,
                           const pa_kv_cache* cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t max_context_len, float scale, void* out,
                           void* workspace, size_t workspace_bytes, int32_t partition_tokens, void* stream) {
  DecodeCall c;
  pa_status s = prepare_append(q, q_dtype, k_new, v_new, in_dtype, num_seqs, num_q_heads, k_cache, v_cache, cache,
                               block_tables, max_blocks_per_seq, context_lens, max_context_len, scale, out,
                               workspace, workspace_bytes, partition_tokens, true, &c);
  if (s != PA_OK) return s;
  s = run_partition(c, stream);
  if (s != PA_OK) return s;
  return run_merge(c, stream);
}

pa_status pa_decode(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads, const void* k_cache,
                    const void* v_cache, const pa_kv_cache* cache, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len, float scale,
                    void* out, void* workspace, size_t workspace_bytes, int32_t partition_tokens, int32_t kernel,
                    void* stream) {
  DecodeCall c;
  pa_status s = prepare_decode(q, q_dtype, num_seqs, num_q_heads, k_cache, v_cache, cache, block_tables,
                               max_blocks_per_seq, context_lens, max_context_len, scale, out, workspace,
                               workspace_bytes, partition_tokens, kernel, true, &c);
  if (s != PA_OK) return s;
  s = run_partition(c, stream);
  if (s != PA_OK) return s;
  return run_merge(c, stream);
}

pa_status pa_merge(const void* workspace, size_t workspace_bytes, int32_t num_seqs, int32_t num_q_heads,
                   int32_t head_dim, const int32_t* context_lens, int32_t max_context_len, int32_t partition_tokens,
                   int32_t out_dtype, void* out, void* stream) {
  if (!context_lens || !out) return PA_ERR_NULL;
  if (num_seqs < 0 || num_q_heads < 1 || max_context_len < 0) return PA_ERR_SHAPE;
  if (num_seqs > 65535) return PA_ERR_UNSUPPORTED;
  if (out_dtype != PA_F32 && out_dtype != PA_BF16) return PA_ERR_DTYPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  const int32_t P = partition_tokens == 0 ? kDefaultPartition : partition_tokens;
  if (!valid_partition(P)) return PA_ERR_UNSUPPORTED;
  Workspace ws;
  if (!workspace_layout(num_seqs, num_q_heads, head_dim, max_context_len, P, &ws)) return PA_ERR_SHAPE;
  if (ws.bytes > 0 && (!workspace || workspace_bytes < ws.bytes)) return PA_ERR_WORKSPACE;
  if (num_seqs == 0 || ws.parts <= 1) return PA_OK;
  const uint8_t* wsb = static_cast<const uint8_t*>(workspace);
  pa::MergeArgs m;
  m.ws_m = reinterpret_cast<const float*>(wsb + ws.m_off);
  m.ws_l = reinterpret_cast<const float*>(wsb + ws.l_off);
  m.ws_o = reinterpret_cast<const float*>(wsb + ws.o_off);
  m.context_lens = context_lens;
  m.out = out;
  m.num_seqs = num_seqs;
  m.num_q_heads = num_q_heads;
  m.head_dim = head_dim;
  m.max_parts = ws.parts;
  m.partition_tokens = P;
  m.out_fmt = out_dtype;
  return pa::launch_merge(m, static_cast<hipStream_t>(stream)) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

const char* pa_status_str(pa_status s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: inconsistent or out-of-range sizes";
    case PA_ERR_DTYPE: return "PA_ERR_DTYPE: unsupported dtype combination";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: unsupported head_dim, block_size, partition or kernel";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: kernel launch failed";
    case PA_ERR_SCRATCH: return "PA_ERR_SCRATCH: the call needs more than the library's static scratch holds";
  }
  return "unknown pa_status";
}

}  // extern "C"
