/*
 * pa.h -- C ABI of the MI355X (gfx950) paged-KV hot path.
 *
 * Two operations, as the LLM stack book "4.6 PagedAttention & KV-Cache Memory
 * Management" states the problem (sections "Block Tables, the Allocator &
 * Copy-on-Write", "The PagedAttention Kernel", "From Python bookkeeping to the
 * tensors the kernel actually takes"):
 *
 *   pa_write_kv  -- scatter each new token's K and V rows into the block pools at
 *                   slot = physical_block * block_size + offset;
 *   pa_decode    -- attention of one query token per sequence over its cached
 *                   tokens, softmax(scale * q . K^T) V, gathering K and V through
 *                   the sequence's block table, with grouped-query heads.
 *
 * pa_decode runs in two stages that are also exported on their own:
 * pa_decode_partition (per-partition softmax pieces, split-K over the sequence:
 * "Performance considerations") and pa_merge (combines the pieces).
 *
 * Conventions for every call:
 *   - Pointers named as device data are device pointers (hipMalloc / torch CUDA
 *     tensors) owned by the caller; arrays are row-major and contiguous.  The
 *     library never allocates or frees device memory and keeps no state between
 *     calls, except pa_decode_noalloc's static scratch array (64 MiB on each GPU
 *     the library's code is loaded on); calls are thread-safe, bar the overlap
 *     rule of pa_decode_noalloc.
 *   - The library links libamdhip64.so.7.  In a process that also runs torch, whose
 *     wheel ships its own HIP runtime under the file name libamdhip64.so, load torch
 *     first: this library then binds to that runtime by its soname; loaded first, it
 *     brings up a second runtime, and its launches on torch's memory and streams fail
 *     (the Python binding imports torch before it loads the library).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *     work: no host synchronization, no allocation, so they can be captured in
 *     a HIP graph.
 *   - A host-checkable contract violation returns a nonzero pa_status before
 *     anything is enqueued and leaves all outputs untouched.  A failed launch
 *     returns PA_ERR_HIP.
 *   - Invalid *data* is undefined behaviour: a slot or block id outside the
 *     pool, context_lens[b] > max_blocks_per_seq * block_size, context_lens[b] >
 *     max_context_len (the decode then covers only the first
 *     ceil(max_context_len / P) partitions of that sequence, and never writes
 *     outside the workspace), duplicate slots in one write, or an `out` that
 *     aliases an input.
 *
 * Pool layout (both pools, same shape and format):
 *   [num_blocks, block_size, num_kv_heads, head_dim]
 * (LLM stack book, "Block Tables, the Allocator & Copy-on-Write"; ai-infra-
 * handbooks "Paged KV cache", section "Implementation").  Viewed as
 * [num_blocks * block_size, num_kv_heads * head_dim] it is slot-major.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = 2,       /* inconsistent or out-of-range sizes */
  PA_ERR_DTYPE = 3,       /* unsupported dtype or dtype combination */
  PA_ERR_UNSUPPORTED = 4, /* supported dtypes, unsupported head_dim / block_size / partition size */
  PA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than pa_decode_workspace_bytes() */
  PA_ERR_HIP = 6,         /* the HIP runtime reported an error when launching */
  PA_ERR_SCRATCH = 7      /* pa_decode_noalloc: the shape needs more than the static scratch */
} pa_status;

typedef enum pa_dtype {
  PA_F32 = 0,             /* IEEE binary32 */
  PA_BF16 = 1,            /* bfloat16: the upper 16 bits of a binary32 */
  PA_FP8_E4M3 = 2,        /* OCP E4M3FN (bias 7, no infinity, S.1111.111 = NaN, max 448) */
  PA_INT8 = 3             /* signed 8-bit integer code, symmetric: -127 .. 127 */
} pa_dtype;

/* Describes both pools.  k_scale / v_scale are used only for the one-byte pools
 * (PA_FP8_E4M3, PA_INT8): the real value of a stored code c is value(c) * scale,
 * one fp32 scale per pool.  The pages only say that quantizing the cache to fp8 or
 * int8 halves the bytes per element (LLM stack book, "The libraries that implement
 * this" and "Why it matters"); the per-tensor scale is this library's reading. */
typedef struct pa_kv_cache {
  int64_t num_blocks;     /* physical blocks in each pool, >= 1 */
  int32_t block_size;     /* tokens per block: a power of two, 1..1024 */
  int32_t num_kv_heads;   /* H_kv >= 1 */
  int32_t head_dim;       /* d_h: 64 or 128 */
  int32_t dtype;          /* pa_dtype of the pool elements */
  float k_scale;          /* fp8 pools: > 0 and finite */
  float v_scale;
} pa_kv_cache;

/* Slot-mapping write (reshape-and-cache).
 *
 * For every token i < num_tokens with s = slot_mapping[i] >= 0, copies row
 * k[i] (num_kv_heads * head_dim elements) to k_cache block s / block_size,
 * offset s % block_size, and likewise v[i] to v_cache (LLM stack book, "From
 * Python bookkeeping ...": the write is one indexed copy into the pool seen as
 * [num_blocks * block_size, H_kv, d_h]; "Putting It Together": divmod of the
 * slot).  A negative slot skips the token (padding).
 *
 *   k, v          device, [num_tokens, num_kv_heads, head_dim] of in_dtype
 *   in_dtype      == cache->dtype for PA_F32 / PA_BF16 pools (bit-exact copy);
 *                 PA_BF16 or PA_F32 for a PA_FP8_E4M3 pool, which stores
 *                 RNE-saturating e4m3(fp32(x * fp32(1 / scale))), NaN -> NaN
 *                 code with the input's sign; PA_BF16 or PA_F32 for a PA_INT8
 *                 pool, which stores clamp(rint(fp32(x * fp32(1 / scale))),
 *                 -127, 127) with ties to even, NaN -> 0
 *   slot_mapping  device int32 [num_tokens]; slots must be distinct and
 *                 < num_blocks * block_size
 *   k_cache, v_cache  device pools, written in place
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (num_tokens < 0, num_blocks * block_size
 * beyond int32 slots), PA_ERR_DTYPE, PA_ERR_UNSUPPORTED, PA_ERR_HIP.
 * num_tokens == 0 is a no-op returning PA_OK. */
pa_status pa_write_kv(const void* k, const void* v, int32_t in_dtype, int32_t num_tokens,
                      const int32_t* slot_mapping, void* k_cache, void* v_cache,
                      const pa_kv_cache* cache, void* stream);

/* Block copy for copy-on-write.
 *
 * For every pair i < num_pairs, copies physical block src[i] to physical block
 * dst[i] in both pools: all block_size rows, all KV heads, bytes as stored
 * (any pool format).  This is the device half of copy-on-write: before a
 * sequence appends into a block that other sequences still reference, the
 * allocator hands it a fresh block, the shared block is copied there, and the
 * sequence's table entry is redirected (LLM stack book, "Copy-on-write for
 * shared prefixes"; ai-infra-handbooks "Paged KV cache", exercise 2).
 *
 *   k_cache, v_cache  device pools, written in place (blocks dst[i] only)
 *   src, dst      device int32 [num_pairs]; a pair with either id outside
 *                 [0, num_blocks) (negative padding included) is skipped
 *   num_pairs     0 .. 65535
 * Every copy reads the pools as they were before the call: no dst may also
 * appear as a src, and dst ids must be distinct (undefined otherwise).
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_UNSUPPORTED,
 * PA_ERR_HIP.  num_pairs == 0 is a no-op returning PA_OK. */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const pa_kv_cache* cache, const int32_t* src,
                         const int32_t* dst, int32_t num_pairs, void* stream);

/* Multi-layer pools.  A model keeps one K and one V pool per layer (ai-infra-
 * handbooks "Paged KV cache", "Implementation": KV storage is one pair of
 * [num_blocks, block_size, H_kv, d_h] tensors per layer), all indexed by the same
 * block tables.  Here they may live in one allocation each for K and V:
 *   [num_layers, num_blocks, block_size, H_kv, d_h],
 * layer l's pool starting num_blocks * block_size * H_kv * d_h elements after layer
 * l - 1's; every per-layer call (pa_write_kv, pa_decode, ...) takes that layer's
 * base address with the same pa_kv_cache.  A copy-on-write copy must move the block
 * in every layer: pa_copy_blocks_layers does pa_copy_blocks for each of num_layers
 * layers in one launch (arguments as pa_copy_blocks; cache describes one layer).
 * Errors: as pa_copy_blocks, and PA_ERR_SHAPE for num_layers outside 1 .. 65535. */
pa_status pa_copy_blocks_layers(void* k_cache, void* v_cache, const pa_kv_cache* cache, int32_t num_layers,
                                const int32_t* src, const int32_t* dst, int32_t num_pairs, void* stream);

/* Partition size (tokens) used when a call passes partition_tokens = 0: 256, except that
 * the whole-decode calls (pa_decode, pa_decode_append, pa_decode_noalloc) on the
 * matrix-core path take pa_partition_tokens_for(max_context_len).  The two-stage calls
 * (pa_decode_partition, pa_decode_partition_append, pa_merge) and
 * pa_decode_workspace_bytes always take 256 for 0, so that a merge finds the pieces its
 * partition launch wrote; a workspace sized for 256 also holds the pieces of any larger
 * partition size. */
int32_t pa_default_partition_tokens(void);

/* The partition size a whole decode on the matrix cores takes for partition_tokens = 0:
 * 512 tokens when max_context_len >= 4096 (half the split-K partial outputs), else 256.
 * Host-only; no error. */
int32_t pa_partition_tokens_for(int32_t max_context_len);

/* Workspace bytes pa_decode / pa_decode_partition / pa_merge need for this shape
 * (0 when max_context_len fits in one partition).  partition_tokens = 0 means the
 * default.  Layout, each region aligned to 256 bytes:
 *   m [num_seqs, J, num_q_heads] f32, l [num_seqs, J, num_q_heads] f32,
 *   o [num_seqs, J, num_q_heads, head_dim] f32,  J = ceil(max_context_len / P)
 * (partition-major: the heads of one partition are contiguous).
 * Calls that share a workspace must be ordered on one stream (they race otherwise).
 * Returns 0 for invalid arguments. */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_tokens);

/* Kernel selection for pa_decode / pa_decode_partition. */
typedef enum pa_kernel {
  PA_KERNEL_AUTO = 0,      /* matrix-core path for bf16/e4m3/int8 pools, vector path for f32 */
  PA_KERNEL_VALU = 1,      /* vector-ALU path (all formats, query-head group <= 8) */
  PA_KERNEL_MFMA = 2       /* matrix-core path, one workgroup per (sequence, partition, up to
                              four KV heads) (bf16 q with bf16, e4m3 or int8 pools, group <= 16) */
} pa_kernel;

/* Paged decode attention for one new token per sequence.
 *
 * out[b, h, :] = softmax_t(scale * q[b, h, :] . K[b, t, kvh, :]) V[b, t, kvh, :]
 * over t < context_lens[b], with kvh = h / (num_q_heads / num_kv_heads) (query
 * heads grouped contiguously, LLM stack book "The PagedAttention Kernel") and
 * token t read from physical block block_tables[b, t / block_size] at offset
 * t % block_size (mohdvasim.com "PagedAttention - Explained", "The Custom CUDA
 * Kernel Overview").  A sequence with context_lens[b] == 0 gets zeros.
 *
 *   q             device [num_seqs, num_q_heads, head_dim] of q_dtype
 *                 (PA_F32 with an f32 pool; PA_BF16 with a bf16, e4m3 or int8 pool)
 *   k_cache, v_cache, cache   the pools (read only)
 *   block_tables  device int32 [num_seqs, max_blocks_per_seq]; entries at index
 *                 >= ceil(context_lens[b] / block_size) are never read
 *   context_lens  device int32 [num_seqs]: tokens valid after this step's write,
 *                 0 <= context_lens[b] <= max_context_len
 *   max_context_len  host-known bound on context_lens (sizes the grid, so no
 *                 device-to-host copy is needed); <= max_blocks_per_seq * block_size
 *   scale         softmax scale (1/sqrt(head_dim) for standard attention), finite
 *   out           device [num_seqs, num_q_heads, head_dim] of q_dtype
 *   workspace     device scratch of >= pa_decode_workspace_bytes(...) bytes
 *                 (may be NULL when that is 0); contents are overwritten
 *   partition_tokens  16, 32, 64, 128, 256, 512 or 1024 (0 = default); 512 and
 *                 1024 only with the matrix-core grid kernel (PA_KERNEL_MFMA, or
 *                 AUTO with a bf16 / e4m3 pool), which splits such a partition
 *                 among 2 or 4 waves per KV head and combines their pieces on chip,
 *                 so fewer pieces reach the workspace.  Results do not depend on
 *                 block_size or on where blocks sit in the pool: the reduction
 *                 order is fixed by logical token positions.
 *   kernel        pa_kernel
 * Outputs are bf16-rounded (nearest even) for bf16 q.  The matrix-core path
 * rounds the softmax probabilities to bf16 before P.V (and sums the same
 * rounded values in the denominator).
 * Launches: the partition stage (pa_decode_partition), then, when J > 1, the merge
 * (pa_merge); the output is bit for bit that of those two calls.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_UNSUPPORTED,
 * PA_ERR_WORKSPACE, PA_ERR_HIP.  num_seqs == 0 is a no-op returning PA_OK. */
pa_status pa_decode(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                    const void* k_cache, const void* v_cache, const pa_kv_cache* cache,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t max_context_len, float scale,
                    void* out, void* workspace, size_t workspace_bytes,
                    int32_t partition_tokens, int32_t kernel, void* stream);

/* pa_decode for callers that cannot allocate: code under HIP graph capture, tight serving
 * loops, or harnesses that forbid device allocation.  Same arguments and results as
 * pa_decode (bit for bit) minus the workspace: the split-K pieces live in a static
 * device array of the library, PA_DECODE_NOALLOC_SCRATCH_BYTES (64 MiB) on each GPU it
 * runs on, held until the process ends.  The first call on a device looks up that
 * device's copy; no call allocates or frees anything.
 *   - Shapes whose pieces exceed the array (pa_decode_workspace_bytes(...) above 64 MiB,
 *     about num_seqs * num_q_heads * ceil(max_context_len / P) * (head_dim + 2) * 4
 *     bytes) return PA_ERR_SCRATCH before anything is enqueued.
 *   - Every call writes the pieces it reads, so nothing needs clearing between calls.
 *     All calls on one GPU share the array: calls that overlap in time on one GPU (two
 *     streams, two threads, a graph replay beside an eager call) race and give
 *     undefined results; order them on one stream.
 * Errors: as pa_decode, with PA_ERR_SCRATCH in place of PA_ERR_WORKSPACE; PA_ERR_HIP if the
 * scratch's device address cannot be obtained. */
#define PA_DECODE_NOALLOC_SCRATCH_BYTES (64u << 20)
pa_status pa_decode_noalloc(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                            const void* k_cache, const void* v_cache, const pa_kv_cache* cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t max_context_len, float scale, void* out,
                            int32_t partition_tokens, int32_t kernel, void* stream);

/* First stage of pa_decode alone (same arguments and checks).  For every
 * sequence with context_lens[b] <= P it writes out[b] directly; for longer
 * sequences it writes partition j's pieces into the workspace, with
 * x_t = scale * q . K_t * log2(e):
 *   m_j = max x_t,  l_j = sum 2^(x_t - m_j),  o_j = sum 2^(x_t - m_j) V_t
 * over the partition's tokens [j*P, min((j+1)*P, ctx)). */
pa_status pa_decode_partition(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                              const void* k_cache, const void* v_cache, const pa_kv_cache* cache,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t max_context_len, float scale,
                              void* out, void* workspace, size_t workspace_bytes,
                              int32_t partition_tokens, int32_t kernel, void* stream);

/* pa_write_kv of this step's tokens and pa_decode in one partition launch (plus the
 * merge), for the decode step where every sequence appends one token.  For each
 * sequence b with ctx = context_lens[b] >= 1 (the length after the append), the
 * rows k_new[b], v_new[b] are stored at position ctx - 1, i.e. at
 *   slot = block_tables[b, (ctx - 1) / block_size] * block_size + (ctx - 1) % block_size
 * (the slot mapping of ai-infra-handbooks "Paged KV cache", "Block tables and slot
 * mapping"), in the pool's format exactly as pa_write_kv would store them,
 * and then attends over positions 0 .. ctx - 1 as pa_decode does.  The workgroup
 * whose partition holds position ctx - 1 writes the rows and waits for the stores
 * before it reads any row, so the results, and the pools afterwards, are bit for bit
 * those of pa_write_kv followed by pa_decode.  A sequence with ctx == 0 appends
 * nothing and gets zeros.
 *   k_new, v_new  device [num_seqs, num_kv_heads, head_dim], in_dtype PA_BF16
 *   k_cache, v_cache  the pools, written at the appended slots and read
 *   partition_tokens  256, 512 or 1024 (0 = the default, 256)
 *   the other arguments as pa_decode; the matrix-core grid kernel runs (bf16 q with
 *   a bf16, e4m3 or int8 pool, query-head group <= 16).
 * Errors: as pa_decode; PA_ERR_NULL for a null k_new or v_new; PA_ERR_DTYPE for
 * another in_dtype; PA_ERR_UNSUPPORTED for an f32 pool or a partition below 256. */
pa_status pa_decode_append(const void* q, int32_t q_dtype, const void* k_new, const void* v_new, int32_t in_dtype,
                           int32_t num_seqs, int32_t num_q_heads, void* k_cache, void* v_cache,
                           const pa_kv_cache* cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t max_context_len, float scale, void* out,
                           void* workspace, size_t workspace_bytes, int32_t partition_tokens, void* stream);

/* First stage of pa_decode_append alone (same arguments and checks; the pieces and
 * outputs as pa_decode_partition). */
pa_status pa_decode_partition_append(const void* q, int32_t q_dtype, const void* k_new, const void* v_new,
                                     int32_t in_dtype, int32_t num_seqs, int32_t num_q_heads, void* k_cache,
                                     void* v_cache, const pa_kv_cache* cache, const int32_t* block_tables,
                                     int32_t max_blocks_per_seq, const int32_t* context_lens,
                                     int32_t max_context_len, float scale, void* out, void* workspace,
                                     size_t workspace_bytes, int32_t partition_tokens, void* stream);

/* Second stage of pa_decode: for every sequence with n = ceil(context_lens[b] / P)
 * >= 2 partitions and every query head,
 *   out = sum_j 2^(m_j - M) o_j / sum_j 2^(m_j - M) l_j,   M = max_j m_j,
 * over j < n, reading the workspace layout above.  Sequences with n <= 1 are
 * left untouched.  out_dtype is PA_F32 or PA_BF16; head_dim is 64 or 128.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_UNSUPPORTED,
 * PA_ERR_WORKSPACE, PA_ERR_HIP. */
pa_status pa_merge(const void* workspace, size_t workspace_bytes, int32_t num_seqs, int32_t num_q_heads,
                   int32_t head_dim, const int32_t* context_lens, int32_t max_context_len,
                   int32_t partition_tokens, int32_t out_dtype, void* out, void* stream);

/* Multi-query paged attention: several new tokens per sequence (chunked prefill,
 * a full prefill, or decode as the one-token case), causal within each sequence.
 *
 * Sequence b's new tokens are rows query_start_loc[b] .. query_start_loc[b+1]-1 of
 * q; they are the last n_b = query_start_loc[b+1] - query_start_loc[b] positions of
 * its context of seq_lens[b] tokens (their K/V already written, e.g. by
 * pa_write_kv).  New token j, at position p = seq_lens[b] - n_b + j, attends to the
 * positions 0 .. p of its own sequence:
 *   out[row, h, :] = softmax_t<=p(scale * q[row, h, :] . K[b, t, kvh, :]) V[b, t, kvh, :]
 * with kvh = h / (num_q_heads / num_kv_heads) and token t read through the block
 * table as in pa_decode (ai-infra-handbooks "Paged KV cache", section "Paged
 * attention": block_tables, seq_lens and query_start_loc; the causal mask offset by
 * seq_len - num_new; the result equals contiguous attention).
 *
 *   q, out        device [num_tokens, num_q_heads, head_dim] bf16 (q_dtype PA_BF16)
 *   cache         a PA_BF16, PA_FP8_E4M3 or PA_INT8 pool; num_q_heads / num_kv_heads in
 *                 {1, 2, 4, 8, 16}
 *   block_tables  device int32 [num_seqs, max_blocks_per_seq]
 *   seq_lens      device int32 [num_seqs], context length including the new tokens
 *   query_start_loc  device int32 [num_seqs + 1], nondecreasing, from 0 to num_tokens
 *   max_query_len host-known bound on n_b (sizes the grid)
 * The matrix-core path rounds probabilities to bf16 before P.V, as pa_decode does.
 * A sequence whose rows fall outside [0, num_tokens) or whose n_b exceeds
 * seq_lens[b] is skipped (its out rows are left untouched).
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_UNSUPPORTED, PA_ERR_HIP.
 * num_tokens == 0 or num_seqs == 0 is a no-op returning PA_OK. */
pa_status pa_paged_attention(const void* q, int32_t q_dtype, int32_t num_tokens, int32_t num_seqs,
                             int32_t num_q_heads, const void* k_cache, const void* v_cache,
                             const pa_kv_cache* cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* seq_lens, const int32_t* query_start_loc, int32_t max_query_len,
                             float scale, void* out, void* stream);

/* Device-side slot mapping for this step (and, optionally, the step's advance of
 * the context lengths), so that a decode loop -- slot mapping, pa_write_kv,
 * pa_decode -- needs no host work between steps and can be captured once in a
 * HIP graph.  The pages have the engine rebuild these tensors on the host each
 * step (LLM stack book, "From Python bookkeeping to the tensors the kernel
 * actually takes"); the formula is theirs: new token j of sequence b, at position
 * p = seq_lens[b] - n_b + j, goes to slot table[b][p / block_size] * block_size
 * + p % block_size (ai-infra-handbooks "Paged KV cache", "Block tables and slot
 * mapping").
 *
 *   block_tables  device int32 [num_seqs, max_blocks_per_seq]; the blocks for this
 *                 step's positions must already be in the table (the host
 *                 allocator appends them ahead of the steps it captures)
 *   seq_lens      device int32 [num_seqs]; with advance != 0 each grows by n_b
 *                 first (in place), so afterwards it counts this step's tokens
 *   query_start_loc  device int32 [num_seqs + 1] rows of each sequence's new
 *                 tokens, or NULL for one new token per sequence in row b
 *   slot_mapping  device int32 [num_tokens], written for every new-token row; a
 *                 position outside the table gets -1 (pa_write_kv skips it)
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED (block_size not a power of
 * two in 1..1024), PA_ERR_HIP.  num_seqs == 0 is a no-op returning PA_OK. */
pa_status pa_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t* seq_lens,
                          const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens, int32_t block_size,
                          int32_t advance, int32_t* slot_mapping, void* stream);

/* Host-side contract checks.  Unlike every other call these take HOST pointers: the
 * integer inputs of a step, inspected on the CPU before they go to the GPU.  The release
 * kernels trust these contracts (a broken one is undefined behaviour, see above); a
 * checked caller runs these first and refuses the step.  Each returns PA_OK, or
 * PA_ERR_SHAPE with *bad_index (if not NULL) naming the first offending entry, or
 * PA_ERR_NULL / PA_ERR_SHAPE for bad sizes (then *bad_index = -1).
 *
 * pa_check_decode_inputs: every context_lens[b] must lie in [0, max_context_len] and fit
 * its table (<= max_blocks_per_seq * block_size) -- *bad_index = b otherwise; every table
 * entry a decode reads (index j < ceil(context_lens[b] / block_size) of row b) must be a
 * block of the pool, [0, num_blocks) -- *bad_index = b * max_blocks_per_seq + j otherwise.
 * Entries past a sequence's context are padding and are not checked (LLM stack book, "From
 * Python bookkeeping to the tensors the kernel actually takes": rows are padded to the
 * longest sequence).
 *
 * pa_check_slots: every slot_mapping[i] >= 0 must be < num_blocks * block_size, and no two
 * tokens may share a slot (the write would race); *bad_index = i of the out-of-range token,
 * or of the first token, in token order, whose slot an earlier token already took.
 * Negative slots are padding and pass. */
pa_status pa_check_decode_inputs(const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                                 int64_t num_blocks, int32_t block_size, int64_t* bad_index);
pa_status pa_check_slots(const int32_t* slot_mapping, int32_t num_tokens, int64_t num_blocks, int32_t block_size,
                         int64_t* bad_index);

/* The checked build.  libpa_checked.so is built from the same sources with
 * -DPA_CHECKED=1: its kernels test what the release kernels trust -- every slot
 * against num_blocks * block_size (pa_write_kv), every block id a call reads against
 * [0, num_blocks) (decode, append, multi-query), every context length against its
 * table (max_blocks_per_seq * block_size) and against max_context_len, and copy ids
 * against the pool -- and on a breach set a bit in a device error word and go on with a
 * safe value (the token skipped, block 0 read, the length clipped, the request or pair
 * skipped), so outputs are then wrong but nothing outside the pools is touched.  The
 * bits: */
#define PA_CHECKED_SLOT   1u  /* a slot past the pool */
#define PA_CHECKED_BLOCK  2u  /* a block id outside the pool */
#define PA_CHECKED_LENGTH 4u  /* a context past its table or past max_context_len */
#define PA_CHECKED_PAIR   8u  /* a copy-on-write id past the pool */

/* 1 in the checked build, 0 in the release build. */
int32_t pa_checked_build(void);

/* Checked build: waits for the current device to finish all its work (a host
 * synchronization; not for capture in a graph), returns the error bits raised since the
 * last call in *flags and clears them.  Release build: *flags = 0, PA_ERR_UNSUPPORTED. */
pa_status pa_checked_errors(uint32_t* flags);

/* Static, human-readable name of a status code. */
const char* pa_status_str(pa_status status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
