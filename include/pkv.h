/*
 * pkv.h -- batch-invariant paged-KV attention forward for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpkv.so.  Plain pointers and sizes; every device pointer is a HIP
 * device address on the current device; every call is asynchronous on the
 * given stream and never synchronises the host.  No exceptions or aborts cross
 * this boundary: each entry point returns PKV_OK (0) or a negative PKV_ERR_*
 * code, and pkv_last_error() gives the calling thread's last message.
 *
 * What is computed (the operation these entry points implement):
 *
 *   RL-Kernel issue #152 "[WS1] KV-cache path consistency (prefill & decode)",
 *   section Scope: attention of a query against N cached keys/values (decode)
 *   must reduce in the same fixed order as the equivalent prefill over the full
 *   sequence, and cache writes/reads must add no precision difference.
 *   RL-Kernel PR #284 "feat(attention): add CP backward drift validation",
 *   section Changes: a fixed KV chunk size, partials merged in ascending global
 *   block index, fp32 accumulation, one downcast at the final write, and an
 *   attention-domain LSE reported with the output.
 *
 *   For sequence b with n = seqlens_k[b] keys and L = cu_seqlens_q[b+1] -
 *   cu_seqlens_q[b] query rows, row r sits at key position p = n - L + r
 *   (bottom-right alignment) and sees keys j < n, and with causal also j <= p.
 *   Query head h reads KV head h / (Hq / Hkv).  For each (row, head):
 *       s_j = softmax_scale * <q, k_j>,   lse = ln(sum_j exp(s_j)),
 *       out = sum_j exp(s_j - lse) v_j.
 *   A row that sees no key gets out = 0 and lse = -inf.
 *
 * Reduction contract (what makes the result independent of batch size,
 * padding, split count, grid and decode/prefill path):
 *   keys are cut into chunks of PKV_CHUNK_KEYS keys at global key positions
 *   [c*PKV_CHUNK_KEYS, (c+1)*PKV_CHUNK_KEYS); inside a chunk, tiles of
 *   PKV_TILE_KEYS keys are accumulated in ascending order with an fp32 running
 *   max; each chunk yields (max, sum, o[d]) in fp32; the chunk results of a row
 *   are folded in ascending chunk index; the output is rounded once, at the
 *   final write.  Every row's bits are a function of that row's query, its
 *   visible keys/values and softmax_scale only.
 *
 * Memory layout (ROCm/aiter commit d293d61bbf19 "test(triton/decode): pin
 * non-contiguous paged KV block stride"): the cache is paged in blocks of
 * block_size tokens; key j of sequence b is in block block_table[b][j /
 * block_size] at slot j % block_size.  K and V are each addressed by element
 * strides (block, slot, head) with the head-dim stride 1, so both the
 * contiguous [num_blocks, block_size, Hkv, d] layout and the K/V-interleaved
 * [num_blocks, 2, block_size, Hkv, d] layout (block stride 2*block_size*Hkv*d)
 * are served from their real strides.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 2
#define PKV_CHUNK_KEYS 1024 /* keys per chunk: the unit partials are merged in */
#define PKV_TILE_KEYS 64    /* keys per tile inside a chunk */

/*
 * Element types.  PKV_F32 / PKV_BF16: q, the cache, new K/V and out share the
 * type.  PKV_FP8_E4M3: q and out are bf16; the cache and new K/V rows hold OCP
 * FP8 E4M3 bytes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; NaN
 * 0x7f/0xff, no infinities), the stored value times the layout's k_scale /
 * v_scale being K / V; the computation after the exact widening to bf16 is the
 * PKV_BF16 one.  lse is always fp32.  The FP8 cache is the step the pages defer
 * (RL-Kernel issue #152, section Out of scope).
 */
enum pkv_dtype { PKV_F32 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2 };

enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_NULL = -1,      /* a required pointer is NULL */
  PKV_ERR_SHAPE = -2,     /* inconsistent or unsupported sizes */
  PKV_ERR_DTYPE = -3,     /* unsupported dtype */
  PKV_ERR_ALIGN = -4,     /* a pointer or stride breaks 16-byte alignment */
  PKV_ERR_WORKSPACE = -5, /* workspace too small or could not be allocated */
  PKV_ERR_HIP = -6,       /* a HIP runtime call or kernel launch failed */
  PKV_ERR_OPTION = -7,    /* unknown option or value */
  PKV_ERR_DEVICE_DATA = -8 /* index data violates a precondition (debug mode, pkv_check_inputs) */
};

/*
 * Shapes and strides of one call.  All strides are in elements.
 *   dtype               pkv_dtype (element types of q/out and of the cache/new K/V)
 *   batch               B, number of sequences, <= 65535 (a launch-grid dimension)
 *   num_heads_q         Hq; num_heads_q % num_heads_k == 0
 *   num_heads_k         Hkv, <= 65535
 *   head_dim            d, 64 or 128
 *   block_size          tokens per cache block, >= 1
 *   max_blocks_per_seq  row length of block_table ([batch, max_blocks_per_seq], int32)
 *   max_seqlen_q        host-side bound on every cu_seqlens_q[b+1] - cu_seqlens_q[b]
 *   max_seqlen_k        host-side bound on every seqlens_k[b]; 0 means
 *                       max_blocks_per_seq * block_size
 *   total_q             rows of q / out / lse (cu_seqlens_q[batch]);
 *                       total_q * num_heads_q <= 2^31 - 1
 *   num_blocks          blocks in the pool (used only by debug checks)
 *   k_* / v_*_stride    element strides of the K and V caches: block, slot, head
 *   k_scale, v_scale    K = stored * k_scale, V = stored * v_scale (0 means 1; must be
 *                       finite and >= 0).  k_scale enters the score multiplier
 *                       (softmax_scale * k_scale); v_scale multiplies each output once,
 *                       after the division by the row sum.  The backward requires 1.
 * q and out are packed [total_q, Hq, d]; lse is [total_q, Hq] fp32.
 */
typedef struct pkv_layout {
  int32_t dtype;
  int32_t batch;
  int32_t num_heads_q;
  int32_t num_heads_k;
  int32_t head_dim;
  int32_t block_size;
  int32_t max_blocks_per_seq;
  int32_t max_seqlen_q;
  int64_t max_seqlen_k;
  int64_t total_q;
  int64_t num_blocks;
  int64_t k_block_stride, k_slot_stride, k_head_stride;
  int64_t v_block_stride, v_slot_stride, v_head_stride;
  float k_scale;
  float v_scale;
} pkv_layout;

/*
 * Attention forward over the paged cache.
 *   q            device, [total_q, Hq, d] of dtype; rows cu_seqlens_q[b]..cu_seqlens_q[b+1]-1
 *                belong to sequence b; Q/K are attention-ready (post-RoPE, RL-Kernel PR #284,
 *                section "RoPE / TE Boundary"): no positional transform is applied here
 *   k_cache      device, K elements addressed by kv_strides->k_* strides
 *   v_cache      device, V elements addressed by kv_strides->v_* strides
 *   kv_strides   host, shapes and strides (read during the call only)
 *   block_table  device int32 [batch, max_blocks_per_seq]; only the first
 *                ceil(seqlens_k[b] / block_size) entries of row b are read
 *   seqlens_k    device int32 [batch]: keys visible to the call, including the keys
 *                of this call's own query rows
 *   cu_seqlens_q device int32 [batch + 1], non-decreasing, cu_seqlens_q[0] = 0
 *   causal       nonzero: row at position p sees keys <= p
 *   softmax_scale  multiplies <q, k> (e.g. 1/sqrt(d)); finite and > 0
 *   out          device, [total_q, Hq, d] of dtype (written)
 *   lse          device fp32 [total_q, Hq] (written): natural-log LSE
 *   stream       HIP stream; all work is enqueued there
 * Buffers must stay alive until the stream passes this call.  Device data
 * preconditions (checked only in debug mode, PKV_OPT_DEBUG): cu_seqlens_q[0] = 0,
 * non-decreasing, cu_seqlens_q[batch] = total_q; row counts <= max_seqlen_q;
 * 0 <= seqlens_k[b] <= min(max_seqlen_k, max_blocks_per_seq * block_size);
 * the block ids a sequence with rows uses in [0, num_blocks) (num_blocks = 0:
 * ids only checked for >= 0).  Not checked at all: cache values at visible
 * positions finite.  A row with no
 * visible key (e.g. seqlens_k[b] = 0, or a causal row at position < 0 when
 * seqlens_k[b] is below the row count) gets out = 0 and lse = -inf.  The split (decode)
 * path needs a workspace for keys beyond one 1024-key chunk (max_seqlen_k above
 * 1024); this entry point takes it from the stream-ordered allocator
 * (hipMallocAsync / hipFreeAsync on `stream`).
 * Errors: PKV_ERR_NULL, PKV_ERR_SHAPE (also softmax_scale <= 0 or not finite),
 * PKV_ERR_DTYPE, PKV_ERR_ALIGN (q, caches,
 * out must be 16-byte aligned and every stride a multiple of 16 bytes),
 * PKV_ERR_WORKSPACE, PKV_ERR_HIP.  Nothing is launched on error.
 */
int pkv_attn_forward(const void* q, const void* k_cache, const void* v_cache,
                     const pkv_layout* kv_strides, const int32_t* block_table,
                     const int32_t* seqlens_k, const int32_t* cu_seqlens_q, int causal,
                     float softmax_scale, void* out, float* lse, hipStream_t stream);

/*
 * As pkv_attn_forward, with a caller-owned device workspace of
 * workspace_bytes >= pkv_attn_workspace_size(kv_strides) bytes (16-byte
 * aligned).  Calls sharing one workspace must be ordered on one stream.
 */
int pkv_attn_forward_ws(const void* q, const void* k_cache, const void* v_cache,
                        const pkv_layout* kv_strides, const int32_t* block_table,
                        const int32_t* seqlens_k, const int32_t* cu_seqlens_q, int causal,
                        float softmax_scale, void* out, float* lse, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/*
 * As pkv_attn_forward, allocating nothing: for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The split path's chunk partials go to a static
 * device array of PKV_NOALLOC_MAX_BYTES bytes that the library holds on each
 * GPU it runs on until the process ends; its address is looked up (with
 * hipGetSymbolAddress) on the first call on each device, so make that first
 * call outside stream capture.  No hipMalloc, hipFree or allocating library
 * call is made.  A call whose split path needs more than PKV_NOALLOC_MAX_BYTES
 * (pkv_attn_workspace_size) fails with PKV_ERR_WORKSPACE before any launch.
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind (nothing in it needs to start at zero): calls that may overlap on
 * one GPU -- on different streams, or from different threads without
 * ordering -- race on it and must not be issued.  Arguments, results and
 * other errors as pkv_attn_forward; the bits equal pkv_attn_forward's.
 */
#define PKV_NOALLOC_MAX_BYTES ((size_t)96 << 20)
int pkv_attn_forward_noalloc(const void* q, const void* k_cache, const void* v_cache,
                             const pkv_layout* kv_strides, const int32_t* block_table,
                             const int32_t* seqlens_k, const int32_t* cu_seqlens_q, int causal,
                             float softmax_scale, void* out, float* lse, hipStream_t stream);

/*
 * Fused append-then-attend: the K/V rows of this call's own query rows are
 * written into the cache and attended in the same launch.  The step before the
 * path on the pages (aiter commit d293d61bbf19: flash_attn_with_kvcache
 * parametrised over new_kv; RL-Kernel issue #152, section Scope: cache writes
 * must add no precision difference).
 *   k_new, v_new  device, [total_q, Hkv, d] of dtype: row cu_seqlens_q[b] + r is the
 *                 key/value of key position seqlens_k[b] - L_b + r (the row's own position)
 *   k_cache, v_cache  written at those positions (and read as in pkv_attn_forward)
 *   seqlens_k     keys visible to the call, the appended ones included (as in
 *                 pkv_attn_forward); requires L_b <= seqlens_k[b]
 *   workspace     NULL: taken from the stream-ordered allocator; else a caller buffer of
 *                 workspace_bytes >= pkv_attn_workspace_size(kv_strides)
 * Result, bit for bit: the cache bytes and out/lse of pkv_cache_write(k_new, v_new,
 * ..., seqlens_k - L, cu_seqlens_q) followed by pkv_attn_forward(...).  Other
 * arguments, ownership and errors as pkv_attn_forward.
 */
int pkv_attn_forward_append(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            const pkv_layout* kv_strides, const int32_t* block_table, const int32_t* seqlens_k,
                            const int32_t* cu_seqlens_q, int causal, float softmax_scale, void* out, float* lse,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes the split path needs for this layout (0 if it is never used,
 * and 0 when every sequence lies within one 1024-key chunk -- max_seqlen_k, or
 * max_blocks_per_seq * block_size when it is 0, at most 1024 -- where the split
 * kernels write out / lse themselves and no merge runs):
 * the fp32 chunk partials (total_q * Hq * chunks * (d + 2) floats) and, when
 * the one-wave bf16/FP8 decode kernels take a longest-first job list (at most
 * 16 chunks of keys and more than 2048 (sequence, KV head, chunk) slots),
 * 2 * (batch + 1) int32 prefix counts; each part rounded up to 256 bytes. */
size_t pkv_attn_workspace_size(const pkv_layout* kv_strides);

/*
 * Context-parallel share of the forward, and the fold that joins the shares.
 * RL-Kernel PR #284, "feat(attention): add CP backward drift validation",
 * section Changes: with context parallelism each rank handles a range of KV
 * chunks and the partial results are merged in a fixed, ascending global block
 * (chunk) order, so the result does not depend on the CP world size.
 *
 * pkv_attn_chunk_partials computes, for every row and query head, the partial
 * of each global chunk c in [chunk_begin, chunk_end) that the row can see (the
 * chunk core of pkv_attn_forward, the same bits), and writes it chunk-major:
 *   part_ml  device fp32 [max_chunks, total_q * Hq, 2]: (m, l) of the chunk, in the
 *            library's score units (bf16 and FP8 caches: base 2, m scaled by
 *            softmax_scale * k_scale * log2(e); fp32: natural units), so
 *            chunk LSE = (m + log2 l) * ln 2 (fp32 caches: m + ln l); m = -inf if the
 *            row sees no key of the chunk
 *   part_o   device fp32 [max_chunks, total_q * Hq, d]: sum over the chunk of
 *            exp(score - m) * stored V (the chunk output is part_o / l * v_scale)
 * A rank's range is one contiguous slab of both buffers, ready for an
 * all-gather.  Slots of chunks a row cannot see are not written.  Arguments
 * as pkv_attn_forward otherwise; 0 <= chunk_begin <= chunk_end <= max_chunks.
 *
 * pkv_attn_merge_partials folds, per row and head, chunks 0 .. ceil(visible
 * keys / PKV_CHUNK_KEYS) - 1 of such buffers in ascending chunk index and
 * writes out / lse.  When the buffers hold the partials of every chunk (the
 * union of the ranks' ranges covers them; precondition), the result is bit
 * for bit that of pkv_attn_forward on the same inputs, for any split of the
 * chunk range.  kv_strides supplies shapes, dtype and v_scale.
 */
int pkv_attn_chunk_partials(const void* q, const void* k_cache, const void* v_cache,
                            const pkv_layout* kv_strides, const int32_t* block_table,
                            const int32_t* seqlens_k, const int32_t* cu_seqlens_q, int causal,
                            float softmax_scale, int32_t chunk_begin, int32_t chunk_end,
                            int32_t max_chunks, float* part_o, float* part_ml, hipStream_t stream);
int pkv_attn_merge_partials(const float* part_o, const float* part_ml, int32_t max_chunks,
                            const pkv_layout* kv_strides, const int32_t* seqlens_k,
                            const int32_t* cu_seqlens_q, int causal, void* out, float* lse,
                            hipStream_t stream);

/*
 * Backward of pkv_attn_forward: gradients of out with respect to q and to each
 * sequence's visible keys and values.  RL-Kernel PR #284, "feat(attention):
 * add CP backward drift validation", sections Summary and Changes: a
 * deterministic training backward (dq, dk, dv) for causal prefill and chunked
 * prefill over the same forward, fp32 accumulation, one downcast at the final
 * write.  The cotangent of lse is taken as zero.
 *   q, k_cache, v_cache, kv_strides, block_table, seqlens_k, cu_seqlens_q,
 *   causal, softmax_scale   exactly as given to the forward
 *   out, lse        device, the forward's outputs for those inputs
 *   dout            device, [total_q, Hq, d] of dtype: the cotangent of out
 *   cu_seqlens_k    device int32 [batch + 1]: exclusive prefix sum of seqlens_k
 *                   (precondition, not checked on the device)
 *   total_k         host copy of cu_seqlens_k[batch]
 *   dq              device, [total_q, Hq, d] of dtype (written, every row)
 *   dk, dv          device, [total_k, Hkv, d] of dtype: row cu_seqlens_k[b] + j is
 *                   key/value position j of sequence b; every such row is written
 *                   (query heads of a GQA group add up)
 *   workspace       NULL: taken from the stream-ordered allocator; else a caller
 *                   buffer of workspace_bytes >= pkv_attn_backward_workspace_size()
 * Every sum runs in an order fixed by global key positions and column indices
 * (no atomics): results are bitwise reproducible, independent of the batch, and
 * a row's dq does not depend on how the rows were split into calls.
 * Errors as pkv_attn_forward; dout, dq, dk, dv, out must be 16-byte aligned.
 */
int pkv_attn_backward(const void* q, const void* k_cache, const void* v_cache,
                      const pkv_layout* kv_strides, const int32_t* block_table,
                      const int32_t* seqlens_k, const int32_t* cu_seqlens_q,
                      const int32_t* cu_seqlens_k, int64_t total_k, int causal,
                      float softmax_scale, const void* out, const float* lse, const void* dout,
                      void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* Workspace bytes pkv_attn_backward needs for this layout (total_q * Hq floats). */
size_t pkv_attn_backward_workspace_size(const pkv_layout* kv_strides);

/*
 * Append new K/V rows to the paged cache.  RL-Kernel issue #152, section Scope:
 * the write is a bit copy, so the path that wrote the cache and the path that
 * reads it see the same values.
 *   k_new, v_new    device, [total_new, Hkv, d] of dtype, packed
 *   k_cache/v_cache device, addressed by kv_strides (written)
 *   block_table     device int32 [batch, max_blocks_per_seq]
 *   seqlens_k       device int32 [batch]: tokens already in the cache; token t of
 *                   sequence b goes to position seqlens_k[b] + t.  Not updated: the
 *                   caller advances it.
 *   cu_seqlens_new  device int32 [batch + 1]
 *   total_new       host copy of cu_seqlens_new[batch]: the launch has one work group
 *                   per new token, and reading the count from cu_seqlens_new on the
 *                   device would cost a host synchronisation per call
 * Only the written slots change.  Preconditions (checked only in debug mode):
 * cu_seqlens_new[0] = 0, non-decreasing, cu_seqlens_new[batch] = total_new;
 * seqlens_k[b] >= 0; every target position < max_blocks_per_seq * block_size
 * and its block id in [0, num_blocks).
 */
int pkv_cache_write(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                    const pkv_layout* kv_strides, const int32_t* block_table,
                    const int32_t* seqlens_k, const int32_t* cu_seqlens_new,
                    int64_t total_new, hipStream_t stream);

/* Host-only check of a layout (no device call).  Returns PKV_OK or an error. */
int pkv_validate_layout(const pkv_layout* kv_strides);

/*
 * Process-wide tuning and test hooks.  None changes a result bit: they choose
 * which kernels run and how work is split (debug mode adds checks).  They are
 * process-wide on purpose: a setting made on one thread governs calls made on
 * any other, and since no option changes a bit, concurrent calls stay correct.
 *   PKV_OPT_PATH          0 auto, 1 split (decode kernels + merge), 2 full (prefill kernel)
 *   PKV_OPT_SPLIT_CHUNKS  chunks handled by one split work item (0 = auto = 1, 1..64);
 *                         with one chunk per item, ragged batches spanning at most 16
 *                         chunks take the decode kernels' longest-first job order
 *   PKV_OPT_FULL_KERNEL   bf16/FP8 full path: 0 auto (3 when max_seqlen_q * Hq/Hkv <=
 *                         1024 and the keys reach 16384, else 2), 1 pipelined 8 waves x
 *                         16 columns per work group, 2 4 waves x 32 columns, 3 8 waves x
 *                         32 columns (not for the fused append, which takes 2)
 *   PKV_OPT_DECODE_ORDER  one-wave decode kernels: dispatch order of the work items, 0 auto
 *                         (2 when the grid has at most 2048 work items and each (sequence,
 *                         KV head) at least 4 of them, else 1), 1 the items of one
 *                         (sequence, KV head) consecutive, 2 the sequence fastest
 *   PKV_OPT_DEBUG         0 off, 1 debug mode: every call first enqueues a check of
 *                         its index data (the device-data preconditions above) on its
 *                         stream; when one fails, the call's kernels return without
 *                         touching memory and a per-GPU error word records the
 *                         violation, read by pkv_check_device_errors.  The word is
 *                         sticky: until it is collected, every debug-mode call on that
 *                         GPU does nothing.  Initially 1 when the environment variable
 *                         PKV_DEBUG is set to a nonzero value.  The first debug-mode call
 *                         on a device clears the word synchronously: make it outside
 *                         stream capture.
 */
enum pkv_option {
  PKV_OPT_PATH = 1,
  PKV_OPT_SPLIT_CHUNKS = 2,
  PKV_OPT_FULL_KERNEL = 3,
  PKV_OPT_DEBUG = 4,
  PKV_OPT_DECODE_ORDER = 5
};
int pkv_set_option(int option, int64_t value);
int64_t pkv_get_option(int option);

/*
 * Collect the device-side errors of the work enqueued so far (synchronises
 * `stream`).  Returns PKV_ERR_HIP if the stream or an earlier launch failed,
 * PKV_ERR_DEVICE_DATA (message: the violated preconditions and the lowest bad
 * sequence) if a debug-mode check on the current device recorded a violation
 * since the last collection -- the word is then cleared -- and PKV_OK
 * otherwise.  Not capturable (it synchronises).
 *   ROCm/aiter commit d293d61bbf19, commit message: a block address computed
 *   from the wrong stride read memory outside the sequence's blocks and
 *   "produced garbage" with no error; RL-Kernel issue #152, section Scope: the
 *   cache write and the reads must agree on every slot.  These checks turn
 *   such index data into an error instead of a silent wrong result.
 */
int pkv_check_device_errors(hipStream_t stream);

/*
 * The same precondition checks on host copies of the index data (no device
 * call): block_table [batch, max_blocks_per_seq], seqlens_k [batch] and
 * cu_seqlens [batch + 1], int32 host arrays, as they will be passed to
 *   op = PKV_CHECK_ATTENTION   pkv_attn_forward* / chunk partials (total_rows = total_q)
 *        PKV_CHECK_APPEND      pkv_attn_forward_append (also rows <= seqlens_k[b])
 *        PKV_CHECK_CACHE_WRITE pkv_cache_write (seqlens_k before the append,
 *                              total_rows = total_new)
 * Returns PKV_OK or PKV_ERR_DEVICE_DATA with the violated preconditions and
 * the first bad sequence in pkv_last_error().
 */
enum pkv_check_op { PKV_CHECK_ATTENTION = 0, PKV_CHECK_APPEND = 1, PKV_CHECK_CACHE_WRITE = 2 };
int pkv_check_inputs(const pkv_layout* kv_strides, const int32_t* block_table, const int32_t* seqlens_k,
                     const int32_t* cu_seqlens, int64_t total_rows, int op);

const char* pkv_error_string(int code);
/* Message of the calling thread's last failed call ("" if none). */
const char* pkv_last_error(void);
int pkv_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PKV_H */
