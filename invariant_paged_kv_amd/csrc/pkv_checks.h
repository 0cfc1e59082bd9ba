// pkv_checks.h -- the device-data preconditions of libpkv's entry points, as
// one function that runs on the host (pkv_check_inputs, on host copies) and
// on the device (the debug-mode check kernel, before the call's kernels).
//
// The pages' stride bug read memory outside a sequence's blocks and "produced
// garbage" silently (ROCm/aiter commit d293d61bbf19, commit message); the
// cache write and the reads must agree on every slot (RL-Kernel issue #152,
// section Scope).  These checks name the index data that decides which slots
// are touched: the cumulative row counts, the key counts, the block ids a
// sequence uses and the positions a cache write targets.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Violations (bit flags of the error word).
enum CheckFlag : int32_t {
  kBadCu = 1,        // cumulative row counts: cu[0] != 0, decreasing, or cu[batch] != the row total
  kBadSeqlen = 2,    // seqlens_k[b] < 0, or above min(max_seqlen_k, max_blocks_per_seq * block_size)
  kBadBlockId = 4,   // a block id the call uses is < 0 or >= num_blocks
  kBadRows = 8,      // a sequence has more rows than max_seqlen_q
  kBadAppend = 16,   // fused append: more new rows than visible keys
  kBadWritePos = 32, // cache write: a target position beyond max_blocks_per_seq * block_size
  kBadCuK = 64,      // backward: cu_seqlens_k is not the prefix sum of seqlens_k, or != total_k
};

// What an entry point reads.
enum CheckOp : int32_t { kOpAttention = 0, kOpAppend = 1, kOpCacheWrite = 2, kOpBackward = 3 };

struct CheckLimits {
  int64_t total_rows;    // total_q (attention) or total_new (cache write)
  int64_t max_k;         // min(max_seqlen_k, max_blocks_per_seq * block_size); cache write: table capacity
  int64_t num_blocks;    // 0: block ids are only checked for >= 0
  int64_t total_k;       // backward: rows of dk / dv
  int32_t max_rows;      // max_seqlen_q (unused by the cache write)
  int32_t mbps;          // max_blocks_per_seq
  int32_t bs;            // block_size
  int32_t batch;
  int32_t op;
};

__host__ __device__ inline int32_t check_block_ids(const int32_t* row, int64_t first, int64_t last, int64_t num_blocks) {
  int32_t f = 0;
  for (int64_t i = first; i <= last; ++i) {
    const int32_t id = row[i];
    if (id < 0 || (num_blocks > 0 && id >= num_blocks)) f |= kBadBlockId;
  }
  return f;
}

// Flags of sequence b.  Reads cu[b], cu[b + 1], seqlens_k[b], the block ids
// the call would use (only when the counts that bound them are valid) and,
// for the backward, cu_k[b], cu_k[b + 1].
__host__ __device__ inline int32_t check_sequence(const CheckLimits& l, int b, const int32_t* cu, const int32_t* sk,
                                                  const int32_t* block_table, const int32_t* cu_k) {
  int32_t f = 0;
  const int64_t c0 = cu[b], c1 = cu[b + 1];
  if ((b == 0 && c0 != 0) || c1 < c0 || c1 > l.total_rows || (b == l.batch - 1 && c1 != l.total_rows)) f |= kBadCu;
  const int64_t rows = c1 - c0;
  const int64_t n = sk[b];
  if (l.op != kOpCacheWrite && rows > l.max_rows) f |= kBadRows;
  if (n < 0 || (l.op != kOpCacheWrite && n > l.max_k)) f |= kBadSeqlen;
  if (l.op == kOpAppend && rows > n) f |= kBadAppend;
  if (l.op == kOpBackward) {
    const int64_t k0 = cu_k[b], k1 = cu_k[b + 1];
    if ((b == 0 && k0 != 0) || k1 - k0 != n || (b == l.batch - 1 && k1 != l.total_k)) f |= kBadCuK;
  }
  if ((f & (kBadCu | kBadSeqlen)) || block_table == nullptr) return f;  // (the merge reads no block ids)
  const int32_t* row = block_table + static_cast<int64_t>(b) * l.mbps;
  if (l.op == kOpCacheWrite) {
    if (rows > 0) {
      const int64_t last = n + rows - 1;  // the last written position
      if (last >= static_cast<int64_t>(l.mbps) * l.bs) f |= kBadWritePos;
      else f |= check_block_ids(row, n / l.bs, last / l.bs, l.num_blocks);
    }
  } else if ((rows > 0 || l.op == kOpBackward) && n > 0) {
    f |= check_block_ids(row, 0, (n - 1) / l.bs, l.num_blocks);
  }
  return f;
}

}  // namespace pkv
