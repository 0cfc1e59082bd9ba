// pkv_internal.h -- argument blocks shared by the host launcher and the kernels
// of libpkv.  Not part of the public ABI (include/pkv.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Arguments of attn_kernel (both paths).  Strides are in elements.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_table;
  const int32_t* seqlens_k;
  const int32_t* cu_q;
  void* out;
  float* lse;
  float* part_o;   // split path: [total_q, Hq, maxc, d] fp32
  float* part_ml;  // split path: [total_q, Hq, maxc, 2] fp32 (max, sum)
  int64_t kbs, kss, khs, vbs, vss, vhs;
  int32_t hq, g, bs, mbps;
  int32_t ncb;     // column blocks per (sequence, KV head)
  int32_t maxc;    // chunk capacity of the partial buffers
  int32_t cpi;     // chunks per split work item
  int32_t chunk0;  // split path: global chunks [chunk0, chunk1) are computed
  int32_t chunk1;
  int64_t ps_row;    // partial index of (row*Hq + head, chunk c) = rowhead*ps_row + c*ps_chunk
  int64_t ps_chunk;
  int32_t causal;
  float mul;       // score multiplier: scale * k_scale (fp32), times log2(e) for base-2 types
  float v_scale;   // stored-V scale, applied at the final write (1: unscaled)
  uint32_t bs_mul; // j / bs == (j * bs_mul) >> bs_shift for 0 <= j < 2^30
  int32_t bs_shift;
  // Fused append (pkv_attn_forward_append): the K/V rows of this call's query
  // rows, [total_q, Hkv, d]; row r of sequence b holds key position
  // seqlens_k[b] - L_b + r.  Reads of those positions take them from here and
  // one work group per (sequence, KV head) stores them into the cache.
  const void* k_new;
  const void* v_new;
  void* k_store;
  void* v_store;
  // One-wave decode kernels: when set, work item x of a one-dimensional grid
  // takes the x-th job of a longest-first list -- every full 1024-key chunk of
  // every (sequence, KV head) in (sequence, head, chunk) order, then the
  // partial last chunks -- from the per-sequence prefix counts written by
  // decode_plan_kernel: job_pref[b] = full chunks of sequences < b (b <= batch),
  // job_pref[batch + 1 + b] = partial chunks of sequences < b.
  const int32_t* job_pref;
  int32_t nbatch;
  int32_t nhk;
  // Debug mode: the device error word the call's check kernel wrote; every
  // kernel of the call returns at once when it is nonzero.  NULL otherwise.
  const int32_t* dbg_word;
  // One-wave decode kernels, plain grid: dispatch order of the work items
  // (0: items of one (sequence, KV head) consecutive; 1: sequence fastest).
  int32_t dorder;
  // Split kernels: every column's visible keys lie in chunk 0 (at most 1024
  // keys per sequence), so a row's fold has a single term; the kernels write
  // out / lse themselves instead of partials, and no merge is launched.
  int32_t direct;
};

struct MergeArgs {
  const int32_t* cu_q;
  const int32_t* seqlens_k;
  const float* part_o;
  const float* part_ml;
  void* out;
  float* lse;
  int64_t total_q;
  int32_t batch, hq, maxc, causal;
  float v_scale;
  int64_t ps_row, ps_chunk;  // partial layout, as in AttnArgs
  const int32_t* dbg_word;   // as in AttnArgs
};

// Column groups of 16 per wave in the 4-wave split kernel (more than 16
// columns per KV head): each K/V tile read serves 16 * 4 * kSplitGroups columns.
#ifndef PKV_SPLIT_NT
#define PKV_SPLIT_NT 2
#endif
constexpr int kSplitGroups = PKV_SPLIT_NT;

struct LaunchPlan {
  bool full;       // prefill kernel (true) or split kernels + merge (false)
  bool full4;      // full path, bf16/FP8: 4 waves x 32 columns (attn_kernel) instead of the 8-wave pipelined kernel
  bool full8;      // full path, bf16/FP8, no fused append: 8 waves x 32 columns (attn_kernel), one work group per CU
  bool lpt;        // split path, one-wave kernels: longest-first job list (AttnArgs::job_pref)
  bool two_stage;  // split path, one-wave bf16 kernel: two tiles in flight (decode2_kernel)
  bool append;     // fused append of k_new / v_new
  bool skip_merge; // split path: write the chunk partials only
  bool direct;     // split path: out / lse written by the split kernels (AttnArgs::direct), no merge
  int fold_waves;  // split path, one-wave bf16 kernel: 0, or waves per work group folding its chunks (no merge)
  int waves;       // split path: waves per work group (1 or 4)
  int items;       // split path: work items per column block along the keys
  int batch, hk;
  int64_t total_q;
};

struct CacheWriteArgs {
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  const int32_t* block_table;
  const int32_t* seqlens_k;
  const int32_t* cu_new;
  int64_t kbs, kss, khs, vbs, vss, vhs;
  int32_t batch, hk, bs, mbps, row_bytes;
  uint32_t bs_mul;
  int32_t bs_shift;
  const int32_t* dbg_word;  // as in AttnArgs
};

// True when debug mode found bad device data for this call (or an earlier
// one not yet collected by pkv_check_device_errors): the kernel does nothing.
__device__ __forceinline__ bool dbg_skip(const int32_t* w) {
  return w != nullptr && *w != 0;
}

// Division by the block size as a multiply and shift: with l = ceil(log2 bs),
// s = 30 + l and m = ceil(2^s / bs), floor(j / bs) == (j * m) >> s for every
// 0 <= j < 2^30 (m*bs = 2^s + e with 0 <= e < bs, so the error term
// j*e / (bs * 2^s) < 2^-l <= 1/bs never crosses an integer), and m < 2^32.
inline void block_size_divisor(int32_t bs, uint32_t* mul, int32_t* shift) {
  int l = 0;
  while ((int64_t{1} << l) < bs) ++l;
  const int s = 30 + l;
  *mul = static_cast<uint32_t>(((uint64_t{1} << s) + static_cast<uint64_t>(bs) - 1) / static_cast<uint64_t>(bs));
  *shift = s;
}

__device__ __forceinline__ int div_block(int j, uint32_t mul, int shift) {
  return static_cast<int>((static_cast<uint64_t>(static_cast<uint32_t>(j)) * mul) >> shift);
}

// The sequence of packed row `row`: the largest b in [0, batch] with
// cu[b] <= row (cu nondecreasing from cu[0] = 0, so rows at or past
// cu[batch] give batch).  A 64-way search by the whole wave (row must be the
// same in every lane and every lane active): each round the lanes probe 64
// evenly spaced offsets and a ballot counts those <= row, so batches of up to
// 64 sequences take one round of loads, up to 4096 two, instead of one
// dependent load per halving.
__device__ __forceinline__ int row_sequence(const int32_t* cu, int batch, int64_t row) {
  int lo = 0, hi = batch;
  while (lo < hi) {
    const int stride = (hi - lo + 63) >> 6;
    const int p = lo + (static_cast<int>(__lane_id()) + 1) * stride;
    const bool le = p <= hi && cu[p] <= row;
    const int c = __popcll(__ballot(le));
    hi = min(hi, lo + (c + 1) * stride - 1);
    lo += c * stride;
  }
  return lo;
}

// row_sequence together with that sequence's row offsets cu[b], cu[b + 1]
// and its length seqlens[b] (b < batch; with b == batch the row lies past the
// last sequence and the other fields are unset).  For batches of up to 63
// sequences every lane loads its own sequence's three values in the same
// round as the probe, and the wave takes sequence b's from lane b: one round
// of dependent loads instead of two.  Same whole-wave, uniform-row contract
// as row_sequence.
struct SeqOfRow {
  int b, cu0, cu1, n;
};
__device__ __forceinline__ SeqOfRow seq_of_row(const int32_t* cu, const int32_t* seqlens, int batch, int64_t row) {
  SeqOfRow r{batch, 0, 0, 0};
  if (batch <= 0) return r;
  if (batch < 64) {
    const int lane = static_cast<int>(__lane_id());
    const int c0 = cu[min(lane, batch)];          // lanes past the batch re-read the last entry
    const int c1 = cu[min(lane + 1, batch)];
    const int sn = seqlens[min(lane, batch - 1)];
    r.b = __popcll(__ballot(lane < batch && c1 <= row));
    if (r.b < batch) {
      r.cu0 = __builtin_amdgcn_readlane(c0, r.b);
      r.cu1 = __builtin_amdgcn_readlane(c1, r.b);
      r.n = __builtin_amdgcn_readlane(sn, r.b);
    }
    return r;
  }
  r.b = row_sequence(cu, batch, row);
  if (r.b < batch) {
    r.cu0 = cu[r.b];
    r.cu1 = cu[r.b + 1];
    r.n = seqlens[r.b];
  }
  return r;
}

// Arguments of the backward kernels.  `f` carries the forward's inputs
// (q, caches, table, lengths, strides, GQA factor, block-size divisor,
// causal flag; f.mul is the score multiplier of the forward).
struct BwdArgs {
  AttnArgs f;
  const int32_t* cu_k;  // [batch + 1] row offsets of each sequence's keys in dk/dv
  const void* out;      // forward output [total_q, Hq, d]
  const float* lse;     // forward natural-log LSE [total_q, Hq]
  const void* dout;     // cotangent of out [total_q, Hq, d]
  void* dq;             // [total_q, Hq, d]
  void* dk;             // [total_k, Hkv, d]
  void* dv;             // [total_k, Hkv, d]
  float* delta;         // workspace [total_q, Hq]: <dout, out> per (row, head)
  float scale;          // softmax scale (multiplies the dq and dk sums)
  int32_t nkb;          // key blocks per (sequence, KV head) of the dk/dv kernel
};

struct BwdPlan {
  int batch, hk;
  int64_t total_q;
  int64_t cols;  // max_seqlen_q * (Hq / Hkv): columns per (sequence, KV head)
  int64_t max_k; // bound on seqlens_k
};

hipError_t launch_attention(const AttnArgs& a, const LaunchPlan& pl, int dtype, int d, hipStream_t stream);
// Debug mode: one thread per sequence checks the call's index data
// (pkv_checks.h) and ORs its flags into word[0], the lowest bad sequence into
// word[1] (atomic min).
struct CheckLimits;
hipError_t launch_check(const CheckLimits& l, const int32_t* cu, const int32_t* sk, const int32_t* block_table,
                        const int32_t* cu_k, int32_t* word, hipStream_t stream);
hipError_t launch_backward(const BwdArgs& a, const BwdPlan& pl, int dtype, int d, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& m, int dtype, int d, hipStream_t stream);
hipError_t launch_cache_write(const CacheWriteArgs& a, int elem_bytes, int64_t total_new, hipStream_t stream);

}  // namespace pkv
