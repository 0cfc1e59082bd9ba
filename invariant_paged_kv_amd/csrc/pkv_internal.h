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
  int32_t causal;
  float mul;       // score multiplier: scale (fp32) or scale*log2(e) (bf16)
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
};

struct LaunchPlan {
  bool full;       // prefill kernel (true) or split kernels + merge (false)
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
};

hipError_t launch_attention(const AttnArgs& a, const LaunchPlan& pl, int dtype, int d, hipStream_t stream);
hipError_t launch_cache_write(const CacheWriteArgs& a, int elem_bytes, int64_t total_new, hipStream_t stream);

}  // namespace pkv
