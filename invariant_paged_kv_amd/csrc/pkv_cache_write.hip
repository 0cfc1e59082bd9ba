// pkv_cache_write.hip -- append new K/V rows to the paged cache (bit copy).
//
// RL-Kernel issue #152 "[WS1] KV-cache path consistency (prefill & decode)",
// section Scope: the cache write must not change the stored values, so the
// path that wrote the cache and the path that reads it see the same bits.
// Token t of sequence b lands at key position seqlens_k[b] + t: block
// block_table[b][pos / block_size], slot pos % block_size, addressed with the
// cache's real strides (aiter commit d293d61bbf19: contiguous or
// K/V-interleaved blocks).
#include "pkv_internal.h"

namespace pkv {

typedef uint32_t u32x4_cw __attribute__((ext_vector_type(4)));

// One work group per new token; threads copy 16-byte pieces of the token's
// K and V rows (all KV heads).  A thread's first piece is loaded before the
// token's position is looked up (its source does not depend on it), so the
// lookup's loads and the row's load are in flight together.
__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteArgs a, int eb) {
  if (dbg_skip(a.dbg_word)) return;
  const int64_t tok = blockIdx.x;
  const int cpr = a.row_bytes / 16;
  const int per_tensor = a.hk * cpr;
  const int npieces = 2 * per_tensor;
  auto src_of = [&](int i) {
    const int tensor = i / per_tensor;
    const int rem = i - tensor * per_tensor;
    return static_cast<const unsigned char*>(tensor ? a.v_new : a.k_new) + (tok * a.hk + rem / cpr) * a.row_bytes +
           16 * (rem % cpr);
  };
  const int i0 = static_cast<int>(threadIdx.x);
  u32x4_cw first = {0, 0, 0, 0};
  if (i0 < npieces) first = *reinterpret_cast<const u32x4_cw*>(src_of(i0));
  const SeqOfRow sr = seq_of_row(a.cu_new, a.seqlens_k, a.batch, tok);
  const int b = sr.b;
  if (b >= a.batch) return;
  const int pos = sr.n + static_cast<int>(tok - sr.cu0);
  const int bi = div_block(pos, a.bs_mul, a.bs_shift);
  const int64_t blk = a.block_table[(int64_t)b * a.mbps + bi];
  const int64_t slot = pos - bi * a.bs;
  for (int i = i0; i < npieces; i += blockDim.x) {
    const int tensor = i / per_tensor;
    const int rem = i - tensor * per_tensor;
    const int h = rem / cpr;
    const int part = rem - h * cpr;
    const u32x4_cw val = i == i0 ? first : *reinterpret_cast<const u32x4_cw*>(src_of(i));
    const int64_t off = tensor ? (blk * a.vbs + slot * a.vss + h * a.vhs) : (blk * a.kbs + slot * a.kss + h * a.khs);
    unsigned char* dst = static_cast<unsigned char*>(tensor ? a.v_cache : a.k_cache) + off * eb + 16 * part;
    *reinterpret_cast<u32x4_cw*>(dst) = val;
  }
}

hipError_t launch_cache_write(const CacheWriteArgs& a, int elem_bytes, int64_t total_new, hipStream_t stream) {
  (void)hipGetLastError();
  if (total_new == 0) return hipSuccess;
  hipLaunchKernelGGL(cache_write_kernel, dim3(static_cast<unsigned>(total_new)), dim3(256), 0, stream, a, elem_bytes);
  return hipGetLastError();
}

}  // namespace pkv
