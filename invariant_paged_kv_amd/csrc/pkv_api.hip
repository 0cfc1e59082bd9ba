// pkv_api.hip -- host side of libpkv: the C ABI declared in include/pkv.h.
//
// Validates every argument on the host before anything is launched, picks the
// path (split + merge for few query columns per KV head, full/prefill kernel
// otherwise), sizes the split path's fp32 partial buffers, and enqueues the
// kernels on the caller's stream.  No host synchronisation, no exceptions
// across the boundary: every entry point returns a pkv_status code and leaves
// a message for pkv_last_error().
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "pkv.h"
#include "pkv_checks.h"
#include "pkv_internal.h"

// Device scratch of pkv_attn_forward_noalloc: the split path's chunk
// partials (and job-order counts) for callers that cannot allocate.  Every
// GPU the library runs on holds its own copy until the process ends.  In host
// code `scratch` is only a stand-in for the symbol; its device address on
// each GPU comes from hipGetSymbolAddress and is kept per device
// (g_scratch_ptr); only that address is ever handed to a kernel or copy.
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_MAX_BYTES];

// Debug mode's error word on each GPU: [0] violation flags (pkv_checks.h),
// [1] 0x7fffffff minus the lowest bad sequence (0: none).  Sticky until
// pkv_check_device_errors reads and clears it.
static __device__ __align__(256) int32_t dbg_word[4];

namespace {

constexpr size_t kScratchBytes = PKV_NOALLOC_MAX_BYTES;
constexpr int kChunk = PKV_CHUNK_KEYS;
static_assert(PKV_CHUNK_KEYS == 1024 && PKV_TILE_KEYS == 64, "header constants must match the device code");

thread_local char g_msg[512] = "";
std::atomic<int64_t> g_opt_path{0};
std::atomic<int64_t> g_opt_split_chunks{0};
std::atomic<int64_t> g_opt_full_kernel{0};
std::atomic<int64_t> g_opt_decode_order{0};
// Debug mode: PKV_OPT_DEBUG, initially on when the environment sets PKV_DEBUG to a nonzero value.
int64_t env_debug() {
  const char* e = std::getenv("PKV_DEBUG");
  return (e && *e && std::strcmp(e, "0") != 0) ? 1 : 0;
}
std::atomic<int64_t> g_opt_debug{env_debug()};
#ifndef PKV_DECODE_LPT
#define PKV_DECODE_LPT 1
#endif
#ifndef PKV_DECODE_FOLD
#define PKV_DECODE_FOLD 1
#endif

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof g_msg, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_msg[0] = '\0';
  return PKV_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address, looked up once per device (with that
// device current) on the first call that needs it.
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(PKV_ERR_HIP, "no usable current device for the static scratch (device %d)", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PKV_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

// The current device's debug error word, looked up (and cleared) once per
// device; debug mode only.
int32_t* g_dbg_ptr[kMaxDevices] = {};

int dbg_word_ptr(int32_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(PKV_ERR_HIP, "no usable current device for the debug error word (device %d)", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_dbg_ptr[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(dbg_word));
    const int32_t zero[4] = {0, 0, 0, 0};
    if (e == hipSuccess && p) e = hipMemcpy(p, zero, sizeof zero, hipMemcpyHostToDevice);
    if (e != hipSuccess || !p)
      return fail(PKV_ERR_HIP, "debug error word on device %d: %s", dev, hipGetErrorString(e));
    g_dbg_ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = g_dbg_ptr[dev];
  return PKV_OK;
}

// Debug mode (PKV_OPT_DEBUG): enqueue the check kernel of the call's index
// data ahead of its kernels and hand them the error word; otherwise nothing
// (*word = NULL: the kernels skip no work).
int debug_check(const pkv::CheckLimits& lim, const int32_t* cu, const int32_t* sk, const int32_t* bt,
                const int32_t* cu_k, hipStream_t stream, const int32_t** word) {
  *word = nullptr;
  if (!g_opt_debug.load()) return PKV_OK;
  int32_t* w = nullptr;
  int rc = dbg_word_ptr(&w);
  if (rc) return rc;
  const hipError_t e = pkv::launch_check(lim, cu, sk, bt, cu_k, w, stream);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "debug check launch failed: %s", hipGetErrorString(e));
  *word = w;
  return PKV_OK;
}

int64_t max_seqlen_k_of(const pkv_layout& l);

pkv::CheckLimits check_limits(const pkv_layout& l, int op, int64_t total_rows) {
  pkv::CheckLimits c{};
  c.total_rows = total_rows;
  c.max_k = op == pkv::kOpCacheWrite ? static_cast<int64_t>(l.max_blocks_per_seq) * l.block_size : max_seqlen_k_of(l);
  c.num_blocks = l.num_blocks;
  c.max_rows = l.max_seqlen_q;
  c.mbps = l.max_blocks_per_seq;
  c.bs = l.block_size;
  c.batch = l.batch;
  c.op = op;
  return c;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Bytes per element of the cache / new K/V rows, and of q / out.
int elem_bytes(int dtype) { return dtype == PKV_F32 ? 4 : dtype == PKV_BF16 ? 2 : 1; }
int q_elem_bytes(int dtype) { return dtype == PKV_F32 ? 4 : 2; }

// Stored-value scales: 0 means 1.
float kv_scale(float s) { return s == 0.f ? 1.f : s; }

// Score multiplier: softmax_scale * k_scale, times log2(e) for the base-2
// (bf16-computing) types; one rounding, from double.
float score_mul(const pkv_layout& l, float softmax_scale) {
  double m = static_cast<double>(softmax_scale) * static_cast<double>(kv_scale(l.k_scale));
  if (l.dtype != PKV_F32) m *= 1.4426950408889634074;
  return static_cast<float>(m);
}

int64_t max_seqlen_k_of(const pkv_layout& l) {
  const int64_t cap = static_cast<int64_t>(l.max_blocks_per_seq) * l.block_size;
  return (l.max_seqlen_k > 0 && l.max_seqlen_k < cap) ? l.max_seqlen_k : cap;
}

int validate(const pkv_layout* l) {
  if (!l) return fail(PKV_ERR_NULL, "kv_strides (layout) is NULL");
  if (l->dtype != PKV_F32 && l->dtype != PKV_BF16 && l->dtype != PKV_FP8_E4M3)
    return fail(PKV_ERR_DTYPE, "dtype %d is not PKV_F32, PKV_BF16 or PKV_FP8_E4M3", l->dtype);
  if (!std::isfinite(l->k_scale) || !std::isfinite(l->v_scale) || l->k_scale < 0.f || l->v_scale < 0.f)
    return fail(PKV_ERR_SHAPE, "k_scale and v_scale must be finite and >= 0 (0 means 1)");
  if (l->batch < 0) return fail(PKV_ERR_SHAPE, "batch %d < 0", l->batch);
  if (l->num_heads_k < 1 || l->num_heads_q < 1 || l->num_heads_q % l->num_heads_k != 0)
    return fail(PKV_ERR_SHAPE, "num_heads_q %d must be a positive multiple of num_heads_k %d", l->num_heads_q, l->num_heads_k);
  // launch-grid limits: sequences and KV heads are grid dimensions of at most
  // 65535, and (row, query head) pairs are counted in 31 bits
  if (l->batch > 65535 || l->num_heads_k > 65535)
    return fail(PKV_ERR_SHAPE, "batch %d and num_heads_k %d must be at most 65535", l->batch, l->num_heads_k);
  if (l->total_q > 0 && static_cast<int64_t>(l->total_q) * l->num_heads_q > INT32_MAX)
    return fail(PKV_ERR_SHAPE, "total_q * num_heads_q exceeds 2^31 - 1");
  if (l->head_dim != 64 && l->head_dim != 128) return fail(PKV_ERR_SHAPE, "head_dim %d is not 64 or 128", l->head_dim);
  if (l->block_size < 1) return fail(PKV_ERR_SHAPE, "block_size %d < 1", l->block_size);
  if (l->max_blocks_per_seq < 0) return fail(PKV_ERR_SHAPE, "max_blocks_per_seq %d < 0", l->max_blocks_per_seq);
  if (static_cast<int64_t>(l->max_blocks_per_seq) * l->block_size > (int64_t{1} << 30))
    return fail(PKV_ERR_SHAPE, "max_blocks_per_seq * block_size exceeds 2^30 keys");
  if (l->max_seqlen_q < 0 || l->total_q < 0 || l->max_seqlen_k < 0 || l->num_blocks < 0)
    return fail(PKV_ERR_SHAPE, "negative max_seqlen_q, max_seqlen_k, total_q or num_blocks");
  if (static_cast<int64_t>(l->max_seqlen_q) * (l->num_heads_q / l->num_heads_k) > (int64_t{1} << 30))
    return fail(PKV_ERR_SHAPE, "max_seqlen_q * (num_heads_q / num_heads_k) too large");
  const int64_t s[6] = {l->k_block_stride, l->k_slot_stride, l->k_head_stride,
                        l->v_block_stride, l->v_slot_stride, l->v_head_stride};
  const int eb = elem_bytes(l->dtype);
  for (int i = 0; i < 6; ++i) {
    if (s[i] < 0) return fail(PKV_ERR_SHAPE, "negative cache stride");
    if ((s[i] * eb) % 16 != 0) return fail(PKV_ERR_ALIGN, "cache stride %lld elements is not a multiple of 16 bytes", (long long)s[i]);
  }
  return ok();
}

struct Plan {
  pkv::LaunchPlan lp;
  int ncb;
  int maxc;
  int cpi;
  size_t ws_bytes;
  size_t off_ml;
  size_t off_jobs;  // longest-first job list: prefix counts (lp.lpt)
  bool grid_ok;  // work items along the first grid dimension fit in 31 bits
};

size_t round256(size_t x) { return (x + 255) & ~size_t{255}; }

Plan make_plan(const pkv_layout& l, bool append = false) {
  Plan p{};
  const int g = l.num_heads_q / l.num_heads_k;
  const int64_t cols = static_cast<int64_t>(l.max_seqlen_q) * g;
  const int64_t mk = max_seqlen_k_of(l);
  p.maxc = static_cast<int>((mk + kChunk - 1) / kChunk);
  const int64_t force = g_opt_path.load();
  bool full;
  int waves = 1;
  if (force == 1) {
    full = false;
  } else if (force == 2) {
    full = true;
  } else if (cols <= 16) {
    full = false;
  } else {
    const int64_t full_items = static_cast<int64_t>(l.batch) * l.num_heads_k * ((cols + 127) / 128);
    full = full_items >= 512;
  }
  if (!full) waves = cols <= 16 ? 1 : 4;
  // bf16/FP8 full path: 4 waves x 32 columns per work group (two column
  // groups per wave: every K/V tile read from LDS serves 32 columns) unless
  // the pipelined 8-wave x 16-column kernel is asked for; both give the same
  // bits.  Measured on the 8 x 8192 prefill 609-618 against 441 TFLOP/s, and
  // on 64 rows x 131072 keys 560-565 against 366.
  // bf16/FP8 full path: 8 waves x 32 columns (one work group per CU, 256
  // columns sharing each K/V tile stream) when a (sequence, KV head) has few
  // columns over a long context -- the re-score of a generated sequence, where
  // every column block streams the whole cache: 64-256 rows x 32768-131072
  // keys measured 5-9% faster, 1024 columns 2%; with more columns per KV head
  // the 4-wave kernel's extra work groups balance better (2800-8192 columns:
  // 1-11% slower with 8 waves, 32768: equal).  Both give the same bits.
  bool full4 = false, full8 = false;
  if (full && l.dtype != PKV_F32) {
    const int64_t fk = g_opt_full_kernel.load();
    full4 = fk != 1;
    full8 = !append && (fk == 3 || (fk == 0 && cols <= 1024 && mk >= 16384));
  }
  p.lp.full4 = full4;
  p.lp.full8 = full8;
  const int cols_per_block = full ? (full8 ? 256 : 128) : (waves == 1 ? 16 : 16 * 4 * pkv::kSplitGroups);
  p.ncb = static_cast<int>(std::max<int64_t>(1, (cols + cols_per_block - 1) / cols_per_block));
  int64_t cpi = g_opt_split_chunks.load();
  if (cpi <= 0) cpi = 1;
  p.cpi = static_cast<int>(cpi);
  p.lp.full = full;
  p.lp.waves = waves;
  p.lp.items = std::max(1, (p.maxc + p.cpi - 1) / p.cpi);
  p.grid_ok = static_cast<int64_t>(p.ncb) * (full ? 1 : p.lp.items) <= INT32_MAX;
  // One-wave bf16/FP8 decode kernels: a longest-first job list (same bits)
  // when the sequences span few chunks, so that their partial last chunks are
  // a large share of the jobs, and the jobs exceed one round of wave slots
  // (256 CUs x 8 waves): a ragged batch of 128 sequences of up to 8192 keys
  // measured 0.592 -> 0.409 ms.  Its extra plan launch (a few us) is not
  // repaid by uniform batches or long contexts (64 x 4096: +3.7%, 16 x
  // 131072: +0.4%).
  const int64_t jobs = static_cast<int64_t>(l.batch) * l.num_heads_k * p.maxc;
  // Every sequence within one 1024-key chunk: a row's fold has one term, so
  // the split kernels write out / lse themselves (the merge's operations on
  // that term) -- no partials, no workspace, no merge launch.
  p.lp.direct = !full && p.maxc == 1;
  p.lp.lpt = PKV_DECODE_LPT && !full && waves == 1 && l.dtype != PKV_F32 && p.cpi == 1 && p.maxc <= 16 &&
             jobs > 2048 && jobs <= INT32_MAX && !p.lp.direct;
  // One-wave bf16 decode: the two-stage kernel (two tiles in flight, 416
  // registers, one wave per SIMD; same bits) once the grid exceeds one round
  // of one-wave slots (256 CUs x 4 SIMDs).  In-process A/B against the
  // one-stage kernel (two waves per SIMD): 128 ragged sequences of up to 8192
  // keys 0.407 -> 0.393 ms, 16 x 131072 keys 1.484 -> 1.476 ms; 64 x 4096
  // keys (1024 work items) 0.108 -> 0.110, hence the condition.
  p.lp.two_stage = !full && waves == 1 && l.dtype == PKV_BF16 &&
                   static_cast<int64_t>(p.lp.items) * l.num_heads_k * l.batch > 1024;
  // One-wave bf16 decode in one round of wave slots over two chunks, with at
  // least one (sequence, KV head) per CU: one work group per (sequence, KV
  // head) whose two waves take a chunk each and fold them in LDS -- no
  // partials in HBM and no merge launch (same bits; measured 5% faster).
  if (!full && waves == 1 && l.dtype == PKV_BF16 && !append && !p.lp.two_stage && !p.lp.lpt && !p.lp.direct &&
      p.cpi == 1 && p.maxc == 2 && static_cast<int64_t>(l.batch) * l.num_heads_k * p.ncb >= 256 && PKV_DECODE_FOLD)
    p.lp.fold_waves = 2;
  p.lp.batch = l.batch;
  p.lp.hk = l.num_heads_k;
  p.lp.total_q = l.total_q;
  if (full || l.total_q == 0 || p.maxc == 0 || p.lp.direct || p.lp.fold_waves) {
    p.ws_bytes = 0;
    p.lp.lpt = false;
  } else {
    const size_t parts = static_cast<size_t>(l.total_q) * l.num_heads_q * p.maxc;
    p.off_ml = round256(parts * l.head_dim * sizeof(float));
    p.ws_bytes = p.off_ml + round256(parts * 2 * sizeof(float));
    if (p.lp.lpt) {  // prefix counts of the job list: 2 * (batch + 1) int32
      p.off_jobs = p.ws_bytes;
      p.ws_bytes += round256((2 * static_cast<size_t>(l.batch) + 2) * sizeof(int32_t));
    }
  }
  return p;
}

int check_attn_ptrs(const void* q, const void* k, const void* v, const int32_t* bt, const int32_t* sk,
                    const int32_t* cu, const void* out, const float* lse, const pkv_layout& l) {
  if (l.total_q > 0 && (!q || !out || !lse)) return fail(PKV_ERR_NULL, "q, out or lse is NULL");
  if (l.batch > 0 && (!sk || !cu)) return fail(PKV_ERR_NULL, "seqlens_k or cu_seqlens_q is NULL");
  if (l.batch > 0 && l.max_blocks_per_seq > 0 && (!k || !v || !bt)) return fail(PKV_ERR_NULL, "k_cache, v_cache or block_table is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(PKV_ERR_ALIGN, "q, k_cache, v_cache and out must be 16-byte aligned");
  return PKV_OK;
}

int run_attention(const void* q, const void* k_cache, const void* v_cache, const pkv_layout* l,
                  const int32_t* block_table, const int32_t* seqlens_k, const int32_t* cu_seqlens_q, int causal,
                  float softmax_scale, void* out, float* lse, void* ws, size_t ws_bytes, bool own_ws,
                  hipStream_t stream, const void* k_new = nullptr, const void* v_new = nullptr,
                  void* k_store = nullptr, void* v_store = nullptr) {
  int rc = validate(l);
  if (rc) return rc;
  rc = check_attn_ptrs(q, k_cache, v_cache, block_table, seqlens_k, cu_seqlens_q, out, lse, *l);
  if (rc) return rc;
  const bool append = k_store != nullptr;
  if (append && l->total_q > 0 && (!k_new || !v_new)) return fail(PKV_ERR_NULL, "k_new or v_new is NULL");
  if (append && (!aligned16(k_new) || !aligned16(v_new)))
    return fail(PKV_ERR_ALIGN, "k_new and v_new must be 16-byte aligned");
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return fail(PKV_ERR_SHAPE, "softmax_scale must be finite and > 0");
  if (l->batch == 0 || l->total_q == 0) return ok();
  Plan p = make_plan(*l, append);
  p.lp.append = append;
  if (!p.grid_ok) return fail(PKV_ERR_SHAPE, "too many column blocks x key splits for one launch");
  bool allocated = false;
  if (p.ws_bytes > 0) {
    if (own_ws) {
      if (hipMallocAsync(&ws, p.ws_bytes, stream) != hipSuccess)
        return fail(PKV_ERR_WORKSPACE, "hipMallocAsync of %zu workspace bytes failed", p.ws_bytes);
      allocated = true;
    } else if (!ws || ws_bytes < p.ws_bytes || !aligned16(ws)) {
      return fail(PKV_ERR_WORKSPACE, "workspace needs %zu bytes, 16-byte aligned (got %zu)", p.ws_bytes, ws_bytes);
    }
  }
  pkv::AttnArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.block_table = block_table;
  a.seqlens_k = seqlens_k;
  a.cu_q = cu_seqlens_q;
  a.out = out;
  a.lse = lse;
  a.part_o = p.ws_bytes ? static_cast<float*>(ws) : nullptr;
  a.part_ml = p.ws_bytes ? reinterpret_cast<float*>(static_cast<char*>(ws) + p.off_ml) : nullptr;
  a.kbs = l->k_block_stride;
  a.kss = l->k_slot_stride;
  a.khs = l->k_head_stride;
  a.vbs = l->v_block_stride;
  a.vss = l->v_slot_stride;
  a.vhs = l->v_head_stride;
  a.hq = l->num_heads_q;
  a.g = l->num_heads_q / l->num_heads_k;
  a.bs = l->block_size;
  a.mbps = l->max_blocks_per_seq;
  a.ncb = p.ncb;
  a.maxc = p.maxc;
  a.cpi = p.cpi;
  a.chunk0 = 0;
  a.chunk1 = p.maxc;
  a.ps_row = p.maxc;
  a.ps_chunk = 1;
  a.causal = causal ? 1 : 0;
  a.mul = score_mul(*l, softmax_scale);
  a.v_scale = kv_scale(l->v_scale);
  pkv::block_size_divisor(l->block_size, &a.bs_mul, &a.bs_shift);
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_store = k_store;
  a.v_store = v_store;
  a.job_pref = p.lp.lpt ? reinterpret_cast<const int32_t*>(static_cast<char*>(ws) + p.off_jobs) : nullptr;
  a.nbatch = l->batch;
  a.nhk = l->num_heads_k;
  a.direct = p.lp.direct ? 1 : 0;
  {
    // One-wave decode kernels: sequence-fastest dispatch for grids of at most
    // two rounds of wave slots whose (sequence, KV head) pairs span at least 4
    // work items; in one process, same bits, against items-consecutive order:
    // 64 x 4096 keys (Hq 16 / Hkv 4) 0.1095 -> 0.1002 ms, 16 x 16384 0.1166 ->
    // 0.1058, 8 x 32768 (32 / 8) 0.2191 -> 0.2106, 4 x 65536 (64 / 8) 0.2250 ->
    // 0.2153; 32 x 2048 (2 items) 0.0622 -> 0.0654 and 16 x 131072 (16384
    // work items) 1.4603 -> 1.4776 keep the items-consecutive order.
    const int64_t o = g_opt_decode_order.load();
    const int64_t total = static_cast<int64_t>(l->batch) * l->num_heads_k * p.ncb * p.lp.items;
    a.dorder = o == 0 ? (total <= 2048 && p.lp.items >= 4 ? 1 : 0) : static_cast<int32_t>(o - 1);
  }
  rc = debug_check(check_limits(*l, append ? pkv::kOpAppend : pkv::kOpAttention, l->total_q), cu_seqlens_q,
                   seqlens_k, block_table, nullptr, stream, &a.dbg_word);
  if (rc) {
    if (allocated) (void)hipFreeAsync(ws, stream);
    return rc;
  }
  hipError_t e = pkv::launch_attention(a, p.lp, l->dtype, l->head_dim, stream);
  if (allocated) {
    hipError_t fe = hipFreeAsync(ws, stream);
    if (e == hipSuccess && fe != hipSuccess) e = fe;
  }
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Context-parallel share: the chunk partials of global chunks [c0, c1), chunk-major.
int run_partials(const void* q, const void* k_cache, const void* v_cache, const pkv_layout* l,
                 const int32_t* block_table, const int32_t* seqlens_k, const int32_t* cu_seqlens_q, int causal,
                 float softmax_scale, int32_t c0, int32_t c1, int32_t max_chunks, float* part_o, float* part_ml,
                 hipStream_t stream) {
  int rc = validate(l);
  if (rc) return rc;
  rc = check_attn_ptrs(q, k_cache, v_cache, block_table, seqlens_k, cu_seqlens_q, part_o, part_ml, *l);
  if (rc) return rc;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return fail(PKV_ERR_SHAPE, "softmax_scale must be finite and > 0");
  if (max_chunks < 1 || c0 < 0 || c0 > c1 || c1 > max_chunks)
    return fail(PKV_ERR_SHAPE, "need 0 <= chunk_begin <= chunk_end <= max_chunks, max_chunks >= 1");
  if (!aligned16(part_ml)) return fail(PKV_ERR_ALIGN, "part_ml must be 16-byte aligned");
  if (l->batch == 0 || l->total_q == 0 || c0 == c1) return ok();
  const int g = l->num_heads_q / l->num_heads_k;
  const int64_t cols = static_cast<int64_t>(l->max_seqlen_q) * g;
  const int waves = cols <= 16 ? 1 : 4;
  int64_t cpi = g_opt_split_chunks.load();
  if (cpi <= 0) cpi = 1;
  pkv::LaunchPlan lp{};
  lp.full = false;
  lp.skip_merge = true;
  lp.waves = waves;
  lp.items = static_cast<int>((c1 - c0 + cpi - 1) / cpi);
  lp.batch = l->batch;
  lp.hk = l->num_heads_k;
  lp.total_q = l->total_q;
  pkv::AttnArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.block_table = block_table;
  a.seqlens_k = seqlens_k;
  a.cu_q = cu_seqlens_q;
  a.part_o = part_o;
  a.part_ml = part_ml;
  a.kbs = l->k_block_stride;
  a.kss = l->k_slot_stride;
  a.khs = l->k_head_stride;
  a.vbs = l->v_block_stride;
  a.vss = l->v_slot_stride;
  a.vhs = l->v_head_stride;
  a.hq = l->num_heads_q;
  a.g = g;
  a.bs = l->block_size;
  a.mbps = l->max_blocks_per_seq;
  const int cpb = waves == 1 ? 16 : 16 * 4 * pkv::kSplitGroups;
  a.ncb = static_cast<int>(std::max<int64_t>(1, (cols + cpb - 1) / cpb));
  if (static_cast<int64_t>(a.ncb) * lp.items > INT32_MAX)
    return fail(PKV_ERR_SHAPE, "too many column blocks x key splits for one launch");
  a.maxc = max_chunks;
  a.cpi = static_cast<int>(cpi);
  a.chunk0 = c0;
  a.chunk1 = c1;
  a.ps_row = 1;
  a.ps_chunk = l->total_q * l->num_heads_q;
  a.causal = causal ? 1 : 0;
  a.mul = score_mul(*l, softmax_scale);
  a.v_scale = kv_scale(l->v_scale);
  pkv::block_size_divisor(l->block_size, &a.bs_mul, &a.bs_shift);
  rc = debug_check(check_limits(*l, pkv::kOpAttention, l->total_q), cu_seqlens_q, seqlens_k, block_table, nullptr,
                   stream, &a.dbg_word);
  if (rc) return rc;
  hipError_t e = pkv::launch_attention(a, lp, l->dtype, l->head_dim, stream);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "partials launch failed: %s", hipGetErrorString(e));
  return ok();
}

int run_merge(const float* part_o, const float* part_ml, int32_t max_chunks, const pkv_layout* l,
              const int32_t* seqlens_k, const int32_t* cu_seqlens_q, int causal, void* out, float* lse,
              hipStream_t stream) {
  int rc = validate(l);
  if (rc) return rc;
  if (max_chunks < 1) return fail(PKV_ERR_SHAPE, "max_chunks must be >= 1");
  if (l->total_q > 0 && (!part_o || !part_ml || !out || !lse)) return fail(PKV_ERR_NULL, "a merge pointer is NULL");
  if (l->batch > 0 && (!seqlens_k || !cu_seqlens_q)) return fail(PKV_ERR_NULL, "seqlens_k or cu_seqlens_q is NULL");
  if (!aligned16(part_o) || !aligned16(part_ml)) return fail(PKV_ERR_ALIGN, "part_o and part_ml must be 16-byte aligned");
  if (l->batch == 0 || l->total_q == 0) return ok();
  pkv::MergeArgs m{};
  m.cu_q = cu_seqlens_q;
  m.seqlens_k = seqlens_k;
  m.part_o = part_o;
  m.part_ml = part_ml;
  m.out = out;
  m.lse = lse;
  m.total_q = l->total_q;
  m.batch = l->batch;
  m.hq = l->num_heads_q;
  m.maxc = max_chunks;
  m.causal = causal ? 1 : 0;
  m.v_scale = kv_scale(l->v_scale);
  m.ps_row = 1;
  m.ps_chunk = l->total_q * l->num_heads_q;
  rc = debug_check(check_limits(*l, pkv::kOpAttention, l->total_q), cu_seqlens_q, seqlens_k, nullptr, nullptr, stream,
                   &m.dbg_word);
  if (rc) return rc;
  hipError_t e = pkv::launch_merge(m, l->dtype, l->head_dim, stream);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "merge launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t backward_ws_bytes(const pkv_layout& l) {
  return round256(static_cast<size_t>(l.total_q) * l.num_heads_q * sizeof(float));
}

int run_backward(const void* q, const void* k_cache, const void* v_cache, const pkv_layout* l,
                 const int32_t* block_table, const int32_t* seqlens_k, const int32_t* cu_seqlens_q,
                 const int32_t* cu_seqlens_k, int64_t total_k, int causal, float softmax_scale, const void* out,
                 const float* lse, const void* dout, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                 hipStream_t stream) {
  int rc = validate(l);
  if (rc) return rc;
  if (l->dtype == PKV_FP8_E4M3) return fail(PKV_ERR_DTYPE, "the backward takes PKV_F32 or PKV_BF16 caches");
  if (kv_scale(l->k_scale) != 1.f || kv_scale(l->v_scale) != 1.f)
    return fail(PKV_ERR_SHAPE, "the backward requires k_scale = v_scale = 1");
  rc = check_attn_ptrs(q, k_cache, v_cache, block_table, seqlens_k, cu_seqlens_q, out, lse, *l);
  if (rc) return rc;
  if (total_k < 0) return fail(PKV_ERR_SHAPE, "total_k %lld < 0", (long long)total_k);
  if (l->total_q > 0 && (!dout || !dq)) return fail(PKV_ERR_NULL, "dout or dq is NULL");
  if (total_k > 0 && (!dk || !dv)) return fail(PKV_ERR_NULL, "dk or dv is NULL");
  if (l->batch > 0 && !cu_seqlens_k) return fail(PKV_ERR_NULL, "cu_seqlens_k is NULL");
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(PKV_ERR_ALIGN, "dout, dq, dk and dv must be 16-byte aligned");
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return fail(PKV_ERR_SHAPE, "softmax_scale must be finite and > 0");
  if (l->batch == 0 || (l->total_q == 0 && total_k == 0)) return ok();
  const size_t need = backward_ws_bytes(*l);
  bool allocated = false;
  if (need > 0) {
    if (!ws) {
      if (hipMallocAsync(&ws, need, stream) != hipSuccess)
        return fail(PKV_ERR_WORKSPACE, "hipMallocAsync of %zu workspace bytes failed", need);
      allocated = true;
    } else if (ws_bytes < need || !aligned16(ws)) {
      return fail(PKV_ERR_WORKSPACE, "backward workspace needs %zu bytes, 16-byte aligned (got %zu)", need, ws_bytes);
    }
  }
  constexpr int kWaves = 4;
  const int g = l->num_heads_q / l->num_heads_k;
  const int64_t cols = static_cast<int64_t>(l->max_seqlen_q) * g;
  const int64_t mk = max_seqlen_k_of(*l);
  pkv::BwdArgs b{};
  pkv::AttnArgs& a = b.f;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.block_table = block_table;
  a.seqlens_k = seqlens_k;
  a.cu_q = cu_seqlens_q;
  a.kbs = l->k_block_stride;
  a.kss = l->k_slot_stride;
  a.khs = l->k_head_stride;
  a.vbs = l->v_block_stride;
  a.vss = l->v_slot_stride;
  a.vhs = l->v_head_stride;
  a.hq = l->num_heads_q;
  a.g = g;
  a.bs = l->block_size;
  a.mbps = l->max_blocks_per_seq;
  a.ncb = static_cast<int>((cols + 16 * kWaves - 1) / (16 * kWaves));
  a.causal = causal ? 1 : 0;
  a.mul = score_mul(*l, softmax_scale);
  a.v_scale = kv_scale(l->v_scale);
  pkv::block_size_divisor(l->block_size, &a.bs_mul, &a.bs_shift);
  b.cu_k = cu_seqlens_k;
  b.out = out;
  b.lse = lse;
  b.dout = dout;
  b.dq = dq;
  b.dk = dk;
  b.dv = dv;
  b.delta = static_cast<float*>(ws);
  b.scale = softmax_scale;
  b.nkb = total_k > 0 ? static_cast<int>((mk + 16 * kWaves - 1) / (16 * kWaves)) : 0;
  pkv::BwdPlan pl{l->batch, l->num_heads_k, l->total_q, cols, mk};
  pkv::CheckLimits lim = check_limits(*l, pkv::kOpBackward, l->total_q);
  lim.total_k = total_k;
  rc = debug_check(lim, cu_seqlens_q, seqlens_k, block_table, cu_seqlens_k, stream, &a.dbg_word);
  if (rc) {
    if (allocated) (void)hipFreeAsync(ws, stream);
    return rc;
  }
  hipError_t e = pkv::launch_backward(b, pl, l->dtype, l->head_dim, stream);
  if (allocated) {
    hipError_t fe = hipFreeAsync(ws, stream);
    if (e == hipSuccess && fe != hipSuccess) e = fe;
  }
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
  return ok();
}


}  // namespace

extern "C" {

int pkv_validate_layout(const pkv_layout* kv_strides) { return validate(kv_strides); }

size_t pkv_attn_workspace_size(const pkv_layout* kv_strides) {
  if (validate(kv_strides) != PKV_OK) return 0;
  return make_plan(*kv_strides).ws_bytes;
}

int pkv_attn_forward(const void* q, const void* k_cache, const void* v_cache, const pkv_layout* kv_strides,
                     const int32_t* block_table, const int32_t* seqlens_k, const int32_t* cu_seqlens_q, int causal,
                     float softmax_scale, void* out, float* lse, hipStream_t stream) {
  return run_attention(q, k_cache, v_cache, kv_strides, block_table, seqlens_k, cu_seqlens_q, causal, softmax_scale,
                       out, lse, nullptr, 0, true, stream);
}

int pkv_attn_forward_ws(const void* q, const void* k_cache, const void* v_cache, const pkv_layout* kv_strides,
                        const int32_t* block_table, const int32_t* seqlens_k, const int32_t* cu_seqlens_q, int causal,
                        float softmax_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  return run_attention(q, k_cache, v_cache, kv_strides, block_table, seqlens_k, cu_seqlens_q, causal, softmax_scale,
                       out, lse, workspace, workspace_bytes, false, stream);
}

int pkv_attn_forward_noalloc(const void* q, const void* k_cache, const void* v_cache, const pkv_layout* kv_strides,
                             const int32_t* block_table, const int32_t* seqlens_k, const int32_t* cu_seqlens_q,
                             int causal, float softmax_scale, void* out, float* lse, hipStream_t stream) {
  // every host-side check first: nothing touches the device before they pass
  int rc = validate(kv_strides);
  if (rc) return rc;
  rc = check_attn_ptrs(q, k_cache, v_cache, block_table, seqlens_k, cu_seqlens_q, out, lse, *kv_strides);
  if (rc) return rc;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return fail(PKV_ERR_SHAPE, "softmax_scale must be finite and > 0");
  const size_t need = make_plan(*kv_strides).ws_bytes;
  if (need > kScratchBytes)
    return fail(PKV_ERR_WORKSPACE, "the split path needs %zu scratch bytes; the static scratch holds %zu "
                "(use pkv_attn_forward_ws with a caller workspace)", need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0 && kv_strides->batch > 0 && kv_strides->total_q > 0) {
    rc = scratch_ptr(&ws);
    if (rc) return rc;
  }
  return run_attention(q, k_cache, v_cache, kv_strides, block_table, seqlens_k, cu_seqlens_q, causal, softmax_scale,
                       out, lse, ws, ws ? kScratchBytes : 0, false, stream);
}

int pkv_attn_forward_append(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            const pkv_layout* kv_strides, const int32_t* block_table, const int32_t* seqlens_k,
                            const int32_t* cu_seqlens_q, int causal, float softmax_scale, void* out, float* lse,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!k_cache || !v_cache) return fail(PKV_ERR_NULL, "k_cache or v_cache is NULL");
  return run_attention(q, k_cache, v_cache, kv_strides, block_table, seqlens_k, cu_seqlens_q, causal, softmax_scale,
                       out, lse, workspace, workspace_bytes, workspace == nullptr, stream, k_new, v_new, k_cache,
                       v_cache);
}

int pkv_attn_backward(const void* q, const void* k_cache, const void* v_cache, const pkv_layout* kv_strides,
                      const int32_t* block_table, const int32_t* seqlens_k, const int32_t* cu_seqlens_q,
                      const int32_t* cu_seqlens_k, int64_t total_k, int causal, float softmax_scale, const void* out,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  return run_backward(q, k_cache, v_cache, kv_strides, block_table, seqlens_k, cu_seqlens_q, cu_seqlens_k, total_k,
                      causal, softmax_scale, out, lse, dout, dq, dk, dv, workspace, workspace_bytes, stream);
}

size_t pkv_attn_backward_workspace_size(const pkv_layout* kv_strides) {
  if (validate(kv_strides) != PKV_OK) return 0;
  return backward_ws_bytes(*kv_strides);
}

int pkv_attn_chunk_partials(const void* q, const void* k_cache, const void* v_cache, const pkv_layout* kv_strides,
                            const int32_t* block_table, const int32_t* seqlens_k, const int32_t* cu_seqlens_q,
                            int causal, float softmax_scale, int32_t chunk_begin, int32_t chunk_end,
                            int32_t max_chunks, float* part_o, float* part_ml, hipStream_t stream) {
  return run_partials(q, k_cache, v_cache, kv_strides, block_table, seqlens_k, cu_seqlens_q, causal, softmax_scale,
                      chunk_begin, chunk_end, max_chunks, part_o, part_ml, stream);
}

int pkv_attn_merge_partials(const float* part_o, const float* part_ml, int32_t max_chunks,
                            const pkv_layout* kv_strides, const int32_t* seqlens_k, const int32_t* cu_seqlens_q,
                            int causal, void* out, float* lse, hipStream_t stream) {
  return run_merge(part_o, part_ml, max_chunks, kv_strides, seqlens_k, cu_seqlens_q, causal, out, lse, stream);
}

int pkv_cache_write(const void* k_new, const void* v_new, void* k_cache, void* v_cache, const pkv_layout* l,
                    const int32_t* block_table, const int32_t* seqlens_k, const int32_t* cu_seqlens_new,
                    int64_t total_new, hipStream_t stream) {
  int rc = validate(l);
  if (rc) return rc;
  if (total_new < 0) return fail(PKV_ERR_SHAPE, "total_new %lld < 0", (long long)total_new);
  if (total_new > 0x7fffffff) return fail(PKV_ERR_SHAPE, "total_new %lld exceeds 2^31-1", (long long)total_new);
  if (total_new == 0 || l->batch == 0) return ok();
  if (!k_new || !v_new || !k_cache || !v_cache || !block_table || !seqlens_k || !cu_seqlens_new)
    return fail(PKV_ERR_NULL, "a cache_write pointer is NULL");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_ALIGN, "k_new, v_new, k_cache and v_cache must be 16-byte aligned");
  pkv::CacheWriteArgs a{};
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.seqlens_k = seqlens_k;
  a.cu_new = cu_seqlens_new;
  a.kbs = l->k_block_stride;
  a.kss = l->k_slot_stride;
  a.khs = l->k_head_stride;
  a.vbs = l->v_block_stride;
  a.vss = l->v_slot_stride;
  a.vhs = l->v_head_stride;
  a.batch = l->batch;
  a.hk = l->num_heads_k;
  a.bs = l->block_size;
  a.mbps = l->max_blocks_per_seq;
  a.row_bytes = l->head_dim * elem_bytes(l->dtype);
  pkv::block_size_divisor(l->block_size, &a.bs_mul, &a.bs_shift);
  rc = debug_check(check_limits(*l, pkv::kOpCacheWrite, total_new), cu_seqlens_new, seqlens_k, block_table, nullptr,
                   stream, &a.dbg_word);
  if (rc) return rc;
  hipError_t e = pkv::launch_cache_write(a, elem_bytes(l->dtype), total_new, stream);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "cache_write launch failed: %s", hipGetErrorString(e));
  return ok();
}

int pkv_check_device_errors(hipStream_t stream) {
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "stream synchronisation failed: %s", hipGetErrorString(e));
  e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "pending HIP error: %s", hipGetErrorString(e));
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ok();
  int32_t* w = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    w = g_dbg_ptr[dev];
  }
  if (!w) return ok();  // debug mode never ran on this device
  int32_t h[4] = {0, 0, 0, 0};
  e = hipMemcpy(h, w, sizeof h, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "reading the debug error word failed: %s", hipGetErrorString(e));
  if (h[0] == 0) return ok();
  const int32_t zero[4] = {0, 0, 0, 0};
  e = hipMemcpy(w, zero, sizeof zero, hipMemcpyHostToDevice);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "clearing the debug error word failed: %s", hipGetErrorString(e));
  return fail(PKV_ERR_DEVICE_DATA, "device data violates preconditions (flags 0x%x:%s%s%s%s%s%s%s), first at sequence %d",
              h[0], (h[0] & pkv::kBadCu) ? " cu_seqlens" : "", (h[0] & pkv::kBadSeqlen) ? " seqlens_k" : "",
              (h[0] & pkv::kBadBlockId) ? " block_id" : "", (h[0] & pkv::kBadRows) ? " rows>max_seqlen_q" : "",
              (h[0] & pkv::kBadAppend) ? " append_rows>keys" : "", (h[0] & pkv::kBadWritePos) ? " write_position" : "",
              (h[0] & pkv::kBadCuK) ? " cu_seqlens_k" : "", 0x7fffffff - h[1]);
}

int pkv_check_inputs(const pkv_layout* kv_strides, const int32_t* block_table, const int32_t* seqlens_k,
                     const int32_t* cu_seqlens, int64_t total_rows, int op) {
  int rc = validate(kv_strides);
  if (rc) return rc;
  if (op != PKV_CHECK_ATTENTION && op != PKV_CHECK_APPEND && op != PKV_CHECK_CACHE_WRITE)
    return fail(PKV_ERR_OPTION, "op %d is not PKV_CHECK_ATTENTION, PKV_CHECK_APPEND or PKV_CHECK_CACHE_WRITE", op);
  if (total_rows < 0) return fail(PKV_ERR_SHAPE, "total_rows %lld < 0", (long long)total_rows);
  if (kv_strides->batch == 0) return ok();
  if (!seqlens_k || !cu_seqlens || (kv_strides->max_blocks_per_seq > 0 && !block_table))
    return fail(PKV_ERR_NULL, "block_table, seqlens_k or cu_seqlens is NULL");
  const int cop = op == PKV_CHECK_ATTENTION ? pkv::kOpAttention : op == PKV_CHECK_APPEND ? pkv::kOpAppend : pkv::kOpCacheWrite;
  const pkv::CheckLimits lim = check_limits(*kv_strides, cop, total_rows);
  int32_t flags = 0;
  int first = -1;
  for (int b = 0; b < kv_strides->batch; ++b) {
    const int32_t f = pkv::check_sequence(lim, b, cu_seqlens, seqlens_k, block_table, nullptr);
    if (f && first < 0) first = b;
    flags |= f;
  }
  if (!flags) return ok();
  return fail(PKV_ERR_DEVICE_DATA, "index data violates preconditions (flags 0x%x:%s%s%s%s%s%s), first at sequence %d",
              flags, (flags & pkv::kBadCu) ? " cu_seqlens" : "", (flags & pkv::kBadSeqlen) ? " seqlens_k" : "",
              (flags & pkv::kBadBlockId) ? " block_id" : "", (flags & pkv::kBadRows) ? " rows>max_seqlen_q" : "",
              (flags & pkv::kBadAppend) ? " append_rows>keys" : "", (flags & pkv::kBadWritePos) ? " write_position" : "",
              first);
}

int pkv_set_option(int option, int64_t value) {
  switch (option) {
    case PKV_OPT_PATH:
      if (value < 0 || value > 2) return fail(PKV_ERR_OPTION, "PKV_OPT_PATH must be 0, 1 or 2");
      g_opt_path.store(value);
      return ok();
    case PKV_OPT_SPLIT_CHUNKS:
      if (value < 0 || value > 64) return fail(PKV_ERR_OPTION, "PKV_OPT_SPLIT_CHUNKS must be in 0..64");
      g_opt_split_chunks.store(value);
      return ok();
    case PKV_OPT_FULL_KERNEL:
      if (value < 0 || value > 3) return fail(PKV_ERR_OPTION, "PKV_OPT_FULL_KERNEL must be in 0..3");
      g_opt_full_kernel.store(value);
      return ok();
    case PKV_OPT_DEBUG:
      if (value < 0 || value > 1) return fail(PKV_ERR_OPTION, "PKV_OPT_DEBUG must be 0 or 1");
      g_opt_debug.store(value);
      return ok();
    case PKV_OPT_DECODE_ORDER:
      if (value < 0 || value > 2) return fail(PKV_ERR_OPTION, "PKV_OPT_DECODE_ORDER must be 0, 1 or 2");
      g_opt_decode_order.store(value);
      return ok();
    default:
      return fail(PKV_ERR_OPTION, "unknown option %d", option);
  }
}

int64_t pkv_get_option(int option) {
  switch (option) {
    case PKV_OPT_PATH: return g_opt_path.load();
    case PKV_OPT_SPLIT_CHUNKS: return g_opt_split_chunks.load();
    case PKV_OPT_FULL_KERNEL: return g_opt_full_kernel.load();
    case PKV_OPT_DEBUG: return g_opt_debug.load();
    case PKV_OPT_DECODE_ORDER: return g_opt_decode_order.load();
    default: return -1;
  }
}

const char* pkv_error_string(int code) {
  switch (code) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "null pointer";
    case PKV_ERR_SHAPE: return "invalid or unsupported shape";
    case PKV_ERR_DTYPE: return "unsupported dtype";
    case PKV_ERR_ALIGN: return "misaligned pointer or stride";
    case PKV_ERR_WORKSPACE: return "workspace too small or unavailable";
    case PKV_ERR_HIP: return "HIP runtime error";
    case PKV_ERR_OPTION: return "invalid option";
    case PKV_ERR_DEVICE_DATA: return "device data violates a precondition";
    default: return "unknown error";
  }
}

const char* pkv_last_error(void) { return g_msg; }

int pkv_abi_version(void) { return PKV_ABI_VERSION; }

}  // extern "C"
