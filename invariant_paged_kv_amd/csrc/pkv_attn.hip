// pkv_attn.hip -- attention kernels of libpkv for gfx950.
//
//   attn_kernel<SPLIT=true>   decode path: one work item per (sequence, KV head,
//                             column block, run of chunks); writes one fp32
//                             partial (max, sum, o[d]) per chunk and column.
//   merge_kernel              decode path: folds a row's chunk partials in
//                             ascending chunk index, then the final write.
//   attn_kernel<SPLIT=false>  prefill path: one work item per (sequence, KV head,
//                             column block); runs the chunks in ascending order
//                             and folds them in registers, then the final write.
//
// A "column" is one (query row, query head) pair of a sequence; the g = Hq/Hkv
// query heads of a KV head share every K/V tile a work item stages in LDS, so
// one read of K/V serves the whole GQA group (aiter commit d293d61bbf19 "pin
// non-contiguous paged KV block stride": query head h reads KV head h // g).
// Both paths call the same chunk core (pkv_device.hpp) on the same tiles in the
// same order, so a row's bits do not depend on the path, the batch, padding,
// the split count or the grid.
#include "pkv_device.hpp"
#include "pkv_internal.h"

namespace pkv {

// K/V tile loader: keys j0 .. j0+KT-1 of one sequence and KV head into LDS,
// 16-byte loads, consecutive lanes on consecutive 16 bytes of a key row.  The
// block address uses the real block stride (contiguous or K/V-interleaved
// caches alike).  Keys >= jmax are not read; their rows are zero.
template <class T, int D, int W>
__device__ __forceinline__ void load_tile(const AttnArgs& a, const int32_t* bt, int hk, int j0, int jmax,
                                          unsigned char* k_lds, unsigned char* v_lds) {
  using G_ = TileGeom<T, D>;
  constexpr int NCH = KT * G_::CPR;
  constexpr int PER = NCH / (64 * W);
  static_assert(PER * 64 * W == NCH, "tile chunks must split evenly over the work group");
  constexpr int R = PER < 16 ? PER : 16;
  const unsigned char* kb = static_cast<const unsigned char*>(a.k);
  const unsigned char* vb = static_cast<const unsigned char*>(a.v);
#pragma unroll
  for (int r0 = 0; r0 < PER; r0 += R) {
    u32x4 kr[R], vr[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int qi = threadIdx.x + (r0 + i) * 64 * W;
      const int row = qi / G_::CPR, part = qi % G_::CPR;
      const int j = j0 + row;
      if (j < jmax) {
        const int64_t blk = bt[j / a.bs];
        const int64_t slot = j % a.bs;
        kr[i] = *reinterpret_cast<const u32x4*>(kb + (blk * a.kbs + slot * a.kss + hk * a.khs) * T::EB + 16 * part);
        vr[i] = *reinterpret_cast<const u32x4*>(vb + (blk * a.vbs + slot * a.vss + hk * a.vhs) * T::EB + 16 * part);
      } else {
        kr[i] = u32x4{0, 0, 0, 0};
        vr[i] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int qi = threadIdx.x + (r0 + i) * 64 * W;
      const int row = qi / G_::CPR, part = qi % G_::CPR;
      *reinterpret_cast<u32x4*>(k_lds + row * G_::PITCH + 16 * part) = kr[i];
      *reinterpret_cast<u32x4*>(v_lds + row * G_::PITCH + 16 * part) = vr[i];
    }
  }
}

// Keys visible to column `col` of a sequence: j < limit.  Columns are ordered
// row-major over (row r, head-in-group hh): col = r * g + hh.  Row r sits at
// key position n - L + r (bottom-right alignment).
__device__ __forceinline__ int column_limit(int col, int ncols, int g, int n, int L, int causal) {
  if (col >= ncols) return 0;
  const int p = n - L + col / g;
  return causal ? min(p + 1, n) : n;
}

template <class T, int D>
__device__ __forceinline__ void store_out(void* out, int64_t elem, const f32x4 (&o)[D / 16], float M, float Ls) {
  const int G = lane_id() >> 4;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const int e = 16 * dt + 4 * G;
    float v0 = final_val(M, o[dt][0], Ls), v1 = final_val(M, o[dt][1], Ls);
    float v2 = final_val(M, o[dt][2], Ls), v3 = final_val(M, o[dt][3], Ls);
    if constexpr (T::EB == 2) {
      u32x2 w = {bf16_rne_bits(v0) | (bf16_rne_bits(v1) << 16), bf16_rne_bits(v2) | (bf16_rne_bits(v3) << 16)};
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + elem + e) = w;
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(out) + elem + e) = f32x4{v0, v1, v2, v3};
    }
  }
}

template <class T, int D, int W, int NT, bool SPLIT>
__global__ __launch_bounds__(64 * W, 2) void attn_kernel(AttnArgs a) {
  using G_ = TileGeom<T, D>;
  constexpr int COLS = W * NT * 16;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * G_::BYTES];
  unsigned char* k_lds = lds;
  unsigned char* v_lds = lds + G_::BYTES;

  const int b = blockIdx.z;
  const int hk = blockIdx.y;
  int cb, item;
  if constexpr (SPLIT) {
    cb = blockIdx.x % a.ncb;
    item = blockIdx.x / a.ncb;
  } else {
    cb = a.ncb - 1 - static_cast<int>(blockIdx.x);  // heaviest causal blocks first
    item = 0;
  }
  const int n = a.seqlens_k[b];
  const int q0 = a.cu_q[b];
  const int L = a.cu_q[b + 1] - q0;
  const int g = a.g;
  const int ncols = L * g;
  const int col0 = cb * COLS;
  if (col0 >= ncols) return;
  const int last_col = min(col0 + COLS, ncols) - 1;
  const int jmax = column_limit(last_col, ncols, g, n, L, a.causal);
  const int nchunks = jmax > 0 ? (jmax + KC - 1) / KC : 0;
  int c_begin = 0, c_end = nchunks;
  if constexpr (SPLIT) {
    c_begin = item * a.cpi;
    c_end = min(min(c_begin + a.cpi, nchunks), a.maxc);
    if (c_begin >= c_end) return;
  }

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int G = lane >> 4;
  int lim[NT];
  int cols[NT];
  QOps<T, D> q[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int col = col0 + (wave * NT + nt) * 16 + (lane & 15);
    cols[nt] = col;
    lim[nt] = column_limit(col, ncols, g, n, L, a.causal);
    if (col < ncols) {
      const int64_t qelem = ((int64_t)(q0 + col / g) * a.hq + hk * g + col % g) * D;
      const unsigned char* qp = static_cast<const unsigned char*>(a.q) + qelem * T::EB + 16 * G;
#pragma unroll
      for (int k = 0; k < G_::NK; ++k) q[nt].v[k] = *reinterpret_cast<const u32x4*>(qp + 64 * k);
    } else {
#pragma unroll
      for (int k = 0; k < G_::NK; ++k) q[nt].v[k] = u32x4{0, 0, 0, 0};
    }
  }

  float M[NT], Ls[NT];
  f32x4 O[NT][D / 16];
  if constexpr (!SPLIT) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      M[nt] = -INFINITY;
      Ls[nt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) O[nt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  const int32_t* bt = a.block_table + (int64_t)b * a.mbps;
  ChunkState<D, NT> st;
  for (int c = c_begin; c < c_end; ++c) {
    chunk_reset(st);
    const int jend = min((c + 1) * KC, jmax);
    for (int j0 = c * KC; j0 < jend; j0 += KT) {
      __syncthreads();
      load_tile<T, D, W>(a, bt, hk, j0, jmax, k_lds, v_lds);
      __syncthreads();
      f32x4 s[NT][KT / 16];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) qk_tile<T, D>(k_lds, q[nt], s[nt]);
      softmax_pv_tile<T, D, NT>(st, s, lim, j0, a.mul, v_lds);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float lc = column_sum(st.l[nt]);
      if constexpr (SPLIT) {
        const int col = cols[nt];
        if (col < ncols) {
          const int64_t idx = ((int64_t)(q0 + col / g) * a.hq + hk * g + col % g) * a.maxc + c;
          if (G == 0) {
            a.part_ml[2 * idx] = st.m[nt];
            a.part_ml[2 * idx + 1] = lc;
          }
          float* po = a.part_o + idx * D;
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<f32x4*>(po + 16 * dt + 4 * G) = st.o[nt][dt];
        }
      } else {
        if (st.m[nt] != -INFINITY) {
          const FoldCoef<T> f = fold_coef<T>(M[nt], st.m[nt]);
          Ls[nt] = fold_val(Ls[nt], f.a, lc, f.b);
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) O[nt][dt][i] = fold_val(O[nt][dt][i], f.a, st.o[nt][dt][i], f.b);
          M[nt] = f.mn;
        }
      }
    }
  }

  if constexpr (!SPLIT) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int col = cols[nt];
      if (col < ncols) {
        const int64_t rh = (int64_t)(q0 + col / g) * a.hq + hk * g + col % g;
        if (G == 0) a.lse[rh] = final_lse<T>(M[nt], Ls[nt]);
        store_out<T, D>(a.out, rh * D, O[nt], M[nt], Ls[nt]);
      }
    }
  }
}

// Fold of one row's chunk partials, ascending chunk index, then the final
// write.  One wave per (row, query head); lane holds head-dim elements
// 2*lane, 2*lane+1 (d = 128) or lane (d = 64).
template <class T, int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int EPL = D / 64;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= a.total_q * a.hq) return;
  const int64_t row = w / a.hq;
  const int head = static_cast<int>(w % a.hq);
  int lo = 0, hi = a.batch;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.cu_q[mid] <= row) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  if (b >= a.batch) return;
  const int n = a.seqlens_k[b];
  const int L = a.cu_q[b + 1] - a.cu_q[b];
  const int p = n - L + static_cast<int>(row - a.cu_q[b]);
  const int lim = a.causal ? min(p + 1, n) : n;
  const int nck = lim > 0 ? min((lim + KC - 1) / KC, a.maxc) : 0;
  const int lane = lane_id();
  float M = -INFINITY, Ls = 0.f;
  float O[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) O[e] = 0.f;
  const int64_t base = w * a.maxc;
  for (int c = 0; c < nck; ++c) {
    const float mc = a.part_ml[2 * (base + c)];
    const float lc = a.part_ml[2 * (base + c) + 1];
    const float* po = a.part_o + (base + c) * D + EPL * lane;
    float oc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) oc[e] = po[e];
    if (mc == -INFINITY) continue;
    const FoldCoef<T> f = fold_coef<T>(M, mc);
    Ls = fold_val(Ls, f.a, lc, f.b);
#pragma unroll
    for (int e = 0; e < EPL; ++e) O[e] = fold_val(O[e], f.a, oc[e], f.b);
    M = f.mn;
  }
  if (lane == 0) a.lse[w] = final_lse<T>(M, Ls);
  if constexpr (T::EB == 2) {
    uint16_t* o = static_cast<uint16_t*>(a.out) + w * D + EPL * lane;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = static_cast<uint16_t>(bf16_rne_bits(final_val(M, O[e], Ls)));
  } else {
    float* o = static_cast<float*>(a.out) + w * D + EPL * lane;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = final_val(M, O[e], Ls);
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers (called by pkv_api.hip after validation).
// ---------------------------------------------------------------------------
template <class T, int D>
static hipError_t launch_attn_t(const AttnArgs& a, const LaunchPlan& pl, hipStream_t stream) {
  if (pl.full) {
    dim3 grid(a.ncb, pl.hk, pl.batch);
    hipLaunchKernelGGL((attn_kernel<T, D, 4, 2, false>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  dim3 grid(a.ncb * pl.items, pl.hk, pl.batch);
  if (pl.waves == 1) {
    hipLaunchKernelGGL((attn_kernel<T, D, 1, 1, true>), grid, dim3(64), 0, stream, a);
  } else {
    hipLaunchKernelGGL((attn_kernel<T, D, 4, 1, true>), grid, dim3(256), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MergeArgs m;
  m.cu_q = a.cu_q;
  m.seqlens_k = a.seqlens_k;
  m.part_o = a.part_o;
  m.part_ml = a.part_ml;
  m.out = a.out;
  m.lse = a.lse;
  m.total_q = pl.total_q;
  m.batch = pl.batch;
  m.hq = a.hq;
  m.maxc = a.maxc;
  m.causal = a.causal;
  const int64_t waves = pl.total_q * a.hq;
  if (waves == 0) return hipSuccess;
  dim3 mgrid(static_cast<unsigned>((waves + 3) / 4));
  hipLaunchKernelGGL((merge_kernel<T, D>), mgrid, dim3(256), 0, stream, m);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, const LaunchPlan& pl, int dtype, int d, hipStream_t stream) {
  (void)hipGetLastError();
  if (dtype == 1) {
    return d == 128 ? launch_attn_t<TBf16, 128>(a, pl, stream) : launch_attn_t<TBf16, 64>(a, pl, stream);
  }
  return d == 128 ? launch_attn_t<TF32, 128>(a, pl, stream) : launch_attn_t<TF32, 64>(a, pl, stream);
}

}  // namespace pkv
