// pkv_attn_bwd.hip -- backward of the paged-KV attention for gfx950.
//
// RL-Kernel PR #284, "feat(attention): add CP backward drift validation",
// sections "Summary" and "Changes": a deterministic training backward (dq, dk,
// dv) over the same forward, with fp32 accumulation, a fixed summation order
// and one downcast at the final write.  With P the softmax weights recomputed
// from the forward's LSE, dO the cotangent of out and delta = <dO, out> per
// (row, head):
//
//   dP = dO V^T,  dS = P (dP - delta),  dQ = scale dS K,
//   dK = scale dS^T Q (summed over the heads of a GQA group),  dV = P^T dO.
//
// Three kernels, no atomics, every sum in an order fixed by global positions:
//   bwd_delta_kernel  delta per (row, head): 16 lanes, a fixed butterfly.
//   bwd_dq_kernel     one work group per (sequence, KV head, 16 W columns);
//                     K/V tiles staged in LDS in ascending key order from
//                     key 0, so a column's dq is the same sum whichever call,
//                     batch or grid computes it.
//   bwd_dkdv_kernel   one work group per (sequence, KV head, 16 W keys); each
//                     wave holds its 16 keys' K and V as MFMA operands in
//                     registers and walks the sequence's columns in
//                     ascending 32-column steps from column 0 (the first
//                     steps that cannot see its keys are skipped).
//
// A "column" is one (query row, query head of the group) pair, col = r g + hh,
// as in the forward.  bf16 products use v_mfma_f32_16x16x32_bf16 with P and dS
// rounded once to bf16 (round to nearest even) as MFMA operands; fp32 uses
// v_mfma_f32_16x16x4_f32.
#include "pkv_device.hpp"
#include "pkv_internal.h"
#include "pkv_tiles.hpp"

namespace pkv {

// Natural-log LSE in the score units of T (bf16 scores are in base 2).
template <class T> __device__ __forceinline__ float lse_units(float lse) {
  if constexpr (T::kBase2) return lse * 1.44269504088896340736f;
  else return lse;
}

__device__ __forceinline__ float elem_f32(const void* p, int64_t i, int eb) {
  if (eb == 2) return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
  return static_cast<const float*>(p)[i];
}

#ifndef PKV_BWD_XCD
#define PKV_BWD_XCD 1
#endif
#ifndef PKV_DQ_NT
#define PKV_DQ_NT 2
#endif
#ifndef PKV_DKDV_KW
#define PKV_DKDV_KW 1
#endif
// Raised wave priority over the MFMA blocks that follow the exponentials, so
// the other wave's VALU work fills the MFMA latency (measured 2-4% faster).
#ifndef PKV_BWD_PRIO
#define PKV_BWD_PRIO 1
#endif

// Work groups are dispatched round-robin over the 8 XCDs (each with its own
// L2); renumber them so that one XCD runs consecutive blocks of the same
// (sequence, KV head), whose shared tiles its L2 then serves.  Returns the
// (x, y, z) the work group takes on.
__device__ __forceinline__ void xcd_order(int& x, int& y, int& z) {
#if PKV_BWD_XCD
  const int nwg = gridDim.x * gridDim.y * gridDim.z;
  const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int full8 = nwg / 8 * 8;
  const int w = lin < full8 ? (lin % 8) * (nwg / 8) + lin / 8 : lin;
  x = w % gridDim.x;
  y = (w / gridDim.x) % gridDim.y;
  z = w / (gridDim.x * gridDim.y);
#else
  x = blockIdx.x;
  y = blockIdx.y;
  z = blockIdx.z;
#endif
}

// ---------------------------------------------------------------------------
// delta[w] = <dout[w], out[w]> for each (row, head) w, in fp32: 16 lanes per w,
// each lane sums D/16 consecutive elements in ascending order, then a fixed
// xor butterfly over the 16 lanes.
// ---------------------------------------------------------------------------
template <class T, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a, int64_t pairs) {
  if (dbg_skip(a.f.dbg_word)) return;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  constexpr int EPL = D / 16;
  float acc = 0.f;
  if (w < pairs) {
    const int64_t e0 = w * D + sub * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc = fmaf(elem_f32(a.dout, e0 + e, T::EB), elem_f32(a.out, e0 + e, T::EB), acc);
  }
  acc = acc + __shfl_xor(acc, 8);
  acc = acc + __shfl_xor(acc, 4);
  acc = acc + __shfl_xor(acc, 2);
  acc = acc + __shfl_xor(acc, 1);
  if (w < pairs && sub == 0) a.delta[w] = acc;
}

// A-operand rows of an LDS tile (row pitch `pitch`): rows 16 mt + l%16,
// bytes [64k + 16G, +16) -- the layout of KOps, for any row-major tile.
template <class T, int D>
__device__ __forceinline__ void row_operands_lds(const unsigned char* lds, int pitch, KOps<T, D>& op) {
  using G_ = TileGeom<T, D>;
  const int lane = lane_id();
  const unsigned char* base = lds + (lane & 15) * pitch + 16 * (lane >> 4);
#pragma unroll
  for (int mt = 0; mt < G_::MT; ++mt)
#pragma unroll
    for (int k = 0; k < G_::NK; ++k) op[mt][k] = *reinterpret_cast<const u32x4*>(base + mt * 16 * pitch + 64 * k);
}

// One 16x16 product over the head dimension: sum over d of A[m][d] B[n][d],
// both operands in the QK layout (16 bytes per lane per step), ascending
// steps from a zero accumulator.
template <class T, int NK>
__device__ __forceinline__ f32x4 dot_tile(const u32x4 (&x)[NK], const u32x4 (&y)[NK]) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    if constexpr (T::EB == 2) {
      acc = mfma_bf16(x[k], y[k], acc);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = mfma_f32(__uint_as_float(x[k][e]), __uint_as_float(y[k][e]), acc);
    }
  }
  return acc;
}

// Two fp32 quadruples rounded to bf16 and packed as one 16x16x32 operand:
// slots 8G + e hold a[e] (e < 4) and b[e - 4] (e >= 4).
__device__ __forceinline__ u32x4 pack_bf16(const f32x4& a, const f32x4& b) {
  const bf16x2 p0 = {(__bf16)a[0], (__bf16)a[1]};
  const bf16x2 p1 = {(__bf16)a[2], (__bf16)a[3]};
  const bf16x2 p2 = {(__bf16)b[0], (__bf16)b[1]};
  const bf16x2 p3 = {(__bf16)b[2], (__bf16)b[3]};
  return u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1), __builtin_bit_cast(uint32_t, p2),
               __builtin_bit_cast(uint32_t, p3)};
}

// Final write of a transposed accumulator (lane l: output row l%16, head-dim
// elements 16 dt + 4G + i), times `mul`, rounded once to the output type.
template <class T, int D>
__device__ __forceinline__ void store_grad(void* dst, int64_t elem, const f32x4 (&acc)[D / 16], float mul) {
  const int G = lane_id() >> 4;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const int e = 16 * dt + 4 * G;
    const float v0 = acc[dt][0] * mul, v1 = acc[dt][1] * mul, v2 = acc[dt][2] * mul, v3 = acc[dt][3] * mul;
    if constexpr (T::EB == 2) {
      u32x2 w = {bf16_rne_bits(v0) | (bf16_rne_bits(v1) << 16), bf16_rne_bits(v2) | (bf16_rne_bits(v3) << 16)};
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(dst) + elem + e) = w;
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(dst) + elem + e) = f32x4{v0, v1, v2, v3};
    }
  }
}

// The QK-layout operands (16 bytes per lane per step) of one row of a
// [rows, Hq, d] tensor: `row_head` = row * Hq + head.
template <class T, int D>
__device__ __forceinline__ void row_operands_global(const void* base, int64_t row_head, bool exists, QOps<T, D>& op) {
  using G_ = TileGeom<T, D>;
  const unsigned char* p = static_cast<const unsigned char*>(base) + row_head * D * T::EB + 16 * (lane_id() >> 4);
#pragma unroll
  for (int k = 0; k < G_::NK; ++k) op.v[k] = exists ? *reinterpret_cast<const u32x4*>(p + 64 * k) : u32x4{0, 0, 0, 0};
}

// ---------------------------------------------------------------------------
// dq: per column, over key tiles 0, 64, 128, ... up to its last visible key:
//   S^T = K Q^T, dP^T = V dO^T (keys as M, columns as N, as the forward's QK),
//   P = exp(S * mul - lse), dS = P (dP - delta) (0 for invisible keys),
//   dQ^T += K^T dS^T (head dim as M, keys as the k-dimension, as the forward's PV).
// ---------------------------------------------------------------------------
template <class T, int D, int W, int NT, bool U>
__global__ __launch_bounds__(64 * W, 2) void bwd_dq_kernel(BwdArgs ba) {
  if (dbg_skip(ba.f.dbg_word)) return;
  const AttnArgs& a = ba.f;
  using G_ = TileGeom<T, D>;
  constexpr int COLS = 16 * W * NT;
  __shared__ __attribute__((aligned(16))) unsigned char lds[G_::BYTES];
  unsigned char* k_lds = lds;
  unsigned char* v_lds = lds + G_::KBYTES;

  int bx, hk, b;
  xcd_order(bx, hk, b);
  const int cb = a.ncb - 1 - bx;  // heaviest causal blocks first
  const int n = a.seqlens_k[b];
  const int q0 = a.cu_q[b];
  const int L = a.cu_q[b + 1] - q0;
  const int g = a.g;
  const int ncols = L * g;
  const int col0 = cb * COLS;
  if (col0 >= ncols) return;
  const int last_col = min(col0 + COLS, ncols) - 1;
  const int jmax = column_limit(last_col, ncols, g, n, L, a.causal);

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int G = lane >> 4;
  // NT groups of 16 columns per wave: every K/V operand read from LDS serves them all.
  int lim[NT];
  bool exists[NT];
  int64_t rh[NT];
  float lse_u[NT], dlt[NT];
  QOps<T, D> q[NT], dout[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int col = col0 + (wave * NT + nt) * 16 + (lane & 15);
    exists[nt] = col < ncols;
    lim[nt] = exists[nt] ? column_limit(col, ncols, g, n, L, a.causal) : 0;
    rh[nt] = static_cast<int64_t>(q0 + col / g) * a.hq + hk * g + col % g;
    row_operands_global<T, D>(a.q, rh[nt], exists[nt], q[nt]);
    row_operands_global<T, D>(ba.dout, rh[nt], exists[nt], dout[nt]);
    lse_u[nt] = (exists[nt] && lim[nt] > 0) ? lse_units<T>(ba.lse[rh[nt]]) : 0.f;
    dlt[nt] = exists[nt] ? ba.delta[rh[nt]] : 0.f;
  }

  f32x4 acc[NT][D / 16];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc[nt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.mbps;
  const Append none;
  for (int j0 = 0; j0 < jmax; j0 += KT) {
    __syncthreads();
    load_tile<T, D, W, false, U>(a, bt, hk, j0, jmax, k_lds, v_lds, none);
    __syncthreads();
    f32x4 s[NT][G_::MT], dp[NT][G_::MT];
#pragma unroll
    for (int mt = 0; mt < G_::MT; ++mt) {
      u32x4 kx[G_::NK], vx[G_::NK];
      const unsigned char* kr = k_lds + (16 * mt + (lane & 15)) * G_::KPITCH + 16 * G;
      const unsigned char* vr = v_lds + (16 * mt + (lane & 15)) * G_::VPITCH + 16 * G;
#pragma unroll
      for (int k = 0; k < G_::NK; ++k) {
        kx[k] = *reinterpret_cast<const u32x4*>(kr + 64 * k);
        vx[k] = *reinterpret_cast<const u32x4*>(vr + 64 * k);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        s[nt][mt] = dot_tile<T, G_::NK>(kx, q[nt].v);
        dp[nt][mt] = dot_tile<T, G_::NK>(vx, dout[nt].v);
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (__all(j0 + KT <= lim[nt])) {  // the whole tile is visible to every lane: no mask
#pragma unroll
        for (int mt = 0; mt < G_::MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            s[nt][mt][i] = pkv_exp<T>(fmaf(s[nt][mt][i], a.mul, -lse_u[nt])) * (dp[nt][mt][i] - dlt[nt]);
      } else {
#pragma unroll
        for (int mt = 0; mt < G_::MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = j0 + 16 * mt + 4 * G + i;
            const bool vis = key < lim[nt];
            const float p = vis ? pkv_exp<T>(fmaf(s[nt][mt][i], a.mul, -lse_u[nt])) : 0.f;
            s[nt][mt][i] = vis ? p * (dp[nt][mt][i] - dlt[nt]) : 0.f;  // dS^T
          }
      }
    }
    if constexpr (T::EB == 2) {
#if PKV_BWD_PRIO
      __builtin_amdgcn_s_setprio(1);
#endif
#pragma unroll
      for (int dt = 0; dt < G_::DT; ++dt) {
#pragma unroll
        for (int ks = 0; ks < KT / 32; ++ks) {
          const u32x4 kt = v_operand_bf16(k_lds, G_::KPITCH, ks, dt);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[nt][dt] = mfma_bf16(kt, pack_bf16(s[nt][2 * ks], s[nt][2 * ks + 1]), acc[nt][dt]);
        }
      }
#if PKV_BWD_PRIO
      __builtin_amdgcn_s_setprio(0);
#endif
    } else {
      const unsigned char* colp = k_lds + 4 * (lane & 15);
#pragma unroll
      for (int dt = 0; dt < G_::DT; ++dt)
#pragma unroll
        for (int mt = 0; mt < G_::MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float kt = *reinterpret_cast<const float*>(colp + (16 * mt + 4 * G + i) * G_::KPITCH + 4 * 16 * dt);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[nt][dt] = mfma_f32(kt, s[nt][mt][i], acc[nt][dt]);
          }
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    if (exists[nt]) store_grad<T, D>(ba.dq, rh[nt] * D, acc[nt], ba.scale);
}

// ---------------------------------------------------------------------------
// dk, dv: per key, over 32-column steps in ascending order:
//   S = Q K^T, dP = dO V^T (columns as M, keys as N),
//   P = exp(S * mul - lse), dS = P (dP - delta) (0 where the key is invisible),
//   dV^T += dO^T P, dK^T += Q^T dS (head dim as M, columns as the k-dimension:
//   k-slot 8G + e <-> column 4G + e (e < 4) or 16 + 4G + (e - 4)).
// ---------------------------------------------------------------------------
constexpr int kBwdCols = 32;  // columns per step of the dk/dv kernel

template <class T, int D>
struct ColTile {
  static constexpr int ROW_BYTES = D * T::EB;
  static constexpr int PITCH = ROW_BYTES + 32;  // the transposing read's bank-friendly pitch
  static constexpr int BYTES = kBwdCols * PITCH;
  static constexpr int CPR = ROW_BYTES / 16;
  static constexpr int NK = ROW_BYTES / 64;
};

// Register stage of one 32-column step: this thread's 16-byte pieces of the
// Q and dO rows, and (threads < 32) one column's LSE (score units) and delta.
template <class T, int D, int W>
struct ColStage {
  static constexpr int PER = kBwdCols * ColTile<T, D>::CPR / (64 * W);
  u32x4 q[PER];
  u32x4 d[PER];
  float lu, dl;
};

template <class T, int D, int W>
__device__ __forceinline__ void col_stage_load(const BwdArgs& ba, int q0, int hk, int ncols, int n, int L, int c0,
                                               ColStage<T, D, W>& st) {
  const AttnArgs& a = ba.f;
  using C_ = ColTile<T, D>;
  using S_ = ColStage<T, D, W>;
  static_assert(S_::PER * 64 * W == kBwdCols * C_::CPR, "column tile pieces must split evenly over the work group");
  const int g = a.g;
#pragma unroll
  for (int i = 0; i < S_::PER; ++i) {
    const int qi = threadIdx.x + i * 64 * W;
    const int row = qi / C_::CPR, part = qi % C_::CPR;
    const int c = min(c0 + row, ncols - 1);  // columns past the end load a real row, then read as zero
    const int64_t off = (static_cast<int64_t>(q0 + c / g) * a.hq + hk * g + c % g) * D * T::EB + 16 * part;
    const bool in = c0 + row < ncols;
    const u32x4 xq = *reinterpret_cast<const u32x4*>(static_cast<const unsigned char*>(a.q) + off);
    const u32x4 xd = *reinterpret_cast<const u32x4*>(static_cast<const unsigned char*>(ba.dout) + off);
    st.q[i] = in ? xq : u32x4{0, 0, 0, 0};
    st.d[i] = in ? xd : u32x4{0, 0, 0, 0};
  }
  if (threadIdx.x < kBwdCols) {
    const int c = c0 + threadIdx.x;
    st.lu = 0.f;
    st.dl = 0.f;
    if (c < ncols) {
      const int64_t rh = static_cast<int64_t>(q0 + c / g) * a.hq + hk * g + c % g;
      if (column_limit(c, ncols, g, n, L, a.causal) > 0) st.lu = lse_units<T>(ba.lse[rh]);
      st.dl = ba.delta[rh];
    }
  }
}

template <class T, int D, int W>
__device__ __forceinline__ void col_stage_store(unsigned char* buf, const ColStage<T, D, W>& st) {
  using C_ = ColTile<T, D>;
  using S_ = ColStage<T, D, W>;
#pragma unroll
  for (int i = 0; i < S_::PER; ++i) {
    const int qi = threadIdx.x + i * 64 * W;
    const int row = qi / C_::CPR, part = qi % C_::CPR;
    *reinterpret_cast<u32x4*>(buf + row * C_::PITCH + 16 * part) = st.q[i];
    *reinterpret_cast<u32x4*>(buf + C_::BYTES + row * C_::PITCH + 16 * part) = st.d[i];
  }
  if (threadIdx.x < kBwdCols) {
    float* f = reinterpret_cast<float*>(buf + 2 * C_::BYTES);
    f[threadIdx.x] = st.lu;
    f[kBwdCols + threadIdx.x] = st.dl;
  }
}

// Each 32-column step is computed from one LDS buffer while the next step's
// rows are in flight in registers; they go to the other buffer afterwards, and
// one barrier per step separates the two.  Each wave owns KW tiles of 16 keys:
// every Q / dO operand read from LDS serves all of them.
template <class T, int D, int W, int KW>
__global__ __launch_bounds__(64 * W, (T::EB == 2 && KW == 1) ? 3 : 2) void bwd_dkdv_kernel(BwdArgs ba) {
  if (dbg_skip(ba.f.dbg_word)) return;
  const AttnArgs& a = ba.f;
  using C_ = ColTile<T, D>;
  constexpr int NK = C_::NK;
  constexpr int DT = D / 16;
  constexpr int BUF = 2 * C_::BYTES + 2 * kBwdCols * sizeof(float);
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * BUF];

  int bx, hk, b;
  xcd_order(bx, hk, b);
  const int key0 = bx * 16 * W * KW;
  const int n = a.seqlens_k[b];
  if (key0 >= n) return;
  const int q0 = a.cu_q[b];
  const int L = a.cu_q[b + 1] - q0;
  const int g = a.g;
  const int ncols = L * g;

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int G = lane >> 4;

  // Columns before c_start cannot see key0 (causal); the step grid stays at multiples of 32 from column 0.
  int c_start = 0;
  if (a.causal) {
    const int r_min = max(key0 - (n - L), 0);
    c_start = (min(r_min, L) * g) & ~(kBwdCols - 1);
  }
  ColStage<T, D, W> stage;
  if (c_start < ncols) col_stage_load<T, D, W>(ba, q0, hk, ncols, n, L, c_start, stage);

  // This lane's keys (one per 16-key tile) as the N operand of S and dP: bytes
  // [64k + 16G, +16) of their K and V rows.  A key is visible to column c (row
  // c / g at position n - L + c / g) iff c >= c_vis: key <= n - L + floor(c / g)
  // <=> c >= (key - n + L) * g.
  int keyv[KW], c_vis[KW];
  bool kin[KW];
  u32x4 kb[KW][NK], vb[KW][NK];
  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.mbps;
#pragma unroll
  for (int kt = 0; kt < KW; ++kt) {
    const int key = key0 + (wave * KW + kt) * 16 + (lane & 15);
    keyv[kt] = key;
    kin[kt] = key < n;
    c_vis[kt] = !kin[kt] ? INT_MAX : (a.causal ? max(key - (n - L), 0) * g : 0);
    const int kc = min(key, n - 1);
    const int bi = div_block(kc, a.bs_mul, a.bs_shift);
    const int64_t blk = bt[bi];
    const int64_t slot = kc - bi * a.bs;
    const unsigned char* kp = static_cast<const unsigned char*>(a.k) + (blk * a.kbs + slot * a.kss + static_cast<int64_t>(hk) * a.khs) * T::EB + 16 * G;
    const unsigned char* vp = static_cast<const unsigned char*>(a.v) + (blk * a.vbs + slot * a.vss + static_cast<int64_t>(hk) * a.vhs) * T::EB + 16 * G;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      kb[kt][k] = kin[kt] ? *reinterpret_cast<const u32x4*>(kp + 64 * k) : u32x4{0, 0, 0, 0};
      vb[kt][k] = kin[kt] ? *reinterpret_cast<const u32x4*>(vp + 64 * k) : u32x4{0, 0, 0, 0};
    }
  }

  f32x4 dk[KW][DT], dv[KW][DT];
#pragma unroll
  for (int kt = 0; kt < KW; ++kt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      dk[kt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      dv[kt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  if (c_start < ncols) col_stage_store<T, D, W>(lds, stage);
  __syncthreads();
  int cur = 0;
  for (int c0 = c_start; c0 < ncols; c0 += kBwdCols) {
    const bool more = c0 + kBwdCols < ncols;
    if (more) col_stage_load<T, D, W>(ba, q0, hk, ncols, n, L, c0 + kBwdCols, stage);
    const unsigned char* q_lds = lds + cur * BUF;
    const unsigned char* do_lds = q_lds + C_::BYTES;
    const float* lse_lds = reinterpret_cast<const float*>(q_lds + 2 * C_::BYTES);
    const float* dl_lds = lse_lds + kBwdCols;

    f32x4 s[2][KW], dp[2][KW];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      u32x4 x[NK];
      const unsigned char* rq = q_lds + (16 * ct + (lane & 15)) * C_::PITCH + 16 * G;
#pragma unroll
      for (int k = 0; k < NK; ++k) x[k] = *reinterpret_cast<const u32x4*>(rq + 64 * k);
#pragma unroll
      for (int kt = 0; kt < KW; ++kt) s[ct][kt] = dot_tile<T, NK>(x, kb[kt]);
      const unsigned char* rd = do_lds + (16 * ct + (lane & 15)) * C_::PITCH + 16 * G;
#pragma unroll
      for (int k = 0; k < NK; ++k) x[k] = *reinterpret_cast<const u32x4*>(rd + 64 * k);
#pragma unroll
      for (int kt = 0; kt < KW; ++kt) dp[ct][kt] = dot_tile<T, NK>(x, vb[kt]);
    }
    // s[ct][kt][i], dp[ct][kt][i] at lane l: key tile kt's key l%16, column c0 + 16 ct + 4G + i.
    // When every lane sees the whole step the per-element mask is skipped (it would select nothing).
#pragma unroll
    for (int kt = 0; kt < KW; ++kt) {
      if (__all(c0 >= c_vis[kt]) && c0 + kBwdCols <= ncols) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int lc = 16 * ct + 4 * G + i;
            const float p = pkv_exp<T>(fmaf(s[ct][kt][i], a.mul, -lse_lds[lc]));
            dp[ct][kt][i] = p * (dp[ct][kt][i] - dl_lds[lc]);  // dS
            s[ct][kt][i] = p;                                  // P
          }
      } else {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int lc = 16 * ct + 4 * G + i;
            const int c = c0 + lc;
            const bool vis = c >= c_vis[kt] && c < ncols;
            const float p = vis ? pkv_exp<T>(fmaf(s[ct][kt][i], a.mul, -lse_lds[lc])) : 0.f;
            dp[ct][kt][i] = vis ? p * (dp[ct][kt][i] - dl_lds[lc]) : 0.f;  // dS
            s[ct][kt][i] = p;                                             // P
          }
      }
    }
    if constexpr (T::EB == 2) {
      u32x4 pp[KW], pd[KW];
#pragma unroll
      for (int kt = 0; kt < KW; ++kt) {
        pp[kt] = pack_bf16(s[0][kt], s[1][kt]);
        pd[kt] = pack_bf16(dp[0][kt], dp[1][kt]);
      }
#if PKV_BWD_PRIO
      __builtin_amdgcn_s_setprio(1);
#endif
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const u32x4 xo = v_operand_bf16(do_lds, C_::PITCH, 0, dt);
#pragma unroll
        for (int kt = 0; kt < KW; ++kt) dv[kt][dt] = mfma_bf16(xo, pp[kt], dv[kt][dt]);
        const u32x4 xq = v_operand_bf16(q_lds, C_::PITCH, 0, dt);
#pragma unroll
        for (int kt = 0; kt < KW; ++kt) dk[kt][dt] = mfma_bf16(xq, pd[kt], dk[kt][dt]);
      }
#if PKV_BWD_PRIO
      __builtin_amdgcn_s_setprio(0);
#endif
    } else {
      // fp32 step (ct, i): k-slot G <-> column 16 ct + 4G + i.
      const int dcol = 4 * (lane & 15);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * ct + 4 * G + i;
            const float xo = *reinterpret_cast<const float*>(do_lds + row * C_::PITCH + 4 * 16 * dt + dcol);
            const float xq = *reinterpret_cast<const float*>(q_lds + row * C_::PITCH + 4 * 16 * dt + dcol);
#pragma unroll
            for (int kt = 0; kt < KW; ++kt) {
              dv[kt][dt] = mfma_f32(xo, s[ct][kt][i], dv[kt][dt]);
              dk[kt][dt] = mfma_f32(xq, dp[ct][kt][i], dk[kt][dt]);
            }
          }
    }
    if (more) col_stage_store<T, D, W>(lds + (cur ^ 1) * BUF, stage);
    __syncthreads();
    cur ^= 1;
  }

#pragma unroll
  for (int kt = 0; kt < KW; ++kt) {
    if (kin[kt]) {
      const int64_t kr = (static_cast<int64_t>(ba.cu_k[b]) + keyv[kt]) * (a.hq / g) + hk;
      store_grad<T, D>(ba.dk, kr * D, dk[kt], ba.scale);
      store_grad<T, D>(ba.dv, kr * D, dv[kt], 1.0f);
    }
  }
}

// ---------------------------------------------------------------------------
template <class T, int D>
static hipError_t launch_bwd_t(const BwdArgs& a_in, const BwdPlan& pl, hipStream_t stream) {
  constexpr int W = 4;
  constexpr int NT = PKV_DQ_NT;  // column groups per wave of the dq kernel
  BwdArgs a = a_in;
  a.f.ncb = static_cast<int>((pl.cols + 16 * W * NT - 1) / (16 * W * NT));
  const int64_t pairs = pl.total_q * a.f.hq;
  if (pairs > 0) {
    hipLaunchKernelGGL((bwd_delta_kernel<T, D>), dim3(static_cast<unsigned>((pairs + 15) / 16)), dim3(256), 0, stream,
                       a, pairs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.f.ncb > 0) {
      // scalar block ids per 16 rows when the block size allows (as the forward's tile loader)
      const AttnArgs& f = a.f;
      const int64_t span = (static_cast<int64_t>(f.bs) - 1) * std::max(f.kss, f.vss) * T::KVB + D * T::KVB;
      const bool uni = f.bs % 16 == 0 && f.kss >= 0 && f.vss >= 0 && span < (int64_t{1} << 31) && f.kbs >= 0 &&
                       f.vbs >= 0 && std::max(f.kbs, f.vbs) * T::KVB < (int64_t{1} << 32);
      const dim3 grid(a.f.ncb, pl.hk, pl.batch);
      if (uni)
        hipLaunchKernelGGL((bwd_dq_kernel<T, D, W, NT, true>), grid, dim3(64 * W), 0, stream, a);
      else
        hipLaunchKernelGGL((bwd_dq_kernel<T, D, W, NT, false>), grid, dim3(64 * W), 0, stream, a);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  constexpr int KW = (T::EB == 2) ? PKV_DKDV_KW : 1;  // key tiles per wave of the dk/dv kernel
  if (a.nkb > 0) {
    a.nkb = static_cast<int>((pl.max_k + 16 * W * KW - 1) / (16 * W * KW));
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, W, KW>), dim3(a.nkb, pl.hk, pl.batch), dim3(64 * W), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_backward(const BwdArgs& a, const BwdPlan& pl, int dtype, int d, hipStream_t stream) {
  (void)hipGetLastError();
  if (dtype == 1) return d == 128 ? launch_bwd_t<TBf16, 128>(a, pl, stream) : launch_bwd_t<TBf16, 64>(a, pl, stream);
  return d == 128 ? launch_bwd_t<TF32, 128>(a, pl, stream) : launch_bwd_t<TF32, 64>(a, pl, stream);
}

}  // namespace pkv
