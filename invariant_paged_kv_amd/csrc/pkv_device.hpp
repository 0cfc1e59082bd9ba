// pkv_device.hpp -- device code shared by every attention kernel of libpkv (gfx950).
//
// Everything that decides a result bit lives here, in one copy, and every
// kernel (split/decode, merge, full/prefill) calls it: the QK^T and PV MFMA
// chains with their fixed k-slot assignment, the tile softmax with its fixed
// summation order, the chunk fold and the final division/rounding.  Kernels
// differ only in how data reaches these functions (which loads, which lanes,
// which grid), never in the arithmetic.
//
// The reduction order is the one RL-Kernel PR #284 ("feat(attention): add CP
// backward drift validation", section Changes) records for its deterministic
// reference: a fixed KV chunk size, partials merged in ascending global block
// index, fp32 accumulation, and a single downcast at the final write.  Keys
// are cut into chunks at global positions, so the same key always lands in the
// same chunk, tile and MFMA k-slot, whichever call, batch or grid computes it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int KT = 64;   // keys per tile (online-softmax step inside a chunk)
constexpr int KC = 1024;  // keys per chunk (unit of split partials and of the fold)
static_assert(KC % KT == 0, "a chunk is a whole number of tiles");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define PKV_LDS __attribute__((address_space(3)))
#ifndef PKV_V_AHEAD
#define PKV_V_AHEAD 1
#endif
#ifndef PKV_MFMA_PRIO
#define PKV_MFMA_PRIO 1
#endif

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ---------------------------------------------------------------------------
// Element types.  TBf16: bf16 storage, MFMA 16x16x32 bf16 -> fp32, base-2
// softmax (scores pre-multiplied by scale*log2(e), exp2 via v_exp_f32).
// TF32: fp32 storage, MFMA 16x16x4 fp32, natural-base expf/logf (the fp32
// tolerances leave no room for the base-2 rewrite's extra rounding).
// TFp8: bf16 queries and outputs, K/V cache stored as OCP FP8 E4M3 bytes;
// the loaders widen each byte exactly to bf16, so everything after the load is
// the TBf16 computation (the per-tensor K/V scales are applied to the score
// multiplier and to the final output).
// EB: bytes per query/output element; KVB: bytes per stored K/V element.
// ---------------------------------------------------------------------------
struct TBf16 {
  static constexpr int EB = 2;
  static constexpr int KVB = 2;
  static constexpr bool kBase2 = true;
};
struct TF32 {
  static constexpr int EB = 4;
  static constexpr int KVB = 4;
  static constexpr bool kBase2 = false;
};
struct TFp8 {
  static constexpr int EB = 2;
  static constexpr int KVB = 1;
  static constexpr bool kBase2 = true;
};

template <class T> __device__ __forceinline__ float pkv_exp(float x) {
  if constexpr (T::kBase2) return __builtin_amdgcn_exp2f(x);
  else return expf(x);
}

// How far a column's tile max may exceed its reference max before the
// reference moves (and o, l are rescaled): 8 score units, so p <= 2^8 (bf16,
// base 2) or e^8 (fp32) -- far from fp32 overflow, and most tiles keep alpha = 1.
template <class T> constexpr float kRescaleSlack = 8.0f;

// Natural-log LSE from the running max m and sum l (m in the score units of T).
template <class T> __device__ __forceinline__ float pkv_lse(float m, float l) {
  if constexpr (T::kBase2) return (m + __builtin_amdgcn_logf(l)) * 0.69314718055994530942f;  // v_log_f32 is log2
  else return m + logf(l);
}

// Stored K/V bytes that feed one 16-byte (compute-type) operand piece: 16
// bytes for bf16/fp32 caches, 8 FP8 bytes for 8 bf16 elements.
template <class T> struct KvRaw { using type = u32x4; };
template <> struct KvRaw<TFp8> { using type = u32x2; };
template <class T> constexpr int kKvPiece = 16 * T::KVB / T::EB;

// Byte offset, in a compute-type row, of the 16-byte QK operand piece that
// lane group G feeds to QK step k (the k-slot map: the 8 elements of the piece
// fill slots 8G .. 8G+7).  bf16/fp32: piece 64k + 16G (bf16: d = 32k + 8G + e).
// FP8 caches: 128*(k/2) + 32G + 16*(k%2) (d = 64*(k/2) + 16G + 8*(k%2) + e),
// so the stored bytes of steps 2j and 2j+1 are one contiguous 16-byte load
// (twice the bytes per load instruction of the bf16 map).  Every kernel of a
// type uses its type's map for both Q and K, so the bits never depend on the path.
template <class T> __device__ __forceinline__ constexpr int qk_piece_off(int k, int G) {
  if constexpr (T::KVB == 1) return 128 * (k >> 1) + 32 * G + 16 * (k & 1);
  else return 64 * k + 16 * G;
}

// Widen stored K/V bytes to the compute type.  FP8 E4M3 -> bf16 is exact
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1: every E4M3 value, subnormals
// included, is a bf16 value); element e of the piece is byte e.
template <class T>
__device__ __forceinline__ u32x4 kv_widen(const typename KvRaw<T>::type& r) {
  if constexpr (T::KVB == T::EB) {
    return r;
  } else {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[0], 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[0], 1.0f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[1], 1.0f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[1], 1.0f, true);
    return u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
                 __builtin_bit_cast(uint32_t, d)};
  }
}

template <class T>
__device__ __forceinline__ typename KvRaw<T>::type kv_load_raw(const unsigned char* p) {
  return *reinterpret_cast<const typename KvRaw<T>::type*>(p);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN).  Result in the low 16 bits.
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// LDS tiles.  A tile holds KT consecutive keys (tile-local row = key - j0) of
// one KV head, row-major with a 16-byte pad per row.
// ---------------------------------------------------------------------------
// Row pitches are chosen for the LDS banks: V rows are read by
// ds_read_b64_tr_b16, 4 rows x 32 bytes per 16 lanes (a 32-byte pad puts
// those 4 rows on disjoint banks).  K rows are read 16 bytes per lane from 16
// consecutive rows, and by the backward's dq kernel also through the
// transposing read; the same 32-byte pad measured faster than a 16-byte one
// (same bits: 8 x 8192 prefill +0.8%, its backward +2.4%).
#ifndef PKV_KPAD
#define PKV_KPAD 32
#endif
template <class T, int D>
struct TileGeom {
  static constexpr int ROW_BYTES = D * T::EB;          // 256 for bf16 d=128
  static constexpr int KPITCH = ROW_BYTES + PKV_KPAD;  // bytes between K rows in LDS
  static constexpr int VPITCH = ROW_BYTES + 32;        // bytes between V rows in LDS
  static constexpr int CPR = ROW_BYTES / 16;           // 16-byte chunks per row
  static constexpr int KBYTES = KT * KPITCH;           // K tile
  static constexpr int VBYTES = KT * VPITCH;           // V tile
  static constexpr int BYTES = KBYTES + VBYTES;        // K + V tile
  static constexpr int NK = ROW_BYTES / 64;            // 64-byte column groups (QK steps)
  static constexpr int DT = D / 16;                    // PV output d-tiles
  static constexpr int MT = KT / 16;                   // 16-key M tiles per tile
};

// ---------------------------------------------------------------------------
// Per-wave state of one chunk (online softmax over its tiles), for NT groups
// of 16 query columns.  Lane l serves column 16*nt + l%16 and, in the O^T
// accumulators, head-dim rows 16*dt + 4*(l/16) + i.
// ---------------------------------------------------------------------------
template <int D, int NT>
struct ChunkState {
  f32x4 o[NT][D / 16];
  float m[NT];  // running max of the chunk (score units)
  float l[NT];  // this lane's partial row sum (lanes of a column are summed at chunk end)
};

template <int D, int NT>
__device__ __forceinline__ void chunk_reset(ChunkState<D, NT>& st) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    st.m[nt] = -INFINITY;
    st.l[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) st.o[nt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// Q operands of one column group: lane l holds bytes [qk_piece_off(k, l/16), +16)
// of its column's query row, k = 0 .. NK-1 (64k + 16*(l/16) for bf16/fp32).  (bf16: the 8 elements that fill MFMA
// k-slots 8G..8G+7 of QK step k; fp32: 4 elements feeding 4 MFMA steps.)
template <class T, int D>
struct QOps {
  u32x4 v[TileGeom<T, D>::NK];
};

// ---------------------------------------------------------------------------
// QK^T for one tile: S^T[key][col] = sum over d of K[key][d] * Q[col][d].
// K operands (A): kop[mt][k] at lane l holds bytes [64k + 16G, +16) of key row
// 16mt + l%16 of the tile (G = l/16); Q operands (B) come from QOps.
// bf16 k-slot map of step k: slot 8G+e <-> d = 32k + 8G + e.
// fp32 step (k, e):          slot G    <-> d = 16k + 4G + e.
// The MFMA chain runs k (then e) in ascending order from a zero accumulator.
// Output s[mt][i] at lane l: key 16mt + 4G + i, column l%16.
// ---------------------------------------------------------------------------
template <class T, int D>
using KOps = u32x4[KT / 16][TileGeom<T, D>::NK];

template <class T, int D>
__device__ __forceinline__ void qk_tile(const KOps<T, D>& kop, const QOps<T, D>& q, f32x4 (&s)[KT / 16]) {
  using G_ = TileGeom<T, D>;
#pragma unroll
  for (int mt = 0; mt < G_::MT; ++mt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < G_::NK; ++k) {
      if constexpr (T::EB == 2) {
        acc = mfma_bf16(kop[mt][k], q.v[k], acc);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc = mfma_f32(__uint_as_float(kop[mt][k][e]), __uint_as_float(q.v[k][e]), acc);
      }
    }
    s[mt] = acc;
  }
}

// K operands of a tile staged row-major in LDS (row pitch G_::KPITCH).
template <class T, int D>
__device__ __forceinline__ void k_operands_lds(const unsigned char* k_lds, KOps<T, D>& kop) {
  using G_ = TileGeom<T, D>;
  const int lane = lane_id();
  const unsigned char* base = k_lds + (lane & 15) * G_::KPITCH;
#pragma unroll
  for (int mt = 0; mt < G_::MT; ++mt)
#pragma unroll
    for (int k = 0; k < G_::NK; ++k)
      kop[mt][k] = *reinterpret_cast<const u32x4*>(base + mt * 16 * G_::KPITCH + qk_piece_off<T>(k, lane >> 4));
}

// QK^T with the K operands read from the LDS tile one M tile at a time (same
// MFMA chain as qk_tile).
template <class T, int D>
__device__ __forceinline__ void qk_tile_lds(const unsigned char* k_lds, const QOps<T, D>& q, f32x4 (&s)[KT / 16]) {
  using G_ = TileGeom<T, D>;
  const int lane = lane_id();
  const unsigned char* base = k_lds + (lane & 15) * G_::KPITCH;
#pragma unroll
  for (int mt = 0; mt < G_::MT; ++mt) {
    KOps<T, D> kop;
#pragma unroll
    for (int k = 0; k < G_::NK; ++k)
      kop[0][k] = *reinterpret_cast<const u32x4*>(base + mt * 16 * G_::KPITCH + qk_piece_off<T>(k, lane >> 4));
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < G_::NK; ++k) {
      if constexpr (T::EB == 2) {
        acc = mfma_bf16(kop[0][k], q.v[k], acc);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc = mfma_f32(__uint_as_float(kop[0][k][e]), __uint_as_float(q.v[k][e]), acc);
      }
    }
    s[mt] = acc;
  }
}

// QK^T for one tile with all K operands read first and the M tiles' MFMA
// chains interleaved (k outer, M tile inner): each accumulator sees the
// qk_tile chain, but consecutive MFMAs are independent.
template <class T, int D>
__device__ __forceinline__ void qk_tile_lds_ilp(const unsigned char* k_lds, const QOps<T, D>& q,
                                                f32x4 (&s)[KT / 16]) {
  using G_ = TileGeom<T, D>;
  static_assert(T::EB == 2, "bf16 compute type");
  KOps<T, D> kop;
  k_operands_lds<T, D>(k_lds, kop);
#pragma unroll
  for (int mt = 0; mt < G_::MT; ++mt) s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < G_::NK; ++k)
#pragma unroll
    for (int mt = 0; mt < G_::MT; ++mt) s[mt] = mfma_bf16(kop[mt][k], q.v[k], s[mt]);
}

// QK^T of NT column groups with the K operands read from LDS one M tile at a
// time, each M tile's operands serving every group (the qk_tile chain per group).
template <class T, int D, int NT>
__device__ __forceinline__ void qk_tiles_lds(const unsigned char* k_lds, const QOps<T, D> (&q)[NT],
                                             f32x4 (&s)[NT][KT / 16]) {
  using G_ = TileGeom<T, D>;
  const int lane = lane_id();
  const unsigned char* base = k_lds + (lane & 15) * G_::KPITCH;
#pragma unroll
  for (int mt = 0; mt < G_::MT; ++mt) {
    u32x4 kx[G_::NK];
#pragma unroll
    for (int k = 0; k < G_::NK; ++k)
      kx[k] = *reinterpret_cast<const u32x4*>(base + mt * 16 * G_::KPITCH + qk_piece_off<T>(k, lane >> 4));
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < G_::NK; ++k) {
        if constexpr (T::EB == 2) {
          acc = mfma_bf16(kx[k], q[nt].v[k], acc);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = mfma_f32(__uint_as_float(kx[k][e]), __uint_as_float(q[nt].v[k][e]), acc);
        }
      }
      s[nt][mt] = acc;
    }
  }
}

// V^T operand (A) of PV step ks for d-tile dt, bf16: slot 8G+e <-> key
// 32ks + 4G + e (e < 4) and 32ks + 16 + 4G + (e - 4) (e >= 4), head-dim row
// 16dt + l%16.  ds_read_b64_tr_b16 turns four 8-byte row pieces of the 16
// lanes of a group into one column per lane.
__device__ __forceinline__ u32x4 v_operand_bf16(const unsigned char* v_lds, int pitch, int ks, int dt) {
  const int lane = lane_id();
  const int G = lane >> 4;
  const int j = lane & 15;
#if PKV_V_TRANSPOSE_READ
  const unsigned char* p0 = v_lds + (32 * ks + 4 * G + (j >> 2)) * pitch + 2 * (16 * dt + 4 * (j & 3));
  const unsigned char* p1 = p0 + 16 * pitch;
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PKV_LDS i16x4*)(p0));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PKV_LDS i16x4*)(p1));
  u32x2 a = __builtin_bit_cast(u32x2, lo);
  u32x2 b = __builtin_bit_cast(u32x2, hi);
  return u32x4{a[0], a[1], b[0], b[1]};
#else
  const unsigned char* col = v_lds + 2 * (16 * dt + j);
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int key = 32 * ks + (e < 4 ? 4 * G + e : 16 + 4 * G + (e - 4));
    h[e] = *reinterpret_cast<const uint16_t*>(col + key * pitch);
  }
  return u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
#endif
}

// Butterfly steps across lanes 16 and 32 apart without an LDS round trip:
// v_permlane16_swap / v_permlane32_swap with both operands x give, in every
// lane, the pair (value of the lower lane, value of the upper lane) of its
// xor partner pair, so both lanes of a pair combine the same two values in the
// same operand order (max and add are commutative, so the bits equal those of
// a shuffle-based butterfly).
// max of two lane values after a permlane swap.  fmaxf would first quiet
// each operand (two v_max_f32 x, x, which the compiler cannot prove
// redundant for permlane results); the operands are arithmetic results, so
// never signalling NaNs, and one v_max_f32 gives the value fmaxf would (same
// bits; 8 fewer VALU instructions per 64-key tile of two column groups:
// re-score +2.8%, prefill +0.9%, 17-token chunked prefill +1.5%).
__device__ __forceinline__ float max_pair(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_pair(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_pair(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// One tile of the chunk core for NT column groups.
//   s        raw QK^T accumulators per column group (from qk_tile), consumed
//   lim[nt]  this lane's column sees keys < lim (global positions); columns
//            that do not exist carry lim = INT_MAX (their values are never
//            stored)
//   j0       global position of the tile's first key
//   mul      score multiplier, > 0 (scale, times log2(e) for bf16)
// Steps per column: raw scores of invisible keys set to -inf; tile max of the
// raw scores (exact) times mul gives the tile max m_tile of the scaled scores.
// The column keeps a reference max m (-inf before its first visible key); it
// moves to m_tile only when m is -inf or m_tile > m + slack, with alpha =
// exp(m_old - m_new) (0 from -inf), else alpha = 1 exactly.  p = exp(s*mul -
// m) with the product fused (exactly 0 for invisible keys, at most
// exp(slack)); l = fma(l, alpha, sum of this lane's fp32 p in (mt, i) order);
// o = o * alpha; o += P V by MFMA in PV-step order, where the bf16 path feeds
// P to the MFMA rounded once to bf16 (v_cvt_pk_bf16_f32, round to nearest
// even).  The row sum uses the unrounded p: summing the rounded values would
// bias the LSE of short rows by up to 2^-9.  Every decision is per column, so
// a column's bits never depend on the other columns sharing its wave.
// Two shortcuts change no bit: when every column of the wave sees the whole
// tile the per-key mask is skipped (kShortcuts; it would select nothing), and
// when every column's alpha is exactly 1 the multiply of o is skipped.
// ---------------------------------------------------------------------------
struct NoMid {
  __device__ __forceinline__ void operator()() const {}
};

// `mid` runs between the softmax and the P.V products (the full-path kernels
// issue the next tile's loads there, into registers the scores no longer use).
// The softmax half of the chunk core: masks, max, alpha, p, l, o *= alpha and,
// for the bf16 compute type, the bf16 P operands pb (fp32 keeps p in s).
template <class T, int D, int NT, bool kShortcuts = true>
__device__ __forceinline__ void softmax_part(ChunkState<D, NT>& st, f32x4 (&s)[NT][KT / 16],
                                             const int (&lim)[NT], int j0, float mul, u32x4 (&pb)[NT][KT / 32]) {
  using G_ = TileGeom<T, D>;
  const int lane = lane_id();
  const int G = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const bool whole = kShortcuts && __all(j0 + KT <= lim[nt]);
    if (!whole) {
      // key j0 + 16mt + 4G + i is past the limit iff 16mt + i >= lim - j0 - 4G
      // (one bound per lane; the offsets are compile-time constants)
      const int bound = lim[nt] - j0 - 4 * G;
#pragma unroll
      for (int mt = 0; mt < G_::MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (16 * mt + i >= bound) s[nt][mt][i] = -INFINITY;
        }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < G_::MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, s[nt][mt][i]);
    tmax = max_xor16(tmax);
    tmax = max_xor32(tmax);
    // mul > 0, so the max of the scaled scores is the scaled max (rounding is monotone).
    const float m_tile = tmax * mul;
    const float m_old = st.m[nt];
    float m_new = m_old;
    float alpha = 1.f;
    if (m_old == -INFINITY || m_tile > m_old + kRescaleSlack<T>) {
      m_new = m_tile;
      alpha = (m_old == -INFINITY) ? 0.f : pkv_exp<T>(m_old - m_new);
    }
    // Invisible keys hold -inf, so exp gives exactly 0 once the column has a
    // finite reference; a column with nothing visible yet subtracts 0 instead
    // of -inf (its p are all exp(-inf) = 0).
    const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
    float tsum = 0.f;
#pragma unroll
    for (int mt = 0; mt < G_::MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = pkv_exp<T>(fmaf(s[nt][mt][i], mul, -m_ref));
        s[nt][mt][i] = p;
        tsum = tsum + p;
      }
    st.l[nt] = fmaf(st.l[nt], alpha, tsum);
    st.m[nt] = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < G_::DT; ++dt) st.o[nt][dt] = st.o[nt][dt] * alpha;
    }
    if constexpr (T::EB == 2) {
#pragma unroll
      for (int ks = 0; ks < KT / 32; ++ks) {
        const f32x4 a = s[nt][2 * ks];
        const f32x4 b = s[nt][2 * ks + 1];
        const bf16x2 p0 = {(__bf16)a[0], (__bf16)a[1]};
        const bf16x2 p1 = {(__bf16)a[2], (__bf16)a[3]};
        const bf16x2 p2 = {(__bf16)b[0], (__bf16)b[1]};
        const bf16x2 p3 = {(__bf16)b[2], (__bf16)b[3]};
        pb[nt][ks] = u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                           __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
      }
    }
  }
}

// The P.V half of the chunk core for the bf16 compute type: o += P V by MFMA
// in PV-step order.
// kAhead: V operand reads in flight ahead of the MFMAs (with kPinVReads).
template <class T, int D, int NT, bool kPinVReads = false, int kAhead = 1>
__device__ __forceinline__ void pv_part(ChunkState<D, NT>& st, const u32x4 (&pb)[NT][KT / 32],
                                        const unsigned char* v_lds) {
  using G_ = TileGeom<T, D>;
  static_assert(T::EB == 2, "bf16 compute type");
  {
#if PKV_MFMA_PRIO
    __builtin_amdgcn_s_setprio(1);
#endif
#if PKV_V_AHEAD
    if constexpr (kPinVReads) {
      // V operands read kAhead steps ahead of the MFMAs that use them
      constexpr int KS = KT / 32;
      constexpr int NS = G_::DT * KS;
      u32x4 vq[kAhead];
#pragma unroll
      for (int i = 0; i < kAhead; ++i) vq[i] = v_operand_bf16(v_lds, G_::VPITCH, i / G_::DT, i % G_::DT);
#pragma unroll
      for (int step = 0; step < NS; ++step) {
        // ks outer: consecutive MFMAs go to different d-tiles (each d-tile
        // still takes its steps in ascending ks; 1-2% faster than dt outer)
        const int dt = step % G_::DT, ks = step / G_::DT;
        const u32x4 va = vq[step % kAhead];
        if (step + kAhead < NS)
          vq[step % kAhead] = v_operand_bf16(v_lds, G_::VPITCH, (step + kAhead) / G_::DT, (step + kAhead) % G_::DT);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) st.o[nt][dt] = mfma_bf16(va, pb[nt][ks], st.o[nt][dt]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else
#endif
#pragma unroll
    for (int dt = 0; dt < G_::DT; ++dt) {
#pragma unroll
      for (int ks = 0; ks < KT / 32; ++ks) {
        const u32x4 va = v_operand_bf16(v_lds, G_::VPITCH, ks, dt);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) st.o[nt][dt] = mfma_bf16(va, pb[nt][ks], st.o[nt][dt]);
      }
      // Optionally keep each d-tile's V operand reads next to its MFMAs, so the
      // scheduler cannot hoist all of them (caps live registers; no effect on
      // the arithmetic).
      if constexpr (kPinVReads) __builtin_amdgcn_sched_barrier(0);
    }
#if PKV_MFMA_PRIO
    __builtin_amdgcn_s_setprio(0);
#endif
  }
}

template <class T, int D, int NT, bool kPinVReads = false, bool kShortcuts = true, int kAhead = 1,
          class Mid = NoMid>
__device__ __forceinline__ void softmax_pv_tile(ChunkState<D, NT>& st, f32x4 (&s)[NT][KT / 16],
                                                const int (&lim)[NT], int j0, float mul,
                                                const unsigned char* v_lds, const Mid& mid = Mid{}) {
  using G_ = TileGeom<T, D>;
  const int lane = lane_id();
  const int G = lane >> 4;
  // P operands: bf16 -> 2 PV steps of 32 keys (packed u32x4); fp32 -> s itself.
  u32x4 pb[NT][KT / 32];
  softmax_part<T, D, NT, kShortcuts>(st, s, lim, j0, mul, pb);
  mid();
  if constexpr (T::EB == 2) {
    pv_part<T, D, NT, kPinVReads, kAhead>(st, pb, v_lds);
  } else {
    // fp32 PV step (mt, i): slot G <-> key 16mt + 4G + i.
    const unsigned char* col = v_lds + 4 * (lane & 15);
#pragma unroll
    for (int dt = 0; dt < G_::DT; ++dt)
#pragma unroll
      for (int mt = 0; mt < G_::MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float va = *reinterpret_cast<const float*>(col + (16 * mt + 4 * G + i) * G_::VPITCH + 4 * 16 * dt);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) st.o[nt][dt] = mfma_f32(va, s[nt][mt][i], st.o[nt][dt]);
        }
  }
}

// Column sum of the per-lane partial l (lanes 16 apart hold the same column):
// a fixed xor butterfly, so every lane of the column gets the same bits.
__device__ __forceinline__ float column_sum(float x) {
  x = add_xor16(x);
  x = add_xor32(x);
  return x;
}

// ---------------------------------------------------------------------------
// The fold of one chunk result (mc, lc, oc) into a row state (M, L, O), in
// ascending chunk order.  A chunk with no visible key (mc = -inf) is skipped.
// ---------------------------------------------------------------------------
template <class T>
struct FoldCoef {
  float mn, a, b;
};

template <class T>
__device__ __forceinline__ FoldCoef<T> fold_coef(float M, float mc) {
  FoldCoef<T> f;
  f.mn = fmaxf(M, mc);
  f.a = (M == -INFINITY) ? 0.f : pkv_exp<T>(M - f.mn);
  f.b = pkv_exp<T>(mc - f.mn);
  return f;
}
__device__ __forceinline__ float fold_val(float acc, float a, float x, float b) { return fmaf(acc, a, x * b); }

// Final write: out = O / L rounded once to the output type; lse in natural log.
// fp32: M + ln L evaluated in double and rounded once to fp32, so the final
// step adds at most half an fp32 ulp of the result (in fp32, logf's error and
// the rounding of the sum came on top of it: 1.06e-6 at a 5000-key LSE near 9,
// where the ulp is 9.5e-7).  Every kernel's final write calls this, so the
// decode and prefill paths keep the same bits.
template <class T>
__device__ __forceinline__ float final_lse(float M, float L) {
  if (M == -INFINITY) return -INFINITY;
  if constexpr (T::kBase2) return pkv_lse<T>(M, L);
  else return static_cast<float>(static_cast<double>(M) + log(static_cast<double>(L)));
}
// vs: the stored-V scale (1 for unscaled caches: the multiply is then exact).
__device__ __forceinline__ float final_val(float M, float O, float L, float vs) {
  return M == -INFINITY ? 0.f : (O / L) * vs;
}

}  // namespace pkv
