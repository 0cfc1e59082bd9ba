// pkv_tiles.hpp -- data movement shared by the forward and backward kernels
// of libpkv: the paged K/V tile loader (with the fused-append redirection) and
// the per-column visibility limit.  No arithmetic that decides a result bit.
#pragma once

#include "pkv_device.hpp"
#include "pkv_internal.h"

#ifndef PKV_TILE_IDS_FAST
#define PKV_TILE_IDS_FAST 1
#endif

namespace pkv {

// Fused append: key positions >= n_old are this call's own rows and are read
// from k_new / v_new (row row0 + position - n_old); the work group with
// writer set also stores them into the cache, so after the call the cache
// holds exactly what pkv_cache_write would have put there, and every read saw
// the same bits it would have read after that write.
struct Append {
  int n_old = INT_MAX;  // first appended key position (INT_MAX: no append)
  int64_t row0 = 0;     // k_new row holding position n_old
  bool writer = false;  // this work group stores the appended rows
};

template <bool APPEND>
__device__ __forceinline__ Append make_append(int n, int L, int q0, bool last_block) {
  Append ap;
  if constexpr (APPEND) {
    ap.n_old = n - L;
    ap.row0 = q0;
    ap.writer = last_block;
  }
  return ap;
}

// Address of the stored piece at byte `byte_off` of key row jc (cache address
// `cache`), redirected to the caller's new rows under fused append (the new
// rows are in the cache's storage type).
template <class T, int D, bool APPEND>
__device__ __forceinline__ const unsigned char* kv_src(const void* new_base, int nhk, int hk, int jc,
                                                        const Append& ap, const unsigned char* cache, int byte_off) {
  if constexpr (APPEND) {
    const int64_t nrow = (ap.row0 + (jc - ap.n_old)) * nhk + hk;
    const unsigned char* np = static_cast<const unsigned char*>(new_base) + nrow * D * T::KVB + byte_off;
    return jc >= ap.n_old ? np : cache;
  } else {
    return cache;
  }
}

template <class T, bool APPEND>
__device__ __forceinline__ void kv_store_new(const Append& ap, bool in, int jc, void* store_base, const void* load_base,
                                             const unsigned char* cache, const typename KvRaw<T>::type& x) {
  if constexpr (APPEND) {
    if (ap.writer && in && jc >= ap.n_old) {
      unsigned char* dst = static_cast<unsigned char*>(store_base) + (cache - static_cast<const unsigned char*>(load_base));
      *reinterpret_cast<typename KvRaw<T>::type*>(dst) = x;
    }
  }
}

// K/V tile loader: keys j0 .. j0+KT-1 of one sequence and KV head into LDS
// (in the compute type), consecutive lanes on consecutive 16-byte pieces of a
// key row (16 stored bytes, or 8 FP8 bytes widened to 16).  The block address
// uses the real block stride (contiguous or K/V-interleaved caches alike).
// Keys >= jmax are not read; their rows are zero.
// U (block size a multiple of 16, in-block offsets below 2^31 bytes, block
// strides below 2^32 bytes): the rows
// one wave loads with one instruction lie in one 16-row group, hence in one
// cache block; its id is a scalar load and the address a scalar block base
// plus a 32-bit lane offset, instead of a per-lane table lookup and 64-bit
// address arithmetic for every piece.
template <class T, int D, int W, bool APPEND, bool U = false>
__device__ __forceinline__ void load_tile(const AttnArgs& a, const int32_t* bt, int hk, int j0, int jmax,
                                          unsigned char* k_lds, unsigned char* v_lds, const Append& ap) {
  using G_ = TileGeom<T, D>;
  constexpr int NCH = KT * G_::CPR;
  constexpr int PER = NCH / (64 * W);
  static_assert(PER * 64 * W == NCH, "tile chunks must split evenly over the work group");
  constexpr int R = PER < 16 ? PER : 16;
  const unsigned char* kb = static_cast<const unsigned char*>(a.k);
  const unsigned char* vb = static_cast<const unsigned char*>(a.v);
#pragma unroll
  for (int r0 = 0; r0 < PER; r0 += R) {
    // U: the block ids of this wave's row groups, all scalar loads issued
    // before any of them is used.  Clamped rows stay in their group's block:
    // a group holds rows past jmax only if jmax - 1 is in it, or the whole
    // group clamps to it.
    // Unsigned (block ids are non-negative): widening it needs no instruction,
    // whereas a sign extension next to the load would wait for the load.
    uint32_t ublk[R];
    int ubase[R];
    if constexpr (U) {
      static_assert(64 % G_::CPR == 0 && 64 / G_::CPR <= 16, "a wave's rows must lie in one 16-row group");
      using cint = const __attribute__((address_space(4))) int32_t;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int row = (threadIdx.x + (r0 + i) * 64 * W) / G_::CPR;
        const int g0 = __builtin_amdgcn_readfirstlane(row) & ~15;
        const int bi = div_block(min(j0 + g0, jmax - 1), a.bs_mul, a.bs_shift);
        ublk[i] = static_cast<uint32_t>(((cint*)bt)[bi]);  // the table is not written while a kernel runs
        ubase[i] = bi * a.bs;
      }
    }
    u32x4 kr[R], vr[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int qi = threadIdx.x + (r0 + i) * 64 * W;
      const int row = qi / G_::CPR, part = qi % G_::CPR;
      const int j = j0 + row;
      const int jc = min(j, jmax - 1);  // rows past jmax load a visible row, then read as zero
      const int off = kKvPiece<T> * part;
      const unsigned char* kc;
      const unsigned char* vc;
      if constexpr (U) {
        const int slot = jc - ubase[i];
        const int64_t blk = static_cast<int64_t>(static_cast<uint64_t>(ublk[i]));
        kc = kb + (blk * a.kbs + (int64_t)hk * a.khs) * T::KVB +
             static_cast<uint32_t>(slot * static_cast<int>(a.kss) * T::KVB + off);
        vc = vb + (blk * a.vbs + (int64_t)hk * a.vhs) * T::KVB +
             static_cast<uint32_t>(slot * static_cast<int>(a.vss) * T::KVB + off);
      } else {
        const int bi = div_block(jc, a.bs_mul, a.bs_shift);
        const int64_t blk = bt[bi];
        const int64_t slot = jc - bi * a.bs;
        kc = kb + (blk * a.kbs + slot * a.kss + hk * a.khs) * T::KVB + off;
        vc = vb + (blk * a.vbs + slot * a.vss + hk * a.vhs) * T::KVB + off;
      }
      const int nhk = a.hq / a.g;
      const auto kv = kv_load_raw<T>(kv_src<T, D, APPEND>(a.k_new, nhk, hk, jc, ap, kc, off));
      const auto vv = kv_load_raw<T>(kv_src<T, D, APPEND>(a.v_new, nhk, hk, jc, ap, vc, off));
      const bool in = j < jmax;
      kv_store_new<T, APPEND>(ap, in, jc, a.k_store, a.k, kc, kv);
      kv_store_new<T, APPEND>(ap, in, jc, a.v_store, a.v, vc, vv);
      kr[i] = kv_widen<T>(kv);
      vr[i] = kv_widen<T>(vv);
    }
    // rows past jmax read as zero; only a tile reaching past jmax has any
    if (j0 + KT > jmax) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int row = (threadIdx.x + (r0 + i) * 64 * W) / G_::CPR;
        if (j0 + row >= jmax) {
          kr[i] = u32x4{0, 0, 0, 0};
          vr[i] = u32x4{0, 0, 0, 0};
        }
      }
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int qi = threadIdx.x + (r0 + i) * 64 * W;
      const int row = qi / G_::CPR, part = qi % G_::CPR;
      *reinterpret_cast<u32x4*>(k_lds + row * G_::KPITCH + 16 * part) = kr[i];
      *reinterpret_cast<u32x4*>(v_lds + row * G_::VPITCH + 16 * part) = vr[i];
    }
  }
}

// The same tile load split in two, so the loads can be in flight while the
// previous tile is computed: tile_issue loads a tile's stored bytes into a
// register stage (nothing waits for them there); tile_commit, after the
// barrier that frees the LDS tile, widens them, zeroes rows past jmax, does
// the fused-append store and writes the LDS tile.  Same bytes, same LDS
// layout as load_tile.
template <class T, int D, int W>
struct TileStage {
  static constexpr int PER = KT * TileGeom<T, D>::CPR / (64 * W);
  typename KvRaw<T>::type k[PER], v[PER];
};

// Block ids of a tile's row groups fetched one tile ahead of the loads that
// use them (U only): lane i < PER holds the id of the wave's i-th row group.
// A vector load, issued right after the previous tile's K/V loads, so the wait
// for it comes where those loads are waited for anyway; a scalar id load
// issued together with the K/V loads put the table's latency in front of
// every tile's loads.
struct TileIds {
  uint32_t v = 0;
};

// `tid` (tile_ids_fetch, tile_issue, tile_commit): the thread's index among
// the 64 * W threads that share the tile's pieces (default: threadIdx.x, the
// whole work group; a subset of the waves passes its own numbering).
template <class T, int D, int W, bool U>
__device__ __forceinline__ void tile_ids_fetch(const AttnArgs& a, const int32_t* bt, int j0, int jmax, TileIds& ids,
                                               int tid = -1) {
  if constexpr (U) {
    using G_ = TileGeom<T, D>;
    constexpr int PER = TileStage<T, D, W>::PER;
    const int t = tid < 0 ? static_cast<int>(threadIdx.x) : tid;
    const int i = min(lane_id(), PER - 1);
    const int g0 = ((t & ~63) + i * 64 * W) / G_::CPR & ~15;
    ids.v = static_cast<uint32_t>(bt[div_block(min(j0 + g0, jmax - 1), a.bs_mul, a.bs_shift)]);
  }
}

template <class T, int D, int W, bool APPEND, bool U, bool kFetched = false>
__device__ __forceinline__ void tile_issue(const AttnArgs& a, const int32_t* bt, int hk, int j0, int jmax,
                                           TileStage<T, D, W>& stg, const Append& ap, const TileIds& ids = {},
                                           int tid = -1) {
  using G_ = TileGeom<T, D>;
  constexpr int PER = TileStage<T, D, W>::PER;
  const int t = tid < 0 ? static_cast<int>(threadIdx.x) : tid;
  const unsigned char* kb = static_cast<const unsigned char*>(a.k);
  const unsigned char* vb = static_cast<const unsigned char*>(a.v);
  uint32_t ublk[PER];  // U: block ids of the wave's row groups (see load_tile)
  int ubase[PER];
  if constexpr (U) {
    static_assert(64 % G_::CPR == 0 && 64 / G_::CPR <= 16, "a wave's rows must lie in one 16-row group");
    using cint = const __attribute__((address_space(4))) int32_t;
    auto per_group = [&] {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int row = (t + i * 64 * W) / G_::CPR;
        const int g0 = __builtin_amdgcn_readfirstlane(row) & ~15;
        const int bi = div_block(min(j0 + g0, jmax - 1), a.bs_mul, a.bs_shift);
        if constexpr (kFetched)
          ublk[i] = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(ids.v), i));
        else
          ublk[i] = static_cast<uint32_t>(((cint*)bt)[bi]);
        ubase[i] = bi * a.bs;
      }
    };
#if PKV_TILE_IDS_FAST
    // A tile below jmax (no clamped rows): with a block size that is a
    // multiple of the tile, the whole tile lies in one block (one id); with
    // 16-key blocks and 16 rows between a lane's pieces (4 waves, 16 pieces
    // per row), piece i of every wave lies in the tile's i-th block, so the
    // ids are four consecutive table entries.
    if constexpr (!kFetched) {
      if (j0 + KT <= jmax && (a.bs & (KT - 1)) == 0) {
        const int bi = div_block(j0, a.bs_mul, a.bs_shift);
        const uint32_t id = static_cast<uint32_t>(((cint*)bt)[bi]);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          ublk[i] = id;
          ubase[i] = bi * a.bs;
        }
      } else if (64 * W / G_::CPR == 16 && PER == KT / 16 && j0 + KT <= jmax && a.bs == 16) {
        const int b0 = j0 >> 4;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          ublk[i] = static_cast<uint32_t>(((cint*)bt)[b0 + i]);
          ubase[i] = (b0 + i) << 4;
        }
      } else {
        per_group();
      }
    } else
#endif
      per_group();
  }
  // U: block strides below 2^32 bytes, so a block's base offset is one
  // 32 x 32-bit product (measured 3% faster on the 8 x 8192 prefill than the
  // 64-bit product)
  const uint32_t kbsb = static_cast<uint32_t>(a.kbs) * T::KVB, vbsb = static_cast<uint32_t>(a.vbs) * T::KVB;
  const unsigned char* const kbh = kb + (int64_t)hk * a.khs * T::KVB;
  const unsigned char* const vbh = vb + (int64_t)hk * a.vhs * T::KVB;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int qi = t + i * 64 * W;
    const int row = qi / G_::CPR, part = qi % G_::CPR;
    const int jc = min(j0 + row, jmax - 1);
    const int off = kKvPiece<T> * part;
    const unsigned char* kc;
    const unsigned char* vc;
    if constexpr (U) {
      const int slot = jc - ubase[i];
      kc = kbh + static_cast<uint64_t>(ublk[i]) * kbsb + static_cast<uint32_t>(slot * static_cast<int>(a.kss) * T::KVB + off);
      vc = vbh + static_cast<uint64_t>(ublk[i]) * vbsb + static_cast<uint32_t>(slot * static_cast<int>(a.vss) * T::KVB + off);
    } else {
      const int bi = div_block(jc, a.bs_mul, a.bs_shift);
      const int64_t blk = bt[bi];
      const int64_t slot = jc - bi * a.bs;
      kc = kb + (blk * a.kbs + slot * a.kss + hk * a.khs) * T::KVB + off;
      vc = vb + (blk * a.vbs + slot * a.vss + hk * a.vhs) * T::KVB + off;
    }
    const int nhk = a.hq / a.g;
    stg.k[i] = kv_load_raw<T>(kv_src<T, D, APPEND>(a.k_new, nhk, hk, jc, ap, kc, off));
    stg.v[i] = kv_load_raw<T>(kv_src<T, D, APPEND>(a.v_new, nhk, hk, jc, ap, vc, off));
  }
}

template <class T, int D, int W, bool APPEND>
__device__ __forceinline__ void tile_commit(const AttnArgs& a, const int32_t* bt, int hk, int j0, int jmax,
                                            const TileStage<T, D, W>& stg, unsigned char* k_lds,
                                            unsigned char* v_lds, const Append& ap, int tid = -1) {
  using G_ = TileGeom<T, D>;
  constexpr int PER = TileStage<T, D, W>::PER;
  const int t = tid < 0 ? static_cast<int>(threadIdx.x) : tid;
  if constexpr (APPEND) {
    // the writer stores this call's new rows (only the tiles reaching them)
    if (ap.writer && j0 + KT > ap.n_old) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int qi = t + i * 64 * W;
        const int row = qi / G_::CPR, part = qi % G_::CPR;
        const int j = j0 + row;
        const int jc = min(j, jmax - 1);
        const int bi = div_block(jc, a.bs_mul, a.bs_shift);
        const int64_t blk = bt[bi];
        const int64_t slot = jc - bi * a.bs;
        const int off = kKvPiece<T> * part;
        const unsigned char* kc = static_cast<const unsigned char*>(a.k) + (blk * a.kbs + slot * a.kss + hk * a.khs) * T::KVB + off;
        const unsigned char* vc = static_cast<const unsigned char*>(a.v) + (blk * a.vbs + slot * a.vss + hk * a.vhs) * T::KVB + off;
        kv_store_new<T, APPEND>(ap, j < jmax, jc, a.k_store, a.k, kc, stg.k[i]);
        kv_store_new<T, APPEND>(ap, j < jmax, jc, a.v_store, a.v, vc, stg.v[i]);
      }
    }
  }
  u32x4 kr[PER], vr[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    kr[i] = kv_widen<T>(stg.k[i]);
    vr[i] = kv_widen<T>(stg.v[i]);
  }
  // piece i of this lane is tile row row0 + i * STEP, 16-byte part `part`
  constexpr int STEP = 64 * W / G_::CPR;
  static_assert(STEP * G_::CPR == 64 * W, "a work group's pieces cover whole rows");
  const int row0 = t / G_::CPR, part = t % G_::CPR;
  if (j0 + KT > jmax) {  // rows past jmax read as zero
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (j0 + row0 + i * STEP >= jmax) {
        kr[i] = u32x4{0, 0, 0, 0};
        vr[i] = u32x4{0, 0, 0, 0};
      }
    }
  }
  unsigned char* const kp = k_lds + row0 * G_::KPITCH + 16 * part;
  unsigned char* const vp = v_lds + row0 * G_::VPITCH + 16 * part;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    *reinterpret_cast<u32x4*>(kp + i * STEP * G_::KPITCH) = kr[i];
    *reinterpret_cast<u32x4*>(vp + i * STEP * G_::VPITCH) = vr[i];
  }
}

// Keys visible to column `col` of a sequence: j < limit.  Columns are ordered
// row-major over (row r, head-in-group hh): col = r * g + hh.  Row r sits at
// key position n - L + r (bottom-right alignment).
__device__ __forceinline__ int column_limit(int col, int ncols, int g, int n, int L, int causal) {
  if (col >= ncols) return INT_MAX;  // no such column: its values are never stored
  const int p = n - L + col / g;
  return causal ? min(p + 1, n) : n;
}

}  // namespace pkv
