// pkv_attn.hip -- attention kernels of libpkv for gfx950.
//
// Split (decode) path: one work item per (sequence, KV head, column block, run
// of chunks) writes one fp32 partial (max, sum, o[d]) per chunk and column;
// merge_kernel then folds a row's partials in ascending chunk index and makes
// the final write.
//   decode_kernel             bf16, up to 16 columns per KV head: one wave, K/V
//                             loaded straight into registers a tile ahead.
//   decode2_kernel            the same with two tiles in flight: FP8 caches,
//                             and bf16 when the grid exceeds 1024 work items.
//   attn_kernel<SPLIT=true>   more columns (or fp32): 8 waves x 16 columns
//                             sharing LDS tiles (bf16/FP8: three tile buffers,
//                             the odd waves' P.V one tile late; with at most 96
//                             columns the two column-less waves load and stage
//                             every tile and the others only compute).
//   decode_plan_kernel        ragged batches: prefix counts for the one-wave
//                             kernels' longest-first job order.
// Full (prefill) path: one work item per (sequence, KV head, column block)
// runs the chunks in ascending order, folds them in registers and makes the
// final write.
//   attn_kernel<SPLIT=false>  4 (or, for few columns per KV head over long
//                             contexts, 8) waves x 2 column groups, LDS tiles
//                             double-buffered from a register stage.
//   prefill_kernel            the 8-wave x 16-column pipelined variant (kept as a
//                             bitwise cross-check, PKV_OPT_FULL_KERNEL = 1).
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
#include "pkv_tiles.hpp"

namespace pkv {

template <class T, int D>
__device__ __forceinline__ void store_out(void* out, int64_t elem, const f32x4 (&o)[D / 16], float M, float Ls,
                                          float vs) {
  const int G = lane_id() >> 4;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const int e = 16 * dt + 4 * G;
    float v0 = final_val(M, o[dt][0], Ls, vs), v1 = final_val(M, o[dt][1], Ls, vs);
    float v2 = final_val(M, o[dt][2], Ls, vs), v3 = final_val(M, o[dt][3], Ls, vs);
    if constexpr (T::EB == 2) {
      u32x2 w = {bf16_rne_bits(v0) | (bf16_rne_bits(v1) << 16), bf16_rne_bits(v2) | (bf16_rne_bits(v3) << 16)};
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + elem + e) = w;
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(out) + elem + e) = f32x4{v0, v1, v2, v3};
    }
  }
}

// A row with a single chunk (AttnArgs::direct): the chunk result (mc, lc, oc)
// folded into the empty row state and written, the same operations the merge
// and the full path apply to a row whose keys lie in one chunk (mc = -inf, no
// visible key: out = 0, lse = -inf).
template <class T, int D>
__device__ __forceinline__ void write_one_chunk(const AttnArgs& a, int64_t rh, float mc, float lc,
                                                const f32x4 (&oc)[D / 16]) {
  float M = -INFINITY, Ls = 0.f;
  f32x4 O[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (mc != -INFINITY) {
    const FoldCoef<T> f = fold_coef<T>(M, mc);
    Ls = fold_val(Ls, f.a, lc, f.b);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) O[dt][i] = fold_val(O[dt][i], f.a, oc[dt][i], f.b);
    M = f.mn;
  }
  if ((lane_id() >> 4) == 0) a.lse[rh] = final_lse<T>(M, Ls);
  store_out<T, D>(a.out, rh * D, O, M, Ls, a.v_scale);
}

// The direct write of columns without a visible key (a column block whose
// sequence has no key for any of its rows: no chunk to compute).
template <class T, int D>
__device__ __forceinline__ void write_empty_column(const AttnArgs& a, int64_t rh) {
  f32x4 z[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) z[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  write_one_chunk<T, D>(a, rh, -INFINITY, 0.f, z);
}

#ifndef PKV_ATTN_XCD
#define PKV_ATTN_XCD 1
#endif
#ifndef PKV_QK_PER_MT
#define PKV_QK_PER_MT 1
#endif
#ifndef PKV_FULL_PIN
#define PKV_FULL_PIN 1
#endif
#ifndef PKV_FULL_PREFETCH
#define PKV_FULL_PREFETCH 1
#endif
#ifndef PKV_FULL_DB
#define PKV_FULL_DB 1
#endif
#ifndef PKV_SKIP_DEAD_WAVES
#define PKV_SKIP_DEAD_WAVES 1
#endif
#ifndef PKV_SPLIT_W
#define PKV_SPLIT_W 8
#endif
#ifndef PKV_IDS_AHEAD
#define PKV_IDS_AHEAD 1
#endif
#ifndef PKV_SPLIT_LATE_COMMIT
#define PKV_SPLIT_LATE_COMMIT 1
#endif
#ifndef PKV_JOB_SEARCH_WAVE
#define PKV_JOB_SEARCH_WAVE 1
#endif
#ifndef PKV_SPLIT_STAGGER
#define PKV_SPLIT_STAGGER 1
#endif
#ifndef PKV_SPLIT_QK_ILP
#define PKV_SPLIT_QK_ILP 1
#endif
#ifndef PKV_SPLIT_LOADERS
#define PKV_SPLIT_LOADERS 1
#endif

template <class T, int D, int W, int NT, bool SPLIT, bool APPEND, bool U>
__global__ __launch_bounds__(64 * W, W >= 8 ? 1 : 2) void attn_kernel(AttnArgs a) {
  if (dbg_skip(a.dbg_word)) return;
  using G_ = TileGeom<T, D>;
  constexpr int COLS = W * NT * 16;
  // bf16/FP8 with 4 waves: the next tile's loads are issued between the
  // softmax and the P.V products of the current one (into registers the
  // scores have freed).  With PKV_FULL_DB the K/V tile is double-buffered in
  // LDS: at the start of tile t the staged tile t+1 is written into the buffer
  // tile t-1 used, so one barrier per tile both publishes tile t and frees
  // that buffer (two work groups per CU still fit).  fp32 and the
  // fused-append variant (whose store of the new rows would spill) load each
  // tile when it starts.  Past the item's last tile the rows clamp to
  // jmax - 1, so the extra loads stay in bounds.
  // (the 8-wave split kernel has the registers for it with fused append too)
  constexpr bool kPrefetch = PKV_FULL_PREFETCH && T::EB == 2 && (W == 4 || W == 8) && (!APPEND || (SPLIT && W == 8));
  constexpr bool kDouble = kPrefetch && PKV_FULL_DB;
  // Split kernel (no running fold state, so registers to spare): the staged
  // tile t+1 is written into the idle LDS buffer between the softmax and the
  // P.V products of tile t, right before tile t+2's loads are issued into the
  // same registers, so its loads have a whole tile to land instead of the
  // second half of one.  The buffer is free there: every wave passed the
  // barrier that ended tile t-1, its last reader.
  constexpr bool kLateCommit = kDouble && SPLIT && PKV_SPLIT_LATE_COMMIT;
  constexpr bool kSkipDead = SPLIT && PKV_SKIP_DEAD_WAVES != 0;
  // Split kernel, 8 waves x 16 columns: the odd waves run each tile's P.V
  // one barrier interval late, at the start of the next tile, so that while
  // the even waves read K for Q.K^T the odd ones read V, and their softmaxes
  // fall at different times: the LDS reads of a tile are spread over the
  // interval instead of coming in two bursts from every wave at once.  The
  // tile buffers rotate over three (the tile being computed, the one whose
  // late P.V is still to come, the one being staged).  Each column's
  // operations keep their order (softmax t, P.V t, softmax t+1), so the bits
  // are those of the unstaggered kernel.
  constexpr bool kStagger = kLateCommit && NT == 1 && W == 8 && PKV_SPLIT_STAGGER != 0;
  constexpr int kBufs = kStagger ? 3 : (kDouble ? 2 : 1);
  // Staggered split kernel whose column block leaves the last two waves
  // without a column (at most 16 * (W - 2) columns, e.g. 17 rows x 4 heads):
  // those two waves load and stage every tile in a loop of their own, and the
  // waves with columns issue no tile loads or LDS tile writes -- the staging
  // leaves their per-tile chain.  The same bytes reach the same LDS tiles
  // between the same barriers, so no bit changes.  Not with the fused append
  // (measured slower there: 16.90 -> 17.12 ms on 17-token chunks, where the
  // plain call went 17.14 -> 15.82 ms).
  constexpr bool kLoaders = kStagger && !APPEND && PKV_SPLIT_LOADERS != 0;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kBufs * G_::BYTES];
  unsigned char* k_lds = lds;
  unsigned char* v_lds = lds + G_::KBYTES;

  int b = blockIdx.z;
  int hk = blockIdx.y;
  int cb, item;
  if constexpr (SPLIT) {
    cb = blockIdx.x % a.ncb;
    item = blockIdx.x / a.ncb;
  } else {
#if PKV_ATTN_XCD
    // Work groups are dispatched round-robin over the 8 XCDs; renumber them so
    // one XCD runs consecutive column blocks of the same (sequence, KV head)
    // and its L2 serves the K/V tiles they share (as in prefill_kernel).
    const int nwg = gridDim.x * gridDim.y * gridDim.z;
    const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int full8 = nwg / 8 * 8;
    const int w = lin < full8 ? (lin % 8) * (nwg / 8) + lin / 8 : lin;
    b = w / (gridDim.x * gridDim.y);
    hk = (w / gridDim.x) % gridDim.y;
    cb = a.ncb - 1 - w % gridDim.x;  // heaviest causal blocks first
#else
    cb = a.ncb - 1 - static_cast<int>(blockIdx.x);  // heaviest causal blocks first
#endif
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
    c_begin = a.chunk0 + item * a.cpi;
    c_end = min(min(c_begin + a.cpi, nchunks), a.chunk1);
    if (c_begin >= c_end) {
      if (a.direct && item == 0) {  // no visible key in the block: its rows still get out and lse
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int col = col0 + ((static_cast<int>(threadIdx.x) >> 6) * NT + nt) * 16 + (lane_id() & 15);
          if (col < ncols) write_empty_column<T, D>(a, (int64_t)(q0 + col / g) * a.hq + hk * g + col % g);
        }
      }
      return;
    }
  }

  const Append ap = make_append<APPEND>(n, L, q0, col0 + COLS >= ncols);
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
      const unsigned char* qp = static_cast<const unsigned char*>(a.q) + qelem * T::EB;
#pragma unroll
      for (int k = 0; k < G_::NK; ++k) q[nt].v[k] = *reinterpret_cast<const u32x4*>(qp + qk_piece_off<T>(k, G));
    } else {
#pragma unroll
      for (int k = 0; k < G_::NK; ++k) q[nt].v[k] = u32x4{0, 0, 0, 0};
    }
  }

  // A wave none of whose columns exists (the last column block of a
  // sequence) skips the arithmetic; its lanes still load their share of every
  // tile.  Wave-uniform, so barriers and loads stay the same for all waves.
  const bool live = __builtin_amdgcn_readfirstlane(col0 + wave * NT * 16 < ncols ? 1 : 0) != 0;
  const bool lmode = kLoaders && ncols - col0 <= 16 * (W - 2);   // the same in every wave
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
  // No visible key (only when seqlens_k is below the sequence's row count):
  // nothing is loaded and the columns get out = 0, lse = -inf.
  if (c_begin < c_end) {
    TileStage<T, D, W> stg;
    // block ids of the next tile to issue, fetched one tile ahead (U)
    TileIds ids;
    // (split kernel only: 20.55 against 21.13 ms on the 17-token chunked
    // prefill; the full path, with two work groups per CU hiding the id
    // loads, measured 1.7% slower with it)
    constexpr bool kIds = kPrefetch && U && SPLIT && PKV_IDS_AHEAD;
    const int jb = c_begin * KC;
    if constexpr (kLoaders) {
      if (lmode && wave >= W - 2) {
        // Loader waves: the tile schedule of the waves below (tile jb into
        // buffer 0 first; after the barrier that starts tile t, tile t + 1
        // from the register stage into buffer (t + 1) % 3, then tile t + 2's
        // loads into the stage), each thread with a quarter of the tile.
        const int ltid = static_cast<int>(threadIdx.x) - 64 * (W - 2);
        TileStage<T, D, 2> lstg;
        TileIds lids;
        auto lissue = [&](int j) {
          tile_issue<T, D, 2, APPEND, U, kIds>(a, bt, hk, j, jmax, lstg, ap, lids, ltid);
          if constexpr (kIds) tile_ids_fetch<T, D, 2, U>(a, bt, j + KT, jmax, lids, ltid);
        };
        if constexpr (kIds) tile_ids_fetch<T, D, 2, U>(a, bt, jb, jmax, lids, ltid);
        lissue(jb);
        tile_commit<T, D, 2, APPEND>(a, bt, hk, jb, jmax, lstg, lds, lds + G_::KBYTES, ap, ltid);
        lissue(jb + KT);
        for (int c = c_begin; c < c_end; ++c) {
          const int jend = min((c + 1) * KC, jmax);
          for (int j0 = c * KC; j0 < jend; j0 += KT) {
            __syncthreads();
            unsigned char* const nk = lds + (((j0 - jb) / KT + 1) % 3) * G_::BYTES;
            tile_commit<T, D, 2, APPEND>(a, bt, hk, j0 + KT, jmax, lstg, nk, nk + G_::KBYTES, ap, ltid);
            lissue(j0 + 2 * KT);
          }
        }
        return;  // no column: nothing to write
      }
    }
    auto issue = [&](int j, TileStage<T, D, W>& into) {
      if (kLoaders && lmode) return;  // the loader waves stage the tiles
      tile_issue<T, D, W, APPEND, U, kIds>(a, bt, hk, j, jmax, into, ap, ids);
      if constexpr (kIds) tile_ids_fetch<T, D, W, U>(a, bt, j + KT, jmax, ids);
    };
    if constexpr (kIds) {
      if (!(kLoaders && lmode)) tile_ids_fetch<T, D, W, U>(a, bt, jb, jmax, ids);
    }
    if constexpr (kPrefetch) issue(jb, stg);
    if constexpr (kDouble) {
      // first tile into buffer 0, the second one's loads in flight
      if (!(kLoaders && lmode)) tile_commit<T, D, W, APPEND>(a, bt, hk, jb, jmax, stg, k_lds, v_lds, ap);
      issue(jb + KT, stg);
    }
    ChunkState<D, NT> st;
    // One tile.  `ready`: the register stage holding the next tile to commit,
    // refilled with the tile after it (kPrefetch).
    // kStagger: an odd wave's P.V of its previous tile, still to be done
    const bool late = kStagger && (wave & 1) != 0;
    u32x4 pb_late[NT][KT / 32];
    const unsigned char* v_late = nullptr;
    auto late_pv = [&] {
      if constexpr (kStagger) {
        if (late && v_late != nullptr) {
          pv_part<T, D, NT, PKV_FULL_PIN != 0, U ? 2 : 1>(st, pb_late, v_late);
          v_late = nullptr;
        }
      }
    };
    auto tile = [&](int j0, TileStage<T, D, W>& ready) {
      __syncthreads();
      if constexpr (kStagger) {
        // tile j0 in buffer ((j0 - jb) / KT) % 3 (the first one in buffer 0);
        // tile j0 + KT is staged into the next one
        const int cur = ((j0 - jb) / KT) % 3;
        k_lds = lds + cur * G_::BYTES;
        v_lds = k_lds + G_::KBYTES;
      } else if constexpr (kDouble) {
        // tile j0 is in buffer (j0 / KT) & 1; the other one is free: stage tile j0 + KT there
        const int cur = (j0 / KT) & 1;
        if constexpr (!kLateCommit) {
          unsigned char* const nk = lds + (cur ^ 1) * G_::BYTES;
          tile_commit<T, D, W, APPEND>(a, bt, hk, j0 + KT, jmax, ready, nk, nk + G_::KBYTES, ap);
        }
        k_lds = lds + cur * G_::BYTES;
        v_lds = k_lds + G_::KBYTES;
      } else {
        if constexpr (kPrefetch)
          tile_commit<T, D, W, APPEND>(a, bt, hk, j0, jmax, ready, k_lds, v_lds, ap);
        else
          load_tile<T, D, W, APPEND, U>(a, bt, hk, j0, jmax, k_lds, v_lds, ap);
        __syncthreads();
      }
      const int jn = j0 + (kDouble ? 2 : 1) * KT;
      auto mid = [&] {
        if constexpr (kPrefetch) {
          if constexpr (kLateCommit) {
            unsigned char* const nk = lds + (kStagger ? ((j0 - jb) / KT + 1) % 3 : ((j0 / KT) & 1) ^ 1) * G_::BYTES;
            if (!(kLoaders && lmode)) tile_commit<T, D, W, APPEND>(a, bt, hk, j0 + KT, jmax, ready, nk, nk + G_::KBYTES, ap);
          }
          issue(jn, ready);
        }
      };
      if (kSkipDead && !live) {  // no column of this wave exists: only its share of the tile loads
        mid();
        return;
      }
      late_pv();
      f32x4 s[NT][KT / 16];
      if constexpr (NT == 1 && SPLIT && W == 8 && T::EB == 2 && PKV_SPLIT_QK_ILP) {
        qk_tile_lds_ilp<T, D>(k_lds, q[0], s[0]);  // registers to spare: all K operands, chains interleaved
      } else if constexpr (NT == 1) {
        qk_tile_lds<T, D>(k_lds, q[0], s[0]);  // one M tile of K operands live at a time
      } else {
#if PKV_QK_PER_MT
        qk_tiles_lds<T, D, NT>(k_lds, q, s);   // one M tile of K operands, all column groups
#else
        KOps<T, D> kop;
        k_operands_lds<T, D>(k_lds, kop);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) qk_tile<T, D>(kop, q[nt], s[nt]);
#endif
      }
      if constexpr (kStagger) {
        if (late) {
          softmax_part<T, D, NT>(st, s, lim, j0, a.mul, pb_late);
          mid();
          v_late = v_lds;
          return;
        }
      }
      if constexpr (kPrefetch) {
        // V operands two P.V steps ahead where registers allow (scalar block ids)
        softmax_pv_tile<T, D, NT, PKV_FULL_PIN != 0, true, U ? 2 : 1>(st, s, lim, j0, a.mul, v_lds, mid);
      } else {
        softmax_pv_tile<T, D, NT, PKV_FULL_PIN != 0>(st, s, lim, j0, a.mul, v_lds);
      }
    };
    for (int c = c_begin; c < c_end; ++c) {
      chunk_reset(st);
      const int jend = min((c + 1) * KC, jmax);
      for (int j0 = c * KC; j0 < jend; j0 += KT) tile(j0, stg);
      late_pv();  // the chunk's last P.V (its buffer is not restaged before two more tiles)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float lc = column_sum(st.l[nt]);
        if constexpr (SPLIT) {
          const int col = cols[nt];
          if (col < ncols && a.direct) {
            write_one_chunk<T, D>(a, (int64_t)(q0 + col / g) * a.hq + hk * g + col % g, st.m[nt], lc, st.o[nt]);
          } else if (col < ncols) {
            const int64_t idx = ((int64_t)(q0 + col / g) * a.hq + hk * g + col % g) * a.ps_row + c * a.ps_chunk;
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
  }

  if constexpr (!SPLIT) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int col = cols[nt];
      if (col < ncols) {
        const int64_t rh = (int64_t)(q0 + col / g) * a.hq + hk * g + col % g;
        if (G == 0) a.lse[rh] = final_lse<T>(M[nt], Ls[nt]);
        store_out<T, D>(a.out, rh * D, O[nt], M[nt], Ls[nt], a.v_scale);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Longest-first job list of the one-wave decode kernels.  With one chunk per
// work item the items of a ragged batch differ only in their last chunk, so
// dispatching every full chunk first and the partial last chunks after them
// keeps short items for the end of the grid instead of long ones.  A job is
// identified by (sequence, KV head, chunk) exactly as in the grid mapping, so
// the order changes no bit.
//
// decode_plan_kernel (one work group) writes the exclusive prefix counts, over
// sequences in order, of full chunks F_b = n_b / KC and partial chunks
// P_b = (n_b % KC != 0) of the sequences that have rows (with one column
// block, the last row of a sequence sees all n_b keys).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void decode_plan_kernel(const int32_t* seqlens_k, const int32_t* cu_q, int batch,
                                                           int32_t* pref) {
  __shared__ int32_t sf[1024], sp[1024];
  __shared__ int32_t carry[2];
  const int t = threadIdx.x;
  if (t == 0) carry[0] = carry[1] = 0;
  __syncthreads();
  for (int base = 0; base < batch; base += 1024) {
    const int b = base + t;
    int f = 0, p = 0;
    if (b < batch) {
      const int n = seqlens_k[b];
      const int L = cu_q[b + 1] - cu_q[b];
      if (L > 0 && n > 0) {
        f = n / KC;
        p = (n % KC) != 0;
      }
    }
    sf[t] = f;
    sp[t] = p;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {  // inclusive scan
      const int xf = t >= d ? sf[t - d] : 0;
      const int xp = t >= d ? sp[t - d] : 0;
      __syncthreads();
      sf[t] += xf;
      sp[t] += xp;
      __syncthreads();
    }
    if (b < batch) {
      pref[b] = carry[0] + sf[t] - f;
      pref[batch + 1 + b] = carry[1] + sp[t] - p;
    }
    __syncthreads();
    if (t == 0) {
      carry[0] += sf[1023];
      carry[1] += sp[1023];
    }
    __syncthreads();
  }
  if (t == 0) {
    pref[batch] = carry[0];
    pref[2 * batch + 1] = carry[1];
  }
}

// The (sequence, KV head, chunk) of job x; false past the last job.
__device__ __forceinline__ bool decode_job(const AttnArgs& a, int x, int& b, int& hk, int& c) {
  using cint = const __attribute__((address_space(4))) int32_t;
  cint* pf = (cint*)a.job_pref;
  cint* pp = pf + a.nbatch + 1;
  const int H = a.nhk;
  const int nfull = pf[a.nbatch] * H;
  int m = x;
  cint* pr = pf;
  if (m >= nfull) {
    m -= nfull;
    pr = pp;
    if (m >= pp[a.nbatch] * H) return false;
  }
#if PKV_JOB_SEARCH_WAVE
  // The largest b with H * pr[b] <= m (pr nondecreasing, pr[0] = 0, H *
  // pr[batch] > m) is the count of k in [1, batch] with H * pr[k] <= m: the
  // wave counts 256 entries per round of loads (4 per lane, ballots) instead
  // of one dependent scalar load per halving.
  {
    const int32_t* prv = a.job_pref + (pr == pf ? 0 : a.nbatch + 1);
    const int lane = lane_id();
    int cnt = 0;
    for (int base = 1; base <= a.nbatch; base += 256) {
      int v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = prv[min(base + 4 * lane + i, a.nbatch)];
#pragma unroll
      for (int i = 0; i < 4; ++i) cnt += __popcll(__ballot(base + 4 * lane + i <= a.nbatch && v[i] * H <= m));
    }
    b = cnt;
  }
#else
  int lo = 0, hi = a.nbatch;  // largest b with H * pr[b] <= m (pr[0] = 0, H * pr[batch] > m)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pr[mid] * H <= m) lo = mid; else hi = mid;
  }
  b = lo;
#endif
  const int r = m - pr[b] * H;
  if (pr == pf) {
    const int f = pf[b + 1] - pf[b];  // this sequence's full chunks, per KV head
    hk = r / f;
    c = r - hk * f;
  } else {
    hk = r;
    c = a.seqlens_k[b] / KC;
  }
  return true;
}

// The (sequence, KV head, column block, item) of a one-wave decode work group
// of the plain grid (x: column block and item, y: KV head, z: sequence), in
// one of two dispatch orders (work groups go round-robin over the 8 XCDs):
//   0  consecutive work groups run consecutive items of one (sequence, KV
//      head) -- the faster order for grids of many rounds of wave slots (16 x
//      131072 keys: 1.541 against 1.582 ms with order 1)
//   1  the sequence fastest, then the item, then the KV head -- faster for
//      grids of one or two rounds (64 x 4096 keys: 0.1058 against 0.1133 ms)
// Orders that put the KV heads of one chunk next to each other, or on one
// XCD, measured 4-16% slower on both.  Same (sequence, head, item) jobs in
// every order, so the order changes no bit.
__device__ __forceinline__ void decode_item(const AttnArgs& a, int& b, int& hk, int& cb, int& item) {
  int x = blockIdx.x;
  b = blockIdx.z;
  hk = blockIdx.y;
  if (a.dorder == 1) {
    const int X = gridDim.x, B = gridDim.z;
    const int lin = blockIdx.x + X * (blockIdx.y + gridDim.y * blockIdx.z);
    b = lin % B;
    x = (lin / B) % X;
    hk = lin / (B * X);
  }
  cb = x % a.ncb;
  item = x / a.ncb;
}

// ---------------------------------------------------------------------------
// Decode split kernel: one wave per work item (sequence, KV head, 16 columns,
// run of chunks), for up to 16 query columns per KV head (g * L <= 16).
//
// Data movement only differs from attn_kernel: each lane loads the K and V
// pieces it feeds to the MFMAs straight into registers (K row 16mt + l%16,
// bytes 64k + 16G), one tile ahead of the tile being computed, with the block
// ids one tile further ahead, so a wave keeps ~32 KiB of HBM reads in flight
// while it computes.  K goes from registers into the QK MFMAs; V goes through
// a private LDS tile for the transposing read.  The arithmetic is the shared
// chunk core, so the bits equal those of the prefill kernel.
// ---------------------------------------------------------------------------
template <class T, int D>
struct TileRegs {
  using Raw = typename KvRaw<T>::type;  // stored bytes; widened where they are used
  Raw k[KT / 16][TileGeom<T, D>::NK];
  Raw v[KT / 16][TileGeom<T, D>::NK];
};

// QK^T of a tile whose K operands are held as stored bytes: the qk_tile chain,
// each operand widened just before its MFMA.
template <class T, int D>
__device__ __forceinline__ void qk_tile_regs(const TileRegs<T, D>& r, const QOps<T, D>& q, f32x4 (&s)[KT / 16]) {
  using G_ = TileGeom<T, D>;
#pragma unroll
  for (int mt = 0; mt < G_::MT; ++mt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < G_::NK; ++k) {
      const u32x4 kw = kv_widen<T>(r.k[mt][k]);
      if constexpr (T::EB == 2) {
        acc = mfma_bf16(kw, q.v[k], acc);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = mfma_f32(__uint_as_float(kw[e]), __uint_as_float(q.v[k][e]), acc);
      }
    }
    s[mt] = acc;
  }
}

// Block ids of this lane's four tile rows (rows past jlast use the last
// visible row's block, so every read stays inside the sequence's blocks).
// U (block size a multiple of 16): the 16 rows of an M tile lie in one cache
// block, so its id is wave-uniform and comes from a scalar load -- scalar
// loads are not counted with the vector loads, so using the ids never makes
// the wave wait for K/V loads issued before them.
template <bool U>
__device__ __forceinline__ void tile_block_ids(const AttnArgs& a, const int32_t* bt, int j0, int jlast,
                                               int (&ids)[KT / 16]) {
  if constexpr (U) {
    using cint = const __attribute__((address_space(4))) int32_t;
    cint* cbt = (cint*)bt;  // the table is not written while a kernel runs
#pragma unroll
    for (int mt = 0; mt < KT / 16; ++mt) ids[mt] = cbt[div_block(min(j0 + 16 * mt, jlast - 1), a.bs_mul, a.bs_shift)];
  } else {
    const int r = lane_id() & 15;
#pragma unroll
    for (int mt = 0; mt < KT / 16; ++mt) {
      const int j = min(j0 + 16 * mt + r, jlast - 1);
      ids[mt] = bt[div_block(j, a.bs_mul, a.bs_shift)];
    }
  }
}

template <class T, int D, bool APPEND, bool U>
__device__ __forceinline__ void tile_load_regs(const AttnArgs& a, int hk, int j0, int jlast, const int (&ids)[KT / 16],
                                               TileRegs<T, D>& r, bool want_k, bool want_v, const Append& ap) {
  using G_ = TileGeom<T, D>;
  const int lane = lane_id();
  const unsigned char* kb = static_cast<const unsigned char*>(a.k);
  const unsigned char* vb = static_cast<const unsigned char*>(a.v);
#pragma unroll
  for (int mt = 0; mt < G_::MT; ++mt) {
    // rows past jlast load a visible row; tile_edge zeroes them before use
    const int jc = min(j0 + 16 * mt + (lane & 15), jlast - 1);
    const int64_t blk = ids[mt];
    const int slot = jc - div_block(jc, a.bs_mul, a.bs_shift) * a.bs;
    constexpr int P = kKvPiece<T>;  // stored bytes per 16-byte operand piece
    const int off = P * (lane >> 4);
    const unsigned char* kp;
    const unsigned char* vp;
    if constexpr (U) {
      // wave-uniform block base (scalar registers) + 32-bit per-lane offset
      const unsigned char* kbase = kb + (blk * a.kbs + (int64_t)hk * a.khs) * T::KVB;
      const unsigned char* vbase = vb + (blk * a.vbs + (int64_t)hk * a.vhs) * T::KVB;
      kp = kbase + static_cast<uint32_t>(slot * static_cast<int>(a.kss) * T::KVB + off);
      vp = vbase + static_cast<uint32_t>(slot * static_cast<int>(a.vss) * T::KVB + off);
    } else {
      kp = kb + (blk * a.kbs + (int64_t)slot * a.kss + (int64_t)hk * a.khs) * T::KVB + off;
      vp = vb + (blk * a.vbs + (int64_t)slot * a.vss + (int64_t)hk * a.vhs) * T::KVB + off;
    }
    const int nhk = a.hq / a.g;
    const unsigned char* ks = kv_src<T, D, APPEND>(a.k_new, nhk, hk, jc, ap, kp, off);
    const unsigned char* vs = kv_src<T, D, APPEND>(a.v_new, nhk, hk, jc, ap, vp, off);
    if constexpr (T::KVB == 1) {
      // FP8: pieces k = 2j and 2j+1 of this lane are 16 contiguous stored bytes
      // at 64j + 16G (the FP8 k-slot map of qk_piece_off).
      const unsigned char* ks2 = ks - off + 16 * (lane >> 4);
      const unsigned char* vs2 = vs - off + 16 * (lane >> 4);
#pragma unroll
      for (int j = 0; j < G_::NK / 2; ++j) {
        if (want_k) {
          const u32x4 x = *reinterpret_cast<const u32x4*>(ks2 + 64 * j);
          r.k[mt][2 * j] = u32x2{x[0], x[1]};
          r.k[mt][2 * j + 1] = u32x2{x[2], x[3]};
        }
        if (want_v) {
          const u32x4 x = *reinterpret_cast<const u32x4*>(vs2 + 64 * j);
          r.v[mt][2 * j] = u32x2{x[0], x[1]};
          r.v[mt][2 * j + 1] = u32x2{x[2], x[3]};
        }
      }
      continue;
    }
#pragma unroll
    for (int k = 0; k < G_::NK; ++k) {
      if (want_k) r.k[mt][k] = kv_load_raw<T>(ks + 4 * P * k);
      if (want_v) r.v[mt][k] = kv_load_raw<T>(vs + 4 * P * k);
    }
  }
}

// Rows past jlast hold a copy of row jlast - 1 (tile_load_regs clamps them);
// zero them when the tile is about to be used rather than when its loads are
// issued: a select on a loaded register makes the wave wait for that load.
// Only the last tile of an item can reach past jlast (a wave-uniform test).
template <class T, int D>
__device__ __forceinline__ void tile_edge(int j0, int jlast, TileRegs<T, D>& r) {
  using G_ = TileGeom<T, D>;
  using Raw = typename KvRaw<T>::type;
  if (j0 + KT > jlast) {
    const int lane = lane_id();
#pragma unroll
    for (int mt = 0; mt < G_::MT; ++mt) {
      const bool in = j0 + 16 * mt + (lane & 15) < jlast;
#pragma unroll
      for (int k = 0; k < G_::NK; ++k) {
        r.k[mt][k] = in ? r.k[mt][k] : Raw{};
        r.v[mt][k] = in ? r.v[mt][k] : Raw{};
      }
    }
  }
}

// Fused append in the split kernels: the writer copies this call's new rows
// in [lo, hi) (positions >= n_old) of KV head hk from k_new / v_new into
// their cache slots once, before its tile loop.  Every read of those rows in
// this call goes to k_new / v_new (kv_src), so the copy's position in the
// kernel does not matter, and the tile loop carries no stores.
template <class T, int D>
__device__ __forceinline__ void append_rows(const AttnArgs& a, const int32_t* bt, int hk, int lo, int hi,
                                            const Append& ap) {
  constexpr int PR = D * T::KVB / 16;  // 16-byte pieces per stored row
  const int nhk = a.hq / a.g;
  for (int i = lane_id(); i < (hi - lo) * PR; i += 64) {
    const int j = lo + i / PR;
    const int p = i % PR;
    const int bi = div_block(j, a.bs_mul, a.bs_shift);
    const int64_t blk = bt[bi];
    const int64_t slot = j - bi * a.bs;
    const int64_t nrow = (ap.row0 + (j - ap.n_old)) * nhk + hk;
    const u32x4 kx = *reinterpret_cast<const u32x4*>(static_cast<const unsigned char*>(a.k_new) + nrow * D * T::KVB + 16 * p);
    const u32x4 vx = *reinterpret_cast<const u32x4*>(static_cast<const unsigned char*>(a.v_new) + nrow * D * T::KVB + 16 * p);
    *reinterpret_cast<u32x4*>(static_cast<unsigned char*>(a.k_store) +
                              (blk * a.kbs + slot * a.kss + (int64_t)hk * a.khs) * T::KVB + 16 * p) = kx;
    *reinterpret_cast<u32x4*>(static_cast<unsigned char*>(a.v_store) +
                              (blk * a.vbs + slot * a.vss + (int64_t)hk * a.vhs) * T::KVB + 16 * p) = vx;
  }
}

template <class T, int D>
__device__ __forceinline__ void tile_store_v(unsigned char* v_lds, const TileRegs<T, D>& r) {
  using G_ = TileGeom<T, D>;
  const int lane = lane_id();
  unsigned char* base = v_lds + (lane & 15) * G_::VPITCH;
#pragma unroll
  for (int mt = 0; mt < G_::MT; ++mt)
#pragma unroll
    for (int k = 0; k < G_::NK; ++k)
      *reinterpret_cast<u32x4*>(base + mt * 16 * G_::VPITCH + qk_piece_off<T>(k, lane >> 4)) = kv_widen<T>(r.v[mt][k]);
}

#ifndef PKV_PF_XCD
#define PKV_PF_XCD 1
#endif
// ---------------------------------------------------------------------------
// Prefill kernel: one work group of W waves per (sequence, KV head, W*16
// columns); every wave owns 16 columns (one MFMA N tile) and runs the chunk
// core over all chunks in ascending order, folding each chunk result into its
// row state in registers, then writes out/lse.  K/V tiles are staged in LDS
// by all W*64 threads and shared by the W waves (one HBM read serves the
// whole GQA group); the LDS tiles are double-buffered and the next tile's
// global loads are issued before the current tile is computed.
// ---------------------------------------------------------------------------
template <class T, int D, int W>
struct PrefillStage {
  static constexpr int NCH = KT * TileGeom<T, D>::CPR;  // 16-byte pieces per tensor per tile
  static constexpr int PER = NCH / (64 * W);
  typename KvRaw<T>::type k[PER];  // stored bytes, widened when written to LDS
  typename KvRaw<T>::type v[PER];
};

template <class T, int D, int W, bool APPEND>
__device__ __forceinline__ void prefill_load(const AttnArgs& a, const int32_t* bt, int hk, int j0, int jmax,
                                             PrefillStage<T, D, W>& r, const Append& ap) {
  using G_ = TileGeom<T, D>;
  using S_ = PrefillStage<T, D, W>;
  static_assert(S_::PER * 64 * W == S_::NCH, "tile pieces must split evenly over the work group");
  const unsigned char* kb = static_cast<const unsigned char*>(a.k);
  const unsigned char* vb = static_cast<const unsigned char*>(a.v);
#pragma unroll
  for (int i = 0; i < S_::PER; ++i) {
    const int qi = threadIdx.x + i * 64 * W;
    const int row = qi / G_::CPR, part = qi % G_::CPR;
    const int j = j0 + row;
    const int jc = min(j, jmax - 1);  // rows past jmax load a visible row, then read as zero
    const int bi = div_block(jc, a.bs_mul, a.bs_shift);
    const int64_t blk = bt[bi];
    const int64_t slot = jc - bi * a.bs;
    const int off = kKvPiece<T> * part;
    const unsigned char* kc = kb + (blk * a.kbs + slot * a.kss + (int64_t)hk * a.khs) * T::KVB + off;
    const unsigned char* vc = vb + (blk * a.vbs + slot * a.vss + (int64_t)hk * a.vhs) * T::KVB + off;
    const int nhk = a.hq / a.g;
    const auto kv = kv_load_raw<T>(kv_src<T, D, APPEND>(a.k_new, nhk, hk, jc, ap, kc, off));
    const auto vv = kv_load_raw<T>(kv_src<T, D, APPEND>(a.v_new, nhk, hk, jc, ap, vc, off));
    const bool in = j < jmax;
    kv_store_new<T, APPEND>(ap, in, jc, a.k_store, a.k, kc, kv);
    kv_store_new<T, APPEND>(ap, in, jc, a.v_store, a.v, vc, vv);
    r.k[i] = in ? kv : typename KvRaw<T>::type{};
    r.v[i] = in ? vv : typename KvRaw<T>::type{};
  }
}

template <class T, int D, int W>
__device__ __forceinline__ void prefill_store(unsigned char* k_lds, unsigned char* v_lds, const PrefillStage<T, D, W>& r) {
  using G_ = TileGeom<T, D>;
  using S_ = PrefillStage<T, D, W>;
#pragma unroll
  for (int i = 0; i < S_::PER; ++i) {
    const int qi = threadIdx.x + i * 64 * W;
    const int row = qi / G_::CPR, part = qi % G_::CPR;
    *reinterpret_cast<u32x4*>(k_lds + row * G_::KPITCH + 16 * part) = kv_widen<T>(r.k[i]);
    *reinterpret_cast<u32x4*>(v_lds + row * G_::VPITCH + 16 * part) = kv_widen<T>(r.v[i]);
  }
}

// One prefill tile: `cur` is refilled with tile t+2 while tile t is computed
// from LDS buffer t&1; `nxt` (tile t+1) goes to LDS buffer (t+1)&1 afterwards.
template <class T, int D, int W, bool APPEND>
__device__ __forceinline__ void prefill_tile(const AttnArgs& a, const int32_t* bt, int hk, int t, int ntiles, int jmax,
                                             unsigned char* lds, PrefillStage<T, D, W>& cur,
                                             PrefillStage<T, D, W>& nxt, const QOps<T, D>& q, const int (&lim)[1],
                                             ChunkState<D, 1>& st, float& M, float& Ls, f32x4 (&O)[D / 16],
                                             const Append& ap) {
  using G_ = TileGeom<T, D>;
  const int j0 = t * KT;
  if (t + 2 < ntiles) prefill_load<T, D, W, APPEND>(a, bt, hk, j0 + 2 * KT, jmax, cur, ap);
  const unsigned char* k_lds = lds + (t & 1) * G_::BYTES;
  f32x4 s[1][KT / 16];
  qk_tile_lds<T, D>(k_lds, q, s[0]);
  softmax_pv_tile<T, D, 1, true>(st, s, lim, j0, a.mul, k_lds + G_::KBYTES);
  // chunk end: fold the chunk result into the row state
  if ((j0 + KT) % KC == 0 || t + 1 == ntiles) {
    const float lc = column_sum(st.l[0]);
    if (st.m[0] != -INFINITY) {
      const FoldCoef<T> f = fold_coef<T>(M, st.m[0]);
      Ls = fold_val(Ls, f.a, lc, f.b);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[dt][i] = fold_val(O[dt][i], f.a, st.o[0][dt][i], f.b);
      M = f.mn;
    }
    chunk_reset(st);
  }
  if (t + 1 < ntiles) {
    unsigned char* nb = lds + ((t + 1) & 1) * G_::BYTES;
    prefill_store<T, D, W>(nb, nb + G_::KBYTES, nxt);
  }
  __syncthreads();
}

template <class T, int D, int W, bool APPEND>
__global__ __launch_bounds__(64 * W, 2) void prefill_kernel(AttnArgs a) {
  if (dbg_skip(a.dbg_word)) return;
  using G_ = TileGeom<T, D>;
  constexpr int COLS = W * 16;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * G_::BYTES];  // 2 x (K, V)

#if PKV_PF_XCD
  // Work groups are dispatched round-robin over the 8 XCDs (each with its own
  // L2); renumber them so that one XCD runs consecutive column blocks of the
  // same (sequence, KV head) and its L2 serves their shared K/V tiles.
  const int nwg = gridDim.x * gridDim.y * gridDim.z;
  const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int full8 = nwg / 8 * 8;
  const int w = lin < full8 ? (lin % 8) * (nwg / 8) + lin / 8 : lin;
  const int b = w / (gridDim.x * gridDim.y);
  const int hk = (w / gridDim.x) % gridDim.y;
  const int cb = a.ncb - 1 - w % gridDim.x;  // heaviest causal blocks first
#else
  const int b = blockIdx.z;
  const int hk = blockIdx.y;
  const int cb = a.ncb - 1 - static_cast<int>(blockIdx.x);  // heaviest causal blocks first
#endif
  const int n = a.seqlens_k[b];
  const int q0 = a.cu_q[b];
  const int L = a.cu_q[b + 1] - q0;
  const int g = a.g;
  const int ncols = L * g;
  const int col0 = cb * COLS;
  if (col0 >= ncols) return;
  const int last_col = min(col0 + COLS, ncols) - 1;
  const int jmax = column_limit(last_col, ncols, g, n, L, a.causal);
  const int ntiles = jmax > 0 ? (jmax + KT - 1) / KT : 0;
  const Append ap = make_append<APPEND>(n, L, q0, col0 + COLS >= ncols);

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int G = lane >> 4;
  const int col = col0 + wave * 16 + (lane & 15);
  const int lim[1] = {column_limit(col, ncols, g, n, L, a.causal)};
  QOps<T, D> q;
  if (col < ncols) {
    const int64_t qelem = ((int64_t)(q0 + col / g) * a.hq + hk * g + col % g) * D;
    const unsigned char* qp = static_cast<const unsigned char*>(a.q) + qelem * T::EB;
#pragma unroll
    for (int k = 0; k < G_::NK; ++k) q.v[k] = *reinterpret_cast<const u32x4*>(qp + qk_piece_off<T>(k, G));
  } else {
#pragma unroll
    for (int k = 0; k < G_::NK; ++k) q.v[k] = u32x4{0, 0, 0, 0};
  }

  float M = -INFINITY, Ls = 0.f;
  f32x4 O[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t* bt = a.block_table + (int64_t)b * a.mbps;
  // Tile t is computed from LDS buffer t&1 while one register stage holds tile
  // t+1 (loaded during tile t-1) and the other receives tile t+2.
  PrefillStage<T, D, W> sa, sb;
  if (ntiles > 0) {
    prefill_load<T, D, W, APPEND>(a, bt, hk, 0, jmax, sa, ap);
    if (ntiles > 1) prefill_load<T, D, W, APPEND>(a, bt, hk, KT, jmax, sb, ap);
    prefill_store<T, D, W>(lds, lds + G_::KBYTES, sa);
  }
  __syncthreads();
  ChunkState<D, 1> st;
  chunk_reset(st);
  for (int t = 0; t < ntiles; ++t) {
    if ((t & 1) == 0) {
      prefill_tile<T, D, W, APPEND>(a, bt, hk, t, ntiles, jmax, lds, sa, sb, q, lim, st, M, Ls, O, ap);
    } else {
      prefill_tile<T, D, W, APPEND>(a, bt, hk, t, ntiles, jmax, lds, sb, sa, q, lim, st, M, Ls, O, ap);
    }
  }

  if (col < ncols) {
    const int64_t rh = (int64_t)(q0 + col / g) * a.hq + hk * g + col % g;
    if (G == 0) a.lse[rh] = final_lse<T>(M, Ls);
    store_out<T, D>(a.out, rh * D, O, M, Ls, a.v_scale);
  }
}

// Two waves per SIMD (<= 256 registers): 8 waves per CU, each with one tile
// (32 KiB at d = 128) of K/V loads in flight while it computes the previous one.
//
// NW > 1: the work group is one (sequence, KV head, column block) and wave w
// computes chunk w (sequences of at most NW chunks).  The waves leave their
// chunk results (m, l, o of 16 columns) in LDS instead of HBM, and after one
// barrier the work group folds them in ascending chunk order and writes out /
// lse: the merge's operations on the same values (chunks past a column's own
// limit hold m = -inf and are skipped, as the merge never reaches them), so
// the same bits, without the partials' HBM round trip or the merge launch.
// Used with NW = 2: one round of 2-chunk decode, 64 x 2048 keys (Hq 16 / Hkv
// 4) 0.0593 -> 0.0564 ms, 32 x 2048 (32 / 8) 0.0592 -> 0.0562.  With 4 chunks
// per group the 64 x 4096 shard went 0.1003 -> 0.1056 ms (the one-wave kernels'
// order puts the 4 KV heads of one chunk on one CU, reading the same DRAM rows
// together; a group holds one KV head's chunks instead), and with 8 (16 x 8192,
// Hq 64 / Hkv 8: 128 groups) half the CUs idled, 0.1051 -> 0.1358 ms.
template <class T, int D, bool APPEND, bool U, int NW = 1>
__global__ __launch_bounds__(64 * NW, NW == 1 ? 2 : 1) void decode_kernel(AttnArgs a) {
  if (dbg_skip(a.dbg_word)) return;
  using G_ = TileGeom<T, D>;
  static_assert(NW == 1 || !APPEND, "the in-group fold is not combined with the fused append");
  static_assert(NW == 1 || 16 * (D + 2) * 4 <= G_::VBYTES, "a wave's chunk result fits its V area");
  __shared__ __attribute__((aligned(16))) unsigned char lds[NW * G_::VBYTES];
  // the wave index is the same in every lane: say so, so that the chunk range,
  // the loop bounds and the block ids derived from it stay scalar
  const int wave_u = NW == 1 ? 0 : __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  unsigned char* const v_lds = lds + wave_u * G_::VBYTES;

  // Consecutive work groups take consecutive chunks of one (sequence, KV
  // head): concurrently running waves then read different cache blocks
  // (ordering the KV heads of one chunk next to each other measured ~9%
  // slower on the long-context workload).
  int b, hk, cb, item;
  if constexpr (NW > 1) {
    cb = blockIdx.x;
    hk = blockIdx.y;
    b = blockIdx.z;
    item = wave_u;
  } else {
    decode_item(a, b, hk, cb, item);
    if (a.job_pref) {  // longest-first job list (one column block, one chunk per item)
      cb = 0;
      if (!decode_job(a, blockIdx.x, b, hk, item)) return;
    }
  }
  const int n = a.seqlens_k[b];
  const int q0 = a.cu_q[b];
  const int L = a.cu_q[b + 1] - q0;
  const int g = a.g;
  const int ncols = L * g;
  const int col0 = cb * 16;
  if (col0 >= ncols) return;
  const int last_col = min(col0 + 16, ncols) - 1;
  const int jmax = column_limit(last_col, ncols, g, n, L, a.causal);
  const int nchunks = jmax > 0 ? (jmax + KC - 1) / KC : 0;
  const int c_begin = a.chunk0 + item * a.cpi;
  const int c_end = min(min(c_begin + a.cpi, nchunks), a.chunk1);
  const bool has = c_begin < c_end;  // NW > 1: a wave past the sequence's last chunk only joins the fold
  if (!has) {
    if constexpr (NW == 1) {
      if (a.direct && item == 0) {  // no visible key in the block: its rows still get out and lse
        const int col = col0 + (lane_id() & 15);
        if (col < ncols) write_empty_column<T, D>(a, (int64_t)(q0 + col / g) * a.hq + hk * g + col % g);
      }
      return;
    }
  }
  if (has) {
    const int jlast = min(c_end * KC, jmax);   // keys this item reads: [c_begin*KC, jlast)
    const Append ap = make_append<APPEND>(n, L, q0, col0 + 16 >= ncols);

    const int lane = lane_id();
    const int G = lane >> 4;
    const int col = col0 + (lane & 15);
    const int lim[1] = {column_limit(col, ncols, g, n, L, a.causal)};
    QOps<T, D> q;
    if (col < ncols) {
      const int64_t qelem = ((int64_t)(q0 + col / g) * a.hq + hk * g + col % g) * D;
      const unsigned char* qp = static_cast<const unsigned char*>(a.q) + qelem * T::EB;
  #pragma unroll
      for (int k = 0; k < G_::NK; ++k) q.v[k] = *reinterpret_cast<const u32x4*>(qp + qk_piece_off<T>(k, G));
    } else {
  #pragma unroll
      for (int k = 0; k < G_::NK; ++k) q.v[k] = u32x4{0, 0, 0, 0};
    }

    const int32_t* bt = a.block_table + (int64_t)b * a.mbps;
    if constexpr (APPEND) {
      if (ap.writer) append_rows<T, D>(a, bt, hk, max(ap.n_old, c_begin * KC), jlast, ap);
    }
    int j0 = c_begin * KC;
    int ids[KT / 16];
    TileRegs<T, D> r;
    tile_block_ids<U>(a, bt, j0, jlast, ids);
    // V then K, the order the loop issues them in (see below)
    tile_load_regs<T, D, APPEND, U>(a, hk, j0, jlast, ids, r, false, true, ap);
    __builtin_amdgcn_sched_barrier(0);
    tile_load_regs<T, D, APPEND, U>(a, hk, j0, jlast, ids, r, true, false, ap);
    tile_block_ids<U>(a, bt, j0 + KT, jlast, ids);
    __builtin_amdgcn_sched_barrier(0);

    // Per tile: copy V(t) to LDS and refill those registers with V(t+1); QK on
    // K(t) and refill with K(t+1); then softmax + PV(t) while t+1 is in flight.
    ChunkState<D, 1> st;
    for (int c = c_begin; c < c_end; ++c) {
      chunk_reset(st);
      const int jend = min((c + 1) * KC, jmax);
      for (; j0 < jend; j0 += KT) {
        // The next tile's loads are issued unconditionally: past the item's
        // last key every row clamps to row jlast - 1 (a cache hit), and a load
        // under a branch would make the compiler wait for all loads in flight
        // where the branch rejoins.
        const int jn = j0 + KT;
        tile_edge<T, D>(j0, jlast, r);
        tile_store_v<T, D>(v_lds, r);
        tile_load_regs<T, D, APPEND, U>(a, hk, jn, jlast, ids, r, false, true, ap);
        // Loads complete in issue order: keep all of V(t+1) ahead of K(t+1), so
        // waiting for V(t+1) at the next tile leaves K(t+1) in flight.
        __builtin_amdgcn_sched_barrier(0);
        f32x4 s[1][KT / 16];
        qk_tile_regs<T, D>(r, q, s[0]);
        tile_load_regs<T, D, APPEND, U>(a, hk, jn, jlast, ids, r, true, false, ap);
        tile_block_ids<U>(a, bt, jn + KT, jlast, ids);
        __builtin_amdgcn_sched_barrier(0);
        softmax_pv_tile<T, D, 1, true, false>(st, s, lim, j0, a.mul, v_lds);
      }
      const float lc = column_sum(st.l[0]);
      if constexpr (NW > 1) {  // this wave's chunk result into its V area, for the fold below
        float* pc = reinterpret_cast<float*>(v_lds) + (lane & 15) * (D + 2);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<f32x4*>(pc + 16 * dt + 4 * G) = st.o[0][dt];
        if (G == 0) {
          pc[D] = st.m[0];
          pc[D + 1] = lc;
        }
      } else if (col < ncols && a.direct) {
        write_one_chunk<T, D>(a, (int64_t)(q0 + col / g) * a.hq + hk * g + col % g, st.m[0], lc, st.o[0]);
      } else if (col < ncols) {
        const int64_t idx = ((int64_t)(q0 + col / g) * a.hq + hk * g + col % g) * a.ps_row + c * a.ps_chunk;
        if (G == 0) {
          a.part_ml[2 * idx] = st.m[0];
          a.part_ml[2 * idx + 1] = lc;
        }
        float* po = a.part_o + idx * D;
  #pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<f32x4*>(po + 16 * dt + 4 * G) = st.o[0][dt];
      }
    }
  }
  if constexpr (NW > 1) {
    // every wave's chunk result is in LDS (16 columns x (d values, m, l)); fold
    // them per column in ascending chunk order, each thread D / TPC elements
    __syncthreads();
    constexpr int TPC = 64 * NW / 16;  // threads per column
    constexpr int EPT = D / TPC;       // head-dim elements per thread
    static_assert(EPT * TPC == D, "columns split evenly over the work group");
    const int t = threadIdx.x;
    const int cl = t / TPC, e0 = (t % TPC) * EPT;
    float M = -INFINITY, Ls = 0.f;
    float O[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) O[e] = 0.f;
    for (int c = 0; c < min(nchunks, NW); ++c) {
      const float* pc = reinterpret_cast<const float*>(lds + c * G_::VBYTES) + cl * (D + 2);
      const float mc = pc[D];
      if (mc == -INFINITY) continue;
      const FoldCoef<T> f = fold_coef<T>(M, mc);
      Ls = fold_val(Ls, f.a, pc[D + 1], f.b);
#pragma unroll
      for (int e = 0; e < EPT; ++e) O[e] = fold_val(O[e], f.a, pc[e0 + e], f.b);
      M = f.mn;
    }
    const int col = col0 + cl;
    if (col < ncols) {
      const int64_t rh = (int64_t)(q0 + col / g) * a.hq + hk * g + col % g;
      if (t % TPC == 0) a.lse[rh] = final_lse<T>(M, Ls);
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const float v = final_val(M, O[e], Ls, a.v_scale);
        if constexpr (T::EB == 2)
          static_cast<uint16_t*>(a.out)[rh * D + e0 + e] = static_cast<uint16_t>(bf16_rne_bits(v));
        else
          static_cast<float*>(a.out)[rh * D + e0 + e] = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decode split kernel for FP8 caches: stored tiles are half the bytes, so two
// tiles are kept in flight (register stages ra, rb: tile t is computed from
// one while the other holds tile t+1, and the consumed one is refilled with
// tile t+2) -- the same 32 KiB of HBM reads per wave as the bf16 kernel with
// one tile ahead.  Same chunk core and partial writes as decode_kernel.
// ---------------------------------------------------------------------------
template <class T, int D, bool APPEND, bool U>
__device__ __forceinline__ void decode2_tile(const AttnArgs& a, const int32_t* bt, int hk, int t, int t_end, int jlast,
                                             int (&ids)[KT / 16], TileRegs<T, D>& r, unsigned char* v_lds,
                                             const QOps<T, D>& q, const int (&lim)[1], ChunkState<D, 1>& st,
                                             const Append& ap, bool col_ok, int64_t part_row) {
  constexpr int TPC = KC / KT;  // tiles per chunk
  const int j0 = t * KT;
  // Tile t exists unless it is the odd tile after the item's last one; the
  // loads below are issued either way, so every pass through the loop issues
  // the same loads in the same order and the waits for a stage's tile never
  // include the other stage's loads.
  const bool valid = t < t_end;
  f32x4 s[1][KT / 16];
  if (valid) {
    tile_edge<T, D>(j0, jlast, r);
    tile_store_v<T, D>(v_lds, r);
    qk_tile_regs<T, D>(r, q, s[0]);
  }
  // past jlast the rows clamp to jlast - 1 (a cache hit); ids (this register
  // stage's own) then move on to tile t+4
  tile_load_regs<T, D, APPEND, U>(a, hk, j0 + 2 * KT, jlast, ids, r, true, true, ap);
  tile_block_ids<U>(a, bt, j0 + 4 * KT, jlast, ids);
  if (!valid) return;
  softmax_pv_tile<T, D, 1, true, false>(st, s, lim, j0, a.mul, v_lds);
  if ((t + 1) % TPC == 0 || t + 1 == t_end) {
    const float lc = column_sum(st.l[0]);
    if (col_ok && a.direct) {
      write_one_chunk<T, D>(a, part_row, st.m[0], lc, st.o[0]);
    } else if (col_ok) {
      const int64_t idx = part_row * a.ps_row + static_cast<int64_t>(t / TPC) * a.ps_chunk;
      if ((lane_id() >> 4) == 0) {
        a.part_ml[2 * idx] = st.m[0];
        a.part_ml[2 * idx + 1] = lc;
      }
      float* po = a.part_o + idx * D;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<f32x4*>(po + 16 * dt + 4 * (lane_id() >> 4)) = st.o[0][dt];
    }
    chunk_reset(st);
  }
}

template <class T, int D, bool APPEND, bool U>
__global__ __launch_bounds__(64, T::KVB == 1 ? 2 : 1) void decode2_kernel(AttnArgs a) {
  if (dbg_skip(a.dbg_word)) return;
  using G_ = TileGeom<T, D>;
  __shared__ __attribute__((aligned(16))) unsigned char v_lds[G_::VBYTES];

  int b, hk, cb, item;
  decode_item(a, b, hk, cb, item);
  if (a.job_pref) {  // longest-first job list (one column block, one chunk per item)
    cb = 0;
    if (!decode_job(a, blockIdx.x, b, hk, item)) return;
  }
  const int n = a.seqlens_k[b];
  const int q0 = a.cu_q[b];
  const int L = a.cu_q[b + 1] - q0;
  const int g = a.g;
  const int ncols = L * g;
  const int col0 = cb * 16;
  if (col0 >= ncols) return;
  const int last_col = min(col0 + 16, ncols) - 1;
  const int jmax = column_limit(last_col, ncols, g, n, L, a.causal);
  const int nchunks = jmax > 0 ? (jmax + KC - 1) / KC : 0;
  const int c_begin = a.chunk0 + item * a.cpi;
  const int c_end = min(min(c_begin + a.cpi, nchunks), a.chunk1);
  if (c_begin >= c_end) {
    if (a.direct && item == 0) {  // no visible key in the block: its rows still get out and lse
      const int col = col0 + (lane_id() & 15);
      if (col < ncols) write_empty_column<T, D>(a, (int64_t)(q0 + col / g) * a.hq + hk * g + col % g);
    }
    return;
  }
  const int jlast = min(c_end * KC, jmax);   // keys this item reads: [c_begin*KC, jlast)
  const Append ap = make_append<APPEND>(n, L, q0, col0 + 16 >= ncols);

  const int lane = lane_id();
  const int G = lane >> 4;
  const int col = col0 + (lane & 15);
  const int lim[1] = {column_limit(col, ncols, g, n, L, a.causal)};
  QOps<T, D> q;
  if (col < ncols) {
    const int64_t qelem = ((int64_t)(q0 + col / g) * a.hq + hk * g + col % g) * D;
    const unsigned char* qp = static_cast<const unsigned char*>(a.q) + qelem * T::EB;
#pragma unroll
    for (int k = 0; k < G_::NK; ++k) q.v[k] = *reinterpret_cast<const u32x4*>(qp + qk_piece_off<T>(k, G));
  } else {
#pragma unroll
    for (int k = 0; k < G_::NK; ++k) q.v[k] = u32x4{0, 0, 0, 0};
  }
  const int64_t part_row = (int64_t)(q0 + col / g) * a.hq + hk * g + col % g;

  const int32_t* bt = a.block_table + (int64_t)b * a.mbps;
  if constexpr (APPEND) {
    if (ap.writer) append_rows<T, D>(a, bt, hk, max(ap.n_old, c_begin * KC), jlast, ap);
  }
  const int t_begin = c_begin * (KC / KT);
  const int t_end = (jlast + KT - 1) / KT;
  int ida[KT / 16], idb[KT / 16];  // block ids of the next tile of each register stage
  TileRegs<T, D> ra, rb;
  // The prologue leaves the loads in the loop's steady-state order (stage a's
  // tile and ids, then stage b's), so the waits at the top of the loop are the
  // same on the first and on every later pass.
  tile_block_ids<U>(a, bt, t_begin * KT, jlast, ida);
  tile_block_ids<U>(a, bt, (t_begin + 1) * KT, jlast, idb);
  tile_load_regs<T, D, APPEND, U>(a, hk, t_begin * KT, jlast, ida, ra, true, true, ap);
  tile_block_ids<U>(a, bt, (t_begin + 2) * KT, jlast, ida);
  __builtin_amdgcn_sched_barrier(0);
  tile_load_regs<T, D, APPEND, U>(a, hk, (t_begin + 1) * KT, jlast, idb, rb, true, true, ap);
  tile_block_ids<U>(a, bt, (t_begin + 3) * KT, jlast, idb);
  __builtin_amdgcn_sched_barrier(0);

  ChunkState<D, 1> st;
  chunk_reset(st);
  for (int t = t_begin; t < t_end; t += 2) {
    decode2_tile<T, D, APPEND, U>(a, bt, hk, t, t_end, jlast, ida, ra, v_lds, q, lim, st, ap, col < ncols, part_row);
    decode2_tile<T, D, APPEND, U>(a, bt, hk, t + 1, t_end, jlast, idb, rb, v_lds, q, lim, st, ap, col < ncols, part_row);
  }
}

// Waves per (row, query head) of the merge.  One wave (two head-dim elements
// per lane at d = 128) against two: the same time for 128 chunks per row
// (long-context decode), and for rows of few chunks, where the merge is a
// chain of dependent loads per wave and half the waves means fewer rounds of
// them, 128 ragged sequences 0.3983 -> 0.3928 ms, 17-token chunked prefill
// 17.35 -> 16.96 ms (in-process A/B, same bits; four waves were slower).
#ifndef PKV_MERGE_WPR
#define PKV_MERGE_WPR 1
#endif
constexpr int kMergeWavesPerRow = PKV_MERGE_WPR;
// Chunks per round of the merge: two rounds in flight are 3 * 2 * PF loads,
// which must stay within the 63 outstanding loads the wave's counter tracks
// (with 16, the fold of one round waited for part of the next).  In-process
// A/B against one round of 16 at a time: 64 x 4096 keys 0.1081 -> 0.1068 ms,
// 16 x 131072 keys 1.4711 -> 1.4668 ms, same bits.
#ifndef PKV_MERGE_PF
#define PKV_MERGE_PF 10
#endif

// PF chunk partials of one row from chunk c0 on (indices clamped to the last
// one, so every load is in bounds and none sits under a branch).
template <int PF, int EPL, int D>
__device__ __forceinline__ void merge_load(const MergeArgs& a, int64_t base, int e0, int c0, int nck, float (&mc)[PF],
                                           float (&lc)[PF], float (&oc)[PF][EPL]) {
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    const int64_t pi = base + min(c0 + i, nck - 1) * a.ps_chunk;
    mc[i] = a.part_ml[2 * pi];
    lc[i] = a.part_ml[2 * pi + 1];
    const float* po = a.part_o + pi * D + e0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) oc[i][e] = po[e];
  }
}

// The fold of those partials into the running (M, Ls, O), ascending.
template <class T, int PF, int EPL>
__device__ __forceinline__ void merge_fold(int c0, int nck, const float (&mc)[PF], const float (&lc)[PF],
                                           const float (&oc)[PF][EPL], float& M, float& Ls, float (&O)[EPL]) {
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    if (c0 + i >= nck || mc[i] == -INFINITY) continue;
    const FoldCoef<T> f = fold_coef<T>(M, mc[i]);
    Ls = fold_val(Ls, f.a, lc[i], f.b);
#pragma unroll
    for (int e = 0; e < EPL; ++e) O[e] = fold_val(O[e], f.a, oc[i][e], f.b);
    M = f.mn;
  }
}

// Fold of one row's chunk partials, ascending chunk index, then the final
// write.  WPR waves per (row, query head), each owning D / WPR head-dim
// elements (EPL per lane).  The partials come in rounds of PF chunks, double
// buffered: the next round's loads are issued before this round is folded,
// so a wave waits for one round's latency at a time, not for every round.
template <class T, int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  if (dbg_skip(a.dbg_word)) return;
  constexpr int WPR = kMergeWavesPerRow;
  constexpr int EPL = D / 64 / WPR > 0 ? D / 64 / WPR : 1;
  constexpr int PF = PKV_MERGE_PF;
  // the wave's index in the work group is the same in every lane: say so, so
  // that the row, its chunk count and the fold loop are scalar
  const int64_t wg = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t w = wg / WPR;
  const int part = static_cast<int>(wg % WPR);
  if (w >= a.total_q * a.hq) return;
  const int64_t row = w / a.hq;
  const SeqOfRow sr = seq_of_row(a.cu_q, a.seqlens_k, a.batch, row);
  if (sr.b >= a.batch) return;
  const int n = sr.n;
  const int L = sr.cu1 - sr.cu0;
  const int p = n - L + static_cast<int>(row - sr.cu0);
  const int lim = a.causal ? min(p + 1, n) : n;
  const int nck = lim > 0 ? min((lim + KC - 1) / KC, a.maxc) : 0;
  const int lane = lane_id();
  const int e0 = part * (D / WPR) + EPL * lane;
  const bool active = EPL * lane < D / WPR;
  // lanes past the wave's elements (d = 64) read the wave's first element and store nothing
  const int e0c = active ? e0 : part * (D / WPR);
  float M = -INFINITY, Ls = 0.f;
  float O[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) O[e] = 0.f;
  const int64_t base = w * a.ps_row;
  if (nck > 0) {
    float ma[PF], la[PF], oa[PF][EPL], mb[PF], lb[PF], ob[PF][EPL];
    merge_load<PF, EPL, D>(a, base, e0c, 0, nck, ma, la, oa);
    for (int c0 = 0;; c0 += 2 * PF) {
      merge_load<PF, EPL, D>(a, base, e0c, c0 + PF, nck, mb, lb, ob);
      merge_fold<T, PF, EPL>(c0, nck, ma, la, oa, M, Ls, O);
      if (c0 + PF >= nck) break;
      merge_load<PF, EPL, D>(a, base, e0c, c0 + 2 * PF, nck, ma, la, oa);
      merge_fold<T, PF, EPL>(c0 + PF, nck, mb, lb, ob, M, Ls, O);
      if (c0 + 2 * PF >= nck) break;
    }
  }
  if (lane == 0 && part == 0) a.lse[w] = final_lse<T>(M, Ls);
  if (!active) return;
  if constexpr (T::EB == 2) {
    uint16_t* o = static_cast<uint16_t*>(a.out) + w * D + e0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = static_cast<uint16_t>(bf16_rne_bits(final_val(M, O[e], Ls, a.v_scale)));
  } else {
    float* o = static_cast<float*>(a.out) + w * D + e0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = final_val(M, O[e], Ls, a.v_scale);
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers (called by pkv_api.hip after validation).
// ---------------------------------------------------------------------------
template <class T, int D, bool APPEND>
static hipError_t launch_attn_t(const AttnArgs& a, const LaunchPlan& pl, hipStream_t stream) {
  // Uniform block ids per 16 rows (block size a multiple of 16) with 32-bit
  // in-block offsets and block strides below 2^32 bytes: scalar id loads and
  // scalar-based addresses.
  const int64_t span = (static_cast<int64_t>(a.bs) - 1) * std::max(a.kss, a.vss) * T::KVB + D * T::KVB;
  const bool uni = a.bs % 16 == 0 && a.kss >= 0 && a.vss >= 0 && span < (int64_t{1} << 31) && a.kbs >= 0 &&
                   a.vbs >= 0 && std::max(a.kbs, a.vbs) * T::KVB < (int64_t{1} << 32);
  if (pl.full) {
    dim3 grid(a.ncb, pl.hk, pl.batch);
    if constexpr (T::EB == 2 && !APPEND) {
      if (pl.full8) {
        if (uni)
          hipLaunchKernelGGL((attn_kernel<T, D, 8, 2, false, APPEND, true>), grid, dim3(512), 0, stream, a);
        else
          hipLaunchKernelGGL((attn_kernel<T, D, 8, 2, false, APPEND, false>), grid, dim3(512), 0, stream, a);
        return hipGetLastError();
      }
    }
    if (T::EB == 2 && !pl.full4) {
      if constexpr (T::EB == 2) hipLaunchKernelGGL((prefill_kernel<T, D, 8, APPEND>), grid, dim3(512), 0, stream, a);
    } else if (uni) {
      hipLaunchKernelGGL((attn_kernel<T, D, 4, 2, false, APPEND, true>), grid, dim3(256), 0, stream, a);
    } else {
      hipLaunchKernelGGL((attn_kernel<T, D, 4, 2, false, APPEND, false>), grid, dim3(256), 0, stream, a);
    }
    return hipGetLastError();
  }
  dim3 grid(a.ncb * pl.items, pl.hk, pl.batch);
  if constexpr (T::EB == 2 && T::KVB == 2 && !APPEND) {
    if (pl.fold_waves == 2) {  // one work group per (sequence, KV head, column block), a wave per chunk
      const dim3 fgrid(a.ncb, pl.hk, pl.batch);
      if (uni)
        hipLaunchKernelGGL((decode_kernel<T, D, false, true, 2>), fgrid, dim3(128), 0, stream, a);
      else
        hipLaunchKernelGGL((decode_kernel<T, D, false, false, 2>), fgrid, dim3(128), 0, stream, a);
      return hipGetLastError();
    }
  }
  if (pl.lpt) {
    // prefix counts of the longest-first job list, then one work item per job slot
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, stream, a.seqlens_k, a.cu_q, pl.batch,
                       const_cast<int32_t*>(a.job_pref));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    grid = dim3(static_cast<unsigned>(static_cast<int64_t>(pl.batch) * pl.hk * a.maxc), 1, 1);
  }
  if (pl.waves == 1) {
    // FP8 always, bf16 when the grid exceeds one round of one-wave slots:
    // the two-stage kernel (two tiles in flight, one wave per SIMD)
    if constexpr (T::KVB == 1) {
      if (uni)
        hipLaunchKernelGGL((decode2_kernel<T, D, APPEND, true>), grid, dim3(64), 0, stream, a);
      else
        hipLaunchKernelGGL((decode2_kernel<T, D, APPEND, false>), grid, dim3(64), 0, stream, a);
    } else if constexpr (T::EB == 2) {
      if (pl.two_stage && uni)
        hipLaunchKernelGGL((decode2_kernel<T, D, APPEND, true>), grid, dim3(64), 0, stream, a);
      else if (pl.two_stage)
        hipLaunchKernelGGL((decode2_kernel<T, D, APPEND, false>), grid, dim3(64), 0, stream, a);
      else if (uni)
        hipLaunchKernelGGL((decode_kernel<T, D, APPEND, true>), grid, dim3(64), 0, stream, a);
      else
        hipLaunchKernelGGL((decode_kernel<T, D, APPEND, false>), grid, dim3(64), 0, stream, a);
    } else {
      hipLaunchKernelGGL((attn_kernel<T, D, 1, 1, true, APPEND, false>), grid, dim3(64), 0, stream, a);
    }
  } else if constexpr (PKV_SPLIT_W == 8) {
    // 8 waves x kSplitGroups/2 column groups: the same columns per work group
    constexpr int NT8 = kSplitGroups / 2;
    if (uni)
      hipLaunchKernelGGL((attn_kernel<T, D, 8, NT8, true, APPEND, true>), grid, dim3(512), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_kernel<T, D, 8, NT8, true, APPEND, false>), grid, dim3(512), 0, stream, a);
  } else if (uni) {
    hipLaunchKernelGGL((attn_kernel<T, D, 4, kSplitGroups, true, APPEND, true>), grid, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((attn_kernel<T, D, 4, kSplitGroups, true, APPEND, false>), grid, dim3(256), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.skip_merge || pl.direct || pl.fold_waves) return e;
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
  m.ps_row = a.ps_row;
  m.ps_chunk = a.ps_chunk;
  m.causal = a.causal;
  m.v_scale = a.v_scale;
  m.dbg_word = a.dbg_word;
  const int64_t waves = pl.total_q * a.hq;
  if (waves == 0) return hipSuccess;
  dim3 mgrid(static_cast<unsigned>((waves * kMergeWavesPerRow + 3) / 4));
  hipLaunchKernelGGL((merge_kernel<T, D>), mgrid, dim3(256), 0, stream, m);
  return hipGetLastError();
}

template <bool APPEND>
static hipError_t launch_attention_t(const AttnArgs& a, const LaunchPlan& pl, int dtype, int d, hipStream_t stream) {
  if (dtype == 1) {
    return d == 128 ? launch_attn_t<TBf16, 128, APPEND>(a, pl, stream) : launch_attn_t<TBf16, 64, APPEND>(a, pl, stream);
  }
  if (dtype == 2) {
    return d == 128 ? launch_attn_t<TFp8, 128, APPEND>(a, pl, stream) : launch_attn_t<TFp8, 64, APPEND>(a, pl, stream);
  }
  return d == 128 ? launch_attn_t<TF32, 128, APPEND>(a, pl, stream) : launch_attn_t<TF32, 64, APPEND>(a, pl, stream);
}

template <class T, int D>
static hipError_t launch_merge_t(const MergeArgs& m, hipStream_t stream) {
  const int64_t waves = m.total_q * m.hq;
  if (waves == 0) return hipSuccess;
  dim3 mgrid(static_cast<unsigned>((waves * kMergeWavesPerRow + 3) / 4));
  hipLaunchKernelGGL((merge_kernel<T, D>), mgrid, dim3(256), 0, stream, m);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& m, int dtype, int d, hipStream_t stream) {
  (void)hipGetLastError();
  if (dtype == 0) return d == 128 ? launch_merge_t<TF32, 128>(m, stream) : launch_merge_t<TF32, 64>(m, stream);
  // bf16 and FP8 caches share the bf16 output path
  return d == 128 ? launch_merge_t<TBf16, 128>(m, stream) : launch_merge_t<TBf16, 64>(m, stream);
}

hipError_t launch_attention(const AttnArgs& a, const LaunchPlan& pl, int dtype, int d, hipStream_t stream) {
  (void)hipGetLastError();
  return pl.append ? launch_attention_t<true>(a, pl, dtype, d, stream) : launch_attention_t<false>(a, pl, dtype, d, stream);
}

}  // namespace pkv
