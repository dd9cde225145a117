// Tile-skip walk over the 128 x 128 mask cells (block-sparse FlashAttention,
// FlashAttention reading guide, "Ekstensi: Block-Sparse FlashAttention": only
// blocks whose mask entry is 1 are evaluated).  A cell (i, j) is visited iff
//     block_mask[i][j] != 0  and  (not causal or j <= i)  and  128*j < kv_len[b]
// -- a cell that fails the causal or padding test holds only -inf scores and
// is skipped exactly like a zero mask cell.  Visited cells are walked in
// ascending order, each split into 64- or 32-wide tiles; trailing tiles that
// lie wholly past the valid range are dropped.
#pragma once

#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

struct Walk {
  int base;          // first cell index along the walked direction
  int ncells;        // visited cells
  int ntiles;        // tiles to process
  int tsh;           // log2 of the tile width (32 or 64)
  const int* list;   // LDS list of visited cell offsets (block-sparse), or null

  // (The list entry is wave-uniform; reading it as a scalar keeps all tile
  // address arithmetic on the scalar unit.)
  __device__ __forceinline__ int cell(int c) const {
    return base + (list ? __builtin_amdgcn_readfirstlane(list[c]) : c);
  }
  __device__ __forceinline__ int tile_start(int it) const {
    const int per = 7 - tsh;   // log2(tiles per cell)
    return cell(it >> per) * CELL + ((it & ((1 << per) - 1)) << tsh);
  }
  __device__ __forceinline__ bool first_of_cell(int it) const { return (it & ((1 << (7 - tsh)) - 1)) == 0; }
  // Tiles of the last visited cell that start at or past `limit` are dropped.
  __device__ __forceinline__ void finish(int limit) {
    const int per = 7 - tsh;
    ntiles = ncells << per;
    if (ncells > 0) {
      const int rest = limit - cell(ncells - 1) * CELL;   // > 0 for every visited cell
      const int valid = min(1 << per, (rest + (1 << tsh) - 1) >> tsh);
      ntiles -= (1 << per) - valid;
    }
  }
};

__device__ __forceinline__ int clamp_kv_len(const AttnArgs& a, int b) {
  int kvl = a.N;
  if (a.kv_len) kvl = min(max(a.kv_len[b], 0), a.N);
  return kvl;
}

// Row walk: key tiles for query cell qi (forward and dQ kernels).  kv_end is
// the first key position past every allowed key of the cell's rows.
__device__ inline Walk row_walk(const AttnArgs& a, int qi, int kv_end, int T, int* list, int* scratch4,
                                int tsh = 6) {
  Walk w;
  w.base = 0;
  w.tsh = tsh;
  const int jlim = (kv_end + CELL - 1) / CELL;
  if (a.mask) {
    const uint8_t* row = a.mask + (size_t)qi * T;
    w.ncells = build_list(jlim, [&](int j) { return row[j] != 0; }, list, scratch4);
    w.list = list;
  } else {
    w.ncells = jlim;
    w.list = nullptr;
  }
  w.finish(kv_end);
  return w;
}

// Column walk: query tiles for key cell kj (dK/dV kernel).  *listed gets the
// number of cells the mask and the causal test allow in the column, whether
// or not the column holds any key below kv_len (the split plan counts the
// same cells).
__device__ inline Walk col_walk(const AttnArgs& a, int kj, int kvl, int T, int* list, int* scratch4,
                                int tsh = 6, int* listed = nullptr) {
  Walk w;
  w.base = a.causal ? kj : 0;
  w.tsh = tsh;
  w.list = nullptr;
  const bool any_key = kj * CELL < kvl;
  const int count = T - w.base;
  int n = count;
  if (a.mask) {
    const uint8_t* col = a.mask + kj;
    const int base = w.base;
    n = build_list(count, [&](int c) { return col[(size_t)(base + c) * T] != 0; }, list, scratch4);
    w.list = list;
  }
  if (listed) *listed = n;
  w.ncells = any_key ? n : 0;
  w.finish(a.N);
  return w;
}

// Walk of one key range of a split-key forward: 64-key tiles [t0, t0 + n)
// (t0 even, so the range starts on a 128-key cell).
__device__ inline Walk range_walk(int t0, int n) {
  Walk w;
  w.base = t0 >> 1;
  w.tsh = 6;
  w.list = nullptr;
  w.ntiles = max(n, 0);
  w.ncells = (w.ntiles + 1) >> 1;
  return w;
}

// Restrict a block-sparse walk to its visited cells [c0, c0 + cnt) (one chunk
// of a split column).
__device__ inline void take_chunk(Walk& w, int c0, int cnt, int limit) {
  w.list += c0;
  w.ncells = max(0, min(w.ncells - c0, cnt));
  w.finish(limit);
}

}  // namespace fa
