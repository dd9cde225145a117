// Tile-skip walk over the 128 x 128 mask cells (block-sparse FlashAttention,
// FlashAttention reading guide, "Ekstensi: Block-Sparse FlashAttention": only
// blocks whose mask entry is 1 are evaluated).  A cell (i, j) is visited iff
//     block_mask[i][j] != 0  and  (not causal or j <= i)  and  128*j < kv_len[b]
// -- a cell that fails the causal or padding test holds only -inf scores and
// is skipped exactly like a zero mask cell.  Visited cells are walked in
// ascending order, each split into two 64-wide tiles; a trailing tile that
// lies wholly past the valid range is dropped.
#pragma once

#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

struct Walk {
  int base;          // first cell index along the walked direction
  int ncells;        // visited cells
  int ntiles;        // 64-wide tiles to process
  const int* list;   // LDS list of visited cell offsets (block-sparse), or null

  __device__ __forceinline__ int cell(int c) const { return base + (list ? list[c] : c); }
  __device__ __forceinline__ int tile_start(int it) const { return cell(it >> 1) * CELL + (it & 1) * 64; }
  __device__ __forceinline__ bool first_of_cell(int it) const { return (it & 1) == 0; }
};

__device__ __forceinline__ int clamp_kv_len(const AttnArgs& a, int b) {
  int kvl = a.N;
  if (a.kv_len) kvl = min(max(a.kv_len[b], 0), a.N);
  return kvl;
}

// Row walk: key tiles for query cell qi (forward and dQ kernels).  kv_end is
// the first key position past every allowed key of the cell's rows.
__device__ inline Walk row_walk(const AttnArgs& a, int qi, int kv_end, int T, int* list, int* scratch4) {
  Walk w;
  w.base = 0;
  const int jlim = (kv_end + CELL - 1) / CELL;
  if (a.mask) {
    const uint8_t* row = a.mask + (size_t)qi * T;
    w.ncells = build_list(jlim, [&](int j) { return row[j] != 0; }, list, scratch4);
    w.list = list;
  } else {
    w.ncells = jlim;
    w.list = nullptr;
  }
  w.ntiles = 2 * w.ncells;
  if (w.ncells > 0 && w.cell(w.ncells - 1) * CELL + 64 >= kv_end) w.ntiles -= 1;
  return w;
}

// Column walk: query tiles for key cell kj (dK/dV kernel).
__device__ inline Walk col_walk(const AttnArgs& a, int kj, int kvl, int T, int* list, int* scratch4) {
  Walk w;
  w.base = a.causal ? kj : 0;
  w.list = nullptr;
  w.ncells = 0;
  const bool any_key = kj * CELL < kvl;
  const int count = T - w.base;
  if (a.mask) {
    const uint8_t* col = a.mask + kj;
    const int base = w.base;
    const int n = build_list(any_key ? count : 0, [&](int c) { return col[(size_t)(base + c) * T] != 0; },
                             list, scratch4);
    w.ncells = n;
    w.list = list;
  } else {
    w.ncells = any_key ? count : 0;
  }
  w.ntiles = 2 * w.ncells;
  if (w.ncells > 0 && w.cell(w.ncells - 1) * CELL + 64 >= a.N) w.ntiles -= 1;
  return w;
}

}  // namespace fa
