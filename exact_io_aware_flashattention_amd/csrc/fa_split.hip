// Plan of the dK/dV work split under a block mask (block-sparse
// FlashAttention, FlashAttention reading guide, "Ekstensi: Block-Sparse
// FlashAttention": the work of a key column is one term per visited cell, and
// a column visited by many query cells carries many terms).
//
// Chunk size.  With V visited cells over all heads (an upper estimate: every
// batch entry counted as unpadded) the plan takes CH = max(16, ceil(V / 512)),
// 512 being the number of dK/dV work-groups the chip holds at once, so a
// chunk is about one work-group's fair share of the work.  A column with more
// than CH cells is cut into chunks of CH consecutive visited cells.  Bound on
// the number of chunks: every cut column holds more than CH cells, so there
// are fewer than V / CH <= 512 cut columns (over all heads), and they have at
// most V / CH + (number of cut columns) < 1024 chunks together.
#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

namespace {

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }
int cells_of(int N) { return (N + CELL - 1) / CELL; }
int bands_of(int T) { return (T + SPLIT_COUNT_ROWS - 1) / SPLIT_COUNT_ROWS; }

// Visited cells of column kj among mask rows [64 band, 64 band + 64): one
// thread per column, so the byte loads of a row are contiguous across lanes.
__global__ __launch_bounds__(NT) void split_count_kernel(AttnArgs a) {
  const int T = (a.N + CELL - 1) / CELL;
  const int kj = blockIdx.x * NT + threadIdx.x;
  const int band = blockIdx.y;
  if (kj >= T) return;
  const int i0 = max(band * SPLIT_COUNT_ROWS, a.causal ? kj : 0);
  const int i1 = min(T, (band + 1) * SPLIT_COUNT_ROWS);
  int n = 0;
#pragma unroll 8
  for (int i = i0; i < i1; ++i) n += a.mask[(size_t)i * T + kj] != 0;
  a.split.part[(size_t)band * T + kj] = n;
}

// One work-group: per-column totals, CH, the chunk table, cleared counters.
__global__ __launch_bounds__(NT) void split_plan_kernel(AttnArgs a) {
  __shared__ int cnt[MAX_T];
  __shared__ int heavy[MAX_T];
  __shared__ int heavy_off[MAX_T];
  __shared__ int scratch4[4];
  __shared__ unsigned long long red[NT / 64];
  __shared__ int sh[3];
  const int T = (a.N + CELL - 1) / CELL;
  const int bands = (T + SPLIT_COUNT_ROWS - 1) / SPLIT_COUNT_ROWS;
  const int tid = threadIdx.x;

  unsigned long long local = 0;
  for (int kj = tid; kj < T; kj += NT) {
    int n = 0;
    for (int band = 0; band < bands; ++band) n += a.split.part[(size_t)band * T + kj];
    cnt[kj] = n;
    local += (unsigned long long)n;
  }
  for (int off = 32; off > 0; off >>= 1) local += __shfl_down(local, off);
  if ((tid & 63) == 0) red[tid >> 6] = local;
  __syncthreads();
  unsigned long long per_head = 0;
  for (int w = 0; w < NT / 64; ++w) per_head += red[w];
  const unsigned long long total = per_head * (unsigned long long)a.B * (unsigned long long)a.H;
  const unsigned long long want = (total + SPLIT_TARGET - 1) / SPLIT_TARGET;
  const int CH = (int)(want < (unsigned long long)SPLIT_MIN_CELLS ? SPLIT_MIN_CELLS
                                                                  : (want > MAX_T ? MAX_T + 1 : want));
  const int nh = build_list(T, [&](int kj) { return cnt[kj] > CH; }, heavy, scratch4);

  if (tid == 0) {
    int P = 0;
    for (int m = 0; m < nh; ++m) {
      heavy_off[m] = P;
      P += (cnt[heavy[m]] + CH - 1) / CH;
    }
    long long items = (long long)P * a.B * a.H;
    int ch = CH;
    if (items > SPLIT_MAX_ITEMS) {   // excluded by the bound above; kept as a guard
      P = 0;
      items = 0;
      ch = MAX_T + 1;
    }
    sh[0] = (int)items;
    sh[1] = P;
    sh[2] = ch;
    a.split.hdr[0] = (int)items;
    a.split.hdr[1] = P;
    a.split.hdr[2] = ch;
  }
  __syncthreads();
  const int items = sh[0];
  if (sh[1] > 0) {
    for (int m = tid; m < nh; m += NT) {
      const int kj = heavy[m], off = heavy_off[m];
      const int nc = (cnt[kj] + CH - 1) / CH;
      for (int c = 0; c < nc; ++c) {
        int* e = a.split.table + 4 * (off + c);
        e[0] = kj;
        e[1] = off;
        e[2] = nc;
        e[3] = 0;
      }
    }
  }
  for (int i = tid; i < items; i += NT) a.split.ctr[i] = 0u;
}

}  // namespace

size_t split_ws_bytes(int N, int d) {
  const int T = cells_of(N);
  return up256(4 * sizeof(int)) + up256((size_t)SPLIT_MAX_ITEMS * 4 * sizeof(int)) +
         up256((size_t)SPLIT_MAX_ITEMS * sizeof(unsigned)) +
         up256((size_t)SPLIT_MAX_ITEMS * 2 * CELL * d * sizeof(float)) +
         up256((size_t)bands_of(T) * T * sizeof(int));
}

SplitWs split_ws_carve(void* base, int N, int d) {
  const int T = cells_of(N);
  unsigned char* p = static_cast<unsigned char*>(base);
  SplitWs w;
  w.hdr = reinterpret_cast<int*>(p);
  p += up256(4 * sizeof(int));
  w.table = reinterpret_cast<int*>(p);
  p += up256((size_t)SPLIT_MAX_ITEMS * 4 * sizeof(int));
  w.ctr = reinterpret_cast<unsigned*>(p);
  p += up256((size_t)SPLIT_MAX_ITEMS * sizeof(unsigned));
  w.slots = reinterpret_cast<float*>(p);
  p += up256((size_t)SPLIT_MAX_ITEMS * 2 * CELL * d * sizeof(float));
  w.part = reinterpret_cast<int*>(p);
  (void)T;
  return w;
}

hipError_t launch_split_plan(const AttnArgs& a, hipStream_t s) {
  const int T = cells_of(a.N);
  const dim3 grid((unsigned)((T + NT - 1) / NT), (unsigned)bands_of(T));
  hipLaunchKernelGGL(split_count_kernel, grid, dim3(NT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(split_plan_kernel, dim3(1), dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace fa
