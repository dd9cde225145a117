// Kernel argument blocks and the host-side launchers exported by each
// kernel translation unit (internal to libfa.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Which kernel fa_debug_visits walks.
enum WalkKind { WALK_FWD = 0, WALK_DKDV = 1, WALK_DQ = 2 };

// Work split of the dK/dV column walks under a block mask.  Without it one
// key column of the mask that many query cells visit (a global column) is
// walked by a single work-group while the rest of the chip idles.  A plan
// fixes a chunk size CH (cells); every column with more than CH visited cells
// is cut into chunks of CH consecutive cells, each chunk its own work-group
// ("split item"); each chunk writes its fp32 partial dK/dV into a slot and
// the last chunk of a column to finish adds the slots in chunk order (so the
// result does not depend on the finishing order) and stores dK/dV.
constexpr int NT_HOST = 256;              // threads per attention work-group
constexpr int SPLIT_TARGET = 512;          // concurrent dK/dV work-groups on the chip
constexpr int SPLIT_MAX_ITEMS = 2 * SPLIT_TARGET;   // bound on split items, see the plan kernel
constexpr int SPLIT_MIN_CELLS = 16;        // smallest chunk
constexpr int SPLIT_COUNT_ROWS = 64;       // mask rows per partial column count

struct SplitWs {
  int* hdr;          // [0] split items, [1] P = split items per head, [2] CH
  int* table;        // [P][4]: key cell, first entry of that cell, its chunks, 0
  unsigned* ctr;     // [items] arrival counters (entry of a column's first chunk)
  float* slots;      // [items][2][D/4][128][4] fp32 partial dK, dV
  int* part;         // [ceil(T/64)][T] visited-cell counts per column and row band
};

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;        // forward output (read by the backward preprocess)
  const void* dO;
  void* out0;           // fwd: O;  dkdv: dK;  dq: dQ
  void* out1;           // dkdv: dV
  float* lse;           // fwd: written;  bwd: read
  float* delta;         // bwd: rowsum(dO * O)
  int B, H, N;
  float scale;          // softmax scale (> 0)
  float c;              // scale * log2(e): scores enter exp2 through this factor
  int causal;
  const uint8_t* mask;  // [T][T] or null
  const int32_t* kv_len;  // [B] or null
  uint32_t* counts;     // visit counters (walk-only instances)
  SplitWs split;        // dK/dV work split (bf16 with a block mask), else zeros
  // dropout on P (bf16 kernels): keep iff the Philox byte >= drop_t; 0 = off
  uint32_t drop_t, drop_k0, drop_k1;
  float drop_inv;       // 1 / (1 - drop_t / 256)
  // split-key forward (N = queries): Nk keys, causal limit key <= query +
  // causal_off, nsplit key ranges of split_tiles 64-key tiles each; partial
  // outputs part_o [nsplit][B*H*N][d] and (m, l) part_ml [nsplit][B*H*N][2]
  int Nk, causal_off, nsplit, split_tiles;
  float* part_o;
  float* part_ml;
  // FP8 forward: real V = E4M3 code * v_descale (the Q and K descales are
  // folded into c)
  float v_descale;
};

// Bytes of the dK/dV split workspace for N keys and head dimension d; the
// offsets of its parts follow the order of SplitWs.
size_t split_ws_bytes(int N, int d);
SplitWs split_ws_carve(void* base, int N, int d);

// dtype: 0 = bf16, 1 = f32;  d: 64 or 128.
hipError_t launch_fwd(const AttnArgs& a, int dtype, int d, bool walk_only, hipStream_t s);
hipError_t launch_bwd_pre(const AttnArgs& a, int dtype, int d, hipStream_t s);
hipError_t launch_bwd_dkdv(const AttnArgs& a, int dtype, int d, bool walk_only, hipStream_t s);
hipError_t launch_bwd_dq(const AttnArgs& a, int dtype, int d, bool walk_only, hipStream_t s);

// bf16 instances (fa_bf16.hip)
hipError_t launch_fwd_bf16(const AttnArgs& a, int d, bool walk_only, hipStream_t s);
hipError_t launch_dkdv_bf16(const AttnArgs& a, int d, bool walk_only, hipStream_t s);
hipError_t launch_dq_bf16(const AttnArgs& a, int d, bool walk_only, hipStream_t s);
// Column counts + plan of the dK/dV split (needs a.mask and a.split).
hipError_t launch_split_plan(const AttnArgs& a, hipStream_t s);
// Split-key forward (bf16): partial outputs of every key range, then their merge.
hipError_t launch_fwd_splitkv_bf16(const AttnArgs& a, int d, hipStream_t s);
// The same for at most four queries per head (one wave per key range).
hipError_t launch_fwd_decode_bf16(const AttnArgs& a, int d, hipStream_t s);
// Decoding against E4M3 K and V (bf16 queries; a.c holds the K descale).
hipError_t launch_fwd_decode_e4m3kv(const AttnArgs& a, int d, hipStream_t s);
// Forward on E4M3 Q, K, V (d = 64 or 128).
hipError_t launch_fwd_fp8(const AttnArgs& a, int d, hipStream_t s);
// Merge of the partial outputs a.part_o / a.part_ml into a.out0 and a.lse.
hipError_t launch_splitkv_merge(const AttnArgs& a, int d, hipStream_t s);

}  // namespace fa
