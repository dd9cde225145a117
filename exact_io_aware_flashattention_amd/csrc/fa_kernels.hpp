// Kernel argument blocks and the host-side launchers exported by each
// kernel translation unit (internal to libfa.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Which kernel fa_debug_visits walks.
enum WalkKind { WALK_FWD = 0, WALK_DKDV = 1, WALK_DQ = 2 };

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
};

// dtype: 0 = bf16, 1 = f32;  d: 64 or 128.
hipError_t launch_fwd(const AttnArgs& a, int dtype, int d, bool walk_only, hipStream_t s);
hipError_t launch_bwd_pre(const AttnArgs& a, int dtype, int d, hipStream_t s);
hipError_t launch_bwd_dkdv(const AttnArgs& a, int dtype, int d, bool walk_only, hipStream_t s);
hipError_t launch_bwd_dq(const AttnArgs& a, int dtype, int d, bool walk_only, hipStream_t s);

// bf16 instances (fa_bf16.hip)
hipError_t launch_fwd_bf16(const AttnArgs& a, int d, bool walk_only, hipStream_t s);
hipError_t launch_dkdv_bf16(const AttnArgs& a, int d, bool walk_only, hipStream_t s);
hipError_t launch_dq_bf16(const AttnArgs& a, int d, bool walk_only, hipStream_t s);

}  // namespace fa
