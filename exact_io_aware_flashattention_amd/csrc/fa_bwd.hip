// Backward kernels.  Only O and lse are kept from the forward pass; S and P
// are recomputed tile by tile from Q, K and lse (FlashAttention reading
// guide, "Ide Utama", recomputation bullet; bornlex.github.io "Flash
// Attention", section "Recomputation").  The pages print no backward
// equations; the chain rule through O = PV and the row softmax gives, with
// delta_i = sum_j P_ij dP_ij = dO_i . O_i:
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - delta),
//     dQ = scale dS K,  dK = scale dS^T Q.
//
//   preprocess  delta = rowsum(dO * O)                       (memory bound)
//   dkdv        one work-group per 128 keys; walks the query tiles that see
//               them (column walk); dV, dK accumulate in registers
//   dq          one work-group per 128 queries; walks the same key tiles as
//               the forward pass (row walk); dQ accumulates in registers
//
// Keeping dQ in its own pass makes every output a plain store (no atomics,
// bit-reproducible) at the price of recomputing S and dP a second time.
#include "fa_device.hpp"
#include "fa_kernels.hpp"
#include "fa_walk.hpp"

namespace fa {

// ---------------------------------------------------------------- preprocess

// Threads per row of the delta pre-pass: one 16-byte chunk each, rounded up
// to a power of two for the shuffle reduction (d = 96, 160: the extra
// threads add zero).
template <typename T, int D>
constexpr int pre_threads_per_row() {
  int t = 1;
  while (t < D / ET<T>::CW) t *= 2;
  return t;
}

template <typename T, int D>
__global__ __launch_bounds__(NT) void bwd_pre_kernel(AttnArgs a) {
  constexpr int CW = ET<T>::CW;
  constexpr int TPR = pre_threads_per_row<T, D>();   // threads per row
  constexpr int RPB = NT / TPR;         // rows per block
  const long long rows = (long long)a.B * a.H * a.N;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows && part < D / CW) {
    const T* o = reinterpret_cast<const T*>(a.o) + row * D + part * CW;
    const T* g = reinterpret_cast<const T*>(a.dO) + row * D + part * CW;
    const u32x4 ov = ld16(o), gv = ld16(g);
    if constexpr (sizeof(T) == 2) {
      const bf16x8 ob = __builtin_bit_cast(bf16x8, ov), gb = __builtin_bit_cast(bf16x8, gv);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)ob[e], (float)gb[e], acc);
    } else {
      const f32x4 of = __builtin_bit_cast(f32x4, ov), gf = __builtin_bit_cast(f32x4, gv);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(of[e], gf[e], acc);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) a.delta[row] = acc;
}

// ---------------------------------------------------------------- shared tile layout

// A 64-row tile of a [N][D] tensor staged as 4-row x 16-byte units: each
// unit is written to LDS both row-major (pitch RP) and transposed
// (element e of row r at [e][r], pitch TP).
template <typename T, int D>
struct Tile64 {
  static constexpr int R = 64;
  static constexpr int CW = ET<T>::CW;
  static constexpr int RP = D + 16 / (int)sizeof(T);   // row-major pitch (elements)
  static constexpr int TP = R + 4;                     // transposed pitch (elements)
  static constexpr int ROW_ELEMS = R * RP;
  static constexpr int TR_ELEMS = D * TP;
  static constexpr int CPR = D / CW;
  static constexpr int UNITS = (R / 4) * CPR;
  static constexpr int UPT = (UNITS + NT - 1) / NT;    // units per thread
  static constexpr int SSTEPS = D / (2 * CW);
  static constexpr int NB = D / 32;
};

template <typename T, int D>
struct UnitRegs {
  u32x4 r[Tile64<T, D>::UPT][4];
};

template <typename T, int D>
__device__ __forceinline__ void unit_load(UnitRegs<T, D>& u, const T* __restrict__ src, int row0, int N) {
  using TL = Tile64<T, D>;
#pragma unroll
  for (int i = 0; i < TL::UPT; ++i) {
    const int unit = threadIdx.x + i * NT;
    if (unit < TL::UNITS) {
      const int kg = unit % (TL::R / 4), dc = unit / (TL::R / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + 4 * kg + r;
        u.r[i][r] = row < N ? ld16(src + (size_t)row * D + dc * TL::CW) : u32x4{0, 0, 0, 0};
      }
    }
  }
}

template <typename T, int D>
__device__ __forceinline__ void unit_store(const UnitRegs<T, D>& u, T* rowmajor, T* transposed) {
  using TL = Tile64<T, D>;
#pragma unroll
  for (int i = 0; i < TL::UPT; ++i) {
    const int unit = threadIdx.x + i * NT;
    if (unit < TL::UNITS) {
      const int kg = unit % (TL::R / 4), dc = unit / (TL::R / 4);
      if (rowmajor) {
#pragma unroll
        for (int r = 0; r < 4; ++r) st16(rowmajor + (4 * kg + r) * TL::RP + dc * TL::CW, u.r[i][r]);
      }
      if (transposed) write_transposed4(transposed + (dc * TL::CW) * TL::TP + 4 * kg, TL::TP, u.r[i]);
    }
  }
}

// acc(32 x 32 block nb of the head dim, accumulator layout) += A x X where
// the A side is read from a transposed LDS tile (rows = head dim, columns =
// the 64 tile rows) for contraction rows 32*half + 8*g + 4*h + 0..3.
template <typename T, int D>
__device__ __forceinline__ void mma_from_transposed(f32x16& acc, const T* tr, int nb, int half, const f32x16& x) {
  using TL = Tile64<T, D>;
  const int lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
  Quad<T> q[4];
  const T* row = tr + (32 * nb + l32) * TL::TP + 32 * half + 4 * h;
#pragma unroll
  for (int g = 0; g < 4; ++g) q[g].load(row + 8 * g);
  mma_acc_operand(acc, q, x);
}

template <typename T, int D>
__device__ __forceinline__ void store_acc_rows(T* base, int row, int N, const f32x16 (&acc)[D / 32], float mul) {
  const int lane = threadIdx.x & 63, h = lane >> 5;
  if (row >= N) return;
  T* p = base + (size_t)row * D;
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      store4(p + 32 * nb + 8 * g + 4 * h, acc[nb][4 * g] * mul, acc[nb][4 * g + 1] * mul,
             acc[nb][4 * g + 2] * mul, acc[nb][4 * g + 3] * mul);
}

// ---------------------------------------------------------------- dK / dV

template <typename T, int D>
struct DkdvCfg {
  using TL = Tile64<T, D>;
  // d = 128 needs more than 256 registers per wave (two fp32 accumulators of
  // 32 x 128 plus K, V fragments): one wave per SIMD, double-buffered LDS.
  static constexpr int OCC = (sizeof(T) == 2 && D == 64) ? 2 : 1;
  static constexpr int STAGE = 2 * TL::ROW_ELEMS + 2 * TL::TR_ELEMS;   // Q, dO row-major + transposed
  static constexpr int STAGE_BYTES = STAGE * (int)sizeof(T) + 2 * 64 * 4;
  static constexpr int NSTAGE = (2 * STAGE_BYTES + MAX_T * 4 <= 160 * 1024 / OCC) ? 2 : 1;
};

template <typename T, int D, bool WALK_ONLY>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(DkdvCfg<T, D>::OCC, DkdvCfg<T, D>::OCC))) void bwd_dkdv_kernel(AttnArgs a) {
  using TL = Tile64<T, D>;
  using CF = DkdvCfg<T, D>;
  constexpr int CW = TL::CW;
  constexpr int SB = CF::STAGE_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char smem[WALK_ONLY ? 16 : CF::NSTAGE * SB];
  __shared__ int cell_list[MAX_T];
  __shared__ int scratch4[4];

  const int N = a.N;
  const int T_cells = (N + CELL - 1) / CELL;
  const WorkUnit u = work_unit(blockIdx.x, gridDim.x, a.B * a.H, T_cells, a.causal);
  const int bh = u.bh, kj = u.t;   // causal: low kj sees the most queries
  const int b = bh / a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int kvl = clamp_kv_len(a, b);
  const Walk walk = col_walk(a, kj, kvl, T_cells, cell_list, scratch4);

  if constexpr (WALK_ONLY) {
    for (int it = 0; it < walk.ntiles; ++it)
      if (tid == 0 && walk.first_of_cell(it))
        atomicAdd(&a.counts[((size_t)b * T_cells + walk.cell(it >> 1)) * T_cells + kj], 1u);
    return;
  } else {
    const size_t head = (size_t)bh * N * D;
    const T* __restrict__ Qg = reinterpret_cast<const T*>(a.q) + head;
    const T* __restrict__ Kg = reinterpret_cast<const T*>(a.k) + head;
    const T* __restrict__ Vg = reinterpret_cast<const T*>(a.v) + head;
    const T* __restrict__ dOg = reinterpret_cast<const T*>(a.dO) + head;
    const float* lse_g = a.lse + (size_t)bh * N;
    const float* del_g = a.delta + (size_t)bh * N;

    const int kw0 = kj * CELL + wave * 32;   // first key of this wave
    const int myk = kw0 + l32;               // the key this lane owns
    const bool wave_has_keys = kw0 < kvl;

    u32x4 kf[TL::SSTEPS], vf[TL::SSTEPS];
#pragma unroll
    for (int s = 0; s < TL::SSTEPS; ++s) {
      const bool ok = myk < N;
      kf[s] = ok ? ld16(Kg + (size_t)myk * D + s * 2 * CW + CW * h) : u32x4{0, 0, 0, 0};
      vf[s] = ok ? ld16(Vg + (size_t)myk * D + s * 2 * CW + CW * h) : u32x4{0, 0, 0, 0};
    }
    f32x16 dk[TL::NB], dv[TL::NB];
#pragma unroll
    for (int nb = 0; nb < TL::NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dk[nb][r] = 0.f;
        dv[nb][r] = 0.f;
      }

    UnitRegs<T, D> uq, ug;
    float stat_lse = 0.f, stat_del = 0.f;
    auto gload = [&](int q0) {
      unit_load<T, D>(uq, Qg, q0, N);
      unit_load<T, D>(ug, dOg, q0, N);
      if (tid < 64) {
        const int q = q0 + tid;
        const float l = q < N ? lse_g[q] : neg_inf();
        // rows with no allowed key (lse = -inf) and rows past N get P = 0
        stat_lse = (l == neg_inf()) ? pos_inf() : l * LOG2E;
        stat_del = q < N ? del_g[q] : 0.f;
      }
    };
    auto stage_ptr = [&](int st) { return smem + (CF::NSTAGE == 2 ? st : 0) * SB; };
    auto swrite = [&](int st) {
      T* base = reinterpret_cast<T*>(stage_ptr(st));
      T* Qs = base;
      T* dOs = Qs + TL::ROW_ELEMS;
      T* Qt = dOs + TL::ROW_ELEMS;
      T* dOt = Qt + TL::TR_ELEMS;
      float* ls = reinterpret_cast<float*>(dOt + TL::TR_ELEMS);
      unit_store<T, D>(uq, Qs, Qt);
      unit_store<T, D>(ug, dOs, dOt);
      if (tid < 64) {
        ls[tid] = stat_lse;
        ls[64 + tid] = stat_del;
      }
    };

    if (walk.ntiles > 0) {
      gload(walk.tile_start(0));
      swrite(0);
    }
    __syncthreads();

    for (int it = 0; it < walk.ntiles; ++it) {
      const int q0 = walk.tile_start(it);
      const bool has_next = it + 1 < walk.ntiles;
      if (has_next) gload(walk.tile_start(it + 1));
      const T* Qs = reinterpret_cast<const T*>(stage_ptr(it & 1));
      const T* dOs = Qs + TL::ROW_ELEMS;
      const T* Qt = dOs + TL::ROW_ELEMS;
      const T* dOt = Qt + TL::TR_ELEMS;
      const float* ls = reinterpret_cast<const float*>(dOt + TL::TR_ELEMS);

      const bool active = wave_has_keys && !(a.causal && kw0 > q0 + 63);
      if (active) {
        const bool edge = (kw0 + 32 > kvl) || (a.causal && kw0 + 31 > q0);
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
          // S = Q K^T and dP = dO V^T for 32 queries x this wave's 32 keys
          f32x16 s, dp;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            s[r] = 0.f;
            dp[r] = 0.f;
          }
          const T* qrow = Qs + (32 * qs + l32) * TL::RP + CW * h;
          const T* grow = dOs + (32 * qs + l32) * TL::RP + CW * h;
#pragma unroll
          for (int st = 0; st < TL::SSTEPS; ++st) {
            mma_chunk(s, ld16(qrow + st * 2 * CW), kf[st], (T*)nullptr);
            mma_chunk(dp, ld16(grow + st * 2 * CW), vf[st], (T*)nullptr);
          }
          // P = exp2(s c - lse log2 e), dS = P (dP - delta); register r <-> query
          // 32*qs + 8*(r/4) + 4*h + r%4 of the tile
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int qq = 32 * qs + 8 * g + 4 * h;
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(ls + qq);
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(ls + 64 + qq);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * g + e;
              float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.c, -l4[e]));
              if (edge) {
                const int q = q0 + qq + e;
                if (myk >= kvl || (a.causal && myk > q)) p = 0.f;
              }
              s[r] = p;
              dp[r] = p * (dp[r] - d4[e]);
            }
          }
          // dV^T += dO^T P,  dK^T += Q^T dS
#pragma unroll
          for (int nb = 0; nb < TL::NB; ++nb) {
            mma_from_transposed<T, D>(dv[nb], dOt, nb, qs, s);
            mma_from_transposed<T, D>(dk[nb], Qt, nb, qs, dp);
          }
        }
      }
      if (CF::NSTAGE == 1) __syncthreads();
      if (has_next) swrite((it + 1) & 1);
      __syncthreads();
    }

    // lane owns key myk; registers hold the head dim (accumulator layout)
    store_acc_rows<T, D>(reinterpret_cast<T*>(a.out0) + head, myk, N, dk, a.scale);
    store_acc_rows<T, D>(reinterpret_cast<T*>(a.out1) + head, myk, N, dv, 1.f);
  }
}

// ---------------------------------------------------------------- dQ

template <typename T, int D>
struct DqCfg {
  using TL = Tile64<T, D>;
  static constexpr int STAGE = 2 * TL::ROW_ELEMS + TL::TR_ELEMS;   // K, V row-major + K transposed
  static constexpr int STAGE_BYTES = STAGE * (int)sizeof(T);
  static constexpr int NSTAGE = (2 * STAGE_BYTES + MAX_T * 4 <= 160 * 1024 / Occ<T>::W) ? 2 : 1;
};

template <typename T, int D, bool WALK_ONLY>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(Occ<T>::W, Occ<T>::W))) void bwd_dq_kernel(AttnArgs a) {
  using TL = Tile64<T, D>;
  using CF = DqCfg<T, D>;
  constexpr int CW = TL::CW;
  constexpr int SB = CF::STAGE_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char smem[WALK_ONLY ? 16 : CF::NSTAGE * SB];
  __shared__ int cell_list[MAX_T];
  __shared__ int scratch4[4];

  const int N = a.N;
  const int T_cells = (N + CELL - 1) / CELL;
  const WorkUnit u = work_unit(blockIdx.x, gridDim.x, a.B * a.H, T_cells, a.causal);
  const int bh = u.bh;
  const int qi = a.causal ? T_cells - 1 - u.t : u.t;
  const int b = bh / a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int kvl = clamp_kv_len(a, b);
  const int q_lo = qi * CELL, q_hi = min(q_lo + CELL, N);
  const int kv_end = a.causal ? min(kvl, q_hi) : kvl;
  const Walk walk = row_walk(a, qi, kv_end, T_cells, cell_list, scratch4);

  if constexpr (WALK_ONLY) {
    for (int it = 0; it < walk.ntiles; ++it)
      if (tid == 0 && walk.first_of_cell(it))
        atomicAdd(&a.counts[((size_t)b * T_cells + qi) * T_cells + walk.cell(it >> 1)], 1u);
    return;
  } else {
    const size_t head = (size_t)bh * N * D;
    const T* __restrict__ Qg = reinterpret_cast<const T*>(a.q) + head;
    const T* __restrict__ Kg = reinterpret_cast<const T*>(a.k) + head;
    const T* __restrict__ Vg = reinterpret_cast<const T*>(a.v) + head;
    const T* __restrict__ dOg = reinterpret_cast<const T*>(a.dO) + head;

    const int qw0 = q_lo + wave * 32;
    const int myq = qw0 + l32;
    const bool wave_has_rows = qw0 < N;

    u32x4 qf[TL::SSTEPS], gf[TL::SSTEPS];
#pragma unroll
    for (int s = 0; s < TL::SSTEPS; ++s) {
      const bool ok = myq < N;
      qf[s] = ok ? ld16(Qg + (size_t)myq * D + s * 2 * CW + CW * h) : u32x4{0, 0, 0, 0};
      gf[s] = ok ? ld16(dOg + (size_t)myq * D + s * 2 * CW + CW * h) : u32x4{0, 0, 0, 0};
    }
    float lse2 = pos_inf(), del = 0.f;
    if (myq < N) {
      const float l = a.lse[(size_t)bh * N + myq];
      lse2 = (l == neg_inf()) ? pos_inf() : l * LOG2E;
      del = a.delta[(size_t)bh * N + myq];
    }
    f32x16 dq[TL::NB];
#pragma unroll
    for (int nb = 0; nb < TL::NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[nb][r] = 0.f;

    UnitRegs<T, D> uk, uv;
    auto gload = [&](int kb0) {
      unit_load<T, D>(uk, Kg, kb0, N);
      unit_load<T, D>(uv, Vg, kb0, N);
    };
    auto stage_ptr = [&](int st) { return smem + (CF::NSTAGE == 2 ? st : 0) * SB; };
    auto swrite = [&](int st) {
      T* Ks = reinterpret_cast<T*>(stage_ptr(st));
      T* Vs = Ks + TL::ROW_ELEMS;
      T* Kt = Vs + TL::ROW_ELEMS;
      unit_store<T, D>(uk, Ks, Kt);
      unit_store<T, D>(uv, Vs, (T*)nullptr);
    };

    if (walk.ntiles > 0) {
      gload(walk.tile_start(0));
      swrite(0);
    }
    __syncthreads();

    for (int it = 0; it < walk.ntiles; ++it) {
      const int kb0 = walk.tile_start(it);
      const bool has_next = it + 1 < walk.ntiles;
      if (has_next) gload(walk.tile_start(it + 1));
      const T* Ks = reinterpret_cast<const T*>(stage_ptr(it & 1));
      const T* Vs = Ks + TL::ROW_ELEMS;
      const T* Kt = Vs + TL::ROW_ELEMS;

      const bool active = wave_has_rows && !(a.causal && kb0 > qw0 + 31);
      if (active) {
        const bool edge = (kb0 + 64 > kvl) || (a.causal && kb0 + 63 > qw0);
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          // S^T = K Q^T and dP^T = V dO^T for 32 keys x this wave's 32 queries
          f32x16 s, dp;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            s[r] = 0.f;
            dp[r] = 0.f;
          }
          const T* krow = Ks + (32 * sb + l32) * TL::RP + CW * h;
          const T* vrow = Vs + (32 * sb + l32) * TL::RP + CW * h;
#pragma unroll
          for (int st = 0; st < TL::SSTEPS; ++st) {
            mma_chunk(s, ld16(krow + st * 2 * CW), qf[st], (T*)nullptr);
            mma_chunk(dp, ld16(vrow + st * 2 * CW), gf[st], (T*)nullptr);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.c, -lse2));
            if (edge) {
              const int key = kb0 + 32 * sb + 8 * (r >> 2) + 4 * h + (r & 3);
              if (key >= kvl || (a.causal && key > myq)) p = 0.f;
            }
            dp[r] = p * (dp[r] - del);
          }
          // dQ^T += K^T dS^T
#pragma unroll
          for (int nb = 0; nb < TL::NB; ++nb) mma_from_transposed<T, D>(dq[nb], Kt, nb, sb, dp);
        }
      }
      if (CF::NSTAGE == 1) __syncthreads();
      if (has_next) swrite((it + 1) & 1);
      __syncthreads();
    }
    store_acc_rows<T, D>(reinterpret_cast<T*>(a.out0) + head, myq, N, dq, a.scale);
  }
}

// ---------------------------------------------------------------- launchers

template <typename T, int D>
static hipError_t launch_pre_t(const AttnArgs& a, hipStream_t s) {
  constexpr int RPB = NT / pre_threads_per_row<T, D>();
  const long long rows = (long long)a.B * a.H * a.N;
  const long long nblk = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)nblk), dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_dkdv_t(const AttnArgs& a, bool walk_only, hipStream_t s) {
  const long long nwg = (long long)((a.N + CELL - 1) / CELL) * a.H * a.B;
  if (walk_only)
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, true>), dim3((unsigned)nwg), dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, false>), dim3((unsigned)nwg), dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_dq_t(const AttnArgs& a, bool walk_only, hipStream_t s) {
  const long long nwg = (long long)((a.N + CELL - 1) / CELL) * a.H * a.B;
  if (walk_only)
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, true>), dim3((unsigned)nwg), dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, false>), dim3((unsigned)nwg), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_pre(const AttnArgs& a, int dtype, int d, hipStream_t s) {
  if (dtype == 0) {
    switch (d) {
      case 64: return launch_pre_t<bf16, 64>(a, s);
      case 96: return launch_pre_t<bf16, 96>(a, s);
      case 160: return launch_pre_t<bf16, 160>(a, s);
      case 256: return launch_pre_t<bf16, 256>(a, s);
      default: return launch_pre_t<bf16, 128>(a, s);
    }
  }
  return d == 64 ? launch_pre_t<float, 64>(a, s) : launch_pre_t<float, 128>(a, s);
}

hipError_t launch_bwd_dkdv(const AttnArgs& a, int dtype, int d, bool walk_only, hipStream_t s) {
  if (dtype == 0) return launch_dkdv_bf16(a, d, walk_only, s);
  return d == 64 ? launch_dkdv_t<float, 64>(a, walk_only, s) : launch_dkdv_t<float, 128>(a, walk_only, s);
}

hipError_t launch_bwd_dq(const AttnArgs& a, int dtype, int d, bool walk_only, hipStream_t s) {
  if (dtype == 0) return launch_dq_bf16(a, d, walk_only, s);
  return d == 64 ? launch_dq_t<float, 64>(a, walk_only, s) : launch_dq_t<float, 128>(a, walk_only, s);
}

}  // namespace fa
