// Forward pass on FP8 (OCP E4M3) Q, K and V with per-tensor descale factors.
//
// FlashAttention-3 computes attention on 8-bit floating point inputs, halving
// the memory traffic of bf16 (datacamp "Penjelasan Flash Attention", Flash
// Attention 3, "Presisi FP8 native").  Here both products run on the gfx950
// fp8 matrix core (v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 operands, unit
// block scales, fp32 accumulation): S^T = K Q^T exactly (products of E4M3
// values are exact in fp32), and O^T += V^T P~^T with the probabilities P~
// converted to E4M3.  The running max, row sum and the division by it are
// fp32, as in the bf16 forward (FlashAttention reading guide, "Metode" steps
// 2-4, division by l deferred); the descales enter the exponent factor
// (scale * dq * dk * log2 e) and the final division (dv / l).
//
// Operand layouts (32x32x64: lane (i, h) = (lane % 32, lane / 32) supplies
// contraction indices 32 h .. 32 h + 31 of row i of A, and of column i of B):
//   * S^T: A lane i takes K row rho(i) of the 32-key sub-block, with
//     rho(i) = 16 ((i >> 2) & 1) + 4 (i >> 3) + (i & 3), so accumulator
//     register r of lane half h holds key 16 h + r (the 32x32 accumulator row
//     of register r is 8 (r / 4) + 4 h + r % 4); B lane q takes Q row q.  The
//     bytes of one contraction step are 32 contiguous features, the same for
//     A and B, so any assignment of features to steps is a valid product.
//   * P~ (B of the PV product, 64 keys = two sub-blocks): byte b of lane half
//     h is key 32 (b / 16) + 16 h + b % 16, i.e. registers 0..15 of the two
//     sub-blocks in order, packed with v_cvt_pk_fp8_f32.
//   * V^T (A of the PV product): lane (f, h) needs V[key][f] for the same 32
//     keys -- four 8-row column segments.  ds_read_b64_tr_b8 returns them:
//     in a group of 16 lanes, lane u < 8 receives byte u of the 8 bytes that
//     the even lanes 0, 2, .., 14 address (one byte per source lane, in
//     order), and lane u >= 8 byte u - 8 of those the odd lanes address; so
//     source lane s addresses row (8-row segment base + s / 2), 8-byte column
//     chunk 16 (G & 1) + 8 (s & 1) of the feature block.
// K and V tiles (64 keys x d bytes) reach LDS by buffer-to-LDS loads with an
// XOR swizzle of 16-byte chunks per row, one per tile kind, chosen so that the
// 16 rows of a K row read and the 8 rows of a V transposed read fall on
// distinct bank positions.
#include "fa_device.hpp"
#include "fa_kernels.hpp"
#include "fa_tile.hpp"
#include "fa_walk.hpp"

#include <type_traits>

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int acc_row8(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

template <int D>
struct F8 {
  static constexpr int TILE = 64 * D;    // bytes of a 64-key K or V tile
  static constexpr int KS = D / 64;      // contraction steps of the score product
  static constexpr int NB = D / 32;      // 32-feature blocks of O
  static constexpr int CPR = D / 16;     // 16-byte chunks per row
  static constexpr int RPL = 1024 / D;   // rows per wave-wide load
  // K tile: rows rho(0..15) (and rho(16..31)) at one logical chunk must hit
  // 16 distinct (row within the 256-byte bank line, chunk) positions
  __host__ __device__ static constexpr int swk(int r) {
    return D == 128 ? (((r >> 1) & 3) | (((r >> 4) & 1) << 2)) : (((r >> 2) & 1) | (((r >> 4) & 1) << 1));
  }
  // V tile: 8 consecutive rows at one logical chunk must hit 8 distinct positions
  __host__ __device__ static constexpr int swv(int r) { return D == 128 ? ((r >> 1) & 3) : ((r >> 2) & 1); }
  // waves per SIMD the compiler is asked for: three at d = 128 (168 registers;
  // 6 % faster than two), and at d = 64 the kernel's 109 registers already let
  // four waves share a SIMD
  static constexpr int OCC = D == 128 ? 3 : 2;
};

// Loads of a 64-row tile of one kind (V = false: K swizzle, true: V swizzle),
// spread over the 4 waves; both swizzles repeat every 4 * RPL rows, so the
// per-lane offsets are computed once.
template <int D, bool V>
struct Dma8 {
  using C = F8<D>;
  static constexpr int NJ = 64 / C::RPL / 4;
  int voff[NJ];
  __device__ __forceinline__ Dma8() {
    const int lane = threadIdx.x & 63, wave = wave_id();
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int lr = (j * 4 + wave) * C::RPL + lane / C::CPR;
      const int c = (lane % C::CPR) ^ (V ? C::swv(lr) : C::swk(lr));
      voff[j] = lr * D + 16 * c;
    }
  }
  // rows [row0, row0 + 64) of head (N rows of D bytes); rows past N read as zeros
  __device__ __forceinline__ void load(const void* head, int N, int row0, unsigned char* lds) const {
    const u32x4 rsrc = rows_rsrc(head, N, D / 2, row0);   // D / 2 bf16 = D bytes per row
    const int wave = wave_id();
#pragma unroll
    for (int j = 0; j < NJ; ++j) dma16(rsrc, lds + (j * 4 + wave) * 1024, voff[j]);
  }
};

__device__ __forceinline__ void mma8(f32x16& acc, i32x8 a, i32x8 b) {
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ float max16f(const f32x16& s) {
  float m = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) m = fmaxf(m, s[r]);
  return m;
}

template <int D>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(F8<D>::OCC, F8<D>::OCC))) void fwd_fp8_kernel(AttnArgs a) {
  using C = F8<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char kbuf[2 * C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vbuf[2 * C::TILE];
  __shared__ int cell_list[MAX_T];
  __shared__ int scratch4[4];

  const int N = a.N;
  const int T_cells = (N + CELL - 1) / CELL;
  const WorkUnit u = work_unit(blockIdx.x, gridDim.x, a.B * a.H, T_cells, a.causal);
  const int bh = u.bh;
  const int qi = a.causal ? T_cells - 1 - u.t : u.t;   // heaviest causal rows first
  const int b = bh / a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int h = lane >> 5, l32 = lane & 31;

  const int kvl = clamp_kv_len(a, b);
  const int q_lo = qi * CELL, q_hi = min(q_lo + CELL, N);
  const int kv_end = a.causal ? min(kvl, q_hi) : kvl;
  const Walk walk = row_walk(a, qi, kv_end, T_cells, cell_list, scratch4, 6);

  const size_t head = (size_t)bh * N * D;
  const unsigned char* Q = reinterpret_cast<const unsigned char*>(a.q) + head;
  const unsigned char* Kh = reinterpret_cast<const unsigned char*>(a.k) + head;
  const unsigned char* Vh = reinterpret_cast<const unsigned char*>(a.v) + head;
  const Dma8<D, false> kdma;
  const Dma8<D, true> vdma;

  const int qw0 = q_lo + wave * 32;
  const int myq = qw0 + l32;
  const int ntiles = walk.ntiles;

  i32x8 qf[C::KS];   // Q row myq, features 64 ks + 32 h .. +31
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    u32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
    if (myq < N) {
      x = ld16(Q + (size_t)myq * D + 64 * ks + 32 * h);
      y = ld16(Q + (size_t)myq * D + 64 * ks + 32 * h + 16);
    }
    qf[ks] = i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
  }
  f32x16 acc[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[nb][r] = 0.f;
  float m_run = neg_inf(), l_run = 0.f, neg_mu = 0.f, thr = neg_inf();
  const float inv_c = 1.f / a.c;

  const int krow = 16 * ((l32 >> 2) & 1) + 4 * (l32 >> 3) + (l32 & 3);   // rho(l32)
  const int G = lane >> 4, us = lane & 15;

  if (ntiles > 0) {
    kdma.load(Kh, N, walk.tile_start(0), kbuf);
    vdma.load(Vh, N, walk.tile_start(0), vbuf);
  }
  // One 64-key tile j held in LDS stage STG.  The walk is unrolled by two
  // tiles so the stage is a compile-time constant and every LDS address a
  // per-lane base plus an immediate.
  auto tile_step = [&](int j, auto stg) {
    constexpr int STG = decltype(stg)::value;
    wait_loads_all();
    __syncthreads();
    if (j + 1 < ntiles) {
      const int nxt = walk.tile_start(j + 1);
      kdma.load(Kh, N, nxt, kbuf + (1 - STG) * C::TILE);
      vdma.load(Vh, N, nxt, vbuf + (1 - STG) * C::TILE);
    }
    const unsigned char* kt = kbuf + STG * C::TILE;
    const unsigned char* vt = vbuf + STG * C::TILE;
    const int k0 = walk.tile_start(j);

    // S^T of the two 32-key sub-blocks: register r of lane half h = key k0 + 32 sb + 16 h + r
    f32x16 s[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[sb][r] = 0.f;
      const int row = 32 * sb + krow;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const int c0 = 4 * ks + 2 * h;
        const u32x4 x = *reinterpret_cast<const u32x4*>(kt + row * D + 16 * (c0 ^ C::swk(row)));
        const u32x4 y = *reinterpret_cast<const u32x4*>(kt + row * D + 16 * ((c0 + 1) ^ C::swk(row)));
        mma8(s[sb], i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]},
             qf[ks]);
      }
    }
    // mask (key at or past kv_len, or past the query under the causal mask)
    if ((k0 + 64 > kvl) || (a.causal && k0 + 63 > qw0)) {
      const int lim = min(kvl, a.causal ? myq + 1 : kvl) - k0 - 16 * h;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * sb + r >= lim) s[sb][r] = neg_inf();
    }
    // lazy running max: moved only when a score passes it by 2^TAU, so the
    // probabilities stay below 2^TAU = 256, inside E4M3's range (448)
    const float lane_mx = fmaxf(max16f(s[0]), max16f(s[1]));
    if (wave_any(lane_mx > thr)) {
      const float mx = max_halves(lane_mx);
      const float m_new = fmaxf(m_run, mx * a.c);
      const float alpha = (m_new == neg_inf()) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[nb][r] *= alpha;
      m_run = m_new;
      const bool live = m_new != neg_inf();
      neg_mu = live ? -m_new : 0.f;
      thr = live ? (m_new + TAU) * inv_c : neg_inf();
    }
    // P~ = exp2(s c - m), its row sum (fp32), and the E4M3 operand
    i32x8 pk;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[sb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][r], a.c, neg_mu));
        l_run += s[sb][r];
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        unsigned x = __builtin_amdgcn_cvt_pk_fp8_f32(s[sb][4 * w], s[sb][4 * w + 1], 0u, false);
        x = __builtin_amdgcn_cvt_pk_fp8_f32(s[sb][4 * w + 2], s[sb][4 * w + 3], x, true);
        pk[4 * sb + w] = (int)x;
      }
    }
    // O^T += V^T P~^T, V^T read down the key rows of the P~ operand
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
      const int c = 2 * nb + (G & 1);
      i32x8 va;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int row = 32 * (t >> 1) + 16 * h + 8 * (t & 1) + (us >> 1);
        typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
        const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (lds_i32x2*)(vt + row * D + 16 * (c ^ C::swv(row)) + 8 * (us & 1)));
        va[2 * t] = x[0];
        va[2 * t + 1] = x[1];
      }
      mma8(acc[nb], va, pk);
    }
  };
  for (int j = 0; j < ntiles; j += 2) {
    tile_step(j, std::integral_constant<int, 0>());
    if (j + 1 < ntiles) tile_step(j + 1, std::integral_constant<int, 1>());
  }

  const float l_tot = sum_halves(l_run);
  if (myq < N) {
    const float inv = l_tot > 0.f ? a.v_descale / l_tot : 0.f;
    bf16* orow = reinterpret_cast<bf16*>(a.out0) + (size_t)bh * N * D + (size_t)myq * D;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4(orow + 32 * nb + 8 * g + 4 * h, acc[nb][4 * g] * inv, acc[nb][4 * g + 1] * inv,
               acc[nb][4 * g + 2] * inv, acc[nb][4 * g + 3] * inv);
    if (h == 0) a.lse[(size_t)bh * N + myq] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * LN2 : neg_inf();
  }
}

}  // namespace

hipError_t launch_fwd_fp8(const AttnArgs& a, int d, hipStream_t s) {
  const long long nwg = (long long)((a.N + CELL - 1) / CELL) * a.H * a.B;
  if (d == 64)
    hipLaunchKernelGGL((fwd_fp8_kernel<64>), dim3((unsigned)nwg), dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<128>), dim3((unsigned)nwg), dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace fa
