// Split-key forward for a few queries per head (decoding, Nq <= 4).
//
// Decoding reads every key and value of a head once for one (or a handful
// of) queries: about one flop per byte, far below the matrix cores' ridge
// point, so the kernel is built for HBM bandwidth rather than for the MFMA
// tiles of the attention kernels.  Each wave is an independent unit of work
// -- one key range of one (b, h) -- and runs the incremental softmax of the
// forward pass (FlashAttention reading guide, "Metode" steps 2-4, division by
// l deferred) over its range; its unnormalised partial output and (m, l) are
// combined with the other ranges by the merge kernel (the two-block rule of
// "Pelacakan Softmax Inkremental").  Splitting one head over many waves is the
// sequence-length parallelism the pages motivate for small-batch inference
// (datacamp "Penjelasan Flash Attention", Flash Attention 2, "Paralelisme
// sepanjang panjang sekuens").
//
// Data movement.  A key row of d bf16 is d/8 16-byte chunks, served by LPR
// lanes (d/8 rounded up to a power of two); one load instruction of a wave
// covers 64 / LPR whole consecutive rows (1 KB contiguous when d is a power
// of two), lane l taking chunk l % LPR of row l / LPR.  Lanes past a row's
// last chunk (d = 96, 160) load from past the end of the buffer, read zeros
// and add nothing.  A block is G
// such loads of K and G of V; the next block's loads are issued before the
// current block is computed, so each wave keeps 2 G KB in flight and needs no
// LDS and no barrier.  Loads go through a buffer resource whose size ends at
// the range's last allowed key, so a ragged last block reads zeros, and are
// marked non-temporal.
//
// Arithmetic.  q . k of a row: each lane forms the dot product of its chunk
// with the query's chunk (bf16 pairs, fp32 accumulation), then the d/8 lanes
// of the row add their partial sums by DPP lane exchanges, after which every
// lane of the row holds the row's score.  P V: each lane accumulates p times
// its 8 features of V for the rows it holds; the rows of a wave are summed
// once at the end.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_kernels.hpp"
#include "fa_tile.hpp"

namespace fa {
namespace {

// F8: K and V are E4M3 codes (one byte per feature) instead of bf16.
template <int D, bool F8>
struct DecCfg {
  static constexpr int RB = F8 ? D : 2 * D;   // bytes per key row
  static constexpr int EPL = F8 ? 16 : 8;     // features per lane (one 16-byte chunk)
  static constexpr int CPR = RB / 16;         // chunks per key row
  static constexpr int LPR = CPR <= 4 ? 4 : CPR <= 8 ? 8 : CPR <= 16 ? 16 : 32;   // lanes per key row
  static constexpr int KPI = 64 / LPR;        // key rows per load instruction
  static constexpr int G = 8;                 // load instructions per block and tensor
  static constexpr int KB = G * KPI;          // keys per block: 16 .. 64 (bf16), 32 .. 128 (E4M3)
};

// Cache policy of the K and V loads: non-temporal (each byte is read once).
// On this part streaming reads with it sustain about 7 TB/s, without it
// about 6 TB/s.
constexpr int kStream = 2;

// Sum over the LPR lanes of a key row; every lane of the row gets the same
// bits (each step adds a lane and its partner in both orders, which fp
// addition's commutativity makes equal).
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  auto xch = [](float v, auto ctrl) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), decltype(ctrl)::value, 0xf, 0xf, false));
  };
  x += xch(x, std::integral_constant<int, 0xB1>());    // quad_perm [1,0,3,2]: lane ^ 1
  x += xch(x, std::integral_constant<int, 0x4E>());    // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (LPR >= 8) x += xch(x, std::integral_constant<int, 0x141>());    // row_half_mirror: 7 - lane
  if constexpr (LPR >= 16) x += xch(x, std::integral_constant<int, 0x140>());   // row_mirror: 15 - lane
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16);                                  // the other row of 16
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

// (Vector elements are copied to scalars before __builtin_bit_cast: the
// compiler used here reads element 0 for a bit cast of the lvalue a[i].)
__device__ __forceinline__ float dot8(u32x4 a, u32x4 b, float acc) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t ai = a[i], bi = b[i];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, ai), __builtin_bit_cast(b2, bi), acc, false);
  }
  return acc;
}

// q . k over one lane's 16 E4M3 features (16 c .. 16 c + 15) of a key row:
// each byte pair becomes a bf16 pair exactly (E4M3 values are bf16 values)
// and meets the matching bf16 pair of the query, q[u] holding features
// 16 c + 8 u .. + 7.
__device__ __forceinline__ float dot16_e4m3(u32x4 k, const u32x4 (&q)[2], float acc) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t kw = k[w];
    const uint32_t q0 = q[w >> 1][2 * (w & 1)], q1 = q[w >> 1][2 * (w & 1) + 1];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kw, 1.0f, false),
                                          __builtin_bit_cast(b2, q0), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kw, 1.0f, true),
                                          __builtin_bit_cast(b2, q1), acc, false);
  }
  return acc;
}

template <int D, int NQ, bool F8>
__global__ __launch_bounds__(NT) void decode_kernel(AttnArgs a) {
  using C = DecCfg<D, F8>;
  const int lane = threadIdx.x & 63;
  const long long gw = (long long)blockIdx.x * (NT / 64) + wave_id();   // wave-uniform
  const int BH = a.B * a.H, S = a.nsplit;
  if (gw >= (long long)S * BH) return;   // whole waves only; no barrier follows
  const int split = (int)(gw % S), bh = (int)(gw / S);
  const int b = bh / a.H;
  const int Nq = a.N, NK = a.Nk;
  const int r = lane / C::LPR, c = lane % C::LPR;
  const bool pad = c >= C::CPR;   // a lane past the row's last chunk (d = 96, 160)

  // key j is allowed for query i iff j < lim[i]
  const int kvl = a.kv_len ? min(max(a.kv_len[b], 0), NK) : NK;
  int lim[NQ];
  int lim_lo = kvl, lim_hi = 0;
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    lim[i] = i < Nq ? (a.causal ? min(kvl, max(i + a.causal_off + 1, 0)) : kvl) : 0;
    if (i < Nq) lim_lo = min(lim_lo, lim[i]);
    lim_hi = max(lim_hi, lim[i]);
  }
  const int R = a.split_tiles * 64;
  const int k_lo = split * R, k_hi = min(k_lo + R, lim_hi);
  // A block (KB keys) can reach past the range when KB > 64 (E4M3 at d = 64):
  // keys at or past k_hi read as zeros and must be masked like disallowed keys.
  lim_lo = min(lim_lo, k_hi);
#pragma unroll
  for (int i = 0; i < NQ; ++i) lim[i] = min(lim[i], k_hi);

  const bf16* Qh = reinterpret_cast<const bf16*>(a.q) + (size_t)bh * Nq * D;
  u32x4 qv[NQ][C::EPL / 8];   // features EPL c .. EPL c + EPL - 1 of each query
#pragma unroll
  for (int i = 0; i < NQ; ++i)
#pragma unroll
    for (int u = 0; u < C::EPL / 8; ++u)
      qv[i][u] = i < Nq && !pad ? ld16(Qh + (size_t)i * D + C::EPL * c + 8 * u) : u32x4{0, 0, 0, 0};

  float m_run[NQ], neg_mu[NQ], thr[NQ], l_run[NQ], acc[NQ][C::EPL];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    m_run[i] = neg_inf();
    neg_mu[i] = 0.f;
    thr[i] = neg_inf();
    l_run[i] = 0.f;
#pragma unroll
    for (int e = 0; e < C::EPL; ++e) acc[i][e] = 0.f;
  }
  const float inv_c = 1.f / a.c;

  if (k_lo < k_hi) {
    const size_t head = (size_t)bh * NK * C::RB;   // bytes
    const uint32_t bytes = (uint32_t)k_hi * C::RB;
    const __amdgpu_buffer_rsrc_t rsK = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(reinterpret_cast<const unsigned char*>(a.k) + head), (short)0, (int)bytes,
        0x00020000);
    const __amdgpu_buffer_rsrc_t rsV = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(reinterpret_cast<const unsigned char*>(a.v) + head), (short)0, (int)bytes,
        0x00020000);
    const int voff0 = r * C::RB + 16 * c;
    // pad lanes: an offset past the range (bytes <= PAD_OFF), read as zeros
    auto offset = [&](int j) { return pad ? (int)PAD_OFF : voff0 + j * C::RB; };

    u32x4 kA[C::G], vA[C::G], kB[C::G], vB[C::G];
    auto load = [&](u32x4 (&kb)[C::G], u32x4 (&vb)[C::G], int j0) {
#pragma unroll
      for (int g = 0; g < C::G; ++g)
        kb[g] = __builtin_amdgcn_raw_buffer_load_b128(rsK, offset(j0 + g * C::KPI), 0, kStream);
#pragma unroll
      for (int g = 0; g < C::G; ++g)
        vb[g] = __builtin_amdgcn_raw_buffer_load_b128(rsV, offset(j0 + g * C::KPI), 0, kStream);
    };
    auto compute = [&](const u32x4 (&kb)[C::G], const u32x4 (&vb)[C::G], int j0) {
      float s[NQ][C::G];
      const bool full = j0 + C::KB <= lim_lo;   // no key of the block is masked for any query
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
#pragma unroll
        for (int g = 0; g < C::G; ++g) {
          if constexpr (F8)
            s[i][g] = row_sum<C::LPR>(dot16_e4m3(kb[g], qv[i], 0.f));
          else
            s[i][g] = row_sum<C::LPR>(dot8(kb[g], qv[i][0], 0.f));
          if (!full && j0 + g * C::KPI + r >= lim[i]) s[i][g] = neg_inf();
        }
        float mx = s[i][0];
#pragma unroll
        for (int g = 1; g < C::G; ++g) mx = fmaxf(mx, s[i][g]);
        // lazy running max: move it only when a score passes it by 2^TAU
        if (wave_any(mx > thr[i])) {
          const float m_new = fmaxf(m_run[i], wave_max(mx) * a.c);
          const float alpha = (m_new == neg_inf()) ? 1.f : __builtin_amdgcn_exp2f(m_run[i] - m_new);
          l_run[i] *= alpha;
#pragma unroll
          for (int e = 0; e < C::EPL; ++e) acc[i][e] *= alpha;
          m_run[i] = m_new;
          const bool live = m_new != neg_inf();
          neg_mu[i] = live ? -m_new : 0.f;
          thr[i] = live ? (m_new + TAU) * inv_c : neg_inf();
        }
      }
#pragma unroll
      for (int g = 0; g < C::G; ++g) {
        float v[C::EPL];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = vb[g][e];
          if constexpr (F8) {   // E4M3 features 16 c + 4 e .. + 3
            typedef float f2 __attribute__((ext_vector_type(2)));
            const f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false), hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
            v[4 * e] = lo[0];
            v[4 * e + 1] = lo[1];
            v[4 * e + 2] = hi[0];
            v[4 * e + 3] = hi[1];
          } else {   // bf16 features 8c + 2e (low half), 8c + 2e + 1 (high half)
            const uint32_t lo = w << 16, hi = w & 0xffff0000u;
            v[2 * e] = __builtin_bit_cast(float, lo);
            v[2 * e + 1] = __builtin_bit_cast(float, hi);
          }
        }
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i][g], a.c, neg_mu[i]));
          l_run[i] += p;
#pragma unroll
          for (int e = 0; e < C::EPL; ++e) acc[i][e] = __builtin_fmaf(p, v[e], acc[i][e]);
        }
      }
    };

    load(kA, vA, k_lo);
    for (int j0 = k_lo;;) {
      if (j0 + C::KB < k_hi) load(kB, vB, j0 + C::KB);
      compute(kA, vA, j0);
      j0 += C::KB;
      if (j0 >= k_hi) break;
      if (j0 + C::KB < k_hi) load(kA, vA, j0 + C::KB);
      compute(kB, vB, j0);
      j0 += C::KB;
      if (j0 >= k_hi) break;
    }
  }

  // Sum the rows of the wave: lanes c, c + LPR, c + 2 LPR, ... hold the same
  // features for different keys; every lane of a row holds the same p, so l
  // is counted once per row.
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
#pragma unroll
    for (int o = C::LPR; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < C::EPL; ++e) acc[i][e] += __shfl_xor(acc[i][e], o);
    const float l_tot = wave_sum(c == 0 ? l_run[i] : 0.f);
    if (i < Nq) {
      const size_t prow = ((size_t)split * BH + bh) * Nq + i;
      if (r == 0 && !pad) {
        // the value descale (E4M3 V) is applied here, so the merge is shared
        const float vs = F8 ? a.v_descale : 1.f;
        float* po = a.part_o + prow * D + C::EPL * c;
#pragma unroll
        for (int e = 0; e < C::EPL; e += 4)
          *reinterpret_cast<f32x4*>(po + e) =
              f32x4{acc[i][e] * vs, acc[i][e + 1] * vs, acc[i][e + 2] * vs, acc[i][e + 3] * vs};
      }
      if (lane == 0) *reinterpret_cast<float2*>(a.part_ml + 2 * prow) = float2{m_run[i], l_tot};
    }
  }
}

template <int D, int NQ, bool F8>
hipError_t launch_decode(const AttnArgs& a, hipStream_t s) {
  const long long waves = (long long)a.B * a.H * a.nsplit;
  const long long nwg = (waves + NT / 64 - 1) / (NT / 64);
  hipLaunchKernelGGL((decode_kernel<D, NQ, F8>), dim3((unsigned)nwg), dim3(NT), 0, s, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_splitkv_merge(a, D, s);
}

template <int D, bool F8>
hipError_t launch_decode_d(const AttnArgs& a, hipStream_t s) {
  if (a.N <= 1) return launch_decode<D, 1, F8>(a, s);
  if (a.N <= 2) return launch_decode<D, 2, F8>(a, s);
  return launch_decode<D, 4, F8>(a, s);
}

template <bool F8>
hipError_t launch_decode_any(const AttnArgs& a, int d, hipStream_t s) {
  switch (d) {
    case 64: return launch_decode_d<64, F8>(a, s);
    case 96: return launch_decode_d<96, F8>(a, s);
    case 160: return launch_decode_d<160, F8>(a, s);
    case 256: return launch_decode_d<256, F8>(a, s);
    default: return launch_decode_d<128, F8>(a, s);
  }
}

}  // namespace

hipError_t launch_fwd_decode_bf16(const AttnArgs& a, int d, hipStream_t s) { return launch_decode_any<false>(a, d, s); }

hipError_t launch_fwd_decode_e4m3kv(const AttnArgs& a, int d, hipStream_t s) { return launch_decode_any<true>(a, d, s); }

}  // namespace fa
