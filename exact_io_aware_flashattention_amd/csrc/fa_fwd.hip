// Forward kernel: O = softmax(scale * Q K^T [masked]) V and lse, one
// work-group per (batch, head, 128-query cell).
//
// Per 64-key tile (FlashAttention reading guide, "Metode", steps 1-4):
//   step 1  S^T = K Q^T on the matrix cores (scores of 32 queries per wave);
//   step 2  row maximum of the tile (lane-local + one half-wave exchange);
//   step 3  running maximum / normaliser update (the merge of "Pelacakan
//           Softmax Inkremental");
//   step 4  O^T += V^T P~^T with the running output rescaled by
//           exp(m_old - m_new).
// The division by l is done once at the end instead of at every step (the
// two are equal in exact arithmetic), and the running maximum is refreshed
// only when a tile exceeds it by more than 2^TAU: between refreshes the
// exponentials stay below 2^TAU and both l and O carry the same reference,
// so the result is unchanged while most tiles skip the O rescale.
//
// Memory: the Q fragments of a wave live in registers for the whole walk;
// K and V tiles are double-buffered in LDS (K row-major, V transposed so the
// second product reads 4 consecutive keys per lane), prefetched into
// registers one tile ahead so the global loads overlap the matrix work.
#include "fa_device.hpp"
#include "fa_kernels.hpp"
#include "fa_walk.hpp"

namespace fa {

template <typename T, int D>
struct FwdTile {
  static constexpr int BC = 64;                    // keys per tile
  static constexpr int CW = ET<T>::CW;             // elements per 16-byte chunk
  static constexpr int KP = D + 16 / (int)sizeof(T);  // K row pitch in LDS (elements)
  static constexpr int VP = BC + 4;                // V^T row pitch in LDS (elements)
  static constexpr int K_ELEMS = BC * KP;
  static constexpr int V_ELEMS = D * VP;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int CPR = D / CW;               // 16-byte chunks per row
  static constexpr int KCH = BC * CPR / NT;        // K chunks staged per thread
  static constexpr int VUNITS = (BC / 4) * CPR;    // (4 keys x 1 chunk) units of V
  static constexpr int VU = (VUNITS + NT - 1) / NT;
  static constexpr int SSTEPS = D / (2 * CW);      // chunk steps of the score product
  static constexpr int NB = D / 32;                // 32-wide blocks of the head dim
  static_assert(BC * CPR % NT == 0, "K staging must divide evenly");
};

template <typename T, int D, bool WALK_ONLY>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(Occ<T>::W, Occ<T>::W))) void fwd_kernel(AttnArgs a) {
  using TL = FwdTile<T, D>;
  constexpr int CW = TL::CW;
  __shared__ __attribute__((aligned(16))) T smem[WALK_ONLY ? 8 : 2 * TL::STAGE];
  __shared__ int cell_list[MAX_T];
  __shared__ int scratch4[4];

  const int N = a.N;
  const int T_cells = (N + CELL - 1) / CELL;
  const WorkUnit u = work_unit(blockIdx.x, gridDim.x, a.B * a.H, T_cells, a.causal);
  const int bh = u.bh;
  const int qi = a.causal ? T_cells - 1 - u.t : u.t;   // heaviest causal rows first
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
    const T* __restrict__ Q = reinterpret_cast<const T*>(a.q) + head;
    const T* __restrict__ K = reinterpret_cast<const T*>(a.k) + head;
    const T* __restrict__ V = reinterpret_cast<const T*>(a.v) + head;
    T* __restrict__ O = reinterpret_cast<T*>(a.out0) + head;

    const int qw0 = q_lo + wave * 32;    // first query of this wave
    const int myq = qw0 + l32;           // the query this lane owns
    const bool wave_has_rows = qw0 < N;

    u32x4 qf[TL::SSTEPS];
#pragma unroll
    for (int s = 0; s < TL::SSTEPS; ++s)
      qf[s] = (myq < N) ? ld16(Q + (size_t)myq * D + s * 2 * CW + CW * h) : u32x4{0, 0, 0, 0};

    f32x16 acc[TL::NB];
#pragma unroll
    for (int nb = 0; nb < TL::NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nb][r] = 0.f;
    float m_run = neg_inf();   // running max of scale*log2(e)*s (log2 units)
    float l_run = 0.f;         // this lane's share of the running normaliser

    u32x4 kreg[TL::KCH];
    u32x4 vreg[TL::VU][4];
    auto gload = [&](int kb0) {
#pragma unroll
      for (int i = 0; i < TL::KCH; ++i) {
        const int c = tid + i * NT, row = c / TL::CPR, cc = c - row * TL::CPR, key = kb0 + row;
        kreg[i] = key < N ? ld16(K + (size_t)key * D + cc * CW) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < TL::VU; ++u) {
        const int unit = tid + u * NT;
        if (unit < TL::VUNITS) {
          const int kg = unit % (TL::BC / 4), dc = unit / (TL::BC / 4);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kb0 + 4 * kg + r;
            vreg[u][r] = key < N ? ld16(V + (size_t)key * D + dc * CW) : u32x4{0, 0, 0, 0};
          }
        }
      }
    };
    auto swrite = [&](int stage) {
      T* Ks = smem + stage * TL::STAGE;
      T* Vt = Ks + TL::K_ELEMS;
#pragma unroll
      for (int i = 0; i < TL::KCH; ++i) {
        const int c = tid + i * NT, row = c / TL::CPR, cc = c - row * TL::CPR;
        st16(Ks + row * TL::KP + cc * CW, kreg[i]);
      }
#pragma unroll
      for (int u = 0; u < TL::VU; ++u) {
        const int unit = tid + u * NT;
        if (unit < TL::VUNITS) {
          const int kg = unit % (TL::BC / 4), dc = unit / (TL::BC / 4);
          write_transposed4(Vt + (dc * CW) * TL::VP + 4 * kg, TL::VP, vreg[u]);
        }
      }
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
      const T* Ks = smem + (it & 1) * TL::STAGE;
      const T* Vt = Ks + TL::K_ELEMS;

      // A wave whose queries all precede the tile (causal) has nothing to add.
      const bool active = wave_has_rows && !(a.causal && kb0 > qw0 + 31);
      if (active) {
        // step 1: S^T for the two 32-key halves of the tile
        f32x16 s[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) s[sb][r] = 0.f;
          const T* krow = Ks + (32 * sb + l32) * TL::KP + CW * h;
#pragma unroll
          for (int st = 0; st < TL::SSTEPS; ++st) mma_chunk(s[sb], ld16(krow + st * 2 * CW), qf[st], (T*)nullptr);
        }
        // masks inside partial tiles (causal diagonal, key padding, tail)
        const bool edge = (kb0 + TL::BC > kvl) || (a.causal && kb0 + TL::BC - 1 > qw0);
        if (edge) {
#pragma unroll
          for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kb0 + 32 * sb + 8 * (r >> 2) + 4 * h + (r & 3);
              if (key >= kvl || (a.causal && key > myq)) s[sb][r] = neg_inf();
            }
        }
        // step 2: tile row max
        float mx = neg_inf();
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sb][r]);
        mx = max_halves(mx);
        const float mt = mx * a.c;
        // step 3: refresh the running max (and rescale) only when needed
        if (wave_any(mt > m_run + TAU)) {
          const float m_new = fmaxf(m_run, mt);
          const float alpha = (m_new == neg_inf()) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
          l_run *= alpha;
#pragma unroll
          for (int nb = 0; nb < TL::NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[nb][r] *= alpha;
          m_run = m_new;
        }
        const float mu = (m_run == neg_inf()) ? 0.f : m_run;
        float ls = 0.f;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][r], a.c, -mu));
            s[sb][r] = p;
            ls += p;
          }
        l_run += ls;
        // step 4: O^T += V^T P~^T
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
          for (int nb = 0; nb < TL::NB; ++nb) {
            Quad<T> vq[4];
            const T* vrow = Vt + (32 * nb + l32) * TL::VP + 32 * sb + 4 * h;
#pragma unroll
            for (int g = 0; g < 4; ++g) vq[g].load(vrow + 8 * g);
            mma_acc_operand(acc[nb], vq, s[sb]);
          }
        }
      }
      if (has_next) swrite((it + 1) & 1);
      __syncthreads();
    }

    // epilogue: O = O / l, lse = (m + log2 l) ln 2
    const float l_tot = sum_halves(l_run);
    if (myq < N) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      T* orow = O + (size_t)myq * D;
#pragma unroll
      for (int nb = 0; nb < TL::NB; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          store4(orow + 32 * nb + 8 * g + 4 * h, acc[nb][4 * g] * inv, acc[nb][4 * g + 1] * inv,
                 acc[nb][4 * g + 2] * inv, acc[nb][4 * g + 3] * inv);
      if (h == 0) a.lse[(size_t)bh * N + myq] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * LN2 : neg_inf();
    }
  }
}

template <typename T, int D>
static hipError_t launch_fwd_t(const AttnArgs& a, bool walk_only, hipStream_t s) {
  const int T_cells = (a.N + CELL - 1) / CELL;
  const long long nwg = (long long)T_cells * a.H * a.B;
  if (walk_only)
    hipLaunchKernelGGL((fwd_kernel<T, D, true>), dim3((unsigned)nwg), dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_kernel<T, D, false>), dim3((unsigned)nwg), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fwd(const AttnArgs& a, int dtype, int d, bool walk_only, hipStream_t s) {
  if (dtype == 0) return launch_fwd_bf16(a, d, walk_only, s);
  return d == 64 ? launch_fwd_t<float, 64>(a, walk_only, s) : launch_fwd_t<float, 128>(a, walk_only, s);
}

}  // namespace fa
