// bf16 kernels: forward, dK/dV and dQ.
//
// The arithmetic is the same as in the float kernels (fa_fwd.hip, fa_bwd.hip):
//   forward  FlashAttention reading guide, "Metode" steps 1-4, with the
//            division by l deferred to the end and a lazily refreshed row max;
//   backward dV = P^T dO, dP = dO V^T, dS = P (dP - delta), dQ = scale dS K,
//            dK = scale dS^T Q, recomputing S and P from lse (reading guide,
//            "Ide Utama", recomputation bullet).
// What differs is how tiles reach the matrix cores on gfx950: every K, V, Q
// and dO tile travels HBM -> LDS by buffer-to-LDS loads (no register staging,
// no LDS writes by the waves), is stored once, row-major and swizzled, and is
// read back either by rows (ds_read_b128) or transposed (ds_read_b64_tr_b16)
// for the products that contract over the tile rows.  Up to d = 128 all three
// kernels run at least two waves per SIMD (at most 256 registers per wave) so
// one wave's softmax and mask work overlaps another wave's matrix-core work;
// the forward and dQ at d = 64 run three.
// Head dimensions: multiples of 32 from 64 to 256 (instantiated: 64, 96, 128,
// 160, 256); a dimension that is not a power of two uses the LDS tile layout
// of the next power of two (fa_tile.hpp) and the loops run over its D / 16
// contraction steps and D / 32 output blocks.
#include "fa_device.hpp"
#include "fa_kernels.hpp"
#include "fa_tile.hpp"
#include "fa_dropout.hpp"
#include "fa_walk.hpp"

#include <type_traits>

namespace fa {

// Scores of one 32 x 32 block in accumulator layout: register r of lane l
// belongs to the key/query pair (8*(r/4) + 4*h + r%4, l % 32).
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Kernel instances: the attention arithmetic, the tile walk alone (visit
// counters), or the arithmetic with dropout on P.
constexpr int K_PLAIN = 0, K_WALK = 1, K_DROP = 2, K_SPLITKV = 3;

// Scheduling hint for a branch-free region holding 16 MFMAs and the VALU work
// of one 32-key sub-block: alternate one MFMA with up to six VALU
// instructions, so that the VALU work of each wave is spread under the
// matrix-core work instead of bunching (about 2 % on the forward).
__device__ __forceinline__ void interleave_mfma_valu() {
#pragma unroll
  for (int g = 0; g < 16; ++g) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // VALU
  }
}
// The same for a region of NM MFMAs with up to NV VALU instructions after each.
template <int NM, int NV>
__device__ __forceinline__ void interleave_mfma_valu_n() {
#pragma unroll
  for (int g = 0; g < NM; ++g) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);   // VALU
  }
}

// Max of the 16 accumulator entries of a lane as a depth-3 tree of v_max3.
__device__ __forceinline__ float max16(const f32x16& s) {
  const float m0 = fmaxf(fmaxf(s[0], s[1]), s[2]), m1 = fmaxf(fmaxf(s[3], s[4]), s[5]);
  const float m2 = fmaxf(fmaxf(s[6], s[7]), s[8]), m3 = fmaxf(fmaxf(s[9], s[10]), s[11]);
  const float m4 = fmaxf(fmaxf(s[12], s[13]), s[14]);
  return fmaxf(fmaxf(fmaxf(m0, m1), m2), fmaxf(fmaxf(m3, m4), s[15]));
}

__device__ __forceinline__ void zero(f32x16& x) {
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = 0.f;
}

// ---------------------------------------------------------------- forward

template <int D>
struct FwdB {
  static constexpr int BC = 64;                 // keys per tile (one DMA unit of K or V)
  static constexpr int TILE = BC * BTile<D>::ROWB;   // LDS bytes of one K or V tile
  static constexpr int SSTEPS = D / 16;
  static constexpr int NB = D / 32;
  // waves per SIMD: three at d = 64 (<= 168 registers: the softmax VALU work
  // of one wave then has two others to overlap, and short walks hide their
  // start and end), two (<= 256 registers) up to d = 128; above, the
  // accumulation and operand registers need a single wave per SIMD
  static constexpr int OCC = D > 128 ? 1 : (D == 64 ? 3 : 2);
};

// Forward, software-pipelined over 32-key sub-blocks t = 0, 1, ... of the walk:
//   A(t): S(t+1) = K(t+1) Q^T on the matrix cores (K fragments read one phase
//         earlier) while the VALU turns S(t) into P~(t) (exp2, row sum, bf16);
//         V^T(t) fragments are read from LDS;
//   B(t): O^T += V^T(t) P~^T(t) on the matrix cores while the VALU masks S(t+1)
//         (edge steps only) and, above d = 128, takes its row max; K fragments
//         of t+2 are read.
// K and V tiles have separate two-deep LDS rings.  Per 64-key tile j there is
// one barrier and one DMA issue (K of tile j+2, V of tile j+1), so every tile
// is requested two sub-block steps before it is read.
template <int D, int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(FwdB<D>::OCC, FwdB<D>::OCC))) void fwd_bf16_kernel(
    AttnArgs a) {
  using C = FwdB<D>;
  constexpr bool WALK_ONLY = MODE == K_WALK, DROP = MODE == K_DROP, SPLITKV = MODE == K_SPLITKV;
  __shared__ u32x4 drop_xch[DROP ? NT : 1];
  __shared__ __attribute__((aligned(1024))) unsigned char kbuf[WALK_ONLY ? 16 : 2 * C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vbuf[WALK_ONLY ? 16 : 2 * C::TILE];
  __shared__ int cell_list[MAX_T];
  __shared__ int scratch4[4];

  const int N = a.N;                       // queries (and keys, unless SPLITKV)
  const int NK = SPLITKV ? a.Nk : N;       // keys
  const int off = SPLITKV ? a.causal_off : 0;   // causal: key <= query + off
  const int T_cells = (N + CELL - 1) / CELL;
  int bh, qi, split = 0;
  if constexpr (SPLITKV) {
    // work-group = (key range, head, query cell): ranges fastest, then heads,
    // then query cells, heaviest (last) causal cells first as in the plain
    // forward; the work-groups of one (head, range) sit nsplit * B * H apart.
    split = blockIdx.x % a.nsplit;
    const int L = blockIdx.x / a.nsplit, BH = a.B * a.H;
    const int t = L / BH;
    bh = L - t * BH;
    qi = a.causal ? T_cells - 1 - t : t;
  } else {
    const WorkUnit u = work_unit(blockIdx.x, gridDim.x, a.B * a.H, T_cells, a.causal);
    bh = u.bh;
    qi = a.causal ? T_cells - 1 - u.t : u.t;   // heaviest causal rows first
  }
  const int b = bh / a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int h = lane >> 5, l32 = lane & 31;

  const int kvl = SPLITKV ? (a.kv_len ? min(max(a.kv_len[b], 0), NK) : NK) : clamp_kv_len(a, b);
  const int q_lo = qi * CELL, q_hi = min(q_lo + CELL, N);
  const int kv_end = a.causal ? min(kvl, q_hi + off) : kvl;
  const Walk walk = SPLITKV ? range_walk(split * a.split_tiles,
                                         min((kv_end + 63) >> 6, (split + 1) * a.split_tiles) - split * a.split_tiles)
                            : row_walk(a, qi, kv_end, T_cells, cell_list, scratch4, 6);

  if constexpr (WALK_ONLY) {
    for (int it = 0; it < walk.ntiles; ++it)
      if (tid == 0 && walk.first_of_cell(it))
        atomicAdd(&a.counts[((size_t)b * T_cells + qi) * T_cells + walk.cell(it >> 1)], 1u);
    return;
  } else {
    const size_t head = (size_t)bh * N * D, khead = (size_t)bh * NK * D;
    const bf16* Q = reinterpret_cast<const bf16*>(a.q) + head;
    const bf16* Kh = reinterpret_cast<const bf16*>(a.k) + khead;
    const bf16* Vh = reinterpret_cast<const bf16*>(a.v) + khead;
    const TileDma<D, 64> dma;

    const int qw0 = q_lo + wave * 32;
    const int myq = qw0 + l32;
    const int ntiles = walk.ntiles, nsub = 2 * ntiles;
    // With few queries (decode) most waves of a split-key work-group hold no
    // query row: they still move their share of every tile but skip the math.
    const bool live = !SPLITKV || qw0 < N;

    u32x4 qf[C::SSTEPS];
#pragma unroll
    for (int s = 0; s < C::SSTEPS; ++s)
      qf[s] = (myq < N) ? ld16(Q + (size_t)myq * D + s * 16 + 8 * h) : u32x4{0, 0, 0, 0};
    f32x16 acc[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) zero(acc[nb]);
    // Running max m_run (log2 units), kept with the two values the tile loop
    // uses: neg_mu = -m_run (0 while m_run = -inf) enters every exponent, and
    // thr = (m_run + TAU) / c is the raw-score level above which the running
    // max must move (-inf while m_run = -inf).
    float m_run = neg_inf(), l_run = 0.f, neg_mu = 0.f, thr = neg_inf();
    const float inv_c = 1.f / a.c;

    auto issue_k = [&](int j) { dma.load(Kh, NK, walk.tile_start(j), kbuf + (j & 1) * C::TILE); };
    auto issue_v = [&](int j) { dma.load(Vh, NK, walk.tile_start(j), vbuf + (j & 1) * C::TILE); };
    auto key0 = [&](int t) { return walk.tile_start(t >> 1) + 32 * (t & 1); };

    u32x4 kfrag[C::SSTEPS];          // K rows of one sub-block: row l32, chunk 2 st + h
    bf16x8 vfrag[C::NB][2];          // V^T operands of one sub-block
    // Stage and half are compile-time constants so every LDS address is a
    // per-lane base plus an immediate offset.
    auto read_k = [&](auto stage, auto half) {
      const unsigned char* ks = kbuf + decltype(stage)::value * C::TILE;
#pragma unroll
      for (int st = 0; st < C::SSTEPS; ++st)
        kfrag[st] = row_chunk<D>(ks, 32 * decltype(half)::value + l32, 2 * st + h);
    };
    auto read_v = [&](auto stage, auto half) {
      const unsigned char* vs = vbuf + decltype(stage)::value * C::TILE;
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
          vfrag[nb][mm] = tr_operand<D>(vs, 32 * decltype(half)::value + 16 * mm, 32 * nb);
    };
    auto scores = [&](f32x16& s) {
      zero(s);
#pragma unroll
      for (int st = 0; st < C::SSTEPS; ++st) mma(s, as_bf16x8(kfrag[st]), as_bf16x8(qf[st]));
    };
    // Mask S(t) where needed and return the lane's raw max over its 16
    // entries (-inf past the walk).
    // Register r holds key k0 + acc_row(r, h), which is masked iff it is at or
    // past kv_len or (causal) past the lane's query: acc_row(r, 0) >= lim.
    auto mask_max = [&](f32x16& s, int t) -> float {
      if (t >= nsub) return neg_inf();
      const int k0 = key0(t);
      if ((k0 + 32 > kvl) || (a.causal && k0 + 31 > qw0 + off)) {
        const int lim = min(kvl, a.causal ? myq + 1 + off : kvl) - k0 - 4 * h;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (acc_row(r, 0) >= lim) s[r] = neg_inf();
      }
      return max16(s);
    };
    // The same mask without the max (every entry -inf past the walk).
    auto mask = [&](f32x16& s, int t) {
      if (t >= nsub) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = neg_inf();
        return;
      }
      mask_max(s, t);
    };
    // Refresh the running max only when a score exceeds it by more than 2^TAU.
    // The two lane halves hold different keys of the same query and share
    // thr, so the test needs only the lane's own max; the max over both
    // halves is formed inside the (rare) refresh.
    auto refresh = [&](float lane_mx) {
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
    };
    // Up to d = 128 the max test is replaced by a test of the row sum the
    // softmax forms anyway (SUMT): a lane's 16 probabilities of a sub-block,
    // relative to the running max, sum to at most lim = 2^TAU unless one of
    // its scores exceeds the running max by more than TAU (or several come
    // close); only then is the max formed, the running max moved and the
    // probabilities formed again.  An overflowed exponential makes the sum
    // +inf, which also triggers it; while m_run = -inf, lim = -1 sends every
    // sub-block through the refresh.  This saves the max tree of every
    // sub-block (1-3 % of the forward).  Above d = 128 the separate max test
    // is kept: there the extra probability registers turned the tile loop
    // into a divergent one.
    constexpr bool SUMT = D <= 128;
    constexpr float LIM = 256.f;
    static_assert(TAU == 8.f, "LIM = 2^TAU");
    float lim = -1.f;
    auto move_max = [&](float lane_mx) {
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
      lim = live ? LIM : -1.f;
    };
    // P~(t) from S(t) (in place), its row sum into l_run, and O^T += V^T P~^T.
    // (The row sum stays in fp32 VALU adds: v_dot2 on the packed bf16 values
    // would halve the instruction count but does not co-execute with the
    // matrix core.)  With dropout the row sum is of the kept and dropped
    // entries alike; dropped entries are then zeroed, and the 1 / (1 - p)
    // factor is applied with the final division by the row sum.
    const DropQuad dquad(drop_xch);
    // probabilities of S(t) into p (may be s itself) and the lane's row sum
    auto probs = [&](const f32x16& s, f32x16& p) -> float {
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.c, neg_mu));
      float t8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t8[i] = p[2 * i] + p[2 * i + 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) t8[i] += t8[i + 4];
      return (t8[0] + t8[2]) + (t8[1] + t8[3]);
    };
    // dropout on P~(t) in p, then O^T += V^T P~^T
    auto drop_pv = [&](f32x16& s, int t) {
      if constexpr (DROP) {
        // lane (l & 3) of the quad generates the block of key group (l & 3):
        // keys key0 + 8 (l & 3) + 4 h .. +3 x the quad's four queries
        const int gq = lane & 3;
        const u32x4 w = philox4x32_10((uint32_t)(key0(t) + 8 * gq + 4 * h) >> 2, (uint32_t)myq >> 2,
                                      (uint32_t)bh, 0u, a.drop_k0, a.drop_k1);
        const u32x4 keepw = dquad.exchange(w);   // word of group g for this lane's query
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!keep_byte(keepw[r >> 2], r & 3, a.drop_t)) s[r] = 0.f;
      }
      // keys 0-15 of the sub-block first, so the exponentials of keys 16-31
      // can overlap the first half of the products
      const PackedB pb = pack_bf16(s);
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) mma(acc[nb], vfrag[nb][mm], pb.p[mm]);
    };
    // max test form: P~(t) in place of S(t)
    auto softmax_pv = [&](f32x16& s, int t) {
      l_run += probs(s, s);
      drop_pv(s, t);
    };
    // sum test form (SUMT): S(t) is kept for a refresh; the region before the
    // test holds the scores of the next sub-block (hint_scores)
    auto softmax_pv_sum = [&](f32x16& s, int t) {
      f32x16 p;
      float psum = probs(s, p);
      interleave_mfma_valu_n<C::SSTEPS, (48 + C::SSTEPS - 1) / C::SSTEPS>();
      if (wave_any(psum > lim)) {
        move_max(max16(s));
        psum = probs(s, p);
      }
      l_run += psum;
      drop_pv(p, t);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    // One 64-key tile j held in LDS stage STG: sub-blocks 2j (in sa) and 2j+1.
    f32x16 sa, sb;
    auto tile_begin = [&](int j) {
      if (j > 0) wait_loads();     // K of tile j+1 and V of tile j, issued one tile ago
      __syncthreads();
      if (j + 2 < ntiles) issue_k(j + 2);
      if (j + 1 < ntiles) issue_v(j + 1);
    };
    // Sub-block t needs no mask: it exists and every key of it is below
    // kv_len and (causal) at or before every query of this wave.  Along a
    // walk the keys only grow, so the sub-blocks that need no mask are a
    // prefix of it.
    auto clean = [&](int t) -> bool {
      if (t >= nsub) return false;
      const int k0 = key0(t);
      return k0 + 32 <= kvl && (!a.causal || k0 + 31 <= qw0 + off);
    };
    // Tile step whose scores S(2j+1) and S(2j+2) need no mask (every tile but
    // the last one or two of a walk): each sub-block -- scores of the next
    // sub-block, softmax and P V of this one, row sum and max of the next --
    // is one branch-free region closed by the refresh test, so the row sum
    // and the max overlap the P V products.
    auto interior_step = [&](auto stg, int j) {
      constexpr int STG = decltype(stg)::value;
      using S0 = std::integral_constant<int, STG>;
      using S1 = std::integral_constant<int, 1 - STG>;
      tile_begin(j);
      if (!live) return;
      if constexpr (SUMT) {
        read_v(S0(), I0());
        scores(sb);
        softmax_pv_sum(sa, 2 * j);
        read_k(S1(), I0());
        interleave_mfma_valu_n<C::SSTEPS, 2>();
        read_v(S0(), I1());
        scores(sa);
        softmax_pv_sum(sb, 2 * j + 1);
        read_k(S1(), I1());
        interleave_mfma_valu_n<C::SSTEPS, 2>();
        return;
      }
      read_v(S0(), I0());
      scores(sb);
      softmax_pv(sa, 2 * j);
      read_k(S1(), I0());
      const float mx1 = max16(sb);
      interleave_mfma_valu();
      refresh(mx1);
      read_v(S0(), I1());
      scores(sa);
      softmax_pv(sb, 2 * j + 1);
      read_k(S1(), I1());
      const float mx2 = max16(sa);
      interleave_mfma_valu();
      refresh(mx2);
    };
    // Sub-blocks from nlive on hold no key that any query of this wave may
    // see (past the causal diagonal of the wave's last query, or wholly past
    // kv_len): their probabilities are exactly zero, so the edge steps skip
    // their products (the tile loads and barriers go on for the other waves).
    // Keys only grow along the walk, so they are a suffix of it.  Not in the
    // split-key instances (built with the skip, the d = 64 one returned wrong
    // values in the last two accumulator registers of rows that pass from the
    // interior to the edge steps, though those rows skip nothing; without it
    // it is exact) nor in the d = 256 dropout one (the branches cost spills).
    constexpr bool SKIP = (D <= 160 && !SPLITKV) || MODE == K_PLAIN;
    int nlive = nsub;
    if constexpr (SKIP) {
      const int klim = min(kvl, a.causal ? qw0 + 32 + off : kvl);   // first key no query of the wave sees
      while (nlive > 0 && key0(nlive - 1) >= klim) --nlive;
    }
    auto tile_step = [&](auto stg, int j) {
      constexpr int STG = decltype(stg)::value;
      using S0 = std::integral_constant<int, STG>;
      using S1 = std::integral_constant<int, 1 - STG>;
      tile_begin(j);
      if (!live) return;
      const bool l0 = !SKIP || 2 * j < nlive, l1 = !SKIP || 2 * j + 1 < nlive, l2 = !SKIP || 2 * j + 2 < nlive;
      if constexpr (SUMT) {
        read_v(S0(), I0());
        if (l1) scores(sb);
        if (l0) softmax_pv_sum(sa, 2 * j);
        read_k(S1(), I0());
        interleave_mfma_valu_n<C::SSTEPS, 2>();
        if (l1) mask(sb, 2 * j + 1);
        read_v(S0(), I1());
        if (l2) scores(sa);
        if (l1) softmax_pv_sum(sb, 2 * j + 1);
        read_k(S1(), I1());
        interleave_mfma_valu_n<C::SSTEPS, 2>();
        if (l2) mask(sa, 2 * j + 2);
        return;
      }
      // sub-block 2j: S(2j+1) while softmax(2j); then O += P~ V
      read_v(S0(), I0());
      if (l1) scores(sb);
      if (l0) softmax_pv(sa, 2 * j);
      read_k(S1(), I0());
      interleave_mfma_valu();
      if (l1) refresh(mask_max(sb, 2 * j + 1));
      // sub-block 2j+1: S(2j+2) (next tile) while softmax(2j+1)
      read_v(S0(), I1());
      if (l2) scores(sa);
      if (l1) softmax_pv(sb, 2 * j + 1);
      read_k(S1(), I1());
      interleave_mfma_valu();
      if (l2) refresh(mask_max(sa, 2 * j + 2));
    };

    if (nsub > 0) {
      issue_k(0);
      issue_v(0);
      if (ntiles > 1) issue_k(1);
      wait_loads();
      __syncthreads();
      if (live) {
        read_k(I0(), I0());
        scores(sa);
        read_k(I0(), I1());
        if constexpr (SUMT) {
          mask(sa, 0);
          move_max(max16(sa));
        } else {
          refresh(mask_max(sa, 0));
        }
      }
      // steps j and j + 1 are interior iff sub-block 2j + 4 needs no mask
      int j = 0;
      for (; clean(2 * j + 4); j += 2) {
        interior_step(I0(), j);
        interior_step(I1(), j + 1);
      }
      for (; j < ntiles; j += 2) {
        tile_step(I0(), j);
        if (j + 1 < ntiles) tile_step(I1(), j + 1);
      }
    }

    const float l_tot = sum_halves(l_run);
    if constexpr (SPLITKV) {
      // partial result of this key range: unnormalised O (relative to m_run)
      // and (m_run in log2 units, l); the merge kernel combines the ranges
      if (myq < N) {
        const size_t prow = ((size_t)split * a.B * a.H + bh) * N + myq;
        float* po = a.part_o + prow * D;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<f32x4*>(po + 32 * nb + 8 * g + 4 * h) =
                f32x4{acc[nb][4 * g], acc[nb][4 * g + 1], acc[nb][4 * g + 2], acc[nb][4 * g + 3]};
        if (h == 0) *reinterpret_cast<float2*>(a.part_ml + 2 * prow) = float2{m_run, l_tot};
      }
      return;
    }
    if (myq < N) {
      const float inv = l_tot > 0.f ? (DROP ? a.drop_inv : 1.f) / l_tot : 0.f;
      bf16* orow = reinterpret_cast<bf16*>(a.out0) + head + (size_t)myq * D;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          store4(orow + 32 * nb + 8 * g + 4 * h, acc[nb][4 * g] * inv, acc[nb][4 * g + 1] * inv,
                 acc[nb][4 * g + 2] * inv, acc[nb][4 * g + 3] * inv);
      if (h == 0) a.lse[(size_t)bh * N + myq] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * LN2 : neg_inf();
    }
  }
}

// ---------------------------------------------------------------- dK / dV

template <int D>
struct DkdvB {
  static constexpr int BQ = D > 64 ? 32 : 64;       // queries per stage
  static constexpr int TSH = D > 64 ? 5 : 6;
  static constexpr int QS = BQ / 32;
  static constexpr int TILE = BQ * BTile<D>::ROWB;  // one Q or dO tile (LDS bytes)
  static constexpr int STAGE = 2 * TILE + 2 * BQ * 4;   // Q, dO, lse*log2e, delta
  static constexpr int VRES = CELL * BTile<D>::ROWB;    // V of the work-group's 128 keys
  static constexpr int SSTEPS = D / 16;
  static constexpr int NB = D / 32;
  // waves per SIMD: above d = 128 one wave holds dK, dV (up to 256
  // accumulator registers at d = 256) and K in its 512 registers
  static constexpr int OCC = D > 128 ? 1 : 2;
};

// SPLIT (block mask present): work-groups [0, SPLIT_MAX_ITEMS) take the split
// items of the plan (a chunk of a long column each; surplus ones exit), the
// rest take one column each and exit if the column is split.
template <int D, int MODE, bool SPLIT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(DkdvB<D>::OCC, DkdvB<D>::OCC))) void
dkdv_bf16_kernel(AttnArgs a) {
  using C = DkdvB<D>;
  constexpr bool WALK_ONLY = MODE == K_WALK, DROP = MODE == K_DROP;
  __shared__ u32x4 drop_xch[DROP ? NT : 1];
  constexpr int VRES = C::VRES;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[WALK_ONLY ? 16 : VRES + 2 * C::STAGE];
  __shared__ int cell_list[MAX_T];
  __shared__ int scratch4[4];

  const int N = a.N;
  const int T_cells = (N + CELL - 1) / CELL;
  const bool split_item = SPLIT && blockIdx.x < (unsigned)SPLIT_MAX_ITEMS;
  int bh, kj, c0 = 0, ch = 0;   // split item: the chunk's first cell and CH
  if (split_item) {
    const int g = blockIdx.x;
    if (g >= a.split.hdr[0]) return;
    const int P = a.split.hdr[1];
    ch = a.split.hdr[2];
    bh = g / P;
    const int r = g - bh * P;
    const int* e = a.split.table + 4 * r;
    kj = e[0];
    c0 = (r - e[1]) * ch;
  } else {
    const int off = SPLIT ? SPLIT_MAX_ITEMS : 0;
    const WorkUnit u = work_unit(blockIdx.x - off, gridDim.x - off, a.B * a.H, T_cells, a.causal);
    bh = u.bh;
    kj = u.t;   // causal: low kj sees the most queries
  }
  const int b = bh / a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int h = lane >> 5, l32 = lane & 31;
  const int kvl = clamp_kv_len(a, b);
  int listed = 0;
  Walk walk = col_walk(a, kj, kvl, T_cells, cell_list, scratch4, C::TSH, &listed);
  if constexpr (SPLIT) {
    if (split_item)
      take_chunk(walk, c0, ch, N);
    else if (listed > a.split.hdr[2])
      return;   // the split items of this column cover it
  }

  if constexpr (WALK_ONLY) {
    for (int it = 0; it < walk.ntiles; ++it)
      if (tid == 0 && walk.first_of_cell(it))
        atomicAdd(&a.counts[((size_t)b * T_cells + walk.cell(it >> (7 - C::TSH))) * T_cells + kj], 1u);
    return;
  } else {
    const size_t head = (size_t)bh * N * D;
    const bf16* Kg = reinterpret_cast<const bf16*>(a.k) + head;
    const float* lse_g = a.lse + (size_t)bh * N;
    const float* del_g = a.delta + (size_t)bh * N;
    const bf16* Qh = reinterpret_cast<const bf16*>(a.q) + head;
    const bf16* dOh = reinterpret_cast<const bf16*>(a.dO) + head;
    const TileDma<D, C::BQ> dma;

    const int kw0 = kj * CELL + wave * 32;   // first key of this wave
    const int myk = kw0 + l32;               // the key this lane owns
    const bool wave_has_keys = kw0 < kvl;
    unsigned char* Vs = smem;

    u32x4 kf[C::SSTEPS];
#pragma unroll
    for (int s = 0; s < C::SSTEPS; ++s)
      kf[s] = myk < N ? ld16(Kg + (size_t)myk * D + s * 16 + 8 * h) : u32x4{0, 0, 0, 0};
    // Up to d = 96 the wave's V rows stay in registers (16 or 24 per lane)
    // after the first tile instead of being read from LDS for every query
    // tile (d = 96 dK/dV 1-3 % faster).  At d = 128 the 32 more registers
    // spill inside the loop (measured 4-8 % slower), so V is read from LDS.
    constexpr bool VREG = D <= 96;
    u32x4 vfr[VREG ? C::SSTEPS : 1];
    f32x16 dk[C::NB], dv[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
      zero(dk[nb]);
      zero(dv[nb]);
    }

    // This thread's row statistics of the next tile, as loaded.  Nothing
    // may wait for these loads inside the current tile: counted in order, a
    // wait for them is also a wait for the tile loads issued just before.
    // So they are converted only at the next tile, and they take their
    // address from a scalar buffer resource and a loop-invariant lane offset
    // (a per-tile address register that a later LDS read reuses makes the
    // compiler wait for the loads first).  Rows past N read 0 and are
    // treated at the conversion.
    float st_l = 0.f, st_d = 0.f;
    int st_q = 0;
    auto issue = [&](int it) {
      unsigned char* st = smem + VRES + (it & 1) * C::STAGE;
      const int q0 = walk.tile_start(it);
      dma.load(Qh, N, q0, st);
      dma.load(dOh, N, q0, st + C::TILE);
      if (tid < C::BQ) {
        st_q = q0 + tid;
        const int bytes = (N - q0) * 4;
        st_l = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
            __builtin_amdgcn_make_buffer_rsrc((void*)(lse_g + q0), (short)0, bytes, 0x00020000), tid * 4, 0, 0));
        st_d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
            __builtin_amdgcn_make_buffer_rsrc((void*)(del_g + q0), (short)0, bytes, 0x00020000), tid * 4, 0, 0));
      }
    };
    if (walk.ntiles > 0) {
      TileDma<D, CELL>().load(reinterpret_cast<const bf16*>(a.v) + head, N, kj * CELL, Vs);
      issue(0);
    }

    // The leading tiles of the walk may hold masked entries for some wave
    // (the diagonal cell under a causal mask; every tile when the work-group's
    // keys straddle kv_len).  Up to d = 128 they run the masked body and the
    // rest a body with no mask code, one basic block from the first product to
    // the last, walked in pairs of tiles with compile-time LDS stages (1-7 %
    // faster at d = 64 to 128 than one masked loop).  At d = 128 the dropout
    // and block-mask instances keep one masked loop (the split form spills
    // there, and measured 1 % slower with dropout); above d = 128 every tile
    // takes the masked body.
    constexpr bool PLAIN_LOOP = D < 128 || (D == 128 && !DROP && !SPLIT);
    int n_edge = 0;
    if (!PLAIN_LOOP || kj * CELL + CELL > kvl)
      n_edge = walk.ntiles;
    else if (a.causal)
      while (n_edge < walk.ntiles && walk.tile_start(n_edge) < kj * CELL + CELL - 1) ++n_edge;

    auto tile = [&](int it, auto plain_c, auto stage_c) {
      constexpr bool PLAIN = decltype(plain_c)::value && !DROP;
      constexpr int STG = decltype(stage_c)::value;   // LDS stage, or -1: it & 1
      wait_loads_all();
      unsigned char* st = smem + VRES + (STG < 0 ? (it & 1) : STG) * C::STAGE;
      float* stats = reinterpret_cast<float*>(st + 2 * C::TILE);
      if (tid < C::BQ) {
        // empty rows and rows past N get P = 0
        stats[tid] = (st_q >= N || st_l == neg_inf()) ? pos_inf() : st_l * LOG2E;
        stats[C::BQ + tid] = st_q < N ? st_d : 0.f;
      }
      __syncthreads();
      if constexpr (VREG) {
        if (it == 0) {   // the wave's V rows, resident in LDS since the first barrier
#pragma unroll
          for (int k = 0; k < C::SSTEPS; ++k) vfr[k] = row_chunk<D>(Vs, wave * 32 + l32, 2 * k + h);
        }
      }
      if (it + 1 < walk.ntiles) issue(it + 1);
      const int q0 = walk.tile_start(it);
      const unsigned char* Qs = st;
      const unsigned char* dOs = st + C::TILE;
      if constexpr (PLAIN) {
        // with two 32-query halves (d = 64) both halves' S and dP products
        // come first, so the vector work of the first half runs under the
        // products of the second (dK/dV 2-6 % faster at d = 64)
        f32x16 s[C::QS], dp[C::QS];
#pragma unroll
        for (int qs = 0; qs < C::QS; ++qs) {
          zero(s[qs]);
          zero(dp[qs]);
#pragma unroll
          for (int k = 0; k < C::SSTEPS; ++k) {
            mma(s[qs], as_bf16x8(row_chunk<D>(Qs, 32 * qs + l32, 2 * k + h)), as_bf16x8(kf[k]));
            mma(dp[qs], as_bf16x8(row_chunk<D>(dOs, 32 * qs + l32, 2 * k + h)),
                as_bf16x8(VREG ? vfr[k] : row_chunk<D>(Vs, wave * 32 + l32, 2 * k + h)));
          }
        }
#pragma unroll
        for (int qs = 0; qs < C::QS; ++qs) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(stats + 32 * qs + 8 * g + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              s[qs][4 * g + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qs][4 * g + e], a.c, -l4[e]));
          }
          const PackedB pb = pack_bf16(s[qs]);
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
            for (int mm = 0; mm < 2; ++mm) mma(dv[nb], tr_operand<D>(dOs, 32 * qs + 16 * mm, 32 * nb), pb.p[mm]);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(stats + C::BQ + 32 * qs + 8 * g + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) dp[qs][4 * g + e] = s[qs][4 * g + e] * (dp[qs][4 * g + e] - d4[e]);
          }
          const PackedB db = pack_bf16(dp[qs]);
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
            for (int mm = 0; mm < 2; ++mm) mma(dk[nb], tr_operand<D>(Qs, 32 * qs + 16 * mm, 32 * nb), db.p[mm]);
        }
        return;
      }
      if (!wave_has_keys || (a.causal && kw0 > q0 + C::BQ - 1)) return;
      const bool edge = (kw0 + 32 > kvl) || (a.causal && kw0 + 31 > q0);
#pragma unroll
      for (int qs = 0; qs < C::QS; ++qs) {
        if (C::QS > 1 && a.causal && q0 + 32 * qs + 31 < kw0) continue;   // every query before every key
        // S = Q K^T and dP = dO V^T: 32 queries x this wave's 32 keys (lane = key)
        f32x16 s, dp;
        zero(s);
        zero(dp);
#pragma unroll
        for (int k = 0; k < C::SSTEPS; ++k) {
          mma(s, as_bf16x8(row_chunk<D>(Qs, 32 * qs + l32, 2 * k + h)), as_bf16x8(kf[k]));
          mma(dp, as_bf16x8(row_chunk<D>(dOs, 32 * qs + l32, 2 * k + h)),
              as_bf16x8(VREG ? vfr[k] : row_chunk<D>(Vs, wave * 32 + l32, 2 * k + h)));
        }
        // P = exp2(s c - lse log2 e), dS = P (dP - delta); register r <-> query
        // q0 + 32 qs + acc_row(r, h).  On edge tiles an entry is masked iff the
        // lane's key is at or past kv_len, or (causal) the key is past the
        // query: acc_row(r, 0) < lim.
        u32x4 keepw;   // dropout: byte m of word g keeps query q0 + 32 qs + 8 g + 4 h + m
        if constexpr (DROP) {
          // lane (l & 3) of the quad (4 consecutive keys) generates the block
          // of query group (l & 3) and turns it key-major for the exchange
          const int gq = lane & 3;
          const u32x4 w = philox4x32_10((uint32_t)myk >> 2, (uint32_t)(q0 + 32 * qs + 8 * gq + 4 * h) >> 2,
                                        (uint32_t)bh, 0u, a.drop_k0, a.drop_k1);
          keepw = DropQuad(drop_xch).exchange(byte_transpose4(w));
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int qq = 32 * qs + 8 * g + 4 * h;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(stats + qq);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(stats + C::BQ + qq);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.c, -l4[e]));
            if constexpr (DROP) {
              // dV uses P Z (the 1 / (1 - p) factor is applied at the end);
              // dS = P ((dO V^T) Z - delta)
              const bool keep = keep_byte(keepw[g], e, a.drop_t);
              dp[r] = s[r] * ((keep ? dp[r] * a.drop_inv : 0.f) - d4[e]);
              if (!keep) s[r] = 0.f;
            } else {
              dp[r] = s[r] * (dp[r] - d4[e]);
            }
          }
        }
        if (edge) {   // a masked entry has P = 0 and so dS = 0
          const int lim = myk >= kvl ? CELL : (a.causal ? myk - q0 - 32 * qs - 4 * h : -1);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (acc_row(r, 0) < lim) s[r] = dp[r] = 0.f;
        }
        // dV^T += dO^T P and dK^T += Q^T dS, the transposed operands read from the row-major tiles
        const PackedB pb = pack_bf16(s), db = pack_bf16(dp);
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
          for (int mm = 0; mm < 2; ++mm) {
            mma(dv[nb], tr_operand<D>(dOs, 32 * qs + 16 * mm, 32 * nb), pb.p[mm]);
            mma(dk[nb], tr_operand<D>(Qs, 32 * qs + 16 * mm, 32 * nb), db.p[mm]);
          }
      }
    };
    using RT = std::integral_constant<int, -1>;
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    int it = 0;
    if constexpr (PLAIN_LOOP) {
      for (; it < n_edge; ++it) tile(it, std::false_type(), RT());
      // the mask-free tiles with the LDS stage a compile-time constant, so
      // every LDS address is a per-lane base plus an immediate
      if ((it & 1) && it < walk.ntiles) tile(it++, std::true_type(), S1());
      for (; it + 1 < walk.ntiles; it += 2) {
        tile(it, std::true_type(), S0());
        tile(it + 1, std::true_type(), S1());
      }
      if (it < walk.ntiles) tile(it++, std::true_type(), S0());
    } else if constexpr (D > 128) {
      // pairs of tiles with the LDS stage a compile-time constant, so every
      // LDS address is a per-lane base plus an immediate (dK/dV 20 % faster at
      // d = 256, 28 % at d = 160)
      for (; it < walk.ntiles; it += 2) {
        tile(it, std::false_type(), S0());
        if (it + 1 < walk.ntiles) tile(it + 1, std::false_type(), S1());
      }
    } else {
      for (; it < walk.ntiles; ++it) tile(it, std::false_type(), RT());
    }

    if constexpr (SPLIT) {
      if (split_item) {
        // partial sums of this chunk -> slot [2][D/4][128 keys][4]; lanes of a
        // half write 512 contiguous bytes per store.  (Item data are read again
        // here rather than kept live through the main loop.)
        const int item = blockIdx.x, P = a.split.hdr[1];
        const int* e = a.split.table + 4 * (item - bh * P);
        const int first = bh * P + e[1], nchunk = e[2];
        const int kl = wave * 32 + l32;
        float* slot = a.split.slots + (size_t)item * (2 * CELL * D);
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const size_t o = ((size_t)(8 * nb + 2 * g + h) * CELL + kl) * 4;
            *reinterpret_cast<f32x4*>(slot + o) =
                f32x4{dk[nb][4 * g], dk[nb][4 * g + 1], dk[nb][4 * g + 2], dk[nb][4 * g + 3]};
            *reinterpret_cast<f32x4*>(slot + CELL * D + o) =
                f32x4{dv[nb][4 * g], dv[nb][4 * g + 1], dv[nb][4 * g + 2], dv[nb][4 * g + 3]};
          }
        __threadfence();   // release this thread's partials at device scope
        __syncthreads();
        if (tid == 0) scratch4[0] = atomicAdd(a.split.ctr + first, 1u) == (unsigned)(nchunk - 1);
        __syncthreads();
        if (!scratch4[0]) return;   // another chunk of the column finishes later
        __threadfence();   // acquire the other chunks' partials
        // the last chunk adds all partials of the column in chunk order
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          zero(dk[nb]);
          zero(dv[nb]);
        }
        for (int c = 0; c < nchunk; ++c) {
          const float* sl = a.split.slots + (size_t)(first + c) * (2 * CELL * D);
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const size_t o = ((size_t)(8 * nb + 2 * g + h) * CELL + kl) * 4;
              const f32x4 x = *reinterpret_cast<const f32x4*>(sl + o);
              const f32x4 y = *reinterpret_cast<const f32x4*>(sl + CELL * D + o);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                dk[nb][4 * g + e] += x[e];
                dv[nb][4 * g + e] += y[e];
              }
            }
        }
      }
    }
    if (myk < N) {
      bf16* dkp = reinterpret_cast<bf16*>(a.out0) + head + (size_t)myk * D;
      bf16* dvp = reinterpret_cast<bf16*>(a.out1) + head + (size_t)myk * D;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = 32 * nb + 8 * g + 4 * h;
          store4(dkp + c, dk[nb][4 * g] * a.scale, dk[nb][4 * g + 1] * a.scale, dk[nb][4 * g + 2] * a.scale,
                 dk[nb][4 * g + 3] * a.scale);
          const float vs = DROP ? a.drop_inv : 1.f;
          store4(dvp + c, dv[nb][4 * g] * vs, dv[nb][4 * g + 1] * vs, dv[nb][4 * g + 2] * vs,
                 dv[nb][4 * g + 3] * vs);
        }
    }
  }
}

// ---------------------------------------------------------------- dQ

template <int D>
struct DqB {
  static constexpr int BC = 64;
  static constexpr int TILE = BC * BTile<D>::ROWB;
  static constexpr int STAGE = 2 * TILE;        // K, V
  static constexpr int SSTEPS = D / 16;
  static constexpr int NB = D / 32;
  // waves per SIMD: three at d = 64 (the kernel fits in 168 registers
  // without spilling; 8-13 % faster than two on d = 64 shapes), two up to
  // d = 128, one above
  static constexpr int OCC = D == 64 ? 3 : D > 128 ? 1 : 2;
};

template <int D, int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(DqB<D>::OCC, DqB<D>::OCC))) void dq_bf16_kernel(
    AttnArgs a) {
  using C = DqB<D>;
  constexpr bool WALK_ONLY = MODE == K_WALK, DROP = MODE == K_DROP;
  __shared__ u32x4 drop_xch[DROP ? NT : 1];
  __shared__ __attribute__((aligned(1024))) unsigned char smem[WALK_ONLY ? 16 : 2 * C::STAGE];
  __shared__ int cell_list[MAX_T];
  __shared__ int scratch4[4];

  const int N = a.N;
  const int T_cells = (N + CELL - 1) / CELL;
  const WorkUnit u = work_unit(blockIdx.x, gridDim.x, a.B * a.H, T_cells, a.causal);
  const int bh = u.bh;
  const int qi = a.causal ? T_cells - 1 - u.t : u.t;
  const int b = bh / a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int h = lane >> 5, l32 = lane & 31;
  const int kvl = clamp_kv_len(a, b);
  const int q_lo = qi * CELL, q_hi = min(q_lo + CELL, N);
  const int kv_end = a.causal ? min(kvl, q_hi) : kvl;
  const Walk walk = row_walk(a, qi, kv_end, T_cells, cell_list, scratch4, 6);

  if constexpr (WALK_ONLY) {
    for (int it = 0; it < walk.ntiles; ++it)
      if (tid == 0 && walk.first_of_cell(it))
        atomicAdd(&a.counts[((size_t)b * T_cells + qi) * T_cells + walk.cell(it >> 1)], 1u);
    return;
  } else {
    const size_t head = (size_t)bh * N * D;
    const bf16* Qg = reinterpret_cast<const bf16*>(a.q) + head;
    const bf16* dOg = reinterpret_cast<const bf16*>(a.dO) + head;
    const bf16* Kh = reinterpret_cast<const bf16*>(a.k) + head;
    const bf16* Vh = reinterpret_cast<const bf16*>(a.v) + head;
    const TileDma<D, 64> dma;

    const int qw0 = q_lo + wave * 32;
    const int myq = qw0 + l32;
    const bool wave_has_rows = qw0 < N;

    u32x4 qf[C::SSTEPS], gf[C::SSTEPS];
#pragma unroll
    for (int s = 0; s < C::SSTEPS; ++s) {
      const bool ok = myq < N;
      qf[s] = ok ? ld16(Qg + (size_t)myq * D + s * 16 + 8 * h) : u32x4{0, 0, 0, 0};
      gf[s] = ok ? ld16(dOg + (size_t)myq * D + s * 16 + 8 * h) : u32x4{0, 0, 0, 0};
    }
    float lse2 = pos_inf(), del = 0.f;
    if (myq < N) {
      const float l = a.lse[(size_t)bh * N + myq];
      lse2 = (l == neg_inf()) ? pos_inf() : l * LOG2E;
    }
    if (a.o) {
      // delta_i = dO_i . O_i of this lane's row, formed here and stored for
      // the dK/dV stage: the two lane halves hold alternate 8-element chunks
      // of the row, as for dO, so each sums its half in fp32 and the halves
      // are added
      const bf16* Og = reinterpret_cast<const bf16*>(a.o) + head;
      float part = 0.f;
#pragma unroll
      for (int s = 0; s < C::SSTEPS; ++s) {
        const u32x4 o4 = myq < N ? ld16(Og + (size_t)myq * D + s * 16 + 8 * h) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          part = __builtin_fmaf(__uint_as_float(o4[w] << 16), __uint_as_float(gf[s][w] << 16), part);
          part = __builtin_fmaf(__uint_as_float(o4[w] & 0xffff0000u), __uint_as_float(gf[s][w] & 0xffff0000u), part);
        }
      }
      del = sum_halves(part);
      if (myq < N && h == 0) a.delta[(size_t)bh * N + myq] = del;
    } else if (myq < N) {
      del = a.delta[(size_t)bh * N + myq];
    }
    f32x16 dq[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) zero(dq[nb]);

    auto issue = [&](int it) {
      unsigned char* st = smem + (it & 1) * C::STAGE;
      const int kb0 = walk.tile_start(it);
      dma.load(Kh, N, kb0, st);
      dma.load(Vh, N, kb0, st + C::TILE);
    };
    if (walk.ntiles > 0) issue(0);

    // The trailing tiles of the walk may hold masked entries for some wave
    // (the diagonal cell under a causal mask, the tile that straddles
    // kv_len).  Up to d = 128 the tiles before them run a body with no mask
    // code, one basic block over both 32-key halves, software-pipelined
    // across the halves (dQ 3-5 % faster at d = 64 than one masked loop; the
    // pipelining 1-2 % at d = 64 and 128, 4 % at d = 96).
    constexpr bool PLAIN_LOOP = D <= 128;
    int n_plain = PLAIN_LOOP ? walk.ntiles : 0;
    while (n_plain > 0 && (walk.tile_start(n_plain - 1) + C::BC > kvl ||
                           (a.causal && walk.tile_start(n_plain - 1) + C::BC - 1 > q_lo)))
      --n_plain;

    auto tile = [&](int it, auto plain_c, auto stage_c) {
      constexpr bool PLAIN = decltype(plain_c)::value && !DROP;
      constexpr int STG = decltype(stage_c)::value;   // LDS stage, or -1: it & 1
      wait_loads_all();
      __syncthreads();
      if (it + 1 < walk.ntiles) issue(it + 1);
      const int kb0 = walk.tile_start(it);
      const unsigned char* Ks = smem + (STG < 0 ? (it & 1) : STG) * C::STAGE;
      const unsigned char* Vs = Ks + C::TILE;
      if (!wave_has_rows) return;
      if constexpr (PLAIN) {
        // both halves' S and dP products first, so that the exponentials and
        // dS of the first half run under the products of the second, and its
        // dQ products under the second half's vector work
        f32x16 s[2], dp[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          zero(s[sb]);
          zero(dp[sb]);
#pragma unroll
          for (int k = 0; k < C::SSTEPS; ++k) {
            mma(s[sb], as_bf16x8(row_chunk<D>(Ks, 32 * sb + l32, 2 * k + h)), as_bf16x8(qf[k]));
            mma(dp[sb], as_bf16x8(row_chunk<D>(Vs, 32 * sb + l32, 2 * k + h)), as_bf16x8(gf[k]));
          }
        }
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) s[sb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][r], a.c, -lse2));
#pragma unroll
          for (int r = 0; r < 16; ++r) dp[sb][r] = s[sb][r] * (dp[sb][r] - del);
          const PackedB db = pack_bf16(dp[sb]);
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
            for (int mm = 0; mm < 2; ++mm) mma(dq[nb], tr_operand<D>(Ks, 32 * sb + 16 * mm, 32 * nb), db.p[mm]);
        }
        if constexpr (D == 128) {
          // the first half's products alone, the second half's under the
          // first half's vector work, then the first half's dQ products
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * C::SSTEPS, 0);
          interleave_mfma_valu_n<2 * C::SSTEPS, 4>();
          interleave_mfma_valu_n<2 * C::NB, 8>();
        }
        return;
      }
      if (a.causal && kb0 > qw0 + 31) return;
      const bool edge = (kb0 + C::BC > kvl) || (a.causal && kb0 + C::BC - 1 > qw0);
      // the second 32-key half holds no key that a query of this wave sees
      const bool half1_dead = kb0 + 32 >= kvl || (a.causal && kb0 + 32 > qw0 + 31);
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        if (sb == 1 && half1_dead) break;
        // S^T = K Q^T and dP^T = V dO^T: 32 keys x this wave's 32 queries (lane = query)
        f32x16 s, dp;
        zero(s);
        zero(dp);
#pragma unroll
        for (int k = 0; k < C::SSTEPS; ++k) {
          mma(s, as_bf16x8(row_chunk<D>(Ks, 32 * sb + l32, 2 * k + h)), as_bf16x8(qf[k]));
          mma(dp, as_bf16x8(row_chunk<D>(Vs, 32 * sb + l32, 2 * k + h)), as_bf16x8(gf[k]));
        }
        // register r holds key kb0 + 32 sb + acc_row(r, h): masked iff at or
        // past kv_len or (causal) past the lane's query, i.e. acc_row(r, 0) >= lim
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.c, -lse2));
        if (edge) {
          const int lim = min(kvl, a.causal ? myq + 1 : kvl) - kb0 - 32 * sb - 4 * h;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (acc_row(r, 0) >= lim) s[r] = 0.f;
        }
        if constexpr (DROP) {
          // as in the forward: lane (l & 3) generates key group (l & 3) of the
          // quad's four queries; dS = P ((dO V^T) Z - delta)
          const int gq = lane & 3;
          const u32x4 w = philox4x32_10((uint32_t)(kb0 + 32 * sb + 8 * gq + 4 * h) >> 2, (uint32_t)myq >> 2,
                                        (uint32_t)bh, 0u, a.drop_k0, a.drop_k1);
          const u32x4 keepw = DropQuad(drop_xch).exchange(w);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            dp[r] = s[r] * ((keep_byte(keepw[r >> 2], r & 3, a.drop_t) ? dp[r] * a.drop_inv : 0.f) - del);
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) dp[r] = s[r] * (dp[r] - del);
        }
        // dQ^T += K^T dS^T, K^T read transposed from the row-major tile
        const PackedB db = pack_bf16(dp);
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
          for (int mm = 0; mm < 2; ++mm) mma(dq[nb], tr_operand<D>(Ks, 32 * sb + 16 * mm, 32 * nb), db.p[mm]);
      }
    };
    using RT = std::integral_constant<int, -1>;
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    int it = 0;
    if constexpr (PLAIN_LOOP) {
      // the mask-free tiles with the LDS stage a compile-time constant (dQ
      // 1.5-5 % faster at d = 64 and 96)
      for (; it + 1 < n_plain; it += 2) {
        tile(it, std::true_type(), S0());
        tile(it + 1, std::true_type(), S1());
      }
      if (it < n_plain) tile(it++, std::true_type(), S0());
      for (; it < walk.ntiles; ++it) tile(it, std::false_type(), RT());
    } else {
      // pairs of tiles with the LDS stage a compile-time constant, so every
      // LDS address is a per-lane base plus an immediate (dQ 1.5 % faster at
      // d = 128, 8 % at d = 160 and 256)
      for (; it < walk.ntiles; it += 2) {
        tile(it, std::false_type(), S0());
        if (it + 1 < walk.ntiles) tile(it + 1, std::false_type(), S1());
      }
    }

    if (myq < N) {
      bf16* p = reinterpret_cast<bf16*>(a.out0) + head + (size_t)myq * D;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          store4(p + 32 * nb + 8 * g + 4 * h, dq[nb][4 * g] * a.scale, dq[nb][4 * g + 1] * a.scale,
                 dq[nb][4 * g + 2] * a.scale, dq[nb][4 * g + 3] * a.scale);
    }
  }
}

// ---------------------------------------------------------------- launchers

#define FA_DEFINE_LAUNCH(NAME, KERNEL)                                                                   \
  template <int D>                                                                                       \
  static hipError_t NAME(const AttnArgs& a, bool walk_only, hipStream_t s) {                            \
    const long long nwg = (long long)((a.N + CELL - 1) / CELL) * a.H * a.B;                              \
    if (walk_only)                                                                                       \
      hipLaunchKernelGGL((KERNEL<D, K_WALK>), dim3((unsigned)nwg), dim3(NT), 0, s, a);                   \
    else if (a.drop_t)                                                                                   \
      hipLaunchKernelGGL((KERNEL<D, K_DROP>), dim3((unsigned)nwg), dim3(NT), 0, s, a);                   \
    else                                                                                                 \
      hipLaunchKernelGGL((KERNEL<D, K_PLAIN>), dim3((unsigned)nwg), dim3(NT), 0, s, a);                  \
    return hipGetLastError();                                                                            \
  }

FA_DEFINE_LAUNCH(launch_fwd_b, fwd_bf16_kernel)
FA_DEFINE_LAUNCH(launch_dq_b, dq_bf16_kernel)

// dK/dV: with a block mask the split plan runs first and SPLIT_MAX_ITEMS
// work-groups for split items precede the per-column ones.
template <int D>
static hipError_t launch_dkdv_b(const AttnArgs& a, bool walk_only, hipStream_t s) {
  const long long ncol = (long long)((a.N + CELL - 1) / CELL) * a.H * a.B;
  const long long nwg = a.mask ? SPLIT_MAX_ITEMS + ncol : ncol;
  if (a.mask) {
    // (the plan also clears the arrival counters)
    const hipError_t e = launch_split_plan(a, s);
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)nwg), block(NT);
  if (walk_only) {
    if (a.mask)
      hipLaunchKernelGGL((dkdv_bf16_kernel<D, K_WALK, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((dkdv_bf16_kernel<D, K_WALK, false>), grid, block, 0, s, a);
    return hipGetLastError();
  }
  if (a.mask) {
    if (a.drop_t)
      hipLaunchKernelGGL((dkdv_bf16_kernel<D, K_DROP, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((dkdv_bf16_kernel<D, K_PLAIN, true>), grid, block, 0, s, a);
  } else {
    if (a.drop_t)
      hipLaunchKernelGGL((dkdv_bf16_kernel<D, K_DROP, false>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((dkdv_bf16_kernel<D, K_PLAIN, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

// Merge of the key ranges of a split-key forward (one thread per row and four
// output features): m = max_s m_s, w_s = 2^(m_s - m), l = sum_s w_s l_s,
// O = sum_s w_s O_s / l, lse = (m + log2 l) ln 2 -- the two-block combination
// of the incremental softmax (FlashAttention reading guide, "Pelacakan
// Softmax Inkremental"), applied across ranges.  A range without keys has
// m = -inf and l = 0 and gets weight 0.
template <int D>
__global__ __launch_bounds__(NT) void splitkv_merge_kernel(AttnArgs a) {
  const long long rows = (long long)a.B * a.H * a.N;
  const long long idx = (long long)blockIdx.x * NT + threadIdx.x;
  const long long row = idx / (D / 4);
  const int g = (int)(idx - row * (D / 4));
  if (row >= rows) return;
  float m = neg_inf();
  for (int s = 0; s < a.nsplit; ++s) m = fmaxf(m, a.part_ml[2 * (s * rows + row)]);
  float l = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.nsplit; ++s) {
    const float ms = a.part_ml[2 * (s * rows + row)];
    if (ms == neg_inf()) continue;
    const float w = __builtin_amdgcn_exp2f(ms - m);
    l += w * a.part_ml[2 * (s * rows + row) + 1];
    const f32x4 x = *reinterpret_cast<const f32x4*>(a.part_o + (s * rows + row) * D + 4 * g);
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] += w * x[e];
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  bf16* orow = reinterpret_cast<bf16*>(a.out0) + row * D + 4 * g;
  store4(orow, o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
  if (g == 0) a.lse[row] = l > 0.f ? (m + __log2f(l)) * LN2 : neg_inf();
}

// Calls F<D>() for the head dimension d (one of 64, 96, 128, 160, 256; the
// entry points have checked it).
template <typename F>
static hipError_t by_head_dim(int d, F&& f) {
  using std::integral_constant;
  switch (d) {
    case 64: return f(integral_constant<int, 64>());
    case 96: return f(integral_constant<int, 96>());
    case 160: return f(integral_constant<int, 160>());
    case 256: return f(integral_constant<int, 256>());
    default: return f(integral_constant<int, 128>());
  }
}

hipError_t launch_splitkv_merge(const AttnArgs& a, int d, hipStream_t s) {
  const long long threads = (long long)a.B * a.H * a.N * (d / 4);
  const dim3 grid((unsigned)((threads + NT - 1) / NT));
  return by_head_dim(d, [&](auto D) {
    hipLaunchKernelGGL((splitkv_merge_kernel<decltype(D)::value>), grid, dim3(NT), 0, s, a);
    return hipGetLastError();
  });
}

template <int D>
static hipError_t launch_splitkv_b(const AttnArgs& a, hipStream_t s) {
  const long long nwg = (long long)((a.N + CELL - 1) / CELL) * a.H * a.B * a.nsplit;
  if (nwg > 0) {
    hipLaunchKernelGGL((fwd_bf16_kernel<D, K_SPLITKV>), dim3((unsigned)nwg), dim3(NT), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_splitkv_merge(a, D, s);
}

hipError_t launch_fwd_splitkv_bf16(const AttnArgs& a, int d, hipStream_t s) {
  return by_head_dim(d, [&](auto D) { return launch_splitkv_b<decltype(D)::value>(a, s); });
}

hipError_t launch_fwd_bf16(const AttnArgs& a, int d, bool walk_only, hipStream_t s) {
  return by_head_dim(d, [&](auto D) { return launch_fwd_b<decltype(D)::value>(a, walk_only, s); });
}
hipError_t launch_dkdv_bf16(const AttnArgs& a, int d, bool walk_only, hipStream_t s) {
  return by_head_dim(d, [&](auto D) { return launch_dkdv_b<decltype(D)::value>(a, walk_only, s); });
}
hipError_t launch_dq_bf16(const AttnArgs& a, int d, bool walk_only, hipStream_t s) {
  return by_head_dim(d, [&](auto D) { return launch_dq_b<decltype(D)::value>(a, walk_only, s); });
}

}  // namespace fa
