// Device-side building blocks shared by the attention kernels (gfx950 / CDNA4).
//
// Matrix-core conventions (wave64, v_mfma_f32_32x32x16_bf16 and
// v_mfma_f32_32x32x2_f32): for D = A x B + C with A of M x K and B of K x N,
// lane l supplies row m = l % 32 of A and column n = l % 32 of B, each with the
// K-slice that belongs to lane half h = l / 32; accumulator register r of lane
// l holds D[8*(r/4) + 4*h + (r%4)][l % 32].  Which K-slice a lane half holds
// does not matter as long as A and B agree, so operands are loaded as 16-byte
// chunks and the same chunk index is used on both sides.
//
// Scores are computed transposed, S^T = K Q^T: lane l then owns query l % 32
// and 16 keys per 32-key block, so the row statistics of the incremental
// softmax (FlashAttention reading guide, "Pelacakan Softmax Inkremental") are
// lane-local apart from one exchange between the two lane halves, and the
// probabilities feed the next product (O^T += V^T P^T) straight from
// registers as its B operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int CELL = 128;      // block-mask cell edge
constexpr int NT = 256;        // threads per work-group: 4 waves of 64
constexpr int MAX_T = 2048;    // largest number of mask cells per side
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float TAU = 8.0f;    // the running max is refreshed only when a tile
                               // exceeds it by more than 2^TAU (the refresh step of
                               // the bf16 forward, fa_bf16.hip)

// Waves per SIMD the bf16 kernels are register-limited to: two resident waves
// let one wave's softmax VALU work overlap the other's matrix-core work.
template <typename T> struct Occ { static constexpr int W = sizeof(T) == 2 ? 2 : 1; };

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }
__device__ __forceinline__ float pos_inf() { return __builtin_inff(); }

// Elements per 16-byte chunk.
template <typename T> struct ET;
template <> struct ET<bf16> { static constexpr int CW = 8; };
template <> struct ET<float> { static constexpr int CW = 4; };

// ---------------------------------------------------------------- memory

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

// 4 consecutive elements of type T starting at p (8 bytes for bf16, 16 for f32).
template <typename T> struct Quad;
template <> struct Quad<bf16> {
  u32x2 v;
  __device__ __forceinline__ void load(const bf16* p) { v = ld8(p); }
};
template <> struct Quad<float> {
  u32x4 v;
  __device__ __forceinline__ void load(const float* p) { v = ld16(p); }
};

// Store 4 fp32 values as 4 consecutive elements of T.
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
  bf16x4 x = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
  st8(p, __builtin_bit_cast(u32x2, x));
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  f32x4 x = {a, b, c, d};
  st16(p, __builtin_bit_cast(u32x4, x));
}

// Transposed LDS write of 4 rows x one 16-byte chunk: rows r[0..3] hold
// elements [e0, e0 + CW) of 4 consecutive keys; element e goes to
// dst[e * pitch + 0..3].
__device__ __forceinline__ void write_transposed4(bf16* dst, int pitch, const u32x4 (&r)[4]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int w = e >> 1;
    const int sh = (e & 1) * 16;
    uint32_t a = (r[0][w] >> sh) & 0xffffu, b = (r[1][w] >> sh) & 0xffffu;
    uint32_t c = (r[2][w] >> sh) & 0xffffu, d = (r[3][w] >> sh) & 0xffffu;
    u32x2 x = {a | (b << 16), c | (d << 16)};
    st8(dst + e * pitch, x);
  }
}
__device__ __forceinline__ void write_transposed4(float* dst, int pitch, const u32x4 (&r)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    u32x4 x = {r[0][e], r[1][e], r[2][e], r[3][e]};
    st16(dst + e * pitch, x);
  }
}

// ---------------------------------------------------------------- matrix core

// acc += A_chunk x B_chunk over one 16-byte chunk per lane on both sides.
__device__ __forceinline__ void mma_chunk(f32x16& acc, u32x4 a, u32x4 b, bf16*) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
// (The whole vector is reinterpreted before indexing: bit-casting single
// elements of a u32 vector inside the unrolled loop made hipcc feed element 0
// to all four products.)
__device__ __forceinline__ void mma_chunk(f32x16& acc, u32x4 a, u32x4 b, float*) {
  const f32x4 af = __builtin_bit_cast(f32x4, a), bf = __builtin_bit_cast(f32x4, b);
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i], bf[i], acc, 0, 0, 0);
}

// acc (32 x 32, rows = A rows) += A x X over the 32-long contraction whose
// B-side values sit in the accumulator layout `x` of a previous product
// (register r <-> contraction index 8*(r/4) + 4*h + r%4).  a[g] holds the
// 4 A-side elements for contraction indices 8*g + 4*h + 0..3 of this lane's
// A row (fp32 path).
__device__ __forceinline__ void mma_acc_operand(f32x16& acc, const Quad<float> (&a)[4], const f32x16& x) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 af = __builtin_bit_cast(f32x4, a[g].v);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[e], x[4 * g + e], acc, 0, 0, 0);
  }
}

// Accumulator-layout values (probabilities, dS) rounded to bf16 and packed as
// the two 8-element B operands of a 32x32x16 product over their 32 indices.
struct PackedB { bf16x8 p[2]; };
__device__ __forceinline__ PackedB pack_bf16(const f32x16& x) {
  PackedB r;
#pragma unroll
  for (int mm = 0; mm < 2; ++mm)
#pragma unroll
    for (int j = 0; j < 8; ++j) r.p[mm][j] = (bf16)x[8 * mm + j];
  return r;
}

// ---------------------------------------------------------------- cross-lane

// max(x[l], x[l ^ 32]) in every lane.  v_permlane32_swap exchanges one half
// of its two operands; with both operands equal to x, the two results hold x
// of lane l and x of lane l ^ 32 between them (in an order that does not
// matter for a max), so no LDS round trip is needed.
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(x, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
// x[l] + x[l ^ 32] in every lane.
__device__ __forceinline__ float sum_halves(float x) { return x + __shfl_xor(x, 32); }

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// ---------------------------------------------------------------- scheduling

// Work-groups are handed to the 8 XCDs of the chip round-robin (w -> w % 8).
// Renumber them so that each XCD receives one contiguous range of logical
// ids: consecutive logical ids share a (batch, head) and therefore the same
// K/V stream, which then stays in that XCD's L2.
__device__ __forceinline__ int xcd_logical_id(int w, int n) {
  const int x = w & 7, k = w >> 3;
  const int per = n >> 3, rem = n & 7;
  return (x < rem) ? x * (per + 1) + k : rem * (per + 1) + (x - rem) * per + k;
}

// (head, step) of work-group w of n = BH * T.  The step t indexes the cells
// along the walked direction; for a causal walk step 0 is the heaviest (the
// caller maps it to the last query cell or the first key cell).
//   causal:     t = w / BH, head = w % BH.  All heads' heaviest cells are
//               dispatched first, so no heavy cell is left to start at the end;
//               and since work-group w goes to XCD w % 8, an XCD keeps serving
//               the heads head = XCD (mod 8) when 8 divides BH.
//   non-causal: equal work per cell; XCD-contiguous ranges of one head
//               (xcd_logical_id) keep each head's K/V stream in one L2.
struct WorkUnit {
  int bh, t;
};
__device__ __forceinline__ WorkUnit work_unit(int w, int n, int BH, int T, bool causal) {
  if (causal) return WorkUnit{w % BH, w / BH};
  const int L = xcd_logical_id(w, n);
  return WorkUnit{L / T, L % T};
}

// Build, in LDS, the ascending list of indices c in [0, count) with
// pred(c) true.  All threads of the work-group must call it.  Returns the
// list length (same value in every thread).
template <typename Pred>
__device__ int build_list(int count, Pred pred, int* list, int* scratch4) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int n = 0;
  for (int base = 0; base < count; base += NT) {
    const int c = base + tid;
    const bool ok = c < count && pred(c);
    const uint64_t bal = __builtin_amdgcn_ballot_w64(ok);
    const int before = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) scratch4[wave] = __builtin_popcountll(bal);
    __syncthreads();
    int off = n;
    for (int w = 0; w < wave; ++w) off += scratch4[w];
    if (ok) list[off + before] = c;
    n += scratch4[0] + scratch4[1] + scratch4[2] + scratch4[3];
    __syncthreads();
  }
  return n;
}

}  // namespace fa
