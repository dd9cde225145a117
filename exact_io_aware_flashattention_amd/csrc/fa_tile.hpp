// bf16 tiles staged in LDS by direct buffer-to-LDS loads, and the two ways the
// matrix-core operands are read back from them (gfx950).
//
// Layout: a tile of R rows x D bf16 columns is stored row-major (ROWB bytes
// per row, D * 2 when D is a power of two) with its 16-byte chunks
// XOR-swizzled per row: logical chunk c of
// row r sits at physical chunk c ^ swz(r).  The LDS has 64 four-byte banks
// (256 bytes per bank line), so a 256-byte row covers every bank once and a
// 128-byte row half of them.  The two read kinds and what they need:
//   * row reads (ds_read_b128, lane l reads one chunk of row l % 32): served
//     16 lanes per cycle, i.e. 16 consecutive rows at the same logical chunk
//     must land on 16 different chunk positions of the bank line;
//   * transposed reads (ds_read_b64_tr_b16): served 32 lanes per cycle, i.e.
//     4 consecutive rows (4k .. 4k+3) x 4 consecutive chunks.
// d = 128: swz(r) = 4 (r % 4) + (r / 4) % 4;  d = 64: swz(r) = 4 ((r / 2) % 2)
// + (r / 4) % 4.  Both satisfy both conditions (checked with the LDS bank
// conflict counter: 4 cycles per row read, 2 per transposed read).  A 512-byte
// row (d = 256) spans two bank lines; the bank of chunk p is p % 16, and the
// XOR with swz(r) < 16 changes only those four bits, so the d = 128 swizzle
// serves d = 256 unchanged.
//
// Head dimensions that are not a power of two (96, 160) keep the LDS layout of
// the next power of two (128, 256): each LDS row has room for DL columns, of
// which the first D hold the row and the rest are never read.  The swizzles,
// bank analysis and transposed reads are then those of d = DL; only the global
// rows are D * 2 bytes apart.
//
// Loads: buffer_load_dwordx4 with the LDS-destination form writes 64 lanes x
// 16 bytes contiguously at the LDS address in M0, so lane t of a load
// instruction fetches the global chunk that belongs at physical position t.
// The buffer resource spans exactly the valid rows of the head, so rows at or
// beyond N read as zeros without any per-lane branch.  Lanes whose LDS
// position holds a pad chunk (logical chunk >= D / 8) get the offset PAD_OFF,
// past the end of every head's range, so they write zeros and read no memory;
// this needs every head to span at most PAD_OFF bytes.  The load is issued by
// inline assembly: when the compiler sees an LDS-destination load it cannot
// tell which LDS bytes it writes, and waits for it (vmcnt(0)) before every
// later LDS read -- including the reads of the tile being computed, which
// would serialise the prefetch of the next tile.  Completion is instead
// established explicitly: s_waitcnt vmcnt(0) in every wave, then a barrier.
// (Loads the compiler does not know about can only make its own vmcnt waits
// stricter, since vector-memory loads complete in issue order.)
#pragma once

#include "fa_device.hpp"

namespace fa {

typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t PAD_OFF = 0x80000000u;

template <int D>
struct BTile {
  static_assert(D % 32 == 0 && D >= 64 && D <= 256, "head dimension: a multiple of 32 in [64, 256]");
  static constexpr int DL = D <= 64 ? 64 : D <= 128 ? 128 : 256;   // columns an LDS row has room for
  static constexpr int ROWB = DL * 2;         // LDS bytes per row
  static constexpr int CPR = DL / 8;          // 16-byte chunk positions per LDS row
  static constexpr int VC = D / 8;            // chunks that hold data (the rest is padding)
  static constexpr int ROWS_PER_LOAD = 1024 / ROWB;   // rows one wave-wide load fills
  __host__ __device__ static constexpr int swz(int r) {
    return DL >= 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
  __device__ static __forceinline__ int off(int r, int c) { return r * ROWB + ((c ^ swz(r)) << 4); }
};

// Index of the calling wave within the work-group, as a scalar.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Buffer resource (V#) over rows [row0, N) of one head ([N][D] bf16 at head):
// base address of row row0, stride 0, num_records = (N - row0) * D * 2 bytes,
// raw-buffer format bits.  All fields are wave-uniform (scalar registers).
__device__ __forceinline__ u32x4 rows_rsrc(const void* head, int N, int D, int row0) {
  const uint64_t p = reinterpret_cast<uint64_t>(head) + (uint64_t)(uint32_t)row0 * (uint32_t)(D * 2);
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p),
               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xffffu),
               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)max(N - row0, 0) * (uint32_t)(D * 2)), 0x00020000u};
}

// One wave-wide 16-byte-per-lane load into LDS at lds (+ 16 * lane).
__device__ __forceinline__ void dma16(u32x4 rsrc, unsigned char* lds, int voff) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)lds;
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// Loads of an R-row tile spread over the NW waves of the work-group: wave w
// issues the wave-wide loads i = j * NW + w (j < NJ), load i filling rows
// [i * RPL, (i + 1) * RPL) (RPL rows per 1024 LDS bytes).  When the swizzle
// repeats every NW * RPL rows (d <= 128) the logical chunk a lane fetches
// is the same for every j and the lane's byte offset inside the head is
// voff[0] + j * NW * RPL * D * 2; otherwise (d > 128, two rows per load) the offsets
// of one swizzle period are kept and each later period gets its own buffer
// resource based at its first row (the range check of a buffer load covers the
// per-lane offset, so rows past N still read as zeros).  Either way the
// per-lane offsets are computed once per kernel, and a tile load costs only
// scalar work plus the load instructions.
template <int D, int NW>
__host__ __device__ constexpr bool swizzle_repeats(int nj) {
  for (int w = 0; w < NW; ++w)
    for (int r = 0; r < BTile<D>::ROWS_PER_LOAD; ++r)
      for (int j = 0; j < nj; ++j)
        if (BTile<D>::swz((j * NW + w) * BTile<D>::ROWS_PER_LOAD + r) != BTile<D>::swz(w * BTile<D>::ROWS_PER_LOAD + r))
          return false;
  return true;
}

// Smallest k such that the swizzle repeats every k * NW loads (1 for d <= 128;
// 2 for d > 128, whose 16-row swizzle period spans 8 two-row loads).
template <int D, int NW>
__host__ __device__ constexpr int swizzle_period_loads() {
  for (int k = 1; k < 16; ++k) {
    bool ok = true;
    for (int r = 0; r < 64; ++r)
      if (BTile<D>::swz(r + k * NW * BTile<D>::ROWS_PER_LOAD) != BTile<D>::swz(r)) ok = false;
    if (ok) return k;
  }
  return 16;
}

template <int D, int R, int NW = NT / 64>
struct TileDma {
  using TL = BTile<D>;
  static constexpr int NLOAD = R / TL::ROWS_PER_LOAD;
  static constexpr int NJ = NLOAD / NW;
  static constexpr int KP = swizzle_period_loads<D, NW>();
  static_assert(NLOAD % NW == 0, "wave-wide loads must divide evenly over the waves");
  static_assert(KP == 1 ? swizzle_repeats<D, NW>(NJ) : NJ % KP == 0, "loads must cover whole swizzle periods");
  // KP == 1: one offset per load; KP > 1: the KP offsets of one period,
  // relative to the period's first row.
  int voff[KP == 1 ? NJ : KP];

  __device__ __forceinline__ TileDma() {
    const int lane = threadIdx.x & 63, wave = wave_id();
    if constexpr (KP == 1) {
      const int lr = wave * TL::ROWS_PER_LOAD + lane / TL::CPR;   // row of load j = 0
      const int c = (lane % TL::CPR) ^ TL::swz(lr);               // logical chunk at position lane
      const int off0 = (lr * D + c * 8) * 2;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        voff[j] = c < TL::VC ? off0 + j * NW * TL::ROWS_PER_LOAD * D * 2 : (int)PAD_OFF;
    } else {
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        const int lr = (j * NW + wave) * TL::ROWS_PER_LOAD + lane / TL::CPR;
        const int c = (lane % TL::CPR) ^ TL::swz(lr);
        voff[j] = c < TL::VC ? (lr * D + c * 8) * 2 : (int)PAD_OFF;
      }
    }
  }
  // Issue the loads of rows [row0, row0 + R) of head (N rows) into lds
  // (R * BTile<D>::ROWB bytes); rows at or past N read as zeros.  Completion:
  // s_waitcnt vmcnt(0) in every wave, then a barrier.
  __device__ __forceinline__ void load(const void* head, int N, int row0, unsigned char* lds) const {
    const int wave = wave_id();
    if constexpr (KP == 1) {
      const u32x4 rsrc = rows_rsrc(head, N, D, row0);
#pragma unroll
      for (int j = 0; j < NJ; ++j) dma16(rsrc, lds + (j * NW + wave) * 1024, voff[j]);
    } else {
#pragma unroll
      for (int p = 0; p < NJ / KP; ++p) {
        const u32x4 rsrc = rows_rsrc(head, N, D, row0 + p * KP * NW * TL::ROWS_PER_LOAD);
#pragma unroll
        for (int jj = 0; jj < KP; ++jj) dma16(rsrc, lds + ((p * KP + jj) * NW + wave) * 1024, voff[jj]);
      }
    }
  }
};

__device__ __forceinline__ void wait_loads() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// The same wait issued through the builtin, so that the compiler's own wait
// accounting knows every vector-memory load issued before it (register loads
// made before a tile loop included) has completed, and adds no wait for them
// later in the loop, where it would be counted in order behind the tile
// loads issued since.  (vmcnt 0; expcnt and lgkmcnt at their maxima.)
__device__ __forceinline__ void wait_loads_all() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __asm__ volatile("" ::: "memory");
}

// One 16-byte chunk (8 bf16) of row r.
template <int D>
__device__ __forceinline__ u32x4 row_chunk(const unsigned char* tile, int r, int c) {
  return *reinterpret_cast<const u32x4*>(tile + BTile<D>::off(r, c));
}

// Matrix-core operand for a product whose contraction runs over tile rows:
// lane l receives column col0 + l % 32 at rows row_base + 4*h + {0..3} and
// row_base + 8 + 4*h + {0..3} (h = l / 32), i.e. the contraction indices of
// accumulator registers 8*mm .. 8*mm + 7 when row_base = 16*mm.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const unsigned char* tile, int row_base, int col0) {
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4, u = lane & 15, h = lane >> 5;
  const int col = col0 + 16 * (G & 1) + 4 * (u & 3);
  const int c = col >> 3, within = (col & 7) * 2;
  const int r1 = row_base + 4 * h + (u >> 2);
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(tile + BTile<D>::off(r1, c) + within));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(tile + BTile<D>::off(r1 + 8, c) + within));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// acc += A x B on the 32x32x16 bf16 matrix core.
__device__ __forceinline__ void mma(f32x16& acc, bf16x8 a, bf16x8 b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

}  // namespace fa
