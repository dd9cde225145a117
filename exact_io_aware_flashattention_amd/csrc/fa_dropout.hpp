// Dropout on the attention probabilities, fused into the bf16 kernels.
//
// The pages name dropout among the operations the fused kernel performs
// (FlashAttention reading guide, "Ide Utama", kernel-fusion bullet) without a
// formula or generator.  Here: entry (b, h, query i, key j) is kept iff its
// random byte u >= t (p = t / 256), kept entries are scaled by 1 / (1 - p),
// and u is byte (j & 3) of word (i & 3) of Philox4x32-10 (Salmon, Moraes,
// Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011) with
// key (seed low, seed high) and counter (j >> 2, i >> 2, b * H + h, 0).  One
// generator call therefore covers a 4 x 4 block of queries x keys, and the
// backward kernels regenerate exactly the bytes the forward used.
//
// Sharing the calls inside a wave.  In both register layouts the four lanes
// of a quad (l & ~3 .. +3) hold four consecutive queries (forward, dQ: lane =
// query, 4 consecutive keys per register group) or four consecutive keys
// (dK/dV: lane = key, 4 consecutive queries per group), and together need the
// same four blocks, one per register group g.  Lane a of the quad computes the
// block of group a, stores its four words in the wave's LDS exchange area and
// reads back, for each group g, the word it needs from lane g of its quad.
#pragma once

#include "fa_device.hpp"

namespace fa {

constexpr uint32_t PHILOX_M0 = 0xD2511F53u, PHILOX_M1 = 0xCD9E8D57u;
constexpr uint32_t PHILOX_W0 = 0x9E3779B9u, PHILOX_W1 = 0xBB67AE85u;

// a ^ b ^ c in one instruction (v_bitop3_b32 with the XOR3 truth table
// 0x96); the compiler otherwise emits two v_xor_b32.
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

// Philox4x32 with 10 rounds.  A round maps (c0, c1, c2, c3) to
// (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key
// advances by (W0, W1) between rounds.
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                               uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // one 32 x 32 -> 64-bit product gives both halves (v_mad_u64_u32, half
    // the multiply instructions of separate high and low products)
    const uint64_t p0 = (uint64_t)PHILOX_M0 * c0, p1 = (uint64_t)PHILOX_M1 * c2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    c0 = xor3(hi1, c1, k0);
    c1 = lo1;
    c2 = xor3(hi0, c3, k1);
    c3 = lo0;
    k0 += PHILOX_W0;
    k1 += PHILOX_W1;
  }
  return u32x4{c0, c1, c2, c3};
}

// Transpose of the 4 x 4 byte matrix held in four words (row m = word m,
// column k = byte k): word k of the result holds byte k of words 0..3.
// v_perm_b32 takes bytes 0-3 from its second operand and 4-7 from its first.
__device__ __forceinline__ u32x4 byte_transpose4(u32x4 w) {
  const uint32_t x01l = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);   // w0.b0 w1.b0 w0.b1 w1.b1
  const uint32_t x01h = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);   // w0.b2 w1.b2 w0.b3 w1.b3
  const uint32_t x23l = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
  const uint32_t x23h = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
  return u32x4{__builtin_amdgcn_perm(x23l, x01l, 0x05040100u), __builtin_amdgcn_perm(x23l, x01l, 0x07060302u),
               __builtin_amdgcn_perm(x23h, x01h, 0x05040100u), __builtin_amdgcn_perm(x23h, x01h, 0x07060302u)};
}

struct DropoutArgs {
  uint32_t t;        // drop threshold: keep iff random byte >= t; 0 = dropout off
  uint32_t k0, k1;   // Philox key (seed low, high word)
  float inv_keep;    // 1 / (1 - t / 256)
};

// Per-wave exchange of the generator words through LDS (16 bytes per lane).
// xch: the work-group's exchange area (NT u32x4).
struct DropQuad {
  unsigned char* base;   // this lane's read base: quad start (x16) + own lane-in-quad (x4)
  unsigned char* mine;   // this lane's 16-byte slot
  __device__ __forceinline__ DropQuad(u32x4* xch) {
    const int tid = threadIdx.x;
    mine = reinterpret_cast<unsigned char*>(xch + tid);
    base = reinterpret_cast<unsigned char*>(xch + (tid & ~3)) + 4 * (tid & 3);
  }
  // Store this lane's four words and return, for g = 0..3, word (lane & 3) of
  // the words stored by lane g of the quad.
  __device__ __forceinline__ u32x4 exchange(u32x4 w) const {
    *reinterpret_cast<u32x4*>(mine) = w;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    u32x4 r;
#pragma unroll
    for (int g = 0; g < 4; ++g) r[g] = *reinterpret_cast<const uint32_t*>(base + 16 * g);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return r;
  }
};

// keep bit of byte e (0..3) of word x
__device__ __forceinline__ bool keep_byte(uint32_t x, int e, uint32_t t) { return ((x >> (8 * e)) & 0xffu) >= t; }

}  // namespace fa
