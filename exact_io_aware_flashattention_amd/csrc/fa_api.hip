// C ABI of libfa.so: argument checks, then stream-ordered kernel launches.
// Every check runs before any HIP call, so a rejected call touches neither
// the device nor the stream.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "fa.h"
#include "fa_kernels.hpp"

namespace {

constexpr int kCell = 128;
constexpr int kMaxCells = 2048;

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

struct Shape {
  int B, H, N, d, dtype;
};

// Size and type checks shared by every entry point.  Sets *empty when there
// is nothing to compute.
// Head dimensions of the bf16 kernels; fp32 has 64 and 128.
bool bf16_head_dim(int d) { return d == 64 || d == 96 || d == 128 || d == 160 || d == 256; }

// d = 96 and 160 are staged in LDS with padded rows whose pad chunks are
// loaded from the offset 2^31 (past the head), so a head (N rows) must span
// at most 2^31 bytes.
bool head_fits(long long N, int d) {
  const bool padded = d == 96 || d == 160;
  return N * d <= (padded ? (1LL << 30) : 0x7fffffffLL);
}

int check_shape(const Shape& s, const uint8_t* block_mask, bool* empty) {
  if (s.dtype != FA_BF16 && s.dtype != FA_F32) return FA_ERR_DTYPE;
  if (s.B < 0 || s.H < 0 || s.N < 0) return FA_ERR_SHAPE;
  if (s.dtype == FA_BF16 ? !bf16_head_dim(s.d) : (s.d != 64 && s.d != 128)) return FA_ERR_SHAPE;
  *empty = (s.B == 0 || s.H == 0 || s.N == 0);
  if (*empty) return FA_OK;
  const long long T = (s.N + kCell - 1) / kCell;
  if (block_mask && T > kMaxCells) return FA_ERR_SHAPE;
  // A launch covers fewer than 2^32 work-items: the attention kernels run
  // T*H*B work-groups of 256 (plus the split items of dK/dV), the backward
  // preprocess at most 32 threads per row.  In-head offsets stay within int.
  if (T * s.H * s.B + fa::SPLIT_MAX_ITEMS >= (1LL << 32) / fa::NT_HOST) return FA_ERR_SHAPE;
  if ((long long)s.B * s.H * s.N >= (1LL << 32) / 32 - fa::NT_HOST) return FA_ERR_SHAPE;
  if (!head_fits(s.N, s.d)) return FA_ERR_SHAPE;
  return FA_OK;
}

int check_scale(float scale) { return (isfinite(scale) && scale > 0.f) ? FA_OK : FA_ERR_ARG; }

int check_tensors(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (!p) return FA_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned(p, 16)) return FA_ERR_ALIGN;
  return FA_OK;
}

int check_rowstats(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (!p) return FA_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned(p, 4)) return FA_ERR_ALIGN;
  return FA_OK;
}

int check_masks(const uint8_t* block_mask, const int32_t* kv_len) {
  (void)block_mask;
  if (kv_len && !aligned(kv_len, 4)) return FA_ERR_ALIGN;
  return FA_OK;
}

fa::AttnArgs make_args(const Shape& s, float scale, int causal, const uint8_t* block_mask,
                       const int32_t* kv_len) {
  fa::AttnArgs a{};
  a.B = s.B;
  a.H = s.H;
  a.N = s.N;
  a.scale = scale;
  a.c = scale * 1.4426950408889634f;
  a.causal = causal ? 1 : 0;
  a.mask = block_mask;
  a.kv_len = kv_len;
  return a;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// Dropout request: p in [0, 1) becomes the byte threshold t = round(256 p)
// (keep iff the random byte >= t, so the effective rate is t / 256); t must
// be at most 255.  t = 0 is no dropout.  Only the bf16 kernels implement it.
struct Drop {
  uint32_t t = 0;
  uint64_t seed = 0;
};

int make_drop(float p, uint64_t seed, int dtype, Drop* out) {
  if (!isfinite(p) || p < 0.f || p >= 1.f) return FA_ERR_ARG;
  const long t = lrintf(p * 256.f);
  if (t > 255) return FA_ERR_ARG;
  if (t > 0 && dtype != FA_BF16) return FA_ERR_DTYPE;
  out->t = (uint32_t)t;
  out->seed = seed;
  return FA_OK;
}

void set_drop(fa::AttnArgs& a, const Drop& d) {
  a.drop_t = d.t;
  a.drop_k0 = (uint32_t)(d.seed & 0xffffffffu);
  a.drop_k1 = (uint32_t)(d.seed >> 32);
  a.drop_inv = 256.f / (256.f - (float)d.t);
}

size_t delta_bytes(int B, int H, int N) {
  const size_t bytes = (size_t)B * H * N * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

// The dK/dV split workspace, when this call needs one.
int split_workspace(fa::AttnArgs& a, const Shape& s, void* ws, size_t ws_bytes) {
  const size_t need = s.dtype == FA_BF16 && a.mask ? fa::split_ws_bytes(s.N, s.d) : 0;
  if (need == 0) return FA_OK;
  if (!ws) return FA_ERR_NULL;
  if (!aligned(ws, 16)) return FA_ERR_ALIGN;
  if (ws_bytes < need) return FA_ERR_WORKSPACE;
  a.split = fa::split_ws_carve(ws, s.N, s.d);
  return FA_OK;
}

#define FA_TRY(expr)            \
  do {                          \
    const int _st = (expr);     \
    if (_st != FA_OK) return _st; \
  } while (0)

int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
             float scale, int causal, const uint8_t* block_mask, const int32_t* kv_len, int dtype, const Drop& drop,
             void* stream) {
  const Shape s{B, H, N, d, dtype};
  bool empty = false;
  FA_TRY(check_shape(s, block_mask, &empty));
  if (empty) return FA_OK;
  FA_TRY(check_tensors({q, k, v, o}));
  FA_TRY(check_rowstats({lse}));
  FA_TRY(check_masks(block_mask, kv_len));
  FA_TRY(check_scale(scale));
  fa::AttnArgs a = make_args(s, scale, causal, block_mask, kv_len);
  set_drop(a, drop);
  a.q = q;
  a.k = k;
  a.v = v;
  a.out0 = o;
  a.lse = lse;
  return hip_status(fa::launch_fwd(a, dtype, d, false, static_cast<hipStream_t>(stream)));
}

int dkdv_impl(const void* q, const void* k, const void* v, const void* dO, const float* lse, const float* delta,
              void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, const uint8_t* block_mask,
              const int32_t* kv_len, int dtype, const Drop& drop, void* workspace, size_t workspace_bytes,
              void* stream) {
  const Shape s{B, H, N, d, dtype};
  bool empty = false;
  FA_TRY(check_shape(s, block_mask, &empty));
  if (empty) return FA_OK;
  FA_TRY(check_tensors({q, k, v, dO, dk, dv}));
  FA_TRY(check_rowstats({lse, delta}));
  FA_TRY(check_masks(block_mask, kv_len));
  FA_TRY(check_scale(scale));
  fa::AttnArgs a = make_args(s, scale, causal, block_mask, kv_len);
  set_drop(a, drop);
  a.q = q;
  a.k = k;
  a.v = v;
  a.dO = dO;
  a.lse = const_cast<float*>(lse);
  a.delta = const_cast<float*>(delta);
  a.out0 = dk;
  a.out1 = dv;
  FA_TRY(split_workspace(a, s, workspace, workspace_bytes));
  return hip_status(fa::launch_bwd_dkdv(a, dtype, d, false, static_cast<hipStream_t>(stream)));
}

int dq_impl(const void* q, const void* k, const void* v, const void* dO, const float* lse, const float* delta,
            void* dq, int B, int H, int N, int d, float scale, int causal, const uint8_t* block_mask,
            const int32_t* kv_len, int dtype, const Drop& drop, void* stream) {
  const Shape s{B, H, N, d, dtype};
  bool empty = false;
  FA_TRY(check_shape(s, block_mask, &empty));
  if (empty) return FA_OK;
  FA_TRY(check_tensors({q, k, v, dO, dq}));
  FA_TRY(check_rowstats({lse, delta}));
  FA_TRY(check_masks(block_mask, kv_len));
  FA_TRY(check_scale(scale));
  fa::AttnArgs a = make_args(s, scale, causal, block_mask, kv_len);
  set_drop(a, drop);
  a.q = q;
  a.k = k;
  a.v = v;
  a.dO = dO;
  a.lse = const_cast<float*>(lse);
  a.delta = const_cast<float*>(delta);
  a.out0 = dq;
  return hip_status(fa::launch_bwd_dq(a, dtype, d, false, static_cast<hipStream_t>(stream)));
}


int pre_impl(const void* o, const void* dO, float* delta, int B, int H, int N, int d, int dtype,
                      void* stream) {
  const Shape s{B, H, N, d, dtype};
  bool empty = false;
  FA_TRY(check_shape(s, nullptr, &empty));
  if (empty) return FA_OK;
  FA_TRY(check_tensors({o, dO}));
  FA_TRY(check_rowstats({delta}));
  fa::AttnArgs a = make_args(s, 1.f, 0, nullptr, nullptr);
  a.o = o;
  a.dO = dO;
  a.delta = delta;
  return hip_status(fa::launch_bwd_pre(a, dtype, d, static_cast<hipStream_t>(stream)));
}

// dq, with delta = rowsum(dO * O) formed by the dQ kernel itself and stored
// (bf16); float32 runs the preprocess and then dq.
int dq_delta_impl(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                  float* delta, void* dq, int B, int H, int N, int d, float scale, int causal,
                  const uint8_t* block_mask, const int32_t* kv_len, int dtype, const Drop& drop, void* stream) {
  if (dtype != FA_BF16) {
    FA_TRY(pre_impl(o, dO, delta, B, H, N, d, dtype, stream));
    return dq_impl(q, k, v, dO, lse, delta, dq, B, H, N, d, scale, causal, block_mask, kv_len, dtype, drop, stream);
  }
  const Shape s{B, H, N, d, dtype};
  bool empty = false;
  FA_TRY(check_shape(s, block_mask, &empty));
  if (empty) return FA_OK;
  FA_TRY(check_tensors({q, k, v, o, dO, dq}));
  FA_TRY(check_rowstats({lse, delta}));
  FA_TRY(check_masks(block_mask, kv_len));
  FA_TRY(check_scale(scale));
  fa::AttnArgs a = make_args(s, scale, causal, block_mask, kv_len);
  set_drop(a, drop);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dO = dO;
  a.lse = const_cast<float*>(lse);
  a.delta = delta;
  a.out0 = dq;
  return hip_status(fa::launch_bwd_dq(a, dtype, d, false, static_cast<hipStream_t>(stream)));
}

size_t split_bytes(int N, int d, int dtype, int has_block_mask) {
  if (N <= 0 || !bf16_head_dim(d) || dtype != FA_BF16 || !has_block_mask) return 0;
  return fa::split_ws_bytes(N, d);
}

int bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
             void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal,
             const uint8_t* block_mask, const int32_t* kv_len, int dtype, const Drop& drop, void* workspace,
             size_t workspace_bytes, void* stream) {
  const Shape s{B, H, N, d, dtype};
  bool empty = false;
  FA_TRY(check_shape(s, block_mask, &empty));
  if (empty) return FA_OK;
  FA_TRY(check_tensors({q, k, v, o, dO, dq, dk, dv}));
  FA_TRY(check_rowstats({lse}));
  FA_TRY(check_masks(block_mask, kv_len));
  FA_TRY(check_scale(scale));
  if (!workspace) return FA_ERR_NULL;
  if (!aligned(workspace, 16)) return FA_ERR_ALIGN;
  const size_t db = delta_bytes(B, H, N);
  if (workspace_bytes < db + split_bytes(N, d, dtype, block_mask != nullptr)) return FA_ERR_WORKSPACE;
  float* delta = static_cast<float*>(workspace);
  FA_TRY(dq_delta_impl(q, k, v, o, dO, lse, delta, dq, B, H, N, d, scale, causal, block_mask, kv_len, dtype, drop,
                       stream));
  return dkdv_impl(q, k, v, dO, lse, delta, dk, dv, B, H, N, d, scale, causal, block_mask, kv_len, dtype, drop,
                   static_cast<unsigned char*>(workspace) + db, workspace_bytes - db, stream);
}

// Key ranges of a split-key forward: nsplit ranges of tps 64-key tiles each.
// Few queries (Nq <= kDecodeMaxQ) take the decoding kernel: one wave per
// (range, b, h), ranges of whole tiles.  Otherwise one 256-thread work-group
// per (range, b, h, 128 queries), ranges of whole 128-key cells (tps even).
// num_splits = 0 picks the largest count that keeps every unit of work
// resident at once -- 256 compute units, each holding two work-groups of the
// attention kernel: the ranges are of equal length, so a second, partly
// filled round would cost as much as the first.  Decoding waves are capped
// at one per SIMD (1024): measured on this part, more concurrent read
// streams lower the bandwidth they reach together.
constexpr int kSplitKvMax = 1024;
constexpr int kDecodeMaxQ = 4;
constexpr long long kResidentGroups = 256 * 2;
constexpr long long kResidentWaves = 256 * 4;

struct KvPlan {
  int nsplit, tps;
  bool decode;
};

int splitkv_plan(int B, int H, int Nq, int Nk, int num_splits, KvPlan* p) {
  if (num_splits < 0 || num_splits > kSplitKvMax) return FA_ERR_ARG;
  p->decode = Nq <= kDecodeMaxQ;
  const long long Tq = (Nq + kCell - 1) / kCell;
  const long long tiles = (Nk + 63) / 64;
  const long long unit = p->decode ? 1 : 2;   // tiles per range step
  const long long groups = p->decode ? (long long)B * H : Tq * B * H;
  const long long slots = p->decode ? kResidentWaves : kResidentGroups;
  long long want = num_splits;
  if (want == 0) want = groups > 0 ? slots / groups : 1;
  want = std::max(1LL, std::min<long long>(want, kSplitKvMax));
  long long tps = (tiles + want - 1) / want;
  tps = std::max(unit, (tps + unit - 1) / unit * unit);
  p->tps = (int)tps;
  p->nsplit = (int)std::max(1LL, (tiles + tps - 1) / tps);
  // the launch runs groups * nsplit work-groups (waves, when decoding) of 256
  if (groups * p->nsplit >= (1LL << 32) / fa::NT_HOST) return FA_ERR_SHAPE;
  return FA_OK;
}

int check_splitkv_shape(int B, int H, int Nq, int Nk, int d, int dtype, bool* empty) {
  if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_DTYPE;
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return FA_ERR_SHAPE;
  if (!bf16_head_dim(d)) return FA_ERR_SHAPE;
  *empty = (B == 0 || H == 0 || Nq == 0);
  if (*empty) return FA_OK;
  if (dtype != FA_BF16) return FA_ERR_DTYPE;
  if ((long long)B * H * Nq * (d / 4) >= (1LL << 32) - fa::NT_HOST) return FA_ERR_SHAPE;
  if (!head_fits(Nq, d) || !head_fits(Nk, d)) return FA_ERR_SHAPE;
  return FA_OK;
}

size_t splitkv_o_bytes(int B, int H, int Nq, int d, int nsplit) {
  return (size_t)nsplit * B * H * Nq * d * sizeof(float);
}

size_t splitkv_bytes(int B, int H, int Nq, int Nk, int d, int num_splits) {
  bool empty = false;
  KvPlan p;
  if (check_splitkv_shape(B, H, Nq, Nk, d, FA_BF16, &empty) != FA_OK || empty) return 0;
  if (splitkv_plan(B, H, Nq, Nk, num_splits, &p) != FA_OK) return 0;
  return splitkv_o_bytes(B, H, Nq, d, p.nsplit) + (size_t)p.nsplit * B * H * Nq * 2 * sizeof(float);
}

// ---------------------------------------------------------------- fixed scratch

// Device buffer of fa_fwd_splitkv_noalloc, for callers that cannot allocate:
// one per GPU (the code object is loaded on every device the library runs
// on), held until the process ends.  In host code `scratch` names a host-side
// stand-in, not the device memory: its device address is looked up once per
// device with hipGetSymbolAddress, and only that address is passed to kernels.
__device__ __attribute__((aligned(256))) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (the first call on a
// device looks it up with that device current).
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

int splitkv_run(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                int d, float scale, int causal, const int32_t* kv_len, int dtype, int num_splits, void* workspace,
                size_t workspace_bytes, void* stream, bool use_scratch);

}  // namespace

extern "C" {

const char* fa_status_str(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: unsupported or inconsistent sizes";
    case FA_ERR_DTYPE: return "FA_ERR_DTYPE: dtype must be FA_BF16 or FA_F32";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: a pointer is not suitably aligned";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace too small";
    case FA_ERR_HIP: return "FA_ERR_HIP: a HIP launch failed";
    case FA_ERR_SCRATCH:
      return "FA_ERR_SCRATCH: the sizes need more than the library's fixed scratch (FA_NOALLOC_SCRATCH_BYTES)";
    case FA_ERR_ARG: return "FA_ERR_ARG: invalid scale or selector";
    default: return "unknown fa status";
  }
}

size_t fa_bwd_dkdv_workspace_bytes(int N, int d, int dtype, int has_block_mask) {
  return split_bytes(N, d, dtype, has_block_mask);
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d, int dtype, int has_block_mask) {
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  return delta_bytes(B, H, N) + split_bytes(N, d, dtype, has_block_mask);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
           float scale, int causal, const uint8_t* block_mask, const int32_t* kv_len, int dtype,
           void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, N, d, scale, causal, block_mask, kv_len, dtype, Drop{}, stream);
}

int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   float scale, int causal, const uint8_t* block_mask, const int32_t* kv_len, int dtype,
                   float dropout_p, uint64_t seed, void* stream) {
  Drop drop;
  FA_TRY(make_drop(dropout_p, seed, dtype, &drop));
  return fwd_impl(q, k, v, o, lse, B, H, N, d, scale, causal, block_mask, kv_len, dtype, drop, stream);
}

int fa_bwd_preprocess(const void* o, const void* dO, float* delta, int B, int H, int N, int d, int dtype,
                      void* stream) {
  return pre_impl(o, dO, delta, B, H, N, d, dtype, stream);
}

int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                const float* delta, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal,
                const uint8_t* block_mask, const int32_t* kv_len, int dtype, void* workspace,
                size_t workspace_bytes, void* stream) {
  return dkdv_impl(q, k, v, dO, lse, delta, dk, dv, B, H, N, d, scale, causal, block_mask, kv_len, dtype, Drop{},
                   workspace, workspace_bytes, stream);
}

int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dO, const float* lse,
              const float* delta, void* dq, int B, int H, int N, int d, float scale, int causal,
              const uint8_t* block_mask, const int32_t* kv_len, int dtype, void* stream) {
  return dq_impl(q, k, v, dO, lse, delta, dq, B, H, N, d, scale, causal, block_mask, kv_len, dtype, Drop{}, stream);
}

int fa_bwd_dq_delta(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                    float* delta, void* dq, int B, int H, int N, int d, float scale, int causal,
                    const uint8_t* block_mask, const int32_t* kv_len, int dtype, void* stream) {
  return dq_delta_impl(q, k, v, o, dO, lse, delta, dq, B, H, N, d, scale, causal, block_mask, kv_len, dtype, Drop{},
                       stream);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
           void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal,
           const uint8_t* block_mask, const int32_t* kv_len, int dtype, void* workspace,
           size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, block_mask, kv_len, dtype, Drop{},
                  workspace, workspace_bytes, stream);
}

int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                   void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal,
                   const uint8_t* block_mask, const int32_t* kv_len, int dtype, float dropout_p, uint64_t seed,
                   void* workspace, size_t workspace_bytes, void* stream) {
  Drop drop;
  FA_TRY(make_drop(dropout_p, seed, dtype, &drop));
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, block_mask, kv_len, dtype, drop,
                  workspace, workspace_bytes, stream);
}

size_t fa_fwd_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits) {
  return splitkv_bytes(B, H, Nq, Nk, d, num_splits);
}

int fa_fwd_splitkv_num_splits(int B, int H, int Nq, int Nk, int num_splits) {
  KvPlan p;
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk < 0) return 0;
  if (splitkv_plan(B, H, Nq, Nk, num_splits, &p) != FA_OK) return 0;
  return p.nsplit;
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                   int d, float scale, int causal, const int32_t* kv_len, int dtype, int num_splits,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return splitkv_run(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, kv_len, dtype, num_splits, workspace,
                     workspace_bytes, stream, false);
}

int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
                           int Nk, int d, float scale, int causal, const int32_t* kv_len, int dtype, int num_splits,
                           void* stream) {
  return splitkv_run(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, kv_len, dtype, num_splits, nullptr, 0,
                     stream, true);
}

}  // extern "C"

namespace {

// fa_fwd_splitkv with the caller's workspace, or (use_scratch) with the
// library's fixed scratch of the current device; every check runs first.
int splitkv_run(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                int d, float scale, int causal, const int32_t* kv_len, int dtype, int num_splits, void* workspace,
                size_t workspace_bytes, void* stream, bool use_scratch) {
  bool empty = false;
  FA_TRY(check_splitkv_shape(B, H, Nq, Nk, d, dtype, &empty));
  if (empty) return FA_OK;
  KvPlan p;
  FA_TRY(splitkv_plan(B, H, Nq, Nk, num_splits, &p));
  FA_TRY(check_tensors({q, o}));
  if (Nk > 0) FA_TRY(check_tensors({k, v}));
  FA_TRY(check_rowstats({lse}));
  FA_TRY(check_masks(nullptr, kv_len));
  FA_TRY(check_scale(scale));
  const size_t need = splitkv_bytes(B, H, Nq, Nk, d, num_splits);
  if (use_scratch) {
    if (need > FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
    FA_TRY(scratch_on_current_device(&workspace));
  } else {
    if (!workspace) return FA_ERR_NULL;
    if (!aligned(workspace, 16)) return FA_ERR_ALIGN;
    if (workspace_bytes < need) return FA_ERR_WORKSPACE;
  }
  fa::AttnArgs a = make_args(Shape{B, H, Nq, d, dtype}, scale, causal, nullptr, kv_len);
  a.q = q;
  a.k = k;
  a.v = v;
  a.out0 = o;
  a.lse = lse;
  a.Nk = Nk;
  a.causal_off = Nk - Nq;
  a.nsplit = p.nsplit;
  a.split_tiles = p.tps;
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) +
                                       splitkv_o_bytes(B, H, Nq, d, p.nsplit));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(p.decode ? fa::launch_fwd_decode_bf16(a, d, st) : fa::launch_fwd_splitkv_bf16(a, d, st));
}

}  // namespace

extern "C" {

int fa_fwd_splitkv_fp8kv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
                         int Nk, int d, float scale, int causal, const int32_t* kv_len, float k_descale,
                         float v_descale, int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  bool empty = false;
  FA_TRY(check_splitkv_shape(B, H, Nq, Nk, d, FA_BF16, &empty));
  if (empty) return FA_OK;
  if (Nq > kDecodeMaxQ) return FA_ERR_SHAPE;
  KvPlan p;
  FA_TRY(splitkv_plan(B, H, Nq, Nk, num_splits, &p));
  FA_TRY(check_tensors({q, o}));
  if (Nk > 0) FA_TRY(check_tensors({k, v}));
  FA_TRY(check_rowstats({lse}));
  FA_TRY(check_masks(nullptr, kv_len));
  FA_TRY(check_scale(scale));
  FA_TRY(check_scale(k_descale));
  FA_TRY(check_scale(v_descale));
  const float c = scale * k_descale;
  if (!isfinite(c) || !(c > 0.f)) return FA_ERR_ARG;
  if (!workspace) return FA_ERR_NULL;
  if (!aligned(workspace, 16)) return FA_ERR_ALIGN;
  if (workspace_bytes < splitkv_bytes(B, H, Nq, Nk, d, num_splits)) return FA_ERR_WORKSPACE;
  fa::AttnArgs a = make_args(Shape{B, H, Nq, d, FA_BF16}, c, causal, nullptr, kv_len);
  a.q = q;
  a.k = k;
  a.v = v;
  a.out0 = o;
  a.lse = lse;
  a.Nk = Nk;
  a.causal_off = Nk - Nq;
  a.nsplit = p.nsplit;
  a.split_tiles = p.tps;
  a.v_descale = v_descale;
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) +
                                       splitkv_o_bytes(B, H, Nq, d, p.nsplit));
  return hip_status(fa::launch_fwd_decode_e4m3kv(a, d, static_cast<hipStream_t>(stream)));
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
               float scale, int causal, const uint8_t* block_mask, const int32_t* kv_len, float q_descale,
               float k_descale, float v_descale, void* stream) {
  const Shape s{B, H, N, d, FA_BF16};
  bool empty = false;
  if (d != 64 && d != 128) return FA_ERR_SHAPE;
  FA_TRY(check_shape(s, block_mask, &empty));
  if (empty) return FA_OK;
  FA_TRY(check_tensors({q, k, v, o}));
  FA_TRY(check_rowstats({lse}));
  FA_TRY(check_masks(block_mask, kv_len));
  FA_TRY(check_scale(scale));
  FA_TRY(check_scale(q_descale));
  FA_TRY(check_scale(k_descale));
  FA_TRY(check_scale(v_descale));
  const float c = scale * q_descale * k_descale;
  if (!isfinite(c) || !(c > 0.f)) return FA_ERR_ARG;
  fa::AttnArgs a = make_args(s, c, causal, block_mask, kv_len);
  a.q = q;
  a.k = k;
  a.v = v;
  a.out0 = o;
  a.lse = lse;
  a.v_descale = v_descale;
  return hip_status(fa::launch_fwd_fp8(a, d, static_cast<hipStream_t>(stream)));
}

int fa_debug_visits(int which, int B, int H, int N, int d, int causal, const uint8_t* block_mask,
                    const int32_t* kv_len, int dtype, uint32_t* counts, void* workspace, size_t workspace_bytes,
                    void* stream) {
  const Shape s{B, H, N, d, dtype};
  bool empty = false;
  if (which < fa::WALK_FWD || which > fa::WALK_DQ) return FA_ERR_ARG;
  FA_TRY(check_shape(s, block_mask, &empty));
  if (empty) return FA_OK;
  if (!counts) return FA_ERR_NULL;
  if (!aligned(counts, 4)) return FA_ERR_ALIGN;
  FA_TRY(check_masks(block_mask, kv_len));
  fa::AttnArgs a = make_args(s, 1.f, causal, block_mask, kv_len);
  a.counts = counts;
  if (which == fa::WALK_DKDV) FA_TRY(split_workspace(a, s, workspace, workspace_bytes));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (which == fa::WALK_FWD)
    e = fa::launch_fwd(a, dtype, d, true, st);
  else if (which == fa::WALK_DKDV)
    e = fa::launch_bwd_dkdv(a, dtype, d, true, st);
  else
    e = fa::launch_bwd_dq(a, dtype, d, true, st);
  return hip_status(e);
}

}  // extern "C"
