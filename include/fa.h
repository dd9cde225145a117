/*
 * fa.h -- C ABI of the MI355X (gfx950) exact IO-aware attention library (libfa.so).
 *
 * The library computes exact scaled dot-product attention
 *     S = scale * Q K^T  (masked entries -inf),   P = rowsoftmax(S),   O = P V
 * block by block, keeping per query row a running maximum m and normaliser l
 * so that no N x N matrix is ever written to device memory, and the backward
 * pass that keeps only O and the per-row log-sum-exp and recomputes S and P
 * tile by tile.
 *   - Definition of attention: bornlex.github.io "Flash Attention", section
 *     "Standard Attention"; FlashAttention reading guide (xyznot.com),
 *     "Masalah dan Motivasi".
 *   - Tiling with the running (m, l) statistics: reading guide, "Pelacakan
 *     Softmax Inkremental" and "Metode" steps 1-4; bornlex "Tiling".
 *   - Recomputation in the backward pass: reading guide, "Ide Utama";
 *     bornlex "Recomputation".
 *   - Block-sparse skipping of zero mask blocks: reading guide, "Ekstensi:
 *     Block-Sparse FlashAttention".
 *
 * Conventions shared by every entry point
 *   Layout     q, k, v, o, dO, dq, dk, dv are contiguous [B][H][N][d] with d
 *              innermost, all of the element type given by `dtype`.  lse and
 *              delta are float32 [B][H][N].  Every pointer must be 16-byte
 *              aligned.
 *   dtype      FA_BF16 (bf16 storage, bf16 matrix-core products, float32
 *              accumulation and softmax) or FA_F32 (float32 throughout; no
 *              step goes through a narrower type).
 *   d          64 or 128; with FA_BF16 also 96, 160 and 256 (FA2 extends
 *              the head dimension up to 256, datacamp "Penjelasan Flash
 *              Attention", Flash Attention 2, "Dukungan untuk dimensi head
 *              yang lebih besar").  Above d = 128 a work-group's tiles fill
 *              the LDS and its accumulators a whole wave's registers, so one
 *              wave runs per SIMD.  d = 96 and 160 are staged in LDS as rows
 *              of 128 and 256 columns, and need N * d <= 2^30 (else
 *              FA_ERR_SHAPE).
 *   scale      finite and > 0 (the pages write S = QK^T, i.e. scale = 1).
 *   causal     nonzero: key j is allowed for query i only if j <= i (queries
 *              and keys share positions, top-left aligned).
 *   block_mask NULL, or device uint8 [T][T], T = ceil(N/128), row-major,
 *              shared by every (b, h): cell (i, j) covers queries
 *              [128i, 128i+128) and keys [128j, 128j+128); a zero cell is
 *              skipped (all its scores are -inf).  T <= 2048.
 *   kv_len     NULL (all N keys valid), or device int32 [B]: for batch b only
 *              keys j < kv_len[b] are allowed (values are clamped to [0, N]
 *              on the device).
 *   Masks combine with AND.  A query row with no allowed key gets O = 0,
 *   lse = -inf and zero gradient contributions.
 *   Ownership  every buffer is caller-owned device memory; the library never
 *              allocates, frees or synchronises, and keeps no state between
 *              calls.  Calls are stream-ordered on `stream` (a hipStream_t;
 *              NULL = the default stream) and return before the work ends.
 *   Errors     arguments are checked before anything is launched; a check
 *              that fails returns its code and launches nothing.  A launch
 *              failure returns FA_ERR_HIP.  Faults during execution surface
 *              at the caller's next synchronisation, as usual for HIP.  The
 *              library never prints.  Empty problems (B, H or N = 0) return
 *              FA_OK without launching.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fa_dtype { FA_BF16 = 0, FA_F32 = 1 };

enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,      /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,     /* negative size, d not 64/128 (or 96/160/256 in bf16), T > 2048 or too large */
  FA_ERR_DTYPE = 3,     /* dtype not FA_BF16 / FA_F32 */
  FA_ERR_ALIGN = 4,     /* a tensor pointer is not 16-byte aligned */
  FA_ERR_WORKSPACE = 5, /* workspace smaller than the matching *_workspace_bytes() */
  FA_ERR_HIP = 6,       /* a HIP launch failed */
  FA_ERR_ARG = 7,       /* scale not finite and > 0, bad selector, or bad dropout rate */
  FA_ERR_SCRATCH = 8    /* fa_fwd_splitkv_noalloc: sizes need more than FA_NOALLOC_SCRATCH_BYTES */
};

/* Size of the fixed device scratch behind fa_fwd_splitkv_noalloc (64 MiB per
 * GPU the library runs on). */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * Forward pass.  Writes o [B,H,N,d] (dtype) and lse [B,H,N] (float32), with
 * lse_i = m_i + ln(l_i), the natural log of the row normaliser of the scaled
 * scores; together with O it is all the backward pass needs (the reading
 * guide's recomputation bullet stores the pair (l, m); lse carries the same
 * information because P = exp(S - lse)).  Each work-group owns 128 query rows
 * and walks the allowed 64-key tiles of its row of mask cells in ascending
 * order, applying the incremental softmax update of "Metode" steps 2-4 with
 * the division by l deferred to the end.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal,
           const uint8_t* block_mask, const int32_t* kv_len, int dtype, void* stream);

/*
 * Bytes of workspace fa_bwd needs: the float32 row terms
 * delta_i = sum_k dO_ik O_ik, [B,H,N], rounded up to 256, followed by
 * fa_bwd_dkdv_workspace_bytes(N, d, dtype, has_block_mask) bytes.
 * has_block_mask: nonzero if the call will pass a block mask.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d, int dtype, int has_block_mask);

/*
 * Bytes of workspace fa_bwd_dkdv needs.  Zero unless dtype is FA_BF16 and a
 * block mask is passed: then the key columns of the mask that many query
 * cells visit are split over several work-groups, which need a plan, arrival
 * counters and float32 partial sums for at most 1024 column chunks
 * (1024 * 2 * 128 * d * 4 bytes plus about ceil(N/128)^2 / 16 bytes; 64 MiB
 * at d = 64, 128 MiB at d = 128, 256 MiB at d = 256; d / 64 * 64 MiB in
 * general).  Independent of B and H.
 */
size_t fa_bwd_dkdv_workspace_bytes(int N, int d, int dtype, int has_block_mask);

/*
 * Backward pass for the loss gradient dO: writes dq, dk, dv (dtype).  Runs
 * fa_bwd_dq_delta and then fa_bwd_dkdv on `stream` (FA_F32: fa_bwd_preprocess,
 * fa_bwd_dq, fa_bwd_dkdv), with delta, then the dk/dv workspace, in
 * `workspace` (at least
 * fa_bwd_workspace_bytes bytes for the same sizes and mask presence, 16-byte
 * aligned; its contents need no initialisation and are overwritten).  o and lse must be the outputs of fa_fwd on the same q, k, v,
 * scale and masks.  The pages print no backward equations; the ones used
 * follow from the definition by the chain rule:
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - delta),
 *   dQ = scale dS K,  dK = scale dS^T Q,  with delta_i = sum_j P_ij dP_ij
 *   = dO_i . O_i.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
           const float* lse, void* dq, void* dk, void* dv,
           int B, int H, int N, int d, float scale, int causal,
           const uint8_t* block_mask, const int32_t* kv_len, int dtype,
           void* workspace, size_t workspace_bytes, void* stream);

/* Backward stage 1: delta [B,H,N] float32 = rowsum(dO * O). */
int fa_bwd_preprocess(const void* o, const void* dO, float* delta,
                      int B, int H, int N, int d, int dtype, void* stream);

/*
 * Backward stage 2: dk, dv.  Each work-group owns 128 keys (one mask cell
 * column) and walks the query tiles that visit it, recomputing S and P from
 * q, k and lse.  With a block mask (FA_BF16), a column with more visited
 * cells than a plan's chunk size is split into chunks, one work-group each,
 * whose float32 partial sums are added in chunk order (the result does not
 * depend on the order in which they finish).  workspace: at least
 * fa_bwd_dkdv_workspace_bytes bytes, 16-byte aligned (may be NULL when that
 * is zero); two calls that share a workspace must not overlap in time.
 */
int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                const float* lse, const float* delta, void* dk, void* dv,
                int B, int H, int N, int d, float scale, int causal,
                const uint8_t* block_mask, const int32_t* kv_len, int dtype,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward stage 3: dq.  Each work-group owns 128 queries and walks the same
 * key tiles as the forward pass, recomputing S, P and dP.
 */
int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dO,
              const float* lse, const float* delta, void* dq,
              int B, int H, int N, int d, float scale, int causal,
              const uint8_t* block_mask, const int32_t* kv_len, int dtype, void* stream);

/*
 * Backward stages 1 and 3 in one: dq as fa_bwd_dq, with delta [B,H,N] float32
 * = rowsum(dO * O) formed by the dQ kernel from o and dO (each row by the
 * work-group that owns it, fp32 accumulation) and written to `delta` for
 * fa_bwd_dkdv, which must run after it on the same stream.  The same
 * quantities as fa_bwd_preprocess followed by fa_bwd_dq (delta may differ in
 * the last bits: another summation order), without the separate pass over dO
 * and O.  FA_F32 runs exactly those two calls.  Errors as fa_bwd_dq; o as for
 * fa_bwd.
 */
int fa_bwd_dq_delta(const void* q, const void* k, const void* v, const void* o, const void* dO,
                    const float* lse, float* delta, void* dq,
                    int B, int H, int N, int d, float scale, int causal,
                    const uint8_t* block_mask, const int32_t* kv_len, int dtype, void* stream);

/*
 * Test hook for the tile-skip schedule.  Runs the tile walk of the forward
 * (which = 0), dk/dv (1) or dq (2) kernel -- the same iteration code, with the
 * arithmetic compiled out -- and adds 1 to counts[b][i][j] (uint32, [B][T][T],
 * zeroed by the caller) for every head h and every visited cell (query cell i,
 * key cell j).  A cell is visited iff block_mask[i][j] != 0, (not causal or
 * j <= i) and 128*j < kv_len[b].  d and dtype select the kernel instance.
 * workspace: as for fa_bwd_dkdv when which = 1, else unused (may be NULL);
 * with a split column each chunk counts its own cells.
 */
int fa_debug_visits(int which, int B, int H, int N, int d, int causal,
                    const uint8_t* block_mask, const int32_t* kv_len, int dtype,
                    uint32_t* counts, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward and backward passes with dropout on the attention probabilities.
 * The pages list dropout among the operations fused into the attention
 * kernel (FlashAttention reading guide, "Ide Utama", kernel-fusion bullet)
 * but give no formula; these entry points implement:
 *   O = (P * Z) V,  Z_ij = keep_ij / (1 - p),  lse as without dropout,
 * with keep_ij decided by byte (j & 3) of word (i & 3) of Philox4x32-10
 * (Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011)
 * with key (seed & 0xffffffff, seed >> 32) and counter
 * (j >> 2, i >> 2, b * H + h, 0): kept iff that byte >= t, where
 * t = round(256 * dropout_p) must be <= 255 (the effective rate is t / 256;
 * t = 0 is no dropout).  The backward pass regenerates the same bytes from
 * the same seed; fa_bwd_dropout must get the dropout_p and seed fa_fwd_dropout
 * used.  Gradients: dV = (P * Z)^T dO, dP = (dO V^T) * Z,
 * dS = P * (dP - delta), dQ = scale dS K, dK = scale dS^T Q.
 * Errors as fa_fwd / fa_bwd, plus FA_ERR_ARG if dropout_p is not in [0, 1)
 * or rounds to 256, and FA_ERR_DTYPE for a nonzero rate with FA_F32 (the
 * float32 path has no dropout).  Workspace as fa_bwd.
 */
int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int causal,
                   const uint8_t* block_mask, const int32_t* kv_len, int dtype,
                   float dropout_p, uint64_t seed, void* stream);

int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dO,
                   const float* lse, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, float scale, int causal,
                   const uint8_t* block_mask, const int32_t* kv_len, int dtype,
                   float dropout_p, uint64_t seed,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Split-key forward for few queries against many keys (decoding, chunked
 * prefill).  The pages motivate splitting attention along the sequence when
 * batch x heads alone cannot fill the device (datacamp "Penjelasan Flash
 * Attention", Flash Attention 2, "Paralelisme sepanjang panjang sekuens").
 * Here the keys of each (b, h) are cut into num_splits contiguous ranges;
 * each range runs the forward pass's incremental softmax over its keys and
 * writes an unnormalised float32 partial output with its row statistics
 * (m, l); a second kernel combines the ranges of every row with the
 * two-block rule of the incremental softmax (FlashAttention reading guide,
 * "Pelacakan Softmax Inkremental": m = max m_s, l = sum_s e^{m_s - m} l_s,
 * O = sum_s e^{m_s - m} O_s / l).  With Nq <= 4 one wave handles a range of
 * one (b, h) (a bandwidth-bound kernel, ranges of whole 64-key tiles);
 * otherwise one work-group handles a range for 128 queries of one (b, h)
 * (the matrix-core forward kernel, ranges of whole 128-key cells).
 *   q, o     [B,H,Nq,d] bf16;  k, v  [B,H,Nk,d] bf16;  lse [B,H,Nq] float32.
 *   d        64, 96, 128, 160 or 256 (with 96 and 160, Nq * d and Nk * d
 *            <= 2^30).
 *   causal   nonzero: queries are the last Nq of Nk positions, so key j is
 *            allowed for query i iff j <= i + Nk - Nq (for Nk = Nq this is
 *            fa_fwd's mask; queries with i + Nk - Nq < 0 have no key).
 *   kv_len   NULL or device int32 [B], clamped to [0, Nk]; no block mask.
 *   dtype    FA_BF16 only (FA_ERR_DTYPE otherwise).
 *   num_splits  0 = chosen from the sizes (as many ranges as keep every
 *            wave or work-group resident at once), else 1..1024; ranges are
 *            whole tiles or cells, so fewer may be used
 *            (fa_fwd_splitkv_num_splits reports the count).
 *   workspace  at least fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d,
 *            num_splits) bytes, 16-byte aligned, no initialisation needed
 *            (nsplit x B*H*Nq x (d + 2) float32); calls sharing a workspace
 *            must not overlap in time.
 * Errors as fa_fwd; FA_ERR_ARG also for num_splits outside 0..1024.  Nk = 0
 * gives O = 0 and lse = -inf.  k and v may be NULL when Nk = 0.
 */
size_t fa_fwd_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits);

/* Number of key ranges fa_fwd_splitkv uses for these sizes (0 for empty or
 * invalid sizes). */
int fa_fwd_splitkv_num_splits(int B, int H, int Nq, int Nk, int num_splits);

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Nq, int Nk, int d, float scale, int causal,
                   const int32_t* kv_len, int dtype, int num_splits,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_fwd_splitkv without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The partial results go to a fixed
 * device buffer of FA_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends; the call itself allocates nothing.
 * Arguments, results and errors are those of fa_fwd_splitkv (the same kernels
 * and range plan, so the outputs are bit-identical), plus FA_ERR_SCRATCH when
 * fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, num_splits) exceeds
 * FA_NOALLOC_SCRATCH_BYTES (checked before anything is launched; an explicit
 * smaller num_splits needs less).  The stream must belong to the current
 * device, whose buffer is used.  Every call on one GPU shares that GPU's
 * buffer, which keeps the last call's contents (nothing in it needs to start
 * at zero): calls that overlap in time on one GPU race.
 */
int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Nq, int Nk, int d, float scale, int causal,
                           const int32_t* kv_len, int dtype, int num_splits, void* stream);

/*
 * Decoding against an 8-bit key/value cache: fa_fwd_splitkv for Nq <= 4 bf16
 * queries with K and V stored as OCP E4M3 codes ([B,H,Nk,d] uint8, real
 * value = decode(code) * k_descale or * v_descale; the format as for
 * fa_fwd_fp8 below).  Reading K and V is the whole cost of decoding, so the
 * 8-bit cache halves it -- the memory-traffic saving the pages give for FP8
 * (datacamp "Penjelasan Flash Attention", Flash Attention 3, "Presisi FP8
 * native").  Scores are bf16 query x E4M3 key products (each E4M3 value is
 * exactly a bf16 value) with fp32 accumulation; probabilities and the P V
 * accumulation stay fp32.  Arguments, masks, splits, workspace
 * (fa_fwd_splitkv_workspace_bytes) and errors as fa_fwd_splitkv;
 * FA_ERR_SHAPE if Nq > 4; FA_ERR_ARG for a descale that is not finite and
 * > 0.
 */
int fa_fwd_splitkv_fp8kv(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int H, int Nq, int Nk, int d, float scale, int causal,
                         const int32_t* kv_len, float k_descale, float v_descale, int num_splits,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward pass on 8-bit floating point inputs.  The pages name native FP8 as
 * FlashAttention-3's way to halve memory traffic (datacamp "Penjelasan Flash
 * Attention", Flash Attention 3, "Presisi FP8 native") without a format or
 * scaling rule; this entry point reads it as:
 *   q, k, v  [B,H,N,d] OCP E4M3 codes (uint8: 1 sign, 4 exponent bits with
 *            bias 7, 3 mantissa bits, subnormals, S.1111.111 = NaN), each
 *            tensor with one float32 descale: real value = decode(code) *
 *            descale (q_descale, k_descale, v_descale finite and > 0);
 *   o        [B,H,N,d] bf16 and lse [B,H,N] float32 as fa_fwd, of the real
 *            values: O = softmax(scale (dq Q)(dk K)^T [masked]) (dv V).
 * Both products run on the fp8 matrix core with fp32 accumulation; the
 * probabilities are converted to E4M3 for the P V product (relative rounding
 * up to 2^-4 per entry), while the running max, row sum and final division
 * stay fp32.  d = 64 or 128; masks, errors and conventions as fa_fwd.  There
 * is no FP8 backward pass.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal,
               const uint8_t* block_mask, const int32_t* kv_len,
               float q_descale, float k_descale, float v_descale, void* stream);

/* Static, NUL-terminated name of a status code. */
const char* fa_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
