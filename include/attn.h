/*
 * attn.h - C ABI of the MI355X (gfx950) fused attention forward library.
 *
 * Operations (definitions from the pages, in their notation):
 *   attn_fwd             fused attention forward, O = softmax(scale * Q K^T [+causal]) V,
 *                        computed tile by tile with an online softmax so that the score
 *                        and probability matrices never reach HBM ("fmha sm120: beyond
 *                        torch.sdpa", section 1 "flash attention" and section 2 "fmha
 *                        implementation").
 *   attn_fwd_fp8qk       attn_fwd with Q and K as FP8 E4M3 codes and per-tensor scales
 *                        (Q K^T on the FP8 matrix cores).
 *   attn_decode_splitkv  Flash-Decoding step 1: per-chunk partial outputs O_c and
 *                        log-sum-exp lse_c of a single query ("CUDA Flash Decoding",
 *                        section 2.2, step 1).
 *   attn_decode_paged_splitkv  the same partials over a paged KV cache with
 *                        per-sequence lengths (attention over KV-cache blocks, listed
 *                        as future work on the "fmha sm120" page; layout is the
 *                        library's, see attn_paged_kv_t).
 *   attn_decode_fp8kv_splitkv  the same partials with K and V stored as FP8 E4M3
 *                        codes and per-tensor scales (fp8 KV quantisation, listed as
 *                        future work on the "fmha sm120" page).
 *   attn_decode_paged_fp8kv_splitkv  both: a paged cache of FP8 codes.
 *   attn_decode_fused    both Flash-Decoding steps in one launch, the merge done by the
 *                        last workgroup of each row (a per-row counter in a caller-owned
 *                        workspace); attn_decode_paged_fused, attn_decode_fp8kv_fused and
 *                        attn_decode_paged_fp8kv_fused do the same for the paged, FP8 and
 *                        paged FP8 partials.
 *   lse_merge            Flash-Decoding step 2: O = sum_c w_c O_c with
 *                        w_c = exp(lse_c - logsumexp_c lse_c) ("CUDA Flash Decoding",
 *                        section 2.2, step 2, and section 6 "reduce kernel").
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are device memory owned by the caller, contiguous in the
 *     stated layout, and 16-byte aligned.  The library never allocates, frees,
 *     synchronises or throws; work is enqueued on `stream` (NULL = the default
 *     stream) and completes asynchronously.
 *   - The return value is ATTN_OK (0) or a negative attn_status_t.  On any error
 *     nothing is launched and no output is touched, except ATTN_ERR_LAUNCH, which
 *     reports a failed kernel launch (outputs are then undefined).
 *   - Outputs must not alias inputs.  fp16/bf16 outputs are rounded to nearest even
 *     from fp32.  All accumulation is fp32.
 *   - Inputs holding Inf/NaN propagate NaN to the affected outputs.
 */
#ifndef ATTN_MI355X_H
#define ATTN_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP stream type, declared exactly as HIP declares it. */
typedef struct ihipStream_t* hipStream_t;

typedef enum {
  ATTN_F16 = 0,  /* IEEE binary16 */
  ATTN_BF16 = 1  /* bfloat16 */
} attn_dtype_t;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL_POINTER = -1,   /* a required pointer is NULL */
  ATTN_ERR_BAD_DIMENSION = -2,  /* a size is <= 0 */
  ATTN_ERR_HEAD_DIM = -3,       /* head dimension d not supported by the call (attn_fwd:
                                   {32, 64, 128, 256}; attn_fwd_fp8qk: {64, 128}; 16-bit
                                   decode, fused decode and merge: {32, 64, 128, 256};
                                   FP8-KV decode: {32, 64, 128}) */
  ATTN_ERR_DTYPE = -4,          /* dtype not an attn_dtype_t value */
  ATTN_ERR_GQA_GROUPS = -5,     /* Hq is not a multiple of Hkv */
  ATTN_ERR_CAUSAL_SHAPE = -6,   /* causal requested with N > M */
  ATTN_ERR_CHUNK_SIZE = -7,     /* decode chunk size not a multiple of 128 or above 8192 */
  ATTN_ERR_LAUNCH = -8,         /* the HIP launch failed (the launch's own status) */
  ATTN_ERR_TOO_LARGE = -9,      /* a size exceeds the library's index range */
  ATTN_ERR_ALIGNMENT = -10,     /* a tensor pointer is not 16-byte aligned */
  ATTN_ERR_SCALE = -11,         /* scale is negative, infinite or NaN */
  ATTN_ERR_LAYOUT = -12,        /* strides: negative, not a multiple of 8 elements, or k and v
                                   token strides differ or are below d */
  ATTN_ERR_WORKSPACE = -13,     /* workspace NULL, not 16-byte aligned, or too small */
  ATTN_ERR_SCRATCH = -14        /* attn_decode_fused_noalloc: the sizes need more than the
                                   library's static scratch */
} attn_status_t;

/*
 * Element strides of the four prefill tensors, each {batch, token, head}; the
 * head-dimension elements of one (batch, token, head) are contiguous.  For the
 * contiguous layouts of attn_fwd they are q, o: {N*Hq*d, Hq*d, d} and
 * k, v: {M*Hkv*d, Hkv*d, d}.
 */
typedef struct {
  int64_t q[3], k[3], v[3], o[3];
} attn_strides_t;

/*
 * attn_fwd - fused multi-head / grouped-query attention forward (prefill).
 *
 *   q   [B, N, Hq, d]   dtype, read        o   [B, N, Hq, d]  dtype, written
 *   k   [B, M, Hkv, d]  dtype, read        lse [B, Hq, N]     fp32, written (may be NULL)
 *   v   [B, M, Hkv, d]  dtype, read
 *
 * For batch b and query head h the key/value head is h / (Hq / Hkv) (contiguous
 * groups, "fmha sm120", section 2).  S = scale * Q K^T; with causal != 0 key j is
 * masked for query i when j > i + (M - N): the N queries are the last N positions
 * of the key sequence (a chunk of a longer prefill), so the last query sees every
 * key; for N == M this is the page's top-left mask.  Causal requires N <= M;
 * O = softmax(S) V row by row, and lse[b,h,i] = ln sum_j exp(S_ij) (natural log,
 * including the row maximum).  Requires d in {32, 64, 128, 256}, Hq % Hkv == 0, a finite
 * scale >= 0, (M+64)*Hkv*d below 2^31 (one batch's K or V, read with 32-bit
 * offsets) and B*Hq*ceil(N/64) below 2^31; q, o and lse have no size limit
 * of their own (64-bit offsets).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int N, int M, int d, int causal, float scale,
             attn_dtype_t dtype, hipStream_t stream);

/*
 * attn_fwd_strided - attn_fwd on tensors laid out with arbitrary element strides
 * (views such as the q, k, v slices of one fused [B, N, 3, H, d] projection, or
 * head-major [B, H, N, d] tensors); same operation, masks, outputs and errors as
 * attn_fwd ("fmha sm120: beyond torch.sdpa", sections 1 and 2).  lse stays
 * [B, Hq, N] contiguous.  strides == NULL means the contiguous layouts.  Every
 * stride must be >= 0 and a multiple of 8 elements (so that every row of d
 * values starts 16-byte aligned), and k and v must share one token stride of at
 * least d (otherwise ATTN_ERR_LAYOUT).  (M + 64) times the k/v token stride must
 * stay below 2^31 (otherwise ATTN_ERR_TOO_LARGE).  Outputs must not overlap inputs or each other.
 */
int attn_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int N, int M, int d, int causal, float scale,
                     attn_dtype_t dtype, const attn_strides_t* strides, hipStream_t stream);

/*
 * attn_fwd_fp8qk - attn_fwd with Q and K given as FP8 E4M3 codes and one fp32
 * scale each (fp8 attention, listed as future work on the "fmha sm120" page,
 * which fixes no format; the format is the library's).
 *
 *   q8  [B, N, Hq, d]   E4M3 codes, read     o   [B, N, Hq, d]  dtype, written
 *   k8  [B, M, Hkv, d]  E4M3 codes, read     lse [B, Hq, N]     fp32, written (may be NULL)
 *   v   [B, M, Hkv, d]  dtype (fp16/bf16), read
 *
 * The queries and keys are Q = q_scale * e4m3(q8) and K = k_scale * e4m3(k8)
 * (OCP E4M3: sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, S.1111.111 is NaN); the result is attn_fwd on Q, K and v:
 * O = softmax(scale * Q K^T [+ causal mask]) V and its lse, with the masks,
 * layouts, outputs and errors of attn_fwd.  Q K^T runs on the FP8 matrix
 * cores (products of E4M3 values are exact, accumulation fp32); the softmax
 * and P V are those of the 16-bit path.  Requires d in {64, 128} (else
 * ATTN_ERR_HEAD_DIM) and finite scales >= 0 (else ATTN_ERR_SCALE).
 */
int attn_fwd_fp8qk(const void* q8, const void* k8, const void* v, void* o, float* lse,
                   float q_scale, float k_scale,
                   int B, int Hq, int Hkv, int N, int M, int d, int causal, float scale,
                   attn_dtype_t dtype, hipStream_t stream);

/*
 * attn_decode_workspace_bytes - bytes of fp32 partials that one split-KV decode call
 * writes: B*Hq*C*(d+1)*4 with C = ceil(M / chunk_size).  The caller may carve
 * o_part (B*Hq*C*d floats) and lse_part (B*Hq*C floats) out of one buffer of this
 * size.  Returns 0 for invalid sizes.
 */
size_t attn_decode_workspace_bytes(int B, int Hq, int M, int d, int chunk_size);

/*
 * attn_decode_splitkv - per-chunk partials of single-query attention.
 *
 *   q   [B, Hq, d]        dtype, read     o_part   [B, Hq, C, d]  fp32, written
 *   k   [B, Hkv, M, d]    dtype, read     lse_part [B, Hq, C]     fp32, written
 *   v   [B, Hkv, M, d]    dtype, read
 *
 * Chunk c covers keys [c*chunk_size, min((c+1)*chunk_size, M)); the last chunk may
 * be shorter.  For each chunk: s_j = scale * q.k_j, m_c = max_j s_j,
 * p_j = exp(s_j - m_c), l_c = sum p_j, o_part = (sum_j p_j v_j) / l_c (normalised),
 * lse_part = m_c + ln l_c ("CUDA Flash Decoding", section 2.2 step 1).  No mask.
 * Requires chunk_size a multiple of 128 and at most 8192 (longer chunks mean fewer
 * partials for lse_merge to read), d in {32, 64, 128, 256}, Hq % Hkv == 0, a finite
 * scale >= 0, B*Hq <= 65535, B*Hq*C and (M + 128)*d below 2^31 (one (batch, kv
 * head) slice of K or V is read with 32-bit offsets).
 */
int attn_decode_splitkv(const void* q, const void* k, const void* v,
                        float* o_part, float* lse_part,
                        int B, int Hq, int Hkv, int M, int d, int chunk_size, float scale,
                        attn_dtype_t dtype, hipStream_t stream);

/*
 * attn_decode_fused_workspace_bytes - bytes of device workspace that
 * attn_decode_fused needs for these sizes (0 for invalid sizes).  It holds one
 * counter per (batch, kv head, head slice) and the fp32 partial output and
 * log-sum-exp of every segment the launch may split the keys into.
 */
size_t attn_decode_fused_workspace_bytes(int B, int Hq, int Hkv, int M, int d);

/*
 * attn_decode_fused - split-KV decode end to end in one launch: the partials
 * of attn_decode_splitkv and the merge of lse_merge ("CUDA Flash Decoding",
 * section 2.2 steps 1 and 2; fusing the reduce into the chunk kernel is the
 * page's section 8 lever of a last-block reduce).
 *
 *   q   [B, Hq, d]      dtype, read     o   [B, Hq, d]  dtype, written
 *   k   [B, Hkv, M, d]  dtype, read     lse [B, Hq]     fp32, written (may be NULL)
 *   v   [B, Hkv, M, d]  dtype, read
 *
 * The keys of each (batch, query head) are split into segments of whole
 * 128-key chunks (the library picks how many from the sizes and the GPU, at
 * most attn_decode_fused_workspace_bytes' worth); each segment's normalised
 * output O_s and lse_s go to the workspace, and the workgroup that finishes a
 * row's last segment merges them with w_s = exp(lse_s - logsumexp_s lse_s).
 * The result is that of attn_decode_splitkv + lse_merge up to rounding.
 *
 * workspace: device memory of at least attn_decode_fused_workspace_bytes(B,
 * Hq, Hkv, M, d) bytes, 16-byte aligned, owned by the caller.  Its counters
 * must be zero before the first call (fill the buffer with zeros once); every
 * call that completes leaves them zero again, so the same workspace serves
 * any later call of any size that fits.  Calls that may run at the same time
 * (other streams) need workspaces of their own.  Requires the conditions of
 * attn_decode_splitkv for chunk_size 128 (else its status codes) and
 * ATTN_ERR_WORKSPACE for a NULL, misaligned or short workspace.
 */
int attn_decode_fused(const void* q, const void* k, const void* v, void* o, float* lse,
                      void* workspace, size_t workspace_bytes,
                      int B, int Hq, int Hkv, int M, int d, float scale,
                      attn_dtype_t dtype, hipStream_t stream);

/*
 * attn_decode_fused_noalloc - attn_decode_fused without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The call
 * allocates nothing: its workspace is a static 16 MiB device array of the
 * library (one per GPU, held until the process ends), whose counters start
 * at zero and are set back to zero by every completed call.  Same operation,
 * arguments, outputs and status codes as attn_decode_fused, plus
 * ATTN_ERR_SCRATCH when attn_decode_fused_workspace_bytes(B, Hq, Hkv, M, d)
 * exceeds 16 MiB.  All calls on one GPU share the array: calls that may
 * overlap on one GPU (several streams or threads) race and must not be made.
 */
int attn_decode_fused_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int Hq, int Hkv, int M, int d, float scale,
                              attn_dtype_t dtype, hipStream_t stream);

/*
 * Paged KV cache for attn_decode_paged_splitkv (the "fmha sm120" page lists
 * attention over KV-cache blocks as future work and defines no layout; this is
 * the library's).  A page holds block_size consecutive keys of every KV head;
 * element (page p, key row r, kv head h, column c) of k_cache / v_cache is at
 * p*page_stride + r*token_stride + h*head_stride + c (elements; the columns are
 * contiguous).  [num_blocks, block_size, Hkv, d] token-major pages have strides
 * {block_size*Hkv*d, Hkv*d, d}; [num_blocks, Hkv, block_size, d] head-major pages
 * {Hkv*block_size*d, d, block_size*d}.  Key t of sequence b is row
 * t % block_size of page block_table[b*max_blocks + t / block_size]; sequence b
 * holds seq_lens[b] keys (0 .. max_blocks*block_size; a length above that is
 * taken as max_blocks*block_size, a negative one as 0).  A sequence of 0 keys
 * has no chunk with a key: after lse_merge its o is 0 and its lse is -inf.
 * The page ids of a sequence's first ceil(seq_lens[b] / block_size) table
 * entries must lie in [0, num_blocks); entries past those are never used.  An
 * id out of range is never dereferenced: its rows are taken as keys and values
 * of all zeros (so they still enter the softmax, with score 0), which is the
 * result of no valid cache.  block_table and seq_lens are device memory, read
 * by the kernel.
 */
typedef struct {
  const int32_t* block_table;   /* [B, max_blocks] page ids in [0, num_blocks) */
  const int32_t* seq_lens;      /* [B] keys per sequence */
  int num_blocks;               /* pages in each cache */
  int block_size;               /* keys per page, a multiple of 16 */
  int max_blocks;               /* columns of block_table */
  int64_t page_stride, token_stride, head_stride;  /* element strides, multiples of 8 */
} attn_paged_kv_t;

/*
 * attn_decode_paged_splitkv - attn_decode_splitkv over a paged KV cache with
 * per-sequence lengths.
 *
 *   q        [B, Hq, d]     dtype, read
 *   k_cache, v_cache        dtype, read (layout in attn_paged_kv_t, same strides)
 *   o_part   [B, Hq, C, d]  fp32, written;  lse_part [B, Hq, C] fp32, written
 *
 * with C = ceil(max_blocks*block_size / chunk_size).  Sequence b's chunks are
 * those of attn_decode_splitkv on its keys; chunks past its end get o_part = 0
 * and lse_part = -inf, which lse_merge gives no weight.  Requires the attn_decode_splitkv conditions on
 * B, Hq, Hkv, d, chunk_size and scale, block_size % 16 == 0, strides >= 0 and
 * multiples of 8 with 15*token_stride + d below 2^31 (else ATTN_ERR_LAYOUT),
 * and max_blocks*block_size below 2^30.  The workspace size is
 * attn_decode_workspace_bytes(B, Hq, max_blocks*block_size, d, chunk_size).
 */
int attn_decode_paged_splitkv(const void* q, const void* k_cache, const void* v_cache,
                              const attn_paged_kv_t* pages, float* o_part, float* lse_part,
                              int B, int Hq, int Hkv, int d, int chunk_size, float scale,
                              attn_dtype_t dtype, hipStream_t stream);

/*
 * attn_decode_paged_fused - attn_decode_paged_splitkv at chunk size 128 and
 * lse_merge in one launch (the paged counterpart of attn_decode_fused).
 *
 *   q        [B, Hq, d]  dtype, read      o   [B, Hq, d]  dtype, written
 *   k_cache, v_cache     dtype, read      lse [B, Hq]     fp32, written (may be NULL)
 *                        (layout in attn_paged_kv_t)
 *
 * The keys of sequence b (see attn_paged_kv_t) are split into segments of
 * whole 128-key chunks of the longest sequence the table can describe
 * (max_blocks*block_size keys); segments past the sequence's end have no key
 * and no weight, and a sequence of 0 keys gets o = 0 and lse = -inf.  The
 * result is that of attn_decode_paged_splitkv + lse_merge up to rounding.
 * workspace: at least attn_decode_fused_workspace_bytes(B, Hq, Hkv,
 * max_blocks*block_size, d) bytes, 16-byte aligned, with the conventions of
 * attn_decode_fused (its counters zero before the first call and left zero
 * by every completed call; calls that may run at the same time need
 * workspaces of their own).  Requires the attn_decode_paged_splitkv
 * conditions at chunk size 128, a 16-byte aligned o, and ATTN_ERR_WORKSPACE
 * for a NULL, misaligned or short workspace.
 */
int attn_decode_paged_fused(const void* q, const void* k_cache, const void* v_cache, const attn_paged_kv_t* pages,
                            void* o, float* lse, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                            int d, float scale, attn_dtype_t dtype, hipStream_t stream);

/*
 * attn_decode_paged_fp8kv_splitkv - attn_decode_paged_splitkv over a paged cache
 * of FP8 E4M3 codes with per-tensor scales (as attn_decode_fp8kv_splitkv): key
 * and value elements are one byte, so the element strides are byte strides and
 * must be multiples of 16, and d in {32, 64, 128}.  Otherwise as
 * attn_decode_paged_splitkv, including
 * the zero rows in place of out-of-range page ids (for those the kernel reads
 * 16 bytes at the start of the cache, page 0, which num_blocks >= 1
 * guarantees, and discards them).
 */
int attn_decode_paged_fp8kv_splitkv(const void* q, const void* k_cache, const void* v_cache,
                                    float k_scale, float v_scale, const attn_paged_kv_t* pages,
                                    float* o_part, float* lse_part, int B, int Hq, int Hkv, int d,
                                    int chunk_size, float scale, attn_dtype_t dtype, hipStream_t stream);

/*
 * attn_decode_fp8kv_splitkv - attn_decode_splitkv with K and V stored as FP8.
 *
 *   q        [B, Hq, d]     dtype (fp16 or bf16), read
 *   k, v     [B, Hkv, M, d] OCP FP8 E4M3 codes (one byte each), read
 *   o_part, lse_part        as attn_decode_splitkv
 *
 * The keys and values are K = k_scale * e4m3(k) and V = v_scale * e4m3(v) (one
 * fp32 scale per tensor; the "fmha sm120" page lists fp8 KV quantisation as
 * future work and fixes no format).  Codes are converted exactly to dtype
 * inside the kernel; the products and sums are those of attn_decode_splitkv.
 * NaN codes (S.1111.111) give NaN.  Requires the attn_decode_splitkv
 * conditions with d in {32, 64, 128} (else ATTN_ERR_HEAD_DIM) and finite
 * scales >= 0 (else ATTN_ERR_SCALE).
 */
int attn_decode_fp8kv_splitkv(const void* q, const void* k, const void* v, float k_scale, float v_scale,
                              float* o_part, float* lse_part,
                              int B, int Hq, int Hkv, int M, int d, int chunk_size, float scale,
                              attn_dtype_t dtype, hipStream_t stream);

/*
 * attn_decode_fp8kv_fused - attn_decode_fp8kv_splitkv at chunk size 128 and
 * lse_merge in one launch (the FP8 counterpart of attn_decode_fused).
 *
 *   q    [B, Hq, d]     dtype (fp16 or bf16), read   o   [B, Hq, d] dtype, written
 *   k, v [B, Hkv, M, d] FP8 E4M3 codes, read         lse [B, Hq]    fp32, written (may be NULL)
 *
 * K = k_scale * e4m3(k), V = v_scale * e4m3(v) as in attn_decode_fp8kv_splitkv;
 * segments, merge and workspace (attn_decode_fused_workspace_bytes(B, Hq, Hkv,
 * M, d) bytes, counters zero before the first call and left zero by every
 * completed call, one workspace per concurrently running call) as in
 * attn_decode_fused.  The result is that of attn_decode_fp8kv_splitkv +
 * lse_merge up to rounding.  Requires the attn_decode_fp8kv_splitkv conditions
 * at chunk size 128, a 16-byte aligned o, and ATTN_ERR_WORKSPACE for a NULL,
 * misaligned or short workspace.
 */
int attn_decode_fp8kv_fused(const void* q, const void* k, const void* v, float k_scale, float v_scale,
                            void* o, float* lse, void* workspace, size_t workspace_bytes,
                            int B, int Hq, int Hkv, int M, int d, float scale,
                            attn_dtype_t dtype, hipStream_t stream);

/*
 * attn_decode_paged_fp8kv_fused - attn_decode_paged_fp8kv_splitkv at chunk size
 * 128 and lse_merge in one launch: attn_decode_paged_fused over a paged cache
 * of FP8 E4M3 codes with per-tensor scales (byte strides, multiples of 16; d in
 * {32, 64, 128}).  Segments past a sequence's end have no key and no weight;
 * a sequence of 0 keys gets o = 0 and lse = -inf.  Requires the
 * attn_decode_paged_fp8kv_splitkv conditions at chunk size 128, a 16-byte
 * aligned o, and a workspace as for attn_decode_paged_fused (else
 * ATTN_ERR_WORKSPACE).
 */
int attn_decode_paged_fp8kv_fused(const void* q, const void* k_cache, const void* v_cache,
                                  float k_scale, float v_scale, const attn_paged_kv_t* pages,
                                  void* o, float* lse, void* workspace, size_t workspace_bytes,
                                  int B, int Hq, int Hkv, int d, float scale,
                                  attn_dtype_t dtype, hipStream_t stream);

/*
 * lse_merge - combine chunk partials into the decode output.
 *
 *   o_part   [B, Hq, C, d] fp32, read     o   [B, Hq, d]  out_dtype, written
 *   lse_part [B, Hq, C]    fp32, read     lse [B, Hq]     fp32, written (may be NULL)
 *
 * g = max_c lse_c + ln sum_c exp(lse_c - max_c lse_c), w_c = exp(lse_c - g),
 * o = sum_c w_c o_part[c], lse = g ("CUDA Flash Decoding", section 2.2 step 2).
 * A row whose lse_part are all -inf (no key at all, e.g. an empty paged
 * sequence) gets o = 0 and lse = -inf.  Requires num_chunks >= 1, d in
 * {32, 64, 128, 256}, B*Hq <= 65535 and B*Hq*num_chunks below 2^31.
 */
int lse_merge(const float* o_part, const float* lse_part, void* o, float* lse,
              int B, int Hq, int num_chunks, int d, attn_dtype_t out_dtype,
              hipStream_t stream);

/* A static, human-readable description of a status code (never NULL). */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_H */
