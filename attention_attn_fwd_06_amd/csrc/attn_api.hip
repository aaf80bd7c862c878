// C ABI of the attention library: argument validation, status codes and
// kernel dispatch.  Every entry point validates all arguments before touching
// the GPU, launches asynchronously on the caller's stream, never allocates and
// never synchronises.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "../../include/attn.h"

namespace attn {
hipError_t prefill_dispatch(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                            int Hq, int Hkv, int N, int M, int d, bool causal, bool bf16, float scale,
                            const attn_strides_t& st, hipStream_t stream);
hipError_t prefill_fp8qk_dispatch(const void* q8, const void* k8, const void* v, void* o, float* lse, int B, int Hq,
                                  int Hkv, int N, int M, int d, bool causal, bool bf16, float scale, float q_scale,
                                  float k_scale, const attn_strides_t& st, hipStream_t stream);
hipError_t decode_dispatch(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                           int B, int Hq, int Hkv, int M, int d, int chunk, bool bf16, float scale,
                           hipStream_t stream);
hipError_t merge_dispatch(const float* o_part, const float* lse_part, void* o, float* lse, int B, int Hq,
                          int C, int d, bool bf16, hipStream_t stream);
hipError_t decode_paged_dispatch(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, const int32_t* seq_lens, int num_blocks,
                                 int block_size, int max_blocks, int64_t page_stride, int64_t token_stride,
                                 int64_t head_stride, float* o_part, float* lse_part, int B, int Hq, int Hkv,
                                 int d, int chunk, bool bf16, float scale, bool fp8, float k_scale,
                                 float v_scale, hipStream_t stream);
hipError_t decode_fp8kv_dispatch(const void* q, const void* k, const void* v, float k_scale, float v_scale,
                                 float* o_part, float* lse_part, int B, int Hq, int Hkv, int M, int d, int chunk,
                                 bool bf16, float scale, hipStream_t stream);
hipError_t decode_fused_dispatch(const void* q, const void* k, const void* v, void* o, float* lse, void* ws,
                                 size_t ws_bytes, int B, int Hq, int Hkv, int M, int d, bool bf16, float scale,
                                 hipStream_t stream);
hipError_t decode_fp8kv_fused_dispatch(const void* q, const void* k, const void* v, float k_scale, float v_scale,
                                       void* o, float* lse, void* ws, size_t ws_bytes, int B, int Hq, int Hkv, int M,
                                       int d, bool bf16, float scale, hipStream_t stream);
hipError_t decode_paged_fused_dispatch(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_table, const int32_t* seq_lens, int num_blocks,
                                       int block_size, int max_blocks, int64_t page_stride, int64_t token_stride,
                                       int64_t head_stride, void* o, float* lse, void* ws, size_t ws_bytes, int B,
                                       int Hq, int Hkv, int d, bool bf16, float scale, bool fp8, float k_scale,
                                       float v_scale, hipStream_t stream);
size_t fused_workspace_layout(int B, int Hq, int Hkv, int d, int S, size_t* off_lse, size_t* off_o);
int fused_segment_cap(int B, int Hq, int Hkv, int M);
size_t scratch_capacity();
void* scratch_address();
}  // namespace attn

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 31;  // 32-bit element offsets per dimension product
constexpr int kDecodeChunk = 128;       // chunk sizes are multiples of this
constexpr int kDecodeChunkMax = 8192;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool valid_head_dim(int d) { return d == 32 || d == 64 || d == 128; }
bool valid_prefill_head_dim(int d) { return valid_head_dim(d) || d == 256; }
// the 16-bit decode, its merge and the fused decode (the FP8-KV decode keeps valid_head_dim)
bool valid_decode_head_dim(int d) { return valid_head_dim(d) || d == 256; }
bool valid_dtype(int dt) { return dt == ATTN_F16 || dt == ATTN_BF16; }

int launch_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH; }

// Index ranges of the split-KV decode: a (batch, kv head) slice of K or V is
// read through 32-bit offsets (up to one 128-key sub-chunk past M); the
// partials and q are addressed with 64-bit offsets; the chunk items
// (B * Hq * C at most) are counted in 32-bit integers; the merge grid has
// B * Hq workgroups in one dimension.
bool decode_too_large(int B, int Hq, int64_t M, int d, int chunk_size) {
  const int64_t C = (M + chunk_size - 1) / chunk_size;
  return (int64_t)B * Hq * C >= kMaxElems || (int64_t)B * Hq > 65535 || (M + kDecodeChunk) * d >= kMaxElems;
}

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NULL_POINTER: return "a required pointer is NULL";
    case ATTN_ERR_BAD_DIMENSION: return "a size argument is not positive";
    case ATTN_ERR_HEAD_DIM: return "unsupported head dimension (prefill and 16-bit decode: 32, 64, 128, 256; FP8 prefill: 64, 128; FP8-KV decode: 32, 64, 128)";
    case ATTN_ERR_DTYPE: return "dtype must be ATTN_F16 or ATTN_BF16";
    case ATTN_ERR_GQA_GROUPS: return "Hq must be a multiple of Hkv";
    case ATTN_ERR_CAUSAL_SHAPE: return "causal attention requires N <= M (bottom-right mask)";
    case ATTN_ERR_CHUNK_SIZE: return "decode chunk size must be a multiple of 128, at most 8192";
    case ATTN_ERR_LAUNCH: return "HIP kernel launch failed";
    case ATTN_ERR_TOO_LARGE: return "a size exceeds the supported index range";
    case ATTN_ERR_ALIGNMENT: return "tensor pointers must be 16-byte aligned";
    case ATTN_ERR_SCALE: return "scales must be finite and >= 0";
    case ATTN_ERR_WORKSPACE: return "workspace missing, misaligned or smaller than attn_decode_fused_workspace_bytes";
    case ATTN_ERR_SCRATCH: return "the call needs more than the library's static scratch (16 MiB)";
    case ATTN_ERR_LAYOUT:
      return "strides must be >= 0 and multiples of 8 elements (k and v: one token stride >= d; paged: "
             "block_size a multiple of 16, 15 * token_stride + d < 2^31)";
    default: return "unknown status";
  }
}

int attn_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                     int N, int M, int d, int causal, float scale, attn_dtype_t dtype,
                     const attn_strides_t* strides, hipStream_t stream) {
  if (!q || !k || !v || !o) return ATTN_ERR_NULL_POINTER;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || M <= 0 || d <= 0) return ATTN_ERR_BAD_DIMENSION;
  if (!valid_prefill_head_dim(d)) return ATTN_ERR_HEAD_DIM;
  if (!valid_dtype(dtype)) return ATTN_ERR_DTYPE;
  if (Hq % Hkv != 0) return ATTN_ERR_GQA_GROUPS;
  if (causal && N > M) return ATTN_ERR_CAUSAL_SHAPE;
  if (!std::isfinite(scale) || scale < 0.f) return ATTN_ERR_SCALE;
  attn_strides_t st;
  if (strides) {
    st = *strides;
  } else {
    const int64_t qn = (int64_t)Hq * d, kn = (int64_t)Hkv * d;
    st = attn_strides_t{{N * qn, qn, d}, {M * kn, kn, d}, {M * kn, kn, d}, {N * qn, qn, d}};
  }
  const int64_t* all[4] = {st.q, st.k, st.v, st.o};
  for (const int64_t* t : all)
    for (int i = 0; i < 3; ++i)
      if (t[i] < 0 || t[i] % 8 != 0) return ATTN_ERR_LAYOUT;
  // k and v share one token stride of at least d (key rows past M must lie
  // beyond the last key row, where the bounds-checked tile loads return zeros)
  if (st.k[1] != st.v[1] || st.k[1] < d) return ATTN_ERR_LAYOUT;
  // q, o and lse are addressed with 64-bit offsets; the kernel reads one
  // (batch, kv head) slice of K or V through a buffer descriptor with 32-bit
  // byte offsets, up to one tile of 64 rows past M, so (M + 64) token rows
  // must stay below 2^31 elements.  The grid holds B * Hq * ceil(N / 64)
  // workgroups at most.
  if ((int64_t)(M + 64) * st.k[1] + d >= kMaxElems || (int64_t)B * Hq * ((N + 63) / 64) >= kMaxElems)
    return ATTN_ERR_TOO_LARGE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return ATTN_ERR_ALIGNMENT;
  return launch_status(attn::prefill_dispatch(q, k, v, o, lse, B, Hq, Hkv, N, M, d, causal != 0,
                                              dtype == ATTN_BF16, scale, st, stream));
}

int attn_fwd_fp8qk(const void* q8, const void* k8, const void* v, void* o, float* lse, float q_scale, float k_scale,
                   int B, int Hq, int Hkv, int N, int M, int d, int causal, float scale, attn_dtype_t dtype,
                   hipStream_t stream) {
  if (!q8 || !k8 || !v || !o) return ATTN_ERR_NULL_POINTER;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || M <= 0 || d <= 0) return ATTN_ERR_BAD_DIMENSION;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (!valid_dtype(dtype)) return ATTN_ERR_DTYPE;
  if (Hq % Hkv != 0) return ATTN_ERR_GQA_GROUPS;
  if (causal && N > M) return ATTN_ERR_CAUSAL_SHAPE;
  if (!std::isfinite(scale) || scale < 0.f || !std::isfinite(q_scale) || q_scale < 0.f || !std::isfinite(k_scale) ||
      k_scale < 0.f)
    return ATTN_ERR_SCALE;
  const int64_t qn = (int64_t)Hq * d, kn = (int64_t)Hkv * d;
  // contiguous layouts (element strides; the FP8 elements are bytes)
  const attn_strides_t st{{N * qn, qn, d}, {M * kn, kn, d}, {M * kn, kn, d}, {N * qn, qn, d}};
  if ((int64_t)(M + 64) * kn + d >= kMaxElems || (int64_t)B * Hq * ((N + 63) / 64) >= kMaxElems)
    return ATTN_ERR_TOO_LARGE;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v) || !aligned16(o) ||
      (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return ATTN_ERR_ALIGNMENT;
  return launch_status(attn::prefill_fp8qk_dispatch(q8, k8, v, o, lse, B, Hq, Hkv, N, M, d, causal != 0,
                                                    dtype == ATTN_BF16, scale, q_scale, k_scale, st, stream));
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int N,
             int M, int d, int causal, float scale, attn_dtype_t dtype, hipStream_t stream) {
  return attn_fwd_strided(q, k, v, o, lse, B, Hq, Hkv, N, M, d, causal, scale, dtype, nullptr, stream);
}

size_t attn_decode_workspace_bytes(int B, int Hq, int M, int d, int chunk_size) {
  if (B <= 0 || Hq <= 0 || M <= 0 || d <= 0 || chunk_size <= 0) return 0;
  const int64_t C = ((int64_t)M + chunk_size - 1) / chunk_size;
  return (size_t)((int64_t)B * Hq * C * (d + 1) * 4);
}

int attn_decode_splitkv(const void* q, const void* k, const void* v, float* o_part, float* lse_part, int B,
                        int Hq, int Hkv, int M, int d, int chunk_size, float scale, attn_dtype_t dtype,
                        hipStream_t stream) {
  if (!q || !k || !v || !o_part || !lse_part) return ATTN_ERR_NULL_POINTER;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || M <= 0 || d <= 0 || chunk_size <= 0) return ATTN_ERR_BAD_DIMENSION;
  if (!valid_decode_head_dim(d)) return ATTN_ERR_HEAD_DIM;
  if (!valid_dtype(dtype)) return ATTN_ERR_DTYPE;
  if (Hq % Hkv != 0) return ATTN_ERR_GQA_GROUPS;
  if (chunk_size % kDecodeChunk != 0 || chunk_size > kDecodeChunkMax) return ATTN_ERR_CHUNK_SIZE;
  if (!std::isfinite(scale) || scale < 0.f) return ATTN_ERR_SCALE;
  if (decode_too_large(B, Hq, M, d, chunk_size)) return ATTN_ERR_TOO_LARGE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (reinterpret_cast<uintptr_t>(o_part) & 3u) ||
      (reinterpret_cast<uintptr_t>(lse_part) & 3u))
    return ATTN_ERR_ALIGNMENT;
  return launch_status(attn::decode_dispatch(q, k, v, o_part, lse_part, B, Hq, Hkv, M, d, chunk_size,
                                             dtype == ATTN_BF16, scale, stream));
}

size_t attn_decode_fused_workspace_bytes(int B, int Hq, int Hkv, int M, int d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || M <= 0 || d <= 0 || Hq % Hkv != 0 || !valid_decode_head_dim(d)) return 0;
  return attn::fused_workspace_layout(B, Hq, Hkv, d, attn::fused_segment_cap(B, Hq, Hkv, M), nullptr, nullptr);
}

int attn_decode_fused(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                      size_t workspace_bytes, int B, int Hq, int Hkv, int M, int d, float scale, attn_dtype_t dtype,
                      hipStream_t stream) {
  if (!q || !k || !v || !o) return ATTN_ERR_NULL_POINTER;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || M <= 0 || d <= 0) return ATTN_ERR_BAD_DIMENSION;
  if (!valid_decode_head_dim(d)) return ATTN_ERR_HEAD_DIM;
  if (!valid_dtype(dtype)) return ATTN_ERR_DTYPE;
  if (Hq % Hkv != 0) return ATTN_ERR_GQA_GROUPS;
  if (!std::isfinite(scale) || scale < 0.f) return ATTN_ERR_SCALE;
  if (decode_too_large(B, Hq, M, d, kDecodeChunk)) return ATTN_ERR_TOO_LARGE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return ATTN_ERR_ALIGNMENT;
  if (!workspace || !aligned16(workspace) ||
      workspace_bytes < attn_decode_fused_workspace_bytes(B, Hq, Hkv, M, d))
    return ATTN_ERR_WORKSPACE;
  return launch_status(attn::decode_fused_dispatch(q, k, v, o, lse, workspace, workspace_bytes, B, Hq, Hkv, M, d,
                                                   dtype == ATTN_BF16, scale, stream));
}

int attn_decode_fused_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                              int Hkv, int M, int d, float scale, attn_dtype_t dtype, hipStream_t stream) {
  if (!q || !k || !v || !o) return ATTN_ERR_NULL_POINTER;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || M <= 0 || d <= 0) return ATTN_ERR_BAD_DIMENSION;
  if (!valid_decode_head_dim(d)) return ATTN_ERR_HEAD_DIM;
  if (!valid_dtype(dtype)) return ATTN_ERR_DTYPE;
  if (Hq % Hkv != 0) return ATTN_ERR_GQA_GROUPS;
  if (!std::isfinite(scale) || scale < 0.f) return ATTN_ERR_SCALE;
  if (decode_too_large(B, Hq, M, d, kDecodeChunk)) return ATTN_ERR_TOO_LARGE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return ATTN_ERR_ALIGNMENT;
  // the same bound as a caller's workspace, so the outcome does not depend on the GPU
  if (attn_decode_fused_workspace_bytes(B, Hq, Hkv, M, d) > attn::scratch_capacity()) return ATTN_ERR_SCRATCH;
  void* ws = attn::scratch_address();
  if (ws == nullptr) return ATTN_ERR_LAUNCH;
  return launch_status(attn::decode_fused_dispatch(q, k, v, o, lse, ws, attn::scratch_capacity(), B, Hq, Hkv, M, d,
                                                   dtype == ATTN_BF16, scale, stream));
}

int attn_decode_fp8kv_splitkv(const void* q, const void* k, const void* v, float k_scale, float v_scale,
                              float* o_part, float* lse_part, int B, int Hq, int Hkv, int M, int d, int chunk_size,
                              float scale, attn_dtype_t dtype, hipStream_t stream) {
  if (!q || !k || !v || !o_part || !lse_part) return ATTN_ERR_NULL_POINTER;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || M <= 0 || d <= 0 || chunk_size <= 0) return ATTN_ERR_BAD_DIMENSION;
  if (!valid_head_dim(d)) return ATTN_ERR_HEAD_DIM;
  if (!valid_dtype(dtype)) return ATTN_ERR_DTYPE;
  if (Hq % Hkv != 0) return ATTN_ERR_GQA_GROUPS;
  if (chunk_size % kDecodeChunk != 0 || chunk_size > kDecodeChunkMax) return ATTN_ERR_CHUNK_SIZE;
  if (!std::isfinite(scale) || scale < 0.f || !std::isfinite(k_scale) || k_scale < 0.f || !std::isfinite(v_scale) ||
      v_scale < 0.f)
    return ATTN_ERR_SCALE;
  if (decode_too_large(B, Hq, M, d, chunk_size)) return ATTN_ERR_TOO_LARGE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (reinterpret_cast<uintptr_t>(o_part) & 3u) ||
      (reinterpret_cast<uintptr_t>(lse_part) & 3u))
    return ATTN_ERR_ALIGNMENT;
  return launch_status(attn::decode_fp8kv_dispatch(q, k, v, k_scale, v_scale, o_part, lse_part, B, Hq, Hkv, M, d,
                                                   chunk_size, dtype == ATTN_BF16, scale, stream));
}

int attn_decode_fp8kv_fused(const void* q, const void* k, const void* v, float k_scale, float v_scale, void* o,
                            float* lse, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int M, int d,
                            float scale, attn_dtype_t dtype, hipStream_t stream) {
  if (!q || !k || !v || !o) return ATTN_ERR_NULL_POINTER;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || M <= 0 || d <= 0) return ATTN_ERR_BAD_DIMENSION;
  if (!valid_head_dim(d)) return ATTN_ERR_HEAD_DIM;
  if (!valid_dtype(dtype)) return ATTN_ERR_DTYPE;
  if (Hq % Hkv != 0) return ATTN_ERR_GQA_GROUPS;
  if (!std::isfinite(scale) || scale < 0.f || !std::isfinite(k_scale) || k_scale < 0.f || !std::isfinite(v_scale) ||
      v_scale < 0.f)
    return ATTN_ERR_SCALE;
  if (decode_too_large(B, Hq, M, d, kDecodeChunk)) return ATTN_ERR_TOO_LARGE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return ATTN_ERR_ALIGNMENT;
  if (!workspace || !aligned16(workspace) ||
      workspace_bytes < attn_decode_fused_workspace_bytes(B, Hq, Hkv, M, d))
    return ATTN_ERR_WORKSPACE;
  return launch_status(attn::decode_fp8kv_fused_dispatch(q, k, v, k_scale, v_scale, o, lse, workspace,
                                                         workspace_bytes, B, Hq, Hkv, M, d, dtype == ATTN_BF16, scale,
                                                         stream));
}

}  // extern "C"

namespace {

// Checks shared by the paged entry points: pointers, sizes, head dim, dtype,
// groups, scales, the page layout, index ranges and alignment of the inputs
// (chunk_size 128 for the fused call).
int check_paged(const void* q, const void* k_cache, const void* v_cache, const attn_paged_kv_t* pages, int B,
                int Hq, int Hkv, int d, int chunk_size, float scale, attn_dtype_t dtype, bool fp8, float k_scale,
                float v_scale) {
  if (!q || !k_cache || !v_cache || !pages || !pages->block_table || !pages->seq_lens) return ATTN_ERR_NULL_POINTER;
  const attn_paged_kv_t& pk = *pages;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || chunk_size <= 0 || pk.num_blocks <= 0 || pk.block_size <= 0 ||
      pk.max_blocks <= 0)
    return ATTN_ERR_BAD_DIMENSION;
  if (fp8 ? !valid_head_dim(d) : !valid_decode_head_dim(d)) return ATTN_ERR_HEAD_DIM;
  if (!valid_dtype(dtype)) return ATTN_ERR_DTYPE;
  if (Hq % Hkv != 0) return ATTN_ERR_GQA_GROUPS;
  if (chunk_size % kDecodeChunk != 0 || chunk_size > kDecodeChunkMax) return ATTN_ERR_CHUNK_SIZE;
  if (!std::isfinite(scale) || scale < 0.f || !std::isfinite(k_scale) || k_scale < 0.f || !std::isfinite(v_scale) ||
      v_scale < 0.f)
    return ATTN_ERR_SCALE;
  // element strides; FP8 elements are bytes, so the 16-byte alignment of a row needs multiples of 16 there
  const int64_t align = fp8 ? 16 : 8;
  if (pk.block_size % 16 != 0 || pk.page_stride < 0 || pk.token_stride < 0 || pk.head_stride < 0 ||
      pk.page_stride % align || pk.token_stride % align || pk.head_stride % align ||
      15 * pk.token_stride + d >= kMaxElems)
    return ATTN_ERR_LAYOUT;
  const int64_t M = (int64_t)pk.max_blocks * pk.block_size;
  if (M >= ((int64_t)1 << 30) || decode_too_large(B, Hq, M, d, chunk_size)) return ATTN_ERR_TOO_LARGE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (reinterpret_cast<uintptr_t>(pk.block_table) & 3u) || (reinterpret_cast<uintptr_t>(pk.seq_lens) & 3u))
    return ATTN_ERR_ALIGNMENT;
  return ATTN_OK;
}

int paged_decode(const void* q, const void* k_cache, const void* v_cache, const attn_paged_kv_t* pages,
                 float* o_part, float* lse_part, int B, int Hq, int Hkv, int d, int chunk_size, float scale,
                 attn_dtype_t dtype, bool fp8, float k_scale, float v_scale, hipStream_t stream) {
  if (!o_part || !lse_part) return ATTN_ERR_NULL_POINTER;
  const int st = check_paged(q, k_cache, v_cache, pages, B, Hq, Hkv, d, chunk_size, scale, dtype, fp8, k_scale,
                             v_scale);
  if (st != ATTN_OK) return st;
  if ((reinterpret_cast<uintptr_t>(o_part) & 3u) || (reinterpret_cast<uintptr_t>(lse_part) & 3u))
    return ATTN_ERR_ALIGNMENT;
  const attn_paged_kv_t& pk = *pages;
  return launch_status(attn::decode_paged_dispatch(q, k_cache, v_cache, pk.block_table, pk.seq_lens, pk.num_blocks,
                                                   pk.block_size, pk.max_blocks, pk.page_stride, pk.token_stride,
                                                   pk.head_stride, o_part, lse_part, B, Hq, Hkv, d, chunk_size,
                                                   dtype == ATTN_BF16, scale, fp8, k_scale, v_scale, stream));
}

int paged_fused(const void* q, const void* k_cache, const void* v_cache, const attn_paged_kv_t* pages, void* o,
                float* lse, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int d, float scale,
                attn_dtype_t dtype, bool fp8, float k_scale, float v_scale, hipStream_t stream) {
  if (!o) return ATTN_ERR_NULL_POINTER;
  const int st = check_paged(q, k_cache, v_cache, pages, B, Hq, Hkv, d, kDecodeChunk, scale, dtype, fp8, k_scale,
                             v_scale);
  if (st != ATTN_OK) return st;
  if (!aligned16(o) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u))) return ATTN_ERR_ALIGNMENT;
  const attn_paged_kv_t& pk = *pages;
  const int M = pk.max_blocks * pk.block_size;
  if (!workspace || !aligned16(workspace) ||
      workspace_bytes < attn_decode_fused_workspace_bytes(B, Hq, Hkv, M, d))
    return ATTN_ERR_WORKSPACE;
  return launch_status(attn::decode_paged_fused_dispatch(q, k_cache, v_cache, pk.block_table, pk.seq_lens,
                                                         pk.num_blocks, pk.block_size, pk.max_blocks, pk.page_stride,
                                                         pk.token_stride, pk.head_stride, o, lse, workspace,
                                                         workspace_bytes, B, Hq, Hkv, d, dtype == ATTN_BF16, scale,
                                                         fp8, k_scale, v_scale, stream));
}

}  // namespace

extern "C" {

int attn_decode_paged_splitkv(const void* q, const void* k_cache, const void* v_cache,
                              const attn_paged_kv_t* pages, float* o_part, float* lse_part, int B, int Hq,
                              int Hkv, int d, int chunk_size, float scale, attn_dtype_t dtype, hipStream_t stream) {
  return paged_decode(q, k_cache, v_cache, pages, o_part, lse_part, B, Hq, Hkv, d, chunk_size, scale, dtype, false,
                      1.f, 1.f, stream);
}

int attn_decode_paged_fused(const void* q, const void* k_cache, const void* v_cache, const attn_paged_kv_t* pages,
                            void* o, float* lse, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                            int d, float scale, attn_dtype_t dtype, hipStream_t stream) {
  return paged_fused(q, k_cache, v_cache, pages, o, lse, workspace, workspace_bytes, B, Hq, Hkv, d, scale, dtype,
                     false, 1.f, 1.f, stream);
}

int attn_decode_paged_fp8kv_fused(const void* q, const void* k_cache, const void* v_cache, float k_scale,
                                  float v_scale, const attn_paged_kv_t* pages, void* o, float* lse, void* workspace,
                                  size_t workspace_bytes, int B, int Hq, int Hkv, int d, float scale,
                                  attn_dtype_t dtype, hipStream_t stream) {
  return paged_fused(q, k_cache, v_cache, pages, o, lse, workspace, workspace_bytes, B, Hq, Hkv, d, scale, dtype,
                     true, k_scale, v_scale, stream);
}

int attn_decode_paged_fp8kv_splitkv(const void* q, const void* k_cache, const void* v_cache, float k_scale,
                                    float v_scale, const attn_paged_kv_t* pages, float* o_part, float* lse_part,
                                    int B, int Hq, int Hkv, int d, int chunk_size, float scale, attn_dtype_t dtype,
                                    hipStream_t stream) {
  return paged_decode(q, k_cache, v_cache, pages, o_part, lse_part, B, Hq, Hkv, d, chunk_size, scale, dtype, true,
                      k_scale, v_scale, stream);
}

int lse_merge(const float* o_part, const float* lse_part, void* o, float* lse, int B, int Hq, int num_chunks,
              int d, attn_dtype_t out_dtype, hipStream_t stream) {
  if (!o_part || !lse_part || !o) return ATTN_ERR_NULL_POINTER;
  if (B <= 0 || Hq <= 0 || num_chunks <= 0 || d <= 0) return ATTN_ERR_BAD_DIMENSION;
  if (!valid_decode_head_dim(d)) return ATTN_ERR_HEAD_DIM;
  if (!valid_dtype(out_dtype)) return ATTN_ERR_DTYPE;
  if ((int64_t)B * Hq * num_chunks >= kMaxElems || (int64_t)B * Hq > 65535) return ATTN_ERR_TOO_LARGE;
  if (!aligned16(o_part) || (reinterpret_cast<uintptr_t>(lse_part) & 3u) ||
      (reinterpret_cast<uintptr_t>(o) & 1u) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return ATTN_ERR_ALIGNMENT;
  return launch_status(
      attn::merge_dispatch(o_part, lse_part, o, lse, B, Hq, num_chunks, d, out_dtype == ATTN_BF16, stream));
}

}  // extern "C"
