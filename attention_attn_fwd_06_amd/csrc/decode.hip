// Split-KV decode ("Flash Decoding") for gfx950: the per-chunk partial kernel
// and the log-sum-exp merge kernel ("CUDA Flash Decoding", section 2.2: chunk
// partials O_c, lse_c and the weighted reduce; section 3: the two-kernel data
// flow; section 6: the reduce kernel).
//
// MI355X design (not the page's CUDA design):
//  * chunk kernel: one 256-thread workgroup per (chunk of 128 keys, batch,
//    query head).  Every K and V load of the chunk (64 KB at d = 128) is issued
//    up front: V does not depend on the scores, so the whole chunk is in flight
//    at once and the kernel streams HBM.  A row of K/V (d * 2 bytes) is read by
//    d/8 consecutive lanes, 16 bytes each (fully coalesced).
//  * scores use fp32 accumulation (v_dot2_f32_{f16,bf16}) and a DPP sum over the
//    lanes that share a key row; softmax statistics use exp2 with the scale
//    folded into one multiply; partials are written in fp32, O_c normalised.
//  * merge kernel: one workgroup per (batch, query head, 32-column slice of d),
//    so the fp32 partials are read by many CUs at once; chunk weights are
//    recomputed from lse_c (no staging limit on the number of chunks).
#include "device_common.h"

namespace attn {

constexpr int kDecThreads = 256;
constexpr int kChunk = 128;

template <bool BF16>
__device__ __forceinline__ float dot8(const uint4& a, const uint4& b, float acc) {
  const uint32_t* x = reinterpret_cast<const uint32_t*>(&a);
  const uint32_t* y = reinterpret_cast<const uint32_t*>(&b);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (BF16)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x[e]), __builtin_bit_cast(bf16x2, y[e]),
                                            acc, false);
    else
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x[e]), __builtin_bit_cast(f16x2, y[e]), acc, false);
  }
  return acc;
}

// Sum over the kLanes (8 or 16) consecutive lanes that share one key row.
template <int kLanes>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (kLanes == 16) return sum16(x);
  else return sum8(x);
}

template <int D, bool BF16>
__global__ __launch_bounds__(kDecThreads)
void decode_chunk_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                         const uint16_t* __restrict__ v, float* __restrict__ o_part,
                         float* __restrict__ lse_part, int Hq, int Hkv, int M, int C,
                         float scale_log2) {
  constexpr int kLanes = D / 8;                     // lanes per key row
  constexpr int kRowsPerPass = kDecThreads / kLanes;  // 16 (d=128) or 32 (d=64)
  constexpr int kPasses = kChunk / kRowsPerPass;      // rows per thread
  constexpr int kWaves = kDecThreads / 64;
  __shared__ float red[kWaves];
  __shared__ float opart[kWaves][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x;
  const int bh = blockIdx.y;
  const int h = bh % Hq, b = bh / Hq;
  const int kvh = h / (Hq / Hkv);
  const int col = tid % kLanes;  // 16-byte column chunk
  const int r0 = tid / kLanes;   // first row of this thread
  const int key0 = c * kChunk;
  const int len = min(kChunk, M - key0);

  const uint16_t* kp = k + (((int64_t)b * Hkv + kvh) * M + key0) * D + col * 8;
  const uint16_t* vp = v + (((int64_t)b * Hkv + kvh) * M + key0) * D + col * 8;
  const uint4 qv = *reinterpret_cast<const uint4*>(q + ((int64_t)b * Hq + h) * D + col * 8);

  // issue the whole chunk: K then V
  uint4 kr[kPasses], vr[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int row = r0 + p * kRowsPerPass;
    kr[p] = row < len ? *reinterpret_cast<const uint4*>(kp + (int64_t)row * D) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int row = r0 + p * kRowsPerPass;
    vr[p] = row < len ? *reinterpret_cast<const uint4*>(vp + (int64_t)row * D) : make_uint4(0, 0, 0, 0);
  }

  // scores in log2 units: x_j = scale * log2(e) * q.k_j
  float x[kPasses];
  float mx = -INFINITY;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int row = r0 + p * kRowsPerPass;
    float sdot = row_sum<kLanes>(dot8<BF16>(qv, kr[p], 0.f));
    x[p] = row < len ? sdot * scale_log2 : -INFINITY;
    mx = fmaxf(mx, x[p]);
  }
  // chunk max: over the rows of this wave, then over the waves
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, max_xor32(mx));
  if (kLanes == 8) mx = fmaxf(mx, __shfl_xor(mx, 8));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) m = fmaxf(m, red[w]);

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int row = r0 + p * kRowsPerPass;
    const float e = row < len ? __builtin_amdgcn_exp2f(x[p] - m) : 0.f;
    l += e;
    const uint32_t* vw = reinterpret_cast<const uint32_t*>(&vr[p]);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f32x2 vv = unpack2<BF16>(vw[t]);
      acc[2 * t] = fmaf(e, vv[0], acc[2 * t]);
      acc[2 * t + 1] = fmaf(e, vv[1], acc[2 * t + 1]);
    }
  }
  // l: every lane of a row group holds the same e, so sum one lane per row group
  // over the rows of the wave, then across waves.
  l += __shfl_xor(l, 16);
  l = sum_xor32(l);
  if (kLanes == 8) l += __shfl_xor(l, 8);
  // column partials: reduce lanes with the same column chunk within the wave
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    float a = acc[t];
    if (kLanes == 8) a += __shfl_xor(a, 8);
    a += __shfl_xor(a, 16);
    a = sum_xor32(a);
    acc[t] = a;
  }
  __syncthreads();  // red[] reused below
  if (lane < kLanes) {
#pragma unroll
    for (int t = 0; t < 8; ++t) opart[wave][lane * 8 + t] = acc[t];
  }
  if (lane == 0) red[wave] = l;
  __syncthreads();
  if (tid < D) {
    float lt = 0.f, ot = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      lt += red[w];
      ot += opart[w][tid];
    }
    const int64_t base = ((int64_t)b * Hq + h) * C + c;
    o_part[base * D + tid] = ot / lt;
    if (tid == 0) lse_part[base] = (m + log2f(lt)) * kLn2;
  }
}

constexpr int kMergeThreads = 256;
constexpr int kMergeCols = 32;

template <int D, bool BF16>
__global__ __launch_bounds__(kMergeThreads)
void lse_merge_kernel(const float* __restrict__ o_part, const float* __restrict__ lse_part,
                      uint16_t* __restrict__ o, float* __restrict__ lse, int C) {
  constexpr int kGroups = kMergeThreads / kMergeCols;  // chunk groups
  constexpr int kWaves = kMergeThreads / 64;
  __shared__ float red[kWaves];
  __shared__ float part[kGroups][kMergeCols];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.x;
  const int slice = blockIdx.y;
  const float* lp = lse_part + (int64_t)bh * C;

  // g2 = log2 sum_c exp(lse_c), computed as max + log2 sum 2^(lse2_c - max)
  float mx = -INFINITY;
  for (int c = tid; c < C; c += kMergeThreads) mx = fmaxf(mx, lp[c] * kLog2e);
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  float gmax = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) gmax = fmaxf(gmax, red[w]);
  __syncthreads();
  float se = 0.f;
  for (int c = tid; c < C; c += kMergeThreads) se += __builtin_amdgcn_exp2f(lp[c] * kLog2e - gmax);
  for (int off = 32; off >= 1; off >>= 1) se += __shfl_xor(se, off);
  if (lane == 0) red[wave] = se;
  __syncthreads();
  float sum = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) sum += red[w];
  const float g2 = gmax + log2f(sum);

  // O[col] = sum_c 2^(lse2_c - g2) * O_c[col]
  const int col = tid % kMergeCols, grp = tid / kMergeCols;
  const int dcol = slice * kMergeCols + col;
  const float* op = o_part + (int64_t)bh * C * D + dcol;
  float acc = 0.f;
  for (int c = grp; c < C; c += kGroups)
    acc = fmaf(__builtin_amdgcn_exp2f(lp[c] * kLog2e - g2), op[(int64_t)c * D], acc);
  part[grp][col] = acc;
  __syncthreads();
  if (tid < kMergeCols) {
    float t = 0.f;
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi) t += part[gi][tid];
    const int d = slice * kMergeCols + tid;
    uint32_t packed = pack2<BF16>(t, 0.f);
    o[(int64_t)bh * D + d] = (uint16_t)(packed & 0xffffu);
    if (slice == 0 && tid == 0 && lse != nullptr) lse[bh] = g2 * kLn2;
  }
}

hipError_t decode_dispatch(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                           int B, int Hq, int Hkv, int M, int d, bool bf16, float scale, hipStream_t stream) {
  const int C = (M + kChunk - 1) / kChunk;
  const dim3 grid(C, B * Hq);
  const float sl2 = scale * kLog2e;
#define ATTN_DEC_CASE(DD, BB)                                                                         \
  if (d == DD && bf16 == BB) {                                                                        \
    hipLaunchKernelGGL((decode_chunk_kernel<DD, BB>), grid, dim3(kDecThreads), 0, stream,             \
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, o_part, lse_part,  \
                       Hq, Hkv, M, C, sl2);                                                           \
    return hipGetLastError();                                                                         \
  }
  ATTN_DEC_CASE(64, false)
  ATTN_DEC_CASE(64, true)
  ATTN_DEC_CASE(128, false)
  ATTN_DEC_CASE(128, true)
#undef ATTN_DEC_CASE
  return hipErrorInvalidValue;
}

hipError_t merge_dispatch(const float* o_part, const float* lse_part, void* o, float* lse, int B, int Hq,
                          int C, int d, bool bf16, hipStream_t stream) {
  const dim3 grid(B * Hq, d / kMergeCols);
#define ATTN_MERGE_CASE(DD, BB)                                                                  \
  if (d == DD && bf16 == BB) {                                                                   \
    hipLaunchKernelGGL((lse_merge_kernel<DD, BB>), grid, dim3(kMergeThreads), 0, stream, o_part, \
                       lse_part, (uint16_t*)o, lse, C);                                          \
    return hipGetLastError();                                                                    \
  }
  ATTN_MERGE_CASE(64, false)
  ATTN_MERGE_CASE(64, true)
  ATTN_MERGE_CASE(128, false)
  ATTN_MERGE_CASE(128, true)
#undef ATTN_MERGE_CASE
  return hipErrorInvalidValue;
}

}  // namespace attn
