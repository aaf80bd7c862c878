// Split-KV decode ("Flash Decoding") for gfx950: the per-chunk partial kernel
// and the log-sum-exp merge kernel ("CUDA Flash Decoding", section 2.2: chunk
// partials O_c, lse_c and the weighted reduce; section 3: the two-kernel data
// flow; section 6: the reduce kernel).
//
// MI355X design (not the page's CUDA design):
//  * chunk kernel: persistent grid of 256-thread workgroups (as many as fit
//    on the chip at once), each taking (chunk of 128 keys, batch, query head)
//    items in turn, so the grid drains evenly.  Every K and V load of a chunk
//    (64 KB at d = 128) is issued up front, with a nontemporal hint: V does not depend on the scores, so the whole chunk is in flight
//    at once and the kernel streams HBM.  A row of K/V (d * 2 bytes) is read by
//    d/8 consecutive lanes, 16 bytes each (fully coalesced).
//  * scores use fp32 accumulation (v_dot2_f32_{f16,bf16}) and a DPP sum over the
//    lanes that share a key row; softmax statistics use exp2 with the scale
//    folded into one multiply; partials are written in fp32, O_c normalised.
//  * merge kernel: one workgroup per (batch, query head, 16-column slice of d),
//    one pass over the partials with a running max (no separate pass for the
//    global log-sum-exp, no limit on the number of chunks), 16-byte loads, and
//    eight independent loads in flight per thread; the 64 per-thread states
//    of a column are combined by lane shuffles and one LDS step.
#include <algorithm>

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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load that streams past the caches (K/V are read exactly once).
__device__ __forceinline__ uint4 load_stream(const uint16_t* p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Persistent grid: workgroup w handles items w, w + gridDim.x, ... where item
// = c + C * (G-head slice of one GQA group, b, kv head), so every workgroup
// ends at about the same time.  An item reads its chunk of K and V once and
// serves G query heads of the group that share them (G = 1 without GQA).
template <int D, bool BF16, int G>
__global__ __launch_bounds__(kDecThreads)
void decode_chunk_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                         const uint16_t* __restrict__ v, float* __restrict__ o_part,
                         float* __restrict__ lse_part, int Hq, int Hkv, int M, int C,
                         int n_items, float scale_log2) {
  constexpr int kLanes = D / 8;                       // lanes per key row
  constexpr int kRowsPerPass = kDecThreads / kLanes;  // 16 (d=128) or 32 (d=64)
  constexpr int kPasses = kChunk / kRowsPerPass;      // rows per thread
  constexpr int kWaves = kDecThreads / 64;
  __shared__ float red[2][kWaves][G];
  __shared__ float opart[kWaves][G][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = tid % kLanes;  // 16-byte column chunk
  const int r0 = tid / kLanes;   // first row of this thread
  const int group = Hq / Hkv;
  const int slices = group / G;  // G-head slices per GQA group

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int c = item % C;
    const int rest = item / C;
    const int hs = rest % slices, bkv = rest / slices;
    const int kvh = bkv % Hkv, b = bkv / Hkv;
    const int h0 = kvh * group + hs * G;  // first query head of this item
    const int key0 = c * kChunk;
    const int len = min(kChunk, M - key0);

    const uint16_t* kp = k + (((int64_t)b * Hkv + kvh) * M + key0) * D + col * 8;
    const uint16_t* vp = v + (((int64_t)b * Hkv + kvh) * M + key0) * D + col * 8;
    uint4 qv[G];
#pragma unroll
    for (int i = 0; i < G; ++i)
      qv[i] = *reinterpret_cast<const uint4*>(q + ((int64_t)b * Hq + h0 + i) * D + col * 8);

    // issue the whole chunk: K then V
    uint4 kr[kPasses], vr[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int row = r0 + p * kRowsPerPass;
      kr[p] = row < len ? load_stream(kp + (int64_t)row * D) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int row = r0 + p * kRowsPerPass;
      vr[p] = row < len ? load_stream(vp + (int64_t)row * D) : make_uint4(0, 0, 0, 0);
    }

    // scores in log2 units: x_j = scale * log2(e) * q.k_j, per head
    float x[kPasses][G];
    float mx[G];
#pragma unroll
    for (int i = 0; i < G; ++i) mx[i] = -INFINITY;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int row = r0 + p * kRowsPerPass;
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const float sdot = row_sum<kLanes>(dot8<BF16>(qv[i], kr[p], 0.f));
        x[p][i] = row < len ? sdot * scale_log2 : -INFINITY;
        mx[i] = fmaxf(mx[i], x[p][i]);
      }
    }
    // chunk max: over the rows of this wave, then over the waves
#pragma unroll
    for (int i = 0; i < G; ++i) {
      float m = fmaxf(mx[i], __shfl_xor(mx[i], 16));
      m = max_xor32(m);
      if (kLanes == 8) m = fmaxf(m, __shfl_xor(m, 8));
      if (lane == 0) red[0][wave][i] = m;
    }
    __syncthreads();
    float m[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      m[i] = red[0][0][i];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) m[i] = fmaxf(m[i], red[0][w][i]);
    }

    float acc[G][8];
    float l[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      l[i] = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[i][t] = 0.f;
    }
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int row = r0 + p * kRowsPerPass;
      const uint32_t* vw = reinterpret_cast<const uint32_t*>(&vr[p]);
      f32x2 vv[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) vv[t] = unpack2<BF16>(vw[t]);
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const float e = row < len ? __builtin_amdgcn_exp2f(x[p][i] - m[i]) : 0.f;
        l[i] += e;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          acc[i][2 * t] = fmaf(e, vv[t][0], acc[i][2 * t]);
          acc[i][2 * t + 1] = fmaf(e, vv[t][1], acc[i][2 * t + 1]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      // l: the lanes of a row group hold the same e; sum over the row groups
      // of the wave, then across waves.
      float li = l[i] + __shfl_xor(l[i], 16);
      li = sum_xor32(li);
      if (kLanes == 8) li += __shfl_xor(li, 8);
      // column partials: reduce the lanes that share a column chunk
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        float a = acc[i][t];
        if (kLanes == 8) a += __shfl_xor(a, 8);
        a += __shfl_xor(a, 16);
        a = sum_xor32(a);
        acc[i][t] = a;
      }
      if (lane < kLanes) {
#pragma unroll
        for (int t = 0; t < 8; ++t) opart[wave][i][lane * 8 + t] = acc[i][t];
      }
      if (lane == 0) red[1][wave][i] = li;
    }
    __syncthreads();
    if (tid < D) {
#pragma unroll
      for (int i = 0; i < G; ++i) {
        float lt = 0.f, ot = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          lt += red[1][w][i];
          ot += opart[w][i][tid];
        }
        const int64_t base = ((int64_t)b * Hq + h0 + i) * C + c;
        o_part[base * D + tid] = ot / lt;
        if (tid == 0) lse_part[base] = (m[i] + log2f(lt)) * kLn2;
      }
    }
    __syncthreads();  // opart / red reused by the next item
  }
}

constexpr int kMergeThreads = 256;
constexpr int kMergeCols = 16;                          // d columns per workgroup
constexpr int kMergeGroups = kMergeThreads / (kMergeCols / 4);  // chunk groups (64)

// (m, s, a[4]) merge of two running states, in log2 units: both rescaled to
// the larger reference max.  A state with m = -inf (no chunk yet) is empty.
struct MergeState {
  float m, s, a[4];
};
__device__ __forceinline__ MergeState merge_states(const MergeState& x, const MergeState& y) {
  const float mm = fmaxf(x.m, y.m);
  const float rx = (x.m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(x.m - mm);
  const float ry = (y.m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(y.m - mm);
  MergeState r;
  r.m = mm;
  r.s = fmaf(x.s, rx, y.s * ry);
#pragma unroll
  for (int c = 0; c < 4; ++c) r.a[c] = fmaf(x.a[c], rx, y.a[c] * ry);
  return r;
}

// One pass over the partials: each thread walks chunks grp, grp + 64, ... of one
// (batch, head) and 4 consecutive columns, keeping a running max of lse_c (log2
// units) with the matching rescaled weight sum and weighted output; the 64
// group states are then combined with the same rule, first across the lanes
// of each wave (xor shuffles over the group bits of the lane id), then across
// the 4 waves.  O = sum_c 2^(l_c - M) O_c / sum_c 2^(l_c - M) for any
// reference M equals sum_c w_c O_c.
template <int D, bool BF16>
__global__ __launch_bounds__(kMergeThreads)
void lse_merge_kernel(const float* __restrict__ o_part, const float* __restrict__ lse_part,
                      uint16_t* __restrict__ o, float* __restrict__ lse, int C) {
  constexpr int kWaves = kMergeThreads / 64;
  __shared__ MergeState part[kWaves][4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cq = tid & 3, grp = tid >> 2;
  const int bh = blockIdx.x;
  const int col0 = blockIdx.y * kMergeCols + cq * 4;
  const float* lp = lse_part + (int64_t)bh * C;
  const float* op = o_part + (int64_t)bh * C * D + col0;

  MergeState st = {-INFINITY, 0.f, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll 8
  for (int c = grp; c < C; c += kMergeGroups) {
    const float l2 = lp[c] * kLog2e;
    const float4 ov = *reinterpret_cast<const float4*>(op + (int64_t)c * D);
    const float mn = fmaxf(st.m, l2);
    const float r = __builtin_amdgcn_exp2f(st.m - mn);   // 0 on the first chunk (m = -inf)
    const float w = __builtin_amdgcn_exp2f(l2 - mn);
    st.s = fmaf(st.s, r, w);
    st.a[0] = fmaf(st.a[0], r, w * ov.x);
    st.a[1] = fmaf(st.a[1], r, w * ov.y);
    st.a[2] = fmaf(st.a[2], r, w * ov.z);
    st.a[3] = fmaf(st.a[3], r, w * ov.w);
    st.m = mn;
  }
  // lanes that share cq differ in lane bits 2..5
#pragma unroll
  for (int mask = 4; mask < 64; mask <<= 1) {
    MergeState y;
    y.m = __shfl_xor(st.m, mask);
    y.s = __shfl_xor(st.s, mask);
#pragma unroll
    for (int c = 0; c < 4; ++c) y.a[c] = __shfl_xor(st.a[c], mask);
    st = merge_states(st, y);
  }
  if (lane < 4) part[wave][lane] = st;
  __syncthreads();
  if (tid < 4) {
    MergeState r = part[0][tid];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) r = merge_states(r, part[w][tid]);
    const float inv = 1.f / r.s;
    const int d0 = blockIdx.y * kMergeCols + tid * 4;
    const uint32_t w01 = pack2<BF16>(r.a[0] * inv, r.a[1] * inv);
    const uint32_t w23 = pack2<BF16>(r.a[2] * inv, r.a[3] * inv);
    *reinterpret_cast<uint2*>(o + (int64_t)bh * D + d0) = make_uint2(w01, w23);
    if (blockIdx.y == 0 && tid == 0 && lse != nullptr) lse[bh] = (r.m + log2f(r.s)) * kLn2;
  }
}

// Resident workgroups per CU for a kernel, times the CU count (cached per device).
template <typename K>
static int resident_grid(K kernel, int threads) {
  constexpr int kMaxDev = 64;
  static int cache[kMaxDev] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < kMaxDev && cache[dev] > 0) return cache[dev];
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  const int g = cus * per_cu;
  if (dev < kMaxDev) cache[dev] = g;
  return g;
}

hipError_t decode_dispatch(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                           int B, int Hq, int Hkv, int M, int d, bool bf16, float scale, hipStream_t stream) {
  const int C = (M + kChunk - 1) / kChunk;
  const float sl2 = scale * kLog2e;
  // query heads per item: the largest of 4, 2, 1 that divides the GQA group
  const int group = Hq / Hkv;
  const int g = group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
  const int n_items = B * (Hq / g) * C;
#define ATTN_DEC_CASE(DD, BB, GG)                                                                      \
  if (d == DD && bf16 == BB && g == GG) {                                                              \
    const int grid = std::min(n_items, resident_grid(decode_chunk_kernel<DD, BB, GG>, kDecThreads));   \
    hipLaunchKernelGGL((decode_chunk_kernel<DD, BB, GG>), dim3(grid), dim3(kDecThreads), 0, stream,    \
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, o_part, lse_part,   \
                       Hq, Hkv, M, C, n_items, sl2);                                                   \
    return hipGetLastError();                                                                          \
  }
  ATTN_DEC_CASE(64, false, 1) ATTN_DEC_CASE(64, false, 2) ATTN_DEC_CASE(64, false, 4)
  ATTN_DEC_CASE(64, true, 1) ATTN_DEC_CASE(64, true, 2) ATTN_DEC_CASE(64, true, 4)
  ATTN_DEC_CASE(128, false, 1) ATTN_DEC_CASE(128, false, 2) ATTN_DEC_CASE(128, false, 4)
  ATTN_DEC_CASE(128, true, 1) ATTN_DEC_CASE(128, true, 2) ATTN_DEC_CASE(128, true, 4)
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
