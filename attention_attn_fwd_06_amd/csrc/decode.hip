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
#include "lds_stage.h"

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

// GQA decode on the matrix cores.  Item = (chunk c of 128 keys, batch b, kv
// head, slice of G <= 16 query heads of its group).  The G heads are the 16
// columns of v_mfma_f32_16x16x32 (columns >= G carry q = 0 and are never
// stored):
//   S^T[key][head] = K Q^T   A = K rows loaded from HBM straight into VGPRs,
//                            B = Q^T (the q rows of the slice's heads)
//   O^T[d][head]  = V^T P^T  A = V^T via ds_read_b64_tr_b16 from the V chunk
//                            fetched into LDS (swizzled, rows past M read as
//                            zeros), B = P^T from LDS as hi + lo 16-bit parts
// so the chunk's K and V are read from HBM once for all G heads.  Wave w
// scores keys 32w .. 32w + 31 and accumulates d rows w*D/4 .. +D/4 - 1 over all
// 128 keys.  The chunk max and sum are exchanged through LDS; P is the fp32
// 2^(x - m) split into two 16-bit parts, so the products keep fp32-level
// accuracy in P while l is the sum of the unrounded values.
constexpr int kGqaCols = 16;         // MFMA columns: query heads per item
constexpr int kPRow = kChunk + 8;    // P row stride in elements (16-byte pad)

template <int D, bool BF16>
__global__ __launch_bounds__(kDecThreads)
void decode_gqa_mfma_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                            const uint16_t* __restrict__ v, float* __restrict__ o_part,
                            float* __restrict__ lse_part, int Hq, int Hkv, int M, int C, int G,
                            int n_items, float scale_log2) {
  constexpr int kS = D / 32;                        // QK contraction steps
  constexpr int kDB = D / 64;                       // 16-row d blocks per wave
  constexpr int kWaves = kDecThreads / 64;
  constexpr int kU = D / 8;                         // 16-byte units per row
  constexpr int kRowsPerInst = kDecThreads / kU;    // rows per fetch instruction index
  constexpr int kFetch = kChunk / kRowsPerInst;     // fetch instructions per wave
  constexpr uint32_t kPBytes = kGqaCols * kPRow * 2;  // one P part
  static_assert(kRowsPerInst % 16 == 0, "swizzle must repeat across fetch instructions");
  __shared__ __attribute__((aligned(1024))) uint16_t vbuf[kChunk * D];
  __shared__ __attribute__((aligned(16))) uint16_t pbuf[2 * kGqaCols * kPRow];
  __shared__ float red[2][kWaves][kGqaCols];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int group = Hq / Hkv, slices = group / G;
  const uint32_t v_lds = (uint32_t)(uintptr_t)(lds_u16*)vbuf;
  const uint32_t p_lds = (uint32_t)(uintptr_t)(lds_u16*)pbuf;
  const bool out16 = ((uintptr_t)o_part & 15) == 0;

  // V fetch: instruction i of wave w fills LDS units (i*kWaves + w)*64 + lane,
  // i.e. row kRowsPerInst*i + rl, physical 16-byte chunk pc (holding logical
  // chunk pc ^ swz(row)).
  const int rl = (wave * 64 + lane) / kU, pc = lane % kU;
  const uint32_t voff_lane = (uint32_t)(rl * D * 2 + ((pc ^ swz<D>(rl)) << 4));
  // V^T operand: in each 16-lane group of a ds_read_b64_tr_b16, lane s
  // addresses V[K0 + s/4][D0 + 4*(s%4)], so lane i receives V[K0 + 0..3][D0 + i].
  // Group g reads keys 32*ks + 8*g + 4*hh + 0..3 (k-step ks, half hh): slots
  // 8g .. 8g + 7 of the k-step, the same key order the P^T read uses.
  uint32_t va[kDB][2];
#pragma unroll
  for (int db = 0; db < kDB; ++db) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int row = 8 * g + 4 * hh + (j >> 2);
      const int col = wave * (D / 4) + 16 * db + 4 * (j & 3);
      va[db][hh] = v_lds + (uint32_t)(row * D * 2 + ((((col >> 3) ^ swz<D>(row)) << 4) | ((col & 7) * 2)));
    }
  }
  const uint32_t pa = p_lds + (uint32_t)((j * kPRow + 8 * g) * 2);               // P[j][32ks + 8g ..]
  const uint32_t pw = p_lds + (uint32_t)((j * kPRow + 32 * wave + 4 * g) * 2);   // P[j][32w + 16kb + 4g ..]

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int c = item % C;
    const int rest = item / C;
    const int hs = rest % slices, bkv = rest / slices;
    const int kvh = bkv % Hkv, b = bkv / Hkv;
    const int h0 = kvh * group + hs * G;  // first query head of this item
    const int key0 = c * kChunk;
    const int len = min(kChunk, M - key0);
    const int64_t slice = ((int64_t)b * Hkv + kvh) * M * D;

    // V chunk -> LDS, no registers (bounds-checked: rows past M are zeros)
    const i32x4 vdesc = make_desc(v + slice, D, M, D);
#pragma unroll
    for (int i = 0; i < kFetch; ++i)
      dma16(vdesc, v_lds + (uint32_t)(i * kWaves + wave) * 1024u,
            voff_lane + (uint32_t)(key0 + kRowsPerInst * i) * (uint32_t)(D * 2));

    // A operand of S^T: K row 32w + 16kb + j, d = 32s + 8g .. +7
    s16x8 ka[2][kS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int row = 32 * wave + 16 * kb + j;
      const uint16_t* kp = k + slice + (int64_t)(key0 + row) * D + 8 * g;
#pragma unroll
      for (int s = 0; s < kS; ++s) {
        const uint4 t = row < len ? load_stream(kp + 32 * s) : make_uint4(0, 0, 0, 0);
        ka[kb][s] = __builtin_bit_cast(s16x8, t);
      }
    }
    // B operand of S^T: q of head h0 + j, d = 32s + 8g .. +7
    s16x8 qb[kS];
#pragma unroll
    for (int s = 0; s < kS; ++s)
      qb[s] = j < G ? *reinterpret_cast<const s16x8*>(q + ((int64_t)b * Hq + h0 + j) * D + 32 * s + 8 * g)
                    : (s16x8){};

    // scores in log2 units; element r of block kb is key 32w + 16kb + 4g + r
    float x[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4 sa = {};
#pragma unroll
      for (int s = 0; s < kS; ++s) sa = mfma16x16x32<BF16>(ka[kb][s], qb[s], sa);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = 32 * wave + 16 * kb + 4 * g + r;
        x[kb][r] = key < len ? sa[r] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, x[kb][r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = max_xor32(mx);
    if (g == 0) red[0][wave][j] = mx;
    wait_tile_loads();  // this wave's part of the V chunk is in LDS
    __syncthreads();    // V chunk and the per-wave maxima visible
    float m = red[0][0][j];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = fmaxf(m, red[0][w][j]);

    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = __builtin_amdgcn_exp2f(x[kb][r] - m);
        lsum += p[r];
      }
      const uint32_t h01 = pack2<BF16>(p[0], p[1]), h23 = pack2<BF16>(p[2], p[3]);
      const f32x2 r01 = unpack2<BF16>(h01), r23 = unpack2<BF16>(h23);
      const uint32_t l01 = pack2<BF16>(p[0] - r01[0], p[1] - r01[1]);
      const uint32_t l23 = pack2<BF16>(p[2] - r23[0], p[3] - r23[1]);
      lds_write_b64(pw + 32u * kb, (u32x2){h01, h23});
      lds_write_b64(pw + kPBytes + 32u * kb, (u32x2){l01, l23});
    }
    lsum += __shfl_xor(lsum, 16);
    lsum = sum_xor32(lsum);
    if (g == 0) red[1][wave][j] = lsum;
    __syncthreads();  // P and the per-wave sums visible

    f32x4 oacc[kDB];
#pragma unroll
    for (int db = 0; db < kDB; ++db) oacc[db] = (f32x4){};
#pragma unroll
    for (int ks = 0; ks < kChunk / 32; ++ks) {
      const s16x8 ph = lds_read_b128(pa + 64u * ks);
      const s16x8 pl = lds_read_b128(pa + kPBytes + 64u * ks);
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const s16x4 lo = lds_read_tr16_b64(va[db][0] + (uint32_t)(32 * ks * D * 2));
        const s16x4 hi = lds_read_tr16_b64(va[db][1] + (uint32_t)(32 * ks * D * 2));
        const s16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[db] = mfma16x16x32<BF16>(a, ph, oacc[db]);
        oacc[db] = mfma16x16x32<BF16>(a, pl, oacc[db]);
      }
    }
    float lt = red[1][0][j];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) lt += red[1][w][j];
    if (j < G) {
      const int64_t base = ((int64_t)b * Hq + h0 + j) * C + c;
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        float* op = o_part + base * D + wave * (D / 4) + 16 * db + 4 * g;
        const float4 o4 = make_float4(oacc[db][0] / lt, oacc[db][1] / lt, oacc[db][2] / lt, oacc[db][3] / lt);
        if (out16) {
          *reinterpret_cast<float4*>(op) = o4;
        } else {
          op[0] = o4.x; op[1] = o4.y; op[2] = o4.z; op[3] = o4.w;
        }
      }
      if (wave == 0 && g == 0) lse_part[base] = (m + log2f(lt)) * kLn2;
    }
    __syncthreads();  // V, P and the sums are refilled by the next item
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
  const int group = Hq / Hkv;
  if (group >= 2) {
    // query heads per item: the largest divisor of the group that fits the
    // 16 MFMA columns
    int g = std::min(group, kGqaCols);
    while (group % g != 0) --g;
    const int n_items = B * (Hq / g) * C;
#define ATTN_GQA_CASE(DD, BB)                                                                          \
    if (d == DD && bf16 == BB) {                                                                       \
      const int grid = std::min(n_items, resident_grid(decode_gqa_mfma_kernel<DD, BB>, kDecThreads));  \
      hipLaunchKernelGGL((decode_gqa_mfma_kernel<DD, BB>), dim3(grid), dim3(kDecThreads), 0, stream,   \
                         (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, o_part, lse_part, \
                         Hq, Hkv, M, C, g, n_items, sl2);                                              \
      return hipGetLastError();                                                                        \
    }
    ATTN_GQA_CASE(64, false) ATTN_GQA_CASE(64, true) ATTN_GQA_CASE(128, false) ATTN_GQA_CASE(128, true)
#undef ATTN_GQA_CASE
    return hipErrorInvalidValue;
  }
  const int n_items = B * Hq * C;
#define ATTN_DEC_CASE(DD, BB)                                                                          \
  if (d == DD && bf16 == BB) {                                                                         \
    const int grid = std::min(n_items, resident_grid(decode_chunk_kernel<DD, BB, 1>, kDecThreads));    \
    hipLaunchKernelGGL((decode_chunk_kernel<DD, BB, 1>), dim3(grid), dim3(kDecThreads), 0, stream,     \
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, o_part, lse_part,   \
                       Hq, Hkv, M, C, n_items, sl2);                                                   \
    return hipGetLastError();                                                                          \
  }
  ATTN_DEC_CASE(64, false) ATTN_DEC_CASE(64, true) ATTN_DEC_CASE(128, false) ATTN_DEC_CASE(128, true)
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
