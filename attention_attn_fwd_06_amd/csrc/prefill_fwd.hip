// Fused attention forward (prefill) for gfx950.
//
// Computes O = softmax(scale * Q K^T [+ causal mask]) V with an online softmax
// ("fmha sm120: beyond torch.sdpa", section 1 "flash attention": load a Q tile,
// loop over K/V tiles, rescale the running row max m and sum l, write O once;
// section 2: GQA head map and top-left causal tile skipping).
//
// MI355X design (not the page's CUDA design):
//  * one workgroup = 4 waves = BM = 128 queries of one (batch, query head);
//    each wave owns 32 queries for the whole KV loop.
//  * both products run on v_mfma_f32_32x32x16_{bf16,f16} with fp32 accumulators,
//    transposed so that one lane owns one query:
//      S^T[key][query] = K Q^T   (A = K rows from LDS, B = Q^T kept in VGPRs)
//      O^T[d][query]  += V^T P^T (A = V^T via ds_read_b64_tr_b16, B = P^T
//                                 taken straight from the S^T accumulator)
//    so the row max / row sum are in-lane plus one v_permlane32_swap, and the
//    rescale factor is a per-lane scalar.  The accumulator's key order (runs of
//    4 keys interleaved between the lane halves) only permutes the contracted
//    index, so the V^T read simply uses the same key order.
//  * K and V tiles (BN = 64 keys) are double-buffered in LDS, row-major with a
//    16-byte-chunk XOR swizzle that keeps both the K row reads (8 rows per LDS
//    cycle) and the transposed V reads (4 rows x 2 chunks per cycle) free of
//    bank conflicts.  The next tile's global loads are issued before the
//    current tile's math, so V (and K) arrive while QK and softmax run.
//  * exp2 domain with scale*log2(e) folded into one FMA; the O / l rescale is
//    skipped unless some row's max grew by more than 2^8 (exact: O and l always
//    share the same reference max).
//  * bf16 only: on the first KV tile P is split into hi + lo bf16 parts (two PV
//    MFMAs), so rows with very few keys (early causal rows, where |O| is large)
//    keep full fp32-level accuracy in P.
//  * causal: tiles beyond the diagonal are never loaded; a wave whose 32
//    queries all precede a tile skips that tile's math; only diagonal tiles are
//    masked.  Grid: longest causal q-tiles first, heads of one GQA group
//    adjacent, and an XCD-aware remap so heads sharing K/V share an L2.
#include "device_common.h"

namespace attn {

constexpr int kBM = 128;       // queries per workgroup
constexpr int kBN = 64;        // keys per K/V tile
constexpr int kThreads = 256;  // 4 waves of 64

// 16-byte chunk swizzle: physical chunk = logical chunk ^ swz(row).
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }

template <int D>
struct TileCfg {
  static constexpr int kChunks = D / 8;                      // 16-byte chunks per row
  static constexpr int kTileElems = kBN * D;                  // one K or V tile
  static constexpr int kLoads = kBN * kChunks / kThreads;     // 16-byte loads per thread per tile
};

// Global -> registers: the 16-byte chunks of one K or V tile owned by this thread.
template <int D>
__device__ __forceinline__ void load_tile(uint4 (&r)[TileCfg<D>::kLoads], const uint16_t* __restrict__ base,
                                          int64_t row_stride, int rows_valid, int tid) {
#pragma unroll
  for (int i = 0; i < TileCfg<D>::kLoads; ++i) {
    const int cid = tid + i * kThreads;
    const int row = cid / TileCfg<D>::kChunks, c = cid % TileCfg<D>::kChunks;
    if (row < rows_valid)
      r[i] = *reinterpret_cast<const uint4*>(base + row * row_stride + c * 8);
    else
      r[i] = make_uint4(0, 0, 0, 0);  // keys past M: zeros, masked later
  }
}

// Registers -> LDS (swizzled row-major tile).
template <int D>
__device__ __forceinline__ void store_tile(uint16_t* lds, const uint4 (&r)[TileCfg<D>::kLoads], int tid) {
#pragma unroll
  for (int i = 0; i < TileCfg<D>::kLoads; ++i) {
    const int cid = tid + i * kThreads;
    const int row = cid / TileCfg<D>::kChunks, c = cid % TileCfg<D>::kChunks;
    *reinterpret_cast<uint4*>(lds + row * D + ((c ^ swz(row)) << 3)) = r[i];
  }
}

template <int D, bool BF16, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_fwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                        const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                        float* __restrict__ lse, int N, int M, int Hq, int Hkv,
                        int n_qtiles, int total, float scale_log2) {
  constexpr int kDT = D / 16;  // contraction steps of QK^T
  constexpr int kDB = D / 32;  // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * TileCfg<D>::kTileElems];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;

  // ---- tile id -> (b, h, q-tile); see the file comment for the order ----
  const int lid = xcd_remap(blockIdx.x, total);
  const int group = Hq / Hkv;
  const int hg = lid % group;
  const int rest = lid / group;
  const int qt = n_qtiles - 1 - rest % n_qtiles;  // longest (causal) first
  const int bkv = rest / n_qtiles;
  const int kvh = bkv % Hkv, b = bkv / Hkv;
  const int h = kvh * group + hg;

  const int q_start = qt * kBM;
  const int qw = q_start + wave * 32;  // first query of this wave
  const int qi = qw + l32;             // this lane's query (column of S^T / O^T)

  const int64_t q_row_stride = (int64_t)Hq * D;
  const int64_t kv_row_stride = (int64_t)Hkv * D;
  const uint16_t* kb = k + ((int64_t)b * M * Hkv + kvh) * D;
  const uint16_t* vb = v + ((int64_t)b * M * Hkv + kvh) * D;

  // ---- Q^T operand: 16 bytes per contraction step, kept for the whole loop ----
  s16x8 qreg[kDT];
  {
    const uint16_t* qp = q + ((int64_t)b * N + qi) * q_row_stride + (int64_t)h * D + 8 * g;
#pragma unroll
    for (int t = 0; t < kDT; ++t) {
      uint4 u = (qi < N) ? *reinterpret_cast<const uint4*>(qp + 16 * t) : make_uint4(0, 0, 0, 0);
      qreg[t] = __builtin_bit_cast(s16x8, u);
    }
  }

  f32x16 acc_o[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i) acc_o[i] = (f32x16){};
  float m_run = -INFINITY;  // running max of scale*log2e*s for query qi
  float l_run = 0.f;        // running sum over this lane's half of the keys

  const int kv_end = CAUSAL ? min(M, q_start + kBM) : M;
  const int n_tiles = (kv_end + kBN - 1) / kBN;

  // LDS: [buf][K tile, V tile]
  constexpr int kBufElems = 2 * TileCfg<D>::kTileElems;

  uint4 rk[TileCfg<D>::kLoads], rv[TileCfg<D>::kLoads];
  load_tile<D>(rk, kb, kv_row_stride, min(kBN, M), tid);
  load_tile<D>(rv, vb, kv_row_stride, min(kBN, M), tid);
  store_tile<D>(smem, rk, tid);
  store_tile<D>(smem + TileCfg<D>::kTileElems, rv, tid);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    const int n0 = j * kBN;
    const bool has_next = j + 1 < n_tiles;
    if (has_next) {
      const int n1 = n0 + kBN;
      load_tile<D>(rk, kb + n1 * kv_row_stride, kv_row_stride, min(kBN, M - n1), tid);
      load_tile<D>(rv, vb + n1 * kv_row_stride, kv_row_stride, min(kBN, M - n1), tid);
    }

    const bool wave_active = !CAUSAL || n0 <= qw + 31;
    if (wave_active) {
      const uint16_t* Kt = smem + buf * kBufElems;
      const uint16_t* Vt = Kt + TileCfg<D>::kTileElems;
      // ---- S^T = K Q^T for two 32-key blocks ----
      f32x16 s[2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        s[kb2] = (f32x16){};
        const int row = 32 * kb2 + l32;
        const uint16_t* rp = Kt + row * D;
        const int sw = swz(row);
#pragma unroll
        for (int t = 0; t < kDT; ++t) {
          s16x8 a = *reinterpret_cast<const s16x8*>(rp + (((2 * t + g) ^ sw) << 3));
          s[kb2] = mfma32x32x16<BF16>(a, qreg[t], s[kb2]);
        }
      }

      // ---- mask (diagonal tiles and the key tail only) ----
      const bool need_mask = (CAUSAL && n0 + kBN - 1 > qw) || (n0 + kBN > M);
      if (need_mask) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = n0 + 32 * kb2 + 8 * (i >> 2) + 4 * g + (i & 3);
            const bool ok = key < M && (!CAUSAL || key <= qi);
            s[kb2][i] = ok ? s[kb2][i] : -INFINITY;
          }
      }

      // ---- online softmax (exp2 domain, one query per lane) ----
      float mx = -INFINITY;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb2][i]);
      mx = max_xor32(mx);
      const float m_tile = (mx == -INFINITY) ? -INFINITY : mx * scale_log2;
      // Move the reference max only when it grows by more than 2^8; otherwise
      // p may reach 2^8, which fp32 accumulation and 16-bit P represent fine.
      const bool grow = m_tile > m_run + 8.0f;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = fmaxf(m_run, m_tile);
        const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < kDB; ++i) acc_o[i] *= alpha;
        m_run = m_new;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;

      float p[2][16];
      float lsum = 0.f;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float e = __builtin_amdgcn_exp2f(fmaf(s[kb2][i], scale_log2, -m_use));
          if (need_mask) e = (s[kb2][i] == -INFINITY) ? 0.f : e;  // exact zero for scale == 0
          p[kb2][i] = e;
          lsum += e;
        }
      l_run += lsum;

      // ---- P^T operand straight from the accumulator layout ----
      // k-step (kb2, st) uses accumulator elements 8*st .. 8*st+7, i.e. keys
      // 32*kb2 + 16*st + 8*(jj/4) + 4*g + jj%4 for slot jj.
      s16x8 pb[2][2];
      s16x8 pl[2][2];  // bf16 only, first tile: p - bf16(p), rounded to bf16
      const bool split_p = BF16 && j == 0;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = pack2<BF16>(p[kb2][8 * st + 2 * e], p[kb2][8 * st + 2 * e + 1]);
          pb[kb2][st] = __builtin_bit_cast(s16x8, make_uint4(w[0], w[1], w[2], w[3]));
          if (split_p) {
            uint32_t wl[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const f32x2 hv = unpack2<BF16>(w[e]);
              wl[e] = pack2<BF16>(p[kb2][8 * st + 2 * e] - hv[0], p[kb2][8 * st + 2 * e + 1] - hv[1]);
            }
            pl[kb2][st] = __builtin_bit_cast(s16x8, make_uint4(wl[0], wl[1], wl[2], wl[3]));
          }
        }

      // ---- O^T += V^T P^T ----
      // ds_read_b64_tr_b16: in each 16-lane group, lane i receives element i%4
      // of the 8 bytes addressed by lane 4*jj + i/4, for jj = 0..3.  Lane s of
      // group G addresses V[K0 + s/4][D0 + 4*(s%4)] with D0 = 32*db + 16*(G&1)
      // and K0 = first key of the slot run, so lane i gets 4 consecutive keys
      // of column D0 + i%16 = 32*db + l%32.
      const int G = lane >> 4, sl = lane & 15;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int r0 = 32 * kb2 + 16 * st + 4 * (G >> 1) + (sl >> 2);  // slots 0..3
          const int r1 = r0 + 8;                                         // slots 4..7
#pragma unroll
          for (int db = 0; db < kDB; ++db) {
            const int col = 32 * db + 16 * (G & 1) + 4 * (sl & 3);
            const int off0 = r0 * D + (((col >> 3) ^ swz(r0)) << 3) + (col & 7);
            const int off1 = r1 * D + (((col >> 3) ^ swz(r1)) << 3) + (col & 7);
            s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vt + off0));
            s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vt + off1));
            s16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            acc_o[db] = mfma32x32x16<BF16>(a, pb[kb2][st], acc_o[db]);
            if (split_p) acc_o[db] = mfma32x32x16<BF16>(a, pl[kb2][st], acc_o[db]);
          }
        }
    }

    if (has_next) {
      store_tile<D>(smem + (buf ^ 1) * kBufElems, rk, tid);
      store_tile<D>(smem + (buf ^ 1) * kBufElems + TileCfg<D>::kTileElems, rv, tid);
    }
    __syncthreads();
  }

  // ---- epilogue: O / l -> 16-bit, lse = ln2 * (m + log2 l) ----
  const float l_tot = sum_xor32(l_run);
  const float inv = 1.f / l_tot;
  if (qi < N) {
    uint16_t* op = o + ((int64_t)b * N + qi) * q_row_stride + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d0 = 32 * db + 8 * r + 4 * g;
        uint2 w;
        w.x = pack2<BF16>(acc_o[db][4 * r + 0] * inv, acc_o[db][4 * r + 1] * inv);
        w.y = pack2<BF16>(acc_o[db][4 * r + 2] * inv, acc_o[db][4 * r + 3] * inv);
        *reinterpret_cast<uint2*>(op + d0) = w;
      }
    if (lse != nullptr && g == 0)
      lse[((int64_t)b * Hq + h) * N + qi] = (m_run + log2f(l_tot)) * kLn2;
  }
}

// Host-side launcher (one instance per head dim, dtype and mask).
template <int D, bool BF16, bool CAUSAL>
hipError_t launch_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                          int Hq, int Hkv, int N, int M, float scale, hipStream_t stream) {
  const int n_qtiles = (N + kBM - 1) / kBM;
  const int total = B * Hq * n_qtiles;
  hipLaunchKernelGGL((prefill_fwd_kernel<D, BF16, CAUSAL>), dim3(total), dim3(kThreads), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, N, M,
                     Hq, Hkv, n_qtiles, total, scale * kLog2e);
  return hipGetLastError();
}

hipError_t prefill_dispatch(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                            int Hq, int Hkv, int N, int M, int d, bool causal, bool bf16, float scale,
                            hipStream_t stream) {
#define ATTN_PREFILL_CASE(DD, BB, CC)                                                      \
  if (d == DD && bf16 == BB && causal == CC)                                               \
    return launch_prefill<DD, BB, CC>(q, k, v, o, lse, B, Hq, Hkv, N, M, scale, stream);
  ATTN_PREFILL_CASE(64, false, false)
  ATTN_PREFILL_CASE(64, false, true)
  ATTN_PREFILL_CASE(64, true, false)
  ATTN_PREFILL_CASE(64, true, true)
  ATTN_PREFILL_CASE(128, false, false)
  ATTN_PREFILL_CASE(128, false, true)
  ATTN_PREFILL_CASE(128, true, false)
  ATTN_PREFILL_CASE(128, true, true)
#undef ATTN_PREFILL_CASE
  return hipErrorInvalidValue;
}

}  // namespace attn
