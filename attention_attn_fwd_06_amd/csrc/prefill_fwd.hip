// Fused attention forward (prefill) for gfx950.
//
// Computes O = softmax(scale * Q K^T [+ causal mask]) V with an online softmax
// ("fmha sm120: beyond torch.sdpa", section 1 "flash attention": load a Q tile,
// loop over K/V tiles, rescale the running row max m and sum l, write O once;
// section 2: GQA head map and top-left causal tile skipping).
//
// MI355X design (not the page's CUDA design):
//  * one workgroup = 8 waves, two per SIMD (256 VGPRs each); each wave owns
//    32 queries of one (batch, query head) for the whole KV loop, so BM = 256
//    queries share every K/V tile fetched into LDS (one workgroup per CU).
//  * both products run on v_mfma_f32_32x32x16_{bf16,f16} with fp32
//    accumulators, transposed so that one lane owns one query per block:
//      S^T[key][query] = K Q^T   (A = K rows from LDS, B = Q^T kept in VGPRs)
//      O^T[d][query]  += V^T P^T (A = V^T via ds_read_b64_tr_b16, B = P^T
//                                 taken straight from the S^T accumulator)
//    so the row max / row sum are in-lane plus one v_permlane32_swap, and the
//    rescale factor is a per-lane scalar.  The accumulator's key order (runs
//    of 4 keys interleaved between the lane halves) only permutes the
//    contracted index, so the V^T read uses the same key order.
//  * software pipeline: K runs one tile ahead of V.  Iteration j issues the
//    MFMAs of S(j+1) = K(j+1) Q^T, which do not depend on the softmax of tile
//    j, so the in-order issue interleaves them with the softmax VALU work;
//    then O += V(j)^T P(j).  K(j+2) and V(j+1) are fetched straight into LDS
//    (buffer_load ... lds, no staging registers) during the iteration.
//  * K and V tiles (BN = 64 keys) are double-buffered in LDS, row-major with a
//    16-byte-chunk XOR swizzle that keeps both the K row reads and the
//    transposed V reads free of bank conflicts; tile rows past M come back as
//    zeros from bounds-checked buffer loads (no branches).
//  * exp2 domain with scale*log2(e) folded into one FMA; the O / l rescale is
//    skipped unless some row's max grew by more than 2^8 (exact: O and l
//    always share the same reference max).
//  * bf16 only: on the first KV tile P is split into hi + lo bf16 parts (two
//    PV MFMAs), so rows with very few keys (early causal rows, where |O| is
//    large) keep fp32-level accuracy in P.
//  * causal: tiles beyond the diagonal are never loaded; a wave whose 64
//    queries all precede a tile skips its math; only diagonal tiles are
//    masked.  Grid: longest causal q-tiles first, heads of one GQA group
//    adjacent, and an XCD-aware remap so heads sharing K/V share an L2.
#include "device_common.h"

namespace attn {

constexpr int kQB = 1;             // 32-query blocks per wave
constexpr int kBN = 64;            // keys per K/V tile
constexpr int kWavesPerEU = 2;     // waves per SIMD
constexpr int kWaves = 8;          // waves per workgroup
constexpr int kKB = kBN / 32;      // 32-key blocks per tile
constexpr int kThreads = 64 * kWaves;
constexpr int kQW = 32 * kQB;      // queries per wave
constexpr int kBM = kWaves * kQW;  // queries per workgroup

// 16-byte chunk swizzle: physical chunk = logical chunk ^ swz<D>(row).  The
// LDS serves 256 bytes (64 banks) per cycle: 16 lanes of a ds_read_b128 or 32
// lanes of a ds_read_b64_tr_b16.  The K operand read has 16 consecutive rows
// at one logical chunk; the transposed V read has 4 consecutive rows (first
// row a multiple of 4) times 4 consecutive chunks (first a multiple of 4).
// Both must land on 16 distinct 16-byte bank groups:
//  d = 128 (256-byte rows): swz = 4*(row%4) + (row/4)%4 is a permutation of
//    0..15 over 16 consecutive rows, and over 4 consecutive rows its top two
//    bits take 4 distinct values;
//  d = 64 (128-byte rows, two per bank row): swz = 4*((row/2)%2) + (row/4)%4
//    permutes 0..7 over the 8 rows of one parity, and rows 2 apart differ in
//    bit 2.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

template <int D>
struct TileCfg {
  static constexpr int kChunks = D / 8;                   // 16-byte chunks per row
  static constexpr int kTileElems = kBN * D;              // one K or V tile
  static constexpr int kLoads = kBN * kChunks / kThreads;  // 16-byte loads per thread per tile
};

// Buffer resource over one (batch, kv head) slice of K or V: rows past M read
// as zero.  gfx9 descriptor word 3.  The host guarantees (M + 64) rows of the
// slice stay below 2^32 bytes, so offsets of rows past M never wrap around.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint16_t* base, int64_t row_stride, int M,
                                                            int D) {
  const int64_t bytes = ((int64_t)(M - 1) * row_stride + D) * 2;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, (int)bytes, 0x00020000);
}

typedef __attribute__((address_space(3))) void lds_void;

// Global -> LDS without registers: each buffer_load_dwordx4 ... lds writes the
// 16 bytes of lane L at M0 + 16 * L, so a wave fills 64 consecutive 16-byte
// units of the swizzled tile per instruction and picks, per lane, the global
// chunk that belongs at that unit (physical chunk pc of row r holds logical
// chunk pc ^ swz<D>(r)).  Rows past M come back as zeros.  Completion is tracked
// by vmcnt; the caller waits before the barrier that publishes the tile.
template <int D>
__device__ __forceinline__ void load_tile_lds(uint16_t* lds_tile, __amdgpu_buffer_rsrc_t rsrc, int n0,
                                              int row_stride_bytes, int wave, int lane) {
  constexpr int kU = D / 8;                     // 16-byte units per row
  constexpr int kInst = kBN * kU / kThreads;    // instructions per thread
  static_assert(kBN * kU % kThreads == 0, "tile must split evenly over the workgroup");
#pragma unroll
  for (int i = 0; i < kInst; ++i) {
    const int base = (i * kWaves + wave) * 64;   // first unit written by this instruction
    const int P = base + lane;
    const int row = P / kU, pc = P % kU;
    const int c = pc ^ swz<D>(row);
    const uint32_t off = (uint32_t)(n0 + row) * (uint32_t)row_stride_bytes + (uint32_t)(c * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds_tile + base * 8), 16, (int)off, 0, 0, 0);
  }
}

__device__ __forceinline__ void wait_tile_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// S^T[qb][kb] = K(tile) Q^T for the wave's two query blocks.
template <int D, bool BF16>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[kQB][kKB], const uint16_t* Kt, const s16x8 (&qreg)[kQB][D / 16],
                                        int l32, int g) {
  constexpr int kDT = D / 16;
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) s[qb][kb] = (f32x16){};
#pragma unroll
  for (int t = 0; t < kDT; ++t)
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
      const int row = 32 * kb + l32;
      const s16x8 a = *reinterpret_cast<const s16x8*>(Kt + row * D + (((2 * t + g) ^ swz<D>(row)) << 3));
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) s[qb][kb] = mfma32x32x16<BF16>(a, qreg[qb][t], s[qb][kb]);
    }
}

template <int D, bool BF16, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEU, kWavesPerEU)))
void prefill_fwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                        const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                        float* __restrict__ lse, int N, int M, int Hq, int Hkv,
                        int n_qtiles, int total, float scale_log2) {
  constexpr int kDT = D / 16;  // contraction steps of QK^T
  constexpr int kDB = D / 32;  // 32-row blocks of O^T
  constexpr int kTE = TileCfg<D>::kTileElems;
  // LDS: K buffers 0, 1 then V buffers 0, 1
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * kTE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int G = lane >> 4, sl = lane & 15;

  // ---- tile id -> (b, h, q-tile) ----
  const int lid = xcd_remap(blockIdx.x, total);
  const int group = Hq / Hkv;
  const int hg = lid % group;
  const int rest = lid / group;
  const int qt = n_qtiles - 1 - rest % n_qtiles;  // longest (causal) first
  const int bkv = rest / n_qtiles;
  const int kvh = bkv % Hkv, b = bkv / Hkv;
  const int h = kvh * group + hg;

  const int q_start = qt * kBM;
  const int qw = q_start + wave * kQW;  // first query of this wave
  const int qlast = qw + kQW - 1;       // last query of this wave

  const int64_t q_row_stride = (int64_t)Hq * D;
  const int64_t kv_row_stride = (int64_t)Hkv * D;
  const int kv_row_bytes = (int)(kv_row_stride * 2);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + ((int64_t)b * M * Hkv + kvh) * D, kv_row_stride, M, D);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + ((int64_t)b * M * Hkv + kvh) * D, kv_row_stride, M, D);

  // ---- Q^T operands: 16 bytes per contraction step and query block ----
  s16x8 qreg[kQB][kDT];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int qi = qw + 32 * qb + l32;
    const uint16_t* qp = q + ((int64_t)b * N + qi) * q_row_stride + (int64_t)h * D + 8 * g;
#pragma unroll
    for (int t = 0; t < kDT; ++t) {
      uint4 u = (qi < N) ? *reinterpret_cast<const uint4*>(qp + 16 * t) : make_uint4(0, 0, 0, 0);
      qreg[qb][t] = __builtin_bit_cast(s16x8, u);
    }
  }

  f32x16 acc_o[kQB][kDB];
  float m_run[kQB];  // running max of scale*log2e*s
  float l_run[kQB];  // running sum over this lane's keys
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int i = 0; i < kDB; ++i) acc_o[qb][i] = (f32x16){};
  }

  const int kv_end = CAUSAL ? min(M, q_start + kBM) : M;
  const int n_tiles = (kv_end + kBN - 1) / kBN;
  // last tile that holds a key <= some query of this wave
  const int wave_tiles = CAUSAL ? min(n_tiles, qlast / kBN + 1) : n_tiles;

  uint16_t* const kbuf = smem;
  uint16_t* const vbuf = smem + 2 * kTE;

  // ---- prologue: K(0), V(0), K(1) to LDS; S(0) ----
  load_tile_lds<D>(kbuf, krs, 0, kv_row_bytes, wave, lane);
  load_tile_lds<D>(vbuf, vrs, 0, kv_row_bytes, wave, lane);
  if (n_tiles > 1) load_tile_lds<D>(kbuf + kTE, krs, kBN, kv_row_bytes, wave, lane);
  wait_tile_loads();
  __syncthreads();
  f32x16 s_a[kQB][kKB], s_b[kQB][kKB];
  qk_tile<D, BF16>(s_a, kbuf, qreg, l32, g);
  __syncthreads();  // K buffer 0 is refilled at the end of iteration 0

  // O^T += V(j)^T P(j) for one 16-key k-step (kb, st) and all d blocks.
  // ds_read_b64_tr_b16: in each 16-lane group, lane i receives element i%4 of
  // the 8 bytes addressed by lane 4*jj + i/4, for jj = 0..3.  Lane s of group G
  // addresses V[K0 + s/4][D0 + 4*(s%4)] with D0 = 32*db + 16*(G&1) and K0 =
  // the first key of the slot run, so lane i gets 4 consecutive keys of column
  // D0 + i%16 = 32*db + l%32.
  auto pv_kstep = [&](const uint16_t* Vt, int kb, int st, const s16x8 (&pbq)[kQB], const s16x8* plq) {
    const int r0 = 32 * kb + 16 * st + 4 * (G >> 1) + (sl >> 2);  // slots 0..3
    const int r1 = r0 + 8;                                         // slots 4..7
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      const int col = 32 * db + 16 * (G & 1) + 4 * (sl & 3);
      const int off0 = r0 * D + (((col >> 3) ^ swz<D>(r0)) << 3) + (col & 7);
      const int off1 = r1 * D + (((col >> 3) ^ swz<D>(r1)) << 3) + (col & 7);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vt + off0));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vt + off1));
      const s16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        acc_o[qb][db] = mfma32x32x16<BF16>(a, pbq[qb], acc_o[qb][db]);
        if (plq != nullptr) acc_o[qb][db] = mfma32x32x16<BF16>(a, plq[qb], acc_o[qb][db]);
      }
    }
  };

  // Row max of tile j and the rare move of the reference max (see below).
  auto row_max_update = [&](f32x16 (&s_cur)[kQB][kKB]) {
    float m_tile[kQB];
    bool grow = false;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s_cur[qb][kb][i]);
      mx = max_xor32(mx);
      m_tile[qb] = (mx == -INFINITY) ? -INFINITY : mx * scale_log2;
      grow |= m_tile[qb] > m_run[qb] + 8.0f;
    }
    // Move the reference max only when it grows by more than 2^8; otherwise
    // p may reach 2^8, which fp32 accumulation and 16-bit P represent fine.
    if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        const float m_new = fmaxf(m_run[qb], m_tile[qb]);
        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        l_run[qb] *= alpha;
#pragma unroll
        for (int i = 0; i < kDB; ++i) acc_o[qb][i] *= alpha;
        m_run[qb] = m_new;
      }
    }
  };

  // p = 2^(s*scale*log2e - m) for 8 accumulator elements, packed to the PV B
  // operand; k-step (kb, st) uses accumulator elements 8*st .. 8*st+7, i.e.
  // keys 32*kb + 16*st + 8*(jj/4) + 4*g + jj%4 for slot jj.  The row sum l is
  // accumulated from the unrounded fp32 p (a sum of 16-bit-rounded weights
  // can be off by 2^-9 relative when a few keys dominate, too much for lse).
  auto exp_pack = [&](const f32x16& sv, int st, float m_use, float& lsum, bool masked, s16x8& pb, s16x8* pl) {
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = sv[8 * st + e];
      float y = __builtin_amdgcn_exp2f(fmaf(x, scale_log2, -m_use));
      if (masked) y = (x == -INFINITY) ? 0.f : y;  // exact zero also for scale == 0
      pv[e] = y;
      lsum += y;
    }
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack2<BF16>(pv[2 * e], pv[2 * e + 1]);
    pb = __builtin_bit_cast(s16x8, make_uint4(w[0], w[1], w[2], w[3]));
    if (pl != nullptr) {
      uint32_t wl[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x2 hv = unpack2<BF16>(w[e]);
        wl[e] = pack2<BF16>(pv[2 * e] - hv[0], pv[2 * e + 1] - hv[1]);
      }
      *pl = __builtin_bit_cast(s16x8, make_uint4(wl[0], wl[1], wl[2], wl[3]));
    }
  };

  // General step (first tile, diagonal and tail tiles, last tile of a wave):
  // S(j+1) -> s_next if this wave needs it, then mask, softmax and PV of tile j.
  auto step_general = [&](const int j, f32x16 (&s_cur)[kQB][kKB], f32x16 (&s_next)[kQB][kKB]) {
    const int n0 = j * kBN;
    if (j + 1 < wave_tiles) qk_tile<D, BF16>(s_next, kbuf + ((j + 1) & 1) * kTE, qreg, l32, g);
    if (j >= wave_tiles) return;
    const bool need_mask = (CAUSAL && n0 + kBN - 1 > qw) || (n0 + kBN > M);
    if (need_mask) {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        const int qi = qw + 32 * qb + l32;
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = n0 + 32 * kb + 8 * (i >> 2) + 4 * g + (i & 3);
            const bool ok = key < M && (!CAUSAL || key <= qi);
            s_cur[qb][kb][i] = ok ? s_cur[qb][kb][i] : -INFINITY;
          }
      }
    }
    row_max_update(s_cur);
    const bool split_p = BF16 && j == 0;  // bf16: hi/lo split of P on the first tile
    const uint16_t* Vt = vbuf + (j & 1) * kTE;
    float lsum[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) lsum[qb] = 0.f;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        s16x8 pb[kQB], pl[kQB];
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
          const float m_use = (m_run[qb] == -INFINITY) ? 0.f : m_run[qb];
          exp_pack(s_cur[qb][kb], st, m_use, lsum[qb], need_mask, pb[qb], split_p ? &pl[qb] : nullptr);
        }
        pv_kstep(Vt, kb, st, pb, split_p ? pl : nullptr);
      }
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) l_run[qb] += lsum[qb];
  };

  // Steady-state step (no mask, reference max already finite, S(j+1) needed):
  // after the row max, the QK MFMAs of tile j+1, the exp/pack VALU work of
  // tile j and its PV MFMAs form one basic block, and the scheduler is asked
  // to interleave them (each MFMA followed by the next LDS read, 2-4 VALU and,
  // during the QK half, 2 exp2) so that the matrix core and the VALU run at the
  // same time and every LDS read is issued one MFMA ahead of its use.
  auto step_fast = [&](const int j, f32x16 (&s_cur)[kQB][kKB], f32x16 (&s_next)[kQB][kKB]) {
    row_max_update(s_cur);
    __builtin_amdgcn_sched_barrier(0);
    qk_tile<D, BF16>(s_next, kbuf + ((j + 1) & 1) * kTE, qreg, l32, g);
    const uint16_t* Vt = vbuf + (j & 1) * kTE;
    float lsum[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) lsum[qb] = 0.f;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        s16x8 pb[kQB];
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) exp_pack(s_cur[qb][kb], st, m_run[qb], lsum[qb], false, pb[qb], nullptr);
        pv_kstep(Vt, kb, st, pb, nullptr);
      }
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) l_run[qb] += lsum[qb];
    // QK: kDT*kKB LDS reads, kDT*kKB*kQB MFMAs; PV: 2*kDB*2*kKB tr reads,
    // kDB*2*kKB*kQB MFMAs; about 4 VALU per MFMA overall.
    constexpr int kMfmaQK = kDT * kKB * kQB, kMfmaPV = kDB * 2 * kKB * kQB;
    // Per MFMA: the QK half also takes one K-fragment read (kLead reads ahead),
    // kQkValu VALU and kQkTrans exp2; the PV half takes its two transposed V
    // reads and kPvValu VALU.  d = 64 has twice the softmax work per MFMA.
    constexpr int kLead = 4;
    constexpr int kQkValu = D == 128 ? 2 : 6, kQkTrans = D == 128 ? 1 : 2, kPvValu = D == 128 ? 4 : 6;
    __builtin_amdgcn_sched_group_barrier(0x100, kLead, 0);  // LDS reads ahead
#pragma unroll
    for (int i = 0; i < kMfmaQK; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);         // LDS read
      __builtin_amdgcn_sched_group_barrier(0x002, kQkValu, 0);   // VALU
      __builtin_amdgcn_sched_group_barrier(0x400, kQkTrans, 0);  // exp2
    }
#pragma unroll
    for (int i = 0; i < kMfmaPV; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);         // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x002, kPvValu, 0);   // VALU
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  auto step = [&](const int j, f32x16 (&s_cur)[kQB][kKB], f32x16 (&s_next)[kQB][kKB]) {
    const int n0 = j * kBN;
    if (j + 2 < n_tiles) load_tile_lds<D>(kbuf + (j & 1) * kTE, krs, n0 + 2 * kBN, kv_row_bytes, wave, lane);
    if (j + 1 < n_tiles) load_tile_lds<D>(vbuf + ((j + 1) & 1) * kTE, vrs, n0 + kBN, kv_row_bytes, wave, lane);
    const bool fast = j >= 1 && j + 1 < wave_tiles && !(CAUSAL && n0 + kBN - 1 > qw) && n0 + kBN <= M;
    if (fast)
      step_fast(j, s_cur, s_next);
    else
      step_general(j, s_cur, s_next);
    wait_tile_loads();
    __syncthreads();
  };

  for (int j = 0; j < n_tiles; j += 2) {
    step(j, s_a, s_b);
    if (j + 1 < n_tiles) step(j + 1, s_b, s_a);
  }

  // ---- epilogue: O / l -> 16-bit, lse = ln2 * (m + log2 l) ----
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int qi = qw + 32 * qb + l32;
    const float l_tot = sum_xor32(l_run[qb]);
    const float inv = 1.f / l_tot;
    if (qi < N) {
      uint16_t* op = o + ((int64_t)b * N + qi) * q_row_stride + (int64_t)h * D;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d0 = 32 * db + 8 * r + 4 * g;
          uint2 w;
          w.x = pack2<BF16>(acc_o[qb][db][4 * r + 0] * inv, acc_o[qb][db][4 * r + 1] * inv);
          w.y = pack2<BF16>(acc_o[qb][db][4 * r + 2] * inv, acc_o[qb][db][4 * r + 3] * inv);
          *reinterpret_cast<uint2*>(op + d0) = w;
        }
      if (lse != nullptr && g == 0) lse[((int64_t)b * Hq + h) * N + qi] = (m_run[qb] + log2f(l_tot)) * kLn2;
    }
  }
}

// Host-side launcher (one instance per head dim, dtype and mask).
template <int D, bool BF16, bool CAUSAL>
hipError_t launch_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                          int Hkv, int N, int M, float scale, hipStream_t stream) {
  const int n_qtiles = (N + kBM - 1) / kBM;
  const int total = B * Hq * n_qtiles;
  hipLaunchKernelGGL((prefill_fwd_kernel<D, BF16, CAUSAL>), dim3(total), dim3(kThreads), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, N, M, Hq,
                     Hkv, n_qtiles, total, scale * kLog2e);
  return hipGetLastError();
}

hipError_t prefill_dispatch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                            int Hkv, int N, int M, int d, bool causal, bool bf16, float scale,
                            hipStream_t stream) {
#define ATTN_PREFILL_CASE(DD, BB, CC) \
  if (d == DD && bf16 == BB && causal == CC) return launch_prefill<DD, BB, CC>(q, k, v, o, lse, B, Hq, Hkv, N, M, scale, stream);
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
