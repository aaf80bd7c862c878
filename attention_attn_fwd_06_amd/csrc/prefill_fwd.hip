// Fused attention forward (prefill) for gfx950.
//
// Computes O = softmax(scale * Q K^T [+ causal mask]) V with an online softmax
// ("fmha sm120: beyond torch.sdpa", section 1 "flash attention": load a Q tile,
// loop over K/V tiles, rescale the running row max m and sum l, write O once;
// section 2: GQA head map and causal tile skipping).  With fewer queries than
// keys the causal mask is aligned bottom-right: the N queries are the last N
// positions of the key sequence, so query i sees keys 0 .. i + M - N (for
// N == M the pages' top-left mask).
//
// MI355X design (not the page's CUDA design):
//  * one workgroup = 4 waves (one per SIMD), 64 KB of LDS at d = 128, and two
//    workgroups per CU (256 VGPRs per wave): the two run independently, so
//    while one waits at a barrier, fetches its first tiles or writes O, the
//    other's wave keeps the SIMD busy.  Each wave owns 32 queries of one
//    (batch, query head) for the whole KV loop; with GQA a workgroup takes two
//    query heads of a group x 64 rows (one head x 128 rows without GQA), so 128
//    query rows share every K/V tile fetched into LDS while the causal
//    diagonal stays one 64-key tile per head and no wave idles past it.
//  * both products run on v_mfma_f32_32x32x16_{bf16,f16} with fp32
//    accumulators, transposed so that one lane owns one query per block:
//      S^T[key][query] = K Q^T   (A = K rows from LDS, B = Q^T kept in VGPRs
//                                 for the whole KV loop)
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
//    (buffer_load ... lds, no staging registers) during the iteration; in the
//    steady state the fetch instructions are spread over the QK MFMAs rather
//    than issued back to back, so no wave stalls on a full load queue.
//  * K and V tiles (BN = 64 keys) are double-buffered in LDS, row-major with a
//    16-byte-chunk XOR swizzle that keeps both the K row reads and the
//    transposed V reads free of bank conflicts; tile rows past M come back as
//    zeros from bounds-checked buffer loads (no branches).
//  * exp2 domain with scale*log2(e) folded into one FMA; the O / l rescale is
//    skipped unless some row's max grew by more than 2^8 (O and l always
//    share the same reference max, so the result is the same up to rounding).
//  * the steps of a first pass do not track the row max at all; the
//    reference stays at the first tile's row max, and weights above it keep
//    their relative precision in P and fp32 up to P's largest value (2^127
//    in bf16, 65504 in fp16).  A workgroup whose pass ends with a lane's row
//    sum of 2^100 (bf16) or 2^15 (fp16) or more, or with a non-finite
//    accumulator, runs the pass again with the exact steps.
//  * bf16 only: where a wave's first KV tile is masked or is its only tile
//    (rows with at most 64 keys: early causal rows, where |O| is large), P of
//    that tile is split into hi + lo bf16 parts (two PV MFMAs), so those rows
//    keep fp32-level accuracy in P.  Any other wave runs the steady-state
//    step from tile 0 on.
//  * causal: tiles beyond the diagonal are never loaded; a wave whose 32
//    queries all precede a tile skips its math; only diagonal tiles are
//    masked.  Grid: longest causal q-tiles first, heads of one GQA group
//    adjacent, and an XCD-aware remap so heads sharing K/V share an L2.
//  * epilogue: O rows go through LDS (the K/V buffers, free by then) so that
//    every store writes whole 128-byte lines.
#include <type_traits>

#include "../../include/attn.h"
#include "device_common.h"
#include "launch.h"
#include "lds_stage.h"

namespace attn {

constexpr int kBN = 64;            // keys per K/V tile
constexpr int kWaves = 4;          // waves per workgroup
// Waves per SIMD: two workgroups per CU (256 registers per wave), or at
// d = 256 one (the wave needs more than 256 registers: 128 for O^T alone,
// and the 128 KB of K/V tiles leave room for one workgroup per CU).
template <int D>
constexpr int waves_per_eu() { return D == 256 ? 1 : 2; }
constexpr int kKB = kBN / 32;      // 32-key blocks per tile
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = kWaves * 32;   // queries per workgroup (32 per wave)

// Global -> LDS without registers: each fetch instruction writes 64
// consecutive 16-byte units of the swizzled tile, lane L picking the global
// chunk that belongs at unit L (physical chunk pc of row r holds logical chunk
// pc ^ swz<D>(r)).  Instruction i of wave w covers units (i*kWaves + w)*64 ..
// +63, i.e. rows kRowsPerInst*i + (w*64 + L)/kU; the row-in-instruction part
// and the chunk are per-lane constants (voff_lane below).  When kRowsPerInst
// is a multiple of the swizzle period (16 rows) one offset serves every
// instruction; at d = 256 (8 rows per instruction index) odd instructions
// take a second one.
template <int D>
struct Fetch {
  static constexpr int kU = D / 8;                          // 16-byte units per row
  static constexpr int kInst = kBN * kU / kThreads;         // instructions per wave per tile
  static constexpr int kRowsPerInst = kWaves * 64 / kU;     // rows covered by one instruction index
  static constexpr uint32_t kInstBytes = 64 * 16;           // LDS bytes written per instruction
  static constexpr int kVar = (kInst == 1 || kRowsPerInst % 16 == 0) ? 1 : 16 / kRowsPerInst;
  static_assert(kBN * kU % kThreads == 0, "tile must split evenly over the workgroup");
  static_assert(kVar == 1 || 16 % kRowsPerInst == 0, "swizzle must repeat across instructions");
  struct Voff {
    uint32_t v[kVar];  // per-lane byte offsets of instructions 0 .. kVar-1 (then repeating)
  };
  static __device__ __forceinline__ Voff voff_lane(int wave, int lane, int row_stride_bytes) {
    const int rl = (wave * 64 + lane) / kU, pc = lane % kU;
    Voff o;
#pragma unroll
    for (int x = 0; x < kVar; ++x)
      o.v[x] = (uint32_t)rl * (uint32_t)row_stride_bytes + (uint32_t)((pc ^ swz<D>(rl + kRowsPerInst * x)) * 16);
    return o;
  }
  // instruction i of the tile starting at key row n0, into the LDS tile at lds_tile
  // (the tile's row offset goes in the scalar offset operand)
  static __device__ __forceinline__ void issue(i32x4 desc, uint32_t lds_tile, int n0, int i, int wave,
                                               const Voff& voff, int row_stride_bytes) {
    dma16_so(desc, lds_tile + (uint32_t)(i * kWaves + wave) * kInstBytes, voff.v[i % kVar],
             (uint32_t)(n0 + kRowsPerInst * i) * (uint32_t)row_stride_bytes);
  }
  static __device__ __forceinline__ void tile(i32x4 desc, uint32_t lds_tile, int n0, int wave, const Voff& voff,
                                              int row_stride_bytes) {
#pragma unroll
    for (int i = 0; i < kInst; ++i) issue(desc, lds_tile, n0, i, wave, voff, row_stride_bytes);
  }
};

// (a ^ b) + c in one instruction, opaque to the compiler, so constant offsets
// added to the result become instruction offsets instead of being
// reassociated into extra live base registers.
__device__ __forceinline__ uint32_t xor_add(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_xad_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(b), "v"(c));
  return r;
}

// Row max over this lane and lane ^ 32.  A plain v_max_f32: its inputs are
// MFMA results or -inf, never signalling NaNs, so the quieting that fmaxf
// adds to each operand is not needed.
__device__ __forceinline__ float row_max_xor32(float x) {
  const int xi = __float_as_int(x);
  const auto pr = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(__int_as_float(pr[0])), "v"(__int_as_float(pr[1])));
  return r;
}

// Per-lane LDS addressing of the two MFMA operands that come from LDS.
//  K (A operand of S^T = K Q^T): lane l reads row 32*kb + l%32, logical chunk
//    2t + l/32 of contraction step t.  swz of that row equals swz(l%32), and
//    (2t + g) ^ s = 2t ^ (g ^ s), so the byte offset within the row is
//    32t ^ kx with kx = 16 * (g ^ swz(l%32)).
//  V (A operand of O^T += V^T P^T, ds_read_b64_tr_b16): see pv_kstep.  For
//    k-step (kb, st) the rows are 32*kb + 16*st + rb (+ 8), and swz only sees
//    the low four row bits, so kb and st are constant offsets and each lane
//    needs one address per (32-column block of O^T, row half).
template <int D>
struct LdsAddr {
  uint32_t k_row;       // lds base + (l%32) * row bytes
  uint32_t kx;          // 16 * (g ^ swz(l%32))
  uint32_t v[D / 32][2];  // lds base + V row/chunk offset for (d block, row half)
};

// Geometry of the S^T = K Q^T operands.  16-bit Q and K: one
// v_mfma_f32_32x32x16 per 16 head-dim elements.  FP8 Q and K (QK8, E4M3 codes):
// one v_mfma_f32_32x32x64_f8f6f4 per 64 head-dim bytes; a K row of D bytes is
// stored, swizzled and fetched exactly like a 16-bit row of D / 2 elements,
// and FP8 step u reads the two 16-byte chunks that the 16-bit kernel reads at
// its steps 2u and 2u + 1 (so the conflict-free read pattern is the same).
// The Q operand of a lane holds the same chunks of its query row in the same
// order, so each contraction slot pairs equal head-dim indices of q and k.
typedef short s16x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
template <int D, bool QK8>
struct QkGeom {
  static constexpr int kDK = QK8 ? D / 2 : D;          // K row in LDS as 16-bit elements
  static constexpr int kSteps = QK8 ? D / 64 : D / 16;  // QK MFMAs per 32-key block
  using Op = typename std::conditional<QK8, s16x16, s16x8>::type;  // Q or K operand of one MFMA
};

template <bool BF16, bool QK8, typename Op>
__device__ __forceinline__ f32x16 qk_mfma(const Op& a, const Op& b, f32x16 c) {
  if constexpr (QK8)
    // format code 0 for both operands: FP8 E4M3; no block scales
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, a), __builtin_bit_cast(i32x8, b),
                                                           c, 0, 0, 0, 0, 0, 0);
  else
    return mfma32x32x16<BF16>(a, b, c);
}

// K operand of QK step t at a K row address (k_row + k_tile + block offset,
// with the per-lane chunk XOR kx): one 16-byte read, or two for FP8.
template <int D, bool QK8>
__device__ __forceinline__ typename QkGeom<D, QK8>::Op k_operand(uint32_t kx, uint32_t base, int t) {
  if constexpr (QK8) {
    const s16x8 lo = lds_read_b128(base + ((uint32_t)(64 * t) ^ kx));
    const s16x8 hi = lds_read_b128(base + ((uint32_t)(64 * t + 32) ^ kx));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
  } else {
    return lds_read_b128(base + ((uint32_t)(32 * t) ^ kx));
  }
}

// S^T[kb] = K(tile) Q^T for the wave's 32 queries (first tile, diagonal and
// tail tiles).  qreg[t]: this lane's Q^T operand of contraction step t.
template <int D, bool BF16, bool QK8>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[kKB], uint32_t k_tile, uint32_t k_row, uint32_t kx,
                                        const typename QkGeom<D, QK8>::Op (&qreg)[QkGeom<D, QK8>::kSteps]) {
  using Gq = QkGeom<D, QK8>;
#pragma unroll
  for (int kb = 0; kb < kKB; ++kb) s[kb] = (f32x16){};
#pragma unroll
  for (int t = 0; t < Gq::kSteps; ++t) {
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
      const auto a = k_operand<D, QK8>(kx, k_row + k_tile + (uint32_t)(kb * 32 * Gq::kDK * 2), t);
      s[kb] = qk_mfma<BF16, QK8>(a, qreg[t], s[kb]);
    }
  }
}

// The same with 16-bit K and this lane's K operand address of each step t
// in K buffer 0 given (kaddr[t]; k_tile selects the buffer).
template <int D, bool BF16>
__device__ __forceinline__ void qk_tile_addr(f32x16 (&s)[kKB], uint32_t k_tile, const uint32_t (&kaddr)[D / 16],
                                             const s16x8 (&qreg)[D / 16]) {
#pragma unroll
  for (int kb = 0; kb < kKB; ++kb) s[kb] = (f32x16){};
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
      const s16x8 a = lds_read_b128(kaddr[t] + k_tile + (uint32_t)(kb * 32 * D * 2));
      s[kb] = mfma32x32x16<BF16>(a, qreg[t], s[kb]);
    }
  }
}

// Division of a non-negative int below 2^31 by a fixed divisor d >= 1 with a
// multiplier and a shift worked out on the host (round-up method of
// Granlund and Montgomery): q = (mulhi(n, mul) + n) >> shift, with
// shift = ceil(log2 d) and mul = floor(2^32 (2^shift - d) / d) + 1.  Exact for
// every n < 2^31; scalar instructions only.
struct FastDiv {
  uint32_t mul, shift, d;
};
__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) { return (__umulhi(n, f.mul) + n) >> f.shift; }

// Grid decomposition constants of one launch (see the tile-id decode in the kernel).
struct TileDecode {
  FastDiv packs, qtiles, hkv;  // divisors: head packs per GQA group, q-tiles, KV heads
  int group;                   // query heads per KV head
  int pack_shift;              // log2 of the query heads per workgroup
};

// QK8: q and k hold FP8 E4M3 codes (byte strides in st.q and st.k) and
// scale_log2 carries their per-tensor scales; v and o are 16-bit.
template <int D, bool BF16, bool CAUSAL, bool QK8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(waves_per_eu<D>(), waves_per_eu<D>())))
void prefill_fwd_kernel(const void* __restrict__ q, const void* __restrict__ k,
                        const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                        float* __restrict__ lse, int N, int M, int Hq, int Hkv,
                        int n_qtiles, int total, TileDecode td, int causal_off, attn_strides_t st,
                        float scale_log2) {
  using Gq = QkGeom<D, QK8>;
  constexpr int kDT = Gq::kSteps;  // contraction steps of QK^T
  constexpr int kDB = D / 32;  // 32-row blocks of O^T
  constexpr uint32_t kTBK = kBN * Gq::kDK * 2;  // bytes of one K tile
  constexpr uint32_t kTB = kBN * D * 2;         // bytes of one V tile
  using FK = Fetch<Gq::kDK>;
  using F = Fetch<D>;
  constexpr int kEB = QK8 ? 1 : 2;  // bytes per q or k element
  // LDS: K buffers 0, 1, V buffers 0, 1 (64 KB at d = 128; 48 KB with FP8 K).
  __shared__ __attribute__((aligned(1024))) uint16_t smem[(2 * kTBK + 2 * kTB) / 2];
  __shared__ int restart_flag[kWaves];  // bf16: a wave's pass left its range (see the KV pass)
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u16*)smem;
  const uint32_t kbuf0 = lds0, vbuf0 = lds0 + 2 * kTBK;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int G = lane >> 4, sl = lane & 15;

  // ---- tile id -> (b, kv head, heads, q-tile) ----
  // A workgroup takes `pack` query heads of one GQA group (they share K/V) and
  // kBM / pack query rows of each: wave w works on head pack-slot
  // w / (kWaves / pack), rows 32 (w % (kWaves / pack)) .. +31 of the tile.  With causal masking
  // a shorter row span per head means a smaller masked diagonal and fewer
  // waves idle past their diagonal, at the same K/V reuse per tile.
  const int lid = xcd_remap(blockIdx.x, total);
  const int group = td.group;
  const int rows = kBM >> td.pack_shift;          // query rows per head in this tile
  static_assert(kWaves == 4, "log2(kWaves) below");
  const int wshift = 2 - td.pack_shift;           // log2 of the waves per head
  const uint32_t rest = fdiv((uint32_t)lid, td.packs);
  const int hp = lid - (int)(rest * td.packs.d);  // head pack within the GQA group
  const uint32_t bkv = fdiv(rest, td.qtiles);
  const int qt = n_qtiles - 1 - (int)(rest - bkv * (uint32_t)n_qtiles);  // longest (causal) first
  const uint32_t bq = fdiv(bkv, td.hkv);
  const int kvh = (int)(bkv - bq * (uint32_t)Hkv), b = (int)bq;
  const int h = kvh * group + (hp << td.pack_shift) + (wave >> wshift);  // this wave's query head

  const int q_start = qt * rows;
  const int qw = q_start + (wave & ((1 << wshift) - 1)) * 32;  // first query of this wave
  const int qlast = qw + 31;           // last query of this wave
  const int qi = qw + l32;             // this lane's query (prologue; see query_now)
  // the same, recomputed where the general steps and the epilogue need it,
  // instead of one register held for the whole kernel
  auto query_now = [&]() __attribute__((always_inline)) { return qw + (int)(lane_id_now() & 31); };

  // element strides {batch, token, head}; k and v share their token stride
  // (in elements; FP8 k elements are bytes)
  const int64_t kv_row_stride = st.k[1];
  const int kv_row_bytes = (int)(kv_row_stride * 2);
  const int k_row_bytes = (int)(kv_row_stride * kEB);
  const i32x4 kdesc = make_desc_bytes(static_cast<const uint8_t*>(k) + (b * st.k[0] + kvh * st.k[2]) * kEB,
                                      k_row_bytes, M, D * kEB);
  const i32x4 vdesc = make_desc(v + b * st.v[0] + kvh * st.v[2], kv_row_stride, M, D);
  const auto voff = F::voff_lane(wave, lane, kv_row_bytes);
  const auto voffk = FK::voff_lane(wave, lane, k_row_bytes);  // the same values without QK8

  // ---- Q^T operand: lane l of step t holds Q[qw + l%32][16t + 8g .. +7] ----
  typename Gq::Op qreg[kDT];

  f32x16 acc_o[kDB];
  float m_run = -INFINITY;  // running max of scale*log2e*s (the reference max)
  float l_run = 0.f;        // running sum over this lane's keys
#pragma unroll
  for (int i = 0; i < kDB; ++i) acc_o[i] = (f32x16){};

  // causal: query i sees keys 0 .. i + causal_off (causal_off = M - N >= 0)
  const int kv_end = CAUSAL ? min(M, q_start + rows + causal_off) : M;
  const int n_tiles = (kv_end + kBN - 1) / kBN;
  // last tile that holds a key <= some query of this wave
  const int wave_tiles = CAUSAL ? min(n_tiles, (qlast + causal_off) / kBN + 1) : n_tiles;

  // ---- prologue: K(0), V(0), K(1) to LDS, Q^T to registers; S(0) ----
  // The tile fetches go out first, and the Q loads without a branch (a row
  // past N loads row N-1, whose result is never stored), so that the wait
  // for all of them starts as early as possible.
  FK::tile(kdesc, kbuf0, 0, wave, voffk, k_row_bytes);
  F::tile(vdesc, vbuf0, 0, wave, voff, kv_row_bytes);
  if (n_tiles > 1) FK::tile(kdesc, kbuf0 + kTBK, kBN, wave, voffk, k_row_bytes);
  {
    // lane half g holds head-dim chunks 2t + g (16 bytes each) of step t
    // (FP8: chunks 4t + g and 4t + 2 + g, as the K operand)
    const uint8_t* qp = static_cast<const uint8_t*>(q) +
                        (b * st.q[0] + (int64_t)min(qi, N - 1) * st.q[1] + h * st.q[2]) * kEB + 16 * g;
#pragma unroll
    for (int t = 0; t < kDT; ++t) {
      if constexpr (QK8) {
        const s16x8 lo = *reinterpret_cast<const s16x8*>(qp + 64 * t);
        const s16x8 hi = *reinterpret_cast<const s16x8*>(qp + 64 * t + 32);
        qreg[t] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
      } else {
        qreg[t] = *reinterpret_cast<const s16x8*>(qp + 32 * t);
      }
    }
  }
  // ---- per-lane LDS operand addresses ----
  LdsAddr<D> la;
  la.k_row = lds0 + (uint32_t)l32 * Gq::kDK * 2;
  la.kx = (uint32_t)((g ^ swz<Gq::kDK>(l32)) << 4);
  // 16-bit Q and K: this lane's K operand address of each contraction step t
  // in K buffer 0, worked out once per item; the K buffer (16 KB apart) and
  // the 32-key block (8 KB) are instruction offsets of the reads.
  uint32_t kaddr[QK8 ? 1 : kDT];
  if constexpr (!QK8) {
#pragma unroll
    for (int t = 0; t < kDT; ++t) kaddr[t] = la.k_row + ((uint32_t)(32 * t) ^ la.kx);
  }
  {
    // ds_read_b64_tr_b16: in each 16-lane group, lane i receives element i%4
    // of the 8 bytes addressed by lane 4*jj + i/4, for jj = 0..3.  Lane s of
    // group G addresses V[K0 + s/4][D0 + 4*(s%4)] with D0 = 32*db + 16*(G&1)
    // and K0 the first key of the slot run, so lane i gets 4 consecutive keys
    // of column D0 + i%16 = 32*db + l%32.  Rows: rb = 4*(G/2) + s/4 for slots
    // 0..3 and rb + 8 for slots 4..7.
    const int rb = 4 * (G >> 1) + (sl >> 2);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int row = rb + 8 * hh;
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const int col = 32 * db + 16 * (G & 1) + 4 * (sl & 3);
        la.v[db][hh] = vbuf0 + (uint32_t)(row * D * 2 + ((((col >> 3) ^ swz<D>(row)) << 4) | ((col & 7) * 2)));
      }
    }
  }

  f32x16 s_a[kKB], s_b[kKB];  // S of the current tile is always in s_a between steps

  // O^T += V(j)^T P(j) for one 16-key k-step (kb, st) and all d blocks; v_tile
  // is the V buffer's offset from V buffer 0.
  auto pv_kstep = [&](uint32_t v_tile, int kb, int st, const s16x8& pb, const s16x8* pl) __attribute__((always_inline)) {
    const uint32_t koff = v_tile + (uint32_t)((32 * kb + 16 * st) * D * 2);
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      const s16x4 lo = lds_read_tr16_b64(la.v[db][0] + koff);
      const s16x4 hi = lds_read_tr16_b64(la.v[db][1] + koff);
      const s16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      acc_o[db] = mfma32x32x16<BF16>(a, pb, acc_o[db]);
      if (pl != nullptr) acc_o[db] = mfma32x32x16<BF16>(a, *pl, acc_o[db]);
    }
  };

  // Multiply O and l by alpha = 2^(m_run - m_new) when the reference max moves
  // up to m_new.  Moves happen only where O and l hold weights of at most 2^8
  // per key (exact steps, or a wave's first tile), so an alpha that flushes
  // to zero (a move of more than 126 log2 units) drops contributions below
  // 2^-100 of the new tile's.
  auto move_reference_to = [&](const float m_new) __attribute__((always_inline)) {
    const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    l_run = l_run * alpha;
#pragma unroll
    for (int i = 0; i < kDB; ++i) acc_o[i] = acc_o[i] * alpha;
    m_run = m_new;
  };

  // Row max of tile j and the rare move of the reference max (see below).
  auto row_max_update = [&](f32x16 (&s_cur)[kKB]) __attribute__((always_inline)) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s_cur[kb][i]);
    mx = max_xor32(mx);
    const float m_tile = (mx == -INFINITY) ? -INFINITY : mx * scale_log2;
    // Move the reference max only when it grows by more than 2^8; otherwise
    // p may reach 2^8, which fp32 accumulation and 16-bit P represent fine.
    if (__builtin_amdgcn_ballot_w64(m_tile > m_run + 8.0f)) {
      move_reference_to(fmaxf(m_run, m_tile));
    }
  };

  // p = 2^(s*scale*log2e - m) for 8 accumulator elements, packed to the PV B
  // operand; k-step (kb, st) uses accumulator elements 8*st .. 8*st+7, i.e.
  // keys 32*kb + 16*st + 8*(jj/4) + 4*g + jj%4 for slot jj.  The row sum l is
  // accumulated from the unrounded fp32 p (a sum of 16-bit-rounded weights
  // can be off by 2^-9 relative when a few keys dominate, too much for lse).
  auto exp_pack = [&](const f32x16& sv, int st, float m_use, float& lsum, bool masked, s16x8& pb, s16x8* pl) __attribute__((always_inline)) {
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

  // General step (a masked or only first tile, diagonal and tail tiles, last
  // tile of a wave):
  // fetches K(j+2) and V(j+1), computes S(j+1) into s_b if this wave needs it,
  // then mask, softmax and PV of tile j from s_a; ends with S(j+1) in s_a.  The
  // buffer parity is a run-time value here (these steps are few).
  // exact == false (the max-free pass, tiles after the first): the reference
  // max stays where it is, as in the steady-state steps, so the tile needs no
  // row max; its masked keys get weight 0 after the exponential instead of a
  // score of -inf before it.
  auto step_general = [&](const int j, auto first, auto exact) __attribute__((always_inline)) {
    constexpr bool kFirst = decltype(first)::value;
    constexpr bool kFree = !decltype(exact)::value && !kFirst;
    // bf16: P is split into hi + lo parts on the first tile
    constexpr bool kSplit = BF16 && kFirst;
    const uint32_t par = (uint32_t)(j & 1);
    const uint32_t k_next = (1 - par) * kTBK, v_cur = par * kTB;
    const int n0 = j * kBN;
    if (j + 2 < n_tiles) FK::tile(kdesc, kbuf0 + par * kTBK, n0 + 2 * kBN, wave, voffk, k_row_bytes);
    if (j + 1 < n_tiles) F::tile(vdesc, vbuf0 + (1 - par) * kTB, n0 + kBN, wave, voff, kv_row_bytes);
    if (j + 1 < wave_tiles) {
      if constexpr (QK8)
        qk_tile<D, BF16, QK8>(s_b, k_next, la.k_row, opaque(la.kx), qreg);
      else
        qk_tile_addr<D, BF16>(s_b, k_next, kaddr, qreg);
    }
    if (j < wave_tiles) {
      const bool need_mask = (CAUSAL && n0 + kBN - 1 > qw + causal_off) || (n0 + kBN > M);
      // element i of block kb holds key n0 + 4 g + kc(kb, i), kc = 32 kb +
      // 8 (i / 4) + i % 4; the key is valid iff kc <= lim (key < M and, causal,
      // key <= query + causal_off)
      auto key_limit = [&]() __attribute__((always_inline)) {
        const int last = CAUSAL ? min(query_now() + causal_off, M - 1) : M - 1;
        return last - n0 - 4 * g;
      };
      if constexpr (kFree) {
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;  // finite after tile 0
        const int lim = need_mask ? key_limit() : kBN;
        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int kc = 32 * kb + 16 * st + 8 * (e >> 2) + (e & 3);
              const float y = __builtin_amdgcn_exp2f(fmaf(s_a[kb][8 * st + e], scale_log2, -m_use));
              pv[e] = kc <= lim ? y : 0.f;
              lsum += pv[e];
            }
            uint32_t w[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) w[u] = pack2<BF16>(pv[2 * u], pv[2 * u + 1]);
            pv_kstep(v_cur, kb, st, __builtin_bit_cast(s16x8, make_uint4(w[0], w[1], w[2], w[3])), nullptr);
          }
        l_run += lsum;
      } else {
        if (need_mask) {
          const int lim = key_limit();
#pragma unroll
          for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int kc = 32 * kb + 8 * (i >> 2) + (i & 3);
              s_a[kb][i] = kc <= lim ? s_a[kb][i] : -INFINITY;
            }
        }
        row_max_update(s_a);
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            s16x8 pb, pl;
            exp_pack(s_a[kb], st, m_use, lsum, need_mask, pb, kSplit ? &pl : nullptr);
            pv_kstep(v_cur, kb, st, pb, kSplit ? &pl : nullptr);
          }
        l_run += lsum;
      }
    }
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) s_a[kb] = s_b[kb];
    wait_tile_loads();
    kv_barrier();
  };

  // Raw row max of a tile's S (unscaled, over this lane and lane ^ 32).
  auto tile_max = [&](const f32x16 (&sv)[kKB]) __attribute__((always_inline)) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sv[kb][i]);
    return max_xor32(mx);
  };

  // Steady-state step (no mask, reference max finite, S(j+1) needed), written
  // as an explicit software pipeline of kN slots, one MFMA each: the 2 kDT QK
  // MFMAs of S(j+1) = K(j+1) Q^T, then the 4 kDB PV MFMAs of O^T += V(j)^T P(j)
  // (k-step ks = 2 kb + st, d block db).  Slot i issues MFMA i, the LDS reads
  // of MFMA i + kL, a share of the exp/pack work of tile j (the first few
  // exponentials come before slot 0; each P k-step is complete before its
  // first PV MFMA), in its first odd slots one of the
  // step's tile fetches, and in the last slots the row max of S(j+1) (whose
  // MFMAs have finished by then), which the next step uses.  The slots are
  // separated by scheduling fences, so the order is the one written here.
  // mx: row max of tile j on entry, of tile j+1 on return.  first: j == 0.
  // exact == false: the step neither takes the row max of
  // S(j+1) nor moves the reference max, which stays where the first tile put
  // it (see the KV pass below).
  auto step_fast = [&](const uint32_t k_next, const uint32_t v_cur, f32x16 (&s_cur)[kKB],
                       f32x16 (&s_next)[kKB], float& mx, auto&& fetch, auto first, auto exact) __attribute__((always_inline)) {
    constexpr bool kFirst = decltype(first)::value;
    constexpr bool kExact = decltype(exact)::value;
    auto move_reference = [&]() __attribute__((always_inline)) {
      // mx is finite here: the tile has no masked key (inputs holding Inf or
      // NaN give NaN outputs either way)
      const float m_tile = mx * scale_log2;
      if (__builtin_amdgcn_ballot_w64(m_tile > m_run + 8.0f)) {
        move_reference_to(fmaxf(m_run, m_tile));
      }
    };
    if constexpr (kFirst) {
      // O and l are still zero: the reference max is simply set
      m_run = (mx == -INFINITY) ? -INFINITY : mx * scale_log2;
    } else if constexpr (kExact) {
      move_reference();
    }
    // FP8 K: fresh copies per step keep the per-step K addresses from being
    // hoisted out of the KV loop as live registers (16-bit K uses kaddr)
    const uint32_t kx = opaque(la.kx);
    const uint32_t kbase = opaque(la.k_row + k_next);
    constexpr int kNQ = 2 * kDT, kNP = 4 * kDB, kN = kNQ + kNP;
    constexpr int kL = 4;                  // MFMAs whose operands are read ahead
    constexpr int kNF = F::kInst + FK::kInst;  // tile fetch instructions per step
    constexpr int kExpEnd = kNQ + 3 * kDB;  // first PV MFMA of the last k-step
    static_assert(kN >= 2 * kNF, "fetch slots");
    typename Gq::Op qv[kDT], ka[kNQ];
    s16x8 va[kNP], pb[4];
    float pe[4][8];
    float lsum = 0.f, mxn = -INFINITY;
    const float neg_m = (kFirst && m_run == -INFINITY) ? 0.f : -m_run;

    auto reads = [&](const int i) __attribute__((always_inline)) {
      if (i < kNQ) {
        const int t = i >> 1, kb = i & 1;
        if (kb == 0) qv[t] = qreg[t];
        if constexpr (QK8) {
          ka[i] = k_operand<D, QK8>(kx, kbase + (uint32_t)(kb * 32 * Gq::kDK * 2), t);
        } else {
          ka[i] = lds_read_b128(kaddr[t] + k_next + (uint32_t)(kb * 32 * D * 2));
        }
      } else if (i < kN) {
        const int pi = i - kNQ, ks = pi / kDB, db = pi % kDB;
        const uint32_t koff = v_cur + (uint32_t)(16 * ks * D * 2);  // keys 16 ks .. 16 ks + 15
        const s16x4 lo = lds_read_tr16_b64(la.v[db][0] + koff);
        const s16x4 hi = lds_read_tr16_b64(la.v[db][1] + koff);
        va[pi] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    };
    // element e of P k-step ks (see exp_pack for the key order)
    auto exp_elem = [&](const int k) __attribute__((always_inline)) {
      const int ks = k >> 3, e = k & 7;
      const float y = __builtin_amdgcn_exp2f(fmaf(s_cur[ks >> 1][8 * (ks & 1) + e], scale_log2, neg_m));
      pe[ks][e] = y;
      lsum += y;
      if (e == 7) {
        uint32_t w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = pack2<BF16>(pe[ks][2 * u], pe[ks][2 * u + 1]);
        pb[ks] = __builtin_bit_cast(s16x8, make_uint4(w[0], w[1], w[2], w[3]));
      }
    };

    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kL; ++i) reads(i);
    // the first exponentials go before the first MFMA, which waits for its K
    // operand from LDS right after the step's barrier
    constexpr int kPre = 4;
#pragma unroll
    for (int k = 0; k < kPre; ++k) exp_elem(k);
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i < kNQ) {
        const int t = i >> 1, kb = i & 1;
        s_next[kb] = qk_mfma<BF16, QK8>(ka[i], qv[t], t == 0 ? (f32x16){} : s_next[kb]);
      } else {
        const int pi = i - kNQ, ks = pi / kDB, db = pi % kDB;
        acc_o[db] = mfma32x32x16<BF16>(va[pi], pb[ks], acc_o[db]);
      }
      reads(i + kL);
      if ((i & 1) && (i >> 1) < kNF) fetch(i >> 1);
      // the other elements k: floor((k - kPre) * kExpEnd / (32 - kPre)) == i
#pragma unroll
      for (int k = kPre; k < 32; ++k)
        if ((k - kPre) * kExpEnd / (32 - kPre) == i) exp_elem(k);
      if (kExact && i >= kExpEnd) {
        // row max of S(j+1), spread over the slots after the exp work
        constexpr int kMaxSlots = kN - kExpEnd;
        const int r = i - kExpEnd;
#pragma unroll
        for (int k = 0; k < 32; ++k)
          if (k * kMaxSlots / 32 == r) mxn = fmaxf(mxn, s_next[k >> 4][k & 15]);
        if (i == kN - 1) mx = row_max_xor32(mxn);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    l_run += lsum;
  };

  // One steady-state iteration; P is the parity of j (buffers alternate
  // between tiles): S(j+1) reads K buffer 1-P, PV(j) reads V buffer P, and the
  // iteration fetches K(j+2) into K buffer P and V(j+1) into V buffer 1-P.
  auto step_fast_p = [&](const int j, f32x16 (&s_cur)[kKB], f32x16 (&s_next)[kKB], float& mx, auto parity,
                         auto first, auto exact) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
    const uint32_t k_fill = kbuf0 + P * kTBK, v_fill = vbuf0 + (1 - P) * kTB;
    const int n0 = j * kBN;
    // j + 1 < wave_tiles <= n_tiles, so V(j+1) exists; without a K(j+2) the K
    // slots repeat the V(j+1) fetches (same bytes to the same place).  With
    // FP8 K (other fetch geometry) K(j+2) is fetched anyway: the K buffer is
    // free, and rows past M read as zeros.
    const bool has_k = QK8 || j + 2 < n_tiles;
    const i32x4 d2 = has_k ? kdesc : vdesc;
    const uint32_t l2 = has_k ? k_fill : v_fill;
    const int r2 = has_k ? n0 + 2 * kBN : n0 + kBN;
    auto fetch = [&](int i) __attribute__((always_inline)) {
      if (i < F::kInst)
        F::issue(vdesc, v_fill, n0 + kBN, i, wave, voff, kv_row_bytes);
      else if constexpr (QK8)
        FK::issue(kdesc, k_fill, n0 + 2 * kBN, i - F::kInst, wave, voffk, k_row_bytes);
      else
        F::issue(d2, l2, r2, i - F::kInst, wave, voff, kv_row_bytes);
    };
    step_fast((1 - P) * kTBK, P * kTB, s_cur, s_next, mx, fetch, first, exact);
    wait_tile_loads();
    kv_barrier();
  };

  // Steps 0 .. fast_end-1 take the steady-state path: no key of the tile is
  // masked and S(j+1) is needed (if fast_end is 0, tile 0 is a general step).
  // Every wave runs n_tiles steps, each ending in one barrier.
  const int fast_end =
      min(min(wave_tiles - 1, M / kBN), CAUSAL ? (qw + causal_off + 1) / kBN : wave_tiles);

  // One pass over the KV tiles: S(0) from K(0) (fetched before the pass), then
  // every tile through the steady-state or the general step.
  auto kv_pass = [&](auto exact) __attribute__((always_inline)) {
    wait_tile_loads();
    kv_barrier();
    if constexpr (QK8)
      qk_tile<D, BF16, QK8>(s_a, 0, la.k_row, la.kx, qreg);
    else
      qk_tile_addr<D, BF16>(s_a, 0, kaddr, qreg);
    kv_barrier();  // K buffer 0 is refilled in iteration 0
    // tile 0 takes the steady-state path too when it has no masked key and S(1)
    // is needed (fast_end >= 1); O and l start at zero there
    float mx;  // row max of the tile in s_a, carried by the fast steps
    if (fast_end >= 1) {
      mx = tile_max(s_a);
      step_fast_p(0, s_a, s_b, mx, std::integral_constant<int, 0>{}, std::true_type{}, exact);
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) s_a[kb] = s_b[kb];
    } else {
      step_general(0, std::true_type{}, exact);
      mx = tile_max(s_a);
    }
    int j = 1;
    for (; j + 1 < fast_end; j += 2) {
      step_fast_p(j, s_a, s_b, mx, std::integral_constant<int, 1>{}, std::false_type{}, exact);
      step_fast_p(j + 1, s_b, s_a, mx, std::integral_constant<int, 0>{}, std::false_type{}, exact);
    }
    if (j < fast_end) {
      step_fast_p(j, s_a, s_b, mx, std::integral_constant<int, 1>{}, std::false_type{}, exact);
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) s_a[kb] = s_b[kb];
      ++j;
    }
    for (; j < n_tiles; ++j) step_general(j, std::false_type{}, exact);
  };

  // A first pass runs without a moving reference max (the reference is the
  // first tile's row max).  Tiles whose scores exceed it give large weights,
  // which P and the fp32 accumulators hold at full relative precision up to
  // P's largest value, so the result is the same up to rounding.  A pass
  // whose weights may have outgrown that range leaves a lane's row sum at or
  // above kRerun (2^100 for bf16, whose weights reach 2^127; 2^15 for fp16,
  // so that no kept weight exceeds 2^15 < 65504: a weight that rounded to Inf
  // in fp16 passed 2^15), or an accumulator that is not finite; then the
  // whole workgroup runs the pass again with the exact steps (all four waves
  // share the K/V fetches, so the decision is taken jointly through LDS).
  {
    constexpr float kRerun = BF16 ? 0x1p100f : 0x1p15f;
    kv_pass(std::false_type{});
    // z is NaN iff some O accumulator is Inf or NaN (o * 0 is NaN exactly
    // then); one chain per d block, so the chains run side by side
    float zc[kDB];
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      zc[db] = acc_o[db][0] * 0.f;
#pragma unroll
      for (int i = 1; i < 16; ++i) zc[db] = fmaf(acc_o[db][i], 0.f, zc[db]);
    }
    float z = zc[0];
#pragma unroll
    for (int db = 1; db < kDB; ++db) z += zc[db];
    const bool bad = !(l_run < kRerun) || z != z;
    const bool wave_bad = __builtin_amdgcn_ballot_w64(bad) != 0;
    if (lane == 0) restart_flag[wave] = wave_bad ? 1 : 0;
    __syncthreads();
    // uniform by construction; readfirstlane tells the compiler so
    const bool again =
        __builtin_amdgcn_readfirstlane(restart_flag[0] | restart_flag[1] | restart_flag[2] | restart_flag[3]) != 0;
    if (again) {
      m_run = -INFINITY;
      l_run = 0.f;
#pragma unroll
      for (int i = 0; i < kDB; ++i) acc_o[i] = (f32x16){};
      FK::tile(kdesc, kbuf0, 0, wave, voffk, k_row_bytes);
      F::tile(vdesc, vbuf0, 0, wave, voff, kv_row_bytes);
      if (n_tiles > 1) FK::tile(kdesc, kbuf0 + kTBK, kBN, wave, voffk, k_row_bytes);
      kv_pass(std::true_type{});
    }
  }

  // ---- epilogue: O / l -> 16-bit, lse = ln2 * (m + log2 l) ----
  // Lane (l32, g) holds d = 32 db + 8 r + 4 g + (0..3) of its query row: half g
  // of 16-byte chunk 4 db + r.  The rows go through LDS (this wave's share of
  // the K/V buffers, free after the last step's barrier: 32 rows of D 16-bit
  // values), row-major with the chunk index XOR-swizzled by the row, and come
  // back as whole rows, so every global store writes complete 128-byte lines
  // instead of 16 bytes of 32 rows.
  const float l_tot = sum_xor32(l_run);
  const float inv = 1.f / l_tot;
  {
    constexpr int kRowB = D * 2;              // bytes per O row
    constexpr int kCh = D / 8;                // 16-byte chunks per row
    constexpr int kRowsPerRead = 64 / kCh;    // rows covered by one wave-wide 16-byte read
    const uint32_t ob = kbuf0 + (uint32_t)wave * (uint32_t)(32 * D * 2);  // K/V buffers are free now
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const u32x2 w = {pack2<BF16>(acc_o[db][4 * r + 0] * inv, acc_o[db][4 * r + 1] * inv),
                         pack2<BF16>(acc_o[db][4 * r + 2] * inv, acc_o[db][4 * r + 3] * inv)};
        const int chunk = (4 * db + r) ^ (l32 % kCh);
        lds_write_b64(ob + (uint32_t)(l32 * kRowB + chunk * 16 + g * 8), w);
      }
    lds_lane_fence();
    const int c = lane % kCh;
    constexpr int kReads = 32 / kRowsPerRead;
    s16x8 val[kReads];
#pragma unroll
    for (int k = 0; k < kReads; ++k) {
      const int row = k * kRowsPerRead + lane / kCh;
      val[k] = lds_read_b128(ob + (uint32_t)(row * kRowB + ((c ^ (row % kCh)) * 16)));
    }
#pragma unroll
    for (int k = 0; k < kReads; ++k) {
      const int qrow = qw + k * kRowsPerRead + lane / kCh;
      if (qrow < N)
        *reinterpret_cast<s16x8*>(o + b * st.o[0] + (int64_t)qrow * st.o[1] + h * st.o[2] + 8 * c) = val[k];
    }
  }
  const int qe = query_now();
  if (lse != nullptr && g == 0 && qe < N) lse[((int64_t)b * Hq + h) * N + qe] = (m_run + log2f(l_tot)) * kLn2;
}

// Host-side launcher (one instance per head dim, dtype, mask and Q/K format).
template <int D, bool BF16, bool CAUSAL, bool QK8>
hipError_t launch_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                          int Hkv, int N, int M, float scale_log2, const attn_strides_t& st, hipStream_t stream) {
  // query heads per workgroup: the largest power of two that divides the GQA
  // group and leaves at least 64 rows (one K/V tile) per head
  const int group = Hq / Hkv;
  int pack = 1;
  while (pack * 2 * 64 <= kBM && group % (pack * 2) == 0) pack *= 2;
  const int rows = kBM / pack;
  const int n_qtiles = (N + rows - 1) / rows;
  const int total = B * (Hq / pack) * n_qtiles;
  auto fast_div = [](uint32_t d) {
    uint32_t l = 0;
    while ((1u << l) < d) ++l;
    const uint64_t mul = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
    return FastDiv{(uint32_t)mul, l, d};
  };
  int pack_shift = 0;
  while ((1 << pack_shift) < pack) ++pack_shift;
  const TileDecode td{fast_div((uint32_t)(group / pack)), fast_div((uint32_t)n_qtiles), fast_div((uint32_t)Hkv),
                      group, pack_shift};
  return launch(&prefill_fwd_kernel<D, BF16, CAUSAL, QK8>, dim3(total), dim3(kThreads), stream, q, k, v, o, lse, N,
                M, Hq, Hkv, n_qtiles, total, td, CAUSAL ? M - N : 0, st, scale_log2);
}

hipError_t prefill_dispatch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                            int Hkv, int N, int M, int d, bool causal, bool bf16, float scale,
                            const attn_strides_t& st, hipStream_t stream) {
  const float sl2 = scale * kLog2e;
#define ATTN_PREFILL_CASE(DD, BB, CC) \
  if (d == DD && bf16 == BB && causal == CC) \
    return launch_prefill<DD, BB, CC, false>(q, k, v, o, lse, B, Hq, Hkv, N, M, sl2, st, stream);
  ATTN_PREFILL_CASE(32, false, false)
  ATTN_PREFILL_CASE(32, false, true)
  ATTN_PREFILL_CASE(32, true, false)
  ATTN_PREFILL_CASE(32, true, true)
  ATTN_PREFILL_CASE(64, false, false)
  ATTN_PREFILL_CASE(64, false, true)
  ATTN_PREFILL_CASE(64, true, false)
  ATTN_PREFILL_CASE(64, true, true)
  ATTN_PREFILL_CASE(128, false, false)
  ATTN_PREFILL_CASE(128, false, true)
  ATTN_PREFILL_CASE(128, true, false)
  ATTN_PREFILL_CASE(128, true, true)
  ATTN_PREFILL_CASE(256, false, false)
  ATTN_PREFILL_CASE(256, false, true)
  ATTN_PREFILL_CASE(256, true, false)
  ATTN_PREFILL_CASE(256, true, true)
#undef ATTN_PREFILL_CASE
  return hipErrorInvalidValue;
}

// Q and K as FP8 E4M3 codes with per-tensor scales: the scores are
// scale * q_scale * k_scale * (codes' values), folded into one factor.
hipError_t prefill_fp8qk_dispatch(const void* q8, const void* k8, const void* v, void* o, float* lse, int B, int Hq,
                                  int Hkv, int N, int M, int d, bool causal, bool bf16, float scale, float q_scale,
                                  float k_scale, const attn_strides_t& st, hipStream_t stream) {
  const float sl2 = scale * q_scale * k_scale * kLog2e;
#define ATTN_FP8QK_CASE(DD, BB, CC) \
  if (d == DD && bf16 == BB && causal == CC) \
    return launch_prefill<DD, BB, CC, true>(q8, k8, v, o, lse, B, Hq, Hkv, N, M, sl2, st, stream);
  ATTN_FP8QK_CASE(64, false, false)
  ATTN_FP8QK_CASE(64, false, true)
  ATTN_FP8QK_CASE(64, true, false)
  ATTN_FP8QK_CASE(64, true, true)
  ATTN_FP8QK_CASE(128, false, false)
  ATTN_FP8QK_CASE(128, false, true)
  ATTN_FP8QK_CASE(128, true, false)
  ATTN_FP8QK_CASE(128, true, true)
#undef ATTN_FP8QK_CASE
  return hipErrorInvalidValue;
}

}  // namespace attn
