// Split-KV decode ("Flash Decoding") for gfx950: the per-chunk partial kernel
// and the log-sum-exp merge kernel ("CUDA Flash Decoding", section 2.2: chunk
// partials O_c, lse_c and the weighted reduce; section 3: the two-kernel data
// flow; section 6: the reduce kernel).
//
// MI355X design (not the page's CUDA design):
//  * both chunk kernels run a persistent grid of 256-thread workgroups (as
//    many as fit on the chip at once) that take chunk items in turn, so the
//    grid drains evenly.  Every K and V load of a chunk (64 KB at d = 128) is
//    issued up front with a nontemporal hint: V does not depend on the
//    scores, so the whole chunk is in flight at once and the kernel streams
//    HBM.  Partials are written in fp32 (O_c normalised) with nontemporal
//    stores: through the write-back caches they cost several percent of the
//    chunk kernel's time.
//  * matrix-core kernel (GQA groups, chunks longer than 128 keys, MHA
//    launches of at least 2048 items, and every paged or FP8 call): an item
//    is (chunk, batch, kv head, up to 16 query heads of the group), the heads
//    being the columns of v_mfma_f32_16x16x32, so K and V are read once per
//    kv head; Q, K and V are staged in LDS, V^T read back through transposed
//    reads.  Its paged mode fetches each instruction's rows from their page
//    through a per-page descriptor; its FP8 mode streams E4M3 code rows and
//    converts them to 16 bits on the way into LDS.
//  * VALU kernel (small MHA launches): an item is (chunk, batch, query head);
//    a row of K/V is read by d/8 consecutive lanes, 16 bytes each, scores use
//    fp32 accumulation (v_dot2_f32_{f16,bf16}) and a DPP sum over the lanes
//    of a row.  Its per-item path is shorter, which wins when the grid runs
//    only a few rounds of items.
//  * softmax statistics use exp2 with the scale folded into one multiply.
//  * merge kernel: one workgroup per (batch, query head, slice of 16 to 128
//    columns; the widest slice that still gives 512 workgroups), one pass
//    over the partials with a running max (no separate pass for the global
//    log-sum-exp, no limit on the number of chunks), 16-byte loads, and eight
//    independent loads in flight per thread; the per-thread states of a
//    column are combined by lane shuffles and one LDS step.
#include <algorithm>
#include <mutex>

#include "device_common.h"
#include "launch.h"
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

// Sum over the kLanes (4, 8 or 16) consecutive lanes that share one key row.
template <int kLanes>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (kLanes == 16) return sum16(x);
  else if constexpr (kLanes == 8) return sum8(x);
  else return sum4(x);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16 bytes of FP8 codes, streamed.
__device__ __forceinline__ uint4 load_stream8(const uint8_t* p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// 16-byte load that streams past the caches (K/V are read exactly once).
__device__ __forceinline__ uint4 load_stream(const uint16_t* p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Persistent grid: workgroup w handles items w, w + gridDim.x, ... where item
// = c + C * (b * Hq + h), so every workgroup ends at about the same time.
template <int D, bool BF16>
__global__ __launch_bounds__(kDecThreads)
void decode_chunk_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                         const uint16_t* __restrict__ v, float* __restrict__ o_part,
                         float* __restrict__ lse_part, int Hq, int Hkv, int M, int C,
                         int n_items, float scale_log2) {
  constexpr int kLanes = D / 8;                       // lanes per key row
  constexpr int kRowsPerPass = kDecThreads / kLanes;  // 16, 32 or 64 (d = 128, 64, 32)
  constexpr int kPasses = kChunk / kRowsPerPass;      // rows per thread
  constexpr int kWaves = kDecThreads / 64;
  __shared__ float red[2][kWaves];
  __shared__ float opart[kWaves][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = tid % kLanes;  // 16-byte column chunk
  const int r0 = tid / kLanes;   // first row of this thread

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int c = item % C;
    const int bh = item / C;
    const int h = bh % Hq, b = bh / Hq;
    const int kvh = h / (Hq / Hkv);
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
      kr[p] = row < len ? load_stream(kp + (int64_t)row * D) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int row = r0 + p * kRowsPerPass;
      vr[p] = row < len ? load_stream(vp + (int64_t)row * D) : make_uint4(0, 0, 0, 0);
    }

    // scores in log2 units: x_j = scale * log2(e) * q.k_j
    float x[kPasses];
    float mx = -INFINITY;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int row = r0 + p * kRowsPerPass;
      const float sdot = row_sum<kLanes>(dot8<BF16>(qv, kr[p], 0.f));
      x[p] = row < len ? sdot * scale_log2 : -INFINITY;
      mx = fmaxf(mx, x[p]);
    }
    // chunk max: over the rows of this wave, then over the waves
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = max_xor32(mx);
    if (kLanes <= 8) mx = fmaxf(mx, __shfl_xor(mx, 8));
    if (kLanes == 4) mx = fmaxf(mx, __shfl_xor(mx, 4));
    if (lane == 0) red[0][wave] = mx;
    __syncthreads();
    float m = red[0][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = fmaxf(m, red[0][w]);

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
    // l: the lanes of a row group hold the same e; sum over the row groups of
    // the wave, then across waves.
    l += __shfl_xor(l, 16);
    l = sum_xor32(l);
    if (kLanes <= 8) l += __shfl_xor(l, 8);
    if (kLanes == 4) l += __shfl_xor(l, 4);
    // column partials: reduce the lanes that share a column chunk
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      float a = acc[t];
      if (kLanes == 4) a += __shfl_xor(a, 4);
      if (kLanes <= 8) a += __shfl_xor(a, 8);
      a += __shfl_xor(a, 16);
      a = sum_xor32(a);
      acc[t] = a;
    }
    if (lane < kLanes) {
#pragma unroll
      for (int t = 0; t < 8; ++t) opart[wave][lane * 8 + t] = acc[t];
    }
    if (lane == 0) red[1][wave] = l;
    __syncthreads();
    if (tid < D) {
      float lt = 0.f, ot = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        lt += red[1][w];
        ot += opart[w][tid];
      }
      const int64_t base = (int64_t)bh * C + c;
      __builtin_nontemporal_store(ot / lt, o_part + base * D + tid);
      if (tid == 0) __builtin_nontemporal_store((m + log2f(lt)) * kLn2, lse_part + base);
    }
    __syncthreads();  // opart / red reused by the next item
  }
}

// GQA decode on the matrix cores.  Item = (chunk c of `chunk` keys, a
// multiple of 128, batch b, kv head, slice of G <= 16 query heads of its
// group); the chunk is walked in 128-key sub-chunks with the online-softmax
// rescale between them.  The G heads are the 16 columns of
// v_mfma_f32_16x16x32 (columns >= G carry q = 0 and are never stored):
//   S^T[key][head] = K Q^T   A = K rows, B = Q^T (the q rows of the slice's
//                            heads), both read from LDS
//   O^T[d][head]  = V^T P^T  A = V^T via ds_read_b64_tr_b16 from LDS,
//                            B = P^T from LDS as hi + lo 16-bit parts
// so the chunk's K and V are read from HBM once for all G heads.  Q, K and V
// reach LDS through bounds-checked buffer loads (rows past the end read as
// zeros) that write whole swizzled rows, so every fetch instruction reads
// 1 KB of contiguous HBM; K and V carry the streaming hint.  (K read straight
// into MFMA operand registers would take each 128-byte line in two 64-byte
// halves from separate instructions, which streams markedly slower.)  Wave w
// scores keys 32w .. 32w + 31 and accumulates d rows w*D/4 .. +D/4 - 1 over
// all 128 keys (at d = 32 waves 0 and 1 hold the two 16-row blocks).  The
// chunk max and sum are exchanged through LDS; P is the fp32 2^(x - m) split
// into two 16-bit parts, so the products keep fp32-level accuracy in P while
// l is the sum of the unrounded values.
//   PAGED: K/V rows come from a paged cache (PagedKv); rows past a sequence's
// end read as zeros and chunks past it store O_c = 0, lse_c = -inf.
//   KV8: K/V are FP8 E4M3 codes; k_scale is folded into scale_log2 by the
// host and v_scale multiplies the stored partial.  With PAGED as well, each
// lane looks up its own row's page.
// (m, s, a[4]) merge of two running states, in log2 units: both rescaled to
// the larger reference max.  A state with m = -inf (no chunk yet) is empty.
struct MergeState {
  float m, s, a[4];
};
// Adds one chunk (lse l2 in log2 units, normalised output ov) to a running
// state: both rescaled to the larger reference max.  An empty state (m =
// -inf) or an empty chunk (lse = -inf) has no weight, also when both are
// empty.
__device__ __forceinline__ void merge_chunk(MergeState& st, float l2, const float4& ov) {
  const float mn = fmaxf(st.m, l2);
  const float r = st.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.m - mn);
  const float w = l2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(l2 - mn);
  st.s = fmaf(st.s, r, w);
  st.a[0] = fmaf(st.a[0], r, w * ov.x);
  st.a[1] = fmaf(st.a[1], r, w * ov.y);
  st.a[2] = fmaf(st.a[2], r, w * ov.z);
  st.a[3] = fmaf(st.a[3], r, w * ov.w);
  st.m = mn;
}
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

constexpr int kGqaCols = 16;         // MFMA columns: query heads per item
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// Paged KV cache (device pointers and element strides; K and V share them).
// Page p holds block_size consecutive keys of every KV head: key row r of kv
// head h starts at p*page_stride + r*token_stride + h*head_stride.
// A key's page (key / block_size) uses a multiplier and a shift worked out on
// the host (round-up method of Granlund and Montgomery, exact for keys below
// 2^31): three instructions instead of a division sequence per lane.
struct PagedKv {
  const int32_t* block_table;  // [B, max_blocks]
  const int32_t* seq_lens;     // [B]
  int64_t page_stride, token_stride, head_stride;
  int num_blocks, block_size, max_blocks;
  uint32_t bs_mul, bs_shift;   // key / block_size == (mulhi(key, bs_mul) + key) >> bs_shift
  __device__ int page_of(int key) const {
    return (int)((__umulhi((uint32_t)key, bs_mul) + (uint32_t)key) >> bs_shift);
  }
  __device__ int row_in_page(int key) const { return key - page_of(key) * block_size; }
};

static PagedKv make_paged_kv(const int32_t* block_table, const int32_t* seq_lens, int64_t page_stride,
                             int64_t token_stride, int64_t head_stride, int num_blocks, int block_size,
                             int max_blocks) {
  uint32_t l = 0;
  while ((1u << l) < (uint32_t)block_size) ++l;
  const uint64_t mul = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - (uint32_t)block_size)) / (uint32_t)block_size + 1;
  return PagedKv{block_table, seq_lens, page_stride, token_stride, head_stride, num_blocks, block_size, max_blocks,
                 (uint32_t)mul, l};
}
// Fused decode (split-KV with the merge inside the chunk kernel): an item is
// (row, segment), a row being (batch, kv head, head slice) and a segment a run
// of consecutive 128-key chunks of that row.  Each item leaves its
// normalised partial and its log-sum-exp (log2 units) in seg_o / seg_lse; the
// workgroup that finishes a row's last segment (a per-row counter, reset by
// that workgroup) merges the row's partials into o and lse.  With one segment
// per row the item writes o and lse directly.
struct FusedOut {
  float* seg_o;      // [rows, S, G, D] normalised segment outputs
  float* seg_lse;    // [rows, S, G] segment log-sum-exp, log2 units
  uint32_t* count;   // [rows] segments finished; 0 between calls
  uint16_t* o;       // [B, Hq, D] final output (16-bit)
  float* lse;        // [B, Hq] final log-sum-exp (natural log), or null
  int n_chunks;      // 128-key chunks per row, ceil(M / 128)
};

// Two E4M3 codes (bytes 0, 1 of w, or 2, 3 with HI) to two 16-bit values in
// one instruction.  The scale operand is 1: every E4M3 value (normal,
// subnormal or zero) is exact in fp16 and in bf16, so the result is the exact
// decode; NaN codes give NaN.
template <bool BF16, bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_16(uint32_t w) {
  if constexpr (BF16)
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.f, HI));
  else
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.f, HI));
}

// LDS service model of gfx950 (measured with rocprofv3's SQ_LDS_BANK_CONFLICT
// on single-wave probes): reads serve 256 bytes a cycle over 64 four-byte
// banks, ds_read_b128 in four 16-lane groups (within each 32-lane half, the
// 4-lane quads whose index has even, resp. odd, bit parity), ds_read_b64 and
// ds_read_b64_tr_b16 in the two 32-lane halves; writes serve 128 bytes a cycle
// over 32 banks, ds_write_b128 in groups of 8 consecutive lanes.  A group is
// conflict-free when its lanes touch distinct banks (or the same address).
//
// P^T in LDS: per part (hi, lo) 16 rows (query heads) of 128 16-bit slots,
// 256 bytes per row; 16-byte unit u of row j sits at unit u ^ j.  Slots
// 32w .. 32w + 31 hold wave w's keys, in the order the P.V contraction uses:
// slot 32w + 8 * perm4(g) + 4 kb + r holds key 32w + 16 kb + 4 g + r, so the
// QK lane (j, g) writes its 8 values with one 16-byte store.
constexpr int kPRow = kChunk;  // P row in 16-bit elements
__device__ __forceinline__ int perm4(int g) { return ((g & 1) << 1) | (g >> 1); }  // swaps 1 and 2
// Contraction chunk of QK step s for lane group g (16-byte chunks of d): both
// operands read it, so any bijection is valid; this one makes the K and Q
// reads (16 rows x 4 chunks, rows swizzled by swz<D>) conflict-free under the
// ds_read_b128 lane groups.
template <int D>
__device__ __forceinline__ int qk_chunk(int s, int g) {
  constexpr int kS = D / 32, kX = D == 32 ? 2 : (D == 64 ? 1 : 0);  // d = 128, 256: kX = 0
  return (kS * g + s) ^ ((g & 1) ? kX : 0);
}
constexpr int kMfmaMinItems = 2048;  // MHA chunk items from which the MFMA kernel is used

template <int D, bool BF16, bool PAGED, bool KV8, bool FUSED = false>
__global__ __launch_bounds__(kDecThreads)
void decode_gqa_mfma_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                            const uint16_t* __restrict__ v, float* __restrict__ o_part,
                            float* __restrict__ lse_part, int Hq, int Hkv, int M, int C, int G,
                            int chunk, int n_items, float scale_log2, PagedKv pk, float v_scale, FusedOut fo) {
  static_assert(!KV8 || D <= 128, "FP8 K/V: head dims up to 128");
  constexpr int kS = D / 32;                        // QK contraction steps
  constexpr int kWaves = kDecThreads / 64;
  constexpr int kDB = D / 16 >= kWaves ? D / 16 / kWaves : 1;  // 16-row d blocks per wave
  constexpr int kPVWaves = D / 16 / kDB;            // waves with O^T rows (all but at d = 32)
  constexpr int kU = D / 8;                         // 16-byte units per row
  constexpr int kRowsPerInst = kDecThreads / kU;    // rows per fetch instruction index
  constexpr int kFetch = kChunk / kRowsPerInst;     // fetch instructions per wave
  constexpr uint32_t kPBytes = kGqaCols * kPRow * 2;  // one P part
  // the swizzle repeats every 16 rows: with 8 rows per fetch instruction
  // (d = 256) the odd instructions take the lane offsets of rows 8 .. 15
  static_assert(kRowsPerInst % 16 == 0 || kRowsPerInst == 8, "rows per fetch instruction");
  constexpr bool kOddRows = kRowsPerInst == 8;
  __shared__ __attribute__((aligned(1024))) uint16_t kbuf[kChunk * D];
  __shared__ __attribute__((aligned(1024))) uint16_t vbuf[kChunk * D];
  __shared__ __attribute__((aligned(1024))) uint16_t qbuf[kGqaCols * D];
  __shared__ __attribute__((aligned(16))) uint16_t pbuf[2 * kGqaCols * kPRow];
  __shared__ float red[2][kWaves][kGqaCols];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int group = Hq / Hkv, slices = group / G;
  const uint32_t k_lds = (uint32_t)(uintptr_t)(lds_u16*)kbuf;
  const uint32_t v_lds = (uint32_t)(uintptr_t)(lds_u16*)vbuf;
  const uint32_t q_lds = (uint32_t)(uintptr_t)(lds_u16*)qbuf;
  const uint32_t p_lds = (uint32_t)(uintptr_t)(lds_u16*)pbuf;
  const bool out16 = ((uintptr_t)o_part & 15) == 0;

  // K/V fetch: instruction i of wave w fills LDS units (i*kWaves + w)*64 +
  // lane, i.e. row kRowsPerInst*i + rl, physical 16-byte chunk pc (holding
  // logical chunk pc ^ swz(row)).  The Q fetch (16 rows) takes kQInst
  // instructions the same way: instruction 0 of the first kQInst waves, or
  // (d = 256) instructions 0 and 1 of every wave.
  constexpr int kQInst = kGqaCols * kU / 64;
  const int rl = (wave * 64 + lane) / kU, pc = lane % kU;
  const uint32_t voff_lane = (uint32_t)(rl * D * 2 + ((pc ^ swz<D>(rl)) << 4));
  const uint32_t voff_odd = (uint32_t)(rl * D * 2 + ((pc ^ swz<D>(rl + 8)) << 4));  // rows 8 .. 15 (d = 256)
  auto voff_inst = [&](int i) { return (kOddRows && (i & 1)) ? voff_odd : voff_lane; };
  // paged: a wave's fetch instruction covers kWaveRows consecutive key rows
  // (4, 8 or 16), which never straddle a page (block_size % 16 == 0), so each
  // instruction gets its own page descriptor and the lanes offset into it
  constexpr int kWaveRows = 64 / kU;
  const uint32_t voff_paged =
      PAGED ? (uint32_t)((int64_t)(lane / kU) * pk.token_stride * 2) + (uint32_t)((pc ^ swz<D>(rl)) << 4) : 0u;
  const uint32_t voff_paged_odd =
      PAGED ? (uint32_t)((int64_t)(lane / kU) * pk.token_stride * 2) + (uint32_t)((pc ^ swz<D>(rl + 8)) << 4) : 0u;
  // V^T operand: in each 16-lane group of a ds_read_b64_tr_b16, lane s
  // addresses V[K0 + s/4][D0 + 4*(s%4)], so lane i receives V[K0 + 0..3][D0 + i].
  // Group g fills slots 8g .. 8g + 7 of k-step ks: keys 32 ks + 4 perm4(g) +
  // 16 hh + 0..3 for half hh, the slot order of P^T.
  uint32_t va[kDB][2];
#pragma unroll
  for (int db = 0; db < kDB; ++db) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int row = 4 * perm4(g) + 16 * hh + (j >> 2);
      const int col = 16 * (wave * kDB + db) + 4 * (j & 3);
      va[db][hh] = v_lds + (uint32_t)(row * D * 2 + ((((col >> 3) ^ swz<D>(row)) << 4) | ((col & 7) * 2)));
    }
  }
  // P^T row j: read unit 4 ks + g (slots 32ks + 8g ..), written unit 4 w + perm4(g)
  const uint32_t p_row = p_lds + (uint32_t)(j * kPRow * 2);
  const uint32_t pw = p_row + (uint32_t)(((4 * wave + perm4(g)) ^ j) << 4);

  // paged: the page ids of the next sub-chunk (and, across items, the next
  // sequence length) are loaded right after the current fetches are issued,
  // so their latency hides behind those fetches.  Lane i of one VGPR holds
  // fetch instruction i's page (read out with v_readlane where it is used):
  // kept in SGPRs the ids spilled, and each spill waited for its load at once.
  // Table reads are clamped to the table; entries past a sequence's end are
  // read but never used.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // keeps page descriptors scalar
  int nx_item = -1, nx_key0 = 0, nx_seq = 0;
  // a sequence's length through the scalar cache (the lengths are read-only
  // here): a scalar load is waited for on its own counter, not behind the
  // vector loads and fetches in flight
  auto seq_len = [&](int bb) {
    return ((const __attribute__((address_space(4))) int*)pk.seq_lens)[bb];
  };
  int pgv = 0;  // lane i < kFetch: page id of fetch instruction i (current, then prefetched)
  auto load_pages = [&](int bb, int kk, int& pv) {
    const int i = min(lane, kFetch - 1);
    const int e = min(pk.page_of(kk + kRowsPerInst * i + wave_u * kWaveRows), pk.max_blocks - 1);
    pv = pk.block_table[(int64_t)bb * pk.max_blocks + e];
  };

  // FP8 KV: each thread's 16-byte pieces of a 128-key sub-chunk.  After the
  // current pieces are converted, the next sub-chunk's (or next item's first)
  // are loaded into the same registers, so that load overlaps this sub-chunk's
  // products.  kv8_item / kv8_key0 name what the registers hold (-1: nothing);
  // bit p of kv8_ok says piece p is a row that exists (otherwise it was read
  // from a safe address and is converted as zeros).
  constexpr int kPR8 = D / 16;                       // 16-byte pieces per FP8 row
  constexpr int kPieces8 = kChunk * kPR8 / kDecThreads;
  // Piece u of a sub-chunk is piece u % kPR8 of row piece_row(u): the row
  // index u / kPR8 with bit 2 flipped when bit 2 of u is set.  Each group of 8
  // consecutive lanes (one ds_write_b128 cycle) then writes two rows whose
  // swizzles differ in their low bit, so its 16-byte units land on 8 distinct
  // bank groups; a wave's 64 pieces still cover whole consecutive rows.
  auto piece_row = [](int u) { return (u / kPR8) ^ (((u >> 2) & 1) << 2); };
  uint4 kr8[kPieces8], vr8[kPieces8];
  int kv8_item = -1, kv8_key0 = 0;
  uint32_t kv8_ok = 0;
  // paged FP8: each lane's page id per piece for the fetch after the one in
  // flight (pg_item / pg_key0 name it, -1: none), looked up right after that
  // fetch is issued, so the table's latency overlaps the same products.  The
  // guess ignores the sequence's length; when it turns out wrong the ids are
  // looked up again.  Table reads are clamped to the table.
  int pg8[kPieces8];
  int pg_item = -1, pg_key0 = 0;
  auto lookup8 = [&](int bb, int kk) {
#pragma unroll
    for (int p = 0; p < kPieces8; ++p) {
      const int key = kk + piece_row(p * kDecThreads + tid);
      const int e = min(pk.page_of(key), pk.max_blocks - 1);
      pg8[p] = pk.block_table[(int64_t)bb * pk.max_blocks + e];
    }
  };
  auto fetch8 = [&](int bb, int kvhh, int kk) {
    const uint8_t* k8 = reinterpret_cast<const uint8_t*>(k);
    const uint8_t* v8 = reinterpret_cast<const uint8_t*>(v);
    kv8_ok = 0;
    if constexpr (PAGED) {
      // a row past the sequence's end may read another page's bytes; put()
      // zeroes it.  An out-of-range page id reads offset 0 (page 0 exists).
#pragma unroll
      for (int p = 0; p < kPieces8; ++p) {
        const int u = p * kDecThreads + tid, key = kk + piece_row(u);
        const bool ok = pg8[p] >= 0 && pg8[p] < pk.num_blocks;
        const int64_t off = ok ? (int64_t)pg8[p] * pk.page_stride + (int64_t)kvhh * pk.head_stride +
                                     (int64_t)pk.row_in_page(key) * pk.token_stride + 16 * (u % kPR8)
                               : 0;
        kv8_ok |= (uint32_t)ok << p;
        kr8[p] = load_stream8(k8 + off);
        vr8[p] = load_stream8(v8 + off);
      }
    } else {
      // rows past M read the slice's first row (M >= 1); put() zeroes them
      const int64_t base = ((int64_t)bb * Hkv + kvhh) * M * D;
#pragma unroll
      for (int p = 0; p < kPieces8; ++p) {
        const int u = p * kDecThreads + tid, row = piece_row(u);
        const bool ok = kk + row < M;
        const int64_t off = base + (ok ? (int64_t)(kk + row) * D + 16 * (u % kPR8) : 0);
        kv8_ok |= (uint32_t)ok << p;
        kr8[p] = load_stream8(k8 + off);
        vr8[p] = load_stream8(v8 + off);
      }
    }
  };

  // FP8 KV: Q comes through registers as well, loaded together with the
  // prefetch of its item's first sub-chunk, so its latency is hidden too.
  // Thread tid holds LDS unit tid of the Q block (the layout of the Q fetch
  // below): row tid / kU, logical chunk (tid % kU) ^ swz(row); rows >= G are 0.
  uint4 q8 = make_uint4(0, 0, 0, 0);
  int q8_item = -1;
  auto loadq8 = [&](int bb, int hh0) {
    const int rq = tid / kU, lc = (tid % kU) ^ swz<D>(rq);
    q8 = make_uint4(0, 0, 0, 0);
    if (tid < kGqaCols * kU && rq < G)
      q8 = *reinterpret_cast<const uint4*>(q + ((int64_t)bb * Hq + hh0 + rq) * D + 8 * lc);
  };

  // Fused mode, after item (row, seg): with one segment per row, o and lse
  // directly.  Otherwise the segment's partial goes to seg_o / seg_lse and the
  // row's counter is incremented; the workgroup that brings it to C (the
  // row's last segment) merges the row's partials ("CUDA Flash Decoding",
  // section 2.2 step 2: w_s = exp(lse_s - logsumexp lse), o = sum_s w_s o_s)
  // and resets the counter for the next call.
  //   Visibility across the XCDs (each has its own L2): the partials are
  // written and read with device-scope relaxed atomic stores and loads, which
  // go through to the memory side instead of staying in an XCD's L2, and
  // every thread waits for its stores to complete before the workgroup
  // barrier that precedes the counter increment; the merging workgroup reads
  // only after seeing the count.  A release/acquire fence pair would write
  // back and invalidate the whole L2 in every wave instead (measured: it
  // doubles the kernel's time).
  __shared__ int fused_last;
  auto fused_epilogue = [&](int row, int b, int h0, int seg, float lt, float m_ref, const f32x4 (&acc)[kDB]) {
    // lt == 0: a segment (or row) with no key (past a paged sequence's end):
    // O = 0 and lse = -inf, which the merge gives no weight
    const bool has = !(lt == 0.f);
    const float inv = has ? 1.f / lt : 0.f;
    const float l2 = has ? m_ref + log2f(lt) : -INFINITY;
    if (C == 1) {
      if (j < G) {
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          if (wave >= kPVWaves) break;
          const f32x4 o4 = acc[db] * inv;
          *reinterpret_cast<uint2*>(fo.o + ((int64_t)b * Hq + h0 + j) * D + 16 * (wave * kDB + db) + 4 * g) =
              make_uint2(pack2<BF16>(o4[0], o4[1]), pack2<BF16>(o4[2], o4[3]));
        }
        if (wave == 0 && g == 0 && fo.lse != nullptr) fo.lse[(int64_t)b * Hq + h0 + j] = l2 * kLn2;
      }
      return;
    }
    auto put = [](float* p, float x) { __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
    auto get = [](const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
    if (j < G) {
      const int64_t e = ((int64_t)row * C + seg) * G + j;
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        if (wave >= kPVWaves) break;
        float* op = fo.seg_o + e * D + 16 * (wave * kDB + db) + 4 * g;
#pragma unroll
        for (int r = 0; r < 4; ++r) put(op + r, acc[db][r] * inv);
      }
      if (wave == 0 && g == 0) put(fo.seg_lse + e, l2);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's partial stores have completed
    __syncthreads();
    if (tid == 0)
      fused_last = __hip_atomic_fetch_add(fo.count + row, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   (uint32_t)(C - 1);
    __syncthreads();
    if (!fused_last) return;
    // (head, column quad) pairs, each merged over the row's C segments by SG
    // threads (segments sg, sg + SG, ...); their states meet in LDS (the V
    // buffer, free after the barrier above)
    constexpr int kQuads = D / 4;
    const int pairs = G * kQuads;
    const int SG = pairs >= kDecThreads ? 1 : min(16, kDecThreads / pairs);
    MergeState* sts = reinterpret_cast<MergeState*>(vbuf);
    for (int u = tid; u < pairs * SG; u += kDecThreads) {
      const int p = u % pairs, sg = u / pairs, jj = p / kQuads, quad = p % kQuads;
      MergeState st = {-INFINITY, 0.f, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll 4
      for (int sgm = sg; sgm < C; sgm += SG) {
        const int64_t e = ((int64_t)row * C + sgm) * G + jj;
        const float* op = fo.seg_o + e * D + 4 * quad;
        merge_chunk(st, get(fo.seg_lse + e), make_float4(get(op), get(op + 1), get(op + 2), get(op + 3)));
      }
      sts[u] = st;
    }
    __syncthreads();
    for (int p = tid; p < pairs; p += kDecThreads) {
      MergeState r = sts[p];
      for (int sg = 1; sg < SG; ++sg) r = merge_states(r, sts[sg * pairs + p]);
      const int jj = p / kQuads, quad = p % kQuads;
      const float inv = r.s > 0.f ? 1.f / r.s : 0.f;
      *reinterpret_cast<uint2*>(fo.o + ((int64_t)b * Hq + h0 + jj) * D + 4 * quad) =
          make_uint2(pack2<BF16>(r.a[0] * inv, r.a[1] * inv), pack2<BF16>(r.a[2] * inv, r.a[3] * inv));
      if (quad == 0 && fo.lse != nullptr) fo.lse[(int64_t)b * Hq + h0 + jj] = (r.m + log2f(r.s)) * kLn2;
    }
    if (tid == 0) __hip_atomic_store(fo.count + row, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  // Keys of item n: chunk n % C, or in fused mode segment n % C of the row's
  // 128-key chunks; the end is nominal (not clamped to a sequence's length).
  auto item_key0 = [&](int n) {
    return FUSED ? (int)((int64_t)(n % C) * fo.n_chunks / C) * kChunk : (n % C) * chunk;
  };
  auto item_key_end = [&](int n) {
    return FUSED ? (int)((int64_t)(n % C + 1) * fo.n_chunks / C) * kChunk : (n % C + 1) * chunk;
  };

  // contiguous K/V: the item and first key of the K sub-chunk already
  // fetched ahead (-1: none)
  int pf_item = -1, pf_key0 = -1;
  auto fetch_k = [&](const i32x4& desc, int kk) {
#pragma unroll
    for (int i = 0; i < kFetch; ++i)
      dma16<true>(desc, k_lds + (uint32_t)(i * kWaves + wave) * 1024u,
                  voff_inst(i) + (uint32_t)(kk + kRowsPerInst * i) * (uint32_t)(D * 2));
  };

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int c = item % C;
    const int rest = item / C;
    const int hs = rest % slices, bkv = rest / slices;
    const int kvh = bkv % Hkv, b = bkv / Hkv;
    const int h0 = kvh * group + hs * G;  // first query head of this item
    int seq = M;  // keys of this sequence
    if constexpr (PAGED) {
      seq = nx_item == item ? nx_seq : seq_len(b);
      seq = min(max(seq, 0), pk.max_blocks * pk.block_size);
      if constexpr (FUSED) {
        if (item_key0(item) >= seq) {
          // a segment past the sequence's end still counts towards its row
          f32x4 zero[kDB];
#pragma unroll
          for (int db = 0; db < kDB; ++db) zero[db] = (f32x4){};
          fused_epilogue(rest, b, h0, c, 0.f, -INFINITY, zero);
          __syncthreads();  // the merge states are refilled by the next item
          continue;
        }
      } else if (c * chunk >= seq) {
        // chunk past the sequence's end: O_c = 0, lse_c = -inf (no weight in the merge)
        if (j < G) {
          const int64_t base = ((int64_t)b * Hq + h0 + j) * C + c;
#pragma unroll
          for (int db = 0; db < kDB; ++db) {
            if (wave >= kPVWaves) break;
            float* op = o_part + base * D + 16 * (wave * kDB + db) + 4 * g;
#pragma unroll
            for (int r = 0; r < 4; ++r) __builtin_nontemporal_store(0.f, op + r);
          }
          if (wave == 0 && g == 0) __builtin_nontemporal_store(-INFINITY, lse_part + base);
        }
        continue;  // uniform over the workgroup; no LDS was touched
      }
    }
    // keys of this item: chunk c, or (fused) segment c of the row's chunks
    const int k_begin = item_key0(item);
    const int c_end = min(seq, item_key_end(item));
    const int64_t slice = PAGED ? 0 : ((int64_t)b * Hkv + kvh) * M * D;

    // Q rows h0 .. h0 + 15 (once per item), then per 128-key sub-chunk its K
    // and V -> LDS, no registers; the buffer loads are bounds-checked, so Q
    // rows >= G and K/V rows past M read as zeros.  K and V are streamed
    // (read once).
    const i32x4 qdesc = make_desc(q + ((int64_t)b * Hq + h0) * D, D, G, D);
    const i32x4 kdesc = make_desc(k + slice, D, M, D);
    const i32x4 vdesc = make_desc(v + slice, D, M, D);
    if constexpr (KV8) {
      if (q8_item != item) loadq8(b, h0);  // written to LDS after the first sub-chunk's conversion
    } else if constexpr (kQInst > kWaves) {
#pragma unroll
      for (int i = 0; i < kQInst / kWaves; ++i)
        dma16(qdesc, q_lds + (uint32_t)(i * kWaves + wave) * 1024u,
              voff_inst(i) + (uint32_t)(kRowsPerInst * i) * (uint32_t)(D * 2));
    } else if (wave < kQInst) {
      dma16(qdesc, q_lds + (uint32_t)wave * 1024u, voff_lane);
    }

    // running state of head j across the sub-chunks: the reference max (log2
    // units, shared by all waves), this wave's sum and its O^T rows
    float m_run = -INFINITY, l_w = 0.f;
    f32x4 oacc[kDB];
#pragma unroll
    for (int db = 0; db < kDB; ++db) oacc[db] = (f32x4){};
    for (int key0 = k_begin; key0 < c_end; key0 += kChunk) {
      const int len = min(kChunk, c_end - key0);
      const bool last = key0 + kChunk >= c_end;
      if constexpr (KV8) {
        // FP8 KV: 16-byte pieces of E4M3 rows (consecutive threads read
        // consecutive pieces), converted exactly to 16 bits in registers and
        // written to the same swizzled layout; rows past M read as zeros
        if (kv8_item != item || kv8_key0 != key0) {  // nothing in flight for this sub-chunk
          if constexpr (PAGED) lookup8(b, key0);
          fetch8(b, kvh, key0);
        }
        const uint32_t ok8 = kv8_ok;
        // the next fetch: this item's next sub-chunk, or the next item's first
        int nt_item = -1, nt_key0 = 0, nt_b = b, nt_kvh = kvh;
        if (key0 + kChunk < c_end) {
          nt_item = item;
          nt_key0 = key0 + kChunk;
        } else if (item + (int)gridDim.x < n_items) {
          nt_item = item + (int)gridDim.x;
          const int bkv_n = nt_item / C / slices;
          nt_key0 = item_key0(nt_item);
          nt_b = bkv_n / Hkv;
          nt_kvh = bkv_n % Hkv;
        }
        if constexpr (PAGED) {
          if (nt_item >= 0 && nt_item != item) {
            nx_item = nt_item;
            nx_seq = seq_len(nt_b);
          }
        }
        // u: the piece's index in the sub-chunk
        auto put = [&](uint32_t base, const uint4& w, int u) {
          const int row = piece_row(u), pc8 = u % kPR8;
          const uint32_t* b4 = reinterpret_cast<const uint32_t*>(&w);
          uint32_t h[8];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            h[2 * t] = e4m3x2_to_16<BF16, false>(b4[t]);
            h[2 * t + 1] = e4m3x2_to_16<BF16, true>(b4[t]);
          }
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int lc = 2 * pc8 + half;
            *(lds_u32x4*)(uintptr_t)(base + (uint32_t)(row * D * 2 + ((lc ^ swz<D>(row)) << 4))) =
                (u32x4){h[4 * half], h[4 * half + 1], h[4 * half + 2], h[4 * half + 3]};
          }
        };
        const uint4 zero4 = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int p = 0; p < kPieces8; ++p) {
          const int u = p * kDecThreads + tid;
          // a row that does not exist, or lies past the sequence's end
          const bool bad = !((ok8 >> p) & 1u) || (PAGED && key0 + piece_row(u) >= seq);
          put(k_lds, bad ? zero4 : kr8[p], u);
          put(v_lds, bad ? zero4 : vr8[p], u);
        }
        if (key0 == k_begin && tid < kGqaCols * kU)  // Q, before q8 is reloaded below
          *(lds_u32x4*)(uintptr_t)(q_lds + (uint32_t)tid * 16u) = (u32x4){q8.x, q8.y, q8.z, q8.w};
        // prefetch the next sub-chunk, or the next item's first one
        kv8_item = nt_item;
        kv8_key0 = nt_key0;
        if (nt_item >= 0) {
          if constexpr (PAGED) {
            if (pg_item != nt_item || pg_key0 != nt_key0) lookup8(nt_b, nt_key0);
          }
          if (nt_item != item) {
            q8_item = nt_item;
            loadq8(nt_b, nt_kvh * group + (nt_item / C) % slices * G);
          }
          fetch8(nt_b, nt_kvh, nt_key0);
          if constexpr (PAGED) {
            // guess the fetch after it and look up its pages now
            pg_item = -1;
            if (nt_key0 + kChunk < item_key_end(nt_item)) {
              pg_item = nt_item;
              pg_key0 = nt_key0 + kChunk;
              lookup8(nt_b, pg_key0);
            } else if (nt_item + (int)gridDim.x < n_items) {
              pg_item = nt_item + (int)gridDim.x;
              pg_key0 = item_key0(pg_item);
              lookup8(pg_item / C / slices / Hkv, pg_key0);
            }
          }
        }
      } else if constexpr (PAGED) {
        // this wave's rows of instruction i: rg .. rg + kWaveRows - 1, of which
        // nv exist; page ids outside [0, num_blocks) read as no rows
        if (nx_item != item || nx_key0 != key0) load_pages(b, key0, pgv);
#pragma unroll
        for (int i = 0; i < kFetch; ++i) {
          const int rg = key0 + kRowsPerInst * i + wave_u * kWaveRows;
          int nv = min(kWaveRows, seq - rg);
          int page = __builtin_amdgcn_readlane(pgv, i);
          if (page < 0 || page >= pk.num_blocks) nv = 0;
          if (nv <= 0) page = 0;
          const int64_t off = (int64_t)page * pk.page_stride + (int64_t)kvh * pk.head_stride +
                              (int64_t)pk.row_in_page(rg) * pk.token_stride;
          const uint32_t vo = (kOddRows && (i & 1)) ? voff_paged_odd : voff_paged;
          dma16<true>(make_desc_rows(k + off, pk.token_stride, max(nv, 0), D),
                      k_lds + (uint32_t)(i * kWaves + wave) * 1024u, vo);
          dma16<true>(make_desc_rows(v + off, pk.token_stride, max(nv, 0), D),
                      v_lds + (uint32_t)(i * kWaves + wave) * 1024u, vo);
        }
        // prefetch the next sub-chunk's page ids (the next item's, with its length)
        if (key0 + kChunk < c_end) {
          nx_item = item;
          nx_key0 = key0 + kChunk;
          nx_seq = seq;
          load_pages(b, nx_key0, pgv);
        } else {
          const int n = item + (int)gridDim.x;
          nx_item = -1;
          if (n < n_items) {
            const int bn = n / C / slices / Hkv;
            nx_item = n;
            nx_key0 = item_key0(n);
            nx_seq = seq_len(bn);
            load_pages(bn, nx_key0, pgv);
          }
        }
      } else {
        if (pf_item != item || pf_key0 != key0) fetch_k(kdesc, key0);
#pragma unroll
        for (int i = 0; i < kFetch; ++i)
          dma16<true>(vdesc, v_lds + (uint32_t)(i * kWaves + wave) * 1024u,
                      voff_inst(i) + (uint32_t)(key0 + kRowsPerInst * i) * (uint32_t)(D * 2));
      }
      // paged: K and V of one instruction are issued together (each descriptor
      // lives briefly, and this measured faster than K first), so wait for both
      if constexpr (KV8) {
        // nothing is fetched straight to LDS: the threads wrote Q, K and V
      } else if constexpr (PAGED) wait_tile_loads();
      else wait_vm<kFetch>();  // this wave's Q and K fetches have landed (V may not)
      __syncthreads();    // Q and K visible

      // A operand of S^T: K row 32w + 16kb + j, d chunk qk_chunk(s, g); B
      // operand: q of head h0 + j, same d.  The row's swizzle is swz(j) (rows
      // of a 16-row block share their low four bits with j).
      s16x8 ka[2][kS], qb[kS];
#pragma unroll
      for (int s = 0; s < kS; ++s) {
        const uint32_t cx = (uint32_t)((qk_chunk<D>(s, g) ^ swz<D>(j)) << 4);
        qb[s] = lds_read_b128(q_lds + (uint32_t)(j * D * 2) + cx);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          ka[kb][s] = lds_read_b128(k_lds + (uint32_t)((32 * wave + 16 * kb + j) * D * 2) + cx);
      }

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
      if constexpr (!KV8) wait_tile_loads();  // this wave's part of the V sub-chunk is in LDS
      __syncthreads();    // V sub-chunk and the per-wave maxima visible
      if constexpr (!PAGED && !KV8) {
        // Every wave is done reading K: fetch the item's next sub-chunk of K
        // now, so that the fetch overlaps this sub-chunk's softmax and P.V
        // instead of following them.  (Fetching the next item's Q and first
        // K here as well made the 128-key chunk kernel slower: 92.4 against
        // 89-90 us on the long decode workload.)
        if (!last) {
          pf_item = item;
          pf_key0 = key0 + kChunk;
          fetch_k(kdesc, pf_key0);
        }
      }
      float m = m_run;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) m = fmaxf(m, red[0][w][j]);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m);  // 0 on the first sub-chunk
      m_run = m;

      float lsum = 0.f;
      uint32_t pwh[4], pwl[4];  // this lane's 8 P slots, hi and lo parts
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
        pwh[2 * kb] = h01;
        pwh[2 * kb + 1] = h23;
        pwl[2 * kb] = pack2<BF16>(p[0] - r01[0], p[1] - r01[1]);
        pwl[2 * kb + 1] = pack2<BF16>(p[2] - r23[0], p[3] - r23[1]);
      }
      *(lds_u32x4*)(uintptr_t)pw = (u32x4){pwh[0], pwh[1], pwh[2], pwh[3]};
      *(lds_u32x4*)(uintptr_t)(pw + kPBytes) = (u32x4){pwl[0], pwl[1], pwl[2], pwl[3]};
      lsum += __shfl_xor(lsum, 16);
      lsum = sum_xor32(lsum);
      l_w = fmaf(l_w, alpha, lsum);
      if (last && g == 0) red[1][wave][j] = l_w;
      __syncthreads();  // P (and, after the last sub-chunk, the per-wave sums) visible

#pragma unroll
      for (int db = 0; db < kDB; ++db) oacc[db] *= alpha;
#pragma unroll
      for (int ks = 0; ks < kChunk / 32; ++ks) {
        if (wave >= kPVWaves) break;
        const uint32_t pr = p_row + (uint32_t)(((4 * ks + g) ^ j) << 4);
        const s16x8 ph = lds_read_b128(pr);
        const s16x8 pl = lds_read_b128(pr + kPBytes);
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const s16x4 lo = lds_read_tr16_b64(va[db][0] + (uint32_t)(32 * ks * D * 2));
          const s16x4 hi = lds_read_tr16_b64(va[db][1] + (uint32_t)(32 * ks * D * 2));
          const s16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[db] = mfma16x16x32<BF16>(a, ph, oacc[db]);
          oacc[db] = mfma16x16x32<BF16>(a, pl, oacc[db]);
        }
      }
      if (!last) __syncthreads();  // K, V, P and the maxima are refilled by the next sub-chunk
    }
    float lt = red[1][0][j];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) lt += red[1][w][j];
    if constexpr (FUSED) {
      if constexpr (KV8) {
#pragma unroll
        for (int db = 0; db < kDB; ++db) oacc[db] *= v_scale;  // V = v_scale * e4m3(v)
      }
      fused_epilogue(rest, b, h0, c, lt, m_run, oacc);
      __syncthreads();  // Q, K, V, P, the sums and the merge states are refilled by the next item
      continue;
    }
    if (j < G) {
      const int64_t base = ((int64_t)b * Hq + h0 + j) * C + c;
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        if (wave >= kPVWaves) break;
        float* op = o_part + base * D + 16 * (wave * kDB + db) + 4 * g;
        f32x4 o4 = oacc[db] / lt;
        if constexpr (KV8) o4 *= v_scale;  // V = v_scale * e4m3(v)
        if (out16) {
          __builtin_nontemporal_store(o4, reinterpret_cast<f32x4*>(op));
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) __builtin_nontemporal_store(o4[r], op + r);
        }
      }
      if (wave == 0 && g == 0) __builtin_nontemporal_store((m_run + log2f(lt)) * kLn2, lse_part + base);
    }
    __syncthreads();  // Q, K, V, P and the sums are refilled by the next item
  }
}

constexpr int kMergeThreads = 256;

// One pass over the partials.  A workgroup covers one (batch, head) and QW
// column quads (4*QW columns); thread t takes quad t % QW and chunk group
// t / QW, walking chunks grp, grp + G, ... (G = 256 / QW groups) with a running
// max of lse_c (log2 units), the matching rescaled weight sum and the weighted
// output.  Lanes of one wave that share a quad read consecutive chunks' pieces
// of 16*QW contiguous bytes.  The G group states are combined with the same
// rule, first across the lanes of each wave (xor shuffles over the group bits
// of the lane id), then across the 4 waves.  O = sum_c 2^(l_c - M) O_c /
// sum_c 2^(l_c - M) for any reference M equals sum_c w_c O_c.
template <int D, bool BF16, int QW>
__global__ __launch_bounds__(kMergeThreads)
void lse_merge_kernel(const float* __restrict__ o_part, const float* __restrict__ lse_part,
                      uint16_t* __restrict__ o, float* __restrict__ lse, int C) {
  constexpr int kWaves = kMergeThreads / 64;
  constexpr int kGroups = kMergeThreads / QW;
  static_assert(QW >= 1 && QW <= 32 && 4 * QW <= D, "column quads per workgroup");
  __shared__ MergeState part[kWaves][QW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cq = tid % QW, grp = tid / QW;
  const int bh = blockIdx.x;
  const int col0 = blockIdx.y * (4 * QW) + cq * 4;
  const float* lp = lse_part + (int64_t)bh * C;
  const float* op = o_part + (int64_t)bh * C * D + col0;

  MergeState st = {-INFINITY, 0.f, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll 8
  for (int c = grp; c < C; c += kGroups) {
    merge_chunk(st, lp[c] * kLog2e, *reinterpret_cast<const float4*>(op + (int64_t)c * D));
  }
  // lanes that share cq differ in the lane bits from log2(QW) up
#pragma unroll
  for (int mask = QW; mask < 64; mask <<= 1) {
    MergeState y;
    y.m = __shfl_xor(st.m, mask);
    y.s = __shfl_xor(st.s, mask);
#pragma unroll
    for (int c = 0; c < 4; ++c) y.a[c] = __shfl_xor(st.a[c], mask);
    st = merge_states(st, y);
  }
  if (lane < QW) part[wave][lane] = st;
  __syncthreads();
  if (tid < QW) {
    MergeState r = part[0][tid];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) r = merge_states(r, part[w][tid]);
    // a row whose chunks are all empty (an empty sequence) has no weight:
    // O = 0 and lse = -inf
    const float inv = r.s > 0.f ? 1.f / r.s : 0.f;
    const int d0 = blockIdx.y * (4 * QW) + tid * 4;
    const uint32_t w01 = pack2<BF16>(r.a[0] * inv, r.a[1] * inv);
    const uint32_t w23 = pack2<BF16>(r.a[2] * inv, r.a[3] * inv);
    *reinterpret_cast<uint2*>(o + (int64_t)bh * D + d0) = make_uint2(w01, w23);
    if (blockIdx.y == 0 && tid == 0 && lse != nullptr) lse[bh] = (r.m + log2f(r.s)) * kLn2;
  }
}

// Resident workgroups per CU for a kernel, times the CU count (cached per
// kernel and device: the template parameter gives every kernel its own cache).
template <auto Kernel>
static int resident_grid(int threads) {
  constexpr int kMaxDev = 64;
  static int cache[kMaxDev] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < kMaxDev && cache[dev] > 0) return cache[dev];
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, Kernel, threads, 0) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  const int g = cus * per_cu;
  if (dev < kMaxDev) cache[dev] = g;
  return g;
}

hipError_t decode_dispatch(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                           int B, int Hq, int Hkv, int M, int d, int chunk, bool bf16, float scale,
                           hipStream_t stream) {
  const int C = (M + chunk - 1) / chunk;
  const float sl2 = scale * kLog2e;
  const int group = Hq / Hkv;
  // GQA groups and chunks longer than 128 keys run on the matrix-core kernel
  // (K/V read once per kv head), and so do large MHA launches; a small MHA
  // launch (a few rounds of items) finishes sooner on the VALU kernel's
  // shorter per-item path.
  if (group >= 2 || chunk != kChunk || (int64_t)B * Hq * C >= kMfmaMinItems || d == 256) {
    // query heads per item: the largest divisor of the group that fits the
    // 16 MFMA columns
    int g = std::min(group, kGqaCols);
    while (group % g != 0) --g;
    const int n_items = B * (Hq / g) * C;
#define ATTN_GQA_CASE(DD, BB)                                                                          \
    if (d == DD && bf16 == BB) {                                                                       \
      const int grid = std::min(n_items, resident_grid<decode_gqa_mfma_kernel<DD, BB, false, false>>(kDecThreads)); \
      return launch(&decode_gqa_mfma_kernel<DD, BB, false, false>, dim3(grid), dim3(kDecThreads), stream,  \
                         (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, o_part, lse_part,      \
                         Hq, Hkv, M, C, g, chunk, n_items, sl2, PagedKv{}, 1.f, FusedOut{});                                                                        \
    }
    ATTN_GQA_CASE(32, false) ATTN_GQA_CASE(32, true)
    ATTN_GQA_CASE(64, false) ATTN_GQA_CASE(64, true) ATTN_GQA_CASE(128, false) ATTN_GQA_CASE(128, true)
    ATTN_GQA_CASE(256, false) ATTN_GQA_CASE(256, true)
#undef ATTN_GQA_CASE
    return hipErrorInvalidValue;
  }
  const int n_items = B * Hq * C;
#define ATTN_DEC_CASE(DD, BB)                                                                          \
  if (d == DD && bf16 == BB) {                                                                         \
    const int grid = std::min(n_items, resident_grid<decode_chunk_kernel<DD, BB>>(kDecThreads));    \
    return launch(&decode_chunk_kernel<DD, BB>, dim3(grid), dim3(kDecThreads), stream,     \
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, o_part, lse_part,   \
                       Hq, Hkv, M, C, n_items, sl2);                                                                          \
  }
  ATTN_DEC_CASE(32, false) ATTN_DEC_CASE(32, true)
  ATTN_DEC_CASE(64, false) ATTN_DEC_CASE(64, true) ATTN_DEC_CASE(128, false) ATTN_DEC_CASE(128, true)
#undef ATTN_DEC_CASE
  return hipErrorInvalidValue;
}

// ---- fused decode: plan, workspace layout and launch ----

constexpr int kFusedGridCap = 2048;  // most resident workgroups a plan assumes

static int heads_per_item(int group) {
  // the largest divisor of the group that fits the 16 MFMA columns
  int g = std::min(group, kGqaCols);
  while (group % g != 0) --g;
  return g;
}

// Workspace of a fused decode with S segments per row: the per-row counters,
// then seg_lse, then seg_o, each section starting at a multiple of 256 bytes.
size_t fused_workspace_layout(int B, int Hq, int Hkv, int d, int S, size_t* off_lse, size_t* off_o) {
  const int G = heads_per_item(Hq / Hkv);
  const size_t rows = (size_t)B * (size_t)(Hq / G);
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t cnt = up(rows * 4);
  const size_t lse_bytes = up(rows * (size_t)S * G * 4);
  if (off_lse) *off_lse = cnt;
  if (off_o) *off_o = cnt + lse_bytes;
  return cnt + lse_bytes + rows * (size_t)S * G * (size_t)d * 4;
}

// Largest segment count any launch may choose for these sizes (twice the
// rows' share of the largest grid assumed, at most one segment per chunk):
// the workspace is sized for it.
int fused_segment_cap(int B, int Hq, int Hkv, int M) {
  const int64_t rows = (int64_t)B * (Hq / heads_per_item(Hq / Hkv));
  const int64_t chunks = ((int64_t)M + kChunk - 1) / kChunk;
  return (int)std::min<int64_t>(chunks, 2 * ((kFusedGridCap + rows - 1) / rows));
}

// Segments per row: the S in [1, cap] that minimises the rounds of the
// resident grid times the chunks of the longest segment (the smallest S on
// a tie, so fewer partials to merge).
static int fused_segments(int64_t rows, int64_t chunks, int64_t grid, int cap) {
  int best = 1;
  int64_t best_cost = ((rows + grid - 1) / grid) * chunks;
  for (int S = 2; S <= cap; ++S) {
    const int64_t cost = ((rows * S + grid - 1) / grid) * ((chunks + S - 1) / S);
    if (cost < best_cost) {
      best_cost = cost;
      best = S;
    }
  }
  return best;
}

// One fused launch: S segments per row chosen for the resident grid, the
// workspace laid out for that S (the caller's buffer holds the largest S any
// launch may pick).  scale_log2 carries k_scale and v_scale multiplies O for
// FP8 K/V.
template <int D, bool BF16, bool PAGED, bool KV8>
hipError_t launch_fused(const void* q, const void* k, const void* v, void* o, float* lse, void* ws, size_t ws_bytes,
                        int B, int Hq, int Hkv, int M, float scale_log2, float v_scale, const PagedKv& pk,
                        hipStream_t stream) {
  auto* kern = &decode_gqa_mfma_kernel<D, BF16, PAGED, KV8, true>;
  const int G = heads_per_item(Hq / Hkv);
  const int64_t rows = (int64_t)B * (Hq / G);
  const int chunks = (M + kChunk - 1) / kChunk;
  const int resident = resident_grid<decode_gqa_mfma_kernel<D, BF16, PAGED, KV8, true>>(kDecThreads);
  const int S = fused_segments(rows, chunks, std::min(resident, kFusedGridCap), fused_segment_cap(B, Hq, Hkv, M));
  size_t off_lse = 0, off_o = 0;
  if (fused_workspace_layout(B, Hq, Hkv, D, S, &off_lse, &off_o) > ws_bytes) return hipErrorInvalidValue;
  char* base = static_cast<char*>(ws);
  const FusedOut fo{reinterpret_cast<float*>(base + off_o), reinterpret_cast<float*>(base + off_lse),
                    reinterpret_cast<uint32_t*>(base), static_cast<uint16_t*>(o), lse, chunks};
  const int n_items = (int)(rows * S);
  return launch(kern, dim3(std::min(n_items, resident)), dim3(kDecThreads), stream, q, k, v, (float*)nullptr,
                (float*)nullptr, Hq, Hkv, M, S, G, kChunk, n_items, scale_log2, pk, v_scale, fo);
}

hipError_t decode_fused_dispatch(const void* q, const void* k, const void* v, void* o, float* lse, void* ws,
                                 size_t ws_bytes, int B, int Hq, int Hkv, int M, int d, bool bf16, float scale,
                                 hipStream_t stream) {
  const float sl2 = scale * kLog2e;
#define ATTN_FUSED_CASE(DD, BB) \
  if (d == DD && bf16 == BB)    \
    return launch_fused<DD, BB, false, false>(q, k, v, o, lse, ws, ws_bytes, B, Hq, Hkv, M, sl2, 1.f, PagedKv{}, stream);
  ATTN_FUSED_CASE(32, false) ATTN_FUSED_CASE(32, true) ATTN_FUSED_CASE(64, false)
  ATTN_FUSED_CASE(64, true) ATTN_FUSED_CASE(128, false) ATTN_FUSED_CASE(128, true)
  ATTN_FUSED_CASE(256, false) ATTN_FUSED_CASE(256, true)
#undef ATTN_FUSED_CASE
  return hipErrorInvalidValue;
}

// The fused decode with K and V as FP8 E4M3 codes (K = k_scale e4m3(k),
// V = v_scale e4m3(v)).
hipError_t decode_fp8kv_fused_dispatch(const void* q, const void* k, const void* v, float k_scale, float v_scale,
                                       void* o, float* lse, void* ws, size_t ws_bytes, int B, int Hq, int Hkv, int M,
                                       int d, bool bf16, float scale, hipStream_t stream) {
  const float sl2 = scale * k_scale * kLog2e;
#define ATTN_FUSED8_CASE(DD, BB) \
  if (d == DD && bf16 == BB)     \
    return launch_fused<DD, BB, false, true>(q, k, v, o, lse, ws, ws_bytes, B, Hq, Hkv, M, sl2, v_scale, PagedKv{}, stream);
  ATTN_FUSED8_CASE(32, false) ATTN_FUSED8_CASE(32, true) ATTN_FUSED8_CASE(64, false)
  ATTN_FUSED8_CASE(64, true) ATTN_FUSED8_CASE(128, false) ATTN_FUSED8_CASE(128, true)
#undef ATTN_FUSED8_CASE
  return hipErrorInvalidValue;
}

// Fused decode over a paged cache (16-bit, or FP8 codes with their scales):
// rows of the longest sequence the table can describe (max_blocks *
// block_size keys) split into segments as in the contiguous case; segments
// past a row's sequence end count as empty.
hipError_t decode_paged_fused_dispatch(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_table, const int32_t* seq_lens, int num_blocks,
                                       int block_size, int max_blocks, int64_t page_stride, int64_t token_stride,
                                       int64_t head_stride, void* o, float* lse, void* ws, size_t ws_bytes, int B,
                                       int Hq, int Hkv, int d, bool bf16, float scale, bool fp8, float k_scale,
                                       float v_scale, hipStream_t stream) {
  const int M = max_blocks * block_size;
  const float sl2 = scale * (fp8 ? k_scale : 1.f) * kLog2e;  // FP8: the scores carry k_scale
  const PagedKv pk = make_paged_kv(block_table, seq_lens, page_stride, token_stride, head_stride, num_blocks,
                                   block_size, max_blocks);
#define ATTN_PFUSED_CASE(DD, BB, F8) \
  if (d == DD && bf16 == BB && fp8 == F8) \
    return launch_fused<DD, BB, true, F8>(q, k_cache, v_cache, o, lse, ws, ws_bytes, B, Hq, Hkv, M, sl2, \
                                          F8 ? v_scale : 1.f, pk, stream);
  ATTN_PFUSED_CASE(32, false, false) ATTN_PFUSED_CASE(32, true, false) ATTN_PFUSED_CASE(64, false, false)
  ATTN_PFUSED_CASE(64, true, false) ATTN_PFUSED_CASE(128, false, false) ATTN_PFUSED_CASE(128, true, false)
  ATTN_PFUSED_CASE(256, false, false) ATTN_PFUSED_CASE(256, true, false)
  ATTN_PFUSED_CASE(32, false, true) ATTN_PFUSED_CASE(32, true, true) ATTN_PFUSED_CASE(64, false, true)
  ATTN_PFUSED_CASE(64, true, true) ATTN_PFUSED_CASE(128, false, true) ATTN_PFUSED_CASE(128, true, true)
#undef ATTN_PFUSED_CASE
  return hipErrorInvalidValue;
}

// ---- fused decode without allocation: the library's static scratch ----
//
// For callers that cannot allocate (code under graph capture, tight serving
// loops): the workspace of attn_decode_fused_noalloc is this array.  Each
// GPU the library runs on holds its own copy until the process ends.  Its
// row counters start at zero (the array is zero-initialised when the code
// object is loaded) and every completed call sets them back to zero; the
// partials are written before they are read in every call.  Calls that
// overlap on one GPU share the array and race.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

size_t scratch_capacity() { return kScratchBytes; }

// Device address of the current device's copy of the scratch array, looked
// up once per device (with that device current) and kept; nullptr if the
// lookup fails.  Host code passes this address, never the array's name.
void* scratch_address() {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void* addr[kMaxDev] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

hipError_t decode_paged_dispatch(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, const int32_t* seq_lens, int num_blocks,
                                 int block_size, int max_blocks, int64_t page_stride, int64_t token_stride,
                                 int64_t head_stride, float* o_part, float* lse_part, int B, int Hq, int Hkv,
                                 int d, int chunk, bool bf16, float scale, bool fp8, float k_scale,
                                 float v_scale, hipStream_t stream) {
  const int M = max_blocks * block_size;  // longest sequence the table can describe
  const int C = (M + chunk - 1) / chunk;
  const float sl2 = scale * (fp8 ? k_scale : 1.f) * kLog2e;  // FP8: the scores carry k_scale
  const int group = Hq / Hkv;
  int g = std::min(group, kGqaCols);
  while (group % g != 0) --g;
  const int n_items = B * (Hq / g) * C;
  const PagedKv pk = make_paged_kv(block_table, seq_lens, page_stride, token_stride, head_stride, num_blocks,
                                   block_size, max_blocks);
#define ATTN_PAGED_CASE(DD, BB, F8)                                                                    \
  if (d == DD && bf16 == BB && fp8 == F8) {                                                            \
    const int grid = std::min(n_items, resident_grid<decode_gqa_mfma_kernel<DD, BB, true, F8>>(kDecThreads)); \
    return launch(&decode_gqa_mfma_kernel<DD, BB, true, F8>, dim3(grid), dim3(kDecThreads), stream,  \
                       (const uint16_t*)q, (const uint16_t*)k_cache, (const uint16_t*)v_cache, o_part,     \
                       lse_part, Hq, Hkv, M, C, g, chunk, n_items, sl2, pk, F8 ? v_scale : 1.f, FusedOut{});                                                                          \
  }
  ATTN_PAGED_CASE(32, false, false) ATTN_PAGED_CASE(32, true, false) ATTN_PAGED_CASE(64, false, false)
  ATTN_PAGED_CASE(64, true, false) ATTN_PAGED_CASE(128, false, false) ATTN_PAGED_CASE(128, true, false)
  ATTN_PAGED_CASE(256, false, false) ATTN_PAGED_CASE(256, true, false)
  ATTN_PAGED_CASE(32, false, true) ATTN_PAGED_CASE(32, true, true) ATTN_PAGED_CASE(64, false, true)
  ATTN_PAGED_CASE(64, true, true) ATTN_PAGED_CASE(128, false, true) ATTN_PAGED_CASE(128, true, true)
#undef ATTN_PAGED_CASE
  return hipErrorInvalidValue;
}

hipError_t decode_fp8kv_dispatch(const void* q, const void* k, const void* v, float k_scale, float v_scale,
                                 float* o_part, float* lse_part, int B, int Hq, int Hkv, int M, int d, int chunk,
                                 bool bf16, float scale, hipStream_t stream) {
  const int C = (M + chunk - 1) / chunk;
  const float sl2 = scale * k_scale * kLog2e;  // K = k_scale * e4m3(k): the scores carry k_scale
  const int group = Hq / Hkv;
  int g = std::min(group, kGqaCols);
  while (group % g != 0) --g;
  const int n_items = B * (Hq / g) * C;
#define ATTN_FP8_CASE(DD, BB)                                                                          \
  if (d == DD && bf16 == BB) {                                                                         \
    const int grid = std::min(n_items, resident_grid<decode_gqa_mfma_kernel<DD, BB, false, true>>(kDecThreads)); \
    return launch(&decode_gqa_mfma_kernel<DD, BB, false, true>, dim3(grid), dim3(kDecThreads), stream, \
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, o_part, lse_part, Hq, Hkv,   \
                       M, C, g, chunk, n_items, sl2, PagedKv{}, v_scale, FusedOut{});                                                                          \
  }
  ATTN_FP8_CASE(32, false) ATTN_FP8_CASE(32, true) ATTN_FP8_CASE(64, false) ATTN_FP8_CASE(64, true)
  ATTN_FP8_CASE(128, false) ATTN_FP8_CASE(128, true)
#undef ATTN_FP8_CASE
  return hipErrorInvalidValue;
}

hipError_t merge_dispatch(const float* o_part, const float* lse_part, void* o, float* lse, int B, int Hq,
                          int C, int d, bool bf16, hipStream_t stream) {
  // Column quads per workgroup: the widest (longest contiguous reads, fewest
  // chunk groups to combine) that still gives at least kMergeMinGroups
  // workgroups, and at least 4 quads.
  constexpr int64_t kMergeMinGroups = 512;
  int qw = 32;
  while (qw > 4 && (qw * 4 > d || (int64_t)B * Hq * (d / (4 * qw)) < kMergeMinGroups)) qw >>= 1;
  const dim3 grid(B * Hq, d / (4 * qw));
#define ATTN_MERGE_CASE(DD, BB, QQ)                                                                  \
  if (d == DD && bf16 == BB && qw == QQ) {                                                           \
    return launch(&lse_merge_kernel<DD, BB, QQ>, grid, dim3(kMergeThreads), stream, o_part, \
                       lse_part, (uint16_t*)o, lse, C);                                                                        \
  }
#define ATTN_MERGE_QW(DD, BB) ATTN_MERGE_CASE(DD, BB, 4) ATTN_MERGE_CASE(DD, BB, 8) ATTN_MERGE_CASE(DD, BB, 16)
  ATTN_MERGE_CASE(32, false, 4) ATTN_MERGE_CASE(32, false, 8)
  ATTN_MERGE_CASE(32, true, 4) ATTN_MERGE_CASE(32, true, 8)
  ATTN_MERGE_QW(64, false)
  ATTN_MERGE_QW(64, true)
  ATTN_MERGE_QW(128, false)
  ATTN_MERGE_QW(128, true)
  ATTN_MERGE_CASE(128, false, 32)
  ATTN_MERGE_CASE(128, true, 32)
  ATTN_MERGE_QW(256, false) ATTN_MERGE_CASE(256, false, 32)
  ATTN_MERGE_QW(256, true) ATTN_MERGE_CASE(256, true, 32)
#undef ATTN_MERGE_QW
#undef ATTN_MERGE_CASE
  return hipErrorInvalidValue;
}

}  // namespace attn
