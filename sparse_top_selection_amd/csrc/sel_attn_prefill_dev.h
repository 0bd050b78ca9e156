#pragma once

// Device code of the attention over each group's selection union (INT8 paged
// K/V, FP16 MFMA, FP32 online softmax with a per-position chooser mask), shared
// by the kernels of sel_attn_prefill.hip (one work-group per (group, KV head))
// and sel_attn_prefill_split.hip (shares of a union, then a merge).
//
// Page: #2808 "sycl: prompt attention over 8-query selection unions on XMX".
//   section Summary: chunks of the union are dequantised once to FP16 (the
//     page's chunks hold 64 cells, these 32);
//     S^T = K Q^T and O += P V run on matrix units with FP32 sums for all 96 rows
//     (8 positions x 12 heads); a cell that a position did not select takes no
//     part in that position's softmax (its logit counts as -inf); both products
//     take their operands (Q, K, V, P) in FP16.
//   section What changed: one work-group per 8 positions and KV head.
//   section Extra Notes: cells of non-resident pages are masked (here the union
//     carries each cell's pool row, resolved through the page table once per
//     cell when the union is built, instead of once per KV head here).
//
// gfx950 mapping (the page's 16-lane sub-group / 256-GRF shape is Xe2 prior art
// and is not reproduced):
//   * one 256-thread workgroup (4 wave64s, under 80 KB of LDS, so that two
//     share a CU and one's prologue and epilogue overlap the other's chunk
//     loop) per (group g, KV head h); grid order is XCD-aware so that each XCD
//     walks consecutive groups of one KV head;
//   * waves 0..2 consume, wave 3 produces (at raised priority: every wave waits
//     for its stage at the barrier). The producer turns the union's pool rows
//     into this KV head's offsets (two chunks at a time, every other
//     iteration) and gathers the INT8 K/V rows with 16-byte loads, every read
//     consumed at least kLead iterations after it was issued, converts the
//     rows to FP16 and stores them into LDS (K tiles in two stages, V tiles
//     and per-cell factors in four); a chunk's V tile and factors are stored
//     one iteration after its K tile, at the start of an iteration, so that
//     only the K stores are waited for at the barrier; the consumers only
//     read LDS;
//   * row n of the 96 = 8*hq + i (query head h*12+hq, position 8g+i), so the
//     chooser bit of row n is n & 7; consumer wave w owns row block w (32 rows)
//     and every cell of each chunk, with its own softmax state;
//   * S^T (32 cells x 32 rows, K=128) is 8 v_mfma_f32_32x32x16_f16 from the K
//     tile (LDS) and the wave's Q rows (FP16, held in registers for the whole
//     work-group); the first takes as its accumulator input a register set
//     that holds the K offset's term of each row; O^T (128 dims x 32 rows)
//     += V^T P'^T is 8 more MFMAs whose B operand (P'^T) comes straight from
//     the S^T accumulator registers, and whose A operand is read transposed
//     from the [cell][dim] V tile (ds_read_b64_tr_b16) in the same cell order;
//   * each consumer iteration issues the O^T update of chunk c-1, then the
//     S^T(c+1) chain with the softmax of chunk c between its MFMAs, so the
//     matrix pipe and the VALU work at the same time;
//   * K and V integers (plus the +1152 offset of the byte-to-FP16 trick) are
//     exact in FP16; the K offset is removed by starting each S^T chain from
//     -1152 sum(Q) of its row (FP32, kept in registers); k_scale *
//     softmax_scale * log2(e) multiplies the score in FP32, and the FP16
//     probabilities are multiplied by the FP16 v factor v_scale * 2^6 (2^-6
//     returns in the epilogue). Each lane tracks
//     the sum of the P' values it feeds the MFMA; 1152 times that sum (the V
//     offset) is removed once at the end;
//   * keep masks: the producers expand the chooser bytes into 16-bit all-ones
//     or zero masks per (position bit, cell), laid out so that a consumer lane
//     reads the eight words of its cell pairs with two 16-byte loads and
//     applies them with one AND per pair of packed FP16 probabilities;
//   * online softmax with a lazy stabiliser: probabilities are taken against
//     the running maximum (set from chunk 0's scores), and only when a lane's
//     chunk sum exceeds 128 does the wave recompute the chunk maximum and
//     rescale O, l and the P' sum.

#include "sel_attn_internal.h"

namespace selattn {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kConsumerWaves = 3;   // one per row block of 32
constexpr int kProducerWaves = 1;   // translate, gather, convert
constexpr int kThreads = 64 * (kConsumerWaves + kProducerWaves);
constexpr int kChunk = 32;          // union cells per iteration
constexpr int kD = 128;             // head dim
constexpr int kQPerKv = 12;
constexpr int kStages = 4;          // V tiles and factors: chunks c (read), c+1, c+2 (written)
constexpr int kKStages = 2;         // K tiles: chunks c+1 (read), c+2 (written)
constexpr int kKRow = kD + 8;       // K tile rows: 128 dims + 16 bytes of padding
constexpr int kLead = 3;            // iterations between a read and its first use (producers)
constexpr int kRing = 8;            // translated chunks (ring slots, indexed by chunk & 7)
constexpr float kLazyLimit = 128.f;  // a lane's chunk probability sum, against the running maximum
constexpr float kNoMax = -1e30f;    // stabiliser before a row has seen a chosen cell
constexpr float kVFold = 64.f;      // the FP16 v factor is v_scale * 2^6
constexpr float kVScaleLimit = 4.f; // so that v factor (<= 2^8) times probability (<= 2^7) fits FP16

// LDS: the four stages' K tiles, then their V tiles, so that a stage's tile
// addresses differ by multiples of the tile size that fit the 16-bit immediate
// offset of the LDS instructions (a per-lane base register serves every stage).
struct __align__(16) Ring {
  uint32_t off[kChunk];        // byte offset of the cell's K/V row in a pool:
                               // ((phys * n_kv + h) * 64 + slot) * 128; 0 = unusable
  uint8_t mask[kChunk];        // chooser byte; 0 for unusable cells
};

struct __align__(16) Smem {
  _Float16 k[kKStages][kChunk * kKRow]; // [cell][dim], rows of kKRow
  _Float16 v[kStages][kChunk * kD];     // [cell][dim], swizzled by v_pos()
  float kf[kStages][kChunk];            // k_scale * softmax_scale * log2(e); 0 where unusable
  _Float16 vf[kStages][kChunk];         // FP16(v_scale * 2^6); 0 where unusable
  uint32_t keep[kStages][4 * kChunk];   // keep masks, 16-byte units laid out by keep_unit()
  Ring ring[kRing];
};
// two work-groups share a CU (LDS 160 KB): one's prologue and epilogue overlap
// the other's chunk loop
static_assert(sizeof(Smem) <= 80 * 1024, "two work-groups per CU");

// The parts of the stages that hold chunk c.
struct Stage {
  _Float16* k;
  _Float16* v;
  float* kf;
  _Float16* vf;
  uint32_t* keep;
};

__device__ __forceinline__ Stage stage(Smem& sm, int c) {
  const int s = c & (kStages - 1);
  return Stage{sm.k[c & (kKStages - 1)], sm.v[s], sm.kf[s], sm.vf[s], sm.keep[s]};
}

// Keep masks of a chunk: for position bit b (row & 7) and lane half hb, eight
// words; word 2q + j holds in its low and high 16 bits all-ones or zero for
// cells 8q + 4hb + 2j and +1 (the cells, in order, whose scores a consumer
// lane packs into its j-th probability pair of group q). Words 4u..4u+3 form
// 16-byte unit keep_unit(b, hb, u): the eight position bits of a unit are
// adjacent, so the eight rows of a lane octet read eight distinct bank groups.
__device__ __forceinline__ int keep_unit(int b, int hb, int u) { return (2 * hb + u) * 8 + b; }

// ---------------------------------------------------------------------------
// Workgroup barrier that orders LDS only. Threads of a workgroup talk to each
// other through LDS alone (global memory is only read, plus the output stores
// and the status atomic), so the barrier need not wait for outstanding global
// loads: the producers' gathers stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The consumers' iteration barrier. A consumer wave writes no LDS inside its
// loop, and the only LDS reads it may still have in flight here are of a V tile
// that the producers rewrite two barriers later (by then the reads have been
// consumed), so it need not wait for them: the barrier only keeps the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void consumer_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// INT8 -> FP16: bias each byte to unsigned (v + 128) and place it under the
// FP16 exponent of 1024 (bit pattern 0x64XX = 1024 + XX): the exact FP16 value
// of v + 1152.
// four int8 in one dword -> the FP16 bit patterns of x + 1152 (exact), two per
// dword.
__device__ __forceinline__ uint2 i8x4_to_biased_half(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  return uint2{__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u),
               __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)};
}

// ---------------------------------------------------------------------------
// LDS tile layouts, chosen so that the producers' 16-byte stores and the
// consumers' MFMA-operand loads are free of bank conflicts (each lane octet
// of a 16-byte access touches 8 distinct units of a 128-byte bank period).
//
// K tile [cell][dim], rows of 272 bytes (128 dims + 16 bytes of padding): the
// 16 consecutive cells a consumer half-wave reads at one 16-byte unit fall on
// 16 distinct bank groups; a producer octet stores units 2p (then 2p + 1),
// p = 0..3 or 4..7, of an even cell and the odd cell after it, 17 units
// apart. Every consumer K address is one base plus an immediate.
// V tile [cell][dim], rows of 256 bytes, unit u of cell c at u ^ vswz(c),
// vswz(c) = ((c & 3) << 2) | (c & 1). A producer octet stores the same units
// as for K, the odd cell's moved by 5 modulo 8; consumers read it transposed,
// 8 bytes per lane, four consecutive cells x 64 bytes per 32 lanes
// (4(mb ^ x) + (v ^ (x & 1)) are 16 distinct positions).
__device__ __forceinline__ int v_pos(int u, int cell) {
  return u ^ (((cell & 3) << 2) | (cell & 1));
}

// ---------------------------------------------------------------------------
// Producer staging tasks. Task t in [0,512) covers cell task_cell(t), dims
// 16 task_block(t) .. +15: one 16-byte load from the K pool and one from the
// V pool at the same offset. Each lane octet takes blocks 0..3 (or 4..7) of an
// even cell and of the odd cell after it, so that its 16-byte stores fall on
// eight distinct bank groups in both tiles: even and odd rows of the K tile
// are 17 units apart, and the V swizzle moves odd cells by 5 units (mod 8).
// Unusable cells (padding, non-resident, bad) read pool row 0, which always
// exists; their chooser byte and scales are 0, so the values never count.
// A scale is zeroed exactly when its cell's chooser byte is 0 (such a cell
// contributes nothing either way).
__device__ __forceinline__ int task_cell(int t) { return 2 * (t >> 4) + ((t >> 2) & 1); }
__device__ __forceinline__ int task_block(int t) { return 4 * ((t >> 3) & 1) + (t & 3); }

__device__ __forceinline__ uint32_t task_offset(const Ring& rg, int t) {
  return rg.off[task_cell(t)] + 16u * task_block(t);
}

// K keeps the offset too: Q.(k + 1152) = Q.k + 1152 sum(Q), and every S^T
// chain starts from -1152 sum(Q) of its row instead of zero.
__device__ __forceinline__ void store_k_task(const Stage& st, int t, u32x4 raw) {
  const int cell = task_cell(t);
  const int u0 = 2 * task_block(t);
  const uint2 b0 = i8x4_to_biased_half(raw.x), b1 = i8x4_to_biased_half(raw.y);
  const uint2 b2 = i8x4_to_biased_half(raw.z), b3 = i8x4_to_biased_half(raw.w);
  _Float16* base = st.k + cell * kKRow + 8 * u0;
  *reinterpret_cast<u32x4*>(base) = u32x4{b0.x, b0.y, b1.x, b1.y};
  *reinterpret_cast<u32x4*>(base + 8) = u32x4{b2.x, b2.y, b3.x, b3.y};
}

// The V tile keeps v + 1152: the consumers track the sum of the FP16
// probabilities they multiply with it and remove 1152 times that sum at the end.
__device__ __forceinline__ void store_v_task(const Stage& st, int t, u32x4 raw) {
  const int cell = task_cell(t);
  const int u0 = 2 * task_block(t);
  const uint2 b0 = i8x4_to_biased_half(raw.x), b1 = i8x4_to_biased_half(raw.y);
  const uint2 b2 = i8x4_to_biased_half(raw.z), b3 = i8x4_to_biased_half(raw.w);
  _Float16* base = st.v + cell * kD;
  *reinterpret_cast<u32x4*>(base + (v_pos(u0, cell) << 3)) = u32x4{b0.x, b0.y, b1.x, b1.y};
  *reinterpret_cast<u32x4*>(base + (v_pos(u0 + 1, cell) << 3)) = u32x4{b2.x, b2.y, b3.x, b3.y};
}

// ---------------------------------------------------------------------------
// Translation of one chunk cell (one lane per cell; the two lane halves take
// the two chunks of a pair), in two steps: read the union entry (the cell's
// pool row for KV head 0, resolved through the page table when the union was
// built, and its chooser byte), then, four iterations later (at least the lead
// of the K/V gathers, so that no wait for an early read also waits for gathers
// still in flight), form this KV head's pool offset and publish it in the ring.
// Records carry only loaded words (each in a register of its own: packing a
// field next to another would read the in-flight load at once); whether an
// entry lies inside the union is recomputed from the chunk index.
struct UnionRec {
  int32_t row;
  uint32_t mask;
};

__device__ __forceinline__ bool in_union(int U, int cc, int lane) { return cc * kChunk + lane < U; }

// Both steps are branch-free (clamped, always-valid addresses plus selects) so
// that a producer iteration stays one basic block.
__device__ __forceinline__ UnionRec read_union_entry(const PrefillArgs& a, int64_t ubase, int U,
                                                     int cc, int lane) {
  // union rows hold at least 8 entries, so index 0 is always readable
  const int64_t at = ubase + (in_union(U, cc, lane) ? cc * kChunk + lane : 0);
  UnionRec u;
  u.row = a.union_rows[at];
  u.mask = a.union_mask[at];
  return u;
}

// A row of -1 is a page that is not resident; a row whose KV-head rows would
// leave the pools is flagged and treated the same way.
__device__ __forceinline__ void finish_translation(const PrefillArgs& a, const UnionRec& u, int U,
                                                   int cc, int h, Ring& rg, int lane,
                                                   uint32_t& flags) {
  const bool valid = in_union(U, cc, lane);
  const bool usable = valid && (uint32_t)u.row < a.row_limit;
  flags |= (valid && u.row != -1 && !usable) ? SEL_ATTN_STATUS_PAGE_RANGE : 0u;
  const uint32_t row = (uint32_t)u.row + 64u * (uint32_t)h;
  rg.off[lane] = usable ? row * kD : 0u;
  rg.mask[lane] = (uint8_t)(usable ? u.mask : 0u);
}

// ---------------------------------------------------------------------------
// Consumer waves 0..2: row block w (32 rows).
// The K tile holds k + 1152, so every S^T chain starts from -1152 sum(Q) of
// each row instead of zero: the first MFMA reads it as its accumulator input
// from a register set filled once per work-group (the value is the same for
// all 16 accumulator entries of a lane, which share the lane's row).

// S^T (the chunk's 32 cells x this wave's 32 rows). q: this lane's Q operands
// (k-step ks: dims 16ks + 8hb .. +7 of its row), in registers for the whole
// work-group.
__device__ __forceinline__ float16v scores_t(const Stage& st, const half8 q[8],
                                             const float16v& s_init, int hb, int l32) {
  float16v s = s_init;
  const _Float16* krow = st.k + l32 * kKRow + 8 * hb;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const half8 ka = *reinterpret_cast<const half8*>(krow + 16 * ks);
    s = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, q[ks], s, 0, 0, 0);
  }
  return s;
}
// The A operand of O^T (dims 32mb + 0..31) += V^T P'^T for k-step ks, read
// transposed from the [cell][dim] V tile with ds_read_b64_tr_b16: within each
// group of 16 lanes, lane i receives element i % 4 of the 8-byte rows addressed
// by lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4. Lane l addresses cell
// 16ks + 4hb + ((l & 15) >> 2) (and the same + 8 for the second half)
// at dims 32mb + 16((l >> 4) & 1) + 4(l & 3), so it receives dim 32mb + (l & 31)
// of the eight cells whose P'^T values it holds, in the same order.
typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));

__device__ __forceinline__ half8 load_v_operand(const Stage& st, int ks, int mb, int lane) {
  const int hb = lane >> 5;
  const int c0 = 16 * ks + 4 * hb + ((lane & 15) >> 2);
  const int dimb = 64 * mb + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);   // byte in the row
  const int pos = v_pos(dimb >> 4, c0);   // the same for cell c0 + 8
  const char* row0 = reinterpret_cast<const char*>(st.v) + c0 * (kD * 2) + (pos << 4) + (dimb & 15);
  typedef __attribute__((address_space(3))) fp16x4_t* lds_ptr;
  const fp16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_ptr)(row0));
  const fp16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_ptr)(row0 + 8 * kD * 2));
  return half8{(_Float16)a[0], (_Float16)a[1], (_Float16)a[2], (_Float16)a[3],
               (_Float16)b[0], (_Float16)b[1], (_Float16)b[2], (_Float16)b[3]};
}

// Registers a consumer wave carries from one iteration to the next.
struct ConsState {
  float16v o[4];      // O^T (128 dims x this wave's 32 rows), scaled by 2^6
  float16v s_cur;     // S^T of the current chunk (issued in the previous iteration)
  half8 q[8];          // this lane's Q operands (FP16), for every chunk
  float16v s_init;    // every S^T chain's start: -1152 sum(Q) of this lane's row
  half8 pb[2];        // P'^T of the previous chunk
  half8 vfrag[8];     // V^T operands of the previous chunk
  float m_run;        // running maximum (log2 domain) of this lane's row
  float l_run;        // running sum of probabilities against m_run
  float lp;           // running sum of this lane's FP16 P'^T values (the V tile
                      // holds v + 1152: O^T carries 1152 times the row's sum)
};

// Per-chunk operands of a lane's softmax: k factors of its 16 cells, v factors
// and keep masks of its 8 cell pairs.
struct ChunkFactors {
  float4v k4[4];
  half2 vf[8];
  uint32_t keep[8];
};

// Keep masks, v factors and the first two k-factor groups of chunk c.
__device__ __forceinline__ void load_factors(ChunkFactors& f, const Stage& st, int hb, int l32) {
  const u32x4* kp = reinterpret_cast<const u32x4*>(st.keep);
  const u32x4 a0 = kp[keep_unit(l32 & 7, hb, 0)], a1 = kp[keep_unit(l32 & 7, hb, 1)];
  f.keep[0] = a0.x; f.keep[1] = a0.y; f.keep[2] = a0.z; f.keep[3] = a0.w;
  f.keep[4] = a1.x; f.keep[5] = a1.y; f.keep[6] = a1.z; f.keep[7] = a1.w;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const half4 v = *reinterpret_cast<const half4*>(st.vf + 8 * q + 4 * hb);
    f.vf[2 * q] = half2{v[0], v[1]};
    f.vf[2 * q + 1] = half2{v[2], v[3]};
  }
  f.k4[0] = *reinterpret_cast<const float4v*>(st.kf + 4 * hb);
  f.k4[1] = *reinterpret_cast<const float4v*>(st.kf + 8 + 4 * hb);
}

// Probability pair j (scores 2j, 2j+1) of chunk c: FP16, masked, summed into
// psum; times the v factors into P'^T, summed into lpc.
__device__ __forceinline__ void prob_pair(ConsState& cs, const ChunkFactors& f, int j, float u0,
                                          float u1, float& psum, float& lpc) {
  const half2 one = {(_Float16)1.f, (_Float16)1.f};
  const half2 p = {(_Float16)__builtin_amdgcn_exp2f(u0), (_Float16)__builtin_amdgcn_exp2f(u1)};
  const half2 pm = __builtin_bit_cast(half2, __builtin_bit_cast(uint32_t, p) & f.keep[j]);
  psum = __builtin_amdgcn_fdot2(pm, one, psum, false);
  const half2 pv = pm * f.vf[j];
  lpc = __builtin_amdgcn_fdot2(pv, one, lpc, false);
  cs.pb[j >> 2][2 * (j & 3)] = pv[0];
  cs.pb[j >> 2][2 * (j & 3) + 1] = pv[1];
}

// The S^T(c+1) chain with the softmax of chunk c between its MFMAs (one
// probability pair per MFMA); K operands are read two MFMAs ahead, the
// remaining k factors on the way. Leaves P'^T(c) in cs.pb and returns this
// lane's probability sum and P'^T sum.
__device__ __forceinline__ void chain_softmax(ConsState& cs, const Stage& st, const _Float16* krow,
                                              ChunkFactors& f, half8 kfrag[8], float16v& s_next,
                                              float& psum, float& lpc, int hb) {
  psum = 0.f;
  lpc = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    s_next = __builtin_amdgcn_mfma_f32_32x32x16_f16(kfrag[j], cs.q[j], j == 0 ? cs.s_init : s_next,
                                                    0, 0, 0);
    if (j + 2 < 8) kfrag[j + 2] = *reinterpret_cast<const half8*>(krow + 16 * (j + 2));
    const int r = 2 * j;
    prob_pair(cs, f, j, __builtin_fmaf(cs.s_cur[r], f.k4[r >> 2][r & 3], -cs.m_run),
              __builtin_fmaf(cs.s_cur[r + 1], f.k4[r >> 2][(r + 1) & 3], -cs.m_run), psum, lpc);
    if (j == 1 || j == 3) {   // k factors two MFMAs ahead of their scores
      const int q4 = (j + 3) >> 1;
      f.k4[q4] = *reinterpret_cast<const float4v*>(st.kf + 8 * q4 + 4 * hb);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Iteration c (phase P = c & 3). On entry S^T(c) is complete and chunk c-1's
// P'^T and V^T operands are in registers. The iteration issues O^T += V^T P'^T
// for chunk c-1, runs the S^T(c+1) chain with the softmax of chunk c placed
// between its MFMAs, one probability pair per MFMA, so the matrix pipe and the
// VALU work at the same time, forms P'^T(c) and reads chunk c's V^T operands
// (their LDS latency passes during the barrier).
template <int P>
__device__ __forceinline__ void consume_step(ConsState& cs, Smem& sm, int hb, int l32) {
  const Stage st = stage(sm, P);            // chunk c: factors, keep masks, V
  const Stage st_next = stage(sm, P + 1);   // chunk c+1: K
  const float ninf = -__builtin_inff();

  // LDS reads: chunk c's keep masks and v factors of this lane's cell pairs,
  // the first k factors
  ChunkFactors f;
  load_factors(f, st, hb, l32);

  // O^T += V^T P'^T of chunk c-1
#pragma unroll
  for (int j = 0; j < 8; ++j)
    cs.o[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cs.vfrag[j], cs.pb[j >> 2], cs.o[j & 3], 0, 0, 0);

  // the first two of chunk c+1's K operands (the others are read two MFMAs
  // ahead of their use in the chain below)
  half8 kfrag[8];
  const _Float16* krow = st_next.k + l32 * kKRow + 8 * hb;
#pragma unroll
  for (int j = 0; j < 2; ++j) kfrag[j] = *reinterpret_cast<const half8*>(krow + 16 * j);

  float16v s_next;
  float psum, lpc;
  chain_softmax(cs, st, krow, f, kfrag, s_next, psum, lpc, hb);

  // the lazy stabiliser: only when some lane's chunk sum leaves [0, 128] is the
  // running maximum moved (what is accumulated is rescaled; this waits for the
  // MFMAs issued above) and the chunk redone against it
  if (__ballot(!(psum <= kLazyLimit))) {
    // the chunk's factors again from LDS (registers are not held for this rare path)
    ChunkFactors g;
    load_factors(g, st, hb, l32);
#pragma unroll
    for (int q4 = 2; q4 < 4; ++q4)
      g.k4[q4] = *reinterpret_cast<const float4v*>(st.kf + 8 * q4 + 4 * hb);
    float cmax = ninf;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const bool keep = (g.keep[r >> 1] >> (16 * (r & 1))) & 1u;
      cmax = fmaxf(cmax, keep ? cs.s_cur[r] * g.k4[r >> 2][r & 3] : ninf);
    }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(cs.m_run, cmax);
    const float alpha = __builtin_amdgcn_exp2f(cs.m_run - m_new);
    cs.m_run = m_new;
    cs.l_run *= alpha;
    cs.lp *= alpha;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) cs.o[mb][r] *= alpha;
    psum = 0.f;
    lpc = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 2 * j;
      prob_pair(cs, g, j, __builtin_fmaf(cs.s_cur[r], g.k4[r >> 2][r & 3], -cs.m_run),
                __builtin_fmaf(cs.s_cur[r + 1], g.k4[r >> 2][(r + 1) & 3], -cs.m_run), psum, lpc);
    }
  }
  cs.l_run += psum;
  cs.lp += lpc;

  // chunk c's V^T operands for the next iteration's update (stage c & 3 is
  // rewritten only three iterations from now)
#pragma unroll
  for (int j = 0; j < 8; ++j) cs.vfrag[j] = load_v_operand(st, j >> 2, j & 3, (hb << 5) | l32);
  cs.s_cur = s_next;
  consumer_barrier();
}

__device__ __forceinline__ void consume_chunks(ConsState& cs, Smem& sm, int hb, int l32, int nch) {
  int c = 0;
  for (; c + 4 <= nch; c += 4) {
    consume_step<0>(cs, sm, hb, l32);
    consume_step<1>(cs, sm, hb, l32);
    consume_step<2>(cs, sm, hb, l32);
    consume_step<3>(cs, sm, hb, l32);
  }
  const int rem = nch - c;
  if (rem > 0) consume_step<0>(cs, sm, hb, l32);
  if (rem > 1) consume_step<1>(cs, sm, hb, l32);
  if (rem > 2) consume_step<2>(cs, sm, hb, l32);
}

template <bool kSplit>
__device__ __forceinline__ void consume(const PrefillArgs& a, Smem& sm, int g, int h,
                                        int nch, int wave, int lane, PrefillPartial* rec) {
  const int rb = wave;
  const int hb = lane >> 5;
  const int l32 = lane & 31;
  const int n_qh = a.n_kv * kQPerKv;

  // this lane's row: query head h*12 + hq, query index 8g + i
  const int row_n = 32 * rb + l32;
  const int hq = row_n >> 3;
  const int qi = 8 * g + (row_n & 7);
  const bool row_ok = qi < a.n_q;

  ConsState cs;
  // Q in FP16, straight into the B operands of S^T = K Q^T (k-step s: dims
  // 16s + 8hb .. +7 of this lane's row)
  {
    const float* qg = a.q + ((int64_t)(row_ok ? qi : 0) * n_qh + h * kQPerKv + hq) * kD;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      float4v x0 = *reinterpret_cast<const float4v*>(qg + 16 * s + 8 * hb);
      float4v x1 = *reinterpret_cast<const float4v*>(qg + 16 * s + 8 * hb + 4);
      if (!row_ok) x0 = x1 = float4v{0.f, 0.f, 0.f, 0.f};
      cs.q[s] = half8{(_Float16)x0.x, (_Float16)x0.y, (_Float16)x0.z, (_Float16)x0.w,
                      (_Float16)x1.x, (_Float16)x1.y, (_Float16)x1.z, (_Float16)x1.w};
    }
  }

  lds_barrier();   // prologue: ring filled
  lds_barrier();   // prologue: chunks 0 and 1 staged

  cs.m_run = kNoMax;
  cs.l_run = 0.f;
  cs.lp = 0.f;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) cs.o[mb][r] = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) cs.vfrag[j][e] = (_Float16)0.f;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) cs.pb[ks][e] = (_Float16)0.f;
  {
    // -1152 times the sum of this lane's row of FP16 Q (both lane halves'
    // dims): the accumulator input of every chain's first MFMA
    const half2 one = {(_Float16)1.f, (_Float16)1.f};
    float qs = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        qs = __builtin_amdgcn_fdot2(half2{cs.q[s][2 * e], cs.q[s][2 * e + 1]}, one, qs, false);
    const float init = -1152.f * (qs + __shfl_xor(qs, 32));
#pragma unroll
    for (int r = 0; r < 16; ++r) cs.s_init[r] = init;
  }
  cs.s_cur = scores_t(stage(sm, 0), cs.q, cs.s_init, hb, l32);
  {
    // the running maximum starts at chunk 0's maximum over this row's chosen
    // cells, so that the first chunk needs no rescale (the sinks lead the union)
    const Stage st = stage(sm, 0);
    ChunkFactors g;
    load_factors(g, st, hb, l32);
#pragma unroll
    for (int q4 = 2; q4 < 4; ++q4)
      g.k4[q4] = *reinterpret_cast<const float4v*>(st.kf + 8 * q4 + 4 * hb);
    float cmax = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const bool keep = (g.keep[r >> 1] >> (16 * (r & 1))) & 1u;
      cmax = fmaxf(cmax, keep ? cs.s_cur[r] * g.k4[r >> 2][r & 3] : -__builtin_inff());
    }
    cs.m_run = fmaxf(kNoMax, fmaxf(cmax, __shfl_xor(cmax, 32)));
  }
  lds_barrier();   // prologue: chunk 0's K tile read (the producers rewrite it next)

  consume_chunks(cs, sm, hb, l32, nch);
  // the last chunk's O^T update
#pragma unroll
  for (int j = 0; j < 8; ++j)
    cs.o[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cs.vfrag[j], cs.pb[j >> 2], cs.o[j & 3], 0, 0, 0);

  // out = (O^T - 1152 sum(P'), the V tile's offset) * 2^-6 / l; the row's sums
  // are split over the two lane halves (their cells)
  const float corr = 1152.f * (cs.lp + __shfl_xor(cs.lp, 32));
  const float lt = cs.l_run + __shfl_xor(cs.l_run, 32);
  if constexpr (kSplit) {
    // one share of the union: its unnormalised state, for the merge (rows of
    // absent positions are never merged)
    if (row_ok) {
      float* orow = rec->o[row_n];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          float4v r;
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = cs.o[mb][4 * q4 + e] - corr;
          *reinterpret_cast<float4v*>(orow + 32 * mb + 8 * q4 + 4 * hb) = r;
        }
      if (hb == 0) {
        rec->m[row_n] = cs.m_run;
        rec->l[row_n] = lt;
      }
    }
    return;
  }
  const float inv = lt > 0.f ? (1.f / kVFold) / lt : 0.f;
  if (row_ok) {
    float* orow = a.out + ((int64_t)qi * n_qh + h * kQPerKv + hq) * kD;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float4v r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = (cs.o[mb][4 * q4 + e] - corr) * inv;
        *reinterpret_cast<float4v*>(orow + 32 * mb + 8 * q4 + 4 * hb) = r;
      }
  }
}

// ---------------------------------------------------------------------------
// Producer wave 3 (64 threads, ptid = tid - 192). Iteration c (while the
// consumers work on chunks c and c+1): store chunk c+1's V tile and factors,
// on even c translate a pair of chunks (union entries of c+10, c+11 read, ring
// slots of c+6, c+7 written; lane half hb takes the pair's chunk hb, cell
// ptid & 31), gather chunk c+kAheadGather into registers (its
// ring slot read at the end of the previous iteration), store the K tile of
// chunk c+2 (gathered kLead iterations earlier) and read the ring slot of the
// next iteration's gather. Each
// thread owns tasks ptid + 64k (k = 0..3) of both pools, and the k scale
// (ptid < 32) or v scale of cell ptid & 31.
struct Raw {
  u32x4 k[4];
  u32x4 v[4];
  float sc;     // k scale (ptid < 32) or v scale of cell ptid & 31 (row 0's if unusable)
  uint32_t m;   // chooser byte of that cell; 0 if unusable
  uint32_t kw;  // chooser bytes of the four cells whose keep masks this thread forms
};

// Thread ptid forms keep words 2q and 2q + 1 for position bit b = ptid & 7,
// group q = (ptid >> 3) & 3 and lane half hb = ptid >> 5: they cover cells
// 4w..4w+3, w = 2q + hb, whose chooser bytes are word w of the ring's.
__device__ __forceinline__ int keep_word(int ptid) { return 2 * ((ptid >> 3) & 3) + (ptid >> 5); }

// What a gather reads from its ring slot, read one iteration ahead so that the
// gather's loads need not wait for LDS.
struct GatherAddr {
  uint32_t off[4];
  uint32_t soff;
  uint32_t m;
  uint32_t kw;
};

__device__ __forceinline__ GatherAddr gather_addr(const Ring& rg, int ptid) {
  GatherAddr g;
#pragma unroll
  for (int k = 0; k < 4; ++k) g.off[k] = task_offset(rg, ptid + 64 * k);
  const int cell = ptid & (kChunk - 1);
  g.soff = rg.off[cell];
  g.m = rg.mask[cell];
  g.kw = reinterpret_cast<const uint32_t*>(rg.mask)[keep_word(ptid)];
  return g;
}

__device__ __forceinline__ void gather(const PrefillArgs& a, const GatherAddr& g, int ptid, Raw& r) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    r.k[k] = *reinterpret_cast<const u32x4*>(a.k_pool + g.off[k]);
    r.v[k] = *reinterpret_cast<const u32x4*>(a.v_pool + g.off[k]);
  }
  const float* sp = (ptid < kChunk) ? a.k_scale : a.v_scale;
  r.sc = sp[g.soff / kD];   // zeroed at conversion, when the load has landed
  r.m = g.m;
  r.kw = g.kw;
}

// Keep masks from the chooser bytes of cells 4w..4w+3 (word w of the ring's
// bytes) for position bit b: shifted so that bit b of bytes 0 and 2 lands on
// bits 15 and 31 of lo, of bytes 1 and 3 on bits 15 and 31 of hi; byte
// selectors 8..11 of v_perm replicate bits 15 and 31 of either source.
__device__ __forceinline__ uint2 keep_words(uint32_t x, int b) {
  const uint32_t lo = x << (15 - b);
  const uint32_t hi = x << (7 - b);
  return uint2{__builtin_amdgcn_perm(lo, hi, 0x08080a0au), __builtin_amdgcn_perm(lo, hi, 0x09090b0bu)};
}

// K tile of a chunk (read by the consumers' S^T chain in the next iteration)
__device__ __forceinline__ void convert_k(const Stage& st, int ptid, const Raw& r) {
#pragma unroll
  for (int k = 0; k < 4; ++k) store_k_task(st, ptid + 64 * k, r.k[k]);
}

// V tile, k and v factors and keep masks of a chunk (read by the consumers two
// iterations later than its K tile)
__device__ __forceinline__ void convert_v(const PrefillArgs& a, const Stage& st, int ptid, bool kwave,
                                          const Raw& r, uint32_t& flags) {
#pragma unroll
  for (int k = 0; k < 4; ++k) store_v_task(st, ptid + 64 * k, r.v[k]);
  // the lower lane half stores the k factors, the upper the v factors
  const int lane = ptid & (kChunk - 1);
  const float sc = r.m ? r.sc : 0.f;
  if (kwave) {
    st.kf[lane] = sc * a.score_scale;
  } else {
    const bool v_ok = fabsf(sc) < kVScaleLimit;
    flags |= v_ok ? 0u : SEL_ATTN_STATUS_V_SCALE;
    st.vf[lane] = (_Float16)(v_ok ? sc * kVFold : 0.f);
  }
  // keep words 2q and 2q + 1 (q = (ptid >> 3) & 3) of position bit ptid & 7
  const int q = (ptid >> 3) & 3;
  uint32_t* kp = st.keep + 4 * keep_unit(ptid & 7, ptid >> 5, q >> 1) + 2 * (q & 1);
  *reinterpret_cast<uint2*>(kp) = keep_words(r.kw, ptid & 7);
}

// Producer state: gathered rows, indexed by chunk & 3 (chunk x is gathered in
// iteration x-2-kLead and converted in x-2), and union records (read four
// iterations before the ring slots of their chunks are written). Every index
// below is a compile-time constant once a step is instantiated for its phase
// P = c & 3, so the sets stay in registers and the stage addresses fold into
// immediates.
constexpr int kAheadGather = 2 + kLead;        // chunk gathered in iteration c: c + 5
// Translation runs on even iterations c, for a pair of chunks at once (lane
// half hb takes chunk c' + hb of the pair starting at c'): the ring slots of
// chunks c+6, c+7 are written from union records read four iterations earlier.
// Chunk x's slot is thus written one or two iterations before x is gathered
// (x - 5).
constexpr int kPairFinish = 6;                 // pair whose ring slots are written: c + 6, c + 7
constexpr int kPairUnion = 10;                 // pair whose union entries are read: c + 10, c + 11
static_assert(kAheadGather < kPairFinish && kPairFinish + 1 < kAheadGather + kRing,
              "ring slots are written before their gather and kept until it");
static_assert(kPairUnion == kPairFinish + 4, "union records are consumed four iterations later");

struct ProdState {
  Raw raw[4];
  UnionRec un[2];   // by phase: set P / 2 is read and consumed in phase P (0 or 2)
  GatherAddr ga;    // ring reads of the next iteration's gather
};

// Iteration c (phase P = c & 3), while the consumers work on chunks c-1..c+1.
// It opens with the V tile and factors of chunk c+1, so that those stores drain
// while the rest of the iteration runs, and closes with the K tile of chunk c+2,
// the only stores the consumers need right after this iteration's barrier.
// Reads are issued union, gather; union records are consumed four iterations
// later, gathers kLead; the gather of chunk c+5 reuses the register
// set that chunk c+1's V conversion has just emptied. `lower` (ptid < 32): this
// lane stores k factors, else v factors.
template <int P>
__device__ __forceinline__ void produce_step(const PrefillArgs& a, Smem& sm, ProdState& ps, int c,
                                             int h, int U, int64_t ubase, int ptid, bool lower,
                                             uint32_t& flags) {
  const int lane = ptid & (kChunk - 1);
  convert_v(a, stage(sm, P + 1), ptid, lower, ps.raw[(P + 1) & 3], flags);
  if constexpr ((P & 1) == 0) {
    // the record set of this phase was read four iterations ago for the pair
    // finished now, and is refilled for the one finished four iterations on
    constexpr int s = P / 2;
    const int hb = ptid >> 5;
    const int cf = c + kPairFinish + hb;
    finish_translation(a, ps.un[s], U, cf, h, sm.ring[cf & (kRing - 1)], lane, flags);
    ps.un[s] = read_union_entry(a, ubase, U, c + kPairUnion + hb, lane);
  }
  gather(a, ps.ga, ptid, ps.raw[(P + kAheadGather) & 3]);
  convert_k(stage(sm, P + 2), ptid, ps.raw[(P + 2) & 3]);
  // the next gather's slot (chunk c+1+kAheadGather) is written by now: on even c
  // just above, on odd c one iteration ago
  ps.ga = gather_addr(sm.ring[(c + 1 + kAheadGather) & (kRing - 1)], ptid);
  lds_barrier();
}

__device__ __forceinline__ void produce(const PrefillArgs& a, Smem& sm, int h, int U, int nch,
                                        int64_t ubase, int ptid, bool lower,
                                        uint32_t& flags) {
  static_assert(kLead >= 1 && kLead <= 3 && kStages == 4, "register sets cover the lead");
  static_assert(kPairFinish == 6 && kPairUnion == 10, "the prologue below");
  const int lane = ptid & (kChunk - 1);
  const int hb = ptid >> 5;
  ProdState ps;
  // prologue: what iteration 0 expects. Chunks 0..5 translated into their ring
  // slots; the union records of chunks 6, 7 (set 0, finished in iteration 0)
  // and 8, 9 (set 1, iteration 2) read; chunk 0 staged, chunk 1's K tile
  // staged, chunks 1 .. kAheadGather-1 gathered.
  {
    UnionRec u[3];
#pragma unroll
    for (int m = 0; m < 3; ++m) u[m] = read_union_entry(a, ubase, U, 2 * m + hb, lane);
    ps.un[0] = read_union_entry(a, ubase, U, kPairFinish + hb, lane);
    ps.un[1] = read_union_entry(a, ubase, U, kPairFinish + 2 + hb, lane);
#pragma unroll
    for (int m = 0; m < 3; ++m)
      finish_translation(a, u[m], U, 2 * m + hb, h, sm.ring[2 * m + hb], lane, flags);
  }
  lds_barrier();
  static_assert(kAheadGather == 5, "the prologue stages chunk 0 before gathering chunk 4");
#pragma unroll
  for (int x = 0; x < kAheadGather; ++x) {
    if (x == 4) {   // chunk 0 in full, which frees its register set
      convert_k(stage(sm, 0), ptid, ps.raw[0]);
      convert_v(a, stage(sm, 0), ptid, lower, ps.raw[0], flags);
    }
    gather(a, gather_addr(sm.ring[x], ptid), ptid, ps.raw[x & 3]);
  }
  ps.ga = gather_addr(sm.ring[kAheadGather], ptid);
  // chunk 1's K tile (its V tile and factors open iteration 0)
  convert_k(stage(sm, 1), ptid, ps.raw[1]);
  lds_barrier();
  lds_barrier();   // the consumers have read chunk 0's K tile

  int c = 0;
  for (; c + 4 <= nch; c += 4) {
    produce_step<0>(a, sm, ps, c, h, U, ubase, ptid, lower, flags);
    produce_step<1>(a, sm, ps, c + 1, h, U, ubase, ptid, lower, flags);
    produce_step<2>(a, sm, ps, c + 2, h, U, ubase, ptid, lower, flags);
    produce_step<3>(a, sm, ps, c + 3, h, U, ubase, ptid, lower, flags);
  }
  const int rem = nch - c;   // 0..3 more iterations, phases 0, 1, 2
  if (rem > 0) produce_step<0>(a, sm, ps, c, h, U, ubase, ptid, lower, flags);
  if (rem > 1) produce_step<1>(a, sm, ps, c + 1, h, U, ubase, ptid, lower, flags);
  if (rem > 2) produce_step<2>(a, sm, ps, c + 2, h, U, ubase, ptid, lower, flags);
}

}  // namespace
}  // namespace selattn
