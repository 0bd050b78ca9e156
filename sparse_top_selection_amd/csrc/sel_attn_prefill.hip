// Attention over each group's selection union: INT8 paged K/V, FP16 MFMA,
// FP32 online softmax with a per-position chooser mask.
//
// Page: #2808 "sycl: prompt attention over 8-query selection unions on XMX".
//   section Summary: 64-cell chunks of the union are dequantised once to FP16;
//     S^T = K Q^T and O += P V run on matrix units with FP32 sums for all 96 rows
//     (8 positions x 12 heads); in the online softmax a cell is -inf for the
//     positions that did not choose it; Q, K, V and P enter the products as FP16.
//   section What changed: one work-group per 8 positions and KV head.
//   section Extra Notes: cells of non-resident pages are masked.
//
// gfx950 mapping (the page's 16-lane sub-group / 256-GRF shape is Xe2 prior art
// and is not reproduced):
//   * one 512-thread workgroup (8 wave64s, one per CU at this register budget,
//     two per SIMD) per (group g, KV head h); grid order is XCD-aware so that
//     each XCD walks consecutive groups of one KV head;
//   * waves 0..5 consume, waves 6..7 produce. The producers translate union
//     cells through the page table, gather the INT8 K/V rows with 16-byte /
//     8-byte loads two chunks ahead of their use, convert them to FP16 and store
//     them into a 4-stage LDS ring of tiles; the consumers only read LDS;
//   * row n of the 96 = 8*hq + i (query head h*12+hq, position 8g+i), so the
//     chooser bit of row n is n & 7; consumer wave w owns row block rb = w % 3
//     (32 rows) and cell half ch = w / 3 (32 of each chunk's 64 cells) with its
//     own softmax state; the two halves are merged once at the end;
//   * S^T (32 cells x 32 rows, K=128) is 8 v_mfma_f32_32x32x16_f16 from the LDS K
//     tile with Q^T held in registers; O^T (128 dims x 32 rows) += V^T P^T is 8
//     more MFMAs whose B operand (P^T) comes straight from the S^T accumulator
//     registers: the V^T tile is stored in the matching cell permutation;
//   * each consumer iteration issues the MFMAs of S^T for chunk c+1 and of
//     O^T += V^T P^T for chunk c-1, interleaved with the softmax of chunk c, so
//     the matrix pipe and the VALU work at the same time;
//   * K and V integers are exact in FP16, so the scales are applied in FP32:
//     k_scale * softmax_scale * log2(e) multiplies the score, v_scale * 2^10 the
//     probability before its FP16 rounding (2^-10 returns in the epilogue);
//   * the chooser byte of a cell becomes a 64-bit SGPR lane mask (the byte
//     replicated 4x per 32 lanes) and one v_cndmask applies it per score;
//   * online softmax with a lazy stabiliser: probabilities are taken against
//     the running maximum, and only when a lane's chunk sum exceeds 16 does the
//     wave recompute the chunk maximum and rescale O and l (always on a row's
//     first chosen chunk, rarely after).

#include "sel_attn_internal.h"

namespace selattn {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kConsumerWaves = 6;   // 3 row blocks x 2 cell halves
constexpr int kProducerWaves = 2;   // translate, gather, convert
constexpr int kThreads = 64 * (kConsumerWaves + kProducerWaves);
constexpr int kChunk = 64;          // union cells per iteration
constexpr int kD = 128;             // head dim
constexpr int kQPerKv = 12;
constexpr int kStages = 4;          // LDS tiles: chunks c-1 (V), c, c+1 (K), c+2 (being written)
constexpr int kLead = 2;            // iterations between a read and its first use (producers)
constexpr int kRing = 8;            // translated chunks (ring slots, indexed by chunk & 7)
constexpr float kLazyLimit = 16.f;
constexpr float kNoMax = -1e30f;    // stabiliser before a row has seen a chosen cell
constexpr float kVFold = 1024.f;    // probabilities carry v_scale * 2^10 into FP16
constexpr float kVScaleLimit = 4.f;

// LDS: the four stages' K tiles fill the first 64 KiB and their V^T tiles the
// next 64 KiB, so that a stage's tile addresses differ by multiples of 16 KiB
// that fit the 16-bit immediate offset of the LDS instructions (a per-lane
// base register serves every stage).
struct __align__(16) Ring {
  uint32_t off[kChunk];        // byte offset of the cell's K/V row in a pool:
                               // ((phys * n_kv + h) * 64 + slot) * 128; 0 = unusable
  uint8_t mask[kChunk];        // chooser byte; 0 for unusable cells
};

struct __align__(16) Smem {
  _Float16 k[kStages][kChunk * kD];     // [cell][dim] holding k + 1152, swizzled by k_unit()
  _Float16 vt[kStages][kD * kChunk];    // [dim][slot], swizzled by v_unit()
  float kf[kStages][kChunk];            // k_scale * softmax_scale * log2(e); 0 where unusable
  float vf[kStages][kChunk];            // v_scale * 2^10; 0 where unusable
  uint32_t emask[kStages][kChunk / 4];  // chooser bytes, 0 for padding / non-resident cells
  uint32_t emask_spare[kStages][kChunk / 4];  // written by the producer wave that owns vf
  Ring ring[kRing + 1];   // the last slot takes the second producer wave's copies
};

// One stage's parts.
struct Stage {
  _Float16* k;
  _Float16* vt;
  float* kf;
  float* vf;
  uint32_t* emask;
  uint32_t* emask_spare;
};

__device__ __forceinline__ Stage stage(Smem& sm, int s) {
  return Stage{sm.k[s], sm.vt[s], sm.kf[s], sm.vf[s], sm.emask[s], sm.emask_spare[s]};
}

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

// ---------------------------------------------------------------------------
// INT8 -> FP16: bias each byte to unsigned (v + 128), place it under the FP16
// exponent of 1024 (bit pattern 0x64XX = 1024 + XX), subtract 1152 exactly.
__device__ __forceinline__ half2 biased_pair_to_half2(uint32_t pair_bits) {
  half2 h = __builtin_bit_cast(half2, pair_bits);
  return h - half2{(_Float16)1152.f, (_Float16)1152.f};
}

// four int8 in one dword -> the FP16 bit patterns of k + 1152 (exact), two per
// dword. The K tile keeps this bias: the S^T accumulator starts at
// -1152 * sum_d q_d instead of 0, which removes it (see consume()).
__device__ __forceinline__ uint2 i8x4_to_biased_half(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  return uint2{__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u),
               __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)};
}

// ---------------------------------------------------------------------------
// LDS tile layouts. Both are XOR-swizzled in 16-byte units so that the
// producers' stores and the consumers' MFMA-operand loads are free of bank
// conflicts (8 consecutive lanes always touch 8 distinct units of a 128-byte
// bank period).
//
// K tile [cell][dim], 16 units of 8 dims per cell row. Unit u (dims 8u..8u+7)
// of cell c lives at rot(u) ^ (c & 15), rot(u) = ((u & 1) << 3) | (u >> 1).
// Consumers load unit 2ks+hb of 8 consecutive cells; producers store units 2p
// and 2p+1 (p = 0..7) of one cell.
__device__ __forceinline__ int k_unit(int u, int cell) {
  return (((u & 1) << 3) | (u >> 1)) ^ (cell & 15);
}

// V^T tile [dim][slot], 8 units of 8 cells per dim row. Unit w = 4ch + 2ks + hb
// holds cells 16(2ch+ks) + 4hb + {0..3} then the same + 8: the order in which a
// lane of the S^T accumulator holds its cells, so P^T feeds the PV MFMA from
// registers. Unit w of dim d lives at w ^ vswz(d), vswz(d) = (d ^ (d >> 3)) & 7.
// Consumers load unit w of 8 consecutive dims; producers store unit w of dims
// 8k + jd for 8 consecutive k.
__device__ __forceinline__ int v_unit(int w, int d) { return w ^ ((d ^ (d >> 3)) & 7); }

// first cell of the k-th 4-cell quad (k = 0, 1) held by V^T unit w
__device__ __forceinline__ int v_unit_cell(int w, int k) {
  return 16 * (w >> 1) + 4 * (w & 1) + 8 * k;
}

// ---------------------------------------------------------------------------
// Producer staging tasks. K task t in [0,512): cell t>>3, dims 16*(t&7)..+15 (one
// 16-byte load). V task t in [0,128): unit w = t>>4 (eight cells), dims
// 8*(t&15)..+7 (eight 8-byte loads, transposed to eight dims x eight cells).
// Unusable cells (padding, non-resident, bad) read pool row 0, which always
// exists; their chooser byte and scales are 0, so the values never count.
// A scale is zeroed exactly when its cell's chooser byte is 0 (such a cell
// contributes nothing either way).
__device__ __forceinline__ u32x4 load_k_task(const PrefillArgs& a, const Ring& rg, int t) {
  const uint32_t off = rg.off[t >> 3] + 16u * (t & 7);
  return *reinterpret_cast<const u32x4*>(a.k_pool + off);
}

__device__ __forceinline__ void store_k_task(const Stage& st, int t, u32x4 raw) {
  const int cell = t >> 3;
  const int u0 = 2 * (t & 7);
  const uint2 b0 = i8x4_to_biased_half(raw.x), b1 = i8x4_to_biased_half(raw.y);
  const uint2 b2 = i8x4_to_biased_half(raw.z), b3 = i8x4_to_biased_half(raw.w);
  const u32x4 a0 = u32x4{b0.x, b0.y, b1.x, b1.y};
  const u32x4 a1 = u32x4{b2.x, b2.y, b3.x, b3.y};
  _Float16* base = st.k + cell * kD;
  *reinterpret_cast<u32x4*>(base + (k_unit(u0, cell) << 3)) = a0;
  *reinterpret_cast<u32x4*>(base + (k_unit(u0 + 1, cell) << 3)) = a1;
}

struct VRaw {
  u32x4 lo0, lo1;   // dims 8dq..8dq+3 of the unit's first / second cell quad
  u32x4 hi0, hi1;   // dims 8dq+4..8dq+7
};

__device__ __forceinline__ VRaw load_v_task(const PrefillArgs& a, const Ring& rg, int t) {
  const int w = t >> 4;
  const uint32_t d8 = 8u * (t & 15);
  const u32x4 o0 = *reinterpret_cast<const u32x4*>(rg.off + v_unit_cell(w, 0));
  const u32x4 o1 = *reinterpret_cast<const u32x4*>(rg.off + v_unit_cell(w, 1));
  VRaw r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint2 x = *reinterpret_cast<const uint2*>(a.v_pool + o0[k] + d8);
    const uint2 y = *reinterpret_cast<const uint2*>(a.v_pool + o1[k] + d8);
    r.lo0[k] = x.x;
    r.hi0[k] = x.y;
    r.lo1[k] = y.x;
    r.hi1[k] = y.y;
  }
  return r;
}

// four int8 dwords (cells 0..3, bytes = dims 0..3) -> for each dim jd the four
// cells' halves, via a 4x4 byte transpose and the biased FP16 trick.
__device__ __forceinline__ void transpose_quad(u32x4 raw, half4 out[4]) {
  const uint32_t w0 = raw.x ^ 0x80808080u, w1 = raw.y ^ 0x80808080u;
  const uint32_t w2 = raw.z ^ 0x80808080u, w3 = raw.w ^ 0x80808080u;
  const uint32_t t01lo = __builtin_amdgcn_perm(w1, w0, 0x05010400u);  // c0d0 c1d0 c0d1 c1d1
  const uint32_t t01hi = __builtin_amdgcn_perm(w1, w0, 0x07030602u);  // c0d2 c1d2 c0d3 c1d3
  const uint32_t t23lo = __builtin_amdgcn_perm(w3, w2, 0x05010400u);
  const uint32_t t23hi = __builtin_amdgcn_perm(w3, w2, 0x07030602u);
  const uint32_t src01[2] = {t01lo, t01hi};
  const uint32_t src23[2] = {t23lo, t23hi};
#pragma unroll
  for (int jd = 0; jd < 4; ++jd) {
    const uint32_t sel = (jd & 1) ? 0x04030402u : 0x04010400u;
    const half2 a01 = biased_pair_to_half2(__builtin_amdgcn_perm(0x64646464u, src01[jd >> 1], sel));
    const half2 a23 = biased_pair_to_half2(__builtin_amdgcn_perm(0x64646464u, src23[jd >> 1], sel));
    out[jd] = half4{a01.x, a01.y, a23.x, a23.y};
  }
}

__device__ __forceinline__ void store_v_task(const Stage& st, int t, const VRaw& raw) {
  const int w = t >> 4;
  const int d0 = 8 * (t & 15);
  half4 a0[4], a1[4], b0[4], b1[4];
  transpose_quad(raw.lo0, a0);
  transpose_quad(raw.lo1, a1);
  transpose_quad(raw.hi0, b0);
  transpose_quad(raw.hi1, b1);
#pragma unroll
  for (int jd = 0; jd < 4; ++jd) {
    const int d = d0 + jd;
    *reinterpret_cast<half8*>(st.vt + d * kChunk + (v_unit(w, d) << 3)) =
        half8{a0[jd].x, a0[jd].y, a0[jd].z, a0[jd].w, a1[jd].x, a1[jd].y, a1[jd].z, a1[jd].w};
    const int e = d0 + 4 + jd;
    *reinterpret_cast<half8*>(st.vt + e * kChunk + (v_unit(w, e) << 3)) =
        half8{b0[jd].x, b0[jd].y, b0[jd].z, b0[jd].w, b1[jd].x, b1[jd].y, b1[jd].z, b1[jd].w};
  }
}

// ---------------------------------------------------------------------------
// Page translation of one chunk cell (one lane per cell), in three steps whose
// global reads are each consumed kLead iterations after they were issued (the
// same lead as the K/V gathers, so that no wait for an early read also waits
// for gathers still in flight): read the union entry, then the page-table
// entry, then form the pool row and publish it in the ring.
// Records carry only loaded words (each in a register of its own: packing a
// field next to another would read the in-flight load at once); whether an
// entry lies inside the union is recomputed from the chunk index.
struct UnionRec {
  int32_t cell;
  uint32_t mask;
};

struct PageRec {
  int32_t cell;
  uint32_t mask;
  int32_t page_raw;   // page_table entry (of page 0 when the cell is not in [0, n_ctx))
};

__device__ __forceinline__ bool in_union(int U, int cc, int lane) { return cc * kChunk + lane < U; }

// All steps are branch-free (clamped, always-valid addresses plus selects) so
// that a producer iteration stays one basic block.
__device__ __forceinline__ UnionRec read_union_entry(const PrefillArgs& a, int64_t ubase, int U,
                                                     int cc, int lane) {
  // union rows hold at least 8 entries, so index 0 is always readable
  const int64_t at = ubase + (in_union(U, cc, lane) ? cc * kChunk + lane : 0);
  UnionRec u;
  u.cell = a.union_cells[at];
  u.mask = a.union_mask[at];
  return u;
}

__device__ __forceinline__ PageRec read_page_entry(const PrefillArgs& a, const UnionRec& u) {
  PageRec p;
  p.cell = u.cell;
  p.mask = u.mask;
  const bool in_ctx = u.cell >= 0 && u.cell < a.n_ctx;
  p.page_raw = a.page_table[in_ctx ? (u.cell >> 6) : 0];
  return p;
}

__device__ __forceinline__ void finish_translation(const PrefillArgs& a, const PageRec& p, int U,
                                                   int cc, int h, Ring& rg, int lane,
                                                   uint32_t& flags) {
  const bool valid = in_union(U, cc, lane);
  const bool in_ctx = valid && p.cell >= 0 && p.cell < a.n_ctx;
  const int32_t page = in_ctx ? p.page_raw : -1;
  const bool cell_bad = valid && !in_ctx;
  const bool page_bad = in_ctx && (page >= a.n_pages || page < -1);
  flags |= (cell_bad ? SEL_ATTN_STATUS_CELL_RANGE : 0u) | (page_bad ? SEL_ATTN_STATUS_PAGE_RANGE : 0u);
  const bool usable = in_ctx && !page_bad && page >= 0;
  const uint32_t row = (uint32_t)((page * a.n_kv + h) * 64 + (p.cell & 63));
  rg.off[lane] = usable ? row * kD : 0u;
  rg.mask[lane] = (uint8_t)(usable ? p.mask : 0u);
}

// ---------------------------------------------------------------------------
// Consumer waves 0..5: row block rb = w % 3 (32 rows), cell half ch = w / 3.
__device__ __forceinline__ float16v scores_t(const Stage& st, const half8 qf[8], int ch, int hb,
                                             int l32, float s_init) {
  float16v s;
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = s_init;
  const int cell = 32 * ch + l32;
  const _Float16* krow = st.k + cell * kD;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const half8 ka = *reinterpret_cast<const half8*>(krow + (k_unit(2 * ks + hb, cell) << 3));
    s = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qf[ks], s, 0, 0, 0);
  }
  return s;
}

// O^T (128 dims x 32 rows) += V^T (dims x this wave's 32 cells) P'^T
__device__ __forceinline__ void pv_accumulate(const Stage& st, const half8 pb[2], float16v o[4],
                                              int ch, int hb, int l32) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int d = 32 * mb + l32;
      const int w = 4 * ch + 2 * ks + hb;
      const half8 va = *reinterpret_cast<const half8*>(st.vt + d * kChunk + (v_unit(w, d) << 3));
      o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb[ks], o[mb], 0, 0, 0);
    }
  }
}

__device__ __forceinline__ void consume(const PrefillArgs& a, Smem& sm, int g, int h,
                                        int nch, int wave, int lane) {
  const int rb = wave % 3;
  const int ch = wave / 3;
  const int hb = lane >> 5;
  const int l32 = lane & 31;
  const int n_qh = a.n_kv * kQPerKv;

  // this lane's row: query head h*12 + hq, query index 8g + i
  const int row_n = 32 * rb + l32;
  const int hq = row_n >> 3;
  const int qi = 8 * g + (row_n & 7);
  const bool row_ok = qi < a.n_q;

  // Q^T as the B operand of S^T = K Q^T: k-step s covers dims 16s..16s+15,
  // this lane holds dims 16s + 8hb .. +7 of its row.
  half8 qf[8];
  {
    const float* qrow = a.q + ((int64_t)(row_ok ? qi : 0) * n_qh + h * kQPerKv + hq) * kD;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      float4v x0 = *reinterpret_cast<const float4v*>(qrow + 16 * s + 8 * hb);
      float4v x1 = *reinterpret_cast<const float4v*>(qrow + 16 * s + 8 * hb + 4);
      if (!row_ok) x0 = x1 = float4v{0.f, 0.f, 0.f, 0.f};
      qf[s] = half8{(_Float16)x0.x, (_Float16)x0.y, (_Float16)x0.z, (_Float16)x0.w,
                    (_Float16)x1.x, (_Float16)x1.y, (_Float16)x1.z, (_Float16)x1.w};
    }
  }

  // the K tile holds k + 1152: start every S^T accumulator at -1152 * sum_d q_d
  // of this lane's row (its 64 dims here, the other 64 in lane ^ 32)
  float qsum = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) qsum += (float)qf[s][e];
  const float s_init = -1152.f * (qsum + __shfl_xor(qsum, 32));

  lds_barrier();   // prologue: ring filled
  lds_barrier();   // prologue: chunks 0 and 1 staged, stage 3's V^T zeroed

  // running softmax state of this lane's row (over this wave's cell half)
  float m_run = kNoMax;
  float l_run = 0.f;
  float16v o[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[mb][r] = 0.f;
  const float ninf = -__builtin_inff();

  // Software pipeline: iteration c issues the MFMAs of S^T(c+1) and of
  // O^T += V^T P^T for chunk c-1 (whose P^T is already in registers), then runs
  // the softmax of chunk c on the VALU while those MFMAs execute. The first
  // iteration multiplies a zeroed P^T with stage 3's V^T (zero-filled by the
  // producers); the last one computes a discarded S^T.
  float16v s_cur = scores_t(stage(sm, 0), qf, ch, hb, l32, s_init);
  half8 pb[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) pb[ks][e] = (_Float16)0.f;

  for (int c = 0; c < nch; ++c) {
    const Stage st = stage(sm, c % kStages);
    const Stage st_prev = stage(sm, (c + kStages - 1) % kStages);
    const Stage st_next = stage(sm, (c + 1) % kStages);

    // ---- phase 1: LDS reads of chunk c's chooser bytes and factors and of
    // chunk c-1's V^T operands
    const u32x4 em_lo = *reinterpret_cast<const u32x4*>(st.emask + 8 * ch);
    const u32x4 em_hi = *reinterpret_cast<const u32x4*>(st.emask + 8 * ch + 4);
    float4v k4[4], v4[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      k4[q4] = *reinterpret_cast<const float4v*>(st.kf + 32 * ch + 8 * q4 + 4 * hb);
      v4[q4] = *reinterpret_cast<const float4v*>(st.vf + 32 * ch + 8 * q4 + 4 * hb);
    }
    half8 frag[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ks = i >> 2, mb = i & 3;
      const int d = 32 * mb + l32;
      frag[i] = *reinterpret_cast<const half8*>(st_prev.vt + d * kChunk +
                                                (v_unit(4 * ch + 2 * ks + hb, d) << 3));
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- phase 2: softmax of chunk c (VALU) interleaved with O^T += V^T P^T
    // of chunk c-1 (MFMA)
    uint32_t em[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      em[k] = __builtin_amdgcn_readfirstlane(em_lo[k]);
      em[4 + k] = __builtin_amdgcn_readfirstlane(em_hi[k]);
    }
    bool keep[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t lo = (em[2 * (r >> 2)] >> (8 * (r & 3))) & 0xffu;
      const uint32_t hi = (em[2 * (r >> 2) + 1] >> (8 * (r & 3))) & 0xffu;
      const uint64_t lm = (uint64_t)(lo * 0x01010101u) | ((uint64_t)(hi * 0x01010101u) << 32);
      keep[r] = __builtin_amdgcn_inverse_ballot_w64(lm);
    }
    float psum = 0.f;
    half8 pn[2];   // this chunk's P'^T (pb still feeds chunk c-1's MFMAs)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float u = keep[r] ? __builtin_fmaf(s_cur[r], k4[r >> 2][r & 3], -m_run) : ninf;
      const float pr = __builtin_amdgcn_exp2f(u);
      psum += pr;
      pn[r >> 3][r & 7] = (_Float16)(pr * v4[r >> 2][r & 3]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      o[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(frag[i], pb[i >> 2], o[i & 3], 0, 0, 0);

    // ---- phase 3: chunk c+1's K operands (loaded as phase 2's MFMAs free
    // their registers), its S^T chain interleaved with packing chunk c's P'^T
    half8 kfrag[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int cell = 32 * ch + l32;
      kfrag[ks] = *reinterpret_cast<const half8*>(st_next.k + cell * kD +
                                                  (k_unit(2 * ks + hb, cell) << 3));
    }
    float16v s_next;
#pragma unroll
    for (int r = 0; r < 16; ++r) s_next[r] = s_init;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      s_next = __builtin_amdgcn_mfma_f32_32x32x16_f16(kfrag[ks], qf[ks], s_next, 0, 0, 0);
    pb[0] = pn[0];
    pb[1] = pn[1];
    // schedule: PV MFMAs each followed by one K-operand load and a slice of
    // the softmax, then the S^T chain
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
      __builtin_amdgcn_sched_group_barrier(0x402, 7, 0);   // VALU incl. transcendental
      __builtin_amdgcn_sched_group_barrier(0x004, 5, 0);   // SALU
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);   // VALU
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- phase 4: the lazy stabiliser check
    if (__ballot(!(psum <= kLazyLimit))) {
      // the running maximum moves: rescale what is accumulated (this waits
      // for the MFMAs issued above) and redo the chunk against the new maximum
      // (its factors are read again from the stage, which is still intact)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        k4[q4] = *reinterpret_cast<const float4v*>(st.kf + 32 * ch + 8 * q4 + 4 * hb);
        v4[q4] = *reinterpret_cast<const float4v*>(st.vf + 32 * ch + 8 * q4 + 4 * hb);
      }
      float cmax = ninf;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        cmax = fmaxf(cmax, keep[r] ? s_cur[r] * k4[r >> 2][r & 3] : ninf);
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
      const float m_new = fmaxf(m_run, cmax);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[mb][r] *= alpha;
      psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float u = keep[r] ? __builtin_fmaf(s_cur[r], k4[r >> 2][r & 3], -m_run) : ninf;
        const float pr = __builtin_amdgcn_exp2f(u);
        psum += pr;
        pb[r >> 3][r & 7] = (_Float16)(pr * v4[r >> 2][r & 3]);
      }
    }
    l_run += psum;
    s_cur = s_next;
    lds_barrier();
  }
  // the last chunk's P'^T
  if (nch > 0) pv_accumulate(stage(sm, (nch - 1) % kStages), pb, o, ch, hb, l32);
  lds_barrier();   // every wave is done with the tiles the merge reuses

  // ---- merge the two cell halves of each row block and write the output
  float* xo = reinterpret_cast<float*>(&sm.k[0][0]);   // [3][16 float4 groups][64 lanes][4]
  float* xm = xo + 3 * 64 * 64;                      // [3][64]
  float* xl = xm + 3 * 64;                           // [3][64]
  if (ch == 1) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4v v = {o[mb][4 * q4], o[mb][4 * q4 + 1], o[mb][4 * q4 + 2], o[mb][4 * q4 + 3]};
        *reinterpret_cast<float4v*>(xo + ((rb * 16 + mb * 4 + q4) * 64 + lane) * 4) = v;
      }
    xm[rb * 64 + lane] = m_run;
    xl[rb * 64 + lane] = l_run;
  }
  lds_barrier();
  if (ch == 0) {
    const float m1 = xm[rb * 64 + lane];
    const float l1 = xl[rb * 64 + lane] + xl[rb * 64 + (lane ^ 32)];
    const float l0 = l_run + __shfl_xor(l_run, 32);
    const float mm = fmaxf(m_run, m1);
    const float a0 = __builtin_amdgcn_exp2f(m_run - mm);
    const float a1 = __builtin_amdgcn_exp2f(m1 - mm);
    const float lt = a0 * l0 + a1 * l1;
    const float inv = lt > 0.f ? (1.f / kVFold) / lt : 0.f;
    if (row_ok) {
      float* orow = a.out + ((int64_t)qi * n_qh + h * kQPerKv + hq) * kD;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4v o1 =
              *reinterpret_cast<const float4v*>(xo + ((rb * 16 + mb * 4 + q4) * 64 + lane) * 4);
          float4v r;
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = (a0 * o[mb][4 * q4 + e] + a1 * o1[e]) * inv;
          *reinterpret_cast<float4v*>(orow + 32 * mb + 8 * q4 + 4 * hb) = r;
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Producer waves 6..7 (128 threads, ptid = tid - 384). Iteration c (while the
// consumers work on chunks c and c+1): translate chunk c+4 (union entry read two
// iterations earlier, page entry one), gather chunk c+3 into registers, convert
// chunk c+2 (gathered one iteration earlier) into its LDS stage. Each thread
// owns K tasks ptid + 128k (k = 0..3) and V task ptid, and
// the k scale (ptid < 64) or v scale of cell ptid & 63; wave 6 translates.
struct Raw {
  u32x4 k[4];
  VRaw v;
  float sc;     // k scale (wave 6) or v scale (wave 7) of cell ptid & 63 (row 0's if unusable)
  uint32_t m;   // chooser byte of that cell; 0 if unusable
};

__device__ __forceinline__ void gather(const PrefillArgs& a, const Ring& rg, int ptid, Raw& r) {
#pragma unroll
  for (int k = 0; k < 4; ++k) r.k[k] = load_k_task(a, rg, ptid + 128 * k);
  r.v = load_v_task(a, rg, ptid);
  const int cell = ptid & 63;
  const float* sp = (ptid < kChunk) ? a.k_scale : a.v_scale;
  r.sc = sp[rg.off[cell] / kD];   // zeroed at conversion, when the load has landed
  r.m = rg.mask[cell];
}

__device__ __forceinline__ void convert(const PrefillArgs& a, const Stage& st, int ptid, const Raw& r,
                                        uint32_t& flags) {
#pragma unroll
  for (int k = 0; k < 4; ++k) store_k_task(st, ptid + 128 * k, r.k[k]);
  store_v_task(st, ptid, r.v);
  // wave 6 stores the k factors and chooser bytes, wave 7 the v factors (and
  // a spare copy of the chooser bytes), without a branch
  const bool kwave = ptid < kChunk;
  const int lane = ptid & 63;
  const float sc = r.m ? r.sc : 0.f;
  const bool v_ok = fabsf(sc) < kVScaleLimit;
  flags |= (!kwave && !v_ok) ? SEL_ATTN_STATUS_V_SCALE : 0u;
  const float mult = kwave ? a.score_scale : (v_ok ? kVFold : 0.f);
  (kwave ? st.kf : st.vf)[lane] = sc * mult;
  reinterpret_cast<uint8_t*>(kwave ? st.emask : st.emask_spare)[lane] = (uint8_t)r.m;
}

// Producer state, each array indexed by chunk & 3: gathered rows (chunk x is
// gathered in iteration x-2-kLead and converted in x-2), union records (read in
// x-4-3*kLead, consumed in x-4-2*kLead) and page records (read then, consumed
// in x-4-kLead, when the ring slot of chunk x is written). Every index below is
// a compile-time constant once a step is instantiated for its phase P = c & 3,
// so the sets stay in registers and the stage addresses fold into immediates.
constexpr int kAheadGather = 2 + kLead;        // chunk gathered in iteration c: c + 5
constexpr int kAheadFinish = 3 + kLead;        // ring slot written: c + 6
constexpr int kAheadPage = 3 + 2 * kLead;      // page entry read: c + 9
constexpr int kAheadUnion = 3 + 3 * kLead;     // union entry read: c + 12

struct ProdState {
  Raw raw[4];
  UnionRec un[4];
  PageRec pg[4];
};

// Iteration c (phase P = c & 3), while the consumers work on chunks c-1..c+1.
// Reads are issued union, page, gather (oldest consumer first), and each one
// issued here is consumed kLead iterations later.
template <int P>
__device__ __forceinline__ void produce_step(const PrefillArgs& a, Smem& sm, ProdState& ps, int c,
                                             int h, int U, int64_t ubase, int ptid, bool translator,
                                             uint32_t& flags) {
  const int lane = ptid & 63;
  ps.un[(P + kAheadUnion) & 3] = read_union_entry(a, ubase, U, c + kAheadUnion, lane);
  ps.pg[(P + kAheadPage) & 3] = read_page_entry(a, ps.un[(P + kAheadPage) & 3]);
  const int cf = c + kAheadFinish;
  finish_translation(a, ps.pg[(P + kAheadFinish) & 3], U, cf, h,
                     sm.ring[translator ? (cf & (kRing - 1)) : kRing], lane, flags);
  gather(a, sm.ring[(c + kAheadGather) & (kRing - 1)], ptid, ps.raw[(P + kAheadGather) & 3]);
  convert(a, stage(sm, (P + 2) & 3), ptid, ps.raw[(P + 2) & 3], flags);
  lds_barrier();
}

__device__ __forceinline__ void produce(const PrefillArgs& a, Smem& sm, int h, int U, int nch,
                                        int64_t ubase, int ptid, bool translator,
                                        uint32_t& flags) {
  static_assert(kLead >= 1 && kLead <= 3 && kStages == 4 && kAheadFinish <= kRing,
                "register sets and ring slots cover the lead");
  const int lane = ptid & 63;
  ProdState ps;
  // prologue: what iteration 0 expects. Chunks below kAheadFinish translated
  // into their ring slots; page records of the next kLead chunks and union
  // records of the kLead after those read; chunks 0 and 1 staged, chunks 2 ..
  // kAheadGather-1 gathered. Both producer waves translate the same lanes;
  // wave 7 writes its copy to the spare slot.
  {
    UnionRec u[kAheadPage];
#pragma unroll
    for (int i = 0; i < kAheadPage; ++i) u[i] = read_union_entry(a, ubase, U, i, lane);
#pragma unroll
    for (int i = kAheadPage; i < kAheadUnion; ++i) ps.un[i & 3] = read_union_entry(a, ubase, U, i, lane);
    PageRec p[kAheadFinish];
#pragma unroll
    for (int i = 0; i < kAheadFinish; ++i) p[i] = read_page_entry(a, u[i]);
#pragma unroll
    for (int i = kAheadFinish; i < kAheadPage; ++i) ps.pg[i & 3] = read_page_entry(a, u[i]);
#pragma unroll
    for (int i = 0; i < kAheadFinish; ++i)
      finish_translation(a, p[i], U, i, h, sm.ring[translator ? i : kRing], lane, flags);
  }
  // stage 3's V^T meets a zeroed P^T in the consumers' first iteration: keep
  // it finite
  {
    u32x4* z = reinterpret_cast<u32x4*>(sm.vt[kStages - 1]);
#pragma unroll
    for (int i = 0; i < (kD * kChunk * 2) / (16 * 128); ++i) z[ptid + 128 * i] = u32x4{0u, 0u, 0u, 0u};
  }
  lds_barrier();
#pragma unroll
  for (int x = 0; x < kAheadGather; ++x) {
    if (x >= 4) convert(a, stage(sm, x - 4), ptid, ps.raw[x & 3], flags);   // frees the set
    gather(a, sm.ring[x], ptid, ps.raw[x & 3]);
  }
#pragma unroll
  for (int x = (kAheadGather > 4 ? kAheadGather - 4 : 0); x < 2; ++x)
    convert(a, stage(sm, x), ptid, ps.raw[x & 3], flags);
  lds_barrier();

  int c = 0;
  for (; c + 4 <= nch; c += 4) {
    produce_step<0>(a, sm, ps, c, h, U, ubase, ptid, translator, flags);
    produce_step<1>(a, sm, ps, c + 1, h, U, ubase, ptid, translator, flags);
    produce_step<2>(a, sm, ps, c + 2, h, U, ubase, ptid, translator, flags);
    produce_step<3>(a, sm, ps, c + 3, h, U, ubase, ptid, translator, flags);
  }
  const int rem = nch - c;   // 0..3 more iterations, phases 0, 1, 2
  if (rem > 0) produce_step<0>(a, sm, ps, c, h, U, ubase, ptid, translator, flags);
  if (rem > 1) produce_step<1>(a, sm, ps, c + 1, h, U, ubase, ptid, translator, flags);
  if (rem > 2) produce_step<2>(a, sm, ps, c + 2, h, U, ubase, ptid, translator, flags);
  lds_barrier();   // consumers finish their last O^T update
  lds_barrier();   // merge of the consumers' two cell halves
}

__global__ __launch_bounds__(kThreads) void sel_attn_prefill_kernel(PrefillArgs a) {
  __shared__ Smem sm;

  const int b = blockIdx.x;
  const int L = (b & 7) * a.per_xcd + (b >> 3);
  if (L >= a.n_groups * a.n_kv) return;
  const int h = L / a.n_groups;
  const int g = L - h * a.n_groups;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t ucap = 8LL * a.sel_cap;
  const int64_t ubase = (int64_t)g * ucap;
  uint32_t flags = 0;

  int U = a.union_len[g];
  if (U < 0 || U > ucap) {
    flags |= SEL_ATTN_STATUS_UNION_LEN;
    U = U < 0 ? 0 : (int)ucap;
  }
  const int nch = (U + kChunk - 1) / kChunk;   // 64-cell chunks of the union

  if (wave < kConsumerWaves) {
    consume(a, sm, g, h, nch, wave, lane);
  } else {
    const int ptid = tid - 64 * kConsumerWaves;
    produce(a, sm, h, U, nch, ubase, ptid, wave == kConsumerWaves, flags);
  }
  if (flags) atomicOr(a.status, flags);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const int grid = 8 * a.per_xcd;
  hipLaunchKernelGGL(sel_attn_prefill_kernel, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace selattn
