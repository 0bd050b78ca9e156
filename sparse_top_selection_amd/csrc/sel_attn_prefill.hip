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
//   * one 384-thread workgroup (6 wave64s) per (group g, KV head h); grid order
//     is XCD-aware so that each XCD walks consecutive groups of one KV head;
//   * row n of the 96 = 8*hq + i (query head h*12+hq, position 8g+i), so the
//     chooser bit of row n is n & 7; wave w owns row block rb = w % 3 (32 rows)
//     and cell half ch = w / 3 (32 of the chunk's 64 cells) with its own softmax
//     state; the two halves are merged once at the end;
//   * S^T (32 cells x 32 rows, K=128) is 8 v_mfma_f32_32x32x16_f16 from an LDS K
//     tile and Q^T held in registers; O^T (128 dims x 32 rows) += V^T P^T is 8
//     more MFMAs whose B operand (P^T) comes straight from the S^T accumulator
//     registers: the V^T tile in LDS is stored in the matching cell permutation;
//   * K and V integers are exact in FP16, so the scales are applied in FP32:
//     k_scale * softmax_scale * log2(e) multiplies the score, v_scale * 2^10 the
//     probability before its FP16 rounding (2^-10 returns in the epilogue);
//   * the chooser byte of a cell becomes a 64-bit SGPR lane mask (the byte
//     replicated 4x per 32 lanes) and one v_cndmask applies it per score;
//   * online softmax with a lazy stabiliser: probabilities are taken against
//     the running maximum, and only when a lane's chunk sum exceeds 16 does the
//     wave recompute the chunk maximum and rescale O and l (always on a row's
//     first chosen chunk, rarely after);
//   * a chunk's INT8 K/V are gathered through the page table with 16-byte loads
//     one chunk ahead (and the page translation two chunks ahead), converted
//     to FP16 in registers (byte permute + magic-number subtract, V transposed
//     4x4 on the way) and written to the other half of a double-buffered tile.

#include "sel_attn_internal.h"

namespace selattn {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 6;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 64;        // union cells per iteration
constexpr int kD = 128;           // head dim
constexpr int kQPerKv = 12;
constexpr float kLazyLimit = 16.f;
constexpr float kNoMax = -1e30f;  // stabiliser before a row has seen a chosen cell
constexpr float kVFold = 1024.f;  // probabilities carry v_scale * 2^10 into FP16
constexpr float kVScaleLimit = 4.f;

struct __align__(16) Stage {
  _Float16 k[kChunk * kD];   // [cell][dim]; 16-byte unit u of a row stored at u ^ (cell & 15)
  _Float16 vt[kD * kChunk];  // [dim][slot]; 16-byte unit w of a row stored at w ^ (dim & 7)
  float kf[kChunk];          // k_scale * softmax_scale * log2(e); 0 where unusable
  float vf[kChunk];          // v_scale * 2^10; 0 where unusable
  uint32_t emask[kChunk / 4];  // chooser bytes, 0 for padding / non-resident cells
};

struct Ring {
  int32_t row[kChunk];       // pool row (phys * n_kv + h) * 64 + slot; -1 = unusable
  uint8_t mask[kChunk];
};

struct __align__(16) Smem {
  Stage st[2];
  Ring ring[2];
};

// ---------------------------------------------------------------------------
// INT8 -> FP16: bias each byte to unsigned (v + 128), place it under the FP16
// exponent of 1024 (bit pattern 0x64XX = 1024 + XX), subtract 1152 exactly.
__device__ __forceinline__ half2 biased_pair_to_half2(uint32_t pair_bits) {
  half2 h = __builtin_bit_cast(half2, pair_bits);
  return h - half2{(_Float16)1152.f, (_Float16)1152.f};
}

// four int8 in one dword -> four halves (bytes 0..3 in order)
__device__ __forceinline__ half4 i8x4_to_half4(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  const half2 lo = biased_pair_to_half2(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u));
  const half2 hi = biased_pair_to_half2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u));
  return half4{lo.x, lo.y, hi.x, hi.y};
}

// ---------------------------------------------------------------------------
// Staging tasks. K task t in [0,512): cell t>>3, dims 16*(t&7)..+15 (one 16-byte
// load). V task t in [0,512): cells 4*(t>>5)..+3, dims 4*(t&31)..+3 (four dword
// loads, transposed to four dims x four cells).
__device__ __forceinline__ u32x4 load_k_task(const PrefillArgs& a, const Ring& rg, int t) {
  const int row = rg.row[t >> 3];
  if (row < 0) return u32x4{0u, 0u, 0u, 0u};
  const u32x4* p = reinterpret_cast<const u32x4*>(a.k_pool + (int64_t)row * kD + 16 * (t & 7));
  return *p;
}

__device__ __forceinline__ void store_k_task(Stage& st, int t, u32x4 raw) {
  const int cell = t >> 3;
  const int u0 = 2 * (t & 7);
  const half4 h0 = i8x4_to_half4(raw.x), h1 = i8x4_to_half4(raw.y);
  const half4 h2 = i8x4_to_half4(raw.z), h3 = i8x4_to_half4(raw.w);
  const half8 a0 = half8{h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
  const half8 a1 = half8{h2.x, h2.y, h2.z, h2.w, h3.x, h3.y, h3.z, h3.w};
  _Float16* base = st.k + cell * kD;
  *reinterpret_cast<half8*>(base + ((u0 ^ (cell & 15)) << 3)) = a0;
  *reinterpret_cast<half8*>(base + (((u0 + 1) ^ (cell & 15)) << 3)) = a1;
}

__device__ __forceinline__ u32x4 load_v_task(const PrefillArgs& a, const Ring& rg, int t) {
  const int c0 = 4 * (t >> 5);
  const int dq = t & 31;
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int row = rg.row[c0 + k];
    uint32_t w = 0u;
    if (row >= 0)
      w = reinterpret_cast<const uint32_t*>(a.v_pool + (int64_t)row * kD)[dq];
    r[k] = w;
  }
  return r;
}

// V^T slot layout: within a row (one dim), 16-byte unit w = 4*ch + 2*ks + hb
// holds cells 32ch + 16ks + 4hb + {0..3} then 32ch + 16ks + 8 + 4hb + {0..3},
// which is the order in which an S^T accumulator lane holds its cells.
__device__ __forceinline__ void store_v_task(Stage& st, int t, u32x4 raw) {
  const int c0 = 4 * (t >> 5);     // first of four consecutive cells
  const int d0 = 4 * (t & 31);
  const int w = ((c0 >> 5) << 2) | (((c0 >> 4) & 1) << 1) | ((c0 >> 2) & 1);
  const int sub = ((c0 >> 3) & 1) << 2;   // first or second half of the unit
  // 4x4 byte transpose: t01 = cells 0,1 interleaved, t23 = cells 2,3 interleaved
  const uint32_t w0 = raw.x ^ 0x80808080u, w1 = raw.y ^ 0x80808080u;
  const uint32_t w2 = raw.z ^ 0x80808080u, w3 = raw.w ^ 0x80808080u;
  const uint32_t t01lo = __builtin_amdgcn_perm(w1, w0, 0x05010400u);
  const uint32_t t01hi = __builtin_amdgcn_perm(w1, w0, 0x07030602u);
  const uint32_t t23lo = __builtin_amdgcn_perm(w3, w2, 0x05010400u);
  const uint32_t t23hi = __builtin_amdgcn_perm(w3, w2, 0x07030602u);
  const uint32_t src01[2] = {t01lo, t01hi};
  const uint32_t src23[2] = {t23lo, t23hi};
#pragma unroll
  for (int jd = 0; jd < 4; ++jd) {
    const uint32_t sel = (jd & 1) ? 0x04030402u : 0x04010400u;
    const half2 a01 = biased_pair_to_half2(__builtin_amdgcn_perm(0x64646464u, src01[jd >> 1], sel));
    const half2 a23 = biased_pair_to_half2(__builtin_amdgcn_perm(0x64646464u, src23[jd >> 1], sel));
    const int d = d0 + jd;
    *reinterpret_cast<half4*>(st.vt + d * kChunk + ((w ^ (d & 7)) << 3) + sub) =
        half4{a01.x, a01.y, a23.x, a23.y};
  }
}

// Page translation for chunk cc, split in two so the union read overlaps work.
struct Pending {
  int32_t cell;
  uint32_t mask;
  bool valid;
};

__device__ __forceinline__ Pending translate_issue(const PrefillArgs& a, int64_t ubase, int U,
                                                   int cc, int tid) {
  Pending p{0, 0u, false};
  const int idx = cc * kChunk + tid;
  if (idx < U) {
    p.cell = a.union_cells[ubase + idx];
    p.mask = a.union_mask[ubase + idx];
    p.valid = true;
  }
  return p;
}

__device__ __forceinline__ void translate_finish(const PrefillArgs& a, const Pending& p, int h,
                                                 Ring& rg, int tid, uint32_t& flags) {
  int32_t row = -1;
  if (p.valid) {
    if (p.cell < 0 || p.cell >= a.n_ctx) {
      flags |= SEL_ATTN_STATUS_CELL_RANGE;
    } else {
      const int32_t pp = a.page_table[p.cell >> 6];
      if (pp >= a.n_pages || pp < -1) {
        flags |= SEL_ATTN_STATUS_PAGE_RANGE;
      } else if (pp >= 0) {
        row = (pp * a.n_kv + h) * 64 + (p.cell & 63);
      }
    }
  }
  rg.row[tid] = row;
  rg.mask[tid] = (row >= 0) ? (uint8_t)p.mask : (uint8_t)0;
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void sel_attn_prefill_kernel(PrefillArgs a) {
  __shared__ Smem sm;

  const int b = blockIdx.x;
  const int L = (b & 7) * a.per_xcd + (b >> 3);
  if (L >= a.n_groups * a.n_kv) return;
  const int h = L / a.n_groups;
  const int g = L - h * a.n_groups;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rb = wave % 3;          // row block: rows 32rb..32rb+31
  const int ch = wave / 3;          // cell half of every chunk
  const int hb = lane >> 5;         // which half of the wave
  const int l32 = lane & 31;
  const int n_qh = a.n_kv * kQPerKv;
  const int64_t ucap = 8LL * a.sel_cap;
  const int64_t ubase = (int64_t)g * ucap;
  uint32_t flags = 0;

  int U = a.union_len[g];
  if (U < 0 || U > ucap) {
    flags |= SEL_ATTN_STATUS_UNION_LEN;
    U = U < 0 ? 0 : (int)ucap;
  }
  const int nch = (U + kChunk - 1) / kChunk;

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
      float4v x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
      if (row_ok) {
        x0 = *reinterpret_cast<const float4v*>(qrow + 16 * s + 8 * hb);
        x1 = *reinterpret_cast<const float4v*>(qrow + 16 * s + 8 * hb + 4);
      }
      qf[s] = half8{(_Float16)x0.x, (_Float16)x0.y, (_Float16)x0.z, (_Float16)x0.w,
                    (_Float16)x1.x, (_Float16)x1.y, (_Float16)x1.z, (_Float16)x1.w};
    }
  }

  // staging task ids of this thread
  const int kA = tid;
  const int kB = tid + kThreads;            // valid for tid < 128
  const int vA = tid - 128;                 // valid for tid >= 128
  const int vB = tid + 256;                 // valid for tid < 256

  // prologue: translate chunks 0 and 1, stage chunk 0
  if (tid < kChunk) {
    Pending p0 = translate_issue(a, ubase, U, 0, tid);
    Pending p1 = translate_issue(a, ubase, U, 1, tid);
    translate_finish(a, p0, h, sm.ring[0], tid, flags);
    translate_finish(a, p1, h, sm.ring[1], tid, flags);
  }
  __syncthreads();

  u32x4 rkA, rkB, rvA, rvB;
  float sc = 0.f;
  auto issue_loads = [&](const Ring& rg) {
    rkA = load_k_task(a, rg, kA);
    if (tid < 128) rkB = load_k_task(a, rg, kB);
    if (tid >= 128) rvA = load_v_task(a, rg, vA);
    if (tid < 256) rvB = load_v_task(a, rg, vB);
    sc = 0.f;
    if (tid < 2 * kChunk) {
      const int row = rg.row[tid & 63];
      if (row >= 0) sc = (tid < kChunk) ? a.k_scale[row] : a.v_scale[row];
    }
  };
  auto finish_stage = [&](Stage& st, const Ring& rg) {
    store_k_task(st, kA, rkA);
    if (tid < 128) store_k_task(st, kB, rkB);
    if (tid >= 128) store_v_task(st, vA, rvA);
    if (tid < 256) store_v_task(st, vB, rvB);
    if (tid < kChunk) {
      st.kf[tid] = sc * a.score_scale;
      reinterpret_cast<uint8_t*>(st.emask)[tid] = rg.mask[tid];
    } else if (tid < 2 * kChunk) {
      float vf = sc * kVFold;
      if (!(fabsf(sc) < kVScaleLimit)) {
        flags |= SEL_ATTN_STATUS_V_SCALE;
        vf = 0.f;
      }
      st.vf[tid - kChunk] = vf;
    }
  };

  if (nch > 0) {
    issue_loads(sm.ring[0]);
    finish_stage(sm.st[0], sm.ring[0]);
  }
  __syncthreads();

  // running softmax state of this lane's row (over this wave's cell half)
  float m_run = kNoMax;
  float l_run = 0.f;
  float16v o[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[mb][r] = 0.f;

  const float ninf = -__builtin_inff();

  for (int c = 0; c < nch; ++c) {
    const Stage& st = sm.st[c & 1];
    Pending nx{0, 0u, false};
    if (c + 2 < nch && tid < kChunk) nx = translate_issue(a, ubase, U, c + 2, tid);
    if (c + 1 < nch) issue_loads(sm.ring[(c + 1) & 1]);

    // ---- S^T = K Q^T for cells 32ch..32ch+31 of the chunk
    float16v s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    {
      const int cell = 32 * ch + l32;
      const _Float16* krow = st.k + cell * kD;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const half8 ka = *reinterpret_cast<const half8*>(krow + (((2 * ks + hb) ^ (cell & 15)) << 3));
        s = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qf[ks], s, 0, 0, 0);
      }
    }

    // ---- chooser masks (wave-uniform) and per-cell factors
    uint32_t em[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) em[k] = __builtin_amdgcn_readfirstlane(st.emask[8 * ch + k]);
    float kf[16], vf[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4v k4 = *reinterpret_cast<const float4v*>(st.kf + 32 * ch + 8 * q4 + 4 * hb);
      const float4v v4 = *reinterpret_cast<const float4v*>(st.vf + 32 * ch + 8 * q4 + 4 * hb);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[4 * q4 + e] = k4[e];
        vf[4 * q4 + e] = v4[e];
      }
    }
    bool keep[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t lo = (em[2 * (r >> 2)] >> (8 * (r & 3))) & 0xffu;
      const uint32_t hi = (em[2 * (r >> 2) + 1] >> (8 * (r & 3))) & 0xffu;
      const uint64_t lm = (uint64_t)(lo * 0x01010101u) | ((uint64_t)(hi * 0x01010101u) << 32);
      keep[r] = __builtin_amdgcn_inverse_ballot_w64(lm);
    }

    // ---- masked online softmax (log2 domain)
    float p[16];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float u = keep[r] ? __builtin_fmaf(s[r], kf[r], -m_run) : ninf;
      p[r] = __builtin_amdgcn_exp2f(u);
      psum += p[r];
    }
    if (__ballot(!(psum <= kLazyLimit))) {
      float cmax = ninf;
#pragma unroll
      for (int r = 0; r < 16; ++r) cmax = fmaxf(cmax, keep[r] ? s[r] * kf[r] : ninf);
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
        const float u = keep[r] ? __builtin_fmaf(s[r], kf[r], -m_run) : ninf;
        p[r] = __builtin_amdgcn_exp2f(u);
        psum += p[r];
      }
    }
    l_run += psum;

    // ---- O^T += V^T P^T
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      half8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (_Float16)(p[8 * ks + e] * vf[8 * ks + e]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int d = 32 * mb + l32;
        const int w = 4 * ch + 2 * ks + hb;
        const half8 va = *reinterpret_cast<const half8*>(st.vt + d * kChunk + ((w ^ (d & 7)) << 3));
        o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb, o[mb], 0, 0, 0);
      }
    }

    if (c + 2 < nch && tid < kChunk) translate_finish(a, nx, h, sm.ring[c & 1], tid, flags);
    if (c + 1 < nch) finish_stage(sm.st[(c + 1) & 1], sm.ring[(c + 1) & 1]);
    __syncthreads();
  }

  // ---- merge the two cell halves of each row block and write the output
  float* xo = reinterpret_cast<float*>(&sm.st[0]);   // [3][16 float4 groups][64 lanes][4]
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
  __syncthreads();
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
          const float4v o1 = *reinterpret_cast<const float4v*>(xo + ((rb * 16 + mb * 4 + q4) * 64 + lane) * 4);
          float4v r;
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = (a0 * o[mb][4 * q4 + e] + a1 * o1[e]) * inv;
          *reinterpret_cast<float4v*>(orow + 32 * mb + 8 * q4 + 4 * hb) = r;
        }
    }
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
