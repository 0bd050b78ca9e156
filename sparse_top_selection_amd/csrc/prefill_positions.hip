// Per-position attention: every query position gathers its own selected cells,
// with no union. The output is the same as the union path's.
//
// Page: #2808 "sycl: prompt attention over 8-query selection unions on XMX".
// - Section Summary: the FP32 kernel in which every position gathers its own
//   ~2,051 selected cells. That is the definition both paths compute.
// - Section Extra Notes: the union path wins only where adjacent positions'
//   selections share cells and gains nothing when they are unrelated. This
//   kernel serves that case: its gather is each position's own cells, not a
//   union that can reach 8 times a selection.
//
// gfx950 design: one work-group per query position, 4 waves.
// Phase 1 (the whole work-group) turns the selection row into a list of pool
// rows, then the work-group synchronises once:
// - repeats are dropped through an LDS hash that keeps each cell's first entry
//   (a strictly ascending row, which has none, skips the hash);
// - cells out of range and non-resident pages are dropped;
// - the kept entries are compacted in row order.
// Phase 2: wave w handles KV heads w, w+4, ... (12 query rows each) over the
// list, in 32-cell chunks, with no barriers. Each chunk's rows are loaded two
// chunks ahead into registers (three register sets in rotation; two work-groups
// per CU, since a third would not leave the registers for the second chunk in
// flight):
// - K rows, 16 bytes a lane, already in the operand layout of S^T = K Q^T;
// - V rows, 16 bytes a lane, which go to the wave's LDS tile at the start of
//   the chunk's own step. Which lane loads which 16 bytes is chosen so that the
//   tile is swizzled, and the transposing byte read ds_read_b64_tr_b8 then
//   gives each lane 8 cells of one dim, free of bank conflicts;
// - one scale a lane (the k scales, then the v scales of the chunk's cells).
// Integers enter FP16 with the exact +1152 bias (two byte permutes per four
// values), and the bias terms are removed in FP32: S^T starts from -1152 sum(Q)
// of its row, O loses 1152 sum(P'). S^T and O^T = V^T P'^T run on
// v_mfma_f32_16x16x32_f16 (12 of 16 columns used). P' feeds the second product
// straight from the first's accumulator layout, in a cell order that V's
// transposing read reproduces.

#include "sel_attn_internal.h"

namespace selattn {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i* lds_v2i_t;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kD = 128;
constexpr int kQPerKv = 12;
constexpr int kChunk = 32;
constexpr int kHashSlots = 4096;          // dedup table (load factor <= 0.625)
constexpr int kPer = (SEL_ATTN_POSITIONS_MAX_CAP + kThreads - 1) / kThreads;  // entries per thread
constexpr float kVFold = 64.f;            // P' = p * v_scale * 2^6 in FP16
constexpr float kVScaleLimit = 4.f;
constexpr float kNoMax = -1e30f;

// LDS: per wave, one chunk's V rows (int8, 16-byte units swizzled) and its
// scales; in phase 1 the same bytes hold the dedup table. Then the position's
// kept cells, (page * n_kv) * 64 + slot.
struct __align__(16) WaveTile {
  uint8_t v[kChunk * kD];
  float sc[2 * kChunk];        // k scales of cells 0..31, then v scales
};
struct __align__(16) Smem {
  union {
    struct {
      int32_t key[kHashSlots];   // cell, or -1
      int32_t first[kHashSlots]; // lowest entry index holding the cell
    } hash;
    WaveTile tile[kWaves];
  } u;
  uint32_t rows[SEL_ATTN_POSITIONS_MAX_CAP];
  int32_t wave_count[2][kWaves];
};
static_assert(sizeof(Smem) <= 80 * 1024, "two work-groups per CU");

// A chunk's loads, held in registers until the chunk's step.
struct ChunkRegs {
  u32x4 k[2][2];   // K: cells 16t + i, dims 64q + 16g .. +15
  u32x4 v[4];      // V: cell 8m + (lane >> 3), unit (lane & 7) ^ vkey(cell)
  float sc;        // k scale (lane < 32) or v scale of cell lane & 31
};

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint32_t hash_slot(int32_t c) {
  return ((uint32_t)c * 2654435761u) >> 20;   // top 12 bits: [0, 4096)
}

// four int8 in one dword -> the FP16 bit patterns of x + 1152 (exact), two per
// dword: the byte, biased to unsigned, under the exponent of 1024 (0x64XX)
__device__ __forceinline__ uint2 biased_half4(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  return uint2{__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u),
               __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)};
}

__device__ __forceinline__ half8 biased_half8(uint32_t w0, uint32_t w1) {
  const uint2 a = biased_half4(w0), b = biased_half4(w1);
  return __builtin_bit_cast(half8, u32x4{a.x, a.y, b.x, b.y});
}

// Swizzle of a chunk's V tile: cell c's 16-byte unit u (dims 16u..16u+15) sits
// at unit position u ^ vkey(c) of the cell's 128-byte row. The eight cells a
// lane group reads together (4g+s for s < 4, 16+4g+s-4 for s >= 4) have keys
// 0..7, so their 8-byte reads cover all 32 banks once.
__device__ __forceinline__ int vkey(int c) { return (c & 3) | (((c >> 4) & 1) << 2); }

// Cell of the chunk behind k index 8g + s of the P'^T / V^T operands: the
// accumulator of S^T tile t holds cells 16t + 4g + i (i < 4) in lane group g.
__device__ __forceinline__ int operand_cell(int g, int s) {
  return s < 4 ? 4 * g + s : 16 + 4 * g + (s - 4);
}

// Loads of chunk c for KV head h into registers.
__device__ __forceinline__ void load_chunk(const PositionsArgs& a, const uint32_t* rows, int c,
                                           int n, int h, int lane, ChunkRegs& r) {
  const int g = lane >> 4, i = lane & 15;
  const uint32_t hoff = (uint32_t)h * 64u;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint32_t row = rows[min(kChunk * c + 16 * t + i, n - 1)] + hoff;
    const int8_t* src = a.k_pool + (size_t)row * kD + 16 * g;
#pragma unroll
    for (int q = 0; q < 2; ++q) r.k[t][q] = *reinterpret_cast<const u32x4*>(src + 64 * q);
  }
  // V: lane l fills unit position l & 7 of cell 8m + (l >> 3) of the tile, so
  // it loads that cell's unit (l & 7) ^ vkey(cell)
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int cc = 8 * m + (lane >> 3);
    const uint32_t row = rows[min(kChunk * c + cc, n - 1)] + hoff;
    r.v[m] = *reinterpret_cast<const u32x4*>(a.v_pool + (size_t)row * kD +
                                             16 * ((lane & 7) ^ vkey(cc)));
  }
  const uint32_t row = rows[min(kChunk * c + (lane & 31), n - 1)] + hoff;
  r.sc = (lane < 32 ? a.k_scale : a.v_scale)[row];
}

// Running state of one head's 12 rows (each lane: its row's share).
struct ChunkState {
  float4v o[8];   // O^T, dims 16mt + 4g .. +3 of row i, scaled by 2^6
  float m_run;    // running maximum (log2 domain)
  float l_run;    // this lane's share of the probability sum
  float lp;       // this lane's share of sum(P'), for the V bias
};

// Chunk c of KV head h from register set rc, while chunk c+2 (the last chunk
// again at the end, so that every step issues the same loads) goes into set rn.
__device__ __forceinline__ void chunk_step(const PositionsArgs& a, const uint32_t* rows,
                                           WaveTile& tile, ChunkState& st, int c, int nch, int n,
                                           int h, int lane, float s_init, const half8 (&qb)[4],
                                           const ChunkRegs& rc, ChunkRegs& rn, uint32_t& flags) {
  const int g = lane >> 4;
  // chunk c's V rows and scales into the tile (the previous step's reads of
  // it come first in the wave's LDS order)
#pragma unroll
  for (int m = 0; m < 4; ++m) *reinterpret_cast<u32x4*>(tile.v + 1024 * m + 16 * lane) = rc.v[m];
  tile.sc[lane] = rc.sc;
  load_chunk(a, rows, min(c + 2, nch - 1), n, h, lane, rn);

  // S^T tiles (16 cells x 16 rows), starting from the bias term
  float4v s[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    s[t] = float4v{s_init, s_init, s_init, s_init};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const u32x4 w = rc.k[t][q];
      s[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(biased_half8(w.x, w.y), qb[2 * q], s[t], 0, 0, 0);
      s[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(biased_half8(w.z, w.w), qb[2 * q + 1], s[t], 0, 0, 0);
    }
  }

  // log2-domain scores of this lane's 8 cells (tile t, cells 16t + 4g + e)
  const float* sc = tile.sc;
  const float4v ks0 = *reinterpret_cast<const float4v*>(sc + 4 * g);
  const float4v ks1 = *reinterpret_cast<const float4v*>(sc + 16 + 4 * g);
  const float4v vs0 = *reinterpret_cast<const float4v*>(sc + kChunk + 4 * g);
  const float4v vs1 = *reinterpret_cast<const float4v*>(sc + kChunk + 16 + 4 * g);
  float u[8], vf[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int c0 = kChunk * c + 4 * g + e, c1 = c0 + 16;
    u[e] = c0 < n ? s[0][e] * (ks0[e] * a.score_scale) : -__builtin_inff();
    u[4 + e] = c1 < n ? s[1][e] * (ks1[e] * a.score_scale) : -__builtin_inff();
    vf[e] = vs0[e];
    vf[4 + e] = vs1[e];
  }
  float cmax = u[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) cmax = fmaxf(cmax, u[e]);
  cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
  cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
  const float m_new = fmaxf(st.m_run, cmax);
  if (__ballot(m_new > st.m_run)) {
    const float alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);
    st.l_run *= alpha;
    st.lp *= alpha;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) st.o[mt] *= alpha;
    st.m_run = m_new;
  }
  half8 pb;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = __builtin_amdgcn_exp2f(u[e] - st.m_run);
    const bool v_ok = fabsf(vf[e]) < kVScaleLimit;
    flags |= v_ok ? 0u : SEL_ATTN_STATUS_V_SCALE;
    st.l_run += p;
    const _Float16 pv = (_Float16)(v_ok ? p * (vf[e] * kVFold) : 0.f);
    pb[e] = pv;
    st.lp += (float)pv;
  }

  // O^T (dims 16mt..+15 x 16 rows) += V^T P'^T. Lane m of a group addresses
  // cell operand_cell(g, m >> 1), dims 16mt + 8(m & 1): lane i receives byte
  // i & 7 of the rows of lanes (i >> 3) + 2s, i.e. dim 16mt + i of the 8 cells
  const int sidx = (lane & 15) >> 1;
  const uint8_t* vrow = tile.v + operand_cell(g, sidx) * kD + 8 * (lane & 1);
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    const v2i raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t)(vrow + 16 * (mt ^ sidx)));
    st.o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
        biased_half8((uint32_t)raw.x, (uint32_t)raw.y), pb, st.o[mt], 0, 0, 0);
  }
}

// Row i = lane & 15 of query head h*12 + i at position j (rows 12..15 read row
// 0 and are zeroed later), dims 64q + 16g + 8hf .. +7 in x[2(2q + hf)] and the
// next, g = lane >> 4. The kernels issue these loads before the cell list is
// built, so that they land meanwhile.
struct QRaw {
  float4v x[8];
};

__device__ __forceinline__ void load_q(const PositionsArgs& a, int j, int h, int lane, QRaw& r) {
  const int g = lane >> 4, i = lane & 15;
  const int n_qh = a.n_kv * kQPerKv;
  const float* qg = a.q + ((int64_t)j * n_qh + h * kQPerKv + (i < kQPerKv ? i : 0)) * kD + 16 * g;
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      r.x[2 * (2 * q + hf)] = *reinterpret_cast<const float4v*>(qg + 64 * q + 8 * hf);
      r.x[2 * (2 * q + hf) + 1] = *reinterpret_cast<const float4v*>(qg + 64 * q + 8 * hf + 4);
    }
}

// KV head h's 12 query rows over the n cells rows[0..n): the running state,
// with the row's probability sum and sum(P') gathered over its four lanes.
__device__ __forceinline__ void attend_range(const PositionsArgs& a, const uint32_t* rows,
                                             WaveTile& tile, int j, int h, int n, int lane,
                                             const QRaw& qr, uint32_t& flags, ChunkState& st,
                                             float& l_row, float& lp_row) {
  const int i = lane & 15;
  const bool row_ok = i < kQPerKv;

  // Q operands of row i: k-step 2q + hf holds dims 64q + 16g + 8hf .. +7
  half8 qb[4];
  float qsum = 0.f;
  {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float4v x0 = qr.x[2 * (2 * q + hf)];
        float4v x1 = qr.x[2 * (2 * q + hf) + 1];
        if (!row_ok) x0 = x1 = float4v{0.f, 0.f, 0.f, 0.f};
        const half8 v = half8{(_Float16)x0.x, (_Float16)x0.y, (_Float16)x0.z, (_Float16)x0.w,
                              (_Float16)x1.x, (_Float16)x1.y, (_Float16)x1.z, (_Float16)x1.w};
        qb[2 * q + hf] = v;
#pragma unroll
        for (int e = 0; e < 8; ++e) qsum += (float)v[e];
      }
  }
  // the row's sum over all 128 dims (4 lane groups), times the K bias
  qsum += __shfl_xor(qsum, 16);
  qsum += __shfl_xor(qsum, 32);
  const float s_init = -1152.f * qsum;

#pragma unroll
  for (int mt = 0; mt < 8; ++mt) st.o[mt] = float4v{0.f, 0.f, 0.f, 0.f};
  st.m_run = kNoMax;
  st.l_run = 0.f;
  st.lp = 0.f;

  // three register sets in rotation: copying one into another would wait for
  // the loads just issued
  const int nch = (n + kChunk - 1) / kChunk;
  if (nch > 0) {
    ChunkRegs r0, r1, r2;
    load_chunk(a, rows, 0, n, h, lane, r0);
    load_chunk(a, rows, min(1, nch - 1), n, h, lane, r1);
    int c = 0;
    for (; c + 3 <= nch; c += 3) {
      chunk_step(a, rows, tile, st, c, nch, n, h, lane, s_init, qb, r0, r2, flags);
      chunk_step(a, rows, tile, st, c + 1, nch, n, h, lane, s_init, qb, r1, r0, flags);
      chunk_step(a, rows, tile, st, c + 2, nch, n, h, lane, s_init, qb, r2, r1, flags);
    }
    if (c < nch) chunk_step(a, rows, tile, st, c, nch, n, h, lane, s_init, qb, r0, r2, flags);
    if (c + 1 < nch) chunk_step(a, rows, tile, st, c + 1, nch, n, h, lane, s_init, qb, r1, r0, flags);
  }
  l_row = st.l_run;
  lp_row = st.lp;
  l_row += __shfl_xor(l_row, 16);
  l_row += __shfl_xor(l_row, 32);
  lp_row += __shfl_xor(lp_row, 16);
  lp_row += __shfl_xor(lp_row, 32);
}

// Thread tid's entries tid + kThreads * k of position j's row (-1 past its
// length L, which is clamped to [0, sel_cap] and flagged when outside). The
// entries are read up to sel_cap without waiting for the length, so both reads
// take one round trip. Returns whether this thread's entries rise strictly
// (each below the row's next entry).
__device__ __forceinline__ bool read_row(const PositionsArgs& a, int j, int tid, int32_t (&cell)[kPer],
                                         int& L, uint32_t& flags) {
  const int32_t* srow = a.sel + (int64_t)j * a.sel_cap;
  int32_t nxt[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int e = tid + kThreads * k;
    cell[k] = e < a.sel_cap ? srow[e] : -1;
    nxt[k] = e + 1 < a.sel_cap ? srow[e + 1] : 0;
  }
  L = a.sel_len[j];
  if (L < 0 || L > a.sel_cap) {
    flags |= SEL_ATTN_STATUS_SEL_LEN;
    L = L < 0 ? 0 : a.sel_cap;
  }
  bool asc = true;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int e = tid + kThreads * k;
    if (e >= L) cell[k] = -1;
    asc = asc && (e + 1 >= L || cell[k] < nxt[k]);
    if (e < L && (cell[k] < 0 || cell[k] >= a.n_ctx)) flags |= SEL_ATTN_STATUS_CELL_RANGE;
  }
  return asc;
}

// Phase 1 (the whole work-group): position j's list of pool rows in sm.rows,
// repeats, cells out of range and non-resident pages dropped, in row order.
// Returns the list's length.
__device__ __forceinline__ int build_list(const PositionsArgs& a, Smem& sm, int j, int tid,
                                          int lane, int wave, uint32_t& flags) {
  int32_t* hash_key = sm.u.hash.key;
  int32_t* hash_first = sm.u.hash.first;
  int32_t cell[kPer];
  int L;
  // a strictly ascending row has no repeats; any other row goes through the hash
  const bool sorted = __syncthreads_and(read_row(a, j, tid, cell, L, flags));
  if (!sorted) {
    for (int s = tid; s < kHashSlots; s += kThreads) {
      hash_key[s] = -1;
      hash_first[s] = 0x7fffffff;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int e = tid + kThreads * k;
      const int32_t c = cell[k];
      if (e >= L || c < 0 || c >= a.n_ctx) continue;
      // at most kPer * kThreads < kHashSlots distinct cells: an empty slot or
      // the cell itself is always found
      uint32_t s = hash_slot(c);
      while (true) {
        const int32_t prev = atomicCAS(&hash_key[s], -1, c);
        if (prev == -1 || prev == c) {
          atomicMin(&hash_first[s], e);
          break;
        }
        s = (s + 1) & (kHashSlots - 1);
      }
    }
    __syncthreads();
  }
  // each cell's first entry looks up its page; all lookups are issued before
  // the first is used (one memory round trip, not one per round)
  int32_t page[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int e = tid + kThreads * k;
    const int32_t c = cell[k];
    page[k] = -1;
    if (e < L && c >= 0 && c < a.n_ctx) {
      bool first = true;
      if (!sorted) {
        uint32_t s = hash_slot(c);
        while (hash_key[s] != c) s = (s + 1) & (kHashSlots - 1);
        first = hash_first[s] == e;
      }
      if (first) page[k] = a.page_table[c >> 6];
      else cell[k] = -1;                 // a repeat
    }
  }
  int base = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int e = tid + kThreads * k;
    const int32_t c = cell[k];
    const bool first = e < L && c >= 0 && c < a.n_ctx;
    if (first && (page[k] >= a.n_pages || page[k] < -1)) flags |= SEL_ATTN_STATUS_PAGE_RANGE;
    const bool keep = first && page[k] >= 0 && page[k] < a.n_pages;
    const uint32_t row = ((uint32_t)page[k] * (uint32_t)a.n_kv) * 64u + (uint32_t)(c & 63);
    const uint64_t m = __ballot(keep);
    if (lane == 0) sm.wave_count[k & 1][wave] = __popcll(m);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int cnt = sm.wave_count[k & 1][w];
      before += w < wave ? cnt : 0;
      total += cnt;
    }
    if (keep) sm.rows[base + before + lanes_below(m)] = row;
    base += total;
  }
  __syncthreads();   // the list is complete; the hash area becomes the waves' tiles
  return base;
}

__global__ __launch_bounds__(kThreads, 2) void prefill_positions_kernel(PositionsArgs a) {
  __shared__ Smem sm;
  const int b = blockIdx.x;
  const int j = (b & 7) * a.per_xcd + (b >> 3);   // neighbouring positions on one XCD
  if (j >= a.n_q) return;                          // whole work-groups
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t flags = 0;
  QRaw q0;   // Q of the first KV head this wave takes
  if (wave < a.n_kv) load_q(a, j, wave, lane, q0);
  const int n = build_list(a, sm, j, tid, lane, wave, flags);

  // phase 2: wave w takes KV heads w, w + 4, ...;
  // out = (O^T - 1152 sum(P')) / (2^6 sum(p))
  const int g = lane >> 4, i = lane & 15;
  const int n_qh = a.n_kv * kQPerKv;
  auto head = [&](int h, const QRaw& qr) {
    ChunkState st;
    float l_row, lp_row;
    attend_range(a, sm.rows, sm.u.tile[wave], j, h, n, lane, qr, flags, st, l_row, lp_row);
    const float corr = 1152.f * lp_row;
    const float inv = l_row > 0.f ? (1.f / kVFold) / l_row : 0.f;
    if (i < kQPerKv) {
      float* orow = a.out + ((int64_t)j * n_qh + h * kQPerKv + i) * kD + 4 * g;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
        *reinterpret_cast<float4v*>(orow + 16 * mt) = (st.o[mt] - corr) * inv;
    }
  };
  if (wave < a.n_kv) head(wave, q0);
  for (int h = wave + kWaves; h < a.n_kv; h += kWaves) {
    QRaw qr;
    load_q(a, j, h, lane, qr);
    head(h, qr);
  }
  if (flags) atomicOr(a.status, flags);
}

// ---------------------------------------------------------------------------
// Decode: a few positions (one, or a speculative verify window), each split
// over its cells so that the GPU has enough work-groups. Work-group (s, j)
// takes the kept cells among entries [64s, 64s + 64) of position j's row and
// attends to them for every KV head. It writes
// the split's unnormalised state; a second kernel merges the splits of each
// (position, head) in the usual way: weights exp2(m_s - max m), sums of those
// times O_s and l_s, then O / l.

// Decode split s of position j: the kept cells among the row's entries
// [64s, 64s + 64), in entry order, in sm.rows. A cell counts at its first entry
// in the row: a strictly ascending row has no repeats; any other row goes
// through the LDS hash, which keeps each cell's first entry. Cells out of range
// (checked over the whole row, as every split reports them) and non-resident
// pages are dropped. Returns the count.
__device__ __forceinline__ int build_split_list(const PositionsArgs& a, Smem& sm, int j, int first,
                                                int tid, int lane, int wave, uint32_t& flags) {
  int32_t* hash_key = sm.u.hash.key;
  int32_t* hash_first = sm.u.hash.first;
  int32_t cell[kPer];
  int L;
  const bool sorted = __syncthreads_and(read_row(a, j, tid, cell, L, flags));
  if (!sorted) {
    for (int s = tid; s < kHashSlots; s += kThreads) {
      hash_key[s] = -1;
      hash_first[s] = 0x7fffffff;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int e = tid + kThreads * k;
      const int32_t c = cell[k];
      if (e >= L || c < 0 || c >= a.n_ctx) continue;
      // at most kPer * kThreads < kHashSlots distinct cells: an empty slot or
      // the cell itself is always found
      uint32_t s = hash_slot(c);
      while (true) {
        const int32_t prev = atomicCAS(&hash_key[s], -1, c);
        if (prev == -1 || prev == c) {
          atomicMin(&hash_first[s], e);
          break;
        }
        s = (s + 1) & (kHashSlots - 1);
      }
    }
    __syncthreads();
  }
  // the split's entries first + lane are already in the registers of wave
  // (first / 64) & 3, at index first / 256
  const int owner = (first >> 6) & (kWaves - 1);
  if (wave == owner) {
    const int e = first + lane;
    const int ks = first >> 8;
    int32_t c = -1;
#pragma unroll
    for (int k = 0; k < kPer; ++k) c = k == ks ? cell[k] : c;
    bool counts = e < L && c >= 0 && c < a.n_ctx;
    if (counts && !sorted) {
      uint32_t s = hash_slot(c);
      while (hash_key[s] != c) s = (s + 1) & (kHashSlots - 1);
      counts = hash_first[s] == e;
    }
    const int32_t page = counts ? a.page_table[c >> 6] : -1;
    if (counts && (page >= a.n_pages || page < -1)) flags |= SEL_ATTN_STATUS_PAGE_RANGE;
    const bool keep = counts && page >= 0 && page < a.n_pages;
    const uint64_t m = __ballot(keep);
    if (keep)
      sm.rows[lanes_below(m)] = ((uint32_t)page * (uint32_t)a.n_kv) * 64u + (uint32_t)(c & 63);
    if (lane == 0) sm.wave_count[0][0] = __popcll(m);
  }
  __syncthreads();   // the list is complete; the hash area becomes the waves' tiles
  return sm.wave_count[0][0];
}

__global__ __launch_bounds__(kThreads, 2) void decode_split_kernel(PositionsArgs a,
                                                                  DecodePartial* part) {
  __shared__ Smem sm;
  const int s = blockIdx.x;
  const int j = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t flags = 0;
  const int first = kDecodeSplit * s;
  QRaw q0;   // Q of the first KV head this wave takes
  if (wave < a.n_kv) load_q(a, j, wave, lane, q0);
  const int n_s = build_split_list(a, sm, j, first, tid, lane, wave, flags);

  const int g = lane >> 4, i = lane & 15;
  auto head = [&](int h, const QRaw& qr) {
    ChunkState st;
    float l_row, lp_row;
    attend_range(a, sm.rows, sm.u.tile[wave], j, h, n_s, lane, qr, flags, st, l_row, lp_row);
    DecodePartial& p = part[((int64_t)j * a.n_kv + h) * a.n_splits + s];
    if (i < kQPerKv) {
      const float corr = 1152.f * lp_row;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
        *reinterpret_cast<float4v*>(&p.o[i][16 * mt + 4 * g]) = st.o[mt] - corr;
      if (g == 0) {
        p.m[i] = st.m_run;
        p.l[i] = l_row;
      }
    }
  };
  if (wave < a.n_kv) head(wave, q0);
  for (int h = wave + kWaves; h < a.n_kv; h += kWaves) {
    QRaw qr;
    load_q(a, j, h, lane, qr);
    head(h, qr);
  }
  if (flags) atomicOr(a.status, flags);
}

// One work-group per (query row, KV head, position), one thread per dim.
// Every thread first issues the loads of its dim in all splits (at most 40);
// meanwhile thread s of the first wave reads split s's m and l, the wave
// reduces them, and the weights go through LDS; then every thread sums its dim
// over the splits. One memory round trip in all.
constexpr int kMaxSplits = (SEL_ATTN_POSITIONS_MAX_CAP + kDecodeSplit - 1) / kDecodeSplit;
static_assert(kMaxSplits <= 64, "one wave reduces the splits' maxima");

__global__ __launch_bounds__(kD) void decode_merge_kernel(PositionsArgs a, const DecodePartial* part) {
  __shared__ float wsh[64];
  __shared__ float lsh;
  const int r = blockIdx.x;
  const int h = blockIdx.y;
  const int j = blockIdx.z;
  const int d = threadIdx.x;
  const DecodePartial* p = part + ((int64_t)j * a.n_kv + h) * a.n_splits;
  float od[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) od[s] = s < a.n_splits ? p[s].o[r][d] : 0.f;
  if (d < 64) {
    const bool ok = d < a.n_splits;
    const float ms = ok ? p[d].m[r] : kNoMax;
    const float ls = ok ? p[d].l[r] : 0.f;
    float m = ms;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    const float w = ok ? __builtin_amdgcn_exp2f(ms - m) : 0.f;
    float l = w * ls;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
    wsh[d] = w;
    if (d == 0) lsh = l;
  }
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) acc += s < a.n_splits ? wsh[s] * od[s] : 0.f;
  const float l = lsh;
  const int n_qh = a.n_kv * kQPerKv;
  a.out[((int64_t)j * n_qh + h * kQPerKv + r) * kD + d] = l > 0.f ? acc * ((1.f / kVFold) / l) : 0.f;
}

}  // namespace

hipError_t launch_prefill_positions(const PositionsArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(prefill_positions_kernel, dim3(8 * a.per_xcd), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const PositionsArgs& a, DecodePartial* part, hipStream_t stream) {
  hipLaunchKernelGGL(decode_split_kernel, dim3(a.n_splits, a.n_q), dim3(kThreads), 0, stream, a,
                     part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(kQPerKv, a.n_kv, a.n_q), dim3(kD), 0, stream, a,
                     (const DecodePartial*)part);
  return hipGetLastError();
}

}  // namespace selattn
