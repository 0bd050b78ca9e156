// Union builder: for each group of 8 adjacent query positions, one sorted list
// of every cell any of them selected and, per entry, a byte whose bit i is set
// when position i of the group selected that cell, and the cell's pool row for
// KV head 0 (its page-table entry resolved once here, not once per KV head by
// the attention step).
//
// Page: #2808 "sycl: prompt attention over 8-query selection unions on XMX",
// section Summary (the union and its marks) and section What changed (one
// work-group per 8 positions, local bitmaps); section Extra Notes (a cell is an
// int32, its mask a separate byte, so any context length works; cells of pages
// that are not resident are masked: their row is -1).
//
// gfx950 design: one 512-thread workgroup per group, four per CU (32 KiB of LDS
// and at most 64 VGPRs each), so that the 1,024 groups of an 8,192-position
// chunk are all resident at once and the kernel is one round of workgroups.
//   * The group's 8 selection rows are one contiguous span of 8 * sel_cap
//     int32. It is read with 16-byte loads of the aligned 16-byte blocks that
//     overlap it (a block holding one byte of the span lies in a mapped page),
//     in batches of four per thread whose loads are all issued before the first
//     is used (the first batch at entry, before the row lengths are read and
//     the bitmap cleared); entries outside the span or past their row's length
//     are skipped.
//   * Every counted entry ORs bit i (its row) into the chooser byte of its cell
//     in an LDS bitmap of one byte per cell, 32K cells per window (ds_or
//     atomics); longer contexts take several windows in ascending order, each
//     reading the span again (from cache).
//   * Compaction walks the window in cell order: wave w owns an eighth of its
//     cells (rounded up to whole 256-cell slabs, so a context shorter than the
//     window is still shared by every wave). One pass of word reads counts its
//     nonzero bytes and marks its nonempty 256-cell slabs; an eight-entry prefix over the waves gives its output
//     offset; then each nonempty slab is emitted 64 cells at a time (byte
//     reads, ballot, mbcnt), so that consecutive lanes store consecutive union
//     entries. The 64 cells of one emission step lie in one logical page, so
//     one page-table entry per step gives every lane's row; a wave's 64
//     entries are read with one load, one per lane, before the counting pass.
// Output order is ascending cell index, and the result is independent of row
// order and repeats.

#include "sel_attn_internal.h"

namespace selattn {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kWindowCells = 32768;                 // one chooser byte per cell
constexpr int kWindowWords = kWindowCells / 4;       // 32 KiB of LDS
constexpr int kWaveWords = kWindowWords / kWaves;    // compaction share of a wave
constexpr int kBatch = 4;                            // 16-byte loads per thread in flight
constexpr int kSlabs = kWaveWords / 64;              // 256-cell slabs per wave (16)

// number of nonzero bytes of x
__device__ __forceinline__ int nonzero_bytes(uint32_t x) {
  const uint32_t hi = ((x & 0x7f7f7f7fu) + 0x7f7f7f7fu) | x;
  return __builtin_popcount(hi & 0x80808080u);
}

// 16-byte block b of the span's aligned cover (b < n_blocks; others read block
// 0). kOnce: the span is read only once (a single window), so the load is
// marked non-temporal and does not displace cached data; with several windows
// the span is read again from cache.
template <bool kOnce>
__device__ __forceinline__ i32x4 load_block(const int32_t* base, int b, int n_blocks) {
  const i32x4* p = reinterpret_cast<const i32x4*>(base + 4 * (b < n_blocks ? b : 0));
  if constexpr (kOnce) return __builtin_nontemporal_load(p);
  return *p;
}

// The rows of a block's four entries (f0 = flat index of entry 0 in the
// span): byte j = row of entry j, or 0xff when the entry does not count
// (outside the span, past its row's length, or a cell outside [0, n_ctx):
// flagged).
__device__ __forceinline__ uint32_t classify_block(const i32x4 x, int f0, int cap, float inv_cap,
                                                   const int* row_end, int n_ctx, uint32_t& flags) {
  const int vals[4] = {x.x, x.y, x.z, x.w};
  uint32_t rw = 0xffffffffu;
  if (cap >= 4) {
    // rows of at least 4 entries: a block crosses at most one row end. Row of
    // entry max(f0, 0): a float estimate, corrected to the exact one.
    const int fc = max(f0, 0);
    int row = min((int)((float)fc * inv_cap), 7);
    if (row * cap > fc) --row;
    if ((row + 1) * cap <= fc) ++row;
    const int next = (row + 1) * cap;   // first entry of the next row
    const int end0 = row_end[row];
    const int end1 = row_end[min(row + 1, 7)];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int f = f0 + j;
      const bool second = f >= next;
      const bool counts = f >= 0 && f < (second ? end1 : end0);
      const bool in_ctx = (unsigned)vals[j] < (unsigned)n_ctx;
      flags |= (counts && !in_ctx) ? SEL_ATTN_STATUS_CELL_RANGE : 0u;
      const uint32_t r = (uint32_t)(second ? row + 1 : row);
      if (counts && in_ctx) rw = (rw & ~(0xffu << (8 * j))) | (r << (8 * j));
    }
  } else {
    // shorter rows: each entry's row by division
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int f = f0 + j;
      if (f < 0 || f >= 8 * cap) continue;
      const int r = f / cap;
      if (f >= row_end[r]) continue;
      if ((unsigned)vals[j] >= (unsigned)n_ctx) {
        flags |= SEL_ATTN_STATUS_CELL_RANGE;
        continue;
      }
      rw = (rw & ~(0xffu << (8 * j))) | ((uint32_t)r << (8 * j));
    }
  }
  return rw;
}

// OR bit r into the chooser byte of every counted entry's cell in this window
__device__ __forceinline__ void scatter_block(uint32_t* bitmap, const i32x4 x, uint32_t rw, int w0,
                                              int win) {
  const int vals[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t r = (rw >> (8 * j)) & 0xffu;
    const unsigned rel = (unsigned)(vals[j] - w0);
    if (r != 0xffu && rel < (unsigned)win) atomicOr(&bitmap[rel >> 2], (1u << r) << ((rel & 3u) * 8u));
  }
}

// zero the window's chooser bytes
__device__ __forceinline__ void clear_bitmap(uint32_t* bitmap, int tid) {
  for (int i = tid; i < kWindowWords / 4; i += kThreads)
    reinterpret_cast<u32x4*>(bitmap)[i] = u32x4{0u, 0u, 0u, 0u};
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
  return x;
}

// kOnce: the context fits one window (n_ctx <= kWindowCells).
template <bool kOnce>
__global__ __launch_bounds__(kThreads, 8) void union_build_kernel(UnionArgs a) {
  __shared__ uint32_t bitmap[kWindowWords];
  __shared__ int wave_cnt[2][kWaves];
  __shared__ int row_end[8];   // flat index (within the span) past row i's entries

  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n_pos = min(8, a.n_q - 8 * g);
  const int cap = a.sel_cap;
  const int64_t ucap = 8LL * cap;
  int32_t* out_cells = a.union_cells + (int64_t)g * ucap;
  uint8_t* out_mask = a.union_mask + (int64_t)g * ucap;
  int32_t* out_rows = a.union_rows + (int64_t)g * ucap;
  const int last_page = (a.n_ctx - 1) >> 6;   // logical pages of the context: 0 .. last_page
  const int kv_rows = 64 * a.n_kv;            // pool rows per physical page

  // the span: n_pos rows from sel + 8g * cap, read as the aligned 16-byte
  // blocks that overlap it; flat index f of a loaded entry = 4 * block - shift
  const int32_t* span = a.sel + (int64_t)8 * g * cap;
  const int shift = (int)((reinterpret_cast<uintptr_t>(span) >> 2) & 3u);
  const int32_t* base = span - shift;
  const int span_len = n_pos * cap;
  const float inv_cap = 1.f / (float)cap;

  // blocks of the span's aligned 16-byte cover
  const int n_blocks = (int)(((int64_t)span_len + shift + 3) / 4);

  // the first batch of blocks goes out before anything waits: it needs neither
  // the row lengths (read next) nor the cleared bitmap until it is scattered
  i32x4 first[kBatch];
#pragma unroll
  for (int k = 0; k < kBatch; ++k) first[k] = load_block<kOnce>(base, tid + kThreads * k, n_blocks);

  uint32_t flags = 0;
  if (tid < 8) {
    int L = 0;
    if (tid < n_pos) {
      L = a.sel_len[8 * g + tid];
      if (L < 0 || L > cap) {
        flags |= SEL_ATTN_STATUS_SEL_LEN;
        L = L < 0 ? 0 : cap;
      }
    }
    row_end[tid] = tid * cap + L;
  }
  __syncthreads();   // row_end

  int written = 0;  // union cells emitted so far (same value in every thread)
  // windows counted, not stepped, so that no cell index passes INT32_MAX
  const int n_windows = (int)(((int64_t)a.n_ctx + kWindowCells - 1) / kWindowCells);

  // the first window's bitmap cleared (the barrier orders it before the
  // marking) and its first batch scattered, here rather than in the loop so
  // that the batch's registers are free before it
  clear_bitmap(bitmap, tid);
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kBatch; ++k) {
    const int b = tid + kThreads * k;
    if (b < n_blocks)
      scatter_block(bitmap, first[k],
                    classify_block(first[k], 4 * b - shift, cap, inv_cap, row_end, a.n_ctx, flags), 0,
                    min(kWindowCells, a.n_ctx));
  }

  for (int round = 0; round < n_windows; ++round) {
    const int w0 = round * kWindowCells;
    const int win = min(kWindowCells, a.n_ctx - w0);
    if (round > 0) {
      clear_bitmap(bitmap, tid);
      __syncthreads();
    }

    // scatter: the span in batches of kBatch blocks per thread, all loads of a
    // batch issued before the first is used (one memory round trip per batch;
    // the first window's first batch is done above, later windows find the
    // span in cache)
    for (int b0 = round == 0 ? kThreads * kBatch : 0; b0 < n_blocks; b0 += kThreads * kBatch) {
      i32x4 raw[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
        raw[k] = load_block<kOnce>(base, b0 + tid + kThreads * k, n_blocks);
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int b = b0 + tid + kThreads * k;
        if (b < n_blocks)
          scatter_block(bitmap, raw[k],
                        classify_block(raw[k], 4 * b - shift, cap, inv_cap, row_end, a.n_ctx, flags),
                        w0, win);
      }
    }
    // this wave's share of the window: words [wb, wb + share), an eighth of
    // the window's words rounded up to whole slabs of 64 words (256 cells), at
    // most 16 slabs, so that short contexts keep every wave busy. It covers
    // logical pages pw .. pw + 63 at most: lane l reads entry pw + l now, and
    // emission takes entry 4s + k of slab s, step k from that lane (clamped to
    // the table; a page past the context holds no union cell)
    const int words = (win + 3) >> 2;
    const int share = min(kWaveWords, ((words + kWaves - 1) / kWaves + 63) & ~63);
    const int wb = wave * share;
    const int pw = (w0 + 4 * wb) >> 6;
    const int32_t page_of_lane = a.page_table[min(pw + lane, last_page)];
    __syncthreads();

    // compaction of this wave's share. One pass of word reads counts the
    // nonzero bytes and marks the nonempty slabs.
    const int lim = min(share, words - wb);   // words of the share inside the window
    int cnt = 0;
    uint32_t nonempty = 0;   // bit s: slab s holds a union cell (same in every lane)
#pragma unroll
    for (int s = 0; s < kSlabs; ++s) {
      const uint32_t x = (64 * s < lim) ? bitmap[wb + 64 * s + lane] : 0u;
      cnt += nonzero_bytes(x);
      nonempty |= __ballot(x != 0u) ? (1u << s) : 0u;
    }
    cnt = wave_sum(cnt);
    if (lane == 0) wave_cnt[round & 1][wave] = cnt;
    __syncthreads();
    int o = written, total = 0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
      const int t = wave_cnt[round & 1][k];
      o += (k < wave) ? t : 0;
      total += t;
    }
    // emission: nonempty slabs in order, 64 cells at a time, so that
    // consecutive lanes store consecutive union entries
    const uint8_t* bytes = reinterpret_cast<const uint8_t*>(bitmap);
    while (nonempty) {
      const int s = __builtin_ctz(nonempty);
      nonempty &= nonempty - 1;
      const int rel0 = 4 * (wb + 64 * s) + lane;   // cell within the window, k = 0
      // the 64 cells of step k are logical page pw + 4s + k, cell lane of it
      int32_t pg[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) pg[k] = __builtin_amdgcn_readlane(page_of_lane, 4 * s + k);
      uint32_t m[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) m[k] = bytes[rel0 + 64 * k];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint64_t b = __ballot(m[k] != 0u);
        if (m[k]) {
          const int at = o + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
          const bool resident = pg[k] >= 0 && pg[k] < a.n_pages;
          flags |= (pg[k] < -1 || pg[k] >= a.n_pages) ? SEL_ATTN_STATUS_PAGE_RANGE : 0u;
          out_cells[at] = w0 + rel0 + 64 * k;
          out_mask[at] = (uint8_t)m[k];
          out_rows[at] = resident ? pg[k] * kv_rows + lane : -1;
        }
        o += __builtin_popcountll(b);
      }
    }
    written += total;
    __syncthreads();   // the bitmap is cleared for the next window
  }

  if (tid == 0) a.union_len[g] = written;
  if (flags) atomicOr(a.status, flags);
}

}  // namespace

hipError_t launch_union_build(const UnionArgs& a, hipStream_t stream) {
  const int groups = (a.n_q + 7) / 8;
  if (a.n_ctx <= kWindowCells)
    hipLaunchKernelGGL(union_build_kernel<true>, dim3(groups), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(union_build_kernel<false>, dim3(groups), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace selattn
