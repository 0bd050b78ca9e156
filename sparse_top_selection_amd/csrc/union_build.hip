// Union builder: for each group of 8 neighbouring query positions, the sorted
// union of their selected cells and, per union cell, a byte whose bit i marks
// position i of the group as one that chose it.
//
// Page: #2808 "sycl: prompt attention over 8-query selection unions on XMX",
// section Summary (the union and its marks) and section What changed (one
// work-group per 8 positions, local bitmaps); section Extra Notes (a cell is an
// int32, its mask a separate byte, so any context length works).
//
// gfx950 design: one 512-thread workgroup per group. The group's cells are
// scattered into an LDS bitmap that holds one chooser byte per cell (4 cells per
// 32-bit word, ds_or atomics), 32K cells per window (four workgroups fit a CU);
// longer contexts take several windows in ascending order. When the rows fit
// one pass of loads (2,560 entries each) they are read once into registers and
// every window scatters from there. Compaction is one pass: thread t owns a contiguous
// run of words, counts its nonzero bytes, a workgroup prefix sum (wave64 shuffles
// plus one LDS exchange) gives its output offset, and it writes its cells in
// ascending order. The bitmap is padded by one word per 32 so that 64 threads
// reading word i of their runs fall on 64 distinct banks. Output order is
// therefore ascending cell index, and the result is independent of row order and
// repeats.

#include "sel_attn_internal.h"

namespace selattn {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kWindowCells = 32768;                       // one chooser byte per cell
constexpr int kWindowWords = kWindowCells / 4;
constexpr int kPaddedWords = kWindowWords + kWindowWords / 32;   // 33 KiB of LDS
constexpr int kPer = 5;                                   // entries per thread, row and pass

// word w of the window lives at w + w / 32
__device__ __forceinline__ int padded(int w) { return w + (w >> 5); }

// number of nonzero bytes of x
__device__ __forceinline__ int nonzero_bytes(uint32_t x) {
  const uint32_t hi = ((x & 0x7f7f7f7fu) + 0x7f7f7f7fu) | x;
  return __builtin_popcount(hi & 0x80808080u);
}

__global__ __launch_bounds__(kThreads) void union_build_kernel(UnionArgs a) {
  __shared__ uint32_t bitmap[kPaddedWords];
  __shared__ int wave_sum[2][kWaves];

  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n_pos = min(8, a.n_q - 8 * g);
  const int64_t ucap = 8LL * a.sel_cap;
  int32_t* out_cells = a.union_cells + (int64_t)g * ucap;
  uint8_t* out_mask = a.union_mask + (int64_t)g * ucap;

  uint32_t flags = 0;
  int len[8];
  int max_len = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int L = 0;
    if (i < n_pos) {
      L = a.sel_len[8 * g + i];
      if (L < 0 || L > a.sel_cap) {
        flags |= SEL_ATTN_STATUS_SEL_LEN;
        L = L < 0 ? 0 : a.sel_cap;
      }
    }
    len[i] = L;
    max_len = max(max_len, L);
  }

  int32_t v[8][kPer];
  auto load_pass = [&](int base) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int32_t* row = a.sel + (int64_t)(8 * g + (i < n_pos ? i : 0)) * a.sel_cap;
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int e = base + tid + kThreads * k;
        v[i][k] = (i < n_pos && e < len[i]) ? row[e] : -1;
      }
    }
  };
  auto scatter_pass = [&](int base, int w0, int win) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int e = base + tid + kThreads * k;
        if (i >= n_pos || e >= len[i]) continue;
        const int c = v[i][k];
        if (c < 0 || c >= a.n_ctx) {
          flags |= SEL_ATTN_STATUS_CELL_RANGE;
          continue;
        }
        const unsigned r = (unsigned)(c - w0);
        if (r < (unsigned)win) atomicOr(&bitmap[padded(r >> 2)], (1u << i) << ((r & 3u) * 8u));
      }
    }
  };
  const bool one_pass = max_len <= kThreads * kPer;
  if (one_pass) load_pass(0);

  int written = 0;  // union cells emitted so far (same value in every thread)
  int round = 0;
  for (int w0 = 0; w0 < a.n_ctx; w0 += kWindowCells, ++round) {
    const int win = min(kWindowCells, a.n_ctx - w0);
    const int words = (win + 3) >> 2;
    const int pwords = padded(words - 1) + 1;
    for (int i = tid; i < pwords; i += kThreads) bitmap[i] = 0u;
    __syncthreads();

    // scatter: OR bit i into the byte of every cell row i selected. Entries are
    // read in passes of kPer per thread and row, all loads of a pass issued
    // before its atomics (one memory round trip per pass); with a single pass
    // the registers are filled once, before the first window.
    if (!one_pass) {
      for (int base = 0; base < max_len; base += kThreads * kPer) {
        load_pass(base);
        scatter_pass(base, w0, win);
      }
    } else {
      scatter_pass(0, w0, win);
    }
    __syncthreads();

    // compaction: thread tid owns words [b0, b1)
    const int per = (words + kThreads - 1) / kThreads;
    const int b0 = min(tid * per, words);
    const int b1 = min(b0 + per, words);
    int cnt = 0;
    for (int w = b0; w < b1; ++w) cnt += nonzero_bytes(bitmap[padded(w)]);
    // inclusive prefix over the wave, then over the waves
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    if (lane == 63) wave_sum[round & 1][wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
      const int t = wave_sum[round & 1][k];
      before += (k < wave) ? t : 0;
      total += t;
    }
    int o = written + before + incl - cnt;
    for (int w = b0; w < b1; ++w) {
      const uint32_t x = bitmap[padded(w)];
      if (x == 0u) continue;
      const int cell0 = w0 + 4 * w;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t m = (x >> (8 * k)) & 0xffu;
        if (m) {
          out_cells[o] = cell0 + k;
          out_mask[o] = (uint8_t)m;
          ++o;
        }
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
  hipLaunchKernelGGL(union_build_kernel, dim3(groups), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace selattn
