// Union builder: for each group of 8 neighbouring query positions, the sorted
// union of their selected cells and, per union cell, a byte whose bit i marks
// position i of the group as one that chose it.
//
// Page: #2808 "sycl: prompt attention over 8-query selection unions on XMX",
// section Summary (the union and its marks) and section What changed (one
// work-group per 8 positions, local bitmaps); section Extra Notes (a cell is an
// int32, its mask a separate byte, so any context length works).
//
// gfx950 design: one 256-thread workgroup per group. The group's cells are
// scattered into an LDS bitmap that holds one chooser byte per cell (4 cells per
// 32-bit word, ds_or atomics), 64K cells per window; longer contexts take several
// windows in ascending order. Compaction walks the bitmap 256 words at a time:
// each lane owns one word (4 cells), four wave64 ballots give every lane the
// count of nonzero bytes below it, a two-slot LDS array of per-wave totals gives
// the workgroup offset with one barrier per round, and the lane writes its
// nonzero cells in ascending order. Output order is therefore ascending cell
// index, and the result is independent of row order and repeats.

#include "sel_attn_internal.h"

namespace selattn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kWindowCells = 65536;            // one chooser byte per cell
constexpr int kWindowWords = kWindowCells / 4; // 64 KiB of LDS

__device__ __forceinline__ int popc64(uint64_t x) { return __builtin_popcountll(x); }

__global__ __launch_bounds__(kThreads) void union_build_kernel(UnionArgs a) {
  __shared__ uint32_t bitmap[kWindowWords];
  __shared__ int wave_total[2][kWaves];

  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n_pos = min(8, a.n_q - 8 * g);
  const int64_t ucap = 8LL * a.sel_cap;
  int32_t* out_cells = a.union_cells + (int64_t)g * ucap;
  uint8_t* out_mask = a.union_mask + (int64_t)g * ucap;
  const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  uint32_t flags = 0;
  int len[8];
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
  }

  int written = 0;  // union cells emitted so far (same value in every thread)
  for (int w0 = 0; w0 < a.n_ctx; w0 += kWindowCells) {
    const int win = min(kWindowCells, a.n_ctx - w0);
    const int words = (win + 3) >> 2;
    for (int i = tid; i < words; i += kThreads) bitmap[i] = 0u;
    __syncthreads();

    // scatter: OR bit i into the byte of every cell row i selected
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i >= n_pos) break;
      const int32_t* row = a.sel + (int64_t)(8 * g + i) * a.sel_cap;
      for (int e = tid; e < len[i]; e += kThreads) {
        const int c = row[e];
        if (c < 0 || c >= a.n_ctx) {
          flags |= SEL_ATTN_STATUS_CELL_RANGE;
          continue;
        }
        const unsigned r = (unsigned)(c - w0);
        if (r < (unsigned)win) atomicOr(&bitmap[r >> 2], (1u << i) << ((r & 3u) * 8u));
      }
    }
    __syncthreads();

    // compaction in ascending cell order
    const int rounds = (words + kThreads - 1) / kThreads;
    for (int rd = 0; rd < rounds; ++rd) {
      const int wi = rd * kThreads + tid;
      const uint32_t w = (wi < words) ? bitmap[wi] : 0u;
      const uint64_t b0 = __ballot((w & 0x000000ffu) != 0u);
      const uint64_t b1 = __ballot((w & 0x0000ff00u) != 0u);
      const uint64_t b2 = __ballot((w & 0x00ff0000u) != 0u);
      const uint64_t b3 = __ballot((w & 0xff000000u) != 0u);
      const int below = popc64(b0 & lanes_below) + popc64(b1 & lanes_below) +
                        popc64(b2 & lanes_below) + popc64(b3 & lanes_below);
      if (lane == 0) wave_total[rd & 1][wave] = popc64(b0) + popc64(b1) + popc64(b2) + popc64(b3);
      __syncthreads();
      int before = 0, total = 0;
#pragma unroll
      for (int k = 0; k < kWaves; ++k) {
        const int t = wave_total[rd & 1][k];
        before += (k < wave) ? t : 0;
        total += t;
      }
      int o = written + before + below;
      const int cell0 = w0 + 4 * wi;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t m = (w >> (8 * k)) & 0xffu;
        if (m) {
          out_cells[o] = cell0 + k;
          out_mask[o] = (uint8_t)m;
          ++o;
        }
      }
      written += total;
    }
    __syncthreads();
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
