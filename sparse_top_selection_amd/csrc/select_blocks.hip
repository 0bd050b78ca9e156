// Selection step: per-position block scores -> the selection rows that the
// union step reads.
//
// Page: #2808 "sycl: prompt attention over 8-query selection unions on XMX",
// section What changed (the selection, block scores then top-k, is the step
// before the prompt attention) and the accuracy list in section Summary (the
// selection layout's cap of 2,051 cells). A row is the three sink cells, the 31 earlier full blocks
// with the highest scores, and the position's own block up to the position:
// 3 + 31*64 + 64 = 2,051 cells at most. A position with at most 31 earlier
// blocks takes them all, so its row is [0, p]. Equal scores go to the lower
// block index first; a NaN score counts as -inf; -0.0 equals +0.0.
//
// gfx950 design: one wave64 per position, four positions per work-group, no
// barriers. Lane l holds the ordered keys of blocks 64s + l (s < S, a
// compile-time slot count) in registers. The 31st largest key is found bit by
// bit from the top, counting keys at or above each candidate with wave
// ballots. To keep that search short, a lower bound comes first: the 31st
// largest of the 64 lane maxima. Usually fewer than 64 keys reach it; they
// move into a single slot (through 512 bytes of LDS per wave), and the search
// runs there. Otherwise (many equal scores, say) it runs over every slot. Ties
// at the 31st key are resolved in block order by a ballot prefix count. The
// chosen blocks come out of the ballot masks in ascending order, and each is
// written as one coalesced 256-byte store of its 64 cell indices.

#include "sel_attn_internal.h"

namespace selattn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlock = SEL_ATTN_PAGE_SIZE;
constexpr int kSinks = SEL_ATTN_SINKS;
constexpr int kTop = SEL_ATTN_TOP_BLOCKS;

// A key whose unsigned order is the order of the scores. Adding +0.0 turns
// -0.0 into +0.0 (and quiets a NaN); fmaxf with -inf then turns a NaN into
// -inf. A positive float's key sets the sign bit, a negative float's inverts
// every bit. Every score's key is at least that of -inf (0x007fffff), so key 0
// marks a slot with no block.
__device__ __forceinline__ uint32_t score_key(float s) {
  const uint32_t u = __float_as_uint(fmaxf(s + 0.0f, -__builtin_inff()));
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// lanes below this one whose bit is set in m
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// The 31st largest of the keys held in S slots, rounded down to a multiple of
// 2^low: the largest such t with at least 31 keys >= t, found bit by bit from
// the top (low = 0 gives the key itself).
template <int S, int low = 0>
__device__ __forceinline__ uint32_t top_key(const uint32_t (&key)[S]) {
  constexpr int kUnroll = S == 1 ? 32 : 1;   // one slot: no loop control at all
  uint32_t t = 0u;
#pragma unroll kUnroll
  for (int bit = 31; bit >= low; --bit) {
    const uint32_t cand = t | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int s = 0; s < S; ++s) cnt += __popcll(__ballot(key[s] >= cand));
    if (cnt >= kTop) t = cand;
  }
  return t;
}

// Which of one slot's keys are taken, given t = top_key over every key: those
// above t, then keys equal to t in order (eq_before: equal keys in earlier
// slots) until 31 are taken.
__device__ __forceinline__ bool taken(uint32_t key, uint32_t t, int need, int eq_before,
                                      uint64_t eq) {
  return key > t || (key == t && eq_before + lanes_below(eq) < need);
}

template <int S>
__global__ __launch_bounds__(kThreads) void select_blocks_kernel(SelectArgs a) {
  __shared__ uint2 cand[kWaves][64];      // (key, block) of the candidates
  __shared__ int32_t chosen[kWaves][32];  // the taken blocks, ascending
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = blockIdx.x * kWaves + wave;
  if (j >= a.n_q) return;   // whole waves leave together; no barriers below
  const int p = a.first_pos + j;
  const int own = p / kBlock;
  int32_t* row = a.sel + (int64_t)j * a.sel_cap;

  if (own <= kTop) {   // every causal cell
    for (int e = lane; e <= p; e += 64) row[e] = e;
    if (lane == 0) a.sel_len[j] = p + 1;
    return;
  }

  // every load is issued before the first is used: the index is clamped to a
  // block that exists (own >= 32) instead of branching around the load
  const float* srow = a.scores + (int64_t)j * a.n_blocks;
  float score[S];
#pragma unroll
  for (int s = 0; s < S; ++s) score[s] = srow[min(64 * s + lane, own - 1)];
  // slots wholly below own need no per-lane test (own is the same in every lane)
  uint32_t key[S];
  uint32_t lane_max = 0u;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    if (64 * s + 64 <= own)
      key[s] = score_key(score[s]);
    else
      key[s] = 64 * s + lane < own ? score_key(score[s]) : 0u;
    lane_max = max(lane_max, key[s]);
  }

  // The 31st largest lane maximum is a lower bound of the answer (31 distinct
  // keys reach it; lanes 0..31 all hold a block), and so is that value with
  // its low 16 bits cleared, which takes half the search. Only keys at or
  // above the bound can be taken; when at most 64 are, they move into one slot
  // (ascending block order, through LDS) and the search runs on that slot
  // alone.
  const uint32_t lane_max_slot[1] = {lane_max};
  const uint32_t lo = top_key<1, 16>(lane_max_slot);
  int n_cand = 0;
#pragma unroll
  for (int s = 0; s < S; ++s) n_cand += __popcll(__ballot(key[s] >= lo));

  // the taken blocks go to chosen[wave][0..30] in ascending order
  if (n_cand <= 64) {
    int base = 0;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const bool c = key[s] >= lo;
      const uint64_t m = __ballot(c);
      if (c) cand[wave][base + lanes_below(m)] = uint2{key[s], (uint32_t)(64 * s + lane)};
      base += __popcll(m);
    }
    __builtin_amdgcn_wave_barrier();
    const uint2 cl = cand[wave][lane];
    const uint32_t ck[1] = {lane < n_cand ? cl.x : 0u};
    const uint32_t t = top_key<1>(ck);
    const int need = kTop - __popcll(__ballot(ck[0] > t));
    const bool pick = taken(ck[0], t, need, 0, __ballot(ck[0] == t));
    const uint64_t m = __ballot(pick);
    if (pick) chosen[wave][lanes_below(m)] = (int)cl.y;
  } else {
    const uint32_t t = top_key<S>(key);
    int above = 0;
#pragma unroll
    for (int s = 0; s < S; ++s) above += __popcll(__ballot(key[s] > t));
    const int need = kTop - above;   // keys equal to t that are taken (>= 1)
    int eq_before = 0, base = 0;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint64_t eq = __ballot(key[s] == t);
      const bool pick = taken(key[s], t, need, eq_before, eq);
      const uint64_t m = __ballot(pick);
      if (pick) chosen[wave][base + lanes_below(m)] = 64 * s + lane;
      eq_before += __popcll(eq);
      base += __popcll(m);
    }
  }
  __builtin_amdgcn_wave_barrier();

  // the row: the sinks unless block 0 is taken, the 31 blocks, then the own
  // block's causal cells; every store is 64 consecutive cells
  const bool block0 = chosen[wave][0] == 0;
  const int off = block0 ? 0 : kSinks;
  if (!block0 && lane < kSinks) row[lane] = lane;
  int32_t* dst = row + off + lane;
#pragma unroll
  for (int k = 0; k < kTop; ++k) dst[kBlock * k] = chosen[wave][k] * kBlock + lane;
  const int n_own = p - own * kBlock + 1;
  if (lane < n_own) dst[kBlock * kTop] = own * kBlock + lane;
  if (lane == 0) a.sel_len[j] = off + kBlock * kTop + n_own;
}

template <int S>
hipError_t launch_slots(const SelectArgs& a, hipStream_t stream) {
  const int grid = (a.n_q + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(select_blocks_kernel<S>, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select_blocks(const SelectArgs& a, hipStream_t stream) {
  // slots cover the largest own block index of the call
  const int max_own = (a.first_pos + a.n_q - 1) / kBlock;
  const int slots = (max_own + 63) / 64;
  if (slots <= 1) return launch_slots<1>(a, stream);
  if (slots <= 2) return launch_slots<2>(a, stream);
  if (slots <= 4) return launch_slots<4>(a, stream);
  if (slots <= 8) return launch_slots<8>(a, stream);
  if (slots <= 16) return launch_slots<16>(a, stream);
  if (slots <= 32) return launch_slots<32>(a, stream);
  return launch_slots<64>(a, stream);   // the host admits at most 4,096 blocks
}

}  // namespace selattn
