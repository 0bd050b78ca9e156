// The attention step for grids too small to fill the GPU: each (group, KV head)'s
// union divided at chunk boundaries over several work-groups, each running the
// same kernel body over its share and writing its unnormalised state, then a
// merge of the shares of every row. In a translation unit of its own, so that
// the single-share kernel of sel_attn_prefill.hip compiles exactly as alone.
//
// Page: #2808 "sycl: prompt attention over 8-query selection unions on XMX",
// section Summary: the online softmax over a union's chunks, whose partial
// states combine by their maxima.

#include "sel_attn_prefill_dev.h"

namespace selattn {
namespace {

// One share of a (group, KV head)'s union (sel_attn_prefill_split): the same
// work-group as sel_attn_prefill_kernel over chunks [c0, c1) of the union,
// walked as a union of its own that starts at entry 32 c0 (inside the group's
// row, or its first entry), writing a PrefillPartial record instead of out.
__global__ __launch_bounds__(kThreads, 2) void sel_attn_prefill_split_kernel(PrefillArgs a) {
  __shared__ Smem sm;

  const int b = blockIdx.x;
  const int S = a.n_splits;
  const int W = (b & 7) * a.per_xcd + (b >> 3);   // (group, KV head) L times S, split sp
  if (W >= a.n_groups * a.n_kv * S) return;
  const int L = W / S;
  const int sp = W - L * S;
  const int h = L / a.n_groups;
  const int g = L - h * a.n_groups;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t ucap = 8LL * a.sel_cap;
  uint32_t flags = 0;

  int U_all = a.union_len[g];
  if (U_all < 0 || U_all > ucap) {
    flags |= SEL_ATTN_STATUS_UNION_LEN;
    U_all = U_all < 0 ? 0 : (int)ucap;
  }
  const int nch_all = (U_all + kChunk - 1) / kChunk;
  const int c0 = (int)((int64_t)sp * nch_all / S);
  const int c1 = (int)((int64_t)(sp + 1) * nch_all / S);
  const int64_t ubase = (int64_t)g * ucap + (int64_t)c0 * kChunk;
  const int U = max(0, min(U_all, c1 * kChunk) - c0 * kChunk);
  const int nch = c1 - c0;

  if (wave < kConsumerWaves) {
    consume<true>(a, sm, g, h, nch, wave, lane, a.part + W);
  } else {
    __builtin_amdgcn_s_setprio(1);
    const int ptid = tid - 64 * kConsumerWaves;
    produce(a, sm, h, U, nch, ubase, ptid, ptid < kChunk, flags);
  }
  if (flags) atomicOr(a.status, flags);
}

// Merge of the splits of one (group, KV head): a work-group per query head of
// the KV head (8 rows, one per position), 32 threads per row, 4 dims each. The
// splits' states are weighted by exp2(m_s - max m), then O / (2^6 l); 0 when no
// split saw a kept cell. Every split's loads are issued before the first is
// used.
constexpr int kMergeThreads = 256;
constexpr int kMaxSplits = kPrefillMaxSplits;

__global__ __launch_bounds__(kMergeThreads) void prefill_merge_kernel(PrefillArgs a) {
  const int L = blockIdx.x / kQPerKv;
  const int hq = blockIdx.x - kQPerKv * L;
  const int i = threadIdx.x >> 5;           // position within the group
  const int d4 = threadIdx.x & 31;          // dims 4 d4 .. 4 d4 + 3
  const int h = L / a.n_groups;
  const int g = L - h * a.n_groups;
  const int qi = 8 * g + i;
  if (qi >= a.n_q) return;
  const int row_n = 8 * hq + i;
  const int S = a.n_splits;
  const PrefillPartial* p = a.part + (int64_t)L * S;

  float ms[kMaxSplits], ls[kMaxSplits];
  float4v os[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    const int sc = s < S ? s : 0;
    ms[s] = p[sc].m[row_n];
    ls[s] = p[sc].l[row_n];
    os[s] = *reinterpret_cast<const float4v*>(&p[sc].o[row_n][4 * d4]);
  }
  float m = ms[0];
#pragma unroll
  for (int s = 1; s < kMaxSplits; ++s) m = s < S ? fmaxf(m, ms[s]) : m;
  float l = 0.f;
  float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    const float w = s < S ? __builtin_amdgcn_exp2f(ms[s] - m) : 0.f;
    l = __builtin_fmaf(w, ls[s], l);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(w, os[s][e], acc[e]);
  }
  const float inv = l > 0.f ? (1.f / kVFold) / l : 0.f;
  float4v r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = acc[e] * inv;
  const int n_qh = a.n_kv * kQPerKv;
  *reinterpret_cast<float4v*>(a.out + ((int64_t)qi * n_qh + h * kQPerKv + hq) * kD + 4 * d4) = r;
}

}  // namespace

hipError_t launch_prefill_split(const PrefillArgs& a, hipStream_t stream) {
  const int grid = 8 * a.per_xcd;
  hipLaunchKernelGGL(sel_attn_prefill_split_kernel, dim3(grid), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prefill_merge_kernel, dim3(a.n_groups * a.n_kv * kQPerKv), dim3(kMergeThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace selattn
