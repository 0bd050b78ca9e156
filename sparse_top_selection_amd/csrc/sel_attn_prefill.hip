// The attention step over each group's union: one work-group per (group of 8
// positions, KV head). The design and the page's sections it follows are
// described in sel_attn_prefill_dev.h, which holds the device code.

#include "sel_attn_prefill_dev.h"

namespace selattn {
namespace {

__global__ __launch_bounds__(kThreads, 2) void sel_attn_prefill_kernel(PrefillArgs a) {
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
  const int nch = (U + kChunk - 1) / kChunk;   // chunks of the union

  if (wave < kConsumerWaves) {
    consume<false>(a, sm, g, h, nch, wave, lane, nullptr);
  } else {
    // the producers' work paces every wave (all wait for its stage at the
    // barrier), so their instructions go first on the SIMDs they share
    __builtin_amdgcn_s_setprio(1);
    const int ptid = tid - 64 * kConsumerWaves;
    produce(a, sm, h, U, nch, ubase, ptid, ptid < kChunk, flags);
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
