// kvq_decode.hip -- the second pass of split-KV decode attention: the
// log-sum-exp merge of the splits (TriAxialKV page, "Facts": flash-decoding
// splits merged by online log-sum-exp). Each split left its rows normalised
// over its own tokens, plus their log-sum-exp; the merge weights split s by
// exp(lse_s - max lse) and renormalises. Splits without tokens (lse = -inf)
// get weight 0; a row with no tokens at all gets 0 and lse = -inf.
#include "kvq_internal.h"

namespace kvq {
namespace {

// The common case (at most kFast splits) loads every lse and every partial
// of the thread's channel in one go, so the merge waits on memory once;
// more splits take the loop.
constexpr int kFast = 8;

__device__ __forceinline__ void merge_store(const MergeArgs& a, int row, int c, float res, float out_lse) {
  if (a.out_f32)
    ((float*)a.out)[(size_t)row * D + c] = res;
  else
    ((_Float16*)a.out)[(size_t)row * D + c] = (_Float16)res;
  if (c == 0 && a.lse_out) a.lse_out[row] = out_lse;
}

__global__ __launch_bounds__(128) void merge_kernel(MergeArgs a) {
  const int row = blockIdx.x;
  const int c = threadIdx.x;
  const float* lse = a.part_lse + (size_t)row * a.splits;
  const float* po = a.part_o + (size_t)row * a.splits * D + c;
  if (a.splits <= kFast) {
    float ls[kFast], o[kFast];
#pragma unroll
    for (int s = 0; s < kFast; ++s) {
      ls[s] = s < a.splits ? lse[s] : -INFINITY;
      o[s] = s < a.splits ? po[(size_t)s * D] : 0.f;
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < kFast; ++s) M = fmaxf(M, ls[s]);
    float res = 0.f, out_lse = -INFINITY;
    if (M != -INFINITY) {
      float wsum = 0.f, acc = 0.f;
#pragma unroll
      for (int s = 0; s < kFast; ++s) {
        if (ls[s] == -INFINITY) continue;
        const float w = expf(ls[s] - M);
        wsum += w;
        acc = fmaf(w, o[s], acc);
      }
      res = acc / wsum;
      out_lse = M + logf(wsum);
    }
    merge_store(a, row, c, res, out_lse);
    return;
  }
  float M = -INFINITY;
  for (int s = 0; s < a.splits; ++s) M = fmaxf(M, lse[s]);
  float res = 0.f, out_lse = -INFINITY;
  if (M != -INFINITY) {
    float wsum = 0.f, acc = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      const float ls = lse[s];
      if (ls == -INFINITY) continue;
      const float w = expf(ls - M);
      wsum += w;
      acc = fmaf(w, po[(size_t)s * D], acc);
    }
    res = acc / wsum;
    out_lse = M + logf(wsum);
  }
  merge_store(a, row, c, res, out_lse);
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t s, const EventPair* ev) {
  return launch_timed(merge_kernel, dim3(a.rows), dim3(128), s, ev, a);
}

}  // namespace kvq
