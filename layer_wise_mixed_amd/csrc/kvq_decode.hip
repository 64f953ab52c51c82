// kvq_decode.hip -- the second pass of split-KV decode attention: the
// log-sum-exp merge of the splits (TriAxialKV page, "Facts": flash-decoding
// splits merged by online log-sum-exp). Each split left its rows normalised
// over its own tokens, plus their log-sum-exp; the merge weights split s by
// exp(lse_s - max lse) and renormalises. Splits without tokens (lse = -inf)
// get weight 0; a row with no tokens at all gets 0 and lse = -inf.
#include "kvq_internal.h"

namespace kvq {
namespace {

__global__ __launch_bounds__(128) void merge_kernel(MergeArgs a) {
  const int row = blockIdx.x;
  const int c = threadIdx.x;
  const float* lse = a.part_lse + (size_t)row * a.splits;
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
      acc = fmaf(w, a.part_o[((size_t)row * a.splits + s) * D + c], acc);
    }
    res = acc / wsum;
    out_lse = M + logf(wsum);
  }
  if (a.out_f32)
    ((float*)a.out)[(size_t)row * D + c] = res;
  else
    ((_Float16*)a.out)[(size_t)row * D + c] = (_Float16)res;
  if (c == 0 && a.lse_out) a.lse_out[row] = out_lse;
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t s, const EventPair* ev) {
  return launch_timed(merge_kernel, dim3(a.rows), dim3(128), s, ev, a);
}

}  // namespace kvq
