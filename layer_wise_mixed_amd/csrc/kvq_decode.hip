// kvq_decode.hip -- the second pass of split-KV decode attention: the
// log-sum-exp merge of the splits (TriAxialKV page, "Facts": flash-decoding
// splits merged by online log-sum-exp). Each split left its rows normalised
// over its own tokens, plus their log-sum-exp; the merge weights split s by
// exp(lse_s - max lse) and renormalises. Splits without tokens (lse = -inf)
// get weight 0; a row with no tokens at all gets 0 and lse = -inf.
#include "kvq_internal.h"

namespace kvq {
namespace {

// Four rows a 128-thread workgroup, four channels a thread (16-byte loads and
// stores). The common case (at most kFast splits) loads every lse and every
// partial of the thread's channels in one go, so the merge waits on memory
// once; more splits take the loop.
constexpr int kFast = 8;
constexpr int kRowsPerBlock = 4;

typedef float f4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void merge_store(const MergeArgs& a, int row, int c, f4_t res, float out_lse) {
  if (a.out_f32) {
    *(f4_t*)((float*)a.out + (size_t)row * D + c) = res;
  } else {
    typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
    h4_t h;
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = (_Float16)res[i];
    *(h4_t*)((_Float16*)a.out + (size_t)row * D + c) = h;
  }
  if (c == 0 && a.lse_out) a.lse_out[row] = out_lse;
}

__global__ __launch_bounds__(128) void merge_kernel(MergeArgs a) {
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 5);
  const int c = 4 * (threadIdx.x & 31);
  if (row >= a.rows) return;
  const float* lse = a.part_lse + (size_t)row * a.splits;
  const float* po = a.part_o + (size_t)row * a.splits * D + c;
  if (a.splits <= kFast) {
    float ls[kFast];
    f4_t o[kFast];
#pragma unroll
    for (int s = 0; s < kFast; ++s) {
      ls[s] = s < a.splits ? lse[s] : -INFINITY;
      o[s] = s < a.splits ? *(const f4_t*)(po + (size_t)s * D) : f4_t{0.f, 0.f, 0.f, 0.f};
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < kFast; ++s) M = fmaxf(M, ls[s]);
    f4_t res = {0.f, 0.f, 0.f, 0.f};
    float out_lse = -INFINITY;
    if (M != -INFINITY) {
      float wsum = 0.f;
      f4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < kFast; ++s) {
        if (ls[s] == -INFINITY) continue;
        const float w = expf(ls[s] - M);
        wsum += w;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(w, o[s][i], acc[i]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) res[i] = acc[i] / wsum;
      out_lse = M + logf(wsum);
    }
    merge_store(a, row, c, res, out_lse);
    return;
  }
  float M = -INFINITY;
  for (int s = 0; s < a.splits; ++s) M = fmaxf(M, lse[s]);
  f4_t res = {0.f, 0.f, 0.f, 0.f};
  float out_lse = -INFINITY;
  if (M != -INFINITY) {
    float wsum = 0.f;
    f4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < a.splits; ++s) {
      const float ls = lse[s];
      if (ls == -INFINITY) continue;
      const float w = expf(ls - M);
      wsum += w;
      const f4_t x = *(const f4_t*)(po + (size_t)s * D);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(w, x[i], acc[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) res[i] = acc[i] / wsum;
    out_lse = M + logf(wsum);
  }
  merge_store(a, row, c, res, out_lse);
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t s, const EventPair* ev) {
  return launch_timed(merge_kernel, dim3((a.rows + kRowsPerBlock - 1) / kRowsPerBlock), dim3(128), s, ev, a);
}

}  // namespace kvq
