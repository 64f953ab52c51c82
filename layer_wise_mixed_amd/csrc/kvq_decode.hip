// kvq_decode.hip -- split-KV decode attention over the packed cache, and the
// log-sum-exp merge of the splits (TriAxialKV page, "Facts": flash-decoding
// splits merged by online log-sum-exp).
//
// Split pass: one workgroup per (split, KV head, request). The split walks its
// share of the stream's 32-token groups (the fp16 tail counts as one more,
// partial group, so it lands in the last non-empty split), dequantizes each
// group in registers into LDS, forms the scores of the G query rows of the
// GQA group, and keeps a running max and sum per row (exp2 domain). It writes
// the row outputs normalised over its own tokens and their log-sum-exp.
#include "kvq_internal.h"

namespace kvq {
namespace {

__device__ inline float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

__device__ inline float elem(const uint8_t* blk, const float* meta, int bits, int mi, int lane, int e) {
  uint32_t off;
  int sh;
  code_site(lane, e, bits, &off, &sh);
  const uint32_t word = *(const uint32_t*)(blk + off);
  if (bits == 16) return h2f((uint16_t)(word >> sh));
  const uint32_t code = (word >> sh) & ((1u << bits) - 1u);
  return fmaf((float)code, meta[mi], meta[128 + mi]);
}

constexpr int kMaxG = 16;

__global__ __launch_bounds__(256) void split_kernel_lds(DecodeArgs a) {
  __shared__ float qs[kMaxG][D];
  __shared__ float ks[GS][D + 1];
  __shared__ float vs[GS][D];
  __shared__ float sc[kMaxG][GS];
  const LayerGeom& g = a.geo;
  const int tid = threadIdx.x;
  const int split = blockIdx.x, h = blockIdx.y, r = blockIdx.z;
  const int G = g.g;
  int L = a.seq_lens[r];
  if (L < 0) L = 0;
  if (L > g.max_tokens) L = g.max_tokens;
  const int nq = L / GS;
  const int T = L - nq * GS;
  const int nvg = nq + (T > 0);
  const int g0 = split * a.groups_per_split;
  const int g1 = min(g0 + a.groups_per_split, nvg);
  const int sigma = r * g.hkv + h;
  const uint8_t* stream = g.base + (size_t)sigma * g.stream_bytes;

  for (int idx = tid; idx < G * D; idx += blockDim.x) {
    const int gg = idx >> 7, c = idx & 127;
    qs[gg][c] = h2f(a.q[((size_t)r * g.hq + h * G + gg) * D + c]);
  }
  // this thread accumulates channel c of rows gr, gr + 2, ...
  const int c = tid & 127;
  const int gr = tid >> 7;
  float o[kMaxG / 2], m[kMaxG / 2], l[kMaxG / 2];
#pragma unroll
  for (int k = 0; k < kMaxG / 2; ++k) {
    o[k] = 0.f;
    m[k] = -INFINITY;
    l[k] = 0.f;
  }

  for (int vg = g0; vg < g1; ++vg) {
    const bool full = vg < nq;
    const uint8_t* rec = full ? stream + (size_t)vg * g.record_bytes : stream + g.tail_offset;
    const int kb = full ? g.kb : 16, vb = full ? g.vb : 16;
    const int ntok = full ? GS : T;
    const RecordParts parts = record_parts(kb, vb);
    const float* kmeta = (const float*)(rec + parts.kmeta);
    const float* vmeta = (const float*)(rec + parts.vmeta);
    __syncthreads();  // previous group's LDS reads are done
    for (int idx = tid; idx < GS * D; idx += blockDim.x) {
      const int j = idx >> 7, cc = idx & 127;
      float kv = 0.f, vv = 0.f;
      if (j < ntok) {
        int lane, e;
        k_site(j, cc, &lane, &e);
        kv = elem(rec, kmeta, kb, g.k_token ? meta_token(j, cc >> 5) : meta_channel(cc), lane, e);
        v_site(j, cc, &lane, &e);
        vv = elem(rec + parts.vcode, vmeta, vb, meta_token(j, cc >> 5), lane, e);
      }
      ks[j][cc] = kv;
      vs[j][cc] = vv;
    }
    __syncthreads();
    for (int idx = tid; idx < G * GS; idx += blockDim.x) {
      const int gg = idx >> 5, j = idx & 31;
      float acc = 0.f;
#pragma unroll 8
      for (int cc = 0; cc < D; ++cc) acc = fmaf(qs[gg][cc], ks[j][cc], acc);
      sc[gg][j] = (j < ntok) ? acc * a.scale_log2 : -INFINITY;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kMaxG / 2; ++k) {
      const int gg = gr + 2 * k;
      if (gg >= G) break;
      float mb = -INFINITY;
      for (int j = 0; j < GS; ++j) mb = fmaxf(mb, sc[gg][j]);
      const float mnew = fmaxf(m[k], mb);
      const float alpha = (m[k] == -INFINITY) ? 0.f : exp2f(m[k] - mnew);
      float ps = 0.f, acc = 0.f;
      for (int j = 0; j < GS; ++j) {
        const float p = exp2f(sc[gg][j] - mnew);
        ps += p;
        acc = fmaf(p, vs[j][c], acc);
      }
      o[k] = o[k] * alpha + acc;
      l[k] = l[k] * alpha + ps;
      m[k] = mnew;
    }
  }
#pragma unroll
  for (int k = 0; k < kMaxG / 2; ++k) {
    const int gg = gr + 2 * k;
    if (gg >= G) break;
    const size_t row = ((size_t)r * g.hq + h * G + gg) * a.splits + split;
    a.part_o[row * D + c] = (l[k] > 0.f) ? o[k] / l[k] : 0.f;
    if (c == 0) a.part_lse[row] = (l[k] > 0.f) ? (m[k] + log2f(l[k])) * 0.69314718055994531f : -INFINITY;
  }
}

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

hipError_t launch_decode_split(const DecodeArgs& a, int batch, hipStream_t s) {
  dim3 grid(a.splits, a.geo.hkv, batch);
  hipLaunchKernelGGL(split_kernel_lds, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(merge_kernel, dim3(a.rows), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
