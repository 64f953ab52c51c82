// kvq_append.hip -- quantize-and-pack on append, and the checking dequantizer.
//
// The group quantizer and packer are in kvq_quantize.h. Keys are grouped per
// channel over 32 tokens (KVTuner summary page, "Facts": keys have
// channel-wise outliers) or per token over 32 channels; values per token.
// Tokens that do not fill a group stay fp16 in the stream's tail record.
#include "kvq_internal.h"
#include "kvq_quantize.h"

#pragma clang fp contract(off)

namespace kvq {
namespace {

// One workgroup of two waves per (x, stream, tensor): it completes the
// tensor's part (keys for blockIdx.z = 0, values for 1) of the x-th of
// gridDim.x runs of consecutive groups of this call; keys and values of one
// group are quantized by different workgroups that never wait on each other.
// While one group is quantized the fp16 rows of its next whole-new group are
// already loading (in registers), so that the stream of loads does not stop
// for the arithmetic.
__global__ __launch_bounds__(128) void append_kernel(AppendArgs a) {
  typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(16))) uint16_t xs[GS][D];
  __shared__ __attribute__((aligned(16))) uint8_t cs[GS][CS];
  const LayerGeom& g = a.geo;
  const int tid = threadIdx.x;
  const int sigma = blockIdx.y;
  const int is_v = blockIdx.z;
  const int r = sigma / g.hkv;
  const int L0 = a.seq_lens[r];
  const int L1 = L0 + a.n_new;
  if (L0 < 0 || L1 > g.max_tokens) return;  // would pass the planned capacity
  const int m0 = L0 / GS;
  const int F = L1 / GS - m0;  // groups this call completes
  uint8_t* stream = g.base + (size_t)sigma * g.stream_bytes;
  uint8_t* tail = stream + g.tail_offset;
  const uint16_t* src = (is_v ? a.v_new : a.k_new) + (size_t)sigma * a.n_new * D;

  // a whole-new group's 32 contiguous rows of this tensor, 8 KiB: four
  // 16-byte pieces a thread, non-temporal (read once; measured 4-15% faster
  // for the whole prompt than ordinary loads)
  constexpr int kPer = GS * D / 8 / 128;
  u4_t xa[kPer];
  auto fetch = [&](int y) {
    const u4_t* xsrc = (const u4_t*)(src + (size_t)(GS * (m0 + y) - L0) * D);
#pragma unroll
    for (int q = 0; q < kPer; ++q) xa[q] = __builtin_nontemporal_load(&xsrc[tid + 128 * q]);
  };
  auto whole_new = [&](int y) { return GS * (m0 + y) >= L0; };

  const int run = (F + gridDim.x - 1) / gridDim.x;
  const int yend = min(F, (blockIdx.x + 1) * run);
  int y = blockIdx.x * run;
  if (y < yend && whole_new(y)) fetch(y);
  for (; y < yend; ++y) {
    const int m = m0 + y;
    if (whole_new(y)) {
#pragma unroll
      for (int q = 0; q < kPer; ++q) ((u4_t*)&xs[0][0])[tid + 128 * q] = xa[q];
    } else {
#pragma unroll 1
      for (int idx = tid; idx < GS * D; idx += blockDim.x) {
        const int i = idx >> 7, c = idx & 127;
        const int t = GS * m + i;
        // earlier tokens of this group wait in the tail
        xs[i][c] = t < L0 ? tail_get(tail, is_v, i, c) : src[(size_t)(t - L0) * D + c];
      }
    }
    __syncthreads();
    if (y + 1 < yend && whole_new(y + 1)) fetch(y + 1);  // in flight during the quantization
    quantize_tensor(xs, cs, stream + (size_t)m * g.record_bytes, is_v, g.kb, g.vb, g.k_token, tid);
    __syncthreads();  // the next group rewrites xs and cs
  }
  if (blockIdx.x == 0) {  // after its flush (if any) has read the old tail slots
    const int tstart = max(L0, GS * (L1 / GS));
    const int nt = L1 - tstart;
    for (int idx = tid; idx < nt * D; idx += blockDim.x) {
      const int t = tstart + (idx >> 7), c = idx & 127;
      tail_put(tail, is_v, t % GS, c, src[(size_t)(t - L0) * D + c]);
    }
  }
}

__device__ inline float read_elem(const uint8_t* rec, const RecordParts& parts, int kb, int vb, int k_token,
                                  bool is_v, int j, int c) {
  const int bits = is_v ? vb : kb;
  const uint8_t* blk = rec + (is_v ? parts.vcode : 0);
  int lane, e;
  if (is_v) v_site(j, c, &lane, &e); else k_site(j, c, &lane, &e);
  uint32_t off;
  int sh;
  code_site(lane, e, bits, &off, &sh);
  const uint32_t word = *(const uint32_t*)(blk + off);
  if (bits == 16) return h2f((uint16_t)(word >> sh));
  const uint32_t code = (word >> sh) & ((1u << bits) - 1u);
  const float* meta = (const float*)(rec + (is_v ? parts.vmeta : parts.kmeta));
  const int mi = (is_v || k_token) ? meta_token(j, c >> 5) : meta_channel(c);
  return fmaf((float)code, meta[mi], meta[128 + mi]);
}

__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a) {
  const LayerGeom& g = a.geo;
  const int m = blockIdx.x;
  const int sigma = blockIdx.y;
  const int r = sigma / g.hkv;
  const int L = a.seq_lens[r];
  if (L < 0 || L > g.max_tokens) return;
  const int lw = min(L, a.max_seq_len);  // rows past max_seq_len have no room in k_out
  const int nq = L / GS;
  if (m * GS >= lw) return;
  const uint8_t* stream = g.base + (size_t)sigma * g.stream_bytes;
  const bool full = m < nq;
  const uint8_t* rec = full ? stream + (size_t)m * g.record_bytes : stream + g.tail_offset;
  const int kb = full ? g.kb : 16, vb = full ? g.vb : 16;
  const RecordParts parts = record_parts(kb, vb);
  for (int idx = threadIdx.x; idx < GS * D; idx += blockDim.x) {
    const int j = idx >> 7, c = idx & 127;
    const int t = m * GS + j;
    if (t >= lw) continue;
    const size_t o = ((size_t)sigma * a.max_seq_len + t) * D + c;
    a.k_out[o] = read_elem(rec, parts, kb, vb, g.k_token, false, j, c);
    a.v_out[o] = read_elem(rec, parts, kb, vb, g.k_token, true, j, c);
  }
}

// Paged append, one workgroup per (block x, request, KV head). Blocks
// x < n_new / 32 quantize INT2 group x (new tokens 32x .. 32x+31, when they
// are among the request's first int2_add[r] new tokens) into its page pair;
// the others write INT4 page int4_len[r] / 16 + (x - n_new / 32) with the new
// INT4 tokens that fall in it (TriAxialKV page, "Facts": leftover INT2
// tokens take the INT4 per-token path).
__global__ __launch_bounds__(256) void paged_append_kernel(AppendArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][GS][D];
  __shared__ __attribute__((aligned(16))) uint8_t cs[2][GS][CS];
  const LayerGeom& g = a.geo;
  const PagedGeom& pg = a.pg;
  const int tid = threadIdx.x;
  const int x = blockIdx.x;
  const int sigma = blockIdx.y;
  const int r = sigma / g.hkv, h = sigma % g.hkv;
  const int n2_old = pg.int2_len[r], n4_old = pg.int4_len[r];
  const int add2 = pg.int2_add ? pg.int2_add[r] : 0;
  if (n2_old < 0 || n4_old < 0 || add2 < 0 || add2 > a.n_new || (add2 % GS) != 0 || (n2_old % GS) != 0) return;
  const int32_t* table = pg.table + (size_t)r * pg.max_pages;
  const uint16_t* kn = a.k_new + (size_t)sigma * a.n_new * D;
  const uint16_t* vn = a.v_new + (size_t)sigma * a.n_new * D;
  const int x2 = a.n_new / GS;

  if (x < x2) {  // ------------------------------------------- INT2 group
    if (GS * (x + 1) > add2) return;
    for (int idx = tid; idx < GS * D; idx += blockDim.x) {
      const int i = idx >> 7, c = idx & 127;
      xs[0][i][c] = kn[(size_t)(GS * x + i) * D + c];
      xs[1][i][c] = vn[(size_t)(GS * x + i) * D + c];
    }
    __syncthreads();
    const int entry = (n2_old + GS * x) / PAGE_TOKENS;
    const int pair = entry + 1 < pg.max_pages ? table[entry] : -1;
    if (!int2_pair_ok(pg, entry, pair)) return;  // a bad table entry: nothing is written
    uint8_t* rec = g.base + (size_t)pair * pg.int2_page_bytes + (size_t)h * INT2_RECORD;
    quantize_record(xs, cs, rec, 2, 2, 0, tid);
    return;
  }

  // ------------------------------------------------------ one INT4 page
  const int n4_add = a.n_new - add2;
  const int P = n4_old / PAGE_TOKENS + (x - x2);
  const int t_lo = max(n4_old, PAGE_TOKENS * P), t_hi = min(n4_old + n4_add, PAGE_TOKENS * (P + 1));
  if (t_lo >= t_hi) return;
  const int p_lo = t_lo - PAGE_TOKENS * P, p_hi = t_hi - PAGE_TOKENS * P;  // slots written
  const int entry = (n2_old + add2) / PAGE_TOKENS + P;
  const int id = entry < pg.max_pages ? table[entry] : -1;
  if (!int4_page_ok(pg, entry, id)) return;  // a bad table entry: nothing is written
  uint8_t* page = g.base + pg.int4_offset + (size_t)(id - pg.int2_pages) * pg.int4_page_bytes + (size_t)h * INT4_HEAD;
  for (int idx = tid; idx < PAGE_TOKENS * D; idx += blockDim.x) {
    const int p = idx >> 7, c = idx & 127;
    if (p < p_lo || p >= p_hi) continue;
    const size_t i = (size_t)(add2 + PAGE_TOKENS * P + p - n4_old);  // index among the new tokens
    xs[0][p][c] = kn[i * D + c];
    xs[1][p][c] = vn[i * D + c];
  }
  __syncthreads();
  page_append_int4(page, xs, cs, p_lo, p_hi, tid);
}

__global__ __launch_bounds__(256) void paged_dequant_kernel(DequantArgs a) {
  const LayerGeom& g = a.geo;
  const PagedGeom& pg = a.pg;
  const int m = blockIdx.x;
  const int sigma = blockIdx.y;
  const int r = sigma / g.hkv, h = sigma % g.hkv;
  const int n2 = pg.int2_len[r], n4 = pg.int4_len[r];
  if (n2 < 0 || n4 < 0 || (n2 % GS) != 0) return;
  const int lw = min(n2 + n4, a.max_seq_len);
  const int32_t* table = pg.table + (size_t)r * pg.max_pages;
  const RecordParts parts = record_parts(2, 2);
  for (int idx = threadIdx.x; idx < GS * D; idx += blockDim.x) {
    const int t = m * GS + (idx >> 7), c = idx & 127;
    if (t >= lw) continue;
    const size_t o = ((size_t)sigma * a.max_seq_len + t) * D + c;
    if (t < n2) {
      const uint8_t* rec =
          g.base + (size_t)table[t / PAGE_TOKENS & ~1] * pg.int2_page_bytes + (size_t)h * INT2_RECORD;
      a.k_out[o] = read_elem(rec, parts, 2, 2, 0, false, t % GS, c);
      a.v_out[o] = read_elem(rec, parts, 2, 2, 0, true, t % GS, c);
    } else {
      const int u = t - n2, p = u % PAGE_TOKENS;
      const uint8_t* page = g.base + pg.int4_offset +
                            (size_t)(table[n2 / PAGE_TOKENS + u / PAGE_TOKENS] - pg.int2_pages) * pg.int4_page_bytes +
                            (size_t)h * INT4_HEAD;
      const float* km = (const float*)(page + INT4_KMETA);
      const float* vm = (const float*)(page + INT4_VMETA);
      const int mi = 16 * (c >> 5) + p;
      int sh;
      uint32_t off = page_k_offset(p, c, &sh);
      a.k_out[o] = fmaf((float)((*(const uint32_t*)(page + off) >> sh) & 15u), km[mi], km[64 + mi]);
      off = page_v_offset(p, c, &sh);
      a.v_out[o] = fmaf((float)((*(const uint32_t*)(page + off) >> sh) & 15u), vm[mi], vm[64 + mi]);
    }
  }
}

}  // namespace

hipError_t launch_append_paged(const AppendArgs& a, int batch, hipStream_t s, const EventPair* ev) {
  if (a.n_new == 0 || batch == 0) return hipSuccess;
  const int x = a.n_new / GS + (a.n_new + PAGE_TOKENS - 1) / PAGE_TOKENS + 1;
  return launch_timed(paged_append_kernel, dim3(x, batch * a.geo.hkv), dim3(256), s, ev, a);
}

hipError_t launch_dequant_paged(const DequantArgs& a, int batch, hipStream_t s) {
  const int y = (a.max_seq_len + GS - 1) / GS;
  if (y == 0 || batch == 0) return hipSuccess;
  hipLaunchKernelGGL(paged_dequant_kernel, dim3(y, batch * a.geo.hkv), dim3(256), 0, s, a);
  return hipGetLastError();
}

// (run, stream) workgroups per tensor of a long append, about: with both
// tensors about 4.5 rounds of the 8 two-wave workgroups a CU holds at this
// kernel's register count (256 CUs). Measured on a 2047-token prefill of 512
// streams (63 full groups each): runs of 13 groups (2,560 workgroups a
// tensor) 163-165 us, of 9 (3,584) 159-163 us, of 7 (4,608) 157-160 us, of 8
// (4,096) 204-207 us. A run of 2^k groups starts 2^k x 8 KiB into its
// stream's fp16 input, and that stride is avoided.
constexpr int kAppendRuns = 4608;

hipError_t launch_append(const AppendArgs& a, int batch, hipStream_t s, const EventPair* ev) {
  const int y = a.n_new > 0 ? (a.n_new + GS - 1) / GS : 0;
  if (y == 0 || batch == 0) return hipSuccess;
  // long appends (prefill): about kAppendRuns (run, stream) workgroups per
  // tensor, each looping over a run of equal length of its stream's groups
  // (sized on the full groups of an append to an empty stream); short ones: a
  // workgroup per group
  const int streams = batch * a.geo.hkv;
  int x = y;
  if (y > 8) {
    const int full = a.n_new / GS;
    const int x0 = (kAppendRuns + streams - 1) / streams;
    int r = (full + x0 - 1) / x0;  // groups a run
    if (r >= 4 && (r & (r - 1)) == 0) --r;
    x = (full + r - 1) / r;
    if (x > y) x = y;
  }
  return launch_timed(append_kernel, dim3(x, streams, 2), dim3(128), s, ev, a);
}

hipError_t launch_dequant(const DequantArgs& a, int batch, hipStream_t s) {
  const int y = (a.max_seq_len + GS - 1) / GS;
  if (y == 0 || batch == 0) return hipSuccess;
  dim3 grid(y, batch * a.geo.hkv);
  hipLaunchKernelGGL(dequant_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
