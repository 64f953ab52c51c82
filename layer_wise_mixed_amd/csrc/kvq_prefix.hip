// kvq_prefix.hip -- attention over a quantized prefix for chunked prefill.
//
// A chunk brings many query rows per KV head (chunk tokens x G heads), so the
// work per packed group is a dense contraction and the matrix cores, not HBM,
// set the pace. Unlike the decode split pass, which folds the scales into
// the per-row operands (cheap for a few rows, costly for many), each group is
// dequantized ONCE per workgroup into LDS and shared by all its rows:
//
//   workgroup = 8 waves x kNT 16-row column tiles = 256 rows of one (request,
//               KV head), walking every group of its split;
//   per group  the 512 threads dequantize the record (fmaf(code, scale, zero)
//              in fp32, KIVI and KVTuner summary pages: asymmetric groupwise
//              codes; keys per channel or per token, values per token) into
//              fp16 operands kept in the record's own lane order: octet o of
//              lane l is the MFMA operand lane l needs (16x16x32 f16 tiles).
//              Keys as a high and a low plane, x = hi + lo with lo = fp16(x -
//              hi); values as one plane, rounded to nearest;
//   scores     S[token][row] = (K_hi.q + K_lo.q) * softmax_scale * log2(e):
//              q is fp16 already, so two products keep ~22 significant bits
//              (a score's absolute error sets the weights' relative error);
//   softmax    exp2 of (score - reference max); the reference is raised
//              (and the sums rescaled) only when a score exceeds it by more
//              than kSlack, so most groups need no cross-lane max at all;
//   output     O^T[ch][row] += V^T . P with V and P each rounded once to fp16
//              (nearest): a relative error of about 2^-11 a term, unbiased,
//              in fp32 sums.
// The next group's record loads are in flight while the current group is
// multiplied; its dequantization goes to the second LDS buffer, and one
// barrier per group separates the two. The fp16 tail is dequantized the same
// way (its values are already fp16: lo = 0) with its empty slots masked.
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kNT = 2;                    // 16-row column tiles per wave
constexpr int kRows = kWaves * kNT * 16;  // rows per workgroup
constexpr float kSlack = 8.0f;            // p = exp2(score - reference) stays <= 2^8

__device__ inline f4_t mfma(h8_t a, h8_t b, f4_t c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

// x = hi + lo for 8 floats: hi a round-toward-zero fp16 (one packed
// conversion per pair), lo the fp16 of what it missed
__device__ inline void split8(const float* x, h8_t& hi, h8_t& lo) {
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const auto h = __builtin_amdgcn_cvt_pkrtz(x[i], x[i + 1]);
    const auto l = __builtin_amdgcn_cvt_pkrtz(x[i] - (float)h[0], x[i + 1] - (float)h[1]);
    hi[i] = h[0];
    hi[i + 1] = h[1];
    lo[i] = l[0];
    lo[i + 1] = l[1];
  }
}

// 8 floats rounded to nearest fp16
__device__ inline h8_t to_h8(const float* x) {
  h8_t h;
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (_Float16)x[i];
  return h;
}

__device__ inline float sum_lane_groups(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__device__ inline float max_lane_groups(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

// One group's operands: octet o (8 fp16) of lane l at [o][l]. Keys: octet
// 4t + s holds token 16t + l%16, channels 32s + 8(l/16) .. + 7. Values:
// octet u holds channel 16u + l%16 for the tokens 16(i/4) + 4(l/16) + i%4,
// i = 0..7, the order in which the score tile leaves them in each lane.
struct GroupBuf {
  h8_t khi[8][64], klo[8][64], vhi[8][64];
};

// A thread's share of a record: lane `lane`, key octet w (token
// 16(w/4) + lane%16, channels 32(w%4) + 8(lane/16) .. + 7) and value octet w
// (channel 16w + lane%16, the tokens of slots 8(lane/16) + i), with the
// scales and zeros they need; w = the thread's wave.
template <int KB, int VB, bool KTOK>
struct Share {
  static constexpr int NKW = KB < 4 ? 1 : KB / 4, NVW = VB < 4 ? 1 : VB / 4;  // words per octet
  static constexpr int NKM = KB == 16 ? 1 : (KTOK ? 1 : 8);
  static constexpr int NVM = VB == 16 ? 1 : 8;
  uint32_t kw[NKW], vw[NVW];
  float ks[NKM], kz[NKM], vs[NVM], vz[NVM];
};

// The words of `lane` that hold octet o (positions 8o .. 8o + 7) of a code
// block of B-bit codes (32 / B positions a word, see word_offset); 2-bit
// octets are half a word.
template <int B>
__device__ __forceinline__ void load_octet(const uint8_t* blk, int o, int lane, uint32_t* out) {
  if constexpr (B == 2) {
    out[0] = *(const uint32_t*)(blk + word_offset(lane, o >> 1));
  } else if constexpr (B == 4) {
    out[0] = *(const uint32_t*)(blk + word_offset(lane, o));
  } else if constexpr (B == 8) {
    const u2_t v = *(const u2_t*)(blk + word_offset(lane, 2 * o));
    out[0] = v[0];
    out[1] = v[1];
  } else {
    const u4_t v = *(const u4_t*)(blk + (size_t)o * 1024 + lane * 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) out[k] = v[k];
  }
}

// element i of octet o from its words: the code, or for B = 16 the fp16 value
template <int B>
__device__ __forceinline__ float octet_value(const uint32_t* words, int o, int i) {
  constexpr int per = 32 / B;
  const int pos = (B == 2 ? 8 * (o & 1) : 0) + i;
  const uint32_t x = words[pos / per];
  const int pp = pos % per;
  const int sh = (pp & 1) * 16 + (pp >> 1) * B;
  if constexpr (B == 16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> sh));
  } else {
    return (float)((x >> sh) & ((1u << B) - 1u));
  }
}

template <int KB, int VB, bool KTOK>
__device__ __forceinline__ void load_share(const uint8_t* rec, int w, int lane, Share<KB, VB, KTOK>& sh) {
  const RecordParts parts = record_parts(KB, VB);
  const int a = lane >> 4;
  load_octet<KB>(rec, w, lane, sh.kw);
  load_octet<VB>(rec + parts.vcode, w, lane, sh.vw);
  if constexpr (KB < 16) {
    const float* km = (const float*)(rec + parts.kmeta);
    if constexpr (KTOK) {
      // token 16(w/4) + lane%16, channel group w%4
      const int m = 32 * (w & 3) + kappa(16 * (w >> 2) + (lane & 15));
      sh.ks[0] = km[m];
      sh.kz[0] = km[128 + m];
    } else {
      // channels 32(w%4) + 8a + i: meta 32a + 8(w%4) + i
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const f4_t s4 = *(const f4_t*)(km + 32 * a + 8 * (w & 3) + 4 * v);
        const f4_t z4 = *(const f4_t*)(km + 128 + 32 * a + 8 * (w & 3) + 4 * v);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sh.ks[4 * v + i] = s4[i];
          sh.kz[4 * v + i] = z4[i];
        }
      }
    }
  }
  if constexpr (VB < 16) {
    // channel group w/2, the tokens of slots 8a + i
    const float* vm = (const float*)(rec + parts.vmeta);
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const f4_t s4 = *(const f4_t*)(vm + 32 * (w >> 1) + 8 * a + 4 * v);
      const f4_t z4 = *(const f4_t*)(vm + 128 + 32 * (w >> 1) + 8 * a + 4 * v);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sh.vs[4 * v + i] = s4[i];
        sh.vz[4 * v + i] = z4[i];
      }
    }
  }
}

// The thread's octets into LDS. MASK (the tail): tokens at or past ntok
// become 0 (their slots may hold stale or never-written bytes).
template <int KB, int VB, bool KTOK, bool MASK>
__device__ __forceinline__ void dequant_share(const Share<KB, VB, KTOK>& sh, GroupBuf& b, int w, int lane, int ntok) {
  const int a = lane >> 4;
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float c = octet_value<KB>(sh.kw, w, i);
    if constexpr (KB == 16) {
      x[i] = c;
    } else if constexpr (KTOK) {
      x[i] = fmaf(c, sh.ks[0], sh.kz[0]);
    } else {
      x[i] = fmaf(c, sh.ks[i], sh.kz[i]);
    }
    if constexpr (MASK) x[i] = 16 * (w >> 2) + (lane & 15) < ntok ? x[i] : 0.f;
  }
  split8(x, b.khi[w][lane], b.klo[w][lane]);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float c = octet_value<VB>(sh.vw, w, i);
    if constexpr (VB == 16) {
      x[i] = c;
    } else {
      x[i] = fmaf(c, sh.vs[i], sh.vz[i]);
    }
    if constexpr (MASK) x[i] = 16 * (i >> 2) + 4 * a + (i & 3) < ntok ? x[i] : 0.f;
  }
  b.vhi[w][lane] = to_h8(x);
}

struct Acc {
  f4_t o[kNT][8];  // O^T tiles: channels 16u + 4(l/16) + i, row l%16 of column tile n
  float m[kNT], lpart[kNT];
};

// One group from LDS for the wave's kNT column tiles. MASK: tokens at or
// past ntok score -inf.
template <bool MASK>
__device__ __forceinline__ void group_step(const GroupBuf& b, const h8_t (*qv)[4], float scale_log2, int lane,
                                           int ntok, Acc& acc) {
  const int a = lane >> 4;
  // raw products q.k of every column tile: 2 kNT independent accumulation
  // chains, interleaved so that consecutive matrix ops do not depend on
  // each other
  f4_t c[kNT][2];
#pragma unroll
  for (int n = 0; n < kNT; ++n) c[n][0] = c[n][1] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const h8_t kh0 = b.khi[s][lane], kh1 = b.khi[4 + s][lane];
    const h8_t kl0 = b.klo[s][lane], kl1 = b.klo[4 + s][lane];
#pragma unroll
    for (int n = 0; n < kNT; ++n) {
      c[n][0] = mfma(kh0, qv[n][s], c[n][0]);
      c[n][1] = mfma(kh1, qv[n][s], c[n][1]);
    }
#pragma unroll
    for (int n = 0; n < kNT; ++n) {
      c[n][0] = mfma(kl0, qv[n][s], c[n][0]);
      c[n][1] = mfma(kl1, qv[n][s], c[n][1]);
    }
  }
  // token 16t + 4a + i of column tile n has raw product c[n][t][i]; its
  // score is raw * scale_log2 (log2 units)
  float hi[kNT];  // this lane's largest score per column tile
  bool raise = false;
#pragma unroll
  for (int n = 0; n < kNT; ++n) {
    hi[n] = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = !MASK || 16 * t + 4 * a + i < ntok;
        hi[n] = ok ? fmaxf(hi[n], c[n][t][i] * scale_log2) : hi[n];
      }
    raise = raise || hi[n] > acc.m[n] + kSlack;
  }
  if (__any(raise)) {
    // raise each column's reference to its max (the same in the column's
    // four lane groups) and rescale what was summed against the old one
#pragma unroll
    for (int n = 0; n < kNT; ++n) {
      const float mnew = fmaxf(acc.m[n], max_lane_groups(hi[n]));
      const float alpha = __builtin_amdgcn_exp2f(acc.m[n] - mnew);  // 0 for the first group
#pragma unroll
      for (int u = 0; u < 8; ++u) acc.o[n][u] *= alpha;
      acc.lpart[n] *= alpha;
      acc.m[n] = mnew;
    }
  }
  h8_t ph[kNT];
#pragma unroll
  for (int n = 0; n < kNT; ++n) {
    float p[8];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = __builtin_amdgcn_exp2f(fmaf(c[n][t][i], scale_log2, -acc.m[n]));
        if constexpr (MASK) x = 16 * t + 4 * a + i < ntok ? x : 0.f;
        p[4 * t + i] = x;
        acc.lpart[n] += x;
      }
    ph[n] = to_h8(p);
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const h8_t vh = b.vhi[u][lane];
#pragma unroll
    for (int n = 0; n < kNT; ++n) acc.o[n][u] = mfma(vh, ph[n], acc.o[n][u]);
  }
}

// The wave's rows: o = O / l, lse = (m + log2 l) ln 2, into the output (one
// partial a row) or into partial `split` of a.part_stride (or a.splits) a row.
__device__ __forceinline__ void store_rows(const DecodeArgs& a, const Acc& acc, int row0, int nrows, int r, int h,
                                           int split, int lane) {
  const LayerGeom& g = a.geo;
  const int G = g.g;
  const int a4 = lane >> 4;
#pragma unroll
  for (int n = 0; n < kNT; ++n) {
    const float l = sum_lane_groups(acc.lpart[n]);
    const int row = row0 + 16 * n + (lane & 15);
    if (row >= nrows) continue;
    const size_t orow = ((size_t)r * a.chunk + row / G) * g.hq + h * G + row % G;
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    const float lse = l > 0.f ? (acc.m[n] + __log2f(l)) * 0.69314718055994531f : -INFINITY;
    const int ps = a.part_stride ? a.part_stride : a.splits;
    float* dst = ps == 1 ? (float*)a.out + orow * D : a.part_o + (orow * ps + split) * D;
#pragma unroll
    for (int u = 0; u < 8; ++u) *(f4_t*)(dst + 16 * u + 4 * a4) = acc.o[n][u] * inv;
    if (a4 == 0) {
      if (ps > 1)
        a.part_lse[orow * ps + split] = lse;
      else if (a.lse_out)
        a.lse_out[orow] = lse;
    }
  }
}

// One workgroup per (split, block of kRows rows, KV head, request), split
// fastest. Rows of a (request, KV head): row i is chunk token i / G, query
// head h G + i % G; q and the outputs are [request][token][Hq] rows.
template <int KB, int VB, bool KTOK>
__global__ __launch_bounds__(kWaves * 64, 1) void prefix_kernel(DecodeArgs a) {
  __shared__ GroupBuf buf[2];
  const LayerGeom& g = a.geo;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = blockIdx.x % a.splits, blk = blockIdx.x / a.splits;
  const int h = blockIdx.y, r = blockIdx.z;
  const int L = min(max(a.seq_lens[r], 0), g.max_tokens);
  const int nq = L / GS, T = L - nq * GS;
  const int nvg = nq + (T > 0);
  const int g0 = split * a.groups_per_split;
  const int g1 = min(g0 + a.groups_per_split, nvg);
  const int nk = max(min(g1, nq) - g0, 0);
  const bool tail = T > 0 && nq >= g0 && nq < g1;
  const uint8_t* stream = g.base + (size_t)(r * g.hkv + h) * g.stream_bytes;
  const int G = g.g, nrows = a.chunk * G;
  const int row0 = blk * kRows + wave * (16 * kNT);

  // the wave's q rows as score operands: lane l, tile n, step s holds row
  // row0 + 16n + l%16, channels 32s + 8(l/16) .. + 7 (rows past the chunk
  // read the last row and are not written)
  h8_t qv[kNT][4];
#pragma unroll
  for (int n = 0; n < kNT; ++n) {
    const int row = min(row0 + 16 * n + (lane & 15), nrows - 1);
    const uint16_t* qp = a.q + (((size_t)r * a.chunk + row / G) * g.hq + h * G + row % G) * D + 8 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < 4; ++s) qv[n][s] = __builtin_bit_cast(h8_t, *(const u4_t*)(qp + 32 * s));
  }
  Acc acc;
#pragma unroll
  for (int n = 0; n < kNT; ++n) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc.o[n][u] = f4_t{0.f, 0.f, 0.f, 0.f};
    acc.m[n] = -INFINITY;
    acc.lpart[n] = 0.f;
  }

  // packed groups g0 .. g0 + nk - 1; the loads of the next one are issued
  // before the current one is multiplied (for the last, a harmless reload of
  // itself: a load under a condition would make the compiler wait for every
  // load in flight at the join)
  const size_t rb = g.record_bytes;
  if (nk > 0) {
    Share<KB, VB, KTOK> sh;
    load_share<KB, VB, KTOK>(stream + (size_t)g0 * rb, wave, lane, sh);
    dequant_share<KB, VB, KTOK, false>(sh, buf[0], wave, lane, GS);
  }
  __syncthreads();
  for (int k = 0; k < nk; ++k) {
    Share<KB, VB, KTOK> sh;
    load_share<KB, VB, KTOK>(stream + (size_t)(g0 + min(k + 1, nk - 1)) * rb, wave, lane, sh);
    group_step<false>(buf[k & 1], qv, a.scale_log2, lane, GS, acc);
    dequant_share<KB, VB, KTOK, false>(sh, buf[(k + 1) & 1], wave, lane, GS);
    __syncthreads();
  }
  if (tail) {  // workgroup-uniform
    Share<16, 16, false> sh;
    load_share<16, 16, false>(stream + g.tail_offset, wave, lane, sh);
    dequant_share<16, 16, false, true>(sh, buf[nk & 1], wave, lane, T);
    __syncthreads();
    group_step<true>(buf[nk & 1], qv, a.scale_log2, lane, T, acc);
  }

  store_rows(a, acc, row0, nrows, r, h, split, lane);
}

// Paged pool: a request's INT2 tokens (K2V2 records in page pairs) and then
// its INT4 tokens (page pairs of per-token 4-bit keys and values, the last
// pair partly filled), as one sequence of 32-token groups that the splits
// share out (TriAxialKV page, "Facts": page pools and page tables).

// One INT4 page pair (tokens 0..31 of it: page a holds 0..15, page b
// 16..31) into LDS: the thread's key and value octets dequantized straight
// from the pages (fmaf(code, scale, zero), per-token meta); tokens at or past
// ntok become 0.
__device__ __forceinline__ void dequant_int4_pair(const uint8_t* pa, const uint8_t* pb, int ntok, GroupBuf& b, int w,
                                                  int lane) {
  const int a = lane >> 4;
  float x[8];
  {  // key octet w: token 16(w/4) + lane%16, channels 32(w%4) + 8a + i
    const int t = 16 * (w >> 2) + (lane & 15);
    const uint8_t* pg = t < PAGE_TOKENS ? pa : pb;
    const int p = t & 15;
    const float* km = (const float*)(pg + INT4_KMETA);
    const int mi = 16 * (w & 3) + p;
    const float sc = km[mi], zr = km[64 + mi];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int sh;
      const uint32_t off = page_k_offset(p, 32 * (w & 3) + 8 * a + i, &sh);
      const float code = (float)((*(const uint32_t*)(pg + off) >> sh) & 15u);
      x[i] = t < ntok ? fmaf(code, sc, zr) : 0.f;
    }
  }
  split8(x, b.khi[w][lane], b.klo[w][lane]);
  {  // value octet w: channel 16w + lane%16, tokens 16(i/4) + 4a + i%4
    const int c = 16 * w + (lane & 15);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = 16 * (i >> 2) + 4 * a + (i & 3);
      const uint8_t* pg = j < PAGE_TOKENS ? pa : pb;
      const int p = j & 15;
      int sh;
      const uint32_t off = page_v_offset(p, c, &sh);
      const float code = (float)((*(const uint32_t*)(pg + off) >> sh) & 15u);
      const float* vm = (const float*)(pg + INT4_VMETA);
      const int mi = 16 * (c >> 5) + p;
      x[i] = j < ntok ? fmaf(code, vm[mi], vm[64 + mi]) : 0.f;
    }
  }
  b.vhi[w][lane] = to_h8(x);
}

__global__ __launch_bounds__(kWaves * 64, 1) void prefix_paged_kernel(DecodeArgs a) {
  __shared__ GroupBuf buf;
  const LayerGeom& g = a.geo;
  const PagedGeom& pg = a.pg;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = blockIdx.x % a.splits, blk = blockIdx.x / a.splits;
  const int h = blockIdx.y, r = blockIdx.z;
  const int n2 = max(pg.int2_len[r], 0), n4 = max(pg.int4_len[r], 0);
  const int n2g = n2 / GS, nvg = n2g + (n4 + GS - 1) / GS;
  const int g0 = split * a.groups_per_split;
  const int g1 = min(g0 + a.groups_per_split, nvg);
  const int32_t* table = pg.table + (size_t)r * pg.max_pages;
  const int G = g.g, nrows = a.chunk * G;
  const int row0 = blk * kRows + wave * (16 * kNT);
  h8_t qv[kNT][4];
#pragma unroll
  for (int n = 0; n < kNT; ++n) {
    const int row = min(row0 + 16 * n + (lane & 15), nrows - 1);
    const uint16_t* qp = a.q + (((size_t)r * a.chunk + row / G) * g.hq + h * G + row % G) * D + 8 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < 4; ++s) qv[n][s] = __builtin_bit_cast(h8_t, *(const u4_t*)(qp + 32 * s));
  }
  Acc acc;
#pragma unroll
  for (int n = 0; n < kNT; ++n) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc.o[n][u] = f4_t{0.f, 0.f, 0.f, 0.f};
    acc.m[n] = -INFINITY;
    acc.lpart[n] = 0.f;
  }
  for (int gi = g0; gi < g1; ++gi) {  // workgroup-uniform branches
    int ntok = GS;
    if (gi < n2g) {
      const uint8_t* rec = g.base + (size_t)table[2 * gi] * pg.int2_page_bytes + (size_t)h * INT2_RECORD;
      Share<2, 2, false> sh;
      load_share<2, 2, false>(rec, wave, lane, sh);
      dequant_share<2, 2, false, false>(sh, buf, wave, lane, GS);
    } else {
      const int i = gi - n2g;
      const int e = n2 / PAGE_TOKENS + 2 * i;
      ntok = min(GS, n4 - GS * i);
      const uint8_t* base4 = g.base + pg.int4_offset + (size_t)h * INT4_HEAD;
      const uint8_t* pa = base4 + (size_t)(table[e] - pg.int2_pages) * pg.int4_page_bytes;
      const uint8_t* pb = ntok > PAGE_TOKENS ? base4 + (size_t)(table[e + 1] - pg.int2_pages) * pg.int4_page_bytes : pa;
      dequant_int4_pair(pa, pb, ntok, buf, wave, lane);
    }
    __syncthreads();
    if (ntok == GS)
      group_step<false>(buf, qv, a.scale_log2, lane, GS, acc);
    else
      group_step<true>(buf, qv, a.scale_log2, lane, ntok, acc);
    __syncthreads();
  }
  store_rows(a, acc, row0, nrows, r, h, split, lane);
}

// ------------------------------------------------------ chunked prefill
// The chunk's own part of chunked-prefill attention: each query row (chunk
// token i, query head) over the chunk's fp16 keys and values 0 .. i, causally
// (the chunk is not in the cache yet). Its (o, lse) is one more partial of the
// row, which the merge pass joins with the prefix splits by log-sum-exp
// (TriAxialKV page, "Facts": partial attentions merged by online
// log-sum-exp). Keys and values are fp16 and q is fp16, so the score products
// are exact with one fp16 operand each (no low planes); p is rounded to fp16
// as in the prefix pass.

// Block kb of the chunk's keys and values (tokens 32 kb .. 32 kb + 31; those
// at or past `chunk` become 0) into the record lane order of GroupBuf.
__device__ __forceinline__ void load_chunk_block(const uint16_t* kc, const uint16_t* vc, int chunk, int kb, int w,
                                                 int lane, GroupBuf& b) {
  const int a = lane >> 4;
  {  // key octet w: token 16(w/4) + lane%16, channels 32(w%4) + 8a .. + 7
    const int t = 32 * kb + 16 * (w >> 2) + (lane & 15);
    u4_t x = {0, 0, 0, 0};
    if (t < chunk) x = *(const u4_t*)(kc + (size_t)t * D + 32 * (w & 3) + 8 * a);
    b.khi[w][lane] = __builtin_bit_cast(h8_t, x);
  }
  {  // value octet w: channel 16w + lane%16, tokens 16(i/4) + 4a + i%4
    h8_t x;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = 32 * kb + 16 * (i >> 2) + 4 * a + (i & 3);
      const uint16_t bits = t < chunk ? vc[(size_t)t * D + 16 * w + (lane & 15)] : (uint16_t)0;
      x[i] = __builtin_bit_cast(_Float16, bits);
    }
    b.vhi[w][lane] = x;
  }
}

// One key block for the wave's column tiles; lim[n]: the last key (index in
// the block) that column n's lane may see (its token minus 32 kb; < 0: none).
__device__ __forceinline__ void chunk_step(const GroupBuf& b, const h8_t (*qv)[4], float scale_log2, int lane,
                                           const int* lim, Acc& acc) {
  const int a = lane >> 4;
  f4_t c[kNT][2];
#pragma unroll
  for (int n = 0; n < kNT; ++n) c[n][0] = c[n][1] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const h8_t k0 = b.khi[s][lane], k1 = b.khi[4 + s][lane];
#pragma unroll
    for (int n = 0; n < kNT; ++n) {
      c[n][0] = mfma(k0, qv[n][s], c[n][0]);
      c[n][1] = mfma(k1, qv[n][s], c[n][1]);
    }
  }
  float hi[kNT];
  bool raise = false;
#pragma unroll
  for (int n = 0; n < kNT; ++n) {
    hi[n] = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        hi[n] = 16 * t + 4 * a + i <= lim[n] ? fmaxf(hi[n], c[n][t][i] * scale_log2) : hi[n];
    raise = raise || hi[n] > acc.m[n] + kSlack;
  }
  if (__any(raise)) {
#pragma unroll
    for (int n = 0; n < kNT; ++n) {
      const float mnew = fmaxf(acc.m[n], max_lane_groups(hi[n]));
      const float alpha = mnew == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(acc.m[n] - mnew);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc.o[n][u] *= alpha;
      acc.lpart[n] *= alpha;
      acc.m[n] = mnew;
    }
  }
  h8_t ph[kNT];
#pragma unroll
  for (int n = 0; n < kNT; ++n) {
    float p[8];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = 16 * t + 4 * a + i <= lim[n] && acc.m[n] != -INFINITY;
        const float x = ok ? __builtin_amdgcn_exp2f(fmaf(c[n][t][i], scale_log2, -acc.m[n])) : 0.f;
        p[4 * t + i] = x;
        acc.lpart[n] += x;
      }
    ph[n] = to_h8(p);
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const h8_t vh = b.vhi[u][lane];
#pragma unroll
    for (int n = 0; n < kNT; ++n) acc.o[n][u] = mfma(vh, ph[n], acc.o[n][u]);
  }
}

// One workgroup per (block of kRows rows, KV head, request); writes partial
// index a.splits of each row (a.part_stride partials a row).
__global__ __launch_bounds__(kWaves * 64, 1) void chunk_causal_kernel(DecodeArgs a) {
  __shared__ GroupBuf buf;
  const LayerGeom& g = a.geo;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int blk = blockIdx.x, h = blockIdx.y, r = blockIdx.z;
  const int G = g.g, nrows = a.chunk * G;
  const int row0 = blk * kRows + wave * (16 * kNT);
  const size_t sigma = (size_t)r * g.hkv + h;
  const uint16_t* kc = a.k_chunk + sigma * a.chunk * D;
  const uint16_t* vc = a.v_chunk + sigma * a.chunk * D;
  h8_t qv[kNT][4];
  int tok[kNT];
#pragma unroll
  for (int n = 0; n < kNT; ++n) {
    const int row = min(row0 + 16 * n + (lane & 15), nrows - 1);
    tok[n] = row / G;
    const uint16_t* qp = a.q + (((size_t)r * a.chunk + row / G) * g.hq + h * G + row % G) * D + 8 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < 4; ++s) qv[n][s] = __builtin_bit_cast(h8_t, *(const u4_t*)(qp + 32 * s));
  }
  Acc acc;
#pragma unroll
  for (int n = 0; n < kNT; ++n) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc.o[n][u] = f4_t{0.f, 0.f, 0.f, 0.f};
    acc.m[n] = -INFINITY;
    acc.lpart[n] = 0.f;
  }
  // key blocks up to the last token any row of the workgroup has
  const int last = min((min(blk * kRows + kRows, nrows) - 1) / G, a.chunk - 1);
  for (int kb = 0; kb <= last / GS; ++kb) {
    load_chunk_block(kc, vc, a.chunk, kb, wave, lane, buf);
    __syncthreads();
    int lim[kNT];
#pragma unroll
    for (int n = 0; n < kNT; ++n) lim[n] = tok[n] - GS * kb;
    chunk_step(buf, qv, a.scale_log2, lane, lim, acc);
    __syncthreads();
  }
  const int a4 = lane >> 4;
#pragma unroll
  for (int n = 0; n < kNT; ++n) {
    const float l = sum_lane_groups(acc.lpart[n]);
    const int row = row0 + 16 * n + (lane & 15);
    if (row >= nrows) continue;
    const size_t orow = ((size_t)r * a.chunk + row / G) * g.hq + h * G + row % G;
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    const float lse = l > 0.f ? (acc.m[n] + __log2f(l)) * 0.69314718055994531f : -INFINITY;
    float* dst = a.part_o + (orow * a.part_stride + a.splits) * D;
#pragma unroll
    for (int u = 0; u < 8; ++u) *(f4_t*)(dst + 16 * u + 4 * a4) = acc.o[n][u] * inv;
    if (a4 == 0) a.part_lse[orow * a.part_stride + a.splits] = lse;
  }
}

template <int KB, int VB>
hipError_t launch_kv(const DecodeArgs& a, int batch, hipStream_t s, const EventPair* ev) {
  const int blocks = (a.chunk * a.geo.g + kRows - 1) / kRows;
  const dim3 grid(a.splits * blocks, a.geo.hkv, batch), block(kWaves * 64);
  if constexpr (KB < 16) {
    if (a.geo.k_token) return launch_timed(prefix_kernel<KB, VB, true>, grid, block, s, ev, a);
  }
  return launch_timed(prefix_kernel<KB, VB, false>, grid, block, s, ev, a);
}

template <int KB>
hipError_t launch_k(const DecodeArgs& a, int batch, hipStream_t s, const EventPair* ev) {
  switch (a.geo.vb) {
    case 2: return launch_kv<KB, 2>(a, batch, s, ev);
    case 4: return launch_kv<KB, 4>(a, batch, s, ev);
    case 8: return launch_kv<KB, 8>(a, batch, s, ev);
    default: return launch_kv<KB, 16>(a, batch, s, ev);
  }
}

}  // namespace

int prefix_rows_per_block() { return kRows; }

hipError_t launch_chunk_causal(const DecodeArgs& a, int batch, hipStream_t s, const EventPair* ev) {
  const int blocks = (a.chunk * a.geo.g + kRows - 1) / kRows;
  if (blocks == 0 || batch == 0) return hipSuccess;
  return launch_timed(chunk_causal_kernel, dim3(blocks, a.geo.hkv, batch), dim3(kWaves * 64), s, ev, a);
}

hipError_t launch_prefix(const DecodeArgs& a, int batch, hipStream_t s, const EventPair* ev) {
  if (a.pg.table) {
    const int blocks = (a.chunk * a.geo.g + kRows - 1) / kRows;
    return launch_timed(prefix_paged_kernel, dim3(a.splits * blocks, a.geo.hkv, batch), dim3(kWaves * 64), s, ev, a);
  }
  switch (a.geo.kb) {
    case 2: return launch_k<2>(a, batch, s, ev);
    case 4: return launch_k<4>(a, batch, s, ev);
    case 8: return launch_k<8>(a, batch, s, ev);
    default: return launch_k<16>(a, batch, s, ev);
  }
}

}  // namespace kvq
