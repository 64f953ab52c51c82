// kvq_quantize.h -- the group quantizer and record packer, shared by the
// append kernels and the fused append-and-decode split pass.
//
// Quantizer (TriAxialKV page, "Facts", quantizer bullet: asymmetric groupwise,
// group size 32): scale = (max - min) / (2^b - 1) in fp32, zero = min,
// code = clamp(rint((x - zero) / scale), 0, 2^b - 1) with IEEE subtraction
// and division (explicitly rounded operations, so no contraction can change
// them) and round-half-even; a constant group gets scale 0 and codes 0.
#pragma once

#include "kvq_internal.h"

namespace kvq {
namespace {

__device__ inline float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

__device__ inline uint16_t tail_get(const uint8_t* rec, bool is_v, int j, int c) {
  int lane, e;
  if (is_v) v_site(j, c, &lane, &e); else k_site(j, c, &lane, &e);
  const uint8_t* blk = rec + (is_v ? 8192 : 0);
  return *(const uint16_t*)(blk + word_offset(lane, e >> 1) + (e & 1) * 2);
}

__device__ inline void tail_put(uint8_t* rec, bool is_v, int j, int c, uint16_t x) {
  int lane, e;
  if (is_v) v_site(j, c, &lane, &e); else k_site(j, c, &lane, &e);
  uint8_t* blk = rec + (is_v ? 8192 : 0);
  *(uint16_t*)(blk + word_offset(lane, e >> 1) + (e & 1) * 2) = x;
}

// LDS row stride (bytes) of the code staging: 33 words, so that a wave's
// per-token groups (rows j, column blocks 32n) and the packer's reads of 16
// rows at once spread over the LDS banks.
constexpr int CS = D + 4;

// One group of 32 values x[i * stride]; writes codes[i * cstride], returns
// scale/zero. The elements are visited from position rot on (mod 32): a lane
// that starts elsewhere than its neighbours reads another LDS bank (the
// result does not depend on the order).
__device__ __forceinline__ void quantize32(const uint16_t* x, int stride, int bits, uint8_t* codes,
                                  int cstride, float* scale, float* zero, int rot = 0) {
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll 8
  for (int i = 0; i < GS; ++i) {
    const float v = h2f(x[((i + rot) & (GS - 1)) * stride]);
    mn = fminf(mn, v);
    mx = fmaxf(mx, v);
  }
  const float levels = (float)((1 << bits) - 1);
  const float s = __fdiv_rn(__fsub_rn(mx, mn), levels);
  *scale = s;
  *zero = mn;
  if (s == 0.0f) {
#pragma unroll 8
    for (int i = 0; i < GS; ++i) codes[((i + rot) & (GS - 1)) * cstride] = 0;
    return;
  }
  // The code is rint of the correctly rounded quotient Q = RN(t / scale),
  // t = x - zero. q = RN(t RN(1 / scale)) differs from t / scale by at most
  // 2^-23 relative (two roundings) and Q by 2^-24 more: below 1.5 * 2^-23 *
  // 255 < 2^-14 for every quotient up to 255. So rint(q) = rint(Q) unless q
  // lies within 2^-14 of a half-integer; those elements are marked and
  // recoded with the IEEE division after the loop (a fraction of a percent
  // of fp16 inputs, exact ties included).
  const float y = __fdiv_rn(1.0f, s);
  uint32_t redo = 0;
#pragma unroll 8
  for (int i = 0; i < GS; ++i) {
    const int k = (i + rot) & (GS - 1);
    // (t = x - zero >= 0, so q >= 0 and only the top needs clamping)
    const float q = __fmul_rn(__fsub_rn(h2f(x[k * stride]), mn), y);
    redo |= fabsf(__fsub_rn(__builtin_amdgcn_fractf(q), 0.5f)) < 0x1p-14f ? 1u << k : 0u;
    codes[k * cstride] = (uint8_t)fminf(rintf(q), levels);
  }
  while (redo != 0) {
    const int k = __builtin_ctz(redo);
    redo &= redo - 1;
    const float q = __fdiv_rn(__fsub_rn(h2f(x[k * stride]), mn), s);
    codes[k * cstride] = (uint8_t)fminf(fmaxf(rintf(q), 0.0f), levels);
  }
}

// Write the 512*BITS bytes of a code block from src[32][ROW] (token,
// channel): the codes (BITS <= 8, uint8 rows of the staging) or the fp16
// values themselves (BITS = 16).
template <int BITS, bool IS_V, class T, int ROW>
__device__ inline void pack_block(uint8_t* blk, const T (*src)[ROW], int tid, int nthreads) {
  constexpr int per_word = 32 / BITS;
  constexpr int nwords = 128 * BITS;
  for (int W = tid; W < nwords; W += nthreads) {
    const int lane = (W & 255) >> 2;
    const int w = (W >> 8) * 4 + (W & 3);
    uint32_t word = 0;
#pragma unroll
    for (int p = 0; p < per_word; ++p) {
      const int e = w * per_word + p;
      int j, c;
      if (IS_V) v_inverse(lane, e, &j, &c); else k_inverse(lane, e, &j, &c);
      word |= (uint32_t)src[j][c] << ((p & 1) * 16 + (p >> 1) * BITS);
    }
    *(uint32_t*)(blk + (size_t)W * 4) = word;
  }
}

template <bool IS_V>
__device__ inline void pack_block_bits(uint8_t* blk, int bits, const uint16_t (*xs)[D], const uint8_t (*cs)[CS],
                                       int tid, int nthreads) {
  switch (bits) {
    case 2: pack_block<2, IS_V>(blk, cs, tid, nthreads); break;
    case 4: pack_block<4, IS_V>(blk, cs, tid, nthreads); break;
    case 8: pack_block<8, IS_V>(blk, cs, tid, nthreads); break;
    default: pack_block<16, IS_V>(blk, xs, tid, nthreads); break;
  }
}

// Quantize one full 32-token group (xs: fp16 K and V [32][128], in LDS) and
// write its record; cs is LDS scratch for the codes. 256 threads. A
// per-token group (row j) starts at position 2j: the 16 rows a wave covers
// then read 16 different banks.
__device__ __forceinline__ void quantize_record(const uint16_t (*xs)[GS][D], uint8_t (*cs)[GS][CS], uint8_t* rec, int kb,
                                       int vb, int k_token, int tid) {
  const RecordParts parts = record_parts(kb, vb);
  float* kmeta = (float*)(rec + parts.kmeta);
  float* vmeta = (float*)(rec + parts.vmeta);
  if (tid < 128) {
    if (kb == 16) {
      // the fp16 values are packed as they are, straight from xs
    } else if (!k_token) {
      const int c = tid;
      float s, z;
      quantize32(&xs[0][0][c], D, kb, &cs[0][0][c], CS, &s, &z);
      kmeta[meta_channel(c)] = s;
      kmeta[128 + meta_channel(c)] = z;
    } else {
      const int j = tid >> 2, n = tid & 3;
      float s, z;
      quantize32(&xs[0][j][32 * n], 1, kb, &cs[0][j][32 * n], 1, &s, &z, 2 * j);
      kmeta[meta_token(j, n)] = s;
      kmeta[128 + meta_token(j, n)] = z;
    }
  } else {
    const int t2 = tid - 128;
    if (vb == 16) {
      // packed from xs
    } else {
      const int j = t2 >> 2, n = t2 & 3;
      float s, z;
      quantize32(&xs[1][j][32 * n], 1, vb, &cs[1][j][32 * n], 1, &s, &z, 2 * j);
      vmeta[meta_token(j, n)] = s;
      vmeta[128 + meta_token(j, n)] = z;
    }
  }
  __syncthreads();
  pack_block_bits<false>(rec, kb, xs[0], cs[0], tid, blockDim.x);
  pack_block_bits<true>(rec + parts.vcode, vb, xs[1], cs[1], tid, blockDim.x);
}

// Write slots p_lo .. p_hi - 1 of one KV head's share of an INT4 page (keys
// and values per-token at 4 bits, TriAxialKV page, "Facts": INT4 per-token
// path): their fp16 rows are in xs[tensor][slot] (LDS, visible to every
// thread); cs is LDS scratch for the codes. 256 threads, all of them must
// call. Value words hold four slots: the slots outside the range keep their
// bits.
__device__ inline void page_append_int4(uint8_t* page, const uint16_t (*xs)[GS][D], uint8_t (*cs)[GS][CS], int p_lo,
                                        int p_hi, int tid) {
  if (tid < 128) {  // per-token quantization: (tensor, slot, channel group)
    const int tensor = tid >> 6, p = (tid >> 2) & 15, n = tid & 3;
    if (p >= p_lo && p < p_hi) {
      float s, z;
      quantize32(&xs[tensor][p][32 * n], 1, 4, &cs[tensor][p][32 * n], 1, &s, &z, 2 * p);
      float* meta = (float*)(page + (tensor ? INT4_VMETA : INT4_KMETA));
      meta[16 * n + p] = s;
      meta[64 + 16 * n + p] = z;
    }
  }
  __syncthreads();
  {  // key words: the 8 codes of a word belong to one slot
    const int p = tid >> 4, a4 = (tid >> 2) & 3, w = tid & 3;
    if (p >= p_lo && p < p_hi) {
      uint32_t word = 0;
      for (int pos = 0; pos < 8; ++pos) {
        int sh;
        const int c = 32 * w + 8 * a4 + pos;
        (void)page_k_offset(p, c, &sh);
        word |= (uint32_t)cs[0][p][c] << sh;
      }
      int sh0;
      *(uint32_t*)(page + page_k_offset(p, 32 * w + 8 * a4, &sh0)) = word;
    }
  }
  {  // value words: four slots share a word; keep the slots not written now
    const int quad = tid >> 6, c16 = (tid >> 2) & 15, wv = tid & 3;
    if (4 * quad + 3 >= p_lo && 4 * quad < p_hi) {
      int sh;
      const uint32_t off = page_v_offset(4 * quad, 32 * wv + c16, &sh);
      uint32_t word = (4 * quad < p_lo || 4 * quad + 3 >= p_hi) ? *(const uint32_t*)(page + off) : 0u;
      for (int i = 0; i < 4; ++i) {
        const int p = 4 * quad + i;
        if (p < p_lo || p >= p_hi) continue;
        for (int hh = 0; hh < 2; ++hh) {
          const int c = 16 * (2 * wv + hh) + c16;
          (void)page_v_offset(p, c, &sh);
          word = (word & ~(0xFu << sh)) | ((uint32_t)cs[1][p][c] << sh);
        }
      }
      *(uint32_t*)(page + off) = word;
    }
  }
}

}  // namespace
}  // namespace kvq
