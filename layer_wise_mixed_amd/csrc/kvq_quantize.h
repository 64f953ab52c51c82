// kvq_quantize.h -- the group quantizer and record packer, shared by the
// append kernels and the fused append-and-decode split pass.
//
// Quantizer (TriAxialKV page, "Facts", quantizer bullet: asymmetric groupwise,
// group size 32): scale = (max - min) / (2^b - 1) in fp32, zero = min,
// code = clamp(rint((x - zero) / scale), 0, 2^b - 1) with IEEE subtraction
// and division (explicitly rounded operations, so no contraction can change
// them) and round-half-even; a constant group gets scale 0 and codes 0. The
// codes come from a reciprocal quotient, with the IEEE division only for the
// values whose quotient lies near a rounding boundary (code_fast): the same
// codes, bit for bit.
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

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

// Minimum and maximum of 32 fp16 values held two a word, on packed fp16
// (exact: fp16 min and max lose nothing, and the order does not matter).
__device__ __forceinline__ void minmax32(const uint32_t (&w)[16], float* mn, float* mx) {
  const uint32_t w0 = w[0];  // (each word copied to a scalar before the cast)
  h2_t lo = __builtin_bit_cast(h2_t, w0), hi = lo;
#pragma unroll
  for (int d = 1; d < 16; ++d) {
    const uint32_t u = w[d];
    const h2_t v = __builtin_bit_cast(h2_t, u);
    lo = __builtin_elementwise_minimum(lo, v);
    hi = __builtin_elementwise_maximum(hi, v);
  }
  *mn = fminf((float)lo[0], (float)lo[1]);
  *mx = fmaxf((float)hi[0], (float)hi[1]);
}

// The code is rint of the correctly rounded quotient Q = RN(t / scale),
// t = RN(x - zero). q = RN(t RN(1 / scale)) differs from t / scale by at most
// 2^-23 relative (two roundings) and Q by 2^-24 more: below 1.5 * 2^-23 *
// 255 < 2^-14 for every quotient up to 255, so rint(q) = rint(Q) unless q
// lies within 2^-14 of a half-integer. code_fast returns rint(q) and the
// distance d of t RN(1 / scale) from it (within 2^-17 of |q - rint(q)|); a
// value with d > 1/2 - 2^-14 is recoded with the IEEE division (a fraction of
// a percent of fp16 inputs, most of them exact ties). No clamp is needed on
// the fast path: t <= RN(max - min) and y = RN(1 / scale) put q below
// levels (1 + 2^-22) < levels + 1/2, and t >= 0.
constexpr float kNear = 0.5f - 0x1p-14f;

// Bit k of the result is set when value k is near a rounding boundary in some
// lane of the wave: one compare into a lane mask, the rest scalar.
__device__ __forceinline__ uint32_t near_bit(float d, int k) {
  return __builtin_amdgcn_ballot_w64(d > kNear) != 0 ? 1u << k : 0u;
}

__device__ __forceinline__ float code_of_t(float t, float y, float* d) {
  const float r = rintf(__fmul_rn(t, y));
  *d = fabsf(__builtin_fmaf(t, y, -r));
  return r;
}

__device__ __forceinline__ float code_fast(uint16_t h, float mn, float y, float* d) {
  return code_of_t(__fsub_rn(h2f(h), mn), y, d);
}

// t = RN(x - mn) for the fp16 value x in half HI of w, as one mixed-precision
// fma (x * 1 - mn with the fp16 operand widened exactly, one rounding): the
// same value as converting x and subtracting.
template <int HI>
__device__ __forceinline__ float sub_half(uint32_t w, float mn) {
  float t;
  if constexpr (HI)
    asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(t) : "v"(w), "v"(mn));
  else
    asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel_hi:[1,0,0]" : "=v"(t) : "v"(w), "v"(mn));
  return t;
}

template <int HI>
__device__ __forceinline__ float code_half(uint32_t w, float mn, float y, float* d) {
  return code_of_t(sub_half<HI>(w, mn), y, d);
}

__device__ __forceinline__ uint8_t code_exact(uint16_t h, float mn, float s, float levels) {
  const float q = __fdiv_rn(__fsub_rn(h2f(h), mn), s);
  return (uint8_t)fminf(fmaxf(rintf(q), 0.0f), levels);
}

// One per-token group: the 32 fp16 values row[0..31] (LDS, 16-byte aligned)
// to codes crow[0..31] (LDS, 4-byte aligned); returns scale/zero. The values
// are read as four 16-byte pieces starting with piece rot & 3 (callers spread
// the lanes of a wave over the LDS banks with it) and held in registers for
// both passes; codes are packed four a word. Values near a rounding boundary
// (positions the wave marks together, so the recode loop visits only those)
// are recoded with the IEEE division; a constant group takes y = 0, so all
// its codes are 0.
__device__ __forceinline__ void quantize_token32(const uint16_t* row, int rot, int bits, uint8_t* crow,
                                                 float* scale, float* zero) {
  typedef uint32_t w4_t __attribute__((ext_vector_type(4)));
  w4_t x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = *(const w4_t*)(row + 8 * ((i + rot) & 3));
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) w[i] = x[i >> 2][i & 3];
  float mn, mx;
  minmax32(w, &mn, &mx);
  const float levels = (float)((1 << bits) - 1);
  const float s = __fdiv_rn(__fsub_rn(mx, mn), levels);
  *scale = s;
  *zero = mn;
  const float y = s == 0.0f ? 0.0f : __fdiv_rn(1.0f, s);
  uint32_t near = 0;  // bit 8 i + k: value k of the piece read i-th
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t c[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
      float d0, d1;
      const uint32_t u = w[4 * i + (k >> 1)];
      const float r0 = code_half<0>(u, mn, y, &d0), r1 = code_half<1>(u, mn, y, &d1);
      near |= near_bit(d0, 8 * i + k) | near_bit(d1, 8 * i + k + 1);
      c[k >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(r0, k & 3, c[k >> 2]);
      c[k >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(r1, (k & 3) + 1, c[k >> 2]);
    }
    uint8_t* dst = crow + 8 * ((i + rot) & 3);
    *(uint32_t*)dst = c[0];
    *(uint32_t*)(dst + 4) = c[1];
  }
  while (near != 0) {  // rare
    const int b = __builtin_ctz(near);
    near &= near - 1;
    const int pos = 8 * (((b >> 3) + rot) & 3) + (b & 7);
    float d;
    (void)code_fast(row[pos], mn, y, &d);
    if (d > kNear) crow[pos] = code_exact(row[pos], mn, s, levels);
  }
}

// The value of lane l ^ 32 (h: 1 in lanes 32..63). v_permlane32_swap trades
// lanes 32..63 of its first operand with lanes 0..31 of its second.
__device__ __forceinline__ uint32_t lane_xor32(uint32_t x, int h) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  const uint32_t a = r[0], b = r[1];
  return h ? a : b;
}

// Two per-channel groups, channels c0 and c0 + 1, by lanes l and l ^ 32 of
// one wave (h = l >> 5; the whole wave must call): lane h reads the channel
// pair at rows 2i + h (i < 16) as one 32-bit word (pair: &x[h][c0], row
// stride D, LDS), the two lanes combine their minima and maxima, lane h
// computes the scale of channel c0 + h (returned with its zero), and each
// lane codes its 16 rows of both channels, two codes a 16-bit store (cpair:
// &codes[h][c0], row stride CS). Values near a rounding boundary are recoded
// as in quantize_token32.
__device__ __forceinline__ void quantize_channel_pair(const uint16_t* pair, int h, int bits, uint8_t* cpair,
                                                      float* scale, float* zero) {
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) w[i] = *(const uint32_t*)(pair + 2 * i * D);
  const uint32_t w0 = w[0];
  h2_t lo = __builtin_bit_cast(h2_t, w0), hi = lo;
#pragma unroll
  for (int i = 1; i < 16; ++i) {
    const uint32_t u = w[i];
    const h2_t v = __builtin_bit_cast(h2_t, u);
    lo = __builtin_elementwise_minimum(lo, v);
    hi = __builtin_elementwise_maximum(hi, v);
  }
  {
    const uint32_t ul = __builtin_bit_cast(uint32_t, lo), uh = __builtin_bit_cast(uint32_t, hi);
    const uint32_t pl = lane_xor32(ul, h), ph = lane_xor32(uh, h);
    lo = __builtin_elementwise_minimum(lo, __builtin_bit_cast(h2_t, pl));
    hi = __builtin_elementwise_maximum(hi, __builtin_bit_cast(h2_t, ph));
  }
  const float mn0 = (float)lo[0], mn1 = (float)lo[1];
  const float mn = h ? mn1 : mn0, mx = h ? (float)hi[1] : (float)hi[0];
  const float levels = (float)((1 << bits) - 1);
  const float s = __fdiv_rn(__fsub_rn(mx, mn), levels);
  *scale = s;
  *zero = mn;
  // a constant group (s = 0) takes y = 0: every t is 0 there, so every code 0
  const float y = s == 0.0f ? 0.0f : __fdiv_rn(1.0f, s);
  const float yp = __builtin_bit_cast(float, lane_xor32(__builtin_bit_cast(uint32_t, y), h));
  const float y0 = h ? yp : y, y1 = h ? y : yp;
  uint32_t near = 0;  // bit 2 i + e: row 2i + h, channel c0 + e
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t u = w[i];
    float d0, d1;
    const float r0 = code_half<0>(u, mn0, y0, &d0);
    const float r1 = code_half<1>(u, mn1, y1, &d1);
    near |= near_bit(d0, 2 * i) | near_bit(d1, 2 * i + 1);
    const uint32_t c = __builtin_amdgcn_cvt_pk_u8_f32(r1, 1, __builtin_amdgcn_cvt_pk_u8_f32(r0, 0, 0u));
    *(uint16_t*)(cpair + 2 * i * CS) = (uint16_t)c;
  }
  const float sp = __builtin_bit_cast(float, lane_xor32(__builtin_bit_cast(uint32_t, s), h));
  const float s0 = h ? sp : s, s1 = h ? s : sp;
  while (near != 0) {  // rare
    const int b = __builtin_ctz(near);
    near &= near - 1;
    const int i = b >> 1, e = b & 1;
    const uint16_t x = pair[2 * i * D + e];
    float d;
    (void)code_fast(x, e ? mn1 : mn0, e ? y1 : y0, &d);
    if (d > kNear) cpair[2 * i * CS + e] = code_exact(x, e ? mn1 : mn0, e ? s1 : s0, levels);
  }
}

// Word W = tid + NT k of a code block (NT = 128 or 256 threads, tid < NT):
// its lane, (W mod 256) / 4, and its word index in that lane, 4 (W / 256) +
// W mod 4, written so that the compiler sees them as per-thread bases plus
// constants.
__device__ __forceinline__ void word_of(int tid, int k, int NT, int* lane, int* w) {
  if (NT == 128) {
    *lane = (tid >> 2) + 32 * (k & 1);
    *w = 4 * (k >> 1) + (tid & 3);
  } else {
    *lane = tid >> 2;
    *w = 4 * k + (tid & 3);
  }
}

// A word of a code block into the record. STREAM: a non-temporal store, for
// records written by a prefill append and read only by later launches
// (measured: the packed words of a whole prompt stream out 3-12% faster).
template <bool STREAM>
__device__ __forceinline__ void put_word(uint8_t* p, uint32_t w) {
  if constexpr (STREAM)
    __builtin_nontemporal_store(w, (uint32_t*)p);
  else
    *(uint32_t*)p = w;
}

// Write the 512*BITS bytes of a code block from src[32][ROW] (token,
// channel): the codes (BITS <= 8, uint8 rows of the staging) or the fp16
// values themselves (BITS = 16).
template <int BITS, bool IS_V, int NT, bool STREAM, class T, int ROW>
__device__ inline void pack_block(uint8_t* blk, const T (*src)[ROW], int tid) {
  constexpr int per_word = 32 / BITS;
  constexpr int nwords = 128 * BITS;
  static_assert(nwords % NT == 0, "whole words a thread");
#pragma unroll 1
  for (int k = 0; k < nwords / NT; ++k) {
    const int W = tid + NT * k;
    int lane, w;
    word_of(tid, k, NT, &lane, &w);
    uint32_t word = 0;
#pragma unroll
    for (int p = 0; p < per_word; ++p) {
      const int e = w * per_word + p;
      int j, c;
      if (IS_V) v_inverse(lane, e, &j, &c); else k_inverse(lane, e, &j, &c);
      word |= (uint32_t)src[j][c] << ((p & 1) * 16 + (p >> 1) * BITS);
    }
    put_word<STREAM>(blk + (size_t)W * 4, word);
  }
}

// The key code block (BITS = 2, 4 or 8) from the staged codes c[32][CS]
// (token, channel). A key word holds codes of consecutive channels of one
// token (8 for 4 bits; two runs of 8 for 2 bits; 4 for 8 bits), read as
// 32-bit words and moved into place with shifts and byte permutes instead
// of one LDS read a code.
template <int BITS, int NT, bool STREAM>
__device__ inline void pack_key_codes(uint8_t* blk, const uint8_t (*c)[CS], int tid) {
  constexpr int nwords = 128 * BITS;
  static_assert(nwords % NT == 0, "whole words a thread");
#pragma unroll
  for (int k = 0; k < nwords / NT; ++k) {
    const int W = tid + NT * k;
    int lane, w;
    word_of(tid, k, NT, &lane, &w);
    const int a = lane >> 4, r = lane & 15;
    uint32_t word;
    if constexpr (BITS == 8) {
      // codes p = 0..3 of channels c0 + p go to bytes 0, 2, 1, 3
      const uint32_t d = *(const uint32_t*)&c[16 * (w >> 3) + r][32 * ((w >> 1) & 3) + 8 * a + 4 * (w & 1)];
      word = __builtin_amdgcn_perm(d, d, 0x03010200u);
    } else if constexpr (BITS == 4) {
      // codes p = 0..7: even p to nibbles 0..3, odd p to nibbles 4..7
      const uint8_t* src = &c[16 * (w >> 2) + r][32 * (w & 3) + 8 * a];
      const uint32_t d0 = *(const uint32_t*)src, d1 = *(const uint32_t*)(src + 4);
      const uint32_t f0 = d0 | d0 >> 12, f1 = d1 | d1 >> 12;  // bytes 0, 1: (p0 p2), (p1 p3) and (p4 p6), (p5 p7)
      word = __builtin_amdgcn_perm(f1, f0, 0x05010400u);
    } else {
      // codes p = 0..15 (channels of run p >> 3): even p to bits 0..15 in
      // pairs, odd p to bits 16..31
      const uint8_t* ra = &c[16 * (w >> 1) + r][32 * ((2 * w) & 3) + 8 * a];
      const uint8_t* rb = &c[16 * (w >> 1) + r][32 * ((2 * w + 1) & 3) + 8 * a];
      const uint32_t x = *(const uint32_t*)ra | *(const uint32_t*)(ra + 4) << 4;
      const uint32_t z = *(const uint32_t*)rb | *(const uint32_t*)(rb + 4) << 4;
      const uint32_t y0 = x | x >> 14, y1 = z | z >> 14;  // byte 0: even codes, byte 1: odd codes
      word = __builtin_amdgcn_perm(y1, y0, 0x05010400u);
    }
    put_word<STREAM>(blk + (size_t)W * 4, word);
  }
}

// NT threads (128 or 256), tid < NT.
template <bool IS_V, int NT, bool STREAM = false>
__device__ inline void pack_block_bits(uint8_t* blk, int bits, const uint16_t (*xs)[D], const uint8_t (*cs)[CS],
                                       int tid) {
  if constexpr (IS_V) {
    switch (bits) {
      case 2: pack_block<2, true, NT, STREAM>(blk, cs, tid); break;
      case 4: pack_block<4, true, NT, STREAM>(blk, cs, tid); break;
      case 8: pack_block<8, true, NT, STREAM>(blk, cs, tid); break;
      default: pack_block<16, true, NT, STREAM>(blk, xs, tid); break;
    }
  } else {
    switch (bits) {
      case 2: pack_key_codes<2, NT, STREAM>(blk, cs, tid); break;
      case 4: pack_key_codes<4, NT, STREAM>(blk, cs, tid); break;
      case 8: pack_key_codes<8, NT, STREAM>(blk, cs, tid); break;
      default: pack_block<16, false, NT, STREAM>(blk, xs, tid); break;
    }
  }
}

// Quantize one full 32-token group (xs: fp16 K and V [32][128], in LDS) and
// write its record; cs is LDS scratch for the codes (4-byte aligned). 256
// threads. The per-token group (row j, channels 32n ..) starts at piece
// j + 2 (n >> 1): the 16-byte reads of a wave's 64 groups then fall on
// distinct LDS banks.
__device__ __forceinline__ void quantize_record(const uint16_t (*xs)[GS][D], uint8_t (*cs)[GS][CS], uint8_t* rec, int kb,
                                       int vb, int k_token, int tid) {
  const RecordParts parts = record_parts(kb, vb);
  float* kmeta = (float*)(rec + parts.kmeta);
  float* vmeta = (float*)(rec + parts.vmeta);
  if (tid < 128) {
    if (kb == 16) {
      // the fp16 values are packed as they are, straight from xs
    } else if (!k_token) {
      // channel pair 2 p, 2 p + 1 by lanes l and l ^ 32 of wave tid / 64
      const int h = (tid >> 5) & 1, p = ((tid >> 6) << 5) | (tid & 31), c = 2 * p + h;
      float s, z;
      quantize_channel_pair(&xs[0][h][2 * p], h, kb, &cs[0][h][2 * p], &s, &z);
      kmeta[meta_channel(c)] = s;
      kmeta[128 + meta_channel(c)] = z;
    } else {
      const int j = tid >> 2, n = tid & 3;
      float s, z;
      quantize_token32(&xs[0][j][32 * n], j + 2 * (n >> 1), kb, &cs[0][j][32 * n], &s, &z);
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
      quantize_token32(&xs[1][j][32 * n], j + 2 * (n >> 1), vb, &cs[1][j][32 * n], &s, &z);
      vmeta[meta_token(j, n)] = s;
      vmeta[128 + meta_token(j, n)] = z;
    }
  }
  __syncthreads();
  pack_block_bits<false, 256>(rec, kb, xs[0], cs[0], tid);
  pack_block_bits<true, 256>(rec + parts.vcode, vb, xs[1], cs[1], tid);
}

// Quantize and pack one tensor (keys: is_v = 0, values: 1) of a full
// 32-token group (x: its fp16 rows [32][128], in LDS) into the record; c is
// LDS scratch for the codes (4-byte aligned). 128 threads (two waves), all of
// which must call; the same group split as quantize_record: per-channel keys
// by lane pairs, per-token groups one a thread.
__device__ __forceinline__ void quantize_tensor(const uint16_t (*x)[D], uint8_t (*c)[CS], uint8_t* rec, int is_v,
                                                int kb, int vb, int k_token, int tid) {
  const RecordParts parts = record_parts(kb, vb);
  const int bits = is_v ? vb : kb;
  if (bits < 16) {
    float* meta = (float*)(rec + (is_v ? parts.vmeta : parts.kmeta));
    float s, z;
    if (!is_v && !k_token) {
      const int h = (tid >> 5) & 1, p = ((tid >> 6) << 5) | (tid & 31), ch = 2 * p + h;
      quantize_channel_pair(&x[h][2 * p], h, bits, &c[h][2 * p], &s, &z);
      meta[meta_channel(ch)] = s;
      meta[128 + meta_channel(ch)] = z;
    } else {
      const int j = tid >> 2, n = tid & 3;
      quantize_token32(&x[j][32 * n], j + 2 * (n >> 1), bits, &c[j][32 * n], &s, &z);
      meta[meta_token(j, n)] = s;
      meta[128 + meta_token(j, n)] = z;
    }
  }
  __syncthreads();
  if (is_v) pack_block_bits<true, 128, true>(rec + parts.vcode, bits, x, c, tid);
  else pack_block_bits<false, 128, true>(rec, bits, x, c, tid);
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
      quantize_token32(&xs[tensor][p][32 * n], p + 2 * (n >> 1), 4, &cs[tensor][p][32 * n], &s, &z);
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
