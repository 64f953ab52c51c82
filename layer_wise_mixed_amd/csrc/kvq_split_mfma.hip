// kvq_split_mfma.hip -- the split pass of decode attention on CDNA4 matrix cores.
//
// One workgroup (4 waves) per (split, KV head, request). Wave w walks groups
// w, w+4, w+8, ... of the split (32 tokens each) with the next group's loads in
// flight, keeps its own running max / sum / output, and the four waves are
// combined through LDS at the end. With a single split the combine writes the
// final output and log-sum-exp directly; otherwise it writes the split's
// partial for the merge pass. Per group:
//
//  scores  S[token][col] = sum_ch A[token][ch] * B[ch][col]   (two 16x16x32 f16 MFMA tiles)
//          A = the packed key codes, fed to the MFMA as fp16 denormals: a b-bit
//              code x sits in the mantissa as the exact value x * 2^-u(b)
//              (u = 16, 20, 24 for 2, 4, 8 bits; one mask, or a shift and a mask,
//              or one byte permute per register);
//          B = q'' * scale_k, q'' = q * softmax_scale * log2 e * 2^-E with a
//              power of two per query row that brings max |q''| into [1/2, 1)
//              (so |B| <= 43669 for any fp16 keys), as an fp16 high part and the
//              fp16 rounding of what it missed (taken from the exact product),
//              both into one accumulator: ~21 significant bits;
//          score = S * 2^u * 2^E + sum_ch q'_ch * zero_ch.
//  softmax exp2 of (score - running max), rescaled lazily when the max grows.
//  output  O^T[ch][col] += sum_tok V[tok][ch] * Pt[tok][col]  (eight 16x16x32 MFMA tiles)
//          V: the value codes as denormals again, Pt = p * scale_v (high part
//          and a 2^10-scaled low part with its own accumulator, so that values
//          of tiny groups keep their precision); the zero-point term sum_tok p *
//          zero_v is kept on the side.
//
// Columns. The 16 columns of the 16x16 tiles carry (query row g of the GQA
// group = col % G, slot = col / G). On the output side the slot is a 32-channel
// group of the values (value scales are per token and channel group); with
// NS = min(4, 16/G) slots, 4/NS passes cover the four channel groups. On the
// score side of per-channel keys the slot is one of the next NS groups of the
// wave: the B operand q' * scale_k is built once for NS groups, each group's
// scores come out in the columns of its slot, and one ds_bpermute per score
// hands them to the lanes of the other slots.
//
// The token order inside a group follows the cache layout: the score-tile rows
// land in exactly the registers the P.V tile needs as its reduction index.
// The fp16 tail (tokens that do not fill a group) is processed first, in true
// units, by the wave that owns it, with invalid token slots masked.
#include <type_traits>

#include "kvq_internal.h"
#include "kvq_quantize.h"


namespace kvq {
namespace {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

constexpr int kMaxG = 16;
constexpr int kWaves = 4;

__device__ inline f4_t mfma(h8_t a, h8_t b, f4_t c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

// 2^u(b): the value of code 1 as the MFMA sees it is 2^-u(b).
template <int B>
__device__ constexpr float code_scale() {
  return B == 2 ? 65536.0f : B == 4 ? 1048576.0f : B == 8 ? 16777216.0f : 1.0f;
}

// The 8 codes at positions 8u..8u+7 of a lane's sequence as an MFMA operand:
// consecutive position pairs become the two fp16 halves of one register, each
// code in the mantissa of an fp16 denormal: 8-bit codes at bits 0..7 (one
// byte permute), 4-bit codes at bits 4..7, 2-bit codes at bits 8..9. Codes
// of two or four bits are kept away from the bottom of the mantissa: the
// matrix cores add products of the smallest denormals with less precision
// (measured on gfx950 against exact sums: relative error ~1e-6 for 2- and
// 4-bit codes at bits 0.., ~2e-8 at bits 4.. and 8.., ~7e-8 for 8-bit
// codes at bits 0..).
template <int B>
__device__ inline h8_t unpack8(const uint32_t* w, int u) {
  u4_t r;
  if constexpr (B == 8) {
    const uint32_t x = w[2 * u], y = w[2 * u + 1];
    r[0] = __builtin_amdgcn_perm(0u, x, 0x0c020c00u);  // bytes 0 and 2: positions 0 and 1
    r[1] = __builtin_amdgcn_perm(0u, x, 0x0c030c01u);  // bytes 1 and 3: positions 2 and 3
    r[2] = __builtin_amdgcn_perm(0u, y, 0x0c020c00u);
    r[3] = __builtin_amdgcn_perm(0u, y, 0x0c030c01u);
  } else if constexpr (B == 4) {
    const uint32_t x = w[u];
    r[0] = (x << 4) & 0x00F000F0u;
    r[1] = x & 0x00F000F0u;
    r[2] = (x >> 4) & 0x00F000F0u;
    r[3] = (x >> 8) & 0x00F000F0u;
  } else if constexpr (B == 2) {
    const uint32_t x = w[u >> 1];
    if (u & 1) {
      r[0] = x & 0x03000300u;
      r[1] = (x >> 2) & 0x03000300u;
      r[2] = (x >> 4) & 0x03000300u;
      r[3] = (x >> 6) & 0x03000300u;
    } else {
      r[0] = (x << 8) & 0x03000300u;
      r[1] = (x << 6) & 0x03000300u;
      r[2] = (x << 4) & 0x03000300u;
      r[3] = (x << 2) & 0x03000300u;
    }
  } else {
    r[0] = w[4 * u];
    r[1] = w[4 * u + 1];
    r[2] = w[4 * u + 2];
    r[3] = w[4 * u + 3];
  }
  return __builtin_bit_cast(h8_t, r);
}

// A lane's 2*B words of a code block: B/2 rows of 1 KiB, 16 bytes each.
template <int B>
__device__ inline void load_codes(const uint8_t* blk, int lane, uint32_t* w) {
#pragma unroll
  for (int k = 0; k < B / 2; ++k) {
    const u4_t v = __builtin_nontemporal_load((const u4_t*)(blk + k * 1024 + lane * 16));
    w[4 * k + 0] = v[0];
    w[4 * k + 1] = v[1];
    w[4 * k + 2] = v[2];
    w[4 * k + 3] = v[3];
  }
}

// Value side, elements i, i+1 of (hi, lo): an fp16 rounding of x and what it
// missed, scaled by 2^10 and rounded to fp16, so hi + lo / 2^10 keeps ~21
// significant bits of x, also for the tiny x of tiny value groups. The high
// part is one packed round-toward-zero conversion, an operation the compiler
// cannot re-form from the product behind x (were it to round that product
// once in one place and twice in another, the parts would disagree by an
// ulp). Its residual is below one fp16 ulp of x, so the scaled low part stays
// below |x| (x = p * scale_v <= (65504 + 65504) / 3 for fp16 values: no
// overflow).
constexpr float kLoUp = 1024.0f;
constexpr float kLoDown = 1.0f / 1024.0f;

__device__ inline void set_hi_lo2(h8_t& hi, h8_t& lo, int i, float x0, float x1) {
  const auto h = __builtin_amdgcn_cvt_pkrtz(x0, x1);
  hi[i] = h[0];
  hi[i + 1] = h[1];
  lo[i] = (_Float16)fmaf(-(float)h[0], kLoUp, x0 * kLoUp);
  lo[i + 1] = (_Float16)fmaf(-(float)h[1], kLoUp, x1 * kLoUp);
}

// Score side, elements i, i+1 of (hi, lo) for x = a * b: the packed
// round-toward-zero fp16 of x, and the fp16 rounding of a * b - hi (the
// compiler takes it from the exact product in one mixed-precision fma), both
// multiplied into one accumulator. Scores need absolute, not relative,
// accuracy, and the low part's absolute error is at most 2^-25 even where it
// falls in the fp16 denormal range.
__device__ inline void set_hi_lo2_prod(h8_t& hi, h8_t& lo, int i, float a0, float b0, float a1, float b1) {
  const auto h = __builtin_amdgcn_cvt_pkrtz(a0 * b0, a1 * b1);
  hi[i] = h[0];
  hi[i + 1] = h[1];
  lo[i] = (_Float16)(a0 * b0 - (float)h[0]);
  lo[i + 1] = (_Float16)(a1 * b1 - (float)h[1]);
}

__device__ inline void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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

__device__ inline float bpermute(int addr, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(addr, __builtin_bit_cast(int, v)));
}

struct Lane {
  int lane, la, gcol, slot, g;
  bool col_ok;
  const float* qv;  // LDS: q'' = q' 2^-E of the lane's row at channels 32 s + 8 la + i is qv[32 s + i]
  float qe;         // 2^E of the lane's row
  float qn[4];      // per 32-channel group sums of q' (per-token keys)
};

struct Acc {
  f4_t o[8], ol[8];  // P.V with the high and with the (2^10-scaled) low parts of Pt
  float m, lpart, zpart[4];
};

// The score B operand lives in the wave's own LDS, not in registers (it is
// reused by up to four groups, and 32 registers held across the group loop
// are what would spill): for K-step s, the high parts at bst[2s][lane] and
// the low parts at bst[2s + 1][lane], one 16-byte piece per lane. Each lane
// reads back only what it wrote, so program order is the only ordering
// needed.
typedef u4_t BStore[8][64];

__device__ __forceinline__ void store_b(BStore& bst, int s, int lane, const h8_t& hi, const h8_t& lo) {
  bst[2 * s][lane] = __builtin_bit_cast(u4_t, hi);
  bst[2 * s + 1][lane] = __builtin_bit_cast(u4_t, lo);
}

// B operand of q'' alone (keys without per-channel scale: fp16 tail, 16-bit
// and per-token keys)
__device__ inline void q_operands(const Lane& ln, BStore& bst) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    h8_t qh, ql;
#pragma unroll
    for (int i = 0; i < 8; i += 2)
      set_hi_lo2_prod(qh, ql, i, ln.qv[32 * s + i], 1.0f, ln.qv[32 * s + i + 1], 1.0f);
    store_b(bst, s, ln.lane, qh, ql);
  }
}

// B operand q'' * scale_k of per-channel keys for the group of this lane's
// slot, and beta = sum over all 128 channels of q' * zero_k for the lane's
// column.
__device__ inline float k_operands(const Lane& ln, const float* kmeta, BStore& bst) {
  const float* ks = kmeta + 32 * ln.la;
  float beta = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    h8_t bh, bl;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float q0 = ln.qv[32 * s + i], q1 = ln.qv[32 * s + i + 1];
      set_hi_lo2_prod(bh, bl, i, q0, ks[8 * s + i], q1, ks[8 * s + i + 1]);
      beta = fmaf(q1, ks[128 + 8 * s + i + 1], fmaf(q0, ks[128 + 8 * s + i], beta));
    }
    store_b(bst, s, ln.lane, bh, bl);
  }
  return sum_lane_groups(beta) * ln.qe;
}

// Scores of one 32-token group in log2 units, token 16 t + 4 la + i at index
// 4 t + i. KB: key code width (16 = fp16 values, as in the tail); bh/bl: the
// score B operand; beta: the key zero-point term (per-channel keys); src: byte
// address of the lane whose scores this lane takes (per-channel keys stacked
// over slots; < 0: its own); kmeta: LDS copy of the group's key meta
// (per-token keys). Tail slots at or past ntok get -inf.
template <int KB, bool KTOK, bool TAIL>
__device__ __forceinline__ void group_scores(const uint32_t* kw, const float* kmeta, int ntok, const BStore& bst,
                                             float beta, int src, const Lane& ln, float* sc) {
  const float cs = code_scale<KB>() * ln.qe;
  if constexpr (!KTOK || KB == 16) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const h8_t A = unpack8<KB>(kw, 4 * t + s);
        c = mfma(A, __builtin_bit_cast(h8_t, bst[2 * s][ln.lane]), c);
        c = mfma(A, __builtin_bit_cast(h8_t, bst[2 * s + 1][ln.lane]), c);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[4 * t + i] = fmaf(c[i], cs, beta);
    }
    if constexpr (KB < 16) {
      if (src >= 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) sc[i] = bpermute(src, sc[i]);
      }
    }
  } else {
    // per-token keys: one accumulator per 32-channel group n (= K-step)
#pragma unroll
    for (int i = 0; i < 8; ++i) sc[i] = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        f4_t c = {0.f, 0.f, 0.f, 0.f};
        const h8_t A = unpack8<KB>(kw, 4 * t + s);
        c = mfma(A, __builtin_bit_cast(h8_t, bst[2 * s][ln.lane]), c);
        c = mfma(A, __builtin_bit_cast(h8_t, bst[2 * s + 1][ln.lane]), c);
        const float* km = kmeta + 32 * s + 8 * ln.la + 4 * t;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sc[4 * t + i] = fmaf(c[i] * cs, km[i], fmaf(km[128 + i], ln.qn[s], sc[4 * t + i]));
      }
    }
  }
  if constexpr (TAIL) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (16 * t + 4 * ln.la + i >= ntok) sc[4 * t + i] = -INFINITY;
  }
}

// The softmax reference acc.m only has to bound every score seen so far
// (weights exp2(score - m) <= 1, the fp16 operand range relies on it): when
// a block's scores pass it, it moves to the block max plus kHeadroom, so that
// later blocks rarely pass it again and the accumulators are rescaled (64
// multiplies) a few times per wave instead of at most groups. The largest
// weight is then between 2^-kHeadroom and 1, which costs the hi/lo operand
// split nothing but that many bits of exponent range. Whether anything passed
// is one vote over each lane's own scores against its column's reference;
// only then is the column max formed across the four lane groups.
constexpr float kHeadroom = 3.0f;

__device__ __forceinline__ void raise_max(float bm, Acc& acc) {
  if (__any(bm > acc.m)) {
    bm = max_lane_groups(bm);
    const float mnew = bm > acc.m ? bm + kHeadroom : acc.m;
    // 0 while nothing is accumulated (acc.m = -inf; also when mnew is)
    const float alpha = acc.m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(acc.m - mnew);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      acc.o[u] *= alpha;
      acc.ol[u] *= alpha;
    }
    acc.lpart *= alpha;
#pragma unroll
    for (int k = 0; k < 4; ++k) acc.zpart[k] *= alpha;
    acc.m = mnew;
  }
}

// The P.V operand of value tile u (channels 16u..16u+15). VPAGE: vw holds the
// V words of two INT4 pages, [page a words 0..3][page b words 0..3]; the
// record word u is bytes h, h+2 of page a's word u/2 interleaved with the same
// bytes of page b's (h = u % 2).
template <int VB, bool VPAGE>
__device__ __forceinline__ h8_t value_operand(const uint32_t* vw, int u) {
  if constexpr (VPAGE) {
    const uint32_t x = vw[u >> 1], y = vw[4 + (u >> 1)];
    const uint32_t w = (u & 1) ? (((x >> 8) & 0x00FF00FFu) | (y & 0xFF00FF00u))
                               : ((x & 0x00FF00FFu) | ((y << 8) & 0xFF00FF00u));
    return unpack8<4>(&w, 0);
  } else {
    return unpack8<VB>(vw, u);
  }
}

// p = exp2(score - max) of one group, and its P.V products. VB: value code
// width; vmeta: LDS copy of the group's value meta.
template <int VB, int NS, bool TAIL, bool VPAGE = false>
__device__ __forceinline__ void group_pv(const uint32_t* vw, const float* vmeta, int ntok, const float* sc,
                                         const Lane& ln, Acc& acc) {
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = __builtin_amdgcn_exp2f(sc[i] - acc.m);
    acc.lpart += p[i];
  }
  u4_t vmask = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
  if constexpr (TAIL) {
    // reduction index i' of this lane holds token 16 (i'/4) + 4 la + i' % 4
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j0 = 16 * (q >> 1) + 4 * ln.la + 2 * (q & 1);
      vmask[q] = (j0 < ntok ? 0x0000FFFFu : 0u) | (j0 + 1 < ntok ? 0xFFFF0000u : 0u);
    }
  }
#pragma unroll
  for (int pass = 0; pass < 4 / NS; ++pass) {
    h8_t vh, vl;
    if constexpr (VB == 16) {
#pragma unroll
      for (int i = 0; i < 8; i += 2) set_hi_lo2(vh, vl, i, p[i], p[i + 1]);
    } else {
      const int n = ln.col_ok ? pass * NS + ln.slot : 0;
      const float* vs = vmeta + 32 * n + 8 * ln.la;
      float zp = 0.f;
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        set_hi_lo2(vh, vl, i, p[i] * vs[i], p[i + 1] * vs[i + 1]);
        zp = fmaf(p[i + 1], vs[128 + i + 1], fmaf(p[i], vs[128 + i], zp));
      }
      acc.zpart[pass] += zp;
    }
    // the two 16-channel tiles of each of channel groups pass*NS .. pass*NS + NS - 1
#pragma unroll
    for (int u = 2 * pass * NS; u < 2 * (pass + 1) * NS; ++u) {
      h8_t A = value_operand<VB, VPAGE>(vw, u);
      if constexpr (TAIL) {
        u4_t x = __builtin_bit_cast(u4_t, A);
        x &= vmask;
        A = __builtin_bit_cast(h8_t, x);
      }
      acc.o[u] = mfma(A, vh, acc.o[u]);
      acc.ol[u] = mfma(A, vl, acc.ol[u]);
    }
  }
}

template <int KB, int VB, bool KTOK, int NS, bool TAIL, bool VPAGE = false>
__device__ __forceinline__ void process_group(const uint32_t* kw, const uint32_t* vw, const float* kmeta,
                                              const float* vmeta, int ntok, const BStore& bst,
                                              float beta, int src, const Lane& ln, Acc& acc) {
  float sc[8];
  group_scores<KB, KTOK, TAIL>(kw, kmeta, ntok, bst, beta, src, ln, sc);
  raise_max(fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7]))),
            acc);
  group_pv<VB, NS, TAIL, VPAGE>(vw, vmeta, ntok, sc, ln, acc);
}

// Every member is a multiple of 16 bytes long, so with the struct aligned
// each member is too (LDS reads of q', meta and results stay 16 bytes wide).
// The per-wave results of the combine have storage of their own, so a wave
// writes its result as soon as it is done, and one barrier starts the combine.
template <int R>
struct alignas(16) SplitSmem {
  struct Loop {
    float kmeta[kWaves][R][256];  // per wave: the key meta of up to R groups
    float vmeta[kWaves][256];     // per wave: the value meta of the current group
  };
  struct Flush {
    uint16_t xs[2][GS][D];   // fused append: the group's fp16 K and V
    uint8_t cs[2][GS][CS];   // and its codes
  };
  union {
    Loop loop;
    Flush flush;
  };
  // per wave: the score B operand during its group loop, then its result
  // for the combine (a wave writes its result once its own loop is done)
  union WaveLds {
    BStore b;
    float o[kMaxG][D];
  } wl[kWaves];
  float ml[kWaves][2][kMaxG];
  float q[kMaxG][D];  // q'' of the G query rows (every wave writes the same values)
  float qe[kMaxG];    // 2^E of each row
};

// The query rows of a workgroup, the G query heads of one KV head
// (consecutive rows): row i reads q at ptr(i) and writes output row out(i).
struct HeadRows {
  const uint16_t* q;
  size_t row0;
  __device__ __forceinline__ size_t out(int i) const { return row0 + i; }
  __device__ __forceinline__ const uint16_t* ptr(int i) const { return q + (row0 + i) * D; }
};

// The lane's roles, q' = q * softmax_scale * log2(e) of the G rows into LDS,
// and (per-token keys) the sums of q' over each 32-channel group. Every wave
// writes all of q' (the same values), so no wave waits for another.
template <int NS, bool QN>
__device__ __forceinline__ void setup_lane(const DecodeArgs& a, int G, const HeadRows& rows, float (*s_q)[D],
                                           float* s_qe, Lane& ln, Acc& acc) {
  const int tid = threadIdx.x;
  ln.lane = tid & 63;
  ln.la = ln.lane >> 4;
  ln.g = G;
  const int c16 = ln.lane & 15;
  ln.gcol = c16 % G;
  ln.slot = c16 / G;
  ln.col_ok = ln.slot < NS;
  // 8 values a lane at a time: in each pass the 16 lanes 16k .. 16k + 15 hold
  // one whole row, so the row's largest |q'| is a max over those 16 lanes
  for (int c = ln.lane; c < G * (D / 8); c += 64) {
    const u4_t w = *(const u4_t*)(rows.ptr(0) + 8 * c);
    const h8_t x = __builtin_bit_cast(h8_t, w);
    float v[8], mx = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = (float)x[i] * a.scale_log2;
      mx = fmaxf(mx, fabsf(v[i]));
    }
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) mx = fmaxf(mx, __shfl_xor(mx, d));
    int E = 0;
    (void)frexpf(mx, &E);  // max |q'| = f 2^E, f in [1/2, 1); E = 0 for a zero row
    float* dst = &s_q[c >> 4][8 * (c & 15)];
    f4_t lo4, hi4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo4[i] = ldexpf(v[i], -E);
      hi4[i] = ldexpf(v[4 + i], -E);
    }
    *(f4_t*)dst = lo4;
    *(f4_t*)(dst + 4) = hi4;
    if ((c & 15) == 0) s_qe[c >> 4] = ldexpf(1.0f, E);
  }
  wave_sync_lds();
  ln.qv = &s_q[ln.gcol][8 * ln.la];
  ln.qe = s_qe[ln.gcol];
  if constexpr (QN) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) part += ln.qv[32 * s + i];
      ln.qn[s] = sum_lane_groups(part) * ln.qe;
    }
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    acc.o[u] = f4_t{0.f, 0.f, 0.f, 0.f};
    acc.ol[u] = f4_t{0.f, 0.f, 0.f, 0.f};
  }
  acc.m = -INFINITY;
  acc.lpart = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) acc.zpart[k] = 0.f;
}

// Each wave's result into LDS, the four waves combined, and the split's
// output written: the final output when it is the only split, else the
// split's partial (o, lse) for the merge pass. VB: the value code width the
// wave's accumulators are in.
template <int VB, int NS, int R>
__device__ __forceinline__ void finish(const DecodeArgs& a, const HeadRows& rows, int split, int wave, SplitSmem<R>& sm,
                                       const Lane& ln, Acc& acc) {
  const int tid = threadIdx.x;
  const int G = ln.g;
  const float l = sum_lane_groups(acc.lpart);
  const float vmul = code_scale<VB>();
#pragma unroll
  for (int pass = 0; pass < 4 / NS; ++pass) {
    const float z = sum_lane_groups(acc.zpart[pass]);
    // the lane's column holds channel group n = pass * NS + slot: tiles 2n, 2n + 1
    // (picked by selects: a runtime index would send the accumulators to scratch)
    f4_t o[2], ol[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      o[t] = acc.o[2 * pass * NS + t];
      ol[t] = acc.ol[2 * pass * NS + t];
#pragma unroll
      for (int q = 1; q < NS; ++q) {
        const bool take = ln.slot == q;
        o[t] = take ? acc.o[2 * (pass * NS + q) + t] : o[t];
        ol[t] = take ? acc.ol[2 * (pass * NS + q) + t] : ol[t];
      }
    }
    if (ln.col_ok) {
      const int n = pass * NS + ln.slot;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sm.wl[wave].o[ln.gcol][32 * n + 16 * t + 4 * ln.la + i] = fmaf(fmaf(ol[t][i], kLoDown, o[t][i]), vmul, z);
    }
  }
  if (ln.lane < G) {
    sm.ml[wave][0][ln.lane] = acc.m;
    sm.ml[wave][1][ln.lane] = l;
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += blockDim.x) {
    const int gg = idx >> 7, c = idx & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.ml[w][0][gg]);
    float num = 0.f, den = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = sm.ml[w][0][gg];
        if (mw == -INFINITY) continue;
        const float e = __builtin_amdgcn_exp2f(mw - M);
        num = fmaf(e, sm.wl[w].o[gg][c], num);
        den = fmaf(e, sm.ml[w][1][gg], den);
      }
    }
    const float o = den > 0.f ? num / den : 0.f;
    const float lse = den > 0.f ? (M + __log2f(den)) * 0.69314718055994531f : -INFINITY;
    const size_t qrow = rows.out(gg);
    if (a.splits == 1) {  // the only split: final output
      if (a.out_f32)
        ((float*)a.out)[qrow * D + c] = o;
      else
        ((_Float16*)a.out)[qrow * D + c] = (_Float16)o;
      if (c == 0 && a.lse_out) a.lse_out[qrow] = lse;
    } else {
      const size_t row = qrow * a.splits + split;
      a.part_o[row * D + c] = o;
      if (c == 0) a.part_lse[row] = lse;
    }
  }
}

// ---------------------------------------------------------- group sources
// Where the wave's k-th packed group lives. Each source loads a lane's code
// words (and, for per-token values, its 16 bytes of value meta) and its 16
// bytes of key meta, in the layout of a 32-token record.

// Records first, first + 4, first + 8, ... of one contiguous stream.
template <int KB, int VB>
struct StreamSrc {
  const uint8_t* first;  // the wave's first record
  uint32_t stride;       // kWaves records
  RecordParts parts;
  static constexpr bool kVPage = false;
  __device__ __forceinline__ const uint8_t* rec(int k) const { return first + (size_t)k * stride; }
  __device__ __forceinline__ void load(int k, int lane, uint32_t* kw, uint32_t* vw, u4_t& vm) const {
    const uint8_t* r = rec(k);
    load_codes<KB>(r, lane, kw);
    load_codes<VB>(r + parts.vcode, lane, vw);
    if constexpr (VB < 16) vm = *(const u4_t*)(r + parts.vmeta + lane * 16);
  }
  __device__ __forceinline__ u4_t kmeta(int k, int lane) const { return *(const u4_t*)(rec(k) + parts.kmeta + lane * 16); }
};

// INT2 groups of a paged request: the K2V2 record of one KV head in the page
// pair of group first + 4 k. ids: lane i holds the even page id of the wave's
// group i (i < 64).
struct Int2Src {
  const uint8_t* base;  // pool + h * 4096
  uint64_t page_bytes;
  int ids;
  static constexpr bool kVPage = false;
  __device__ __forceinline__ const uint8_t* rec(int k) const {
    return base + (size_t)__builtin_amdgcn_readlane(ids, k) * page_bytes;
  }
  __device__ __forceinline__ void load(int k, int lane, uint32_t* kw, uint32_t* vw, u4_t& vm) const {
    const uint8_t* r = rec(k);
    load_codes<2>(r, lane, kw);
    load_codes<2>(r + 1024, lane, vw);
    vm = *(const u4_t*)(r + 3072 + lane * 16);
  }
  __device__ __forceinline__ u4_t kmeta(int k, int lane) const { return *(const u4_t*)(rec(k) + 2048 + lane * 16); }
};

// INT4 page pairs of a paged request: group i is the pages of table entries
// 2i, 2i + 1 of its INT4 part (tokens 32 i .. 32 i + 31). ida/idb: lane i
// holds the two pages' region indices for the wave's group i (i < 64).
struct Int4Src {
  const uint8_t* base;  // INT4 region + h * 3072
  uint64_t page_bytes;
  int ida, idb;
  static constexpr bool kVPage = true;
  __device__ __forceinline__ const uint8_t* page(int id) const { return base + (size_t)id * page_bytes; }
  __device__ __forceinline__ void load(int k, int lane, uint32_t* kw, uint32_t* vw, u4_t& vm) const {
    const uint8_t* pa = page(__builtin_amdgcn_readlane(ida, k));
    const uint8_t* pb = page(__builtin_amdgcn_readlane(idb, k));
    load_codes<2>(pa, lane, kw);  // one 16-byte row per page: key words 0..3 and 4..7
    load_codes<2>(pb, lane, kw + 4);
    load_codes<2>(pa + INT4_VCODE, lane, vw);
    load_codes<2>(pb + INT4_VCODE, lane, vw + 4);
    vm = *(const u4_t*)(meta_site(pa, pb, lane) + INT4_VMETA);
  }
  // lane l's 16 bytes of a record's per-token meta (record floats 4l .. 4l+3)
  // come from page l % 2: scales for l < 32, zeros after, channel group
  // (l % 32) / 8, slots 4 ((l % 8) / 2) + 0..3
  __device__ __forceinline__ static const uint8_t* meta_site(const uint8_t* pa, const uint8_t* pb, int lane) {
    return ((lane & 1) ? pb : pa) + (lane >> 5) * 256 + ((lane & 31) >> 1) * 16;
  }
  __device__ __forceinline__ u4_t kmeta(int k, int lane) const {
    const uint8_t* pa = page(__builtin_amdgcn_readlane(ida, k));
    const uint8_t* pb = page(__builtin_amdgcn_readlane(idb, k));
    return *(const u4_t*)(meta_site(pa, pb, lane) + INT4_KMETA);
  }
};

// Issue priority from the wave's progress: 1 until three quarters of its
// groups are done, then 0. Two workgroups share each CU and the older one's
// waves win the issue arbitration, so with equal work the younger one used
// to finish a quarter later and run alone meanwhile; the waves that reach
// three quarters first now yield until the others get there too.
__device__ __forceinline__ void progress_priority(int done, int nk) {
  if (4 * done < 3 * nk) {
    __builtin_amdgcn_s_setprio(1);
  } else {
    __builtin_amdgcn_s_setprio(0);
  }
}

// The wave's nk packed groups from `src`, one group loading ahead in a second
// register buffer; the loop is unrolled by two so every buffer index is
// static (no register copies). setup() (the wave's q' setup) runs once the
// first group's loads are issued, so that the two memory waits overlap.
template <int KB, int VB, bool KTOK, int NS, int R, class Src, class Setup>
__device__ __forceinline__ void run_groups(const Src& src, int nk, float* kmeta, float* vmeta, BStore& bst,
                                           const Lane& ln, Acc& acc, Setup&& setup) {
  constexpr bool STACK = KB < 16 && !KTOK;  // per-channel keys: one B operand for R groups
  constexpr int NKW = 2 * KB, NVW = 2 * VB;
  constexpr bool VPAGE = Src::kVPage;
  struct Buf {
    uint32_t kw[NKW];
    uint32_t vw[NVW];
    u4_t vm;
  };
  Buf buf[2];
  u4_t kmr[R];
  const int lane = threadIdx.x & 63;
  if (nk > 0) {  // the first group loads while setup() waits on q
    src.load(0, lane, buf[0].kw, buf[0].vw, buf[0].vm);
    if constexpr (KB < 16) {
#pragma unroll
      for (int f = 0; f < R; ++f) kmr[f] = f < nk ? src.kmeta(f, lane) : u4_t{0, 0, 0, 0};
    }
  }
  setup();
  if (nk <= 0) return;
  progress_priority(0, nk);
  float beta = 0.f;
  if constexpr (!STACK) q_operands(ln, bst);
  auto step = [&](auto J, int k) {
    constexpr int j = decltype(J)::value;
    const int e = STACK ? k % R : 0;  // slot of this group in its stack
    if constexpr (KB < 16) {
      if (e == 0) {
#pragma unroll
        for (int f = 0; f < R; ++f) *(u4_t*)(kmeta + 256 * f + 4 * ln.lane) = kmr[f];
      }
    }
    if constexpr (VB < 16) *(u4_t*)(vmeta + 4 * ln.lane) = buf[j].vm;
    wave_sync_lds();
    if (k + 1 < nk) src.load(k + 1, ln.lane, buf[j ^ 1].kw, buf[j ^ 1].vw, buf[j ^ 1].vm);
    if constexpr (KB < 16) {
      if (k + 1 < nk && (k + 1) % R == 0) {
#pragma unroll
        for (int f = 0; f < R; ++f) kmr[f] = k + 1 + f < nk ? src.kmeta(k + 1 + f, ln.lane) : u4_t{0, 0, 0, 0};
      }
    }
    int srcl = -1;  // the lane holding this lane's scores: same row, column of slot e
    if constexpr (STACK) {
      if (e == 0) beta = k_operands(ln, kmeta + 256 * (ln.col_ok ? ln.slot : 0), bst);
      srcl = ((ln.lane & 48) | (ln.gcol + ln.g * e)) * 4;
    }
    process_group<KB, VB, KTOK, NS, false, VPAGE>(buf[j].kw, buf[j].vw, kmeta, vmeta, GS, bst, beta, srcl, ln,
                                                  acc);
    wave_sync_lds();
    progress_priority(k + 1, nk);
  };
  for (int k = 0; k < nk; k += 2) {
    step(std::integral_constant<int, 0>{}, k);
    if (k + 1 < nk) step(std::integral_constant<int, 1>{}, k + 1);
  }
}

// Fused append, new token completes group m: the whole workgroup quantizes
// the tail's 31 tokens and the new one into record m (the same quantizer and
// packer as the append kernel), with xs/cs as LDS staging; the closing
// barrier makes the record visible to the waves that load it.
__device__ __forceinline__ void flush_group(uint8_t* stream, const LayerGeom& g, int m, const uint16_t* kn,
                                            const uint16_t* vn, uint16_t (*xs)[GS][D], uint8_t (*cs)[GS][CS]) {
  const int tid = threadIdx.x;
  const uint8_t* tail = stream + g.tail_offset;
  // the tail record as 1024 16-byte rows (lane l of 1 KiB row w: words 4w ..
  // 4w + 3 of lane l), four a thread, all loads issued before any is used
  u4_t rows[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) rows[q] = *(const u4_t*)(tail + (size_t)(tid + 256 * q) * 16);
  const uint16_t nk = kn[tid & 127], nv = vn[tid & 127];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ch = tid + 256 * q;  // rows 0..511: keys, 512..1023: values
    const bool is_v = ch >= 512;
    const int lane = ch & 63, w0 = 4 * ((ch & 511) >> 6);
#pragma unroll
    for (int e2 = 0; e2 < 8; ++e2) {
      const int e = 2 * w0 + e2;
      int j, c;
      if (is_v) v_inverse(lane, e, &j, &c); else k_inverse(lane, e, &j, &c);
      if (j < GS - 1) xs[is_v][j][c] = (uint16_t)(rows[q][e2 >> 1] >> (16 * (e2 & 1)));
    }
  }
  xs[tid >> 7][GS - 1][tid & 127] = tid < 128 ? nk : nv;  // the new token is slot 31
  __syncthreads();
  quantize_record(xs, cs, stream + (size_t)m * g.record_bytes, g.kb, g.vb, g.k_token, tid);
  __syncthreads();
}

// Fused append, otherwise: the new token into tail slot j, for the wave
// that owns the tail, once it has loaded the tail record into kw/vw (the
// K16V16 layout). Each lane loads its own pieces of the token (keys: lanes
// j%16 + 16a hold channels 32s + 8a .. + 7 at words 16(j/16) + 4s .. + 3;
// values: lanes 16((j%16)/4) + c%16 hold channel c%16 + 16u at word
// 4u + 2(j/16) + (j%4)/2, half j%2), puts them into its registers, and
// stores them into the tail record for later steps (the bytes the append
// kernel writes).
__device__ __forceinline__ void merge_new_token(uint8_t* tail, const uint16_t* kn, const uint16_t* vn, int j, int lane,
                                                uint32_t* kw, uint32_t* vw) {
  const bool kl = (lane & 15) == (j & 15);
  const bool vl = (lane >> 4) == ((j & 15) >> 2);
  const int a4 = lane >> 4, cl = lane & 15;
  // every lane loads (valid addresses for all): a load under a lane condition
  // would make the compiler wait for all loads in flight (the tail's too)
  // before the other lanes' values could be written to the same registers
  u4_t kv[4];
  uint16_t vv[8];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) kv[s4] = *(const u4_t*)(kn + 32 * s4 + 8 * a4);
#pragma unroll
  for (int u = 0; u < 8; ++u) vv[u] = vn[16 * u + cl];
  if (kl) {
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) *(u4_t*)(tail + word_offset(lane, 16 * (j >> 4) + 4 * s4)) = kv[s4];
  }
  if (vl) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = 8 * u + 4 * (j >> 4) + (j & 3);
      *(uint16_t*)(tail + 8192 + word_offset(lane, e >> 1) + (e & 1) * 2) = vv[u];
    }
  }
  // every register index static: each word takes the new piece or keeps its
  // value by a select (an index computed from j would put kw/vw in scratch)
  const bool hi16 = j >= 16;
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kw[4 * s4 + i] = kl && !hi16 ? kv[s4][i] : kw[4 * s4 + i];
      kw[16 + 4 * s4 + i] = kl && hi16 ? kv[s4][i] : kw[16 + 4 * s4 + i];
    }
  const int wsel = 2 * (j >> 4) + ((j & 3) >> 1);
  const int hs = 16 * (j & 1);
  const uint32_t keep = ~(0xFFFFu << hs);
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w)
      vw[4 * u + w] = vl && w == wsel ? (vw[4 * u + w] & keep) | ((uint32_t)vv[u] << hs) : vw[4 * u + w];
}

// The fp16 tail (T tokens) from its words kw/vw, by the wave that owns it,
// in true units: the accumulators go to true units and back. kn/vn (fused
// append, the token went to the tail): the new token, merged into the tail's
// registers and stored into its record.
// The tail record's words for a lane (K16V16 layout) into kw/vw.
__device__ __forceinline__ void load_tail(const uint8_t* rec, int T, int lane, uint32_t* kw, uint32_t* vw) {
  // only the 16-byte pieces that hold a token below T come from their own
  // address: key row k (words 4k .. 4k+3) of lane l holds token 16 (k / 4) +
  // l % 16, every value row of lane l tokens 4 (l / 16) + 0..3 and 16 more.
  // The other lanes read the record's first piece (one line for all; the tail
  // masking ignores what they get), so no load waits on a lane condition.
  const uint32_t voff = 4 * (lane >> 4) < T ? 8192u + lane * 16u : 0u;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t koff = 16 * (k >> 2) + (lane & 15) < T ? k * 1024u + lane * 16u : 0u;
    const u4_t x = __builtin_nontemporal_load((const u4_t*)(rec + koff));
    const u4_t y = __builtin_nontemporal_load((const u4_t*)(rec + (voff ? voff + k * 1024u : 0u)));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kw[4 * k + i] = x[i];
      vw[4 * k + i] = y[i];
    }
  }
}

template <int VB, int NS>
__device__ __forceinline__ void tail_pass(uint8_t* rec, int T, const uint16_t* kn, const uint16_t* vn, uint32_t* kw,
                                          uint32_t* vw, float* kmeta, float* vmeta, BStore& bst, const Lane& ln,
                                          Acc& acc) {
  const int lane = ln.lane;
  if (kn) merge_new_token(rec, kn, vn, T - 1, lane, kw, vw);
  if constexpr (VB < 16) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      acc.o[u] *= code_scale<VB>();
      acc.ol[u] *= code_scale<VB>();
    }
  }
  q_operands(ln, bst);
  process_group<16, 16, false, NS, true>(kw, vw, kmeta, vmeta, T, bst, 0.f, -1, ln, acc);
  if constexpr (VB < 16) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      acc.o[u] *= 1.0f / code_scale<VB>();
      acc.ol[u] *= 1.0f / code_scale<VB>();
    }
  }
}

// Contiguous streams: one workgroup per (split, KV head, request). With
// a.k_new set, the pass also appends one token per request (as the append
// kernel would with n_new = 1) and attends over the cache including it: a
// token that completes a group is packed before the loop starts; one that
// goes to the tail joins the tail pass at the end.
template <int KB, int VB, bool KTOK, int NS>
__global__ __launch_bounds__(256, 2) void split_mfma_kernel(DecodeArgs a) {
  constexpr int R = (KB < 16 && !KTOK) ? NS : 1;
  __shared__ SplitSmem<R> sm;
  const LayerGeom& g = a.geo;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x, h = blockIdx.y, r = blockIdx.z;
  const int L0 = a.seq_lens[r];
  // a fused append adds token L0 where the append kernel would (0 <= L0 <
  // capacity); the attention covers the lengths a decode after it would see
  const bool app = a.k_new != nullptr && L0 >= 0 && L0 < g.max_tokens;
  int L = a.k_new != nullptr && L0 < g.max_tokens ? L0 + 1 : L0;
  if (L < 0) L = 0;
  if (L > g.max_tokens) L = g.max_tokens;
  const int nq = L / GS;
  const int T = L - nq * GS;
  const int nvg = nq + (T > 0);
  const int g0 = split * a.groups_per_split;
  const int g1 = min(g0 + a.groups_per_split, nvg);
  uint8_t* stream = g.base + (size_t)(r * g.hkv + h) * g.stream_bytes;
  const size_t sigma = (size_t)r * g.hkv + h;
  const uint16_t* kn = app ? a.k_new + sigma * D : nullptr;
  const uint16_t* vn = app ? a.v_new + sigma * D : nullptr;
  if (app) {
    if (L0 % GS == GS - 1) {
      const int m = L0 / GS;
      if (m >= g0 && m < g1) {
        flush_group(stream, g, m, kn, vn, sm.flush.xs, sm.flush.cs);
      }
    }
  }

  Lane ln;
  Acc acc;
  float* kmeta = &sm.loop.kmeta[wave][0][0];
  float* vmeta = sm.loop.vmeta[wave];

  // The wave's packed groups: g0 + wave + 4 k, and the tail (if this split
  // has it) by wave (nq - g0) % 4 after its groups. A short split (at most
  // two groups a wave) gives the tail wave no packed groups instead: the other
  // three waves share them, g0 + i + 3 k for the i-th of them, and the tail
  // wave loads the tail at once, so that it does not start its tail only
  // when the others are done.
  const int qend = min(g1, nq);
  const bool has_tail = T > 0 && nq >= g0 && nq < g1;
  const int tail_wave = (nq - g0) & (kWaves - 1);
  const bool own_tail = has_tail && wave == tail_wave;
  const bool solo = has_tail && qend - g0 <= 2 * kWaves;
  const int ways = solo ? kWaves - 1 : kWaves;
  const int first = solo ? (own_tail ? qend : g0 + wave - (wave > tail_wave)) : g0 + wave;
  const int nk = first < qend ? (qend - first + ways - 1) / ways : 0;
  StreamSrc<KB, VB> src;
  src.first = stream + (size_t)first * g.record_bytes;
  src.stride = (uint32_t)(ways * g.record_bytes);
  src.parts = record_parts(KB, VB);
  const HeadRows rows{a.q, (size_t)r * g.hq + h * g.g};
  uint8_t* tail = stream + g.tail_offset;
  uint32_t tkw[32], tvw[32];
  if (own_tail && nk == 0) {
    load_tail(tail, T, threadIdx.x & 63, tkw, tvw);
    setup_lane<NS, KTOK && KB < 16>(a, g.g, rows, sm.q, sm.qe, ln, acc);
    tail_pass<VB, NS>(tail, T, kn, vn, tkw, tvw, kmeta, vmeta, sm.wl[wave].b, ln, acc);
  } else {
    run_groups<KB, VB, KTOK, NS, R>(src, nk, kmeta, vmeta, sm.wl[wave].b, ln, acc,
                                    [&] { setup_lane<NS, KTOK && KB < 16>(a, g.g, rows, sm.q, sm.qe, ln, acc); });
    if (own_tail) {
      load_tail(tail, T, threadIdx.x & 63, tkw, tvw);
      tail_pass<VB, NS>(tail, T, kn, vn, tkw, tvw, kmeta, vmeta, sm.wl[wave].b, ln, acc);
    }
  }
  finish<VB, NS>(a, rows, split, wave, sm, ln, acc);
}

// Paged pool: the splits of a request cover its INT2 groups first, then its
// INT4 page pairs, each split of one kind only (TriAxialKV page, "Facts": the
// page table puts INT2 pages first, so flash-decoding splits are
// bitwidth-homogeneous; their partials merge by log-sum-exp).
template <int NS>
__device__ __forceinline__ void paged_int2_split(const DecodeArgs& a, SplitSmem<NS>& sm, int r, int h, int split,
                                                 int g0, int g1, const int32_t* table) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  Lane ln;
  Acc acc;
  const int first = g0 + wave;
  const int nk = first < g1 ? (g1 - first + kWaves - 1) / kWaves : 0;
  Int2Src src;
  src.base = a.geo.base + (size_t)h * INT2_RECORD;
  src.page_bytes = a.pg.int2_page_bytes;
  src.ids = lane < nk ? table[2 * (first + kWaves * lane)] : 0;
  const HeadRows rows{a.q, (size_t)r * a.geo.hq + h * a.geo.g};
  run_groups<2, 2, false, NS, NS>(src, nk, &sm.loop.kmeta[wave][0][0], sm.loop.vmeta[wave], sm.wl[wave].b, ln, acc,
                                  [&] { setup_lane<NS, false>(a, a.geo.g, rows, sm.q, sm.qe, ln, acc); });
  finish<2, NS>(a, rows, split, wave, sm, ln, acc);
}

// Fused append in a paged pool: one wave writes a new token into slot p of
// its KV head's share of an INT4 page (per-token 4-bit codes and meta, the
// same arithmetic and layout as the append kernel, TriAxialKV page, "Facts":
// decoded tokens take the INT4 per-token path). Lanes 8g .. 8g + 7 quantize
// group g (tensor g / 4, channel group g % 4), four channels a lane; the codes
// meet in the wave's LDS scratch (256 bytes) for the packing. Value words
// hold four slots: only this slot's nibbles change.
__device__ __forceinline__ void append_int4_token_wave(uint8_t* page, const uint16_t* kn, const uint16_t* vn, int p,
                                                       int lane, uint8_t* scratch) {
  const int g = lane >> 3, tensor = g >> 2, n = g & 3, sub = lane & 7;
  const int c0 = 32 * n + 4 * sub;
  typedef uint16_t us4_t __attribute__((ext_vector_type(4)));
  const us4_t raw = *(const us4_t*)((tensor ? vn : kn) + c0);
  float x[4], mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = h2f(raw[i]);
    mn = fminf(mn, x[i]);
    mx = fmaxf(mx, x[i]);
  }
#pragma unroll
  for (int d = 1; d < 8; d <<= 1) {
    mn = fminf(mn, __shfl_xor(mn, d));
    mx = fmaxf(mx, __shfl_xor(mx, d));
  }
  const float s = __fdiv_rn(__fsub_rn(mx, mn), 15.0f);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float r = 0.f;
    if (s != 0.0f) r = fminf(fmaxf(rintf(__fdiv_rn(__fsub_rn(x[i], mn), s)), 0.0f), 15.0f);
    scratch[128 * tensor + c0 + i] = (uint8_t)r;
  }
  if (sub == 0) {
    float* meta = (float*)(page + (tensor ? INT4_VMETA : INT4_KMETA));
    meta[16 * n + p] = s;
    meta[64 + 16 * n + p] = mn;
  }
  wave_sync_lds();
  if (lane < 16) {  // key word (a4, w): the 8 codes of channels 32w + 8a4 .. + 7, this slot only
    const int a4 = lane >> 2, w = lane & 3;
    uint32_t word = 0;
#pragma unroll
    for (int pos = 0; pos < 8; ++pos)
      word |= (uint32_t)scratch[32 * w + 8 * a4 + pos] << (16 * (pos & 1) + 4 * (pos >> 1));
    int sh;
    *(uint32_t*)(page + page_k_offset(p, 32 * w + 8 * a4, &sh)) = word;
  }
  {  // value word (channel c % 16 = lane % 16, u / 2 = lane / 16): channels 16u + c15 for u = 2(lane/16), + 1
    const int c15 = lane & 15, uh = lane >> 4;
    int sh;
    const uint32_t off = page_v_offset(p, 16 * (2 * uh) + c15, &sh);
    uint32_t word = *(const uint32_t*)(page + off);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int c = 16 * (2 * uh + e) + c15;
      (void)page_v_offset(p, c, &sh);
      word = (word & ~(0xFu << sh)) | ((uint32_t)scratch[128 + c] << sh);
    }
    *(uint32_t*)(page + off) = word;
  }
}

template <int NS>
__device__ __forceinline__ void paged_int4_split(const DecodeArgs& a, SplitSmem<NS>& sm, int r, int h, int split,
                                                 int g0, int g1, int n4, int n4_old, const int32_t* table,
                                                 int e4) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  Lane ln;
  Acc acc;
  float* kmeta = &sm.loop.kmeta[wave][0][0];
  float* vmeta = sm.loop.vmeta[wave];
  const int full = n4 / GS;  // page pairs holding 32 tokens
  const int np = (n4 + PAGE_TOKENS - 1) / PAGE_TOKENS;
  Int4Src src;
  src.base = a.geo.base + a.pg.int4_offset + (size_t)h * INT4_HEAD;
  src.page_bytes = a.pg.int4_page_bytes;
  auto region = [&](int e) { return e < np ? table[e] - a.pg.int2_pages : 0; };

  const int first = g0 + wave;
  const int qend = min(g1, full);
  const int nk = first < qend ? (qend - first + kWaves - 1) / kWaves : 0;
  const int gi = first + kWaves * lane;
  src.ida = lane < nk ? region(2 * gi) : 0;
  src.idb = lane < nk ? region(2 * gi + 1) : 0;
  const HeadRows rows{a.q, (size_t)r * a.geo.hq + h * a.geo.g};
  // fused append: the wave that reads the new token's pair writes the token,
  // and no other wave reads that pair. run_groups issues the loads of the
  // wave's first group before setup(): when that group is the pair, the
  // token goes in first; otherwise while the first group loads. The fence
  // completes the writes before the wave's later loads.
  const int pn = n4_old / GS;
  // (e4: the table entry of the request's first INT4 page; a page id the
  // table gives for the new token must be an INT4 page, or nothing is written)
  const int entry = e4 + n4_old / PAGE_TOKENS;
  const bool own = a.k_new != nullptr && pn >= g0 && pn < g1 && ((pn - g0) & (kWaves - 1)) == wave &&
                   entry < a.pg.max_pages && int4_page_ok(a.pg, entry, table[n4_old / PAGE_TOKENS]);
  const bool early = own && pn == first && pn < qend;
  auto append = [&] {
    const size_t sigma = (size_t)r * a.geo.hkv + h;
    uint8_t* page = a.geo.base + a.pg.int4_offset +
                    (size_t)(table[n4_old / PAGE_TOKENS] - a.pg.int2_pages) * a.pg.int4_page_bytes +
                    (size_t)h * INT4_HEAD;
    append_int4_token_wave(page, a.k_new + sigma * D, a.v_new + sigma * D, n4_old % PAGE_TOKENS, lane,
                           reinterpret_cast<uint8_t*>(vmeta));
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  };
  if (early) append();
  run_groups<4, 4, true, NS, 1>(src, nk, kmeta, vmeta, sm.wl[wave].b, ln, acc, [&] {
    setup_lane<NS, true>(a, a.geo.g, rows, sm.q, sm.qe, ln, acc);
    if (own && !early) append();
  });

  // the last, partly filled pair (same units as the full ones), by its wave
  const int pg = full;
  if (pg < (n4 + GS - 1) / GS && pg >= g0 && pg < g1 && ((pg - g0) & (kWaves - 1)) == wave) {
    const int ntok = n4 - GS * pg;
    src.ida = region(2 * pg);
    src.idb = ntok > PAGE_TOKENS ? region(2 * pg + 1) : src.ida;
    uint32_t kw[8], vw[8];
    u4_t vm;
    src.load(0, lane, kw, vw, vm);
    u4_t km = src.kmeta(0, lane);
    // slots at or past ntok hold no token: zero their meta (scores are masked
    // to -inf and value codes to 0 by the group's tail handling)
    const int j0 = 16 * (lane & 1) + 4 * (((lane & 31) >> 1) & 3);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (j0 + i >= ntok) {
        vm[i] = 0u;
        km[i] = 0u;
      }
    }
    *(u4_t*)(kmeta + 4 * lane) = km;
    *(u4_t*)(vmeta + 4 * lane) = vm;
    wave_sync_lds();
    q_operands(ln, sm.wl[wave].b);
    process_group<4, 4, true, NS, true, true>(kw, vw, kmeta, vmeta, ntok, sm.wl[wave].b, 0.f, -1, ln, acc);
    wave_sync_lds();
  }
  finish<4, NS>(a, rows, split, wave, sm, ln, acc);
}

template <int NS>
__global__ __launch_bounds__(256, 2) void paged_split_kernel(DecodeArgs a) {
  __shared__ SplitSmem<NS> sm;
  const int split = blockIdx.x, h = blockIdx.y, r = blockIdx.z;
  const int n2 = max(a.pg.int2_len[r], 0), n4_old = max(a.pg.int4_len[r], 0);
  // a fused append adds INT4 token n4_old (int4_len counts the tokens before
  // it); the attention covers the lengths a decode after it would see
  const int n4 = a.k_new != nullptr ? n4_old + 1 : n4_old;
  const int gps = a.groups_per_split;
  const int n2g = n2 / GS, n4g = (n4 + GS - 1) / GS, full4 = n4 / GS;
  const int s2 = (n2g + gps - 1) / gps;  // splits of the INT2 part
  // splits of the INT4 part: gps complete page pairs each; a last, partly
  // filled pair joins the last of them (a split of its own without complete
  // pairs); splits past these stay empty
  const int s4 = full4 > 0 ? (full4 + gps - 1) / gps : (n4g > 0 ? 1 : 0);
  const int32_t* table = a.pg.table + (size_t)r * a.pg.max_pages;
  if (split < s2) {
    const int g0 = split * gps;
    paged_int2_split<NS>(a, sm, r, h, split, g0, min(g0 + gps, n2g), table);
  } else {
    const int i = split - s2;
    const int g0 = i < s4 ? i * gps : n4g;
    const int g1 = i < s4 - 1 ? g0 + gps : n4g;
    const int32_t* table4 = table + n2 / PAGE_TOKENS;
    paged_int4_split<NS>(a, sm, r, h, split, g0, g1, n4, n4_old, table4, n2 / PAGE_TOKENS);
  }
}

template <int KB, int VB, int NS>
hipError_t launch_kvn(const DecodeArgs& a, int batch, hipStream_t s, const EventPair* ev) {
  const dim3 grid(a.splits, a.geo.hkv, batch), block(256);
  if constexpr (KB < 16) {
    if (a.geo.k_token) return launch_timed(split_mfma_kernel<KB, VB, true, NS>, grid, block, s, ev, a);
  }
  return launch_timed(split_mfma_kernel<KB, VB, false, NS>, grid, block, s, ev, a);
}

template <int KB, int VB>
hipError_t launch_kv(const DecodeArgs& a, int batch, hipStream_t s, const EventPair* ev) {
  const int per = 16 / a.geo.g;
  if (per >= 4) return launch_kvn<KB, VB, 4>(a, batch, s, ev);
  if (per >= 2) return launch_kvn<KB, VB, 2>(a, batch, s, ev);
  return launch_kvn<KB, VB, 1>(a, batch, s, ev);
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

hipError_t launch_decode_paged(const DecodeArgs& a, int batch, hipStream_t s, const EventPair* ev) {
  const dim3 grid(a.splits, a.geo.hkv, batch), block(256);
  const int per = 16 / a.geo.g;
  if (per >= 4) return launch_timed(paged_split_kernel<4>, grid, block, s, ev, a);
  if (per >= 2) return launch_timed(paged_split_kernel<2>, grid, block, s, ev, a);
  return launch_timed(paged_split_kernel<1>, grid, block, s, ev, a);
}

hipError_t launch_decode_split_mfma(const DecodeArgs& a, int batch, hipStream_t s, const EventPair* ev) {
  switch (a.geo.kb) {
    case 2: return launch_k<2>(a, batch, s, ev);
    case 4: return launch_k<4>(a, batch, s, ev);
    case 8: return launch_k<8>(a, batch, s, ev);
    default: return launch_k<16>(a, batch, s, ev);
  }
}

}  // namespace kvq
