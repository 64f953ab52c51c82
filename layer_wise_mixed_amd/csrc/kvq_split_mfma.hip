// kvq_split_mfma.hip -- the split pass of decode attention on CDNA4 matrix cores.
//
// One workgroup (4 waves) per (split, KV head, request); each wave walks every
// fourth 32-token group of the split and keeps its own running max / sum /
// output, and the four are combined through LDS at the end. Per group:
//
//  scores  S[token][col] = sum_ch A[token][ch] * B[ch][col]   (two 16x16x32 f16 MFMA tiles)
//          A = the packed key codes, fed to the MFMA as fp16 *denormals* (the code
//              bits, shifted to the top of the fp16 mantissa, so a b-bit code x is
//              the exact value x * 2^(-14-b); unpacking is one shift and one mask
//              per register);
//          B = q' * scale_k for per-channel keys (q' = q * softmax_scale * log2 e),
//              split into an fp16 high part and an fp16 low part, each its own
//              MFMA, so the product keeps ~22 significant bits;
//          score = S * 2^(14+b) + sum_ch q'_ch * zero_ch.
//  softmax exp2 of (score - running max), lazily rescaled when the max grows.
//  output  O^T[ch][col] += sum_tok V[tok][ch] * Pt[tok][col]  (eight 16x16x32 MFMA tiles)
//          with V the value codes as denormals again and Pt = p * scale_v (hi and
//          lo fp16 parts); the zero-point term sum_tok p * zero_v is kept on the side.
//
// The column index of the B operand and of the outputs carries the query row g of
// the GQA group (col % G) and, on the output side, a 32-channel group of the
// values (col / G), because value scales are per (token, channel group).
// The token order inside a group follows the cache layout: the score tile rows
// land in exactly the registers the P.V tile needs as its reduction index, so
// no data moves between lanes between the two products.
//
// The fp16 tail (tokens that do not fill a group) is processed first by the
// wave that owns it, in true units, with invalid token slots masked to zero.
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

constexpr int kMaxG = 16;
constexpr int kWaves = 4;

__device__ inline f4_t mfma(h8_t a, h8_t b, f4_t c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

// The 8 codes at positions 8u..8u+7 of a lane's sequence as an MFMA operand:
// consecutive position pairs become the two fp16 halves of one register. A
// b-bit code x goes to mantissa bits 10-b .. 9 of an fp16 denormal, i.e. the
// exact value x * 2^(-14-b) (code_scale<b>() undoes it). Keeping the code at
// the top of the mantissa matters: the matrix cores add products of tiny
// denormals with visibly less precision than the same products placed high.
template <int B>
__device__ constexpr float code_scale() {
  return B == 2 ? 65536.0f : B == 4 ? 262144.0f : B == 8 ? 4194304.0f : 1.0f;  // 2^(14+B)
}

template <int B>
__device__ inline h8_t unpack8(const uint32_t* w, int u) {
  u4_t r;
  if constexpr (B == 8) {
    const uint32_t x = w[2 * u], y = w[2 * u + 1];
    r[0] = (x << 2) & 0x03FC03FCu;
    r[1] = (x >> 6) & 0x03FC03FCu;
    r[2] = (y << 2) & 0x03FC03FCu;
    r[3] = (y >> 6) & 0x03FC03FCu;
  } else if constexpr (B == 4) {
    const uint32_t x = w[u];
    r[0] = (x << 6) & 0x03C003C0u;
    r[1] = (x << 2) & 0x03C003C0u;
    r[2] = (x >> 2) & 0x03C003C0u;
    r[3] = (x >> 6) & 0x03C003C0u;
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

// element i of (hi, lo): the fp16 rounding of x, and what it missed scaled by 2^11
// (exact), so that the low part stays in the normal fp16 range whenever x does;
// products with hi and with lo accumulate separately and meet as hi + lo * 2^-11.
constexpr float kLoUp = 2048.0f;
constexpr float kLoDown = 1.0f / 2048.0f;

__device__ inline void set_hi_lo(h8_t& hi, h8_t& lo, int i, float x) {
  const _Float16 h = (_Float16)x;
  hi[i] = h;
  lo[i] = (_Float16)((x - (float)h) * kLoUp);
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

struct Lane {
  int lane, la, c16, gcol, ns, NS;
  bool col_ok;
  float qv[32];  // q' of the lane's column for channels 32 s + 8 la + i, index 8 s + i
  float qn[4];   // per 32-channel group sums of q' (per-token keys)
};

struct Acc {
  f4_t o[8], ol[8];  // P.V products with the high and with the (2^11-scaled) low parts of P
  float m, lpart, zpart[4];
};

// One 32-token group. KB/VB: code widths (16 = fp16 values, as in the tail);
// meta: this wave's LDS copy of the group's K meta (256 floats) then V meta.
// q' as hi/lo fp16 B operands (keys without a per-channel scale)
__device__ inline void q_operands(const Lane& ln, h8_t* qh, h8_t* ql) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) set_hi_lo(qh[s], ql[s], i, ln.qv[8 * s + i]);
}

template <int KB, int VB, bool KTOK, bool TAIL>
__device__ __forceinline__ void process_group(const uint32_t* kw, const uint32_t* vw, const float* meta, int ntok,
                                              const Lane& ln, const h8_t* qh, const h8_t* ql, Acc& acc) {
  float sc[2][4];
  // ---------------------------------------------------------------- scores
  if constexpr (KB == 16) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f4_t c = {0.f, 0.f, 0.f, 0.f}, cl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const h8_t A = unpack8<16>(kw, 4 * t + s);
        c = mfma(A, qh[s], c);
        cl = mfma(A, ql[s], cl);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[t][i] = fmaf(cl[i], kLoDown, c[i]);
    }
  } else if constexpr (!KTOK) {
    h8_t bh[4], bl[4];
    float beta = 0.f;
    const float* ks = meta + 32 * ln.la;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float qt = ln.qv[8 * s + i] * ks[8 * s + i];
        set_hi_lo(bh[s], bl[s], i, qt);
        beta = fmaf(ln.qv[8 * s + i], ks[128 + 8 * s + i], beta);
      }
    }
    beta = sum_lane_groups(beta);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f4_t c = {0.f, 0.f, 0.f, 0.f}, cl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const h8_t A = unpack8<KB>(kw, 4 * t + s);
        c = mfma(A, bh[s], c);
        cl = mfma(A, bl[s], cl);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[t][i] = fmaf(fmaf(cl[i], kLoDown, c[i]), code_scale<KB>(), beta);
    }
  } else {
    // per-token keys: one accumulator per 32-channel group n (= K-step)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[t][i] = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        f4_t c = {0.f, 0.f, 0.f, 0.f}, cl = {0.f, 0.f, 0.f, 0.f};
        const h8_t A = unpack8<KB>(kw, 4 * t + s);
        c = mfma(A, qh[s], c);
        cl = mfma(A, ql[s], cl);
        const float* km = meta + 32 * s + 8 * ln.la + 4 * t;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sc[t][i] = fmaf(fmaf(cl[i], kLoDown, c[i]) * code_scale<KB>(), km[i], fmaf(km[128 + i], ln.qn[s], sc[t][i]));
      }
    }
  }
  if constexpr (TAIL) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (16 * t + 4 * ln.la + i >= ntok) sc[t][i] = -INFINITY;
  }
  // --------------------------------------------------------------- softmax
  float bm = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                   fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
  bm = max_lane_groups(bm);
  const float mnew = fmaxf(acc.m, bm);
  if (__any(mnew > acc.m)) {
    const float alpha = __builtin_amdgcn_exp2f(acc.m - mnew);  // exp2(-inf) = 0 for the first group
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
  float p[8];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = __builtin_amdgcn_exp2f(sc[t][i] - acc.m);
      p[4 * t + i] = e;
      acc.lpart += e;
    }
  // ------------------------------------------------------------ P . V
  u4_t vmask = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
  if constexpr (TAIL) {
    // reduction index i' of this lane holds token 16 (i'/4) + 4 la + i' % 4
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j0 = 16 * (q >> 1) + 4 * ln.la + 2 * (q & 1);
      vmask[q] = (j0 < ntok ? 0x0000FFFFu : 0u) | (j0 + 1 < ntok ? 0xFFFF0000u : 0u);
    }
  }
  const int NP = 4 / ln.NS;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    if (pass >= NP) continue;
    const int n = ln.col_ok ? pass * ln.NS + ln.ns : 0;
    h8_t bh, bl;
    if constexpr (VB == 16) {
#pragma unroll
      for (int i = 0; i < 8; ++i) set_hi_lo(bh, bl, i, p[i]);
    } else {
      const float* vs = meta + 256 + 32 * n + 8 * ln.la;
      float zp = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        set_hi_lo(bh, bl, i, p[i] * vs[i]);
        zp = fmaf(p[i], vs[128 + i], zp);
      }
      acc.zpart[pass] += zp;
    }
    // M-tiles of channel groups pass*NS .. pass*NS + NS - 1 (two 16-channel tiles each)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u / 2 < pass * ln.NS || u / 2 >= (pass + 1) * ln.NS) continue;
      h8_t A = unpack8<VB>(vw, u);
      if constexpr (TAIL) {
        u4_t x = __builtin_bit_cast(u4_t, A);
        x &= vmask;
        A = __builtin_bit_cast(h8_t, x);
      }
      acc.o[u] = mfma(A, bh, acc.o[u]);
      acc.ol[u] = mfma(A, bl, acc.ol[u]);
    }
  }
}

template <int KB, int VB, bool KTOK>
__global__ __launch_bounds__(256) void split_mfma_kernel(DecodeArgs a) {
  __shared__ float s_meta[kWaves][512];
  __shared__ float s_o[kWaves][kMaxG][D];
  __shared__ float s_ml[kWaves][2][kMaxG];
  const LayerGeom& g = a.geo;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
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

  Lane ln;
  ln.lane = tid & 63;
  ln.la = ln.lane >> 4;
  ln.c16 = ln.lane & 15;
  ln.gcol = ln.c16 % G;
  ln.NS = (16 / G >= 4) ? 4 : (16 / G >= 2 ? 2 : 1);  // channel groups per output pass (divides 4)
  ln.ns = ln.c16 / G;
  ln.col_ok = ln.ns < ln.NS;
  {
    const uint16_t* qrow = a.q + ((size_t)r * g.hq + h * G + ln.gcol) * D;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u4_t v = *(const u4_t*)(qrow + 32 * s + 8 * ln.la);
      const h8_t hv = __builtin_bit_cast(h8_t, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) ln.qv[8 * s + i] = (float)hv[i] * a.scale_log2;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) part += ln.qv[8 * s + i];
      ln.qn[s] = sum_lane_groups(part);
    }
  }
  Acc acc;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    acc.o[u] = f4_t{0.f, 0.f, 0.f, 0.f};
    acc.ol[u] = f4_t{0.f, 0.f, 0.f, 0.f};
  }
  acc.m = -INFINITY;
  acc.lpart = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) acc.zpart[k] = 0.f;
  float* meta = s_meta[wave];

  // the tail group first (true units), then the packed groups
  const bool has_tail = T > 0 && nq >= g0 && nq < g1;
  if (has_tail && ((nq - g0) & (kWaves - 1)) == wave) {
    const uint8_t* rec = stream + g.tail_offset;
    uint32_t kw[32], vw[32];
    load_codes<16>(rec, ln.lane, kw);
    load_codes<16>(rec + 8192, ln.lane, vw);
    h8_t th[4], tl[4];
    q_operands(ln, th, tl);
    process_group<16, 16, false, true>(kw, vw, meta, T, ln, th, tl, acc);
    if constexpr (VB < 16) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {  // into the packed groups' units
        acc.o[u] *= 1.0f / code_scale<VB>();
        acc.ol[u] *= 1.0f / code_scale<VB>();
      }
    }
  }
  const int qend = min(g1, nq);
  int vg = g0 + wave;
  if (vg < qend) {
    constexpr int NKW = 2 * KB, NVW = 2 * VB;
    const uint32_t rb = (uint32_t)g.record_bytes;
    const RecordParts parts = record_parts(KB, VB);
    uint32_t kw[NKW], vw[NVW];
    u4_t km = {0, 0, 0, 0}, vm = {0, 0, 0, 0};
    h8_t mh[4], ml[4];
    if constexpr (KB == 16 || KTOK) q_operands(ln, mh, ml);
    const uint8_t* rec = stream + (size_t)vg * rb;
    load_codes<KB>(rec, ln.lane, kw);
    load_codes<VB>(rec + parts.vcode, ln.lane, vw);
    if constexpr (KB < 16) km = *(const u4_t*)(rec + parts.kmeta + ln.lane * 16);
    if constexpr (VB < 16) vm = *(const u4_t*)(rec + parts.vmeta + ln.lane * 16);
    for (; vg < qend; vg += kWaves) {
      // meta of this group into the wave's LDS slot
      if constexpr (KB < 16) *(u4_t*)(meta + 4 * ln.lane) = km;
      if constexpr (VB < 16) *(u4_t*)(meta + 256 + 4 * ln.lane) = vm;
      wave_sync_lds();
      uint32_t kc[NKW], vc[NVW];
#pragma unroll
      for (int i = 0; i < NKW; ++i) kc[i] = kw[i];
#pragma unroll
      for (int i = 0; i < NVW; ++i) vc[i] = vw[i];
      const int nx = vg + kWaves;
      if (nx < qend) {  // prefetch the wave's next group
        const uint8_t* nrec = stream + (size_t)nx * rb;
        load_codes<KB>(nrec, ln.lane, kw);
        load_codes<VB>(nrec + parts.vcode, ln.lane, vw);
        if constexpr (KB < 16) km = *(const u4_t*)(nrec + parts.kmeta + ln.lane * 16);
        if constexpr (VB < 16) vm = *(const u4_t*)(nrec + parts.vmeta + ln.lane * 16);
      }
      process_group<KB, VB, KTOK, false>(kc, vc, meta, GS, ln, mh, ml, acc);
      wave_sync_lds();
    }
  }

  // ------------------------------------------- this wave's result into LDS
  const float l = sum_lane_groups(acc.lpart);
  const float vmul = code_scale<VB>();
  const int NP = 4 / ln.NS;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    if (pass >= NP) continue;
    const float z = sum_lane_groups(acc.zpart[pass]);
    const int n = pass * ln.NS + ln.ns;
    if (ln.col_ok) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (u / 2 != n) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s_o[wave][ln.gcol][16 * u + 4 * ln.la + i] = fmaf(fmaf(acc.ol[u][i], kLoDown, acc.o[u][i]), vmul, z);
      }
    }
  }
  if (ln.lane < G) {
    s_ml[wave][0][ln.lane] = acc.m;
    s_ml[wave][1][ln.lane] = l;
  }
  __syncthreads();
  // ------------------------------------ combine the four waves, write partial
  for (int idx = tid; idx < G * D; idx += blockDim.x) {
    const int gg = idx >> 7, c = idx & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_ml[w][0][gg]);
    float num = 0.f, den = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = s_ml[w][0][gg];
        if (mw == -INFINITY) continue;
        const float e = __builtin_amdgcn_exp2f(mw - M);
        num = fmaf(e, s_o[w][gg][c], num);
        den = fmaf(e, s_ml[w][1][gg], den);
      }
    }
    const size_t row = ((size_t)r * g.hq + h * G + gg) * a.splits + split;
    a.part_o[row * D + c] = den > 0.f ? num / den : 0.f;
    if (c == 0) a.part_lse[row] = den > 0.f ? (M + __log2f(den)) * 0.69314718055994531f : -INFINITY;
  }
}

template <int KB, int VB>
hipError_t launch_kv(const DecodeArgs& a, int batch, hipStream_t s, const EventPair* ev) {
  const dim3 grid(a.splits, a.geo.hkv, batch), block(256);
  if (a.geo.k_token && KB < 16) return launch_timed(split_mfma_kernel<KB, VB, true>, grid, block, s, ev, a);
  return launch_timed(split_mfma_kernel<KB, VB, false>, grid, block, s, ev, a);
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

hipError_t launch_decode_split_mfma(const DecodeArgs& a, int batch, hipStream_t s, const EventPair* ev) {
  switch (a.geo.kb) {
    case 2: return launch_k<2>(a, batch, s, ev);
    case 4: return launch_k<4>(a, batch, s, ev);
    case 8: return launch_k<8>(a, batch, s, ev);
    default: return launch_k<16>(a, batch, s, ev);
  }
}

}  // namespace kvq
