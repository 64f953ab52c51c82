/*
 * kvq_oracle.c -- plain, slow CPU reference of the layer-wise mixed-precision
 * KV-cache path. TEST INFRASTRUCTURE ONLY: the library under test never links,
 * loads or calls this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do. It shares no code with the HIP library.
 *
 * What it follows:
 *  - Quantizer: asymmetric groupwise min/max with group size 32
 *    (TriAxialKV page, "Facts": the quantizer is asymmetric groupwise with
 *    group size 32; KVTuner summary page, "Facts": asymmetric quantization,
 *    keys per-channel because of channel-wise outliers). The exact arithmetic
 *    is: scale = (max - min) / (2^b - 1) in fp32, zero = min,
 *    code = clamp(round-half-even((x - zero) / scale), 0, 2^b - 1),
 *    IEEE fp32 subtraction and division, no contraction.
 *  - Key axis: per-channel (one scale/zero per channel per 32-token group) or
 *    per-token (one per token per 32-channel group); values per-token
 *    (TriAxialKV page, "Facts": INT2 per-channel keys, per-token values, INT4
 *    per-token for both).
 *  - Per-layer (bK, bV) pairs such as K8V4 / K4V2 (KVTuner summary page,
 *    "Approach"); b = 16 is a passthrough (fp16 stored as is).
 *  - Tokens that do not fill a 32-token group stay fp16 (the residual the
 *    TriAxialKV page contrasts its leftover routing with, "Facts").
 *  - Attention: plain softmax attention of one decode query over all cached
 *    tokens, in fp64, on the dequantized cache; dequantization is
 *    fmaf(code, scale, zero).
 *  - Split merge by log-sum-exp (TriAxialKV page, "Facts": flash-decoding
 *    splits merged by online log-sum-exp).
 *  - Byte layout of packed codes: the layout this project defines for its
 *    cache (no page prescribes one); written here from its definition,
 *    independently of the GPU code.
 *
 * Build: gcc -O2 -fPIC -shared -ffp-contract=off -fno-fast-math -fopenmp.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OQ_D 128
#define OQ_G 32

/* ---------------------------------------------------------------- fp16 -- */

/* IEEE binary16 -> binary32, exact. */
float oq_half_to_float(uint16_t h)
{
    uint32_t sign = (h >> 15) & 1u;
    uint32_t ex = (h >> 10) & 0x1Fu;
    uint32_t man = h & 0x3FFu;
    float v;
    if (ex == 0)
        v = ldexpf((float)man, -24);
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexpf((float)(man | 0x400u), (int)ex - 25);
    return sign ? -v : v;
}

/* ----------------------------------------------------------- quantizer -- */

/* One group of n fp16 values (stride apart) at `bits` in {2,4,8}. */
void oq_quantize_group(const uint16_t *x, int64_t stride, int n, int bits,
                       float *scale, float *zero, uint8_t *codes)
{
    float mn = INFINITY, mx = -INFINITY;
    for (int i = 0; i < n; ++i) {
        float xf = oq_half_to_float(x[(int64_t)i * stride]);
        if (xf < mn) mn = xf;
        if (xf > mx) mx = xf;
    }
    float levels = (float)((1 << bits) - 1);
    float s = (mx - mn) / levels;
    *scale = s;
    *zero = mn;
    for (int i = 0; i < n; ++i) {
        float xf = oq_half_to_float(x[(int64_t)i * stride]);
        uint8_t c = 0;
        if (s != 0.0f) {
            float t = (xf - mn) / s;
            float r = nearbyintf(t); /* default rounding mode: half to even */
            if (r < 0.0f) r = 0.0f;
            if (r > levels) r = levels;
            c = (uint8_t)r;
        }
        codes[i] = c;
    }
}

float oq_dequant(uint32_t code, float scale, float zero)
{
    return fmaf((float)code, scale, zero);
}

/*
 * Quantize one (layer, request, KV head) stream of L tokens, fp16 [L][128]
 * for k and v. Tokens below Lq = 32*floor(L/32) are quantized; the rest stay
 * fp16. Logical outputs:
 *   kcode/vcode [Lq][128] (unused for b = 16)
 *   K per-channel meta: kscale/kzero [Lq/32][128]
 *   K per-token meta and V meta: [Lq][4] (one per 32-channel group)
 */
void oq_quantize_stream(const uint16_t *k, const uint16_t *v, int64_t L,
                        int kb, int vb, int kaxis_token,
                        uint8_t *kcode, float *kscale, float *kzero,
                        uint8_t *vcode, float *vscale, float *vzero)
{
    int64_t lq = (L / OQ_G) * OQ_G;
    uint8_t tmp[OQ_G];
    if (kb < 16) {
        if (!kaxis_token) {
            for (int64_t m = 0; m < lq / OQ_G; ++m)
                for (int c = 0; c < OQ_D; ++c) {
                    oq_quantize_group(k + (m * OQ_G) * OQ_D + c, OQ_D, OQ_G, kb,
                                      &kscale[m * OQ_D + c], &kzero[m * OQ_D + c], tmp);
                    for (int i = 0; i < OQ_G; ++i)
                        kcode[(m * OQ_G + i) * OQ_D + c] = tmp[i];
                }
        } else {
            for (int64_t j = 0; j < lq; ++j)
                for (int n = 0; n < OQ_D / OQ_G; ++n)
                    oq_quantize_group(k + j * OQ_D + n * OQ_G, 1, OQ_G, kb,
                                      &kscale[j * 4 + n], &kzero[j * 4 + n],
                                      kcode + j * OQ_D + n * OQ_G);
        }
    }
    if (vb < 16) {
        for (int64_t j = 0; j < lq; ++j)
            for (int n = 0; n < OQ_D / OQ_G; ++n)
                oq_quantize_group(v + j * OQ_D + n * OQ_G, 1, OQ_G, vb,
                                  &vscale[j * 4 + n], &vzero[j * 4 + n],
                                  vcode + j * OQ_D + n * OQ_G);
    }
}

/* Dequantized stream, float [L][128] each. */
void oq_dequant_stream(const uint16_t *k, const uint16_t *v, int64_t L,
                       int kb, int vb, int kaxis_token,
                       const uint8_t *kcode, const float *kscale, const float *kzero,
                       const uint8_t *vcode, const float *vscale, const float *vzero,
                       float *kdeq, float *vdeq)
{
    int64_t lq = (L / OQ_G) * OQ_G;
    for (int64_t j = 0; j < L; ++j)
        for (int c = 0; c < OQ_D; ++c) {
            int64_t e = j * OQ_D + c;
            if (j < lq && kb < 16) {
                int64_t mi = kaxis_token ? j * 4 + c / OQ_G : (j / OQ_G) * OQ_D + c;
                kdeq[e] = oq_dequant(kcode[e], kscale[mi], kzero[mi]);
            } else {
                kdeq[e] = oq_half_to_float(k[e]);
            }
            if (j < lq && vb < 16) {
                int64_t mi = j * 4 + c / OQ_G;
                vdeq[e] = oq_dequant(vcode[e], vscale[mi], vzero[mi]);
            } else {
                vdeq[e] = oq_half_to_float(v[e]);
            }
        }
}

/* -------------------------------------------------------------- layout -- */
/*
 * A 32-token group is stored as one record:
 *   [K codes 512*bK B][V codes 512*bV B][K meta 1 KiB if bK<16][V meta 1 KiB if bV<16]
 * Codes of a block are split among 64 "lanes"; each lane owns an ordered
 * sequence of codes, packed into 32-bit little-endian words: inside a word the
 * even positions fill bits 0..15 and the odd positions bits 16..31, each from
 * the least significant bit up. Lane word w lives at byte
 * (w / 4) * 1024 + lane * 16 + (w % 4) * 4 of the block.
 *   K (token j in 0..31, channel c): lane = 16*((c/8)%4) + j%16,
 *       position e = 32*(j/16) + 8*(c/32) + c%8.
 *   V (token j, channel c): lane = 16*((j%16)/4) + c%16,
 *       position e = 8*(c/16) + 4*(j/16) + j%4.
 * Meta block (1 KiB) = 128 fp32 scales then 128 fp32 zeros:
 *   per-channel K: index 32*((c/8)%4) + 8*(c/32) + c%8
 *   per-token (V, or K per-token): index 32*n + 8*((j%16)/4) + 4*(j/16) + j%4,
 *       n = channel group c/32.
 * A stream (one request, one KV head of one layer) is groups_cap records
 * followed by one tail record in the K16V16 format, whose token slot s holds
 * token 32*floor(L/32) + s.
 */

static int64_t oq_word_addr(int lane, int w)
{
    return (int64_t)(w / 4) * 1024 + (int64_t)lane * 16 + (int64_t)(w % 4) * 4;
}

static void oq_code_site(int lane, int e, int bits, int64_t *byte, int *shift)
{
    int per_word = 32 / bits;
    int w = e / per_word;
    int ep = e % per_word;
    *byte = oq_word_addr(lane, w);
    *shift = (ep % 2) * 16 + (ep / 2) * bits;
}

static void oq_put(uint8_t *blk, int lane, int e, int bits, uint32_t code, uint8_t *mask)
{
    int64_t b;
    int sh;
    oq_code_site(lane, e, bits, &b, &sh);
    uint32_t w;
    memcpy(&w, blk + b, 4);
    uint32_t m = (bits == 32 ? 0xFFFFFFFFu : ((1u << bits) - 1u)) << sh;
    w = (w & ~m) | ((code << sh) & m);
    memcpy(blk + b, &w, 4);
    if (mask) {
        for (int i = 0; i < bits; ++i) {
            int bit = sh + i;
            mask[b + bit / 8] = 1;
        }
    }
}

static uint32_t oq_get(const uint8_t *blk, int lane, int e, int bits)
{
    int64_t b;
    int sh;
    oq_code_site(lane, e, bits, &b, &sh);
    uint32_t w;
    memcpy(&w, blk + b, 4);
    return (w >> sh) & ((1u << bits) - 1u);
}

void oq_k_site(int j, int c, int *lane, int *e)
{
    *lane = 16 * ((c / 8) % 4) + j % 16;
    *e = 32 * (j / 16) + 8 * (c / 32) + c % 8;
}

void oq_v_site(int j, int c, int *lane, int *e)
{
    *lane = 16 * ((j % 16) / 4) + c % 16;
    *e = 8 * (c / 16) + 4 * (j / 16) + j % 4;
}

int oq_meta_channel_index(int c) { return 32 * ((c / 8) % 4) + 8 * (c / 32) + c % 8; }

int oq_meta_token_index(int j, int n) { return 32 * n + 8 * ((j % 16) / 4) + 4 * (j / 16) + j % 4; }

int64_t oq_record_bytes(int kb, int vb)
{
    return 512 * (int64_t)kb + 512 * (int64_t)vb + (kb < 16 ? 1024 : 0) + (vb < 16 ? 1024 : 0);
}

int64_t oq_stream_bytes(int kb, int vb, int64_t groups_cap)
{
    return groups_cap * oq_record_bytes(kb, vb) + oq_record_bytes(16, 16);
}

static void oq_put_f32(uint8_t *blk, int64_t idx, float f, uint8_t *mask)
{
    memcpy(blk + idx * 4, &f, 4);
    if (mask) memset(mask + idx * 4, 1, 4);
}

/*
 * Pack the logical result of oq_quantize_stream into stream bytes `out`
 * (oq_stream_bytes long). `mask`, if not NULL, gets 1 on every byte that the
 * call defines (records of full groups, and the tail slots below L % 32).
 */
void oq_pack_stream(const uint16_t *k, const uint16_t *v, int64_t L, int kb, int vb,
                    int kaxis_token, int64_t groups_cap,
                    const uint8_t *kcode, const float *kscale, const float *kzero,
                    const uint8_t *vcode, const float *vscale, const float *vzero,
                    uint8_t *out, uint8_t *mask)
{
    int64_t ng = L / OQ_G;
    int64_t rb = oq_record_bytes(kb, vb);
    int64_t vc_off = 512 * (int64_t)kb;
    int64_t km_off = vc_off + 512 * (int64_t)vb;
    int64_t vm_off = km_off + (kb < 16 ? 1024 : 0);
    for (int64_t m = 0; m < ng; ++m) {
        uint8_t *rec = out + m * rb;
        uint8_t *rmask = mask ? mask + m * rb : NULL;
        for (int j = 0; j < OQ_G; ++j)
            for (int c = 0; c < OQ_D; ++c) {
                int64_t t = (m * OQ_G + j) * OQ_D + c;
                int lane, e;
                oq_k_site(j, c, &lane, &e);
                oq_put(rec, lane, e, kb, kb < 16 ? kcode[t] : k[t], rmask);
                oq_v_site(j, c, &lane, &e);
                oq_put(rec + vc_off, lane, e, vb, vb < 16 ? vcode[t] : v[t], rmask ? rmask + vc_off : NULL);
            }
        if (kb < 16) {
            uint8_t *mb = rec + km_off;
            uint8_t *mm = rmask ? rmask + km_off : NULL;
            if (!kaxis_token) {
                for (int c = 0; c < OQ_D; ++c) {
                    int ix = oq_meta_channel_index(c);
                    oq_put_f32(mb, ix, kscale[m * OQ_D + c], mm);
                    oq_put_f32(mb, 128 + ix, kzero[m * OQ_D + c], mm);
                }
            } else {
                for (int j = 0; j < OQ_G; ++j)
                    for (int n = 0; n < 4; ++n) {
                        int ix = oq_meta_token_index(j, n);
                        oq_put_f32(mb, ix, kscale[(m * OQ_G + j) * 4 + n], mm);
                        oq_put_f32(mb, 128 + ix, kzero[(m * OQ_G + j) * 4 + n], mm);
                    }
            }
        }
        if (vb < 16) {
            uint8_t *mb = rec + vm_off;
            uint8_t *mm = rmask ? rmask + vm_off : NULL;
            for (int j = 0; j < OQ_G; ++j)
                for (int n = 0; n < 4; ++n) {
                    int ix = oq_meta_token_index(j, n);
                    oq_put_f32(mb, ix, vscale[(m * OQ_G + j) * 4 + n], mm);
                    oq_put_f32(mb, 128 + ix, vzero[(m * OQ_G + j) * 4 + n], mm);
                }
        }
    }
    /* tail record, K16V16 format */
    uint8_t *tail = out + groups_cap * rb;
    uint8_t *tmask = mask ? mask + groups_cap * rb : NULL;
    for (int64_t j = ng * OQ_G; j < L; ++j) {
        int s = (int)(j - ng * OQ_G);
        for (int c = 0; c < OQ_D; ++c) {
            int lane, e;
            oq_k_site(s, c, &lane, &e);
            oq_put(tail, lane, e, 16, k[j * OQ_D + c], tmask);
            oq_v_site(s, c, &lane, &e);
            oq_put(tail + 8192, lane, e, 16, v[j * OQ_D + c], tmask ? tmask + 8192 : NULL);
        }
    }
}

/*
 * Read a stream of L tokens back from its bytes and dequantize it,
 * float [L][128] each (the oracle's own packed cache; used for round trips
 * and for the CPU baseline).
 */
void oq_unpack_stream(const uint8_t *bytes, int64_t L, int kb, int vb, int kaxis_token,
                      int64_t groups_cap, float *kdeq, float *vdeq)
{
    int64_t ng = L / OQ_G;
    int64_t rb = oq_record_bytes(kb, vb);
    int64_t vc_off = 512 * (int64_t)kb;
    int64_t km_off = vc_off + 512 * (int64_t)vb;
    int64_t vm_off = km_off + (kb < 16 ? 1024 : 0);
    for (int64_t j = 0; j < L; ++j) {
        int64_t m = j / OQ_G;
        int s = (int)(j % OQ_G);
        const uint8_t *rec = (m < ng) ? bytes + m * rb : bytes + groups_cap * rb;
        int kbits = (m < ng) ? kb : 16, vbits = (m < ng) ? vb : 16;
        int64_t voff = (m < ng) ? vc_off : 8192;
        for (int c = 0; c < OQ_D; ++c) {
            int lane, e;
            float f;
            oq_k_site(s, c, &lane, &e);
            uint32_t kc = oq_get(rec, lane, e, kbits);
            if (kbits == 16) {
                kdeq[j * OQ_D + c] = oq_half_to_float((uint16_t)kc);
            } else {
                int ix = kaxis_token ? oq_meta_token_index(s, c / OQ_G) : oq_meta_channel_index(c);
                float sc, zr;
                memcpy(&sc, rec + km_off + 4 * ix, 4);
                memcpy(&zr, rec + km_off + 4 * (128 + ix), 4);
                kdeq[j * OQ_D + c] = oq_dequant(kc, sc, zr);
            }
            oq_v_site(s, c, &lane, &e);
            uint32_t vcd = oq_get(rec + voff, lane, e, vbits);
            if (vbits == 16) {
                f = oq_half_to_float((uint16_t)vcd);
            } else {
                int ix = oq_meta_token_index(s, c / OQ_G);
                float sc, zr;
                memcpy(&sc, rec + vm_off + 4 * ix, 4);
                memcpy(&zr, rec + vm_off + 4 * (128 + ix), 4);
                f = oq_dequant(vcd, sc, zr);
            }
            vdeq[j * OQ_D + c] = f;
        }
    }
}

/* ---------------------------------------------------------- paged pool -- */
/*
 * The paged pool of one layer (TriAxialKV page, "Facts": INT2 and INT4 page
 * pools share one address space split at an offset; INT2 keys per-channel
 * and values per-token, INT4 keys and values per-token; INT2 tokens that do
 * not fill a 32-token group go to the INT4 per-token path; each request's
 * page table lists its INT2 pages before its INT4 pages). A page holds 16
 * tokens of every KV head. Page ids below int2_pages are INT2 pages, the
 * rest INT4 pages.
 *  - INT2 region at byte 0, int2_page_bytes = hkv * 2048 per page. A 32-token
 *    group needs an aligned pair of pages (P even, P + 1): the pair holds one
 *    K2V2 group record (layout above, keys per-channel) per KV head, head h
 *    at P * int2_page_bytes + h * 4096.
 *  - INT4 region at int4_offset = int2_pages * int2_page_bytes,
 *    int4_page_bytes = hkv * 3072 per page; page P, head h at
 *    int4_offset + (P - int2_pages) * int4_page_bytes + h * 3072:
 *      [K codes 1024 B][V codes 1024 B][K meta 512 B][V meta 512 B]
 *    for token slots p = 0..15, 4-bit codes, lane word w at lane * 16 + w * 4:
 *      K (p, c): lane 16*((c/8)%4) + p, word c/32, position c%8 of the word
 *                (even positions in bits 0..15, odd in 16..31, 4 bits each)
 *      V (p, c): lane 16*(p/4) + c%16, word (c/16)/2,
 *                bit 8*((c/16)%2) + 4*((p%4)/2) + 16*(p%2)
 *      meta: 64 fp32 scales then 64 fp32 zeros, index 16*(c/32) + p.
 * A request's table holds n2/16 INT2 entries (entry 2i = the even id of
 * the pair of INT2 group i; entry 2i+1 = that id + 1) then ceil(n4/16) INT4
 * entries (entry n2/16 + t/16 holds INT4 token t in slot t % 16). Its
 * logical token list is the n2 INT2 tokens, then the n4 INT4 tokens.
 */

void oq_page_k_site(int p, int c, int *byte, int *shift)
{
    int lane = 16 * ((c / 8) % 4) + p;
    int pos = c % 8;
    *byte = lane * 16 + (c / 32) * 4;
    *shift = 16 * (pos % 2) + 4 * (pos / 2);
}

void oq_page_v_site(int p, int c, int *byte, int *shift)
{
    int lane = 16 * (p / 4) + c % 16;
    int u = c / 16;
    *byte = 1024 + lane * 16 + (u / 2) * 4;
    *shift = 8 * (u % 2) + 4 * ((p % 4) / 2) + 16 * (p % 2);
}

int oq_page_meta_index(int p, int n) { return 16 * n + p; }

static void oq_put4(uint8_t *page, int byte, int shift, uint32_t code, uint8_t *mask)
{
    uint32_t w;
    memcpy(&w, page + byte, 4);
    w = (w & ~(0xFu << shift)) | ((code & 0xFu) << shift);
    memcpy(page + byte, &w, 4);
    if (mask) mask[byte + shift / 8] = 1;
}

static uint32_t oq_get4(const uint8_t *page, int byte, int shift)
{
    uint32_t w;
    memcpy(&w, page + byte, 4);
    return (w >> shift) & 0xFu;
}

/* Per-token quantization of L tokens (any L), each token in four 32-channel
 * groups: code [L][128], scale/zero [L][4]. */
void oq_quantize_tokens(const uint16_t *x, int64_t L, int bits, uint8_t *code, float *scale,
                        float *zero)
{
    for (int64_t j = 0; j < L; ++j)
        for (int n = 0; n < OQ_D / OQ_G; ++n)
            oq_quantize_group(x + j * OQ_D + n * OQ_G, 1, OQ_G, bits, &scale[j * 4 + n],
                              &zero[j * 4 + n], code + j * OQ_D + n * OQ_G);
}

static int64_t oq_int2_record_at(int32_t pair_page, int hkv, int h)
{
    return (int64_t)pair_page * hkv * 2048 + (int64_t)h * 4096;
}

static int64_t oq_int4_page_at(int32_t page, int32_t int2_pages, int hkv, int h)
{
    return (int64_t)int2_pages * hkv * 2048 + (int64_t)(page - int2_pages) * hkv * 3072 +
           (int64_t)h * 3072;
}

/*
 * Quantize and place the tokens of one (request, KV head) into the pool:
 * k, v fp16 [n2 + n4][128] in logical order (n2 a multiple of 32). mask, if
 * not NULL, gets 1 on every byte the call defines.
 */
void oq_pack_paged(const uint16_t *k, const uint16_t *v, int64_t n2, int64_t n4,
                   const int32_t *table, int32_t int2_pages, int hkv, int h, uint8_t *pool,
                   uint8_t *mask)
{
    /* INT2 groups: the K2V2 per-channel record of a 32-token group */
    uint8_t kc[OQ_G * OQ_D], vc[OQ_G * OQ_D];
    float ks[OQ_D], kz[OQ_D], vs[OQ_G * 4], vz[OQ_G * 4];
    for (int64_t m = 0; m < n2 / OQ_G; ++m) {
        const uint16_t *kg = k + m * OQ_G * OQ_D, *vg = v + m * OQ_G * OQ_D;
        oq_quantize_stream(kg, vg, OQ_G, 2, 2, 0, kc, ks, kz, vc, vs, vz);
        int64_t at = oq_int2_record_at(table[2 * m], hkv, h);
        oq_pack_stream(kg, vg, OQ_G, 2, 2, 0, 0, kc, ks, kz, vc, vs, vz, pool + at,
                       mask ? mask + at : NULL);
    }
    /* INT4 tokens: per-token keys and values, one page slot each */
    uint8_t ck[OQ_D], cv[OQ_D];
    float sk[4], zk[4], sv[4], zv[4];
    for (int64_t t = 0; t < n4; ++t) {
        const uint16_t *kt = k + (n2 + t) * OQ_D, *vt = v + (n2 + t) * OQ_D;
        oq_quantize_tokens(kt, 1, 4, ck, sk, zk);
        oq_quantize_tokens(vt, 1, 4, cv, sv, zv);
        int64_t at = oq_int4_page_at(table[n2 / 16 + t / 16], int2_pages, hkv, h);
        uint8_t *page = pool + at;
        uint8_t *pm = mask ? mask + at : NULL;
        int p = (int)(t % 16);
        for (int c = 0; c < OQ_D; ++c) {
            int b, sh;
            oq_page_k_site(p, c, &b, &sh);
            oq_put4(page, b, sh, ck[c], pm);
            oq_page_v_site(p, c, &b, &sh);
            oq_put4(page, b, sh, cv[c], pm);
        }
        for (int n = 0; n < 4; ++n) {
            int ix = oq_page_meta_index(p, n);
            oq_put_f32(page + 2048, ix, sk[n], pm ? pm + 2048 : NULL);
            oq_put_f32(page + 2048, 64 + ix, zk[n], pm ? pm + 2048 : NULL);
            oq_put_f32(page + 2560, ix, sv[n], pm ? pm + 2560 : NULL);
            oq_put_f32(page + 2560, 64 + ix, zv[n], pm ? pm + 2560 : NULL);
        }
    }
}

/* Read one (request, KV head) back from the pool, dequantized, float
 * [n2 + n4][128] each, in logical order. */
void oq_unpack_paged(const uint8_t *pool, int64_t n2, int64_t n4, const int32_t *table,
                     int32_t int2_pages, int hkv, int h, float *kdeq, float *vdeq)
{
    for (int64_t m = 0; m < n2 / OQ_G; ++m)
        oq_unpack_stream(pool + oq_int2_record_at(table[2 * m], hkv, h), OQ_G, 2, 2, 0, 1,
                         kdeq + m * OQ_G * OQ_D, vdeq + m * OQ_G * OQ_D);
    for (int64_t t = 0; t < n4; ++t) {
        const uint8_t *page = pool + oq_int4_page_at(table[n2 / 16 + t / 16], int2_pages, hkv, h);
        int p = (int)(t % 16);
        float *ko = kdeq + (n2 + t) * OQ_D, *vo = vdeq + (n2 + t) * OQ_D;
        for (int c = 0; c < OQ_D; ++c) {
            int b, sh, ix = oq_page_meta_index(p, c / OQ_G);
            float s, z;
            oq_page_k_site(p, c, &b, &sh);
            memcpy(&s, page + 2048 + 4 * ix, 4);
            memcpy(&z, page + 2048 + 4 * (64 + ix), 4);
            ko[c] = oq_dequant(oq_get4(page, b, sh), s, z);
            oq_page_v_site(p, c, &b, &sh);
            memcpy(&s, page + 2560 + 4 * ix, 4);
            memcpy(&z, page + 2560 + 4 * (64 + ix), 4);
            vo[c] = oq_dequant(oq_get4(page, b, sh), s, z);
        }
    }
}

/* ----------------------------------------------------------- attention -- */

/*
 * Softmax attention, fp64, of G query rows q (fp16 [G][D]) over L cached
 * tokens (float [L][D] each):
 *   s_j = scale * sum_c q_c k_jc ; m = max_j s_j ; l = sum_j exp(s_j - m)
 *   out_c = sum_j exp(s_j - m) v_jc / l ; lse = m + log(l)
 * L == 0 gives out = 0 and lse = -inf.
 */
void oq_attention(const uint16_t *q, int G, int D, const float *kd, const float *vd,
                  int64_t L, double scale, double *out, double *lse)
{
    double *s = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    for (int g = 0; g < G; ++g) {
        double *o = out + (int64_t)g * D;
        for (int c = 0; c < D; ++c) o[c] = 0.0;
        if (L == 0) {
            lse[g] = -INFINITY;
            continue;
        }
        double m = -INFINITY;
        for (int64_t j = 0; j < L; ++j) {
            double acc = 0.0;
            for (int c = 0; c < D; ++c)
                acc += (double)oq_half_to_float(q[(int64_t)g * D + c]) * (double)kd[j * D + c];
            s[j] = acc * scale;
            if (s[j] > m) m = s[j];
        }
        double l = 0.0;
        for (int64_t j = 0; j < L; ++j) {
            double p = exp(s[j] - m);
            l += p;
            for (int c = 0; c < D; ++c) o[c] += p * (double)vd[j * D + c];
        }
        for (int c = 0; c < D; ++c) o[c] /= l;
        lse[g] = m + log(l);
    }
    free(s);
}

/*
 * Merge S partial results (each normalised over its own tokens, with its own
 * log-sum-exp) into one: M = max lse_s, w_s = exp(lse_s - M),
 * out = sum w_s o_s / sum w_s, lse = M + log(sum w_s). Partials with
 * lse = -inf (no tokens) get weight 0.
 */
void oq_lse_merge(const double *o, const double *lse, int S, int D, double *out, double *out_lse)
{
    double M = -INFINITY;
    for (int s = 0; s < S; ++s)
        if (lse[s] > M) M = lse[s];
    for (int c = 0; c < D; ++c) out[c] = 0.0;
    if (M == -INFINITY) {
        *out_lse = -INFINITY;
        return;
    }
    double wsum = 0.0;
    for (int s = 0; s < S; ++s) {
        if (lse[s] == -INFINITY) continue;
        double w = exp(lse[s] - M);
        wsum += w;
        for (int c = 0; c < D; ++c) out[c] += w * o[(int64_t)s * D + c];
    }
    for (int c = 0; c < D; ++c) out[c] /= wsum;
    *out_lse = M + log(wsum);
}

/*
 * One decode step of one layer from the oracle's own packed cache: for each
 * listed stream, unpack + dequantize its L tokens, then fp64 attention of its
 * G query rows. Streams are independent; they are spread over `nthreads`
 * OpenMP threads (0 = the runtime's default). Returns the thread count used.
 *   cache: layer base; stream s lives at cache + stream_ids[s] * stream_stride
 *   q: fp16 [n_streams][G][128]; out: [n_streams][G][128]; lse: [n_streams][G]
 */
int oq_decode_packed(const uint8_t *cache, int64_t stream_stride, int n_streams,
                     const int64_t *stream_ids, const int64_t *lens, int kb, int vb,
                     int kaxis_token, int64_t groups_cap, const uint16_t *q, int G,
                     double scale, double *out, double *lse, int nthreads)
{
    int used = 1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
    {
#pragma omp single
        used = omp_get_num_threads();
    }
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int s = 0; s < n_streams; ++s) {
        int64_t L = lens[s];
        float *kd = (float *)malloc(sizeof(float) * (size_t)(L > 0 ? L : 1) * OQ_D);
        float *vd = (float *)malloc(sizeof(float) * (size_t)(L > 0 ? L : 1) * OQ_D);
        oq_unpack_stream(cache + stream_ids[s] * stream_stride, L, kb, vb, kaxis_token,
                         groups_cap, kd, vd);
        oq_attention(q + (int64_t)s * G * OQ_D, G, OQ_D, kd, vd, L, scale,
                     out + (int64_t)s * G * OQ_D, lse + (int64_t)s * G);
        free(kd);
        free(vd);
    }
    return used;
}

/*
 * One decode step of one layer from the oracle's own paged pool: for each
 * listed (request, KV head), unpack its INT2 and INT4 tokens, then fp64
 * attention of its G query rows. Returns the thread count used.
 *   tables: int32 [n_req][max_pages]; req/head/n2/n4: per stream
 *   q: fp16 [n_streams][G][128]; out: [n_streams][G][128]; lse: [n_streams][G]
 */
int oq_decode_paged(const uint8_t *pool, int n_streams, const int64_t *req, const int64_t *head,
                    const int64_t *n2, const int64_t *n4, const int32_t *tables, int64_t max_pages,
                    int32_t int2_pages, int hkv, const uint16_t *q, int G, double scale,
                    double *out, double *lse, int nthreads)
{
    int used = 1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
    {
#pragma omp single
        used = omp_get_num_threads();
    }
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int s = 0; s < n_streams; ++s) {
        int64_t L = n2[s] + n4[s];
        float *kd = (float *)malloc(sizeof(float) * (size_t)(L > 0 ? L : 1) * OQ_D);
        float *vd = (float *)malloc(sizeof(float) * (size_t)(L > 0 ? L : 1) * OQ_D);
        oq_unpack_paged(pool, n2[s], n4[s], tables + req[s] * max_pages, int2_pages, hkv,
                        (int)head[s], kd, vd);
        oq_attention(q + (int64_t)s * G * OQ_D, G, OQ_D, kd, vd, L, scale,
                     out + (int64_t)s * G * OQ_D, lse + (int64_t)s * G);
        free(kd);
        free(vd);
    }
    return used;
}
