// kvq_internal.h -- device-side layout helpers and launch interfaces shared by
// the HIP translation units of libkvq. Not part of the public ABI.
//
// Cache layout (this library's own; no page prescribes one). A 32-token group
// of one (layer, request, KV head) stream is one record:
//   [K codes 512*bK B][V codes 512*bV B][K meta 1 KiB if bK<16][V meta 1 KiB if bV<16]
// A code block is 64 lanes x (8*b bytes); lane word w sits at byte
// (w/4)*1024 + lane*16 + (w%4)*4, so word w of all 64 lanes is one coalesced
// 1 KiB row and a lane's words 4k..4k+3 are one 16-byte load. Inside a word,
// even code positions fill bits 0..15 and odd positions bits 16..31, so that
// a pair of consecutive positions unpacks to the two halves of a register.
// Lane/position of token j (0..31) and channel c (0..127):
//   K: lane 16*((c/8)%4) + j%16, position 32*(j/16) + 8*(c/32) + c%8
//   V: lane 16*((j%16)/4) + c%16, position 8*(c/16) + 4*(j/16) + j%4
// which are the operand layouts of a 16x16x32 f16 MFMA with tokens as rows of
// the score tile (K) and tokens as the reduction index of the P.V tile (V).
// Meta: 128 fp32 scales then 128 fp32 zeros, per-channel index
// 32*((c/8)%4) + 8*(c/32) + c%8, per-token index 32*n + kappa(j),
// kappa(j) = 8*((j%16)/4) + 4*(j/16) + j%4.
// A stream is groups_cap records then one tail record in the K16V16 format.
//
// Paged pool (TriAxialKV page, "Facts": INT2 and INT4 page pools in one
// address space split at an offset; INT4 keys and values per-token). Pages
// hold 16 tokens of every KV head; ids below int2_pages are INT2 pages.
//   INT2: an aligned page pair (P even, P + 1) holds one K2V2 record (keys
//         per-channel) per KV head, head h at P * int2_page_bytes + h * 4096.
//   INT4: page P, head h at int4_offset + (P - int2_pages) * int4_page_bytes
//         + h * 3072: [K codes 1 KiB][V codes 1 KiB][K meta 512][V meta 512]
//         for slots p = 0..15, 4-bit codes, lane word w at lane * 16 + w * 4.
//         K (p, c): lane 16*((c/8)%4) + p, word c/32, position c%8 (the
//         token half of a K4V4 record's key block); V (p, c): lane
//         16*(p/4) + c%16, word (c/16)/2, bit 8*((c/16)%2) + 4*((p%4)/2) +
//         16*(p%2), so that two pages' words interleave bytewise into the V
//         words of a 32-token record. Meta: 64 scales then 64 zeros, index
//         16*(c/32) + p.
// A request's page table lists its INT2 pairs (entry 2i = even id of group i)
// and then its INT4 pages (entry int2_len/16 + t/16 holds INT4 token t).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int D = 128;
constexpr int GS = 32;
constexpr int TAIL_BYTES = 16384;
constexpr int META_BYTES = 1024;

__host__ __device__ inline uint32_t word_offset(int lane, int w) {
  return (uint32_t)(w >> 2) * 1024u + (uint32_t)lane * 16u + (uint32_t)(w & 3) * 4u;
}

// byte offset of the word holding position e of `lane`, and the bit shift
__host__ __device__ inline void code_site(int lane, int e, int bits, uint32_t* off, int* shift) {
  const int per_word = 32 / bits;
  const int w = e / per_word;
  const int p = e - w * per_word;
  *off = word_offset(lane, w);
  *shift = (p & 1) * 16 + (p >> 1) * bits;
}

__host__ __device__ inline void k_site(int j, int c, int* lane, int* e) {
  *lane = 16 * ((c >> 3) & 3) + (j & 15);
  *e = 32 * (j >> 4) + 8 * (c >> 5) + (c & 7);
}

__host__ __device__ inline void v_site(int j, int c, int* lane, int* e) {
  *lane = 16 * ((j & 15) >> 2) + (c & 15);
  *e = 8 * (c >> 4) + 4 * (j >> 4) + (j & 3);
}

// inverse maps: (lane, position) -> (token, channel)
__host__ __device__ inline void k_inverse(int lane, int e, int* j, int* c) {
  const int a = lane >> 4, r = lane & 15;
  *j = 16 * (e >> 5) + r;
  *c = 32 * ((e >> 3) & 3) + 8 * a + (e & 7);
}

__host__ __device__ inline void v_inverse(int lane, int e, int* j, int* c) {
  const int a = lane >> 4, r = lane & 15;
  const int ip = e & 7;
  *c = 16 * (e >> 3) + r;
  *j = 16 * (ip >> 2) + 4 * a + (ip & 3);
}

__host__ __device__ inline int meta_channel(int c) { return 32 * ((c >> 3) & 3) + 8 * (c >> 5) + (c & 7); }

__host__ __device__ inline int kappa(int j) { return 8 * ((j & 15) >> 2) + 4 * (j >> 4) + (j & 3); }

__host__ __device__ inline int meta_token(int j, int n) { return 32 * n + kappa(j); }

__host__ __device__ inline uint32_t record_bytes(int kb, int vb) {
  return 512u * kb + 512u * vb + (kb < 16 ? META_BYTES : 0) + (vb < 16 ? META_BYTES : 0);
}

// byte offsets of the four parts of a record
struct RecordParts {
  uint32_t vcode, kmeta, vmeta;
};

__host__ __device__ inline RecordParts record_parts(int kb, int vb) {
  RecordParts p;
  p.vcode = 512u * kb;
  p.kmeta = p.vcode + 512u * vb;
  p.vmeta = p.kmeta + (kb < 16 ? META_BYTES : 0);
  return p;
}

constexpr int PAGE_TOKENS = 16;
constexpr int INT2_RECORD = 4096;  // K2V2 record of one KV head in a page pair
constexpr int INT4_HEAD = 3072;    // one KV head's share of an INT4 page
constexpr int INT4_VCODE = 1024, INT4_KMETA = 2048, INT4_VMETA = 2560;

__host__ __device__ inline uint32_t page_k_offset(int p, int c, int* shift) {
  const int pos = c & 7;
  *shift = 16 * (pos & 1) + 4 * (pos >> 1);
  return (uint32_t)(16 * ((c >> 3) & 3) + p) * 16u + (uint32_t)(c >> 5) * 4u;
}

__host__ __device__ inline uint32_t page_v_offset(int p, int c, int* shift) {
  const int u = c >> 4;
  *shift = 8 * (u & 1) + 4 * ((p & 3) >> 1) + 16 * (p & 1);
  return INT4_VCODE + (uint32_t)(16 * (p >> 2) + (c & 15)) * 16u + (uint32_t)(u >> 1) * 4u;
}

// ------------------------------------------------------------ launch args

// Paged-pool view of one layer (all pointers device, caller-owned).
struct PagedGeom {
  const int32_t* table;     // [batch][max_pages]; null = contiguous mode
  const int32_t* int2_len;  // [batch]
  const int32_t* int4_len;  // [batch]
  const int32_t* int2_add;  // append: [batch] or null (= 0)
  int max_pages;
  int int2_pages;
  int int4_pages;
  uint64_t int4_offset;
  uint64_t int2_page_bytes;
  uint64_t int4_page_bytes;
};

struct LayerGeom {
  uint8_t* base;          // layer region
  uint64_t stream_bytes;  // per (request, KV head)
  uint64_t record_bytes;
  uint64_t tail_offset;
  int groups_cap;
  int kb, vb, k_token;
  int hkv, hq, g;
  int max_tokens;
};

// Page ids a write may use (the kernels check them before writing, so a bad
// table never sends a write outside the layer's pool): an INT2 pair needs an
// even id P with P + 1 < int2_pages, an INT4 page an id in [int2_pages,
// int2_pages + int4_pages), and both a table entry below max_pages.
__device__ inline bool int2_pair_ok(const PagedGeom& pg, int entry, int id) {
  return entry >= 0 && entry + 1 < pg.max_pages && id >= 0 && (id & 1) == 0 && id + 1 < pg.int2_pages;
}
__device__ inline bool int4_page_ok(const PagedGeom& pg, int entry, int id) {
  return entry >= 0 && entry < pg.max_pages && id >= pg.int2_pages && id < pg.int2_pages + pg.int4_pages;
}

struct AppendArgs {
  LayerGeom geo;
  PagedGeom pg;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int32_t* seq_lens;
  int n_new;
};

struct DequantArgs {
  LayerGeom geo;
  PagedGeom pg;
  const int32_t* seq_lens;
  int max_seq_len;
  float* k_out;
  float* v_out;
};

struct DecodeArgs {
  LayerGeom geo;
  PagedGeom pg;
  const uint16_t* q;
  const int32_t* seq_lens;
  int splits;
  int groups_per_split;  // virtual groups (32 tokens; the tail counts as one)
  float scale_log2;      // softmax_scale * log2(e)
  float* part_o;         // [batch][Hq][splits][128]
  float* part_lse;       // [batch][Hq][splits]  natural log
  void* out;             // with one split the split pass writes the final output ...
  int out_f32;
  float* lse_out;        // ... and log-sum-exp (nullable)
  // Fused append of one token per request (contiguous streams): k_new/v_new
  // fp16 [batch][hkv][128]; seq_lens then count the tokens before it. Null:
  // a plain decode.
  const uint16_t* k_new = nullptr;
  const uint16_t* v_new = nullptr;
  // Prefix attention: q holds `chunk` tokens a request, [batch][chunk][Hq][128],
  // and the rows of out (fp32), lse and the partials follow that order.
  int chunk = 0;
  // Partials per row in the workspace (0 = splits). A chunked-prefill call
  // keeps one more for the chunk's own causal part (partial index `splits`),
  // so that the merge pass joins the prefix splits and the chunk part.
  int part_stride = 0;
  // Chunked prefill: the chunk's own fp16 keys and values, [batch][hkv][chunk][128].
  const uint16_t* k_chunk = nullptr;
  const uint16_t* v_chunk = nullptr;
};

struct MergeArgs {
  const float* part_o;
  const float* part_lse;
  int splits;
  int rows;  // output rows (batch * Hq; prefix attention: batch * chunk * Hq)
  void* out;
  int out_f32;
  float* lse_out;
};

// Launches. When `ev` is given, its two events are bound to the kernel's own
// dispatch (start and end of the kernel), for the optional timer.
struct EventPair {
  hipEvent_t start = nullptr, stop = nullptr;
};

hipError_t launch_append(const AppendArgs& a, int batch, hipStream_t s, const EventPair* ev);
hipError_t launch_dequant(const DequantArgs& a, int batch, hipStream_t s);
hipError_t launch_decode_split_mfma(const DecodeArgs& a, int batch, hipStream_t s, const EventPair* ev);
hipError_t launch_decode_paged(const DecodeArgs& a, int batch, hipStream_t s, const EventPair* ev);
hipError_t launch_prefix(const DecodeArgs& a, int batch, hipStream_t s, const EventPair* ev);
hipError_t launch_chunk_causal(const DecodeArgs& a, int batch, hipStream_t s, const EventPair* ev);
int prefix_rows_per_block();  // query rows one prefix-attention workgroup takes
hipError_t launch_append_paged(const AppendArgs& a, int batch, hipStream_t s, const EventPair* ev);
hipError_t launch_dequant_paged(const DequantArgs& a, int batch, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s, const EventPair* ev);

// Record the message kvq_last_error() returns on this thread, and return code
// (for entry points defined outside kvq_api.cpp).
int set_error(int code, const char* msg);

// kernel launch with optional dispatch-bound events
template <typename K, typename A>
inline hipError_t launch_timed(K kernel, dim3 grid, dim3 block, hipStream_t s, const EventPair* ev, const A& args) {
  if (ev && ev->start)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev->start, ev->stop, 0, args);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args);
  return hipGetLastError();
}

}  // namespace kvq
