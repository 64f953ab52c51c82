// kvq_api.cpp -- host side of libkvq: the layer planner, argument checks,
// launches, the error string and the optional kernel timer. Every function of
// include/kvq.h is defined here; the kernels live in the .hip files.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kvq.h"
#include "kvq_internal.h"

namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int ok() {
  g_error.clear();
  return KVQ_OK;
}

bool valid_bits(int b) { return b == 2 || b == 4 || b == 8 || b == 16; }

uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------- timer

// 0 = append, 1 = decode split pass, 2 = merge pass, 3 = prefix split pass
constexpr int kTimerKinds = 4;

struct Timer {
  std::mutex mu;
  bool armed = false;
  int capacity = 0;
  std::vector<hipEvent_t> ev[kTimerKinds][2];
  int used[kTimerKinds] = {};
} g_timer;

void timer_free_locked() {
  for (int k = 0; k < kTimerKinds; ++k)
    for (int i = 0; i < 2; ++i) {
      for (hipEvent_t e : g_timer.ev[k][i]) (void)hipEventDestroy(e);
      g_timer.ev[k][i].clear();
    }
  g_timer.armed = false;
  g_timer.capacity = 0;
  for (int k = 0; k < kTimerKinds; ++k) g_timer.used[k] = 0;
}

// Event pair for the next launch of `kind` if the timer is armed and has room.
bool timer_slot(int kind, kvq::EventPair* ev) {
  std::lock_guard<std::mutex> lk(g_timer.mu);
  if (!g_timer.armed || g_timer.used[kind] >= g_timer.capacity) return false;
  const int slot = g_timer.used[kind]++;
  ev->start = g_timer.ev[kind][0][slot];
  ev->stop = g_timer.ev[kind][1][slot];
  return true;
}

// ----------------------------------------------------------- arguments

// The kernels read the cache, the new tokens and q in 16-byte pieces.
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_plan_layer(const kvq_plan* plan, int32_t layer) {
  if (!plan) return fail(KVQ_ERR_INVALID_ARG, "plan is NULL");
  if (plan->num_layers < 1 || plan->num_layers > KVQ_MAX_LAYERS)
    return fail(KVQ_ERR_INVALID_ARG, "plan has %d layers (not planned?)", plan->num_layers);
  if (layer < 0 || layer >= plan->num_layers)
    return fail(KVQ_ERR_INVALID_ARG, "layer %d out of range [0, %d)", layer, plan->num_layers);
  return KVQ_OK;
}

kvq::LayerGeom geom(const kvq_plan* plan, int32_t layer, const void* cache) {
  const kvq_layer_plan& lp = plan->layers[layer];
  kvq::LayerGeom g;
  g.base = (uint8_t*)cache + lp.offset;
  g.stream_bytes = lp.stream_bytes;
  g.record_bytes = lp.record_bytes;
  g.tail_offset = lp.tail_offset;
  g.groups_cap = (int)lp.groups_cap;
  g.kb = lp.k_bits;
  g.vb = lp.v_bits;
  g.k_token = lp.k_axis == KVQ_AXIS_TOKEN;
  g.hkv = plan->shape.num_kv_heads;
  g.hq = plan->shape.num_q_heads;
  g.g = g.hq / g.hkv;
  g.max_tokens = plan->shape.max_tokens;
  return g;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool is_paged(const kvq_plan* plan) { return plan->shape.page_tokens != 0; }

// Paged-pool view for the kernels; all zero in contiguous mode.
kvq::PagedGeom paged_geom(const kvq_plan* plan, int32_t layer, const kvq_pages* pages) {
  kvq::PagedGeom pg;
  std::memset(&pg, 0, sizeof pg);
  if (!pages) return pg;
  const kvq_layer_plan& lp = plan->layers[layer];
  pg.table = pages->page_table;
  pg.int2_len = pages->int2_len;
  pg.int4_len = pages->int4_len;
  pg.int2_add = pages->int2_add;
  pg.max_pages = pages->max_pages_per_req;
  pg.int2_pages = plan->shape.int2_pages;
  pg.int4_pages = plan->shape.int4_pages;
  pg.int4_offset = lp.int4_offset;
  pg.int2_page_bytes = lp.int2_page_bytes;
  pg.int4_page_bytes = lp.int4_page_bytes;
  return pg;
}

// pages must be given exactly for a paged plan, with its device arrays
int check_pages(const kvq_plan* plan, const kvq_pages* pages) {
  if (!is_paged(plan)) {
    if (pages) return fail(KVQ_ERR_INVALID_ARG, "pages given for a contiguous plan");
    return KVQ_OK;
  }
  if (!pages) return fail(KVQ_ERR_INVALID_ARG, "a paged plan needs pages");
  if (!pages->page_table || !pages->int2_len || !pages->int4_len)
    return fail(KVQ_ERR_INVALID_ARG, "pages: null page_table, int2_len or int4_len");
  if (pages->max_pages_per_req <= 0)
    return fail(KVQ_ERR_INVALID_ARG, "pages: max_pages_per_req %d", pages->max_pages_per_req);
  return KVQ_OK;
}

// Token capacity of one request.
int64_t capacity_tokens(const kvq_plan* plan, const kvq_pages* pages) {
  return is_paged(plan) ? (int64_t)pages->max_pages_per_req * kvq::PAGE_TOKENS : plan->shape.max_tokens;
}

// A paged split walks at most 256 complete groups (64 per wave).
constexpr int64_t kPagedMaxGroupsPerSplit = 256;

int32_t auto_splits(const kvq_plan* plan, int32_t batch, int32_t max_seq_len) {
  const int64_t streams = (int64_t)batch * plan->shape.num_kv_heads;
  const int64_t nvg = (max_seq_len + kvq::GS - 1) / kvq::GS;
  if (nvg <= 0 || streams <= 0) return 1;
  if (is_paged(plan)) {
    // one kind per split, so ceil(nvg / gps) + 1 splits cover a request's
    // INT2 groups and its INT4 page pairs together (gps = ceil(nvg / (splits
    // - 1)) <= 256). Aim for ~1024 workgroups, two full rounds at two per CU:
    // INT4 splits carry 1.5x the bytes of INT2 ones, and a second round lets
    // the CUs that drew INT2 splits take more work (one round of 512, or a
    // round and a half, measured 15-25% slower).
    int64_t s = (1024 + streams - 1) / streams;
    const int64_t s_min = (nvg + kPagedMaxGroupsPerSplit - 1) / kPagedMaxGroupsPerSplit + 1;
    if (s < s_min) s = s_min;
    if (s > nvg + 1) s = nvg + 1;
    return (int32_t)(s > 1024 ? 1024 : s);
  }
  // 4-wave workgroups: aim for ~512 of them (2 per CU on 256 CUs), but keep
  // at least 8 groups (2 per wave) in each split
  int64_t s = (512 + streams - 1) / streams;
  const int64_t max_s = nvg / 8 > 1 ? nvg / 8 : 1;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  if (s > 1024) s = 1024;
  return (int32_t)s;
}

// Groups per split for `splits` splits of max_seq_len tokens. A paged pool
// gives a request's INT2 and INT4 parts splits of their own, so it needs one
// split more and at most kPagedMaxGroupsPerSplit groups a split.
int split_groups(const kvq_pages* pages, int32_t splits, int32_t max_seq_len, int32_t* gps) {
  const int32_t nvg = (max_seq_len + kvq::GS - 1) / kvq::GS;
  if (!pages) {
    *gps = nvg > 0 ? (nvg + splits - 1) / splits : 0;
    return KVQ_OK;
  }
  if (nvg == 0) {
    *gps = 1;  // no tokens anywhere; the kernels divide by gps
    return KVQ_OK;
  }
  if (splits < 2) return fail(KVQ_ERR_INVALID_ARG, "a paged decode needs at least 2 splits");
  *gps = (nvg + splits - 2) / (splits - 1);
  if (*gps > kPagedMaxGroupsPerSplit)
    return fail(KVQ_ERR_INVALID_ARG, "num_splits %d too small: a paged split walks at most %lld groups", splits,
                (long long)kPagedMaxGroupsPerSplit);
  return KVQ_OK;
}

// Prefix attention: the row blocks already give batch * Hkv * blocks
// workgroups (8 waves, one per CU); split the prefix only while that is
// under one round of 256, keeping at least 8 groups in each split (a second
// round, or more splits, measured slower once the merge is counted).
int64_t prefix_blocks(const kvq_plan* plan, int32_t chunk) {
  const int64_t rows = (int64_t)chunk * (plan->shape.num_q_heads / plan->shape.num_kv_heads);
  return (rows + kvq::prefix_rows_per_block() - 1) / kvq::prefix_rows_per_block();
}

int32_t prefix_splits(const kvq_plan* plan, int32_t batch, int32_t chunk, int32_t max_seq_len) {
  const int64_t wgs = (int64_t)batch * plan->shape.num_kv_heads * prefix_blocks(plan, chunk);
  const int64_t nvg = (max_seq_len + kvq::GS - 1) / kvq::GS;
  if (nvg <= 0 || wgs <= 0) return 1;
  int64_t s = (256 + wgs - 1) / wgs;
  const int64_t max_s = nvg / 8 > 1 ? nvg / 8 : 1;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  return (int32_t)s;
}

}  // namespace

int kvq::set_error(int code, const char* msg) {
  g_error = msg;
  return code;
}

extern "C" {

const char* kvq_last_error(void) { return g_error.c_str(); }

int kvq_plan_layers(const kvq_shape* shape, const kvq_layer_cfg* cfg, int32_t num_layers, kvq_plan* out) {
  if (!shape || !cfg || !out) return fail(KVQ_ERR_INVALID_ARG, "null argument");
  if (num_layers < 1 || num_layers > KVQ_MAX_LAYERS)
    return fail(KVQ_ERR_INVALID_ARG, "num_layers %d out of range [1, %d]", num_layers, KVQ_MAX_LAYERS);
  const kvq_shape& s = *shape;
  if (s.head_dim != KVQ_HEAD_DIM) return fail(KVQ_ERR_UNSUPPORTED, "head_dim %d (only 128)", s.head_dim);
  if (s.group_size != KVQ_GROUP) return fail(KVQ_ERR_UNSUPPORTED, "group_size %d (only 32)", s.group_size);
  if (s.num_q_heads <= 0 || s.num_kv_heads <= 0 || s.max_batch <= 0)
    return fail(KVQ_ERR_INVALID_ARG, "heads and max_batch must be positive");
  if (s.num_q_heads % s.num_kv_heads != 0)
    return fail(KVQ_ERR_UNSUPPORTED, "num_q_heads %d is not a multiple of num_kv_heads %d", s.num_q_heads,
                s.num_kv_heads);
  if (s.num_q_heads / s.num_kv_heads > 16)
    return fail(KVQ_ERR_UNSUPPORTED, "GQA group %d > 16", s.num_q_heads / s.num_kv_heads);
  if (s.page_tokens != 0 && s.page_tokens != 16)
    return fail(KVQ_ERR_UNSUPPORTED, "page_tokens %d (0 or 16)", s.page_tokens);
  const bool paged = s.page_tokens == 16;
  if (!paged && s.max_tokens <= 0) return fail(KVQ_ERR_INVALID_ARG, "max_tokens must be positive");
  if (paged) {
    if (s.int2_pages < 0 || s.int4_pages < 0 || (s.int2_pages & 1) || s.int2_pages + s.int4_pages <= 0)
      return fail(KVQ_ERR_INVALID_ARG, "paged pool needs an even int2_pages >= 0 and int4_pages >= 0");
  }
  for (int l = 0; l < num_layers; ++l) {
    const kvq_layer_cfg& c = cfg[l];
    if (!valid_bits(c.k_bits) || !valid_bits(c.v_bits))
      return fail(KVQ_ERR_UNSUPPORTED, "layer %d: bits K%d V%d (each of 2, 4, 8, 16)", l, c.k_bits, c.v_bits);
    if (c.k_axis != KVQ_AXIS_CHANNEL && c.k_axis != KVQ_AXIS_TOKEN)
      return fail(KVQ_ERR_UNSUPPORTED, "layer %d: k_axis %d", l, c.k_axis);
    if (c.v_axis != KVQ_AXIS_TOKEN) return fail(KVQ_ERR_UNSUPPORTED, "layer %d: v_axis must be per-token", l);
    if (paged && !(c.k_bits == 2 && c.v_bits == 2 && c.k_axis == KVQ_AXIS_CHANNEL))
      return fail(KVQ_ERR_UNSUPPORTED, "layer %d: a paged pool needs K2V2 per-channel keys", l);
  }
  std::memset(out, 0, sizeof *out);
  out->shape = s;
  out->num_layers = num_layers;
  uint64_t off = 0;
  double bits = 0.0;
  const uint64_t hkv = (uint64_t)s.num_kv_heads;
  for (int l = 0; l < num_layers; ++l) {
    const kvq_layer_cfg& c = cfg[l];
    kvq_layer_plan& lp = out->layers[l];
    lp.k_bits = c.k_bits;
    lp.v_bits = c.v_bits;
    lp.k_axis = c.k_axis;
    lp.v_axis = c.v_axis;
    lp.offset = off;
    lp.record_bytes = kvq::record_bytes(c.k_bits, c.v_bits);
    if (!paged) {
      lp.groups_cap = (uint64_t)s.max_tokens / kvq::GS;
      lp.stream_bytes = lp.groups_cap * lp.record_bytes + kvq::TAIL_BYTES;
      lp.tail_offset = lp.groups_cap * lp.record_bytes;
      lp.bytes = (uint64_t)s.max_batch * hkv * lp.stream_bytes;
      bits += (c.k_bits + c.v_bits) / 2.0;
    } else {
      // INT2 page: half of a K2V2 group record per KV head; INT4 page: 16
      // tokens of per-token K4 and V4 codes plus their meta per KV head.
      lp.int2_page_bytes = hkv * 2048u;
      lp.int4_page_bytes = hkv * 3072u;
      lp.int4_offset = (uint64_t)s.int2_pages * lp.int2_page_bytes;
      lp.bytes = lp.int4_offset + (uint64_t)s.int4_pages * lp.int4_page_bytes;
    }
    off = align_up(off + lp.bytes, 4096);
  }
  out->total_bytes = off;
  if (paged) {
    const double n = (double)s.int2_pages + (double)s.int4_pages;
    out->int2_fraction = s.int2_pages / n;
    out->equiv_bits = 2.0 * out->int2_fraction + 4.0 * (1.0 - out->int2_fraction);
  } else {
    out->equiv_bits = bits / num_layers;
  }
  return ok();
}

int kvq_quantize_append(const kvq_plan* plan, int32_t layer, void* cache, const uint16_t* k_new,
                        const uint16_t* v_new, const int32_t* seq_lens, int32_t batch, int32_t n_new,
                        const kvq_pages* pages, kvq_stream_t stream) {
  int st = check_plan_layer(plan, layer);
  if (st) return st;
  if (!cache || !k_new || !v_new) return fail(KVQ_ERR_INVALID_ARG, "null cache or input pointer");
  if (!aligned16(cache) || !aligned16(k_new) || !aligned16(v_new))
    return fail(KVQ_ERR_INVALID_ARG, "cache, k_new and v_new must be 16-byte aligned");
  if (batch < 0 || batch > plan->shape.max_batch)
    return fail(KVQ_ERR_INVALID_ARG, "batch %d out of range [0, %d]", batch, plan->shape.max_batch);
  if (n_new < 0) return fail(KVQ_ERR_INVALID_ARG, "n_new %d < 0", n_new);
  if ((st = check_pages(plan, pages))) return st;
  if (!pages && !seq_lens) return fail(KVQ_ERR_INVALID_ARG, "seq_lens is NULL");
  if (n_new > capacity_tokens(plan, pages))
    return fail(KVQ_ERR_CAPACITY, "n_new %d > %lld tokens of capacity", n_new, (long long)capacity_tokens(plan, pages));
  if (batch == 0 || n_new == 0) return ok();
  kvq::AppendArgs a;
  a.geo = geom(plan, layer, cache);
  a.pg = paged_geom(plan, layer, pages);
  a.k_new = k_new;
  a.v_new = v_new;
  a.seq_lens = seq_lens;
  a.n_new = n_new;
  hipStream_t s = (hipStream_t)stream;
  kvq::EventPair ev;
  const bool timed = timer_slot(0, &ev);
  const hipError_t e = pages ? kvq::launch_append_paged(a, batch, s, timed ? &ev : nullptr)
                             : kvq::launch_append(a, batch, s, timed ? &ev : nullptr);
  return hip_status(e, "append launch");
}

size_t kvq_decode_workspace_bytes(const kvq_plan* plan, int32_t batch, int32_t max_seq_len, int32_t num_splits) {
  if (!plan || batch < 0 || max_seq_len < 0 || num_splits < 0 || num_splits > 1024) return 0;
  if (num_splits == 1 && is_paged(plan) && max_seq_len > 0) return 0;
  const int32_t s = num_splits ? num_splits : auto_splits(plan, batch, max_seq_len);
  return (size_t)batch * plan->shape.num_q_heads * s * (kvq::D + 1) * sizeof(float);
}

int32_t kvq_decode_num_splits(const kvq_plan* plan, int32_t layer, int32_t batch, int32_t max_seq_len) {
  (void)layer;
  if (!plan || batch < 0 || max_seq_len < 0) return 0;
  return auto_splits(plan, batch, max_seq_len);
}

int kvq_decode_attention(const kvq_plan* plan, int32_t layer, const void* cache, const uint16_t* q,
                         const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, float softmax_scale,
                         void* out, int32_t out_dtype, float* lse_out, void* workspace, size_t workspace_bytes,
                         int32_t num_splits, const kvq_pages* pages, kvq_stream_t stream) {
  int st = check_plan_layer(plan, layer);
  if (st) return st;
  if (!cache || !q || !out) return fail(KVQ_ERR_INVALID_ARG, "null cache, q or out");
  if (!aligned16(cache) || !aligned16(q) || !aligned16(out) || !aligned16(workspace))
    return fail(KVQ_ERR_INVALID_ARG, "cache, q, out and workspace must be 16-byte aligned");
  if (batch < 0 || batch > plan->shape.max_batch)
    return fail(KVQ_ERR_INVALID_ARG, "batch %d out of range [0, %d]", batch, plan->shape.max_batch);
  if (out_dtype != KVQ_OUT_F16 && out_dtype != KVQ_OUT_F32)
    return fail(KVQ_ERR_INVALID_ARG, "out_dtype %d", out_dtype);
  if (num_splits < 0 || num_splits > 1024) return fail(KVQ_ERR_INVALID_ARG, "num_splits %d", num_splits);
  if (!std::isfinite(softmax_scale)) return fail(KVQ_ERR_INVALID_ARG, "softmax_scale is not finite");
  if (max_seq_len < 0) return fail(KVQ_ERR_INVALID_ARG, "max_seq_len %d < 0", max_seq_len);
  if ((st = check_pages(plan, pages))) return st;
  if (!pages && !seq_lens) return fail(KVQ_ERR_INVALID_ARG, "seq_lens is NULL");
  if (max_seq_len > capacity_tokens(plan, pages))
    return fail(KVQ_ERR_CAPACITY, "max_seq_len %d > %lld tokens of capacity", max_seq_len,
                (long long)capacity_tokens(plan, pages));
  if (batch == 0) return ok();
  const int32_t splits = num_splits ? num_splits : auto_splits(plan, batch, max_seq_len);
  int32_t gps = 0;
  if ((st = split_groups(pages, splits, max_seq_len, &gps))) return st;
  const size_t need = (size_t)batch * plan->shape.num_q_heads * splits * (kvq::D + 1) * sizeof(float);
  if (!workspace || workspace_bytes < need)
    return fail(KVQ_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  kvq::DecodeArgs a;
  a.geo = geom(plan, layer, cache);
  a.pg = paged_geom(plan, layer, pages);
  a.q = q;
  a.seq_lens = seq_lens;
  a.splits = splits;
  a.groups_per_split = gps;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.part_o = (float*)workspace;
  a.part_lse = a.part_o + (size_t)batch * plan->shape.num_q_heads * splits * kvq::D;
  a.out = out;
  a.out_f32 = out_dtype == KVQ_OUT_F32;
  a.lse_out = lse_out;
  hipStream_t s = (hipStream_t)stream;
  kvq::EventPair ev;
  bool timed = timer_slot(1, &ev);
  hipError_t e = pages ? kvq::launch_decode_paged(a, batch, s, timed ? &ev : nullptr)
                       : kvq::launch_decode_split_mfma(a, batch, s, timed ? &ev : nullptr);
  if (e != hipSuccess) return hip_status(e, "decode split launch");
  if (splits == 1) return ok();  // the split pass wrote the final output
  kvq::MergeArgs m;
  m.part_o = a.part_o;
  m.part_lse = a.part_lse;
  m.splits = splits;
  m.rows = batch * plan->shape.num_q_heads;
  m.out = out;
  m.out_f32 = out_dtype == KVQ_OUT_F32;
  m.lse_out = lse_out;
  timed = timer_slot(2, &ev);
  e = kvq::launch_merge(m, s, timed ? &ev : nullptr);
  return hip_status(e, "merge launch");
}

int kvq_append_decode_attention(const kvq_plan* plan, int32_t layer, void* cache, const uint16_t* k_new,
                                const uint16_t* v_new, const uint16_t* q, const int32_t* seq_lens, int32_t batch,
                                int32_t max_seq_len, float softmax_scale, void* out, int32_t out_dtype,
                                float* lse_out, void* workspace, size_t workspace_bytes, int32_t num_splits,
                                const kvq_pages* pages, kvq_stream_t stream) {
  int st = check_plan_layer(plan, layer);
  if (st) return st;
  if (!cache || !k_new || !v_new || !q || !out) return fail(KVQ_ERR_INVALID_ARG, "null cache, input or output");
  if (!aligned16(cache) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(q) || !aligned16(out) ||
      !aligned16(workspace))
    return fail(KVQ_ERR_INVALID_ARG, "cache, k_new, v_new, q, out and workspace must be 16-byte aligned");
  if ((st = check_pages(plan, pages))) return st;
  if (!pages && !seq_lens) return fail(KVQ_ERR_INVALID_ARG, "seq_lens is NULL");
  if (pages && pages->int2_add)
    return fail(KVQ_ERR_INVALID_ARG, "a fused paged step appends one INT4 token a request: int2_add must be NULL");
  if (batch < 0 || batch > plan->shape.max_batch)
    return fail(KVQ_ERR_INVALID_ARG, "batch %d out of range [0, %d]", batch, plan->shape.max_batch);
  if (out_dtype != KVQ_OUT_F16 && out_dtype != KVQ_OUT_F32)
    return fail(KVQ_ERR_INVALID_ARG, "out_dtype %d", out_dtype);
  if (num_splits < 0 || num_splits > 1024) return fail(KVQ_ERR_INVALID_ARG, "num_splits %d", num_splits);
  if (!std::isfinite(softmax_scale)) return fail(KVQ_ERR_INVALID_ARG, "softmax_scale is not finite");
  if (max_seq_len < 1) return fail(KVQ_ERR_INVALID_ARG, "max_seq_len %d < 1 (it counts the appended token)", max_seq_len);
  if (max_seq_len > capacity_tokens(plan, pages))
    return fail(KVQ_ERR_CAPACITY, "max_seq_len %d > %lld tokens of capacity", max_seq_len,
                (long long)capacity_tokens(plan, pages));
  if (batch == 0) return ok();
  const int32_t splits = num_splits ? num_splits : auto_splits(plan, batch, max_seq_len);
  int32_t gps = 0;
  if ((st = split_groups(pages, splits, max_seq_len, &gps))) return st;
  const size_t need = (size_t)batch * plan->shape.num_q_heads * splits * (kvq::D + 1) * sizeof(float);
  if (!workspace || workspace_bytes < need)
    return fail(KVQ_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  kvq::DecodeArgs a;
  a.geo = geom(plan, layer, cache);
  a.pg = paged_geom(plan, layer, pages);
  a.q = q;
  a.seq_lens = seq_lens;
  a.splits = splits;
  a.groups_per_split = gps;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.part_o = (float*)workspace;
  a.part_lse = a.part_o + (size_t)batch * plan->shape.num_q_heads * splits * kvq::D;
  a.out = out;
  a.out_f32 = out_dtype == KVQ_OUT_F32;
  a.lse_out = lse_out;
  a.k_new = k_new;
  a.v_new = v_new;
  hipStream_t s = (hipStream_t)stream;
  kvq::EventPair ev;
  bool timed = timer_slot(1, &ev);
  hipError_t e = pages ? kvq::launch_decode_paged(a, batch, s, timed ? &ev : nullptr)
                       : kvq::launch_decode_split_mfma(a, batch, s, timed ? &ev : nullptr);
  if (e != hipSuccess) return hip_status(e, "fused append and split launch");
  if (splits == 1) return ok();
  kvq::MergeArgs m;
  m.part_o = a.part_o;
  m.part_lse = a.part_lse;
  m.splits = splits;
  m.rows = batch * plan->shape.num_q_heads;
  m.out = out;
  m.out_f32 = out_dtype == KVQ_OUT_F32;
  m.lse_out = lse_out;
  timed = timer_slot(2, &ev);
  e = kvq::launch_merge(m, s, timed ? &ev : nullptr);
  return hip_status(e, "merge launch");
}

size_t kvq_prefix_workspace_bytes(const kvq_plan* plan, int32_t batch, int32_t chunk, int32_t max_seq_len,
                                  int32_t num_splits) {
  if (!plan || batch < 0 || chunk < 0 || max_seq_len < 0 || num_splits < 0 || num_splits > 1024) return 0;
  const int32_t s = num_splits ? num_splits : prefix_splits(plan, batch, chunk, max_seq_len);
  if (s == 1) return 0;
  return (size_t)batch * chunk * plan->shape.num_q_heads * s * (kvq::D + 1) * sizeof(float);
}

int kvq_prefix_attention(const kvq_plan* plan, int32_t layer, const void* cache, const uint16_t* q, int32_t chunk,
                         const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, float softmax_scale,
                         float* out, float* lse_out, void* workspace, size_t workspace_bytes, int32_t num_splits,
                         const kvq_pages* pages, kvq_stream_t stream) {
  int st = check_plan_layer(plan, layer);
  if (st) return st;
  if ((st = check_pages(plan, pages))) return st;
  if (!cache || !q || !out || (!pages && !seq_lens)) return fail(KVQ_ERR_INVALID_ARG, "null cache, q, seq_lens or out");
  if (!aligned16(cache) || !aligned16(q) || !aligned16(out) || !aligned16(workspace))
    return fail(KVQ_ERR_INVALID_ARG, "cache, q, out and workspace must be 16-byte aligned");
  if (batch < 0 || batch > plan->shape.max_batch)
    return fail(KVQ_ERR_INVALID_ARG, "batch %d out of range [0, %d]", batch, plan->shape.max_batch);
  if (chunk < 0 || (int64_t)batch * chunk * plan->shape.num_q_heads > (1 << 26))
    return fail(KVQ_ERR_INVALID_ARG, "chunk %d: batch * chunk * Hq rows must be at most 2^26", chunk);
  if (num_splits < 0 || num_splits > 1024) return fail(KVQ_ERR_INVALID_ARG, "num_splits %d", num_splits);
  if (!std::isfinite(softmax_scale)) return fail(KVQ_ERR_INVALID_ARG, "softmax_scale is not finite");
  if (max_seq_len < 0) return fail(KVQ_ERR_INVALID_ARG, "max_seq_len %d < 0", max_seq_len);
  if (max_seq_len > capacity_tokens(plan, pages))
    return fail(KVQ_ERR_CAPACITY, "max_seq_len %d > %lld tokens of capacity", max_seq_len,
                (long long)capacity_tokens(plan, pages));
  if (batch == 0 || chunk == 0) return ok();
  const int32_t splits = num_splits ? num_splits : prefix_splits(plan, batch, chunk, max_seq_len);
  const int32_t nvg = (max_seq_len + kvq::GS - 1) / kvq::GS;
  const int32_t gps = nvg > 0 ? (nvg + splits - 1) / splits : 1;
  const size_t rows = (size_t)batch * chunk * plan->shape.num_q_heads;
  const size_t need = splits > 1 ? rows * splits * (kvq::D + 1) * sizeof(float) : 0;
  if (need && (!workspace || workspace_bytes < need))
    return fail(KVQ_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  if ((int64_t)splits * prefix_blocks(plan, chunk) > 0x7FFFFFFF)
    return fail(KVQ_ERR_INVALID_ARG, "num_splits %d times the row blocks exceeds the grid", splits);
  kvq::DecodeArgs a;
  a.geo = geom(plan, layer, cache);
  a.pg = paged_geom(plan, layer, pages);
  a.q = q;
  a.seq_lens = seq_lens;
  a.splits = splits;
  a.groups_per_split = gps;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.part_o = (float*)workspace;
  a.part_lse = need ? a.part_o + rows * splits * kvq::D : nullptr;
  a.out = out;
  a.out_f32 = 1;
  a.lse_out = lse_out;
  a.chunk = chunk;
  hipStream_t s = (hipStream_t)stream;
  kvq::EventPair ev;
  bool timed = timer_slot(3, &ev);
  hipError_t e = kvq::launch_prefix(a, batch, s, timed ? &ev : nullptr);
  if (e != hipSuccess) return hip_status(e, "prefix split launch");
  if (splits == 1) return ok();
  kvq::MergeArgs m;
  m.part_o = a.part_o;
  m.part_lse = a.part_lse;
  m.splits = splits;
  m.rows = (int)rows;
  m.out = out;
  m.out_f32 = 1;
  m.lse_out = lse_out;
  timed = timer_slot(2, &ev);
  e = kvq::launch_merge(m, s, timed ? &ev : nullptr);
  return hip_status(e, "merge launch");
}

size_t kvq_chunk_prefill_workspace_bytes(const kvq_plan* plan, int32_t batch, int32_t chunk, int32_t max_seq_len,
                                         int32_t num_splits) {
  if (!plan || batch < 0 || chunk < 0 || max_seq_len < 0 || num_splits < 0 || num_splits > 1024) return 0;
  const int32_t s = num_splits ? num_splits : prefix_splits(plan, batch, chunk, max_seq_len);
  return (size_t)batch * chunk * plan->shape.num_q_heads * (s + 1) * (kvq::D + 1) * sizeof(float);
}

int kvq_chunk_prefill_attention(const kvq_plan* plan, int32_t layer, const void* cache, const uint16_t* q,
                                const uint16_t* k_chunk, const uint16_t* v_chunk, int32_t chunk,
                                const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, float softmax_scale,
                                float* out, float* lse_out, void* workspace, size_t workspace_bytes,
                                int32_t num_splits, const kvq_pages* pages, kvq_stream_t stream) {
  int st = check_plan_layer(plan, layer);
  if (st) return st;
  if ((st = check_pages(plan, pages))) return st;
  if (!cache || !q || !k_chunk || !v_chunk || !out || (!pages && !seq_lens))
    return fail(KVQ_ERR_INVALID_ARG, "null cache, q, k_chunk, v_chunk, seq_lens or out");
  if (!aligned16(cache) || !aligned16(q) || !aligned16(k_chunk) || !aligned16(v_chunk) || !aligned16(out) ||
      !aligned16(workspace))
    return fail(KVQ_ERR_INVALID_ARG, "cache, q, k_chunk, v_chunk, out and workspace must be 16-byte aligned");
  if (batch < 0 || batch > plan->shape.max_batch)
    return fail(KVQ_ERR_INVALID_ARG, "batch %d out of range [0, %d]", batch, plan->shape.max_batch);
  if (chunk < 0 || (int64_t)batch * chunk * plan->shape.num_q_heads > (1 << 26))
    return fail(KVQ_ERR_INVALID_ARG, "chunk %d: batch * chunk * Hq rows must be at most 2^26", chunk);
  if (num_splits < 0 || num_splits > 1023) return fail(KVQ_ERR_INVALID_ARG, "num_splits %d", num_splits);
  if (!std::isfinite(softmax_scale)) return fail(KVQ_ERR_INVALID_ARG, "softmax_scale is not finite");
  if (max_seq_len < 0) return fail(KVQ_ERR_INVALID_ARG, "max_seq_len %d < 0", max_seq_len);
  if (max_seq_len > capacity_tokens(plan, pages))
    return fail(KVQ_ERR_CAPACITY, "max_seq_len %d > %lld tokens of capacity", max_seq_len,
                (long long)capacity_tokens(plan, pages));
  if (batch == 0 || chunk == 0) return ok();
  const int32_t splits = num_splits ? num_splits : prefix_splits(plan, batch, chunk, max_seq_len);
  const int32_t nvg = (max_seq_len + kvq::GS - 1) / kvq::GS;
  const int32_t gps = nvg > 0 ? (nvg + splits - 1) / splits : 1;
  const size_t rows = (size_t)batch * chunk * plan->shape.num_q_heads;
  const size_t need = rows * (splits + 1) * (kvq::D + 1) * sizeof(float);
  if (!workspace || workspace_bytes < need)
    return fail(KVQ_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  if ((int64_t)splits * prefix_blocks(plan, chunk) > 0x7FFFFFFF)
    return fail(KVQ_ERR_INVALID_ARG, "num_splits %d times the row blocks exceeds the grid", splits);
  kvq::DecodeArgs a;
  a.geo = geom(plan, layer, cache);
  a.pg = paged_geom(plan, layer, nullptr);
  a.q = q;
  a.seq_lens = seq_lens;
  a.splits = splits;
  a.groups_per_split = gps;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.part_o = (float*)workspace;
  a.part_lse = a.part_o + rows * (splits + 1) * kvq::D;
  a.out = out;
  a.out_f32 = 1;
  a.lse_out = lse_out;
  a.chunk = chunk;
  a.part_stride = splits + 1;
  a.pg = paged_geom(plan, layer, pages);
  a.k_chunk = k_chunk;
  a.v_chunk = v_chunk;
  hipStream_t s = (hipStream_t)stream;
  kvq::EventPair ev;
  bool timed = timer_slot(3, &ev);
  hipError_t e = kvq::launch_prefix(a, batch, s, timed ? &ev : nullptr);
  if (e != hipSuccess) return hip_status(e, "prefix split launch");
  e = kvq::launch_chunk_causal(a, batch, s, nullptr);
  if (e != hipSuccess) return hip_status(e, "chunk causal launch");
  kvq::MergeArgs m;
  m.part_o = a.part_o;
  m.part_lse = a.part_lse;
  m.splits = splits + 1;
  m.rows = (int)rows;
  m.out = out;
  m.out_f32 = 1;
  m.lse_out = lse_out;
  timed = timer_slot(2, &ev);
  e = kvq::launch_merge(m, s, timed ? &ev : nullptr);
  return hip_status(e, "merge launch");
}

int kvq_dequantize(const kvq_plan* plan, int32_t layer, const void* cache, const int32_t* seq_lens, int32_t batch,
                   int32_t max_seq_len, float* k_out, float* v_out, const kvq_pages* pages, kvq_stream_t stream) {
  int st = check_plan_layer(plan, layer);
  if (st) return st;
  if (!cache || !k_out || !v_out) return fail(KVQ_ERR_INVALID_ARG, "null cache or output");
  if (batch < 0 || batch > plan->shape.max_batch)
    return fail(KVQ_ERR_INVALID_ARG, "batch %d out of range [0, %d]", batch, plan->shape.max_batch);
  if (max_seq_len < 0) return fail(KVQ_ERR_INVALID_ARG, "max_seq_len %d < 0", max_seq_len);
  if ((st = check_pages(plan, pages))) return st;
  if (!pages && !seq_lens) return fail(KVQ_ERR_INVALID_ARG, "seq_lens is NULL");
  if (max_seq_len > capacity_tokens(plan, pages))
    return fail(KVQ_ERR_CAPACITY, "max_seq_len %d > %lld tokens of capacity", max_seq_len,
                (long long)capacity_tokens(plan, pages));
  if (batch == 0 || max_seq_len == 0) return ok();
  kvq::DequantArgs a;
  a.geo = geom(plan, layer, cache);
  a.pg = paged_geom(plan, layer, pages);
  a.seq_lens = seq_lens;
  a.max_seq_len = max_seq_len;
  a.k_out = k_out;
  a.v_out = v_out;
  const hipError_t e = pages ? kvq::launch_dequant_paged(a, batch, (hipStream_t)stream)
                             : kvq::launch_dequant(a, batch, (hipStream_t)stream);
  return hip_status(e, "dequantize launch");
}

int kvq_timer_start(int32_t capacity) {
  if (capacity <= 0 || capacity > (1 << 20)) return fail(KVQ_ERR_INVALID_ARG, "timer capacity %d", capacity);
  std::lock_guard<std::mutex> lk(g_timer.mu);
  timer_free_locked();
  for (int k = 0; k < kTimerKinds; ++k)
    for (int i = 0; i < 2; ++i) {
      g_timer.ev[k][i].resize(capacity);
      for (int n = 0; n < capacity; ++n) {
        hipError_t e = hipEventCreate(&g_timer.ev[k][i][n]);
        if (e != hipSuccess) {
          g_timer.ev[k][i].resize(n);
          timer_free_locked();
          return fail(KVQ_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(e));
        }
      }
    }
  g_timer.capacity = capacity;
  g_timer.armed = true;
  return ok();
}

int kvq_timer_read(int32_t kind, double* total_ms, int32_t* launches) {
  if (kind < 0 || kind >= kTimerKinds || !total_ms || !launches)
    return fail(KVQ_ERR_INVALID_ARG, "bad timer read arguments");
  std::lock_guard<std::mutex> lk(g_timer.mu);
  double sum = 0.0;
  const int n = g_timer.used[kind];
  for (int i = 0; i < n; ++i) {
    hipError_t e = hipEventSynchronize(g_timer.ev[kind][1][i]);
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "hipEventSynchronize: %s", hipGetErrorString(e));
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, g_timer.ev[kind][0][i], g_timer.ev[kind][1][i]);
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "hipEventElapsedTime: %s", hipGetErrorString(e));
    sum += ms;
  }
  *total_ms = sum;
  *launches = n;
  return ok();
}

int kvq_timer_stop(void) {
  std::lock_guard<std::mutex> lk(g_timer.mu);
  timer_free_locked();
  return ok();
}

}  // extern "C"
