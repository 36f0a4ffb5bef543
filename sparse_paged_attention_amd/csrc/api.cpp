// C ABI of libspa.so: argument checks on the host, launch planning, and the
// host-side physical-page allocator. Every check runs before anything is
// enqueued; kernels only see arguments that passed them.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/spa.h"
#include "spa_internal.h"

namespace {

thread_local std::string g_last_error;

spa_status fail(spa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

spa_status ok() {
  g_last_error.clear();
  return SPA_OK;
}

spa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SPA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Attention blocks per work item (16 tokens each). All work-groups of a
// launch are resident at once and the dispatcher spreads them evenly over
// the compute units, so the launch lasts as long as the busiest unit: the
// item size is picked to minimise max(ceil(items / CUs), 2) * blocks per
// item. The floor of 2: one wave's own chain of dependent tile loads lasts
// about as long as two items' share of a unit's bandwidth, so below two
// items per unit shorter items win (256K single sequence: 9 blocks, one item
// per unit, 14.8 us per call; 5 or 6 blocks, two per unit, 12.7-13.0 us).
// spa_set_attn_blocks_per_item() or the SPA_ATTN_BLOCKS_PER_ITEM environment
// variable (one of kBpiChoices) fixes it instead.
constexpr int32_t kBpiChoices[] = {4, 5, 6, 7, 8, 9, 10, 12, 16};
constexpr int32_t kBpiMin = 4;

bool valid_bpi(int32_t x) {
  for (int32_t c : kBpiChoices)
    if (x == c) return true;
  return false;
}

std::atomic<int32_t> g_forced_bpi{-1};   // -1: not read yet, 0: automatic

int32_t forced_blocks_per_item() {
  int32_t v = g_forced_bpi.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* e = std::getenv("SPA_ATTN_BLOCKS_PER_ITEM");
    const int32_t x = e ? std::atoi(e) : 0;
    v = valid_bpi(x) ? x : 0;
    int32_t expect = -1;
    if (!g_forced_bpi.compare_exchange_strong(expect, v)) v = expect;
  }
  return v;
}

// Compute units of the current device (queried once per device).
int32_t device_cus() {
  static int32_t cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Largest page count a selection row can score (top-k keeps 32 keys per thread).
constexpr int64_t kMaxScoredPages = 32768;

spa_status check_pool(const spa_pool* pool, spa::PoolArgs* out) {
  if (!pool) return fail(SPA_ERR_INVALID, "pool is NULL");
  if (pool->num_kv_heads < 1 || pool->num_kv_heads > spa::kMaxKvHeads)
    return fail(SPA_ERR_INVALID, "num_kv_heads %d outside [1, %d]", pool->num_kv_heads, spa::kMaxKvHeads);
  if (pool->head_dim != spa::kHeadDim)
    return fail(pool->head_dim < 1 ? SPA_ERR_INVALID : SPA_ERR_UNSUPPORTED,
                "head_dim %d: only 128 is built", pool->head_dim);
  const int32_t p = pool->logical_page, P = pool->physical_page;
  if (p < 1 || p > 64) return fail(SPA_ERR_INVALID, "logical_page %d outside [1, 64]", p);
  if (p != 16 && p != 32 && p != 64)
    return fail(SPA_ERR_UNSUPPORTED, "logical_page %d: only 16, 32 and 64 are built", p);
  if (P < p || P % p != 0) return fail(SPA_ERR_INVALID, "physical_page %d is not a multiple of logical_page %d", P, p);
  if (P / p > 64) return fail(SPA_ERR_INVALID, "physical_page / logical_page = %d exceeds 64", P / p);
  if (pool->num_phys_pages < 1) return fail(SPA_ERR_INVALID, "num_phys_pages %d < 1", pool->num_phys_pages);
  if (!pool->k_pool || !pool->v_pool) return fail(SPA_ERR_INVALID, "k_pool / v_pool is NULL");
  const int32_t hs = pool->head_slots == 0 ? pool->num_kv_heads : pool->head_slots;
  if (hs < 1 || hs > pool->num_kv_heads)
    return fail(SPA_ERR_INVALID, "head_slots %d outside [1, num_kv_heads = %d] (0: num_kv_heads)", pool->head_slots,
                pool->num_kv_heads);
  if ((int64_t)pool->num_phys_pages * hs * (P / p) >= (int64_t)UINT32_MAX)
    return fail(SPA_ERR_UNSUPPORTED, "pool of %d pages x %d head slots x %d logical pages has 2^32 or more "
                "summary records", pool->num_phys_pages, hs, P / p);
  out->hkv = pool->num_kv_heads;
  out->hs = hs;
  out->p = p;
  out->P = P;
  out->r = P / p;
  out->N = pool->num_phys_pages;
  out->k = static_cast<uint16_t*>(pool->k_pool);
  out->v = static_cast<uint16_t*>(pool->v_pool);
  out->summ = static_cast<uint16_t*>(pool->summary);
  if (pool->kv_format != SPA_KV_BF16 && pool->kv_format != SPA_KV_FP8)
    return fail(SPA_ERR_INVALID, "kv_format %d is neither SPA_KV_BF16 nor SPA_KV_FP8", pool->kv_format);
  out->q8 = pool->kv_format == SPA_KV_FP8;
  out->ks = out->q8 ? pool->k_scale : nullptr;
  out->vs = out->q8 ? pool->v_scale : nullptr;
  if (out->q8 && (!out->ks || !out->vs)) return fail(SPA_ERR_INVALID, "an fp8 pool needs k_scale and v_scale");
  return SPA_OK;
}

spa_status check_heads(const spa_heads* heads, const spa::PoolArgs& pl, int32_t* G,
                       spa::HeadList* dyn, uint8_t* kind) {
  if (!heads) return fail(SPA_ERR_INVALID, "heads is NULL");
  if (heads->num_q_heads < 1 || heads->num_q_heads % pl.hkv != 0)
    return fail(SPA_ERR_INVALID, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                heads->num_q_heads, pl.hkv);
  const int32_t g = heads->num_q_heads / pl.hkv;
  if (g > 16) return fail(SPA_ERR_UNSUPPORTED, "query group size %d: groups of up to 16 are built", g);
  if (heads->sink < 0) return fail(SPA_ERR_INVALID, "sink %d < 0", heads->sink);
  if (heads->window < 1) return fail(SPA_ERR_INVALID, "window %d < 1", heads->window);
  if (!heads->kind) return fail(SPA_ERR_INVALID, "heads->kind is NULL");
  dyn->n = 0;
  for (int32_t h = 0; h < pl.hkv; ++h) {
    const uint8_t k = heads->kind[h];
    if (k > 1) return fail(SPA_ERR_INVALID, "kind[%d] = %u is neither 0 nor 1", h, (unsigned)k);
    if (kind) kind[h] = k;
    if (k) dyn->id[dyn->n++] = (int16_t)h;
  }
  if (dyn->n > 0 && !pl.summ) return fail(SPA_ERR_INVALID, "dynamic heads need pool->summary");
  if (pl.hs < pl.hkv && (dyn->n > pl.hs || pl.hkv - dyn->n > pl.hs))
    return fail(SPA_ERR_INVALID, "head_slots %d holds neither the %d dynamic nor the %d streaming heads", pl.hs,
                dyn->n, pl.hkv - dyn->n);
  *G = g;
  return SPA_OK;
}

spa_status check_batch(const spa_batch* batch, const spa::PoolArgs& pl, spa::BatchArgs* out) {
  if (!batch) return fail(SPA_ERR_INVALID, "batch is NULL");
  if (batch->batch < 0) return fail(SPA_ERR_INVALID, "batch %d < 0", batch->batch);
  if (batch->batch > 65535) return fail(SPA_ERR_INVALID, "batch %d > 65535", batch->batch);
  if (batch->max_pages < 1) return fail(SPA_ERR_INVALID, "max_pages %d < 1", batch->max_pages);
  if ((int64_t)batch->max_pages * pl.P > INT32_MAX)
    return fail(SPA_ERR_INVALID, "max_pages * physical_page exceeds 2^31 - 1 tokens");
  if (batch->batch > 0 && (!batch->page_table || !batch->seq_lens))
    return fail(SPA_ERR_INVALID, "page_table / seq_lens is NULL");
  out->B = batch->batch;
  out->max_pp = batch->max_pages;
  out->pt = batch->page_table;
  out->lens = batch->seq_lens;
  out->ring = batch->stream_pages;
  out->ring_sink = 0;
  out->ring_win = 1;
  return SPA_OK;
}

// Pages of the ring that keeps a sequence's streaming heads: the sink's pages
// and the pages a window of `window` tokens can touch at once (one more than
// it fills when it is not aligned to a page).
void ring_geometry(const spa_heads* heads, int32_t P, int32_t* sink_pages, int32_t* win_pages) {
  *sink_pages = (int32_t)(((int64_t)heads->sink + P - 1) / P);
  *win_pages = (int32_t)(((int64_t)heads->window + P - 1) / P) + 1;
}

// Completes the batch's ring geometry (streaming heads kept in a ring when
// stream_pages is given), which needs the head kinds.
// A compact pool (fewer head slots than heads) keeps streaming heads in rings
// only, so its calls need the head kinds and, with streaming heads, the rings.
bool has_streaming(const spa_heads* heads, int32_t hkv) {
  for (int32_t h = 0; h < hkv; ++h)
    if (!heads->kind[h]) return true;
  return false;
}

spa_status set_ring(const spa_heads* heads, const spa::PoolArgs& pl, spa::BatchArgs* bt) {
  if (pl.hs < pl.hkv) {
    if (!heads) return fail(SPA_ERR_INVALID, "a pool with head_slots < num_kv_heads needs the head kinds");
    if (!bt->ring && has_streaming(heads, pl.hkv))
      return fail(SPA_ERR_INVALID, "a pool with head_slots < num_kv_heads keeps streaming heads in rings: "
                  "stream_pages is NULL");
  }
  if (!bt->ring) return SPA_OK;
  if (!heads) return fail(SPA_ERR_INVALID, "stream_pages needs the head kinds (heads is NULL)");
  ring_geometry(heads, pl.P, &bt->ring_sink, &bt->ring_win);
  if ((int64_t)bt->ring_sink + bt->ring_win > pl.N)
    return fail(SPA_ERR_INVALID, "a ring of %d pages does not fit a pool of %d", bt->ring_sink + bt->ring_win, pl.N);
  return SPA_OK;
}

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

int32_t n_max_pages(const spa::PoolArgs& pl, int32_t max_pp) {
  return (int32_t)((int64_t)max_pp * pl.r);   // logical pages a page-table row can address
}

// Items per head for a given item size: streaming heads cover the sink and
// window blocks (+1 when the window is unaligned), dynamic heads k_max pages
// plus one item for the tokens appended since the selection.
void size_items(const spa::PoolArgs& pl, const spa_heads* heads, int32_t k_max, int32_t bpi,
                spa::AttnPlan* plan) {
  const int64_t nb_stream = (heads->sink + 15) / 16 + (heads->window + 15) / 16 + 1;
  const int64_t nb_dyn = (int64_t)k_max * (pl.p / 16);
  plan->blocks_per_item = bpi;
  plan->items_stream = (int32_t)((nb_stream + bpi - 1) / bpi);
  plan->items_dyn = (int32_t)((nb_dyn + bpi - 1) / bpi) + 1;
  // one slot more: the partial of a token appended inside the attention launch
  plan->item_stride = std::max(plan->items_stream, plan->items_dyn) + 1;
  plan->extra_partial = 0;
}

// batch < 0: size for the largest item count any batch size can use
// (workspace sizing); otherwise pick the item size for this batch.
void plan_attention(const spa::PoolArgs& pl, const spa_heads* heads, int32_t k_max, const uint8_t* kind,
                    int32_t batch, spa::AttnPlan* plan) {
  std::memset(plan, 0, sizeof *plan);
  int32_t n_dyn = 0;
  for (int32_t h = 0; h < pl.hkv; ++h)
    if (kind[h]) {
      plan->dyn_mask[h / 32] |= 1u << (h % 32);
      ++n_dyn;
    }
  const int32_t n_str = pl.hkv - n_dyn;
  int32_t bpi = forced_blocks_per_item();
  if (batch < 0) {
    bpi = kBpiMin;
  } else if (bpi == 0) {
    const int64_t cus = device_cus();
    int64_t best = -1;
    for (int32_t c : kBpiChoices) {
      spa::AttnPlan t;
      size_items(pl, heads, k_max, c, &t);
      const int64_t items = (int64_t)std::max(batch, 1) * (n_str * (int64_t)t.items_stream +
                                                           n_dyn * (int64_t)(t.items_dyn - 1));
      const int64_t cost = std::max<int64_t>((items + cus - 1) / cus, 2) * c;
      if (best < 0 || cost <= best) {      // ties go to the larger item
        best = cost;
        bpi = c;
      }
    }
  }
  size_items(pl, heads, k_max, bpi, plan);
  plan->items_per_seq = n_str * plan->items_stream + n_dyn * plan->items_dyn;
  plan->sink = heads->sink;
  plan->window = heads->window;
  plan->k_max = k_max;
}

// Workspace: a scratch area used by selection (page scores) and by attention
// (per-item partials); nothing in it lives from one call to the next.
size_t attn_bytes(const spa::PoolArgs& pl, const spa::AttnPlan& plan, int32_t B, int32_t G, size_t* ml_off) {
  const size_t slots = (size_t)B * pl.hkv * plan.item_stride * G;
  const size_t o = align_up(slots * spa::kHeadDim * sizeof(float));
  *ml_off = o;
  return o + align_up(slots * 2 * sizeof(float));
}

size_t select_bytes(const spa::PoolArgs& pl, int32_t B, int32_t max_pp) {
  return align_up((size_t)B * pl.hkv * n_max_pages(pl, max_pp) * sizeof(float));
}

}  // namespace

extern "C" {

const char* spa_status_string(spa_status s) {
  switch (s) {
    case SPA_OK: return "ok";
    case SPA_ERR_INVALID: return "invalid argument";
    case SPA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SPA_ERR_POOL_EXHAUSTED: return "page pool exhausted";
    case SPA_ERR_WORKSPACE: return "workspace missing or too small";
    case SPA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* spa_last_error(void) { return g_last_error.c_str(); }

spa_status spa_set_attn_blocks_per_item(int32_t blocks) {
  if (blocks != 0 && !valid_bpi(blocks))
    return fail(SPA_ERR_INVALID, "blocks per item %d: use 0 or one of 4, 5, 6, 7, 8, 9, 10, 12, 16", blocks);
  g_forced_bpi.store(blocks, std::memory_order_relaxed);
  return ok();
}

int32_t spa_stream_ring_pages(const spa_pool* pool, const spa_heads* heads) {
  spa::PoolArgs pl;
  spa::HeadList dyn;
  int32_t G;
  const std::string keep = g_last_error;
  int32_t n = 0;
  if (check_pool(pool, &pl) == SPA_OK && check_heads(heads, pl, &G, &dyn, nullptr) == SPA_OK) {
    int32_t a, b;
    ring_geometry(heads, pl.P, &a, &b);
    n = a + b;
  }
  g_last_error = keep;
  return n;
}

int32_t spa_default_budget(int64_t context_len) {
  if (context_len < 0) return 0;
  const int64_t b = context_len / 32;
  return (int32_t)std::min<int64_t>(b, 4096);
}

spa_status spa_kv_pool_append(const spa_pool* pool, const spa_heads* heads, const spa_batch* batch,
                              const void* k_new, const void* v_new, hipStream_t stream) {
  spa::PoolArgs pl;
  spa::BatchArgs bt;
  spa::HeadList dyn;
  int32_t G;
  spa_status s;
  if ((s = check_pool(pool, &pl)) != SPA_OK) return s;
  if (heads && (s = check_heads(heads, pl, &G, &dyn, nullptr)) != SPA_OK) return s;
  if ((s = check_batch(batch, pl, &bt)) != SPA_OK) return s;
  if ((s = set_ring(heads, pl, &bt)) != SPA_OK) return s;
  if (bt.B == 0) return ok();
  if (!k_new || !v_new) return fail(SPA_ERR_INVALID, "k_new / v_new is NULL");
  return hip_status(spa::launch_append(pl, bt, static_cast<const uint16_t*>(k_new),
                                       static_cast<const uint16_t*>(v_new), heads ? &dyn : nullptr, stream),
                    "kv_pool_append launch");
}

spa_status spa_kv_pool_write(const spa_pool* pool, const spa_heads* heads, const int32_t* page_table_row,
                             int32_t max_pages, int32_t stream_base, int64_t start, int64_t count, const void* k,
                             const void* v, hipStream_t stream) {
  spa::PoolArgs pl;
  spa::HeadList dyn;
  int32_t G;
  spa_status s;
  if ((s = check_pool(pool, &pl)) != SPA_OK) return s;
  if (heads && (s = check_heads(heads, pl, &G, &dyn, nullptr)) != SPA_OK) return s;
  if (max_pages < 1) return fail(SPA_ERR_INVALID, "max_pages %d < 1", max_pages);
  if (start < 0 || count < 0) return fail(SPA_ERR_INVALID, "start %lld / count %lld negative",
                                          (long long)start, (long long)count);
  if (start + count > (int64_t)max_pages * pl.P)
    return fail(SPA_ERR_INVALID, "tokens [%lld, %lld) exceed max_pages * physical_page = %lld",
                (long long)start, (long long)(start + count), (long long)max_pages * pl.P);
  int32_t ring_sink = 0, ring_win = 1;
  if (pl.hs < pl.hkv) {
    if (!heads) return fail(SPA_ERR_INVALID, "a pool with head_slots < num_kv_heads needs the head kinds");
    if (stream_base < 0 && has_streaming(heads, pl.hkv))
      return fail(SPA_ERR_INVALID, "a pool with head_slots < num_kv_heads keeps streaming heads in rings: "
                  "stream_base < 0");
  }
  if (stream_base >= 0) {
    if (!heads) return fail(SPA_ERR_INVALID, "stream_base needs the head kinds (heads is NULL)");
    ring_geometry(heads, pl.P, &ring_sink, &ring_win);
    if ((int64_t)stream_base + ring_sink + ring_win > pl.N)
      return fail(SPA_ERR_INVALID, "ring [%d, %d) exceeds the pool's %d pages", stream_base,
                  stream_base + ring_sink + ring_win, pl.N);
  }
  if (count == 0) return ok();
  if (!page_table_row || !k || !v) return fail(SPA_ERR_INVALID, "page_table_row / k / v is NULL");
  return hip_status(spa::launch_write(pl, page_table_row, start, count, static_cast<const uint16_t*>(k),
                                      static_cast<const uint16_t*>(v), heads ? &dyn : nullptr,
                                      stream_base >= 0 ? stream_base : -1, ring_sink, ring_win, stream),
                    "kv_pool_write launch");
}

spa_status spa_page_summary_update(const spa_pool* pool, const spa_heads* heads, const spa_batch* batch,
                                   const int32_t* first_pos, int32_t max_tokens, hipStream_t stream) {
  spa::PoolArgs pl;
  spa::BatchArgs bt;
  spa::HeadList dyn;
  int32_t G;
  spa_status s;
  if ((s = check_pool(pool, &pl)) != SPA_OK) return s;
  if ((s = check_heads(heads, pl, &G, &dyn, nullptr)) != SPA_OK) return s;
  if ((s = check_batch(batch, pl, &bt)) != SPA_OK) return s;
  if ((s = set_ring(heads, pl, &bt)) != SPA_OK) return s;
  if (max_tokens < 1) return fail(SPA_ERR_INVALID, "max_tokens %d < 1", max_tokens);
  if (!first_pos && max_tokens != 1) return fail(SPA_ERR_INVALID, "first_pos NULL requires max_tokens == 1");
  if ((int64_t)max_tokens > (int64_t)bt.max_pp * pl.P)
    return fail(SPA_ERR_INVALID, "max_tokens %d exceeds max_pages * physical_page", max_tokens);
  if (bt.B == 0 || dyn.n == 0) return ok();
  return hip_status(spa::launch_summary(pl, bt, dyn, first_pos, max_tokens, stream), "page_summary_update launch");
}

size_t spa_workspace_bytes(const spa_pool* pool, const spa_heads* heads, int32_t batch, int32_t max_pages,
                           int32_t k_max) {
  spa::PoolArgs pl;
  spa::HeadList dyn;
  int32_t G;
  uint8_t kind[spa::kMaxKvHeads];
  const std::string keep = g_last_error;
  size_t bytes = 0;
  if (check_pool(pool, &pl) == SPA_OK && check_heads(heads, pl, &G, &dyn, kind) == SPA_OK &&
      batch >= 0 && max_pages >= 1 && k_max >= 1) {
    spa::AttnPlan plan;
    plan_attention(pl, heads, k_max, kind, -1, &plan);
    size_t ml_off;
    bytes = std::max(attn_bytes(pl, plan, batch, G, &ml_off), select_bytes(pl, batch, max_pages));
    bytes = std::max<size_t>(bytes, 256);
  }
  g_last_error = keep;
  return bytes;
}

namespace {

// Shared by the selection entry points; k_new / v_new NULL: no token appended.
spa_status select_pages(const spa_pool* pool, const spa_heads* heads, const spa_batch* batch, const void* k_new,
                        const void* v_new, const void* q, const int32_t* budget_tokens, int32_t k_max,
                        int32_t* sel_pages, int32_t* sel_count, int32_t* sel_len, int32_t* sel_phys,
                        float* scores, void* ws, size_t ws_bytes, hipStream_t stream, const char* what) {
  spa::PoolArgs pl;
  spa::BatchArgs bt;
  spa::HeadList dyn;
  int32_t G;
  spa_status s;
  if ((s = check_pool(pool, &pl)) != SPA_OK) return s;
  if ((s = check_heads(heads, pl, &G, &dyn, nullptr)) != SPA_OK) return s;
  if ((s = check_batch(batch, pl, &bt)) != SPA_OK) return s;
  if ((s = set_ring(heads, pl, &bt)) != SPA_OK) return s;
  if (k_max < 1) return fail(SPA_ERR_INVALID, "k_max %d < 1", k_max);
  const int32_t n_max = n_max_pages(pl, bt.max_pp);
  if (n_max > kMaxScoredPages)
    return fail(SPA_ERR_UNSUPPORTED, "max_pages * P / p = %d logical pages exceeds %lld", n_max,
                (long long)kMaxScoredPages);
  if ((int64_t)bt.B * dyn.n > 2147483647LL / 1) return fail(SPA_ERR_INVALID, "too many heads");
  if (bt.B == 0) return ok();
  const bool fresh = k_new != nullptr || v_new != nullptr;
  if (fresh && (!k_new || !v_new)) return fail(SPA_ERR_INVALID, "k_new / v_new is NULL");
  float* sc = scores;
  if (dyn.n > 0) {
    if (!q || !budget_tokens || !sel_pages || !sel_count || !sel_len)
      return fail(SPA_ERR_INVALID, "q / budget_tokens / sel_pages / sel_count / sel_len is NULL");
    if (!sc) {
      const size_t need = select_bytes(pl, bt.B, bt.max_pp);
      if (!ws || ws_bytes < need)
        return fail(SPA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, need);
      sc = static_cast<float*>(ws);
    }
  }
  if (dyn.n == 0)                   // nothing to select: the append alone
    return fresh ? hip_status(spa::launch_select(pl, bt, dyn, G, nullptr, nullptr, k_max, nullptr, nullptr,
                                                 nullptr, nullptr, nullptr, n_max,
                                                 static_cast<const uint16_t*>(k_new),
                                                 static_cast<const uint16_t*>(v_new), stream),
                              what)
                 : ok();
  return hip_status(spa::launch_select(pl, bt, dyn, G, static_cast<const uint16_t*>(q), budget_tokens, k_max,
                                       sel_pages, sel_count, sel_len, sel_phys, sc, n_max,
                                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                                       stream),
                    what);
}

}  // namespace

spa_status spa_select_pages(const spa_pool* pool, const spa_heads* heads, const spa_batch* batch,
                            const void* q, const int32_t* budget_tokens, int32_t k_max,
                            int32_t* sel_pages, int32_t* sel_count, int32_t* sel_len, int32_t* sel_phys,
                            float* scores, void* ws, size_t ws_bytes, hipStream_t stream) {
  return select_pages(pool, heads, batch, nullptr, nullptr, q, budget_tokens, k_max, sel_pages, sel_count, sel_len,
                      sel_phys, scores, ws, ws_bytes, stream, "select_pages launch");
}

spa_status spa_append_select_pages(const spa_pool* pool, const spa_heads* heads, const spa_batch* batch,
                                   const void* k_new, const void* v_new, const void* q,
                                   const int32_t* budget_tokens, int32_t k_max, int32_t* sel_pages,
                                   int32_t* sel_count, int32_t* sel_len, int32_t* sel_phys, float* scores,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
  if (batch && batch->batch > 0 && (!k_new || !v_new)) return fail(SPA_ERR_INVALID, "k_new / v_new is NULL");
  return select_pages(pool, heads, batch, k_new, v_new, q, budget_tokens, k_max, sel_pages, sel_count, sel_len,
                      sel_phys, scores, ws, ws_bytes, stream, "append_select_pages launch");
}

namespace {

// Shared by the attention entry points; k_new / v_new NULL: no token appended.
spa_status decode_attn(const spa_pool* pool, const spa_heads* heads, const spa_batch* batch, const void* k_new,
                       const void* v_new, const void* q, const int32_t* sel_pages, const int32_t* sel_count,
                       const int32_t* sel_len, const int32_t* sel_phys, int32_t k_max, float* out, float* lse,
                       void* ws, size_t ws_bytes, hipStream_t stream, const char* what,
                       bool use_scratch = false) {
  spa::PoolArgs pl;
  spa::BatchArgs bt;
  spa::HeadList dyn;
  int32_t G;
  uint8_t kind[spa::kMaxKvHeads];
  spa_status s;
  if ((s = check_pool(pool, &pl)) != SPA_OK) return s;
  if ((s = check_heads(heads, pl, &G, &dyn, kind)) != SPA_OK) return s;
  if ((s = check_batch(batch, pl, &bt)) != SPA_OK) return s;
  if ((s = set_ring(heads, pl, &bt)) != SPA_OK) return s;
  if (k_max < 1) return fail(SPA_ERR_INVALID, "k_max %d < 1", k_max);
  if (bt.B == 0) return ok();
  if (!q || !out) return fail(SPA_ERR_INVALID, "q / out is NULL");
  if (dyn.n > 0 && (!sel_pages || !sel_count || !sel_len))
    return fail(SPA_ERR_INVALID, "dynamic heads need sel_pages / sel_count / sel_len");
  spa::AttnPlan plan;
  plan_attention(pl, heads, k_max, kind, bt.B, &plan);
  if ((int64_t)bt.B * plan.items_per_seq + (int64_t)bt.B * pl.hkv > INT32_MAX)
    return fail(SPA_ERR_INVALID, "grid too large");
  plan.sel_mask = dyn.n > 0 ? ~int64_t(0) : 0;
  plan.use_phys = dyn.n > 0 && sel_phys != nullptr;
  if (dyn.n == 0) {                 // never used; read at index 0 to keep the loads branch-free
    sel_pages = bt.lens;
    sel_count = bt.lens;
    sel_len = bt.lens;
  }
  if (!plan.use_phys) sel_phys = sel_pages;     // read alongside the ids, never used
  size_t ml_off;
  const size_t need = attn_bytes(pl, plan, bt.B, G, &ml_off);
  if (use_scratch) {                // the library's static scratch in place of a workspace
    const hipError_t e = spa::scratch_area(&ws, &ws_bytes);
    if (e != hipSuccess) return hip_status(e, "scratch address");
    if (ws_bytes < need)
      return fail(SPA_ERR_WORKSPACE, "these shapes need %zu bytes of scratch; the library's static scratch "
                  "holds %zu (use spa_sparse_decode_attn with a workspace)", need, ws_bytes);
  }
  if (!ws || ws_bytes < need) return fail(SPA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, need);
  float* part_o = static_cast<float*>(ws);
  float* part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + ml_off);
  return hip_status(spa::launch_attn(pl, bt, plan, G, static_cast<const uint16_t*>(q), sel_pages, sel_count,
                                     sel_len, sel_phys, out, lse, part_o, part_ml,
                                     static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                                     stream),
                    what);
}

}  // namespace

spa_status spa_sparse_decode_attn(const spa_pool* pool, const spa_heads* heads, const spa_batch* batch,
                                  const void* q, const int32_t* sel_pages, const int32_t* sel_count,
                                  const int32_t* sel_len, const int32_t* sel_phys, int32_t k_max, float* out,
                                  float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  return decode_attn(pool, heads, batch, nullptr, nullptr, q, sel_pages, sel_count, sel_len, sel_phys, k_max, out,
                     lse, ws, ws_bytes, stream, "sparse_decode_attn launch");
}

spa_status spa_sparse_decode_attn_noalloc(const spa_pool* pool, const spa_heads* heads, const spa_batch* batch,
                                          const void* q, const int32_t* sel_pages, const int32_t* sel_count,
                                          const int32_t* sel_len, const int32_t* sel_phys, int32_t k_max,
                                          float* out, float* lse, hipStream_t stream) {
  return decode_attn(pool, heads, batch, nullptr, nullptr, q, sel_pages, sel_count, sel_len, sel_phys, k_max, out,
                     lse, nullptr, 0, stream, "sparse_decode_attn_noalloc launch", true);
}

spa_status spa_append_decode_attn(const spa_pool* pool, const spa_heads* heads, const spa_batch* batch,
                                  const void* k_new, const void* v_new, const void* q, const int32_t* sel_pages,
                                  const int32_t* sel_count, const int32_t* sel_len, const int32_t* sel_phys,
                                  int32_t k_max, float* out, float* lse, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  if (batch && batch->batch > 0 && (!k_new || !v_new)) return fail(SPA_ERR_INVALID, "k_new / v_new is NULL");
  return decode_attn(pool, heads, batch, k_new, v_new, q, sel_pages, sel_count, sel_len, sel_phys, k_max, out,
                     lse, ws, ws_bytes, stream, "append_decode_attn launch");
}

// ------------------------------------------------------------- prefill

namespace {

struct PrefillPlan {
  int32_t G, nb, kb, sparse, any_dynamic;
  uint32_t dyn_mask[spa::kMaxKvHeads / 32];
  size_t qp_off, kp_off, sel_off, cnt_off, bytes;
};

spa_status check_prefill(const spa_heads* heads, int32_t hkv, const spa_prefill* cfg, int64_t L,
                         PrefillPlan* pp) {
  if (!cfg) return fail(SPA_ERR_INVALID, "cfg is NULL");
  if (hkv < 1 || hkv > spa::kMaxKvHeads) return fail(SPA_ERR_INVALID, "num_kv_heads %d outside [1, %d]", hkv,
                                                     spa::kMaxKvHeads);
  if (cfg->head_dim != spa::kHeadDim)
    return fail(cfg->head_dim < 1 ? SPA_ERR_INVALID : SPA_ERR_UNSUPPORTED, "head_dim %d: only 128 is built",
                cfg->head_dim);
  if (cfg->block != spa::kPrefillBlock)
    return fail(cfg->block < 1 ? SPA_ERR_INVALID : SPA_ERR_UNSUPPORTED, "block %d: only 64 is built",
                cfg->block);
  if (cfg->budget < 1) return fail(SPA_ERR_INVALID, "budget %d < 1", cfg->budget);
  if (L < 0) return fail(SPA_ERR_INVALID, "seq_len %lld < 0", (long long)L);
  if (L > ((int64_t)1 << 31) / spa::kHeadDim) return fail(SPA_ERR_UNSUPPORTED, "seq_len %lld too long", (long long)L);
  spa::PoolArgs pl{};
  pl.hkv = hkv;
  pl.hs = hkv;
  pl.summ = reinterpret_cast<uint16_t*>(1);       // summaries are not used here
  spa::HeadList dyn;
  uint8_t kind[spa::kMaxKvHeads];
  int32_t G;
  spa_status s;
  if ((s = check_heads(heads, pl, &G, &dyn, kind)) != SPA_OK) return s;
  std::memset(pp, 0, sizeof *pp);
  pp->G = G;
  pp->nb = (int32_t)((L + spa::kPrefillBlock - 1) / spa::kPrefillBlock);
  pp->kb = std::max(1, cfg->budget / spa::kPrefillBlock);
  pp->kb = std::min(pp->kb, std::max(pp->nb, 1));
  pp->any_dynamic = dyn.n > 0;
  for (int32_t h = 0; h < hkv; ++h)
    if (kind[h]) pp->dyn_mask[h / 32] |= 1u << (h % 32);
  pp->sparse = dyn.n > 0 && L >= cfg->dense_below;
  if (pp->sparse && pp->nb > spa::kPrefillMaxBlocks)
    return fail(SPA_ERR_UNSUPPORTED, "seq_len %lld: selection rows hold at most %d blocks of 64", (long long)L,
                spa::kPrefillMaxBlocks);
  size_t o = 0;
  if (pp->sparse) {
    const size_t proj = (size_t)hkv * pp->nb * (spa::kHeadDim / 8) * sizeof(double);
    pp->qp_off = o; o = align_up(o + proj);
    pp->kp_off = o; o = align_up(o + proj);
    pp->sel_off = o; o = align_up(o + (size_t)hkv * pp->nb * pp->kb * sizeof(int32_t));
    pp->cnt_off = o; o = align_up(o + (size_t)hkv * pp->nb * sizeof(int32_t));
  }
  pp->bytes = std::max<size_t>(o, 256);
  return SPA_OK;
}

}  // namespace

size_t spa_prefill_workspace_bytes(const spa_heads* heads, int32_t num_kv_heads, const spa_prefill* cfg,
                                   int64_t seq_len) {
  const std::string keep = g_last_error;
  PrefillPlan pp;
  const size_t n = check_prefill(heads, num_kv_heads, cfg, seq_len, &pp) == SPA_OK ? pp.bytes : 0;
  g_last_error = keep;
  return n;
}

spa_status spa_prefill_attn(const spa_heads* heads, int32_t num_kv_heads, const spa_prefill* cfg, int64_t seq_len,
                            const void* q, const void* k, const void* v, const void* w_q, const void* w_k,
                            float* out, float* lse, int32_t* sel_blocks, int32_t* sel_count, float* block_scores,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  PrefillPlan pp;
  spa_status s;
  if ((s = check_prefill(heads, num_kv_heads, cfg, seq_len, &pp)) != SPA_OK) return s;
  if (seq_len == 0) return ok();
  if (!q || !k || !v || !out) return fail(SPA_ERR_INVALID, "q / k / v / out is NULL");
  if (pp.sparse && (!w_q || !w_k)) return fail(SPA_ERR_INVALID, "w_q / w_k is NULL (the dynamic heads select)");
  if (!ws || ws_bytes < pp.bytes) return fail(SPA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes,
                                              pp.bytes);
  spa::PrefillArgs a{};
  a.hq = heads->num_q_heads;
  a.hkv = num_kv_heads;
  a.G = pp.G;
  a.L = seq_len;
  a.nb = pp.nb;
  a.kb = pp.kb;
  a.sink = heads->sink;
  a.window = heads->window;
  a.dense = !pp.sparse;
  a.any_dynamic = pp.any_dynamic;
  std::memcpy(a.dyn_mask, pp.dyn_mask, sizeof a.dyn_mask);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.wq = static_cast<const uint16_t*>(w_q);
  a.wk = static_cast<const uint16_t*>(w_k);
  char* w = static_cast<char*>(ws);
  a.qp = reinterpret_cast<double*>(w + pp.qp_off);
  a.kp = reinterpret_cast<double*>(w + pp.kp_off);
  a.sel = sel_blocks ? sel_blocks : reinterpret_cast<int32_t*>(w + pp.sel_off);
  a.cnt = sel_count ? sel_count : reinterpret_cast<int32_t*>(w + pp.cnt_off);
  a.scores = block_scores;
  a.out = out;
  a.lse = lse;
  return hip_status(spa::launch_prefill(a, stream), "prefill_attn launch");
}

// ------------------------------------------------------------- allocator

struct spa_allocator {
  std::vector<int32_t> free_list;    // stack: back() is handed out next
  std::vector<uint8_t> in_use;
};

spa_status spa_alloc_create(int32_t num_pages, spa_allocator** out) {
  if (!out) return fail(SPA_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (num_pages < 1) return fail(SPA_ERR_INVALID, "num_pages %d < 1", num_pages);
  spa_allocator* a = new (std::nothrow) spa_allocator;
  if (!a) return fail(SPA_ERR_INVALID, "out of host memory");
  a->free_list.resize(num_pages);
  for (int32_t i = 0; i < num_pages; ++i) a->free_list[i] = num_pages - 1 - i;   // lowest id on top
  a->in_use.assign(num_pages, 0);
  *out = a;
  return ok();
}

spa_status spa_alloc_pages(spa_allocator* a, int32_t count, int32_t* ids_out) {
  if (!a) return fail(SPA_ERR_INVALID, "allocator is NULL");
  if (count < 0) return fail(SPA_ERR_INVALID, "count %d < 0", count);
  if (count > 0 && !ids_out) return fail(SPA_ERR_INVALID, "ids_out is NULL");
  if ((size_t)count > a->free_list.size())
    return fail(SPA_ERR_POOL_EXHAUSTED, "No free pages available: %d requested, %zu free", count,
                a->free_list.size());
  for (int32_t i = 0; i < count; ++i) {
    const int32_t id = a->free_list.back();
    a->free_list.pop_back();
    a->in_use[id] = 1;
    ids_out[i] = id;
  }
  return ok();
}

spa_status spa_alloc_free(spa_allocator* a, int32_t count, const int32_t* ids) {
  if (!a) return fail(SPA_ERR_INVALID, "allocator is NULL");
  if (count < 0) return fail(SPA_ERR_INVALID, "count %d < 0", count);
  if (count > 0 && !ids) return fail(SPA_ERR_INVALID, "ids is NULL");
  std::vector<uint8_t> seen;
  for (int32_t i = 0; i < count; ++i) {
    const int32_t id = ids[i];
    if (id < 0 || (size_t)id >= a->in_use.size()) return fail(SPA_ERR_INVALID, "page id %d out of range", id);
    if (!a->in_use[id]) return fail(SPA_ERR_INVALID, "page %d is not allocated", id);
    if (seen.empty()) seen.assign(a->in_use.size(), 0);
    if (seen[id]) return fail(SPA_ERR_INVALID, "page %d freed twice in one call", id);
    seen[id] = 1;
  }
  for (int32_t i = 0; i < count; ++i) {
    a->in_use[ids[i]] = 0;
    a->free_list.push_back(ids[i]);
  }
  return ok();
}

int32_t spa_alloc_num_free(const spa_allocator* a) { return a ? (int32_t)a->free_list.size() : -1; }

void spa_alloc_destroy(spa_allocator* a) { delete a; }

}  // extern "C"
