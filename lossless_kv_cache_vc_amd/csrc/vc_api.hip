// Host side of the C ABI: argument validation, launch planning and the exported entry points.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "vc_internal.h"

namespace vc {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

int fail(int code, const std::string& msg) {
  set_error(msg);
  return code;
}

int hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return VC_OK;
  return fail(VC_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

// The device error word: [flag, page-table row, logical page, entry].  Each device holds its own
// copy of the array; its address is looked up once per device.
static __device__ __attribute__((aligned(16))) int32_t g_error_word[4];

constexpr int kMaxDevices = 64;
static std::mutex g_word_mu;
static int32_t* g_word_ptr[kMaxDevices];

int32_t* device_error_word() {
  int dev = 0;
  if (hip_check(hipGetDevice(&dev), "hipGetDevice")) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    fail(VC_EUNSUPPORTED, "device index beyond the library's table");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_word_mu);
  if (!g_word_ptr[dev]) {
    void* p = nullptr;
    if (hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(g_error_word)), "hipGetSymbolAddress")) return nullptr;
    g_word_ptr[dev] = static_cast<int32_t*>(p);
  }
  return g_word_ptr[dev];
}

static int check_shape(const vc_shape* s) {
  if (!s) return fail(VC_EINVAL, "shape is NULL");
  if (s->num_layers < 1 || s->num_q_heads < 1 || s->num_kv_heads < 1)
    return fail(VC_EINVAL, "layers and head counts must be >= 1");
  if (s->num_q_heads % s->num_kv_heads)
    return fail(VC_EINVAL, "num_q_heads must be a multiple of num_kv_heads");
  if (s->num_q_heads / s->num_kv_heads > 16)
    return fail(VC_EUNSUPPORTED, "more than 16 query heads per kv head");
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(VC_EUNSUPPORTED, "head_dim must be 64 or 128");
  if (s->max_rows < 16 || s->max_rows > VC_MAX_ROWS || s->max_rows % 16)
    return fail(VC_EINVAL, "max_rows must be a multiple of 16 in [16, 64]");
  return VC_OK;
}

static int check_pool(const vc_pool* p, int head_dim, int num_layers, int num_kv_heads, const char* name) {
  char buf[160];
  if (!p) {
    snprintf(buf, sizeof buf, "%s pool is NULL", name);
    return fail(VC_EINVAL, buf);
  }
  if (p->bits != 16 && p->bits != 2 && p->bits != 4) {
    snprintf(buf, sizeof buf, "%s pool: bits must be 16, 2 or 4 (got %d)", name, p->bits);
    return fail(VC_EINVAL, buf);
  }
  if (!p->page_table || !p->k || !p->v) {
    snprintf(buf, sizeof buf, "%s pool: page_table, k and v must be set", name);
    return fail(VC_EINVAL, buf);
  }
  if (p->bits != 16 && (!p->k_sz || !p->v_sz)) {
    snprintf(buf, sizeof buf, "%s pool: KIVI pools need k_sz and v_sz", name);
    return fail(VC_EINVAL, buf);
  }
  if (p->num_blocks < 1 || p->max_pages < 1) {
    snprintf(buf, sizeof buf, "%s pool: num_blocks and max_pages must be >= 1", name);
    return fail(VC_EINVAL, buf);
  }
  // the kernels index (layer, block, kv head) page units with 32-bit integers
  if ((int64_t)num_layers * p->num_blocks * num_kv_heads >= (1LL << 31)) {
    snprintf(buf, sizeof buf, "%s pool: layers x blocks x kv heads must be below 2^31", name);
    return fail(VC_EUNSUPPORTED, buf);
  }
  // the KIVI draft ring addresses a pool's pages of one (layer, kv head) with 32-bit byte offsets
  if (p->bits != 16) {
    const int64_t page_bytes = std::max<int64_t>((int64_t)kBlock * head_dim * p->bits / 8, 4LL * head_dim);
    if ((int64_t)p->num_blocks * num_kv_heads * page_bytes >= (1LL << 32)) {
      snprintf(buf, sizeof buf, "%s pool: blocks x kv heads x page code bytes must be below 2^32", name);
      return fail(VC_EUNSUPPORTED, buf);
    }
  }
  return VC_OK;
}

static PoolDev to_dev(const vc_pool& p) {
  PoolDev d;
  d.k = static_cast<const uint8_t*>(p.k);
  d.v = static_cast<const uint8_t*>(p.v);
  d.ksz = static_cast<const uint8_t*>(p.k_sz);
  d.vsz = static_cast<const uint8_t*>(p.v_sz);
  d.page_table = p.page_table;
  d.nblk = p.num_blocks;
  d.max_pages = p.max_pages;
  d.bits = p.bits;
  return d;
}

// Verify-only launches whose largest request has more than 128 query rows (rows x G) per
// (layer, kv head) use the wide verify: those rows are cut into as few groups of at most
// 32 * kWideMaxWaves as possible, and the work-group has one wave per 32 rows of a group.
static int plan_vwaves(int G, int nreq, const vc_req* reqs) {
  int64_t maxrows = 0;
  for (int i = 0; i < nreq; ++i) {
    if (reqs[i].kind != VC_VERIFY) return 0;
    maxrows = std::max<int64_t>(maxrows, (int64_t)reqs[i].rows * G);
  }
  if (maxrows <= 128 || maxrows > (1 << 20)) return 0;  // (bad row counts are rejected later)
  const int64_t cap = 32 * kWideMaxWaves;
  const int64_t groups = (maxrows + cap - 1) / cap;
  const int64_t per = (maxrows + groups - 1) / groups;
  return (int)((per + 31) / 32);
}

// The launch holds drafting and verifying requests (it runs the mixed kernel).
static bool is_mixed(int nreq, const vc_req* reqs) {
  bool has_v = false, has_d = false;
  for (int i = 0; i < nreq; ++i) (reqs[i].kind == VC_VERIFY ? has_v : has_d) = true;
  return has_v && has_d;
}

static int64_t row_groups(const vc_req& r, int G, int vwaves) {
  if (r.kind != VC_VERIFY) return 1;
  const int64_t per = vwaves ? 32 * vwaves : 128;
  return ((int64_t)r.rows * G + per - 1) / per;
}

static int auto_chunk(const vc_shape* s, int nreq, const vc_req* reqs, int vwaves) {
  // aim for about 2048 work items (8 per CU) so the 256 CUs see several waves of work-groups;
  // a launch that mixes drafting and verifying requests aims for about 1024 (4 per CU): its
  // items' fixed costs (page-table load, ring fill and drain, split partials) outweigh the
  // finer balance (64-request ragged batch, 32K mean context: 0.93-0.95 ms against 0.97-1.01)
  const int G = s->num_q_heads / s->num_kv_heads;
  int64_t total = 0;
  for (int i = 0; i < nreq; ++i) {
    const int pages = (reqs[i].ctx_len + kBlock - 1) / kBlock;
    total += (int64_t)s->num_layers * s->num_kv_heads * row_groups(reqs[i], G, vwaves) * pages;
  }
  const int64_t target = is_mixed(nreq, reqs) ? 1024 : 2048;
  int64_t chunk = (total + target - 1) / target;
  chunk = std::max<int64_t>(16, (chunk + 3) / 4 * 4);
  return (int)std::min<int64_t>(chunk, 1 << 28);
}

int plan_attn(const vc_shape* s, int nreq, const vc_req* reqs, int npools, const vc_pool* pools,
              int split_pages, AttnArgs* args, Plan* plan, std::vector<ReqDev>* table) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (nreq < 0 || nreq > VC_MAX_REQS) return fail(VC_EINVAL, "num_reqs must be in [0, 1024]");
  if (nreq > 0 && !reqs) return fail(VC_EINVAL, "reqs is NULL");
  if (npools < 1 || npools > kMaxPools) return fail(VC_EINVAL, "num_pools must be in [1, 4]");
  if (split_pages < 0 || split_pages % 4) return fail(VC_EINVAL, "split_pages must be a multiple of 4");
  const int G = s->num_q_heads / s->num_kv_heads;
  const int D = s->head_dim;
  memset(args, 0, sizeof(*args));
  for (int i = 0; i < npools; ++i) args->pools[i] = to_dev(pools[i]);
  std::vector<char> pool_used(npools, 0);
  const int vwaves = plan_vwaves(G, nreq, reqs);
  const int chunk = split_pages > 0 ? split_pages : auto_chunk(s, nreq, reqs, vwaves);
  plan->any_split = 0;
  plan->has_verify = plan->has_draft = 0;
  plan->draft_bits = 0;
  table->assign(nreq, ReqDev{});
  std::vector<double> item_cost(nreq, 0.0);
  for (int i = 0; i < nreq; ++i) {
    const vc_req& r = reqs[i];
    char buf[200];
    if (r.kind != VC_VERIFY && r.kind != VC_DRAFT) {
      snprintf(buf, sizeof buf, "request %d: kind must be VC_VERIFY or VC_DRAFT", i);
      return fail(VC_EINVAL, buf);
    }
    if (r.pool < 0 || r.pool >= npools) {
      snprintf(buf, sizeof buf, "request %d: pool index %d out of range", i, r.pool);
      return fail(VC_EINVAL, buf);
    }
    if (r.slot < 0 || r.ctx_len < 0 || r.page_row < 0 || r.q0 < 0 || r.rows < 1 ||
        r.q0 + r.rows > s->max_rows) {
      snprintf(buf, sizeof buf, "request %d: bad slot/ctx_len/page_row/q0/rows", i);
      return fail(VC_EINVAL, buf);
    }
    if (r.kind == VC_DRAFT && r.rows * G > 16) {
      snprintf(buf, sizeof buf, "request %d: a draft step needs rows * G <= 16", i);
      return fail(VC_EINVAL, buf);
    }
    const vc_pool& p = pools[r.pool];
    if (!pool_used[r.pool]) {
      rc = check_pool(&p, D, s->num_layers, s->num_kv_heads, "attention");
      if (rc) return rc;
      pool_used[r.pool] = 1;
    }
    if (r.kind == VC_VERIFY && p.bits != 16) {
      snprintf(buf, sizeof buf, "request %d: the verify pass reads a bf16 pool", i);
      return fail(VC_EINVAL, buf);
    }
    const int pages = (r.ctx_len + kBlock - 1) / kBlock;
    if (pages > p.max_pages) {
      snprintf(buf, sizeof buf, "request %d: %d pages exceed the page table width %d", i, pages,
               p.max_pages);
      return fail(VC_EINVAL, buf);
    }
    (r.kind == VC_VERIFY ? plan->has_verify : plan->has_draft) = 1;
    if (r.kind == VC_DRAFT) plan->draft_bits = (plan->draft_bits == 0 || plan->draft_bits == p.bits) ? p.bits : -1;
    ReqDev& d = (*table)[i];
    d.slot = r.slot;
    d.pool = r.pool;
    d.ctx_len = r.ctx_len;
    d.page_row = r.page_row;
    d.q0 = r.q0;
    d.rows = r.rows;
    d.kind = r.kind;
    const int target = std::min(chunk, kMaxChunkPages);
    d.chunk_pages = split_context(pages, target, &d.nsplit);
    d.nrg = (int32_t)row_groups(r, G, vwaves);
    // bytes one of the request's items streams: its pages times the bytes of a page of its pool
    // (bf16 K and V, or 2/4-bit codes with their scales and zeros)
    const double page_bytes = p.bits == 16 ? 64.0 * D : (p.bits == 2 ? 12.0 : 20.0) * D;
    item_cost[i] = std::min(pages, d.chunk_pages) * page_bytes;
  }
  // Item numbering follows the table order.  In a ragged batch that mixes drafting and verifying
  // requests the table lists requests by decreasing cost per item, so the most expensive items
  // are dispatched first and the launch does not end on a tail of long items (longest processing
  // time first); other launches keep the caller's order.  Nothing outside the plan depends on the
  // order: each entry carries its request's own slot, rows and page-table row.
  std::vector<int> order(nreq);
  for (int i = 0; i < nreq; ++i) order[i] = i;
  if (is_mixed(nreq, reqs))
    std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return item_cost[x] > item_cost[y]; });
  {
    std::vector<ReqDev> sorted(nreq);
    for (int j = 0; j < nreq; ++j) sorted[j] = (*table)[order[j]];
    table->swap(sorted);
  }
  int64_t items = 0, part = 0, merge = 0;
  for (int j = 0; j < nreq; ++j) {
    ReqDev& d = (*table)[j];
    d.item_base = (int32_t)items;
    items += (int64_t)s->num_layers * s->num_kv_heads * d.nsplit * d.nrg;
    // merge work-groups are counted for every request (a request without splits owns none), so
    // merge_base ascends and the merge kernel finds a work-group's request like an item's
    d.merge_base = (int32_t)std::min<int64_t>(merge, INT32_MAX);
    if (d.nsplit > 1) {
      d.part_base = part;
      part += (int64_t)s->num_layers * s->num_kv_heads * d.nsplit * d.rows * G * (D + 4);
      const int64_t rows = (int64_t)s->num_layers * s->num_kv_heads * d.rows * G;
      const int rpg = merge_rows_per_group(D);
      merge += (rows + rpg - 1) / rpg;
      plan->any_split = 1;
    } else {
      d.part_base = -1;
    }
    if (items > (1LL << 30)) return fail(VC_EINVAL, "too many work items");
  }
  if (items > (1LL << 30)) return fail(VC_EINVAL, "too many work items");
  if (merge > (1LL << 30)) return fail(VC_EINVAL, "too many split rows");
  for (int i = 0; i < std::min(nreq, kInlineReqs); ++i) args->reqs[i] = (*table)[i];
  args->L = s->num_layers;
  args->Hq = s->num_q_heads;
  args->Hkv = s->num_kv_heads;
  args->G = G;
  args->xmax = s->max_rows;
  args->nreq = nreq;
  args->nitems = (int)items;
  args->nitems_pad = (int)((items + 7) / 8 * 8);
  args->scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
  args->vwaves = vwaves;
  // a launch mixing drafting and verifying requests is a ragged batch: spread every request over
  // the XCDs (64-request batch: 0.91-0.92 ms against 0.94-0.95 with XCD ranges)
  args->xcd_ranges = is_mixed(nreq, reqs) ? 0 : 1;
  args->nmerge = (int32_t)merge;
  plan->nitems = (int)items;
  plan->vwaves = vwaves;
  plan->part_floats = part;
  plan->head_dim = D;
  return VC_OK;
}

static int attn_common(const vc_shape* s, int nreq, const vc_req* reqs, const void* q,
                       const void* blk_k, const void* blk_v, int npools, const vc_pool* pools,
                       float* out, void* ws, size_t ws_bytes, int split_pages, void* stream) {
  AttnArgs args;
  Plan plan;
  std::vector<ReqDev> table;
  int rc = plan_attn(s, nreq, reqs, npools, pools, split_pages, &args, &plan, &table);
  if (rc) return rc;
  if (nreq == 0 || plan.nitems == 0) return VC_OK;
  if (!q || !blk_k || !blk_v || !out) return fail(VC_EINVAL, "q, blk_k, blk_v and out must be set");
  // workspace: [request table (more than kInlineReqs requests)][split partials]
  const size_t tbytes = req_table_bytes(nreq);
  const size_t need = tbytes + (size_t)plan.part_floats * sizeof(float);
  if (need > 0 && (!ws || ws_bytes < need)) {
    char buf[160];
    snprintf(buf, sizeof buf, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
    return fail(VC_ENOSPACE, buf);
  }
  if (need > 0 && reinterpret_cast<uintptr_t>(ws) % 16)
    return fail(VC_EINVAL, "workspace must be 16-byte aligned");
  args.err = device_error_word();
  if (!args.err) return VC_EHIP;
  args.q = static_cast<const uint16_t*>(q);
  args.blk_k = static_cast<const uint16_t*>(blk_k);
  args.blk_v = static_cast<const uint16_t*>(blk_v);
  args.out = out;
  args.part = need > tbytes ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + tbytes) : nullptr;
  args.reqs_dev = nullptr;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (tbytes) {
    ReqDev* dtab = static_cast<ReqDev*>(ws);
    rc = upload_req_table(table, dtab, st);
    if (rc) return rc;
    args.reqs_dev = dtab;
  }
  return launch_attn(args, plan, s->head_dim, st);
}

}  // namespace vc

using namespace vc;

extern "C" {

const char* vc_last_error(void) { return g_last_error.c_str(); }

const char* vc_version(void) { return "vc 0.2 gfx950"; }

size_t vc_attn_workspace_size(const vc_shape* shape, int num_reqs, const vc_req* reqs,
                              int split_pages) {
  // pools are not needed for sizing: validate with a permissive dummy pool per index
  if (check_shape(shape)) return 0;
  if (num_reqs <= 0 || num_reqs > VC_MAX_REQS || !reqs) return 0;
  for (int i = 0; i < num_reqs; ++i)
    if (reqs[i].ctx_len < 0 || reqs[i].rows < 1 || reqs[i].rows > VC_MAX_ROWS) return 0;
  const int G = shape->num_q_heads / shape->num_kv_heads;
  const int chunk =
      split_pages > 0 ? split_pages : auto_chunk(shape, num_reqs, reqs, plan_vwaves(G, num_reqs, reqs));
  if (chunk <= 0) return 0;
  size_t floats = 0;
  for (int i = 0; i < num_reqs; ++i) {
    const int pages = (reqs[i].ctx_len + kBlock - 1) / kBlock;
    const int target = std::min(chunk, kMaxChunkPages);
    int nsplit;
    split_context(pages, target, &nsplit);
    if (nsplit > 1)
      floats += (size_t)shape->num_layers * shape->num_kv_heads * nsplit * reqs[i].rows * G *
                (shape->head_dim + 4);
  }
  return req_table_bytes(num_reqs) + floats * sizeof(float);
}

int vc_verify_attn(const vc_shape* shape, int num_reqs, const vc_req* reqs, const void* q,
                   const void* blk_k, const void* blk_v, const vc_pool* full, float* out,
                   void* workspace, size_t workspace_bytes, int split_pages, void* stream) {
  set_error("");
  if (num_reqs < 0 || num_reqs > VC_MAX_REQS) return fail(VC_EINVAL, "num_reqs must be in [0, 1024]");
  if (num_reqs > 0 && !reqs) return fail(VC_EINVAL, "reqs is NULL");
  if (!full) return fail(VC_EINVAL, "full pool is NULL");
  std::vector<vc_req> rr(reqs, reqs + num_reqs);
  for (vc_req& r : rr) {
    r.pool = 0;
    r.kind = VC_VERIFY;
  }
  return attn_common(shape, num_reqs, rr.data(), q, blk_k, blk_v, 1, full, out, workspace,
                     workspace_bytes, split_pages, stream);
}

int vc_draft_attn(const vc_shape* shape, int num_reqs, const vc_req* reqs, const void* q,
                  const void* blk_k, const void* blk_v, const vc_pool* comp, float* out,
                  void* workspace, size_t workspace_bytes, int split_pages, void* stream) {
  set_error("");
  if (num_reqs < 0 || num_reqs > VC_MAX_REQS) return fail(VC_EINVAL, "num_reqs must be in [0, 1024]");
  if (num_reqs > 0 && !reqs) return fail(VC_EINVAL, "reqs is NULL");
  if (!comp) return fail(VC_EINVAL, "compressed pool is NULL");
  std::vector<vc_req> rr(reqs, reqs + num_reqs);
  for (vc_req& r : rr) {
    r.pool = 0;
    r.kind = VC_DRAFT;
  }
  return attn_common(shape, num_reqs, rr.data(), q, blk_k, blk_v, 1, comp, out, workspace,
                     workspace_bytes, split_pages, stream);
}

int vc_attn_mixed(const vc_shape* shape, int num_reqs, const vc_req* reqs, const void* q,
                  const void* blk_k, const void* blk_v, int num_pools, const vc_pool* pools,
                  float* out, void* workspace, size_t workspace_bytes, int split_pages,
                  void* stream) {
  set_error("");
  if (!pools) return fail(VC_EINVAL, "pools is NULL");
  return attn_common(shape, num_reqs, reqs, q, blk_k, blk_v, num_pools, pools, out, workspace,
                     workspace_bytes, split_pages, stream);
}

// Kind of memory `p` points into: hipMemoryTypeHost (pinned host), hipMemoryTypeDevice, ..., or
// -1 for memory HIP does not know (pageable host memory; depending on the runtime version the
// query fails for it, and the error it leaves is cleared here).
static int memory_kind(const void* p) {
  hipPointerAttribute_t attr;
  memset(&attr, 0, sizeof attr);
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return -1;
  }
  return (int)attr.type;
}

int vc_stage_kv(void* dst_device, const void* src_pinned_host, size_t bytes, void* side_stream,
                void* event) {
  set_error("");
  hipStream_t st = static_cast<hipStream_t>(side_stream);
  if (bytes > 0) {
    if (!dst_device || !src_pinned_host) return fail(VC_EINVAL, "dst and src must be set");
    if (memory_kind(src_pinned_host) != (int)hipMemoryTypeHost)
      return fail(VC_EINVAL, "the staging source is not pinned host memory (hipHostMalloc): a pageable "
                             "source would make the copy synchronous");
    if (memory_kind(dst_device) != (int)hipMemoryTypeDevice)
      return fail(VC_EINVAL, "the staging destination is not device memory");
    const int rc = hip_check(hipMemcpyAsync(dst_device, src_pinned_host, bytes, hipMemcpyHostToDevice, st),
                             "hipMemcpyAsync");
    if (rc) return rc;
  }
  return event ? hip_check(hipEventRecord(static_cast<hipEvent_t>(event), st), "hipEventRecord") : VC_OK;
}

int vc_check_device(void* stream) {
  set_error("");
  int32_t* w = device_error_word();
  if (!w) return VC_EHIP;
  int rc = hip_check(hipStreamSynchronize(static_cast<hipStream_t>(stream)), "hipStreamSynchronize");
  if (rc) return rc;
  int32_t h[4] = {0, 0, 0, 0};
  rc = hip_check(hipMemcpy(h, w, sizeof h, hipMemcpyDeviceToHost), "hipMemcpy (error word)");
  if (rc) return rc;
  if (!h[0]) return VC_OK;
  const int32_t zero[4] = {0, 0, 0, 0};
  rc = hip_check(hipMemcpy(w, zero, sizeof zero, hipMemcpyHostToDevice), "hipMemcpy (error word)");
  if (rc) return rc;
  char buf[200];
  snprintf(buf, sizeof buf,
           "a kernel read page-table row %d, logical page %d: block id %d is outside [-1, num_blocks) "
           "(the page was treated as absent)", h[1], h[2], h[3]);
  return fail(VC_EDEVICE, buf);
}

}  // extern "C"
