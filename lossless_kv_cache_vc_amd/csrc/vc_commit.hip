// Committing accepted drafted rows into a bf16 pool (and the kept lists of a token-drop cache).
//
// VeriCache review, §Draft–Verify Pipeline, per-request cycle: drafting appends each drafted
// position's K/V, and at the first mismatch the cache is rolled back to the accepted position;
// after the verify the accepted positions' rows join the full cache.  Here the drafted block's
// K/V live in their own tensor until the accept is known, and only the accepted prefix is
// copied, so the rollback is the rows that are never copied.
#include "vc_internal.h"

namespace vc {

namespace {

constexpr int kMaxCommits = VC_MAX_BATCH;

struct CommitInfo {
  int32_t n;
  vc_commit c[kMaxCommits];
};

// job = (commit, layer, kv head): copy rows [0, count) of the block into the pool
template <int D>
__global__ __launch_bounds__(256) void commit_rows_kernel(CommitInfo ci, int L, int Hkv, int xmax,
                                                          const uint16_t* blk_k, const uint16_t* blk_v,
                                                          PoolDev pool, int32_t* kept, int64_t kstride,
                                                          int32_t* err) {
  const int job = blockIdx.x;
  const int g = job % Hkv, l = (job / Hkv) % L, i = job / (Hkv * L);
  const vc_commit cm = ci.c[i];
  // block pages of this (slot, layer, head): [xmax / 16][16][d] keys, [xmax / 16][d][16] values
  const int64_t bunit0 = (((int64_t)cm.slot * L + l) * Hkv + g) * (xmax / kBlock);
  // keys: one 16-byte chunk (8 channels) of one row per thread step
  for (int e = threadIdx.x; e < cm.count * (D / 8); e += blockDim.x) {
    const int j = e / (D / 8), c8 = e % (D / 8);
    const uint16_t* src = blk_k + (bunit0 + j / kBlock) * (kBlock * D) + (j % kBlock) * D + 8 * c8;
    const int pos = cm.pos + j;
    const int phys = pool.page_table[(int64_t)cm.page_row * pool.max_pages + pos / kBlock];
    if (phys < 0 || phys >= pool.nblk) {  // an unmapped page: nothing to write; a corrupt id is reported
      if (phys != -1) report_bad_page(err, cm.page_row, pos / kBlock, phys);
      continue;
    }
    const int64_t unit = ((int64_t)l * pool.nblk + phys) * Hkv + g;
    uint16_t* dst = reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(pool.k) + unit * (kBlock * D * 2)) +
                    (pos % kBlock) * D + 8 * c8;
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
  }
  // values: one element per thread step (channel-major pages on both sides)
  for (int e = threadIdx.x; e < cm.count * D; e += blockDim.x) {
    const int j = e / D, dd = e % D;
    const uint16_t v = blk_v[(bunit0 + j / kBlock) * (kBlock * D) + dd * kBlock + j % kBlock];
    const int pos = cm.pos + j;
    const int phys = pool.page_table[(int64_t)cm.page_row * pool.max_pages + pos / kBlock];
    if (phys < 0 || phys >= pool.nblk) {
      if (phys != -1) report_bad_page(err, cm.page_row, pos / kBlock, phys);
      continue;
    }
    const int64_t unit = ((int64_t)l * pool.nblk + phys) * Hkv + g;
    reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(pool.v) + unit * (kBlock * D * 2))[dd * kBlock + pos % kBlock] = v;
  }
  if (kept)
    for (int j = threadIdx.x; j < cm.count; j += blockDim.x)
      kept[(((int64_t)cm.slot * L + l) * Hkv + g) * kstride + cm.kept_len + j] = cm.pos + j;
}

}  // namespace

}  // namespace vc

using namespace vc;

extern "C" {

int vc_commit_rows(const vc_shape* shape, int num, const vc_commit* commits, const void* blk_k,
                   const void* blk_v, const vc_pool* pool, int32_t* kept, int64_t kept_stride,
                   void* stream) {
  set_error("");
  if (!shape) return fail(VC_EINVAL, "shape is NULL");
  const int L = shape->num_layers, Hkv = shape->num_kv_heads, d = shape->head_dim, xmax = shape->max_rows;
  if (L < 1 || Hkv < 1) return fail(VC_EINVAL, "bad shape");
  if (d != 64 && d != 128) return fail(VC_EUNSUPPORTED, "head_dim must be 64 or 128");
  if (xmax < kBlock || xmax > VC_MAX_ROWS || xmax % kBlock) return fail(VC_EINVAL, "max_rows must be 16, 32, 48 or 64");
  if (num < 0 || num > kMaxCommits) return fail(VC_EINVAL, "num must be in [0, 128]");
  if (num == 0) return VC_OK;
  if (!commits || !blk_k || !blk_v || !pool) return fail(VC_EINVAL, "NULL argument");
  if (pool->bits != 16 || !pool->k || !pool->v || !pool->page_table) return fail(VC_EINVAL, "commit writes a bf16 pool");
  CommitInfo ci;
  ci.n = num;
  for (int i = 0; i < num; ++i) {
    const vc_commit& c = commits[i];
    if (c.slot < 0 || c.page_row < 0) return fail(VC_EINVAL, "negative slot or page_row");
    if (c.count < 0 || c.count > xmax) return fail(VC_EINVAL, "count must be in [0, max_rows]");
    if (c.pos < 0 || (int64_t)c.pos + c.count > (int64_t)pool->max_pages * kBlock)
      return fail(VC_EINVAL, "positions beyond the page-table row");
    if (kept && (c.kept_len < 0 || (int64_t)c.kept_len + c.count > kept_stride))
      return fail(VC_EINVAL, "kept list too short");
    ci.c[i] = c;
  }
  PoolDev p = {static_cast<const uint8_t*>(pool->k), static_cast<const uint8_t*>(pool->v), nullptr, nullptr,
               pool->page_table, pool->num_blocks, pool->max_pages, 16};
  int32_t* err = device_error_word();
  if (!err) return VC_EHIP;
  const dim3 grid(num * L * Hkv);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint16_t* bk = static_cast<const uint16_t*>(blk_k);
  const uint16_t* bv = static_cast<const uint16_t*>(blk_v);
  if (d == 128)
    hipLaunchKernelGGL(commit_rows_kernel<128>, grid, dim3(256), 0, st, ci, L, Hkv, xmax, bk, bv, p, kept, kept_stride, err);
  else
    hipLaunchKernelGGL(commit_rows_kernel<64>, grid, dim3(256), 0, st, ci, L, Hkv, xmax, bk, bv, p, kept, kept_stride, err);
  return hip_check(hipGetLastError(), "commit launch");
}

}  // extern "C"
