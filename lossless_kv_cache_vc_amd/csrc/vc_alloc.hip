// Page allocator with two page kinds (host code only).
//
// VeriCache review, §Implementation notes worth absorbing, "Page table tricks": every request
// holds compressed-resident pages (allocated for its whole life) and full-transient pages
// (allocated when its full cache is reloaded for a verify, freed after it); the free list keeps
// the two kinds apart so that transient frees do not fragment the resident pool.
//
// Here the kinds own disjoint ranges of one pool's physical block ids: resident blocks are
// [0, num_resident), transient blocks [num_resident, num_blocks).  Each kind has a LIFO free
// stack (a freed block is the next one handed out, which keeps recently used blocks warm) and an
// owner map, so a block freed twice or freed as the wrong kind is an error.  The device memory
// itself belongs to the caller; the allocator only hands out ids, which the caller writes into
// its page tables (the row helpers below do that for one request).
#include <vector>

#include "vc_internal.h"

namespace vc {

namespace {

struct Allocator {
  int32_t num_blocks = 0, num_resident = 0;
  std::vector<int32_t> free_ids[2];  // per kind, used as a stack
  std::vector<uint8_t> in_use;       // per block id
};

bool kind_ok(int kind) { return kind == VC_PAGE_RESIDENT || kind == VC_PAGE_TRANSIENT; }

int kind_of(const Allocator& a, int32_t id) { return id < a.num_resident ? VC_PAGE_RESIDENT : VC_PAGE_TRANSIENT; }

int take(Allocator& a, int kind, int n, int32_t* out) {
  std::vector<int32_t>& f = a.free_ids[kind];
  if ((int64_t)f.size() < n) return fail(VC_ENOMEM, "not enough free pages of this kind");
  for (int i = 0; i < n; ++i) {
    out[i] = f.back();
    f.pop_back();
    a.in_use[out[i]] = 1;
  }
  return VC_OK;
}

int give_back(Allocator& a, int kind, int n, const int32_t* ids) {
  // validate everything first: a bad call changes nothing
  std::vector<uint8_t> seen;
  for (int i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (id < 0 || id >= a.num_blocks) return fail(VC_EINVAL, "page id out of range");
    if (kind_of(a, id) != kind) return fail(VC_EINVAL, "page id belongs to the other kind");
    if (!a.in_use[id]) return fail(VC_EINVAL, "page is not allocated (double free?)");
    for (int j = 0; j < i; ++j)
      if (ids[j] == id) return fail(VC_EINVAL, "page id listed twice");
  }
  for (int i = 0; i < n; ++i) {
    a.in_use[ids[i]] = 0;
    a.free_ids[kind].push_back(ids[i]);
  }
  return VC_OK;
}

}  // namespace

}  // namespace vc

using namespace vc;

extern "C" {

int vc_alloc_create(int32_t num_blocks, int32_t num_resident, void** alloc) {
  set_error("");
  if (!alloc) return fail(VC_EINVAL, "NULL argument");
  *alloc = nullptr;
  if (num_blocks < 0 || num_resident < 0 || num_resident > num_blocks)
    return fail(VC_EINVAL, "need 0 <= num_resident <= num_blocks");
  Allocator* a = new Allocator;
  a->num_blocks = num_blocks;
  a->num_resident = num_resident;
  a->in_use.assign(num_blocks, 0);
  // stacks hold the lowest ids on top, so a fresh allocator hands out ids in ascending order
  for (int32_t id = num_resident - 1; id >= 0; --id) a->free_ids[VC_PAGE_RESIDENT].push_back(id);
  for (int32_t id = num_blocks - 1; id >= num_resident; --id) a->free_ids[VC_PAGE_TRANSIENT].push_back(id);
  *alloc = a;
  return VC_OK;
}

void vc_alloc_destroy(void* alloc) { delete static_cast<Allocator*>(alloc); }

int vc_alloc_pages(void* alloc, int kind, int n, int32_t* ids) {
  set_error("");
  if (!alloc || (n > 0 && !ids)) return fail(VC_EINVAL, "NULL argument");
  if (!kind_ok(kind)) return fail(VC_EINVAL, "bad page kind");
  if (n < 0) return fail(VC_EINVAL, "n must be >= 0");
  return take(*static_cast<Allocator*>(alloc), kind, n, ids);
}

int vc_alloc_release(void* alloc, int kind, int n, const int32_t* ids) {
  set_error("");
  if (!alloc || (n > 0 && !ids)) return fail(VC_EINVAL, "NULL argument");
  if (!kind_ok(kind)) return fail(VC_EINVAL, "bad page kind");
  if (n < 0) return fail(VC_EINVAL, "n must be >= 0");
  return give_back(*static_cast<Allocator*>(alloc), kind, n, ids);
}

int32_t vc_alloc_free_count(const void* alloc, int kind) {
  if (!alloc || !kind_ok(kind)) return -1;
  return (int32_t)static_cast<const Allocator*>(alloc)->free_ids[kind].size();
}

int vc_page_row_extend(void* alloc, int kind, int32_t* row, int32_t max_pages, int32_t old_len, int32_t new_len) {
  set_error("");
  if (!alloc || !row) return fail(VC_EINVAL, "NULL argument");
  if (!kind_ok(kind)) return fail(VC_EINVAL, "bad page kind");
  if (old_len < 0 || new_len < old_len) return fail(VC_EINVAL, "need 0 <= old_len <= new_len");
  const int p0 = (old_len + kBlock - 1) / kBlock, p1 = (new_len + kBlock - 1) / kBlock;
  if (p1 > max_pages) return fail(VC_EINVAL, "page row too short for new_len");
  if (p1 == p0) return VC_OK;
  std::vector<int32_t> got(p1 - p0);
  const int rc = take(*static_cast<Allocator*>(alloc), kind, p1 - p0, got.data());
  if (rc) return rc;
  for (int p = p0; p < p1; ++p) row[p] = got[p - p0];
  return VC_OK;
}

int vc_page_row_truncate(void* alloc, int kind, int32_t* row, int32_t max_pages, int32_t old_len, int32_t new_len) {
  set_error("");
  if (!alloc || !row) return fail(VC_EINVAL, "NULL argument");
  if (!kind_ok(kind)) return fail(VC_EINVAL, "bad page kind");
  if (new_len < 0 || new_len > old_len) return fail(VC_EINVAL, "need 0 <= new_len <= old_len");
  const int p0 = (new_len + kBlock - 1) / kBlock, p1 = (old_len + kBlock - 1) / kBlock;
  if (p1 > max_pages) return fail(VC_EINVAL, "page row too short for old_len");
  if (p1 == p0) return VC_OK;
  const int rc = give_back(*static_cast<Allocator*>(alloc), kind, p1 - p0, row + p0);
  if (rc) return rc;
  for (int p = p0; p < p1; ++p) row[p] = -1;
  return VC_OK;
}

}  // extern "C"
