// Internal declarations shared by the library's translation units (host and device).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>
#include <vector>

#include "../../include/vc.h"

namespace vc {

// ---------------------------------------------------------------- error reporting (host)
void set_error(const std::string& msg);
int fail(int code, const std::string& msg);
int hip_check(hipError_t e, const char* what);

// ---------------------------------------------------------------- device vector types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = VC_BLOCK_TOKENS;
constexpr int kMaxReqs = VC_MAX_REQS;    // requests of one attention launch
constexpr int kInlineReqs = 64;          // of those, carried in the kernel argument block
constexpr int kMaxBatch = VC_MAX_BATCH;  // requests of one cache-building or commit call

// ---------------------------------------------------------------- device error word
// One word block per device (a file-scope __device__ array of the library): a kernel that reads a
// page-table entry outside [-1, num_blocks) stores [1, page-table row, logical page, entry] into
// it with ordinary vector stores and treats the page as missing.  vc_check_device() reads and
// clears it.  Returns the current device's copy (NULL and a recorded error if HIP fails).
int32_t* device_error_word();

// Record a bad page-table entry (any lane may call it; concurrent writers store the same kind of
// report, and one of them is kept).
__device__ __forceinline__ void report_bad_page(int32_t* err, int row, int page, int id) {
  if (err) {
    err[1] = row;
    err[2] = page;
    err[3] = id;
    err[0] = 1;
  }
}

// Pool descriptor as the kernels see it (passed by value in kernel arguments).
struct PoolDev {
  const uint8_t* k;
  const uint8_t* v;
  const uint8_t* ksz;
  const uint8_t* vsz;
  const int32_t* page_table;
  int64_t nblk;
  int32_t max_pages;
  int32_t bits;
};

// Per-request launch plan (host computed; in the kernel arguments for up to kInlineReqs
// requests, else in a device table at the head of the workspace).
struct ReqDev {
  int32_t slot, pool, ctx_len, page_row, q0, rows, kind;
  int32_t item_base;    // first work item of this request
  int32_t nsplit;       // context splits per (layer, kv head)
  int32_t nrg;          // row groups per (layer, kv head, split) (verify); 1 for draft
  int32_t chunk_pages;  // context pages per split
  int32_t merge_base;   // first merge row of this request (split requests; -1 otherwise)
  int64_t part_base;    // float offset of this request's partials in the workspace (-1: none)
};
static_assert(sizeof(ReqDev) == 56, "request table entry");

constexpr int kMaxPools = 4;

struct AttnArgs {
  PoolDev pools[kMaxPools];
  const uint16_t* q;
  const uint16_t* blk_k;
  const uint16_t* blk_v;
  float* out;
  float* part;
  int32_t L, Hq, Hkv, G, xmax, nreq, nitems, nitems_pad;
  float scale_log2;  // log2(e) / sqrt(d)
  int32_t vwaves;    // verify work-group: 0 = 8 waves over 128-row groups; else that many
                     // waves, one per 32 rows, over groups of 32 * vwaves rows (wide verify)
  int32_t xcd_ranges;  // 1: each XCD takes a contiguous range of items (row groups of a unit
                       // share an L2); 0: work-group b takes item b (ragged batches)
  int32_t nmerge;      // merge rows of the split requests
  int32_t* err;        // device error word (bad page-table entries)
  const ReqDev* reqs_dev;  // request table in device memory when nreq > kInlineReqs, else NULL
  ReqDev reqs[kInlineReqs];
};

static_assert(sizeof(AttnArgs) <= 4096, "kernel arguments must fit 4 KiB");

// Plan an attention launch: fills reqs/nitems and returns workspace floats needed.
struct Plan {
  int nitems = 0;
  int vwaves = 0;  // wide verify waves (0: the 8-wave verify)
  int64_t part_floats = 0;
  int any_split = 0;
  int head_dim = 0;
  int has_verify = 0;  // the launch holds verifying / drafting requests (over all of them, not
  int has_draft = 0;   // only the ones the kernel arguments carry)
  int draft_bits = 0;  // bits of every drafting request's pool (16, 2 or 4), -1 if they differ
};
int plan_attn(const vc_shape* s, int nreq, const vc_req* reqs, int npools, const vc_pool* pools,
              int split_pages, AttnArgs* args, Plan* plan, std::vector<ReqDev>* table);

// Bytes at the head of the workspace that hold the request table of an nreq-request launch
// (0 when the table fits the kernel arguments), rounded up to 256.
inline size_t req_table_bytes(int nreq) {
  return nreq > kInlineReqs ? ((size_t)nreq * sizeof(ReqDev) + 255) / 256 * 256 : 0;
}

// Enqueue the copy of a request table into device memory at `dst` (small kernels whose arguments
// carry the entries, so nothing is staged on the host and nothing synchronises).
int upload_req_table(const std::vector<ReqDev>& table, ReqDev* dst, hipStream_t stream);

int launch_attn(const AttnArgs& args, const Plan& plan, int head_dim, hipStream_t stream);

// Rows of split partials one merge work-group combines (256 threads, d / 4 per row).
int merge_rows_per_group(int head_dim);

// Largest wide-verify work-group: 12 waves (3 per SIMD), 384 query rows.
constexpr int kWideMaxWaves = 12;

// Waves of a wide verify work-group for nrb 32-row blocks per item.  Waves are dealt to the 4
// SIMDs in turn, so nrb = 4q + 1 or 4q + 2 whole-block waves would leave one or two SIMDs a wave
// more than the others; instead the last nrb - 4q blocks are split by key half over two waves
// each, and every SIMD carries at most q + 1/2 waves of work.  Returns the waves and sets *nfull
// (the waves that own a whole block: waves nfull + 2j and nfull + 2j + 1 share block nfull + j).
__host__ __device__ inline int wide_waves(int nrb, int* nfull) {
  const int q = nrb / 4, rem = nrb % 4;
  if (q >= 1 && (rem == 1 || rem == 2) && 4 * q + 2 * rem <= kWideMaxWaves) {
    *nfull = 4 * q;
    return 4 * q + 2 * rem;
  }
  *nfull = nrb;
  return nrb;
}

// Context pages of one work item are capped so that their block ids fit the kernels' LDS.
constexpr int kMaxChunkPages = 2048;

// Split of one request's context into chunks of at most `target` pages (a multiple of 4), with
// the chunks made as even as possible: returns the chunk size and sets *nsplit.
inline int split_context(int pages, int target, int* nsplit) {
  if (pages <= 0) {
    *nsplit = 1;
    return target;
  }
  const int n = (pages + target - 1) / target;
  int chunk = (pages + n - 1) / n;
  chunk = (chunk + 3) / 4 * 4;
  *nsplit = (pages + chunk - 1) / chunk;
  return chunk;
}

}  // namespace vc
