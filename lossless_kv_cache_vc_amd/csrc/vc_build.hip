// Building the paged caches: packing dense KV into pages, choosing kept tokens, and compressing
// (token drop copy or KIVI-style quantisation).  These run once before serving (VeriCache
// review, §Compression Method Integration: offline compression); none of them is timed.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "vc_internal.h"

namespace vc {

namespace {

struct BatchInfo {
  int32_t n;                 // requests
  int32_t lens[kMaxBatch];   // tokens per request
  int32_t base[kMaxBatch + 1];  // prefix of per-request job counts
};

__device__ __forceinline__ int find_req(const BatchInfo& bi, int job) {
  int r = 0;
  for (int i = 1; i < bi.n; ++i)
    if (job >= bi.base[i]) r = i;
  return r;
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// ---------------------------------------------------------------- dense -> paged bf16 layer
// job = (request, page, kv head); src bf16 [batch][Hkv][src_rows][d]
template <int D>
__global__ __launch_bounds__(256) void pack_kernel(BatchInfo bi, int Hkv, int layer, const uint16_t* src,
                                                   int64_t src_rows, PoolDev pool, int which, int32_t* err) {
  const int job = blockIdx.x;
  const int r = find_req(bi, job);
  int local = job - bi.base[r];
  const int g = local % Hkv, p = local / Hkv;
  const int len = bi.lens[r];
  const int phys = pool.page_table[(int64_t)r * pool.max_pages + p];
  if (phys < 0 || phys >= pool.nblk) {  // an unmapped page is not written; a corrupt id is reported
    if (phys != -1) report_bad_page(err, r, p, phys);
    return;
  }
  const int64_t unit = ((int64_t)layer * pool.nblk + phys) * Hkv + g;
  const uint16_t* s = src + (((int64_t)r * Hkv + g) * src_rows) * D;
  if (which == 0) {
    uint8_t* dst = const_cast<uint8_t*>(pool.k) + unit * (kBlock * D * 2);
    for (int c = threadIdx.x; c < 2 * D; c += blockDim.x) {
      const int t = c / (D / 8), cc = c % (D / 8);
      const int pos = p * kBlock + t;
      u32x4 v = {0, 0, 0, 0};
      if (pos < len) v = ld16(s + (int64_t)pos * D + 8 * cc);
      *reinterpret_cast<u32x4*>(dst + c * 16) = v;
    }
  } else {
    uint16_t* dst = reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(pool.v) + unit * (kBlock * D * 2));
    for (int e = threadIdx.x; e < kBlock * D; e += blockDim.x) {
      const int dd = e / kBlock, t = e % kBlock;
      const int pos = p * kBlock + t;
      dst[e] = pos < len ? s[(int64_t)pos * D + dd] : (uint16_t)0;
    }
  }
}

// ---------------------------------------------------------------- kept-set selection
// One work-group per (request, layer, kv head).  The top `top` scores among positions
// [0, n - recent) are found by an MSB-first radix select on the 32-bit scores; positions with a
// score above the threshold are kept, and of those equal to it the lowest positions fill the
// remainder.  Kept positions are written ascending, the recent window last.
struct SelectInfo {
  int32_t n;
  int32_t lens[kMaxBatch];
  int32_t recent[kMaxBatch];
  int32_t top[kMaxBatch];
};

constexpr int kSelThreads = 1024;

__device__ int block_exclusive_scan(int v, int* tmp /* >= 16 ints */, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) {
      const int t = tmp[i];
      tmp[i] = acc;
      acc += t;
    }
    tmp[16] = acc;
  }
  __syncthreads();
  const int res = tmp[w] + x - v;
  *total = tmp[16];
  __syncthreads();
  return res;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectInfo si, int L, int Hkv,
                                                             const uint32_t* scores, int64_t sstride,
                                                             int32_t* kept, int64_t kstride) {
  __shared__ int hist[256];
  __shared__ int tmp[20];
  __shared__ uint32_t sh_prefix, sh_mask;
  __shared__ int sh_need;
  const int unit = blockIdx.x;  // (r, l, g)
  const int g = unit % Hkv, l = (unit / Hkv) % L, r = unit / (Hkv * L);
  const int n = si.lens[r];
  const int recent = min(si.recent[r], n);
  const int older = n - recent;
  const int top = min(si.top[r], older);
  const uint32_t* sc = scores + ((int64_t)(r * L + l) * Hkv + g) * sstride;
  int32_t* out = kept + ((int64_t)(r * L + l) * Hkv + g) * kstride;

  uint32_t prefix = 0, mask = 0;
  int need = top;
  if (top > 0 && top < older) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0;
      __syncthreads();
      for (int p = threadIdx.x; p < older; p += blockDim.x) {
        const uint32_t s = sc[p];
        if ((s & mask) == prefix) atomicAdd(&hist[(s >> shift) & 255], 1);
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        int rem = need, b = 255;
        for (; b > 0; --b) {
          if (hist[b] >= rem) break;
          rem -= hist[b];
        }
        sh_need = rem;
        sh_prefix = prefix | ((uint32_t)b << shift);
        sh_mask = mask | (255u << shift);
      }
      __syncthreads();
      need = sh_need;
      prefix = sh_prefix;
      mask = sh_mask;
      __syncthreads();
    }
  }
  // threshold T = prefix; keep all s > T and the first `need` positions with s == T
  const bool all = top >= older;
  const uint32_t T = prefix;
  const int chunk = (older + blockDim.x - 1) / blockDim.x;
  const int lo = min(older, (int)threadIdx.x * chunk), hi = min(older, lo + chunk);
  int gt = 0, eq = 0;
  if (top > 0) {
    for (int p = lo; p < hi; ++p) {
      const uint32_t s = sc[p];
      if (all || s > T) ++gt;
      else if (s == T) ++eq;
    }
  }
  int tot;
  const int eq_before = block_exclusive_scan(eq, tmp, &tot);
  const int my_eq = all ? 0 : max(0, min(eq, need - eq_before));
  const int mine = gt + my_eq;
  const int off = block_exclusive_scan(mine, tmp, &tot);
  if (top > 0) {
    int o = off, seen = 0;
    for (int p = lo; p < hi; ++p) {
      const uint32_t s = sc[p];
      if (all || s > T) {
        out[o++] = p;
      } else if (s == T && seen < my_eq) {
        out[o++] = p;
        ++seen;
      }
    }
  }
  for (int j = threadIdx.x; j < recent; j += blockDim.x) out[top + j] = older + j;
}

// ---------------------------------------------------------------- compression
struct CompInfo {
  int32_t n;
  int32_t lens[kMaxBatch];     // stored tokens per request (k_r)
  int32_t from[kMaxBatch];     // first stored token to rebuild (its page / group is rebuilt whole)
  int32_t base[kMaxBatch + 1];  // prefix of jobs
};

// a source position maps to a block of the source pool (missing pages read as zeros; a corrupt
// table entry is reported and read as zeros too)
__device__ __forceinline__ bool src_ok(const PoolDev& s, int r, int pos, int32_t* err) {
  if (pos < 0 || pos >= s.max_pages * kBlock) return false;
  const int phys = s.page_table[(int64_t)r * s.max_pages + pos / kBlock];
  if (phys >= 0 && phys < s.nblk) return true;
  if (phys != -1) report_bad_page(err, r, pos / kBlock, phys);
  return false;
}

// a destination page of a compressed pool: its block id, or -1 when it is unmapped (not written)
// or corrupt (reported, not written)
__device__ __forceinline__ int dst_block(const PoolDev& d, int r, int page, int32_t* err) {
  const int phys = d.page_table[(int64_t)r * d.max_pages + page];
  if (phys >= 0 && phys < d.nblk) return phys;
  if (phys != -1) report_bad_page(err, r, page, phys);
  return -1;
}

// source token `pos` of (r, l, g) in a bf16 pool: key row / value element pointers
template <int D>
__device__ __forceinline__ const uint16_t* src_k_row(const PoolDev& s, int Hkv, int r, int l, int g, int pos) {
  const int phys = s.page_table[(int64_t)r * s.max_pages + pos / kBlock];
  const int64_t unit = ((int64_t)l * s.nblk + phys) * Hkv + g;
  return reinterpret_cast<const uint16_t*>(s.k + unit * (kBlock * D * 2)) + (pos % kBlock) * D;
}
template <int D>
__device__ __forceinline__ const uint16_t* src_v_page(const PoolDev& s, int Hkv, int r, int l, int g, int pos) {
  const int phys = s.page_table[(int64_t)r * s.max_pages + pos / kBlock];
  const int64_t unit = ((int64_t)l * s.nblk + phys) * Hkv + g;
  return reinterpret_cast<const uint16_t*>(s.v + unit * (kBlock * D * 2));
}

// bf16 token drop: job = (r, l, g, destination page)
template <int D>
__global__ __launch_bounds__(256) void gather_bf16_kernel(CompInfo ci, int L, int Hkv, PoolDev src,
                                                          const int32_t* kept, int64_t kstride, PoolDev dst,
                                                          int32_t* err) {
  const int job = blockIdx.x;
  int r = 0;
  for (int i = 1; i < ci.n; ++i)
    if (job >= ci.base[i]) r = i;
  int local = job - ci.base[r];
  const int pfirst = ci.from[r] / kBlock;
  const int npages = (ci.lens[r] + kBlock - 1) / kBlock - pfirst;
  const int p = pfirst + local % npages;
  local /= npages;
  const int g = local % Hkv, l = local / Hkv;
  const int T = ci.lens[r];
  const int32_t* kp = kept ? kept + ((int64_t)(r * L + l) * Hkv + g) * kstride : nullptr;
  const int phys = dst_block(dst, r, p, err);
  if (phys < 0) return;  // unmapped (or corrupt) destination page
  const int64_t unit = ((int64_t)l * dst.nblk + phys) * Hkv + g;
  uint8_t* dk = const_cast<uint8_t*>(dst.k) + unit * (kBlock * D * 2);
  uint16_t* dv = reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(dst.v) + unit * (kBlock * D * 2));
  for (int c = threadIdx.x; c < 2 * D; c += blockDim.x) {
    const int t = c / (D / 8), cc = c % (D / 8);
    const int j = p * kBlock + t;
    u32x4 v = {0, 0, 0, 0};
    if (j < T) {
      const int pos = kp ? kp[j] : j;
      if (src_ok(src, r, pos, err)) v = ld16(src_k_row<D>(src, Hkv, r, l, g, pos) + 8 * cc);
    }
    *reinterpret_cast<u32x4*>(dk + c * 16) = v;
  }
  for (int e = threadIdx.x; e < kBlock * D; e += blockDim.x) {
    const int dd = e / kBlock, t = e % kBlock;
    const int j = p * kBlock + t;
    uint16_t v = 0;
    if (j < T) {
      const int pos = kp ? kp[j] : j;
      if (src_ok(src, r, pos, err)) v = src_v_page<D>(src, Hkv, r, l, g, pos)[dd * kBlock + pos % kBlock];
    }
    dv[e] = v;
  }
}

// float64 -> fp16 bits, round to nearest even, one rounding (IEEE 754 binary16).
__device__ uint16_t f64_to_f16_rne(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint32_t sign = (uint32_t)(b >> 63) << 15;
  const int ex = (int)((b >> 52) & 0x7FF);
  uint64_t man = b & ((1ull << 52) - 1);
  if (ex == 0x7FF) return (uint16_t)(sign | 0x7C00 | (man ? 0x200 : 0));
  if (ex == 0 && man == 0) return (uint16_t)sign;
  int e = ex - 1023;
  uint64_t m = ex ? (man | (1ull << 52)) : man;
  if (ex == 0) e = -1022;
  if (e >= -14) {
    // normal fp16 candidate: keep 11 significant bits
    uint64_t keep = m >> 42, rem = m & ((1ull << 42) - 1), half = 1ull << 41;
    if (rem > half || (rem == half && (keep & 1))) ++keep;
    if (keep == (1ull << 11)) {
      keep >>= 1;
      ++e;
    }
    if (e > 15) return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | ((uint32_t)(e + 15) << 10) | (uint32_t)(keep & 0x3FF));
  }
  // subnormal: units of 2^-24, value = m * 2^(e - 52)
  const int shift = 28 - e;  // = 52 - 24 - e
  if (shift > 60) return (uint16_t)sign;
  uint64_t keep = m >> shift, rem = m & ((1ull << shift) - 1), half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (keep & 1))) ++keep;
  return (uint16_t)(sign | (uint32_t)keep);  // keep == 1024 encodes the smallest normal
}

__device__ __forceinline__ double f16_bits_to_f64(uint16_t h) {
  return (double)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ double bf16_to_f64(uint16_t b) {
  return (double)__builtin_bit_cast(float, (uint32_t)b << 16);
}

__device__ __forceinline__ uint32_t quant_code(double x, uint16_t s16, uint16_t z16, int levels) {
  const double s = f16_bits_to_f64(s16), z = f16_bits_to_f64(z16);
  if (s == 0.0) return 0;
  double c = rint((x - z) / s);
  c = fmin(fmax(c, 0.0), (double)levels);
  return (uint32_t)c;
}

__device__ __forceinline__ int code_bitpos(int u, int bits) { return (u & 1) * 16 + bits * (u >> 1); }

// KIVI-style quantisation: job = (r, l, g, 32-token group j) of the stored sequence.
template <int D>
__global__ __launch_bounds__(256) void kivi_kernel(CompInfo ci, int L, int Hkv, PoolDev src,
                                                   const int32_t* kept, int64_t kstride, PoolDev dst,
                                                   int32_t* err) {
  __shared__ uint16_t xk[32][D];   // gathered bf16 keys of the group
  __shared__ uint16_t xv[32][D];
  __shared__ uint8_t ck[32][D];    // codes
  __shared__ uint8_t cv[32][D];
  const int bits = dst.bits, levels = (1 << bits) - 1;
  const int job = blockIdx.x;
  int r = 0;
  for (int i = 1; i < ci.n; ++i)
    if (job >= ci.base[i]) r = i;
  int local = job - ci.base[r];
  const int T = ci.lens[r];
  const int jfirst = ci.from[r] / 32;
  const int ngrp = (T + 31) / 32 - jfirst;
  const int j = jfirst + local % ngrp;
  local /= ngrp;
  const int g = local % Hkv, l = local / Hkv;
  const int t0 = 32 * j, cnt = min(32, T - t0);
  const int32_t* kp = kept ? kept + ((int64_t)(r * L + l) * Hkv + g) * kstride : nullptr;

  for (int e = threadIdx.x; e < 32 * D; e += blockDim.x) {
    const int t = e / D, c = e % D;
    uint16_t kv = 0, vv = 0;
    if (t < cnt) {
      const int pos = kp ? kp[t0 + t] : t0 + t;
      if (src_ok(src, r, pos, err)) {
        kv = src_k_row<D>(src, Hkv, r, l, g, pos)[c];
        vv = src_v_page<D>(src, Hkv, r, l, g, pos)[c * kBlock + pos % kBlock];
      }
    }
    xk[t][c] = kv;
    xv[t][c] = vv;
  }
  __syncthreads();

  const int p_even = 2 * j;
  const int phys_e = dst_block(dst, r, p_even, err);
  if (phys_e < 0) return;  // unmapped (or corrupt) destination: the group is skipped
  const int64_t unit_e = ((int64_t)l * dst.nblk + phys_e) * Hkv + g;
  // keys: one channel per thread, group over the cnt tokens
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    double mn = INFINITY, mx = -INFINITY;
    for (int t = 0; t < cnt; ++t) {
      const double x = bf16_to_f64(xk[t][c]);
      mn = fmin(mn, x);
      mx = fmax(mx, x);
    }
    const uint16_t s16 = f64_to_f16_rne((mx - mn) / (double)levels);
    const uint16_t z16 = f64_to_f16_rne(mn);
    for (int t = 0; t < 32; ++t)
      ck[t][c] = t < cnt ? (uint8_t)quant_code(bf16_to_f64(xk[t][c]), s16, z16, levels) : 0;
    uint16_t* ksz = reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(dst.ksz) + unit_e * (D * 4));
    ksz[c] = s16;       // scale plane
    ksz[D + c] = z16;   // zero plane
  }
  // values: one (token, 32-channel group) per thread
  for (int task = threadIdx.x; task < 32 * (D / 32); task += blockDim.x) {
    const int t = task / (D / 32), gq = task % (D / 32);
    if (t < cnt) {
      double mn = INFINITY, mx = -INFINITY;
      for (int c = 32 * gq; c < 32 * gq + 32; ++c) {
        const double x = bf16_to_f64(xv[t][c]);
        mn = fmin(mn, x);
        mx = fmax(mx, x);
      }
      const uint16_t s16 = f64_to_f16_rne((mx - mn) / (double)levels);
      const uint16_t z16 = f64_to_f16_rne(mn);
      for (int c = 32 * gq; c < 32 * gq + 32; ++c)
        cv[t][c] = (uint8_t)quant_code(bf16_to_f64(xv[t][c]), s16, z16, levels);
      const int page = (t0 + t) / kBlock, tt = (t0 + t) % kBlock;
      const int phys = dst_block(dst, r, page, err);
      if (phys >= 0) {
        const int64_t unit = ((int64_t)l * dst.nblk + phys) * Hkv + g;
        uint16_t* vsz = reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(dst.vsz) + unit * (D / 32 * kBlock * 4));
        vsz[(gq * 2) * kBlock + tt] = s16;      // [group][scale plane][token]
        vsz[(gq * 2 + 1) * kBlock + tt] = z16;  // [group][zero plane][token]
      }
    } else {
      for (int c = 32 * gq; c < 32 * gq + 32; ++c) cv[t][c] = 0;
    }
  }
  __syncthreads();
  // pack codes of the (up to) two pages of the group
  const int per = 32 / bits;
  for (int hp = 0; hp < 2; ++hp) {
    const int page = p_even + hp;
    if (16 * hp >= cnt) break;
    const int phys = dst_block(dst, r, page, err);
    if (phys < 0) continue;
    const int64_t unit = ((int64_t)l * dst.nblk + phys) * Hkv + g;
    uint32_t* kw = reinterpret_cast<uint32_t*>(const_cast<uint8_t*>(dst.k) + unit * (2 * D * bits));
    uint32_t* vw = reinterpret_cast<uint32_t*>(const_cast<uint8_t*>(dst.v) + unit * (2 * D * bits));
    const int kwords = kBlock * D / per;  // key words per page: [16 tokens][D / per]
    for (int wi = threadIdx.x; wi < kwords; wi += blockDim.x) {
      const int t = wi / (D / per), c0 = (wi % (D / per)) * per;
      uint32_t word = 0;
      for (int u = 0; u < per; ++u) word |= (uint32_t)ck[16 * hp + t][c0 + u] << code_bitpos(u, bits);
      kw[wi] = word;
    }
    const int vwords = D * kBlock / per;  // value words per page: [D][16 / per]
    for (int wi = threadIdx.x; wi < vwords; wi += blockDim.x) {
      const int c = wi / (kBlock / per), tb = (wi % (kBlock / per)) * per;
      uint32_t word = 0;
      for (int u = 0; u < per; ++u) word |= (uint32_t)cv[16 * hp + tb + u][c] << code_bitpos(u, bits);
      vw[wi] = word;
    }
  }
}

int fill_batch(int batch, const int32_t* lens, BatchInfo* bi, int per_page_jobs) {
  if (batch < 1 || batch > kMaxBatch) return fail(VC_EINVAL, "batch must be in [1, 128]");
  if (!lens) return fail(VC_EINVAL, "lens is NULL");
  memset(bi, 0, sizeof(*bi));
  bi->n = batch;
  int64_t acc = 0;
  for (int i = 0; i < batch; ++i) {
    if (lens[i] < 0) return fail(VC_EINVAL, "negative length");
    bi->lens[i] = lens[i];
    bi->base[i] = (int32_t)acc;
    acc += (int64_t)((lens[i] + kBlock - 1) / kBlock) * per_page_jobs;
    if (acc > (1 << 30)) return fail(VC_EINVAL, "too many pages");
  }
  bi->base[batch] = (int32_t)acc;
  return VC_OK;
}

}  // namespace

static int shape_ok(const vc_shape* s) {
  if (!s) return fail(VC_EINVAL, "shape is NULL");
  if (s->num_layers < 1 || s->num_kv_heads < 1) return fail(VC_EINVAL, "bad shape");
  if (s->head_dim != 64 && s->head_dim != 128) return fail(VC_EUNSUPPORTED, "head_dim must be 64 or 128");
  return VC_OK;
}

}  // namespace vc

using namespace vc;

extern "C" {

int vc_pack_bf16(const vc_shape* shape, int batch, const int32_t* lens, int layer, const void* src,
                 int64_t src_rows, const vc_pool* pool, int which, void* stream) {
  set_error("");
  int rc = shape_ok(shape);
  if (rc) return rc;
  if (!pool || pool->bits != 16 || !pool->page_table || !pool->k || !pool->v)
    return fail(VC_EINVAL, "pack needs a bf16 pool with page_table, k and v");
  if (!src) return fail(VC_EINVAL, "src is NULL");
  if (layer < 0 || layer >= shape->num_layers) return fail(VC_EINVAL, "layer out of range");
  if (which != 0 && which != 1) return fail(VC_EINVAL, "which must be 0 (keys) or 1 (values)");
  BatchInfo bi;
  rc = fill_batch(batch, lens, &bi, shape->num_kv_heads);
  if (rc) return rc;
  for (int i = 0; i < batch; ++i) {
    if (lens[i] > src_rows) return fail(VC_EINVAL, "length exceeds src_rows");
    if ((lens[i] + kBlock - 1) / kBlock > pool->max_pages) return fail(VC_EINVAL, "page table too narrow");
  }
  if (bi.base[batch] == 0) return VC_OK;
  PoolDev pd = {static_cast<const uint8_t*>(pool->k), static_cast<const uint8_t*>(pool->v), nullptr,
                nullptr, pool->page_table, pool->num_blocks, pool->max_pages, 16};
  int32_t* err = device_error_word();
  if (!err) return VC_EHIP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (shape->head_dim == 128)
    hipLaunchKernelGGL(pack_kernel<128>, dim3(bi.base[batch]), dim3(256), 0, st, bi, shape->num_kv_heads,
                       layer, static_cast<const uint16_t*>(src), src_rows, pd, which, err);
  else
    hipLaunchKernelGGL(pack_kernel<64>, dim3(bi.base[batch]), dim3(256), 0, st, bi, shape->num_kv_heads,
                       layer, static_cast<const uint16_t*>(src), src_rows, pd, which, err);
  return hip_check(hipGetLastError(), "pack launch");
}

int vc_select_kept(const vc_shape* shape, int batch, const int32_t* lens, const int32_t* recent,
                   const int32_t* top, const uint32_t* scores, int64_t score_stride, int32_t* kept,
                   int64_t kept_stride, void* stream) {
  set_error("");
  int rc = shape_ok(shape);
  if (rc) return rc;
  if (batch < 1 || batch > kMaxBatch) return fail(VC_EINVAL, "batch must be in [1, 128]");
  if (!lens || !recent || !top || !scores || !kept) return fail(VC_EINVAL, "NULL argument");
  SelectInfo si;
  memset(&si, 0, sizeof si);
  si.n = batch;
  for (int i = 0; i < batch; ++i) {
    if (lens[i] < 0 || recent[i] < 0 || top[i] < 0) return fail(VC_EINVAL, "negative size");
    if (lens[i] > score_stride) return fail(VC_EINVAL, "length exceeds score_stride");
    const int k = std::min(lens[i], recent[i]) + std::min(top[i], lens[i] - std::min(lens[i], recent[i]));
    if (k > kept_stride) return fail(VC_EINVAL, "kept_stride too small");
    si.lens[i] = lens[i];
    si.recent[i] = recent[i];
    si.top[i] = top[i];
  }
  const int units = batch * shape->num_layers * shape->num_kv_heads;
  hipLaunchKernelGGL(select_kernel, dim3(units), dim3(kSelThreads), 0, static_cast<hipStream_t>(stream), si,
                     shape->num_layers, shape->num_kv_heads, scores, score_stride, kept, kept_stride);
  return hip_check(hipGetLastError(), "select launch");
}

int vc_compress_tail(const vc_shape* shape, int batch, const int32_t* from_lens, const int32_t* comp_lens,
                     const vc_pool* src, const int32_t* kept, int64_t kept_stride, const vc_pool* dst,
                     void* stream) {
  set_error("");
  int rc = shape_ok(shape);
  if (rc) return rc;
  if (!src || src->bits != 16 || !src->k || !src->v || !src->page_table)
    return fail(VC_EINVAL, "compress reads a bf16 source pool");
  if (!dst || !dst->k || !dst->v || !dst->page_table) return fail(VC_EINVAL, "bad destination pool");
  if (dst->bits != 16 && dst->bits != 2 && dst->bits != 4) return fail(VC_EINVAL, "dst bits must be 16, 2 or 4");
  if (dst->bits != 16 && (!dst->k_sz || !dst->v_sz)) return fail(VC_EINVAL, "KIVI pool needs k_sz and v_sz");
  if (batch < 1 || batch > kMaxBatch || !comp_lens) return fail(VC_EINVAL, "bad batch");
  CompInfo ci;
  memset(&ci, 0, sizeof ci);
  ci.n = batch;
  const int L = shape->num_layers, Hkv = shape->num_kv_heads;
  int64_t acc = 0;
  for (int i = 0; i < batch; ++i) {
    if (comp_lens[i] < 0) return fail(VC_EINVAL, "negative length");
    const int from = from_lens ? from_lens[i] : 0;
    if (from < 0 || from > comp_lens[i]) return fail(VC_EINVAL, "from_lens must be in [0, comp_lens]");
    if (kept && comp_lens[i] > kept_stride) return fail(VC_EINVAL, "kept_stride too small");
    if ((comp_lens[i] + kBlock - 1) / kBlock > dst->max_pages) return fail(VC_EINVAL, "dst page table too narrow");
    ci.lens[i] = comp_lens[i];
    ci.from[i] = from;
    ci.base[i] = (int32_t)acc;
    const int64_t per = dst->bits == 16 ? (comp_lens[i] + kBlock - 1) / kBlock - from / kBlock
                                        : (comp_lens[i] + 31) / 32 - from / 32;
    acc += per * L * Hkv;
    if (acc > (1LL << 31) - 1) return fail(VC_EINVAL, "too many jobs");
  }
  ci.base[batch] = (int32_t)acc;
  if (acc == 0) return VC_OK;
  PoolDev s = {static_cast<const uint8_t*>(src->k), static_cast<const uint8_t*>(src->v), nullptr, nullptr,
               src->page_table, src->num_blocks, src->max_pages, 16};
  PoolDev d = {static_cast<const uint8_t*>(dst->k), static_cast<const uint8_t*>(dst->v),
               static_cast<const uint8_t*>(dst->k_sz), static_cast<const uint8_t*>(dst->v_sz),
               dst->page_table, dst->num_blocks, dst->max_pages, dst->bits};
  int32_t* err = device_error_word();
  if (!err) return VC_EHIP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool d128 = shape->head_dim == 128;
  if (dst->bits == 16) {
    if (d128) hipLaunchKernelGGL(gather_bf16_kernel<128>, dim3(acc), dim3(256), 0, st, ci, L, Hkv, s, kept, kept_stride, d, err);
    else hipLaunchKernelGGL(gather_bf16_kernel<64>, dim3(acc), dim3(256), 0, st, ci, L, Hkv, s, kept, kept_stride, d, err);
  } else {
    if (d128) hipLaunchKernelGGL(kivi_kernel<128>, dim3(acc), dim3(256), 0, st, ci, L, Hkv, s, kept, kept_stride, d, err);
    else hipLaunchKernelGGL(kivi_kernel<64>, dim3(acc), dim3(256), 0, st, ci, L, Hkv, s, kept, kept_stride, d, err);
  }
  return hip_check(hipGetLastError(), "compress launch");
}

int vc_compress(const vc_shape* shape, int batch, const int32_t* comp_lens, const vc_pool* src,
                const int32_t* kept, int64_t kept_stride, const vc_pool* dst, void* stream) {
  return vc_compress_tail(shape, batch, nullptr, comp_lens, src, kept, kept_stride, dst, stream);
}

}  // extern "C"
