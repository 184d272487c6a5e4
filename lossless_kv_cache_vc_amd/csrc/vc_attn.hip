// Draft and verify attention over paged KV caches for gfx950 (CDNA4).
//
// VeriCache review, §Draft–Verify Pipeline: the verifier runs one pass over the x drafted
// positions against the full cache (position i conditioned on drafted rows before and at i);
// the drafter runs one single-token step against the compressed cache.  Both are
// softmax(q k^T / sqrt(d)) v (§Prerequisites, attention equation) over different key sets.
//
// One launch processes a list of work items; an item is (request, layer, kv head, context
// split, row group), and each work-group takes one item:
//
//  * verify path — the x*G query rows of a kv head are a dense block: each wave owns 32 rows,
//    K/V tiles of 64 keys (4 pages) stream from HBM straight into an LDS ring and are shared by
//    all waves; S^T = K Q^T and O^T += V^T P^T use v_mfma_f32_32x32x16_bf16, so each lane holds
//    one query row of both accumulators and the softmax needs only one cross-lane exchange.
//    verify_kernel (8 waves) covers up to 128 rows per item with two waves per row block, each
//    taking one key half of every tile; verify_wide_kernel (5 to 12 waves) covers up to 384 rows
//    per item with one wave per row block.
//  * draft path — G <= 16 rows: the waves split the keys of the item, each wave streaming its
//    own pages through a private LDS ring (v_mfma_f32_16x16x32, rows padded to 16); KIVI codes
//    are expanded in registers, and the per-wave softmax states merge through LDS.
//
// Long contexts are split into chunks of pages; partial (max, sum, output) states go to the
// workspace and a merge kernel combines them with log-sum-exp weights.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "vc_internal.h"

namespace vc {

namespace {

constexpr int kDWaves = 4;            // waves of a draft-only work-group (bf16 caches)
constexpr int kDThreads = 64 * kDWaves;
constexpr int kKWaves = 12;           // waves of a draft-only work-group (KIVI caches): three per SIMD
constexpr int kKThreads = 64 * kKWaves;
// Headroom (log2 units) a row's maximum may gain before the running maximum is moved and the
// accumulators rescaled.  Where the weights enter the value product as bf16 (8 significant bits)
// a key that raises the maximum must not be left with a large share of its row: the key that sets
// the running maximum has weight exactly 1, which bf16 holds exactly, but a key above it by d
// keeps weight 2^d, rounded by up to 2^-8 relative (an output error of up to 2^-8 |v| when it
// dominates, over 5e-3 for short rows).  The draft paths move the maximum whenever it grows; the
// verify paths allow the headroom rescale_headroom gives.  fp16 weights (11 bits) keep 8 units.
constexpr float kRescaleBf16 = 0.0f;
constexpr float kRescaleF16 = 8.0f;
constexpr float kLimF16 = 256.0f;  // 2^kRescaleF16

// Verify headroom after a move of the running maximum, from the lane's running sum l (in units of
// the new maximum): floor(log2 l) - 3, between 0 and 8.  A key that later raises the maximum by
// d <= headroom keeps weight 2^d <= l / 8, at most a ninth of its row (l only grows until the next
// move, and the lane's sum is part of its row's).  Short rows, and the first tiles of long ones,
// move the maximum on every rise; later tiles almost never.
__device__ __forceinline__ float rescale_headroom(float l) {
  const int e = __builtin_amdgcn_frexp_expf(l);  // l = f 2^e, f in [0.5, 1): floor(log2 l) = e - 1
  return fminf(8.f, fmaxf(0.f, (float)(e - 4)));
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ bf16x8 as_bf(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 t;
  t[0] = (__bf16)a;
  t[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, t);
}

// maximum of 16 floats as a chain the compiler turns into 3-input maxima (8 instructions)
__device__ __forceinline__ float max16(const f32x16& v) {
  float m = fmaxf(fmaxf(v[0], v[1]), v[2]);
#pragma unroll
  for (int r = 3; r + 1 < 16; r += 2) m = fmaxf(fmaxf(m, v[r]), v[r + 1]);
  return fmaxf(m, v[15]);
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  f16x2 t;
  t[0] = (_Float16)a;
  t[1] = (_Float16)b;
  return __builtin_bit_cast(uint32_t, t);
}

// 8 bf16 -> 8 fp16 (round to nearest even)
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = pack_f16(__builtin_bit_cast(float, v[i] << 16), __builtin_bit_cast(float, v[i] & 0xFFFF0000u));
  return o;
}

// 16x16x32 MFMA on packed operands: bf16 for caches that are bf16, fp16 where the operands are
// produced in-register (dequantised KIVI values and the softmax weights that multiply them)
template <bool F16>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(a), as_bf(b), c, 0, 0, 0);
}

__device__ __forceinline__ float fp16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// zero the bf16 lanes t (0..7) of a 16-byte chunk with first + t >= valid
__device__ __forceinline__ u32x4 mask_tokens(u32x4 v, int first, int valid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t w = v[i];
    if (first + 2 * i >= valid) w &= 0xFFFF0000u;
    if (first + 2 * i + 1 >= valid) w &= 0x0000FFFFu;
    v[i] = w;
  }
  return v;
}

__device__ __forceinline__ float wave_xor_max(float x, int mask) {
  return fmaxf(x, __shfl_xor(x, mask));
}
__device__ __forceinline__ float wave_xor_sum(float x, int mask) { return x + __shfl_xor(x, mask); }

// Page descriptor of one page slot of an item: where its K/V live and which keys are visible.
struct PageRef {
  const uint8_t* k;  // page base of keys (bf16 or codes)
  const uint8_t* v;
  const uint8_t* ksz;  // KIVI: key group params of this page's pair (from the even page)
  const uint8_t* vsz;
  int kind;   // 0 context, 1 drafted block, 2 none
  int valid;  // tokens present in the page
  int bpos;   // drafted block: block position of token 0
};

// Descriptors are held by value: a pointer into the kernel's argument block would make the
// compiler copy the whole block to scratch memory.
struct ItemCtx {
  ReqDev rq;
  PoolDev pool;
  int l, g, split;
  int nctx, nbk, npages, p_lo;
  int rows_total;
};

template <int D>
__device__ __forceinline__ PageRef page_ref(const AttnArgs& a, const ItemCtx& it, int ip,
                                            bool kivi) {
  PageRef pr;
  pr.k = pr.v = pr.ksz = pr.vsz = nullptr;
  pr.bpos = 0;
  const ReqDev& rq = it.rq;
  if (ip < it.nctx) {
    const PoolDev& pl = it.pool;
    int p = it.p_lo + ip;
    int phys = pl.page_table[(int64_t)rq.page_row * pl.max_pages + p];
    if (phys < 0 || phys >= pl.nblk) {  // an invalid table entry reads as an empty page
      pr.kind = 2;
      pr.valid = 0;
      return pr;
    }
    int64_t unit = ((int64_t)it.l * pl.nblk + phys) * a.Hkv + it.g;
    if (!kivi) {
      pr.k = pl.k + unit * (kBlock * D * 2);
      pr.v = pl.v + unit * (kBlock * D * 2);
    } else {
      const int wb = D * pl.bits / 8;  // bytes of one token row (keys) / one channel row (values)
      pr.k = pl.k + unit * (kBlock * wb);
      pr.v = pl.v + unit * (int64_t)(D * 2 * pl.bits);  // d channels x 16 tokens x bits / 8
      // the key parameters of the page's 32-token group live in the block of its even page; a
      // missing even page removes its odd partner too
      const int pe = p & ~1;
      const int phys_e = pe == p ? phys : pl.page_table[(int64_t)rq.page_row * pl.max_pages + pe];
      if (phys_e < 0 || phys_e >= pl.nblk) {
        pr.kind = 2;
        pr.valid = 0;
        return pr;
      }
      int64_t unit_e = ((int64_t)it.l * pl.nblk + phys_e) * a.Hkv + it.g;
      pr.ksz = pl.ksz + unit_e * (D * 4);
      pr.vsz = pl.vsz + unit * (D / 32 * kBlock * 4);
    }
    pr.kind = 0;
    pr.valid = min(kBlock, rq.ctx_len - kBlock * p);
  } else if (ip < it.npages) {
    int j = ip - it.nctx;
    int64_t unit = (((int64_t)rq.slot * a.L + it.l) * a.Hkv + it.g) * (a.xmax / kBlock) + j;
    pr.k = reinterpret_cast<const uint8_t*>(a.blk_k) + unit * (kBlock * D * 2);
    pr.v = reinterpret_cast<const uint8_t*>(a.blk_v) + unit * (kBlock * D * 2);
    pr.kind = 1;
    pr.valid = min(kBlock, rq.q0 + rq.rows - kBlock * j);
    pr.bpos = kBlock * j;
  } else {
    pr.kind = 2;
    pr.valid = 0;
  }
  return pr;
}

__device__ __forceinline__ bool key_visible(const PageRef& pr, int tt, int qpos) {
  if (pr.kind == 0) return tt < pr.valid;
  if (pr.kind == 1) return tt < pr.valid && pr.bpos + tt <= qpos;
  return false;
}

// Writes a finished row (normalised) or a split partial (unnormalised, with max and sum).
template <int D>
__device__ __forceinline__ float* out_row(const AttnArgs& a, const ItemCtx& it, int row,
                                          bool* partial) {
  const ReqDev& rq = it.rq;
  if (rq.nsplit == 1) {
    *partial = false;
    int tok = row / a.G, jh = row % a.G;
    int64_t o = ((((int64_t)rq.slot * a.L + it.l) * a.xmax + rq.q0 + tok) * a.Hq + it.g * a.G + jh);
    return a.out + o * D;
  }
  *partial = true;
  int64_t prow = (((int64_t)it.l * a.Hkv + it.g) * rq.nsplit + it.split) * it.rows_total + row;
  return a.part + rq.part_base + prow * (D + 4);
}

// key slot of MFMA row M within a 32-key block: lanes' accumulator registers then hold
// 8 consecutive tokens of one page, which is the B-operand order of the value product.
__device__ __forceinline__ int key_of_m32(int M) {
  return 16 * (M >> 4) + 8 * ((M >> 2) & 1) + 4 * ((M >> 3) & 1) + (M & 3);
}

// XOR swizzle of the 16-byte chunks of a key row in LDS (bank-conflict-free MFMA operand reads)
template <int D>
__device__ __forceinline__ int swz_k(int key) {
  return D == 128 ? (key & 15) : ((key >> 1) & 7);
}

// ------------------------------------------------------------------ verify path (32x32x16)
// A verify work-group has 8 waves: wave w owns row block w & 3 (32 query rows) and key half
// w >> 2 of every 64-key tile.  K/V pages move from HBM straight into a 4-stage LDS ring with
// gfx950's global_load_lds_dwordx4 (no register staging); each wave moves one 4 KB page of every
// tile (waves 0-3 keys, 4-7 values), so each wave's vmcnt counts its own share of the ring.
// Keys run one tile ahead of values: the scores of tile t + 1 (MFMA) are computed while the
// softmax of tile t (VALU) runs.  The two key halves of a row block are merged through LDS at
// the end.
constexpr int kVWaves = 8;
constexpr int kVThreads = 64 * kVWaves;
constexpr int kVStages = 4;   // key stages (keys are loaded 4 tiles ahead)
constexpr int kVVStages = 5;  // value stages (values are loaded 4 tiles ahead, consumed a tile later)

// LDS: the 4 key stages, then the 5 value stages, then the page units of the item.  With the
// key stages in the first 64 KB, every key read is an invariant per-lane offset plus a 16-bit
// immediate once the stage is known at compile time; value reads add one per-tile base.
template <int D>
struct VRing {
  static constexpr int kPage = kBlock * D * 2;      // bytes of one K or V page
  static constexpr int kTileK = 4 * kPage;          // one stage: 64 keys (or their values)
  static constexpr int kV0 = kVStages * kTileK;     // offset of the value stages
  static constexpr int kRing = kV0 + kVVStages * kTileK;
  static constexpr int kIds = kRing;                // LDS offset of the page units
  static constexpr int kBytes = kRing + kMaxChunkPages * 4 + 16;
  static constexpr int kLoads = kPage / 1024;       // 16-byte-per-lane loads per wave per tile
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Cache policy of the ring loads: nontemporal ("nt").  K/V pages are read exactly once, and
// streaming them without it leaves chip-wide HBM throughput near 6.3 TB/s instead of about
// 7.2 TB/s on an MI355X.  The exception is a verifying request cut into several row groups,
// whose items all read the same K/V: those loads keep the default policy, so the lines stay in
// L2 for the sibling items (placed on the same XCD; see decode_item).
constexpr int kNontemporal = 2;
constexpr int kTemporal = 0;

// wait until at most N (< 64) of this wave's vector memory loads are outstanding (loads
// complete in issue order).  gfx9 s_waitcnt fields: vmcnt [3:0] and [15:14], expcnt [6:4] and
// lgkmcnt [11:8] (the last two left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Work-group barrier of the ring loop.  It carries no release fence: a release would wait for
// the ring's in-flight LDS loads as if they were pending LDS stores.  None is needed: LDS is
// written only by those loads, whose completion each wave establishes with wait_vmem() before
// the barrier, and every LDS read of the previous tile has been consumed (by the MFMAs) before
// the barrier.  The acquire fence keeps the next tile's LDS reads and the following ring loads
// below the barrier.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left at their maxima
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One ring load: 16 bytes per lane from a wave-uniform page base plus a 32-bit lane offset into
// LDS.  The empty asm keeps the offset's zero-extension beside the load, so the compiler selects
// the scalar-base form of global_load_lds (one VGPR per lane offset) instead of hoisting a 64-bit
// address per offset out of the loop.
__device__ __forceinline__ void ring_load(const uint8_t* page, uint32_t off, uint8_t* dst) {
  asm volatile("" : "+v"(off));
  __builtin_amdgcn_global_load_lds(page + off, (lds_ptr_t)dst, 16, 0, kNontemporal);
}

struct VPage {
  int kind;   // 0 context, 1 drafted block, 2 none
  int valid;  // tokens present
  int bpos;   // drafted block position of token 0
};

__device__ __forceinline__ VPage vpage_info(const ItemCtx& it, const int32_t* ids, int ip) {
  VPage p;
  p.bpos = 0;
  const ReqDev& rq = it.rq;
  if (ip < it.nctx) {
    p.kind = ids[ip] < 0 ? 2 : 0;
    p.valid = p.kind == 0 ? min(kBlock, rq.ctx_len - kBlock * (it.p_lo + ip)) : 0;
  } else if (ip < it.npages) {
    const int j = ip - it.nctx;
    p.kind = 1;
    p.valid = min(kBlock, rq.q0 + rq.rows - kBlock * j);
    p.bpos = kBlock * j;
  } else {
    p.kind = 2;
    p.valid = 0;
  }
  return p;
}

__device__ __forceinline__ bool vkey_visible(const VPage& p, int tt, int qpos) {
  return tt < p.valid && (p.kind == 0 || p.bpos + tt <= qpos);
}

// Max / sum with the lane 32 positions away (the other half of a 32x32 MFMA column), on the
// VALU: v_permlane32_swap exchanges the two 32-lane halves of its operands, so with both
// operands equal to x each lane ends up holding its own value and its partner's.
__device__ __forceinline__ float half_swap_max(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Everything a verify work item keeps across its tiles.
template <int D>
struct VerifyState {
  static constexpr int NS = D / 16;  // MFMA k-steps of the score product
  static constexpr int ND = D / 32;  // 32-wide d blocks of the output
  static constexpr int NL = VRing<D>::kLoads;
  const int32_t* units;   // LDS: unit index of each context page of the item, -1 if invalid
  int64_t dummy_unit;     // block 0 of this (layer, kv head): a readable page for missing ones
  int64_t blk_unit0;      // drafted-block page 0 of this (request, layer, kv head)
  int ntiles, t_full;
  int pf_unit;            // unit of the page this wave loads next (read from LDS one tile early)
  int vst;                // value stage of the tile being consumed (t % 5)
  int ps;                 // page of every tile this wave loads
  bool kwave;             // loads keys (waves 0-3) or values (4-7)
  bool wave_on;           // the wave's row block holds rows
  bool shared_kv;         // other items (row groups) read the same K/V: loads keep lines in L2
  int kh, n, h, qpos;
  uint32_t lane_off[NL];  // byte offsets inside a page of this lane's loads
  uint32_t koff[NS];      // LDS offsets (inside a key stage) of this lane's score operands
  uint32_t voff;          // LDS offset of this lane's value operand (stage 0, page 2 kh, d block 0)
  u32x4 qreg[NS];         // query rows: B operand of S^T = K Q^T
  f32x16 acc_o[ND];
  float m_run, l_run, sc;
  float thr;              // headroom before the running maximum moves (rescale_headroom)
  float lim;              // 2^thr: a lane's tile weights summing below it need no row maxima;
                          // -1 while the running maximum is unset
  const uint8_t* kv_pool;  // the pool this wave loads from (K for key waves, V for value waves)
  const uint16_t* kv_blk;  // and its drafted-block array
};

// Global address of page `ip` of the item (scalar): a context page (its unit, or the dummy when
// the table entry is invalid), a drafted-block page, or the dummy past the item's pages.
template <int D>
__device__ __forceinline__ const uint8_t* verify_page(const uint8_t* pool_base, const uint16_t* blk,
                                                      const ItemCtx& it, const VerifyState<D>& vs, int ip,
                                                      int unit) {
  constexpr int P = VRing<D>::kPage;
  if (ip < it.nctx) {
    const int u = __builtin_amdgcn_readfirstlane(unit);
    return pool_base + (u >= 0 ? (int64_t)u : vs.dummy_unit) * P;
  }
  if (ip < it.npages) return reinterpret_cast<const uint8_t*>(blk) + (vs.blk_unit0 + (ip - it.nctx)) * P;
  return pool_base + vs.dummy_unit * P;
}

// Issue this wave's page of tile t into ring stage `stage`.  Every wave issues the same number
// of loads per tile (a missing page reads the dummy and is masked when consumed), so vmcnt
// counts are exact.
// SHARED: the loads keep their lines in L2 for other row groups of the unit (else they stream).
// CTX: tile t is one of the item's leading full, valid context tiles (t < t_full), whose pages
// are the units themselves.
// KW: the wave loads keys (1) or values (0), known at compile time, or -1 (read from vs.kwave).
template <int D, bool SHARED, bool CTX = false, int KW = -1>
__device__ __forceinline__ void verify_issue(const ItemCtx& it, const VerifyState<D>& vs, uint8_t* smem,
                                             int t, int stage, int unit) {
  using R = VRing<D>;
  const uint8_t* page;
  if constexpr (CTX)
    page = vs.kv_pool + (int64_t)__builtin_amdgcn_readfirstlane(unit) * R::kPage;
  else
    page = verify_page<D>(vs.kv_pool, vs.kv_blk, it, vs, 4 * t + vs.ps, unit);
  const bool kwave = KW >= 0 ? KW == 1 : vs.kwave;
  uint8_t* dst = smem + (kwave ? 0 : R::kV0) + stage * R::kTileK + vs.ps * R::kPage;  // stage < 4 (K) or < 5 (V)
#pragma unroll
  for (int i = 0; i < R::kLoads; ++i) {
    const void* src = page + vs.lane_off[i];
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(dst + i * 1024), 16, 0, SHARED ? kTemporal : kNontemporal);
  }
}

// wait until at most `tiles` of this wave's ring tiles are in flight
template <int D>
__device__ __forceinline__ void wait_tiles(int tiles) {
  constexpr int L = VRing<D>::kLoads;
  if (tiles >= 3) wait_vmem<3 * L>();
  else if (tiles == 2) wait_vmem<2 * L>();
  else if (tiles == 1) wait_vmem<L>();
  else wait_vmem<0>();
}

// S^T for this wave's 32 keys (key half kh) of the tile in key stage `st`
template <int D>
__device__ __forceinline__ f32x16 verify_scores(const uint8_t* smem, int st, const VerifyState<D>& vs) {
  using R = VRing<D>;
  f32x16 acc = f32x16{};
  const uint8_t* kst = smem + st * R::kTileK;
#pragma unroll
  for (int s = 0; s < VerifyState<D>::NS; ++s) {
    const u32x4 av = ld16(kst + vs.koff[s]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(av), as_bf(vs.qreg[s]), acc, 0, 0, 0);
  }
  return acc;
}

// Online softmax of one key half's scores and O^T += V^T P^T from value stage `vst` (the wide
// verify: its waves score a half and consume it in turn).  MASK: the tile holds a partial,
// missing or drafted-block page (per-key visibility and value masking); otherwise every key of
// the tile is a visible context key.
// Move a lane's running maximum to m_new (the work-group's moves are wave-uniform): rescale its
// sum and accumulators, and take the headroom and the fast-path bound from the rescaled sum.
template <int D>
__device__ __forceinline__ void verify_move(VerifyState<D>& vs, float m_new) {
  const float alpha = (vs.m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(vs.m_run - m_new);
  vs.l_run *= alpha;
  vs.thr = rescale_headroom(vs.l_run);
  vs.lim = (m_new == -INFINITY) ? -1.f : __builtin_ldexpf(1.f, (int)vs.thr);
#pragma unroll
  for (int i = 0; i < VerifyState<D>::ND; ++i) vs.acc_o[i] *= alpha;
  vs.m_run = m_new;
}

template <int D, bool MASK>
__device__ __forceinline__ void verify_consume(const ItemCtx& it, VerifyState<D>& vs, const uint8_t* smem,
                                               int t, int vst, f32x16 s_acc) {
  using R = VRing<D>;
  constexpr int ND = VerifyState<D>::ND;
  const int h = vs.h;
  VPage p0, p1;
  if constexpr (MASK) {
    p0 = vpage_info(it, vs.units, 4 * t + 2 * vs.kh);
    p1 = vpage_info(it, vs.units, 4 * t + 2 * vs.kh + 1);
    // register r holds key (page 2 kh + r / 8, token 8 h + r % 8) of row n
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (!vkey_visible(r < 8 ? p0 : p1, 8 * h + (r & 7), vs.qpos)) s_acc[r] = -INFINITY;
  }
  float mloc = max16(s_acc);
  mloc = half_swap_max(mloc);
  const float sc = vs.sc;
  const float m_new = fmaxf(vs.m_run, mloc * sc);
  if (__any(m_new > vs.m_run + vs.thr)) verify_move(vs, m_new);
  const float m_use = (vs.m_run == -INFINITY) ? 0.f : vs.m_run;
  uint32_t pb[8];
  float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const float e0 = __builtin_amdgcn_exp2f(fmaf(s_acc[r], sc, -m_use));
    const float e1 = __builtin_amdgcn_exp2f(fmaf(s_acc[r + 1], sc, -m_use));
    ls0 += e0;
    ls1 += e1;
    pb[r >> 1] = pack_bf16(e0, e1);
  }
  vs.l_run += ls0 + ls1;
  const uint8_t* vbase = smem + vst * R::kTileK + vs.voff;
#pragma unroll
  for (int pj = 0; pj < 2; ++pj) {
    const u32x4 bv = {pb[4 * pj], pb[4 * pj + 1], pb[4 * pj + 2], pb[4 * pj + 3]};
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      u32x4 av = ld16(vbase + pj * R::kPage + db * 1024);
      if constexpr (MASK) av = mask_tokens(av, 8 * h, (pj ? p1 : p0).valid);
      vs.acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(av), as_bf(bv), vs.acc_o[db], 0, 0, 0);
    }
  }
}

// Online softmax of tile t (scores s_acc) fused with the score product of tile t + 1 (key
// stage `stn`), for one wave: the running max moves first (the lazy rescale is a branch), so the
// exponentials of tile t, the score MFMAs of tile t + 1 and the value MFMAs of tile t sit in one
// basic block, which the compiler interleaves (a score chain alone in its own block overlapped
// nothing but the row max).  Returns the scores of tile t + 1.  MASK as in verify_consume.
template <int D, bool MASK>
__device__ __forceinline__ f32x16 verify_fused(const ItemCtx& it, VerifyState<D>& vs, const uint8_t* smem,
                                               int t, int stn, int vst, f32x16 s_acc) {
  using R = VRing<D>;
  constexpr int NS = VerifyState<D>::NS;
  constexpr int ND = VerifyState<D>::ND;
  const int h = vs.h;
  VPage p0, p1;
  if constexpr (MASK) {
    p0 = vpage_info(it, vs.units, 4 * t + 2 * vs.kh);
    p1 = vpage_info(it, vs.units, 4 * t + 2 * vs.kh + 1);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (!vkey_visible(r < 8 ? p0 : p1, 8 * h + (r & 7), vs.qpos)) s_acc[r] = -INFINITY;
  }
  const float sc = vs.sc;

  // score operands of tile t + 1, then its MFMA chain beside tile t's exponentials
  const uint8_t* kst = smem + stn * R::kTileK;
  u32x4 kop[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) kop[s] = ld16(kst + vs.koff[s]);
  f32x16 s_nxt = f32x16{};
#pragma unroll
  for (int s = 0; s < NS; ++s)
    s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(kop[s]), as_bf(vs.qreg[s]), s_nxt, 0, 0, 0);

  // Weights relative to the running maximum.  If every lane's weights sum below 2^thr, no score
  // is more than thr above the running maximum and the maximum stays: the row maxima are taken
  // (and the move rule applied to them, then the weights taken again after a move) only when
  // some lane's sum reaches the bound, or its maximum is unset.
  float e[16], ls[4];
  auto weights = [&]() {
    const float m_use = (vs.m_run == -INFINITY) ? 0.f : vs.m_run;
#pragma unroll
    for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(fmaf(s_acc[r], sc, -m_use));
#pragma unroll
    for (int r = 0; r < 4; ++r) ls[r] = e[r];
#pragma unroll
    for (int r = 4; r < 16; ++r) ls[r & 3] += e[r];
  };
  weights();
  if (__any(!((ls[0] + ls[1]) + (ls[2] + ls[3]) < vs.lim))) {
    float mloc = max16(s_acc);
    mloc = half_swap_max(mloc);
    const float m_new = fmaxf(vs.m_run, mloc * sc);
    if (__any(m_new > vs.m_run + vs.thr)) {
      verify_move(vs, m_new);
      weights();
    }
  }

  // value operands and the value product of tile t
  const uint8_t* vbase = smem + vst * R::kTileK + vs.voff;
  u32x4 vop[2][ND];
#pragma unroll
  for (int pj = 0; pj < 2; ++pj)
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      vop[pj][db] = ld16(vbase + pj * R::kPage + db * 1024);
      if constexpr (MASK) vop[pj][db] = mask_tokens(vop[pj][db], 8 * h, (pj ? p1 : p0).valid);
    }
  uint32_t pb[8];
#pragma unroll
  for (int r = 0; r < 16; r += 2) pb[r >> 1] = pack_bf16(e[r], e[r + 1]);
#pragma unroll
  for (int pj = 0; pj < 2; ++pj) {
    const u32x4 bv = {pb[4 * pj], pb[4 * pj + 1], pb[4 * pj + 2], pb[4 * pj + 3]};
#pragma unroll
    for (int db = 0; db < ND; ++db)
      vs.acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(vop[pj][db]), as_bf(bv), vs.acc_o[db], 0, 0, 0);
  }
  vs.l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);

  return s_nxt;
}

// One tile: wait for K(t + 1) (key waves) / V(t) (value waves), refill the dead stages (K(t + 4)
// into key stage t % 4, V(t + 3) into value stage (t - 1) % 4), score tile t + 1 into s_nxt (the
// last tile scores a stale stage, unused) and consume tile t.  STC >= 0: t % 4 == STC known at
// compile time.
template <int D, bool SHARED, int STC, bool MASK, bool STEADY = false, bool CTX = false, int KW = -1>
__device__ __forceinline__ void verify_step(const ItemCtx& it, VerifyState<D>& vs, uint8_t* smem, int t,
                                            f32x16& s_cur, f32x16& s_nxt) {
  const int st = STC >= 0 ? STC : (t & (kVStages - 1));
  const int ntiles = vs.ntiles;
  const bool kwave = KW >= 0 ? KW == 1 : vs.kwave;
  // keys: K(t + 1) must have landed (K issued up to t + 3); values: V(t) (V issued up to t + 3).
  // STEADY: t + 4 < ntiles, so both waits leave three tiles in flight and the refill is issued.
  if constexpr (STEADY) {
    if (kwave) wait_tiles<D>(2);
    else wait_tiles<D>(3);
  } else if (kwave) {
    if (t + 1 < ntiles) wait_tiles<D>(min(2, ntiles - t - 2));
  } else {
    wait_tiles<D>(min(3, ntiles - t - 1));
  }
  ring_barrier();
  // K(t + 4) into key stage t % 4 (K(t) was scored last tile), or V(t + 4) into value stage
  // (t + 4) % 5 (V(t - 1) was consumed last tile), with the page unit read one tile earlier;
  // then read the unit for the next tile's load
  const int vst = vs.vst;
  const int vst4 = vst == 0 ? kVVStages - 1 : vst - 1;  // (t + 4) % 5
  if (STEADY || t + 4 < ntiles) verify_issue<D, SHARED, CTX, KW>(it, vs, smem, t + 4, kwave ? st : vst4, vs.pf_unit);
  {
    // (CTX: tile t + 5 is a full context tile too, except at the last step of a group of four)
    const int ipn = 4 * (t + 5) + vs.ps;
    vs.pf_unit = ((CTX && STC >= 0 && STC < 3) || ipn < it.nctx) ? vs.units[ipn] : -1;
  }
  vs.vst = vst == kVVStages - 1 ? 0 : vst + 1;
  if (!vs.wave_on) return;
  s_nxt = verify_fused<D, MASK>(it, vs, smem, t, (st + 1) & (kVStages - 1), vst, s_cur);
}

// Byte offset inside a K or V page of this lane's part of ring load i.  The LDS side of
// global_load_lds is lane-linear, so the XOR swizzle of the ring is applied by choosing which
// global 16-byte chunk each lane fetches: keys by swz_k of the key row, values (pages stored d
// major, 16 tokens of one channel per 32 bytes) by bit 3 of the channel.
template <int D>
__device__ __forceinline__ uint32_t ring_lane_off(bool key, int lane, int i) {
  if (key) {
    constexpr int CPR = D / 8;           // 16-byte chunks per key row
    constexpr int RPI = 1024 / (2 * D);  // key rows per load
    const int tk = RPI * i + lane / CPR, sl = lane % CPR;
    return tk * (2 * D) + ((sl ^ swz_k<D>(tk)) * 16);
  }
  const int dd = 32 * i + (lane >> 1), sl = lane & 1;
  return dd * 32 + ((sl ^ ((dd >> 3) & 1)) * 16);
}

// Start of a verify item (both verify work-group shapes): the query registers of `row`, the
// unit of every context page into LDS at `ids`, and the tile counts.  Returns with the
// work-group synchronised and this wave's vector memory loads complete, so the ring loop's vmcnt
// waits count ring loads only.
template <int D>
__device__ __forceinline__ void verify_begin(const AttnArgs& a, const ItemCtx& it, int row, VerifyState<D>& vs,
                                             int32_t* units, int nthreads) {
  constexpr int NS = VerifyState<D>::NS;
  const int tid = threadIdx.x;
  const ReqDev& rq = it.rq;
  const int G = a.G;
  const bool row_ok = row < it.rows_total;
  const int tok = row_ok ? row / G : 0;
  vs.qpos = rq.q0 + tok;
  vs.sc = a.scale_log2;
  {
    const uint16_t* qp = a.q + ((((int64_t)rq.slot * a.L + it.l) * a.xmax + rq.q0 + tok) * a.Hq +
                                it.g * G + (row_ok ? row % G : 0)) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) vs.qreg[s] = row_ok ? ld16(qp + 16 * s + 8 * vs.h) : u32x4{0, 0, 0, 0};
  }
  int* first_bad = units + kMaxChunkPages;
  {
    const PoolDev& pl = it.pool;
    vs.dummy_unit = (int64_t)it.l * pl.nblk * a.Hkv + it.g;
    vs.blk_unit0 = (((int64_t)rq.slot * a.L + it.l) * a.Hkv + it.g) * (a.xmax / kBlock);
    if (tid == 0) *first_bad = it.nctx;
    __syncthreads();
    const int32_t* pt = pl.page_table + (int64_t)rq.page_row * pl.max_pages + it.p_lo;
    for (int i = tid; i < it.nctx; i += nthreads) {
      const int phys = pt[i];
      const bool ok = phys >= 0 && phys < pl.nblk;
      units[i] = ok ? (int32_t)(vs.dummy_unit + (int64_t)phys * a.Hkv) : -1;
      if (!ok) {
        atomicMin(first_bad, i);
        if (phys != -1) report_bad_page(a.err, rq.page_row, it.p_lo + i, phys);
      }
    }
  }
  wait_vmem<0>();
  __syncthreads();
  vs.units = units;
  vs.ntiles = (it.npages + 3) >> 2;
  const int nfull = min(it.nctx, max(0, (rq.ctx_len - kBlock * it.p_lo) / kBlock));
  vs.t_full = min(nfull, *first_bad) >> 2;  // leading tiles of 4 full, valid context pages
#pragma unroll
  for (int i = 0; i < VerifyState<D>::ND; ++i) vs.acc_o[i] = f32x16{};
  vs.m_run = -INFINITY;
  vs.l_run = 0.f;
  vs.thr = 0.f;
  vs.lim = -1.f;
}

// Steady tiles of a verify item whose refills are leading full context tiles, four at a time,
// for a key (KW = 1) or value (KW = 0) wave; returns the first tile not taken.
template <int D, bool SHARED, int KW>
__device__ __forceinline__ int verify_ctx_tiles(const ItemCtx& it, VerifyState<D>& vs, uint8_t* smem, f32x16& s_a,
                                                f32x16& s_b) {
  int t = 0;
  for (; t + 7 < vs.t_full; t += 4) {
    verify_step<D, SHARED, 0, false, true, true, KW>(it, vs, smem, t, s_a, s_b);
    verify_step<D, SHARED, 1, false, true, true, KW>(it, vs, smem, t + 1, s_b, s_a);
    verify_step<D, SHARED, 2, false, true, true, KW>(it, vs, smem, t + 2, s_a, s_b);
    verify_step<D, SHARED, 3, false, true, true, KW>(it, vs, smem, t + 3, s_b, s_a);
  }
  return t;
}

// The ring loop of a verify item: prologue, then full tiles (no masking) four at a time, so ring
// stages are compile-time and the scores alternate between s_a and s_b without register copies;
// then the rest, with masking.  The accumulators are left in vs.
template <int D, bool SHARED>
__device__ __forceinline__ void verify_tiles(const ItemCtx& it, VerifyState<D>& vs, uint8_t* smem,
                                          const int32_t* units) {
  const int ntiles = vs.ntiles;
  // prologue: K(0..3) and V(0..3) into stages 0..3; scores of tile 0
  const int kpro = min(ntiles, 4);
  for (int j = 0; j < kpro; ++j) {
    const int ip = 4 * j + vs.ps;
    verify_issue<D, SHARED>(it, vs, smem, j, j, ip < it.nctx ? units[ip] : -1);
  }
  {
    const int ipn = 4 * 4 + vs.ps;
    vs.pf_unit = ipn < it.nctx ? units[ipn] : -1;
  }
  vs.vst = 0;
  if (vs.kwave) wait_tiles<D>(kpro - 1);  // K(0)
  ring_barrier();
  f32x16 s_a = vs.wave_on ? verify_scores<D>(smem, 0, vs) : f32x16{};
  f32x16 s_b = f32x16{};

  int t = 0;
  // steady state: every step of the group issues its refill (t + 7 < ntiles); while the
  // refills are full context tiles too (t + 7 < t_full) their pages are the units themselves,
  // and the wave's role (keys or values) is a compile-time constant
  if (vs.kwave) t = verify_ctx_tiles<D, SHARED, 1>(it, vs, smem, s_a, s_b);
  else t = verify_ctx_tiles<D, SHARED, 0>(it, vs, smem, s_a, s_b);
  for (; t + 3 < vs.t_full && t + 7 < ntiles; t += 4) {
    verify_step<D, SHARED, 0, false, true>(it, vs, smem, t, s_a, s_b);
    verify_step<D, SHARED, 1, false, true>(it, vs, smem, t + 1, s_b, s_a);
    verify_step<D, SHARED, 2, false, true>(it, vs, smem, t + 2, s_a, s_b);
    verify_step<D, SHARED, 3, false, true>(it, vs, smem, t + 3, s_b, s_a);
  }
  for (; t + 3 < vs.t_full; t += 4) {
    verify_step<D, SHARED, 0, false>(it, vs, smem, t, s_a, s_b);
    verify_step<D, SHARED, 1, false>(it, vs, smem, t + 1, s_b, s_a);
    verify_step<D, SHARED, 2, false>(it, vs, smem, t + 2, s_a, s_b);
    verify_step<D, SHARED, 3, false>(it, vs, smem, t + 3, s_b, s_a);
  }
  for (; t < vs.t_full; ++t) {
    verify_step<D, SHARED, -1, false>(it, vs, smem, t, s_a, s_b);
    s_a = s_b;
  }
  for (; t < ntiles; ++t) {
    verify_step<D, SHARED, -1, true>(it, vs, smem, t, s_a, s_b);
    s_a = s_b;
  }
}

template <int D>
__device__ __forceinline__ void verify_item(const AttnArgs& a, const ItemCtx& it, int rg, uint8_t* smem) {
  using R = VRing<D>;
  using VS = VerifyState<D>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;
  const int rb = w & 3;
  const int row = rg * 128 + 32 * rb + n;
  const bool row_ok = row < it.rows_total;

  VS vs;
  vs.kh = w >> 2;
  vs.n = n;
  vs.h = h;
  vs.kwave = w < 4;
  vs.ps = w & 3;
  vs.wave_on = rg * 128 + 32 * rb < it.rows_total;
  vs.shared_kv = it.rq.nrg > 1;
  int32_t* units = reinterpret_cast<int32_t*>(smem + R::kIds);
  verify_begin<D>(a, it, row, vs, units, kVThreads);
  const int ntiles = vs.ntiles;

#pragma unroll
  for (int i = 0; i < VS::NL; ++i) vs.lane_off[i] = ring_lane_off<D>(vs.kwave, lane, i);
  {
    const int key = 32 * vs.kh + key_of_m32(n);
    const int ksw = swz_k<D>(key);
#pragma unroll
    for (int s = 0; s < VS::NS; ++s) vs.koff[s] = key * (2 * D) + (((2 * s + h) ^ ksw) * 16);
    vs.voff = R::kV0 + 2 * vs.kh * R::kPage + n * 32 + ((h ^ ((n >> 3) & 1)) * 16);
  }

  // K and V are chosen by value here, once: choosing between descriptor fields by reference
  // would make the compiler copy the kernel argument block to scratch
  vs.kv_pool = vs.kwave ? it.pool.k : it.pool.v;
  vs.kv_blk = vs.kwave ? a.blk_k : a.blk_v;
  if (vs.shared_kv) verify_tiles<D, true>(it, vs, smem, units);  // wave-uniform
  else verify_tiles<D, false>(it, vs, smem, units);

  // merge the two key halves of every row block through LDS (the ring is free now)
  __syncthreads();
  constexpr int ND = VS::ND;
  constexpr int NR = ND * 16;  // accumulator floats per lane
  float* red = reinterpret_cast<float*>(smem) + rb * (64 * (NR + 2));
  if (vs.kh == 1 && vs.wave_on) {
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(red + ((db * 4 + q) * 64 + lane) * 4) =
            f32x4{vs.acc_o[db][4 * q], vs.acc_o[db][4 * q + 1], vs.acc_o[db][4 * q + 2], vs.acc_o[db][4 * q + 3]};
    red[NR * 64 + lane] = vs.m_run;
    red[NR * 64 + 64 + lane] = vs.l_run;
  }
  __syncthreads();
  if (vs.kh == 1 || !vs.wave_on) return;
  const float m1 = red[NR * 64 + lane], l1 = red[NR * 64 + 64 + lane];
  const float M = fmaxf(vs.m_run, m1);
  const float f0 = (vs.m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(vs.m_run - M);
  const float f1 = (m1 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
  const float l_tot = half_swap_sum(f0 * vs.l_run + f1 * l1);
  if (!row_ok) return;
  bool partial;
  float* dst = out_row<D>(a, it, row, &partial);
  const float inv = partial ? 1.f : (l_tot > 0.f ? 1.f / l_tot : 0.f);
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 o1 = *reinterpret_cast<const f32x4*>(red + ((db * 4 + q) * 64 + lane) * 4);
      f32x4 o = {vs.acc_o[db][4 * q], vs.acc_o[db][4 * q + 1], vs.acc_o[db][4 * q + 2], vs.acc_o[db][4 * q + 3]};
      o = (f0 * o + f1 * o1) * inv;
      *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * q + 4 * h) = o;
    }
  if (partial && h == 0) {
    dst[D] = M;
    dst[D + 1] = l_tot;
  }
}

// ------------------------------------------------------------------ wide verify
// Verify launches with more than 128 query rows per (layer, kv head) (x * G > 128, e.g. G = 8
// and x = 40) take up to 384 rows in one work item, one wave per 32 rows (up to 12 waves, 3 per
// SIMD), so a unit's K/V pages stream through a CU once for all its rows instead of once per
// 128-row group.  Each wave scores both 32-key halves of every 64-key tile and folds each half
// into its online softmax in turn; no key halves are merged at the end.  K and V pages go into
// a 4-stage ring each (stages hold 64-key tiles; tile t + 3 is loaded while tile t is
// consumed).  The 8 pages of a tile are dealt over the waves as ring slots, slot s < 4 being key
// page s and slot s >= 4 value page s - 4: wave w loads slots w and w + waves (those below 8).
constexpr int kWStages = 4;
constexpr int kWThreads = 64 * kWideMaxWaves;

template <int D>
struct WRing {
  static constexpr int kPage = kBlock * D * 2;
  static constexpr int kTile = 4 * kPage;
  static constexpr int kV0 = kWStages * kTile;  // value stages after the key stages
  static constexpr int kIds = 2 * kWStages * kTile;
  static constexpr int kBytes = kIds + kMaxChunkPages * 4 + 16;
  static constexpr int kLoads = kPage / 1024;
};
// the value product (verify_consume) addresses value stage j at kV0 + j * kTile of either ring
static_assert(WRing<128>::kV0 == VRing<128>::kV0 && WRing<64>::kV0 == VRing<64>::kV0, "value stage base");
static_assert(WRing<128>::kTile == VRing<128>::kTileK && WRing<64>::kTile == VRing<64>::kTileK, "stage size");

// ring_lane_off(key, lane, i) == ring_lane_off(key, lane, 0) ^ (i * step): load i of a page
// covers the next 1 KB (keys: 4 rows of 256 bytes or 8 of 128, the row swizzle advancing by
// 4 or 8 with them; values: 32 channels of 32 bytes)
__device__ __forceinline__ uint32_t ring_load_step(bool key) { return key ? 1088u : 1024u; }

struct WideLoads {
  int nslot;  // ring slots this wave loads: 0, 1 or 2 (the planner uses at least 5 waves)
  int s0, s1;
  int pf0, pf1;         // units of the pages the slots load next (read from LDS a tile early)
  uint32_t off0, off1;  // lane offsets of each slot's load 0 (see ring_load_step)
  // each slot's pool and drafted-block array (K for slots 0-3, V for 4-7), chosen once by value
  const uint8_t* pool0;
  const uint8_t* pool1;
  const uint16_t* blk0;
  const uint16_t* blk1;
};

// Unit of context page ip of the item, -1 past the context (drafted block or nothing).
__device__ __forceinline__ int unit_at(const int32_t* units, const ItemCtx& it, int ip) {
  return ip < it.nctx ? units[ip] : -1;
}

// Issue ring slot `slot` of tile t into stage `stage`.
// CTX: tile t is one of the item's leading full, valid context tiles (its pages are the units).
template <int D, bool CTX = false>
__device__ __forceinline__ void wide_issue(const ItemCtx& it, const VerifyState<D>& vs, uint8_t* smem, int slot,
                                           const uint8_t* pool, const uint16_t* blk, uint32_t off, int t,
                                           int stage, int unit) {
  using R = WRing<D>;
  const int ps = slot & 3;
  const bool key = slot < 4;
  const uint8_t* page;
  if constexpr (CTX)
    page = pool + (int64_t)__builtin_amdgcn_readfirstlane(unit) * R::kPage;
  else
    page = verify_page<D>(pool, blk, it, vs, 4 * t + ps, unit);
  uint8_t* dst = smem + (key ? 0 : R::kV0) + stage * R::kTile + ps * R::kPage;
  const uint32_t step = ring_load_step(key);
  asm volatile("" : "+v"(off));  // derive the load offsets here, not as registers held in the loop
#pragma unroll
  for (int i = 0; i < R::kLoads; ++i) ring_load(page, off ^ (i * step), dst + i * 1024);
}

// wait until this wave's ring loads of the current tile have landed, with `ahead` (0..2) later
// tiles' loads still in flight
template <int D>
__device__ __forceinline__ void wide_wait(int nslot, int ahead) {
  constexpr int L = WRing<D>::kLoads;
  if (nslot == 1) {
    if (ahead >= 2) wait_vmem<2 * L>();
    else if (ahead == 1) wait_vmem<L>();
    else wait_vmem<0>();
  } else if (nslot == 2) {
    if (ahead >= 2) wait_vmem<4 * L>();
    else if (ahead == 1) wait_vmem<2 * L>();
    else wait_vmem<0>();
  }
}

// S^T for key half KH of the tile in key stage `st`.  kx = key row * 2D | ((h ^ swz_k) << 4):
// the XOR-swizzled chunk (2 s + h) ^ swz_k of the row is kx ^ (32 s), the row offset having
// zero low bits.
template <int D, int KH>
__device__ __forceinline__ f32x16 wide_scores(const uint8_t* smem, int st, uint32_t kx, const u32x4* qreg) {
  constexpr int NS = VerifyState<D>::NS;
  const uint8_t* kst = smem + st * WRing<D>::kTile + KH * 32 * (2 * D);
  u32x4 av[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) av[s] = ld16(kst + (kx ^ (32u * s)));
  f32x16 acc = f32x16{};
#pragma unroll
  for (int s = 0; s < NS; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(av[s]), as_bf(qreg[s]), acc, 0, 0, 0);
  return acc;
}

// One tile: wait for tile t, refill the stage freed by tile t - 1 with tile t + 3, then both
// key halves of tile t, one after the other.  STC >= 0: t % 4 == STC known at compile time.
template <int D, int STC, bool MASK, bool SPLIT, bool CTX = false>
__device__ __forceinline__ void wide_step(const ItemCtx& it, VerifyState<D>& vs, WideLoads& ld, uint8_t* smem,
                                          int t, uint32_t kx, uint32_t voff0, int kh_only) {
  const int st = STC >= 0 ? STC : (t & (kWStages - 1));
  const int ntiles = vs.ntiles;
  // (CTX: tile t + 3 is a full context tile, so two tiles are always ahead; so is tile t + 4,
  // whose units are read next, except at the last step of a group of four)
  wide_wait<D>(ld.nslot, CTX ? 2 : min(2, ntiles - 1 - t));
  ring_barrier();
  if (CTX || t + 3 < ntiles) {
    const int sn = (st + 3) & (kWStages - 1);
    if (ld.nslot >= 1) wide_issue<D, CTX>(it, vs, smem, ld.s0, ld.pool0, ld.blk0, ld.off0, t + 3, sn, ld.pf0);
    if (ld.nslot == 2) wide_issue<D, CTX>(it, vs, smem, ld.s1, ld.pool1, ld.blk1, ld.off1, t + 3, sn, ld.pf1);
  }
  if constexpr (CTX && STC >= 0 && STC < 3) {
    ld.pf0 = vs.units[4 * (t + 4) + (ld.s0 & 3)];
    ld.pf1 = vs.units[4 * (t + 4) + (ld.s1 & 3)];
  } else {
    ld.pf0 = unit_at(vs.units, it, 4 * (t + 4) + (ld.s0 & 3));
    ld.pf1 = unit_at(vs.units, it, 4 * (t + 4) + (ld.s1 & 3));
  }
  if (!vs.wave_on) return;
  asm volatile("" : "+v"(kx));  // the 8 operand offsets kx ^ 32 s are derived here, not held
  if constexpr (SPLIT) {  // one key half (kh_only) of a shared row block
    vs.kh = kh_only;
    vs.voff = voff0 + 2 * WRing<D>::kPage * kh_only;
    verify_consume<D, MASK>(it, vs, smem, t, st, wide_scores<D, 0>(smem + kh_only * 32 * (2 * D), st, kx, vs.qreg));
  } else {
    vs.kh = 0;
    vs.voff = voff0;
    verify_consume<D, MASK>(it, vs, smem, t, st, wide_scores<D, 0>(smem, st, kx, vs.qreg));
    vs.kh = 1;
    vs.voff = voff0 + 2 * WRing<D>::kPage;
    verify_consume<D, MASK>(it, vs, smem, t, st, wide_scores<D, 1>(smem, st, kx, vs.qreg));
  }
}

// The tile loop of a wide verify wave: full tiles four at a time with compile-time ring stages,
// then the rest, then the masked tiles.  SPLIT: the wave takes one key half of every tile.
template <int D, bool SPLIT>
__device__ __forceinline__ void wide_loop(const ItemCtx& it, VerifyState<D>& vs, WideLoads& ld, uint8_t* smem,
                                          uint32_t kx, uint32_t voff0, int kh_only) {
  const int ntiles = vs.ntiles;
  int t = 0;
  // while the refills (tiles t + 3 .. t + 6) are leading full context tiles too, their pages
  // are the units themselves
  for (; t + 6 < vs.t_full; t += 4) {
    wide_step<D, 0, false, SPLIT, true>(it, vs, ld, smem, t, kx, voff0, kh_only);
    wide_step<D, 1, false, SPLIT, true>(it, vs, ld, smem, t + 1, kx, voff0, kh_only);
    wide_step<D, 2, false, SPLIT, true>(it, vs, ld, smem, t + 2, kx, voff0, kh_only);
    wide_step<D, 3, false, SPLIT, true>(it, vs, ld, smem, t + 3, kx, voff0, kh_only);
  }
  for (; t + 3 < vs.t_full; t += 4) {
    wide_step<D, 0, false, SPLIT>(it, vs, ld, smem, t, kx, voff0, kh_only);
    wide_step<D, 1, false, SPLIT>(it, vs, ld, smem, t + 1, kx, voff0, kh_only);
    wide_step<D, 2, false, SPLIT>(it, vs, ld, smem, t + 2, kx, voff0, kh_only);
    wide_step<D, 3, false, SPLIT>(it, vs, ld, smem, t + 3, kx, voff0, kh_only);
  }
  for (; t < vs.t_full; ++t) wide_step<D, -1, false, SPLIT>(it, vs, ld, smem, t, kx, voff0, kh_only);
  for (; t < ntiles; ++t) wide_step<D, -1, true, SPLIT>(it, vs, ld, smem, t, kx, voff0, kh_only);
}

template <int D>
__device__ void verify_wide_item(const AttnArgs& a, const ItemCtx& it, int rg, uint8_t* smem) {
  using R = WRing<D>;
  using VS = VerifyState<D>;
  const int nrb = a.vwaves;  // 32-row blocks per item
  int nfull;
  const int nw = wide_waves(nrb, &nfull);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;
  // a whole row block (both key halves of every tile), or one key half of a shared block
  const bool split = w >= nfull;
  const int rb = split ? nfull + ((w - nfull) >> 1) : w;
  const int kh_only = split ? ((w - nfull) & 1) : -1;
  const int rows0 = rg * 32 * nrb + 32 * rb;  // first row of this wave
  const int row = rows0 + n;
  const bool row_ok = row < it.rows_total;

  VS vs;
  vs.n = n;
  vs.h = h;
  vs.wave_on = rows0 < it.rows_total;
  vs.shared_kv = false;  // the wide ring loads (wide_issue) always stream
  int32_t* units = reinterpret_cast<int32_t*>(smem + R::kIds);
  verify_begin<D>(a, it, row, vs, units, 64 * nw);
  const int ntiles = vs.ntiles;

  WideLoads ld;
  ld.s0 = w;
  ld.s1 = w + nw;
  ld.nslot = (ld.s0 < 8) + (ld.s1 < 8);
  ld.off0 = ring_lane_off<D>(ld.s0 < 4, lane, 0);
  ld.off1 = ring_lane_off<D>(ld.s1 < 4, lane, 0);
  ld.pool0 = ld.s0 < 4 ? it.pool.k : it.pool.v;
  ld.pool1 = ld.s1 < 4 ? it.pool.k : it.pool.v;
  ld.blk0 = ld.s0 < 4 ? a.blk_k : a.blk_v;
  ld.blk1 = ld.s1 < 4 ? a.blk_k : a.blk_v;
  const int key = key_of_m32(n);
  const uint32_t kx = key * (2 * D) | ((h ^ swz_k<D>(key)) << 4);
  const uint32_t voff0 = R::kV0 + n * 32 + ((h ^ ((n >> 3) & 1)) * 16);

  // prologue: tiles 0..2 into stages 0..2
  const int kpro = min(ntiles, 3);
  for (int j = 0; j < kpro; ++j) {
    if (ld.nslot >= 1)
      wide_issue<D>(it, vs, smem, ld.s0, ld.pool0, ld.blk0, ld.off0, j, j, unit_at(units, it, 4 * j + (ld.s0 & 3)));
    if (ld.nslot == 2)
      wide_issue<D>(it, vs, smem, ld.s1, ld.pool1, ld.blk1, ld.off1, j, j, unit_at(units, it, 4 * j + (ld.s1 & 3)));
  }
  ld.pf0 = unit_at(units, it, 12 + (ld.s0 & 3));
  ld.pf1 = unit_at(units, it, 12 + (ld.s1 & 3));

  if (split) wide_loop<D, true>(it, vs, ld, smem, kx, voff0, kh_only);
  else wide_loop<D, false>(it, vs, ld, smem, kx, voff0, kh_only);

  // the two halves of a shared row block merge through LDS (the ring is free now): the key-half-1
  // wave leaves its state, the key-half-0 wave combines and writes
  constexpr int NR = VS::ND * 16;  // accumulator floats per lane
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem) + (split ? ((w - nfull) >> 1) : 0) * (64 * (NR + 2));
  if (kh_only == 1 && vs.wave_on) {
#pragma unroll
    for (int db = 0; db < VS::ND; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(red + ((db * 4 + q) * 64 + lane) * 4) =
            f32x4{vs.acc_o[db][4 * q], vs.acc_o[db][4 * q + 1], vs.acc_o[db][4 * q + 2], vs.acc_o[db][4 * q + 3]};
    red[NR * 64 + lane] = vs.m_run;
    red[NR * 64 + 64 + lane] = vs.l_run;
  }
  __syncthreads();
  if (kh_only == 1 || !vs.wave_on) return;
  float M = vs.m_run, f0 = 1.f, f1 = 0.f, l_own = vs.l_run;
  if (split) {
    const float m1 = red[NR * 64 + lane], l1 = red[NR * 64 + 64 + lane];
    M = fmaxf(vs.m_run, m1);
    f0 = (vs.m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(vs.m_run - M);
    f1 = (m1 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
    l_own = f0 * vs.l_run + f1 * l1;
  }
  // the row's keys are split over the two 32-lane halves (tokens 8 h .. 8 h + 7 of each page)
  const float l_tot = half_swap_sum(l_own);
  if (!row_ok) return;
  bool partial;
  float* dst = out_row<D>(a, it, row, &partial);
  const float inv = partial ? 1.f : (l_tot > 0.f ? 1.f / l_tot : 0.f);
#pragma unroll
  for (int db = 0; db < VS::ND; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4 o = f32x4{vs.acc_o[db][4 * q], vs.acc_o[db][4 * q + 1], vs.acc_o[db][4 * q + 2], vs.acc_o[db][4 * q + 3]};
      if (split) o = f0 * o + f1 * *reinterpret_cast<const f32x4*>(red + ((db * 4 + q) * 64 + lane) * 4);
      *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * q + 4 * h) = o * inv;
    }
  if (partial && h == 0) {
    dst[D] = M;
    dst[D + 1] = l_tot;
  }
}

// Combine the NW waves' softmax states of a draft item (rows n < 16, lane (n, kg) holding
// channels 16 db + 4 kg .. + 3) through LDS and write the rows (or the split partials).
template <int D, int NW>
__device__ __forceinline__ void draft_merge(const AttnArgs& a, const ItemCtx& it, uint8_t* smem,
                                            const f32x4* acc_o, float m_run, float l_run) {
  constexpr int ND = D / 16;
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, kg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar loop control
  float* red = reinterpret_cast<float*>(smem);  // [wave][16 rows][D + 4]
  constexpr int RS = D + 4;
#pragma unroll
  for (int db = 0; db < ND; ++db)
    *reinterpret_cast<f32x4*>(red + (w * 16 + n) * RS + 16 * db + 4 * kg) = acc_o[db];
  if (kg == 0) {
    red[(w * 16 + n) * RS + D] = m_run;
    red[(w * 16 + n) * RS + D + 1] = l_run;
  }
  __syncthreads();
  constexpr int NQ = D / 4;  // float4 chunks per row
  for (int task = tid; task < 16 * NQ; task += 64 * NW) {
    const int rr = task / NQ, cq = task % NQ;
    if (rr >= it.rows_total) continue;
    float mw[NW], M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      mw[ww] = red[(ww * 16 + rr) * RS + D];
      M = fmaxf(M, mw[ww]);
    }
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float f = (mw[ww] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw[ww] - M);
      lsum += f * red[(ww * 16 + rr) * RS + D + 1];
      const f32x4 ow = *reinterpret_cast<const f32x4*>(red + (ww * 16 + rr) * RS + 4 * cq);
      o += f * ow;
    }
    bool partial;
    float* dst = out_row<D>(a, it, rr, &partial);
    if (!partial) o *= lsum > 0.f ? 1.f / lsum : 0.f;
    *reinterpret_cast<f32x4*>(dst + 4 * cq) = o;
    if (partial && cq == 0) {
      dst[D] = M;
      dst[D + 1] = lsum;
    }
  }
}


// ------------------------------------------------------------------ draft path, bf16 caches
// A draft step has G <= 16 query rows, so the work is a stream over the item's pages with little
// arithmetic per byte.  Every wave takes pages w, w + NW, w + 2 NW, ... of the item and streams
// them through a private ring of STG one-page slots (keys then values) in LDS, filled with
// global_load_lds_dwordx4 STG - 1 pages ahead; a wave reads only what it loaded itself, so the
// loop has no barrier, only the wave's own vmcnt wait.  Scores S^T = K Q^T use
// v_mfma_f32_16x16x32_bf16 (rows padded to 16); the softmax weights then sit exactly where the
// B operand of v_mfma_f32_16x16x16_bf16 wants them for O^T += V^T P^T.
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D>
struct DRing {
  static constexpr int kPage = kBlock * D * 2;  // bytes of one K or V page
  static constexpr int kSlot = 2 * kPage;       // one page of keys then one of values
  static constexpr int kLoads = kPage / 1024;   // 16-byte-per-lane loads per page and tensor
  static constexpr int kRing = 16 * kSlot;      // LDS the rings may take (8 waves x 2 slots in a mixed launch)
  static constexpr int kIds = kRing;
  static constexpr int kBytes = kRing + kMaxChunkPages * 4;
};

// XOR swizzle of a key row's 16-byte chunks (conflict-free 16-byte reads of 16 rows)
template <int D>
__device__ __forceinline__ int dswz(int tok) {
  return D == 128 ? (tok & 15) : (tok & 7);
}

// wait for this wave's loads of the page it consumes next (N loads may stay in flight), then
// keep the compiler from moving LDS reads above the wait
template <int N>
__device__ __forceinline__ void ring_wait_own() {
  wait_vmem<N>();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int D, bool V>
__device__ __forceinline__ void draft_issue_kv(const uint8_t* pool_base, const uint16_t* blk,
                                               const AttnArgs& a, const ItemCtx& it,
                                               const int32_t* ids, uint8_t* slot, int ip, int lane) {
  using R = DRing<D>;
  const uint8_t* page;
  if (ip < it.nctx || ip >= it.npages) {
    int phys = ip < it.nctx ? ids[ip] : 0;
    if (phys < 0) phys = 0;  // missing page: block 0 (in bounds), masked when consumed
    page = pool_base + (((int64_t)it.l * it.pool.nblk + phys) * a.Hkv + it.g) * R::kPage;
  } else {
    const int64_t unit = (((int64_t)it.rq.slot * a.L + it.l) * a.Hkv + it.g) * (a.xmax / kBlock) +
                         (ip - it.nctx);
    page = reinterpret_cast<const uint8_t*>(blk) + unit * R::kPage;
  }
  uint8_t* dst = slot + (V ? R::kPage : 0);
#pragma unroll
  for (int i = 0; i < R::kLoads; ++i) {
    int off;
    if constexpr (!V) {
      constexpr int CPR = D / 8;
      constexpr int RPI = 1024 / (2 * D);
      const int tok = RPI * i + lane / CPR, s = lane % CPR;
      off = tok * (2 * D) + ((s ^ dswz<D>(tok)) * 16);
    } else {
      const int dd = 32 * i + (lane >> 1), s = lane & 1;
      off = dd * 32 + ((s ^ ((dd >> 2) & 1)) * 16);
    }
    __builtin_amdgcn_global_load_lds(page + off, (lds_ptr_t)(dst + i * 1024), 16, 0, kNontemporal);
  }
}

// zero the bf16 lanes t (0..3) of an 8-byte chunk with first + t >= valid
__device__ __forceinline__ u32x2 mask_tokens4(u32x2 v, int first, int valid) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    uint32_t x = v[i];
    if (first + 2 * i >= valid) x &= 0xFFFF0000u;
    if (first + 2 * i + 1 >= valid) x &= 0x0000FFFFu;
    v[i] = x;
  }
  return v;
}

// LDS of a bf16 draft work-group of NW waves with STG ring slots each: the rings, then the page
// ids of the item
template <int D, int NW, int STG>
constexpr int draft_bf16_lds() { return NW * STG * DRing<D>::kSlot + kMaxChunkPages * 4; }

template <int D, int NW, int STG>
__device__ __forceinline__ void draft_bf16_item(const AttnArgs& a, const ItemCtx& it, uint8_t* smem) {
  using R = DRing<D>;
  static_assert(NW * STG * R::kSlot <= R::kRing, "draft rings exceed their LDS");
  constexpr int kIdsOff = NW * STG * R::kSlot;
  constexpr int NS = D / 32;  // k-steps of the score product
  constexpr int ND = D / 16;  // 16-wide d blocks of the output
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, kg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar loop control
  const ReqDev& rq = it.rq;
  const int G = a.G;
  const bool row_ok = n < it.rows_total;
  const int tok = row_ok ? n / G : 0;
  const int qpos = rq.q0 + tok;

  u32x4 qreg[NS];
  {
    const uint16_t* qp = a.q + ((((int64_t)rq.slot * a.L + it.l) * a.xmax + rq.q0 + tok) * a.Hq +
                                it.g * G + (row_ok ? n % G : 0)) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) qreg[s] = row_ok ? ld16(qp + 32 * s + 8 * kg) : u32x4{0, 0, 0, 0};
  }
  int32_t* ids = reinterpret_cast<int32_t*>(smem + kIdsOff);
  {
    const PoolDev& pl = it.pool;
    const int32_t* pt = pl.page_table + (int64_t)rq.page_row * pl.max_pages + it.p_lo;
    for (int i = tid; i < it.nctx; i += 64 * NW) {
      const int phys = pt[i];
      const bool ok = phys >= 0 && phys < pl.nblk;
      ids[i] = ok ? phys : -1;
      if (!ok && phys != -1) report_bad_page(a.err, rq.page_row, it.p_lo + i, phys);
    }
  }
  wait_vmem<0>();
  __syncthreads();

  uint8_t* ring = smem + w * (STG * R::kSlot);
  const int mine = it.npages > w ? (it.npages - w + NW - 1) / NW : 0;
  auto issue = [&](int k) {
    uint8_t* slot = ring + (k % STG) * R::kSlot;
    const int ip = w + NW * k;
    draft_issue_kv<D, false>(it.pool.k, a.blk_k, a, it, ids, slot, ip, lane);
    draft_issue_kv<D, true>(it.pool.v, a.blk_v, a, it, ids, slot, ip, lane);
  };
#pragma unroll
  for (int k = 0; k < STG - 1; ++k)
    if (k < mine) issue(k);

  f32x4 acc_o[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc_o[i] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sc = a.scale_log2;
  constexpr int PER = 2 * R::kLoads;  // loads per page

  for (int k = 0; k < mine; ++k) {
    const int ahead = min(STG - 2, mine - 1 - k);
    if (STG > 3 && ahead >= 2) ring_wait_own<2 * PER>();
    else if (STG > 2 && ahead >= 1) ring_wait_own<PER>();
    else ring_wait_own<0>();
    if (k + STG - 1 < mine) issue(k + STG - 1);

    const uint8_t* sk = ring + (k % STG) * R::kSlot;
    const uint8_t* sv = sk + R::kPage;
    // S^T: lane (n, kg) ends with keys 4kg..4kg+3 of row n
    f32x4 s_acc = f32x4{};
    {
      const uint8_t* krow = sk + n * (2 * D);
      const int sw = dswz<D>(n);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const u32x4 av = ld16(krow + (((4 * s + kg) ^ sw) * 16));
        s_acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(av), as_bf(qreg[s]), s_acc, 0, 0, 0);
      }
    }
    const VPage pg = vpage_info(it, ids, w + NW * k);
    const bool full = pg.kind == 0 && pg.valid == kBlock;
    if (!full) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!vkey_visible(pg, 4 * kg + i, qpos)) s_acc[i] = -INFINITY;
    }
    float mloc = fmaxf(fmaxf(s_acc[0], s_acc[1]), fmaxf(s_acc[2], s_acc[3]));
    mloc = wave_xor_max(mloc, 16);
    mloc = wave_xor_max(mloc, 32);
    const float m_new = fmaxf(m_run, mloc * sc);
    if (__any(m_new > m_run + kRescaleBf16)) {
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < ND; ++i) acc_o[i] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = __builtin_amdgcn_exp2f(fmaf(s_acc[i], sc, -m_use));
    l_run += (e[0] + e[1]) + (e[2] + e[3]);
    const u32x2 pbits = {pack_bf16(e[0], e[1]), pack_bf16(e[2], e[3])};
    const s16x4 pv = __builtin_bit_cast(s16x4, pbits);
    // O^T += V^T P^T: lane (m, kg) feeds channel 16 db + m, tokens 4kg..4kg+3
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const int dd = 16 * db + n;
      u32x2 av = *reinterpret_cast<const u32x2*>(sv + dd * 32 + ((((kg >> 1) ^ ((dd >> 2) & 1))) * 16) +
                                                 (kg & 1) * 8);
      if (!full) av = mask_tokens4(av, 4 * kg, pg.valid);
      acc_o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, av), pv, acc_o[db],
                                                            0, 0, 0);
    }
  }

  // ---- merge the waves' states through LDS (rings are free once every wave is here)
  __syncthreads();
  l_run = wave_xor_sum(l_run, 16);
  l_run = wave_xor_sum(l_run, 32);
  draft_merge<D, NW>(a, it, smem, acc_o, m_run, l_run);
}

// ------------------------------------------------------------------ draft path, KIVI caches (16x16x32)
// Channel order of the draft path: lane group kg (lane / 16) owns channels [kg*D/4, (kg+1)*D/4)
// and k-step s covers 8 of them, so a lane's codes of one key row are contiguous.
template <int D>
__device__ __forceinline__ int draft_chan(int kg, int s) {
  return kg * (D / 4) + 8 * s;
}

// extract 8 consecutive codes u0..u0+7 of a word stream (pair-interleaved packing)
template <int BITS>
__device__ __forceinline__ void unpack8(const uint32_t* words, int u0, float* out) {
  constexpr int PER = 32 / BITS;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int u = u0 + j;
    const uint32_t wv = words[u / PER];
    const int uu = u % PER;
    out[j] = (float)((wv >> ((uu & 1) * 16 + BITS * (uu >> 1))) & MASK);
  }
}

// One page pair (32 keys) of a draft item from global memory, dequantising KIVI codes (or
// converting drafted-block bf16 rows) to fp16 in registers: the path for pairs the LDS ring
// does not cover (an odd last context page, drafted-block pages).  Updates the running softmax
// state (m_run, l_run, acc_o) of lane (row n, group kg).
template <int D, int BITS>
__device__ __forceinline__ void draft_pair_generic(const AttnArgs& a, const ItemCtx& it, int pp,
                                                   const u32x4* qreg, int qpos, float sc,
                                                   f32x4* acc_o, float& m_run, float& l_run) {
  constexpr bool KIVI = BITS != 16;
  constexpr int NS = D / 32;
  constexpr int ND = D / 16;
  const int lane = threadIdx.x & 63, n = lane & 15, kg = lane >> 4;
  PageRef pr[2];
  pr[0] = page_ref<D>(a, it, 2 * pp, KIVI);
  pr[1] = page_ref<D>(a, it, 2 * pp + 1, KIVI);

  // ---- scores S^T (16 keys x 16 rows) for the two 16-key blocks of the pair
  f32x4 s_acc[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    s_acc[b] = f32x4{};
    const int m = n;  // A-operand row = key slot m: page m/8, token 8*((m>>2)&1) + 4b + (m&3)
    const PageRef p = (m >> 3) ? pr[1] : pr[0];
    const int ktok = 8 * ((m >> 2) & 1) + 4 * b + (m & 3);
    u32x4 av[NS];
    if (p.kind == 2 || ktok >= p.valid) {
#pragma unroll
      for (int s = 0; s < NS; ++s) av[s] = u32x4{0, 0, 0, 0};
    } else if (!KIVI || p.kind == 1) {
      const uint8_t* krow = p.k + ktok * (D * 2);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        av[s] = ld16(krow + 2 * (KIVI ? draft_chan<D>(kg, s) : 32 * s + 8 * kg));
        if constexpr (KIVI) av[s] = bf16x8_to_f16x8(av[s]);
      }
    } else {
      // KIVI key row: codes of channels [kg*D/4, (kg+1)*D/4), dequantised with the
      // per-channel (scale, zero) of this 32-token group
      constexpr int WPG = D / 4 * BITS / 32;  // words per lane group
      uint32_t words[WPG];
      const uint32_t* wrow = reinterpret_cast<const uint32_t*>(p.k + ktok * (D * BITS / 8)) + kg * WPG;
#pragma unroll
      for (int i = 0; i < WPG; ++i) words[i] = wrow[i];
      // planar (scale, zero) of the group: scales of channels 0..d-1, then zeros
      const uint16_t* ksc = reinterpret_cast<const uint16_t*>(p.ksz) + kg * (D / 4);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        float code[8];
        unpack8<BITS>(words, 8 * s, code);
        uint32_t pk[4];
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const int c = 8 * s + j;
          const float k0 = fmaf(code[j], fp16_bits_to_f32(ksc[c]), fp16_bits_to_f32(ksc[D + c]));
          const float k1 = fmaf(code[j + 1], fp16_bits_to_f32(ksc[c + 1]), fp16_bits_to_f32(ksc[D + c + 1]));
          pk[j >> 1] = pack_f16(k0, k1);
        }
        av[s] = u32x4{pk[0], pk[1], pk[2], pk[3]};
      }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) s_acc[b] = mfma16<KIVI>(av[s], qreg[s], s_acc[b]);
  }

  // ---- softmax over this lane's 8 keys: page kg/2, tokens 8*(kg&1) + 4b + r
  const PageRef mp = (kg >> 1) ? pr[1] : pr[0];
  float sv[8];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tt = 8 * (kg & 1) + 4 * b + r;
      sv[4 * b + r] = key_visible(mp, tt, qpos) ? s_acc[b][r] : -INFINITY;
    }
  float mloc = -INFINITY;
#pragma unroll
  for (int j = 0; j < 8; ++j) mloc = fmaxf(mloc, sv[j]);
  mloc = wave_xor_max(mloc, 16);
  mloc = wave_xor_max(mloc, 32);
  const float m_new = fmaxf(m_run, mloc * sc);
  if (__any(m_new > m_run + (KIVI ? kRescaleF16 : kRescaleBf16))) {
    const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc_o[i][r] *= alpha;
    m_run = m_new;
  }
  const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
  uint32_t pb[4];
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[j], sc, -m_use));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[j + 1], sc, -m_use));
    l_run += p0 + p1;
    pb[j >> 1] = KIVI ? pack_f16(p0, p1) : pack_bf16(p0, p1);
  }
  const u32x4 bv = {pb[0], pb[1], pb[2], pb[3]};

  // ---- O^T += V^T P^T: lane (d = 16*db + n, kg) feeds tokens 8*(kg&1)..+8 of page kg/2
  const PageRef& vp = mp;
  const int t0 = 8 * (kg & 1);
#pragma unroll
  for (int db = 0; db < ND; ++db) {
    const int dd = 16 * db + n;
    u32x4 av = {0, 0, 0, 0};
    if (vp.kind != 2) {
      if (!KIVI || vp.kind == 1) {
        av = ld16(vp.v + dd * 32 + t0 * 2);
        if (vp.valid < kBlock) av = mask_tokens(av, t0, vp.valid);
        if constexpr (KIVI) av = bf16x8_to_f16x8(av);
      } else {
        constexpr int WPC = 16 * BITS / 32;  // words per channel (16 tokens)
        uint32_t words[WPC];
        const uint32_t* wrow = reinterpret_cast<const uint32_t*>(vp.v) + dd * WPC;
#pragma unroll
        for (int i = 0; i < WPC; ++i) words[i] = wrow[i];
        float code[8];
        unpack8<BITS>(words, t0, code);
        // this channel group's token scales, then token zeros
        const uint16_t* vsc = reinterpret_cast<const uint16_t*>(vp.vsz) + (dd >> 5) * 2 * kBlock + t0;
        uint32_t pk[4];
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          float v0 = fmaf(code[j], fp16_bits_to_f32(vsc[j]), fp16_bits_to_f32(vsc[kBlock + j]));
          float v1 = fmaf(code[j + 1], fp16_bits_to_f32(vsc[j + 1]), fp16_bits_to_f32(vsc[kBlock + j + 1]));
          if (t0 + j >= vp.valid) v0 = 0.f;
          if (t0 + j + 1 >= vp.valid) v1 = 0.f;
          pk[j >> 1] = pack_f16(v0, v1);
        }
        av = u32x4{pk[0], pk[1], pk[2], pk[3]};
      }
    }
    acc_o[db] = mfma16<KIVI>(av, bv, acc_o[db]);
  }
}


// ------------------------------------------------------------------ draft path, KIVI caches (ring)
// Whole context page pairs (one 32-token key-quantisation group each) stream through a private
// per-wave LDS ring, as in the bf16 draft path.  The scales are folded out of the inner loops:
//   scores   q.k^ = sum_c code_c (s_c q_c) + sum_c z_c q_c       (key scale/zero per channel)
//   outputs  sum_t p_t v^_t,c = sum_t code_t,c (s_t,g p_t) + sum_t z_t,g p_t   (value per token)
// so the per-element work is only expanding 2- or 4-bit codes to exact fp16 (one and-or per
// pair, see Expand).  Every product runs on 16x16x32 fp16 MFMA, the bias terms included: with
// an A operand that is the same for every row (the zeros of the lane's channels or tokens, or the
// negated expansion offsets), one MFMA sums over all 32 keys of the k-step, so the bias of row n
// lands in every output row of column n without cross-lane sums.  Key biases initialise the score
// accumulators; value biases accumulate per 32-channel group and join the outputs once the ring
// pairs are done.  Pairs the ring does not cover (an odd last context page, drafted-block pages)
// go through draft_pair_generic.
template <int D, int BITS, int NW>
struct KRing {
  static constexpr int kCodes = kBlock * D * BITS / 8;    // one page's key (or value) codes
  static constexpr int kKsz = 2 * D * 2;                  // key scale and zero planes of a group
  static constexpr int kVsz = (D / 32) * 2 * kBlock * 2;  // value scales and zeros of a page
  static constexpr int kOffV = 2 * kCodes;
  static constexpr int kOffKsz = 4 * kCodes;
  static constexpr int kOffVsz = kOffKsz + kKsz;
  static constexpr int kParams = kKsz + 2 * kVsz;          // key and value parameters of a pair
  static constexpr int kSlot = (kOffVsz + 2 * kVsz + 1023) / 1024 * 1024;
  static constexpr int kCodeLoads = 2 * kCodes <= 1024 ? 1 : 2;  // loads of both pages' codes
  static constexpr int kLoads = 2 * kCodeLoads + 1;              // ring loads per slot
  static constexpr int kIds = 144 * 1024 * D / 128;         // LDS offset of the page ids
  static constexpr int kStg0 = kIds / (NW * kSlot);
  static constexpr int kStg = kStg0 > 8 ? 8 : kStg0;        // slots per wave
  static constexpr int kBytes = kIds + kMaxChunkPages * 4 + 16;  // ids, then the first missing page
  static_assert(kParams % 16 == 0 && kParams <= 1024, "the parameters of a pair are one load");
  // LDS layout of a slot's codes (64 banks of 4 bytes).  The ring is written lane-linearly, 16
  // bytes per lane, so a layout is a permutation of 16-byte chunks chosen by which global chunk a
  // lane fetches.  One read takes rows of both pages at once (key rows 4 b + i and 8 + 4 b + i,
  // value channels 16 db + n), and the two pages of a pair would sit a multiple of the bank span
  // apart.  So the pages' codes are interleaved in 128-byte blocks (block q of the even page, then
  // block q of the odd page): a row of the odd page is always 128 bytes after the same row of the
  // even page, on the other half of the banks, and every read is a per-lane base plus a constant.
  // Key rows t and t + 8, which land on the same banks, also have their chunks permuted
  // (krow_xor).  The scale and zero planes are read one address per 16 lanes (broadcast).
  static constexpr int kCPR = D * BITS / 8 / 16;  // 16-byte chunks of a key row
  static constexpr int kRowB = 16 * kCPR;         // bytes of a key row
  static constexpr int kRPB = kRowB >= 128 ? 1 : 128 / kRowB;  // key rows per 128-byte block
  static_assert(kRowB <= 128 && kCodes % 128 == 0, "pages interleave in 128-byte blocks");
  static __device__ __forceinline__ int krow_xor(int t) {
    if constexpr (kCPR >= 4) return ((t >> 1) & 1) | (((t >> 3) & 1) << 1);
    else if constexpr (kCPR == 2) return (t >> 3) & 1;
    else return 0;
  }
  // LDS byte offset (inside the slot's key codes) of chunk j of token row t of page `page`
  static __device__ __forceinline__ int kcode_pos(int page, int t, int j) {
    return 256 * (t / kRPB) + 128 * page + kRowB * (t % kRPB) + 16 * (j ^ krow_xor(t));
  }
  // key rows 4 b on: kcode_pos(p, t + 4 b, j) = kcode_pos(p, t, j) + b * kKeyStepB when bit 2 of t is clear
  static constexpr int kKeyStepB = kRPB >= 8 ? 4 * kRowB : 256 * (4 / kRPB);
  // the global byte offset (page, offset inside the page) of the chunk at LDS byte B of the key codes
  static __device__ __forceinline__ int kcode_src(int B, int* page) {
    const int q = B >> 8, r = B & 255;
    *page = r >> 7;
    const int tt = q * kRPB + (r & 127) / kRowB;
    const int jj = ((r & 127) % kRowB) >> 4;
    return tt * kRowB + 16 * (jj ^ krow_xor(tt));
  }
  // value codes: byte o of page `page` sits at LDS byte vcode_pos(page, o)
  static constexpr int kVRow = kBlock * BITS / 8;  // bytes of a value channel row
  static __device__ __forceinline__ int vcode_pos(int page, int o) { return 256 * (o >> 7) + 128 * page + (o & 127); }
  static __device__ __forceinline__ int vcode_src(int B, int* page) {
    *page = (B >> 7) & 1;
    return 128 * (B >> 8) + (B & 127);
  }
};

// wait until at most `ahead` slots (PER loads each) of this wave are still in flight
template <int PER, int A>
__device__ __forceinline__ void wait_ahead(int ahead) {
  if constexpr (A == 0) {
    wait_vmem<0>();
  } else {
    if (ahead >= A) wait_vmem<A * PER>();
    else wait_ahead<PER, A - 1>(ahead);
  }
}

// ring load of one contiguous piece of `bytes` (a multiple of 16, at most 1024) into LDS `dst`
template <int BYTES>
__device__ __forceinline__ void ring_piece(const uint8_t* src, uint8_t* dst, int lane) {
  static_assert(BYTES % 16 == 0 && BYTES <= 1024, "ring piece");
  if (BYTES == 1024 || lane < BYTES / 16) ring_load(src, 16 * lane, dst);
}

// ring loads of two pages' pieces of BYTES each, contiguous in LDS at dst: one load when both fit
// in 1 KB (lanes split between the pages), else one per page
template <int BYTES>
__device__ __forceinline__ void ring_pair(const uint8_t* src0, const uint8_t* src1, uint8_t* dst, int lane) {
  if constexpr (2 * BYTES <= 1024) {
    const int o = 16 * lane;
    const uint8_t* src = o < BYTES ? src0 + o : src1 + (o - BYTES);
    if (2 * BYTES == 1024 || o < 2 * BYTES)
      __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)dst, 16, 0, kNontemporal);
  } else {
    ring_piece<BYTES>(src0, dst, lane);
    ring_piece<BYTES>(src1, dst + BYTES, lane);
  }
}

// Code expansion.  A pair of codes sitting at mantissa bits [p, p + BITS) of both 16-bit
// halves of a word becomes two exact fp16 values with one and-or: the or-ed exponent makes
// mantissa bit p worth 1, so each half reads 2^(10 - p) + code.  The constant 2^(10 - p) is the
// pair's offset; the MFMAs that consume the expanded codes cancel it with one more product of
// the negated offsets (row-independent A operand) against the same B operand.
//   2-bit: a word holds 8 pairs (pair i at bits 2i of each half).  Pairs 0-3 are rotated left
//          by 2 and pairs 4-7 right by 6, which puts them at bits 2, 4, 6, 8: offsets 256, 64,
//          16, 4.
//   4-bit: a word holds 4 pairs (pair i at bits 4i).  A left rotation by 2 puts pairs 0 and 1
//          at bits 2 and 6, a right rotation by 6 does the same for pairs 2 and 3: offsets 256,
//          16, 256, 16.
// Bits rotated across a half boundary land outside every mask.
// Masks and exponents of the expansion, per pair position, held in registers: as literals the
// compiler would split each and-or into an and and an or (a VOP3 instruction of this
// architecture takes no literal operand).  The empty asm statements only make the values opaque
// so that they stay in an SGPR (mask) and a VGPR (exponent); they emit no instruction.
template <int BITS>
struct Expand {
  uint32_t mask[4], magic[4];
  __device__ __forceinline__ Expand() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // 2-bit: positions 2, 4, 6, 8; 4-bit: positions 2, 6, 2, 6
      const int p = BITS == 2 ? 2 + 2 * i : 2 + 4 * (i & 1);
      mask[i] = (((1u << BITS) - 1u) << p) * 0x00010001u;
      magic[i] = ((uint32_t)(25 - p) << 10) * 0x00010001u;
      asm volatile("" : "+s"(mask[i]));
      asm volatile("" : "+v"(magic[i]));
    }
  }
  __device__ __forceinline__ uint32_t pair(uint32_t x, int i) const { return (x & mask[i]) | magic[i]; }
  // 2-bit: the 4 pairs (8 codes) of word `w` selected by `hi` (0: pairs 0-3, 1: pairs 4-7)
  __device__ __forceinline__ u32x4 bits2(uint32_t w, int hi) const {
    const uint32_t x = __builtin_rotateright32(w, hi ? 6 : 30);
    return u32x4{pair(x, 0), pair(x, 1), pair(x, 2), pair(x, 3)};
  }
  // 4-bit: the 4 pairs (8 codes) of word `w`
  __device__ __forceinline__ u32x4 bits4(uint32_t w) const {
    const uint32_t x0 = __builtin_rotateright32(w, 30), x1 = __builtin_rotateright32(w, 6);
    return u32x4{pair(x0, 0), pair(x0, 1), pair(x1, 2), pair(x1, 3)};
  }
};

// negated offsets of the expanded pairs, as an fp16 A operand (the same for every row)
template <int BITS>
__device__ __forceinline__ u32x4 neg_offsets() {
  if constexpr (BITS == 2) return u32x4{0xDC00DC00u, 0xD400D400u, 0xCC00CC00u, 0xC400C400u};  // -256 -64 -16 -4
  else return u32x4{0xDC00DC00u, 0xCC00CC00u, 0xDC00DC00u, 0xCC00CC00u};                   // -256 -16 -256 -16
}

// Vector elements are copied to scalars before __builtin_bit_cast: a cast applied to a
// subscripted ext_vector lvalue reads the vector's first element whatever the index.
__device__ __forceinline__ u32x4 mul_f16x8(u32x4 a, u32x4 b) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t ai = a[i], bi = b[i];
    r[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, ai) * __builtin_bit_cast(f16x2, bi));
  }
  return r;
}

// maximum over the 4 lanes of a row (lanes n, n + 16, n + 32, n + 48)
__device__ __forceinline__ float row_max4(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return half_swap_max(fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1])));
}

// f(integral_constant<int, 0>) .. f(integral_constant<int, N - 1>), in order
template <int N, int J = 0, class F>
__device__ __forceinline__ void unroll(F&& f) {
  if constexpr (J < N) {
    f(std::integral_constant<int, J>{});
    unroll<N, J + 1>(f);
  }
}

// a0 .. a3 by a lane's slot j (0 .. 3)
__device__ __forceinline__ float sel_slot(float a0, float a1, float a2, float a3, int j) {
  const float t0 = (j & 1) ? a1 : a0, t1 = (j & 1) ? a3 : a2;
  return (j & 2) ? t1 : t0;
}
// Four slots of 4 columns in each 16-lane row (lane bits 2-3 the slot, 0-1 the row): every lane
// takes slot J's value of its row.  ds_swizzle in bit-mask mode (within 32 lanes): keep lane bits
// 0, 1 and 4, set bits 2-3 to J.
template <int J>
__device__ __forceinline__ uint32_t slot_bcast(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x13 | (J << 7));
}
// sum over the four slots of a lane's row (lanes 4 and 8 apart)
__device__ __forceinline__ float slot_sum4(float x) {
  x += __shfl_xor(x, 4, 64);
  return x + __shfl_xor(x, 8, 64);
}

// RP: query rows padded to 4, 8 or 16 (rows_total <= RP).  The 16 columns of the MFMAs are
// 16 / RP slots of RP columns, and every slot holds the same query rows: the scores and softmax
// weights of a column depend only on its row.  The value product then takes, in slot j of its
// B operand, the weights scaled for channel group j (of the set), so one operand serves 16 / RP
// groups; for a 16-channel output block only the slot of its group is kept, and the join moves
// that slot to columns 0 .. RP - 1.
template <int D, int BITS, int NW, int RP>
__device__ void draft_kivi_item(const AttnArgs& a, const ItemCtx& it, uint8_t* smem) {
  using R = KRing<D, BITS, NW>;
  constexpr int STG = R::kStg;
  static_assert(STG >= 2, "KIVI draft ring needs two slots per wave");
  static_assert(RP == 4 || RP == 8 || RP == 16, "rows padded to 4, 8 or 16");
  constexpr int NS = D / 32;              // k-steps of the score product
  constexpr int ND = D / 16;              // 16-wide channel blocks of the output
  constexpr int NGQ = D / 32;             // value channel groups
  constexpr int SL = 16 / RP;             // column slots
  constexpr int NB = (NGQ + SL - 1) / SL; // value operands (sets of SL groups)
  constexpr int KW = (D / 4) * BITS / 32; // words of a key row held by one lane (its D/4 channels)
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, kg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar loop control
  const ReqDev& rq = it.rq;
  const int G = a.G;
  const int row = n % RP, slot_n = n / RP;  // this column's query row and slot
  const bool row_ok = row < it.rows_total;
  const int tok = row_ok ? row / G : 0;
  const int qpos = rq.q0 + tok;

  // query of this column's row, channels kg * D/4 .. + D/4 (8 per k-step), in fp16
  u32x4 qh[NS];
  {
    const uint16_t* qp = a.q + ((((int64_t)rq.slot * a.L + it.l) * a.xmax + rq.q0 + tok) * a.Hq +
                                it.g * G + (row_ok ? row % G : 0)) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      qh[s] = bf16x8_to_f16x8(row_ok ? ld16(qp + draft_chan<D>(kg, s)) : u32x4{0, 0, 0, 0});
  }
  int32_t* ids = reinterpret_cast<int32_t*>(smem + R::kIds);
  int* first_bad = ids + kMaxChunkPages;
  {
    const PoolDev& pl = it.pool;
    if (tid == 0) *first_bad = it.nctx;
    __syncthreads();
    const int32_t* pt = pl.page_table + (int64_t)rq.page_row * pl.max_pages + it.p_lo;
    for (int i = tid; i < it.nctx; i += 64 * NW) {
      const int phys = pt[i];
      const bool ok = phys >= 0 && phys < pl.nblk;
      ids[i] = ok ? phys : -1;
      if (!ok) {
        atomicMin(first_bad, i);
        if (phys != -1) report_bad_page(a.err, rq.page_row, it.p_lo + i, phys);
      }
    }
  }
  wait_vmem<0>();
  __syncthreads();

  const PoolDev& pl = it.pool;
  const int64_t unit0 = (int64_t)it.l * pl.nblk * a.Hkv + it.g;  // block 0 of (layer, kv head)
  uint8_t* ring = smem + w * (STG * R::kSlot);
  const int ring_pairs = it.nctx >> 1;  // pairs of two context pages
  const int mine = ring_pairs > w ? (ring_pairs - w + NW - 1) / NW : 0;
  // Lane-only parts of the ring loads, the same for every slot: the byte offset of this lane's 16
  // bytes inside its source page or plane, and which page or plane that is (KRing layouts).
  const int o16 = 16 * lane;
  // (codes: load i covers LDS bytes 1024 i .. 1024 i + 1023 of the interleaved pages)
  // (the page is bit 7 of the LDS byte in both layouts, so one flag serves every code load)
  int lpg;
  const uint32_t kc_off = R::kcode_src(o16, &lpg), vc_off = R::vcode_src(o16, &lpg);
  uint32_t kc_off1 = 0, vc_off1 = 0;
  if constexpr (2 * R::kCodes > 1024) {
    static_assert(R::kCodes == 1024, "one load per page's worth of codes");
    kc_off1 = R::kcode_src(1024 + o16, &lpg);
    vc_off1 = R::vcode_src(1024 + o16, &lpg);
  }
  const int pr_src = o16 < R::kKsz ? 0 : o16 < R::kKsz + R::kVsz ? 1 : 2;  // key planes, even, odd page
  const uint32_t pr_off = pr_src == 0 ? o16 : pr_src == 1 ? o16 - R::kKsz : o16 - R::kKsz - R::kVsz;
  // Each load has a scalar base (the pool at this layer and kv head) and a 32-bit per-lane offset
  // (block id x kv heads x page bytes, plus the lane's offset in the page; the host keeps a KIVI
  // pool's blocks x kv heads x page bytes below 2^32).  A lane's choice between the pair's two
  // pages is a mask fixed for the item, so a pair's addresses cost a few integer instructions.
  const uint8_t* kbase = pl.k + unit0 * R::kCodes;
  const uint8_t* vbase = pl.v + unit0 * R::kCodes;
  // (the parameter planes come from two pools: a per-lane base, fixed for the item)
  const uint8_t* pbase = (pr_src == 0 ? pl.ksz + unit0 * R::kKsz : pl.vsz + unit0 * R::kVsz) + pr_off;
  // lane masks, kept in vector registers (the empty asm statements emit nothing) so that each
  // selection is one and / and-or with the scalar operand
  uint32_t csel = lpg ? ~0u : 0u;  // lanes fetching the odd page's codes
  uint32_t pselk = pr_src == 0 ? ~0u : 0u, psel0 = pr_src == 1 ? ~0u : 0u, psel1 = pr_src == 2 ? ~0u : 0u;
  asm volatile("" : "+v"(csel), "+v"(pselk), "+v"(psel0), "+v"(psel1));
  const uint32_t cstride = (uint32_t)a.Hkv * R::kCodes;
  const uint32_t kpstride = (uint32_t)a.Hkv * R::kKsz, vpstride = (uint32_t)a.Hkv * R::kVsz;
  auto issue = [&](uint8_t* slot, int id0, int id1) {
    const uint32_t i0 = id0 < 0 ? 0u : (uint32_t)id0, i1 = id1 < 0 ? 0u : (uint32_t)id1;
    // (the differences wrap in 32 bits; every sum stays below 2^32)
    const uint32_t co = i0 * cstride + (csel & ((i1 - i0) * cstride));
    if constexpr (2 * R::kCodes <= 1024) {
      if (2 * R::kCodes == 1024 || o16 < 2 * R::kCodes) {
        __builtin_amdgcn_global_load_lds(kbase + (co + kc_off), (lds_ptr_t)slot, 16, 0, kNontemporal);
        __builtin_amdgcn_global_load_lds(vbase + (co + vc_off), (lds_ptr_t)(slot + R::kOffV), 16, 0, kNontemporal);
      }
    } else {
      __builtin_amdgcn_global_load_lds(kbase + (co + kc_off), (lds_ptr_t)slot, 16, 0, kNontemporal);
      __builtin_amdgcn_global_load_lds(kbase + (co + kc_off1), (lds_ptr_t)(slot + 1024), 16, 0, kNontemporal);
      __builtin_amdgcn_global_load_lds(vbase + (co + vc_off), (lds_ptr_t)(slot + R::kOffV), 16, 0, kNontemporal);
      __builtin_amdgcn_global_load_lds(vbase + (co + vc_off1), (lds_ptr_t)(slot + R::kOffV + 1024), 16, 0, kNontemporal);
    }
    // the group's key parameters and both pages' value parameters are contiguous in the slot:
    // one load, each lane fetching its 16 bytes from the plane they come from
    const uint32_t po = (pselk & (i0 * kpstride)) | (psel0 & (i0 * vpstride)) | (psel1 & (i1 * vpstride));
    if (R::kParams == 1024 || o16 < R::kParams)
      __builtin_amdgcn_global_load_lds(pbase + po, (lds_ptr_t)(slot + R::kOffKsz), 16, 0, kNontemporal);
  };
  // page ids of this wave's pair k, straight from the page table: the table is not written while
  // the kernel runs, so it is read through the constant address space and the uniform index gives
  // scalar loads into SGPRs; an entry outside the pool loads block 0 (such pages are masked, or
  // never full, by the validity taken from the table in LDS)
  using const_i32 = const __attribute__((address_space(4))) int32_t*;
  const const_i32 pt_k = (const_i32)(pl.page_table + (int64_t)rq.page_row * pl.max_pages + it.p_lo);
  const uint32_t nblk_u = (uint32_t)pl.nblk;
  auto pair_ids = [&](int k, int& id0, int& id1) {
    id0 = id1 = 0;
    if (k < mine) {
      const int pp = w + NW * k;
      const int a0 = pt_k[2 * pp], a1 = pt_k[2 * pp + 1];
      id0 = (uint32_t)a0 < nblk_u ? a0 : 0;
      id1 = (uint32_t)a1 < nblk_u ? a1 : 0;
    }
  };
#pragma unroll
  for (int k = 0; k < STG - 1; ++k)
    if (k < mine) {
      int i0, i1;
      pair_ids(k, i0, i1);
      issue(ring + k * R::kSlot, __builtin_amdgcn_readfirstlane(i0), __builtin_amdgcn_readfirstlane(i1));
    }
  int pf0, pf1;  // page ids of the next slot to load, read one pair early
  pair_ids(STG - 1, pf0, pf1);

  f32x4 acc_o[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc_o[i] = f32x4{};
  // offset part of the value biases, -sum_t off_t s_t,g p_t, per column: operand set b, slot j
  // holds group b SL + j
  f32x4 vb[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) vb[i] = f32x4{};
  // value scale plane of this lane's group in set 0; set b adds b SL groups (with more than one
  // set, SL divides NGQ; slots past the last group, with one set, read group slot % NGQ's)
  const int vs_lane = SL == 1 ? 0 : 2 * (slot_n % NGQ) * kBlock;
  // zero part of the value biases, sum_t z_t,g p_t, of every group in one product: A-operand row m
  // (this lane's n) holds the zeros of group m % NGQ, so output row g of column n is group g's
  f32x4 vzs = f32x4{};
  const int zrow = n % NGQ;
  const u32x4 noff = neg_offsets<BITS>();
  const Expand<BITS> ex;
  float m_run = -INFINITY, l_run = 0.f;
  float lim = -1.f;    // 2^kRescaleF16 once the running maximum is set
  float m_use = 0.f;   // the running maximum, 0 while unset
  // The key rows 4..7 of a 16-key half are kKeyStepB bytes further.  The offset is opaque to the
  // optimiser (set once per item), so the two 8-byte reads of 2-bit codes stay separate
  // instructions: fused into one paired read, its two halves, 256 bytes apart, would share banks.
  uint32_t kstep1 = R::kKeyStepB;
  asm volatile("" : "+v"(kstep1));
  const float sc = a.scale_log2;
  const int vtok0 = 8 * (kg & 1), vpage = kg >> 1;  // this lane's 8 tokens of a pair

  // Scores of the pair in `slot` (biases included), and the softmax and value products of pair k
  // given its scores.
  auto scores = [&](const uint8_t* slot, f32x4 (&s_acc)[2]) {
    // ---- key side: q' = q * scale (per channel); bias of column n = sum_c (z_c q_c - off_c q'_c)
    u32x4 qs[NS];
    f32x4 kb = f32x4{};
    {
      const uint16_t* ksc = reinterpret_cast<const uint16_t*>(slot + R::kOffKsz) + kg * (D / 4);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        qs[s] = mul_f16x8(qh[s], ld16(ksc + 8 * s));
        kb = mfma16<true>(ld16(ksc + D + 8 * s), qh[s], kb);
        kb = mfma16<true>(noff, qs[s], kb);
      }
    }
    // ---- scores S^T for the pair's two 16-key halves: A-operand row m is key (page m / 8,
    // token 8 ((m >> 2) & 1) + 4 b + (m & 3)), so lane (n, kg) ends with tokens 8 (kg & 1) + 4 b + i
    // of page kg / 2 -- exactly the B operand of the value product
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int tk = 8 * ((n >> 2) & 1) + 4 * b + (n & 3);
      constexpr int LB = 4 * KW;  // bytes of a row this lane reads: one LDS read of that width
      const int ob = kg * LB;
      // rows 4 b on are kKeyStepB further (kstep1, opaque: see its definition)
      const uint32_t kstep = b ? kstep1 : 0u;
      const uint8_t* kp = slot + R::kcode_pos(n >> 3, tk - 4 * b, ob >> 4) + kstep + (ob & 15);
      uint32_t words[KW];
      if constexpr (KW == 4) {
        const u32x4 v = ld16(kp);
#pragma unroll
        for (int i = 0; i < 4; ++i) words[i] = v[i];
      } else if constexpr (KW == 2) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(kp);
        words[0] = v[0];
        words[1] = v[1];
      } else {
        words[0] = *reinterpret_cast<const uint32_t*>(kp);
      }
      s_acc[b] = kb;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        // the lane's channels 8s .. 8s + 7
        const u32x4 av = BITS == 2 ? ex.bits2(words[s >> 1], s & 1) : ex.bits4(words[s]);
        s_acc[b] = mfma16<true>(av, qs[s], s_acc[b]);
      }
    }
  };
  // FULL: the pair is known to be two full, present pages (no validity reads or masking)
  auto consume = [&](int k, const uint8_t* slot, const f32x4 (&s_acc)[2], auto full_pair) {
    constexpr bool FULL = decltype(full_pair)::value;
    const int pp = w + NW * k;
    // ---- page validity (full pairs need no masking)
    int v0 = kBlock, v1 = kBlock;
    bool full = true;
    if constexpr (!FULL) {
      const int ip0 = 2 * pp;
      v0 = ids[ip0] < 0 ? 0 : min(kBlock, rq.ctx_len - kBlock * (it.p_lo + ip0));
      // the odd page's keys use the group parameters stored with the even page
      v1 = (ids[ip0] < 0 || ids[ip0 + 1] < 0) ? 0 : min(kBlock, rq.ctx_len - kBlock * (it.p_lo + ip0 + 1));
      full = v0 == kBlock && v1 == kBlock;
    }
    // ---- online softmax over this lane's 8 keys
    float sv[8];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[4 * b + i] = s_acc[b][i];
    if (!full) {
      const int valid = vpage ? v1 : v0;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (vtok0 + j >= valid) sv[j] = -INFINITY;
    }
    // weights against the running maximum; while every lane's weights sum below 2^headroom none
    // can exceed it, so the row maxima and the move test run only when some sum reaches it (or a
    // maximum is unset), and the weights are taken again after a move.  With four slots, a lane
    // takes only tokens 2 j, 2 j + 1 of its 8 (j its slot: the other slots hold the same row) and
    // gathers the rest from the slots that took them.
    constexpr int NE = SL == 4 ? 2 : 8;
    float x[NE], e[NE];
    if constexpr (SL == 4) {
      x[0] = sel_slot(sv[0], sv[2], sv[4], sv[6], slot_n);
      x[1] = sel_slot(sv[1], sv[3], sv[5], sv[7], slot_n);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = sv[j];
    }
    auto weights = [&]() {
#pragma unroll
      for (int j = 0; j < NE; ++j) e[j] = __builtin_amdgcn_exp2f(fmaf(x[j], sc, -m_use));
    };
    weights();
    float esum;
    if constexpr (SL == 4) esum = e[0] + e[1];
    else esum = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
    if (__any(!(esum < lim))) {
      float mloc = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
      mloc = row_max4(mloc);
      const float m_new = fmaxf(m_run, mloc * sc);
      if (__any(m_new > m_run + kRescaleF16)) {
        const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < ND; ++i) acc_o[i] *= alpha;
#pragma unroll
        for (int i = 0; i < NB; ++i) vb[i] *= alpha;
        vzs *= alpha;
        m_run = m_new;
        lim = m_new == -INFINITY ? -1.f : kLimF16;
        m_use = m_new == -INFINITY ? 0.f : m_new;
        weights();
      }
    }
    u32x4 p16;
    if constexpr (SL == 4) {
      l_run += e[0] + e[1];  // this lane's share; the slots' shares are summed after the loop
      const uint32_t ph = pack_f16(e[0], e[1]);
      p16 = u32x4{slot_bcast<0>(ph), slot_bcast<1>(ph), slot_bcast<2>(ph), slot_bcast<3>(ph)};
    } else {
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        l_run += e[j] + e[j + 1];
        p16[j >> 1] = pack_f16(e[j], e[j + 1]);
      }
    }
    // ---- value side: P'_g = p * scale_t,g; bias_g += sum_t (z_t,g p_t - off_t P'_t,g)
    const uint16_t* vsz = reinterpret_cast<const uint16_t*>(slot + R::kOffVsz + vpage * R::kVsz) + vtok0;
    const uint8_t* vcodes = slot + R::kOffV;
    {
      u32x4 vz = ld16(vsz + (2 * zrow + 1) * kBlock);
      if (!full) vz = mask_tokens(vz, vtok0, vpage ? v1 : v0);  // tokens past the valid ones: no zero
      vzs = mfma16<true>(vz, p16, vzs);
    }
    u32x4 pv;
#pragma unroll
    for (int gq = 0; gq < NGQ; ++gq) {
      if (gq % SL == 0) {  // the weights scaled for the next set of groups (slot j: group gq + j)
        const int b = gq / SL;
        u32x4 vs = ld16(vsz + vs_lane + 2 * b * SL * kBlock);
        if (!full) vs = mask_tokens(vs, vtok0, vpage ? v1 : v0);  // tokens past the valid ones: no scale
        pv = mul_f16x8(p16, vs);
        vb[b] = mfma16<true>(noff, pv, vb[b]);
      }
      // O^T += V^T P'^T for the two 16-channel blocks of this group (its slot of the set)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int db = 2 * gq + h2;
        const int dd = 16 * db + n;
        const uint32_t* vw = reinterpret_cast<const uint32_t*>(vcodes + R::vcode_pos(vpage, dd * R::kVRow));
        // the lane's tokens vtok0 .. vtok0 + 7 of channel dd
        const u32x4 av = BITS == 2 ? ex.bits2(vw[0], kg & 1) : ex.bits4(vw[kg & 1]);
        acc_o[db] = mfma16<true>(av, pv, acc_o[db]);
      }
    }
  };
  // pair k sits in slot `j` (k % STG), and the slot it refills is the one before it
  auto step = [&](int k, int j, auto full_pair) {
    wait_ahead<R::kLoads, STG - 2>(min(STG - 2, mine - 1 - k));
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    if (k + STG - 1 < mine)
      issue(ring + ((j + STG - 1) % STG) * R::kSlot, __builtin_amdgcn_readfirstlane(pf0),
            __builtin_amdgcn_readfirstlane(pf1));
    pair_ids(k + STG, pf0, pf1);
    const uint8_t* slot = ring + j * R::kSlot;
    f32x4 s_acc[2];
    scores(slot, s_acc);
    consume(k, slot, s_acc, full_pair);
  };
  // pairs before the first missing or partial page are full; this wave's k-th pair is w + NW k
  const int nfull = min(it.nctx, max(0, (rq.ctx_len - kBlock * it.p_lo) / kBlock));
  const int pairs_full = min(nfull, *first_bad) >> 1;
  const int k_full = min(mine, pairs_full > w ? (pairs_full - w + NW - 1) / NW : 0);
  int k = 0;
  // full pairs a ring's turn at a time: every slot offset is a constant
  for (; k + STG <= k_full; k += STG)
    unroll<STG>([&](auto j) { step(k + decltype(j)::value, decltype(j)::value, std::true_type{}); });
  for (; k < k_full; ++k) step(k, k % STG, std::true_type{});
  for (; k < mine; ++k) step(k, k % STG, std::false_type{});

  // the value bias joins the outputs before any pair that rescales without it; the zero part of
  // group g for column n is element g of lane n's accumulator (output row g).  Then each block's
  // slot moves to columns 0 .. RP - 1 (the rows past RP take other columns' values; no one reads
  // them).
#pragma unroll
  for (int gq = 0; gq < NGQ; ++gq) {
    const float z = __shfl(vzs[gq], n, 64);
    const f32x4 bias = vb[gq / SL] + f32x4{z, z, z, z};
    acc_o[2 * gq] += bias;
    acc_o[2 * gq + 1] += bias;
    if constexpr (SL > 1) {
      const int src = lane + (gq % SL) * RP;
      if (gq % SL != 0) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc_o[2 * gq + h2][i] = __shfl(acc_o[2 * gq + h2][i], src, 64);
      }
    }
  }
  // with four slots each lane summed its slot's tokens only: the row's full share per lane again
  if constexpr (SL == 4) l_run = slot_sum4(l_run);
  // pairs outside the ring: an odd last context page and the drafted block
  const int npairs = (it.npages + 1) >> 1;
  for (int pp = ring_pairs + w; pp < npairs; pp += NW)
    draft_pair_generic<D, BITS>(a, it, pp, qh, qpos, sc, acc_o, m_run, l_run);

  __syncthreads();  // every wave is done with its ring before the merge reuses the LDS
  l_run = wave_xor_sum(l_run, 16);
  l_run = wave_xor_sum(l_run, 32);
  draft_merge<D, NW>(a, it, smem, acc_o, m_run, l_run);
}

// the KIVI draft for the item's row count: four slots of 4 columns, or one of 16 (a variant of
// two slots for 5 to 8 rows measured no faster, with 4-bit codes: 0.877 against 0.869 ms)
template <int D, int BITS, int NW>
__device__ __forceinline__ void draft_kivi_rows(const AttnArgs& a, const ItemCtx& it, uint8_t* smem) {
  if (it.rows_total <= 4) draft_kivi_item<D, BITS, NW, 4>(a, it, smem);
  else draft_kivi_item<D, BITS, NW, 16>(a, it, smem);
}

// Work item -> (request, row group, split, kv head, layer).  Work-groups are dealt round-robin
// over the 8 XCDs.  With xcd_ranges, consecutive items are mapped to one XCD so that items that
// share K/V (row groups of one unit) run on the same L2; without, work-group b takes item b, so
// every request of a ragged batch is spread over all XCDs instead of each XCD holding a range of
// requests of unequal cost.
// Request of a work item (or merge work-group) in a device request table: the last entry whose
// base (item_base, or merge_base when MERGE) is at most `key`.  The bases ascend, and entry 0's
// is 0.  The wave narrows the range 64-fold per step (1024 requests: two loads per lane), and
// the result is wave-uniform.
template <bool MERGE>
__device__ __forceinline__ int find_req_dev(const ReqDev* t, int n, int key) {
  const int lane = threadIdx.x & 63;
  int lo = 0, cnt = n;
  while (cnt > 1) {
    const int step = (cnt + 63) >> 6;
    const bool in = lane * step < cnt;
    const int idx = lo + (in ? lane * step : 0);
    const int base = MERGE ? t[idx].merge_base : t[idx].item_base;
    const uint64_t m = __ballot(in && base <= key);
    const int j = 63 - __builtin_clzll(m | 1ull);  // lane 0 always qualifies
    lo += j * step;
    cnt = min(step, cnt - j * step);
  }
  return __builtin_amdgcn_readfirstlane(lo);
}

// Entry r of a device request table as wave-uniform values: the loads are vector loads (the
// compiler cannot prove the table unchanged by the kernel's own stores, so it does not use the
// scalar cache), and reading every word back through readfirstlane keeps the request's fields in
// scalar registers, as they are when they come from the kernel arguments.
__device__ __forceinline__ ReqDev uniform_req(const ReqDev* t, int r) {
  constexpr int W = sizeof(ReqDev) / 4;
  const int32_t* src = reinterpret_cast<const int32_t*>(t + r);
  int32_t w[W];
#pragma unroll
  for (int i = 0; i < W; ++i) w[i] = __builtin_amdgcn_readfirstlane(src[i]);
  return __builtin_bit_cast(ReqDev, w);
}

__device__ __forceinline__ bool decode_item(const AttnArgs& a, ItemCtx* it, int* rg) {
  const int b = blockIdx.x;
  const int per = a.nitems_pad >> 3;
  const int item = a.xcd_ranges ? (b & 7) * per + (b >> 3) : b;
  if (item >= a.nitems) return false;
  ReqDev rq;
  if (a.reqs_dev) {
    rq = uniform_req(a.reqs_dev, find_req_dev<false>(a.reqs_dev, a.nreq, item));
  } else {
    int r = 0;
    for (int i = 1; i < a.nreq; ++i)
      if (item >= a.reqs[i].item_base) r = i;
    rq = a.reqs[r];
  }
  int local = item - rq.item_base;
  if (a.xcd_ranges || rq.nrg == 1) {
    *rg = local % rq.nrg;
    local /= rq.nrg;
  } else {
    // work-group b takes item b (ragged batches): the row groups of one unit are placed 8 items
    // apart, so they run on one XCD at about the same time and share its L2; consecutive units
    // still go to different XCDs
    const int R = rq.nrg;
    const int U = a.L * a.Hkv * rq.nsplit;  // units of this request
    const int full = U & ~7;
    if (local < full * R) {
      const int rem = local % (8 * R);
      *rg = rem >> 3;
      local = (local / (8 * R)) * 8 + (rem & 7);
    } else {
      const int t = U - full, j = local - full * R;
      *rg = j / t;
      local = full + j % t;
    }
  }
  const int split = local % rq.nsplit;
  local /= rq.nsplit;
  it->rq = rq;
  it->pool = a.pools[rq.pool];
  it->g = local % a.Hkv;
  it->l = local / a.Hkv;
  it->split = split;
  const int ctx_pages = (rq.ctx_len + kBlock - 1) / kBlock;
  it->p_lo = split * rq.chunk_pages;
  it->nctx = max(0, min(ctx_pages, it->p_lo + rq.chunk_pages) - it->p_lo);
  it->nbk = (split == rq.nsplit - 1) ? (rq.q0 + rq.rows + kBlock - 1) / kBlock : 0;
  it->npages = it->nctx + it->nbk;
  it->rows_total = rq.rows * a.G;
  return true;
}

template <int D, int NW>
__device__ __forceinline__ void draft_dispatch(const AttnArgs& a, const ItemCtx& it, uint8_t* smem) {
  const int bits = it.pool.bits;
  if (bits == 16) draft_bf16_item<D, NW, (NW <= 4 ? 4 : 2)>(a, it, smem);
  else if (bits == 2) draft_kivi_rows<D, 2, NW>(a, it, smem);
  else draft_kivi_rows<D, 4, NW>(a, it, smem);
}

// Verify items only: 8 waves, one work-group per CU (the ring takes most of the LDS).
template <int D>
__global__ __launch_bounds__(kVThreads) void verify_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[VRing<D>::kBytes];
  ItemCtx it;
  int rg;
  if (!decode_item(a, &it, &rg)) return;
  verify_item<D>(a, it, rg, smem);
}

// Verify items only, wide work-groups (a.vwaves waves of 32 rows).
template <int D>
__global__ __launch_bounds__(kWThreads) void verify_wide_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[WRing<D>::kBytes];
  ItemCtx it;
  int rg;
  if (!decode_item(a, &it, &rg)) return;
  verify_wide_item<D>(a, it, rg, smem);
}

// Draft items only, one pool (so one bit width) per launch: 4 waves that split the item's keys.
template <int D>
__global__ __launch_bounds__(kDThreads) void draft_bf16_kernel(const AttnArgs a) {
  // two slots per wave: 72 KB at d = 128, so two work-groups share a CU and one streams while the
  // other starts or finishes an item (four slots, one work-group per CU, was 1 % slower)
  __shared__ __attribute__((aligned(16))) uint8_t smem[draft_bf16_lds<D, kDWaves, 2>()];
  ItemCtx it;
  int rg;
  if (!decode_item(a, &it, &rg)) return;
  draft_bf16_item<D, kDWaves, 2>(a, it, smem);
}

template <int D, int BITS>
__global__ __launch_bounds__(kKThreads) void draft_kivi_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[KRing<D, BITS, kKWaves>::kBytes];
  ItemCtx it;
  int rg;
  if (!decode_item(a, &it, &rg)) return;
  draft_kivi_rows<D, BITS, kKWaves>(a, it, smem);
}

// One launch over a mixed list (drafting and verifying requests of a batch together).
template <int D>
__global__ __launch_bounds__(kVThreads) void mixed_kernel(const AttnArgs a) {
  constexpr int kA = VRing<D>::kBytes > DRing<D>::kBytes ? VRing<D>::kBytes : DRing<D>::kBytes;
  constexpr int kB = KRing<D, 2, kVWaves>::kBytes > KRing<D, 4, kVWaves>::kBytes ? KRing<D, 2, kVWaves>::kBytes
                                                                                  : KRing<D, 4, kVWaves>::kBytes;
  constexpr int kBytes = kA > kB ? kA : kB;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kBytes];
  ItemCtx it;
  int rg;
  if (!decode_item(a, &it, &rg)) return;
  if (it.rq.kind == VC_VERIFY) verify_item<D>(a, it, rg, smem);
  else draft_dispatch<D, kVWaves>(a, it, smem);
}

// Combine split partials with log-sum-exp weights.  A row's D outputs are spread over D / 4
// lanes (4 channels each), so a work-group of 256 threads merges 256 / (D / 4) rows; rows are
// numbered over the (layer, kv head) units of the split requests in request order.  One pass
// over the splits: the running maximum moves when a split's is larger (the sum and the output
// are rescaled then).
// Merge work-groups are dealt per request: request r owns work-groups merge_base[r] ..
// merge_base[r + 1] - 1 (merge_base is the running count, so requests without splits own none).
template <int D>
constexpr int merge_rows_per_group() {
  return 256 / (D / 4);
}

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const AttnArgs a) {
  constexpr int LPR = D / 4;
  constexpr int RPB = merge_rows_per_group<D>();
  const int b = blockIdx.x;
  ReqDev rq;
  if (a.reqs_dev) {
    rq = uniform_req(a.reqs_dev, find_req_dev<true>(a.reqs_dev, a.nreq, b));
  } else {
    int r = 0;
    for (int i = 1; i < a.nreq; ++i)
      if (b >= a.reqs[i].merge_base) r = i;
    rq = a.reqs[r];
  }
  if (rq.nsplit <= 1) return;
  const int rows_total = rq.rows * a.G;
  const int64_t rg = (int64_t)(b - rq.merge_base) * RPB + threadIdx.x / LPR;
  if (rg >= (int64_t)a.L * a.Hkv * rows_total) return;
  const int cq = threadIdx.x % LPR;
  const int64_t unit = rg / rows_total;  // l * Hkv + g
  const int row = (int)(rg % rows_total);
  const int g = (int)(unit % a.Hkv), l = (int)(unit / a.Hkv);
  const float* base = a.part + rq.part_base + ((unit * rq.nsplit) * rows_total + row) * (D + 4);
  const int64_t sstride = (int64_t)rows_total * (D + 4);
  float M = -INFINITY, lsum = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int s = 0; s < rq.nsplit; ++s) {
    const float* p = base + s * sstride;
    const float ms = p[D], ls = p[D + 1];
    const f32x4 os = *reinterpret_cast<const f32x4*>(p + 4 * cq);
    if (ms == -INFINITY) continue;  // a split with no visible key
    if (ms > M) {
      const float c = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - ms);
      o *= c;
      lsum *= c;
      M = ms;
    }
    const float f = __builtin_amdgcn_exp2f(ms - M);
    lsum += f * ls;
    o += f * os;
  }
  o *= lsum > 0.f ? 1.f / lsum : 0.f;
  const int tok = row / a.G, jh = row % a.G;
  float* dst = a.out + ((((int64_t)rq.slot * a.L + l) * a.xmax + rq.q0 + tok) * a.Hq + g * a.G + jh) * D;
  *reinterpret_cast<f32x4*>(dst + 4 * cq) = o;
}

}  // namespace

int launch_attn(const AttnArgs& args, const Plan& plan, int head_dim, hipStream_t stream) {
  if (plan.nitems == 0) return VC_OK;
  const dim3 grid(args.nitems_pad);
  // (args.reqs holds only the first kInlineReqs requests: the kinds come from the plan)
  const bool has_v = plan.has_verify, has_d = plan.has_draft;
  if (args.vwaves) {
    // verify-only launches; the kernel deals the 8 ring slots of a tile over its waves, at most
    // two per wave
    if (has_d || args.vwaves < 4 || args.vwaves > kWideMaxWaves)
      return fail(VC_EINVAL, "internal: bad wide verify plan");
    int nfull;
    const dim3 block(64 * wide_waves(args.vwaves, &nfull));
    if (head_dim == 128) hipLaunchKernelGGL(verify_wide_kernel<128>, grid, block, 0, stream, args);
    else hipLaunchKernelGGL(verify_wide_kernel<64>, grid, block, 0, stream, args);
  } else {
    // a draft-only launch runs the draft kernel of its pools' kind; drafting requests over pools
    // of several kinds (any pool index) take the mixed kernel, which picks the path per item
    const bool mixed = (has_v && has_d) || (has_d && plan.draft_bits < 0);
    if (head_dim == 128) {
      if (mixed) hipLaunchKernelGGL(mixed_kernel<128>, grid, dim3(kVThreads), 0, stream, args);
      else if (has_v) hipLaunchKernelGGL(verify_kernel<128>, grid, dim3(kVThreads), 0, stream, args);
      else if (plan.draft_bits == 16) hipLaunchKernelGGL(draft_bf16_kernel<128>, grid, dim3(kDThreads), 0, stream, args);
      else if (plan.draft_bits == 2) hipLaunchKernelGGL((draft_kivi_kernel<128, 2>), grid, dim3(kKThreads), 0, stream, args);
      else hipLaunchKernelGGL((draft_kivi_kernel<128, 4>), grid, dim3(kKThreads), 0, stream, args);
    } else {
      if (mixed) hipLaunchKernelGGL(mixed_kernel<64>, grid, dim3(kVThreads), 0, stream, args);
      else if (has_v) hipLaunchKernelGGL(verify_kernel<64>, grid, dim3(kVThreads), 0, stream, args);
      else if (plan.draft_bits == 16) hipLaunchKernelGGL(draft_bf16_kernel<64>, grid, dim3(kDThreads), 0, stream, args);
      else if (plan.draft_bits == 2) hipLaunchKernelGGL((draft_kivi_kernel<64, 2>), grid, dim3(kKThreads), 0, stream, args);
      else hipLaunchKernelGGL((draft_kivi_kernel<64, 4>), grid, dim3(kKThreads), 0, stream, args);
    }
  }
  int rc = hip_check(hipGetLastError(), "attention launch");
  if (rc) return rc;
  if (plan.any_split && args.nmerge > 0) {
    const dim3 mgrid((unsigned)args.nmerge);
    if (head_dim == 128) hipLaunchKernelGGL(merge_kernel<128>, mgrid, dim3(256), 0, stream, args);
    else hipLaunchKernelGGL(merge_kernel<64>, mgrid, dim3(256), 0, stream, args);
    rc = hip_check(hipGetLastError(), "merge launch");
  }
  return rc;
}

int merge_rows_per_group(int head_dim) {
  return head_dim == 128 ? merge_rows_per_group<128>() : merge_rows_per_group<64>();
}

// ------------------------------------------------------------------ request table upload
// A launch with more requests than the kernel arguments hold reads its request table from device
// memory.  The table is written there by kernels whose own arguments carry the entries (up to
// kUploadReqs per launch), so the copy is ordered on the stream like the attention launch and
// needs no host staging buffer.
namespace {
constexpr int kUploadReqs = 64;
struct ReqUpload {
  ReqDev* dst;
  int32_t n;
  ReqDev reqs[kUploadReqs];
};
static_assert(sizeof(ReqUpload) <= 4096, "kernel arguments must fit 4 KiB");

__global__ __launch_bounds__(256) void upload_reqs_kernel(const ReqUpload u) {
  constexpr int W = sizeof(ReqDev) / 4;  // 32-bit words per entry
  const int32_t* src = reinterpret_cast<const int32_t*>(u.reqs);
  int32_t* dst = reinterpret_cast<int32_t*>(u.dst);
  for (int i = threadIdx.x; i < u.n * W; i += blockDim.x) dst[i] = src[i];
}
}  // namespace

int upload_req_table(const std::vector<ReqDev>& table, ReqDev* dst, hipStream_t stream) {
  for (size_t i0 = 0; i0 < table.size(); i0 += kUploadReqs) {
    ReqUpload u;
    u.dst = dst + i0;
    u.n = (int32_t)std::min<size_t>(kUploadReqs, table.size() - i0);
    for (int j = 0; j < u.n; ++j) u.reqs[j] = table[i0 + j];
    hipLaunchKernelGGL(upload_reqs_kernel, dim3(1), dim3(256), 0, stream, u);
    const int rc = hip_check(hipGetLastError(), "request table upload");
    if (rc) return rc;
  }
  return VC_OK;
}

}  // namespace vc
