// Draft and verify attention over paged KV caches for gfx950 (CDNA4).
//
// VeriCache review, §Draft–Verify Pipeline: the verifier runs one pass over the x drafted
// positions against the full cache (position i conditioned on drafted rows before and at i);
// the drafter runs one single-token step against the compressed cache.  Both are
// softmax(q k^T / sqrt(d)) v (§Prerequisites, attention equation) over different key sets.
//
// One launch processes a list of work items; an item is (request, layer, kv head, context
// split, row group).  Each work-group has 4 wave64s and takes one of two paths:
//
//  * verify path — the x*G query rows of a kv head are a dense block: each wave owns 32 rows,
//    K/V tiles of 64 keys (4 pages) are staged through LDS (double buffered) and shared by the
//    4 waves; S^T = K Q^T and O^T += V^T P^T use v_mfma_f32_32x32x16_bf16, so each lane holds
//    one query row of both accumulators and the softmax needs only one cross-lane exchange.
//  * draft path — G <= 16 rows: the waves split the keys of the item, load K/V pages straight
//    into registers in MFMA operand order (v_mfma_f32_16x16x32_bf16, rows padded to 16),
//    dequantise KIVI codes in registers, and merge the per-wave softmax states through LDS.
//
// Long contexts are split into chunks of pages; partial (max, sum, output) states go to the
// workspace and a merge kernel combines them with log-sum-exp weights.
#include <math.h>

#include "vc_internal.h"

namespace vc {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileKeys = 64;        // keys per verify tile (4 pages)
constexpr int kRowsPerGroup = 32 * kWaves;
constexpr float kLazyRescale = 8.0f;  // log2 headroom before the running max is moved

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ bf16x8 as_bf(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 t;
  t[0] = (__bf16)a;
  t[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, t);
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

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __builtin_bit_cast(float, b << 16);
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

struct ItemCtx {
  const ReqDev* rq;
  const PoolDev* pool;
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
  const ReqDev& rq = *it.rq;
  if (ip < it.nctx) {
    const PoolDev& pl = *it.pool;
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
      int pe = p & ~1;
      int phys_e = pl.page_table[(int64_t)rq.page_row * pl.max_pages + pe];
      if (phys_e < 0 || phys_e >= pl.nblk) phys_e = phys;
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
  const ReqDev& rq = *it.rq;
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

// ------------------------------------------------------------------ verify path (32x32x16)
template <int D>
struct VerifySmem {
  static constexpr int kStageK = kTileKeys * D * 2;  // bytes
  static constexpr int kStage = 2 * kStageK;          // K then V
  static constexpr int kBytes = 2 * kStage;           // double buffered
};

// key slot of MFMA row M within a 32-key block: lanes' accumulator registers then hold
// 8 consecutive tokens of one page, which is the B-operand order of the value product.
__device__ __forceinline__ int key_of_m32(int M) {
  return 16 * (M >> 4) + 8 * ((M >> 2) & 1) + 4 * ((M >> 3) & 1) + (M & 3);
}

template <int D>
__device__ __forceinline__ int swz_k(int key) {
  return D == 128 ? (key & 15) : ((key >> 1) & 7);
}

template <int D>
__device__ void verify_item(const AttnArgs& a, const ItemCtx& it, int rg, uint8_t* smem) {
  constexpr int CPP = 2 * D;                 // 16-byte chunks per page (K or V)
  constexpr int NCH = 4 * CPP / kThreads;    // chunks per thread per tensor per tile
  constexpr int CPR = D / 8;                 // chunks per key row
  constexpr int NS = D / 16;                 // MFMA k-steps of the score product
  constexpr int ND = D / 32;                 // 32-wide d blocks of the output
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 31, h = lane >> 5;
  const ReqDev& rq = *it.rq;
  const int G = a.G;
  const int row = rg * kRowsPerGroup + 32 * w + n;
  const bool wave_on = rg * kRowsPerGroup + 32 * w < it.rows_total;
  const bool row_ok = row < it.rows_total;
  const int tok = row_ok ? row / G : 0;
  const int qpos = rq.q0 + tok;

  // query rows as the B operand of S^T = K Q^T
  u32x4 qreg[NS];
  {
    const uint16_t* qp = a.q + ((((int64_t)rq.slot * a.L + it.l) * a.xmax + rq.q0 + tok) * a.Hq +
                                it.g * G + (row_ok ? row % G : 0)) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) qreg[s] = row_ok ? ld16(qp + 16 * s + 8 * h) : u32x4{0, 0, 0, 0};
  }

  f32x16 acc_o[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc_o[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sc = a.scale_log2;

  const int ntiles = (it.npages + 3) >> 2;
  u32x4 kbuf[NCH], vbuf[NCH];

  // chunk j of this thread: page (j * kThreads + tid) / CPP, which is j for d = 128 and
  // 2j + (tid >= 128) for d = 64 (uniform per wave either way)
  auto load_tile = [&](int t) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = tid + kThreads * j;
      const int off = c % CPP;
      PageRef p;
      if (CPP == kThreads) {
        p = page_ref<D>(a, it, 4 * t + j, false);
      } else {
        const PageRef p0 = page_ref<D>(a, it, 4 * t + 2 * j, false);
        const PageRef p1 = page_ref<D>(a, it, 4 * t + 2 * j + 1, false);
        p = (tid >= CPP) ? p1 : p0;
      }
      u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (p.kind != 2) {
        const int ktok = off / CPR;
        if (ktok < p.valid) kv = ld16(p.k + off * 16);
        vv = ld16(p.v + off * 16);
        if (p.valid < kBlock) vv = mask_tokens(vv, (off & 1) * 8, p.valid);
      }
      kbuf[j] = kv;
      vbuf[j] = vv;
    }
  };
  auto store_tile = [&](int st) {
    uint8_t* sk = smem + st * VerifySmem<D>::kStage;
    uint8_t* sv = sk + VerifySmem<D>::kStageK;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = tid + kThreads * j;
      const int ps = (CPP == kThreads) ? j : 2 * j + (tid >= CPP ? 1 : 0), off = c % CPP;
      const int key = ps * kBlock + off / CPR, cc = off % CPR;
      *reinterpret_cast<u32x4*>(sk + key * (2 * D) + ((cc ^ swz_k<D>(key)) * 16)) = kbuf[j];
      const int dd = off >> 1, half = off & 1;
      *reinterpret_cast<u32x4*>(sv + (ps * D + dd) * 32 + ((half ^ ((dd >> 3) & 1)) * 16)) = vbuf[j];
    }
  };

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int st = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);

    if (wave_on) {
      const uint8_t* sk = smem + st * VerifySmem<D>::kStage;
      const uint8_t* sv = sk + VerifySmem<D>::kStageK;
      f32x16 s_acc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s_acc[kb] = f32x16{};
        const int key = 32 * kb + key_of_m32(n);
        const uint8_t* krow = sk + key * (2 * D);
        const int sw = swz_k<D>(key);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          u32x4 av = ld16(krow + (((2 * s + h) ^ sw) * 16));
          s_acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(av), as_bf(qreg[s]), s_acc[kb],
                                                              0, 0, 0);
        }
      }
      // masking: only tiles holding a partial or drafted-block page need it
      PageRef pr[4];
      bool need_mask = false;
#pragma unroll
      for (int ps = 0; ps < 4; ++ps) {
        pr[ps] = page_ref<D>(a, it, 4 * t + ps, false);
        need_mask |= (pr[ps].kind != 0) || (pr[ps].valid < kBlock);
      }
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ps = 2 * kb + (r >> 3), tt = 8 * h + (r & 7);
            if (!key_visible(pr[ps], tt, qpos)) s_acc[kb][r] = -INFINITY;
          }
      }
      float mloc = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, s_acc[kb][r]);
      mloc = wave_xor_max(mloc, 32);
      const float m_new = fmaxf(m_run, mloc * sc);
      if (__any(m_new > m_run + kLazyRescale)) {
        const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < ND; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc_o[i][r] *= alpha;
        m_run = m_new;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      float lsum = 0.f;
      uint32_t pb[2][8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s_acc[kb][r], sc, -m_use));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s_acc[kb][r + 1], sc, -m_use));
          lsum += p0 + p1;
          pb[kb][r >> 1] = pack_bf16(p0, p1);
        }
      l_run += lsum;
      // O^T += V^T P^T, one page (16 keys) per k-step
#pragma unroll
      for (int pj = 0; pj < 4; ++pj) {
        const int kb = pj >> 1, hf = pj & 1;
        u32x4 bv = {pb[kb][4 * hf], pb[kb][4 * hf + 1], pb[kb][4 * hf + 2], pb[kb][4 * hf + 3]};
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const int dd = 32 * db + n;
          u32x4 av = ld16(sv + (pj * D + dd) * 32 + ((h ^ ((dd >> 3) & 1)) * 16));
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(av), as_bf(bv), acc_o[db], 0, 0, 0);
        }
      }
    }

    if (t + 1 < ntiles) store_tile(st ^ 1);
    __syncthreads();
  }

  if (!wave_on) return;
  const float l_tot = wave_xor_sum(l_run, 32);
  if (!row_ok) return;
  bool partial;
  float* dst = out_row<D>(a, it, row, &partial);
  const float inv = partial ? 1.f : 1.f / l_tot;
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4 o = {acc_o[db][4 * q] * inv, acc_o[db][4 * q + 1] * inv, acc_o[db][4 * q + 2] * inv,
                 acc_o[db][4 * q + 3] * inv};
      *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * q + 4 * h) = o;
    }
  if (partial && h == 0) {
    dst[D] = m_run;
    dst[D + 1] = l_tot;
  }
}

// ------------------------------------------------------------------ draft path (16x16x32)
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

template <int D, int BITS>
__device__ void draft_item(const AttnArgs& a, const ItemCtx& it, uint8_t* smem) {
  constexpr bool KIVI = BITS != 16;
  constexpr int NS = D / 32;   // k-steps of the score product (16x16x32)
  constexpr int ND = D / 16;   // 16-wide d blocks of the output
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, kg = lane >> 4;
  const ReqDev& rq = *it.rq;
  const int G = a.G;
  const bool row_ok = n < it.rows_total;
  const int tok = row_ok ? n / G : 0;
  const int qpos = rq.q0 + tok;

  u32x4 qreg[NS];
  {
    const uint16_t* qp = a.q + ((((int64_t)rq.slot * a.L + it.l) * a.xmax + rq.q0 + tok) * a.Hq +
                                it.g * G + (row_ok ? n % G : 0)) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      qreg[s] = row_ok ? ld16(qp + (KIVI ? draft_chan<D>(kg, s) : 32 * s + 8 * kg)) : u32x4{0, 0, 0, 0};
    if constexpr (KIVI) {
#pragma unroll
      for (int s = 0; s < NS; ++s) qreg[s] = bf16x8_to_f16x8(qreg[s]);
    }
  }

  f32x4 acc_o[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc_o[i] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sc = a.scale_log2;
  const int npairs = (it.npages + 1) >> 1;

  for (int pp = w; pp < npairs; pp += kWaves) {
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
        const uint32_t* szp = reinterpret_cast<const uint32_t*>(p.ksz) + kg * (D / 4);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          float code[8];
          unpack8<BITS>(words, 8 * s, code);
          uint32_t pk[4];
#pragma unroll
          for (int j = 0; j < 8; j += 2) {
            const uint32_t sz0 = szp[8 * s + j], sz1 = szp[8 * s + j + 1];
            const float k0 = fmaf(code[j], fp16_bits_to_f32(sz0 & 0xFFFF), fp16_bits_to_f32(sz0 >> 16));
            const float k1 = fmaf(code[j + 1], fp16_bits_to_f32(sz1 & 0xFFFF), fp16_bits_to_f32(sz1 >> 16));
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
    if (__any(m_new > m_run + kLazyRescale)) {
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
          const uint32_t* szp = reinterpret_cast<const uint32_t*>(vp.vsz) + (dd >> 5) * kBlock + t0;
          uint32_t pk[4];
#pragma unroll
          for (int j = 0; j < 8; j += 2) {
            const uint32_t sz0 = szp[j], sz1 = szp[j + 1];
            float v0 = fmaf(code[j], fp16_bits_to_f32(sz0 & 0xFFFF), fp16_bits_to_f32(sz0 >> 16));
            float v1 = fmaf(code[j + 1], fp16_bits_to_f32(sz1 & 0xFFFF), fp16_bits_to_f32(sz1 >> 16));
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

  // ---- merge the 4 waves' states through LDS
  l_run = wave_xor_sum(l_run, 16);
  l_run = wave_xor_sum(l_run, 32);
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
  for (int task = tid; task < 16 * NQ; task += kThreads) {
    const int rr = task / NQ, cq = task % NQ;
    if (rr >= it.rows_total) continue;
    float mw[kWaves], M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      mw[ww] = red[(ww * 16 + rr) * RS + D];
      M = fmaxf(M, mw[ww]);
    }
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = (mw[ww] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw[ww] - M);
      lsum += f * red[(ww * 16 + rr) * RS + D + 1];
      const f32x4 ow = *reinterpret_cast<const f32x4*>(red + (ww * 16 + rr) * RS + 4 * cq);
      o += f * ow;
    }
    bool partial;
    float* dst = out_row<D>(a, it, rr, &partial);
    if (!partial) o *= 1.f / lsum;
    *reinterpret_cast<f32x4*>(dst + 4 * cq) = o;
    if (partial && cq == 0) {
      dst[D] = M;
      dst[D + 1] = lsum;
    }
  }
}

// MODE 0: verify items only, 1: draft items only, 2: both (one launch over a mixed batch)
template <int D, int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[VerifySmem<D>::kBytes];
  // consecutive items run on the same XCD (work-groups are dealt round-robin over 8 XCDs)
  const int b = blockIdx.x;
  const int per = a.nitems_pad >> 3;
  const int item = (b & 7) * per + (b >> 3);
  if (item >= a.nitems) return;
  int r = 0;
  for (int i = 1; i < a.nreq; ++i)
    if (item >= a.reqs[i].item_base) r = i;
  const ReqDev& rq = a.reqs[r];
  int local = item - rq.item_base;
  const int rg = local % rq.nrg;
  local /= rq.nrg;
  const int split = local % rq.nsplit;
  local /= rq.nsplit;
  const int g = local % a.Hkv;
  const int l = local / a.Hkv;

  ItemCtx it;
  it.rq = &rq;
  it.pool = &a.pools[rq.pool];
  it.l = l;
  it.g = g;
  it.split = split;
  const int ctx_pages = (rq.ctx_len + kBlock - 1) / kBlock;
  it.p_lo = split * rq.chunk_pages;
  it.nctx = max(0, min(ctx_pages, it.p_lo + rq.chunk_pages) - it.p_lo);
  it.nbk = (split == rq.nsplit - 1) ? (rq.q0 + rq.rows + kBlock - 1) / kBlock : 0;
  it.npages = it.nctx + it.nbk;
  it.rows_total = rq.rows * a.G;

  if (MODE != 1 && rq.kind == VC_VERIFY) {
    verify_item<D>(a, it, rg, smem);
  } else if (MODE != 0) {
    const int bits = it.pool->bits;
    if (bits == 16) draft_item<D, 16>(a, it, smem);
    else if (bits == 2) draft_item<D, 2>(a, it, smem);
    else draft_item<D, 4>(a, it, smem);
  }
}

// Combine split partials: one work-group per (request, layer, kv head) with nsplit > 1.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const AttnArgs a) {
  int b = blockIdx.x;
  int r = -1;
  for (int i = 0; i < a.nreq; ++i) {
    if (a.reqs[i].nsplit <= 1) continue;
    const int cnt = a.L * a.Hkv;
    if (b < cnt) {
      r = i;
      break;
    }
    b -= cnt;
  }
  if (r < 0) return;
  const ReqDev& rq = a.reqs[r];
  const int g = b % a.Hkv, l = b / a.Hkv;
  const int rows_total = rq.rows * a.G;
  constexpr int NQ = D / 4;
  for (int task = threadIdx.x; task < rows_total * NQ; task += 256) {
    const int row = task / NQ, cq = task % NQ;
    const float* base = a.part + rq.part_base +
                        ((((int64_t)l * a.Hkv + g) * rq.nsplit) * rows_total + row) * (D + 4);
    const int64_t sstride = (int64_t)rows_total * (D + 4);
    float M = -INFINITY;
    for (int s = 0; s < rq.nsplit; ++s) M = fmaxf(M, base[s * sstride + D]);
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
    for (int s = 0; s < rq.nsplit; ++s) {
      const float ms = base[s * sstride + D];
      const float f = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - M);
      lsum += f * base[s * sstride + D + 1];
      o += f * *reinterpret_cast<const f32x4*>(base + s * sstride + 4 * cq);
    }
    o *= 1.f / lsum;
    const int tok = row / a.G, jh = row % a.G;
    float* dst = a.out + ((((int64_t)rq.slot * a.L + l) * a.xmax + rq.q0 + tok) * a.Hq + g * a.G + jh) * D;
    *reinterpret_cast<f32x4*>(dst + 4 * cq) = o;
  }
}

}  // namespace

int launch_attn(const AttnArgs& args, const Plan& plan, int head_dim, hipStream_t stream) {
  if (plan.nitems == 0) return VC_OK;
  dim3 grid(args.nitems_pad), block(kThreads);
  bool has_v = false, has_d = false;
  for (int i = 0; i < args.nreq; ++i) (args.reqs[i].kind == VC_VERIFY ? has_v : has_d) = true;
  const int mode = has_v && has_d ? 2 : (has_v ? 0 : 1);
  if (head_dim == 128) {
    if (mode == 0) hipLaunchKernelGGL((attn_kernel<128, 0>), grid, block, 0, stream, args);
    else if (mode == 1) hipLaunchKernelGGL((attn_kernel<128, 1>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((attn_kernel<128, 2>), grid, block, 0, stream, args);
  } else {
    if (mode == 0) hipLaunchKernelGGL((attn_kernel<64, 0>), grid, block, 0, stream, args);
    else if (mode == 1) hipLaunchKernelGGL((attn_kernel<64, 1>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((attn_kernel<64, 2>), grid, block, 0, stream, args);
  }
  int rc = hip_check(hipGetLastError(), "attention launch");
  if (rc) return rc;
  if (plan.any_split) {
    int nmerge = 0;
    for (int i = 0; i < args.nreq; ++i)
      if (args.reqs[i].nsplit > 1) nmerge += args.L * args.Hkv;
    if (head_dim == 128) hipLaunchKernelGGL(merge_kernel<128>, dim3(nmerge), dim3(256), 0, stream, args);
    else hipLaunchKernelGGL(merge_kernel<64>, dim3(nmerge), dim3(256), 0, stream, args);
    rc = hip_check(hipGetLastError(), "merge launch");
  }
  return rc;
}

}  // namespace vc
