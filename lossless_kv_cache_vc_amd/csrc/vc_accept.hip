// Greedy accept and the LM-head stand-in.
//
// VeriCache review, §Draft–Verify Pipeline steps 5–6: the drafted token of slot j is kept while
// it equals the verifier's argmax for slot j; at the first difference the verifier's token is
// emitted instead, and when all x agree the verifier's extra (bonus) prediction follows.
#include <math.h>

#include "vc_internal.h"

namespace vc {

namespace {

constexpr int kAccThreads = 1024;  // 16 waves per instance: its draft and verify rows in parallel

// fold (z, v) into a lane's running (best, index): larger value wins, ties to the lower index
__device__ __forceinline__ void arg_fold(float z, int v, float& best, int& bi) {
  if (z > best || (z == best && v < bi)) {
    best = z;
    bi = v;
  }
}

// argmax of one row by one wave: ties go to the lowest index.  VEC: the row is 16-byte aligned
// and vocab % 4 == 0, so each lane reads 4 consecutive logits per load, 4 loads in flight.
template <bool VEC>
__device__ int wave_argmax(const float* row, int vocab) {
  const int lane = threadIdx.x & 63;
  float best = -INFINITY;
  int bi = 0x7FFFFFFF;
  if constexpr (VEC) {
    const f32x4* r4 = reinterpret_cast<const f32x4*>(row);
    const int n4 = vocab >> 2;
    int i = lane;
    for (; i + 192 < n4; i += 256) {
      f32x4 c[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) c[u] = r4[i + 64 * u];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) arg_fold(c[u][e], 4 * (i + 64 * u) + e, best, bi);
    }
    for (; i < n4; i += 64) {
      const f32x4 c = r4[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) arg_fold(c[e], 4 * i + e, best, bi);
    }
  } else {
    for (int v = lane; v < vocab; v += 64) arg_fold(row[v], v, best, bi);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ob = __shfl_xor(best, o);
    const int oi = __shfl_xor(bi, o);
    arg_fold(ob, oi, best, bi);
  }
  return bi == 0x7FFFFFFF ? 0 : bi;
}

template <bool VEC>
__global__ __launch_bounds__(kAccThreads) void accept_kernel(int max_x, int max_xv, int vocab, const int32_t* x,
                                                             const int32_t* xv, const float* dl,
                                                             const float* vl, int32_t* dtok,
                                                             int32_t* vtok, int32_t* alen,
                                                             int32_t* ntok) {
  __shared__ int td[VC_MAX_ROWS + 1];
  __shared__ int tv[VC_MAX_ROWS + 1];  // max_xv <= 65
  const int inst = blockIdx.x;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nx = min(max(x[inst], 0), max_x), nxv = min(max(xv[inst], 0), max_xv);
  const int nw = kAccThreads / 64;
  // draft rows then verify rows, one row per wave at a time
  for (int rr = w; rr < nx + nxv; rr += nw) {
    if (rr < nx) {
      const int t = wave_argmax<VEC>(dl + ((int64_t)inst * max_x + rr) * vocab, vocab);
      if (lane == 0) td[rr] = t;
    } else {
      const int j = rr - nx;
      const int t = wave_argmax<VEC>(vl + ((int64_t)inst * max_xv + j) * vocab, vocab);
      if (lane == 0) tv[j] = t;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    // only slots that both passes predicted are compared: a verifier with fewer rows than
    // drafted slots (xv < x) ends the block at its last row
    const int ncmp = min(nx, nxv);
    int a = ncmp;
    for (int i = 0; i < ncmp; ++i)
      if (td[i] != tv[i]) {
        a = i;
        break;
      }
    alen[inst] = a;
    ntok[inst] = a < nxv ? tv[a] : -1;
  }
  for (int i = threadIdx.x; i < max_x; i += kAccThreads)
    dtok[(int64_t)inst * max_x + i] = i < nx ? td[i] : -1;
  for (int i = threadIdx.x; i < max_xv; i += kAccThreads)
    vtok[(int64_t)inst * max_xv + i] = i < nxv ? tv[i] : -1;
}

// z = o * W_u on bf16 MFMA with fp32 accumulation.  Each fp32 element x of o is split into
// bf16 hi = RNE(x) and lo = RNE(x - hi) (x - hi is exact in fp32, so |x - hi - lo| <= 2^-18 |x|);
// W_u is bf16, so hi * w and lo * w are exact in fp32 and z carries only fp32 accumulation error.
// A work-group of 4 waves computes a 128 x 256 tile of z, each wave 64 x 128 (2 x 4 blocks of
// 32 x 32, v_mfma_f32_32x32x16_bf16, so each LDS operand read feeds 2 to 8 products), over K
// steps of 32 staged in LDS: o as hi and lo [m][k],
// W_u transposed to [n][k], so every MFMA operand is one 16-byte LDS read; rows are padded to 40
// bf16 (80 bytes) so the reads of a 32-lane half fall on distinct banks.  The next K step's
// global loads are issued into registers before this step's MFMAs.  VEC: o rows, W_u rows and
// the bases allow 16-byte global loads.
constexpr int kLM = 128, kLN = 256, kLK = 32, kLPad = 40;

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// One K step's global data of a thread: 4 runs of 4 consecutive o elements (rows mm, k kq..kq+3)
// and two k rows of 8 consecutive W_u entries (k 2kp, 2kp + 1; n nq..nq+7).
struct LogitsTile {
  float o[4][4];
  uint32_t w[2][kLN / 128][4];  // [k row][128-column half][packed pairs]
};

template <bool VEC>
__device__ __forceinline__ void logits_fetch(LogitsTile& t, int rows, int width, int vocab, const float* o,
                                             int64_t ld_o, const uint16_t* wu, int m0, int n0, int k0) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid + 256 * i;
    const int mm = e / (kLK / 4), kq = (e % (kLK / 4)) * 4;
    const int gm = m0 + mm, gk = k0 + kq;
    if constexpr (VEC) {  // width % 4 == 0: the 4 elements are all inside or all outside
      const f32x4 v = (gm < rows && gk < width) ? *reinterpret_cast<const f32x4*>(o + (int64_t)gm * ld_o + gk)
                                                : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) t.o[i][j] = v[j];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) t.o[i][j] = (gm < rows && gk + j < width) ? o[(int64_t)gm * ld_o + gk + j] : 0.f;
    }
  }
  const int kp = tid % (kLK / 2), nq = (tid / (kLK / 2)) * 8;
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int hf = 0; hf < kLN / 128; ++hf) {
      const int gk = k0 + 2 * kp + r, gn = n0 + 128 * hf + nq;
      if constexpr (VEC) {  // vocab % 8 == 0
        const u32x4 v = (gk < width && gn < vocab) ? *reinterpret_cast<const u32x4*>(wu + (int64_t)gk * vocab + gn)
                                                   : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < 4; ++j) t.w[r][hf][j] = v[j];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t lo = (gk < width && gn + 2 * j < vocab) ? wu[(int64_t)gk * vocab + gn + 2 * j] : 0;
          const uint32_t hi = (gk < width && gn + 2 * j + 1 < vocab) ? wu[(int64_t)gk * vocab + gn + 2 * j + 1] : 0;
          t.w[r][hf][j] = lo | (hi << 16);
        }
      }
    }
}

// o as bf16 hi and lo parts [m][k]; W_u transposed [n][k], the thread's two k rows packed into
// one 32-bit store per n (consecutive threads take consecutive k pairs: distinct banks)
__device__ __forceinline__ void logits_stage(const LogitsTile& t, uint16_t* s_hi, uint16_t* s_lo, uint16_t* s_w) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid + 256 * i;
    const int mm = e / (kLK / 4), kq = (e % (kLK / 4)) * 4;
    uint32_t hi[2], lo[2];
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      const uint16_t h0 = bf16_bits(t.o[i][j]), h1 = bf16_bits(t.o[i][j + 1]);
      const float r0 = t.o[i][j] - __builtin_bit_cast(float, (uint32_t)h0 << 16);
      const float r1 = t.o[i][j + 1] - __builtin_bit_cast(float, (uint32_t)h1 << 16);
      hi[j >> 1] = h0 | ((uint32_t)h1 << 16);
      lo[j >> 1] = bf16_bits(r0) | ((uint32_t)bf16_bits(r1) << 16);
    }
    *reinterpret_cast<u32x2*>(s_hi + mm * kLPad + kq) = u32x2{hi[0], hi[1]};
    *reinterpret_cast<u32x2*>(s_lo + mm * kLPad + kq) = u32x2{lo[0], lo[1]};
  }
  const int kp = tid % (kLK / 2), nq = (tid / (kLK / 2)) * 8;
#pragma unroll
  for (int hf = 0; hf < kLN / 128; ++hf)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t w0 = (t.w[0][hf][j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      const uint32_t w1 = (t.w[1][hf][j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      *reinterpret_cast<uint32_t*>(s_w + (128 * hf + nq + j) * kLPad + 2 * kp) = w0 | (w1 << 16);
    }
}

template <bool VEC>
__global__ __launch_bounds__(256) void logits_kernel(int rows, int width, int vocab, const float* o,
                                                     int64_t ld_o, const uint16_t* wu, float* z) {
  __shared__ __attribute__((aligned(16))) uint16_t s_hi[kLM * kLPad];
  __shared__ __attribute__((aligned(16))) uint16_t s_lo[kLM * kLPad];
  __shared__ __attribute__((aligned(16))) uint16_t s_w[kLN * kLPad];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int m0 = blockIdx.y * kLM, n0 = blockIdx.x * kLN;
  constexpr int NJ = kLN / 64;  // 32-column blocks of a wave
  const int wm = (w & 1) * 64, wn = (w >> 1) * (kLN / 2);  // this wave's 64 x kLN/2 part of the tile
  const int r32 = lane & 31, kh = lane >> 5;
  f32x16 acc[2][NJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};
  LogitsTile t;
  logits_fetch<VEC>(t, rows, width, vocab, o, ld_o, wu, m0, n0, 0);
  for (int k0 = 0; k0 < width; k0 += kLK) {
    logits_stage(t, s_hi, s_lo, s_w);
    __syncthreads();
    // the next K step's loads are in flight while this step's MFMAs run
    if (k0 + kLK < width) logits_fetch<VEC>(t, rows, width, vocab, o, ld_o, wu, m0, n0, k0 + kLK);
#pragma unroll
    for (int ks = 0; ks < kLK / 16; ++ks) {
      const int kc = ks * 16 + kh * 8;  // lane's 8 k of this 16-k step
      u32x4 ah[2], al[2], bw[NJ];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        ah[i] = *reinterpret_cast<const u32x4*>(s_hi + (wm + 32 * i + r32) * kLPad + kc);
        al[i] = *reinterpret_cast<const u32x4*>(s_lo + (wm + 32 * i + r32) * kLPad + kc);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) bw[j] = *reinterpret_cast<const u32x4*>(s_w + (wn + 32 * j + r32) * kLPad + kc);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ah[i]),
                                                              __builtin_bit_cast(bf16x8, bw[j]), acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, al[i]),
                                                              __builtin_bit_cast(bf16x8, bw[j]), acc[i][j], 0, 0, 0);
        }
    }
    __syncthreads();
  }
  // accumulator r of a 32 x 32 block: row 8 (r / 4) + 4 kh + r % 4, column r32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int gn = n0 + wn + 32 * j + r32;
      if (gn >= vocab) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gm = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * kh + (r & 3);
        if (gm < rows) z[(int64_t)gm * vocab + gn] = acc[i][j][r];
      }
    }
}

}  // namespace

}  // namespace vc

using namespace vc;

extern "C" {

int vc_accept(int n_inst, int max_x, int max_xv, int vocab, const int32_t* x, const int32_t* xv,
              const float* draft_logits, const float* verify_logits, int32_t* draft_tok,
              int32_t* verify_tok, int32_t* accept_len, int32_t* next_tok, void* stream) {
  set_error("");
  if (n_inst < 0) return fail(VC_EINVAL, "n_inst must be >= 0");
  if (n_inst == 0) return VC_OK;
  if (max_x < 1 || max_x > VC_MAX_ROWS) return fail(VC_EINVAL, "max_x must be in [1, 64]");
  if (max_xv < 1 || max_xv > VC_MAX_ROWS + 1) return fail(VC_EINVAL, "max_xv must be in [1, 65]");
  if (vocab < 1) return fail(VC_EINVAL, "vocab must be >= 1");
  if (!x || !xv || !draft_logits || !verify_logits || !draft_tok || !verify_tok || !accept_len ||
      !next_tok)
    return fail(VC_EINVAL, "NULL argument");
  const bool vec = vocab % 4 == 0 && reinterpret_cast<uintptr_t>(draft_logits) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(verify_logits) % 16 == 0;
  if (vec)
    hipLaunchKernelGGL(accept_kernel<true>, dim3(n_inst), dim3(kAccThreads), 0, static_cast<hipStream_t>(stream),
                       max_x, max_xv, vocab, x, xv, draft_logits, verify_logits, draft_tok, verify_tok, accept_len,
                       next_tok);
  else
    hipLaunchKernelGGL(accept_kernel<false>, dim3(n_inst), dim3(kAccThreads), 0, static_cast<hipStream_t>(stream),
                       max_x, max_xv, vocab, x, xv, draft_logits, verify_logits, draft_tok, verify_tok, accept_len,
                       next_tok);
  return hip_check(hipGetLastError(), "accept launch");
}

int vc_logits(int rows, int width, int vocab, const float* o, int64_t ld_o, const void* w_u, float* z,
              void* stream) {
  set_error("");
  if (rows < 0 || width < 1 || vocab < 1 || ld_o < width) return fail(VC_EINVAL, "bad logits shape");
  if (rows == 0) return VC_OK;
  if (!o || !w_u || !z) return fail(VC_EINVAL, "NULL argument");
  if ((rows + kLM - 1) / kLM > 65535) return fail(VC_EINVAL, "too many logits rows");
  const dim3 grid((vocab + kLN - 1) / kLN, (rows + kLM - 1) / kLM);
  const bool vec = ld_o % 4 == 0 && width % 4 == 0 && vocab % 8 == 0 &&
                   reinterpret_cast<uintptr_t>(o) % 16 == 0 && reinterpret_cast<uintptr_t>(w_u) % 16 == 0;
  const uint16_t* wu = static_cast<const uint16_t*>(w_u);
  if (vec)
    hipLaunchKernelGGL(logits_kernel<true>, grid, dim3(256), 0, static_cast<hipStream_t>(stream), rows, width,
                       vocab, o, ld_o, wu, z);
  else
    hipLaunchKernelGGL(logits_kernel<false>, grid, dim3(256), 0, static_cast<hipStream_t>(stream), rows, width,
                       vocab, o, ld_o, wu, z);
  return hip_check(hipGetLastError(), "logits launch");
}

}  // extern "C"
