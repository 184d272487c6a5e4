// Greedy accept and the LM-head stand-in.
//
// VeriCache review, §Draft–Verify Pipeline steps 5–6: the drafted token of slot j is kept while
// it equals the verifier's argmax for slot j; at the first difference the verifier's token is
// emitted instead, and when all x agree the verifier's extra (bonus) prediction follows.
#include <math.h>

#include "vc_internal.h"

namespace vc {

namespace {

constexpr int kAccThreads = 256;

// argmax of one row by one wave: ties go to the lowest index
__device__ int wave_argmax(const float* row, int vocab) {
  const int lane = threadIdx.x & 63;
  float best = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int v = lane; v < vocab; v += 64) {
    const float z = row[v];
    if (z > best || (z == best && v < bi)) {
      best = z;
      bi = v;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ob = __shfl_xor(best, o);
    const int oi = __shfl_xor(bi, o);
    if (ob > best || (ob == best && oi < bi)) {
      best = ob;
      bi = oi;
    }
  }
  return bi == 0x7FFFFFFF ? 0 : bi;
}

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
      const int t = wave_argmax(dl + ((int64_t)inst * max_x + rr) * vocab, vocab);
      if (lane == 0) td[rr] = t;
    } else {
      const int j = rr - nx;
      const int t = wave_argmax(vl + ((int64_t)inst * max_xv + j) * vocab, vocab);
      if (lane == 0) tv[j] = t;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int a = nx;
    for (int i = 0; i < nx; ++i)
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

// z = o * W_u, fp32 accumulate.  64x64 output tile per work-group, 4x4 per thread, K steps of 32.
constexpr int kTM = 64, kTN = 64, kTK = 32;

__global__ __launch_bounds__(256) void logits_kernel(int rows, int width, int vocab, const float* o,
                                                     int64_t ld_o, const uint16_t* wu, float* z) {
  __shared__ float sa[kTK][kTM + 4];  // o tile, transposed: [k][m]
  __shared__ float sb[kTK][kTN + 4];  // W tile: [k][n]
  const int m0 = blockIdx.y * kTM, n0 = blockIdx.x * kTN;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < width; k0 += kTK) {
    for (int e = threadIdx.x; e < kTM * kTK; e += 256) {
      const int mm = e / kTK, kk = e % kTK;
      const int gm = m0 + mm, gk = k0 + kk;
      sa[kk][mm] = (gm < rows && gk < width) ? o[(int64_t)gm * ld_o + gk] : 0.f;
    }
    for (int e = threadIdx.x; e < kTK * kTN; e += 256) {
      const int kk = e / kTN, nn = e % kTN;
      const int gk = k0 + kk, gn = n0 + nn;
      sb[kk][nn] = (gk < width && gn < vocab)
                       ? __builtin_bit_cast(float, (uint32_t)wu[(int64_t)gk * vocab + gn] << 16)
                       : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < kTK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = sa[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = sb[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gm = m0 + ty * 4 + i;
    if (gm >= rows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + tx * 4 + j;
      if (gn < vocab) z[(int64_t)gm * vocab + gn] = acc[i][j];
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
  hipLaunchKernelGGL(accept_kernel, dim3(n_inst), dim3(kAccThreads), 0, static_cast<hipStream_t>(stream),
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
  dim3 grid((vocab + kTN - 1) / kTN, (rows + kTM - 1) / kTM);
  hipLaunchKernelGGL(logits_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream), rows, width,
                     vocab, o, ld_o, static_cast<const uint16_t*>(w_u), z);
  return hip_check(hipGetLastError(), "logits launch");
}

}  // extern "C"
