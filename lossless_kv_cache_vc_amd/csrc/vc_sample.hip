// Rejection-sampling accept (temperature > 0) and the drafter's sampling step.
//
// VeriCache review, §Implementation notes worth absorbing, "Rejection sampling for non-greedy":
// the drafter samples t_i from its own distribution p_lossy; the verifier keeps t_i with
// probability min(1, p_full(t_i) / p_lossy(t_i)); at the first slot it does not keep, one token
// is drawn from the residual (p_full - p_lossy, negative parts removed) and the block ends; the
// emitted tokens then follow p_full exactly.
//
// Probabilities are float64 softmax(z / T) of the fp32 logits.  The keep test compares
// u * p_lossy(t) with p_full(t) (no division).  A draw takes one uniform u in (0, 1) and returns
// the smallest index whose prefix sum exceeds u times the total weight (inverse CDF).  Uniforms
// are inputs: the caller owns the random numbers.
//
// One work-group per row (sampling) or per drafted block (accept: each wave decides whole slots,
// then the work-group draws once).  A draw sums contiguous chunks of the vocabulary per thread,
// scans the chunk sums, and lets the thread whose chunk holds the crossing walk it.
#include <limits.h>
#include <math.h>

#include "vc_internal.h"

namespace vc {

namespace {

constexpr int kSThreads = 256;    // sampling: one work-group per row
constexpr int kAThreads = 1024;   // accept: one work-group of 16 waves per drafted block

template <int NT>
struct SampleLds {
  static constexpr int NW = NT / 64;
  double part[NW];  // per-wave partials (reductions; the draw's exclusive prefix of wave sums)
  int ipart[NW];
  double total;
  int flag;
  int keep[VC_MAX_ROWS];  // accept: keep decision of each slot
};

template <int NT>
__device__ double block_sum(double v, SampleLds<NT>& s) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s.part[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < SampleLds<NT>::NW; ++i) t += s.part[i];
  return t;
}

template <int NT>
__device__ double block_max(double v, SampleLds<NT>& s) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s.part[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = s.part[0];
#pragma unroll
  for (int i = 1; i < SampleLds<NT>::NW; ++i) t = fmax(t, s.part[i]);
  return t;
}

template <int NT>
__device__ int block_min_int(int v, SampleLds<NT>& s) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s.ipart[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = s.ipart[0];
#pragma unroll
  for (int i = 1; i < SampleLds<NT>::NW; ++i) t = min(t, s.ipart[i]);
  return t;
}

template <int NT>
__device__ int block_max_int(int v, SampleLds<NT>& s) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s.ipart[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = s.ipart[0];
#pragma unroll
  for (int i = 1; i < SampleLds<NT>::NW; ++i) t = max(t, s.ipart[i]);
  return t;
}

// softmax(z / T) of one row: p(k) = exp((z_k - m) / T) / s
struct Softmax {
  const float* z;
  double m, s, t;
  __device__ double p(int k) const { return exp(((double)z[k] - m) / t) / s; }
};

template <int NT>
__device__ Softmax row_softmax(const float* z, int vocab, double t, SampleLds<NT>& s) {
  double mx = -INFINITY;
  for (int k = threadIdx.x; k < vocab; k += NT) mx = fmax(mx, (double)z[k]);
  Softmax r{z, block_max(mx, s), 1.0, t};
  double e = 0.0;
  for (int k = threadIdx.x; k < vocab; k += NT) e += exp(((double)z[k] - r.m) / t);
  r.s = block_sum(e, s);
  return r;
}

// The same softmax statistics computed by one wave alone (no work-group synchronisation).
__device__ Softmax wave_softmax(const float* z, int vocab, double t) {
  const int lane = threadIdx.x & 63;
  double mx = -INFINITY;
  for (int k = lane; k < vocab; k += 64) mx = fmax(mx, (double)z[k]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
  double e = 0.0;
  for (int k = lane; k < vocab; k += 64) e += exp(((double)z[k] - mx) / t);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) e += __shfl_xor(e, o);
  return Softmax{z, mx, e, t};
}

// Inverse-CDF draws.  Each thread owns a contiguous chunk of the vocabulary; the chunk sums are
// scanned within each wave (shuffles) and across the waves; the thread whose chunk holds the
// crossing walks it.  Chunks of up to kCache weights are evaluated once and kept in registers.
constexpr int kCache = 16;

// The draw over chunk weights wc[0 .. k1 - k0) of this thread (sum cs), from uniform u.
template <int NT>
__device__ int draw_cached(const double (&wc)[kCache], int k0, int k1, double cs, double u, SampleLds<NT>& s) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  double inc = cs;  // inclusive scan of the chunk sums within the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double v = __shfl_up(inc, o);
    if (lane >= o) inc += v;
  }
  __syncthreads();
  if (lane == 63) s.part[wv] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double run = 0.0;
    for (int i = 0; i < SampleLds<NT>::NW; ++i) {
      const double c = s.part[i];
      s.part[i] = run;
      run += c;
    }
    s.total = run;
  }
  __syncthreads();
  const double target = u * s.total;
  double run = s.part[wv] + (inc - cs);
  int found = INT_MAX, last = -1;
#pragma unroll
  for (int i = 0; i < kCache; ++i) {
    if (k0 + i >= k1) break;
    const double wk = wc[i];
    run += wk;
    if (wk > 0.0) last = k0 + i;
    if (found == INT_MAX && run > target) found = k0 + i;
  }
  found = block_min_int(found, s);
  if (found == INT_MAX) found = block_max_int(last, s);  // rounding left u * total above every prefix
  return found < 0 ? 0 : found;
}

// Draw with uniform u from the non-negative weights w(k), k < vocab (the smallest index whose
// prefix sum exceeds u times the total).
template <int NT, class W>
__device__ int block_draw(const W& w, int vocab, double u, SampleLds<NT>& s) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int per = (vocab + NT - 1) / NT;
  const int k0 = min((int)threadIdx.x * per, vocab), k1 = min(k0 + per, vocab);
  if (per <= kCache) {
    double wc[kCache];
    double cs = 0.0;
#pragma unroll
    for (int i = 0; i < kCache; ++i) {
      wc[i] = k0 + i < k1 ? w(k0 + i) : 0.0;
      cs += wc[i];
    }
    return draw_cached(wc, k0, k1, cs, u, s);
  }
  double cs = 0.0;
  for (int k = k0; k < k1; ++k) cs += w(k);
  double inc = cs;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double v = __shfl_up(inc, o);
    if (lane >= o) inc += v;
  }
  __syncthreads();
  if (lane == 63) s.part[wv] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double run = 0.0;
    for (int i = 0; i < SampleLds<NT>::NW; ++i) {
      const double c = s.part[i];
      s.part[i] = run;
      run += c;
    }
    s.total = run;
  }
  __syncthreads();
  const double target = u * s.total;
  double run = s.part[wv] + (inc - cs);
  int found = INT_MAX, last = -1;
  for (int k = k0; k < k1; ++k) {
    const double wk = w(k);
    run += wk;
    if (wk > 0.0) last = k;
    if (found == INT_MAX && run > target) found = k;
  }
  found = block_min_int(found, s);
  if (found == INT_MAX) found = block_max_int(last, s);  // rounding left u * total above every prefix
  return found < 0 ? 0 : found;
}

__global__ __launch_bounds__(kSThreads) void sample_kernel(int vocab, double t, const float* logits,
                                                           const double* u, int32_t* tokens) {
  __shared__ SampleLds<kSThreads> s;
  const int row = blockIdx.x;
  const float* z = logits + (int64_t)row * vocab;
  const int per = (vocab + kSThreads - 1) / kSThreads;
  int tok;
  if (per <= kCache) {
    // one exponential per entry: the row maximum over the thread's chunk, then unnormalised
    // weights exp((z - m) / T), drawn from directly (normalising does not move the crossing)
    const int k0 = min((int)threadIdx.x * per, vocab), k1 = min(k0 + per, vocab);
    double mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kCache; ++i)
      if (k0 + i < k1) mx = fmax(mx, (double)z[k0 + i]);
    const double m = block_max(mx, s);
    double wc[kCache];
    double cs = 0.0;
#pragma unroll
    for (int i = 0; i < kCache; ++i) {
      wc[i] = k0 + i < k1 ? exp(((double)z[k0 + i] - m) / t) : 0.0;
      cs += wc[i];
    }
    tok = draw_cached(wc, k0, k1, cs, u[row], s);
  } else {
    const Softmax sm = row_softmax(z, vocab, t, s);
    tok = block_draw([&](int k) { return sm.p(k); }, vocab, u[row], s);
  }
  if (threadIdx.x == 0) tokens[row] = tok;
}

// One drafted block: every slot's keep test at once (one wave per slot, 16 slots at a time),
// then the first slot not kept draws from the residual, or, with every slot kept, the
// verifier's extra row gives the bonus token.
__global__ __launch_bounds__(kAThreads) void accept_sampled_kernel(int max_x, int max_xv, int vocab, double t,
                                                                   const int32_t* x, const int32_t* xv,
                                                                   const float* dl, const float* vl,
                                                                   const int32_t* dtok, const double* ua,
                                                                   const double* ur, int32_t* alen,
                                                                   int32_t* ntok) {
  __shared__ SampleLds<kAThreads> s;
  constexpr int NW = SampleLds<kAThreads>::NW;
  const int inst = blockIdx.x;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nx = min(max(x[inst], 0), max_x), nxv = min(max(xv[inst], 0), max_xv);
  const int nslots = min(nx, nxv);  // a slot needs its verifier row
  for (int i = wv; i < nslots; i += NW) {
    const Softmax pl = wave_softmax(dl + ((int64_t)inst * max_x + i) * vocab, vocab, t);
    const Softmax pf = wave_softmax(vl + ((int64_t)inst * max_xv + i) * vocab, vocab, t);
    if (lane == 0) {
      const int tok = dtok[(int64_t)inst * max_x + i];
      // a token outside the vocabulary is never kept
      s.keep[i] = (tok >= 0 && tok < vocab) ? (ua[(int64_t)inst * max_x + i] * pl.p(tok) < pf.p(tok)) : 0;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int first = nslots;
    for (int i = 0; i < nslots; ++i)
      if (!s.keep[i]) {
        first = i;
        break;
      }
    s.flag = first;
  }
  __syncthreads();
  const int first = s.flag;
  if (first < nslots) {
    const Softmax pl = row_softmax(dl + ((int64_t)inst * max_x + first) * vocab, vocab, t, s);
    const Softmax pf = row_softmax(vl + ((int64_t)inst * max_xv + first) * vocab, vocab, t, s);
    auto resid = [&](int k) { return fmax(pf.p(k) - pl.p(k), 0.0); };
    double r = 0.0;
    for (int k = threadIdx.x; k < vocab; k += kAThreads) r += resid(k);
    r = block_sum(r, s);
    const double u = ur[(int64_t)inst * (max_x + 1) + first];
    const int tok = r > 0.0 ? block_draw(resid, vocab, u, s) : block_draw([&](int k) { return pf.p(k); }, vocab, u, s);
    if (threadIdx.x == 0) {
      alen[inst] = first;
      ntok[inst] = tok;
    }
    return;
  }
  // every slot kept: the bonus token comes from the verifier's extra row, if there is one
  int next = -1;
  if (nxv > nslots && nslots == nx) {
    const Softmax pf = row_softmax(vl + ((int64_t)inst * max_xv + nx) * vocab, vocab, t, s);
    next = block_draw([&](int k) { return pf.p(k); }, vocab, ur[(int64_t)inst * (max_x + 1) + nx], s);
  }
  if (threadIdx.x == 0) {
    alen[inst] = nslots;
    ntok[inst] = next;
  }
}

}  // namespace

}  // namespace vc

using namespace vc;

extern "C" {

int vc_sample_tokens(int rows, int vocab, float temperature, const float* logits, const double* u,
                     int32_t* tokens, void* stream) {
  set_error("");
  if (rows < 0) return fail(VC_EINVAL, "rows must be >= 0");
  if (rows == 0) return VC_OK;
  if (vocab < 1) return fail(VC_EINVAL, "vocab must be >= 1");
  if (!(temperature > 0.f) || !isfinite(temperature)) return fail(VC_EINVAL, "temperature must be finite and > 0");
  if (!logits || !u || !tokens) return fail(VC_EINVAL, "NULL argument");
  hipLaunchKernelGGL(sample_kernel, dim3(rows), dim3(kSThreads), 0, static_cast<hipStream_t>(stream), vocab,
                     (double)temperature, logits, u, tokens);
  return hip_check(hipGetLastError(), "sample launch");
}

int vc_accept_sampled(int n_inst, int max_x, int max_xv, int vocab, float temperature, const int32_t* x,
                      const int32_t* xv, const float* draft_logits, const float* verify_logits,
                      const int32_t* draft_tok, const double* u_accept, const double* u_resample,
                      int32_t* accept_len, int32_t* next_tok, void* stream) {
  set_error("");
  if (n_inst < 0) return fail(VC_EINVAL, "n_inst must be >= 0");
  if (n_inst == 0) return VC_OK;
  if (max_x < 1 || max_x > VC_MAX_ROWS) return fail(VC_EINVAL, "max_x must be in [1, 64]");
  if (max_xv < 1 || max_xv > VC_MAX_ROWS + 1) return fail(VC_EINVAL, "max_xv must be in [1, 65]");
  if (vocab < 1) return fail(VC_EINVAL, "vocab must be >= 1");
  if (!(temperature > 0.f) || !isfinite(temperature)) return fail(VC_EINVAL, "temperature must be finite and > 0");
  if (!x || !xv || !draft_logits || !verify_logits || !draft_tok || !u_accept || !u_resample || !accept_len ||
      !next_tok)
    return fail(VC_EINVAL, "NULL argument");
  hipLaunchKernelGGL(accept_sampled_kernel, dim3(n_inst), dim3(kAThreads), 0, static_cast<hipStream_t>(stream),
                     max_x, max_xv, vocab, (double)temperature, x, xv, draft_logits, verify_logits, draft_tok,
                     u_accept, u_resample, accept_len, next_tok);
  return hip_check(hipGetLastError(), "sampled accept launch");
}

}  // extern "C"
