// Admit scheduler with a link (BW) ring and an HBM ring (host code only).
//
// VeriCache review, §Runtime Algorithm Deep Dive: a sliding window of W future iterations; the
// BW ring holds the host-link time reserved for reloads in each window (at most T_iter per
// window, the link being serial), the HBM ring the full caches occupying HBM in each window (at
// most the HBM left after weights and resident caches).  Admit(r) gives request r's full-cache
// reload a span of S_r = max(1, ceil(l_r)) windows, l_r = KV_full / (BW * T_iter), ending at its
// verify iteration d; d is searched outward from the target draft length x (x, x+1, x-1, x+2,
// ...), clamped to [S_r, W-1], and the first d whose span fits both rings is reserved.
//
// Readings: a reload's link time is spread evenly over its span (KV_full / (BW * S_r) per
// window, at most T_iter since S_r >= l_r); its whole KV_full is counted in HBM for every window
// of the span (bytes arrive over the span and stay until the verify ends).  Window indexes are
// relative to the current iteration; vc_sched_advance slides the window by one.
#include <math.h>

#include <deque>
#include <map>
#include <vector>

#include "vc_internal.h"

namespace vc {

namespace {

struct Reservation {
  int64_t verify_iter;  // absolute iteration of the verify
  int32_t span;         // S_r
};

struct Sched {
  vc_sched_cfg cfg;
  int64_t now = 0;
  std::deque<double> link;   // per window from now: reserved link seconds
  std::deque<double> hbm;    // per window from now: reserved bytes
  std::map<int32_t, Reservation> res;
};

}  // namespace

}  // namespace vc

using namespace vc;

extern "C" {

int vc_sched_create(const vc_sched_cfg* cfg, void** sched) {
  set_error("");
  if (!cfg || !sched) return fail(VC_EINVAL, "NULL argument");
  *sched = nullptr;
  if (cfg->window < 2 || cfg->window > (1 << 20)) return fail(VC_EINVAL, "window must be in [2, 2^20]");
  if (cfg->draft_len < 1) return fail(VC_EINVAL, "draft_len must be >= 1");
  if (!(cfg->t_iter > 0) || !(cfg->link_bw > 0) || !(cfg->hbm_budget >= 0) || !isfinite(cfg->t_iter) ||
      !isfinite(cfg->link_bw) || !isfinite(cfg->hbm_budget))
    return fail(VC_EINVAL, "t_iter and link_bw must be > 0, hbm_budget >= 0, all finite");
  Sched* s = new Sched;
  s->cfg = *cfg;
  s->link.assign(cfg->window, 0.0);
  s->hbm.assign(cfg->window, 0.0);
  *sched = s;
  return VC_OK;
}

void vc_sched_destroy(void* sched) { delete static_cast<Sched*>(sched); }

int vc_sched_admit(void* sched, int32_t req, double kv_full_bytes, int64_t* verify_iter) {
  set_error("");
  if (!sched || !verify_iter) return fail(VC_EINVAL, "NULL argument");
  if (!(kv_full_bytes >= 0) || !isfinite(kv_full_bytes)) return fail(VC_EINVAL, "kv_full_bytes must be >= 0");
  Sched& s = *static_cast<Sched*>(sched);
  if (s.res.count(req)) return fail(VC_EINVAL, "request already holds a reservation");
  const int W = s.cfg.window;
  const double ell = kv_full_bytes / (s.cfg.link_bw * s.cfg.t_iter);
  const double span_d = fmax(1.0, ceil(ell));
  if (span_d > W - 1) {  // the reload can never fit in the lookahead window
    *verify_iter = -1;
    set_error("reload longer than the lookahead window");
    return VC_EAGAIN;
  }
  const int S = (int)span_d;
  const double per_window = kv_full_bytes / (s.cfg.link_bw * S);
  const int lo = S, hi = W - 1;
  const int anchor = s.cfg.draft_len < lo ? lo : (s.cfg.draft_len > hi ? hi : s.cfg.draft_len);
  // candidates anchor, anchor+1, anchor-1, anchor+2, ... inside [lo, hi]
  for (int k = 0; k <= 2 * (hi - lo) + 1; ++k) {
    const int off = (k + 1) / 2;
    const int d = (k % 2 == 1) ? anchor + off : anchor - off;
    if (d < lo || d > hi) continue;
    bool fits = true;
    for (int i = d - S + 1; i <= d && fits; ++i)
      fits = s.link[i] + per_window <= s.cfg.t_iter && s.hbm[i] + kv_full_bytes <= s.cfg.hbm_budget;
    if (!fits) continue;
    for (int i = d - S + 1; i <= d; ++i) {
      s.link[i] += per_window;
      s.hbm[i] += kv_full_bytes;
    }
    s.res[req] = Reservation{s.now + d, S};
    *verify_iter = s.now + d;
    return VC_OK;
  }
  *verify_iter = -1;
  set_error("no span of the lookahead window fits both rings");
  return VC_EAGAIN;
}

int vc_sched_advance(void* sched) {
  set_error("");
  if (!sched) return fail(VC_EINVAL, "NULL argument");
  Sched& s = *static_cast<Sched*>(sched);
  // reservations whose verify is the iteration now ending are complete
  for (auto it = s.res.begin(); it != s.res.end();)
    it = it->second.verify_iter <= s.now ? s.res.erase(it) : std::next(it);
  s.link.pop_front();
  s.link.push_back(0.0);
  s.hbm.pop_front();
  s.hbm.push_back(0.0);
  ++s.now;
  return VC_OK;
}

int64_t vc_sched_now(const void* sched) { return sched ? static_cast<const Sched*>(sched)->now : -1; }

int vc_sched_ring(const void* sched, int32_t i, double* link_s, double* hbm_bytes) {
  set_error("");
  if (!sched || !link_s || !hbm_bytes) return fail(VC_EINVAL, "NULL argument");
  const Sched& s = *static_cast<const Sched*>(sched);
  if (i < 0 || i >= s.cfg.window) return fail(VC_EINVAL, "window index out of range");
  *link_s = s.link[i];
  *hbm_bytes = s.hbm[i];
  return VC_OK;
}

int vc_sched_due(const void* sched, int32_t cap, int32_t* reload_ids, int32_t* n_reload, int32_t* verify_ids,
                 int32_t* n_verify) {
  set_error("");
  if (!sched || !n_reload || !n_verify || (cap > 0 && (!reload_ids || !verify_ids)))
    return fail(VC_EINVAL, "NULL argument");
  const Sched& s = *static_cast<const Sched*>(sched);
  int nr = 0, nv = 0;
  for (const auto& kv : s.res) {
    const Reservation& r = kv.second;
    if (r.verify_iter - r.span + 1 == s.now) {
      if (nr >= cap) return fail(VC_EINVAL, "cap too small");
      reload_ids[nr++] = kv.first;
    }
    if (r.verify_iter == s.now) {
      if (nv >= cap) return fail(VC_EINVAL, "cap too small");
      verify_ids[nv++] = kv.first;
    }
  }
  *n_reload = nr;
  *n_verify = nv;
  return VC_OK;
}

}  // extern "C"
