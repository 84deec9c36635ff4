// Host side of packing: geometry, launch plan, and the wavefront schedule.
//
// The schedule answers obstacle (2) of Tuteja et al., Sec. 1 (output channels with very
// different non-zero counts leave processing elements idle; their Sec. 5.2 mapping is
// balanced only when channels are similarly sparse): output channels are dealt to
// wavefront slots largest-first, each to the least-loaded wavefront that still has a free
// slot, so every wavefront of a workgroup carries about the same number of non-zeros
// whatever the per-channel density.
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <numeric>

#include "plan.h"

namespace sc {

bool make_geom(int M, int C, int R, int S, int H, int W, int st, int pad, Geom* g) {
  if (M < 1 || C < 1 || R < 1 || S < 1 || H < 1 || W < 1 || st < 1 || pad < 0) return false;
  const long long hp = (long long)H + 2LL * pad, wp = (long long)W + 2LL * pad;
  if (hp < R || wp < S) return false;
  g->M = M; g->C = C; g->R = R; g->S = S; g->H = H; g->W = W; g->st = st; g->pad = pad;
  g->E = (int)((hp - R) / st + 1);
  g->F = (int)((wp - S) / st + 1);
  g->Pp = (int)((wp + st - 1) / st);
  g->HYp = (int)((hp + st - 1) / st);
  g->Rr = (R - 1) / st + 1;
  return true;
}

// Phase rows touched by a run of 64*K extended positions starting anywhere in a row, plus
// the rows the filter reaches below them.
int plan_nrmax(const Geom& g, int K) { return (g.Pp + 64 * K - 2) / g.Pp + g.Rr; }

static int env_int(const char* s, const char* key, int dflt) {
  if (!s) return dflt;
  const char* p = std::strstr(s, key);
  if (!p) return dflt;
  p += std::strlen(key);
  if (*p != '=') return dflt;
  return std::atoi(p + 1);
}

static bool fill_layout(const Geom& g, int K, int budget, int cc_cap, Plan* p) {
  p->K = K;
  p->NRmax = plan_nrmax(g, K);
  p->PH = p->NRmax * g.Pp;
  p->CHS = g.st * g.st * p->PH;
  const int tail = ((g.S - 1) / g.st + 1 + 3) & ~3;  // junk positions may read this far past
  const int fixed = 4 * tail + 4 * g.st * p->NRmax;
  if ((long long)fixed + 4LL * p->CHS > budget) return false;
  p->Cc = std::min<long long>(g.C, (budget - fixed) / (4LL * p->CHS));
  if (cc_cap > 0) p->Cc = std::min(p->Cc, cc_cap);
  p->nch = (g.C + p->Cc - 1) / p->Cc;
  p->lds_floats = p->Cc * p->CHS + tail;
  p->lds_bytes = 4 * p->lds_floats + 4 * g.st * p->NRmax;
  return true;
}

// Launch plan.  K (positions per lane) trades staging overhead (halo rows per position)
// against the number of workgroups; OCW (channel slots per wavefront) is the smallest
// power of two that lets one workgroup hold all output channels, capped at 16, and G
// workgroups share a tile when M needs more slots.  SPARSECONV_PLAN="K=..,OCW=..,CC=.."
// overrides the choice (tuning only).
Plan choose_plan(const Geom& g, const std::vector<int32_t>& row_nnz) {
  (void)row_nnz;
  Plan p{};
  const long long img_ext = (long long)g.HYp * g.Pp;
  int K = img_ext >= 4096 ? 4 : img_ext >= 1024 ? 2 : 1;
  int OCW = 1;
  while (OCW < 16 && OCW * kWaves < g.M) OCW *= 2;
  const char* env = std::getenv("SPARSECONV_PLAN");
  K = env_int(env, "K", K);
  OCW = env_int(env, "OCW", OCW);
  const int cc_cap = env_int(env, "CC", 0);
  if (K != 1 && K != 2 && K != 4 && K != 8) K = 4;
  if (OCW != 1 && OCW != 2 && OCW != 4 && OCW != 8 && OCW != 16) OCW = 16;
  while (OCW * K > 128 && K > 1) K /= 2;
  p.OCW = OCW;
  p.G = (g.M + kWaves * OCW - 1) / (kWaves * OCW);
  // Prefer the 64 KB budget (two workgroups per CU); fall back to smaller K, then to the
  // whole 160 KB of LDS for very wide rows.
  for (int budget : {kLdsBudget, 160 * 1024}) {
    for (int k = K; k >= 1; k /= 2)
      if (fill_layout(g, k, budget, cc_cap, &p)) return p;
  }
  p.K = 0;  // does not fit: caller reports SC_EUNSUPPORTED
  return p;
}

}  // namespace sc
