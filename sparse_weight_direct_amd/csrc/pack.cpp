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

// Deal rows to (group, wavefront, slot), largest first onto the least-loaded wavefront with
// a free slot (weights nnz + 1 so empty rows are spread too).
static std::vector<int32_t> schedule_rows(int M, int waves, int OCW, const std::vector<int32_t>& rowptr,
                                          int32_t* max_wave_nnz) {
  std::vector<int> order(M);
  std::iota(order.begin(), order.end(), 0);
  auto nnz_of = [&](int m) { return rowptr[m + 1] - rowptr[m]; };
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return nnz_of(a) > nnz_of(b); });
  std::vector<long long> load(waves, 0), nz(waves, 0);
  std::vector<int> cnt(waves, 0);
  std::vector<int32_t> slot_row((size_t)waves * OCW, -1);
  for (int m : order) {
    int best = -1;
    for (int w = 0; w < waves; w++)
      if (cnt[w] < OCW && (best < 0 || load[w] < load[best])) best = w;
    slot_row[(size_t)best * OCW + cnt[best]] = m;
    cnt[best]++;
    load[best] += nnz_of(m) + 1;
    nz[best] += nnz_of(m);
  }
  *max_wave_nnz = (int32_t)*std::max_element(nz.begin(), nz.end());
  return slot_row;
}

int block_header(int OCW) { return (OCW + 1) & ~1; }

// Input layout for K positions per lane: the channel stride and the largest chunk whose
// two ring slots (input rows plus `ent_words` of non-zeros each) fit in `lds_free` bytes.
// Chunks are then evened out: nch = ceil(C / Cc_max) chunks of ceil(C / nch) channels.
static bool fill_layout(const Geom& g, int K, int ent_words, int lds_free, int cc_cap, Plan* p) {
  p->K = K;
  p->NRmax = plan_nrmax(g, K);
  p->PH = p->NRmax * g.Pp;
  p->CHS = (g.st * g.st * p->PH + 63) / 64 * 64;
  p->nblk = p->CHS / 64;
  const int slack = 64;  // junk positions read at most (S-1)/st + 1 words past a plane
  if ((g.S - 1) / g.st + 1 > slack) return false;
  const long long room = (long long)lds_free / 8 - ent_words - slack;  // words per slot for rows
  if (room < p->CHS) return false;
  int cc = (int)std::min<long long>(g.C, room / p->CHS);
  if (cc_cap > 0) cc = std::min(cc, cc_cap);
  const int nch = (g.C + cc - 1) / cc;
  p->Cc = (g.C + nch - 1) / nch;
  p->nch = (g.C + p->Cc - 1) / p->Cc;  // every chunk non-empty
  p->nin = p->Cc * p->CHS + slack;
  return true;
}

// Largest block one wavefront gets for one chunk: header entries (OCW rounded up to even)
// plus each slot's non-zeros of the chunk rounded up to even.
static int max_block(const Geom& g, const Plan& p, const std::vector<int32_t>& rowptr,
                     const std::vector<int32_t>& col, const std::vector<int32_t>& slot_row) {
  const int RS = g.R * g.S;
  std::vector<int> cnt(p.nch), tot(p.nch);
  int best = 0;
  for (size_t wv = 0; wv < slot_row.size() / p.OCW; wv++) {
    std::fill(tot.begin(), tot.end(), 0);
    for (int o = 0; o < p.OCW; o++) {
      const int m = slot_row[wv * p.OCW + o];
      if (m < 0) continue;
      std::fill(cnt.begin(), cnt.end(), 0);
      for (int j = rowptr[m]; j < rowptr[m + 1]; j++) cnt[(col[j] / RS) / p.Cc]++;
      for (int k = 0; k < p.nch; k++) tot[k] += (cnt[k] + 1) & ~1;
    }
    for (int k = 0; k < p.nch; k++) best = std::max(best, block_header(p.OCW) + tot[k]);
  }
  return best;
}

// Launch plan.  K (positions per lane) trades staging overhead (halo rows per position)
// against the number of work units; OCW (channel slots per wavefront) is the smallest
// power of two that lets one workgroup hold all output channels, capped at 8, and G work
// units share a tile when M needs more slots.  The two ring slots take the CU's LDS: large
// chunks mean few steps, and the per-step and per-run bookkeeping runs on the scalar unit,
// which all wavefronts of a CU share.  QE is the smallest number of 32-entry loads that
// holds every wavefront's block of non-zeros for one chunk.
// SPARSECONV_PLAN="K=..,OCW=..,NW=..,CC=.." overrides the choice (tuning only).
Plan choose_plan(const Geom& g, const std::vector<int32_t>& rowptr, const std::vector<int32_t>& col,
                 std::vector<int32_t>* slot_row, int32_t* max_wave_nnz) {
  Plan p{};
  const long long img_ext = (long long)g.HYp * g.Pp;
  int K = img_ext >= 4096 ? 8 : img_ext >= 1024 ? 4 : img_ext >= 256 ? 2 : 1;
  int NW = 16;
  int OCW = 1;
  while (OCW < 8 && OCW * NW < g.M) OCW *= 2;
  const char* env = std::getenv("SPARSECONV_PLAN");
  K = env_int(env, "K", K);
  NW = env_int(env, "NW", NW);
  OCW = env_int(env, "OCW", OCW);
  const int cc_cap = env_int(env, "CC", 0);
  if (K != 1 && K != 2 && K != 4 && K != 8 && K != 16) K = 4;
  if (OCW != 1 && OCW != 2 && OCW != 4 && OCW != 8 && OCW != 16) OCW = 8;
  if (NW != 8 && NW != 16) NW = 16;
  while (OCW * K > 64 && K > 1) K /= 2;
  const int T = 64 * NW;
  p.NW = NW;
  for (int ocw = OCW; ocw >= 1; ocw /= 2) {
    p.OCW = ocw;
    p.G = (g.M + NW * ocw - 1) / (NW * ocw);
    int32_t mwn = 0;
    std::vector<int32_t> sr = schedule_rows(g.M, p.G * NW, ocw, rowptr, &mwn);
    for (int k = K; k >= 1; k /= 2) {
      p.rt = (g.st * plan_nrmax(g, k) + 63) / 64 * 64;
      const int fixed = 4 * NW * p.rt + 4 * p.G * NW * (g.C + 1) + 256;  // tables, upper bound
      bool ok = false;
      for (int qe = 1; qe <= 64 && !ok; qe++) {
        if (!fill_layout(g, k, qe * T, kLdsMax - fixed, cc_cap, &p)) break;
        if (max_block(g, p, rowptr, col, sr) <= 32 * qe) {
          p.QE = qe;
          ok = true;
        }
      }
      if (!ok) continue;
      p.slot_words = p.nin + p.QE * T;
      const int table = p.G * NW * (p.nch + 1);
      p.lds_bytes = 2 * 4 * p.slot_words + 4 * NW * p.rt + 4 * table;
      if (p.lds_bytes > kLdsMax) continue;
      p.span_images = (p.NRmax + g.HYp - 2) / g.HYp + 1;
      if (slot_row) *slot_row = sr;
      if (max_wave_nnz) *max_wave_nnz = mwn;
      return p;
    }
  }
  p.K = 0;  // does not fit: caller reports SC_EUNSUPPORTED
  return p;
}

}  // namespace sc
