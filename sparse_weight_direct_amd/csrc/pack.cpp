// Host side of packing: geometry, launch plan, and the wavefront schedule.
//
// The schedule answers obstacle (2) of Tuteja et al., Sec. 1 (output channels with very
// different non-zero counts leave processing elements idle; their Sec. 5.2 mapping is
// balanced only when channels are similarly sparse): output channels are dealt to
// wavefront slots largest-first so that, chunk by chunk, every wavefront of a workgroup
// carries about the same number of non-zeros whatever the per-channel density.
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
  g->HYp = (int)((hp + st - 1) / st);
  g->Rr = (R - 1) / st + 1;
  g->wide = (st == 1 && W % 4 == 0 && pad <= 2) ? 1 : 0;
  if (const char* e = std::getenv("SPARSECONV_PLAN"))
    if (std::strstr(e, "NARROW")) g->wide = 0;  // tuning only
  g->xoff = g->wide ? 4 : pad;
  g->cshift = g->xoff - pad;
  g->Pp = g->wide ? W + 4 : (int)((wp + st - 1) / st);
  return true;
}

// Phase-plane words a tile of 64*K extended positions reads: the tile plus the reach of
// the filter below and to the right of it.
int plan_pl(const Geom& g, int K) { return 64 * K + (g.Rr - 1) * g.Pp + (g.S - 1) / g.st; }

static int env_int(const char* s, const char* key, int dflt) {
  if (!s) return dflt;
  const char* p = std::strstr(s, key);
  if (!p) return dflt;
  p += std::strlen(key);
  if (*p != '=') return dflt;
  return std::atoi(p + 1);
}

// Deal rows to (group, wavefront, slot).  The kernel synchronises the wavefronts of a
// workgroup once per chunk, so a step lasts as long as its busiest wavefront: each row is
// described by its per-chunk entry counts (padded to even, as stored) and rows are dealt
// largest first to the wavefront with a free slot that least increases the sum over chunks
// of the busiest wavefront's count (ties: the smaller total, then the lower index).  With
// several groups, rows are first dealt to groups largest-first onto the least-loaded group
// with room.  Empty rows weigh 1 so that they are spread too.
static std::vector<int32_t> schedule_rows(const Geom& g, const Plan& p, const std::vector<int32_t>& rowptr,
                                          const std::vector<int32_t>& col, int32_t* max_wave_nnz) {
  const int M = g.M, NW = p.NW, OCW = p.OCW, G = p.G, nch = p.nch, RS = g.R * g.S;
  std::vector<int32_t> vec((size_t)M * nch, 0);
  std::vector<long long> tot(M, 1);
  for (int m = 0; m < M; m++) {
    int32_t* v = &vec[(size_t)m * nch];
    for (int j = rowptr[m]; j < rowptr[m + 1]; j++) v[(col[j] / RS) / p.Cc]++;
    for (int k = 0; k < nch; k++) {
      v[k] = (v[k] + 1) & ~1;
      tot[m] += v[k];
    }
  }
  std::vector<int> order(M);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return tot[a] > tot[b]; });
  // rows -> groups
  std::vector<std::vector<int>> grp(G);
  {
    std::vector<long long> gl(G, 0);
    for (int m : order) {
      int best = -1;
      for (int q = 0; q < G; q++)
        if ((int)grp[q].size() < NW * OCW && (best < 0 || gl[q] < gl[best])) best = q;
      grp[best].push_back(m);  // stays in largest-first order
      gl[best] += tot[m];
    }
  }
  std::vector<int32_t> slot_row((size_t)G * NW * OCW, -1);
  long long mwn = 0;
  std::vector<long long> load((size_t)NW * nch), wt(NW);
  std::vector<long long> gmax(nch);
  std::vector<int> cnt(NW);
  for (int q = 0; q < G; q++) {
    std::fill(load.begin(), load.end(), 0);
    std::fill(wt.begin(), wt.end(), 0);
    std::fill(gmax.begin(), gmax.end(), 0);
    std::fill(cnt.begin(), cnt.end(), 0);
    for (int m : grp[q]) {
      const int32_t* v = &vec[(size_t)m * nch];
      int best = -1;
      long long bcost = 0;
      for (int w = 0; w < NW; w++) {
        if (cnt[w] >= OCW) continue;
        long long cost = 0;
        for (int k = 0; k < nch; k++) cost += std::max(gmax[k], load[(size_t)w * nch + k] + v[k]);
        if (best < 0 || cost < bcost || (cost == bcost && wt[w] < wt[best])) {
          best = w;
          bcost = cost;
        }
      }
      for (int k = 0; k < nch; k++) {
        long long& l = load[(size_t)best * nch + k];
        l += v[k];
        gmax[k] = std::max(gmax[k], l);
      }
      wt[best] += tot[m];
      slot_row[((size_t)q * NW + best) * OCW + cnt[best]] = m;
      cnt[best]++;
    }
    for (int w = 0; w < NW; w++) {
      long long nz = 0;
      for (int o = 0; o < OCW; o++) {
        const int m = slot_row[((size_t)q * NW + w) * OCW + o];
        if (m >= 0) nz += rowptr[m + 1] - rowptr[m];
      }
      mwn = std::max(mwn, nz);
    }
  }
  *max_wave_nnz = (int32_t)mwn;
  return slot_row;
}

int block_header(int OCW) { return (OCW + 1) & ~1; }

// Input layout for K positions per lane with D ring slots whose non-zero part takes
// QE loads per wavefront: the largest chunk that fits the LDS beside the block-start table
// and keeps QE + QR loads per wavefront per step within what the counted wait can express
// (vmcnt <= 63 covers the D-2 later steps in flight).  Chunks are then evened out:
// nch = ceil(C / Cc_max) chunks of about C / nch channels.
static bool fill_layout(const Geom& g, int K, int D, int QE, int cc_cap, Plan* p) {
  const int T = 64 * p->NW;
  p->K = K;
  p->D = D;
  p->QE = QE;
  p->PL = plan_pl(g, K);
  const int align = g.wide ? 256 : 64;
  const long long chs = ((long long)g.st * g.st * p->PL + align - 1) / align * align;
  if (chs > (1 << 24)) return false;
  p->CHS = (int)chs;
  p->nblk = p->CHS / 64;
  const int qmax = D > 2 ? 63 / (D - 2) : 63;
  int nch = 1;
  for (int it = 0; it < 16; it++) {  // the block-start table grows with the chunk count
    const long long table = 4LL * p->G * p->NW * (nch + 1);
    const long long room = (kLdsMax - table) / (4LL * D) - (long long)QE * 4 * T;  // row words per slot
    if (room < p->CHS) return false;
    int cc = (int)std::min<long long>(g.C, room / p->CHS);
    if (cc_cap > 0) cc = std::min(cc, cc_cap);
    // the 4-byte count bounds both (it is used when the wide layout meets a misaligned input)
    while (cc > 0 && QE + (p->nblk * cc + p->NW - 1) / p->NW > qmax) cc--;
    if (cc < 1) return false;
    const int n2 = (g.C + cc - 1) / cc;
    if (n2 <= nch) break;
    nch = n2;
  }
  p->Cc = (g.C + nch - 1) / nch;
  p->nch = (g.C + p->Cc - 1) / p->Cc;  // every chunk non-empty
  p->QR1 = (p->nblk * p->Cc + p->NW - 1) / p->NW;
  p->QR = g.wide ? (p->nblk / 4 * p->Cc + p->NW - 1) / p->NW : p->QR1;
  p->QB = p->QE + p->QR;
  p->nin = p->Cc * p->CHS;
  p->slot_words = p->nin + QE * 4 * T;
  return true;
}

// Largest block one wavefront gets for one chunk: header entries (OCW rounded up to even)
// plus each slot's non-zeros of the chunk rounded up to even.
// Also returns (step_permille) the cost of the per-chunk synchronisation: 1000 * the sum
// over groups and chunks of the busiest wavefront's entries over the sum of the means.
static int max_block(const Geom& g, const Plan& p, const std::vector<int32_t>& rowptr,
                     const std::vector<int32_t>& col, const std::vector<int32_t>& slot_row,
                     int32_t* step_permille = nullptr) {
  const int RS = g.R * g.S;
  std::vector<int> cnt(p.nch), tot(p.nch);
  std::vector<long long> kmax((size_t)p.G * p.nch, 0), ksum((size_t)p.G * p.nch, 0);
  int best = 0;
  for (size_t wv = 0; wv < slot_row.size() / p.OCW; wv++) {
    const size_t q = wv / p.NW;
    std::fill(tot.begin(), tot.end(), 0);
    for (int o = 0; o < p.OCW; o++) {
      const int m = slot_row[wv * p.OCW + o];
      if (m < 0) continue;
      std::fill(cnt.begin(), cnt.end(), 0);
      for (int j = rowptr[m]; j < rowptr[m + 1]; j++) cnt[(col[j] / RS) / p.Cc]++;
      for (int k = 0; k < p.nch; k++) tot[k] += (cnt[k] + 1) & ~1;
    }
    for (int k = 0; k < p.nch; k++) {
      best = std::max(best, block_header(p.OCW) + tot[k]);
      kmax[q * p.nch + k] = std::max<long long>(kmax[q * p.nch + k], tot[k]);
      ksum[q * p.nch + k] += tot[k];
    }
  }
  if (step_permille) {
    long long mx = 0, sm = 0;
    for (size_t i = 0; i < kmax.size(); i++) {
      mx += kmax[i];
      sm += ksum[i];
    }
    *step_permille = sm > 0 ? (int32_t)(1000.0 * (double)mx * p.NW / (double)sm + 0.5) : 1000;
  }
  return best;
}

// Launch plan.  K (positions per lane) trades staging overhead (the filter's reach past
// the tile) against the number of work units; OCW (channel slots per wavefront) is the
// smallest power of two that lets one workgroup hold all output channels, capped at 8,
// and G work units share a tile when M needs more slots.  D ring slots (2 by default: one
// chunk in flight while one is computed) share the CU's LDS; large chunks mean few steps
// and few per-step synchronisations.  QE is the smallest number of 128-entry loads that holds every
// wavefront's block of non-zeros for one chunk.
// SPARSECONV_PLAN="K=..,OCW=..,NW=..,D=..,CC=.." overrides the choice (tuning only).
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
  int D = env_int(env, "D", 2);
  const int issue_late = env_int(env, "LATE", 0);
  const int cc_cap = env_int(env, "CC", 0);
  if (K != 1 && K != 2 && K != 4 && K != 8 && K != 16) K = 4;
  if (OCW != 1 && OCW != 2 && OCW != 4 && OCW != 8 && OCW != 16) OCW = 8;
  if (NW != 8 && NW != 16) NW = 16;
  if (D < 2 || D > 4) D = 2;
  while (OCW * K > 64 && K > 1) K /= 2;
  p.NW = NW;
  for (int ocw = OCW; ocw >= 1; ocw /= 2) {
    p.issue_late = issue_late != 0 ? 1 : 0;
    p.OCW = ocw;
    p.G = (g.M + NW * ocw - 1) / (NW * ocw);
    for (int k = K; k >= 1; k /= 2) {
      bool ok = false;
      int32_t mwn = 0;
      std::vector<int32_t> sr;
      for (int qe = 1; qe <= 63 && !ok; qe++) {
        if (!fill_layout(g, k, D, qe, cc_cap, &p)) break;
        sr = schedule_rows(g, p, rowptr, col, &mwn);
        if (max_block(g, p, rowptr, col, sr, &p.step_permille) <= 128 * qe) ok = true;
      }
      if (!ok) continue;
      const int table = p.G * NW * (p.nch + 1);
      p.lds_bytes = 4 * p.D * p.slot_words + 4 * table;
      if (p.lds_bytes > kLdsMax) continue;
      p.span_images = (int)((p.PL + img_ext - 2) / img_ext + 1);
      if (slot_row) *slot_row = sr;
      if (max_wave_nnz) *max_wave_nnz = mwn;
      return p;
    }
  }
  p.K = 0;  // does not fit: caller reports SC_EUNSUPPORTED
  return p;
}

}  // namespace sc
