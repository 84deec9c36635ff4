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

// Deal rows to (group, consumer wavefront, slot).  A workgroup's consumers share each
// chunk's ring slot, so a step is released only when its busiest consumer is done: each row is
// described by its per-chunk entry counts (padded to even, as stored) and rows are dealt
// largest first to the wavefront with a free slot that least increases the sum over chunks
// of the busiest wavefront's count (ties: the smaller total, then the lower index).  With
// several groups, rows are first dealt to groups largest-first onto the least-loaded group
// with room.  Empty rows weigh 1 so that they are spread too.
static std::vector<int32_t> schedule_rows(const Geom& g, const Plan& p, const std::vector<int32_t>& rowptr,
                                          const std::vector<int32_t>& col, int32_t* max_wave_nnz) {
  const int M = g.M, NC = p.NW - 1, OCW = p.OCW, G = p.G, nch = p.nch, RS = g.R * g.S;
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
        if ((int)grp[q].size() < NC * OCW && (best < 0 || gl[q] < gl[best])) best = q;
      grp[best].push_back(m);  // stays in largest-first order
      gl[best] += tot[m];
    }
  }
  std::vector<int32_t> slot_row((size_t)G * NC * OCW, -1);
  long long mwn = 0;
  std::vector<long long> load((size_t)NC * nch), wt(NC);
  std::vector<long long> gmax(nch);
  std::vector<int> cnt(NC);
  for (int q = 0; q < G; q++) {
    std::fill(load.begin(), load.end(), 0);
    std::fill(wt.begin(), wt.end(), 0);
    std::fill(gmax.begin(), gmax.end(), 0);
    std::fill(cnt.begin(), cnt.end(), 0);
    for (int m : grp[q]) {
      const int32_t* v = &vec[(size_t)m * nch];
      int best = -1;
      long long bcost = 0;
      for (int w = 0; w < NC; w++) {
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
      slot_row[((size_t)q * NC + best) * OCW + cnt[best]] = m;
      cnt[best]++;
    }
    for (int w = 0; w < NC; w++) {
      long long nz = 0;
      for (int o = 0; o < OCW; o++) {
        const int m = slot_row[((size_t)q * NC + w) * OCW + o];
        if (m >= 0) nz += rowptr[m + 1] - rowptr[m];
      }
      mwn = std::max(mwn, nz);
    }
  }
  *max_wave_nnz = (int32_t)mwn;
  return slot_row;
}

int block_header(int OCW) { return (OCW + 1) & ~1; }

// Input layout for K positions per lane with D ring slots whose non-zero part takes QE
// loads per consumer: the largest chunk that fits the LDS beside the counters and the
// block-start table.  Chunks are then evened out: nch = ceil(C / Cc_max) chunks of about
// C / nch channels.
static bool fill_layout(const Geom& g, int K, int D, int QE, int cc_cap, int lds_max, Plan* p) {
  const int NC = p->NW - 1;
  p->K = K;
  p->D = D;
  p->QE = QE;
  p->PL = plan_pl(g, K);
  const int align = g.wide ? 256 : 64;
  const long long chs = ((long long)g.st * g.st * p->PL + align - 1) / align * align;
  if (chs > (1 << 24)) return false;
  p->CHS = (int)chs;
  p->nblk = p->CHS / 64;
  int nch = 1;
  for (int it = 0; it < 16; it++) {  // the block-start table grows with the chunk count
    const long long fixed = 4LL * p->G * NC * (nch + 1) + 8LL * kMaxDepth;
    const long long room = (lds_max - fixed) / (4LL * D) - (long long)QE * 256 * NC;  // row words per slot
    if (room < p->CHS) return false;
    int cc = (int)std::min<long long>(g.C, room / p->CHS);
    if (cc_cap > 0) cc = std::min(cc, cc_cap);
    const int n2 = (g.C + cc - 1) / cc;
    if (n2 <= nch) break;
    nch = n2;
  }
  p->Cc = (g.C + nch - 1) / nch;
  p->nch = (g.C + p->Cc - 1) / p->Cc;  // every chunk non-empty
  p->nin = p->Cc * p->CHS;
  p->slot_words = p->nin + QE * 256 * NC;
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
    const size_t q = wv / (p.NW - 1);
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
    *step_permille = sm > 0 ? (int32_t)(1000.0 * (double)mx * (p.NW - 1) / (double)sm + 0.5) : 1000;
  }
  return best;
}

// Launch plan.  A workgroup has NW = 16 wavefronts: NC = 15 consumers with OCW output-
// channel slots each and one producer.  OCW is the smallest instantiated count (1, 2, 3, 5,
// 9) that lets one workgroup hold all output channels, else 9 with G groups of channels per
// tile.  K (positions per lane) trades staging overhead (the filter's reach past the
// tile) against the number of work units: the largest instantiated K with OCW*K <= 64
// accumulators, capped by the image size.  D ring slots (3 by default: a consumer may run
// a step ahead of the slowest) share the CU's LDS with the counters and the block-start
// table; large chunks mean few steps.  QE is the smallest number of 128-entry loads that
// holds every consumer's block of non-zeros for one chunk.
// SPARSECONV_PLAN="K=..,OCW=..,D=..,CC=..,LDSKB=..,NARROW" overrides the choice (tuning only).
static bool instantiated(int K, int OCW) {
  static const int kk[] = {1, 2, 4, 6, 7, 8, 12, 16};
  static const int oo[] = {1, 2, 3, 5, 9};
  bool okk = false, oko = false;
  for (int v : kk) okk = okk || v == K;
  for (int v : oo) oko = oko || v == OCW;
  return okk && oko && K * OCW <= 64;
}

Plan choose_plan(const Geom& g, const std::vector<int32_t>& rowptr, const std::vector<int32_t>& col,
                 std::vector<int32_t>* slot_row, int32_t* max_wave_nnz) {
  static const int kOcw[] = {1, 2, 3, 5, 9};
  static const int kKs[] = {16, 12, 8, 7, 6, 4, 2, 1};
  Plan p{};
  p.NW = 16;
  const int NC = p.NW - 1;
  const long long img_ext = (long long)g.HYp * g.Pp;
  const int kmax = img_ext >= 4096 ? 8 : img_ext >= 1024 ? 4 : img_ext >= 256 ? 2 : 1;
  int OCW = 9;
  for (int o : kOcw)
    if (NC * o >= g.M) {
      OCW = o;
      break;
    }
  const char* env = std::getenv("SPARSECONV_PLAN");
  OCW = env_int(env, "OCW", OCW);
  const int kenv = env_int(env, "K", 0);
  int D = env_int(env, "D", 3);
  const int cc_cap = env_int(env, "CC", 0);
  const int lds_max = std::min(kLdsMax, 1024 * env_int(env, "LDSKB", kLdsMax / 1024));
  if (D < 2 || D > kMaxDepth) D = 3;
  bool oko = false;
  for (int o : kOcw) oko = oko || o == OCW;
  if (!oko) OCW = 9;
  // fewer slots per consumer (more groups) when the blocks of non-zeros do not fit
  for (int oi = 4; oi >= 0; oi--) {
    if (kOcw[oi] > OCW) continue;
    p.OCW = kOcw[oi];
    p.G = (g.M + NC * p.OCW - 1) / (NC * p.OCW);
    for (int k : kKs) {
      if (!instantiated(k, p.OCW)) continue;
      if (kenv > 0 ? k > kenv : k > kmax) continue;
      bool ok = false;
      int32_t mwn = 0;
      std::vector<int32_t> sr;
      for (int qe = 1; qe <= 64 && !ok; qe++) {
        if (!fill_layout(g, k, D, qe, cc_cap, lds_max, &p)) break;
        sr = schedule_rows(g, p, rowptr, col, &mwn);
        if (max_block(g, p, rowptr, col, sr, &p.step_permille) <= 128 * qe) ok = true;
      }
      if (!ok) continue;
      const int table = p.G * NC * (p.nch + 1);
      p.lds_bytes = 4 * p.D * p.slot_words + 8 * kMaxDepth + 4 * table;
      if (p.lds_bytes > lds_max) continue;
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
