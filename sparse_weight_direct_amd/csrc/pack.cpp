// Host side of packing: geometry, launch plan, and the wavefront schedule.
//
// The schedule answers obstacle (2) of Tuteja et al., Sec. 1 (output channels with very
// different non-zero counts leave processing elements idle; their Sec. 5.2 mapping is
// balanced only when channels are similarly sparse): output channels are dealt to
// wavefront slots largest-first so that, chunk by chunk, every wavefront of a workgroup
// carries about the same number of non-zeros whatever the per-channel density.
#include <algorithm>
#include <cmath>
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
  // wide layout: input column x at phase column x + 4 in rows of W + 4 words, output column f
  // at extended column f + 4 - pad.  The last output column F - 1 = W + 2 pad - S fits in the
  // row only if pad < S, and the right padding wraps into the next row's 4 zero columns only
  // if pad <= 2 (pad <= 4 would do; 2 keeps the halo small)
  g->wide = (st == 1 && W % 4 == 0 && pad <= 2 && pad < S) ? 1 : 0;
  if (const char* e = std::getenv("SPARSECONV_PLAN"))
    if (std::strstr(e, "NARROW")) g->wide = 0;  // tuning only
  g->xoff = g->wide ? 4 : pad;
  g->cshift = g->xoff - pad;
  g->Pp = g->wide ? W + 4 : (int)((wp + st - 1) / st);
  return true;
}

// Phase-plane words a tile of 64*K extended positions reads: the tile plus the reach of
// the filter below and to the right of it.  A quad tile (504 positions) reads 508 words
// plus the reach: lane 63's second quad, whose words only feed lane 62, ends at word 507.
int plan_pl(const Geom& g, int K, int quad) {
  return (quad ? kQuadTile + 4 : 64 * K) + (g.Rr - 1) * g.Pp + (g.S - 1) / g.st;
}

static int env_int(const char* s, const char* key, int dflt) {
  if (!s) return dflt;
  const char* p = std::strstr(s, key);
  if (!p) return dflt;
  p += std::strlen(key);
  if (*p != '=') return dflt;
  return std::atoi(p + 1);
}

// Deal rows to (group, consumer wavefront, slot).  A workgroup's consumers share each
// chunk's ring slot, so a step is released only when its busiest consumer is done: each
// item (a row, or a piece of a split row) is described by its per-chunk entry counts
// (as stored), and items are dealt largest first to the consumer with a
// free slot that least increases the sum over chunks of the busiest consumer's count
// (ties: the smaller total, then the lower index), preferring consumers that hold no other
// piece of the same row.  A row whose entries exceed a consumer's fair share of the group
// is split into pieces of at most half that share (at most one per consumer, and as many
// as the free slots allow).  Rows are first dealt, with all their pieces, to groups
// largest-first onto the least-loaded group with room.  Empty rows weigh 1 so that they
// are spread too.
static Sched schedule_rows(const Geom& g, const Plan& p, const std::vector<int32_t>& rowptr,
                           const std::vector<int32_t>& col) {
  const int M = g.M, NC = p.NW - 1, OCW = p.OCW, G = p.G, nch = p.nch, RS = g.R * g.S;
  std::vector<int32_t> raw((size_t)M * nch, 0);
  std::vector<long long> tot(M, 1);
  long long total = 0;
  for (int m = 0; m < M; m++) {
    int32_t* v = &raw[(size_t)m * nch];
    for (int j = rowptr[m]; j < rowptr[m + 1]; j++) v[(col[j] / RS) / p.Cc]++;
    for (int k = 0; k < nch; k++) tot[m] += v[k];
    total += tot[m];
  }
  // pieces per row
  const double fair = (double)total / ((double)G * NC);
  std::vector<int> P(M, 1);
  long long pieces = M;
  for (int m = 0; m < M; m++)
    if (rowptr[m + 1] > rowptr[m] && (double)tot[m] > fair) {
      P[m] = std::min<long long>(NC, (long long)std::ceil(2.0 * (double)tot[m] / fair));
      pieces += P[m] - 1;
    }
  const long long slots = (long long)G * NC * OCW;
  while (pieces > slots) {  // not enough slots: take pieces from the most split rows
    int big = 0;
    for (int m = 1; m < M; m++)
      if (P[m] > P[big]) big = m;
    if (P[big] <= 1) break;
    P[big]--;
    pieces--;
  }
  // rows (with all their pieces) -> groups, largest first onto the least-loaded group with
  // room.  A row whose pieces fit no group (the free slots are spread over groups) gets as
  // many pieces as the roomiest group has slots left; the total never exceeds the slots, so
  // one piece always fits.
  std::vector<int> order(M);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return tot[a] > tot[b]; });
  std::vector<int> row_group(M, 0);
  {
    std::vector<long long> gl(G, 0);
    std::vector<int> used(G, 0);
    for (int m : order) {
      int best = -1;
      for (int q = 0; q < G; q++)
        if (used[q] + P[m] <= NC * OCW && (best < 0 || gl[q] < gl[best])) best = q;
      if (best < 0) {
        for (int q = 0; q < G; q++)
          if (best < 0 || used[q] < used[best]) best = q;
        const int fit = std::max(1, NC * OCW - used[best]);
        pieces -= P[m] - fit;
        P[m] = fit;
      }
      row_group[m] = best;
      gl[best] += tot[m];
      used[best] += P[m];
    }
  }
  // items: (row, piece) with their per-chunk counts
  struct Item { int m, p; long long tot; };
  std::vector<Item> items;
  std::vector<int32_t> ivec;
  std::vector<std::vector<int>> grp(G);  // item indices per group
  for (int m = 0; m < M; m++)
    for (int q = 0; q < P[m]; q++) {
      long long t = 1;
      for (int k = 0; k < nch; k++) {
        int pb, pe;
        piece_range(0, raw[(size_t)m * nch + k], q, P[m], &pb, &pe);
        const int n = pe - pb;
        ivec.push_back(n);
        t += n;
      }
      grp[row_group[m]].push_back((int)items.size());
      items.push_back({m, q, t});
    }
  Sched sc;
  sc.slot_row.assign((size_t)G * NC * OCW, -1);
  sc.slot_comb.assign((size_t)G * NC * OCW, 0);
  sc.src_row.assign((size_t)G * NC * OCW, -1);
  sc.piece.assign((size_t)G * NC * OCW, 0);
  sc.npieces.assign((size_t)G * NC * OCW, 1);
  std::vector<long long> load((size_t)NC * nch), wt(NC);
  std::vector<long long> gmax(nch);
  std::vector<int> cnt(NC);
  std::vector<int> holder((size_t)NC * M, 0);  // consumer w holds a piece of row m
  // partial-sum buffers are numbered across all groups: a buffer belongs to one group, so it
  // is used once in every unit of that group (the kernel counts its uses per group)
  int nb = 0;
  for (int q = 0; q < G; q++) {
    std::fill(load.begin(), load.end(), 0);
    std::fill(wt.begin(), wt.end(), 0);
    std::fill(gmax.begin(), gmax.end(), 0);
    std::fill(cnt.begin(), cnt.end(), 0);
    std::vector<int> its = grp[q];
    std::stable_sort(its.begin(), its.end(), [&](int a, int b) { return items[a].tot > items[b].tot; });
    for (int i : its) {
      const Item& it = items[i];
      const int32_t* v = &ivec[(size_t)i * nch];
      int best = -1;
      long long bcost = 0;
      bool bfree = false;
      for (int w = 0; w < NC; w++) {
        if (cnt[w] >= OCW) continue;
        const bool fr = !holder[(size_t)w * M + it.m];
        long long cost = 0;
        for (int k = 0; k < nch; k++) cost += std::max(gmax[k], load[(size_t)w * nch + k] + v[k]);
        if (best < 0 || (fr && !bfree) ||
            (fr == bfree && (cost < bcost || (cost == bcost && wt[w] < wt[best])))) {
          best = w;
          bcost = cost;
          bfree = fr;
        }
      }
      for (int k = 0; k < nch; k++) {
        long long& l = load[(size_t)best * nch + k];
        l += v[k];
        gmax[k] = std::max(gmax[k], l);
      }
      wt[best] += it.tot;
      holder[(size_t)best * M + it.m] = 1;
      const size_t sl = ((size_t)q * NC + best) * OCW + cnt[best];
      sc.src_row[sl] = it.m;
      sc.piece[sl] = it.p;
      sc.npieces[sl] = P[it.m];
      cnt[best]++;
    }
    std::fill(holder.begin(), holder.end(), 0);
    // kernel tables: piece 0 owns the row; later pieces get partial buffers in order
    std::vector<int> first_buf(M, -1);
    for (int w = 0; w < NC; w++)
      for (int o = 0; o < OCW; o++) {
        const size_t sl = ((size_t)q * NC + w) * OCW + o;
        const int m = sc.src_row[sl];
        if (m >= 0 && P[m] > 1 && first_buf[m] < 0) {
          first_buf[m] = nb;
          nb += P[m] - 1;
        }
      }
    sc.nbuf = nb;
    for (int w = 0; w < NC; w++) {
      long long nz = 0;
      for (int o = 0; o < OCW; o++) {
        const size_t sl = ((size_t)q * NC + w) * OCW + o;
        const int m = sc.src_row[sl];
        if (m < 0) continue;
        if (P[m] == 1) {
          sc.slot_row[sl] = m;
        } else if (sc.piece[sl] == 0) {
          sc.slot_row[sl] = m;
          sc.slot_comb[sl] = (first_buf[m] << 8) | (P[m] - 1);
        } else {
          sc.slot_row[sl] = -2 - (first_buf[m] + sc.piece[sl] - 1);
        }
        for (int k = 0; k < nch; k++) {
          int pb, pe;
          piece_range(0, raw[(size_t)m * nch + k], sc.piece[sl], P[m], &pb, &pe);
          nz += pe - pb;
        }
      }
      sc.max_wave_nnz = std::max<int32_t>(sc.max_wave_nnz, (int32_t)nz);
    }
  }
  sc.split_pieces = (int32_t)(pieces - M);
  return sc;
}

int block_header(int OCW) { return (OCW + 1) & ~1; }

// Input layout for K positions per lane with D ring slots: the largest chunk that fits the
// LDS beside the counters, the block-start table and the partial-sum buffers of split rows.
// Chunks are then evened out: nch = ceil(C / Cc_max) chunks of about C / nch channels.
static bool fill_layout(const Geom& g, int K, int D, int cc_cap, int lds_max, Plan* p) {
  const int NC = p->NW - 1;
  p->K = K;
  p->D = D;
  p->PL = plan_pl(g, K, p->quad);
  p->tp = p->quad ? kQuadTile : 64 * K;
  // stride > 1: phase planes start on 64-word blocks, so that no staging block straddles two
  // planes and the producer can step its offsets from plane to plane without divisions
  if (g.st > 1) p->PL = (p->PL + 63) / 64 * 64;
  const int align = g.wide ? 256 : 64;
  const long long chs = ((long long)g.st * g.st * p->PL + align - 1) / align * align;
  if (chs > (1 << 24)) return false;
  p->CHS = (int)chs;
  p->nblk = p->CHS / 64;
  int nch = 1;
  for (int it = 0; it < 16; it++) {  // the block-start table grows with the chunk count
    const long long fixed = 4LL * p->G * NC * (nch + 1) + 8LL * kMaxDepth + 8LL * p->nbuf + 256LL * p->nbuf * K +
                            (p->quad ? 16LL + (long long)kQuadRingBytes * NC : 0);
    const long long room = (lds_max - fixed) / (4LL * D);  // input words per slot
    if (room < p->CHS) return false;
    int cc = (int)std::min<long long>(g.C, room / p->CHS);
    if (cc_cap > 0) cc = std::min(cc, cc_cap);
    const int n2 = (g.C + cc - 1) / cc;
    if (n2 <= nch) break;
    nch = n2;
  }
  p->Cc = (g.C + nch - 1) / nch;
  p->nch = (g.C + p->Cc - 1) / p->Cc;  // every chunk non-empty
  p->slot_words = p->Cc * p->CHS;
  return true;
}

// Largest block one wavefront gets for one chunk: header entries (OCW rounded up to even)
// plus each slot's non-zeros of the chunk.
// Also returns (step_permille) the cost of the per-chunk synchronisation: 1000 * the sum
// over groups and chunks of the busiest wavefront's entries over the sum of the means.
static int max_block(const Geom& g, const Plan& p, const std::vector<int32_t>& rowptr,
                     const std::vector<int32_t>& col, const Sched& sc, int32_t* step_permille = nullptr) {
  const int RS = g.R * g.S;
  std::vector<int> cnt(p.nch), tot(p.nch);
  std::vector<long long> kmax((size_t)p.G * p.nch, 0), ksum((size_t)p.G * p.nch, 0);
  int best = 0;
  for (size_t wv = 0; wv < sc.src_row.size() / p.OCW; wv++) {
    const size_t q = wv / (p.NW - 1);
    std::fill(tot.begin(), tot.end(), 0);
    for (int o = 0; o < p.OCW; o++) {
      const size_t sl = wv * p.OCW + o;
      const int m = sc.src_row[sl];
      if (m < 0) continue;
      std::fill(cnt.begin(), cnt.end(), 0);
      for (int j = rowptr[m]; j < rowptr[m + 1]; j++) cnt[(col[j] / RS) / p.Cc]++;
      for (int k = 0; k < p.nch; k++) {
        int pb, pe;
        piece_range(0, cnt[k], sc.piece[sl], sc.npieces[sl], &pb, &pe);
        tot[k] += pe - pb;
      }
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
// table; large chunks mean few steps.
// SPARSECONV_PLAN="K=..,OCW=..,D=..,CC=..,LDSKB=..,NARROW" overrides the choice (tuning only).
static bool instantiated(int K, int OCW, int quad) {
  if (quad) return K == 8 && (OCW == 3 || OCW == 5 || OCW == 9);
  static const int kk[] = {1, 2, 4, 6, 7, 8, 12, 16};
  static const int oo[] = {1, 2, 3, 5, 9};
  bool okk = false, oko = false;
  for (int v : kk) okk = okk || v == K;
  for (int v : oo) oko = oko || v == OCW;
  return okk && oko && K * OCW <= 64;
}

Plan choose_plan(const Geom& g, const std::vector<int32_t>& rowptr, const std::vector<int32_t>& col,
                 Sched* sched, int k_cap, int ocw_cap, int d, int quad) {
  static const int kOcw[] = {1, 2, 3, 5, 9};
  static const int kKs[] = {16, 12, 8, 7, 6, 4, 2, 1};
  Plan p{};
  p.NW = 16;
  const int NC = p.NW - 1;
  const char* env0 = std::getenv("SPARSECONV_PLAN");
  if (env_int(env0, "QUAD", -1) >= 0) quad = env_int(env0, "QUAD", 0) ? 1 : 0;  // tuning only
  p.quad = quad;
  const long long img_ext = (long long)g.HYp * g.Pp;
  const int kmax = img_ext >= 4096 ? 8 : img_ext >= 1024 ? 4 : img_ext >= 256 ? 2 : 1;
  // slots for every row plus the extra pieces of rows longer than a consumer's fair share
  long long extra = 0;
  {
    const double fair = std::max(1.0, (double)rowptr[g.M] / NC);
    for (int m = 0; m < g.M; m++) {
      const int n = rowptr[m + 1] - rowptr[m];
      if (n > fair) extra += std::min<long long>(NC, (long long)std::ceil(2.0 * n / fair)) - 1;
    }
  }
  int OCW = 9;
  for (int o : kOcw)
    if (NC * o >= g.M + extra) {
      OCW = o;
      break;
    }
  const char* env = std::getenv("SPARSECONV_PLAN");
  OCW = env_int(env, "OCW", OCW);
  const int kenv = env_int(env, "K", 0);
  int D = env_int(env, "D", d > 0 ? d : 3);
  const int cc_cap = env_int(env, "CC", 0);
  const int lds_max = std::min(kLdsMax, 1024 * env_int(env, "LDSKB", kLdsMax / 1024));
  if (D < 2 || D > kMaxDepth) D = 3;
  bool oko = false;
  for (int o : kOcw) oko = oko || o == OCW;
  if (!oko) OCW = 9;
  if (quad && OCW < 3) OCW = 3;  // quad kernels exist for 3, 5 and 9 slots
  if (ocw_cap > 0 && OCW > ocw_cap) {  // the largest instantiated count within the cap
    int best = kOcw[0];
    for (int o : kOcw)
      if (o <= ocw_cap) best = o;
    OCW = best;
  }
  // fewer slots per consumer (more groups) when nothing fits
  for (int oi = 4; oi >= 0; oi--) {
    if (kOcw[oi] > OCW) continue;
    p.OCW = kOcw[oi];
    p.G = (g.M + NC * p.OCW - 1) / (NC * p.OCW);
    for (int k : kKs) {
      if (!instantiated(k, p.OCW, quad)) continue;
      if (!quad && k > (kenv > 0 ? kenv : k_cap > 0 ? std::min(kmax, k_cap) : kmax)) continue;
      bool fits = true;
      Sched sc;
      p.nbuf = 0;
      for (int attempt = 0; attempt < 2; attempt++) {  // the partial buffers take LDS too
        if (!fill_layout(g, k, D, cc_cap, lds_max, &p)) {
          fits = false;
          break;
        }
        sc = schedule_rows(g, p, rowptr, col);
        if (sc.nbuf <= p.nbuf) break;
        p.nbuf = sc.nbuf;
      }
      if (!fits) continue;
      max_block(g, p, rowptr, col, sc, &p.step_permille);
      p.nbuf = sc.nbuf;
      const int table = p.G * NC * (p.nch + 1);
      p.lds_bytes = 4 * p.D * p.slot_words + 8 * kMaxDepth + 4 * table + 8 * p.nbuf + 4 * p.nbuf * 64 * k;
      p.ring_words = 0;
      if (quad) {  // 16-byte aligned entry rings after everything else
        p.ring_words = (p.lds_bytes / 4 + 3) & ~3;
        p.lds_bytes = 4 * p.ring_words + kQuadRingBytes * NC;
      }
      if (p.lds_bytes > lds_max) continue;
      p.span_images = (int)((p.PL + img_ext - 2) / img_ext + 1);
      if (sched) *sched = std::move(sc);
      return p;
    }
  }
  p.K = 0;  // does not fit: caller reports SC_EUNSUPPORTED
  return p;
}

}  // namespace sc
