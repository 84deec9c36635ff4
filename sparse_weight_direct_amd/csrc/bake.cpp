// Weights-in-code kernels: code generation (GCN assembly for gfx950) and assembly with
// amd_comgr.  The mapping and its guarantees are described in bake.h.
//
// Prior art kept from the pages: a non-zero's weight is the same for every output position
// of its channel, so it is broadcast to the whole wavefront (the wave-uniform weight of the
// "Escoin" dataflow, the shared weight of Tuteja et al., Sec. 5.4); the input is reused by
// every output channel of a group (Tuteja et al., Sec. 5.1: staged once, reused across
// output channels), here from the registers of one wavefront rather than from shared
// memory; the stretched offset c*H*W + r*W + s of "Escoin" (weight stretching) survives as
// the channel's scalar offset c*H*W*4 plus the row vector's per-lane offset r*W + sp.
#include "bake.h"

#include <amd_comgr/amd_comgr.h>

#include <algorithm>
#include <cmath>
#include <functional>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <numeric>
#include <string>

namespace sc {

void bake_magic(uint32_t d, uint32_t* m, int* l) {
  int L = 0;
  while ((1ull << L) < d) L++;  // ceil(log2 d)
  const int ll = L - 1;         // d >= 2: ll >= 0
  *m = (uint32_t)(((1ull << (32 + ll)) + d - 1) / d);
  *l = ll;
}

static int env_key(const char* s, const char* key, int dflt) {
  if (!s) return dflt;
  const size_t n = std::strlen(key);
  for (const char* p = s; (p = std::strstr(p, key)) != nullptr; p += n) {
    if ((p == s || p[-1] == ',') && p[n] == '=') return std::atoi(p + n + 1);
  }
  return dflt;
}

BakeForce bake_force_from_env() {
  BakeForce f;
  const char* e = std::getenv("SPARSECONV_BAKE");
  if (!e || !*e) return f;
  f.G = env_key(e, "G", -1);
  f.Q = env_key(e, "Q", -1);
  f.T = env_key(e, "T", -1);
  f.D = env_key(e, "D", -1);
  f.dpp = env_key(e, "DPP", -1);
  f.perm = env_key(e, "PERM", -1);
  f.stage = env_key(e, "STAGE", -1);
  f.nb = env_key(e, "NB", -1);
  f.cc = env_key(e, "CC", -1);
  f.ra = env_key(e, "RA", -1);
  f.cb = env_key(e, "CB", -1);
  f.seq = env_key(e, "SEQ", -1);
  f.gw = env_key(e, "GW", -1);
  f.c0 = env_key(e, "C0", -1);
  f.es = env_key(e, "ES", -2);
  f.esnt = env_key(e, "ESNT", -1);
  f.vt = env_key(e, "VT", -1);
  f.pb = env_key(e, "PB", -1);
  return f;
}

namespace {

constexpr int kMaxVgpr = 256;   // architectural VGPRs a VALU instruction can name
constexpr int kFixedV = 6;      // v0 id, v1 lane, v2 zero, v3 out-of-range marker, v4 output offset,
                                 // v5 lane * 4 (the lane-shift address)
constexpr int kTemps = 12;      // prologue temporaries
constexpr long long kCodeMax = 2ll << 20;  // refuse kernels above 2 MB of code (~250K non-zeros)
constexpr int kVgprTarget = 168;  // three wavefronts per SIMD
constexpr int kMinDepth = 4;      // row loads in flight a plan keeps if the registers allow
constexpr int kSimdVgprs = 512;   // VGPRs per lane of a SIMD (wave64), allocated in blocks of 8
constexpr int kLdsBytes = 160 * 1024;  // LDS of a CU

// A workgroup runs on one CU: its wavefronts are spread over the 4 SIMDs, so ceil(W / 4) of
// them share one SIMD's registers, and its LDS must fit the CU's.  A plan that does not fit
// cannot be dispatched at all.
bool fits_cu(int waves, int vgprs, int lds, std::string* why) {
  if ((waves + 3) / 4 * ((vgprs + 7) & ~7) > kSimdVgprs) {
    *why = "the workgroup's wavefronts need more registers than a CU has";
    return false;
  }
  if (lds > kLdsBytes) {
    *why = "the workgroup needs more LDS than a CU has";
    return false;
  }
  return true;
}
constexpr int kReduceChannels = 32;  // channels per round of the channel-split reduction
constexpr int kStagedChunk = 12;     // channels per staged chunk (fewer barriers than 8: ~1 us
                                     // faster on the 112x112 layers; 16 no faster)
constexpr int kStagedBases = 1;     // fixed per-slot LDS bases (pb): imb95 0.15-0.35 us, imb90
                                     // ~4 us faster than a base made per channel
constexpr int kStagedFirst = 0;      // channels of the first staged chunk (0: a full chunk)
constexpr int kStagedEarly = 0;      // units from the end at which the stores of output channels
                                     // that are already final start (0: all stores after the walk;
                                     // -1: at once).  Measured on the 112x112 layers: early stores
                                     // (with ORD=1) save 1.5-2 us when the input comes from the
                                     // Infinity Cache, but cost 1-2.5 us on inputs read from HBM,
                                     // where the writes slow the input copies of the slowest
                                     // workgroups (even when issued only in the last chunk, ES=1)

// Row vectors of one filter row: the stride phases of the filter columns (lane shifts give
// the other columns), or every column when lane shifts are off.
inline int row_vectors(const Geom& g, int dpp) { return dpp ? std::min(g.st, g.S) : g.S; }

// Registers of a plan with Mg accumulators and load depth D: the fixed registers, the row
// offsets, the load ring, the shifted copies (two sets when the shifts of the next step are
// in flight through the LDS crossbar while this step's FMAs run) and the accumulators.
inline int shift_regs(const Geom& g, const BakePlan& p) { return row_vectors(g, p.dpp) * p.maxsq * (p.perm ? 2 : 1); }
inline int plan_vgprs(const Geom& g, const BakePlan& p, int Mg, int D) {
  const int P = row_vectors(g, p.dpp);
  const int acc0 = (kFixedV + g.R * P + (D + 1) * P + shift_regs(g, p) + 1) & ~1;  // even: 16-byte LDS writes
  return (std::max(acc0 + Mg, acc0 + kTemps) + 3) & ~3;
}

struct Step {
  int c, r;
  uint64_t used;    // bit p: row vector p of this step is read by some non-zero
  int sqmax[64];    // per row vector: largest lane shift read (-1 unused)
  std::vector<int> nz;  // indices (into the sorted non-zero list) of the step's non-zeros
  int loads() const {
    int n = 0;
    for (int k = 0; k < 64; k++) n += (int)(used >> k & 1ull);
    return n;
  }
  int shifts() const {
    int n = 0;
    for (int k = 0; k < 64; k++) n += std::max(0, sqmax[k]);
    return n;
  }
};

// The non-zeros of a group sorted by (c, r, lane shift, phase, row), split into steps.
struct Nz {
  int m, c, r, pv, sq;
  uint32_t bits;
};

std::vector<Step> group_steps(const Geom& g, int dpp, const std::vector<Nz>& L) {
  std::vector<Step> steps;
  for (size_t i = 0; i < L.size(); i++) {
    if (steps.empty() || steps.back().c != L[i].c || steps.back().r != L[i].r) {
      Step st;
      st.c = L[i].c;
      st.r = L[i].r;
      st.used = 0;
      for (int k = 0; k < 64; k++) st.sqmax[k] = -1;
      steps.push_back(st);
    }
    Step& st = steps.back();
    st.used |= 1ull << L[i].pv;
    st.sqmax[L[i].pv] = std::max(st.sqmax[L[i].pv], L[i].sq);
    st.nz.push_back((int)i);
  }
  (void)g;
  (void)dpp;
  return steps;
}

// Rows to groups: largest first onto the least-loaded group with room (balance by
// non-zeros, at most mg rows per group).
std::vector<std::vector<int>> deal_rows(int M, int G, const std::vector<int32_t>& rowptr) {
  const int mg = (M + G - 1) / G;
  std::vector<int> order(M);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return rowptr[a + 1] - rowptr[a] > rowptr[b + 1] - rowptr[b]; });
  std::vector<std::vector<int>> rows(G);
  std::vector<long long> load(G, 0);
  for (int m : order) {
    int best = -1;
    for (int q = 0; q < G; q++) {
      if ((int)rows[q].size() >= mg) continue;
      if (best < 0 || load[q] < load[best]) best = q;
    }
    rows[best].push_back(m);
    load[best] += rowptr[m + 1] - rowptr[m];
  }
  for (auto& r : rows) std::sort(r.begin(), r.end());
  return rows;
}

// The order in which every weights-in-code kernel of a layer walks the input channels
// (rank[c] = position of channel c in the walk); all plans of a layer share it, so every plan
// adds each output's products in the same order.  Ascending by default.  With ORD=1 (tuning
// option, for early stores): an output channel's result is final after the last input channel
// it has a non-zero in, and from then on its store can overlap the rest of the walk, so the
// walk greedily completes the output channel with the fewest input channels still to walk,
// taking that channel's remaining input channels in ascending order; input channels without
// any non-zero come last.  Measured on the 112x112 layers: on inputs read from HBM the
// ascending order is ~0.6 us faster (the copies then read neighbouring channel planes).
std::vector<int> channel_rank(const Geom& g, const std::vector<int32_t>& rowptr, const std::vector<int32_t>& col) {
  const int RS = g.R * g.S;
  if (env_key(std::getenv("SPARSECONV_BAKE"), "ORD", 0) != 1) {
    std::vector<int> id(g.C);
    std::iota(id.begin(), id.end(), 0);
    return id;
  }
  std::vector<std::vector<int>> sup(g.M), users(g.C);
  for (int m = 0; m < g.M; m++) {
    for (int j = rowptr[m]; j < rowptr[m + 1]; j++) sup[m].push_back(col[j] / RS);
    std::sort(sup[m].begin(), sup[m].end());
    sup[m].erase(std::unique(sup[m].begin(), sup[m].end()), sup[m].end());
    for (int c : sup[m]) users[c].push_back(m);
  }
  std::vector<int> remaining(g.M), rank(g.C, -1);
  for (int m = 0; m < g.M; m++) remaining[m] = (int)sup[m].size();
  int next = 0;
  for (;;) {
    int best = -1;
    for (int m = 0; m < g.M; m++)
      if (remaining[m] > 0 && (best < 0 || remaining[m] < remaining[best])) best = m;
    if (best < 0) break;
    for (int c : sup[best]) {
      if (rank[c] >= 0) continue;
      rank[c] = next++;
      for (int m : users[c]) remaining[m]--;
    }
  }
  for (int c = 0; c < g.C; c++)
    if (rank[c] < 0) rank[c] = next++;
  return rank;
}

// Sorted non-zeros of each group: by input channel in the walk's order (channel_rank), then
// filter row, lane shift, phase and output channel.
std::vector<std::vector<Nz>> group_nonzeros(const Geom& g, int dpp, const std::vector<std::vector<int>>& rows,
                                            const std::vector<int32_t>& rowptr, const std::vector<int32_t>& col,
                                            const std::vector<float>* val) {
  const int RS = g.R * g.S;
  const std::vector<int> rank = channel_rank(g, rowptr, col);
  std::vector<int> group_of(g.M, -1);
  for (size_t q = 0; q < rows.size(); q++)
    for (int m : rows[q]) group_of[m] = (int)q;
  std::vector<std::vector<Nz>> nzs(rows.size());
  for (int m = 0; m < g.M; m++)
    for (int j = rowptr[m]; j < rowptr[m + 1]; j++) {
      const int c = col[j] / RS, r = (col[j] / g.S) % g.R, s = col[j] % g.S;
      Nz z;
      z.m = m;
      z.c = c;
      z.r = r;
      z.pv = dpp ? s % g.st : s;
      z.sq = dpp ? s / g.st : 0;
      z.bits = 0;
      if (val) std::memcpy(&z.bits, &(*val)[j], 4);
      nzs[group_of[m]].push_back(z);
    }
  for (auto& L : nzs)
    std::stable_sort(L.begin(), L.end(), [&](const Nz& a, const Nz& b) {
      if (a.c != b.c) return rank[a.c] < rank[b.c];
      if (a.r != b.r) return a.r < b.r;
      if (a.sq != b.sq) return a.sq < b.sq;
      if (a.pv != b.pv) return a.pv < b.pv;
      return a.m < b.m;
    });
  return nzs;
}

// Cost of a step in VALU instructions (FMAs and lane shifts), with a load weighed like
// two: the steps of a group are split over the Q channel-split wavefronts by this cost.
inline long long step_cost(const Step& st) { return (long long)st.nz.size() + st.shifts() + 2 * st.loads(); }

// Split [0, steps) into Q contiguous parts of about equal cost, counting extra0 more for part 0
// (split 0 also adds the other parts' partial sums); returns Q + 1 bounds.
std::vector<int> split_steps(const std::vector<Step>& steps, int Q, long long extra0 = 0) {
  long long total = extra0;
  for (const Step& st : steps) total += step_cost(st);
  std::vector<int> b(Q + 1, (int)steps.size());
  b[0] = 0;
  long long acc = extra0;
  int q = 1;
  for (int i = 0; i < (int)steps.size() && q < Q; i++) {
    acc += step_cost(steps[i]);
    while (q < Q && acc * Q >= total * q) b[q++] = i + 1;
  }
  return b;
}

// VALU cost of split 0's additions of the other splits' partial sums.
// Extra cost of split 0 over the others (none: every split reduces and stores its share).
inline long long reduce_cost(const BakePlan&) { return 0; }

// Fill the plan's derived fields (registers, LDS, section sizes) for given G, Q, T, D.
bool complete_plan(const Geom& g, const std::vector<int32_t>& rowptr, const std::vector<int32_t>& col, BakePlan* pp,
                   int D_forced, std::string* why) {
  BakePlan& p = *pp;
  const int P = row_vectors(g, p.dpp);
  p.rows = deal_rows(g.M, p.G, rowptr);
  int mg = 0;
  for (auto& r : p.rows) mg = std::max(mg, (int)r.size());
  p.Mg = p.Q > 1 ? (mg + 3) & ~3 : mg;
  // lane shifts through the LDS crossbar are issued a step ahead, so a step waits for the next
  // step's row vectors: they need a load depth of at least 2 (else DPP moves)
  if (D_forced == 1) p.perm = 0;
  int D = D_forced;
  for (int pass = 0; pass < 2 && D_forced <= 0; pass++) {
    // deepest ring that keeps the target occupancy (or, past it, fits at all)
    const int cap = std::max(1, 63 / P);
    const int vt = p.vt > 0 ? p.vt : kVgprTarget;
    const int target = plan_vgprs(g, p, p.Mg, 1) <= vt ? vt : kMaxVgpr;
    D = 1;
    while (D < cap && plan_vgprs(g, p, p.Mg, D + 1) <= target) D++;
    // a shallower ring leaves the loads' latency exposed: deepen it to kMinDepth where the
    // registers allow, at the cost of occupancy (11x11 stride-4 layer, 810 wavefronts, one per
    // SIMD at most: D = 4 15.1 us against 16.6 with D = 2; D = 6, 8, 15 15.4, 15.9, 17.6)
    while (D < std::min(cap, kMinDepth) && plan_vgprs(g, p, p.Mg, D + 1) <= kMaxVgpr) D++;
    if (!p.perm || D >= 2) break;
    p.perm = 0;
  }
  if (D * P > 63 || plan_vgprs(g, p, p.Mg, D) > kMaxVgpr) {
    *why = "output channels per group and load ring exceed the registers";
    return false;
  }
  if (p.Q > 1 && g.R * P + (D + 1) * P + shift_regs(g, p) < 6) {
    // split 0 reads the partial sums into registers of the offset, ring and shift region
    *why = "channel splits need a load depth of at least 3";
    return false;
  }
  p.D = D;
  p.vgprs = plan_vgprs(g, p, p.Mg, D);
  // rounds of rc channels: every split's part of a round (rc/4 KB) for all Q splits within the
  // 16-bit LDS offsets of one unit's region
  p.rc = std::min({p.Mg, kReduceChannels, std::max(4, (256 / p.Q) & ~3)});
  p.lds_bytes = p.Q > 1 ? p.T * p.Q * (p.rc / 4) * 1024 : 0;
  if (p.lds_bytes > kLdsBytes) {
    *why = "channel-split partial sums exceed the LDS";
    return false;
  }
  if (!fits_cu(p.Q * p.T, p.vgprs, p.lds_bytes, why)) return false;
  if (p.Q > 1 && std::min(16, (g.R * P + (D + 1) * P + shift_regs(g, p) - 2) / 4) < p.Q - 1) {
    // a split reads the other Q - 1 parts of a block into registers of the offset, ring and
    // shift region
    *why = "channel splits need 4 (Q - 1) free registers for the reduction";
    return false;
  }
  // section sizes
  auto nzs = group_nonzeros(g, p.dpp, p.rows, rowptr, col, nullptr);
  p.sec_valu = 0;
  p.sec_steps = 0;
  p.sec_loads = 0;
  long long code = 2048;
  for (auto& L : nzs) {
    auto steps = group_steps(g, p.dpp, L);
    auto b = split_steps(steps, p.Q, reduce_cost(p));
    for (int q = 0; q < p.Q; q++) {
      long long v = 0, st = 0, ld = 0;
      for (int i = b[q]; i < b[q + 1]; i++) {
        v += (long long)steps[i].nz.size() + (p.perm ? 0 : steps[i].shifts());
        st++;
        ld += steps[i].loads();
        code += 8 * (long long)steps[i].nz.size() + 8 * steps[i].shifts() + 8 * steps[i].loads() + 8;
      }
      v += p.Q > 1 ? (p.Q - 1) * p.Mg / p.Q + p.Mg / 4 : p.Mg / 4;
      p.sec_valu = std::max(p.sec_valu, v);
      p.sec_steps = std::max(p.sec_steps, st);
      p.sec_loads = std::max(p.sec_loads, ld);
    }
  }
  p.code_bytes = code;
  return true;
}

// Staged plans: registers of the fixed part, the DMA source offsets and the two sets of tap
// reads, then the accumulators.
// Batches of tap reads a staged kernel issues ahead (a batch is a step, or with channel
// batches a channel's steps): at most 15 LDS instructions may be outstanding (the lgkm
// counter), the current batch's and the ra batches ahead.
inline int staged_batch_reads(const Geom& g, int cb) {
  return cb == 2 ? g.R * g.S : cb ? (g.R * g.S + 1) / 2 : g.S;
}
inline int staged_read_ahead(const Geom& g, int forced, int cb) {
  if (cb == 2) return 1;  // a batch's reads go out once the previous batch's have landed
  const int cap = std::max(1, 15 / staged_batch_reads(g, cb) - 1);
  return std::min(cap, forced > 0 ? forced : 1);  // more measured no faster
}

// Channel batches need every tap of a channel within reach of one base register's 8-bit
// dword offsets (ds_read2_b32), and two batches of reads within the lgkm counter.
inline bool staged_cb_ok(const Geom& g) {
  return (g.R - 1) * g.Pp + g.S - 1 <= 255 && 2 * staged_batch_reads(g, 1) <= 15;
}

// Channel-pair batches (cb = 2, a tuning option): one base register per filter tap (r, s)
// points at that tap in the first channel window of the LDS region; ds_read2st64_b32 reads the
// tap of two channels of a chunk at once, its 8-bit offsets counting 256 bytes (a channel
// window is a multiple of 64 words), so the whole region of chunk buffers must lie within
// 255 * 256 bytes of the bases, and one batch's reads (one per tap) within the lgkm counter.
// It saves the per-channel base register and half the waits (imb95: 7073 instead of 7313
// instructions per wavefront) but measured 1 us slower on the 112x112 layers (likely because
// the two words a lane reads lie a multiple of 64 words apart, in the same LDS bank).
inline bool staged_cb2_ok(const Geom& g) { return g.R * g.S <= 15; }

// VGPR layout of a staged kernel: v0..v5 fixed, the DMA source offsets, the read sets
// (even-aligned pairs with channel batches), the base registers (channel batches: one per
// read set, or npb > 0 fixed ones, one per chunk slot and buffer), then the accumulators.
struct StagedRegs {
  int setw, rd, base, acc;
};
inline StagedRegs staged_regs(const Geom& g, int nvb, int ra, int cb, int npb = 0) {
  StagedRegs r;
  const int NS = ra + 1;
  r.setw = cb == 2 ? 2 * g.R * g.S : cb ? (g.R * g.S + 1) & ~1 : g.S;
  r.rd = cb ? (kFixedV + nvb + 1) & ~1 : kFixedV + nvb;
  r.base = r.rd + NS * r.setw;
  r.acc = (r.base + (cb == 2 ? g.R * g.S : cb ? (npb > 0 ? npb : NS) : 0) + 1) & ~1;
  return r;
}

inline int staged_vgprs(const Geom& g, int nvb, int Mg, int ra, int cb, int npb = 0) {
  const int acc0 = staged_regs(g, nvb, ra, cb, npb).acc;
  return (std::max(acc0 + Mg, acc0 + kTemps) + 3) & ~3;
}

// Fill a staged plan's derived fields for its G, T and (if > 0) forced buffer count and chunk
// channels (stride 1, no channel splits).
bool complete_staged(const Geom& g, const std::vector<int32_t>& rowptr, const std::vector<int32_t>& col,
                     int nb, int cc, int ra, int cb, BakePlan* pp, std::string* why) {
  BakePlan& p = *pp;
  if (g.st != 1) {
    *why = "staged plans need stride 1";
    return false;
  }
  if (g.S > 7) {  // the reads of two steps (up to 2 S) must fit the 15 LDS reads in flight
    *why = "staged plans read at most 7 taps per step";
    return false;
  }
  p.Q = 1;
  p.dpp = 1;  // a tap's column s is its lane shift sq: here an LDS offset
  p.perm = 0;
  p.maxsq = g.S - 1;
  p.cb = cb == 2 ? (staged_cb2_ok(g) ? 2 : staged_cb_ok(g) ? 1 : 0)
                 : cb >= 0 ? (cb > 0 && staged_cb_ok(g)) : staged_cb_ok(g);
  p.ra = staged_read_ahead(g, ra, p.cb);
  p.V = 64;
  p.Pb = g.Pp;
  p.bw = g.wide ? 256 : 64;  // 16 bytes per lane in the wide layout, else 4
  p.chs = (p.T * 64 + (g.R - 1) * g.Pp + g.S - 1 + p.bw - 1) / p.bw * p.bw;
  p.nblk = p.chs / p.bw;
  const int W = p.wpb();  // the wavefronts that share the window's DMA
  if (W > 16) {
    *why = "more than 16 wavefronts per workgroup";
    return false;
  }
  p.pairdist = (W % p.nblk == 0) ? 1 : 0;
  const int nvb = p.pairdist ? 1 : (p.nblk + W - 1) / W;
  // nbuf chunk buffers (the DMA runs nbuf - 1 chunks ahead); every ds_read offset (buffer +
  // channel + tap) must fit 16 bits
  const int reach = 4 * ((g.R - 1) * g.Pp + g.S);
  p.nbuf = nb > 0 ? std::max(2, std::min(nb, 8)) : 2;  // deeper prefetch measured no faster
  p.Cc = std::min(g.C, cc > 0 ? cc : kStagedChunk);
  for (;;) {
    while (p.Cc > 1 && p.nbuf * p.Cc * p.chs * 4 + reach > 65535) p.Cc--;
    if (p.nbuf * p.Cc * p.chs * 4 + reach <= 65535) break;
    if (p.nbuf == 2 || nb > 0) {
      *why = "staged window too large for 16-bit LDS offsets";
      return false;
    }
    p.nbuf--;
    p.Cc = std::min(g.C, cc > 0 ? cc : kStagedChunk);
  }
  // at most 48 DMAs of the chunks ahead outstanding per wavefront (the counter holds 63)
  auto dmas = [&](int cc) { return p.pairdist ? (cc + W / p.nblk - 1) / (W / p.nblk) : cc * nvb; };
  while (p.Cc > 1 && (p.nbuf - 1) * dmas(p.Cc) > 48) p.Cc--;
  if (p.cb == 2 && p.nbuf * p.Cc * p.chs * 4 > 255 * 256) p.cb = staged_cb_ok(g) ? 1 : 0;
  if ((p.nbuf - 1) * dmas(p.Cc) > 48) {
    *why = "staged window needs too many DMAs per chunk";
    return false;
  }
  p.rows = deal_rows(g.M, p.G, rowptr);
  int mg = 0;
  for (auto& r : p.rows) mg = std::max(mg, (int)r.size());
  p.Mg = mg;
  p.D = 0;
  if (p.cb != 1) p.pb = 0;
  p.vgprs = staged_vgprs(g, nvb, p.Mg, p.ra, p.cb, p.pb ? p.nbuf * p.Cc : 0);
  if (p.vgprs > kMaxVgpr) {
    *why = "output channels per group exceed the registers";
    return false;
  }
  p.lds_bytes = p.nbuf * p.Cc * p.chs * 4;
  p.rc = 0;
  if (!fits_cu(W, p.vgprs, p.lds_bytes, why)) return false;
  auto nzs = group_nonzeros(g, p.dpp, p.rows, rowptr, col, nullptr);
  p.sec_valu = p.sec_steps = p.sec_loads = 0;
  long long code = 4096;
  for (auto& L : nzs) {
    auto steps = group_steps(g, p.dpp, L);
    long long v = 0, ld = 0;
    for (const Step& st : steps) {
      v += (long long)st.nz.size();
      code += 8 * (long long)st.nz.size() + 8 * (st.sqmax[0] + 1) + 4;
    }
    ld = (long long)((g.C + p.Cc - 1) / p.Cc) * p.Cc * ((p.nblk + p.T - 1) / p.T);
    p.sec_valu = std::max(p.sec_valu, v + p.Mg / 4);
    p.sec_steps = std::max<long long>(p.sec_steps, (long long)steps.size());
    p.sec_loads = std::max(p.sec_loads, ld);
    code += ld * 24;
  }
  p.code_bytes = code;
  return true;
}

}  // namespace

std::vector<BakePlan> bake_candidates(const Geom& g, const std::vector<int32_t>& rowptr,
                                      const std::vector<int32_t>& col, const BakeForce& f, std::string* why) {
  std::vector<BakePlan> out;
  BakePlan p;
  p.dpp = f.dpp >= 0 ? f.dpp : 1;
  if (row_vectors(g, p.dpp) > 32) {
    *why = "more than 32 row vectors per filter row";
    return out;
  }
  p.maxsq = p.dpp ? (g.S - 1) / g.st : 0;
  if (p.maxsq >= 32) {
    *why = "filter reach too wide for lane shifts";
    return out;
  }
  // lane shifts through the LDS crossbar unless a step's shifts exceed what one
  // s_waitcnt lgkmcnt can leave outstanding (15), or there are none
  p.perm = f.perm >= 0 ? f.perm : 1;
  if (!p.dpp || p.maxsq == 0 || row_vectors(g, p.dpp) * p.maxsq > 15) p.perm = 0;
  p.V = 64 - p.maxsq;
  p.Pb = g.F + p.maxsq;
  const int M = g.M;
  const long long nnz = rowptr[M];
  if (nnz * 8 > kCodeMax) {  // 8 bytes of code per non-zero: refuse before generating
    *why = "too many non-zeros for a weights-in-code kernel (" + std::to_string(nnz) + ")";
    return out;
  }
  // base groups: the fewest whose accumulators fit the register target (measured on the
  // 112x112 layers, one group per wavefront beats more groups even with several hundred KB of
  // code: more groups repeat the row loads and lane shifts per group)
  const int vtarget = f.vt > 0 ? std::min(f.vt, kMaxVgpr) : kVgprTarget;
  p.vt = vtarget;
  auto fewest_groups = [&](const BakePlan& q) {
    int n = 1;
    while (n < M && plan_vgprs(g, q, (M + n - 1) / n, 2) > vtarget) n++;
    return n;
  };
  int G0 = fewest_groups(p);
  if (p.perm) {
    // the second set of shift registers must not cost a group: DPP shifts if they need fewer
    BakePlan q = p;
    q.perm = 0;
    const int g_dpp = fewest_groups(q);
    if (g_dpp < G0 && f.perm < 0) {
      p.perm = 0;
      G0 = g_dpp;
    }
  }
  struct Shape {
    int G, Q, T;
  };
  std::vector<Shape> shapes;
  if (f.any()) {
    const int G = f.G > 0 ? std::min(f.G, M) : G0;
    const int Q = f.Q > 0 ? f.Q : 1;
    shapes.push_back({G, Q, f.T > 0 ? f.T : std::max(1, 4 / Q)});
  } else {
    // the base plan, then variants that give small batches more wavefronts: channel splits
    // (no repeated loads, a reduction in LDS) and more groups (repeated loads, no reduction);
    // the forward's estimate or sparseconv_tune chooses among them per batch size
    shapes = {{G0, 1, 4}, {G0, 2, 1}, {G0, 3, 1}, {G0, 4, 1}, {std::min(M, 2 * G0), 1, 4},
              {std::min(M, 4 * G0), 1, 4}, {std::min(M, 2 * G0), 2, 1}};
  }
  // staged plan: forced (STAGE=1), or appended to the candidates for stride-1 layers
  auto add_staged = [&](int G, int T, int seq, int gw) {
    BakePlan c = p;
    c.stage = 1;
    c.G = G;
    c.T = T;
    c.seq = G > 1 ? seq : 0;
    c.gw = G > 1 && !c.seq ? gw : 0;
    std::string w;
    c.c0 = f.c0 >= 0 ? f.c0 : kStagedFirst;
    c.es = f.es >= -1 ? f.es : kStagedEarly;
    c.esnt = f.esnt >= 0 ? f.esnt : 0;
    c.pb = f.pb >= 0 ? f.pb : kStagedBases;
    if (complete_staged(g, rowptr, col, f.nb, f.cc, f.ra, f.cb, &c, &w))
      out.push_back(std::move(c));
    else if (out.empty())
      *why = w;
  };
  auto staged_groups = [&](int nvb) {
    int n = 1;
    const int cb = f.cb >= 0 ? (f.cb > 0 && staged_cb_ok(g)) : staged_cb_ok(g);
    while (n < M && staged_vgprs(g, nvb, (M + n - 1) / n, staged_read_ahead(g, f.ra, cb), cb) > kVgprTarget) n++;
    return n;
  };
  if (f.stage == 1 || f.nb > 0 || f.cc > 0 || f.ra > 0 || f.cb >= 0 || f.seq >= 0 || f.gw >= 0 || f.c0 >= 0 ||
      f.es >= -1 || f.esnt >= 0 || f.pb >= 0) {
    const int T = f.T > 0 ? f.T : 4;
    add_staged(f.G > 0 ? std::min(f.G, M) : staged_groups(2), T, f.seq > 0 ? 1 : 0, f.gw > 0 ? 1 : 0);
    return out;
  }
  for (const Shape& sh : shapes) {
    if (sh.Q < 1 || sh.Q > 16) {
      *why = "channel splits must be 1 to 16";
      continue;
    }
    if (sh.Q * sh.T > 16) {
      *why = "more than 16 wavefronts per workgroup";
      continue;
    }
    bool dup = false;
    for (const BakePlan& o : out) dup = dup || (o.G == sh.G && o.Q == sh.Q && o.T == sh.T);
    if (dup) continue;
    BakePlan c = p;
    c.G = sh.G;
    c.Q = sh.Q;
    c.T = sh.T;
    std::string w;
    if (complete_plan(g, rowptr, col, &c, f.D, &w))
      out.push_back(std::move(c));
    else if (out.empty())
      *why = w;
  }
  if (!f.any() && g.st == 1) {
    // staged kernels: one group per workgroup, and twice the groups sharing each workgroup's
    // window (more, lighter wavefronts that repeat the tap reads; faster where the FMAs
    // dominate)
    const int G1 = staged_groups(2);
    add_staged(G1, 4, 0, 0);
    if (2 * G1 <= M && 4 * 2 * G1 <= 16) add_staged(2 * G1, 4, 0, 1);
  }
  return out;
}

double bake_estimate(const Geom& g, const BakePlan& p, int N, int cus) {
  const long long qtot = p.stage ? (long long)N * g.HYp * g.Pp : (long long)N * g.E * p.Pb;
  const long long ntiles = p.stage ? (qtot + 64LL * p.T - 1) / (64LL * p.T) * p.T : (qtot + p.V - 1) / p.V;
  const long long waves = ntiles * (p.seq ? 1 : p.G) * p.Q;  // gw: the same waves, fewer workgroups
  const double simds = 4.0 * cus;
  // VALU: a SIMD runs about ceil(waves / SIMDs) sections' instructions one after the other
  const double valu = std::ceil((double)waves / simds) * (double)p.sec_valu * 4.0;
  // loads: a section's row loads are issued one step after another (~35 cycles each)
  const double loads = (double)p.sec_loads * 35.0;
  // HBM: input read once, output written once, at about 5 TB/s (2.3 KB per cycle at 2.2 GHz)
  const double hbm = 4.0 * ((double)N * g.C * g.H * g.W + (double)N * g.M * g.E * g.F) / 2300.0;
  // launch, first loads and the final stores (~5 us)
  return 11000.0 + std::max(valu, std::max(loads, hbm));
}

namespace {

std::string fmt(const char* f, ...) __attribute__((format(printf, 1, 2)));
std::string fmt(const char* f, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, f);
  vsnprintf(buf, sizeof buf, f, ap);
  va_end(ap);
  return buf;
}

// The 8-byte instructions of the hot loops (FMAs with a literal weight, LDS and buffer
// accesses) are placed at 8-byte aligned addresses: a wavefront issues such an instruction
// markedly slower when it straddles an 8-byte boundary (measured on a stream of literal FMAs:
// 5.9 against 4.5 cycles with one wavefront per SIMD, 2.9 against 2.3 with two).  The
// assembler pads with s_nop 0 where a 4-byte instruction (a wait, a barrier) left the
// stream misaligned.  AL=0 in SPARSECONV_BAKE turns this off (measurement only).
static bool hot_align() { return env_key(std::getenv("SPARSECONV_BAKE"), "AL", 1) != 0; }

struct Emitter {
  std::string s;
  long long valu = 0;                 // VALU instructions (and nop wait states) issued
  std::vector<long long> wr;          // per VGPR: index of its last VALU write
  long long code = 0;                 // bytes
  const bool align = hot_align();
  Emitter() : wr(kMaxVgpr, -100) {}
  void line(const char* f, ...) __attribute__((format(printf, 2, 3))) {
    char buf[256];
    va_list ap;
    va_start(ap, f);
    vsnprintf(buf, sizeof buf, f, ap);
    va_end(ap);
    if (align && (!std::strncmp(buf, "v_fmac_f32_e32", 14) || !std::strncmp(buf, "v_fmamk_f32", 11) ||
                  !std::strncmp(buf, "ds_", 3) || !std::strncmp(buf, "buffer_", 7)))
      s += "\t.p2align 3\n";
    s += '\t';
    s += buf;
    s += '\n';
  }
  void label(const std::string& l) { s += l + ":\n"; }
  // a VALU instruction writing VGPR d (d < 0: none); bytes: its encoded size
  void valu_op(int d, int bytes) {
    if (d >= 0) wr[d] = valu;
    valu++;
    code += bytes;
  }
  // wait states gfx950 needs (the hardware does not interlock these):
  //  - a DPP read of a VGPR: 2 after a VALU write of it or the issue of a load into it
  //  - v_readfirstlane of a VGPR: 1 after a VALU write of it
  //  - a VALU read of VCC (v_cndmask): 2 after a VALU write of VCC (v_cmp)
  long long vcc_wr = -100;
  void guard(long long since, int need) {
    const long long gap = valu - since - 1;
    if (gap < need) {
      const int n = (int)(need - gap);
      line("s_nop %d", n - 1);
      valu += n;
      code += 4;
    }
  }
  void dpp_guard(int v) { guard(wr[v], 2); }
  void rfl_guard(int v) { guard(wr[v], 1); }
  void vcc_guard() { guard(vcc_wr, 2); }
  void cmp(const std::string& text) {
    line("%s", text.c_str());
    vcc_wr = valu;
    valu_op(-1, 4);
  }
  void cnd(int d, const std::string& text) {
    vcc_guard();
    line("%s", text.c_str());
    valu_op(d, 4);
  }
  void v(int d, int bytes, const std::string& text) {
    line("%s", text.c_str());
    valu_op(d, bytes);
  }
};

}  // namespace

// Kernel descriptor and code-object metadata of a generated kernel (symbol sc_baked, the
// 40-byte BakeArgs argument segment), appended to its code.
void finish_kernel(Emitter& E, BakePlan& p, int nv, int WPB, std::string* src) {
  p.sgprs = 40;
  char kd[2048];
  snprintf(kd, sizeof kd,
           "\t.section .rodata,\"a\",@progbits\n"
           "\t.p2align 6, 0x0\n"
           "\t.amdhsa_kernel sc_baked\n"
           "\t\t.amdhsa_group_segment_fixed_size %d\n"
           "\t\t.amdhsa_private_segment_fixed_size 0\n"
           "\t\t.amdhsa_kernarg_size 40\n"
           "\t\t.amdhsa_user_sgpr_count 2\n"
           "\t\t.amdhsa_user_sgpr_kernarg_segment_ptr 1\n"
           "\t\t.amdhsa_system_sgpr_workgroup_id_x 1\n"
           "\t\t.amdhsa_system_vgpr_workitem_id 0\n"
           "\t\t.amdhsa_next_free_vgpr %d\n"
           "\t\t.amdhsa_next_free_sgpr %d\n"
           "\t\t.amdhsa_accum_offset %d\n"
           "\t\t.amdhsa_reserve_vcc 1\n"
           "\t\t.amdhsa_float_denorm_mode_32 3\n"
           "\t\t.amdhsa_float_denorm_mode_16_64 3\n"
           "\t\t.amdhsa_dx10_clamp 1\n"
           "\t\t.amdhsa_ieee_mode 1\n"
           "\t.end_amdhsa_kernel\n"
           "\t.text\n",
           p.lds_bytes, nv, p.sgprs, nv);
  E.s += kd;
  char md[2048];
  snprintf(md, sizeof md,
           "\t.amdgpu_metadata\n"
           "---\n"
           "amdhsa.kernels:\n"
           "  - .agpr_count: 0\n"
           "    .args:\n"
           "      - .address_space: global\n        .offset: 0\n        .size: 8\n        .value_kind: global_buffer\n"
           "      - .address_space: global\n        .offset: 8\n        .size: 8\n        .value_kind: global_buffer\n"
           "      - .offset: 16\n        .size: 4\n        .value_kind: by_value\n"
           "      - .offset: 20\n        .size: 4\n        .value_kind: by_value\n"
           "      - .offset: 24\n        .size: 4\n        .value_kind: by_value\n"
           "      - .offset: 28\n        .size: 4\n        .value_kind: by_value\n"
           "      - .offset: 32\n        .size: 4\n        .value_kind: by_value\n"
           "      - .offset: 36\n        .size: 4\n        .value_kind: by_value\n"
           "    .group_segment_fixed_size: %d\n"
           "    .kernarg_segment_align: 8\n"
           "    .kernarg_segment_size: 40\n"
           "    .max_flat_workgroup_size: %d\n"
           "    .name: sc_baked\n"
           "    .private_segment_fixed_size: 0\n"
           "    .sgpr_count: %d\n"
           "    .symbol: sc_baked.kd\n"
           "    .vgpr_count: %d\n"
           "    .wavefront_size: 64\n"
           "amdhsa.target: amdgcn-amd-amdhsa--gfx950\n"
           "amdhsa.version:\n  - 1\n  - 2\n"
           "...\n"
           "\t.end_amdgpu_metadata\n",
           p.lds_bytes, WPB * 64, p.sgprs + 6, nv);
  E.s += md;
  *src = std::move(E.s);
}

// LDS DMA instructions of a chunk of cn channels that every wavefront of a staged workgroup
// issues at least (wavefronts skip the blocks and channels past the chunk's end).
static int staged_dmas_min(const BakePlan& p, int cn) {
  int best = 1 << 30;
  const int W = p.wpb();  // the wavefronts sharing the window
  for (int w = 0; w < W; w++) {
    int n = 0;
    if (p.pairdist) {
      const int per = W / p.nblk;
      for (int i = 0; i * per < cn; i++) n += (w / p.nblk + i * per < cn) ? 1 : 0;
    } else {
      const int nvb = (p.nblk + W - 1) / W;
      for (int k2 = 0; k2 < nvb; k2++) n += (k2 * W + w < p.nblk) ? cn : 0;
    }
    best = std::min(best, n);
  }
  return best;
}

// Staged kernel (stride 1).  Positions I = n*HYp*Pp + yp*Pp + xq of the padded layout (the
// LDS-tile kernel's: HYp = H + 2 pad rows per image, pitch Pp, input column x at xq = x + xoff;
// output (yp, xq - cshift) valid for yp < E, 0 <= xq - cshift < F); tap (r, s) of position I
// is the padded word I + r*Pp + s.  Workgroup b covers positions [I0, I0 + T*64) of one group:
// wavefront w holds I0 + 64 w + lane.  Per chunk of Cc channels each channel's window
// [I0, I0 + chs) is copied into LDS once (LDS DMA: lane i writes M0 + 4*i*(bw/64); zero where
// the source lies in the padding: out-of-range offset) into one of nbuf buffers, nbuf - 1
// chunks ahead of the FMAs; a channel's taps are read as one batch (ds_read2_b32 pairs from the
// base register of its chunk slot and buffer, set in the prologue, or made per channel), a
// batch ahead, or a step's by ds_read_b32 from the lane's base v5 at immediate offsets
// (cb = 0), or two channels' (cb = 2).  After the walk the outputs are stored through VGPR
// bases (store_slots).
bool generate_staged(const Geom& g, const std::vector<int32_t>& rowptr, const std::vector<int32_t>& col,
                     const std::vector<float>& val, BakePlan& p, std::string* src, std::string* err) {
  const int T = p.T, S = g.S;
  const int W = p.wpb();  // wavefronts per workgroup: T tiles (x G groups with a shared window)
  const int nvb = p.pairdist ? 1 : (p.nblk + W - 1) / W;
  const int lw = p.bw / 64;  // DMA words per lane
  const int vB = kFixedV;              // DMA source offsets
  const int NS = p.ra + 1;             // read sets: the current batch's and ra batches ahead
  const int npb = p.pb ? p.nbuf * p.Cc : 0;
  const StagedRegs sr = staged_regs(g, nvb, p.ra, p.cb, npb);
  const int SETW = sr.setw, vRd = sr.rd, vBase = sr.base, vAcc = sr.acc;
  const int vTmp = vAcc;               // prologue temporaries overlap the accumulators
  const int nv = staged_vgprs(g, nvb, p.Mg, p.ra, p.cb, npb);
  if (nv > kMaxVgpr || vAcc + p.Mg > nv) {
    *err = "staged kernel needs more than 256 VGPRs";
    return false;
  }
  p.vgprs = nv;
  const long long HW4 = 4ll * g.H * g.W;
  const long long EF4 = 4ll * g.E * g.F;
  const int BUF = p.Cc * p.chs * 4;  // bytes of one chunk buffer
  // the walk takes the input channels in the layer's order (channel_rank); chunk k holds the
  // channels of ranks [cstart[k], cstart[k] + csize[k]).  The first chunks are smaller (c0
  // channels, doubling up to Cc), so the FMAs start once a few channels have arrived.
  const std::vector<int> rank = channel_rank(g, rowptr, col);
  std::vector<int> corder(g.C), cstart, csize, chunk_of(g.C);
  for (int c = 0; c < g.C; c++) corder[rank[c]] = c;
  for (int c0 = 0, sz = p.c0 > 0 ? std::min(p.c0, p.Cc) : p.Cc; c0 < g.C; c0 += csize.back(), sz = std::min(p.Cc, 2 * sz)) {
    cstart.push_back(c0);
    csize.push_back(std::min(sz, g.C - c0));
    for (int j = c0; j < c0 + csize.back(); j++) chunk_of[j] = (int)cstart.size() - 1;
  }
  const int nchunks = (int)cstart.size();
  bool ascending = true;
  for (int c = 0; c < g.C; c++) ascending = ascending && rank[c] == c;

  Emitter E;
  E.s.reserve((size_t)rowptr[g.M] * 48 + 65536);
  E.s += "\t.amdgcn_target \"amdgcn-amd-amdhsa--gfx950\"\n";
  E.s += "\t.amdhsa_code_object_version 6\n";
  E.s += "\t.text\n\t.globl sc_baked\n\t.p2align 8\n\t.type sc_baked,@function\n";
  E.label("sc_baked");
  E.line("s_load_dwordx8 s[20:27], s[0:1], 0x0");
  E.line("s_load_dwordx2 s[28:29], s[0:1], 0x20");
  E.v(vTmp, 4, fmt("v_lshrrev_b32_e32 v%d, 6, v0", vTmp));
  E.v(1, 4, "v_and_b32_e32 v1, 63, v0");
  E.v(2, 4, "v_mov_b32_e32 v2, 0");
  E.v(3, 4, "v_bfrev_b32_e32 v3, 1");  // 0x80000000
  E.rfl_guard(vTmp);
  E.v(-1, 8, fmt("v_readfirstlane_b32 s14, v%d", vTmp));
  E.line("s_waitcnt lgkmcnt(0)");
  // logical workgroup -> (group s16, block of T tiles s15); s25 = blocks per group (with
  // sequential groups or a shared window every workgroup covers all groups)
  E.line("s_and_b32 s15, s2, 7");
  E.line("s_mul_i32 s15, s15, s29");
  E.line("s_lshr_b32 s16, s2, 3");
  E.line("s_add_u32 s15, s15, s16");
  E.line("s_mov_b32 s16, 0");
  // sections: one per group, or one that runs every group in turn (sequential groups); the
  // workgroups cover every group, or (sequential groups, shared window) all of them at once
  const int nsec = p.seq ? 1 : p.G;
  const int wg_groups = (p.seq || p.gw) ? 1 : p.G;
  for (int q = 0; q < wg_groups; q++) {
    E.line("s_cmp_lt_u32 s15, s25");
    E.line("s_cbranch_scc1 .Lunit");
    E.line("s_sub_u32 s15, s15, s25");
    E.line("s_add_u32 s16, s16, 1");
  }
  E.line("s_endpgm");
  E.label(".Lunit");
  E.line("s_mov_b32 s4, s20");
  E.line("s_and_b32 s5, s21, 0xffff");
  E.line("s_mov_b32 s6, s26");
  E.line("s_mov_b32 s7, 0x20000");
  E.line("s_mov_b32 s8, s22");
  E.line("s_and_b32 s9, s23, 0xffff");
  E.line("s_mov_b32 s10, s27");
  E.line("s_mov_b32 s11, 0x20000");
  const int tPos = vTmp, tN = vTmp + 1, tRem = vTmp + 2, tY = vTmp + 3, tX = vTmp + 4, t0 = vTmp + 5,
            t1 = vTmp + 6, t2 = vTmp + 7;
  auto divide = [&](int dst, int num, uint32_t d, int sreg) {
    if (d == 1) {
      E.v(dst, 4, fmt("v_mov_b32_e32 v%d, v%d", dst, num));
      return;
    }
    uint32_t m;
    int l;
    bake_magic(d, &m, &l);
    E.line("s_mov_b32 s%d, 0x%x", sreg, m);
    E.v(dst, 8, fmt("v_mul_hi_u32 v%d, v%d, s%d", dst, num, sreg));
    if (l > 0) E.v(dst, 4, fmt("v_lshrrev_b32_e32 v%d, %d, v%d", dst, l, dst));
  };
  const uint32_t IMG = (uint32_t)g.HYp * (uint32_t)g.Pp;
  // (n, yp, xq) of the extended index in vector register num
  auto decompose = [&](int num) {
    divide(tN, num, IMG, 17);
    E.line("s_mov_b32 s18, 0x%x", IMG);
    E.v(t0, 8, fmt("v_mul_lo_u32 v%d, v%d, s18", t0, tN));
    E.v(tRem, 4, fmt("v_sub_u32_e32 v%d, v%d, v%d", tRem, num, t0));
    divide(tY, tRem, (uint32_t)g.Pp, 17);
    E.line("s_mov_b32 s18, 0x%x", (uint32_t)g.Pp);
    E.v(t0, 8, fmt("v_mul_lo_u32 v%d, v%d, s18", t0, tY));
    E.v(tX, 4, fmt("v_sub_u32_e32 v%d, v%d, v%d", tX, tRem, t0));
  };
  // the wavefront's tile s37 (and with a shared window its group: s16 = w / T, s37 = w % T)
  if (p.gw) {
    E.line("s_mul_i32 s16, s14, %d", (65536 + T - 1) / T);
    E.line("s_lshr_b32 s16, s16, 16");
    E.line("s_mul_i32 s37, s16, %d", T);
    E.line("s_sub_u32 s37, s14, s37");
  } else {
    E.line("s_mov_b32 s37, s14");
  }
  // this wavefront's position and LDS base
  E.line("s_mul_i32 s17, s15, %d", T);
  E.line("s_add_u32 s17, s17, s37");
  E.line("s_mul_i32 s17, s17, 64");
  E.v(tPos, 4, fmt("v_add_u32_e32 v%d, s17, v1", tPos));
  E.line("s_mul_i32 s18, s37, 64");
  E.v(5, 4, "v_add_u32_e32 v5, s18, v1");
  E.v(5, 4, "v_lshlrev_b32_e32 v5, 2, v5");
  if (p.cb == 2)  // channel-pair batches: the base of tap (r, s) in the region's first window
    for (int t = 0; t < g.R * S; t++)
      E.v(vBase + t, 8, fmt("v_add_u32_e32 v%d, 0x%x, v5", vBase + t, ((t / S) * g.Pp + t % S) * 4));
  for (int b = 0; b < (npb ? p.nbuf : 0); b++)  // fixed bases: slot j of buffer b
    for (int j = 0; j < p.Cc; j++)
      E.v(vBase + b * p.Cc + j, 8, fmt("v_add_u32_e32 v%d, 0x%x, v5", vBase + b * p.Cc + j, b * BUF + j * p.chs * 4));
  decompose(tPos);
  // output offset 4*((n*M*E + yp)*F + f), f = xq - cshift; out of range unless yp < E,
  // f < F (unsigned) and n < N
  E.v(t1, 8, fmt("v_add_u32_e32 v%d, 0x%x, v%d", t1, (uint32_t)(-g.cshift), tX));
  E.line("s_mov_b32 s18, 0x%x", (uint32_t)((uint64_t)g.M * g.E));
  E.v(t0, 8, fmt("v_mul_lo_u32 v%d, v%d, s18", t0, tN));
  E.v(t0, 4, fmt("v_add_u32_e32 v%d, v%d, v%d", t0, t0, tY));
  E.line("s_mov_b32 s18, 0x%x", (uint32_t)g.F);
  E.v(t0, 8, fmt("v_mul_lo_u32 v%d, v%d, s18", t0, t0));
  E.v(t0, 4, fmt("v_add_u32_e32 v%d, v%d, v%d", t0, t0, t1));
  E.v(t0, 4, fmt("v_lshlrev_b32_e32 v%d, 2, v%d", t0, t0));
  E.cmp(fmt("v_cmp_gt_u32_e32 vcc, s18, v%d", t1));
  E.cnd(t0, fmt("v_cndmask_b32_e32 v%d, v3, v%d, vcc", t0, t0));
  E.line("s_mov_b32 s18, 0x%x", (uint32_t)g.E);
  E.cmp(fmt("v_cmp_gt_u32_e32 vcc, s18, v%d", tY));
  E.cnd(t0, fmt("v_cndmask_b32_e32 v%d, v3, v%d, vcc", t0, t0));
  E.cmp(fmt("v_cmp_gt_u32_e32 vcc, s24, v%d", tN));
  E.cnd(4, fmt("v_cndmask_b32_e32 v4, v3, v%d, vcc", t0));
  // DMA source offsets: word J = I0 + blk*bw + lane*lw of the window; input (yp - pad,
  // xq - xoff) of image n, out of range in the padding and past the batch
  if (p.pairdist) {
    // wave w stages block w % nblk of the chunk's slots w / nblk + i * (W / nblk): s31 = w / nblk
    E.line("s_mul_i32 s31, s14, %d", (65536 + p.nblk - 1) / p.nblk);
    E.line("s_lshr_b32 s31, s31, 16");
    E.line("s_mul_i32 s30, s31, %d", p.nblk);
    E.line("s_sub_u32 s30, s14, s30");                    // w % nblk
    E.line("s_mul_i32 s32, s31, %d", p.chs * 4);
    E.line("s_mul_i32 s17, s30, %d", p.bw * 4);
    E.line("s_add_u32 s32, s32, s17");                    // LDS part of M0
    E.line("s_mov_b32 s17, 0x%llx", HW4);
    E.line("s_mul_i32 s33, s31, s17");                    // channel part of the scalar offset
  }
  E.line("s_mul_i32 s19, s15, %d", T * 64);                // I0
  for (int k = 0; k < nvb; k++) {
    if (p.pairdist)
      E.line("s_mov_b32 s17, s30");
    else
      E.line("s_add_u32 s17, s14, %d", k * W);
    E.line("s_mul_i32 s17, s17, %d", p.bw);
    E.line("s_add_u32 s17, s17, s19");
    E.v(t2, 4, fmt("v_lshlrev_b32_e32 v%d, %d, v1", t2, lw == 4 ? 2 : 0));
    E.v(t2, 4, fmt("v_add_u32_e32 v%d, s17, v%d", t2, t2));
    decompose(t2);
    E.v(tY, 8, fmt("v_add_u32_e32 v%d, 0x%x, v%d", tY, (uint32_t)(-g.pad), tY));   // iy
    E.v(tX, 8, fmt("v_add_u32_e32 v%d, 0x%x, v%d", tX, (uint32_t)(-g.xoff), tX));  // ix
    E.line("s_mov_b32 s18, 0x%x", (uint32_t)((uint64_t)g.C * g.H));
    E.v(t0, 8, fmt("v_mul_lo_u32 v%d, v%d, s18", t0, tN));
    E.v(t0, 4, fmt("v_add_u32_e32 v%d, v%d, v%d", t0, t0, tY));
    E.line("s_mov_b32 s18, 0x%x", (uint32_t)g.W);
    E.v(t0, 8, fmt("v_mul_lo_u32 v%d, v%d, s18", t0, t0));
    E.v(t0, 4, fmt("v_add_u32_e32 v%d, v%d, v%d", t0, t0, tX));
    E.v(t0, 4, fmt("v_lshlrev_b32_e32 v%d, 2, v%d", t0, t0));
    E.cmp(fmt("v_cmp_gt_u32_e32 vcc, s18, v%d", tX));
    E.cnd(t0, fmt("v_cndmask_b32_e32 v%d, v3, v%d, vcc", t0, t0));
    E.line("s_mov_b32 s18, 0x%x", (uint32_t)g.H);
    E.cmp(fmt("v_cmp_gt_u32_e32 vcc, s18, v%d", tY));
    E.cnd(t0, fmt("v_cndmask_b32_e32 v%d, v3, v%d, vcc", t0, t0));
    E.cmp(fmt("v_cmp_gt_u32_e32 vcc, s24, v%d", tN));
    E.cnd(vB + k, fmt("v_cndmask_b32_e32 v%d, v3, v%d, vcc", vB + k, t0));
  }
  // select the group's section
  for (int k = 1; k < nsec; k++) {
    E.line("s_cmp_eq_u32 s16, %d", k);
    E.line("s_cbranch_scc0 .Lnot%d", k);
    E.line("s_getpc_b64 s[34:35]");
    E.label(".Lpc" + std::to_string(k));
    E.line("s_add_u32 s34, s34, .Lsec%d-.Lpc%d", k, k);
    E.line("s_addc_u32 s35, s35, 0");
    E.line("s_setpc_b64 s[34:35]");
    E.label(".Lnot" + std::to_string(k));
  }

  std::vector<int> slot_of(g.M, -1);
  for (int q = 0; q < p.G; q++)
    for (size_t i = 0; i < p.rows[q].size(); i++) slot_of[p.rows[q][i]] = (int)i;
  auto nzs = group_nonzeros(g, p.dpp, p.rows, rowptr, col, &val);
  const char* dma = p.bw == 256 ? "buffer_load_dwordx4" : "buffer_load_dword";
  long long fmas = 0;
  int lbl = 0;
  p.sec_valu = 0;
  int nstores = 0;  // stores issued so far in the current section
  // outputs of group q, slots ks: +0 for accumulators no FMA touched, one store per output
  // channel (an accumulator is never written again once its store has been issued)
  // After the walk (free: the read sets, no read in flight) the stores address output channel
  // m = NB*a + j through the VGPR base v4 + j*E*F*4 (vS_j, made in the read-set registers; vS_0
  // is v4) and the scalar offset NB*a*E*F*4, which changes only with a (channels stored in
  // ascending order): one instruction per store instead of two.  Lanes off the output keep an
  // offset past the buffer's range (v4 = 0x80000000 there, and the offsets added stay below
  // 2^32 because the output is smaller than 2^31 bytes).
  const int NBASE = std::min(16, NS * SETW + 1);
  auto store_slots = [&](int q, const std::vector<int>& ks, const std::vector<char>& touched, bool early) {
    for (int k : ks)
      if (!touched[k]) E.v(vAcc + k, 4, fmt("v_mov_b32_e32 v%d, 0", vAcc + k));
    const char* pol = early && p.esnt == 1 ? " nt" : early && p.esnt == 2 ? " sc0 sc1" : early && p.esnt == 3 ? " sc1" : "";
    if (early || NBASE < 2 || ks.size() < 8) {
      for (int k : ks) {
        E.line("s_mov_b32 s13, 0x%llx", (long long)p.rows[q][k] * EF4);
        E.line("buffer_store_dword v%d, v4, s[8:11], s13 offen%s", vAcc + k, pol);
        E.code += 16;
      }
    } else {
      auto vS = [&](int j) { return j == 0 ? 4 : vRd + j - 1; };
      E.line("s_mov_b32 s13, 0x%llx", (long long)EF4);
      for (int j = 1; j < NBASE; j++) E.v(vS(j), 4, fmt("v_add_u32_e32 v%d, s13, v%d", vS(j), vS(j - 1)));
      std::vector<int> order(ks);
      std::sort(order.begin(), order.end(), [&](int x, int y) { return p.rows[q][x] < p.rows[q][y]; });
      int cur = -1;
      for (int k : order) {
        const int m = p.rows[q][k], a = m / NBASE;
        if (a != cur) {
          E.line("s_mov_b32 s13, 0x%llx", (long long)a * NBASE * EF4);
          cur = a;
        }
        E.line("buffer_store_dword v%d, v%d, s[8:11], s13 offen", vAcc + k, vS(m % NBASE));
        E.code += 8;
      }
    }
    nstores += (int)ks.size();
  };
  for (int sec = 0; sec < nsec; sec++) {
    if (sec > 0) E.label(".Lsec" + std::to_string(sec));
    const long long v0 = E.valu;
    // the section's groups, in order, and its units of work: (group, chunk that holds steps
    // of that group, those steps); the DMA pipeline runs over the units, across groups
    std::vector<int> gl;
    for (int q = 0; q < p.G; q++)
      if (p.seq || q == sec) gl.push_back(q);
    std::vector<std::vector<Step>> alls;
    for (int q : gl) alls.push_back(group_steps(g, p.dpp, nzs[q]));
    struct Unit {
      int gi, k;
      std::vector<int> ts;
    };
    std::vector<Unit> units;
    for (int gi = 0; gi < (int)gl.size(); gi++) {
      if (p.gw) {
        // the waves of every group stage the shared window together: every section runs every
        // chunk (empty ones too), so all pass the same copies and barriers
        for (int k = 0; k < nchunks; k++) units.push_back({gi, k, {}});
        for (int t = 0; t < (int)alls[gi].size(); t++) units[chunk_of[rank[alls[gi][t].c]]].ts.push_back(t);
        continue;
      }
      for (int t = 0; t < (int)alls[gi].size(); t++) {
        const int k = chunk_of[rank[alls[gi][t].c]];
        if (units.empty() || units.back().gi != gi || units.back().k != k) units.push_back({gi, k, {}});
        units.back().ts.push_back(t);
      }
    }
    std::vector<char> touched(p.Mg, 0), stored(gl.size(), 0);
    nstores = 0;
    // the unit holding each slot's last FMA (-1: none): an output channel's store is issued at
    // the start of the group's next unit, so it overlaps the rest of the walk (the channel
    // order puts many channels' last FMAs early), or after the group's last unit
    std::vector<std::vector<int>> last_unit(gl.size());
    for (int gi = 0; gi < (int)gl.size(); gi++) last_unit[gi].assign(p.rows[gl[gi]].size(), -1);
    for (int ci = 0; ci < (int)units.size(); ci++) {
      const int gi = units[ci].gi;
      for (int t : units[ci].ts)
        for (int i : alls[gi][t].nz) last_unit[gi][slot_of[nzs[gl[gi]][i].m]] = ci;
    }
    // with es >= 0 early stores start only at the group's es-th unit from the end (es = 0: all
    // stores after the group's last unit)
    std::vector<int> gfirst(gl.size(), -1), glast(gl.size(), -1);
    for (int ci = 0; ci < (int)units.size(); ci++) {
      if (gfirst[units[ci].gi] < 0) gfirst[units[ci].gi] = ci;
      glast[units[ci].gi] = ci;
    }
    // the slots of group gi whose stores are issued at the start of unit ci (ci = glast + 1:
    // after the group's last unit)
    auto slots_at = [&](int gi, int ci) {
      const int from = p.es < 0 ? gfirst[gi] : std::max(gfirst[gi], glast[gi] + 1 - p.es);
      std::vector<int> ks;
      for (int k = 0; k < (int)last_unit[gi].size(); k++) {
        const int u = std::max(from, last_unit[gi][k] + 1);  // -1: at the first unit
        if (u == ci || (ci == glast[gi] + 1 && u > ci)) ks.push_back(k);
      }
      return ks;
    };
    auto stage = [&](int k, int buf) {
      const int c0 = cstart[k], cn = csize[k], boff = buf * BUF;
      if (p.pairdist && ascending) {
        // the wavefronts of part s31 copy slots s31, s31 + per, ... of the chunk: channel
        // c0 + s31 + i * per, whose scalar offset is s33 = s31 * H*W*4 plus a constant
        const int per = W / p.nblk;
        const int npw = (cn + per - 1) / per;
        for (int i = 0; i < npw; i++) {
          const bool guard = (i + 1) * per > cn;
          const std::string skip = ".Ls" + std::to_string(lbl++);
          if (guard) {
            E.line("s_add_u32 s17, s31, %d", i * per);
            E.line("s_cmp_lt_u32 s17, %d", cn);
            E.line("s_cbranch_scc0 %s", skip.c_str());
          }
          E.line("s_add_u32 m0, s32, 0x%x", boff + i * per * p.chs * 4);
          E.line("s_add_u32 s12, s33, 0x%llx", (long long)(c0 + i * per) * HW4);  // m0's wait state
          E.line("%s v%d, s[4:7], s12 offen lds", dma, vB);
          E.code += 28;
          if (guard) E.label(skip);
        }
      } else if (p.pairdist) {
        // the same slots when the walk's order is not ascending: the slots' channels are not
        // affine in s31, so each part has its own code (a branch per part)
        const int per = W / p.nblk;
        for (int part = 0; part < per && part < cn; part++) {
          const std::string skip = ".Ls" + std::to_string(lbl++);
          if (per > 1) {
            E.line("s_cmp_eq_u32 s31, %d", part);
            E.line("s_cbranch_scc0 %s", skip.c_str());
          }
          for (int j = part; j < cn; j += per) {
            E.line("s_add_u32 m0, s32, 0x%x", boff + (j - part) * p.chs * 4);
            E.line("s_mov_b32 s12, 0x%llx", (long long)corder[c0 + j] * HW4);  // m0's wait state
            E.line("%s v%d, s[4:7], s12 offen lds", dma, vB);
            E.code += 28;
          }
          if (per > 1) E.label(skip);
        }
      } else {
        for (int c = 0; c < cn; c++)
          for (int k2 = 0; k2 < nvb; k2++) {
            const bool guard = (k2 + 1) * W > p.nblk;
            const std::string skip = ".Ls" + std::to_string(lbl++);
            E.line("s_add_u32 s17, s14, %d", k2 * W);
            if (guard) {
              E.line("s_cmp_lt_u32 s17, %d", p.nblk);
              E.line("s_cbranch_scc0 %s", skip.c_str());
            }
            E.line("s_mul_i32 s18, s17, %d", p.bw * 4);
            E.line("s_add_u32 m0, s18, 0x%x", boff + c * p.chs * 4);
            E.line("s_mov_b32 s12, 0x%llx", (long long)corder[c0 + c] * HW4);  // m0's wait state
            E.line("%s v%d, s[4:7], s12 offen lds", dma, vB + k2);
            E.code += 32;
            if (guard) E.label(skip);
          }
      }
    };
    // tap reads go out in batches, ra batches ahead of the FMAs, into read sets of SETW
    // registers: a batch is one step (reads from the lane's base v5 at full offsets, tap
    // column s in register s of the set), or with channel batches all steps of one channel
    // (a base register points at the channel's window: the fixed one of its chunk slot and
    // buffer, or with pb = 0 one per read set made here; pairs of taps come in one
    // ds_read2_b32, into consecutive registers in the order of the channel's taps)
    // Channel-pair batches (cb = 2): the steps of two channels a, b of the chunk; per tap used
    // by either, one ds_read2st64_b32 from the tap's base register reads it for both channels
    // (offsets: the two windows, in units of 256 bytes) into registers 2i (a) and 2i + 1 (b).
    struct Batch {
      std::vector<int> steps;   // indices into all
      std::vector<int> taps;    // channel batches: used taps r*S + s, in order
      std::vector<int> reg_of;  // channel batches: register slot of tap r*S + s (-1 unused)
      int ca = -1, cbch = -1;   // channel-pair batches: the two channels (cbch -1: one)
    };
    auto tapreg = [&](const Batch& bt, int set, int r, int sq, int c) {
      if (p.cb == 2) return vRd + set * SETW + 2 * bt.reg_of[r * S + sq] + (c == bt.ca ? 0 : 1);
      return p.cb ? vRd + set * SETW + bt.reg_of[r * S + sq] : vRd + set * SETW + sq;
    };
    // issue batch bt's reads into read set `set`; returns the LDS instructions issued
    auto reads = [&](const Batch& bt, int gi, int set, int boff, int c0) {
      const std::vector<Step>& all = alls[gi];
      const std::vector<Nz>& L = nzs[gl[gi]];
      int n = 0;
      if (p.cb == 2) {
        const int base = vRd + set * SETW;
        const int wa = boff + (rank[bt.ca] - c0) * p.chs * 4;
        for (size_t i = 0; i < bt.taps.size(); i++) {
          const int t = bt.taps[i];
          if (bt.cbch >= 0) {
            const int wb = boff + (rank[bt.cbch] - c0) * p.chs * 4;
            E.line("ds_read2st64_b32 v[%d:%d], v%d offset0:%d offset1:%d", base + 2 * (int)i, base + 2 * (int)i + 1,
                   vBase + t, wa / 256, wb / 256);
          } else {
            E.line("ds_read_b32 v%d, v%d offset:%d", base + 2 * (int)i, vBase + t, wa);
          }
          E.code += 8;
          n++;
        }
        return n;
      }
      if (p.cb) {
        const int c = all[bt.steps[0]].c;
        const int vb = npb ? vBase + boff / BUF * p.Cc + (rank[c] - c0) : vBase + set;
        if (!npb) E.v(vb, 8, fmt("v_add_u32_e32 v%d, 0x%x, v5", vb, boff + (rank[c] - c0) * p.chs * 4));
        const int base = vRd + set * SETW;
        const size_t nt = bt.taps.size();
        for (size_t i = 0; i < nt; i += 2) {
          const int t0 = bt.taps[i], o0 = (t0 / S) * g.Pp + t0 % S;
          if (i + 1 < nt) {
            const int t1 = bt.taps[i + 1], o1 = (t1 / S) * g.Pp + t1 % S;
            E.line("ds_read2_b32 v[%d:%d], v%d offset0:%d offset1:%d", base + (int)i, base + (int)i + 1,
                   vb, o0, o1);
          } else {
            E.line("ds_read_b32 v%d, v%d offset:%d", base + (int)i, vb, o0 * 4);
          }
          E.code += 8;
          n++;
        }
        return n;
      }
      const Step& st = all[bt.steps[0]];
      std::vector<char> used(S, 0);
      for (int i : st.nz) used[L[i].sq] = 1;
      for (int sidx = 0; sidx < S; sidx++) {
        if (!used[sidx]) continue;
        const int off = boff + (rank[st.c] - c0) * p.chs * 4 + (st.r * g.Pp + sidx) * 4;
        E.line("ds_read_b32 v%d, v5 offset:%d", vRd + set * SETW + sidx, off);
        E.code += 8;
        n++;
      }
      return n;
    };
    // the DMA runs P = nbuf - 1 chunks ahead: chunk i goes to buffer i % nbuf, which chunk
    // i - nbuf read before the barrier that precedes its staging
    const int nch = (int)units.size(), P = p.nbuf - 1;
    int issued = 0;
    std::vector<int> stores_at(nch, 0);  // stores issued before unit j's chunk was staged
    auto wait_for = [&](int k) {
      // unit k's chunk is in LDS once this wavefront's DMAs of it are done and every wavefront
      // has passed the barrier.  Buffer loads (LDS DMA included) and stores report completion
      // in the order they were issued, so at most the operations issued after them may still
      // be outstanding: the DMAs of later units (the fewest any wavefront issues) and the
      // stores issued since (every wavefront of a section issues the same stores)
      int later = nstores - stores_at[k];
      for (int j = k + 1; j < issued; j++) later += staged_dmas_min(p, csize[units[j].k]);
      E.line("s_waitcnt vmcnt(%d)", std::min(later, 63));
      E.line("s_barrier");
    };
    auto stage_unit = [&](int j) {
      stores_at[j] = nstores;
      stage(units[j].k, j % p.nbuf);
    };
    for (; issued < std::min(P, nch); issued++) stage_unit(issued);
    if (nch > 0) wait_for(0);
    for (int ci = 0; ci < nch; ci++) {
      const int gi = units[ci].gi;
      const std::vector<Step>& all = alls[gi];
      const std::vector<Nz>& L = nzs[gl[gi]];
      const int boff = (ci % p.nbuf) * BUF, c0 = cstart[units[ci].k];
      if (ci + P < nch) {
        stage_unit(ci + P);
        issued++;
      }
      // with early stores (ES), the stores of outputs already final: channels without a
      // non-zero in the group, channels whose last FMA was in an earlier unit (slots_at)
      if (ci == gfirst[gi]) std::fill(touched.begin(), touched.end(), 0);
      store_slots(gl[gi], slots_at(gi, ci), touched, true);
      // the unit's batches
      std::vector<Batch> bts;
      for (int t : units[ci].ts) {
        const int c = all[t].c;
        if (p.cb == 2) {
          // a new batch unless c is one of the current pair's channels or the pair has room
          const bool fits = !bts.empty() && (bts.back().ca == c || bts.back().cbch == c ||
                                             bts.back().cbch < 0);
          if (!fits) {
            bts.emplace_back();
            bts.back().reg_of.assign(g.R * S, -1);
          }
          Batch& bt = bts.back();
          if (bt.ca < 0) bt.ca = c;
          else if (bt.ca != c) bt.cbch = c;
          bt.steps.push_back(t);
          std::vector<char> used(S, 0);
          for (int i : all[t].nz) used[L[i].sq] = 1;
          for (int sq = 0; sq < S; sq++)
            if (used[sq] && bt.reg_of[all[t].r * S + sq] < 0) {
              bt.reg_of[all[t].r * S + sq] = (int)bt.taps.size();
              bt.taps.push_back(all[t].r * S + sq);
            }
          continue;
        }
        if (!p.cb || bts.empty() || all[bts.back().steps[0]].c != all[t].c) {
          bts.emplace_back();
          if (p.cb) bts.back().reg_of.assign(g.R * S, -1);
        }
        Batch& bt = bts.back();
        bt.steps.push_back(t);
        if (p.cb) {
          std::vector<char> used(S, 0);
          for (int i : all[t].nz) used[L[i].sq] = 1;
          for (int sq = 0; sq < S; sq++)
            if (used[sq]) {
              bt.reg_of[all[t].r * S + sq] = (int)bt.taps.size();
              bt.taps.push_back(all[t].r * S + sq);
            }
        }
      }
      // batch j's taps go to read set j % NS, issued ra batches ahead; before batch j's FMAs
      // only the reads of the batches after it may be outstanding
      const int nbt = (int)bts.size();
      std::vector<int> nrd(nbt, 0);
      for (int j = 0; j < std::min(p.ra, nbt); j++) nrd[j] = reads(bts[j], gi, j % NS, boff, c0);
      for (int j = 0; j < nbt; j++) {
        if (p.cb == 2) {
          // batch j's reads have landed before batch j + 1's go out (at most one batch's
          // reads, one per tap, in flight), which then overlap batch j's FMAs
          E.line("s_waitcnt lgkmcnt(0)");
          if (j + 1 < nbt) nrd[j + 1] = reads(bts[j + 1], gi, (j + 1) % NS, boff, c0);
        } else {
          if (j + p.ra < nbt) nrd[j + p.ra] = reads(bts[j + p.ra], gi, (j + p.ra) % NS, boff, c0);
          int later = 0;
          for (int k = j + 1; k < std::min(nbt, j + p.ra + 1); k++) later += nrd[k];
          E.line("s_waitcnt lgkmcnt(%d)", later);
        }
        E.code += 4;
        for (int t : bts[j].steps) {
          const Step& st = all[t];
          for (int i : st.nz) {
            const Nz& z = L[i];
            const int a = vAcc + slot_of[z.m];
            const int sr = tapreg(bts[j], j % NS, st.r, z.sq, st.c);
            if (!touched[slot_of[z.m]]) {
              touched[slot_of[z.m]] = 1;
              E.v(a, 8, fmt("v_fmamk_f32 v%d, v%d, 0x%08x, v2", a, sr, z.bits));
            } else {
              E.v(a, 8, fmt("v_fmac_f32_e32 v%d, 0x%08x, v%d", a, z.bits, sr));
            }
            fmas++;
          }
        }
      }
      const bool last = ci + 1 == nch || units[ci + 1].gi != gi;
      if (last) {
        store_slots(gl[gi], slots_at(gi, ci + 1), touched, false);
        stored[gi] = 1;
      }
      if (ci + 1 < nch) wait_for(ci + 1);
    }
    // groups without any unit (all their channels empty) store +0
    for (int gi = 0; gi < (int)gl.size(); gi++)
      if (!stored[gi]) {
        std::fill(touched.begin(), touched.end(), 0);
        std::vector<int> ks(p.rows[gl[gi]].size());
        std::iota(ks.begin(), ks.end(), 0);
        store_slots(gl[gi], ks, touched, false);
      }
    E.line("s_endpgm");
    p.sec_valu = std::max(p.sec_valu, E.valu - v0);
  }
  E.code += 1024;
  p.fmas = fmas;
  p.code_bytes = E.code;
  if (E.code > kCodeMax) {
    *err = "baked kernel code too large";
    return false;
  }
  finish_kernel(E, p, nv, W, src);
  return true;
}

bool bake_generate(const Geom& g, const std::vector<int32_t>& rowptr, const std::vector<int32_t>& col,
                   const std::vector<float>& val, BakePlan* plan, std::string* src, std::string* err) {
  BakePlan& p = *plan;
  if (p.stage) return generate_staged(g, rowptr, col, val, p, src, err);
  const int P = row_vectors(g, p.dpp);
  const int RV = g.R * P;
  const int Q = p.Q, T = p.T, WPB = p.wpb();
  int lq = 0;
  while ((1 << lq) < Q) lq++;
  // register map
  const int vOff = kFixedV;                 // RV per-row-vector input offsets
  const int vRing = vOff + RV;              // (D+1) * P loaded row vectors
  const int vSh = vRing + (p.D + 1) * P;    // P * maxsq shifted copies (two sets with perm)
  const int vAcc = (vSh + shift_regs(g, p) + 1) & ~1;  // Mg accumulators (even: 16-byte LDS writes)
  const int vTmp = vAcc;                    // prologue temporaries overlap the accumulators
  const int nv = plan_vgprs(g, p, p.Mg, p.D);
  if (nv > kMaxVgpr || vAcc + p.Mg > nv) {
    *err = "baked kernel needs more than 256 VGPRs";
    return false;
  }
  p.vgprs = nv;
  const long long HW4 = 4ll * g.H * g.W;
  const long long EF4 = 4ll * g.E * g.F;

  Emitter E;
  E.s.reserve((size_t)rowptr[g.M] * 48 + 65536);
  E.s += "\t.amdgcn_target \"amdgcn-amd-amdhsa--gfx950\"\n";
  E.s += "\t.amdhsa_code_object_version 6\n";
  E.s += "\t.text\n\t.globl sc_baked\n\t.p2align 8\n\t.type sc_baked,@function\n";
  E.label("sc_baked");
  // ---- prologue: kernel arguments, wavefront -> (unit, split), unit -> (tile, group) ----
  E.line("s_load_dwordx8 s[20:27], s[0:1], 0x0");
  E.line("s_load_dwordx2 s[28:29], s[0:1], 0x20");
  E.v(vTmp, 4, fmt("v_lshrrev_b32_e32 v%d, 6, v0", vTmp));
  E.v(1, 4, "v_and_b32_e32 v1, 63, v0");
  E.v(2, 4, "v_mov_b32_e32 v2, 0");
  E.v(3, 4, "v_bfrev_b32_e32 v3, 1");  // 0x80000000
  E.v(5, 4, "v_lshlrev_b32_e32 v5, 2, v1");
  E.rfl_guard(vTmp);
  E.v(-1, 8, fmt("v_readfirstlane_b32 s14, v%d", vTmp));
  E.line("s_waitcnt lgkmcnt(0)");
  // split q = wave % Q (s3), unit within the workgroup = wave / Q
  if ((Q & (Q - 1)) == 0) {
    E.line("s_and_b32 s3, s14, %d", Q - 1);
    E.line("s_lshr_b32 s14, s14, %d", lq);
  } else {
    // wave / Q = (wave * ceil(2^16 / Q)) >> 16, exact for wave < 16 and Q <= 16
    E.line("s_mul_i32 s3, s14, %d", (65536 + Q - 1) / Q);
    E.line("s_lshr_b32 s3, s3, 16");
    E.line("s_mul_i32 s17, s3, %d", Q);
    E.line("s_sub_u32 s17, s14, s17");
    E.line("s_mov_b32 s14, s3");
    E.line("s_mov_b32 s3, s17");
  }
  // logical workgroup: consecutive logical ids on one XCD (the grid is 8 * per_xcd)
  E.line("s_and_b32 s15, s2, 7");
  E.line("s_mul_i32 s15, s15, s29");
  E.line("s_lshr_b32 s16, s2, 3");
  E.line("s_add_u32 s15, s15, s16");
  E.line("s_mul_i32 s15, s15, %d", T);
  E.line("s_add_u32 s15, s15, s14");  // unit; units are ordered group-major
  E.line("s_mov_b32 s16, 0");
  for (int q = 0; q < p.G; q++) {
    E.line("s_cmp_lt_u32 s15, s25");
    E.line("s_cbranch_scc1 .Lunit");
    E.line("s_sub_u32 s15, s15, s25");
    E.line("s_add_u32 s16, s16, 1");
  }
  E.line("s_endpgm");
  E.label(".Lunit");
  // buffer descriptors: x in s[4:7], y in s[8:11] (raw, stride 0)
  E.line("s_mov_b32 s4, s20");
  E.line("s_and_b32 s5, s21, 0xffff");
  E.line("s_mov_b32 s6, s26");
  E.line("s_mov_b32 s7, 0x20000");
  E.line("s_mov_b32 s8, s22");
  E.line("s_and_b32 s9, s23, 0xffff");
  E.line("s_mov_b32 s10, s27");
  E.line("s_mov_b32 s11, 0x20000");
  // ---- per-lane position: q = tile*V + lane = (n*E + e)*Pb + f ----
  const int tPos = vTmp, tN = vTmp + 1, tRem = vTmp + 2, tE = vTmp + 3, tF = vTmp + 4, tIy = vTmp + 5,
            tIx = vTmp + 6, tRb = vTmp + 7, t0 = vTmp + 8, t1 = vTmp + 9, t2 = vTmp + 10;
  E.line("s_mul_i32 s17, s15, %d", p.V);
  E.v(tPos, 4, fmt("v_add_u32_e32 v%d, s17, v1", tPos));
  auto divide = [&](int dst, int num, uint32_t d, int sreg) {
    if (d == 1) {
      E.v(dst, 4, fmt("v_mov_b32_e32 v%d, v%d", dst, num));
      return;
    }
    uint32_t m;
    int l;
    bake_magic(d, &m, &l);
    E.line("s_mov_b32 s%d, 0x%x", sreg, m);
    E.v(dst, 8, fmt("v_mul_hi_u32 v%d, v%d, s%d", dst, num, sreg));
    if (l > 0) E.v(dst, 4, fmt("v_lshrrev_b32_e32 v%d, %d, v%d", dst, l, dst));
  };
  const uint32_t EPb = (uint32_t)g.E * (uint32_t)p.Pb;
  divide(tN, tPos, EPb, 17);
  E.line("s_mov_b32 s18, 0x%x", EPb);
  E.v(t0, 8, fmt("v_mul_lo_u32 v%d, v%d, s18", t0, tN));
  E.v(tRem, 4, fmt("v_sub_u32_e32 v%d, v%d, v%d", tRem, tPos, t0));
  divide(tE, tRem, (uint32_t)p.Pb, 17);
  E.line("s_mov_b32 s18, 0x%x", (uint32_t)p.Pb);
  E.v(t0, 8, fmt("v_mul_lo_u32 v%d, v%d, s18", t0, tE));
  E.v(tF, 4, fmt("v_sub_u32_e32 v%d, v%d, v%d", tF, tRem, t0));
  // iy0 = e*st - pad, ix0 = f*st - pad (32-bit two's complement)
  E.line("s_mov_b32 s18, 0x%x", (uint32_t)g.st);
  E.line("s_mov_b32 s19, 0x%x", (uint32_t)(-g.pad));
  E.v(tIy, 8, fmt("v_mul_lo_u32 v%d, v%d, s18", tIy, tE));
  E.v(tIy, 4, fmt("v_add_u32_e32 v%d, s19, v%d", tIy, tIy));
  E.v(tIx, 8, fmt("v_mul_lo_u32 v%d, v%d, s18", tIx, tF));
  E.v(tIx, 4, fmt("v_add_u32_e32 v%d, s19, v%d", tIx, tIx));
  // row base rb = n*C*H + iy0 (input word of (n, c=0, iy0, 0) divided by W)
  E.line("s_mov_b32 s18, 0x%x", (uint32_t)((uint64_t)g.C * g.H));
  E.v(t0, 8, fmt("v_mul_lo_u32 v%d, v%d, s18", t0, tN));
  E.v(tRb, 4, fmt("v_add_u32_e32 v%d, v%d, v%d", tRb, t0, tIy));
  E.line("s_mov_b32 s30, 0x%x", (uint32_t)g.H);
  E.line("s_mov_b32 s31, 0x%x", (uint32_t)g.W);
  // per row vector (r, p): offset 4*((rb + r)*W + ix0 + cp), or out of range when the input
  // row or column lies in the padding or the image is past the batch (s24 = N)
  for (int r = 0; r < g.R; r++) {
    for (int pp = 0; pp < P; pp++) {
      const int dst = vOff + r * P + pp;
      E.v(t0, 4, fmt("v_add_u32_e32 v%d, %d, v%d", t0, r, tIy));   // iy
      E.v(t1, 4, fmt("v_add_u32_e32 v%d, %d, v%d", t1, pp, tIx));  // ix
      E.cmp(fmt("v_cmp_gt_u32_e32 vcc, s30, v%d", t0));
      E.v(t2, 4, fmt("v_add_u32_e32 v%d, %d, v%d", t2, r, tRb));
      E.v(t2, 8, fmt("v_mul_lo_u32 v%d, v%d, s31", t2, t2));
      E.v(t2, 4, fmt("v_add_u32_e32 v%d, v%d, v%d", t2, t2, t1));
      E.v(t2, 4, fmt("v_lshlrev_b32_e32 v%d, 2, v%d", t2, t2));
      E.cnd(t2, fmt("v_cndmask_b32_e32 v%d, v3, v%d, vcc", t2, t2));
      E.cmp(fmt("v_cmp_gt_u32_e32 vcc, s31, v%d", t1));
      E.cnd(t2, fmt("v_cndmask_b32_e32 v%d, v3, v%d, vcc", t2, t2));
      E.cmp(fmt("v_cmp_gt_u32_e32 vcc, s24, v%d", tN));
      E.cnd(dst, fmt("v_cndmask_b32_e32 v%d, v3, v%d, vcc", dst, t2));
    }
  }
  // output offset 4*((n*M*E + e)*F + f), out of range for junk lanes (lane >= V, f >= F,
  // image past the batch)
  E.line("s_mov_b32 s18, 0x%x", (uint32_t)((uint64_t)g.M * g.E));
  E.v(t0, 8, fmt("v_mul_lo_u32 v%d, v%d, s18", t0, tN));
  E.v(t0, 4, fmt("v_add_u32_e32 v%d, v%d, v%d", t0, t0, tE));
  E.line("s_mov_b32 s18, 0x%x", (uint32_t)g.F);
  E.cmp(fmt("v_cmp_gt_u32_e32 vcc, s18, v%d", tF));
  E.v(t0, 8, fmt("v_mul_lo_u32 v%d, v%d, s18", t0, t0));
  E.v(t0, 4, fmt("v_add_u32_e32 v%d, v%d, v%d", t0, t0, tF));
  E.v(t0, 4, fmt("v_lshlrev_b32_e32 v%d, 2, v%d", t0, t0));
  E.cnd(t0, fmt("v_cndmask_b32_e32 v%d, v3, v%d, vcc", t0, t0));
  E.cmp(fmt("v_cmp_gt_u32_e32 vcc, s24, v%d", tN));
  E.cnd(t0, fmt("v_cndmask_b32_e32 v%d, v3, v%d, vcc", t0, t0));
  E.cmp(fmt("v_cmp_gt_u32_e32 vcc, %d, v1", p.V));
  E.cnd(4, fmt("v_cndmask_b32_e32 v4, v3, v%d, vcc", t0));
  // ---- select the section of (group, split): s16 * Q + s3 ----
  // (sections can lie further than a 16-bit branch offset reaches: jump with s_setpc)
  const int nsec = p.G * Q;
  if (nsec > 1) {
    E.line("s_mul_i32 s16, s16, %d", Q);
    E.line("s_add_u32 s16, s16, s3");
  }
  for (int k = 1; k < nsec; k++) {
    E.line("s_cmp_eq_u32 s16, %d", k);
    E.line("s_cbranch_scc0 .Lnot%d", k);
    E.line("s_getpc_b64 s[34:35]");
    E.label(".Lpc" + std::to_string(k));
    E.line("s_add_u32 s34, s34, .Lsec%d-.Lpc%d", k, k);
    E.line("s_addc_u32 s35, s35, 0");
    E.line("s_setpc_b64 s[34:35]");
    E.label(".Lnot" + std::to_string(k));
  }

  std::vector<int> slot_of(g.M, -1);
  for (int q = 0; q < p.G; q++)
    for (size_t i = 0; i < p.rows[q].size(); i++) slot_of[p.rows[q][i]] = (int)i;
  auto nzs = group_nonzeros(g, p.dpp, p.rows, rowptr, col, &val);
  long long fmas = 0;
  p.sec_valu = 0;
  p.sec_steps = 0;
  const long long prologue_valu = E.valu;
  for (int gq = 0; gq < p.G; gq++) {
    const std::vector<Nz>& L = nzs[gq];
    const std::vector<Step> all = group_steps(g, p.dpp, L);
    const std::vector<int> bnd = split_steps(all, Q, reduce_cost(p));
    const int nrow = (int)p.rows[gq].size();
    for (int sq_ = 0; sq_ < Q; sq_++) {
      const int sec = gq * Q + sq_;
      if (sec > 0) E.label(".Lsec" + std::to_string(sec));
      const long long v0 = E.valu;
      const int t_begin = bnd[sq_], t_end = bnd[sq_ + 1];
      const int T_ = t_end - t_begin;
      std::vector<char> touched(p.Mg, 0);
      long long cur_coff = -1;
      auto step_at = [&](int t) -> const Step& { return all[t_begin + t]; };
      auto issue_loads = [&](int t) {
        const Step& st = step_at(t);
        const long long coff = (long long)st.c * HW4;
        if (coff != cur_coff) {
          E.line("s_mov_b32 s12, 0x%llx", coff);
          cur_coff = coff;
        }
        const int slot = t % (p.D + 1);
        for (int pv = 0; pv < P; pv++) {
          if (!(st.used >> pv & 1ull)) continue;
          E.line("buffer_load_dword v%d, v%d, s[4:7], s12 offen", vRing + slot * P + pv, vOff + st.r * P + pv);
          E.wr[vRing + slot * P + pv] = E.valu;  // a DPP read needs 2 wait states after the issue
          E.code += 8;
        }
      };
      for (int t = 0; t < std::min(T_, p.D); t++) issue_loads(t);
      // FMAs of step t at shift level lvl (0: the loaded row vector)
      size_t nzi = 0;
      auto emit_fmas = [&](int t, int lvl, const std::function<int(int, int)>& src_reg) {
        const Step& st = step_at(t);
        for (; nzi < st.nz.size() && L[st.nz[nzi]].sq == lvl; nzi++) {
          const Nz& z = L[st.nz[nzi]];
          const int a = vAcc + slot_of[z.m];
          const int sr = src_reg(z.pv, z.sq);
          if (!touched[slot_of[z.m]]) {
            touched[slot_of[z.m]] = 1;
            E.v(a, 8, fmt("v_fmamk_f32 v%d, v%d, 0x%08x, v2", a, sr, z.bits));
          } else {
            E.v(a, 8, fmt("v_fmac_f32_e32 v%d, 0x%08x, v%d", a, z.bits, sr));
          }
          fmas++;
        }
      };
      auto loads_between = [&](int u0, int u1) {
        int n = 0;
        for (int u = u0; u < std::min(T_, u1); u++) n += step_at(u).loads();
        return n;
      };
      if (p.perm) {
        // Lane shifts through the LDS crossbar: the copy of row vector pv shifted down by sq
        // lanes is ds_bpermute_b32 with lane address 4*lane + 4*sq (v5 + offset; lanes past
        // 63 wrap and are junk).  The shifts of step t + 1 are issued before the FMAs of step
        // t, into the other set of shift registers, so their latency hides behind step t.
        auto sh_reg = [&](int t, int pv, int sq) { return vSh + ((t & 1) * P + pv) * p.maxsq + (sq - 1); };
        auto issue_shifts = [&](int t) {
          const Step& st = step_at(t);
          const int slot = t % (p.D + 1);
          int n = 0;
          for (int pv = 0; pv < P; pv++)
            for (int sq = 1; sq <= st.sqmax[pv]; sq++) {
              E.line("ds_bpermute_b32 v%d, v5, v%d offset:%d", sh_reg(t, pv, sq), vRing + slot * P + pv, 4 * sq);
              E.code += 8;
              n++;
            }
          return n;
        };
        if (T_ > 0) {
          E.line("s_waitcnt vmcnt(%d)", loads_between(1, p.D));
          E.code += 4;
          issue_shifts(0);
        }
        for (int t = 0; t < T_; t++) {
          const Step& st = step_at(t);
          const int slot = t % (p.D + 1);
          int next = 0;
          if (t + 1 < T_) {
            E.line("s_waitcnt vmcnt(%d)", loads_between(t + 2, t + p.D));
            E.code += 4;
          }
          if (t + p.D < T_) issue_loads(t + p.D);
          if (t + 1 < T_) next = issue_shifts(t + 1);
          auto src_reg = [&](int pv, int sq) { return sq == 0 ? vRing + slot * P + pv : sh_reg(t, pv, sq); };
          nzi = 0;
          emit_fmas(t, 0, src_reg);
          int maxlvl = 0;
          for (int pv = 0; pv < P; pv++) maxlvl = std::max(maxlvl, st.sqmax[pv]);
          if (maxlvl > 0) {
            E.line("s_waitcnt lgkmcnt(%d)", next);  // this step's shifts have arrived
            E.code += 4;
          }
          for (int lvl = 1; lvl <= maxlvl; lvl++) emit_fmas(t, lvl, src_reg);
        }
      } else {
        for (int t = 0; t < T_; t++) {
          const Step& st = step_at(t);
          E.line("s_waitcnt vmcnt(%d)", loads_between(t + 1, t + p.D));
          E.code += 4;
          if (t + p.D < T_) issue_loads(t + p.D);
          const int slot = t % (p.D + 1);
          // DPP lane shifts and FMAs, level by level: shift level k reads level k-1 (a VALU
          // result, hence the wait states), FMAs of level k-1 fill the gap
          auto src_reg = [&](int pv, int sq) {
            return sq == 0 ? vRing + slot * P + pv : vSh + pv * p.maxsq + (sq - 1);
          };
          nzi = 0;
          int maxlvl = 0;
          for (int pv = 0; pv < P; pv++) maxlvl = std::max(maxlvl, st.sqmax[pv]);
          for (int lvl = 0; lvl <= maxlvl; lvl++) {
            if (lvl > 0) {
              for (int pv = 0; pv < P; pv++) {
                if (st.sqmax[pv] < lvl) continue;
                const int s_reg = src_reg(pv, lvl - 1), d_reg = src_reg(pv, lvl);
                E.dpp_guard(s_reg);
                E.v(d_reg, 8, fmt("v_mov_b32_dpp v%d, v%d wave_shl:1 row_mask:0xf bank_mask:0xf", d_reg, s_reg));
              }
            }
            emit_fmas(t, lvl, src_reg);
          }
        }
      }
      // accumulators without a non-zero in this section hold +0
      const int nacc = Q > 1 ? p.Mg : nrow;
      for (int k = 0; k < nacc; k++)
        if (!touched[k]) E.v(vAcc + k, 4, fmt("v_mov_b32_e32 v%d, 0", vAcc + k));
      if (Q > 1) {
        // Reduce-scatter of the partial sums through LDS, in rounds of KC channels: block k4
        // (channels 4 k4 .. 4 k4 + 3) belongs to split k4 % Q.  Each round every split writes
        // the blocks the others own (16 bytes per lane and block, its own part of the unit's
        // LDS), barrier; each split adds the Q partial sums of its own blocks in split order,
        // ((p0 + p1) + ...) + p(Q-1), barrier.  Every split then stores its own blocks.  The
        // lane's byte address in the unit's LDS lives in the first row-vector offset register,
        // dead once the last load is issued; the rest of the offset, ring and shift registers
        // hold the partial sums read.
        const int KC = p.rc;
        const int kbr = (KC / 4) * 1024;  // bytes of one split's part per round
        const int rounds = (p.Mg + KC - 1) / KC;
        const int va = vOff;
        E.line("s_mul_i32 s17, s14, %d", Q * kbr);
        E.v(va, 4, fmt("v_lshlrev_b32_e32 v%d, 4, v1", va));
        E.v(va, 4, fmt("v_add_u32_e32 v%d, s17, v%d", va, va));
        const int t0r = (vOff + 2) & ~1;  // even-aligned temporaries
        const int ntmp = std::min(16, (vAcc - t0r) / 4);
        if (ntmp < Q - 1) {
          *err = "too few free registers for the channel-split reduction";
          return false;
        }
        const int bpb = ntmp / (Q - 1);  // own blocks per batch of reads
        const int vb = vOff + 1;                       // base register of a batch of reads
        for (int j = 0; j < rounds; j++) {
          const int k40 = j * KC / 4, k41 = std::min(p.Mg, (j + 1) * KC) / 4;
          const bool last = j + 1 == rounds;
          for (int k4 = k40; k4 < k41; k4++)
            if (k4 % Q != sq_)
              E.line("ds_write_b128 v%d, v[%d:%d] offset:%d", va, vAcc + 4 * k4, vAcc + 4 * k4 + 3,
                     sq_ * kbr + (k4 - k40) * 1024);
          E.line("s_waitcnt lgkmcnt(0)");
          E.line("s_barrier");
          std::vector<int> mine;
          for (int k4 = k40; k4 < k41; k4++)
            if (k4 % Q == sq_) mine.push_back(k4);
          for (size_t m0 = 0; m0 < mine.size(); m0 += bpb) {
            const size_t m1 = std::min(mine.size(), m0 + bpb);
            // the other splits' parts of these blocks: temporary block i holds part q of own
            // block m, in (block, split) order
            auto off = [&](int k4, int q) { return q * kbr + (k4 - k40) * 1024; };
            const int first = off(mine[m0], sq_ == 0 ? 1 : 0);
            E.v(vb, 8, fmt("v_add_u32_e32 v%d, 0x%x, v%d", vb, first, va));
            std::vector<int> tmp_of;  // per (block, q): temporary block index, -1 for the own part
            int nt = 0;
            for (size_t m = m0; m < m1; m++)
              for (int q = 0; q < Q; q++) {
                if (q == sq_) {
                  tmp_of.push_back(-1);
                  continue;
                }
                E.line("ds_read_b128 v[%d:%d], v%d offset:%d", t0r + 4 * nt, t0r + 4 * nt + 3, vb,
                       off(mine[m], q) - first);
                tmp_of.push_back(nt++);
              }
            E.line("s_waitcnt lgkmcnt(0)");
            for (size_t m = m0; m < m1; m++) {
              const int k4 = mine[m];
              const int* to = &tmp_of[(m - m0) * Q];
              for (int jj = 0; jj < 4; jj++) {
                const int acc = vAcc + 4 * k4 + jj;
                auto part = [&](int q) { return to[q] < 0 ? acc : t0r + 4 * to[q] + jj; };
                if (sq_ == 0) {
                  for (int q = 1; q < Q; q++) E.v(acc, 4, fmt("v_add_f32_e32 v%d, v%d, v%d", acc, acc, part(q)));
                } else {
                  // prefix p0 + ... + p(sq-1) in part 0's temporary, then the own part, then the rest
                  const int pre = part(0);
                  for (int q = 1; q < sq_; q++) E.v(pre, 4, fmt("v_add_f32_e32 v%d, v%d, v%d", pre, pre, part(q)));
                  E.v(acc, 4, fmt("v_add_f32_e32 v%d, v%d, v%d", acc, pre, acc));
                  for (int q = sq_ + 1; q < Q; q++) E.v(acc, 4, fmt("v_add_f32_e32 v%d, v%d, v%d", acc, acc, part(q)));
                }
              }
            }
          }
          if (!last) E.line("s_barrier");  // every split has read this round's parts
        }
      }
      for (int k = 0; k < nrow; k++) {
        if (Q > 1 && (k / 4) % Q != sq_) continue;
        E.line("s_mov_b32 s13, 0x%llx", (long long)p.rows[gq][k] * EF4);
        E.line("buffer_store_dword v%d, v4, s[8:11], s13 offen", vAcc + k);
        E.code += 16;
      }
      E.line("s_endpgm");
      p.sec_valu = std::max(p.sec_valu, E.valu - v0);
      p.sec_steps = std::max<long long>(p.sec_steps, T_);
    }
  }
  (void)prologue_valu;
  E.code += 512;  // prologue (approximate)
  p.fmas = fmas;
  p.code_bytes = E.code;
  if (E.code > kCodeMax) {
    *err = "baked kernel code too large";
    return false;
  }
  finish_kernel(E, p, nv, WPB, src);
  return true;
}

bool bake_assemble(const std::string& src, std::vector<char>* elf, std::string* err) {
  amd_comgr_data_t d{};
  amd_comgr_data_set_t in{}, rel{}, exe{};
  amd_comgr_action_info_t ai{};
  bool ok = false;
  std::string log;
  auto get_logs = [&](amd_comgr_data_set_t set) {
    size_t n = 0;
    if (amd_comgr_action_data_count(set, AMD_COMGR_DATA_KIND_LOG, &n) != AMD_COMGR_STATUS_SUCCESS) return;
    for (size_t i = 0; i < n; i++) {
      amd_comgr_data_t l;
      if (amd_comgr_action_data_get_data(set, AMD_COMGR_DATA_KIND_LOG, i, &l) != AMD_COMGR_STATUS_SUCCESS) continue;
      size_t sz = 0;
      if (amd_comgr_get_data(l, &sz, nullptr) == AMD_COMGR_STATUS_SUCCESS && sz) {
        std::string s(sz, '\0');
        amd_comgr_get_data(l, &sz, &s[0]);
        log += s;
      }
      amd_comgr_release_data(l);
    }
  };
  do {
    if (amd_comgr_create_data(AMD_COMGR_DATA_KIND_SOURCE, &d) != AMD_COMGR_STATUS_SUCCESS) break;
    if (amd_comgr_set_data(d, src.size(), src.data()) != AMD_COMGR_STATUS_SUCCESS) break;
    if (amd_comgr_set_data_name(d, "sc_baked.s") != AMD_COMGR_STATUS_SUCCESS) break;
    if (amd_comgr_create_data_set(&in) != AMD_COMGR_STATUS_SUCCESS) break;
    if (amd_comgr_create_data_set(&rel) != AMD_COMGR_STATUS_SUCCESS) break;
    if (amd_comgr_create_data_set(&exe) != AMD_COMGR_STATUS_SUCCESS) break;
    if (amd_comgr_data_set_add(in, d) != AMD_COMGR_STATUS_SUCCESS) break;
    if (amd_comgr_create_action_info(&ai) != AMD_COMGR_STATUS_SUCCESS) break;
    if (amd_comgr_action_info_set_isa_name(ai, "amdgcn-amd-amdhsa--gfx950") != AMD_COMGR_STATUS_SUCCESS) break;
    amd_comgr_action_info_set_logging(ai, true);
    if (amd_comgr_do_action(AMD_COMGR_ACTION_ASSEMBLE_SOURCE_TO_RELOCATABLE, ai, in, rel) != AMD_COMGR_STATUS_SUCCESS) {
      get_logs(rel);
      log = "assembly failed: " + log;
      break;
    }
    if (amd_comgr_do_action(AMD_COMGR_ACTION_LINK_RELOCATABLE_TO_EXECUTABLE, ai, rel, exe) != AMD_COMGR_STATUS_SUCCESS) {
      get_logs(exe);
      log = "link failed: " + log;
      break;
    }
    size_t n = 0;
    if (amd_comgr_action_data_count(exe, AMD_COMGR_DATA_KIND_EXECUTABLE, &n) != AMD_COMGR_STATUS_SUCCESS || n != 1)
      break;
    amd_comgr_data_t e;
    if (amd_comgr_action_data_get_data(exe, AMD_COMGR_DATA_KIND_EXECUTABLE, 0, &e) != AMD_COMGR_STATUS_SUCCESS) break;
    size_t sz = 0;
    if (amd_comgr_get_data(e, &sz, nullptr) == AMD_COMGR_STATUS_SUCCESS) {
      elf->resize(sz);
      ok = amd_comgr_get_data(e, &sz, elf->data()) == AMD_COMGR_STATUS_SUCCESS;
    }
    amd_comgr_release_data(e);
  } while (false);
  if (ai.handle) amd_comgr_destroy_action_info(ai);
  if (exe.handle) amd_comgr_destroy_data_set(exe);
  if (rel.handle) amd_comgr_destroy_data_set(rel);
  if (in.handle) amd_comgr_destroy_data_set(in);
  if (d.handle) amd_comgr_release_data(d);
  if (!ok) *err = log.empty() ? "amd_comgr failed" : log;
  return ok;
}

}  // namespace sc
