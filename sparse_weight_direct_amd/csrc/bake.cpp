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
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <numeric>

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
  f.D = env_key(e, "D", -1);
  f.dpp = env_key(e, "DPP", -1);
  f.WPB = env_key(e, "WPB", -1);
  return f;
}

namespace {

constexpr int kMaxVgpr = 256;   // architectural VGPRs a VALU instruction can name
constexpr int kFixedV = 5;      // v0 id, v1 lane, v2 zero, v3 out-of-range marker, v4 output offset
constexpr int kTemps = 12;      // prologue temporaries
constexpr long long kCodeMax = 4ll << 20;  // refuse kernels above 4 MB of code

// Row vectors of one filter row: the stride phases of the filter columns (lane shifts give
// the other columns), or every column when lane shifts are off.
inline int row_vectors(const Geom& g, int dpp) { return dpp ? std::min(g.st, g.S) : g.S; }

struct Step {
  int c, r;
  uint64_t used;    // bit p: row vector p of this step is read by some non-zero
  int sqmax[64];    // per row vector: largest lane shift read (-1 unused)
  std::vector<int> nz;  // indices (into the sorted non-zero list) of the step's non-zeros
};

}  // namespace

bool bake_choose(const Geom& g, const std::vector<int32_t>& rowptr, const std::vector<int32_t>& col,
                 const BakeForce& f, BakePlan* plan, std::string* why) {
  const int M = g.M;
  BakePlan p;
  p.dpp = f.dpp >= 0 ? f.dpp : 1;
  if (row_vectors(g, p.dpp) > 32) {
    *why = "more than 32 row vectors per filter row";
    return false;
  }
  p.maxsq = p.dpp ? (g.S - 1) / g.st : 0;
  if (p.maxsq >= 32) {
    *why = "filter reach too wide for lane shifts";
    return false;
  }
  p.V = 64 - p.maxsq;
  p.Pb = g.F + p.maxsq;
  p.WPB = f.WPB > 0 ? f.WPB : 4;
  const int P = row_vectors(g, p.dpp);
  const int RV = g.R * P;
  // registers besides the accumulators: fixed, per-row-vector offsets, the shifted copies
  // of one step; the load ring takes (D+1)*P.  Target at most 168 (three wavefronts per
  // SIMD) with at least two steps in flight, else up to 256.
  const int base = kFixedV + RV + P * p.maxsq;
  const long long nnz = rowptr[M];
  long long steps_total = 0;
  {
    std::vector<char> seen((size_t)g.C * g.R, 0);
    for (int j = 0; j < (int)nnz; j++) {
      const int c = col[j] / (g.R * g.S), r = (col[j] / g.S) % g.R;
      if (!seen[(size_t)c * g.R + r]) {
        seen[(size_t)c * g.R + r] = 1;
        steps_total++;
      }
    }
  }
  int G = f.G > 0 ? f.G : 0;
  if (G == 0) {
    // the fewest groups that keep a group's accumulators in registers and its code within
    // the 64 KB instruction cache a pair of CUs shares (a group's waves run one section)
    for (G = 1; G <= M; G++) {
      const int mg = (M + G - 1) / G;
      const long long code = nnz / G * 8 + steps_total * (8 + P * 8 + P * p.maxsq * 8) + mg * 16 + 2048;
      if (base + mg + 2 * P <= 168 && code <= 56 * 1024) break;
      if (base + mg + 2 * P <= 168 && G >= 8) break;
    }
    if (G > M) G = M;
  }
  const int mg = (M + G - 1) / G;
  if (base + mg + 2 * P > kMaxVgpr - 4) {
    *why = "output channels per group exceed the registers";
    return false;
  }
  int D = f.D > 0 ? f.D : 0;
  const int budget = (base + mg + 2 * P <= 168) ? 168 : kMaxVgpr - 4;
  if (D == 0) {
    D = (budget - base - mg) / P - 1;
    D = std::min(D, std::max(1, 63 / P));
    D = std::min(D, 16);
    D = std::max(D, 1);
  }
  if (D * P > 63 || base + mg + (D + 1) * P > kMaxVgpr - 4) {
    *why = "load ring does not fit";
    return false;
  }
  p.G = G;
  p.D = D;
  // rows to groups: largest first onto the least-loaded group with room (balance by
  // non-zeros, at most mg rows per group)
  std::vector<int> order(M);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return rowptr[a + 1] - rowptr[a] > rowptr[b + 1] - rowptr[b]; });
  p.rows.assign(G, {});
  std::vector<long long> load(G, 0);
  for (int m : order) {
    int best = -1;
    for (int q = 0; q < G; q++) {
      if ((int)p.rows[q].size() >= mg) continue;
      if (best < 0 || load[q] < load[best]) best = q;
    }
    p.rows[best].push_back(m);
    load[best] += rowptr[m + 1] - rowptr[m];
  }
  for (auto& r : p.rows) std::sort(r.begin(), r.end());
  *plan = p;
  return true;
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

struct Emitter {
  std::string s;
  long long valu = 0;                 // VALU instructions (and nop wait states) issued
  std::vector<long long> wr;          // per VGPR: index of its last VALU write
  long long code = 0;                 // bytes
  Emitter() : wr(kMaxVgpr, -100) {}
  void line(const char* fmt, ...) __attribute__((format(printf, 2, 3))) {
    char buf[256];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
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
  // a v_cmp writing VCC
  void cmp(const char* text) {
    line("%s", text);
    vcc_wr = valu;
    valu_op(-1, 4);
  }
  // a v_cndmask reading VCC
  void cnd(int d, const char* text) {
    vcc_guard();
    line("%s", text);
    valu_op(d, 4);
  }
};

}  // namespace

bool bake_generate(const Geom& g, const std::vector<int32_t>& rowptr, const std::vector<int32_t>& col,
                   const std::vector<float>& val, BakePlan* plan, std::string* src, std::string* err) {
  BakePlan& p = *plan;
  const int P = row_vectors(g, p.dpp);
  const int RV = g.R * P;
  const int RS = g.R * g.S;
  const int mg = 0 == p.G ? 0 : (int)std::max_element(p.rows.begin(), p.rows.end(),
                                                       [](const std::vector<int>& a, const std::vector<int>& b) {
                                                         return a.size() < b.size();
                                                       })->size();
  // register map
  const int vOff = kFixedV;                 // RV per-row-vector input offsets
  const int vRing = vOff + RV;              // (D+1) * P loaded row vectors
  const int vSh = vRing + (p.D + 1) * P;    // P * maxsq shifted copies
  const int vAcc = vSh + P * p.maxsq;       // mg accumulators
  const int vTmp = vAcc;                    // prologue temporaries overlap the accumulators
  const int nv = (std::max(vAcc + mg, vTmp + kTemps) + 3) & ~3;  // granule of the unified register file
  if (nv > kMaxVgpr) {
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
  // ---- prologue: kernel arguments, unit -> (tile, group) ----
  E.line("s_load_dwordx8 s[20:27], s[0:1], 0x0");
  E.line("s_load_dwordx2 s[28:29], s[0:1], 0x20");
  E.line("v_lshrrev_b32_e32 v%d, 6, v0", vTmp);
  E.valu_op(vTmp, 4);
  E.line("v_and_b32_e32 v1, 63, v0");
  E.valu_op(1, 4);
  E.line("v_mov_b32_e32 v2, 0");
  E.valu_op(2, 4);
  E.line("v_bfrev_b32_e32 v3, 1");  // 0x80000000
  E.valu_op(3, 4);
  E.rfl_guard(vTmp);
  E.line("v_readfirstlane_b32 s14, v%d", vTmp);
  E.valu_op(-1, 8);
  E.line("s_waitcnt lgkmcnt(0)");
  // logical workgroup: consecutive logical ids on one XCD (the grid is 8 * per_xcd)
  E.line("s_and_b32 s15, s2, 7");
  E.line("s_mul_i32 s15, s15, s29");
  E.line("s_lshr_b32 s16, s2, 3");
  E.line("s_add_u32 s15, s15, s16");
  E.line("s_mul_i32 s15, s15, %d", p.WPB);
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
  E.line("v_add_u32_e32 v%d, s17, v1", tPos);
  E.valu_op(tPos, 4);
  auto divide = [&](int dst, int num, uint32_t d, int sreg) {
    if (d == 1) {
      E.line("v_mov_b32_e32 v%d, v%d", dst, num);
      E.valu_op(dst, 4);
      return;
    }
    uint32_t m;
    int l;
    bake_magic(d, &m, &l);
    E.line("s_mov_b32 s%d, 0x%x", sreg, m);
    E.line("v_mul_hi_u32 v%d, v%d, s%d", dst, num, sreg);
    E.valu_op(dst, 8);
    if (l > 0) {
      E.line("v_lshrrev_b32_e32 v%d, %d, v%d", dst, l, dst);
      E.valu_op(dst, 4);
    }
  };
  const uint32_t EPb = (uint32_t)g.E * (uint32_t)p.Pb;
  divide(tN, tPos, EPb, 17);
  E.line("s_mov_b32 s18, 0x%x", EPb);
  E.line("v_mul_lo_u32 v%d, v%d, s18", t0, tN);
  E.valu_op(t0, 8);
  E.line("v_sub_u32_e32 v%d, v%d, v%d", tRem, tPos, t0);
  E.valu_op(tRem, 4);
  divide(tE, tRem, (uint32_t)p.Pb, 17);
  E.line("s_mov_b32 s18, 0x%x", (uint32_t)p.Pb);
  E.line("v_mul_lo_u32 v%d, v%d, s18", t0, tE);
  E.valu_op(t0, 8);
  E.line("v_sub_u32_e32 v%d, v%d, v%d", tF, tRem, t0);
  E.valu_op(tF, 4);
  // iy0 = e*st - pad, ix0 = f*st - pad (32-bit two's complement)
  E.line("s_mov_b32 s18, 0x%x", (uint32_t)g.st);
  E.line("s_mov_b32 s19, 0x%x", (uint32_t)(-g.pad));
  E.line("v_mul_lo_u32 v%d, v%d, s18", tIy, tE);
  E.valu_op(tIy, 8);
  E.line("v_add_u32_e32 v%d, s19, v%d", tIy, tIy);
  E.valu_op(tIy, 4);
  E.line("v_mul_lo_u32 v%d, v%d, s18", tIx, tF);
  E.valu_op(tIx, 8);
  E.line("v_add_u32_e32 v%d, s19, v%d", tIx, tIx);
  E.valu_op(tIx, 4);
  // row base rb = n*C*H + iy0 (input word of (n, c=0, iy0, 0) divided by W)
  E.line("s_mov_b32 s18, 0x%x", (uint32_t)((uint64_t)g.C * g.H));
  E.line("v_mul_lo_u32 v%d, v%d, s18", t0, tN);
  E.valu_op(t0, 8);
  E.line("v_add_u32_e32 v%d, v%d, v%d", tRb, t0, tIy);
  E.valu_op(tRb, 4);
  E.line("s_mov_b32 s30, 0x%x", (uint32_t)g.H);   // H
  E.line("s_mov_b32 s31, 0x%x", (uint32_t)g.W);   // W
  // s24 = N (kernel argument)
  // per row vector (r, p): offset 4*((rb + r)*W + ix0 + cp), or out of range when the input
  // row or column lies in the padding or the image is past the batch
  for (int r = 0; r < g.R; r++) {
    for (int pp = 0; pp < P; pp++) {
      const int cp = pp;  // column offset: stride phase sp (lane shifts) or the column s
      const int dst = vOff + r * P + pp;
      E.line("v_add_u32_e32 v%d, %d, v%d", t0, r, tIy);  // iy
      E.valu_op(t0, r <= 64 ? 4 : 8);
      E.line("v_add_u32_e32 v%d, %d, v%d", t1, cp, tIx);  // ix
      E.valu_op(t1, cp <= 64 ? 4 : 8);
      E.line("v_add_u32_e32 v%d, %d, v%d", t2, r, tRb);
      E.valu_op(t2, r <= 64 ? 4 : 8);
      E.line("v_mul_lo_u32 v%d, v%d, s31", t2, t2);
      E.valu_op(t2, 8);
      E.line("v_add_u32_e32 v%d, v%d, v%d", t2, t2, t1);
      E.valu_op(t2, 4);
      E.line("v_lshlrev_b32_e32 v%d, 2, v%d", t2, t2);
      E.valu_op(t2, 4);
      E.cmp(fmt("v_cmp_gt_u32_e32 vcc, s30, v%d", t0).c_str());
      E.cnd(t2, fmt("v_cndmask_b32_e32 v%d, v3, v%d, vcc", t2, t2).c_str());
      E.cmp(fmt("v_cmp_gt_u32_e32 vcc, s31, v%d", t1).c_str());
      E.cnd(t2, fmt("v_cndmask_b32_e32 v%d, v3, v%d, vcc", t2, t2).c_str());
      E.cmp(fmt("v_cmp_gt_u32_e32 vcc, s24, v%d", tN).c_str());
      E.cnd(dst, fmt("v_cndmask_b32_e32 v%d, v3, v%d, vcc", dst, t2).c_str());
    }
  }
  // output offset 4*((n*M*E + e)*F + f), out of range for junk lanes (lane >= V, f >= F,
  // image past the batch)
  E.line("s_mov_b32 s18, 0x%x", (uint32_t)((uint64_t)g.M * g.E));
  E.line("v_mul_lo_u32 v%d, v%d, s18", t0, tN);
  E.valu_op(t0, 8);
  E.line("v_add_u32_e32 v%d, v%d, v%d", t0, t0, tE);
  E.valu_op(t0, 4);
  E.line("s_mov_b32 s18, 0x%x", (uint32_t)g.F);
  E.line("v_mul_lo_u32 v%d, v%d, s18", t0, t0);
  E.valu_op(t0, 8);
  E.line("v_add_u32_e32 v%d, v%d, v%d", t0, t0, tF);
  E.valu_op(t0, 4);
  E.line("v_lshlrev_b32_e32 v%d, 2, v%d", t0, t0);
  E.valu_op(t0, 4);
  E.cmp(fmt("v_cmp_gt_u32_e32 vcc, s18, v%d", tF).c_str());
  E.cnd(t0, fmt("v_cndmask_b32_e32 v%d, v3, v%d, vcc", t0, t0).c_str());
  E.cmp(fmt("v_cmp_gt_u32_e32 vcc, s24, v%d", tN).c_str());
  E.cnd(t0, fmt("v_cndmask_b32_e32 v%d, v3, v%d, vcc", t0, t0).c_str());
  E.cmp(fmt("v_cmp_gt_u32_e32 vcc, %d, v1", p.V).c_str());
  E.cnd(4, fmt("v_cndmask_b32_e32 v4, v3, v%d, vcc", t0).c_str());
  // ---- select the group's section ----
  // (sections can lie further than a 16-bit branch offset reaches: jump with s_setpc)
  for (int q = 1; q < p.G; q++) {
    E.line("s_cmp_eq_u32 s16, %d", q);
    E.line("s_cbranch_scc0 .Lnot%d", q);
    E.line("s_getpc_b64 s[34:35]");
    E.label(".Lpc" + std::to_string(q));
    E.line("s_add_u32 s34, s34, .Lsec%d-.Lpc%d", q, q);
    E.line("s_addc_u32 s35, s35, 0");
    E.line("s_setpc_b64 s[34:35]");
    E.label(".Lnot" + std::to_string(q));
  }

  // non-zeros sorted by (c, r, lane shift, phase, row) so a step's FMAs are contiguous and
  // consecutive FMAs mostly hit different accumulators
  struct Nz {
    int m, c, r, pv, sq;
    uint32_t bits;
  };
  std::vector<int> group_of(g.M, -1), slot_of(g.M, -1);
  for (int q = 0; q < p.G; q++)
    for (size_t i = 0; i < p.rows[q].size(); i++) {
      group_of[p.rows[q][i]] = q;
      slot_of[p.rows[q][i]] = (int)i;
    }
  std::vector<std::vector<Nz>> nzs(p.G);
  for (int m = 0; m < g.M; m++)
    for (int j = rowptr[m]; j < rowptr[m + 1]; j++) {
      const int c = col[j] / RS, r = (col[j] / g.S) % g.R, s = col[j] % g.S;
      Nz z;
      z.m = m;
      z.c = c;
      z.r = r;
      z.pv = p.dpp ? s % g.st : s;
      z.sq = p.dpp ? s / g.st : 0;
      std::memcpy(&z.bits, &val[j], 4);
      nzs[group_of[m]].push_back(z);
    }
  long long fmas = 0;
  for (int q = 0; q < p.G; q++) {
    std::vector<Nz>& L = nzs[q];
    std::stable_sort(L.begin(), L.end(), [](const Nz& a, const Nz& b) {
      if (a.c != b.c) return a.c < b.c;
      if (a.r != b.r) return a.r < b.r;
      if (a.sq != b.sq) return a.sq < b.sq;
      if (a.pv != b.pv) return a.pv < b.pv;
      return a.m < b.m;
    });
    // steps: runs of equal (c, r)
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
    if (q > 0) E.label(".Lsec" + std::to_string(q));
    std::vector<char> touched(p.rows[q].size(), 0);
    const int T = (int)steps.size();
    long long cur_coff = -1;
    auto issue_loads = [&](int t) {
      const Step& st = steps[t];
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
    auto nloads = [&](int t) {
      int n = 0;
      for (int pv = 0; pv < P; pv++) n += (int)(steps[t].used >> pv & 1ull);
      return n;
    };
    for (int t = 0; t < std::min(T, p.D); t++) issue_loads(t);
    for (int t = 0; t < T; t++) {
      const Step& st = steps[t];
      int after = 0;
      for (int u = t + 1; u < std::min(T, t + p.D); u++) after += nloads(u);
      E.line("s_waitcnt vmcnt(%d)", after);
      E.code += 4;
      if (t + p.D < T) issue_loads(t + p.D);
      const int slot = t % (p.D + 1);
      // lane shifts and FMAs, level by level: shift level k reads level k-1 (a VALU
      // result, hence the wait states), FMAs of level k-1 fill the gap
      auto src_reg = [&](int pv, int sq) { return sq == 0 ? vRing + slot * P + pv : vSh + pv * p.maxsq + (sq - 1); };
      size_t i = 0;
      int maxlvl = 0;
      for (int pv = 0; pv < P; pv++) maxlvl = std::max(maxlvl, st.sqmax[pv]);
      for (int lvl = 0; lvl <= maxlvl; lvl++) {
        if (lvl > 0) {
          for (int pv = 0; pv < P; pv++) {
            if (st.sqmax[pv] < lvl) continue;
            const int s_reg = src_reg(pv, lvl - 1), d_reg = src_reg(pv, lvl);
            E.dpp_guard(s_reg);
            E.line("v_mov_b32_dpp v%d, v%d wave_shl:1 row_mask:0xf bank_mask:0xf", d_reg, s_reg);
            E.valu_op(d_reg, 8);
          }
        }
        for (; i < st.nz.size() && L[st.nz[i]].sq == lvl; i++) {
          const Nz& z = L[st.nz[i]];
          const int a = vAcc + slot_of[z.m];
          const int sr = src_reg(z.pv, z.sq);
          if (!touched[slot_of[z.m]]) {
            touched[slot_of[z.m]] = 1;
            E.line("v_fmamk_f32 v%d, v%d, 0x%08x, v2", a, sr, z.bits);
          } else {
            E.line("v_fmac_f32_e32 v%d, 0x%08x, v%d", a, z.bits, sr);
          }
          E.valu_op(a, 8);
          fmas++;
        }
      }
    }
    // stores: output channels without a non-zero in this group hold +0
    for (size_t k = 0; k < p.rows[q].size(); k++) {
      if (!touched[k]) {
        E.line("v_mov_b32_e32 v%d, 0", vAcc + (int)k);
        E.valu_op(vAcc + (int)k, 4);
      }
    }
    for (size_t k = 0; k < p.rows[q].size(); k++) {
      E.line("s_mov_b32 s13, 0x%llx", (long long)p.rows[q][k] * EF4);
      E.line("buffer_store_dword v%d, v4, s[8:11], s13 offen", vAcc + (int)k);
      E.code += 16;
    }
    E.line("s_endpgm");
  }
  E.code += 512;  // prologue (approximate)
  p.fmas = fmas;
  p.code_bytes = E.code;
  if (E.code > kCodeMax) {
    *err = "baked kernel code too large";
    return false;
  }
  p.sgprs = 40;
  char kd[2048];
  snprintf(kd, sizeof kd,
           "\t.section .rodata,\"a\",@progbits\n"
           "\t.p2align 6, 0x0\n"
           "\t.amdhsa_kernel sc_baked\n"
           "\t\t.amdhsa_group_segment_fixed_size 0\n"
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
           nv, p.sgprs, nv);
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
           "    .group_segment_fixed_size: 0\n"
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
           p.WPB * 64, p.sgprs + 6, nv);
  E.s += md;
  *src = std::move(E.s);
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
