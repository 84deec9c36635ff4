// C ABI of the sparse direct convolution library (declared in include/sparseconv.h).
//
// sparseconv_pack: validate -> CSR rows ("Escoin", CSR section; columns sorted within a row,
// values moved with them) -> stretched u32 input offsets c*H*W + r*W + s ("Escoin", weight
// stretching) kept as the canonical host copy -> (with SC_PACK_FP16_WORD) the 32-bit packed
// words of Tuteja et al., Sec. 5.3 / Fig. 4 and fp16-rounded values -> wavefront schedule
// (pack.cpp) -> kernel stream of {LDS-encoded offset, value} (8 bytes) or {LDS-encoded
// offset, fp16 value} (4 bytes) per (workgroup group, wavefront, channel chunk, slot) ->
// one device allocation.  sparseconv_forward validates against the handle and
// launches asynchronously on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <mutex>
#include <numeric>
#include <string>
#include <thread>
#include <unordered_set>
#include <vector>

#include "../../include/sparseconv.h"
#include "bake.h"
#include "plan.h"

namespace {

constexpr uint64_t kMagic = 0x53434f4e56484e44ull;  // live handle

thread_local std::string g_err;

// Live handles: every entry point checks its handle against this set before touching it, so
// a destroyed (or never created) handle is reported as invalid instead of being read.
std::mutex g_live_mu;
std::unordered_set<const void*> g_live;

void live_add(const void* h) {
  std::lock_guard<std::mutex> lk(g_live_mu);
  g_live.insert(h);
}
bool live_remove(const void* h) {
  std::lock_guard<std::mutex> lk(g_live_mu);
  return g_live.erase(h) == 1;
}
bool live_has(const void* h) {
  std::lock_guard<std::mutex> lk(g_live_mu);
  return g_live.count(h) == 1;
}

sc_status fail(sc_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

bool fail_alloc_hook() {
  const char* e = std::getenv("SPARSECONV_TEST_FAIL_ALLOC");
  return e && e[0] == '1';
}

}  // namespace

// One launch plan of a handle with its own kernel stream and tables on the device.  A handle
// holds the default plan (variant 0, the most positions per lane that fit) and a few plans
// with fewer positions per lane or fewer rows per wavefront, which make more work units: the
// forward pass picks the one a cost model rates fastest for its batch size.
struct Variant {
  sc::Plan p;
  sc::Sched sched;
  int32_t max_wave_nnz;
  int32_t split_pieces;
  int cus, per_cu;  // device CUs and workgroups of this plan's kernel per CU
  std::vector<uint32_t> ent;
  std::vector<int32_t> bstart;
  const uint32_t* d_ent;
  const int32_t* d_seg;
  const int32_t* d_slot;
  const int32_t* d_comb;
};

struct BakedKernel {
  sc::BakePlan p;
  std::string src;
  std::vector<char> elf;
  hipModule_t mod = nullptr;
  hipFunction_t fn = nullptr;
};

struct sc_handle {
  uint64_t magic;
  sc::Geom g;
  int64_t nnz;
  bool h16;                      // packed with SC_PACK_FP16_WORD
  std::vector<int32_t> rowptr;   // canonical CSR row pointers
  std::vector<uint32_t> off;     // canonical stretched offsets
  std::vector<float> val;        // canonical values (fp16-rounded when h16)
  std::vector<uint32_t> words;   // h16: the 32-bit packed words, canonical order
  std::vector<Variant> var;      // LDS-tile mapping: launch plans (empty for escoin)
  bool escoin;                   // packed with SC_PACK_ESCOIN_MAP
  sc::EscoinArgs esc;            // escoin: geometry part of the kernel arguments
  const uint32_t* d_esc_ent;     // escoin: {padded-pitch offset, value bits} per non-zero
  const int32_t* d_esc_rowptr;   // escoin: M + 1 row pointers
  int device;
  bool host_only;
  void* dmem;
  size_t dbytes;
  // weights-in-code mapping (bake.h): the generated kernels (the base plan first, then the
  // variants for small batches), their code objects and modules
  bool baked;
  std::vector<BakedKernel> bk;
  std::string bake_why;           // why the layer was not baked ("" if it was)
  int cus;                        // compute units of the device (256 on the host)
  uint32_t* d_status;             // device status word (bit 0: a bounded wait gave up)
  // kernels chosen by measurement (sparseconv_tune): {N, kind (0: weights-in-code kernel bk[i],
  // 1: LDS-tile plan var[i]), i}; forwards of those batch sizes launch them
  mutable std::mutex tune_mu;
  std::vector<std::array<int, 3>> tuned;
};

namespace {

bool valid_handle(const sc_handle* h) { return h && live_has(h) && h->magic == kMagic; }

// IEEE 754 binary16 bits of an fp32 value, rounded to nearest with ties to even, by integer
// operations on the fp32 encoding: rebias the exponent (normal halves) or shift the full
// significand to the 2^-24 grid (subnormal halves), then round the dropped bits.  Values at
// or above 65520 in magnitude become infinity; NaN stays a quiet NaN.
uint16_t half_bits(float f) {
  uint32_t x;
  std::memcpy(&x, &f, 4);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7fffffffu;
  if (ax > 0x7f800000u) return (uint16_t)(sign | 0x7e00u | ((ax >> 13) & 0x3ffu));
  if (ax >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);  // >= 65520 (and infinity)
  auto rne = [](uint32_t v, int sh) {
    const uint32_t q = v >> sh, rem = v & ((1u << sh) - 1u), half = 1u << (sh - 1);
    return q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);
  };
  if (ax >= 0x38800000u)  // >= 2^-14: normal half; a carry into the exponent is correct
    return (uint16_t)(sign | rne(ax - 0x38000000u, 13));
  if (ax <= 0x33000000u) return (uint16_t)sign;  // <= 2^-25: rounds to zero (2^-25 is a tie)
  const uint32_t e = ax >> 23, m = (ax & 0x7fffffu) | 0x800000u;
  return (uint16_t)(sign | rne(m, (int)(126 - e)));  // value / 2^-24 = m * 2^(e - 126)
}

float half_value(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  const uint32_t ex = (h >> 10) & 31u, man = h & 1023u;
  uint32_t x;
  if (ex == 31) {
    x = sign | 0x7f800000u | (man << 13);
  } else if (ex != 0) {
    x = sign | ((ex + 112u) << 23) | (man << 13);
  } else {
    float v = std::ldexp((float)man, -24);  // exact
    std::memcpy(&x, &v, 4);
    x |= sign;
  }
  float f;
  std::memcpy(&f, &x, 4);
  return f;
}

// CSR rows from the caller's weights, columns ascending within each row.
sc_status build_csr(const sc_weights* w, int M, long long crs, bool all_taps, std::vector<int32_t>& rowptr,
                    std::vector<int32_t>& col, std::vector<float>& val) {
  rowptr.assign(M + 1, 0);
  if (all_taps && w->format != SC_WEIGHTS_DENSE) return fail(SC_EINVAL, "SC_PACK_ALL_TAPS needs dense weights");
  if (w->format == SC_WEIGHTS_DENSE) {
    if (!w->values) return fail(SC_EINVAL, "dense weights: values is NULL");
    if (w->colidx || w->rowptr) return fail(SC_EINVAL, "dense weights: colidx/rowptr must be NULL");
    long long nnz = 0;
    for (int m = 0; m < M; m++) {
      const float* wr = w->values + (long long)m * crs;
      const uint8_t* mr = w->mask ? w->mask + (long long)m * crs : nullptr;
      for (long long c = 0; c < crs; c++) nnz += all_taps ? 1 : mr ? (mr[c] != 0) : (wr[c] != 0.0f);
      if (nnz >= (1LL << 31)) return fail(SC_EUNSUPPORTED, "more than 2^31-1 non-zeros");
      rowptr[m + 1] = (int32_t)nnz;
    }
    col.resize(nnz);
    val.resize(nnz);
    long long j = 0;
    for (int m = 0; m < M; m++) {
      const float* wr = w->values + (long long)m * crs;
      const uint8_t* mr = w->mask ? w->mask + (long long)m * crs : nullptr;
      for (long long c = 0; c < crs; c++) {
        const bool keep = all_taps || (mr ? (mr[c] != 0) : (wr[c] != 0.0f));
        if (keep) {
          col[j] = (int32_t)c;
          val[j] = wr[c];
          j++;
        }
      }
    }
    return SC_OK;
  }
  if (w->format != SC_WEIGHTS_CSR) return fail(SC_EINVAL, "unknown weights format");
  if (!w->rowptr) return fail(SC_EINVAL, "CSR weights: rowptr is NULL");
  if (w->mask) return fail(SC_EINVAL, "CSR weights: mask must be NULL");
  if (w->rowptr[0] != 0) return fail(SC_EINVAL, "CSR weights: rowptr[0] != 0");
  for (int m = 0; m < M; m++)
    if (w->rowptr[m + 1] < w->rowptr[m]) return fail(SC_EINVAL, "CSR weights: rowptr decreases at row " + std::to_string(m));
  const long long nnz = w->rowptr[M];
  if (nnz > 0 && (!w->colidx || !w->values)) return fail(SC_EINVAL, "CSR weights: colidx/values is NULL");
  col.resize(nnz);
  val.resize(nnz);
  std::vector<long long> idx;
  for (int m = 0; m < M; m++) {
    const int b = w->rowptr[m], e = w->rowptr[m + 1];
    idx.resize(e - b);
    for (int j = b; j < e; j++) {
      if (w->colidx[j] < 0 || w->colidx[j] >= crs)
        return fail(SC_EINVAL, "CSR weights: colidx out of range at entry " + std::to_string(j));
      idx[j - b] = j;
    }
    std::stable_sort(idx.begin(), idx.end(), [&](long long a, long long c) { return w->colidx[a] < w->colidx[c]; });
    for (int j = b; j < e; j++) {
      col[j] = w->colidx[idx[j - b]];
      val[j] = w->values[idx[j - b]];
      if (j > b && col[j] == col[j - 1])
        return fail(SC_EINVAL, "CSR weights: duplicate column " + std::to_string(col[j]) + " in row " + std::to_string(m));
    }
    rowptr[m + 1] = e;
  }
  return SC_OK;
}

}  // namespace

extern "C" {

const char* sparseconv_last_error(void) { return g_err.c_str(); }

sc_status sparseconv_pack(const sc_weights* w, int32_t M, int32_t C, int32_t R, int32_t S,
                          int32_t H, int32_t W, int32_t stride, int32_t pad, uint32_t flags,
                          sc_handle** out) {
  g_err.clear();
  if (!out) return fail(SC_EINVAL, "out is NULL");
  *out = nullptr;
  if (!w) return fail(SC_EINVAL, "weights descriptor is NULL");
  if (flags & ~(SC_PACK_HOST_ONLY | SC_PACK_ALL_TAPS | SC_PACK_FP16_WORD | SC_PACK_ESCOIN_MAP | SC_PACK_LDS_TILE))
    return fail(SC_EINVAL, "unknown pack flag");
  if ((flags & SC_PACK_ESCOIN_MAP) && (flags & SC_PACK_LDS_TILE))
    return fail(SC_EINVAL, "SC_PACK_ESCOIN_MAP and SC_PACK_LDS_TILE select different mappings");
  const bool h16 = (flags & SC_PACK_FP16_WORD) != 0;
  const bool escoin = (flags & SC_PACK_ESCOIN_MAP) != 0;
  if (h16 && escoin) return fail(SC_EINVAL, "SC_PACK_FP16_WORD and SC_PACK_ESCOIN_MAP cannot be combined");
  sc::Geom g;
  if (!sc::make_geom(M, C, R, S, H, W, stride, pad, &g))
    return fail(SC_ESHAPE, "invalid layer geometry (dims >= 1, stride >= 1, pad >= 0, output >= 1x1)");
  const long long crs = (long long)C * R * S;
  if ((long long)M * crs >= (1LL << 31)) return fail(SC_EUNSUPPORTED, "M*C*R*S >= 2^31");
  if ((long long)C * H * W >= (1LL << 32)) return fail(SC_EUNSUPPORTED, "C*H*W >= 2^32: offsets do not fit u32");
  if (escoin && (long long)C * (H + 2LL * pad) * (W + 2LL * pad) >= (1LL << 30))
    return fail(SC_EUNSUPPORTED, "SC_PACK_ESCOIN_MAP: C*(H+2pad)*(W+2pad) >= 2^30 (32-bit byte offsets)");
  if (h16 && (C > 256 || R > 16 || S > 16))
    return fail(SC_EUNSUPPORTED, "SC_PACK_FP16_WORD: the 32-bit word holds C <= 256 and R, S <= 16");
  if (fail_alloc_hook()) return fail(SC_ENOMEM, "allocation failure (injected by SPARSECONV_TEST_FAIL_ALLOC)");
  sc_handle* h = nullptr;
  try {
    std::vector<int32_t> rowptr, col;
    std::vector<float> val;
    sc_status s = build_csr(w, M, crs, (flags & SC_PACK_ALL_TAPS) != 0, rowptr, col, val);
    if (s != SC_OK) return s;
    const long long nnz = (long long)col.size();
    std::vector<uint32_t> words;
    if (h16) {  // the packed word of each non-zero; the kernel uses the rounded weight
      words.resize(nnz);
      for (long long j = 0; j < nnz; j++) {
        const uint16_t hb = half_bits(val[j]);
        if ((hb & 0x7fffu) == 0x7c00u && !std::isinf(val[j]))
          return fail(SC_EINVAL, "SC_PACK_FP16_WORD: weight " + std::to_string(val[j]) + " overflows fp16");
        const int c = col[j] / (R * S), r = (col[j] / S) % R, sx = col[j] % S;
        words[j] = ((uint32_t)hb << 16) | ((uint32_t)c << 8) | ((uint32_t)sx << 4) | (uint32_t)r;
        val[j] = half_value(hb);
      }
    }
    // plan variants: the default, then caps on positions per lane and rows per wavefront
    // (none when SPARSECONV_PLAN forces a plan)
    std::vector<Variant> vars;
    if (!escoin) {
      static const int caps[][2] = {{0, 0}, {4, 0}, {2, 0}, {1, 0}, {2, 2}, {2, 1}, {1, 1}};
      const char* plan_env = std::getenv("SPARSECONV_PLAN");
      const bool forced = plan_env != nullptr && plan_env[0] != '\0';
      for (const auto& cap : caps) {
        Variant v;
        v.p = sc::choose_plan(g, rowptr, col, &v.sched, cap[0], cap[1]);
        if (v.p.K == 0) {
          if (vars.empty()) break;
          continue;
        }
        if (v.p.quad && h16) continue;  // quad plans take the 8-byte entries only
        bool dup = false;
        for (const Variant& u : vars) dup = dup || (u.p.K == v.p.K && u.p.OCW == v.p.OCW && u.p.quad == v.p.quad);
        if (!dup) vars.push_back(std::move(v));
        if (forced) break;
      }
      // quad plans (8-byte entries): four consecutive positions per lane read with 16-byte
      // LDS reads
      if (!forced && !h16) {
        Variant v;
        v.p = sc::choose_plan(g, rowptr, col, &v.sched, 0, 0, 0, 1);
        if (v.p.K != 0 && v.p.quad) vars.push_back(std::move(v));
      }
      // two ring slots where that makes all input channels one chunk: a unit is then a
      // single step (no per-chunk synchronisation), and one slot is staged while the other
      // is walked
      const size_t nv = forced ? 0 : vars.size();
      for (size_t i = 0; i < nv; i++) {
        if (vars[i].p.nch <= 1 || vars[i].p.D == 2) continue;
        Variant v;
        v.p = sc::choose_plan(g, rowptr, col, &v.sched, vars[i].p.K, vars[i].p.OCW, 2, vars[i].p.quad);
        if (v.p.K == vars[i].p.K && v.p.OCW == vars[i].p.OCW && v.p.quad == vars[i].p.quad && v.p.nch == 1)
          vars.push_back(std::move(v));
      }
    }
    // weights-in-code kernel (bake.h): the default mapping for fp32 weights, unless the
    // caller asks for the LDS-tile kernel, forces one of its plans (SPARSECONV_PLAN), or
    // turns baking off (SPARSECONV_BAKE=off)
    std::vector<BakedKernel> bk;
    std::string bake_why;
    {
      const char* plan_env = std::getenv("SPARSECONV_PLAN");
      const char* bake_env = std::getenv("SPARSECONV_BAKE");
      if (escoin) bake_why = "SC_PACK_ESCOIN_MAP";
      else if (flags & SC_PACK_LDS_TILE) bake_why = "SC_PACK_LDS_TILE";
      else if (flags & SC_PACK_ALL_TAPS) bake_why = "SC_PACK_ALL_TAPS (every tap: the code would not fit the caches)";
      else if (h16) bake_why = "SC_PACK_FP16_WORD (the kernel reads the 32-bit words)";
      else if (plan_env && plan_env[0]) bake_why = "SPARSECONV_PLAN forces an LDS-tile plan";
      else if (bake_env && std::strcmp(bake_env, "off") == 0) bake_why = "SPARSECONV_BAKE=off";
      else {
        // generate and assemble the candidate kernels in parallel (one thread each)
        std::vector<sc::BakePlan> cands = sc::bake_candidates(g, rowptr, col, sc::bake_force_from_env(), &bake_why);
        std::vector<BakedKernel> built(cands.size());
        std::vector<std::string> whys(cands.size());
        std::vector<char> good(cands.size(), 0);
        auto work = [&](size_t i) {
          built[i].p = cands[i];
          good[i] = sc::bake_generate(g, rowptr, col, val, &built[i].p, &built[i].src, &whys[i]) &&
                    sc::bake_assemble(built[i].src, &built[i].elf, &whys[i]);
        };
        std::vector<std::thread> th;
        for (size_t i = 1; i < cands.size(); i++) th.emplace_back(work, i);
        if (!cands.empty()) work(0);
        for (auto& t : th) t.join();
        for (size_t i = 0; i < cands.size(); i++) {
          if (good[i]) bk.push_back(std::move(built[i]));
          else if (bk.empty() && i == 0) bake_why = whys[i];
        }
        if (!bk.empty() && !good[0]) bk.clear();  // the base kernel is required
      }
    }
    const bool baked = !bk.empty();
    if (baked) bake_why.clear();
    if (vars.empty() && !escoin && !baked)
      return fail(SC_EUNSUPPORTED, "no launch plan fits (rows too wide or too dense for the LDS ring)");

    h = new sc_handle();
    h->magic = kMagic;
    live_add(h);
    h->baked = baked;
    h->bk = std::move(bk);
    h->bake_why = std::move(bake_why);
    h->cus = 256;
    h->d_status = nullptr;
    h->g = g;
    h->nnz = nnz;
    h->h16 = h16;
    h->words = std::move(words);
    h->host_only = (flags & SC_PACK_HOST_ONLY) != 0;
    h->dmem = nullptr;
    h->dbytes = 0;
    h->off.resize(nnz);
    for (long long j = 0; j < nnz; j++) {
      const int c = col[j] / (R * S), r = (col[j] / S) % R, sx = col[j] % S;
      h->off[j] = (uint32_t)(((long long)c * H + r) * W + sx);
    }
    h->val = val;
    h->rowptr = rowptr;

    for (Variant& v : vars) {
      v.p.h16 = h16 ? 1 : 0;
      const sc::Plan& p = v.p;
      const sc::Sched& sched = v.sched;
      v.max_wave_nnz = sched.max_wave_nnz;
      v.split_pieces = sched.split_pieces;
      // Kernel stream: per (group, consumer wavefront), one block per chunk holding header
      // entries {count of slot o, 0} (OCW of them, rounded up to even) followed by the slots'
      // non-zeros {enc, value} in slot order; each block starts at a multiple of 64 entries
      // (the kernel loads whole groups of 64), with zero entries in the gaps.  In the 4-byte
      // form an entry is one word: a header holds the count, a non-zero (enc << 16) | fp16
      // bits of its weight.
      const int ew = h16 ? 1 : 2;  // words per entry
      // bstart[(group*NC + consumer)*(nch+1) + k] is the first entry of block k and
      // bstart[.. + nch] the end of the last one.
      const int waves = p.G * (p.NW - 1);  // consumer wavefronts
      std::vector<int32_t> chunk_start((size_t)M * (p.nch + 1));
      for (int m = 0; m < M; m++) {
        int j = rowptr[m];
        for (int k = 0; k <= p.nch; k++) {
          while (j < rowptr[m + 1] && col[j] / (R * S) < k * p.Cc) j++;
          chunk_start[(size_t)m * (p.nch + 1) + k] = j;
        }
        chunk_start[(size_t)m * (p.nch + 1) + p.nch] = rowptr[m + 1];
      }
      const int hdr_n = sc::block_header(p.OCW);
      // quad plans: two zero entries close every block, so that the walk, which reads one
      // entry ahead, never reads past its block
      const int tail = p.quad ? 2 : 0;
      const size_t n_ent = (size_t)nnz + (size_t)waves * p.nch * (hdr_n + tail + 63) + 64;
      if (n_ent >= (size_t)1 << 31) {
        sparseconv_destroy(h);
        return fail(SC_EUNSUPPORTED, "kernel stream too large");
      }
      std::vector<uint32_t>& ent = v.ent;
      std::vector<int32_t>& bstart = v.bstart;
      ent.assign(ew * std::max<size_t>(n_ent, 1), 0);
      bstart.assign((size_t)waves * (p.nch + 1), 0);
      size_t pos = 0;
      for (int wv = 0; wv < waves; wv++) {
        for (int k = 0; k < p.nch; k++) {
          pos = (pos + 63) & ~(size_t)63;
          bstart[(size_t)wv * (p.nch + 1) + k] = (int32_t)pos;
          const size_t hdr = pos;
          pos += hdr_n;
          for (int o = 0; o < p.OCW; o++) {
            const size_t sl = (size_t)wv * p.OCW + o;
            const int m = sched.src_row[sl];
            int cnt = 0;
            uint32_t ncls[4] = {0, 0, 0, 0};
            if (m >= 0) {  // this slot's piece of row m: part of the row's entries of chunk k
              int b = chunk_start[(size_t)m * (p.nch + 1) + k];
              int e = chunk_start[(size_t)m * (p.nch + 1) + k + 1];
              sc::piece_range(b, e, sched.piece[sl], sched.npieces[sl], &b, &e);
              auto enc_of = [&](int j) {
                const int c = col[j] / (R * S), r = (col[j] / S) % R, sx = col[j] % S;
                return (uint32_t)((c % p.Cc) * p.CHS + ((r % stride) * stride + (sx % stride)) * p.PL +
                                  (r / stride) * g.Pp + sx / stride);
              };
              if (p.quad) {
                // class-sorted (stable): {byte offset of the aligned quad, fp32 weight}
                for (int cls = 0; cls < 4; cls++)
                  for (int j = b; j < e; j++) {
                    const uint32_t enc = enc_of(j);
                    if ((int)(enc & 3u) != cls) continue;
                    uint32_t vbits;
                    std::memcpy(&vbits, &val[j], 4);
                    ent[2 * pos] = 4u * (enc & ~3u);
                    ent[2 * pos + 1] = vbits;
                    pos++;
                    ncls[cls]++;
                  }
                if (ncls[0] > 0xffffu || ncls[1] > 0xffffu || ncls[2] > 0xffffu || ncls[3] > 0xffffu) {
                  sparseconv_destroy(h);
                  return fail(SC_EUNSUPPORTED, "quad plan: more than 65535 non-zeros of one class in a block");
                }
                ent[2 * (hdr + o)] = ncls[0] | (ncls[1] << 16);
                ent[2 * (hdr + o) + 1] = ncls[2] | (ncls[3] << 16);
                continue;
              }
              for (int j = b; j < e; j++) {
                const uint32_t enc = enc_of(j);
                if (h16) {
                  if (enc > 0xffffu) {
                    sparseconv_destroy(h);
                    return fail(SC_EUNSUPPORTED, "SC_PACK_FP16_WORD: LDS offset does not fit 16 bits");
                  }
                  ent[pos] = (enc << 16) | (h->words[j] >> 16);
                } else {
                  uint32_t vbits;
                  std::memcpy(&vbits, &val[j], 4);
                  ent[2 * pos] = enc;
                  ent[2 * pos + 1] = vbits;
                }
                pos++;
              }
              cnt = e - b;
            }
            ent[ew * (hdr + o)] = (uint32_t)cnt;
          }
          pos += tail;
        }
        bstart[(size_t)wv * (p.nch + 1) + p.nch] = (int32_t)pos;
      }
      v.cus = 256;
      v.per_cu = 1;
    }
    h->var = std::move(vars);
    h->escoin = escoin;
    h->d_esc_ent = nullptr;
    h->d_esc_rowptr = nullptr;
    std::vector<uint32_t> esc_ent;
    if (escoin) {
      // "Escoin" weight stretching against the padded input: (c*Hp + r)*Wp + s
      sc::EscoinArgs& e = h->esc;
      e = sc::EscoinArgs{};
      e.C = C; e.H = H; e.W = W; e.M = M; e.E = g.E; e.F = g.F; e.st = stride; e.pad = pad;
      e.Hp = H + 2 * pad;
      e.Wp = W + 2 * pad;
      e.img_words = C * e.Hp * e.Wp;
      e.tiles = (g.E * g.F + 256 * sc::kEscoinP - 1) / (256 * sc::kEscoinP);
      int longest = 1;
      for (int m = 0; m < M; m++) longest = std::max(longest, rowptr[m + 1] - rowptr[m]);
      e.chunk = std::min(longest, sc::kEscoinChunk);
      esc_ent.assign(2 * std::max<long long>(nnz, 1), 0);
      for (long long j = 0; j < nnz; j++) {
        const int c = col[j] / (R * S), r = (col[j] / S) % R, sx = col[j] % S;
        esc_ent[2 * j] = (uint32_t)((c * e.Hp + r) * e.Wp + sx);
        std::memcpy(&esc_ent[2 * j + 1], &val[j], 4);
      }
    }

    if (!h->host_only) {
      if (hipGetDevice(&h->device) != hipSuccess) {
        sparseconv_destroy(h);
        return fail(SC_EDEVICE, "no HIP device available");
      }
      auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
      size_t total = 256 + al(esc_ent.size() * 4) + (escoin ? al(rowptr.size() * 4) : 0);  // status word first
      for (const Variant& v : h->var)
        total += al(v.ent.size() * 4) + al(v.bstart.size() * 4) + al(v.sched.slot_row.size() * 4) +
                 al(v.sched.slot_comb.size() * 4);
      h->dbytes = total;
      if (hipMalloc(&h->dmem, h->dbytes) != hipSuccess) {
        h->dmem = nullptr;
        sparseconv_destroy(h);
        return fail(SC_ENOMEM, "hipMalloc of the packed filter bank failed");
      }
      char* base = static_cast<char*>(h->dmem);
      h->d_status = reinterpret_cast<uint32_t*>(base);
      if (hipMemset(base, 0, 256) != hipSuccess) {
        sparseconv_destroy(h);
        return fail(SC_EDEVICE, "clearing the device status word failed");
      }
      base += 256;
      if (escoin) {
        h->d_esc_ent = reinterpret_cast<const uint32_t*>(base);
        h->d_esc_rowptr = reinterpret_cast<const int32_t*>(base + al(esc_ent.size() * 4));
        hipError_t e1 = hipMemcpy(base, esc_ent.data(), esc_ent.size() * 4, hipMemcpyHostToDevice);
        hipError_t e2 = hipMemcpy(base + al(esc_ent.size() * 4), rowptr.data(), rowptr.size() * 4,
                                  hipMemcpyHostToDevice);
        if (e1 != hipSuccess || e2 != hipSuccess) {
          sparseconv_destroy(h);
          return fail(SC_EDEVICE, "upload of the packed filter bank failed");
        }
        base += al(esc_ent.size() * 4) + al(rowptr.size() * 4);
        // set-up for sparseconv_forward_noalloc: resolve the static workspace's address on this
        // device now, outside any stream capture (a failure is reported by that call)
        void* sp = nullptr;
        (void)sc::scratch_address(&sp);
      }
      for (Variant& v : h->var) {
        const size_t b_ent = al(v.ent.size() * 4), b_seg = al(v.bstart.size() * 4);
        const size_t b_slot = al(v.sched.slot_row.size() * 4), b_comb = al(v.sched.slot_comb.size() * 4);
        v.d_ent = reinterpret_cast<const uint32_t*>(base);
        v.d_seg = reinterpret_cast<const int32_t*>(base + b_ent);
        v.d_slot = reinterpret_cast<const int32_t*>(base + b_ent + b_seg);
        v.d_comb = reinterpret_cast<const int32_t*>(base + b_ent + b_seg + b_slot);
        hipError_t e1 = hipMemcpy(base, v.ent.data(), v.ent.size() * 4, hipMemcpyHostToDevice);
        hipError_t e2 = hipMemcpy(base + b_ent, v.bstart.data(), v.bstart.size() * 4, hipMemcpyHostToDevice);
        hipError_t e3 = hipMemcpy(base + b_ent + b_seg, v.sched.slot_row.data(), v.sched.slot_row.size() * 4,
                                  hipMemcpyHostToDevice);
        hipError_t e4 = hipMemcpy(base + b_ent + b_seg + b_slot, v.sched.slot_comb.data(),
                                  v.sched.slot_comb.size() * 4, hipMemcpyHostToDevice);
        const int eo = sc::occupancy(v.p, &v.cus, &v.per_cu);
        if (e1 != hipSuccess || e2 != hipSuccess || e3 != hipSuccess || e4 != hipSuccess || eo != (int)hipSuccess) {
          sparseconv_destroy(h);
          return fail(SC_EDEVICE, "upload of the packed filter bank failed");
        }
        base += b_ent + b_seg + b_slot + b_comb;
      }
    }
    if (h->baked && !h->host_only) {
      int cus = 0;
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, h->device) == hipSuccess && cus > 0)
        h->cus = cus;
      for (BakedKernel& k : h->bk) {
        if (hipModuleLoadData(&k.mod, k.elf.data()) != hipSuccess) {
          k.mod = nullptr;
          sparseconv_destroy(h);
          return fail(SC_EDEVICE, "loading the weights-in-code kernel failed (hipModuleLoadData)");
        }
        if (hipModuleGetFunction(&k.fn, k.mod, "sc_baked") != hipSuccess) {
          sparseconv_destroy(h);
          return fail(SC_EDEVICE, "weights-in-code kernel symbol not found (hipModuleGetFunction)");
        }
        std::vector<char>().swap(k.elf);
      }
    }
    for (Variant& v : h->var) {  // the host copies are not needed any more
      std::vector<uint32_t>().swap(v.ent);
      std::vector<int32_t>().swap(v.bstart);
    }
    *out = h;
    return SC_OK;
  } catch (const std::bad_alloc&) {
    if (h) sparseconv_destroy(h);
    return fail(SC_ENOMEM, "host allocation failed");
  } catch (...) {
    if (h) sparseconv_destroy(h);
    return fail(SC_EINVAL, "unexpected error while packing");
  }
}

sc_status sparseconv_query(const sc_handle* h, sc_info* info) {
  g_err.clear();
  if (!valid_handle(h)) return fail(SC_EINVAL, "invalid or destroyed handle");
  if (!info) return fail(SC_EINVAL, "info is NULL");
  std::memset(info, 0, sizeof(*info));
  info->M = h->g.M; info->C = h->g.C; info->R = h->g.R; info->S = h->g.S;
  info->H = h->g.H; info->W = h->g.W; info->stride = h->g.st; info->pad = h->g.pad;
  info->E = h->g.E; info->F = h->g.F;
  info->nnz = h->nnz;
  info->packed_bytes = ((h->h16 ? 1 : 2) * h->nnz + h->g.M + 1) * 4;
  info->device_bytes = (int64_t)h->dbytes;
  info->entry_bytes = h->h16 ? 4 : 8;
  info->mapping = h->escoin ? 1 : h->baked ? 2 : 0;
  if (h->baked) {
    const sc::BakePlan& b = h->bk[0].p;
    info->bake_groups = b.G;
    info->bake_splits = b.Q;
    info->bake_units_per_wg = b.T;
    info->bake_valid_lanes = b.V;
    info->bake_pitch = b.Pb;
    info->bake_depth = b.D;
    info->bake_vgprs = b.vgprs;
    info->bake_lds_bytes = b.lds_bytes;
    info->bake_variants = (int32_t)h->bk.size();
    info->bake_stage = b.stage;
    info->bake_chunk_channels = b.Cc;
    info->bake_buffers = b.stage ? b.nbuf : 0;
    info->bake_sequential = b.seq;
    info->bake_shared_window = b.gw;
    info->bake_code_bytes = b.code_bytes;
  }
  if (h->escoin) {
    info->tile_pixels = 256 * sc::kEscoinP;
    info->rows_per_wave = 1;
    info->row_groups = 1;
    info->chunk_channels = h->g.C;
    info->lds_bytes = h->esc.chunk * 8;
    info->waves_per_group = 4;
    int64_t longest = 0;
    for (int m = 0; m < h->g.M; m++) longest = std::max<int64_t>(longest, h->rowptr[m + 1] - h->rowptr[m]);
    info->max_wave_nnz = (int32_t)longest;
    return SC_OK;
  }
  if (h->var.empty()) return SC_OK;  // baked only: no LDS-tile plan fits this layer
  const Variant& v = h->var[0];  // the default plan
  info->tile_pixels = v.p.tp;
  info->waves_per_group = v.p.NW - 1;
  info->pipeline_depth = v.p.D;
  info->step_balance_permille = v.p.step_permille;
  info->split_pieces = v.split_pieces;
  info->rows_per_wave = v.p.OCW;
  info->row_groups = v.p.G;
  info->chunk_channels = v.p.Cc;
  info->lds_bytes = v.p.lds_bytes;
  info->max_wave_nnz = v.max_wave_nnz;
  info->plan_variants = (int32_t)h->var.size();
  return SC_OK;
}

sc_status sparseconv_export_packed(const sc_handle* h, int32_t* rowptr, uint32_t* offsets, float* values) {
  g_err.clear();
  if (!valid_handle(h)) return fail(SC_EINVAL, "invalid or destroyed handle");
  if (rowptr) std::memcpy(rowptr, h->rowptr.data(), h->rowptr.size() * 4);
  if (offsets && h->nnz) std::memcpy(offsets, h->off.data(), h->off.size() * 4);
  if (values && h->nnz) std::memcpy(values, h->val.data(), h->val.size() * 4);
  return SC_OK;
}

sc_status sparseconv_export_words(const sc_handle* h, int32_t* rowptr, uint32_t* words) {
  g_err.clear();
  if (!valid_handle(h)) return fail(SC_EINVAL, "invalid or destroyed handle");
  if (!h->h16) return fail(SC_EINVAL, "handle was not packed with SC_PACK_FP16_WORD");
  if (rowptr) std::memcpy(rowptr, h->rowptr.data(), h->rowptr.size() * 4);
  if (words && h->nnz) std::memcpy(words, h->words.data(), h->words.size() * 4);
  return SC_OK;
}

sc_status sparseconv_export_kernel_source(const sc_handle* h, char* buf, int64_t cap, int64_t* len) {
  g_err.clear();
  if (!valid_handle(h)) return fail(SC_EINVAL, "invalid or destroyed handle");
  if (!len) return fail(SC_EINVAL, "len is NULL");
  if (!h->baked) return fail(SC_EINVAL, "handle holds no weights-in-code kernel: " + h->bake_why);
  const std::string& src = h->bk[0].src;
  *len = (int64_t)src.size() + 1;
  if (buf && cap > 0) {
    const size_t n = std::min<size_t>((size_t)cap - 1, src.size());
    std::memcpy(buf, src.data(), n);
    buf[n] = '\0';
  }
  return SC_OK;
}

void sparseconv_destroy(sc_handle* h) {
  if (!h || !live_remove(h)) return;
  for (BakedKernel& k : h->bk)
    if (k.mod) (void)hipModuleUnload(k.mod);
  if (h->dmem) (void)hipFree(h->dmem);
  delete h;
}

}  // extern "C"

namespace {

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const char* pa = static_cast<const char*>(a);
  const char* pb = static_cast<const char*>(b);
  return pa < pb + nb && pb < pa + na;
}

sc_status check_io(const sc::Geom& g, const sc::Plan& p, const float* in, const float* outp, int N) {
  const long long nin = (long long)N * g.C * g.H * g.W;
  if ((long long)p.span_images * g.C * g.H * g.W * 4 >= (1LL << 31) - (1LL << 20))
    return fail(SC_EUNSUPPORTED, "C*H*W too large for 32-bit staging offsets");
  const long long nout = (long long)N * g.M * g.E * g.F;
  if (nin >= (1LL << 31) || nout >= (1LL << 31))
    return fail(SC_EUNSUPPORTED, "N*C*H*W or N*M*E*F >= 2^31 elements");
  if ((long long)N * g.HYp * g.Pp >= (1LL << 31) - (1LL << 12))
    return fail(SC_EUNSUPPORTED, "padded batch extent >= 2^31");
  if (!in || !outp) return fail(SC_EINVAL, "input or output is NULL");
  if (ranges_overlap(in, nin * 4, outp, nout * 4)) return fail(SC_EINVAL, "input and output overlap");
  return SC_OK;
}

sc::KArgs make_args(const sc::Geom& g, const sc::Plan& p, const float* in, float* outp, int N) {
  sc::KArgs a{};
  a.x = in; a.y = outp;
  a.N = N; a.C = g.C; a.H = g.H; a.W = g.W; a.M = g.M; a.E = g.E; a.F = g.F;
  a.R = g.R; a.S = g.S; a.st = g.st; a.pad = g.pad;
  a.Pp = g.Pp; a.HYp = g.HYp; a.img_ext = g.HYp * g.Pp;
  a.PL = p.PL; a.CHS = p.CHS; a.nblk = p.nblk; a.Cc = p.Cc; a.nch = p.nch; a.G = p.G;
  a.xoff = g.xoff; a.cshift = g.cshift;
  a.wide16 = (g.wide && (reinterpret_cast<uintptr_t>(in) & 15) == 0) ? 1 : 0;
  a.nsb = a.wide16 ? p.nblk / 4 : p.nblk;
  a.D = p.D; a.nbuf = p.nbuf;
  a.slot_words = p.slot_words;
  a.HW = g.H * g.W;
  a.x_words = (long long)N * g.C * g.H * g.W;
  a.ext_total = (long long)N * a.img_ext;
  a.tp = p.tp;
  a.ring_words = p.ring_words;
  a.ntiles = (int)((a.ext_total + p.tp - 1) / p.tp);
  a.spin_limit = 1 << 22;
  if (const char* e = std::getenv("SPARSECONV_SPIN_LIMIT"))  // tests of the failure report only
    if (std::atoi(e) > 0) a.spin_limit = std::atoi(e);
  return a;
}

// Estimated cycles of a forward over N images with plan variant v: the busiest CU's units
// times a unit's cost, the larger of its input copy (LDS DMA at ~15 B/cycle with 16-byte
// loads, ~3.7 with 4-byte ones) and its walk (~2.3 cycles per non-zero and 64-position block
// of LDS reads), plus a fixed cost per chunk step and per launch.  A quad plan's walk costs
// 0.83 + 0.30 / r of a K = 7 walk per non-zero, r being the mean run of one class of one slot
// in one chunk (a run boundary breaks its pipeline), and its steps ~1000 cycles more (36 class
// runs per consumer per step); both fitted to imb80/95/99 on MI355X.  Only used to rank the
// handle's variants.
double estimate_cycles(const sc::Geom& g, const Variant& v, int N, long long nnz) {
  const sc::Plan& p = v.p;
  const long long ext = (long long)N * g.HYp * g.Pp;
  const long long units = (ext + p.tp - 1) / p.tp * p.G;
  const long long per_cu = (units + v.cus - 1) / v.cus;
  const double stage = (double)g.C * p.CHS * 4.0 / (g.wide ? 15.0 : 3.7);
  double walk = (double)nnz / p.G * p.K * (p.K >= 2 ? 2.3 : 3.0);
  double step = 1500.0;
  if (p.quad) {
    const double r = std::max(0.05, (double)nnz / ((double)g.M * p.nch * 4.0));
    walk = (double)nnz / p.G * 7 * 2.3 * (0.83 + 0.30 / r);
    step += 1000.0;
  }
  return 6000.0 + (double)per_cu * (step * p.nch + std::max(stage, walk));
}

// The kernel sparseconv_tune chose for N images (-1: none).
int tuned_choice(const sc_handle* h, int N, int kind) {
  std::lock_guard<std::mutex> lk(h->tune_mu);
  for (const auto& t : h->tuned)
    if (t[0] == N && t[1] == kind) return t[2];
  return -1;
}

size_t pick_variant(const sc_handle* h, int N) {
  const int t = tuned_choice(h, N, 1);
  if (t >= 0 && (size_t)t < h->var.size()) return (size_t)t;
  size_t best = 0;
  double bc = 0;
  for (size_t i = 0; i < h->var.size(); i++) {
    const double c = estimate_cycles(h->g, h->var[i], N, h->nnz);
    if (i == 0 || c < bc) {
      best = i;
      bc = c;
    }
  }
  return best;
}

// Whether a batch of N images fits the weights-in-code kernels' 32-bit buffer ranges.
bool baked_fits(const sc_handle* h, int N) {
  if (!h->baked) return false;
  const sc::Geom& g = h->g;
  const long long nin = (long long)N * g.C * g.H * g.W, nout = (long long)N * g.M * g.E * g.F;
  long long pb = 0;
  for (const BakedKernel& k : h->bk) pb = std::max<long long>(pb, k.p.stage ? (long long)g.HYp * g.Pp / g.E + 1 : k.p.Pb);
  return nin * 4 < (1LL << 31) && nout * 4 < (1LL << 31) && (long long)N * g.E * pb < (1LL << 31) - 4096;
}

// The weights-in-code kernel a forward of N images launches (-1: none, use the LDS-tile
// plans): the one sparseconv_tune pinned for N; else, when it gives every SIMD a wavefront, a
// staged kernel (measured best on the 112x112 layers: up to 1.2x faster than the base kernel
// where the traffic dominates) -- the one whose workgroups share their window between twice
// the groups when the layer has at least kSharedNnzPerChannel non-zeros per output channel
// (1.07-1.1x faster at 80-90% sparsity, slower at 95-99%) -- or the base kernel; else the
// handle's kernel with the lowest estimated cycles for N among the unstaged ones (few
// wavefronts leave the staged kernel's DMA latency exposed).
constexpr long long kSharedNnzPerChannel = 64;
long long baked_waves(const sc_handle* h, const sc::BakePlan& bp, int N);

// Whether weights-in-code kernel i can read this input: staged kernels of the wide layout copy
// 16 bytes per lane, which needs a 16-byte aligned input.
bool bk_usable(const sc_handle* h, size_t i, const float* input) {
  const sc::BakePlan& p = h->bk[i].p;
  return !(p.stage && p.bw == 256 && (reinterpret_cast<uintptr_t>(input) & 15));
}

int pick_baked(const sc_handle* h, int N) {
  if (!baked_fits(h, N)) return -1;
  const int t = tuned_choice(h, N, 0);
  if (t >= 0 && (size_t)t < h->bk.size()) return t;
  const bool shared = h->nnz >= kSharedNnzPerChannel * h->g.M;
  int staged = -1;
  for (size_t i = 0; i < h->bk.size(); i++) {
    const sc::BakePlan& bp = h->bk[i].p;
    if (!bp.stage || baked_waves(h, bp, N) < 4LL * h->cus) continue;
    if (staged < 0 || (bool)bp.gw == shared) staged = (int)i;
  }
  if (staged >= 0) return staged;
  if (baked_waves(h, h->bk[0].p, N) >= 4LL * h->cus) return 0;
  int best = 0;
  double bc = 0;
  bool any = false;
  for (size_t i = 0; i < h->bk.size(); i++) {
    if (h->bk[i].p.stage && h->bk.size() > 1) continue;
    const double c = sc::bake_estimate(h->g, h->bk[i].p, N, h->cus);
    if (!any || c < bc) {
      best = (int)i;
      bc = c;
      any = true;
    }
  }
  return best;
}

// Kernel arguments and grid of a weights-in-code kernel for N images (pointers left 0).
sc::BakeArgs baked_args(const sc_handle* h, const sc::BakePlan& bp, int N) {
  const sc::Geom& g = h->g;
  sc::BakeArgs a{};
  a.N = (uint32_t)N;
  a.x_bytes = (uint32_t)((long long)N * g.C * g.H * g.W * 4);
  a.y_bytes = (uint32_t)((long long)N * g.M * g.E * g.F * 4);
  if (bp.stage) {
    // positions of the padded layout; ntiles = workgroups (blocks of T tiles of 64) per group
    const long long qtot = (long long)N * g.HYp * g.Pp;
    a.qtot = (uint32_t)qtot;
    a.ntiles = (uint32_t)((qtot + 64LL * bp.T - 1) / (64LL * bp.T));
    a.per_xcd = (uint32_t)(((long long)a.ntiles * (bp.seq || bp.gw ? 1 : bp.G) + 7) / 8);
    return a;
  }
  const long long qtot = (long long)N * g.E * bp.Pb;
  a.qtot = (uint32_t)qtot;
  a.ntiles = (uint32_t)((qtot + bp.V - 1) / bp.V);
  const long long units = (long long)a.ntiles * bp.G;
  const long long wgs = (units + bp.T - 1) / bp.T;
  a.per_xcd = (uint32_t)((wgs + 7) / 8);
  return a;
}

// Wavefronts a weights-in-code kernel runs for N images.
long long baked_waves(const sc_handle* h, const sc::BakePlan& bp, int N) {
  const sc::BakeArgs a = baked_args(h, bp, N);
  return bp.stage ? (long long)a.ntiles * bp.T * (bp.seq ? 1 : bp.G) : (long long)a.ntiles * bp.G * bp.Q;
}

// Bytes of the padded input the "Escoin" mapping writes for N images (0 for other handles).
long long workspace_bytes(const sc_handle* h, int N) {
  if (!h->escoin || N <= 0) return 0;
  return ((long long)N * h->esc.img_words * 4 + 255) & ~255LL;
}

sc_status launch_bk(const sc_handle* h, int bi, const float* input, float* output, int N, void* hip_stream);
sc_status launch_var(const sc_handle* h, size_t vi, const float* input, float* output, int N, void* hip_stream);

sc_status forward_impl(const sc_handle* h, const float* input, float* output, int32_t N, int32_t C, int32_t H,
                       int32_t W, int32_t M, int32_t R, int32_t S, int32_t stride, int32_t pad, void* workspace,
                       int64_t ws_bytes, bool with_ws, void* hip_stream) {
  if (!valid_handle(h)) return fail(SC_EINVAL, "invalid or destroyed handle");
  if (h->host_only) return fail(SC_EINVAL, "handle was packed with SC_PACK_HOST_ONLY");
  const sc::Geom& g = h->g;
  if (N < 0) return fail(SC_ESHAPE, "N < 0");
  if (C != g.C || H != g.H || W != g.W || M != g.M || R != g.R || S != g.S || stride != g.st || pad != g.pad)
    return fail(SC_ESHAPE, "forward dims differ from the packed handle");
  if (N == 0) return SC_OK;
  int dev = -1;
  if (h->escoin) {
    if (!with_ws)
      return fail(SC_EINVAL, "handle was packed with SC_PACK_ESCOIN_MAP: it needs a workspace (sparseconv_forward_workspace)");
    const long long nin = (long long)N * g.C * g.H * g.W, nout = (long long)N * g.M * g.E * g.F;
    if (nin >= (1LL << 31) || nout >= (1LL << 31))
      return fail(SC_EUNSUPPORTED, "N*C*H*W or N*M*E*F >= 2^31 elements");
    const long long runs = (h->esc.Hp * (long long)h->esc.Wp + 255) / 256;
    if ((long long)N * g.C * runs >= (1LL << 31) || (long long)N * g.M * h->esc.tiles >= (1LL << 31))
      return fail(SC_EUNSUPPORTED, "too many workgroups for one launch");
    if (!input || !output) return fail(SC_EINVAL, "input or output is NULL");
    const long long need = workspace_bytes(h, N);
    if (!workspace || ws_bytes < need)
      return fail(SC_EINVAL, "workspace is NULL or smaller than sparseconv_workspace_size (" + std::to_string(need) +
                                 " bytes)");
    if ((reinterpret_cast<uintptr_t>(workspace) & 3) != 0) return fail(SC_EINVAL, "workspace is not 4-byte aligned");
    if (ranges_overlap(input, nin * 4, output, nout * 4)) return fail(SC_EINVAL, "input and output overlap");
    if (ranges_overlap(workspace, need, input, nin * 4) || ranges_overlap(workspace, need, output, nout * 4))
      return fail(SC_EINVAL, "workspace overlaps input or output");
    if (hipGetDevice(&dev) != hipSuccess || dev != h->device)
      return fail(SC_EINVAL, "current device differs from the device the handle was packed on");
    sc::EscoinArgs a = h->esc;
    a.N = N;
    const int e = sc::launch_escoin(a, input, static_cast<float*>(workspace), output, h->d_esc_ent, h->d_esc_rowptr,
                                    hip_stream);
    if (e != (int)hipSuccess)
      return fail(SC_EDEVICE, std::string("kernel launch failed: ") + hipGetErrorString((hipError_t)e));
    return SC_OK;
  }
  int bi = pick_baked(h, N);
  if (bi >= 0) {
    const long long nin = (long long)N * g.C * g.H * g.W, nout = (long long)N * g.M * g.E * g.F;
    if (!input || !output) return fail(SC_EINVAL, "input or output is NULL");
    if (ranges_overlap(input, nin * 4, output, nout * 4)) return fail(SC_EINVAL, "input and output overlap");
    if ((reinterpret_cast<uintptr_t>(input) & 3) || (reinterpret_cast<uintptr_t>(output) & 3))
      return fail(SC_EINVAL, "input or output is not 4-byte aligned");
    if (hipGetDevice(&dev) != hipSuccess || dev != h->device)
      return fail(SC_EINVAL, "current device differs from the device the handle was packed on");
    if (!bk_usable(h, (size_t)bi, input)) {
      // a staged kernel on an input that is not 16-byte aligned: the first kernel that reads
      // rows directly
      int alt = -1;
      for (size_t i = 0; i < h->bk.size() && alt < 0; i++)
        if (bk_usable(h, i, input)) alt = (int)i;
      if (alt < 0) return fail(SC_EUNSUPPORTED, "this handle's kernel needs a 16-byte aligned input");
      bi = alt;
    }
    return launch_bk(h, bi, input, output, N, hip_stream);
  }
  if (h->var.empty())
    return fail(SC_EUNSUPPORTED, "batch too large for the weights-in-code kernel's 32-bit buffer ranges");
  const size_t vi = pick_variant(h, N);
  sc_status s = check_io(g, h->var[vi].p, input, output, N);
  if (s != SC_OK) return s;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->device)
    return fail(SC_EINVAL, "current device differs from the device the handle was packed on");
  return launch_var(h, vi, input, output, N, hip_stream);
}

// Launch weights-in-code kernel bi / LDS-tile plan vi (arguments already checked).
sc_status launch_bk(const sc_handle* h, int bi, const float* input, float* output, int N, void* hip_stream) {
  const BakedKernel& k = h->bk[bi];
  sc::BakeArgs a = baked_args(h, k.p, N);
  a.x = reinterpret_cast<uint64_t>(input);
  a.y = reinterpret_cast<uint64_t>(output);
  size_t asz = sizeof(a);
  void* cfg[] = {HIP_LAUNCH_PARAM_BUFFER_POINTER, &a, HIP_LAUNCH_PARAM_BUFFER_SIZE, &asz, HIP_LAUNCH_PARAM_END};
  const hipError_t e = hipModuleLaunchKernel(k.fn, 8 * a.per_xcd, 1, 1, 64 * k.p.wpb(), 1, 1, 0,
                                             reinterpret_cast<hipStream_t>(hip_stream), nullptr, cfg);
  if (e != hipSuccess) return fail(SC_EDEVICE, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return SC_OK;
}

sc_status launch_var(const sc_handle* h, size_t vi, const float* input, float* output, int N, void* hip_stream) {
  const sc::Geom& g = h->g;
  const Variant& v = h->var[vi];
  sc::KArgs a = make_args(g, v.p, input, output, N);
  a.status = h->d_status;
  a.ent = v.d_ent;
  a.seg = v.d_seg;
  a.slot_row = v.d_slot;
  a.slot_comb = v.d_comb;
  const long long units = (long long)a.ntiles * v.p.G;
  const long long slots = (long long)v.cus * v.per_cu;
  const int nb = (int)(units < slots ? units : slots);
  const int e = sc::launch_sparse(v.p, a, hip_stream, nb);
  if (e != (int)hipSuccess) return fail(SC_EDEVICE, std::string("kernel launch failed: ") + hipGetErrorString((hipError_t)e));
  return SC_OK;
}

}  // namespace

extern "C" {

sc_status sparseconv_forward(const sc_handle* h, const float* input, float* output, int32_t N, int32_t C,
                             int32_t H, int32_t W, int32_t M, int32_t R, int32_t S, int32_t stride,
                             int32_t pad, void* hip_stream) {
  g_err.clear();
  return forward_impl(h, input, output, N, C, H, W, M, R, S, stride, pad, nullptr, 0, false, hip_stream);
}

sc_status sparseconv_tune(sc_handle* h, const float* input, float* output, int32_t N, int32_t C, int32_t H,
                          int32_t W, int32_t M, int32_t R, int32_t S, int32_t stride, int32_t pad, int32_t reps,
                          void* hip_stream, int32_t* chosen) {
  g_err.clear();
  if (chosen) *chosen = -1;
  if (!valid_handle(h)) return fail(SC_EINVAL, "invalid or destroyed handle");
  if (reps < 1 || reps > 1000) return fail(SC_EINVAL, "reps must be 1..1000");
  if (N < 1) return fail(SC_ESHAPE, "N < 1");
  if (h->escoin) {  // a single kernel: nothing to choose
    if (chosen) *chosen = 0;
    return SC_OK;
  }
  // one forward with the current choice checks every argument (and warms up)
  sc_status st = forward_impl(h, input, output, N, C, H, W, M, R, S, stride, pad, nullptr, 0, false, hip_stream);
  if (st != SC_OK) return st;
  const bool bk = pick_baked(h, N) >= 0;
  const int n = bk ? (int)h->bk.size() : (int)h->var.size();
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    return fail(SC_EDEVICE, "hipEventCreate failed");
  }
  int best = -1;
  float best_ms = 0.0f;
  for (int i = 0; i < n && st == SC_OK; i++) {
    if (bk && !bk_usable(h, (size_t)i, input)) continue;
    auto launch = [&]() { return bk ? launch_bk(h, i, input, output, N, hip_stream)
                                    : launch_var(h, (size_t)i, input, output, N, hip_stream); };
    st = launch();  // first launch of a kernel: not timed
    if (st != SC_OK) break;
    if (hipEventRecord(e0, s) != hipSuccess) st = fail(SC_EDEVICE, "hipEventRecord failed");
    for (int r = 0; r < reps && st == SC_OK; r++) st = launch();
    if (st != SC_OK) break;
    float ms = 0.0f;
    if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
        hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
      st = fail(SC_EDEVICE, "timing the kernels failed");
      break;
    }
    if (best < 0 || ms < best_ms) {
      best = i;
      best_ms = ms;
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (st != SC_OK) return st;
  {
    std::lock_guard<std::mutex> lk(h->tune_mu);
    const int kind = bk ? 0 : 1;
    bool found = false;
    for (auto& t : h->tuned)
      if (t[0] == N && t[1] == kind) {
        t[2] = best;
        found = true;
      }
    if (!found) h->tuned.push_back({N, kind, best});
  }
  // leave the chosen kernel's result in the output
  st = bk ? launch_bk(h, best, input, output, N, hip_stream) : launch_var(h, (size_t)best, input, output, N, hip_stream);
  if (st != SC_OK) return st;
  if (chosen) *chosen = best;
  return SC_OK;
}

sc_status sparseconv_launch_info(const sc_handle* h, int32_t N, sc_launch* out) {
  g_err.clear();
  if (!valid_handle(h)) return fail(SC_EINVAL, "invalid or destroyed handle");
  if (!out) return fail(SC_EINVAL, "out is NULL");
  if (N < 1) return fail(SC_ESHAPE, "N < 1");
  std::memset(out, 0, sizeof(*out));
  if (h->escoin) {
    out->mapping = 1;
    const long long runs = (h->esc.Hp * (long long)h->esc.Wp + 255) / 256;
    out->grid = (int64_t)N * h->g.M * h->esc.tiles;
    out->block = 256;
    out->pre_grid = (int64_t)N * h->g.C * runs;
    out->lds_bytes = h->esc.chunk * 8;
    return SC_OK;
  }
  const int bi = pick_baked(h, N);
  if (bi >= 0) {
    const sc::BakePlan& p = h->bk[bi].p;
    const sc::BakeArgs a = baked_args(h, p, N);
    out->mapping = 2;
    out->variant = bi;
    out->grid = 8LL * a.per_xcd;
    out->block = 64 * p.wpb();
    out->lds_bytes = p.lds_bytes;
    out->vgprs = p.vgprs;
    out->groups = p.G;
    out->splits = p.Q;
    out->units_per_wg = p.T;
    out->depth = p.D;
    out->valid_lanes = p.V;
    out->waves = baked_waves(h, p, N);
    if (p.stage) {
      out->chunk_channels = p.Cc;
      out->tile_pixels = p.T * 64;
      out->stage = 1;
    }
    return SC_OK;
  }
  if (h->var.empty()) return fail(SC_EUNSUPPORTED, "batch too large for the weights-in-code kernel");
  const size_t vi = pick_variant(h, N);
  const Variant& v = h->var[vi];
  const sc::Geom& g = h->g;
  const long long ext = (long long)N * g.HYp * g.Pp;
  const long long units = (ext + v.p.tp - 1) / v.p.tp * v.p.G;
  const long long slots = (long long)v.cus * v.per_cu;
  out->mapping = 0;
  out->variant = (int32_t)vi;
  out->grid = units < slots ? units : slots;
  out->block = 64 * v.p.NW;
  out->lds_bytes = v.p.lds_bytes;
  out->tile_pixels = v.p.tp;
  out->rows_per_wave = v.p.OCW;
  out->groups = v.p.G;
  out->chunk_channels = v.p.Cc;
  out->quad = v.p.quad;
  out->waves = out->grid * v.p.NW;
  return SC_OK;
}

sc_status sparseconv_device_status(const sc_handle* h, uint32_t* status, int32_t clear) {
  g_err.clear();
  if (!valid_handle(h)) return fail(SC_EINVAL, "invalid or destroyed handle");
  if (!status) return fail(SC_EINVAL, "status is NULL");
  if (h->host_only || !h->d_status) return fail(SC_EINVAL, "handle was packed with SC_PACK_HOST_ONLY");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->device)
    return fail(SC_EINVAL, "current device differs from the device the handle was packed on");
  if (hipMemcpy(status, h->d_status, 4, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(SC_EDEVICE, "reading the device status word failed");
  if (clear && *status != 0 && hipMemset(h->d_status, 0, 4) != hipSuccess)
    return fail(SC_EDEVICE, "clearing the device status word failed");
  return SC_OK;
}

sc_status sparseconv_dense_forward(const float* w_dense_dev, const float* input, float* output, int32_t N,
                                   int32_t C, int32_t H, int32_t W, int32_t M, int32_t R, int32_t S,
                                   int32_t stride, int32_t pad, void* hip_stream) {
  g_err.clear();
  if (N < 0) return fail(SC_ESHAPE, "N < 0");
  if (M < 1 || C < 1 || R < 1 || S < 1 || H < 1 || W < 1 || stride < 1 || pad < 0)
    return fail(SC_ESHAPE, "M, C, R, S, H, W and stride must be >= 1 and pad >= 0");
  const long long E = ((long long)H + 2LL * pad - R) / stride + 1, F = ((long long)W + 2LL * pad - S) / stride + 1;
  if (H + 2LL * pad < R || W + 2LL * pad < S || E < 1 || F < 1) return fail(SC_ESHAPE, "E or F < 1");
  const long long nw = (long long)M * C * R * S;
  if (nw >= (1LL << 31)) return fail(SC_EUNSUPPORTED, "M*C*R*S >= 2^31");
  if (N == 0) return SC_OK;
  const long long nin = (long long)N * C * H * W, nout = (long long)N * M * E * F;
  if (nin * 4 >= (1LL << 31) || nout * 4 >= (1LL << 31))
    return fail(SC_EUNSUPPORTED, "N*C*H*W*4 or N*M*E*F*4 >= 2^31 bytes (32-bit buffer offsets)");
  if (!w_dense_dev || !input || !output) return fail(SC_EINVAL, "weights, input or output is NULL");
  if ((reinterpret_cast<uintptr_t>(w_dense_dev) | reinterpret_cast<uintptr_t>(input) |
       reinterpret_cast<uintptr_t>(output)) & 3)
    return fail(SC_EINVAL, "weights, input or output is not 4-byte aligned");
  if (ranges_overlap(input, nin * 4, output, nout * 4)) return fail(SC_EINVAL, "input and output overlap");
  if (ranges_overlap(w_dense_dev, nw * 4, output, nout * 4)) return fail(SC_EINVAL, "weights and output overlap");
  sc::DenseArgs a{};
  a.C = C, a.H = H, a.W = W, a.M = M, a.R = R, a.S = S, a.st = stride, a.pad = pad;
  a.E = (int)E, a.F = (int)F;
  a.EF = (int)(E * F);
  a.MEF = (int)(M * E * F);
  a.CHW = (int)((long long)C * H * W);
  a.HW4 = (int)((long long)H * W * 4);
  a.RS = R * S;
  a.CRS = (int)((long long)C * R * S);
  a.qtot = (int)(N * E * F);
  a.x_bytes = (uint32_t)(nin * 4);
  a.y_bytes = (uint32_t)(nout * 4);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess)
    return fail(SC_EDEVICE, "no current HIP device");
  const int e = sc::launch_dense(a, w_dense_dev, input, output, 4 * cus, hip_stream);
  if (e != (int)hipSuccess)
    return fail(SC_EDEVICE, std::string("kernel launch failed: ") + hipGetErrorString((hipError_t)e));
  return SC_OK;
}

sc_status sparseconv_forward_noalloc(const sc_handle* h, const float* input, float* output, int32_t N, int32_t C,
                                     int32_t H, int32_t W, int32_t M, int32_t R, int32_t S, int32_t stride,
                                     int32_t pad, void* hip_stream) {
  g_err.clear();
  if (!valid_handle(h)) return fail(SC_EINVAL, "invalid or destroyed handle");
  if (!h->escoin) return forward_impl(h, input, output, N, C, H, W, M, R, S, stride, pad, nullptr, 0, false, hip_stream);
  const sc::Geom& g = h->g;
  if (N < 0) return fail(SC_ESHAPE, "N < 0");
  if (C != g.C || H != g.H || W != g.W || M != g.M || R != g.R || S != g.S || stride != g.st || pad != g.pad)
    return fail(SC_ESHAPE, "forward dims differ from the packed handle");
  const long long need = workspace_bytes(h, N);
  if (need > sc::kScratchBytes)
    return fail(SC_EUNSUPPORTED, "this batch needs a " + std::to_string(need) +
                                     "-byte workspace, more than the library's static " +
                                     std::to_string(sc::kScratchBytes) + " bytes (use sparseconv_forward_workspace)");
  void* scratch = nullptr;
  if (N > 0) {
    const int e = sc::scratch_address(&scratch);
    if (e != (int)hipSuccess)
      return fail(SC_EDEVICE, std::string("resolving the static workspace failed: ") +
                                  hipGetErrorString((hipError_t)e));
  }
  return forward_impl(h, input, output, N, C, H, W, M, R, S, stride, pad, scratch, sc::kScratchBytes, true,
                      hip_stream);
}

sc_status sparseconv_workspace_size(const sc_handle* h, int32_t N, int64_t* bytes) {
  g_err.clear();
  if (!valid_handle(h)) return fail(SC_EINVAL, "invalid or destroyed handle");
  if (!bytes) return fail(SC_EINVAL, "bytes is NULL");
  if (N < 0) return fail(SC_ESHAPE, "N < 0");
  *bytes = workspace_bytes(h, N);
  return SC_OK;
}

sc_status sparseconv_forward_workspace(const sc_handle* h, const float* input, float* output, int32_t N,
                                       int32_t C, int32_t H, int32_t W, int32_t M, int32_t R, int32_t S,
                                       int32_t stride, int32_t pad, void* workspace, int64_t workspace_bytes,
                                       void* hip_stream) {
  g_err.clear();
  return forward_impl(h, input, output, N, C, H, W, M, R, S, stride, pad, workspace, workspace_bytes, true,
                      hip_stream);
}

}  // extern "C"
