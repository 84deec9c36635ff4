// Host-only packing of seeded random layers through the C ABI, built with AddressSanitizer
// and UndefinedBehaviorSanitizer: CSR construction from dense weights (with and without a
// mask) and from CSR input, the canonical export, the packed words, the LDS-tile schedule and
// kernel streams, the "Escoin" entries, and the weights-in-code plans, code generation and
// assembly.  Also malformed CSR and invalid arguments.  Exits non-zero on any inconsistency.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "sparseconv.h"

static int fails = 0;
#define CHECK(c)                                                              \
  do {                                                                        \
    if (!(c)) {                                                               \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      fails++;                                                                \
    }                                                                         \
  } while (0)

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 120;
  std::mt19937 rng(20260);
  auto U = [&](int a, int b) { return std::uniform_int_distribution<int>(a, b)(rng); };
  int ok = 0, refused = 0;
  for (int it = 0; it < iters; it++) {
    const int RSv[] = {1, 2, 3, 5, 7, 11};
    const int R = RSv[U(0, 5)], S = U(0, 2) ? R : RSv[U(0, 5)];
    const int st = U(1, 4), pad = U(0, 3);
    const int H = U(std::max(1, R - 2 * pad), 60), W = U(std::max(1, S - 2 * pad), 60);
    const int M = U(1, 300), C = U(1, 200);
    const long long crs = (long long)C * R * S;
    if ((long long)M * crs > 600000) continue;
    const double dens = std::uniform_real_distribution<double>(0.0, 1.0)(rng);
    const double p = dens < 0.15 ? 0.0 : dens < 0.4 ? 0.01 : dens < 0.8 ? 0.05 : 0.4;
    std::vector<float> w((size_t)(M * crs), 0.0f);
    std::vector<uint8_t> mask((size_t)(M * crs), 0);
    std::bernoulli_distribution keep(p);
    const int dense_rows = U(0, 2);
    for (int m = 0; m < M; m++)
      for (long long j = 0; j < crs; j++)
        if (m < dense_rows || keep(rng)) {
          w[(size_t)(m * crs + j)] = (float)U(-7, 7) * 0.25f;
          mask[(size_t)(m * crs + j)] = 1;
        }
    const int form = U(0, 5);  // 0-1 default, 2 fp16 word, 3 Escoin, 4 LDS tile, 5 every tap
    uint32_t flags = SC_PACK_HOST_ONLY;
    if (form == 2) flags |= SC_PACK_FP16_WORD;
    if (form == 3) flags |= SC_PACK_ESCOIN_MAP;
    if (form == 4) flags |= SC_PACK_LDS_TILE;
    if (form == 5) flags |= SC_PACK_ALL_TAPS;
    const bool use_mask = U(0, 1) == 1;
    sc_weights d{SC_WEIGHTS_DENSE, w.data(), nullptr, nullptr, use_mask ? mask.data() : nullptr};
    sc_handle* h = nullptr;
    const int s = sparseconv_pack(&d, M, C, R, S, H, W, st, pad, flags, &h);
    if (s != SC_OK) {
      CHECK(h == nullptr);
      CHECK(s == SC_EUNSUPPORTED || s == SC_ESHAPE);
      refused++;
      continue;
    }
    ok++;
    sc_info info;
    CHECK(sparseconv_query(h, &info) == SC_OK);
    std::vector<int32_t> rowptr(M + 1);
    std::vector<uint32_t> off((size_t)info.nnz + 1);
    std::vector<float> val((size_t)info.nnz + 1);
    CHECK(sparseconv_export_packed(h, rowptr.data(), off.data(), val.data()) == SC_OK);
    CHECK(rowptr[0] == 0 && rowptr[M] == info.nnz);
    for (int m = 0; m < M; m++) CHECK(rowptr[m] <= rowptr[m + 1]);
    for (long long j = 0; j < info.nnz; j++) CHECK(off[(size_t)j] < (uint32_t)((long long)C * H * W));
    if (flags & SC_PACK_FP16_WORD) {
      std::vector<uint32_t> words((size_t)info.nnz + 1);
      CHECK(sparseconv_export_words(h, nullptr, words.data()) == SC_OK);
    }
    if (info.mapping == 2) {
      int64_t len = 0;
      CHECK(sparseconv_export_kernel_source(h, nullptr, 0, &len) == SC_OK && len > 1);
      std::string src((size_t)len, '\0');
      CHECK(sparseconv_export_kernel_source(h, &src[0], len, &len) == SC_OK);
      CHECK(std::strstr(src.c_str(), "sc_baked") != nullptr);
    }
    for (int n : {1, 3, 17}) {
      sc_launch li;
      CHECK(sparseconv_launch_info(h, n, &li) == SC_OK);
    }
    // CSR input built from the export must give the same canonical form
    std::vector<int32_t> col((size_t)info.nnz + 1);
    for (int m = 0; m < M; m++)
      for (int j = rowptr[m]; j < rowptr[m + 1]; j++) {
        const uint32_t o = off[(size_t)j];
        const int c = (int)(o / (uint32_t)(H * W)), rem = (int)(o % (uint32_t)(H * W));
        const int r = rem / W, sx = rem % W;
        col[(size_t)j] = (c * R + r) * S + sx;
      }
    if (!(flags & (SC_PACK_FP16_WORD | SC_PACK_ALL_TAPS)) && R <= H && S <= W) {
      sc_weights c{SC_WEIGHTS_CSR, val.data(), col.data(), rowptr.data(), nullptr};
      sc_handle* h2 = nullptr;
      if (sparseconv_pack(&c, M, C, R, S, H, W, st, pad, SC_PACK_HOST_ONLY, &h2) == SC_OK) {
        std::vector<uint32_t> off2((size_t)info.nnz + 1);
        CHECK(sparseconv_export_packed(h2, nullptr, off2.data(), nullptr) == SC_OK);
        CHECK(std::memcmp(off.data(), off2.data(), (size_t)info.nnz * 4) == 0);
        sparseconv_destroy(h2);
      }
    }
    sparseconv_destroy(h);
    sc_info dead;
    CHECK(sparseconv_query(h, &dead) == SC_EINVAL);  // the registry rejects a destroyed handle
  }
  // malformed CSR inputs are refused before anything is built
  {
    float v[3] = {1, 2, 3};
    int32_t colidx[3] = {0, 0, 5};
    int32_t rp_dup[3] = {0, 2, 3};
    int32_t rp_dec[3] = {0, 3, 2};
    int32_t colbad[3] = {0, 1, 99};
    sc_handle* h = nullptr;
    sc_weights a{SC_WEIGHTS_CSR, v, colidx, rp_dup, nullptr};
    CHECK(sparseconv_pack(&a, 2, 1, 3, 3, 5, 5, 1, 1, SC_PACK_HOST_ONLY, &h) == SC_EINVAL && !h);
    sc_weights b{SC_WEIGHTS_CSR, v, colidx, rp_dec, nullptr};
    CHECK(sparseconv_pack(&b, 2, 1, 3, 3, 5, 5, 1, 1, SC_PACK_HOST_ONLY, &h) == SC_EINVAL && !h);
    sc_weights c{SC_WEIGHTS_CSR, v, colbad, rp_dup, nullptr};
    CHECK(sparseconv_pack(&c, 2, 1, 3, 3, 5, 5, 1, 1, SC_PACK_HOST_ONLY, &h) == SC_EINVAL && !h);
    CHECK(sparseconv_pack(nullptr, 2, 1, 3, 3, 5, 5, 1, 1, SC_PACK_HOST_ONLY, &h) == SC_EINVAL);
    CHECK(sparseconv_query(nullptr, nullptr) == SC_EINVAL);
  }
  std::printf("packed %d, refused %d, failed checks %d\n", ok, refused, fails);
  return fails == 0 && ok > iters / 3 ? 0 : 1;
}
