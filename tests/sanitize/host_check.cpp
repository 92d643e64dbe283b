// CPU check of the library's host-side planning (sffn_host.h) and of the fp64 oracle
// (oracle.c), built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitize.py: randomized inputs, including ragged sizes, NaN and out-of-range
// frequencies, and every fp16 bit pattern; each result is checked for its invariants and any
// sanitizer report fails the run. Test infrastructure only.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "sffn_host.h"

extern "C" {
double oracle_half_to_double(uint16_t h);
int oracle_predict(int32_t d, int32_t n, int32_t r, int32_t B, const float* X, const void* P1,
                   const void* P2, int32_t p_dtype, const float* c, double* S, double* Q);
int oracle_threshold(int32_t B, int32_t n, const double* S, double tau, uint8_t* M);
int oracle_compact(int32_t B, int32_t n, const uint8_t* M, int32_t* idx, int32_t* count,
                   uint64_t* tokmask);
int oracle_forward(int32_t d, int32_t n, int32_t B, int32_t gated, const float* X, const void* Wa,
                   const void* Wu, const void* Wo, int32_t w_dtype, const float* b_a,
                   const float* b_o, const int32_t* idx, int32_t count, const uint64_t* tokmask,
                   double* Y);
int oracle_dense(int32_t d, int32_t n, int32_t B, int32_t gated, const float* X, const void* Wa,
                 const void* Wu, const void* Wo, int32_t w_dtype, const float* b_a,
                 const float* b_o, double* Y);
int oracle_preact(int32_t d, int32_t n, int32_t B, const float* X, const void* Wa,
                  int32_t w_dtype, const float* b_a, double* A);
int oracle_profile_counts(int32_t d, int32_t n, int32_t N, const float* X, const void* Wa,
                          int32_t w_dtype, const float* b_a, int64_t* counts);
int oracle_permutation(const int64_t* counts, int32_t n, int32_t n_hot, int32_t* perm);
int oracle_pack_rows(const void* src, const int32_t* perm, void* dst, int32_t rows,
                     int64_t row_bytes);
}

static int failures = 0;
#define CHECK(c)                                                         \
  do {                                                                   \
    if (!(c)) {                                                          \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

int main() {
  std::mt19937_64 rng(12345);
  auto uni = [&](double a, double b) { return std::uniform_real_distribution<double>(a, b)(rng); };
  auto irand = [&](int a, int b) { return std::uniform_int_distribution<int>(a, b)(rng); };

  // ---- ranges and splits
  for (int it = 0; it < 300; ++it) {
    const int n = irand(1, it % 10 == 0 ? 140000 : 20000);
    std::vector<float> f(n);
    for (auto& v : f) {
      const int k = irand(0, 19);
      v = k == 0 ? NAN : k == 1 ? -0.5f : k == 2 ? 3.f : k < 6 ? 0.f : (float)uni(0, 1);
    }
    const bool nofreq = it % 7 == 0;
    const int target = irand(1, 3000);
    const auto rs = sffn::host::balanced_ranges(n, nofreq ? nullptr : f.data(), 512.0, 8192.0,
                                                target, 64);
    if (rs.empty()) continue;
    CHECK(rs.front() == 0 && rs.back() == n);
    for (size_t u = 0; u + 1 < rs.size(); ++u) {
      CHECK(rs[u + 1] > rs[u]);
      CHECK(rs[u + 1] - rs[u] <= 64);
    }
    CHECK((int)rs.size() - 1 <= std::max(target, 1) || (int)rs.size() - 1 >= (n + 63) / 64);
    CHECK(sffn::host::max_range_cost(rs, nofreq ? nullptr : f.data(), 512.0, 8192.0) > 0.0);
    const int ks = irand(1, 16);
    int upt = 0;
    const auto s = sffn::host::split_ranges(rs, nofreq ? nullptr : f.data(), ks, upt);
    CHECK((int)s.size() == ks + 1 && s[0] == 0 && s[ks] == (int)rs.size() - 1);
    int widest = 0;
    for (int k = 0; k < ks; ++k) {
      CHECK(s[k + 1] >= s[k]);
      widest = std::max(widest, s[k + 1] - s[k]);
    }
    CHECK(upt >= 1 && upt <= 16 && (upt & (upt - 1)) == 0);
    CHECK(upt * 256 >= widest || upt == 16);
    // dense crossover: the returned batch is the first whose expected union exceeds it
    const double thr = uni(0.05, 0.95);
    const int b = sffn::host::dense_from_batch(f.data(), n, thr, 64, 65);
    auto uni_at = [&](int bb) {
      double u = 0.0;
      for (int i = 0; i < n; ++i) u += 1.0 - std::pow(1.0 - sffn::host::clamp_freq(f[i]), (double)bb);
      return u / n;
    };
    if (b <= 64) {
      CHECK(uni_at(b) > thr);
      if (b > 1) CHECK(uni_at(b - 1) <= thr);
    } else {
      CHECK(uni_at(64) <= thr);
    }
    // half-tile batches: the last batch whose expected union stays within the bound
    const double rows = uni(0.0, 1.2) * n;
    const int hb = sffn::host::union_within_batch(nofreq ? nullptr : f.data(), n, rows, 15);
    CHECK(hb == 0 || (hb >= 2 && hb <= 15));
    if (nofreq) {
      CHECK(hb == (n <= rows ? 15 : 0));
    } else {
      auto rows_at = [&](int bb) {
        double u = 0.0;
        for (int i = 0; i < n; ++i) u += 1.0 - std::pow(1.0 - sffn::host::clamp_freq(f[i]), (double)bb);
        return u;
      };
      if (hb >= 2) CHECK(rows_at(hb) <= rows);
      if (hb < 15) CHECK(rows_at(hb < 2 ? 2 : hb + 1) > rows);
    }
  }

  // ---- dense prefill plan: for random shapes, compute-unit counts and chunk sizes, every
  // chunk up to the requested size fits the scratch sized for it, its h rows cover the
  // row length of the tile its plan takes, and its partial-sum region covers its splits
  for (int it = 0; it < 400; ++it) {
    const int d = 128 * irand(1, 64), n = irand(1, 60000), cus = irand(1, 320);
    const int chunk = irand(1, 3000);
    const size_t work = sffn::host::pf_work_bytes(d, n, cus, chunk);
    CHECK(sffn::host::pf_work_bytes(d, n, cus, 0) == 0);
    // the chunk a scratch holds: the largest tile multiple whose scratch fits, checked
    // against a linear scan from there (the scratch size never falls as the chunk grows)
    for (int probe = 0; probe < 3; ++probe) {
      const size_t wb = probe == 0 ? work : probe == 1 ? work - 1 : work + (size_t)irand(0, 1 << 26);
      const int ct = sffn::host::pf_chunk_tokens(d, n, cus, wb);
      CHECK(ct % 128 == 0 && ct >= 0 && ct <= (1 << 20));
      if (ct > 0) CHECK(sffn::host::pf_work_bytes(d, n, cus, ct) <= wb);
      if (ct < (1 << 20)) CHECK(sffn::host::pf_work_bytes(d, n, cus, ct + 128) > wb);
      if (probe == 0) CHECK(ct >= (chunk + 127) / 128 * 128);
    }
    for (int t = 128; t + 128 <= 4096; t += 128)
      CHECK(sffn::host::pf_work_bytes(d, n, cus, t) <= sffn::host::pf_work_bytes(d, n, cus, t + 128));
    const int cbp = (chunk + 127) / 128 * 128;
    for (int bp = 128; bp <= cbp; bp += 128) {
      const sffn::host::PfCarve c = sffn::host::pf_carve(d, n, cus, (size_t)bp);
      CHECK(c.end <= work);
      CHECK(c.xh == 0 && c.xl % 256 == 0 && c.hh % 256 == 0 && c.hl % 256 == 0 && c.part % 256 == 0);
      CHECK(c.xl - c.xh >= (size_t)bp * d * 2 && c.hh - c.xl >= (size_t)bp * d * 2);
      for (int gated = 0; gated < 2; ++gated) {
        for (int lo = 0; lo < 2; ++lo) {
          const int ut = sffn::host::pf_up_it(n, gated, lo, bp / 128, cus);
          CHECK(gated ? (ut == 2 || ut == 3) : (ut == 2 || ut == 4 || ut == 6));
          const int np = sffn::host::pf_np(n, ut);
          CHECK(np >= n && np % (32 * ut) == 0 && (size_t)np <= sffn::host::pf_rows(n));
          CHECK(c.hl - c.hh >= (size_t)bp * np * 2 && c.part - c.hl >= (size_t)bp * np * 2);
          const int S = sffn::host::pf_splits(d, cus, bp / 128, (size_t)np);
          CHECK(S >= 1 && S <= sffn::host::kPfMaxSplits && (S & (S - 1)) == 0);
          if (S > 1) {
            CHECK(c.end - c.part >= (size_t)S * bp * d * 4);
            CHECK(np / 32 >= 8 * S);  // each split keeps at least 8 stages of 32 neurons
          }
        }
      }
    }
  }

  // ---- permutation: the library's and the oracle's, equal, and valid
  for (int it = 0; it < 200; ++it) {
    const int n = irand(1, 5000), n_hot = irand(0, n);
    std::vector<int64_t> c(n);
    for (auto& v : c) v = irand(0, 7);
    std::vector<int32_t> p(n), q(n);
    sffn::host::hot_first_permutation(c.data(), n, n_hot, p.data());
    CHECK(oracle_permutation(c.data(), n, n_hot, q.data()) == 0);
    CHECK(p == q);
    std::vector<char> seen(n, 0);
    for (int k = 0; k < n; ++k) {
      CHECK(p[k] >= 0 && p[k] < n);
      if (p[k] >= 0 && p[k] < n) seen[p[k]]++;
    }
    for (int i = 0; i < n; ++i) CHECK(seen[i] == 1);
  }

  // ---- fp16 decoding: every bit pattern against the IEEE 754 binary16 definition (sign,
  // 5-bit exponent with bias 15, 10-bit fraction; subnormals at exponent 0; all-ones
  // exponent is infinity or NaN)
  for (uint32_t h = 0; h < 65536; ++h) {
    const double v = oracle_half_to_double((uint16_t)h);
    const int sgn = (h >> 15) & 1, ex = (h >> 10) & 31, fr = h & 1023;
    double ref;
    if (ex == 31)
      ref = fr ? NAN : INFINITY;
    else if (ex == 0)
      ref = std::ldexp((double)fr, -24);
    else
      ref = std::ldexp(1024.0 + fr, ex - 25);
    if (sgn) ref = -ref;
    CHECK((std::isnan(v) && std::isnan(ref)) || (v == ref && std::signbit(v) == std::signbit(ref)));
  }

  // ---- oracle on random small layers: every function, masks with and without token bits
  for (int it = 0; it < 60; ++it) {
    const int d = irand(1, 40), n = irand(1, 50), r = irand(1, 12), B = irand(1, 64);
    const int gated = it % 2;
    const int wdt = it % 3 == 0 ? 0 : 1;  // fp32 or fp16 storage
    std::vector<float> X(B * d), ba(n), bo(d), c(n);
    for (auto& v : X) v = (float)uni(-1, 1);
    for (auto& v : ba) v = (float)uni(-1, 1);
    for (auto& v : bo) v = (float)uni(-1, 1);
    for (auto& v : c) v = (float)uni(-1, 1);
    auto weights = [&](int rows, int cols) {
      std::vector<uint8_t> w((size_t)rows * cols * (wdt ? 2 : 4));
      for (int i = 0; i < rows * cols; ++i) {
        if (wdt) {  // random finite fp16 of magnitude below 2 (exponent field at most 15)
          const uint16_t h = (uint16_t)((irand(0, 1) << 15) | (irand(0, 15) << 10) | irand(0, 1023));
          __builtin_memcpy(&w[2 * (size_t)i], &h, 2);
        } else {
          float g = (float)uni(-1, 1);
          __builtin_memcpy(&w[4 * (size_t)i], &g, 4);
        }
      }
      return w;
    };
    auto Wa = weights(n, d), Wu = weights(n, d), Wo = weights(n, d), P1 = weights(r, d),
         P2 = weights(n, r);
    std::vector<double> S(B * n), Q(B * r), Y(B * d), D(B * d), A(B * n);
    CHECK(oracle_predict(d, n, r, B, X.data(), P1.data(), P2.data(), wdt, c.data(), S.data(),
                         Q.data()) == 0);
    std::vector<uint8_t> M(B * n);
    CHECK(oracle_threshold(B, n, S.data(), 0.0, M.data()) == 0);
    std::vector<int32_t> idx(n);
    std::vector<uint64_t> tok(n);
    int32_t cnt = -1;
    CHECK(oracle_compact(B, n, M.data(), idx.data(), &cnt, tok.data()) == 0);
    CHECK(cnt >= 0 && cnt <= n);
    CHECK(oracle_forward(d, n, B, gated, X.data(), Wa.data(), Wu.data(), Wo.data(), wdt, ba.data(),
                         bo.data(), idx.data(), cnt, tok.data(), Y.data()) == 0);
    CHECK(oracle_forward(d, n, B, gated, X.data(), Wa.data(), Wu.data(), Wo.data(), wdt, nullptr,
                         nullptr, idx.data(), cnt, nullptr, Y.data()) == 0);
    // every neuron listed, no token bits: the forward equals the dense FFN exactly
    std::vector<int32_t> all(n);
    for (int i = 0; i < n; ++i) all[i] = i;
    CHECK(oracle_forward(d, n, B, gated, X.data(), Wa.data(), Wu.data(), Wo.data(), wdt, ba.data(),
                         bo.data(), all.data(), n, nullptr, Y.data()) == 0);
    CHECK(oracle_dense(d, n, B, gated, X.data(), Wa.data(), Wu.data(), Wo.data(), wdt, ba.data(),
                       bo.data(), D.data()) == 0);
    for (int k = 0; k < B * d; ++k) CHECK(Y[k] == D[k]);
    CHECK(oracle_preact(d, n, B, X.data(), Wa.data(), wdt, ba.data(), A.data()) == 0);
    std::vector<int64_t> counts(n);
    CHECK(oracle_profile_counts(d, n, B, X.data(), Wa.data(), wdt, ba.data(), counts.data()) == 0);
    for (int i = 0; i < n; ++i) {
      int64_t ref = 0;
      for (int b = 0; b < B; ++b) ref += A[(size_t)b * n + i] > 0.0;
      CHECK(counts[i] == ref);
    }
    std::vector<int32_t> perm(n);
    CHECK(oracle_permutation(counts.data(), n, n / 5, perm.data()) == 0);
    std::vector<uint8_t> packed(Wa.size());
    CHECK(oracle_pack_rows(Wa.data(), perm.data(), packed.data(), n,
                           (int64_t)d * (wdt ? 2 : 4)) == 0);
    // rejected arguments leave no trace
    CHECK(oracle_forward(d, n, B, gated, X.data(), Wa.data(), Wu.data(), Wo.data(), wdt, ba.data(),
                         bo.data(), idx.data(), n + 1, tok.data(), Y.data()) != 0);
    CHECK(oracle_compact(65, n, M.data(), idx.data(), &cnt, tok.data()) != 0);
  }
  std::printf("host and oracle checks: %d failures\n", failures);
  return failures == 0 ? 0 : 1;
}
