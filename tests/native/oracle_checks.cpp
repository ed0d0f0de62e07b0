// Memory and undefined-behaviour checks of the C++ oracle
// (oracle/nanospec_oracle.cpp), built together with it under AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_sanitizers.py (CPU only).
//
// Drives every exported function over edge sizes: windows of one slot,
// appends longer than the window, empty tuples, vocabularies of one id, an
// output capacity below |I|, empty projections, k above the candidate count,
// all three element types and several thread counts.  The results are only
// checked for shape (sorted, in range, padded); their values are pinned by
// the Python tests.  Exit status 0 when every check passes.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <cmath>
#include <random>
#include <vector>

extern "C" {
void* nso_seq_new(int w_max);
void nso_seq_free(void* p);
void nso_seq_append(void* p, const int32_t* ids, int n);
void nso_seq_step(void* p, const int32_t* tree, int nt, const int32_t* ver, int nv);
int64_t nso_seq_len(void* p);
int nso_seq_active(void* p, int32_t* out, int cap);
int nso_project(const void* W, int d, int dtype, const int32_t* I, int n, const void* h, int M, double* logits,
                int threads);
void nso_topk(const double* logits, const int32_t* I, int n, int M, int k, int64_t* ids, double* vals);
}

#define CHECK(c)                                                     \
  do {                                                               \
    if (!(c)) {                                                      \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      return 1;                                                      \
    }                                                                \
  } while (0)

namespace {

std::mt19937 rng(12345);

std::vector<int32_t> random_ids(int n, int V) {
  std::uniform_int_distribution<int> u(0, V - 1);
  std::vector<int32_t> v(n);
  for (auto& x : v) x = u(rng);
  return v;
}

uint16_t to_bf16(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  return (uint16_t)(b >> 16);
}

uint16_t to_fp16(float f) {                  // |f| < 2: normal or subnormal half, truncated
  uint16_t s = f < 0 ? 0x8000 : 0;
  double a = std::fabs((double)f);
  if (a < std::ldexp(1.0, -14)) return (uint16_t)(s | (uint16_t)(a / std::ldexp(1.0, -24)));
  int e;
  double m = std::frexp(a, &e);              // a = m 2^e, m in [0.5, 1)
  const int E = e - 1 + 15;
  const int F = (int)((m * 2.0 - 1.0) * 1024.0);
  return (uint16_t)(s | (E << 10) | F);
}

int check_sequences() {
  const int Vs[] = {1, 5, 300};
  const int Ws[] = {1, 2, 7, 64};
  for (int V : Vs)
    for (int w_max : Ws) {
      void* s = nso_seq_new(w_max);
      std::vector<int32_t> prompt = random_ids(3 * w_max + 1, V);
      nso_seq_append(s, prompt.data(), (int)prompt.size());
      nso_seq_append(s, nullptr, 0);
      int64_t len = (int64_t)prompt.size();
      for (int t = 0; t < 12; ++t) {
        std::vector<int32_t> tree = random_ids(t % 5 == 0 ? 0 : 2 * w_max + t, V);
        std::vector<int32_t> ver = random_ids(t % 3, V);
        nso_seq_step(s, tree.data(), (int)tree.size(), ver.data(), (int)ver.size());
        std::vector<bool> seen(V, false);
        int distinct = 0;
        for (int32_t x : tree)
          if (!seen[x]) { seen[x] = true; ++distinct; }
        len += distinct + (int64_t)ver.size();
        CHECK(nso_seq_len(s) == len);
        const int cap = t % 2 ? 1 : (w_max < V ? w_max : V);
        std::vector<int32_t> out(cap + 4, -7);
        const int n = nso_seq_active(s, out.data(), cap);
        CHECK(n >= 1 && n <= w_max && n <= V);
        for (int j = 0; j < n && j < cap; ++j) CHECK(out[j] >= 0 && out[j] < V);
        for (int j = 1; j < n && j < cap; ++j) CHECK(out[j - 1] < out[j]);
        for (int j = cap; j < cap + 4; ++j) CHECK(out[j] == -7);   // nothing past cap
      }
      nso_seq_free(s);
    }
  return 0;
}

int check_projection_and_topk() {
  std::normal_distribution<float> nd(0.f, 1.f);
  const int shapes[][4] = {{1, 8, 1, 1}, {9, 16, 3, 4}, {50, 24, 5, 0}, {17, 8, 2, 0}};   // V, d, M, n
  for (auto& sh : shapes) {
    const int V = sh[0], d = sh[1], M = sh[2];
    const int n = sh[3] ? (sh[3] < V ? sh[3] : V) : 0;
    std::vector<int32_t> I(n > 0 ? n : 1);
    for (int j = 0; j < n; ++j) I[j] = (int32_t)((j * 7 + 3) % V);
    for (int dtype = 0; dtype < 3; ++dtype) {
      const size_t esz = dtype == 1 ? 4 : 2;
      std::vector<unsigned char> W((size_t)V * d * esz), h((size_t)M * d * esz);
      for (size_t e = 0; e < (size_t)V * d; ++e) {
        const float f = nd(rng) * 0.02f;
        if (dtype == 1) memcpy(&W[e * 4], &f, 4);
        else { const uint16_t u = dtype == 0 ? to_bf16(f) : to_fp16(f); memcpy(&W[e * 2], &u, 2); }
      }
      for (size_t e = 0; e < (size_t)M * d; ++e) {
        const float f = nd(rng) * 0.5f;
        if (dtype == 1) memcpy(&h[e * 4], &f, 4);
        else { const uint16_t u = dtype == 0 ? to_bf16(f) : to_fp16(f); memcpy(&h[e * 2], &u, 2); }
      }
      for (int threads : {0, 1, 3}) {
        std::vector<double> z((size_t)M * (n > 0 ? n : 1), 0.0);
        const int used = nso_project(W.data(), d, dtype, I.data(), n, h.data(), M, z.data(), threads);
        CHECK(used >= 1);
        for (int j = 0; j < M * n; ++j) CHECK(std::isfinite(z[j]));
        for (int k : {1, n > 0 ? n : 1, n + 3}) {
          std::vector<int64_t> ids((size_t)M * k, 99);
          std::vector<double> vals((size_t)M * k, 0.0);
          nso_topk(z.data(), I.data(), n, M, k, ids.data(), vals.data());
          for (int m = 0; m < M; ++m)
            for (int r = 0; r < k; ++r) {
              const int64_t id = ids[(size_t)m * k + r];
              if (r < n) CHECK(id >= 0 && id < V);
              else CHECK(id == -1 && std::isinf(vals[(size_t)m * k + r]));
              if (r > 0 && r < n) CHECK(vals[(size_t)m * k + r - 1] >= vals[(size_t)m * k + r]);
            }
        }
      }
    }
  }
  // Ties and signed zeros.
  const double z[6] = {1.0, 2.0, 2.0, -0.0, 0.0, 2.0};
  const int32_t I[6] = {10, 3, 7, 1, 2, 5};
  int64_t ids[8];
  double vals[8];
  nso_topk(z, I, 6, 1, 8, ids, vals);
  const int64_t want[8] = {3, 5, 7, 10, 1, 2, -1, -1};
  for (int r = 0; r < 8; ++r) CHECK(ids[r] == want[r]);
  return 0;
}

}  // namespace

int main() {
  if (check_sequences()) return 1;
  if (check_projection_and_topk()) return 1;
  printf("oracle checks passed\n");
  return 0;
}
