// C++17 CPU oracle of the dynamic-vocabulary draft step.
//
// TEST INFRASTRUCTURE ONLY.  Nothing on the product path links or calls this
// library: it is loaded by tests/ (cross-checked against the numpy oracle,
// oracle/nanospec_oracle.py) and by bench.py's cpu_baseline leg, which times
// the decode step on the host's cores.  It shares no code with the HIP path.
//
// Every result is the plain definition written out (MicroSpec/NanoSpec,
// arXiv 2605.26444):
//   * Sec. 3.2 "Dynamic Stream Update (Decoding Phase)":
//       S_new = S_old (+) tuple(C_draft) (+) tuple(C_ver), C_draft the distinct
//       ids of the draft tree in first-occurrence order, C_ver as given;
//   * Sec. 3.2 "Vocabulary Construction via Sliding Window":
//       I = Unique(Suffix(S, W_max)) in ascending id order (the suffix is all
//       of S while |S| < W_max);
//   * Sec. 3.1 Eq. 1 restricted to W_head[I, :]:
//       z[m][j] = sum over c = 0 .. d-1, ascending, of h[m][c] * W[I[j]][c],
//       each product and sum in float64 (no fused multiply-add, no
//       reordering; the inputs widen exactly);
//   * Sec. 3.2 T_K: per hidden row the k largest (value desc, id asc),
//       padded with (-1, -inf) when k > |I|.
// The projection may run its (m, j) pairs on several OpenMP threads; each
// pair's sum is the same sequential loop, so the result does not depend on
// the thread count.
#include <omp.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cstddef>
#include <cmath>
#include <limits>
#include <unordered_set>
#include <vector>

namespace {

struct Sequence {
  int w_max;
  std::vector<int32_t> S;
};

// Exact float64 value of a stored element: dtype 0 bf16 (bits << 16 is the
// float32), 1 float32, 2 IEEE binary16 decoded from its fields.
double widen(const void* base, size_t idx, int dtype) {
  if (dtype == 1) return (double)static_cast<const float*>(base)[idx];
  const uint16_t u = static_cast<const uint16_t*>(base)[idx];
  if (dtype == 0) {
    const uint32_t b = (uint32_t)u << 16;
    float f;
    memcpy(&f, &b, 4);
    return (double)f;
  }
  const double sign = (u >> 15) ? -1.0 : 1.0;
  const int e = (u >> 10) & 0x1F;
  const double f = (double)(u & 0x3FF);
  const double mag = e == 0 ? f * std::ldexp(1.0, -24) : (1024.0 + f) * std::ldexp(1.0, e - 25);
  return sign * mag;
}

}  // namespace

extern "C" {

void* nso_seq_new(int w_max) {
  Sequence* s = new Sequence;
  s->w_max = w_max;
  return s;
}

void nso_seq_free(void* p) { delete static_cast<Sequence*>(p); }

// Appends ids as given (the prompt).
void nso_seq_append(void* p, const int32_t* ids, int n) {
  Sequence* s = static_cast<Sequence*>(p);
  s->S.insert(s->S.end(), ids, ids + n);
}

// One decode step: S += first occurrences of the tree ids, then the verify ids.
void nso_seq_step(void* p, const int32_t* tree, int nt, const int32_t* ver, int nv) {
  Sequence* s = static_cast<Sequence*>(p);
  std::unordered_set<int32_t> seen;
  for (int i = 0; i < nt; ++i)
    if (seen.insert(tree[i]).second) s->S.push_back(tree[i]);
  s->S.insert(s->S.end(), ver, ver + nv);
}

int64_t nso_seq_len(void* p) { return (int64_t)static_cast<Sequence*>(p)->S.size(); }

// I = sorted unique ids of the last w_max entries; returns |I| (ids written
// to out while they fit in cap).
int nso_seq_active(void* p, int32_t* out, int cap) {
  Sequence* s = static_cast<Sequence*>(p);
  const size_t len = s->S.size();
  const size_t from = len > (size_t)s->w_max ? len - (size_t)s->w_max : 0;
  std::vector<int32_t> w(s->S.begin() + (std::ptrdiff_t)from, s->S.end());
  std::sort(w.begin(), w.end());
  w.erase(std::unique(w.begin(), w.end()), w.end());
  for (size_t j = 0; j < w.size() && (int)j < cap; ++j) out[j] = w[j];
  return (int)w.size();
}

// logits[m * n + j] = sum_c h[m][c] * W[I[j]][c] in float64, c ascending.
// `threads` OpenMP threads share the (m, j) pairs (0: the OpenMP default);
// returns the number of threads that ran.
int nso_project(const void* W, int d, int dtype, const int32_t* I, int n, const void* h, int M, double* logits,
                int threads) {
  // h is kept as [c][m], so the M sums of one row advance together over c
  // (each sum still adds its products in ascending c).
  std::vector<double> ht((size_t)M * d);
  for (int m = 0; m < M; ++m)
    for (int c = 0; c < d; ++c) ht[(size_t)c * M + m] = widen(h, (size_t)m * d + c, dtype);
  int used = 1;
  const int nth = threads > 0 ? threads : omp_get_max_threads();
#pragma omp parallel num_threads(nth)
  {
#pragma omp single
    used = omp_get_num_threads();
    std::vector<double> acc(M);
#pragma omp for schedule(static)
    for (int j = 0; j < n; ++j) {
      for (int m = 0; m < M; ++m) acc[m] = 0.0;
      for (int c = 0; c < d; ++c) {
        const double w = widen(W, (size_t)I[j] * d + c, dtype);
        const double* hc = ht.data() + (size_t)c * M;
        for (int m = 0; m < M; ++m) {
          const double prod = hc[m] * w;
          acc[m] = acc[m] + prod;
        }
      }
      for (int m = 0; m < M; ++m) logits[(size_t)m * n + j] = acc[m];
    }
  }
  return used;
}

// Per row m: the k best (value desc, id asc) of (logits[m][j], I[j]).
void nso_topk(const double* logits, const int32_t* I, int n, int M, int k, int64_t* ids, double* vals) {
  std::vector<int> order(n);
  for (int m = 0; m < M; ++m) {
    const double* z = logits + (size_t)m * n;
    for (int j = 0; j < n; ++j) order[j] = j;
    std::sort(order.begin(), order.end(), [&](int a, int b) {
      if (z[a] != z[b]) return z[a] > z[b];
      return I[a] < I[b];
    });
    for (int r = 0; r < k; ++r) {
      ids[(size_t)m * k + r] = r < n ? I[order[r]] : -1;
      vals[(size_t)m * k + r] = r < n ? z[order[r]] : -std::numeric_limits<double>::infinity();
    }
  }
}

}  // extern "C"
