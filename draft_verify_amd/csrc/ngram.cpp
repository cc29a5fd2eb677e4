// ngram.cpp -- n-gram prompt-lookup proposer and adaptive K (host C++).
//
// The proposer finds where the last few tokens occurred earlier in the
// history and proposes what followed them (TensorSharp speculative decoding
// page, n-gram section: an incrementally maintained index per n-gram order
// makes each lookup O(1)).  Orders run from n_max down to n_min (drafting only
// off a match of at least n_min tokens: coreai-model-zoo dense n-gram note,
// adaptive-K section).  The index keys are the exact token tuples, so a hash
// collision never proposes anything, and each key maps to its most recent end
// position, which gives the latest earlier occurrence.
#include <stdint.h>

#include <algorithm>
#include <array>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/specv.h"

namespace {

constexpr int kMaxOrder = 8;

struct Gram {
  std::array<int32_t, kMaxOrder> t;
  int n;
  bool operator==(const Gram& o) const {
    if (n != o.n) return false;
    for (int i = 0; i < n; ++i)
      if (t[i] != o.t[i]) return false;
    return true;
  }
};

struct GramHash {
  size_t operator()(const Gram& g) const {
    uint64_t h = 1469598103934665603ull ^ (uint64_t)g.n;
    for (int i = 0; i < g.n; ++i) {
      h ^= (uint32_t)g.t[i];
      h *= 1099511628211ull;
    }
    return (size_t)(h ^ (h >> 29));
  }
};

}  // namespace

struct spec_ngram {
  int n_min, n_max, capacity;
  std::vector<int32_t> h;
  std::vector<std::unordered_map<Gram, int32_t, GramHash>> index;  // per order

  Gram gram_ending_at(int e, int n) const {
    Gram g;
    g.n = n;
    for (int i = 0; i < n; ++i) g.t[i] = h[e - n + 1 + i];
    return g;
  }
  // After h grows to length L, the occurrence ending at L-2 becomes eligible
  // (an occurrence must end before the suffix's own last token).
  void index_end(int e) {
    for (int n = n_min; n <= n_max; ++n)
      if (e - n + 1 >= 0) index[n - n_min][gram_ending_at(e, n)] = e;
  }
};

extern "C" {

int spec_ngram_create(int n_min, int n_max, int capacity, spec_ngram** out) {
  if (!out || n_min < 1 || n_max < n_min || n_max > kMaxOrder || capacity < 0) return SPEC_EINVAL;
  spec_ngram* ng = new (std::nothrow) spec_ngram;
  if (!ng) return SPEC_ECAPACITY;
  ng->n_min = n_min;
  ng->n_max = n_max;
  ng->capacity = capacity;
  ng->h.reserve((size_t)capacity);
  ng->index.resize((size_t)(n_max - n_min + 1));
  *out = ng;
  return SPEC_OK;
}

int spec_ngram_destroy(spec_ngram* ng) {
  delete ng;
  return SPEC_OK;
}

int spec_ngram_append(spec_ngram* ng, const int32_t* toks, int n) {
  if (!ng || (n > 0 && !toks) || n < 0) return SPEC_EINVAL;
  if ((int64_t)ng->h.size() + n > ng->capacity) return SPEC_ECAPACITY;
  for (int i = 0; i < n; ++i) {
    ng->h.push_back(toks[i]);
    const int L = (int)ng->h.size();
    if (L >= 2) ng->index_end(L - 2);
  }
  return SPEC_OK;
}

int spec_ngram_truncate(spec_ngram* ng, int len) {
  if (!ng || len < 0) return SPEC_EINVAL;
  if (len > (int)ng->h.size()) return SPEC_ESTATE;
  ng->h.resize((size_t)len);
  for (auto& m : ng->index) m.clear();
  for (int e = 0; e + 2 <= len; ++e) ng->index_end(e);
  return SPEC_OK;
}

int spec_ngram_len(spec_ngram* ng) { return ng ? (int)ng->h.size() : SPEC_EINVAL; }

int spec_ngram_propose(spec_ngram* ng, int K, int32_t* drafts) {
  if (!ng || K < 0 || (K > 0 && !drafts)) return SPEC_EINVAL;
  const int L = (int)ng->h.size();
  if (K == 0) return 0;
  for (int n = ng->n_max; n >= ng->n_min; --n) {
    if (L < n + 1) continue;
    const auto& m = ng->index[n - ng->n_min];
    auto it = m.find(ng->gram_ending_at(L - 1, n));
    if (it == m.end()) continue;
    int c = 0;
    for (int i = it->second + 1; i <= L - 1 && c < K; ++i) drafts[c++] = ng->h[i];
    return c;
  }
  return 0;
}

int spec_adapt_k(int k, int drafted, int accepted, int k_cap) {
  if (drafted <= 0) return k;
  int next = accepted >= drafted ? k + 2 : k - 1;
  return std::max(1, std::min(next, k_cap));
}

}  // extern "C"
