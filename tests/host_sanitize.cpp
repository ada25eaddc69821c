// Host entry points of the C ABI run under AddressSanitizer and
// UndefinedBehaviorSanitizer (built by tests/test_host_sanitize.py with g++,
// linking the library's host source directly; no device code).
//
// Reads a stream of cases (op code and arguments, little-endian) from the
// file named by argv[1] and writes, per case, the status code and, when it is
// HK_OK, the outputs, to the file named by argv[2].  The test compares them
// with the same calls on the production library.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "heatkv.h"

namespace {

FILE* in = nullptr;
FILE* out = nullptr;

template <typename T>
T get() {
  T v;
  if (std::fread(&v, sizeof(T), 1, in) != 1) {
    std::fprintf(stderr, "truncated input\n");
    std::exit(3);
  }
  return v;
}

template <typename T>
std::vector<T> get_vec(size_t n) {
  std::vector<T> v(n);
  if (n && std::fread(v.data(), sizeof(T), n, in) != n) {
    std::fprintf(stderr, "truncated input\n");
    std::exit(3);
  }
  return v;
}

template <typename T>
void put(const T* p, size_t n) {
  if (n) std::fwrite(p, sizeof(T), n, out);
}

template <typename T>
void put1(T v) {
  put(&v, 1);
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) return 2;
  in = std::fopen(argv[1], "rb");
  out = std::fopen(argv[2], "wb");
  if (!in || !out) return 2;
  int32_t op;
  while (std::fread(&op, sizeof(op), 1, in) == 1) {
    const int L = get<int32_t>(), H = get<int32_t>(), K = get<int32_t>();
    const size_t lh = size_t(L) * H, lhk = lh * K, lhkk = lhk * K;
    int rc = 0;
    if (op == 9) {  // hk_scas_mean
      const auto sum = get_vec<double>(lhkk);
      const double images = get<double>();
      std::vector<float> res(lhkk);
      rc = hk_scas_mean(L, H, K, sum.data(), images, res.data());
      put1<int32_t>(rc);
      if (rc == HK_OK) put(res.data(), res.size());
      continue;
    }
    const auto tok = get_vec<int32_t>(K);
    if (op == 1) {  // hk_build_schedule
      const auto scas = get_vec<float>(lhkk);
      const double beta = get<double>();
      const int n_sink = get<int32_t>();
      std::vector<uint8_t> keep(lhk);
      std::vector<int64_t> ret(K);
      int32_t npr = -1;
      rc = hk_build_schedule(L, H, K, tok.data(), scas.data(), beta, n_sink, keep.data(), ret.data(),
                             &npr);
      put1<int32_t>(rc);
      if (rc == HK_OK) {
        put(keep.data(), keep.size());
        put(ret.data(), ret.size());
        put1<int32_t>(npr);
      }
    } else if (op == 2) {  // hk_build_progressive_schedule
      const auto scas = get_vec<float>(lhkk);
      const double beta = get<double>();
      const int n_sink = get<int32_t>(), per_layer = get<int32_t>();
      std::vector<uint8_t> expire(lhk);
      std::vector<int32_t> prefix(K);
      std::vector<int64_t> live(size_t(K) * L);
      rc = hk_build_progressive_schedule(L, H, K, tok.data(), scas.data(), beta, n_sink, per_layer,
                                         expire.data(), prefix.data(), live.data());
      put1<int32_t>(rc);
      if (rc == HK_OK) {
        put(expire.data(), expire.size());
        put(prefix.data(), prefix.size());
        put(live.data(), live.size());
      }
    } else if (op == 3 || op == 8) {  // hk_layout_expiry / hk_layout
      const auto sched = get_vec<uint8_t>(lhk);
      const int B = get<int32_t>(), D = get<int32_t>();
      int64_t elems = -1;
      std::vector<int64_t> cap(lh), base(lh);
      rc = op == 3 ? hk_layout_expiry(L, H, K, tok.data(), sched.data(), B, D, &elems, cap.data(),
                                      base.data())
                   : hk_layout(L, H, K, tok.data(), sched.data(), B, D, &elems, cap.data(),
                               base.data());
      put1<int32_t>(rc);
      if (rc == HK_OK) {
        put1<int64_t>(elems);
        put(cap.data(), cap.size());
        put(base.data(), base.size());
      }
    } else if (op == 4) {  // hk_cache_size_after_layer
      const auto expire = get_vec<uint8_t>(lhk);
      const int step = get<int32_t>(), layer = get<int32_t>();
      int64_t size = -1;
      rc = hk_cache_size_after_layer(L, H, K, tok.data(), expire.data(), step, layer, &size);
      put1<int32_t>(rc);
      if (rc == HK_OK) put1<int64_t>(size);
    } else if (op == 5) {  // hk_build_scale_window_schedule
      const int nc = get<int32_t>(), w = get<int32_t>(), wd = get<int32_t>();
      const auto sim = get_vec<float>(L);
      const int nd = get<int32_t>();
      std::vector<uint8_t> expire(lhk);
      rc = hk_build_scale_window_schedule(L, H, K, tok.data(), nc, w, wd, sim.data(), nd,
                                          expire.data());
      put1<int32_t>(rc);
      if (rc == HK_OK) put(expire.data(), expire.size());
    } else if (op == 6) {  // hk_layout_int4
      const auto keep = get_vec<uint8_t>(lhk);
      const int B = get<int32_t>(), D = get<int32_t>(), m = get<int32_t>();
      int64_t store = -1, param = -1;
      rc = hk_layout_int4(L, H, K, tok.data(), keep.data(), B, D, m, &store, &param);
      put1<int32_t>(rc);
      if (rc == HK_OK) {
        put1<int64_t>(store);
        put1<int64_t>(param);
      }
    } else if (op == 7) {  // hk_ranking_stability
      const auto a = get_vec<float>(lhkk);
      const auto b = get_vec<float>(lhkk);
      const double beta = get<double>();
      const int n_sink = get<int32_t>();
      std::vector<double> rho(K);
      double jac = -1;
      rc = hk_ranking_stability(L, H, K, tok.data(), a.data(), b.data(), beta, n_sink, rho.data(),
                                &jac);
      put1<int32_t>(rc);
      if (rc == HK_OK) {
        put(rho.data(), rho.size());
        put1<double>(jac);
      }
    } else {
      std::fprintf(stderr, "unknown op %d\n", op);
      return 3;
    }
  }
  std::fclose(out);
  std::fclose(in);
  return 0;
}
