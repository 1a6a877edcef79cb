// Native driver for the C ABI's host-side code: shape checks, workspace
// sizes, argument validation and status strings, over shapes up to and past
// every documented limit.  tests/test_abi_sanitized.py builds it together
// with the library's host code under AddressSanitizer and
// UndefinedBehaviorSanitizer (host pass only) and runs it.  No call made
// here gets as far as a kernel launch: every rejected call returns before
// touching a pointer, and the pointers passed are never dereferenced.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "clsa.h"

namespace {

int g_fail = 0;

#define EXPECT(c)                                                               \
  do {                                                                          \
    if (!(c)) {                                                                 \
      std::fprintf(stderr, "expectation failed at line %d: %s\n", __LINE__, #c); \
      ++g_fail;                                                                 \
    }                                                                           \
  } while (0)

// stands in for device buffers: validation must reject before any use
void* const kFake = reinterpret_cast<void*>(uintptr_t{0x1000});

bool route_shape_valid(int B, int M, int d, int64_t n_cap, int cap) {
  return B >= 1 && M >= 1 && cap >= 1 && (d == 32 || d == 64 || d == 128) && n_cap >= 1 &&
         n_cap <= 0x7fffffffLL && int64_t{B} * M <= 65535;
}

void route_sizes() {
  const int Bs[] = {-1, 0, 1, 2, 8, 255, 256, 65535, 65536, 1 << 30};
  const int Ms[] = {-3, 0, 1, 63, 64, 4096, 65535, 65536};
  const int ds[] = {0, 16, 32, 48, 64, 128, 256};
  const int64_t ns[] = {-5, 0, 1, 4095, 4096, 131072, 524288, 524289, 0x7fffffffLL,
                        0x80000000LL, int64_t{1} << 40};
  const int ks[] = {-1, 0, 1, 256, 2048, 2049, 8192, 1 << 20};
  const clsa_dtype dts[] = {CLSA_BF16, CLSA_F32};
  for (int B : Bs)
    for (int M : Ms)
      for (int d : ds)
        for (int64_t n : ns)
          for (int k : ks)
            for (clsa_dtype dt : dts) {
              const size_t w = clsa_route_workspace_size(B, M, d, n, k, k, dt);
              const size_t wt = clsa_route_threshold_workspace_size(B, M, d, n, k, dt);
              const bool ok = route_shape_valid(B, M, d, n, k);
              if (!ok || k < 1) EXPECT(w == 0);
              if (!ok) EXPECT(wt == 0);
              if (ok) EXPECT(wt > 0);
              if (ok && k >= 1) EXPECT(w > 0);
            }
}

void attn_sizes() {
  const int Ls[] = {-1, 0, 1, 16, 64, 65};
  const int Bs[] = {0, 1, 8, 65535, 65536};
  const int Ms[] = {0, 1, 4096};
  const int heads[][2] = {{32, 8}, {8, 8}, {64, 4}, {30, 8}, {4, 0}, {128, 64}, {1024, 64}};
  const int Ds[] = {0, 8, 64, 128, 130, 256, 264};
  const int caps[] = {0, 1, 300, 2048, 8192, 1 << 20};
  const clsa_dtype dts[] = {CLSA_BF16, CLSA_F32};
  for (int L : Ls)
    for (int B : Bs)
      for (int M : Ms)
        for (const auto& h : heads)
          for (int D : Ds)
            for (int cap : caps)
              for (clsa_dtype dt : dts) {
                const size_t w = clsa_sparse_attn_workspace_size(L, B, M, h[0], h[1], D, cap, dt);
                if (L < 1 || L > 64 || B < 1 || M < 1 || cap < 1 || h[1] < 1 || D % 8 != 0)
                  EXPECT(w == 0);
              }
}

void route_rejects() {
  // a valid base call, each case breaking one argument
  struct Case {
    const void *q, *K;
    int B, M, d;
    int64_t n_cap;
    int k;
    int dt;
    int32_t *idx, *counts;
    int cap;
    void* ws;
    size_t ws_bytes;
    int want;
  };
  int32_t* fi = static_cast<int32_t*>(kFake);
  const size_t big = size_t{1} << 40;
  const Case cases[] = {
      {nullptr, kFake, 1, 1, 64, 4096, 256, CLSA_BF16, fi, fi, 256, kFake, big, CLSA_ERR_INVALID},
      {kFake, nullptr, 1, 1, 64, 4096, 256, CLSA_BF16, fi, fi, 256, kFake, big, CLSA_ERR_INVALID},
      {kFake, kFake, 1, 1, 64, 4096, 256, CLSA_BF16, nullptr, fi, 256, kFake, big, CLSA_ERR_INVALID},
      {kFake, kFake, 1, 1, 64, 4096, 256, CLSA_BF16, fi, nullptr, 256, kFake, big, CLSA_ERR_INVALID},
      {kFake, kFake, 0, 1, 64, 4096, 256, CLSA_BF16, fi, fi, 256, kFake, big, CLSA_ERR_INVALID},
      {kFake, kFake, 1, 0, 64, 4096, 256, CLSA_BF16, fi, fi, 256, kFake, big, CLSA_ERR_INVALID},
      {kFake, kFake, 1, 1, 48, 4096, 256, CLSA_BF16, fi, fi, 256, kFake, big, CLSA_ERR_INVALID},
      {kFake, kFake, 1, 1, 64, 0, 256, CLSA_BF16, fi, fi, 256, kFake, big, CLSA_ERR_INVALID},
      {kFake, kFake, 1, 1, 64, 0x80000000LL, 256, CLSA_BF16, fi, fi, 256, kFake, big,
       CLSA_ERR_INVALID},
      {kFake, kFake, 1, 1, 64, 4096, 0, CLSA_BF16, fi, fi, 256, kFake, big, CLSA_ERR_INVALID},
      {kFake, kFake, 1, 1, 64, 4096, 256, CLSA_BF16, fi, fi, 100, kFake, big, CLSA_ERR_INVALID},
      {kFake, kFake, 256, 256, 64, 4096, 256, CLSA_BF16, fi, fi, 256, kFake, big,
       CLSA_ERR_INVALID},
      {kFake, kFake, 1, 1, 64, 4096, 256, 7, fi, fi, 256, kFake, big, CLSA_ERR_UNSUPPORTED_DTYPE},
      {kFake, kFake, 1, 1, 64, 4096, 256, CLSA_BF16, fi, fi, 256, nullptr, big, CLSA_ERR_WORKSPACE},
      {kFake, kFake, 1, 1, 64, 4096, 256, CLSA_BF16, fi, fi, 256, kFake, 1024, CLSA_ERR_WORKSPACE},
      {kFake, kFake, 1, 4096, 64, 131072, 2048, CLSA_BF16, fi, fi, 2048, kFake, 4096,
       CLSA_ERR_WORKSPACE},
      {kFake, kFake, 8, 1, 64, 131072, 2048, CLSA_F32, fi, fi, 2048, kFake, 4096,
       CLSA_ERR_WORKSPACE},
  };
  for (const Case& c : cases) {
    const int st = clsa_route(c.q, c.K, c.B, c.M, c.d, c.n_cap, nullptr, -1, c.k,
                              static_cast<clsa_dtype>(c.dt), c.idx, c.counts, c.cap, c.ws,
                              c.ws_bytes, nullptr);
    EXPECT(st == c.want);
  }
  // the allocation-free variant validates the same way, then refuses shapes
  // that need more than its fixed array, all before any GPU call
  EXPECT(clsa_route_static(nullptr, kFake, 1, 1, 64, 4096, nullptr, -1, 256, CLSA_BF16, fi, fi,
                           256, nullptr) == CLSA_ERR_INVALID);
  EXPECT(clsa_route_static(kFake, kFake, 1, 1, 64, 4096, nullptr, -1, 256,
                           static_cast<clsa_dtype>(5), fi, fi, 256, nullptr) ==
         CLSA_ERR_UNSUPPORTED_DTYPE);
  EXPECT(clsa_route_static(kFake, kFake, 114, 1, 64, 131072, nullptr, -1, 2048, CLSA_BF16, fi, fi,
                           2048, nullptr) == CLSA_ERR_SCRATCH_LIMIT);
  EXPECT(clsa_route_static(kFake, kFake, 1, 4096, 64, 131072, nullptr, -1, 2048, CLSA_BF16, fi,
                           fi, 2048, nullptr) == CLSA_ERR_SCRATCH_LIMIT);
  const float* ft = static_cast<const float*>(kFake);
  EXPECT(clsa_route_threshold(kFake, kFake, 1, 1, 64, 4096, nullptr, -1, nullptr, CLSA_BF16, fi,
                              fi, 64, kFake, big, nullptr) == CLSA_ERR_INVALID);
  EXPECT(clsa_route_threshold(kFake, kFake, 1, 1, 64, 4096, nullptr, -1, ft, CLSA_BF16, fi, fi,
                              0, kFake, big, nullptr) == CLSA_ERR_INVALID);
  EXPECT(clsa_route_threshold(kFake, kFake, 1, 1, 64, 4096, nullptr, -1, ft, CLSA_BF16, fi, fi,
                              64, kFake, 16, nullptr) == CLSA_ERR_WORKSPACE);
  EXPECT(clsa_route_threshold(kFake, kFake, 1, 1, 64, 4096, nullptr, -1, ft,
                              static_cast<clsa_dtype>(3), fi, fi, 64, kFake, big,
                              nullptr) == CLSA_ERR_UNSUPPORTED_DTYPE);
}

void attn_rejects() {
  const void* p[65];
  void* o[65];
  for (int l = 0; l < 65; ++l) {
    p[l] = kFake;
    o[l] = kFake;
  }
  const int32_t* fi = static_cast<const int32_t*>(kFake);
  const size_t big = size_t{1} << 40;
  auto call = [&](int L, int Hq, int Hkv, int D, int cap, float scale, int dt, const int32_t* idx,
                  void* ws, size_t ws_bytes) {
    return clsa_sparse_attn(L, 1, 1, Hq, Hkv, D, p, p, p, 131072, idx, fi, cap, scale,
                            static_cast<clsa_dtype>(dt), o, nullptr, ws, ws_bytes, nullptr);
  };
  EXPECT(call(0, 32, 8, 128, 2048, 0.f, CLSA_BF16, fi, kFake, big) == CLSA_ERR_INVALID);
  EXPECT(call(65, 32, 8, 128, 2048, 0.f, CLSA_BF16, fi, kFake, big) == CLSA_ERR_INVALID);
  EXPECT(call(2, 30, 8, 128, 2048, 0.f, CLSA_BF16, fi, kFake, big) == CLSA_ERR_INVALID);
  EXPECT(call(2, 64, 2, 128, 2048, 0.f, CLSA_BF16, fi, kFake, big) == CLSA_ERR_INVALID);
  EXPECT(call(2, 32, 8, 130, 2048, 0.f, CLSA_BF16, fi, kFake, big) == CLSA_ERR_INVALID);
  EXPECT(call(2, 32, 8, 264, 2048, 0.f, CLSA_BF16, fi, kFake, big) == CLSA_ERR_INVALID);
  EXPECT(call(2, 32, 8, 128, 0, 0.f, CLSA_BF16, fi, kFake, big) == CLSA_ERR_INVALID);
  EXPECT(call(2, 32, 8, 128, 2048, -1.f, CLSA_BF16, fi, kFake, big) == CLSA_ERR_INVALID);
  EXPECT(call(2, 32, 8, 128, 2048, __builtin_inff(), CLSA_BF16, fi, kFake, big) == CLSA_ERR_INVALID);
  EXPECT(call(2, 32, 8, 128, 2048, 0.f, 5, fi, kFake, big) == CLSA_ERR_UNSUPPORTED_DTYPE);
  EXPECT(call(2, 32, 8, 128, 2048, 0.f, CLSA_BF16, nullptr, kFake, big) == CLSA_ERR_INVALID);
  EXPECT(call(16, 32, 8, 128, 2048, 0.f, CLSA_BF16, fi, nullptr, big) == CLSA_ERR_WORKSPACE);
  EXPECT(call(16, 32, 8, 128, 2048, 0.f, CLSA_BF16, fi, kFake, 8) == CLSA_ERR_WORKSPACE);
  p[1] = nullptr;
  EXPECT(call(2, 32, 8, 128, 2048, 0.f, CLSA_BF16, fi, kFake, big) == CLSA_ERR_INVALID);
  p[1] = kFake;
  o[1] = nullptr;
  EXPECT(call(2, 32, 8, 128, 2048, 0.f, CLSA_BF16, fi, kFake, big) == CLSA_ERR_INVALID);
  EXPECT(clsa_sparse_attn(2, 1, 1, 32, 8, 128, nullptr, p, p, 131072, fi, fi, 2048, 0.f,
                          CLSA_BF16, o, nullptr, kFake, big, nullptr) == CLSA_ERR_INVALID);
}

void append_rejects() {
  void* a[65];
  for (int l = 0; l < 65; ++l) a[l] = kFake;
  const int32_t* fi = static_cast<const int32_t*>(kFake);
  const void* const* ca = a;
  EXPECT(clsa_kv_append(2, 8, 8, 128, 64, 4096, nullptr, kFake, kFake, ca, a, ca, a, CLSA_BF16,
                        nullptr) == CLSA_ERR_INVALID);
  EXPECT(clsa_kv_append(2, 8, 8, 128, 64, 4096, fi, kFake, nullptr, ca, a, ca, a, CLSA_BF16,
                        nullptr) == CLSA_ERR_INVALID);
  EXPECT(clsa_kv_append(2, 8, 8, 128, 12, 4096, fi, kFake, kFake, ca, a, ca, a, CLSA_BF16,
                        nullptr) == CLSA_ERR_INVALID);
  EXPECT(clsa_kv_append(65, 8, 8, 128, 64, 4096, fi, kFake, kFake, ca, a, ca, a, CLSA_BF16,
                        nullptr) == CLSA_ERR_INVALID);
  EXPECT(clsa_kv_append(2, 8, 8, 128, 64, 4096, fi, kFake, kFake, ca, a, ca, a,
                        static_cast<clsa_dtype>(9), nullptr) == CLSA_ERR_UNSUPPORTED_DTYPE);
  a[1] = nullptr;
  EXPECT(clsa_kv_append(2, 8, 8, 128, 64, 4096, fi, kFake, kFake, ca, a, ca, a, CLSA_BF16,
                        nullptr) == CLSA_ERR_INVALID);
}

void router_paths() {
  const int32_t* fi = static_cast<const int32_t*>(kFake);
  int32_t* o = static_cast<int32_t*>(kFake);
  const size_t big = size_t{1} << 40;
  // aggregated routing: sizes over head counts and shapes, then rejects
  const int Hs[] = {-1, 0, 1, 16, 64, 65, 1 << 20};
  for (int H : Hs)
    for (int64_t n : {int64_t{1}, int64_t{131072}, int64_t{524289}, int64_t{1} << 40}) {
      const size_t w = clsa_route_aggregated_workspace_size(H, 8, 1, 64, n, 2048, 2048, CLSA_BF16);
      EXPECT((w == 0) == (H < 1 || H > 64 || !route_shape_valid(8, 1, 64, n, 2048)));
    }
  const void* hp[64];
  for (int h = 0; h < 64; ++h) hp[h] = kFake;
  EXPECT(clsa_route_aggregated(0, hp, hp, 2, 1, 64, 4096, nullptr, -1, 64, CLSA_BF16, o, o, 64,
                               kFake, big, nullptr) == CLSA_ERR_INVALID);
  EXPECT(clsa_route_aggregated(65, hp, hp, 2, 1, 64, 4096, nullptr, -1, 64, CLSA_BF16, o, o, 64,
                               kFake, big, nullptr) == CLSA_ERR_INVALID);
  EXPECT(clsa_route_aggregated(2, nullptr, hp, 2, 1, 64, 4096, nullptr, -1, 64, CLSA_BF16, o, o,
                               64, kFake, big, nullptr) == CLSA_ERR_INVALID);
  EXPECT(clsa_route_aggregated(2, hp, hp, 2, 1, 64, 4096, nullptr, -1, 64,
                               static_cast<clsa_dtype>(4), o, o, 64, kFake, big, nullptr) ==
         CLSA_ERR_UNSUPPORTED_DTYPE);
  EXPECT(clsa_route_aggregated(2, hp, hp, 2, 1, 64, 4096, nullptr, -1, 64, CLSA_BF16, o, o, 64,
                               nullptr, 0, nullptr) == CLSA_ERR_WORKSPACE);
  // centroid table: sizes up to and past every limit
  const int Cs[] = {-1, 0, 1, 64, 256, 512, 1024, 1025, 1 << 20};
  const int Ts[] = {-1, 0, 1, 2048, 2049};
  const int ds[] = {16, 32, 64, 128};
  for (int C : Cs)
    for (int T : Ts)
      for (int d : ds) {
        const bool ok = C >= 1 && C <= 1024 && T >= 1 && T <= 2048 &&
                        (d == 32 || d == 64 || d == 128) && int64_t{C} * d * 4 <= 65536;
        const size_t wb = clsa_csa_build_workspace_size(8, 4096, d, 131072, C, T);
        EXPECT((wb > 0) == (ok && C <= 4096));
        for (int P : {0, 1, 3, 16, 17}) {
          const size_t wr = clsa_csa_route_workspace_size(8, d, 131072, C, T, P);
          EXPECT((wr > 0) == (ok && P >= 1 && P <= 16 && P <= C));
        }
      }
  EXPECT(clsa_csa_build_workspace_size(1 << 20, 1 << 20, 64, 131072, 64, 256) == 0);
  EXPECT(clsa_csa_build(kFake, kFake, 2, 256, 64, 4096, nullptr, 16, 4, 256, CLSA_F32, kFake, o,
                        kFake, big, nullptr) == CLSA_ERR_UNSUPPORTED_DTYPE);
  EXPECT(clsa_csa_build(kFake, kFake, 5000, 256, 64, 4096, nullptr, 16, 4, 256, CLSA_BF16, kFake,
                        o, kFake, big, nullptr) == CLSA_ERR_INVALID);
  EXPECT(clsa_csa_build(kFake, kFake, 2, 256, 64, 4096, nullptr, 16, 101, 256, CLSA_BF16, kFake,
                        o, kFake, big, nullptr) == CLSA_ERR_INVALID);
  EXPECT(clsa_csa_build(kFake, kFake, 2, 256, 64, 4096, nullptr, 16, 4, 256, CLSA_BF16, kFake, o,
                        kFake, 16, nullptr) == CLSA_ERR_WORKSPACE);
  EXPECT(clsa_csa_route(kFake, kFake, 2, 64, int64_t{1} << 40, nullptr, kFake, fi, 16, 256, 0, 4,
                        64, CLSA_BF16, o, o, 64, kFake, big, nullptr) == CLSA_ERR_INVALID);
  EXPECT(clsa_csa_route(kFake, kFake, 2, 64, 8192, nullptr, kFake, fi, 16, 256, 1000, 4, 64,
                        CLSA_BF16, o, o, 64, kFake, big, nullptr) == CLSA_ERR_INVALID);
  EXPECT(clsa_csa_route(kFake, kFake, 2, 64, 4096, nullptr, kFake, fi, 16, 256, 4000, 4, 64,
                        CLSA_BF16, o, o, 64, kFake, 8, nullptr) == CLSA_ERR_WORKSPACE);
  // Louver index: sizes over extreme shapes (no overflow, zero when refused)
  for (int64_t n : {int64_t{-1}, int64_t{0}, int64_t{1}, int64_t{131072}, int64_t{1} << 24,
                    (int64_t{1} << 24) + 1, int64_t{1} << 40})
    for (int S : {0, 1, 2, 3, 4, 8})
      for (int r : {0, 8, 64, 256, 257}) {
        const size_t ib = clsa_louver_index_bytes(16, 128, n, S, r);
        const size_t wb = clsa_louver_build_workspace_size(16, 128, n, S, r);
        EXPECT((ib == 0) == (wb == 0));
        if (n < 1 || n > (int64_t{1} << 24)) EXPECT(ib == 0);
      }
}

void strings() {
  for (int s = -1000; s <= 1000; ++s) {
    const char* t = clsa_status_string(s);
    EXPECT(t != nullptr && std::strlen(t) > 0);
  }
  EXPECT(clsa_version() > 0);
}

}  // namespace

int main() {
  route_sizes();
  attn_sizes();
  route_rejects();
  attn_rejects();
  append_rejects();
  router_paths();
  strings();
  if (g_fail) {
    std::fprintf(stderr, "%d expectations failed\n", g_fail);
    return 1;
  }
  std::printf("host ABI paths clean\n");
  return 0;
}
