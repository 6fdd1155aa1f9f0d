// Drives every entry point of the C ABI through its validation branches, its
// size arithmetic and its workspace carving, on fake device addresses, for a
// host build under AddressSanitizer and UBSan (the kernel launchers are the
// counting stand-ins of abi_stubs.cpp). Prints "<n> checks, <f> failures".
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <vector>

#include "ssd.h"

extern int g_launches;

static int g_checks = 0, g_fail = 0;

#define EXPECT_EQ(got, want)                                                                  \
  do {                                                                                        \
    ++g_checks;                                                                               \
    const long long g_ = (long long)(got), w_ = (long long)(want);                            \
    if (g_ != w_) {                                                                           \
      ++g_fail;                                                                               \
      std::printf("FAIL %s:%d: %s = %lld, expected %lld\n", __FILE__, __LINE__, #got, g_, w_); \
    }                                                                                         \
  } while (0)
#define EXPECT_TRUE(c) EXPECT_EQ((c) ? 1 : 0, 1)

static void* const A16 = reinterpret_cast<void*>(uintptr_t{1} << 20);         // 16-byte aligned
static void* const MIS = reinterpret_cast<void*>((uintptr_t{1} << 20) + 8);  // not 16-byte aligned
static float* const F16A = static_cast<float*>(A16);

static ssd_shape shape(int64_t b = 1, int64_t L = 256, int64_t H = 4, int64_t P = 16, int64_t N = 16,
                       int64_t G = 1, int64_t l = 64, int32_t dtype = SSD_DTYPE_F16, int32_t sched = 0) {
  ssd_shape s;
  s.batch = b;
  s.seqlen = L;
  s.nheads = H;
  s.headdim = P;
  s.dstate = N;
  s.ngroups = G;
  s.chunk = l;
  s.dtype = dtype;
  s.schedule = sched;
  return s;
}

static ssd_scales fake_scales() {
  ssd_scales sc;
  sc.s_B = sc.s_C = sc.inv_B = sc.inv_C = sc.inv_X = sc.s_S = sc.M_req = sc.s_X = sc.s_Xq = sc.inv_Xq = F16A;
  return sc;
}

static int fwd(const ssd_shape& s, int path, const ssd_scales* sc, void* X = A16, void* ws = A16,
               size_t wsb = SIZE_MAX, const void* init = nullptr, void* fin = nullptr, const ssd_taps* taps = nullptr) {
  if (wsb == SIZE_MAX) wsb = ssd_workspace_bytes(&s, path);
  return ssd_forward(&s, path, X, A16, F16A, A16, A16, F16A, sc, A16, init, fin, ws, wsb, taps, nullptr);
}

static void status_strings() {
  for (int rc = 0; rc <= SSD_E_TOO_LARGE; ++rc) {
    const char* m = ssd_status_string(rc);
    EXPECT_TRUE(m && std::strlen(m) > 0 && std::strcmp(m, "unknown status") != 0);
  }
  EXPECT_EQ(std::strcmp(ssd_status_string(99), "unknown status"), 0);
  EXPECT_EQ(std::strcmp(ssd_status_string(-1), "unknown status"), 0);
}

static void shapes() {
  const int64_t big = std::numeric_limits<int64_t>::max();
  struct Case {
    ssd_shape s;
    int rc;
  } cases[] = {
      {shape(), SSD_OK},
      {shape(1, 256, 4, 16, 16, 1, 32), SSD_E_UNSUPPORTED},
      {shape(1, 256, 4, 16, 16, 1, 100), SSD_E_UNSUPPORTED},
      {shape(1, 256, 4, 8), SSD_E_UNSUPPORTED},
      {shape(1, 256, 4, 16, 256), SSD_E_UNSUPPORTED},
      {shape(1, 256, 4, 16, 16, 3), SSD_E_SHAPE},
      {shape(1, 256, 0), SSD_E_SHAPE},
      {shape(-1), SSD_E_SHAPE},
      {shape(1, -5), SSD_E_SHAPE},
      {shape(70000), SSD_E_SHAPE},
      {shape(1 << 15, int64_t{1} << 40, 1 << 12), SSD_E_SHAPE},
      {shape(big, big, big, 16, 16, 1, 64), SSD_E_SHAPE},
      {shape(1, big, 4), SSD_E_SHAPE},
      {shape(1, 256, big, 16, 16, big), SSD_E_SHAPE},
      {shape(1, int64_t{65536} * 256, 4, 16, 16, 1, 256), SSD_E_SHAPE},  // 65536 chunks
      {shape(1, 256, 4, 16, 16, 1, 64, 3), SSD_E_UNSUPPORTED},
      {shape(1, 256, 4, 16, 16, 1, 64, -1), SSD_E_UNSUPPORTED},
      {shape(1, 256, 4, 16, 16, 1, 64, SSD_DTYPE_F16, -1), SSD_E_SHAPE},
      {shape(1, 256, 4, 16, 16, 1, 64, SSD_DTYPE_F16, 3), SSD_E_SHAPE},
      {shape(1, 256, 4, 16, 16, 1, 64, SSD_DTYPE_F16, std::numeric_limits<int32_t>::min()), SSD_E_SHAPE},
  };
  for (const Case& c : cases) {
    g_launches = 0;
    EXPECT_EQ(fwd(c.s, SSD_PATH_FLOAT, nullptr), c.rc);
    if (c.rc != SSD_OK) {
      EXPECT_EQ(g_launches, 0);
      EXPECT_EQ(ssd_workspace_bytes(&c.s, SSD_PATH_FLOAT), 0);
      EXPECT_EQ(ssd_workspace_bytes(&c.s, SSD_PATH_INT8), 0);
    }
  }
  EXPECT_EQ(ssd_workspace_bytes(nullptr, SSD_PATH_FLOAT), 0);
  ssd_shape s = shape();
  EXPECT_EQ(ssd_workspace_bytes(&s, 7), 0);
}

static void forward_paths() {
  const ssd_scales sc = fake_scales();
  ssd_taps taps;
  taps.q_xs = static_cast<int8_t*>(A16);
  taps.s32 = static_cast<int32_t*>(A16);
  taps.s8_local = static_cast<int8_t*>(A16);
  taps.passed = static_cast<int8_t*>(A16);
  const int32_t dtypes[] = {SSD_DTYPE_F32, SSD_DTYPE_F16, SSD_DTYPE_BF16};
  const int64_t chunks[] = {64, 128, 256};
  const int64_t Ps[] = {16, 32, 64};
  const int64_t Ns[] = {16, 32, 64, 128};
  for (int32_t dt : dtypes)
    for (int64_t l : chunks)
      for (int64_t P : Ps)
        for (int64_t N : Ns)
          for (int32_t sched = 0; sched <= 2; ++sched) {
            const ssd_shape s = shape(3, 1000, 8, P, N, 2, l, dt, sched);
            for (int path = SSD_PATH_FLOAT; path <= SSD_PATH_ABL_RECON; ++path) {
              const bool i8 = path == SSD_PATH_INT8;
              const size_t need = ssd_workspace_bytes(&s, path);
              EXPECT_TRUE(need > 0);
              g_launches = 0;
              EXPECT_EQ(fwd(s, path, path == SSD_PATH_FLOAT ? nullptr : &sc, A16, A16, need, nullptr, A16,
                            i8 ? &taps : nullptr),
                        SSD_OK);
              EXPECT_TRUE(g_launches > 0);
              if (need > 16) EXPECT_EQ(fwd(s, path, &sc, A16, A16, need - 16), SSD_E_WORKSPACE);
              EXPECT_EQ(fwd(s, path, &sc, A16, nullptr, need), SSD_E_WORKSPACE);
            }
            // initial state: float and INT8 only
            EXPECT_EQ(fwd(s, SSD_PATH_INT8, &sc, A16, A16, SIZE_MAX, A16, A16), SSD_OK);
            EXPECT_EQ(fwd(s, SSD_PATH_ABL_QX, &sc, A16, A16, SIZE_MAX, A16), SSD_E_UNSUPPORTED);
          }
  const ssd_shape s = shape();
  EXPECT_EQ(fwd(s, SSD_PATH_INT8, nullptr), SSD_E_NULL);
  EXPECT_EQ(fwd(s, SSD_PATH_FLOAT, nullptr, nullptr), SSD_E_NULL);
  EXPECT_EQ(fwd(s, SSD_PATH_FLOAT, nullptr, MIS), SSD_E_ALIGN);
  EXPECT_EQ(fwd(s, SSD_PATH_FLOAT, nullptr, A16, MIS), SSD_E_ALIGN);
  EXPECT_EQ(fwd(s, 4, nullptr), SSD_E_UNSUPPORTED);
  EXPECT_EQ(fwd(s, -1, nullptr), SSD_E_UNSUPPORTED);
  ssd_scales half = fake_scales();
  half.M_req = nullptr;
  EXPECT_EQ(fwd(s, SSD_PATH_INT8, &half), SSD_E_NULL);
  ssd_scales odd = fake_scales();
  odd.s_S = reinterpret_cast<const float*>(reinterpret_cast<uintptr_t>(A16) + 2);
  EXPECT_EQ(fwd(s, SSD_PATH_INT8, &odd), SSD_E_ALIGN);
}

static void empty_problems() {
  const ssd_scales sc = fake_scales();
  for (int path = SSD_PATH_FLOAT; path <= SSD_PATH_INT8; ++path) {
    g_launches = 0;
    EXPECT_EQ(fwd(shape(0), path, &sc, A16, nullptr, 0, nullptr, A16), SSD_OK);
    EXPECT_EQ(g_launches, 0);
    // no positions: the final state is the initial one (a copy), or zeros
    g_launches = 0;
    EXPECT_EQ(fwd(shape(2, 0), path, &sc, A16, nullptr, 0, A16, A16), SSD_OK);
    EXPECT_EQ(g_launches, 1);
    g_launches = 0;
    EXPECT_EQ(fwd(shape(2, 0), path, &sc, A16, nullptr, 0, nullptr, A16), SSD_OK);
    EXPECT_EQ(g_launches, 1);
    g_launches = 0;
    EXPECT_EQ(fwd(shape(2, 0), path, &sc, A16, nullptr, 0), SSD_OK);
    EXPECT_EQ(g_launches, 0);
  }
}

static void modules() {
  const ssd_scales sc = fake_scales();
  int8_t* q = static_cast<int8_t*>(A16);
  for (int32_t dt = SSD_DTYPE_F32; dt <= SSD_DTYPE_BF16; ++dt) {
    const ssd_shape s = shape(2, 700, 8, 64, 128, 2, 256, dt);
    EXPECT_EQ(ssd_quantize_bc(&s, A16, A16, &sc, q, q, nullptr), SSD_OK);
    EXPECT_EQ(ssd_quantize_bc(&s, A16, A16, nullptr, q, q, nullptr), SSD_E_NULL);
    EXPECT_EQ(ssd_chunk_cumsum(&s, A16, F16A, F16A, F16A, static_cast<uint8_t*>(A16), nullptr), SSD_OK);
    EXPECT_EQ(ssd_chunk_cumsum(&s, A16, F16A, F16A, nullptr, nullptr, nullptr), SSD_OK);
    EXPECT_EQ(ssd_chunk_cumsum(&s, MIS, F16A, F16A, F16A, nullptr, nullptr), SSD_E_ALIGN);
    for (int path = SSD_PATH_FLOAT; path <= SSD_PATH_INT8; ++path) {
      const ssd_scales* p = path == SSD_PATH_INT8 ? &sc : nullptr;
      EXPECT_EQ(ssd_chunk_state(&s, path, A16, F16A, A16, p, A16, nullptr, nullptr), SSD_OK);
      EXPECT_EQ(ssd_state_passing(&s, path, A16, F16A, static_cast<uint8_t*>(A16), A16, A16, nullptr), SSD_OK);
      EXPECT_EQ(ssd_chunk_bmm(&s, path, A16, A16, A16, nullptr), SSD_OK);
      EXPECT_EQ(ssd_chunk_scan(&s, path, A16, A16, F16A, A16, A16, A16, nullptr, F16A, p, A16, nullptr), SSD_OK);
      EXPECT_EQ(ssd_chunk_scan(&s, path, A16, A16, F16A, A16, A16, A16, MIS, F16A, p, A16, nullptr), SSD_E_ALIGN);
    }
    EXPECT_EQ(ssd_chunk_state(&s, SSD_PATH_INT8, A16, F16A, A16, nullptr, A16, nullptr, nullptr), SSD_E_NULL);
    EXPECT_EQ(ssd_chunk_bmm(&s, SSD_PATH_ABL_QX, A16, A16, A16, nullptr), SSD_E_UNSUPPORTED);
    // decode: one position per call
    const ssd_shape d1 = shape(1024, 1, 80, 64, 128, 1, 256, dt);
    for (int path = SSD_PATH_FLOAT; path <= SSD_PATH_INT8; ++path)
      EXPECT_EQ(ssd_decode_step(&d1, path, A16, A16, F16A, A16, A16, F16A, &sc, A16, A16, nullptr), SSD_OK);
    EXPECT_EQ(ssd_decode_step(&s, SSD_PATH_FLOAT, A16, A16, F16A, A16, A16, F16A, &sc, A16, A16, nullptr),
              SSD_E_SHAPE);
    EXPECT_EQ(ssd_decode_step(&d1, SSD_PATH_INT8, A16, A16, F16A, A16, A16, F16A, nullptr, A16, A16, nullptr),
              SSD_E_NULL);
    // epilogue and the mean correction
    EXPECT_EQ(ssd_epilogue(&s, A16, F16A, 0.15f, F16A, 1e-5f, A16, nullptr), SSD_OK);
    EXPECT_EQ(ssd_epilogue(&s, A16, nullptr, 0.0f, F16A, 1e-5f, A16, nullptr), SSD_OK);
    EXPECT_EQ(ssd_mean_correction(&s, A16, A16, F16A, nullptr), SSD_OK);
    const ssd_shape e = shape(0);
    EXPECT_EQ(ssd_mean_correction(&e, A16, A16, F16A, nullptr), SSD_E_SHAPE);
    // calibration
    const size_t cw = ssd_calibrate_workspace_bytes(&s);
    EXPECT_TRUE(cw > 0);
    EXPECT_EQ(ssd_calibrate_amax(&s, A16, A16, F16A, A16, A16, F16A, A16, cw, nullptr), SSD_OK);
    EXPECT_EQ(ssd_calibrate_amax(&s, A16, A16, F16A, A16, A16, F16A, A16, cw - 1, nullptr), SSD_E_WORKSPACE);
  }
}

static void scales_from_amax() {
  const int64_t G = 2, H = 4, P = 16;
  const size_t n = 2 * G + 2 * H * P;
  std::vector<float> amax(n), pack(4 * G + 4 * H * P, -7.0f);
  for (size_t i = 0; i < n; ++i) amax[i] = 0.25f * (float)(i % 13);  // zeros included
  EXPECT_EQ(ssd_scales_from_amax(G, H, P, amax.data(), pack.data()), SSD_OK);
  for (int64_t g = 0; g < G; ++g) {
    const float a = amax[g];
    const float s = a > 0 ? (float)((double)a / 127.0) : 1.0f;
    EXPECT_EQ(pack[g] == s, 1);
    EXPECT_EQ(pack[2 * G + g] == (float)(1.0 / (double)s), 1);
  }
  for (int64_t i = 0; i < H * P; ++i) {
    const float sx = pack[4 * G + i], ss = pack[4 * G + 2 * H * P + i], m = pack[4 * G + 3 * H * P + i];
    const float sb = pack[i / (P * (H / G))];
    EXPECT_TRUE(std::isfinite(m) && m > 0);
    EXPECT_EQ(m == (float)((double)sx * (double)sb / (double)ss), 1);
  }
  const float bad[] = {-1.0f, std::numeric_limits<float>::quiet_NaN(), std::numeric_limits<float>::infinity()};
  for (float v : bad) {
    for (size_t at : {size_t{0}, size_t{2 * G}, n - 1}) {
      std::vector<float> a2 = amax, p2(pack.size(), -7.0f);
      a2[at] = v;
      EXPECT_EQ(ssd_scales_from_amax(G, H, P, a2.data(), p2.data()), SSD_E_VALUE);
      bool untouched = true;
      for (float x : p2) untouched = untouched && x == -7.0f;
      EXPECT_TRUE(untouched);
    }
  }
  EXPECT_EQ(ssd_scales_from_amax(G, H, P, nullptr, pack.data()), SSD_E_NULL);
  EXPECT_EQ(ssd_scales_from_amax(3, H, P, amax.data(), pack.data()), SSD_E_SHAPE);
  EXPECT_EQ(ssd_scales_from_amax(0, H, P, amax.data(), pack.data()), SSD_E_SHAPE);
  EXPECT_EQ(ssd_scales_from_amax(G, H, -1, amax.data(), pack.data()), SSD_E_SHAPE);
  EXPECT_EQ(ssd_scales_from_amax(G, std::numeric_limits<int64_t>::max(), std::numeric_limits<int64_t>::max(),
                                 amax.data(), pack.data()),
            SSD_E_SHAPE);
}

int main() {
  status_strings();
  shapes();
  forward_paths();
  empty_problems();
  modules();
  scales_from_amax();
  std::printf("%d checks, %d failures\n", g_checks, g_fail);
  return g_fail == 0 ? 0 : 1;
}
