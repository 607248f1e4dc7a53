// Host-side sanitizer driver: runs the C ABI of libprnn through every path
// the host library plans and checks (dense layers in each math mode, sparse
// layers at each wave count, the floor, projection, layers, stacks, both
// dispatch kinds, tracing, argument errors) with the host code built under AddressSanitizer and
// UndefinedBehaviorSanitizer (device code is built normally).  Every launch
// stays inside the buffers allocated here.  Prints "driver ok" on success.
#include <hip/hip_runtime.h>
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <vector>
#include "prnn.h"
#define CHECK(x, want)                                                                      \
  do {                                                                                     \
    prnnStatus_t s_ = (x);                                                                 \
    if (s_ != (want)) {                                                                    \
      printf("FAIL line %d: %s -> %d (want %d)\n", __LINE__, #x, (int)s_, (int)(want));    \
      return 1;                                                                            \
    }                                                                                      \
  } while (0)
template <typename T> T* dalloc(size_t n) { void* p = nullptr; if (hipMalloc(&p, n * sizeof(T)) != hipSuccess) { printf("hipMalloc failed\n"); exit(2); } return (T*)p; }
int main() {
  const prnnStatus_t OK = PRNN_STATUS_SUCCESS, BP = PRNN_STATUS_BAD_PARAM, NS = PRNN_STATUS_NOT_SUPPORTED;
  prnnHandle_t h = nullptr;
  CHECK(prnn_create(nullptr), BP);
  CHECK(prnn_create(&h), OK);
  const int N = 5760, B = 4, T = 12, K = 288, I = 1792;
  float* X = dalloc<float>((size_t)T * B * N);
  float* H = dalloc<float>((size_t)T * B * N);
  float* Xb = dalloc<float>((size_t)T * B * N);
  float* h0 = dalloc<float>((size_t)B * N);
  float* x = dalloc<float>((size_t)T * B * I);
  uint16_t* W = dalloc<uint16_t>((size_t)2048 * 2048);
  uint16_t* U = dalloc<uint16_t>((size_t)N * I);
  int16_t* col = dalloc<int16_t>((size_t)N * K);
  uint16_t* val = dalloc<uint16_t>((size_t)N * K);
  std::vector<float> hx((size_t)T * B * N, 0.25f), hh0((size_t)B * N, 0.f), hxi((size_t)T * B * I, 0.5f);
  std::vector<uint16_t> hw((size_t)2048 * 2048, 0x1419), hu((size_t)N * I, 0x0c00), hv((size_t)N * K, 0x211f);
  std::vector<int16_t> hc((size_t)N * K);
  for (int i = 0; i < N; ++i) {
    for (int k = 0; k < K; ++k) hc[(size_t)i * K + k] = (int16_t)((k * 20 + i) % N);
    std::sort(hc.begin() + (size_t)i * K, hc.begin() + (size_t)(i + 1) * K);
  }
  (void)hipMemcpy(X, hx.data(), hx.size() * 4, hipMemcpyHostToDevice);
  (void)hipMemcpy(h0, hh0.data(), hh0.size() * 4, hipMemcpyHostToDevice);
  (void)hipMemcpy(x, hxi.data(), hxi.size() * 4, hipMemcpyHostToDevice);
  (void)hipMemcpy(W, hw.data(), hw.size() * 2, hipMemcpyHostToDevice);
  (void)hipMemcpy(U, hu.data(), hu.size() * 2, hipMemcpyHostToDevice);
  (void)hipMemcpy(val, hv.data(), hv.size() * 2, hipMemcpyHostToDevice);
  (void)hipMemcpy(col, hc.data(), hc.size() * 2, hipMemcpyHostToDevice);
  // dense layers in every math mode, sparse layers at every wave count
  for (int math : {PRNN_MATH_AUTO, PRNN_MATH_EXACT, PRNN_MATH_SPLIT, PRNN_MATH_HALF}) {
    CHECK(prnn_set_math(h, (prnnMath_t)math), OK);
    for (int n : {7, 257, 1152, 1792, 2048})
      CHECK(prnn_forward_dense(h, n, B, T, PRNN_DATA_HALF, W, X, h0, H, nullptr), OK);
  }
  CHECK(prnn_set_math(h, PRNN_MATH_AUTO), OK);
  for (int waves : {0, 8, 12, 16}) {
    CHECK(prnn_set_team_waves(h, waves), OK);
    CHECK(prnn_forward_sparse(h, N, B, T, 58, col, PRNN_DATA_HALF, val, X, h0, H, nullptr), OK);
    CHECK(prnn_sync_floor(h, N, B, T, H, nullptr), OK);
  }
  CHECK(prnn_set_team_waves(h, 0), OK);
  // both dispatch kinds (the occupancy cache of plain launches fills on the way)
  for (int kind : {PRNN_LAUNCH_COOPERATIVE, PRNN_LAUNCH_PLAIN}) {
    CHECK(prnn_set_launch(h, (prnnLaunch_t)kind), OK);
    CHECK(prnn_forward_dense(h, 1792, B, T, PRNN_DATA_HALF, W, X, h0, H, nullptr), OK);
    CHECK(prnn_forward_sparse(h, N, B, T, 58, col, PRNN_DATA_HALF, val, X, h0, H, nullptr), OK);
  }
  CHECK(prnn_set_launch(h, (prnnLaunch_t)5), BP);
  CHECK(prnn_set_launch(nullptr, PRNN_LAUNCH_PLAIN), BP);
  CHECK(prnn_forward_sparse(h, 2304, B, T, 230, col, PRNN_DATA_HALF, val, X, h0, H, nullptr), OK);
  CHECK(prnn_forward_sparse(h, 1792, B, T, 179, col, PRNN_DATA_HALF, val, X, nullptr, H, nullptr), OK);
  // projection and layers
  CHECK(prnn_project(h, T * B, 1792, I, PRNN_DATA_FLOAT, x, PRNN_DATA_HALF, U, h0, Xb, nullptr), OK);
  CHECK(prnn_forward_layer_dense(h, 1792, I, B, T, PRNN_DATA_FLOAT, x, PRNN_DATA_HALF, U, nullptr, PRNN_DATA_HALF, W,
                                 h0, Xb, H, nullptr), OK);
  // tracing
  CHECK(prnn_set_trace(h, 1), OK);
  CHECK(prnn_forward_dense(h, 1792, B, T, PRNN_DATA_HALF, W, X, h0, H, nullptr), OK);
  int records = 0;
  CHECK(prnn_get_trace(h, nullptr, 0, &records, nullptr), BP);
  std::vector<uint64_t> tr((size_t)records * 8);
  CHECK(prnn_get_trace(h, tr.data(), tr.size(), &records, nullptr), OK);
  CHECK(prnn_sync_floor(h, N, B, T, H, nullptr), OK);
  CHECK(prnn_get_trace(h, nullptr, 0, &records, nullptr), BP);
  tr.assign((size_t)records * 8, 0);
  CHECK(prnn_get_trace(h, tr.data(), tr.size(), &records, nullptr), OK);
  CHECK(prnn_set_trace(h, 0), OK);
  prnnPlanInfo_t info;
  CHECK(prnn_get_last_plan(h, &info), OK);
  // argument errors and unsupported shapes
  CHECK(prnn_forward_dense(h, 0, B, T, PRNN_DATA_HALF, W, X, h0, H, nullptr), BP);
  CHECK(prnn_forward_dense(h, 64, 9, T, PRNN_DATA_HALF, W, X, h0, H, nullptr), BP);
  CHECK(prnn_forward_dense(h, 64, B, T, PRNN_DATA_HALF, nullptr, X, h0, H, nullptr), BP);
  CHECK(prnn_forward_dense(h, 64, B, T, PRNN_DATA_HALF, W, X, h0, X, nullptr), BP);
  CHECK(prnn_forward_sparse(h, 64, B, T, 0, col, PRNN_DATA_HALF, val, X, h0, H, nullptr), BP);
  CHECK(prnn_forward_dense(h, 64, B, 0, PRNN_DATA_HALF, W, X, h0, H, nullptr), OK);
  CHECK(prnn_set_team_waves(h, 10), BP);
  CHECK(prnn_set_math(h, (prnnMath_t)7), BP);
  CHECK(prnn_set_math(h, PRNN_MATH_HALF), OK);
  uint16_t* W4 = dalloc<uint16_t>((size_t)4096 * 4096);
  (void)hipMemset(W4, 0, (size_t)4096 * 4096 * 2);
  CHECK(prnn_forward_dense(h, 4096, 1, 2, PRNN_DATA_HALF, W4, X, h0, H, nullptr), NS);
  CHECK(prnn_set_math(h, PRNN_MATH_AUTO), OK);
  // dense fp16 split over 2 and 4 XCDs per batch row, forced and automatic, and its floor
  CHECK(prnn_forward_dense(h, 4096, 2, 2, PRNN_DATA_HALF, W4, X, h0, H, nullptr), OK);
  CHECK(prnn_forward_dense(h, 3072, 4, 3, PRNN_DATA_HALF, W4, X, h0, H, nullptr), OK);
  CHECK(prnn_sync_floor(h, 3072, 4, 3, H, nullptr), OK);
  CHECK(prnn_set_xcds_per_row(h, 3), BP);
  CHECK(prnn_set_xcds_per_row(h, 2), OK);
  CHECK(prnn_forward_dense(h, 1792, 4, 3, PRNN_DATA_HALF, W4, X, h0, H, nullptr), OK);
  CHECK(prnn_set_xcds_per_row(h, 1), OK);
  CHECK(prnn_forward_dense(h, 3072, 4, 3, PRNN_DATA_HALF, W4, X, h0, H, nullptr), NS);
  CHECK(prnn_set_xcds_per_row(h, 0), OK);
  CHECK(prnn_get_last_plan(h, &info), OK);
  // sparse rows of unequal length
  int32_t* rl = dalloc<int32_t>(2304);
  std::vector<int32_t> hrl(2304);
  for (int i = 0; i < 2304; ++i) hrl[i] = (i * 37) % 700 - 20;  // also below 0 and above K
  (void)hipMemcpy(rl, hrl.data(), hrl.size() * 4, hipMemcpyHostToDevice);
  CHECK(prnn_forward_sparse_rows(h, 2304, B, T, 617, col, PRNN_DATA_HALF, val, rl, X, h0, H, nullptr), OK);
  CHECK(prnn_forward_sparse_rows(h, 2304, B, T, 617, col, PRNN_DATA_HALF, val, nullptr, X, h0, H, nullptr), BP);
  CHECK(prnn_forward_sparse_rows(h, 2304, B, T, 617, col, PRNN_DATA_FLOAT, val, rl, X, h0, H, nullptr), NS);
  // a stack of two sparse layers, one after another
  float* H2 = dalloc<float>((size_t)T * B * N);
  const void* Us[2] = {U, U};
  const int16_t* cols[2] = {col, col};
  const void* vals[2] = {val, val};
  float* Hs[2] = {H, H2};
  CHECK(prnn_forward_stack_sparse(h, 2, 1152, 1152, B, T, 115, PRNN_DATA_FLOAT, x, Us, nullptr, cols, PRNN_DATA_HALF,
                                  vals, nullptr, Xb, Hs, nullptr), OK);
  float* Hsame[2] = {H, H};
  CHECK(prnn_forward_stack_sparse(h, 2, 1152, 1152, B, T, 115, PRNN_DATA_FLOAT, x, Us, nullptr, cols, PRNN_DATA_HALF,
                                  vals, nullptr, Xb, Hsame, nullptr), BP);
  // a stack of two dense layers in each mode (blocked: the input products inside the launches)
  const void* Ws[2] = {W, W};
  for (int mode : {PRNN_STACK_BLOCKED, PRNN_STACK_FUSED, PRNN_STACK_LAYERS}) {
    CHECK(prnn_set_stack_mode(h, (prnnStackMode_t)mode), OK);
    CHECK(prnn_forward_stack_dense(h, 2, 1152, 1152, B, T, PRNN_DATA_FLOAT, x, Us, nullptr, Ws, nullptr, Xb, Hs,
                                   nullptr), OK);
  }
  CHECK(prnn_set_stack_mode(h, PRNN_STACK_AUTO), OK);
  CHECK(prnn_synchronize(h, nullptr), OK);
  CHECK(prnn_destroy(h), OK);
  CHECK(prnn_destroy(nullptr), OK);
  printf("driver ok: %d trace records, last plan grid %d waves %d\n", records, info.grid, info.waves_per_wg);
  return 0;
}
