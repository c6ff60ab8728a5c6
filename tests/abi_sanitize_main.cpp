// Host-side driver for the sanitizer build of the C ABI (CPU only, no GPU call).
//
// Every entry point is called with arguments its checks must reject, so each call
// returns before anything is enqueued; built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code, any out-of-bounds read, overflow or
// undefined operation in the validation layer aborts the program. Exit status 0
// means every call returned the expected status and the sanitizers stayed quiet.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "fa.h"

namespace {

int failures = 0;

void expect(const char* what, int got, int want) {
  if (got != want) {
    std::fprintf(stderr, "%s: got %d, want %d\n", what, got, want);
    ++failures;
  }
}

fa_desc desc(int B = 2, int H = 3, int N = 256, int d = 64, int dtype = FA_BF16) {
  fa_desc x;
  std::memset(&x, 0, sizeof(x));
  x.B = B;
  x.H = H;
  x.N = N;
  x.d = d;
  x.dtype = dtype;
  x.stride_n = d;
  x.stride_h = (int64_t)N * d;
  x.stride_b = (int64_t)H * N * d;
  return x;
}

}  // namespace

int main() {
  // Never dereferenced: every call below fails its checks first.
  void* const A = reinterpret_cast<void*>(uintptr_t{4096});
  float* const F = reinterpret_cast<float*>(uintptr_t{4096});
  const uint8_t* const M = reinterpret_cast<const uint8_t*>(uintptr_t{4096});
  const fa_desc d = desc();

  expect("version", fa_version(), FA_VERSION);
  for (int s = -7; s <= 1; ++s) {
    const char* t = fa_status_string(s);
    if (!t || !*t) {
      std::fprintf(stderr, "status string %d empty\n", s);
      ++failures;
    }
  }

  // Descriptors: null, empty, bad dtype / head dim / reserved field / strides, overflowing sizes.
  expect("fwd null desc", fa_fwd(nullptr, A, A, A, 0.1f, 0, nullptr, A, F, nullptr), FA_ERR_INVALID);
  const fa_desc bad[] = {desc(0), desc(2, 0), desc(2, 3, 0), desc(2, 3, 256, 64, 7), desc(-1), desc(2, 3, -5)};
  for (const fa_desc& b : bad) expect("fwd bad desc", fa_fwd(&b, A, A, A, 0.1f, 0, nullptr, A, F, nullptr), FA_ERR_INVALID);
  fa_desc res = d;
  res.reserved = 1;
  expect("fwd reserved", fa_fwd(&res, A, A, A, 0.1f, 0, nullptr, A, F, nullptr), FA_ERR_INVALID);
  fa_desc odd = d;
  odd.stride_n = 65;
  expect("fwd odd stride", fa_fwd(&odd, A, A, A, 0.1f, 0, nullptr, A, F, nullptr), FA_ERR_INVALID);
  fa_desc neg = d;
  neg.stride_b = -1;
  expect("fwd negative stride", fa_fwd(&neg, A, A, A, 0.1f, 0, nullptr, A, F, nullptr), FA_ERR_INVALID);
  // Sizes whose products overflow 64 bits, spans no device holds, and sizes past the
  // kernels' 32-bit row arithmetic.
  fa_desc huge = desc(1, 1, 256, 128);
  huge.B = huge.H = huge.N = 0x7FFFFFFF;
  huge.stride_n = 128;
  huge.stride_h = int64_t{1} << 40;
  huge.stride_b = int64_t{1} << 60;
  expect("fwd huge", fa_fwd(&huge, A, A, A, 0.1f, 0, nullptr, A, F, nullptr), FA_ERR_INVALID);
  fa_desc wide = d;
  wide.stride_b = INT64_MAX - 7;
  expect("fwd stride near int64 max", fa_fwd(&wide, A, A, A, 0.1f, 0, nullptr, A, F, nullptr), FA_ERR_INVALID);
  fa_desc longest = desc(1, 1, 256, 64);
  longest.N = 0x7FFFFFFF;  // span 2^37 elements: allowed, but N > 2^30
  longest.stride_h = longest.stride_b = int64_t{1} << 37;
  expect("fwd N = 2^31 - 1", fa_fwd(&longest, A, A, A, 0.1f, 0, nullptr, A, F, nullptr), FA_ERR_UNSUPPORTED);
  fa_desc heads = desc(1, 1, 128, 64);
  heads.B = heads.H = 1 << 16;  // B H = 2^32 instances
  heads.stride_h = 128 * 64;
  heads.stride_b = int64_t{128} * 64 << 16;
  expect("fwd 2^32 instances", fa_fwd(&heads, A, A, A, 0.1f, 0, nullptr, A, F, nullptr), FA_ERR_UNSUPPORTED);
  // Row strides at the tile copies' 32-bit limit (256-row tiles): 2^23 - 8 elements passes
  // the descriptor checks (the null Q is what is rejected), 2^23 does not.
  fa_desc rs = desc(2, 3, 256, 64);
  rs.stride_n = (int64_t{1} << 23) - 8;
  rs.stride_h = rs.stride_n * 256;
  rs.stride_b = rs.stride_h * 3;
  expect("fwd stride_n 2^23 - 8", fa_fwd(&rs, nullptr, A, A, 0.1f, 0, nullptr, A, F, nullptr), FA_ERR_INVALID);
  rs.stride_n = int64_t{1} << 23;
  rs.stride_h = rs.stride_n * 256;
  rs.stride_b = rs.stride_h * 3;
  expect("fwd stride_n 2^23", fa_fwd(&rs, A, A, A, 0.1f, 0, nullptr, A, F, nullptr), FA_ERR_UNSUPPORTED);
  expect("bwd stride_n 2^23", fa_bwd(&rs, A, A, A, A, A, F, 0.1f, 0, nullptr, A, A, A, A, size_t{1} << 40, nullptr),
         FA_ERR_UNSUPPORTED);
  const fa_desc d96 = desc(2, 3, 256, 96);
  expect("fwd d=96", fa_fwd(&d96, A, A, A, 0.1f, 0, nullptr, A, F, nullptr), FA_ERR_UNSUPPORTED);

  // Pointers and scale.
  expect("fwd null Q", fa_fwd(&d, nullptr, A, A, 0.1f, 0, nullptr, A, F, nullptr), FA_ERR_INVALID);
  expect("fwd misaligned", fa_fwd(&d, static_cast<char*>(A) + 2, A, A, 0.1f, 0, nullptr, A, F, nullptr),
         FA_ERR_INVALID);
  expect("fwd negative scale", fa_fwd(&d, A, A, A, -0.5f, 0, nullptr, A, F, nullptr), FA_ERR_INVALID);
  expect("fwd nan scale", fa_fwd(&d, A, A, A, std::nanf(""), 0, nullptr, A, F, nullptr), FA_ERR_INVALID);
  expect("fwd inf scale", fa_fwd(&d, A, A, A, INFINITY, 0, nullptr, A, F, nullptr), FA_ERR_INVALID);

  // Backward: fp32 unsupported, workspace size and pointer.
  const fa_desc f32 = desc(2, 3, 256, 64, FA_F32);
  expect("bwd fp32", fa_bwd(&f32, A, A, A, A, A, F, 0.1f, 0, nullptr, A, A, A, A, size_t{1} << 30, nullptr),
         FA_ERR_UNSUPPORTED);
  const size_t need = fa_bwd_workspace_bytes(&d);
  if (need == 0) {
    std::fprintf(stderr, "bwd workspace size 0\n");
    ++failures;
  }
  expect("bwd null desc workspace size", (int)fa_bwd_workspace_bytes(nullptr), 0);
  expect("bwd short workspace", fa_bwd(&d, A, A, A, A, A, F, 0.1f, 0, nullptr, A, A, A, A, need - 1, nullptr),
         FA_ERR_WORKSPACE);
  expect("bwd null workspace", fa_bwd(&d, A, A, A, A, A, F, 0.1f, 0, nullptr, A, A, A, nullptr, need, nullptr),
         FA_ERR_WORKSPACE);
  expect("bwd null dO", fa_bwd(&d, A, A, A, A, nullptr, F, 0.1f, 0, nullptr, A, A, A, A, need, nullptr),
         FA_ERR_INVALID);

  // No-alloc backward: the same checks as fa_bwd, then the static scratch's size limit (2^21
  // rows), all before the scratch's device address is looked up.
  expect("bwd noalloc fp32", fa_bwd_noalloc(&f32, A, A, A, A, A, F, 0.1f, 0, nullptr, A, A, A, nullptr),
         FA_ERR_UNSUPPORTED);
  expect("bwd noalloc null dQ", fa_bwd_noalloc(&d, A, A, A, A, A, F, 0.1f, 0, nullptr, nullptr, A, A, nullptr),
         FA_ERR_INVALID);
  expect("bwd noalloc nan scale", fa_bwd_noalloc(&d, A, A, A, A, A, F, std::nanf(""), 0, nullptr, A, A, A, nullptr),
         FA_ERR_INVALID);
  const fa_desc rows_over = desc(1, 1, (1 << 21) + 1, 64);
  expect("bwd noalloc 2^21 + 1 rows", fa_bwd_noalloc(&rows_over, A, A, A, A, A, F, 0.1f, 0, nullptr, A, A, A, nullptr),
         FA_ERR_SCRATCH);
  const fa_desc rows_over2 = desc(4, 8, 65537, 128);
  expect("bwd noalloc 4 x 8 x 65537 rows", fa_bwd_noalloc(&rows_over2, A, A, A, A, A, F, 0.1f, 1, nullptr, A, A, A,
                                                           nullptr), FA_ERR_SCRATCH);

  // Dropout: probability range, fp32.
  const float bad_p[] = {-0.1f, 1.0f, 1.5f, std::nanf(""), 0.999f};
  for (float p : bad_p) {
    expect("fwd dropout p", fa_fwd_dropout(&d, A, A, A, 0.1f, 0, nullptr, p, 1, 0, A, F, nullptr), FA_ERR_INVALID);
    expect("bwd dropout p", fa_bwd_dropout(&d, A, A, A, A, A, F, 0.1f, 0, nullptr, p, 1, 0, A, A, A, A,
                                           size_t{1} << 30, nullptr), FA_ERR_INVALID);
  }
  expect("fwd dropout fp32", fa_fwd_dropout(&f32, A, A, A, 0.1f, 0, nullptr, 0.1f, 1, 0, A, F, nullptr),
         FA_ERR_UNSUPPORTED);

  // Block-sparse: block size, mask pointer, block count, workspace.
  const int32_t bad_bs[] = {0, -128, 64, 100, 192, 512};
  for (int32_t bs : bad_bs) {
    expect("sparse fwd block size", fa_blocksparse_fwd(&d, A, A, A, 0.1f, 0, nullptr, M, bs, A, F, nullptr, 0, nullptr),
           FA_ERR_INVALID);
    expect("sparse workspace size", (int)fa_blocksparse_workspace_bytes(&d, bs, 1), 0);
  }
  expect("sparse fwd null mask", fa_blocksparse_fwd(&d, A, A, A, 0.1f, 0, nullptr, nullptr, 128, A, F, nullptr, 0,
                                                    nullptr), FA_ERR_INVALID);
  const fa_desc big = desc(1, 1, 128 * 1025, 64);
  expect("sparse fwd too many blocks", fa_blocksparse_fwd(&big, A, A, A, 0.1f, 0, nullptr, M, 128, A, F, nullptr, 0,
                                                          nullptr), FA_ERR_UNSUPPORTED);
  expect("sparse fwd workspace size", (int)fa_blocksparse_workspace_bytes(&d, 128, 0), 0);
  expect("sparse bwd workspace size", (int)(fa_blocksparse_workspace_bytes(&d, 128, 1) == need), 1);
  expect("sparse bwd short workspace", fa_blocksparse_bwd(&d, A, A, A, A, A, F, 0.1f, 1, nullptr, M, 128, A, A, A, A,
                                                          need - 1, nullptr), FA_ERR_WORKSPACE);
  expect("sparse bwd fp32", fa_blocksparse_bwd(&f32, A, A, A, A, A, F, 0.1f, 0, nullptr, M, 128, A, A, A, A,
                                               size_t{1} << 30, nullptr), FA_ERR_UNSUPPORTED);

  // Timer reads without a recording: no launches, no GPU call.
  double ms = -1.0;
  int64_t n = -1;
  expect("timer read", fa_timer_read("fa_fwd_bf16", &ms, &n), FA_OK);
  expect("timer launches", (int)n, 0);
  expect("timer null name", fa_timer_read(nullptr, &ms, &n), FA_ERR_INVALID);

  if (failures) {
    std::fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  std::printf("abi sanitizer driver: all checks passed\n");
  return 0;
}
