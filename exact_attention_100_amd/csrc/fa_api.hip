// The C ABI of include/fa.h: argument checks, workspace carving and dispatch.
// No device memory is allocated here; every buffer comes from the caller.
#include <math.h>
#include <string.h>

#include <atomic>

#include "fa.h"
#include "fa_internal.hpp"

namespace fa {

// ------------------------------------------------------------------------------ timer
//
// The optional kernel timer keeps its state per calling thread: a launch consults only
// its own thread's record (one thread_local flag while the timer is off), so calls from
// different threads share nothing and no lock is taken on any path.

namespace {
constexpr int kTimerSlots = 8192;
struct Timer {
  bool created = false;
  hipEvent_t start[kTimerSlots];
  hipEvent_t stop[kTimerSlots];
  const char* name[kTimerSlots];
  int n = 0;
  int open = -1;  // slot whose start event was recorded and whose stop is pending
};
thread_local bool t_enabled = false;  // this thread's timer is on (nothing is allocated until it is)
thread_local Timer* t_timer = nullptr;
Timer& timer() {
  // Never destroyed: its events may outlive thread and static teardown.
  if (!t_timer) t_timer = new Timer();
  return *t_timer;
}
}  // namespace

void timer_begin(const char* name, hipStream_t stream) {
  if (!t_enabled) return;
  Timer& t = timer();
  t.open = -1;
  if (t.n >= kTimerSlots) return;
  const int i = t.n++;
  t.name[i] = name;
  (void)hipEventRecord(t.start[i], stream);
  t.open = i;
}

void timer_end(hipStream_t stream) {
  if (!t_enabled) return;
  Timer& t = timer();
  if (t.open >= 0) (void)hipEventRecord(t.stop[t.open], stream);
  t.open = -1;
}

}  // namespace fa

using namespace fa;

extern "C" int fa_timer_enable(int enable) {
  if (!enable) {
    t_enabled = false;
    return FA_OK;
  }
  Timer& t = timer();
  if (!t.created) {
    for (int i = 0; i < kTimerSlots; ++i) {
      if (hipEventCreate(&t.start[i]) != hipSuccess || hipEventCreate(&t.stop[i]) != hipSuccess)
        return FA_ERR_HIP;
    }
    t.created = true;
  }
  t_enabled = true;
  return FA_OK;
}

extern "C" void fa_timer_reset(void) {
  if (!t_timer) return;
  t_timer->n = 0;
  t_timer->open = -1;
}

extern "C" int fa_timer_read(const char* kernel, double* total_ms, int64_t* launches) {
  if (!kernel || !total_ms || !launches) return FA_ERR_INVALID;
  double sum = 0.0;
  int64_t cnt = 0;
  if (t_timer) {
    Timer& t = *t_timer;
    for (int i = 0; i < t.n; ++i) {
      if (strcmp(t.name[i], kernel) != 0) continue;
      if (hipEventSynchronize(t.stop[i]) != hipSuccess) return FA_ERR_HIP;
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, t.start[i], t.stop[i]) != hipSuccess) return FA_ERR_HIP;
      sum += ms;
      ++cnt;
    }
  }
  *total_ms = sum;
  *launches = cnt;
  return FA_OK;
}

// ------------------------------------------------------------------------------ checks

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_bytes(int dtype) { return dtype == FA_F32 ? 4 : 2; }

// Shape, dtype and stride checks common to every call.
int check_desc(const fa_desc* d) {
  if (!d) return FA_ERR_INVALID;
  if (d->B < 1 || d->H < 1 || d->N < 1 || d->reserved != 0) return FA_ERR_INVALID;
  if (d->dtype != FA_BF16 && d->dtype != FA_F32) return FA_ERR_INVALID;
  if (d->d != 64 && d->d != 128) return FA_ERR_UNSUPPORTED;
  // Rows start 16-byte aligned: every stride is a multiple of 16 bytes (tested in
  // elements, so that no product can overflow).
  const int64_t align = 16 / (int64_t)elem_bytes(d->dtype);
  if (d->stride_n < d->d || d->stride_h < 1 || d->stride_b < 1) return FA_ERR_INVALID;
  if (d->stride_n % align || d->stride_h % align || d->stride_b % align) return FA_ERR_INVALID;
  // The tile copies keep each lane's offset from a tile's first row in 32 bits, and the
  // largest tile has 256 rows (the dK/dV pass's resident V block): 256 stride_n must
  // stay below 2^31.
  if (d->stride_n >= ((int64_t)1 << 23)) return FA_ERR_UNSUPPORTED;
  // The largest element offset, (B-1) stride_b + (H-1) stride_h + (N-1) stride_n + d, must
  // be an address a device can hold (2^48 elements): the kernels form it in 64 bits.
  int64_t span = d->d, part = 0;
  if (__builtin_mul_overflow((int64_t)d->B - 1, d->stride_b, &part) || __builtin_add_overflow(span, part, &span) ||
      __builtin_mul_overflow((int64_t)d->H - 1, d->stride_h, &part) || __builtin_add_overflow(span, part, &span) ||
      __builtin_mul_overflow((int64_t)d->N - 1, d->stride_n, &part) || __builtin_add_overflow(span, part, &span) ||
      span > ((int64_t)1 << 48))
    return FA_ERR_INVALID;
  // Grid and index limits of the kernels. B, H, N are positive int32, so B H < 2^62
  // and, once B H <= 2^31 - 1, both products below stay under 2^62.
  const int64_t inst = (int64_t)d->B * d->H;
  if (inst > 0x7FFFFFFFll) return FA_ERR_UNSUPPORTED;
  // The kernels index rows and tiles in 32-bit arithmetic (row + tile size, tile
  // counts rounded up): N <= 2^30 keeps every such sum below 2^31.
  if (d->N > (1 << 30)) return FA_ERR_UNSUPPORTED;
  if (inst * (((int64_t)d->N + 127) / 128) > 0x7FFFFFFFll) return FA_ERR_UNSUPPORTED;
  if (inst * d->N > (int64_t)1 << 40) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

int check_scale(float scale) { return (isfinite(scale) && scale >= 0.f) ? FA_OK : FA_ERR_INVALID; }

int check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!p || !aligned16(p)) return FA_ERR_INVALID;
  return FA_OK;
}

size_t round_up(size_t x) { return (x + 255) & ~(size_t)255; }

size_t bwd_ws_bytes(const fa_desc* d) {
  const size_t rows = (size_t)d->B * d->H * d->N;
  return 2 * round_up(rows * sizeof(float));
}

int check_block(const fa_desc* d, int32_t bs) {
  if (bs < 128 || bs % 128 != 0 || d->N % bs != 0) return FA_ERR_INVALID;
  if (d->N / bs > 1024) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

void carve_bwd(const fa_desc* d, void* ws, BwdArgs& a) {
  const size_t rows = (size_t)d->B * d->H * d->N;
  char* p = static_cast<char*>(ws);
  a.delta = reinterpret_cast<float*>(p);
  p += round_up(rows * sizeof(float));
  a.lse2 = reinterpret_cast<float*>(p);
}

int hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

FwdArgs fwd_args(const fa_desc* d, const void* Q, const void* K, const void* V, float scale, int causal,
                 const int32_t* key_len, void* O, float* LSE) {
  FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = Q;
  a.k = K;
  a.v = V;
  a.o = O;
  a.lse = LSE;
  a.sb = d->stride_b;
  a.sh = d->stride_h;
  a.sn = d->stride_n;
  a.B = d->B;
  a.H = d->H;
  a.N = d->N;
  a.d = d->d;
  a.scale = scale;
  a.causal = causal != 0;
  a.key_len = key_len;
  return a;
}

BwdArgs bwd_args(const fa_desc* d, const void* Q, const void* K, const void* V, const void* O,
                 const void* dO, const float* LSE, float scale, int causal, const int32_t* key_len,
                 void* dQ, void* dK, void* dV) {
  BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = Q;
  a.k = K;
  a.v = V;
  a.o = O;
  a.dout = dO;
  a.lse = LSE;
  a.dq = dQ;
  a.dk = dK;
  a.dv = dV;
  a.sb = d->stride_b;
  a.sh = d->stride_h;
  a.sn = d->stride_n;
  a.B = d->B;
  a.H = d->H;
  a.N = d->N;
  a.d = d->d;
  a.scale = scale;
  a.causal = causal != 0;
  a.key_len = key_len;
  return a;
}

}  // namespace

// ------------------------------------------------------------------------------ entry points

extern "C" int fa_version(void) { return FA_VERSION; }

extern "C" const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID: return "FA_ERR_INVALID: invalid argument (pointer, shape, stride, alignment or scale)";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dim, dtype or size not supported by this call";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime reported an error";
    case FA_ERR_SCRATCH:
      return "FA_ERR_SCRATCH: the problem needs more workspace than the static scratch of fa_bwd_noalloc holds";
    default: return "unknown status";
  }
}

extern "C" int fa_fwd(const fa_desc* desc, const void* Q, const void* K, const void* V, float scale,
                      int causal, const int32_t* key_len, void* O, float* LSE, void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  if ((st = check_scale(scale))) return st;
  if ((st = check_ptrs({Q, K, V, O, LSE}))) return st;
  const FwdArgs a = fwd_args(desc, Q, K, V, scale, causal, key_len, O, LSE);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(desc->dtype == FA_BF16 ? launch_fwd_bf16(a, s) : launch_fwd_f32(a, s));
}

extern "C" size_t fa_bwd_workspace_bytes(const fa_desc* desc) {
  if (check_desc(desc)) return 0;
  return bwd_ws_bytes(desc);
}

extern "C" int fa_bwd(const fa_desc* desc, const void* Q, const void* K, const void* V, const void* O,
                      const void* dO, const float* LSE, float scale, int causal, const int32_t* key_len,
                      void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  if (desc->dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if ((st = check_scale(scale))) return st;
  if ((st = check_ptrs({Q, K, V, O, dO, LSE, dQ, dK, dV}))) return st;
  if (!workspace || !aligned16(workspace) || workspace_bytes < bwd_ws_bytes(desc)) return FA_ERR_WORKSPACE;
  BwdArgs a = bwd_args(desc, Q, K, V, O, dO, LSE, scale, causal, key_len, dQ, dK, dV);
  carve_bwd(desc, workspace, a);
  return hip_status(launch_bwd_bf16(a, static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------------------ no-alloc backward
//
// fa_bwd_noalloc: fa_bwd with its workspace (D and lse2, 8 bytes per row) in a static
// device array instead of a caller buffer, for callers that cannot allocate. The array's
// name is a host-side stand-in; its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is passed on.

namespace {
constexpr size_t kScratchBytes = size_t{16} << 20;  // 16 MiB per device
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device (null: not looked up)

// The current device's address of `scratch`, or null with *err set.
void* scratch_for_current_device(int* err) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = FA_ERR_HIP;
    return nullptr;
  }
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  // Looked up on the first call on this device (the lookup is idempotent, so two threads
  // racing here store the same address).
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
    *err = FA_ERR_HIP;
    return nullptr;
  }
  g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  return ptr;
}
}  // namespace

extern "C" int fa_bwd_noalloc(const fa_desc* desc, const void* Q, const void* K, const void* V, const void* O,
                              const void* dO, const float* LSE, float scale, int causal, const int32_t* key_len,
                              void* dQ, void* dK, void* dV, void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  if (desc->dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if ((st = check_scale(scale))) return st;
  if ((st = check_ptrs({Q, K, V, O, dO, LSE, dQ, dK, dV}))) return st;
  if (bwd_ws_bytes(desc) > kScratchBytes) return FA_ERR_SCRATCH;
  void* ws = scratch_for_current_device(&st);
  if (!ws) return st;
  BwdArgs a = bwd_args(desc, Q, K, V, O, dO, LSE, scale, causal, key_len, dQ, dK, dV);
  // Every workspace entry is written by the first backward kernel before the second reads it,
  // so nothing has to be cleared between calls.
  carve_bwd(desc, ws, a);
  return hip_status(launch_bwd_bf16(a, static_cast<hipStream_t>(stream)));
}

// Dropout parameters: p in [0, 1), quantised to p8 = round(256 p) <= 255.
int make_dropout(float p, uint64_t seed, uint32_t offset, Dropout& d) {
  if (!(p >= 0.f) || !(p < 1.f)) return FA_ERR_INVALID;  // (also rejects NaN)
  const int p8 = (int)lrintf(p * 256.f);
  if (p8 > 255) return FA_ERR_INVALID;
  d.p8 = (uint32_t)p8;
  d.k0 = (uint32_t)(seed & 0xFFFFFFFFu);
  d.k1 = (uint32_t)(seed >> 32);
  d.offset = offset;
  d.scale = 256.f / (float)(256 - p8);
  return FA_OK;
}

extern "C" int fa_fwd_dropout(const fa_desc* desc, const void* Q, const void* K, const void* V, float scale,
                              int causal, const int32_t* key_len, float dropout_p, uint64_t seed,
                              uint32_t offset, void* O, float* LSE, void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  if ((st = check_scale(scale))) return st;
  if ((st = check_ptrs({Q, K, V, O, LSE}))) return st;
  FwdArgs a = fwd_args(desc, Q, K, V, scale, causal, key_len, O, LSE);
  if ((st = make_dropout(dropout_p, seed, offset, a.dropout))) return st;
  if (a.dropout.p8 && desc->dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(desc->dtype == FA_BF16 ? launch_fwd_bf16(a, s) : launch_fwd_f32(a, s));
}

extern "C" int fa_bwd_dropout(const fa_desc* desc, const void* Q, const void* K, const void* V, const void* O,
                              const void* dO, const float* LSE, float scale, int causal, const int32_t* key_len,
                              float dropout_p, uint64_t seed, uint32_t offset, void* dQ, void* dK, void* dV,
                              void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  if (desc->dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if ((st = check_scale(scale))) return st;
  if ((st = check_ptrs({Q, K, V, O, dO, LSE, dQ, dK, dV}))) return st;
  if (!workspace || !aligned16(workspace) || workspace_bytes < bwd_ws_bytes(desc)) return FA_ERR_WORKSPACE;
  BwdArgs a = bwd_args(desc, Q, K, V, O, dO, LSE, scale, causal, key_len, dQ, dK, dV);
  if ((st = make_dropout(dropout_p, seed, offset, a.dropout))) return st;
  carve_bwd(desc, workspace, a);
  return hip_status(launch_bwd_bf16(a, static_cast<hipStream_t>(stream)));
}

extern "C" size_t fa_blocksparse_workspace_bytes(const fa_desc* desc, int32_t block_size, int backward) {
  if (check_desc(desc) || check_block(desc, block_size)) return 0;
  return backward ? bwd_ws_bytes(desc) : 0;
}

extern "C" int fa_blocksparse_fwd(const fa_desc* desc, const void* Q, const void* K, const void* V,
                                  float scale, int causal, const int32_t* key_len,
                                  const uint8_t* block_mask, int32_t block_size, void* O, float* LSE,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;  // the forward needs none (each workgroup reads its row of the block mask)
  (void)workspace_bytes;
  int st = check_desc(desc);
  if (st) return st;
  if (desc->dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if ((st = check_scale(scale))) return st;
  if ((st = check_ptrs({Q, K, V, O, LSE}))) return st;
  if (!block_mask) return FA_ERR_INVALID;
  if ((st = check_block(desc, block_size))) return st;
  FwdArgs a = fwd_args(desc, Q, K, V, scale, causal != 0, key_len, O, LSE);
  a.block_mask = block_mask;
  a.nb = desc->N / block_size;
  a.block_size = block_size;
  return hip_status(launch_fwd_bf16(a, static_cast<hipStream_t>(stream)));
}

extern "C" int fa_blocksparse_bwd(const fa_desc* desc, const void* Q, const void* K, const void* V,
                                  const void* O, const void* dO, const float* LSE, float scale, int causal,
                                  const int32_t* key_len, const uint8_t* block_mask, int32_t block_size,
                                  void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  if (desc->dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if ((st = check_scale(scale))) return st;
  if ((st = check_ptrs({Q, K, V, O, dO, LSE, dQ, dK, dV}))) return st;
  if (!block_mask) return FA_ERR_INVALID;
  if ((st = check_block(desc, block_size))) return st;
  if (!workspace || !aligned16(workspace) || workspace_bytes < bwd_ws_bytes(desc)) return FA_ERR_WORKSPACE;
  BwdArgs a = bwd_args(desc, Q, K, V, O, dO, LSE, scale, causal != 0, key_len, dQ, dK, dV);
  carve_bwd(desc, workspace, a);
  a.block_mask = block_mask;
  a.nb = desc->N / block_size;
  a.block_size = block_size;
  return hip_status(launch_bwd_bf16(a, static_cast<hipStream_t>(stream)));
}

extern "C" int fa_blocksparse_fwd_dropout(const fa_desc* desc, const void* Q, const void* K, const void* V,
                                          float scale, int causal, const int32_t* key_len,
                                          const uint8_t* block_mask, int32_t block_size, float dropout_p,
                                          uint64_t seed, uint32_t offset, void* O, float* LSE, void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  if (desc->dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if ((st = check_scale(scale))) return st;
  if ((st = check_ptrs({Q, K, V, O, LSE}))) return st;
  if (!block_mask) return FA_ERR_INVALID;
  if ((st = check_block(desc, block_size))) return st;
  FwdArgs a = fwd_args(desc, Q, K, V, scale, causal != 0, key_len, O, LSE);
  if ((st = make_dropout(dropout_p, seed, offset, a.dropout))) return st;
  a.block_mask = block_mask;
  a.nb = desc->N / block_size;
  a.block_size = block_size;
  return hip_status(launch_fwd_bf16(a, static_cast<hipStream_t>(stream)));
}

extern "C" int fa_blocksparse_bwd_dropout(const fa_desc* desc, const void* Q, const void* K, const void* V,
                                          const void* O, const void* dO, const float* LSE, float scale, int causal,
                                          const int32_t* key_len, const uint8_t* block_mask, int32_t block_size,
                                          float dropout_p, uint64_t seed, uint32_t offset, void* dQ, void* dK,
                                          void* dV, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  if (desc->dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if ((st = check_scale(scale))) return st;
  if ((st = check_ptrs({Q, K, V, O, dO, LSE, dQ, dK, dV}))) return st;
  if (!block_mask) return FA_ERR_INVALID;
  if ((st = check_block(desc, block_size))) return st;
  if (!workspace || !aligned16(workspace) || workspace_bytes < bwd_ws_bytes(desc)) return FA_ERR_WORKSPACE;
  BwdArgs a = bwd_args(desc, Q, K, V, O, dO, LSE, scale, causal != 0, key_len, dQ, dK, dV);
  if ((st = make_dropout(dropout_p, seed, offset, a.dropout))) return st;
  carve_bwd(desc, workspace, a);
  a.block_mask = block_mask;
  a.nb = desc->N / block_size;
  a.block_size = block_size;
  return hip_status(launch_bwd_bf16(a, static_cast<hipStream_t>(stream)));
}

