// Host-side interface between the C ABI (fa_api.hip) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include "fa_common.hpp"
#include <stdint.h>

namespace fa {

// Everything a forward launch needs. Pointers are device pointers.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t sb, sh, sn;  // element strides shared by q, k, v, o
  int B, H, N, d;
  float scale;
  int causal;
  const int32_t* key_len;  // device [B] or nullptr
  // Block-sparse (block_mask != nullptr): device uint8 [nb][nb], row = query block.
  const uint8_t* block_mask;
  int nb;
  int block_size;
  Dropout dropout;  // p8 == 0: none
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int64_t sb, sh, sn;
  int B, H, N, d;
  float scale;
  int causal;
  const int32_t* key_len;
  // workspace sections
  float* delta;   // [B, H, N]: rowsum(dO o O)
  float* lse2;    // [B, H, N]: LSE * log2(e) (+inf for rows with no key)
  // Block-sparse (block_mask != nullptr): device uint8 [nb][nb], row = query block.
  const uint8_t* block_mask;
  int nb;
  int block_size;
  Dropout dropout;  // p8 == 0: none
};

// Kernel timer hooks (fa_api.hip): bracket one launch with events.
void timer_begin(const char* name, hipStream_t stream);
void timer_end(hipStream_t stream);

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s);

}  // namespace fa
