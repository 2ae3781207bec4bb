// Kernel launchers behind the C ABI. Arguments arrive validated (abi.cpp); these only pick
// the compiled instance and enqueue on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smqa {

struct FwdArgs {
  const void* q;
  const void* kv;
  const float* sink;
  const int32_t* idx;
  void* o;
  float* lse;
  int64_t B, S, S_kv, H, D, topk;
  float sm_scale;
};

struct BwdMainArgs {
  const void* q;
  const void* kv;
  const void* d_o;
  const int32_t* idx;
  const float* lse;
  const float* delta;
  void* dq;
  float* dkv_accum;
  int64_t B, S, S_kv, H, D, topk;
  float sm_scale;
};

hipError_t launch_fwd(const FwdArgs& a, hipStream_t st);
hipError_t launch_bwd_preprocess(const void* o, const void* d_o, float* delta, int64_t rows, int64_t D,
                                 hipStream_t st);
hipError_t launch_fill_zero_f32(float* p, int64_t n, hipStream_t st);
// which: 1 = dQ kernel, 2 = dKV scatter kernel, 3 = both.
hipError_t launch_bwd_main(const BwdMainArgs& a, int which, hipStream_t st);
hipError_t launch_bwd_postprocess(const float* acc, void* dkv, int64_t n, hipStream_t st);

}  // namespace smqa
