// Internal launch interface between the C ABI (fa_api.cpp) and the kernels.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace fa {

constexpr int kDtypeF32 = 0;
constexpr int kDtypeF16 = 1;
constexpr int kDtypeBF16 = 2;

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv;  // query heads, key/value heads (Hq a multiple of Hkv)
  int Nq, Nk, d;   // query rows, key rows (causal: Nq <= Nk), head dimension
  float scale;
  bool causal;
  int dtype;
  hipStream_t stream;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dO;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  float* delta;  // workspace: D_i = sum_j P_ij dP_ij (B*Hq*Nq floats), then lse_i*log2(e) (B*Hq*Nq)
  int B, Hq, Hkv;
  int Nq, Nk, d;
  float scale;
  bool causal;
  int dtype;
  hipStream_t stream;
};

constexpr int kStageDq = 1;    // dQ kernel (also writes D and lse*log2(e))
constexpr int kStageDkdv = 2;  // dK/dV kernel (reads D and lse*log2(e))

hipError_t launch_forward(const FwdArgs& a);
hipError_t launch_backward(const BwdArgs& a, int stages);

}  // namespace fa
