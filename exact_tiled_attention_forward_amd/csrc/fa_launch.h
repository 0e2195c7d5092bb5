// Internal launch interface between the C ABI (fa_api.cpp) and the kernels.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

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
  int nsplit = 1;          // > 1: split each query block's key range (16-bit inputs only)
  float* part = nullptr;   // workspace for the split partials (fwd_split_bytes)
  const uint8_t* bmask = nullptr;  // block-sparse mask (mask_heads, ceil(Nq/128), ceil(Nk/128))
  int mask_heads = 0;              // 1 (shared) or Hq
};

// Bytes of the split partials: nsplit x (B*Hq*Nq rows) x (d + 3) floats.
inline size_t fwd_split_bytes(int B, int Hq, int Nq, int d, int nsplit) {
  return (size_t)nsplit * B * Hq * Nq * (d + 3) * sizeof(float);
}

// Split count the library suggests: none when the unsplit grid already gives every CU
// two workgroups, else enough chunks of the longest query block's key range to reach
// about 512 workgroups (causal: about 460 workgroups that have tiles to process).
int fwd_suggest_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d, bool causal, int dtype);

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
  const uint8_t* bmask = nullptr;  // block-sparse mask, as in FwdArgs
  int mask_heads = 0;
};

constexpr int kStageDq = 1;    // dQ kernel (also writes D and lse*log2(e))
constexpr int kStageDkdv = 2;  // dK/dV kernel (reads D and lse*log2(e))

// FP8 forward: E4M3 codes with Q/K scales per 128 rows of a head and V scales per channel
struct Fwd8Args {
  const void* q;
  const void* k;
  const void* v;
  const float* q_scale;  // (B*Hq, ceil(Nq/128))
  const float* k_scale;  // (B*Hkv, ceil(Nk/128))
  const float* v_scale;  // (B*Hkv, d)
  void* o;               // bf16 (B, Hq, Nq, d)
  float* lse;
  int B, Hq, Hkv, Nq, Nk, d;
  float scale;
  bool causal;
  hipStream_t stream;
};

struct QuantArgs {
  const void* x;
  uint8_t* codes;
  float* scales;  // rows: (B*H, ceil(N/128)); per channel: (B*H, d)
  int B, H, N, d;
  bool per_channel;
  int dtype;
  hipStream_t stream;
};

hipError_t launch_forward_fp8(const Fwd8Args& a);
hipError_t launch_quantize_fp8(const QuantArgs& a);

hipError_t launch_forward(const FwdArgs& a);
hipError_t launch_backward(const BwdArgs& a, int stages);

}  // namespace fa
