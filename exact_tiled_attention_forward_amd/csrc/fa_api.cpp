// C ABI of the attention library: argument validation, then dispatch to the kernels.
// Every check runs before any HIP call, so a rejected call touches no device state.
#include "fa.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "fa_launch.h"

namespace {

constexpr int kVersion = 300;  // 0.3.0
constexpr int kMaxSplits = 1024;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int elem_size(int dtype) {
  switch (dtype) {
    case FA_F32: return 4;
    case FA_F16: return 2;
    case FA_BF16: return 2;
    default: return 0;
  }
}

// Shape checks shared by forward and backward.
int check_shape(int B, int Hq, int Hkv, int Nq, int Nk, int d, int dtype, int causal) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (causal && Nq > Nk) return FA_ERR_SHAPE;  // rows with no visible key
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  const int es = elem_size(dtype);
  if (es == 0) return FA_ERR_UNSUPPORTED;
  // one head of a tensor addressed with 32-bit byte offsets (fp32 gradients: 4 bytes)
  if ((int64_t)Nq * d * 4 >= (int64_t)1 << 31 || (int64_t)Nk * d * 4 >= (int64_t)1 << 31) return FA_ERR_SHAPE;
  // grids: B*Hq*ceil(Nq/32) and B*Hkv*ceil(Nk/32) workgroups at most
  if ((int64_t)B * Hq * ((Nq + 31) / 32) >= (int64_t)1 << 31) return FA_ERR_SHAPE;
  if ((int64_t)B * Hkv * ((Nk + 31) / 32) >= (int64_t)1 << 31) return FA_ERR_SHAPE;
  if ((int64_t)B * Hq >= (int64_t)1 << 30) return FA_ERR_SHAPE;
  return FA_OK;
}

// The 16-bit forward kernels address the G*Nq query rows of one key/value head's group
// (G = Hq/Hkv consecutive query heads) through one buffer resource with 32-bit byte
// offsets, so the packed group, G*Nq*d*2 bytes, must stay below 2^31.
int check_group_rows(int Hq, int Hkv, int Nq, int d, int dtype) {
  if (dtype == FA_F32) return FA_OK;  // the fp32 kernel addresses one head at a time
  if ((int64_t)(Hq / Hkv) * Nq * d * elem_size(dtype) >= (int64_t)1 << 31) return FA_ERR_SHAPE;
  return FA_OK;
}

int check_scale(float scale) {
  if (!isfinite(scale) || !(scale > 0.0f)) return FA_ERR_SCALE;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_forward_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Nq,
                  int Nk, int d, float scale, int causal, fa_dtype_t dtype, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int st = check_shape(B, Hq, Hkv, Nq, Nk, d, (int)dtype, causal);
  if (st != FA_OK) return st;
  if ((st = check_group_rows(Hq, Hkv, Nq, d, (int)dtype)) != FA_OK) return st;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse)) return FA_ERR_ALIGN;

  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal != 0, (int)dtype, stream};
  (void)hipGetLastError();  // clear a pending error so the check below is about this launch
  if (fa::launch_forward(a) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

int fa_forward_split_count(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, fa_dtype_t dtype) {
  if (check_shape(B, Hq, Hkv, Nq, Nk, d, (int)dtype, causal) != FA_OK) return 1;
  return fa::fwd_suggest_splits(B, Hq, Hkv, Nq, Nk, d, causal != 0, (int)dtype);
}

size_t fa_forward_split_workspace_bytes(int B, int Hq, int Nq, int d, int nsplit) {
  if (B < 1 || Hq < 1 || Nq < 1 || nsplit < 2 || nsplit > kMaxSplits) return 0;
  return fa::fwd_split_bytes(B, Hq, Nq, d, nsplit);
}

int fa_forward_split(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Nq,
                     int Nk, int d, float scale, int causal, int nsplit, void* workspace, size_t workspace_bytes,
                     fa_dtype_t dtype, hipStream_t stream) {
  if (nsplit == 1) return fa_forward_ex(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, stream);
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (nsplit < 1 || nsplit > kMaxSplits) return FA_ERR_SHAPE;
  int st = check_shape(B, Hq, Hkv, Nq, Nk, d, (int)dtype, causal);
  if (st != FA_OK) return st;
  if ((st = check_group_rows(Hq, Hkv, Nq, d, (int)dtype)) != FA_OK) return st;
  // grid: every (key/value head, query block) times the splits
  if ((int64_t)B * Hq * ((Nq + 31) / 32 + 1) * nsplit >= (int64_t)1 << 31) return FA_ERR_SHAPE;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse)) return FA_ERR_ALIGN;
  if (!workspace || workspace_bytes < fa::fwd_split_bytes(B, Hq, Nq, d, nsplit)) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;

  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal != 0, (int)dtype, stream};
  a.nsplit = nsplit;
  a.part = (float*)workspace;
  (void)hipGetLastError();
  if (fa::launch_forward(a) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

int fa_forward_sparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                      int Nq, int Nk, int d, float scale, int causal, const void* block_mask, int mask_heads,
                      int nsplit, void* workspace, size_t workspace_bytes, fa_dtype_t dtype, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !block_mask) return FA_ERR_NULL;
  if (nsplit < 1 || nsplit > kMaxSplits) return FA_ERR_SHAPE;
  int st = check_shape(B, Hq, Hkv, Nq, Nk, d, (int)dtype, causal);
  if (st != FA_OK) return st;
  if (mask_heads != 1 && mask_heads != Hq) return FA_ERR_SHAPE;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if ((st = check_group_rows(Hq, Hkv, Nq, d, (int)dtype)) != FA_OK) return st;
  if ((int64_t)B * Hq * ((Nq + 31) / 32 + 1) * nsplit >= (int64_t)1 << 31) return FA_ERR_SHAPE;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse)) return FA_ERR_ALIGN;
  if (nsplit > 1) {
    if (!workspace || workspace_bytes < fa::fwd_split_bytes(B, Hq, Nq, d, nsplit)) return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_ALIGN;
  }
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal != 0, (int)dtype, stream};
  a.nsplit = nsplit;
  a.part = nsplit > 1 ? (float*)workspace : nullptr;
  a.bmask = (const uint8_t*)block_mask;
  a.mask_heads = mask_heads;
  (void)hipGetLastError();
  if (fa::launch_forward(a) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
               float scale, int causal, fa_dtype_t dtype, hipStream_t stream) {
  return fa_forward_ex(q, k, v, o, lse, B, H, H, N, N, d, scale, causal, dtype, stream);
}

size_t fa_backward_workspace_bytes(int B, int H, int N, int d) {
  (void)d;
  if (B < 1 || H < 1 || N < 1) return 0;
  return (size_t)2 * B * H * N * sizeof(float);  // D_i, then lse_i * log2(e)
}

namespace {

// Shared checks of the backward entry points; pointers a stage does not use are passed
// as a valid stand-in (q) by the caller of this helper.
int check_backward(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                   const float* dq, const float* dk, const float* dv, const void* workspace, size_t workspace_bytes,
                   int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal, fa_dtype_t dtype) {
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  int st = check_shape(B, Hq, Hkv, Nq, Nk, d, (int)dtype, causal);
  if (st != FA_OK) return st;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dO) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || !aligned4(lse))
    return FA_ERR_ALIGN;
  if (!workspace || workspace_bytes < fa_backward_workspace_bytes(B, Hq, Nq, d)) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  return FA_OK;
}

int run_backward(const void* q, const void* k, const void* v, const void* dO, const float* lse, float* dq,
                 float* dk, float* dv, void* workspace, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                 int causal, fa_dtype_t dtype, hipStream_t stream, int stages, const void* block_mask = nullptr,
                 int mask_heads = 0) {
  fa::BwdArgs a{q, k, v, nullptr, dO, lse, dq, dk, dv, (float*)workspace, B, Hq, Hkv, Nq, Nk, d, scale, causal != 0,
                (int)dtype, stream};
  a.bmask = (const uint8_t*)block_mask;
  a.mask_heads = mask_heads;
  (void)hipGetLastError();
  if (fa::launch_backward(a, stages) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

}  // namespace

int fa_backward_ex(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                   float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                   int Nq, int Nk, int d, float scale, int causal, fa_dtype_t dtype, hipStream_t stream) {
  const int st = check_backward(q, k, v, o, dO, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, Nq, Nk, d,
                                scale, causal, dtype);
  if (st != FA_OK) return st;
  return run_backward(q, k, v, dO, lse, dq, dk, dv, workspace, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, stream,
                      fa::kStageDq | fa::kStageDkdv);
}

int fa_backward_dq_ex(const void* q, const void* k, const void* v, const void* dO, const float* lse, float* dq,
                      void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                      float scale, int causal, fa_dtype_t dtype, hipStream_t stream) {
  const float* f = (const float*)q;  // stand-in for the gradients this stage does not touch
  const int st = check_backward(q, k, v, q, dO, lse, dq, f, f, workspace, workspace_bytes, B, Hq, Hkv, Nq, Nk, d,
                                scale, causal, dtype);
  if (st != FA_OK) return st;
  return run_backward(q, k, v, dO, lse, dq, nullptr, nullptr, workspace, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype,
                      stream, fa::kStageDq);
}

int fa_backward_dkdv_ex(const void* q, const void* k, const void* v, const void* dO, float* dk, float* dv,
                        const void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                        float scale, int causal, fa_dtype_t dtype, hipStream_t stream) {
  const float* f = (const float*)q;
  const int st = check_backward(q, k, v, q, dO, f, f, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, Nq, Nk, d,
                                scale, causal, dtype);
  if (st != FA_OK) return st;
  return run_backward(q, k, v, dO, nullptr, nullptr, dk, dv, const_cast<void*>(workspace), B, Hq, Hkv, Nq, Nk, d,
                      scale, causal, dtype, stream, fa::kStageDkdv);
}

int fa_backward_sparse(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                       float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes, int B, int Hq,
                       int Hkv, int Nq, int Nk, int d, float scale, int causal, const void* block_mask,
                       int mask_heads, fa_dtype_t dtype, hipStream_t stream) {
  if (!block_mask) return FA_ERR_NULL;
  const int st = check_backward(q, k, v, o, dO, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, Nq, Nk, d,
                                scale, causal, dtype);
  if (st != FA_OK) return st;
  if (mask_heads != 1 && mask_heads != Hq) return FA_ERR_SHAPE;
  return run_backward(q, k, v, dO, lse, dq, dk, dv, workspace, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, stream,
                      fa::kStageDq | fa::kStageDkdv, block_mask, mask_heads);
}

}  // extern "C"

// ----------------------------------------------------------------------------------
// Backward without a caller workspace: the per-row statistics (D_i, lse_i*log2(e)) live in
// a fixed device array of this library.  Each device holds its own copy of the array at
// its own address, looked up once per device; kernels receive that address, never the
// array's host-side name.
// ----------------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on device `dev` (looked up with that device current the first
// time, then cached); nullptr if the runtime refuses.
void* scratch_on(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (p) return p;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void* addr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
  if (cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess || !addr) {
    (void)hipGetLastError();
    return nullptr;
  }
  g_scratch[dev].store(addr, std::memory_order_release);
  return addr;
}

}  // namespace

extern "C" {

int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                        float* dq, float* dk, float* dv, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                        int causal, fa_dtype_t dtype, hipStream_t stream) {
  if (B < 1 || Hq < 1 || Nq < 1) return check_shape(B, Hq, Hkv, Nq, Nk, d, (int)dtype, causal);
  const size_t need = fa_backward_workspace_bytes(B, Hq, Nq, d);
  if (need > (size_t)FA_NOALLOC_SCRATCH_BYTES) {
    // the other checks first, so that a call wrong in several ways reports the usual status
    const int st = check_backward(q, k, v, o, dO, lse, dq, dk, dv, q, need, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                                  dtype);
    return st != FA_OK ? st : FA_ERR_SCRATCH;
  }
  // every check but the workspace's, which the static array satisfies by construction
  int st = check_backward(q, k, v, o, dO, lse, dq, dk, dv, q, need, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype);
  if (st != FA_OK) return st;
  int dev = -1;
  if (stream) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return FA_ERR_HIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return FA_ERR_HIP;
  }
  void* ws = scratch_on(dev);
  if (!ws) return FA_ERR_HIP;
  return run_backward(q, k, v, dO, lse, dq, dk, dv, ws, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, stream,
                      fa::kStageDq | fa::kStageDkdv);
}

int fa_backward(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes, int B, int H, int N,
                int d, float scale, int causal, fa_dtype_t dtype, hipStream_t stream) {
  return fa_backward_ex(q, k, v, o, dO, lse, dq, dk, dv, workspace, workspace_bytes, B, H, H, N, N, d, scale, causal,
                        dtype, stream);
}

int fa_backward_dq(const void* q, const void* k, const void* v, const void* dO, const float* lse, float* dq,
                   void* workspace, size_t workspace_bytes, int B, int H, int N, int d, float scale, int causal,
                   fa_dtype_t dtype, hipStream_t stream) {
  return fa_backward_dq_ex(q, k, v, dO, lse, dq, workspace, workspace_bytes, B, H, H, N, N, d, scale, causal, dtype,
                           stream);
}

int fa_backward_dkdv(const void* q, const void* k, const void* v, const void* dO, float* dk, float* dv,
                     const void* workspace, size_t workspace_bytes, int B, int H, int N, int d, float scale,
                     int causal, fa_dtype_t dtype, hipStream_t stream) {
  return fa_backward_dkdv_ex(q, k, v, dO, dk, dv, workspace, workspace_bytes, B, H, H, N, N, d, scale, causal, dtype,
                             stream);
}

size_t fa_fp8_scale_count(int B, int H, int N, int d, int per_channel) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return 0;
  return per_channel ? (size_t)B * H * d : (size_t)B * H * ((N + 127) / 128);
}

int fa_quantize_fp8(const void* x, void* codes, float* scales, int B, int H, int N, int d, int per_channel,
                    fa_dtype_t dtype, hipStream_t stream) {
  if (!x || !codes || !scales) return FA_ERR_NULL;
  int st = check_shape(B, H, H, N, N, d, (int)dtype, 0);
  if (st != FA_OK) return st;
  if (!aligned4(x) || !aligned16(codes) || !aligned16(scales)) return FA_ERR_ALIGN;
  fa::QuantArgs a{x, (uint8_t*)codes, scales, B, H, N, d, per_channel != 0, (int)dtype, stream};
  (void)hipGetLastError();
  if (fa::launch_quantize_fp8(a) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

int fa_forward_fp8(const void* q8, const float* q_scale, const void* k8, const float* k_scale, const void* v8,
                   const float* v_scale, void* o, float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                   float scale, int causal, hipStream_t stream) {
  if (!q8 || !q_scale || !k8 || !k_scale || !v8 || !v_scale || !o || !lse) return FA_ERR_NULL;
  int st = check_shape(B, Hq, Hkv, Nq, Nk, d, FA_BF16, causal);
  if (st != FA_OK) return st;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8) || !aligned16(o) || !aligned4(lse) || !aligned4(q_scale) ||
      !aligned4(k_scale) || !aligned16(v_scale))
    return FA_ERR_ALIGN;
  fa::Fwd8Args a{q8, k8, v8, q_scale, k_scale, v_scale, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal != 0, stream};
  (void)hipGetLastError();
  if (fa::launch_forward_fp8(a) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE:
      return "a size < 1, Hq not a multiple of Hkv, causal with Nq > Nk, or a tensor too large for the kernels' "
             "32-bit offsets";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension (d must be 64 or 128), dtype, or fp32 backward";
    case FA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned (lse: 4-byte)";
    case FA_ERR_WORKSPACE: return "backward workspace is NULL or smaller than fa_backward_workspace_bytes()";
    case FA_ERR_HIP: return "the HIP runtime rejected a kernel launch";
    case FA_ERR_SCALE: return "scale must be finite and > 0";
    case FA_ERR_SCRATCH:
      return "fa_backward_noalloc: 8*B*Hq*Nq bytes of row statistics exceed its static scratch "
             "(FA_NOALLOC_SCRATCH_BYTES); use fa_backward_ex with a caller workspace";
    default: return "unknown status";
  }
}

int fa_version(void) { return kVersion; }

}  // extern "C"
