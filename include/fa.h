/*
 * fa.h -- exact tiled attention on AMD Instinct MI355X (gfx950), C ABI.
 *
 * The library computes exact softmax attention, O = softmax(scale * Q K^T) V, one tile at
 * a time with the online-softmax rescaling (running max m, running sum l, unnormalised
 * output o), so the N x N score matrix is never written to device memory, and its
 * gradient by recomputing the score tiles from Q, K and the saved per-row logsumexp.
 *
 * Where the operations are defined (page title, section):
 *   - "Flash Attention" (mlx.void.app, chapter 4 deep-dive): intro (the same
 *     softmax(QK^T/sqrt(d)) V, exact up to rounding order); 地基：流式 softmax (safe and
 *     online softmax, the e^(old max - new max) patch); FlashAttention——把整件事分块塞进
 *     SRAM (tiles, recomputation from the saved (m, l) in the backward pass);
 *     FlashAttention-2 (query blocks across the grid, one division by l at the end,
 *     skipping fully masked causal blocks).
 *   - "FlashAttention：IO 感知的快速内存高效精确注意力" (NeurIPS 2022 summary, trdm.cn):
 *     基准/方法设计 (tiling and the (m, l) merge rule), 方法细节 (backward recomputation,
 *     kernel fusion, correctness theorem).
 *   - "大模型数学速成（17）：Flash Attention——不物化注意力矩阵" (shiguol.github.io):
 *     二 (S = QK^T/sqrt(d), P = softmax(S), O = PV), 三 (tiles + online softmax).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *   Layout    Q, K, V, O, dO, dQ, dK, dV are contiguous row-major (B, H, N, d) tensors:
 *             element (b, h, i, c) is at ((b*H + h)*N + i)*d + c.  lse and the
 *             backward workspace are (B, H, N) float.
 *   dtype     q, k, v, o and dO share one storage type, fa_dtype_t.  Arithmetic is
 *             fp32 (products of 16-bit inputs accumulate in fp32; the probabilities are
 *             rounded to the input type before the P V product).
 *   scale     multiplies Q K^T; callers normally pass 1/sqrt(d).  Must be finite and > 0.
 *   causal    non-zero: key j is visible to query i only if j <= i (diagonal included).
 *   lse       natural-log logsumexp of each scaled, masked score row:
 *             lse_i = m_i + ln(l_i), the pages' saved statistics (m, l) in one number.
 *   memory    all pointers are device pointers the caller allocated (e.g. with
 *             hipMalloc or a framework's allocator); the library allocates nothing,
 *             keeps no state between calls, and never frees caller memory.
 *   async     work is enqueued on `stream` (0 = the null stream) and the call returns
 *             without waiting.  Faults inside a kernel surface at the caller's next
 *             synchronisation, not as a return code.
 *   errors    every argument is checked before anything is enqueued; a failing check
 *             returns a negative fa_status_t and enqueues nothing.  FA_ERR_HIP means
 *             the HIP runtime rejected a launch (hipGetLastError after the launch; the
 *             runtime's pending error is cleared before launching).
 *   threads   entry points are stateless and may be called from several host threads.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_F32 = 0,  /* IEEE fp32 storage (forward only) */
  FA_F16 = 1,  /* IEEE fp16 storage */
  FA_BF16 = 2  /* bfloat16 storage */
} fa_dtype_t;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,        /* a required pointer is NULL */
  FA_ERR_SHAPE = -2,       /* a size < 1, Hq not a multiple of Hkv, causal with Nq > Nk,
                              or a tensor too large for 32-bit offsets within a head */
  FA_ERR_UNSUPPORTED = -3, /* d not in {64, 128}, unknown dtype, or fp32 backward */
  FA_ERR_ALIGN = -4,       /* a tensor pointer is not 16-byte aligned */
  FA_ERR_WORKSPACE = -5,   /* backward workspace NULL or smaller than required */
  FA_ERR_HIP = -6,         /* the HIP runtime rejected a kernel launch */
  FA_ERR_SCALE = -7,       /* scale is not finite or not > 0 */
  FA_ERR_SCRATCH = -8      /* fa_backward_noalloc: the call needs more than its static scratch */
} fa_status_t;

/*
 * Largest N for head dimension d and element size s (bytes): one (b, h) slice of a
 * tensor, N*d*4 bytes (the fp32 gradients' size), must stay below 2^31 (the kernels
 * address within a head with 32-bit offsets).  The 16-bit forward entry points also
 * address the G*Nq query rows of a key/value head's group (G = Hq/Hkv) together, so
 * G*Nq*d*2 must stay below 2^31 there.  Larger shapes return FA_ERR_SHAPE.
 * B*H*ceil(N/32) must also fit a grid dimension.
 */

/*
 * fa_forward -- O and lse for one attention call.
 *   q, k, v  in : (B, H, N, d) of `dtype`.
 *   o        out: (B, H, N, d) of `dtype`, O_i = sum_j P_ij V_j with
 *                 P = softmax(scale * Q K^T) (causal-masked if `causal`).
 *   lse      out: (B, H, N) float, lse_i = ln sum_j exp(scale * q_i . k_j) over visible j.
 *   B, H, N  batch, heads, sequence length (>= 1; any N, no padding needed).
 *   d        head dimension, 64 or 128.
 * Returns FA_OK or a negative fa_status_t (nothing enqueued on error).
 * o and lse must not overlap the inputs.
 */
int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal,
               fa_dtype_t dtype, hipStream_t stream);

/*
 * fa_backward_workspace_bytes -- bytes of device workspace fa_backward needs:
 * 8*B*H*N (per query row, D_i = sum_j P_ij dP_ij and lse_i*log2(e) as floats).  For the
 * _ex entry points pass the query heads and query rows (Hq, Nq).  Returns 0 if B, H or
 * N < 1.
 */
size_t fa_backward_workspace_bytes(int B, int H, int N, int d);

/*
 * fa_backward -- gradients of sum(O * dO) with respect to Q, K and V.
 *   q, k, v, o, dO  in : (B, H, N, d) of `dtype` (fp16 or bf16); o is the forward
 *                        output for the same q, k, v, scale and causal.
 *   lse             in : (B, H, N) float from fa_forward for the same call.
 *   dq, dk, dv      out: (B, H, N, d) float (fp32 gradients).
 *   workspace       scratch of at least fa_backward_workspace_bytes(B, H, N, d) bytes,
 *                   16-byte aligned; its contents on entry are ignored.
 * The score tiles are recomputed from Q, K and lse ("FlashAttention：IO 感知…",
 * 方法细节; "Flash Attention", FlashAttention section on training): with
 * P = exp(scale*QK^T - lse), dV = P^T dO, dP = dO V^T, D_i = sum_j P_ij dP_ij
 * (= dO_i . O_i), dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.
 * D is summed from the recomputed fp32 P and dP rather than from the 16-bit o, and P
 * and dS enter the products as hi + lo 16-bit pairs; o is checked (non-NULL, aligned)
 * but its values are not read.  The result is deterministic (no atomics).
 * With fp16 inputs both halves of dS are fp16, whose largest value is 65504, so every
 * |dP_ij - D_i| must stay below it; d * max|dO| * max|V| < 32752 guarantees that.
 * Larger values give non-finite gradients (no status reports it).  bf16 has no such
 * limit short of fp32 overflow.
 * Equivalent to fa_backward_dq followed by fa_backward_dkdv on the same stream and
 * workspace.  Returns FA_OK or a negative fa_status_t.
 */
int fa_backward(const void* q, const void* k, const void* v, const void* o, const void* dO,
                const float* lse, float* dq, float* dk, float* dv,
                void* workspace, size_t workspace_bytes,
                int B, int H, int N, int d, float scale, int causal,
                fa_dtype_t dtype, hipStream_t stream);

/*
 * fa_backward_dq -- first stage of fa_backward: dq, and D_i and lse_i*log2(e) into
 * `workspace` for the second stage.  Arguments as for fa_backward.
 */
int fa_backward_dq(const void* q, const void* k, const void* v, const void* dO,
                   const float* lse, float* dq, void* workspace, size_t workspace_bytes,
                   int B, int H, int N, int d, float scale, int causal,
                   fa_dtype_t dtype, hipStream_t stream);

/*
 * fa_backward_dkdv -- second stage of fa_backward: dk and dv, reading the workspace a
 * preceding fa_backward_dq with the same arguments filled (on the same stream, or
 * ordered after it by the caller).  Arguments as for fa_backward.
 */
int fa_backward_dkdv(const void* q, const void* k, const void* v, const void* dO,
                     float* dk, float* dv, const void* workspace, size_t workspace_bytes,
                     int B, int H, int N, int d, float scale, int causal,
                     fa_dtype_t dtype, hipStream_t stream);

/*
 * Query and key lengths that differ, and grouped key/value heads
 * ----------------------------------------------------------------
 * The pages allow Q and K/V of different lengths (cross-attention, a decode step
 * against a cached K/V: cf-1.com article, section 3.4) and name grouped-query
 * attention and causal masks as variants that only skip or mask (i, j) pairs inside
 * the block loop ("大模型数学速成（17）", section 四).  The _ex entry points take
 *   q, o, dO, dq    (B, Hq, Nq, d),    lse (B, Hq, Nq) float,
 *   k, v, dk, dv    (B, Hkv, Nk, d),
 * with Hq a multiple of Hkv: query head h reads key/value head h / (Hq/Hkv)
 * (consecutive query heads share one key/value head).  dk and dv of a shared head
 * are the sums over its query heads (computed in one pass, no atomics).  With
 * causal != 0 the Nq queries are the last Nq positions of the Nk-long sequence: key j
 * is visible to query i iff j <= i + (Nk - Nq) (a decode step's query sees the whole
 * cache); causal with Nq > Nk is rejected with FA_ERR_SHAPE (some rows would see no
 * key).  Hq % Hkv != 0 is FA_ERR_SHAPE.  The workspace of the backward is
 * fa_backward_workspace_bytes(B, Hq, Nq, d).  The square entry points above are these
 * with Hq = Hkv = H and Nq = Nk = N.
 */
int fa_forward_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                  fa_dtype_t dtype, hipStream_t stream);

int fa_backward_ex(const void* q, const void* k, const void* v, const void* o, const void* dO,
                   const float* lse, float* dq, float* dk, float* dv,
                   void* workspace, size_t workspace_bytes,
                   int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                   fa_dtype_t dtype, hipStream_t stream);

int fa_backward_dq_ex(const void* q, const void* k, const void* v, const void* dO,
                      const float* lse, float* dq, void* workspace, size_t workspace_bytes,
                      int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                      fa_dtype_t dtype, hipStream_t stream);

int fa_backward_dkdv_ex(const void* q, const void* k, const void* v, const void* dO,
                        float* dk, float* dv, const void* workspace, size_t workspace_bytes,
                        int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                        fa_dtype_t dtype, hipStream_t stream);

/*
 * Split key range (decode steps and other small grids)
 * ----------------------------------------------------
 * When B*Hkv*ceil(G*Nq / rows-per-workgroup) workgroups cannot fill the 256 CUs (a
 * decode step has one query row per head; a short batch of long causal rows leaves the
 * longest row to one workgroup), fa_forward_split cuts the key range of every query
 * block into up to `nsplit` chunks, computes each chunk's partial result (unnormalised
 * o, running max m and sums l in the tiled recurrence) in its own workgroup, and merges
 * them with the pages' (m, l) merge rule ("FlashAttention：IO 感知…", 基准/方法设计:
 * m = max(m1, m2), l = e^(m1-m) l1 + e^(m2-m) l2, and the same factors on o), which is
 * exact up to rounding order.  The rows of one key/value head's group are processed
 * together, so the group's K and V are read once per chunk.  A group of at most 32 rows
 * (G*Nq <= 32, a decode step) spreads each chunk's keys over the workgroup's waves
 * instead of its rows, with three key tiles in flight.
 *   fa_forward_split_count    the split count the library suggests for these arguments
 *                             (1: the unsplit grid already gives each CU two workgroups;
 *                             for groups of at most 32 rows, and for fp32, about one
 *                             workgroup per CU).
 *   fa_forward_split_workspace_bytes
 *                             nsplit * B*Hq*Nq * (d + 3) * 4 bytes for nsplit >= 2 (0 for
 *                             nsplit < 2 or > 1024).
 *   fa_forward_split          as fa_forward_ex plus nsplit in [1, 1024] and a 16-byte
 *                             aligned device workspace of at least that size (contents on
 *                             entry ignored; NULL allowed when nsplit == 1, which is exactly
 *                             fa_forward_ex).  Any dtype (fp32 splits each 64-row block of a
 *                             query head into chunks of its 32-key tiles).  Two kernels on
 *                             `stream`.
 */
int fa_forward_split_count(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, fa_dtype_t dtype);

size_t fa_forward_split_workspace_bytes(int B, int Hq, int Nq, int d, int nsplit);

int fa_forward_split(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                     int nsplit, void* workspace, size_t workspace_bytes,
                     fa_dtype_t dtype, hipStream_t stream);

/*
 * Block-sparse masks
 * ------------------
 * Block-sparse attention ("FlashAttention：IO 感知…", 方法细节, and its long-range
 * results) skips whole zero blocks of a given block mask.  block_mask is a device array
 * of uint8 with shape (mask_heads, ceil(Nq/128), ceil(Nk/128)), row-major, shared by
 * every batch element; mask_heads is 1 (one layer for every query head) or Hq (one per
 * query head).  Byte (h, i, j) == 0 hides keys 128j .. 128j+127 from queries
 * 128i .. 128i+127 of query head h, on top of the causal mask.  Hidden blocks are
 * neither loaded nor computed.  A query row left with no visible key gets O = 0,
 * lse = -inf and zero gradients.  Other arguments as for fa_forward_split /
 * fa_backward_ex (nsplit >= 1; the workspace only for nsplit > 1); 16-bit inputs only
 * (FA_ERR_UNSUPPORTED for fp32); mask_heads not 1 or Hq is FA_ERR_SHAPE; a NULL mask is
 * FA_ERR_NULL.  The mask must not change between the forward and backward calls.
 */
int fa_forward_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                      const void* block_mask, int mask_heads, int nsplit,
                      void* workspace, size_t workspace_bytes,
                      fa_dtype_t dtype, hipStream_t stream);

int fa_backward_sparse(const void* q, const void* k, const void* v, const void* o, const void* dO,
                       const float* lse, float* dq, float* dk, float* dv,
                       void* workspace, size_t workspace_bytes,
                       int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                       const void* block_mask, int mask_heads,
                       fa_dtype_t dtype, hipStream_t stream);

/*
 * FP8 (E4M3) forward
 * ------------------
 * "Flash Attention" (mlx.void.app), section FlashAttention-3: fp8 products run at about
 * twice the 16-bit rate; an E4M3 number has 256 bit patterns and a largest value of 448,
 * so everything rests on the scale factors, and block quantization gives each block its
 * own scale so that an outlier only coarsens its block.  Here:
 *   fa_fp8_scale_count  floats of scales for x (B, H, N, d): B*H*ceil(N/128) per-row-block
 *                       scales, or B*H*d per-channel scales (per_channel != 0); 0 on bad sizes.
 *   fa_quantize_fp8     x (B, H, N, d) of `dtype` (fp32, fp16, bf16; 4-byte aligned) ->
 *                       codes (uint8 E4M3 bit patterns, 16-byte aligned) and scales
 *                       (float, 16-byte aligned): scale = max |x| / 448 over each 128-row
 *                       block of a head (or each channel of a head), 1 for an all-zero block;
 *                       code = E4M3(x / scale), nearest even, clamped to +-448.
 *   fa_forward_fp8      O (bf16, like q) and lse (float) from codes q8 (B, Hq, Nq, d) with
 *                       row-block scales (B*Hq, ceil(Nq/128)), k8 (B, Hkv, Nk, d) with
 *                       row-block scales (B*Hkv, ceil(Nk/128)), and v8 (B, Hkv, Nk, d) with
 *                       channel scales (B*Hkv, d), i.e. Q ~ code * q_scale of the row's block.
 *                       The scores use the exact products of the codes (fp32 accumulation)
 *                       times the two block scales; the probabilities (relative to the
 *                       running max, updated every 64 keys) are summed in fp32 for the
 *                       normaliser and lse, and rounded to E4M3 for the P V product; O is
 *                       multiplied by the channel scales at the end.  Grouping, causal
 *                       alignment and errors as for fa_forward_ex; d is 64 or 128.
 * The error this adds over fp16 inputs is that of E4M3 rounding (see the tests' bounds);
 * a fixed random rotation of Q and K before quantization (the page's incoherent
 * processing) is the caller's choice and leaves the scores unchanged before rounding.
 */
size_t fa_fp8_scale_count(int B, int H, int N, int d, int per_channel);

int fa_quantize_fp8(const void* x, void* codes, float* scales, int B, int H, int N, int d, int per_channel,
                    fa_dtype_t dtype, hipStream_t stream);

int fa_forward_fp8(const void* q8, const float* q_scale, const void* k8, const float* k_scale,
                   const void* v8, const float* v_scale, void* o, float* lse,
                   int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                   hipStream_t stream);

/*
 * Backward for callers that cannot allocate
 * -----------------------------------------
 * For code under HIP graph capture, tight serving or training loops, and harnesses that
 * forbid device allocation: fa_backward_noalloc is fa_backward_ex without the workspace
 * argument.  The per-query-row statistics the two backward kernels exchange (D_i and
 * lse_i*log2(e), 8 bytes per row) live in a static device array of the library,
 * FA_NOALLOC_SCRATCH_BYTES (16 MiB) on every device the library runs on, held until the
 * process ends.  That limits a call to B*Hq*Nq <= FA_NOALLOC_SCRATCH_BYTES / 8 = 2^21
 * query rows (e.g. 2 x 16 x 8192 = 2^18); larger calls return FA_ERR_SCRATCH and enqueue
 * nothing.  The call allocates no memory: on its first use on a device it looks up that
 * device's copy of the array (with the stream's device current), then only launches the
 * two kernels on `stream` (the null stream: the current device).  The array needs no
 * clearing: the first kernel writes every row the second reads.  All calls on one device
 * share its one array, so calls that overlap in time on one device (on different
 * streams, or from several host threads without ordering) race and give wrong results;
 * calls in stream order are safe.  Other arguments, results and errors as for
 * fa_backward_ex (the same kernels; the results are bitwise equal).
 */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)

int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                        const float* lse, float* dq, float* dk, float* dv,
                        int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                        fa_dtype_t dtype, hipStream_t stream);

/* fa_status_string -- static, human-readable text for a status code. */
const char* fa_status_string(int status);

/* fa_version -- library version as major*10000 + minor*100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
