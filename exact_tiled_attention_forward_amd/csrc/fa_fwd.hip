// Exact attention forward on gfx950: O = softmax(scale * Q K^T) V, one tile at a time.
//
// Method ("Flash Attention", mlx.void.app, sections 地基：流式 softmax and
// FlashAttention-2; "FlashAttention：IO 感知的快速内存高效精确注意力", trdm.cn, section
// 基准/方法设计): every workgroup owns one (batch, head, query block); it streams the key
// and value tiles of that head through LDS and keeps, per query row, a running max m, a
// running sum l and an unnormalised output o.  When a tile raises the max, l and o are
// multiplied by e^(m_old - m_new); after the last tile O = o / l.  The N x N score
// matrix never leaves the chip.  The per-row logsumexp m + ln l is written for the
// backward pass.  With causal masking, tiles that lie wholly in a query's future are
// not computed (same page, FlashAttention-2 section).
//
// Mapping to CDNA4 (one wave = 64 lanes owns 32 query rows):
//   * o and l are rescaled only when a row's exponent reference must move: when a
//     tile's max passes it by more than 8 in log2 units, or, in the d = 64 kernel
//     without a block mask, when a tile's probabilities against it add up to more than
//     the 16-bit P can safely hold (kSumLimit).
//   * S^T = K Q^T on v_mfma_f32_32x32x16: K (A operand) is read row-wise from LDS, Q (B
//     operand) stays in registers for the whole kernel.  In the accumulator, lane l holds
//     query l%32 and 16 of the tile's 32 keys, so the row max and row sum are in-lane
//     reductions plus one v_permlane32_swap between the wave's halves.
//   * exponentials in base 2: p = exp2(s*c - m) with c = scale*log2(e), one FMA + one
//     v_exp_f32 per score; m and l live in base 2 and LSE is converted at the end.
//   * O^T += V^T P^T: P^T is the S^T accumulator converted to 16 bits in place (B
//     operand); V^T is read from the row-major V tile with ds_read_b64_tr_b16.  Besides
//     the fp32 row sum l (for the logsumexp), a second sum adds up the 16-bit
//     probabilities the product actually used and normalises O: at d = 128 on the matrix
//     core (a 16x16x32 product against a constant operand of ones, row_sum_operand), at
//     d = 64 with one v_dot2 against (1, 1) per pair.
//   * K/V tiles are fetched HBM -> LDS with buffer_load ... lds, double-buffered, so the
//     next tile's fetch overlaps this tile's math.
#include <algorithm>
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

// ----------------------------------------------------------------------------------
// 16-bit inputs (bf16 or fp16), fp32 accumulation.
//   NW waves per workgroup, 32 query rows per wave -> BR = 32*NW rows per workgroup.
//   BC keys per tile; K and V tiles double-buffered in LDS, the next tile's fetch issued
//   right after the barrier so it overlaps this tile's math.
//
// Lazy rescaling: the exponent reference m of a row only moves when a tile's max exceeds
// it by more than kRescaleSlack (log2 units).  Until then p = exp2(s*c - m) <= 2^slack and
// o, l need no rescale: exp2(s - m_old) exp2(m_old - m_new) = exp2(s - m_new) holds for
// any reference, so O = o/l and lse = m + log2(l) are unchanged.  The decision is
// wave-uniform (one branch per tile) and after the first tiles of a row it is almost
// never taken, which removes the multiply of every accumulator by alpha from the loop.
//
// Several waves share each SIMD (two at d = 128, four at d = 64).  Waves that run this
// code in lock step multiply together and then exponentiate together; the two-phase
// kernel below (d = 128 without a block mask or split) holds the two waves of a SIMD half
// a tile apart, so that one's products run beside the other's softmax.
// ----------------------------------------------------------------------------------
constexpr float kRescaleSlack = 8.0f;
// Products the two-phase kernel reads its LDS operands ahead of use.
constexpr int kPpRing = 6;
// Largest sum of one lane's probabilities in a tile before the 256-row kernel at d = 64
// moves its exponent reference.  The sum bounds every probability, and the P V product
// takes each one in the input's 16-bit format: bf16 reaches about 2^128, so there the
// bound is 2^64, far from fp32 overflow of o and l too; fp16 holds at most 65504, so there
// it is 2^15 (a tile whose scores pass the reference by about 15 in log2 units moves it).
// Skipping the per-tile row max saves about a tenth of the softmax's vector instructions
// (long non-causal d = 64 workload: 1.171 -> 1.127 ms).
template <class T>
constexpr float kSumLimit = 18446744073709551616.0f;  // 2^64
template <>
constexpr float kSumLimit<f16_t> = 32768.0f;  // 2^15

// Rows of the 16-bit kernel: the G*Nq query rows of one key/value head's group, packed.
// The group's query heads are consecutive, so its rows are contiguous in Q and O, and
// packed row r is position r % Nq of query head (group's first head + r / Nq).  Packing
// lets one workgroup serve a whole group when G*Nq is small (a decode step), so the
// group's K/V tiles are read once.
//
// Positions of the packed rows [r0, r1] (r0 <= r1): contiguous inside one head, else
// every position (a conservative range for the causal skip and mask decisions).
__host__ __device__ inline void pos_range(int r0, int r1, int Nq, int& pmin, int& pmax) {
  if (r0 / Nq == r1 / Nq) {
    pmin = r0 % Nq;
    pmax = r1 % Nq;
  } else {
    pmin = 0;
    pmax = Nq - 1;
  }
}

// Key tiles a query block of packed rows [q0, q0 + BR) needs: all of them, or with causal
// masking those up to the last position of the block plus Nk - Nq.  The split epilogue's
// merge uses the same count to know which partial results exist.
template <int BR, int BC, bool CAUSAL>
__host__ __device__ inline int block_key_tiles(int q0, int R, int Nq, int Nk) {
  const int nkt_all = (Nk + BC - 1) / BC;
  if (!CAUSAL) return nkt_all;
  int pmin, pmax;
  const int r1 = q0 + BR - 1 < R - 1 ? q0 + BR - 1 : R - 1;
  pos_range(q0, r1, Nq, pmin, pmax);
  const int kt = (pmax + Nk - Nq) / BC + 1;
  return kt < nkt_all ? kt : nkt_all;
}

struct Fwd16Params {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  uint16_t* O;
  float* LSE;
  int BHkv, G, Nq, Nk;  // key/value heads (B*Hkv), query heads per group, lengths
  float c;              // scale * log2(e)
  int ct;               // key tiles per split (>= every block's tile count: no split)
  int nsplit;           // splits the partial buffer holds
  float* part;          // split partials: o [s][row][D], then m, l, lr [s][row]
  // block-sparse mask: (mask heads, nbq, nbk) bytes, 0 = hidden 128 x 128 block; a
  // query head's layer is at its index within the batch times bm_hstride (0: shared)
  const uint8_t* bmask;
  int Hkv, bm_hstride, nbk;
};

constexpr int kMaskBlock = 128;  // rows and columns of one block of a block-sparse mask

// Does any packed row in [r0, r1) of key/value head bkv need key tile j (tile keys
// [j*BC, j*BC + BC), inside one mask block because BC divides 128)?  Walks the rows in
// segments that share a query head and a 128-row mask block.
template <int BC>
__device__ __forceinline__ bool rows_need_tile(const Fwd16Params& P, int bkv, int r0, int r1, int j) {
  static_assert(kMaskBlock % BC == 0, "a key tile must lie inside one mask block");
  const int kblk = (j * BC) / kMaskBlock;
  const int hbase = (bkv % P.Hkv) * P.G;  // the group's first query head within the batch
  const int nbq = (P.Nq + kMaskBlock - 1) / kMaskBlock;
  for (int r = r0; r < r1;) {
    const int pos = r % P.Nq;
    const int hq = hbase + r / P.Nq;
    if (P.bmask[(size_t)hq * P.bm_hstride + (size_t)(pos / kMaskBlock) * P.nbk + kblk]) return true;
    const int step = min(kMaskBlock - pos % kMaskBlock, P.Nq - pos);
    r += step;
  }
  (void)nbq;
  return false;
}

// Merge of the split partials of one packed row with the (m, l) rule of the tiled
// method ("FlashAttention：IO 感知…", 基准/方法设计): with M = max_s m_s and
// a_s = 2^(m_s - M), O = sum_s a_s o_s / sum_s a_s lr_s and lse = M + log2(sum_s a_s l_s)
// (base 2, converted to natural log).  D / E lanes per row, E columns each (E = 4 for
// the 256-row kernel's many rows, E = 2 for the few-row kernel's handful).  The splits
// are taken MC at a time: all loads of a chunk are issued together (one memory round
// trip per chunk), then the chunk joins the running (M, sums) by the same rule.  With at
// most MC splits there is one chunk, whose sums run in split order against the global M.
template <class T, int D, int E, int BR, int BC, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_merge_kernel(const Fwd16Params P) {
  static_assert(E == 2 || E == 4, "columns per lane");
  typedef float fE __attribute__((ext_vector_type(E)));
  constexpr int LPR = D / E;      // lanes per row
  constexpr int RPB = 256 / LPR;  // rows per workgroup
  constexpr int MC = 8;           // splits per chunk
  const int R = P.G * P.Nq;
  const size_t nrows = (size_t)P.BHkv * R;
  const size_t g = (size_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int c0 = (threadIdx.x % LPR) * E;
  if (g >= nrows) return;
  const int r = (int)(g % R);
  const int ktiles = block_key_tiles<BR, BC, CAUSAL>((r / BR) * BR, R, P.Nq, P.Nk);
  const int ns = (ktiles + P.ct - 1) / P.ct;  // splits that wrote a partial for this row
  const float* pm = P.part + (size_t)P.nsplit * nrows * D;
  const float* pl = pm + (size_t)P.nsplit * nrows;
  const float* plr = pl + (size_t)P.nsplit * nrows;
  float M = -INFINITY;  // stays -inf only for a row with no visible key
  float acc[E] = {};
  float lt = 0.f, lr = 0.f;
  for (int s0 = 0; s0 < ns; s0 += MC) {
    float ms[MC], ls[MC], lrs[MC];
    fE os[MC];
#pragma unroll
    for (int k = 0; k < MC; ++k) {
      const int s = s0 + k;
      ms[k] = -INFINITY;
      ls[k] = lrs[k] = 0.f;
      os[k] = (fE){};
      if (s < ns) {  // partials past the row's last split were not written
        ms[k] = pm[s * nrows + g];
        ls[k] = pl[s * nrows + g];
        lrs[k] = plr[s * nrows + g];
        os[k] = *(const fE*)(P.part + (s * nrows + g) * D + c0);
      }
    }
    float Mc = M;
#pragma unroll
    for (int k = 0; k < MC; ++k) Mc = fmaxf(Mc, ms[k]);
    if (Mc > M && M != -INFINITY) {  // a later chunk raised the max: rescale what is summed
      const float f = fast_exp2(M - Mc);
      lt *= f;
      lr *= f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] *= f;
    }
    M = Mc;
#pragma unroll
    for (int k = 0; k < MC; ++k) {
      const float a = (ms[k] == -INFINITY) ? 0.f : fast_exp2(ms[k] - M);
      lt += a * ls[k];
      lr += a * lrs[k];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += a * os[k][e];
    }
  }
  const float inv = lr > 0.f ? 1.0f / lr : 0.f;
  uint16_t* orow = P.O + g * D + c0;
  if constexpr (E == 4) {
    u32x2 w;
    w.x = T::pack(acc[0] * inv, acc[1] * inv);
    w.y = T::pack(acc[2] * inv, acc[3] * inv);
    *(u32x2*)orow = w;
  } else {
    *(uint32_t*)orow = T::pack(acc[0] * inv, acc[1] * inv);
  }
  if (c0 == 0) P.LSE[g] = lt > 0.f ? (M + log2f(lt)) * kLn2 : -INFINITY;
}

template <class T, int D, int NW, int BC, int WPE, bool CAUSAL, bool SPLIT, bool SPARSE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void fwd16_kernel(
    const Fwd16Params P) {
  constexpr int BR = 32 * NW;
  constexpr int NT = NW * 64;
  constexpr int TB = BC * D * 2;  // bytes of one K or V tile
  constexpr int KB = BC / 32;     // 32-key accumulator blocks per tile
  constexpr int DS = D / 16;      // contraction steps over the head dimension
  constexpr int DB = D / 32;      // 32-wide blocks of the output's head dimension
  static_assert(BC % 32 == 0, "key tile");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TB];  // K0 K1 V0 V1
  FA_LDS uint8_t* lds = (FA_LDS uint8_t*)(smem);

  const int Nq = P.Nq, Nk = P.Nk, R = P.G * P.Nq;
  const float c = P.c;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), half = lane >> 5, c32 = lane & 31;
  const int nqb = (R + BR - 1) / BR;
  const int bkv = blockIdx.x % P.BHkv;
  const int t = blockIdx.x / P.BHkv;
  int qb = t % nqb;
  const int split = t / nqb;
  if (CAUSAL) qb = nqb - 1 - qb;  // longest rows first
  const int q0 = qb * BR;
  const int qw0 = q0 + 32 * wave;
  const int qrow = qw0 + c32;          // packed row of this lane
  const int pos = qrow % Nq;           // its position among the Nq queries
  const int off = Nk - Nq;             // causal: position i sees keys j <= i + off
  const bool wave_rows = qw0 < R;      // the wave holds at least one real row
  int wpmin = 0, wpmax = -1;
  if (wave_rows) pos_range(qw0, min(qw0 + 31, R - 1), Nq, wpmin, wpmax);

  const int ktiles = block_key_tiles<BR, BC, CAUSAL>(q0, R, Nq, Nk);
  const int j0 = SPLIT ? split * P.ct : 0;
  const int j1 = SPLIT ? min(j0 + P.ct, ktiles) : ktiles;
  if (j0 >= j1) return;  // an empty split: the merge does not read it

  const size_t head = (size_t)bkv * R * D;   // the group's first query row
  const size_t kvhead = (size_t)bkv * Nk * D;
  const auto rq = make_rsrc(P.Q + head, (uint32_t)R * D * 2);
  const auto rk = make_rsrc(P.K + kvhead, (uint32_t)Nk * D * 2);
  const auto rv = make_rsrc(P.V + kvhead, (uint32_t)Nk * D * 2);

  // block-sparse: tiles no row of the workgroup needs are neither loaded nor computed.  The
  // next needed tile is searched 64 tiles at a time, one tile per lane, so that a run of
  // hidden tiles costs one round of mask reads instead of one read after another.
  const int rend = min(q0 + BR, R);
  auto next_tile = [&](int j) {
    if (SPARSE) {
      for (; j < j1; j += 64) {
        const int jl = j + lane;
        const uint64_t need = __builtin_amdgcn_ballot_w64(jl < j1 && rows_need_tile<BC>(P, bkv, q0, rend, jl));
        if (need != 0) return j + (int)__builtin_ctzll(need);
      }
      return j1;
    }
    return j;
  };
  // this lane's row of the mask (its query head and 128-row block)
  const uint8_t* mrow = nullptr;
  if (SPARSE) {
    const int r = qrow < R ? qrow : q0;
    mrow = P.bmask + (size_t)((bkv % P.Hkv) * P.G + r / Nq) * P.bm_hstride +
           (size_t)((r % Nq) / kMaskBlock) * P.nbk;
  }

  int j = next_tile(j0);
  if (j < j1) {
    tile_load_async<D, BC, NT>(lds, rk, j * BC, tid);
    tile_load_async<D, BC, NT>(lds + 2 * TB, rv, j * BC, tid);
  }

  u32x4 qf[DS];
#pragma unroll
  for (int st = 0; st < DS; ++st) qf[st] = buffer_load16(rq, qrow * (D * 2) + ((2 * st + half) << 4));

  // base-2 exponent reference m (of s*c); running sums: l (this half's keys) of the fp32
  // probabilities, for the logsumexp, and the sum of the same probabilities rounded to 16
  // bits, for O.  At d = 128 the rounded sum is taken on the matrix core beside the P V
  // products (lsum, row_sum_operand); at d = 64, where the kernel runs four waves per SIMD
  // in 128 VGPRs, the 8 registers that takes spill, so there it is one v_dot2 per pair
  // (lr, this half's keys).  m stays -inf while every key seen so far is masked for the
  // row (only possible in a split that starts past a row's last visible key).
  constexpr bool kMfmaSum = D == 128;
  float m = -INFINITY, l = 0.f, lr = 0.f;
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x16){};
  const u32x4 ones = row_sum_operand<T>(lane);
  f32x4 lsum = (f32x4){};

  // block-sparse masking: the lane's last visible key, less the 4 * half rows its
  // accumulator layout adds
  const int lane_lim = (SPARSE && D == 128) ? (CAUSAL ? min(pos + off, Nk - 1) : Nk - 1) - 4 * half : 0;
  for (int cur = 0; j < j1; cur ^= 1) {
    wait_vmem();
    fa_sync();
    const int k0 = j * BC;
    // block-sparse: this lane's row keeps the tile's mask block.  Read and consumed (the
    // ballot) before the next tile's fill is issued, so that waiting for this byte does not
    // wait for the fill.
    const bool lane_keep = SPARSE ? mrow[k0 / kMaskBlock] != 0 : true;
    const uint64_t keep = SPARSE ? __builtin_amdgcn_ballot_w64(lane_keep) : ~0ull;
    const int jn = next_tile(j + 1);
    if (jn < j1) {
      tile_load_async<D, BC, NT>(lds + (cur ^ 1) * TB, rk, jn * BC, tid);
      tile_load_async<D, BC, NT>(lds + (2 + (cur ^ 1)) * TB, rv, jn * BC, tid);
    }
    j = jn;
    if (!wave_rows || (CAUSAL && k0 > wpmax + off)) continue;  // no row of the wave sees the tile
    bool mask_lanes = false;
    if (SPARSE) {
      if (keep == 0) continue;
      mask_lanes = keep != ~0ull;
    }
    const FA_LDS uint8_t* kt = lds + cur * TB;
    const FA_LDS uint8_t* vt = lds + (2 + cur) * TB;

    // S^T = K Q^T for the tile
    f32x16 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[kb] = (f32x16){};
#pragma unroll
      for (int st = 0; st < DS; ++st) s[kb] = T::mfma(lds_row16<D>(kt, 32 * kb + c32, 2 * st + half), qf[st], s[kb]);
    }

    // masks: keys past the end, (causal) keys after the query's position, and
    // (block-sparse) rows whose mask block is 0
    if ((k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > wpmin + off) || mask_lanes) {
      if constexpr (SPARSE && D == 128) {
        // the key's offset in the tile, a constant per register, against the lane's last
        // visible offset (-1: the lane's mask block is hidden): one compare per score.
        // Block-masked d = 128 launches only: in the causal split kernel the same form
        // spills (46 VGPRs at d = 64) and runs twice as long, and at d = 64 it spills too.
        const int lim = lane_keep ? lane_lim - k0 : -1;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) s[kb][i] = 32 * kb + acc_row(i, 0) > lim ? -INFINITY : s[kb][i];
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + 32 * kb + acc_row(i, half);
            s[kb][i] = (!lane_keep || key >= Nk || (CAUSAL && key > pos + off)) ? -INFINITY : s[kb][i];
          }
      }
    }

    // online softmax: exponentials, sums, 16-bit P
    uint32_t pk[KB][8];
    if constexpr (D == 64 && !SPARSE) {
      // The tile's row max is only taken when the exponent reference has to move: when
      // some lane's sum of this tile's probabilities exceeds kSumLimit (or is not finite),
      // which bounds every probability, or before the row's first visible key (m = -inf).
      float rs, rsr;
      auto exponentials = [&](float mu) {
        rs = 0.f;
        rsr = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int t2 = 0; t2 < 8; ++t2) {
            const float p0 = fast_exp2(fmaf(s[kb][2 * t2], c, -mu));
            const float p1 = fast_exp2(fmaf(s[kb][2 * t2 + 1], c, -mu));
            rs += p0 + p1;
            pk[kb][t2] = T::pack(p0, p1);
            if constexpr (!kMfmaSum) rsr = T::sum2(pk[kb][t2], rsr);
          }
      };
      bool move = __builtin_amdgcn_ballot_w64(m == -INFINITY) != 0;
      if (!move) {
        exponentials(m);
        move = __builtin_amdgcn_ballot_w64(!(rs <= kSumLimit<T>)) != 0;
      }
      if (move) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; i += 2) mx = max_nan(max_nan(mx, s[kb][i]), s[kb][i + 1]);
        mx = max_halves(mx) * c;
        const float m_new = fmaxf(m, mx);
        const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m - m_new);  // o, l are 0 while m = -inf
        l *= alpha;
        lr *= alpha;
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
        m = m_new;
        exponentials(m == -INFINITY ? 0.f : m);  // every score of such a row is -inf: p = 0
      }
      l += rs;
      lr += rsr;
    } else {
      // Row max every tile, and the lazy rule for the reference: the large-head
      // workload's outlier rows would send many tiles through a second pass of
      // exponentials under the sum check above (0.529 -> 0.559 ms).  Block-sparse
      // launches keep it too (the sum check spills there).
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) mx = max_nan(max_nan(mx, s[kb][i]), s[kb][i + 1]);
      mx = max_halves(mx) * c;
      if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleSlack) != 0) {
        const float m_new = fmaxf(m, mx);
        const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m - m_new);  // o, l are 0 while m = -inf
        l *= alpha;
        lr *= alpha;
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
        m = m_new;
      }
      const float mu = (m == -INFINITY) ? 0.f : m;  // every score of such a row is -inf: p = 0
      float rs = 0.f, rsr = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int t2 = 0; t2 < 8; ++t2) {
          const float p0 = fast_exp2(fmaf(s[kb][2 * t2], c, -mu));
          const float p1 = fast_exp2(fmaf(s[kb][2 * t2 + 1], c, -mu));
          rs += p0 + p1;
          pk[kb][t2] = T::pack(p0, p1);
          if constexpr (!kMfmaSum) rsr = T::sum2(pk[kb][t2], rsr);
        }
      l += rs;
      lr += rsr;
    }

    // O^T += V^T P^T, and the rounded sums
#pragma unroll
    for (int ks = 0; ks < BC / 16; ++ks) {
      const int kb = ks >> 1, mm = ks & 1;
      const u32x4 b = (u32x4){pk[kb][4 * mm], pk[kb][4 * mm + 1], pk[kb][4 * mm + 2], pk[kb][4 * mm + 3]};
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = T::mfma(lds_colop<D>(vt, 16 * ks, 32 * db, lane), b, o[db]);
      if constexpr (kMfmaSum) lsum = T::mfma16(ones, b, lsum);
    }
  }

  const float lt = sum_halves(l);
  const float ltr = kMfmaSum ? lsum[0] : sum_halves(lr);
  if (qrow >= R) return;
  if (SPLIT) {
    // partial result of this split: unnormalised o (fp32), the exponent reference m and
    // both sums, merged by fwd_merge_kernel with the (m, l) rule
    const size_t nrows = (size_t)P.BHkv * R;
    const size_t row = (size_t)split * nrows + (size_t)bkv * R + qrow;
    float* prow = P.part + row * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * half;
        *(f32x4*)(prow + d) = (f32x4){o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
      }
    if (half == 0) {
      float* pm = P.part + (size_t)P.nsplit * nrows * D;  // m [s][row], l, lr after it
      const size_t i = (size_t)split * nrows + (size_t)bkv * R + qrow;
      pm[i] = m;
      pm[(size_t)P.nsplit * nrows + i] = lt;
      pm[(size_t)2 * P.nsplit * nrows + i] = ltr;
    }
    return;
  }
  // epilogue: one division per row, 16-bit O, natural-log LSE.  O divides by the sum of
  // the rounded probabilities the P V product used, which makes it an exact weighted
  // average of V rows; the logsumexp uses the fp32 sum.  A row with no visible key (only
  // under a block-sparse mask) gets O = 0 and lse = -inf.
  const float inv = ltr > 0.f ? 1.0f / ltr : 0.f;
  uint16_t* orow = P.O + head + (size_t)qrow * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * db + 8 * g + 4 * half;
      u32x2 w;
      w.x = T::pack(o[db][4 * g] * inv, o[db][4 * g + 1] * inv);
      w.y = T::pack(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
      *(u32x2*)(orow + d) = w;
    }
  if (half == 0) P.LSE[(size_t)bkv * R + qrow] = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
}


// ----------------------------------------------------------------------------------
// Two-phase schedule at d = 128 (no block mask, no split).  The hardware places waves w
// and w + 4 of a workgroup on one SIMD, and a wave does not issue past its own MFMA while
// the matrix core runs it, so only the other wave of the SIMD can fill that time.  Here
// the two waves of a SIMD are held half a tile apart, so that one runs its products while
// the other runs its softmax.
//
// Every wave runs the same sequence per tile t: the products of tile t (P V of tile
// t - 1, whose P is in s, then S of tile t into s), then the softmax of tile t.  Waves
// 0-3 (group A) and 4-7 (group B) pass the workgroup barriers at different points of it:
//   B:  products(t) | softmax(t)  |
//   A:  | products(t) | softmax(t)
// so between two barriers one group multiplies while the other exponentiates.  Barrier
// k closes phase k - 1; B runs products(t) in phase 2t and A in phase 2t + 1, so both
// read K_t and V_{t-1} in phases 2t and 2t + 1.
//
// Tile fills are spread out, one 1 KiB load at a time, so that they never stall a wave on
// the memory pipeline's issue queue.  B fetches K_{t+1} in the score half of its products
// (phase 2t, into the buffer K_{t-1} left) and waits for it before the barrier that ends
// phase 2t + 1.  A fetches V_{t+1} during its softmax of tile t (phase 2t + 2, into the
// buffer V_{t-1} left: the products of tile t read it in phases 2t and 2t + 1, so no
// earlier phase is free of readers) and waits for it a tile later.  Rows past the end of
// the sequence read as zeros.  The fills are issued as assembly (dma16), which the
// compiler does not count, so the waits are explicit.
//
// Each product's LDS operand is read RING products ahead into a register ring, so the
// product phase does not wait on LDS with no second wave to cover the wait.  LDS
// addresses are per-lane offsets held in registers plus constants; bit 15 of each offset
// selects the buffer and flips after every product phase.  A product phase runs its P V
// half only for a tile the wave's rows see (so never in the first phase, which has no P
// yet) and its score half only for such a tile (so never in the last); the offsets flip
// either way, so that each phase addresses the buffers of its tile.
//
// The sum of the 16-bit probabilities, which normalises O, is left to the matrix core:
// one 16x16x32 product per P V step against a constant operand of ones (below), instead
// of four VALU instructions per pair of scores.  (A v_dot2 per pair would wait for the
// matrix core, which the other wave of the SIMD keeps busy in this schedule: measured on
// gfx950, VALU work with one v_dot2 per pair of scores does not overlap another wave's
// MFMAs at all; without it, 70-100% of it does.)
// ----------------------------------------------------------------------------------
template <class T, bool CAUSAL, int RING>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd16_pp_kernel(
    const Fwd16Params P) {
  constexpr int D = 128, NW = 8, BR = 32 * NW, BC = 128;
  constexpr int TB = BC * D * 2;       // bytes of one K or V tile
  constexpr int KB = BC / 32;          // 32-key accumulator blocks per tile
  constexpr int DS = D / 16;           // contraction steps over the head dimension
  constexpr int DB = D / 32;           // 32-wide blocks of the output's head dimension
  constexpr int NPV = (BC / 16) * DB;  // P V products per tile
  constexpr int NSC = DS * KB;         // score products per tile
  constexpr int FPW = TB / (4 * 1024); // 1 KiB fills per wave of a group per tile
  static_assert(RING >= 1 && RING <= 7, "operand ring");
  static_assert(TB == 32768, "buffer parity is bit 15 of an LDS offset");
  static_assert(NSC == 4 * FPW, "one fill every four score products");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TB];  // K0 K1 V0 V1
  FA_LDS uint8_t* lds = (FA_LDS uint8_t*)(smem);

  const int Nq = P.Nq, Nk = P.Nk, R = P.G * P.Nq;
  const float c = P.c;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), half = lane >> 5, c32 = lane & 31;
  const int grp = wave >> 2, wg = wave & 3;
  const int nqb = (R + BR - 1) / BR;
  const int bkv = blockIdx.x % P.BHkv;
  int qb = blockIdx.x / P.BHkv;
  if (CAUSAL) qb = nqb - 1 - qb;  // longest rows first
  const int q0 = qb * BR;
  const int qw0 = q0 + 32 * wave;
  const int qrow = qw0 + c32;
  const int pos = qrow % Nq;
  const int off = Nk - Nq;
  const bool wave_rows = qw0 < R;
  int wpmin = 0, wpmax = -1;
  if (wave_rows) pos_range(qw0, min(qw0 + 31, R - 1), Nq, wpmin, wpmax);
  const int NTL = block_key_tiles<BR, BC, CAUSAL>(q0, R, Nq, Nk);
  // the wave's rows see the tiles [0, Tw)
  int Tw = wave_rows ? NTL : 0;
  if (CAUSAL && wave_rows) Tw = wpmax + off < 0 ? 0 : min(NTL, (wpmax + off) / BC + 1);

  const size_t head = (size_t)bkv * R * D;
  const size_t kvhead = (size_t)bkv * Nk * D;
  const auto rq = make_rsrc(P.Q + head, (uint32_t)R * D * 2);
  // group B fills K tiles into K buffer (t + 1) % 2, group A V tiles into V buffer (t + 1) % 2
  const uint16_t* fsrc = (grp == 1 ? P.K : P.V) + kvhead;
  const int fbuf0 = grp == 1 ? 0 : 2;

  // Per-lane LDS offsets, for the buffers of the first product phase (K_0 in buffer 0;
  // V buffer 1, which that phase does not read).  Score operand of step st (key block kb adds kb * 32 rows):
  // row c32 of the K tile, chunk 2 st + half.  P V operand of output block db (step ks
  // adds 16 rows): the two transposing reads of lds_colop, rows r and r + 8.
  int koff[DS], voff[DB][2];
#pragma unroll
  for (int st = 0; st < DS; ++st) koff[st] = tile_off<D>(c32, 2 * st + half);
  {
    const int li = lane & 15, g = lane >> 4, h = g >> 1;
    const int r = 4 * h + (li >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int col = 32 * db + 16 * (g & 1) + 4 * (li & 3);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int rr = r + 8 * e;
        voff[db][e] = 3 * TB + rr * (D * 2) + ((((col >> 3) ^ swz<D>(rr)) << 4) | ((col & 7) << 1));
      }
    }
  }
  // A group's fill of one tile: wave wg of the group moves the 1 KiB pieces f * 4 + wg
  // (f < FPW), i.e. rows 16 f + 4 wg + lane / 16, chunk lane % 16 of each; the swizzle
  // of those rows depends on the lane and wg only.  The buffer resource is moved to the
  // tile (base and size), so that rows past the end of the sequence read as zeros.
  int foff[FPW];
  {
    const int frow = 4 * wg + (lane >> 4);
#pragma unroll
    for (int f = 0; f < FPW; ++f) foff[f] = (16 * f + frow) * (D * 2) + (((lane & 15) ^ swz<D>(frow)) << 4);
  }
  auto tile_rsrc = [&](const uint16_t* base, int tile) __attribute__((always_inline)) -> u32x4 {
    const long rem = (long)Nk * (D * 2) - (long)tile * TB;  // bytes of the head from the tile on
    return rsrc_words(base + (size_t)max(tile, 0) * BC * D, rem > 0 ? (uint32_t)rem : 0u);
  };

  // prologue: K_0 (group B) and V_0 (group A), Q.  A block with
  // no key tile (only causal masking with Nq > Nk could make one; the library rejects
  // that shape) would skip the loop.
  if (NTL > 0) {
    const u32x4 rs = tile_rsrc(fsrc, 0);
#pragma unroll
    for (int f = 0; f < FPW; ++f) dma16(lds + fbuf0 * TB + (f * 4 + wg) * 1024, rs, foff[f]);
  }
  u32x4 qf[DS];
#pragma unroll
  for (int st = 0; st < DS; ++st) qf[st] = buffer_load16(rq, qrow * (D * 2) + ((2 * st + half) << 4));

  float m = -INFINITY, l = 0.f;
  f32x16 o[DB], s[KB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x16){};
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) s[kb] = (f32x16){};
  // sum of the 16-bit probabilities, on the matrix core (row_sum_operand)
  const u32x4 ones = row_sum_operand<T>(lane);
  f32x4 lsum = (f32x4){};

  // Product i < NPV is P V step i / DB of output block i % DB; product NPV + j is score
  // step j / KB of key block j % KB.
  auto operand = [&](int i) __attribute__((always_inline)) -> u32x4 {
    if (i < NPV) {
      const int ks = i / DB, db = i % DB;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(lds + voff[db][0] + ks * 16 * D * 2));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(lds + voff[db][1] + ks * 16 * D * 2));
      const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
      return (u32x4){a.x, a.y, b.x, b.y};
    }
    const int j = i - NPV;
    return *(const FA_LDS u32x4*)(lds + koff[j / KB] + (j % KB) * 32 * (D * 2));
  };
  // The products of tile t.  Each half runs only where it contributes: P V of tile t - 1
  // if the wave's rows see that tile, S of tile t if they see this one.  Each half streams
  // its own operands through the ring.  Group B fetches K_{t+1} in the S half, one 1 KiB
  // load every four products (in a row when the S half does not run).
  auto products = [&](int t) __attribute__((always_inline)) {
    const u32x4 rs = tile_rsrc(fsrc, t + 1);
    FA_LDS uint8_t* fdst = lds + (fbuf0 + ((t + 1) & 1)) * TB + wg * 1024;
    auto half_of = [&](auto first, auto count) __attribute__((always_inline)) {
      constexpr int I0 = decltype(first)::value, N = decltype(count)::value;
      u32x4 ring[RING];
#pragma unroll
      for (int i = 0; i < RING; ++i) ring[i] = operand(I0 + i);
#pragma unroll
      for (int i = I0; i < I0 + N; ++i) {
        const u32x4 a = ring[(i - I0) % RING];
        if (i + RING < I0 + N) ring[(i - I0) % RING] = operand(i + RING);
        if (i < NPV) {
          const int ks = i / DB, db = i % DB, kb = ks >> 1, mm = ks & 1;
          const u32x4 b = (u32x4){__float_as_uint(s[kb][4 * mm]), __float_as_uint(s[kb][4 * mm + 1]),
                                  __float_as_uint(s[kb][4 * mm + 2]), __float_as_uint(s[kb][4 * mm + 3])};
          o[db] = T::mfma(a, b, o[db]);
          if (db == DB - 1) lsum = T::mfma16(ones, b, lsum);
        } else {
          const int j = i - NPV, st = j / KB, kb = j % KB;
          s[kb] = T::mfma(a, qf[st], st == 0 ? (f32x16){} : s[kb]);
          if (j % 4 == 0 && grp == 1) dma16(fdst + (j / 4) * 4 * 1024, rs, foff[j / 4]);
        }
      }
      // issue order: the ring's first reads, then each product followed by the reads of
      // the product RING places later
      constexpr int FIRST = RING * (I0 < NPV ? 2 : 1);
      __builtin_amdgcn_sched_group_barrier(0x100, FIRST, 0);
#pragma unroll
      for (int i = I0; i < I0 + N; ++i) {
        if (i < NPV && i % DB == DB - 1)
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // with the sum's product
        else
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + RING < I0 + N) __builtin_amdgcn_sched_group_barrier(0x100, I0 < NPV ? 2 : 1, 0);
      }
    };
    if (t >= 1 && t - 1 < Tw) half_of(std::integral_constant<int, 0>{}, std::integral_constant<int, NPV>{});
    if (t < Tw) {
      half_of(std::integral_constant<int, NPV>{}, std::integral_constant<int, NSC>{});
    } else if (grp == 1 && t + 1 < NTL) {
#pragma unroll
      for (int f = 0; f < FPW; ++f) dma16(fdst + f * 4 * 1024, rs, foff[f]);
    }
    // the next product phase reads the other K and V buffers
#pragma unroll
    for (int st = 0; st < DS; ++st) koff[st] ^= TB;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      voff[db][0] ^= TB;
      voff[db][1] ^= TB;
    }
  };

  // Group A fetches V_{t+1} during its softmax of tile t (phase 2t + 2, when no wave reads
  // the buffer V_{t-1} left), one 1 KiB load every four pairs of exponentials.
  auto vfill = [&](int t, int f) __attribute__((always_inline)) {
    if (grp == 0 && t + 1 < NTL)
      dma16(lds + (fbuf0 + ((t + 1) & 1)) * TB + (f * 4 + wg) * 1024, tile_rsrc(fsrc, t + 1), foff[f]);
  };
  // softmax of tile t: masks, row max, lazy rescale, exponentials, sums, 16-bit P (none
  // past the wave's last visible tile)
  auto softmax_of = [&](int t) __attribute__((always_inline)) {
    if (t >= Tw) {
#pragma unroll
      for (int f = 0; f < FPW; ++f) vfill(t, f);
      return;
    }
    const int k0 = t * BC;
    if ((k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > wpmin + off)) {
      // keys past the end and (causal) after the row's position: the key's offset in the
      // tile, a constant per register, against the lane's last visible offset
      const int lim = (CAUSAL ? min(pos + off, Nk - 1) : Nk - 1) - k0 - 4 * half;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = 32 * kb + acc_row(i, 0) > lim ? -INFINITY : s[kb][i];
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) mx = max_nan(max_nan(mx, s[kb][i]), s[kb][i + 1]);
    mx = max_halves(mx) * c;
    if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m, mx);
      const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m - m_new);  // o, l are 0 while m = -inf
      l *= alpha;
      lsum *= alpha;  // the P V products of the tiles so far are all in (none is pending)
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      m = m_new;
    }
    const float mu = (m == -INFINITY) ? 0.f : m;  // every score of such a row is -inf: p = 0
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int t2 = 0; t2 < 8; ++t2) {
        const float p0 = fast_exp2(fmaf(s[kb][2 * t2], c, -mu));
        const float p1 = fast_exp2(fmaf(s[kb][2 * t2 + 1], c, -mu));
        rs += p0 + p1;
        s[kb][t2] = __uint_as_float(T::pack(p0, p1));
        if (t2 % 4 == 0) vfill(t, 2 * kb + t2 / 4);
      }
    l += rs;
  };

  // Q, K_0 (and V_0) have landed; the wait also settles the compiler's count of the Q
  // loads, so that no wait for them is left inside the loop (where it would count the
  // fills in flight too)
  wait_vmem();
  fa_sync();  // barrier 0: K_0 and V_0 are in LDS
  for (int t = 0; t <= NTL && NTL > 0; ++t) {
    if (grp == 0) fa_sync();  // A: barrier 2t + 1
    products(t);
    if (grp == 0) wait_vmem();  // A: V_t (fetched during its previous softmax) has landed
    fa_sync();                      // A: barrier 2t + 2, B: barrier 2t + 1
    softmax_of(t);
    if (grp == 1) {
      wait_vmem();      // B: K_{t+1} has landed
      fa_sync();  // B: barrier 2t + 2
    }
  }

  wait_vmem();  // no fill may outlive the workgroup's LDS
  const float lt = sum_halves(l);
  const float ltr = lsum[0];
  if (qrow >= R) return;
  const float inv = ltr > 0.f ? 1.0f / ltr : 0.f;
  uint16_t* orow = P.O + head + (size_t)qrow * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * db + 8 * g + 4 * half;
      u32x2 w;
      w.x = T::pack(o[db][4 * g] * inv, o[db][4 * g + 1] * inv);
      w.y = T::pack(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
      *(u32x2*)(orow + d) = w;
    }
  if (half == 0) P.LSE[(size_t)bkv * R + qrow] = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
}

// ----------------------------------------------------------------------------------
// Few query rows: a key/value head whose group holds at most 32 packed rows (G * Nq <=
// 32, e.g. a decode step).  The rows fill one 32-row block, so the 256-row kernel would
// run every product of a tile on one wave.  Here the keys are spread over the waves
// instead: tile t (64 keys) goes to the pair of waves 2 (t % 2), 2 (t % 2) + 1, one 32-key
// half each.  Every wave keeps its own online-softmax state (m, l, lr, o) over the keys it
// saw; at the end the four states are merged with the (m, l) rule of the tiled method
// ("FlashAttention：IO 感知…", 基准/方法设计).  Tiles stream through a ring of four
// K/V stages in LDS, so up to three tiles are in flight while one is in use: the work per
// byte is small, and the kernel lives on how many bytes it keeps in flight.
// ----------------------------------------------------------------------------------
constexpr int kFewRows = 32;
constexpr long kFewTarget = 256;  // workgroups the split count aims at: one per CU
constexpr int kFewMinTiles = 4;

template <class T, int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(256) void fwd16_few_kernel(const Fwd16Params P) {
  constexpr int NT = 256, BC = 64, ST = 4;
  constexpr int TB = BC * D * 2;                 // bytes of one K or V tile
  constexpr int LPT = 2 * (BC * D / 8) / NT;     // loads per wave per tile (K and V)
  constexpr int DS = D / 16, DB = D / 32;
  // ring stage s: K at 2s TB, V at (2s + 1) TB; then the 32 query rows
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * ST * TB + kFewRows * D * 2];
  FA_LDS uint8_t* lds = (FA_LDS uint8_t*)(smem);
  FA_LDS uint8_t* qt = lds + 2 * ST * TB;

  const int Nq = P.Nq, Nk = P.Nk, R = P.G * P.Nq;
  const float c = P.c;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), half = lane >> 5, c32 = lane & 31;
  const int bkv = blockIdx.x % P.BHkv;
  const int split = blockIdx.x / P.BHkv;
  const int qrow = c32;             // packed row of this lane (rows >= R read as zeros)
  const int pos = qrow % Nq;
  const int off = Nk - Nq;
  int pmin, pmax;
  pos_range(0, R - 1, Nq, pmin, pmax);
  const int ntiles = block_key_tiles<kFewRows, BC, CAUSAL>(0, R, Nq, Nk);
  const int j0 = SPLIT ? split * P.ct : 0;
  const int j1 = SPLIT ? min(j0 + P.ct, ntiles) : ntiles;
  if (j0 >= j1) return;  // an empty split: the merge does not read it
  const int n = j1 - j0;

  const size_t head = (size_t)bkv * R * D;
  const size_t kvhead = (size_t)bkv * Nk * D;
  const u32x4 rq = rsrc_words(P.Q + head, (uint32_t)R * D * 2);
  const u32x4 rk = rsrc_words(P.K + kvhead, (uint32_t)Nk * D * 2);
  const u32x4 rv = rsrc_words(P.V + kvhead, (uint32_t)Nk * D * 2);

  // Every global load of the kernel goes through the ring's accounting: the query rows
  // first, then up to ST - 1 tiles ahead.
  tile_load_async_asm<D, kFewRows, NT>(qt, rq, 0, tid);
  auto load = [&](int t) {  // tile t of the range into stage t % ST
    FA_LDS uint8_t* st_ = lds + (t % ST) * 2 * TB;
    tile_load_async_asm<D, BC, NT>(st_, rk, (j0 + t) * BC, tid);
    tile_load_async_asm<D, BC, NT>(st_ + TB, rv, (j0 + t) * BC, tid);
  };
#pragma unroll
  for (int t = 0; t < ST - 1; ++t)
    if (t < n) load(t);
  if (n >= ST - 1) wait_vmem_upto<(ST - 1) * LPT>();  // the query rows have landed
  else if (n == 2) wait_vmem_upto<2 * LPT>();
  else wait_vmem_upto<LPT>();
  fa_sync();
  u32x4 qf[DS];
#pragma unroll
  for (int st = 0; st < DS; ++st) qf[st] = lds_row16<D>(qt, qrow, 2 * st + half);

  const int kb = wave & 1;      // which 32-key half of a tile this wave takes
  const int parity = wave >> 1; // which tiles: t % 2 == parity
  float m = -INFINITY, l = 0.f, lr = 0.f;
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x16){};

  for (int t = 0; t < n; ++t) {
    // this wave's loads of tile t have landed once at most those of tiles t+1, t+2 remain
    if (t + 2 < n) wait_vmem_upto<2 * LPT>();
    else if (t + 1 < n) wait_vmem_upto<LPT>();
    else wait_vmem_upto<0>();
    fa_sync();  // every wave's part of tile t is in LDS; stage (t - 1) % ST is free
    if (t + ST - 1 < n) load(t + ST - 1);
    if ((t & 1) != parity) continue;
    const int k0 = (j0 + t) * BC + 32 * kb;  // this wave's 32 keys
    if (CAUSAL && k0 > pmax + off) continue;  // no row sees them
    const FA_LDS uint8_t* kt = lds + (t % ST) * 2 * TB;
    const FA_LDS uint8_t* vt = kt + TB;

    f32x16 s = (f32x16){};
#pragma unroll
    for (int st = 0; st < DS; ++st) s = T::mfma(lds_row16<D>(kt, 32 * kb + c32, 2 * st + half), qf[st], s);
    if ((k0 + 32 > Nk) || (CAUSAL && k0 + 31 > pmin + off)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + acc_row(i, half);
        s[i] = (key >= Nk || (CAUSAL && key > pos + off)) ? -INFINITY : s[i];
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; i += 2) mx = max_nan(max_nan(mx, s[i]), s[i + 1]);
    mx = max_halves(mx) * c;
    if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m, mx);
      const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m - m_new);
      l *= alpha;
      lr *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      m = m_new;
    }
    const float mu = (m == -INFINITY) ? 0.f : m;
    float rs = 0.f, rsr = 0.f;
    uint32_t pk[8];
#pragma unroll
    for (int t2 = 0; t2 < 8; ++t2) {
      const float p0 = fast_exp2(fmaf(s[2 * t2], c, -mu));
      const float p1 = fast_exp2(fmaf(s[2 * t2 + 1], c, -mu));
      rs += p0 + p1;
      pk[t2] = T::pack(p0, p1);
      rsr = T::sum2(pk[t2], rsr);
    }
    l += rs;
    lr += rsr;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4 b = (u32x4){pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]};
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = T::mfma(lds_colop<D>(vt, 32 * kb + 16 * ks, 32 * db, lane), b, o[db]);
    }
  }

  // merge the four waves' states: o [w][row][D], then m, l, lr [w][row]
  const float lt = sum_halves(l), ltr = sum_halves(lr);
  fa_sync();  // every wave is done with the ring
  float* xo = (float*)smem;
  float* xm = xo + 4 * 32 * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * db + 8 * g + 4 * half;
      *(f32x4*)(xo + (wave * 32 + c32) * D + d) = (f32x4){o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
    }
  if (half == 0) {
    xm[wave * 32 + c32] = m;
    xm[128 + wave * 32 + c32] = lt;
    xm[256 + wave * 32 + c32] = ltr;
  }
  fa_sync();
  // thread -> (row, 16 consecutive columns)
  constexpr int CPT = D * 32 / NT;
  const int r = tid / (D / CPT), d0 = (tid % (D / CPT)) * CPT;
  if (r >= R) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, xm[w * 32 + r]);  // -inf only for a row that saw no key
  float a[4], L = 0.f, LR = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float mw = xm[w * 32 + r];
    a[w] = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
    L += a[w] * xm[128 + w * 32 + r];
    LR += a[w] * xm[256 + w * 32 + r];
  }
  float acc[CPT];
#pragma unroll
  for (int e = 0; e < CPT; ++e) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) v += a[w] * xo[(w * 32 + r) * D + d0 + e];
    acc[e] = v;
  }
  if (SPLIT) {
    // partial result of this split, in the layout fwd_merge_kernel reads
    const size_t nrows = (size_t)P.BHkv * R;
    const size_t row = (size_t)split * nrows + (size_t)bkv * R + r;
    float* prow = P.part + row * D + d0;
#pragma unroll
    for (int e = 0; e < CPT; e += 4) *(f32x4*)(prow + e) = (f32x4){acc[e], acc[e + 1], acc[e + 2], acc[e + 3]};
    if (d0 == 0) {
      float* pm = P.part + (size_t)P.nsplit * nrows * D;
      pm[row] = M;
      pm[(size_t)P.nsplit * nrows + row] = L;
      pm[(size_t)2 * P.nsplit * nrows + row] = LR;
    }
    return;
  }
  const float inv = LR > 0.f ? 1.0f / LR : 0.f;
  uint16_t* orow = P.O + head + (size_t)r * D + d0;
#pragma unroll
  for (int e = 0; e < CPT; e += 8) {
    u32x4 w4;
    w4.x = T::pack(acc[e] * inv, acc[e + 1] * inv);
    w4.y = T::pack(acc[e + 2] * inv, acc[e + 3] * inv);
    w4.z = T::pack(acc[e + 4] * inv, acc[e + 5] * inv);
    w4.w = T::pack(acc[e + 6] * inv, acc[e + 7] * inv);
    *(u32x4*)(orow + e) = w4;
  }
  if (d0 == 0) P.LSE[(size_t)bkv * R + r] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}
// ----------------------------------------------------------------------------------
// fp32 inputs: the same schedule on v_mfma_f32_32x32x2_f32 (fp32 in, fp32 accumulate).
// Tiles go through registers into padded LDS rows (K stride D+2, V stride D+8 floats),
// which keeps both operand reads free of bank conflicts.
// ----------------------------------------------------------------------------------
// Split key range (SPLIT): workgroup t covers the tiles [split*ct, split*ct + ct) of its
// query block and writes the partial (unnormalised o, m, l) to `part` in the layout of the
// 16-bit kernels' partials (o [s][row][D], then m, l, l [s][row]; rows are (query head,
// position)), merged by fwd32_merge_kernel.
template <int D, int NW, int BC, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void fwd32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                        const float* __restrict__ V, float* __restrict__ O,
                                                        float* __restrict__ LSE, int BH, int G, int Nq, int Nk, float c,
                                                        int ct, int nsplit, float* __restrict__ part) {
  constexpr int BR = 32 * NW;
  constexpr int NT = NW * 64;
  constexpr int KS = D + 2, VS = D + 8;
  constexpr int KB = BC / 32;
  constexpr int DB = D / 32;
  __shared__ __attribute__((aligned(16))) float ks_[BC * KS];
  __shared__ __attribute__((aligned(16))) float vs_[BC * VS];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), half = lane >> 5, c32 = lane & 31;
  const int nqb = (Nq + BR - 1) / BR;
  const int bh = blockIdx.x % BH;
  const int t = blockIdx.x / BH;
  int qb = t % nqb;
  const int split = t / nqb;
  if (CAUSAL) qb = nqb - 1 - qb;
  const int q0 = qb * BR;
  const int qw0 = q0 + 32 * wave;
  const int qrow = qw0 + c32;
  const size_t head = (size_t)bh * Nq * D;
  const size_t kvhead = (size_t)(bh / G) * Nk * D;
  const int off = Nk - Nq;
  const auto rq = make_rsrc(Q + head, (uint32_t)Nq * D * 4);
  const auto rk = make_rsrc(K + kvhead, (uint32_t)Nk * D * 4);
  const auto rv = make_rsrc(V + kvhead, (uint32_t)Nk * D * 4);

  float qv[D / 2];  // this lane's query at d = 2*st + half
#pragma unroll
  for (int st = 0; st < D / 8; ++st) {
    // 4 consecutive floats d = 8*st' + 4*? are not what the operand needs; load the
    // pairs (2*st4 + half) for st4 in 4 steps: d = 8*st + 2*e + half, e = 0..3
    const u32x4 w0 = buffer_load16(rq, qrow * D * 4 + (8 * st) * 4);
    const u32x4 w1 = buffer_load16(rq, qrow * D * 4 + (8 * st + 4) * 4);
    const float f[8] = {__uint_as_float(w0.x), __uint_as_float(w0.y), __uint_as_float(w0.z), __uint_as_float(w0.w),
                        __uint_as_float(w1.x), __uint_as_float(w1.y), __uint_as_float(w1.z), __uint_as_float(w1.w)};
#pragma unroll
    for (int e = 0; e < 4; ++e) qv[4 * st + e] = half ? f[2 * e + 1] : f[2 * e];
  }

  const int nkt_all = (Nk + BC - 1) / BC;
  const int nkt = CAUSAL ? min(nkt_all, (q0 + BR - 1 + off) / BC + 1) : nkt_all;
  const int j0 = SPLIT ? split * ct : 0;
  const int j1 = SPLIT ? min(j0 + ct, nkt) : nkt;
  if (j0 >= j1) return;  // an empty split: the merge does not read it
  float m = -INFINITY, l = 0.f;
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x16){};

  for (int j = j0; j < j1; ++j) {
    const int k0 = j * BC;
    fa_sync();  // previous tile fully consumed
    constexpr int V4 = BC * D / 4;  // float4 chunks per tile
    for (int p = tid; p < V4; p += NT) {
      const int r = p / (D / 4), cc = (p % (D / 4)) * 4;
      const u32x4 kw = buffer_load16(rk, (k0 + r) * D * 4 + cc * 4);
      const u32x4 vw = buffer_load16(rv, (k0 + r) * D * 4 + cc * 4);
      float* kd = ks_ + r * KS + cc;
      *(f32x2*)kd = (f32x2){__uint_as_float(kw.x), __uint_as_float(kw.y)};
      *(f32x2*)(kd + 2) = (f32x2){__uint_as_float(kw.z), __uint_as_float(kw.w)};
      *(u32x4*)(vs_ + r * VS + cc) = vw;
    }
    fa_sync();
    if (CAUSAL && k0 > qw0 + 31 + off) continue;

    f32x16 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[kb] = (f32x16){};
#pragma unroll
      for (int st = 0; st < D / 2; ++st)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(ks_[(32 * kb + c32) * KS + 2 * st + half], qv[st], s[kb], 0, 0, 0);
    }
    if ((k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > qw0 + off)) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + 32 * kb + acc_row(i, half);
          if (key >= Nk || (CAUSAL && key > qrow + off)) s[kb][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = max_halves(mx);
    const float m_new = fmaxf(m, mx * c);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[kb][i] = fast_exp2(fmaf(s[kb][i], c, -m_use));
        rs += s[kb][i];
      }
    l = l * alpha + rs;
    m = m_new;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 32 * kb + acc_row(i, half);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs_[key * VS + 32 * db + c32], s[kb][i], o[db], 0, 0, 0);
      }
  }

  const float lt = sum_halves(l);
  if (SPLIT) {
    if (qrow >= Nq) return;
    const size_t nrows = (size_t)BH * Nq;
    const size_t row = (size_t)split * nrows + (size_t)bh * Nq + qrow;
    float* prow = part + row * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * half;
        *(f32x4*)(prow + d) = (f32x4){o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
      }
    if (half == 0) {
      float* pm = part + (size_t)nsplit * nrows * D;
      pm[row] = m;
      pm[(size_t)nsplit * nrows + row] = lt;
      pm[(size_t)2 * nsplit * nrows + row] = lt;  // the fp32 P V product uses the unrounded P
    }
    return;
  }
  const float inv = 1.0f / lt;
  if (qrow < Nq) {
    float* orow = O + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * half;
        *(f32x4*)(orow + d) = (f32x4){o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                                      o[db][4 * g + 3] * inv};
      }
    if (half == 0) LSE[(size_t)bh * Nq + qrow] = (m + log2f(lt)) * kLn2;
  }
}

// Merge of the fp32 kernel's split partials with the (m, l) rule of the tiled method
// ("FlashAttention：IO 感知…", 基准/方法设计): with M = max_s m_s and a_s = 2^(m_s - M),
// O = sum_s a_s o_s / sum_s a_s l_s and lse = M + log2(sum_s a_s l_s) (natural log at the
// end).  One wave per row (query head, position), D/64 elements per lane.
template <int D, int NW, int BR, int BC, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void fwd32_merge_kernel(float* __restrict__ O, float* __restrict__ LSE,
                                                              const float* __restrict__ part, int BH, int Nq, int Nk,
                                                              int ct, int nsplit) {
  const size_t nrows = (size_t)BH * Nq;
  const size_t g = (size_t)blockIdx.x * NW + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (g >= nrows) return;
  const int pos = (int)(g % Nq);
  const int q0 = (pos / BR) * BR;
  const int nkt_all = (Nk + BC - 1) / BC;
  const int ktiles = CAUSAL ? min(nkt_all, (q0 + BR - 1 + Nk - Nq) / BC + 1) : nkt_all;
  const int ns = (ktiles + ct - 1) / ct;  // splits that wrote a partial for this row
  const float* pm = part + (size_t)nsplit * nrows * D;
  const float* pl = pm + (size_t)nsplit * nrows;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, pm[s * nrows + g]);
  constexpr int E = D / 64;
  float acc[E] = {};
  float lt = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float ms = pm[s * nrows + g];
    const float a = (ms == -INFINITY) ? 0.f : fast_exp2(ms - M);
    lt += a * pl[s * nrows + g];
    const float* po = part + (s * nrows + g) * D + E * lane;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += a * po[e];
  }
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  float* orow = O + g * D + E * lane;
#pragma unroll
  for (int e = 0; e < E; ++e) orow[e] = acc[e] * inv;
  if (lane == 0) LSE[g] = lt > 0.f ? (M + log2f(lt)) * kLn2 : -INFINITY;
}

// ----------------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------------
namespace {
// Tile shapes per head dimension (waves per workgroup, keys per tile, waves per SIMD):
//   d = 128: 8 waves x 32 rows = 256 query rows against 128-key tiles; K and V double
//            buffered take 128 KiB of LDS, so one workgroup (two waves per SIMD) per CU.
//            The larger query block halves the LDS fill traffic per score.
//   d = 64:  8 waves against 64-key tiles at four waves per SIMD (128 VGPRs): the
//            softmax dominates at this head size, and more resident waves hide it.
template <int D>
struct Fwd16Shape;
template <>
struct Fwd16Shape<128> { static constexpr int NW = 8, BC = 128, WPE = 2; };
template <>
struct Fwd16Shape<64> { static constexpr int NW = 8, BC = 64, WPE = 4; };
constexpr int kNW32 = 2, kBC32 = 32;

// A group of at most kFewRows packed rows: the key-parallel kernel, split over the key
// range like the 256-row kernel and merged by the same merge kernel.
template <class T, int D, bool CAUSAL>
hipError_t go_few(const FwdArgs& a, Fwd16Params p) {
  constexpr int BC = 64;
  const int R = (a.Hq / a.Hkv) * a.Nq;
  const int tiles = block_key_tiles<kFewRows, BC, CAUSAL>(0, R, a.Nq, a.Nk);
  if (a.nsplit <= 1) {
    p.ct = tiles;
    hipLaunchKernelGGL((fwd16_few_kernel<T, D, CAUSAL, false>), dim3(p.BHkv), dim3(256), 0, a.stream, p);
    return hipGetLastError();
  }
  p.ct = (tiles + a.nsplit - 1) / a.nsplit;
  const int ns = (tiles + p.ct - 1) / p.ct;
  p.nsplit = a.nsplit;
  p.part = a.part;
  hipLaunchKernelGGL((fwd16_few_kernel<T, D, CAUSAL, true>), dim3(p.BHkv * ns), dim3(256), 0, a.stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // few rows: two columns per lane, more lanes per row
  const long nrows = (long)p.BHkv * R;
  constexpr int RPB = 256 / (D / 2);
  hipLaunchKernelGGL((fwd_merge_kernel<T, D, 2, kFewRows, BC, CAUSAL>), dim3((nrows + RPB - 1) / RPB), dim3(256), 0,
                     a.stream, p);
  return hipGetLastError();
}

template <class T, int D, bool CAUSAL, bool SPARSE>
hipError_t go16(const FwdArgs& a) {
  using S = Fwd16Shape<D>;
  constexpr int BR = 32 * S::NW;
  const int R = (a.Hq / a.Hkv) * a.Nq;
  const int nqb = (R + BR - 1) / BR;
  const int BHkv = a.B * a.Hkv;
  const int nbq = (a.Nq + kMaskBlock - 1) / kMaskBlock, nbk = (a.Nk + kMaskBlock - 1) / kMaskBlock;
  Fwd16Params p{(const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.lse,
                BHkv, a.Hq / a.Hkv, a.Nq, a.Nk, a.scale * kLog2e, 0, 1, nullptr,
                a.bmask, a.Hkv, a.mask_heads == 1 ? 0 : nbq * nbk, nbk};
  if (!SPARSE && R <= kFewRows) return go_few<T, D, CAUSAL>(a, p);
  if (a.nsplit <= 1) {
    p.ct = (a.Nk + S::BC - 1) / S::BC;
    if constexpr (D == 128 && !SPARSE) {
      hipLaunchKernelGGL((fwd16_pp_kernel<T, CAUSAL, kPpRing>), dim3(BHkv * nqb), dim3(512), 0, a.stream, p);
      return hipGetLastError();
    }
    hipLaunchKernelGGL((fwd16_kernel<T, D, S::NW, S::BC, S::WPE, CAUSAL, false, SPARSE>), dim3(BHkv * nqb),
                       dim3(S::NW * 64), 0, a.stream, p);
    return hipGetLastError();
  }
  // split the key range of the longest query block into nsplit chunks of ct tiles
  int max_tiles = 0;
  for (int qb = 0; qb < nqb; ++qb) {
    const int kt = block_key_tiles<BR, S::BC, CAUSAL>(qb * BR, R, a.Nq, a.Nk);
    max_tiles = kt > max_tiles ? kt : max_tiles;
  }
  p.ct = (max_tiles + a.nsplit - 1) / a.nsplit;
  const int ns = (max_tiles + p.ct - 1) / p.ct;
  p.nsplit = a.nsplit;
  p.part = a.part;
  hipLaunchKernelGGL((fwd16_kernel<T, D, S::NW, S::BC, S::WPE, CAUSAL, true, SPARSE>), dim3(BHkv * nqb * ns),
                     dim3(S::NW * 64), 0, a.stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long nrows = (long)BHkv * R;
  constexpr int RPB = 256 / (D / 4);
  hipLaunchKernelGGL((fwd_merge_kernel<T, D, 4, BR, S::BC, CAUSAL>), dim3((nrows + RPB - 1) / RPB), dim3(256), 0,
                     a.stream, p);
  return hipGetLastError();
}

template <class T, int D, bool CAUSAL>
hipError_t go16(const FwdArgs& a) {
  return a.bmask ? go16<T, D, CAUSAL, true>(a) : go16<T, D, CAUSAL, false>(a);
}

template <int D, bool CAUSAL>
hipError_t go32(const FwdArgs& a) {
  constexpr int BR = 32 * kNW32;
  const int nqb = (a.Nq + BR - 1) / BR;
  const int BH = a.B * a.Hq;
  const int nkt = (a.Nk + kBC32 - 1) / kBC32;
  if (a.nsplit <= 1) {
    hipLaunchKernelGGL((fwd32_kernel<D, kNW32, kBC32, CAUSAL, false>), dim3(BH * nqb), dim3(kNW32 * 64), 0, a.stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, BH,
                       a.Hq / a.Hkv, a.Nq, a.Nk, a.scale * kLog2e, nkt, 1, nullptr);
    return hipGetLastError();
  }
  // split the longest query block's key range (every block's, without causal masking)
  int max_tiles = nkt;
  if (CAUSAL) max_tiles = min(nkt, (BR * nqb - 1 + a.Nk - a.Nq) / kBC32 + 1);
  const int ct = (max_tiles + a.nsplit - 1) / a.nsplit;
  const int ns = (max_tiles + ct - 1) / ct;
  hipLaunchKernelGGL((fwd32_kernel<D, kNW32, kBC32, CAUSAL, true>), dim3(BH * nqb * ns), dim3(kNW32 * 64), 0, a.stream,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, BH, a.Hq / a.Hkv,
                     a.Nq, a.Nk, a.scale * kLog2e, ct, a.nsplit, a.part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int NWM = 4;
  const long nrows = (long)BH * a.Nq;
  hipLaunchKernelGGL((fwd32_merge_kernel<D, NWM, BR, kBC32, CAUSAL>), dim3((nrows + NWM - 1) / NWM), dim3(NWM * 64), 0,
                     a.stream, (float*)a.o, a.lse, (const float*)a.part, BH, a.Nq, a.Nk, ct, a.nsplit);
  return hipGetLastError();
}

template <int D>
hipError_t by_dtype(const FwdArgs& a) {
  switch (a.dtype) {
    case kDtypeBF16: return a.causal ? go16<bf16_t, D, true>(a) : go16<bf16_t, D, false>(a);
    case kDtypeF16: return a.causal ? go16<f16_t, D, true>(a) : go16<f16_t, D, false>(a);
    case kDtypeF32: return a.causal ? go32<D, true>(a) : go32<D, false>(a);
  }
  return hipErrorInvalidValue;
}
}  // namespace

namespace {
template <int D, bool CAUSAL>
int max_block_tiles(int R, int Nq, int Nk) {
  using S = Fwd16Shape<D>;
  constexpr int BR = 32 * S::NW;
  const int nqb = (R + BR - 1) / BR;
  int mt = 0;
  for (int qb = 0; qb < nqb; ++qb) {
    const int kt = block_key_tiles<BR, S::BC, CAUSAL>(qb * BR, R, Nq, Nk);
    mt = kt > mt ? kt : mt;
  }
  return mt;
}
}  // namespace

int fwd_suggest_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d, bool causal, int dtype) {
  if (dtype == kDtypeF32) {
    // fp32 kernel: 64-row blocks per query head, 32-key tiles; aim at about 256
    // workgroups (one per CU), down to one tile per split
    constexpr int BR = 32 * kNW32;
    const long wg = (long)B * Hq * ((Nq + BR - 1) / BR);
    const int nkt = (Nk + kBC32 - 1) / kBC32;
    const int mt = causal ? std::min(nkt, (int)((BR * ((Nq + BR - 1) / BR) - 1 + Nk - Nq) / kBC32 + 1)) : nkt;
    long want = (256 + wg - 1) / wg;
    if (want > mt) want = mt;
    if (want > 64) want = 64;
    if (want < 2) return 1;
    const int ct = (int)((mt + want - 1) / want);
    return (mt + ct - 1) / ct;
  }
  if ((long)(Hq / Hkv) * Nq <= kFewRows) {
    // key-parallel kernel: one workgroup per CU (128 KiB of LDS at d = 128), at least
    // kFewMinTiles 64-key tiles per split so that the ring's fill and drain stay small
    const int R = (Hq / Hkv) * Nq;
    const int tiles = causal ? block_key_tiles<kFewRows, 64, true>(0, R, Nq, Nk)
                             : block_key_tiles<kFewRows, 64, false>(0, R, Nq, Nk);
    const long wg = (long)B * Hkv;
    long want = (kFewTarget + wg - 1) / wg;
    if (want > tiles / kFewMinTiles) want = tiles / kFewMinTiles;
    if (want > 64) want = 64;
    if (want < 2) return 1;
    const int ct = (int)((tiles + want - 1) / want);
    return (tiles + ct - 1) / ct;
  }
  const int NW = d == 64 ? Fwd16Shape<64>::NW : Fwd16Shape<128>::NW;
  const int BR = 32 * NW;
  const long R = (long)(Hq / Hkv) * Nq;
  const long wg = (long)B * Hkv * ((R + BR - 1) / BR);
  constexpr long kTarget = 512;  // two workgroups for each of the 256 CUs
  if (wg >= kTarget) return 1;
  const int mt = d == 64 ? (causal ? max_block_tiles<64, true>((int)R, Nq, Nk) : max_block_tiles<64, false>((int)R, Nq, Nk))
                         : (causal ? max_block_tiles<128, true>((int)R, Nq, Nk)
                                   : max_block_tiles<128, false>((int)R, Nq, Nk));
  if (causal) {
    // Causal query blocks need fewer key tiles than the longest one, so a split count
    // yields fewer than wg * nsplit working workgroups (splits past a block's last tile
    // exit at once).  Take the most splits whose working workgroups stay within 9/10 of
    // the target: each split adds merge work, and near the full target it costs more
    // than the shorter chunks save (causal 8 x 4096 x 64 prefill: 4 splits 57.5 us with
    // 320 working workgroups, 5: 54.2 with 392, 6: 53.2 with 456, 7: 56.1 with 488,
    // 8: 59.0 with 576).
    const int nqb = (int)((R + BR - 1) / BR);
    auto working = [&](int ct) {
      long n = 0;
      for (int qb = 0; qb < nqb; ++qb) {
        const int kt = d == 64 ? block_key_tiles<32 * Fwd16Shape<64>::NW, Fwd16Shape<64>::BC, true>(qb * BR, (int)R, Nq, Nk)
                               : block_key_tiles<32 * Fwd16Shape<128>::NW, Fwd16Shape<128>::BC, true>(qb * BR, (int)R, Nq, Nk);
        n += (kt + ct - 1) / ct;
      }
      return n * B * Hkv;
    };
    int best = 1;
    for (int ns = 2; ns <= mt && ns <= 64; ++ns) {
      const int ct = (mt + ns - 1) / ns;
      if ((mt + ct - 1) / ct != ns) continue;  // the same chunks as a smaller count
      if (working(ct) > kTarget * 9 / 10) break;
      best = ns;
    }
    return best;
  }
  long want = (kTarget + wg - 1) / wg;
  if (want > mt) want = mt;
  if (want > 64) want = 64;
  if (want < 2) return 1;
  const int ct = (int)((mt + want - 1) / want);
  return (mt + ct - 1) / ct;
}

hipError_t launch_forward(const FwdArgs& a) {
  return a.d == 64 ? by_dtype<64>(a) : by_dtype<128>(a);
}

}  // namespace fa
