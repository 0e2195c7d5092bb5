// Exact attention backward on gfx950, recomputing the score tiles instead of storing P.
//
// Method ("Flash Attention", mlx.void.app, FlashAttention section on training: only O and
// the per-row statistics are kept and the score tiles are rebuilt from Q and K on chip;
// "FlashAttention：IO 感知的快速内存高效精确注意力", trdm.cn, 方法细节: backward
// recomputation as selective checkpointing).  With the saved logsumexp lse the
// probabilities come back in one step, P = exp(scale*QK^T - lse), with no running max.
// The gradient formulas are the calculus of O = softmax(S) V (the pages give none):
//   dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,  dS = P * (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q.
//
// Accuracy choices (the gradients must hold an absolute error bar at magnitudes ~30):
//   * D_i is summed from the recomputed fp32 P and dP, not as dO_i . O_i from the stored
//     16-bit O, whose rounding (and the forward's 16-bit P) would otherwise reach the
//     gradients amplified by sum_j P_ij K_j.
//   * P and dS enter the dV, dK and dQ products as a 16-bit pair hi + lo (split2), two
//     MFMAs against the exactly representable Q, K or dO operand.
//
// Two kernels on the caller's stream, deterministic (no atomics):
//   1. dq:    one workgroup per (batch, head, block of 32*NW queries), Q and dO in
//             registers, K and V tiles streamed through LDS twice.  Pass 1: S^T = K Q^T,
//             dP^T = V dO^T, D_i = sum_j P_ij dP_ij.  Pass 2: the same tiles again,
//             dS^T = P^T (dP^T - D), dQ^T += K^T dS^T (K^T by ds_read_b64_tr_b16).
//             Writes D and lse*log2(e) to the workspace for kernel 2.
//   2. dkdv:  one workgroup per (batch, head, block of 32*NP keys), Q and dO tiles (and
//             their D, lse) streamed through LDS.  Per 32 keys a pair of waves: one
//             holds K, computes S = Q K^T, P and dV^T += dO^T P; the other holds V,
//             computes dP = dO V^T, dS and dK^T += Q^T dS (dO^T / Q^T from transposing
//             LDS reads), with P handed over through LDS.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {


// Block-sparse mask as the kernels see it: (mask heads, ceil(Nq/128), ceil(Nk/128)) bytes,
// 0 = hidden 128 x 128 block; query head h (index within the batch) reads layer
// h * hstride (0: one layer shared by every head).
struct BwdMask {
  const uint8_t* bytes;
  int Hq, hstride, nbk;
};
constexpr int kMaskBlock = 128;

// ----------------------------------------------------------------------------------
// 1. dQ (and D, lse2).  NW waves x 32 queries per workgroup; BC keys per tile.
// ----------------------------------------------------------------------------------
template <class T, int D, int NW, int BC, int WPE, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, float* __restrict__ delta,
    float* __restrict__ lse2, float* __restrict__ dQ, int BH, int G, int Nq, int Nk, float c, float scale,
    const BwdMask mask) {
  constexpr int BR = 32 * NW;
  constexpr int NT = NW * 64;
  constexpr int TB = BC * D * 2;
  constexpr int KB = BC / 32;
  constexpr int DS = D / 16;
  constexpr int DB = D / 32;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TB];  // K0 K1 V0 V1
  FA_LDS uint8_t* lds = (FA_LDS uint8_t*)(smem);

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), half = lane >> 5, c32 = lane & 31;
  const int nqb = (Nq + BR - 1) / BR;
  const int bh = blockIdx.x % BH;  // query head; it reads key/value head bh / G
  int qb = blockIdx.x / BH;
  if (CAUSAL) qb = nqb - 1 - qb;  // longest rows first
  const int q0 = qb * BR;
  const int qw0 = q0 + 32 * wave;
  const int qrow = qw0 + c32;

  const size_t head = (size_t)bh * Nq * D;
  const size_t kvhead = (size_t)(bh / G) * Nk * D;
  const int off = Nk - Nq;  // causal: query row i sees keys j <= i + off
  const auto rq = make_rsrc(Q + head, (uint32_t)Nq * D * 2);
  const auto rk = make_rsrc(K + kvhead, (uint32_t)Nk * D * 2);
  const auto rv = make_rsrc(V + kvhead, (uint32_t)Nk * D * 2);
  const auto rdo = make_rsrc(dO + head, (uint32_t)Nq * D * 2);

  const int nkt_all = (Nk + BC - 1) / BC;
  const int nkt = CAUSAL ? min(nkt_all, (q0 + BR - 1 + off) / BC + 1) : nkt_all;

  u32x4 qf[DS], of[DS];
#pragma unroll
  for (int st = 0; st < DS; ++st) {
    qf[st] = buffer_load16(rq, qrow * (D * 2) + ((2 * st + half) << 4));
    of[st] = buffer_load16(rdo, qrow * (D * 2) + ((2 * st + half) << 4));
  }
  const bool qvalid = qrow < Nq;
  const float l2 = qvalid ? LSE[(size_t)bh * Nq + qrow] * kLog2e : 0.f;

  float dsum = 0.f;  // pass 1: this half's part of D_i = sum_j P_ij dP_ij
  float dl = 0.f;    // pass 2: D_i
  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = (f32x16){};

  // block-sparse: the workgroup's rows form one 128-row mask block; key tiles in hidden
  // blocks are neither loaded nor computed
  static_assert(!SPARSE || (kMaskBlock % BR == 0 && kMaskBlock % BC == 0), "tiles inside mask blocks");
  const uint8_t* mrow = SPARSE ? mask.bytes + (size_t)(bh % mask.Hq) * mask.hstride +
                                     (size_t)(q0 / kMaskBlock) * mask.nbk
                               : nullptr;
  auto next_tile = [&](int j) {  // searched 64 tiles at a time, one tile per lane
    if (SPARSE) {
      for (; j < nkt; j += 64) {
        const int jl = j + lane;
        const uint64_t need = __builtin_amdgcn_ballot_w64(jl < nkt && mrow[(jl * BC) / kMaskBlock] != 0);
        if (need != 0) return j + (int)__builtin_ctzll(need);
      }
      return nkt;
    }
    return j;
  };

  // the two passes as separate code (pass 0 sums D, pass 1 accumulates dQ), and the
  // per-score step of each in a masked and an unmasked version behind a wave-uniform
  // branch, so that no score pays for the other pass or for the mask test
  auto run_pass = [&](auto pass_tag) {
    constexpr int pass = decltype(pass_tag)::value;
    fa_sync();  // the previous pass is done with both LDS buffers
    int j = next_tile(0);
    if (j < nkt) {
      tile_load_async<D, BC, NT>(lds, rk, j * BC, tid);
      tile_load_async<D, BC, NT>(lds + 2 * TB, rv, j * BC, tid);
    }
    for (int cur = 0; j < nkt; cur ^= 1) {
      wait_vmem();
      fa_sync();
      const int jn = next_tile(j + 1);
      if (jn < nkt) {
        tile_load_async<D, BC, NT>(lds + (cur ^ 1) * TB, rk, jn * BC, tid);
        tile_load_async<D, BC, NT>(lds + (2 + (cur ^ 1)) * TB, rv, jn * BC, tid);
      }
      const int k0 = j * BC;
      j = jn;
      if (CAUSAL && k0 > qw0 + 31 + off) continue;
      const FA_LDS uint8_t* kt = lds + cur * TB;
      const FA_LDS uint8_t* vt = lds + (2 + cur) * TB;
      const bool need_mask = (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > qw0 + off);

      uint32_t sh[KB][8], sl[KB][8];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        f32x16 s = (f32x16){}, dp = (f32x16){};
#pragma unroll
        for (int st = 0; st < DS; ++st) {
          s = T::mfma(lds_row16<D>(kt, 32 * kb + c32, 2 * st + half), qf[st], s);
          dp = T::mfma(lds_row16<D>(vt, 32 * kb + c32, 2 * st + half), of[st], dp);
        }
        auto scores = [&](auto masked) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float p = fast_exp2(fmaf(s[i], c, -l2));
            if constexpr (decltype(masked)::value) {
              const int key = k0 + 32 * kb + acc_row(i, half);
              if (key >= Nk || (CAUSAL && key > qrow + off)) p = 0.f;
            }
            if constexpr (pass == 0) dsum = fmaf(p, dp[i], dsum);
            else dp[i] = p * (dp[i] - dl);
          }
        };
        if (need_mask) scores(std::true_type{});
        else scores(std::false_type{});
        if constexpr (pass == 1) {
#pragma unroll
          for (int t = 0; t < 8; ++t) split2<T>(dp[2 * t], dp[2 * t + 1], sh[kb][t], sl[kb][t]);
        }
      }
      if constexpr (pass == 1) {
        // dQ^T += K^T (dS^T hi) + K^T (dS^T lo)
#pragma unroll
        for (int ks = 0; ks < BC / 16; ++ks) {
          const int kb = ks >> 1, mm = ks & 1;
          const u32x4 bh_ = (u32x4){sh[kb][4 * mm], sh[kb][4 * mm + 1], sh[kb][4 * mm + 2], sh[kb][4 * mm + 3]};
          const u32x4 bl_ = (u32x4){sl[kb][4 * mm], sl[kb][4 * mm + 1], sl[kb][4 * mm + 2], sl[kb][4 * mm + 3]};
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const u32x4 a = lds_colop<D>(kt, 16 * ks, 32 * db, lane);
            dq[db] = T::mfma(a, bh_, dq[db]);
            dq[db] = T::mfma(a, bl_, dq[db]);
          }
        }
      }
    }
    if constexpr (pass == 0) {
      dl = sum_halves(dsum);
      if (qvalid && half == 0) {
        delta[(size_t)bh * Nq + qrow] = dl;
        lse2[(size_t)bh * Nq + qrow] = l2;
      }
    }
  };
  run_pass(std::integral_constant<int, 0>{});
  run_pass(std::integral_constant<int, 1>{});

  if (qvalid) {
    float* dqr = dQ + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * half;
        *(f32x4*)(dqr + d) = (f32x4){dq[db][4 * g] * scale, dq[db][4 * g + 1] * scale, dq[db][4 * g + 2] * scale,
                                     dq[db][4 * g + 3] * scale};
      }
  }
}

// ----------------------------------------------------------------------------------
// 2. dK, dV.  NP wave pairs per workgroup, 32 keys per pair; BQ queries per streamed tile.
//
// The two waves of a pair share their 32 keys and split the work by operand:
//   wave A (rows 0..NP-1):  K in registers.  S = Q K^T, P = exp2(S c - lse2), P to LDS,
//                           dV^T += dO^T (P hi + P lo).
//   wave B (rows NP..2NP-1): V in registers.  dP = dO V^T, P from LDS,
//                           dS = P (dP - D), dK^T += Q^T (dS hi + dS lo).
// Each wave holds one operand block and one accumulator (about 170 VGPRs instead of the
// 270 one wave doing all of it needs), so two waves fit per SIMD.  Waves w and w + NP
// land on the same SIMD: while one runs its softmax arithmetic on the VALU the other's
// products run on the matrix core.  Per tile: barrier (Q, dO, statistics in LDS), A
// computes and publishes P while B computes dP, barrier, both finish their products.
// ----------------------------------------------------------------------------------
template <class T, int D, int NP, int BQ, int WPE, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(2 * NP * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ delta, const float* __restrict__ lse2,
    float* __restrict__ dK, float* __restrict__ dV, int BHkv, int G, int Nq, int Nk, float c, float scale,
    const BwdMask mask) {
  constexpr int NW = 2 * NP;
  constexpr int BKV = 32 * NP;
  constexpr int NT = NW * 64;
  constexpr int TB = BQ * D * 2;
  constexpr int QB = BQ / 32;  // 32-query accumulator blocks per tile
  constexpr int DS = D / 16;
  constexpr int DB = D / 32;
  constexpr int PB = QB * 16 * 64 * 4;  // bytes of one pair's P tile (QB accumulators, 64 lanes)
  static_assert(BQ % 32 == 0 && BQ <= 64, "query tile");
  // Q0 Q1 dO0 dO1 | stats [buffer][lse2 | delta][64 floats] (a dword DMA instruction writes
  // all 64 lanes, so each array gets a full 64-float slot) | P exchange [pair]
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TB + 2 * 2 * 64 * 4 + NP * PB];
  FA_LDS uint8_t* lds = (FA_LDS uint8_t*)(smem);
  FA_LDS float* stats = (FA_LDS float*)(smem + 4 * TB);

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), half = lane >> 5, c32 = lane & 31;
  const bool role_b = wave >= NP;
  const int pair = role_b ? wave - NP : wave;
  FA_LDS f32x4* pex = (FA_LDS f32x4*)(smem + 4 * TB + 2 * 2 * 64 * 4 + pair * PB);
  const int bkv = blockIdx.x % BHkv;  // key/value head; its query heads are bkv*G .. bkv*G + G-1
  const int kblk = blockIdx.x / BHkv;  // causal: block 0 sees the most queries and starts first
  const int k0 = kblk * BKV;
  const int kw0 = k0 + 32 * pair;
  const int krow = kw0 + c32;

  const size_t kvhead = (size_t)bkv * Nk * D;
  const int off = Nk - Nq;  // causal: query row i sees keys j <= i + off

  const int nqt = (Nq + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? max(k0 - off, 0) / BQ : 0;  // earlier query tiles see none of these keys
  const int nt = nqt - qt0;                             // query tiles per query head of the group
  const int ntiles = G * nt;

  // streamed tile t: query tile qt0 + t % nt of query head bkv*G + t / nt
  auto load_tile = [&](int t, int buf) {
    const int bhq = bkv * G + t / nt;
    const int qt = qt0 + t % nt;
    const size_t qhead = (size_t)bhq * Nq * D;
    tile_load_async<D, BQ, NT>(lds + buf * TB, make_rsrc(Q + qhead, (uint32_t)Nq * D * 2), qt * BQ, tid);
    tile_load_async<D, BQ, NT>(lds + (2 + buf) * TB, make_rsrc(dO + qhead, (uint32_t)Nq * D * 2), qt * BQ, tid);
    if (wave == 0) {
      // 64 floats of lse2 and of delta from the tile's first query (the first BQ used)
      const auto rl = make_rsrc(lse2 + (size_t)bhq * Nq, (uint32_t)Nq * 4);
      const auto rd = make_rsrc(delta + (size_t)bhq * Nq, (uint32_t)Nq * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (FA_LDS void*)(stats + buf * 128), 4, (qt * BQ + lane) * 4, 0,
                                               0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (FA_LDS void*)(stats + buf * 128 + 64), 4,
                                               (qt * BQ + lane) * 4, 0, 0, 0);
      race_check_fill_wait();
    }
  };

  // block-sparse: the workgroup's keys form one 128-key mask block, each query tile lies in
  // one 128-row block: hidden tiles are neither loaded nor computed
  static_assert(!SPARSE || (BKV == kMaskBlock && kMaskBlock % BQ == 0), "tiles inside mask blocks");
  auto next_tile = [&](int t) {  // searched 64 tiles at a time, one tile per lane
    if (SPARSE) {
      const int hbase = (bkv % (mask.Hq / G)) * G;  // the group's first query head within the batch
      for (; t < ntiles; t += 64) {
        const int tl = t + lane;
        bool need = false;
        if (tl < ntiles) {
          const int hq = hbase + tl / nt;
          const int qblk = ((qt0 + tl % nt) * BQ) / kMaskBlock;
          need = mask.bytes[(size_t)hq * mask.hstride + (size_t)qblk * mask.nbk + k0 / kMaskBlock] != 0;
        }
        const uint64_t b = __builtin_amdgcn_ballot_w64(need);
        if (b != 0) return t + (int)__builtin_ctzll(b);
      }
      return ntiles;
    }
    return t;
  };
  int t = next_tile(0);
  if (t < ntiles) load_tile(t, 0);

  // this wave's keys (A) or values (B) as B operands (lane = key, 8 consecutive d per lane)
  u32x4 kv[DS];
  {
    const auto rkv = make_rsrc((role_b ? V : K) + kvhead, (uint32_t)Nk * D * 2);
#pragma unroll
    for (int st = 0; st < DS; ++st) kv[st] = buffer_load16(rkv, krow * (D * 2) + ((2 * st + half) << 4));
  }

  f32x16 acc[DB];  // dV^T (A) or dK^T (B): lane = key, registers = head-dimension rows
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = (f32x16){};

  for (int cur = 0; t < ntiles; cur ^= 1) {
    wait_vmem();
    fa_sync();
    const int tn = next_tile(t + 1);
    if (tn < ntiles) load_tile(tn, cur ^ 1);
    const int q0 = (qt0 + t % nt) * BQ;
    t = tn;
    // every query of the tile precedes this pair's keys: P = 0 (both waves of the pair
    // agree, and both still meet the barrier below)
    const bool active = !(CAUSAL && q0 + BQ - 1 + off < kw0);
    const FA_LDS uint8_t* qtile = lds + cur * TB;
    const FA_LDS uint8_t* otile = lds + (2 + cur) * TB;
    const FA_LDS float* l2 = stats + cur * 128;
    const FA_LDS float* dl = l2 + 64;
    const bool need_mask = (q0 + BQ > Nq) || (CAUSAL && q0 + off < kw0 + 31);

    // phase 1: A computes P and publishes it, B computes dP
    f32x16 x[QB];  // A: P, B: dP (rows = queries q0 + 32*qb + acc_row(i, half))
    if (active) {
      // d = 128: A reads its 32 statistics before the score products, so that their LDS
      // latency hides under the products, and stores P only after the last read (the
      // compiler cannot tell the two LDS regions apart: a store between two reads would
      // serialise each read behind the previous store).  At d = 64 (four waves per
      // SIMD, 128 VGPRs) the 32 registers this holds would spill, so there the reads
      // stay next to their use.
      f32x4 lvh[QB][4];
      if constexpr (D == 128) {
        if (!role_b) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int a = 0; a < 4; ++a) lvh[qb][a] = *(const FA_LDS f32x4*)(l2 + 32 * qb + 8 * a + 4 * half);
        }
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        x[qb] = (f32x16){};
#pragma unroll
        for (int st = 0; st < DS; ++st)
          x[qb] = T::mfma(lds_row16<D>(role_b ? otile : qtile, 32 * qb + c32, 2 * st + half), kv[st], x[qb]);
      }
      // P = exp2(S c - lse2), in two versions behind a wave-uniform branch so that tiles
      // off the diagonal and the ragged end skip the per-score mask arithmetic
      auto probabilities = [&](auto masked) {
        auto prob = [&](int qb, int a, const f32x4& lv) {
          const int r0 = 32 * qb + 8 * a + 4 * half;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * a + e;
            float p = fast_exp2(fmaf(x[qb][i], c, -lv[e]));
            if constexpr (decltype(masked)::value) {
              const int q = q0 + r0 + e;
              if (q >= Nq || (CAUSAL && krow > q + off)) p = 0.f;
            }
            x[qb][i] = p;
          }
        };
        auto publish = [&](int qb, int a) {
          pex[(qb * 4 + a) * 64 + lane] = (f32x4){x[qb][4 * a], x[qb][4 * a + 1], x[qb][4 * a + 2], x[qb][4 * a + 3]};
        };
        if constexpr (D == 128) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int a = 0; a < 4; ++a) prob(qb, a, lvh[qb][a]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int a = 0; a < 4; ++a) publish(qb, a);
        } else {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
            for (int a = 0; a < 4; ++a) {
              const int r0 = 32 * qb + 8 * a + 4 * half;
              const f32x4 lv = *(const FA_LDS f32x4*)(l2 + r0);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int i = 4 * a + e;
                float p = fast_exp2(fmaf(x[qb][i], c, -lv[e]));
                if constexpr (decltype(masked)::value) {
                  const int q = q0 + r0 + e;
                  if (q >= Nq || (CAUSAL && krow > q + off)) p = 0.f;
                }
                x[qb][i] = p;
              }
              pex[(qb * 4 + a) * 64 + lane] =
                  (f32x4){x[qb][4 * a], x[qb][4 * a + 1], x[qb][4 * a + 2], x[qb][4 * a + 3]};
            }
          }
        }
      };
      if (!role_b) {
        if (need_mask) probabilities(std::true_type{});
        else probabilities(std::false_type{});
      }
    }
    fa_sync();
    if (!active) continue;

    // phase 2: A: dV^T += dO^T (P hi + P lo);  B: dS = P (dP - D), dK^T += Q^T (dS hi + dS lo)
    const FA_LDS uint8_t* atile = role_b ? qtile : otile;  // Q^T for dK, dO^T for dV
    auto split_block = [&](int qb, uint32_t* hi, uint32_t* lo) {
      if (role_b) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int r0 = 32 * qb + 8 * a + 4 * half;
          const f32x4 dlv = *(const FA_LDS f32x4*)(dl + r0);
          const f32x4 pv = pex[(qb * 4 + a) * 64 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) x[qb][4 * a + e] = pv[e] * (x[qb][4 * a + e] - dlv[e]);
        }
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) split2<T>(x[qb][2 * t], x[qb][2 * t + 1], hi[t], lo[t]);
    };
    auto products = [&](int qb, const uint32_t* hi, const uint32_t* lo) {
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const u32x4 bh_ = (u32x4){hi[4 * mm], hi[4 * mm + 1], hi[4 * mm + 2], hi[4 * mm + 3]};
        const u32x4 bl_ = (u32x4){lo[4 * mm], lo[4 * mm + 1], lo[4 * mm + 2], lo[4 * mm + 3]};
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x4 a = lds_colop<D>(atile, 32 * qb + 16 * mm, 32 * db, lane);
          acc[db] = T::mfma(a, bh_, acc[db]);
          acc[db] = T::mfma(a, bl_, acc[db]);
        }
      }
    };
    if constexpr (D == 128) {
      // every block's split first, then all products: the compiler interleaves the
      // products with the transposing reads best this way (3% faster than block by block)
      uint32_t hi[QB][8], lo[QB][8];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) split_block(qb, hi[qb], lo[qb]);
#pragma unroll
      for (int ks = 0; ks < BQ / 16; ++ks) {
        const int qb = ks >> 1, mm = ks & 1;
        const u32x4 bh_ = (u32x4){hi[qb][4 * mm], hi[qb][4 * mm + 1], hi[qb][4 * mm + 2], hi[qb][4 * mm + 3]};
        const u32x4 bl_ = (u32x4){lo[qb][4 * mm], lo[qb][4 * mm + 1], lo[qb][4 * mm + 2], lo[qb][4 * mm + 3]};
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x4 a = lds_colop<D>(atile, 16 * ks, 32 * db, lane);
          acc[db] = T::mfma(a, bh_, acc[db]);
          acc[db] = T::mfma(a, bl_, acc[db]);
        }
      }
    } else {
      // block by block, so that only one block's pairs are live: at 128 VGPRs this
      // halves the spilled registers and runs 4.5% faster
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        uint32_t hi[8], lo[8];
        split_block(qb, hi, lo);
        products(qb, hi, lo);
      }
    }
  }

  // lane = key (column of dK^T / dV^T), registers = head-dimension rows
  if (krow < Nk) {
    float* out = (role_b ? dK : dV) + kvhead + (size_t)krow * D;
    const float f = role_b ? scale : 1.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * half;
        *(f32x4*)(out + d) = (f32x4){acc[db][4 * g] * f, acc[db][4 * g + 1] * f, acc[db][4 * g + 2] * f,
                                     acc[db][4 * g + 3] * f};
      }
  }
}

// ----------------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------------
namespace {
constexpr int kNPkv = 4;
constexpr int kNWq = 4, kBCq = 32;
// dQ at d = 128 without a block mask: 8 waves (256 queries) per workgroup against 64-key
// tiles, so that each K/V tile filled into LDS serves twice the queries and each barrier
// twice the products (large-head causal workload: 1.417 -> 1.377 ms against 4 x 32 rows
// with 32-key tiles; 8 x 32-key: 1.390, 4 x 64-key: 1.407).  A block mask needs the
// workgroup's rows inside one 128-row mask block, so masked launches keep 4 waves.
constexpr int kNWqWide = 8, kBCqWide = 64;

// 64 queries per streamed Q/dO tile: two accumulator blocks per wave between barriers
constexpr int kBQkv = 64;

// Waves per SIMD of the dQ and dK/dV kernels, per head dimension.  At d = 64 the
// per-score VALU work weighs twice as much against the products as at d = 128, and the
// kernels fit in fewer registers: three dQ waves (168 VGPRs) and four dK/dV waves (128
// VGPRs, two workgroups per CU) hide it better than two (GPT-2-medium shape, causal
// N = 1024: dQ 174 -> 148 us, dK/dV 211 -> 164 us).
template <int D>
struct BwdOcc;
template <>
struct BwdOcc<128> { static constexpr int Q = 2, KV = 2; };
template <>
struct BwdOcc<64> { static constexpr int Q = 3, KV = 4; };

template <class T, int D, bool CAUSAL, bool SPARSE>
hipError_t go(const BwdArgs& a, int stages) {
  const int nbq = (a.Nq + kMaskBlock - 1) / kMaskBlock, nbk = (a.Nk + kMaskBlock - 1) / kMaskBlock;
  const BwdMask mask{a.bmask, a.Hq, a.mask_heads == 1 ? 0 : nbq * nbk, nbk};
  const int BHq = a.B * a.Hq;
  const int BHkv = a.B * a.Hkv;
  const int G = a.Hq / a.Hkv;
  const long rows = (long)BHq * a.Nq;
  float* delta = a.delta;
  float* lse2 = a.delta + rows;
  const float c = a.scale * kLog2e;
  if (stages & kStageDq) {
    constexpr bool wide = D == 128 && !SPARSE;
    constexpr int NWq = wide ? kNWqWide : kNWq;
    constexpr int BCq = wide ? kBCqWide : kBCq;
    constexpr int BR = 32 * NWq;
    const int nqb = (a.Nq + BR - 1) / BR;
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, NWq, BCq, BwdOcc<D>::Q, CAUSAL, SPARSE>), dim3(BHq * nqb), dim3(NWq * 64), 0,
                       a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dO, a.lse, delta, lse2, a.dq, BHq, G, a.Nq, a.Nk, c, a.scale, mask);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & kStageDkdv) {
    constexpr int BKV = 32 * kNPkv;
    const int nkb = (a.Nk + BKV - 1) / BKV;
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, kNPkv, kBQkv, BwdOcc<D>::KV, CAUSAL, SPARSE>), dim3(BHkv * nkb),
                       dim3(2 * kNPkv * 64), 0, a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (const uint16_t*)a.dO, delta, lse2, a.dk, a.dv, BHkv, G, a.Nq, a.Nk, c,
                       a.scale, mask);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <class T, int D, bool CAUSAL>
hipError_t go(const BwdArgs& a, int stages) {
  return a.bmask ? go<T, D, CAUSAL, true>(a, stages) : go<T, D, CAUSAL, false>(a, stages);
}

template <int D>
hipError_t by_dtype(const BwdArgs& a, int stages) {
  switch (a.dtype) {
    case kDtypeBF16: return a.causal ? go<bf16_t, D, true>(a, stages) : go<bf16_t, D, false>(a, stages);
    case kDtypeF16: return a.causal ? go<f16_t, D, true>(a, stages) : go<f16_t, D, false>(a, stages);
  }
  return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_backward(const BwdArgs& a, int stages) {
  return a.d == 64 ? by_dtype<64>(a, stages) : by_dtype<128>(a, stages);
}

}  // namespace fa
