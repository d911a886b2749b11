// PSA self-attention kernels for gfx950 (CDNA4).
//
// The method (PsaFa2Backward page, vision_rs psa kernels, struct
// description): Flash-Attention-2 over the N = H*W tokens of one (batch,
// head) slice, where queries and keys are the same N tokens and every query
// sees every key.  The page's own schedule (one CTA per query row, dq/dk
// summed with float atomics) is not used here.  Instead:
//
//   psa_fwd_kernel   one workgroup per (slice, tile of BM queries); each wave
//                    keeps QW queries stationary in registers and streams key
//                    tiles through LDS: S^T = K Q^T, online softmax in log2
//                    units (rescale only when the running max grows by more
//                    than 2^8), O^T += V^T P^T and the row sums l += 1 P^T,
//                    all on MFMA.  Writes O and LSE.
//   psa_bwd_pre      D_i = sum_c dO_ic O_ic and LSE in log2 units.
//   bwd_dkdv_body    one workgroup per (slice, tile of keys); keys stationary,
//                    query tiles streamed: S = Q K^T, dP = dO V^T,
//                    P = exp(S - LSE), dS = P (dP - D), dV^T += dO^T P,
//                    dK^T += Q^T dS.
//   bwd_dq_body      one workgroup per (slice, tile of queries); queries
//                    stationary, key tiles streamed: S^T, dP^T, dS^T as
//                    above, dQ^T += K^T dS^T.
//   psa_bwd_fused_kernel runs both bodies in one grid (dK/dV workgroups
//                    first).
// Every output element is written exactly once by one lane (with the
// V-slice calls' accumulate flag: read, added to and written once): no
// atomics, no zero-initialisation, bitwise reproducible.
//
// Orientation: outputs are accumulated transposed (channels as MFMA rows,
// tokens as MFMA columns) so that accumulator lanes run along tokens and
// stores into the channel-major tensors are coalesced.  Scores are S^T where
// the next GEMM contracts over keys (fwd, dQ) and S where it contracts over
// queries (dK/dV); their rows are permuted within each 32-token chunk (see
// psa_common.h) so that P and dS become the next MFMA operand in place.
#pragma once
#include <type_traits>

#include "psa_common.h"

namespace psa {

constexpr float kRescaleSlack = 8.f;  // log2 units: P may reach 2^8 before a rescale

template <int D> struct Chunks {
  static constexpr int n = (D + 31) / 32;  // 32-wide contraction chunks
  static_assert(D % 16 == 0, "head dims must be multiples of 16");
};

// Where one call's channels sit in the packed buffers.  qkv and d_packed
// hold cs channels per slice: Q at [0, dk), K at [dk, 2dk), and this call's
// V rows from channel voff (cs = 2dk + dv, voff = 2dk for a call over all
// of V; a call over a slice of V has cs = 2dk + dv_total and DV = its own
// width).  accum != 0: the backward adds its dQ and dK to what d_packed
// holds instead of overwriting them (dV rows are always overwritten).
// ld: row stride of the inputs (qkv, and o and dO in the backward): N, or N
// rounded up to 8 when they were staged into zero-padded rows; outputs
// (o, lse, d_packed, statistics) always have rows of N.
struct PackView {
  int cs, voff, accum, ld;
};

// =================================================================== forward
// OCC > 0: the register allocator is held to OCC waves per SIMD.
template <typename T, int DK, int DV, int QB, int NW, int BN, bool VECOK, int OCC = 0>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(OCC > 0 ? OCC : 1, OCC > 0 ? OCC : 8)))
void psa_fwd_kernel(const T* __restrict__ qkv, T* __restrict__ o, float* __restrict__ lse, int N, int n_qtiles,
                    int n_blocks, float c /* scale * log2(e) */, const PackView pv) {
  constexpr int QW = 16 * QB, BM = NW * QW, NT = NW * 64;
  constexpr int KC = Chunks<DK>::n;
  // Wave priority raised over the score MFMAs and lowered for the softmax
  // (16-bit, dk >= 64, wide tiles): N = 6400 383-384 vs 387-388 us; raised
  // over the PV MFMAs as well it cost 1.5 %.
  constexpr bool PRIO = is_16bit<T>() && DK >= 64 && QB > 1;
  static_assert(BN % 32 == 0 && DV % 16 == 0, "tile shape");
  // K|V tile, channel-major: K rows read as token rows for S^T, V rows as
  // channel rows for PV.  16-bit types with 16-byte rows (VECOK) bring it
  // into LDS by direct loads (DKV), others through registers (SKV); both
  // write the same layout.
  constexpr bool DMA = VECOK && is_16bit<T>();
  using SKV = Stager<T, DK + DV, BN, NT, VECOK, DK>;
  using DKV = DmaStage<std::conditional_t<DMA, T, bf16>, DK + DV, DMA ? BN : 32, NW, DK>;
  using SQ = Stager<T, DK, BM, NT, VECOK, DK>;
  constexpr int BUF = DMA ? DKV::ELEMS : SKV::NAT_ELEMS;
  constexpr int QE = SQ::NAT_ELEMS;
  constexpr int SMEM = 2 * BUF > QE ? 2 * BUF : QE;
  __shared__ __attribute__((aligned(1024))) T smem[SMEM];

  const int tid = thread_id(), w = tid >> 6, lane = tid & 63, g = lane >> 4, t = lane & 15;
  const int blk = xcd_remap(block_id(), n_blocks);
  const int bh = blk / n_qtiles, i0 = (blk - bh * n_qtiles) * BM;
  const int ld = pv.ld;
  const T* Qg = qkv + (size_t)bh * pv.cs * ld;
  const T* KVg = Qg + (size_t)DK * ld;
  const T* Vg = Qg + (size_t)pv.voff * ld;

  // Stationary queries: B operands of S^T = K Q^T (lane = query column).
  Frag<T> qf[QB][KC];
  {
    SQ sq;
    sq.load(Qg, Qg, ld, N, i0, tid);
    sq.store(smem, tid);
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < QB; ++nb)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        frag_tok<DK, false>(qf[nb][kc], smem, SQ::LDN, w * QW + 16 * nb, 0, 32 * kc);
      }
    __syncthreads();
  }

  SKV st;
  DKV dst;
  const int wv = __builtin_amdgcn_readfirstlane(w);
  if constexpr (DMA) {
    dst.init(wv, lane, DK * ld, pv.voff * ld, ld);
    dst.issue(Qg, 0, ld, smem, wv, lane);
    barrier_vmcnt<0>();
  } else {
    st.load(KVg, Vg, ld, N, 0, tid);
    st.store(smem, tid);
    __syncthreads();
  }

  const Frag<T> ones = ones_frag<T>();
  // m: running column maximum (log2 units, scale included); thr: the raw
  // score above which a column has outgrown m by more than the slack.
  float m[QB], thr[QB];
  const float cinv = 1.f / c;
  f32x4 oacc[DV / 16][QB], lacc[QB];
#pragma unroll
  for (int nb = 0; nb < QB; ++nb) {
    m[nb] = kNegInf;
    thr[nb] = kNegInf;
    lacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < DV / 16; ++cb) oacc[cb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int nkt = (N + BN - 1) / BN;
  for (int kt = 0; kt < nkt; ++kt) {
    T* nat = smem + (kt & 1) * BUF;
    const T* Vt = nat + DK * SKV::LDN;
    if (kt + 1 < nkt) {
      // the other stage was last read before the previous iteration's barrier
      if constexpr (DMA)
        dst.issue(Qg, (kt + 1) * BN, ld, smem + ((kt + 1) & 1) * BUF, wv, lane);
      else
        st.load(KVg, Vg, ld, N, (kt + 1) * BN, tid);
    }
    const int j0 = kt * BN;

#pragma unroll
    for (int c2 = 0; c2 < BN / 32; ++c2) {
      f32x4 s[2][QB];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int nb = 0; nb < QB; ++nb) s[h][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          Frag<T> a;
          frag_tok<DK, true>(a, nat, SKV::LDN, 32 * c2, h, 32 * kc);
#pragma unroll
          for (int nb = 0; nb < QB; ++nb) mma(s[h][nb], a, qf[nb][kc]);
        }
      }
      if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
      if (j0 + 32 * c2 + 32 > N) {  // keys past the end get zero weight
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (j0 + 32 * c2 + 8 * g + 4 * h + r >= N)
#pragma unroll
              for (int nb = 0; nb < QB; ++nb) s[h][nb][r] = kNegInf;
      }

      // Online softmax per query column; the 4 lane groups hold the rows.
      // Each lane checks only its own 8 rows against the running maximum
      // plus the slack; the exact column maximum (a reduction over the lane
      // groups) is formed only when some lane's scores outgrew it.
      // (A chain of maxima, so that it maps onto three-operand max.)
      float mx[QB];
      bool grow = false;
#pragma unroll
      for (int nb = 0; nb < QB; ++nb) {
        float v = fmaxf(fmaxf(s[0][nb][0], s[0][nb][1]), s[0][nb][2]);
        v = fmaxf(fmaxf(v, s[0][nb][3]), s[1][nb][0]);
        v = fmaxf(fmaxf(v, s[1][nb][1]), s[1][nb][2]);
        mx[nb] = fmaxf(v, s[1][nb][3]);
        grow |= mx[nb] > thr[nb];
      }
      if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
        for (int nb = 0; nb < QB; ++nb) {
          const float mn = fmaxf(m[nb], wave_max4(mx[nb]) * c);
          const float alpha = fast_exp2(m[nb] - mn);
          m[nb] = mn;
          thr[nb] = (mn + kRescaleSlack) * cinv;
          lacc[nb][0] *= alpha;  // only row 0 of the ones-product is read (epilogue)
#pragma unroll
          for (int cb = 0; cb < DV / 16; ++cb) {
            // With one query block, element by element: the vector form made
            // the compiler copy an accumulator at every iteration's end (and
            // the element form costs the wider tiles registers).
            if constexpr (QB == 1) {
#pragma unroll
              for (int r = 0; r < 4; ++r) oacc[cb][nb][r] *= alpha;
            } else {
              oacc[cb][nb] *= alpha;
            }
          }
        }
      }
      Frag<T> pf[QB];
#pragma unroll
      for (int nb = 0; nb < QB; ++nb) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r) s[h][nb][r] = fast_exp2(__builtin_fmaf(s[h][nb][r], c, -m[nb]));
        acc_to_frag(pf[nb], s[0][nb], s[1][nb]);
        mma(lacc[nb], ones, pf[nb]);
      }
      // O^T += V^T P^T over this chunk's 32 keys.
#pragma unroll
      for (int cb = 0; cb < DV / 16; ++cb) {
        Frag<T> a;
        frag_ch(a, Vt, SKV::LDN, 16 * cb, 32 * c2);
#pragma unroll
        for (int nb = 0; nb < QB; ++nb) mma(oacc[cb][nb], a, pf[nb]);
      }
    }

    if constexpr (DMA) {
      barrier_vmcnt<0>();  // this wave's loads of the next tile landed, then everyone's
    } else {
      if (kt + 1 < nkt) {
        T* nx = smem + ((kt + 1) & 1) * BUF;
        st.store(nx, tid);
      }
      __syncthreads();
    }
  }

  // Epilogue: every row of the ones-product holds the column sum l.
#pragma unroll
  for (int nb = 0; nb < QB; ++nb) {
    const float l = lacc[nb][0];
    const float inv = fast_rcp(l);
    const int i = i0 + w * QW + 16 * nb + t;
    if (i < N) {
#pragma unroll
      for (int cb = 0; cb < DV / 16; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          o[((size_t)bh * DV + 16 * cb + 4 * g + r) * N + i] = from_f32<T>(oacc[cb][nb][r] * inv);
      if (g == 0) lse[(size_t)bh * N + i] = (m[nb] + fast_log2(l)) * kLn2;
    }
  }
}

// ========================================================= backward: D, LSE2
// nl[q] = -LSE_q * log2(e) and nd[q] = -D_q for every query of every slice
// (two planes of `total` floats): both are only ever subtracted (exp2(S c -
// LSE log2 e) and dP - D), and stored negated they enter an FMA or an MFMA
// accumulator input as they are; four consecutive queries are one 16-byte
// LDS read.
//
// VEC = true (ld a multiple of the 16-byte vector): lane (tg, cg) of a wave
// owns the 16-byte token group tg (8 bf16/fp16 or 4 fp32 tokens) and the
// channel group cg (dv / 8 channels), so that each lane issues all its loads
// at once; the 8 channel groups' partial sums are then added across lanes,
// as ((p0 + p1) + (p2 + p3)) + ((p4 + p5) + (p6 + p7)).
// VEC = false: one thread per query, walking the dv channels with the same
// 8 partial sums added in the same order, so both variants give the same
// bits (padded and unpadded rows of one input give one result).
// o and dO rows have stride ld (>= N; tokens past N are zero padding and
// write nothing); lse and the two planes have rows of N.
template <typename T, int DV, bool VEC>
__global__ __launch_bounds__(256) void psa_bwd_pre_kernel(const T* __restrict__ o, const T* __restrict__ dO,
                                                          const float* __restrict__ lse, float* __restrict__ stats,
                                                          int N, int ld, int total) {
  if constexpr (!VEC) {
    const int idx = block_id() * 256 + thread_id();
    if (idx >= total) return;
    const int bh = idx / N, i = idx - bh * N;
    const T* op = o + (size_t)bh * DV * ld + i;
    const T* gp = dO + (size_t)bh * DV * ld + i;
    constexpr int NCG = 8, CPT = DV / NCG;
    static_assert(DV % NCG == 0, "channel groups");
    float p[NCG];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      p[cg] = 0.f;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const size_t off = (size_t)(cg * CPT + c) * ld;
        p[cg] = __builtin_fmaf(to_f32(op[off]), to_f32(gp[off]), p[cg]);
      }
    }
    const float d = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    stats[idx] = -lse[idx] * kLog2e;
    stats[(size_t)total + idx] = -d;
  } else {
    constexpr int TV = 16 / (int)sizeof(T), NCG = 8, CPT = DV / NCG;
    static_assert(DV % NCG == 0, "channel groups");
    typedef T V __attribute__((ext_vector_type(TV)));
    const int tid = thread_id(), lane = tid & 63, tg = lane & 7, cg = lane >> 3;
    const int grp = (block_id() * 4 + (tid >> 6)) * 8 + tg;  // 16-byte token group
    const int gpr = ld / TV;                                  // token groups per slice
    const int bh = grp / gpr, i0 = (grp - bh * gpr) * TV;
    const bool live = bh < total / N;
    float d[TV];
#pragma unroll
    for (int e = 0; e < TV; ++e) d[e] = 0.f;
    if (live) {
      const size_t base = ((size_t)bh * DV + cg * CPT) * ld + i0;
      V ov[CPT], gv[CPT];
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        ov[c] = *(const V*)(o + base + (size_t)c * ld);
        gv[c] = *(const V*)(dO + base + (size_t)c * ld);
      }
#pragma unroll
      for (int c = 0; c < CPT; ++c)
#pragma unroll
        for (int e = 0; e < TV; ++e) d[e] = __builtin_fmaf(to_f32<T>(ov[c][e]), to_f32<T>(gv[c][e]), d[e]);
    }
    // Channel groups are lane bits 3..5: add across them (every lane active).
#pragma unroll
    for (int e = 0; e < TV; ++e) {
      d[e] += __shfl_xor(d[e], 8);
      d[e] += __shfl_xor(d[e], 16);
      d[e] += __shfl_xor(d[e], 32);
    }
    if (live && cg == 0) {
      const size_t q0 = (size_t)bh * N + i0;
#pragma unroll
      for (int e = 0; e < TV; ++e)
        if (i0 + e < N) {
          stats[q0 + e] = -lse[q0 + e] * kLog2e;
          stats[(size_t)total + q0 + e] = -d[e];
        }
    }
  }
}

// Copies rows of n elements (16-bit) into rows of ld (a multiple of 8) with
// zeros past n: the inputs of a call whose N is not a multiple of 8, so that
// the kernels stage them with aligned 16-byte loads.  One 16-byte output
// chunk per thread; load8_funnel reads the source rows.
template <typename T>
__global__ __launch_bounds__(256) void psa_pad_rows_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                                           long long rows, int n, int ld) {
  static_assert(is_16bit<T>(), "16-bit element type");
  const long long q = (long long)block_id() * 256 + thread_id();
  const int cpr = ld / 8;
  if (q >= rows * cpr) return;
  const long long r = q / cpr;
  const int j = (int)(q - r * cpr) * 8;
  const u32x4 v = j < n ? load8_funnel(src + r * n + j, n - j) : u32x4{0u, 0u, 0u, 0u};
  *(u32x4*)(dst + r * ld + j) = v;
}

// ============================================================ backward dK/dV
// Key-stationary body: workgroup `blk` owns BNK = NW*16*KB keys of one slice
// and streams the queries in tiles of BMQ through a double-buffered LDS tile.
template <typename T, int DK, int DV, int KB, int NW, int BMQ>
struct DkdvShape {
  static constexpr int KW = 16 * KB, BNK = NW * KW, NT = NW * 64;
  // Q|dO streamed tile and K|V stationary tile, both channel-major.  16-bit
  // types stream Q and dO by direct loads where rows are 16-byte aligned
  // (DQP, DGP: the Q rows, then the dO rows from a 1 KB boundary, each in
  // the layout of the register staging SQG); a stage has room for either.
  using T16 = std::conditional_t<is_16bit<T>(), T, bf16>;
  using SQG = Stager<T, DK + DV, BMQ, NT, true, DK>;
  using DQP = DmaStage<T16, DK, BMQ, NW>;
  using DGP = DmaStage<T16, DV, BMQ, NW>;
  using SKV = Stager<T, DK + DV, BNK, NT, true, DK>;
  static constexpr int DTILE = DQP::ELEMS + DGP::ELEMS;
  static constexpr int TILE = is_16bit<T>() && DTILE > SQG::NAT_ELEMS ? DTILE : (int)SQG::NAT_ELEMS;
  static constexpr int QG_BYTES = 2 * TILE * (int)sizeof(T) + 4 * BMQ * (int)sizeof(float);
  static_assert(2 * TILE * sizeof(T) % 16 == 0, "statistics must be 16-byte aligned");
  static constexpr int KV_BYTES = SKV::NAT_ELEMS * (int)sizeof(T);
  static constexpr int SMEM = QG_BYTES > KV_BYTES ? QG_BYTES : KV_BYTES;
};

template <typename T, int DK, int DV, int KB, int NW, int BMQ, bool VECOK, bool DEEP = false>
__device__ __forceinline__ void bwd_dkdv_body(const T* __restrict__ qkv, const T* __restrict__ dO,
                                              const float* __restrict__ nlg, const float* __restrict__ ndg,
                                              T* __restrict__ dpk, int N,
                                              int n_ktiles, float c, float scale, const PackView pv,
                                              int blk, unsigned char* smem_raw) {
  using Shape = DkdvShape<T, DK, DV, KB, NW, BMQ>;
  constexpr int KW = Shape::KW, BNK = Shape::BNK, NT = Shape::NT;
  constexpr int KC = Chunks<DK>::n, CC = Chunks<DV>::n;
  static_assert(BMQ % 32 == 0, "query tile must be a multiple of 32");
  static_assert(BMQ <= NT, "one statistics entry per thread");
  using SQG = Stager<T, DK + DV, BMQ, NT, VECOK, DK>;
  using SKV = Stager<T, DK + DV, BNK, NT, VECOK, DK>;
  // Direct loads for the streamed tiles except in the two-deep register
  // prefetch (DEEP), which keeps register staging.
  constexpr bool DMA = VECOK && is_16bit<T>() && !DEEP;
  // Wave priority raised over the score MFMAs (S and dP) and lowered for the
  // softmax (16-bit, dk >= 64): the N = 6400 backward about 1 % faster than
  // with no raise, and than with it raised over every MFMA block; in the dQ
  // body as well it changed nothing (1002-1005 vs 1001-1002 us), in the dQ
  // body alone it cost 1.3 %; at dk = 32 it cost 3 % at N = 400 to 800.
  constexpr bool PRIO = is_16bit<T>() && DK >= 64;
  using DQP = typename Shape::DQP;
  using DGP = typename Shape::DGP;
  constexpr int TILE = Shape::TILE, LDN = SQG::LDN;
  constexpr int GOFF = DMA ? (int)DQP::ELEMS : DK * LDN;  // where the dO rows of a stage start
  T* smem = (T*)smem_raw;
  float* snl = (float*)(smem_raw + 2 * TILE * sizeof(T));  // [2][BMQ], then snd [2][BMQ]
  float* snd = snl + 2 * BMQ;

  const int tid = thread_id(), w = tid >> 6, lane = tid & 63, g = lane >> 4, t = lane & 15;
  const int bh = blk / n_ktiles, j0 = (blk - bh * n_ktiles) * BNK;
  const size_t C = pv.cs;
  const int ld = pv.ld;
  const T* Qg = qkv + (size_t)bh * C * ld;
  const T* KVg = Qg + (size_t)DK * ld;
  const T* Vg = Qg + (size_t)pv.voff * ld;
  const T* dOg = dO + (size_t)bh * DV * ld;
  const float* nlq = nlg + (size_t)bh * N;
  const float* ndq = ndg + (size_t)bh * N;

  // Stationary keys: B operands of S = Q K^T and dP = dO V^T (lane = key).
  Frag<T> kf[KB][KC], vf[KB][CC];
  {
    SKV sk;
    sk.load(KVg, Vg, ld, N, j0, tid);
    sk.store(smem, tid);
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int row0 = w * KW + 16 * kb;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        frag_tok<DK, false>(kf[kb][kc], smem, SKV::LDN, row0, 0, 32 * kc);
      }
#pragma unroll
      for (int cc = 0; cc < CC; ++cc) {
        frag_tok<DV, false>(vf[kb][cc], smem + DK * SKV::LDN, SKV::LDN, row0, 0, 32 * cc);
      }
    }
    __syncthreads();
  }

  f32x4 dvacc[DV / 16][KB], dkacc[DK / 16][KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
    for (int cb = 0; cb < DV / 16; ++cb) dvacc[cb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < DK / 16; ++db) dkacc[db][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  SQG sg;
  DQP dqp;
  DGP dgp;
  const int wv = __builtin_amdgcn_readfirstlane(w);
  // Direct loads of query tile qt's Q and dO rows into a stage.
  auto issue_tile = [&](int qt, T* stage) {
    if constexpr (DMA) {
      dqp.issue(Qg, qt * BMQ, ld, stage, wv, lane);
      dgp.issue(dOg, qt * BMQ, ld, stage + GOFF, wv, lane);
    }
  };
  if constexpr (DMA) {
    dqp.init(wv, lane, 0, 0, ld);
    dgp.init(wv, lane, 0, 0, ld);
    issue_tile(0, smem);
  } else {
    sg.load(Qg, dOg, ld, N, 0, tid);
    sg.store(smem, tid);
  }
  for (int q = tid; q < BMQ; q += NT) {  // padding rows: P = 0
    snl[q] = q < N ? nlq[q] : kNegInf;
    snd[q] = q < N ? ndq[q] : 0.f;
  }
  if constexpr (DMA)
    barrier_vmcnt<0>();
  else
    __syncthreads();

  // DEEP: the two thread halves take turns, each keeping one tile in flight
  // in its registers from the top of iteration qt to the end of qt + 1: a
  // prefetch distance of two tiles, at the register cost of one wherever a
  // tile needs no more than half the threads.
  using SQH = Stager<T, DK + DV, BMQ, NT / 2, VECOK, DK, true>;  // queries past N weigh 0: clamped loads
  static_assert(!DEEP || BMQ <= NT / 2, "one statistics entry per thread of a half");
  const int half = tid >= NT / 2, htid = tid - half * (NT / 2);
  SQH sh;
  float pnl = kNegInf, pnd = 0.f;
  auto load_tile = [&](int qt, int lt) {  // rows and statistics of query tile qt (lt = thread index)
    if constexpr (DEEP)
      sh.load(Qg, dOg, ld, N, qt * BMQ, lt);
    else if constexpr (!DMA)
      sg.load(Qg, dOg, ld, N, qt * BMQ, lt);
    const int q = qt * BMQ + lt;
    pnl = kNegInf, pnd = 0.f;
    if (lt < BMQ && q < N) {  // padding queries: P = 0
      pnl = nlq[q];
      pnd = ndq[q];
    }
  };
  const int nqt = (N + BMQ - 1) / BMQ;
  if constexpr (DEEP) {
    if (half == 1 && 1 < nqt) load_tile(1, htid);
  }
  for (int qt = 0; qt < nqt; ++qt) {
    const int cur = qt & 1;
    const T* nat = smem + cur * TILE;   // rows: Q channels, then dO channels
    const float* sl = snl + cur * BMQ;
    const float* sd = snd + cur * BMQ;
    // Prefetch a later tile (rows and its queries' statistics) into
    // registers; they reach LDS after this tile's MFMAs.
    if constexpr (DEEP) {
      if (qt + 2 < nqt && half == cur) load_tile(qt + 2, htid);
    } else if (qt + 1 < nqt) {
      // the other stage was last read before the previous iteration's barrier
      issue_tile(qt + 1, smem + (cur ^ 1) * TILE);
      load_tile(qt + 1, tid);
    }

#pragma unroll
    for (int c2 = 0; c2 < BMQ / 32; ++c2) {
      // Rows of block h are the queries 32*c2 + 8g + 4h + r (r = register).
      f32x4 nl[2], nd[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        nl[h] = *(const f32x4*)(sl + 32 * c2 + 8 * g + 4 * h);
        nd[h] = *(const f32x4*)(sd + 32 * c2 + 8 * g + 4 * h);
      }
      f32x4 s[2][KB], dp[2][KB];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // dP accumulates on top of -D, so that dS = P * acc.
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          s[h][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
          dp[h][kb] = nd[h];
        }
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          Frag<T> a;
          frag_tok<DK, true>(a, nat, LDN, 32 * c2, h, 32 * kc);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) mma(s[h][kb], a, kf[kb][kc]);
        }
#pragma unroll
        for (int cc = 0; cc < CC; ++cc) {
          Frag<T> a;
          frag_tok<DV, true>(a, nat + GOFF, LDN, 32 * c2, h, 32 * cc);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) mma(dp[h][kb], a, vf[kb][cc]);
        }
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            const float p = fast_exp2(__builtin_fmaf(s[h][kb][r], c, nl[h][r]));
            s[h][kb][r] = p;
            dp[h][kb][r] *= p;
          }
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS over this chunk's 32 queries.
      Frag<T> pf[KB], dsf[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        acc_to_frag(pf[kb], s[0][kb], s[1][kb]);
        acc_to_frag(dsf[kb], dp[0][kb], dp[1][kb]);
      }
#pragma unroll
      for (int cb = 0; cb < DV / 16; ++cb) {
        Frag<T> a;
        frag_ch(a, nat + GOFF, LDN, 16 * cb, 32 * c2);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) mma(dvacc[cb][kb], a, pf[kb]);
      }
#pragma unroll
      for (int db = 0; db < DK / 16; ++db) {
        Frag<T> a;
        frag_ch(a, nat, LDN, 16 * db, 32 * c2);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) mma(dkacc[db][kb], a, dsf[kb]);
      }
    }

    if (qt + 1 < nqt && (!DEEP || half != cur)) {
      T* nx = smem + (cur ^ 1) * TILE;
      const int lt = DEEP ? htid : tid;
      if constexpr (DEEP)
        sh.store(nx, lt);
      else if constexpr (!DMA)
        sg.store(nx, lt);
      if (lt < BMQ) {
        snl[(cur ^ 1) * BMQ + lt] = pnl;
        snd[(cur ^ 1) * BMQ + lt] = pnd;
      }
    }
    if constexpr (DMA)
      barrier_vmcnt<0>();  // this wave's loads of the next tile landed, then everyone's
    else
      __syncthreads();
  }

  auto epilogue = [&](auto accum) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int j = j0 + w * KW + 16 * kb + t;
      if (j < N) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
          for (int db = 0; db < DK / 16; ++db) {
            T* p = dpk + ((size_t)bh * C + DK + 16 * db + 4 * g + r) * N + j;
            const float v = dkacc[db][kb][r] * scale;
            *p = from_f32<T>(decltype(accum)::value ? to_f32(*p) + v : v);
          }
#pragma unroll
          for (int cb = 0; cb < DV / 16; ++cb)
            dpk[((size_t)bh * C + pv.voff + 16 * cb + 4 * g + r) * N + j] = from_f32<T>(dvacc[cb][kb][r]);
        }
      }
    }
  };
  if (pv.accum)
    epilogue(std::true_type{});
  else
    epilogue(std::false_type{});
}

// =============================================================== backward dQ
// Query-stationary body: workgroup `blk` owns BM = NW*16*QB queries of one
// slice and streams the keys in tiles of BN through a double-buffered tile.
template <typename T, int DK, int DV, int QB, int NW, int BN>
struct DqShape {
  static constexpr int QW = 16 * QB, BM = NW * QW, NT = NW * 64;
  // Streamed K|V tile and stationary Q|dO tile, both channel-major.  16-bit
  // types stream K|V by direct loads where rows are 16-byte aligned: a
  // stage is BN / SUB sub-tiles of SUB keys (DKV, one set of per-lane
  // offsets for all of them), each in the layout the register staging (SKV)
  // gives a whole tile; a stage has room for either.
  static constexpr int SUB = BN < 64 ? BN : 64, NSUB = BN / SUB;
  using SKV = Stager<T, DK + DV, BN, NT, true, DK>;
  using DKV = DmaStage<std::conditional_t<is_16bit<T>(), T, bf16>, DK + DV, SUB, NW, DK>;
  using SQG = Stager<T, DK + DV, BM, NT, true, DK>;
  static constexpr int DBUF = NSUB * DKV::ELEMS;
  static constexpr int BUF = is_16bit<T>() && DBUF > SKV::NAT_ELEMS ? DBUF : (int)SKV::NAT_ELEMS;
  static constexpr int QE = SQG::NAT_ELEMS;
  static constexpr int SMEM = (2 * BUF > QE ? 2 * BUF : QE) * (int)sizeof(T);
};

template <typename T, int DK, int DV, int QB, int NW, int BN, bool VECOK>
__device__ __forceinline__ void bwd_dq_body(const T* __restrict__ qkv, const T* __restrict__ dO,
                                            const float* __restrict__ nlg, const float* __restrict__ ndg,
                                            T* __restrict__ dpk, int N, int n_qtiles, float c, float scale,
                                            const PackView pv, int blk, unsigned char* smem_raw) {
  using Shape = DqShape<T, DK, DV, QB, NW, BN>;
  constexpr int QW = Shape::QW, BM = Shape::BM, NT = Shape::NT;
  constexpr int KC = Chunks<DK>::n, CC = Chunks<DV>::n;
  static_assert(BN % 32 == 0, "key tile must be a multiple of 32");
  constexpr bool DMA = VECOK && is_16bit<T>();
  using SKV = Stager<T, DK + DV, BN, NT, VECOK, DK>;
  using DKV = typename Shape::DKV;
  using SQG = Stager<T, DK + DV, BM, NT, VECOK, DK>;
  constexpr int BUF = Shape::BUF;
  T* smem = (T*)smem_raw;

  const int tid = thread_id(), w = tid >> 6, lane = tid & 63, g = lane >> 4, t = lane & 15;
  const int bh = blk / n_qtiles, i0 = (blk - bh * n_qtiles) * BM;
  const size_t C = pv.cs;
  const int ld = pv.ld;
  const T* Qg = qkv + (size_t)bh * C * ld;
  const T* KVg = Qg + (size_t)DK * ld;
  const T* Vg = Qg + (size_t)pv.voff * ld;
  const T* dOg = dO + (size_t)bh * DV * ld;

  // Stationary queries: B operands of S^T = K Q^T and dP^T = V dO^T.  Their
  // LSE (log2 units, negated) and -D are per lane (lane column = query).
  Frag<T> qf[QB][KC], gf[QB][CC];
  float nl[QB], nd[QB];
  {
    SQG sq;
    sq.load(Qg, dOg, ld, N, i0, tid);
    sq.store(smem, tid);
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < QB; ++nb) {
      const int row0 = w * QW + 16 * nb;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        frag_tok<DK, false>(qf[nb][kc], smem, SQG::LDN, row0, 0, 32 * kc);
      }
#pragma unroll
      for (int cc = 0; cc < CC; ++cc) {
        frag_tok<DV, false>(gf[nb][cc], smem + DK * SQG::LDN, SQG::LDN, row0, 0, 32 * cc);
      }
      const int i = i0 + row0 + t;
      nl[nb] = i < N ? nlg[(size_t)bh * N + i] : kNegInf;
      nd[nb] = i < N ? ndg[(size_t)bh * N + i] : 0.f;
    }
    __syncthreads();
  }

  f32x4 dqacc[DK / 16][QB];
#pragma unroll
  for (int nb = 0; nb < QB; ++nb)
#pragma unroll
    for (int db = 0; db < DK / 16; ++db) dqacc[db][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  SKV sk;
  DKV dkv;
  const int wv = __builtin_amdgcn_readfirstlane(w);
  constexpr int SUB = Shape::SUB, NSUB = Shape::NSUB;
  auto issue = [&](int j0, T* stage) {
    if constexpr (DMA) {
#pragma unroll
      for (int u = 0; u < NSUB; ++u) dkv.issue(Qg, j0 + u * SUB, ld, stage + u * DKV::ELEMS, wv, lane);
    }
  };
  // Where chunk c2's 32 keys sit: sub-tile c2 / (SUB / 32) of a direct-load
  // stage, or the register-staged tile.
  constexpr int LDN = DMA ? nat_pitch<T>(SUB) : SKV::LDN;
  auto chunk = [&](const T* nat, int c2) -> const T* {
    return DMA ? nat + (c2 / (SUB / 32)) * DKV::ELEMS : nat;
  };
  auto ckey = [&](int c2) { return DMA ? 32 * (c2 % (SUB / 32)) : 32 * c2; };
  if constexpr (DMA) {
    dkv.init(wv, lane, DK * ld, pv.voff * ld, ld);
    issue(0, smem);
    barrier_vmcnt<0>();
  } else {
    sk.load(KVg, Vg, ld, N, 0, tid);
    sk.store(smem, tid);
    __syncthreads();
  }

  const int nkt = (N + BN - 1) / BN;
  for (int kt = 0; kt < nkt; ++kt) {
    const T* nat = smem + (kt & 1) * BUF;  // K then V channels, channel-major
    const int j0 = kt * BN;
    if (kt + 1 < nkt) {
      // the other stage was last read before the previous iteration's barrier
      if constexpr (DMA)
        issue((kt + 1) * BN, smem + ((kt + 1) & 1) * BUF);
      else
        sk.load(KVg, Vg, ld, N, (kt + 1) * BN, tid);
    }

#pragma unroll
    for (int c2 = 0; c2 < BN / 32; ++c2) {
      f32x4 s[2][QB], dp[2][QB];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // dP^T accumulates on top of -D, so that dS^T = P^T * acc.
#pragma unroll
        for (int nb = 0; nb < QB; ++nb) {
          s[h][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
          dp[h][nb] = f32x4{nd[nb], nd[nb], nd[nb], nd[nb]};
        }
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          Frag<T> a;
          frag_tok<DK, true>(a, chunk(nat, c2), LDN, ckey(c2), h, 32 * kc);
#pragma unroll
          for (int nb = 0; nb < QB; ++nb) mma(s[h][nb], a, qf[nb][kc]);
        }
#pragma unroll
        for (int cc = 0; cc < CC; ++cc) {
          Frag<T> a;
          frag_tok<DV, true>(a, chunk(nat, c2) + DK * LDN, LDN, ckey(c2), h, 32 * cc);
#pragma unroll
          for (int nb = 0; nb < QB; ++nb) mma(dp[h][nb], a, gf[nb][cc]);
        }
        // Keys past N: direct loads leave other tokens' (finite) values in
        // their K and V rows, so their scores get zero weight here; the
        // register staging leaves zero rows, whose score 0 the clamp below
        // keeps finite.
        if constexpr (DMA) {
          if (j0 + 32 * c2 + 32 > N) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (j0 + 32 * c2 + 8 * g + 4 * h + r >= N)
#pragma unroll
                for (int nb = 0; nb < QB; ++nb) s[h][nb][r] = kNegInf;
          }
        }
        // P is clamped to [0, 1] (the exp's output modifier, no extra
        // instruction).  A real key has P = exp(S - LSE) <= 1 already; a key
        // past N with a zero K row has score 0 and P = exp(-LSE), which
        // for a query with a very negative LSE overflows the operand type,
        // and inf times its zero K row would be NaN.  Clamped, its dS^T stays
        // finite and meets only zeros.
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
          for (int nb = 0; nb < QB; ++nb)
            dp[h][nb][r] *= __builtin_amdgcn_fmed3f(fast_exp2(__builtin_fmaf(s[h][nb][r], c, nl[nb])), 0.f, 1.f);
        }
      }
      // dQ^T += K^T dS^T over this chunk's 32 keys.
      Frag<T> dsf[QB];
#pragma unroll
      for (int nb = 0; nb < QB; ++nb) acc_to_frag(dsf[nb], dp[0][nb], dp[1][nb]);
#pragma unroll
      for (int db = 0; db < DK / 16; ++db) {
        Frag<T> a;
        frag_ch(a, chunk(nat, c2), LDN, 16 * db, ckey(c2));
#pragma unroll
        for (int nb = 0; nb < QB; ++nb) mma(dqacc[db][nb], a, dsf[nb]);
      }
    }

    if constexpr (DMA) {
      barrier_vmcnt<0>();  // this wave's loads of the next tile landed, then everyone's
    } else {
      if (kt + 1 < nkt) {
        T* nx = smem + ((kt + 1) & 1) * BUF;
        sk.store(nx, tid);
      }
      __syncthreads();
    }
  }

  auto epilogue = [&](auto accum) {
#pragma unroll
    for (int nb = 0; nb < QB; ++nb) {
      const int i = i0 + w * QW + 16 * nb + t;
      if (i < N) {
#pragma unroll
        for (int db = 0; db < DK / 16; ++db)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            T* p = dpk + ((size_t)bh * C + 16 * db + 4 * g + r) * N + i;
            const float v = dqacc[db][nb][r] * scale;
            *p = from_f32<T>(decltype(accum)::value ? to_f32(*p) + v : v);
          }
      }
    }
  };
  if (pv.accum)
    epilogue(std::true_type{});
  else
    epilogue(std::false_type{});
}

// ========================================================= backward kernels
// Both backward GEMM chains in one launch: the first n_kblocks workgroups
// are key-stationary (dK, dV), the rest query-stationary (dQ).  The long
// dK/dV workgroups are dispatched first and the shorter dQ ones fill the
// machine behind them, so neither pass leaves a partly idle last wave of
// workgroups on its own; both share one LDS allocation.
template <typename T, int DK, int DV, int KB, int BMQ, int QB, int BN, int NW, bool VECOK, bool DEEP>
__global__ __launch_bounds__(NW * 64) void psa_bwd_fused_kernel(
    const T* __restrict__ qkv, const T* __restrict__ dO, const float* __restrict__ nl, const float* __restrict__ nd,
    T* __restrict__ dpk, int N, int n_ktiles, int n_qtiles, int n_kblocks, int n_qblocks, float c, float scale,
    const PackView pv) {
  constexpr int S1 = DkdvShape<T, DK, DV, KB, NW, BMQ>::SMEM, S2 = DqShape<T, DK, DV, QB, NW, BN>::SMEM;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[S1 > S2 ? S1 : S2];
  const int b = block_id();
  if (b < n_kblocks)
    bwd_dkdv_body<T, DK, DV, KB, NW, BMQ, VECOK, DEEP>(qkv, dO, nl, nd, dpk, N, n_ktiles, c, scale, pv,
                                                      xcd_remap(b, n_kblocks), smem);
  else
    bwd_dq_body<T, DK, DV, QB, NW, BN, VECOK>(qkv, dO, nl, nd, dpk, N, n_qtiles, c, scale, pv,
                                             xcd_remap(b - n_kblocks, n_qblocks), smem);
}

}  // namespace psa
