// PSA self-attention kernels for gfx950 (CDNA4).
//
// The method (PsaFa2Backward page, vision_rs psa kernels, struct
// description): Flash-Attention-2 over the N = H*W tokens of one (batch,
// head) slice, where queries and keys are the same N tokens and every query
// sees every key.  The page's own schedule (one CTA per query row, dq/dk
// summed with float atomics) is not used here.  Instead:
//
//   psa_fwd_kernel   one workgroup per (slice, tile of BM queries); each wave
//                    keeps QW queries stationary and streams key tiles of BN
//                    through LDS: S^T = K Q^T (MFMA), online softmax in
//                    log2 units, O^T += V^T P^T (MFMA).  Writes O and LSE.
//   psa_bwd_pre      D_i = sum_c dO_ic O_ic and LSE in log2 units, one
//                    thread per query (coalesced over tokens).
//   psa_bwd_dkdv     one workgroup per (slice, tile of keys); keys
//                    stationary, query tiles streamed: S = Q K^T,
//                    dP = dO V^T, P = exp(S - LSE), dS = P (dP - D),
//                    dV^T += dO^T P, dK^T += Q^T dS.
//   psa_bwd_dq       one workgroup per (slice, tile of queries); queries
//                    stationary, key tiles streamed: S^T, dP^T, dS^T as
//                    above, dQ^T += K^T dS^T.
// Every output element is written exactly once by one lane: no atomics, no
// zero-initialisation, bitwise reproducible.
//
// Orientation: outputs are accumulated transposed (channels as MFMA rows,
// tokens as MFMA columns) so that accumulator lanes run along tokens and
// stores to the channel-major tensors are coalesced; the score matrix is
// built as S^T where the next GEMM contracts over keys (fwd, dQ) and as S
// where it contracts over queries (dK/dV), so that P and dS feed the next
// MFMA straight from registers (acc_to_frag).
#pragma once
#include "psa_common.h"

namespace psa {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();

template <int D> struct Chunks {
  static constexpr int n = (D + 31) / 32;            // 32-wide contraction chunks
  static constexpr int last = (D % 32 == 16) ? 4 : 8; // data slots in the last one
  static_assert(D % 16 == 0, "head dims must be multiples of 16");
};

template <typename T> constexpr int lds_pad() { return 16 / (int)sizeof(T); }

// =================================================================== forward
template <typename T, int DK, int DV, int QB, int NW, int BN, bool VECOK>
__global__ __launch_bounds__(NW * 64) void psa_fwd_kernel(
    const T* __restrict__ qkv, T* __restrict__ o, float* __restrict__ lse, int N, int n_qtiles,
    float c /* scale * log2(e) */) {
  constexpr int QW = 16 * QB, BM = NW * QW, NT = NW * 64;
  constexpr int KC = Chunks<DK>::n, KSL = Chunks<DK>::last;
  constexpr int MB = BN / 16;
  constexpr int LDK = BN + lds_pad<T>(), LDQ = BM + lds_pad<T>();
  constexpr int KV_ELEMS = (DK + DV) * LDK;
  constexpr int SMEM = 2 * KV_ELEMS > DK * LDQ ? 2 * KV_ELEMS : DK * LDQ;
  static_assert(BN % 32 == 0 && DV % 16 == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) T smem[SMEM];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, t = lane & 15;
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = blk / n_qtiles, i0 = (blk - bh * n_qtiles) * BM;
  const T* Qg = qkv + (size_t)bh * (2 * DK + DV) * N;
  const T* KVg = Qg + (size_t)DK * N;

  // Stationary queries: B operand of S^T = K Q^T (lane = query, slots = channels).
  Frag<T> qf[QB][KC];
  {
    TileLoader<T, DK, BM, NT, VECOK> ql;
    ql.load(Qg, N, i0, tid);
    ql.store(smem, LDQ, tid);
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < QB; ++nb)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        if (kc == KC - 1) load_tr<KSL>(qf[nb][kc], smem, LDQ, 32 * kc, w * QW + 16 * nb);
        else load_tr<8>(qf[nb][kc], smem, LDQ, 32 * kc, w * QW + 16 * nb);
      }
    __syncthreads();
  }

  TileLoader<T, DK + DV, BN, NT, VECOK> kvl;
  kvl.load(KVg, N, 0, tid);
  kvl.store(smem, LDK, tid);
  __syncthreads();

  float m[QB], l[QB];
  f32x4 oacc[DV / 16][QB];
#pragma unroll
  for (int nb = 0; nb < QB; ++nb) {
    m[nb] = kNegInf;
    l[nb] = 0.f;
#pragma unroll
    for (int cb = 0; cb < DV / 16; ++cb) oacc[cb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int nkt = (N + BN - 1) / BN;
  for (int kt = 0; kt < nkt; ++kt) {
    const T* Kt = smem + (kt & 1) * KV_ELEMS;
    const T* Vt = Kt + DK * LDK;
    if (kt + 1 < nkt) kvl.load(KVg, N, (kt + 1) * BN, tid);

    f32x4 s[MB][QB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int nb = 0; nb < QB; ++nb) s[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        Frag<T> a;
        if (kc == KC - 1) {
          load_tr<KSL>(a, Kt, LDK, 32 * kc, 16 * mb);
#pragma unroll
          for (int nb = 0; nb < QB; ++nb) mma<KSL>(s[mb][nb], a, qf[nb][kc]);
        } else {
          load_tr<8>(a, Kt, LDK, 32 * kc, 16 * mb);
#pragma unroll
          for (int nb = 0; nb < QB; ++nb) mma<8>(s[mb][nb], a, qf[nb][kc]);
        }
      }
    }
    const int j0 = kt * BN;
    if (j0 + BN > N) {  // keys past the end of the sequence get zero weight
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (j0 + 16 * mb + 4 * g + r >= N)
#pragma unroll
            for (int nb = 0; nb < QB; ++nb) s[mb][nb][r] = kNegInf;
    }

    // Online softmax per query column (this lane's column, rows over 4 lane groups).
#pragma unroll
    for (int nb = 0; nb < QB; ++nb) {
      float mx = s[0][nb][0];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[mb][nb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m[nb], mx * c);
      const float alpha = fast_exp2(m[nb] - mnew);
      m[nb] = mnew;
      float ls = l[nb] * alpha;
#pragma unroll
      for (int cb = 0; cb < DV / 16; ++cb) oacc[cb][nb] *= alpha;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(__builtin_fmaf(s[mb][nb][r], c, -mnew));
          s[mb][nb][r] = p;
          ls += p;
        }
      l[nb] = ls;
    }

    // O^T += V^T P^T, contraction over this tile's keys.
#pragma unroll
    for (int kc2 = 0; kc2 < MB / 2; ++kc2) {
      Frag<T> pf[QB];
#pragma unroll
      for (int nb = 0; nb < QB; ++nb) acc_to_frag(pf[nb], s[2 * kc2][nb], s[2 * kc2 + 1][nb]);
#pragma unroll
      for (int cb = 0; cb < DV / 16; ++cb) {
        Frag<T> a;
        load_nat(a, Vt, LDK, 16 * cb, 32 * kc2);
#pragma unroll
        for (int nb = 0; nb < QB; ++nb) mma<8>(oacc[cb][nb], a, pf[nb]);
      }
    }

    if (kt + 1 < nkt) kvl.store(smem + ((kt + 1) & 1) * KV_ELEMS, LDK, tid);
    __syncthreads();
  }

  // Epilogue: O = O_acc / l, LSE = ln(sum_j exp(S_ij)) = (m + log2 l) * ln 2.
#pragma unroll
  for (int nb = 0; nb < QB; ++nb) {
    float lt = l[nb] + __shfl_xor(l[nb], 16);
    lt += __shfl_xor(lt, 32);
    const float inv = fast_rcp(lt);
    const int i = i0 + w * QW + 16 * nb + t;
    if (i < N) {
#pragma unroll
      for (int cb = 0; cb < DV / 16; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          o[((size_t)bh * DV + 16 * cb + 4 * g + r) * N + i] = from_f32<T>(oacc[cb][nb][r] * inv);
      if (g == 0) lse[(size_t)bh * N + i] = (m[nb] + fast_log2(lt)) * kLn2;
    }
  }
}

// ========================================================= backward: D, LSE2
// stats[q] = {LSE_q * log2(e), D_q} for every query of every slice.
template <typename T, int DV>
__global__ __launch_bounds__(256) void psa_bwd_pre_kernel(const T* __restrict__ o, const T* __restrict__ dO,
                                                          const float* __restrict__ lse,
                                                          float2* __restrict__ stats, int N, int total) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int bh = idx / N, i = idx - bh * N;
  const T* op = o + (size_t)bh * DV * N + i;
  const T* gp = dO + (size_t)bh * DV * N + i;
  float d = 0.f;
#pragma unroll 16
  for (int ch = 0; ch < DV; ++ch) d = __builtin_fmaf(to_f32(op[(size_t)ch * N]), to_f32(gp[(size_t)ch * N]), d);
  stats[idx] = make_float2(lse[idx] * kLog2e, d);
}

// Per-query statistics of one query tile staged beside the Q/dO tile.
// Queries past the end get LSE = +inf (so P = 0) and D = 0.
template <int BMQ, int NT>
__device__ __forceinline__ void load_stats(float2* dst, const float2* __restrict__ src, int N, int q0, int tid) {
  for (int q = tid; q < BMQ; q += NT) dst[q] = (q0 + q < N) ? src[q0 + q] : make_float2(kPosInf, 0.f);
}

// ============================================================ backward dK/dV
template <typename T, int DK, int DV, int KB, int NW, int BMQ, bool VECOK>
__global__ __launch_bounds__(NW * 64) void psa_bwd_dkdv_kernel(
    const T* __restrict__ qkv, const T* __restrict__ dO, const float2* __restrict__ stats,
    T* __restrict__ dpk, int N, int n_ktiles, float c, float scale) {
  constexpr int KW = 16 * KB, BNK = NW * KW, NT = NW * 64;
  constexpr int KC = Chunks<DK>::n, KSL = Chunks<DK>::last;
  constexpr int CC = Chunks<DV>::n, CSL = Chunks<DV>::last;
  constexpr int MBQ = BMQ / 16;
  constexpr int LDQ = BMQ + lds_pad<T>(), LDK = BNK + lds_pad<T>();
  constexpr int QD_ELEMS = (DK + DV) * LDQ;
  constexpr int QD_BYTES = 2 * QD_ELEMS * (int)sizeof(T) + 2 * BMQ * (int)sizeof(float2);
  constexpr int KV_BYTES = (DK + DV) * LDK * (int)sizeof(T);
  constexpr int SMEM = QD_BYTES > KV_BYTES ? QD_BYTES : KV_BYTES;
  static_assert(BMQ % 32 == 0, "query tile must be a multiple of 32");
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[SMEM];
  T* smem = (T*)smem_raw;
  float2* sstats = (float2*)(smem_raw + 2 * QD_ELEMS * sizeof(T));

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, t = lane & 15;
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = blk / n_ktiles, j0 = (blk - bh * n_ktiles) * BNK;
  const size_t C = 2 * DK + DV;
  const T* Qg = qkv + (size_t)bh * C * N;
  const T* KVg = Qg + (size_t)DK * N;
  const T* dOg = dO + (size_t)bh * DV * N;
  const float2* st = stats + (size_t)bh * N;

  // Stationary keys: B operands of S = Q K^T and dP = dO V^T (lane = key).
  Frag<T> kf[KB][KC], vf[KB][CC];
  {
    TileLoader<T, DK + DV, BNK, NT, VECOK> kvl;
    kvl.load(KVg, N, j0, tid);
    kvl.store(smem, LDK, tid);
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        if (kc == KC - 1) load_tr<KSL>(kf[kb][kc], smem, LDK, 32 * kc, w * KW + 16 * kb);
        else load_tr<8>(kf[kb][kc], smem, LDK, 32 * kc, w * KW + 16 * kb);
      }
#pragma unroll
      for (int cc = 0; cc < CC; ++cc) {
        if (cc == CC - 1) load_tr<CSL>(vf[kb][cc], smem, LDK, DK + 32 * cc, w * KW + 16 * kb);
        else load_tr<8>(vf[kb][cc], smem, LDK, DK + 32 * cc, w * KW + 16 * kb);
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

  TileLoader<T, DK, BMQ, NT, VECOK> ql;
  TileLoader<T, DV, BMQ, NT, VECOK> gl;
  ql.load(Qg, N, 0, tid);
  gl.load(dOg, N, 0, tid);
  ql.store(smem, LDQ, tid);
  gl.store(smem + DK * LDQ, LDQ, tid);
  load_stats<BMQ, NT>(sstats, st, N, 0, tid);
  __syncthreads();

  const int nqt = (N + BMQ - 1) / BMQ;
  for (int qt = 0; qt < nqt; ++qt) {
    const int cur = qt & 1;
    const T* Qt = smem + cur * QD_ELEMS;
    const T* Gt = Qt + DK * LDQ;
    const float2* sq = sstats + cur * BMQ;
    if (qt + 1 < nqt) {
      ql.load(Qg, N, (qt + 1) * BMQ, tid);
      gl.load(dOg, N, (qt + 1) * BMQ, tid);
    }

    f32x4 s[MBQ][KB], dp[MBQ][KB];
#pragma unroll
    for (int mb = 0; mb < MBQ; ++mb) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        s[mb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[mb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        Frag<T> a;
        if (kc == KC - 1) {
          load_tr<KSL>(a, Qt, LDQ, 32 * kc, 16 * mb);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) mma<KSL>(s[mb][kb], a, kf[kb][kc]);
        } else {
          load_tr<8>(a, Qt, LDQ, 32 * kc, 16 * mb);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) mma<8>(s[mb][kb], a, kf[kb][kc]);
        }
      }
#pragma unroll
      for (int cc = 0; cc < CC; ++cc) {
        Frag<T> a;
        if (cc == CC - 1) {
          load_tr<CSL>(a, Gt, LDQ, 32 * cc, 16 * mb);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) mma<CSL>(dp[mb][kb], a, vf[kb][cc]);
        } else {
          load_tr<8>(a, Gt, LDQ, 32 * cc, 16 * mb);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) mma<8>(dp[mb][kb], a, vf[kb][cc]);
        }
      }
      // rows of this block: queries 16*mb + 4*g + r
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float2 q = sq[16 * mb + 4 * g + r];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const float p = fast_exp2(__builtin_fmaf(s[mb][kb][r], c, -q.x));
          s[mb][kb][r] = p;
          dp[mb][kb][r] = p * (dp[mb][kb][r] - q.y);
        }
      }
    }

    // dV^T += dO^T P and dK^T += Q^T dS, contraction over this tile's queries.
#pragma unroll
    for (int qc = 0; qc < MBQ / 2; ++qc) {
      Frag<T> pf[KB], dsf[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        acc_to_frag(pf[kb], s[2 * qc][kb], s[2 * qc + 1][kb]);
        acc_to_frag(dsf[kb], dp[2 * qc][kb], dp[2 * qc + 1][kb]);
      }
#pragma unroll
      for (int cb = 0; cb < DV / 16; ++cb) {
        Frag<T> a;
        load_nat(a, Gt, LDQ, 16 * cb, 32 * qc);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) mma<8>(dvacc[cb][kb], a, pf[kb]);
      }
#pragma unroll
      for (int db = 0; db < DK / 16; ++db) {
        Frag<T> a;
        load_nat(a, Qt, LDQ, 16 * db, 32 * qc);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) mma<8>(dkacc[db][kb], a, dsf[kb]);
      }
    }

    if (qt + 1 < nqt) {
      T* nq = smem + (cur ^ 1) * QD_ELEMS;
      ql.store(nq, LDQ, tid);
      gl.store(nq + DK * LDQ, LDQ, tid);
      load_stats<BMQ, NT>(sstats + (cur ^ 1) * BMQ, st, N, (qt + 1) * BMQ, tid);
    }
    __syncthreads();
  }

#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int j = j0 + w * KW + 16 * kb + t;
    if (j < N) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int db = 0; db < DK / 16; ++db)
          dpk[((size_t)bh * C + DK + 16 * db + 4 * g + r) * N + j] = from_f32<T>(dkacc[db][kb][r] * scale);
#pragma unroll
        for (int cb = 0; cb < DV / 16; ++cb)
          dpk[((size_t)bh * C + 2 * DK + 16 * cb + 4 * g + r) * N + j] = from_f32<T>(dvacc[cb][kb][r]);
      }
    }
  }
}

// =============================================================== backward dQ
template <typename T, int DK, int DV, int QB, int NW, int BN, bool VECOK>
__global__ __launch_bounds__(NW * 64) void psa_bwd_dq_kernel(
    const T* __restrict__ qkv, const T* __restrict__ dO, const float2* __restrict__ stats,
    T* __restrict__ dpk, int N, int n_qtiles, float c, float scale) {
  constexpr int QW = 16 * QB, BM = NW * QW, NT = NW * 64;
  constexpr int KC = Chunks<DK>::n, KSL = Chunks<DK>::last;
  constexpr int CC = Chunks<DV>::n, CSL = Chunks<DV>::last;
  constexpr int MB = BN / 16;
  constexpr int LDK = BN + lds_pad<T>(), LDQ = BM + lds_pad<T>();
  constexpr int KV_ELEMS = (DK + DV) * LDK;
  constexpr int SMEM = 2 * KV_ELEMS > (DK + DV) * LDQ ? 2 * KV_ELEMS : (DK + DV) * LDQ;
  static_assert(BN % 32 == 0, "key tile must be a multiple of 32");
  __shared__ __attribute__((aligned(16))) T smem[SMEM];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, t = lane & 15;
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = blk / n_qtiles, i0 = (blk - bh * n_qtiles) * BM;
  const size_t C = 2 * DK + DV;
  const T* Qg = qkv + (size_t)bh * C * N;
  const T* KVg = Qg + (size_t)DK * N;
  const T* dOg = dO + (size_t)bh * DV * N;

  // Stationary queries: B operands of S^T = K Q^T and dP^T = V dO^T.
  Frag<T> qf[QB][KC], gf[QB][CC];
  float lse2[QB], dd[QB];
  {
    TileLoader<T, DK, BM, NT, VECOK> ql;
    TileLoader<T, DV, BM, NT, VECOK> gl;
    ql.load(Qg, N, i0, tid);
    gl.load(dOg, N, i0, tid);
    ql.store(smem, LDQ, tid);
    gl.store(smem + DK * LDQ, LDQ, tid);
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < QB; ++nb) {
      const int col = w * QW + 16 * nb;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        if (kc == KC - 1) load_tr<KSL>(qf[nb][kc], smem, LDQ, 32 * kc, col);
        else load_tr<8>(qf[nb][kc], smem, LDQ, 32 * kc, col);
      }
#pragma unroll
      for (int cc = 0; cc < CC; ++cc) {
        if (cc == CC - 1) load_tr<CSL>(gf[nb][cc], smem, LDQ, DK + 32 * cc, col);
        else load_tr<8>(gf[nb][cc], smem, LDQ, DK + 32 * cc, col);
      }
      const int i = i0 + col + t;
      const float2 q = (i < N) ? stats[(size_t)bh * N + i] : make_float2(kPosInf, 0.f);
      lse2[nb] = q.x;
      dd[nb] = q.y;
    }
    __syncthreads();
  }

  f32x4 dqacc[DK / 16][QB];
#pragma unroll
  for (int nb = 0; nb < QB; ++nb)
#pragma unroll
    for (int db = 0; db < DK / 16; ++db) dqacc[db][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  TileLoader<T, DK + DV, BN, NT, VECOK> kvl;
  kvl.load(KVg, N, 0, tid);
  kvl.store(smem, LDK, tid);
  __syncthreads();

  const int nkt = (N + BN - 1) / BN;
  for (int kt = 0; kt < nkt; ++kt) {
    const T* Kt = smem + (kt & 1) * KV_ELEMS;
    const T* Vt = Kt + DK * LDK;
    if (kt + 1 < nkt) kvl.load(KVg, N, (kt + 1) * BN, tid);
    const int j0 = kt * BN;

    f32x4 s[MB][QB], dp[MB][QB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int nb = 0; nb < QB; ++nb) {
        s[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        Frag<T> a;
        if (kc == KC - 1) {
          load_tr<KSL>(a, Kt, LDK, 32 * kc, 16 * mb);
#pragma unroll
          for (int nb = 0; nb < QB; ++nb) mma<KSL>(s[mb][nb], a, qf[nb][kc]);
        } else {
          load_tr<8>(a, Kt, LDK, 32 * kc, 16 * mb);
#pragma unroll
          for (int nb = 0; nb < QB; ++nb) mma<8>(s[mb][nb], a, qf[nb][kc]);
        }
      }
#pragma unroll
      for (int cc = 0; cc < CC; ++cc) {
        Frag<T> a;
        if (cc == CC - 1) {
          load_tr<CSL>(a, Vt, LDK, 32 * cc, 16 * mb);
#pragma unroll
          for (int nb = 0; nb < QB; ++nb) mma<CSL>(dp[mb][nb], a, gf[nb][cc]);
        } else {
          load_tr<8>(a, Vt, LDK, 32 * cc, 16 * mb);
#pragma unroll
          for (int nb = 0; nb < QB; ++nb) mma<8>(dp[mb][nb], a, gf[nb][cc]);
        }
      }
      const bool tail = j0 + BN > N;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool dead = tail && (j0 + 16 * mb + 4 * g + r >= N);
#pragma unroll
        for (int nb = 0; nb < QB; ++nb) {
          const float p = dead ? 0.f : fast_exp2(__builtin_fmaf(s[mb][nb][r], c, -lse2[nb]));
          dp[mb][nb][r] = p * (dp[mb][nb][r] - dd[nb]);
        }
      }
    }

    // dQ^T += K^T dS^T, contraction over this tile's keys.
#pragma unroll
    for (int kc2 = 0; kc2 < MB / 2; ++kc2) {
      Frag<T> dsf[QB];
#pragma unroll
      for (int nb = 0; nb < QB; ++nb) acc_to_frag(dsf[nb], dp[2 * kc2][nb], dp[2 * kc2 + 1][nb]);
#pragma unroll
      for (int db = 0; db < DK / 16; ++db) {
        Frag<T> a;
        load_nat(a, Kt, LDK, 16 * db, 32 * kc2);
#pragma unroll
        for (int nb = 0; nb < QB; ++nb) mma<8>(dqacc[db][nb], a, dsf[nb]);
      }
    }

    if (kt + 1 < nkt) kvl.store(smem + ((kt + 1) & 1) * KV_ELEMS, LDK, tid);
    __syncthreads();
  }

#pragma unroll
  for (int nb = 0; nb < QB; ++nb) {
    const int i = i0 + w * QW + 16 * nb + t;
    if (i < N) {
#pragma unroll
      for (int db = 0; db < DK / 16; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          dpk[((size_t)bh * C + 16 * db + 4 * g + r) * N + i] = from_f32<T>(dqacc[db][nb][r] * scale);
    }
  }
}

}  // namespace psa
