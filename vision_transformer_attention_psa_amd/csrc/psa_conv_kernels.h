// Backward of the 1x1 convolution that produces the packed projection qkv
// from the block input x (Conv2dBackward page, struct description, in its
// kh = kw = 1, stride 1, no padding, g = 1 case).  Per batch b:
//   y[co][n]  = sum_ci w[co][ci] x[ci][n]              (the forward, not built)
//   dx[ci][n] = sum_co w[co][ci] dy[co][n]              (psa_conv_dx_kernel)
//   dw[co][ci] = sum_b sum_n dy[co][n] x[ci][n]         (psa_conv_dw_kernel)
// dy is the packed gradient [B, heads*(2dk+dv), N] that psa_attn_bwd writes.
// The page accumulates both with atomics into zeroed buffers; here every
// output element is written once, dw's sum over b and n is split into S
// fixed ranges whose fp32 partials a third kernel adds in range order, so
// the results are deterministic.
//
// Both GEMMs run on MFMA with 4 waves per workgroup, each owning a 64 x 64
// output tile (2 x 2 waves: 128 x 128 per workgroup).
//   dx: contraction over co, which is the slow index of both w and dy: both
//       tiles are staged channel-major (rows co) and read as token rows
//       (frag_tok: the transpose read for 16-bit types).
//   dw: contraction over n, the fast index of both dy and x: both tiles are
//       channel-major and read with frag_ch, as the attention's dV/dK GEMMs.
#pragma once
#include <type_traits>

#include "psa_common.h"

namespace psa {

constexpr int kConvTile = 128;  // output rows and columns per workgroup

// ------------------------------------------------------------------- dx
// Workgroup: batch b, ci tile [ci0, ci0 + 128), token tile [n0, n0 + 128).
// dy rows are ld >= N tokens apart (columns N .. ld - 1 zero, or ld = N);
// dx rows are N tokens long.
// co is consumed in chunks of KCH (64, fp32: 32) through a double-buffered
// pair of channel-major tiles holding w [KCH co][128 ci] and dy [KCH co][128 n].
//
// Channel-cat fold (ChannelCatBackward page, struct description): when x is
// the channel concatenation of up to kCatMaxParts inputs, x = cat(x_0, ...),
// the gradient of input k is rows [begin_k, begin_k + ch_k) of dx.  The
// epilogue writes each row straight into its input's own [B, ch_k, N]
// buffer instead of materialising dx and slicing it afterwards.  A plain dx
// is the one-part case.
constexpr int kCatMaxParts = 4;
template <typename T>
struct DxParts {
  T* p[kCatMaxParts];
  int begin[kCatMaxParts];  // first channel of each part, ascending; begin[0] = 0
  int ch[kCatMaxParts];     // channels of each part
  int n;                    // parts in use, 1..kCatMaxParts
};

template <typename T, bool VECOK>
__global__ __launch_bounds__(256) void psa_conv_dx_kernel(const T* __restrict__ w, const T* __restrict__ dy,
                                                          const DxParts<T> parts, int cin, int cout, int N,
                                                          int ld, int n_ntiles, int n_citiles, int n_blocks) {
  constexpr int KCH = is_16bit<T>() ? 64 : 32, BT = kConvTile, NT = 256;  // fp32 tiles are twice as wide
  constexpr int KC = KCH / 32;
  // rows = co (channels of the chunk), tokens = ci (w) or n (dy)
  using SW = Stager<T, KCH, BT, NT, true, KCH>;
  using SY = Stager<T, KCH, BT, NT, VECOK, KCH>;
  constexpr int BUF = SW::NAT_ELEMS;  // one operand tile
  __shared__ __attribute__((aligned(16))) T smem[4 * BUF];

  const int tid = thread_id(), wv = tid >> 6, lane = tid & 63, g = lane >> 4, t = lane & 15;
  // ci tiles innermost: the workgroups that read one dy tile are
  // consecutive, so they run together on one XCD and share it through L2.
  const int blk = xcd_remap(block_id(), n_blocks);
  const int per_b = n_ntiles * n_citiles;
  const int b = blk / per_b, r = blk - b * per_b;
  const int nt = r / n_citiles;
  const int ci0 = (r - nt * n_citiles) * BT, n0 = nt * BT;
  const T* dyb = dy + (size_t)b * cout * ld;
  const int wr = (wv >> 1) * 64, wc = (wv & 1) * 64;  // this wave's rows (ci) and columns (n)

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  SW sw;
  SY sy;
  auto stage = [&](int slot) {
    T* a = smem + slot * 2 * BUF;
    T* y = a + BUF;
    sw.store(a, tid);
    sy.store(y, tid);
  };
  sw.load(w, w, cin, ci0, tid);
  sy.load(dyb, dyb, ld, n0, tid);
  stage(0);
  __syncthreads();

  const int nch = cout / KCH;
  for (int k = 0; k < nch; ++k) {
    const T* a = smem + (k & 1) * 2 * BUF;
    const T* y = a + BUF;
    if (k + 1 < nch) {
      sw.load(w + (size_t)(k + 1) * KCH * cin, w + (size_t)(k + 1) * KCH * cin, cin, ci0, tid);
      sy.load(dyb + (size_t)(k + 1) * KCH * ld, dyb + (size_t)(k + 1) * KCH * ld, ld, n0, tid);
    }
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      Frag<T> fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) frag_tok<KCH, false>(fa[i], a, SW::LDN, wr + 16 * i, 0, 32 * kc);
#pragma unroll
      for (int j = 0; j < 4; ++j) frag_tok<KCH, false>(fb[j], y, SY::LDN, wc + 16 * j, 0, 32 * kc);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mma(acc[i][j], fa[i], fb[j]);
    }
    if (k + 1 < nch) stage((k + 1) & 1);
    __syncthreads();
  }

  // acc[i][j]: rows ci0 + wr + 16i + 4g + r, column n0 + wc + 16j + t.
  // Each row's part is picked with selects (no dynamic index into the
  // kernel-argument struct).
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int ci = ci0 + wr + 16 * i + 4 * g + rr;
      T* base = parts.p[0];
      int first = 0, ch = parts.ch[0];
#pragma unroll
      for (int q = 1; q < kCatMaxParts; ++q)
        if (q < parts.n && ci >= parts.begin[q]) {
          base = parts.p[q];
          first = parts.begin[q];
          ch = parts.ch[q];
        }
      T* row = base + ((size_t)b * ch + (ci - first)) * N;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + wc + 16 * j + t;
        if (n < N) row[n] = from_f32<T>(acc[i][j][rr]);
      }
    }
}

// ------------------------------------------------------------------- dw
// Workgroup: co tile [co0, co0 + 128), ci tile [ci0, ci0 + 128), and range
// s of the token chunks: the B * ceil(N / BT) chunks (b-major) are cut into
// n_splits contiguous ranges.  Tiles: dy [128 co][BT n] and x [128 ci][BT n],
// channel-major (BT = 64 tokens, 32 for fp32).  With n_splits == 1 the result goes to dw in the storage
// type, otherwise to part[s] in fp32.
template <typename T, bool VECOK>
__global__ __launch_bounds__(256) void psa_conv_dw_kernel(const T* __restrict__ x, const T* __restrict__ dy,
                                                          T* __restrict__ dw, float* __restrict__ part, int B,
                                                          int cin, int cout, int N, int n_citiles, int n_cotiles,
                                                          int n_splits, int n_blocks) {
  constexpr int BT = is_16bit<T>() ? 64 : 32, R = kConvTile, NT = 256;
  using ST = Stager<T, R, BT, NT, VECOK, R>;
  constexpr int BUF = ST::NAT_ELEMS;
  __shared__ __attribute__((aligned(16))) T smem[4 * BUF];

  const int tid = thread_id(), wv = tid >> 6, lane = tid & 63, g = lane >> 4, t = lane & 15;
  const int blk = xcd_remap(block_id(), n_blocks);
  const int tiles = n_citiles * n_cotiles;
  const int s = blk / tiles, rr0 = blk - s * tiles;
  const int co0 = (rr0 / n_citiles) * R, ci0 = (rr0 - (rr0 / n_citiles) * n_citiles) * R;
  const int cpb = (N + BT - 1) / BT, nchunk = B * cpb;
  const int c0 = (int)((long long)nchunk * s / n_splits), c1 = (int)((long long)nchunk * (s + 1) / n_splits);
  const int wr = (wv >> 1) * 64, wc = (wv & 1) * 64;  // this wave's rows (co) and columns (ci)

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  ST sa, sb;
  auto load = [&](int ck) {
    const int b = ck / cpb, nn = (ck - b * cpb) * BT;
    const T* yb = dy + ((size_t)b * cout + co0) * N;
    const T* xb = x + ((size_t)b * cin + ci0) * N;
    sa.load(yb, yb, N, nn, tid);
    sb.load(xb, xb, N, nn, tid);
  };
  auto stage = [&](int slot) {
    T* a = smem + slot * 2 * BUF;
    sa.store(a, tid);
    sb.store(a + BUF, tid);
  };
  if (c0 < c1) {
    load(c0);
    stage(0);
  }
  __syncthreads();
  for (int ck = c0; ck < c1; ++ck) {
    const T* a = smem + ((ck - c0) & 1) * 2 * BUF;
    const T* xt = a + BUF;
    if (ck + 1 < c1) load(ck + 1);
#pragma unroll
    for (int kc = 0; kc < BT / 32; ++kc) {
      Frag<T> fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) frag_ch(fa[i], a, ST::LDN, wr + 16 * i, 32 * kc);
#pragma unroll
      for (int j = 0; j < 4; ++j) frag_ch(fb[j], xt, ST::LDN, wc + 16 * j, 32 * kc);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mma(acc[i][j], fa[i], fb[j]);
    }
    if (ck + 1 < c1) stage((ck + 1 - c0) & 1);
    __syncthreads();
  }

  // acc[i][j]: row co0 + wr + 16i + 4g + r, column ci0 + wc + 16j + t.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const size_t e = (size_t)(co0 + wr + 16 * i + 4 * g + q) * cin + ci0 + wc + 16 * j + t;
        if (n_splits == 1) dw[e] = from_f32<T>(acc[i][j][q]);
        else part[(size_t)s * cout * cin + e] = acc[i][j][q];
      }
}

// dw = sum over s of part[s], in s order; n4 = cout * cin / 4 (cin is a
// multiple of 128), four consecutive elements per thread.
template <typename T>
__global__ __launch_bounds__(256) void psa_conv_dw_reduce_kernel(const float* __restrict__ part, T* __restrict__ dw,
                                                                 long long n4, int n_splits) {
  const long long i = (long long)block_id() * 256 + thread_id();
  if (i >= n4) return;
  const f32x4* p = (const f32x4*)part + i;
  f32x4 v = p[0];
  for (int s = 1; s < n_splits; ++s) v += p[(size_t)s * n4];
#pragma unroll
  for (int q = 0; q < 4; ++q) dw[4 * i + q] = from_f32<T>(v[q]);
}

// ------------------------------------------------------------ row copies
// Channel concatenation and its backward move whole channel ranges, which
// in a [n][channels][tokens] tensor are contiguous runs: for every outer
// index n (batch, or batch x head) one run of `run` elements per part,
//   dst_p[n * dst_row_p + e] = src_p[n * src_row_p + e],   e < run,
// with any channel offset folded into the part's base pointers.
//   channel-cat backward (ChannelCatBackward page, struct description):
//     one part, src = dy + offset, src_row = total, dst_row = chunk;
//   PSA merge forward / backward (PsaMergeAttnRuntimeOp page): two parts,
//     the lo and hi halves of each head's channels.
// Workgroup blk: part p = blk / (per_row * n_outer), then run n and segment
// (256 * kCatUnroll vectors) of it; 16-byte vectors when every row length
// and base offset allows, else single elements.
constexpr int kCatUnroll = 2;  // vectors (or elements) per thread (swept 1-16)

template <typename T>
struct RowCopy {
  const T* src[2];
  T* dst[2];
  long long src_row[2], dst_row[2];
};

// NT: non-temporal loads and stores, for copies too large to stay in the
// last-level cache, where they measured faster; smaller copies measured
// faster with ordinary accesses.
template <typename T, bool VEC, bool NT>
__global__ __launch_bounds__(256) void psa_rows_copy_kernel(const RowCopy<T> rc, long long run, int per_row,
                                                            int n_outer) {
  constexpr int V = VEC ? 16 / (int)sizeof(T) : 1;
  typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
  using Vec = typename std::conditional<VEC, u32x4v, T>::type;
  const int per_part = per_row * n_outer;
  const int blk0 = block_id();
  const bool p1 = blk0 >= per_part;  // uniform: selects, no indexing into the argument struct
  const int blk = p1 ? blk0 - per_part : blk0;
  const int n = blk / per_row, seg = blk - n * per_row;
  const T* sbase = p1 ? rc.src[1] : rc.src[0];
  T* dbase = p1 ? rc.dst[1] : rc.dst[0];
  const long long srow = p1 ? rc.src_row[1] : rc.src_row[0], drow = p1 ? rc.dst_row[1] : rc.dst_row[0];
  const Vec* src = (const Vec*)(sbase + (size_t)n * srow);
  Vec* dst = (Vec*)(dbase + (size_t)n * drow);
  const long long nv = run / V, k0 = (long long)seg * 256 * kCatUnroll + thread_id();
  Vec r[kCatUnroll];
#pragma unroll
  for (int u = 0; u < kCatUnroll; ++u)
    if (k0 + u * 256 < nv) {
      if constexpr (NT)
        r[u] = __builtin_nontemporal_load(src + k0 + u * 256);
      else
        r[u] = src[k0 + u * 256];
    }
#pragma unroll
  for (int u = 0; u < kCatUnroll; ++u)
    if (k0 + u * 256 < nv) {
      if constexpr (NT)
        __builtin_nontemporal_store(r[u], dst + k0 + u * 256);
      else
        dst[k0 + u * 256] = r[u];
    }
}

}  // namespace psa
