// The qkv 1x1-convolution's dx GEMM (Conv2dBackward page, struct
// description, in its kh = kw = 1, stride 1, g = 1 case) with large
// workgroup tiles: dx[b][ci][n] = sum_co w[co][ci] dy[b][co][n].  Both
// operands are read with transpose reads (w is [co][ci] and dy [co][n], the
// contraction index the slow one in both).
//
// psa_conv_dx_pipe_kernel (dy rows of ld tokens, a multiple of 8, of which
// the first N count; dx rows of N): 256 x 256 or 128 x 256 tiles,
// 8 waves, operands brought into LDS by direct global-to-LDS loads three
// stages ahead.  Rows of other lengths reach it through zero-padded copies
// of dy (the caller's staging).  This file is built without the option that
// holds MFMA accumulators in ordinary VGPRs (the attention kernels, which
// rescale and read theirs with VALU instructions, need it), so the
// accumulators live in AGPRs.  The epilogue writes each dx row into its part
// of a channel concatenation (see DxParts), as psa_conv_dx_kernel does.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <type_traits>

#include "psa_conv_wide.h"
#include "psa_conv_kernels.h"

namespace psa {

// LDS layout of one [32 channel][RE token] 16-bit tile filled by 1 KB direct
// loads (Q = 1024 / row bytes rows per load).  A transpose read (frag_tr's
// lane pattern) has each half-wave read 32 bytes from each of 8 rows whose
// channels share bits 1 and 4 and take all values of bits 0, 2, 3.  So rows
// that share a load differ in bit 1 or 4 (never read together), and load
// slot i starts at i * (1 KB + 32 bytes): the 8 rows of a read sit in 8
// slots with distinct i mod 8 = h(channel), i.e. on disjoint 8-bank groups.
template <typename T, int RE>
struct DmaTile {
  static constexpr int R = RE * (int)sizeof(T);  // row bytes
  static constexpr int Q = 1024 / R;              // rows per load
  static_assert(Q == 1 || Q == 2 || Q == 4, "rows of 256, 512 or 1024 bytes");
  static constexpr int NI = 32 / Q;     // loads per tile
  static constexpr int IB = 1024 + 32;  // bytes per load slot
  static constexpr int BYTES = NI * IB;
  // byte distance from channel c's row to channel c + 2's (c with bit 1 clear)
  static constexpr int HI = Q >= 2 ? R : 8 * IB;
  __device__ static __forceinline__ int h(int c) { return (c & 1) | ((c >> 1) & 6); }
  __device__ static __forceinline__ int row_off(int c) {
    const int b1 = (c >> 1) & 1, b4 = (c >> 4) & 1;
    if constexpr (Q == 4) return h(c) * IB + (b1 + 2 * b4) * R;
    else if constexpr (Q == 2) return (h(c) + 8 * b4) * IB + b1 * R;
    else return (h(c) + 8 * b1 + 16 * b4) * IB;
  }
  // channel held at row position p of load slot i
  __device__ static __forceinline__ int channel(int i, int p) {
    const int hh = i & 7, c = (hh & 1) | ((hh & 6) << 1);
    if constexpr (Q == 4) return c | ((p & 1) << 1) | ((p >> 1) << 4);
    else if constexpr (Q == 2) return c | (p << 1) | ((i >> 3) << 4);
    else return c | (((i >> 3) & 1) << 1) | ((i >> 4) << 4);
  }
};

// A fragment (frag_tr's lane pattern) from a DmaTile: transpose reads at p
// and p + hi (channels + 2).
template <typename T>
__device__ __forceinline__ void frag_lds(Frag<T>& f, const unsigned char* p, int hi) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + hi));
  f.v = __builtin_bit_cast(typename Vec8<T>::type, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
}

// The same GEMM with a BM ci x 256 n workgroup tile (BM = 256 or 128) for N
// a multiple of 8 (16-byte aligned rows): 8 waves (two per SIMD, 2 x 4), each
// BM/2 ci x 64 n.  The operand tiles come into LDS by direct loads (DmaTile
// layout, no staging registers) through a ring of 4 slots of 32 output
// channels, three stages ahead of the MFMAs.  Step k, per wave: wait for its
// own loads of stage k; one barrier (then all of stage k is in LDS and every
// wave has finished reading stage k - 1); issue the loads of stage k + 3
// into stage k - 1's slot; read stage k's fragments and run its 32 MFMAs.
template <typename T, int BM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void psa_conv_dx_pipe_kernel(const T* __restrict__ w, const T* __restrict__ dy, const DxParts<T> parts, int cin,
                             int cout, int N, int ld, int n_ntiles, int n_mtiles, int n_blocks) {
  static_assert(BM == 256 || BM == 128, "ci tile");
  constexpr int NW = 8, BN = 256, BK = 32, JN = 4;  // JN: 16-token fragments per wave
  constexpr int IA = BM / 32;                       // 16-channel fragments per wave
  using TA = DmaTile<T, BM>;
  using TB = DmaTile<T, BN>;
  constexpr int SB = TA::BYTES + TB::BYTES;                         // bytes per stage
  constexpr int AI = TA::NI / NW, BI = TB::NI / NW, L = AI + BI;  // loads per wave per stage
  __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * SB];

  const int tid = thread_id(), lane = tid & 63, g = lane >> 4, t = lane & 15, e = t >> 2;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int blk = xcd_remap(block_id(), n_blocks);
  const int per_b = n_ntiles * n_mtiles;
  const int b = blk / per_b, r = blk - b * per_b;
  const int nt = r / n_mtiles;
  const int m0 = (r - nt * n_mtiles) * BM, n0 = nt * BN;
  const T* dyb = dy + (size_t)b * cout * ld;
  const int wr = (wv & 1) * (BM / 2), wc = (wv >> 1) * 16 * JN;  // this wave's rows (ci) and columns (n)

  // This lane's source of each direct load of a stage (element offsets):
  // lane l fills the 16 bytes at 16 l of its load's 1 KB.
  int a_src[AI], b_src[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int slot = wv * AI + i, p = lane / (64 / TA::Q), x = lane % (64 / TA::Q);
    a_src[i] = TA::channel(slot, p) * cin + m0 + 8 * x;
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int slot = wv * BI + i, p = lane / (64 / TB::Q), x = lane % (64 / TB::Q);
    const int n = n0 + 8 * x;
    b_src[i] = TB::channel(slot, p) * ld + (n < N ? n : n0);  // chunks past N read a valid one; unstored columns
  }
  auto issue = [&](int kk, int slot) {
    const unsigned char* sb = smem + slot * SB;
    const T* wa = w + (size_t)kk * BK * cin;
    const T* db = dyb + (size_t)kk * BK * ld;
#pragma unroll
    for (int i = 0; i < AI; ++i) lds_dma16(wa + a_src[i], sb + (wv * AI + i) * TA::IB);
#pragma unroll
    for (int i = 0; i < BI; ++i) lds_dma16(db + b_src[i], sb + TA::BYTES + (wv * BI + i) * TB::IB);
  };
  // Fragment reads: lane (t, g) reads channel 8g + (e & 1) + 4(e >> 1) (and
  // + 2) at tokens tok0 + 4(t & 3) .. + 3; fragment i of a wave is 32 bytes
  // further along its rows.
  const int ch = 8 * g + (e & 1) + 4 * (e >> 1);
  const unsigned char* abase = smem + TA::row_off(ch) + 2 * (wr + 4 * (t & 3));
  const unsigned char* bbase = smem + TA::BYTES + TB::row_off(ch) + 2 * (wc + 4 * (t & 3));

  f32x4 acc[IA][JN];
#pragma unroll
  for (int i = 0; i < IA; ++i)
#pragma unroll
    for (int j = 0; j < JN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = cout / BK;
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  if (nk > 2) issue(2, 2);
  for (int k = 0; k < nk; ++k) {
    // this wave's loads of stage k done (those of k + 1, k + 2 may fly)
    if (k + 2 < nk)
      barrier_vmcnt<2 * L>();
    else if (k + 1 < nk)
      barrier_vmcnt<L>();
    else
      barrier_vmcnt<0>();
    // every wave is past its reads of stage k - 1: reuse that slot
    if (k + 3 < nk) issue(k + 3, (k + 3) & 3);
    const int so = (k & 3) * SB;
    Frag<T> fa[IA], fb[JN];
#pragma unroll
    for (int j = 0; j < JN; ++j) frag_lds(fb[j], bbase + so + 32 * j, TB::HI);
#pragma unroll
    for (int i = 0; i < IA; ++i) frag_lds(fa[i], abase + so + 32 * i, TA::HI);
#pragma unroll
    for (int i = 0; i < IA; ++i)
#pragma unroll
      for (int j = 0; j < JN; ++j) mma(acc[i][j], fa[i], fb[j]);
  }

  // acc[i][j]: row ci = m0 + wr + 16i + 4g + rr, column n = n0 + wc + 16j + t.
#pragma unroll
  for (int i = 0; i < IA; ++i)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int ci = m0 + wr + 16 * i + 4 * g + rr;
      T* base = parts.p[0];
      int first = 0, chn = parts.ch[0];
#pragma unroll
      for (int pq = 1; pq < kCatMaxParts; ++pq)
        if (pq < parts.n && ci >= parts.begin[pq]) {
          base = parts.p[pq];
          first = parts.begin[pq];
          chn = parts.ch[pq];
        }
      T* row = base + ((size_t)b * chn + (ci - first)) * N;
#pragma unroll
      for (int j = 0; j < JN; ++j) {
        const int n = n0 + wc + 16 * j + t;
        if (n < N) row[n] = from_f32<T>(acc[i][j][rr]);
      }
    }
}

// dw[co][ci] = sum_b sum_n dy[b][co][n] x[b][ci][n] over 128 co x 256 ci
// workgroup tiles, for rows of ld tokens (a multiple of 8; tokens in [N, ld)
// are the zeros of the caller's padded copies).  Workgroup: tile rr and
// range s of the (b, 64-token stage) sequence, cut into n_splits contiguous
// ranges as in psa_conv_dw_kernel (fp32 partials when n_splits > 1).
// 8 waves, two per SIMD: wave w computes the 128 co x 64 ci block at ci
// column 64 (w & 3) over the 32-token half (w >> 2) of every stage, so a
// wave reads 12 fragments per 32 MFMAs while the workgroup's partial stays
// the size of its tile; at the end each wave adds its partner's sums of
// half of the rows (through LDS) and writes them.  The operand tiles come
// into LDS by direct loads through a ring of 3 stage slots, two stages
// ahead.  Each 1 KB load fills 8 rows of 128 bytes, and 16-byte chunk c of
// row p holds the row's token chunk c ^ p: the 8 rows that a fragment read
// takes at one token chunk sit on 8 different 16-byte bank groups.
template <typename T>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void psa_conv_dw_pipe_kernel(const T* __restrict__ x, const T* __restrict__ dy, T* __restrict__ dw,
                             float* __restrict__ part, int cin, int cout, int ld, int n_citiles, int nchunk,
                             int n_splits, int n_blocks) {
  constexpr int BM = 128, BN = 256, BT = 64;  // co rows, ci rows, tokens per stage
  constexpr int RB = BT * (int)sizeof(T);     // bytes per row of a stage
  constexpr int RPL = 1024 / RB;              // rows per 1 KB load
  constexpr int NA = BM / RPL, NB = BN / RPL, NW = 8;
  constexpr int AI = NA / NW, BI = NB / NW, L = AI + BI;  // loads per wave per stage
  constexpr int IB = 1024, SB = (NA + NB) * IB;            // bytes per load slot, per stage
  constexpr int IA = BM / 16, JN = 4;                      // fragments per wave: co, ci
  static_assert(RPL == 8 && NA % NW == 0 && NB % NW == 0, "stage layout");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[3 * SB];
  static_assert(NW * (IA / 2) * JN * 64 * 16 <= 3 * SB, "exchange area");

  const int tid = thread_id(), lane = tid & 63, g = lane >> 4, t = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), h = wv >> 2, wq = wv & 3;
  const int blk = xcd_remap(block_id(), n_blocks);
  const int tiles = n_citiles * (cout / BM);
  const int s = blk / tiles, rr = blk - s * tiles;
  const int cot = rr / n_citiles, co0 = cot * BM, ci0 = (rr - cot * n_citiles) * BN;
  const int cps = (ld + BT - 1) / BT;  // stages per batch
  const int c0 = (int)((long long)nchunk * s / n_splits), c1 = (int)((long long)nchunk * (s + 1) / n_splits);

  // This lane's part of each load: row p = lane / 8 of the load's 8, token
  // chunk (lane % 8) ^ p; byte offsets from the tile's first row.
  const int p = lane >> 3, tokl = 8 * ((lane & 7) ^ p);
  unsigned a_row[AI], b_row[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) a_row[i] = (unsigned)((RPL * (wv * AI + i) + p) * ld) * (unsigned)sizeof(T);
#pragma unroll
  for (int i = 0; i < BI; ++i) b_row[i] = (unsigned)((RPL * (wv * BI + i) + p) * ld) * (unsigned)sizeof(T);
  auto issue = [&](int ck, int slot) {
    const int b = ck / cps, nn = (ck - b * cps) * BT;
    const T* ya = dy + ((size_t)b * cout + co0) * ld;
    const T* xb = x + ((size_t)b * cin + ci0) * ld;
    const unsigned char* sb = smem + slot * SB;
    // chunks past the row end (the batch's last stage) re-read its last
    // chunk; their fragments are zeroed before use
    const unsigned to = (unsigned)min(nn + tokl, ld - 8) * (unsigned)sizeof(T);
#pragma unroll
    for (int i = 0; i < AI; ++i) lds_dma16(ya, a_row[i] + to, sb + (wv * AI + i) * IB);
#pragma unroll
    for (int i = 0; i < BI; ++i) lds_dma16(xb, b_row[i] + to, sb + (NA + wv * BI + i) * IB);
  };
  // Fragment reads: lane (t, g) reads row 16 i + t (co) or 64 wq + 16 j + t
  // (ci) at token chunk 4 h + g of the stage; rows 16 i .. 16 i + 15 are the
  // loads 2 i and 2 i + 1.
  const int jc = 4 * h + g, pr = t & 7;
  const int rd = (t >> 3) * IB + pr * RB + 16 * (jc ^ pr);
  const unsigned char* abase = smem + rd;
  const unsigned char* bbase = smem + (NA + 8 * wq) * IB + rd;

  f32x4 acc[IA][JN];
#pragma unroll
  for (int i = 0; i < IA; ++i)
#pragma unroll
    for (int j = 0; j < JN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = c1 - c0;
  if (nk > 0) issue(c0, 0);
  if (nk > 1) issue(c0 + 1, 1);
  for (int k = 0; k < nk; ++k) {
    // this wave's loads of stage k done (those of k + 1 may fly), then
    // everyone's; every wave is past its reads of stage k - 1
    if (k + 1 < nk)
      barrier_vmcnt<L>();
    else
      barrier_vmcnt<0>();
    if (k + 2 < nk) issue(c0 + k + 2, (k + 2) % 3);
    const int so = (k % 3) * SB;
    typedef typename Vec8<T>::type V8;
    Frag<T> fa[IA], fb[JN];
#pragma unroll
    for (int j = 0; j < JN; ++j) fb[j].v = *(const V8*)(bbase + so + 2 * j * IB);
#pragma unroll
    for (int i = 0; i < IA; ++i) fa[i].v = *(const V8*)(abase + so + 2 * i * IB);
    const int ck = c0 + k, nn = (ck - (ck / cps) * cps) * BT;
    if (nn + BT > ld && nn + 8 * jc >= ld) {  // past the row end: zero
#pragma unroll
      for (int j = 0; j < JN; ++j) fb[j].v = V8{};
#pragma unroll
      for (int i = 0; i < IA; ++i) fa[i].v = V8{};
    }
#pragma unroll
    for (int i = 0; i < IA; ++i)
#pragma unroll
      for (int j = 0; j < JN; ++j) mma(acc[i][j], fa[i], fb[j]);
  }

  // Halves: wave (h, wq) keeps rows i in [4 h, 4 h + 4) and hands the other
  // four to its partner (1 - h, wq); the sum is lower half + upper half.
  // (H is a constant in each branch: an index that varies at run time
  // would put the accumulators in scratch memory.)
  constexpr int IH = IA / 2;
  f32x4* ex = (f32x4*)smem;
  auto finish = [&](auto hc) {
    constexpr int H = decltype(hc)::value;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < IH; ++i)
#pragma unroll
      for (int j = 0; j < JN; ++j) ex[(((wq * 2 + H) * IH + i) * JN + j) * 64 + lane] = acc[(1 - H) * IH + i][j];
    __syncthreads();
    // acc[i][j]: row co0 + 16 i + 4 g + q, column ci0 + 64 wq + 16 j + t.
#pragma unroll
    for (int i = 0; i < IH; ++i)
#pragma unroll
      for (int j = 0; j < JN; ++j) {
        const f32x4 o = ex[(((wq * 2 + 1 - H) * IH + i) * JN + j) * 64 + lane];
        const f32x4 v = H == 0 ? acc[i][j] + o : o + acc[IH + i][j];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const size_t e = (size_t)(co0 + 16 * (H * IH + i) + 4 * g + q) * cin + ci0 + 64 * wq + 16 * j + t;
          if (n_splits == 1)
            dw[e] = from_f32<T>(v[q]);
          else
            part[(size_t)s * cout * cin + e] = v[q];
        }
      }
  };
  if (h == 0)
    finish(std::integral_constant<int, 0>{});
  else
    finish(std::integral_constant<int, 1>{});
}

namespace {

// The pipeline needs this many workgroups (one per CU) to pay off.
// Measured (bf16, us, against the 64 x 64-wave kernel): B 4, cin 512, cout
// 1536, N 6400: 256 x 256 (200 tiles) 49-52, 128 x 256 (400) 54, small
// tiles 72-74; B 8, cin 512, cout 1024, N 1600: 256 x 256 (112 tiles) 35,
// 128 x 256 (224) 24, small tiles 30.
constexpr long long kPipe256MinBlocks = 192;
constexpr long long kPipe128MinBlocks = 128;

long long tiles(int B, int cin, int N, int bm, int bn) {
  return (long long)B * (cin / bm) * ((N + bn - 1) / bn);
}

template <typename T, int BM>
void pipe(const void* w, const void* dy, const DxParts<T>& dx, int B, int cin, int cout, int N, int ld,
          hipStream_t st) {
  const int n_mtiles = cin / BM, n_ntiles = (N + 255) / 256, blocks = B * n_mtiles * n_ntiles;
  hipLaunchKernelGGL((psa_conv_dx_pipe_kernel<T, BM>), dim3(blocks), dim3(512), 0, st, (const T*)w, (const T*)dy, dx,
                     cin, cout, N, ld, n_ntiles, n_mtiles, blocks);
}

template <typename T>
void launch(DxLarge kind, const void* w, const void* dy, const DxParts<T>& dx, int B, int cin, int cout, int N,
            int ld, hipStream_t st) {
  switch (kind) {
    case DxLarge::pipe256: pipe<T, 256>(w, dy, dx, B, cin, cout, N, ld, st); break;
    case DxLarge::pipe128: pipe<T, 128>(w, dy, dx, B, cin, cout, N, ld, st); break;
    case DxLarge::none: break;
  }
}

template <typename T>
void dw_pipe(const void* x, const void* dy, void* dw, float* part, int B, int cin, int cout, int ld, int S,
             hipStream_t st) {
  const int n_citiles = cin / 256, tiles = n_citiles * (cout / 128), blocks = tiles * S;
  const int nchunk = B * ((ld + 63) / 64);
  hipLaunchKernelGGL((psa_conv_dw_pipe_kernel<T>), dim3(blocks), dim3(512), 0, st, (const T*)x, (const T*)dy, (T*)dw,
                     part, cin, cout, ld, n_citiles, nchunk, S, blocks);
}

}  // namespace

int conv_dw_pipe_splits(int B, int cin, int cout, int ld, int cus) {
  if (ld % 8 != 0 || cin % 256 != 0 || cout % 128 != 0) return 0;
  if ((long long)256 * ld * 2 >= INT32_MAX) return 0;  // 32-bit byte offsets within a tile's rows
  const long long tiles = (long long)(cin / 256) * (cout / 128);
  const long long nchunk = (long long)B * ((ld + 63) / 64);
  // one workgroup per CU (its LDS ring takes 144 KB), each range >= 4 stages
  long long S = std::min<long long>(cus / tiles, std::min<long long>(64, nchunk / 4));
  if (S < 1 || tiles * S < (3LL * cus) / 4) return 0;  // too few workgroups to fill the CUs
  return (int)S;
}

void conv_dw_pipe_launch(const bf16* x, const bf16* dy, bf16* dw, float* part, int B, int cin, int cout, int ld,
                         int S, hipStream_t st) {
  dw_pipe<bf16>(x, dy, dw, part, B, cin, cout, ld, S, st);
}
void conv_dw_pipe_launch(const f16* x, const f16* dy, f16* dw, float* part, int B, int cin, int cout, int ld,
                         int S, hipStream_t st) {
  dw_pipe<f16>(x, dy, dw, part, B, cin, cout, ld, S, st);
}

DxLarge conv_dx_large_kind(int B, int cin, int N, int ld) {
  if (ld % 8 != 0) return DxLarge::none;  // 16-byte rows of a 16-bit type only
  if (cin % 256 == 0 && tiles(B, cin, N, 256, 256) >= kPipe256MinBlocks) return DxLarge::pipe256;
  if (tiles(B, cin, N, 128, 256) >= kPipe128MinBlocks) return DxLarge::pipe128;
  return DxLarge::none;
}

void conv_dx_large_launch(DxLarge kind, const void* w, const void* dy, const DxParts<bf16>& dx, int B, int cin,
                          int cout, int N, int ld, hipStream_t st) {
  launch<bf16>(kind, w, dy, dx, B, cin, cout, N, ld, st);
}
void conv_dx_large_launch(DxLarge kind, const void* w, const void* dy, const DxParts<f16>& dx, int B, int cin,
                          int cout, int N, int ld, hipStream_t st) {
  launch<f16>(kind, w, dy, dx, B, cin, cout, N, ld, st);
}

}  // namespace psa
