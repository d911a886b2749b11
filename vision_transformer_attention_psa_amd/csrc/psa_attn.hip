// libpsa_attn.so: C ABI for PSA self-attention forward and backward on
// MI355X (gfx950).  Argument meaning, layouts, ownership and error behaviour
// are specified in include/psa_attn.h; this file validates, picks the
// compiled instance for (dtype, dk, dv) and enqueues on the caller's stream.
#include "psa_attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "psa_conv_kernels.h"
#include "psa_conv_wide.h"
#include "psa_kernels.h"

// Device memory of psa_attn_bwd_noalloc, for callers that cannot allocate:
// one fixed array per GPU (each device that runs the library holds its own
// copy until the process ends), 16 MiB: the two fp32 statistics planes for
// up to B*heads*N = 2^21 queries.  Host code uses only the device address
// that hipGetSymbolAddress returns for it, never the array's name.
static __device__ __align__(256) unsigned char scratch[size_t(16) << 20];

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

// Tile shapes.  Wide tiles (the forward: 8 waves of 32 queries sharing one
// K/V tile, at about 126 registers, so four waves fit a SIMD; the backward:
// 4 waves of 32 keys or queries, two waves per SIMD) reuse each LDS fragment
// over more MFMAs; small sequences use 16 per wave so that the grid still
// fills 256 CUs.  (Measured: 8-wave backward workgroups were slower.)
// 16-bit fragments (bf16, fp16) take half the registers of fp32 ones and
// share one set of tiles.
constexpr int kFwdQB = 2, kFwdNW = 8;
constexpr int kFwdBN = 64;  // 128-key tiles measured 16% slower at N = 6400
constexpr int kBwdNW = 4;
constexpr int kDkdvKB = 2, kDkdvKBDk64 = 3, kDkdvBMQ = 64;
constexpr int kDqQB = 2, kDqBN = 64, kDqBNDk64 = 128;
// Forward: sequences up to this length use the narrow tiles.
constexpr int kSmallNMax = 512;
// Backward: measured at B*heads = 64 (dk 32, dv 64), the narrow tiles win up
// to N = 256 (13.3 vs 13.9 us) and the wide ones from N = 320 (16.8 vs 17.8 us;
// N = 400: 22.3 vs 24.2 us, N = 512: 24.2 vs 27.6 us).
constexpr int kSmallNMaxBwd = 256;
// Head dims with dk + dv > 128 ("wide heads") halve the per-wave register
// tiles (their accumulators and stationary fragments are twice as large)
// and the streamed LDS tiles (their rows are twice as long), so that two
// workgroups still fit one CU.
template <int DK, int DV> constexpr bool wide_heads() { return DK + DV > 128; }
// dK/dV body: query tiles prefetched two iterations ahead (the thread halves
// take turns; measured -4% at N = 400, -3% at N = 1600, -0.7% at N = 6400;
// the same for the dQ body's and the forward's key tiles measured no gain).
// It costs no registers only while one streamed Q|dO tile (4-channel x
// 8-token blocks) needs at most half of the threads.
template <int DK, int DV, int BMQ, int NW> constexpr bool deep_fits() {
  return (DK + DV) / 4 * (BMQ / 8) <= NW * 32;
}

template <typename T, int DK, int DV> struct TilesWide {  // bf16 and fp16
  static constexpr bool W = wide_heads<DK, DV>();
  // Forward at dk = 64: 4 waves of 48 queries held to three waves per SIMD
  // (172 registers otherwise) reuse each K/V fragment 1.5x as often as 8
  // waves of 32 (427-429 vs 440-441 us at N = 6400); at dk = 32 the 8-wave
  // tiles stay (67-69 vs 59 us at N = 1600).
  static constexpr bool F48 = !W && DK > 32;
  static constexpr int FWD_NW = F48 ? 4 : kFwdNW, FWD_QB = W ? 2 : (F48 ? 3 : kFwdQB),
                       FWD_BN = W ? 64 : kFwdBN, FWD_OCC = F48 ? 3 : 0;
  static constexpr int BWD_NW = kBwdNW;
  // dk = 32: 32-query dK/dV tiles bring the kernel to about 162 registers,
  // three waves per SIMD (measured 5% faster at N = 1600); dk = 64 stays at
  // two waves per SIMD either way and runs faster with 64-query tiles.
  // dk = 64: 48 keys per dK/dV wave (each streamed Q/dO fragment feeds three
  // MFMAs instead of two) at 246 registers, with the one-tile prefetch (the
  // two-deep one would need 270): 1126 vs 1168 us at N = 6400.  At dk = 32
  // the 32-key waves with the two-deep prefetch stay faster.
  static constexpr int DKDV_KB = W ? 1 : (DK <= 32 ? kDkdvKB : kDkdvKBDk64);
  static constexpr int DKDV_BMQ = W ? 32 : (DK <= 32 ? 32 : kDkdvBMQ);
  // dk = 64: 48 queries per dQ wave fit within the registers the dK/dV body
  // already needs, so the launch keeps two waves per SIMD with 1.5x the reuse
  // of each K/V fragment (measured 3% faster at N = 6400); at dk = 32 the
  // extra registers would cost a wave per SIMD.  dk = 64: 128-key dQ tiles
  // (half the barriers per key; same registers, 70 KB of LDS) measured
  // 1044 vs 1059 us at N = 6400; at dk = 32 they cost 2-6%.
  static constexpr int DQ_QB = W ? 1 : (DK <= 32 ? kDqQB : 3), DQ_BN = W ? 32 : (DK <= 32 ? kDqBN : kDqBNDk64);
  static constexpr bool DKDV_DEEP = DKDV_KB <= 2 && deep_fits<DK, DV, DKDV_BMQ, BWD_NW>();
};
template <int DK, int DV> struct TilesWide<float, DK, DV> {
  static constexpr int FWD_NW = 4, FWD_QB = 1, FWD_BN = 32, FWD_OCC = 0;
  static constexpr int BWD_NW = 4;
  static constexpr int DKDV_KB = 1, DKDV_BMQ = 32;
  static constexpr int DQ_QB = 1, DQ_BN = 32;
  static constexpr bool DKDV_DEEP = false;
};
// Narrow backward: 32-query dK/dV tiles keep the kernel at about 113
// registers and 36 KB of LDS, so four workgroups share a CU (measured 10%
// faster than 64-query tiles at two workgroups per CU, at N = 400).
template <typename T, int DK, int DV> struct TilesNarrow {  // bf16 and fp16
  static constexpr bool W = wide_heads<DK, DV>();
  static constexpr int FWD_NW = 4, FWD_QB = 1, FWD_BN = 64, FWD_OCC = 0;
  static constexpr int BWD_NW = 4;
  static constexpr int DKDV_KB = 1, DKDV_BMQ = 32;
  static constexpr int DQ_QB = 1, DQ_BN = W ? 32 : 64;
  static constexpr bool DKDV_DEEP = deep_fits<DK, DV, DKDV_BMQ, BWD_NW>();
};
template <int DK, int DV> struct TilesNarrow<float, DK, DV> : TilesWide<float, DK, DV> {};

// ------------------------------------------------------- per-kernel timing
// Slots: forward; D/LSE preprocessing; the backward GEMM launch (dK/dV and
// dQ in one grid); a reserved slot with no kernel (kept so that the slot
// numbers of the ABI stay fixed); the 1x1-conv backward's dx GEMM; its dw
// GEMM (with the split reduction); the channel-cat slice copy; the PSA merge
// forward and backward copies.
enum { K_FWD = 0, K_PRE = 1, K_MAIN = 2, K_RESERVED = 3, K_CONV_DX = 4, K_CONV_DW = 5, K_CAT = 6, K_MERGE_FWD = 7,
       K_MERGE_BWD = 8 };

struct Timing {
  std::mutex mu;
  bool on = false;
  struct Rec {
    int slot;
    hipEvent_t a, b;
  };
  std::vector<Rec> pending;
  std::vector<hipEvent_t> pool;
  double ms[PSA_TIMING_SLOTS] = {0};
  long long n[PSA_TIMING_SLOTS] = {0};

  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
Timing g_timing;

// Brackets one launch with events when timing is enabled.
struct TimedLaunch {
  int slot;
  hipStream_t st;
  hipEvent_t a = nullptr;
  TimedLaunch(int s, hipStream_t stream) : slot(s), st(stream) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (g_timing.on && (a = g_timing.get()) != nullptr && hipEventRecord(a, st) != hipSuccess) {
      g_timing.pool.push_back(a);
      a = nullptr;
    }
  }
  ~TimedLaunch() {
    if (!a) return;
    std::lock_guard<std::mutex> lk(g_timing.mu);
    hipEvent_t b = g_timing.get();
    if (b && hipEventRecord(b, st) == hipSuccess) {
      g_timing.pending.push_back({slot, a, b});
    } else {
      g_timing.pool.push_back(a);
      if (b) g_timing.pool.push_back(b);
    }
  }
};

// ------------------------------------------------------------ scratch cache
// One grow-only device buffer per (device, stream).  A buffer is only ever
// reused by later calls on the same stream, which stream order serialises;
// growing waits for the stream before releasing the old buffer.  Buffers
// live until the process ends.
struct ScratchCache {
  std::mutex mu;
  std::map<std::pair<int, hipStream_t>, std::pair<void*, size_t>> bufs;
};
ScratchCache g_scratch;

void* scratch_for(hipStream_t st, size_t bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    g_err = "library scratch: no HIP device";
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch.mu);
  auto& slot = g_scratch.bufs[{dev, st}];
  if (slot.second >= bytes) return slot.first;
  if (slot.first) {
    if (hipStreamSynchronize(st) != hipSuccess || hipFree(slot.first) != hipSuccess) {
      g_err = "library scratch: releasing the old buffer failed";
      return nullptr;
    }
    slot = {nullptr, 0};
  }
  const size_t want = bytes + bytes / 4;  // headroom against repeated growth
  void* p = nullptr;
  if (hipMalloc(&p, want) != hipSuccess || p == nullptr) {
    g_err = "library scratch: allocation of " + std::to_string(want) + " bytes failed";
    return nullptr;
  }
  slot = {p, want};
  return p;
}

constexpr size_t kStaticScratchBytes = sizeof(scratch);

// The static array's device address on device `dev`, looked up once per
// device (with that device current) and kept.
struct StaticScratch {
  std::mutex mu;
  void* ptr[64] = {nullptr};
};
StaticScratch g_static;

void* static_scratch(const char* fn, int dev) {
  std::lock_guard<std::mutex> lk(g_static.mu);
  if (g_static.ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      fail(PSA_ERR_HIP, std::string(fn) + ": hipGetSymbolAddress of the static scratch failed: " +
                            hipGetErrorString(e));
      return nullptr;
    }
    g_static.ptr[dev] = p;
  }
  return g_static.ptr[dev];
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PSA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return PSA_OK;
}

template <typename T> constexpr bool vec_ok(int N) { return N % (16 / (int)sizeof(T)) == 0; }
// The aligned attention instances (16-byte loads; for 16-bit types direct
// loads into LDS) address a slice with 32-bit element offsets, and the direct
// loads with 32-bit byte offsets from a scalar base: a slice of 2^31 bytes or
// more goes to the instances with 64-bit offsets.
template <typename T> bool aligned_ok(const psa::PackView& pv) {
  return vec_ok<T>(pv.ld) && (long long)pv.cs * pv.ld * (long long)sizeof(T) < INT32_MAX;
}

// Inputs whose rows (N tokens of a 16-bit type) are not a multiple of 8 are
// staged once into zero-padded rows of N rounded up to 8, so that the
// kernels load them with aligned 16-byte loads.  Measured (bf16, whole
// calls, about 32 K tokens x 8 heads): attention gains from N = 127 on
// (fwd 54 -> 46 us; N = 1021: 212 -> 120, bwd 583 -> 302) and loses below
// (N = 61: fwd 39.5 -> 43, the copy's launch and traffic outweigh the
// narrower loads), so attention pads from this length on; the convolution
// gradient (B x 512 x 1536 at 25.6 K tokens) gains at every N
// (N = 61: 975 -> 312 us, N = 6399: 580 -> 199) and always pads.
constexpr int kAttnPadMinN = 96;

// Row stride for a call's inputs: N, or N rounded up to 8 when N >= min_n.
int input_ld(int dtype, int N, long long rows, int min_n) {
  if (dtype == PSA_F32 || N % 8 == 0 || N < min_n) return N;
  const int ld = (N + 7) & ~7;
  if (rows * (ld / 8) / 256 >= INT32_MAX) return N;  // the copy's grid
  return ld;
}

// dst[r][0, ld) = src[r][0, n) then zeros, for `rows` rows.
int pad_rows(int dtype, const void* src, void* dst, long long rows, int n, int ld, hipStream_t st) {
  const long long chunks = rows * (ld / 8);
  const dim3 g((unsigned)((chunks + 255) / 256)), b(256);
  if (dtype == PSA_BF16)
    hipLaunchKernelGGL((psa::psa_pad_rows_kernel<psa::bf16>), g, b, 0, st, (const psa::bf16*)src, (psa::bf16*)dst,
                       rows, n, ld);
  else
    hipLaunchKernelGGL((psa::psa_pad_rows_kernel<psa::f16>), g, b, 0, st, (const psa::f16*)src, (psa::f16*)dst, rows,
                       n, ld);
  return check_launch("psa_attn input staging launch");
}

constexpr size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

template <typename T, int DK, int DV, class C>
int run_fwd(const void* qkv, void* o, float* lse, int BH, int N, float scale, psa::PackView pv, hipStream_t st) {
  constexpr int BM = C::FWD_NW * 16 * C::FWD_QB;
  const int nqt = (N + BM - 1) / BM;
  const long long grid = (long long)BH * nqt;
  if (grid > INT32_MAX) return fail(PSA_ERR_SHAPE, "psa_attn_fwd: grid too large");
  const float c = scale * psa::kLog2e;
  const dim3 g((unsigned)grid), b(C::FWD_NW * 64);
  TimedLaunch tl(K_FWD, st);
  if (aligned_ok<T>(pv))
    hipLaunchKernelGGL((psa::psa_fwd_kernel<T, DK, DV, C::FWD_QB, C::FWD_NW, C::FWD_BN, true, C::FWD_OCC>), g, b, 0, st,
                       (const T*)qkv, (T*)o, lse, N, nqt, (int)grid, c, pv);
  else
    hipLaunchKernelGGL((psa::psa_fwd_kernel<T, DK, DV, C::FWD_QB, C::FWD_NW, C::FWD_BN, false, C::FWD_OCC>), g, b, 0, st,
                       (const T*)qkv, (T*)o, lse, N, nqt, (int)grid, c, pv);
  return check_launch("psa_attn_fwd launch");
}

// stats: the two fp32 statistics planes (2 * BH * N floats), or nullptr for
// the per-stream scratch cache.
template <typename T, int DK, int DV, class C>
int run_bwd(const void* qkv, const void* o, const float* lse, const void* dO, void* dpk, int BH, int N,
            float scale, psa::PackView pv, float* stats, hipStream_t st) {
  const float c = scale * psa::kLog2e;
  const long long total = (long long)BH * N;
  constexpr int NW = C::BWD_NW;              // waves per workgroup
  constexpr int BNK = NW * 16 * C::DKDV_KB;  // keys per dK/dV workgroup
  constexpr int BMD = NW * 16 * C::DQ_QB;    // queries per dQ workgroup
  const int nkt = (N + BNK - 1) / BNK, nqt = (N + BMD - 1) / BMD;
  if ((long long)BH * (nkt + nqt) > INT32_MAX) return fail(PSA_ERR_SHAPE, "psa_attn_bwd: grid too large");
  const int nkb = BH * nkt, nqb = BH * nqt;

  if (stats == nullptr) stats = (float*)scratch_for(st, (size_t)total * 2 * sizeof(float));  // -LSE log2 e, -D
  if (stats == nullptr) return PSA_ERR_NOMEM;
  const float* nl = stats;
  const float* nd = stats + total;

  int rc;
  {
    TimedLaunch tl(K_PRE, st);
    if (vec_ok<T>(pv.ld)) {  // 16-byte token groups x 8 channel groups, 256 lanes per 256 x 16 bytes of tokens
      const long long lanes = (long long)BH * (pv.ld / (16 / (int)sizeof(T))) * 8;
      hipLaunchKernelGGL((psa::psa_bwd_pre_kernel<T, DV, true>), dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0,
                         st, (const T*)o, (const T*)dO, lse, stats, N, pv.ld, (int)total);
    } else {
      hipLaunchKernelGGL((psa::psa_bwd_pre_kernel<T, DV, false>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                         st, (const T*)o, (const T*)dO, lse, stats, N, pv.ld, (int)total);
    }
    rc = check_launch("psa_attn_bwd preprocess launch");
  }
  if (rc != PSA_OK) return rc;
  {
    TimedLaunch tl(K_MAIN, st);
    const dim3 grid((unsigned)(nkb + nqb)), block(NW * 64);
    if (aligned_ok<T>(pv))
      hipLaunchKernelGGL(
          (psa::psa_bwd_fused_kernel<T, DK, DV, C::DKDV_KB, C::DKDV_BMQ, C::DQ_QB, C::DQ_BN, NW, true, C::DKDV_DEEP>), grid, block, 0,
          st, (const T*)qkv, (const T*)dO, nl, nd, (T*)dpk, N, nkt, nqt, nkb, nqb, c, scale, pv);
    else
      hipLaunchKernelGGL(
          (psa::psa_bwd_fused_kernel<T, DK, DV, C::DKDV_KB, C::DKDV_BMQ, C::DQ_QB, C::DQ_BN, NW, false, C::DKDV_DEEP>), grid, block, 0,
          st, (const T*)qkv, (const T*)dO, nl, nd, (T*)dpk, N, nkt, nqt, nkb, nqb, c, scale, pv);
    rc = check_launch("psa_attn_bwd launch");
  }
  return rc;
}

template <typename T>
int run_conv_bwd(const void* x, const void* w, const void* dy, const psa::DxParts<T>& dx, void* dw, int B, int cin,
                 int cout, int N, int dtype, hipStream_t st) {
  constexpr int R = psa::kConvTile;
  const int n_ntiles = (N + R - 1) / R, n_citiles = cin / R, n_cotiles = cout / R;
  const long long gx = (long long)B * n_citiles * n_ntiles;
  if (gx > INT32_MAX) return fail(PSA_ERR_SHAPE, "psa_qkv_conv_bwd: grid too large");
  // Rows of x and dy in padded copies (see kAttnPadMinN): dx reads dy with
  // row stride ld and writes rows of N; dw sums over all ld tokens, the zero
  // columns adding nothing.
  const int ld = input_ld(dtype, N, (long long)B * (cin + cout), 1);
  // dw: the (b, token chunk) sum is split into S ranges so that tiles x S
  // fills the two workgroups per CU that its 74 KB of LDS allow, rounded
  // down: one more workgroup than the CUs hold would cost a second round.
  // Each range keeps >= 4 chunks.
  constexpr int BT = psa::is_16bit<T>() ? 64 : 32;
  const long long nchunk = (long long)B * ((ld + BT - 1) / BT);
  const int tiles = n_citiles * n_cotiles;
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return fail(PSA_ERR_HIP, "psa_qkv_conv_bwd: device query failed");
  long long S = (2LL * cus) / tiles;
  S = std::min<long long>(S, std::max<long long>(1, nchunk / 4));
  S = std::max<long long>(1, std::min<long long>(S, 64));
  // 16-bit types: the large-tile kernel when it applies (its own split count)
  int S_pipe = 0;
  if constexpr (psa::is_16bit<T>()) S_pipe = psa::conv_dw_pipe_splits(B, cin, cout, ld, cus);
  if (S_pipe > 0) S = S_pipe;
  // one scratch buffer: dw's fp32 partials, then the padded x and dy
  const size_t pb = S > 1 ? round256((size_t)S * cout * cin * sizeof(float)) : 0;
  const size_t xb = ld != N ? round256((size_t)B * cin * ld * sizeof(T)) : 0;
  const size_t yb = ld != N ? round256((size_t)B * cout * ld * sizeof(T)) : 0;
  float* part = nullptr;
  int rc;
  if (pb + xb + yb > 0) {
    unsigned char* base = (unsigned char*)scratch_for(st, pb + xb + yb);
    if (base == nullptr) return fail(PSA_ERR_NOMEM, std::string("psa_qkv_conv_bwd: ") + g_err);
    if (S > 1) part = (float*)base;
    if (ld != N) {
      if ((rc = pad_rows(dtype, x, base + pb, (long long)B * cin, N, ld, st)) != PSA_OK ||
          (rc = pad_rows(dtype, dy, base + pb + xb, (long long)B * cout, N, ld, st)) != PSA_OK)
        return rc;
      x = base + pb;
      dy = base + pb + xb;
    }
  }
  // 16-bit types: a large-tile kernel when the problem has enough large
  // tiles to fill the CUs; small problems keep more, smaller workgroups.
  psa::DxLarge large = psa::DxLarge::none;
  if constexpr (psa::is_16bit<T>()) large = psa::conv_dx_large_kind(B, cin, N, ld);
  {
    TimedLaunch tl(K_CONV_DX, st);
    if (large != psa::DxLarge::none) {
      if constexpr (psa::is_16bit<T>()) psa::conv_dx_large_launch(large, w, dy, dx, B, cin, cout, N, ld, st);
    } else if (vec_ok<T>(ld)) {
      hipLaunchKernelGGL((psa::psa_conv_dx_kernel<T, true>), dim3((unsigned)gx), dim3(256), 0, st, (const T*)w,
                         (const T*)dy, dx, cin, cout, N, ld, n_ntiles, n_citiles, (int)gx);
    } else {
      hipLaunchKernelGGL((psa::psa_conv_dx_kernel<T, false>), dim3((unsigned)gx), dim3(256), 0, st, (const T*)w,
                         (const T*)dy, dx, cin, cout, N, ld, n_ntiles, n_citiles, (int)gx);
    }
    rc = check_launch("psa_qkv_conv_bwd dx launch");
  }
  if (rc != PSA_OK) return rc;
  TimedLaunch tl(K_CONV_DW, st);
  const int gw = (int)(tiles * S);
  if (S_pipe > 0) {
    if constexpr (psa::is_16bit<T>())
      psa::conv_dw_pipe_launch((const T*)x, (const T*)dy, (T*)dw, part, B, cin, cout, ld, (int)S, st);
  } else if (vec_ok<T>(ld))
    hipLaunchKernelGGL((psa::psa_conv_dw_kernel<T, true>), dim3((unsigned)gw), dim3(256), 0, st, (const T*)x,
                       (const T*)dy, (T*)dw, part, B, cin, cout, ld, n_citiles, n_cotiles, (int)S, gw);
  else
    hipLaunchKernelGGL((psa::psa_conv_dw_kernel<T, false>), dim3((unsigned)gw), dim3(256), 0, st, (const T*)x,
                       (const T*)dy, (T*)dw, part, B, cin, cout, ld, n_citiles, n_cotiles, (int)S, gw);
  rc = check_launch("psa_qkv_conv_bwd dw launch");
  if (rc == PSA_OK && S > 1) {
    const long long n4 = (long long)cout * cin / 4;  // cin is a multiple of 128
    hipLaunchKernelGGL((psa::psa_conv_dw_reduce_kernel<T>), dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st,
                       (const float*)part, (T*)dw, n4, (int)S);
    rc = check_launch("psa_qkv_conv_bwd dw reduce launch");
  }
  return rc;
}

// n_parts (1 or 2) parts of n_outer runs of `run` elements; see
// psa_rows_copy_kernel.
template <typename T>
int run_rows_copy(const char* fn, int slot, const psa::RowCopy<T>& rc, int n_parts, long long run, int n_outer,
                  hipStream_t st) {
  constexpr int V = 16 / (int)sizeof(T);
  bool vec = run % V == 0;
  for (int p = 0; p < n_parts; ++p)
    vec = vec && rc.src_row[p] % V == 0 && rc.dst_row[p] % V == 0 && ((uintptr_t)rc.src[p] & 15u) == 0 &&
          ((uintptr_t)rc.dst[p] & 15u) == 0;
  const long long per_launch = 256LL * psa::kCatUnroll;
  const long long per_row = ((vec ? run / V : run) + per_launch - 1) / per_launch;
  const long long grid = per_row * n_outer * n_parts;
  if (grid > INT32_MAX) return fail(PSA_ERR_SHAPE, std::string(fn) + ": grid too large");
  // non-temporal accesses once the copy (read + write) outgrows the 256 MiB
  // last-level cache
  const bool nt = vec && 2.0 * n_parts * n_outer * run * sizeof(T) > 256.0 * (1 << 20);
  TimedLaunch tl(slot, st);
  const dim3 g((unsigned)grid), blk(256);
  if (nt)
    hipLaunchKernelGGL((psa::psa_rows_copy_kernel<T, true, true>), g, blk, 0, st, rc, run, (int)per_row, n_outer);
  else if (vec)
    hipLaunchKernelGGL((psa::psa_rows_copy_kernel<T, true, false>), g, blk, 0, st, rc, run, (int)per_row, n_outer);
  else
    hipLaunchKernelGGL((psa::psa_rows_copy_kernel<T, false, false>), g, blk, 0, st, rc, run, (int)per_row, n_outer);
  return check_launch((std::string(fn) + " launch").c_str());
}

template <typename T>
int run_channel_cat_bwd(const void* dy, void* dx, int n_outer, int chunk, int total, int offset, hipStream_t st) {
  psa::RowCopy<T> rc{};
  rc.src[0] = rc.src[1] = (const T*)dy + offset;
  rc.dst[0] = rc.dst[1] = (T*)dx;
  rc.src_row[0] = rc.src_row[1] = total;
  rc.dst_row[0] = rc.dst_row[1] = chunk;
  return run_rows_copy<T>("psa_channel_cat_bwd", K_CAT, rc, 1, chunk, n_outer, st);
}

// merged [BH, 2*half, N] <-> (lo, hi) [BH, half, N]
template <typename T>
int run_merge(bool forward, const void* a, const void* b, const void* m, int BH, int half, int N, hipStream_t st) {
  const long long run = (long long)half * N;
  psa::RowCopy<T> rc{};
  const T* lo = (const T*)a;
  const T* hi = (const T*)b;
  T* mg = (T*)m;
  if (forward) {
    rc.src[0] = lo, rc.src[1] = hi, rc.dst[0] = mg, rc.dst[1] = mg + run;
    rc.src_row[0] = rc.src_row[1] = run, rc.dst_row[0] = rc.dst_row[1] = 2 * run;
    return run_rows_copy<T>("psa_merge_fwd", K_MERGE_FWD, rc, 2, run, BH, st);
  }
  rc.src[0] = mg, rc.src[1] = mg + run, rc.dst[0] = (T*)lo, rc.dst[1] = (T*)hi;
  rc.src_row[0] = rc.src_row[1] = 2 * run, rc.dst_row[0] = rc.dst_row[1] = run;
  return run_rows_copy<T>("psa_merge_bwd", K_MERGE_BWD, rc, 2, run, BH, st);
}

// ------------------------------------------------------------ instance table
#define PSA_INSTANCES(X)   \
  X(PSA_F32, float, 16, 16)     \
  X(PSA_F32, float, 32, 32)     \
  X(PSA_F32, float, 32, 64)     \
  X(PSA_F32, float, 64, 32)     \
  X(PSA_F32, float, 64, 64)     \
  X(PSA_F32, float, 64, 128)    \
  X(PSA_F32, float, 128, 128)   \
  X(PSA_BF16, psa::bf16, 32, 32) \
  X(PSA_BF16, psa::bf16, 32, 64) \
  X(PSA_BF16, psa::bf16, 64, 32) \
  X(PSA_BF16, psa::bf16, 64, 64) \
  X(PSA_BF16, psa::bf16, 64, 128) \
  X(PSA_BF16, psa::bf16, 128, 128) \
  X(PSA_F16, psa::f16, 32, 32)   \
  X(PSA_F16, psa::f16, 32, 64)   \
  X(PSA_F16, psa::f16, 64, 32)   \
  X(PSA_F16, psa::f16, 64, 64)   \
  X(PSA_F16, psa::f16, 64, 128)  \
  X(PSA_F16, psa::f16, 128, 128)

bool supported(int dk, int dv, int dtype) {
#define X(DT, T, K, V) if (dtype == DT && dk == K && dv == V) return true;
  PSA_INSTANCES(X)
#undef X
  return false;
}

size_t elem_size(int dtype) { return dtype == PSA_F32 ? 4 : 2; }

struct Range {
  uintptr_t lo, hi;
};
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Shape/pointer validation shared by both entry points.
int validate_common(const char* fn, int B, int heads, int N, int dk, int dv, float scale, int dtype) {
  if (dtype != PSA_F32 && dtype != PSA_BF16 && dtype != PSA_F16)
    return fail(PSA_ERR_UNSUPPORTED, std::string(fn) + ": unknown dtype");
  if (B < 1 || heads < 1 || N < 1 || dk < 1 || dv < 1)
    return fail(PSA_ERR_SHAPE, std::string(fn) + ": B, heads, N, dk, dv must all be >= 1");
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(PSA_ERR_SHAPE, std::string(fn) + ": scale must be finite and > 0");
  const __int128 BH = (__int128)B * heads;
  const __int128 elems = BH * (2 * (__int128)dk + dv) * N;
  if (BH * N > INT32_MAX || elems > ((__int128)1 << 46))
    return fail(PSA_ERR_SHAPE, std::string(fn) + ": problem too large");
  if (!supported(dk, dv, dtype)) {
    char buf[160];
    snprintf(buf, sizeof buf, "%s: no compiled instance for dk=%d dv=%d dtype=%s", fn, dk, dv,
             dtype == PSA_F32 ? "f32" : dtype == PSA_BF16 ? "bf16" : "f16");
    return fail(PSA_ERR_UNSUPPORTED, buf);
  }
  return PSA_OK;
}

bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

// gfx950 is the only compiled target; refuse other devices before any launch.
// On success *dev_out is the current device.
int check_device(const char* fn, int* dev_out) {
  static std::mutex mu;
  static int known[64] = {0};  // 0 unknown, 1 ok, 2 wrong arch
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PSA_ERR_HIP, std::string(fn) + ": no HIP device");
  if (dev < 0 || dev >= 64) return fail(PSA_ERR_HIP, std::string(fn) + ": device index out of range");
  std::lock_guard<std::mutex> lk(mu);
  if (known[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return fail(PSA_ERR_HIP, std::string(fn) + ": hipGetDeviceProperties failed");
    known[dev] = std::string(prop.gcnArchName).rfind("gfx950", 0) == 0 ? 1 : 2;
  }
  if (known[dev] != 1) return fail(PSA_ERR_UNSUPPORTED, std::string(fn) + ": device is not gfx950");
  *dev_out = dev;
  return PSA_OK;
}

// One caller buffer: its name for messages, base address and extent.
struct Buf {
  const char* name;
  Range r;
};

// Every buffer must be memory the GPU can address as device memory of the
// current device (a host address handed to a kernel faults the GPU), and its
// whole extent must lie inside one allocation (an undersized buffer would be
// written past its end).  A failed query leaves HIP's last-error state
// cleared, so that the launch checks that follow see only their own errors.
int check_buffers(const char* fn, int dev, const Buf* bufs, int n) {
  for (int k = 0; k < n; ++k) {
    const Buf& b = bufs[k];
    hipPointerAttribute_t a{};
    if (hipPointerGetAttributes(&a, (const void*)b.r.lo) != hipSuccess) {
      (void)hipGetLastError();
      return fail(PSA_ERR_DEVICE, std::string(fn) + ": " + b.name + " is not device memory");
    }
    const bool managed = a.type == hipMemoryTypeManaged || a.type == hipMemoryTypeUnified || a.isManaged;
    if (!managed && a.type != hipMemoryTypeDevice)
      return fail(PSA_ERR_DEVICE, std::string(fn) + ": " + b.name + " is not device memory");
    if (!managed && a.device != dev)
      return fail(PSA_ERR_DEVICE, std::string(fn) + ": " + b.name + " is on device " + std::to_string(a.device) +
                                      ", not the current device " + std::to_string(dev));
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)b.r.lo) == hipSuccess) {
      if (b.r.hi > (uintptr_t)base + size)
        return fail(PSA_ERR_DEVICE, std::string(fn) + ": " + b.name + " extends past the end of its allocation (" +
                                        std::to_string(b.r.hi - b.r.lo) + " bytes needed, " +
                                        std::to_string((uintptr_t)base + size - b.r.lo) + " available)");
    } else {
      (void)hipGetLastError();
    }
  }
  return PSA_OK;
}

// One attention call over V rows [v0, v0 + dv) of a packed buffer with
// 2dk + dv_total channels per slice (v0 = 0, dv = dv_total: all of V).
int check_vslice(const char* fn, int dv_total, int v0, int dv) {
  if (dv_total < 1 || v0 < 0 || (long long)v0 + dv > dv_total)
    return fail(PSA_ERR_SHAPE, std::string(fn) + ": need 0 <= v0 and v0 + dv <= dv_total");
  return PSA_OK;
}

int attn_fwd_impl(const char* fn, const void* qkv, void* o, float* lse, int B, int heads, int N, int dk,
                  int dv_total, int v0, int dv, float scale, int dtype, void* stream) {
  g_err.clear();
  if (!qkv || !o || !lse) return fail(PSA_ERR_NULL, std::string(fn) + ": qkv, o and lse must be non-NULL");
  int rc = validate_common(fn, B, heads, N, dk, dv, scale, dtype);
  if (rc != PSA_OK) return rc;
  if ((rc = check_vslice(fn, dv_total, v0, dv)) != PSA_OK) return rc;
  if ((__int128)B * heads * (2 * (__int128)dk + dv_total) * N > ((__int128)1 << 46))
    return fail(PSA_ERR_SHAPE, std::string(fn) + ": problem too large");
  if (misaligned(qkv) || misaligned(o) || misaligned(lse))
    return fail(PSA_ERR_ALIGN, std::string(fn) + ": base pointers must be 16-byte aligned");
  const size_t e = elem_size(dtype), BH = (size_t)B * heads;
  const Range rq{(uintptr_t)qkv, (uintptr_t)qkv + BH * (2 * dk + dv_total) * N * e};
  const Range ro{(uintptr_t)o, (uintptr_t)o + BH * dv * N * e};
  const Range rl{(uintptr_t)lse, (uintptr_t)lse + BH * N * 4};
  if (overlap(ro, rq) || overlap(rl, rq) || overlap(ro, rl))
    return fail(PSA_ERR_ALIAS, std::string(fn) + ": o, lse and qkv must not overlap");
  int dev = 0;
  if ((rc = check_device(fn, &dev)) != PSA_OK) return rc;
  const Buf bufs[] = {{"qkv", rq}, {"o", ro}, {"lse", rl}};
  if ((rc = check_buffers(fn, dev, bufs, 3)) != PSA_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  const long long rows = (long long)BH * (2 * dk + dv_total);
  const int ld = input_ld(dtype, N, rows, kAttnPadMinN);
  const void* qin = qkv;
  if (ld != N) {
    void* q = scratch_for(st, (size_t)rows * ld * e);
    if (q == nullptr) return fail(PSA_ERR_NOMEM, std::string(fn) + ": " + g_err);
    if ((rc = pad_rows(dtype, qkv, q, rows, N, ld, st)) != PSA_OK) return rc;
    qin = q;
  }
  const psa::PackView pv{2 * dk + dv_total, 2 * dk + v0, 0, ld};
#define X(DT, T, K, V)                                                                                   \
  if (dtype == DT && dk == K && dv == V)                                                                 \
    return N <= kSmallNMax ? run_fwd<T, K, V, TilesNarrow<T, K, V>>(qin, o, lse, (int)BH, N, scale, pv, st) \
                                : run_fwd<T, K, V, TilesWide<T, K, V>>(qin, o, lse, (int)BH, N, scale, pv, st);
  PSA_INSTANCES(X)
#undef X
  return fail(PSA_ERR_UNSUPPORTED, std::string(fn) + ": no instance");
}

// noalloc: the statistics planes live in the static device array instead
// of the per-stream cache (no allocation at all).
int attn_bwd_impl(const char* fn, const void* qkv, const void* o, const float* lse, const void* dO, void* d_packed,
                  int B, int heads, int N, int dk, int dv_total, int v0, int dv, bool accum, float scale, int dtype,
                  void* stream, bool noalloc = false) {
  g_err.clear();
  if (!qkv || !o || !lse || !dO || !d_packed)
    return fail(PSA_ERR_NULL, std::string(fn) + ": qkv, o, lse, dO and d_packed must be non-NULL");
  int rc = validate_common(fn, B, heads, N, dk, dv, scale, dtype);
  if (rc != PSA_OK) return rc;
  if (noalloc && (size_t)B * heads * N * 2 * sizeof(float) > kStaticScratchBytes)
    return fail(PSA_ERR_SHAPE, std::string(fn) + ": B*heads*N = " + std::to_string((long long)B * heads * N) +
                                   " exceeds the static scratch limit of " +
                                   std::to_string(kStaticScratchBytes / (2 * sizeof(float))) + " (" +
                                   std::to_string(kStaticScratchBytes >> 20) + " MiB of statistics)");
  if ((rc = check_vslice(fn, dv_total, v0, dv)) != PSA_OK) return rc;
  if ((__int128)B * heads * (2 * (__int128)dk + dv_total) * N > ((__int128)1 << 46))
    return fail(PSA_ERR_SHAPE, std::string(fn) + ": problem too large");
  if (misaligned(qkv) || misaligned(o) || misaligned(lse) || misaligned(dO) || misaligned(d_packed))
    return fail(PSA_ERR_ALIGN, std::string(fn) + ": base pointers must be 16-byte aligned");
  const size_t e = elem_size(dtype), BH = (size_t)B * heads;
  const Range rd{(uintptr_t)d_packed, (uintptr_t)d_packed + BH * (2 * dk + dv_total) * N * e};
  const Range rq{(uintptr_t)qkv, (uintptr_t)qkv + BH * (2 * dk + dv_total) * N * e};
  const Range ro{(uintptr_t)o, (uintptr_t)o + BH * dv * N * e};
  const Range rg{(uintptr_t)dO, (uintptr_t)dO + BH * dv * N * e};
  const Range rl{(uintptr_t)lse, (uintptr_t)lse + BH * N * 4};
  if (overlap(rd, rq) || overlap(rd, ro) || overlap(rd, rg) || overlap(rd, rl))
    return fail(PSA_ERR_ALIAS, std::string(fn) + ": d_packed must not overlap any input");
  int dev = 0;
  if ((rc = check_device(fn, &dev)) != PSA_OK) return rc;
  const Buf bufs[] = {{"qkv", rq}, {"o", ro}, {"lse", rl}, {"dO", rg}, {"d_packed", rd}};
  if ((rc = check_buffers(fn, dev, bufs, 5)) != PSA_OK) return rc;
  float* stats = nullptr;
  if (noalloc && (stats = (float*)static_scratch(fn, dev)) == nullptr) return PSA_ERR_HIP;
  hipStream_t st = (hipStream_t)stream;
  const long long qrows = (long long)BH * (2 * dk + dv_total), grows = (long long)BH * dv;
  const int ld = noalloc ? N : input_ld(dtype, N, qrows, kAttnPadMinN);
  const void *qin = qkv, *oin = o, *gin = dO;
  if (ld != N) {  // statistics, then the three inputs in padded rows, in one scratch buffer
    const size_t sb = round256((size_t)BH * N * 2 * sizeof(float)), qb = round256((size_t)qrows * ld * e),
                 gb = round256((size_t)grows * ld * e);
    unsigned char* base = (unsigned char*)scratch_for(st, sb + qb + 2 * gb);
    if (base == nullptr) return fail(PSA_ERR_NOMEM, std::string(fn) + ": " + g_err);
    stats = (float*)base;
    qin = base + sb;
    oin = base + sb + qb;
    gin = base + sb + qb + gb;
    if ((rc = pad_rows(dtype, qkv, (void*)qin, qrows, N, ld, st)) != PSA_OK ||
        (rc = pad_rows(dtype, o, (void*)oin, grows, N, ld, st)) != PSA_OK ||
        (rc = pad_rows(dtype, dO, (void*)gin, grows, N, ld, st)) != PSA_OK)
      return rc;
  }
  const psa::PackView pv{2 * dk + dv_total, 2 * dk + v0, accum ? 1 : 0, ld};
#define X(DT, T, K, V)                                                                                          \
  if (dtype == DT && dk == K && dv == V)                                                                        \
    return N <= kSmallNMaxBwd                                                                                   \
               ? run_bwd<T, K, V, TilesNarrow<T, K, V>>(qin, oin, lse, gin, d_packed, (int)BH, N, scale, pv, stats, st) \
               : run_bwd<T, K, V, TilesWide<T, K, V>>(qin, oin, lse, gin, d_packed, (int)BH, N, scale, pv, stats, st);
  PSA_INSTANCES(X)
#undef X
  return fail(PSA_ERR_UNSUPPORTED, std::string(fn) + ": no instance");
}

int conv_bwd_impl(const char* fn, const void* x, const void* w, const void* dy, void* const* dx_parts,
                  const int* part_channels, int n_parts, void* dw, int B, int cin, int cout, int N, int dtype,
                  void* stream) {
  g_err.clear();
  if (!x || !w || !dy || !dw || !dx_parts || !part_channels)
    return fail(PSA_ERR_NULL, std::string(fn) + ": all pointers must be non-NULL");
  if (n_parts < 1 || n_parts > psa::kCatMaxParts)
    return fail(PSA_ERR_SHAPE, std::string(fn) + ": n_parts must be in [1, 4]");
  if (B < 1 || cin < 1 || cout < 1 || N < 1) return fail(PSA_ERR_SHAPE, std::string(fn) + ": B, cin, cout, N must be >= 1");
  if (dtype != PSA_F32 && dtype != PSA_BF16 && dtype != PSA_F16)
    return fail(PSA_ERR_UNSUPPORTED, std::string(fn) + ": unknown dtype");
  if (cin % psa::kConvTile != 0 || cout % psa::kConvTile != 0)
    return fail(PSA_ERR_UNSUPPORTED, std::string(fn) + ": cin and cout must be multiples of 128");
  const size_t e = elem_size(dtype);
  if ((size_t)B * cout * N > (size_t)INT32_MAX * 4 || (size_t)B * cin * N > (size_t)INT32_MAX * 4)
    return fail(PSA_ERR_SHAPE, std::string(fn) + ": tensors too large");
  long long csum = 0;
  for (int k = 0; k < n_parts; ++k) {
    if (!dx_parts[k]) return fail(PSA_ERR_NULL, std::string(fn) + ": all pointers must be non-NULL");
    if (part_channels[k] < 1) return fail(PSA_ERR_SHAPE, std::string(fn) + ": every part needs >= 1 channel");
    csum += part_channels[k];
  }
  if (csum != cin) return fail(PSA_ERR_SHAPE, std::string(fn) + ": part channels must add up to cin");
  if (misaligned(x) || misaligned(w) || misaligned(dy) || misaligned(dw))
    return fail(PSA_ERR_ALIGN, std::string(fn) + ": base pointers must be 16-byte aligned");
  for (int k = 0; k < n_parts; ++k)
    if (misaligned(dx_parts[k])) return fail(PSA_ERR_ALIGN, std::string(fn) + ": base pointers must be 16-byte aligned");
  const Range rx{(uintptr_t)x, (uintptr_t)x + (size_t)B * cin * N * e};
  const Range rw{(uintptr_t)w, (uintptr_t)w + (size_t)cout * cin * e};
  const Range ry{(uintptr_t)dy, (uintptr_t)dy + (size_t)B * cout * N * e};
  const Range rdw{(uintptr_t)dw, (uintptr_t)dw + (size_t)cout * cin * e};
  Range outs[psa::kCatMaxParts + 1];
  outs[0] = rdw;
  for (int k = 0; k < n_parts; ++k)
    outs[k + 1] = Range{(uintptr_t)dx_parts[k], (uintptr_t)dx_parts[k] + (size_t)B * part_channels[k] * N * e};
  for (int k = 0; k <= n_parts; ++k) {
    if (overlap(outs[k], rx) || overlap(outs[k], rw) || overlap(outs[k], ry))
      return fail(PSA_ERR_ALIAS, std::string(fn) + ": outputs must not overlap any input");
    for (int q = 0; q < k; ++q)
      if (overlap(outs[k], outs[q])) return fail(PSA_ERR_ALIAS, std::string(fn) + ": outputs must not overlap");
  }
  int rc, dev = 0;
  if ((rc = check_device(fn, &dev)) != PSA_OK) return rc;
  {
    Buf bufs[3 + 1 + psa::kCatMaxParts] = {{"x", rx}, {"w", rw}, {"dy", ry}, {"dw", rdw}};
    for (int k = 0; k < n_parts; ++k) bufs[4 + k] = Buf{"dx", outs[k + 1]};
    if ((rc = check_buffers(fn, dev, bufs, 4 + n_parts)) != PSA_OK) return rc;
  }
  hipStream_t st = (hipStream_t)stream;
  auto go = [&](auto tag) {
    using T = decltype(tag);
    psa::DxParts<T> parts{};
    int first = 0;
    for (int k = 0; k < psa::kCatMaxParts; ++k) {
      const int kk = k < n_parts ? k : n_parts - 1;  // unused slots repeat the last part
      parts.p[k] = (T*)dx_parts[kk];
      parts.begin[k] = k < n_parts ? first : parts.begin[kk];
      parts.ch[k] = part_channels[kk];
      if (k < n_parts) first += part_channels[k];
    }
    parts.n = n_parts;
    return run_conv_bwd<T>(x, w, dy, parts, dw, B, cin, cout, N, dtype, st);
  };
  if (dtype == PSA_F32) return go(float{});
  if (dtype == PSA_BF16) return go(psa::bf16{});
  return go(psa::f16{});
}

}  // namespace

extern "C" {

int psa_attn_supported(int dk, int dv, int dtype) { return supported(dk, dv, dtype) ? 1 : 0; }

const char* psa_last_error(void) { return g_err.c_str(); }

int psa_attn_version(void) { return 100; }

int psa_attn_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.on = on != 0;
  return PSA_OK;
}

int psa_attn_timing_read(double* ms, long long* launches, int n) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  int rc = PSA_OK;
  for (auto& r : g_timing.pending) {
    float t = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) {
      rc = fail(PSA_ERR_HIP, "psa_attn_timing_read: event query failed");
    } else {
      g_timing.ms[r.slot] += t;
      g_timing.n[r.slot] += 1;
    }
    g_timing.pool.push_back(r.a);
    g_timing.pool.push_back(r.b);
  }
  g_timing.pending.clear();
  for (int k = 0; k < n && k < PSA_TIMING_SLOTS; ++k) {
    if (ms) ms[k] = g_timing.ms[k];
    if (launches) launches[k] = g_timing.n[k];
  }
  return rc;
}

int psa_attn_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  for (auto& r : g_timing.pending) {
    (void)hipEventSynchronize(r.b);
    g_timing.pool.push_back(r.a);
    g_timing.pool.push_back(r.b);
  }
  g_timing.pending.clear();
  for (int k = 0; k < PSA_TIMING_SLOTS; ++k) {
    g_timing.ms[k] = 0;
    g_timing.n[k] = 0;
  }
  return PSA_OK;
}

int psa_attn_fwd(const void* qkv, void* o, float* lse, int B, int heads, int N, int dk, int dv, float scale,
                 int dtype, void* stream) {
  return attn_fwd_impl("psa_attn_fwd", qkv, o, lse, B, heads, N, dk, dv, 0, dv, scale, dtype, stream);
}

int psa_attn_bwd(const void* qkv, const void* o, const float* lse, const void* dO, void* d_packed, int B,
                 int heads, int N, int dk, int dv, float scale, int dtype, void* stream) {
  return attn_bwd_impl("psa_attn_bwd", qkv, o, lse, dO, d_packed, B, heads, N, dk, dv, 0, dv, 0, scale, dtype,
                       stream);
}

int psa_attn_bwd_noalloc(const void* qkv, const void* o, const float* lse, const void* dO, void* d_packed, int B,
                         int heads, int N, int dk, int dv, float scale, int dtype, void* stream) {
  return attn_bwd_impl("psa_attn_bwd_noalloc", qkv, o, lse, dO, d_packed, B, heads, N, dk, dv, 0, dv, 0, scale,
                       dtype, stream, true);
}

int psa_attn_fwd_vslice(const void* qkv, void* o, float* lse, int B, int heads, int N, int dk, int dv_total, int v0,
                        int dv, float scale, int dtype, void* stream) {
  return attn_fwd_impl("psa_attn_fwd_vslice", qkv, o, lse, B, heads, N, dk, dv_total, v0, dv, scale, dtype, stream);
}

int psa_attn_bwd_vslice(const void* qkv, const void* o, const float* lse, const void* dO, void* d_packed, int B,
                        int heads, int N, int dk, int dv_total, int v0, int dv, int accumulate, float scale,
                        int dtype, void* stream) {
  return attn_bwd_impl("psa_attn_bwd_vslice", qkv, o, lse, dO, d_packed, B, heads, N, dk, dv_total, v0, dv,
                       accumulate != 0, scale, dtype, stream);
}

int psa_qkv_conv_bwd(const void* x, const void* w, const void* dy, void* dx, void* dw, int B, int cin, int cout,
                     int N, int dtype, void* stream) {
  void* parts[1] = {dx};
  const int ch[1] = {cin};
  return conv_bwd_impl("psa_qkv_conv_bwd", x, w, dy, parts, ch, 1, dw, B, cin, cout, N, dtype, stream);
}

int psa_qkv_conv_cat_bwd(const void* x, const void* w, const void* dy, void* const* dx_parts,
                         const int* part_channels, int n_parts, void* dw, int B, int cin, int cout, int N, int dtype,
                         void* stream) {
  return conv_bwd_impl("psa_qkv_conv_cat_bwd", x, w, dy, dx_parts, part_channels, n_parts, dw, B, cin, cout, N,
                       dtype, stream);
}

int psa_channel_cat_bwd(const void* dy, void* dx, int n_outer, int chunk, int total, int offset, int dtype,
                        void* stream) {
  g_err.clear();
  const char* fn = "psa_channel_cat_bwd";
  if (!dy || !dx) return fail(PSA_ERR_NULL, "psa_channel_cat_bwd: dy and dx must be non-NULL");
  if (dtype != PSA_F32 && dtype != PSA_BF16 && dtype != PSA_F16)
    return fail(PSA_ERR_UNSUPPORTED, "psa_channel_cat_bwd: unknown dtype");
  if (n_outer < 1 || chunk < 1 || offset < 0 || total < 1 || (long long)offset + chunk > total)
    return fail(PSA_ERR_SHAPE, "psa_channel_cat_bwd: need n_outer, chunk >= 1, offset >= 0, offset + chunk <= total");
  if (misaligned(dy) || misaligned(dx))
    return fail(PSA_ERR_ALIGN, "psa_channel_cat_bwd: base pointers must be 16-byte aligned");
  const size_t e = elem_size(dtype);
  const Range ry{(uintptr_t)dy, (uintptr_t)dy + (size_t)n_outer * total * e};
  const Range rx{(uintptr_t)dx, (uintptr_t)dx + (size_t)n_outer * chunk * e};
  if (overlap(rx, ry)) return fail(PSA_ERR_ALIAS, "psa_channel_cat_bwd: dx must not overlap dy");
  int rc, dev = 0;
  if ((rc = check_device(fn, &dev)) != PSA_OK) return rc;
  const Buf bufs[] = {{"dy", ry}, {"dx", rx}};
  if ((rc = check_buffers(fn, dev, bufs, 2)) != PSA_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == PSA_F32) return run_channel_cat_bwd<float>(dy, dx, n_outer, chunk, total, offset, st);
  if (dtype == PSA_BF16) return run_channel_cat_bwd<psa::bf16>(dy, dx, n_outer, chunk, total, offset, st);
  return run_channel_cat_bwd<psa::f16>(dy, dx, n_outer, chunk, total, offset, st);
}

static int merge_impl(bool forward, const char* fn, const void* lo, const void* hi, const void* merged, int B,
                      int heads, int N, int half, int dtype, void* stream) {
  g_err.clear();
  if (!lo || !hi || !merged) return fail(PSA_ERR_NULL, std::string(fn) + ": all pointers must be non-NULL");
  if (dtype != PSA_F32 && dtype != PSA_BF16 && dtype != PSA_F16)
    return fail(PSA_ERR_UNSUPPORTED, std::string(fn) + ": unknown dtype");
  if (B < 1 || heads < 1 || N < 1 || half < 1)
    return fail(PSA_ERR_SHAPE, std::string(fn) + ": B, heads, N, half must be >= 1");
  if ((__int128)B * heads > INT32_MAX || (__int128)B * heads * 2 * half * N > ((__int128)1 << 46))
    return fail(PSA_ERR_SHAPE, std::string(fn) + ": problem too large");
  if (misaligned(lo) || misaligned(hi) || misaligned(merged))
    return fail(PSA_ERR_ALIGN, std::string(fn) + ": base pointers must be 16-byte aligned");
  const size_t e = elem_size(dtype), BH = (size_t)B * heads, part = BH * half * N * e;
  const Range rlo{(uintptr_t)lo, (uintptr_t)lo + part}, rhi{(uintptr_t)hi, (uintptr_t)hi + part};
  const Range rm{(uintptr_t)merged, (uintptr_t)merged + 2 * part};
  if (overlap(rlo, rhi) || overlap(rlo, rm) || overlap(rhi, rm))
    return fail(PSA_ERR_ALIAS, std::string(fn) + ": lo, hi and merged must not overlap");
  int rc, dev = 0;
  if ((rc = check_device(fn, &dev)) != PSA_OK) return rc;
  const Buf bufs[] = {{"lo", rlo}, {"hi", rhi}, {"merged", rm}};
  if ((rc = check_buffers(fn, dev, bufs, 3)) != PSA_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == PSA_F32) return run_merge<float>(forward, lo, hi, merged, (int)BH, half, N, st);
  if (dtype == PSA_BF16) return run_merge<psa::bf16>(forward, lo, hi, merged, (int)BH, half, N, st);
  return run_merge<psa::f16>(forward, lo, hi, merged, (int)BH, half, N, st);
}

int psa_merge_fwd(const void* o_lo, const void* o_hi, void* merged, int B, int heads, int N, int half, int dtype,
                  void* stream) {
  return merge_impl(true, "psa_merge_fwd", o_lo, o_hi, merged, B, heads, N, half, dtype, stream);
}

int psa_merge_bwd(const void* d_merged, void* d_lo, void* d_hi, int B, int heads, int N, int half, int dtype,
                  void* stream) {
  return merge_impl(false, "psa_merge_bwd", d_lo, d_hi, d_merged, B, heads, N, half, dtype, stream);
}

}  // extern "C"
