// Shared device building blocks for the PSA attention kernels on gfx950.
//
// Data in HBM is channel-major: each operand row is one channel and the
// tokens are contiguous.  MFMA operands are 16-row x 32-contraction chunks
// ("fragments"): lane l = row + 16*g holds 8 values, slot s carrying
// contraction index 8*g + s.  The two kinds of fragment the attention GEMMs
// need are
//   frag_ch  : rows = channels, contraction over 32 tokens.  Read straight
//              from a channel-major LDS tile ([channel][token]).
//   frag_tr  : rows = tokens, contraction over 32 channels, read from the
//              same channel-major tile with the gfx950 transpose read (16-bit
//              types, two 8-byte reads per lane); fp32 gathers it element by
//              element (frag_tok).
// frag_ch is one 16-byte LDS read per lane for 16-bit types (bf16, fp16).
//
// Chaining: a 16x16 fp32 accumulator block holds row 4*g + r of column
// (lane & 15) in register r.  Score tiles are computed over 32-token chunks
// whose rows are permuted: block h, row m <-> token 8*(m/4) + 4*h + m%4.
// Then lane (col, g) holds tokens 8g..8g+3 in block 0 and 8g+4..8g+7 in
// block 1, i.e. exactly the slots 0..7 of a fragment whose contraction runs
// over those 32 tokens, so P and dS feed the next MFMA with no data movement
// (acc_to_frag), and its partner operand is a plain frag_ch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace psa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

template <typename T> __device__ __forceinline__ float to_f32(T x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x) { return (T)x; }

// 16-bit element types (bf16, fp16) share one code path: bf16 and fp16 tiles
// have the same shapes and layouts and differ only in the MFMA and the
// conversions.
template <typename T> constexpr bool is_16bit() { return sizeof(T) == 2; }
template <typename T> struct Vec8;
template <> struct Vec8<bf16> { typedef bf16x8 type; };
template <> struct Vec8<f16> { typedef f16x8 type; };

// ---------------------------------------------------------------- fragments
template <typename T> struct Frag;
template <> struct Frag<float> { float v[8]; };
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<f16> { f16x8 v; };

__device__ __forceinline__ void mma(f32x4& c, const Frag<bf16>& a, const Frag<bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& c, const Frag<f16>& a, const Frag<f16>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& c, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], c, 0, 0, 0);
}

template <typename T> __device__ __forceinline__ Frag<T> ones_frag();
template <> __device__ __forceinline__ Frag<bf16> ones_frag<bf16>() {
  Frag<bf16> f;
  f.v = bf16x8{(bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f};
  return f;
}
template <> __device__ __forceinline__ Frag<f16> ones_frag<f16>() {
  Frag<f16> f;
  f.v = f16x8{(f16)1.f, (f16)1.f, (f16)1.f, (f16)1.f, (f16)1.f, (f16)1.f, (f16)1.f, (f16)1.f};
  return f;
}
template <> __device__ __forceinline__ Frag<float> ones_frag<float>() {
  Frag<float> f;
#pragma unroll
  for (int s = 0; s < 8; ++s) f.v[s] = 1.f;
  return f;
}

// Work-item / workgroup ids straight from the hardware registers (the
// threadIdx / blockIdx accessors go through device-library calls that are
// not inlined into code built without packed-fp32 instructions).  Kernels
// take their grid size as an argument rather than reading the dispatch
// packet, which may live in host memory.
__device__ __forceinline__ int thread_id() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ int block_id() { return (int)__builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ int lane_id() { return thread_id() & 63; }

// Token of row m (0..15) of score block h within a 32-token chunk.
__device__ __forceinline__ int perm_row(int m, int h) { return 8 * (m >> 2) + 4 * h + (m & 3); }

// Token rows, channel contraction (see frag_tok), read from a 16-bit channel-major tile
// nat[ch][token] (pitch ldn) with the gfx950 transpose read
// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives as its
// element e (of 4) the 16-bit value at position i % 4 of the 8 bytes that
// lane 4e + i/4 addressed.  So lane (t, g) addresses one channel row at the
// 4 consecutive tokens that result lanes 4(t%4) .. 4(t%4)+3 hold, and two
// reads give lane (t, g) eight channels of its token.
// The first read takes channels k0 + 8g + {0, 1, 4, 5}, the second
// {2, 3, 6, 7}, so that the four rows one read touches are spread over the
// banks (consecutive rows, 16 bytes apart within each row, meet at the same
// banks); the fragment then holds its channels in the order 0 1 4 5 2 3 6 7,
// which is harmless because both operands of every channel contraction are
// read this way.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
template <int CV, bool PERM, typename T>
__device__ __forceinline__ void frag_tr(Frag<T>& f, const T* nat, int ldn, int row0, int h, int k0) {
  static_assert(is_16bit<T>() && CV % 32 == 0, "16-bit element type, whole 32-channel chunks");
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const int lane = lane_id(), t = lane & 15, g = lane >> 4, e = t >> 2;
  const int tok = row0 + (PERM ? 8 * (t & 3) + 4 * h : 4 * (t & 3));
  const int ch = k0 + 8 * g + (e & 1) + 4 * (e >> 1);
  const T* p = nat + ch * ldn + tok;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 2 * ldn));
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  f.v = __builtin_bit_cast(typename Vec8<T>::type, v);
}

// Rows = tokens row0 + (PERM ? perm_row(lane&15, h) : lane&15); contraction
// over channels k0 .. k0+31 of a tensor with CV channels, from the
// channel-major tile nat[ch][token] (pitch ldn): transpose reads for 16-bit
// types; fp32 gathers element by element (CV % 16 == 0; the upper half of a
// chunk past CV reads as zero).
template <int CV, bool PERM, typename T>
__device__ __forceinline__ void frag_tok(Frag<T>& f, const T* nat, int ldn, int row0, int h, int k0) {
  if constexpr (is_16bit<T>()) {
    frag_tr<CV, PERM>(f, nat, ldn, row0, h, k0);
  } else {
    const int lane = lane_id(), t = lane & 15, g = lane >> 4;
    const int tok = row0 + (PERM ? perm_row(t, h) : t);
    const bool live = CV % 32 == 0 || k0 + 8 * g < CV;
    const float* p = nat + (k0 + 8 * g) * ldn + tok;
#pragma unroll
    for (int s = 0; s < 8; ++s) f.v[s] = live ? p[s * ldn] : 0.f;
  }
}

// Rows = channels ch0 .. ch0+15, contraction over tokens tok0 + 8g .. +7.
template <typename T>
__device__ __forceinline__ void frag_ch(Frag<T>& f, const T* nat, int ldn, int ch0, int tok0) {
  static_assert(is_16bit<T>(), "16-bit element type");
  const int lane = lane_id(), t = lane & 15, g = lane >> 4;
  f.v = *(const typename Vec8<T>::type*)(nat + (ch0 + t) * ldn + tok0 + 8 * g);
}
__device__ __forceinline__ void frag_ch(Frag<float>& f, const float* nat, int ldn, int ch0, int tok0) {
  const int lane = lane_id(), t = lane & 15, g = lane >> 4;
  const float* p = nat + (ch0 + t) * ldn + tok0 + 8 * g;
  const f32x4 lo = *(const f32x4*)p, hi = *(const f32x4*)(p + 4);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    f.v[s] = lo[s];
    f.v[4 + s] = hi[s];
  }
}

// Max over the four lanes l, l^16, l^32, l^48 (the four row groups holding
// one accumulator column), with the gfx950 row-swap permutes: no LDS trip.
__device__ __forceinline__ float wave_max4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Score blocks h = 0, 1 of one 32-token chunk -> B operand over those tokens.
template <typename T>
__device__ __forceinline__ void acc_to_frag(Frag<T>& f, const f32x4& a0, const f32x4& a1) {
  static_assert(is_16bit<T>(), "16-bit element type");
  f.v = typename Vec8<T>::type{(T)a0[0], (T)a0[1], (T)a0[2], (T)a0[3], (T)a1[0], (T)a1[1], (T)a1[2], (T)a1[3]};
}
__device__ __forceinline__ void acc_to_frag(Frag<float>& f, const f32x4& a0, const f32x4& a1) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    f.v[s] = a0[s];
    f.v[4 + s] = a1[s];
  }
}

// ------------------------------------------------------------------ staging
// Pitches (elements): 16 bytes of padding per row keeps every row 16-byte
// aligned and spreads the 16 rows one fragment read touches over all banks.
template <typename T> constexpr int nat_pitch(int tokens) { return tokens + 16 / (int)sizeof(T); }

// Eight consecutive 16-bit elements from p, a row position that need not be
// 16-byte aligned (rows of odd length), elements at or past
// `avail` (>= 1) read as zero.  Two aligned 16-byte loads and a byte funnel
// shift instead of eight 2-byte loads; the second load is issued only when
// it holds one of the wanted elements.  Every block read is 16-byte aligned
// and starts at or before a wanted element, so with a 16-byte aligned tensor
// base no read leaves the tensor's pages.
__device__ __forceinline__ u32x4 load8_funnel(const void* p, int avail) {
  const uintptr_t a = (uintptr_t)p;
  const u32x4* pa = (const u32x4*)(a & ~(uintptr_t)15);
  const int sh = (int)(a & 15);                  // byte offset, even
  const int nb = 2 * (avail < 8 ? avail : 8);    // bytes wanted
  const u32x4 x0 = pa[0];
  u32x4 x1 = u32x4{0u, 0u, 0u, 0u};
  if (sh + nb > 16) x1 = pa[1];
  const unsigned w[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  const int qd = sh >> 2, bs = sh & 3;           // whole dwords, then 0 or 2 bytes
  unsigned d[5];
#pragma unroll
  for (int k = 0; k < 5; ++k)
    d[k] = qd == 0 ? w[k] : qd == 1 ? w[k + 1] : qd == 2 ? w[k + 2] : w[k + 3];
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const unsigned v = __builtin_amdgcn_alignbyte(d[k + 1], d[k], bs);
    const int keep = nb - 4 * k;                 // wanted bytes of dword k
    r[k] = keep >= 4 ? v : keep == 2 ? (v & 0xffffu) : 0u;
  }
  return r;
}

// Global -> registers -> LDS for a tile of C channel rows x BT tokens from
// token j0 (tokens >= N read as zero).  Rows [0, SPLIT) come from src_lo and
// rows [SPLIT, C) from src_hi, both channel-major with row stride ld (N, or
// N rounded up to 8 for inputs staged into padded rows, whose tokens past N
// hold zeros).
// All C rows go to the channel-major tile nat[row][nat_pitch(BT)].
//   bf16, fp16: each thread owns 4-channel x 8-token blocks (four 16-byte loads).
//   fp32: 16-byte chunks (4 tokens of one row).
// VECOK: ld is a multiple of the 16-byte vector, so every chunk is aligned;
// a chunk that crosses N (padded rows only) brings the row's zero padding.
// CL (clamp, 16-byte loads only): instead of zeros, chunks past the rows'
// end repeat the row's last full chunk and lanes past the tile repeat its
// last block, so that no lane needs zeroing or a branch.  For streamed tiles
// whose tokens past N get zero weight anyway (the dK/dV body's queries,
// which carry -inf statistics); tokens that are a contraction index (the
// conv's dw) or that must be zero rows keep the default.
template <typename T, int C, int BT, int NT, bool VECOK, int SPLIT, bool CL = false>
struct Stager {  // 16-bit element types (the fp32 specialisation follows)
  static_assert(is_16bit<T>(), "16-bit element type");
  static constexpr int CG = C / 4, TC = BT / 8, NB = CG * TC, PER = (NB + NT - 1) / NT;
  static constexpr int LDN = nat_pitch<T>(BT);
  static constexpr int NAT_ELEMS = C * LDN;
  // Block q: 4 consecutive blocks run along the tokens of one 4-row group
  // (64 contiguous bytes per row in HBM), then the next row group.
  static constexpr int TCL = TC < 4 ? TC : 4;
  static_assert(TC % TCL == 0, "token chunks");
  __device__ static __forceinline__ int blk_tc(int q) { return q % TCL + TCL * (q / (TCL * CG)); }
  __device__ static __forceinline__ int blk_cg(int q) { return (q / TCL) % CG; }
  static_assert(C % 4 == 0 && BT % 8 == 0 && SPLIT % 4 == 0, "tile shape");
  u32x4 r[PER][4];

  // One 16-byte chunk (8 tokens of one row) per (u, i); W bytes per load:
  // 16 when ld is a multiple of 8 (VECOK), else (ld = N) 8 or 4 as the rows'
  // alignment allows (masked per load; a load at token j + k*W/2 < N holds
  // only tokens below N, as N is a multiple of W/2); for odd N (W = 0)
  // load8_funnel.
  // (Measured at N = 6398/6399, dk = dv = 64: 4-byte loads beat the funnel's
  // extra VALU work where they apply; 2-byte loads lose to it.)
  template <int W>
  __device__ __forceinline__ void load_w(const T* __restrict__ lo, const T* __restrict__ hi, int ld, int N, int j0,
                                         int tid) {
    constexpr int TPL = W / 2;  // tokens per load
    constexpr bool CLAMP = W == 16 && CL;  // see CL above
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q = CLAMP && NB % NT != 0 ? min(tid + u * NT, NB - 1) : tid + u * NT;
      const int tc = blk_tc(q), cg = blk_cg(q);
      const int j = j0 + 8 * tc;
      const bool live = NB % NT == 0 || q < NB;
      const T* base = 4 * cg < SPLIT ? lo + (size_t)(4 * cg) * ld : hi + (size_t)(4 * cg - SPLIT) * ld;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (CLAMP) {
          r[u][i] = *(const u32x4*)(base + (size_t)i * ld + min(j, ld - 8));
          continue;
        }
        r[u][i] = u32x4{0u, 0u, 0u, 0u};
        if (!live) continue;
        const T* p = base + (size_t)i * ld + j;
        if constexpr (W == 16) {
          if (j < N) r[u][i] = *(const u32x4*)p;
        } else if constexpr (W == 8) {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const u32x2 v = (j + TPL * e < N) ? ((const u32x2*)p)[e] : u32x2{0u, 0u};
            r[u][i][2 * e] = v[0];
            r[u][i][2 * e + 1] = v[1];
          }
        } else if constexpr (W == 4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) r[u][i][e] = (j + TPL * e < N) ? ((const unsigned*)p)[e] : 0u;
        } else {
          static_assert(W == 0, "16, 8, 4 or 0 (funnel)");
          if (j < N) r[u][i] = load8_funnel(p, N - j);
        }
      }
    }
  }
  __device__ __forceinline__ void load(const T* __restrict__ lo, const T* __restrict__ hi, int ld, int N, int j0,
                                       int tid) {
    if constexpr (VECOK) {
      load_w<16>(lo, hi, ld, N, j0, tid);
    } else if ((ld & 3) == 0) {  // one uniform branch per call, straight-line loads inside
      load_w<8>(lo, hi, ld, N, j0, tid);
    } else if ((ld & 1) == 0) {
      load_w<4>(lo, hi, ld, N, j0, tid);
    } else {
      load_w<0>(lo, hi, ld, N, j0, tid);
    }
  }
  __device__ __forceinline__ void load(const T* __restrict__ lo, const T* __restrict__ hi, int N, int j0,
                                       int tid) {
    load(lo, hi, N, N, j0, tid);
  }
  __device__ __forceinline__ void store(T* nat, int tid) const {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q = tid + u * NT;
      if (NB % NT != 0 && q >= NB) continue;
      const int tc = blk_tc(q), row = 4 * blk_cg(q);
#pragma unroll
      for (int i = 0; i < 4; ++i) *(u32x4*)(nat + (row + i) * LDN + 8 * tc) = r[u][i];
    }
  }
};

template <int C, int BT, int NT, bool VECOK, int SPLIT, bool CL>
struct Stager<float, C, BT, NT, VECOK, SPLIT, CL> {  // zero fill in every case
  static constexpr int CPR = BT / 4, CHUNKS = C * CPR, PER = (CHUNKS + NT - 1) / NT;
  static constexpr int LDN = nat_pitch<float>(BT);
  static constexpr int NAT_ELEMS = C * LDN;
  static_assert(BT % 4 == 0, "tile shape");
  f32x4 r[PER];

  __device__ __forceinline__ void load(const float* __restrict__ lo, const float* __restrict__ hi, int ld, int N,
                                       int j0, int tid) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q = tid + u * NT;
      r[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (CHUNKS % NT != 0 && q >= CHUNKS) continue;
      const int row = q / CPR, j = j0 + (q - row * CPR) * 4;
      const float* p = (row < SPLIT ? lo + (size_t)row * ld : hi + (size_t)(row - SPLIT) * ld) + j;
      if constexpr (VECOK) {
        if (j < N) r[u] = *(const f32x4*)p;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) r[u][e] = (j + e < N) ? p[e] : 0.f;
      }
    }
  }
  __device__ __forceinline__ void load(const float* __restrict__ lo, const float* __restrict__ hi, int N, int j0,
                                       int tid) {
    load(lo, hi, N, N, j0, tid);
  }
  __device__ __forceinline__ void store(float* nat, int tid) const {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q = tid + u * NT;
      if (CHUNKS % NT != 0 && q >= CHUNKS) continue;
      const int row = q / CPR, cc = q - row * CPR;
      *(f32x4*)(nat + row * LDN + cc * 4) = r[u];
    }
  }
};

// 16-byte direct global-to-LDS load: lane l's 16 bytes from g land at
// lds + 16 l (lds wave-uniform, passed in M0).  Written as inline asm so that
// the compiler does not treat the loads still in flight as pending writes to
// every later LDS read (it would wait for all of them before the first
// one); the kernel orders them itself with barrier_vmcnt.  The instruction
// has no register result, so nothing the compiler allocates is written late.
__device__ __forceinline__ void lds_dma16(const void* g, const void* lds) {
  const unsigned a = (unsigned)(size_t)(const __attribute__((address_space(3))) void*)lds;
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(a) : "memory");
}
// The same load addressed as a wave-uniform base (SGPRs) plus this lane's
// 32-bit byte offset: no per-lane 64-bit address arithmetic.  Callers keep
// the offset below 2^31, where a signed and an unsigned reading agree.
__device__ __forceinline__ void lds_dma16(const void* sbase, unsigned voff, const void* lds) {
  const unsigned a = (unsigned)(size_t)(const __attribute__((address_space(3))) void*)lds;
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(a) : "memory");
}

// Workgroup barrier once this wave's LDS reads and all but its last NV
// vector-memory operations have completed (lgkmcnt 0, vmcnt NV; gfx9
// s_waitcnt encoding, expcnt left at its maximum).  Unlike __syncthreads it
// does not wait for every load in flight; the signal fences keep the
// compiler from moving memory accesses across it.
template <int NV>
__device__ __forceinline__ void barrier_vmcnt() {
  static_assert(NV >= 0 && NV < 64, "vmcnt range");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((NV & 15) | (7 << 4) | ((NV >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Direct global-to-LDS staging of a C-row x BT-token 16-bit tile (channel
// rows, row stride ld a multiple of 8) into the layout Stager::store writes
// (row pitch nat_pitch(BT) = BT + 8 elements), with no register round trip.
// LDS slot s (16 bytes) of a stage holds token chunk s % (TC + 1) of row
// s / (TC + 1); chunk TC is the row's pad (filled from a valid address and
// never read).  Each of the NW waves owns L 1 KB loads of 64 slots (wv is
// wave-uniform) and issues those of them that exist.  Rows [0, SPLIT) start
// at element lo_off of the base pointer, rows [SPLIT, C) at hi_off, both in
// rows of ld.  A lane keeps one offset per load (its chunk at token 0); a
// tile that reaches past ld recomputes the chunk from the lane and loads
// chunks past the row's end from its last full chunk (ld - 8): finite data
// of the same row, to which the caller gives zero weight.
template <typename T, int C, int BT, int NW, int SPLIT = C>
struct DmaStage {
  static_assert(is_16bit<T>(), "16-bit element type");
  static constexpr int TC = BT / 8, SLOTS = C * (TC + 1), LOADS = (SLOTS + 63) / 64;
  static constexpr int L = (LOADS + NW - 1) / NW;  // loads per wave
  static constexpr int BYTES = LOADS * 1024;       // LDS bytes of one stage
  static constexpr int ELEMS = BYTES / (int)sizeof(T);
  static_assert(BYTES >= C * nat_pitch<T>(BT) * (int)sizeof(T), "stage holds the tile");
  unsigned off[L];  // byte offset of this lane's chunk at token 0 from the base pointer

  // First token of the chunk that slot s loads, within the tile.
  __device__ static __forceinline__ int chunk_tok(int s) {
    if (s >= SLOTS) return 0;  // past the tile: row C - 1, chunk 0
    const int c = s % (TC + 1);
    return 8 * (c == TC ? TC - 1 : c);  // the pad loads the row's last chunk
  }
  __device__ __forceinline__ void init(int wv, int lane, int lo_off, int hi_off, int ld) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int s = 64 * (wv * L + i) + lane;
      const int r = s < SLOTS ? s / (TC + 1) : C - 1;
      const int e = (r < SPLIT ? lo_off + r * ld : hi_off + (r - SPLIT) * ld) + chunk_tok(s);
      off[i] = (unsigned)e * (unsigned)sizeof(T);
    }
  }
  // Loads of the tile at token j0 into the stage at `lds`.  The callers keep
  // every tile within 2^31 bytes of `base`, so each byte offset is the same
  // read as signed or unsigned.
  __device__ __forceinline__ void issue(const T* base, int j0, int ld, const void* lds, int wv, int lane) const {
    const unsigned char* st = (const unsigned char*)lds + wv * L * 1024;
    if (j0 + BT <= ld) {  // every chunk inside the rows
      const T* tile = base + j0;
#pragma unroll
      for (int i = 0; i < L; ++i) {
        if (LOADS % NW != 0 && wv * L + i >= LOADS) break;
        lds_dma16(tile, off[i], st + i * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < L; ++i) {
        if (LOADS % NW != 0 && wv * L + i >= LOADS) break;
        const int tok = chunk_tok(64 * (wv * L + i) + lane);
        const long long d = (long long)(min(j0 + tok, ld - 8) - tok) * (long long)sizeof(T);
        lds_dma16((const unsigned char*)base + off[i] + d, st + i * 1024);
      }
    }
  }
};

// Workgroups are dispatched round-robin over the 8 XCDs (id % 8).  Remap so
// that consecutive logical ids (tiles of one (batch, head) slice, which share
// K/V or Q/dO) run on the same XCD and share its L2.  Bijective for any n.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int x = b & 7, q = n >> 3, rem = n & 7;
  return x * q + (x < rem ? x : rem) + (b >> 3);
}

}  // namespace psa
