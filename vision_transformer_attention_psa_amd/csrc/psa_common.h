// Shared device building blocks for the PSA attention kernels on gfx950.
//
// Data in HBM is channel-major: every operand row is one channel and the
// tokens are contiguous.  Tiles are staged into LDS in that same natural
// layout ([channel][token], padded rows) and MFMA operands are read from it
// in two ways:
//   load_nat : MFMA row = channel, contraction over tokens (two 8/16-byte
//              reads per lane, straight from the natural layout)
//   load_tr  : MFMA row = token, contraction over channels.  bf16 uses the
//              gfx950 LDS transpose read (ds_read_b64_tr_b16); fp32 reads
//              one element per contraction slot.
// Both produce the same fragment shape: a 16-row x 32-contraction chunk in
// which lane l = row + 16*g holds 8 values and slot s carries contraction
// index kmap(g, s) = 16*(s/4) + 4*g + (s%4).  That ordering is exactly how a
// 16x16 fp32 accumulator block holds its rows (lane col + 16*g, register r ->
// row 4*g + r), so two stacked accumulator blocks convert to a B operand
// without any data movement across lanes (acc_to_frag).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace psa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

template <typename T> __device__ __forceinline__ float to_f32(T x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x) { return (T)x; }

// ---------------------------------------------------------------- fragments
template <typename T> struct Frag;
template <> struct Frag<float> { float v[8]; };
template <> struct Frag<bf16> { bf16x8 v; };

// c += a * b over one 32-wide contraction chunk; KS = slots carrying data
// (8, or 4 when the contraction dimension ends 16 into the chunk).
template <int KS>
__device__ __forceinline__ void mma(f32x4& c, const Frag<bf16>& a, const Frag<bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
template <int KS>
__device__ __forceinline__ void mma(f32x4& c, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int s = 0; s < KS; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], c, 0, 0, 0);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// MFMA rows = tokens col0..col0+15 of the tile, contraction = tile rows
// k0..k0+31 (channels).
template <int KS>
__device__ __forceinline__ void load_tr(Frag<bf16>& f, const bf16* tile, int ld, int k0, int col0) {
  const int lane = lane_id(), t = lane & 15, g = lane >> 4;
  // Each 16-lane group reads a 4 (row) x 16 (token) block; lane t supplies
  // the 4 tokens 4*(t%4).. of row t/4 and receives token t of all 4 rows.
  const bf16* p = tile + (k0 + 4 * g + (t >> 2)) * ld + col0 + 4 * (t & 3);
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  i16x4 hi = {0, 0, 0, 0};
  if constexpr (KS == 8) hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 16 * ld));
  i16x8 r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  f.v = __builtin_bit_cast(bf16x8, r);
}
template <int KS>
__device__ __forceinline__ void load_tr(Frag<float>& f, const float* tile, int ld, int k0, int col0) {
  const int lane = lane_id(), t = lane & 15, g = lane >> 4;
  const float* p = tile + (k0 + 4 * g) * ld + col0 + t;
#pragma unroll
  for (int s = 0; s < 8; ++s) f.v[s] = s < KS ? p[(16 * (s >> 2) + (s & 3)) * ld] : 0.f;
}

// MFMA rows = tile rows row0..row0+15 (channels), contraction = tokens
// col0..col0+31.
__device__ __forceinline__ void load_nat(Frag<bf16>& f, const bf16* tile, int ld, int row0, int col0) {
  const int lane = lane_id(), t = lane & 15, g = lane >> 4;
  const bf16* p = tile + (row0 + t) * ld + col0 + 4 * g;
  bf16x4 lo = *(const bf16x4*)p;
  bf16x4 hi = *(const bf16x4*)(p + 16);
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void load_nat(Frag<float>& f, const float* tile, int ld, int row0, int col0) {
  const int lane = lane_id(), t = lane & 15, g = lane >> 4;
  const float* p = tile + (row0 + t) * ld + col0 + 4 * g;
  f32x4 lo = *(const f32x4*)p;
  f32x4 hi = *(const f32x4*)(p + 16);
#pragma unroll
  for (int s = 0; s < 4; ++s) { f.v[s] = lo[s]; f.v[4 + s] = hi[s]; }
}

// Two vertically stacked 16x16 accumulator blocks (rows 0-15 in a0, 16-31 in
// a1) as a B operand whose contraction index is the accumulator row.
__device__ __forceinline__ void acc_to_frag(Frag<bf16>& f, const f32x4& a0, const f32x4& a1) {
  f.v = bf16x8{(bf16)a0[0], (bf16)a0[1], (bf16)a0[2], (bf16)a0[3],
               (bf16)a1[0], (bf16)a1[1], (bf16)a1[2], (bf16)a1[3]};
}
__device__ __forceinline__ void acc_to_frag(Frag<float>& f, const f32x4& a0, const f32x4& a1) {
#pragma unroll
  for (int s = 0; s < 4; ++s) { f.v[s] = a0[s]; f.v[4 + s] = a1[s]; }
}

// ------------------------------------------------------------- tile loader
// Rows [0, R) x tokens [j0, j0 + BC) of a channel-major slice (row stride N
// elements) -> registers -> LDS tile [R][ld].  Tokens >= N read as zero.
// VECOK: N is a multiple of the 16-byte vector width, so every 16-byte chunk
// is aligned and either wholly inside or wholly past the row end.
template <typename T, int R, int BC, int NT, bool VECOK>
struct TileLoader {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int CPR = BC / VEC;
  static constexpr int CHUNKS = R * CPR;
  static constexpr int PER = (CHUNKS + NT - 1) / NT;
  static_assert(BC % VEC == 0, "tile width must be a whole number of 16-byte chunks");
  uint4 reg[PER];

  __device__ __forceinline__ void load(const T* __restrict__ src, int N, int j0, int tid) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q = tid + u * NT;
      reg[u] = make_uint4(0, 0, 0, 0);
      if (CHUNKS % NT != 0 && q >= CHUNKS) continue;
      const int row = q / CPR, j = j0 + (q - row * CPR) * VEC;
      const T* p = src + (size_t)row * N + j;
      if constexpr (VECOK) {
        if (j < N) reg[u] = *(const uint4*)p;
      } else {
        T tmp[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) tmp[e] = (j + e < N) ? p[e] : (T)0.f;
        __builtin_memcpy(&reg[u], tmp, 16);
      }
    }
  }
  __device__ __forceinline__ void store(T* tile, int ld, int tid) const {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q = tid + u * NT;
      if (CHUNKS % NT != 0 && q >= CHUNKS) continue;
      const int row = q / CPR, cc = q - row * CPR;
      *(uint4*)(tile + row * ld + cc * VEC) = reg[u];
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
