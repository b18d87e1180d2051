// Shared device-side building blocks for the gfx950 attention kernels:
// vector types, the bf16 matrix-core product, conversions and the
// global -> LDS tile stager.
//
// Matrix-core product used throughout: v_mfma_f32_32x32x16_bf16, one wave
// (64 lanes) computes D[32x32] += A[32x16] * B[16x32].  With lane = 32*g + c
// (c in 0..31, g in 0..1):
//   A operand: lane holds A[m = c][k = kmap(g, j)], j = 0..7
//   B operand: lane holds B[k = kmap(g, j)][n = c], j = 0..7
//   D result : lane holds D[m = 8*(r/4) + 4*g + r%4][n = c], r = 0..15
// A product sums over k, so any mapping kmap that is the same for A and B
// gives the same result; the kernels pick, per product, the mapping under
// which an operand produced by an earlier product (scores, probabilities)
// is already in place in the registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gptattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// Two floats -> two bf16 (round to nearest even), packed in one dword.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Eight floats (an MFMA operand's worth) -> bf16x8.
__device__ __forceinline__ bf16x8 pack_bf16x8(const float* p) {
  u32x4 u = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
             pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// 16-byte LDS/global read as an MFMA operand.
__device__ __forceinline__ bf16x8 ld_frag16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// Operand whose eight k-values sit in two runs of four, 8 elements apart
// (the pattern of a result tile's rows r = 0..7 for one lane half).
__device__ __forceinline__ bf16x8 ld_frag_split(const uint16_t* p) {
  u32x2 lo = *reinterpret_cast<const u32x2*>(p);
  u32x2 hi = *reinterpret_cast<const u32x2*>(p + 8);
  u32x4 u = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, u);
}

// ---------------------------------------------------------------------------
// Global -> LDS staging of a ROWS x D bf16 tile (row-major in HBM, D
// contiguous).  The tile is cut into 4x4 micro-blocks; thread t of NT owns
// micro-blocks t, t + NT, ...  Consecutive threads take consecutive column
// quads of the same row quad, so each wave's global reads cover whole rows.
// The tile can be written to LDS row-major ([row][col], leading dimension
// ld) and/or transposed ([col][row]); the transpose is a 4x4 register
// shuffle of 16-bit values followed by 8-byte LDS writes.
// Rows at or beyond `valid` read as zero.
// ---------------------------------------------------------------------------
template <int ROWS, int D, int NT>
struct TileStage {
  static constexpr int CQ = D / 4;             // column quads per row
  static constexpr int MB = ROWS * D / 16;     // micro-blocks in the tile
  static constexpr int PER = MB / NT;          // micro-blocks per thread
  static_assert(MB % NT == 0, "tile must split evenly over the threads");
  u32x2 r[PER][4];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int valid, int tid) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int mb = tid + p * NT;
      const int cq = mb % CQ, rq = mb / CQ;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * rq + i;
        if (row < valid) {
          r[p][i] = *reinterpret_cast<const u32x2*>(src + (size_t)row * D + 4 * cq);
        } else {
          r[p][i] = u32x2{0u, 0u};
        }
      }
    }
  }

  __device__ __forceinline__ void store_rowmajor(uint16_t* dst, int ld, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int mb = tid + p * NT;
      const int cq = mb % CQ, rq = mb / CQ;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x2*>(dst + (4 * rq + i) * ld + 4 * cq) = r[p][i];
    }
  }

  __device__ __forceinline__ void store_transposed(uint16_t* dst, int ld, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int mb = tid + p * NT;
      const int cq = mb % CQ, rq = mb / CQ;
      const u32x2* a = r[p];
      // column j of the micro-block: elements (row 0..3, col j)
      u32x2 c0 = {(a[0][0] & 0xffffu) | (a[1][0] << 16), (a[2][0] & 0xffffu) | (a[3][0] << 16)};
      u32x2 c1 = {(a[0][0] >> 16) | (a[1][0] & 0xffff0000u), (a[2][0] >> 16) | (a[3][0] & 0xffff0000u)};
      u32x2 c2 = {(a[0][1] & 0xffffu) | (a[1][1] << 16), (a[2][1] & 0xffffu) | (a[3][1] << 16)};
      u32x2 c3 = {(a[0][1] >> 16) | (a[1][1] & 0xffff0000u), (a[2][1] >> 16) | (a[3][1] & 0xffff0000u)};
      uint16_t* base = dst + (4 * cq) * ld + 4 * rq;
      *reinterpret_cast<u32x2*>(base + 0 * ld) = c0;
      *reinterpret_cast<u32x2*>(base + 1 * ld) = c1;
      *reinterpret_cast<u32x2*>(base + 2 * ld) = c2;
      *reinterpret_cast<u32x2*>(base + 3 * ld) = c3;
    }
  }
};

}  // namespace gptattn
