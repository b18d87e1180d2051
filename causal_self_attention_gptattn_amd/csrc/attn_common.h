// Shared device-side building blocks for the gfx950 attention kernels:
// vector types, the bf16 matrix-core product, conversions, range-checked
// row loads, the HBM -> LDS tile copy with its swizzled layout, and the
// row-wise epilogue store.
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
#include <limits.h>
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

// 16 x 16 result, K = 32, lane l = 16g + c (g = 0..3): the A operand holds
// A[c][8g + j], the B operand B[8g + j][c], the result D[4g + r][c]
// (r = 0..3), j = 0..7.  (Measured on the GPU with an in-bounds probe.)
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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

// Reductions across the two 32-lane halves of a wave (lane l with l ^ 32)
// with v_permlane32_swap: after the swap, lane l holds x[l] and x[l ^ 32]
// in the two results, in some order, which is all a symmetric op needs.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// 16-byte LDS/global read as an MFMA operand.
__device__ __forceinline__ bf16x8 ld_frag16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// ---------------------------------------------------------------------------
// Transposed operand reads from a row-major LDS tile (gfx950
// ds_read_b64_tr_b16).  Within each group of 16 lanes, lane i receives
// element (i % 4) of the 8-byte chunks addressed by lanes 4j + i / 4,
// j = 0..3.  When the group's lanes address a 4-row x 16-column block
// (lane L -> row L / 4, columns 4 (L % 4) .. +3), lane i therefore gets
// column i of the four rows: four consecutive k-values of one MFMA row m.
//
// For an A operand X^T[m][k] of v_mfma_f32_32x32x16_bf16 read from a
// row-major tile X[k][m], lane (c, g) needs k = kb + 4g + {0..3} and
// kb + 8 + 4g + {0..3} at m = mb + c (the row pattern of a result tile's
// registers 0..7).  tr_rowoff/tr_coloff give this lane's row and column
// inside such a 16 x 32 block; ld_frag_tr2 reads its two 8-row halves
// (rows r and r + 8), each from its own address, as the swizzled LDS
// layout places them.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int tr_rowoff(int lane) { return 4 * (lane >> 5) + ((lane & 15) >> 2); }
__device__ __forceinline__ int tr_coloff(int lane) { return 16 * ((lane >> 4) & 1) + 4 * (lane & 3); }

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// lo = &X[kb + tr_rowoff][mb + tr_coloff], hi = the same column 8 rows down.
__device__ __forceinline__ bf16x8 ld_frag_tr2(const uint16_t* lo, const uint16_t* hi) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lo));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(hi));
  const u32x2 l2 = __builtin_bit_cast(u32x2, a);
  const u32x2 h2 = __builtin_bit_cast(u32x2, b);
  return __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
}

// ---------------------------------------------------------------------------
// Problem description shared by the kernels.
//
// A tensor is a [B][H][T][D] view with the D elements of each row
// contiguous: element (b, h, t, d) sits at p + b * sb + h * sh + t * st + d.
// Query i (of Tq) sees key j (of Tk) when j <= i + off and, with win > 0,
// j > i + off - win (a band of the win most recent positions).  The plain
// causal case is Tq = Tk, off = 0, win = 0.
// ---------------------------------------------------------------------------
struct View {
  const uint16_t* p;
  long long sb, sh, st;
};
struct Problem {
  int N, H, Tq, Tk, off, win;
  float sl2;    // scale * log2(e)
  float scale;
  // attention dropout (used only by the dropout instantiations)
  uint32_t seed_lo, seed_hi;  // Philox key
  uint32_t stream;            // fourth counter word
  uint32_t thr;               // drop iff 16-bit draw < thr, thr = ceil(p * 2^16)
  float inv_keep;             // keep scale 2^16 / (2^16 - thr)
};

// Kernel-side problem description from the host-side one (launch.h); fills
// the dropout threshold thr = ceil(p * 2^16) and the keep scale
// 2^16 / (2^16 - thr).
struct ProblemArg;
Problem make_problem(const ProblemArg& p);

template <typename P>
__device__ __forceinline__ P head_of(P p, long long sb, long long sh, int n, int H) {
  return p + (long long)(n / H) * sb + (long long)(n % H) * sh;
}
__device__ __forceinline__ const uint16_t* head_of(const View& v, int n, int H) {
  return head_of(v.p, v.sb, v.sh, n, H);
}

// Keys query i sees, as a closed interval (empty when hi < lo), and the
// queries that see key j (to be cut at Tq by the caller).
struct Span {
  int lo, hi;
};
__device__ __forceinline__ Span keys_of(int i, const Problem& pb) {
  return Span{pb.win > 0 ? i + pb.off - pb.win + 1 : INT_MIN, min(i + pb.off, pb.Tk - 1)};
}
__device__ __forceinline__ Span queries_of(int j, const Problem& pb) {
  return Span{j - pb.off, pb.win > 0 ? j - pb.off + pb.win - 1 : INT_MAX};
}
__device__ __forceinline__ bool inside(int x, Span s) { return x >= s.lo && x <= s.hi; }
// First / last key visible to some query in [i0, i1] (clamped to the keys
// that exist; lo > hi means none).
__device__ __forceinline__ int keys_lo(int i0, const Problem& pb) {
  return pb.win > 0 ? max(0, i0 + pb.off - pb.win + 1) : 0;
}
__device__ __forceinline__ int keys_hi(int i1, const Problem& pb) {
  return min(pb.Tk - 1, i1 + pb.off);
}
// Does some query in [i0, i1] fail to see some key in [j0, j1] (or is some
// key past the end)?  Only such tiles pay for the element-wise mask.
__device__ __forceinline__ bool needs_mask(int i0, int i1, int j0, int j1, const Problem& pb) {
  return j1 > i0 + pb.off || j1 >= pb.Tk || (pb.win > 0 && j0 <= i1 + pb.off - pb.win);
}
// First / last query that sees some key in [j0, j1].
__device__ __forceinline__ int queries_lo(int j0, const Problem& pb) {
  return max(0, j0 - pb.off);
}
__device__ __forceinline__ int queries_hi(int j1, const Problem& pb) {
  return pb.win > 0 ? min(pb.Tq - 1, j1 - pb.off + pb.win - 1) : pb.Tq - 1;
}

// ---------------------------------------------------------------------------
// Attention dropout.  Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
// "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011): per round the
// words 0 and 2 are multiplied by 0xD2511F53 and 0xCD9E8D57 into 64-bit
// products; the new words are (hi(w2 product) ^ w1 ^ key0, lo(w2 product),
// hi(w0 product) ^ w3 ^ key1, lo(w0 product)); the key advances by
// 0x9E3779B9 and 0xBB67AE85 between rounds.
//
// Each call decides eight weights with 16-bit draws: for head-problem n,
// query i and key j the generator runs on counter (j / 4, i / 2, n, stream)
// with key (seed_lo, seed_hi); the draw is the low half of word j % 4 for
// even i and its high half for odd i.  The weight is kept iff draw >= thr
// (thr = ceil(p * 2^16), so it is dropped with probability thr / 2^16) and
// then scaled by 2^16 / (2^16 - thr), the inverse of the realised keep
// probability, so that the expected scaled weight is the weight itself.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c0 = n0;
    c1 = (uint32_t)p1;
    c2 = n2;
    c3 = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return u32x4{c0, c1, c2, c3};
}

// Keep bits of one call: keys 4 * jb + m (m = 0..3) for queries 2 * ip and
// 2 * ip + 1, in bit 2m (even query) and bit 2m + 1 (odd query).
__device__ __forceinline__ uint32_t keep8(uint32_t jb, uint32_t ip, uint32_t n,
                                          const Problem& pb) {
  const u32x4 w = philox4x32_10(jb, ip, n, pb.stream, pb.seed_lo, pb.seed_hi);
  uint32_t b = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m)
    b |= ((w[m] & 0xFFFFu) >= pb.thr ? 1u : 0u) << (2 * m) |
         ((w[m] >> 16) >= pb.thr ? 1u : 0u) << (2 * m + 1);
  return b;
}

// Bits 2m + q (m = 0..3) of a keep8 result packed into bits 0..3: the four
// keys' bits for the query of parity q.
__device__ __forceinline__ uint32_t keep_of_query(uint32_t b, uint32_t q) {
  return ((b >> q) & 1u) | ((b >> (1 + q)) & 2u) | ((b >> (2 + q)) & 4u) | ((b >> (3 + q)) & 8u);
}

// Keep bits of keys 4 * jb .. 4 * jb + 3 (kb0) and 4 * jb + 8 .. 4 * jb + 11
// (kb1) for query qi, bit k = key k of the group, in kernels where lanes
// 2x and 2x + 1 hold queries 2y and 2y + 1 with the same jb: the even lane
// draws group jb and the odd lane group jb + 2, each for both queries, and
// the two exchange the half the other needs.
__device__ __forceinline__ void keep_bits_pair(uint32_t jb, uint32_t qi, uint32_t n,
                                               const Problem& pb, uint32_t& kb0,
                                               uint32_t& kb1) {
  const uint32_t odd = qi & 1u;
  const uint32_t mine = keep8(jb + 2 * odd, qi >> 1, n, pb);
  // value of lane ^ 1 (DPP quad permute 1, 0, 3, 2)
  const uint32_t other = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mine, 0xB1, 0xF, 0xF, false);
  kb0 = keep_of_query(odd ? other : mine, odd);
  kb1 = keep_of_query(odd ? mine : other, odd);
}

// Value of v in lane SRC of this lane's group of four (DPP quad permute).
template <int SRC>
__device__ __forceinline__ uint32_t quad_lane(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, SRC * 0x55, 0xF, 0xF, false);
}

// ---------------------------------------------------------------------------
// Range-checked loads.  Global reads of tiles and row statistics go through
// a buffer descriptor whose range ends at the last row that exists: the
// hardware returns zero for reads at or past the end, so a ragged last tile
// needs no branch and no select, and the loads of a tile issue back to back.
// Because st >= D, every chunk of a row r < valid lies below valid * st
// elements and every chunk of a row r >= valid lies at or above it.
// ---------------------------------------------------------------------------
constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit buffer access (gfx9 family)

// One float per thread from a range-checked buffer: element i of base[0, n)
// (0.0f for i >= n or n <= 0, with no memory access).  base and n are
// uniform across the workgroup; readfirstlane states that for the record
// count, which keeps the descriptor in scalar registers.
__device__ __forceinline__ float load_f32_or_zero(const float* base, int n, int i) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(base), 0, __builtin_amdgcn_readfirstlane(n <= 0 ? 0 : n * 4),
      kBufferWord3);
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, i * 4, 0, 0));
}

// A wave's block of 32 rows of a bf16 matrix (rows `st` elements apart,
// st >= D): 16-byte pieces of row r (0 <= r < 32, this lane's row) through a
// range-checked descriptor, zero for rows at or past `valid` (no memory
// access), so that the loads need no branch and issue back to back.  base
// (the block's first row) and valid are uniform across the wave.
struct RowBlock {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t roff;  // byte offset of this lane's row

  __device__ __forceinline__ void init(const uint16_t* base, int valid, long long st, int r) {
    const int rows = valid <= 0 ? 0 : valid < 32 ? valid : 32;
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0,
                                           __builtin_amdgcn_readfirstlane(rows * (int)(st * 2)),
                                           kBufferWord3);
    roff = (uint32_t)r * (uint32_t)(st * 2);
  }
  // elements col .. col + 7 of this lane's row
  __device__ __forceinline__ u32x4 load(int col) const {
    return __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(roff + 2u * (uint32_t)col), 0, 0));
  }
};

// ---------------------------------------------------------------------------
// Global -> LDS copy of a ROWS x D bf16 tile (rows `st` elements apart in
// HBM, st >= D, D contiguous) without a register round trip (gfx950
// buffer_load_dwordx4 ... lds).  Thread t of NT moves 16-byte chunks t,
// t + NT, ...  Each lane's 16 bytes land at the lane's position in a
// contiguous 1024-byte block per wave instruction, so the LDS tile is
// unpadded (row stride D) and bank conflicts are avoided by a swizzle
// instead: 16-byte chunk k of row r sits in slot k ^ swz_key(r) of that row.
// Each lane picks the global chunk that belongs in its slot, so a wave still
// reads whole rows.  Rows at or past `valid` read as zero (range check
// above).  The copy completes asynchronously; wait_dma() then a workgroup
// barrier make it visible.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

// The key depends on r mod 16 and was chosen by measurement: a probe
// repeating each operand read of the kernels alone over a tile, under the
// LDS bank-conflict counter, for each candidate key.
//   ds_read_b64_tr_b16 (transposed operands) behaves as 64 banks of 4 bytes
//     serving 32 lanes at a time: conflict-free when the 32 lanes' 8-byte
//     pieces cover the 256-byte window once.  Every prediction of this rule
//     over 270 keys matched the counter.
//   ds_read_b128 (fragments: one chunk in 16 consecutive rows per 16-lane
//     group) follows no rule of that kind that fits the measurements (a key
//     that spreads each group's 16 rows over the window can still cost 4
//     conflict cycles per read), so its keys are measured ones.
// The 32-row kernels read fragments of one chunk in 32 rows and transposed
// pieces of four chunks in rows 4i..4i+3; the keys below (W16 = false) are
// conflict-free for both at D = 64.  The kernels with 16-row waves
// (16 x 16 x 32 products, W16) read fragments of four chunks in 16 rows and
// transposed pieces of two chunks in rows 4i..4i+3 for two consecutive i.
// For them the first key costs 4 conflict cycles per fragment read at
// D = 64, and at D = 128 4 per fragment read and 2 per transposed read.
// r mod 8 (D = 64) and the D = 128 key with bit 2 of r also flipping bit 1
// measure conflict-free for both of their reads.
template <int D, bool W16 = false>
__device__ __forceinline__ int swz_key(int row) {
  static_assert(D == 64 || D == 128, "swizzle defined for rows of 64 or 128 elements");
  if (W16)
    return D == 64 ? (row & 7) : ((row & 3) << 2) | (((row >> 2) & 3) ^ ((row >> 1) & 2));
  return D == 64 ? ((row & 2) << 1) | ((row >> 2) & 3) : ((row & 3) << 2) | ((row >> 2) & 3);
}

// Element offset of (row, col) in a swizzled row-major tile of row length D
// (col a multiple of 4 within one 16-byte chunk, or any col for the chunk's
// first element).
template <int D, bool W16 = false>
__device__ __forceinline__ int swz(int row, int col) {
  return row * D + (((col >> 3) ^ swz_key<D, W16>(row)) << 3) + (col & 7);
}

template <int ROWS, int D, int NT, bool W16 = false>
struct TileDMA {
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int PER = ROWS * CPR / NT;  // chunks per thread
  static constexpr int RSTEP = NT / CPR;       // rows between a thread's chunks
  static_assert((ROWS * CPR) % NT == 0 && NT % CPR == 0 && RSTEP % 16 == 0,
                "tile must split evenly, and each thread's rows share one swizzle");
  uint32_t goff;   // byte offset of the thread's first chunk in the global tile
  uint32_t gstep;  // bytes between the thread's chunks
  uint32_t rowb;   // bytes between rows in the global tile
  int wofs;        // element offset of this wave's first slot in the LDS tile

  __device__ __forceinline__ void init(int tid, long long st) {
    const int row = tid / CPR, slot = tid % CPR;
    rowb = (uint32_t)(st * 2);
    goff = (uint32_t)row * rowb + 16u * (uint32_t)(slot ^ swz_key<D, W16>(row));
    gstep = (uint32_t)RSTEP * rowb;
    wofs = __builtin_amdgcn_readfirstlane(tid >> 6) * 512;  // uniform: the copy writes through M0
  }

  // src: first element of the tile (uniform); lds: the LDS tile.
  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int valid,
                                       uint16_t* lds) const {
    const int rows = valid <= 0 ? 0 : valid < ROWS ? valid : ROWS;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(src), 0, __builtin_amdgcn_readfirstlane(rows * (int)rowb),
        kBufferWord3);
#pragma unroll
    for (int p = 0; p < PER; ++p)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + wofs + p * NT * 8), 16,
                                               (int)goff, (int)(p * gstep), 0, 0);
  }
};

// This lane's element offsets into a swizzled tile for the two MFMA operand
// reads, relative to the first row of a 32-row block: the 16-byte fragment
// of row c (ld_frag16) and the transposed 8-byte pieces of rows trr and
// trr + 8 (ld_frag_tr2).  The swizzle key repeats every 16 rows, so the
// offsets are the same for every block and the block's position becomes an
// immediate offset of the read instruction.
template <int D>
struct SwzLane {
  int fo[D / 16];                // row c, chunk 2s + g
  int tlo[D / 32], thi[D / 32];  // rows trr and trr + 8, columns 32e + trc: transposed
  __device__ __forceinline__ void init(int c, int g, int trr, int trc) {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) fo[s] = swz<D>(c, 16 * s + 8 * g);
#pragma unroll
    for (int e = 0; e < D / 32; ++e) {
      tlo[e] = swz<D>(trr, 32 * e + trc);
      thi[e] = swz<D>(trr + 8, 32 * e + trc);
    }
  }
};

// Wait for this wave's outstanding global loads, including copies into LDS.
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The same wait as a real s_waitcnt instruction (vmcnt(0), the other counters
// left alone: expcnt 7, lgkmcnt 15), which the compiler's own wait insertion
// takes into account: registers loaded before it count as arrived, so no
// wait for them is placed later (inside a loop that follows, every
// iteration would otherwise wait for that iteration's tile copies).
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt vmcnt(N), the other counters left alone, as an instruction the
// compiler's own wait insertion takes into account.
template <int N>
__device__ __forceinline__ void wait_vm_upto() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// ---------------------------------------------------------------------------
// Epilogue: a wave's 32 x D block of results, held in the MFMA result layout
// (lane (c, g) holds, for row c, columns 32e + 8u + 4g + i in acc[e][4u + i]),
// goes to HBM as bf16 through a wave-private LDS region of 16 rows at a time,
// so that every store instruction writes whole rows (D = 64: eight lanes per
// 128-byte row) instead of 8-byte pieces of 32 rows.  All threads of the
// workgroup must call it (it contains workgroup barriers); rows at or past
// `rows_valid` are not written.  lds: this wave's region, 16 * (D + 8)
// elements, not in use by any other wave.
// ---------------------------------------------------------------------------
// The LDS accesses of one wave are carried out in program order; a fence at
// wavefront scope keeps the compiler from moving them across this point.  So
// a wave that stages data in an LDS area of its own needs no workgroup
// barrier between writing and reading it back.
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D>
__device__ __forceinline__ void store_rows(uint16_t* lds, const f32x16* acc, float mul,
                                           uint16_t* out, long long st, int rows_valid, int lane) {
  constexpr int RS = D + 8, DE = D / 32, CPR = D / 8, PASS = 16 * CPR / 64;
  const int c = lane & 31, g = lane >> 5;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if ((c >> 4) == half) {
#pragma unroll
      for (int e = 0; e < DE; ++e)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const u32x2 pk = {pack_bf16x2(acc[e][4 * u] * mul, acc[e][4 * u + 1] * mul),
                            pack_bf16x2(acc[e][4 * u + 2] * mul, acc[e][4 * u + 3] * mul)};
          *reinterpret_cast<u32x2*>(lds + (c & 15) * RS + 32 * e + 8 * u + 4 * g) = pk;
        }
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < PASS; ++p) {
      const int ch = lane + 64 * p, r = ch / CPR, cc = ch % CPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(lds + r * RS + 8 * cc);
      const int row = 16 * half + r;
      if (row < rows_valid) *reinterpret_cast<u32x4*>(out + (long long)row * st + 8 * cc) = v;
    }
    __syncthreads();
  }
}

}  // namespace gptattn
