// Causal scaled dot-product self-attention on gfx950 matrix cores, bfloat16
// storage, float32 accumulation.
//
// The operation (lecture description "Let's build GPT: from scratch, in
// code, spelled out": chapters "version 3: adding softmax" and "version 4:
// self-attention", note 6 and the corrections at 00:57:00 and 01:20:05; heads
// as a batch dimension per exercise EX1 and "batched multi-headed
// self-attention"):  O = softmax(scale Q K^T, keys j <= i only) V, with the
// natural-log normaliser lse kept for the backward pass.
//
// Kernels (one wave = 64 lanes; every product is v_mfma_f32_32x32x16_bf16,
// see attn_common.h for the register layout):
//
//   attn_fwd      one workgroup = 128 queries of one head (4 waves x 32).
//                 Walks key tiles of 64 from position 0 up to the diagonal;
//                 tiles above the diagonal are never visited and only tiles
//                 that straddle it are masked.  Scores are formed transposed,
//                 S^T = K Q^T, so that each lane owns one query: the online
//                 softmax (running max m and sum l) stays in registers, the
//                 row reductions need one cross-half exchange, and the bf16
//                 probabilities feed O^T += V^T P^T straight from registers.
//                 K and V are staged row-major in LDS; V^T is read with
//                 the gfx950 transpose read (attn_common.h).
//   attn_bwd_dq   same tiling as attn_fwd.  First forms the row term
//                 delta_i = sum_d dO_id O_id (written to the workspace for
//                 attn_bwd_dkdv), then recomputes P^T from lse, dP^T = V dO^T,
//                 dS^T = P^T (dP^T - delta) and dQ^T += K^T dS^T.
//   attn_bwd_dkdv one workgroup = 128 keys of one head (4 waves x 32).  Walks
//                 query tiles from the diagonal to the end with the lane ->
//                 key layout: S = Q K^T and dP = dO V^T, then
//                 dV^T += dO^T P and dK^T += Q^T dS with P and dS taken from
//                 registers.  Q and dO are staged row-major in LDS and
//                 read transposed for the dV/dK products.
//
// dQ and dK/dV come from separate kernels, so no result is accumulated with
// atomics and every output is bitwise reproducible run to run.
#include "attn_common.h"
#include "launch.h"

namespace gptattn {

namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr float kLazy = 8.0f;  // log2 headroom before the running max is moved


// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------

// One 64-key tile for one wave (32 queries, one per lane column c), taken
// as two 32-key halves with one online-softmax step each, which keeps only
// half a tile of scores live.  MASK is set only for tiles that straddle the
// diagonal (or the end of the sequence).
template <int D, bool MASK>
__device__ __forceinline__ void fwd_tile(const uint16_t* kb, const uint16_t* vb, const bf16x8* qf,
                                         f32x16* ot, float& m, float& l, int k0, int qi, int c,
                                         int g, int tro, float sl2) {
  constexpr int LD = D + 8, DS = D / 16, DE = D / 32;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    // S^T = K Q^T for 32 keys: rows = keys, columns = this wave's queries
    f32x16 st = mfma32x32x16(ld_frag16(kb + (32 * a + c) * LD + 8 * g), qf[0], zero16());
#pragma unroll
    for (int s = 1; s < DS; ++s)
      st = mfma32x32x16(ld_frag16(kb + (32 * a + c) * LD + 16 * s + 8 * g), qf[s], st);
    if (MASK) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 32 * a + 8 * (r >> 2) + 4 * g + (r & 3);
        if (key > qi) st[r] = -INFINITY;
      }
    }
    float mx = st[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, st[r]);
    mx = half_max(mx) * sl2;
    // Lazy rescaling: the reference max m only moves when some row of the
    // wave sees a score more than 2^kLazy above it.  Until then the
    // probabilities exp2(s - m) stay below 2^kLazy, which bf16 and the
    // float32 accumulators hold exactly as well; O and l share the same
    // reference, so the final O / l is unchanged.
    if (__any(mx > m + kLazy)) {
      const float mnew = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int e = 0; e < DE; ++e) ot[e] *= alpha;
    }
    const float nm = -m;
    bf16x8 pf[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[8 * t + j], sl2, nm));
        l += p[j];
      }
      pf[t] = pack_bf16x8(p);
    }
    // O^T += V^T P^T, V^T read transposed from the row-major V tile
#pragma unroll
    for (int e = 0; e < DE; ++e)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        ot[e] = mfma32x32x16(ld_frag_tr(vb + (32 * a + 16 * t) * LD + 32 * e + tro, LD), pf[t],
                             ot[e]);
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, D == 64 ? 4 : 1) void attn_fwd(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
    float* __restrict__ LSE, int N, int T, float sl2, int nqb) {
  constexpr int BM = 128, BN = 64;
  constexpr int LD = D + 8;     // padded row stride of the LDS tiles
  constexpr int DS = D / 16;    // k-steps of the score product
  constexpr int DE = D / 32;    // 32-row output tiles over the head dim
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * LD];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][BN * LD];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int c = lane & 31, g = lane >> 5;
  const int tro = tr_rowoff(lane) * LD + tr_coloff(lane);
  const int bid = blockIdx.x;
  const int qb = nqb - 1 - bid / N;  // longest query blocks first
  const int n = bid % N;
  const uint16_t* Kh = K + (size_t)n * T * D;
  const uint16_t* Vh = V + (size_t)n * T * D;
  const int q0 = qb * BM;
  const int q0w = q0 + 32 * w;
  const int qi = q0w + c;

  bf16x8 qf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    if (qi < T) {
      qf[s] = ld_frag16(Q + ((size_t)n * T + qi) * D + 16 * s + 8 * g);
    } else {
      qf[s] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
  }

  const int kend = min(q0 + BM, T);
  const int nkt = (kend - 1) / BN + 1;
  const int wnkt = q0w < T ? (min(q0w + 32, T) - 1) / BN + 1 : 0;

  RowStage<BN, D, kThreads> ks, vs;
  ks.init(tid, LD);
  vs.init(tid, LD);
  ks.load(Kh, T);
  vs.load(Vh, T);
  ks.store(Ks[0], LD);
  vs.store(Vs[0], LD);
  __syncthreads();

  f32x16 ot[DE];
#pragma unroll
  for (int e = 0; e < DE; ++e) ot[e] = zero16();
  float m = -INFINITY, l = 0.0f;

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nkt;
    if (more) {
      const int k1 = (kt + 1) * BN;
      ks.load(Kh + (size_t)k1 * D, T - k1);
      vs.load(Vh + (size_t)k1 * D, T - k1);
    }
    if (kt < wnkt) {
      const int k0 = kt * BN;
      if (k0 + BN - 1 > q0w) {
        fwd_tile<D, true>(Ks[buf], Vs[buf], qf, ot, m, l, k0, qi, c, g, tro, sl2);
      } else {
        fwd_tile<D, false>(Ks[buf], Vs[buf], qf, ot, m, l, k0, qi, c, g, tro, sl2);
      }
    }
    if (more) {
      ks.store(Ks[buf ^ 1], LD);
      vs.store(Vs[buf ^ 1], LD);
    }
    __syncthreads();
  }

  const float lt = half_sum(l);
  if (qi < T) {
    const float inv = 1.0f / lt;
    uint16_t* orow = O + ((size_t)n * T + qi) * D;
#pragma unroll
    for (int e = 0; e < DE; ++e)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        u32x2 pk = {pack_bf16x2(ot[e][4 * u] * inv, ot[e][4 * u + 1] * inv),
                    pack_bf16x2(ot[e][4 * u + 2] * inv, ot[e][4 * u + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + 32 * e + 8 * u + 4 * g) = pk;
      }
    if (g == 0) LSE[(size_t)n * T + qi] = (m + log2f(lt)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Backward, part 1: row term delta and dQ (lane -> query layout)
// ---------------------------------------------------------------------------

// One 64-key tile for one wave of the dQ kernel, taken as two 32-key
// halves.  nd holds -delta of this lane's query in all 16 slots; it seeds
// the dP^T accumulator so that the product directly yields dP^T - delta.
template <int D, bool MASK>
__device__ __forceinline__ void dq_tile(const uint16_t* kb, const uint16_t* vb, const bf16x8* qf,
                                        const bf16x8* df, const f32x16& nd, f32x16* acc, int k0,
                                        int qi, int c, int g, int tro, float sl2, float nl) {
  constexpr int LD = D + 8, DS = D / 16, DE = D / 32;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    // S^T = K Q^T and dP^T - delta = V dO^T - delta: rows = keys, columns = queries
    f32x16 st = mfma32x32x16(ld_frag16(kb + (32 * a + c) * LD + 8 * g), qf[0], zero16());
    f32x16 dp = mfma32x32x16(ld_frag16(vb + (32 * a + c) * LD + 8 * g), df[0], nd);
#pragma unroll
    for (int s = 1; s < DS; ++s) {
      st = mfma32x32x16(ld_frag16(kb + (32 * a + c) * LD + 16 * s + 8 * g), qf[s], st);
      dp = mfma32x32x16(ld_frag16(vb + (32 * a + c) * LD + 16 * s + 8 * g), df[s], dp);
    }
    bf16x8 sf[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float ds[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 8 * t + j;
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[r], sl2, nl));
        if (MASK) {
          const int key = k0 + 32 * a + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key > qi) p = 0.0f;
        }
        ds[j] = p * dp[r];
      }
      sf[t] = pack_bf16x8(ds);
    }
    // dQ^T += K^T dS^T, K^T read transposed from the row-major K tile
#pragma unroll
    for (int e = 0; e < DE; ++e)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        acc[e] = mfma32x32x16(ld_frag_tr(kb + (32 * a + 16 * t) * LD + 32 * e + tro, LD), sf[t],
                              acc[e]);
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, D == 64 ? 3 : 1) void attn_bwd_dq(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ O,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE,
    uint16_t* __restrict__ dQ, float* __restrict__ Delta, int N, int T,
    float sl2, float scale, int nqb) {
  constexpr int BM = 128, BN = 64;
  constexpr int LD = D + 8;
  constexpr int DS = D / 16;
  constexpr int DE = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * LD];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][BN * LD];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int c = lane & 31, g = lane >> 5;
  const int tro = tr_rowoff(lane) * LD + tr_coloff(lane);
  const int bid = blockIdx.x;
  const int qb = nqb - 1 - bid / N;
  const int n = bid % N;
  const uint16_t* Kh = K + (size_t)n * T * D;
  const uint16_t* Vh = V + (size_t)n * T * D;
  const int q0 = qb * BM;
  const int q0w = q0 + 32 * w;
  const int qi = q0w + c;

  bf16x8 qf[DS], df[DS];
  float dpart = 0.0f;
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    if (qi < T) {
      const size_t off = ((size_t)n * T + qi) * D + 16 * s + 8 * g;
      qf[s] = ld_frag16(Q + off);
      const u32x4 dou = *reinterpret_cast<const u32x4*>(dO + off);
      const u32x4 ou = *reinterpret_cast<const u32x4*>(O + off);
      df[s] = __builtin_bit_cast(bf16x8, dou);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dpart += bf16_lo(dou[j]) * bf16_lo(ou[j]) + bf16_hi(dou[j]) * bf16_hi(ou[j]);
    } else {
      qf[s] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      df[s] = qf[s];
    }
  }
  const float delta = half_sum(dpart);
  const float nl = qi < T ? -LSE[(size_t)n * T + qi] * kLog2e : 0.0f;
  if (qi < T && g == 0) Delta[(size_t)n * T + qi] = delta;
  f32x16 nd;
#pragma unroll
  for (int r = 0; r < 16; ++r) nd[r] = -delta;

  const int kend = min(q0 + BM, T);
  const int nkt = (kend - 1) / BN + 1;
  const int wnkt = q0w < T ? (min(q0w + 32, T) - 1) / BN + 1 : 0;

  RowStage<BN, D, kThreads> ks, vs;
  ks.init(tid, LD);
  vs.init(tid, LD);
  ks.load(Kh, T);
  vs.load(Vh, T);
  ks.store(Ks[0], LD);
  vs.store(Vs[0], LD);
  __syncthreads();

  f32x16 acc[DE];
#pragma unroll
  for (int e = 0; e < DE; ++e) acc[e] = zero16();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nkt;
    if (more) {
      const int k1 = (kt + 1) * BN;
      ks.load(Kh + (size_t)k1 * D, T - k1);
      vs.load(Vh + (size_t)k1 * D, T - k1);
    }
    if (kt < wnkt) {
      const int k0 = kt * BN;
      if (k0 + BN - 1 > q0w) {
        dq_tile<D, true>(Ks[buf], Vs[buf], qf, df, nd, acc, k0, qi, c, g, tro, sl2, nl);
      } else {
        dq_tile<D, false>(Ks[buf], Vs[buf], qf, df, nd, acc, k0, qi, c, g, tro, sl2, nl);
      }
    }
    if (more) {
      ks.store(Ks[buf ^ 1], LD);
      vs.store(Vs[buf ^ 1], LD);
    }
    __syncthreads();
  }

  if (qi < T) {
    uint16_t* row = dQ + ((size_t)n * T + qi) * D;
#pragma unroll
    for (int e = 0; e < DE; ++e)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        u32x2 pk = {pack_bf16x2(acc[e][4 * u] * scale, acc[e][4 * u + 1] * scale),
                    pack_bf16x2(acc[e][4 * u + 2] * scale, acc[e][4 * u + 3] * scale)};
        *reinterpret_cast<u32x2*>(row + 32 * e + 8 * u + 4 * g) = pk;
      }
  }
}

// ---------------------------------------------------------------------------
// Backward, part 2: dK and dV (lane -> key layout)
// ---------------------------------------------------------------------------

// Query-row statistics in LDS are stored permuted so that the 16 rows a
// lane half needs for one 32-query block (rows 8u + 4g + i in result-
// register order r = 4u + i) are contiguous: row q of the tile goes to
// slot 32 (q / 32) + 16 ((q % 8) / 4) + 4 ((q % 32) / 8) + q % 4.
__device__ __forceinline__ int stat_slot(int q) {
  return 32 * (q >> 5) + 16 * ((q & 7) >> 2) + 4 * ((q & 31) >> 3) + (q & 3);
}

// One BM-query tile for one wave (32 keys, one per lane column c).  ls/es
// hold -lse * log2(e) and -delta of the tile's queries, permuted by
// stat_slot; -delta seeds the dP accumulator so that the product yields
// dP - delta directly.
template <int D, int BM, bool MASK>
__device__ __forceinline__ void dkdv_tile(const uint16_t* qb, const uint16_t* db, const float* ls,
                                          const float* es, const bf16x8* kf, const bf16x8* vf,
                                          f32x16* dvt, f32x16* dkt, int q0, int kj, int g,
                                          int c, int tro, float sl2) {
  constexpr int LD = D + 8, DS = D / 16, DE = D / 32, NH = BM / 32;
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const f32x16 nl = *reinterpret_cast<const f32x16*>(ls + 32 * h + 16 * g);
    const f32x16 nd = *reinterpret_cast<const f32x16*>(es + 32 * h + 16 * g);
    // S = Q K^T and dP - delta = dO V^T - delta: rows = queries, columns = keys
    f32x16 st = mfma32x32x16(ld_frag16(qb + (32 * h + c) * LD + 8 * g), kf[0], zero16());
    f32x16 dp = mfma32x32x16(ld_frag16(db + (32 * h + c) * LD + 8 * g), vf[0], nd);
#pragma unroll
    for (int s = 1; s < DS; ++s) {
      st = mfma32x32x16(ld_frag16(qb + (32 * h + c) * LD + 16 * s + 8 * g), kf[s], st);
      dp = mfma32x32x16(ld_frag16(db + (32 * h + c) * LD + 16 * s + 8 * g), vf[s], dp);
    }
    bf16x8 pf[2], sf[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float p[8], dsv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 8 * t + j;
        float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(st[r], sl2, nl[r]));
        if (MASK && kj > q0 + 32 * h + 8 * (r >> 2) + 4 * g + (r & 3)) pv = 0.0f;
        p[j] = pv;
        dsv[j] = pv * dp[r];
      }
      pf[t] = pack_bf16x8(p);
      sf[t] = pack_bf16x8(dsv);
    }
    // dV^T += dO^T P and dK^T += Q^T dS, dO^T and Q^T read transposed
#pragma unroll
    for (int e = 0; e < DE; ++e)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int off = (32 * h + 16 * t) * LD + 32 * e + tro;
        dvt[e] = mfma32x32x16(ld_frag_tr(db + off, LD), pf[t], dvt[e]);
        dkt[e] = mfma32x32x16(ld_frag_tr(qb + off, LD), sf[t], dkt[e]);
      }
  }
}

template <int D, int BM>
__global__ __launch_bounds__(kThreads, D == 64 ? 2 : 1) void attn_bwd_dkdv(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Delta,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N, int T,
    float sl2, float scale, int nkb) {
  constexpr int BN = 128;
  constexpr int LD = D + 8;     // row-major Q / dO tiles
  constexpr int DS = D / 16;
  constexpr int DE = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[2][BM * LD];
  __shared__ __attribute__((aligned(16))) uint16_t Ds[2][BM * LD];
  __shared__ __attribute__((aligned(64))) float Ls[2][BM];
  __shared__ __attribute__((aligned(64))) float Es[2][BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int c = lane & 31, g = lane >> 5;
  const int tro = tr_rowoff(lane) * LD + tr_coloff(lane);
  const int bid = blockIdx.x;
  const int kb = bid / N;  // block 0 (the most queries) first
  const int n = bid % N;
  const uint16_t* Qh = Q + (size_t)n * T * D;
  const uint16_t* Dh = dO + (size_t)n * T * D;
  const size_t rows = (size_t)n * T;
  const int k0 = kb * BN;
  const int k0w = k0 + 32 * w;
  const int kj = k0w + c;

  bf16x8 kf[DS], vf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    if (kj < T) {
      const size_t off = (rows + kj) * D + 16 * s + 8 * g;
      kf[s] = ld_frag16(K + off);
      vf[s] = ld_frag16(V + off);
    } else {
      kf[s] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      vf[s] = kf[s];
    }
  }

  const int qt0 = k0 / BM;
  const int nqt = (T + BM - 1) / BM;

  RowStage<BM, D, kThreads> qs, ds;
  qs.init(tid, LD);
  ds.init(tid, LD);
  float lv = 0.0f, ev = 0.0f;
  auto load_tile = [&](int qt) {
    const int q1 = qt * BM;
    qs.load(Qh + (size_t)q1 * D, T - q1);
    ds.load(Dh + (size_t)q1 * D, T - q1);
    if (tid < BM) {
      const int q = q1 + tid;
      lv = q < T ? -LSE[rows + q] * kLog2e : -INFINITY;
      ev = q < T ? -Delta[rows + q] : 0.0f;
    }
  };
  auto store_tile = [&](int b) {
    qs.store(Qs[b], LD);
    ds.store(Ds[b], LD);
    if (tid < BM) {
      Ls[b][stat_slot(tid)] = lv;
      Es[b][stat_slot(tid)] = ev;
    }
  };
  load_tile(qt0);
  store_tile(0);
  __syncthreads();

  f32x16 dvt[DE], dkt[DE];
#pragma unroll
  for (int e = 0; e < DE; ++e) {
    dvt[e] = zero16();
    dkt[e] = zero16();
  }

  for (int qt = qt0; qt < nqt; ++qt) {
    const int buf = (qt - qt0) & 1;
    const bool more = qt + 1 < nqt;
    if (more) load_tile(qt + 1);
    const int q0 = qt * BM;
    if (q0 + BM - 1 >= k0w && k0w < T) {  // some query of the tile sees a key of this wave
      if (k0w + 31 > q0) {
        dkdv_tile<D, BM, true>(Qs[buf], Ds[buf], Ls[buf], Es[buf], kf, vf, dvt, dkt, q0, kj, g, c,
                               tro, sl2);
      } else {
        dkdv_tile<D, BM, false>(Qs[buf], Ds[buf], Ls[buf], Es[buf], kf, vf, dvt, dkt, q0, kj, g,
                                c, tro, sl2);
      }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (kj < T) {
    uint16_t* krow = dK + (rows + kj) * D;
    uint16_t* vrow = dV + (rows + kj) * D;
#pragma unroll
    for (int e = 0; e < DE; ++e)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int d = 32 * e + 8 * u + 4 * g;
        u32x2 pk = {pack_bf16x2(dkt[e][4 * u] * scale, dkt[e][4 * u + 1] * scale),
                    pack_bf16x2(dkt[e][4 * u + 2] * scale, dkt[e][4 * u + 3] * scale)};
        *reinterpret_cast<u32x2*>(krow + d) = pk;
        u32x2 pv = {pack_bf16x2(dvt[e][4 * u], dvt[e][4 * u + 1]),
                    pack_bf16x2(dvt[e][4 * u + 2], dvt[e][4 * u + 3])};
        *reinterpret_cast<u32x2*>(vrow + d) = pv;
      }
  }
}

template <typename... Args>
hipError_t launch(void (*kern)(Args...), int blocks, hipStream_t stream, Args... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), dim3(blocks), dim3(kThreads), argv, 0,
                         stream);
}

template <int D>
hipError_t fwd_d(const void* q, const void* k, const void* v, void* o, float* lse, int N, int T,
                 float scale, hipStream_t stream) {
  const int nqb = (T + 127) / 128;
  return launch(attn_fwd<D>, N * nqb, stream, (const uint16_t*)q, (const uint16_t*)k,
                (const uint16_t*)v, (uint16_t*)o, lse, N, T, scale * kLog2e, nqb);
}

template <int D>
hipError_t bwd_dq_d(const void* q, const void* k, const void* v, const void* o, const void* dO,
                    const float* lse, void* dq, float* delta, int N, int T, float scale,
                    hipStream_t stream) {
  const int nqb = (T + 127) / 128;
  return launch(attn_bwd_dq<D>, N * nqb, stream, (const uint16_t*)q, (const uint16_t*)k,
                (const uint16_t*)v, (const uint16_t*)o, (const uint16_t*)dO, lse, (uint16_t*)dq,
                delta, N, T, scale * kLog2e, scale, nqb);
}

template <int D, int BM>
hipError_t bwd_dkdv_d(const void* q, const void* k, const void* v, const void* dO,
                      const float* lse, const float* delta, void* dk, void* dv, int N, int T,
                      float scale, hipStream_t stream) {
  const int nkb = (T + 127) / 128;
  return launch(attn_bwd_dkdv<D, BM>, N * nkb, stream, (const uint16_t*)q, (const uint16_t*)k,
                (const uint16_t*)v, (const uint16_t*)dO, lse, delta, (uint16_t*)dk,
                (uint16_t*)dv, N, T, scale * kLog2e, scale, nkb);
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int N, int T, int D, float scale, hipStream_t stream) {
  switch (D) {
    case 64: return fwd_d<64>(q, k, v, o, lse, N, T, scale, stream);
    case 128: return fwd_d<128>(q, k, v, o, lse, N, T, scale, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_dq_bf16(const void* q, const void* k, const void* v, const void* o,
                              const void* dO, const float* lse, void* dq, float* delta, int N,
                              int T, int D, float scale, hipStream_t stream) {
  switch (D) {
    case 64: return bwd_dq_d<64>(q, k, v, o, dO, lse, dq, delta, N, T, scale, stream);
    case 128: return bwd_dq_d<128>(q, k, v, o, dO, lse, dq, delta, N, T, scale, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_dkdv_bf16(const void* q, const void* k, const void* v, const void* dO,
                                const float* lse, const float* delta, void* dk, void* dv, int N,
                                int T, int D, float scale, hipStream_t stream) {
  switch (D) {
    case 64: return bwd_dkdv_d<64, 64>(q, k, v, dO, lse, delta, dk, dv, N, T, scale, stream);
    case 128: return bwd_dkdv_d<128, 32>(q, k, v, dO, lse, delta, dk, dv, N, T, scale, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gptattn
