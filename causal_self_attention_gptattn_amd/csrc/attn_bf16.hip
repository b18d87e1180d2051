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
//                 K is staged row-major in LDS, V transposed.
//   attn_bwd_dq   same tiling as attn_fwd.  First forms the row term
//                 delta_i = sum_d dO_id O_id (written to the workspace for
//                 attn_bwd_dkdv), then recomputes P^T from lse, dP^T = V dO^T,
//                 dS^T = P^T (dP^T - delta) and dQ^T += K^T dS^T.
//   attn_bwd_dkdv one workgroup = 128 keys of one head (4 waves x 32).  Walks
//                 query tiles from the diagonal to the end with the lane ->
//                 key layout: S = Q K^T and dP = dO V^T, then
//                 dV^T += dO^T P and dK^T += Q^T dS with P and dS taken from
//                 registers.  Q and dO are staged both row-major and
//                 transposed in LDS.
//
// dQ and dK/dV come from separate kernels, so no result is accumulated with
// atomics and every output is bitwise reproducible run to run.
#include "attn_common.h"
#include "launch.h"

namespace gptattn {

namespace {

constexpr int kThreads = 256;  // 4 waves

__device__ __forceinline__ float wave_xor32(float x) { return __shfl_xor(x, 32); }

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, D == 64 ? 2 : 1) void attn_fwd(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
    float* __restrict__ LSE, int N, int T, float sl2, int nqb) {
  constexpr int BM = 128, BN = 64;
  constexpr int KLD = D + 8;    // row-major K tile, padded
  constexpr int VLD = BN + 4;   // transposed V tile, padded
  constexpr int DS = D / 16;    // k-steps of the score product
  constexpr int DE = D / 32;    // 32-row output tiles over the head dim
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * KLD];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * VLD];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int c = lane & 31, g = lane >> 5;
  const int bid = blockIdx.x;
  const int qb = nqb - 1 - bid / N;  // longest query blocks first
  const int n = bid % N;
  const size_t head = (size_t)n * T * D;
  const int q0 = qb * BM;
  const int q0w = q0 + 32 * w;
  const int qi = q0w + c;

  bf16x8 qf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    if (qi < T) {
      qf[s] = ld_frag16(Q + head + (size_t)qi * D + 16 * s + 8 * g);
    } else {
      qf[s] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
  }

  const int kend = min(q0 + BM, T);
  const int nkt = (kend - 1) / BN + 1;
  const int wnkt = q0w < T ? (min(q0w + 32, T) - 1) / BN + 1 : 0;

  TileStage<BN, D, kThreads> ks, vs;
  ks.load(K + head, T, tid);
  vs.load(V + head, T, tid);
  ks.store_rowmajor(Ks[0], KLD, tid);
  vs.store_transposed(Vt[0], VLD, tid);
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
      ks.load(K + head + (size_t)k1 * D, T - k1, tid);
      vs.load(V + head + (size_t)k1 * D, T - k1, tid);
    }
    if (kt < wnkt) {
      const int k0 = kt * BN;
      const uint16_t* kb = Ks[buf];
      const uint16_t* vb = Vt[buf];
      f32x16 st[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        st[a] = zero16();
#pragma unroll
        for (int s = 0; s < DS; ++s)
          st[a] = mfma32x32x16(ld_frag16(kb + (32 * a + c) * KLD + 16 * s + 8 * g), qf[s], st[a]);
      }
      if (k0 + BN - 1 > q0w) {  // tile straddles the diagonal (or the end)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * a + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key > qi) st[a][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[a][r]);
      mx = fmaxf(mx, wave_xor32(mx));
      const float mnew = fmaxf(m, mx * sl2);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      m = mnew;
      float ps = 0.0f;
      bf16x8 pf[2][2];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          float p[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            p[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[a][8 * t + j], sl2, -mnew));
            ps += p[j];
          }
          pf[a][t] = pack_bf16x8(p);
        }
      l = l * alpha + ps;
#pragma unroll
      for (int e = 0; e < DE; ++e) {
        ot[e] *= alpha;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int t = 0; t < 2; ++t)
            ot[e] = mfma32x32x16(ld_frag_split(vb + (32 * e + c) * VLD + 32 * a + 16 * t + 4 * g),
                                 pf[a][t], ot[e]);
      }
    }
    if (more) {
      ks.store_rowmajor(Ks[buf ^ 1], KLD, tid);
      vs.store_transposed(Vt[buf ^ 1], VLD, tid);
    }
    __syncthreads();
  }

  const float lt = l + wave_xor32(l);
  if (qi < T) {
    const float inv = 1.0f / lt;
    uint16_t* orow = O + head + (size_t)qi * D;
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
template <int D>
__global__ __launch_bounds__(kThreads, D == 64 ? 2 : 1) void attn_bwd_dq(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ O,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE,
    uint16_t* __restrict__ dQ, float* __restrict__ Delta, int N, int T,
    float sl2, float scale, int nqb) {
  constexpr int BM = 128, BN = 64;
  constexpr int KLD = D + 8;
  constexpr int TLD = BN + 4;
  constexpr int DS = D / 16;
  constexpr int DE = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * KLD];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][BN * KLD];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[2][D * TLD];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int c = lane & 31, g = lane >> 5;
  const int bid = blockIdx.x;
  const int qb = nqb - 1 - bid / N;
  const int n = bid % N;
  const size_t head = (size_t)n * T * D;
  const int q0 = qb * BM;
  const int q0w = q0 + 32 * w;
  const int qi = q0w + c;

  bf16x8 qf[DS], df[DS];
  float dpart = 0.0f;
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    if (qi < T) {
      const size_t off = head + (size_t)qi * D + 16 * s + 8 * g;
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
  const float delta = dpart + wave_xor32(dpart);
  const float lse2 = qi < T ? LSE[(size_t)n * T + qi] * kLog2e : 0.0f;
  if (qi < T && g == 0) Delta[(size_t)n * T + qi] = delta;

  const int kend = min(q0 + BM, T);
  const int nkt = (kend - 1) / BN + 1;
  const int wnkt = q0w < T ? (min(q0w + 32, T) - 1) / BN + 1 : 0;

  TileStage<BN, D, kThreads> ks, vs;
  ks.load(K + head, T, tid);
  vs.load(V + head, T, tid);
  ks.store_rowmajor(Ks[0], KLD, tid);
  ks.store_transposed(Kt[0], TLD, tid);
  vs.store_rowmajor(Vs[0], KLD, tid);
  __syncthreads();

  f32x16 acc[DE];
#pragma unroll
  for (int e = 0; e < DE; ++e) acc[e] = zero16();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nkt;
    if (more) {
      const int k1 = (kt + 1) * BN;
      ks.load(K + head + (size_t)k1 * D, T - k1, tid);
      vs.load(V + head + (size_t)k1 * D, T - k1, tid);
    }
    if (kt < wnkt) {
      const int k0 = kt * BN;
      const uint16_t* kb = Ks[buf];
      const uint16_t* vb = Vs[buf];
      const uint16_t* tb = Kt[buf];
      f32x16 st[2], dp[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        st[a] = zero16();
        dp[a] = zero16();
#pragma unroll
        for (int s = 0; s < DS; ++s) {
          st[a] = mfma32x32x16(ld_frag16(kb + (32 * a + c) * KLD + 16 * s + 8 * g), qf[s], st[a]);
          dp[a] = mfma32x32x16(ld_frag16(vb + (32 * a + c) * KLD + 16 * s + 8 * g), df[s], dp[a]);
        }
      }
      const bool diag = k0 + BN - 1 > q0w;
      bf16x8 sf[2][2];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          float ds[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int r = 8 * t + j;
            float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[a][r], sl2, -lse2));
            if (diag) {
              const int key = k0 + 32 * a + 8 * (r >> 2) + 4 * g + (r & 3);
              if (key > qi) p = 0.0f;
            }
            ds[j] = p * (dp[a][r] - delta);
          }
          sf[a][t] = pack_bf16x8(ds);
        }
#pragma unroll
      for (int e = 0; e < DE; ++e)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int t = 0; t < 2; ++t)
            acc[e] = mfma32x32x16(ld_frag_split(tb + (32 * e + c) * TLD + 32 * a + 16 * t + 4 * g),
                                  sf[a][t], acc[e]);
    }
    if (more) {
      ks.store_rowmajor(Ks[buf ^ 1], KLD, tid);
      ks.store_transposed(Kt[buf ^ 1], TLD, tid);
      vs.store_rowmajor(Vs[buf ^ 1], KLD, tid);
    }
    __syncthreads();
  }

  if (qi < T) {
    uint16_t* row = dQ + head + (size_t)qi * D;
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
template <int D, int BM>
__global__ __launch_bounds__(kThreads, D == 64 ? 2 : 1) void attn_bwd_dkdv(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Delta,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N, int T,
    float sl2, float scale, int nkb) {
  constexpr int BN = 128;
  constexpr int NH = BM / 32;   // 32-query halves per query tile
  constexpr int RLD = D + 8;    // row-major Q / dO tiles
  constexpr int TLD = BM + 4;   // transposed Q / dO tiles
  constexpr int DS = D / 16;
  constexpr int DE = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[2][BM * RLD];
  __shared__ __attribute__((aligned(16))) uint16_t Qt[2][D * TLD];
  __shared__ __attribute__((aligned(16))) uint16_t Ds[2][BM * RLD];
  __shared__ __attribute__((aligned(16))) uint16_t Dt[2][D * TLD];
  __shared__ __attribute__((aligned(16))) float Ls[2][BM];
  __shared__ __attribute__((aligned(16))) float Es[2][BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int c = lane & 31, g = lane >> 5;
  const int bid = blockIdx.x;
  const int kb = bid / N;  // block 0 (the most queries) first
  const int n = bid % N;
  const size_t head = (size_t)n * T * D;
  const size_t rows = (size_t)n * T;
  const int k0 = kb * BN;
  const int k0w = k0 + 32 * w;
  const int kj = k0w + c;

  bf16x8 kf[DS], vf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    if (kj < T) {
      const size_t off = head + (size_t)kj * D + 16 * s + 8 * g;
      kf[s] = ld_frag16(K + off);
      vf[s] = ld_frag16(V + off);
    } else {
      kf[s] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      vf[s] = kf[s];
    }
  }

  const int qt0 = k0 / BM;
  const int nqt = (T + BM - 1) / BM;

  TileStage<BM, D, kThreads> qs, ds;
  float lv = 0.0f, ev = 0.0f;
  auto load_tile = [&](int qt) {
    const int q1 = qt * BM;
    qs.load(Q + head + (size_t)q1 * D, T - q1, tid);
    ds.load(dO + head + (size_t)q1 * D, T - q1, tid);
    if (tid < BM) {
      const int q = q1 + tid;
      lv = q < T ? LSE[rows + q] * kLog2e : INFINITY;
      ev = q < T ? Delta[rows + q] : 0.0f;
    }
  };
  auto store_tile = [&](int b) {
    qs.store_rowmajor(Qs[b], RLD, tid);
    qs.store_transposed(Qt[b], TLD, tid);
    ds.store_rowmajor(Ds[b], RLD, tid);
    ds.store_transposed(Dt[b], TLD, tid);
    if (tid < BM) {
      Ls[b][tid] = lv;
      Es[b][tid] = ev;
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
      const uint16_t* qb = Qs[buf];
      const uint16_t* db = Ds[buf];
      const uint16_t* qtb = Qt[buf];
      const uint16_t* dtb = Dt[buf];
      const bool diag = k0w + 31 > q0;
      bf16x8 pf[NH][2], sf[NH][2];
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        f32x16 st = zero16(), dp = zero16();
#pragma unroll
        for (int s = 0; s < DS; ++s) {
          st = mfma32x32x16(ld_frag16(qb + (32 * h + c) * RLD + 16 * s + 8 * g), kf[s], st);
          dp = mfma32x32x16(ld_frag16(db + (32 * h + c) * RLD + 16 * s + 8 * g), vf[s], dp);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          float p[8], dsv[8];
#pragma unroll
          for (int u2 = 0; u2 < 2; ++u2) {
            const int rowb = 32 * h + 16 * t + 8 * u2 + 4 * g;  // 4 consecutive query rows
            const f32x4 lq = *reinterpret_cast<const f32x4*>(&Ls[buf][rowb]);
            const f32x4 eq = *reinterpret_cast<const f32x4*>(&Es[buf][rowb]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 8 * t + 4 * u2 + i;
              float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(st[r], sl2, -lq[i]));
              if (diag && kj > q0 + rowb + i) pv = 0.0f;
              p[4 * u2 + i] = pv;
              dsv[4 * u2 + i] = pv * (dp[r] - eq[i]);
            }
          }
          pf[h][t] = pack_bf16x8(p);
          sf[h][t] = pack_bf16x8(dsv);
        }
      }
#pragma unroll
      for (int e = 0; e < DE; ++e)
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int off = (32 * e + c) * TLD + 32 * h + 16 * t + 4 * g;
            dvt[e] = mfma32x32x16(ld_frag_split(dtb + off), pf[h][t], dvt[e]);
            dkt[e] = mfma32x32x16(ld_frag_split(qtb + off), sf[h][t], dkt[e]);
          }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (kj < T) {
    uint16_t* krow = dK + head + (size_t)kj * D;
    uint16_t* vrow = dV + head + (size_t)kj * D;
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
