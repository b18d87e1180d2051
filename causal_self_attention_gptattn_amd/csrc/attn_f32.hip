// Causal scaled dot-product self-attention with every step in float32
// (same operation as attn_bf16.hip; lecture description "Let's build GPT:
// from scratch, in code, spelled out", chapters "version 3: adding softmax"
// and "version 4: self-attention", note 6 and the 00:57:00 / 01:20:05
// corrections).
//
// This path exists for workloads that need float32 results (small heads,
// tight tolerances); it runs on the vector ALUs, one lane per query (forward
// and dQ) or per key (dK/dV), with 64-row tiles of the other operand staged
// in LDS and shared by the wave.  Nothing is rounded below float32.
#include "attn_common.h"
#include "launch.h"

namespace gptattn {

namespace {

constexpr int kRows = 64;  // lanes per workgroup and rows per staged tile

// Stage rows [r0, r0 + 64) of an [T][D] float matrix into LDS (zero past T).
template <int D>
__device__ __forceinline__ void stage_rows(float* dst, const float* __restrict__ src, int r0, int T,
                                           int tid) {
  constexpr int F4 = D / 4;
  for (int i = tid; i < kRows * F4; i += kRows) {
    const int row = i / F4, col = i % F4;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (r0 + row < T) v = *reinterpret_cast<const f32x4*>(src + (size_t)(r0 + row) * D + 4 * col);
    *reinterpret_cast<f32x4*>(dst + row * D + 4 * col) = v;
  }
}

template <int D>
__global__ __launch_bounds__(kRows) void attn_fwd_f32(const float* __restrict__ Q,
                                                      const float* __restrict__ K,
                                                      const float* __restrict__ V,
                                                      float* __restrict__ O,
                                                      float* __restrict__ LSE, int T,
                                                      float scale) {
  __shared__ __attribute__((aligned(16))) float Ks[kRows * D];
  __shared__ __attribute__((aligned(16))) float Vs[kRows * D];
  const int tid = threadIdx.x;
  const int nt = (T + kRows - 1) / kRows;
  const int n = blockIdx.x / nt;
  const int q0 = (blockIdx.x % nt) * kRows;
  const int qi = q0 + tid;
  const size_t head = (size_t)n * T * D;
  float q[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = qi < T ? Q[head + (size_t)qi * D + d] : 0.0f;
    acc[d] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  const int kend = min(q0 + kRows, T);
  for (int k0 = 0; k0 < kend; k0 += kRows) {
    stage_rows<D>(Ks, K + head, k0, T, tid);
    stage_rows<D>(Vs, V + head, k0, T, tid);
    __syncthreads();
    const int jmax = min(kRows, qi - k0 + 1);  // keys k0 + j <= qi
    for (int j = 0; j < jmax; ++j) {
      float s = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = __builtin_fmaf(q[d], Ks[j * D + d], s);
      s *= scale;
      if (s > m) {
        const float corr = expf(m - s);
        l = l * corr + 1.0f;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(acc[d], corr, Vs[j * D + d]);
        m = s;
      } else {
        const float p = expf(s - m);
        l += p;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(p, Vs[j * D + d], acc[d]);
      }
    }
    __syncthreads();
  }
  if (qi < T) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int d = 0; d < D; ++d) O[head + (size_t)qi * D + d] = acc[d] * inv;
    LSE[(size_t)n * T + qi] = m + logf(l);
  }
}

// delta_i = sum_d dO_id O_id, then dQ_i = scale sum_{j<=i} P_ij (dP_ij - delta_i) K_j
template <int D>
__global__ __launch_bounds__(kRows) void attn_bwd_dq_f32(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ O, const float* __restrict__ dO, const float* __restrict__ LSE,
    float* __restrict__ dQ, float* __restrict__ Delta, int T, float scale) {
  __shared__ __attribute__((aligned(16))) float Ks[kRows * D];
  __shared__ __attribute__((aligned(16))) float Vs[kRows * D];
  const int tid = threadIdx.x;
  const int nt = (T + kRows - 1) / kRows;
  const int n = blockIdx.x / nt;
  const int q0 = (blockIdx.x % nt) * kRows;
  const int qi = q0 + tid;
  const size_t head = (size_t)n * T * D;
  float q[D], g[D], acc[D];
  float delta = 0.0f;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const size_t off = head + (size_t)qi * D + d;
    q[d] = qi < T ? Q[off] : 0.0f;
    g[d] = qi < T ? dO[off] : 0.0f;
    delta = __builtin_fmaf(g[d], qi < T ? O[off] : 0.0f, delta);
    acc[d] = 0.0f;
  }
  const float lse = qi < T ? LSE[(size_t)n * T + qi] : 0.0f;
  if (qi < T) Delta[(size_t)n * T + qi] = delta;
  const int kend = min(q0 + kRows, T);
  for (int k0 = 0; k0 < kend; k0 += kRows) {
    stage_rows<D>(Ks, K + head, k0, T, tid);
    stage_rows<D>(Vs, V + head, k0, T, tid);
    __syncthreads();
    const int jmax = min(kRows, qi - k0 + 1);
    for (int j = 0; j < jmax; ++j) {
      float s = 0.0f, dp = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        s = __builtin_fmaf(q[d], Ks[j * D + d], s);
        dp = __builtin_fmaf(g[d], Vs[j * D + d], dp);
      }
      const float p = expf(s * scale - lse);
      const float ds = p * (dp - delta);
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(ds, Ks[j * D + d], acc[d]);
    }
    __syncthreads();
  }
  if (qi < T) {
#pragma unroll
    for (int d = 0; d < D; ++d) dQ[head + (size_t)qi * D + d] = acc[d] * scale;
  }
}

// dV_j = sum_{i>=j} P_ij dO_i,  dK_j = scale sum_{i>=j} P_ij (dP_ij - delta_i) Q_i
template <int D>
__global__ __launch_bounds__(kRows) void attn_bwd_dkdv_f32(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    float* __restrict__ dK, float* __restrict__ dV, int T, float scale) {
  __shared__ __attribute__((aligned(16))) float Qs[kRows * D];
  __shared__ __attribute__((aligned(16))) float Gs[kRows * D];
  __shared__ float Ls[kRows], Es[kRows];
  const int tid = threadIdx.x;
  const int nt = (T + kRows - 1) / kRows;
  const int n = blockIdx.x / nt;
  const int k0 = (blockIdx.x % nt) * kRows;
  const int kj = k0 + tid;
  const size_t head = (size_t)n * T * D;
  float k[D], v[D], dk[D], dv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const size_t off = head + (size_t)kj * D + d;
    k[d] = kj < T ? K[off] : 0.0f;
    v[d] = kj < T ? V[off] : 0.0f;
    dk[d] = 0.0f;
    dv[d] = 0.0f;
  }
  for (int q0 = k0; q0 < T; q0 += kRows) {
    stage_rows<D>(Qs, Q + head, q0, T, tid);
    stage_rows<D>(Gs, dO + head, q0, T, tid);
    const int qt = q0 + tid;
    Ls[tid] = qt < T ? LSE[(size_t)n * T + qt] : 0.0f;
    Es[tid] = qt < T ? Delta[(size_t)n * T + qt] : 0.0f;
    __syncthreads();
    const int imin = max(0, kj - q0);        // queries q0 + i >= kj
    const int imax = min(kRows, T - q0);
    for (int i = imin; i < imax; ++i) {
      float s = 0.0f, dp = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        s = __builtin_fmaf(Qs[i * D + d], k[d], s);
        dp = __builtin_fmaf(Gs[i * D + d], v[d], dp);
      }
      const float p = expf(s * scale - Ls[i]);
      const float ds = p * (dp - Es[i]);
#pragma unroll
      for (int d = 0; d < D; ++d) {
        dv[d] = __builtin_fmaf(p, Gs[i * D + d], dv[d]);
        dk[d] = __builtin_fmaf(ds, Qs[i * D + d], dk[d]);
      }
    }
    __syncthreads();
  }
  if (kj < T) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      dK[head + (size_t)kj * D + d] = dk[d] * scale;
      dV[head + (size_t)kj * D + d] = dv[d];
    }
  }
}

template <typename... Args>
hipError_t launch(void (*kern)(Args...), dim3 grid, hipStream_t stream, Args... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, dim3(kRows), argv, 0, stream);
}

template <int D>
hipError_t fwd_d(const float* q, const float* k, const float* v, float* o, float* lse, int N,
                 int T, float scale, hipStream_t stream) {
  const dim3 grid(N * ((T + kRows - 1) / kRows));
  return launch(attn_fwd_f32<D>, grid, stream, q, k, v, o, lse, T, scale);
}

template <int D>
hipError_t bwd_dq_d(const float* q, const float* k, const float* v, const float* o,
                    const float* dO, const float* lse, float* dq, float* delta, int N, int T,
                    float scale, hipStream_t stream) {
  const dim3 grid(N * ((T + kRows - 1) / kRows));
  return launch(attn_bwd_dq_f32<D>, grid, stream, q, k, v, o, dO, lse, dq, delta, T, scale);
}

template <int D>
hipError_t bwd_dkdv_d(const float* q, const float* k, const float* v, const float* dO,
                      const float* lse, const float* delta, float* dk, float* dv, int N, int T,
                      float scale, hipStream_t stream) {
  const dim3 grid(N * ((T + kRows - 1) / kRows));
  return launch(attn_bwd_dkdv_f32<D>, grid, stream, q, k, v, dO, lse, delta, dk, dv, T, scale);
}

}  // namespace

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int N, int T, int D, float scale, hipStream_t stream) {
  switch (D) {
    case 16: return fwd_d<16>(q, k, v, o, lse, N, T, scale, stream);
    case 32: return fwd_d<32>(q, k, v, o, lse, N, T, scale, stream);
    case 64: return fwd_d<64>(q, k, v, o, lse, N, T, scale, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_dq_f32(const float* q, const float* k, const float* v, const float* o,
                             const float* dO, const float* lse, float* dq, float* delta, int N,
                             int T, int D, float scale, hipStream_t stream) {
  switch (D) {
    case 16: return bwd_dq_d<16>(q, k, v, o, dO, lse, dq, delta, N, T, scale, stream);
    case 32: return bwd_dq_d<32>(q, k, v, o, dO, lse, dq, delta, N, T, scale, stream);
    case 64: return bwd_dq_d<64>(q, k, v, o, dO, lse, dq, delta, N, T, scale, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_dkdv_f32(const float* q, const float* k, const float* v, const float* dO,
                               const float* lse, const float* delta, float* dk, float* dv, int N,
                               int T, int D, float scale, hipStream_t stream) {
  switch (D) {
    case 16: return bwd_dkdv_d<16>(q, k, v, dO, lse, delta, dk, dv, N, T, scale, stream);
    case 32: return bwd_dkdv_d<32>(q, k, v, dO, lse, delta, dk, dv, N, T, scale, stream);
    case 64: return bwd_dkdv_d<64>(q, k, v, dO, lse, delta, dk, dv, N, T, scale, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gptattn
