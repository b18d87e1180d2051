// Causal scaled dot-product self-attention with every step in float32
// (same operation as attn_bf16.hip; lecture description "Let's build GPT:
// from scratch, in code, spelled out", chapters "version 3: adding softmax"
// and "version 4: self-attention", note 6 and the 00:57:00 / 01:20:05
// corrections).
//
// This path exists for workloads that need float32 results (small heads,
// tight tolerances); it runs on the vector ALUs, one lane per query (forward
// and dQ) or per key (dK/dV), with 64-row tiles of the other operand staged
// in LDS and shared by the wave.  Nothing is rounded below float32.  Each
// lane walks exactly the keys (or queries) its row can see under the
// visibility rule of attn_common.h.
#include "attn_common.h"
#include "launch.h"

namespace gptattn {

namespace {

constexpr int kRows = 64;  // lanes per workgroup and rows per staged tile

struct FView {
  const float* p;
  long long sb, sh, st;
};

__device__ __forceinline__ const float* head_of(const FView& v, int n, int H) {
  return gptattn::head_of(v.p, v.sb, v.sh, n, H);
}

// Stage rows [r0, r0 + 64) of one head (rows st floats apart, D contiguous)
// into a dense [64][D] LDS tile; rows at or past `rows` read as zero.
template <int D>
__device__ __forceinline__ void stage_rows(float* dst, const float* __restrict__ src,
                                           long long st, int r0, int rows, int tid) {
  constexpr int F4 = D / 4;
  for (int i = tid; i < kRows * F4; i += kRows) {
    const int row = i / F4, col = i % F4;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (r0 + row < rows)
      v = *reinterpret_cast<const f32x4*>(src + (long long)(r0 + row) * st + 4 * col);
    *reinterpret_cast<f32x4*>(dst + row * D + 4 * col) = v;
  }
}

// Keys query i sees: [lo, hi] (empty when hi < lo or i is past Tq).
__device__ __forceinline__ void key_range(int i, const Problem& pb, int& lo, int& hi) {
  lo = keys_lo(i, pb);
  hi = i < pb.Tq ? keys_hi(i, pb) : -1;
}

// Dropout factor of (query i, key j): 0 or the keep scale 2^16 / (2^16 - thr); `bits` caches the
// keep bits of the call covering j's group of four keys (and query i's
// pair), drawn when j starts a group.
template <bool DROP>
__device__ __forceinline__ float drop_factor(int i, int j, int j0, uint32_t n, uint32_t& bits,
                                             const Problem& pb) {
  if (!DROP) return 1.0f;
  if (j == j0 || (j & 3) == 0) bits = keep8((uint32_t)j >> 2, (uint32_t)i >> 1, n, pb);
  return ((bits >> (2 * (j & 3) + (i & 1))) & 1u) ? pb.inv_keep : 0.0f;
}

template <int D, bool DROP>
__global__ __launch_bounds__(kRows) void attn_fwd_f32(FView Q, FView K, FView V, FView O,
                                                      float* __restrict__ LSE, Problem pb,
                                                      int nt) {
  __shared__ __attribute__((aligned(16))) float Ks[kRows * D];
  __shared__ __attribute__((aligned(16))) float Vs[kRows * D];
  const int tid = threadIdx.x;
  const int n = blockIdx.x / nt;
  const int q0 = (blockIdx.x % nt) * kRows;
  const int qi = q0 + tid;
  const float* Kh = head_of(K, n, pb.H);
  const float* Vh = head_of(V, n, pb.H);
  const float* qr = head_of(Q, n, pb.H) + (long long)qi * Q.st;
  float q[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = qi < pb.Tq ? qr[d] : 0.0f;
    acc[d] = 0.0f;
  }
  int lo, hi;
  key_range(qi, pb, lo, hi);
  float m = -INFINITY, l = 0.0f;
  const int klo = keys_lo(q0, pb), khi = keys_hi(min(q0 + kRows, pb.Tq) - 1, pb);
  for (int k0 = klo / kRows * kRows; k0 <= khi; k0 += kRows) {
    stage_rows<D>(Ks, Kh, K.st, k0, pb.Tk, tid);
    stage_rows<D>(Vs, Vh, V.st, k0, pb.Tk, tid);
    __syncthreads();
    const int j0 = max(0, lo - k0), j1 = min(kRows - 1, hi - k0);
    uint32_t bits = 0;
    for (int j = j0; j <= j1; ++j) {
      float s = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = __builtin_fmaf(q[d], Ks[j * D + d], s);
      s *= pb.scale;
      // the normaliser l is the softmax's own; dropout scales what reaches O
      const float f = drop_factor<DROP>(qi, k0 + j, k0 + j0, n, bits, pb);
      if (s > m) {
        const float corr = expf(m - s);  // 0 for the first key (m = -inf)
        l = l * corr + 1.0f;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(acc[d], corr, f * Vs[j * D + d]);
        m = s;
      } else {
        const float p = expf(s - m);
        l += p;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(p * f, Vs[j * D + d], acc[d]);
      }
    }
    __syncthreads();
  }
  if (qi < pb.Tq) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;  // a row that sees no key outputs 0
    float* orow = const_cast<float*>(head_of(O, n, pb.H)) + (long long)qi * O.st;
#pragma unroll
    for (int d = 0; d < D; ++d) orow[d] = acc[d] * inv;
    LSE[(long long)n * pb.Tq + qi] = l > 0.0f ? m + logf(l) : -INFINITY;
  }
}

// delta_i = sum_d dO_id O_id, then dQ_i = scale sum_j P_ij (dP_ij - delta_i) K_j
// over the keys j that query i sees.
template <int D, bool DROP>
__global__ __launch_bounds__(kRows) void attn_bwd_dq_f32(FView Q, FView K, FView V, FView O,
                                                         FView dO, const float* __restrict__ LSE,
                                                         FView dQ, float* __restrict__ Delta,
                                                         Problem pb, int nt) {
  __shared__ __attribute__((aligned(16))) float Ks[kRows * D];
  __shared__ __attribute__((aligned(16))) float Vs[kRows * D];
  const int tid = threadIdx.x;
  const int n = blockIdx.x / nt;
  const int q0 = (blockIdx.x % nt) * kRows;
  const int qi = q0 + tid;
  const float* Kh = head_of(K, n, pb.H);
  const float* Vh = head_of(V, n, pb.H);
  const float* qr = head_of(Q, n, pb.H) + (long long)qi * Q.st;
  const float* gr = head_of(dO, n, pb.H) + (long long)qi * dO.st;
  const float* orr = head_of(O, n, pb.H) + (long long)qi * O.st;
  const bool live = qi < pb.Tq;
  float q[D], g[D], acc[D];
  float delta = 0.0f;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = live ? qr[d] : 0.0f;
    g[d] = live ? gr[d] : 0.0f;
    delta = __builtin_fmaf(g[d], live ? orr[d] : 0.0f, delta);
    acc[d] = 0.0f;
  }
  const long long row = (long long)n * pb.Tq + qi;
  const float lse = live ? LSE[row] : 0.0f;
  if (live) Delta[row] = delta;
  int lo, hi;
  key_range(qi, pb, lo, hi);
  const int klo = keys_lo(q0, pb), khi = keys_hi(min(q0 + kRows, pb.Tq) - 1, pb);
  for (int k0 = klo / kRows * kRows; k0 <= khi; k0 += kRows) {
    stage_rows<D>(Ks, Kh, K.st, k0, pb.Tk, tid);
    stage_rows<D>(Vs, Vh, V.st, k0, pb.Tk, tid);
    __syncthreads();
    const int j0 = max(0, lo - k0), j1 = min(kRows - 1, hi - k0);
    uint32_t bits = 0;
    for (int j = j0; j <= j1; ++j) {
      float s = 0.0f, dp = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        s = __builtin_fmaf(q[d], Ks[j * D + d], s);
        dp = __builtin_fmaf(g[d], Vs[j * D + d], dp);
      }
      const float p = expf(s * pb.scale - lse);
      const float f = drop_factor<DROP>(qi, k0 + j, k0 + j0, n, bits, pb);
      const float ds = p * (f * dp - delta);
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(ds, Ks[j * D + d], acc[d]);
    }
    __syncthreads();
  }
  if (live) {
    float* out = const_cast<float*>(head_of(dQ, n, pb.H)) + (long long)qi * dQ.st;
#pragma unroll
    for (int d = 0; d < D; ++d) out[d] = acc[d] * pb.scale;
  }
}

// dV_j = sum_i P_ij dO_i,  dK_j = scale sum_i P_ij (dP_ij - delta_i) Q_i over
// the queries i that see key j.
template <int D, bool DROP>
__global__ __launch_bounds__(kRows) void attn_bwd_dkdv_f32(FView Q, FView K, FView V, FView dO,
                                                           const float* __restrict__ LSE,
                                                           const float* __restrict__ Delta,
                                                           FView dK, FView dV, Problem pb,
                                                           int nt) {
  __shared__ __attribute__((aligned(16))) float Qs[kRows * D];
  __shared__ __attribute__((aligned(16))) float Gs[kRows * D];
  __shared__ float Ls[kRows], Es[kRows];
  const int tid = threadIdx.x;
  const int n = blockIdx.x / nt;
  const int k0 = (blockIdx.x % nt) * kRows;
  const int kj = k0 + tid;
  const float* Qh = head_of(Q, n, pb.H);
  const float* Gh = head_of(dO, n, pb.H);
  const float* kr = head_of(K, n, pb.H) + (long long)kj * K.st;
  const float* vr = head_of(V, n, pb.H) + (long long)kj * V.st;
  const long long rows = (long long)n * pb.Tq;
  const bool live = kj < pb.Tk;
  float k[D], v[D], dk[D], dv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    k[d] = live ? kr[d] : 0.0f;
    v[d] = live ? vr[d] : 0.0f;
    dk[d] = 0.0f;
    dv[d] = 0.0f;
  }
  // queries that see key kj: [lo, hi]
  const int lo = queries_lo(kj, pb);
  const int hi = live ? queries_hi(kj, pb) : -1;
  const int qlo = queries_lo(k0, pb), qhi = queries_hi(min(k0 + kRows, pb.Tk) - 1, pb);
  for (int q0 = qlo / kRows * kRows; q0 <= qhi; q0 += kRows) {
    stage_rows<D>(Qs, Qh, Q.st, q0, pb.Tq, tid);
    stage_rows<D>(Gs, Gh, dO.st, q0, pb.Tq, tid);
    const int qt = q0 + tid;
    Ls[tid] = qt < pb.Tq ? LSE[rows + qt] : 0.0f;
    Es[tid] = qt < pb.Tq ? Delta[rows + qt] : 0.0f;
    __syncthreads();
    const int i0 = max(0, lo - q0), i1 = min(kRows - 1, hi - q0);
    for (int i = i0; i <= i1; ++i) {
      float s = 0.0f, dp = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        s = __builtin_fmaf(Qs[i * D + d], k[d], s);
        dp = __builtin_fmaf(Gs[i * D + d], v[d], dp);
      }
      const float p = expf(s * pb.scale - Ls[i]);
      uint32_t bits = 0;
      const float f = drop_factor<DROP>(q0 + i, kj, kj, n, bits, pb);
      const float ds = p * (f * dp - Es[i]);
#pragma unroll
      for (int d = 0; d < D; ++d) {
        dv[d] = __builtin_fmaf(p * f, Gs[i * D + d], dv[d]);
        dk[d] = __builtin_fmaf(ds, Qs[i * D + d], dk[d]);
      }
    }
    __syncthreads();
  }
  if (live) {
    float* kw = const_cast<float*>(head_of(dK, n, pb.H)) + (long long)kj * dK.st;
    float* vw = const_cast<float*>(head_of(dV, n, pb.H)) + (long long)kj * dV.st;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      kw[d] = dk[d] * pb.scale;
      vw[d] = dv[d];
    }
  }
}

template <typename... Args>
hipError_t launch(void (*kern)(Args...), long long blocks, hipStream_t stream, Args... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), dim3((unsigned)blocks),
                         dim3(kRows), argv, 0, stream);
}

FView view(const TensorArg& t) {
  return FView{static_cast<const float*>(t.data), t.sb, t.sh, t.st};
}

template <int D>
hipError_t fwd_d(const TensorArg& q, const TensorArg& k, const TensorArg& v, const TensorArg& o,
                 float* lse, const ProblemArg& p, hipStream_t stream) {
  const int nt = (p.Tq + kRows - 1) / kRows;
  const long long blocks = (long long)p.B * p.H * nt;
  const Problem pb = make_problem(p);
  if (p.dropout > 0.0f)
    return launch(attn_fwd_f32<D, true>, blocks, stream, view(q), view(k), view(v), view(o), lse,
                  pb, nt);
  return launch(attn_fwd_f32<D, false>, blocks, stream, view(q), view(k), view(v), view(o), lse,
                pb, nt);
}

template <int D>
hipError_t bwd_dq_d(const TensorArg& q, const TensorArg& k, const TensorArg& v,
                    const TensorArg& o, const TensorArg& dO, const float* lse,
                    const TensorArg& dq, float* delta, const ProblemArg& p, hipStream_t stream) {
  const int nt = (p.Tq + kRows - 1) / kRows;
  const long long blocks = (long long)p.B * p.H * nt;
  const Problem pb = make_problem(p);
  if (p.dropout > 0.0f)
    return launch(attn_bwd_dq_f32<D, true>, blocks, stream, view(q), view(k), view(v), view(o),
                  view(dO), lse, view(dq), delta, pb, nt);
  return launch(attn_bwd_dq_f32<D, false>, blocks, stream, view(q), view(k), view(v), view(o),
                view(dO), lse, view(dq), delta, pb, nt);
}

template <int D>
hipError_t bwd_dkdv_d(const TensorArg& q, const TensorArg& k, const TensorArg& v,
                      const TensorArg& dO, const float* lse, const float* delta,
                      const TensorArg& dk, const TensorArg& dv, const ProblemArg& p,
                      hipStream_t stream) {
  const int nt = (p.Tk + kRows - 1) / kRows;
  const long long blocks = (long long)p.B * p.H * nt;
  const Problem pb = make_problem(p);
  if (p.dropout > 0.0f)
    return launch(attn_bwd_dkdv_f32<D, true>, blocks, stream, view(q), view(k), view(v),
                  view(dO), lse, delta, view(dk), view(dv), pb, nt);
  return launch(attn_bwd_dkdv_f32<D, false>, blocks, stream, view(q), view(k), view(v),
                view(dO), lse, delta, view(dk), view(dv), pb, nt);
}

}  // namespace

hipError_t launch_fwd_f32(const TensorArg& q, const TensorArg& k, const TensorArg& v,
                          const TensorArg& o, float* lse, const ProblemArg& p,
                          hipStream_t stream) {
  switch (p.D) {
    case 16: return fwd_d<16>(q, k, v, o, lse, p, stream);
    case 32: return fwd_d<32>(q, k, v, o, lse, p, stream);
    case 64: return fwd_d<64>(q, k, v, o, lse, p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_dq_f32(const TensorArg& q, const TensorArg& k, const TensorArg& v,
                             const TensorArg& o, const TensorArg& dO, const float* lse,
                             const TensorArg& dq, float* delta, const ProblemArg& p,
                             hipStream_t stream) {
  switch (p.D) {
    case 16: return bwd_dq_d<16>(q, k, v, o, dO, lse, dq, delta, p, stream);
    case 32: return bwd_dq_d<32>(q, k, v, o, dO, lse, dq, delta, p, stream);
    case 64: return bwd_dq_d<64>(q, k, v, o, dO, lse, dq, delta, p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_dkdv_f32(const TensorArg& q, const TensorArg& k, const TensorArg& v,
                               const TensorArg& dO, const float* lse, const float* delta,
                               const TensorArg& dk, const TensorArg& dv, const ProblemArg& p,
                               hipStream_t stream) {
  switch (p.D) {
    case 16: return bwd_dkdv_d<16>(q, k, v, dO, lse, delta, dk, dv, p, stream);
    case 32: return bwd_dkdv_d<32>(q, k, v, dO, lse, delta, dk, dv, p, stream);
    case 64: return bwd_dkdv_d<64>(q, k, v, dO, lse, delta, dk, dv, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gptattn
