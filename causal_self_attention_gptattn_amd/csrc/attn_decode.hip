// Forward pass for short query blocks (decoding): at most kDecQ queries per
// head-problem against a context of Tk keys, bfloat16, no dropout.
//
// Same operation as attn_fwd (lecture description "Let's build GPT: from
// scratch, in code, spelled out", chapters "version 3: adding softmax" and
// "version 4: self-attention"; queries appended after a context as when
// sampling one token at a time, nanoGPT README's sample.py), arranged for
// the shape: with one query there is nothing to multiply on the matrix
// cores, and the work is reading K and V once.  The causal forward kernel
// would give each head one workgroup with a single busy wave; here one
// workgroup of 1024 threads covers a head and every thread streams keys.
//
// Layout: a key is read by a group of G = D / 8 consecutive threads, each
// holding a 16-byte slice (8 dims) of the key and value rows; the 1024 / G
// groups stride over the visible keys.  Each group keeps its own online
// softmax state per query (running max m, sum l, and its slice of the
// weighted value sum); the score of a key is the dot product reduced across
// the group with DPP row operations.  At the end the groups' states are
// merged, first across the groups of a wave with lane exchanges, then across
// the 16 waves through LDS, and the first threads write O and lse.
#include "attn_common.h"
#include "launch.h"

namespace gptattn {

namespace {

constexpr int kDecQ = 4;          // queries per head-problem this kernel takes
constexpr int kDecThreads = 1024;
constexpr int kDecWaves = kDecThreads / 64;

// Sum over aligned groups of G lanes (G = 8 or 16), result in every lane
// of the group.  DPP: swap neighbours, swap pairs, mirror within 8 lanes,
// then (G = 16) mirror within 16 lanes.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
  if (G == 16)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
  return x;
}

// Online-softmax state of one query in log2 units: weights 2^(s - m).
struct State {
  float m, l;
  float acc[8];
};

// Merge state b into a (both may be empty: m = -inf, l = 0).
__device__ __forceinline__ void merge(State& a, float bm, float bl, const float* bacc) {
  const float mm = fmaxf(a.m, bm);
  const float fa = a.m > -INFINITY ? __builtin_amdgcn_exp2f(a.m - mm) : 0.0f;
  const float fb = bm > -INFINITY ? __builtin_amdgcn_exp2f(bm - mm) : 0.0f;
  a.l = a.l * fa + bl * fb;
#pragma unroll
  for (int d = 0; d < 8; ++d) a.acc[d] = a.acc[d] * fa + bacc[d] * fb;
  a.m = mm;
}

__device__ __forceinline__ void unpack8(const u32x4& u, float* f) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = bf16_lo(u[j]);
    f[2 * j + 1] = bf16_hi(u[j]);
  }
}

template <int D>
__global__ __launch_bounds__(kDecThreads) void attn_decode(View Q, View K, View V, View O,
                                                           float* __restrict__ LSE, Problem pb) {
  constexpr int G = D / 8;              // threads per key
  constexpr int NG = kDecThreads / G;   // key groups per workgroup
  constexpr int GPW = 64 / G;           // key groups per wave
  __shared__ float red[kDecWaves][kDecQ][D + 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int sl = tid % G;   // this thread's 8-dim slice
  const int kg = tid / G;   // this thread's key group
  const int n = blockIdx.x;
  const int nq = pb.Tq;     // <= kDecQ (checked by the launcher)
  const uint16_t* Kh = head_of(K, n, pb.H) + 8 * sl;
  const uint16_t* Vh = head_of(V, n, pb.H) + 8 * sl;

  float qv[kDecQ][8];
  Span seen[kDecQ];
  State st[kDecQ];
#pragma unroll
  for (int i = 0; i < kDecQ; ++i) {
    seen[i] = i < nq ? keys_of(i, pb) : Span{1, 0};
    if (i < nq) {
      unpack8(*reinterpret_cast<const u32x4*>(head_of(Q, n, pb.H) + (long long)i * Q.st + 8 * sl),
              qv[i]);
    } else {
#pragma unroll
      for (int d = 0; d < 8; ++d) qv[i][d] = 0.0f;
    }
    st[i].m = -INFINITY;
    st[i].l = 0.0f;
#pragma unroll
    for (int d = 0; d < 8; ++d) st[i].acc[d] = 0.0f;
  }

  // keys any of the queries sees
  const int lo = keys_lo(0, pb), hi = keys_hi(nq - 1, pb);
  for (int j = lo + kg; j <= hi; j += NG) {
    const u32x4 ku = *reinterpret_cast<const u32x4*>(Kh + (long long)j * K.st);
    const u32x4 vu = *reinterpret_cast<const u32x4*>(Vh + (long long)j * V.st);
    float kf[8], vf[8];
    unpack8(ku, kf);
    unpack8(vu, vf);
#pragma unroll
    for (int i = 0; i < kDecQ; ++i) {
      if (i >= nq) break;
      float s = 0.0f;
#pragma unroll
      for (int d = 0; d < 8; ++d) s = __builtin_fmaf(qv[i][d], kf[d], s);
      s = group_sum<G>(s) * pb.sl2;
      if (!inside(j, seen[i])) continue;  // same key in the whole group
      if (s > st[i].m) {
        const float alpha = st[i].m > -INFINITY ? __builtin_amdgcn_exp2f(st[i].m - s) : 0.0f;
        st[i].l = st[i].l * alpha + 1.0f;
#pragma unroll
        for (int d = 0; d < 8; ++d) st[i].acc[d] = __builtin_fmaf(st[i].acc[d], alpha, vf[d]);
        st[i].m = s;
      } else {
        const float p = __builtin_amdgcn_exp2f(s - st[i].m);
        st[i].l += p;
#pragma unroll
        for (int d = 0; d < 8; ++d) st[i].acc[d] = __builtin_fmaf(p, vf[d], st[i].acc[d]);
      }
    }
  }

  // merge the key groups of this wave: partner groups are G, 2G, ... lanes away
#pragma unroll
  for (int i = 0; i < kDecQ; ++i) {
    if (i >= nq) break;
#pragma unroll
    for (int step = 1; step < GPW; step <<= 1) {
      const int off = step * G;
      float bacc[8];
#pragma unroll
      for (int d = 0; d < 8; ++d) bacc[d] = __shfl_xor(st[i].acc[d], off);
      const float bm = __shfl_xor(st[i].m, off);
      const float bl = __shfl_xor(st[i].l, off);
      merge(st[i], bm, bl, bacc);
    }
    if (lane < G) {
#pragma unroll
      for (int d = 0; d < 8; ++d) red[w][i][8 * sl + d] = st[i].acc[d];
      if (sl == 0) {
        red[w][i][D] = st[i].m;
        red[w][i][D + 1] = st[i].l;
      }
    }
  }
  __syncthreads();

  // merge across waves: thread (i, sl) for i < nq, sl < G
  if (tid < nq * G) {
    const int i = tid / G, s8 = tid % G;
    State a;
    a.m = -INFINITY;
    a.l = 0.0f;
#pragma unroll
    for (int d = 0; d < 8; ++d) a.acc[d] = 0.0f;
    for (int v = 0; v < kDecWaves; ++v) merge(a, red[v][i][D], red[v][i][D + 1], &red[v][i][8 * s8]);
    const float inv = a.l > 0.0f ? 1.0f / a.l : 0.0f;
    uint16_t* orow = const_cast<uint16_t*>(head_of(O, n, pb.H)) + (long long)i * O.st + 8 * s8;
    const u32x4 pk = {pack_bf16x2(a.acc[0] * inv, a.acc[1] * inv),
                      pack_bf16x2(a.acc[2] * inv, a.acc[3] * inv),
                      pack_bf16x2(a.acc[4] * inv, a.acc[5] * inv),
                      pack_bf16x2(a.acc[6] * inv, a.acc[7] * inv)};
    *reinterpret_cast<u32x4*>(orow) = pk;
    if (s8 == 0)
      LSE[(long long)n * pb.Tq + i] = a.l > 0.0f ? (a.m + log2f(a.l)) * kLn2 : -INFINITY;
  }
}

View view(const TensorArg& t) {
  return View{static_cast<const uint16_t*>(t.data), t.sb, t.sh, t.st};
}

}  // namespace

// Short query blocks against at least one full key tile: below that the
// tile kernel is just as fast and keeps its exact arithmetic.
// One workgroup of kDecThreads work-items per head: the dispatch counts
// work-items in 32 bits, so more than 2^32 / kDecThreads heads go to the
// tile kernel instead.
bool decode_applies(const ProblemArg& p) {
  return p.Tq <= kDecQ && p.Tk >= 64 && p.dropout <= 0.0f && (p.D == 64 || p.D == 128) &&
         (long long)p.B * p.H * kDecThreads < (1LL << 32);
}

hipError_t launch_decode_bf16(const TensorArg& q, const TensorArg& k, const TensorArg& v,
                              const TensorArg& o, float* lse, const ProblemArg& p,
                              hipStream_t stream) {
  if (!decode_applies(p)) return hipErrorInvalidValue;
  const Problem pb = make_problem(p);
  View vq = view(q), vk = view(k), vv = view(v), vo = view(o);
  void* argv[] = {&vq, &vk, &vv, &vo, &lse, const_cast<Problem*>(&pb)};
  const void* kern = p.D == 64 ? reinterpret_cast<const void*>(attn_decode<64>)
                               : reinterpret_cast<const void*>(attn_decode<128>);
  return hipLaunchKernel(kern, dim3((unsigned)(p.B * p.H)), dim3(kDecThreads), argv, 0, stream);
}

}  // namespace gptattn
