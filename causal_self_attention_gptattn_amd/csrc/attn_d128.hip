// dK / dV of causal attention at head size 128 without dropout, dense
// tensors, for gfx950 (bf16 storage, float32 accumulation).
//
// The operation is the one attn_bf16.hip computes (lecture description
// "Let's build GPT: from scratch, in code, spelled out", chapters "version 3:
// adding softmax" and "version 4: self-attention"; the chain rule of the
// softmax for the backward pass); this kernel serves the head size of the
// GPT-3 layers (minGPT README notes) once a problem has more (head, key
// block) items than the GPU has compute units.  Organised as the head-size-64
// kernel in attn_d64.hip, within the register and LDS budget of D = 128:
//
//  * Eight waves of 16 keys (the K and V rows of a wave take 32 registers and
//    its dK and dV accumulators 64, on the 16 x 16 x 32 product) make
//    workgroups of 128 keys, one per CU: each Q/dO tile copied into LDS serves
//    128 keys, twice as many as in the 64-key kernel.
//  * The Q/dO tiles go HBM -> LDS through a ring of three buffers (32.5 KiB
//    each, with the tile's seeds): the copy of tile t + 2 is issued as tile t
//    starts, so each copy has two tiles of time to land.
//  * S starts at -lse/scale and dP at -delta (the seeds the dQ kernel stores
//    in the workspace), so P = exp2(S * scale * log2 e) and dS = P * dP.
//  * A persistent grid: each workgroup walks a list of (head, 128-key block)
//    items, and the tile copies run on from one item into the next.
#include "attn_common.h"
#include "launch.h"

namespace gptattn {

namespace {

constexpr int kD = 128;
constexpr int kQT = 64;  // queries per staged tile
constexpr int kNW = 8;   // waves per workgroup, 16 keys each

template <typename... Args>
hipError_t launch_kernel(void (*kern)(Args...), long long blocks, int threads,
                         hipStream_t stream, Args... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), dim3((unsigned)blocks),
                         dim3(threads), argv, 0, stream);
}

// One 64-query tile for one wave (16 keys), in two halves of 32 queries.
// Lane (g, c) owns key c; S and dP come out with rows = queries 4g + r of
// each 16-query block b (S seeded with -lse/scale, dP with -delta from the
// tile's seeds ls and es); P and dS of two blocks are packed into one
// operand each, and dV^T / dK^T (rows = head dims 16m + 4g + r, columns =
// keys) accumulate with dO^T / Q^T read transposed from the swizzled tiles.
// Blocks outside [hb0, hb1] hold no query that sees the wave's keys.
template <bool MASK>
__device__ __forceinline__ void d128_tile(const uint16_t* qb, const uint16_t* db, const float* ls,
                                          const float* es, const bf16x8* kf, const bf16x8* vf,
                                          f32x4* dvt, f32x4* dkt, int q0, Span seers, int g,
                                          const int* fo, const int* tlo, int hb0, int hb1,
                                          float sl2) {
  constexpr int D = kD, NS = D / 32, NM = D / 16;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    if (MASK && (2 * kk + 1 < hb0 || 2 * kk > hb1)) continue;
    f32x4 st[2], dp[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int b = 2 * kk + bb;
      if (MASK && (b < hb0 || b > hb1)) {
        st[bb] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[bb] = st[bb];
        continue;
      }
      st[bb] = *reinterpret_cast<const f32x4*>(ls + 16 * b + 4 * g);
      dp[bb] = *reinterpret_cast<const f32x4*>(es + 16 * b + 4 * g);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        st[bb] = mfma16x16x32(ld_frag16(qb + 16 * b * D + fo[s]), kf[s], st[bb]);
        dp[bb] = mfma16x16x32(ld_frag16(db + 16 * b * D + fo[s]), vf[s], dp[bb]);
      }
    }
    float p[8], dsv[8];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int b = 2 * kk + bb;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float pv = __builtin_amdgcn_exp2f(st[bb][r] * sl2);
        if (MASK && !inside(q0 + 16 * b + 4 * g + r, seers)) pv = 0.0f;
        p[4 * bb + r] = pv;
        dsv[4 * bb + r] = pv * dp[bb][r];
      }
    }
    const bf16x8 pf = pack_bf16x8(p), sf = pack_bf16x8(dsv);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int lo = 32 * kk * D + tlo[m], hi = lo + 16 * D;
      dvt[m] = mfma16x16x32(ld_frag_tr2(db + lo, db + hi), pf, dvt[m]);
      dkt[m] = mfma16x16x32(ld_frag_tr2(qb + lo, qb + hi), sf, dkt[m]);
    }
  }
}

// Stores a wave's 16 rows of dK or dV (lane (g, c) holds key c's head dims
// 16m + 4g + r) through an LDS staging area of its own, whole rows at a time.
__device__ __forceinline__ void store_rows16_wave(uint16_t* stage, const f32x4* acc, float mul,
                                                  uint16_t* out, int rows_valid, int lane) {
  constexpr int D = kD, NM = D / 16, LD = D + 8, CPR = D / 8;
  const int c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const u32x2 pk = {pack_bf16x2(acc[m][0] * mul, acc[m][1] * mul),
                      pack_bf16x2(acc[m][2] * mul, acc[m][3] * mul)};
    *reinterpret_cast<u32x2*>(stage + c * LD + 16 * m + 4 * g) = pk;
  }
  wave_lds_order();
#pragma unroll
  for (int p = 0; p < 16 * CPR / 64; ++p) {
    const int ch = lane + 64 * p, r = ch / CPR, cc = ch % CPR;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * LD + 8 * cc);
    if (r < rows_valid) *reinterpret_cast<u32x4*>(out + (long long)r * D + 8 * cc) = v;
  }
  wave_lds_order();
}

// Persistent grid, one workgroup per CU.  Items and their order as in the
// head-size-64 persistent kernel (attn_d64.hip): sorted longest walk first,
// dealt in snake order within X groups of heads (one per XCD when X = 8).
// On problems of many rounds the heads of an XCD group are further taken in
// groups of HX (a group's items sorted longest first, the groups one after
// the other), so that a head's Q/dO tiles, which every key block of the head
// walks, are re-read close together in time and stay cached; HX = N / X is
// the plain order.
template <int NW>
__global__ __launch_bounds__(64 * NW, 1) void attn_bwd_dkdv128p(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ Seeds, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
    Problem pb, int items, int R, int X, int HX) {
  constexpr int D = kD, QT = kQT, NT = 64 * NW, KB = 16 * NW, NS = D / 32, NM = D / 16;
  constexpr int BUF = 2 * QT * D + 4 * QT;  // elements: Q, dO, then -delta and -lse/scale
  constexpr int LD = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t B0[BUF], B1[BUF], B2[BUF];
  __shared__ __attribute__((aligned(16))) uint16_t Stg[NW * 16 * LD];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int x = blockIdx.x % X, r = blockIdx.x / X;
  const int NX = pb.N / X, M = items / X, nkb = M / NX;

  struct Item {
    int n, k0, qt0, qt1;
  };
  auto item_at = [&](int k) {
    Item it;
    const int m = (k & 1) ? (k + 1) * R - 1 - r : k * R + r;
    if (m >= M) {
      it.n = 0;
      it.k0 = -1;
      it.qt0 = 0;
      it.qt1 = -1;
      return it;
    }
    const int per = HX * nkb, gi = m / per, rr = m - gi * per;
    const int h0 = gi * HX, gn = min(HX, NX - h0);
    const int kb = rr / gn;
    it.n = X * (h0 + rr - kb * gn) + x;
    it.k0 = kb * KB;
    const int qlo = queries_lo(it.k0, pb), qhi = queries_hi(min(it.k0 + KB, pb.Tk) - 1, pb);
    it.qt0 = qlo / QT;
    it.qt1 = qhi >= qlo ? qhi / QT : it.qt0 - 1;
    return it;
  };

  int fo[NS], tlo[NM];
#pragma unroll
  for (int s = 0; s < NS; ++s) fo[s] = swz<D, true>(c, 32 * s + 8 * g);
#pragma unroll
  for (int m = 0; m < NM; ++m) tlo[m] = swz<D, true>(4 * g + (c >> 2), 16 * m + 4 * (c & 3));

  TileDMA<QT, D, NT, true> qs;
  qs.init(tid, D);
  const long long NTq = (long long)pb.N * pb.Tq;
  auto load_tile = [&](int n, int qt, uint16_t* b) {
    const int q1 = qt * QT, valid = pb.Tq - q1;
    const long long row = (long long)n * pb.Tq + q1;
    qs.load(Q + row * D, valid, b);
    qs.load(dO + row * D, valid, b + QT * D);
    if (w == 0 && lane < 16) {
      const int cnt = valid <= 0 ? 0 : valid < QT ? valid : QT;
      const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(Seeds + row), 0, __builtin_amdgcn_readfirstlane(cnt * 4),
          kBufferWord3);
      const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(Seeds + NTq + row), 0, __builtin_amdgcn_readfirstlane(cnt * 4),
          kBufferWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(re, (lds_void*)(b + 2 * QT * D), 16, lane * 16, 0,
                                               0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_void*)(b + 2 * QT * D + 2 * QT), 16,
                                               lane * 16, 0, 0, 0);
    }
  };
  constexpr int kDmaW = 2 * (QT * D / 8 / NT);  // Q and dO instructions per wave
  static_assert(kDmaW + 2 < 16, "vmcnt field");
  auto wait_all_but_one = [&]() {
    if (w == 0)
      wait_vm_upto<kDmaW + 2>();
    else
      wait_vm_upto<kDmaW>();
  };
  auto es_of = [](const uint16_t* b) { return reinterpret_cast<const float*>(b + 2 * QT * D); };
  auto ls_of = [](const uint16_t* b) {
    return reinterpret_cast<const float*>(b + 2 * QT * D) + QT;
  };

  auto load_kv = [&](const Item& it, bf16x8* kf, bf16x8* vf) {
    const int k0w = it.k0 + 16 * w;
    const long long row = (long long)it.n * pb.Tk + k0w;
    RowBlock kr, vr;
    kr.init(K + row * D, pb.Tk - k0w, D, c);
    vr.init(V + row * D, pb.Tk - k0w, D, c);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      kf[s] = __builtin_bit_cast(bf16x8, kr.load(32 * s + 8 * g));
      vf[s] = __builtin_bit_cast(bf16x8, vr.load(32 * s + 8 * g));
    }
  };
  uint16_t* stage = Stg + w * 16 * LD;
  auto store_item = [&](const Item& it, const f32x4* dkt, const f32x4* dvt) {
    const int k0w = it.k0 + 16 * w;
    const long long row = (long long)it.n * pb.Tk + k0w;
    store_rows16_wave(stage, dkt, pb.scale, dK + row * D, pb.Tk - k0w, lane);
    store_rows16_wave(stage, dvt, 1.0f, dV + row * D, pb.Tk - k0w, lane);
  };

  // the copy cursor: item ordinal dk (item di), next tile dqt
  int dk = 0;
  Item di = item_at(0);
  int dqt = di.qt0;
  auto copy_next = [&](uint16_t* b) {
    while (di.k0 >= 0 && dqt > di.qt1) {
      di = item_at(++dk);
      dqt = di.qt0;
    }
    if (di.k0 < 0) return false;
    load_tile(di.n, dqt, b);
    ++dqt;
    return true;
  };

  Item ci = item_at(0);
  if (ci.k0 < 0) return;
  bf16x8 kf[NS], vf[NS];
  load_kv(ci, kf, vf);
  const bool c0 = copy_next(B0);
  const bool c1 = c0 && copy_next(B1);
  if (c1)
    wait_all_but_one();
  else
    wait_vm();
  __syncthreads();

  // One tile position of item ci: copy the position two ahead into nxt
  // (possibly the next item's), compute tile qt from cur unless no query of
  // the tile sees this wave's keys.
  f32x4 dvt[NM], dkt[NM];
  auto step = [&](int qt, const uint16_t* cur, uint16_t* nxt) {
    const bool more = copy_next(nxt);
    const int q0 = qt * QT, k0w = ci.k0 + 16 * w;
    const int wqlo = queries_lo(k0w, pb);
    const int wqhi = k0w < pb.Tk ? queries_hi(min(k0w + 15, pb.Tk - 1), pb) : -1;
    if (q0 + QT - 1 >= wqlo && q0 <= wqhi) {
      const Span seers = queries_of(k0w + c, pb);
      if (needs_mask(q0, q0 + QT - 1, k0w, k0w + 15, pb)) {
        const int hb0 = max(0, (wqlo - q0) >> 4), hb1 = min(QT / 16 - 1, (wqhi - q0) >> 4);
        d128_tile<true>(cur, cur + QT * D, ls_of(cur), es_of(cur), kf, vf, dvt, dkt, q0, seers,
                        g, fo, tlo, hb0, hb1, pb.sl2);
      } else {
        d128_tile<false>(cur, cur + QT * D, ls_of(cur), es_of(cur), kf, vf, dvt, dkt, q0, seers,
                         g, fo, tlo, 0, QT / 16 - 1, pb.sl2);
      }
    }
    if (more)
      wait_all_but_one();
    else
      wait_vm();
    __syncthreads();
  };

  // Before each tile position: if item ci has no tile left, store its dK and
  // dV and move on to the next item (loading its K and V rows).  False when
  // the workgroup's items are done.
  int ck = 0, qt = ci.qt0;
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    dvt[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    dkt[m] = dvt[m];
  }
  auto advance = [&]() {
    while (qt > ci.qt1) {
      store_item(ci, dkt, dvt);
      ci = item_at(++ck);
      if (ci.k0 < 0) return false;
      load_kv(ci, kf, vf);
      qt = ci.qt0;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        dvt[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        dkt[m] = dvt[m];
      }
    }
    return true;
  };
  // The ring goes B0, B1, B2 position by position, across item boundaries.
  for (;;) {
    if (!advance()) break;
    step(qt++, B0, B2);
    if (!advance()) break;
    step(qt++, B1, B0);
    if (!advance()) break;
    step(qt++, B2, B1);
  }
}

}  // namespace

bool dkdv_d128_applies(const TensorArg& q, const TensorArg& k, const TensorArg& v,
                       const TensorArg& dO, const TensorArg& dk, const TensorArg& dv,
                       const ProblemArg& p, hipStream_t stream) {
  if (p.D != kD || p.dropout > 0.0f) return false;
  const long long items = (long long)p.B * p.H * ((p.Tk + 16 * kNW - 1) / (16 * kNW));
  const long long slots = cu_count(stream);
  return slots > 0 && items > slots && dense_bhtd(q, p.H, p.Tq, kD) &&
         dense_bhtd(dO, p.H, p.Tq, kD) && dense_bhtd(k, p.H, p.Tk, kD) &&
         dense_bhtd(v, p.H, p.Tk, kD) && dense_bhtd(dk, p.H, p.Tk, kD) &&
         dense_bhtd(dv, p.H, p.Tk, kD);
}

hipError_t launch_bwd_dkdv_d128(const TensorArg& q, const TensorArg& k, const TensorArg& v,
                                const TensorArg& dO, const float* delta, const TensorArg& dk,
                                const TensorArg& dv, const ProblemArg& p, hipStream_t stream) {
  const Problem pb = make_problem(p);
  const long long items = (long long)pb.N * ((p.Tk + 16 * kNW - 1) / (16 * kNW));
  const long long slots = cu_count(stream);
  const int X = (pb.N % 8 == 0 && slots % 8 == 0) ? 8 : 1;
  const int R = (int)(slots / X);
  // heads of each XCD group in groups of about four rounds of the grid on
  // problems of at least sixteen rounds (whole heads per XCD group; at
  // twelve rounds, the GPT-3 layer at batch 2, the plain order measured
  // 1.7% faster, at 24 rounds the groups 5.4%)
  int HX = pb.N / X;
  if (X == 8 && items >= 16 * slots) {
    const long long groups = (items + 4 * slots - 1) / (4 * slots);
    const long long hx = (HX + groups - 1) / groups;
    HX = (int)(hx < HX ? hx : HX);
  }
  auto P = [](const TensorArg& t) { return static_cast<const uint16_t*>(t.data); };
  auto W = [](const TensorArg& t) {
    return const_cast<uint16_t*>(static_cast<const uint16_t*>(t.data));
  };
  return launch_kernel(attn_bwd_dkdv128p<kNW>, slots, 64 * kNW, stream, P(q), P(k), P(v), P(dO),
                       delta, W(dk), W(dv), pb, (int)items, R, X, HX);
}

}  // namespace gptattn
