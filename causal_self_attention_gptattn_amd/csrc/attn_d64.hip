// dK / dV of causal attention at head size 64 without dropout, for gfx950
// (bf16 storage, float32 accumulation).
//
// The operation is the one attn_bf16.hip computes (lecture description
// "Let's build GPT: from scratch, in code, spelled out", chapters "version 3:
// adding softmax" and "version 4: self-attention"; the chain rule of the
// softmax for the backward pass).  This kernel serves the most common head
// size of the pages' models (GPT-2 124M / XL: 64) on sequences longer than
// 256 keys, and is organised around what bounds it on this chip:
//
//  * Every wave owns 32 keys and runs all four products on
//    v_mfma_f32_32x32x16_bf16: each 1 KiB operand read from LDS feeds 32
//    cycles of matrix work, half the LDS bytes per product of the 16 x 16 x 32
//    product, and 128 keys per workgroup halve the Q/dO tile copies per key
//    against 64.
//  * Q/dO tiles go HBM -> LDS (no registers) through a ring of three
//    buffers: the copy of tile t + 2 is issued as tile t starts, and a wave
//    waits only for the copies older than the newest one, so each copy has
//    two tiles of time to land.  One workgroup barrier per tile.
//  * Row statistics enter the products as accumulator seeds instead of
//    vector work: S starts at -lse/scale and dP at -delta (both stored by the
//    dQ kernel, copied in with the tile), so P = exp2(S * scale * log2 e) and
//    dS = P * dP.
//  * Every tile runs the same products; a tile that straddles the edge of
//    visibility differs only in how its weights are formed (masked element
//    by element), so the accumulators never leave their registers.
#include "attn_common.h"
#include "launch.h"

namespace gptattn {

namespace {

constexpr int kD = 64;

template <typename... Args>
hipError_t launch_kernel(void (*kern)(Args...), long long blocks, int threads,
                         hipStream_t stream, Args... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), dim3((unsigned)blocks),
                         dim3(threads), argv, 0, stream);
}

View view_of(const TensorArg& t) {
  return View{static_cast<const uint16_t*>(t.data), t.sb, t.sh, t.st};
}
constexpr int kQT = 64;  // rows per staged tile

// Seeds of a 32-row block of a 32 x 32 result from a per-row LDS vector:
// lane (c, g) holds rows 8i + 4g + {0..3}, i = 0..3.
__device__ __forceinline__ f32x16 row_seed(const float* v, int g) {
  f32x16 s;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(v + 8 * i + 4 * g);
#pragma unroll
    for (int r = 0; r < 4; ++r) s[4 * i + r] = x[r];
  }
  return s;
}

// ---------------------------------------------------------------------------
// dK / dV.  Lane (c, g) of wave w owns key k0 + 32w + c.  Per staged 64-query
// tile and 32-query half hb:
//   S  = Q K^T      (rows = queries, columns = keys; seeded with -lse/scale)
//   dP = dO V^T     (seeded with -delta)
//   P  = exp2(S * scale * log2 e),  dS = P * dP          (float32, registers)
//   dV^T += dO^T P,  dK^T += Q^T dS   (dO^T, Q^T read transposed from LDS)
// K and V stay in registers as the B operands of S and dP; P and dS are the B
// operands of the dV / dK products without any shuffle (the query order of
// the result rows is the k order of the transposed reads, as in the forward).
// ---------------------------------------------------------------------------
struct DkdvLane {
  int fo[4];          // fragment reads: row c, chunk 2s + g
  int tlo[2], thi[2];  // transposed reads: rows trr, trr + 8, columns 32e + trc
};

struct DkdvHalf {
  f32x16 s, dp;
};

// S and dP of half hb of the tile (q: Q tile, d: dO tile, st: seeds).
__device__ __forceinline__ DkdvHalf dkdv_scores(const uint16_t* q, const uint16_t* d,
                                                const float* ls, const float* es, int hb,
                                                const bf16x8* kf, const bf16x8* vf,
                                                const DkdvLane& sw, int g) {
  DkdvHalf h;
  h.s = row_seed(ls + 32 * hb, g);
  h.dp = row_seed(es + 32 * hb, g);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    h.s = mfma32x32x16(ld_frag16(q + 32 * hb * kD + sw.fo[s]), kf[s], h.s);
    h.dp = mfma32x32x16(ld_frag16(d + 32 * hb * kD + sw.fo[s]), vf[s], h.dp);
  }
  return h;
}

// P (for dV) and dS (for dK) of a half as bf16 operands, two 16-query k-steps.
template <bool MASK>
__device__ __forceinline__ void dkdv_weights(const DkdvHalf& h, float sl2, bf16x8* pf,
                                             bf16x8* sf, int q0, Span seers, int g) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    float p[8], ds[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 8 * t + j;
      float pv = __builtin_amdgcn_exp2f(h.s[r] * sl2);
      if (MASK && !inside(q0 + 8 * (r >> 2) + 4 * g + (r & 3), seers)) pv = 0.0f;
      p[j] = pv;
      ds[j] = pv * h.dp[r];
    }
    pf[t] = pack_bf16x8(p);
    sf[t] = pack_bf16x8(ds);
  }
}

// One 64-query tile for one wave.  Every product of both halves is issued
// on every tile; only the weights differ between a tile that crosses the
// edge of visibility (masked element by element; a half no query of which
// sees the wave's keys gets zero weights) and an interior one.  So the dV/dK
// accumulators go through the same products on every path and stay in their
// registers.  Per half: the S and dP products with the half's transposed
// operand reads behind them, the weights, then the dV and dK products with
// the next half's reads behind them.  The scheduling groups pin that order
// (the compiler would otherwise issue each operand read right before its
// product and wait for it there).
__device__ __forceinline__ void dkdv_tile(const uint16_t* q, const uint16_t* d, const float* ls,
                                          const float* es, const bf16x8* kf, const bf16x8* vf,
                                          f32x16* dvt, f32x16* dkt, const DkdvLane& sw,
                                          float sl2, int g, bool masked, int q0, Span seers) {
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const DkdvHalf h = dkdv_scores(q, d, ls, es, hb, kf, vf, sw, g);
    // A operands of the half's dV and dK products: dO^T and Q^T, read
    // transposed, k-steps t of 16 queries, head-dim blocks e
    bf16x8 td[4], tq[4];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int rb = (32 * hb + 16 * t) * kD;
        td[2 * e + t] = ld_frag_tr2(d + rb + sw.tlo[e], d + rb + sw.thi[e]);
        tq[2 * e + t] = ld_frag_tr2(q + rb + sw.tlo[e], q + rb + sw.thi[e]);
      }
    if (hb == 0) {
      __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
      }
    } else {
      // (same region as half 0's dV/dK products, issued first)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
    bf16x8 pf[2], sf[2];
    if (masked)
      dkdv_weights<true>(h, sl2, pf, sf, q0 + 32 * hb, seers, g);
    else
      dkdv_weights<false>(h, sl2, pf, sf, 0, Span{0, 0}, g);
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        dvt[e] = mfma32x32x16(td[2 * e + t], pf[t], dvt[e]);
        dkt[e] = mfma32x32x16(tq[2 * e + t], sf[t], dkt[e]);
      }
  }
}

// Workgroup = NW waves x 32 keys of one head; walks the 64-query tiles that
// see its keys, from the diagonal to the end, through a ring of three LDS
// buffers: the copy of tile t + 2 is issued as tile t starts, so a copy has
// two tiles of time to land.  A buffer holds the Q and dO tiles (unpadded,
// swizzled) and the tile's seeds: -delta and -lse/scale per query, stored by
// the dQ kernel in the workspace and copied in like the tiles.  Two waves
// per SIMD.
template <int NW>
__global__ __launch_bounds__(64 * NW, 2) void attn_bwd_dkdv64(
    View Q, View K, View V, View dO, const float* __restrict__ Seeds, View dK, View dV,
    Problem pb) {
  constexpr int D = kD, QT = kQT, NT = 64 * NW, KB = 32 * NW;
  constexpr int BUF = 2 * QT * D + 4 * QT;  // elements: Q, dO, then -delta and -lse/scale
  // one array per buffer, so the compiler sees that a copy into one leaves
  // the others alone (reads need not wait for it)
  __shared__ __attribute__((aligned(16))) uint16_t B0[BUF], B1[BUF], B2[BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, g = lane >> 5;
  const int bid = blockIdx.x;
  const int kb = bid / pb.N;  // key blocks from the first (the longest walk)
  const int n = bid % pb.N;
  const uint16_t* Qh = head_of(Q, n, pb.H);
  const uint16_t* Dh = head_of(dO, n, pb.H);
  const long long rows = (long long)n * pb.Tq;
  const float* Eh = Seeds + rows;                             // -delta
  const float* Lh = Seeds + (long long)pb.N * pb.Tq + rows;  // -lse/scale
  const int k0 = kb * KB;
  const int k0w = k0 + 32 * w;
  const int kj = k0w + c;

  DkdvLane sw;
  {
    const int trr = tr_rowoff(lane), trc = tr_coloff(lane);
#pragma unroll
    for (int s = 0; s < 4; ++s) sw.fo[s] = swz<D>(c, 16 * s + 8 * g);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      sw.tlo[e] = swz<D>(trr, 32 * e + trc);
      sw.thi[e] = swz<D>(trr + 8, 32 * e + trc);
    }
  }

  // this lane's key and value rows: B operands of S = Q K^T and dP = dO V^T
  bf16x8 kf[4], vf[4];
  {
    RowBlock kr, vr;
    kr.init(head_of(K, n, pb.H) + (long long)k0w * K.st, pb.Tk - k0w, K.st, c);
    vr.init(head_of(V, n, pb.H) + (long long)k0w * V.st, pb.Tk - k0w, V.st, c);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      kf[s] = __builtin_bit_cast(bf16x8, kr.load(16 * s + 8 * g));
      vf[s] = __builtin_bit_cast(bf16x8, vr.load(16 * s + 8 * g));
    }
  }

  // query tiles seen by the workgroup's keys
  const int qlo = queries_lo(k0, pb), qhi = queries_hi(min(k0 + KB, pb.Tk) - 1, pb);
  const int qt0 = qlo / QT, qt1 = qhi >= qlo ? qhi / QT : qt0 - 1;
  const Span seers = queries_of(kj, pb);

  TileDMA<QT, D, NT> qs, ds;
  qs.init(tid, Q.st);
  ds.init(tid, dO.st);
  // Copy of tile qt into buffer b: every wave moves its share of Q and dO;
  // wave 0 also moves the seeds (16 lanes x 16 bytes each vector, zero past
  // the last query).  Per wave the copy is kDmaW instructions (wave 0:
  // kDmaW + 2), which the waits below count.
  auto load_tile = [&](int qt, uint16_t* b) {
    const int q1 = qt * QT, valid = pb.Tq - q1;
    qs.load(Qh + (long long)q1 * Q.st, valid, b);
    ds.load(Dh + (long long)q1 * dO.st, valid, b + QT * D);
    if (w == 0 && lane < 16) {
      const int cnt = valid <= 0 ? 0 : valid < QT ? valid : QT;
      const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(Eh + q1), 0, __builtin_amdgcn_readfirstlane(cnt * 4), kBufferWord3);
      const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(Lh + q1), 0, __builtin_amdgcn_readfirstlane(cnt * 4), kBufferWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(re, (lds_void*)(b + 2 * QT * D), 16, lane * 16, 0,
                                               0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_void*)(b + 2 * QT * D + 2 * QT), 16,
                                               lane * 16, 0, 0, 0);
    }
  };
  constexpr int kDmaW = 2 * (QT * D / 8 / NT);  // Q and dO instructions per wave
  static_assert(kDmaW + 2 < 16, "vmcnt field");
  // wait until at most one tile's copy is outstanding (the one issued last)
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

  if (qt1 >= qt0) load_tile(qt0, B0);
  if (qt1 >= qt0 + 1) {
    load_tile(qt0 + 1, B1);
    wait_all_but_one();
  } else {
    wait_vm();
  }
  __syncthreads();

  f32x16 dvt[2], dkt[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    dvt[e] = zero16();
    dkt[e] = zero16();
  }

  // Tile qt from buffer cur; the copy of tile qt + 2 goes into buffer nxt
  // (free: its tile qt - 1 was finished before the last barrier).  Before the
  // barrier, wait for the copy of tile qt + 1.
  auto step = [&](int qt, const uint16_t* cur, uint16_t* nxt) __attribute__((always_inline)) {
    const bool two = qt + 2 <= qt1;
    if (two) load_tile(qt + 2, nxt);
    const int q0 = qt * QT;
    dkdv_tile(cur, cur + QT * D, ls_of(cur), es_of(cur), kf, vf, dvt, dkt, sw, pb.sl2, g,
              needs_mask(q0, q0 + QT - 1, k0w, k0w + 31, pb), q0, seers);
    if (two)
      wait_all_but_one();
    else
      wait_vm();
    __syncthreads();
  };
  for (int qt = qt0; qt <= qt1; qt += 3) {
    step(qt, B0, B2);
    if (qt + 1 <= qt1) step(qt + 1, B1, B0);
    if (qt + 2 <= qt1) step(qt + 2, B2, B1);
  }

  // epilogue: lane (c, g) holds key c's head dims 32e + 8u + 4g + i, the
  // layout store_rows takes; 16 rows per wave staged in the buffers
  constexpr int LD = D + 8;
  static_assert(2 * 16 * LD <= BUF, "two waves' epilogue staging must fit one buffer");
  static_assert(NW == 2 || NW == 4, "two or four waves per workgroup");
  uint16_t* stage = (w < 2 ? B0 : B1) + (w & 1) * 16 * LD;
  store_rows<D>(stage, dkt, pb.scale,
                const_cast<uint16_t*>(head_of(dK, n, pb.H)) + (long long)k0w * dK.st, dK.st,
                pb.Tk - k0w, lane);
  store_rows<D>(stage, dvt, 1.0f,
                const_cast<uint16_t*>(head_of(dV, n, pb.H)) + (long long)k0w * dV.st, dV.st,
                pb.Tk - k0w, lane);
}


// store_rows (attn_common.h) for a staging area that only the calling wave
// uses: wave_lds_order replaces the workgroup barriers, and the waves of a
// workgroup store their rows independently.

__device__ __forceinline__ void store_rows_wave(uint16_t* lds, const f32x16* acc, float mul,
                                                uint16_t* out, int rows_valid, int lane) {
  constexpr int D = kD, RS = D + 8, DE = D / 32, CPR = D / 8, PASS = 16 * CPR / 64;
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
    wave_lds_order();
#pragma unroll
    for (int p = 0; p < PASS; ++p) {
      const int ch = lane + 64 * p, r = ch / CPR, cc = ch % CPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(lds + r * RS + 8 * cc);
      const int row = 16 * half + r;
      if (row < rows_valid) *reinterpret_cast<u32x4*>(out + (long long)row * D + 8 * cc) = v;
    }
    wave_lds_order();
  }
}

// The same kernel as a persistent grid, for dense tensors ([B][H][T][64],
// rows contiguous): one workgroup per slot (two per CU), each walking a list
// of (head, 128-key block) items.  The tile copies form one stream across
// the items of a workgroup, so the three-buffer ring runs on from one item
// into the next: the next item's first tiles are copied while the current
// item's last tiles are computed, and the per-item start-up latency of a
// one-shot workgroup is hidden.
//
// Item order: items sorted longest walk first (key block 0 of every head,
// then key block 1, ...).  With X = 8 groups (heads n with n mod 8 = x;
// workgroup g runs on XCD g mod 8, so a head's items stay on one XCD and its
// tiles in one L2) and R workgroups per group, the workgroup with rank r in
// its group takes the group's items r, 2R - 1 - r, 2R + r, 4R - 1 - r, ...:
// a long item is paired with a short one, which balances the walks.
template <int NW>
__global__ __launch_bounds__(64 * NW, 2) void attn_bwd_dkdv64p(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ Seeds, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
    Problem pb, int items, int R, int X) {
  constexpr int D = kD, QT = kQT, NT = 64 * NW, KB = 32 * NW;
  constexpr int BUF = 2 * QT * D + 4 * QT;
  constexpr int LD = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t B0[BUF], B1[BUF], B2[BUF];
  __shared__ __attribute__((aligned(16))) uint16_t Stg[NW * 16 * LD];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, g = lane >> 5;
  const int x = blockIdx.x % X, r = blockIdx.x / X;
  const int NX = pb.N / X, M = items / X;  // heads and items per group

  // k-th item of this workgroup: head n, first key k0 (-1 past the end),
  // query tiles qt0..qt1
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
    const int kb = m / NX;
    it.n = X * (m - kb * NX) + x;
    it.k0 = kb * KB;
    const int qlo = queries_lo(it.k0, pb), qhi = queries_hi(min(it.k0 + KB, pb.Tk) - 1, pb);
    it.qt0 = qlo / QT;
    it.qt1 = qhi >= qlo ? qhi / QT : it.qt0 - 1;
    return it;
  };

  DkdvLane sw;
  {
    const int trr = tr_rowoff(lane), trc = tr_coloff(lane);
#pragma unroll
    for (int s = 0; s < 4; ++s) sw.fo[s] = swz<D>(c, 16 * s + 8 * g);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      sw.tlo[e] = swz<D>(trr, 32 * e + trc);
      sw.thi[e] = swz<D>(trr + 8, 32 * e + trc);
    }
  }

  TileDMA<QT, D, NT> qs;
  qs.init(tid, D);
  const long long NTq = (long long)pb.N * pb.Tq;
  // copy of tile qt of head n into buffer b (as in attn_bwd_dkdv64)
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
  constexpr int kDmaW = 2 * (QT * D / 8 / NT);
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

  // K and V rows of an item's 32 keys for this wave: B operands of S and dP
  auto load_kv = [&](const Item& it, bf16x8* kf, bf16x8* vf) {
    const int k0w = it.k0 + 32 * w;
    const long long row = (long long)it.n * pb.Tk + k0w;
    RowBlock kr, vr;
    kr.init(K + row * D, pb.Tk - k0w, D, c);
    vr.init(V + row * D, pb.Tk - k0w, D, c);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      kf[s] = __builtin_bit_cast(bf16x8, kr.load(16 * s + 8 * g));
      vf[s] = __builtin_bit_cast(bf16x8, vr.load(16 * s + 8 * g));
    }
  };
  uint16_t* stage = Stg + w * 16 * LD;
  auto store_item = [&](const Item& it, const f32x16* dkt, const f32x16* dvt) {
    const int k0w = it.k0 + 32 * w;
    const long long row = (long long)it.n * pb.Tk + k0w;
    store_rows_wave(stage, dkt, pb.scale, dK + row * D, pb.Tk - k0w, lane);
    store_rows_wave(stage, dvt, 1.0f, dV + row * D, pb.Tk - k0w, lane);
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
  bf16x8 kf[4], vf[4];
  load_kv(ci, kf, vf);
  const bool c0 = copy_next(B0);
  const bool c1 = c0 && copy_next(B1);
  if (c1)
    wait_all_but_one();
  else
    wait_vm();
  __syncthreads();

  // One tile position of item ci: copy the position two ahead into nxt
  // (possibly the next item's), compute tile qt from cur.
  f32x16 dvt[2], dkt[2];
  auto step = [&](int qt, const uint16_t* cur, uint16_t* nxt) {
    const bool more = copy_next(nxt);
    const int q0 = qt * QT, k0w = ci.k0 + 32 * w;
    dkdv_tile(cur, cur + QT * D, ls_of(cur), es_of(cur), kf, vf, dvt, dkt, sw, pb.sl2, g,
              needs_mask(q0, q0 + QT - 1, k0w, k0w + 31, pb), q0, queries_of(k0w + c, pb));
    if (more)
      wait_all_but_one();
    else
      wait_vm();
    __syncthreads();
  };

  // Before each tile position: if item ci has no tile left, store its dK and
  // dV and move on to the next item with tiles (loading its K and V rows).
  // False when the workgroup's items are done.
  int ck = 0, qt = ci.qt0;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    dvt[e] = zero16();
    dkt[e] = zero16();
  }
  auto advance = [&]() {
    while (qt > ci.qt1) {
      store_item(ci, dkt, dvt);
      ci = item_at(++ck);
      if (ci.k0 < 0) return false;
      load_kv(ci, kf, vf);
      qt = ci.qt0;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        dvt[e] = zero16();
        dkt[e] = zero16();
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

int cu_count(hipStream_t stream) {
  static int cache[64];
  int dev = 0;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cache[dev] = n;
  }
  return cache[dev];
}

hipError_t launch_bwd_dkdv_d64(const TensorArg& q, const TensorArg& k, const TensorArg& v,
                               const TensorArg& dO, const float* lse, const float* delta,
                               const TensorArg& dk, const TensorArg& dv, const ProblemArg& p,
                               hipStream_t stream) {
  constexpr int NW = 4;
  (void)lse;  // the seeds in the workspace carry lse
  const Problem pb = make_problem(p);
  const long long items = (long long)pb.N * ((p.Tk + 32 * NW - 1) / (32 * NW));
  const long long slots = 2LL * cu_count(stream);
  // dense [B][H][T][64] tensors and more items than slots: the persistent
  // grid, one workgroup per slot, in eight groups of heads (one per XCD)
  // when the heads and the grid split evenly
  auto dense = [&](const TensorArg& t, long long T) { return dense_bhtd(t, p.H, T, kD); };
  if (slots > 0 && items > slots && dense(q, p.Tq) && dense(dO, p.Tq) && dense(k, p.Tk) &&
      dense(v, p.Tk) && dense(dk, p.Tk) && dense(dv, p.Tk)) {
    const int X = (pb.N % 8 == 0 && slots % 8 == 0) ? 8 : 1;
    const int R = (int)(slots / X);
    auto P = [](const TensorArg& t) { return static_cast<const uint16_t*>(t.data); };
    auto W = [](const TensorArg& t) { return const_cast<uint16_t*>(static_cast<const uint16_t*>(t.data)); };
    return launch_kernel(attn_bwd_dkdv64p<NW>, slots, 64 * NW, stream, P(q), P(k), P(v), P(dO),
                         delta, W(dk), W(dv), pb, (int)items, R, X);
  }
  return launch_kernel(attn_bwd_dkdv64<NW>, items, 64 * NW, stream, view_of(q), view_of(k),
                       view_of(v), view_of(dO), delta, view_of(dk), view_of(dv), pb);
}

}  // namespace gptattn
