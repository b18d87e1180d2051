// Causal scaled dot-product self-attention on gfx950 matrix cores, bfloat16
// storage, float32 accumulation.
//
// The operation (lecture description "Let's build GPT: from scratch, in
// code, spelled out": chapters "version 3: adding softmax" and "version 4:
// self-attention", note 6 and the corrections at 00:57:00 and 01:20:05; heads
// as a batch dimension per exercise EX1 and "batched multi-headed
// self-attention"):  O = softmax(scale Q K^T over the visible keys) V, with
// the natural-log normaliser lse kept for the backward pass.  Visibility is
// the causal rule, optionally shifted by an offset (queries appended to a
// longer context) and limited to a band of recent positions (the "locally
// banded" layers of GPT-3 in the minGPT README notes); see attn_common.h.
//
// Kernels (one wave = 64 lanes; the products are v_mfma_f32_32x32x16_bf16
// in attn_fwd and attn_bwd_dq, v_mfma_f32_16x16x32_bf16 in attn_bwd_dq16 and
// attn_bwd_dkdv16w; see attn_common.h for the register layouts):
//
//   attn_fwd      one workgroup = 128 queries of one head (4 waves x 32).
//                 Walks only the 64-key tiles its rows can see and masks
//                 only the tiles that straddle the edge of visibility.
//                 Scores are formed transposed, S^T = K Q^T, so that each
//                 lane owns one query: the online softmax (running max m and
//                 sum l) stays in registers, the row reductions need one
//                 cross-half exchange, and the bf16 probabilities feed
//                 O^T += V^T P^T straight from registers.  K and V are staged
//                 row-major in LDS; V^T is read with the gfx950 transpose
//                 read (attn_common.h).
//   attn_bwd_dq   D = 128; same tiling as attn_fwd.  First forms the row term
//                 delta_i = sum_d dO_id O_id (written to the workspace for
//                 attn_bwd_dkdv16w), then recomputes P^T from lse,
//                 dP^T = V dO^T, dS^T = P^T (dP^T - delta) and
//                 dQ^T += K^T dS^T.
//   attn_bwd_dq16 the same at D = 64 with 16 queries per wave on the
//                 16 x 16 x 32 product (four waves per SIMD instead of three).
//                 The forward and both dQ kernels run longest query blocks
//                 first; a problem of eight or more rounds of the GPU's
//                 workgroup slots takes its heads in groups (grouped_item;
//                 the forward at D = 128 only), so that each head's K/V tiles
//                 are re-read close together in time and stay cached.
//   attn_bwd_dkdv16w  one workgroup = 64 keys of one head (4 waves x 16).
//                 Walks the query tiles that see its keys with the
//                 lane -> key layout: S = Q K^T and dP = dO V^T, then
//                 dV^T += dO^T P and dK^T += Q^T dS with P and dS taken from
//                 registers.  Q and dO are staged row-major in LDS and read
//                 transposed for the dV/dK products.
//
// The tiles a workgroup walks (K/V, or Q/dO) are copied HBM -> LDS by the
// gfx950 buffer-load-to-LDS path into two alternating buffers, unpadded and
// swizzled (TileDMA in attn_common.h): the copy of the next tile runs while
// the current one is computed on, and costs no registers.
//
// dQ and dK/dV come from separate kernels, so no result is accumulated with
// atomics and every output is bitwise reproducible run to run.
#include "attn_common.h"
#include "launch.h"

namespace gptattn {

namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr float kLazy = 8.0f;  // log2 headroom before the running max is moved
constexpr int kBM = 128;       // queries per forward / dQ workgroup
constexpr int kBN = 64;        // keys per staged K/V tile
constexpr int kKBN16 = 64;     // keys per dK/dV workgroup (4 waves x 16)

// Key tiles [t0, t1] a query range sees (t1 < t0 when none).
struct TileSpan {
  int t0, t1;
};
__device__ __forceinline__ TileSpan key_tiles(int i0, int i1, const Problem& pb, int bn) {
  const int lo = keys_lo(i0, pb), hi = i0 < pb.Tq ? keys_hi(min(i1, pb.Tq - 1), pb) : -1;
  return TileSpan{lo / bn, hi >= lo ? hi / bn : lo / bn - 1};
}


// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------

// One 64-key tile for one wave (32 queries, one per lane column c), taken
// as two 32-key halves with one online-softmax step each, which keeps only
// half a tile of scores live.  A row that has seen no key yet keeps
// m = -inf; the guards keep -inf from meeting -inf.
template <int D, bool MASK, bool DROP>
__device__ __forceinline__ void fwd_tile(const uint16_t* kb, const uint16_t* vb, const bf16x8* qf,
                                         f32x16* ot, float& m, float& l, int k0, Span seen, int g,
                                         const SwzLane<D>& sw, int qi, uint32_t n, int h0, int h1,
                                         const Problem& pb) {
  // K and V tiles: unpadded rows of D, 16-byte chunks swizzled (swz)
  constexpr int DS = D / 16, DE = D / 32;
  // scheduling hint: interleave the LDS reads with the matrix products so
  // that more than one read is in flight (2-3% measured)
  __builtin_amdgcn_iglp_opt(0);
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    if (MASK && (a < h0 || a > h1)) continue;  // no row of the wave sees these 32 keys
    // S^T = K Q^T for 32 keys: rows = keys, columns = this wave's queries
    f32x16 st = mfma32x32x16(ld_frag16(kb + 32 * a * D + sw.fo[0]), qf[0], zero16());
#pragma unroll
    for (int s = 1; s < DS; ++s)
      st = mfma32x32x16(ld_frag16(kb + 32 * a * D + sw.fo[s]), qf[s], st);
    if (MASK) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 32 * a + 8 * (r >> 2) + 4 * g + (r & 3);
        if (!inside(key, seen)) st[r] = -INFINITY;
      }
    }
    float mx = st[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, st[r]);
    mx = half_max(mx) * pb.sl2;
    // Lazy rescaling: the reference max m only moves when some row of the
    // wave sees a score more than 2^kLazy above it.  Until then the
    // probabilities exp2(s - m) stay below 2^kLazy, which bf16 and the
    // float32 accumulators hold exactly as well; O and l share the same
    // reference, so the final O / l is unchanged.
    if (__any(mx > m + kLazy)) {
      const float mnew = fmaxf(m, mx);
      const float alpha = m > -INFINITY ? __builtin_amdgcn_exp2f(m - mnew) : 0.0f;
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int e = 0; e < DE; ++e) ot[e] *= alpha;
    }
    const float nm = m > -INFINITY ? -m : 0.0f;
    bf16x8 pf[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // dropout: keep bits of keys k0 + 32a + 16t + {0..3, 8..11} + 4g
      uint32_t kb0 = 0, kb1 = 0;
      if (DROP)
        keep_bits_pair((uint32_t)(k0 + 32 * a + 16 * t) / 4 + g, (uint32_t)qi, n, pb, kb0, kb1);
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(st[8 * t + j], pb.sl2, nm));
        l += pv;  // the normaliser is the softmax's own, before dropout
        if (DROP) pv = (((j < 4 ? kb0 : kb1) >> (j & 3)) & 1u) ? pv * pb.inv_keep : 0.0f;
        p[j] = pv;
      }
      pf[t] = pack_bf16x8(p);
    }
    // O^T += V^T P^T, V^T read transposed from the row-major V tile
#pragma unroll
    for (int e = 0; e < DE; ++e)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint16_t* vr = vb + (32 * a + 16 * t) * D;
        ot[e] = mfma32x32x16(ld_frag_tr2(vr + sw.tlo[e], vr + sw.thi[e]), pf[t], ot[e]);
      }
  }
}

// The item (index into the longest-first list of `items` workgroup items)
// that workgroup b runs.  The dispatcher fills the CUs breadth-first, so
// workgroups b, b + C, b + 2C, ... (C = `deal`, the CU count) share a CU;
// dealing every other round of C items in reverse order pairs long items with
// short ones on each CU.  Reversal is in groups of g (8 when the head count
// is a multiple of 8), so an item keeps its workgroup's index mod 8 and a
// head's workgroups stay on one XCD.  deal = 0: the list order itself.
__device__ __forceinline__ int dealt_item(int b, int items, int deal, int g) {
  if (deal <= 0) return b;
  const int r = b / deal, p = b - r * deal, base = r * deal;
  const int cnt = min(deal, items - base);
  if ((r & 1) == 0 || cnt % g != 0) return b;
  return base + (cnt / g - 1 - p / g) * g + p % g;
}

// Query block qb and head n of workgroup b when heads are taken in groups of
// hg (a multiple of 8, so a head's workgroups keep their index mod 8 and
// stay on one XCD when N is a multiple of 8): a group's workgroups run
// together, longest query blocks first, so each head's K/V tiles are re-read
// close together in time.  hg >= N: one group, the plain longest-first list.
struct QItem {
  int qb, n;
};
__device__ __forceinline__ QItem grouped_item(int b, int N, int nqb, int hg) {
  const int per = hg * nqb, gi = b / per, r = b - gi * per;
  const int h0 = gi * hg, gn = min(hg, N - h0);
  return QItem{nqb - 1 - r / gn, h0 + r % gn};
}

// Occupancy: four waves per SIMD at D = 64 (at most 128 registers), two at
// D = 128 (fits without spilling; 1.6x faster than one wave at the GPT-3
// shape).
template <int D, bool DROP>
__global__ __launch_bounds__(kThreads, D == 64 ? 4 : 2) void attn_fwd(
    View Q, View K, View V, View O, float* __restrict__ LSE, Problem pb, int nqb, int deal,
    int dealg, int hg) {
  constexpr int BM = kBM, BN = kBN;
  constexpr int LD = D + 8;     // row stride of the epilogue staging (padded)
  constexpr int DS = D / 16;    // k-steps of the score product
  constexpr int DE = D / 32;    // 32-row output tiles over the head dim
  // K and V tiles of the two buffers, copied in by the DMA (unpadded,
  // swizzled).  Separate arrays per buffer, and a loop unrolled by two, let
  // the compiler see that the copy into one buffer does not touch the one
  // being read, so reads do not wait for the copy.
  __shared__ __attribute__((aligned(16))) uint16_t K0[BN * D], K1[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t V0[BN * D], V1[BN * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int c = lane & 31, g = lane >> 5;
  SwzLane<D> sw;
  sw.init(c, g, tr_rowoff(lane), tr_coloff(lane));
  const int bid = blockIdx.x;
  // longest query blocks first (heads in groups on large problems), dealt
  // over the CUs
  const QItem qit = grouped_item(dealt_item(bid, nqb * pb.N, deal, dealg), pb.N, nqb, hg);
  const int qb = qit.qb;
  const int n = qit.n;
  const uint16_t* Kh = head_of(K, n, pb.H);
  const uint16_t* Vh = head_of(V, n, pb.H);
  const int q0 = qb * BM;
  const int q0w = q0 + 32 * w;
  const int qi = q0w + c;

  bf16x8 qf[DS];  // this lane's query row (zero past Tq)
  {
    // (the row block's start taken as the uniform value it is, so the load
    // needs no loop over distinct descriptors)
    const int q0u = __builtin_amdgcn_readfirstlane(q0w);
    RowBlock qr;
    qr.init(head_of(Q, n, pb.H) + (long long)q0u * Q.st, pb.Tq - q0u, Q.st, c);
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[s] = __builtin_bit_cast(bf16x8, qr.load(16 * s + 8 * g));
  }

  // key tiles seen by the workgroup's rows, and by this wave's rows
  const TileSpan ws = key_tiles(q0, q0 + BM - 1, pb, BN);
  const TileSpan wv = key_tiles(q0w, q0w + 31, pb, BN);
  const int wlast = min(q0w + 31, pb.Tq - 1);
  const Span seen = keys_of(qi, pb);  // keys this lane's query sees
  // keys some row of this wave sees (32-key halves outside are skipped)
  const int wklo = keys_lo(q0w, pb), wkhi = keys_hi(wlast, pb);

  TileDMA<BN, D, kThreads> ks, vs;
  ks.init(tid, K.st);
  vs.init(tid, V.st);
  auto load_tile = [&](int kt, int valid, uint16_t* kd, uint16_t* vd) {
    const int k1 = kt * BN;
    ks.load(Kh + (long long)k1 * K.st, valid, kd);
    vs.load(Vh + (long long)k1 * V.st, valid, vd);
  };
  // first tile (reads nothing when the workgroup sees no key)
  load_tile(ws.t0, ws.t1 >= ws.t0 ? pb.Tk - ws.t0 * BN : 0, K0, V0);
  wait_dma();
  __syncthreads();

  f32x16 ot[DE];
#pragma unroll
  for (int e = 0; e < DE; ++e) ot[e] = zero16();
  float m = -INFINITY, l = 0.0f;

  // one tile: compute on (kc, vc) while the next tile is copied into (kn, vn)
  auto step = [&](int kt, const uint16_t* kc, const uint16_t* vc, uint16_t* kn, uint16_t* vn) {
    const bool more = kt < ws.t1;
    if (more) load_tile(kt + 1, pb.Tk - (kt + 1) * BN, kn, vn);
    if (kt >= wv.t0 && kt <= wv.t1) {
      const int k0 = kt * BN;
      if (needs_mask(q0w, wlast, k0, k0 + BN - 1, pb)) {
        fwd_tile<D, true, DROP>(kc, vc, qf, ot, m, l, k0, seen, g, sw, qi, n,
                                k0 + 31 < wklo ? 1 : 0, k0 + 32 > wkhi ? 0 : 1, pb);
      } else {
        fwd_tile<D, false, DROP>(kc, vc, qf, ot, m, l, k0, seen, g, sw, qi, n, 0, 1, pb);
      }
    }
    if (more) wait_dma();  // this wave's copies have landed; the barrier publishes them
    __syncthreads();
  };
  for (int kt = ws.t0; kt <= ws.t1; kt += 2) {
    step(kt, K0, V0, K1, V1);
    if (kt + 1 <= ws.t1) step(kt + 1, K1, V1, K0, V0);
  }

  const float lt = half_sum(l);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;  // a row that sees no key outputs 0
  if (qi < pb.Tq && g == 0)
    LSE[(long long)n * pb.Tq + qi] = lt > 0.0f ? (m + log2f(lt)) * kLn2 : -INFINITY;
  // the K tiles are free after the loop's last barrier: 16 rows per wave
  static_assert(2 * 16 * LD <= BN * D, "two waves' epilogue staging must fit one K tile");
  store_rows<D>((w < 2 ? K0 : K1) + (w & 1) * 16 * LD, ot, inv,
                const_cast<uint16_t*>(head_of(O, n, pb.H)) + (long long)q0w * O.st, O.st,
                pb.Tq - q0w, lane);
}

// ---------------------------------------------------------------------------
// Backward, part 1: row term delta and dQ (lane -> query layout)
// ---------------------------------------------------------------------------

// One 64-key tile for one wave of the dQ kernel, taken as two 32-key
// halves.  nd holds -delta of this lane's query in all 16 slots; it seeds
// the dP^T accumulator so that the product directly yields dP^T - delta.
// nl is -lse * log2(e), -inf for a row that sees no key (then P = 0).
template <int D, bool MASK, bool DROP>
__device__ __forceinline__ void dq_tile(const uint16_t* kb, const uint16_t* vb, const bf16x8* qf,
                                        const bf16x8* df, const f32x16& nd, f32x16* acc, int k0,
                                        Span seen, int g, const SwzLane<D>& sw, float nl, int qi,
                                        uint32_t n, int h0, int h1, const Problem& pb) {
  // K and V tiles: unpadded rows of D, 16-byte chunks swizzled (swz)
  constexpr int DS = D / 16, DE = D / 32;
  // scheduling hint: interleave the LDS reads with the matrix products so
  // that more than one read is in flight (2-3% measured)
  __builtin_amdgcn_iglp_opt(0);
  // The halves go one after the other.  Issuing both halves' score
  // products first would let the matrix cores run half 1 while the vector
  // units turn half 0 into dS, but the registers it takes cost a wave per
  // SIMD: three waves instead of two at D = 64 (3% faster), two instead of
  // one at D = 128 (1.5x faster at the GPT-3 shape).
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    if (MASK && (a < h0 || a > h1)) continue;  // no row of the wave sees these 32 keys
    // S^T = K Q^T and dP^T - delta = V dO^T - delta: rows = keys, columns = queries
    f32x16 st = mfma32x32x16(ld_frag16(kb + 32 * a * D + sw.fo[0]), qf[0], zero16());
    f32x16 dp = mfma32x32x16(ld_frag16(vb + 32 * a * D + sw.fo[0]), df[0], nd);
#pragma unroll
    for (int s = 1; s < DS; ++s) {
      st = mfma32x32x16(ld_frag16(kb + 32 * a * D + sw.fo[s]), qf[s], st);
      dp = mfma32x32x16(ld_frag16(vb + 32 * a * D + sw.fo[s]), df[s], dp);
    }
    bf16x8 sf[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint32_t kb0 = 0, kb1 = 0;
      if (DROP)
        keep_bits_pair((uint32_t)(k0 + 32 * a + 16 * t) / 4 + g, (uint32_t)qi, n, pb, kb0, kb1);
      float ds[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 8 * t + j;
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[r], pb.sl2, nl));
        if (MASK) {
          const int key = k0 + 32 * a + 8 * (r >> 2) + 4 * g + (r & 3);
          if (!inside(key, seen)) p = 0.0f;
        }
        if (DROP) {
          // dp holds dO.V - delta; the dropped-out weight's gradient is
          // M * s * dO.V (s: the keep scale), so dS = P * (M * s * dO.V - delta)
          const float delta = -nd[0];
          const bool keep = ((j < 4 ? kb0 : kb1) >> (j & 3)) & 1u;
          ds[j] = p * (keep ? __builtin_fmaf(dp[r] + delta, pb.inv_keep, -delta) : -delta);
        } else {
          ds[j] = p * dp[r];
        }
      }
      sf[t] = pack_bf16x8(ds);
    }
    // dQ^T += K^T dS^T, K^T read transposed from the row-major K tile
#pragma unroll
    for (int e = 0; e < DE; ++e)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint16_t* kr = kb + (32 * a + 16 * t) * D;
        acc[e] = mfma32x32x16(ld_frag_tr2(kr + sw.tlo[e], kr + sw.thi[e]), sf[t], acc[e]);
      }
  }
}

template <int D, bool DROP>
__global__ __launch_bounds__(kThreads, D == 64 ? 3 : 2) void attn_bwd_dq(
    View Q, View K, View V, View O, View dO, const float* __restrict__ LSE, View dQ,
    float* __restrict__ Delta, Problem pb, int nqb, int hg) {
  constexpr int BM = kBM, BN = kBN;
  constexpr int LD = D + 8;
  constexpr int DS = D / 16;
  constexpr int DE = D / 32;
  // K and V tiles of the two buffers, copied in by the DMA (unpadded,
  // swizzled).  Separate arrays per buffer, and a loop unrolled by two, let
  // the compiler see that the copy into one buffer does not touch the one
  // being read, so reads do not wait for the copy.
  __shared__ __attribute__((aligned(16))) uint16_t K0[BN * D], K1[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t V0[BN * D], V1[BN * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int c = lane & 31, g = lane >> 5;
  SwzLane<D> sw;
  sw.init(c, g, tr_rowoff(lane), tr_coloff(lane));
  const int bid = blockIdx.x;
  const QItem qit = grouped_item(bid, pb.N, nqb, hg);
  const int qb = qit.qb;
  const int n = qit.n;
  const uint16_t* Kh = head_of(K, n, pb.H);
  const uint16_t* Vh = head_of(V, n, pb.H);
  const int q0 = qb * BM;
  const int q0w = q0 + 32 * w;
  const int qi = q0w + c;
  const long long row = (long long)n * pb.Tq + qi;

  const TileSpan ws = key_tiles(q0, q0 + BM - 1, pb, BN);
  const TileSpan wv = key_tiles(q0w, q0w + 31, pb, BN);
  const int wlast = min(q0w + 31, pb.Tq - 1);
  const Span seen = keys_of(qi, pb);  // keys this lane's query sees
  // keys some row of this wave sees (32-key halves outside are skipped)
  const int wklo = keys_lo(q0w, pb), wkhi = keys_hi(wlast, pb);

  TileDMA<BN, D, kThreads> ks, vs;
  ks.init(tid, K.st);
  vs.init(tid, V.st);
  auto load_tile = [&](int kt, int valid, uint16_t* kd, uint16_t* vd) {
    const int k1 = kt * BN;
    ks.load(Kh + (long long)k1 * K.st, valid, kd);
    vs.load(Vh + (long long)k1 * V.st, valid, vd);
  };
  // first tile (reads nothing when the workgroup sees no key), issued
  // before the row loads below so that the two latencies overlap
  load_tile(ws.t0, ws.t1 >= ws.t0 ? pb.Tk - ws.t0 * BN : 0, K0, V0);

  const float lse = qi < pb.Tq ? load_f32_or_zero(LSE + (row - c), pb.Tq - q0w, c) : -INFINITY;
  bf16x8 qf[DS], df[DS];  // this lane's query rows of Q and dO (zero past Tq)
  float dpart = 0.0f;
  {
    const int q0u = __builtin_amdgcn_readfirstlane(q0w);  // uniform row block start
    RowBlock qr, dr, orr;
    qr.init(head_of(Q, n, pb.H) + (long long)q0u * Q.st, pb.Tq - q0u, Q.st, c);
    dr.init(head_of(dO, n, pb.H) + (long long)q0u * dO.st, pb.Tq - q0u, dO.st, c);
    orr.init(head_of(O, n, pb.H) + (long long)q0u * O.st, pb.Tq - q0u, O.st, c);
    u32x4 ou[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      qf[s] = __builtin_bit_cast(bf16x8, qr.load(16 * s + 8 * g));
      df[s] = __builtin_bit_cast(bf16x8, dr.load(16 * s + 8 * g));
      ou[s] = orr.load(16 * s + 8 * g);
    }
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      const u32x4 du = __builtin_bit_cast(u32x4, df[s]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dpart += bf16_lo(du[j]) * bf16_lo(ou[s][j]) + bf16_hi(du[j]) * bf16_hi(ou[s][j]);
    }
  }
  const float delta = half_sum(dpart);
  const float nl = lse > -INFINITY ? -lse * kLog2e : -INFINITY;
  if (qi < pb.Tq && g == 0) {
    // workspace: -delta, then the seed -lse/scale of the head-size-64
    // dK/dV kernel's score accumulator (-inf for a query that sees nothing)
    Delta[row] = -delta;
    Delta[(long long)pb.N * pb.Tq + row] = lse > -INFINITY ? -lse / pb.scale : -INFINITY;
  }
  f32x16 nd;
#pragma unroll
  for (int r = 0; r < 16; ++r) nd[r] = -delta;

  wait_dma();
  __syncthreads();

  f32x16 acc[DE];
#pragma unroll
  for (int e = 0; e < DE; ++e) acc[e] = zero16();

  // one tile: compute on (kc, vc) while the next tile is copied into (kn, vn)
  auto step = [&](int kt, const uint16_t* kc, const uint16_t* vc, uint16_t* kn, uint16_t* vn) {
    const bool more = kt < ws.t1;
    if (more) load_tile(kt + 1, pb.Tk - (kt + 1) * BN, kn, vn);
    if (kt >= wv.t0 && kt <= wv.t1) {
      const int k0 = kt * BN;
      if (needs_mask(q0w, wlast, k0, k0 + BN - 1, pb)) {
        dq_tile<D, true, DROP>(kc, vc, qf, df, nd, acc, k0, seen, g, sw, nl, qi, n,
                               k0 + 31 < wklo ? 1 : 0, k0 + 32 > wkhi ? 0 : 1, pb);
      } else {
        dq_tile<D, false, DROP>(kc, vc, qf, df, nd, acc, k0, seen, g, sw, nl, qi, n, 0, 1, pb);
      }
    }
    if (more) wait_dma();  // this wave's copies have landed; the barrier publishes them
    __syncthreads();
  };
  for (int kt = ws.t0; kt <= ws.t1; kt += 2) {
    step(kt, K0, V0, K1, V1);
    if (kt + 1 <= ws.t1) step(kt + 1, K1, V1, K0, V0);
  }

  // the K tiles are free after the loop's last barrier: 16 rows per wave
  static_assert(2 * 16 * LD <= BN * D, "two waves' epilogue staging must fit one K tile");
  store_rows<D>((w < 2 ? K0 : K1) + (w & 1) * 16 * LD, acc, pb.scale,
                const_cast<uint16_t*>(head_of(dQ, n, pb.H)) + (long long)q0w * dQ.st, dQ.st,
                pb.Tq - q0w, lane);
}

// ---------------------------------------------------------------------------
// Backward, part 2: dK and dV (lane -> key layout), 16 keys per wave on the
// 16 x 16 x 32 product.  The K and V rows a wave keeps in registers take 32
// registers and the dK and dV accumulators 64 (with 32 keys per wave, 64 and
// 128: one wave per SIMD at D = 128, two at D = 64).  Two waves per SIMD at
// D = 128, three at D = 64, in workgroups of 64 keys.
// Lane (g, c) owns key c of the wave; S and dP come out with rows = queries
// 4g + r of each 16-query block, P and dS of two such blocks are packed into
// one operand, and dV^T / dK^T (rows = head dims 16m + 4g + r, columns =
// keys) accumulate with dO^T / Q^T read transposed from the swizzled tiles.
// ---------------------------------------------------------------------------

// One 64-query tile for one wave (16 keys), in two halves of 32 queries.
// With dropout, bit 4b + r of kq keeps (query q0 + 16b + 4g + r, this key).
template <int D, bool MASK, bool DROP>
__device__ __forceinline__ void dk16w_tile(const uint16_t* qb, const uint16_t* db, const float* ls,
                                           const float* es, const bf16x8* kf, const bf16x8* vf,
                                           f32x4* dvt, f32x4* dkt, int q0, Span seers, int g,
                                           const int* fo, const int* tlo, int hb0, int hb1,
                                           uint32_t kq, const Problem& pb) {
  constexpr int NS = D / 32, NM = D / 16;
  // (no scheduling hint here: without it this kernel is 2-3% faster)
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    // half kk = 16-query blocks 2kk and 2kk + 1; skipped when neither sees a key
    if (MASK && (2 * kk + 1 < hb0 || 2 * kk > hb1)) continue;
    // S = Q K^T and dP - delta = dO V^T - delta per block (-delta seeds dP;
    // with dropout dP starts at 0 and delta is added after the keep mask)
    f32x4 st[2], dp[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int b = 2 * kk + bb;
      if (MASK && (b < hb0 || b > hb1)) {
        st[bb] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[bb] = st[bb];
        continue;
      }
      const f32x4 nd =
          DROP ? f32x4{0.f, 0.f, 0.f, 0.f} : *reinterpret_cast<const f32x4*>(es + 16 * b + 4 * g);
      st[bb] = mfma16x16x32(ld_frag16(qb + 16 * b * D + fo[0]), kf[0], f32x4{0.f, 0.f, 0.f, 0.f});
      dp[bb] = mfma16x16x32(ld_frag16(db + 16 * b * D + fo[0]), vf[0], nd);
#pragma unroll
      for (int s = 1; s < NS; ++s) {
        st[bb] = mfma16x16x32(ld_frag16(qb + 16 * b * D + fo[s]), kf[s], st[bb]);
        dp[bb] = mfma16x16x32(ld_frag16(db + 16 * b * D + fo[s]), vf[s], dp[bb]);
      }
    }
    float p[8], dsv[8];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int b = 2 * kk + bb;
      const f32x4 nl = *reinterpret_cast<const f32x4*>(ls + 16 * b + 4 * g);
      f32x4 nd;
      if (DROP) nd = *reinterpret_cast<const f32x4*>(es + 16 * b + 4 * g);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(st[bb][r], pb.sl2, nl[r]));
        if (MASK && !inside(q0 + 16 * b + 4 * g + r, seers)) pv = 0.0f;
        if (DROP) {
          const bool keep = (kq >> (4 * b + r)) & 1u;
          p[4 * bb + r] = keep ? pv * pb.inv_keep : 0.0f;                        // for dV
          dsv[4 * bb + r] = pv * ((keep ? dp[bb][r] * pb.inv_keep : 0.0f) + nd[r]);  // nd = -delta
        } else {
          p[4 * bb + r] = pv;
          dsv[4 * bb + r] = pv * dp[bb][r];
        }
      }
    }
    // P and dS of the half's 32 queries as one operand each: dV^T += dO^T P
    // and dK^T += Q^T dS over head-dim blocks m, the transposed reads taking
    // rows 4g + c / 4 of both blocks (the same query order as the operand)
    const bf16x8 pf = pack_bf16x8(p), sf = pack_bf16x8(dsv);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int lo = 32 * kk * D + tlo[m], hi = lo + 16 * D;
      dvt[m] = mfma16x16x32(ld_frag_tr2(db + lo, db + hi), pf, dvt[m]);
      dkt[m] = mfma16x16x32(ld_frag_tr2(qb + lo, qb + hi), sf, dkt[m]);
    }
  }
}

// Workgroup = 64 keys of one head (4 waves x 16); walks the 64-query tiles
// that see its keys, from the diagonal to the end, with double-buffered
// Q / dO copies and the tiles' lse and delta staged beside them.
template <int D, bool DROP>
__global__ __launch_bounds__(kThreads, D == 64 ? 3 : 2) void attn_bwd_dkdv16w(
    View Q, View K, View V, View dO, const float* __restrict__ LSE,
    const float* __restrict__ Delta, View dK, View dV, Problem pb) {
  constexpr int BM = 64, BN = kKBN16, NS = D / 32, NM = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t QD0[2][BM * D];
  __shared__ __attribute__((aligned(16))) uint16_t QD1[2][BM * D];
  __shared__ __attribute__((aligned(16))) float Ls[2][BM];
  __shared__ __attribute__((aligned(16))) float Es[2][BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int bid = blockIdx.x;
  const int kb = bid / pb.N;
  const int n = bid % pb.N;
  const uint16_t* Qh = head_of(Q, n, pb.H);
  const uint16_t* Dh = head_of(dO, n, pb.H);
  const long long rows = (long long)n * pb.Tq;
  const int k0 = kb * BN;
  const int k0w = k0 + 16 * w;
  const int kj = k0w + c;

  int fo[NS], tlo[NM];
#pragma unroll
  for (int s = 0; s < NS; ++s) fo[s] = swz<D, true>(c, 32 * s + 8 * g);
#pragma unroll
  for (int m = 0; m < NM; ++m) tlo[m] = swz<D, true>(4 * g + (c >> 2), 16 * m + 4 * (c & 3));

  bf16x8 kf[NS], vf[NS];
  {
    RowBlock kr, vr;
    kr.init(head_of(K, n, pb.H) + (long long)k0w * K.st, pb.Tk - k0w, K.st, c);
    vr.init(head_of(V, n, pb.H) + (long long)k0w * V.st, pb.Tk - k0w, V.st, c);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      kf[s] = __builtin_bit_cast(bf16x8, kr.load(32 * s + 8 * g));
      vf[s] = __builtin_bit_cast(bf16x8, vr.load(32 * s + 8 * g));
    }
  }

  const int qlo = queries_lo(k0, pb), qhi = queries_hi(min(k0 + BN, pb.Tk) - 1, pb);
  const int qt0 = qlo / BM, qt1 = qhi >= qlo ? qhi / BM : qt0 - 1;
  const int wqlo = queries_lo(k0w, pb);
  const int wqhi = k0w < pb.Tk ? queries_hi(min(k0w + 15, pb.Tk - 1), pb) : -1;
  const Span seers = queries_of(kj, pb);

  TileDMA<BM, D, kThreads, true> qs, ds;
  qs.init(tid, Q.st);
  ds.init(tid, dO.st);
  float lraw = 0.0f, draw = 0.0f;
  int qrow = 0;
  auto load_tile = [&](int qt, int valid, uint16_t (&qd)[2][BM * D]) {
    const int q1 = qt * BM;
    qs.load(Qh + (long long)q1 * Q.st, valid, qd[0]);
    ds.load(Dh + (long long)q1 * dO.st, valid, qd[1]);
    qrow = q1 + tid;
    const int cnt = valid < BM ? valid : BM;
    lraw = load_f32_or_zero(LSE + rows + q1, cnt, tid);
    draw = load_f32_or_zero(Delta + rows + q1, cnt, tid);
  };
  auto publish_tile = [&](int b) {
    if (tid < BM) {
      const bool live = qrow < pb.Tq && lraw > -INFINITY;
      Ls[b][tid] = live ? -lraw * kLog2e : -INFINITY;
      Es[b][tid] = draw;  // the workspace holds -delta
    }
    wait_dma();
  };
  load_tile(qt0, qt1 >= qt0 ? pb.Tq - qt0 * BM : 0, QD0);
  publish_tile(0);
  __syncthreads();

  f32x4 dvt[NM], dkt[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    dvt[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    dkt[m] = dvt[m];
  }

  auto step = [&](int qt, uint16_t (&cur)[2][BM * D], uint16_t (&nxt)[2][BM * D], int b) {
    const bool more = qt < qt1;
    if (more) load_tile(qt + 1, pb.Tq - (qt + 1) * BM, nxt);
    const int q0 = qt * BM;
    if (q0 + BM - 1 >= wqlo && q0 <= wqhi) {
      // Dropout keep bits of the tile: lane x of each quad of keys draws the
      // 16-query block x for the quad's four keys (two calls, one per query
      // pair); each lane then takes its own key's bits from lane b.
      uint32_t kq = 0;
      if (DROP) {
        const uint32_t x = (uint32_t)(c & 3);
        const uint32_t ip = (uint32_t)(q0 + 16 * (int)x + 4 * g) >> 1;
        const uint32_t drawn = keep8((uint32_t)kj >> 2, ip, (uint32_t)n, pb) |
                               keep8((uint32_t)kj >> 2, ip + 1, (uint32_t)n, pb) << 8;
        const uint32_t from[4] = {quad_lane<0>(drawn), quad_lane<1>(drawn),
                                  quad_lane<2>(drawn), quad_lane<3>(drawn)};
#pragma unroll
        for (int bk = 0; bk < 4; ++bk) {
          const uint32_t sft = from[bk] >> (2 * x);  // queries 0, 1 at bits 0, 1; 2, 3 at 8, 9
          kq |= ((sft & 3u) | ((sft >> 6) & 12u)) << (4 * bk);
        }
      }
      if (needs_mask(q0, q0 + BM - 1, k0w, k0w + 15, pb)) {
        const int hb0 = max(0, (wqlo - q0) >> 4), hb1 = min(BM / 16 - 1, (wqhi - q0) >> 4);
        dk16w_tile<D, true, DROP>(cur[0], cur[1], Ls[b], Es[b], kf, vf, dvt, dkt, q0, seers, g,
                                  fo, tlo, hb0, hb1, kq, pb);
      } else {
        dk16w_tile<D, false, DROP>(cur[0], cur[1], Ls[b], Es[b], kf, vf, dvt, dkt, q0, seers, g,
                                   fo, tlo, 0, BM / 16 - 1, kq, pb);
      }
    }
    if (more) publish_tile(b ^ 1);
    __syncthreads();
  };
  for (int qt = qt0; qt <= qt1; qt += 2) {
    step(qt, QD0, QD1, 0);
    if (qt + 1 <= qt1) step(qt + 1, QD1, QD0, 1);
  }

  // epilogue: lane (g, c) holds key c's dims 16m + 4g + r; 16 rows per wave
  // staged in LDS (row stride D + 8), then whole rows stored
  constexpr int LD = D + 8;
  static_assert(4 * 16 * LD <= 2 * BM * D, "epilogue staging must fit one buffer");
  uint16_t* stage = &QD0[0][0] + w * 16 * LD;
  auto store = [&](const f32x4* acc, float mul, View out) {
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const u32x2 pk = {pack_bf16x2(acc[m][0] * mul, acc[m][1] * mul),
                        pack_bf16x2(acc[m][2] * mul, acc[m][3] * mul)};
      *reinterpret_cast<u32x2*>(stage + c * LD + 16 * m + 4 * g) = pk;
    }
    __syncthreads();
    uint16_t* orow = const_cast<uint16_t*>(head_of(out, n, pb.H)) + (long long)k0w * out.st;
    constexpr int CPR = D / 8;  // 16-byte chunks per row
#pragma unroll
    for (int p = 0; p < 16 * CPR / 64; ++p) {
      const int ch = lane + 64 * p, r = ch / CPR, cc = ch % CPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * LD + 8 * cc);
      if (r < pb.Tk - k0w) *reinterpret_cast<u32x4*>(orow + (long long)r * out.st + 8 * cc) = v;
    }
    __syncthreads();
  };
  store(dkt, pb.scale, dK);
  store(dvt, 1.0f, dV);
}

// ---------------------------------------------------------------------------
// dQ at D = 64 with 16 queries per wave on the 16 x 16 x 32 product: 124
// registers (with or without dropout), four waves per SIMD, workgroups of 64
// queries.  Lane (g, c) owns query c of the wave; S^T and dP^T come out with
// rows = keys 4g + r of each 16-key block; dS^T of two blocks is packed into
// one operand and dQ^T (rows = head dims 16m + 4g + r, columns = queries)
// accumulates with K^T read transposed from the swizzled K tile.  (At
// D = 128 every wave reading the whole K and V tile for 16 queries costs
// more than the occupancy gains; the 32-query kernel serves it.)
// ---------------------------------------------------------------------------
constexpr int kBM16 = 64;  // queries per workgroup (4 waves x 16)

// One 64-key tile for one wave (16 queries), in two halves of 32 keys.  With
// dropout, bit 4b + r of kq keeps (this query, key k0 + 16b + 4g + r).
template <int D, bool MASK, bool DROP>
__device__ __forceinline__ void dq16_tile(const uint16_t* kb, const uint16_t* vb, const bf16x8* qf,
                                          const bf16x8* df, float nd, float nl, f32x4* acc,
                                          int k0, Span seen, int g, const int* fo,
                                          const int* tlo, int hb0, int hb1, uint32_t kq,
                                          const Problem& pb) {
  constexpr int NS = D / 32, NM = D / 16;
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
      st[bb] = mfma16x16x32(ld_frag16(kb + 16 * b * D + fo[0]), qf[0], f32x4{0.f, 0.f, 0.f, 0.f});
      dp[bb] = mfma16x16x32(ld_frag16(vb + 16 * b * D + fo[0]), df[0], f32x4{nd, nd, nd, nd});
#pragma unroll
      for (int s = 1; s < NS; ++s) {
        st[bb] = mfma16x16x32(ld_frag16(kb + 16 * b * D + fo[s]), qf[s], st[bb]);
        dp[bb] = mfma16x16x32(ld_frag16(vb + 16 * b * D + fo[s]), df[s], dp[bb]);
      }
    }
    float ds[8];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int b = 2 * kk + bb;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[bb][r], pb.sl2, nl));
        if (MASK && !inside(k0 + 16 * b + 4 * g + r, seen)) p = 0.0f;
        if (DROP) {
          const float delta = -nd;
          const bool keep = (kq >> (4 * b + r)) & 1u;
          ds[4 * bb + r] =
              p * (keep ? __builtin_fmaf(dp[bb][r] + delta, pb.inv_keep, -delta) : -delta);
        } else {
          ds[4 * bb + r] = p * dp[bb][r];
        }
      }
    }
    const bf16x8 sf = pack_bf16x8(ds);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int lo = 32 * kk * D + tlo[m], hi = lo + 16 * D;
      acc[m] = mfma16x16x32(ld_frag_tr2(kb + lo, kb + hi), sf, acc[m]);
    }
  }
}

// Workgroup = 64 queries of one head (4 waves x 16): the row term delta,
// then the key tiles its rows see, as attn_bwd_dq.
template <int D, bool DROP>
__global__ __launch_bounds__(kThreads, 4) void attn_bwd_dq16(
    View Q, View K, View V, View O, View dO, const float* __restrict__ LSE, View dQ,
    float* __restrict__ Delta, Problem pb, int nqb, int hg) {
  constexpr int BM = kBM16, BN = kBN, NS = D / 32, NM = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t K0[BN * D], K1[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t V0[BN * D], V1[BN * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int bid = blockIdx.x;
  const QItem qit = grouped_item(bid, pb.N, nqb, hg);
  const int qb = qit.qb;
  const int n = qit.n;
  const uint16_t* Kh = head_of(K, n, pb.H);
  const uint16_t* Vh = head_of(V, n, pb.H);
  const int q0 = qb * BM;
  const int q0w = q0 + 16 * w;
  const int qi = q0w + c;
  const long long row = (long long)n * pb.Tq + qi;

  int fo[NS], tlo[NM];
#pragma unroll
  for (int s = 0; s < NS; ++s) fo[s] = swz<D, true>(c, 32 * s + 8 * g);
#pragma unroll
  for (int m = 0; m < NM; ++m) tlo[m] = swz<D, true>(4 * g + (c >> 2), 16 * m + 4 * (c & 3));

  const TileSpan ws = key_tiles(q0, q0 + BM - 1, pb, BN);
  const TileSpan wv = key_tiles(q0w, q0w + 15, pb, BN);
  const int wlast = min(q0w + 15, pb.Tq - 1);
  const Span seen = keys_of(qi, pb);
  const int wklo = keys_lo(q0w, pb), wkhi = keys_hi(wlast, pb);

  TileDMA<BN, D, kThreads, true> ks, vs;
  ks.init(tid, K.st);
  vs.init(tid, V.st);
  auto load_tile = [&](int kt, int valid, uint16_t* kd, uint16_t* vd) {
    const int k1 = kt * BN;
    ks.load(Kh + (long long)k1 * K.st, valid, kd);
    vs.load(Vh + (long long)k1 * V.st, valid, vd);
  };
  load_tile(ws.t0, ws.t1 >= ws.t0 ? pb.Tk - ws.t0 * BN : 0, K0, V0);

  const float lse = qi < pb.Tq ? load_f32_or_zero(LSE + (row - c), pb.Tq - q0w, c) : -INFINITY;
  bf16x8 qf[NS], df[NS];
  float dpart = 0.0f;
  {
    RowBlock qr, dr, orr;
    qr.init(head_of(Q, n, pb.H) + (long long)q0w * Q.st, pb.Tq - q0w, Q.st, c);
    dr.init(head_of(dO, n, pb.H) + (long long)q0w * dO.st, pb.Tq - q0w, dO.st, c);
    orr.init(head_of(O, n, pb.H) + (long long)q0w * O.st, pb.Tq - q0w, O.st, c);
    u32x4 ou[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      qf[s] = __builtin_bit_cast(bf16x8, qr.load(32 * s + 8 * g));
      df[s] = __builtin_bit_cast(bf16x8, dr.load(32 * s + 8 * g));
      ou[s] = orr.load(32 * s + 8 * g);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const u32x4 du = __builtin_bit_cast(u32x4, df[s]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dpart += bf16_lo(du[j]) * bf16_lo(ou[s][j]) + bf16_hi(du[j]) * bf16_hi(ou[s][j]);
    }
  }
  // the row's four 16-lane groups hold its four quarters of the head dims
  dpart += __shfl_xor(dpart, 16);
  const float delta = dpart + __shfl_xor(dpart, 32);
  const float nl = lse > -INFINITY ? -lse * kLog2e : -INFINITY;
  if (qi < pb.Tq && g == 0) {
    // workspace: -delta, then the seed -lse/scale of the head-size-64
    // dK/dV kernel's score accumulator (-inf for a query that sees nothing)
    Delta[row] = -delta;
    Delta[(long long)pb.N * pb.Tq + row] = lse > -INFINITY ? -lse / pb.scale : -INFINITY;
  }

  wait_dma();
  __syncthreads();

  f32x4 acc[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto step = [&](int kt, const uint16_t* kc, const uint16_t* vc, uint16_t* kn, uint16_t* vn) {
    const bool more = kt < ws.t1;
    if (more) load_tile(kt + 1, pb.Tk - (kt + 1) * BN, kn, vn);
    if (kt >= wv.t0 && kt <= wv.t1) {
      const int k0 = kt * BN;
      uint32_t kq = 0;
      if (DROP) {
        // lanes 2y and 2y + 1 hold queries 2y' and 2y' + 1: the even lane
        // draws key blocks 0 and 2, the odd lane 1 and 3, each for both
        // queries, and the two exchange the other half
        const uint32_t odd = (uint32_t)qi & 1u, ip = (uint32_t)qi >> 1;
        const uint32_t jb = (uint32_t)k0 / 4 + (uint32_t)g;
        const uint32_t ma = keep8(jb + 4 * odd, ip, (uint32_t)n, pb);
        const uint32_t mb = keep8(jb + 8 + 4 * odd, ip, (uint32_t)n, pb);
        // the neighbour's draws (lane ^ 1, DPP quad permute 1, 0, 3, 2)
        const uint32_t oa = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)ma, 0xB1, 0xF, 0xF,
                                                                  false);
        const uint32_t ob = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mb, 0xB1, 0xF, 0xF,
                                                                  false);
        const uint32_t b0 = odd ? oa : ma, b1 = odd ? ma : oa;
        const uint32_t b2 = odd ? ob : mb, b3 = odd ? mb : ob;
        kq = keep_of_query(b0, odd) | keep_of_query(b1, odd) << 4 | keep_of_query(b2, odd) << 8 |
             keep_of_query(b3, odd) << 12;
      }
      if (needs_mask(q0w, wlast, k0, k0 + BN - 1, pb)) {
        const int hb0 = max(0, (wklo - k0) >> 4), hb1 = min(BN / 16 - 1, (wkhi - k0) >> 4);
        dq16_tile<D, true, DROP>(kc, vc, qf, df, -delta, nl, acc, k0, seen, g, fo, tlo, hb0, hb1,
                                 kq, pb);
      } else {
        dq16_tile<D, false, DROP>(kc, vc, qf, df, -delta, nl, acc, k0, seen, g, fo, tlo, 0,
                                  BN / 16 - 1, kq, pb);
      }
    }
    if (more) wait_dma();
    __syncthreads();
  };
  for (int kt = ws.t0; kt <= ws.t1; kt += 2) {
    step(kt, K0, V0, K1, V1);
    if (kt + 1 <= ws.t1) step(kt + 1, K1, V1, K0, V0);
  }

  // epilogue: lane (g, c) holds query c's dims 16m + 4g + r; 16 rows per
  // wave staged in the K tiles (row stride D + 8), then whole rows stored
  constexpr int LD = D + 8, CPR = D / 8;
  static_assert(2 * 16 * LD <= BN * D, "two waves' epilogue staging must fit one K tile");
  uint16_t* stage = (w < 2 ? K0 : K1) + (w & 1) * 16 * LD;
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const u32x2 pk = {pack_bf16x2(acc[m][0] * pb.scale, acc[m][1] * pb.scale),
                      pack_bf16x2(acc[m][2] * pb.scale, acc[m][3] * pb.scale)};
    *reinterpret_cast<u32x2*>(stage + c * LD + 16 * m + 4 * g) = pk;
  }
  __syncthreads();
  uint16_t* orow = const_cast<uint16_t*>(head_of(dQ, n, pb.H)) + (long long)q0w * dQ.st;
#pragma unroll
  for (int p = 0; p < 16 * CPR / 64; ++p) {
    const int ch = lane + 64 * p, r = ch / CPR, cc = ch % CPR;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * LD + 8 * cc);
    if (r < pb.Tq - q0w) *reinterpret_cast<u32x4*>(orow + (long long)r * dQ.st + 8 * cc) = v;
  }
}

template <typename... Args>
hipError_t launch(void (*kern)(Args...), long long blocks, hipStream_t stream, Args... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), dim3((unsigned)blocks),
                         dim3(kThreads), argv, 0, stream);
}

View view(const TensorArg& t) {
  return View{static_cast<const uint16_t*>(t.data), t.sb, t.sh, t.st};
}

// Heads per group for grouped_item: problems of at least eight rounds of the
// GPU's workgroup slots (per_cu resident workgroups on each CU) take their
// heads in balanced groups of about four rounds each, in multiples of 8
// heads; smaller ones, and head counts that are not multiples of 8, run the
// plain longest-first list (one group of all N heads).
int head_group(int N, int nq, int cus, int per_cu) {
  const long long slots = (long long)cus * per_cu;
  if (slots <= 0 || N % 8 != 0 || (long long)N * nq < 8 * slots) return N;
  const long long groups = ((long long)N * nq + 4 * slots - 1) / (4 * slots);
  const long long h = ((N + groups - 1) / groups + 7) / 8 * 8;
  return (int)(h < N ? h : N);
}

}  // namespace

Problem make_problem(const ProblemArg& p) {
  Problem pb{p.B * p.H, p.H, p.Tq, p.Tk, p.off, p.win, p.scale * kLog2e, p.scale,
             (uint32_t)p.seed, (uint32_t)(p.seed >> 32), p.stream, 0u, 1.0f};
  if (p.dropout > 0.0f) {
    const double t = ceil((double)p.dropout * 65536.0);
    pb.thr = t >= 65536.0 ? 65536u : (uint32_t)t;
    // kept weights are scaled by the inverse of the realised keep
    // probability (2^16 - thr) / 2^16, so the dropped-out weights stay
    // unbiased (all dropped when thr = 2^16: the scale is never used)
    pb.inv_keep = pb.thr >= 65536u ? 0.0f : (float)(65536.0 / (65536.0 - (double)pb.thr));
  }
  return pb;
}

hipError_t launch_fwd_bf16(const TensorArg& q, const TensorArg& k, const TensorArg& v,
                           const TensorArg& o, float* lse, const ProblemArg& p,
                           hipStream_t stream) {
  if (decode_applies(p)) return launch_decode_bf16(q, k, v, o, lse, p, stream);
  const Problem pb = make_problem(p);
  const int nqb = (p.Tq + kBM - 1) / kBM;
  const long long blocks = (long long)pb.N * nqb;
  const bool drop = p.dropout > 0.0f;
  // at D = 64 (four workgroups per CU) the longest-first list is dealt over
  // the CUs (dealt_item); at D = 128 it runs in list order
  const int cus = cu_count(stream);
  const int deal = p.D == 64 && cus > 0 && cus % 8 == 0 ? cus : 0;
  const int dealg = pb.N % 8 == 0 ? 8 : 1;
  // heads in groups on large problems at D = 128 (at D = 64 the dealt order
  // alone measured as fast: 1152 heads of 1024 tokens 251 against 258 us)
  const int hg = p.D == 128 ? head_group(pb.N, nqb, cus, 2) : pb.N;
#define GPTATTN_FWD(D_, DROP_)                                                                  \
  launch(attn_fwd<D_, DROP_>, blocks, stream, view(q), view(k), view(v), view(o), lse, pb, nqb, \
         deal, dealg, hg)
  switch (p.D) {
    case 64: return drop ? GPTATTN_FWD(64, true) : GPTATTN_FWD(64, false);
    case 128: return drop ? GPTATTN_FWD(128, true) : GPTATTN_FWD(128, false);
    default: return hipErrorInvalidValue;
  }
#undef GPTATTN_FWD
}

hipError_t launch_bwd_dq_bf16(const TensorArg& q, const TensorArg& k, const TensorArg& v,
                              const TensorArg& o, const TensorArg& dO, const float* lse,
                              const TensorArg& dq, float* delta, const ProblemArg& p,
                              hipStream_t stream) {
  const Problem pb = make_problem(p);
  const int nqb = (p.Tq + kBM - 1) / kBM;
  const long long blocks = (long long)pb.N * nqb;
  const bool drop = p.dropout > 0.0f;
  // heads in groups on large problems (head_group)
  const int cus = cu_count(stream);
  const int hg = head_group(pb.N, nqb, cus, 2);
#define GPTATTN_DQ(D_, DROP_)                                                                   \
  launch(attn_bwd_dq<D_, DROP_>, blocks, stream, view(q), view(k), view(v), view(o), view(dO),  \
         lse, view(dq), delta, pb, nqb, hg)
  const int nqb16 = (p.Tq + kBM16 - 1) / kBM16;
  const long long blocks16 = (long long)pb.N * nqb16;
  const int hg16 = head_group(pb.N, nqb16, cus, 4);
#define GPTATTN_DQ16(D_, DROP_)                                                                 \
  launch(attn_bwd_dq16<D_, DROP_>, blocks16, stream, view(q), view(k), view(v), view(o),        \
         view(dO), lse, view(dq), delta, pb, nqb16, hg16)
  switch (p.D) {
    case 64: return drop ? GPTATTN_DQ16(64, true) : GPTATTN_DQ16(64, false);
    case 128: return drop ? GPTATTN_DQ(128, true) : GPTATTN_DQ(128, false);
    default: return hipErrorInvalidValue;
  }
#undef GPTATTN_DQ16
#undef GPTATTN_DQ
}

hipError_t launch_bwd_dkdv_bf16(const TensorArg& q, const TensorArg& k, const TensorArg& v,
                                const TensorArg& dO, const float* lse, const float* delta,
                                const TensorArg& dk, const TensorArg& dv, const ProblemArg& p,
                                hipStream_t stream) {
  const bool drop = p.dropout > 0.0f;
  // head size 64 without dropout: the 128-key kernel, except on short key
  // sequences (at most four 64-key blocks), where its coarser workgroups
  // leave the GPU emptier than the 64-key kernel below (character-model
  // shape, 256 keys: 23.5 against 20.0 us)
  if (p.D == 64 && !drop && p.Tk > 256)
    return launch_bwd_dkdv_d64(q, k, v, dO, lse, delta, dk, dv, p, stream);
  // head size 128 without dropout, dense tensors, more 128-key items than
  // compute units: the persistent 128-key kernel
  if (dkdv_d128_applies(q, k, v, dO, dk, dv, p, stream))
    return launch_bwd_dkdv_d128(q, k, v, dO, delta, dk, dv, p, stream);
  const Problem pb = make_problem(p);
  const long long blocks = (long long)pb.N * ((p.Tk + kKBN16 - 1) / kKBN16);
#define GPTATTN_DKDV16(D_, DROP_)                                                               \
  launch(attn_bwd_dkdv16w<D_, DROP_>, blocks, stream, view(q), view(k), view(v), view(dO),     \
         lse, delta, view(dk), view(dv), pb)
  switch (p.D) {
    case 64: return drop ? GPTATTN_DKDV16(64, true) : GPTATTN_DKDV16(64, false);
    case 128: return drop ? GPTATTN_DKDV16(128, true) : GPTATTN_DKDV16(128, false);
    default: return hipErrorInvalidValue;
  }
#undef GPTATTN_DKDV16
}

}  // namespace gptattn
