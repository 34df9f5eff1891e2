// SeKV mixed-resolution decode attention for gfx950.
//
// One decode step of one layer scores the query of every head against the
// span summaries (routing score q.kbar/(|kbar| sqrt(d)) + ln|S|, eq. (5) of the
// long-form summary page with the identity projection; with a routing
// projection W, (W q).Kbar/sqrt(d') + ln|S| on the routing summaries of
// eq. (3), the projected queries coming from a small kernel), zooms the spans whose
// score exceeds logit(tau) (eq. (9)), and runs ONE softmax over three kinds of
// entries (review page, workflow paragraph; summary page Figure 2):
//   anchors          q.k_a / sqrt(d), value v_a
//   non-zoomed span  q.kbar / sqrt(d) + ln|S|, value vbar
//   zoomed span      its tokens rebuilt from the truncated SVD (eq. (6)),
//                    K^ = A_K B_K^T, V^ = A_V B_V^T, scored in rank space:
//                    p = B_K^T q, logit_t = A_K[t].p / sqrt(d),
//                    w = sum_t e_t A_V[t], contribution w . B_V^T.
//
// A layer-step is split over the context into segments (runs of span rows or
// of anchor rows of one (sequence, kv head)), each writing one partial
// (running max in log2 units, sum, d-vector accumulator) per query head into a
// slot of its own:
//   k_planned  (device-resident bases, and host-resident bases read in place)
//              one wave of workgroups, each running a short list of segments
//              planned on the host from the expected cost of every row (the
//              zoom frequency of each span over recent calls).  Its span
//              segments first: routing scores, zoom decisions and the summary
//              entries of the spans a head does not zoom; then its anchor
//              segments (exact tokens); then the zoomed spans of its span rows,
//              cut into units of one token tile each (independent entries of
//              the softmax) spread over the waves.  Rows stream in
//              double-buffered rounds.
//   k_route    (pinned bases copied to staging; and the routing-scores pass)
//              one workgroup per span task: routing scores, decisions, summary
//              entries, and the zoomed spans listed for the host fetch.
//   k_attend   (staged bases) one workgroup per fetched span task, its zoomed
//              spans from the staged bases into the task's second slot, then
//              one workgroup per anchor task.
//   k_combine  log-sum-exp merge of every (sequence, query head)'s slots, in
//              slot order.
// No workgroup waits for another and no atomic shares an address across the
// grid: kernel boundaries order the phases.
// Lanes are grouped in "row slots" of d*elem/16 lanes, each slot streaming
// whole 16-byte row pieces.  The path is HBM-bound (about one flop per byte per
// query head), so no MFMA is used.
#include "sekv_device.h"

namespace sekv {

namespace {

typedef unsigned long long u64;

template <int G>
struct SoftState {
  float m[G];  // running max, log2 units
  float l[G];  // running sum of exp2(logit - m)
};

// Merge (mo, lo, acco) into (m, l, acc) for one head; acc has N elements.
template <int N>
__device__ __forceinline__ void lse_merge(float& m, float& l, float* acc, float mo, float lo,
                                          const float* acco) {
  const float mn = fmaxf(m, mo);
  const float ms = (mn == kNegInf) ? 0.f : mn;
  const float a = fast_exp2(m - ms), b = fast_exp2(mo - ms);
  l = l * a + lo * b;
#pragma unroll
  for (int e = 0; e < N; ++e) acc[e] = acc[e] * a + acco[e] * b;
  m = mn;
}

// A raw 16-byte piece of T as loaded (converted to float at use).
template <typename T>
struct Raw;
template <>
struct Raw<bf16_t> {
  uint4 v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void zero() { v = make_uint4(0u, 0u, 0u, 0u); }
  __device__ __forceinline__ float get(int e) const {
    const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
};
template <>
struct Raw<float> {
  float4 v;
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ void zero() { v = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ float get(int e) const { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }
};

// Marks the raw words as changed (an empty asm statement, no instruction):
// the unpacking of a loaded piece then stays next to its use instead of being
// hoisted out of a loop over the query heads, where it would need G times the
// registers.
__device__ __forceinline__ void keep_packed(Raw<bf16_t>& r) {
  asm volatile("" : "+v"(r.v.x), "+v"(r.v.y), "+v"(r.v.z), "+v"(r.v.w));
}
__device__ __forceinline__ void keep_packed(Raw<float>& r) {
  asm volatile("" : "+v"(r.v.x), "+v"(r.v.y), "+v"(r.v.z), "+v"(r.v.w));
}

// Lane geometry for head dimension D and element type T.
template <int D, typename T>
struct Geo {
  static constexpr int EPL = Elem<T>::kPer16;  // elements per 16-byte piece
  static constexpr int LPR = D / EPL;          // lanes per D-row: one row slot
  static constexpr int RPW = 64 / LPR;         // row slots per wave
  // zoomed spans: lane = rank group (its row slot) x token group (its lane in the slot)
  static constexpr int TILE = LPR * EPL;       // tokens per tile (= D)
  static constexpr int RB = ((int)sizeof(T) == 2 ? 32 : 16) / RPW;  // rank rows per lane per batch
  static constexpr int RBATCH = RB * RPW;
};

// Sum over the row slots of a wave (lanes with the same position in their slot).
template <int LPR>
__device__ __forceinline__ float slots_sum(float x) {
  if constexpr (LPR <= 8) x += __shfl_xor(x, 8, 64);
  if constexpr (LPR <= 16) x = xor16_sum(x);
  if constexpr (LPR <= 32) x = xor32_sum(x);
  return x;
}

// x of the lane `off` apart (off = 8, 16 or 32).
__device__ __forceinline__ float lane_xor(float x, int off) {
  if (off == 16) return xor16_get(x);
  if (off == 32) return xor32_get(x);
  return __shfl_xor(x, off, 64);
}

// One-head groups: a wave takes two units of rank <= RBATCH / 2 in one round.
constexpr bool kPairUnits = true;

// Item flag: the span's bases are read from the device cache (bits 0..7 are head bits).
constexpr uint32_t kCachedBit = 0x100u;

template <int D, int G>
struct MergeLds {
  float m[kWaves][G];
  float l[kWaves][G];
  float acc[kWaves][G][D];
};

// Fold one softmax piece of head h (max sm in log2 units, sum sl, output
// slice o of columns tg*EPL ..) into the wave's running record in LDS.  Every
// row slot holds the same values; row slot 0 writes the slice.
template <int D, int G, int EPL>
__device__ __forceinline__ void fold_record(MergeLds<D, G>& ml, int wave, int h, int lane, int rg, int tg, float sm,
                                            float sl, const float (&o)[EPL]) {
  float mr = ml.m[wave][h], lr = ml.l[wave][h];
  float ar[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) ar[e] = ml.acc[wave][h][tg * EPL + e];
  lse_merge<EPL>(mr, lr, ar, sm, sl, o);
  wave_lds_sync();  // every lane has read the record before it is rewritten
  if (lane == 0) {
    ml.m[wave][h] = mr;
    ml.l[wave][h] = lr;
  }
  if (rg == 0) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) ml.acc[wave][h][tg * EPL + e] = ar[e];
  }
  wave_lds_sync();
}

// ------------------------------------------------------------------ zoomed span tile, one wave

// The rank rows of one unit that a lane holds: rows j = rg + RPW*u, u < NU, of
// B_K^T and B_V^T (the 16-byte piece at column tg*EPL) and of A_K^T and A_V^T
// (the piece of EPL tokens at tokc).  Rows past the rank hold zeros.
template <typename T, int NU>
struct UnitRows {
  Raw<T> bk[NU], ak[NU], av[NU], bv[NU];
};

// Load a unit's rows: the rows that r needs (rows 0..1, 2..3 and 4..7 sit
// behind wave-uniform branches; r is the same for the whole wave).
template <int D, typename T, int NU>
__device__ __forceinline__ void unit_rows_load(UnitRows<T, NU>& x, const T* __restrict__ base, int c8, int r,
                                               int tokc, int rg, int tg) {
  using Gm = Geo<D, T>;
  constexpr int EPL = Gm::EPL, RPW = Gm::RPW;
  const T* AKt = base;
  const T* BKt = AKt + (size_t)r * c8;
  const T* AVt = BKt + (size_t)r * D;
  const T* BVt = AVt + (size_t)r * c8;
  const int rl = r - 1;
  const int nu = (r + RPW - 1) / RPW;
  auto rows = [&](int lo, int hi) {
    if (nu > lo) {
#pragma unroll
      for (int u = lo; u < hi; ++u) {
        const int j = min(rg + RPW * u, rl);
        x.bk[u].load(BKt + (size_t)j * D + tg * EPL);
        x.ak[u].load(AKt + (size_t)j * c8 + tokc);
        x.av[u].load(AVt + (size_t)j * c8 + tokc);
        x.bv[u].load(BVt + (size_t)j * D + tg * EPL);
      }
    } else {
#pragma unroll
      for (int u = lo; u < hi; ++u) {
        x.bk[u].zero();
        x.ak[u].zero();
        x.av[u].zero();
        x.bv[u].zero();
      }
    }
  };
  rows(0, NU >= 2 ? 2 : 1);
  if constexpr (NU >= 4) rows(2, 4);
  if constexpr (NU >= 8) rows(4, 8);
}

// One head's piece of a loaded unit (c tokens, the tile's tokens from tok):
// p = B_K^T q, logits A_K p, softmax, w = A_V^T e, o = B_V w; goes to
// sink(0, max, sum, slice).
template <int D, typename T, int NU, class QGet, class Sink>
__device__ __forceinline__ void unit_rows_attend(const UnitRows<T, NU>& x, int c, int r, int tok, QGet qget,
                                                 Sink sink, float c2, int rg) {
  using Gm = Geo<D, T>;
  constexpr int EPL = Gm::EPL, LPR = Gm::LPR, RPW = Gm::RPW;
  float q[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) q[e] = qget(0, e);
  float p[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    float dp = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) dp += q[e] * x.bk[u].get(e);
    dp = group_sum<LPR>(dp);
    p[u] = (rg + RPW * u < r) ? dp * c2 : 0.f;
  }
  float lg[EPL];
  float mx = kNegInf;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    float y = 0.f;
#pragma unroll
    for (int u = 0; u < NU; ++u) y += p[u] * x.ak[u].get(e);
    y = slots_sum<LPR>(y);
    y = (tok + e < c) ? y : kNegInf;
    lg[e] = y;
    mx = fmaxf(mx, y);
  }
  mx = group_max<LPR>(mx);  // finite: the tile's first token is valid
  float sl = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    lg[e] = fast_exp2(lg[e] - mx);
    sl += lg[e];
  }
  sl = group_sum<LPR>(sl);
  float w[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    float y = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) y += lg[e] * x.av[u].get(e);
    y = group_sum<LPR>(y);
    w[u] = (rg + RPW * u < r) ? y : 0.f;
  }
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    float y = 0.f;
#pragma unroll
    for (int u = 0; u < NU; ++u) y += w[u] * x.bv[u].get(e);
    o[e] = slots_sum<LPR>(y);
  }
  sink(0, mx, sl, o);
}

// One unit of a zoomed span (c tokens, rank r <= D) of one kv head: the
// tokens [t0, min(c, t0 + TILE)), in rank space.  Units of one span are
// independent entries of the softmax and merge by log-sum-exp.
//   base: the span's packed bases A_K^T [r][c8] | B_K^T [r][D] | A_V^T [r][c8] | B_V^T [r][D]
// Lane (rank group rg = its row slot, token group tg = its lane in the slot)
// holds rank rows j = rg + RPW*u: for B_K^T / B_V^T the 16-byte piece at column
// tg*EPL, for A_K^T / A_V^T the piece of EPL tokens starting at t0 + tg*EPL.
// p_j lands, after the reduction inside the row slot, exactly in the lanes
// that hold row j of A_K^T, and w_j in those holding row j of B_V^T, so no
// data moves between the four products.  Addresses are clamped to valid rows
// and tokens; the rank rows a lane loads stop at the first one past r (the
// bound is the same for the whole wave).  A one-head group with
// r <= RBATCH issues every load of the unit in one round.  Otherwise the ranks
// go in batches of RBATCH rows: the key batches (B_K^T, A_K^T) accumulate the
// logits of every head in hb, then the value batches (A_V^T, B_V^T) the
// outputs, two rounds per batch; the heads are taken one after the other on
// each loaded batch.  qget(h, e) is element e of the lane's
// query slice of head h; each head's piece (softmax max in log2 units, sum,
// output slice of columns tg*EPL ..) goes to sink(h, max, sum, slice).
template <int D, typename T, int G, class QGet, class Sink>
__device__ __forceinline__ void zoom_unit(const T* __restrict__ base, int c, int r, int t0, uint32_t hb, QGet qget,
                                          Sink sink, float c2, int rg, int tg) {
  using Gm = Geo<D, T>;
  constexpr int EPL = Gm::EPL, LPR = Gm::LPR, RPW = Gm::RPW;
  constexpr int RB = Gm::RB, RBATCH = Gm::RBATCH;
  const int c8 = (c + 7) & ~7;
  const T* AKt = base;
  const T* BKt = AKt + (size_t)r * c8;
  const T* AVt = BKt + (size_t)r * D;
  const T* BVt = AVt + (size_t)r * c8;
  const int rl = r - 1;
  const int tok = t0 + tg * EPL;
  const int tokc = tok < c8 ? tok : t0;  // t0 < c: a valid piece

  if (G == 1 && r <= RBATCH) {
    // one head, one rank batch: as many rank rows per lane as r needs (r is
    // the same for the whole wave), so that no load repeats another
    UnitRows<T, RB> x;
    unit_rows_load<D, T, RB>(x, base, c8, r, tokc, rg, tg);
    unit_rows_attend<D, T, RB>(x, c, r, tok, qget, sink, c2, rg);
    return;
  }

  // ---------------- rank batches: the key batches accumulate the logits of
  // every head in hb, then the value batches accumulate the outputs
  float lg[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) lg[h][e] = 0.f;
#pragma unroll 1
  for (int j0 = 0; j0 < r; j0 += RBATCH) {
    const int nu = (r - j0 + RPW - 1) / RPW;  // rank rows per lane in this batch (the same for the wave)
    Raw<T> bk[RB], ak[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      if (u < nu) {
        const int j = min(j0 + rg + RPW * u, rl);
        bk[u].load(BKt + (size_t)j * D + tg * EPL);
        ak[u].load(AKt + (size_t)j * c8 + tokc);
      } else {
        bk[u].zero();
        ak[u].zero();
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (!((hb >> h) & 1u)) continue;
      if (G > 1) {
#pragma unroll
        for (int u = 0; u < RB; ++u) {
          keep_packed(bk[u]);
          keep_packed(ak[u]);
        }
      }
      float q[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) q[e] = qget(h, e);
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        float dp = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dp += q[e] * bk[u].get(e);
        dp = group_sum<LPR>(dp);
        const float pv = (j0 + rg + RPW * u < r) ? dp * c2 : 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) lg[h][e] += pv * ak[u].get(e);  // this row slot's ranks
      }
    }
  }
  float sm[G], sl[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = kNegInf;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float x = slots_sum<LPR>(lg[h][e]);
      x = (tok + e < c) ? x : kNegInf;
      lg[h][e] = x;
      mx = fmaxf(mx, x);
    }
    mx = group_max<LPR>(mx);
    float s1 = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      lg[h][e] = fast_exp2(lg[h][e] - mx);
      s1 += lg[h][e];
    }
    sm[h] = mx;
    sl[h] = group_sum<LPR>(s1);
  }
  float acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
#pragma unroll 1
  for (int j0 = 0; j0 < r; j0 += RBATCH) {
    const int nu = (r - j0 + RPW - 1) / RPW;
    Raw<T> av[RB], bv[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      if (u < nu) {
        const int j = min(j0 + rg + RPW * u, rl);
        av[u].load(AVt + (size_t)j * c8 + tokc);
        bv[u].load(BVt + (size_t)j * D + tg * EPL);
      } else {
        av[u].zero();
        bv[u].zero();
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (!((hb >> h) & 1u)) continue;
      if (G > 1) {
#pragma unroll
        for (int u = 0; u < RB; ++u) {
          keep_packed(av[u]);
          keep_packed(bv[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        float x = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) x += lg[h][e] * av[u].get(e);
        x = group_sum<LPR>(x);
        const float wv = (j0 + rg + RPW * u < r) ? x : 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] += wv * bv[u].get(e);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (!((hb >> h) & 1u)) continue;
    float o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = slots_sum<LPR>(acc[h][e]);
    sink(h, sm[h], sl[h], o);
  }
}

// ------------------------------------------------------------------ workgroup state and merges

template <int D, int G>
struct Smem {
  MergeLds<D, G> ml;
  float q[G][D];                 // the group's queries (zoom units)
  uint8_t zb[kMaxSpanChunk];     // zoom head bits of each row of a span chunk
  int2 zmeta[kMaxSpanChunk];     // their basis metadata (rows with zoom bits only)
  int3 zit[kMaxSpanChunk];       // a span task's zoomed spans
  int ustart[kMaxSpanChunk + 1]; // their first work unit (token tile)
  int wcount[kWaves];
  int s_int[4];
};

// Butterfly over the row slots of each wave, then one record per wave in LDS.
template <int D, int G, int EPL, int LPR>
__device__ void slots_to_lds(SoftState<G>& st, float (&acc)[G][EPL], MergeLds<D, G>& ml, int lane,
                             int wave, int slot, int sub) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
      const float mo = lane_xor(st.m[h], off);
      const float lo = lane_xor(st.l[h], off);
      float ao[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) ao[e] = lane_xor(acc[h][e], off);
      lse_merge<EPL>(st.m[h], st.l[h], acc[h], mo, lo, ao);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      ml.m[wave][h] = st.m[h];
      ml.l[wave][h] = st.l[h];
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) ml.acc[wave][h][sub * EPL + e] = acc[h][e];
  }
}

// Merge the per-wave records into one partial per head and store it in `part`,
// with the head's count of zoomed spans zc[h] (none: 0) for the zoom counters.
template <int D, int G>
__device__ void store_partial(const MergeLds<D, G>& ml, const DecodeArgs& a, int b, int g, int part,
                              const int* zc = nullptr) {
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, j = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int r = 0; r < kWaves; ++r) M = fmaxf(M, ml.m[r][h]);
    const float Ms = (M == kNegInf) ? 0.f : M;
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int r = 0; r < kWaves; ++r) {
      const float w = fast_exp2(ml.m[r][h] - Ms);
      L += ml.l[r][h] * w;
      A += ml.acc[r][h][j] * w;
    }
    const size_t slot = ((size_t)b * a.Hq + g * G + h) * a.max_parts + part;
    a.part_acc[slot * D + j] = A;
    if (j == 0) reinterpret_cast<float4*>(a.part_ml)[slot] = make_float4(M, L, zc ? (float)zc[h] : 0.f, 0.f);
  }
}

// An empty partial (no entries) for every head of the group.
template <int D, int G>
__device__ void store_empty(const DecodeArgs& a, int b, int g, int part) {
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, j = idx % D;
    const size_t slot = ((size_t)b * a.Hq + g * G + h) * a.max_parts + part;
    a.part_acc[slot * D + j] = 0.f;
    if (j == 0) reinterpret_cast<float4*>(a.part_ml)[slot] = make_float4(kNegInf, 0.f, 0.f, 0.f);
  }
}

template <int D, int G, typename T>
__device__ __forceinline__ void load_q(const DecodeArgs& a, int b, int g, int sub, float (&qr)[G][Elem<T>::kPer16]) {
  constexpr int EPL = Elem<T>::kPer16;
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; e += 4)
      Elem<float>::load16(a.q + ((size_t)b * a.Hq + g * G + h) * D + sub * EPL + e, qr[h] + e);
}

// ------------------------------------------------------------------ zoomed spans of one span task

static_assert(kMaxSpanChunk <= kThreads, "one thread per zoomed span of a task");

// The zc zoomed spans of one span task, cut into units of one token tile, the
// units spread over the waves (wave w takes units w, w + 4, ...), merged into
// one partial per query head stored in `part` (heads that zoom none of the
// spans get an empty one).  item(j) -> (head bits, basis offset / 8,
// rank | count << 8) is called by thread j < zc only, with j = its index.
template <int D, typename T, int G, bool MERGE, class Item>
__device__ void zoom_group(const DecodeArgs& a, int bg, int part, int zc, Item item, const T* __restrict__ src,
                           Smem<D, G>& sh) {
  using Gm = Geo<D, T>;
  constexpr int EPL = Gm::EPL, LPR = Gm::LPR, TILE = Gm::TILE;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rg = lane / LPR, tg = lane % LPR;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const float c2 = kLog2e * rsqrtf((float)D);
  // (G > 1) the group's queries into LDS; without a merge, empty records to fold into
  if (G > 1)
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads)
      sh.q[idx / D][idx % D] = a.q[((size_t)b * a.Hq + g * G) * D + idx];
  if (!MERGE) {
    for (int idx = lane; idx < G * D; idx += 64) sh.ml.acc[wave][idx / D][idx % D] = 0.f;
    if (lane < G) {
      sh.ml.m[wave][lane] = kNegInf;
      sh.ml.l[wave][lane] = 0.f;
    }
  }
  // unit table: tiles of span j start at ustart[j] (exclusive scan over the threads)
  {
    const int i = threadIdx.x;
    int nt = 0;
    if (i < zc) {
      const int3 it = item(i);
      sh.zit[i] = it;
      nt = ((int)((uint32_t)it.z >> 8) + TILE - 1) / TILE;
    }
    int incl = nt;
#pragma unroll
    for (int sft = 1; sft < 64; sft <<= 1) {
      const int y = __shfl_up(incl, sft, 64);
      if (lane >= sft) incl += y;
    }
    if (lane == 63) sh.wcount[wave] = incl;
    __syncthreads();
    int before = incl - nt, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (w < wave) before += sh.wcount[w];
      total += sh.wcount[w];
    }
    if (i < zc) sh.ustart[i] = before;
    if (i == 0) sh.ustart[zc] = total;  // zc <= kMaxSpanChunk
    __syncthreads();
  }
  const int units = sh.ustart[zc];
  // unit u of item j: the item is the same for the whole wave, in scalar
  // registers (loads then take a scalar base and a 32-bit lane offset)
  struct UnitRef {
    const T* base;
    uint32_t hb;
    int r, cnt, t0;
  };
  auto unit_ref = [&](int u, int j) -> UnitRef {
    const int3 it = sh.zit[j];
    const uint32_t hb = (uint32_t)__builtin_amdgcn_readfirstlane(it.x);  // head bits; kCachedBit: device cache
    const uint32_t iz = (uint32_t)__builtin_amdgcn_readfirstlane(it.z);
    const uint32_t off8 = (uint32_t)__builtin_amdgcn_readfirstlane(it.y);
    const T* from = (hb & kCachedBit) ? reinterpret_cast<const T*>(a.cache) : src;
    return {from + ((int64_t)off8 << 3), hb & 0xffu, (int)(iz & 0xffu), (int)(iz >> 8),
            __builtin_amdgcn_readfirstlane((u - sh.ustart[j]) * TILE)};
  };
  auto for_units = [&](auto qget, auto sink) {
    int j = 0;
#pragma unroll 1
    for (int u = wave; u < units; u += kWaves) {
      while (sh.ustart[j + 1] <= u) ++j;  // units are visited in increasing order
      const UnitRef x = unit_ref(u, j);
      if constexpr (G == 1 && kPairUnits) {
        // two units of rank <= RBATCH / 2 (this one and the wave's next) fit the
        // registers of one full-rank unit: load both in one round
        constexpr int NP = Gm::RB / 2;
        const int u2 = u + kWaves;
        if (x.r <= NP * Gm::RPW && u2 < units) {
          int j2 = j;
          while (sh.ustart[j2 + 1] <= u2) ++j2;
          const UnitRef y = unit_ref(u2, j2);
          if (y.r <= NP * Gm::RPW) {
            UnitRows<T, NP> X, Y;
            const int tx = x.t0 + tg * EPL, ty = y.t0 + tg * EPL;
            unit_rows_load<D, T, NP>(X, x.base, (x.cnt + 7) & ~7, x.r, tx < ((x.cnt + 7) & ~7) ? tx : x.t0, rg, tg);
            unit_rows_load<D, T, NP>(Y, y.base, (y.cnt + 7) & ~7, y.r, ty < ((y.cnt + 7) & ~7) ? ty : y.t0, rg, tg);
            unit_rows_attend<D, T, NP>(X, x.cnt, x.r, tx, qget, sink, c2, rg);
            unit_rows_attend<D, T, NP>(Y, y.cnt, y.r, ty, qget, sink, c2, rg);
            u = u2;
            j = j2;
            continue;
          }
        }
      }
      zoom_unit<D, T, G>(x.base, x.cnt, x.r, x.t0, x.hb, qget, sink, c2, rg, tg);
    }
  };
  if constexpr (G == 1) {
    // one head: the query slice and the running softmax stay in registers,
    // folded into the wave's record once
    if (wave < units) {
      float qr[EPL];
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        Elem<float>::load16(a.q + ((size_t)b * a.Hq + g) * D + tg * EPL + e, qr + e);
      float m = kNegInf, l = 0.f, acc[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
      for_units([&](int, int e) { return qr[e]; },
                [&](int, float sm, float sl, const float (&o)[EPL]) { lse_merge<EPL>(m, l, acc, sm, sl, o); });
      fold_record<D, G, EPL>(sh.ml, wave, 0, lane, rg, tg, m, l, acc);
    }
  } else {
    // several heads: queries from LDS, each head's pieces folded into the wave's records
    for_units([&](int h, int e) { return sh.q[h][tg * EPL + e]; },
              [&](int h, float sm, float sl, const float (&o)[EPL]) {
                fold_record<D, G, EPL>(sh.ml, wave, h, lane, rg, tg, sm, sl, o);
              });
  }
  if (MERGE) return;  // the records of the caller's partial now hold the zoomed entries too
  __syncthreads();
  store_partial<D, G>(sh.ml, a, b, g, part);
}

// ------------------------------------------------------------------ anchor task

// Rows per row slot per pipeline stage of the streaming tasks; two stages are
// in flight.  Span tasks (one round each, with d = 128 bf16: 32 rows of
// summaries and values per stage) run in a lean kernel; anchor tasks share
// the attend kernel's register budget with the zoom and use deeper stages.
constexpr int kSpanStageRows = 2;
constexpr int kAnchorStageRows = 4;

// One pipeline stage of a row slot: U rows of keys (or summaries) and values.
template <typename T, int U>
struct Stage {
  Raw<T> k[U], v[U];
  float ls[U];
  int2 meta[U];      // span rows: {basis offset / 8, rank | count << 8}
  uint32_t zsel[U];  // span rows under the budget cap: zoom bit of each head
  Raw<T> kr[U];      // span rows with a routing projection: piece of the routing summary
};

template <int D, typename T, int G>
__device__ void anchor_task(const DecodeArgs& a, int4 task, Smem<D, G>& sh) {
  MergeLds<D, G>& ml = sh.ml;
  using Gm = Geo<D, T>;
  constexpr int EPL = Gm::EPL, LPR = Gm::LPR, RPW = Gm::RPW;
  constexpr int U = G >= 4 ? 1 : kAnchorStageRows;  // wide groups: registers for the heads
  constexpr int STEP = kWaves * RPW * U;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane / LPR, sub = lane % LPR;
  const int bg = task.x & 0x7fffffff;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const float c2 = kLog2e * rsqrtf((float)D);
  SoftState<G> st;
  float acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = kNegInf;
    st.l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  const int r0 = task.y;
  const int r1 = r0 + task.z;  // the planner clamps the chunk to the anchor count
  const T* Kb = reinterpret_cast<const T*>(a.KA) + (size_t)bg * a.na_max * D + sub * EPL;
  const T* Vb = reinterpret_cast<const T*>(a.VA) + (size_t)bg * a.na_max * D + sub * EPL;
  auto load = [&](Stage<T, U>& sg, int bs) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = bs + u * RPW + slot;
      const int rr = row < r1 ? row : r0;
      sg.k[u].load(Kb + (size_t)rr * D);
      sg.v[u].load(Vb + (size_t)rr * D);
    }
  };
  // wide groups keep the queries in LDS: G x EPL registers less, read once per head and stage
  constexpr bool QLDS = G >= 4;
  float qr[QLDS ? 1 : G][EPL];
  auto consume = [&](const Stage<T, U>& sg, int bs) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float qh[EPL];
      if constexpr (QLDS) {
#pragma unroll
        for (int e = 0; e < EPL; e += 4) *reinterpret_cast<float4*>(qh + e) = *reinterpret_cast<const float4*>(&sh.q[h][sub * EPL + e]);
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) qh[e] = qr[h][e];
      }
      Raw<T> kx[U], vx[U];  // per head, so that their unpacking is not hoisted out of the loop
#pragma unroll
      for (int u = 0; u < U; ++u) {
        kx[u] = sg.k[u];
        vx[u] = sg.v[u];
        if (G > 1) {
          keep_packed(kx[u]);
          keep_packed(vx[u]);
        }
      }
      float lg[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float dp = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dp += qh[e] * kx[u].get(e);
        dp = group_sum<LPR>(dp);
        lg[u] = (bs + u * RPW + slot < r1) ? dp * c2 : kNegInf;
      }
      float mx = st.m[h];
#pragma unroll
      for (int u = 0; u < U; ++u) mx = fmaxf(mx, lg[u]);
      const float ms = (mx == kNegInf) ? 0.f : mx;
      const float sc = fast_exp2(st.m[h] - ms);
      float ls = st.l[h] * sc;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= sc;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = fast_exp2(lg[u] - ms);
        ls += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] += p * vx[u].get(e);
      }
      st.l[h] = ls;
      st.m[h] = mx;
    }
  };
  int bs = r0 + wave * RPW * U;
  if constexpr (QLDS) {
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads)
      sh.q[idx / D][idx % D] = a.q[((size_t)b * a.Hq + g * G) * D + idx];
    __syncthreads();
  }
  if (bs < r1) {
    Stage<T, U> A, B;
    load(A, bs);
    if constexpr (!QLDS) load_q<D, G, T>(a, b, g, sub, qr);
    for (; bs < r1; bs += 2 * STEP) {
      load(B, bs + STEP);
      consume(A, bs);
      if (bs + STEP >= r1) break;
      load(A, bs + 2 * STEP);
      consume(B, bs + STEP);
    }
  }
  slots_to_lds<D, G, EPL, LPR>(st, acc, ml, lane, wave, slot, sub);
  __syncthreads();
  store_partial<D, G>(ml, a, b, g, task.w);
}

// ------------------------------------------------------------------ span task

// MODE 1: zoomed spans appended to the flat list for the host fetch.
// MODE 2: routing scores only.
template <int D, typename T, int G, int MODE, bool ROUTED>
__device__ void span_task(const DecodeArgs& a, int t, int4 task, Smem<D, G>& sh) {
  using Gm = Geo<D, T>;
  constexpr int EPL = Gm::EPL, LPR = Gm::LPR, RPW = Gm::RPW;
  constexpr int U = G >= 4 ? 1 : kSpanStageRows;
  constexpr int STEP = kWaves * RPW * U;
  constexpr bool SCORES = MODE == 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane / LPR, sub = lane % LPR;
  const int bg = task.x;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const float c2 = kLog2e * rsqrtf((float)D);
  const float inv_sqrt_d = rsqrtf((float)D);
  SoftState<G> st;
  float acc[G][EPL];
  float zcl[G];  // zoomed spans per head among this lane's rows (first lane of each row slot)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = kNegInf;
    st.l[h] = 0.f;
    zcl[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  const int k0 = task.y;
  const int k1 = k0 + task.z;  // the planner clamps the chunk to the span count
  const T* Kb = reinterpret_cast<const T*>(a.kbar) + (size_t)bg * a.m_max * D + sub * EPL;
  const T* Vb = reinterpret_cast<const T*>(a.vbar) + (size_t)bg * a.m_max * D + sub * EPL;
  const float* lS = a.logS + (size_t)b * a.m_max;
  auto load = [&](Stage<T, U>& sg, int bs) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = bs + u * RPW + slot;
      const int kk = k < k1 ? k : k0;
      sg.k[u].load(Kb + (size_t)kk * D);
      if (!SCORES) sg.v[u].load(Vb + (size_t)kk * D);
      sg.ls[u] = lS[kk];
      if (!SCORES) sg.meta[u] = a.smeta[(size_t)bg * a.m_max + kk];  // every lane: no load under a lane condition
      if (ROUTED) {
        const int sp = sub * EPL < a.dr ? sub : 0;  // lanes beyond d' load piece 0 (unused)
        sg.kr[u].load(reinterpret_cast<const T*>(a.Kr) + ((size_t)bg * a.m_max + kk) * a.dr + sp * EPL);
      }
      if (!SCORES && a.capped) {
        uint32_t bits = 0u;
#pragma unroll
        for (int h = 0; h < G; ++h)
          bits |= (a.mask[((size_t)b * a.Hq + g * G + h) * a.m_max + kk] != 0 ? 1u : 0u) << h;
        sg.zsel[u] = bits;
      }
    }
  };
  constexpr bool QLDS = G >= 4 && !ROUTED;
  float qr[QLDS ? 1 : G][EPL];
  float qpr[ROUTED ? G : 1][EPL];  // projected query piece (routing projection), zero beyond d'
  constexpr bool routed = ROUTED;
  const float inv_sqrt_dr = routed ? rsqrtf((float)a.dr) : 0.f;
  auto consume = [&](const Stage<T, U>& sg, int bs) {
    float nrm[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float s2 = 0.f;
      if (!routed) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) s2 += sg.k[u].get(e) * sg.k[u].get(e);
        s2 = group_sum<LPR>(s2);
      }
      nrm[u] = s2;
    }
    uint32_t zbits[U];
#pragma unroll
    for (int u = 0; u < U; ++u) zbits[u] = 0u;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float qh[EPL];
      if constexpr (QLDS) {
#pragma unroll
        for (int e = 0; e < EPL; e += 4) *reinterpret_cast<float4*>(qh + e) = *reinterpret_cast<const float4*>(&sh.q[h][sub * EPL + e]);
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) qh[e] = qr[h][e];
      }
      Raw<T> kx[U], vx[U];  // per head, so that their unpacking is not hoisted out of the loop
#pragma unroll
      for (int u = 0; u < U; ++u) {
        kx[u] = sg.k[u];
        vx[u] = sg.v[u];
        if (G > 1) {
          keep_packed(kx[u]);
          keep_packed(vx[u]);
        }
      }
      float lg[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float dp = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dp += qh[e] * kx[u].get(e);
        dp = group_sum<LPR>(dp);
        float score;
        if (routed) {
          float dq = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) dq += qpr[ROUTED ? h : 0][e] * sg.kr[u].get(e);
          score = group_sum<LPR>(dq) * inv_sqrt_dr + sg.ls[u];
        } else {
          score = (nrm[u] > 0.f ? dp * rsqrtf(nrm[u]) * inv_sqrt_d : 0.f) + sg.ls[u];
        }
        const int k = bs + u * RPW + slot;
        const bool ok = k < k1;
        const bool zoom = (!SCORES && a.capped) ? ((sg.zsel[u] >> h) & 1u) != 0u
                                                : (double)score > a.theta[g * G + h];
        if (ok && sub == 0) {
          const size_t mi = ((size_t)b * a.Hq + g * G + h) * a.m_max + k;
          if (SCORES) a.scores[mi] = score;
          else if (!a.capped) a.mask[mi] = zoom ? 1 : 0;
        }
        if (zoom) zbits[u] |= 1u << h;
        lg[u] = (ok && !zoom) ? dp * c2 + sg.ls[u] * kLog2e : kNegInf;
      }
      if (!SCORES) {
        float mx = st.m[h];
#pragma unroll
        for (int u = 0; u < U; ++u) mx = fmaxf(mx, lg[u]);
        const float ms = (mx == kNegInf) ? 0.f : mx;
        const float sc = fast_exp2(st.m[h] - ms);
        float ls = st.l[h] * sc;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= sc;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float p = fast_exp2(lg[u] - ms);
          ls += p;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] += p * vx[u].get(e);
        }
        st.l[h] = ls;
        st.m[h] = mx;
      }
    }
    if (!SCORES && sub == 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = bs + u * RPW + slot;
        if (k < k1) {
          sh.zb[k - k0] = (uint8_t)zbits[u];
          if (zbits[u]) sh.zmeta[k - k0] = sg.meta[u];
#pragma unroll
          for (int h = 0; h < G; ++h) zcl[h] += (float)((zbits[u] >> h) & 1u);
        }
      }
    }
  };
  int bs = k0 + wave * RPW * U;
  if constexpr (QLDS) {
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads)
      sh.q[idx / D][idx % D] = a.q[((size_t)b * a.Hq + g * G) * D + idx];
    __syncthreads();
  }
  if (bs < k1) {
    Stage<T, U> A, B;
    load(A, bs);
    if constexpr (!QLDS) load_q<D, G, T>(a, b, g, sub, qr);
    if constexpr (ROUTED) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const bool in = sub * EPL < a.dr;
        const float* src = a.qp + ((size_t)b * a.Hq + g * G + h) * a.dr + (in ? sub * EPL : 0);
#pragma unroll
        for (int e = 0; e < EPL; e += 4) Elem<float>::load16(src + e, qpr[h] + e);
#pragma unroll
        for (int e = 0; e < EPL; ++e) qpr[h][e] = in ? qpr[h][e] : 0.f;
      }
    }
    for (; bs < k1; bs += 2 * STEP) {
      load(B, bs + STEP);
      consume(A, bs);
      if (bs + STEP >= k1) break;
      load(A, bs + 2 * STEP);
      consume(B, bs + STEP);
    }
  }
  if (SCORES) return;
  if (a.zcount) {
    // the layer's zoom counters: this wave's zoomed spans of each head
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float z = wave_sum(zcl[h]);
      if (lane == 0 && z > 0.f)
        __hip_atomic_fetch_add(a.zcount + (size_t)b * a.Hq + g * G + h, (unsigned long long)z, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  slots_to_lds<D, G, EPL, LPR>(st, acc, sh.ml, lane, wave, slot, sub);
  __syncthreads();  // zoom bits and records complete

  // the chunk's zoomed spans, compacted in span order
  const int cnt = max(0, k1 - k0);
  const int i = threadIdx.x;
  const uint32_t hb = i < cnt ? sh.zb[i] : 0u;
  const u64 bal = __ballot(hb != 0);
  int pos = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) sh.wcount[wave] = __popcll(bal);
  store_partial<D, G>(sh.ml, a, b, g, task.w);
  __syncthreads();
  int zc = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) pos += sh.wcount[w];
    zc += sh.wcount[w];
  }
  if (zc == 0) store_empty<D, G>(a, b, g, task.w + 1);  // the zoom slot, when nothing fills it
  if (threadIdx.x == 0) a.zcnt[t] = zc;
  // MODE 1: list for the host fetch
  if (zc) {
    if (threadIdx.x == 0) sh.s_int[0] = atomicAdd(a.zcounter, zc);
    __syncthreads();
    if (hb) {
      const int2 meta = sh.zmeta[i];
      a.zlist[sh.s_int[0] + pos] = make_int4(bg | (int)(hb << 24), k0 + i, meta.x, meta.y);
    }
  }
}

// ------------------------------------------------------------------ planned layer-step kernel

// The planned kernel runs one wave of workgroups over the whole layer-step.
// The runtime cuts the sequence "span rows of (b, g), anchor rows of (b, g),
// next (b, g) ..." into one contiguous share per workgroup, of equal predicted
// cost: bytes streamed plus the bases of the spans predicted to be zoomed (the
// zoom sets of the previous calls).  A share is a short list of segments, each
// folded into one partial slot of its (sequence, kv head).  A workgroup streams
// its span segments first (routing scores, zoom decisions, summary entries),
// then its anchor segments, then rebuilds its zoomed spans (token-tile units
// spread over the waves), and stores one partial per segment.  The
// rows of a segment are interleaved over the waves by pipeline stage; each
// wave keeps its own running record per segment in LDS, merged at the end.
template <int D, int G, int NS>
struct PlanSmem {
  int4 seg[NS];                    // the workgroup's segment descriptors
  MergeLds<D, G> rec[NS];          // wave records of each segment
  float q[NS][G][D];               // queries of each segment's group
  uint8_t zb[kMaxWgSpanRows];      // zoom head bits of each span row of the share, in segment order
  int2 zmeta[kMaxWgSpanRows];      // basis metadata of the rows with zoom bits
  int4 zit[kMaxWgSpanRows];        // zoomed spans: (head bits | kCachedBit, basis offset / 8, rank | count << 8, segment | bg << 8)
  int ustart[kMaxWgSpanRows + 1];  // their first work unit
  int red[kWaves][2];
  int zcnt[NS][G];                 // spans each head zoomed in each segment
};

// Span rows [k0, k0 + rows) of one (b, g): routing scores and zoom decisions
// (mask, and the head bits and basis metadata of row k at zb[rb + k - k0]),
// and the summary entries of the rows each head does not zoom, folded into the
// wave's record of segment s.
// Rows per row slot per round of the planned kernel's streaming.  One round's
// loads are issued together and consumed before the next round: the stage
// registers are not carried across loop iterations (a carried stage makes the
// compiler copy it at the loop head, which waits for every load in flight).
#ifndef SEKV_PLAN_ROWS
#define SEKV_PLAN_ROWS 2
#endif

template <int G, bool ROUTED = false>
__host__ __device__ constexpr int plan_rows() {
  return G == 1 ? SEKV_PLAN_ROWS : G == 2 ? 2 : 1;
}

// Double-buffered rounds of one wave: round j starts at row first + j * step,
// for the rounds that start before `end`.  The next round's loads are issued
// before the current round is consumed; scheduling barriers keep the compiler
// from moving them below the consumption, and the loop runs over pairs of
// rounds with no early exit and no conditional load, so that neither buffer is
// copied at the loop head and every wait covers one round only.  The load past
// the last round reads rows clamped into the segment (the loaders clamp rows
// at or beyond `end`): L2 hits, never consumed.
template <class Buf, class Load, class Consume>
__device__ __forceinline__ void stream_rounds(int first, int end, int step, Load load, Consume consume) {
  if (first >= end) return;
  const int n = (end - first + step - 1) / step;
  Buf A, B;
  load(A, first);
  int bs = first, i = 0;
  for (; i + 2 <= n; i += 2) {
    load(B, bs + step);
    __builtin_amdgcn_sched_barrier(0);
    consume(A, bs);
    load(A, bs + 2 * step);
    __builtin_amdgcn_sched_barrier(0);
    consume(B, bs + step);
    bs += 2 * step;
  }
  if (i < n) consume(A, bs);
}

// One row's entry added to a running softmax record (logit lg in log2 units,
// -inf for no entry).  The record's reference m moves only when a logit of
// the wave exceeds it by more than kSlack: the weights then stay below
// 2^kSlack, and a row that moves no reference (the common case, decided for
// the whole wave) costs one exp2 and the accumulation, without the rescale of
// the accumulator.  The record keeps its meaning (each entry weighted by
// 2^(logit - m)), so the merges and acc / l are unchanged; m lies at most
// kSlack below the largest logit folded in.
constexpr float kSlack = 8.f;

template <typename T, int EPL>
__device__ __forceinline__ void online_add(float& m, float& l, float (&acc)[EPL], float lg, const Raw<T>& v) {
  if (__builtin_amdgcn_ballot_w64(lg > m + kSlack) != 0) {
    const float mn = fmaxf(m, lg);
    const float ms = (mn == kNegInf) ? 0.f : mn;
    const float sc = fast_exp2(m - ms), p = fast_exp2(lg - ms);
    l = l * sc + p;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = acc[e] * sc + p * v.get(e);
    m = mn;
    return;
  }
  // m = -inf here only with lg = -inf (no entry yet, none now)
  const float p = fast_exp2(lg - ((m == kNegInf) ? 0.f : m));
  l += p;
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] += p * v.get(e);
}

// 16-byte piece at a byte offset from a base shared by the wave: the address is
// a scalar base plus a 32-bit lane offset.
template <typename T>
__device__ __forceinline__ void load_at(Raw<T>& r, const T* base, uint32_t off) {
  r.load(reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + off));
}
template <typename X>
__device__ __forceinline__ X load_off(const X* base, uint32_t off) {
  return *reinterpret_cast<const X*>(reinterpret_cast<const char*>(base) + off);
}

// Span rows [k0, k0 + rows) of one (b, g): routing scores and zoom decisions
// (the head bits and basis metadata of row k at zb / zmeta[rb + k - k0]; the
// mask is written from them after the streaming), and the summary entries of
// the rows each head does not zoom, folded into the wave's record of segment s.
// One round of span rows: the key and value pieces of U rows per row slot,
// and, in lane l < RPW * U, ln|S| and the basis metadata of row l of the round
// (one load each for the whole round).
template <typename T, int U>
struct SpanRound {
  Raw<T> k[U], v[U];
  Raw<T> kr[U];      // with a routing projection: piece of the routing summary
  uint32_t zsel[U];  // under the budget cap: zoom bit of each head
  float ls;
  int2 meta;
};

template <int D, typename T, int G, bool ROUTED, bool CAPPED, int NS>
__device__ void plan_span_rows(const DecodeArgs& a, int4 sg, int s, int rb, PlanSmem<D, G, NS>& sh) {
  using Gm = Geo<D, T>;
  constexpr int EPL = Gm::EPL, LPR = Gm::LPR, RPW = Gm::RPW;
  constexpr int U = plan_rows<G, ROUTED>();
  constexpr int RR = RPW * U;  // rows per wave per round
  static_assert(RR <= 64, "one lane per row of a round");
  constexpr int STEP = kWaves * RR;
  constexpr uint32_t ROWB = D * sizeof(T);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane / LPR, sub = lane % LPR;
  const int bg = sg.x;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const float c2 = kLog2e * rsqrtf((float)D);
  const float inv_sqrt_d = rsqrtf((float)D);
  SoftState<G> st;
  float acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = kNegInf;
    st.l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  const int k0 = sg.y;
  const int k1 = k0 + sg.z;
  // bases of this (b, g): uniform over the wave
  const T* Kb = reinterpret_cast<const T*>(a.kbar) + (size_t)bg * a.m_max * D;
  const T* Vb = reinterpret_cast<const T*>(a.vbar) + (size_t)bg * a.m_max * D;
  const float* lS = a.logS + (size_t)b * a.m_max;
  const int2* Mb = a.smeta + (size_t)bg * a.m_max;
  const T* Rb = ROUTED ? reinterpret_cast<const T*>(a.Kr) + (size_t)bg * a.m_max * a.dr : nullptr;
  const uint32_t sub_off = sub * 16u;
  auto load = [&](SpanRound<T, U>& rd, int bs) {
    // the round's ln|S| and metadata first: the row loop needs them early
    {
      const int kl = bs + (lane < RR ? lane : 0);
      const uint32_t kc = (uint32_t)(kl < k1 ? kl : k0);
      rd.ls = load_off(lS, kc * 4u);
      rd.meta = load_off(Mb, kc * 8u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = bs + u * RPW + slot;
      const uint32_t kk = (uint32_t)(k < k1 ? k : k0);
      load_at(rd.k[u], Kb, kk * ROWB + sub_off);
      load_at(rd.v[u], Vb, kk * ROWB + sub_off);
      if (ROUTED) {
        const uint32_t sp = sub * EPL < a.dr ? sub_off : 0u;  // lanes beyond d' load piece 0 (unused)
        load_at(rd.kr[u], Rb, kk * (uint32_t)a.dr * (uint32_t)sizeof(T) + sp);
      }
      if (CAPPED) {
        uint32_t bits = 0u;
#pragma unroll
        for (int h = 0; h < G; ++h)
          bits |= (a.mask[((size_t)b * a.Hq + g * G + h) * a.m_max + kk] != 0 ? 1u : 0u) << h;
        rd.zsel[u] = bits;
      }
    }
  };
  constexpr bool QLDS = G >= 4 && !ROUTED;
  float qr[QLDS ? 1 : G][EPL];
  float qpr[ROUTED ? G : 1][EPL];  // projected query piece (routing projection), zero beyond d'
  const float inv_sqrt_dr = ROUTED ? rsqrtf((float)a.dr) : 0.f;
  auto consume = [&](const SpanRound<T, U>& rd, int bs) {
    uint32_t zbu[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float nrm = 0.f;
      if (!ROUTED) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) nrm += rd.k[u].get(e) * rd.k[u].get(e);
        nrm = group_sum<LPR>(nrm);
      }
      const float ls = __shfl(rd.ls, u * RPW + slot, 64);
      const int k = bs + u * RPW + slot;
      const bool ok = k < k1;
      uint32_t zbits = 0u;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float qh[EPL];
        if constexpr (QLDS) {
#pragma unroll
          for (int e = 0; e < EPL; e += 4)
            *reinterpret_cast<float4*>(qh + e) = *reinterpret_cast<const float4*>(&sh.q[s][h][sub * EPL + e]);
        } else {
#pragma unroll
          for (int e = 0; e < EPL; ++e) qh[e] = qr[h][e];
        }
        // (the row's unpacked key and value serve every head of the group: 6%
        // faster for groups of four than unpacking them again per head)
        const Raw<T>& kx = rd.k[u];
        const Raw<T>& vx = rd.v[u];
        float dp = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dp += qh[e] * kx.get(e);
        dp = group_sum<LPR>(dp);
        float score;
        if (ROUTED) {
          float dq = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) dq += qpr[ROUTED ? h : 0][e] * rd.kr[u].get(e);
          score = group_sum<LPR>(dq) * inv_sqrt_dr + ls;
        } else {
          score = (nrm > 0.f ? dp * rsqrtf(nrm) * inv_sqrt_d : 0.f) + ls;
        }
        const bool zoom = CAPPED ? ((rd.zsel[u] >> h) & 1u) != 0u : (double)score > a.theta[g * G + h];
        if (zoom) zbits |= 1u << h;
        online_add<T, EPL>(st.m[h], st.l[h], acc[h], (ok && !zoom) ? dp * c2 + ls * kLog2e : kNegInf, vx);
      }
      zbu[u] = zbits;
    }
    // zoom bookkeeping after the round: head bits from the first lane of each
    // row slot, the metadata of every row from the lane that loaded it
    if (sub == 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = bs + u * RPW + slot;
        if (k < k1) sh.zb[rb + k - k0] = (uint8_t)zbu[u];
      }
    }
    if (lane < RR && bs + lane < k1) sh.zmeta[rb + bs + lane - k0] = rd.meta;
  };
  const int first = k0 + wave * RR;
  if (first < k1) {
    if constexpr (!QLDS) load_q<D, G, T>(a, b, g, sub, qr);
    if constexpr (ROUTED) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const bool in = sub * EPL < a.dr;
        const float* src = a.qp + ((size_t)b * a.Hq + g * G + h) * a.dr + (in ? sub * EPL : 0);
#pragma unroll
        for (int e = 0; e < EPL; e += 4) Elem<float>::load16(src + e, qpr[h] + e);
#pragma unroll
        for (int e = 0; e < EPL; ++e) qpr[h][e] = in ? qpr[h][e] : 0.f;
      }
    }
    stream_rounds<SpanRound<T, U>>(first, k1, STEP, load, consume);
  }
  slots_to_lds<D, G, EPL, LPR>(st, acc, sh.rec[s], lane, wave, slot, sub);
}

// Anchor rows [r0, r0 + rows) of one (b, g), exact entries, folded into the
// wave's record of segment s.
template <int D, typename T, int G, int NS>
__device__ void plan_anchor_rows(const DecodeArgs& a, int4 sg, int s, PlanSmem<D, G, NS>& sh) {
  using Gm = Geo<D, T>;
  constexpr int EPL = Gm::EPL, LPR = Gm::LPR, RPW = Gm::RPW;
  constexpr int U = plan_rows<G>();
  constexpr int STEP = kWaves * RPW * U;
  constexpr uint32_t ROWB = D * sizeof(T);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane / LPR, sub = lane % LPR;
  const int bg = sg.x & 0x7fffffff;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const float c2 = kLog2e * rsqrtf((float)D);
  SoftState<G> st;
  float acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = kNegInf;
    st.l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  const int r0 = sg.y;
  const int r1 = r0 + sg.z;
  const T* Kb = reinterpret_cast<const T*>(a.KA) + (size_t)bg * a.na_max * D;
  const T* Vb = reinterpret_cast<const T*>(a.VA) + (size_t)bg * a.na_max * D;
  const uint32_t sub_off = sub * 16u;
  auto load = [&](Stage<T, U>& sgs, int bs) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = bs + u * RPW + slot;
      const uint32_t rr = (uint32_t)(row < r1 ? row : r0);
      load_at(sgs.k[u], Kb, rr * ROWB + sub_off);
      load_at(sgs.v[u], Vb, rr * ROWB + sub_off);
    }
  };
  constexpr bool QLDS = G >= 4;
  float qr[QLDS ? 1 : G][EPL];
  auto consume = [&](const Stage<T, U>& sgs, int bs) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = bs + u * RPW + slot < r1;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float qh[EPL];
        if constexpr (QLDS) {
#pragma unroll
          for (int e = 0; e < EPL; e += 4)
            *reinterpret_cast<float4*>(qh + e) = *reinterpret_cast<const float4*>(&sh.q[s][h][sub * EPL + e]);
        } else {
#pragma unroll
          for (int e = 0; e < EPL; ++e) qh[e] = qr[h][e];
        }
        const Raw<T>& kx = sgs.k[u];
        const Raw<T>& vx = sgs.v[u];
        float dp = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dp += qh[e] * kx.get(e);
        dp = group_sum<LPR>(dp);
        online_add<T, EPL>(st.m[h], st.l[h], acc[h], ok ? dp * c2 : kNegInf, vx);
      }
    }
  };
  const int first = r0 + wave * RPW * U;
  if (first < r1) {
    if constexpr (!QLDS) load_q<D, G, T>(a, b, g, sub, qr);
    stream_rounds<Stage<T, U>>(first, r1, STEP, load, consume);
  }
  slots_to_lds<D, G, EPL, LPR>(st, acc, sh.rec[s], lane, wave, slot, sub);
}

// Zoom phase of a share: the zoomed spans of its R span rows (zoom bits in
// zb, in segment order) compacted in row order, cut into token-tile units
// spread over the waves (wave w takes units w, w + 4, ...), each folded into
// the wave's record of its segment.
template <int D, typename T, int G, int NS>
__device__ void plan_zoom(const DecodeArgs& a, int nseg, int R, PlanSmem<D, G, NS>& sh) {
  using Gm = Geo<D, T>;
  constexpr int EPL = Gm::EPL, TILE = Gm::TILE, LPR = Gm::LPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rg = lane / LPR, tg = lane % LPR;
  // thread i takes rows 2i and 2i + 1 (R <= kMaxWgSpanRows = 2 * kThreads)
  static_assert(kMaxWgSpanRows == 2 * kThreads, "two span rows per thread in the compaction");
  int cnt = 0, tiles = 0;
  uint32_t hb2[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int j = 2 * (int)threadIdx.x + e;
    hb2[e] = j < R ? sh.zb[j] : 0u;
    if (hb2[e]) {
      ++cnt;
      tiles += ((int)((uint32_t)sh.zmeta[j].y >> 8) + TILE - 1) / TILE;
    }
  }
  // exclusive scan of (cnt, tiles) over the workgroup
  int ic = cnt, it = tiles;
#pragma unroll
  for (int sft = 1; sft < 64; sft <<= 1) {
    const int yc = __shfl_up(ic, sft, 64), yt = __shfl_up(it, sft, 64);
    if (lane >= sft) {
      ic += yc;
      it += yt;
    }
  }
  if (lane == 63) {
    sh.red[wave][0] = ic;
    sh.red[wave][1] = it;
  }
  __syncthreads();
  int pc = ic - cnt, pt = it - tiles, zc = 0, units = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) {
      pc += sh.red[w][0];
      pt += sh.red[w][1];
    }
    zc += sh.red[w][0];
    units += sh.red[w][1];
  }
  if (zc == 0) return;  // uniform over the workgroup
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    if (!hb2[e]) continue;
    const int j = 2 * (int)threadIdx.x + e;
    // the segment of span row j
    int s = 0, rs = 0, k = 0, bg = 0;
    {
      int acc = 0;
      for (int t = 0; t < nseg; ++t) {
        const int4 sg = sh.seg[t];
        if (sg.x < 0) continue;
        if (j >= acc && j < acc + sg.z) {
          s = t;
          rs = acc;
          k = sg.y + j - acc;
          bg = sg.x;
        }
        acc += sg.z;
      }
    }
    (void)rs;
    int off8 = sh.zmeta[j].x;
    uint32_t bits = hb2[e];
    if (a.cslot) {  // host-resident bases with a device cache: use the cached copy if any
      const int cs = a.cslot[(size_t)bg * a.m_max + k];
      if (cs >= 0) {
        off8 = cs;
        bits |= kCachedBit;
      }
    }
    sh.zit[pc] = make_int4((int)bits, off8, sh.zmeta[j].y, s | (bg << 8));
    // the segment's zoom counts (its slot reports them to the combine)
#pragma unroll
    for (int h = 0; h < G; ++h)
      if ((hb2[e] >> h) & 1u) atomicAdd(&sh.zcnt[s][h], 1);
    sh.ustart[pc] = pt;
    pt += ((int)((uint32_t)sh.zmeta[j].y >> 8) + TILE - 1) / TILE;
    ++pc;
  }
  if (threadIdx.x == 0) sh.ustart[zc] = units;
  __syncthreads();

  const float c2 = kLog2e * rsqrtf((float)D);
  const T* src = reinterpret_cast<const T*>(a.bases);
  struct UnitRef {
    const T* base;
    uint32_t hb;
    int r, cnt, t0, s, bg;
  };
  auto unit_ref = [&](int u, int j) -> UnitRef {
    const int4 itm = sh.zit[j];
    const uint32_t hb = (uint32_t)__builtin_amdgcn_readfirstlane(itm.x);
    const uint32_t iz = (uint32_t)__builtin_amdgcn_readfirstlane(itm.z);
    const uint32_t off8 = (uint32_t)__builtin_amdgcn_readfirstlane(itm.y);
    const int sw = __builtin_amdgcn_readfirstlane(itm.w);
    const T* from = (hb & kCachedBit) ? reinterpret_cast<const T*>(a.cache) : src;
    return {from + ((int64_t)off8 << 3), hb & 0xffu, (int)(iz & 0xffu), (int)(iz >> 8),
            __builtin_amdgcn_readfirstlane((u - sh.ustart[j]) * TILE), sw & 0xff, sw >> 8};
  };
  if constexpr (G == 1) {
    // one head: each unit's piece folded into the wave's record of its segment
    // (LDS), so that no running record stays in registers across the units
    int j = 0;
#pragma unroll 1
    for (int u = wave; u < units; u += kWaves) {
      while (sh.ustart[j + 1] <= u) ++j;  // units are visited in increasing order
      const UnitRef x = unit_ref(u, j);
      const int s = x.s;
      auto qget = [&](int, int e) { return sh.q[s][0][tg * EPL + e]; };
      auto sink = [&](int, float sm, float sl, const float (&o)[EPL]) {
        fold_record<D, G, EPL>(sh.rec[s], wave, 0, lane, rg, tg, sm, sl, o);
      };
      if constexpr (kPairUnits) {
        // two units of rank <= RBATCH / 2 (this one and the wave's next, of the
        // same segment) fit the registers of one full-rank unit: one round of loads
        constexpr int NP = Gm::RB / 2;
        const int u2 = u + kWaves;
        if (x.r <= NP * Gm::RPW && u2 < units) {
          int j2 = j;
          while (sh.ustart[j2 + 1] <= u2) ++j2;
          const UnitRef y = unit_ref(u2, j2);
          if (y.r <= NP * Gm::RPW && y.s == x.s) {
            UnitRows<T, NP> X, Y;
            const int cx8 = (x.cnt + 7) & ~7, cy8 = (y.cnt + 7) & ~7;
            const int tx = x.t0 + tg * EPL, ty = y.t0 + tg * EPL;
            unit_rows_load<D, T, NP>(X, x.base, cx8, x.r, tx < cx8 ? tx : x.t0, rg, tg);
            unit_rows_load<D, T, NP>(Y, y.base, cy8, y.r, ty < cy8 ? ty : y.t0, rg, tg);
            unit_rows_attend<D, T, NP>(X, x.cnt, x.r, tx, qget, sink, c2, rg);
            unit_rows_attend<D, T, NP>(Y, y.cnt, y.r, ty, qget, sink, c2, rg);
            u = u2;
            j = j2;
            continue;
          }
        }
      }
      zoom_unit<D, T, G>(x.base, x.cnt, x.r, x.t0, x.hb, qget, sink, c2, rg, tg);
    }
  } else {
    // several heads: queries from LDS, each head's pieces folded into the wave's records
    int j = 0;
#pragma unroll 1
    for (int u = wave; u < units; u += kWaves) {
      while (sh.ustart[j + 1] <= u) ++j;
      const UnitRef x = unit_ref(u, j);
      const int s = x.s;
      zoom_unit<D, T, G>(x.base, x.cnt, x.r, x.t0, x.hb,
                         [&](int h, int e) { return sh.q[s][h][tg * EPL + e]; },
                         [&](int h, float sm, float sl, const float (&o)[EPL]) {
                           fold_record<D, G, EPL>(sh.rec[s], wave, h, lane, rg, tg, sm, sl, o);
                         },
                         c2, rg, tg);
    }
  }
}

// The zoom mask of the span rows of a share, from the head bits in LDS: one
// byte per (head, row), written after the streaming so that no store sits
// between the pipelined loads.
template <int D, int G, int NS>
__device__ void plan_write_mask(const DecodeArgs& a, int nseg, PlanSmem<D, G, NS>& sh) {
  int rb = 0;
#pragma unroll 1
  for (int s = 0; s < nseg; ++s) {
    const int4 sg = sh.seg[s];
    const int x = __builtin_amdgcn_readfirstlane(sg.x), k0 = __builtin_amdgcn_readfirstlane(sg.y),
              n = __builtin_amdgcn_readfirstlane(sg.z);
    if (x < 0) continue;
    const int b = x / a.Hkv, g = x % a.Hkv;
    for (int idx = threadIdx.x; idx < G * n; idx += kThreads) {
      const int h = idx / n, k = idx % n;
      a.mask[((size_t)b * a.Hq + g * G + h) * a.m_max + k0 + k] = (sh.zb[rb + k] >> h) & 1u;
    }
    rb += n;
  }
}

template <int D, typename T, int G, bool ROUTED, bool CAPPED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(G == 1 ? 3 : 1))) void k_planned(DecodeArgs a) {
  constexpr int NS = wg_segments(G);
  __shared__ PlanSmem<D, G, NS> sh;
  // the segment descriptors, read before any store (scalar loads), kept in LDS
  int4 sgs[NS];
  const int4* segs = a.wsegs + (size_t)blockIdx.x * NS;
#pragma unroll
  for (int s = 0; s < NS; ++s) sgs[s] = segs[s];
  int nseg = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) nseg += (nseg == s && sgs[s].z > 0) ? 1 : 0;
  if (threadIdx.x == 0) {
#pragma unroll
    for (int s = 0; s < NS; ++s) sh.seg[s] = sgs[s];
  }
  if (threadIdx.x < NS * G) (&sh.zcnt[0][0])[threadIdx.x] = 0;
  // the queries of every segment's group, loaded at the start (one round trip
  // shared with the first streaming round) and written to LDS when needed: at
  // once for wide groups, which stream with the queries in LDS, and before the
  // zoom phase for narrow ones
  constexpr int QN = (NS * G * D + kThreads - 1) / kThreads;
  float qv[QN];
#pragma unroll
  for (int i = 0; i < QN; ++i) {
    const int idx = (int)threadIdx.x + i * kThreads;
    const int sidx = idx / (G * D);
    const float* src = a.q;
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      const int bg = sgs[t].x & 0x7fffffff;
      if (t == sidx) src = a.q + ((size_t)(bg / a.Hkv) * a.Hq + (bg % a.Hkv) * G) * D;
    }
    qv[i] = sidx < nseg ? src[idx % (G * D)] : 0.f;
  }
  auto fill_q = [&]() {
#pragma unroll
    for (int i = 0; i < QN; ++i) {
      const int idx = (int)threadIdx.x + i * kThreads;
      if (idx < NS * G * D) (&sh.q[0][0][0])[idx] = qv[i];
    }
  };
  if constexpr (G >= 4) fill_q();
  __syncthreads();
  // 1. span segments
  int R = 0;
#pragma unroll 1
  for (int s = 0; s < nseg; ++s) {
    const int4 v = sh.seg[s];
    const int4 sg = make_int4(__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y),
                              __builtin_amdgcn_readfirstlane(v.z), __builtin_amdgcn_readfirstlane(v.w));
    if (sg.x < 0) continue;
    plan_span_rows<D, T, G, ROUTED, CAPPED, NS>(a, sg, s, R, sh);
    R += sg.z;
  }
  // 2. anchor segments
#pragma unroll 1
  for (int s = 0; s < nseg; ++s) {
    const int4 v = sh.seg[s];
    const int4 sg = make_int4(__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y),
                              __builtin_amdgcn_readfirstlane(v.z), __builtin_amdgcn_readfirstlane(v.w));
    if (sg.x >= 0) continue;
    plan_anchor_rows<D, T, G, NS>(a, sg, s, sh);
  }
  // 3. the zoomed spans of the span rows (after the anchors: the 128K layers
  // take 33.05 against 33.4 us per layer-step, the GQA batch 294 against 302)
  if (R > 0) {
    if constexpr (G < 4) fill_q();
    __syncthreads();  // zoom bits, wave records and queries complete
    plan_zoom<D, T, G, NS>(a, nseg, R, sh);
  }
  __syncthreads();
  if (!CAPPED && R > 0) plan_write_mask<D, G, NS>(a, nseg, sh);
#pragma unroll 1
  for (int s = 0; s < nseg; ++s) {
    const int4 v = sh.seg[s];
    const int x = __builtin_amdgcn_readfirstlane(v.x), w = __builtin_amdgcn_readfirstlane(v.w);
    const int bg = x & 0x7fffffff;
    // each segment's zoom counts travel with its partials to the combine,
    // which adds them to the layer's counters (no atomics, no round trip)
    store_partial<D, G>(sh.rec[s], a, bg / a.Hkv, bg % a.Hkv, w, sh.zcnt[s]);
  }
}

// ------------------------------------------------------------------ kernels

// Span tasks of the staged path (MODE 1) and of the routing-scores pass (MODE
// 2); the grid covers the span tasks only.
template <int D, typename T, int G, int MODE, bool ROUTED>
__global__ __launch_bounds__(kThreads) void k_route(DecodeArgs a) {
  __shared__ Smem<D, G> sh;
  const int4 task = a.tasks[blockIdx.x];
  if (task.x < 0) return;
  span_task<D, T, G, MODE, ROUTED>(a, (int)blockIdx.x, task, sh);
}

// Staged bases: zoom workgroup i takes group i (span task, first item, items)
// of the fetch, into the task's second slot.
template <int D, typename T, int G>
__device__ void staged_group(const DecodeArgs& a, int i, Smem<D, G>& sh) {
  const int4 grp = a.zgroups[i];
  const int4 task = a.tasks[grp.x];
  const int4* items = a.zitems + grp.y;
  auto item = [&](int j) -> int3 {
    const int4 it = items[j];
    return make_int3((int)((uint32_t)it.x >> 24), it.z, it.w);
  };
  zoom_group<D, T, G, false>(a, task.x, task.w + 1, grp.z, item, reinterpret_cast<const T*>(a.staging), sh);
}


// Host-resident bases: workgroups [0, n_zoom_wgs) take the fetched groups;
// then one workgroup per anchor task.
template <int D, typename T, int G>
__global__ __launch_bounds__(kThreads) void k_attend(DecodeArgs a) {
  __shared__ Smem<D, G> sh;
  const int i = (int)blockIdx.x - a.n_zoom_wgs;
  if (i >= 0) {
    anchor_task<D, T, G>(a, a.tasks[a.n_span_tasks + i], sh);
    return;
  }
  staged_group<D, T, G>(a, blockIdx.x, sh);
}

// One workgroup per (sequence, query head): log-sum-exp merge of its slots in
// slot order.  Thread (group pg, float4 column c4) merges slots pg, pg + PG, ...
// with 8 in flight; the groups are merged at the end.  Also empties the flat
// zoom list for the next launch.
template <int D>
__global__ __launch_bounds__(kCombineThreads) void k_combine(DecodeArgs a) {
  constexpr int NT = kCombineThreads;
  constexpr int C4 = D / 4;
  constexpr int PG = NT / C4;
#ifndef SEKV_COMBINE_UN
#define SEKV_COMBINE_UN 8
#endif
  constexpr int UN = SEKV_COMBINE_UN;
  __shared__ float gm_s[PG], gl_s[PG], gz_s[PG];
  __shared__ float4 ga_s[PG][C4];
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, hq = bh % a.Hq;
  const int g = hq / a.G;
  // the slot count first, before any store, so that it is a scalar load
  const int np = a.parts_n[(size_t)b * a.Hkv + g];
  if (a.mask_h) {
    // the zoom mask back to host memory (the device basis cache predicts the
    // next step from it), spread over the grid; 16-byte pieces when aligned
    const int64_t tid = (int64_t)blockIdx.x * NT + threadIdx.x, nth = (int64_t)gridDim.x * NT;
    const int64_t n = a.mask_bytes;
    int64_t i0 = 0;
    if ((((uintptr_t)a.mask | (uintptr_t)a.mask_h) & 15u) == 0) {
      const int64_t n16 = n >> 4;
      for (int64_t i = tid; i < n16; i += nth)
        reinterpret_cast<uint4*>(a.mask_h)[i] = reinterpret_cast<const uint4*>(a.mask)[i];
      i0 = n16 << 4;
    }
    for (int64_t i = i0 + tid; i < n; i += nth) a.mask_h[i] = a.mask[i];
  }
  // the layer's zoom counters of this (sequence, query head), and the call
  // counter (with bh = 0): read here, with the first batch of slots, and
  // rewritten at the end; only this workgroup touches them in this launch
  unsigned long long zc0 = 0ull, calls0 = 0ull;
  if (a.zcount && threadIdx.x == 0) {
    if (a.zparts) zc0 = a.zcount[bh];
    if (bh == 0) calls0 = a.zcount[(size_t)a.B * a.Hq];
  }
  const int pg = threadIdx.x / C4, c4 = threadIdx.x % C4;
  float M = kNegInf, L = 0.f, Z = 0.f;
  float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
  const float4* pml = reinterpret_cast<const float4*>(a.part_ml) + (size_t)bh * a.max_parts;
  const float4* pa = reinterpret_cast<const float4*>(a.part_acc + (size_t)bh * a.max_parts * D) + c4;

  // the slot loads are bounded by the buffer (max_parts), not by np, so the
  // first batch is in flight together with the load of np; slots >= np are
  // loaded but never merged
  for (int p0 = pg; p0 < a.max_parts; p0 += UN * PG) {
    float4 ml[UN];
    float4 v[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int p = min(p0 + u * PG, a.max_parts - 1);
      ml[u] = pml[p];
      v[u] = pa[(size_t)p * C4];
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      if (p0 + u * PG < np) {
        const float mn = fmaxf(M, ml[u].x);
        const float ms = (mn == kNegInf) ? 0.f : mn;
        const float x = fast_exp2(M - ms), y = fast_exp2(ml[u].x - ms);
        L = L * x + ml[u].y * y;
        Z += ml[u].z;  // whole counts, exact in fp32
        A.x = A.x * x + v[u].x * y;
        A.y = A.y * x + v[u].y * y;
        A.z = A.z * x + v[u].z * y;
        A.w = A.w * x + v[u].w * y;
        M = mn;
      }
    }
    if (p0 + UN * PG >= np) break;
  }
  if (c4 == 0) {
    gm_s[pg] = M;
    gl_s[pg] = L;
    gz_s[pg] = Z;
  }
  ga_s[pg][c4] = A;
  __syncthreads();
  if (a.zcount && threadIdx.x == 0) {
    if (a.zparts) {
      float z = 0.f;
      for (int q = 0; q < PG; ++q) z += gz_s[q];
      a.zcount[bh] = zc0 + (unsigned long long)z;
    }
    if (bh == 0) a.zcount[(size_t)a.B * a.Hq] = calls0 + 1ull;
  }
  if (threadIdx.x < C4) {
    float Mg = kNegInf;
    for (int q = 0; q < PG; ++q) Mg = fmaxf(Mg, gm_s[q]);
    const float Ms = (Mg == kNegInf) ? 0.f : Mg;
    float Lg = 0.f;
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int q = 0; q < PG; ++q) {
      const float w = fast_exp2(gm_s[q] - Ms);
      Lg += gl_s[q] * w;
      const float4 u = ga_s[q][threadIdx.x];
      t.x += u.x * w;
      t.y += u.y * w;
      t.z += u.z * w;
      t.w += u.w * w;
    }
    const float inv = 1.f / Lg;
    reinterpret_cast<float4*>(a.out + (size_t)bh * D)[threadIdx.x] =
        make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
  }
  if (bh == 0 && threadIdx.x == 0 && a.zcounter) *a.zcounter = 0;
}

// ------------------------------------------------------------------ routing projection

// qp[b][h] = W_g q[b][h] (eq. (5): the query is projected into the routing
// space of eq. (3) by its kv head's projection).  One workgroup per (sequence,
// query head); wave w computes outputs w, w + 4, ... as wave-wide dot products.
template <int D>
__global__ __launch_bounds__(kThreads) void k_qproj(DecodeArgs a) {
  const int bh = blockIdx.x;
  const int g = (bh % a.Hq) / a.G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* q = a.q + (size_t)bh * D;
  const float* Wg = a.Wr + (size_t)g * a.dr * D;
  for (int j = wave; j < a.dr; j += kWaves) {
    float x = 0.f;
#pragma unroll
    for (int i = lane; i < D; i += 64) x += Wg[(size_t)j * D + i] * q[i];
    x = wave_sum(x);
    if (lane == 0) a.qp[(size_t)bh * a.dr + j] = x;
  }
}

// ------------------------------------------------------------------ budget cap

// Summary page, section 2.3 (after eq. (9)): when more spans pass a head's
// threshold than its budget k allows, the k with the highest relevance are
// kept.  The gate is monotone in the routing score, so the order is the score
// order; equal scores go to the lower span index.  One workgroup per
// (sequence, query head) takes the decisions from the scores of the routing
// pass and writes them to the zoom mask, which the route kernel then follows:
//   1. c = #{score > theta}; if c <= k every candidate is kept;
//   2. otherwise a radix select (four 8-bit digits of an order-preserving key,
//      histograms in LDS) finds the k-th largest candidate key u* and how many
//      candidates with key u* are kept (need);
//   3. a scan in span order finds the index of the need-th candidate with key
//      u*; the kept set is {key > u*} plus {key = u*, index <= that index}.
constexpr int kSelectThreads = 1024;
constexpr int kSelectWaves = kSelectThreads / 64;

// Order-preserving map of a non-NaN float to uint32 (-0 taken as +0).
__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t u = __float_as_uint(s == 0.f ? 0.f : s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the workgroup (every thread passes x); *total gets the sum.
__device__ int block_excl_scan(int x, int* red, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int sft = 1; sft < 64; sft <<= 1) {
    const int y = __shfl_up(incl, sft, 64);
    if (lane >= sft) incl += y;
  }
  if (lane == 63) red[wave] = incl;
  __syncthreads();
  int before = incl - x, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelectWaves; ++w) {
    if (w < wave) before += red[w];
    tot += red[w];
  }
  __syncthreads();  // red is reused by the next scan
  *total = tot;
  return before;
}

__global__ __launch_bounds__(kSelectThreads) void k_select(DecodeArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ int red[kSelectWaves];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need, s_cut;
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int m = a.m_b[b];
  const int k = a.budget[h];
  const double th = a.theta[h];
  const float* sc = a.scores + (size_t)bh * a.m_max;
  uint8_t* mk = a.mask + (size_t)bh * a.m_max;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  int c = 0;
  for (int i = tid; i < m; i += kSelectThreads) c += (double)sc[i] > th ? 1 : 0;
  int cand = 0;
  (void)block_excl_scan(c, red, &cand);
  if (k < 0 || cand <= k || k == 0) {
    for (int i = tid; i < m; i += kSelectThreads) mk[i] = (k != 0 && (double)sc[i] > th) ? 1 : 0;
    return;
  }
  // 2. radix select of the k-th largest candidate key, most significant digit first
  uint32_t prefix = 0u, pmask = 0u;
  int need = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    for (int i = tid; i < m; i += kSelectThreads) {
      const float s = sc[i];
      if ((double)s > th) {
        const uint32_t u = order_key(s);
        if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds digits 4l .. 4l+3; `above` counts the candidates with a larger digit
      const uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2], c3 = hist[4 * lane + 3];
      const uint32_t tot = c0 + c1 + c2 + c3;
      uint32_t suf = tot;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_down(suf, off, 64);
        if (lane + off < 64) suf += y;
      }
      const uint32_t above = suf - tot;
      const uint32_t nd0 = (uint32_t)need;
      if (above < nd0 && nd0 <= above + tot) {
        uint32_t nd = nd0 - above;
        int dg;
        if (nd <= c3) dg = 3;
        else if ((nd -= c3) <= c2) dg = 2;
        else if ((nd -= c2) <= c1) dg = 1;
        else { nd -= c1; dg = 0; }
        s_prefix = prefix | ((uint32_t)(4 * lane + dg) << shift);
        s_need = (int)nd;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    need = s_need;
    pmask |= 0xFFu << shift;
  }
  // 3. the need-th candidate with key u* = prefix in span order
  const int per = (m + kSelectThreads - 1) / kSelectThreads;
  const int i0 = min(m, tid * per), i1 = min(m, i0 + per);
  int eq = 0;
  for (int i = i0; i < i1; ++i) {
    const float s = sc[i];
    eq += ((double)s > th && order_key(s) == prefix) ? 1 : 0;
  }
  int total = 0;
  const int before = block_excl_scan(eq, red, &total);
  if (before < need && need <= before + eq) {
    int left = need - before;
    for (int i = i0; i < i1; ++i) {
      const float s = sc[i];
      if ((double)s > th && order_key(s) == prefix && --left == 0) {
        s_cut = i;
        break;
      }
    }
  }
  __syncthreads();
  const int cut = s_cut;
  for (int i = tid; i < m; i += kSelectThreads) {
    const float s = sc[i];
    bool z = false;
    if ((double)s > th) {
      const uint32_t u = order_key(s);
      z = u > prefix || (u == prefix && i <= cut);
    }
    mk[i] = z ? 1 : 0;
  }
}

template <int D, typename T, int G>
void launch_t(int which, int mode, int grid, const DecodeArgs& a, hipStream_t s) {
  if (grid <= 0) return;
  const dim3 gd(grid), bd(kThreads);
  if (which == 0 && a.dr > 0) {
    if (mode == 1) hipLaunchKernelGGL((k_route<D, T, G, 1, true>), gd, bd, 0, s, a);
    else hipLaunchKernelGGL((k_route<D, T, G, 2, true>), gd, bd, 0, s, a);
  } else if (which == 0) {
    if (mode == 1) hipLaunchKernelGGL((k_route<D, T, G, 1, false>), gd, bd, 0, s, a);
    else hipLaunchKernelGGL((k_route<D, T, G, 2, false>), gd, bd, 0, s, a);
  } else if (which == 2) {
    if (a.dr > 0) {
      if (a.capped) hipLaunchKernelGGL((k_planned<D, T, G, true, true>), gd, bd, 0, s, a);
      else hipLaunchKernelGGL((k_planned<D, T, G, true, false>), gd, bd, 0, s, a);
    } else {
      if (a.capped) hipLaunchKernelGGL((k_planned<D, T, G, false, true>), gd, bd, 0, s, a);
      else hipLaunchKernelGGL((k_planned<D, T, G, false, false>), gd, bd, 0, s, a);
    }
  } else {
    hipLaunchKernelGGL((k_attend<D, T, G>), gd, bd, 0, s, a);
  }
}

template <int D, typename T>
void launch_g(int which, int mode, int grid, const DecodeArgs& a, hipStream_t s) {
  switch (a.G) {
    case 1: launch_t<D, T, 1>(which, mode, grid, a, s); break;
    case 2: launch_t<D, T, 2>(which, mode, grid, a, s); break;
    case 4: launch_t<D, T, 4>(which, mode, grid, a, s); break;
    case 8: launch_t<D, T, 8>(which, mode, grid, a, s); break;
  }
}

}  // namespace

// This file is compiled once per (head dim, KV dtype) variant of the route and
// attend kernels (SEKV_DECODE_VARIANT 0..3) and once for everything else (no
// SEKV_DECODE_VARIANT), so that the variants build in parallel.
#if defined(SEKV_DECODE_VARIANT)
#if SEKV_DECODE_VARIANT == 0
void decode_variant_d128_bf16(int which, int mode, int grid, const DecodeArgs& a, hipStream_t s) {
  launch_g<128, bf16_t>(which, mode, grid, a, s);
}
#elif SEKV_DECODE_VARIANT == 1
void decode_variant_d128_f32(int which, int mode, int grid, const DecodeArgs& a, hipStream_t s) {
  launch_g<128, float>(which, mode, grid, a, s);
}
#elif SEKV_DECODE_VARIANT == 2
void decode_variant_d64_bf16(int which, int mode, int grid, const DecodeArgs& a, hipStream_t s) {
  launch_g<64, bf16_t>(which, mode, grid, a, s);
}
#else
void decode_variant_d64_f32(int which, int mode, int grid, const DecodeArgs& a, hipStream_t s) {
  launch_g<64, float>(which, mode, grid, a, s);
}
#endif
#else

namespace {
void launch_variant(int which, int d, int kv_bf16, int mode, int grid, const DecodeArgs& a, hipStream_t s) {
  if (d == 128) {
    if (kv_bf16) decode_variant_d128_bf16(which, mode, grid, a, s);
    else decode_variant_d128_f32(which, mode, grid, a, s);
  } else {
    if (kv_bf16) decode_variant_d64_bf16(which, mode, grid, a, s);
    else decode_variant_d64_f32(which, mode, grid, a, s);
  }
}
}  // namespace

void launch_decode_route(int mode, int grid, int d, int kv_bf16, const DecodeArgs& a, hipStream_t s) {
  launch_variant(0, d, kv_bf16, mode, grid, a, s);
}

void launch_decode_attend(int grid, int d, int kv_bf16, const DecodeArgs& a, hipStream_t s) {
  launch_variant(1, d, kv_bf16, 0, grid, a, s);
}

void launch_decode_planned(int grid, int d, int kv_bf16, const DecodeArgs& a, hipStream_t s) {
  launch_variant(2, d, kv_bf16, 0, grid, a, s);
}

void launch_decode_qproj(int d, const DecodeArgs& a, hipStream_t s) {
  if (d == 128) hipLaunchKernelGGL(k_qproj<128>, dim3(a.B * a.Hq), dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(k_qproj<64>, dim3(a.B * a.Hq), dim3(kThreads), 0, s, a);
}

void launch_decode_select(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_select, dim3(a.B * a.Hq), dim3(kSelectThreads), 0, s, a);
}

void launch_decode_combine(int d, const DecodeArgs& a, hipStream_t s) {
  if (d == 128) hipLaunchKernelGGL((k_combine<128>), dim3(a.B * a.Hq), dim3(kCombineThreads), 0, s, a);
  else hipLaunchKernelGGL((k_combine<64>), dim3(a.B * a.Hq), dim3(kCombineThreads), 0, s, a);
}

#endif  // SEKV_DECODE_VARIANT

}  // namespace sekv
