// SeKV mixed-resolution decode attention for gfx950.
//
// One decode step of one layer scores the query of every head against the
// span summaries (routing score q.kbar/(|kbar| sqrt(d)) + ln|S|, eq. (5) of the
// long-form summary page with the identity projection), zooms the spans whose
// score exceeds logit(tau) (eq. (9)), and runs ONE softmax over three kinds of
// entries (review page, workflow paragraph; summary page Figure 2):
//   anchors          q.k_a / sqrt(d), value v_a
//   non-zoomed span  q.kbar / sqrt(d) + ln|S|, value vbar
//   zoomed span      its tokens rebuilt from the truncated SVD (eq. (6)),
//                    K^ = A_K B_K^T, V^ = A_V B_V^T, scored in rank space:
//                    p = B_K^T q, logit_t = A_K[t].p / sqrt(d),
//                    c = sum_t e_t A_V[t], contribution c . B_V^T.
//
// Per layer-step (split-K over the context):
//   k_route    one workgroup per task of the runtime's table.  Anchor tasks:
//              exact tokens.  Span tasks: routing scores, zoom decisions
//              (written to the zoom mask) and the summaries of the spans each
//              head does not zoom; every span zoomed by some head of the group
//              is appended to one global list.  One partial per task.  The
//              anchor tasks run as a separate launch on a second stream,
//              concurrently with the span tasks and the zoom kernel.
//   k_zoom     one wave per listed span, balanced over all heads and
//              sequences: the span's tokens in rank space, one partial per
//              (span, zooming head).
//   k_combine  one workgroup per (sequence, query head): log-sum-exp merge of
//              its task partials and, in span order, of the partials of the
//              spans its mask row marks.
// Lanes are grouped in "row slots" of d*elem/16 lanes, each slot streaming
// whole 16-byte row pieces with its own online-softmax state (max in log2
// units, sum, d-slice of the accumulator) for the G query heads of the kv
// head.  The path is HBM-bound (about one flop per byte per query head), so
// no MFMA is used.
#include "sekv_device.h"

namespace sekv {

namespace {

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

// ------------------------------------------------------------------ zoomed span, one wave

// A raw N-element piece of T as loaded (converted to float at use, so a batch of
// pieces in flight costs N*sizeof(T)/4 registers each).
template <typename T, int N>
struct Raw;
template <>
struct Raw<bf16_t, 8> {
  uint4 v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ float get(int e) const {
    const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
};
template <>
struct Raw<bf16_t, 4> {
  uint2 v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ float get(int e) const {
    const uint32_t w = e < 2 ? v.x : v.y;
    return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
};
template <>
struct Raw<float, 4> {
  float4 v;
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ float get(int e) const { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }
};
template <>
struct Raw<float, 8> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ float get(int e) const {
    const float4& v = e < 4 ? a : b;
    const int k = e & 3;
    return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
  }
};

template <int D, typename T, int G>
struct ZoomCfg {
  static constexpr int EPL = Elem<T>::kPer16;
  static constexpr int RPW = 64 / (D / EPL);  // B rows per wave per load
  static constexpr int TPL = G >= 4 ? 4 : 8;  // tokens per lane in a token tile
  static constexpr int TILE = 64 * TPL;
  // rank components whose A pieces are in flight together: 64 registers of raw data
  static constexpr int BATCH = 64 / (TPL * (int)sizeof(T) / 4);
  // spans with r <= FAST_R and c <= TILE load everything in one round
  static constexpr int FAST_R = BATCH < 4 * RPW ? BATCH : 4 * RPW;
};

template <int G>
struct ZoomLds {
  float P[G][128];  // p = B_K^T q, pre-scaled by log2(e)/sqrt(d); zero beyond r
  float C[G][128];  // c = sum_t e_t A_V[t]
};

// One zoomed span (c tokens, rank r) of one kv head, in rank space, by one wave.
//   base: the span's packed bases A_K^T [r][c8] | B_K^T [r][D] | A_V^T [r][c8] | B_V^T [r][D]
// Lanes cover TPL consecutive tokens of a token tile for A_K^T / A_V^T (wide
// pieces of each rank component's row) and row slots for B_K^T / B_V^T.  All
// loads use clamped, always-valid addresses (no load sits behind a branch),
// and spans with r <= FAST_R, c <= TILE issue every load in one round.
// Out: per head the span's softmax max sm (log2 units) and sum sl, and the
// output c . B_V^T split over the row slots (slot j holds rows i = j mod RPW).
template <int D, typename T, int G>
__device__ void zoom_span(const T* __restrict__ base, int c, int r, const float (&qr)[G][Elem<T>::kPer16],
                          ZoomLds<G>& z, float c2, int lane, int slot, int sub, float (&sm)[G], float (&sl)[G],
                          float (&o)[G][Elem<T>::kPer16]) {
  using Cfg = ZoomCfg<D, T, G>;
  constexpr int EPL = Cfg::EPL, RPW = Cfg::RPW, LPR = D / EPL;
  constexpr int TPL = Cfg::TPL, TILE = Cfg::TILE, BATCH = Cfg::BATCH, FAST_R = Cfg::FAST_R;
  const int c8 = (c + 7) & ~7;
  const T* AKt = base;
  const T* BKt = AKt + (size_t)r * c8;
  const T* AVt = BKt + (size_t)r * D;
  const T* BVt = AVt + (size_t)r * c8;
  const int rl = r - 1;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    sm[h] = kNegInf;
    sl[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = 0.f;
  }

  if (r <= FAST_R && c <= TILE) {
    // ---------------- one round: every piece of the span in flight together
    const int tb = lane * TPL;
    const bool act = tb < c;
    const int tbl = act ? tb : 0;
    Raw<T, EPL> fb[4], fw[4];
    Raw<T, TPL> fa[FAST_R], fv[FAST_R];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = min(u * RPW + slot, rl);
      fb[u].load(BKt + (size_t)i * D + sub * EPL);
      fw[u].load(BVt + (size_t)i * D + sub * EPL);
    }
#pragma unroll
    for (int u = 0; u < FAST_R; ++u) {
      const int i = min(u, rl);
      fa[u].load(AKt + (size_t)i * c8 + tbl);
      fv[u].load(AVt + (size_t)i * c8 + tbl);
    }
    // p (zero beyond r)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float dp = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dp += qr[h][e] * fb[u].get(e);
        dp = group_sum<LPR>(dp);
        const int i = u * RPW + slot;
        if (sub == 0 && i < FAST_R) z.P[h][i] = i < r ? dp * c2 : 0.f;
      }
    wave_lds_sync();
    float ew[G][TPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float lg[TPL];
#pragma unroll
      for (int e = 0; e < TPL; ++e) lg[e] = 0.f;
#pragma unroll
      for (int u = 0; u < FAST_R; ++u) {
        const float pv = z.P[h][u];
#pragma unroll
        for (int e = 0; e < TPL; ++e) lg[e] += fa[u].get(e) * pv;
      }
      float mx = kNegInf;
#pragma unroll
      for (int e = 0; e < TPL; ++e) {
        if (tb + e >= c) lg[e] = kNegInf;
        mx = fmaxf(mx, lg[e]);
      }
      mx = wave_max(mx);
      float ssum = 0.f;
#pragma unroll
      for (int e = 0; e < TPL; ++e) {
        ew[h][e] = fast_exp2(lg[e] - mx);
        ssum += ew[h][e];
      }
      sm[h] = mx;
      sl[h] = wave_sum(ssum);
    }
    // c[i] = sum_t e_t A_V^T[i][t]
#pragma unroll
    for (int u = 0; u < FAST_R; ++u)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float x = 0.f;
#pragma unroll
        for (int e = 0; e < TPL; ++e) x += ew[h][e] * fv[u].get(e);
        x = wave_sum(x);
        if (lane == 0) z.C[h][u] = x;
      }
    wave_lds_sync();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = u * RPW + slot;
      if (i < r) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float cv = z.C[h][i];
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[h][e] += cv * fw[u].get(e);
        }
      }
    }
    wave_lds_sync();  // P and C are rewritten by the next span
    return;
  }

  // ---------------- general spans: rank in batches, tokens in tiles
  for (int j0 = 0; j0 < r; j0 += 4 * RPW) {
    Raw<T, EPL> fb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) fb[u].load(BKt + (size_t)min(j0 + u * RPW + slot, rl) * D + sub * EPL);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float dp = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dp += qr[h][e] * fb[u].get(e);
        dp = group_sum<LPR>(dp);
        const int i = j0 + u * RPW + slot;
        if (sub == 0 && i < r) z.P[h][i] = dp * c2;
      }
  }
  const int rpad = (r + BATCH - 1) / BATCH * BATCH;
  for (int i = r + lane; i < rpad; i += 64)
#pragma unroll
    for (int h = 0; h < G; ++h) z.P[h][i] = 0.f;
  wave_lds_sync();
  for (int t0 = 0; t0 < c; t0 += TILE) {
    const int tb = t0 + lane * TPL;
    const bool act = tb < c;
    const int tbl = act ? tb : t0;
    float lg[G][TPL];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < TPL; ++e) lg[h][e] = 0.f;
    for (int i0 = 0; i0 < r; i0 += BATCH) {
      Raw<T, TPL> fa[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) fa[u].load(AKt + (size_t)min(i0 + u, rl) * c8 + tbl);
#pragma unroll
      for (int u = 0; u < BATCH; ++u)
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float pv = z.P[h][i0 + u];
#pragma unroll
          for (int e = 0; e < TPL; ++e) lg[h][e] += fa[u].get(e) * pv;
        }
    }
    float ew[G][TPL], sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = kNegInf;
#pragma unroll
      for (int e = 0; e < TPL; ++e) {
        if (tb + e >= c) lg[h][e] = kNegInf;
        mx = fmaxf(mx, lg[h][e]);
      }
      mx = wave_max(mx);
      const float mn = fmaxf(sm[h], mx);  // finite: the tile holds a token
      sc[h] = fast_exp2(sm[h] - mn);
      float ssum = 0.f;
#pragma unroll
      for (int e = 0; e < TPL; ++e) {
        ew[h][e] = fast_exp2(lg[h][e] - mn);
        ssum += ew[h][e];
      }
      sl[h] = sl[h] * sc[h] + wave_sum(ssum);
      sm[h] = mn;
    }
    for (int i0 = 0; i0 < r; i0 += BATCH) {
      Raw<T, TPL> fv[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) fv[u].load(AVt + (size_t)min(i0 + u, rl) * c8 + tbl);
#pragma unroll
      for (int u = 0; u < BATCH; ++u)
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float x = 0.f;
#pragma unroll
          for (int e = 0; e < TPL; ++e) x += ew[h][e] * fv[u].get(e);
          x = wave_sum(x);
          const int i = i0 + u;
          if (lane == 0 && i < r) z.C[h][i] = (t0 == 0 ? 0.f : z.C[h][i] * sc[h]) + x;
        }
    }
  }
  wave_lds_sync();
  for (int j0 = 0; j0 < r; j0 += 4 * RPW) {
    Raw<T, EPL> fw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) fw[u].load(BVt + (size_t)min(j0 + u * RPW + slot, rl) * D + sub * EPL);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = j0 + u * RPW + slot;
      if (i < r) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float cv = z.C[h][i];
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[h][e] += cv * fw[u].get(e);
        }
      }
    }
  }
  wave_lds_sync();  // P and C are rewritten by the next span
}

// ------------------------------------------------------------------ workgroup merge

template <int D, int G>
struct MergeLds {
  float m[kWaves][G];
  float l[kWaves][G];
  float acc[kWaves][G][D];
};

// Butterfly over the row slots of each wave, then one record per wave in LDS.
template <int D, int G, int EPL, int LPR>
__device__ void slots_to_lds(SoftState<G>& st, float (&acc)[G][EPL], MergeLds<D, G>& ml, int lane,
                             int wave, int slot, int sub) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    for (int off = LPR; off < 64; off <<= 1) {
      const float mo = __shfl_xor(st.m[h], off, 64);
      const float lo = __shfl_xor(st.l[h], off, 64);
      float ao[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) ao[e] = __shfl_xor(acc[h][e], off, 64);
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

// Merge the per-wave records into one partial per head and store it.
template <int D, int G>
__device__ void store_partial(const MergeLds<D, G>& ml, const DecodeArgs& a, int b, int g, int part) {
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
    const int hq = g * G + h;
    const size_t slot = ((size_t)b * a.Hq + hq) * a.max_parts + part;
    a.part_acc[slot * D + j] = A;
    if (j == 0) reinterpret_cast<float2*>(a.part_ml)[slot] = make_float2(M, L);
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

// ------------------------------------------------------------------ k_route

// One pipeline stage of a row slot: U rows of keys (or summaries) and values.
template <typename T, int U>
struct Stage {
  Raw<T, Elem<T>::kPer16> k[U], v[U];
  float ls[U];
  int2 meta[U];  // span rows: packed {basis offset / 8, rank | count << 8}
};

// SCORES: routing scores only.  Otherwise zoomed spans are appended to the
// global list for the zoom kernel.  Workgroup i runs task task_base + i.
template <int D, typename T, int G, bool SCORES>
__global__ __launch_bounds__(kThreads) void k_route(DecodeArgs a, int task_base) {
  constexpr int EPL = Elem<T>::kPer16;  // elements per 16-byte load
  constexpr int LPR = D / EPL;          // lanes per row
  constexpr int RPW = 64 / LPR;         // rows per wave per load
  constexpr int U = 4;                  // rows per lane slot per stage
  constexpr int STEP = kWaves * RPW * U;

  __shared__ MergeLds<D, G> ml_s;
  __shared__ int4 list_s[1024];  // (bg | head bits << 24, span, packed basis offset, rank | count << 8)
  __shared__ int list_n, s_base;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane / LPR, sub = lane % LPR;
  // rows of the grid in the host's order (most zoom-prone kv heads first);
  // span chunks come before anchor chunks in each row
  // one task per workgroup, in the runtime's order (the busiest first)
  const int4 task = a.tasks[task_base + blockIdx.x];
  const int bg = task.x & 0x7fffffff;
  const bool is_anchor_chunk = task.x < 0;
  const int t_start = task.y, t_count = task.z, part = task.w;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  if (SCORES && is_anchor_chunk) return;
  if (threadIdx.x == 0) list_n = 0;
  const float c2 = kLog2e * rsqrtf((float)D);  // logit scale in log2 units
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
  // fold U rows with logits lg[h][u] (log2 units, -inf = skip) and values vf into the state
  auto fold = [&](const float (&lg)[G][U], const Raw<T, EPL>(&vf)[U]) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = st.m[h];
#pragma unroll
      for (int u = 0; u < U; ++u) mx = fmaxf(mx, lg[h][u]);
      const float ms = (mx == kNegInf) ? 0.f : mx;
      const float sc = fast_exp2(st.m[h] - ms);
      float ls = st.l[h] * sc;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= sc;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = fast_exp2(lg[h][u] - ms);
        ls += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] += p * vf[u].get(e);
      }
      st.l[h] = ls;
      st.m[h] = mx;
    }
  };

  if (is_anchor_chunk) {
    // ---------------- anchor segment: exact tokens, two stages in flight
    const int na = a.na_b[b];
    const int r0 = t_start;
    const int r1 = min(na, r0 + t_count);
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
    float qr[G][EPL];
    auto consume = [&](const Stage<T, U>& sg, int bs) {
      float lg[G][U];
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float dp = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) dp += qr[h][e] * sg.k[u].get(e);
          dp = group_sum<LPR>(dp);
          lg[h][u] = (bs + u * RPW + slot < r1) ? dp * c2 : kNegInf;
        }
      fold(lg, sg.v);
    };
    int bs = r0 + wave * RPW * U;
    if (bs < r1) {
      Stage<T, U> A, B;
      load(A, bs);
      load_q<D, G, T>(a, b, g, sub, qr);
      for (; bs < r1; bs += 2 * STEP) {
        load(B, bs + STEP);
        consume(A, bs);
        if (bs + STEP >= r1) break;
        load(A, bs + 2 * STEP);
        consume(B, bs + STEP);
      }
    }
    slots_to_lds<D, G, EPL, LPR>(st, acc, ml_s, lane, wave, slot, sub);
    __syncthreads();
    store_partial<D, G>(ml_s, a, b, g, part);
    return;
  }

  // ---------------- span chunk: routing, zoom decisions, summaries of non-zoomed spans
  const int m = a.m_b[b];
  const int k0 = t_start;
  const int k1 = min(m, k0 + t_count);
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
      if (!SCORES) sg.meta[u] = a.smeta[(size_t)bg * a.m_max + kk];
    }
  };
  float qr[G][EPL];
  auto consume = [&](const Stage<T, U>& sg, int bs) {
    float nrm[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float s2 = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) s2 += sg.k[u].get(e) * sg.k[u].get(e);
      nrm[u] = group_sum<LPR>(s2);
    }
    float lg[G][U];
    uint32_t zbits[U];
#pragma unroll
    for (int u = 0; u < U; ++u) zbits[u] = 0u;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float dp = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dp += qr[h][e] * sg.k[u].get(e);
        dp = group_sum<LPR>(dp);
        const float score = (nrm[u] > 0.f ? dp * rsqrtf(nrm[u]) * inv_sqrt_d : 0.f) + sg.ls[u];
        const int k = bs + u * RPW + slot;
        const bool ok = k < k1;
        const bool zoom = (double)score > a.theta[g * G + h];
        if (ok && sub == 0) {
          const size_t mi = ((size_t)b * a.Hq + g * G + h) * a.m_max + k;
          if (SCORES) a.scores[mi] = score;
          else a.mask[mi] = zoom ? 1 : 0;
        }
        if (zoom) zbits[u] |= 1u << h;
        lg[h][u] = (ok && !zoom) ? dp * c2 + sg.ls[u] * kLog2e : kNegInf;
      }
    if (SCORES) return;
    fold(lg, sg.v);
    if (sub == 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = bs + u * RPW + slot;
        if (k < k1 && zbits[u]) {
          const int pos = atomicAdd(&list_n, 1);
          list_s[pos] = make_int4(bg | (int)(zbits[u] << 24), k, sg.meta[u].x, sg.meta[u].y);
        }
      }
    }
  };
  __syncthreads();  // list_n
  int bs = k0 + wave * RPW * U;
  if (bs < k1) {
    Stage<T, U> A, B;
    load(A, bs);
    load_q<D, G, T>(a, b, g, sub, qr);
    for (; bs < k1; bs += 2 * STEP) {
      load(B, bs + STEP);
      consume(A, bs);
      if (bs + STEP >= k1) break;
      load(A, bs + 2 * STEP);
      consume(B, bs + STEP);
    }
  }
  if (SCORES) return;
  slots_to_lds<D, G, EPL, LPR>(st, acc, ml_s, lane, wave, slot, sub);
  __syncthreads();  // list_s and the records complete
  if (threadIdx.x == 0) {
    s_base = list_n ? atomicAdd(a.zcounter, list_n) : 0;
    if (list_n) atomicAdd(&a.zstat[bg], list_n);
  }
  store_partial<D, G>(ml_s, a, b, g, part);
  __syncthreads();
  for (int i = threadIdx.x; i < list_n; i += kThreads) a.zlist[s_base + i] = list_s[i];
}

// ------------------------------------------------------------------ k_zoom

// One wave per listed span, over the whole grid.  STAGED: bases in the staging
// buffer at zoff[i] (HOST home); otherwise in the device store at boff.
template <int D, typename T, int G, bool STAGED>
__global__ __launch_bounds__(kThreads) void k_zoom(DecodeArgs a) {
  constexpr int EPL = Elem<T>::kPer16;
  constexpr int LPR = D / EPL;
  __shared__ ZoomLds<G> zl_s[kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane / LPR, sub = lane % LPR;
  const float c2 = kLog2e * rsqrtf((float)D);
  const int total = *a.zn;
  const int stride = gridDim.x * kWaves;
  int i = blockIdx.x * kWaves + wave;
  if (i >= total) return;
  const T* src = reinterpret_cast<const T*>(STAGED ? a.staging : a.bases);
  int4 ent = a.zitems[i];
  while (true) {
    const int inext = i + stride;
    const int4 ent_next = a.zitems[inext < total ? inext : i];  // prefetch
    const int bg = ent.x & 0xffffff;
    const uint32_t hb = (uint32_t)ent.x >> 24;
    const int k = ent.y;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const size_t ti = (size_t)bg * a.m_max + k;
    const int64_t off = STAGED ? a.zoff[i] : (int64_t)(uint32_t)ent.z << 3;
    const int r = ent.w & 0xff;
    const int cnt = (int)((uint32_t)ent.w >> 8);
    float qr[G][EPL];
    load_q<D, G, T>(a, b, g, sub, qr);
    float sm[G], sl[G], o[G][EPL];
    zoom_span<D, T, G>(src + off, cnt, r, qr, zl_s[wave], c2, lane, slot, sub, sm, sl, o);
    // add up the slots' output parts (they share the span's max)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      for (int sh = LPR; sh < 64; sh <<= 1) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[h][e] += __shfl_xor(o[h][e], sh, 64);
      }
      if (hb & (1u << h)) {
        const size_t zi = ti * G + h;
        if (slot == 0) {
#pragma unroll
          for (int e = 0; e < EPL; e += 4) Elem<float>::store16(a.zpart_acc + zi * D + sub * EPL + e, o[h] + e);
        }
        if (lane == 0) reinterpret_cast<float2*>(a.zpart_ml)[zi] = make_float2(sm[h], sl[h]);
      }
    }
    if (inext >= total) break;
    i = inext;
    ent = ent_next;
  }
}

// ------------------------------------------------------------------ k_combine

// One workgroup per (sequence, query head): merges its partials and the
// partials of the zoomed spans its mask row marks, in span order, so the result
// does not depend on the order of the zoom list.  Each thread (group pg, float4
// column c4) keeps an online log-sum-exp over its share of the entries; the
// groups are merged at the end.
template <int D>
__global__ __launch_bounds__(kCombineThreads) void k_combine(DecodeArgs a) {
  constexpr int NT = kCombineThreads;
  constexpr int NW = NT / 64;
  constexpr int C4 = D / 4;     // float4 columns of a partial accumulator
  constexpr int PG = NT / C4;   // entry groups
  constexpr int SPT = 4;        // mask bytes scanned per thread per round
  constexpr int ROUND = SPT * NT;
  __shared__ int zid_s[ROUND];
  __shared__ int cnt_s[NW];
  __shared__ float gm_s[PG], gl_s[PG];
  __shared__ float4 ga_s[PG][C4];
  const int bh = blockIdx.x;  // b * Hq + hq
  const int b = bh / a.Hq, hq = bh % a.Hq;
  const int g = hq / a.G, h = hq % a.G;
  const size_t bg = (size_t)b * a.Hkv + g;
  const int np = a.parts_n[bg], m = a.m_b[b];
  const uint8_t* mrow = a.mask + (size_t)bh * a.m_max;
  const float2* zml = reinterpret_cast<const float2*>(a.zpart_ml);
  const int pg = threadIdx.x / C4, c4 = threadIdx.x % C4;

  float M = kNegInf, L = 0.f;
  float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
  auto merge = [&](float mo, float lo, float4 v) {
    const float mn = fmaxf(M, mo);
    const float ms = (mn == kNegInf) ? 0.f : mn;
    const float x = fast_exp2(M - ms), y = fast_exp2(mo - ms);
    L = L * x + lo * y;
    A.x = A.x * x + v.x * y;
    A.y = A.y * x + v.y * y;
    A.z = A.z * x + v.z * y;
    A.w = A.w * x + v.w * y;
    M = mn;
  };
  // stream partials, 8 entries in flight per thread
  const float2* pml = reinterpret_cast<const float2*>(a.part_ml) + (size_t)bh * a.max_parts;
  const float4* pa = reinterpret_cast<const float4*>(a.part_acc + (size_t)bh * a.max_parts * D) + c4;
  for (int p0 = pg; p0 < np; p0 += 8 * PG) {
    float2 ml[8];
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = min(p0 + u * PG, np - 1);
      ml[u] = pml[p];
      v[u] = pa[(size_t)p * C4];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (p0 + u * PG < np) merge(ml[u].x, ml[u].y, v[u]);
  }
  // zoomed spans, in span order (HOST home: their partials come from the zoom kernel)
  for (int k0 = 0; a.zpart_ml && k0 < m; k0 += ROUND) {
    uint8_t mb[SPT];
    int n = 0;
    const int kb = k0 + threadIdx.x * SPT;
#pragma unroll
    for (int e = 0; e < SPT; ++e) {
      mb[e] = (kb + e < m) ? mrow[kb + e] : 0;
      n += mb[e] ? 1 : 0;
    }
    // exclusive prefix of n over the workgroup: shuffle scan in each wave, then wave offsets
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = n;
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const int y = __shfl_up(incl, sh, 64);
      if (lane >= sh) incl += y;
    }
    if (lane == 63) cnt_s[wave] = incl;
    __syncthreads();
    int pos = incl - n;
    for (int w = 0; w < wave; ++w) pos += cnt_s[w];
    int nz = 0;
    for (int w = 0; w < NW; ++w) nz += cnt_s[w];
#pragma unroll
    for (int e = 0; e < SPT; ++e)
      if (mb[e]) zid_s[pos++] = kb + e;
    __syncthreads();
    for (int j0 = pg; j0 < nz; j0 += 8 * PG) {
      float2 ml[8];
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const size_t zi = (bg * a.m_max + zid_s[min(j0 + u * PG, nz - 1)]) * a.G + h;
        ml[u] = zml[zi];
        v[u] = reinterpret_cast<const float4*>(a.zpart_acc + zi * D)[c4];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (j0 + u * PG < nz) merge(ml[u].x, ml[u].y, v[u]);
    }
    __syncthreads();
  }
  // merge the groups
  if (c4 == 0) {
    gm_s[pg] = M;
    gl_s[pg] = L;
  }
  ga_s[pg][c4] = A;
  __syncthreads();
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
  if (bh == 0 && threadIdx.x == 0 && a.zcounter) *a.zcounter = 0;  // the zoom list is empty again
}

template <int D, typename T, int G>
void launch_route_t(bool scores, int t0, int t1, const DecodeArgs& a, hipStream_t s) {
  if (t1 <= t0) return;
  dim3 grid(t1 - t0);
  if (scores) hipLaunchKernelGGL((k_route<D, T, G, true>), grid, dim3(kThreads), 0, s, a, t0);
  else hipLaunchKernelGGL((k_route<D, T, G, false>), grid, dim3(kThreads), 0, s, a, t0);
}

template <int D, typename T, int G>
void launch_zoom_t(bool staged, const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.n_zoom_wgs);
  if (staged) hipLaunchKernelGGL((k_zoom<D, T, G, true>), grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL((k_zoom<D, T, G, false>), grid, dim3(kThreads), 0, s, a);
}

template <int D, typename T>
void launch_g(int which, int flag, int t0, int t1, const DecodeArgs& a, hipStream_t s) {
  switch (a.G) {
#define SEKV_CASE(GG)                                                    \
  case GG:                                                               \
    if (which == 0) launch_route_t<D, T, GG>(flag != 0, t0, t1, a, s);   \
    else launch_zoom_t<D, T, GG>(flag != 0, a, s);                       \
    break;
    SEKV_CASE(1)
    SEKV_CASE(2)
    SEKV_CASE(4)
    SEKV_CASE(8)
#undef SEKV_CASE
  }
}

template <int D>
void launch_d(int which, int kv_bf16, int flag, int t0, int t1, const DecodeArgs& a, hipStream_t s) {
  if (kv_bf16) launch_g<D, bf16_t>(which, flag, t0, t1, a, s);
  else launch_g<D, float>(which, flag, t0, t1, a, s);
}

}  // namespace

void launch_decode_route(bool scores_only, int t0, int t1, int d, int kv_bf16, const DecodeArgs& a,
                         hipStream_t s) {
  if (d == 128) launch_d<128>(0, kv_bf16, scores_only, t0, t1, a, s);
  else launch_d<64>(0, kv_bf16, scores_only, t0, t1, a, s);
}

void launch_decode_zoom(bool staged, int d, int kv_bf16, const DecodeArgs& a, hipStream_t s) {
  if (d == 128) launch_d<128>(1, kv_bf16, staged, 0, 0, a, s);
  else launch_d<64>(1, kv_bf16, staged, 0, 0, a, s);
}

void launch_decode_combine(int d, const DecodeArgs& a, hipStream_t s) {
  if (d == 128) hipLaunchKernelGGL((k_combine<128>), dim3(a.B * a.Hq), dim3(kCombineThreads), 0, s, a);
  else hipLaunchKernelGGL((k_combine<64>), dim3(a.B * a.Hq), dim3(kCombineThreads), 0, s, a);
}

}  // namespace sekv
