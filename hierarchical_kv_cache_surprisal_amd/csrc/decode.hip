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
// Work decomposition (split-K over the context): grid.y = (sequence, kv head),
// grid.x = chunks of anchor rows and chunks of spans.  Each workgroup keeps an
// online-softmax state (max in log2 units, sum, acc[d]) for the G query heads
// of its kv head, writes it as a partial, and the last workgroup of its
// (sequence, kv head) to arrive merges all partials (log-sum-exp) into the
// output.  Everything streams bf16/f32 rows with 16-byte loads; the kernel is
// HBM-bound, so no MFMA is used.
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
  float mn = fmaxf(m, mo);
  float ms = (mn == kNegInf) ? 0.f : mn;
  float a = fast_exp2(m - ms), b = fast_exp2(mo - ms);
  l = l * a + lo * b;
#pragma unroll
  for (int e = 0; e < N; ++e) acc[e] = acc[e] * a + acco[e] * b;
  m = mn;
}

// ------------------------------------------------------------------ zoomed span, one wave

// Per-wave LDS scratch of the zoom routine.
template <int G>
struct ZoomLds {
  float P[G][128];  // p = B_K^T q, pre-scaled by log2(e)/sqrt(d)
  float E[G][64];   // exp weights of the current token tile
  float C[G][128];  // c = sum_t e_t A_V[t]
};

// dot(A_K row, P[h]) for every head; r elements of type T starting at row.
template <typename T, int G>
__device__ __forceinline__ void row_dot_p(const T* __restrict__ row, int r, const ZoomLds<G>& z,
                                          float (&acc)[G]) {
  constexpr int V = Elem<T>::kPer16;
  int i = 0;
  if ((r % V) == 0) {
    for (; i < r; i += V) {
      float f[V];
      Elem<T>::load16(row + i, f);
#pragma unroll
      for (int e = 0; e < V; ++e)
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] += f[e] * z.P[h][i + e];
    }
    return;
  }
  for (; i < r; ++i) {
    float f = Elem<T>::to_f(row[i]);
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] += f * z.P[h][i];
  }
}

// Accumulate one zoomed span into the wave's zoom state (zm, zl, zacc) for the
// heads in hbits.  base points at the span's packed bases [A_K | B_K^T | A_V | B_V^T].
// zacc holds d/64 output elements per lane: element lane*JPL + j.
template <int D, typename T, int G>
__device__ void zoom_span(const T* __restrict__ base, int c, int r, uint32_t hbits,
                          const float (*q_s)[D], ZoomLds<G>& z, float c2, int lane,
                          float (&zm)[G], float (&zl)[G], float (&zacc)[G][D / 64]) {
  constexpr int JPL = D / 64;
  constexpr int V = Elem<T>::kPer16;
  const T* AK = base;
  const T* BKt = AK + pad8((int64_t)c * r);
  const T* AV = BKt + pad8((int64_t)r * D);
  const T* BVt = AV + pad8((int64_t)c * r);

  // 1. P[h][i] = c2 * sum_j B_K^T[i][j] q_h[j]   (one lane per rank component)
  for (int i = lane; i < r; i += 64) {
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.f;
    const T* row = BKt + (int64_t)i * D;
#pragma unroll 4
    for (int j0 = 0; j0 < D; j0 += V) {
      float f[V];
      Elem<T>::load16(row + j0, f);
#pragma unroll
      for (int e = 0; e < V; ++e)
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] += f[e] * q_s[h][j0 + e];
    }
#pragma unroll
    for (int h = 0; h < G; ++h) z.P[h][i] = acc[h] * c2;
  }
  wave_lds_sync();

  // lane mapping for the A_V accumulation: component il (+64), token slice s
  int RL = 64;
  if (r <= 32) RL = 32;
  if (r <= 16) RL = 16;
  if (r <= 8) RL = 8;
  if (r <= 4) RL = 4;
  if (r <= 2) RL = 2;
  if (r <= 1) RL = 1;
  const int SL = 64 / RL;
  const int il = lane % RL, sl = lane / RL;

  float sm[G], sls[G], cacc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    sm[h] = kNegInf;
    sls[h] = 0.f;
    cacc[h][0] = cacc[h][1] = 0.f;
  }

  for (int t0 = 0; t0 < c; t0 += 64) {
    const int t = t0 + lane;
    const bool valid = t < c;
    float lg[G];
#pragma unroll
    for (int h = 0; h < G; ++h) lg[h] = 0.f;
    if (valid) row_dot_p<T, G>(AK + (int64_t)t * r, r, z, lg);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float x = valid ? lg[h] : kNegInf;
      float tm = wave_max(x);
      float mn = fmaxf(sm[h], tm);
      float ms = (mn == kNegInf) ? 0.f : mn;
      float sc = fast_exp2(sm[h] - ms);
      float e = valid ? fast_exp2(x - ms) : 0.f;
      sls[h] = sls[h] * sc + wave_sum(e);
      sm[h] = mn;
      cacc[h][0] *= sc;
      cacc[h][1] *= sc;
      z.E[h][lane] = e;
    }
    wave_lds_sync();
    const int tl = min(64, c - t0);
    for (int tt = sl; tt < tl; tt += SL) {
      const T* row = AV + (int64_t)(t0 + tt) * r;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int i = il + 64 * jj;
        if (i < r) {
          float a = Elem<T>::to_f(row[i]);
#pragma unroll
          for (int h = 0; h < G; ++h) cacc[h][jj] += z.E[h][tt] * a;
        }
      }
    }
    wave_lds_sync();
  }
  // reduce the token slices, publish c
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      float x = cacc[h][jj];
      for (int off = RL; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
      cacc[h][jj] = x;
    }
  if (sl == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (il < r) z.C[h][il] = cacc[h][0];
      if (il + 64 < r) z.C[h][il + 64] = cacc[h][1];
    }
  }
  wave_lds_sync();
  // out_h[j] = sum_i c_h[i] B_V^T[i][j]
  float o[G][JPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int j = 0; j < JPL; ++j) o[h][j] = 0.f;
  for (int i = 0; i < r; ++i) {
    const T* row = BVt + (int64_t)i * D + lane * JPL;
#pragma unroll
    for (int j = 0; j < JPL; ++j) {
      float b = Elem<T>::to_f(row[j]);
#pragma unroll
      for (int h = 0; h < G; ++h) o[h][j] += z.C[h][i] * b;
    }
  }
  wave_lds_sync();  // P/E/C are reused by the next span
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (hbits & (1u << h)) lse_merge<JPL>(zm[h], zl[h], zacc[h], sm[h], sls[h], o[h]);
  }
}

// ------------------------------------------------------------------ workgroup merge and combine

template <int D, int G>
struct MergeLds {
  float m[2 * kWaves][G];
  float l[2 * kWaves][G];
  float acc[2 * kWaves][G][D];
};

// Merge the 2*kWaves records in LDS into one partial per head and store it.
template <int D, int G>
__device__ void store_partial(const MergeLds<D, G>& ml, int nrec, const DecodeArgs& a, int b, int g,
                              int part) {
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, j = idx % D;
    float M = kNegInf;
    for (int r = 0; r < nrec; ++r) M = fmaxf(M, ml.m[r][h]);
    const float Ms = (M == kNegInf) ? 0.f : M;
    float L = 0.f, A = 0.f;
    for (int r = 0; r < nrec; ++r) {
      const float w = fast_exp2(ml.m[r][h] - Ms);
      L += ml.l[r][h] * w;
      A += ml.acc[r][h][j] * w;
    }
    const int hq = g * G + h;
    const size_t slot = ((size_t)b * a.Hq + hq) * a.n_parts + part;
    a.part_acc[slot * D + j] = A;
    if (j == 0) {
      a.part_ml[slot * 2 + 0] = M;
      a.part_ml[slot * 2 + 1] = L;
    }
  }
}

// Arrival ticket: the last of `total` workgroups of (b, g) merges every
// partial slot into the output.  Partials of other workgroups are made
// visible by the agent-scope fences (L2s of different XCDs are not coherent).
template <int D, int G>
__device__ void ticket_and_combine(const DecodeArgs& a, int b, int g, int total) {
  __shared__ uint32_t s_ticket;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_ticket = atomicAdd(&a.counters[b * a.Hkv + g], 1u);
  __syncthreads();
  if (s_ticket != (uint32_t)(total - 1)) return;
  __threadfence();
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, j = idx % D;
    const int hq = g * G + h;
    const size_t s0 = ((size_t)b * a.Hq + hq) * a.n_parts;
    float M = kNegInf;
    for (int p = 0; p < a.n_parts; ++p) M = fmaxf(M, __builtin_nontemporal_load(&a.part_ml[(s0 + p) * 2]));
    const float Ms = (M == kNegInf) ? 0.f : M;
    float L = 0.f, A = 0.f;
    for (int p = 0; p < a.n_parts; ++p) {
      const float w = fast_exp2(__builtin_nontemporal_load(&a.part_ml[(s0 + p) * 2]) - Ms);
      L += __builtin_nontemporal_load(&a.part_ml[(s0 + p) * 2 + 1]) * w;
      A += __builtin_nontemporal_load(&a.part_acc[(s0 + p) * D + j]) * w;
    }
    a.out[((size_t)b * a.Hq + hq) * D + j] = A / L;
  }
  if (threadIdx.x == 0) a.counters[b * a.Hkv + g] = 0u;
}

// ------------------------------------------------------------------ main kernel

template <int D, typename T, int G, int MODE>
__global__ __launch_bounds__(kThreads) void k_decode_main(DecodeArgs a) {
  constexpr int EPL = Elem<T>::kPer16;  // elements per 16-byte load
  constexpr int LPR = D / EPL;          // lanes per row
  constexpr int RPW = 64 / LPR;         // rows per wave per load
  constexpr int U = 2;                  // rows in flight per lane slot
  constexpr int JPL = D / 64;

  __shared__ float q_s[G][D];
  __shared__ ZoomLds<G> zl_s[MODE == 0 ? kWaves : 1];
  __shared__ MergeLds<D, G> ml_s;
  __shared__ int32_t list_s[1024];
  __shared__ int list_n;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane / LPR, sub = lane % LPR;
  const int bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int chunk = blockIdx.x;
  const bool is_anchor_chunk = chunk < a.n_anchor_chunks;
  if (MODE == 2 && is_anchor_chunk) return;

  for (int i = threadIdx.x; i < G * D; i += kThreads)
    q_s[i / D][i % D] = a.q[((size_t)b * a.Hq + g * G + i / D) * D + i % D];
  if (threadIdx.x == 0) list_n = 0;
  __syncthreads();

  const float c2 = kLog2e * rsqrtf((float)D);   // logit scale in log2 units
  const float inv_sqrt_d = rsqrtf((float)D);
  float qr[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) qr[h][e] = q_s[h][sub * EPL + e];

  SoftState<G> st;
  float acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = kNegInf;
    st.l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  if (is_anchor_chunk) {
    // ---------------- anchor segment: exact tokens
    const int na = a.na_b[b];
    const int r0 = chunk * a.anchor_chunk;
    const int r1 = min(na, r0 + a.anchor_chunk);
    const T* Kb = reinterpret_cast<const T*>(a.KA) + (size_t)bg * a.na_max * D + sub * EPL;
    const T* Vb = reinterpret_cast<const T*>(a.VA) + (size_t)bg * a.na_max * D + sub * EPL;
    for (int base = r0 + wave * RPW * U; base < r1; base += kWaves * RPW * U) {
      float kf[U][EPL], vf[U][EPL];
      bool ok[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int row = base + u * RPW + slot;
        ok[u] = row < r1;
        const int rr = ok[u] ? row : r0;
        Elem<T>::load16(Kb + (size_t)rr * D, kf[u]);
        Elem<T>::load16(Vb + (size_t)rr * D, vf[u]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float lg[U];
        float mx = st.m[h];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float dp = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) dp += qr[h][e] * kf[u][e];
          dp = group_sum<LPR>(dp);
          lg[u] = ok[u] ? dp * c2 : kNegInf;
          mx = fmaxf(mx, lg[u]);
        }
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
          for (int e = 0; e < EPL; ++e) acc[h][e] += p * vf[u][e];
        }
        st.l[h] = ls;
        st.m[h] = mx;
      }
    }
  } else {
    // ---------------- span chunk: routing, summaries of non-zoomed spans
    const int m = a.m_b[b];
    const int k0 = (chunk - a.n_anchor_chunks) * a.span_chunk;
    const int k1 = min(m, k0 + a.span_chunk);
    const T* Kb = reinterpret_cast<const T*>(a.kbar) + (size_t)bg * a.m_max * D + sub * EPL;
    const T* Vb = reinterpret_cast<const T*>(a.vbar) + (size_t)bg * a.m_max * D + sub * EPL;
    const float* lS = a.logS + (size_t)b * a.m_max;
    for (int base = k0 + wave * RPW * U; base < k1; base += kWaves * RPW * U) {
      float kf[U][EPL], vf[U][EPL], ls_k[U];
      bool ok[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = base + u * RPW + slot;
        ok[u] = k < k1;
        const int kk = ok[u] ? k : k0;
        Elem<T>::load16(Kb + (size_t)kk * D, kf[u]);
        if (MODE != 2) Elem<T>::load16(Vb + (size_t)kk * D, vf[u]);
        ls_k[u] = lS[kk];
      }
      float nrm[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float s2 = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) s2 += kf[u][e] * kf[u][e];
        nrm[u] = group_sum<LPR>(s2);
      }
      uint32_t zbits[U];
#pragma unroll
      for (int u = 0; u < U; ++u) zbits[u] = 0u;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float lg[U];
        float mx = st.m[h];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float dp = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) dp += qr[h][e] * kf[u][e];
          dp = group_sum<LPR>(dp);
          const float score =
              (nrm[u] > 0.f ? dp * rsqrtf(nrm[u]) * inv_sqrt_d : 0.f) + ls_k[u];
          const int k = base + u * RPW + slot;
          const bool zoom = (double)score > a.theta[g * G + h];
          if (ok[u] && sub == 0) {
            const size_t mi = ((size_t)b * a.Hq + g * G + h) * a.m_max + k;
            if (MODE == 2) {
              a.scores[mi] = score;
            } else if (a.mask) {
              a.mask[mi] = zoom ? 1 : 0;
            }
          }
          if (zoom) zbits[u] |= 1u << h;
          lg[u] = (ok[u] && !zoom) ? dp * c2 + ls_k[u] * kLog2e : kNegInf;
          mx = fmaxf(mx, lg[u]);
        }
        if (MODE == 2) continue;
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
          for (int e = 0; e < EPL; ++e) acc[h][e] += p * vf[u][e];
        }
        st.l[h] = ls;
        st.m[h] = mx;
      }
      if (MODE != 2 && sub == 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (ok[u] && zbits[u]) {
            const int pos = atomicAdd(&list_n, 1);
            list_s[pos] = (base + u * RPW + slot) | (int)(zbits[u] << 24);
          }
        }
      }
    }
  }
  if (MODE == 2) return;

  // ---------------- merge the row slots of each wave (butterfly over slots)
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
      ml_s.m[wave][h] = st.m[h];
      ml_s.l[wave][h] = st.l[h];
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) ml_s.acc[wave][h][sub * EPL + e] = acc[h][e];
  }
  __syncthreads();  // list_s complete

  int nrec = kWaves;
  if (MODE == 0) {
    // ---------------- zoomed spans of this chunk, one wave per span
    float zm[G], zls[G], zacc[G][JPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      zm[h] = kNegInf;
      zls[h] = 0.f;
#pragma unroll
      for (int j = 0; j < JPL; ++j) zacc[h][j] = 0.f;
    }
    const int nz = list_n;
    const T* bases = reinterpret_cast<const T*>(a.bases);
    for (int i = wave; i < nz; i += kWaves) {
      const int ent = list_s[i];
      const int k = ent & 0xffffff;
      const uint32_t hb = (uint32_t)ent >> 24;
      const size_t ti = (size_t)bg * a.m_max + k;
      zoom_span<D, T, G>(bases + a.boff[ti], a.mcount[(size_t)b * a.m_max + k], a.rank[ti], hb,
                         q_s, zl_s[wave], c2, lane, zm, zls, zacc);
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        ml_s.m[kWaves + wave][h] = zm[h];
        ml_s.l[kWaves + wave][h] = zls[h];
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int j = 0; j < JPL; ++j) ml_s.acc[kWaves + wave][h][lane * JPL + j] = zacc[h][j];
    nrec = 2 * kWaves;
    __syncthreads();
  } else {
    // ---------------- hand the zoomed spans to the host for fetching
    __shared__ int s_base;
    if (threadIdx.x == 0) s_base = list_n ? atomicAdd(&a.zcount[bg], list_n) : 0;
    __syncthreads();
    for (int i = threadIdx.x; i < list_n; i += kThreads)
      a.zlist[(size_t)bg * a.m_max + s_base + i] = list_s[i];
  }

  store_partial<D, G>(ml_s, nrec, a, b, g, chunk);
  if (MODE == 0) ticket_and_combine<D, G>(a, b, g, a.n_anchor_chunks + a.n_span_chunks);
}

// ------------------------------------------------------------------ staged zoom kernel (HOST bases)

template <int D, typename T, int G>
__global__ __launch_bounds__(kThreads) void k_decode_staged_zoom(DecodeArgs a) {
  constexpr int JPL = D / 64;
  __shared__ float q_s[G][D];
  __shared__ ZoomLds<G> zl_s[kWaves];
  __shared__ MergeLds<D, G> ml_s;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  for (int i = threadIdx.x; i < G * D; i += kThreads)
    q_s[i / D][i % D] = a.q[((size_t)b * a.Hq + g * G + i / D) * D + i % D];
  __syncthreads();
  const float c2 = kLog2e * rsqrtf((float)D);

  float zm[G], zls[G], zacc[G][JPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    zm[h] = kNegInf;
    zls[h] = 0.f;
#pragma unroll
    for (int j = 0; j < JPL; ++j) zacc[h][j] = 0.f;
  }
  const int e0 = a.zbase[bg], e1 = a.zbase[bg + 1];
  const T* stg = reinterpret_cast<const T*>(a.staging);
  for (int i = e0 + blockIdx.x * kWaves + wave; i < e1; i += a.n_zoom_chunks * kWaves) {
    const int ent = a.zent[i];
    const int k = ent & 0xffffff;
    const uint32_t hb = (uint32_t)ent >> 24;
    const size_t ti = (size_t)bg * a.m_max + k;
    zoom_span<D, T, G>(stg + a.zoff[i], a.mcount[(size_t)b * a.m_max + k], a.rank[ti], hb, q_s,
                       zl_s[wave], c2, lane, zm, zls, zacc);
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      ml_s.m[wave][h] = zm[h];
      ml_s.l[wave][h] = zls[h];
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int j = 0; j < JPL; ++j) ml_s.acc[wave][h][lane * JPL + j] = zacc[h][j];
  __syncthreads();
  store_partial<D, G>(ml_s, kWaves, a, b, g, a.n_anchor_chunks + a.n_span_chunks + blockIdx.x);
  ticket_and_combine<D, G>(a, b, g, a.n_zoom_chunks);
}

template <int D, typename T, int G>
void launch_main_t(int mode, const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.n_anchor_chunks + a.n_span_chunks, a.B * a.Hkv);
  if (mode == 0) hipLaunchKernelGGL((k_decode_main<D, T, G, 0>), grid, dim3(kThreads), 0, s, a);
  else if (mode == 1) hipLaunchKernelGGL((k_decode_main<D, T, G, 1>), grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL((k_decode_main<D, T, G, 2>), grid, dim3(kThreads), 0, s, a);
}

template <int D, typename T>
void launch_main_g(int mode, const DecodeArgs& a, hipStream_t s) {
  switch (a.G) {
    case 1: launch_main_t<D, T, 1>(mode, a, s); break;
    case 2: launch_main_t<D, T, 2>(mode, a, s); break;
    case 4: launch_main_t<D, T, 4>(mode, a, s); break;
    case 8: launch_main_t<D, T, 8>(mode, a, s); break;
  }
}

template <int D, typename T>
void launch_zoom_g(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.n_zoom_chunks, a.B * a.Hkv);
  switch (a.G) {
    case 1: hipLaunchKernelGGL((k_decode_staged_zoom<D, T, 1>), grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_decode_staged_zoom<D, T, 2>), grid, dim3(kThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_decode_staged_zoom<D, T, 4>), grid, dim3(kThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL((k_decode_staged_zoom<D, T, 8>), grid, dim3(kThreads), 0, s, a); break;
  }
}

}  // namespace

void launch_decode_main(int mode, int d, int kv_bf16, const DecodeArgs& a, hipStream_t s) {
  if (d == 128) {
    if (kv_bf16) launch_main_g<128, bf16_t>(mode, a, s);
    else launch_main_g<128, float>(mode, a, s);
  } else {
    if (kv_bf16) launch_main_g<64, bf16_t>(mode, a, s);
    else launch_main_g<64, float>(mode, a, s);
  }
}

void launch_decode_staged_zoom(int d, int kv_bf16, const DecodeArgs& a, hipStream_t s) {
  if (d == 128) {
    if (kv_bf16) launch_zoom_g<128, bf16_t>(a, s);
    else launch_zoom_g<128, float>(a, s);
  } else {
    if (kv_bf16) launch_zoom_g<64, bf16_t>(a, s);
    else launch_zoom_g<64, float>(a, s);
  }
}

}  // namespace sekv
