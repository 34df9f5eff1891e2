// SeKV prefill builder kernels for gfx950: surprisal segmentation, weighted
// span summaries and the anchor gather.
//
// Segmentation (long-form summary page, section 2.1): a token is a span
// boundary when H_t > mu + alpha*sigma (mu, sigma: mean and population std of
// the sequence's surprisal, accumulated in fp64); boundary tokens and the last
// w positions (local window, Figure 2 / eq. (17)) are anchors; a span's
// members are its positions that are not anchors, which are always one
// contiguous run, and spans without members are dropped.
//
// Summaries (section 2.2, eq. (2); review page): kbar_S = sum_t H_t K_t / sum_t H_t
// over the members (uniform weights when that sum is 0), likewise vbar_S.
// With a routing projection W (d' x d per kv head), the routing summary of
// eq. (3), sum_t w_t W K_t / |sum_t w_t W K_t|, is W kbar_S / |W kbar_S| (the
// sum is linear and the weights sum to one), computed from the unrounded mean.
//
// Soft rank gates (eq. (6)): component i of a span's stored factor A = U Sigma
// is scaled by its gate m_i, the exact product rounded once to the storage type.
#include "sekv_device.h"

#include <algorithm>

namespace sekv {

namespace {

constexpr int kSegThreads = 1024;
constexpr int kSegWaves = kSegThreads / 64;

__device__ double block_sum_f64(double x, double* red) {
  x = wave_sum_f64(x);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = x;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x < 64) {
    t = threadIdx.x < kSegWaves ? red[threadIdx.x] : 0.0;
    t = wave_sum_f64(t);
    if (threadIdx.x == 0) red[kSegWaves] = t;
  }
  __syncthreads();
  t = red[kSegWaves];
  __syncthreads();
  return t;
}

// Exclusive prefix of `flag` over the workgroup; returns the total via *tot.
__device__ int block_scan_flag(bool flag, int* wcnt, int* tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t bal = __ballot(flag);
  const int before = __popcll(bal & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
  if (lane == 0) wcnt[wave] = __popcll(bal);
  __syncthreads();
  int off = 0, all = 0;
  for (int w = 0; w < kSegWaves; ++w) {
    const int c = wcnt[w];
    if (w < wave) off += c;
    all += c;
  }
  __syncthreads();
  *tot = all;
  return off + before;
}

__global__ __launch_bounds__(kSegThreads) void k_segment(SegmentArgs a) {
  __shared__ double red[kSegWaves + 1];
  __shared__ int wcnt[kSegWaves];
  __shared__ int bad_s;
  const int b = blockIdx.x;
  const int n = a.n;
  const float* H = a.H + (size_t)b * n;
  int32_t* flagpos = a.flagpos + (size_t)b * n;
  int32_t* mstart = a.mstart + (size_t)b * n;
  int32_t* mcount = a.mcount + (size_t)b * n;
  int32_t* anchors = a.anchors + (size_t)b * n;
  if (threadIdx.x == 0) bad_s = 0;
  __syncthreads();

  // 1. mean, in fp64, fixed reduction order
  double s = 0.0;
  bool bad = false;
  for (int t = threadIdx.x; t < n; t += kSegThreads) {
    const float h = H[t];
    if (!(h >= 0.f) || isinf(h)) bad = true;  // negative, NaN or infinite
    s += (double)h;
  }
  if (bad) bad_s = 1;
  const double mu = block_sum_f64(s, red) / (double)n;
  // 2. population standard deviation
  double v = 0.0;
  for (int t = threadIdx.x; t < n; t += kSegThreads) {
    const double dlt = (double)H[t] - mu;
    v += dlt * dlt;
  }
  const double sigma = sqrt(block_sum_f64(v, red) / (double)n);
  const double theta = mu + a.alpha * sigma;

  // 3. boundary positions, ascending
  int nflag = 0;
  for (int t0 = 0; t0 < n; t0 += kSegThreads) {
    const int t = t0 + threadIdx.x;
    const bool f = t < n && (double)H[t] > theta;
    int tot;
    const int pos = block_scan_flag(f, wcnt, &tot);
    if (f) flagpos[nflag + pos] = t;
    nflag += tot;
  }
  __syncthreads();
  const bool flag0 = nflag > 0 && flagpos[0] == 0;
  const int wstart = n - a.w > 0 ? n - a.w : 0;

  // 4. spans: raw span j starts at 0 (if position 0 is not a boundary) or at a
  //    boundary; members run from the start (+1 if the start is a boundary)
  //    to min(next start, window start)
  const int nraw = nflag + (flag0 ? 0 : 1);
  int m = 0;
  for (int j0 = 0; j0 < nraw; j0 += kSegThreads) {
    const int j = j0 + threadIdx.x;
    int ms = 0, cnt = 0;
    if (j < nraw) {
      const int fi = flag0 ? j : j - 1;  // index into flagpos of this start (-1: position 0)
      const int st = fi < 0 ? 0 : flagpos[fi];
      const int en = (fi + 1 < nflag) ? flagpos[fi + 1] : n;
      ms = st + (fi >= 0 ? 1 : 0);
      const int me = en < wstart ? en : wstart;
      cnt = me - ms;
    }
    const bool keep = j < nraw && cnt > 0;
    int tot;
    const int pos = block_scan_flag(keep, wcnt, &tot);
    if (keep) {
      mstart[m + pos] = ms;
      mcount[m + pos] = cnt;
    }
    m += tot;
  }
  // 5. anchors: boundaries before the window, then the window
  int nf1 = 0;  // boundaries before the window: a prefix of flagpos
  {
    int c = 0;
    for (int i = threadIdx.x; i < nflag; i += kSegThreads) c += flagpos[i] < wstart ? 1 : 0;
    nf1 = (int)block_sum_f64((double)c, red);
  }
  for (int i = threadIdx.x; i < nf1; i += kSegThreads) anchors[i] = flagpos[i];
  for (int t = wstart + threadIdx.x; t < n; t += kSegThreads) anchors[nf1 + (t - wstart)] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    a.counts[b * 4 + 0] = m;
    a.counts[b * 4 + 1] = nf1 + (n - wstart);
    a.counts[b * 4 + 2] = bad_s;
    a.counts[b * 4 + 3] = nflag;
    a.stats[b * 3 + 0] = mu;
    a.stats[b * 3 + 1] = sigma;
    a.stats[b * 3 + 2] = theta;
  }
}

// Summaries: one wave per span; 16-byte rows loads, RPW rows in flight per wave.
template <int D, typename T>
__global__ __launch_bounds__(kThreads) void k_summaries(SummaryArgs a) {
  constexpr int EPL = Elem<T>::kPer16;
  constexpr int LPR = D / EPL;
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane / LPR, sub = lane % LPR;
  const int bg = blockIdx.y;
  const int b = bg / a.Hkv;
  const float* H = a.H + (size_t)b * a.n;

  if ((int)blockIdx.x >= a.n_span_chunks) {
    // anchor gather
    const int c = blockIdx.x - a.n_span_chunks;
    const int na = a.na_b[b];
    const int r0 = c * a.anchor_chunk, r1 = min(na, r0 + a.anchor_chunk);
    const T* K = reinterpret_cast<const T*>(a.K) + (size_t)bg * a.n * D;
    const T* V = reinterpret_cast<const T*>(a.V) + (size_t)bg * a.n * D;
    T* KA = reinterpret_cast<T*>(a.KA) + (size_t)bg * a.na_cap * D;
    T* VA = reinterpret_cast<T*>(a.VA) + (size_t)bg * a.na_cap * D;
    const int32_t* anc = a.anchors + (size_t)b * a.na_max;
    for (int r = r0 + (threadIdx.x / LPR); r < r1; r += kThreads / LPR) {
      const size_t src = (size_t)anc[r] * D + sub * EPL, dst = (size_t)r * D + sub * EPL;
      *reinterpret_cast<uint4*>(KA + dst) = *reinterpret_cast<const uint4*>(K + src);
      *reinterpret_cast<uint4*>(VA + dst) = *reinterpret_cast<const uint4*>(V + src);
    }
    return;
  }

  const int m = a.m_b[b];
  const int k0 = blockIdx.x * a.span_chunk, k1 = min(m, k0 + a.span_chunk);
  const T* K = reinterpret_cast<const T*>(a.K) + (size_t)bg * a.n * D + sub * EPL;
  const T* V = reinterpret_cast<const T*>(a.V) + (size_t)bg * a.n * D + sub * EPL;
  for (int k = k0 + wave; k < k1; k += kWaves) {
    const int ms = a.mstart[(size_t)b * a.m_max + k];
    const int c = a.mcount[(size_t)b * a.m_max + k];
    float ak[EPL], av[EPL], sk[EPL], sv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) ak[e] = av[e] = sk[e] = sv[e] = 0.f;
    float hs = 0.f;
    for (int t = ms + slot; t < ms + c; t += RPW) {
      float kf[EPL], vf[EPL];
      Elem<T>::load16(K + (size_t)t * D, kf);
      Elem<T>::load16(V + (size_t)t * D, vf);
      const float h = H[t];
      hs += h;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        ak[e] += h * kf[e];
        av[e] += h * vf[e];
        sk[e] += kf[e];
        sv[e] += vf[e];
      }
    }
    // reduce over the RPW row slots
    for (int off = LPR; off < 64; off <<= 1) {
      hs += __shfl_xor(hs, off, 64);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        ak[e] += __shfl_xor(ak[e], off, 64);
        av[e] += __shfl_xor(av[e], off, 64);
        sk[e] += __shfl_xor(sk[e], off, 64);
        sv[e] += __shfl_xor(sv[e], off, 64);
      }
    }
    if (slot == 0) {
      const bool uni = !(hs > 0.f);
      const float inv = uni ? 1.f / (float)c : 1.f / hs;
      float ok[EPL], ov[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        ok[e] = (uni ? sk[e] : ak[e]) * inv;
        ov[e] = (uni ? sv[e] : av[e]) * inv;
      }
      const size_t dst = ((size_t)bg * a.m_max + k) * D + sub * EPL;
      Elem<T>::store16(reinterpret_cast<T*>(a.kbar) + dst, ok);
      Elem<T>::store16(reinterpret_cast<T*>(a.vbar) + dst, ov);
      if (a.dr > 0) {
        // routing summary: y = W kbar (lane sub keeps outputs sub*EPL ..), then unit length
        const float* Wg = a.Wr + (size_t)(bg % a.Hkv) * a.dr * D + sub * EPL;
        float y[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) y[e] = 0.f;
        for (int j = 0; j < a.dr; ++j) {
          float wv[EPL];
#pragma unroll
          for (int e = 0; e < EPL; e += 4) Elem<float>::load16(Wg + (size_t)j * D + e, wv + e);
          float p = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) p += wv[e] * ok[e];
          p = group_sum<LPR>(p);
#pragma unroll
          for (int e = 0; e < EPL; ++e)
            if (j == sub * EPL + e) y[e] = p;
        }
        float s2 = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) s2 += y[e] * y[e];
        s2 = group_sum<LPR>(s2);
        const float inv = s2 > 0.f ? 1.f / sqrtf(s2) : 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) y[e] *= inv;
        if (sub * EPL < a.dr)
          Elem<T>::store16(reinterpret_cast<T*>(a.Kr) + ((size_t)bg * a.m_max + k) * a.dr + sub * EPL, y);
      }
    }
  }
}

// Decode-time append: block (bg, row chunk) copies rows of the new keys and
// values behind the current anchors of sequence b; 16-byte pieces.
__global__ __launch_bounds__(kThreads) void k_append(AppendArgs a, int row_bytes) {
  const int bg = blockIdx.x, b = bg / a.Hkv;
  const int base = a.na[b];
  const int p16 = row_bytes / 16;
  const size_t n16 = (size_t)a.n_new * p16;
  const uint4* ks = reinterpret_cast<const uint4*>(a.K_new) + (size_t)bg * n16;
  const uint4* vs = reinterpret_cast<const uint4*>(a.V_new) + (size_t)bg * n16;
  uint4* kd = reinterpret_cast<uint4*>(a.KA) + ((size_t)bg * a.na_cap + base) * p16;
  uint4* vd = reinterpret_cast<uint4*>(a.VA) + ((size_t)bg * a.na_cap + base) * p16;
  for (size_t i = (size_t)blockIdx.y * kThreads + threadIdx.x; i < n16; i += (size_t)gridDim.y * kThreads) {
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
}

// Block (bg, chunk) gathers rows of one (sequence, kv head) in 16-byte pieces.
// Workgroups [0, n) copy one run each; the workgroups after them copy the
// 16-byte pieces [0, n16) of a table range, one piece per thread.
__global__ __launch_bounds__(kThreads) void k_copy_runs(const int4* list, int n, const void* src, void* dst, int esz,
                                                       const uint4* tsrc, uint4* tdst, int64_t n16) {
  if ((int)blockIdx.x >= n) {
    const int64_t i = (int64_t)(blockIdx.x - n) * kThreads + threadIdx.x;
    if (i < n16) tdst[i] = tsrc[i];
    return;
  }
  const int4 e = list[blockIdx.x];
  const int64_t m16 = (int64_t)e.z * 8 * esz / 16;
  const uint4* in = reinterpret_cast<const uint4*>(static_cast<const char*>(src) + ((int64_t)(uint32_t)e.x << 3) * esz);
  uint4* out = reinterpret_cast<uint4*>(static_cast<char*>(dst) + ((int64_t)(uint32_t)e.y << 3) * esz);
  for (int64_t i = threadIdx.x; i < m16; i += kThreads) out[i] = in[i];
}

__global__ __launch_bounds__(kThreads) void k_gather_rows(GatherArgs a) {
  const int bg = blockIdx.x, b = bg / a.Hkv;
  const int n = a.cnt[b];
  const int p16 = a.row_bytes / 16;
  const uint4* in = reinterpret_cast<const uint4*>(a.in) + (size_t)bg * a.in_rows * p16;
  uint4* out = reinterpret_cast<uint4*>(a.out) + (size_t)bg * a.out_rows * p16;
  const int32_t* idx = a.idx + (size_t)b * a.idx_stride;
  for (int i = blockIdx.y * kThreads + threadIdx.x; i < n * p16; i += gridDim.y * kThreads) {
    const int row = i / p16, piece = i % p16;
    out[(size_t)row * p16 + piece] = in[(size_t)idx[row] * p16 + piece];
  }
}

// The counts follow in their own launch, after every copy has read them.
__global__ void k_append_count(int32_t* na, int B, int n_new) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) na[b] += n_new;
}

// bfloat16 nearest (ties to even) of a double: round to float with the last
// bit made sticky (round to odd: truncate, then set bit 0 if anything was
// dropped), which keeps the information the second rounding needs.
__device__ __forceinline__ bf16_t bf16_from_f64(double x) {
  float f = __double2float_rz(x);
  if ((double)f != x) f = __uint_as_float(__float_as_uint(f) | 1u);
  return f32_to_bf16(f);
}

// One workgroup per span: rows i < rank of A_K^T (and A_V^T) times gate i.
// The product of a stored value and a float32 gate is exact in double.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_rank_gates(GateArgs a) {
  const int k = blockIdx.x;
  const int r = a.rank[k], c = a.mcount[k];
  const int c8 = (int)pad8(c);
  T* AKt = reinterpret_cast<T*>(a.bases) + a.boff[k];
  T* AVt = AKt + (size_t)r * (c8 + a.d);
  for (int w = 0; w < 2; ++w) {
    const float* gt = w == 0 ? a.gk : a.gv;
    if (!gt) continue;
    T* At = w == 0 ? AKt : AVt;
    for (int idx = threadIdx.x; idx < r * c; idx += kThreads) {
      const int i = idx / c, t = idx % c;
      const double x = (double)Elem<T>::to_f(At[(size_t)i * c8 + t]) * (double)gt[(size_t)k * a.d + i];
      if constexpr (sizeof(T) == 2) At[(size_t)i * c8 + t] = bf16_from_f64(x);
      else At[(size_t)i * c8 + t] = (float)x;
    }
  }
}

template <int D, typename T>
void launch_summ_t(const SummaryArgs& a, hipStream_t s) {
  dim3 grid(a.n_span_chunks + a.n_anchor_chunks, a.B * a.Hkv);
  hipLaunchKernelGGL((k_summaries<D, T>), grid, dim3(kThreads), 0, s, a);
}

}  // namespace

void launch_segment(const SegmentArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_segment, dim3(a.B), dim3(kSegThreads), 0, s, a);
}

void launch_append(int d, int kv_bf16, int B, const AppendArgs& a, hipStream_t s) {
  const int row_bytes = d * (kv_bf16 ? 2 : 4);
  const int chunks = std::max(1, std::min(64, (a.n_new * row_bytes / 16 + kThreads - 1) / kThreads));
  hipLaunchKernelGGL(k_append, dim3(B * a.Hkv, chunks), dim3(kThreads), 0, s, a, row_bytes);
  hipLaunchKernelGGL(k_append_count, dim3((B + 255) / 256), dim3(256), 0, s, a.na, B, a.n_new);
}

void launch_copy_runs(const int4* list, int n, const void* src, void* dst, int esz, const void* tsrc, void* tdst,
                      int64_t table_bytes, hipStream_t s) {
  const int64_t n16 = table_bytes / 16;
  const int64_t blocks = n + (n16 + kThreads - 1) / kThreads;
  if (blocks <= 0) return;
  hipLaunchKernelGGL(k_copy_runs, dim3((unsigned)blocks), dim3(kThreads), 0, s, list, n, src, dst, esz,
                     static_cast<const uint4*>(tsrc), static_cast<uint4*>(tdst), n16);
}

void launch_gather_rows(int B, const GatherArgs& a, hipStream_t s) {
  if (a.max_cnt <= 0) return;
  const int chunks = std::max(1, std::min(64, (a.max_cnt * (a.row_bytes / 16) + kThreads - 1) / kThreads));
  hipLaunchKernelGGL(k_gather_rows, dim3(B * a.Hkv, chunks), dim3(kThreads), 0, s, a);
}

void launch_rank_gates(int kv_bf16, const GateArgs& a, hipStream_t s) {
  if (a.m <= 0) return;
  if (kv_bf16) hipLaunchKernelGGL(k_rank_gates<bf16_t>, dim3(a.m), dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(k_rank_gates<float>, dim3(a.m), dim3(kThreads), 0, s, a);
}

void launch_summaries(int d, int kv_bf16, const SummaryArgs& a, hipStream_t s) {
  if (d == 128) {
    if (kv_bf16) launch_summ_t<128, bf16_t>(a, s);
    else launch_summ_t<128, float>(a, s);
  } else {
    if (kv_bf16) launch_summ_t<64, bf16_t>(a, s);
    else launch_summ_t<64, float>(a, s);
  }
}

}  // namespace sekv
