// Batched truncated SVD of SeKV span matrices for gfx950.
//
// For every (sequence, kv head, span, K-or-V) the member rows X (c x d) are
// factorised and the top r = r_eff singular triplets are stored as
// A = U_r Sigma_r (c x r) and B^T = V_r^T (r x d), the truncated SVD of the
// span's key / value matrix (long-form summary page, section 2.2, eq. (6) with
// every rank gate on).
//
// Short spans (c <= 128): one-sided Jacobi (Hestenes) on the c rows of X held
// in LDS: plane rotations of row pairs until all pairs are orthogonal,
// X = J X' with orthogonal rows x'_i.  Then sigma_i = |x'_i|,
// V_i = x'_i / sigma_i, and A = U_r Sigma_r = X V_r is formed from the original
// rows (streamed again from X), so J is never stored.
//
// Tall spans (c > 128): the d x d Gram matrix X^T X is accumulated in fp64
// (upper triangle, packed), factored by Cholesky (R^T R, semidefinite pivots
// dropped) and one-sided Jacobi orthogonalises the rows of R (R = J N with
// orthogonal rows n_i, so R^T R = N^T N and the right singular vectors of X
// are the normalised n_i); sigma_i = |n_i| and A = X V_r is streamed from X.
// fp64 for the Gram and the factorisation keeps the squared condition number
// away from fp32 rounding.
//
// Rotations are applied to disjoint pairs in parallel (round-robin tournament
// ordering), one group of 512/PMAX threads per pair.  Neither path keeps the
// rotations, so a workgroup needs about 78 KB of LDS and two fit on a CU.
#include "sekv_device.h"

namespace sekv {

namespace {

constexpr int kSvdThreads = 512;  // 8 waves per workgroup
// Row stride of the fp32 vectors in LDS: D + 8 floats.  In a Jacobi round on
// 128 vectors each pair has 8 threads, which read 8 consecutive elements of
// their row; rows of neighbouring pairs then start 8 banks apart and a
// half-wave's 32 reads hit 32 different banks (with D + 1, about 11).
constexpr int kVecPad = 8;

// Rotation threshold: a pair is rotated while |x_i . x_j| > tol |x_i| |x_j|.
// fp32 storage: p ulps of fp32; bf16 storage: 1e-4, far below the storage
// rounding of the factors (2^-9).
template <typename T>
__device__ __forceinline__ float jacobi_tol(int p) {
  return sizeof(T) == 2 ? 1e-4f : (float)(p + (p & 1)) * 1.1920929e-7f;
}

// One-sided Jacobi on p vectors (length D, stride XS), in place.  All threads
// of the workgroup; each disjoint pair of a round gets 2 * kSvdThreads / PMAX
// threads.
template <int D, int PMAX>
__device__ void jacobi_sweeps(float* Xv, int XS, int p, float tol, int* s_rot) {
  constexpr int TPP = 2 * kSvdThreads / PMAX;
  constexpr int EPT = D / TPP;  // elements of a vector per thread of its pair group
  static_assert(D % TPP == 0, "pair groups must tile the vector length");
  const int pi = threadIdx.x / TPP, li = threadIdx.x % TPP;
  const int pe = p + (p & 1);
  if (p < 2) return;
  for (int sweep = 0; sweep < 40; ++sweep) {
    if (threadIdx.x == 0) *s_rot = 0;
    __syncthreads();
    for (int t = 0; t < pe - 1; ++t) {
      int i = -1, j = -1;
      if (pi < pe / 2) {
        if (pi == 0) {
          i = pe - 1;
          j = t;
        } else {
          i = (t + pi) % (pe - 1);
          j = (t - pi + pe - 1) % (pe - 1);
        }
      }
      const bool act = i >= 0 && i < p && j < p;
      // the pair's elements stay in registers from the dot products to the rotation
      float u[EPT], v[EPT];
      float al = 0.f, be = 0.f, ga = 0.f;
      float* xi = Xv + (act ? i : 0) * XS + li;
      float* xj = Xv + (act ? j : 0) * XS + li;
      if (act) {
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
          u[k] = xi[k * TPP];
          v[k] = xj[k * TPP];
          al += u[k] * u[k];
          be += v[k] * v[k];
          ga += u[k] * v[k];
        }
      }
      al = group_sum<TPP>(al);
      be = group_sum<TPP>(be);
      ga = group_sum<TPP>(ga);
      if (act && al > 0.f && be > 0.f && fabsf(ga) > tol * sqrtf(al) * sqrtf(be)) {
        const float zeta = (be - al) / (2.f * ga);
        const float az = fabsf(zeta);
        const float tt = (az > 1e15f) ? 0.5f / zeta
                                     : copysignf(1.f, zeta) / (az + sqrtf(1.f + zeta * zeta));
        const float cs = 1.f / sqrtf(1.f + tt * tt);
        const float sn = cs * tt;
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
          xi[k * TPP] = cs * u[k] - sn * v[k];
          xj[k * TPP] = sn * u[k] + cs * v[k];
        }
        if (li == 0) *s_rot = 1;
      }
      __syncthreads();
    }
    const int rot = *s_rot;
    __syncthreads();
    if (!rot) break;
  }
}

// sigma_i = |v_i| for p vectors, and order[kk] = index of the kk-th largest (kk < r).
__device__ void rank_by_norm(const float* Xv, int XS, int len, int p, int r, float* sig, int* order) {
  for (int i = threadIdx.x; i < p; i += kSvdThreads) {
    float s = 0.f;
    for (int e = 0; e < len; ++e) s += Xv[i * XS + e] * Xv[i * XS + e];
    sig[i] = sqrtf(s);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < p; i += kSvdThreads) {
    const float si = sig[i];
    int rk = 0;
    for (int j = 0; j < p; ++j) rk += (sig[j] > si || (sig[j] == si && j < i)) ? 1 : 0;
    if (rk < r) order[rk] = i;
  }
  __syncthreads();
}

struct Prob {
  int bg, b, k, which, c, r, ms;
  int64_t off;
};

__device__ Prob load_prob(const SvdArgs& a, int Hkv) {
  Prob p;
  const int32_t* e = a.problems + 3 * (size_t)blockIdx.x;
  p.bg = e[0];
  p.k = e[1];
  p.which = e[2];
  p.b = p.bg / Hkv;
  p.ms = a.mstart[(size_t)p.b * a.m_max + p.k];
  p.c = a.mcount[(size_t)p.b * a.m_max + p.k];
  p.r = a.rank[(size_t)p.bg * a.m_max + p.k];
  p.off = a.boff[(size_t)p.bg * a.m_max + p.k];
  return p;
}

// Packed blocks of a span: A_K^T [r][c8] | B_K^T [r][D] | A_V^T [r][c8] | B_V^T [r][D].
template <typename T, int D>
__device__ __forceinline__ T* block_ptr(const SvdArgs& a, const Prob& p, bool bt) {
  T* base = reinterpret_cast<T*>(a.bases) + p.off;
  const int64_t ca = (int64_t)p.r * pad8(p.c), rb = (int64_t)p.r * D;
  if (p.which) base += ca + rb;
  return bt ? base + ca : base;
}

// ---------------------------------------------------------------- short spans

// A^T [r][c8] = (X V_r)^T from the original rows of X (streamed ROWS at a time
// through Xr), with V_i = Vt[order[kk]] / sig[order[kk]]; zero beyond c.
template <int D, typename T, int ROWS, int XS>
__device__ void store_a_from_rows(const SvdArgs& a, const Prob& p, const T* src, float* Xr, const float* Vt,
                                  int VS, const float* sig, const int* order) {
  T* At = block_ptr<T, D>(a, p, false);
  const int c8 = (int)pad8(p.c);
  const int r = p.r;
  for (int t0 = 0; t0 < p.c; t0 += ROWS) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < ROWS * D; idx += kSvdThreads) {
      const int t = idx / D, e = idx % D;
      Xr[t * XS + e] = (t0 + t < p.c) ? Elem<T>::to_f(src[(size_t)(t0 + t) * D + e]) : 0.f;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < ROWS * r; idx += kSvdThreads) {
      const int t = idx % ROWS, kk = idx / ROWS;
      if (t0 + t >= p.c) continue;
      const int i = order[kk];
      const float si = sig[i];
      float s = 0.f;
      if (si > 0.f) {
        for (int e = 0; e < D; ++e) s += Xr[t * XS + e] * Vt[i * VS + e];
        s /= si;
      }
      At[(size_t)kk * c8 + t0 + t] = Elem<T>::from_f(s);
    }
  }
  for (int idx = threadIdx.x; idx < r * (c8 - p.c); idx += kSvdThreads) {
    const int kk = idx / (c8 - p.c), t = p.c + idx % (c8 - p.c);
    At[(size_t)kk * c8 + t] = Elem<T>::from_f(0.f);
  }
}

template <int D, typename T, int PMAX>
__global__ __launch_bounds__(kSvdThreads) void k_svd_rows(SvdArgs a) {
  extern __shared__ float smem[];
  constexpr int XS = D + kVecPad;
  constexpr int ROWS = 16;
  float* X = smem;                 // [PMAX][XS]: rows of X, orthogonalised in place
  float* Xr = smem + PMAX * XS;    // [ROWS][XS]: original rows, for A
  __shared__ float sig[PMAX];
  __shared__ int order[PMAX];
  __shared__ int s_rot;

  const Prob p = load_prob(a, a.Hkv);
  const T* src = reinterpret_cast<const T*>(p.which ? a.V : a.K) + ((size_t)p.bg * a.n + p.ms) * D;
  for (int idx = threadIdx.x; idx < p.c * D; idx += kSvdThreads) {
    const int t = idx / D, e = idx % D;
    X[t * XS + e] = Elem<T>::to_f(src[(size_t)t * D + e]);
  }
  __syncthreads();
  jacobi_sweeps<D, PMAX>(X, XS, p.c, jacobi_tol<T>(p.c), &s_rot);
  __syncthreads();
  rank_by_norm(X, XS, D, p.c, p.r, sig, order);

  // B^T rows: the chosen orthogonal rows, normalised
  T* Bt = block_ptr<T, D>(a, p, true);
  for (int idx = threadIdx.x; idx < p.r * D; idx += kSvdThreads) {
    const int kk = idx / D, e = idx % D;
    const int i = order[kk];
    const float s = sig[i];
    Bt[idx] = Elem<T>::from_f(s > 0.f ? X[i * XS + e] / s : 0.f);
  }
  store_a_from_rows<D, T, ROWS, XS>(a, p, src, Xr, X, XS, sig, order);
}

// ---------------------------------------------------------------- tall spans

// Packed upper triangle of a D x D symmetric matrix: (i, j), j >= i.
template <int D>
__device__ __forceinline__ int upk(int i, int j) {
  return i * D - (i * (i - 1)) / 2 + (j - i);
}

template <int D, typename T>
__global__ __launch_bounds__(kSvdThreads) void k_svd_tall(SvdArgs a) {
  extern __shared__ double smd[];
  constexpr int XS = D + kVecPad;  // float vector stride
  constexpr int ROWS = 16;        // X rows staged per step
  constexpr int NB = D / 8;       // 8-column Gram blocks per row of blocks
  constexpr int NP = D * (D + 1) / 2;
  double* Gp = smd;                                       // [NP] packed upper Gram, then R
  float* Xs = reinterpret_cast<float*>(smd + NP);         // [ROWS][D]
  __shared__ float sig[D];
  __shared__ int order[D];
  __shared__ int s_rot;
  __shared__ double s_rkk, s_tol;

  const Prob p = load_prob(a, a.Hkv);
  const T* src = reinterpret_cast<const T*>(p.which ? a.V : a.K) + ((size_t)p.bg * a.n + p.ms) * D;

  // 1. Gram matrix in fp64: 4 x 8 blocks (rows 4 bi.., columns 8 bj..) that
  // reach the upper triangle; 32 fp64 accumulators per thread keep two
  // workgroups per CU
  const int bi = threadIdx.x / NB, bj = threadIdx.x % NB;
  const bool gact = bi < 2 * NB && bj * 8 + 7 >= bi * 4;
  double gacc[4][8];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 8; ++v) gacc[u][v] = 0.0;
  for (int t0 = 0; t0 < p.c; t0 += ROWS) {
    for (int idx = threadIdx.x; idx < ROWS * D; idx += kSvdThreads) {
      const int t = idx / D, e = idx % D;
      Xs[idx] = (t0 + t < p.c) ? Elem<T>::to_f(src[(size_t)(t0 + t) * D + e]) : 0.f;
    }
    __syncthreads();
    if (gact) {
      for (int t = 0; t < ROWS; ++t) {
        double xa[4], xb[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) xa[u] = (double)Xs[t * D + bi * 4 + u];
#pragma unroll
        for (int v = 0; v < 8; ++v) xb[v] = (double)Xs[t * D + bj * 8 + v];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = 0; v < 8; ++v) gacc[u][v] = fma(xa[u], xb[v], gacc[u][v]);
      }
    }
    __syncthreads();
  }
  if (gact) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const int gi = bi * 4 + u, gj = bj * 8 + v;
        if (gj >= gi) Gp[upk<D>(gi, gj)] = gacc[u][v];
      }
  }
  __syncthreads();

  // 2. Cholesky G = R^T R (upper R in place), pivots below tol dropped
  if (threadIdx.x == 0) {
    double mx = 0.0;
    for (int i = 0; i < D; ++i) mx = fmax(mx, Gp[upk<D>(i, i)]);
    s_tol = mx * (double)D * 4.440892098500626e-16;
  }
  __syncthreads();
  const double tolc = s_tol;
  for (int kc = 0; kc < D; ++kc) {
    if (threadIdx.x == 0) {
      const double piv = Gp[upk<D>(kc, kc)];
      s_rkk = piv > tolc ? sqrt(piv) : 0.0;
    }
    __syncthreads();
    const double rkk = s_rkk;
    for (int j = kc + threadIdx.x; j < D; j += kSvdThreads) {
      const int q = upk<D>(kc, j);
      Gp[q] = rkk > 0.0 ? (j == kc ? rkk : Gp[q] / rkk) : 0.0;
    }
    __syncthreads();
    const int w = D - kc - 1;
    for (int idx = threadIdx.x; idx < w * w; idx += kSvdThreads) {
      const int i = kc + 1 + idx / w, j = kc + 1 + idx % w;
      if (j >= i) Gp[upk<D>(i, j)] -= Gp[upk<D>(kc, i)] * Gp[upk<D>(kc, j)];
    }
    __syncthreads();
  }

  // 3. rows of R in fp32 (through registers: they overwrite the packed factor)
  constexpr int PER = D * D / kSvdThreads;
  float rv[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int idx = threadIdx.x + u * kSvdThreads;
    const int row = idx / D, col = idx % D;
    rv[u] = col >= row ? (float)Gp[upk<D>(row, col)] : 0.f;
  }
  __syncthreads();
  float* Rr = reinterpret_cast<float*>(smd);  // [D][XS]: vector row = row `row` of R
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int idx = threadIdx.x + u * kSvdThreads;
    const int row = idx / D, col = idx % D;
    Rr[row * XS + col] = rv[u];
  }
  __syncthreads();
  jacobi_sweeps<D, D>(Rr, XS, D, jacobi_tol<T>(D), &s_rot);
  __syncthreads();
  rank_by_norm(Rr, XS, D, D, p.r, sig, order);

  // 4. B^T rows = the chosen orthogonal rows of R, normalised
  T* Bt = block_ptr<T, D>(a, p, true);
  for (int idx = threadIdx.x; idx < p.r * D; idx += kSvdThreads) {
    const int kk = idx / D, e = idx % D;
    const int i = order[kk];
    Bt[idx] = Elem<T>::from_f(sig[i] > 0.f ? Rr[i * XS + e] / sig[i] : 0.f);
  }
  // 5. A = X V_r, streamed from X through the staging rows
  float* Xr = Rr + D * XS;  // [ROWS][XS], after the rows of R
  store_a_from_rows<D, T, ROWS, XS>(a, p, src, Xr, Rr, XS, sig, order);
}

template <int D, typename T, int PMAX>
void launch_rows(const SvdArgs& a, hipStream_t s) {
  const size_t lds = sizeof(float) * (PMAX + 16) * (D + kVecPad);
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_svd_rows<D, T, PMAX>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    attr = true;
  }
  hipLaunchKernelGGL((k_svd_rows<D, T, PMAX>), dim3(a.n_problems), dim3(kSvdThreads), lds, s, a);
}

template <int D, typename T>
void launch_tall(const SvdArgs& a, hipStream_t s) {
  // max(packed fp64 Gram + 16 staged rows, fp32 rows of R + 16 staged rows)
  const size_t gram = sizeof(double) * (D * (D + 1) / 2) + sizeof(float) * 16 * D;
  const size_t rows = sizeof(float) * (D + 16) * (D + kVecPad);
  const size_t lds = gram > rows ? gram : rows;
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_svd_tall<D, T>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    attr = true;
  }
  hipLaunchKernelGGL((k_svd_tall<D, T>), dim3(a.n_problems), dim3(kSvdThreads), lds, s, a);
}

template <int D, typename T>
void launch_svd_t(int cmax, const SvdArgs& a, hipStream_t s) {
  switch (cmax) {
    case 16: launch_rows<D, T, 16>(a, s); break;
    case 32: launch_rows<D, T, 32>(a, s); break;
    case 64: launch_rows<D, T, 64>(a, s); break;
    case 128: launch_rows<D, T, 128>(a, s); break;
    default: launch_tall<D, T>(a, s); break;
  }
}

}  // namespace

void launch_svd(int cmax, int d, int kv_bf16, const SvdArgs& a, hipStream_t s) {
  if (a.n_problems <= 0) return;
  if (d == 128) {
    if (kv_bf16) launch_svd_t<128, bf16_t>(cmax, a, s);
    else launch_svd_t<128, float>(cmax, a, s);
  } else {
    if (kv_bf16) launch_svd_t<64, bf16_t>(cmax, a, s);
    else launch_svd_t<64, float>(cmax, a, s);
  }
}

}  // namespace sekv
