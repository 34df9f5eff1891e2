// Batched truncated SVD of SeKV span matrices for gfx950.
//
// For every (sequence, kv head, span, K-or-V) the member rows X (c x d) are
// factorised and the top r = r_eff singular triplets are stored as
// A = U_r Sigma_r (c x r) and B^T = V_r^T (r x d), the truncated SVD of the
// span's key / value matrix (long-form summary page, section 2.2, eq. (6) with
// every rank gate on).
//
// Short spans (c <= 128): one-sided Jacobi (Hestenes) on the c rows of X held
// in LDS: plane rotations of row pairs until the pairs that involve the r
// largest rows are orthogonal, X = J X' with rows x'_i (the r largest orthogonal
// to each other and to the rest).  Then sigma_i = |x'_i|,
// V_i = x'_i / sigma_i, and A = U_r Sigma_r = X V_r is formed from the original
// rows (streamed again from X), so J is never stored.
//
// Tall spans (c > 128): the d x d Gram matrix X^T X is accumulated in fp64
// on the matrix cores (the upper triangle of 16 x 16 tiles), factored by a
// blocked Cholesky (R^T R, semidefinite pivots dropped, the trailing updates
// on the matrix cores) and one-sided Jacobi orthogonalises the rows of R (R = J N with
// orthogonal rows n_i, so R^T R = N^T N and the right singular vectors of X
// are the normalised n_i); sigma_i = |n_i| and A = X V_r is streamed from X.
// fp64 for the Gram and the factorisation keeps the squared condition number
// away from fp32 rounding.
//
// The two products that are matrix products, the Gram and A = X V_r, run on
// the matrix cores (fp64 and fp32 MFMA).  The rotations are plane updates of
// two vectors at a time and stay on the vector ALUs: they are applied to
// disjoint pairs in parallel (round-robin tournament ordering), a group of 8
// threads per pair (tall spans with d = 64: 16), one wave per 16 members of a
// short span's bucket and 8 waves for tall spans.  Neither path keeps the
// rotations, so a workgroup needs about 78 KB of LDS and two fit on a CU.
#include "sekv_device.h"

namespace sekv {

namespace {

constexpr int kSvdThreads = 512;  // 8 waves per workgroup (tall spans, and short spans of up to 128 members)

// Threads of a short-span workgroup for at most PMAX members: 8 per pair of a
// round (PMAX / 2 pairs), so that a pair's dot product is a sum over 8 lanes;
// spans of at most 16 members take one wave.  (4 threads per pair took 40 to 50%
// longer for the buckets of 32 to 128 members, 16 per pair 9 to 14% longer.)
constexpr int rows_threads(int pmax) { return pmax >= 128 ? kSvdThreads : (4 * pmax < 64 ? 64 : 4 * pmax); }

// Row stride of the fp32 vectors in LDS: D + 8 floats.  In a Jacobi round on
// 128 vectors each pair has 8 threads, which read 8 consecutive elements of
// their row; rows of neighbouring pairs then start 8 banks apart and a
// half-wave's 32 reads hit 32 different banks (with D + 1, about 11).
constexpr int kVecPad = 8;

// Matrix-core accumulator tiles (one 16 x 16 tile: 4 values per lane).
typedef float flt4 __attribute__((ext_vector_type(4)));
typedef double dbl4 __attribute__((ext_vector_type(4)));

// Rotation threshold: a pair is rotated while |x_i . x_j| > tol |x_i| |x_j|.
// fp32 storage: p ulps of fp32; bf16 storage: 1e-4, far below the storage
// rounding of the factors (2^-9).
template <typename T>
__device__ __forceinline__ float jacobi_tol(int p) {
  return sizeof(T) == 2 ? 1e-4f : (float)(p + (p & 1)) * 1.1920929e-7f;
}

// Stopping bound.  Only the r largest singular triplets are kept (the
// truncation of eq. (6)), so the sweeps end after one in which no pair that
// involves one of the r largest vectors (by norm at the sweep's start) was
// further than this from orthogonal, even if pairs of smaller vectors were
// still rotated.  Such a pair was then rotated to orthogonal in that sweep, and
// the later rotations of the sweep leave of it about p stop^2 at most.  bf16
// storage: 3e-3, which leaves the kept factors orthonormal to about 1e-3, below
// the 2^-9 rounding of their storage, even for spans whose singular values all
// lie in one tight cluster (with 1e-2 such spans stopped after their first
// sweep, 1e-2 from orthonormal).  fp32 storage: the
// rotation threshold, so that with r >= p the rule is the plain one (stop after
// a sweep with no rotation).
template <typename T>
__device__ __forceinline__ float jacobi_stop(int p) {
  return sizeof(T) == 2 ? 3e-3f : jacobi_tol<T>(p);
}

// One-sided Jacobi on p vectors (length D, stride XS), in place.  All threads
// of the workgroup (NT); each disjoint pair of a round gets 2 * NT / PMAX
// threads.  The squared norms of the vectors (nrm, LDS, p entries) are computed
// at the start of every sweep and carried through its rotations: a rotation
// that zeroes x_i . x_j = g with tangent t maps |x_i|^2 to |x_i|^2 - t g and
// |x_j|^2 to |x_j|^2 + t g, so a round needs one dot product per pair, not
// three.  The sweeps end after one with no rotation, or with no pair above the
// stopping bound `stop` among the pairs that involve one of the r largest
// vectors (marked in topf, LDS, p entries, at every sweep's start).  s_flag
// (LDS, 2 entries): a rotation happened; such a pair was seen.
template <int D, int PMAX, int NT = kSvdThreads>
__device__ void jacobi_sweeps(float* Xv, int XS, int p, int r, float tol, float stop, int* s_flag, float* nrm,
                              int* topf) {
  constexpr int TPP = 2 * NT / PMAX;
  constexpr int EPT = D / TPP;  // elements of a vector per thread of its pair group
  static_assert(D % TPP == 0, "pair groups must tile the vector length");
  const int pi = threadIdx.x / TPP, li = threadIdx.x % TPP;
  const int pe = p + (p & 1);
  if (p < 2) return;
  const bool all_top = r >= p;  // uniform
  for (int sweep = 0; sweep < 40; ++sweep) {
    if (threadIdx.x == 0) {
      s_flag[0] = 0;
      s_flag[1] = 0;
    }
    for (int i = pi; i < p; i += NT / TPP) {
      float sq = 0.f;
#pragma unroll
      for (int k = 0; k < EPT; ++k) {
        const float x = Xv[i * XS + li + k * TPP];
        sq += x * x;
      }
      sq = group_sum<TPP>(sq);
      if (li == 0) nrm[i] = sq;
    }
    __syncthreads();
    if (!all_top) {
      // the r largest norms at the sweep's start (ties to the lower index)
      for (int i = threadIdx.x; i < p; i += NT) {
        const float ni = nrm[i];
        int rk = 0;
        for (int j = 0; j < p; ++j) {
          const float nj = nrm[j];
          rk += (nj > ni || (nj == ni && j < i)) ? 1 : 0;
        }
        topf[i] = rk < r ? 1 : 0;
      }
      __syncthreads();
    }
    // round t pairs (pe - 1, t) in group 0 and ((t + pi) mod (pe - 1),
    // (t - pi) mod (pe - 1)) in group pi > 0: both indices advance by one per
    // round, so they are carried instead of recomputed with two modulos
    const int pm = pe - 1;
    int ia = pi == 0 ? pm : pi;
    int ja = pi == 0 ? 0 : pm - pi;
    // this thread's pair group has seen a pair above the stopping bound that
    // involves a marked vector (once set, the test and its mark reads are skipped)
    bool big = false;
    for (int t = 0; t < pm; ++t) {
      const int i = pi < pe / 2 ? ia : -1, j = pi < pe / 2 ? ja : -1;
      if (pi != 0) ia = ia + 1 == pm ? 0 : ia + 1;
      ja = ja + 1 == pm ? 0 : ja + 1;
      const bool act = i >= 0 && i < p && j < p;
      // the pair's elements stay in registers from the dot product to the rotation
      float u[EPT], v[EPT];
      float al = 0.f, be = 0.f, ga = 0.f;
      float* xi = Xv + (act ? i : 0) * XS + li;
      float* xj = Xv + (act ? j : 0) * XS + li;
      if (act) {
        al = nrm[i];
        be = nrm[j];
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
          u[k] = xi[k * TPP];
          v[k] = xj[k * TPP];
          ga += u[k] * v[k];
        }
      }
      ga = group_sum<TPP>(ga);
      // The threshold test needs no correctly rounded square roots, and the
      // angle no correctly rounded division: v_rcp_f32 and v_rsq_f32 (1 ulp)
      // keep cs^2 + sn^2 = 1 to a few ulps, and a pair left slightly off
      // orthogonal is rotated again in a later round.  These instructions take
      // denormal inputs as zero, so a pair is rotated only when |x_i . x_j| is
      // at least 1e-37: 1 / (2 x_i . x_j) is then finite, and zeta is never
      // 0 * inf (vectors this small are zero for the factors).
      const float sab = __builtin_amdgcn_sqrtf(al) * __builtin_amdgcn_sqrtf(be);
      if (!big && act && fabsf(ga) > stop * sab) big = all_top || topf[i] != 0 || topf[j] != 0;
      if (act && al > 0.f && be > 0.f && fabsf(ga) > fmaxf(1e-37f, tol * sab)) {
        const float zeta = (be - al) * __builtin_amdgcn_rcpf(2.f * ga);
        const float az = fabsf(zeta);
        const float tt = (az > 1e15f) ? 0.5f * __builtin_amdgcn_rcpf(zeta)
                                     : copysignf(__builtin_amdgcn_rcpf(az + __builtin_amdgcn_sqrtf(1.f + zeta * zeta)),
                                                 zeta);
        const float cs = __builtin_amdgcn_rsqf(1.f + tt * tt);
        const float sn = cs * tt;
        // all of x_i, then all of x_j: consecutive stores to one row pair up
        // into ds_write2 (interleaved with the other row's, which the compiler
        // must assume may alias, they stay single)
        float nu[EPT], nv[EPT];
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
          nu[k] = cs * u[k] - sn * v[k];
          nv[k] = sn * u[k] + cs * v[k];
        }
#pragma unroll
        for (int k = 0; k < EPT; ++k) xi[k * TPP] = nu[k];
#pragma unroll
        for (int k = 0; k < EPT; ++k) xj[k * TPP] = nv[k];
        if (li == 0) {
          s_flag[0] = 1;
          nrm[i] = al - tt * ga;
          nrm[j] = be + tt * ga;
        }
      }
      __syncthreads();
    }
    if (__builtin_amdgcn_ballot_w64(big) != 0 && (threadIdx.x & 63) == 0) s_flag[1] = 1;
    __syncthreads();
    const int rot = s_flag[0], any_big = s_flag[1];
    __syncthreads();
    if (!rot || !any_big) break;
  }
}

// sigma_i = |v_i| for p vectors, and order[kk] = index of the kk-th largest (kk < r).
template <int NT = kSvdThreads>
__device__ void rank_by_norm(const float* Xv, int XS, int len, int p, int r, float* sig, int* order) {
  for (int i = threadIdx.x; i < p; i += NT) {
    float s = 0.f;
    for (int e = 0; e < len; ++e) s += Xv[i * XS + e] * Xv[i * XS + e];
    sig[i] = sqrtf(s);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < p; i += NT) {
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

// A^T [r][c8] = (X V_r)^T from the original rows of X (streamed 16 at a time
// through Xr), with V_i = Vt[order[kk]] / sig[order[kk]]; zero beyond c.
// A block of 16 rows times 16 ranks is one fp32 matrix-core product over the
// D columns (v_mfma_f32_16x16x4f32, fp32 products and sums like the scalar
// dot products): wave w takes ranks 16w .. 16w + 15, then 16 (w + NT / 64) ..,
// and so on.
// Operand lanes: A[m][k] = X[m][e0 + k] and B[k][n] = V[n][e0 + k] in lane
// m + 16k (resp. n + 16k); the result D[4 (l / 16) + i][l % 16] in lane l.
template <int D, typename T, int XS, int NT = kSvdThreads>
__device__ void store_a_from_rows(const SvdArgs& a, const Prob& p, const T* src, float* Xr, const float* Vt,
                                  int VS, const float* sig, const int* order) {
  constexpr int ROWS = 16;
  T* At = block_ptr<T, D>(a, p, false);
  const int c8 = (int)pad8(p.c);
  const int r = p.r;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* xrow = Xr + (lane & 15) * XS + (lane >> 4);
  for (int t0 = 0; t0 < p.c; t0 += ROWS) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < ROWS * D; idx += NT) {
      const int t = idx / D, e = idx % D;
      Xr[t * XS + e] = (t0 + t < p.c) ? Elem<T>::to_f(src[(size_t)(t0 + t) * D + e]) : 0.f;
    }
    __syncthreads();
    for (int k0 = wave * 16; k0 < r; k0 += NT / 4) {  // uniform over the wave
      const int kk = k0 + (lane & 15);  // this lane's rank in the B operand and the result
      const int vi = (kk < r) ? order[kk] : 0;
      const float si = (kk < r) ? sig[vi] : 0.f;
      const float* vrow = Vt + vi * VS + (lane >> 4);
      flt4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int e0 = 0; e0 < D; e0 += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xrow[e0], kk < r ? vrow[e0] : 0.f, acc, 0, 0, 0);
      if (kk < r) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + 4 * (lane >> 4) + i;
          if (t < p.c) At[(size_t)kk * c8 + t] = Elem<T>::from_f(si > 0.f ? acc[i] / si : 0.f);
        }
      }
    }
  }
  for (int idx = threadIdx.x; idx < r * (c8 - p.c); idx += NT) {
    const int kk = idx / (c8 - p.c), t = p.c + idx % (c8 - p.c);
    At[(size_t)kk * c8 + t] = Elem<T>::from_f(0.f);
  }
}

template <int D, typename T, int PMAX>
__global__ __launch_bounds__(rows_threads(PMAX)) void k_svd_rows(SvdArgs a) {
  constexpr int NT = rows_threads(PMAX);
  static_assert(NT % 64 == 0 && (2 * NT) % PMAX == 0, "whole waves, whole pair groups");
  extern __shared__ float smem[];
  constexpr int XS = D + kVecPad;
  constexpr int ROWS = 16;
  float* X = smem;                 // [PMAX][XS]: rows of X, orthogonalised in place
  float* Xr = smem + PMAX * XS;    // [ROWS][XS]: original rows, for A
  __shared__ float sig[PMAX];
  __shared__ int order[PMAX];
  __shared__ int s_flag[2];

  const Prob p = load_prob(a, a.Hkv);
  const T* src = reinterpret_cast<const T*>(p.which ? a.V : a.K) + ((size_t)p.bg * a.n + p.ms) * D;
  for (int idx = threadIdx.x; idx < p.c * D; idx += NT) {
    const int t = idx / D, e = idx % D;
    X[t * XS + e] = Elem<T>::to_f(src[(size_t)t * D + e]);
  }
  __syncthreads();
  // (order is free until the sweeps end: it holds the marks of the largest vectors)
  jacobi_sweeps<D, PMAX, NT>(X, XS, p.c, p.r, jacobi_tol<T>(p.c), jacobi_stop<T>(p.c), s_flag, sig, order);
  __syncthreads();
  rank_by_norm<NT>(X, XS, D, p.c, p.r, sig, order);

  // B^T rows: the chosen orthogonal rows, normalised
  T* Bt = block_ptr<T, D>(a, p, true);
  for (int idx = threadIdx.x; idx < p.r * D; idx += NT) {
    const int kk = idx / D, e = idx % D;
    const int i = order[kk];
    const float s = sig[i];
    Bt[idx] = Elem<T>::from_f(s > 0.f ? X[i * XS + e] / s : 0.f);
  }
  store_a_from_rows<D, T, XS, NT>(a, p, src, Xr, X, XS, sig, order);
}

// ---------------------------------------------------------------- tall spans

// Upper-triangle tiles of a GT x GT grid of 16 x 16 tiles: (I, J), J >= I.
template <int GT>
__device__ __forceinline__ int utile(int I, int J) {
  return I * GT - (I * (I - 1)) / 2 + (J - I);
}

// (at most 128 VGPRs: two workgroups of 8 waves per CU)
template <int D, typename T>
__global__ __launch_bounds__(kSvdThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_svd_tall(SvdArgs a) {
  extern __shared__ double smd[];
  constexpr int XS = D + kVecPad;  // float vector stride
  constexpr int ROWS = 16;        // X rows staged per step
  constexpr int GS = D + 16;      // staging row stride: the 4 row groups of a tile read distinct banks
  constexpr int GT = D / 16;      // 16 x 16 Gram tiles per side
  constexpr int NT = GT * (GT + 1) / 2;
  constexpr int TPW = (NT + 7) / 8;  // upper-triangle tiles per wave
  // the Gram, then R, as NT row-major 16 x 16 fp64 tiles (the diagonal
  // tiles whole); the staged rows of X share the space before the tiles exist
  double* Tt = smd;                                       // [NT][16][16]
  float* Xs = reinterpret_cast<float*>(smd);              // [ROWS][GS]
  __shared__ float sig[D];
  __shared__ int order[D];
  __shared__ int s_flag[2];
  __shared__ double s_tol;

  const Prob p = load_prob(a, a.Hkv);
  const T* src = reinterpret_cast<const T*>(p.which ? a.V : a.K) + ((size_t)p.bg * a.n + p.ms) * D;

  // 1. Gram matrix in fp64 on the matrix cores: tile (I, J), I <= J, of
  // G = X^T X accumulates v_mfma_f64_16x16x4f64 over 4 staged rows at a time
  // (A[m][k] = X[k][16 I + m] and B[k][n] = X[k][16 J + n] in lane m + 16 k,
  // resp. n + 16 k; exact fp64 products of the stored values, fp64 sums).
  // Wave w takes tiles w, w + 8, ...
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int ti[TPW], tj[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    int q = wave + 8 * u, I = 0;
    while (I < GT && q >= GT - I) {
      q -= GT - I;
      ++I;
    }
    ti[u] = I;
    tj[u] = I + q;  // I == GT: no tile (q >= NT)
  }
  dbl4 gacc[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) gacc[u] = dbl4{0.0, 0.0, 0.0, 0.0};
  for (int t0 = 0; t0 < p.c; t0 += ROWS) {
    for (int idx = threadIdx.x; idx < ROWS * D; idx += kSvdThreads) {
      const int t = idx / D, e = idx % D;
      Xs[t * GS + e] = (t0 + t < p.c) ? Elem<T>::to_f(src[(size_t)(t0 + t) * D + e]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k0 = 0; k0 < ROWS; k0 += 4) {
      const float* xr = Xs + (k0 + (lane >> 4)) * GS + (lane & 15);
#pragma unroll
      for (int u = 0; u < TPW; ++u)
        if (ti[u] < GT)  // uniform over the wave
          gacc[u] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xr[16 * ti[u]], (double)xr[16 * tj[u]], gacc[u],
                                                         0, 0, 0);
    }
    __syncthreads();
  }
  // the fp64 result is row-interleaved: lane l holds G[16 I + l / 16 + 4 i][16 J + l % 16], i < 4
  // (the staging rows are dead: the loop ended with a barrier)
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    if (ti[u] >= GT) continue;
    double* tile = Tt + utile<GT>(ti[u], tj[u]) * 256;
#pragma unroll
    for (int i = 0; i < 4; ++i) tile[((lane >> 4) + 4 * i) * 16 + (lane & 15)] = gacc[u][i];
  }
  __syncthreads();

  // 2. Cholesky G = R^T R (upper R in place), pivots below tol dropped,
  // blocked by tiles (right-looking): for each block row kb, wave 0 factors
  // the diagonal tile; the panel tiles (kb, J > kb) are solved with R_kk^T,
  // one thread per column; the trailing tiles (I, J), kb < I <= J, take
  // X_I^T X_J off with v_mfma_f64_16x16x4f64 (the panel's negated transpose
  // as the A operand).  Three barriers per block row.
  if (threadIdx.x == 0) {
    double mx = 0.0;
    for (int i = 0; i < D; ++i) mx = fmax(mx, Tt[utile<GT>(i >> 4, i >> 4) * 256 + (i & 15) * 17]);
    s_tol = mx * (double)D * 4.440892098500626e-16;
  }
  __syncthreads();
  {
    const double tolc = s_tol;
    for (int kb = 0; kb < GT; ++kb) {
      double* A = Tt + utile<GT>(kb, kb) * 256;
      // (a) the diagonal tile: unblocked, its upper triangle only
      if (wave == 0) {
        const int j = lane & 15, i0 = lane >> 4;
        for (int k = 0; k < 16; ++k) {
          const double piv = A[k * 17];
          const double r = piv > tolc ? sqrt(piv) : 0.0;
          wave_lds_sync();  // every lane has read the pivot before it is rewritten
          if (lane < 16 && j >= k) A[k * 16 + j] = r > 0.0 ? (j == k ? r : A[k * 16 + j] / r) : 0.0;
          wave_lds_sync();
          const double rkj = A[k * 16 + j];
          for (int i = k + 1 + i0; i <= j; i += 4) A[i * 16 + j] -= A[k * 16 + i] * rkj;
          wave_lds_sync();
        }
      }
      __syncthreads();
      // (b) panel tiles: X = R_kk^-T B, column by column (a dropped pivot gives a zero row)
      const int npan = 16 * (GT - 1 - kb);
      for (int c = threadIdx.x; c < npan; c += kSvdThreads) {
        double* bp = Tt + utile<GT>(kb, kb + 1 + (c >> 4)) * 256 + (c & 15);
        double x[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          double v = bp[k * 16];
#pragma unroll
          for (int m = 0; m < k; ++m) v -= A[m * 16 + k] * x[m];
          const double r = A[k * 17];
          x[k] = r > 0.0 ? v / r : 0.0;
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) bp[k * 16] = x[k];
      }
      __syncthreads();
      // (c) trailing tiles, wave w taking tiles w, w + 8, ... of the triangle
      const int nt = GT - 1 - kb;
      for (int q = wave; q < nt * (nt + 1) / 2; q += kSvdThreads / 64) {
        int I = 0, rr = q;
        while (rr >= nt - I) {
          rr -= nt - I;
          ++I;
        }
        const int TI = kb + 1 + I, TJ = TI + rr;
        const double* pI = Tt + utile<GT>(kb, TI) * 256;
        const double* pJ = Tt + utile<GT>(kb, TJ) * 256;
        double* C = Tt + utile<GT>(TI, TJ) * 256;
        dbl4 acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = C[((lane >> 4) + 4 * i) * 16 + (lane & 15)];
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) {
          const int e = (k0 + (lane >> 4)) * 16 + (lane & 15);
          acc = __builtin_amdgcn_mfma_f64_16x16x4f64(-pI[e], pJ[e], acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) C[((lane >> 4) + 4 * i) * 16 + (lane & 15)] = acc[i];
      }
      __syncthreads();
    }
  }

  // 3. rows of R in fp32 (through registers: they overwrite the packed factor)
  constexpr int PER = D * D / kSvdThreads;
  float rv[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int idx = threadIdx.x + u * kSvdThreads;
    const int row = idx / D, col = idx % D;
    rv[u] = col >= row ? (float)Tt[utile<GT>(row >> 4, col >> 4) * 256 + (row & 15) * 16 + (col & 15)] : 0.f;
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
  jacobi_sweeps<D, D>(Rr, XS, D, p.r, jacobi_tol<T>(D), jacobi_stop<T>(D), s_flag, sig, order);
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
  store_a_from_rows<D, T, XS>(a, p, src, Xr, Rr, XS, sig, order);
}

// The kernels take more than 64 KB of dynamic LDS, which needs the attribute
// set on the current device before the launch (a build-time call, not timed):
// a refusal is returned instead of surfacing later as a launch failure.
template <int D, typename T, int PMAX>
hipError_t launch_rows(const SvdArgs& a, hipStream_t s) {
  const size_t lds = sizeof(float) * (PMAX + 16) * (D + kVecPad);
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_svd_rows<D, T, PMAX>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_svd_rows<D, T, PMAX>), dim3(a.n_problems), dim3(rows_threads(PMAX)), lds, s, a);
  return hipGetLastError();
}

template <int D, typename T>
hipError_t launch_tall(const SvdArgs& a, hipStream_t s) {
  // max(fp64 Gram tiles or the 16 staged rows they replace, fp32 rows of R + 16 staged rows)
  const size_t tiles = sizeof(double) * 256 * ((D / 16) * (D / 16 + 1) / 2), stage = sizeof(float) * 16 * (D + 16);
  const size_t gram = tiles > stage ? tiles : stage;
  const size_t rows = sizeof(float) * (D + 16) * (D + kVecPad);
  const size_t lds = gram > rows ? gram : rows;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_svd_tall<D, T>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_svd_tall<D, T>), dim3(a.n_problems), dim3(kSvdThreads), lds, s, a);
  return hipGetLastError();
}

template <int D, typename T>
hipError_t launch_svd_t(int cmax, const SvdArgs& a, hipStream_t s) {
  switch (cmax) {
    case 16: return launch_rows<D, T, 16>(a, s);
    case 32: return launch_rows<D, T, 32>(a, s);
    case 64: return launch_rows<D, T, 64>(a, s);
    case 128: return launch_rows<D, T, 128>(a, s);
    default: return launch_tall<D, T>(a, s);
  }
}

}  // namespace

hipError_t launch_svd(int cmax, int d, int kv_bf16, const SvdArgs& a, hipStream_t s) {
  if (a.n_problems <= 0) return hipSuccess;
  if (d == 128) return kv_bf16 ? launch_svd_t<128, bf16_t>(cmax, a, s) : launch_svd_t<128, float>(cmax, a, s);
  return kv_bf16 ? launch_svd_t<64, bf16_t>(cmax, a, s) : launch_svd_t<64, float>(cmax, a, s);
}

}  // namespace sekv
