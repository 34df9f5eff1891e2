// Internal declarations shared by the HIP kernels and the host runtime of the
// SeKV library (gfx950, wave64).  Not part of the public ABI (include/sekv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sekv {

constexpr int kMaxHq = 64;        // query heads per layer supported by the decode kernels
constexpr int kThreads = 256;     // 4 wave64 per workgroup
constexpr int kWaves = kThreads / 64;

// Every packed basis block starts on a multiple of 8 elements (16 bytes for
// bf16), so wide loads stay aligned.
__host__ __device__ inline int64_t pad8(int64_t x) { return (x + 7) & ~int64_t(7); }

// ---------------------------------------------------------------- decode

struct DecodeArgs {
  int B, Hq, Hkv, G, m_max, na_max;
  const int32_t* m_b;     // [B] spans per sequence
  const int32_t* na_b;    // [B] anchors per sequence
  const int32_t* mcount;  // [B][m_max] member counts
  const float* logS;      // [B][m_max] ln(member count)
  const void* kbar;       // [B][Hkv][m_max][d]
  const void* vbar;
  const void* KA;         // [B][Hkv][na_max][d]
  const void* VA;
  const int32_t* rank;    // [B][Hkv][m_max]
  const int64_t* boff;    // [B][Hkv][m_max] element offset of each span's packed bases
  const void* bases;      // device basis store of the layer (DEVICE home)
  const float* q;         // [B][Hq][d]
  float* out;             // [B][Hq][d]
  uint8_t* mask;          // [B][Hq][m_max] or null
  float* scores;          // [B][Hq][m_max] or null (route-only mode)
  int n_anchor_chunks, anchor_chunk;  // anchor rows per workgroup
  int n_span_chunks, span_chunk;      // spans per workgroup
  int n_zoom_chunks;                  // workgroups per (b, g) of the staged-zoom kernel
  int n_parts;                        // partial slots per (b, h)
  float* part_ml;         // [B][Hq][n_parts][2] (running max in log2 units, sum)
  float* part_acc;        // [B][Hq][n_parts][d]
  uint32_t* counters;     // [B][Hkv] arrival tickets, self-resetting
  int32_t* zlist;         // [B][Hkv][m_max] zoom list (HOST home), unordered
  int32_t* zcount;        // [B][Hkv]
  const int32_t* zent;    // staged zoom entries, sorted per (b, g)
  const int64_t* zoff;    // staging element offset per entry
  const int32_t* zbase;   // [B*Hkv + 1] first entry of each (b, g)
  const void* staging;    // device staging buffer
  double theta[kMaxHq];   // logit(tau) per query head
};

// mode 0: anchors + routing + summaries + zoomed spans from the device store, in-kernel combine
// mode 1: anchors + routing + summaries; zoomed spans appended to the zoom list
// mode 2: routing scores only
void launch_decode_main(int mode, int d, int kv_bf16, const DecodeArgs& a, hipStream_t s);
// zoomed spans from the staging buffer, then the combine over all partial slots
void launch_decode_staged_zoom(int d, int kv_bf16, const DecodeArgs& a, hipStream_t s);

// ---------------------------------------------------------------- build

struct SegmentArgs {
  const float* H;        // [B][n]
  int B, n, w;
  double alpha;
  int32_t* flagpos;      // [B][n] scratch
  int32_t* mstart;       // [B][n] out (capacity n)
  int32_t* mcount;       // [B][n]
  int32_t* anchors;      // [B][n]
  int32_t* counts;       // [B][4]: m, n_anchors, invalid-H flag, boundary count
  double* stats;         // [B][3]: mu, sigma, theta
};
void launch_segment(const SegmentArgs& a, hipStream_t s);

struct SummaryArgs {
  const float* H;        // [B][n]
  const void* K;         // [B][Hkv][n][d]
  const void* V;
  int B, Hkv, n, m_max, na_max;
  const int32_t* m_b;
  const int32_t* mstart;   // [B][m_max]
  const int32_t* mcount;
  const int32_t* na_b;
  const int32_t* anchors;  // [B][na_max]
  void* kbar;              // [B][Hkv][m_max][d]
  void* vbar;
  void* KA;                // [B][Hkv][na_max][d]
  void* VA;
  int span_chunk, n_span_chunks, anchor_chunk, n_anchor_chunks;
};
void launch_summaries(int d, int kv_bf16, const SummaryArgs& a, hipStream_t s);

struct SvdArgs {
  const void* K;           // [B][Hkv][n][d]
  const void* V;
  int Hkv, n, m_max;
  const int32_t* mstart;   // [B][m_max]
  const int32_t* mcount;
  const int32_t* rank;     // [B][Hkv][m_max]
  const int64_t* boff;     // [B][Hkv][m_max]
  void* bases;             // packed store of the layer
  const int32_t* problems; // [n_problems][3]: b*Hkv+g, span k, which (0 = K, 1 = V)
  int n_problems;
};
// cmax: 16, 32, 64 or 128 member rows (one-sided Jacobi on the rows),
// or 0 for taller spans (fp64 Gram, Cholesky, Jacobi on the triangular factor)
void launch_svd(int cmax, int d, int kv_bf16, const SvdArgs& a, hipStream_t s);

}  // namespace sekv
