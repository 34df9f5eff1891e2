// Internal declarations shared by the HIP kernels and the host runtime of the
// SeKV library (gfx950, wave64).  Not part of the public ABI (include/sekv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sekv {

constexpr int kMaxHq = 64;        // query heads per layer supported by the decode kernels
constexpr int kMaxBg = 512;       // sequences x kv heads supported by the decode kernels
constexpr int kThreads = 256;     // 4 wave64 per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kMaxParts = 512;  // split-K partial slots per (sequence, query head)
#ifndef SEKV_COMBINE_THREADS
#define SEKV_COMBINE_THREADS 256
#endif
constexpr int kCombineThreads = SEKV_COMBINE_THREADS;
constexpr int kMaxSpanChunk = 256;  // span rows per span task

// Planned layer-step kernel: every workgroup runs a short list of segments
// (runs of span rows or anchor rows of one (sequence, kv head)), at most
// wg_segments(G) of them, holding at most kMaxWgSpanRows span rows in all.
constexpr int kMaxWgSpanRows = 512;
__host__ __device__ constexpr int wg_segments(int G) { return G == 1 ? 4 : (G <= 4 ? 2 : 1); }

// Every packed basis block starts on a multiple of 8 elements (16 bytes for
// bf16), so wide loads stay aligned.
__host__ __device__ inline int64_t pad8(int64_t x) { return (x + 7) & ~int64_t(7); }

// ---------------------------------------------------------------- decode

struct DecodeArgs {
  int B, Hq, Hkv, G, m_max, na_max;
  const int32_t* m_b;     // [B] spans per sequence
  const int32_t* na_b;    // [B] anchors per sequence
  const float* logS;      // [B][m_max] ln(member count)
  const void* kbar;       // [B][Hkv][m_max][d]
  const void* vbar;
  const void* KA;         // [B][Hkv][na_max][d]
  const void* VA;
  const int2* smeta;      // [B][Hkv][m_max] {basis offset / 8, rank | member count << 8}
  const void* bases;      // device basis store of the layer (DEVICE home), or the mapped pinned store
  const int32_t* cslot;   // [B][Hkv][m_max] device-cache offset / 8 of each span's bases, -1: not cached (or NULL)
  const void* cache;      // the device basis cache
  int64_t basis_elems;    // its size in elements
  const float* q;         // [B][Hq][d]
  float* out;             // [B][Hq][d]
  uint8_t* mask;          // [B][Hq][m_max] zoom decisions (always written)
  uint8_t* mask_h;        // or NULL: the combine kernel copies mask (mask_bytes) here (mapped host memory)
  int64_t mask_bytes;
  float* scores;          // [B][Hq][m_max] (routing-scores mode; input of the budget cap)
  int capped;             // 1: the decisions were taken by the budget cap and are read from mask
  // tasks: span (bg, first span, spans, partial slot; with host-resident bases
  // the next slot holds its zoomed spans) then anchor (bg | 1 << 31, first
  // anchor, anchors, slot)
  const int4* tasks;
  int n_tasks, n_span_tasks;
  const int32_t* parts_n; // [B*Hkv] partial slots used by each (sequence, kv head)
  int max_parts;          // partial slots per (sequence, query head) in the buffers below
  int32_t* zcnt;          // [n_span_tasks] zoomed spans of each span task in the last call (statistics)
  float* part_ml;         // [B][Hq][max_parts][4] (running max in log2 units, sum, zoomed spans, unused)
  float* part_acc;        // [B][Hq][max_parts][d]
  unsigned long long* zcount;  // the layer's counters: [B*Hq] zoomed spans per (sequence, query head)
                               // summed over calls, then the number of calls (or NULL); the combine
                               // kernel counts the call
  int zparts;             // 1: the spans come with the partials (planned kernel) and the combine adds
                          // them; 0: the route kernel adds them (atomics)
  // planned kernel: segments of workgroup i at wsegs[i * wg_segments(G) ..], each
  // (bg | anchors << 31, first row, rows, partial slot); rows = 0 ends a list
  const int4* wsegs;
  int n_zoom_wgs;          // host store: fetched groups at the front of the attend grid
  // host fetch path: flat list (bg | head bits << 24, span, basis offset / 8, rank | count << 8)
  int4* zlist;
  int32_t* zcounter;      // its length (reset by the combine kernel)
  const int4* zitems;     // staged items: (bg | head bits << 24, span, staging offset / 8, rank | count << 8)
  const int4* zgroups;    // (span task, first item, items)
  const void* staging;
  // learned-style routing projection (dr > 0): score = (W q).Kr / sqrt(dr) + ln|S|
  int dr;                 // routing dimension d' (0: identity projection, cosine score on kbar)
  const void* Kr;         // [B][Hkv][m_max][dr] routing summaries, KV dtype
  const float* Wr;        // [Hkv][dr][d] routing projection
  float* qp;              // [B][Hq][dr] projected queries (written by the projection kernel)
  double theta[kMaxHq];   // logit(tau) per query head
  int32_t budget[kMaxHq]; // most zoomed spans per (sequence, query head); < 0: no cap
};

// mode 1 (staged HOST bases): span tasks, zoomed spans to the flat list, grid
// = span tasks.  mode 2: routing scores of the span tasks only, grid = span
// tasks
void launch_decode_route(int mode, int grid, int d, int kv_bf16, const DecodeArgs& a, hipStream_t s);
// the route (which = 0) and attend (which = 1) kernels of one (head dim, KV dtype)
void decode_variant_d128_bf16(int which, int mode, int grid, const DecodeArgs& a, hipStream_t s);
void decode_variant_d128_f32(int which, int mode, int grid, const DecodeArgs& a, hipStream_t s);
void decode_variant_d64_bf16(int which, int mode, int grid, const DecodeArgs& a, hipStream_t s);
void decode_variant_d64_f32(int which, int mode, int grid, const DecodeArgs& a, hipStream_t s);
// the planned layer-step kernel (DEVICE bases, and HOST bases read in place):
// one workgroup per segment list, grid = lists
void launch_decode_planned(int grid, int d, int kv_bf16, const DecodeArgs& a, hipStream_t s);
// HOST bases: n_zoom_wgs workgroups for the fetched groups, then the anchor
// tasks; grid = n_zoom_wgs + anchor tasks
void launch_decode_attend(int grid, int d, int kv_bf16, const DecodeArgs& a, hipStream_t s);
// log-sum-exp merge of every (sequence, query head) into out; resets the counters
void launch_decode_combine(int d, const DecodeArgs& a, hipStream_t s);
// routing projection: qp = W_g q for every (sequence, query head), grid = B * Hq
void launch_decode_qproj(int d, const DecodeArgs& a, hipStream_t s);
// budget cap: zoom decisions of every (sequence, query head) from the routing
// scores (mode 2) into mask, one workgroup each, grid = B * Hq
void launch_decode_select(const DecodeArgs& a, hipStream_t s);

// ---------------------------------------------------------------- no-alloc decode

// Bytes of the per-device scratch array of sekv_decode_attn_noalloc (split-K
// partials, and the zoom mask when the caller passes none).
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;  // SEKV_NOALLOC_SCRATCH_BYTES of sekv.h
// Look up the device address of that array on `device`, which must be the
// current device; once per device, later calls return at once.
hipError_t noalloc_scratch_init(int device);
// The address found by noalloc_scratch_init (NULL before it succeeded).
void* noalloc_scratch(int device);

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
  int dr;                  // routing dimension (0: no routing summaries)
  const float* Wr;         // [Hkv][dr][d]
  void* Kr;                // [B][Hkv][m_max][dr]
  int na_cap;              // anchor rows per (b, g) in KA / VA
};
void launch_summaries(int d, int kv_bf16, const SummaryArgs& a, hipStream_t s);

// Decode-time append: n_new rows per (b, g) copied to KA / VA after the
// sequence's current anchors, then the counts na[b] += n_new (two kernels).
struct AppendArgs {
  const void* K_new;       // [B][Hkv][n_new][d]
  const void* V_new;
  void* KA;                // [B][Hkv][na_cap][d]
  void* VA;
  int32_t* na;             // [B] anchors before the append (device)
  int Hkv, n_new, na_cap;
};
void launch_append(int d, int kv_bf16, int B, const AppendArgs& a, hipStream_t s);

// Row gather per (b, g): out[bg][i] = in[bg][idx[b][i]] for i < cnt[b].
struct GatherArgs {
  const void* in;          // [B*Hkv][in_rows][row_bytes]
  void* out;               // [B*Hkv][out_rows][row_bytes]
  const int32_t* idx;      // [B][idx_stride]
  const int32_t* cnt;      // [B]
  int Hkv, in_rows, out_rows, idx_stride, row_bytes, max_cnt;
};
void launch_gather_rows(int B, const GatherArgs& a, hipStream_t s);

// Copies of element runs, one workgroup per run: list[i] = (source offset / 8,
// destination offset / 8, elements / 8, unused), offsets in elements of esz
// bytes (elements / 8 * esz a multiple of 16); then table_bytes (a multiple of
// 16, both pointers 16-byte aligned) from tsrc to tdst.  The list, src and tsrc
// may be mapped pinned host memory: the device basis cache fills its region and
// updates its slot table this way in one launch.
void launch_copy_runs(const int4* list, int n, const void* src, void* dst, int esz, const void* tsrc, void* tdst,
                      int64_t table_bytes, hipStream_t s);

// Soft rank gates on the stored A factors of the spans of one (sequence, kv head).
struct GateArgs {
  void* bases;             // the layer's packed store (device memory or mapped pinned memory)
  const int64_t* boff;     // [m] element offsets of the spans (of this (b, g))
  const int32_t* rank;     // [m]
  const int32_t* mcount;   // [m]
  const float* gk;         // [m][d] gates of the key components (NULL: keys untouched)
  const float* gv;         // [m][d] gates of the value components (NULL: values untouched)
  int m, d;
};
void launch_rank_gates(int kv_bf16, const GateArgs& a, hipStream_t s);

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
// returns the launch error, or the refusal of the kernel's LDS attribute
hipError_t launch_svd(int cmax, int d, int kv_bf16, const SvdArgs& a, hipStream_t s);

}  // namespace sekv
