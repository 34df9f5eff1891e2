// Host runtime and C ABI of the SeKV library (see include/sekv.h).
//
// Owns the span tables, per-layer artefacts (summaries, anchors, packed SVD
// bases in device memory or in a pinned host store), decode scratch (split-K
// partials, arrival tickets), the zoom fetch path (pinned tables, device
// staging, a side stream) and launches the HIP kernels.
#include "sekv.h"
#include "plan.h"
#include "sekv_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <string>
#include <vector>

using namespace sekv;

namespace {

std::string g_create_err;

uint64_t splitmix64(uint64_t x) {
  // SplitMix64 output for state x (Steele, Lea, Flood 2014).
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int env_int(const char* name, int dflt, int lo, int hi) {
  const char* s = std::getenv(name);
  if (!s || !*s) return dflt;
  int v = std::atoi(s);
  return std::min(hi, std::max(lo, v));
}

// Work schedule of one layer's attend kernel: one task per workgroup.
// Zoom-heavy (sequence, kv head) rows get smaller span chunks, so that a span
// task holds about one zoomed span per wave, and go first; the zoom load of
// each row comes from the per-task zoom counts the kernels store, read back
// without a sync.
struct LayerSched {
  bool valid = false;
  bool anchors_changed = false;  // tokens were appended: replan before the next launch
  std::vector<int4> tasks;        // (bg | anchor << 31, first row, rows, partial slot)
  int n_span_tasks = 0;           // span tasks come first
  std::vector<int32_t> parts_n;   // [B*Hkv]
  std::vector<int32_t> chunk;     // [B*Hkv] span rows per task
  std::vector<int32_t> first_span_task;  // [B*Hkv]
  int max_parts = 0;
  int4* tasks_d = nullptr;
  int32_t* parts_d = nullptr;
  size_t tasks_cap = 0;
  int4* tasks_pin = nullptr;      // pinned staging of the uploads
  int32_t* parts_pin = nullptr;
  int32_t* zcnt_d = nullptr;      // [tasks_cap] zoomed spans of each span task in the last call
  int32_t* stat_pin = nullptr;    // pinned copy [tasks_cap]
  std::vector<int4> stat_tasks;   // the task table the copy in flight belongs to
  hipEvent_t ev = nullptr;        // recorded after the last statistics copy
  bool pending = false;
  uint64_t calls = 0, reads = 0;
  std::vector<double> est;        // zoomed spans per call, per row
  std::vector<double> est_plan;   // the estimates the current tables were planned from

  // Segment lists of the planned kernel (DEVICE bases, HOST bases read in
  // place): one list of at most wg_segments(G) segments per workgroup, cut from
  // the predicted cost of every row.  The prediction is the zoom mask of an
  // earlier call, read back without a sync.
  bool wvalid = false;
  std::vector<int4> wsegs;         // [n_wg * wg_segments(G)]
  int n_wg = 0;
  std::vector<int32_t> wparts;     // [B*Hkv] partial slots of each (sequence, kv head)
  int w_max_parts = 0;
  int4* wsegs_d = nullptr;
  int4* wsegs_pin = nullptr;
  size_t wsegs_cap = 0;
  int32_t* wparts_d = nullptr;
  int32_t* wparts_pin = nullptr;
  std::vector<int32_t> plan_m, plan_na;  // span and anchor counts the lists were cut for
  std::vector<float> zprob;              // [B*Hkv*m_max] zoom frequency (any head of the group), running mean
  std::vector<float> zunits;             // [B*Hkv] expected zoom units per row from zprob
  std::vector<float> zunits_plan;        // ... when the lists were cut
  int zsamples = 0;                      // masks seen
  uint8_t* mask_pin = nullptr;           // pinned copy of the last zoom mask [B*Hq*m_max]
  size_t mask_cap = 0;
  hipEvent_t mev = nullptr;              // recorded after that copy
  bool mpending = false;
  uint64_t plan_calls = 0;               // planned launches of the layer (mask sampling)
};

// Device cache of one layer's host-resident bases: a ring region of the
// context's cache; entries are placed in order and evicted oldest first.
struct CacheEntry {
  int64_t idx;   // (b * Hkv + g) * m_max + k
  int64_t off;   // region-relative element offset
  int64_t len;   // elements
  uint64_t batch;  // the prefetch that placed it
};
struct LayerCache {
  bool init = false;
  int64_t base = 0, size = 0;      // region [base, base + size) elements of the cache
  int64_t head = 0;                // next free position (region-relative)
  uint64_t batch = 0;              // prefetches so far
  std::deque<CacheEntry> fifo;     // resident entries, oldest first
  std::vector<int32_t> slot_h;     // [B*Hkv*m_max, rounded up to 4] (base + off) / 8, or -1
  int32_t* slot_d = nullptr;       // device copy read by the decode kernel
  int32_t* slot_pin = nullptr;     // coherent pinned staging of its updates (read by the copy kernel)
  int32_t* slot_hd = nullptr;      // its device-side address
  uint8_t* zm_pin = nullptr;       // [B*Hq*m_max] zoom mask of the last decode, written back by the combine kernel
  uint8_t* zm_hd = nullptr;        // its device-side address
  int4* runs_pin = nullptr;        // coherent: copy runs of the last prefetch (source, destination, length; / 8)
  int4* runs_hd = nullptr;         // its device-side address
  size_t runs_cap = 0;
  hipEvent_t ev_pref = nullptr;    // after the last prefetch (copies + table upload)
  hipEvent_t ev_done = nullptr;    // after the last decode of the layer
  bool zm_valid = false, pref_pending = false, done_valid = false;
  int64_t dirty_lo = INT64_MAX, dirty_hi = 0;  // slot entries changed since the last upload
};

struct LayerState {
  bool ready = false;      // every head has artefacts
  bool allocated = false;  // layout fixed, buffers allocated
  void* kbar = nullptr;
  void* vbar = nullptr;
  void* KA = nullptr;
  void* VA = nullptr;
  int32_t* rank_d = nullptr;
  int64_t* boff_d = nullptr;
  int2* smeta_d = nullptr;  // [B*Hkv*m_max] {boff / 8, rank | count << 8} for the decode kernels
  void* bases_d = nullptr;  // DEVICE home (and build scratch for HOST home)
  void* bases_h = nullptr;  // host homes: pinned store
  void* bases_hd = nullptr; // its device-side address (the kernels read it in place)
  int64_t basis_elems = 0;
  std::vector<int32_t> rank_h;     // [B*Hkv*m_max]
  std::vector<int64_t> boff_h;     // [B*Hkv*m_max], relative to the layer store
  std::vector<int64_t> head_base;  // [B*Hkv + 1]
  std::vector<uint8_t> head_set;   // [B*Hkv]
  void* Kr = nullptr;              // [B*Hkv*m_max][dr] routing summaries (with a routing projection)
  int na_cap = 0;                  // anchor rows per (b, g) in KA / VA (prefill anchors + appended tokens)
  std::vector<int32_t> na_l;       // [B] anchors of this layer per sequence (grows with appends)
  int32_t* na_l_d = nullptr;       // device copy
  std::vector<uint8_t> route_set;  // [B*Hkv] routing summaries present
  std::vector<int32_t> choices;    // rank choices and seed of its build (re-segmentation ranks)
  uint64_t seed = 0;
  LayerCache lc;                   // device cache of its host-resident bases
  LayerSched sched;
  unsigned long long* zcount_d = nullptr;  // [B*Hq + 1] zoom counters (spans per (b, h) over calls; calls)
};

// Routing projection of one layer (set before the layer's layout exists).
struct RouteProj {
  int dr = 0;            // 0: identity projection
  float* W_d = nullptr;  // [Hkv][dr][d]
};

}  // namespace

struct sekv_ctx {
  sekv_config cfg{};
  int G = 1;
  size_t esz = 4;
  bool bf16 = false;
  std::string err;

  // spans
  bool spans_ready = false;
  bool spans_built = false;
  double alpha = 0.0;
  // window re-segmentation (contexts whose span table came from sekv_build)
  int m_reserve = 0;                            // spare span rows per sequence
  std::vector<std::vector<float>> H_seq;        // [B] surprisal of every position so far
  std::vector<double> theta_b;                  // [B] the prefill's mu + alpha sigma
  std::vector<std::vector<int32_t>> row_pos;    // [B] positions of the anchor rows every layer holds
  std::vector<int32_t> next_pos;                // [B] position of the next appended row
  bool resegmented = false;
  int m_max = 0, na_max = 0;
  std::vector<int32_t> m_b, na_b;
  std::vector<std::vector<int32_t>> mstart, mcount, anchors;
  std::vector<uint8_t> pend;  // imported span tables pending per sequence
  int32_t* m_b_d = nullptr;
  int32_t* na_b_d = nullptr;
  int32_t* mstart_d = nullptr;
  int32_t* mcount_d = nullptr;
  int32_t* anchors_d = nullptr;
  float* logS_d = nullptr;
  int32_t* prob_d[5] = {nullptr, nullptr, nullptr, nullptr, nullptr};
  int n_prob[5] = {0, 0, 0, 0, 0};

  // build scratch
  int32_t* seg_i = nullptr;   // [4][B][n] flagpos, mstart, mcount, anchors
  int32_t* seg_counts = nullptr;
  double* seg_stats = nullptr;
  float* H_d_tmp = nullptr;

  std::vector<LayerState> layers;
  std::vector<RouteProj> route;  // per layer
  float* qp_d = nullptr;         // [B*Hq*d] projected queries

  // device cache of host-resident bases (HOST home), split evenly over the layers
  void* cache_d = nullptr;
  int64_t cache_elems = 0;

  // decode scratch
  float* part_ml = nullptr;
  float* part_acc = nullptr;
  size_t parts_cap = 0;  // partial slots

  uint8_t* mask_d = nullptr;    // [B*Hq*m_max] used when the caller passes no mask
  float* scores_d = nullptr;    // [B*Hq*m_max] routing scores for the budget cap
  size_t zcap = 0;              // spans capacity B*Hkv*m_max of the buffers above

  // HOST-home fetch path: flat list, staged items, groups per span task
  int4* zlist_d = nullptr;      // [B*Hkv*m_max] written by the attend kernel
  int32_t* zcounter_d = nullptr;
  int4* zlist_h = nullptr;      // pinned copy of the zoom list
  int32_t* zcount_h = nullptr;  // pinned
  int4* zitems_h = nullptr;     // pinned, sorted by (b, g, span)
  int4* zgroups_h = nullptr;    // pinned
  int4* zitems_d = nullptr;
  int4* zgroups_d = nullptr;
  int n_fetched = 0;            // items of the last fetch
  void* staging = nullptr;
  int64_t staging_cap = 0;      // elements
  hipStream_t side = nullptr;
  hipEvent_t ev_fetch = nullptr;
  // the copy list of a staged fetch (mapped pinned memory read by the copy
  // kernel), and an event after the last copy kernel that read it
  int4* fruns_pin = nullptr;
  int4* fruns_hd = nullptr;
  size_t fruns_cap = 0;
  hipEvent_t ev_runs = nullptr;
  bool runs_pending = false;
  std::vector<int4> fruns;      // host copy of the list being built

  sekv_stats stats{};
  int anchor_chunk = 256, span_chunk = 64;
  int fill_tasks = 768;           // route workgroups that fill the GPU once (three per CU)
  bool fill_fixed = false;        // fill_tasks given by the environment: used as is
};

namespace {

// The basis store lives in pinned host memory (read in place by the decode
// kernels, or copied to staging per step).
bool host_store(const sekv_ctx* c) {
  return c->cfg.basis_home == SEKV_BASES_HOST || c->cfg.basis_home == SEKV_BASES_HOST_STAGED;
}
bool staged(const sekv_ctx* c) { return c->cfg.basis_home == SEKV_BASES_HOST_STAGED; }

sekv_status fail(sekv_ctx* c, sekv_status s, const std::string& msg) {
  if (c) c->err = msg;
  else g_create_err = msg;
  return s;
}

#define HIPCHK(ctx, call)                                                                  \
  do {                                                                                     \
    hipError_t e_ = (call);                                                                \
    if (e_ != hipSuccess) {                                                                \
      (void)hipGetLastError();                                                             \
      return fail(ctx, e_ == hipErrorOutOfMemory ? SEKV_ERR_OOM : SEKV_ERR_HIP,            \
                  std::string(#call) + ": " + hipGetErrorString(e_));                      \
    }                                                                                      \
  } while (0)

#define TRY(x)                      \
  do {                              \
    sekv_status s_ = (x);           \
    if (s_ != SEKV_OK) return s_;   \
  } while (0)

struct DevGuard {
  int prev = -1;
  explicit DevGuard(int d) {
    if (hipGetDevice(&prev) == hipSuccess && prev != d) (void)hipSetDevice(d);
  }
  ~DevGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

template <typename P>
sekv_status dalloc(sekv_ctx* c, P** p, size_t bytes) {
  *p = nullptr;
  if (bytes == 0) bytes = 16;
  void* q = nullptr;
  hipError_t e = hipMalloc(&q, bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(c, e == hipErrorOutOfMemory ? SEKV_ERR_OOM : SEKV_ERR_HIP,
                "hipMalloc(" + std::to_string(bytes) + "): " + hipGetErrorString(e));
  }
  *p = static_cast<P*>(q);
  return SEKV_OK;
}

// Pinned host memory.  hipHostMallocCoherent where a kernel reads what the host
// rewrites between launches, or writes what the host reads: such accesses then
// bypass the GPU caches.
template <typename P>
sekv_status halloc(sekv_ctx* c, P** p, size_t bytes, unsigned flags = hipHostMallocDefault) {
  *p = nullptr;
  if (bytes == 0) bytes = 16;
  const char* f = std::getenv("SEKV_FAULT");
  if (f && std::strcmp(f, "pinned_oom") == 0)
    return fail(c, SEKV_ERR_OOM, "pinned host allocation refused (SEKV_FAULT=pinned_oom)");
  void* q = nullptr;
  hipError_t e = hipHostMalloc(&q, bytes, flags);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(c, SEKV_ERR_OOM, "hipHostMalloc(" + std::to_string(bytes) + "): " + hipGetErrorString(e));
  }
  *p = static_cast<P*>(q);
  return SEKV_OK;
}

template <typename P>
void dfree(P*& p) {
  if (p) (void)hipFree((void*)p);
  p = nullptr;
}
template <typename P>
void hfree(P*& p) {
  if (p) (void)hipHostFree((void*)p);
  p = nullptr;
}

void free_layer_cache(LayerCache& C) {
  dfree(C.slot_d);
  hfree(C.runs_pin);
  hfree(C.slot_pin);
  hfree(C.zm_pin);
  if (C.ev_pref) (void)hipEventDestroy(C.ev_pref);
  if (C.ev_done) (void)hipEventDestroy(C.ev_done);
  C = LayerCache();
}

// A layer's stored bases are about to change: drop its device cache, whose
// copies would go stale, once no decode and no prefetch copy that may read
// the store or the cache is still in flight.
hipError_t invalidate_layer_cache(LayerState& L) {
  if (!L.lc.init) return hipSuccess;
  const hipError_t e = hipDeviceSynchronize();
  free_layer_cache(L.lc);
  return e;
}

void free_layer(LayerState& L) {
  free_layer_cache(L.lc);
  dfree(L.kbar);
  dfree(L.vbar);
  dfree(L.KA);
  dfree(L.VA);
  dfree(L.rank_d);
  dfree(L.boff_d);
  dfree(L.smeta_d);
  dfree(L.bases_d);
  hfree(L.bases_h);
  dfree(L.Kr);
  dfree(L.na_l_d);
  dfree(L.sched.tasks_d);
  dfree(L.sched.parts_d);
  dfree(L.sched.zcnt_d);
  hfree(L.sched.tasks_pin);
  hfree(L.sched.parts_pin);
  hfree(L.sched.stat_pin);
  if (L.sched.ev) (void)hipEventDestroy(L.sched.ev);
  dfree(L.zcount_d);
  dfree(L.sched.wsegs_d);
  dfree(L.sched.wparts_d);
  hfree(L.sched.wsegs_pin);
  hfree(L.sched.wparts_pin);
  hfree(L.sched.mask_pin);
  if (L.sched.mev) (void)hipEventDestroy(L.sched.mev);
  L = LayerState();
}

// Elements of one span's packed bases: A_K^T [r][c8], B_K^T [r][d], A_V^T, B_V^T.
int64_t span_elems(int c, int r, int d) {
  return 2 * (int64_t)r * (pad8(c) + d);
}

// Install span tables (host vectors already filled); uploads device copies
// and the SVD problem buckets.
sekv_status install_spans(sekv_ctx* c) {
  const int B = c->cfg.batch, Hkv = c->cfg.n_kv_heads;
  c->m_b.assign(B, 0);
  c->na_b.assign(B, 0);
  int mm = 1, nm = 1;
  for (int b = 0; b < B; ++b) {
    c->m_b[b] = (int)c->mstart[b].size();
    c->na_b[b] = (int)c->anchors[b].size();
    mm = std::max(mm, c->m_b[b]);
    nm = std::max(nm, c->na_b[b]);
  }
  c->m_max = mm + c->m_reserve;  // the row stride of every per-span array
  mm = c->m_max;
  c->na_max = nm;
  dfree(c->m_b_d);
  dfree(c->na_b_d);
  dfree(c->mstart_d);
  dfree(c->mcount_d);
  dfree(c->anchors_d);
  dfree(c->logS_d);
  TRY(dalloc(c, &c->m_b_d, sizeof(int32_t) * B));
  TRY(dalloc(c, &c->na_b_d, sizeof(int32_t) * B));
  TRY(dalloc(c, &c->mstart_d, sizeof(int32_t) * B * mm));
  TRY(dalloc(c, &c->mcount_d, sizeof(int32_t) * B * mm));
  TRY(dalloc(c, &c->anchors_d, sizeof(int32_t) * B * nm));
  TRY(dalloc(c, &c->logS_d, sizeof(float) * B * mm));
  std::vector<int32_t> ms((size_t)B * mm, 0), mc((size_t)B * mm, 0), an((size_t)B * nm, 0);
  std::vector<float> ls((size_t)B * mm, 0.f);
  for (int b = 0; b < B; ++b) {
    for (int k = 0; k < c->m_b[b]; ++k) {
      ms[(size_t)b * mm + k] = c->mstart[b][k];
      mc[(size_t)b * mm + k] = c->mcount[b][k];
      ls[(size_t)b * mm + k] = (float)std::log((double)c->mcount[b][k]);
    }
    for (int i = 0; i < c->na_b[b]; ++i) an[(size_t)b * nm + i] = c->anchors[b][i];
  }
  HIPCHK(c, hipMemcpy(c->m_b_d, c->m_b.data(), sizeof(int32_t) * B, hipMemcpyHostToDevice));
  HIPCHK(c, hipMemcpy(c->na_b_d, c->na_b.data(), sizeof(int32_t) * B, hipMemcpyHostToDevice));
  HIPCHK(c, hipMemcpy(c->mstart_d, ms.data(), ms.size() * 4, hipMemcpyHostToDevice));
  HIPCHK(c, hipMemcpy(c->mcount_d, mc.data(), mc.size() * 4, hipMemcpyHostToDevice));
  HIPCHK(c, hipMemcpy(c->anchors_d, an.data(), an.size() * 4, hipMemcpyHostToDevice));
  HIPCHK(c, hipMemcpy(c->logS_d, ls.data(), ls.size() * 4, hipMemcpyHostToDevice));

  // SVD problem buckets by member count
  std::vector<int32_t> pr[5];
  for (int b = 0; b < B; ++b)
    for (int g = 0; g < Hkv; ++g)
      for (int k = 0; k < c->m_b[b]; ++k) {
        const int cnt = c->mcount[b][k];
        const int bk = cnt <= 16 ? 0 : cnt <= 32 ? 1 : cnt <= 64 ? 2 : cnt <= 128 ? 3 : 4;
        for (int w = 0; w < 2; ++w) {
          pr[bk].push_back(b * Hkv + g);
          pr[bk].push_back(k);
          pr[bk].push_back(w);
        }
      }
  for (int i = 0; i < 5; ++i) {
    dfree(c->prob_d[i]);
    c->n_prob[i] = (int)(pr[i].size() / 3);
    TRY(dalloc(c, &c->prob_d[i], pr[i].size() * 4));
    if (!pr[i].empty())
      HIPCHK(c, hipMemcpy(c->prob_d[i], pr[i].data(), pr[i].size() * 4, hipMemcpyHostToDevice));
  }
  c->spans_ready = true;
  return SEKV_OK;
}

// Fix the layout of a layer from per-(b, g, k) ranks and allocate its buffers.
sekv_status alloc_layer(sekv_ctx* c, int layer, const std::vector<int32_t>& rank) {
  const int B = c->cfg.batch, Hkv = c->cfg.n_kv_heads, d = c->cfg.d_head;
  LayerState& L = c->layers[layer];
  free_layer(L);
  const int mm = c->m_max, nm = c->na_max;
  L.rank_h = rank;
  L.boff_h.assign((size_t)B * Hkv * mm, 0);
  L.head_base.assign((size_t)B * Hkv + 1, 0);
  L.head_set.assign((size_t)B * Hkv, 0);
  int64_t off = 0;
  for (int b = 0; b < B; ++b)
    for (int g = 0; g < Hkv; ++g) {
      const size_t bg = (size_t)b * Hkv + g;
      L.head_base[bg] = off;
      for (int k = 0; k < c->m_b[b]; ++k) {
        L.boff_h[bg * mm + k] = off;
        off += span_elems(c->mcount[b][k], rank[bg * mm + k], d);
      }
    }
  L.head_base[(size_t)B * Hkv] = off;
  L.basis_elems = off;
  if ((off >> 3) >= ((int64_t)1 << 32))
    return fail(c, SEKV_ERR_INVALID, "basis store of one layer exceeds 2^35 elements");
  L.na_cap = nm;
  L.na_l = c->na_b;
  const size_t rows_m = (size_t)B * Hkv * mm, rows_a = (size_t)B * Hkv * nm;
  TRY(dalloc(c, &L.kbar, rows_m * d * c->esz));
  TRY(dalloc(c, &L.vbar, rows_m * d * c->esz));
  TRY(dalloc(c, &L.KA, rows_a * d * c->esz));
  TRY(dalloc(c, &L.VA, rows_a * d * c->esz));
  TRY(dalloc(c, &L.rank_d, rows_m * 4));
  TRY(dalloc(c, &L.boff_d, rows_m * 8));
  TRY(dalloc(c, &L.smeta_d, rows_m * sizeof(int2)));
  TRY(dalloc(c, &L.na_l_d, (size_t)B * sizeof(int32_t)));
  HIPCHK(c, hipMemcpy(L.na_l_d, L.na_l.data(), (size_t)B * sizeof(int32_t), hipMemcpyHostToDevice));
  {
    const size_t nz = (size_t)B * c->cfg.n_q_heads + 1;
    TRY(dalloc(c, &L.zcount_d, nz * sizeof(unsigned long long)));
    HIPCHK(c, hipMemset(L.zcount_d, 0, nz * sizeof(unsigned long long)));
  }

  HIPCHK(c, hipEventCreateWithFlags(&L.sched.ev, hipEventDisableTiming));
  HIPCHK(c, hipEventCreateWithFlags(&L.sched.mev, hipEventDisableTiming));
  L.sched.est.assign((size_t)B * Hkv, 0.0);
  HIPCHK(c, hipMemset(L.kbar, 0, rows_m * d * c->esz));
  HIPCHK(c, hipMemset(L.vbar, 0, rows_m * d * c->esz));
  HIPCHK(c, hipMemset(L.KA, 0, rows_a * d * c->esz));
  HIPCHK(c, hipMemset(L.VA, 0, rows_a * d * c->esz));
  HIPCHK(c, hipMemcpy(L.rank_d, L.rank_h.data(), rows_m * 4, hipMemcpyHostToDevice));
  HIPCHK(c, hipMemcpy(L.boff_d, L.boff_h.data(), rows_m * 8, hipMemcpyHostToDevice));
  {
    std::vector<int2> meta(rows_m, make_int2(0, 0));
    for (int b = 0; b < B; ++b)
      for (int g = 0; g < Hkv; ++g)
        for (int k = 0; k < c->m_b[b]; ++k) {
          const size_t i = ((size_t)b * Hkv + g) * mm + k;
          meta[i] = make_int2((int)(uint32_t)(L.boff_h[i] >> 3), L.rank_h[i] | (c->mcount[b][k] << 8));
        }
    HIPCHK(c, hipMemcpy(L.smeta_d, meta.data(), rows_m * sizeof(int2), hipMemcpyHostToDevice));
  }
  TRY(dalloc(c, &L.bases_d, (size_t)off * c->esz));
  if (host_store(c)) {
    TRY(halloc(c, &L.bases_h, (size_t)off * c->esz));
    HIPCHK(c, hipHostGetDevicePointer(&L.bases_hd, L.bases_h, 0));
  }
  const int dr = c->route[layer].dr;
  L.route_set.assign((size_t)B * Hkv, dr > 0 ? 0 : 1);
  if (dr > 0) {
    TRY(dalloc(c, &L.Kr, rows_m * dr * c->esz));
    HIPCHK(c, hipMemset(L.Kr, 0, rows_m * dr * c->esz));
  }
  L.allocated = true;
  return SEKV_OK;
}

// A layer decodes once every (b, g) has its artefacts (and routing summaries).
void update_ready(LayerState& L) {
  auto all = [](const std::vector<uint8_t>& v) {
    return std::all_of(v.begin(), v.end(), [](uint8_t x) { return x != 0; });
  };
  L.ready = L.allocated && all(L.head_set) && all(L.route_set);
}

sekv_status ensure_parts(sekv_ctx* c, size_t slots) {
  if (slots <= c->parts_cap) return SEKV_OK;
  dfree(c->part_ml);
  dfree(c->part_acc);
  c->parts_cap = 0;
  TRY(dalloc(c, &c->part_ml, slots * 4 * sizeof(float)));
  TRY(dalloc(c, &c->part_acc, slots * c->cfg.d_head * sizeof(float)));
  c->parts_cap = slots;
  return SEKV_OK;
}

sekv_status ensure_zoom_buffers(sekv_ctx* c) {
  const size_t spans = (size_t)c->cfg.batch * c->cfg.n_kv_heads * c->m_max;
  if (spans <= c->zcap && c->mask_d) return SEKV_OK;
  dfree(c->mask_d);
  dfree(c->zlist_d);
  dfree(c->zitems_d);
  dfree(c->zgroups_d);
  hfree(c->zlist_h);
  hfree(c->zitems_h);
  hfree(c->zgroups_h);
  c->zcap = 0;
  dfree(c->scores_d);
  TRY(dalloc(c, &c->mask_d, spans * c->G));
  TRY(dalloc(c, &c->scores_d, spans * c->G * sizeof(float)));
  if (host_store(c)) {  // sekv_zoom_fetch works for both host homes
    TRY(dalloc(c, &c->zlist_d, spans * sizeof(int4)));
    TRY(dalloc(c, &c->zitems_d, spans * sizeof(int4)));
    TRY(dalloc(c, &c->zgroups_d, spans * sizeof(int4)));
    TRY(halloc(c, &c->zlist_h, spans * sizeof(int4)));
    TRY(halloc(c, &c->zitems_h, spans * sizeof(int4)));
    TRY(halloc(c, &c->zgroups_h, spans * sizeof(int4)));
  }
  c->zcap = spans;
  return SEKV_OK;
}

// Copy the bases of the listed spans (items: bg | head bits << 24, span id)
// from the pinned store into staging on `side`, runs of adjacent spans
// coalesced, and upload the item list sorted by (bg, span) with each item's
// staging offset / 8 and rank | count << 8.  `groups` (optional, host) gets
// one (span task, first item, items) per span task of the layer's schedule
// holding listed spans; their upload follows the items.
sekv_status fetch_items(sekv_ctx* c, int layer, const int4* items, int count, hipStream_t side,
                        hipEvent_t done, int* n_groups) {
  LayerState& L = c->layers[layer];
  const int Hkv = c->cfg.n_kv_heads, d = c->cfg.d_head, mm = c->m_max;
  int4* z = c->zitems_h;
  if (items != z) std::memcpy(z, items, (size_t)count * sizeof(int4));
  std::sort(z, z + count, [](const int4& x, const int4& y) {
    const int bx = x.x & 0xffffff, by = y.x & 0xffffff;
    return bx != by ? bx < by : x.y < y.y;
  });
  int64_t need = 0;
  for (int i = 0; i < count; ++i) {
    const int bg = z[i].x & 0xffffff, k = z[i].y, b = bg / Hkv;
    if (bg >= c->cfg.batch * Hkv || k < 0 || k >= c->m_b[b])
      return fail(c, SEKV_ERR_INVALID, "zoom entry out of range");
    if (i > 0 && bg == (z[i - 1].x & 0xffffff) && k == z[i - 1].y)
      return fail(c, SEKV_ERR_INVALID, "zoom entry: duplicate span");
    z[i].w = L.rank_h[(size_t)bg * mm + k] | (c->mcount[b][k] << 8);
    need += span_elems(c->mcount[b][k], L.rank_h[(size_t)bg * mm + k], d);
  }
  if ((need >> 3) >= ((int64_t)1 << 31)) return fail(c, SEKV_ERR_INVALID, "zoomed bases exceed the staging limit");
  if (need > c->staging_cap) {
    dfree(c->staging);
    c->staging_cap = 0;
    const int64_t cap = std::max<int64_t>(need, std::min<int64_t>(L.basis_elems, need * 2));
    TRY(dalloc(c, &c->staging, (size_t)cap * c->esz));
    c->staging_cap = cap;
  }
  const char* f = std::getenv("SEKV_FAULT");
  if (f && std::strcmp(f, "fetch") == 0) return fail(c, SEKV_ERR_HIP, "fetch failure forced (SEKV_FAULT=fetch)");
  // the copy list: runs of adjacent spans, cut into pieces of at most
  // kFetchPiece elements (one copy workgroup each); offsets and lengths in
  // units of 8 elements (every span's element count is a multiple of 16)
  constexpr int64_t kFetchPiece = 32768;
  std::vector<int4>& runs = c->fruns;
  runs.clear();
  int64_t pos = 0, run_src = -1, run_dst = 0, run_len = 0;
  auto flush = [&]() {
    for (int64_t o = 0; o < run_len; o += kFetchPiece) {
      const int64_t len = std::min(kFetchPiece, run_len - o);
      runs.push_back(make_int4((int)(uint32_t)((run_src + o) >> 3), (int)(uint32_t)((run_dst + o) >> 3),
                               (int)(len >> 3), 0));
    }
  };
  for (int i = 0; i <= count; ++i) {
    int64_t off = -1, sz = 0;
    if (i < count) {
      const int bg = z[i].x & 0xffffff, k = z[i].y;
      off = L.boff_h[(size_t)bg * mm + k];
      sz = span_elems(c->mcount[bg / Hkv][k], L.rank_h[(size_t)bg * mm + k], d);
      z[i].z = (int)(pos >> 3);
    }
    if (i < count && run_src >= 0 && off == run_src + run_len) {
      run_len += sz;
    } else {
      if (run_src >= 0) flush();
      run_src = off;
      run_dst = pos;
      run_len = sz;
    }
    pos += sz;
  }
  if (!runs.empty()) {
    // the previous list is free once the copy kernel that read it is done
    if (c->runs_pending) HIPCHK(c, hipEventSynchronize(c->ev_runs));
    c->runs_pending = false;
    if (runs.size() > c->fruns_cap) {
      const size_t cap = std::max<size_t>(runs.size(), 2 * c->fruns_cap + 256);
      hfree(c->fruns_pin);
      c->fruns_cap = 0;
      TRY(halloc(c, &c->fruns_pin, cap * sizeof(int4), hipHostMallocCoherent));
      HIPCHK(c, hipHostGetDevicePointer((void**)&c->fruns_hd, c->fruns_pin, 0));
      c->fruns_cap = cap;
    }
    std::memcpy(c->fruns_pin, runs.data(), runs.size() * sizeof(int4));
    // one launch on `side`: every piece from the mapped pinned store into staging
    launch_copy_runs(c->fruns_hd, (int)runs.size(), L.bases_hd, c->staging, (int)c->esz, nullptr, nullptr, 0, side);
    HIPCHK(c, hipGetLastError());
    HIPCHK(c, hipEventRecord(c->ev_runs, side));
    c->runs_pending = true;
  }
  const uint64_t ncopies = runs.empty() ? 0 : 1;
  if (count) HIPCHK(c, hipMemcpyAsync(c->zitems_d, z, (size_t)count * sizeof(int4), hipMemcpyHostToDevice, side));
  if (n_groups) {
    const LayerSched& S = L.sched;
    int ng = 0;
    for (int i = 0; i < count;) {
      const int bg = z[i].x & 0xffffff;
      const int t = S.first_span_task[bg] + z[i].y / S.chunk[bg];
      int j = i + 1;
      while (j < count && (z[j].x & 0xffffff) == bg && S.first_span_task[bg] + z[j].y / S.chunk[bg] == t) ++j;
      c->zgroups_h[ng++] = make_int4(t, i, j - i, 0);
      i = j;
    }
    if (ng) HIPCHK(c, hipMemcpyAsync(c->zgroups_d, c->zgroups_h, (size_t)ng * sizeof(int4), hipMemcpyHostToDevice, side));
    *n_groups = ng;
  }
  if (done) HIPCHK(c, hipEventRecord(done, side));
  c->n_fetched = count;
  c->stats.fetch_calls++;
  c->stats.spans_fetched += count;
  c->stats.bytes_fetched += (uint64_t)pos * c->esz;
  c->stats.memcpy_calls += ncopies;
  return SEKV_OK;
}

// Task table of a layer from the per-row zoom estimates.
void plan_tasks(sekv_ctx* c, LayerState& L) {
  LayerSched& S = L.sched;
  const int B = c->cfg.batch, Hkv = c->cfg.n_kv_heads, BH = B * Hkv;
  int base = std::min(kMaxSpanChunk, env_int("SEKV_SPAN_CHUNK", c->span_chunk, 16, kMaxSpanChunk));
  int ach = env_int("SEKV_ANCHOR_CHUNK", c->anchor_chunk, 16, 1 << 20);
  // small layers: halve the chunks (spans down to 32 rows, anchors down to 64)
  // while the tasks would not fill the GPU once
  for (;;) {
    int64_t total = 0;
    for (int bg = 0; bg < BH; ++bg)
      total += (c->m_b[bg / Hkv] + base - 1) / base + (L.na_l[bg / Hkv] + ach - 1) / ach;
    if (total >= c->fill_tasks || (base <= 32 && ach <= 64)) break;
    if (base > 32) base /= 2;
    if (ach > 64) ach /= 2;
  }
  const double zpw = env_int("SEKV_ZOOM_PER_TASK", 4, 1, 256);
  // a span task folds its zoomed spans into its one slot; with staged bases
  // they go to its second slot (written by the attend kernel)
  const int per_span = staged(c) ? 2 : 1;
  S.chunk.assign(BH, base);
  S.parts_n.assign(BH, 0);
  S.first_span_task.assign(BH, 0);
  std::vector<int> nspan(BH), nanch(BH), anch(BH, ach);
  std::vector<std::pair<double, int>> order;
  for (int bg = 0; bg < BH; ++bg) {
    const int m = c->m_b[bg / Hkv], na = L.na_l[bg / Hkv];
    int n = (m + base - 1) / base;
    n = std::max(n, (int)std::ceil(S.est[bg] / zpw));
    n = std::max(1, std::min(n, std::max(1, (m + 15) / 16)));
    int ch = m > 0 ? ((m + n - 1) / n + 15) / 16 * 16 : 16;
    int a = ach;
    auto parts = [&]() { return per_span * ((m + ch - 1) / ch) + (na + a - 1) / a; };
    while (parts() > kMaxParts) {
      if (ch < kMaxSpanChunk) ch = std::min(kMaxSpanChunk, ch * 2);
      else a *= 2;
    }
    S.chunk[bg] = ch;
    anch[bg] = a;
    nspan[bg] = m > 0 ? (m + ch - 1) / ch : 0;
    nanch[bg] = (na + a - 1) / a;
    S.parts_n[bg] = per_span * nspan[bg] + nanch[bg];
    order.push_back({-(S.est[bg] / std::max(1, nspan[bg])), bg});
  }
  std::stable_sort(order.begin(), order.end());
  S.tasks.clear();
  S.max_parts = 1;
  for (int bg = 0; bg < BH; ++bg) S.max_parts = std::max(S.max_parts, S.parts_n[bg]);
  for (auto& o : order) {  // span chunks, the most zoom-heavy rows first
    const int bg = o.second;
    S.first_span_task[bg] = (int)S.tasks.size();
    // task lengths are clamped to the row's span count: the kernels read no count
    const int m = c->m_b[bg / Hkv];
    for (int j = 0; j < nspan[bg]; ++j) {
      const int k0 = j * S.chunk[bg];
      S.tasks.push_back(make_int4(bg, k0, std::min(S.chunk[bg], m - k0), per_span * j));
    }
  }
  S.n_span_tasks = (int)S.tasks.size();
  int amax = 0;
  for (int bg = 0; bg < BH; ++bg) amax = std::max(amax, nanch[bg]);
  for (int j = 0; j < amax; ++j)  // anchor chunks, interleaved over the rows
    for (int bg = 0; bg < BH; ++bg)
      if (j < nanch[bg])
        S.tasks.push_back(make_int4(bg | (int)0x80000000u, j * anch[bg],
                                    std::min(anch[bg], L.na_l[bg / Hkv] - j * anch[bg]),
                                    per_span * nspan[bg] + j));
}

// Refresh a layer's schedule before a launch on `stream`.  `pending` means a
// statistics copy (and any table upload queued before it) is in flight, with
// S.ev recorded after it.  When that event has completed the counts are read,
// the per-row estimates updated and the tables replanned; new tables are
// uploaded from pinned staging that no copy in flight still reads.  While the
// stream is being captured into a graph nothing changes and nothing is copied.
sekv_status prepare_sched(sekv_ctx* c, int layer, hipStream_t stream, bool* capturing) {
  LayerSched& S = c->layers[layer].sched;
  const int BH = c->cfg.batch * c->cfg.n_kv_heads;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  HIPCHK(c, hipStreamIsCapturing(stream, &cs));
  *capturing = cs != hipStreamCaptureStatusNone;
  if (*capturing) {
    if (!S.valid) return fail(c, SEKV_ERR_STATE, "decode a layer once before capturing it into a graph");
    return SEKV_OK;
  }
  bool replan = !S.valid;
  if (S.pending && hipEventQuery(S.ev) == hipSuccess) {
    // zoomed spans per (sequence, kv head) in the call the copy followed
    S.pending = false;
    std::vector<double> per(BH, 0.0);
    for (size_t t = 0; t < S.stat_tasks.size(); ++t)
      if (S.stat_tasks[t].x >= 0) per[S.stat_tasks[t].x] += S.stat_pin[t];
    for (int bg = 0; bg < BH; ++bg) S.est[bg] = S.reads == 0 ? per[bg] : 0.5 * S.est[bg] + 0.5 * per[bg];
    S.reads++;
    // replan only when some row's zoom load moved by more than a quarter (and
    // one span): steady zoom rates keep the tables, and with them the order of
    // the merges, from call to call
    for (int bg = 0; bg < BH && !replan; ++bg) {
      const double p0 = bg < (int)S.est_plan.size() ? S.est_plan[bg] : 0.0;
      replan = std::fabs(S.est[bg] - p0) > 0.25 * p0 + 1.0;
    }
  }
  if (S.anchors_changed) {
    // appended tokens: the anchor tasks must cover them from this launch on
    if (S.pending) {
      HIPCHK(c, hipEventSynchronize(S.ev));
      S.pending = false;  // those counts are dropped; the next call measures again
    }
    S.anchors_changed = false;
    replan = true;
  }
  if (!replan || S.pending) return SEKV_OK;
  const std::vector<int4> old_tasks = S.tasks;
  plan_tasks(c, c->layers[layer]);
  S.est_plan = S.est;
  // the slot counts follow from the tasks: both tables change together
  if (S.valid && old_tasks.size() == S.tasks.size() &&
      std::memcmp(old_tasks.data(), S.tasks.data(), S.tasks.size() * sizeof(int4)) == 0)
    return SEKV_OK;
  const size_t nrec = S.tasks.size();
  if (nrec > S.tasks_cap) {
    dfree(S.tasks_d);
    dfree(S.zcnt_d);
    hfree(S.tasks_pin);
    hfree(S.stat_pin);
    S.tasks_cap = 0;
    TRY(dalloc(c, &S.tasks_d, nrec * sizeof(int4)));
    TRY(dalloc(c, &S.zcnt_d, nrec * sizeof(int32_t)));
    TRY(halloc(c, &S.tasks_pin, nrec * sizeof(int4)));
    TRY(halloc(c, &S.stat_pin, nrec * sizeof(int32_t)));
    S.tasks_cap = nrec;
  }
  if (!S.parts_d) {
    TRY(dalloc(c, &S.parts_d, (size_t)BH * 4));
    TRY(halloc(c, &S.parts_pin, (size_t)BH * 4));
  }
  std::memcpy(S.tasks_pin, S.tasks.data(), S.tasks.size() * sizeof(int4));
  std::memcpy(S.parts_pin, S.parts_n.data(), (size_t)BH * 4);
  HIPCHK(c, hipMemcpyAsync(S.tasks_d, S.tasks_pin, nrec * sizeof(int4), hipMemcpyHostToDevice, stream));
  HIPCHK(c, hipMemcpyAsync(S.parts_d, S.parts_pin, (size_t)BH * 4, hipMemcpyHostToDevice, stream));
  S.valid = true;
  return SEKV_OK;
}

// After the kernels of a call: start a statistics copy if none is in flight.
sekv_status finish_sched(sekv_ctx* c, int layer, hipStream_t stream, bool capturing) {
  LayerSched& S = c->layers[layer].sched;
  if (capturing) return SEKV_OK;
  S.calls++;
  if (S.pending || S.n_span_tasks == 0) return SEKV_OK;
  HIPCHK(c, hipMemcpyAsync(S.stat_pin, S.zcnt_d, (size_t)S.n_span_tasks * 4, hipMemcpyDeviceToHost, stream));
  HIPCHK(c, hipEventRecord(S.ev, stream));
  S.stat_tasks.assign(S.tasks.begin(), S.tasks.begin() + S.n_span_tasks);
  S.pending = true;
  return SEKV_OK;
}

// Inputs of the planner (plan.h) for one layer: the span table, ranks and
// zoom frequencies, and the cost knobs (environment overrides for tuning:
// SEKV_SPAN_COST in percent of an anchor row, SEKV_UNIT_COST in bytes,
// SEKV_ZOOM_DEV in hundredths).  The costs were tuned on the 128K benchmark
// layer: a span row, which also routes, takes about twice as long as an anchor
// row, and a token-tile unit costs its bases plus 12 KB for its dependent
// round of loads.  `cnt` holds the per-sequence span-count pointers.
PlanInput plan_input(sekv_ctx* c, LayerState& L, std::vector<const int32_t*>& cnt) {
  LayerSched& S = L.sched;
  const int B = c->cfg.batch;
  cnt.resize(B);
  for (int b = 0; b < B; ++b) cnt[b] = c->mcount[b].data();
  PlanInput in;
  in.B = B;
  in.Hkv = c->cfg.n_kv_heads;
  in.d = c->cfg.d_head;
  in.esz = c->esz;
  in.m_max = c->m_max;
  in.segs_per_share = wg_segments(c->G);
  in.max_span_rows = kMaxWgSpanRows;
  in.max_parts = kMaxParts;
  in.m = c->m_b.data();
  in.na = L.na_l.data();
  in.count = cnt.data();
  in.rank = L.rank_h.data();
  in.zprob = S.zprob.data();
  in.zunits = S.zunits.empty() ? nullptr : S.zunits.data();
  in.span_cost = env_int("SEKV_SPAN_COST", 200, 50, 1000) / 100.0;
  in.unit_cost = env_int("SEKV_UNIT_COST", 12288, 0, 1 << 24);
  in.zdev = env_int("SEKV_ZOOM_DEV", 150, 0, 1000) / 100.0;
  return in;
}

// Refresh the segment lists of a layer before a planned launch on `stream`
// (see prepare_sched for the protocol: nothing changes during a capture, and
// the lists are replaced only when no mask copy is in flight).
sekv_status prepare_plan(sekv_ctx* c, int layer, hipStream_t stream, bool capturing) {
  LayerState& L = c->layers[layer];
  LayerSched& S = L.sched;
  const int B = c->cfg.batch, Hkv = c->cfg.n_kv_heads, Hq = c->cfg.n_q_heads, BH = B * Hkv, G = c->G;
  const int d = c->cfg.d_head, mm = c->m_max;
  const size_t rows = (size_t)BH * mm;
  if (capturing) {
    if (!S.wvalid) return fail(c, SEKV_ERR_STATE, "decode a layer once before capturing it into a graph");
    return SEKV_OK;
  }
  bool replan = !S.wvalid || S.plan_m != c->m_b || S.plan_na != L.na_l || S.zprob.size() != rows;
  if (S.zprob.size() != rows) {
    S.zprob.assign(rows, 0.f);
    S.zsamples = 0;
  }
  if (S.mpending && hipEventQuery(S.mev) == hipSuccess) {
    // the zoom mask of an earlier call (union over each group's heads) into
    // the running zoom frequency of every span: the mean of the first masks,
    // then an exponential average
    S.mpending = false;
    const float w = 1.f / (float)std::min(S.zsamples + 1, 8);
    S.zsamples++;
    S.zunits.assign(BH, 0.f);
    for (int b = 0; b < B; ++b)
      for (int g = 0; g < Hkv; ++g) {
        float eu = 0.f;
        for (int k = 0; k < c->m_b[b]; ++k) {
          uint8_t z = 0;
          for (int h = g * G; h < (g + 1) * G; ++h) z |= S.mask_pin[((size_t)b * Hq + h) * mm + k] ? 1 : 0;
          float& p = S.zprob[((size_t)b * Hkv + g) * mm + k];
          p += w * ((float)z - p);
          eu += p * (float)((c->mcount[b][k] + d - 1) / d);
        }
        S.zunits[b * Hkv + g] = eu;
      }
    // replan while the frequencies settle, then only when the expected zoom
    // work of the rows moved: steady zoom keeps the lists, and with them the
    // order of the merges, from call to call
    double moved = 0.0, tot = 0.0;
    for (int bg = 0; bg < BH; ++bg) {
      const double p0 = bg < (int)S.zunits_plan.size() ? S.zunits_plan[bg] : 0.0;
      moved += std::fabs(S.zunits[bg] - p0);
      tot += p0;
    }
    replan |= S.zsamples <= 4 || moved > 0.15 * tot + 2.0;
  }
  if (!replan || S.mpending) return SEKV_OK;
  // the smallest budget that cuts the work into at most the target number of
  // shares: one wave of workgroups, three per CU, or two for large one-head
  // layers (measured on MI355X: the 128K layers of 32 heads take 33.9 against
  // 34.8 us per layer-step at two per CU; the 32K layer and the grouped-query
  // batch are faster at three)
  std::vector<const int32_t*> cnt;
  PlanInput in = plan_input(c, L, cnt);
  int nw = c->fill_tasks;
  if (!c->fill_fixed && c->G == 1 && plan_expected_bytes(in) > 64e6) {
    nw = c->fill_tasks * 2 / 3;
    // and half the cushion of zoom work per share: 32.1 against 32.4 us per
    // 128K layer-step (0.5 to 1 standard deviation: 32.1 to 32.2 us; 0 and 3:
    // 32.4 and 33.2 us); the grouped-query batch is 3 to 5% slower with it
    in.zdev = env_int("SEKV_ZOOM_DEV", 75, 0, 1000) / 100.0;
  }
  PlanOut po;
  plan_shares(in, nw, &po);
  S.wsegs.resize(po.segs.size());
  for (size_t i = 0; i < po.segs.size(); ++i)
    S.wsegs[i] = make_int4(po.segs[i].x, po.segs[i].y, po.segs[i].z, po.segs[i].w);
  S.wparts.swap(po.parts);
  S.n_wg = po.n_shares;
  S.w_max_parts = po.max_parts;
  if (S.w_max_parts > kMaxParts) return fail(c, SEKV_ERR_STATE, "too many partial slots per head");
  S.zunits_plan = S.zunits;
  S.plan_m = c->m_b;
  S.plan_na = L.na_l;
  const size_t nrec = S.wsegs.size();
  if (nrec > S.wsegs_cap) {
    dfree(S.wsegs_d);
    hfree(S.wsegs_pin);
    S.wsegs_cap = 0;
    TRY(dalloc(c, &S.wsegs_d, nrec * sizeof(int4)));
    TRY(halloc(c, &S.wsegs_pin, nrec * sizeof(int4)));
    S.wsegs_cap = nrec;
  }
  if (!S.wparts_d) {
    TRY(dalloc(c, &S.wparts_d, (size_t)BH * 4));
    TRY(halloc(c, &S.wparts_pin, (size_t)BH * 4));
  }
  std::memcpy(S.wsegs_pin, S.wsegs.data(), nrec * sizeof(int4));
  std::memcpy(S.wparts_pin, S.wparts.data(), (size_t)BH * 4);
  HIPCHK(c, hipMemcpyAsync(S.wsegs_d, S.wsegs_pin, nrec * sizeof(int4), hipMemcpyHostToDevice, stream));
  HIPCHK(c, hipMemcpyAsync(S.wparts_d, S.wparts_pin, (size_t)BH * 4, hipMemcpyHostToDevice, stream));
  S.wvalid = true;
  return SEKV_OK;
}

// After a planned launch: copy the zoom mask back for the next plan, if no
// copy is in flight.
sekv_status finish_plan(sekv_ctx* c, int layer, const uint8_t* mask, hipStream_t stream, bool capturing) {
  LayerSched& S = c->layers[layer].sched;
  if (capturing) return SEKV_OK;
  // every call while the frequencies settle, then one call in eight: the
  // readback and the update of the frequencies are host work on every eager call
  const uint64_t k = S.plan_calls++;
  if (S.mpending || (S.zsamples > 4 && k % 8 != 0)) return SEKV_OK;
  const size_t n = (size_t)c->cfg.batch * c->cfg.n_q_heads * c->m_max;
  if (n > S.mask_cap) {
    hfree(S.mask_pin);
    S.mask_cap = 0;
    TRY(halloc(c, &S.mask_pin, n));
    S.mask_cap = n;
  }
  HIPCHK(c, hipMemcpyAsync(S.mask_pin, mask, n, hipMemcpyDeviceToHost, stream));
  HIPCHK(c, hipEventRecord(S.mev, stream));
  S.mpending = true;
  return SEKV_OK;
}

sekv_status check_layer(sekv_ctx* c, int layer) {
  if (layer < 0 || layer >= c->cfg.n_layers)
    return fail(c, SEKV_ERR_INVALID, "layer " + std::to_string(layer) + " out of range");
  if (!c->spans_ready) return fail(c, SEKV_ERR_STATE, "no span table: build or import first");
  if (!c->layers[layer].ready)
    return fail(c, SEKV_ERR_STATE, "layer " + std::to_string(layer) + " has no artefacts");
  return SEKV_OK;
}

// ---------------------------------------------------------------------------- basis cache

sekv_status ensure_layer_cache(sekv_ctx* c, int layer) {
  LayerState& L = c->layers[layer];
  LayerCache& C = L.lc;
  if (C.init) return SEKV_OK;
  const int B = c->cfg.batch, Hkv = c->cfg.n_kv_heads, Hq = c->cfg.n_q_heads, L_ = c->cfg.n_layers;
  const size_t rows = (size_t)B * Hkv * c->m_max;
  C.size = (c->cache_elems / L_) & ~int64_t(7);
  C.base = C.size * layer;
  C.head = 0;
  const size_t rows4 = (rows + 3) & ~size_t(3);  // the slot table moves in 16-byte pieces
  C.slot_h.assign(rows4, -1);
  TRY(dalloc(c, &C.slot_d, rows4 * 4));
  TRY(halloc(c, &C.slot_pin, rows4 * 4, hipHostMallocCoherent));
  TRY(halloc(c, &C.zm_pin, (size_t)B * Hq * c->m_max + 8, hipHostMallocCoherent));  // + 8: the scan reads whole words
  HIPCHK(c, hipHostGetDevicePointer((void**)&C.slot_hd, C.slot_pin, 0));
  HIPCHK(c, hipHostGetDevicePointer((void**)&C.zm_hd, C.zm_pin, 0));
  HIPCHK(c, hipMemset(C.slot_d, 0xff, rows4 * 4));
  HIPCHK(c, hipEventCreateWithFlags(&C.ev_pref, hipEventDisableTiming));
  HIPCHK(c, hipEventCreateWithFlags(&C.ev_done, hipEventDisableTiming));
  C.init = true;
  return SEKV_OK;
}

// Place `len` elements in the ring, evicting the oldest entries it overlaps.
// An entry placed by the same prefetch is never evicted: all of a prefetch's
// copies run at once, so its destinations must not overlap.  Then the span is
// not placed (and is read from the host store).
bool cache_place(LayerCache& C, int64_t len, int64_t* off) {
  if (len > C.size) return false;
  auto evict = [&](int64_t lo, int64_t hi) -> bool {
    while (!C.fifo.empty()) {
      const CacheEntry& f = C.fifo.front();
      if (!(f.off < hi && f.off + f.len > lo)) break;
      if (f.batch == C.batch) return false;
      C.slot_h[f.idx] = -1;
      C.dirty_lo = std::min(C.dirty_lo, f.idx);
      C.dirty_hi = std::max(C.dirty_hi, f.idx + 1);
      C.fifo.pop_front();
    }
    return true;
  };
  int64_t at = C.head;
  if (at + len > C.size) {
    if (!evict(at, C.size)) return false;
    at = 0;
  }
  if (!evict(at, at + len)) return false;
  *off = at;
  C.head = at + len;
  return true;
}

// Elements per piece of a cache fill copy (a multiple of 8).
constexpr int64_t kCopyPiece = 16384;

// Predictive prefetch for `layer` (called while an earlier layer is being
// decoded): the spans its last decode zoomed (any head of the group) are
// expected again at its next decode; those not cached are copied from the
// pinned store into its region on the side stream, then the slot table is
// uploaded.  Its next decode waits for ev_pref.  Entries are evicted only after
// the layer's previous decode has finished (ev_done).
sekv_status cache_prefetch(sekv_ctx* c, int layer) {
  LayerState& L = c->layers[layer];
  LayerCache& C = L.lc;
  if (!C.init || !L.ready || !C.zm_valid || C.size == 0) return SEKV_OK;
  // the layer's last decode is done: its zoom mask is back (no prediction
  // otherwise), and entries can be evicted
  if (hipEventQuery(C.ev_done) != hipSuccess) return SEKV_OK;
  C.zm_valid = false;
  const int B = c->cfg.batch, Hkv = c->cfg.n_kv_heads, Hq = c->cfg.n_q_heads, G = c->G, mm = c->m_max;
  const int d = c->cfg.d_head;
  std::vector<int64_t> need;
  std::vector<uint64_t> un((mm + 7) / 8);
  for (int b = 0; b < B; ++b)
    for (int g = 0; g < Hkv; ++g) {
      const size_t bg = (size_t)b * Hkv + g;
      const int m = c->m_b[b];
      const int nw = (m + 7) / 8;
      // union of the group's mask rows, eight spans per word (bytes beyond m are masked off)
      for (int w = 0; w < nw; ++w) {
        uint64_t x = 0;
        for (int h = 0; h < G; ++h) {
          uint64_t y;
          std::memcpy(&y, C.zm_pin + ((size_t)b * Hq + g * G + h) * mm + (size_t)w * 8, 8);
          x |= y;
        }
        const int left = m - w * 8;
        if (left < 8) x &= (uint64_t(1) << (8 * left)) - 1;
        un[w] = x;
      }
      for (int w = 0; w < nw; ++w) {
        uint64_t x = un[w];
        while (x) {
          const int byte = __builtin_ctzll(x) >> 3;
          x &= ~(uint64_t(0xff) << (8 * byte));
          const int k = w * 8 + byte;
          c->stats.cache_zoomed++;
          if (C.slot_h[bg * mm + k] >= 0) c->stats.cache_hits++;
          else need.push_back((int64_t)bg * mm + k);
        }
      }
    }
  if (need.empty()) return SEKV_OK;
  // the last prefetch's copy kernel has read runs_pin and slot_pin
  if (hipEventQuery(C.ev_pref) != hipSuccess) HIPCHK(c, hipEventSynchronize(C.ev_pref));
  C.batch++;
  const size_t es = c->esz;
  // the misses, merged into runs of consecutive store and cache positions, are
  // copied by one kernel that reads the pinned store in place
  std::vector<int4> runs;
  int64_t run_src = -1, run_dst = -1, run_len = 0;
  auto flush = [&]() -> sekv_status {
    // pieces of at most kCopyPiece elements: one workgroup each
    for (int64_t o = 0; o < run_len; o += kCopyPiece) {
      const int64_t n = std::min<int64_t>(kCopyPiece, run_len - o);
      runs.push_back(make_int4((int)(uint32_t)((run_src + o) >> 3), (int)(uint32_t)((run_dst + o) >> 3),
                               (int)(n >> 3), 0));
    }
    run_len = 0;
    return SEKV_OK;
  };
  for (int64_t idx : need) {
    const int b = (int)(idx / mm / Hkv), k = (int)(idx % mm);
    const int64_t len = span_elems(c->mcount[b][k], L.rank_h[idx], d);
    int64_t off = 0;
    if (!cache_place(C, len, &off)) continue;
    const int64_t dst = C.base + off, src = L.boff_h[idx];
    C.slot_h[idx] = (int32_t)(dst >> 3);
    C.dirty_lo = std::min(C.dirty_lo, idx);
    C.dirty_hi = std::max(C.dirty_hi, idx + 1);
    C.fifo.push_back({idx, off, len, C.batch});
    c->stats.cache_spans_fetched++;
    c->stats.cache_bytes_fetched += (uint64_t)len * es;
    if (run_len > 0 && run_src + run_len == src && run_dst + run_len == dst) {
      run_len += len;
    } else {
      TRY(flush());
      run_src = src;
      run_dst = dst;
      run_len = len;
    }
  }
  TRY(flush());
  if (runs.size() > C.runs_cap) {  // the last prefetch's copy kernel is done (ev_pref)
    const size_t cap = std::max<size_t>(runs.size(), 2 * C.runs_cap + 256);
    hfree(C.runs_pin);
    C.runs_cap = 0;
    TRY(halloc(c, &C.runs_pin, cap * sizeof(int4), hipHostMallocCoherent));
    HIPCHK(c, hipHostGetDevicePointer((void**)&C.runs_hd, C.runs_pin, 0));
    C.runs_cap = cap;
  }
  if (!runs.empty()) std::memcpy(C.runs_pin, runs.data(), runs.size() * sizeof(int4));
  // the changed range of the slot table, in whole 16-byte pieces
  size_t lo = 0, n = 0;
  if (C.dirty_lo < C.dirty_hi) {
    lo = (size_t)C.dirty_lo & ~size_t(3);
    n = (((size_t)C.dirty_hi + 3) & ~size_t(3)) - lo;
    std::memcpy(C.slot_pin + lo, C.slot_h.data() + lo, n * 4);
    C.dirty_lo = INT64_MAX;
    C.dirty_hi = 0;
  }
  // one launch: the runs from the mapped store into the region, then the table
  launch_copy_runs(C.runs_hd, (int)runs.size(), L.bases_hd, c->cache_d, (int)es, C.slot_hd + lo, C.slot_d + lo,
                   (int64_t)n * 4, c->side);
  HIPCHK(c, hipGetLastError());
  c->stats.memcpy_calls++;
  HIPCHK(c, hipEventRecord(C.ev_pref, c->side));
  C.pref_pending = true;
  return SEKV_OK;
}

void fill_decode_geometry(sekv_ctx* c, LayerState& L, DecodeArgs& a) {
  std::memset(&a, 0, sizeof(a));
  a.B = c->cfg.batch;
  a.Hq = c->cfg.n_q_heads;
  a.Hkv = c->cfg.n_kv_heads;
  a.G = c->G;
  a.m_max = c->m_max;
  a.na_max = L.na_cap;
  a.m_b = c->m_b_d;
  a.na_b = L.na_l_d;
  a.logS = c->logS_d;
  a.kbar = L.kbar;
  a.vbar = L.vbar;
  a.KA = L.KA;
  a.VA = L.VA;
  a.smeta = L.smeta_d;
  a.bases = L.bases_d;
  a.basis_elems = L.basis_elems;
  a.tasks = L.sched.tasks_d;
  a.n_tasks = (int)L.sched.tasks.size();
  a.n_span_tasks = L.sched.n_span_tasks;
  a.parts_n = L.sched.parts_d;
  a.max_parts = L.sched.max_parts;
  a.zcnt = L.sched.zcnt_d;
  a.zlist = c->zlist_d;
  a.zcounter = c->zcounter_d;
  const int layer = (int)(&L - c->layers.data());
  a.dr = c->route[layer].dr;
  a.Kr = L.Kr;
  a.Wr = c->route[layer].W_d;
  a.qp = c->qp_d;
}

sekv_status thetas(sekv_ctx* c, const float* tau, DecodeArgs& a) {
  if (!tau) return fail(c, SEKV_ERR_INVALID, "tau is NULL");
  for (int h = 0; h < c->cfg.n_q_heads; ++h) {
    const double t = (double)tau[h];
    if (std::isnan(t)) return fail(c, SEKV_ERR_INVALID, "tau[" + std::to_string(h) + "] is NaN");
    if (t <= 0.0) a.theta[h] = -INFINITY;
    else if (t >= 1.0) a.theta[h] = INFINITY;
    else a.theta[h] = std::log(t) - std::log1p(-t);
  }
  return SEKV_OK;
}

}  // namespace

// ============================================================================ C ABI

extern "C" {

const char* sekv_last_error(const sekv_ctx* ctx) {
  return ctx ? ctx->err.c_str() : g_create_err.c_str();
}

sekv_status sekv_create(const sekv_config* cfg, sekv_ctx** out) {
  if (!cfg || !out) return fail(nullptr, SEKV_ERR_INVALID, "NULL argument");
  *out = nullptr;
  const sekv_config& k = *cfg;
  if (k.n_layers < 1 || k.batch < 1 || k.n_ctx < 1 || k.n_q_heads < 1 || k.n_kv_heads < 1)
    return fail(nullptr, SEKV_ERR_INVALID, "sizes must be >= 1");
  if (k.n_q_heads % k.n_kv_heads != 0)
    return fail(nullptr, SEKV_ERR_INVALID, "n_q_heads must be a multiple of n_kv_heads");
  const int G = k.n_q_heads / k.n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(nullptr, SEKV_ERR_INVALID, "n_q_heads / n_kv_heads must be 1, 2, 4 or 8");
  if (k.n_q_heads > kMaxHq) return fail(nullptr, SEKV_ERR_INVALID, "at most 64 query heads");
  if ((int64_t)k.batch * k.n_kv_heads > kMaxBg)
    return fail(nullptr, SEKV_ERR_INVALID, "batch * n_kv_heads must be <= 512");
  if (k.d_head != 64 && k.d_head != 128) return fail(nullptr, SEKV_ERR_INVALID, "d_head must be 64 or 128");
  if (k.kv_dtype != SEKV_F32 && k.kv_dtype != SEKV_BF16) return fail(nullptr, SEKV_ERR_INVALID, "bad kv_dtype");
  if (k.local_window < 0) return fail(nullptr, SEKV_ERR_INVALID, "local_window must be >= 0");
  if (k.basis_home != SEKV_BASES_HOST && k.basis_home != SEKV_BASES_DEVICE && k.basis_home != SEKV_BASES_HOST_STAGED)
    return fail(nullptr, SEKV_ERR_INVALID, "bad basis_home");
  if (k.n_ctx >= (1 << 24)) return fail(nullptr, SEKV_ERR_INVALID, "n_ctx must be < 2^24");
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || k.device < 0 || k.device >= ndev) {
    (void)hipGetLastError();
    return fail(nullptr, SEKV_ERR_HIP, "HIP device " + std::to_string(k.device) + " not available");
  }
  DevGuard dg(k.device);
  sekv_ctx* c = new sekv_ctx();
  c->cfg = k;
  c->G = G;
  c->bf16 = k.kv_dtype == SEKV_BF16;
  c->esz = c->bf16 ? 2 : 4;
  c->layers.resize(k.n_layers);
  c->route.resize(k.n_layers);
  c->pend.assign(k.batch, 0);
  c->mstart.assign(k.batch, {});
  c->mcount.assign(k.batch, {});
  c->anchors.assign(k.batch, {});
  c->anchor_chunk = env_int("SEKV_ANCHOR_CHUNK", 256, 16, 1 << 20);
  {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, c->cfg.device) == hipSuccess && cus > 0) {
      c->fill_tasks = env_int("SEKV_FILL_TASKS", 3 * cus, 64, 1 << 16);
      c->fill_fixed = std::getenv("SEKV_FILL_TASKS") != nullptr;
    }
  }
  c->span_chunk = env_int("SEKV_SPAN_CHUNK", 64, 8, 1024);
  sekv_status s = dalloc(c, &c->zcounter_d, 4);
  if (s == SEKV_OK) s = dalloc(c, &c->qp_d, (size_t)k.batch * k.n_q_heads * k.d_head * sizeof(float));
  if (s == SEKV_OK) s = halloc(c, &c->zcount_h, 4);
  if (s == SEKV_OK && hipMemset(c->zcounter_d, 0, 4) != hipSuccess) s = fail(c, SEKV_ERR_HIP, "hipMemset");
  if (s == SEKV_OK && hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking) != hipSuccess)
    s = fail(c, SEKV_ERR_HIP, "hipStreamCreate(side)");
  if (s == SEKV_OK && hipEventCreateWithFlags(&c->ev_fetch, hipEventDisableTiming) != hipSuccess)
    s = fail(c, SEKV_ERR_HIP, "hipEventCreate");
  if (s == SEKV_OK && hipEventCreateWithFlags(&c->ev_runs, hipEventDisableTiming) != hipSuccess)
    s = fail(c, SEKV_ERR_HIP, "hipEventCreate");
  if (s == SEKV_OK) {
    // the device address of this GPU's scratch array of sekv_decode_attn_noalloc
    const hipError_t e = noalloc_scratch_init(k.device);
    if (e != hipSuccess) s = fail(c, SEKV_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
  }
  if (s != SEKV_OK) {
    g_create_err = c->err;
    sekv_destroy(c);
    return s;
  }
  const int64_t full = 2ll * k.n_layers * k.batch * k.n_kv_heads * (int64_t)k.n_ctx * k.d_head * c->esz;
  c->stats.full_kv_bytes = full;
  *out = c;
  return SEKV_OK;
}

void sekv_destroy(sekv_ctx* c) {
  if (!c) return;
  DevGuard dg(c->cfg.device);
  if (c->side) (void)hipStreamSynchronize(c->side);
  for (auto& L : c->layers) free_layer(L);
  for (auto& r : c->route) dfree(r.W_d);
  dfree(c->qp_d);
  dfree(c->cache_d);
  dfree(c->m_b_d);
  dfree(c->na_b_d);
  dfree(c->mstart_d);
  dfree(c->mcount_d);
  dfree(c->anchors_d);
  dfree(c->logS_d);
  for (auto& p : c->prob_d) dfree(p);
  dfree(c->seg_i);
  dfree(c->seg_counts);
  dfree(c->seg_stats);
  dfree(c->part_ml);
  dfree(c->part_acc);
  dfree(c->zlist_d);
  dfree(c->zcounter_d);
  dfree(c->mask_d);
  dfree(c->scores_d);
  dfree(c->zitems_d);
  dfree(c->zgroups_d);
  hfree(c->zlist_h);
  hfree(c->zcount_h);
  hfree(c->zitems_h);
  hfree(c->zgroups_h);
  dfree(c->staging);
  hfree(c->fruns_pin);
  if (c->ev_fetch) (void)hipEventDestroy(c->ev_fetch);
  if (c->ev_runs) (void)hipEventDestroy(c->ev_runs);
  if (c->side) (void)hipStreamDestroy(c->side);
  delete c;
}

// ---------------------------------------------------------------------------- build

sekv_status sekv_build(sekv_ctx* c, int32_t layer, const float* H, const void* K, const void* V,
                       double alpha, const int32_t* rank_choices, int32_t n_choices,
                       uint64_t rank_seed, hipStream_t stream) {
  if (!c) return fail(nullptr, SEKV_ERR_INVALID, "NULL context");
  DevGuard dg(c->cfg.device);
  const int B = c->cfg.batch, n = c->cfg.n_ctx, Hkv = c->cfg.n_kv_heads, d = c->cfg.d_head;
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(c, SEKV_ERR_INVALID, "layer out of range");
  if (!H || !K || !V) return fail(c, SEKV_ERR_INVALID, "NULL H, K or V");
  if (!std::isfinite(alpha)) return fail(c, SEKV_ERR_INVALID, "alpha must be finite");
  if (c->resegmented) return fail(c, SEKV_ERR_STATE, "the window was re-segmented: build every layer first");
  if (!rank_choices || n_choices < 1) return fail(c, SEKV_ERR_INVALID, "rank choices missing");
  for (int i = 0; i < n_choices; ++i)
    if (rank_choices[i] < 1) return fail(c, SEKV_ERR_INVALID, "rank choice < 1");

  // 1. segmentation
  if (!c->seg_i) {
    TRY(dalloc(c, &c->seg_i, sizeof(int32_t) * 4 * (size_t)B * n));
    TRY(dalloc(c, &c->seg_counts, sizeof(int32_t) * 4 * B));
    TRY(dalloc(c, &c->seg_stats, sizeof(double) * 3 * B));
  }
  SegmentArgs sa;
  sa.H = H;
  sa.B = B;
  sa.n = n;
  sa.w = c->cfg.local_window;
  sa.alpha = alpha;
  sa.flagpos = c->seg_i;
  sa.mstart = c->seg_i + (size_t)B * n;
  sa.mcount = c->seg_i + 2 * (size_t)B * n;
  sa.anchors = c->seg_i + 3 * (size_t)B * n;
  sa.counts = c->seg_counts;
  sa.stats = c->seg_stats;
  launch_segment(sa, stream);
  HIPCHK(c, hipGetLastError());
  std::vector<int32_t> counts(4 * B);
  HIPCHK(c, hipMemcpyAsync(counts.data(), c->seg_counts, counts.size() * 4, hipMemcpyDeviceToHost, stream));
  HIPCHK(c, hipStreamSynchronize(stream));
  for (int b = 0; b < B; ++b)
    if (counts[4 * b + 2]) return fail(c, SEKV_ERR_INVALID, "surprisal must be finite and >= 0");
  std::vector<std::vector<int32_t>> ms(B), mc(B), an(B);
  for (int b = 0; b < B; ++b) {
    ms[b].resize(counts[4 * b + 0]);
    mc[b].resize(counts[4 * b + 0]);
    an[b].resize(counts[4 * b + 1]);
    HIPCHK(c, hipMemcpy(ms[b].data(), sa.mstart + (size_t)b * n, ms[b].size() * 4, hipMemcpyDeviceToHost));
    HIPCHK(c, hipMemcpy(mc[b].data(), sa.mcount + (size_t)b * n, mc[b].size() * 4, hipMemcpyDeviceToHost));
    HIPCHK(c, hipMemcpy(an[b].data(), sa.anchors + (size_t)b * n, an[b].size() * 4, hipMemcpyDeviceToHost));
  }
  if (c->spans_ready) {
    bool same = true;
    for (int b = 0; b < B && same; ++b)
      same = ms[b] == c->mstart[b] && mc[b] == c->mcount[b] && an[b] == c->anchors[b];
    if (!same) return fail(c, SEKV_ERR_STATE, "surprisal or alpha differ from the span table in use");
  } else {
    c->mstart = ms;
    c->mcount = mc;
    c->anchors = an;
    TRY(install_spans(c));
    c->spans_built = true;
    c->alpha = alpha;
    // what re-segmenting the window needs later: surprisal, thresholds, row positions
    c->H_seq.assign(B, std::vector<float>(n));
    for (int b = 0; b < B; ++b)
      HIPCHK(c, hipMemcpy(c->H_seq[b].data(), H + (size_t)b * n, (size_t)n * 4, hipMemcpyDeviceToHost));
    std::vector<double> st(3 * (size_t)B);
    HIPCHK(c, hipMemcpy(st.data(), c->seg_stats, st.size() * 8, hipMemcpyDeviceToHost));
    c->theta_b.assign(B, 0.0);
    for (int b = 0; b < B; ++b) c->theta_b[b] = st[3 * b + 2];
    c->row_pos = an;
    c->next_pos.assign(B, n);
  }

  // 2. ranks and layout
  const int mm = c->m_max;
  std::vector<int32_t> rank((size_t)B * Hkv * mm, 0);
  for (int b = 0; b < B; ++b)
    for (int g = 0; g < Hkv; ++g)
      for (int k = 0; k < c->m_b[b]; ++k) {
        const uint64_t key = rank_seed ^ ((uint64_t)layer << 40) ^ ((uint64_t)g << 32) ^ (uint64_t)k;
        int r = rank_choices[splitmix64(key) % (uint64_t)n_choices];
        r = std::min(r, std::min(c->mcount[b][k], d));
        rank[((size_t)b * Hkv + g) * mm + k] = r;
      }
  TRY(alloc_layer(c, layer, rank));
  LayerState& L = c->layers[layer];
  L.choices.assign(rank_choices, rank_choices + n_choices);
  L.seed = rank_seed;

  // 3. summaries and anchors
  SummaryArgs su;
  su.H = H;
  su.K = K;
  su.V = V;
  su.B = B;
  su.Hkv = Hkv;
  su.n = n;
  su.m_max = mm;
  su.na_max = c->na_max;
  su.na_cap = L.na_cap;
  su.m_b = c->m_b_d;
  su.mstart = c->mstart_d;
  su.mcount = c->mcount_d;
  su.na_b = c->na_b_d;
  su.anchors = c->anchors_d;
  su.kbar = L.kbar;
  su.vbar = L.vbar;
  su.KA = L.KA;
  su.VA = L.VA;
  su.span_chunk = 16;
  su.n_span_chunks = (mm + su.span_chunk - 1) / su.span_chunk;
  su.anchor_chunk = 256;
  su.n_anchor_chunks = (c->na_max + su.anchor_chunk - 1) / su.anchor_chunk;
  su.dr = c->route[layer].dr;
  su.Wr = c->route[layer].W_d;
  su.Kr = L.Kr;
  launch_summaries(d, c->bf16, su, stream);
  HIPCHK(c, hipGetLastError());

  // 4. truncated SVD of every span, K and V, straight into the packed store
  SvdArgs sv;
  sv.K = K;
  sv.V = V;
  sv.Hkv = Hkv;
  sv.n = n;
  sv.m_max = mm;
  sv.mstart = c->mstart_d;
  sv.mcount = c->mcount_d;
  sv.rank = L.rank_d;
  sv.boff = L.boff_d;
  sv.bases = L.bases_d;
  const int cmax[5] = {16, 32, 64, 128, 0};
  for (int i = 0; i < 5; ++i) {
    sv.problems = c->prob_d[i];
    sv.n_problems = c->n_prob[i];
    HIPCHK(c, launch_svd(cmax[i], d, c->bf16, sv, stream));
  }
  // 5. HOST home: move the store to pinned memory
  if (host_store(c)) {
    HIPCHK(c, hipMemcpyAsync(L.bases_h, L.bases_d, (size_t)L.basis_elems * c->esz, hipMemcpyDeviceToHost,
                             stream));
  }
  HIPCHK(c, hipStreamSynchronize(stream));
  if (host_store(c)) dfree(L.bases_d);
  std::fill(L.head_set.begin(), L.head_set.end(), 1);
  std::fill(L.route_set.begin(), L.route_set.end(), 1);
  update_ready(L);
  return SEKV_OK;
}

sekv_status sekv_get_spans(const sekv_ctx* cc, int32_t b, int32_t* m, int32_t* n_anchors, int32_t* m_max,
                           int32_t* mstart, int32_t* mcount, int32_t* anchors) {
  sekv_ctx* c = const_cast<sekv_ctx*>(cc);
  if (!c) return fail(nullptr, SEKV_ERR_INVALID, "NULL context");
  if (!c->spans_ready) return fail(c, SEKV_ERR_STATE, "no span table yet");
  if (b < 0 || b >= c->cfg.batch) return fail(c, SEKV_ERR_INVALID, "b out of range");
  if (m) *m = c->m_b[b];
  if (n_anchors) *n_anchors = c->na_b[b];
  if (m_max) *m_max = c->m_max;
  if (mstart) std::memcpy(mstart, c->mstart[b].data(), c->mstart[b].size() * 4);
  if (mcount) std::memcpy(mcount, c->mcount[b].data(), c->mcount[b].size() * 4);
  if (anchors) std::memcpy(anchors, c->anchors[b].data(), c->anchors[b].size() * 4);
  return SEKV_OK;
}

sekv_status sekv_get_bases_layout(const sekv_ctx* cc, int32_t layer, int32_t b, int32_t g, int32_t* rank,
                                  int64_t* basis_off, int64_t* basis_elems) {
  sekv_ctx* c = const_cast<sekv_ctx*>(cc);
  if (!c) return fail(nullptr, SEKV_ERR_INVALID, "NULL context");
  if (layer < 0 || layer >= c->cfg.n_layers || b < 0 || b >= c->cfg.batch || g < 0 || g >= c->cfg.n_kv_heads)
    return fail(c, SEKV_ERR_INVALID, "index out of range");
  LayerState& L = c->layers[layer];
  if (!L.allocated) return fail(c, SEKV_ERR_STATE, "layer has no layout");
  const size_t bg = (size_t)b * c->cfg.n_kv_heads + g;
  const int m = c->m_b[b];
  for (int k = 0; k < m; ++k) {
    if (rank) rank[k] = L.rank_h[bg * c->m_max + k];
    if (basis_off) basis_off[k] = L.boff_h[bg * c->m_max + k] - L.head_base[bg];
  }
  if (basis_elems) *basis_elems = L.head_base[bg + 1] - L.head_base[bg];
  return SEKV_OK;
}

// ---------------------------------------------------------------------------- decode

sekv_status sekv_zoom_fetch(sekv_ctx* c, int32_t layer, const int32_t* entries, const int32_t* counts,
                            hipStream_t side, hipEvent_t done) {
  if (!c) return fail(nullptr, SEKV_ERR_INVALID, "NULL context");
  DevGuard dg(c->cfg.device);
  TRY(check_layer(c, layer));
  if (!host_store(c)) return fail(c, SEKV_ERR_STATE, "bases are device-resident");
  if (!entries || !counts) return fail(c, SEKV_ERR_INVALID, "NULL entries or counts");
  TRY(ensure_zoom_buffers(c));
  const int B = c->cfg.batch, Hkv = c->cfg.n_kv_heads, mm = c->m_max;
  int n = 0;
  for (int bg = 0; bg < B * Hkv; ++bg) {
    const int cnt = counts[bg];
    if (cnt < 0 || cnt > c->m_b[bg / Hkv]) return fail(c, SEKV_ERR_INVALID, "zoom count out of range");
    for (int i = 0; i < cnt; ++i) {
      const int32_t e = entries[(size_t)bg * mm + i];
      c->zitems_h[n++] = make_int4(bg | (int)((uint32_t)e & 0xff000000u), e & 0xffffff, 0, 0);
    }
  }
  return fetch_items(c, layer, c->zitems_h, n, side, done, nullptr);
}

}  // extern "C"

namespace {

sekv_status decode_step(sekv_ctx* c, int32_t layer, const float* q, const float* tau, const int32_t* budget,
                        float* out, uint8_t* zoom_mask, hipStream_t stream) {
  if (!c) return fail(nullptr, SEKV_ERR_INVALID, "NULL context");
  DevGuard dg(c->cfg.device);
  TRY(check_layer(c, layer));
  if (!q || !out) return fail(c, SEKV_ERR_INVALID, "NULL q or out");
  LayerState& L = c->layers[layer];
  TRY(ensure_zoom_buffers(c));
  DecodeArgs a;
  TRY(thetas(c, tau, a));  // validates tau before anything is queued
  bool capped = false;
  for (int h = 0; h < kMaxHq; ++h) a.budget[h] = -1;
  if (budget)
    for (int h = 0; h < c->cfg.n_q_heads; ++h) {
      a.budget[h] = budget[h] < 0 ? -1 : budget[h];
      capped |= budget[h] >= 0;
    }
  bool capturing = false;
  TRY(prepare_sched(c, layer, stream, &capturing));
  {
    double th[kMaxHq];
    int32_t bu[kMaxHq];
    std::memcpy(th, a.theta, sizeof(th));
    std::memcpy(bu, a.budget, sizeof(bu));
    fill_decode_geometry(c, L, a);
    std::memcpy(a.theta, th, sizeof(th));
    std::memcpy(a.budget, bu, sizeof(bu));
  }
  a.q = q;
  a.out = out;
  a.mask = zoom_mask ? zoom_mask : c->mask_d;
  if (!staged(c)) {
    // the planned kernel: its segment lists and their partial slots
    TRY(prepare_plan(c, layer, stream, capturing));
    a.wsegs = L.sched.wsegs_d;
    a.zparts = 1;
    a.parts_n = L.sched.wparts_d;
    a.max_parts = L.sched.w_max_parts;
  }
  if (capturing && (size_t)a.B * a.Hq * a.max_parts > c->parts_cap)
    return fail(c, SEKV_ERR_STATE, "partial buffers would grow during graph capture: decode once first");
  TRY(ensure_parts(c, (size_t)a.B * a.Hq * a.max_parts));
  a.part_ml = c->part_ml;
  a.part_acc = c->part_acc;
  a.zcount = L.zcount_d;
  c->stats.decode_calls++;
  const int d = c->cfg.d_head;
  if (a.dr > 0) {
    launch_decode_qproj(d, a, stream);
    HIPCHK(c, hipGetLastError());
  }
  if (capped) {
    // budget cap: routing scores, then the capped decisions into the mask,
    // which the route kernel below follows
    a.scores = c->scores_d;
    launch_decode_route(2, a.n_span_tasks, d, c->bf16, a, stream);
    HIPCHK(c, hipGetLastError());
    launch_decode_select(a, stream);
    HIPCHK(c, hipGetLastError());
    a.capped = 1;
  }
  const bool cached = c->cache_d && c->cfg.basis_home == SEKV_BASES_HOST;
  if (cached) {
    if (capturing) return fail(c, SEKV_ERR_STATE, "decode with a basis cache is not capturable");
    TRY(ensure_layer_cache(c, layer));
    TRY(cache_prefetch(c, layer));  // if the previous mask is back and no earlier call used it
    if (L.lc.pref_pending && hipEventQuery(L.lc.ev_pref) != hipSuccess)
      HIPCHK(c, hipStreamWaitEvent(stream, L.lc.ev_pref, 0));
    L.lc.pref_pending = false;
    a.cslot = L.lc.slot_d;
    a.cache = c->cache_d;
    // the combine kernel writes this step's zoom mask back for the prediction of the next one
    a.mask_h = L.lc.zm_hd;
    a.mask_bytes = (int64_t)a.B * a.Hq * a.m_max;
  }
  if (!staged(c)) {
    // span tasks with their zoomed spans in place (bases in HBM, or read from
    // the pinned host store over the link, or from its device cache), and the
    // anchor tasks
    if (host_store(c)) a.bases = L.bases_hd;
    launch_decode_planned(L.sched.n_wg, d, c->bf16, a, stream);
    HIPCHK(c, hipGetLastError());
  } else {
    // HOST home: learn the zoom list, fetch the bases, then the zoomed segment
    if (capturing) return fail(c, SEKV_ERR_STATE, "host-resident bases need a host sync: not capturable");
    launch_decode_route(1, a.n_span_tasks, d, c->bf16, a, stream);
    HIPCHK(c, hipGetLastError());
    HIPCHK(c, hipMemcpyAsync(c->zcount_h, c->zcounter_d, 4, hipMemcpyDeviceToHost, stream));
    HIPCHK(c, hipStreamSynchronize(stream));
    const int nz = *c->zcount_h;
    if (nz) {
      HIPCHK(c, hipMemcpyAsync(c->zlist_h, c->zlist_d, (size_t)nz * sizeof(int4), hipMemcpyDeviceToHost, stream));
      HIPCHK(c, hipStreamSynchronize(stream));
    }
    int ng = 0;
    sekv_status fs = fetch_items(c, layer, c->zlist_h, nz, c->side, c->ev_fetch, &ng);
    if (fs != SEKV_OK) {
      (void)hipMemsetAsync(c->zcounter_d, 0, 4, stream);  // leave an empty list for the next call
      return fs;
    }
    HIPCHK(c, hipStreamWaitEvent(stream, c->ev_fetch, 0));
    a.zitems = c->zitems_d;
    a.zgroups = c->zgroups_d;
    a.staging = c->staging;
    a.n_zoom_wgs = ng;
    launch_decode_attend(ng + (a.n_tasks - a.n_span_tasks), d, c->bf16, a, stream);
    HIPCHK(c, hipGetLastError());
  }
  launch_decode_combine(d, a, stream);
  HIPCHK(c, hipGetLastError());
  if (cached) {
    // the decode is done, and this step's zoom mask is back (the combine kernel wrote it)
    LayerCache& C = L.lc;
    HIPCHK(c, hipEventRecord(C.ev_done, stream));
    C.done_valid = true;
    C.zm_valid = true;
    // the next layer's prefetch runs on the side stream while this one decodes
    const int nxt = (layer + 1) % c->cfg.n_layers;
    if (nxt != layer && c->layers[nxt].ready) {
      TRY(ensure_layer_cache(c, nxt));
      TRY(cache_prefetch(c, nxt));
    }
  }
  if (!staged(c)) return finish_plan(c, layer, a.mask, stream, capturing);
  return finish_sched(c, layer, stream, capturing);
}

}  // namespace

extern "C" {

sekv_status sekv_decode_attn(sekv_ctx* c, int32_t layer, const float* q, const float* tau, float* out,
                             uint8_t* zoom_mask, hipStream_t stream) {
  return decode_step(c, layer, q, tau, nullptr, out, zoom_mask, stream);
}

sekv_status sekv_decode_attn_budget(sekv_ctx* c, int32_t layer, const float* q, const float* tau,
                                    const int32_t* budget, float* out, uint8_t* zoom_mask, hipStream_t stream) {
  if (c && !budget) return fail(c, SEKV_ERR_INVALID, "budget is NULL");
  return decode_step(c, layer, q, tau, budget, out, zoom_mask, stream);
}

static_assert(kNoAllocScratchBytes == SEKV_NOALLOC_SCRATCH_BYTES, "scratch size of the header and the library");

sekv_status sekv_decode_attn_noalloc(sekv_ctx* c, int32_t layer, const float* q, const float* tau, float* out,
                                     uint8_t* zoom_mask, hipStream_t stream) {
  if (!c) return fail(nullptr, SEKV_ERR_INVALID, "NULL context");
  DevGuard dg(c->cfg.device);
  TRY(check_layer(c, layer));
  if (!q || !out) return fail(c, SEKV_ERR_INVALID, "NULL q or out");
  if (staged(c)) return fail(c, SEKV_ERR_STATE, "staged host bases allocate staging: use sekv_decode_attn");
  if (c->cache_d && c->cfg.basis_home == SEKV_BASES_HOST)
    return fail(c, SEKV_ERR_STATE, "a basis cache refills itself: use sekv_decode_attn");
  LayerState& L = c->layers[layer];
  LayerSched& S = L.sched;
  // the layer's segment lists as the last sekv_decode_attn left them; they
  // must still cover every span and anchor row
  if (!S.valid || !S.wvalid || S.anchors_changed || S.plan_m != c->m_b || S.plan_na != L.na_l)
    return fail(c, SEKV_ERR_STATE, "no current work schedule: decode this layer once with sekv_decode_attn");
  DecodeArgs a;
  fill_decode_geometry(c, L, a);
  TRY(thetas(c, tau, a));
  for (int h = 0; h < kMaxHq; ++h) a.budget[h] = -1;
  // scratch: partials, projected queries, and the zoom mask when the caller passes none
  const int d = c->cfg.d_head;
  auto up = [](size_t n) { return (n + 255) & ~size_t(255); };
  const size_t slots = (size_t)a.B * a.Hq * S.w_max_parts;
  const size_t ml_b = up(slots * 4 * sizeof(float)), acc_b = up(slots * d * sizeof(float));
  const size_t qp_b = a.dr > 0 ? up((size_t)a.B * a.Hq * a.dr * sizeof(float)) : 0;
  const size_t mask_b = zoom_mask ? 0 : up((size_t)a.B * a.Hq * a.m_max);
  const size_t need = ml_b + acc_b + qp_b + mask_b;
  if (need > kNoAllocScratchBytes)
    return fail(c, SEKV_ERR_INVALID, "decode needs " + std::to_string(need) + " scratch bytes, more than the " +
                                         std::to_string(kNoAllocScratchBytes) + " of sekv_decode_attn_noalloc");
  char* base = static_cast<char*>(noalloc_scratch(c->cfg.device));
  if (!base) return fail(c, SEKV_ERR_STATE, "scratch address of this device not initialised");
  a.part_ml = reinterpret_cast<float*>(base);
  a.part_acc = reinterpret_cast<float*>(base + ml_b);
  if (a.dr > 0) a.qp = reinterpret_cast<float*>(base + ml_b + acc_b);
  a.mask = zoom_mask ? zoom_mask : reinterpret_cast<uint8_t*>(base + ml_b + acc_b + qp_b);
  a.q = q;
  a.out = out;
  a.wsegs = S.wsegs_d;
  a.zparts = 1;
  a.parts_n = S.wparts_d;
  a.max_parts = S.w_max_parts;
  a.zcount = L.zcount_d;
  if (host_store(c)) a.bases = L.bases_hd;
  c->stats.decode_calls++;
  if (a.dr > 0) {
    launch_decode_qproj(d, a, stream);
    HIPCHK(c, hipGetLastError());
  }
  launch_decode_planned(S.n_wg, d, c->bf16, a, stream);
  HIPCHK(c, hipGetLastError());
  launch_decode_combine(d, a, stream);
  HIPCHK(c, hipGetLastError());
  return SEKV_OK;
}

sekv_status sekv_route_scores(sekv_ctx* c, int32_t layer, const float* q, float* scores, hipStream_t stream) {
  if (!c) return fail(nullptr, SEKV_ERR_INVALID, "NULL context");
  DevGuard dg(c->cfg.device);
  TRY(check_layer(c, layer));
  if (!q || !scores) return fail(c, SEKV_ERR_INVALID, "NULL q or scores");
  LayerState& L = c->layers[layer];
  bool capturing = false;
  TRY(prepare_sched(c, layer, stream, &capturing));
  DecodeArgs a;
  fill_decode_geometry(c, L, a);
  for (int h = 0; h < kMaxHq; ++h) a.theta[h] = INFINITY;
  a.q = q;
  a.scores = scores;
  if (a.dr > 0) {
    launch_decode_qproj(c->cfg.d_head, a, stream);
    HIPCHK(c, hipGetLastError());
  }
  launch_decode_route(2, a.n_span_tasks, c->cfg.d_head, c->bf16, a, stream);
  HIPCHK(c, hipGetLastError());
  return SEKV_OK;
}

// ---------------------------------------------------------------------------- artefact exchange

sekv_status sekv_import_spans(sekv_ctx* c, int32_t b, int32_t m, const int32_t* mstart, const int32_t* mcount,
                              int32_t n_anchors, const int32_t* anchors) {
  if (!c) return fail(nullptr, SEKV_ERR_INVALID, "NULL context");
  DevGuard dg(c->cfg.device);
  if (c->spans_built) return fail(c, SEKV_ERR_STATE, "span table fixed by sekv_build");
  const int n = c->cfg.n_ctx;
  if (b < 0 || b >= c->cfg.batch) return fail(c, SEKV_ERR_INVALID, "b out of range");
  if (m < 0 || n_anchors < 0 || m + n_anchors > n) return fail(c, SEKV_ERR_INVALID, "bad sizes");
  if ((m && (!mstart || !mcount)) || (n_anchors && !anchors)) return fail(c, SEKV_ERR_INVALID, "NULL arrays");
  std::vector<uint8_t> used(n, 0);
  int prev_end = 0;
  for (int k = 0; k < m; ++k) {
    if (mcount[k] < 1 || mstart[k] < prev_end || (int64_t)mstart[k] + mcount[k] > n)
      return fail(c, SEKV_ERR_INVALID, "spans must be non-empty, ascending, disjoint, inside [0, n)");
    for (int t = mstart[k]; t < mstart[k] + mcount[k]; ++t) used[t] = 1;
    prev_end = mstart[k] + mcount[k];
  }
  for (int i = 0; i < n_anchors; ++i) {
    if (anchors[i] < 0 || anchors[i] >= n || (i && anchors[i] <= anchors[i - 1]) || used[anchors[i]])
      return fail(c, SEKV_ERR_INVALID, "anchors must be ascending, inside [0, n) and not members");
  }
  if (c->spans_ready) {
    // re-import invalidates the layers
    for (auto& L : c->layers) free_layer(L);
    c->spans_ready = false;
  }
  c->mstart[b].assign(mstart, mstart + m);
  c->mcount[b].assign(mcount, mcount + m);
  c->anchors[b].assign(anchors, anchors + n_anchors);
  c->pend[b] = 1;
  for (int i = 0; i < c->cfg.batch; ++i)
    if (!c->pend[i]) return SEKV_OK;
  return install_spans(c);
}

sekv_status sekv_import_layout(sekv_ctx* c, int32_t layer, const int32_t* rank) {
  if (!c) return fail(nullptr, SEKV_ERR_INVALID, "NULL context");
  DevGuard dg(c->cfg.device);
  const int B = c->cfg.batch, Hkv = c->cfg.n_kv_heads, d = c->cfg.d_head;
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(c, SEKV_ERR_INVALID, "layer out of range");
  if (!c->spans_ready) return fail(c, SEKV_ERR_STATE, "import or build the span tables first");
  if (!rank) return fail(c, SEKV_ERR_INVALID, "NULL rank");
  const int mm = c->m_max;
  std::vector<int32_t> rk((size_t)B * Hkv * mm, 0);
  for (int b = 0; b < B; ++b)
    for (int g = 0; g < Hkv; ++g)
      for (int k = 0; k < c->m_b[b]; ++k) {
        const size_t i = ((size_t)b * Hkv + g) * mm + k;
        if (rank[i] < 1 || rank[i] > std::min(c->mcount[b][k], d))
          return fail(c, SEKV_ERR_INVALID, "rank out of range");
        rk[i] = rank[i];
      }
  TRY(alloc_layer(c, layer, rk));
  if (host_store(c)) {
    LayerState& L = c->layers[layer];
    std::memset(L.bases_h, 0, (size_t)L.basis_elems * c->esz);
    dfree(L.bases_d);
  }
  return SEKV_OK;
}

sekv_status sekv_import_head(sekv_ctx* c, int32_t layer, int32_t b, int32_t g, const void* kbar, const void* vbar,
                             const void* KA, const void* VA, const int32_t* rank, const void* bases,
                             int64_t basis_elems) {
  if (!c) return fail(nullptr, SEKV_ERR_INVALID, "NULL context");
  DevGuard dg(c->cfg.device);
  const int B = c->cfg.batch, Hkv = c->cfg.n_kv_heads, d = c->cfg.d_head;
  if (layer < 0 || layer >= c->cfg.n_layers || b < 0 || b >= B || g < 0 || g >= Hkv)
    return fail(c, SEKV_ERR_INVALID, "index out of range");
  if (!c->spans_ready) return fail(c, SEKV_ERR_STATE, "import or build the span tables first");
  const int m = c->m_b[b], na = c->na_b[b], mm = c->m_max;
  if ((m && (!kbar || !vbar || !rank || !bases)) || (na && (!KA || !VA)))
    return fail(c, SEKV_ERR_INVALID, "NULL arrays");
  for (int k = 0; k < m; ++k)
    if (rank[k] < 1 || rank[k] > std::min(c->mcount[b][k], d))
      return fail(c, SEKV_ERR_INVALID, "rank out of range at span " + std::to_string(k));
  LayerState& L = c->layers[layer];
  const size_t bg = (size_t)b * Hkv + g;
  if (!L.allocated) return fail(c, SEKV_ERR_STATE, "layer has no layout (sekv_import_layout)");
  for (int k = 0; k < m; ++k)
    if (L.rank_h[bg * mm + k] != rank[k])
      return fail(c, SEKV_ERR_INVALID, "ranks differ from the layer's layout");
  const int64_t he = L.head_base[bg + 1] - L.head_base[bg];
  if (basis_elems != he)
    return fail(c, SEKV_ERR_INVALID, "basis_elems " + std::to_string(basis_elems) + " != layout " + std::to_string(he));
  const size_t es = c->esz;
  HIPCHK(c, invalidate_layer_cache(L));
  if (m) {
    HIPCHK(c, hipMemcpy((char*)L.kbar + bg * mm * d * es, kbar, (size_t)m * d * es, hipMemcpyHostToDevice));
    HIPCHK(c, hipMemcpy((char*)L.vbar + bg * mm * d * es, vbar, (size_t)m * d * es, hipMemcpyHostToDevice));
  }
  if (na) {
    HIPCHK(c, hipMemcpy((char*)L.KA + bg * L.na_cap * d * es, KA, (size_t)na * d * es, hipMemcpyHostToDevice));
    HIPCHK(c, hipMemcpy((char*)L.VA + bg * L.na_cap * d * es, VA, (size_t)na * d * es, hipMemcpyHostToDevice));
  }
  if (host_store(c)) {
    std::memcpy((char*)L.bases_h + L.head_base[bg] * es, bases, (size_t)he * es);
  } else {
    HIPCHK(c, hipMemcpy((char*)L.bases_d + L.head_base[bg] * es, bases, (size_t)he * es, hipMemcpyHostToDevice));
  }
  L.head_set[bg] = 1;
  update_ready(L);
  return SEKV_OK;
}

sekv_status sekv_export_head(const sekv_ctx* cc, int32_t layer, int32_t b, int32_t g, void* kbar, void* vbar,
                             void* KA, void* VA, int32_t* rank, void* bases) {
  sekv_ctx* c = const_cast<sekv_ctx*>(cc);
  if (!c) return fail(nullptr, SEKV_ERR_INVALID, "NULL context");
  DevGuard dg(c->cfg.device);
  const int B = c->cfg.batch, Hkv = c->cfg.n_kv_heads, d = c->cfg.d_head;
  if (layer < 0 || layer >= c->cfg.n_layers || b < 0 || b >= B || g < 0 || g >= Hkv)
    return fail(c, SEKV_ERR_INVALID, "index out of range");
  LayerState& L = c->layers[layer];
  const size_t bg = (size_t)b * Hkv + g;
  if (!L.allocated || !L.head_set[bg]) return fail(c, SEKV_ERR_STATE, "head has no artefacts");
  const int m = c->m_b[b], na = L.na_l[b], mm = c->m_max;
  const size_t es = c->esz;
  if (kbar && m) HIPCHK(c, hipMemcpy(kbar, (char*)L.kbar + bg * mm * d * es, (size_t)m * d * es, hipMemcpyDeviceToHost));
  if (vbar && m) HIPCHK(c, hipMemcpy(vbar, (char*)L.vbar + bg * mm * d * es, (size_t)m * d * es, hipMemcpyDeviceToHost));
  if (KA && na) HIPCHK(c, hipMemcpy(KA, (char*)L.KA + bg * L.na_cap * d * es, (size_t)na * d * es, hipMemcpyDeviceToHost));
  if (VA && na) HIPCHK(c, hipMemcpy(VA, (char*)L.VA + bg * L.na_cap * d * es, (size_t)na * d * es, hipMemcpyDeviceToHost));
  if (rank) std::memcpy(rank, L.rank_h.data() + bg * mm, (size_t)m * 4);
  if (bases) {
    const int64_t he = L.head_base[bg + 1] - L.head_base[bg];
    if (host_store(c))
      std::memcpy(bases, (char*)L.bases_h + L.head_base[bg] * es, (size_t)he * es);
    else
      HIPCHK(c, hipMemcpy(bases, (char*)L.bases_d + L.head_base[bg] * es, (size_t)he * es, hipMemcpyDeviceToHost));
  }
  return SEKV_OK;
}

// ---------------------------------------------------------------------------- basis cache

sekv_status sekv_set_basis_cache(sekv_ctx* c, int64_t bytes) {
  if (!c) return fail(nullptr, SEKV_ERR_INVALID, "NULL context");
  DevGuard dg(c->cfg.device);
  if (c->cfg.basis_home != SEKV_BASES_HOST)
    return fail(c, SEKV_ERR_INVALID, "the basis cache serves SEKV_BASES_HOST contexts only");
  if (bytes < 0) return fail(c, SEKV_ERR_INVALID, "bytes < 0");
  const int64_t elems = bytes / (int64_t)c->esz;
  if ((elems >> 3) >= ((int64_t)1 << 31)) return fail(c, SEKV_ERR_INVALID, "cache larger than 2^34 elements");
  HIPCHK(c, hipDeviceSynchronize());
  for (auto& L : c->layers) free_layer_cache(L.lc);
  dfree(c->cache_d);
  c->cache_elems = 0;
  if (elems >= 8 * c->cfg.n_layers) {
    TRY(dalloc(c, &c->cache_d, (size_t)elems * c->esz));
    c->cache_elems = elems;
  }
  return SEKV_OK;
}

// ---------------------------------------------------------------------------- window re-segmentation

sekv_status sekv_reserve_spans(sekv_ctx* c, int32_t extra) {
  if (!c) return fail(nullptr, SEKV_ERR_INVALID, "NULL context");
  if (extra < 0 || extra > (1 << 22)) return fail(c, SEKV_ERR_INVALID, "extra out of range");
  if (c->spans_ready) return fail(c, SEKV_ERR_STATE, "the span table exists: reserve before the first build");
  c->m_reserve = extra;
  return SEKV_OK;
}

sekv_status sekv_append_surprisal(sekv_ctx* c, const float* H_new, int32_t n_new) {
  if (!c) return fail(nullptr, SEKV_ERR_INVALID, "NULL context");
  if (c->H_seq.empty()) return fail(c, SEKV_ERR_STATE, "no surprisal record: the span table did not come from sekv_build");
  if (n_new < 0 || (n_new > 0 && !H_new)) return fail(c, SEKV_ERR_INVALID, "bad H_new");
  const int B = c->cfg.batch;
  for (size_t i = 0; i < (size_t)B * n_new; ++i)
    if (!std::isfinite(H_new[i]) || H_new[i] < 0.f) return fail(c, SEKV_ERR_INVALID, "surprisal must be finite and >= 0");
  for (int b = 0; b < B; ++b) c->H_seq[b].insert(c->H_seq[b].end(), H_new + (size_t)b * n_new, H_new + (size_t)(b + 1) * n_new);
  return SEKV_OK;
}

sekv_status sekv_resegment_window(sekv_ctx* c, hipStream_t stream) {
  if (!c) return fail(nullptr, SEKV_ERR_INVALID, "NULL context");
  DevGuard dg(c->cfg.device);
  if (c->H_seq.empty()) return fail(c, SEKV_ERR_STATE, "no surprisal record: the span table did not come from sekv_build");
  const int B = c->cfg.batch, Hkv = c->cfg.n_kv_heads, d = c->cfg.d_head, NL = c->cfg.n_layers;
  const int w = c->cfg.local_window, mm = c->m_max;
  const size_t es = c->esz;
  for (int l = 0; l < NL; ++l) {
    if (!c->layers[l].ready) return fail(c, SEKV_ERR_STATE, "every layer must be built before re-segmenting");
    if (c->layers[l].choices.empty())  // imported artefacts: no rank choices to draw new ranks from
      return fail(c, SEKV_ERR_STATE, "layer " + std::to_string(l) + " was not built by sekv_build");
  }
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  HIPCHK(c, hipStreamIsCapturing(stream, &cs));
  if (cs != hipStreamCaptureStatusNone) return fail(c, SEKV_ERR_STATE, "re-segmentation is not capturable");
  // window rows, bases and cache tables are replaced below: nothing may still read them
  HIPCHK(c, hipDeviceSynchronize());

  // 1. host plan per sequence: row positions, leaving rows, runs
  std::vector<std::vector<int32_t>> pos(B), keep_rows(B), mem_rows(B);
  std::vector<std::vector<int32_t>> run_start(B), run_cnt(B), run_off(B);
  int nm_max = 1, nr_max = 1, any = 0;
  for (int b = 0; b < B; ++b) {
    const int R = c->layers[0].na_l[b];
    for (int l = 1; l < NL; ++l)
      if (c->layers[l].na_l[b] != R) return fail(c, SEKV_ERR_STATE, "layers hold different window rows: append to every layer");
    const int known = (int)c->row_pos[b].size();
    if (R < known) return fail(c, SEKV_ERR_STATE, "window rows fewer than recorded");
    pos[b] = c->row_pos[b];
    for (int i = 0; i < R - known; ++i) pos[b].push_back(c->next_pos[b] + i);
    const int n_tot = c->next_pos[b] + (R - known);
    if ((int)c->H_seq[b].size() < n_tot)
      return fail(c, SEKV_ERR_STATE, "surprisal missing for appended tokens (sekv_append_surprisal)");
    for (int i = 0; i < R; ++i) {
      const int p = pos[b][i];
      const bool leaving = p < n_tot - w && !((double)c->H_seq[b][p] > c->theta_b[b]);
      (leaving ? mem_rows[b] : keep_rows[b]).push_back(i);
    }
    // runs of consecutive positions (the rows are in position order)
    for (size_t j = 0; j < mem_rows[b].size(); ++j) {
      const int p = pos[b][mem_rows[b][j]];
      if (j > 0 && p == pos[b][mem_rows[b][j - 1]] + 1) {
        run_cnt[b].back()++;
      } else {
        run_start[b].push_back(p);
        run_cnt[b].push_back(1);
        run_off[b].push_back((int)j);
      }
    }
    if (c->m_b[b] + (int)run_start[b].size() > mm)
      return fail(c, SEKV_ERR_OOM, "no span rows left for the re-segmented window (sekv_reserve_spans)");
    nm_max = std::max(nm_max, (int)mem_rows[b].size());
    nr_max = std::max(nr_max, (int)run_start[b].size());
    any |= !run_start[b].empty();
  }
  if (!any) {
    // nothing leaves: only the positions of the rows appended since are recorded
    for (int b = 0; b < B; ++b) {
      const int known = (int)c->row_pos[b].size();
      if ((int)pos[b].size() > known) c->next_pos[b] = pos[b].back() + 1;
      c->row_pos[b] = pos[b];
    }
    return SEKV_OK;
  }

  // 2. device inputs shared by the layers: member row indices, their surprisal, the runs
  std::vector<int32_t> idx_h((size_t)B * nm_max, 0), cnt_h(B), kidx_h, kcnt_h(B);
  std::vector<float> Hm_h((size_t)B * nm_max, 0.f);
  std::vector<int32_t> tms_h((size_t)B * nr_max, 0), tmc_h((size_t)B * nr_max, 0), tmb_h(B);
  int nk_max = 1;
  for (int b = 0; b < B; ++b) nk_max = std::max(nk_max, (int)keep_rows[b].size());
  kidx_h.assign((size_t)B * nk_max, 0);
  for (int b = 0; b < B; ++b) {
    cnt_h[b] = (int)mem_rows[b].size();
    for (size_t j = 0; j < mem_rows[b].size(); ++j) {
      idx_h[(size_t)b * nm_max + j] = mem_rows[b][j];
      Hm_h[(size_t)b * nm_max + j] = c->H_seq[b][pos[b][mem_rows[b][j]]];
    }
    tmb_h[b] = (int)run_start[b].size();
    for (size_t j = 0; j < run_start[b].size(); ++j) {
      tms_h[(size_t)b * nr_max + j] = run_off[b][j];
      tmc_h[(size_t)b * nr_max + j] = run_cnt[b][j];
    }
    kcnt_h[b] = (int)keep_rows[b].size();
    for (size_t j = 0; j < keep_rows[b].size(); ++j) kidx_h[(size_t)b * nk_max + j] = keep_rows[b][j];
  }
  struct Tmp {
    std::vector<void*> p;
    ~Tmp() { for (void* q : p) if (q) (void)hipFree(q); }
  } tmp;
  auto talloc = [&](void** q, size_t bytes) -> sekv_status {
    TRY(dalloc(c, q, bytes));
    tmp.p.push_back(*q);
    return SEKV_OK;
  };
  int32_t *idx_d, *cnt_d, *kidx_d, *kcnt_d, *tms_d, *tmc_d, *tmb_d;
  float* Hm_d;
  TRY(talloc((void**)&idx_d, idx_h.size() * 4));
  TRY(talloc((void**)&cnt_d, (size_t)B * 4));
  TRY(talloc((void**)&kidx_d, kidx_h.size() * 4));
  TRY(talloc((void**)&kcnt_d, (size_t)B * 4));
  TRY(talloc((void**)&tms_d, tms_h.size() * 4));
  TRY(talloc((void**)&tmc_d, tmc_h.size() * 4));
  TRY(talloc((void**)&tmb_d, (size_t)B * 4));
  TRY(talloc((void**)&Hm_d, Hm_h.size() * 4));
  HIPCHK(c, hipMemcpy(idx_d, idx_h.data(), idx_h.size() * 4, hipMemcpyHostToDevice));
  HIPCHK(c, hipMemcpy(cnt_d, cnt_h.data(), (size_t)B * 4, hipMemcpyHostToDevice));
  HIPCHK(c, hipMemcpy(kidx_d, kidx_h.data(), kidx_h.size() * 4, hipMemcpyHostToDevice));
  HIPCHK(c, hipMemcpy(kcnt_d, kcnt_h.data(), (size_t)B * 4, hipMemcpyHostToDevice));
  HIPCHK(c, hipMemcpy(tms_d, tms_h.data(), tms_h.size() * 4, hipMemcpyHostToDevice));
  HIPCHK(c, hipMemcpy(tmc_d, tmc_h.data(), tmc_h.size() * 4, hipMemcpyHostToDevice));
  HIPCHK(c, hipMemcpy(tmb_d, tmb_h.data(), (size_t)B * 4, hipMemcpyHostToDevice));
  HIPCHK(c, hipMemcpy(Hm_d, Hm_h.data(), Hm_h.size() * 4, hipMemcpyHostToDevice));
  const size_t rows_t = (size_t)B * Hkv * nm_max, spans_t = (size_t)B * Hkv * nr_max;
  void *Kt, *Vt, *kb_t, *vb_t, *Kr_t = nullptr;
  int32_t *rank_t, *prob_t;
  int64_t* boff_t;
  TRY(talloc(&Kt, rows_t * d * es));
  TRY(talloc(&Vt, rows_t * d * es));
  TRY(talloc(&kb_t, spans_t * d * es));
  TRY(talloc(&vb_t, spans_t * d * es));
  TRY(talloc((void**)&rank_t, spans_t * 4));
  TRY(talloc((void**)&boff_t, spans_t * 8));
  TRY(talloc((void**)&prob_t, spans_t * 2 * 3 * 4));

  for (int layer = 0; layer < NL; ++layer) {
    LayerState& L = c->layers[layer];
    const int dr = c->route[layer].dr;
    // 3. the leaving rows of this layer, in run order
    GatherArgs ga;
    ga.Hkv = Hkv;
    ga.in_rows = L.na_cap;
    ga.out_rows = nm_max;
    ga.idx = idx_d;
    ga.idx_stride = nm_max;
    ga.cnt = cnt_d;
    ga.row_bytes = (int)(d * es);
    ga.max_cnt = nm_max;
    ga.in = L.KA;
    ga.out = Kt;
    launch_gather_rows(B, ga, stream);
    ga.in = L.VA;
    ga.out = Vt;
    launch_gather_rows(B, ga, stream);
    HIPCHK(c, hipGetLastError());
    // 4. summaries of the new spans (and routing summaries)
    if (dr > 0 && !Kr_t) TRY(talloc(&Kr_t, spans_t * dr * es));
    SummaryArgs su;
    std::memset(&su, 0, sizeof(su));
    su.H = Hm_d;
    su.K = Kt;
    su.V = Vt;
    su.B = B;
    su.Hkv = Hkv;
    su.n = nm_max;
    su.m_max = nr_max;
    su.m_b = tmb_d;
    su.mstart = tms_d;
    su.mcount = tmc_d;
    su.kbar = kb_t;
    su.vbar = vb_t;
    su.span_chunk = 16;
    su.n_span_chunks = (nr_max + 15) / 16;
    su.n_anchor_chunks = 0;
    su.dr = dr;
    su.Wr = c->route[layer].W_d;
    su.Kr = Kr_t;
    launch_summaries(d, c->bf16, su, stream);
    HIPCHK(c, hipGetLastError());
    // 5. ranks, the new layout of the basis store (each head's spans stay contiguous)
    const int nch = (int)L.choices.size();
    std::vector<int32_t> rank_th(spans_t, 1);
    std::vector<int64_t> boff_th(spans_t, 0);
    std::vector<int64_t> nbase((size_t)B * Hkv + 1, 0), add((size_t)B * Hkv, 0);
    int64_t new_tot = 0, tmp_tot = 0;
    std::vector<int32_t> probs[5];
    for (int b = 0; b < B; ++b)
      for (int g = 0; g < Hkv; ++g) {
        const size_t bg = (size_t)b * Hkv + g;
        nbase[bg] = new_tot;
        const int64_t old_len = L.head_base[bg + 1] - L.head_base[bg];
        int64_t extra = 0;
        for (int j = 0; j < tmb_h[b]; ++j) {
          const int cnt = run_cnt[b][j], k = c->m_b[b] + j;
          const uint64_t key = L.seed ^ ((uint64_t)layer << 40) ^ ((uint64_t)g << 32) ^ (uint64_t)k;
          int r = L.choices[splitmix64(key) % (uint64_t)nch];
          r = std::min(r, std::min(cnt, d));
          rank_th[bg * nr_max + j] = r;
          boff_th[bg * nr_max + j] = tmp_tot;
          const int64_t el = span_elems(cnt, r, d);
          tmp_tot += el;
          extra += el;
          const int bk = cnt <= 16 ? 0 : cnt <= 32 ? 1 : cnt <= 64 ? 2 : cnt <= 128 ? 3 : 4;
          for (int wv = 0; wv < 2; ++wv) {
            probs[bk].push_back((int)bg);
            probs[bk].push_back(j);
            probs[bk].push_back(wv);
          }
        }
        add[bg] = extra;
        new_tot += old_len + extra;
      }
    nbase[(size_t)B * Hkv] = new_tot;
    if ((new_tot >> 3) >= ((int64_t)1 << 32)) return fail(c, SEKV_ERR_INVALID, "basis store exceeds 2^35 elements");
    void* newb = nullptr;
    TRY(talloc(&newb, (size_t)std::max<int64_t>(tmp_tot, 8) * es));
    HIPCHK(c, hipMemcpy(rank_t, rank_th.data(), spans_t * 4, hipMemcpyHostToDevice));
    HIPCHK(c, hipMemcpy(boff_t, boff_th.data(), spans_t * 8, hipMemcpyHostToDevice));
    // 6. truncated SVD of the new spans into the temporary store
    SvdArgs sv;
    sv.K = Kt;
    sv.V = Vt;
    sv.Hkv = Hkv;
    sv.n = nm_max;
    sv.m_max = nr_max;
    sv.mstart = tms_d;
    sv.mcount = tmc_d;
    sv.rank = rank_t;
    sv.boff = boff_t;
    sv.bases = newb;
    const int cmax[5] = {16, 32, 64, 128, 0};
    for (int i = 0; i < 5; ++i) {
      if (probs[i].empty()) continue;
      HIPCHK(c, hipMemcpy(prob_t, probs[i].data(), probs[i].size() * 4, hipMemcpyHostToDevice));
      sv.problems = prob_t;
      sv.n_problems = (int)(probs[i].size() / 3);
      HIPCHK(c, launch_svd(cmax[i], d, c->bf16, sv, stream));
      HIPCHK(c, hipStreamSynchronize(stream));  // prob_t is reused by the next bucket
    }
    // 7. the new store: each head's old spans, then its new ones
    void* nstore_d = nullptr;
    void* nstore_h = nullptr;
    if (host_store(c)) {
      TRY(halloc(c, &nstore_h, (size_t)std::max<int64_t>(new_tot, 8) * es));
    } else {
      TRY(dalloc(c, &nstore_d, (size_t)std::max<int64_t>(new_tot, 8) * es));
    }
    for (size_t bg = 0; bg < (size_t)B * Hkv; ++bg) {
      const int64_t old_len = L.head_base[bg + 1] - L.head_base[bg];
      if (host_store(c)) {
        std::memcpy((char*)nstore_h + (size_t)nbase[bg] * es, (char*)L.bases_h + (size_t)L.head_base[bg] * es,
                    (size_t)old_len * es);
      } else if (old_len) {
        HIPCHK(c, hipMemcpyAsync((char*)nstore_d + (size_t)nbase[bg] * es, (char*)L.bases_d + (size_t)L.head_base[bg] * es,
                                 (size_t)old_len * es, hipMemcpyDeviceToDevice, stream));
      }
      const int b = (int)(bg / Hkv);
      if (add[bg] && tmb_h[b]) {
        const int64_t src = boff_th[bg * nr_max + 0];
        HIPCHK(c, hipMemcpyAsync(host_store(c) ? (void*)((char*)nstore_h + (size_t)(nbase[bg] + old_len) * es)
                                               : (void*)((char*)nstore_d + (size_t)(nbase[bg] + old_len) * es),
                                 (char*)newb + (size_t)src * es, (size_t)add[bg] * es,
                                 host_store(c) ? hipMemcpyDeviceToHost : hipMemcpyDeviceToDevice, stream));
      }
    }
    // 8. summaries (and routing summaries) of the new spans into the layer's rows
    for (int b = 0; b < B; ++b) {
      if (!tmb_h[b]) continue;
      for (int g = 0; g < Hkv; ++g) {
        const size_t bg = (size_t)b * Hkv + g;
        const size_t dst = bg * mm + c->m_b[b], srcr = bg * nr_max;
        HIPCHK(c, hipMemcpyAsync((char*)L.kbar + dst * d * es, (char*)kb_t + srcr * d * es, (size_t)tmb_h[b] * d * es,
                                 hipMemcpyDeviceToDevice, stream));
        HIPCHK(c, hipMemcpyAsync((char*)L.vbar + dst * d * es, (char*)vb_t + srcr * d * es, (size_t)tmb_h[b] * d * es,
                                 hipMemcpyDeviceToDevice, stream));
        if (dr > 0)
          HIPCHK(c, hipMemcpyAsync((char*)L.Kr + dst * dr * es, (char*)Kr_t + srcr * dr * es,
                                   (size_t)tmb_h[b] * dr * es, hipMemcpyDeviceToDevice, stream));
      }
    }
    // 9. the window rows that stay, compacted
    void *nKA, *nVA;
    TRY(dalloc(c, &nKA, (size_t)B * Hkv * L.na_cap * d * es));
    sekv_status st2 = dalloc(c, &nVA, (size_t)B * Hkv * L.na_cap * d * es);
    if (st2 != SEKV_OK) {
      dfree(nKA);
      return st2;
    }
    GatherArgs gk;
    gk.Hkv = Hkv;
    gk.in_rows = L.na_cap;
    gk.out_rows = L.na_cap;
    gk.idx = kidx_d;
    gk.idx_stride = nk_max;
    gk.cnt = kcnt_d;
    gk.row_bytes = (int)(d * es);
    gk.max_cnt = nk_max;
    gk.in = L.KA;
    gk.out = nKA;
    launch_gather_rows(B, gk, stream);
    gk.in = L.VA;
    gk.out = nVA;
    launch_gather_rows(B, gk, stream);
    HIPCHK(c, hipGetLastError());
    HIPCHK(c, hipStreamSynchronize(stream));
    dfree(L.KA);
    dfree(L.VA);
    L.KA = nKA;
    L.VA = nVA;
    // 10. tables: ranks, offsets, metadata, counts
    for (int b = 0; b < B; ++b)
      for (int g = 0; g < Hkv; ++g) {
        const size_t bg = (size_t)b * Hkv + g;
        for (int k = 0; k < c->m_b[b]; ++k) L.boff_h[bg * mm + k] += nbase[bg] - L.head_base[bg];
        const int64_t old_len = L.head_base[bg + 1] - L.head_base[bg];
        int64_t o = nbase[bg] + old_len;
        for (int j = 0; j < tmb_h[b]; ++j) {
          const size_t i = bg * mm + c->m_b[b] + j;
          L.rank_h[i] = rank_th[bg * nr_max + j];
          L.boff_h[i] = o;
          o += span_elems(run_cnt[b][j], L.rank_h[i], d);
        }
      }
    L.head_base = nbase;
    L.basis_elems = new_tot;
    if (host_store(c)) {
      hfree(L.bases_h);
      L.bases_h = nstore_h;
      HIPCHK(c, hipHostGetDevicePointer(&L.bases_hd, L.bases_h, 0));
    } else {
      dfree(L.bases_d);
      L.bases_d = nstore_d;
    }
    for (int b = 0; b < B; ++b) L.na_l[b] = kcnt_h[b];
    HIPCHK(c, hipMemcpy(L.na_l_d, L.na_l.data(), (size_t)B * 4, hipMemcpyHostToDevice));
    const size_t rows_m = (size_t)B * Hkv * mm;
    HIPCHK(c, hipMemcpy(L.rank_d, L.rank_h.data(), rows_m * 4, hipMemcpyHostToDevice));
    HIPCHK(c, hipMemcpy(L.boff_d, L.boff_h.data(), rows_m * 8, hipMemcpyHostToDevice));
    {
      std::vector<int2> meta(rows_m, make_int2(0, 0));
      for (int b = 0; b < B; ++b)
        for (int g = 0; g < Hkv; ++g)
          for (int k = 0; k < c->m_b[b] + tmb_h[b]; ++k) {
            const size_t i = ((size_t)b * Hkv + g) * mm + k;
            const int cnt = k < c->m_b[b] ? c->mcount[b][k] : run_cnt[b][k - c->m_b[b]];
            meta[i] = make_int2((int)(uint32_t)(L.boff_h[i] >> 3), L.rank_h[i] | (cnt << 8));
          }
      HIPCHK(c, hipMemcpy(L.smeta_d, meta.data(), rows_m * sizeof(int2), hipMemcpyHostToDevice));
    }
    free_layer_cache(L.lc);
    L.sched.valid = false;
    L.sched.anchors_changed = true;
  }

  // 11. the shared span table
  for (int b = 0; b < B; ++b) {
    for (size_t j = 0; j < run_start[b].size(); ++j) {
      c->mstart[b].push_back(run_start[b][j]);
      c->mcount[b].push_back(run_cnt[b][j]);
    }
    c->m_b[b] = (int)c->mstart[b].size();
    std::vector<int32_t> kept;
    for (int r : keep_rows[b]) kept.push_back(pos[b][r]);
    c->next_pos[b] = pos[b].empty() ? c->next_pos[b] : std::max(c->next_pos[b], pos[b].back() + 1);
    c->row_pos[b] = kept;
    c->anchors[b] = kept;
    c->na_b[b] = (int)kept.size();
  }
  {
    std::vector<int32_t> ms((size_t)B * mm, 0), mc((size_t)B * mm, 0);
    std::vector<float> ls((size_t)B * mm, 0.f);
    for (int b = 0; b < B; ++b)
      for (int k = 0; k < c->m_b[b]; ++k) {
        ms[(size_t)b * mm + k] = c->mstart[b][k];
        mc[(size_t)b * mm + k] = c->mcount[b][k];
        ls[(size_t)b * mm + k] = (float)std::log((double)c->mcount[b][k]);
      }
    HIPCHK(c, hipMemcpy(c->mstart_d, ms.data(), ms.size() * 4, hipMemcpyHostToDevice));
    HIPCHK(c, hipMemcpy(c->mcount_d, mc.data(), mc.size() * 4, hipMemcpyHostToDevice));
    HIPCHK(c, hipMemcpy(c->logS_d, ls.data(), ls.size() * 4, hipMemcpyHostToDevice));
    HIPCHK(c, hipMemcpy(c->m_b_d, c->m_b.data(), (size_t)B * 4, hipMemcpyHostToDevice));
    HIPCHK(c, hipMemcpy(c->na_b_d, c->na_b.data(), (size_t)B * 4, hipMemcpyHostToDevice));
  }
  c->resegmented = true;
  return SEKV_OK;
}

// ---------------------------------------------------------------------------- decode-time append

sekv_status sekv_append_tokens(sekv_ctx* c, int32_t layer, const void* K_new, const void* V_new, int32_t n_new,
                               hipStream_t stream) {
  if (!c) return fail(nullptr, SEKV_ERR_INVALID, "NULL context");
  DevGuard dg(c->cfg.device);
  TRY(check_layer(c, layer));
  if (n_new < 0) return fail(c, SEKV_ERR_INVALID, "n_new < 0");
  if (n_new == 0) return SEKV_OK;
  if (!K_new || !V_new) return fail(c, SEKV_ERR_INVALID, "NULL K_new or V_new");
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  HIPCHK(c, hipStreamIsCapturing(stream, &cs));
  if (cs != hipStreamCaptureStatusNone) return fail(c, SEKV_ERR_STATE, "append is not capturable");
  LayerState& L = c->layers[layer];
  const int B = c->cfg.batch, Hkv = c->cfg.n_kv_heads, d = c->cfg.d_head;
  int need = 0;
  for (int b = 0; b < B; ++b) need = std::max(need, L.na_l[b] + n_new);
  if ((int64_t)need >= ((int64_t)1 << 30)) return fail(c, SEKV_ERR_INVALID, "window too large");
  if (need > L.na_cap) {
    // grow the anchor rows of every (b, g) by half at least, keeping the rows in place
    const int cap = std::max(need, L.na_cap + L.na_cap / 2 + 64);
    const size_t es = c->esz, rows = (size_t)B * Hkv * cap;
    void* nk = nullptr;
    void* nv = nullptr;
    TRY(dalloc(c, &nk, rows * d * es));
    sekv_status st = dalloc(c, &nv, rows * d * es);
    if (st != SEKV_OK) {
      dfree(nk);
      return st;
    }
    hipError_t e = hipSuccess;
    if (L.na_cap > 0) {
      const size_t src_pitch = (size_t)L.na_cap * d * es, dst_pitch = (size_t)cap * d * es;
      e = hipMemcpy2DAsync(nk, dst_pitch, L.KA, src_pitch, src_pitch, (size_t)B * Hkv, hipMemcpyDeviceToDevice,
                           stream);
      if (e == hipSuccess)
        e = hipMemcpy2DAsync(nv, dst_pitch, L.VA, src_pitch, src_pitch, (size_t)B * Hkv, hipMemcpyDeviceToDevice,
                             stream);
    }
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) {
      dfree(nk);
      dfree(nv);
      return fail(c, SEKV_ERR_HIP, std::string("growing the window: ") + hipGetErrorString(e));
    }
    dfree(L.KA);
    dfree(L.VA);
    L.KA = nk;
    L.VA = nv;
    L.na_cap = cap;
  }
  AppendArgs ap;
  ap.K_new = K_new;
  ap.V_new = V_new;
  ap.KA = L.KA;
  ap.VA = L.VA;
  ap.na = L.na_l_d;
  ap.Hkv = Hkv;
  ap.n_new = n_new;
  ap.na_cap = L.na_cap;
  launch_append(d, c->bf16, B, ap, stream);
  HIPCHK(c, hipGetLastError());
  for (int b = 0; b < B; ++b) L.na_l[b] += n_new;
  L.sched.anchors_changed = true;
  c->stats.tokens_appended += (uint64_t)n_new * B;
  return SEKV_OK;
}

sekv_status sekv_get_window(const sekv_ctx* cc, int32_t layer, int32_t b, int32_t* n_anchors) {
  sekv_ctx* c = const_cast<sekv_ctx*>(cc);
  if (!c) return fail(nullptr, SEKV_ERR_INVALID, "NULL context");
  if (layer < 0 || layer >= c->cfg.n_layers || b < 0 || b >= c->cfg.batch || !n_anchors)
    return fail(c, SEKV_ERR_INVALID, "bad argument");
  const LayerState& L = c->layers[layer];
  if (!L.allocated) return fail(c, SEKV_ERR_STATE, "layer has no layout");
  *n_anchors = L.na_l[b];
  return SEKV_OK;
}

// ---------------------------------------------------------------------------- routing projection, rank gates

sekv_status sekv_set_routing(sekv_ctx* c, int32_t layer, int32_t d_route, const float* W) {
  if (!c) return fail(nullptr, SEKV_ERR_INVALID, "NULL context");
  DevGuard dg(c->cfg.device);
  const int Hkv = c->cfg.n_kv_heads, d = c->cfg.d_head;
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(c, SEKV_ERR_INVALID, "layer out of range");
  if (c->layers[layer].allocated)
    return fail(c, SEKV_ERR_STATE, "the layer already has a layout: set its routing projection first");
  if (d_route != 0 && (d_route < 8 || d_route > d || d_route % 8 != 0))
    return fail(c, SEKV_ERR_INVALID, "d_route must be 0 or a multiple of 8 in [8, d_head]");
  RouteProj& R = c->route[layer];
  if (d_route == 0) {
    dfree(R.W_d);
    R.dr = 0;
    return SEKV_OK;
  }
  if (!W) return fail(c, SEKV_ERR_INVALID, "NULL W");
  const size_t nw = (size_t)Hkv * d_route * d;
  for (size_t i = 0; i < nw; ++i)
    if (!std::isfinite(W[i])) return fail(c, SEKV_ERR_INVALID, "W is not finite");
  dfree(R.W_d);
  R.dr = 0;
  TRY(dalloc(c, &R.W_d, nw * sizeof(float)));
  HIPCHK(c, hipMemcpy(R.W_d, W, nw * sizeof(float), hipMemcpyHostToDevice));
  R.dr = d_route;
  return SEKV_OK;
}

sekv_status sekv_import_route_summary(sekv_ctx* c, int32_t layer, int32_t b, int32_t g, const void* Kr) {
  if (!c) return fail(nullptr, SEKV_ERR_INVALID, "NULL context");
  DevGuard dg(c->cfg.device);
  const int B = c->cfg.batch, Hkv = c->cfg.n_kv_heads;
  if (layer < 0 || layer >= c->cfg.n_layers || b < 0 || b >= B || g < 0 || g >= Hkv)
    return fail(c, SEKV_ERR_INVALID, "index out of range");
  LayerState& L = c->layers[layer];
  const int dr = c->route[layer].dr;
  if (!L.allocated) return fail(c, SEKV_ERR_STATE, "layer has no layout (sekv_import_layout)");
  if (dr == 0 || !L.Kr) return fail(c, SEKV_ERR_STATE, "the layer has no routing projection");
  const int m = c->m_b[b];
  if (m && !Kr) return fail(c, SEKV_ERR_INVALID, "NULL Kr");
  const size_t bg = (size_t)b * Hkv + g;
  if (m)
    HIPCHK(c, hipMemcpy((char*)L.Kr + bg * c->m_max * dr * c->esz, Kr, (size_t)m * dr * c->esz,
                        hipMemcpyHostToDevice));
  L.route_set[bg] = 1;
  update_ready(L);
  return SEKV_OK;
}

sekv_status sekv_export_route_summary(const sekv_ctx* cc, int32_t layer, int32_t b, int32_t g, void* Kr) {
  sekv_ctx* c = const_cast<sekv_ctx*>(cc);
  if (!c) return fail(nullptr, SEKV_ERR_INVALID, "NULL context");
  DevGuard dg(c->cfg.device);
  const int B = c->cfg.batch, Hkv = c->cfg.n_kv_heads;
  if (layer < 0 || layer >= c->cfg.n_layers || b < 0 || b >= B || g < 0 || g >= Hkv)
    return fail(c, SEKV_ERR_INVALID, "index out of range");
  LayerState& L = c->layers[layer];
  const int dr = c->route[layer].dr;
  const size_t bg = (size_t)b * Hkv + g;
  if (!L.allocated || dr == 0 || !L.Kr || !L.route_set[bg])
    return fail(c, SEKV_ERR_STATE, "no routing summaries for this head");
  const int m = c->m_b[b];
  if (m && Kr)
    HIPCHK(c, hipMemcpy(Kr, (char*)L.Kr + bg * c->m_max * dr * c->esz, (size_t)m * dr * c->esz,
                        hipMemcpyDeviceToHost));
  return SEKV_OK;
}

sekv_status sekv_apply_rank_gates(sekv_ctx* c, int32_t layer, int32_t b, int32_t g, const float* gate_k,
                                  const float* gate_v, hipStream_t stream) {
  if (!c) return fail(nullptr, SEKV_ERR_INVALID, "NULL context");
  DevGuard dg(c->cfg.device);
  const int B = c->cfg.batch, Hkv = c->cfg.n_kv_heads, d = c->cfg.d_head;
  if (layer < 0 || layer >= c->cfg.n_layers || b < 0 || b >= B || g < 0 || g >= Hkv)
    return fail(c, SEKV_ERR_INVALID, "index out of range");
  LayerState& L = c->layers[layer];
  const size_t bg = (size_t)b * Hkv + g;
  if (!L.allocated || !L.head_set[bg]) return fail(c, SEKV_ERR_STATE, "head has no artefacts");
  const int m = c->m_b[b], mm = c->m_max;
  if (m == 0 || (!gate_k && !gate_v)) return SEKV_OK;
  for (int w = 0; w < 2; ++w) {
    const float* gt = w == 0 ? gate_k : gate_v;
    if (!gt) continue;
    for (int k = 0; k < m; ++k) {
      const int r = L.rank_h[bg * mm + k];
      for (int i = 0; i < r; ++i) {
        const float x = gt[(size_t)k * d + i];
        if (!(x >= 0.f && x <= 1.f))
          return fail(c, SEKV_ERR_INVALID, "gate outside [0, 1] at span " + std::to_string(k));
      }
    }
  }
  // the gated factors replace the stored ones: cached copies of this layer's
  // bases go, and no prefetch copy may read a half-gated span
  HIPCHK(c, invalidate_layer_cache(L));
  float* g_d = nullptr;
  const size_t ng = (size_t)m * d;
  TRY(dalloc(c, &g_d, 2 * ng * sizeof(float)));
  GateArgs ga;
  ga.bases = host_store(c) ? L.bases_hd : L.bases_d;
  ga.boff = L.boff_d + bg * mm;
  ga.rank = L.rank_d + bg * mm;
  ga.mcount = c->mcount_d + (size_t)b * mm;
  ga.gk = gate_k ? g_d : nullptr;
  ga.gv = gate_v ? g_d + ng : nullptr;
  ga.m = m;
  ga.d = d;
  hipError_t e = hipSuccess;
  if (gate_k) e = hipMemcpyAsync(g_d, gate_k, ng * sizeof(float), hipMemcpyHostToDevice, stream);
  if (e == hipSuccess && gate_v) e = hipMemcpyAsync(g_d + ng, gate_v, ng * sizeof(float), hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) {
    launch_rank_gates(c->bf16, ga, stream);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  dfree(g_d);
  if (e != hipSuccess) return fail(c, SEKV_ERR_HIP, std::string("rank gates: ") + hipGetErrorString(e));
  return SEKV_OK;
}

sekv_status sekv_get_zoom_counts(sekv_ctx* c, int32_t layer, uint64_t* counts, uint64_t* calls, int32_t reset) {
  if (!c) return fail(nullptr, SEKV_ERR_INVALID, "NULL context");
  DevGuard dg(c->cfg.device);
  if (layer < 0 || layer >= c->cfg.n_layers)
    return fail(c, SEKV_ERR_INVALID, "layer " + std::to_string(layer) + " out of range");
  LayerState& L = c->layers[layer];
  if (!L.zcount_d) return fail(c, SEKV_ERR_STATE, "layer has no layout");
  const size_t n = (size_t)c->cfg.batch * c->cfg.n_q_heads;
  std::vector<unsigned long long> h(n + 1);
  HIPCHK(c, hipDeviceSynchronize());  // every decode call that updates the counters has finished
  HIPCHK(c, hipMemcpy(h.data(), L.zcount_d, (n + 1) * sizeof(unsigned long long), hipMemcpyDeviceToHost));
  if (counts)
    for (size_t i = 0; i < n; ++i) counts[i] = h[i];
  if (calls) *calls = h[n];
  if (reset) HIPCHK(c, hipMemset(L.zcount_d, 0, (n + 1) * sizeof(unsigned long long)));
  return SEKV_OK;
}

sekv_status sekv_get_stats(const sekv_ctx* cc, sekv_stats* out) {
  sekv_ctx* c = const_cast<sekv_ctx*>(cc);
  if (!c || !out) return fail(c, SEKV_ERR_INVALID, "NULL argument");
  sekv_stats s = c->stats;
  const int B = c->cfg.batch, Hkv = c->cfg.n_kv_heads, d = c->cfg.d_head;
  int64_t dev = 0, host = 0;
  for (size_t li = 0; li < c->layers.size(); ++li) {
    const LayerState& L = c->layers[li];
    if (!L.allocated) continue;
    dev += (int64_t)2 * B * Hkv * (c->m_max + L.na_cap) * d * c->esz;   // summaries + anchors
    dev += (int64_t)B * Hkv * c->m_max * c->route[li].dr * c->esz;       // routing summaries
    dev += (int64_t)B * Hkv * c->m_max * 12;                              // rank + offset tables
    if (c->cfg.basis_home == SEKV_BASES_DEVICE) dev += L.basis_elems * c->esz;
    else host += L.basis_elems * c->esz;
  }
  s.device_resident_bytes = dev;
  s.host_basis_bytes = host;
  *out = s;
  return SEKV_OK;
}

}  // extern "C"
