// Host planner of the planned decode kernel: the cut of a layer-step's work
// into one share per workgroup.  Plain C++ with no GPU types, so that its
// invariants can be checked on any host.
//
// The work of a layer-step is the sequence "span rows of (b, g), anchor rows
// of (b, g)" over the (sequence, kv head) pairs bg = b * Hkv + g in order.  A
// share is a list of at most `segs_per_share` segments and `max_span_rows` span
// rows; each segment is a run of span rows or of anchor rows of one bg and gets
// the next partial slot of that bg.
#pragma once

#include <cstdint>
#include <vector>

namespace sekv {

// One segment: (bg | 1 << 31 for anchor rows, first row, rows, partial slot).
// A share's list is padded with all-zero segments (rows = 0 ends a list).
struct PlanSeg {
  int32_t x, y, z, w;
};

struct PlanInput {
  int B = 0, Hkv = 0;          // sequences, kv heads
  int d = 0;                   // head dimension (also the tokens of a zoom unit)
  int esz = 0;                 // bytes per stored key or value element
  int m_max = 0;               // row stride of rank and zprob
  int segs_per_share = 0;      // segment slots of a share's list
  int max_span_rows = 0;       // span rows of a share
  int max_parts = 0;           // partial slots of one bg
  const int32_t* m = nullptr;            // [B] spans of each sequence
  const int32_t* na = nullptr;           // [B] anchor rows of each sequence
  const int32_t* const* count = nullptr; // [B][m[b]] tokens of each span
  const int32_t* rank = nullptr;         // [B * Hkv * m_max] kept rank of each span's bases
  const float* zprob = nullptr;          // [B * Hkv * m_max] zoom frequency of each span row
  const float* zunits = nullptr;         // [B * Hkv] expected zoomed units of each bg, or null
  double span_cost = 2.0;      // cost of a span row in anchor rows
  double unit_cost = 12288.0;  // fixed cost of a zoomed unit, in bytes
  double zdev = 1.5;           // standard deviations of zoom work charged to a share
};

struct PlanOut {
  std::vector<PlanSeg> segs;   // [n_shares * segs_per_share]
  std::vector<int32_t> parts;  // [B * Hkv] partial slots of each bg
  int n_shares = 0;
  int max_parts = 1;           // the largest parts entry (at least 1)
  double budget = 0.0;
};

// Cut the work into shares whose charged cost (streamed bytes, plus the
// expected zoom work and zdev standard deviations of it) stays within
// `budget`; a share takes at least one row.  Returns the number of shares.
// With out == nullptr only counts, and returns INT32_MAX when some bg would
// need more than max_parts slots.
int plan_cut(const PlanInput& in, double budget, PlanOut* out);

// Expected bytes of the layer-step: span rows (two rows of keys and values
// each), anchor rows, and the zoomed units' bases (16 KB each).
double plan_expected_bytes(const PlanInput& in);

// The smallest budget (within 0.5%) that cuts the work into at most `target`
// shares, and its cut.  When the per-share row and segment limits need more
// shares than `target`, the cut takes the smallest count they allow; the
// search for a budget is bounded.  Returns the number of shares.
int plan_shares(const PlanInput& in, int target, PlanOut* out);

}  // namespace sekv
