// Host planner of the planned decode kernel (see plan.h).
#include "plan.h"

#include <algorithm>
#include <climits>
#include <cmath>

namespace sekv {

namespace {
inline int64_t pad8_host(int64_t x) { return (x + 7) & ~int64_t(7); }
}  // namespace

// Costs are in bytes of anchor streaming: an anchor row streams its key and
// value; a span row, which also routes, is charged span_cost anchor rows; a
// zoomed span adds, for each of its d-token units, the unit's bases and a
// fixed cost for its dependent round of loads, times the span's zoom
// frequency.  The zoom sets move from call to call (spans near the threshold
// flip with the query), so a share is charged its expected zoom work plus
// zdev standard deviations of it.
int plan_cut(const PlanInput& in, double budget, PlanOut* out) {
  const int B = in.B, Hkv = in.Hkv, BH = B * Hkv, d = in.d, NS = in.segs_per_share, mm = in.m_max;
  const double row = 2.0 * d * (double)in.esz;
  const double span_row = row * in.span_cost;
  const double unit_cost = in.unit_cost;
  const double zdev = in.zdev;
  std::vector<PlanSeg> segs;
  std::vector<int32_t> parts(BH, 0);
  std::vector<PlanSeg> cur;
  int span_rows = 0, nwg = 0;
  double mean = 0.0, var = 0.0;
  auto cost = [&]() { return mean + zdev * std::sqrt(var); };
  auto close_wg = [&]() {
    if (cur.empty()) return;
    if (out) {
      for (auto& x : cur) segs.push_back(x);
      for (int i = (int)cur.size(); i < NS; ++i) segs.push_back(PlanSeg{0, 0, 0, 0});
    }
    cur.clear();
    span_rows = 0;
    mean = var = 0.0;
    ++nwg;
  };
  for (int bg = 0; bg < BH; ++bg) {
    const int b = bg / Hkv;
    const int m = in.m[b], na = in.na[b];
    for (int k = 0; k < m;) {
      if ((int)cur.size() == NS || span_rows >= in.max_span_rows) close_wg();
      int n = 0;
      while (k < m && span_rows < in.max_span_rows) {
        const float pz = in.zprob[(size_t)bg * mm + k];
        double zm = 0.0, zv = 0.0;
        if (pz > 0.f) {
          const int cnt = in.count[b][k], r = in.rank[(size_t)bg * mm + k];
          const double work = 2.0 * (pad8_host(cnt) + d) * r * in.esz + ((cnt + d - 1) / d) * unit_cost;
          zm = pz * work;
          zv = pz * (1.0 - pz) * work * work;
        }
        const double m2 = mean + span_row + zm, v2 = var + zv;
        if (n > 0 || !cur.empty()) {
          // the row goes to the next share when it would take this one over budget
          if (m2 + zdev * std::sqrt(v2) > budget && cost() > 0.5 * budget) break;
        }
        mean = m2;
        var = v2;
        ++k;
        ++n;
        ++span_rows;
      }
      if (n > 0) cur.push_back(PlanSeg{bg, k - n, n, parts[bg]++});
      if (k < m) close_wg();
    }
    for (int r = 0; r < na;) {
      if ((int)cur.size() == NS) close_wg();
      // (clamped before the conversion: a large budget must not overflow int)
      int n = (int)std::min(std::floor((budget - cost()) / row), (double)(na - r));
      if (n < 1) {
        if (!cur.empty()) {
          close_wg();
          continue;
        }
        n = 1;
      }
      n = std::min(n, na - r);
      mean += n * row;
      cur.push_back(PlanSeg{bg | (int32_t)0x80000000u, r, n, parts[bg]++});
      r += n;
      if (r < na) close_wg();
    }
  }
  close_wg();
  int mp = 1;
  for (int bg = 0; bg < BH; ++bg) mp = std::max(mp, parts[bg]);
  if (out) {
    out->segs.swap(segs);
    out->parts.swap(parts);
    out->n_shares = nwg;
    out->max_parts = mp;
    out->budget = budget;
  } else if (mp > in.max_parts) {
    return INT32_MAX;  // too many slots for one bg: a larger budget is needed
  }
  return nwg;
}

double plan_expected_bytes(const PlanInput& in) {
  const double row = 2.0 * in.d * (double)in.esz;
  double total = 0.0;
  for (int bg = 0; bg < in.B * in.Hkv; ++bg) {
    const int b = bg / in.Hkv;
    total += (double)in.m[b] * 2.0 * row + (double)in.na[b] * row;
    if (in.zunits) total += in.zunits[bg] * 16384.0;
  }
  return total;
}

int plan_shares(const PlanInput& in, int target, PlanOut* out) {
  const double total = plan_expected_bytes(in);
  double lo = 0.25 * total / target, hi = 2.0 * total / target + 1.0;
  // the share count falls as the budget grows, down to a floor set by the
  // per-share row and segment limits; when that floor is above the target no
  // budget reaches it, and the cut takes the floor
  int n_hi = plan_cut(in, hi, nullptr);
  for (int it = 0; it < 40 && n_hi > target; ++it) {
    hi *= 2.0;
    n_hi = plan_cut(in, hi, nullptr);
  }
  if (n_hi <= target) {
    for (int it = 0; it < 16 && hi - lo > 0.005 * hi; ++it) {
      const double mid = 0.5 * (lo + hi);
      if (plan_cut(in, mid, nullptr) > target) lo = mid;
      else hi = mid;
    }
  }
  return plan_cut(in, hi, out);
}

}  // namespace sekv
