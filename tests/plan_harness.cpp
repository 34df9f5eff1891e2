// C entry points over the host planner of the planned decode kernel, for the
// CPU tests (built with g++ together with the package's plan.cpp).
#include <cstring>
#include <vector>

#include "plan.h"

using namespace sekv;

namespace {
PlanInput make_input(int B, int Hkv, int d, int esz, int m_max, int ns, int max_span_rows, int max_parts,
                     const int* m, const int* na, const int* count, const int* rank, const float* zprob,
                     const float* zunits, double span_cost, double unit_cost, double zdev,
                     std::vector<const int32_t*>& rows) {
  rows.resize(B);
  for (int b = 0; b < B; ++b) rows[b] = count + (size_t)b * m_max;
  PlanInput in;
  in.B = B;
  in.Hkv = Hkv;
  in.d = d;
  in.esz = esz;
  in.m_max = m_max;
  in.segs_per_share = ns;
  in.max_span_rows = max_span_rows;
  in.max_parts = max_parts;
  in.m = m;
  in.na = na;
  in.count = rows.data();
  in.rank = rank;
  in.zprob = zprob;
  in.zunits = zunits;
  in.span_cost = span_cost;
  in.unit_cost = unit_cost;
  in.zdev = zdev;
  return in;
}

int emit(const PlanOut& po, int* segs, int cap, int* parts, int bh, double* budget) {
  if ((int)po.segs.size() * 4 > cap) return -1;
  for (size_t i = 0; i < po.segs.size(); ++i) {
    segs[4 * i] = po.segs[i].x;
    segs[4 * i + 1] = po.segs[i].y;
    segs[4 * i + 2] = po.segs[i].z;
    segs[4 * i + 3] = po.segs[i].w;
  }
  std::memcpy(parts, po.parts.data(), (size_t)bh * sizeof(int));
  *budget = po.budget;
  return po.n_shares;
}
}  // namespace

extern "C" {

// plan_cut with budget > 0 (count only when segs is NULL), plan_shares with
// target > 0 otherwise.  Returns the share count, or -1 when segs is too short.
int harness_plan(int B, int Hkv, int d, int esz, int m_max, int ns, int max_span_rows, int max_parts,
                 const int* m, const int* na, const int* count, const int* rank, const float* zprob,
                 const float* zunits, double span_cost, double unit_cost, double zdev, double budget, int target,
                 int* segs, int cap, int* parts, double* budget_out) {
  std::vector<const int32_t*> rows;
  const PlanInput in = make_input(B, Hkv, d, esz, m_max, ns, max_span_rows, max_parts, m, na, count, rank, zprob,
                                  zunits, span_cost, unit_cost, zdev, rows);
  PlanOut po;
  if (target <= 0) {
    if (!segs) return plan_cut(in, budget, nullptr);
    plan_cut(in, budget, &po);
  } else {
    plan_shares(in, target, &po);
  }
  return emit(po, segs, cap, parts, B * Hkv, budget_out);
}

double harness_expected_bytes(int B, int Hkv, int d, int esz, int m_max, const int* m, const int* na,
                              const int* count, const float* zunits) {
  std::vector<const int32_t*> rows;
  const PlanInput in = make_input(B, Hkv, d, esz, m_max, 1, 1, 1, m, na, count, nullptr, nullptr, zunits, 2.0, 0.0,
                                  0.0, rows);
  return plan_expected_bytes(in);
}
}
