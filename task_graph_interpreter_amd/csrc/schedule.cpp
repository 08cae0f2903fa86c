// Static schedule of a lowered graph: which workgroup runs which task.
//
// The persistent kernel can pull tasks from a device-wide ticket counter (dynamic) or
// walk a per-workgroup list fixed here on the host (static).  The list is built by
// simulating list scheduling in emission order (a topological order): each non-NOP
// task goes to the workgroup that can start it earliest, given a byte-count cost
// model (every task is bandwidth-bound) and a fixed dependency hop.  With equal
// tiles this gives each workgroup exactly one tile of every matmul, so no workgroup
// runs two tiles of an op back to back while another idles.  Each list is in
// increasing task order, which keeps the topological-order deadlock argument.
#include <algorithm>
#include <cmath>
#include <queue>
#include <new>
#include <utility>

#include "internal.h"

namespace mk {

namespace {

constexpr double kBytesPerUs = 25e3;  // per-CU streaming share at ~6.4 TB/s
constexpr double kFixedUs = 2.0;      // per-task overhead (descriptor, staging, release)
constexpr double kHopUs = 3.0;        // producer release -> consumer ready

double task_cost_us(const Lowered& L, const mk_task_t& d) {
  const mk_model_cfg& c = L.cfg;
  switch (d.op_id) {
    case MK_OP_GEMV: {
      const double es = c.weight_dtype == MK_DTYPE_F32 ? 4.0 : 2.0;
      const double rows = (double)d.reserved[1] * ((d.flags & MK_FLAG_SILU_MUL) ? 2.0 : 1.0);
      const double passes = std::ceil((double)d.m / 8.0);
      return kFixedUs + passes * rows * d.k * es / kBytesPerUs;
    }
    case MK_OP_ATTENTION_PARTIAL: {
      const double es = c.kv_dtype == MK_DTYPE_F32 ? 4.0 : 2.0;
      const int b = (int)d.reserved[0], ch = (int)d.reserved[3];
      const double keys = std::max(0, std::min(d.kv_len, L.kv_len[b] - ch * d.kv_len));
      const double head_passes = std::ceil((double)d.reserved[2] / 4.0);
      return kFixedUs + head_passes * keys * d.n * 2.0 * es / kBytesPerUs;
    }
    default:
      return kFixedUs;
  }
}

}  // namespace

void build_schedule(const Lowered& L, uint32_t workers, Schedule& S) {
  const size_t n = L.tasks.size();
  std::vector<double> ready(n, 0.0);
  std::vector<std::vector<uint32_t>> lists(workers);
  using Slot = std::pair<double, uint32_t>;  // (free time, workgroup)
  std::priority_queue<Slot, std::vector<Slot>, std::greater<Slot>> freeq;
  for (uint32_t w = 0; w < workers; ++w) freeq.push({0.0, w});
  double makespan = 0.0;
  for (size_t t = 0; t < n; ++t) {
    const mk_task_t& d = L.tasks[t];
    double fin;
    if (d.op_id == MK_OP_NOP) {
      fin = ready[t];  // complete when its last parent counts on it
    } else {
      const Slot s = freeq.top();
      freeq.pop();
      fin = std::max(s.first, ready[t]) + task_cost_us(L, d);
      freeq.push({fin, s.second});
      lists[s.second].push_back((uint32_t)t);
    }
    makespan = std::max(makespan, fin);
    for (int32_t i = 0; i < d.num_dependents; ++i) {
      const uint32_t c = L.edges[d.dependents_offset + i];
      ready[c] = std::max(ready[c], fin + kHopUs);
    }
  }
  S.order.clear();
  S.offsets.assign(workers + 1, 0);
  for (uint32_t w = 0; w < workers; ++w) {
    S.offsets[w] = (uint32_t)S.order.size();
    S.order.insert(S.order.end(), lists[w].begin(), lists[w].end());
  }
  S.offsets[workers] = (uint32_t)S.order.size();
  S.est_us = makespan;
}

}  // namespace mk

namespace mk {

// Level-synchronous lists: the level of a task is one more than its parents' highest
// (tasks are in topological order, so one forward pass over the dependents lists
// settles every level); the non-NOP tasks grouped by level, ascending within a level,
// and levels holding only NOP joins dropped.  Level i is tasks[offsets[i] ..
// offsets[i + 1]).
void build_levels(const Lowered& L, Levels& out) {
  const size_t nt = L.tasks.size();
  std::vector<uint32_t> level(nt, 0);
  uint32_t max_level = 0;
  for (size_t t = 0; t < nt; ++t) {
    const mk_task_t& d = L.tasks[t];
    max_level = std::max(max_level, level[t]);
    for (int32_t i = 0; i < d.num_dependents; ++i) {
      const uint32_t c = L.edges[(size_t)d.dependents_offset + i];
      level[c] = std::max(level[c], level[t] + 1);
    }
  }
  std::vector<std::vector<uint32_t>> by_level(nt ? max_level + 1 : 0);
  for (size_t t = 0; t < nt; ++t)
    if (L.tasks[t].op_id != MK_OP_NOP) by_level[level[t]].push_back((uint32_t)t);
  out.tasks.clear();
  out.offsets.assign(1, 0);
  for (const auto& v : by_level) {
    if (v.empty()) continue;
    out.tasks.insert(out.tasks.end(), v.begin(), v.end());
    out.offsets.push_back((uint32_t)out.tasks.size());
  }
}

}  // namespace mk

extern "C" int mk_lowered_levels(mk_lowered* g, const uint32_t** tasks, const uint32_t** offsets,
                                 uint32_t* n_levels) {
  if (!g || !tasks || !offsets || !n_levels) return mk::set_error(MK_ERR_INVALID, "NULL argument");
  try {
    mk::build_levels(g->low, g->levels);
  } catch (const std::bad_alloc&) {
    return mk::set_error(MK_ERR_NOMEM, "out of host memory while grouping levels");
  }
  *tasks = g->levels.tasks.data();
  *offsets = g->levels.offsets.data();
  *n_levels = (uint32_t)(g->levels.offsets.size() - 1);
  return MK_OK;
}

extern "C" int mk_lowered_schedule(mk_lowered* g, uint32_t workers, const uint32_t** order,
                                   const uint32_t** offsets, double* est_us) {
  if (!g || !order || !offsets || workers == 0) return mk::set_error(MK_ERR_INVALID, "NULL argument or 0 workers");
  try {
    mk::build_schedule(g->low, workers, g->sched);
  } catch (const std::bad_alloc&) {
    return mk::set_error(MK_ERR_NOMEM, "out of host memory while scheduling");
  }
  *order = g->sched.order.data();
  *offsets = g->sched.offsets.data();
  if (est_us) *est_us = g->sched.est_us;
  return MK_OK;
}
