// Schedule planner (host only): a model of the persistent kernel's task
// streams that predicts, for one routing, what each schedule order costs.
//
// The X-Stage paper proposes this in section 6.3 ("Adaptive Burst Shaping
// and Scope"): a runtime should weigh an order's predicted stall against its
// loss of weight locality, for the current routing and working set, and pick
// the original (Expert-Wave) or the interleaved order. Section 4.2 bounds the
// lead D from below by the knee of Eq. 16 (a smaller lead lets Linear-2
// tiles catch up with Linear-1 and wait) and notes that a lead far above it
// grows the concurrent expert-weight working set.
//
// The model runs G instances over exactly the streams of sched.hpp (the
// kernel's own code, built for the host here). Task costs are in units of
// one 128-wide K block of the mainloop: H/128 + 2 for Linear-1 and I/128 + 2
// for Linear-2 (2 for the epilogue). A Linear-2 task of scheduler row p
// starts once every Linear-1 task of p has ended; an instance whose next
// task must wait holds it (a persistent workgroup spins in place). An event
// loop in time order gives the makespan, and the intervals during which
// running tasks read each expert weight matrix give the working set.
//
// Locality: the tasks' reads, in the order the model starts them (time, then
// instance), go through an LRU cache of the Infinity Cache's size at the
// granularity of what a task reads whole: its weight tile (the N-tile's rows
// of an expert's W1 or W2) and its activation block (the M-block's token rows
// for Linear-1, its h rows for Linear-2). The bytes it misses are the HBM
// reads the order predicts; the bytes read at least once are compulsory.
//
// Among configurations predicted within 2% of the fastest (the model's
// resolution) the planner keeps the original Expert-Wave order when it is
// one of them (nothing to gain from reordering), else Interleaved at the knee
// (the lead Eq. 16 shows sufficient), else the first of them; another of them
// replaces it when it is predicted to read less from HBM by more than 2% of
// the compulsory bytes (the one that reads least, the earlier on a tie).
#include <algorithm>
#include <functional>
#include <list>
#include <queue>
#include <unordered_map>
#include <utility>
#include <vector>

#include "internal.hpp"
#include "sched.hpp"

namespace moe {
namespace {

struct Model {
  int P = 0, N1 = 0, N2 = 0, G = 0, L = 0;
  std::vector<int> tile_off;       // [L+1] scheduler rows of each expert
  std::vector<int> row_expert;     // [P]
  double c1 = 0, c2 = 0;           // task costs (units)
  double w1_bytes = 0, w2_bytes = 0;
  // bytes a task reads whole: Linear-1 weight tile and token block,
  // Linear-2 weight tile and h block
  double w1_tile = 0, x_block = 0, w2_tile = 0, h_block = 0;
  double cache_bytes = 0;          // the LRU's capacity
};

// One task as the model starts it.
struct Started {
  double t;
  int g, kind, p, n;
};

// Predicted HBM bytes and compulsory bytes of the reads of the started tasks
// (see the file comment).
void locality(const Model& m, std::vector<Started>& s, double* hbm, double* unique) {
  std::stable_sort(s.begin(), s.end(), [](const Started& a, const Started& b) {
    return a.t < b.t || (a.t == b.t && a.g < b.g);
  });
  // key: 0 W1 tile (e, n), 1 token block p, 2 W2 tile (e, n), 3 h block p
  auto key = [](int type, long long a, long long b) { return (((a << 30) | b) << 2) | type; };
  std::list<std::pair<long long, double>> lru;   // front = most recent
  std::unordered_map<long long, std::list<std::pair<long long, double>>::iterator> where;
  std::unordered_map<long long, char> seen;
  double used = 0.0, miss = 0.0, uniq = 0.0;
  auto touch = [&](long long k, double bytes) {
    if (seen.emplace(k, 1).second) uniq += bytes;
    auto it = where.find(k);
    if (it != where.end()) {
      lru.splice(lru.begin(), lru, it->second);
      return;
    }
    miss += bytes;
    lru.emplace_front(k, bytes);
    where[k] = lru.begin();
    used += bytes;
    while (used > m.cache_bytes && !lru.empty()) {
      used -= lru.back().second;
      where.erase(lru.back().first);
      lru.pop_back();
    }
  };
  for (const Started& x : s) {
    const int e = m.row_expert[x.p];
    if (x.kind == 1) {
      touch(key(0, e, x.n), m.w1_tile);
      touch(key(1, x.p, 0), m.x_block);
    } else {
      touch(key(2, e, x.n), m.w2_tile);
      touch(key(3, x.p, 0), m.h_block);
    }
  }
  *hbm = miss;
  *unique = uniq;
}

struct Interval {
  double s, e;
};

// Runs the streams to completion. Returns false if the streams deadlock
// (an instance waits on a row whose Linear-1 tasks can never run), which the
// streams of a lead D >= 1 never do.
template <class Stream>
bool simulate(const Model& m, std::vector<Stream>& st, double* makespan, double* working_set,
              std::vector<Started>* started) {
  using Ev = std::pair<double, int>;   // (time the instance is free, instance)
  std::priority_queue<Ev, std::vector<Ev>, std::greater<Ev>> q;
  for (int g = 0; g < m.G; ++g) q.push({0.0, g});
  std::vector<Task> held(m.G, Task{-1, 0, 0});
  std::vector<int> done(m.P, 0);
  std::vector<double> ready(m.P, 0.0);
  std::vector<std::vector<Ev>> waiting(m.P);
  std::vector<std::vector<Interval>> use(2 * (size_t)m.L);   // [expert][W1, W2]
  double fin = 0.0;
  int finished = 0;
  while (!q.empty()) {
    const Ev ev = q.top();
    q.pop();
    const double t = ev.first;
    const int g = ev.second;
    Task k = held[g].kind >= 0 ? held[g] : st[g].next();
    held[g].kind = -1;
    if (k.kind == 0) {
      fin = std::max(fin, t);
      ++finished;
      continue;
    }
    const int e = m.row_expert[k.p];
    if (k.kind == 1) {
      const double end = t + m.c1;
      started->push_back({t, g, 1, k.p, k.n});
      use[2 * (size_t)e].push_back({t, end});
      ready[k.p] = std::max(ready[k.p], end);
      if (++done[k.p] == m.N1) {
        for (const Ev& w : waiting[k.p]) q.push({std::max(w.first, ready[k.p]), w.second});
        waiting[k.p].clear();
      }
      q.push({end, g});
    } else {
      if (done[k.p] < m.N1) {
        waiting[k.p].push_back({t, g});
        held[g] = k;
        continue;
      }
      const double s = std::max(t, ready[k.p]);
      started->push_back({s, g, 2, k.p, k.n});
      use[2 * (size_t)e + 1].push_back({s, s + m.c2});
      q.push({s + m.c2, g});
    }
  }
  if (finished != m.G) return false;
  // time-averaged weight bytes in use: the union of each matrix's intervals
  double area = 0.0;
  for (size_t i = 0; i < use.size(); ++i) {
    std::vector<Interval>& v = use[i];
    if (v.empty()) continue;
    std::sort(v.begin(), v.end(), [](const Interval& a, const Interval& b) { return a.s < b.s; });
    double len = 0.0, cs = v[0].s, ce = v[0].e;
    for (size_t j = 1; j < v.size(); ++j) {
      if (v[j].s > ce) {
        len += ce - cs;
        cs = v[j].s;
        ce = v[j].e;
      } else {
        ce = std::max(ce, v[j].e);
      }
    }
    len += ce - cs;
    area += len * (i % 2 == 0 ? m.w1_bytes : m.w2_bytes);
  }
  *makespan = fin;
  *working_set = fin > 0.0 ? area / fin : 0.0;
  return true;
}

bool estimate(const Model& m, moe_schedule_estimate* est) {
  est->makespan = 0.0;
  est->working_set = 0.0;
  est->hbm_bytes = 0.0;
  est->unique_bytes = 0.0;
  if (m.P == 0) return true;
  std::vector<Started> started;
  bool ok;
  if (est->schedule == MOE_SCHED_INTERLEAVED) {
    std::vector<InterleavedStream> st(m.G);
    for (int g = 0; g < m.G; ++g) st[g].init(g, m.G, m.P, m.N1, m.N2, est->lead_d);
    ok = simulate(m, st, &est->makespan, &est->working_set, &started);
  } else {
    std::vector<uint16_t> wave_exp(m.L + 2);
    const int nw = build_waves(m.tile_off.data(), m.L, m.N1, m.G, est->experts_per_wave, wave_exp.data());
    std::vector<ExpertWaveStream> st(m.G);
    for (int g = 0; g < m.G; ++g) st[g].init(g, m.G, m.N1, m.N2, m.tile_off.data(), wave_exp.data(), nw);
    ok = simulate(m, st, &est->makespan, &est->working_set, &started);
  }
  if (ok) locality(m, started, &est->hbm_bytes, &est->unique_bytes);
  return ok;
}

moe_schedule_estimate config(int schedule, int lead_d, int experts_per_wave) {
  moe_schedule_estimate e{};
  e.schedule = schedule;
  e.lead_d = schedule == MOE_SCHED_INTERLEAVED ? lead_d : 0;
  e.experts_per_wave = schedule == MOE_SCHED_INTERLEAVED ? 0 : experts_per_wave;
  return e;
}

}  // namespace
}  // namespace moe

extern "C" int32_t moe_predict_schedule(const moe_shape* s, const moe_plan* plan, const int32_t* counts,
                                        const moe_sched_params* prm, moe_schedule_prediction* out) {
  using namespace moe;
  if (!shape_valid(s) || !plan || !counts || !out) return MOE_ERR_INVALID_ARG;
  if (plan->block_m < 1 || plan->n1_tiles < 1 || plan->n2_tiles < 1 || plan->grid < 1 || plan->lead_d < 1 ||
      plan->max_sched_rows < 1 || plan->block_n1 < 1 || plan->block_n2 < 1)
    return MOE_ERR_INVALID_ARG;
  if (prm && (prm->schedule != MOE_SCHED_EXPERT_WAVE && prm->schedule != MOE_SCHED_INTERLEAVED))
    return MOE_ERR_INVALID_ARG;
  if (prm && (prm->lead_d < 0 || prm->experts_per_wave < 0)) return MOE_ERR_INVALID_ARG;

  Model m;
  m.L = s->num_local_experts;
  m.N1 = plan->n1_tiles;
  m.N2 = plan->n2_tiles;
  m.G = plan->grid;
  m.tile_off.assign(m.L + 1, 0);
  for (int e = 0; e < m.L; ++e) {
    if (counts[e] < 0) return MOE_ERR_INVALID_ARG;
    const long long rows = m.tile_off[e] + ((long long)counts[e] + plan->block_m - 1) / plan->block_m;
    if (rows > plan->max_sched_rows) return MOE_ERR_INVALID_ARG;
    m.tile_off[e + 1] = (int)rows;
  }
  m.P = m.tile_off[m.L];
  m.row_expert.resize(m.P);
  for (int e = 0; e < m.L; ++e)
    for (int p = m.tile_off[e]; p < m.tile_off[e + 1]; ++p) m.row_expert[p] = e;
  m.c1 = s->hidden / 128.0 + 2.0;
  m.c2 = s->inter / 128.0 + 2.0;
  const double sw = s->dtype == MOE_BF16 ? 2.0 : s->dtype == MOE_FP8_E4M3 ? 1.0 : 0.5;
  m.w1_bytes = 2.0 * s->inter * (double)s->hidden * sw;
  m.w2_bytes = (double)s->hidden * s->inter * sw;
  const double sx = s->dtype == MOE_BF16 ? 2.0 : 1.0;   // token and h elements
  m.w1_tile = (double)plan->block_n1 * s->hidden * sw;
  m.x_block = (double)plan->block_m * s->hidden * sx;
  m.w2_tile = (double)plan->block_n2 * s->inter * sw;
  m.h_block = (double)plan->block_m * s->inter * sx;
  m.cache_bytes = MOE_PLANNER_CACHE_BYTES;

  moe_schedule_prediction r{};
  r.sched_rows = m.P;
  r.lower_bound = (double)m.P * (m.N1 * m.c1 + m.N2 * m.c2) / m.G;

  const int knee = plan->lead_d;
  r.given = prm ? config(prm->schedule, prm->lead_d > 0 ? prm->lead_d : knee, prm->experts_per_wave)
                : config(MOE_SCHED_INTERLEAVED, knee, 0);
  if (!estimate(m, &r.given)) return MOE_ERR_INVALID_ARG;

  // candidates in order of preference among equals: the original order with
  // its automatic waves, Interleaved at the knee, then the rest
  int n = 0;
  r.candidates[n++] = config(MOE_SCHED_EXPERT_WAVE, 0, 0);
  r.candidates[n++] = config(MOE_SCHED_INTERLEAVED, knee, 0);
  if (m.L > 1) r.candidates[n++] = config(MOE_SCHED_EXPERT_WAVE, 0, m.L);
  // a lead of P or more behaves as P (Linear-2 waits until every Linear-1
  // tile is out), so candidate leads are capped at P
  const long long cap = std::max(1, m.P);
  const int leads[4] = {(int)std::min<long long>(std::max(1, knee / 2), cap),
                        (int)std::min<long long>(2ll * knee, cap), (int)std::min<long long>(4ll * knee, cap),
                        (int)cap};
  for (int i = 0; i < 4; ++i) {
    bool dup = false;
    for (int j = 0; j < n; ++j)
      dup |= r.candidates[j].schedule == MOE_SCHED_INTERLEAVED && r.candidates[j].lead_d == leads[i];
    if (!dup) r.candidates[n++] = config(MOE_SCHED_INTERLEAVED, leads[i], 0);
  }
  r.num_candidates = n;
  double best = 0.0;
  for (int i = 0; i < n; ++i) {
    if (!estimate(m, &r.candidates[i])) return MOE_ERR_INVALID_ARG;
    if (i == 0 || r.candidates[i].makespan < best) best = r.candidates[i].makespan;
  }
  // within 2% of the fastest: the first of the two preferred candidates,
  // else the first of them; replaced by the one that reads least from HBM
  // when that saves more than 2% of the compulsory bytes
  int pick = -1;
  for (int i = 0; i < n && pick < 0; ++i)
    if (r.candidates[i].makespan <= best * 1.02) pick = i;
  int lean = pick;
  for (int j = 0; j < n; ++j)
    if (r.candidates[j].makespan <= best * 1.02 && r.candidates[j].hbm_bytes < r.candidates[lean].hbm_bytes)
      lean = j;
  if (r.candidates[pick].hbm_bytes - r.candidates[lean].hbm_bytes > 0.02 * r.candidates[pick].unique_bytes)
    pick = lean;
  r.recommended = r.candidates[pick];
  *out = r;
  return MOE_OK;
}
