// Joint placement of streams' virtual ranks onto GPUs (host only).
//
// A stream's stages are packed into virtual ranks and mapped onto physical
// GPUs, one memory position each; a GPU batches the tasks of one block across
// chunks, steps and streams; a new stream is placed by Best-Fit and Limited
// Discrepancy Search on the remaining capacity, admitted only whole and only
// if it meets its SLO alone, and running streams never move (AREX feed
// article on the PhysisServe report, section "三层设计", layer 3; 163.com
// release, bullets "时分复用" and "虚拟 rank 的动态放置", Fig. 3 and Fig. 4).
//
// State per GPU: the virtual ranks it holds and, per block, the task count
// they add up to.  The cycle of a GPU is recomputed from the block counts
// (blocks in ascending order, so the sum has one fixed rounding).  The search
// places a rank by adding its counts to the GPU and undoes it on backtrack.
#include <algorithm>
#include <map>
#include <new>
#include <utility>
#include <vector>

#include "ps_sched.h"

namespace ps {
ps_status set_error(ps_status st, const char* msg);
}

namespace {

struct Rank {
  std::vector<std::pair<int, int>> blocks;   // (block, tasks), ascending block
};

struct Gpu {
  std::vector<std::pair<int64_t, int>> held;   // (stream, rank)
  std::vector<int> tasks;                      // per block
};

}  // namespace

struct ps_sched {
  ps_sched_desc d;
  std::vector<Gpu> gpus;
  std::vector<Rank> ranks;                     // the split of one stream (same model for all)
  std::map<int64_t, std::vector<int>> streams; // stream -> GPU of each rank

  double f(int n) const { return n == 0 ? 0.0 : d.batch_fixed_ms + d.batch_task_ms * n; }

  double cycle(const Gpu& g) const {
    double c = 0.0;
    for (int b = 0; b < d.n_blocks; ++b) c += f(g.tasks[b]);
    return c;
  }
  // cycle of GPU g with rank r added (g's counts unchanged)
  double cycle_with(const Gpu& g, const Rank& r) const {
    double c = 0.0;
    size_t k = 0;
    for (int b = 0; b < d.n_blocks; ++b) {
      int n = g.tasks[b];
      if (k < r.blocks.size() && r.blocks[k].first == b) n += r.blocks[k++].second;
      c += f(n);
    }
    return c;
  }
  void add(Gpu& g, const Rank& r, int sign) {
    for (auto& bt : r.blocks) g.tasks[bt.first] += sign * bt.second;
  }

  // contiguous stage groups that each meet the SLO alone: the fewest, or
  // exactly d.ranks_per_stream of them
  void split() {
    const int B = d.n_blocks, N = d.n_blocks * d.n_steps;
    Gpu empty;
    empty.tasks.assign(B, 0);
    const int r_lo = d.ranks_per_stream ? d.ranks_per_stream : 1;
    const int r_hi = d.ranks_per_stream ? d.ranks_per_stream : N;
    for (int R = r_lo; R <= r_hi && R <= N; ++R) {
      std::vector<Rank> groups(R);
      bool ok = true;
      for (int r = 0; r < R && ok; ++r) {
        std::vector<int> cnt(B, 0);
        // stages in block-major order: stage p is block p / n_steps
        for (int p = (int)((int64_t)r * N / R); p < (int)((int64_t)(r + 1) * N / R); ++p) ++cnt[p / d.n_steps];
        for (int b = 0; b < B; ++b)
          if (cnt[b]) groups[r].blocks.emplace_back(b, cnt[b]);
        ok = cycle_with(empty, groups[r]) <= d.slo_ms;
      }
      if (ok) {
        ranks = std::move(groups);
        return;
      }
    }
    ranks.clear();
  }

  // feasible GPUs for rank r, Best-Fit order: least slack left, then lower index
  std::vector<int> candidates(const Rank& r) const {
    std::vector<std::pair<double, int>> c;
    for (int g = 0; g < d.n_gpus; ++g) {
      if ((int)gpus[g].held.size() + 1 > d.positions) continue;
      const double cy = cycle_with(gpus[g], r);
      if (cy <= d.slo_ms) c.emplace_back(d.slo_ms - cy, g);
    }
    std::sort(c.begin(), c.end());
    std::vector<int> out;
    for (auto& e : c) out.push_back(e.second);
    return out;
  }

  // depth-first placement of ranks r.. with at most `left` discrepancies
  // (recursion depth = rank count <= n_blocks * n_steps <= 4096)
  bool dfs(int r, int left, std::vector<int>& chosen) {
    if (r == (int)ranks.size()) return true;
    const std::vector<int> cand = candidates(ranks[r]);
    for (size_t i = 0; i < cand.size(); ++i) {
      const int cost = i == 0 ? 0 : 1;
      if (cost > left) break;
      Gpu& g = gpus[cand[i]];
      add(g, ranks[r], +1);
      g.held.emplace_back(-1, r);   // placeholder: counts toward the positions
      chosen.push_back(cand[i]);
      if (dfs(r + 1, left - cost, chosen)) return true;
      chosen.pop_back();
      g.held.pop_back();
      add(g, ranks[r], -1);
    }
    return false;
  }
};

extern "C" ps_status ps_sched_create(const ps_sched_desc* desc, ps_sched** out) {
  if (!desc || !out) return ps::set_error(PS_ERR_INVALID_ARG, "ps_sched_create: null argument");
  const ps_sched_desc& d = *desc;
  if (d.n_gpus < 1 || d.positions < 1 || d.n_blocks < 1 || d.n_steps < 1 || d.max_discrepancy < 0 ||
      (int64_t)d.n_blocks * d.n_steps > (1 << 12) || !(d.slo_ms > 0) || !(d.batch_fixed_ms >= 0) ||
      !(d.batch_task_ms > 0) || d.ranks_per_stream < 0)
    return ps::set_error(PS_ERR_INVALID_ARG, "ps_sched_create: field out of range");
  ps_sched* s = new (std::nothrow) ps_sched;
  if (!s) return ps::set_error(PS_ERR_OUT_OF_MEMORY, "ps_sched_create: out of host memory");
  s->d = d;
  s->gpus.resize(d.n_gpus);
  for (auto& g : s->gpus) g.tasks.assign(d.n_blocks, 0);
  s->split();
  *out = s;
  return PS_OK;
}

extern "C" ps_status ps_sched_destroy(ps_sched* s) {
  delete s;
  return PS_OK;
}

extern "C" ps_status ps_sched_split(const ps_sched* s, int32_t* n_ranks) {
  if (!s || !n_ranks) return ps::set_error(PS_ERR_INVALID_ARG, "ps_sched_split: null argument");
  *n_ranks = (int32_t)s->ranks.size();
  return PS_OK;
}

extern "C" ps_status ps_sched_admit(ps_sched* s, int64_t stream, int32_t* gpu_of_rank, int32_t capacity,
                                    int32_t* n_ranks) {
  if (!s || !gpu_of_rank || !n_ranks) return ps::set_error(PS_ERR_INVALID_ARG, "ps_sched_admit: null argument");
  if (s->streams.count(stream)) return ps::set_error(PS_ERR_INVALID_ARG, "ps_sched_admit: stream already admitted");
  const int R = (int)s->ranks.size();
  if (capacity < R) return ps::set_error(PS_ERR_INVALID_ARG, "ps_sched_admit: capacity below the rank count");
  *n_ranks = 0;
  if (R == 0) return PS_OK;   // cannot meet the SLO alone
  std::vector<int> chosen;
  for (int lim = 0; lim <= s->d.max_discrepancy; ++lim) {
    chosen.clear();
    if (s->dfs(0, lim, chosen)) {
      // the search left the ranks applied: name their stream
      for (int r = 0; r < R; ++r) {
        auto& held = s->gpus[chosen[r]].held;
        for (auto& e : held)
          if (e.first == -1 && e.second == r) {
            e.first = stream;
            break;
          }
        gpu_of_rank[r] = chosen[r];
      }
      s->streams[stream] = chosen;
      *n_ranks = R;
      return PS_OK;
    }
  }
  return PS_OK;
}

extern "C" ps_status ps_sched_release(ps_sched* s, int64_t stream, int32_t* n_ranks) {
  if (!s || !n_ranks) return ps::set_error(PS_ERR_INVALID_ARG, "ps_sched_release: null argument");
  *n_ranks = 0;
  auto it = s->streams.find(stream);
  if (it == s->streams.end()) return PS_OK;
  const std::vector<int>& where = it->second;
  for (int r = 0; r < (int)where.size(); ++r) {
    Gpu& g = s->gpus[where[r]];
    s->add(g, s->ranks[r], -1);
    for (size_t k = 0; k < g.held.size(); ++k)
      if (g.held[k].first == stream && g.held[k].second == r) {
        g.held.erase(g.held.begin() + k);
        break;
      }
  }
  *n_ranks = (int32_t)where.size();
  s->streams.erase(it);
  return PS_OK;
}

extern "C" ps_status ps_sched_gpu(const ps_sched* s, int32_t gpu, int32_t* n_ranks, double* cycle_ms) {
  if (!s || !n_ranks || !cycle_ms) return ps::set_error(PS_ERR_INVALID_ARG, "ps_sched_gpu: null argument");
  if (gpu < 0 || gpu >= s->d.n_gpus) return ps::set_error(PS_ERR_INVALID_ARG, "ps_sched_gpu: gpu out of range");
  *n_ranks = (int32_t)s->gpus[gpu].held.size();
  *cycle_ms = s->cycle(s->gpus[gpu]);
  return PS_OK;
}
