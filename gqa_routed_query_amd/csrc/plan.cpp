// Host-side planning of causal prefill grids (declarations and the model in
// plan.h).
#include "plan.h"

#include <algorithm>
#include <functional>
#include <queue>

namespace gqa {
namespace {

int div_up_i(int n, int unit) { return (n + unit - 1) / unit; }

// End of the modelled dispatch: the slots of `order`, each with per_main jobs
// of cost_main[slot] and per_sh of cost_sh[slot], go in order to the CU that
// frees first.
double simulate_dispatch(const std::vector<int>& order, const std::vector<double>& cost_main,
                         const std::vector<double>& cost_sh, int per_main, int per_sh, int n_cu) {
  std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
  for (int i = 0; i < n_cu; ++i) free_at.push(0.0);
  double end = 0.0;
  for (int slot : order)
    for (int j = 0; j < per_main + per_sh; ++j) {
      const double t = free_at.top() + (j < per_main ? cost_main[slot] : cost_sh[slot]);
      free_at.pop();
      free_at.push(t);
      end = std::max(end, t);
    }
  return end;
}

}  // namespace

BandKeys band_keys(int i, int rows, int R, int T, int kBN) {
  const int n_rows = T * R, row0 = i * rows;
  if (row0 >= n_rows) return {0, 0};
  const int t_first = row0 / R, t_last = (std::min(row0 + rows, n_rows) - 1) / R;
  const int n_tiles = div_up_i(t_last + 1, kBN);
  return {n_tiles, std::min(n_tiles / 2, t_first / kBN)};
}

int split_cap(int n_bands, int rows, int R, int T, int kBN, int BG, int n_cu) {
  if ((long long)n_bands * BG >= 2ll * n_cu || n_bands >= kMaxOrder) return 0;
  int eligible = 0;
  for (int i = n_bands / 2; i < n_bands; ++i) {
    const BandKeys k = band_keys(i, rows, R, T, kBN);
    if (k.split >= 1 && k.n_tiles - k.split >= 1) ++eligible;
  }
  // The second part of a split tile waits for the first: with fewer such
  // blocks than CUs, some CU always stays free to run the first parts.
  return std::max(0, std::min({eligible, kMaxOrder - n_bands, (n_cu - 1) / std::max(BG, 1)}));
}

std::vector<Slot> plan_order(const OrderShape& s) {
  const double fixed = 128.0 / s.kBN;  // ≈ 4 tiles of 32 keys
  std::vector<Slot> slots;
  for (int i = 0; i < s.n_bands; ++i) slots.push_back(Slot{(uint16_t)i, 0, 0, 0});
  auto slot_cost = [&](const Slot& sl, int R) {
    const BandKeys k = band_keys(sl.tile, s.rows, R, s.T, s.kBN);
    if (k.n_tiles == 0) return 0.0;
    const int n = sl.part == 0 ? k.n_tiles : sl.part == 1 ? sl.split : k.n_tiles - sl.split;
    return (double)n + fixed;
  };
  // With whole problems per XCD slice (blocks go to XCDs round-robin), one
  // eighth of the CUs and of each band is an exact model.
  int per_main = s.BG_main, per_sh = s.B_sh, n_cu = s.n_cu;
  if (per_main % 8 == 0 && per_sh % 8 == 0 && n_cu % 8 == 0) {
    per_main /= 8;
    per_sh /= 8;
    n_cu /= 8;
  }
  std::vector<double> cost_main, cost_sh;
  auto costs = [&]() {
    cost_main.assign(slots.size(), 0.0);
    cost_sh.assign(slots.size(), 0.0);
    for (size_t i = 0; i < slots.size(); ++i) {
      cost_main[i] = slot_cost(slots[i], s.R);
      cost_sh[i] = slot_cost(slots[i], 1);
    }
  };
  auto heaviest_first = [&]() {
    std::vector<int> order(slots.size());
    for (size_t i = 0; i < order.size(); ++i) order[i] = (int)i;
    std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return cost_main[x] > cost_main[y]; });
    return order;
  };
  // Splits, heaviest row tile first, kept while the end shortens.
  if (s.max_split > 0 && s.B_sh == 0) {
    std::vector<int> cand;
    for (int i = s.n_bands / 2; i < s.n_bands; ++i) {
      const BandKeys k = band_keys(i, s.rows, s.R, s.T, s.kBN);
      if (k.split >= 1 && k.n_tiles - k.split >= 1) cand.push_back(i);
    }
    std::stable_sort(cand.begin(), cand.end(), [&](int x, int y) {
      return band_keys(x, s.rows, s.R, s.T, s.kBN).n_tiles > band_keys(y, s.rows, s.R, s.T, s.kBN).n_tiles;
    });
    costs();
    double best = simulate_dispatch(heaviest_first(), cost_main, cost_sh, per_main, per_sh, n_cu);
    int n_split = 0;
    for (int i : cand) {
      if (n_split == s.max_split) break;
      const uint16_t sp = (uint16_t)band_keys(i, s.rows, s.R, s.T, s.kBN).split;
      std::vector<Slot> keep = slots;
      for (auto& sl : slots)
        if (sl.tile == i) sl = Slot{(uint16_t)i, sp, 1, (uint8_t)n_split};
      slots.push_back(Slot{(uint16_t)i, sp, 2, (uint8_t)n_split});
      costs();
      const double m = simulate_dispatch(heaviest_first(), cost_main, cost_sh, per_main, per_sh, n_cu);
      if (m < best - 1e-9) {
        best = m;
        ++n_split;
      } else {
        slots = keep;
      }
    }
  }
  costs();
  std::vector<int> order = heaviest_first();
  double best = simulate_dispatch(order, cost_main, cost_sh, per_main, per_sh, n_cu);
  for (int pass = 0; pass < 4; ++pass) {
    bool improved = false;
    for (size_t i = 0; i < order.size(); ++i)
      for (size_t j = i + 1; j < order.size(); ++j) {
        std::swap(order[i], order[j]);
        const double m = simulate_dispatch(order, cost_main, cost_sh, per_main, per_sh, n_cu);
        if (m < best - 1e-9) {
          best = m;
          improved = true;
        } else {
          std::swap(order[i], order[j]);
        }
      }
    if (!improved) break;
  }
  std::vector<Slot> out;
  for (int i : order) out.push_back(slots[i]);
  return out;
}


}  // namespace gqa
