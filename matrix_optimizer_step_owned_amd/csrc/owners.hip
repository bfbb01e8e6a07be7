// Owner assignment: which rank owns which dedicated matrix (FAQ, "Why isn't
// DMuon just ZeRO-1?": one owner runs each matrix's whole step; Training
// Guide, "Verify Parameter Assignment": the assignment is reported as
// per-rank loads and an imbalance).  Host code only.
//
// Each matrix gets a cost from one of three models; matrices are taken in
// decreasing cost (ties: lower index first) and each goes to the rank with
// the smallest load so far (ties: lower rank).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <functional>
#include <queue>
#include <string>
#include <utility>
#include <vector>

#include "../../include/dmuon.h"
#include "internal.h"

namespace dmuon {
namespace {

constexpr double kPeakBf16Flops = 2516.6e12;   // dense bf16 matrix-core peak
constexpr double kPeakHbmBytes = 8.0e12;       // HBM bandwidth
constexpr int64_t kMaxOwnerDim = int64_t(1) << 24;

typedef __int128 i128;

// Flops (two per multiply-add) of the products of one NS call; symmetric
// d x d results count m(m+1)/2 entries; the Gram form when the backend is
// "gram" and n >= 2m, as the planner of the step chooses it.
i128 executed_flops(int64_t rows, int64_t cols, int ns_steps, int32_t backend) {
  const i128 m = std::min(rows, cols), n = std::max(rows, cols);
  if (ns_steps == 0) return 0;
  const i128 sym = m * (m + 1);
  if (backend == DMUON_NS_GRAM && n >= 2 * m) {
    i128 total = sym * n;                          // R = X0 X0^T
    for (int k = 0; k < ns_steps; ++k) {
      total += sym * m;                            // P_k
      if (k >= 1) total += sym * m;                // Q <- P_k Q
      if (k + 1 < ns_steps) total += 2 * sym * m;  // T = P_k A, A <- T P_k
    }
    return total + 2 * m * n * m;                  // O = Q X0
  }
  return i128(ns_steps) * (sym * n + sym * m + 2 * m * n * m);
}

// Bytes of the momentum pass (bf16 grad in, fp32 momentum in and out, the
// NS input and its transpose out) and of the update pass (bf16 param in and
// out, O in).
i128 elementwise_bytes(int64_t rows, int64_t cols) {
  const i128 e = i128(rows) * cols;
  return e * (2 + 8 + 2 + 2) + e * (2 * 2 + 2);
}

double cost_of(int64_t rows, int64_t cols, int32_t model, int ns_steps, int32_t backend) {
  const i128 m = std::min(rows, cols), n = std::max(rows, cols);
  switch (model) {
    case DMUON_COST_NUMEL:
      return static_cast<double>(i128(rows) * cols);
    case DMUON_COST_NS_NOMINAL:
      return static_cast<double>(i128(ns_steps) * (4 * m * m * n + 2 * m * m * m));
    default:
      return static_cast<double>(executed_flops(rows, cols, ns_steps, backend)) / kPeakBf16Flops +
             static_cast<double>(elementwise_bytes(rows, cols)) / kPeakHbmBytes;
  }
}

}  // namespace
}  // namespace dmuon

using namespace dmuon;

int dmuon_assign_owners(const int64_t* rows, const int64_t* cols, int32_t n, int32_t nranks,
                        int32_t cost_model, const dmuon_hparams_t* hp, int32_t* owner, double* cost,
                        double* loads, double* imbalance) {
  set_last_error("");
  if (n < 0) return set_last_error(DMUON_ERR_INVALID_ARG, "n < 0");
  if (nranks < 1) return set_last_error(DMUON_ERR_INVALID_ARG, "nranks must be >= 1");
  if (cost_model != DMUON_COST_NUMEL && cost_model != DMUON_COST_NS_NOMINAL && cost_model != DMUON_COST_ROOFLINE)
    return set_last_error(DMUON_ERR_INVALID_ARG, "cost_model must be NUMEL, NS_NOMINAL or ROOFLINE");
  if (n > 0 && (!rows || !cols || !owner)) return set_last_error(DMUON_ERR_INVALID_ARG, "rows, cols or owner is NULL");
  int ns_steps = 5;
  int32_t backend = DMUON_NS_GRAM;
  if (hp) {
    if (hp->ns_steps < 0 || hp->ns_steps > 16) return set_last_error(DMUON_ERR_INVALID_ARG, "ns_steps must be in 0..16");
    if (hp->ns_backend != DMUON_NS_GRAM && hp->ns_backend != DMUON_NS_DIRECT)
      return set_last_error(DMUON_ERR_INVALID_ARG, "ns_backend must be DMUON_NS_GRAM or DMUON_NS_DIRECT");
    ns_steps = hp->ns_steps;
    backend = hp->ns_backend;
  }
  for (int i = 0; i < n; ++i)
    if (rows[i] <= 0 || cols[i] <= 0 || rows[i] > kMaxOwnerDim || cols[i] > kMaxOwnerDim)
      return set_last_error(DMUON_ERR_INVALID_ARG, "matrix " + std::to_string(i) + ": bad shape");
  std::vector<double> c(static_cast<size_t>(n));
  for (int i = 0; i < n; ++i) c[i] = cost_of(rows[i], cols[i], cost_model, ns_steps, backend);
  std::vector<int32_t> order(static_cast<size_t>(n));
  for (int i = 0; i < n; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return c[a] > c[b]; });
  // min-heap on (load, rank): the least loaded rank, the lower one on ties
  typedef std::pair<double, int32_t> Slot;
  std::priority_queue<Slot, std::vector<Slot>, std::greater<Slot>> heap;
  std::vector<double> load(static_cast<size_t>(nranks), 0.0);
  for (int32_t r = 0; r < nranks; ++r) heap.push({0.0, r});
  for (int32_t i : order) {
    const Slot s = heap.top();
    heap.pop();
    owner[i] = s.second;
    load[s.second] += c[i];
    heap.push({load[s.second], s.second});
  }
  if (cost)
    for (int i = 0; i < n; ++i) cost[i] = c[i];
  if (loads)
    for (int32_t r = 0; r < nranks; ++r) loads[r] = load[r];
  if (imbalance) {
    double total = 0.0, mx = load[0];
    for (int32_t r = 0; r < nranks; ++r) {
      total += load[r];
      mx = std::max(mx, load[r]);
    }
    *imbalance = total == 0.0 ? 0.0 : mx / (total / nranks) - 1.0;
  }
  return DMUON_OK;
}
