// Automatic stage partitioning ("Efficient Training on Multiple Consumer GPUs
// with RoundPipe", section 4.4). Host code; no device work.
//
// Model (section 4.4.1): the units are the L decoder layers plus the LM head,
// which always belongs to the fused first backward stage B_1. The forward
// stages F_1 .. F_Sf cover layers [0, L - b1) front to back, B_1 the last b1
// layers (its forward doubles as the recomputation, so it costs h plus their
// backward times), and the backward stages B_2 .. B_Sb cover [0, L - b1) back
// to front at their backward (recompute included) times. Memory adds up per
// stage and is capped. The objective is (M S + N (N - 1)) t_max with S the
// stage count and t_max the slowest stage (section 3.3).
//
// Algorithm (section 4.4.2): t_max can only be a contiguous sum of forward
// times, of backward times, or the LM head plus a suffix of backward times
// (the fused stage): O(L^2) candidates. For each, B_1 takes as many layers as
// fit, then the forward layers and the backward layers are each packed into
// the fewest contiguous stages by a greedy scan, O(L): O(L^3) in total. The
// best objective wins; among equal objectives the smallest candidate, taken
// in increasing order, is kept. A stage fits a candidate when its time is at
// most t (1 + 1e-12): a group summed in another order than the candidate can
// exceed it by a few ulps (the relative error of a sum of L terms is below
// L 2^-53), and exactly equal times must count as fitting.
#include <algorithm>
#include <vector>

#include "ops.h"

namespace rp {
namespace {

// fewest contiguous groups of t[order[0..n)] with each group's time <= tmax
// and memory <= cap; false when one item alone breaks a limit
bool pack(const double* t, const double* m, const std::vector<int>& order, double tmax, double cap,
          std::vector<int>& sizes) {
  sizes.clear();
  double ct = 0.0, cm = 0.0;
  int cn = 0;
  for (int l : order) {
    if (t[l] > tmax || m[l] > cap) return false;
    if (cn > 0 && (ct + t[l] > tmax || cm + m[l] > cap)) {
      sizes.push_back(cn);
      ct = cm = 0.0;
      cn = 0;
    }
    ct += t[l];
    cm += m[l];
    ++cn;
  }
  if (cn > 0) sizes.push_back(cn);
  return true;
}

// largest stage time of a partition, each stage summed in layer order
double slowest(const double* f, const double* b, double h, int L, const std::vector<int>& fwd, int b1,
               const std::vector<int>& bwd) {
  double worst = 0.0;
  int lo = 0;
  for (int n : fwd) {
    double s = 0.0;
    for (int l = lo; l < lo + n; ++l) s += f[l];
    worst = std::max(worst, s);
    lo += n;
  }
  double s1 = 0.0;
  for (int l = L - b1; l < L; ++l) s1 += b[l];
  worst = std::max(worst, h + s1);
  int hi = L - b1;
  for (int n : bwd) {
    double s = 0.0;
    for (int l = hi - n; l < hi; ++l) s += b[l];
    worst = std::max(worst, s);
    hi -= n;
  }
  return worst;
}

}  // namespace
}  // namespace rp

using namespace rp;

extern "C" rp_status rp_partition(int L, const double* f, const double* b, double h, const double* mf,
                                  const double* mb, double mh, double mem_cap, int n_micro, int n_gpus,
                                  int* fwd_sizes, int* n_fwd, int* b1_out, int* bwd_sizes, int* n_bwd,
                                  double* objective) {
  RP_CHECK(L >= 1 && f && b && mf && mb, RP_ERR_INVALID, "partition: need L >= 1 and per-layer arrays");
  RP_CHECK(n_micro >= 1 && n_gpus >= 1, RP_ERR_INVALID, "partition: n_micro and n_gpus must be >= 1");
  RP_CHECK(fwd_sizes && n_fwd && b1_out && bwd_sizes && n_bwd && objective, RP_ERR_INVALID,
           "partition: null output");
  for (int l = 0; l < L; ++l)
    RP_CHECK(f[l] >= 0.0 && b[l] >= 0.0 && mf[l] >= 0.0 && mb[l] >= 0.0, RP_ERR_INVALID,
             "partition: negative time or memory at layer %d", l);
  RP_CHECK(h >= 0.0 && mh >= 0.0, RP_ERR_INVALID, "partition: negative LM-head time or memory");

  std::vector<double> cand;
  cand.reserve((size_t)L * (L + 1) + L);
  for (int i = 0; i < L; ++i) {
    double sf = 0.0, sb = 0.0;
    for (int j = i; j < L; ++j) {
      sf += f[j];
      sb += b[j];
      cand.push_back(sf);
      cand.push_back(sb);
    }
  }
  double suffix = 0.0;
  for (int j = L - 1; j >= 0; --j) {
    suffix += b[j];
    cand.push_back(h + suffix);
  }
  std::sort(cand.begin(), cand.end());
  cand.erase(std::unique(cand.begin(), cand.end()), cand.end());

  const double bubble = (double)n_gpus * (n_gpus - 1);
  bool found = false;
  double best = 0.0;
  std::vector<int> best_fwd, best_bwd, fwd, bwd, order;
  int best_b1 = 0;
  for (double t : cand) {
    if (mh > mem_cap) break;  // the LM head alone exceeds the memory cap
    const double lim = t * (1.0 + 1e-12);
    if (h > lim) continue;    // the fused stage needs t >= h
    // B_1 takes layers from the top while both limits hold
    int b1 = 0;
    double tt = h, mm = mh;
    while (b1 < L) {
      const int l = L - 1 - b1;
      if (tt + b[l] > lim || mm + mb[l] > mem_cap) break;
      tt += b[l];
      mm += mb[l];
      ++b1;
    }
    if (b1 == 0) continue;
    const int rest = L - b1;
    order.resize(rest);
    for (int l = 0; l < rest; ++l) order[l] = l;
    if (!pack(f, mf, order, lim, mem_cap, fwd)) continue;
    for (int l = 0; l < rest; ++l) order[l] = rest - 1 - l;
    if (!pack(b, mb, order, lim, mem_cap, bwd)) continue;
    const double S = (double)fwd.size() + 1.0 + (double)bwd.size();
    const double val = ((double)n_micro * S + bubble) * slowest(f, b, h, L, fwd, b1, bwd);
    if (!found || val < best) {
      found = true;
      best = val;
      best_fwd = fwd;
      best_bwd = bwd;
      best_b1 = b1;
    }
  }
  if (mh > mem_cap) {
    set_error("partition: the LM head alone exceeds the memory cap");
    return RP_ERR_UNSUPPORTED;
  }
  if (!found) {
    set_error("partition: no partition fits the memory cap");
    return RP_ERR_UNSUPPORTED;
  }
  *n_fwd = (int)best_fwd.size();
  std::copy(best_fwd.begin(), best_fwd.end(), fwd_sizes);
  *b1_out = best_b1;
  *n_bwd = (int)best_bwd.size();
  std::copy(best_bwd.begin(), best_bwd.end(), bwd_sizes);
  *objective = best;
  return RP_OK;
}
