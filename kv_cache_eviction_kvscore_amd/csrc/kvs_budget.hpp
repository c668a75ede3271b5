// Exact integer layer budgets (host only; see budget.cpp). Not part of the C ABI.
#pragma once

#include <stdint.h>

#include <vector>

namespace kvs {

// b_l = largest-remainder rounding of x_l = clip(base + lam * w_l, lo, hi), lam such that
// sum x_l = total, with 0 <= base <= hi and 0 <= lo <= hi; w_l finite fp64 >= 0.
// Returns 0, or -1 when the total is out of the map's reach or an argument is invalid.
int exact_budgets_f64(const std::vector<double>& w, int64_t base, int64_t total, int64_t lo, int64_t hi,
                      int32_t* out);
// The same with the integer weights w_l = (L-1-l)^gamma (w = 1 when L = 1) and base = lo.
int exact_budgets_pow(int64_t L, uint64_t gamma, int64_t total, int64_t lo, int64_t hi, int32_t* out);

}  // namespace kvs
