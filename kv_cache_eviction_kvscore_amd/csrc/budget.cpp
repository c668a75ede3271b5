// Exact integer layer budgets (host only).
//
// RippleKV page, Eq. 5 (the budgets sum to B) and Eq. 12 (B/|A| * w_l, then rounded);
// PyramidKV page, "Layer-Adaptive Dynamic Budget Allocation" (lo + (C_max - lo) * f_l).
// Both maps are x_l = clip(base + lam * w_l, lo, hi) with the lam that makes the x_l sum
// to the total (base = 0 for the RippleKV multipliers, base = lo for the pyramid curve),
// then largest-remainder rounding: every layer takes floor(x_l) and the layers with the
// largest fractional parts take one more each, ties to the lower layer.
//
// The weights are fp64 numbers (or, for the pyramid curve with an integer exponent, the
// integers (L-1-l)^gamma); from there everything here is exact. Every fp64 weight is an
// integer times a power of two, so after scaling by the smallest power the weights are
// integers M_l; lam is a ratio of integers, and every fractional part of a layer has the
// same denominator, so the remainders are ordered by comparing integers. Rounding the
// remainders to some precision first would decide near-ties by that precision (two
// remainders 1e-10 apart would tie at 1e-9 and go to the lower layer).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "kvs_budget.hpp"

namespace kvs {
namespace {

// Unsigned integer of any size: base-2^32 digits, least significant first, no leading zeros.
struct Big {
  std::vector<uint32_t> d;
  bool zero() const { return d.empty(); }
};

void trim(Big& a) {
  while (!a.d.empty() && a.d.back() == 0) a.d.pop_back();
}

Big from_u64(uint64_t x) {
  Big r;
  while (x) {
    r.d.push_back((uint32_t)x);
    x >>= 32;
  }
  return r;
}

Big shl(const Big& a, int bits) {
  if (a.zero()) return a;
  Big r;
  const int limbs = bits / 32, sh = bits % 32;
  r.d.assign(limbs, 0u);
  uint32_t carry = 0;
  for (uint32_t x : a.d) {
    r.d.push_back(sh ? (x << sh) | carry : x);
    carry = sh ? x >> (32 - sh) : 0;
  }
  if (carry) r.d.push_back(carry);
  trim(r);
  return r;
}

Big add(const Big& a, const Big& b) {
  Big r;
  const size_t n = std::max(a.d.size(), b.d.size());
  r.d.resize(n + 1);
  uint64_t c = 0;
  for (size_t i = 0; i < n; ++i) {
    c += (i < a.d.size() ? a.d[i] : 0u);
    c += (i < b.d.size() ? b.d[i] : 0u);
    r.d[i] = (uint32_t)c;
    c >>= 32;
  }
  r.d[n] = (uint32_t)c;
  trim(r);
  return r;
}

// a - b for a >= b
Big sub(const Big& a, const Big& b) {
  Big r;
  r.d.resize(a.d.size());
  int64_t c = 0;
  for (size_t i = 0; i < a.d.size(); ++i) {
    c += (int64_t)a.d[i] - (i < b.d.size() ? (int64_t)b.d[i] : 0);
    r.d[i] = (uint32_t)(c & 0xffffffffLL);
    c = (c < 0) ? -1 : 0;
  }
  trim(r);
  return r;
}

Big mul_u32(const Big& a, uint32_t m) {
  Big r;
  if (m == 0 || a.zero()) return r;
  r.d.resize(a.d.size() + 1);
  uint64_t c = 0;
  for (size_t i = 0; i < a.d.size(); ++i) {
    c += (uint64_t)a.d[i] * m;
    r.d[i] = (uint32_t)c;
    c >>= 32;
  }
  r.d[a.d.size()] = (uint32_t)c;
  trim(r);
  return r;
}

// a * m for 0 <= m < 2^64
Big mul_u64(const Big& a, uint64_t m) {
  return add(mul_u32(a, (uint32_t)m), shl(mul_u32(a, (uint32_t)(m >> 32)), 32));
}

int cmp(const Big& a, const Big& b) {
  if (a.d.size() != b.d.size()) return a.d.size() < b.d.size() ? -1 : 1;
  for (size_t i = a.d.size(); i-- > 0;)
    if (a.d[i] != b.d[i]) return a.d[i] < b.d[i] ? -1 : 1;
  return 0;
}

// a ~= top * 2^e from the three leading digits (for a first guess of a quotient only)
long double lead(const Big& a, int& e) {
  const size_t n = a.d.size(), k = std::min<size_t>(n, 3);
  long double r = 0;
  for (size_t i = n; i-- > n - k;) r = r * 4294967296.0L + a.d[i];
  e = (int)(32 * (n - k));
  return r;
}

// q = floor(num / den) for a quotient known to be below 2^62, and the remainder num - q*den
void divmod_small(const Big& num, const Big& den, uint64_t& q, Big& rem) {
  int en = 0, ed = 0;
  const long double tn = lead(num, en), td = lead(den, ed);
  const long double est = (tn == 0) ? 0 : std::ldexp(tn / td, en - ed);
  uint64_t g = est <= 0 ? 0 : (uint64_t)std::min<long double>(est, 4.0e18L);
  // correct the estimate exactly: g*den <= num < (g+1)*den
  while (g > 0 && cmp(mul_u64(den, g), num) > 0) --g;
  while (cmp(mul_u64(den, g + 1), num) <= 0) ++g;
  q = g;
  rem = sub(num, mul_u64(den, g));
}

// weights as integers: w_l = M_l * 2^E with one E for all (every finite double w >= 0 is an
// integer of at most 53 bits times a power of two)
std::vector<Big> scale_to_integers(const std::vector<double>& w) {
  int E = 0;
  bool any = false;
  std::vector<uint64_t> mant(w.size(), 0);
  std::vector<int> ex(w.size(), 0);
  for (size_t l = 0; l < w.size(); ++l) {
    if (w[l] == 0.0) continue;
    int e;
    const double f = std::frexp(w[l], &e);  // w = f * 2^e, f in [0.5, 1)
    mant[l] = (uint64_t)std::ldexp(f, 53);  // exact: f has at most 53 significant bits
    ex[l] = e - 53;
    E = any ? std::min(E, ex[l]) : ex[l];
    any = true;
  }
  std::vector<Big> M(w.size());
  for (size_t l = 0; l < w.size(); ++l)
    if (mant[l]) M[l] = shl(from_u64(mant[l]), ex[l] - E);
  return M;
}

// a breakpoint lam = c / M_l (c >= 0), where layer l leaves lo (or reaches hi)
struct Brk {
  uint64_t c;
  int l;
};

bool brk_less(const std::vector<Big>& M, const Brk& a, const Brk& b) {
  return cmp(mul_u64(M[b.l], a.c), mul_u64(M[a.l], b.c)) < 0;  // a.c/M_a < b.c/M_b
}

// x_l = clip(base + lam * M_l, lo, hi) with sum x_l = total (lo <= base <= hi), rounded by
// largest remainder. Returns 0, or -1 when no lam reaches the total.
int exact_budgets(const std::vector<Big>& M, int64_t base, int64_t total, int64_t lo, int64_t hi, int32_t* out) {
  const int L = (int)M.size();
  if (L == 0 || base < 0 || base > hi || lo < 0 || lo > hi) return -1;
  // lam = 0: every layer at clip(base, lo, hi) = max(base, lo)
  const int64_t x0 = std::max(base, lo);
  if ((int64_t)L * x0 == total) {
    for (int l = 0; l < L; ++l) out[l] = (int32_t)x0;
    return 0;
  }
  if ((int64_t)L * x0 > total) return -1;
  // breakpoints: where a layer leaves lo ((lo - base)/M_l, only when base < lo, which the
  // maps here never need: base is 0 with lo >= 0, or lo itself) and reaches hi
  std::vector<Brk> bp;
  for (int l = 0; l < L; ++l) {
    if (M[l].zero()) continue;
    if (lo > base) bp.push_back({(uint64_t)(lo - base), l});
    bp.push_back({(uint64_t)(hi - base), l});
  }
  std::sort(bp.begin(), bp.end(), [&](const Brk& a, const Brk& b) { return brk_less(M, a, b); });
  // f(lam) * M_k at lam = c / M_k, compared with total * M_k
  auto reaches = [&](const Brk& p) {
    const Big& Mk = M[p.l];
    Big f;
    for (int l = 0; l < L; ++l) {
      Big x = add(mul_u64(Mk, (uint64_t)base), mul_u64(M[l], p.c));  // (base + lam M_l) M_k
      const Big lo_k = mul_u64(Mk, (uint64_t)lo), hi_k = mul_u64(Mk, (uint64_t)hi);
      if (cmp(x, lo_k) < 0) x = lo_k;
      if (cmp(x, hi_k) > 0) x = hi_k;
      f = add(f, x);
    }
    return cmp(f, mul_u64(Mk, (uint64_t)total)) >= 0;
  };
  // first breakpoint at which the sum reaches the total (the sum is nondecreasing in lam)
  size_t lo_i = 0, hi_i = bp.size();
  while (lo_i < hi_i) {
    const size_t mid = (lo_i + hi_i) / 2;
    if (reaches(bp[mid])) hi_i = mid;
    else lo_i = mid + 1;
  }
  if (lo_i == bp.size()) return -1;  // above what the map can reach
  const Brk p = bp[lo_i];
  // on the open interval (a, p) before it (a = the previous distinct breakpoint, or 0), a
  // layer is free when it left lo at or before a and reaches hi at or after p
  std::vector<int> state(L, 0);  // -1 at lo (or base for a zero weight), +1 at hi, 0 free
  Big SF;
  int64_t C = 0, nfree = 0;
  for (int l = 0; l < L; ++l) {
    if (M[l].zero()) {
      state[l] = -1;
      C += x0;
      continue;
    }
    const Brk up = {(uint64_t)(hi - base), l};
    if (brk_less(M, up, p)) {  // reached hi before p
      state[l] = 1;
      C += hi;
      continue;
    }
    if (lo > base) {
      const Brk dn = {(uint64_t)(lo - base), l};
      if (!brk_less(M, dn, p)) {  // leaves lo at or after p: still at lo on (a, p)
        state[l] = -1;
        C += lo;
        continue;
      }
    }
    SF = add(SF, M[l]);
    ++nfree;
  }
  const int64_t TF = total - C - nfree * base;  // sum of lam * M_l over the free layers
  if (SF.zero() || TF < 0) return -1;
  // x_l = base + TF * M_l / SF: floor and the remainder's numerator over SF
  std::vector<int64_t> b(L);
  std::vector<Big> rem(L);
  int64_t assigned = 0;
  for (int l = 0; l < L; ++l) {
    if (state[l] != 0) {
      b[l] = state[l] > 0 ? hi : (M[l].zero() ? x0 : lo);
    } else {
      uint64_t q;
      divmod_small(mul_u64(M[l], (uint64_t)TF), SF, q, rem[l]);
      b[l] = base + (int64_t)q;
    }
    assigned += b[l];
  }
  int64_t extra = total - assigned;
  std::vector<int> order(L);
  for (int l = 0; l < L; ++l) order[l] = l;
  std::stable_sort(order.begin(), order.end(), [&](int i, int j) { return cmp(rem[i], rem[j]) > 0; });
  for (int i = 0; i < L && extra > 0; ++i, --extra) ++b[order[i]];
  if (extra != 0) return -1;
  for (int l = 0; l < L; ++l) out[l] = (int32_t)b[l];
  return 0;
}

}  // namespace

int exact_budgets_f64(const std::vector<double>& w, int64_t base, int64_t total, int64_t lo, int64_t hi,
                      int32_t* out) {
  for (double x : w)
    if (!(x >= 0.0) || !std::isfinite(x)) return -1;
  return exact_budgets(scale_to_integers(w), base, total, lo, hi, out);
}

int exact_budgets_pow(int64_t L, uint64_t gamma, int64_t total, int64_t lo, int64_t hi, int32_t* out) {
  // f_l = ((L-1-l)/(L-1))^gamma: the common denominator goes into lam, the integers stay
  std::vector<Big> M(L);
  for (int64_t l = 0; l < L; ++l) {
    Big x = from_u64(1);
    const uint64_t b = (L == 1) ? 1 : (uint64_t)(L - 1 - l);
    for (uint64_t i = 0; i < gamma; ++i) x = mul_u64(x, b);
    M[l] = x;
  }
  return exact_budgets(M, lo, total, lo, hi, out);
}

}  // namespace kvs
