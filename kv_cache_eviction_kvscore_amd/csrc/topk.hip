// Per-unit selection: the first ns = min(n_sink, n - W) positions (attention sinks), the W
// most recent positions, and the k = b - W - ns competitors in [ns, n - W) with the
// largest ranking key (ties to the lower position), written ascending. The ranking key is
// the score, or its max-pool over a centred odd window truncated to the prefix [0, n - W).
//
// DropKV page, "Methodology in Plain English": rank tokens by their individual shift
// and delete the smallest (i.e. keep the largest); the most recent w tokens are always
// retained; a max-pool over neighbouring scores (after SnapKV). "Preserve Attention
// Sinks": the first tokens stay. RippleKV page, Eq. 4: the retained positions of a layer
// form its compressed cache.
//
// pool_kernel (pool > 1): grid (4096-token tile, unit); the tile and its halo are loaded
// into LDS (-inf outside the prefix) and every token takes the maximum of its window.
//
// topk_kernel: one 1024-thread workgroup per (layer, sequence, KV head) unit, longest
// sequences first. Keys are order-preserving uint32 images of the fp32 scores. The common
// case reads the scores once: a strided sample (a 4-key run per thread) locates a band
// [lo, hi] of keys around the threshold's expected rank; one read sets a bit in an LDS
// bitmask for every competitor above the band ("surely kept") and lists the band's keys
// (key and competitor index) in per-wave LDS regions; if the band held the k-th largest
// key and the regions did not overflow, that key (the threshold T) and the number of keys
// equal to it that are taken follow from an exact select over the list in LDS. Otherwise
// (and for units with more competitors than the bitmasks hold) a radix select in three
// passes of 14, 9 and 9 bits finds them, each pass counted into one shared LDS histogram
// (a wave whose counted lanes share a bin adds their number with one atomic); the digit
// is found by a two-level scan (each thread sums its run of bins, a block scan over the
// threads' totals finds the thread where the count from the top reaches k). When the
// threshold's 14-bit bin holds few enough keys, that route's second pass also lists them
// and marks every competitor above the bin, and its last pass counts over the list. The
// listed keys are then marked against T (a "surely kept" bit above it, a "tied" bit equal
// to it) and the kept positions written from the bitmasks: each thread takes a run of
// words, a block scan of their counts gives its slots, ties are taken by ascending
// position. Without the bitmasks an ordered stream compaction over the scores in rounds of
// 4096 positions does the same from ballots within a wave and LDS sums across waves.
//
// heads_*_kernel (head budgets chosen jointly over a layer's KV heads) run a select of
// their own, spread over many workgroups: four passes of 8 bits, one 256-bin histogram
// per (chunk, head) summed per layer in a fixed order (described at those kernels).
#include <cmath>

#include "kvs_internal.hpp"

namespace kvs {
namespace {

constexpr int NT = 1024;
constexpr int NWAVES = NT / 64;

__device__ inline unsigned f2key(float x) {
  const unsigned b = __float_as_uint(x == 0.f ? 0.f : x);  // +0 and -0 share a key
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Inclusive sum over the lanes of a wave, in registers (DPP, no LDS): Hillis-Steele steps of
// 1, 2, 4 and 8 lanes within each row of 16 (a lane whose source lies outside its row adds
// 0), then the last lane of row 0 is broadcast into row 1 and that of row 2 into row 3, then
// the last lane of row 1 into rows 2 and 3.
__device__ inline int wave_incl_scan(int x, int) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// h[bin] += 1 for every lane with in set. When those lanes share one bin (most of a radix
// pass's first digit falls in a single bin), one lane adds their count: 64 atomics on one
// LDS address would serialise.
__device__ inline void hist_add(unsigned* h, bool in, unsigned bin) {
  const unsigned long long m = __ballot(in);
  if (!m) return;
  const int first = __ffsll((long long)m) - 1;  // uniform
  const unsigned b0 = (unsigned)__builtin_amdgcn_readlane((int)bin, first);
  if (__ballot(in && bin == b0) == m) {
    if ((int)(threadIdx.x & 63) == first) atomicAdd(&h[b0], (unsigned)__popcll(m));
  } else if (in) {
    atomicAdd(&h[bin], 1u);
  }
}

// The same for a pass that counts every lane: a per-lane atomic unless the wave's lanes all
// fall in one bin (then one atomic with their number).
__device__ inline void hist_add_all(unsigned* h, unsigned bin) {
  const unsigned b0 = (unsigned)__builtin_amdgcn_readfirstlane((int)bin);
  if (__ballot(bin != b0) == 0) {
    const unsigned long long ex = __ballot(true);
    if ((int)(threadIdx.x & 63) == __ffsll((long long)ex) - 1) atomicAdd(&h[b0], (unsigned)__popcll(ex));
  } else {
    atomicAdd(&h[bin], 1u);
  }
}

constexpr int PT = 4096;  // tokens per pooling workgroup
constexpr int kMaxPool = 255;

__global__ __launch_bounds__(256) void pool_kernel(Dev p, const float* __restrict__ score, int pool,
                                                   float* __restrict__ pooled) {
  __shared__ float tile[PT + kMaxPool - 1];
  const int u = blockIdx.y;
  int l, s, g;
  unit_coords(p, u, l, s, g);
  const int64_t n = p.cu[s + 1] - p.cu[s];
  const int64_t cand = n - p.W;
  const int64_t j0 = (int64_t)blockIdx.x * PT;
  if (j0 >= cand) return;  // uniform
  const int h = pool >> 1;
  const int64_t base = (int64_t)(l * p.Hkv + g) * p.N + p.cu[s];
  const float* sc = score + base;
  // every load of the tile and its halo in flight before the first LDS write
  constexpr int PER = (PT + kMaxPool - 1 + 255) / 256;
  float vals[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = threadIdx.x + 256 * k;
    const int64_t j = j0 - h + i;
    vals[k] = (i < PT + 2 * h && j >= 0 && j < cand) ? sc[j] : -INFINITY;
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = threadIdx.x + 256 * k;
    if (i < PT + 2 * h) tile[i] = vals[k];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < PT; i += 256) {
    const int64_t j = j0 + i;
    if (j >= cand) break;
    float m = tile[i];
    for (int e = 1; e < pool; ++e) m = fmaxf(m, tile[i + e]);
    pooled[base + j] = m;
  }
}

constexpr int kFew = 64;  // a list select finishes in one wave once this few keys are left
struct SelectSmem {
  unsigned s_digit[2], s_above[2], s_count[2];
  unsigned few_n, few_key[kFew];
  int wsum[2][NWAVES];
  long long red[2][NWAVES];
};

// Radix digits: 14 bits first (sign, exponent and five mantissa bits of the score, so even
// scores packed into a narrow range split into bins small enough for the LDS list below),
// then 9 and 9.
constexpr int kBits0 = 14, kBits12 = 9;
struct HistSmem {
  unsigned hist[1 << kBits0];
  int tsum[NWAVES];
};

// LDS list of candidate keys and their competitor indices: the sampled band's keys (the
// one-read select), or the keys that share the threshold's top 14 bits (filled by the radix
// select's second pass), so that neither the final select nor the emission reads global
// memory again
constexpr int kCandCap = 11264;
struct CandSmem {
  unsigned key[kCandCap];
  unsigned pos[kCandCap];
  unsigned n;
};
// Once the 14-bit counts are no longer needed only the first 2^9 words of the histogram are
// counted into; the rest holds two bitmasks over the competitors (bit c: competitor c),
// "surely kept" and "tied", so the emission reads no score. Units with more competitors
// take the radix select and an emission that reads the scores again.
constexpr int kBitBase = 1 << kBits12;
constexpr int kBitWords = ((1 << kBits0) - kBitBase) / 2;  // words per bitmask
constexpr int64_t kBitCap = (int64_t)kBitWords * 32;       // competitors the bitmasks cover

// For each r < NR: the bin of h[0, nb) (in LDS) where the count from the top first reaches
// kr[r] (1 <= kr[r] <= the total), into sm.s_digit[r], with the count above it
// (s_above[r]) and its own (s_count[r]); every thread returns with them visible. With
// PER > 1, nb = PER * NT and thread t owns bins nb-1-PER*t .. nb-PER*(t+1) (descending);
// with PER = 1, thread t < nb owns bin nb-1-t. A scan over the threads' totals finds the
// owning thread, and that thread the bin.
template <int PER, int NR, class Hist>
__device__ __attribute__((always_inline)) void scan_digit(SelectSmem& sm, Hist& hs, const unsigned* h, int nb,
                                                          const int64_t (&kr)[NR]) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool owns = tid * PER < nb;
  unsigned tot = 0;
  // the run's bins in an order rotated by lane / 2, so a half-wave's reads fall in distinct
  // LDS banks
  if (owns)
#pragma unroll
    for (int e = 0; e < PER; ++e) tot += h[nb - 1 - (PER * tid + ((e + (lane >> 1)) & (PER - 1)))];
  const int incl_w = wave_incl_scan((int)tot, lane);
  if (lane == 63) hs.tsum[wave] = incl_w;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int w = 0; w < NWAVES; ++w) {
    const int t = hs.tsum[w];
    before += w < wave ? t : 0;
  }
  // counts fit 32 bits (a unit has fewer than 2^31 competitors)
  const unsigned incl = (unsigned)(before + incl_w), excl = incl - tot;
  bool mine[NR], any = false;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    mine[r] = owns && excl < (unsigned)kr[r] && (unsigned)kr[r] <= incl;
    any = any || mine[r];
  }
  if (any) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      if (!mine[r]) continue;
      unsigned above = excl;
      int e = 0;
      if constexpr (PER >= 4) {  // runs of four bins first (one 16-byte read each)
        for (; e + 4 < PER; e += 4) {
          const uint4 v = *(const uint4*)(h + nb - 4 - PER * tid - e);
          const unsigned s4 = v.x + v.y + v.z + v.w;
          if (above + s4 >= (unsigned)kr[r]) break;
          above += s4;
        }
      }
      unsigned c = h[nb - 1 - (PER * tid + e)];
      while (above + c < (unsigned)kr[r]) {  // ends at e < PER
        above += c;
        c = h[nb - 1 - (PER * tid + ++e)];
      }
      sm.s_digit[r] = (unsigned)(nb - 1 - (PER * tid + e));
      sm.s_above[r] = above;
      sm.s_count[r] = c;
    }
  }
  __syncthreads();
}
constexpr int kPer0 = (1 << kBits0) / NT;  // bins per thread in a 14-bit scan
static_assert(kPer0 * NT == (1 << kBits0) && (1 << kBits12) <= NT, "scan shapes");

// Radix select of the kr-th largest key among the keys `visit` enumerates (each thread
// calls f(key) on its share, all lanes of a wave together): T = that key, need_eq = how
// many keys equal to T are among the kr largest. Three passes (14, 9 and 9 bits) count
// into one LDS histogram; the digit is found by a two-level scan over the bins in
// descending order. With cs, the second pass also appends the keys that share the
// threshold's top 14 bits to cs when they fit, and the last pass reads that list instead
// (the counts, so T and need_eq, do not depend on the list's order).
// visit(f) calls f(key, c) for every competitor c. With sure, the second pass also sets bit c
// of sure for every key above the threshold's top 14 bits, and listed tells whether the
// list was filled (the caller then marks the listed keys against T itself).
template <class Visit>
__device__ __attribute__((always_inline)) void radix_select(SelectSmem& sm, HistSmem& hs, Visit visit, int64_t kr, unsigned& T, int64_t& need_eq,
                             CandSmem* cs, unsigned* sure, bool& listed) {
  const int tid = threadIdx.x, lane = tid & 63;
  unsigned prefix = 0, pmask = 0;
  listed = false;  // uniform: the last pass reads cs
  for (int pass = 0; pass < 3; ++pass) {
    const int bits = pass == 0 ? kBits0 : kBits12;
    const int shift = pass == 0 ? 32 - kBits0 : (pass == 1 ? kBits12 : 0);
    const int nb = 1 << bits;
    const unsigned dmask = (unsigned)nb - 1u;
    // keys with the current prefix: the last pass's count of its digit
    const bool collect = cs && pass == 1 && sm.s_count[0] <= (unsigned)kCandCap;
    const bool mark = collect && sure;
    for (int i = tid; i < nb; i += NT) hs.hist[i] = 0;
    if (mark)  // both bitmasks
      for (int i = tid; i < 2 * kBitWords; i += NT) hs.hist[kBitBase + i] = 0;
    if (collect && tid == 0) cs->n = 0;
    __syncthreads();
    auto count = [&](unsigned key, int) { hist_add(hs.hist, (key & pmask) == prefix, (key >> shift) & dmask); };
    if (pass == 0) {
      visit([&](unsigned key, int) { hist_add_all(hs.hist, key >> shift); });
    } else if (listed) {
      for (int i = tid; i < (int)cs->n; i += NT) count(cs->key[i], 0);
    } else if (collect) {
      visit([&](unsigned key, int c) {
        const bool in = (key & pmask) == prefix;
        hist_add(hs.hist, in, (key >> shift) & dmask);
        if (mark && (key & pmask) > prefix) atomicOr(&sure[c >> 5], 1u << (c & 31));
        // one slot reservation per wave, then each lane writes at its rank among the wave's
        const unsigned long long m = __ballot(in);
        if (m) {
          unsigned base = 0;
          if (lane == __ffsll((long long)m) - 1) base = atomicAdd(&cs->n, (unsigned)__popcll(m));
          base = __shfl(base, __ffsll((long long)m) - 1, 64);
          if (in) {
            const unsigned slot = base + __popcll(m & ((1ull << lane) - 1));
            cs->key[slot] = key;
            cs->pos[slot] = (unsigned)c;
          }
        }
      });
    } else {
      visit(count);
    }
    __syncthreads();
    listed = listed || collect;
    const int64_t k1[1] = {kr};
    if (pass == 0) scan_digit<kPer0, 1>(sm, hs, hs.hist, nb, k1);
    else scan_digit<1, 1>(sm, hs, hs.hist, nb, k1);
    prefix |= sm.s_digit[0] << shift;
    pmask |= dmask << shift;
    kr -= sm.s_above[0];
  }
  T = prefix;
  need_eq = kr;
}

// Exact select over the cnt keys of a list in LDS: T = the kr-th largest (1 <= kr <= cnt),
// need_eq = how many keys equal to T are among the kr largest, given that every key shares
// the bits of prefix above bit hb. Passes of 9 bits from bit hb down count into
// hs.hist[0, 512), below kBitBase, so the bitmasks are kept. Once at most kFew keys share
// the prefix found so far, they are gathered and one wave ranks them directly: the key
// with fewer than kr keys above it and at least kr at or above it.
template <class Hist>
__device__ __attribute__((always_inline)) void list_select(SelectSmem& sm, Hist& hs, const unsigned* key, int cnt,
                                                           int64_t kr, unsigned prefix, int hb, unsigned& T,
                                                           int64_t& need_eq) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  unsigned pmask = hb >= 32 ? 0u : ~0u << hb;
  unsigned left = (unsigned)cnt;  // keys sharing the prefix
  while (hb > 0 && left > (unsigned)kFew) {
    const int bits = hb < kBits12 ? hb : kBits12;
    const int shift = hb - bits, nb = 1 << bits;
    const unsigned dmask = (unsigned)nb - 1u;
    for (int i = tid; i < nb; i += NT) hs.hist[i] = 0;
    __syncthreads();
    for (int i0 = 0; i0 < cnt; i0 += NT) {  // whole waves through hist_add
      const int i = i0 + tid;
      const unsigned x = i < cnt ? key[i] : 0u;
      hist_add(hs.hist, i < cnt && (x & pmask) == prefix, (x >> shift) & dmask);
    }
    __syncthreads();
    const int64_t k1[1] = {kr};
    scan_digit<1, 1>(sm, hs, hs.hist, nb, k1);
    prefix |= sm.s_digit[0] << shift;
    kr -= sm.s_above[0];
    left = sm.s_count[0];
    pmask |= dmask << shift;
    hb = shift;
  }
  if (hb > 0) {
    if (tid == 0) sm.few_n = 0;
    __syncthreads();
    for (int i0 = 0; i0 < cnt; i0 += NT) {
      const int i = i0 + tid;
      const unsigned x = i < cnt ? key[i] : 0u;
      const bool in = i < cnt && (x & pmask) == prefix;
      const unsigned long long msk = __ballot(in);
      if (msk) {  // one slot reservation per wave
        const int first = __ffsll((long long)msk) - 1;
        unsigned base = 0;
        if (lane == first) base = atomicAdd(&sm.few_n, (unsigned)__popcll(msk));
        base = (unsigned)__builtin_amdgcn_readlane((int)base, first);
        if (in)
          sm.few_key[base + __builtin_amdgcn_mbcnt_hi((unsigned)(msk >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((unsigned)msk, 0u))] = x;
      }
    }
    __syncthreads();
    if (wave == 0) {
      const int nf = (int)left;  // == few_n
      const unsigned x = lane < nf ? sm.few_key[lane] : 0u;
      int gt = 0, eq = 0;
      for (int t = 0; t < nf; ++t) {
        const unsigned y = sm.few_key[t];
        gt += y > x ? 1 : 0;
        eq += y == x ? 1 : 0;
      }
      if (lane < nf && gt < kr && kr <= gt + eq) {  // every lane holding the key writes the same
        sm.s_digit[1] = x;
        sm.s_above[1] = (unsigned)gt;
      }
    }
    __syncthreads();
    prefix = sm.s_digit[1];
    kr -= sm.s_above[1];
  }
  T = prefix;
  need_eq = kr;
}

// Sample-guided select of the kr-th largest competitor key in one read of the scores, into
// the list and bitmasks the emission takes. A strided sample (one 4-key run per thread)
// gives a band [lo, hi] of keys that should hold the threshold: the sample's order
// statistics a few standard deviations of a binomial count either side of the threshold's
// expected rank, widened to whole bins of the top 23 key bits. One read then marks every
// key above hi as surely kept and lists the band's keys (key and competitor index), each
// wave in a region of its own (no atomics). The band held the threshold if A < kr <= A + L
// (A keys above it, L listed, no region overflowed); the regions are then packed into one
// list and the threshold is the (kr - A)-th largest listed key, found in LDS. Returns false
// otherwise (uniform), and the caller selects from scratch: the sample steers only how much
// work is done, never the result. Units with at most kCandCap competitors list them all
// without a sample.
constexpr int kWaveCap = kCandCap / NWAVES;  // listed keys per wave region
constexpr int kPackPer = kCandCap / NT;      // list entries per thread when packing
static_assert(kWaveCap * NWAVES == kCandCap && kPackPer * NT == kCandCap, "regions tile the list");

template <class Visit>
__device__ __attribute__((always_inline)) bool band_select(SelectSmem& sm, HistSmem& hs, CandSmem& cs, Visit visit,
                                                           const float* __restrict__ c0, int64_t m, int64_t kr,
                                                           unsigned* sure, unsigned* tie, unsigned& T,
                                                           int64_t& need_eq) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  unsigned lo = 0u, hi = ~0u;
  if (m > kCandCap) {
    constexpr int MS = 4 * NT;  // sampled keys
    const int64_t j = (int64_t)tid * (m >> 2) / NT * 4;  // <= m - 4
    unsigned x[4];
    if ((((size_t)c0) & 15) == 0) {
      const float4 v = *(const float4*)(c0 + j);
      x[0] = f2key(v.x);
      x[1] = f2key(v.y);
      x[2] = f2key(v.z);
      x[3] = f2key(v.w);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = f2key(c0[j + e]);
    }
    // expected rank of the threshold in the sample, and the band's half-width in sample ranks
    const float rho = (float)kr * (float)MS / (float)m;
    const float half = 4.f * sqrtf(rho * (1.f - rho / (float)MS)) + 16.f;
    const int64_t rh = (int64_t)floorf(rho - half), rl = (int64_t)ceilf(rho + half);
    const int64_t r0 = rh < 1 ? 1 : (rh > MS ? MS : rh), r1 = rl < 1 ? 1 : (rl > MS ? MS : rl);
    // the sample's top 14 bits (one histogram for both ranks), then the next 9 for each
    constexpr int sh0 = 32 - kBits0, sh1 = sh0 - kBits12;
    for (int i = tid; i < (1 << kBits0); i += NT) hs.hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 4; ++e) hist_add_all(hs.hist, x[e] >> sh0);
    __syncthreads();
    const int64_t rr[2] = {r0, r1};
    scan_digit<kPer0, 2>(sm, hs, hs.hist, 1 << kBits0, rr);
    const unsigned d0 = sm.s_digit[0], d1 = sm.s_digit[1];  // d0 >= d1
    // the next 9 bits of the keys in bins d0 and d1, in one histogram of two halves: d0's
    // keys in the upper half, above all of d1's (when the bins differ)
    const int64_t qq[2] = {r0 - sm.s_above[0], r1 - sm.s_above[1] + (d0 != d1 ? sm.s_count[0] : 0u)};
    for (int i = tid; i < 2 << kBits12; i += NT) hs.hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const unsigned top = x[e] >> sh0;
      const unsigned dg = ((x[e] >> sh1) & ((1u << kBits12) - 1u)) | (top == d0 ? 1u << kBits12 : 0u);
      hist_add(hs.hist, top == d0 || top == d1, dg);
    }
    __syncthreads();
    scan_digit<1, 2>(sm, hs, hs.hist, 2 << kBits12, qq);
    const unsigned e0 = sm.s_digit[0] & ((1u << kBits12) - 1u), e1 = sm.s_digit[1] & ((1u << kBits12) - 1u);
    if (rh >= 1) hi = (d0 << sh0) | (e0 << sh1) | ((1u << sh1) - 1u);
    if (rl <= MS) lo = (d1 << sh0) | (e1 << sh1);
  }
  for (int i = tid; i < 2 * kBitWords; i += NT) sure[i] = 0;  // both bitmasks
  __syncthreads();
  const bool all = m <= kCandCap;  // uniform
  unsigned wn = 0;                  // keys this wave listed (uniform)
  if (all) {  // every competitor, at its own index
    visit([&](unsigned key, int c) {
      cs.key[c] = key;
      cs.pos[c] = (unsigned)c;
    });
  } else {
    unsigned* wkey = cs.key + wave * kWaveCap;
    unsigned* wpos = cs.pos + wave * kWaveCap;
    visit([&](unsigned key, int c) {
      if (key > hi) atomicOr(&sure[c >> 5], 1u << (c & 31));
      const bool in = key >= lo && key <= hi;
      const unsigned long long msk = __ballot(in);
      const unsigned slot =
          wn + __builtin_amdgcn_mbcnt_hi((unsigned)(msk >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)msk, 0u));
      if (in && slot < (unsigned)kWaveCap) {
        wkey[slot] = key;
        wpos[slot] = (unsigned)c;
      }
      wn += (unsigned)__popcll(msk);
    });
  }
  if (lane == 0) sm.wsum[1][wave] = (int)wn;
  if (all && tid == 0) cs.n = (unsigned)m;
  __syncthreads();
  if (all) {
    list_select(sm, hs, cs.key, (int)m, kr, 0u, 32, T, need_eq);
    return true;
  }
  // A = the keys above the band, from the bitmask
  unsigned a = 0;
  for (int i = tid; i < kBitWords; i += NT) a += __popc(sure[i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) a += __shfl_xor(a, o, 64);
  if (lane == 0) sm.wsum[0][wave] = (int)a;
  __syncthreads();
  int64_t A = 0;
  int L = 0, before = 0;
  bool over = false;
  for (int w = 0; w < NWAVES; ++w) {
    const int c = sm.wsum[1][w];
    A += (unsigned)sm.wsum[0][w];
    over = over || c > kWaveCap;
    if (w == tid) before = L;
    L += c;
  }
  if (tid < NWAVES) sm.red[0][tid] = before;  // where region tid goes in the packed list
  __syncthreads();
  if (over || A >= kr || kr > A + L) return false;
  // pack the regions into one list: all entries into registers, then to their places
  unsigned pk[kPackPer], pp[kPackPer];
  int pd[kPackPer];
#pragma unroll
  for (int t = 0; t < kPackPer; ++t) {
    const int i = tid + NT * t, w = i / kWaveCap, r = i - w * kWaveCap;
    pd[t] = -1;
    if (r < sm.wsum[1][w]) {
      pk[t] = cs.key[i];
      pp[t] = cs.pos[i];
      pd[t] = (int)sm.red[0][w] + r;
    }
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < kPackPer; ++t)
    if (pd[t] >= 0) {
      cs.key[pd[t]] = pk[t];
      cs.pos[pd[t]] = pp[t];
    }
  if (tid == 0) cs.n = (unsigned)L;
  __syncthreads();
  // keys in [lo, hi] share the bits above the highest bit where lo and hi differ
  const unsigned dif = lo ^ hi;
  const int hb = dif ? 32 - __clz((int)dif) : 0;
  list_select(sm, hs, cs.key, L, kr - A, hb >= 32 ? 0u : lo & (~0u << hb), hb, T, need_eq);
  return true;
}

// Ordered stream compaction of one segment (b rows at out) over positions j in [0, n), in
// rounds of 4 NT positions, 4 per thread: flags(base, sure, tie) gives each of this
// thread's positions base + 4 tid + e its flags (surely kept, or tied with the threshold);
// the first need_eq tied positions are taken. Ballots and a sum over the waves give every
// kept position its slot.
template <class Flags>
__device__ __attribute__((always_inline)) void emit_ordered(SelectSmem& sm, int32_t* __restrict__ out, int64_t b, int64_t need_eq, int64_t n,
                             Flags flags) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int64_t sure_base = 0, eq_base = 0;
  for (int64_t base = 0; base < n; base += 4 * NT) {
    bool sure[4], tie[4];
    flags(base, sure, tie);
    // this lane's exclusive prefix over the wave and the wave's totals, from one ballot per
    // element slot (the flags are bits: no shuffle chain through LDS)
    int ps = 0, pe = 0, tws = 0, twe = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const unsigned long long ms = __ballot(sure[e]), me = __ballot(tie[e]);
      ps += __builtin_amdgcn_mbcnt_hi((unsigned)(ms >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)ms, 0u));
      pe += __builtin_amdgcn_mbcnt_hi((unsigned)(me >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)me, 0u));
      tws += __popcll(ms);
      twe += __popcll(me);
    }
    if (lane == 0) {
      sm.wsum[0][wave] = tws;
      sm.wsum[1][wave] = twe;
    }
    __syncthreads();
    int ts = 0, te = 0;
    for (int w = 0; w < NWAVES; ++w) {
      if (w < wave) {
        ps += sm.wsum[0][w];
        pe += sm.wsum[1][w];
      }
      ts += sm.wsum[0][w];
      te += sm.wsum[1][w];
    }
    int64_t rs = sure_base + ps, re = eq_base + pe;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t j = base + 4 * tid + e;
      if (sure[e]) {
        const int64_t pos = rs + (re < need_eq ? re : need_eq);
        if (pos < b) out[pos] = (int32_t)j;
        ++rs;
      } else if (tie[e]) {
        if (re < need_eq && rs + re < b) out[rs + re] = (int32_t)j;
        ++re;
      }
    }
    sure_base += ts;
    eq_base += te;
    __syncthreads();  // wsum is rewritten next round
  }
}

// The same from the scores: positions j < ns or j >= cand (sinks, window) are kept; the
// selection sel 0 keeps no competitor, 1 all, 2 key > T and the first need_eq keys equal to
// T (ascending position).
__device__ __attribute__((always_inline)) void emit_segment(SelectSmem& sm, int32_t* __restrict__ out, int64_t b, int sel, unsigned T,
                             int64_t need_eq, const float* __restrict__ sc, int64_t n, int64_t cand, int64_t ns) {
  const int tid = threadIdx.x;
  // the keys of a round are loaded three rounds ahead, 16 bytes per lane when aligned (the
  // row holds n keys, so a load never leaves it)
  const bool vec = (((size_t)sc) & 15) == 0;
  auto load = [&](int64_t base, float* x) __attribute__((always_inline)) {
    const int64_t j = base + 4 * tid;
    if (sel != 2 || j >= n) return;
    if (vec && j + 4 <= n) {
      const float4 v = *(const float4*)(sc + j);
      x[0] = v.x;
      x[1] = v.y;
      x[2] = v.z;
      x[3] = v.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j + e < n) x[e] = sc[j + e];
    }
  };
  // three rounds in flight: the emit is bound by the latency of its reads
  float nx[3][4] = {};
  load(0, nx[0]);
  load(4 * NT, nx[1]);
  load(8 * NT, nx[2]);
  emit_ordered(sm, out, b, need_eq, n, [&](int64_t base, bool* sure, bool* tie) __attribute__((always_inline)) {
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = nx[0][e];
      nx[0][e] = nx[1][e];
      nx[1][e] = nx[2][e];
    }
    load(base + 12 * NT, nx[2]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t j = base + 4 * tid + e;
      sure[e] = false;
      tie[e] = false;
      if (j < n) {
        if (j >= cand || j < ns) {
          sure[e] = true;
        } else if (sel == 1) {
          sure[e] = true;
        } else if (sel == 2) {
          const unsigned key = f2key(x[e]);
          sure[e] = key > T;
          tie[e] = key == T;
        }
      }
    }
  });
}

// The same from LDS bitmasks over the competitors (bit c of sure / tie: competitor c, at
// position ns + c), for a selection that filled them: the sinks, then the selected
// competitors, then the window. Thread t takes a run of consecutive words (at most
// kWordsPer); one block scan of the runs' counts gives every thread its first slot.
constexpr int kWordsPer = (kBitWords + NT - 1) / NT;
__device__ __attribute__((always_inline)) void emit_words(SelectSmem& sm, int32_t* __restrict__ out, int64_t b64,
                                                          int64_t need_eq64, const unsigned* sure_bits,
                                                          const unsigned* tie_bits, int64_t n64, int64_t cand64,
                                                          int64_t ns64) {
  // positions fit 32 bits (kept positions are int32)
  const int b = (int)b64, neq = (int)need_eq64, n = (int)n64, cand = (int)cand64, ns = (int)ns64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m = cand - ns;
  for (int j = tid; j < ns; j += NT) out[j] = j;
  const int nw = (m + 31) >> 5;
  const int per = (nw + NT - 1) / NT;  // words per thread, at most kWordsPer
  const int wb = tid * per;
  unsigned sw[kWordsPer], tw[kWordsPer];
  int cs_ = 0, ce = 0;
#pragma unroll
  for (int e = 0; e < kWordsPer; ++e) {
    sw[e] = 0;
    tw[e] = 0;
    if (e < per && wb + e < nw) {
      sw[e] = sure_bits[wb + e];
      tw[e] = tie_bits[wb + e];
    }
    cs_ += __popc(sw[e]);
    ce += __popc(tw[e]);
  }
  const int is = wave_incl_scan(cs_, lane), ie = wave_incl_scan(ce, lane);
  if (lane == 63) {
    sm.wsum[0][wave] = is;
    sm.wsum[1][wave] = ie;
  }
  __syncthreads();
  int ps = is - cs_, pe = ie - ce, ts = 0, te = 0;
#pragma unroll
  for (int v = 0; v < NWAVES; ++v) {
    const int a = sm.wsum[0][v], e = sm.wsum[1][v];
    ps += v < wave ? a : 0;
    pe += v < wave ? e : 0;
    ts += a;
    te += e;
  }
  int rs = ns + ps, re = pe;  // slots before this thread's run
  if (__ballot(ce != 0) == 0) {
    // no tie in the wave's words: this thread's kept competitors take consecutive slots
    int o = rs + (re < neq ? re : neq);
#pragma unroll
    for (int e = 0; e < kWordsPer; ++e) {
      const int j0 = ns + ((wb + e) << 5);
      unsigned bits = sw[e];
      while (bits) {
        const int bit = __ffs(bits) - 1;
        bits &= bits - 1;
        if (o < b) out[o] = j0 + bit;
        ++o;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < kWordsPer; ++e) {
      const int j0 = ns + ((wb + e) << 5);
      unsigned bits = sw[e] | tw[e];
      while (bits) {
        const int bit = __ffs(bits) - 1;
        bits &= bits - 1;
        const bool sb = (sw[e] >> bit) & 1u;
        const int o = rs + (sb ? (re < neq ? re : neq) : re);
        if ((sb || re < neq) && o < b) out[o] = j0 + bit;
        rs += sb ? 1 : 0;
        re += sb ? 0 : 1;
      }
    }
  }
  // the window after the selected competitors
  const int kept_c = ts + (te < neq ? te : neq);
  for (int i = tid; i < n - cand; i += NT) {
    const int pos = ns + kept_c + i;
    if (pos < b) out[pos] = cand + i;
  }
}

__global__ __launch_bounds__(NT) void topk_kernel(Dev p, const float* __restrict__ score, int n_sink,
                                                 const int64_t* __restrict__ seg_off, int32_t* __restrict__ kept) {
  __shared__ SelectSmem sm;
  // longest units first: workgroup w takes the w-th unit in order of decreasing sequence
  // length (ties by sequence), then layer and head. Workgroups are dealt round-robin to the
  // dispatch queues, so every queue gets its share of each length, longest first, and the
  // short units fill in behind the long ones.
  const int per_seq = p.L * p.Hkv, rank = blockIdx.x / per_seq, within = blockIdx.x % per_seq;
  if (threadIdx.x < p.S) {
    const int me = threadIdx.x;
    const int64_t nme = p.cu[me + 1] - p.cu[me];
    int r = 0;
    for (int o = 0; o < p.S; ++o) {
      const int64_t no = p.cu[o + 1] - p.cu[o];
      r += (no > nme || (no == nme && o < me)) ? 1 : 0;
    }
    if (r == rank) sm.s_digit[0] = (unsigned)me;
  }
  __syncthreads();
  const int s = (int)sm.s_digit[0], l = within / p.Hkv, g = within % p.Hkv;
  const int u = (l * p.S + s) * p.Hkv + g;
  __syncthreads();  // s_digit is rewritten by the select
  const int64_t n = p.cu[s + 1] - p.cu[s];
  const int64_t cand = n - p.W;
  const int64_t ns = n_sink < cand ? n_sink : cand;  // pinned sinks [0, ns); competitors [ns, cand)
  const int64_t off0 = seg_off[u];
  const int64_t b = seg_off[u + 1] - off0;
  int64_t k = b - p.W - ns;
  if (k < 0) k = 0;
  if (k > cand - ns) k = cand - ns;
  const float* sc = score + (int64_t)(l * p.Hkv + g) * p.N + p.cu[s];
  const int tid = threadIdx.x;

  // 0: keep no candidate, 1: keep all candidates, 2: keep key > T and the first need_eq keys == T
  const int sel = (k == 0) ? 0 : (k == cand - ns ? 1 : 2);
  unsigned T = 0;
  int64_t need_eq = 0;
  if (sel == 2) {
    __shared__ CandSmem cs;
    __shared__ HistSmem hs;
    const float* c0 = sc + ns;
    const int64_t m = cand - ns;
    unsigned* sure = &hs.hist[kBitBase];
    unsigned* tie = sure + kBitWords;
    bool listed = false;
    // A read of the competitors, visit(f) calling f(key, c) for each. With 16-byte loads,
    // thread tid takes float4s tid + NT r, four rounds r per step, the next step's issued
    // before this one is counted (eight in flight per thread, 128 KB per workgroup); two
    // buffers with fixed roles and two steps per trip (a register rotation would make the
    // compiler wait for the next step's loads at the copy).
    // competitor indices fit 32 bits (kept positions are int32)
    constexpr int V = 4;
    const int mc = (int)m;
    const int m4 = ((((size_t)c0) & 15) == 0 && mc >= 4) ? mc >> 2 : 0;  // competitors read as float4s
    // loads past the row repeat its last float4 (no branch around a load, so the next step's
    // loads need not wait for this one's)
    auto ld = [&](float4* buf, int r0) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int fi = tid + NT * (r0 + i);
        buf[i] = *(const float4*)(c0 + 4 * (fi < m4 ? fi : m4 - 1));
      }
    };
    auto visit = [&](auto f) {
      auto run = [&](const float4* buf, int r0) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < V; ++i) {
          const int fi = tid + NT * (r0 + i);
          if (fi < m4) {
            const int j = 4 * fi;
            f(f2key(buf[i].x), j);
            f(f2key(buf[i].y), j + 1);
            f(f2key(buf[i].z), j + 2);
            f(f2key(buf[i].w), j + 3);
          }
        }
      };
      if (m4 > 0) {
        const int nr = (m4 + NT - 1) / NT;  // rounds
        float4 A[V], B[V];
        ld(A, 0);
        for (int r = 0; r < nr; r += 2 * V) {
          ld(B, r + V);
          run(A, r);
          ld(A, r + 2 * V);
          run(B, r + V);
        }
      }
      for (int j = 4 * m4 + tid; j < mc; j += NT) f(f2key(c0[j]), j);
    };
    // the band's expected width in keys, from the sample half-width at the threshold's rank
    const float q = (float)k / (float)m;
    const float band = 2.f * (4.f * sqrtf(4.f * NT * q * (1.f - q)) + 16.f) * (float)m / (4.f * NT);
    if (m <= kBitCap && (m <= kCandCap || band <= 0.85f * kCandCap)) {
      if (band_select(sm, hs, cs, visit, c0, m, k, sure, tie, T, need_eq)) listed = true;
    }
    if (!listed) radix_select(sm, hs, visit, k, T, need_eq, &cs, m <= kBitCap ? sure : nullptr, listed);
    if (listed && m <= kBitCap) {
      // the listed keys (those sharing T's top 14 bits) against T; the ones above those bits
      // were marked during the second pass
      for (int i = tid; i < (int)cs.n; i += NT) {
        const unsigned key = cs.key[i], c = cs.pos[i];
        if (key > T) atomicOr(&sure[c >> 5], 1u << (c & 31));
        else if (key == T) atomicOr(&tie[c >> 5], 1u << (c & 31));
      }
      __syncthreads();
      emit_words(sm, kept + off0, b, need_eq, sure, tie, n, cand, ns);
      return;
    }
  }
  emit_segment(sm, kept + off0, b, sel, T, need_eq, sc, n, cand, ns);
}

// Head budgets chosen jointly over the KV heads of each (sequence, layer) "group": the
// group keeps Hkv * b rows (b = the segment length seg_off gives its heads); every head
// keeps its sinks and window; the Hkv * (b - W - ns) other slots go to the largest keys over
// all heads' competitors, ties to the lower head, then the lower position. The radix select
// runs over many workgroups: each takes HCH competitors of one head and writes its own
// histogram; a per-group kernel sums them in a fixed order and picks the digit. No atomics,
// so every count is exact and the result deterministic.
constexpr int HCH = 8192;  // competitors per histogram workgroup

struct HeadsState {  // per group
  long long kr;       // rank still to place inside the current prefix
  long long need_eq;  // keys equal to T taken (after the last pass)
  unsigned prefix;    // T after the last pass
  int sel;            // 0: no competitor kept, 1: all, 2: select
  int ns;             // sinks of the group's sequence
  int band;           // sampled band: 0 none (radix passes), 1 set, 2 T found in it
  unsigned lo, hi;    // the band's keys
  unsigned list_n;    // band keys listed (may exceed the list)
  int pad;
};

__device__ inline void group_of(const Dev& p, int grp, int& l, int& s) {
  l = grp / p.S;
  s = grp % p.S;
}

// a group's initial state: its rank to place, its selection kind, its sinks
__device__ inline HeadsState heads_state0(const Dev& p, int grp, int n_sink, const int64_t* __restrict__ seg_off) {
  int l, s;
  group_of(p, grp, l, s);
  const int64_t n = p.cu[s + 1] - p.cu[s];
  const int64_t cand = n - p.W;
  const int64_t ns = n_sink < cand ? n_sink : cand;
  const int64_t M = cand - ns;
  const int64_t b = seg_off[grp * p.Hkv + 1] - seg_off[grp * p.Hkv];
  int64_t kt = (int64_t)p.Hkv * (b - p.W - ns);
  if (kt < 0) kt = 0;
  if (kt > (int64_t)p.Hkv * M) kt = (int64_t)p.Hkv * M;
  HeadsState x;
  x.kr = kt;
  x.need_eq = 0;
  x.prefix = 0;
  x.sel = (kt == 0) ? 0 : (kt == (int64_t)p.Hkv * M ? 1 : 2);
  x.ns = (int)ns;
  x.band = 0;
  x.lo = 0;
  x.hi = 0;
  x.list_n = 0;
  x.pad = 0;
  return x;
}


// The joint select in one read when a sample allows, as the per-unit select does: a
// strided sample over the group's heads (four 4-key runs per thread, the heads taking runs
// in turn) sets a band [lo, hi] around the threshold's expected rank (heads_band_kernel,
// one workgroup per group); every chunk counts its keys above the band and appends the
// band's keys to the group's list in global memory, one slot reservation per workgroup
// (heads_pass_kernel, which also writes each chunk's "above the band" bitmask); if the band
// held the threshold and the list did not overflow, heads_bsel_kernel finds T and need_eq
// in the list (its order, set by the reservations, does not matter: only counts do) and
// each head's counts above and at T, and the radix passes and the count pass skip the
// group; the emission then builds each head's bitmasks from the chunk bitmasks and the
// list, and reads no score. Otherwise the radix passes run.
constexpr int kHeadsRuns = 4;             // sampled 4-key runs per thread
constexpr int kGroupListCap = 32768;      // band keys a group may list
constexpr int kMaxBandHeads = 64;         // KV heads a band select handles
constexpr int kHeadShift = 18;            // list position: head << 18 | competitor index
static_assert(HCH % NWAVES == 0 && HCH % 32 == 0, "chunk split over the waves and words");
static_assert(kBitCap <= (1 << kHeadShift), "competitor index fits below the head");

// (it also writes the group's initial state: no separate init launch)
__global__ __launch_bounds__(NT) void heads_band_kernel(Dev p, const float* __restrict__ score, int n_sink,
                                                        const int64_t* __restrict__ seg_off,
                                                        HeadsState* __restrict__ st, int inner) {
  __shared__ SelectSmem sm;
  __shared__ HistSmem hs;
  const int grp = blockIdx.x, tid = threadIdx.x;
  HeadsState x = heads_state0(p, grp, n_sink, seg_off);
  if (tid == 0) st[grp] = x;  // overwritten below when a band is set
  if (x.sel != 2) return;     // uniform
  int l, s;
  group_of(p, grp, l, s);
  const int64_t M = p.cu[s + 1] - p.cu[s] - p.W - x.ns;
  const int Hkv = p.Hkv;
  const int per_head = NT * kHeadsRuns / Hkv;  // runs per head
  const int runs = per_head * Hkv;
  const int64_t tot = (int64_t)Hkv * M;
  const float MS = 4.f * (float)runs;  // sampled keys
  const float q = (float)x.kr / (float)tot;
  const float band = 2.f * (4.f * sqrtf(MS * q * (1.f - q)) + 16.f) * (float)tot / MS;
  // with inner, the host has checked every group (heads_fast) and no radix pass follows: a
  // group that still fails the exact checks (segment offsets that disagree with the budgets)
  // gets a band that cannot hold T, so the select's own fallback runs
  const bool fits = (M >> 2) >= per_head && M <= kBitCap && Hkv <= kMaxBandHeads;
  if (!fits || (!inner && band > 0.85f * kGroupListCap)) {  // uniform
    if (inner && tid == 0) {
      x.band = 1;
      x.lo = 1u;
      x.hi = 0u;
      x.list_n = kGroupListCap + 1;
      st[grp] = x;
    }
    return;
  }
  unsigned xk[kHeadsRuns][4];
  bool ok[kHeadsRuns];
#pragma unroll
  for (int i = 0; i < kHeadsRuns; ++i) {
    const int r = tid + NT * i;
    ok[i] = r < runs;
    const int h = ok[i] ? r % Hkv : 0, ri = ok[i] ? r / Hkv : 0;
    const int64_t j = (int64_t)ri * (M >> 2) / per_head * 4;  // <= M - 4
    const float* c0 = score + (int64_t)(l * Hkv + h) * p.N + p.cu[s] + x.ns + j;
#pragma unroll
    for (int e = 0; e < 4; ++e) xk[i][e] = f2key(c0[e]);
  }
  const float rho = (float)x.kr * MS / (float)tot;
  const float half = 4.f * sqrtf(rho * (1.f - rho / MS)) + 16.f;
  const int64_t nms = (int64_t)MS;
  const int64_t rh = (int64_t)floorf(rho - half), rl = (int64_t)ceilf(rho + half);
  const int64_t r0 = rh < 1 ? 1 : (rh > nms ? nms : rh), r1 = rl < 1 ? 1 : (rl > nms ? nms : rl);
  constexpr int sh0 = 32 - kBits0, sh1 = sh0 - kBits12;
  for (int i = tid; i < (1 << kBits0); i += NT) hs.hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kHeadsRuns; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) hist_add(hs.hist, ok[i], xk[i][e] >> sh0);
  __syncthreads();
  const int64_t rr[2] = {r0, r1};
  scan_digit<kPer0, 2>(sm, hs, hs.hist, 1 << kBits0, rr);
  const unsigned d0 = sm.s_digit[0], d1 = sm.s_digit[1];
  const int64_t qq[2] = {r0 - sm.s_above[0], r1 - sm.s_above[1] + (d0 != d1 ? sm.s_count[0] : 0u)};
  for (int i = tid; i < 2 << kBits12; i += NT) hs.hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kHeadsRuns; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const unsigned top = xk[i][e] >> sh0;
      const unsigned dg = ((xk[i][e] >> sh1) & ((1u << kBits12) - 1u)) | (top == d0 ? 1u << kBits12 : 0u);
      hist_add(hs.hist, ok[i] && (top == d0 || top == d1), dg);
    }
  __syncthreads();
  scan_digit<1, 2>(sm, hs, hs.hist, 2 << kBits12, qq);
  const unsigned e0 = sm.s_digit[0] & ((1u << kBits12) - 1u), e1 = sm.s_digit[1] & ((1u << kBits12) - 1u);
  if (tid == 0) {
    x.hi = rh >= 1 ? (d0 << sh0) | (e0 << sh1) | ((1u << sh1) - 1u) : ~0u;
    x.lo = rl <= nms ? (d1 << sh0) | (e1 << sh1) : 0u;
    x.band = 1;
    x.list_n = 0;
    st[grp] = x;
  }
}

// per PCH competitors of one head (four histogram chunks): the keys above the band
// (counted, and set in the head's "surely kept" bitmask in global memory; the "tied"
// bitmask's words are cleared) and in it (listed with head and competitor index in the
// group's list). Every thread has its eight float4 loads in flight at once; a word of a
// bitmask is the OR of eight lanes' nibbles. Each wave lists into an LDS region of its own
// (ballots, no atomics), then one reservation per workgroup in the group's list and
// coalesced copies; a region that overflows makes the reservation exceed the list, so the
// group takes the radix passes.
constexpr int PCH = 4 * HCH;
constexpr int kPassWaveCap = 512;  // listed keys per wave region (of the wave's 2048)
static_assert(PCH == 32 * NT, "eight float4s per thread");
__global__ __launch_bounds__(NT) void heads_pass_kernel(Dev p, const float* __restrict__ score,
                                                        HeadsState* __restrict__ st, int n_sink, int npc,
                                                        unsigned* __restrict__ above_cnt,
                                                        unsigned* __restrict__ gsure, unsigned* __restrict__ gtie,
                                                        unsigned* __restrict__ gkey, unsigned* __restrict__ ghp) {
  __shared__ unsigned wl[NWAVES][kPassWaveCap], wp[NWAVES][kPassWaveCap];
  __shared__ unsigned wn[NWAVES], wa[NWAVES];
  __shared__ unsigned s_base;
  const int u = blockIdx.y, pc = blockIdx.x;
  const int grp = u / p.Hkv, g = u % p.Hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int l, s;
  group_of(p, grp, l, s);
  // the loads need nothing from the group's state (ns as heads_state0 sets it), so they
  // are issued before it arrives; a group without a band ignores them
  const int64_t cand = p.cu[s + 1] - p.cu[s] - p.W;
  const int64_t ns = n_sink < cand ? n_sink : cand;
  const int64_t M = cand - ns;
  const int c0 = pc * PCH;  // first competitor of this workgroup (M <= kBitCap here: ints)
  const int mi = M < (int64_t)kBitCap ? (int)M : (int)kBitCap;
  const float* cb = score + (int64_t)(l * p.Hkv + g) * p.N + p.cu[s] + ns;
  const bool vec = (((size_t)cb) & 15) == 0;
  float v[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = c0 + 4 * (tid + NT * i);  // competitors j .. j+3
    if (vec && j + 4 <= mi) {
      const float4 f = *(const float4*)(cb + j);
      v[i][0] = f.x;
      v[i][1] = f.y;
      v[i][2] = f.z;
      v[i][3] = f.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[i][e] = j + e < mi ? cb[j + e] : 0.f;
    }
  }
  const HeadsState x = st[grp];
  if (x.sel != 2 || x.band != 1) return;  // uniform
  unsigned above = 0, n_w = 0;             // n_w: this wave's listed keys (uniform)
  const int64_t wb = ((int64_t)u * npc + pc) * (PCH / 32);  // this workgroup's bitmask words
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = c0 + 4 * (tid + NT * i);
    unsigned nib = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = j + e < mi;
      const unsigned key = f2key(v[i][e]);
      nib |= (ok && key > x.hi) ? 1u << e : 0u;
      const bool in = ok && key >= x.lo && key <= x.hi;
      const unsigned long long msk = __ballot(in);
      const unsigned slot =
          n_w + __builtin_amdgcn_mbcnt_hi((unsigned)(msk >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)msk, 0u));
      if (in && slot < (unsigned)kPassWaveCap) {
        wl[wave][slot] = key;
        wp[wave][slot] = (unsigned)(j + e);
      }
      n_w += (unsigned)__popcll(msk);
    }
    above += __popc(nib);
    unsigned w = nib << (4 * (lane & 7));
    w |= __shfl_xor(w, 1, 64);
    w |= __shfl_xor(w, 2, 64);
    w |= __shfl_xor(w, 4, 64);
    if ((lane & 7) == 0) {
      const int64_t wi = wb + (tid + NT * i) / 8;
      gsure[wi] = w;
      gtie[wi] = 0u;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) above += __shfl_xor(above, o, 64);
  if (lane == 0) {
    wa[wave] = above;
    wn[wave] = n_w;
  }
  __syncthreads();
  if (tid == 0) {
    unsigned ta = 0, tn = 0;
    bool over = false;
    for (int w = 0; w < NWAVES; ++w) {
      ta += wa[w];
      tn += wn[w];
      over = over || wn[w] > (unsigned)kPassWaveCap;
    }
    above_cnt[(int64_t)u * npc + pc] = ta;
    if (over) tn = kGroupListCap + 1;  // the list cannot hold the band: radix passes
    s_base = tn ? atomicAdd(&st[grp].list_n, tn) : 0u;
  }
  __syncthreads();
  unsigned before = s_base;
  for (int w = 0; w < wave; ++w) before += wn[w];
  const unsigned mine = wn[wave] < (unsigned)kPassWaveCap ? wn[wave] : (unsigned)kPassWaveCap;
  for (unsigned i = lane; i < mine; i += 64) {
    const unsigned pos = before + i;
    if (pos < (unsigned)kGroupListCap) {
      gkey[(int64_t)grp * kGroupListCap + pos] = wl[wave][i];
      ghp[(int64_t)grp * kGroupListCap + pos] = ((unsigned)g << kHeadShift) | wp[wave][i];
    }
  }
}

// per group: did the band hold T? Then T and need_eq from the listed keys (in LDS), each
// head's counts above T and at T (into the count pass's slots: chunk 0 of the head, the
// others 0), and the listed keys above T and at T set in the heads' bitmasks. If not: with
// `inner`, the select runs here from scratch over the group's keys (three reads, then a
// count per head: slow, for data the sample misjudges) and the emission reads the scores;
// else the radix passes that follow do it.
struct SmallHist {
  unsigned hist[1 << kBits12];
  int tsum[NWAVES];
};
__global__ __launch_bounds__(NT) void heads_bsel_kernel(Dev p, const float* __restrict__ score,
                                                        HeadsState* __restrict__ st, int nch, int npc, int inner,
                                                        const unsigned* __restrict__ above_cnt,
                                                        const unsigned* __restrict__ gkey,
                                                        const unsigned* __restrict__ ghp, unsigned* __restrict__ cnt,
                                                        unsigned* __restrict__ gsure, unsigned* __restrict__ gtie) {
  __shared__ SelectSmem sm;
  __shared__ SmallHist shs;
  __shared__ union {
    unsigned lk[kGroupListCap];
    HistSmem hs;
  } bu;
  __shared__ unsigned hc[3][kMaxBandHeads];  // per head: above the band, above T, at T
  const int grp = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  HeadsState x = st[grp];
  if (x.sel != 2 || x.band != 1) return;  // uniform
  const int Hkv = p.Hkv, nc = Hkv * npc;
  for (int i = tid; i < 3 * kMaxBandHeads; i += NT) (&hc[0][0])[i] = 0;
  __syncthreads();
  unsigned a = 0;
  for (int i = tid; i < nc; i += NT) {
    const unsigned v = above_cnt[(int64_t)grp * nc + i];
    a += v;
    if (v) atomicAdd(&hc[0][i / npc], v);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) a += __shfl_xor(a, o, 64);
  if (lane == 0) sm.wsum[0][wave] = (int)a;
  __syncthreads();
  int64_t A = 0;
  for (int w = 0; w < NWAVES; ++w) A += (unsigned)sm.wsum[0][w];
  const int64_t L = x.list_n;
  unsigned T;
  int64_t need_eq;
  if (L > kGroupListCap || A >= x.kr || x.kr > A + L) {  // uniform: the band did not hold T
    if (!inner) {
      if (tid == 0) st[grp].band = 0;
      return;
    }
    int l, s;
    group_of(p, grp, l, s);
    const int64_t M = p.cu[s + 1] - p.cu[s] - p.W - x.ns;
    const float* gb = score + (int64_t)l * Hkv * p.N + p.cu[s] + x.ns;  // head h: gb + h * N
    // every competitor of the group's heads, whole waves, eight loads in flight per thread
    auto each = [&](auto f) __attribute__((always_inline)) {
      for (int h = 0; h < Hkv; ++h) {
        const float* hb = gb + (int64_t)h * p.N;
        for (int64_t j0 = 0; j0 < M; j0 += 8 * NT) {
          float vv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int64_t j = j0 + tid + (int64_t)NT * e;
            vv[e] = j < M ? hb[j] : 0.f;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) f(f2key(vv[e]), h, j0 + tid + (int64_t)NT * e < M);
        }
      }
    };
    bool listed = false;
    radix_select(sm, bu.hs, [&](auto f) { each([&](unsigned key, int, bool ok) { if (ok) f(key, 0); }); }, x.kr, T,
                 need_eq, nullptr, nullptr, listed);
    // each head's keys above T and at T (counted per wave, added in LDS)
    each([&](unsigned key, int h, bool ok) {
      const unsigned long long gt = __ballot(ok && key > T), eq = __ballot(ok && key == T);
      if (lane == 0) {
        if (gt) atomicAdd(&hc[1][h], (unsigned)__popcll(gt));
        if (eq) atomicAdd(&hc[2][h], (unsigned)__popcll(eq));
      }
    });
    __syncthreads();
    for (int i = tid; i < Hkv * nch; i += NT) {
      const int h = i / nch, c = i % nch;
      cnt[((int64_t)grp * Hkv * nch + i) * 2] = c == 0 ? hc[1][h] : 0u;
      cnt[((int64_t)grp * Hkv * nch + i) * 2 + 1] = c == 0 ? hc[2][h] : 0u;
    }
    if (tid == 0) {
      x.prefix = T;
      x.need_eq = need_eq;
      x.band = 3;
      st[grp] = x;
    }
    return;
  }
  const unsigned* gk = gkey + (int64_t)grp * kGroupListCap;
  const unsigned* gh = ghp + (int64_t)grp * kGroupListCap;
  for (int i = tid; i < (int)L; i += NT) bu.lk[i] = gk[i];
  __syncthreads();
  const unsigned dif = x.lo ^ x.hi;
  const int hb = dif ? 32 - __clz((int)dif) : 0;
  list_select(sm, shs, bu.lk, (int)L, x.kr - A, hb >= 32 ? 0u : x.lo & (~0u << hb), hb, T, need_eq);
  const int64_t hw = (int64_t)npc * (PCH / 32);  // bitmask words per head
  for (int i = tid; i < (int)L; i += NT) {
    const unsigned key = bu.lk[i];
    if (key < T) continue;
    const unsigned hp = gh[i], h = hp >> kHeadShift, c = hp & ((1u << kHeadShift) - 1u);
    const int64_t wi = (int64_t)(grp * Hkv + (int)h) * hw + (c >> 5);
    if (key > T) {
      atomicAdd(&hc[1][h], 1u);
      atomicOr(&gsure[wi], 1u << (c & 31));
    } else {
      atomicAdd(&hc[2][h], 1u);
      atomicOr(&gtie[wi], 1u << (c & 31));
    }
  }
  __syncthreads();
  for (int i = tid; i < Hkv * nch; i += NT) {
    const int h = i / nch, c = i % nch;
    cnt[((int64_t)grp * Hkv * nch + i) * 2] = c == 0 ? hc[0][h] + hc[1][h] : 0u;
    cnt[((int64_t)grp * Hkv * nch + i) * 2 + 1] = c == 0 ? hc[2][h] : 0u;
  }
  if (tid == 0) {
    x.prefix = T;
    x.need_eq = need_eq;
    x.band = 2;
    st[grp] = x;
  }
}

// pass `pass` of the select: histogram of the 8-bit digit of the keys of one chunk of one
// head (unit) that match the prefix so far; whist[u][chunk][256]
__global__ __launch_bounds__(NT) void heads_hist_kernel(Dev p, const float* __restrict__ score,
                                                        const HeadsState* __restrict__ st, int pass, int nch,
                                                        unsigned* __restrict__ whist) {
  __shared__ unsigned wh[NWAVES][256];
  const int u = blockIdx.y, c = blockIdx.x;
  const int grp = u / p.Hkv, g = u % p.Hkv;
  const HeadsState x = st[grp];
  unsigned* out = whist + ((int64_t)u * nch + c) * 256;
  const int tid = threadIdx.x, wave = tid >> 6;
  if (x.sel != 2 || x.band == 2) return;  // uniform
  int l, s;
  group_of(p, grp, l, s);
  const int64_t cand = p.cu[s + 1] - p.cu[s] - p.W;
  const int64_t j0 = x.ns + (int64_t)c * HCH;
  const int64_t j1 = (j0 + HCH < cand) ? j0 + HCH : cand;
  const int shift = 24 - 8 * pass;
  const unsigned pmask = pass ? (0xFFFFFFFFu << (32 - 8 * pass)) : 0u;
  for (int i = tid; i < NWAVES * 256; i += NT) (&wh[0][0])[i] = 0;
  __syncthreads();
  const float* sc = score + (int64_t)(l * p.Hkv + g) * p.N + p.cu[s];
  auto count = [&](float v) __attribute__((always_inline)) {
    const unsigned key = f2key(v);
    hist_add(wh[wave], (key & pmask) == (x.prefix & pmask), (key >> shift) & 255u);
  };
  static_assert(HCH == 8 * NT, "eight keys per thread");
  const int64_t jt = j0 + 8 * tid;
  if (j1 - j0 == HCH && (((size_t)(sc + j0)) & 15) == 0) {  // a whole aligned chunk: 16-byte loads
    const float4 a = *(const float4*)(sc + jt), b = *(const float4*)(sc + jt + 4);
    count(a.x);
    count(a.y);
    count(a.z);
    count(a.w);
    count(b.x);
    count(b.y);
    count(b.z);
    count(b.w);
  } else {
    for (int64_t j = j0 + tid; j < j1; j += NT) count(sc[j]);
  }
  __syncthreads();
  if (tid < 256) {
    unsigned t = 0;
    for (int w = 0; w < NWAVES; ++w) t += wh[w][tid];
    out[tid] = t;  // a chunk past the head's competitors writes zeros
  }
}

// per group: sum the chunks' histograms (heads and chunks in ascending order) and place the
// rank: the digit where the count from the top first reaches kr
__global__ __launch_bounds__(1024) void heads_digit_kernel(Dev p, HeadsState* __restrict__ st, int pass, int nch,
                                                           const unsigned* __restrict__ whist) {
  __shared__ unsigned part[4][256];
  __shared__ unsigned bins[256];
  __shared__ int s_digit;
  __shared__ long long s_above;
  const int grp = blockIdx.x;
  HeadsState x = st[grp];
  if (x.sel != 2 || x.band == 2) return;  // uniform
  // bin b of histogram i (i = head * nch + chunk) is summed by the threads b + 256q for
  // q = i % 4; integer counts, so the order of the sums does not matter
  const int t = threadIdx.x & 255, q = threadIdx.x >> 8;
  const int nh = p.Hkv * nch;
  const unsigned* h0 = whist + (int64_t)grp * nh * 256 + t;
  unsigned tot = 0;
  int i = q;
  for (; i + 28 < nh; i += 32) {  // eight loads in flight
    unsigned v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = h0[(int64_t)(i + 4 * e) * 256];
#pragma unroll
    for (int e = 0; e < 8; ++e) tot += v[e];
  }
  for (; i < nh; i += 4) tot += h0[(int64_t)i * 256];
  part[q][t] = tot;
  __syncthreads();
  if (threadIdx.x < 256) bins[t] = part[0][t] + part[1][t] + part[2][t] + part[3][t];
  __syncthreads();
  if (threadIdx.x < 64) {
    // lane L owns digits 255-4L .. 252-4L (descending)
    unsigned c4[4], sum = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      c4[e] = bins[255 - 4 * t - e];
      sum += c4[e];
    }
    const int incl = wave_incl_scan((int)sum, t);
    const int excl = incl - (int)sum;
    if ((long long)excl < x.kr && x.kr <= (long long)incl) {
      long long above = excl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (above + c4[e] >= x.kr) {
          s_digit = 255 - 4 * t - e;
          s_above = above;
          break;
        }
        above += c4[e];
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    x.prefix |= (unsigned)s_digit << (24 - 8 * pass);
    x.kr -= s_above;
    if (pass == 3) x.need_eq = x.kr;
    st[grp] = x;
  }
}

// per chunk of one head: how many competitors are above T and how many equal it
__global__ __launch_bounds__(NT) void heads_count_kernel(Dev p, const float* __restrict__ score,
                                                         const HeadsState* __restrict__ st, int nch,
                                                         unsigned* __restrict__ cnt) {
  __shared__ unsigned red[2][NWAVES];
  const int u = blockIdx.y, c = blockIdx.x;
  const int grp = u / p.Hkv, g = u % p.Hkv;
  const HeadsState x = st[grp];
  if (x.sel != 2 || x.band == 2) return;  // uniform (a band select wrote the counts)
  int l, s;
  group_of(p, grp, l, s);
  const int64_t cand = p.cu[s + 1] - p.cu[s] - p.W;
  const int64_t j0 = x.ns + (int64_t)c * HCH;
  const int64_t j1 = (j0 + HCH < cand) ? j0 + HCH : cand;
  const float* sc = score + (int64_t)(l * p.Hkv + g) * p.N + p.cu[s];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  unsigned cs = 0, ce = 0;
  for (int64_t j = j0 + tid; j < j1; j += NT) {
    const unsigned key = f2key(sc[j]);
    cs += key > x.prefix;
    ce += key == x.prefix;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    cs += __shfl_xor(cs, o, 64);
    ce += __shfl_xor(ce, o, 64);
  }
  if (lane == 0) {
    red[0][wave] = cs;
    red[1][wave] = ce;
  }
  __syncthreads();
  if (tid == 0) {
    unsigned ts = 0, te = 0;
    for (int w = 0; w < NWAVES; ++w) {
      ts += red[0][w];
      te += red[1][w];
    }
    cnt[((int64_t)u * nch + c) * 2] = ts;
    cnt[((int64_t)u * nch + c) * 2 + 1] = te;
  }
}

// one workgroup per head: its kept count (above T plus its share of the first need_eq ties
// in (head, position) order), its offset inside the group's block, then its positions
__global__ __launch_bounds__(NT) void heads_emit_kernel(Dev p, const float* __restrict__ score,
                                                        const HeadsState* __restrict__ st, int nch,
                                                        const unsigned* __restrict__ cnt,
                                                        const int64_t* __restrict__ seg_off,
                                                        int64_t* __restrict__ head_off, int32_t* __restrict__ kept,
                                                        int npc, const unsigned* __restrict__ gsure,
                                                        const unsigned* __restrict__ gtie) {
  __shared__ SelectSmem sm;
  __shared__ unsigned bm[2 * kBitWords];
  const int u = blockIdx.x;
  const int grp = u / p.Hkv, g = u % p.Hkv;
  const HeadsState x = st[grp];
  int l, s;
  group_of(p, grp, l, s);
  const int64_t n = p.cu[s + 1] - p.cu[s];
  const int64_t cand = n - p.W;
  const int64_t ns = x.ns;
  const int64_t M = cand - ns;
  // the kept competitors of head h: above T plus its share of the ties
  int64_t ties_before = 0, off = seg_off[grp * p.Hkv], kg = 0, take = 0;
  const int ncs = x.band >= 2 ? 1 : nch;  // the select kernel wrote each head's totals to chunk 0
  for (int h = 0; h <= g; ++h) {
    int64_t sure = 0, eq = 0;
    if (x.sel == 2) {
      for (int c = 0; c < ncs; ++c) {
        sure += cnt[((int64_t)(grp * p.Hkv + h) * nch + c) * 2];
        eq += cnt[((int64_t)(grp * p.Hkv + h) * nch + c) * 2 + 1];
      }
    }
    int64_t tk = x.need_eq - ties_before;
    if (tk < 0) tk = 0;
    if (tk > eq) tk = eq;
    ties_before += eq;
    const int64_t kh = (x.sel == 1) ? M : (x.sel == 2 ? sure + tk : 0);
    if (h < g) off += p.W + ns + kh;
    else {
      kg = kh;
      take = tk;
    }
  }
  const int64_t bg = p.W + ns + kg;
  if (threadIdx.x == 0) {
    head_off[u] = off;
    if (u == p.U - 1) head_off[p.U] = off + bg;
  }
  if (x.sel == 2 && x.band == 2) {
    // the head's bitmasks, complete in global memory
    const int tid = threadIdx.x;
    unsigned* sure = bm;
    unsigned* tie = bm + kBitWords;
    const int nw = (int)((M + 31) >> 5);  // M <= kBitCap
    const int64_t hw = (int64_t)u * npc * (PCH / 32);
    for (int i = tid; i < nw; i += NT) {
      sure[i] = gsure[hw + i];
      tie[i] = gtie[hw + i];
    }
    __syncthreads();
    emit_words(sm, kept + off, bg, take, sure, tie, n, cand, ns);
    return;
  }
  const float* sc = score + (int64_t)(l * p.Hkv + g) * p.N + p.cu[s];
  emit_segment(sm, kept + off, bg, x.sel, x.prefix, take, sc, n, cand, ns);
}

}  // namespace

// Whether every group of a joint select can take the sampled band with the select's own
// fallback (no radix pass launched): competitors within the bitmasks, few enough heads,
// enough competitors for the sample, a band expected to fit the list. budgets: host
// [S][L], the segment lengths.
bool heads_fast(const Dev& p, const int32_t* budgets, int n_sink) {
  const int Hkv = p.Hkv, per_head = NT * kHeadsRuns / Hkv;
  if (Hkv > kMaxBandHeads) return false;
  for (int l = 0; l < p.L; ++l)
    for (int s = 0; s < p.S; ++s) {
      const int64_t cand = p.cu[s + 1] - p.cu[s] - p.W;
      const int64_t ns = n_sink < cand ? n_sink : cand;
      const int64_t M = cand - ns;
      int64_t kt = (int64_t)Hkv * ((int64_t)budgets[(int64_t)s * p.L + l] - p.W - ns);
      if (kt <= 0 || kt >= (int64_t)Hkv * M) continue;  // nothing to select
      if ((M >> 2) < per_head || M > kBitCap) return false;
      const double tot = (double)Hkv * (double)M, MS = 4.0 * per_head * Hkv, q = (double)kt / tot;
      const double band = 2.0 * (4.0 * std::sqrt(MS * q * (1.0 - q)) + 16.0) * tot / MS;
      if (band > 0.8 * kGroupListCap) return false;
    }
  return true;
}

hipError_t launch_topk(const Dev& p, const float* score, const int64_t* seg_off, int32_t* kept, int pool, int n_sink,
                       float* pooled, int64_t* head_off, void* heads_ws, const int32_t* budgets, hipStream_t st) {
  const float* key = score;
  if (pool > 1) {
    const dim3 gp((unsigned)((p.max_n + PT - 1) / PT), p.U);
    hipLaunchKernelGGL(pool_kernel, gp, dim3(256), 0, st, p, score, pool, pooled);
    key = pooled;
  }
  if (!head_off) {
    hipLaunchKernelGGL(topk_kernel, dim3(p.U), dim3(NT), 0, st, p, key, n_sink, seg_off, kept);
    return hipGetLastError();
  }
  // head budgets chosen jointly; scratch: states | chunk histograms | chunk counts | counts
  // above the band | the heads' "surely kept" and "tied" bitmasks | the groups' band lists
  // (keys, then head and competitor index)
  const int groups = p.U / p.Hkv;
  const int nch = heads_chunks(p);
  HeadsState* hs = (HeadsState*)heads_ws;
  unsigned* whist = (unsigned*)((char*)heads_ws + heads_state_bytes(p));
  unsigned* cnt = whist + (size_t)p.U * nch * 256;
  const int npc = (nch + 3) / 4;  // band-pass workgroups per head (PCH competitors each)
  unsigned* above = cnt + (size_t)p.U * nch * 2;
  unsigned* gsure = above + (size_t)p.U * npc;
  unsigned* gtie = gsure + (size_t)p.U * npc * (PCH / 32);
  unsigned* gkey = gtie + (size_t)p.U * npc * (PCH / 32);
  unsigned* ghp = gkey + (size_t)groups * kGroupListCap;
  const int inner = heads_fast(p, budgets, n_sink) ? 1 : 0;
  hipLaunchKernelGGL(heads_band_kernel, dim3(groups), dim3(NT), 0, st, p, key, n_sink, seg_off, hs, inner);
  hipLaunchKernelGGL(heads_pass_kernel, dim3(npc, p.U), dim3(NT), 0, st, p, key, hs, n_sink, npc, above, gsure, gtie,
                     gkey, ghp);
  hipLaunchKernelGGL(heads_bsel_kernel, dim3(groups), dim3(NT), 0, st, p, key, hs, nch, npc, inner,
                     (const unsigned*)above, (const unsigned*)gkey, (const unsigned*)ghp, cnt, gsure, gtie);
  if (!inner) {  // groups without a band: the radix passes, then the count
    for (int pass = 0; pass < 4; ++pass) {
      hipLaunchKernelGGL(heads_hist_kernel, dim3(nch, p.U), dim3(NT), 0, st, p, key, (const HeadsState*)hs, pass, nch,
                         whist);
      hipLaunchKernelGGL(heads_digit_kernel, dim3(groups), dim3(1024), 0, st, p, hs, pass, nch, (const unsigned*)whist);
    }
    hipLaunchKernelGGL(heads_count_kernel, dim3(nch, p.U), dim3(NT), 0, st, p, key, (const HeadsState*)hs, nch, cnt);
  }
  hipLaunchKernelGGL(heads_emit_kernel, dim3(p.U), dim3(NT), 0, st, p, key, (const HeadsState*)hs, nch,
                     (const unsigned*)cnt, seg_off, head_off, kept, npc, (const unsigned*)gsure,
                     (const unsigned*)gtie);
  return hipGetLastError();
}

int heads_chunks(const Dev& p) { return (int)((p.max_n - p.W + HCH - 1) / HCH); }
size_t heads_state_bytes(const Dev& p) { return ((size_t)(p.U / p.Hkv) * sizeof(HeadsState) + 255) / 256 * 256; }
size_t heads_ws_bytes(const Dev& p) {
  const size_t nch = (size_t)heads_chunks(p);
  const size_t npc = (nch + 3) / 4;
  return heads_state_bytes(p) + ((size_t)p.U * nch * (256 + 2) * 4 + (size_t)p.U * npc * (1 + 2 * PCH / 32) * 4 +
                                 (size_t)(p.U / p.Hkv) * kGroupListCap * 2 * 4 + 255) / 256 * 256;
}

}  // namespace kvs
