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
// One 1024-thread workgroup per (layer, sequence, KV head) unit. Radix select of the
// k-th largest key over order-preserving uint32 images of the fp32 scores (4 passes of
// 8 bits, per-wave LDS histograms merged in wave order, digit found by a wave scan),
// which gives the threshold T and how many elements equal to T are taken. Then an
// ordered stream compaction in rounds of 4096 positions: a block scan of "surely
// kept" (window, or key > T) and "tied" (key == T) counts gives every kept position
// its slot; ties are taken by ascending position.
#include "kvs_internal.hpp"

namespace kvs {
namespace {

constexpr int NT = 1024;
constexpr int NWAVES = NT / 64;

__device__ inline unsigned f2key(float x) {
  const unsigned b = __float_as_uint(x == 0.f ? 0.f : x);  // +0 and -0 share a key
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ inline int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
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
  for (int i = threadIdx.x; i < PT + 2 * h; i += 256) {
    const int64_t j = j0 - h + i;
    tile[i] = (j >= 0 && j < cand) ? sc[j] : -INFINITY;
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

__global__ __launch_bounds__(NT) void topk_kernel(Dev p, const float* __restrict__ score, int n_sink,
                                                 const int64_t* __restrict__ seg_off, int32_t* __restrict__ kept) {
  __shared__ unsigned whist[NWAVES][256];
  __shared__ unsigned hist[256];
  __shared__ unsigned s_digit, s_above;
  __shared__ int wsum[2][NWAVES];

  const int u = blockIdx.x;
  int l, s, g;
  unit_coords(p, u, l, s, g);
  const int64_t n = p.cu[s + 1] - p.cu[s];
  const int64_t cand = n - p.W;
  const int64_t ns = n_sink < cand ? n_sink : cand;  // pinned sinks [0, ns); competitors [ns, cand)
  const int64_t off0 = seg_off[u];
  const int64_t b = seg_off[u + 1] - off0;
  int64_t k = b - p.W - ns;
  if (k < 0) k = 0;
  if (k > cand - ns) k = cand - ns;
  const float* sc = score + (int64_t)(l * p.Hkv + g) * p.N + p.cu[s];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  // 0: keep no candidate, 1: keep all candidates, 2: keep key > T and the first need_eq keys == T
  int sel = (k == 0) ? 0 : (k == cand - ns ? 1 : 2);
  unsigned T = 0;
  int64_t need_eq = 0;
  if (sel == 2) {
    unsigned prefix = 0, pmask = 0;
    int64_t kr = k;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < NWAVES * 256; i += NT) (&whist[0][0])[i] = 0;
      __syncthreads();
      for (int64_t j = ns + tid; j < cand; j += NT) {
        const unsigned key = f2key(sc[j]);
        if ((key & pmask) == prefix) atomicAdd(&whist[wave][(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 256) {
        unsigned c = 0;
        for (int w = 0; w < NWAVES; ++w) c += whist[w][tid];
        hist[tid] = c;
      }
      __syncthreads();
      if (wave == 0) {
        // lane L owns digits 255-4L .. 252-4L (descending); find the digit where the
        // running count from the top first reaches kr.
        unsigned c4[4], tot = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          c4[e] = hist[255 - 4 * lane - e];
          tot += c4[e];
        }
        const int incl = wave_incl_scan((int)tot, lane);
        const int excl = incl - (int)tot;
        if ((int64_t)excl < kr && kr <= (int64_t)incl) {
          unsigned above = (unsigned)excl;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if ((int64_t)(above + c4[e]) >= kr) {
              s_digit = 255u - 4u * lane - e;
              s_above = above;
              break;
            }
            above += c4[e];
          }
        }
      }
      __syncthreads();
      prefix |= s_digit << shift;
      pmask |= 255u << shift;
      kr -= s_above;
    }
    T = prefix;
    need_eq = kr;
  }

  int32_t* out = kept + off0;
  int64_t sure_base = 0, eq_base = 0;
  for (int64_t base = 0; base < n; base += 4 * NT) {
    bool sure[4], tie[4];
    int cs = 0, ce = 0;
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
          const unsigned key = f2key(sc[j]);
          sure[e] = key > T;
          tie[e] = key == T;
        }
      }
      cs += sure[e];
      ce += tie[e];
    }
    const int is = wave_incl_scan(cs, lane), ie = wave_incl_scan(ce, lane);
    if (lane == 63) {
      wsum[0][wave] = is;
      wsum[1][wave] = ie;
    }
    __syncthreads();
    int ps = is - cs, pe = ie - ce, ts = 0, te = 0;
    for (int w = 0; w < NWAVES; ++w) {
      if (w < wave) {
        ps += wsum[0][w];
        pe += wsum[1][w];
      }
      ts += wsum[0][w];
      te += wsum[1][w];
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

}  // namespace

hipError_t launch_topk(const Dev& p, const float* score, const int64_t* seg_off, int32_t* kept, int pool, int n_sink,
                       float* pooled, hipStream_t st) {
  const float* key = score;
  if (pool > 1) {
    const dim3 gp((unsigned)((p.max_n + PT - 1) / PT), p.U);
    hipLaunchKernelGGL(pool_kernel, gp, dim3(256), 0, st, p, score, pool, pooled);
    key = pooled;
  }
  hipLaunchKernelGGL(topk_kernel, dim3(p.U), dim3(NT), 0, st, p, key, n_sink, seg_off, kept);
  return hipGetLastError();
}

}  // namespace kvs
