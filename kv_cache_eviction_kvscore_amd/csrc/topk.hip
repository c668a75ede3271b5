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

struct SelectSmem {
  unsigned whist[NWAVES][256];
  unsigned hist[256];
  unsigned s_digit, s_above;
  int wsum[2][NWAVES];
  long long red[2][NWAVES];
};

// Radix select of the kr-th largest key among the keys `visit` enumerates (each thread
// calls f(key) on its share): T = that key, need_eq = how many keys equal to T are among
// the kr largest. 4 passes of 8 bits; per-wave LDS histograms merged in wave order; the
// digit is found by a wave scan.
template <class Visit>
__device__ void radix_select(SelectSmem& sm, Visit visit, int64_t kr, unsigned& T, int64_t& need_eq) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  unsigned prefix = 0, pmask = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < NWAVES * 256; i += NT) (&sm.whist[0][0])[i] = 0;
    __syncthreads();
    visit([&](unsigned key) {
      if ((key & pmask) == prefix) atomicAdd(&sm.whist[wave][(key >> shift) & 255u], 1u);
    });
    __syncthreads();
    if (tid < 256) {
      unsigned c = 0;
      for (int w = 0; w < NWAVES; ++w) c += sm.whist[w][tid];
      sm.hist[tid] = c;
    }
    __syncthreads();
    if (wave == 0) {
      // lane L owns digits 255-4L .. 252-4L (descending); find the digit where the
      // running count from the top first reaches kr.
      unsigned c4[4], tot = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c4[e] = sm.hist[255 - 4 * lane - e];
        tot += c4[e];
      }
      const int incl = wave_incl_scan((int)tot, lane);
      const int excl = incl - (int)tot;
      if ((int64_t)excl < kr && kr <= (int64_t)incl) {
        unsigned above = (unsigned)excl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if ((int64_t)(above + c4[e]) >= kr) {
            sm.s_digit = 255u - 4u * lane - e;
            sm.s_above = above;
            break;
          }
          above += c4[e];
        }
      }
    }
    __syncthreads();
    prefix |= sm.s_digit << shift;
    pmask |= 255u << shift;
    kr -= sm.s_above;
  }
  T = prefix;
  need_eq = kr;
}

// Ordered stream compaction of one segment (b rows at out): positions j in [0, n), kept
// when j < ns or j >= cand (sinks, window), or by the selection: sel 0 none, 1 all,
// 2 key > T and the first need_eq keys equal to T (ascending position). Rounds of 4096
// positions; a block scan gives every kept position its slot.
__device__ void emit_segment(SelectSmem& sm, int32_t* __restrict__ out, int64_t b, int sel, unsigned T,
                             int64_t need_eq, const float* __restrict__ sc, int64_t n, int64_t cand, int64_t ns) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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
      sm.wsum[0][wave] = is;
      sm.wsum[1][wave] = ie;
    }
    __syncthreads();
    int ps = is - cs, pe = ie - ce, ts = 0, te = 0;
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

__global__ __launch_bounds__(NT) void topk_kernel(Dev p, const float* __restrict__ score, int n_sink,
                                                 const int64_t* __restrict__ seg_off, int32_t* __restrict__ kept) {
  __shared__ SelectSmem sm;
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
  const int tid = threadIdx.x;

  // 0: keep no candidate, 1: keep all candidates, 2: keep key > T and the first need_eq keys == T
  const int sel = (k == 0) ? 0 : (k == cand - ns ? 1 : 2);
  unsigned T = 0;
  int64_t need_eq = 0;
  if (sel == 2)
    radix_select(sm, [&](auto f) {
      for (int64_t j = ns + tid; j < cand; j += NT) f(f2key(sc[j]));
    }, k, T, need_eq);
  emit_segment(sm, kept + off0, b, sel, T, need_eq, sc, n, cand, ns);
}

// Head budgets chosen jointly: one workgroup per (sequence, layer). The layer keeps
// Hkv * b rows (b = the segment length seg_off gives its heads); every head keeps its sinks
// and window; the Hkv * (b - W - ns) other slots go to the largest keys over all heads'
// competitors, ties to the lower head, then the lower position. Writes the heads' offsets
// (inside the layer's block of seg_off) to head_off and their positions to kept.
__global__ __launch_bounds__(NT) void topk_heads_kernel(Dev p, const float* __restrict__ score, int n_sink,
                                                       const int64_t* __restrict__ seg_off,
                                                       int64_t* __restrict__ head_off, int32_t* __restrict__ kept) {
  __shared__ SelectSmem sm;
  const int blk = blockIdx.x;  // l*S + s
  const int l = blk / p.S, s = blk % p.S;
  const int H = p.Hkv;
  const int u0 = blk * H;
  const int64_t n = p.cu[s + 1] - p.cu[s];
  const int64_t cand = n - p.W;
  const int64_t ns = n_sink < cand ? n_sink : cand;
  const int64_t M = cand - ns;  // competitors per head
  const int64_t base0 = seg_off[u0];
  const int64_t b = seg_off[u0 + 1] - base0;  // every head of the layer has the layer's budget
  int64_t kt = (int64_t)H * (b - p.W - ns);
  if (kt < 0) kt = 0;
  if (kt > (int64_t)H * M) kt = (int64_t)H * M;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  auto head_sc = [&](int g) { return score + (int64_t)(l * H + g) * p.N + p.cu[s]; };

  const int sel = (kt == 0) ? 0 : (kt == (int64_t)H * M ? 1 : 2);
  unsigned T = 0;
  int64_t need_eq = 0;
  if (sel == 2)
    radix_select(sm, [&](auto f) {
      for (int g = 0; g < H; ++g) {
        const float* sc = head_sc(g);
        for (int64_t j = ns + tid; j < cand; j += NT) f(f2key(sc[j]));
      }
    }, kt, T, need_eq);

  // per head: kept competitors k_g = (key > T) + its share of the first need_eq ties in
  // (head, position) order; then the heads' offsets inside the layer's block
  int64_t off = base0, ties_before = 0;
  for (int g = 0; g < H; ++g) {
    int64_t kg = 0, take = 0;
    if (sel == 1) {
      kg = M;
    } else if (sel == 2) {
      const float* sc = head_sc(g);
      long long cs = 0, ce = 0;
      for (int64_t j = ns + tid; j < cand; j += NT) {
        const unsigned key = f2key(sc[j]);
        cs += key > T;
        ce += key == T;
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        cs += __shfl_xor(cs, o, 64);
        ce += __shfl_xor(ce, o, 64);
      }
      if (lane == 0) {
        sm.red[0][wave] = cs;
        sm.red[1][wave] = ce;
      }
      __syncthreads();
      long long ts = 0, te = 0;
      for (int w = 0; w < NWAVES; ++w) {
        ts += sm.red[0][w];
        te += sm.red[1][w];
      }
      __syncthreads();  // red is rewritten for the next head
      take = need_eq - ties_before;
      if (take < 0) take = 0;
      if (take > te) take = te;
      ties_before += te;
      kg = ts + take;
    }
    const int64_t bg = p.W + ns + kg;
    if (tid == 0) head_off[u0 + g] = off;
    emit_segment(sm, kept + off, bg, sel, T, take, head_sc(g), n, cand, ns);
    off += bg;
  }
  if (tid == 0 && u0 + H == p.U) head_off[p.U] = off;  // the last layer block closes the array
}

}  // namespace

hipError_t launch_topk(const Dev& p, const float* score, const int64_t* seg_off, int32_t* kept, int pool, int n_sink,
                       float* pooled, int64_t* head_off, hipStream_t st) {
  const float* key = score;
  if (pool > 1) {
    const dim3 gp((unsigned)((p.max_n + PT - 1) / PT), p.U);
    hipLaunchKernelGGL(pool_kernel, gp, dim3(256), 0, st, p, score, pool, pooled);
    key = pooled;
  }
  if (head_off)
    hipLaunchKernelGGL(topk_heads_kernel, dim3(p.U / p.Hkv), dim3(NT), 0, st, p, key, n_sink, seg_off, head_off, kept);
  else
    hipLaunchKernelGGL(topk_kernel, dim3(p.U), dim3(NT), 0, st, p, key, n_sink, seg_off, kept);
  return hipGetLastError();
}

}  // namespace kvs
