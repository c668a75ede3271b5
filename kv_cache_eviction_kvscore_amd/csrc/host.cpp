// libkvscore host glue: argument validation, launch sizing, workspace sizes, the
// host-only layer-budget map, and the C ABI declared in include/kvscore.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <vector>

#include "../../include/kvscore.h"
#include "kvs_budget.hpp"
#include "kvs_internal.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return KVSCORE_OK;
}

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

// MI355X compute units, and the measured cost of one more round of workgroups per CU, in
// keys of one unit's chunk, for the forward (prologue, the running max's warm-up, one more
// record) and the score pass (prologue); the score kernel's tile flags cap its chunk
constexpr int64_t kNumCUs = 256;
constexpr int64_t kFwdChunkCost = 4096;
constexpr int64_t kScoreChunkCost = 512;
constexpr int64_t kScoreMaxChunk = 65536;

int64_t next_pow2(int64_t x) {
  int64_t r = 1;
  while (r < x) r <<= 1;
  return r;
}

// Validate the problem and fill the kernels' view of it.
int make_dev(const kvscore_problem* p, kvs::Dev& d) {
  if (!p) return fail(KVSCORE_EINVAL, "problem is NULL");
  if (p->num_seqs < 1 || p->num_seqs > KVSCORE_MAX_SEQS)
    return fail(KVSCORE_EINVAL, "num_seqs=%d outside [1, %d]", p->num_seqs, KVSCORE_MAX_SEQS);
  if (p->num_layers < 1) return fail(KVSCORE_EINVAL, "num_layers=%d < 1", p->num_layers);
  if (p->num_kv_heads < 1 || p->num_q_heads < p->num_kv_heads || p->num_q_heads % p->num_kv_heads != 0)
    return fail(KVSCORE_EINVAL, "num_q_heads=%d must be a positive multiple of num_kv_heads=%d", p->num_q_heads,
                p->num_kv_heads);
  if (p->head_dim != 64 && p->head_dim != 128) return fail(KVSCORE_EINVAL, "head_dim=%d not in {64, 128}", p->head_dim);
  if (p->window < 1) return fail(KVSCORE_EINVAL, "window=%d < 1", p->window);
  const int G = p->num_q_heads / p->num_kv_heads;
  if ((int64_t)G * p->window > KVSCORE_MAX_ROWS)
    return fail(KVSCORE_EINVAL, "G*W=%lld query rows per unit exceeds %d", (long long)G * p->window, KVSCORE_MAX_ROWS);
  if (!std::isfinite(p->softmax_scale))
    return fail(KVSCORE_EINVAL, "softmax_scale must be finite (<= 0 selects 1/sqrt(head_dim))");
  if (p->mode != KVSCORE_MODE_L2 && p->mode != KVSCORE_MODE_SQ && p->mode != KVSCORE_MODE_ATTN)
    return fail(KVSCORE_EINVAL, "mode=%d", p->mode);
  if (!p->cu_seqlens) return fail(KVSCORE_EINVAL, "cu_seqlens is NULL");
  if (p->cu_seqlens[0] != 0) return fail(KVSCORE_EINVAL, "cu_seqlens[0] must be 0");
  int64_t max_n = 0;
  for (int s = 0; s < p->num_seqs; ++s) {
    const int64_t n = p->cu_seqlens[s + 1] - p->cu_seqlens[s];
    if (n <= p->window) return fail(KVSCORE_EINVAL, "sequence %d has length %lld <= window %d", s, (long long)n, p->window);
    if (n >= (int64_t)1 << 30) return fail(KVSCORE_EINVAL, "sequence %d too long", s);
    max_n = std::max(max_n, n);
  }
  for (int t = 0; t < 3; ++t)
    if (p->k_strides[t] < 0 || p->v_strides[t] < 0 || p->k_strides[t] % 8 || p->v_strides[t] % 8)
      return fail(KVSCORE_EINVAL, "k/v strides must be non-negative multiples of 8 elements (16 bytes)");
  if (p->k_strides[2] < p->head_dim || p->v_strides[2] < p->head_dim)
    return fail(KVSCORE_EINVAL, "token stride smaller than head_dim");
  // the kernels address a 64-token tile from its first row with 32-bit byte offsets
  if (p->k_strides[2] >= ((int64_t)1 << 22) || p->v_strides[2] >= ((int64_t)1 << 22))
    return fail(KVSCORE_EINVAL, "token stride must be below 2^22 elements");

  // units index gridDim.y or gridDim.z of every launch, whose limit is 65535
  const int64_t units = (int64_t)p->num_layers * p->num_seqs * p->num_kv_heads;
  if (units > kvs::kMaxUnits)
    return fail(KVSCORE_EINVAL, "num_layers*num_seqs*num_kv_heads = %lld units exceeds %d", (long long)units,
                kvs::kMaxUnits);

  d = kvs::Dev{};
  d.S = p->num_seqs;
  d.L = p->num_layers;
  d.Hq = p->num_q_heads;
  d.Hkv = p->num_kv_heads;
  d.G = G;
  d.d = p->head_dim;
  d.W = p->window;
  d.R = G * p->window;
  d.Tq = (d.R + kvs::kRowsPerTileMax - 1) / kvs::kRowsPerTileMax;
  d.RT = ((d.R + d.Tq - 1) / d.Tq + 31) / 32 * 32;
  d.mode = p->mode;
  d.scale = p->softmax_scale > 0.f ? p->softmax_scale : 1.0f / std::sqrt((float)p->head_dim);
  d.c1 = (float)((double)d.scale * 1.4426950408889634);
  d.ksl = p->k_strides[0];
  d.ksh = p->k_strides[1];
  d.kst = p->k_strides[2];
  d.vsl = p->v_strides[0];
  d.vsh = p->v_strides[1];
  d.vst = p->v_strides[2];
  d.N = p->cu_seqlens[p->num_seqs];
  d.U = d.L * d.S * d.Hkv;
  d.max_n = max_n;
  for (int s = 0; s <= p->num_seqs; ++s) d.cu[s] = p->cu_seqlens[s];
  // Chunk sizes: a power of two of 1024 keys or more that minimises an estimated makespan
  // in keys: rounds x chunk when every workgroup has the same length, else keys per CU +
  // half a chunk of tail; plus a fixed cost per round of workgroups. One workgroup of
  // either pass fills a CU. A forward chunk restarts its running max (a warm-up in which
  // many rows' argmax moves) and adds a record to combine; a score chunk only reloads its
  // row operands.
  int64_t keys = 0;
  for (int s = 0; s < p->num_seqs; ++s) keys += (p->cu_seqlens[s + 1] - p->cu_seqlens[s]);
  const int64_t groups_per_seq = (int64_t)d.L * d.Hkv * d.Tq;
  keys *= groups_per_seq;
  auto pick_chunk = [&](int64_t round_cost, int64_t cap) {
    int64_t best = -1, best_c = 1024;
    for (int64_t c = 1024; c <= std::min(cap, std::max<int64_t>(1024, next_pow2(max_n))); c *= 2) {
      int64_t nwg = 0, lo = INT64_MAX, hi = 0;
      for (int s = 0; s < p->num_seqs; ++s) {
        const int64_t n = p->cu_seqlens[s + 1] - p->cu_seqlens[s];
        nwg += (n + c - 1) / c;
        if (n >= c) lo = std::min(lo, c), hi = std::max(hi, c);
        if (n % c) lo = std::min(lo, n % c), hi = std::max(hi, n % c);
      }
      nwg *= groups_per_seq;
      const int64_t rounds = (nwg + kNumCUs - 1) / kNumCUs, ce = std::min(c, max_n);
      const int64_t span = (lo == hi) ? rounds * ce : std::max((keys + kNumCUs - 1) / kNumCUs, ce) + ce / 2;
      const int64_t cost = span + round_cost * rounds;
      if (best < 0 || cost <= best) {  // ties go to the longer chunk
        best = cost;
        best_c = c;
      }
    }
    return (int)best_c;
  };
  d.fwd_chunk = pick_chunk(kFwdChunkCost, INT64_MAX);
  d.score_chunk = pick_chunk(kScoreChunkCost, kScoreMaxChunk);
  d.fwd_chunks = (int)((max_n + d.fwd_chunk - 1) / d.fwd_chunk);
  d.score_chunks = (int)((max_n + d.score_chunk - 1) / d.score_chunk);
  return ok();
}

// the forward's per-chunk records; none when every sequence is one key chunk (the partial
// kernel then writes the outputs itself)
size_t ws_attn(const kvs::Dev& d) {
  if (d.fwd_chunks == 1) return 0;
  return (size_t)d.U * d.Tq * d.fwd_chunks * kvs::fwd_block_floats(d.RT, d.d) * sizeof(float);
}
size_t ws_score(const kvs::Dev& d) { return kvs::prep_bytes((int64_t)d.U * d.R, d.d); }
size_t ws_topk(const kvs::Dev& d) { return (size_t)d.L * d.Hkv * d.N * sizeof(float); }  // pooled keys

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(KVSCORE_EDEVICE, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

int check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return ok();
  if (!ws) return fail(KVSCORE_EWORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (!aligned(ws, 256)) return fail(KVSCORE_EWORKSPACE, "workspace must be 256-byte aligned");
  if (have < need) return fail(KVSCORE_EWORKSPACE, "workspace has %zu bytes, need %zu", have, need);
  return ok();
}

int check_budgets(const kvscore_problem* p, const int32_t* budgets, int* max_b) {
  if (!budgets) return fail(KVSCORE_EINVAL, "budgets is NULL");
  int mb = 0;
  for (int s = 0; s < p->num_seqs; ++s) {
    const int64_t n = p->cu_seqlens[s + 1] - p->cu_seqlens[s];
    for (int l = 0; l < p->num_layers; ++l) {
      const int32_t b = budgets[(int64_t)s * p->num_layers + l];
      if (b < p->window || b > n)
        return fail(KVSCORE_EBUDGET, "budget[%d][%d]=%d outside [window=%d, n=%lld]", s, l, b, p->window, (long long)n);
      mb = std::max(mb, (int)b);
    }
  }
  if (max_b) *max_b = mb;
  return ok();
}

// Decode attention problem: the model shape of p and the packed segment offsets (host
// copy). Only the shape fields, head_dim and softmax_scale of p are used.
int make_decdev(const kvscore_problem* p, const int64_t* off, kvs::DecDev& d) {
  if (!p) return fail(KVSCORE_EINVAL, "problem is NULL");
  if (p->num_seqs < 1 || p->num_seqs > KVSCORE_MAX_SEQS) return fail(KVSCORE_EINVAL, "num_seqs out of range");
  if (p->num_layers < 1 || p->num_kv_heads < 1 || p->num_q_heads < 1)
    return fail(KVSCORE_EINVAL, "layers and heads must be positive");
  if (p->num_q_heads % p->num_kv_heads) return fail(KVSCORE_EINVAL, "num_q_heads not a multiple of num_kv_heads");
  const int G = p->num_q_heads / p->num_kv_heads;
  if (G > kvs::kDecodeMaxGroup) return fail(KVSCORE_EINVAL, "decode takes at most %d query heads per KV head", kvs::kDecodeMaxGroup);
  if (p->head_dim != 64 && p->head_dim != 128) return fail(KVSCORE_EINVAL, "head_dim must be 64 or 128");
  if (!std::isfinite(p->softmax_scale))
    return fail(KVSCORE_EINVAL, "softmax_scale must be finite (<= 0 selects 1/sqrt(head_dim))");
  if (!off) return fail(KVSCORE_EINVAL, "host segment offsets are NULL");
  const int64_t U = (int64_t)p->num_layers * p->num_seqs * p->num_kv_heads;
  if (U > kvs::kMaxUnits) return fail(KVSCORE_EINVAL, "too many segments (%lld > %d)", (long long)U, kvs::kMaxUnits);
  if (off[0] != 0) return fail(KVSCORE_EINVAL, "segment offsets must start at 0");
  int64_t max_len = 0;
  for (int64_t u = 0; u < U; ++u) {
    const int64_t len = off[u + 1] - off[u];
    if (len < 1) return fail(KVSCORE_EINVAL, "segment %lld is empty or offsets decrease", (long long)u);
    max_len = std::max(max_len, len);
  }
  d = kvs::DecDev{};
  d.Hq = p->num_q_heads;
  d.Hkv = p->num_kv_heads;
  d.G = G;
  d.d = p->head_dim;
  d.U = (int)U;
  const float scale = p->softmax_scale > 0.f ? p->softmax_scale : 1.0f / std::sqrt((float)p->head_dim);
  d.c1 = (float)((double)scale * 1.4426950408889634);
  // Splits of one length for every segment: about 2048 of them in all (8 workgroups per
  // CU), at least 256 keys each, so the longest segments of a ragged batch do not hold the
  // launch while the short ones idle; at most kDecodeMaxSplits splits of the longest segment
  // (the workspace holds that many records per segment). Workgroups past a segment's last
  // split return at once.
  constexpr int64_t kDecodeMaxSplits = 64;
  int64_t chunk = std::max<int64_t>(256, (off[U] + 2047) / 2048);
  chunk = std::max<int64_t>(chunk, (max_len + kDecodeMaxSplits - 1) / kDecodeMaxSplits);
  chunk = (chunk + 63) / 64 * 64;
  if (chunk > (int64_t)1 << 30) return fail(KVSCORE_EINVAL, "segment too long");
  d.chunk = (int)chunk;
  d.nsplit = (int)((max_len + chunk - 1) / chunk);
  return ok();
}

// Arguments of the selection entry points (both share them).
int check_topk(const kvscore_problem* p, kvs::Dev& d, const float* score, const int32_t* budgets,
               const int64_t* seg_offsets, const int32_t* kept_pos, int32_t pool, int32_t n_sink, void* workspace,
               size_t workspace_bytes) {
  if (int rc = make_dev(p, d)) return rc;
  if (!score || !seg_offsets || !kept_pos) return fail(KVSCORE_EINVAL, "NULL tensor argument");
  if (pool < 1 || pool > kvs::kMaxPoolSize || pool % 2 == 0)
    return fail(KVSCORE_EINVAL, "pool=%d must be odd, in [1, %d]", pool, kvs::kMaxPoolSize);
  if (n_sink < 0) return fail(KVSCORE_EINVAL, "n_sink=%d < 0", n_sink);
  if (int rc = check_budgets(p, budgets, nullptr)) return rc;
  for (int s = 0; s < p->num_seqs; ++s) {
    const int64_t cand = p->cu_seqlens[s + 1] - p->cu_seqlens[s] - p->window;
    const int64_t ns = std::min<int64_t>(n_sink, cand);
    for (int l = 0; l < p->num_layers; ++l) {
      const int32_t b = budgets[(int64_t)s * p->num_layers + l];
      if (b < p->window + ns)
        return fail(KVSCORE_EBUDGET, "budget[%d][%d]=%d below window + sinks (%d + %lld)", s, l, b, p->window,
                    (long long)ns);
    }
  }
  return ok();
}

size_t ws_decode(const kvs::DecDev& d) { return (size_t)d.U * d.nsplit * d.G * (d.d + 2) * sizeof(float); }

}  // namespace

extern "C" {

int32_t kvscore_version(void) { return 102; }

const char* kvscore_last_error(void) { return g_err.c_str(); }

int32_t kvscore_num_query_tiles(const kvscore_problem* p) {
  kvs::Dev d;
  if (make_dev(p, d)) return 0;
  return d.Tq;
}

size_t kvscore_workspace_size(const kvscore_problem* p, int32_t which) {
  kvs::Dev d;
  if (make_dev(p, d)) return 0;
  switch (which) {
    case KVSCORE_WS_ATTN_FWD:
      return ws_attn(d);
    case KVSCORE_WS_SCORE:
      return ws_score(d);
    case KVSCORE_WS_TOPK:
      return ws_topk(d);
    case KVSCORE_WS_TOPK_HEADS:
      return kvs::heads_ws_bytes(d) + ws_topk(d);
    default:
      fail(KVSCORE_EINVAL, "unknown workspace kind %d", which);
      return 0;
  }
}

int kvscore_attn_fwd(const kvscore_problem* p, const void* q_win, const void* k, const void* v, float* a, float* lse,
                     int32_t* jstar, float* dom, void* workspace, size_t workspace_bytes, void* stream) {
  kvs::Dev d;
  if (int rc = make_dev(p, d)) return rc;
  if (!q_win || !k || !v || !a || !lse || !jstar || !dom) return fail(KVSCORE_EINVAL, "NULL tensor argument");
  if (!aligned(q_win, 16) || !aligned(k, 16) || !aligned(v, 16)) return fail(KVSCORE_EINVAL, "q/k/v not 16-byte aligned");
  if (!aligned(a, 4) || !aligned(lse, 4) || !aligned(jstar, 4) || !aligned(dom, 4))
    return fail(KVSCORE_EINVAL, "outputs not 4-byte aligned");
  if (int rc = check_ws(workspace, workspace_bytes, ws_attn(d))) return rc;
  return launched(kvs::launch_attn_fwd(d, q_win, k, v, a, lse, jstar, dom, workspace, (hipStream_t)stream),
                  "kvscore_attn_fwd");
}

int kvscore_score(const kvscore_problem* p, const void* q_win, const void* k, const void* v, const float* a,
                  const float* lse, const int32_t* jstar, float* partial, void* workspace, size_t workspace_bytes,
                  void* stream) {
  kvs::Dev d;
  if (int rc = make_dev(p, d)) return rc;
  if (!q_win || !k || !v || !a || !lse || !jstar || !partial) return fail(KVSCORE_EINVAL, "NULL tensor argument");
  if (!aligned(q_win, 16) || !aligned(k, 16) || !aligned(v, 16)) return fail(KVSCORE_EINVAL, "q/k/v not 16-byte aligned");
  if (!aligned(a, 4) || !aligned(lse, 4) || !aligned(jstar, 4) || !aligned(partial, 4))
    return fail(KVSCORE_EINVAL, "buffers not 4-byte aligned");
  if (int rc = check_ws(workspace, workspace_bytes, ws_score(d))) return rc;
  return launched(kvs::launch_score(d, q_win, k, v, a, lse, jstar, partial, workspace, (hipStream_t)stream),
                  "kvscore_score");
}

int kvscore_merge(const kvscore_problem* p, const float* partial, const int32_t* jstar, const float* dom, float* score,
                  void* stream) {
  kvs::Dev d;
  if (int rc = make_dev(p, d)) return rc;
  if (!partial || !jstar || !dom || !score) return fail(KVSCORE_EINVAL, "NULL tensor argument");
  if (partial == score && d.Tq != 1)
    return fail(KVSCORE_EINVAL, "partial and score may be one buffer only with one query tile (Tq = %d)", d.Tq);
  return launched(kvs::launch_merge(d, partial, jstar, dom, score, (hipStream_t)stream), "kvscore_merge");
}

int kvscore_budget(const double* sens, int32_t num_layers, double ratio, double gamma, int64_t total, int32_t lo,
                   int32_t hi, int32_t* budgets_out) {
  if (!sens || !budgets_out) return fail(KVSCORE_EINVAL, "NULL argument");
  if (num_layers < 1) return fail(KVSCORE_EINVAL, "num_layers=%d < 1", num_layers);
  if (!(ratio >= 1.0) || !std::isfinite(ratio)) return fail(KVSCORE_EINVAL, "ratio must be finite and >= 1");
  if (std::isnan(gamma) || (gamma > 0 && gamma < 1.0)) return fail(KVSCORE_EINVAL, "gamma must be >= 1 (or <= 0 / inf)");
  if (lo < 0 || hi < lo) return fail(KVSCORE_EINVAL, "need 0 <= lo <= hi");
  const int L = num_layers;
  if (total < (int64_t)L * lo || total > (int64_t)L * hi)
    return fail(KVSCORE_EBUDGET, "total %lld outside [L*lo, L*hi] = [%lld, %lld]", (long long)total, (long long)L * lo,
                (long long)L * hi);
  for (int l = 0; l < L; ++l)
    if (!std::isfinite(sens[l])) return fail(KVSCORE_EINVAL, "sensitivity %d not finite", l);

  // Eq. 9: min-max normalisation, a constant profile gives s_hat = 0.
  double smin = sens[0], smax = sens[0];
  for (int l = 1; l < L; ++l) {
    smin = std::min(smin, sens[l]);
    smax = std::max(smax, sens[l]);
  }
  std::vector<double> w(L);
  const double lr = std::log(ratio);
  for (int l = 0; l < L; ++l) {
    const double shat = (smax == smin) ? 0.0 : (sens[l] - smin) / (smax - smin);
    w[l] = std::exp(lr * shat);  // Eq. 10
  }
  // Eq. 11: clip to [1/gamma, gamma], rescale to mean one.
  if (gamma > 0 && std::isfinite(gamma))
    for (int l = 0; l < L; ++l) w[l] = std::min(std::max(w[l], 1.0 / gamma), gamma);
  // Eq. 11's mean-one rescale and Eq. 12's B/|A| go into lam: x_l = clip(lam * w_l, lo, hi)
  // with sum x_l = total (lam = total / sum w when no clip is active), rounded exactly
  if (kvs::exact_budgets_f64(w, 0, total, lo, hi, budgets_out))
    return fail(KVSCORE_EBUDGET, "could not distribute the total");
  return ok();
}

int kvscore_budget_pyramid(int32_t num_layers, double gamma, int64_t total, int32_t lo, int32_t hi,
                           int32_t* budgets_out) {
  if (!budgets_out) return fail(KVSCORE_EINVAL, "NULL argument");
  if (num_layers < 1) return fail(KVSCORE_EINVAL, "num_layers=%d < 1", num_layers);
  if (!(gamma >= 0.0) || !std::isfinite(gamma)) return fail(KVSCORE_EINVAL, "gamma must be finite and >= 0");
  if (lo < 0 || hi < lo) return fail(KVSCORE_EINVAL, "need 0 <= lo <= hi");
  const int L = num_layers;
  // PyramidKV curve, 0-based: f_l = (1 - l/(L-1))^gamma (the lowest layer 1, the top 0);
  // for an integer gamma (up to 4096) the curve is rational and is taken exactly, as the
  // integers (L-1-l)^gamma, whose common denominator goes into lam
  std::vector<double> f(L, 1.0);
  if (L > 1)
    for (int l = 0; l < L; ++l) f[l] = std::pow(1.0 - (double)l / (L - 1), gamma);
  int64_t reach = 0;
  for (int l = 0; l < L; ++l) reach += f[l] > 0 ? hi : lo;
  if (total < (int64_t)L * lo || total > reach)
    return fail(KVSCORE_EBUDGET, "total %lld outside [L*lo, %lld] (layers with factor 0 stay at lo)",
                (long long)total, (long long)reach);
  // x_l = clip(lo + lam * f_l, lo, hi) with sum = total
  const bool integral = gamma == std::floor(gamma) && gamma <= 4096.0;
  const int rc = integral ? kvs::exact_budgets_pow(L, (uint64_t)gamma, total, lo, hi, budgets_out)
                          : kvs::exact_budgets_f64(f, lo, total, lo, hi, budgets_out);
  if (rc) return fail(KVSCORE_EBUDGET, "could not distribute the total");
  return ok();
}

int kvscore_segment_offsets(const kvscore_problem* p, const int32_t* budgets, int64_t* offsets_out) {
  kvs::Dev d;
  if (int rc = make_dev(p, d)) return rc;
  if (!offsets_out) return fail(KVSCORE_EINVAL, "offsets_out is NULL");
  if (int rc = check_budgets(p, budgets, nullptr)) return rc;
  int64_t acc = 0;
  for (int u = 0; u < d.U; ++u) {
    int l, s, g;
    kvs::unit_coords(d, u, l, s, g);
    offsets_out[u] = acc;
    acc += budgets[(int64_t)s * d.L + l];
  }
  offsets_out[d.U] = acc;
  return ok();
}

int kvscore_topk(const kvscore_problem* p, const float* score, const int32_t* budgets, const int64_t* seg_offsets,
                 int32_t* kept_pos, int32_t pool, int32_t n_sink, void* workspace, size_t workspace_bytes,
                 void* stream) {
  kvs::Dev d;
  if (int rc = check_topk(p, d, score, budgets, seg_offsets, kept_pos, pool, n_sink, workspace, workspace_bytes))
    return rc;
  if (pool > 1) {
    if (int rc = check_ws(workspace, workspace_bytes, ws_topk(d))) return rc;
  }
  return launched(kvs::launch_topk(d, score, seg_offsets, kept_pos, pool, n_sink, (float*)workspace, nullptr, nullptr,
                                   nullptr, (hipStream_t)stream),
                  "kvscore_topk");
}

int kvscore_topk_heads(const kvscore_problem* p, const float* score, const int32_t* budgets,
                       const int64_t* seg_offsets, int64_t* head_offsets, int32_t* kept_pos, int32_t pool,
                       int32_t n_sink, void* workspace, size_t workspace_bytes, void* stream) {
  kvs::Dev d;
  if (int rc = check_topk(p, d, score, budgets, seg_offsets, kept_pos, pool, n_sink, workspace, workspace_bytes))
    return rc;
  if (!head_offsets) return fail(KVSCORE_EINVAL, "head_offsets is NULL");
  // scratch of the joint select first, the pooled keys (pool > 1) after it
  const size_t hb = kvs::heads_ws_bytes(d);
  if (int rc = check_ws(workspace, workspace_bytes, hb + (pool > 1 ? ws_topk(d) : 0))) return rc;
  return launched(kvs::launch_topk(d, score, seg_offsets, kept_pos, pool, n_sink, (float*)((char*)workspace + hb),
                                   head_offsets, workspace, budgets, (hipStream_t)stream),
                  "kvscore_topk_heads");
}

int kvscore_compact(const kvscore_problem* p, const void* k, const void* v, const int32_t* budgets,
                    const int64_t* seg_offsets, const int32_t* kept_pos, void* k_out, void* v_out, void* stream) {
  kvs::Dev d;
  if (int rc = make_dev(p, d)) return rc;
  if (!k || !v || !seg_offsets || !kept_pos || !k_out || !v_out) return fail(KVSCORE_EINVAL, "NULL tensor argument");
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_out, 16) || !aligned(v_out, 16))
    return fail(KVSCORE_EINVAL, "k/v/k_out/v_out not 16-byte aligned");
  int max_b = 0;
  if (int rc = check_budgets(p, budgets, &max_b)) return rc;
  return launched(kvs::launch_compact(d, k, v, seg_offsets, kept_pos, k_out, v_out, max_b, (hipStream_t)stream),
                  "kvscore_compact");
}

int kvscore_compact_heads(const kvscore_problem* p, const void* k, const void* v, const int32_t* budgets,
                          const int64_t* head_offsets, const int32_t* kept_pos, void* k_out, void* v_out,
                          void* stream) {
  kvs::Dev d;
  if (int rc = make_dev(p, d)) return rc;
  if (!k || !v || !head_offsets || !kept_pos || !k_out || !v_out) return fail(KVSCORE_EINVAL, "NULL tensor argument");
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_out, 16) || !aligned(v_out, 16))
    return fail(KVSCORE_EINVAL, "k/v/k_out/v_out not 16-byte aligned");
  if (int rc = check_budgets(p, budgets, nullptr)) return rc;
  // a head may take up to the layer's whole budget, never more than its sequence
  int64_t max_seg = 0;
  for (int s = 0; s < p->num_seqs; ++s) {
    const int64_t n = p->cu_seqlens[s + 1] - p->cu_seqlens[s];
    for (int l = 0; l < p->num_layers; ++l)
      max_seg = std::max(max_seg, std::min<int64_t>(n, (int64_t)p->num_kv_heads * budgets[(int64_t)s * p->num_layers + l]));
  }
  return launched(kvs::launch_compact(d, k, v, head_offsets, kept_pos, k_out, v_out, (int)max_seg, (hipStream_t)stream),
                  "kvscore_compact_heads");
}

size_t kvscore_decode_workspace_size(const kvscore_problem* p, const int64_t* seg_offsets_host) {
  kvs::DecDev d;
  if (make_decdev(p, seg_offsets_host, d)) return 0;
  return ws_decode(d);
}

int kvscore_decode_attn_noalloc(const kvscore_problem* p, const void* q, const void* k_cache, const void* v_cache,
                                const int64_t* seg_offsets_host, const int64_t* seg_offsets, float* out, float* lse,
                                void* stream) {
  static_assert(kvs::kDecodeScratchBytes == KVSCORE_DECODE_SCRATCH_BYTES, "header and library agree");
  kvs::DecDev d;
  if (int rc = make_decdev(p, seg_offsets_host, d)) return rc;
  if (!q || !k_cache || !v_cache || !seg_offsets || !out || !lse) return fail(KVSCORE_EINVAL, "NULL tensor argument");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(KVSCORE_EINVAL, "q/k_cache/v_cache not 16-byte aligned");
  if (!aligned(out, 4) || !aligned(lse, 4)) return fail(KVSCORE_EINVAL, "out/lse not 4-byte aligned");
  const size_t need = ws_decode(d);
  if (need > kvs::kDecodeScratchBytes)
    return fail(KVSCORE_EWORKSPACE,
                "decode needs %zu bytes of scratch for these segments; the fixed array holds %zu "
                "(use kvscore_decode_attn with a workspace)",
                need, kvs::kDecodeScratchBytes);
  void* ws = nullptr;
  if (hipError_t e = kvs::decode_scratch(&ws)) return fail(KVSCORE_EDEVICE, "decode scratch: %s", hipGetErrorString(e));
  return launched(kvs::launch_decode(d, q, k_cache, v_cache, seg_offsets, out, lse, ws, (hipStream_t)stream),
                  "kvscore_decode_attn_noalloc");
}

int kvscore_decode_attn(const kvscore_problem* p, const void* q, const void* k_cache, const void* v_cache,
                        const int64_t* seg_offsets_host, const int64_t* seg_offsets, float* out, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream) {
  kvs::DecDev d;
  if (int rc = make_decdev(p, seg_offsets_host, d)) return rc;
  if (!q || !k_cache || !v_cache || !seg_offsets || !out || !lse) return fail(KVSCORE_EINVAL, "NULL tensor argument");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(KVSCORE_EINVAL, "q/k_cache/v_cache not 16-byte aligned");
  if (!aligned(out, 4) || !aligned(lse, 4)) return fail(KVSCORE_EINVAL, "out/lse not 4-byte aligned");
  if (int rc = check_ws(workspace, workspace_bytes, ws_decode(d))) return rc;
  return launched(kvs::launch_decode(d, q, k_cache, v_cache, seg_offsets, out, lse, workspace, (hipStream_t)stream),
                  "kvscore_decode_attn");
}

}  // extern "C"
