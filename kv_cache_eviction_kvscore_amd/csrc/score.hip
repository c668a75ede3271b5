// Score pass: per-token output-perturbation score partials for one query tile.
//
// DropKV page, Key Contribution 1 (the score of token j is sum_i p_ij/(1-p_ij) *
// ||a_i - v_j||_2, summed here over the window rows and the query heads of the KV
// group) and "Methodology in Plain English" (the fused scorer's design). Here: p_ij
// comes from q_i.k_j and the forward's lse_i, the distance from the expansion of
// ||a_i - v_j||^2 into norms and a dot product, and every K and V tile is streamed
// once per pass; no (row, token) matrix is ever stored. Mode ATTN scores sum_i p_ij
// instead (PyramidKV page, "Observation Window and Aggregated Attention Eviction").
//
// score_prep: a_hat = fp16(a) (the MFMA operand), ||a_hat||^2 from the rounded values
//   (so the expansion is the exact ||a_hat - v||^2 up to fp32 rounding), lse*log2(e).
//   fp16, not bf16: the distance's error from rounding a is 2 (a - a_hat).(a - v), and
//   fp16's 11-bit significand makes it eight times smaller; with bf16 a pair whose term
//   dominates a token's score could miss a 1e-3 relative bound.
// score_kernel: grid (key chunk, query tile, unit); 8 waves of 32 rows, two per SIMD, so
//   one wave's VALU work overlaps the other's MFMAs. Orientation S = Q.K^T on
//   v_mfma_f32_32x32x16_bf16 and X = A_hat.V^T (rows x keys) on v_mfma_f32_32x32x16_f16,
//   with the row operands held in AGPRs and the accumulators written to VGPRs. K/V tiles
//   of 64 keys go from HBM straight into LDS (global_load_lds_dwordx4, no register
//   staging) through a ring of four buffers, so two tiles are in flight while one is
//   computed. A tile keeps whole key rows (each DMA instruction moves four or eight full
//   rows); the 16-byte chunks of row r are XOR-swizzled with a function of r so that the
//   32 keys x 16 slots an MFMA operand needs are read conflict-free with ds_read_b128. A
//   lane owns one key column and 16 rows of the 32x32 block, so the sum over rows stays in
//   the lane (plus one half-wave exchange); the waves' column sums are added in LDS in
//   wave order.
//   The expansion runs on the matrix cores: one extra bf16 k-step multiplies
//   (1, 1, 1, -||a_hat_i||^2/2 in three parts) by (-||v_j||^2/2 in three parts, 1, 1, 1)
//   into the same accumulator; every part is an exact bf16 split, so X is -D/2 with
//   D = ||a_hat - v||^2. ||v_j||^2 is summed from the tile in LDS (v_dot2_f32_bf16) one
//   tile ahead of its use, and the same pass converts the tile's V to fp16 in place (exact
//   in fp16's normal range) for the A_hat.V^T product. The Q.K^T chain gets an augmented
//   k-step too: (-lse_i/scale in three bf16 parts) times (1, 1, 1), so its accumulator is
//   ln p / scale and needs no per-row register. Per pair: 1/p = exp2(-acc * scale *
//   log2 e), and c*sqrt(D) = sqrt(2) * sqrt(D/2) / (1/p - 1): three transcendentals and
//   three other VALU instructions; the sqrt(2) (2 in mode SQ) is applied once per token.
//   Pairs (i, j*_i) are skipped (their term comes exactly from the forward); so are keys
//   after a row's position. Both masks only act on tiles flagged in LDS, others run
//   unmasked.
//   Every pair that is not masked has p <= 1/2 (the row's argmax is isolated), so
//   1/p - 1 >= 1 needs no guard, and p = 0 gives a zero term.
#include <type_traits>

#include "kvs_internal.hpp"

namespace kvs {
namespace {

constexpr int KT = 64;   // keys per LDS tile
constexpr int KB = 32;   // keys per MFMA block
constexpr int NBUF = 4;  // tile ring: computed, next (its ||v||^2 summed), two in flight
constexpr int NWAVES = 8;                // 32 rows each: one query tile of up to 256 rows
constexpr int NTHREADS = 64 * NWAVES;
static_assert(NWAVES * 32 == kRowsPerTileMax, "a workgroup covers one query tile");
constexpr int kMaxTilesPerChunk = 1024;  // score_chunk <= 65536

template <int D>
struct ScoreSmem {
  // tile ring: [buffer][tensor K, V][key][D] with row r's 16-byte chunks XOR-swizzled
  alignas(16) __bf16 tile[NBUF][2][KT * D];
  alignas(16) __bf16 nvx[2][KT][8];  // (-||v||^2/2 as hi, mid, lo bf16 parts, 1, 1, 1, 0, 0)
  float red[3][NWAVES][KT];
  int tlim[kRowsPerTileMax];
  int jst[kRowsPerTileMax];
  unsigned char flag[kMaxTilesPerChunk];
};

// chunk position of chunk c of key row r is c ^ swz(r): sixteen consecutive rows read at
// one chunk index land on sixteen different 16-byte bank groups (also eight consecutive
// rows within 128 bytes), and swz(r + 32) = swz(r)
template <int D>
__device__ inline int swz(int r) {
  if constexpr (D == 128) return r & 15;
  else return (r & 7) ^ ((r >> 3) & 1);
}

struct BlockAcc {
  f32x16 S, X;
};

// x as three bf16 parts (hi, mid, lo) whose sum is x to about 24 bits
struct Split3 {
  __bf16 hi, mid, lo;
};
__device__ inline Split3 split3(float x) {
  Split3 r;
  r.hi = (__bf16)x;
  const float r1 = x - (float)r.hi;
  r.mid = (__bf16)r1;
  r.lo = (__bf16)(r1 - (float)r.mid);
  return r;
}

template <int D>
__global__ __launch_bounds__(256) void score_prep_kernel(int64_t rows, const float* __restrict__ a,
                                                         const float* __restrict__ lse, _Float16* __restrict__ ahat,
                                                         float* __restrict__ na, float* __restrict__ lse2) {
  constexpr int PER = D / 64;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    const _Float16 b = (_Float16)a[row * D + e];  // round to nearest
    ahat[row * D + e] = b;
    const float f = (float)b;
    s += f * f;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) {
    na[row] = s;
    lse2[row] = lse[row] * 1.4426950408889634f;
  }
}

template <int D, int MODE>
__global__ __launch_bounds__(NTHREADS) void score_kernel(Dev p, const __bf16* __restrict__ q,
                                                         const __bf16* __restrict__ k,
                                                         const __bf16* __restrict__ v,
                                                         const _Float16* __restrict__ ahat,
                                                         const float* __restrict__ na,
                                                         const float* __restrict__ lse2,
                                                         const int32_t* __restrict__ jstar,
                                                         float* __restrict__ partial) {
  constexpr int NKK = D / 16;             // k-steps per row operand
  constexpr int RS = D * 2;               // bytes per key row
  constexpr int CPK = D / 8;              // 16-byte chunks per key row
  constexpr int TB = KT * RS;             // bytes per tensor tile
  constexpr bool WITH_V = MODE != 2;      // the attention-sum mode reads no V, a or norms
  constexpr int IPT = KT * CPK / 64;      // DMA wave instructions per tensor tile
  constexpr int NLD = (WITH_V ? 2 : 1) * IPT / NWAVES;  // DMA instructions per wave per tile
  constexpr int PPR = 4;                  // pairs per lockstep group of the VALU work
  constexpr int KPW = KT / NWAVES;        // keys per wave in the norm pass and the column sums
  constexpr int LPK = 64 / KPW;           // lanes per key in the norm pass
  constexpr int CPN = CPK / LPK;          // 16-byte chunks per lane in the norm pass
  static_assert(IPT % NWAVES == 0 && NLD >= 1 && NLD <= 4 && (NLD & (NLD - 1)) == 0, "tile shape");
  static_assert(KT % NWAVES == 0 && 64 % KPW == 0 && CPK % LPK == 0 && CPN >= 1, "norm pass shape");
  __shared__ ScoreSmem<D> sm;

  const int u = blockIdx.z, qt = blockIdx.y, ch = blockIdx.x;
  int l, s, g;
  unit_coords(p, u, l, s, g);
  const int64_t n = p.cu[s + 1] - p.cu[s];
  const int64_t c0 = (int64_t)ch * p.score_chunk;
  if (c0 >= n) return;
  const int64_t c1 = (n < c0 + p.score_chunk) ? n : c0 + p.score_chunk;
  const int ntiles = (int)((c1 - c0 + KT - 1) / KT);

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const int wrow0 = wave * 32;  // first tile row of this wave
  const bool computing = wrow0 < p.RT;
  const int64_t rbase = (int64_t)u * p.R + (int64_t)qt * p.RT;  // first row of this tile (global row index)
  const int rows_here = min(p.RT, p.R - qt * p.RT);

  // fields the lambdas below use, as locals: a by-reference capture of the by-value
  // argument would be re-read from kernel-argument memory with vector loads
  const int64_t kst = p.kst, vst = p.vst;
  const float c1s = p.c1, nc1s = -p.c1;
  const int W = p.W;
  const __bf16* kb0 = k + l * p.ksl + g * p.ksh + p.cu[s] * p.kst;
  const __bf16* vb0 = v + l * p.vsl + g * p.vsh + p.cu[s] * p.vst;
  float* pout = partial + ((int64_t)(l * p.Hkv + g) * p.Tq + qt) * p.N + p.cu[s];

  // DMA of tile it into ring buffer it % NBUF. Wave instruction f (of NLD * NWAVES) fills
  // the 64 chunk slots 64(f % IPT) .. +63 of tensor f / IPT: slot (row r, position c')
  // takes chunk c' ^ swz(r) of key row r. Keys past the chunk load its last row (in
  // bounds, unconditional); their columns are masked and never written.
  constexpr int TBYTES = KT * D * 2;  // bytes per tensor tile
  const unsigned smb = lds_offset(&sm.tile[0][0][0]);
  auto issue = [&](int it) __attribute__((always_inline)) {
    const int64_t t0 = c0 + (int64_t)it * KT;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int f = i * NWAVES + wave;
      const int tensor = f / IPT, slot = (f % IPT) * 64 + lane;
      const int r = slot / CPK, c = (slot % CPK) ^ swz<D>(r);
      const int rr = (t0 + r < c1) ? r : (int)(c1 - 1 - t0);  // rows past the chunk load its last
      const __bf16* base = tensor == 0 ? kb0 + t0 * kst : vb0 + t0 * vst;
      lds_dma16(base, (unsigned)(rr * (int)(tensor == 0 ? kst : vst) + 8 * c) * 2u,
                smb + (unsigned)(((it % NBUF) * 2 + tensor) * TBYTES + (f % IPT) * 1024));
    }
  };
  // the same for a full tile, from lane byte offsets (from the tile's first row) computed once
  unsigned doff[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int f = i * NWAVES + wave;
    const int tensor = f / IPT, slot = (f % IPT) * 64 + lane;
    const int r = slot / CPK, c = (slot % CPK) ^ swz<D>(r);
    doff[i] = (unsigned)(r * (int)(tensor == 0 ? kst : vst) + 8 * c) * 2u;
  }
  auto issue_full = [&](int it) __attribute__((always_inline)) {
    const int64_t t0 = c0 + (int64_t)it * KT;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int f = i * NWAVES + wave;
      const int tensor = f / IPT;
      const __bf16* base = tensor == 0 ? kb0 + t0 * kst : vb0 + t0 * vst;
      lds_dma16(base, doff[i], smb + (unsigned)(((it % NBUF) * 2 + tensor) * TBYTES + (f % IPT) * 1024));
    }
  };
  // -||v||^2/2 of tile it (landed, visible), into nvx[it & 1]: wave w sums keys
  // KPW*w .. KPW*w+KPW-1, LPK lanes per key (lanes key%KPW + KPW*c), CPN chunks each.
  auto norms = [&](int it) __attribute__((always_inline)) {
    if constexpr (!WITH_V) return;
    char* vt = (char*)sm.tile[it % NBUF][1];
    const int key = KPW * wave + (lane % KPW), cg = lane / KPW;
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < CPN; ++e) {
      const int c = CPN * cg + e;
      u32x4* cp = (u32x4*)(vt + key * RS + ((c ^ swz<D>(key)) << 4));
      const u32x4 w = *cp;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        // copy the element out first: a bit_cast of a vector-element lvalue reads element 0
        const unsigned wm = w[m];
        const bf16x2 x = __builtin_bit_cast(bf16x2, wm);
        ss = __builtin_amdgcn_fdot2_f32_bf16(x, x, ss, false);
      }
      *cp = bf16x8_to_f16x8(w);  // the A_hat.V^T product reads the tile in fp16
    }
    // a shuffle here, not a VALU exchange chain: this side work is off the MFMA path, and
    // the dependent DPP / permlane steps measured slower than LDS shuffles in flight
#pragma unroll
    for (int off = KPW; off < 64; off <<= 1) ss += __shfl_xor(ss, off, 64);
    const Split3 sp = split3(-0.5f * ss);
    bf16x8 w8 = {};
    w8[0] = sp.hi;
    w8[1] = sp.mid;
    w8[2] = sp.lo;
    w8[3] = (__bf16)1.f;
    w8[4] = (__bf16)1.f;
    w8[5] = (__bf16)1.f;
    *(bf16x8*)&sm.nvx[it & 1][key][0] = w8;  // the key's lanes store the same entry
  };

  // ---- per-row masks in LDS, tile flags for rows whose argmax falls in this chunk
  for (int t = tid; t < ntiles; t += NTHREADS) sm.flag[t] = 0;
  for (int t = tid; t < 3 * NWAVES * KT; t += NTHREADS) (&sm.red[0][0][0])[t] = 0.f;  // waves that never compute add zeros
  for (int t = tid; t < kRowsPerTileMax; t += NTHREADS) {
    const bool ok = t < rows_here;
    sm.tlim[t] = ok ? (int)(n - W + (qt * p.RT + t) % W) : -1;
    sm.jst[t] = ok ? jstar[rbase + t] : -1;
  }
  issue(0);
  __syncthreads();
  for (int t = tid; t < rows_here; t += NTHREADS) {
    const int js = sm.jst[t];
    if (js >= c0 && js < c1) sm.flag[(js - c0) / KT] = 1;
  }

  // ---- row operands (A side): lane row l32 of the wave's 32, k-slots 8h..8h+7
  bf16x8 qf[NKK], aug, augs;
  f16x8 af[NKK];
  {
    const int rt = wrow0 + l32;
    const bool ok = computing && rt < rows_here;
    const __bf16* qrow = q + (rbase + (ok ? rt : 0)) * D;
    const _Float16* arow = ahat + (rbase + (ok ? rt : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      bf16x8 z = {};
      f16x8 zh = {};
      qf[kk] = ok ? *(const bf16x8*)(qrow + 16 * kk + 8 * h) : z;
      af[kk] = (ok && WITH_V) ? *(const f16x8*)(arow + 16 * kk + 8 * h) : zh;
    }
    // augmented k-step of the A.V^T chain: (1, 1, 1, -||a_hat||^2/2 in three parts) in slots 0..5
    bf16x8 w8 = {};
    // and of the Q.K^T chain: -lse_i/scale in three parts (slots 0..2), so the accumulator
    // is the log-probability / scale; padding rows get -1e30 (p = 0)
    bf16x8 s8 = {};
    if (h == 0) {
      w8[0] = (__bf16)1.f;
      w8[1] = (__bf16)1.f;
      w8[2] = (__bf16)1.f;
      if (ok && WITH_V) {
        const Split3 sp = split3(-0.5f * na[rbase + rt]);
        w8[3] = sp.hi;
        w8[4] = sp.mid;
        w8[5] = sp.lo;
      }
      const Split3 sp = split3(ok ? -lse2[rbase + rt] / c1s : -1e30f);
      s8[0] = sp.hi;
      s8[1] = sp.mid;
      s8[2] = sp.lo;
    }
    aug = w8;
    augs = s8;
  }
  // B side of the Q.K^T k-step: 1 in slots 0..2 for every key
  bf16x8 ones3 = {};
  if (h == 0) {
    ones3[0] = (__bf16)1.f;
    ones3[1] = (__bf16)1.f;
    ones3[2] = (__bf16)1.f;
  }
  // the row operands live in AGPRs (MFMA reads them there), which leaves the VGPRs to
  // the accumulators the VALU consumes
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    asm volatile("" : "+a"(qf[kk]));
    if constexpr (WITH_V) asm volatile("" : "+a"(af[kk]));
  }
  if constexpr (WITH_V) asm volatile("" : "+a"(aug));
  asm volatile("" : "+a"(augs));
  // sqrt(2) turns sqrt(D/2) into sqrt(D); mode SQ's p^2 (D/2)/(1-p)^2 needs 2; p needs 1
  const float out_scale = (MODE == 0) ? 1.41421356237309515f : (MODE == 1 ? 2.f : 1.f);
  // byte offset, within a tensor tile, of this lane's operand chunk (key l32, slots
  // 16kk + 8h .. +7) for k-step kk; block b adds 32 rows
  const int kbase = l32 * RS, khs = h ^ swz<D>(l32);
  auto koff = [&](int kk) __attribute__((always_inline)) { return kbase + (((2 * kk) ^ khs) << 4); };

  // adds the terms of pairs pi0 .. pi0+PPR-1 (pair = row of the output layout: element r
  // is row 8(r/4) + 4h + (r%4)) to col, written stage by stage so the PPR independent
  // chains interleave
  auto pair_terms = [&](auto masked, const BlockAcc& acc, const int pi0, const int key, float& col)
      __attribute__((always_inline)) {
    float x[PPR], y[PPR];  // the pair's term is x * y
    if constexpr (MODE == 2) {
#pragma unroll
      for (int i = 0; i < PPR; ++i) {
        x[i] = __builtin_amdgcn_exp2f(acc.S[pi0 + i] * c1s);  // p itself
        y[i] = 1.f;
      }
    } else {
      // e = 1/p and r = 1/(e - 1) = p/(1-p): e >= 2 on every unmasked pair, so r is finite
      // (0 when p underflows); a masked pair's value is never added
      float e[PPR], r[PPR];
#pragma unroll
      for (int i = 0; i < PPR; ++i) e[i] = __builtin_amdgcn_exp2f(acc.S[pi0 + i] * nc1s);
#pragma unroll
      for (int i = 0; i < PPR; ++i) r[i] = __builtin_amdgcn_rcpf(e[i] - 1.f);
      if constexpr (MODE == 0) {
        // p/(1-p) sqrt(D/2): three transcendentals and three other VALU instructions. The
        // matrix cores leave room for about four VALU instructions of any kind per MFMA,
        // so this beats a form with one transcendental less and three more plain ones.
#pragma unroll
        for (int i = 0; i < PPR; ++i) {
          x[i] = r[i];
          y[i] = __builtin_amdgcn_sqrtf(fabsf(acc.X[pi0 + i]));
        }
      } else {
        // p^2 (D/2) / (1-p)^2
#pragma unroll
        for (int i = 0; i < PPR; ++i) {
          x[i] = r[i] * r[i];
          y[i] = fabsf(acc.X[pi0 + i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < PPR; ++i) {
      if constexpr (decltype(masked)::value) {
        const int rr = pi0 + i;
        const int rt = wrow0 + 8 * (rr >> 2) + 4 * h + (rr & 3);
        col += (key > sm.tlim[rt] || key == sm.jst[rt]) ? 0.f : x[i] * y[i];
      } else if constexpr (MODE == 2) {
        col += x[i];
      } else {
        col = fmaf(x[i], y[i], col);
      }
    }
  };
  // the MFMAs of 32-key block b of ring tile it: S = ln p / scale, X = -D/2
  auto mfma_block = [&](int it, int b) __attribute__((always_inline)) {
    const char* kt = (const char*)sm.tile[it % NBUF][0] + b * KB * RS;
    BlockAcc acc;
    bf16x8 nv = {};
    if constexpr (WITH_V) nv = *(const bf16x8*)&sm.nvx[it & 1][b * KB + l32][0];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const bf16x8 kx = *(const bf16x8*)(kt + koff(kk));
      acc.S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[kk], kx, kk ? acc.S : f32x16{}, 0, 0, 0);
      if constexpr (WITH_V) {
        const f16x8 vx = *(const f16x8*)(kt + TB + koff(kk));  // converted to fp16 by the norm pass
        acc.X = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[kk], vx, kk ? acc.X : f32x16{}, 0, 0, 0);
      }
      if (kk == NKK / 2) {  // the augmented k-steps sit mid-chain, off the chains' tails
        acc.S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(augs, ones3, acc.S, 0, 0, 0);
        if constexpr (WITH_V) acc.X = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aug, nv, acc.X, 0, 0, 0);
      }
    }
    return acc;
  };
  // a column's sum over the wave rows of red, in wave order (every flush adds the same way)
  auto col_sum = [&](const float(*rd)[KT], int col) __attribute__((always_inline)) {
    float acc = rd[0][col];
#pragma unroll
    for (int w = 1; w < NWAVES; ++w) acc += rd[w][col];
    return acc * out_scale;
  };
  auto flush_share = [&](int it) __attribute__((always_inline)) {  // tile it's columns KPW*w ..
    const int fcol = KPW * wave + (lane % KPW);
    const int64_t j = c0 + (int64_t)it * KT + fcol;
    if (j < c1) pout[j] = col_sum(sm.red[it % 3], fcol);  // the lanes of a column store the same value
  };
  // tile flags as bits: lane L holds tiles 32L .. 32L+31 (a chunk has at most 1024 tiles)
  static_assert(kMaxTilesPerChunk <= 32 * 64, "flag bits");
  unsigned flagbits = 0;
  auto special = [&](int it) __attribute__((always_inline)) {
    const int64_t t0 = c0 + (int64_t)it * KT;
    const unsigned fb = (unsigned)__builtin_amdgcn_readlane((int)flagbits, it >> 5);
    return ((fb >> (it & 31)) & 1u) || (t0 + KT - 1 > n - W) || (t0 + KT > c1);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;

  // Ring schedule (one barrier per tile). At the top of iteration t, tiles t+1 and t+2
  // are in flight; waiting until at most NLD of this wave's DMA instructions are
  // outstanding means tile t+1 has landed. After the barrier: the column sums of tile t-1
  // are complete and are written; buffer (t+3)%4, last read by tile t-1's MFMAs, takes
  // tile t+3; tile t+1's norms are summed; tile t is computed from buffer t%4 with the
  // norms summed one iteration earlier. The two waves on a SIMD (w and w + NWAVES/2) do
  // the side work at different points of the iteration, so the SIMD's MFMA pipe keeps a
  // wave to feed it.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile 0 landed
  __syncthreads();
  for (int i = 0; i < 32; ++i) {
    const int t = 32 * lane + i;
    if (t < ntiles && sm.flag[t]) flagbits |= 1u << i;
  }
  norms(0);
  if (ntiles > 1) issue(1);
  if (ntiles > 2) issue(2);
  for (int t = 0; t < ntiles; ++t) {
    if (t + 2 < ntiles) {
      if constexpr (NLD == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else if constexpr (NLD == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    lds_barrier();  // the column stores of earlier tiles stay in flight
    auto side = [&]() __attribute__((always_inline)) {
      if (t >= 1) flush_share(t - 1);
      if (t + 3 < ntiles) {
        if (c0 + (int64_t)(t + 4) * KT <= c1) issue_full(t + 3);
        else issue(t + 3);
      }
      if (t + 1 < ntiles) norms(t + 1);
    };
    const bool early = !computing || wave < NWAVES / 2;
    if (early) side();
    if (computing) {
      const bool sp = special(t);
#pragma unroll
      for (int b = 0; b < KT / KB; ++b) {
        if (b == 1 && !early) side();
        const BlockAcc acc = mfma_block(t, b);
        float col = 0.f;
        const int key = (int)(c0 + (int64_t)t * KT + b * KB) + l32;
        if (sp) {
#pragma unroll
          for (int pi = 0; pi < 16; pi += PPR) pair_terms(T_{}, acc, pi, key, col);
        } else {
#pragma unroll
          for (int pi = 0; pi < 16; pi += PPR) pair_terms(F_{}, acc, pi, key, col);
        }
        {
          const HalfPair c2 = wave_halves(col);  // both half-waves hold the sum and write it
          col = c2.lo + c2.hi;
        }
        sm.red[t % 3][wave][b * KB + l32] = col;
      }
    }
  }
  __syncthreads();
  flush_share(ntiles - 1);
}

}  // namespace

hipError_t launch_score(const Dev& p, const void* q, const void* k, const void* v, const float* a, const float* lse,
                        const int32_t* jstar, float* partial, void* ws, hipStream_t st) {
  const int64_t rows = (int64_t)p.U * p.R;
  _Float16* ahat = (_Float16*)ws;
  float* na = (float*)((char*)ws + (size_t)rows * p.d * 2);
  float* l2 = na + rows;
  const dim3 gp((unsigned)((rows + 3) / 4)), gs(p.score_chunks, p.Tq, p.U);
  auto run = [&](auto kern) {
    hipLaunchKernelGGL(kern, gs, dim3(NTHREADS), 0, st, p, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v,
                       (const _Float16*)ahat, (const float*)na, (const float*)l2, jstar, partial);
  };
  if (p.d == 128) {
    hipLaunchKernelGGL(score_prep_kernel<128>, gp, dim3(256), 0, st, rows, a, lse, ahat, na, l2);
    if (p.mode == 0) run(score_kernel<128, 0>);
    else if (p.mode == 1) run(score_kernel<128, 1>);
    else run(score_kernel<128, 2>);
  } else {
    hipLaunchKernelGGL(score_prep_kernel<64>, gp, dim3(256), 0, st, rows, a, lse, ahat, na, l2);
    if (p.mode == 0) run(score_kernel<64, 0>);
    else if (p.mode == 1) run(score_kernel<64, 1>);
    else run(score_kernel<64, 2>);
  }
  return hipGetLastError();
}

}  // namespace kvs
