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
// score_kernel: grid (key chunk, query tile, unit); 8 waves of one 32-row block each, two
//   per SIMD (the kernel also builds with 4 waves of two blocks, one per SIMD; measured
//   slower). A query tile of at most seven row blocks (G = 7: 224 rows) leaves the last
//   wave without rows; that instance (HLP) gives it the side work of every wave (all DMA,
//   the tile's norms and V conversion, every column flush) in a loop of its own with the
//   same barriers, and the computing waves run only their half tiles. Orientation S = Q.K^T on v_mfma_f32_32x32x16_bf16 and X = A_hat.V^T (rows x
//   keys) on v_mfma_f32_32x32x16_f16, with the row operands held in AGPRs and the
//   accumulators written to VGPRs. K/V tiles of 64 keys go from HBM straight into LDS
//   (global_load_lds_dwordx4, no register staging) through a ring of four buffers, so two
//   tiles are in flight while one is computed. A tile keeps whole key rows (each DMA
//   instruction moves four or eight full rows); the 16-byte chunks of row r are
//   XOR-swizzled with a function of r so that the 32 keys x 16 slots an MFMA operand needs
//   are read conflict-free with ds_read_b128. A lane owns one key column and 16 rows of the
//   32x32 block, so the sum over rows stays in the lane (plus one half-wave exchange); the
//   waves' column sums are added in LDS in wave order.
//   Software pipeline: a tile is two half tiles of 32 keys; each half tile's MFMAs run
//   with the pair work of the previous half tile spread over their k-steps (one MFMA, then
//   a share of the VALU work, and so on; an empty volatile asm statement ends each share,
//   which keeps the compiler from gathering the VALU work after the MFMAs), so a wave keeps
//   the matrix pipe and the VALU busy at once. Two accumulator sets alternate with fixed
//   roles (block 0 and block 1 of a tile), so no registers are copied.
//   The expansion runs on the matrix cores: one extra bf16 k-step multiplies
//   (1, 1, 1, -||a_hat_i||^2/2 in three parts) by (-||v_j||^2/2 in three parts, 1, 1, 1)
//   into the same accumulator; every part is an exact bf16 split, so X is -D/2 with
//   D = ||a_hat - v||^2. ||v_j||^2 is summed from the tile in LDS (v_dot2_f32_bf16, the
//   key's lanes added by DPP) one tile ahead of its use, and the same pass converts the
//   tile's V to fp16 in place (exact in fp16's normal range) for the A_hat.V^T product. The
//   Q.K^T chain gets an augmented k-step too: (-lse_i/scale in three bf16 parts) times
//   (1, 1, 1), so its accumulator is ln p / scale and needs no per-row register.
//   Per pair, two forms (one wave-wide vote per half tile picks one):
//   - every p of the half tile below 2^-8: p = exp2(acc * scale * log2 e), c = p + p^2,
//     whose relative error against p/(1-p) is p^2 < 2^-16; term c * sqrt(D/2): two
//     transcendentals and three other VALU instructions;
//   - otherwise 1/p = exp2(-acc * scale * log2 e) and c*sqrt(D) = sqrt(2) * sqrt(D/2) /
//     (1/p - 1): three transcendentals and three other VALU instructions.
//   The sqrt(2) (2 in mode SQ) is applied once per token.
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
constexpr int KB = 32;   // keys per half tile (one MFMA column block)
constexpr int NBUF = 4;  // tile ring: computed, next (its ||v||^2 summed), two in flight
// A workgroup covers one query tile of up to 256 rows: 8 waves of one 32-row block each
// (two waves per SIMD) or 4 waves of two blocks (one wave per SIMD); RB = blocks per wave.
constexpr int kMaxWaves = 8;
constexpr int kScoreRowBlocks = 1;
constexpr int kMaxTilesPerChunk = 1024;  // score_chunk <= 65536

template <int D>
struct ScoreSmem {
  // tile ring: [buffer][tensor K, V][key][D] with row r's 16-byte chunks XOR-swizzled
  alignas(16) __bf16 tile[NBUF][2][KT * D];
  alignas(16) __bf16 nvx[2][KT][8];  // (-||v||^2/2 as hi, mid, lo bf16 parts, 1, 1, 1, 0, 0)
  float red[3][kMaxWaves][KT];
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

// accumulators of one half tile: S = ln p / scale and X = -D/2 for each row block
template <int RB>
struct Half {
  f32x16 S[RB], X[RB];
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

template <int D, int MODE, int RB, bool HLP>
__global__ __launch_bounds__(512 / RB) __attribute__((amdgpu_waves_per_eu(2 / RB, 2 / RB))) void score_kernel(
    Dev p, const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const _Float16* __restrict__ ahat, const float* __restrict__ na, const float* __restrict__ lse2,
    const int32_t* __restrict__ jstar, float* __restrict__ partial) {
  constexpr int NWAVES = 8 / RB;
  constexpr int NTHREADS = 64 * NWAVES;
  static_assert(NWAVES * RB * 32 == kRowsPerTileMax && NWAVES <= kMaxWaves, "a workgroup covers one query tile");
  constexpr int NKK = D / 16;             // k-steps per row operand
  constexpr int RS = D * 2;               // bytes per key row
  constexpr int CPK = D / 8;              // 16-byte chunks per key row
  constexpr int TB = KT * RS;             // bytes per tensor tile
  constexpr bool WITH_V = MODE != 2;      // the attention-sum mode reads no V, a or norms
  constexpr int IPT = KT * CPK / 64;      // DMA wave instructions per tensor tile
  constexpr int NLD = (WITH_V ? 2 : 1) * IPT / NWAVES;  // DMA instructions per wave per tile
  constexpr int KPW = KT / NWAVES;        // keys per wave in the norm pass and the column sums
  constexpr int LPK = 64 / KPW;           // lanes per key in the norm pass
  constexpr int CPN = CPK / LPK;          // 16-byte chunks per lane in the norm pass
  static_assert(IPT % NWAVES == 0 && NLD >= 1 && NLD <= 8 && (NLD & (NLD - 1)) == 0, "tile shape");
  static_assert(KT % NWAVES == 0 && 64 % KPW == 0 && CPK % LPK == 0 && CPN >= 1, "norm pass shape");
  __shared__ ScoreSmem<D> sm;

  int ch, qt, u;
  xcd_item3(p, ch, qt, u);
  int l, s, g;
  unit_coords(p, u, l, s, g);
  const int64_t n = p.cu[s + 1] - p.cu[s];
  const int64_t c0 = (int64_t)ch * p.score_chunk;
  if (c0 >= n) return;
  const int64_t c1 = (n < c0 + p.score_chunk) ? n : c0 + p.score_chunk;
  const int ntiles = (int)((c1 - c0 + KT - 1) / KT);

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const int wrow0 = wave * 32 * RB;  // first tile row of this wave
  const int64_t rbase = (int64_t)u * p.R + (int64_t)qt * p.RT;  // first row of this tile (global row index)
  const int rows_here = min(p.RT, p.R - qt * p.RT);
  const bool computing = wrow0 < rows_here;
  // HLP (query tiles of at most seven row blocks): the last wave, which holds no rows, does
  // every wave's side work (all DMA, the whole tile's norms and V conversion, every column
  // flush), and the computing waves run their half tiles only
  static_assert(!HLP || RB == 1, "the helper form has one row block per wave");
  const bool helper = HLP && wave == NWAVES - 1;

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
  auto issue_any = [&](int it) __attribute__((always_inline)) {
    if (c0 + (int64_t)(it + 1) * KT <= c1) issue_full(it);
    else issue(it);
  };
  // -||v||^2/2 of tile it (landed, visible), into nvx[it & 1]: wave w sums keys
  // KPW*w .. KPW*w+KPW-1, LPK lanes per key (lanes key%KPW + KPW*c), CPN chunks each.
  auto norms = [&](int it) __attribute__((always_inline)) {
    if constexpr (!WITH_V) return;
    char* vt = (char*)sm.tile[it % NBUF][1];
    // a key's LPK lanes are consecutive, so its sum is a DPP reduction within the lanes' row
    const int key = KPW * wave + lane / LPK, cg = lane % LPK;
    float ss = 0.f;
    u32x4 w[CPN];
#pragma unroll
    for (int e = 0; e < CPN; ++e) w[e] = *(const u32x4*)(vt + key * RS + (((CPN * cg + e) ^ swz<D>(key)) << 4));
#pragma unroll
    for (int e = 0; e < CPN; ++e) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        // copy the element out first: a bit_cast of a vector-element lvalue reads element 0
        const unsigned wm = w[e][m];
        const bf16x2 x = __builtin_bit_cast(bf16x2, wm);
        ss = __builtin_amdgcn_fdot2_f32_bf16(x, x, ss, false);
      }
      // the A_hat.V^T product reads the tile in fp16
      *(u32x4*)(vt + key * RS + (((CPN * cg + e) ^ swz<D>(key)) << 4)) = bf16x8_to_f16x8(w[e]);
    }
    ss = group_sum<LPK>(ss);
    const Split3 sp = split3(-0.5f * ss);
    bf16x8 w8 = {};
    w8[0] = sp.hi;
    w8[1] = sp.mid;
    w8[2] = sp.lo;
    w8[3] = (__bf16)1.f;
    w8[4] = (__bf16)1.f;
    w8[5] = (__bf16)1.f;
    if (cg == 0) *(bf16x8*)&sm.nvx[it & 1][key][0] = w8;
  };

  // the whole tile's -||v||^2/2 and fp16 V: lane = key, its CPK chunks in two rounds
  constexpr int NLDH = NLD * NWAVES;  // DMA instructions per tile, every wave's share
  auto norms_h = [&](int it) __attribute__((always_inline)) {
    if constexpr (!WITH_V) return;
    char* vt = (char*)sm.tile[it % NBUF][1];
    const int key = lane;
    float ss = 0.f;
    constexpr int CH = CPK / 2;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      u32x4 w[CH];
#pragma unroll
      for (int e = 0; e < CH; ++e) w[e] = *(const u32x4*)(vt + key * RS + (((CH * half + e) ^ swz<D>(key)) << 4));
#pragma unroll
      for (int e = 0; e < CH; ++e) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const unsigned wm = w[e][m];
          const bf16x2 x = __builtin_bit_cast(bf16x2, wm);
          ss = __builtin_amdgcn_fdot2_f32_bf16(x, x, ss, false);
        }
        *(u32x4*)(vt + key * RS + (((CH * half + e) ^ swz<D>(key)) << 4)) = bf16x8_to_f16x8(w[e]);
      }
    }
    const Split3 sp = split3(-0.5f * ss);
    bf16x8 w8 = {};
    w8[0] = sp.hi;
    w8[1] = sp.mid;
    w8[2] = sp.lo;
    w8[3] = (__bf16)1.f;
    w8[4] = (__bf16)1.f;
    w8[5] = (__bf16)1.f;
    *(bf16x8*)&sm.nvx[it & 1][key][0] = w8;
  };

  // ---- per-row masks in LDS, tile flags for rows whose argmax falls in this chunk
  for (int t = tid; t < ntiles; t += NTHREADS) sm.flag[t] = 0;
  for (int t = tid; t < 3 * kMaxWaves * KT; t += NTHREADS) (&sm.red[0][0][0])[t] = 0.f;  // waves that never compute add zeros
  for (int t = tid; t < kRowsPerTileMax; t += NTHREADS) {
    const bool ok = t < rows_here;
    sm.tlim[t] = ok ? (int)(n - W + (qt * p.RT + t) % W) : -1;
    sm.jst[t] = ok ? jstar[rbase + t] : -1;
  }
  // the helper's DMA of tile it: every wave's share (NLDH instructions), the slot mapping of
  // issue(); full tiles take byte offsets from a table the helper builds once (off)
  unsigned off[HLP ? NLDH : 1];
  auto issue_h = [&](int it) __attribute__((always_inline)) {
    const int64_t t0 = c0 + (int64_t)it * KT;
    const bool full = t0 + KT <= c1;
#pragma unroll
    for (int f = 0; f < NLDH; ++f) {
      const int tensor = f / IPT;
      const __bf16* base = tensor == 0 ? kb0 + t0 * kst : vb0 + t0 * vst;
      unsigned o;
      if (full) {
        o = off[f];
      } else {
        const int slot = (f % IPT) * 64 + lane;
        const int r = slot / CPK, c = (slot % CPK) ^ swz<D>(r);
        const int rr = (t0 + r < c1) ? r : (int)(c1 - 1 - t0);  // rows past the chunk load its last
        o = (unsigned)(rr * (int)(tensor == 0 ? kst : vst) + 8 * c) * 2u;
      }
      lds_dma16(base, o, smb + (unsigned)(((it % NBUF) * 2 + tensor) * TBYTES + (f % IPT) * 1024));
    }
  };
  if constexpr (HLP) {
    if (helper) {
#pragma unroll
      for (int f = 0; f < NLDH; ++f) {
        const int tensor = f / IPT, slot = (f % IPT) * 64 + lane;
        const int r = slot / CPK, c = (slot % CPK) ^ swz<D>(r);
        off[f] = (unsigned)(r * (int)(tensor == 0 ? kst : vst) + 8 * c) * 2u;
      }
      issue_h(0);
    }
  } else {
    issue(0);
  }
  __syncthreads();
  for (int t = tid; t < rows_here; t += NTHREADS) {
    const int js = sm.jst[t];
    if (js >= c0 && js < c1) sm.flag[(js - c0) / KT] = 1;
  }

  // ---- row operands (A side) of the wave's RB blocks of 32 rows: lane row l32 of block
  // r, k-slots 8h..8h+7
  bf16x8 qf[RB][NKK], aug[RB], augs[RB];
  f16x8 af[RB][NKK];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int rt = wrow0 + 32 * r + l32;
    const bool ok = rt < rows_here;
    const __bf16* qrow = q + (rbase + (ok ? rt : 0)) * D;
    const _Float16* arow = ahat + (rbase + (ok ? rt : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      bf16x8 z = {};
      f16x8 zh = {};
      qf[r][kk] = ok ? *(const bf16x8*)(qrow + 16 * kk + 8 * h) : z;
      af[r][kk] = (ok && WITH_V) ? *(const f16x8*)(arow + 16 * kk + 8 * h) : zh;
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
    aug[r] = w8;
    augs[r] = s8;
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
  for (int r = 0; r < RB; ++r) {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      asm volatile("" : "+a"(qf[r][kk]));
      if constexpr (WITH_V) asm volatile("" : "+a"(af[r][kk]));
    }
    if constexpr (WITH_V) asm volatile("" : "+a"(aug[r]));
    asm volatile("" : "+a"(augs[r]));
  }
  // sqrt(2) turns sqrt(D/2) into sqrt(D); mode SQ's p^2 (D/2)/(1-p)^2 needs 2; p needs 1
  const float out_scale = (MODE == 0) ? 1.41421356237309515f : (MODE == 1 ? 2.f : 1.f);
  // byte offset, within a tensor tile, of this lane's operand chunk (key l32, slots
  // 16kk + 8h .. +7) for k-step kk; half tile b adds 32 rows
  const int kbase = l32 * RS, khs = h ^ swz<D>(l32);
  auto koff = [&](int kk) __attribute__((always_inline)) { return kbase + (((2 * kk) ^ khs) << 4); };

  // The pair terms of pairs [pi0, pi0 + NP) of a half tile's accumulators, added to col
  // (pair pi = 16r + e: row 32r + 8(e/4) + 4h + (e%4) of the wave, the lane's key
  // column). Stage by stage over the NP pairs, so their chains interleave.
  // kind: 0 = small p (every p of the half tile below 2^-8: p/(1-p) = p + p^2 to 2^-16
  // relative), 1 = the exact form, 2 = the exact form with the masks (causal limit, the
  // row's isolated argmax)
  auto pair_terms = [&](auto kind, auto np, Half<RB>& acc, const int pi0, const int key, float& col)
      __attribute__((always_inline)) {
    constexpr int NP = decltype(np)::value;
    constexpr int KIND = decltype(kind)::value;
    static_assert(16 % NP == 0, "a slice stays within one row block");
    const int rb = pi0 >> 4;
    float sv[NP], xv[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      sv[i] = acc.S[rb][(pi0 + i) & 15];
      if constexpr (MODE != 2) xv[i] = acc.X[rb][(pi0 + i) & 15];
    }
    float x[NP], y[NP];  // the pair's term is x * y
    if constexpr (MODE == 2) {
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        x[i] = __builtin_amdgcn_exp2f(sv[i] * c1s);  // p itself
        y[i] = 1.f;
      }
    } else if constexpr (KIND == 0) {
      // c = p/(1-p) = p (1 + p + p^2 + ...) = p + p^2 up to a relative p^2 < 2^-16
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const float pp = __builtin_amdgcn_exp2f(sv[i] * c1s);
        x[i] = fmaf(pp, pp, pp);
      }
      if constexpr (MODE == 0) {
#pragma unroll
        for (int i = 0; i < NP; ++i) y[i] = __builtin_amdgcn_sqrtf(fabsf(xv[i]));
      } else {
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          x[i] = x[i] * x[i];
          y[i] = fabsf(xv[i]);
        }
      }
    } else {
      // e = 1/p and 1/(e - 1) = p/(1-p): e >= 2 on every unmasked pair, so it is finite
      // (0 when p underflows); a masked pair's value is never added
      float e[NP];
#pragma unroll
      for (int i = 0; i < NP; ++i) e[i] = __builtin_amdgcn_exp2f(sv[i] * nc1s);
#pragma unroll
      for (int i = 0; i < NP; ++i) x[i] = __builtin_amdgcn_rcpf(e[i] - 1.f);
      if constexpr (MODE == 0) {
#pragma unroll
        for (int i = 0; i < NP; ++i) y[i] = __builtin_amdgcn_sqrtf(fabsf(xv[i]));
      } else {
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          x[i] = x[i] * x[i];
          y[i] = fabsf(xv[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if constexpr (KIND == 2) {
        const int pi = pi0 + i, e = pi & 15;
        const int rt = wrow0 + 32 * (pi >> 4) + 8 * (e >> 2) + 4 * h + (e & 3);
        col += (key > sm.tlim[rt] || key == sm.jst[rt]) ? 0.f : x[i] * y[i];
      } else if constexpr (MODE == 2) {
        col += x[i];
      } else {
        col = fmaf(x[i], y[i], col);
      }
    }
    // an empty volatile asm statement that reads and redefines the sum: the slice is complete
    // here (the compiler otherwise gathers every slice after the MFMAs)
    asm volatile("" : "+v"(col));
  };
  // One half tile (it, b): the MFMAs of keys 32b .. 32b+31 of ring tile it against the
  // wave's RB row blocks (S = ln p / scale, X = -D/2; four independent accumulation chains,
  // S and X of two row blocks, keep the matrix pipe issuing back to back), with the pair
  // work of the previous half tile (pv, from tile pit, block pb) spread over its k-steps:
  // each k-step's MFMAs are followed by a slice of that work and a scheduling fence, so the
  // matrix pipe and the VALU run together within the wave. Returns the previous half
  // tile's column sum over the wave's rows (both half-waves hold it).
  constexpr int PPK = 16 * RB / NKK;  // pairs of the previous half tile per k-step
  auto half_tile = [&](auto kind, auto first, int it, int b, Half<RB>& acc, Half<RB>& pv, int pit, int pb)
      __attribute__((always_inline)) {
    constexpr bool FIRST = decltype(first)::value;
    const char* kt = (const char*)sm.tile[it % NBUF][0] + b * KB * RS;
    const int pkey = (int)(c0 + (int64_t)pit * KT + pb * KB) + l32;
    bf16x8 nv = {};
    if constexpr (WITH_V) nv = *(const bf16x8*)&sm.nvx[it & 1][b * KB + l32][0];
    float col = 0.f;
    bf16x8 kx = *(const bf16x8*)(kt + koff(0));
    f16x8 vx = {};
    if constexpr (WITH_V) vx = *(const f16x8*)(kt + TB + koff(0));  // converted to fp16 by the norm pass
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      bf16x8 kxn = kx;
      f16x8 vxn = vx;
      if (kk + 1 < NKK) {  // the next k-step's operands are read while this one's MFMAs run
        kxn = *(const bf16x8*)(kt + koff(kk + 1));
        if constexpr (WITH_V) vxn = *(const f16x8*)(kt + TB + koff(kk + 1));
      }
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        acc.S[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[r][kk], kx, kk ? acc.S[r] : f32x16{}, 0, 0, 0);
        if constexpr (WITH_V) acc.X[r] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[r][kk], vx, kk ? acc.X[r] : f32x16{}, 0, 0, 0);
      }
      if (kk == NKK / 2) {  // the augmented k-steps sit mid-chain, off the chains' tails
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          acc.S[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(augs[r], ones3, acc.S[r], 0, 0, 0);
          if constexpr (WITH_V) acc.X[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aug[r], nv, acc.X[r], 0, 0, 0);
        }
      }
      if constexpr (!FIRST) {
        pair_terms(kind, std::integral_constant<int, PPK>{}, pv, kk * PPK, pkey, col);
        // within the k-step: one MFMA, then a share of the slice's VALU work, and so on; a
        // wave issues in order, so MFMAs issued back to back would hold the VALU work behind
        // them
        constexpr int MPK = (WITH_V ? 2 : 1) * RB;  // MFMAs per k-step (twice that at the augmented one)
        constexpr int VS = PPK * (MODE == 2 ? 3 : 6);  // VALU instructions of the slice
        if (kk == NKK / 2) {
#pragma unroll
          for (int m = 0; m < 2 * MPK; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002 | 0x400, (VS + 2 * MPK - 1) / (2 * MPK), 0);
          }
        } else {
#pragma unroll
          for (int m = 0; m < MPK; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002 | 0x400, (VS + MPK - 1) / MPK, 0);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      kx = kxn;
      vx = vxn;
    }
    if constexpr (FIRST) return 0.f;
    const HalfPair c2 = wave_halves(col);
    return c2.lo + c2.hi;
  };
  // the pair work of the last half tile, alone
  auto tail_pairs = [&](auto kind, Half<RB>& pv, int pit, int pb) __attribute__((always_inline)) {
    const int pkey = (int)(c0 + (int64_t)pit * KT + pb * KB) + l32;
    float col = 0.f;
#pragma unroll
    for (int pi = 0; pi < 16 * RB; pi += PPK) pair_terms(kind, std::integral_constant<int, PPK>{}, pv, pi, pkey, col);
    const HalfPair c2 = wave_halves(col);
    return c2.lo + c2.hi;
  };
  // the column sums of tile it, columns KPW*w .. KPW*w+KPW-1: flush_load reads the waves'
  // row sums from LDS, flush_store adds them in wave order and writes the scores; between
  // the two the LDS reads are in flight
  auto flush_load = [&](int it, float (&fv)[NWAVES]) __attribute__((always_inline)) {
    // the lane index taken afresh (an opaque v_mbcnt): kept from the prologue, the column
    // offset would stay live across the whole loop only for this use
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    const int fcol = KPW * wave + (ln % KPW);
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) fv[w] = sm.red[it % 3][w][fcol];
  };
  auto flush_store = [&](int it, const float (&fv)[NWAVES]) __attribute__((always_inline)) {
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    if (ln >= KPW) return;
    const int64_t j = c0 + (int64_t)it * KT + KPW * wave + ln;
    float acc = fv[0];
#pragma unroll
    for (int w = 1; w < NWAVES; ++w) acc += fv[w];
    if (j < c1) pout[j] = acc * out_scale;
  };
  auto flush_share = [&](int it) __attribute__((always_inline)) {
    float fv[NWAVES];
    flush_load(it, fv);
    flush_store(it, fv);
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
  using K0 = std::integral_constant<int, 0>;
  using K1 = std::integral_constant<int, 1>;
  using K2 = std::integral_constant<int, 2>;
  // whether every pair of a half tile has p below 2^-8: S = ln p / scale, so p < 2^-8 is
  // S < -8 / (scale log2 e); one wave-wide vote
  const float small_lim = -8.f / c1s;
  auto all_small = [&](const Half<RB>& acc) __attribute__((always_inline)) {
    if constexpr (MODE == 2) return false;
    float m = acc.S[0][0];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int e = 0; e < 16; ++e) m = fmaxf(m, acc.S[r][e]);
    return __ballot(m >= small_lim) == 0;
  };
  // the pair work of pv (tile pit, block pb) with the right kind, run with the MFMAs of (it, b)
  auto step = [&](bool special_prev, auto first, int it, int b, Half<RB>& acc, Half<RB>& pv, int pit, int pb)
      __attribute__((always_inline)) {
    if (special_prev) return half_tile(K2{}, first, it, b, acc, pv, pit, pb);
    if (all_small(pv)) return half_tile(K0{}, first, it, b, acc, pv, pit, pb);
    return half_tile(K1{}, first, it, b, acc, pv, pit, pb);
  };
  auto tail = [&](bool special_prev, Half<RB>& pv, int pit, int pb) __attribute__((always_inline)) {
    if (special_prev) return tail_pairs(K2{}, pv, pit, pb);
    if (all_small(pv)) return tail_pairs(K0{}, pv, pit, pb);
    return tail_pairs(K1{}, pv, pit, pb);
  };
  // Ring schedule (one barrier per tile). At the top of iteration t, tiles t+1 and t+2
  // are in flight; waiting until at most NLD of this wave's DMA instructions are
  // outstanding means tile t+1 has landed. After the barrier: the column sums of tile t-2
  // are complete and are written; buffer (t+3)%4, last read by tile t-1's MFMAs, takes
  // tile t+3; tile t+1's norms are summed and its V converted. Then the two half tiles of
  // tile t: each one's MFMAs run with the previous half tile's pair work interleaved (the
  // last half tile of tile t-1, then the first of tile t). The pair work of a half tile
  // therefore ends one half tile later, and a tile's column sums are complete after the
  // barrier two iterations on.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile 0 landed
  __syncthreads();
  for (int i = 0; i < 32; ++i) {
    const int t = 32 * lane + i;
    if (t < ntiles && sm.flag[t]) flagbits |= 1u << i;
  }
  if constexpr (HLP) {
    if (helper) {
      // the helper's own loop: the same barriers as the computing waves' loop below, with
      // the side work of every wave. One wave keeps all DMA of two tiles in flight, and at
      // most 63 vector memory operations may be outstanding: tile 2 waits for the first of
      // tile 1's, and each iteration waits as described at its top.
      norms_h(0);
      if (ntiles > 1) issue_h(1);
      if (ntiles > 2) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NLDH - 1) : "memory");
        issue_h(2);
      }
      // outstanding operations at the top of iteration t, oldest first: tile t+1's NLDH
      // DMAs, the column store of iteration t-1 (from t = 3 on), tile t+2's NLDH DMAs. Tile
      // t+1 has landed once at most NLDH remain; fewer (HW) also leave room for the NLDH + 1
      // the iteration adds, within the counter's 63
      constexpr int HW = (NLDH < 62 - NLDH) ? NLDH : 62 - NLDH;
      for (int t = 0; t < ntiles; ++t) {
        if (t + 2 < ntiles) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(HW) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
        if (t >= 2) {  // the column sums of tile t-2, added in wave order; the store first
          const int64_t j = c0 + (int64_t)(t - 2) * KT + lane;
          float acc = sm.red[(t - 2) % 3][0][lane];
#pragma unroll
          for (int w = 1; w < NWAVES; ++w) acc += sm.red[(t - 2) % 3][w][lane];
          if (j < c1) pout[j] = acc * out_scale;
        }
        if (t + 3 < ntiles) issue_h(t + 3);
        if (t + 1 < ntiles) norms_h(t + 1);
      }
    }
  } else {
    norms(0);
    if (ntiles > 1) issue_any(1);
    if (ntiles > 2) issue_any(2);
  }
  // two accumulator sets with fixed roles: A holds block 0 of a tile, B block 1 (no copies
  // between half tiles)
  Half<RB> A, B;
  bool sp_prev = false;  // tile t-1 needs the masked pair work
  for (int t = 0; t < (helper ? 0 : ntiles); ++t) {
    if constexpr (HLP) {
      // no DMA of this wave's own is in flight
    } else if (t + 2 < ntiles) {
      if constexpr (NLD == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else if constexpr (NLD == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else if constexpr (NLD == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    lds_barrier();  // the column stores of earlier tiles stay in flight
    // the side work (flush, DMA, norms) is mostly waiting on LDS round trips; the two waves
    // of a SIMD (w and w + NWAVES/2 with two waves per SIMD) do it at different points of
    // the iteration, so one wave's MFMAs and VALU work run while the other waits
    auto side = [&]() __attribute__((always_inline)) {
      float fv[NWAVES];
      if (t >= 2) flush_load(t - 2, fv);
      if (t + 3 < ntiles) issue_any(t + 3);
      if (t + 1 < ntiles) norms(t + 1);
      if (t >= 2) flush_store(t - 2, fv);
    };
    const bool early = !HLP && (!computing || RB == 2 || wave < NWAVES / 2);
    if (early) side();
    if (computing) {
      const bool sp = special(t);
      // block 0 of tile t into A, with the pair work of block 1 of tile t-1 (B)
      if (t == 0) {
        half_tile(K1{}, T_{}, t, 0, A, B, 0, 0);
      } else {
        const float cs = step(sp_prev, F_{}, t, 0, A, B, t - 1, 1);
        sm.red[(t - 1) % 3][wave][KB + l32] = cs;
      }
      if (!HLP && !early) side();
      // block 1 of tile t into B, with the pair work of block 0 of tile t (A)
      const float cs = step(sp, F_{}, t, 1, B, A, t, 0);
      sm.red[t % 3][wave][l32] = cs;
      sp_prev = sp;
    }
  }
  if (computing) {  // the pair work of the last half tile
    const float cs = tail(sp_prev, B, ntiles - 1, 1);
    sm.red[(ntiles - 1) % 3][wave][KB + l32] = cs;
  }
  __syncthreads();
  if (ntiles >= 2) flush_share(ntiles - 2);
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
  constexpr int RBL = kScoreRowBlocks;
  // query tiles of at most seven row blocks leave a wave without rows: it takes the side work
  const bool hlp = RBL == 1 && p.RT <= kRowsPerTileMax - 32;
  auto run = [&](auto kern) {
    hipLaunchKernelGGL(kern, gs, dim3(512 / RBL), 0, st, p, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v,
                       (const _Float16*)ahat, (const float*)na, (const float*)l2, jstar, partial);
  };
  auto pick = [&](auto d, auto mode) {
    constexpr int DD = decltype(d)::value, MM = decltype(mode)::value;
    if (hlp) run(score_kernel<DD, MM, RBL, RBL == 1>);
    else run(score_kernel<DD, MM, RBL, false>);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  if (p.d == 128) {
    using D = std::integral_constant<int, 128>;
    hipLaunchKernelGGL(score_prep_kernel<128>, gp, dim3(256), 0, st, rows, a, lse, ahat, na, l2);
    if (p.mode == 0) pick(D{}, I0{});
    else if (p.mode == 1) pick(D{}, I1{});
    else pick(D{}, I2{});
  } else {
    using D = std::integral_constant<int, 64>;
    hipLaunchKernelGGL(score_prep_kernel<64>, gp, dim3(256), 0, st, rows, a, lse, ahat, na, l2);
    if (p.mode == 0) pick(D{}, I0{});
    else if (p.mode == 1) pick(D{}, I1{});
    else pick(D{}, I2{});
  }
  return hipGetLastError();
}

}  // namespace kvs
