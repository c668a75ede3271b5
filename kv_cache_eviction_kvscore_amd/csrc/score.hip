// Score pass: per-token output-perturbation score partials for one query tile.
//
// DropKV page, "Methodology in Plain English" (engineering paragraph): the scoring
// kernel reuses the forward's log-sum-exp, recomputes the logits tile by tile,
// derives the attention weight on the fly and expands the squared distance
// ||a||^2 + ||v||^2 - 2<a, v> so each value tile is read once per pass; the score of
// token j is sum_i p_ij/(1-p_ij) * ||a_i - v_j||_2 (Key Contribution 1), summed over
// the window rows and the query heads of the KV group.
//
// score_prep: a_hat = bf16(a) (the MFMA operand), ||a_hat||^2 from the rounded values
//   (so the expansion is the exact ||a_hat - v||^2 up to fp32 rounding), lse*log2(e).
// score_kernel: grid (key chunk, query tile, unit); up to 8 computing waves of 32 rows.
//   Orientation S = Q.K^T, X = A_hat.V^T (rows x keys) on v_mfma_f32_32x32x16_bf16 with
//   the row operands held in registers and K/V tiles of 64 keys staged in LDS: a lane
//   owns one key column and 16 rows of each 32x32 block, so the sum over rows stays in
//   the lane (plus one half-wave exchange), and the waves' column sums are added in
//   LDS in wave order. The expansion runs on the matrix cores: the A.V^T accumulator
//   starts at -||a_i||^2/2 (loop-invariant C input) and one extra k-step adds
//   1 * (-||v_j||^2/2), the latter split exactly into three bf16 parts, so the accumulator
//   is -D/2 with D = ||a - v||^2. Per pair: t = s*c1 - lse2, p = exp2(t), and
//   c*sqrt(D) = sqrt(2) * p*(D/2)*rsq((D/2)*(1-p)^2): two transcendentals and seven other
//   VALU operations; the sqrt(2) (2 in mode SQ) is applied once per token. Pairs
//   (i, j*_i) are skipped (their term comes exactly from the forward); so are keys after
//   a row's position. Both masks only act on tiles flagged in LDS, others run unmasked.
//   Every pair that is not masked has p <= 1/2 (the row's argmax is isolated), so 1 - p
//   needs no guard.
#include "kvs_internal.hpp"

namespace kvs {
namespace {

constexpr int KT = 64;
constexpr int KPAD = 8;
constexpr int NTHREADS = 512;
constexpr int kMaxTilesPerChunk = 1024;  // score_chunk <= 65536

template <int D>
struct ScoreSmem {
  alignas(16) __bf16 k[KT][D + KPAD];  // 16-byte alignment lets the tile reads be ds_read_b128
  alignas(16) __bf16 v[KT][D + KPAD];
  alignas(16) __bf16 nvx[KT][8];  // -||v||^2/2 as hi, mid, lo bf16 parts, then zeros
  float red[NTHREADS / 64][KT];
  int tlim[kRowsPerTileMax];
  int jst[kRowsPerTileMax];
  unsigned char flag[kMaxTilesPerChunk];
};

template <int D>
__global__ __launch_bounds__(256) void score_prep_kernel(int64_t rows, const float* __restrict__ a,
                                                         const float* __restrict__ lse, __bf16* __restrict__ ahat,
                                                         float* __restrict__ na, float* __restrict__ lse2) {
  constexpr int PER = D / 64;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    const __bf16 b = (__bf16)a[row * D + e];
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
                                                         const __bf16* __restrict__ ahat,
                                                         const float* __restrict__ na,
                                                         const float* __restrict__ lse2,
                                                         const int32_t* __restrict__ jstar,
                                                         float* __restrict__ partial) {
  constexpr int NKK = D / 16;
  constexpr int CPR = D / 8;
  constexpr int NST = KT * CPR / NTHREADS;
  static_assert(NST >= 1 && CPR <= 64, "tile shape");
  __shared__ ScoreSmem<D> sm;

  const int u = blockIdx.z, qt = blockIdx.y, ch = blockIdx.x;
  int l, s, g;
  unit_coords(p, u, l, s, g);
  const int64_t n = p.cu[s + 1] - p.cu[s];
  const int64_t c0 = (int64_t)ch * p.score_chunk;
  if (c0 >= n) return;
  const int64_t c1 = (n < c0 + p.score_chunk) ? n : c0 + p.score_chunk;
  const int ntiles = (int)((c1 - c0 + KT - 1) / KT);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const bool computing = wave * 32 < p.RT;
  const int64_t rbase = (int64_t)u * p.R + (int64_t)qt * p.RT;  // first row of this tile (global row index)
  const int rows_here = min(p.RT, p.R - qt * p.RT);

  // ---- per-row masks in LDS, tile flags for rows whose argmax falls in this chunk
  for (int t = tid; t < ntiles; t += NTHREADS) sm.flag[t] = 0;
  if (tid < p.RT) {
    const bool ok = tid < rows_here;
    sm.tlim[tid] = ok ? (int)(n - p.W + (qt * p.RT + tid) % p.W) : -1;
    sm.jst[tid] = ok ? jstar[rbase + tid] : -1;
  }
  __syncthreads();
  if (tid < rows_here) {
    const int js = sm.jst[tid];
    if (js >= c0 && js < c1) sm.flag[(js - c0) / KT] = 1;
  }

  // ---- row operands (A side): lane row l32, k-slots 8h..8h+7
  bf16x8 qf[NKK], af[NKK];
  {
    const int rt = wave * 32 + l32;
    const bool ok = computing && rt < rows_here;
    const __bf16* qrow = q + (rbase + (ok ? rt : 0)) * D;
    const __bf16* arow = ahat + (rbase + (ok ? rt : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      bf16x8 z = {};
      qf[kk] = ok ? *(const bf16x8*)(qrow + 16 * kk + 8 * h) : z;
      af[kk] = ok ? *(const bf16x8*)(arow + 16 * kk + 8 * h) : z;
    }
  }
  // ---- row constants in the output layout: element r is row 8(r/4) + 4h + (r%4) of the wave
  float LS[16];
  f32x16 XC;  // -||a_hat||^2 / 2, the C input of the A.V^T chain
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rt = wave * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
    const bool ok = computing && rt < rows_here;
    LS[r] = ok ? lse2[rbase + rt] : INFINITY;  // p = 0 for padding rows
    XC[r] = ok ? -0.5f * na[rbase + rt] : 0.f;
  }
  // augmented k-step: A side holds 1 in slots 0..2 (lanes of the first half-wave)
  bf16x8 aug = {};
  if (h == 0) {
    aug[0] = (__bf16)1.f;
    aug[1] = (__bf16)1.f;
    aug[2] = (__bf16)1.f;
  }
  const float out_scale = (MODE == 0) ? 1.41421356237309515f : 2.f;

  const __bf16* kb0 = k + l * p.ksl + g * p.ksh + p.cu[s] * p.kst;
  const __bf16* vb0 = v + l * p.vsl + g * p.vsh + p.cu[s] * p.vst;
  float* pout = partial + ((int64_t)(l * p.Hkv + g) * p.Tq + qt) * p.N + p.cu[s];
  const int nw = (p.RT + 31) / 32;

  // K/V tiles: register ring of two buffers, prefetched two tiles ahead of the LDS write.
  // A tile's column sums are flushed behind the next tile's first barrier.
  struct Ring {
    u32x4 k[NST], v[NST];
  };
  Ring A, B;
  auto load_into = [&](Ring& r, int64_t t0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      const int c = tid + NTHREADS * i, key = c / CPR, part = c % CPR;
      // keys past the chunk load the chunk's last row (always in bounds, unconditional, so the
      // loads of the two ring buffers can be waited for separately); they are masked later
      const int64_t j = (t0 + key < c1) ? t0 + key : c1 - 1;
      r.k[i] = *(const u32x4*)(kb0 + j * p.kst + part * 8);
      r.v[i] = *(const u32x4*)(vb0 + j * p.vst + part * 8);
    }
  };
  auto flush_cols = [&](int64_t tp) __attribute__((always_inline)) {  // tile tp's column sums, in wave order
    if (tid < KT) {
      const int64_t j = tp + tid;
      if (j < c1) {
        float acc = 0.f;
        for (int w = 0; w < nw; ++w) acc += sm.red[w][tid];
        pout[j] = acc * out_scale;
      }
    }
  };
  auto stage = [&](const Ring& r, int64_t t0) __attribute__((always_inline)) {
    __syncthreads();  // the previous tile's operand reads and column sums are complete
    if (t0 > c0) flush_cols(t0 - KT);
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      const int c = tid + NTHREADS * i, key = c / CPR, part = c % CPR;
      *(u32x4*)&sm.k[key][part * 8] = r.k[i];
      *(u32x4*)&sm.v[key][part * 8] = r.v[i];
      // ||v||^2 of this key: 8 squares here, then a sum over the CPR consecutive lanes of the key
      const bf16x8 vv = __builtin_bit_cast(bf16x8, r.v[i]);
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = (float)vv[e];
        ss += f * f;
      }
#pragma unroll
      for (int off = CPR / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
      if (part == 0) {
        const float x = -0.5f * ss;
        const __bf16 hi = (__bf16)x;
        const __bf16 mid = (__bf16)(x - (float)hi);
        const __bf16 lo = (__bf16)(x - (float)hi - (float)mid);
        bf16x8 w8 = {};
        w8[0] = hi;
        w8[1] = mid;
        w8[2] = lo;
        *(bf16x8*)&sm.nvx[key][0] = w8;
      }
    }
    __syncthreads();
  };
  auto compute_tile = [&](const int64_t t0) __attribute__((always_inline)) {
      const bool special = sm.flag[(t0 - c0) / KT] || (t0 + KT - 1 > n - p.W) || (t0 + KT > c1);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 S = {};
        f32x16 X = XC;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const bf16x8 kf = *(const bf16x8*)&sm.k[kb * 32 + l32][16 * kk + 8 * h];
          const bf16x8 vf = *(const bf16x8*)&sm.v[kb * 32 + l32][16 * kk + 8 * h];
          S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[kk], kf, S, 0, 0, 0);
          X = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk], vf, X, 0, 0, 0);
        }
        {
          bf16x8 nvf = {};
          if (h == 0) nvf = *(const bf16x8*)&sm.nvx[kb * 32 + l32][0];
          X = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aug, nvf, X, 0, 0, 0);  // X = -D/2
        }
        float col = 0.f;
        const int key = (int)(t0 + kb * 32 + l32);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = __builtin_amdgcn_exp2f(fmaf(S[r], p.c1, -LS[r]));
          const float dh = fmaxf(-X[r], 1e-30f);  // D/2, kept positive
          const float om = 1.f - pr;
          float term;
          if (MODE == 0)
            term = pr * dh * __builtin_amdgcn_rsqf(dh * om * om);  // p sqrt(D/2) / (1-p)
          else
            term = pr * pr * dh * __builtin_amdgcn_rcpf(om * om);  // p^2 (D/2) / (1-p)^2
          if (special) {
            const int rt = wave * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (key > sm.tlim[rt] || key == sm.jst[rt]) term = 0.f;
          }
          col += term;
        }
        col += __shfl_xor(col, 32, 64);
        if (h == 0) sm.red[wave][kb * 32 + l32] = col;
      }
      };

  load_into(A, c0);
  if (c0 + KT < c1) load_into(B, c0 + KT);
  int64_t last = c0;
  for (int64_t t0 = c0; t0 < c1; t0 += 2 * KT) {
    stage(A, t0);
    if (t0 + 2 * KT < c1) load_into(A, t0 + 2 * KT);
    if (computing) compute_tile(t0);
    last = t0;
    if (t0 + KT < c1) {
      stage(B, t0 + KT);
      if (t0 + 3 * KT < c1) load_into(B, t0 + 3 * KT);
      if (computing) compute_tile(t0 + KT);
      last = t0 + KT;
    }
  }
  __syncthreads();
  flush_cols(last);
}

}  // namespace

hipError_t launch_score(const Dev& p, const void* q, const void* k, const void* v, const float* a, const float* lse,
                        const int32_t* jstar, float* partial, void* ws, hipStream_t st) {
  const int64_t rows = (int64_t)p.U * p.R;
  __bf16* ahat = (__bf16*)ws;
  float* na = (float*)((char*)ws + (size_t)rows * p.d * 2);
  float* l2 = na + rows;
  const dim3 gp((unsigned)((rows + 3) / 4)), gs(p.score_chunks, p.Tq, p.U);
  if (p.d == 128) {
    hipLaunchKernelGGL(score_prep_kernel<128>, gp, dim3(256), 0, st, rows, a, lse, ahat, na, l2);
    if (p.mode == 0)
      hipLaunchKernelGGL((score_kernel<128, 0>), gs, dim3(NTHREADS), 0, st, p, (const __bf16*)q, (const __bf16*)k,
                         (const __bf16*)v, (const __bf16*)ahat, (const float*)na, (const float*)l2, jstar, partial);
    else
      hipLaunchKernelGGL((score_kernel<128, 1>), gs, dim3(NTHREADS), 0, st, p, (const __bf16*)q, (const __bf16*)k,
                         (const __bf16*)v, (const __bf16*)ahat, (const float*)na, (const float*)l2, jstar, partial);
  } else {
    hipLaunchKernelGGL(score_prep_kernel<64>, gp, dim3(256), 0, st, rows, a, lse, ahat, na, l2);
    if (p.mode == 0)
      hipLaunchKernelGGL((score_kernel<64, 0>), gs, dim3(NTHREADS), 0, st, p, (const __bf16*)q, (const __bf16*)k,
                         (const __bf16*)v, (const __bf16*)ahat, (const float*)na, (const float*)l2, jstar, partial);
    else
      hipLaunchKernelGGL((score_kernel<64, 1>), gs, dim3(NTHREADS), 0, st, p, (const __bf16*)q, (const __bf16*)k,
                         (const __bf16*)v, (const __bf16*)ahat, (const float*)na, (const float*)l2, jstar, partial);
  }
  return hipGetLastError();
}

}  // namespace kvs
