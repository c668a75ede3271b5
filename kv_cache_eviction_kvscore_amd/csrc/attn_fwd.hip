// Window-query attention forward with the argmax pair isolated.
//
// DropKV page, Key Contribution 3 / "Methodology in Plain English": the scorer reuses
// the log-sum-exp of a FlashAttention-2-style forward over the full cache. Here the
// forward also keeps each row's argmax key j* out of the bf16 P.V product: the rows'
// dominant pair has p* close to 1, where both 1 - p* and a - v_j* cancel; keeping
// l_rest = sum_{j != j*} exp(s_j - m) and acc_rest = sum_{j != j*} exp(s_j - m) v_j at
// their own scale gives p* = 1/(1 + l_rest), a^(-j*) = acc_rest / l_rest and the
// pair's exact shift p* * ||a^(-j*) - v_j*|| (the identity of the same section:
// c * ||a - v_j|| = p * ||a^(-j) - v_j||).
//
// Pass 1 (fwd_partial): grid (key chunk, query tile, unit). 8 waves; a computing wave
// owns 32 rows, one row per lane (both half-waves hold the row). S^T = K.Q^T on
// v_mfma_f32_32x32x16_bf16 and O^T += V^T.P^T on v_mfma_f32_32x32x16_f16; K/V tiles of
// 64 keys are staged in LDS (registers prefetch the next tile), V converted to fp16
// there (exact for |v| < 65504); V^T fragments come from ds_read_tr16_b64. P enters the
// product in fp16 (unit roundoff 2^-11, eight times finer than bf16: with few keys per
// row the rounding of P does not average out, and a^(-j*) feeds the isolated term),
// pre-scaled by 2^14 so probabilities down to ~4e-9 stay normal; the scale is folded
// into the exp2 argument and removed once at the end.
// Online softmax in the log2 domain. When a row's running max moves to a key of the
// current tile, the previous argmax's value row (kept in LDS, weight 1 at the old
// max) is folded into the rest and the new one is copied in.
// Pass 2 (fwd_combine): one wave per row merges the chunks' (m, l_rest, acc_rest, j*,
// v*) in ascending chunk order and writes a, lse, j*, and the isolated term.
#include "kvs_internal.hpp"

namespace kvs {
namespace {

constexpr int KT = 64;    // keys per compute sub-tile
constexpr int KL = 64;    // keys per LDS tile (one barrier pair, prefetched one tile ahead)
constexpr int KPAD = 8;   // bf16 padding per K row in LDS (b128 reads: 8 lanes hit distinct banks)
constexpr int VPAD = 16;  // bf16 padding per V row in LDS (transpose reads: 4 keys x 32 B distinct banks)
constexpr int SPAD = 4;   // bf16 padding per v* row
constexpr int NTHREADS = 512;
constexpr float kPScale = 16384.f;     // 2^14: P is carried as 2^14 * p in the rest sums
constexpr float kPScaleLog2 = 14.f;
constexpr float kPUnscale = 1.f / 16384.f;

template <int D>
struct FwdSmem {
  alignas(16) __bf16 k[KL][D + KPAD];  // 16-byte alignment lets the tile reads be ds_read_b128
  alignas(16) _Float16 v[KL][D + VPAD];
  alignas(16) _Float16 vstar[kRowsPerTileMax][D + SPAD];
};

// 8 bf16 -> 8 fp16 (exact in fp16's normal range; saturating towards zero beyond it)
__device__ inline u32x4 bf16x8_to_f16x8(u32x4 u) {
  const unsigned w[4] = {u[0], u[1], u[2], u[3]};
  unsigned r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xffff0000u);
    r[i] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  }
  return u32x4{r[0], r[1], r[2], r[3]};
}

__device__ inline float wave_shfl_xor_f(float x, int m) { return __shfl_xor(x, m, 64); }
__device__ inline int wave_shfl_xor_i(int x, int m) { return __shfl_xor(x, m, 64); }

template <int D>
__global__ __launch_bounds__(NTHREADS) void fwd_partial_kernel(Dev p, const __bf16* __restrict__ q,
                                                               const __bf16* __restrict__ k,
                                                               const __bf16* __restrict__ v, float* __restrict__ ws) {
  constexpr int NKK = D / 16;  // k-steps of the QK^T contraction
  constexpr int NDB = D / 32;  // 32-wide d blocks of O^T
  constexpr int CPR = D / 8;   // 16-byte chunks per row
  constexpr int NST = KL * CPR / NTHREADS;  // 16-byte chunks per thread per tensor
  static_assert(NST >= 1, "tile too small for the block");
  __shared__ FwdSmem<D> sm;

  const int u = blockIdx.z, qt = blockIdx.y, ch = blockIdx.x;
  int l, s, g;
  unit_coords(p, u, l, s, g);
  const int64_t n = p.cu[s + 1] - p.cu[s];
  const int64_t c0 = (int64_t)ch * p.fwd_chunk;
  if (c0 >= n) return;  // uniform: this sequence has fewer chunks
  const int64_t c1 = (n < c0 + p.fwd_chunk) ? n : c0 + p.fwd_chunk;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const bool computing = wave * 32 < p.RT;
  const int row_t = wave * 32 + l32;
  const int row = qt * p.RT + row_t;
  const bool row_ok = computing && row < p.R;
  const int64_t tlim = row_ok ? n - p.W + (row % p.W) : n - 1;  // last key the row sees

  bf16x8 qf[NKK];
  {
    const __bf16* qrow = q + ((int64_t)u * p.R + (row_ok ? row : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      bf16x8 z = {};
      qf[kk] = row_ok ? *(const bf16x8*)(qrow + 16 * kk + 8 * h) : z;
    }
  }

  float m = -INFINITY, m2 = -INFINITY, lrest = 0.f;
  int jst = -1;
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};

  const __bf16* kb0 = k + l * p.ksl + g * p.ksh + p.cu[s] * p.kst;
  const __bf16* vb0 = v + l * p.vsl + g * p.vsh + p.cu[s] * p.vst;

  // one 64-key sub-tile starting at key t0, LDS rows lb..lb+63
  auto compute_tile = [&](const int64_t t0, const int lb) {
    // ---- S^T = K Q^T for both 32-key blocks (chains interleaved): lane holds row l32 and,
    // at element r of block kb, key 32kb + 8(r/4) + 4h + (r%4). Values stay raw q.k; the
    // softmax scale enters through one FMA in front of exp2.
    f32x16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const bf16x8 k0 = *(const bf16x8*)&sm.k[lb + l32][16 * kk + 8 * h];
      const bf16x8 k1 = *(const bf16x8*)&sm.k[lb + 32 + l32][16 * kk + 8 * h];
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[kk], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[kk], acc1, 0, 0, 0);
    }
    float tv[32];  // element e = 16*kb + r
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      tv[r] = acc0[r];
      tv[16 + r] = acc1[r];
    }
    const int trel = (int)(t0 - c0);  // tile start relative to the chunk
    if ((t0 + KT - 1 > n - p.W) || (t0 + KT > c1)) {
      const int lim = (int)((tlim < c1 - 1 ? tlim : c1 - 1) - c0);  // last key this row may use, chunk-relative
#pragma unroll
      for (int e = 0; e < 32; ++e)
        if (trel + 32 * (e >> 4) + 8 * ((e & 15) >> 2) + 4 * h + (e & 3) > lim) tv[e] = -INFINITY;
    }
    float lm = tv[0];
#pragma unroll
    for (int e = 1; e < 32; ++e) lm = fmaxf(lm, tv[e]);
    const float mt = fmaxf(lm, wave_shfl_xor_f(lm, 32));

    // Row state (raw q.k units): m = running max (key jst, value row in vstar), m2 = running
    // max over every other key; the rest sums lrest / o are kept relative to m2, so a
    // dominant key never pushes the rest out of fp16's range.
    const bool moved = mt > m;
    const bool any_moved = __any(moved);
    int jr = -1;          // this lane's element index of the new argmax, if it holds it
    int jt = 0x7fffffff;  // chunk-relative key of the new argmax
    float m2n;
    if (any_moved) {
      int jl = 64;
      float hi2 = -INFINITY, lo2 = -INFINITY;
      if (moved) {
        // elements run in key order within a lane: the first equal to mt is the lane's lowest key
#pragma unroll
        for (int e = 31; e >= 0; --e) jl = (tv[e] == mt) ? e : jl;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          lo2 = __builtin_amdgcn_fmed3f(lo2, hi2, tv[e]);
          hi2 = fmaxf(hi2, tv[e]);
        }
      }
      const int keyl = (jl < 64) ? trel + 32 * (jl >> 4) + 8 * ((jl & 15) >> 2) + 4 * h + (jl & 3) : 0x7fffffff;
      jt = min(keyl, wave_shfl_xor_i(keyl, 32));
      jr = (moved && keyl == jt) ? jl : -1;
      // tile max without the new argmax: the lane holding it contributes its second largest
      const float mt2l = moved ? ((jr >= 0) ? lo2 : hi2) : -INFINITY;
      const float mt2 = fmaxf(mt2l, wave_shfl_xor_f(mt2l, 32));
      m2n = moved ? fmaxf(m, mt2) : fmaxf(m2, mt);  // the old max joins the rest when it moves
    } else {
      m2n = fmaxf(m2, mt);
    }
    const float mb = ((m2n == -INFINITY) ? 0.f : m2n * p.c1) - kPScaleLog2;

    float pr[32];  // 2^14 * exp2(c1 * (s - m2n)); the new argmax excluded
#pragma unroll
    for (int e = 0; e < 32; ++e) pr[e] = __builtin_amdgcn_exp2f(fmaf(tv[e], p.c1, -mb));
    if (jr >= 0) {
#pragma unroll
      for (int e = 0; e < 32; ++e) pr[e] = (e == jr) ? 0.f : pr[e];
    }
    // rescale the rest to the new m2
    if (__any(m2n > m2)) {
      const float alpha = (m2n > m2) ? ((m2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m2 - m2n) * p.c1)) : 1.f;
      lrest *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
    if (any_moved && moved) {
      // the previous argmax joins the rest with weight exp2(c1 (m - m2n)) <= 1 (2^14 scaled)
      if (jst >= 0) {
        const float wold = kPScale * __builtin_amdgcn_exp2f((m - m2n) * p.c1);
        lrest += wold;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const f16x4 vs = *(const f16x4*)&sm.vstar[row_t][32 * db + 8 * qq + 4 * h];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[db][4 * qq + e] += wold * (float)vs[e];
          }
      }
      const int jslot = jt - trel;  // new argmax's key in this tile
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          *(f16x4*)&sm.vstar[row_t][32 * db + 8 * qq + 4 * h] =
              *(const f16x4*)&sm.v[lb + jslot][32 * db + 8 * qq + 4 * h];
      jst = (int)c0 + jt;
      m = mt;
    }
    m2 = m2n;

    // ---- O^T += V^T P^T, 16 keys per k-step. B = P^T: lane (row, h) slots 8h..8h+7 =
    // its elements 8ks..8ks+7, i.e. keys 16ks+4h+{0..3} and 16ks+8+4h+{0..3}. lrest sums the
    // same fp16-rounded values that enter the product (packed dot with (1, 1)).
    float ts = 0.f;
    const f16x2 ones = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      f16x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = (_Float16)pr[8 * ks + e];
#pragma unroll
      for (int e = 0; e < 4; ++e) ts = __builtin_amdgcn_fdot2(f16x2{pf[2 * e], pf[2 * e + 1]}, ones, ts, false);
      const int kbase = lb + 16 * ks + 4 * h;  // first key of this lane-half's two 4-key runs
      const int sidx = lane & 15;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d0 = 32 * db + 16 * ((lane >> 4) & 1);
        const _Float16* a0 = &sm.v[kbase + (sidx >> 2)][d0 + 4 * (sidx & 3)];
        const _Float16* a1 = &sm.v[kbase + 8 + (sidx >> 2)][d0 + 4 * (sidx & 3)];
        const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a0);
        const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a1);
        // whole-vector casts: per-element bit casts of the loaded i16x4 were lowered to a
        // broadcast of element 0
        const f16x8 vf = __builtin_shufflevector(__builtin_bit_cast(f16x4, r0), __builtin_bit_cast(f16x4, r1), 0, 1,
                                                 2, 3, 4, 5, 6, 7);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf, o[db], 0, 0, 0);
      }
    }
    lrest += ts + wave_shfl_xor_f(ts, 32);
  };


  // K/V staging: the next LDS tile is loaded into registers while this one is computed.
  // Keys past the chunk load the chunk's last row (in bounds; the loads stay unconditional);
  // they are masked in the sub-tile that holds them.
  u32x4 kst[NST], vst[NST];
#pragma unroll
  for (int i = 0; i < NST; ++i) {
    const int c = tid + NTHREADS * i, key = c / CPR, part = c % CPR;
    const int64_t j = (c0 + key < c1) ? c0 + key : c1 - 1;
    kst[i] = *(const u32x4*)(kb0 + j * p.kst + part * 8);
    vst[i] = *(const u32x4*)(vb0 + j * p.vst + part * 8);
  }
  for (int64_t t0 = c0; t0 < c1; t0 += KL) {
    __syncthreads();  // all waves are done with the previous tile
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      const int c = tid + NTHREADS * i, key = c / CPR, part = c % CPR;
      *(u32x4*)&sm.k[key][part * 8] = kst[i];
      *(u32x4*)&sm.v[key][part * 8] = bf16x8_to_f16x8(vst[i]);
    }
    __syncthreads();
    if (t0 + KL < c1) {
#pragma unroll
      for (int i = 0; i < NST; ++i) {
        const int c = tid + NTHREADS * i, key = c / CPR, part = c % CPR;
        const int64_t j = (t0 + KL + key < c1) ? t0 + KL + key : c1 - 1;
        kst[i] = *(const u32x4*)(kb0 + j * p.kst + part * 8);
        vst[i] = *(const u32x4*)(vb0 + j * p.vst + part * 8);
      }
    }
    if (computing) {
#pragma unroll
      for (int sub = 0; sub < KL / KT; ++sub)
        if (t0 + sub * KT < c1) compute_tile(t0 + sub * KT, sub * KT);
    }
  }

  if (!computing) return;
  float* blk = ws + ((size_t)(u * p.Tq + qt) * p.fwd_chunks + ch) * fwd_block_floats(p.RT, D);
  float* Ob = blk;
  _Float16* Vb = (_Float16*)(blk + (size_t)p.RT * D);
  float* Mb = blk + (size_t)p.RT * D + (size_t)p.RT * D / 2;
  float* M2b = Mb + p.RT;
  float* Lb = M2b + p.RT;
  int* Jb = (int*)(Lb + p.RT);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      float4 w4 = {o[db][4 * qq] * kPUnscale, o[db][4 * qq + 1] * kPUnscale, o[db][4 * qq + 2] * kPUnscale,
                   o[db][4 * qq + 3] * kPUnscale};
      *(float4*)&Ob[(size_t)row_t * D + 32 * db + 8 * qq + 4 * h] = w4;
      *(f16x4*)&Vb[(size_t)row_t * D + 32 * db + 8 * qq + 4 * h] =
          *(const f16x4*)&sm.vstar[row_t][32 * db + 8 * qq + 4 * h];
    }
  if (h == 0) {
    Mb[row_t] = m * p.c1;  // log2 units from here on
    M2b[row_t] = m2 * p.c1;
    Lb[row_t] = lrest * kPUnscale;
    Jb[row_t] = jst;
  }
}

template <int D>
__global__ __launch_bounds__(256) void fwd_combine_kernel(Dev p, const float* __restrict__ ws,
                                                          float* __restrict__ a, float* __restrict__ lse,
                                                          int32_t* __restrict__ jstar, float* __restrict__ dom) {
  constexpr int PER = D / 64;  // d-values per lane
  const int u = blockIdx.y;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= p.R) return;  // uniform per wave
  int l, s, g;
  unit_coords(p, u, l, s, g);
  const int64_t n = p.cu[s + 1] - p.cu[s];
  const int nch = (int)((n + p.fwd_chunk - 1) / p.fwd_chunk);
  const int qt = row / p.RT, row_t = row % p.RT;
  const size_t bf = fwd_block_floats(p.RT, D);
  auto block = [&](int c) { return ws + ((size_t)(u * p.Tq + qt) * p.fwd_chunks + c) * bf; };
  auto stat = [&](int c, int which) { return block(c) + (size_t)p.RT * D + (size_t)p.RT * D / 2 + which * p.RT + row_t; };

  // stat(c, 0) = m (max), 1 = m2 (max of the rest), 2 = l_rest (relative to m2), 3 = j*
  float M = -INFINITY;
  int win = -1;
  for (int c = 0; c < nch; ++c) {
    const float mc = *stat(c, 0);
    const int jc = *(const int*)stat(c, 3);
    if (jc >= 0 && mc > M) {
      M = mc;
      win = c;
    }
  }
  const size_t ro = (size_t)u * p.R + row;
  if (win < 0) {  // no visible key recorded (cannot happen for valid shapes: key 0 is always visible)
    for (int e = lane; e < D; e += 64) a[ro * D + e] = 0.f;
    if (lane == 0) {
      dom[ro] = 0.f;
      lse[ro] = -INFINITY;
      jstar[ro] = -1;
    }
    return;
  }
  float M2 = -INFINITY;  // max over every key but the global argmax
  for (int c = 0; c < nch; ++c) {
    if (*(const int*)stat(c, 3) < 0) continue;
    M2 = fmaxf(M2, *stat(c, 1));
    if (c != win) M2 = fmaxf(M2, *stat(c, 0));
  }
  float acc[PER], vs[PER];
  float lr = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  for (int c = 0; c < nch; ++c) {
    const int jc = *(const int*)stat(c, 3);
    if (jc < 0) continue;
    const float m2c = *stat(c, 1);
    const float w2 = (m2c == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m2c - M2);
    const float w1 = (c != win) ? __builtin_amdgcn_exp2f(*stat(c, 0) - M2) : 0.f;
    const float* Oc = block(c) + (size_t)row_t * D;
    const _Float16* Vc = (const _Float16*)(block(c) + (size_t)p.RT * D) + (size_t)row_t * D;
    lr += w2 * *stat(c, 2) + w1;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + 64 * i;
      const float vv = (float)Vc[e];
      acc[i] += w2 * Oc[e] + w1 * vv;
      if (c == win) vs[i] = vv;
    }
  }
  // p* = 1 / (1 + rel * lr), rel = exp2(M2 - M): the rest's total weight relative to the max
  const float rel = (M2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M2 - M);
  const float lt = rel * lr;
  const float pstar = 1.f / (1.f + lt);
  float d2 = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    a[ro * D + e] = (rel * acc[i] + vs[i]) * pstar;
    const float df = (lr > 0.f ? acc[i] / lr : vs[i]) - vs[i];
    d2 += df * df;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) d2 += __shfl_xor(d2, off, 64);
  if (lane == 0) {
    const float shift = pstar * sqrtf(d2);
    // the isolated pair's term in the call's score: its shift (L2), squared (SQ), or its
    // attention weight p* (attention sum)
    dom[ro] = (p.mode == 1) ? shift * shift : (p.mode == 2 ? pstar : shift);
    lse[ro] = (M + __log2f(1.f + lt)) * 0.69314718055994531f;
    jstar[ro] = *(const int*)stat(win, 3);
  }
}

}  // namespace

hipError_t launch_attn_fwd(const Dev& p, const void* q, const void* k, const void* v, float* a, float* lse,
                           int32_t* jstar, float* dom, void* ws, hipStream_t st) {
  const dim3 g1(p.fwd_chunks, p.Tq, p.U), g2((p.R + 3) / 4, p.U);
  if (p.d == 128) {
    hipLaunchKernelGGL(fwd_partial_kernel<128>, g1, dim3(NTHREADS), 0, st, p, (const __bf16*)q, (const __bf16*)k,
                       (const __bf16*)v, (float*)ws);
    hipLaunchKernelGGL(fwd_combine_kernel<128>, g2, dim3(256), 0, st, p, (const float*)ws, a, lse, jstar, dom);
  } else {
    hipLaunchKernelGGL(fwd_partial_kernel<64>, g1, dim3(NTHREADS), 0, st, p, (const __bf16*)q, (const __bf16*)k,
                       (const __bf16*)v, (float*)ws);
    hipLaunchKernelGGL(fwd_combine_kernel<64>, g2, dim3(256), 0, st, p, (const float*)ws, a, lse, jstar, dom);
  }
  return hipGetLastError();
}

}  // namespace kvs
