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
// Pass 1 (fwd_partial): grid (key chunk, query tile, unit). 8 waves, two per SIMD; a
// computing wave owns 32 rows, one row per lane (both half-waves hold the row). With query
// tiles of at most seven row blocks (G = 7: 224 rows) the HLP instance runs, in which the
// last wave, which has no rows, issues every DMA and converts every V tile in a loop of its
// own with the same barriers, and the computing waves only compute.
// S^T = K.Q^T on v_mfma_f32_32x32x16_bf16 and O^T += V^T.P^T on v_mfma_f32_32x32x16_f16.
// K/V tiles of 64 keys go from HBM straight into LDS (global_load_lds_dwordx4) through
// a ring of four buffers, three tiles in flight while one is computed; the 16-byte chunks
// of each row are XOR-swizzled with a function of the row so that the K operand reads
// (ds_read_b128) and the V^T transpose reads (ds_read_tr16_b64) are conflict-free. One
// tile ahead of its use, V is converted to fp16 in place (exact for |v| < 65504). P
// enters the product in fp16 (unit roundoff 2^-11, eight times finer than bf16: with
// few keys per row the rounding of P does not average out, and a^(-j*) feeds the
// isolated term), pre-scaled by 2^14 so probabilities down to ~4e-9 stay normal; the
// scale is folded into the exp2 argument and removed once at the end.
// Online softmax in the log2 domain; a row's two lanes exchange their maxima with
// v_permlane32_swap and keep their own halves of the row sums. When a row's running max
// moves to a key of the current tile, the previous argmax's value row (held in the lane's
// registers, weight 1 at the old max) is folded into the rest and the new one is read
// from the tile.
// Pass 2 (fwd_combine): one wave per row merges the chunks' (m, l_rest, acc_rest, j*,
// v*) in ascending chunk order and writes a, lse, j*, and the isolated term.
#include <type_traits>

#include "kvs_internal.hpp"

namespace kvs {
namespace {

constexpr int KT = 64;     // keys per tile
constexpr int NBUF = 4;    // tile ring: computed, next (converted to fp16 now), two in flight
constexpr int NWAVES = 8;  // 32 rows each
constexpr int NTHREADS = 64 * NWAVES;
static_assert(NWAVES * 32 == kRowsPerTileMax, "a workgroup covers one query tile");
constexpr float kPScale = 16384.f;     // 2^14: P is carried as 2^14 * p in the rest sums
constexpr float kPScaleLog2 = 14.f;
constexpr float kPUnscale = 1.f / 16384.f;
constexpr float kSlack = 1.5f;  // log2 units the rest's max may exceed its reference: 2^15.5 < fp16 max

template <int D>
struct FwdSmem {
  // [buffer][tensor K, V][key][D]: K in bf16, V in bf16 as it lands and fp16 once converted
  alignas(16) unsigned short tile[NBUF][2][KT * D];
};

// position of 16-byte chunk c of row r is c ^ swz(r).
// K (read as the A operand: 32 rows at one chunk index): sixteen consecutive rows hit
// sixteen different bank groups (D=64: eight rows within 128 bytes), swz(r + 32) = swz(r).
template <int D>
__device__ inline int swz_k(int r) {
  if constexpr (D == 128) return r & 15;
  else return (r & 7) ^ ((r >> 3) & 1);
}
// V (read transposed: a half-wave takes 4 consecutive rows r0..r0+3, r0 = 0 mod 4, at the
// 4 chunks 4b..4b+3): the rows' 64-byte groups must cover 256 distinct bytes of banks.
// D=128 rows are 256 bytes: rows differ in bits 2-3 of the chunk index. D=64 rows are 128
// bytes (rows r, r+2 share banks): rows r0 and r0+2 differ in bit 2.
template <int D>
__device__ inline int swz_v(int r) {
  if constexpr (D == 128) return (r & 3) << 2;
  else return ((r >> 1) & 1) << 2;
}


// wait until at most N of this wave's vector memory instructions are outstanding
template <int N>
__device__ inline void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// max over the two lanes of a row (lanes r and r + 32)
__device__ inline float row_max(float x) {
  const HalfPair v = wave_halves(x);
  return fmaxf(v.lo, v.hi);
}

template <int D, bool HLP>
__global__ __launch_bounds__(NTHREADS) void fwd_partial_kernel(Dev p, const __bf16* __restrict__ q,
                                                               const __bf16* __restrict__ k,
                                                               const __bf16* __restrict__ v, float* __restrict__ ws,
                                                               float* __restrict__ a_out, float* __restrict__ lse_out,
                                                               int32_t* __restrict__ jstar_out,
                                                               float* __restrict__ dom_out) {
  constexpr int NKK = D / 16;              // k-steps of the QK^T contraction
  constexpr int NDB = D / 32;              // 32-wide d blocks of O^T
  constexpr int CPK = D / 8;               // 16-byte chunks per row
  constexpr int RS = D * 2;                // bytes per row
  constexpr int IPT = KT * CPK / 64;       // DMA wave instructions per tensor tile
  constexpr int NLD = 2 * IPT / NWAVES;    // DMA instructions per wave per tile
  static_assert(IPT % NWAVES == 0 && (NLD == 2 || NLD == 4), "tile shape");
  __shared__ FwdSmem<D> sm;

  int ch, qt, u;
  xcd_item3(p, ch, qt, u);
  int l, s, g;
  unit_coords(p, u, l, s, g);
  const int64_t n = p.cu[s + 1] - p.cu[s];
  const int64_t c0 = (int64_t)ch * p.fwd_chunk;
  if (c0 >= n) return;  // uniform: this sequence has fewer chunks
  const int64_t c1 = (n < c0 + p.fwd_chunk) ? n : c0 + p.fwd_chunk;
  const int ntiles = (int)((c1 - c0 + KT - 1) / KT);

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const bool computing = wave * 32 < p.RT;
  const int row_t = wave * 32 + l32;
  const int row = qt * p.RT + row_t;
  const bool row_ok = computing && row < p.R;
  const int64_t tlim = row_ok ? n - p.W + (row % p.W) : n - 1;  // last key the row sees
  const int W = p.W;
  const float c1s = p.c1;
  const int64_t kst = p.kst, vst = p.vst;

  bf16x8 qf[NKK];
  {
    const __bf16* qrow = q + ((int64_t)u * p.R + (row_ok ? row : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      bf16x8 z = {};
      qf[kk] = row_ok ? *(const bf16x8*)(qrow + 16 * kk + 8 * h) : z;
    }
  }
  // retire the row operand loads here, where the compiler sees it: its wait tracking does not
  // see the DMA waits below and would otherwise wait for every load in flight inside the loop
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  float m = -INFINITY, m2 = -INFINITY, lrest = 0.f;
  int jst = -1;
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    o[db] = f32x16{};
  }
  // value row of the running argmax (fp16), the lane's dims 32db + 8qq + 4h + {0..3}
  f16x4 vs[NDB][4];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      vs[db][qq] = f16x4{};
    }

  const __bf16* kb0 = k + l * p.ksl + g * p.ksh + p.cu[s] * p.kst;
  const __bf16* vb0 = v + l * p.vsl + g * p.vsh + p.cu[s] * p.vst;

  // DMA of tile it into ring buffer it % NBUF. Wave instruction f (of NLD * NWAVES) fills
  // the 64 chunk positions 64(f % IPT) .. +63 of tensor f / IPT: position (row r, c')
  // takes chunk c' ^ swz(r) of row r. Keys past the chunk load its last row (in bounds,
  // unconditional); the tile that holds them is masked.
  constexpr int TBYTES = KT * D * 2;  // bytes per tensor tile
  const unsigned smb = lds_offset(&sm.tile[0][0][0]);
  auto issue = [&](int it) __attribute__((always_inline)) {
    const int64_t t0 = c0 + (int64_t)it * KT;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int f = i * NWAVES + wave;
      const int tensor = f / IPT, slot = (f % IPT) * 64 + lane;
      const int r = slot / CPK;
      const int c = (slot % CPK) ^ (tensor == 0 ? swz_k<D>(r) : swz_v<D>(r));
      const int rr = (t0 + r < c1) ? r : (int)(c1 - 1 - t0);  // rows past the chunk load its last
      const __bf16* base = tensor == 0 ? kb0 + t0 * kst : vb0 + t0 * vst;
      lds_dma16(base, (unsigned)(rr * (int)(tensor == 0 ? kst : vst) + 8 * c) * 2u,
                smb + (unsigned)(((it % NBUF) * 2 + tensor) * TBYTES + (f % IPT) * 1024));
    }
  };
  // the same for a tile inside the chunk, from lane byte offsets (from the tile's first row)
  // computed once
  unsigned doff[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int f = i * NWAVES + wave;
    const int tensor = f / IPT, slot = (f % IPT) * 64 + lane;
    const int r = slot / CPK;
    const int c = (slot % CPK) ^ (tensor == 0 ? swz_k<D>(r) : swz_v<D>(r));
    doff[i] = (unsigned)(r * (int)(tensor == 0 ? kst : vst) + 8 * c) * 2u;
  }
  auto issue_full = [&](int it) __attribute__((always_inline)) {
    const int64_t t0 = c0 + (int64_t)it * KT;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int f = i * NWAVES + wave;
      const __bf16* base = (f / IPT) == 0 ? kb0 + t0 * kst : vb0 + t0 * vst;
      lds_dma16(base, doff[i], smb + (unsigned)(((it % NBUF) * 2 + f / IPT) * TBYTES + (f % IPT) * 1024));
    }
  };
  // V of tile it from bf16 to fp16, in place: each lane converts the chunks its own DMA
  // instructions wrote, so it needs only its own loads to have landed
  // (instruction i of a wave moves V exactly when i >= NLD / 2: f = i * NWAVES + wave is
  // then in [IPT, 2 * IPT))
  auto convert_own = [&](int it) __attribute__((always_inline)) {
#pragma unroll
    for (int i = NLD / 2; i < NLD; ++i) {
      const int f = i * NWAVES + wave;
      u32x4* c = (u32x4*)&sm.tile[it % NBUF][1][((f % IPT) * 64 + lane) * 8];
      *c = bf16x8_to_f16x8(*c);
    }
  };
  // the same in two halves, so the LDS reads' latency passes under MFMAs in between
  u32x4 cvt[NLD / 2];
  auto convert_read = [&](int it) __attribute__((always_inline)) {
#pragma unroll
    for (int i = NLD / 2; i < NLD; ++i) {
      const int f = i * NWAVES + wave;
      cvt[i - NLD / 2] = *(const u32x4*)&sm.tile[it % NBUF][1][((f % IPT) * 64 + lane) * 8];
    }
  };
  auto convert_write = [&](int it) __attribute__((always_inline)) {
#pragma unroll
    for (int i = NLD / 2; i < NLD; ++i) {
      const int f = i * NWAVES + wave;
      *(u32x4*)&sm.tile[it % NBUF][1][((f % IPT) * 64 + lane) * 8] = bf16x8_to_f16x8(cvt[i - NLD / 2]);
    }
  };
  auto issue_any = [&](int it) __attribute__((always_inline)) {
    if (c0 + (int64_t)(it + 1) * KT <= c1) issue_full(it);
    else issue(it);
  };
  // instruction i of this wave's share of tile it, alone
  auto issue_one = [&](int it, auto ic) __attribute__((always_inline)) {
    constexpr int i = decltype(ic)::value;
    const int f = i * NWAVES + wave;
    const int tensor = f / IPT;
    const int64_t t0 = c0 + (int64_t)it * KT;
    const unsigned dst = smb + (unsigned)(((it % NBUF) * 2 + tensor) * TBYTES + (f % IPT) * 1024);
    const __bf16* base = tensor == 0 ? kb0 + t0 * kst : vb0 + t0 * vst;
    if (t0 + KT <= c1) {
      lds_dma16(base, doff[i], dst);
    } else {
      const int slot = (f % IPT) * 64 + lane;
      const int r = slot / CPK;
      const int c = (slot % CPK) ^ (tensor == 0 ? swz_k<D>(r) : swz_v<D>(r));
      const int rr = (t0 + r < c1) ? r : (int)(c1 - 1 - t0);
      lds_dma16(base, (unsigned)(rr * (int)(tensor == 0 ? kst : vst) + 8 * c) * 2u, dst);
    }
  };
  // byte offset of the lane's K operand chunk (key l32, slots 16kk + 8h .. +7)
  const int kbase = l32 * RS, khs = h ^ swz_k<D>(l32);
  auto koff = [&](int kk) __attribute__((always_inline)) { return kbase + (((2 * kk) ^ khs) << 4); };
  // V^T operand reads: lane reads 4 dims at key row 16ks + 4h + (lane%16)/4 (+8 for the
  // second half), dims 32db + 16((lane/16)%2) + 4(lane%4). Those rows share their low two
  // bits, so their swizzle is one lane constant that only permutes the 64-byte d blocks
  // (bits 2-3 of the chunk index): block db sits at lane base vtd[db], and ks, the second
  // half and the ring slot are constant offsets.
  int vtd[NDB];
  {
    const int r = 4 * h + ((lane & 15) >> 2);
    const int x = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);  // chunk within the 64-byte block
    const int sw = swz_v<D>(r) >> 2;
#pragma unroll
    for (int db = 0; db < NDB; ++db) vtd[db] = r * RS + ((4 * (db ^ sw) + x) << 4) + ((lane & 1) << 3);
  }
  // byte offset of element (key r, dim d), d a multiple of 4, in a V tile
  auto voff = [&](int r, int d) __attribute__((always_inline)) {
    return r * RS + ((((d >> 3) ^ swz_v<D>(r))) << 4) + ((d & 4) << 1);
  };

  // the 64 keys of ring tile it
  auto compute_tile = [&](const int it, auto&& hook) __attribute__((always_inline)) {
    const int64_t t0 = c0 + (int64_t)it * KT;
    const char* kt = (const char*)sm.tile[it % NBUF][0];
    const char* vt = (const char*)sm.tile[it % NBUF][1];
    // ---- S^T = K Q^T for both 32-key blocks (chains interleaved): lane holds row l32 and,
    // at element r of block kb, key 32kb + 8(r/4) + 4h + (r%4). Values stay raw q.k; the
    // softmax scale enters through one FMA in front of exp2.
    // operands one k-step ahead of their MFMAs (the scheduling barriers keep the compiler
    // from loading all of them up front, which would cost 64 registers)
    f32x16 acc0 = {}, acc1 = {};
    bf16x8 k0 = *(const bf16x8*)(kt + koff(0));
    bf16x8 k1 = *(const bf16x8*)(kt + 32 * RS + koff(0));
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      bf16x8 k0n = k0, k1n = k1;
      if (kk + 1 < NKK) {
        k0n = *(const bf16x8*)(kt + koff(kk + 1));
        k1n = *(const bf16x8*)(kt + 32 * RS + koff(kk + 1));
      }
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[kk], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[kk], acc1, 0, 0, 0);
      if (kk == 0) hook(std::integral_constant<int, 0>{});
      if (kk == 1) hook(std::integral_constant<int, 5>{});
      if (kk == NKK / 2) hook(std::integral_constant<int, 1>{});
      __builtin_amdgcn_sched_barrier(0);
      k0 = k0n;
      k1 = k1n;
    }
    hook(std::integral_constant<int, 2>{});
    float tv[32];  // element e = 16*kb + r
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      tv[r] = acc0[r];
      tv[16 + r] = acc1[r];
    }
    const int trel = (int)(t0 - c0);  // tile start relative to the chunk
    if ((t0 + KT - 1 > n - W) || (t0 + KT > c1)) {
      const int lim = (int)((tlim < c1 - 1 ? tlim : c1 - 1) - c0);  // last key this row may use, chunk-relative
#pragma unroll
      for (int e = 0; e < 32; ++e)
        if (trel + 32 * (e >> 4) + 8 * ((e & 15) >> 2) + 4 * h + (e & 3) > lim) tv[e] = -INFINITY;
    }
    float lm = tv[0];
#pragma unroll
    for (int e = 1; e < 32; ++e) lm = fmaxf(lm, tv[e]);
    const float mt = row_max(lm);

    // Row state (raw q.k units): m = running max (key jst, value row in vs); m2 = the
    // reference of the rest sums lrest / o, within kSlack log2 units of the running max
    // over every other key (never below it by more, never above it), so a dominant key
    // never pushes the rest out of fp16's range and a rescale is needed only when the rest's
    // max climbs past the slack.
    const bool moved = mt > m;
    const bool any_moved = __any(moved);
    int jr = -1;          // this lane's element index of the new argmax, if it holds it
    int jt = 0x7fffffff;  // chunk-relative key of the new argmax
    float cand = mt;      // max over the keys that join the rest in this tile
    if (any_moved) {
      // an opaque copy of the tile max keeps the search below inside this (rarely taken)
      // branch instead of being hoisted onto every tile
      float mtv = mt;
      asm volatile("" : "+v"(mtv));
      int jl = 64;
      if (moved) {
        // elements run in key order within a lane: the first equal to mt is the lane's lowest key
#pragma unroll
        for (int e = 31; e >= 0; --e) jl = (tv[e] == mtv) ? e : jl;
      }
      const int keyl = (jl < 64) ? trel + 32 * (jl >> 4) + 8 * ((jl & 15) >> 2) + 4 * h + (jl & 3) : 0x7fffffff;
      jt = wave_halves_min(keyl);
      jr = (moved && keyl == jt) ? jl : -1;
      // the new argmax stays out of P: its logit becomes -inf (p = 0) in the lane holding it
#pragma unroll
      for (int e = 0; e < 32; ++e) tv[e] = (e == jr) ? -INFINITY : tv[e];
      // tile max without the new argmax (the lane holding it lost that element above)
      float l2 = tv[0];
#pragma unroll
      for (int e = 1; e < 32; ++e) l2 = fmaxf(l2, tv[e]);
      const float mt2 = row_max(moved ? l2 : -INFINITY);
      if (moved) cand = fmaxf(m, mt2);  // the old max joins the rest when it moves
    }
    const bool upd = cand * c1s > m2 * c1s + kSlack;  // -inf references always move
    const float m2n = upd ? cand : m2;
    const bool fold = moved && jst >= 0;  // the previous argmax joins the rest
    if (__any(upd) || any_moved) {
      // o = alpha o + wold v*: the rescale to the new reference and the old argmax's value
      // row with weight exp2(c1 (m - m2n)) (2^14 scaled), in one pass over the accumulators
      const float alpha = upd ? ((m2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m2 - m2n) * c1s)) : 1.f;
      const float wold = fold ? kPScale * __builtin_amdgcn_exp2f((m - m2n) * c1s) : 0.f;
      lrest = fmaf(lrest, alpha, h == 0 ? wold : 0.f);  // the lane's half of the row sum
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
#pragma unroll
          for (int e = 0; e < 4; ++e) o[db][4 * qq + e] = fmaf((float)vs[db][qq][e], wold, o[db][4 * qq + e] * alpha);
      }
      if (moved) {
        const int jslot = jt - trel;  // new argmax's key in this tile
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            vs[db][qq] = *(const f16x4*)(vt + voff(jslot, 32 * db + 8 * qq + 4 * h));
          }
        jst = (int)c0 + jt;
        m = mt;
      }
    }
    m2 = m2n;
    const float mb = ((m2n == -INFINITY) ? 0.f : m2n * c1s) - kPScaleLog2;
    float pr[32];  // 2^14 * exp2(c1 * (s - m2n)) <= 2^(14 + kSlack); the new argmax excluded
#pragma unroll
    for (int e = 0; e < 32; ++e) pr[e] = __builtin_amdgcn_exp2f(fmaf(tv[e], c1s, -mb));

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
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const char* a0 = vt + vtd[db] + 16 * ks * RS;
        const char* a1 = a0 + 8 * RS;
        const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a0);
        const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a1);
        // whole-vector casts: per-element bit casts of the loaded i16x4 were lowered to a
        // broadcast of element 0
        const f16x8 vf = __builtin_shufflevector(__builtin_bit_cast(f16x4, r0), __builtin_bit_cast(f16x4, r1), 0, 1,
                                                 2, 3, 4, 5, 6, 7);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf, o[db], 0, 0, 0);
      }
      if (ks == 1) hook(std::integral_constant<int, 3>{});
      if (ks == 3) hook(std::integral_constant<int, 4>{});
    }
    lrest += ts;
  };

  // Ring schedule (one barrier per tile). Iteration t: after the barrier, buffer (t+3)%4
  // (last read by tile t-1) takes tile t+3, tile t is computed, and each lane waits for its
  // own loads of tile t+1 (tiles t+2 and the part of t+3 issued so far stay in flight) and
  // converts its share of that tile's V, which the next barrier publishes. Three tiles are
  // in flight while one is computed. A computing wave spreads its DMA instructions over
  // the tile's MFMA phases (half with the S^T chain, half with the O^T chain): issued all
  // at once by every wave they back up in the address unit. It reads its V share of tile
  // t+1 at the second k-step of the S^T chain and writes it back converted after the
  // chain, so the LDS round trip runs under the MFMAs.
  if constexpr (HLP) {
    // Query tiles of at most seven row blocks (G = 7: 224 rows): the waves without rows
    // leave the computing waves no DMA and no conversion. The last of them issues every
    // DMA instruction of a tile and converts the whole V tile to fp16, in a loop of its own
    // with the same barriers; any other row-less wave only keeps the barriers. One wave
    // keeps two tiles of DMA in flight, and at most 63 vector memory operations may be
    // outstanding: each wait below leaves room for the next tile's NLDH.
    if (!computing) {
      if (wave == NWAVES - 1) {
        constexpr int NLDH = NLD * NWAVES;
        constexpr int HW = (NLDH < 63 - NLDH) ? NLDH : 63 - NLDH;
        unsigned off[NLDH];
#pragma unroll
        for (int f = 0; f < NLDH; ++f) {
          const int tensor = f / IPT, slot = (f % IPT) * 64 + lane;
          const int r = slot / CPK;
          const int c = (slot % CPK) ^ (tensor == 0 ? swz_k<D>(r) : swz_v<D>(r));
          off[f] = (unsigned)(r * (int)(tensor == 0 ? kst : vst) + 8 * c) * 2u;
        }
        auto issue_h = [&](int it) __attribute__((always_inline)) {
          const int64_t t0 = c0 + (int64_t)it * KT;
          const bool full = t0 + KT <= c1;
#pragma unroll
          for (int f = 0; f < NLDH; ++f) {
            const int tensor = f / IPT;
            const __bf16* base = tensor == 0 ? kb0 + t0 * kst : vb0 + t0 * vst;
            unsigned o = off[f];
            if (!full) {
              const int slot = (f % IPT) * 64 + lane;
              const int r = slot / CPK;
              const int c = (slot % CPK) ^ (tensor == 0 ? swz_k<D>(r) : swz_v<D>(r));
              const int rr = (t0 + r < c1) ? r : (int)(c1 - 1 - t0);  // rows past the chunk load its last
              o = (unsigned)(rr * (int)(tensor == 0 ? kst : vst) + 8 * c) * 2u;
            }
            lds_dma16(base, o, smb + (unsigned)(((it % NBUF) * 2 + tensor) * TBYTES + (f % IPT) * 1024));
          }
        };
        // every 16-byte chunk of the V tile, in place, four at a time
        auto convert_all = [&](int it) __attribute__((always_inline)) {
#pragma unroll
          for (int b = 0; b < IPT; b += 4) {
            u32x4 w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = *(const u32x4*)&sm.tile[it % NBUF][1][((b + e) * 64 + lane) * 8];
#pragma unroll
            for (int e = 0; e < 4; ++e) *(u32x4*)&sm.tile[it % NBUF][1][((b + e) * 64 + lane) * 8] = bf16x8_to_f16x8(w[e]);
          }
        };
        issue_h(0);
        if (ntiles > 1) {
          vm_wait<HW>();
          issue_h(1);
        }
        if (ntiles > 2) {
          vm_wait<HW>();  // tile 0 has landed
          issue_h(2);
        } else if (ntiles > 1) {
          vm_wait<NLDH>();
        } else {
          vm_wait<0>();
        }
        convert_all(0);
        for (int t = 0; t < ntiles; ++t) {
          __syncthreads();
          if (t + 1 < ntiles) {  // tile t+1 has landed once at most HW (t+2's) remain
            if (t + 2 < ntiles) vm_wait<HW>();
            else vm_wait<0>();
          }
          if (t + 3 < ntiles) issue_h(t + 3);
          if (t + 1 < ntiles) convert_all(t + 1);
        }
      } else {
        for (int t = 0; t < ntiles; ++t) __syncthreads();
      }
      return;
    }
  } else {
    issue(0);
    if (ntiles > 1) issue_any(1);
    if (ntiles > 2) issue_any(2);
  }
  if constexpr (HLP) {
    // tile 0 comes from the helper: the loop's first barrier publishes it
  } else if (ntiles > 2) vm_wait<2 * NLD>();
  else if (ntiles > 1) vm_wait<NLD>();
  else vm_wait<0>();
  if constexpr (!HLP) convert_own(0);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
    const bool more3 = t + 3 < ntiles, more2 = t + 2 < ntiles, more1 = t + 1 < ntiles;
    auto wait_convert_next = [&](auto later3) __attribute__((always_inline)) {
      if (!more1) return;
      if (more3) vm_wait<NLD + decltype(later3)::value>();
      else if (more2) vm_wait<NLD>();
      else vm_wait<0>();
      convert_own(t + 1);
    };
    if (computing) {
      compute_tile(t, [&](auto pc) __attribute__((always_inline)) {
        // 0, 5, 1: S^T chain (k-steps 0, 1, NKK/2); 2: after it; 3, 4: O^T chain
        constexpr int point = decltype(pc)::value;
        if constexpr (HLP) {
          // the helper wave streams and converts the tiles
        } else if constexpr (point == 5) {
          // this lane's loads of tile t+1 (t+2 and the one instruction of t+3 issued at
          // point 0 may stay in flight), then its share of that tile's V read for conversion
          if (more1) {
            if (more3) vm_wait<NLD + 1>();
            else if (more2) vm_wait<NLD>();
            else vm_wait<0>();
            convert_read(t + 1);
          }
        } else if constexpr (point == 2) {
          if (more1) convert_write(t + 1);
        } else if (more3) {
          if constexpr (NLD == 4) {
            constexpr int i = point < 2 ? point : point - 1;
            issue_one(t + 3, std::integral_constant<int, i>{});
          } else if constexpr (point == 0 || point == 3) {
            issue_one(t + 3, std::integral_constant<int, point == 0 ? 0 : 1>{});
          }
        }
      });
    } else {
      if (more3) issue_any(t + 3);
      wait_convert_next(std::integral_constant<int, NLD>{});
    }
  }

  if (!computing) return;
  const HalfPair lp = wave_halves(lrest);  // the row's two half sums
  lrest = lp.lo + lp.hi;
  if (n <= p.fwd_chunk) {
    // the sequence is one chunk: this workgroup saw every key of its rows, so it writes the
    // outputs itself (the one-chunk case of fwd_combine, whose record it would otherwise
    // write and which then skips these rows)
    if (!row_ok) return;
    const size_t ro = (size_t)u * p.R + row;
    float* arow = a_out + ro * D;
    if (jst < 0) {  // no visible key recorded (cannot happen for valid shapes: key 0 is always visible)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) *(float4*)&arow[32 * db + 8 * qq + 4 * h] = float4{0.f, 0.f, 0.f, 0.f};
      if (h == 0) {
        dom_out[ro] = 0.f;
        lse_out[ro] = -INFINITY;
        jstar_out[ro] = -1;
      }
      return;
    }
    const float M = m * c1s, M2 = m2 * c1s, lr = lrest * kPUnscale;  // log2 units
    const float w2 = (M2 == -INFINITY) ? 0.f : 1.f;
    const float lrs = w2 * lr;
    const float rel = (M2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M2 - M);
    const float lt = rel * lrs;
    const float pstar = 1.f / (1.f + lt);
    float d2 = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        float4 w4;
        float* wv = (float*)&w4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float acc = w2 * (o[db][4 * qq + e] * kPUnscale), vv = (float)vs[db][qq][e];
          wv[e] = (rel * acc + vv) * pstar;
          const float df = (lrs > 0.f ? acc / lrs : vv) - vv;
          d2 += df * df;
        }
        *(float4*)&arow[32 * db + 8 * qq + 4 * h] = w4;
      }
    const HalfPair dp = wave_halves(d2);
    if (h == 0) {
      const float shift = pstar * sqrtf(dp.lo + dp.hi);
      // the isolated pair's term in the call's score: its shift (L2), squared (SQ), or its
      // attention weight p* (attention sum)
      dom_out[ro] = (p.mode == 1) ? shift * shift : (p.mode == 2 ? pstar : shift);
      lse_out[ro] = (M + __log2f(1.f + lt)) * 0.69314718055994531f;
      jstar_out[ro] = jst;
    }
    return;
  }
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
      *(f16x4*)&Vb[(size_t)row_t * D + 32 * db + 8 * qq + 4 * h] = vs[db][qq];
    }
  if (h == 0) {
    Mb[row_t] = m * c1s;  // log2 units from here on
    M2b[row_t] = m2 * c1s;
    Lb[row_t] = lrest * kPUnscale;
    Jb[row_t] = jst;
  }
}

// A row's outputs from its merged records: acc = the rest's weighted sum and lr its weight
// (both relative to M2, the max over every key but the argmax), vs the argmax's value row.
// p* = 1 / (1 + rel * lr), rel = exp2(M2 - M): the rest's total weight relative to the max.
template <int PER>
__device__ __attribute__((always_inline)) void combine_out(const Dev& p, float* __restrict__ a,
                                                           float* __restrict__ lse, int32_t* __restrict__ jstar,
                                                           float* __restrict__ dom, size_t ro, int lane, float M,
                                                           float M2, float lr, const float (&acc)[PER],
                                                           const float (&vs)[PER], int jwin) {
  constexpr int D = 64 * PER;
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
    jstar[ro] = jwin;
  }
}

// CM > 0: a row's records from at most CM chunks (the launch picks CM from the largest
// chunk count) all loaded at once; CM = 0: one chunk at a time, any count
template <int D, int CM>
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
  const size_t ro = (size_t)u * p.R + row;
  if (nch == 1) return;  // uniform: fwd_partial wrote this row's outputs
  // every chunk's statistics and row loaded at once (one memory latency instead of one per
  // chunk and pass), then the same arithmetic in the same order as the loop below
  if constexpr (CM > 0) {
    float mc[CM], m2c[CM], lc[CM], oc[CM][PER], vc[CM][PER];
    int jc[CM];
#pragma unroll
    for (int c = 0; c < CM; ++c) {
      mc[c] = m2c[c] = -INFINITY;
      lc[c] = 0.f;
      jc[c] = -1;
#pragma unroll
      for (int i = 0; i < PER; ++i) oc[c][i] = vc[c][i] = 0.f;
      if (c < nch) {  // uniform
        mc[c] = *stat(c, 0);
        m2c[c] = *stat(c, 1);
        lc[c] = *stat(c, 2);
        jc[c] = *(const int*)stat(c, 3);
        const float* Oc = block(c) + (size_t)row_t * D;
        const _Float16* Vc = (const _Float16*)(block(c) + (size_t)p.RT * D) + (size_t)row_t * D;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          oc[c][i] = Oc[lane + 64 * i];
          vc[c][i] = (float)Vc[lane + 64 * i];
        }
      }
    }
    float M = -INFINITY;
    int win = -1;
#pragma unroll
    for (int c = 0; c < CM; ++c)
      if (jc[c] >= 0 && mc[c] > M) {
        M = mc[c];
        win = c;
      }
    if (win < 0) {  // no visible key recorded (cannot happen for valid shapes: key 0 is always visible)
      for (int e = lane; e < D; e += 64) a[ro * D + e] = 0.f;
      if (lane == 0) {
        dom[ro] = 0.f;
        lse[ro] = -INFINITY;
        jstar[ro] = -1;
      }
      return;
    }
    float M2 = -INFINITY;
#pragma unroll
    for (int c = 0; c < CM; ++c) {
      if (jc[c] < 0) continue;
      M2 = fmaxf(M2, m2c[c]);
      if (c != win) M2 = fmaxf(M2, mc[c]);
    }
    float acc[PER], vs[PER];
    float lr = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      acc[i] = 0.f;
      vs[i] = 0.f;
    }
#pragma unroll
    for (int c = 0; c < CM; ++c) {
      if (jc[c] < 0) continue;
      const float w2 = (m2c[c] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m2c[c] - M2);
      const float w1 = (c != win) ? __builtin_amdgcn_exp2f(mc[c] - M2) : 0.f;
      lr += w2 * lc[c] + w1;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        acc[i] += w2 * oc[c][i] + w1 * vc[c][i];
        if (c == win) vs[i] = vc[c][i];
      }
    }
    combine_out(p, a, lse, jstar, dom, ro, lane, M, M2, lr, acc, vs, jc[win]);
    return;
  } else {
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
  combine_out(p, a, lse, jstar, dom, ro, lane, M, M2, lr, acc, vs, *(const int*)stat(win, 3));
  }
}

}  // namespace

hipError_t launch_attn_fwd(const Dev& p, const void* q, const void* k, const void* v, float* a, float* lse,
                           int32_t* jstar, float* dom, void* ws, hipStream_t st) {
  const dim3 g1(p.fwd_chunks, p.Tq, p.U), g2((p.R + 3) / 4, p.U);
  // query tiles of at most seven row blocks leave a wave without rows: it takes the streaming
  const bool hlp = p.RT <= kRowsPerTileMax - 32;
  if (p.d == 128) {
    if (hlp)
      hipLaunchKernelGGL((fwd_partial_kernel<128, true>), g1, dim3(NTHREADS), 0, st, p, (const __bf16*)q,
                         (const __bf16*)k, (const __bf16*)v, (float*)ws, a, lse, jstar, dom);
    else
      hipLaunchKernelGGL((fwd_partial_kernel<128, false>), g1, dim3(NTHREADS), 0, st, p, (const __bf16*)q,
                         (const __bf16*)k, (const __bf16*)v, (float*)ws, a, lse, jstar, dom);
    if (p.fwd_chunks > 8)
      hipLaunchKernelGGL((fwd_combine_kernel<128, 0>), g2, dim3(256), 0, st, p, (const float*)ws, a, lse, jstar, dom);
    else if (p.fwd_chunks > 4)
      hipLaunchKernelGGL((fwd_combine_kernel<128, 8>), g2, dim3(256), 0, st, p, (const float*)ws, a, lse, jstar, dom);
    else if (p.fwd_chunks > 1)
      hipLaunchKernelGGL((fwd_combine_kernel<128, 4>), g2, dim3(256), 0, st, p, (const float*)ws, a, lse, jstar, dom);
  } else {
    if (hlp)
      hipLaunchKernelGGL((fwd_partial_kernel<64, true>), g1, dim3(NTHREADS), 0, st, p, (const __bf16*)q,
                         (const __bf16*)k, (const __bf16*)v, (float*)ws, a, lse, jstar, dom);
    else
      hipLaunchKernelGGL((fwd_partial_kernel<64, false>), g1, dim3(NTHREADS), 0, st, p, (const __bf16*)q,
                         (const __bf16*)k, (const __bf16*)v, (float*)ws, a, lse, jstar, dom);
    if (p.fwd_chunks > 8)
      hipLaunchKernelGGL((fwd_combine_kernel<64, 0>), g2, dim3(256), 0, st, p, (const float*)ws, a, lse, jstar, dom);
    else if (p.fwd_chunks > 4)
      hipLaunchKernelGGL((fwd_combine_kernel<64, 8>), g2, dim3(256), 0, st, p, (const float*)ws, a, lse, jstar, dom);
    else if (p.fwd_chunks > 1)
      hipLaunchKernelGGL((fwd_combine_kernel<64, 4>), g2, dim3(256), 0, st, p, (const float*)ws, a, lse, jstar, dom);
  }
  return hipGetLastError();
}

}  // namespace kvs
