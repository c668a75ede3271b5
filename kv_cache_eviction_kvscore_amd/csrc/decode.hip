// Decode attention over the packed ragged cache.
//
// RippleKV page, "Problem Formulation": during decoding every new query attends to the
// cached states, after compression the (k, v) pairs at the retained positions (Eq. 4);
// GraceKV page, physical cache packing: every (layer, KV head) keeps a cache of its own
// length. Query head h = g*G + hl of (layer l, sequence s) attends to every row of
// segment u = (l*S + s)*Hkv + g: out = softmax(scale * K q) V, lse = log sum exp.
//
// The pass reads each packed K/V row once and does a few flops per byte, so it is bound
// by HBM, not by the matrix cores; it runs on the VALU:
// decode_partial: grid (key split, unit), 4 waves. A group of D/8 lanes shares one key
//   row, a lane owns 8 of its dims, so one wave load moves 64/(D/8) consecutive rows
//   (1 KB, coalesced; nontemporal, as a call reads each cached row once). q.k for the G
//   heads of the group is a v_dot2_f32_bf16 chain on the lane's 8 dims plus a DPP
//   reduction over the group. Every group runs its own online softmax over a strided
//   subset of the split's keys (fp32 accumulators, log2 domain; the running max is only
//   moved when a logit exceeds it by more than 8, so the rescale is rare), then the groups
//   merge in the wave (shuffles) and the waves in LDS, in a fixed order. The split's
//   (max, sum, sum p v) per head go to the workspace.
// decode_combine: one wave per (unit, head) merges the splits in ascending order.
//
// Fixed scratch (kvscore_decode_attn_noalloc): the split records live in the file-scope
// array `scratch` instead of a caller workspace. Each GPU the library runs on holds its
// own copy of the array until the process ends. Host code never passes the array's name
// to a kernel (on the host it is only a stand-in for the device symbol): the device
// address comes from hipGetSymbolAddress, once per device, with that device current.
#include <mutex>
#include <type_traits>

#include "kvs_internal.hpp"

namespace kvs {
namespace {

static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

constexpr int NWAVES = 4;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int UNROLL = 4;        // key steps in flight per lane
constexpr float kSlack = 8.f;    // log2 units a logit may exceed the running max before a rescale

__device__ inline float bf16lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ inline float bf16hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

template <int D, int G>
__global__ __launch_bounds__(NTHREADS) void decode_partial_kernel(DecDev p, const __bf16* __restrict__ q,
                                                                  const __bf16* __restrict__ kc,
                                                                  const __bf16* __restrict__ vc,
                                                                  const int64_t* __restrict__ off,
                                                                  float* __restrict__ ws) {
  constexpr int LPK = D / 8;        // lanes per key row
  constexpr int KPS = 64 / LPK;     // keys per wave step
  constexpr int NSTREAM = NWAVES * KPS;
  constexpr int REC = D + 2;        // floats per head in a split record: m, l, acc[D]
  __shared__ float red[NWAVES][G][REC];

  const int u = blockIdx.y, sp = blockIdx.x;
  const int64_t a0 = off[u], len = off[u + 1] - a0;
  const int64_t k0 = (int64_t)sp * p.chunk;
  if (k0 >= len) return;  // uniform: this segment has fewer splits
  const int nk = (int)((len - k0 < p.chunk) ? len - k0 : p.chunk);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ks = lane / LPK, dc = lane % LPK;  // key slot of the lane's group, its 16-byte chunk
  const int stream = wave * KPS + ks;
  // unit -> (l, s, g); query rows of the group's heads
  const int g = u % p.Hkv, ls = u / p.Hkv;  // ls = l*S + s
  const __bf16* qb = q + ((int64_t)ls * p.Hq + (int64_t)g * G) * D + 8 * dc;
  unsigned qw[G][4];  // the lane's 8 dims of every head, as bf16 pairs
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const u32x4 w = *(const u32x4*)(qb + (int64_t)h * D);
#pragma unroll
    for (int i = 0; i < 4; ++i) qw[h][i] = w[i];
  }
  const float c1 = p.c1;
  float m[G], lsum[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
  }
  const __bf16* kb = kc + (a0 + k0) * D + 8 * dc;
  const __bf16* vb = vc + (a0 + k0) * D + 8 * dc;

  // stream `stream` takes keys stream, stream + NSTREAM, ... of the split. A block of R of
  // its keys at a time: the R * G logits first (independent chains), one wave-wide test for
  // a reference move over all of them (with the block's maximum per head), then the
  // weights and the value sums in key order.
  auto block = [&](auto rc, const u32x4* kx, const u32x4* vx) __attribute__((always_inline)) {
    constexpr int R = decltype(rc)::value;
    float x[R][G];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float dsum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const unsigned kw = kx[r][i];
          dsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[h][i]), __builtin_bit_cast(bf16x2, kw),
                                                 dsum, false);
        }
        x[r][h] = group_sum<LPK>(dsum) * c1;  // log2 units
      }
    bool need = false;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int h = 0; h < G; ++h) need |= x[r][h] > m[h] + kSlack;
    if (__any(need)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float xm = x[0][h];
#pragma unroll
        for (int r = 1; r < R; ++r) xm = fmaxf(xm, x[r][h]);
        const bool mv = xm > m[h] + kSlack;
        const float alpha = mv ? __builtin_amdgcn_exp2f(m[h] - xm) : 1.f;  // exp2(-inf) = 0 at the start
        m[h] = mv ? xm : m[h];
        lsum[h] *= alpha;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] *= alpha;
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float vf[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const unsigned vw = vx[r][i];
        vf[2 * i] = bf16lo(vw);
        vf[2 * i + 1] = bf16hi(vw);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pr = __builtin_amdgcn_exp2f(x[r][h] - m[h]);  // <= 2^kSlack
        lsum[h] += pr;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] = fmaf(pr, vf[i], acc[h][i]);
      }
    }
  };

  const int nsteps = (nk - stream + NSTREAM - 1) / NSTREAM;  // keys of this stream (<= 0: none)
  int j = stream;
  int it = 0;
  for (; it + UNROLL <= nsteps; it += UNROLL) {
    u32x4 kx[UNROLL], vx[UNROLL];
#pragma unroll
    for (int r = 0; r < UNROLL; ++r) {
      kx[r] = __builtin_nontemporal_load((const u32x4*)(kb + (int64_t)(j + r * NSTREAM) * D));
      vx[r] = __builtin_nontemporal_load((const u32x4*)(vb + (int64_t)(j + r * NSTREAM) * D));
    }
    block(std::integral_constant<int, UNROLL>{}, kx, vx);
    j += UNROLL * NSTREAM;
  }
  for (; it < nsteps; ++it, j += NSTREAM) {
    const u32x4 kx = __builtin_nontemporal_load((const u32x4*)(kb + (int64_t)j * D));
    const u32x4 vx = __builtin_nontemporal_load((const u32x4*)(vb + (int64_t)j * D));
    block(std::integral_constant<int, 1>{}, &kx, &vx);
  }

  // merge the streams: first the KPS groups of the wave (lanes dc + LPK*ks), ascending
  // stream order by a butterfly whose partners are fixed, then the waves in LDS
  auto merge = [&](float& ma, float& la, float* aa, float mb, float lb, const float* ab) __attribute__((always_inline)) {
    const float mm = fmaxf(ma, mb);
    const float wa = (ma == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ma - mm);
    const float wb = (mb == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mb - mm);
    la = la * wa + lb * wb;
#pragma unroll
    for (int i = 0; i < 8; ++i) aa[i] = aa[i] * wa + ab[i] * wb;
    ma = mm;
  };
#pragma unroll
  for (int sh = LPK; sh < 64; sh <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mb = __shfl_xor(m[h], sh, 64), lb = __shfl_xor(lsum[h], sh, 64);
      float ab[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) ab[i] = __shfl_xor(acc[h][i], sh, 64);
      // both partners compute the same merge in the same operand order (lower stream first)
      if ((lane & sh) == 0) merge(m[h], lsum[h], acc[h], mb, lb, ab);
      else {
        float mo = mb, lo = lb, ao[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) ao[i] = ab[i];
        merge(mo, lo, ao, m[h], lsum[h], acc[h]);
        m[h] = mo;
        lsum[h] = lo;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] = ao[i];
      }
    }
  }
  if (ks == 0) {  // lanes 0 .. LPK-1 hold the wave's merge
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int i = 0; i < 8; ++i) red[wave][h][2 + 8 * dc + i] = acc[h][i];
      if (dc == 0) {
        red[wave][h][0] = m[h];
        red[wave][h][1] = lsum[h];
      }
    }
  }
  __syncthreads();
  // waves in ascending order; thread t handles (head, dim) pairs t, t + NTHREADS, ...
  float* rec = ws + ((int64_t)u * p.nsplit + sp) * G * REC;
  for (int e = tid; e < G * (D + 1); e += NTHREADS) {
    const int h = e / (D + 1), c = e % (D + 1);  // c = D: the (m, l) pair
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) mm = fmaxf(mm, red[w][h][0]);
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) {
      const float mw = red[w][h][0];
      const float wt = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - mm);
      tot += wt * (c < D ? red[w][h][2 + c] : red[w][h][1]);
    }
    if (c < D) rec[h * REC + 2 + c] = tot;
    else {
      rec[h * REC + 0] = mm;
      rec[h * REC + 1] = tot;
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecDev p, const int64_t* __restrict__ off,
                                                             const float* __restrict__ ws, float* __restrict__ out,
                                                             float* __restrict__ lse) {
  constexpr int PER = D / 64;
  constexpr int REC = D + 2;
  const int u = blockIdx.y;
  const int hl = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (hl >= p.G) return;  // uniform per wave
  const int64_t len = off[u + 1] - off[u];
  const int ns = (int)((len + p.chunk - 1) / p.chunk);
  const int g = u % p.Hkv, ls = u / p.Hkv;
  const float* rec = ws + (int64_t)u * p.nsplit * p.G * REC + (int64_t)hl * REC;
  float mm = -INFINITY;
  for (int sp = 0; sp < ns; ++sp) mm = fmaxf(mm, rec[(int64_t)sp * p.G * REC]);
  float tot = 0.f, o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = 0.f;
  for (int sp = 0; sp < ns; ++sp) {
    const float* r = rec + (int64_t)sp * p.G * REC;
    const float wt = __builtin_amdgcn_exp2f(r[0] - mm);
    tot += wt * r[1];
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] += wt * r[2 + lane + 64 * i];
  }
  const int64_t row = (int64_t)ls * p.Hq + (int64_t)g * p.G + hl;
  const float inv = 1.f / tot;
#pragma unroll
  for (int i = 0; i < PER; ++i) out[row * D + lane + 64 * i] = o[i] * inv;
  if (lane == 0) lse[row] = (mm + __log2f(tot)) * 0.69314718055994531f;
}

template <int D, int G>
void launch_partial(const DecDev& p, const __bf16* q, const __bf16* k, const __bf16* v, const int64_t* off, float* ws,
                    hipStream_t st) {
  hipLaunchKernelGGL((decode_partial_kernel<D, G>), dim3(p.nsplit, p.U), dim3(NTHREADS), 0, st, p, q, k, v, off, ws);
}

template <int D>
void launch_partial_g(const DecDev& p, const __bf16* q, const __bf16* k, const __bf16* v, const int64_t* off, float* ws,
                      hipStream_t st) {
  switch (p.G) {
    case 1: launch_partial<D, 1>(p, q, k, v, off, ws, st); break;
    case 2: launch_partial<D, 2>(p, q, k, v, off, ws, st); break;
    case 3: launch_partial<D, 3>(p, q, k, v, off, ws, st); break;
    case 4: launch_partial<D, 4>(p, q, k, v, off, ws, st); break;
    case 5: launch_partial<D, 5>(p, q, k, v, off, ws, st); break;
    case 6: launch_partial<D, 6>(p, q, k, v, off, ws, st); break;
    case 7: launch_partial<D, 7>(p, q, k, v, off, ws, st); break;
    default: launch_partial<D, 8>(p, q, k, v, off, ws, st); break;
  }
}

}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecDev& p, const void* q, const void* k, const void* v, const int64_t* off, float* out,
                         float* lse, void* ws, hipStream_t st) {
  const dim3 gc((unsigned)((p.G + 3) / 4), p.U);
  if (p.d == 128) {
    launch_partial_g<128>(p, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, off, (float*)ws, st);
    hipLaunchKernelGGL(decode_combine_kernel<128>, gc, dim3(256), 0, st, p, off, (const float*)ws, out, lse);
  } else {
    launch_partial_g<64>(p, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, off, (float*)ws, st);
    hipLaunchKernelGGL(decode_combine_kernel<64>, gc, dim3(256), 0, st, p, off, (const float*)ws, out, lse);
  }
  return hipGetLastError();
}

}  // namespace kvs
