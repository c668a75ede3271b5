// Split-K merge: score[l][g][j] = sum over query tiles of the score partials (ascending
// tile order) + the isolated argmax terms of the unit's rows with j*_r = j (row order).
// Two kernels: a streaming sum of the partials, then one workgroup per unit adds the
// isolated terms.
//
// DropKV page, Key Contribution 3 (the split-K merge that reduces the scoring kernel's
// partials); PyramidKV page, aggregated window score (the sum over the heads that share
// the KV head is part of the per-tile partial). No atomics: every token has one writer
// and every sum has a fixed order.
#include <climits>

#include "kvs_internal.hpp"

namespace kvs {
namespace {

constexpr int kMaxRows = 1024;

// score = the sum of the unit's query-tile partials, in ascending tile order. No LDS, so
// many workgroups share a CU and their loads and stores overlap.
__global__ __launch_bounds__(256) void merge_sum_kernel(Dev p, const float* __restrict__ partial,
                                                        float* __restrict__ score) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  constexpr int NV = kMergeChunk / (4 * 256);  // 16-byte pieces per thread
  const int u = blockIdx.y;
  int l, s, g;
  unit_coords(p, u, l, s, g);
  const int64_t n = p.cu[s + 1] - p.cu[s];
  const int64_t j0 = (int64_t)blockIdx.x * kMergeChunk;
  if (j0 >= n) return;
  const int tid = threadIdx.x;
  const float* pb = partial + (int64_t)(l * p.Hkv + g) * p.Tq * p.N + p.cu[s];
  float* out = score + (int64_t)(l * p.Hkv + g) * p.N + p.cu[s];
  // 16-byte pieces when every tile row of this unit and its score row start 16-byte
  // aligned and the chunk is whole (uniform)
  const bool vec = ((p.cu[s] | p.N) & 3) == 0 && (((size_t)partial | (size_t)score) & 15) == 0;
  if (vec && j0 + kMergeChunk <= n) {
    // every load of the thread in flight at once; the partial rows are read once, so they
    // bypass cache allocation
    f32x4v acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = f32x4v{0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t < p.Tq; ++t) {
      const float* row = pb + (int64_t)t * p.N + j0;
      f32x4v x[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) x[i] = __builtin_nontemporal_load((const f32x4v*)(row + 4 * (tid + 256 * i)));
#pragma unroll
      for (int i = 0; i < NV; ++i) acc[i] += x[i];
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) *(f32x4v*)(out + j0 + 4 * (tid + 256 * i)) = acc[i];
    return;
  }
  // otherwise (rows not 16-byte aligned, as with an odd total token count, or the
  // sequence's last chunk) 4-byte pieces, all of the thread's share of the chunk (NB) with
  // every load of a tile in flight before its sums; the same order of additions as above
  constexpr int NB = kMergeChunk / 256;
  const int64_t jend = (n < j0 + kMergeChunk) ? n : j0 + kMergeChunk;
  for (int64_t jb = j0 + tid; jb < jend; jb += 256 * NB) {
    float acc[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) acc[i] = 0.f;
    for (int t = 0; t < p.Tq; ++t) {
      const float* row = pb + (int64_t)t * p.N;
      float x[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int64_t j = jb + 256 * i;
        x[i] = j < jend ? __builtin_nontemporal_load(row + j) : 0.f;
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) acc[i] += x[i];
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int64_t j = jb + 256 * i;
      if (j < jend) out[j] = acc[i];
    }
  }
}

// score[j] += the isolated terms of the unit's rows with j*_r = j, summed in row order;
// the lowest such row writes, so every token has one writer. One workgroup per unit.
__global__ __launch_bounds__(256) void merge_isolated_kernel(Dev p, const int32_t* __restrict__ jstar,
                                                             const float* __restrict__ dom,
                                                             float* __restrict__ score) {
  // rows padded to a multiple of 8 with an argmax no row has (so the scan reads 16 bytes at
  // a time, two reads in flight)
  __shared__ __align__(16) int js[kMaxRows];
  __shared__ __align__(16) float ds[kMaxRows];
  const int u = blockIdx.x;
  int l, s, g;
  unit_coords(p, u, l, s, g);
  const int tid = threadIdx.x;
  const int64_t rb = (int64_t)u * p.R;
  const int Rp = (p.R + 7) & ~7;
  for (int r = tid; r < Rp; r += 256) {
    const bool ok = r < p.R;
    js[r] = ok ? jstar[rb + r] : INT_MIN;
    ds[r] = ok ? dom[rb + r] : 0.f;
  }
  __syncthreads();
  float* out = score + (int64_t)(l * p.Hkv + g) * p.N + p.cu[s];
  const int64_t n = p.cu[s + 1] - p.cu[s];
  for (int r = tid; r < p.R; r += 256) {
    const int jj = js[r];
    // one pass over all rows, the same for every lane (so the LDS reads are broadcasts):
    // whether an earlier row has this argmax (then that row writes), and the sum over this
    // row and the later ones that have it, in row order
    bool earlier = false;
    float a1 = 0.f;
    for (int r8 = 0; r8 < Rp; r8 += 8) {
      const int4 ja = *(const int4*)&js[r8], jb = *(const int4*)&js[r8 + 4];
      const float4 da = *(const float4*)&ds[r8], db = *(const float4*)&ds[r8 + 4];
      const int jv[8] = {ja.x, ja.y, ja.z, ja.w, jb.x, jb.y, jb.z, jb.w};
      const float dv[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool same = jv[e] == jj;
        earlier |= same && r8 + e < r;
        a1 += (same && r8 + e >= r) ? dv[e] : 0.f;
      }
    }
    if (!earlier && jj >= 0 && jj < n) out[jj] += a1;  // no argmax in the sequence: nothing to add
  }
}

}  // namespace

hipError_t launch_merge(const Dev& p, const float* partial, const int32_t* jstar, const float* dom, float* score,
                        hipStream_t st) {
  // one query tile in the score buffer itself: the sum over tiles is that tile, in place
  if (!(p.Tq == 1 && partial == score)) {
    const dim3 grid((unsigned)((p.max_n + kMergeChunk - 1) / kMergeChunk), p.U);
    hipLaunchKernelGGL(merge_sum_kernel, grid, dim3(256), 0, st, p, partial, score);
  }
  hipLaunchKernelGGL(merge_isolated_kernel, dim3(p.U), dim3(256), 0, st, p, jstar, dom, score);
  return hipGetLastError();
}

}  // namespace kvs
