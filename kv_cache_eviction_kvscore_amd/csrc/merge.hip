// Split-K merge: score[l][g][j] = sum over query tiles of the score partials (ascending
// tile order) + the isolated argmax terms of the unit's rows with j*_r = j (row order).
//
// DropKV page, Key Contribution 3 (the split-K merge that reduces the scoring kernel's
// partials); PyramidKV page, aggregated window score (the sum over the heads that share
// the KV head is part of the per-tile partial). No atomics: every token has one writer
// and every sum has a fixed order.
#include "kvs_internal.hpp"

namespace kvs {
namespace {

constexpr int kMaxRows = 1024;

__global__ __launch_bounds__(256) void merge_kernel(Dev p, const float* __restrict__ partial,
                                                    const int32_t* __restrict__ jstar, const float* __restrict__ dom,
                                                    float* __restrict__ score) {
  __shared__ alignas(16) float buf[kMergeChunk];
  __shared__ int js[kMaxRows];
  const int u = blockIdx.y;
  int l, s, g;
  unit_coords(p, u, l, s, g);
  const int64_t n = p.cu[s + 1] - p.cu[s];
  const int64_t j0 = (int64_t)blockIdx.x * kMergeChunk;
  if (j0 >= n) return;
  const int64_t jend = (n < j0 + kMergeChunk) ? n : j0 + kMergeChunk;
  const int tid = threadIdx.x;
  const float* pb = partial + (int64_t)(l * p.Hkv + g) * p.Tq * p.N + p.cu[s];
  // 16-byte loads and stores when every tile row of this unit and its score row start
  // 16-byte aligned (uniform)
  const bool vec = ((p.cu[s] | p.N) & 3) == 0 && (((size_t)partial | (size_t)score) & 15) == 0;
  if (vec) {
    for (int i = 4 * tid; i < kMergeChunk; i += 4 * 256) {
      const int64_t j = j0 + i;
      float4 acc = {0.f, 0.f, 0.f, 0.f};
      if (j + 3 < jend) {
        for (int t = 0; t < p.Tq; ++t) {
          const float4 x = *(const float4*)(pb + (int64_t)t * p.N + j);
          acc.x += x.x;
          acc.y += x.y;
          acc.z += x.z;
          acc.w += x.w;
        }
      } else {
        float a4[4] = {0.f, 0.f, 0.f, 0.f};
        for (int e = 0; e < 4; ++e)
          if (j + e < jend)
            for (int t = 0; t < p.Tq; ++t) a4[e] += pb[(int64_t)t * p.N + j + e];
        acc = float4{a4[0], a4[1], a4[2], a4[3]};
      }
      *(float4*)&buf[i] = acc;
    }
  } else {
    for (int i = tid; i < kMergeChunk; i += 256) {
      const int64_t j = j0 + i;
      float acc = 0.f;
      if (j < jend)
        for (int t = 0; t < p.Tq; ++t) acc += pb[(int64_t)t * p.N + j];
      buf[i] = acc;
    }
  }
  const int64_t rb = (int64_t)u * p.R;
  for (int r = tid; r < p.R; r += 256) js[r] = jstar[rb + r];
  __syncthreads();
  for (int r = tid; r < p.R; r += 256) {
    const int jj = js[r];
    if (jj < j0 || jj >= jend) continue;
    bool first = true;
    for (int r2 = 0; r2 < r; ++r2)
      if (js[r2] == jj) {
        first = false;
        break;
      }
    if (!first) continue;
    float acc = 0.f;
    for (int r2 = r; r2 < p.R; ++r2)
      if (js[r2] == jj) acc += dom[rb + r2];
    buf[jj - j0] += acc;  // one writer per token: the lowest row with this argmax
  }
  __syncthreads();
  float* out = score + (int64_t)(l * p.Hkv + g) * p.N + p.cu[s];
  if (vec) {
    for (int i = 4 * tid; i < kMergeChunk; i += 4 * 256) {
      const int64_t j = j0 + i;
      if (j + 3 < jend) *(float4*)(out + j) = *(const float4*)&buf[i];
      else
        for (int e = 0; e < 4; ++e)
          if (j + e < jend) out[j + e] = buf[i + e];
    }
  } else {
    for (int i = tid; i < kMergeChunk; i += 256) {
      const int64_t j = j0 + i;
      if (j < jend) out[j] = buf[i];
    }
  }
}

}  // namespace

hipError_t launch_merge(const Dev& p, const float* partial, const int32_t* jstar, const float* dom, float* score,
                        hipStream_t st) {
  const dim3 grid((unsigned)((p.max_n + kMergeChunk - 1) / kMergeChunk), p.U);
  hipLaunchKernelGGL(merge_kernel, grid, dim3(256), 0, st, p, partial, jstar, dom, score);
  return hipGetLastError();
}

}  // namespace kvs
