// Compaction into the packed ragged cache (RippleKV page, Eq. 4: the compressed cache
// holds the (k, v) pairs at the retained positions; one independent length per
// (layer, KV head) segment, as the GraceKV page's physical cache packing).
// A bit-exact row gather with 16-byte vector loads and stores; grid (row block, unit).
#include "kvs_internal.hpp"

namespace kvs {
namespace {

template <int D>
__global__ __launch_bounds__(256) void compact_kernel(Dev p, const __bf16* __restrict__ k,
                                                      const __bf16* __restrict__ v,
                                                      const int64_t* __restrict__ seg_off,
                                                      const int32_t* __restrict__ kept, __bf16* __restrict__ ko,
                                                      __bf16* __restrict__ vo) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  const int u = blockIdx.y;
  const int64_t off0 = seg_off[u], b = seg_off[u + 1] - off0;
  const int64_t r0 = (int64_t)blockIdx.x * kCompactRows;
  if (r0 >= b) return;
  int l, s, g;
  unit_coords(p, u, l, s, g);
  const int64_t n = p.cu[s + 1] - p.cu[s];
  const __bf16* kb0 = k + l * p.ksl + g * p.ksh + p.cu[s] * p.kst;
  const __bf16* vb0 = v + l * p.vsl + g * p.vsh + p.cu[s] * p.vst;
  for (int c = threadIdx.x; c < kCompactRows * CPR; c += 256) {
    const int64_t r = r0 + c / CPR;
    const int part = c % CPR;
    if (r >= b) break;
    const int64_t pos = kept[off0 + r];
    if (pos < 0 || pos >= n) continue;  // never read outside the sequence
    const u32x4 kx = *(const u32x4*)(kb0 + pos * p.kst + part * 8);
    const u32x4 vx = *(const u32x4*)(vb0 + pos * p.vst + part * 8);
    *(u32x4*)(ko + (off0 + r) * D + part * 8) = kx;
    *(u32x4*)(vo + (off0 + r) * D + part * 8) = vx;
  }
}

}  // namespace

hipError_t launch_compact(const Dev& p, const void* k, const void* v, const int64_t* seg_off, const int32_t* kept,
                          void* k_out, void* v_out, int max_budget, hipStream_t st) {
  const dim3 grid((unsigned)((max_budget + kCompactRows - 1) / kCompactRows), p.U);
  if (p.d == 128)
    hipLaunchKernelGGL(compact_kernel<128>, grid, dim3(256), 0, st, p, (const __bf16*)k, (const __bf16*)v, seg_off,
                       kept, (__bf16*)k_out, (__bf16*)v_out);
  else
    hipLaunchKernelGGL(compact_kernel<64>, grid, dim3(256), 0, st, p, (const __bf16*)k, (const __bf16*)v, seg_off,
                       kept, (__bf16*)k_out, (__bf16*)v_out);
  return hipGetLastError();
}

}  // namespace kvs
