// Internal definitions shared by the libkvscore HIP sources (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kvs {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// native 16-byte vector (HIP's uint4 is a class type: arrays of it are copied with memcpy and
// are not promoted to registers)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4): lane L
// reads base + off (off: its byte offset, base: the same for every lane, held in SGPRs) and
// writes LDS bytes [lds + 16 L, lds + 16 L + 16); lds (a byte offset in LDS) must be the same
// for every lane. Issued from inline asm so that the compiler does not treat it as an LDS
// store: it would otherwise drain every load in flight (s_waitcnt vmcnt(0)) before each LDS
// read it cannot prove disjoint. The caller orders it with explicit vmcnt waits and a barrier.
// Nontemporal (nt): a pass reads each K/V tile once, and streams far more K/V than the
// caches could hold until the next pass (measured 1-1.5% faster forward and score).
__device__ inline void lds_dma16(const void* base, unsigned off, unsigned lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(off), "s"(base),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
// byte offset in LDS of a __shared__ object (a flat address in the LDS aperture carries the
// offset in its low 32 bits)
__device__ inline unsigned lds_offset(const void* p) { return (unsigned)(size_t)p; }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, not for its
// global stores or loads in flight (__syncthreads' release fence waits for all of them)
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The values of x in lanes i % 32 (lo) and i % 32 + 32 (hi), for lane i: one
// v_permlane32_swap, a VALU exchange of the wave's halves with no LDS round trip (a
// ds_bpermute's wait would also wait for every LDS read issued before it). A reduction
// over (lo, hi) gives the same bits in both lanes of a pair.
struct HalfPair {
  float lo, hi;
};
__device__ inline HalfPair wave_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ inline int wave_halves_min(int x) {
  const auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return min((int)r[0], (int)r[1]);
}

// x summed over the lanes of its group of LANES consecutive lanes (16, 8 or 4), every lane
// of the group receiving the sum: DPP within rows of 16 lanes, no LDS round trip
template <int LANES>
__device__ inline float group_sum(float x) {
  auto dpp = [](float v, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value, 0xF, 0xF, false));
  };
  static_assert(LANES == 16 || LANES == 8 || LANES == 4, "group size");
  if constexpr (LANES == 16) {
    x += dpp(x, std::integral_constant<int, 0x128>{});  // row_ror:8
    x += dpp(x, std::integral_constant<int, 0x124>{});  // row_ror:4
    x += dpp(x, std::integral_constant<int, 0x122>{});  // row_ror:2
    x += dpp(x, std::integral_constant<int, 0x121>{});  // row_ror:1
  } else {
    if constexpr (LANES == 8) x += dpp(x, std::integral_constant<int, 0x141>{});  // row_half_mirror: lane i <-> 7 - i
    x += dpp(x, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
    x += dpp(x, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
  }
  return x;
}

constexpr int kMaxSeqs = 64;
constexpr int kMaxUnits = 65535;  // (layer, sequence, KV head) units: a grid dimension of every launch
constexpr int kRowsPerTileMax = 256;  // query rows one workgroup holds (8 waves x 32 rows)
constexpr int kMergeChunk = 8192;     // tokens per merge workgroup
constexpr int kCompactRows = 32;      // packed rows per compaction workgroup

// Problem as the kernels see it (passed by value as a kernel argument).
struct Dev {
  int S, L, Hq, Hkv, G, d, W;
  int R;       // rows per unit = G*W
  int Tq;      // query tiles per unit
  int RT;      // rows per query tile (multiple of 32, <= kRowsPerTileMax)
  int mode;    // 0 = L2, 1 = SQ, 2 = attention sum
  float scale; // multiplies q.k
  float c1;    // scale * log2(e)
  int64_t ksl, ksh, kst, vsl, vsh, vst;  // element strides
  int64_t N;                             // total tokens
  int U;                                 // units = L*S*Hkv
  int fwd_chunk;                         // keys per forward workgroup (multiple of 64)
  int fwd_chunks;                        // max forward chunks over sequences
  int score_chunk;                       // keys per score workgroup (multiple of 64)
  int score_chunks;                      // max score chunks over sequences
  int64_t max_n;                         // longest sequence
  int64_t cu[kMaxSeqs + 1];
};

// Decode attention over the packed ragged cache, as its kernels see it.
struct DecDev {
  int Hq, Hkv, G, d;
  int U;       // segments = L*S*Hkv
  float c1;    // softmax scale * log2(e)
  int chunk;   // keys per split (multiple of 64)
  int nsplit;  // splits of the longest segment
};

// unit u = (l*S + s)*Hkv + g
__host__ __device__ inline void unit_coords(const Dev& p, int u, int& l, int& s, int& g) {
  g = u % p.Hkv;
  s = (u / p.Hkv) % p.S;
  l = u / (p.Hkv * p.S);
}

// XCD-aware work order for a grid of (x = key chunk, y = query tile, z = unit) items, or a
// grid of units alone. The hardware deals workgroups round-robin by linear id to the chip's
// 8 XCDs and, within an XCD, to its 4 shader engines (8 CUs each): workgroup id w goes to
// queue w % 32 (measured). The identity order therefore hands each queue fixed (chunk,
// tile) pairs, and on a ragged batch the queues that draw first chunks get most of the
// work while the others idle (a 2x slower pass, measured). Here queue q takes the q-th
// 32nd of the logical items, whose order runs chunk fastest, then tile, then unit with the
// sequence fastest, so every queue holds nearly the same mix of sequence lengths. Returns
// the item's chunk, tile and unit (u = (l*S + s)*Hkv + g).
constexpr int kDispatchQueues = 32;
__device__ inline void xcd_item(int S, int Hkv, int nx, int ny, int nz, int lw, int& x, int& y, int& u) {
  const int G = nx * ny * nz, base = G / kDispatchQueues, rem = G % kDispatchQueues;
  const int q = lw % kDispatchQueues, k = lw / kDispatchQueues;
  const int lin = q * base + (q < rem ? q : rem) + k;  // a bijection of [0, G)
  x = lin % nx;
  y = (lin / nx) % ny;
  const int up = lin / (nx * ny);
  const int s = up % S, rest = up / S;
  u = ((rest / Hkv) * S + s) * Hkv + rest % Hkv;
}
__device__ inline void xcd_item3(const Dev& p, int& x, int& y, int& u) {
  xcd_item(p.S, p.Hkv, gridDim.x, gridDim.y, gridDim.z, blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z), x,
           y, u);
}

// Forward split record block: [RT][d] fp32 O_rest | [RT][d] fp16 v* | [RT] m | [RT] m2 | [RT] l_rest | [RT] j*
__host__ __device__ inline size_t fwd_block_floats(int RT, int d) { return (size_t)RT * d + (size_t)RT * d / 2 + 4 * (size_t)RT; }

// Score-prep workspace: [rows][d] fp16 a_hat | [rows] fp32 ||a_hat||^2 | [rows] fp32 lse*log2(e)
__host__ __device__ inline size_t prep_bytes(int64_t rows, int d) { return (size_t)rows * d * 2 + (size_t)rows * 8; }

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

// Launchers (each .hip file owns its kernels). Return hipGetLastError() after launch.
hipError_t launch_attn_fwd(const Dev& p, const void* q, const void* k, const void* v, float* a, float* lse,
                           int32_t* jstar, float* dom, void* ws, hipStream_t st);
hipError_t launch_score(const Dev& p, const void* q, const void* k, const void* v, const float* a,
                        const float* lse, const int32_t* jstar, float* partial, void* ws, hipStream_t st);
hipError_t launch_merge(const Dev& p, const float* partial, const int32_t* jstar, const float* dom, float* score,
                        hipStream_t st);
// head_off != nullptr: head budgets chosen jointly per (sequence, layer), their offsets
// written to head_off [U+1], using heads_ws (heads_ws_bytes(p) bytes) as scratch; budgets
// (host [S][L], the segment lengths) then choose which kernels are launched
hipError_t launch_topk(const Dev& p, const float* score, const int64_t* seg_off, int32_t* kept, int pool, int n_sink,
                       float* pooled, int64_t* head_off, void* heads_ws, const int32_t* budgets, hipStream_t st);
int heads_chunks(const Dev& p);
size_t heads_state_bytes(const Dev& p);
size_t heads_ws_bytes(const Dev& p);
constexpr int kMaxPoolSize = 255;
constexpr int kDecodeMaxGroup = 8;  // query heads per KV head the decode kernels take
hipError_t launch_decode(const DecDev& p, const void* q, const void* k, const void* v, const int64_t* off, float* out,
                         float* lse, void* ws, hipStream_t st);
// device address of the decode pass's fixed scratch array on the current device (looked up
// once per device)
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
hipError_t decode_scratch(void** ptr);
hipError_t launch_compact(const Dev& p, const void* k, const void* v, const int64_t* seg_off, const int32_t* kept,
                          void* k_out, void* v_out, int max_budget, hipStream_t st);

}  // namespace kvs
