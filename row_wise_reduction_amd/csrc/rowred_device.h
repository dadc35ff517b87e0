// rowred_device.h -- device-side helpers shared by the gfx950 kernels:
// operator ids, cached / non-temporal global access, and the wavefront and
// workgroup collectives.  Included only by the .hip sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rowred_internal.h"

namespace rowred {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kOpLayerNorm = ROWRED_OP_LAYERNORM_RESIDUAL;
constexpr int kOpRms = ROWRED_OP_RMSNORM;
constexpr int kOpSoftmax = ROWRED_OP_SOFTMAX;
constexpr int kOpRowSum = ROWRED_OP_ROW_SUM;
constexpr int kOpRowMinMax = ROWRED_OP_ROW_MINMAX;
constexpr int kOpLayerNormAffine = kKernelOpLayerNormAffine;  // LayerNorm with gamma and/or beta
constexpr bool is_row_scalar(int op) { return op == kOpRowSum || op == kOpRowMinMax; }
constexpr bool is_layernorm(int op) { return op == kOpLayerNorm || op == kOpLayerNormAffine; }

constexpr float kLog2e = 1.44269504088896340736f;

// ---------------------------------------------------------------------------
// Memory access.  Each plan picks, per launch, whether global loads and
// stores carry the non-temporal (streaming) hint; the choice is uniform, so
// the kernels branch once around each block of accesses.
// ---------------------------------------------------------------------------
template <bool NT, class T>
__device__ __forceinline__ T load_g(const T *p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT, class T>
__device__ __forceinline__ void store_g(T *p, T v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// ---------------------------------------------------------------------------
// Cross-lane exchange inside a wavefront.
// ---------------------------------------------------------------------------
// DPP16 controls: quad_perm [1,0,3,2] (partner lane ^ 1), quad_perm [2,3,0,1]
// (^ 2), row_half_mirror (lane i <-> 7-i inside 8), row_mirror (i <-> 15-i
// inside 16).  After the ^1 and ^2 steps every lane of a quad holds the
// quad's value, so the two mirrors act as the ^4 and ^8 butterfly steps.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
// ds_swizzle bit-mask mode: and_mask 0x1F, or_mask 0, xor_mask 0x10 -> lane ^ 16
// inside each 32-lane half.
constexpr int kSwizzleXor16 = (0x10 << 10) | 0x1F;

template <int Ctrl>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), Ctrl, 0xF, 0xF, false));
}

__device__ __forceinline__ float swizzle_xor16(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), kSwizzleXor16));
}

__device__ __forceinline__ float readlane(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// 64-bit values move as two 32-bit halves.
struct Halves {
  int lo, hi;
};
__device__ __forceinline__ Halves split(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  return {(int)(uint32_t)b, (int)(uint32_t)(b >> 32)};
}
__device__ __forceinline__ double join(int lo, int hi) {
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

template <int Ctrl>
__device__ __forceinline__ double dpp(double v) {
  const Halves h = split(v);
  return join(__builtin_amdgcn_update_dpp(0, h.lo, Ctrl, 0xF, 0xF, false),
              __builtin_amdgcn_update_dpp(0, h.hi, Ctrl, 0xF, 0xF, false));
}

__device__ __forceinline__ double swizzle_xor16(double v) {
  const Halves h = split(v);
  return join(__builtin_amdgcn_ds_swizzle(h.lo, kSwizzleXor16), __builtin_amdgcn_ds_swizzle(h.hi, kSwizzleXor16));
}

__device__ __forceinline__ double readlane(double v, int lane) {
  const Halves h = split(v);
  return join(__builtin_amdgcn_readlane(h.lo, lane), __builtin_amdgcn_readlane(h.hi, lane));
}

struct SumOp {
  template <class T>
  static __device__ __forceinline__ T apply(T a, T b) { return a + b; }
};
struct MaxOp {
  static __device__ __forceinline__ float apply(float a, float b) { return fmaxf(a, b); }
};
struct MinOp {
  static __device__ __forceinline__ float apply(float a, float b) { return fminf(a, b); }
};

// All-reduce over aligned groups of 2^min(lanes_log2, 6) lanes.  Each step
// combines a lane with its partner commutatively, so every lane of a group
// ends with the same bits.  lanes_log2 is uniform: the branches are scalar.
template <class R, class T>
__device__ __forceinline__ T group_allreduce(T v, int lanes_log2) {
  if (lanes_log2 >= 1) v = R::apply(v, dpp<kDppXor1>(v));
  if (lanes_log2 >= 2) v = R::apply(v, dpp<kDppXor2>(v));
  if (lanes_log2 >= 3) v = R::apply(v, dpp<kDppHalfMirror>(v));
  if (lanes_log2 >= 4) v = R::apply(v, dpp<kDppMirror>(v));
  if (lanes_log2 >= 5) v = R::apply(v, swizzle_xor16(v));
  if (lanes_log2 >= 6) v = R::apply(readlane(v, 0), readlane(v, 32));
  return v;
}

// Row all-reduce: lane group first, then (rows wider than a wavefront) one
// LDS partial per wave, a barrier, and a fixed-order fold of the row's
// partials.  `partials` must be distinct for each reduction of a kernel so
// that a fast wave's next write cannot overtake a slow wave's read.
template <class R, class T>
__device__ __forceinline__ T row_allreduce(T v, int lanes_log2, T *partials) {
  v = group_allreduce<R>(v, lanes_log2 < 6 ? lanes_log2 : 6);
  if (lanes_log2 > 6) {
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) partials[wave] = v;
    __syncthreads();
    const int per_row_log2 = lanes_log2 - 6;
    const int first = (wave >> per_row_log2) << per_row_log2;
    T acc = partials[first];
    for (int w = 1; w < (1 << per_row_log2); ++w) acc = R::apply(acc, partials[first + w]);
    v = acc;
  }
  return v;
}

// Two row all-reduces that share one LDS exchange and one barrier (paired
// min/max): both wave partials are written before the barrier.
template <class R1, class R2>
__device__ __forceinline__ void row_allreduce_pair(float &v1, float &v2, int lanes_log2, float *p1, float *p2) {
  v1 = group_allreduce<R1>(v1, lanes_log2 < 6 ? lanes_log2 : 6);
  v2 = group_allreduce<R2>(v2, lanes_log2 < 6 ? lanes_log2 : 6);
  if (lanes_log2 > 6) {
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
      p1[wave] = v1;
      p2[wave] = v2;
    }
    __syncthreads();
    const int per_row_log2 = lanes_log2 - 6;
    const int first = (wave >> per_row_log2) << per_row_log2;
    float a1 = p1[first], a2 = p2[first];
    for (int w = 1; w < (1 << per_row_log2); ++w) {
      a1 = R1::apply(a1, p1[first + w]);
      a2 = R2::apply(a2, p2[first + w]);
    }
    v1 = a1;
    v2 = a2;
  }
}

// Softmax statistics as (max m, sum s of exp(x - m)) pairs.  A sum taken
// under max m restated under a max M >= m: s * exp(m - M) (s itself when
// m == M, which also keeps (-inf, 0) from becoming NaN).
__device__ __forceinline__ float rescale_sum(float s, float m, float M) {
  return m == M ? s : s * __builtin_amdgcn_exp2f((m - M) * kLog2e);
}

// Row all-reduce of (max, sum) pairs with one barrier: the max over the lane
// group (butterfly), each lane's sum restated under it, the sum over the
// group; then one pair per wave through LDS and a fixed-order fold (the row
// max, then the waves' sums restated under it and added in wave order).  All
// lanes of a row end with the same bits.  Special values: a NaN or +inf in
// any sum gives a NaN sum; pairs (-inf, 0) add nothing.
__device__ __forceinline__ void row_allreduce_online(float &m, float &s, int lanes_log2, float *pm, float *ps) {
  const int g = lanes_log2 < 6 ? lanes_log2 : 6;
  const float mg = group_allreduce<MaxOp>(m, g);
  s = group_allreduce<SumOp>(rescale_sum(s, m, mg), g);
  m = mg;
  if (lanes_log2 > 6) {
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
      pm[wave] = m;
      ps[wave] = s;
    }
    __syncthreads();
    const int per_row_log2 = lanes_log2 - 6;
    const int first = (wave >> per_row_log2) << per_row_log2;
    float M = pm[first];
    for (int w = 1; w < (1 << per_row_log2); ++w) M = fmaxf(M, pm[first + w]);
    float S = 0.0f;
    for (int w = 0; w < (1 << per_row_log2); ++w) S += rescale_sum(ps[first + w], pm[first + w], M);
    m = M;
    s = S;
  }
}

// Workgroup -> row block.  The dispatcher deals workgroups to the 8 XCDs in
// turn; give XCD x the contiguous block range [x*q + min(x, rem), ...).
__device__ __forceinline__ int64_t row_block(uint32_t bid, uint32_t nblk, bool remap) {
  if (!remap) return bid;
  constexpr uint32_t kXcds = 8;
  const uint32_t q = nblk / kXcds, rem = nblk % kXcds;
  const uint32_t xcd = bid % kXcds, i = bid / kXcds;
  return (int64_t)xcd * q + (xcd < rem ? xcd : rem) + i;
}

template <int OP>
__device__ __forceinline__ float identity() {
  return OP == kOpSoftmax ? -__builtin_inff() : 0.0f;
}

}  // namespace
}  // namespace rowred
