// rowred_wide.hip -- RMSNorm and softmax rows of 4097-16384 granules held
// partly in registers, partly in LDS (ROWRED_POLICY_LDS_STRIPE).
//
// A 1024-lane workgroup owns one row, and lane li owns the row's granules
// c*1024 + li (c < CR + CL), as in the register-resident kernels.  Slots
// 0..CR-1 live in registers and slots CR..CR+CL-1 go straight from HBM into
// LDS (16-byte loads that write LDS, no registers in between), CL * 16 KB per
// workgroup.  Every element is read from HBM once; the LDS slots are read
// back by the lane that loaded them (no barrier needed for that) in each
// phase.
//   * 5-8 slots (CR = 4): held entirely in registers such a stripe leaves
//     room for one workgroup per CU; with half of it in LDS two share a CU,
//     and one's loads overlap the other's collectives and stores.  The
//     arithmetic and its order are those of the register-resident kernel
//     with the same stripe, so results are bitwise equal.
//   * 9-16 slots (CR = 8, up to 128 KB of LDS): rows of up to 65536 aligned
//     floats, which no register stripe holds, are read once instead of twice
//     (the looped kernels' two walks).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "rowred_device.h"
#include "rowred_internal.h"

namespace rowred {
namespace {

constexpr int kWideLanes = 1024;

template <int OP, int CR, int CL>
__global__ void __launch_bounds__(kWideLanes) wide_kernel(RowArgs a) {
  constexpr int C = CR + CL;
  constexpr int L = kWideLanes;
  __shared__ f32x4 held[CL * L];
  __shared__ float partials[2][16];
  constexpr int lanes_log2 = 10;
  const int li = threadIdx.x;
  const int width = a.width;
  const int64_t row = row_block(blockIdx.x, gridDim.x, (a.policy & kPolicyXcdRemap) != 0);
  const int64_t base = row * (int64_t)width;
  const float *xrow = a.x + base;
  const int off = (int)(((uintptr_t)xrow >> 2) & 3);
  const int nwin = (width + off + 3) >> 2;
  const int kmax = nwin - 1;
  auto elem = [&](int c, int j) -> int { return 4 * (c * L + li) + j - off; };
  auto valid = [&](int c, int j) -> bool { return (unsigned)elem(c, j) < (unsigned)width; };
  const f32x4 *xw = reinterpret_cast<const f32x4 *>(xrow - off);
  // This wave's part of LDS slot c: lane l of the wave lands at entry l.
  f32x4 *wave_held = held + (li & ~63);
  typedef __attribute__((address_space(3))) void lds_void;

  // ---- load: the LDS slots first, then the register slots; all in flight
  // before any use.  Granules past the row's last one load the last one
  // again (masked below by position), as in the row kernels.
  f32x4 xv[CR];
  auto load_all = [&](auto nt) {
    constexpr bool NT = decltype(nt)::value;
    if constexpr (NT) asm volatile("" ::: "memory");
#pragma unroll
    for (int c = 0; c < CL; ++c)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(xw + min((CR + c) * L + li, kmax)),
                                       (lds_void *)(wave_held + c * L), 16, 0, NT ? 2 : 0);
#pragma unroll
    for (int c = 0; c < CR; ++c) xv[c] = load_g<NT>(xw + min(c * L + li, kmax));
    if constexpr (NT) asm volatile("" ::: "memory");
  };
  if (a.policy & kPolicyNtLoads) load_all(std::true_type{});
  else load_all(std::false_type{});
  // The LDS writes of those loads are done once the loads have completed.
  __builtin_amdgcn_s_waitcnt(0);
  auto lds_slot = [&](int c) -> f32x4 { return held[c * L + li]; };

  float s[4 * CR];  // the register slots, mapped in place
#pragma unroll
  for (int c = 0; c < CR; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) s[4 * c + j] = valid(c, j) ? xv[c][j] : identity<OP>();
  auto lds_value = [&](const f32x4 &v, int c, int j) -> float { return valid(CR + c, j) ? v[j] : identity<OP>(); };

  float scale;  // RMSNorm: 1/rms; softmax: 1/sum
  float m = 0.0f;
  if constexpr (OP == kOpRms) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4 * CR; ++i) acc[i & 3] = fmaf(s[i], s[i], acc[i & 3]);
#pragma unroll
    for (int c = 0; c < CL; ++c) {
      const f32x4 v = lds_slot(c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float t = lds_value(v, c, j);
        acc[j] = fmaf(t, t, acc[j]);
      }
    }
    float ss = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    ss = row_allreduce<SumOp>(ss, lanes_log2, partials[0]);
    scale = __builtin_amdgcn_rsqf(fmaf(ss, a.inv_width, a.eps));
  } else {  // softmax
    float mx[4] = {s[0], s[1], s[2], s[3]};
#pragma unroll
    for (int i = 4; i < 4 * CR; ++i) mx[i & 3] = fmaxf(mx[i & 3], s[i]);
#pragma unroll
    for (int c = 0; c < CL; ++c) {
      const f32x4 v = lds_slot(c);
#pragma unroll
      for (int j = 0; j < 4; ++j) mx[j] = fmaxf(mx[j], lds_value(v, c, j));
    }
    m = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
    m = row_allreduce<MaxOp>(m, lanes_log2, partials[0]);
#pragma unroll
    for (int i = 0; i < 4 * CR; ++i) s[i] = __builtin_amdgcn_exp2f((s[i] - m) * kLog2e);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4 * CR; ++i) acc[i & 3] += s[i];
#pragma unroll
    for (int c = 0; c < CL; ++c) {
      const f32x4 v = lds_slot(c);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += __builtin_amdgcn_exp2f((lds_value(v, c, j) - m) * kLog2e);
    }
    float sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    sum = row_allreduce<SumOp>(sum, lanes_log2, partials[1]);
    scale = __builtin_amdgcn_rcpf(sum);
  }
#pragma unroll
  for (int i = 0; i < 4 * CR; ++i) s[i] *= scale;

  // ---- store: register slots, then the LDS slots mapped on the way out.
  auto out_value = [&](const f32x4 &v, int c, int j) -> float {
    const float t = lds_value(v, c, j);
    if constexpr (OP == kOpRms) return t * scale;
    else return __builtin_amdgcn_exp2f((t - m) * kLog2e) * scale;
  };
  auto store_all = [&](auto nt) {
    constexpr bool NT = decltype(nt)::value;
    float *yrow = a.y + base;
    auto store_slot = [&](int c, const float (&o)[4]) {
      const int k = c * L + li;
      const int e0 = 4 * k - off;
      if (a.y_vec) {
        if (e0 >= 0 && e0 + 4 <= width) {
          store_g<NT>(reinterpret_cast<f32x4 *>(yrow - off) + k, f32x4{o[0], o[1], o[2], o[3]});
        } else if (k < nwin) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if ((unsigned)(e0 + j) < (unsigned)width) store_g<NT>(yrow + e0 + j, o[j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if ((unsigned)(e0 + j) < (unsigned)width) store_g<NT>(yrow + e0 + j, o[j]);
      }
    };
#pragma unroll
    for (int c = 0; c < CR; ++c) {
      const float o[4] = {s[4 * c], s[4 * c + 1], s[4 * c + 2], s[4 * c + 3]};
      store_slot(c, o);
    }
#pragma unroll
    for (int c = 0; c < CL; ++c) {
      const f32x4 v = lds_slot(c);
      const float o[4] = {out_value(v, c, 0), out_value(v, c, 1), out_value(v, c, 2), out_value(v, c, 3)};
      store_slot(CR + c, o);
    }
  };
  if (a.policy & kPolicyNtStores) store_all(std::true_type{});
  else store_all(std::false_type{});
}

using WideFn = void (*)(RowArgs);
#define ROWRED_WIDE_ROW(OP)                                                                                  \
  {wide_kernel<OP, 4, 1>, wide_kernel<OP, 4, 2>, wide_kernel<OP, 4, 3>, wide_kernel<OP, 4, 4>,              \
   wide_kernel<OP, 8, 1>, wide_kernel<OP, 8, 2>, wide_kernel<OP, 8, 3>, wide_kernel<OP, 8, 4>,              \
   wide_kernel<OP, 8, 5>, wide_kernel<OP, 8, 6>, wide_kernel<OP, 8, 7>, wide_kernel<OP, 8, 8>}
// [RMSNorm, softmax][chunks - kWideMinChunks]: 4 register slots up to 8
// chunks, 8 from 9 on.
const WideFn kWide[2][kWideMaxChunks - kWideMinChunks + 1] = {ROWRED_WIDE_ROW(kOpRms), ROWRED_WIDE_ROW(kOpSoftmax)};
#undef ROWRED_WIDE_ROW
static_assert(kWideMinChunks == 5 && kWideMaxChunks == 16, "wide kernel table");

}  // namespace

int launch_wide(int op, int chunks, int64_t rows, const RowArgs &args, hipStream_t stream) {
  if ((op != kOpRms && op != kOpSoftmax) || chunks < kWideMinChunks || chunks > kWideMaxChunks)
    return (int)hipErrorInvalidValue;
  RowArgs a = args;
  void *params[] = {&a};
  return (int)hipLaunchKernel(reinterpret_cast<const void *>(kWide[op == kOpSoftmax][chunks - kWideMinChunks]),
                              dim3((uint32_t)rows),
                              dim3(kWideLanes), params, 0, stream);
}

}  // namespace rowred
