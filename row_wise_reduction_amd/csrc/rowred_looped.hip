// rowred_looped.hip -- rows wider than the register-resident window, in one
// kernel and without a workspace: one workgroup per row walks the row's
// window of 16-byte granules in tiles of T*C granules (lane li holds the
// tile's granules c*T + li), twice:
//
//   pass 1  statistics, tile by tile, with cached loads so that pass 2 can
//           find the row in cache;
//   pass 2  (LayerNorm, RMSNorm, softmax) the row again: map and store.
//
// Row sum and min/max need pass 1 only.  Loads run two tiles deep: the next
// tile's loads are issued before the current tile is used.
//
// Per-lane state across tiles, then one workgroup collective:
//   softmax    online (max m, sum s of exp(x - m)): a tile with a larger
//              max rescales s by exp(m_old - m_new).  Across lanes:
//              M = max m, S = sum of s * exp(m - M).  This is the
//              single-pass (max, sum) reading of the max / exp-sum phases
//              of "Immutable input reuse in Metal reductions" (section
//              "What the transformation actually preserves").
//   LayerNorm  per tile (count, sum, sum of squares about the tile mean),
//              folded into the lane's (n, mean, M2) by the pairwise update of
//              Chan, Golub and LeVeque; across lanes the row mean is the FP64
//              sum over lanes / width and M2 = sum of M2_l + n_l (mean_l -
//              mean)^2, which is the biased two-pass variance about the row
//              mean of "Residual LayerNorm shared-Tile materialization
//              search" (section "Structural finding").
//   RMSNorm    sum of squares; row sum in FP64; min/max (NaN skipped).
// Reading the row again instead of holding it is the mixed cache/reload
// choice "Immutable input reuse in Metal reductions" leaves open for rows
// beyond the private stripe (section "Next decisions and open questions").
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "rowred_device.h"
#include "rowred_internal.h"

namespace rowred {
namespace {

template <int OP, int C>
__global__ void __launch_bounds__(1024) looped_kernel(RowArgs a) {
  __shared__ float partials[2][16];
  __shared__ double partials_d[2][16];
  const int T = blockDim.x;
  const int li = threadIdx.x;
  const int lanes_log2 = a.lanes_log2;
  // one row per workgroup; XCD_REMAP gives each XCD a contiguous run of rows
  const int64_t row = row_block(blockIdx.x, gridDim.x, (a.policy & kPolicyXcdRemap) != 0);
  const int width = a.width;
  const int64_t base = row * (int64_t)width;
  const float *xrow = a.x + base;
  const bool has_r = is_layernorm(OP) && a.r != nullptr;
  const float *rrow = has_r ? a.r + base : nullptr;
  const int off = (int)(((uintptr_t)xrow >> 2) & 3);
  const int nwin = (width + off + 3) >> 2;
  const int kmax = nwin - 1;
  const int G = T * C;
  const int ntiles = (nwin + G - 1) / G;

  auto granule = [&](int t, int c) -> int { return t * G + c * T + li; };
  auto elem = [&](int t, int c, int j) -> int { return 4 * granule(t, c) + j - off; };
  auto valid = [&](int t, int c, int j) -> bool { return (unsigned)elem(t, c, j) < (unsigned)width; };

  // Loads of tile t; past the row's last granule they load that granule
  // again (masked by position).  The empty asm statements keep a
  // non-temporal copy of this block apart from the cached one.
  auto load_tile = [&](auto nt, int t, f32x4(&xv)[C], f32x4(&rv)[C]) {
    constexpr bool NT = decltype(nt)::value;
    if constexpr (NT) asm volatile("" ::: "memory");
    const f32x4 *xw = reinterpret_cast<const f32x4 *>(xrow - off);
#pragma unroll
    for (int c = 0; c < C; ++c) xv[c] = load_g<NT>(xw + min(granule(t, c), kmax));
    if (has_r) {
      if (a.r_vec) {
        const f32x4 *rw = reinterpret_cast<const f32x4 *>(rrow - off);
#pragma unroll
        for (int c = 0; c < C; ++c) rv[c] = load_g<NT>(rw + min(granule(t, c), kmax));
      } else {
        const int emax = width - 1;
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
          for (int j = 0; j < 4; ++j) rv[c][j] = load_g<NT>(rrow + max(0, min(elem(t, c, j), emax)));
      }
    } else {
#pragma unroll
      for (int c = 0; c < C; ++c) rv[c] = f32x4(0.0f);
    }
    if constexpr (NT) asm volatile("" ::: "memory");
  };

  // Walk the tiles two deep: f(t, xv, rv) on each tile in order.
  f32x4 xa[C], ra[C], xb[C], rb[C];
  auto walk = [&](auto nt, auto f) {
    load_tile(nt, 0, xa, ra);
    for (int t = 0; t < ntiles; t += 2) {
      if (t + 1 < ntiles) load_tile(nt, t + 1, xb, rb);
      f(t, xa, ra);
      if (t + 2 < ntiles) load_tile(nt, t + 2, xa, ra);
      if (t + 1 < ntiles) f(t + 1, xb, rb);
    }
  };

  // x + r as an exact pair hi + lo (Knuth's TwoSum); 0 outside the row.
  auto two_sum = [&](int t, const f32x4(&xv)[C], const f32x4(&rv)[C], float(&hi)[4 * C], float(&lo)[4 * C]) {
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = valid(t, c, j) ? xv[c][j] : 0.0f;
        const float r = valid(t, c, j) ? rv[c][j] : 0.0f;
        const float h = x + r;
        const float bb = h - x;
        hi[4 * c + j] = h;
        lo[4 * c + j] = (x - (h - bb)) + (r - bb);
      }
  };

  // ---- pass 1: statistics
  if constexpr (OP == kOpRowSum) {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    walk(std::false_type{}, [&](int t, const f32x4(&xv)[C], const f32x4(&)[C]) {
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += valid(t, c, j) ? (double)xv[c][j] : 0.0;
    });
    const double s = row_allreduce<SumOp>((acc[0] + acc[1]) + (acc[2] + acc[3]), lanes_log2, partials_d[0]);
    if (li == 0) a.y[row] = (float)s;
    return;
  } else if constexpr (OP == kOpRowMinMax) {
    float mn = __builtin_inff(), mx = -__builtin_inff();
    walk(std::false_type{}, [&](int t, const f32x4(&xv)[C], const f32x4(&)[C]) {
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          mn = fminf(mn, valid(t, c, j) ? xv[c][j] : __builtin_inff());
          mx = fmaxf(mx, valid(t, c, j) ? xv[c][j] : -__builtin_inff());
        }
    });
    row_allreduce_pair<MinOp, MaxOp>(mn, mx, lanes_log2, partials[0], partials[1]);
    if (li == 0) {
      a.y[row] = mn;
      a.y2[row] = mx;
    }
    return;
  }

  // Matrix operators: the statistics, then the map.
  float scale = 0.0f;           // RMSNorm: 1 / sqrt(mean square + eps); LayerNorm: rstd; softmax: 1 / sum
  float m_row = 0.0f;           // softmax: row max
  float m_hi = 0.0f, m_lo = 0.0f;  // LayerNorm: row mean as an FP32 pair
  // RMSNorm and softmax sum each tile's terms in FP32 and the lane's running
  // total in FP64 (a lane of a 2^31-column row adds up 2^21 terms).
  if constexpr (OP == kOpRms) {
    double total = 0.0;
    walk(std::false_type{}, [&](int t, const f32x4(&xv)[C], const f32x4(&)[C]) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x = valid(t, c, j) ? xv[c][j] : 0.0f;
          acc[j] = fmaf(x, x, acc[j]);
        }
      total += (double)((acc[0] + acc[1]) + (acc[2] + acc[3]));
    });
    const double ss = row_allreduce<SumOp>(total, lanes_log2, partials_d[0]);
    scale = __builtin_amdgcn_rsqf(fmaf((float)ss, a.inv_width, a.eps));
  } else if constexpr (OP == kOpSoftmax) {
    float m = -__builtin_inff();
    double s = 0.0;
    walk(std::false_type{}, [&](int t, const f32x4(&xv)[C], const f32x4(&)[C]) {
      float mt = -__builtin_inff();
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) mt = fmaxf(mt, valid(t, c, j) ? xv[c][j] : -__builtin_inff());
      const float m_new = fmaxf(m, mt);
      // rescale the running sum to the new max (no rescale while the max
      // stays, which also covers a lane that has seen only -inf)
      if (m_new != m) s *= (double)__builtin_amdgcn_exp2f((m - m_new) * kLog2e);
      m = m_new;
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x = xv[c][j];
          const bool zero = !valid(t, c, j) || x == -__builtin_inff();  // weight 0, even when m is -inf
          acc[j] += zero ? 0.0f : __builtin_amdgcn_exp2f((x - m) * kLog2e);
        }
      s += (double)((acc[0] + acc[1]) + (acc[2] + acc[3]));
    });
    const float M = row_allreduce<MaxOp>(m, lanes_log2, partials[0]);
    // an all -inf row: M = -inf, every s = 0, sum 0 and 1/sum = inf, and
    // the map's exp(-inf - -inf) makes the row NaN, as in one pass
    const double term = (m == M) ? s : s * (double)__builtin_amdgcn_exp2f((m - M) * kLog2e);
    const double S = row_allreduce<SumOp>(term, lanes_log2, partials_d[0]);
    m_row = M;
    scale = __builtin_amdgcn_rcpf((float)S);
  } else {  // LayerNorm
    double n_l = 0.0, mean_l = 0.0, m2_l = 0.0;
    walk(std::false_type{}, [&](int t, const f32x4(&xv)[C], const f32x4(&rv)[C]) {
      float hi[4 * C], lo[4 * C];
      two_sum(t, xv, rv, hi, lo);
      double acc[4] = {0.0, 0.0, 0.0, 0.0};
      float acc_lo = 0.0f;
      int n_t = 0;
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[j] += (double)hi[4 * c + j];
          acc_lo += lo[4 * c + j];
          n_t += valid(t, c, j) ? 1 : 0;
        }
      if (n_t == 0) return;
      const double s_t = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + (double)acc_lo;
      const double mu_t = s_t / (double)n_t;
      const float th = (float)mu_t;
      const float tl = (float)(mu_t - (double)th);
      float sq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * c + j;
          const float d = valid(t, c, j) ? (hi[i] - th) + (lo[i] - tl) : 0.0f;
          sq[j] = fmaf(d, d, sq[j]);
        }
      const double m2_t = (double)((sq[0] + sq[1]) + (sq[2] + sq[3]));
      const double n = n_l + (double)n_t;
      const double delta = mu_t - mean_l;
      mean_l += delta * ((double)n_t / n);
      m2_l += m2_t + delta * delta * (n_l * (double)n_t / n);
      n_l = n;
    });
    const double sum = row_allreduce<SumOp>(n_l * mean_l, lanes_log2, partials_d[0]);
    const double mean = sum / (double)width;
    const double dm = mean_l - mean;
    const double m2 = row_allreduce<SumOp>(m2_l + n_l * dm * dm, lanes_log2, partials_d[1]);
    m_hi = (float)mean;
    m_lo = (float)(mean - (double)m_hi);
    scale = __builtin_amdgcn_rsqf(fmaf((float)m2, a.inv_width, a.eps));
  }

  // ---- pass 2: map and store
  float *yrow = a.y + base;
  const bool affine = is_layernorm(OP) && (a.gamma != nullptr || a.beta != nullptr);
  auto map_store = [&](auto nt_store, int t, const f32x4(&xv)[C], const f32x4(&rv)[C]) {
    constexpr bool NT = decltype(nt_store)::value;
    float s[4 * C];
    if constexpr (OP == kOpRms) {
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) s[4 * c + j] = xv[c][j] * scale;
    } else if constexpr (OP == kOpSoftmax) {
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) s[4 * c + j] = __builtin_amdgcn_exp2f((xv[c][j] - m_row) * kLog2e) * scale;
    } else {
      float hi[4 * C], lo[4 * C];
      two_sum(t, xv, rv, hi, lo);
      const int emax = width - 1;
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * c + j;
          float y = ((hi[i] - m_hi) + (lo[i] - m_lo)) * scale;
          if (affine) {
            const int e = max(0, min(elem(t, c, j), emax));
            const float g = a.gamma ? a.gamma[e] : 1.0f;
            const float b = a.beta ? a.beta[e] : 0.0f;
            y = fmaf(y, g, b);
          }
          s[i] = y;
        }
    }
    if (a.y_vec) {
      f32x4 *yw = reinterpret_cast<f32x4 *>(yrow - off);
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int k = granule(t, c);
        const int e0 = 4 * k - off;
        if (e0 >= 0 && e0 + 4 <= width) {
          store_g<NT>(yw + k, f32x4{s[4 * c], s[4 * c + 1], s[4 * c + 2], s[4 * c + 3]});
        } else if (k <= kmax) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if ((unsigned)(e0 + j) < (unsigned)width) store_g<NT>(yrow + e0 + j, s[4 * c + j]);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (valid(t, c, j)) store_g<NT>(yrow + elem(t, c, j), s[4 * c + j]);
    }
  };
  auto pass2 = [&](auto nt_load, auto nt_store) {
    walk(nt_load, [&](int t, const f32x4(&xv)[C], const f32x4(&rv)[C]) { map_store(nt_store, t, xv, rv); });
  };
  const bool ntl = (a.policy & kPolicyNtLoads) != 0, nts = (a.policy & kPolicyNtStores) != 0;
  if (ntl && nts) pass2(std::true_type{}, std::true_type{});
  else if (ntl) pass2(std::true_type{}, std::false_type{});
  else if (nts) pass2(std::false_type{}, std::true_type{});
  else pass2(std::false_type{}, std::false_type{});
}

using KernelFn = void (*)(RowArgs);
#define ROWRED_LOOPED_ROW(OP) {looped_kernel<OP, 2>, looped_kernel<OP, 4>}
// [kernel op 0-4][chunks 2, 4]; affine LayerNorm runs the LayerNorm kernel,
// whose two-deep x and r tiles fit registers at 2 chunks only
const KernelFn kLooped[5][2] = {
    {looped_kernel<kOpLayerNorm, 2>, nullptr}, ROWRED_LOOPED_ROW(kOpRms), ROWRED_LOOPED_ROW(kOpSoftmax),
    ROWRED_LOOPED_ROW(kOpRowSum),              ROWRED_LOOPED_ROW(kOpRowMinMax),
};
#undef ROWRED_LOOPED_ROW

}  // namespace

int launch_looped(int op, int chunks, int64_t rows, int threads, const RowArgs &args, hipStream_t stream) {
  if (op == kKernelOpLayerNormAffine) op = kOpLayerNorm;
  const int ci = chunks == 2 ? 0 : chunks == 4 ? 1 : -1;
  if (op < 0 || op > 4 || ci < 0 || !kLooped[op][ci]) return (int)hipErrorInvalidValue;
  RowArgs a = args;
  void *params[] = {&a};
  return (int)hipLaunchKernel(reinterpret_cast<const void *>(kLooped[op][ci]), dim3((uint32_t)rows), dim3(threads),
                              params, 0, stream);
}

}  // namespace rowred
