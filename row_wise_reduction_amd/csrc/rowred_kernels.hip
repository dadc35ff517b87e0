// rowred_kernels.hip -- gfx950 kernels for fused FP32 row reductions.
//
// One skeleton serves residual LayerNorm, RMSNorm and softmax.  A row is
// owned by L = 2^lanes_log2 consecutive lanes of a workgroup; lane l holds
// the row's 16-byte slots c*L + l (c < C) in registers (the "stripe"), so
// every input element is fetched from HBM once and reused by all phases:
//
//   load (+ residual add)  ->  reduction 1  ->  element map + reduction 2
//   ->  output map  ->  predicated store
//
// This follows the element ownership map and cross-phase input reuse of
// "Immutable input reuse in Metal reductions" (section "What the
// transformation actually preserves"), and the row packing, two-level
// collective and tail replay of "Cooperating-program packing:
// implementation and fixed-plan evidence" (section "Implementation
// boundary"), re-planned for 64-lane wavefronts:
//   * L <= 64: 64/L rows per wavefront; the collective is a DPP / ds_swizzle
//     butterfly inside the lane group, no LDS and no barrier.
//   * L > 64: the wavefront total goes to one LDS float per wave, one
//     barrier, then every lane folds its row's L/64 partials in a fixed
//     order (so all lanes hold bitwise-identical statistics).
//   * Rows whose start is not 16-byte aligned are read as the run of whole
//     16-byte granules that contain them; elements outside the row take the
//     reduction's identity and are never stored.
//   * Surplus row slots of the last workgroup recompute the last row and
//     skip the store, so every barrier is reached by every wave.
//   * Workgroups are handed out round-robin over the 8 XCDs; the block index
//     is remapped so each XCD walks one contiguous range of rows, which
//     keeps the granule shared by two neighbouring rows in one L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "rowred_device.h"
#include "rowred_internal.h"

namespace rowred {
namespace {

// ---------------------------------------------------------------------------
// The row kernel.  C = 16-byte slots per lane.  x fixes the window: slot k of
// a row is the k-th 16-byte granule holding any of its elements, and lane
// li of the row holds slots c*L + li.  r and y are accessed 16 bytes at a
// time when they share x's address modulo 16 (a.r_vec / a.y_vec), otherwise
// 4 bytes at a time at the same element positions.
// ---------------------------------------------------------------------------
// `threads` is blockDim.x, read in the kernel itself: there the compiler
// knows workgroups are uniform and reads it with a scalar load.
//
// SHIFT (affine LayerNorm only): gamma / beta at another 16-byte phase than
// the rows.  The four elements e0 = 4k - off .. e0 + 3 of a slot (k its
// granule) are gamma[e0 .. e0 + 3]: one 16-byte load from a 4-byte boundary
// (gfx950 serves such loads; the compiler emits them for 4-byte-aligned
// 16-byte copies) instead of four 4-byte loads.  A kernel of its own, so the
// other affine kernels keep their code.
template <int OP, int C, bool RELOAD, bool SHIFT = false>
__device__ __forceinline__ void row_body(const RowArgs &a, const int threads) {
  __shared__ float partials[2][16];
  __shared__ double partials_d[16];

  const int lanes_log2 = a.lanes_log2;
  const int L = 1 << lanes_log2;
  const int li = threadIdx.x & (L - 1);
  const int slot = threadIdx.x >> lanes_log2;
  const int rows_per_group = threads >> lanes_log2;
  const int width = a.width;

  int64_t row = row_block(blockIdx.x, gridDim.x, (a.policy & kPolicyXcdRemap) != 0) * rows_per_group + slot;
  const bool live = row < a.rows;
  if (!live) row = a.rows - 1;  // tail replay: recompute the last row, store nothing
  const int64_t base = row * (int64_t)width;

  // Position of this row inside its first granule and the number of
  // granules it touches.
  const float *xrow = a.x + base;
  const int off = (int)(((uintptr_t)xrow >> 2) & 3);
  const int nwin = (width + off + 3) >> 2;
  const int kmax = nwin - 1;

  // Element index (inside the row) of stripe element 4c+j; < 0 or >= width
  // at the window edges and in slots past the window.
  auto elem = [&](int c, int j) -> int { return 4 * (c * L + li) + j - off; };
  auto valid = [&](int c, int j) -> bool { return (unsigned)elem(c, j) < (unsigned)width; };

  float s[4 * C];

  // ---- load: every input element once, all loads issued back to back
  // before any use.  Slots past the row's last granule load the last granule
  // again instead of branching around the load (a cache hit that keeps the
  // loads unconditional); they are masked to the identity below by their
  // unclamped position.
  const f32x4 *xw = reinterpret_cast<const f32x4 *>(xrow - off);
  const bool nt_loads = (a.policy & kPolicyNtLoads) != 0;
  const bool has_r = is_layernorm(OP) && a.r != nullptr;
  const float *rrow = has_r ? a.r + base : nullptr;
  f32x4 xv[C], rv[C];
  auto load_rows = [&](auto nt) {
    constexpr bool NT = decltype(nt)::value;
    // The two instances of this block are the same instructions except for
    // the loads' cache hint, which is metadata until late in code generation:
    // the optimizer would hoist (or sink) the common loads out of the branch
    // on the policy and drop the non-temporal hint.  Empty asm statements
    // around the non-temporal loads keep the two copies apart.
    if constexpr (NT) asm volatile("" ::: "memory");
#pragma unroll
    for (int c = 0; c < C; ++c) xv[c] = load_g<NT>(xw + min(c * L + li, kmax));
    if constexpr (NT) asm volatile("" ::: "memory");
    if (has_r) {
      if (a.r_vec) {
        const f32x4 *rw = reinterpret_cast<const f32x4 *>(rrow - off);
#pragma unroll
        for (int c = 0; c < C; ++c) rv[c] = load_g<NT>(rw + min(c * L + li, kmax));
      } else {
        // r sits at another phase of the 16-byte grid: read the same elements
        // one by one, each index clamped into the row.
        const int emax = width - 1;
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
          for (int j = 0; j < 4; ++j) rv[c][j] = load_g<NT>(rrow + max(0, min(elem(c, j), emax)));
      }
    } else {
#pragma unroll
      for (int c = 0; c < C; ++c) rv[c] = f32x4(0.0f);
    }
  };
  if (nt_loads) load_rows(std::true_type{});
  else load_rows(std::false_type{});
  // Per-phase reload (RELOAD kernels, a diagnostic): read the row again.
  // The empty asm with a memory clobber keeps the compiler from reusing the
  // values of the earlier loads.
  auto reload = [&]() {
    asm volatile("" ::: "memory");
    if (nt_loads) load_rows(std::true_type{});
    else load_rows(std::false_type{});
  };
  // ---- scalar-per-row reductions: no output map, one lane writes the row.
  if constexpr (OP == kOpRowSum) {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += valid(c, j) ? (double)xv[c][j] : 0.0;
    double sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    sum = row_allreduce<SumOp>(sum, lanes_log2, partials_d);
    if (live && li == 0) a.y[row] = (float)sum;
    return;
  } else if constexpr (OP == kOpRowMinMax) {
    float lo[4], hi[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo[j] = __builtin_inff();
      hi[j] = -__builtin_inff();
    }
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lo[j] = fminf(lo[j], valid(c, j) ? xv[c][j] : __builtin_inff());
        hi[j] = fmaxf(hi[j], valid(c, j) ? xv[c][j] : -__builtin_inff());
      }
    float mn = fminf(fminf(lo[0], lo[1]), fminf(lo[2], lo[3]));
    float mx = fmaxf(fmaxf(hi[0], hi[1]), fmaxf(hi[2], hi[3]));
    row_allreduce_pair<MinOp, MaxOp>(mn, mx, lanes_log2, partials[0], partials[1]);
    if (live && li == 0) {
      a.y[row] = mn;
      a.y2[row] = mx;
    }
    return;
  }

  // The stripe of x, with the reduction's identity outside the row.
  auto fill_stripe = [&]() {
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) s[4 * c + j] = valid(c, j) ? xv[c][j] : identity<OP>();
  };
  if constexpr (!is_layernorm(OP)) fill_stripe();

  // ---- phases.
  if constexpr (OP == kOpRms) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4 * C; ++i) acc[i & 3] = fmaf(s[i], s[i], acc[i & 3]);
    float ss = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    ss = row_allreduce<SumOp>(ss, lanes_log2, partials[0]);
    const float scale = __builtin_amdgcn_rsqf(fmaf(ss, a.inv_width, a.eps));
    if constexpr (RELOAD) {
      reload();
      fill_stripe();
    }
#pragma unroll
    for (int i = 0; i < 4 * C; ++i) s[i] *= scale;
  } else if constexpr (OP == kOpSoftmax) {
    float mx[4] = {s[0], s[1], s[2], s[3]};
#pragma unroll
    for (int i = 4; i < 4 * C; ++i) mx[i & 3] = fmaxf(mx[i & 3], s[i]);
    float m = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
    if (!RELOAD && (a.policy & kPolicyOnline)) {
      // One collective (ROWRED_POLICY_ONLINE): this lane's exp(x - m) and
      // their sum, (max, sum) merged over the row, then each value scaled by
      // exp(m - M) / S.  A lane holding nothing but -inf (or no element of
      // the row) sums exp(-inf - 0) = 0s.
      const float ms = m == -__builtin_inff() ? 0.0f : m;
#pragma unroll
      for (int i = 0; i < 4 * C; ++i) s[i] = __builtin_amdgcn_exp2f((s[i] - ms) * kLog2e);
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4 * C; ++i) acc[i & 3] += s[i];
      float M = m, S = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      row_allreduce_online(M, S, lanes_log2, partials[0], partials[1]);
      const float f = __builtin_amdgcn_exp2f((m - M) * kLog2e) * __builtin_amdgcn_rcpf(S);
#pragma unroll
      for (int i = 0; i < 4 * C; ++i) s[i] *= f;
    } else {
      m = row_allreduce<MaxOp>(m, lanes_log2, partials[0]);
      auto exp_stripe = [&]() {
#pragma unroll
        for (int i = 0; i < 4 * C; ++i) s[i] = __builtin_amdgcn_exp2f((s[i] - m) * kLog2e);  // exp(x - m); -inf -> 0
      };
      if constexpr (RELOAD) {
        reload();
        fill_stripe();
      }
      exp_stripe();
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4 * C; ++i) acc[i & 3] += s[i];
      float sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      sum = row_allreduce<SumOp>(sum, lanes_log2, partials[1]);
      const float inv = __builtin_amdgcn_rcpf(sum);
      if constexpr (RELOAD) {
        reload();
        fill_stripe();
        exp_stripe();
      }
#pragma unroll
      for (int i = 0; i < 4 * C; ++i) s[i] *= inv;
    }
  } else {  // LayerNorm
    // The centred values d = (x + r) - mean must be correct to FP32 rounding
    // even when a row's spread is far below its magnitude (a large common
    // offset, or variance << eps), where the FP32 rounding of x + r and of
    // the mean would be amplified by 1/sqrt(var + eps).  So:
    //  * x + r is kept exactly as an unevaluated sum hi + lo (Knuth's
    //    TwoSum: hi = fl(x + r), lo = the rounding error, both FP32);
    //  * the row sum accumulates hi in FP64 and lo in FP32 (lo is below one
    //    ulp of hi, so its FP32 sum is exact to far below the FP64 sum's
    //    own error), and the mean is split into m_hi + m_lo;
    //  * d = (hi - m_hi) + (lo - m_lo) in FP32: the first difference is
    //    rounded relative to itself, which is d up to terms of ulp size, the
    //    second is tiny.
    // From here on every error is relative; variance and output are FP32.
    float hi[4 * C], lo[4 * C];
    auto combine = [&]() {
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float xv_ = valid(c, j) ? xv[c][j] : 0.0f;
          const float rv_ = valid(c, j) ? rv[c][j] : 0.0f;
          const float h = xv_ + rv_;
          const float bb = h - xv_;
          const float l = (xv_ - (h - bb)) + (rv_ - bb);  // exact: h + l == xv_ + rv_
          hi[4 * c + j] = h;
          lo[4 * c + j] = l;
        }
    };
    combine();
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    float acc_lo = 0.0f;
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[j] += (double)hi[4 * c + j];
        acc_lo += lo[4 * c + j];
      }
    double sum = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + (double)acc_lo;
    sum = row_allreduce<SumOp>(sum, lanes_log2, partials_d);
    const double mean = sum / (double)width;
    const float m_hi = (float)mean;
    const float m_lo = (float)(mean - (double)m_hi);
    auto centre = [&]() {
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * c + j;
          s[i] = valid(c, j) ? (hi[i] - m_hi) + (lo[i] - m_lo) : 0.0f;  // outside the row: 0
        }
    };
    if constexpr (RELOAD) {
      reload();
      combine();
    }
    centre();
    float sq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4 * C; ++i) sq[i & 3] = fmaf(s[i], s[i], sq[i & 3]);
    float var = (sq[0] + sq[1]) + (sq[2] + sq[3]);
    // Affine LayerNorm: gamma and beta hold one value per column.  They are
    // cached loads (every row reuses them).  With few chunks they go out
    // before the second collective, which hides their latency; wider
    // stripes load them just before use to stay within their registers.
    constexpr bool kAffine = OP == kOpLayerNormAffine;
    constexpr bool kEarlyAffine = kAffine && C <= 4;
    f32x4 gv[kEarlyAffine ? C : 1], bv[kEarlyAffine ? C : 1];
    // SHIFT: gamma / beta elements e0 = 4k - off .. e0 + 3 of slot c (k its
    // unclamped granule): one 16-byte load at a 4-byte boundary where all
    // four lie in the row, element by element (indices clamped into the
    // vector) in the slots at the row's two ends and past it.
    auto shifted = [&](const float *v, int c, float dflt) -> f32x4 {
      if (!v) return f32x4(dflt);
      const int e0 = 4 * (c * L + li) - off;
      f32x4 r;
      if (e0 >= 0 && e0 + 4 <= width) {
        __builtin_memcpy(&r, v + e0, sizeof(r));
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = v[max(0, min(e0 + j, width - 1))];
      }
      return r;
    };
    auto load_affine = [&]() {
      if constexpr (kEarlyAffine && SHIFT) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
          gv[c] = shifted(a.gamma, c, 1.0f);
          bv[c] = shifted(a.beta, c, 0.0f);
        }
      } else if constexpr (kEarlyAffine) {
        if (a.affine_vec) {  // rows start on 16-byte boundaries: row granule k is gamma/beta granule k
#pragma unroll
          for (int c = 0; c < C; ++c) {
            const int k = min(c * L + li, kmax);
            gv[c] = a.gamma ? load_g<false>(reinterpret_cast<const f32x4 *>(a.gamma) + k) : f32x4(1.0f);
            bv[c] = a.beta ? load_g<false>(reinterpret_cast<const f32x4 *>(a.beta) + k) : f32x4(0.0f);
          }
        } else {
          const int emax = width - 1;
#pragma unroll
          for (int c = 0; c < C; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int e = max(0, min(elem(c, j), emax));
              gv[c][j] = a.gamma ? load_g<false>(a.gamma + e) : 1.0f;
              bv[c][j] = a.beta ? load_g<false>(a.beta + e) : 0.0f;
            }
        }
      }
    };
    if constexpr (kEarlyAffine) load_affine();
    var = row_allreduce<SumOp>(var, lanes_log2, partials[1]);
    const float rstd = __builtin_amdgcn_rsqf(fmaf(var, a.inv_width, a.eps));
    if constexpr (RELOAD) {
      reload();
      combine();
      centre();
    }
    if constexpr (kEarlyAffine) {
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) s[4 * c + j] = fmaf(s[4 * c + j] * rstd, gv[c][j], bv[c][j]);
    } else if constexpr (kAffine) {
      // one chunk at a time: two 16-byte (or four 4-byte) loads per vector
#pragma unroll
      for (int c = 0; c < C; ++c) {
        f32x4 g, b;
        if (SHIFT) {
          g = shifted(a.gamma, c, 1.0f);
          b = shifted(a.beta, c, 0.0f);
        } else if (a.affine_vec) {
          const int k = min(c * L + li, kmax);
          g = a.gamma ? load_g<false>(reinterpret_cast<const f32x4 *>(a.gamma) + k) : f32x4(1.0f);
          b = a.beta ? load_g<false>(reinterpret_cast<const f32x4 *>(a.beta) + k) : f32x4(0.0f);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int e = max(0, min(elem(c, j), width - 1));
            g[j] = a.gamma ? load_g<false>(a.gamma + e) : 1.0f;
            b[j] = a.beta ? load_g<false>(a.beta + e) : 0.0f;
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) s[4 * c + j] = fmaf(s[4 * c + j] * rstd, g[j], b[j]);
        __builtin_amdgcn_sched_barrier(0);  // keep the next chunk's loads after this chunk's use
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4 * C; ++i) s[i] *= rstd;
    }
  }

  // ---- predicated store: replayed row slots write nothing.
  auto store_rows = [&](auto nt) {
    constexpr bool NT = decltype(nt)::value;
    float *yrow = a.y + base;
    if (a.y_vec) {
      f32x4 *yw = reinterpret_cast<f32x4 *>(yrow - off);
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int k = c * L + li;
        const int e0 = 4 * k - off;
        if (e0 >= 0 && e0 + 4 <= width) {
          store_g<NT>(yw + k, f32x4{s[4 * c], s[4 * c + 1], s[4 * c + 2], s[4 * c + 3]});
        } else if (k < nwin) {
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
          if (valid(c, j)) store_g<NT>(yrow + elem(c, j), s[4 * c + j]);
    }
  };

  // Staged stores (ROWRED_POLICY_STAGE_STORES; the host sets it only with y
  // at x's 16-byte phase, <= 512 threads and <= 4 chunks -- short rows; wider
  // stripes compile without it).  The workgroup's rows are consecutive, so
  // its outputs form one contiguous run of y.  When rows do not start on
  // 16-byte boundaries, the cache lines at row boundaries hold two rows'
  // outputs written by different lanes at different times, and each part
  // leaves as its own partial line write-back.  Here every lane first puts
  // its outputs into the run's image in LDS (whole granules land 16-byte
  // aligned there, since the run and the row share the phase), and after
  // one barrier consecutive threads store consecutive whole granules, so each
  // line is written by one instruction; only the run's two end granules are
  // partial.
  if constexpr (C <= kMaxStageChunks) {
    if (a.policy & kPolicyStageStores) {
      extern __shared__ f32x4 stage[];  // stage_lds_bytes(C, threads), sized at launch
      float *stage_f = reinterpret_cast<float *>(stage);
      const int64_t row_first = row_block(blockIdx.x, gridDim.x, (a.policy & kPolicyXcdRemap) != 0) * rows_per_group;
      const int64_t row_stop = row_first + rows_per_group < a.rows ? row_first + rows_per_group : a.rows;
      const int64_t e_begin = row_first * (int64_t)width, e_end = row_stop * (int64_t)width;
      const int fb = (int)((((uintptr_t)a.x >> 2) + e_begin) & 3);  // phase of the run's first element
      if (live) {
        // LDS float index of this row's element e: fb + slot*width + e;
        // of its granule k: 4 * (granule0 + k) with granule0 below.
        const int granule0 = (fb + slot * width - off) >> 2;
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const int k = c * L + li;
          const int e0 = 4 * k - off;
          if (e0 >= 0 && e0 + 4 <= width) {
            stage[granule0 + k] = f32x4{s[4 * c], s[4 * c + 1], s[4 * c + 2], s[4 * c + 3]};
          } else if (k < nwin) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if ((unsigned)(e0 + j) < (unsigned)width) stage_f[4 * (granule0 + k) + j] = s[4 * c + j];
          }
        }
      }
      __syncthreads();
      const int n_granules = (int)((fb + (e_end - e_begin) + 3) >> 2);
      f32x4 *yg = reinterpret_cast<f32x4 *>(a.y + e_begin - fb);  // 16-byte aligned: y shares x's phase
      auto store_run = [&](auto nt) {
        constexpr bool NT = decltype(nt)::value;
        for (int g = threadIdx.x; g < n_granules; g += threads) {
          const f32x4 v = stage[g];
          const int64_t e0 = e_begin - fb + 4 * (int64_t)g;
          if (e0 >= e_begin && e0 + 4 <= e_end) {
            store_g<NT>(yg + g, v);
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (e0 + j >= e_begin && e0 + j < e_end) store_g<NT>(a.y + e0 + j, v[j]);
          }
        }
      };
      if (a.policy & kPolicyNtStores) store_run(std::true_type{});
      else store_run(std::false_type{});
      return;
    }
  }
  if (!live) return;
  if (a.policy & kPolicyNtStores) store_rows(std::true_type{});
  else store_rows(std::false_type{});
}

template <int OP, int C>
__global__ void __launch_bounds__(max_threads_for(OP, C)) rows_kernel(RowArgs a) {
  row_body<OP, C, false>(a, blockDim.x);
}

// Affine LayerNorm on rows off 16-byte boundaries with gamma and beta on
// them (see row_body).
template <int C>
__global__ void __launch_bounds__(max_threads_for(kOpLayerNormAffine, C)) affine_shift_kernel(RowArgs a) {
  row_body<kOpLayerNormAffine, C, false, true>(a, blockDim.x);
}

// The per-phase reload variant (ROWRED_POLICY_RELOAD): same arithmetic, the
// row read again in every phase after the first.
template <int OP, int C>
__global__ void __launch_bounds__(reload_max_threads_for(OP, C)) reload_kernel(RowArgs a) {
  row_body<OP, C, true>(a, blockDim.x);
}

// Plain streaming copy: one 16-byte slot per lane, 64-lane workgroups.  Of
// the copy shapes measured on MI355X (1-8 slots per lane, 64-1024 threads,
// one pass or grid-stride, cached or streaming) this is the fastest: 6.8 TB/s
// on 1 GiB, against 6.2 TB/s for 4 slots x 256 threads.
constexpr int kCopyThreads = 64;
__global__ void __launch_bounds__(kCopyThreads) copy_kernel(const f32x4 *x, f32x4 *y, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x;
  if (i < n4) store_g<true>(y + i, load_g<true>(x + i));
}

using KernelFn = void (*)(RowArgs);

template <int OP, int C>
constexpr KernelFn kernel_or_null() {
  if constexpr (kernel_exists(OP, C)) return rows_kernel<OP, C>;
  else return nullptr;
}

#define ROWRED_CHUNK_ROW(OP)                                                                          \
  {kernel_or_null<OP, 1>(), kernel_or_null<OP, 2>(),  kernel_or_null<OP, 3>(),  kernel_or_null<OP, 4>(), \
   kernel_or_null<OP, 5>(), kernel_or_null<OP, 6>(),  kernel_or_null<OP, 7>(),  kernel_or_null<OP, 8>(), \
   kernel_or_null<OP, 10>(), kernel_or_null<OP, 12>(), kernel_or_null<OP, 16>()}

// [kernel op][chunk index in kChunkSet]
const KernelFn kKernels[kNumKernelOps][kNumChunkSizes] = {
    ROWRED_CHUNK_ROW(kOpLayerNorm),
    ROWRED_CHUNK_ROW(kOpRms),
    ROWRED_CHUNK_ROW(kOpSoftmax),
    ROWRED_CHUNK_ROW(kOpRowSum),
    ROWRED_CHUNK_ROW(kOpRowMinMax),
    ROWRED_CHUNK_ROW(kOpLayerNormAffine),
};
static_assert(kOpLayerNormAffine == 5 && kOpRowSum == 3 && kOpRowMinMax == 4, "kernel table order");
#undef ROWRED_CHUNK_ROW

static_assert(kNumChunkSizes == 11, "kernel table rows must match kChunkSet");

// [chunk index in kChunkSet]; affine LayerNorm stops at 12 slots
const KernelFn kAffineShift[kNumChunkSizes] = {
    affine_shift_kernel<1>, affine_shift_kernel<2>, affine_shift_kernel<3>, affine_shift_kernel<4>,
    affine_shift_kernel<5>, affine_shift_kernel<6>, affine_shift_kernel<7>, affine_shift_kernel<8>,
    affine_shift_kernel<10>, affine_shift_kernel<12>, nullptr};

template <int OP, int C>
constexpr KernelFn reload_or_null() {
  if constexpr (reload_kernel_exists(OP, C)) return reload_kernel<OP, C>;
  else return nullptr;
}

#define ROWRED_RELOAD_ROW(OP)                                                                         \
  {reload_or_null<OP, 1>(), reload_or_null<OP, 2>(),  reload_or_null<OP, 3>(),  reload_or_null<OP, 4>(), \
   reload_or_null<OP, 5>(), reload_or_null<OP, 6>(),  reload_or_null<OP, 7>(),  reload_or_null<OP, 8>(), \
   reload_or_null<OP, 10>(), reload_or_null<OP, 12>(), reload_or_null<OP, 16>()}

// [matrix operator][chunk index in kChunkSet]
const KernelFn kReloadKernels[3][kNumChunkSizes] = {
    ROWRED_RELOAD_ROW(kOpLayerNorm),
    ROWRED_RELOAD_ROW(kOpRms),
    ROWRED_RELOAD_ROW(kOpSoftmax),
};
#undef ROWRED_RELOAD_ROW

int chunk_index(int chunks) {
  for (int i = 0; i < kNumChunkSizes; ++i)
    if (kChunkSet[i] == chunks) return i;
  return -1;
}

}  // namespace

int launch_rows(int op, int chunks, int64_t grid, int threads, const RowArgs &args, hipStream_t stream) {
  const int ci = chunk_index(chunks);
  if (op < 0 || op >= kNumKernelOps || ci < 0) return (int)hipErrorInvalidValue;
  const bool reload = (args.policy & kPolicyReload) != 0;
  if (reload && op > 2) return (int)hipErrorInvalidValue;
  const bool shift = op == kOpLayerNormAffine && args.affine_shift;
  KernelFn fn = reload ? kReloadKernels[op][ci] : shift ? kAffineShift[ci] : kKernels[op][ci];
  if (!fn) return (int)hipErrorInvalidValue;
  RowArgs a = args;
  void *params[] = {&a};
  size_t lds = (a.policy & kPolicyStageStores) ? stage_lds_bytes(chunks, threads) : 0;
  const int cap = ROWRED_POLICY_CU_GROUPS_OF(a.policy);
  if (cap >= 1 && cap <= 14 && cu_groups_lds_bytes(cap) > lds) lds = cu_groups_lds_bytes(cap);
  return (int)hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3((uint32_t)grid), dim3(threads), params, lds,
                              stream);
}

int launch_copy(const float *x, float *y, int64_t n4, hipStream_t stream) {
  const int64_t grid = (n4 + kCopyThreads - 1) / kCopyThreads;
  const f32x4 *xs = reinterpret_cast<const f32x4 *>(x);
  f32x4 *ys = reinterpret_cast<f32x4 *>(y);
  int64_t n = n4;
  void *params[] = {&xs, &ys, &n};
  return (int)hipLaunchKernel(reinterpret_cast<const void *>(copy_kernel), dim3((uint32_t)grid), dim3(kCopyThreads),
                              params, 0, stream);
}

}  // namespace rowred
