// rowred_split.hip -- split-row kernels: rows wider than one workgroup's
// registers can hold, and shapes with too few rows to fill the chip.
//
// A row's window of 16-byte granules (as in the row kernels) is cut into S
// segments of G = T*C granules.  Workgroup (row, k) owns segment k; its lane
// li holds granules k*G + c*T + li (c < C), so consecutive lanes read
// consecutive granules.
//
//   seg_stats_kernel  loads its segment (cached loads: the segment is read
//                     again by the apply kernel), reduces it and writes one
//                     record of two doubles to the workspace.
//   seg_merge_kernel  one wavefront per row folds the row's S records in a
//                     fixed order: into the outputs (row sum, row min/max)
//                     or into one row record (LayerNorm, RMSNorm, softmax).
//   seg_apply_kernel  reads its segment again, applies the row record and
//                     stores.  No collective, no barrier.
//
// Records (segment k holding n_k of the row's elements):
//   LayerNorm  (sum_k of x + r, M2_k = sum of squares about the segment mean)
//              merged with the pairwise update of Chan, Golub and LeVeque:
//              mean = sum / n, M2 = sum_k (M2_k + n_k (sum_k / n_k - mean)^2).
//              It equals the sum of squares about the row mean, so the
//              variance is still the biased two-pass one of "Residual
//              LayerNorm shared-Tile materialization search" (section
//              "Structural finding").
//   RMSNorm    (sum of x^2, 0)
//   softmax    (m_k = max, s_k = sum of exp(x - m_k)); m = max m_k and
//              s = sum of s_k exp(m_k - m): the max / exp-sum / normalise
//              phases of "Immutable input reuse in Metal reductions" (section
//              "What the transformation actually preserves") per segment.
//   row sum    (sum, 0) in FP64;  row min/max  (min, max), NaN skipped.
// The row record: LayerNorm (mean, M2), RMSNorm (sum of squares, 0),
// softmax (m, s).
//
// Reading a row once per kernel pass instead of keeping it in registers is
// the mixed cache/reload choice "Immutable input reuse in Metal reductions"
// leaves open (section "Next decisions and open questions") for rows beyond
// the private stripe; the segments give short rows' shapes such as 7x1537
// ("Fixed-width GPU and dispatch results") more than 7 workgroups.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "rowred_device.h"
#include "rowred_internal.h"

namespace rowred {
namespace {

struct Rec {
  double v0, v1;
};

// (row, segment) of this workgroup; the apply kernel may walk them backwards.
__device__ __forceinline__ void segment_of(const SegArgs &a, bool reverse, int64_t &row, int &seg) {
  uint32_t b = blockIdx.x;
  if (reverse) b = gridDim.x - 1 - b;
  const uint32_t q = b / (uint32_t)a.segments;
  row = q;
  seg = (int)(b - q * (uint32_t)a.segments);
}

// Elements of a row (first element `off` floats into its first granule)
// that fall in granules [k*G, (k+1)*G).
__device__ __forceinline__ int64_t segment_count(int64_t k, int64_t G, int off, int width) {
  const int64_t lo = 4 * k * G - off, hi = 4 * (k + 1) * G - off;
  const int64_t a = lo > 0 ? lo : 0, b = hi < width ? hi : (int64_t)width;
  return b > a ? b - a : 0;
}

// gamma (absent: 1) or beta (absent: 0) of the four elements e0 .. e0 + 3
// of one slot: one 16-byte load from a 4-byte boundary where all four lie in
// the row (the vectors may sit at any 16-byte phase against the row), element
// loads clamped into the vector at the row's two ends and past it.
__device__ __forceinline__ f32x4 affine_slot(const float *p, int e0, int width, float absent) {
  if (!p) return f32x4(absent);
  f32x4 r;
  if (e0 >= 0 && e0 + 4 <= width) {
    __builtin_memcpy(&r, p + e0, sizeof(r));
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = p[max(0, min(e0 + j, width - 1))];
  }
  return r;
}

// Where one workgroup's segment lies.
struct SegView {
  const float *xrow, *rrow;
  int off, kmax, g0, T, li, width;
  __device__ __forceinline__ int granule(int c) const { return g0 + c * T + li; }
  __device__ __forceinline__ int elem(int c, int j) const { return 4 * granule(c) + j - off; }
  __device__ __forceinline__ bool valid(int c, int j) const { return (unsigned)elem(c, j) < (unsigned)width; }
};

__device__ __forceinline__ SegView make_view(const SegArgs &a, int64_t row, int seg, int T, int C) {
  SegView v;
  const int64_t base = row * (int64_t)a.width;
  v.xrow = a.x + base;
  v.rrow = a.r ? a.r + base : nullptr;
  v.off = (int)(((uintptr_t)v.xrow >> 2) & 3);
  v.kmax = ((a.width + v.off + 3) >> 2) - 1;
  v.T = T;
  v.g0 = seg * T * C;
  v.li = threadIdx.x;
  v.width = a.width;
  return v;
}

// Loads of a segment: granules past the row's last one load the last one
// again (unconditional loads, masked by position), as in the row kernels.
// Empty asm statements keep the non-temporal copy of this block apart from
// the cached one (otherwise the optimizer merges them and drops the hint).
template <bool NT, int C>
__device__ __forceinline__ void load_segment(const SegArgs &a, const SegView &v, bool has_r, f32x4 (&xv)[C],
                                             f32x4 (&rv)[C]) {
  if constexpr (NT) asm volatile("" ::: "memory");
  const f32x4 *xw = reinterpret_cast<const f32x4 *>(v.xrow - v.off);
#pragma unroll
  for (int c = 0; c < C; ++c) xv[c] = load_g<NT>(xw + min(v.granule(c), v.kmax));
  if (has_r) {
    if (a.r_vec) {
      const f32x4 *rw = reinterpret_cast<const f32x4 *>(v.rrow - v.off);
#pragma unroll
      for (int c = 0; c < C; ++c) rv[c] = load_g<NT>(rw + min(v.granule(c), v.kmax));
    } else {
      const int emax = v.width - 1;
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) rv[c][j] = load_g<NT>(v.rrow + max(0, min(v.elem(c, j), emax)));
    }
  } else {
#pragma unroll
    for (int c = 0; c < C; ++c) rv[c] = f32x4(0.0f);
  }
  if constexpr (NT) asm volatile("" ::: "memory");
}

// x + r as an exact pair hi + lo (Knuth's TwoSum); 0 outside the row.
template <int C>
__device__ __forceinline__ void two_sum(const SegView &v, const f32x4 (&xv)[C], const f32x4 (&rv)[C],
                                        float (&hi)[4 * C], float (&lo)[4 * C]) {
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x = v.valid(c, j) ? xv[c][j] : 0.0f;
      const float r = v.valid(c, j) ? rv[c][j] : 0.0f;
      const float h = x + r;
      const float bb = h - x;
      hi[4 * c + j] = h;
      lo[4 * c + j] = (x - (h - bb)) + (r - bb);
    }
}

__device__ __forceinline__ Rec *records(const SegArgs &a) { return reinterpret_cast<Rec *>(a.ws); }
// One row record per row, after the rows * S segment records.
__device__ __forceinline__ Rec *row_records(const SegArgs &a) { return records(a) + a.rows * (int64_t)a.segments; }

// ---------------------------------------------------------------------------
// Statistics of one segment.
// ---------------------------------------------------------------------------
template <int OP, int C>
__global__ void __launch_bounds__(1024) seg_stats_kernel(SegArgs a) {
  __shared__ float partials[2][16];
  __shared__ double partials_d[16];
  const int T = blockDim.x;
  const int lanes_log2 = a.lanes_log2;
  int64_t row;
  int seg;
  segment_of(a, false, row, seg);
  const SegView v = make_view(a, row, seg, T, C);
  const bool has_r = OP == kOpLayerNorm && a.r != nullptr;
  f32x4 xv[C], rv[C];
  load_segment<false, C>(a, v, has_r, xv, rv);

  double v0 = 0.0, v1 = 0.0;
  if constexpr (OP == kOpRowSum) {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += v.valid(c, j) ? (double)xv[c][j] : 0.0;
    v0 = row_allreduce<SumOp>((acc[0] + acc[1]) + (acc[2] + acc[3]), lanes_log2, partials_d);
  } else if constexpr (OP == kOpRowMinMax) {
    float mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        mn = fminf(mn, v.valid(c, j) ? xv[c][j] : __builtin_inff());
        mx = fmaxf(mx, v.valid(c, j) ? xv[c][j] : -__builtin_inff());
      }
    row_allreduce_pair<MinOp, MaxOp>(mn, mx, lanes_log2, partials[0], partials[1]);
    v0 = mn;
    v1 = mx;
  } else if constexpr (OP == kOpRms) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = v.valid(c, j) ? xv[c][j] : 0.0f;
        acc[j] = fmaf(x, x, acc[j]);
      }
    v0 = row_allreduce<SumOp>((acc[0] + acc[1]) + (acc[2] + acc[3]), lanes_log2, partials[0]);
  } else if constexpr (OP == kOpSoftmax) {
    float m = -__builtin_inff();
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) m = fmaxf(m, v.valid(c, j) ? xv[c][j] : -__builtin_inff());
    m = row_allreduce<MaxOp>(m, lanes_log2, partials[0]);
    // -inf entries weigh 0 even in a segment whose max is -inf (where
    // x - m would be NaN); NaN and +inf entries give NaN, as in one pass.
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = xv[c][j];
        const bool zero = !v.valid(c, j) || x == -__builtin_inff();
        acc[j] += zero ? 0.0f : __builtin_amdgcn_exp2f((x - m) * kLog2e);
      }
    v0 = m;
    v1 = row_allreduce<SumOp>((acc[0] + acc[1]) + (acc[2] + acc[3]), lanes_log2, partials[1]);
  } else {  // LayerNorm: sum and sum of squares about the segment's own mean
    float hi[4 * C], lo[4 * C];
    two_sum<C>(v, xv, rv, hi, lo);
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    float acc_lo = 0.0f;
#pragma unroll
    for (int i = 0; i < 4 * C; ++i) {
      acc[i & 3] += (double)hi[i];
      acc_lo += lo[i];
    }
    const double sum =
        row_allreduce<SumOp>(((acc[0] + acc[1]) + (acc[2] + acc[3])) + (double)acc_lo, lanes_log2, partials_d);
    const int64_t n = segment_count(seg, (int64_t)T * C, v.off, a.width);
    const double mean = n > 0 ? sum / (double)n : 0.0;
    const float m_hi = (float)mean;
    const float m_lo = (float)(mean - (double)m_hi);
    float sq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * c + j;
        const float d = v.valid(c, j) ? (hi[i] - m_hi) + (lo[i] - m_lo) : 0.0f;
        sq[j] = fmaf(d, d, sq[j]);
      }
    v0 = sum;
    v1 = row_allreduce<SumOp>((sq[0] + sq[1]) + (sq[2] + sq[3]), lanes_log2, partials[0]);
  }
  if (threadIdx.x == 0) records(a)[row * a.segments + seg] = Rec{v0, v1};
}

// ---------------------------------------------------------------------------
// Fold a row's records: one wavefront per row, lanes stride over the
// records, then the wavefront butterfly.  Wavefronts past the last row
// return at once (no barrier in this kernel).  The loops over a row's
// records are unrolled so that a lane's loads issue together (S = 1024
// records take 16 per lane); the additions keep their order.
// ---------------------------------------------------------------------------
template <int OP>
__global__ void __launch_bounds__(256) seg_merge_kernel(SegArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int S = a.segments;
  const Rec *rec = records(a) + row * S;
  if constexpr (OP == kOpRowSum) {
    double s = 0.0;
#pragma unroll 16
    for (int k = lane; k < S; k += 64) s += rec[k].v0;
    s = group_allreduce<SumOp>(s, 6);
    if (lane == 0) a.y[row] = (float)s;
  } else if constexpr (OP == kOpRowMinMax) {
    float mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll 16
    for (int k = lane; k < S; k += 64) {
      mn = fminf(mn, (float)rec[k].v0);
      mx = fmaxf(mx, (float)rec[k].v1);
    }
    mn = group_allreduce<MinOp>(mn, 6);
    mx = group_allreduce<MaxOp>(mx, 6);
    if (lane == 0) {
      a.y[row] = mn;
      a.y2[row] = mx;
    }
  } else if constexpr (OP == kOpRms) {
    double s = 0.0;
#pragma unroll 16
    for (int k = lane; k < S; k += 64) s += rec[k].v0;
    s = group_allreduce<SumOp>(s, 6);
    if (lane == 0) row_records(a)[row] = Rec{s, 0.0};
  } else if constexpr (OP == kOpSoftmax) {
    float m = -__builtin_inff();
#pragma unroll 16
    for (int k = lane; k < S; k += 64) m = fmaxf(m, (float)rec[k].v0);
    m = group_allreduce<MaxOp>(m, 6);
    // An all -inf row has m = -inf and s_k = 0 everywhere: 0 * exp(NaN)
    // makes s NaN, and the row NaN, as in one pass.  The sum is FP64: a row
    // of 2^31 columns has 2^19 segments, 2^13 per lane.
    double s = 0.0;
#pragma unroll 16
    for (int k = lane; k < S; k += 64)
      s += rec[k].v1 * (double)__builtin_amdgcn_exp2f(((float)rec[k].v0 - m) * kLog2e);
    s = group_allreduce<SumOp>(s, 6);
    if (lane == 0) row_records(a)[row] = Rec{(double)m, (double)s};
  } else {  // LayerNorm
    const int off = (int)((((uintptr_t)a.x >> 2) + row * (int64_t)a.width) & 3);
    double s = 0.0;
#pragma unroll 16
    for (int k = lane; k < S; k += 64) s += rec[k].v0;
    s = group_allreduce<SumOp>(s, 6);
    const double mean = s / (double)a.width;
    double m2 = 0.0;
#pragma unroll 16
    for (int k = lane; k < S; k += 64) {
      const int64_t n = segment_count(k, a.seg_granules, off, a.width);
      if (n > 0) {
        const double dm = rec[k].v0 / (double)n - mean;
        m2 += rec[k].v1 + (double)n * dm * dm;
      }
    }
    m2 = group_allreduce<SumOp>(m2, 6);
    if (lane == 0) row_records(a)[row] = Rec{mean, m2};
  }
}

// ---------------------------------------------------------------------------
// Apply a row record to one segment held in registers and store it.
// ---------------------------------------------------------------------------
// PAIR (LayerNorm): xv and rv already hold the TwoSum pair (hi, lo) of x + r.
// The exchange words in y's rows (defined with the exchange kernels below).
__device__ __forceinline__ bool holds_row_words(const SegArgs &a, int64_t row, int rounds, int e0);

// HOLD (LayerNorm exchange) with rounds > 0 (segment 0 with the words in
// y): slot 0's granule is not stored where it overlaps the words (the
// workgroup that completes the row stores it).  Without HOLD the code is
// that of a plain apply.
template <int OP, int C, bool PAIR = false, bool HOLD = false>
__device__ __forceinline__ void apply_store(const SegArgs &a, const SegView &v, int64_t row, const f32x4 (&xv)[C],
                                            const f32x4 (&rv)[C], Rec rr, int rounds = 0) {
  float s[4 * C];
  if constexpr (OP == kOpRms) {
    const float scale = __builtin_amdgcn_rsqf(fmaf((float)rr.v0, a.inv_width, a.eps));
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) s[4 * c + j] = xv[c][j] * scale;
  } else if constexpr (OP == kOpSoftmax) {
    const float m = (float)rr.v0;
    const float inv = __builtin_amdgcn_rcpf((float)rr.v1);
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) s[4 * c + j] = __builtin_amdgcn_exp2f((xv[c][j] - m) * kLog2e) * inv;
  } else {  // LayerNorm, optionally affine
    const double mean = rr.v0;
    const float m_hi = (float)mean;
    const float m_lo = (float)(mean - (double)m_hi);
    const float rstd = __builtin_amdgcn_rsqf(fmaf((float)rr.v1, a.inv_width, a.eps));
    float hi[4 * C], lo[4 * C];
    if constexpr (PAIR) {
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          hi[4 * c + j] = xv[c][j];
          lo[4 * c + j] = rv[c][j];
        }
    } else {
      two_sum<C>(v, xv, rv, hi, lo);
    }
    // two loops, so that gamma / beta take no registers without them
    if (a.gamma != nullptr || a.beta != nullptr) {
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const f32x4 g = affine_slot(a.gamma, v.elem(c, 0), a.width, 1.0f);
        const f32x4 b = affine_slot(a.beta, v.elem(c, 0), a.width, 0.0f);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * c + j;
          s[i] = fmaf(((hi[i] - m_hi) + (lo[i] - m_lo)) * rstd, g[j], b[j]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4 * C; ++i) s[i] = ((hi[i] - m_hi) + (lo[i] - m_lo)) * rstd;
    }
  }

  bool skip0 = false;
  if constexpr (HOLD) skip0 = rounds > 0 && holds_row_words(a, row, rounds, v.elem(0, 0));
  auto store = [&](auto nt) {
    constexpr bool NT = decltype(nt)::value;
    float *yrow = a.y + row * (int64_t)a.width;
    if (a.y_vec) {
      f32x4 *yw = reinterpret_cast<f32x4 *>(yrow - v.off);
#pragma unroll
      for (int c = 0; c < C; ++c) {
        if constexpr (HOLD) {
          if (c == 0 && skip0) continue;
        }
        const int k = v.granule(c);
        const int e0 = 4 * k - v.off;
        if (e0 >= 0 && e0 + 4 <= a.width) {
          store_g<NT>(yw + k, f32x4{s[4 * c], s[4 * c + 1], s[4 * c + 2], s[4 * c + 3]});
        } else if (k <= v.kmax) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if ((unsigned)(e0 + j) < (unsigned)a.width) store_g<NT>(yrow + e0 + j, s[4 * c + j]);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < C; ++c) {
        if constexpr (HOLD) {
          if (c == 0 && skip0) continue;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (v.valid(c, j)) store_g<NT>(yrow + v.elem(c, j), s[4 * c + j]);
      }
    }
  };
  if (a.policy & kPolicyNtStores) store(std::true_type{});
  else store(std::false_type{});
}

// ---------------------------------------------------------------------------
// Apply the row record to one segment and store it.
// ---------------------------------------------------------------------------
template <int OP, int C>
__global__ void __launch_bounds__(1024) seg_apply_kernel(SegArgs a) {
  const int T = blockDim.x;
  int64_t row;
  int seg;
  segment_of(a, (a.policy & kPolicyReverse) != 0, row, seg);
  const SegView v = make_view(a, row, seg, T, C);
  const bool has_r = OP == kOpLayerNorm && a.r != nullptr;
  f32x4 xv[C], rv[C];
  if (a.policy & kPolicyNtLoads) load_segment<true, C>(a, v, has_r, xv, rv);
  else load_segment<false, C>(a, v, has_r, xv, rv);
  apply_store<OP, C>(a, v, row, xv, rv, row_records(a)[row]);
}

// ---------------------------------------------------------------------------
// One-kernel split rows (ROWRED_POLICY_EXCHANGE).  Each workgroup keeps its
// segment in registers; the S workgroups of a row swap their statistics
// through the workspace, and each folds all S of them in the same fixed
// order, so every segment applies bitwise the same row record and x (and r)
// are read once.
//
// Workspace, 64-bit words: word 0 is a status word (nonzero after a wait
// gave up), then one slot per (round, row, segment).  A slot holds 0 until
// its owner publishes.  A published slot holds the complement of the value's
// bits, NaN made canonical first, which is never 0; value and flag are one
// word, so relaxed agent-scope atomics order them.  A clear kernel zeroes the
// words before every launch.
//
// One exchange per kernel: RMSNorm publishes the segment's sum of squares;
// softmax its pair (max m_k, sum of exp(x - m_k)) as two floats in one word;
// LayerNorm two words, its sum of x + r and its sum of squares about its own
// mean (slots of rounds 0 and 1), each waited for on its own.  The pairs and
// the LayerNorm records merge as in the split kernels (Chan, Golub and
// LeVeque for LayerNorm).
//
// Waiting on other workgroups needs them to run.  Workgroups reach each XCD
// in index order and a row's segments have consecutive indices, so a
// segment that is not yet resident waits only for workgroups of its own row
// or of earlier rows, and earlier rows can all finish: the oldest waiting
// row always completes.  S is capped (kMaxExchangeSegments) far below the
// workgroups the chip holds at once.  Every wait is bounded all the same:
// after a.spin_limit polls (kExchangeSpinLimit unless the host overrides
// it) a lane gives up, sets the status word and the row comes out NaN.
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint64_t encode(double v) {
  if (v != v) v = __builtin_nan("");
  return ~__builtin_bit_cast(uint64_t, v);
}
__device__ __forceinline__ double decode(uint64_t w) { return __builtin_bit_cast(double, ~w); }
__device__ __forceinline__ uint64_t encode_pair(float m, float s) {
  if (m != m) m = __builtin_nanf("");
  if (s != s) s = __builtin_nanf("");
  return ~(((uint64_t)__builtin_bit_cast(uint32_t, s) << 32) | __builtin_bit_cast(uint32_t, m));
}

// The exchange words of a row kept in y itself (ws_in_y): from the first
// 16-byte boundary of the row's outputs.
// (Pointer arithmetic, not an integer round trip, so that the compiler keeps
// the global address space and emits global, not flat, accesses.)
__device__ __forceinline__ uint64_t *row_words(const SegArgs &a, int64_t row) {
  float *yrow = a.y + row * (int64_t)a.width;
  const int pad = (int)((16 - (reinterpret_cast<uintptr_t>(yrow) & 15)) & 15);
  return reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(yrow) + pad);
}

__device__ __forceinline__ uint64_t *exchange_slots(const SegArgs &a, int round, int64_t row) {
  if (a.ws_in_y) return row_words(a, row) + (int64_t)round * a.segments;
  return reinterpret_cast<uint64_t *>(a.ws) + 1 + ((int64_t)round * a.rows + row) * a.segments;
}

// With the words in y's row, their granules may be stored only once every
// segment of the row has read them.  Each workgroup counts itself done after
// its fold -- every lane's slot reads have returned by then: the fold's
// barrier (or, for one wavefront, program order) follows the values' use, so
// a relaxed count suffices.  Two ways to honour the count:
//  - RMSNorm and softmax (one round of words): segment 0 waits for the count
//    to reach S (bounded like the slot waits) before any of its stores
//    (release_row_words); the other workgroups add to it without waiting
//    for the result.
//  - LayerNorm (two rounds, a longer wait): every workgroup learns whether
//    its count completed the row (count_row_words_read); segment 0 leaves
//    its first-slot granules over the words unstored (the host keeps the
//    words within them) and the completing workgroup stores them
//    (finish_row_words), so no workgroup waits for another.  One returning
//    atomic per workgroup: measured faster for LayerNorm (residual
//    1024x65536 137.0 -> 133.6 us, 4096x32768 260.0 -> 255.5 us), slower
//    for softmax (8192x32768 340.0 -> 343.2 us) and RMSNorm.
//
// The wait: true when it gave up; the caller then writes NaN over the row's
// segment (segments that had not read yet may see outputs as words).
__device__ __forceinline__ bool release_row_words(const SegArgs &a, int64_t row, int seg, int rounds) {
  if (!a.ws_in_y) return false;
  __shared__ int gave_up;
  uint64_t *done = row_words(a, row) + (int64_t)rounds * a.segments;
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(done, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (seg != 0) return false;  // uniform over the workgroup
  if (threadIdx.x == 0) {
    uint64_t n = __hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t it = 0;
#pragma nounroll
    for (; n < (uint64_t)a.segments && it < a.spin_limit; ++it) {
      __builtin_amdgcn_s_sleep(2);
      n = __hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    gave_up = n < (uint64_t)a.segments ? 1 : 0;
  }
  __syncthreads();
  return gave_up != 0;
}

// The count that completes the row: true in wavefront 0 of the workgroup
// whose count completed it, false elsewhere.
__device__ __forceinline__ bool count_row_words_read(const SegArgs &a, int64_t row, int rounds) {
  uint64_t old = 0;
  if (threadIdx.x == 0)
    old = __hip_atomic_fetch_add(row_words(a, row) + (int64_t)rounds * a.segments, (uint64_t)1, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
  if (threadIdx.x >= 64) return false;
  return __builtin_amdgcn_readfirstlane(old + 1 == (uint64_t)a.segments ? 1 : 0) != 0;
}

// Whether segment 0's first-slot granule starting at row element e0 overlaps
// the row's words (it is then stored by finish_row_words).
__device__ __forceinline__ bool holds_row_words(const SegArgs &a, int64_t row, int rounds, int e0) {
  const char *yrow = reinterpret_cast<const char *>(a.y + row * (int64_t)a.width);
  const char *end = reinterpret_cast<const char *>(row_words(a, row) + (int64_t)rounds * a.segments + 1);
  return 4 * (int64_t)e0 < end - yrow;
}

// Wavefront 0 of the workgroup that completed the row: segment 0's granules
// over the words, recomputed from x (and r, gamma, beta) with the row record
// by the arithmetic of the exchange kernels' output map, and stored as
// segment 0 stores them.  Cached loads: a few granules per row.
template <int OP>
__device__ __forceinline__ void finish_row_words(const SegArgs &a, int64_t row, Rec rr, int rounds) {
  const float *xrow = a.x + row * (int64_t)a.width;
  const float *rrow = a.r ? a.r + row * (int64_t)a.width : nullptr;
  float *yrow = a.y + row * (int64_t)a.width;
  const int off = (int)(((uintptr_t)xrow >> 2) & 3);
  const int kmax = ((a.width + off + 3) >> 2) - 1;
  const char *end = reinterpret_cast<const char *>(row_words(a, row) + (int64_t)rounds * a.segments + 1);
  const int held = (int)((end - reinterpret_cast<const char *>(yrow) + 3) / 4);  // elements [0, held)
  const int kh = (held + off + 3) >> 2;                                          // granules [0, kh)
  float scale = 0.0f, m = 0.0f, m_hi = 0.0f, m_lo = 0.0f;
  if constexpr (OP == kOpRms) {
    scale = __builtin_amdgcn_rsqf(fmaf((float)rr.v0, a.inv_width, a.eps));
  } else if constexpr (OP == kOpSoftmax) {
    m = (float)rr.v0;
    scale = __builtin_amdgcn_rcpf((float)rr.v1);
  } else {
    m_hi = (float)rr.v0;
    m_lo = (float)(rr.v0 - (double)m_hi);
    scale = __builtin_amdgcn_rsqf(fmaf((float)rr.v1, a.inv_width, a.eps));
  }
  const bool affine = OP == kOpLayerNorm && (a.gamma != nullptr || a.beta != nullptr);
  for (int k = (int)threadIdx.x; k < kh; k += 64) {
    const int e0 = 4 * k - off;
    const f32x4 xx = reinterpret_cast<const f32x4 *>(xrow - off)[k < kmax ? k : kmax];
    float o[4];
    if constexpr (OP == kOpRms) {
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = xx[j] * scale;
    } else if constexpr (OP == kOpSoftmax) {
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = __builtin_amdgcn_exp2f((xx[j] - m) * kLog2e) * scale;
    } else {
      f32x4 r4 = f32x4(0.0f);
      if (rrow) {
        if (a.r_vec) {
          r4 = reinterpret_cast<const f32x4 *>(rrow - off)[k < kmax ? k : kmax];
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) r4[j] = rrow[max(0, min(e0 + j, a.width - 1))];
        }
      }
      f32x4 g = f32x4(1.0f), b = f32x4(0.0f);
      if (affine) {
        g = affine_slot(a.gamma, e0, a.width, 1.0f);
        b = affine_slot(a.beta, e0, a.width, 0.0f);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = xx[j], r = r4[j];
        const float h = x + r;  // TwoSum, as the exchange kernels form the pair
        const float bb = h - x;
        const float l = (x - (h - bb)) + (r - bb);
        const float y = ((h - m_hi) + (l - m_lo)) * scale;
        o[j] = affine ? fmaf(y, g[j], b[j]) : y;
      }
    }
    if (a.y_vec && e0 >= 0 && e0 + 4 <= a.width) {
      reinterpret_cast<f32x4 *>(yrow - off)[k] = f32x4{o[0], o[1], o[2], o[3]};
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if ((unsigned)(e0 + j) < (unsigned)a.width) yrow[e0 + j] = o[j];
    }
  }
}

__device__ __forceinline__ void publish(uint64_t *slot, uint64_t w) {
  if (threadIdx.x == 0) __hip_atomic_store(slot, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Lane k < S of the workgroup waits for slot k and returns its word; other
// lanes return 0 without touching memory.  A lane that gives up returns 0
// (decoded: NaN) and raises the status word.
__device__ __forceinline__ uint64_t await_slot(const SegArgs &a, const uint64_t *slots) {
  const int k = threadIdx.x;
  if (k >= a.segments) return 0;
  uint64_t w = __hip_atomic_load(slots + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma nounroll
  for (uint32_t it = 0; w == 0; ++it) {
    if (it >= a.spin_limit) {
      if (!a.ws_in_y)  // words in y's rows have no status word: the row turns NaN only
        __hip_atomic_store(reinterpret_cast<uint64_t *>(a.ws), (uint64_t)1, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
    w = __hip_atomic_load(slots + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return w;
}

// Row sum of one published double per segment: every workgroup of the row
// gets the same bits (same lanes, same reduction tree).
__device__ __forceinline__ double exchange_sum(const SegArgs &a, const uint64_t *slots, double *partials) {
  const bool mine = (int)threadIdx.x < a.segments;
  const uint64_t w = await_slot(a, slots);
  return row_allreduce<SumOp>(mine ? decode(w) : 0.0, a.lanes_log2, partials);
}

// The row's softmax record from the S published pairs: m = max m_k,
// s = sum s_k exp(m_k - m), the same bits in every segment.
__device__ __forceinline__ Rec softmax_row_record(const SegArgs &a, const uint64_t *slots, int lanes_log2,
                                                  float *pm, float *ps) {
  const bool mine = (int)threadIdx.x < a.segments;
  const uint64_t w = ~await_slot(a, slots);
  const float mk = mine ? __builtin_bit_cast(float, (uint32_t)w) : -__builtin_inff();
  const float sk = mine ? __builtin_bit_cast(float, (uint32_t)(w >> 32)) : 0.0f;
  const float mrow = row_allreduce<MaxOp>(mk, lanes_log2, pm);
  // An all -inf row has mrow = -inf and s_k = 0: 0 * exp(NaN) is NaN, and
  // so is the row, as in one pass.
  const float t = mine ? sk * __builtin_amdgcn_exp2f((mk - mrow) * kLog2e) : 0.0f;
  return Rec{(double)mrow, (double)row_allreduce<SumOp>(t, lanes_log2, ps)};
}

// The row's LayerNorm record (mean, M2) from the S published (sum, M2)
// words, segments of G granules of a row at phase `off`: Chan, Golub and
// LeVeque's merge, the same bits in every segment.  p1 and p0 are the LDS
// partials of its two reductions.
__device__ __forceinline__ Rec layernorm_row_record(const SegArgs &a, const uint64_t *slots0, const uint64_t *slots1,
                                                    int64_t G, int off, int lanes_log2, double *p1, double *p0) {
  // Both words of segment k, each written once: wait for each.
  const int k = threadIdx.x;
  const bool mine = k < a.segments;
  const double sum_k = decode(await_slot(a, slots0));
  const double m2_k = decode(await_slot(a, slots1));
  const double mean = row_allreduce<SumOp>(mine ? sum_k : 0.0, lanes_log2, p1) / (double)a.width;
  const int64_t n_k = mine ? segment_count(k, G, off, a.width) : 0;
  double t = 0.0;
  if (n_k > 0) {
    const double dm = sum_k / (double)n_k - mean;
    t = m2_k + (double)n_k * dm * dm;
  } else if (mine) {
    t = m2_k + sum_k;  // 0 + 0, but a wait that gave up still turns the row NaN
  }
  return Rec{mean, row_allreduce<SumOp>(t, lanes_log2, p0)};
}

template <int OP, int C>
__global__ void __launch_bounds__(C >= 8 ? 512 : 1024) seg_exchange_kernel(SegArgs a) {
  __shared__ float partials[4][16];
  __shared__ double partials_d[2][16];
  const int T = blockDim.x;
  const int lanes_log2 = a.lanes_log2;
  int64_t row;
  int seg;
  segment_of(a, false, row, seg);
  const SegView v = make_view(a, row, seg, T, C);
  const bool has_r = OP == kOpLayerNorm && a.r != nullptr;
  f32x4 xv[C], rv[C];
  if (a.policy & kPolicyNtLoads) load_segment<true, C>(a, v, has_r, xv, rv);
  else load_segment<false, C>(a, v, has_r, xv, rv);

  Rec rr;
  if constexpr (OP == kOpRms) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = v.valid(c, j) ? xv[c][j] : 0.0f;
        acc[j] = fmaf(x, x, acc[j]);
      }
    const float sq = row_allreduce<SumOp>((acc[0] + acc[1]) + (acc[2] + acc[3]), lanes_log2, partials[0]);
    uint64_t *slots = exchange_slots(a, 0, row);
    publish(slots + seg, encode((double)sq));
    rr = Rec{exchange_sum(a, slots, partials_d[0]), 0.0};
  } else if constexpr (OP == kOpSoftmax) {
    float m = -__builtin_inff();
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) m = fmaxf(m, v.valid(c, j) ? xv[c][j] : -__builtin_inff());
    m = row_allreduce<MaxOp>(m, lanes_log2, partials[0]);
    // -inf entries weigh 0 even in a segment whose max is -inf; NaN and
    // +inf entries give NaN, as in one pass.
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = xv[c][j];
        const bool zero = !v.valid(c, j) || x == -__builtin_inff();
        acc[j] += zero ? 0.0f : __builtin_amdgcn_exp2f((x - m) * kLog2e);
      }
    const float s = row_allreduce<SumOp>((acc[0] + acc[1]) + (acc[2] + acc[3]), lanes_log2, partials[1]);
    uint64_t *slots = exchange_slots(a, 0, row);
    publish(slots + seg, encode_pair(m, s));
    rr = softmax_row_record(a, slots, lanes_log2, partials[2], partials[3]);
  } else {  // LayerNorm: (sum, squares about the segment mean), merged as the split kernels merge them
    float hi[4 * C], lo[4 * C];
    two_sum<C>(v, xv, rv, hi, lo);
    // from here on the segment lives as the pair: x and r are dropped
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xv[c][j] = hi[4 * c + j];
        rv[c][j] = lo[4 * c + j];
      }
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    float acc_lo = 0.0f;
#pragma unroll
    for (int i = 0; i < 4 * C; ++i) {
      acc[i & 3] += (double)hi[i];
      acc_lo += lo[i];
    }
    const double sum =
        row_allreduce<SumOp>(((acc[0] + acc[1]) + (acc[2] + acc[3])) + (double)acc_lo, lanes_log2, partials_d[0]);
    const int64_t G = (int64_t)T * C;
    const int64_t n = segment_count(seg, G, v.off, a.width);
    const double seg_mean = n > 0 ? sum / (double)n : 0.0;
    const float s_hi = (float)seg_mean;
    const float s_lo = (float)(seg_mean - (double)s_hi);
    float sq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * c + j;
        const float d = v.valid(c, j) ? (hi[i] - s_hi) + (lo[i] - s_lo) : 0.0f;
        sq[j] = fmaf(d, d, sq[j]);
      }
    const float m2 = row_allreduce<SumOp>((sq[0] + sq[1]) + (sq[2] + sq[3]), lanes_log2, partials[0]);
    uint64_t *slots0 = exchange_slots(a, 0, row);
    uint64_t *slots1 = exchange_slots(a, 1, row);
    publish(slots0 + seg, encode(sum));
    publish(slots1 + seg, encode((double)m2));
    // partials_d[0] again: every wave read it before the barrier that
    // partials_d[1]'s reduction passed.
    rr = layernorm_row_record(a, slots0, slots1, G, v.off, lanes_log2, partials_d[1], partials_d[0]);
  }
  if constexpr (OP == kOpLayerNorm) {
    const bool last = a.ws_in_y && count_row_words_read(a, row, 2);
    apply_store<OP, C, true, true>(a, v, row, xv, rv, rr, a.ws_in_y && seg == 0 ? 2 : 0);
    if (last) finish_row_words<OP>(a, row, rr, 2);  // wavefront 0 of the row's last workgroup
  } else {
    if (release_row_words(a, row, seg, 1)) rr = Rec{__builtin_nan(""), __builtin_nan("")};
    apply_store<OP, C>(a, v, row, xv, rv, rr);
  }
}

// ---------------------------------------------------------------------------
// Exchange kernels with part of the segment in LDS (ROWRED_POLICY_EXCHANGE |
// ROWRED_POLICY_LDS_STRIPE), 256 threads: a lane's slots 0..CR-1 stay in
// registers and slots CR..CR+CL-1 go straight from HBM into LDS (x, and r
// for LayerNorm) with 16-byte LDS-writing loads; each lane reads back only
// its own LDS slots, so that needs no barrier.  A segment carries (CR + CL)
// slots per lane for the registers of CR: fewer segments per row and more
// bytes in flight per CU.  Statistics, their exchange and the merges are
// those of seg_exchange_kernel.
// ---------------------------------------------------------------------------
template <int OP, int CR, int CL>
__global__ void __launch_bounds__(kXldsThreads) seg_xlds_kernel(SegArgs a) {
  constexpr int T = kXldsThreads;
  constexpr int C = CR + CL;
  constexpr bool kLN = OP == kOpLayerNorm;
  constexpr int lanes_log2 = 8;
  __shared__ f32x4 held_x[CL * T];
  __shared__ f32x4 held_r[kLN ? CL * T : 1];
  __shared__ float partials[4][16];
  __shared__ double partials_d[2][16];
  typedef __attribute__((address_space(3))) void lds_void;
  int64_t row;
  int seg;
  segment_of(a, false, row, seg);
  const SegView v = make_view(a, row, seg, T, C);
  const int li = threadIdx.x;
  const bool has_r = kLN && a.r != nullptr;
  f32x4 *wave_x = held_x + (li & ~63);  // lane l of the wave lands at entry l
  f32x4 *wave_r = held_r + (li & ~63);

  f32x4 xv[CR], rv[CR];
  auto load_all = [&](auto nt) {
    constexpr bool NT = decltype(nt)::value;
    if constexpr (NT) asm volatile("" ::: "memory");
    const f32x4 *xw = reinterpret_cast<const f32x4 *>(v.xrow - v.off);
#pragma unroll
    for (int c = 0; c < CL; ++c)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(xw + min(v.granule(CR + c), v.kmax)),
                                       (lds_void *)(wave_x + c * T), 16, 0, NT ? 2 : 0);
    if constexpr (kLN) {
      if (has_r && a.r_vec) {
        const f32x4 *rw = reinterpret_cast<const f32x4 *>(v.rrow - v.off);
#pragma unroll
        for (int c = 0; c < CL; ++c)
          __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(rw + min(v.granule(CR + c), v.kmax)),
                                           (lds_void *)(wave_r + c * T), 16, 0, NT ? 2 : 0);
      }
    }
#pragma unroll
    for (int c = 0; c < CR; ++c) xv[c] = load_g<NT>(xw + min(v.granule(c), v.kmax));
    if (has_r) {
      if (a.r_vec) {
        const f32x4 *rw = reinterpret_cast<const f32x4 *>(v.rrow - v.off);
#pragma unroll
        for (int c = 0; c < CR; ++c) rv[c] = load_g<NT>(rw + min(v.granule(c), v.kmax));
      } else {
        const int emax = v.width - 1;
#pragma unroll
        for (int c = 0; c < CR; ++c)
#pragma unroll
          for (int j = 0; j < 4; ++j) rv[c][j] = load_g<NT>(v.rrow + max(0, min(v.elem(c, j), emax)));
      }
    } else {
#pragma unroll
      for (int c = 0; c < CR; ++c) rv[c] = f32x4(0.0f);
    }
    if constexpr (NT) asm volatile("" ::: "memory");
  };
  if (a.policy & kPolicyNtLoads) load_all(std::true_type{});
  else load_all(std::false_type{});
  // The LDS writes of those loads are done once the loads have completed.
  __builtin_amdgcn_s_waitcnt(0);
  if constexpr (kLN) {
    if (has_r && !a.r_vec) {
      // r at another 16-byte phase than x: 4-byte loads into the lane's own
      // LDS slots
      const int emax = v.width - 1;
#pragma unroll
      for (int c = 0; c < CL; ++c) {
        f32x4 t;
#pragma unroll
        for (int j = 0; j < 4; ++j) t[j] = v.rrow[max(0, min(v.elem(CR + c, j), emax))];
        held_r[c * T + li] = t;
      }
    }
  }
  // Elements outside the row take the reduction's identity here, once (x and
  // r 0; softmax x -inf), so that the phases below need no per-element masks
  // (LayerNorm's squares and the stores excepted).
  constexpr float kIdent = OP == kOpSoftmax ? -__builtin_inff() : 0.0f;
#pragma unroll
  for (int c = 0; c < CR; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool in = v.valid(c, j);
      xv[c][j] = in ? xv[c][j] : kIdent;
      if constexpr (kLN) rv[c][j] = in ? rv[c][j] : 0.0f;
    }
#pragma unroll
  for (int c = 0; c < CL; ++c) {
    f32x4 t = held_x[c * T + li];
#pragma unroll
    for (int j = 0; j < 4; ++j) t[j] = v.valid(CR + c, j) ? t[j] : kIdent;
    held_x[c * T + li] = t;
    if constexpr (kLN) {
      if (has_r) {
        f32x4 u = held_r[c * T + li];
#pragma unroll
        for (int j = 0; j < 4; ++j) u[j] = v.valid(CR + c, j) ? u[j] : 0.0f;
        held_r[c * T + li] = u;
      }
    }
  }
  // Slot c of the lane, from registers or LDS (c is a constant once unrolled).
  auto x_at = [&](int c) -> f32x4 { return c < CR ? xv[c < CR ? c : 0] : held_x[(c - CR) * T + li]; };
  auto r_at = [&](int c) -> f32x4 {
    if constexpr (!kLN) {
      return f32x4(0.0f);
    } else {
      if (!has_r) return f32x4(0.0f);
      return c < CR ? rv[c < CR ? c : 0] : held_r[(c - CR) * T + li];
    }
  };
  // x + r as the exact pair (h, l) (TwoSum); 0 outside the row.
  auto pair = [&](const f32x4 &xx, const f32x4 &rr_, int j, float &h, float &l) {
    const float x = xx[j];
    const float r = rr_[j];
    h = x + r;
    const float bb = h - x;
    l = (x - (h - bb)) + (r - bb);
  };
  // After each LDS slot: keep the compiler from reading every LDS slot up
  // front, which would hold them all in registers at once.
  auto slot_done = [&](int c) {
    if (c >= CR) __builtin_amdgcn_sched_barrier(0);
  };

  Rec rr;
  float m = 0.0f;
  if constexpr (OP == kOpRms) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const f32x4 xx = x_at(c);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = fmaf(xx[j], xx[j], acc[j]);
      slot_done(c);
    }
    const float sq = row_allreduce<SumOp>((acc[0] + acc[1]) + (acc[2] + acc[3]), lanes_log2, partials[0]);
    uint64_t *slots = exchange_slots(a, 0, row);
    publish(slots + seg, encode((double)sq));
    rr = Rec{exchange_sum(a, slots, partials_d[0]), 0.0};
  } else if constexpr (OP == kOpSoftmax) {
    m = -__builtin_inff();
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const f32x4 xx = x_at(c);
#pragma unroll
      for (int j = 0; j < 4; ++j) m = fmaxf(m, xx[j]);
      slot_done(c);
    }
    m = row_allreduce<MaxOp>(m, lanes_log2, partials[0]);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const f32x4 xx = x_at(c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool zero = xx[j] == -__builtin_inff();  // outside the row too
        acc[j] += zero ? 0.0f : __builtin_amdgcn_exp2f((xx[j] - m) * kLog2e);
      }
      slot_done(c);
    }
    const float s = row_allreduce<SumOp>((acc[0] + acc[1]) + (acc[2] + acc[3]), lanes_log2, partials[1]);
    uint64_t *slots = exchange_slots(a, 0, row);
    publish(slots + seg, encode_pair(m, s));
    rr = softmax_row_record(a, slots, lanes_log2, partials[2], partials[3]);
  } else {  // LayerNorm
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    float acc_lo = 0.0f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const f32x4 xx = x_at(c), r4 = r_at(c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float h, l;
        pair(xx, r4, j, h, l);
        acc[j] += (double)h;
        acc_lo += l;
      }
      slot_done(c);
    }
    const double sum =
        row_allreduce<SumOp>(((acc[0] + acc[1]) + (acc[2] + acc[3])) + (double)acc_lo, lanes_log2, partials_d[0]);
    const int64_t G = (int64_t)T * C;
    const int64_t n = segment_count(seg, G, v.off, a.width);
    const double seg_mean = n > 0 ? sum / (double)n : 0.0;
    const float s_hi = (float)seg_mean;
    const float s_lo = (float)(seg_mean - (double)s_hi);
    float sq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const f32x4 xx = x_at(c), r4 = r_at(c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float h, l;
        pair(xx, r4, j, h, l);
        const float d = v.valid(c, j) ? (h - s_hi) + (l - s_lo) : 0.0f;
        sq[j] = fmaf(d, d, sq[j]);
      }
      slot_done(c);
    }
    const float m2 = row_allreduce<SumOp>((sq[0] + sq[1]) + (sq[2] + sq[3]), lanes_log2, partials[0]);
    uint64_t *slots0 = exchange_slots(a, 0, row);
    uint64_t *slots1 = exchange_slots(a, 1, row);
    publish(slots0 + seg, encode(sum));
    publish(slots1 + seg, encode((double)m2));
    rr = layernorm_row_record(a, slots0, slots1, G, v.off, lanes_log2, partials_d[1], partials_d[0]);
  }
  // LayerNorm, segment 0 with the words in y: its first-slot granule over
  // them is left to the workgroup that completes the row; RMSNorm and
  // softmax: segment 0 waits for the row's reads before its stores
  bool last = false, skip0 = false;
  if constexpr (kLN) {
    last = a.ws_in_y && count_row_words_read(a, row, 2);
    skip0 = a.ws_in_y && seg == 0 && holds_row_words(a, row, 2, v.elem(0, 0));
  } else {
    if (release_row_words(a, row, seg, 1)) rr = Rec{__builtin_nan(""), __builtin_nan("")};
  }

  // ---- map and store, slot by slot.
  float scale = 0.0f, m_hi = 0.0f, m_lo = 0.0f;
  if constexpr (OP == kOpRms) {
    scale = __builtin_amdgcn_rsqf(fmaf((float)rr.v0, a.inv_width, a.eps));
  } else if constexpr (OP == kOpSoftmax) {
    m = (float)rr.v0;
    scale = __builtin_amdgcn_rcpf((float)rr.v1);
  } else {
    m_hi = (float)rr.v0;
    m_lo = (float)(rr.v0 - (double)m_hi);
    scale = __builtin_amdgcn_rsqf(fmaf((float)rr.v1, a.inv_width, a.eps));
  }
  const bool affine = kLN && (a.gamma != nullptr || a.beta != nullptr);
  auto map_slot = [&](int c, float (&o)[4]) {
    const f32x4 xx = x_at(c);
    if constexpr (OP == kOpRms) {
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = xx[j] * scale;
    } else if constexpr (OP == kOpSoftmax) {
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = __builtin_amdgcn_exp2f((xx[j] - m) * kLog2e) * scale;
    } else {
      const f32x4 r4 = r_at(c);
      // two loops, so that gamma / beta take no registers without them
      if (affine) {
        const f32x4 g = affine_slot(a.gamma, v.elem(c, 0), a.width, 1.0f);
        const f32x4 b = affine_slot(a.beta, v.elem(c, 0), a.width, 0.0f);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float h, l;
          pair(xx, r4, j, h, l);
          o[j] = fmaf(((h - m_hi) + (l - m_lo)) * scale, g[j], b[j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float h, l;
          pair(xx, r4, j, h, l);
          o[j] = ((h - m_hi) + (l - m_lo)) * scale;
        }
      }
    }
  };
  auto store_all = [&](auto nt) {
    constexpr bool NT = decltype(nt)::value;
    float *yrow = a.y + row * (int64_t)a.width;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      if (c == 0 && skip0) continue;
      float o[4];
      map_slot(c, o);
      const int k = v.granule(c);
      const int e0 = 4 * k - v.off;
      if (a.y_vec) {
        if (e0 >= 0 && e0 + 4 <= a.width) {
          store_g<NT>(reinterpret_cast<f32x4 *>(yrow - v.off) + k, f32x4{o[0], o[1], o[2], o[3]});
        } else if (k <= v.kmax) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if ((unsigned)(e0 + j) < (unsigned)a.width) store_g<NT>(yrow + e0 + j, o[j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (v.valid(c, j)) store_g<NT>(yrow + v.elem(c, j), o[j]);
      }
      slot_done(c);
    }
  };
  if (a.policy & kPolicyNtStores) store_all(std::true_type{});
  else store_all(std::false_type{});
  if constexpr (kLN) {
    if (last) finish_row_words<OP>(a, row, rr, 2);  // wavefront 0 of the row's last workgroup
  }
}

// Zero the 64-bit words [first, 2 * n128) of the exchange area (16-byte
// aligned): first = 0 clears the status word with the slots, first = 1 the
// slots only.
__global__ void __launch_bounds__(256) exchange_clear_kernel(uint64_t *w, int64_t first, int64_t n128) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
  if (i >= n128) return;
  if (i == 0 && first == 1) w[1] = 0;  // keep the status word
  else reinterpret_cast<u64x2 *>(w)[i] = u64x2{0, 0};
}

// Zero `words` 64-bit words of each row's exchange area in y (ws_in_y).
__global__ void __launch_bounds__(256) exchange_clear_row_words_kernel(float *y, int64_t rows, int32_t width,
                                                                       int32_t words) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * words) return;
  const int64_t row = i / words;
  float *yrow = y + row * (int64_t)width;
  const int pad = (int)((16 - (reinterpret_cast<uintptr_t>(yrow) & 15)) & 15);
  reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(yrow) + pad)[i - row * words] = 0;
}

using SegFn = void (*)(SegArgs);

#define ROWRED_SPLIT_ROW(K, OP) {K<OP, 1>, K<OP, 2>, K<OP, 4>}
const SegFn kStats[5][kNumSplitChunks] = {
    ROWRED_SPLIT_ROW(seg_stats_kernel, kOpLayerNorm), ROWRED_SPLIT_ROW(seg_stats_kernel, kOpRms),
    ROWRED_SPLIT_ROW(seg_stats_kernel, kOpSoftmax),   ROWRED_SPLIT_ROW(seg_stats_kernel, kOpRowSum),
    ROWRED_SPLIT_ROW(seg_stats_kernel, kOpRowMinMax),
};
const SegFn kApply[3][kNumSplitChunks] = {
    ROWRED_SPLIT_ROW(seg_apply_kernel, kOpLayerNorm),
    ROWRED_SPLIT_ROW(seg_apply_kernel, kOpRms),
    ROWRED_SPLIT_ROW(seg_apply_kernel, kOpSoftmax),
};
#undef ROWRED_SPLIT_ROW
#define ROWRED_EXCHANGE_ROW(OP) \
  {seg_exchange_kernel<OP, 1>, seg_exchange_kernel<OP, 2>, seg_exchange_kernel<OP, 4>, seg_exchange_kernel<OP, 8>}
const SegFn kExchange[3][kNumExchangeChunks] = {
    {seg_exchange_kernel<kOpLayerNorm, 1>, seg_exchange_kernel<kOpLayerNorm, 2>, seg_exchange_kernel<kOpLayerNorm, 4>,
     nullptr},
    ROWRED_EXCHANGE_ROW(kOpRms),
    ROWRED_EXCHANGE_ROW(kOpSoftmax),
};
#undef ROWRED_EXCHANGE_ROW
// [op][stripe: 0 = 4 + 4 slots, 1 = 8 + 4, 2 = 8 + 8] (registers + LDS);
// LayerNorm at 4 + 4 only (its x and r both take the slots).
const SegFn kXlds[3][kNumXldsStripes] = {
    {seg_xlds_kernel<kOpLayerNorm, 4, 4>, seg_xlds_kernel<kOpLayerNorm, 8, 4>, seg_xlds_kernel<kOpLayerNorm, 8, 8>},
    {seg_xlds_kernel<kOpRms, 4, 4>, seg_xlds_kernel<kOpRms, 8, 4>, seg_xlds_kernel<kOpRms, 8, 8>},
    {seg_xlds_kernel<kOpSoftmax, 4, 4>, seg_xlds_kernel<kOpSoftmax, 8, 4>, seg_xlds_kernel<kOpSoftmax, 8, 8>},
};
const SegFn kMerge[5] = {seg_merge_kernel<kOpLayerNorm>, seg_merge_kernel<kOpRms>, seg_merge_kernel<kOpSoftmax>,
                         seg_merge_kernel<kOpRowSum>, seg_merge_kernel<kOpRowMinMax>};
static_assert(kNumSplitChunks == 3 && kSplitChunkSet[0] == 1 && kSplitChunkSet[1] == 2 && kSplitChunkSet[2] == 4,
              "split kernel tables follow kSplitChunkSet");

constexpr int kMergeThreads = 256;  // four rows (wavefronts) per workgroup
constexpr int kClearThreads = 256;

}  // namespace

int64_t exchange_words(int op, int64_t rows, int64_t segments) {
  return 1 + (op == kOpLayerNorm ? 2 : 1) * rows * segments;
}

namespace {

// The exchange kernel of a plan, or nullptr.
SegFn exchange_kernel(int op, int chunks, int threads, int policy) {
  if (op < 0 || op > 2) return nullptr;
  if (policy & kPolicyLdsStripe) {
    const int si = xlds_stripe_index(op, chunks);
    return si < 0 || threads != kXldsThreads ? nullptr : kXlds[op][si];
  }
  const int ci = chunks == 1 ? 0 : chunks == 2 ? 1 : chunks == 4 ? 2 : chunks == 8 ? 3 : -1;
  if (ci < 0 || !exchange_kernel_exists(op, chunks) || threads > exchange_max_threads(chunks)) return nullptr;
  return kExchange[op][ci];
}

}  // namespace

// The workspace of rowred_static_ws, for callers that cannot allocate: one
// copy per GPU, held until the process ends.  Host code must not pass the
// array's name to a kernel (on the host it is only a stand-in for the symbol):
// static_workspace() looks up each device's address once and hands that out.
static __device__ __align__(256) uint8_t scratch[ROWRED_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;

int static_workspace(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p || ((uintptr_t)p & 255)) return (int)hipErrorInvalidValue;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return 0;
}

int64_t exchange_resident_groups(int op, int chunks, int threads, int policy) {
  const SegFn fn = exchange_kernel(op, chunks, threads, policy);
  if (!fn) return 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  static std::mutex mu;
  static std::map<std::pair<int, const void *>, int64_t> cache;
  const std::pair<int, const void *> key{dev, reinterpret_cast<const void *>(fn)};
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(fn), threads, 0) !=
      hipSuccess)
    return 0;
  const int64_t groups = (int64_t)cus * per_cu;
  std::lock_guard<std::mutex> lock(mu);
  cache[key] = groups;
  return groups;
}

int launch_exchange(int op, int chunks, int64_t grid, int threads, const SegArgs &args, bool clear_status,
                    hipStream_t stream) {
  const SegFn fn = exchange_kernel(op, chunks, threads, args.policy);
  if (!fn || args.segments > threads || args.segments > kMaxExchangeSegments) return (int)hipErrorInvalidValue;
  int err = 0;
  if (args.ws_in_y) {  // each row's words in y: its slots and its done count
    float *y = args.y;
    int64_t rows = args.rows;
    int32_t width = args.width;
    int32_t words = (op == kOpLayerNorm ? 2 : 1) * args.segments + 1;
    void *clear_params[] = {&y, &rows, &width, &words};
    err = (int)hipLaunchKernel(reinterpret_cast<const void *>(exchange_clear_row_words_kernel),
                               dim3((uint32_t)((rows * words + kClearThreads - 1) / kClearThreads)),
                               dim3(kClearThreads), clear_params, 0, stream);
  } else {
    uint64_t *w = reinterpret_cast<uint64_t *>(args.ws);
    int64_t n128 = (exchange_words(op, args.rows, args.segments) + 1) / 2;
    int64_t first = clear_status ? 0 : 1;  // 64-bit word to start clearing at
    void *clear_params[] = {&w, &first, &n128};
    err = (int)hipLaunchKernel(reinterpret_cast<const void *>(exchange_clear_kernel),
                               dim3((uint32_t)((n128 + kClearThreads - 1) / kClearThreads)), dim3(kClearThreads),
                               clear_params, 0, stream);
  }
  if (err) return err;
  SegArgs a = args;
  void *params[] = {&a};
  return (int)hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3((uint32_t)grid), dim3(threads), params, 0,
                              stream);
}

int launch_split(int op, int chunks, int64_t grid, int threads, const SegArgs &args, hipStream_t stream) {
  const int ci = chunks == 1 ? 0 : chunks == 2 ? 1 : chunks == 4 ? 2 : -1;
  if (op < 0 || op > 4 || ci < 0) return (int)hipErrorInvalidValue;
  SegArgs a = args;
  void *params[] = {&a};
  int err = (int)hipLaunchKernel(reinterpret_cast<const void *>(kStats[op][ci]), dim3((uint32_t)grid),
                                 dim3(threads), params, 0, stream);
  if (err) return err;
  const int64_t merge_grid = (a.rows + kMergeThreads / 64 - 1) / (kMergeThreads / 64);
  err = (int)hipLaunchKernel(reinterpret_cast<const void *>(kMerge[op]), dim3((uint32_t)merge_grid),
                             dim3(kMergeThreads), params, 0, stream);
  if (err || op > 2) return err;
  return (int)hipLaunchKernel(reinterpret_cast<const void *>(kApply[op][ci]), dim3((uint32_t)grid), dim3(threads),
                              params, 0, stream);
}

}  // namespace rowred
