// rowred_flat.hip -- short rows that do not start on 16-byte boundaries,
// read as one stream of granules (ROWRED_POLICY_FLAT): RMSNorm and softmax.
//
// A workgroup owns P consecutive rows, which are one contiguous run of x.
// Its lanes take the run's 16-byte granules in order: lane t of wave w holds,
// for slot c < C, granule w*64*C + c*64 + t of the run, so each load
// instruction of a wave reads 1 KB of consecutive memory and no slot is idle
// past a row's end.  (The row kernels give each row its own L lanes; a
// 127-column row spans 32 or 33 granules, so 16 lanes x 3 slots leave a
// third of the slots idle and the rows' shared boundary granules are written
// by two lanes.)
//
// Rows have at least 4 elements, so a granule holds elements of at most two
// rows.  Per granule a lane keeps two partial statistics: A for the row of
// its first element and B for the next row.  The rows are then reduced in
// LDS in a fixed order: every lane writes its partials; after a barrier a
// group of lanes per row folds that row's granules (its first granule's B
// part when the row starts inside it, then A parts) and a DPP butterfly
// finishes the group; after a second barrier every lane reads the statistics
// of its granules' rows.  Two barriers per call: softmax folds (max, sum of
// exp) pairs in one pass.  The elements stay in registers through every phase
// (read once, the pages' input reuse), and each lane stores whole 16-byte
// granules; only the run's first and last granules, which it shares with the
// neighbouring workgroups, are stored element by element.  Results are
// bitwise reproducible for a fixed plan.
//
// Phases: RMSNorm sums squares; softmax takes the row max and the sum of
// exp(x - max) (the max and exp-sum phases of "Immutable input reuse in
// Metal reductions", section "What the transformation actually preserves",
// folded as (max, sum) pairs), then normalises.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "rowred_device.h"
#include "rowred_internal.h"

namespace rowred {
namespace {

// Row (counted from the group's first row) of element e >= 0 of the run, for
// e < 2^24: a float quotient, corrected by one either way.
__device__ __forceinline__ int row_of(int e, int width, float inv_width) {
  int q = (int)((float)e * inv_width);
  if (q * width > e) --q;
  else if ((q + 1) * width <= e) ++q;
  return q;
}

template <int OP, int C>
__global__ void __launch_bounds__(kFlatMaxThreads) flat_kernel(RowArgs a) {
  static_assert(OP == kOpRms || OP == kOpSoftmax, "flat kernels: RMSNorm and softmax");
  extern __shared__ float lds[];
  const int T = blockDim.x;
  const int G = T * C;  // granule slots of the workgroup
  const int P = a.group_rows;
  float *partA = lds, *partB = lds + G;  // RMSNorm; softmax keeps four parts per granule
  float *tot0 = lds + 4 * G;  // P + 1 row statistics: RMSNorm sum of squares, softmax max
  float *tot1 = tot0 + P + 1;  // softmax: P + 1 reciprocal row sums
  const int width = a.width;
  const int64_t r0 = row_block(blockIdx.x, gridDim.x, (a.policy & kPolicyXcdRemap) != 0) * P;
  const int nr = (int)(a.rows - r0 < P ? a.rows - r0 : P);  // rows of this group, >= 1
  const int n_el = nr * width;                               // elements of the run
  const int64_t e_begin = r0 * (int64_t)width;
  const int phase = (int)(((uintptr_t)a.x >> 2) & 3);
  const int64_t g_first = (e_begin + phase) >> 2;  // the run's first granule, from x's 16-byte base
  const int d0 = (int)((e_begin + phase) & 3);     // position of the run's first element in it
  const int ng = (d0 + n_el + 3) >> 2;             // granules of the run, <= G
  const f32x4 *xg = reinterpret_cast<const f32x4 *>(a.x - phase) + g_first;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  auto slot_k = [&](int c) -> int { return wave * 64 * C + c * 64 + lane; };

  // ---- load: every granule of the run once; slots past its end load the
  // last granule again (a cache hit; masked below).
  f32x4 xv[C];
  auto load_all = [&](auto nt) {
    constexpr bool NT = decltype(nt)::value;
    if constexpr (NT) asm volatile("" ::: "memory");
#pragma unroll
    for (int c = 0; c < C; ++c) xv[c] = load_g<NT>(xg + min(slot_k(c), ng - 1));
    if constexpr (NT) asm volatile("" ::: "memory");
  };
  if (a.policy & kPolicyNtLoads) load_all(std::true_type{});
  else load_all(std::false_type{});

  // Per slot: element index of its first element in the run (e0, may be
  // negative in the first granule), row qa of its first element inside the
  // run, and the split s: elements j < s belong to row qa, j >= s to qa + 1.
  int e0[C], qa[C], split[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    e0[c] = 4 * slot_k(c) - d0;
    qa[c] = row_of(e0[c] > 0 ? e0[c] : 0, width, a.inv_width);
    split[c] = (qa[c] + 1) * width - e0[c];
  }
  auto in_run = [&](int c, int j) -> bool { return (unsigned)(e0[c] + j) < (unsigned)n_el; };

  // One reduction: per-granule partials (A, B) -> LDS -> per-row fold ->
  // tot[row].  part(c, j) gives element j of slot c's term (identity outside
  // the run).  R is SumOp or MaxOp.
  const int lpr_log2 = a.lanes_log2;  // lanes folding one row
  auto reduce_rows = [&](auto rop, auto part, float ident, float *tot) {
    using Rop = decltype(rop);
#pragma unroll
    for (int c = 0; c < C; ++c) {
      float pa = ident, pb = ident;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float t = part(c, j);
        if (j < split[c]) pa = Rop::apply(pa, t);
        else pb = Rop::apply(pb, t);
      }
      partA[slot_k(c)] = pa;
      partB[slot_k(c)] = pb;
    }
    __syncthreads();
    const int q = threadIdx.x >> lpr_log2, i = threadIdx.x & ((1 << lpr_log2) - 1);
    float acc = ident;
    if (q < nr) {
      const int first = q * width + d0;  // the row's first element, counted from the run's first granule
      const int g0 = first >> 2, g1 = (first + width - 1) >> 2;
      const bool starts_inside = q > 0 && (first & 3) != 0;  // the row is the B part of its first granule
      for (int g = g0 + i; g <= g1; g += 1 << lpr_log2)
        acc = Rop::apply(acc, (g == g0 && starts_inside) ? partB[g] : partA[g]);
    }
    acc = group_allreduce<Rop>(acc, lpr_log2);
    if (i == 0 && q < nr) tot[q] = acc;
    __syncthreads();
  };

  // Statistics of slot c's two rows (row indices clamped: slots past the run
  // read an entry whose value is never stored).
  auto stat = [&](const float *tot, int c, int j) -> float {
    const int row = qa[c] + (j < split[c] ? 0 : 1);
    return tot[row < P ? row : P];
  };

  float o[4 * C];
  if constexpr (OP == kOpRms) {
    reduce_rows(SumOp{}, [&](int c, int j) { return in_run(c, j) ? xv[c][j] * xv[c][j] : 0.0f; }, 0.0f, tot0);
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const float sa = __builtin_amdgcn_rsqf(fmaf(tot0[qa[c] < P ? qa[c] : P], a.inv_width, a.eps));
      const float sb = __builtin_amdgcn_rsqf(fmaf(tot0[qa[c] + 1 < P ? qa[c] + 1 : P], a.inv_width, a.eps));
#pragma unroll
      for (int j = 0; j < 4; ++j) o[4 * c + j] = xv[c][j] * (j < split[c] ? sa : sb);
    }
  } else {
    // One pass of statistics: per granule part its max m and the sum s of
    // exp(x - m) over its elements; per row the parts fold into the row's
    // (max, sum) by m = max m_k, s = sum s_k exp(m_k - m) -- the max and
    // exp-sum phases merged as in the split kernels, which halves the
    // barriers.  -inf elements weigh 0 (also in a part whose max is -inf);
    // NaN and +inf poison the row's sum, as in one pass.
    float *pm = lds, *ps = lds + 2 * G;  // [A parts | B parts] of the max, then of the sum
    // The exponentials stay in o[] (against their part's max); the output
    // scales each part by exp(part max - row max) / row sum.
    float ma[C], mb[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      ma[c] = -__builtin_inff();
      mb[c] = -__builtin_inff();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float t = in_run(c, j) ? xv[c][j] : -__builtin_inff();
        if (j < split[c]) ma[c] = fmaxf(ma[c], t);
        else mb[c] = fmaxf(mb[c], t);
      }
      float sa = 0.0f, sb = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = xv[c][j];
        const bool a_part = j < split[c];
        const float e = (!in_run(c, j) || x == -__builtin_inff())
                            ? 0.0f
                            : __builtin_amdgcn_exp2f((x - (a_part ? ma[c] : mb[c])) * kLog2e);
        o[4 * c + j] = e;
        if (a_part) sa += e;
        else sb += e;
      }
      const int k = slot_k(c);
      pm[k] = ma[c];
      pm[G + k] = mb[c];
      ps[k] = sa;
      ps[G + k] = sb;
    }
    __syncthreads();
    // Per row: the max over its granule parts (a butterfly finishes the
    // group), then each part's sum restated under it (s * exp(m - M), s
    // itself when m == M, so two -inf maxima give 0 rather than NaN) and
    // added, a second butterfly; the exponentials are independent.
    const int q = threadIdx.x >> lpr_log2, i = threadIdx.x & ((1 << lpr_log2) - 1);
    int g0 = 0, g1 = -1;
    bool starts_inside = false;
    if (q < nr) {
      const int first = q * width + d0;
      g0 = first >> 2;
      g1 = (first + width - 1) >> 2;
      starts_inside = q > 0 && (first & 3) != 0;
    }
    float m = -__builtin_inff();
    for (int g = g0 + i; g <= g1; g += 1 << lpr_log2) m = fmaxf(m, pm[(g == g0 && starts_inside) ? G + g : g]);
    m = group_allreduce<MaxOp>(m, lpr_log2);
    float sum = 0.0f;
    for (int g = g0 + i; g <= g1; g += 1 << lpr_log2) {
      const int at = (g == g0 && starts_inside) ? G + g : g;
      sum += rescale_sum(ps[at], pm[at], m);
    }
    sum = group_allreduce<SumOp>(sum, lpr_log2);
    if (i == 0 && q < nr) {
      tot0[q] = m;
      tot1[q] = __builtin_amdgcn_rcpf(sum);
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int ra = qa[c] < P ? qa[c] : P, rb = qa[c] + 1 < P ? qa[c] + 1 : P;
      const float fa = __builtin_amdgcn_exp2f((ma[c] - tot0[ra]) * kLog2e) * tot1[ra];
      const float fb = __builtin_amdgcn_exp2f((mb[c] - tot0[rb]) * kLog2e) * tot1[rb];
#pragma unroll
      for (int j = 0; j < 4; ++j) o[4 * c + j] *= j < split[c] ? fa : fb;
    }
  }

  // ---- store: whole granules, except where the run shares a granule with
  // a neighbouring group (or y sits at another 16-byte phase than x).
  float *yrun = a.y + e_begin;  // element e of the run is yrun[e]
  auto store_all = [&](auto nt) {
    constexpr bool NT = decltype(nt)::value;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int k = slot_k(c);
      if (k >= ng) continue;
      if (a.y_vec && e0[c] >= 0 && e0[c] + 4 <= n_el) {
        store_g<NT>(reinterpret_cast<f32x4 *>(yrun + e0[c]), f32x4{o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]});
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (in_run(c, j)) store_g<NT>(yrun + e0[c] + j, o[4 * c + j]);
      }
    }
  };
  if (a.policy & kPolicyNtStores) store_all(std::true_type{});
  else store_all(std::false_type{});
}

using FlatFn = void (*)(RowArgs);
// [RMSNorm, softmax][chunk index: 1, 2, 4]
const FlatFn kFlat[2][3] = {
    {flat_kernel<kOpRms, 1>, flat_kernel<kOpRms, 2>, flat_kernel<kOpRms, 4>},
    {flat_kernel<kOpSoftmax, 1>, flat_kernel<kOpSoftmax, 2>, flat_kernel<kOpSoftmax, 4>},
};

}  // namespace

int launch_flat(int op, int chunks, int64_t grid, int threads, const RowArgs &args, hipStream_t stream) {
  const int ci = chunks == 1 ? 0 : chunks == 2 ? 1 : chunks == 4 ? 2 : -1;
  if ((op != kOpRms && op != kOpSoftmax) || ci < 0 || threads > kFlatMaxThreads) return (int)hipErrorInvalidValue;
  RowArgs a = args;
  void *params[] = {&a};
  const size_t lds = flat_lds_bytes(chunks, threads, a.group_rows);
  return (int)hipLaunchKernel(reinterpret_cast<const void *>(kFlat[op == kOpSoftmax][ci]), dim3((uint32_t)grid),
                              dim3(threads), params, lds, stream);
}

}  // namespace rowred
