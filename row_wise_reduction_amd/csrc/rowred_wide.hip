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

  float scale;  // RMSNorm: 1/rms; softmax: 1/sum (ROWRED_POLICY_ONLINE: exp(m - M)/sum)
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
    float m = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
    // ROWRED_POLICY_ONLINE: exponentials against this lane's own max (0
    // for a lane with nothing but -inf), one (max, sum) collective, and the
    // lane's factor exp(m - M) / S folded into scale; as in the register
    // kernels, in the same order.
    const bool online = (a.policy & kPolicyOnline) != 0;
    const float m_lane = m;
    if (online) m = m == -__builtin_inff() ? 0.0f : m;
    else m = row_allreduce<MaxOp>(m, lanes_log2, partials[0]);
#pragma unroll
    for (int i = 0; i < 4 * CR; ++i) s[i] = __builtin_amdgcn_exp2f((s[i] - m) * kLog2e);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4 * CR; ++i) acc[i & 3] += s[i];
    // The LDS slots' exponentials replace their x in LDS (each lane its
    // own entries), so the output pass only scales them.
#pragma unroll
    for (int c = 0; c < CL; ++c) {
      const f32x4 v = lds_slot(c);
      f32x4 e;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        e[j] = __builtin_amdgcn_exp2f((lds_value(v, c, j) - m) * kLog2e);
        acc[j] += e[j];
      }
      held[c * L + li] = e;
    }
    float sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    if (online) {
      float M = m_lane;
      row_allreduce_online(M, sum, lanes_log2, partials[0], partials[1]);
      scale = __builtin_amdgcn_exp2f((m_lane - M) * kLog2e) * __builtin_amdgcn_rcpf(sum);
    } else {
      sum = row_allreduce<SumOp>(sum, lanes_log2, partials[1]);
      scale = __builtin_amdgcn_rcpf(sum);
    }
  }
#pragma unroll
  for (int i = 0; i < 4 * CR; ++i) s[i] *= scale;

  // ---- store: register slots, then the LDS slots mapped on the way out.
  auto out_value = [&](const f32x4 &v, int c, int j) -> float {
    if constexpr (OP == kOpRms) return lds_value(v, c, j) * scale;
    else return v[j] * scale;  // softmax: the slot holds exp(x - m) by now
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

// ---------------------------------------------------------------------------
// Rows wider than the LDS stripe (ROWRED_POLICY_LDS_STRIPE | ROWRED_POLICY_LOOPED):
// the row's first 16384 granules are held as above (8 register + 8 LDS
// slots per lane) and read once; the rest is walked in tiles of 4096
// granules twice (statistics with cached loads, then map and store), as
// the looped kernels walk a whole row.  Softmax keeps an online (max, sum)
// per lane over the held part and then the tiles; RMSNorm sums squares.
// ---------------------------------------------------------------------------
constexpr int kTailChunks = 4;

template <int OP>
__global__ void __launch_bounds__(kWideLanes) wide_tail_kernel(RowArgs a) {
  constexpr int CR = 8, CL = 8, C = CR + CL, L = kWideLanes, TC = kTailChunks;
  constexpr int kHead = C * L;  // granules held
  constexpr int kTile = TC * L;
  __shared__ f32x4 held[CL * L];
  __shared__ float partials[2][16];
  __shared__ double partials_d[16];
  constexpr int lanes_log2 = 10;
  const int li = threadIdx.x;
  const int width = a.width;
  const int64_t row = row_block(blockIdx.x, gridDim.x, (a.policy & kPolicyXcdRemap) != 0);
  const int64_t base = row * (int64_t)width;
  const float *xrow = a.x + base;
  const int off = (int)(((uintptr_t)xrow >> 2) & 3);
  const int nwin = (width + off + 3) >> 2;
  const int kmax = nwin - 1;
  // >= 0: nwin >= kHead (see the head below); 0 when the row ends in the head
  const int ntiles = (nwin - kHead + kTile - 1) / kTile;
  auto valid_k = [&](int k, int j) -> bool { return (unsigned)(4 * k + j - off) < (unsigned)width; };
  const f32x4 *xw = reinterpret_cast<const f32x4 *>(xrow - off);
  f32x4 *wave_held = held + (li & ~63);
  typedef __attribute__((address_space(3))) void lds_void;
  constexpr float kIdent = OP == kOpSoftmax ? -__builtin_inff() : 0.0f;

  // ---- the head: LDS slots, then register slots, then a full wait.
  f32x4 xv[CR];
  auto load_head = [&](auto nt) {
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
  if (a.policy & kPolicyNtLoads) load_head(std::true_type{});
  else load_head(std::false_type{});
  __builtin_amdgcn_s_waitcnt(0);
  // Head granule of slot c: c * L + li.  The plan needs some row's window to
  // exceed the head, and windows at the four 16-byte phases differ by at
  // most one granule, so every head granule lies inside this row's window.
  // Only the first granule (a register slot) can start before the row, and
  // only the last (an LDS slot) can run past its end -- when this row's
  // window is exactly the head.  Both are masked to the identity.
#pragma unroll
  for (int c = 0; c < CR; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) xv[c][j] = valid_k(c * L + li, j) ? xv[c][j] : kIdent;
  {
    f32x4 &last = held[(CL - 1) * L + li];  // this lane's own entry of the last LDS slot
    f32x4 v = last;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = valid_k((C - 1) * L + li, j) ? v[j] : kIdent;
    last = v;
  }
  auto head_at = [&](int c) -> f32x4 { return c < CR ? xv[c < CR ? c : 0] : held[(c - CR) * L + li]; };

  // ---- the tail: tiles of TC slots, two deep.
  auto tile_k = [&](int t, int c) -> int { return kHead + t * kTile + c * L + li; };
  auto load_tile = [&](auto nt, int t, f32x4(&tv)[TC]) {
    constexpr bool NT = decltype(nt)::value;
    if constexpr (NT) asm volatile("" ::: "memory");
#pragma unroll
    for (int c = 0; c < TC; ++c) tv[c] = load_g<NT>(xw + min(tile_k(t, c), kmax));
    if constexpr (NT) asm volatile("" ::: "memory");
  };
  f32x4 ta[TC], tb[TC];
  // rev: the tiles last to first (the second walk then starts on what the
  // first walk read last, the likeliest to be still in cache)
  auto walk = [&](auto nt, auto f, bool rev) {
    if (ntiles == 0) return;  // the row ends inside the head
    auto at = [&](int t) { return rev ? ntiles - 1 - t : t; };
    load_tile(nt, at(0), ta);
    for (int t = 0; t < ntiles; t += 2) {
      if (t + 1 < ntiles) load_tile(nt, at(t + 1), tb);
      f(at(t), ta);
      if (t + 2 < ntiles) load_tile(nt, at(t + 2), ta);
      if (t + 1 < ntiles) f(at(t + 1), tb);
    }
  };

  // ---- pass 1: statistics over the head, then the tail tiles.  The head's
  // and each tile's terms are summed in FP32, the lane's running total in
  // FP64: a lane of a 2^31-column row adds up 2^21 terms.
  float scale, m_row = 0.0f;
  if constexpr (OP == kOpRms) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const f32x4 v = head_at(c);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = fmaf(v[j], v[j], acc[j]);
    }
    double total = (double)((acc[0] + acc[1]) + (acc[2] + acc[3]));
    walk(std::false_type{}, [&](int t, const f32x4(&tv)[TC]) {
      float tacc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < TC; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x = valid_k(tile_k(t, c), j) ? tv[c][j] : 0.0f;
          tacc[j] = fmaf(x, x, tacc[j]);
        }
      total += (double)((tacc[0] + tacc[1]) + (tacc[2] + tacc[3]));
    }, false);
    const double ss = row_allreduce<SumOp>(total, lanes_log2, partials_d);
    scale = __builtin_amdgcn_rsqf(fmaf((float)ss, a.inv_width, a.eps));
  } else {  // softmax: online (max m, sum s of exp(x - m)) per lane
    float m = -__builtin_inff();
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const f32x4 v = head_at(c);
#pragma unroll
      for (int j = 0; j < 4; ++j) m = fmaxf(m, v[j]);
    }
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const f32x4 v = head_at(c);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += v[j] == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f((v[j] - m) * kLog2e);
    }
    double s = (double)((acc[0] + acc[1]) + (acc[2] + acc[3]));
    walk(std::false_type{}, [&](int t, const f32x4(&tv)[TC]) {
      float mt = -__builtin_inff();
#pragma unroll
      for (int c = 0; c < TC; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) mt = fmaxf(mt, valid_k(tile_k(t, c), j) ? tv[c][j] : -__builtin_inff());
      const float m_new = fmaxf(m, mt);
      // rescale the running sum to the new max (no rescale while the max
      // stays, which also covers a lane that has seen only -inf)
      if (m_new != m) s *= (double)__builtin_amdgcn_exp2f((m - m_new) * kLog2e);
      m = m_new;
      float tacc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < TC; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x = tv[c][j];
          const bool zero = !valid_k(tile_k(t, c), j) || x == -__builtin_inff();
          tacc[j] += zero ? 0.0f : __builtin_amdgcn_exp2f((x - m) * kLog2e);
        }
      s += (double)((tacc[0] + tacc[1]) + (tacc[2] + tacc[3]));
    }, false);
    const float M = row_allreduce<MaxOp>(m, lanes_log2, partials[0]);
    // an all -inf row: M = -inf, every s = 0, sum 0 and 1/sum = inf, and the
    // map's exp(-inf - -inf) makes the row NaN, as in one pass
    const double term = (m == M) ? s : s * (double)__builtin_amdgcn_exp2f((m - M) * kLog2e);
    const double S = row_allreduce<SumOp>(term, lanes_log2, partials_d);
    m_row = M;
    scale = __builtin_amdgcn_rcpf((float)S);
  }

  // ---- pass 2: map and store, the head from registers and LDS, the tail
  // read again.
  auto map = [&](float x) -> float {
    if constexpr (OP == kOpRms) return x * scale;
    else return __builtin_amdgcn_exp2f((x - m_row) * kLog2e) * scale;
  };
  float *yrow = a.y + base;
  auto store_granule = [&](auto nt, int k, const float (&o)[4]) {
    constexpr bool NT = decltype(nt)::value;
    const int e0 = 4 * k - off;
    if (a.y_vec && e0 >= 0 && e0 + 4 <= width) {
      store_g<NT>(reinterpret_cast<f32x4 *>(yrow - off) + k, f32x4{o[0], o[1], o[2], o[3]});
    } else if (k <= kmax) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if ((unsigned)(e0 + j) < (unsigned)width) store_g<NT>(yrow + e0 + j, o[j]);
    }
  };
  // ROWRED_POLICY_REVERSE: the tail last tile first, then the head.
  const bool rev = (a.policy & kPolicyReverse) != 0;
  auto pass2 = [&](auto ntl, auto nts) {
    auto head = [&] {
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const f32x4 v = head_at(c);
        const float o[4] = {map(v[0]), map(v[1]), map(v[2]), map(v[3])};
        store_granule(nts, c * L + li, o);
      }
    };
    if (!rev) head();
    walk(ntl, [&](int t, const f32x4(&tv)[TC]) {
#pragma unroll
      for (int c = 0; c < TC; ++c) {
        const float o[4] = {map(tv[c][0]), map(tv[c][1]), map(tv[c][2]), map(tv[c][3])};
        store_granule(nts, tile_k(t, c), o);
      }
    }, rev);
    if (rev) head();
  };
  const bool ntl = (a.policy & kPolicyNtLoads) != 0, nts = (a.policy & kPolicyNtStores) != 0;
  if (ntl && nts) pass2(std::true_type{}, std::true_type{});
  else if (ntl) pass2(std::true_type{}, std::false_type{});
  else if (nts) pass2(std::false_type{}, std::true_type{});
  else pass2(std::false_type{}, std::false_type{});
}

// ---------------------------------------------------------------------------
// LayerNorm (residual, plain, affine) rows wider than 8192 granules
// (ROWRED_POLICY_LDS_STRIPE | ROWRED_POLICY_LOOPED with chunks 8): x and r of
// the row's first 8192 granules are held -- 4 slots of each per lane in
// registers, 4 of each in LDS (128 KB) -- and read once; the rest is walked
// in tiles of 2048 granules twice, as the looped LayerNorm kernel walks a
// whole row.  Per lane, the head's (count, sum, sum of squares about its
// mean) and then each tile's are folded into (n, mean, M2) by the pairwise
// update of Chan, Golub and LeVeque; across lanes as in the looped kernel.
// ---------------------------------------------------------------------------
constexpr int kLnHeadReg = 4, kLnHeadLds = 4, kLnTailChunks = 2;
static_assert(kLnHeadReg + kLnHeadLds == kLnTailHeadChunks, "LayerNorm head");

// AFFINE: 0 none, 1 gamma/beta read 4 bytes at a time, 2 gamma/beta read
// 16 bytes at a time (rows start on 16-byte boundaries and so do gamma and
// beta: row granule k is gamma/beta granule k).
template <int AFFINE>
__global__ void __launch_bounds__(kWideLanes) ln_tail_kernel(RowArgs a) {
  constexpr int CR = kLnHeadReg, CL = kLnHeadLds, C = CR + CL, L = kWideLanes, TC = kLnTailChunks;
  constexpr int kHead = C * L;
  constexpr int kTile = TC * L;
  __shared__ f32x4 held_x[CL * L];
  __shared__ f32x4 held_r[CL * L];
  __shared__ double partials_d[2][16];
  constexpr int lanes_log2 = 10;
  const int li = threadIdx.x;
  const int width = a.width;
  const int64_t row = row_block(blockIdx.x, gridDim.x, (a.policy & kPolicyXcdRemap) != 0);
  const int64_t base = row * (int64_t)width;
  const float *xrow = a.x + base;
  const bool has_r = a.r != nullptr;
  const float *rrow = has_r ? a.r + base : nullptr;
  const int off = (int)(((uintptr_t)xrow >> 2) & 3);
  const int nwin = (width + off + 3) >> 2;
  const int kmax = nwin - 1;
  // >= 0: nwin >= kHead (see the head below); 0 when the row ends in the head
  const int ntiles = (nwin - kHead + kTile - 1) / kTile;
  auto valid_k = [&](int k, int j) -> bool { return (unsigned)(4 * k + j - off) < (unsigned)width; };
  const f32x4 *xw = reinterpret_cast<const f32x4 *>(xrow - off);
  const f32x4 *rw = has_r ? reinterpret_cast<const f32x4 *>(rrow - off) : nullptr;
  typedef __attribute__((address_space(3))) void lds_void;
  f32x4 *wave_x = held_x + (li & ~63);
  f32x4 *wave_r = held_r + (li & ~63);

  // r of granule k: 16 bytes when r shares x's phase, else 4 bytes at a time
  // at the same element positions (each index clamped into the row).
  auto load_r = [&](auto nt, int k) -> f32x4 {
    constexpr bool NT = decltype(nt)::value;
    if (!has_r) return f32x4(0.0f);
    if (a.r_vec) return load_g<NT>(rw + min(k, kmax));
    f32x4 v;
    const int emax = width - 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = load_g<NT>(rrow + max(0, min(4 * k + j - off, emax)));
    return v;
  };

  // ---- the head.
  f32x4 xv[CR], rv[CR];
  auto load_head = [&](auto nt) {
    constexpr bool NT = decltype(nt)::value;
    if constexpr (NT) asm volatile("" ::: "memory");
#pragma unroll
    for (int c = 0; c < CL; ++c)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(xw + (CR + c) * L + li),
                                       (lds_void *)(wave_x + c * L), 16, 0, NT ? 2 : 0);
    if (has_r && a.r_vec) {
#pragma unroll
      for (int c = 0; c < CL; ++c)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(rw + (CR + c) * L + li),
                                         (lds_void *)(wave_r + c * L), 16, 0, NT ? 2 : 0);
    }
#pragma unroll
    for (int c = 0; c < CR; ++c) xv[c] = load_g<NT>(xw + c * L + li);
#pragma unroll
    for (int c = 0; c < CR; ++c) rv[c] = load_r(nt, c * L + li);
    if constexpr (NT) asm volatile("" ::: "memory");
  };
  if (a.policy & kPolicyNtLoads) load_head(std::true_type{});
  else load_head(std::false_type{});
  __builtin_amdgcn_s_waitcnt(0);
  if (!(has_r && a.r_vec)) {
    // r at another phase than x (4-byte loads), or no residual: the lane
    // fills its own LDS slots of r
#pragma unroll
    for (int c = 0; c < CL; ++c) held_r[c * L + li] = load_r(std::false_type{}, (CR + c) * L + li);
  }
  // The plan needs some row's window to exceed the head, and windows at the
  // four 16-byte phases differ by at most one granule, so every head granule
  // lies inside this row's window.  Only the first (a register slot) can
  // start before the row, and only the last (an LDS slot) can run past its
  // end -- when this row's window is exactly the head.  Their elements
  // outside the row become 0 (x and r).
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool in = valid_k(li, j);
    xv[0][j] = in ? xv[0][j] : 0.0f;
    rv[0][j] = in ? rv[0][j] : 0.0f;
  }
  {
    f32x4 &lx = held_x[(CL - 1) * L + li], &lr = held_r[(CL - 1) * L + li];  // this lane's own entries
    f32x4 vx = lx, vr = lr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool in = valid_k((C - 1) * L + li, j);
      vx[j] = in ? vx[j] : 0.0f;
      vr[j] = in ? vr[j] : 0.0f;
    }
    lx = vx;
    lr = vr;
  }
  // Elements of the head inside the row: slots 1 .. C-2 are whole.
  int n_head = 4 * (C - 2);
#pragma unroll
  for (int j = 0; j < 4; ++j) n_head += (valid_k(li, j) ? 1 : 0) + (valid_k((C - 1) * L + li, j) ? 1 : 0);
  auto head_x = [&](int c) -> f32x4 { return c < CR ? xv[c < CR ? c : 0] : held_x[(c - CR) * L + li]; };
  auto head_r = [&](int c) -> f32x4 { return c < CR ? rv[c < CR ? c : 0] : held_r[(c - CR) * L + li]; };
  // x + r as the exact pair (h, l) (TwoSum).
  auto pair = [&](float x, float r, float &h, float &l) {
    h = x + r;
    const float bb = h - x;
    l = (x - (h - bb)) + (r - bb);
  };

  // ---- the tail: tiles of TC slots of x and r, two deep.
  auto tile_k = [&](int t, int c) -> int { return kHead + t * kTile + c * L + li; };
  auto load_tile = [&](auto nt, int t, f32x4(&tx)[TC], f32x4(&tr)[TC]) {
    constexpr bool NT = decltype(nt)::value;
    if constexpr (NT) asm volatile("" ::: "memory");
#pragma unroll
    for (int c = 0; c < TC; ++c) tx[c] = load_g<NT>(xw + min(tile_k(t, c), kmax));
#pragma unroll
    for (int c = 0; c < TC; ++c) tr[c] = load_r(nt, tile_k(t, c));
    if constexpr (NT) asm volatile("" ::: "memory");
  };
  f32x4 xa[TC], ra[TC], xb[TC], rb[TC];
  // rev: the tiles last to first (as in the RMSNorm/softmax kernel)
  auto walk = [&](auto nt, auto f, bool rev) {
    if (ntiles == 0) return;  // the row ends inside the head
    auto at = [&](int t) { return rev ? ntiles - 1 - t : t; };
    load_tile(nt, at(0), xa, ra);
    for (int t = 0; t < ntiles; t += 2) {
      if (t + 1 < ntiles) load_tile(nt, at(t + 1), xb, rb);
      f(at(t), xa, ra);
      if (t + 2 < ntiles) load_tile(nt, at(t + 2), xa, ra);
      if (t + 1 < ntiles) f(at(t + 1), xb, rb);
    }
  };

  // ---- pass 1: per-lane (n, mean, M2), the head first.
  double n_l, mean_l, m2_l;
  {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    float acc_lo = 0.0f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const f32x4 xx = head_x(c), r4 = head_r(c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float h, l;
        pair(xx[j], r4[j], h, l);
        acc[j] += (double)h;
        acc_lo += l;
      }
    }
    const int n_h = n_head;
    const double s_h = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + (double)acc_lo;
    const double mu = s_h / (double)n_h;
    const float th = (float)mu;
    const float tl = (float)(mu - (double)th);
    float sq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const f32x4 xx = head_x(c), r4 = head_r(c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float h, l;
        pair(xx[j], r4[j], h, l);
        const float d = ((c == 0 || c == C - 1) && !valid_k(c * L + li, j)) ? 0.0f : (h - th) + (l - tl);
        sq[j] = fmaf(d, d, sq[j]);
      }
    }
    n_l = (double)n_h;
    mean_l = mu;
    m2_l = (double)((sq[0] + sq[1]) + (sq[2] + sq[3]));
  }
  walk(std::false_type{}, [&](int t, const f32x4(&tx)[TC], const f32x4(&tr)[TC]) {
    float hi[4 * TC], lo[4 * TC];
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    float acc_lo = 0.0f;
    int n_t = 0;
#pragma unroll
    for (int c = 0; c < TC; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool in = valid_k(tile_k(t, c), j);
        pair(in ? tx[c][j] : 0.0f, in ? tr[c][j] : 0.0f, hi[4 * c + j], lo[4 * c + j]);
        acc[j] += (double)hi[4 * c + j];
        acc_lo += lo[4 * c + j];
        n_t += in ? 1 : 0;
      }
    if (n_t == 0) return;
    const double mu_t = (((acc[0] + acc[1]) + (acc[2] + acc[3])) + (double)acc_lo) / (double)n_t;
    const float th = (float)mu_t;
    const float tl = (float)(mu_t - (double)th);
    float sq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < TC; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * c + j;
        const float d = valid_k(tile_k(t, c), j) ? (hi[i] - th) + (lo[i] - tl) : 0.0f;
        sq[j] = fmaf(d, d, sq[j]);
      }
    const double m2_t = (double)((sq[0] + sq[1]) + (sq[2] + sq[3]));
    const double n = n_l + (double)n_t;
    const double delta = mu_t - mean_l;
    mean_l += delta * ((double)n_t / n);
    m2_l += m2_t + delta * delta * (n_l * (double)n_t / n);
    n_l = n;
  }, false);
  const double mean = row_allreduce<SumOp>(n_l * mean_l, lanes_log2, partials_d[0]) / (double)width;
  const double dm = mean_l - mean;
  const double m2 = row_allreduce<SumOp>(m2_l + n_l * dm * dm, lanes_log2, partials_d[1]);
  const float m_hi = (float)mean;
  const float m_lo = (float)(mean - (double)m_hi);
  const float rstd = __builtin_amdgcn_rsqf(fmaf((float)m2, a.inv_width, a.eps));

  // ---- pass 2: map and store.
  float *yrow = a.y + base;
  constexpr bool affine = AFFINE != 0;
  const int emax = width - 1;
  auto map_granule = [&](int k, const f32x4 &xx, const f32x4 &r4, float (&o)[4]) {
    f32x4 g4 = f32x4(1.0f), b4 = f32x4(0.0f);
    if constexpr (AFFINE == 2) {
      const int kk = min(k, kmax);
      if (a.gamma) g4 = load_g<false>(reinterpret_cast<const f32x4 *>(a.gamma) + kk);
      if (a.beta) b4 = load_g<false>(reinterpret_cast<const f32x4 *>(a.beta) + kk);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float h, l;
      pair(xx[j], r4[j], h, l);
      const float y = ((h - m_hi) + (l - m_lo)) * rstd;
      if constexpr (AFFINE == 1) {
        const int e = max(0, min(4 * k + j - off, emax));
        o[j] = fmaf(y, a.gamma ? a.gamma[e] : 1.0f, a.beta ? a.beta[e] : 0.0f);
      } else {
        o[j] = affine ? fmaf(y, g4[j], b4[j]) : y;
      }
    }
  };
  auto store_granule = [&](auto nt, int k, const float (&o)[4]) {
    constexpr bool NT = decltype(nt)::value;
    const int e0 = 4 * k - off;
    if (a.y_vec && e0 >= 0 && e0 + 4 <= width) {
      store_g<NT>(reinterpret_cast<f32x4 *>(yrow - off) + k, f32x4{o[0], o[1], o[2], o[3]});
    } else if (k <= kmax) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if ((unsigned)(e0 + j) < (unsigned)width) store_g<NT>(yrow + e0 + j, o[j]);
    }
  };
  // ROWRED_POLICY_REVERSE: the tail last tile first, then the head.
  const bool rev = (a.policy & kPolicyReverse) != 0;
  auto pass2 = [&](auto ntl, auto nts) {
    auto head = [&] {
#pragma unroll
      for (int c = 0; c < C; ++c) {
        float o[4];
        map_granule(c * L + li, head_x(c), head_r(c), o);
        store_granule(nts, c * L + li, o);
      }
    };
    if (!rev) head();
    walk(ntl, [&](int t, const f32x4(&tx)[TC], const f32x4(&tr)[TC]) {
#pragma unroll
      for (int c = 0; c < TC; ++c) {
        float o[4];
        map_granule(tile_k(t, c), tx[c], tr[c], o);
        store_granule(nts, tile_k(t, c), o);
      }
    }, rev);
    if (rev) head();
  };
  const bool ntl = (a.policy & kPolicyNtLoads) != 0, nts = (a.policy & kPolicyNtStores) != 0;
  if (ntl && nts) pass2(std::true_type{}, std::true_type{});
  else if (ntl) pass2(std::true_type{}, std::false_type{});
  else if (nts) pass2(std::false_type{}, std::true_type{});
  else pass2(std::false_type{}, std::false_type{});
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

int launch_wide_tail(int op, int64_t rows, const RowArgs &args, hipStream_t stream) {
  if (op != kOpRms && op != kOpSoftmax && op != kOpLayerNorm && op != kOpLayerNormAffine)
    return (int)hipErrorInvalidValue;
  RowArgs a = args;
  void *params[] = {&a};
  const void *fn = op == kOpRms       ? reinterpret_cast<const void *>(wide_tail_kernel<kOpRms>)
                   : op == kOpSoftmax ? reinterpret_cast<const void *>(wide_tail_kernel<kOpSoftmax>)
                   : op == kOpLayerNorm ? reinterpret_cast<const void *>(ln_tail_kernel<0>)
                   : a.affine_vec       ? reinterpret_cast<const void *>(ln_tail_kernel<2>)
                                        : reinterpret_cast<const void *>(ln_tail_kernel<1>);
  return (int)hipLaunchKernel(fn, dim3((uint32_t)rows), dim3(kWideLanes), params, 0, stream);
}

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
