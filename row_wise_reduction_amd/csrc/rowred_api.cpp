// rowred_api.cpp -- C ABI of the row-reduction library: argument checks, the
// launch-geometry chooser and the entry points.  Host code only; the kernels
// live in rowred_kernels.hip.
#include <math.h>
#include <stdint.h>

#include "rowred_internal.h"

#define ROWRED_API extern "C" __attribute__((visibility("default")))


namespace rowred {
namespace {

constexpr int kNumMatrixOps = 3;  // LayerNorm, RMSNorm, softmax: rows x width outputs

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int ilog2(int64_t v) {
  int l = 0;
  while ((int64_t(1) << l) < v) ++l;
  return l;
}

bool chunks_supported(int chunks) {
  for (int c : kChunkSet)
    if (c == chunks) return true;
  return false;
}

// Smallest instantiated chunk count >= want, or -1.
int round_up_chunks(int64_t want) {
  for (int c : kChunkSet)
    if (c >= want) return c;
  return -1;
}

// Shape of one call after argument checks.
struct Call {
  int op;
  const float *x, *r;
  const float *gamma = nullptr, *beta = nullptr;  // LayerNorm only
  float *y;
  float *y2 = nullptr;  // row max (min/max reduction)
  int64_t rows, width;
  bool r_vec, y_vec;  // r / y share x's address modulo 16
  int window;         // largest number of 16-byte granules a row of x spans
};

bool overlaps(const void *a, const void *b, int64_t bytes) {
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return pa < pb + (uintptr_t)bytes && pb < pa + (uintptr_t)bytes;
}

// Largest granule window over the rows: a row starting `o` floats past a
// 16-byte boundary spans ceil((width + o) / 4) granules.  Row i starts at
// (x + i*width) so its offset cycles with period <= 4 rows.
int max_window(const float *x, int64_t rows, int64_t width) {
  const int64_t off0 = (int64_t)(((uintptr_t)x >> 2) & 3);
  int64_t worst = 0;
  const int64_t probe = rows < 4 ? rows : 4;
  for (int64_t i = 0; i < probe; ++i) {
    const int64_t off = (off0 + i * width) & 3;
    const int64_t w = (width + off + 3) / 4;
    if (w > worst) worst = w;
  }
  return worst > INT32_MAX ? INT32_MAX : (int)worst;
}

// Checks shared by every entry point.  `need_eps` marks ops with an eps.
int check_call(int op, const float *x, const float *r, const float *y, int64_t rows, int64_t width, bool need_r,
               bool need_eps, float eps, Call *out, bool cap = false) {
  if (op < 0 || op >= kNumMatrixOps) return ROWRED_ERR_INVALID_ARG;
  if (rows < 0 || width < 0) return ROWRED_ERR_INVALID_ARG;
  if (need_eps && (!isfinite(eps) || eps < 0.0f)) return ROWRED_ERR_INVALID_ARG;
  out->op = op;
  out->x = x;
  out->r = r;
  out->y = const_cast<float *>(y);
  out->rows = rows;
  out->width = width;
  out->r_vec = out->y_vec = false;
  out->window = 0;
  if (rows == 0 || width == 0) return ROWRED_OK;
  if (width > ROWRED_MAX_WIDTH || rows > INT64_MAX / width || rows * width > INT64_MAX / 4) return ROWRED_ERR_UNSUPPORTED;
  if (!x || !y || (need_r && !r)) return ROWRED_ERR_INVALID_ARG;
  if (((uintptr_t)x & 3) || ((uintptr_t)y & 3) || (r && ((uintptr_t)r & 3))) return ROWRED_ERR_INVALID_ARG;
  const int64_t bytes = rows * width * 4;
  if (overlaps(x, y, bytes) || (r && overlaps(r, y, bytes))) return ROWRED_ERR_ALIAS;
  const uintptr_t ax = (uintptr_t)x & 15;
  out->y_vec = ((uintptr_t)y & 15) == ax;
  out->r_vec = r && ((uintptr_t)r & 15) == ax;
  out->window = max_window(x, rows, width);
  if (cap && out->window > kMaxWindow) return ROWRED_ERR_UNSUPPORTED;
  return ROWRED_OK;
}

// The kernel operator a call runs: affine LayerNorm has its own kernels.
int kernel_op(const Call &c) { return (c.gamma || c.beta) ? kKernelOpLayerNormAffine : c.op; }

// Fill grid / rows_per_group / window and check every plan constraint.
// A looped plan (ROWRED_POLICY_LOOPED): one row per workgroup, any width.
int finish_looped_plan(const Call &c, rowred_plan *p) {
  const int64_t L = p->lanes_per_row, T = p->threads;
  if (L != T || !is_pow2(T) || T < 64 || T > 1024) return ROWRED_ERR_INVALID_ARG;
  if (!looped_kernel_exists(kernel_op(c), p->chunks)) return ROWRED_ERR_INVALID_ARG;
  if (p->policy & ~(kPolicyLooped | kPolicyNtLoads | kPolicyNtStores | kPolicyXcdRemap)) return ROWRED_ERR_INVALID_ARG;
  if (p->reserved != 0) return ROWRED_ERR_INVALID_ARG;
  p->window = c.window;
  p->vector_io = c.y_vec && (c.r == nullptr || c.r_vec) ? 1 : 0;
  p->rows_per_group = 1;
  p->grid = c.rows;
  if (p->grid > INT32_MAX || p->grid * T > (int64_t)UINT32_MAX) return ROWRED_ERR_UNSUPPORTED;
  return ROWRED_OK;
}

// An LDS-stripe plan (ROWRED_POLICY_LDS_STRIPE): RMSNorm or softmax, one
// 1024-lane workgroup per row, 5-16 chunks.
int finish_lds_plan(const Call &c, rowred_plan *p) {
  const int kop = kernel_op(c);
  if ((kop != ROWRED_OP_RMSNORM && kop != ROWRED_OP_SOFTMAX) || p->lanes_per_row != 1024 || p->threads != 1024 ||
      p->chunks < kWideMinChunks || p->chunks > kWideMaxChunks)
    return ROWRED_ERR_INVALID_ARG;
  if (p->policy & ~(kPolicyLdsStripe | kPolicyNtLoads | kPolicyNtStores | kPolicyXcdRemap | kPolicyOnline))
    return ROWRED_ERR_INVALID_ARG;
  if ((p->policy & kPolicyOnline) && kop != ROWRED_OP_SOFTMAX) return ROWRED_ERR_INVALID_ARG;
  if (p->reserved != 0) return ROWRED_ERR_INVALID_ARG;
  p->window = c.window;
  p->vector_io = c.y_vec ? 1 : 0;
  if ((int64_t)1024 * p->chunks < p->window) return ROWRED_ERR_INVALID_ARG;
  p->rows_per_group = 1;
  p->grid = c.rows;
  if (p->grid > INT32_MAX || p->grid * 1024 > (int64_t)UINT32_MAX) return ROWRED_ERR_UNSUPPORTED;
  return ROWRED_OK;
}

// A plan with the head of the row in registers and LDS and the rest walked
// twice (ROWRED_POLICY_LDS_STRIPE | ROWRED_POLICY_LOOPED), one 1024-lane
// workgroup per row: RMSNorm or softmax with chunks 16 (the head), LayerNorm
// (any) with chunks 8 (x and r of 8192 granules); rows wider than the head.
int finish_wide_tail_plan(const Call &c, rowred_plan *p) {
  const int kop = kernel_op(c);
  const bool ln = kop == ROWRED_OP_LAYERNORM_RESIDUAL || kop == kKernelOpLayerNormAffine;
  if ((kop != ROWRED_OP_RMSNORM && kop != ROWRED_OP_SOFTMAX && !ln) || p->lanes_per_row != 1024 ||
      p->threads != 1024 || p->chunks != (ln ? kLnTailHeadChunks : kWideMaxChunks))
    return ROWRED_ERR_INVALID_ARG;
  if (p->policy & ~(kPolicyLdsStripe | kPolicyLooped | kPolicyNtLoads | kPolicyNtStores | kPolicyXcdRemap |
                    kPolicyReverse))
    return ROWRED_ERR_INVALID_ARG;
  if (p->reserved != 0 || c.window <= (int64_t)1024 * p->chunks) return ROWRED_ERR_INVALID_ARG;
  p->window = c.window;
  p->vector_io = c.y_vec ? 1 : 0;
  p->rows_per_group = 1;
  p->grid = c.rows;
  if (p->grid > INT32_MAX || p->grid * 1024 > (int64_t)UINT32_MAX) return ROWRED_ERR_UNSUPPORTED;
  return ROWRED_OK;
}

// A flat plan (ROWRED_POLICY_FLAT): RMSNorm or softmax, rows of at least 4
// elements; the workgroup takes rows_per_group consecutive rows as one run of
// threads * chunks granules, lane after lane.
int finish_flat_plan(const Call &c, rowred_plan *p) {
  const int kop = kernel_op(c);
  const int64_t T = p->threads, C = p->chunks;
  if ((kop != ROWRED_OP_RMSNORM && kop != ROWRED_OP_SOFTMAX) || c.width < 4) return ROWRED_ERR_INVALID_ARG;
  if (T < 64 || T > kFlatMaxThreads || T % 64 != 0 || (C != 1 && C != 2 && C != 4))
    return ROWRED_ERR_INVALID_ARG;
  if (p->policy & ~(kPolicyFlat | kPolicyNtLoads | kPolicyNtStores | kPolicyXcdRemap)) return ROWRED_ERR_INVALID_ARG;
  if (p->reserved != 0) return ROWRED_ERR_INVALID_ARG;
  // rows_per_group: the run of P rows at any 16-byte phase fits T * C granules
  int64_t P = (4 * T * C - 3) / c.width;
  if (P > T) P = T;
  if (P < 1) return ROWRED_ERR_INVALID_ARG;
  int64_t lpr = 1;
  while (lpr < 64 && 2 * lpr * P <= T) lpr *= 2;
  p->lanes_per_row = (int32_t)lpr;
  p->rows_per_group = (int32_t)P;
  p->window = c.window;
  p->vector_io = c.y_vec ? 1 : 0;
  p->grid = (c.rows + P - 1) / P;
  if (p->grid > INT32_MAX || p->grid * T > (int64_t)UINT32_MAX) return ROWRED_ERR_UNSUPPORTED;
  return ROWRED_OK;
}

// The exchange path (defined with the split plans below).
bool choose_exchange(int op, int64_t rows, int64_t window, rowred_split_plan *p);
int finish_split(const Call &c, rowred_split_plan *p);
bool exchange_fits(int op, const rowred_split_plan &p);
int finish_row_exchange_plan(const Call &c, rowred_plan *p, rowred_split_plan *sp);
int run_row_exchange(const Call &c, const rowred_plan &plan, float eps, hipStream_t stream);

int finish_plan(const Call &c, rowred_plan *p) {
  if (p->policy & kPolicyExchange) return finish_row_exchange_plan(c, p, nullptr);
  if (p->policy & kPolicyFlat) return finish_flat_plan(c, p);
  if ((p->policy & kPolicyLooped) && (p->policy & kPolicyLdsStripe)) return finish_wide_tail_plan(c, p);
  if (p->policy & kPolicyLooped) return finish_looped_plan(c, p);
  if (p->policy & kPolicyLdsStripe) return finish_lds_plan(c, p);
  const int64_t L = p->lanes_per_row, T = p->threads;
  if (!is_pow2(L) || L > 1024) return ROWRED_ERR_INVALID_ARG;
  if (T < 64 || T > 1024 || T % 64 != 0 || T % L != 0) return ROWRED_ERR_INVALID_ARG;
  const int kop = kernel_op(c);
  if (!chunks_supported(p->chunks) || !kernel_exists(kop, p->chunks) || T > max_threads_for(kop, p->chunks))
    return ROWRED_ERR_INVALID_ARG;
  if (p->policy & ~kPolicyAll) return ROWRED_ERR_INVALID_ARG;
  const int cap = ROWRED_POLICY_CU_GROUPS_OF(p->policy);
  if (cap == 15) return ROWRED_ERR_INVALID_ARG;
  if ((p->policy & kPolicyOnline) && (kop != ROWRED_OP_SOFTMAX || (p->policy & kPolicyReload)))
    return ROWRED_ERR_INVALID_ARG;
  if ((p->policy & kPolicyReload) &&
      (!reload_kernel_exists(kop, p->chunks) || T > reload_max_threads_for(kop, p->chunks)))
    return ROWRED_ERR_INVALID_ARG;
  if (p->reserved != 0) return ROWRED_ERR_INVALID_ARG;
  p->window = c.window;
  p->vector_io = c.y_vec && (c.r == nullptr || c.r_vec) ? 1 : 0;
  if (L * p->chunks < p->window) return ROWRED_ERR_INVALID_ARG;
  p->rows_per_group = (int32_t)(T / L);
  if ((p->policy & kPolicyStageStores) && (!c.y_vec || T > kMaxStageThreads || p->chunks > kMaxStageChunks))
    return ROWRED_ERR_INVALID_ARG;
  p->grid = (c.rows + p->rows_per_group - 1) / p->rows_per_group;
  // The dispatch packet counts work-items in 32 bits.
  if (p->grid > INT32_MAX || p->grid * T > (int64_t)UINT32_MAX) return ROWRED_ERR_UNSUPPORTED;
  return ROWRED_OK;
}

// The chooser, keyed on the row window and the matrix size; its rules come
// from sweeps of every geometry and memory policy on MI355X at the workload
// shapes (widths 127, 257, 1537, 4096, 8192, 32768), each call on buffers
// rotated through >= 2 GiB so that no call runs from the last-level cache.
//
// Geometry: every input element is loaded once into registers, so the
// per-lane stripe sets register use and the serial work per lane.  Short
// stripes with many lanes per row win: at most 2 slots (8 floats) per lane --
// the pages' 8-float stripe at 4096 columns -- or 4 slots for inputs of at
// most 32 MiB, which run in a single round of waves where fewer, fatter
// waves amortise the wave start-up (8 slots for some of them, below), and for rows of at most 256 granules
// whose outputs are staged in LDS (below), where 4 slots per lane measured
// 4-8% faster than 2 (at 1537 columns 2 slots stay 10% faster).  L is the smallest power of two meeting
// that bound (at most 1024), chunks the smallest instantiated count covering
// the window.  Workgroups have max(256, L) threads for small inputs and
// max(512, L) for large ones.
//
// Memory policy: streaming (non-temporal) loads are 3-9% faster than cached
// ones at every workload shape except short rows that do not start on
// 16-byte boundaries (127 and 257 columns, 3-4% slower): neighbouring rows
// there share their boundary granule, which is read twice, once by each
// row's lanes.  Streaming (non-temporal) stores are fastest.  Where rows
// do not start on 16-byte boundaries, the cache lines at row boundaries
// hold two rows' outputs written by different lanes at different times,
// and each part leaves as its own partial line write-back (up to 1.46x the
// algorithmic write traffic at width 127, and 3x slower with streaming
// stores when a lane holds more than 2 slots).  Staging a workgroup's
// outputs in LDS and storing them as whole granules from consecutive threads
// removes that (ROWRED_POLICY_STAGE_STORES); without it (y at another
// 16-byte phase than x) stores stay cached beyond 2 slots per lane.  The XCD
// remap (each XCD walks one contiguous range of rows) pays off for aligned
// rows once the grid runs in several rounds (> 64 MiB per input).
//
// Row sum and min/max read only: nothing waits on stores, and idle slots
// cost more than long stripes.  With at most 4 slots per lane and at least
// 512 threads, 16384x8192 runs at 78-80 us and 131072x257 at 23-24 us,
// against 90-100 us and 32-36 us with the 2-slot stripes above (L = 64 x 2
// slots leaves half of each 257-column row's lanes idle).
// Rows wider than the register-resident kernels hold (or affine LayerNorm
// beyond its 6144-granule kernels) loop over the row: 1024 lanes, tiles of
// One workgroup per wide row: XCD remap from 2048 rows that start on 16-byte
// boundaries (measured for the looped and head+tail kernels below).
bool remap_many_aligned_rows(const Call &c) {
  return c.rows >= 2048 && c.width % 4 == 0 && ((uintptr_t)c.x & 15) == 0;
}

// 4 slots per lane (2 for LayerNorm), streaming loads and stores in the
// second walk.  Rows over the XCDs in contiguous runs from 2048 aligned rows
// (MI355X, row sum: 2048x131072 180 -> 172 us, row min/max 180 -> 174 us;
// 8192x40000 unchanged; 512x524288 and misaligned 4096x65537 1-4% slower).
void choose_looped(const Call &c, rowred_plan *p) {
  const int kop = kernel_op(c);
  *p = rowred_plan{};
  p->lanes_per_row = 1024;
  p->threads = 1024;
  p->chunks = looped_kernel_exists(kop, 4) ? 4 : 2;
  p->policy = kPolicyLooped | kPolicyNtLoads | kPolicyNtStores | (remap_many_aligned_rows(c) ? kPolicyXcdRemap : 0);
}

constexpr int64_t kLdsStripeMaxGranules = int64_t(2048) * 8192;

void choose_plan(const Call &c, rowred_plan *p) {
  // LayerNorm, RMSNorm and softmax rows wider than the register-resident
  // window: the exchange kernels with their words in y's own rows (no
  // workspace), so the row is read once, where the device holds twice a
  // row's segments; the geometry is the _ws entry points' (choose_exchange).
  // Faster than the LDS-stripe and head+tail kernels below at every shape
  // measured (MI355X): softmax 1024x50257 83.4 -> 75.1 us, 4096x65536 377
  // -> 336 us, 1024x262144 446 -> 357 us, 128x1048576 295 -> 211 us;
  // RMSNorm 2048x40000 116 -> 110 us, 2048x131072 385 -> 346 us, 64x1048576
  // 183 -> 108 us; residual LayerNorm 1024x65536 160 -> 137 us, 4096x32772
  // 299 -> 276 us, 256x262144 198 -> 154 us.
  // Affine LayerNorm keeps the head+tail kernels there from 256 rows (one
  // workgroup per row fills MI355X's 256 CUs; 2048x40000 141 -> 131 us,
  // 256x262144 145 -> 134 us, 4096x32772 265 -> 226 us); fewer rows leave
  // CUs idle (64x1048576 377 -> 167 us, 16x65536 20.3 -> 10.8 us through
  // the exchange kernels).
  if (c.window > kMaxWindow && c.op <= ROWRED_OP_SOFTMAX && ((!c.gamma && !c.beta) || c.rows < 256)) {
    rowred_split_plan sp;
    if (choose_exchange(c.op, c.rows, c.window, &sp)) {
      rowred_plan q = rowred_plan{};
      q.lanes_per_row = sp.threads;
      q.threads = sp.threads;
      q.chunks = sp.chunks;
      q.policy = sp.policy;
      rowred_plan t = q;
      if (finish_row_exchange_plan(c, &t, &sp) == ROWRED_OK && exchange_fits(c.op, sp)) {
        *p = q;
        return;
      }
    }
  }
  // RMSNorm and softmax rows of 8193-16384 granules: 8 register and up to 8
  // LDS slots per lane hold the whole row, read once (the looped kernels
  // read it twice).
  if (c.window > kMaxWindow && c.window <= kWideMaxWindow &&
      (c.op == ROWRED_OP_RMSNORM || c.op == ROWRED_OP_SOFTMAX)) {
    const bool aligned = c.width % 4 == 0 && ((uintptr_t)c.x & 15) == 0;
    p->lanes_per_row = 1024;
    p->threads = 1024;
    p->chunks = (int32_t)((c.window + 1023) / 1024);
    // softmax with one (max, sum) collective: 1024x50257 86.7 -> 83.4 us,
    // 4096x65536 383 -> 377 us (MI355X)
    p->policy = kPolicyLdsStripe | kPolicyNtLoads | kPolicyNtStores |
                (aligned && c.rows * c.width * 4 > (int64_t(64) << 20) ? kPolicyXcdRemap : 0) |
                (c.op == ROWRED_OP_SOFTMAX ? kPolicyOnline : 0);
    p->reserved = 0;
    return;
  }
  // Wider RMSNorm and softmax rows: the first 16384 granules held the same
  // way, the rest walked twice.  Faster than the looped kernels at every
  // width measured (MI355X): 4096x65540 softmax 486 -> 417 us, 2048x128256
  // 436 -> 381 us, 2048x131072 RMSNorm 493 -> 434 us, 1024x262144 softmax
  // 491 -> 446 us, 512x524288 491 -> 473 us, 128x1048576 321 -> 297 us.
  // Remapping rows over the XCDs pays from 2048 aligned rows (RMSNorm
  // 2048x131072 423 -> 382 us, softmax 2048x131072 429 -> 388 us, 4096x65540
  // 424 -> 405 us, RMSNorm 8192x65544 797 -> 777 us) and costs 2-6% at 128-1024
  // rows (softmax 512x524288 473 -> 499 us).
  if (c.window > kWideMaxWindow && (c.op == ROWRED_OP_RMSNORM || c.op == ROWRED_OP_SOFTMAX)) {
    p->lanes_per_row = 1024;
    p->threads = 1024;
    p->chunks = kWideMaxChunks;
    p->policy = kPolicyLdsStripe | kPolicyLooped | kPolicyNtLoads | kPolicyNtStores |
                (remap_many_aligned_rows(c) ? kPolicyXcdRemap : 0);
    p->reserved = 0;
    return;
  }
  // LayerNorm (residual, plain, affine) rows wider than 8192 granules: x and r
  // of the first 8192 held in registers and LDS, the rest walked twice.
  // Faster than the looped kernel at every shape measured (MI355X): residual
  // 1024x65536 191 -> 164 us, 2048x40000 233 -> 171 us, 4096x32772 400 ->
  // 298 us, 8192x36864 826 -> 635 us, 256x262144 211 -> 200 us; plain
  // 1024x65536 128 -> 109 us.  Remapping rows over the XCDs pays beyond 256
  // MiB per input (4-7%) and costs below (7%).
  if (c.window > kMaxWindow && c.op == ROWRED_OP_LAYERNORM_RESIDUAL) {
    const bool aligned = c.width % 4 == 0 && ((uintptr_t)c.x & 15) == 0;
    p->lanes_per_row = 1024;
    p->threads = 1024;
    p->chunks = kLnTailHeadChunks;
    p->policy = kPolicyLdsStripe | kPolicyLooped | kPolicyNtLoads | kPolicyNtStores |
                (aligned && c.rows * c.width * 4 > (int64_t(256) << 20) ? kPolicyXcdRemap : 0);
    p->reserved = 0;
    return;
  }
  if (c.window > kMaxWindow) {
    choose_looped(c, p);
    return;
  }
  // Large calls of rows of up to 8192 granules: the exchange kernels with
  // their words in y's rows too, in segments of 1024 granules (256 x 4;
  // softmax rows beyond 6144 granules 128 x 8), LayerNorm in segments of
  // 2048 (256 x 8, half in LDS) where they pad no more than segments of 1024
  // would.  Taken, from 128 MiB per input, for LayerNorm rows on 16-byte
  // boundaries beyond 2048 granules (residual LayerNorm from 4096), other
  // LayerNorm rows beyond 4096, RMSNorm / softmax rows on 16-byte boundaries
  // beyond 4096 granules whose segments pad at most 1/16 of the row (beyond
  // 6144 granules from 256 MiB: RMSNorm 1024x32768 49.1 -> 50.7 us at 128),
  // and from 512 MiB any RMSNorm / softmax rows beyond 4096; aligned RMSNorm / softmax
  // rows of exactly 4096 granules at 128-256 MiB run as two 2048-granule LDS
  // segments.  MI355X, against the register, LDS-stripe and looped kernels,
  // alternating order: residual LayerNorm 6553x20480 332 -> 255 us,
  // 4096x32768 280 -> 259 us, 8192x16384 270 -> 259 us, 8192x16383 312 -> 288
  // us; plain 11915x11264 238 -> 205 us, 8192x16384 217 -> 189 us; affine
  // 11915x11264 258 -> 243 us, 4096x32768 415 -> 234 us; softmax 8192x32768
  // 364 -> 339 us, 32768x16383 823 -> 711 us, 2048x16384 53.3 -> 49.8 us;
  // RMSNorm 8192x32768 357 -> 337 us, 4096x16384 93.6 -> 92.4 us.  They lose
  // elsewhere: in calls of 16 MiB by 20-30% (a second launch and the waits),
  // ragged LayerNorm of 2049-3001 granules by 5-34% (16384x8191 residual 260
  // -> 317 us), residual LayerNorm below 4096 granules and RMSNorm / softmax
  // rows of 3073-4095 by up to 13%, and ragged RMSNorm / softmax rows below
  // 512 MiB by 2-9%.
  {
    const bool ln = c.op == ROWRED_OP_LAYERNORM_RESIDUAL;
    const bool aligned = c.width % 4 == 0 && ((uintptr_t)c.x & 15) == 0;
    const int64_t bytes = c.rows * c.width * 4;
    const int64_t MiB = int64_t(1) << 20;
    const int64_t pad = (c.window + 1023) / 1024 * 1024 - c.window;  // of 1024-granule segments
    const bool rms_sm = c.op == ROWRED_OP_RMSNORM || c.op == ROWRED_OP_SOFTMAX;
    bool large = false;
    if (ln)
      large = bytes >= 128 * MiB && (aligned ? c.window > (c.r ? 4095 : 2048) : c.window > 4096);
    else if (rms_sm)
      large = (c.window > 4096 && (bytes >= 512 * MiB || (aligned && 16 * pad <= c.window &&
                                                            bytes >= (c.window > 6144 ? 256 : 128) * MiB))) ||
              (aligned && c.window == 4096 && bytes >= 128 * MiB && bytes <= 256 * MiB);
    if (large) {
      rowred_plan q = rowred_plan{};
      q.threads = 256;
      q.chunks = 4;
      q.policy = kPolicyExchange | kPolicyNtLoads | kPolicyNtStores;
      if ((ln && ((c.window + 1023) / 1024) % 2 == 0) || (!ln && c.window <= 4096)) {
        q.chunks = 8;
        q.policy |= kPolicyLdsStripe;
      } else if (c.op == ROWRED_OP_SOFTMAX && c.window > 6144) {
        q.threads = 128;
        q.chunks = 8;
      }
      q.lanes_per_row = q.threads;
      rowred_plan t = q;
      rowred_split_plan sp;
      if (finish_row_exchange_plan(c, &t, &sp) == ROWRED_OK && exchange_fits(c.op, sp)) {
        *p = q;
        return;
      }
    }
  }
  const int64_t w = c.window;
  const int64_t in_bytes = c.rows * c.width * 4;
  const bool small = in_bytes <= (int64_t(32) << 20);
  const bool rows_aligned = c.width % 4 == 0 && ((uintptr_t)c.x & 15) == 0;
  const bool scalar_out = c.op == ROWRED_OP_ROW_SUM || c.op == ROWRED_OP_ROW_MINMAX;
  const int kop = kernel_op(c);
  const bool affine = kop == kKernelOpLayerNormAffine;
  // Small calls (at most 2^19 elements, rows of at most 512 granules) are
  // latency-bound: one round of short-lived workgroups.  Two slots per lane
  // (L the smallest power of two >= half the window), one wavefront per
  // workgroup up to 2^16 elements and 256 threads beyond, streaming loads,
  // nothing staged: 0.4-1.3 us faster than the rules below at 1-4096 rows
  // of 127, 257 and 1537 columns (softmax and residual LayerNorm, MI355X;
  // 17x257 LayerNorm 3.38 -> 2.51 us, 1x127 3.20 -> 2.09 us, softmax
  // 7x1537 3.60 -> 2.69 us).  Affine LayerNorm, which also reads gamma and
  // beta per element, runs best with one slot per lane up to 256 granules
  // (1024x127 4.19 -> 2.91 us, 64x257 4.26 -> 2.90 us, 7x1537 4.47 -> 3.42 us
  // against its general rule).
  const bool tiny = c.rows * c.width <= (int64_t(1) << 19);
  if (!scalar_out && w <= 512 && tiny) {
    const int64_t slots = affine && w <= 256 ? 1 : 2;
    int64_t L = 8;
    while (L < 1024 && slots * L < w) L *= 2;
    p->lanes_per_row = (int32_t)L;
    p->chunks = round_up_chunks((w + L - 1) / L);
    const int64_t t_min = c.rows * c.width <= (int64_t(1) << 16) ? 64 : 256;
    p->threads = (int32_t)(L > t_min ? L : t_min);
    p->policy = kPolicyNtLoads;
    p->reserved = 0;
    return;
  }
  // RMSNorm and softmax rows that do not start on 16-byte boundaries, up to
  // 384 granules (1536 columns): the flat kernels, whose lanes take a
  // workgroup's rows as one run of granules (no slot idles past a row's end,
  // whole-granule stores).  MI355X, 2^25 elements per matrix, against the
  // rules below: RMSNorm 63, 127, 257 and 1023 columns 46.6 -> 43.2,
  // 46.2 -> 43.4, 46.2 -> 45.3, 54.2 -> 45.5 us (512 lanes x 2 granules);
  // softmax 63, 127, 257, 509, 1023 columns 51.4 -> 46.0, 50.5 -> 45.9,
  // 51.2 -> 49.9, 48.4 -> 47.5, 64.6 -> 48.7 us (256 x 4; softmax keeps the
  // rules below for rows of under 16 granules, 17 columns: 47.1 against 47.8).
  // 1537 columns and up: within 1% either way.
  const bool flat = (c.op == ROWRED_OP_RMSNORM || c.op == ROWRED_OP_SOFTMAX) && !rows_aligned && c.y_vec &&
                    c.width >= 4 && w <= 384 && (c.op == ROWRED_OP_RMSNORM || w >= 16);
  if (flat) {
    const bool rms = c.op == ROWRED_OP_RMSNORM;
    p->lanes_per_row = 0;  // derived by finish_plan
    p->threads = rms ? 512 : 256;
    p->chunks = rms ? 2 : 4;
    p->policy = kPolicyFlat | kPolicyNtLoads | kPolicyNtStores;
    p->reserved = 0;
    return;
  }
  // Large calls (beyond 64 MiB per input) on 16-byte aligned rows of
  // 128-2048 granules (RMSNorm, softmax, LayerNorm without gamma/beta;
  // residual LayerNorm to 8192 granules): a geometry per width band and a cap
  // on the workgroups sharing a CU (ROWRED_POLICY_CU_GROUPS).  Sweeps of
  // geometry x cap (0-10) at 2^27 elements per matrix (MI355X) put the
  // fastest plans at about 40-64 KiB of loads in flight per CU (threads per
  // CU x slots x 16 bytes) for one input and 64-128 KiB with r; more waves
  // than that only queue behind one another.  Against the rules below (both
  // timed in alternating order after a warm-up):
  //   RMSNorm    512, 1024, 2048, 4096, 8192 columns: 175.7 -> 163.7,
  //              170.5 -> 164.3, 170.6 -> 166.8, 170.3 -> 167.8, 169.4 -> 167.2 us
  //   softmax    171.3 -> 166.2, 170.8 -> 164.7, 169.6 -> 165.1, 167.9 -> 166.4,
  //              171.3 -> 166.4 us
  //   residual LayerNorm 1024, 2048, 4096, 8192, 16384, 32768 columns:
  //              259.5 -> 246.2, 259.4 -> 251.7, 256.8 -> 248.6, 253.8 -> 247.9,
  //              292.2 -> 269.0, 290.0 -> 279.9 us
  // (caps of 3 and 5 measured as 2 and 4: use even caps above 1).
  const bool two_in = c.r != nullptr && c.op == ROWRED_OP_LAYERNORM_RESIDUAL;
  if (rows_aligned && in_bytes > (int64_t(64) << 20) && !scalar_out && !affine && w >= 128 &&
      w <= (two_in ? 8192 : 2048)) {
    const bool sm = c.op == ROWRED_OP_SOFTMAX;
    int64_t L = 0, C = 0, T = 0, cap = 0;
    if (w <= 256) {
      L = 1;
      while (2 * L < w) L *= 2;
      C = 2;
      T = sm ? 256 : (L > 128 ? L : 128);
      cap = sm ? 6 : 10;
    } else if (w <= 512) {
      L = 256;
      C = 2;
      T = 256;
      cap = 6;
    } else if (w <= 1024) {
      L = two_in ? 256 : 128;
      C = two_in ? 4 : 8;
      T = two_in ? 512 : 256;
      cap = 2;
    } else if (w <= 2048) {
      L = two_in ? 512 : 256;
      C = two_in ? 4 : 8;
      T = two_in ? 512 : 256;
      cap = two_in ? 0 : 2;
    } else {  // residual LayerNorm: 512 lanes, 8 or 16 slots
      L = 512;
      C = w <= 4096 ? 8 : 16;
      T = 512;
    }
    p->lanes_per_row = (int32_t)L;
    p->chunks = (int32_t)C;
    p->threads = (int32_t)T;
    p->policy = kPolicyNtLoads | kPolicyNtStores | kPolicyXcdRemap | ROWRED_POLICY_CU_GROUPS(cap);
    p->reserved = 0;
    return;
  }
  // RMSNorm and softmax rows off 16-byte boundaries of 513-3072 granules
  // beyond 64 MiB: three slots per lane in one row per workgroup (L the
  // smallest power of two >= a third of the window, at least 256), at most 6
  // workgroups per CU at 256 lanes.  MI355X, against the rules below: RMSNorm
  // 65568x2047, 32776x4095, 16386x8191: 187.4 -> 173.6, 198.7 -> 175.7,
  // 178.7 -> 178.6 us; softmax 219.4 -> 173.5, 232.8 -> 176.9 (283.4 with
  // one collective), 186.4 -> 181.6 us (the rules below leave up to half of
  // each lane's slots past the row).
  if ((c.op == ROWRED_OP_RMSNORM || c.op == ROWRED_OP_SOFTMAX) && !rows_aligned && in_bytes > (int64_t(64) << 20) &&
      w > 512 && w <= 3072) {
    int64_t L = 256;
    while (3 * L < w) L *= 2;
    p->lanes_per_row = (int32_t)L;
    p->chunks = (int32_t)((w + L - 1) / L);
    p->threads = (int32_t)L;
    p->policy = kPolicyNtLoads | kPolicyNtStores | (L == 256 ? ROWRED_POLICY_CU_GROUPS(6) : 0);
    p->reserved = 0;
    return;
  }
  // Outputs are staged only for rows of at most 256 granules, where a
  // workgroup holds many rows whose boundary lines it shares: at 127-769
  // columns staging is 1-40% faster at 65536-262144 rows; from 1537 columns
  // it is 4% faster to 19% slower (65536x2049 softmax 266 -> 216 us
  // unstaged), so longer rows store unstaged and streaming.
  const bool stage_ok = !rows_aligned && c.y_vec && w <= 256;
  // Staged rows that fit one wavefront (<= 64 lanes x 4 slots) store through
  // LDS, so their lanes can hold more slots.
  int64_t max_chunks = (small || scalar_out || stage_ok) ? 4 : 2;
  // Single-round inputs of 8-32 MiB per input with two input streams
  // (residual LayerNorm), or of 16-32 MiB with rows of >= 1024 granules,
  // keep more loads in flight per lane with 8 slots: 5-10% and 0-6% faster
  // at 1024x4096, 2048x2048, 4096x1024, 8192x512 and 512x8192 (measured on
  // 16-byte-aligned rows; below 8 MiB 8 slots were up to 17% slower).
  const bool two_inputs = c.r != nullptr && c.op == ROWRED_OP_LAYERNORM_RESIDUAL;
  if (small && !scalar_out && !stage_ok && !affine &&
      ((two_inputs && in_bytes >= (int64_t(8) << 20)) || (w >= 1024 && in_bytes >= (int64_t(16) << 20))))
    max_chunks = 8;
  // Affine LayerNorm reads gamma and beta for every row it maps (from cache).
  // On aligned rows it runs best in 256-thread workgroups with 4 slots per
  // lane, 8 for rows of 1024-2048 granules beyond 32 MiB: 8-19% faster than
  // the rules above at 16384x8192, 32768x4096, 65536x2048, 131072x1024 and
  // 1024x4096, within 2% at 262144x512 (sweep of every geometry on MI355X).
  // Wider rows keep the rules above (16384 columns: 1024 x 4 best).  Beyond
  // 32 MiB, rows of at most 256 granules take 2 slots (131072x1024 175.5 ->
  // 168.8 us) and 8-slot stripes at most 4 workgroups per CU (16384x8192
  // 182.3 -> 179.0 us).
  bool affine_256 = false;
  if (affine && rows_aligned && w <= 2048) {
    max_chunks = !small && w >= 1024 ? 8 : !small && w <= 256 ? 2 : 4;
    affine_256 = true;
  }
  // Row sum and min/max on rows of 33-160 granules: of 4 and 5 slots per
  // lane take the one whose lane group wastes fewer slots (the smaller L x C;
  // 5 at 127, 257 and 511 columns: 8 x 5, 16 x 5, 32 x 5 -- 2%, 0% and 6%
  // faster than 4 slots; measured on MI355X).
  auto lanes_for = [&](int64_t mc) {
    int64_t l = 1;
    while (l < 1024 && (w + l - 1) / l > mc) l *= 2;
    return l;
  };
  if (scalar_out && w > 32 && w <= 160) {
    const int64_t l4 = lanes_for(4), l5 = lanes_for(5);
    if (l5 * round_up_chunks((w + l5 - 1) / l5) < l4 * round_up_chunks((w + l4 - 1) / l4)) max_chunks = 5;
  }
  int64_t L = lanes_for(max_chunks);
  // LayerNorm (plain, residual, affine) on rows longer than 256 granules
  // that do not start on 16-byte boundaries, beyond 32 MiB: 4 slots per lane
  // (5 beyond 1024 granules) with at most 512 lanes while that takes at most
  // 8 slots, one row per workgroup (at least 256 threads), rows remapped over
  // the XCDs (not affine: 1-2% slower there).  7-40% faster than the rules
  // above at 1023-12287 columns (MI355X, plain 16384x8191 299 -> 179 us,
  // 131200x1023 236 -> 170 us, residual 16384x8191 366 -> 262 us, affine
  // 16386x8191 468 -> 365 us, 32776x4095 407 -> 317 us, and with gamma /
  // beta on 16-byte boundaries read 16 bytes at a time and shifted into the
  // row's phase: 285 and 256 us; 16384x8191 283.6 us); 16383 columns keep
  // 1024 x 5.
  // Affine rows of at most 2560 granules (gamma and beta read 16 bytes at a
  // time from 4-byte boundaries) take 5 slots per lane, 128-thread
  // workgroups at 64 lanes: 131072x1023 335 -> 217 us, 65536x2047 333 -> 212
  // us (32768x4095 and 16384x8191 already 5: 215 and 238 us).
  const bool ln_ragged =
      (kop == ROWRED_OP_LAYERNORM_RESIDUAL || affine) && !rows_aligned && !small && w > 256;
  if (ln_ragged && affine && w <= 2560) {
    L = 1;
    while (5 * L < w) L *= 2;
    if (L > 1024) L = 1024;
  } else if (ln_ragged) {
    L = lanes_for(w <= 1024 ? 4 : 5);
    if (w > 384 && w <= 512) L = 256;  // 2 slots: 1537 columns 1-6% faster than 128 x 4
    if (L > 512 && (w + 511) / 512 <= 8) L = 512;
  }
  int chunks = round_up_chunks((w + L - 1) / L);
  // A stripe too wide for a 1024-lane workgroup of this kernel: halve the
  // lanes (and so double the stripe) until the kernel exists and fits.
  while (L > 1 && (L > max_threads_for(kop, chunks) || !kernel_exists(kop, chunks))) {
    L /= 2;
    chunks = round_up_chunks((w + L - 1) / L);
    if (chunks < 0) break;
  }
  if (chunks < 0) {  // affine LayerNorm beyond its widest register-resident kernel
    choose_looped(c, p);
    return;
  }
  p->lanes_per_row = (int32_t)L;
  p->chunks = chunks;
  // Row sum and min/max take 512 threads, except calls of at most 2^19
  // elements, where 256 are 0.05-0.2 us faster (1x4096 2.41 -> 2.24 us,
  // 256x1024 2.84 -> 2.68 us).
  const int64_t t_min = ln_ragged && affine && L <= 64 ? 128
                        : (small && !scalar_out) || affine_256 || (scalar_out && tiny) || ln_ragged ? 256
                                                                                                     : 512;
  p->threads = (int32_t)(L > t_min ? L : t_min);
  const bool can_stage = stage_ok && p->chunks > 0 && p->chunks <= kMaxStageChunks && p->threads <= kMaxStageThreads;
  int policy = 0;
  // Row sum and min/max on rows of at most 40 granules read them cached (the
  // boundary granule two neighbouring rows share is read by both): 2-7%
  // faster at 63 and 127 columns.
  if (!can_stage && !(scalar_out && w <= 40)) policy |= kPolicyNtLoads;
  if (!scalar_out && (rows_aligned || can_stage || p->chunks <= 2 || w > 256)) policy |= kPolicyNtStores;
  if (can_stage) policy |= kPolicyStageStores;
  if ((rows_aligned || (ln_ragged && !affine)) && in_bytes > (int64_t(64) << 20)) policy |= kPolicyXcdRemap;
  // Rows of 5-8 slots per 1024-lane workgroup: half the stripe in LDS lets
  // two workgroups share a CU.  Softmax 512x32768 and 2048x32768: 14% and 7%
  // faster, RMSNorm 512x32768 6% (MI355X).  Softmax, whose exponentials add
  // ALU work to overlap, keeps the LDS stripe at every row count (8192x32768
  // 383 -> 364 us, 16384x32768 763 -> 720 us, with one (max, sum)
  // collective); RMSNorm only up to 2048 rows of 8192 granules (8192x32768
  // 355 us in registers, 363 with the LDS stripe).
  if ((c.op == ROWRED_OP_RMSNORM || c.op == ROWRED_OP_SOFTMAX) && L == 1024 && p->threads == 1024 &&
      p->chunks >= 5 && p->chunks <= 8 && (c.op == ROWRED_OP_SOFTMAX || c.rows * w <= kLdsStripeMaxGranules))
    policy |= kPolicyLdsStripe;
  // Softmax across a 1024-lane row beyond 64 MiB: one (max, sum) collective
  // instead of two (8192x16384 177.4 -> 174.9 us; 2048x32768 97.7 -> 94.1 us
  // with the LDS stripe) -- on 16-byte aligned rows: rows off the boundaries
  // in registers measured slower with it (32776x4095 in 1024 x 2: 233 -> 283 us,
  // in 512 x 3: 176.9 -> 178.6 us).
  if (c.op == ROWRED_OP_SOFTMAX && L == 1024 &&
      ((policy & kPolicyLdsStripe) || (rows_aligned && in_bytes > (int64_t(64) << 20))))
    policy |= kPolicyOnline;
  if (affine_256 && !small && max_chunks == 8) policy |= ROWRED_POLICY_CU_GROUPS(4);
  p->policy = policy;
  p->reserved = 0;
}

int run(const Call &c, const rowred_plan &plan, float eps, hipStream_t stream) {
  if (plan.policy & kPolicyExchange) return run_row_exchange(c, plan, eps, stream);
  RowArgs a;
  a.x = c.x;
  a.r = c.r;
  a.y = c.y;
  a.rows = c.rows;
  a.width = (int32_t)c.width;
  a.lanes_log2 = ilog2(plan.lanes_per_row);
  a.eps = eps;
  a.inv_width = 1.0f / (float)c.width;
  a.policy = plan.policy;
  a.r_vec = c.r_vec ? 1 : 0;
  a.y_vec = c.y_vec ? 1 : 0;
  a.gamma = c.gamma;
  a.beta = c.beta;
  a.y2 = c.y2;
  // gamma/beta granule k is row granule k when every row starts on a
  // 16-byte boundary and both vectors are 16-byte aligned.
  a.affine_vec = (c.width % 4 == 0 && ((uintptr_t)c.x & 15) == 0 && ((uintptr_t)c.gamma & 15) == 0 &&
                  ((uintptr_t)c.beta & 15) == 0)
                     ? 1
                     : 0;
  a.group_rows = plan.rows_per_group;
  // affine rows at another 16-byte phase than gamma / beta: 16-byte gamma /
  // beta loads from 4-byte boundaries (a kernel of its own)
  a.affine_shift = (c.gamma || c.beta) && !a.affine_vec ? 1 : 0;
  const bool looped = (plan.policy & kPolicyLooped) != 0, lds = (plan.policy & kPolicyLdsStripe) != 0;
  const int err = (plan.policy & kPolicyFlat) ? launch_flat(kernel_op(c), plan.chunks, plan.grid, plan.threads, a, stream)
                  : looped && lds ? launch_wide_tail(kernel_op(c), plan.grid, a, stream)
                  : looped      ? launch_looped(kernel_op(c), plan.chunks, plan.grid, plan.threads, a, stream)
                  : lds         ? launch_wide(kernel_op(c), plan.chunks, plan.grid, a, stream)
                                : launch_rows(kernel_op(c), plan.chunks, plan.grid, plan.threads, a, stream);
  return err == 0 ? ROWRED_OK : ROWRED_ERR_HIP;
}

int entry(int op, const float *x, const float *r, float *y, int64_t rows, int64_t width, float eps, bool need_r,
          bool need_eps, hipStream_t stream) {
  Call c;
  int st = check_call(op, x, r, y, rows, width, need_r, need_eps, eps, &c);
  if (st != ROWRED_OK || rows == 0 || width == 0) return st;
  rowred_plan p;
  choose_plan(c, &p);
  if (p.chunks < 0) return ROWRED_ERR_UNSUPPORTED;
  st = finish_plan(c, &p);
  if (st != ROWRED_OK) return st;
  return run(c, p, eps, stream);
}

// Row sum / row min-max: outputs are `rows` floats each.
int check_reduce_call(int op, const float *x, float *out0, float *out1, int64_t rows, int64_t width, Call *out,
                      bool cap = false) {
  if (op != ROWRED_OP_ROW_SUM && op != ROWRED_OP_ROW_MINMAX) return ROWRED_ERR_INVALID_ARG;
  if (rows < 0 || width < 0) return ROWRED_ERR_INVALID_ARG;
  out->op = op;
  out->x = x;
  out->r = nullptr;
  out->y = out0;
  out->y2 = op == ROWRED_OP_ROW_MINMAX ? out1 : nullptr;
  out->rows = rows;
  out->width = width;
  out->r_vec = out->y_vec = false;
  out->window = 0;
  if (rows == 0) return ROWRED_OK;
  if (width == 0) return ROWRED_ERR_INVALID_ARG;  // a row needs at least one element
  if (width > ROWRED_MAX_WIDTH || rows > INT64_MAX / width || rows * width > INT64_MAX / 4) return ROWRED_ERR_UNSUPPORTED;
  if (!x || !out0 || (op == ROWRED_OP_ROW_MINMAX && !out1)) return ROWRED_ERR_INVALID_ARG;
  if (((uintptr_t)x & 3) || ((uintptr_t)out0 & 3) || (out->y2 && ((uintptr_t)out1 & 3))) return ROWRED_ERR_INVALID_ARG;
  const uintptr_t px = (uintptr_t)x, nx = (uintptr_t)(rows * width * 4), no = (uintptr_t)rows * 4;
  auto hits = [&](const void *o, const void *b, uintptr_t nb) {
    return (uintptr_t)o < (uintptr_t)b + nb && (uintptr_t)b < (uintptr_t)o + no;
  };
  if (hits(out0, (const void *)px, nx) || (out->y2 && (hits(out1, (const void *)px, nx) || hits(out1, out0, no))))
    return ROWRED_ERR_ALIAS;
  out->window = max_window(x, rows, width);
  if (cap && out->window > kMaxWindow) return ROWRED_ERR_UNSUPPORTED;
  return ROWRED_OK;
}

int row_reduce_entry(int op, const float *x, float *out0, float *out1, int64_t rows, int64_t width,
                     const rowred_plan *plan, hipStream_t stream) {
  Call c;
  int st = check_reduce_call(op, x, out0, out1, rows, width, &c);
  if (st != ROWRED_OK || rows == 0) return st;
  rowred_plan p;
  if (plan) {
    p = *plan;
  } else {
    choose_plan(c, &p);
    if (p.chunks < 0) return ROWRED_ERR_UNSUPPORTED;
  }
  st = finish_plan(c, &p);
  if (st != ROWRED_OK) return st;
  return run(c, p, 0.0f, stream);
}

bool op_has_eps(int op) { return op == ROWRED_OP_LAYERNORM_RESIDUAL || op == ROWRED_OP_RMSNORM; }

// LayerNorm with optional residual and affine vectors: check gamma / beta
// (width floats each, 4-byte aligned, not overlapping y) and attach them.
int attach_affine(Call *c, const float *gamma, const float *beta) {
  if (c->rows == 0 || c->width == 0) return ROWRED_OK;
  for (const float *v : {gamma, beta}) {
    if (!v) continue;
    if ((uintptr_t)v & 3) return ROWRED_ERR_INVALID_ARG;
    const uintptr_t pv = (uintptr_t)v, py = (uintptr_t)c->y;
    const uintptr_t nv = (uintptr_t)c->width * 4, ny = (uintptr_t)(c->rows * c->width * 4);
    if (pv < py + ny && py < pv + nv) return ROWRED_ERR_ALIAS;
  }
  c->gamma = gamma;
  c->beta = beta;
  return ROWRED_OK;
}

int layernorm_entry(const float *x, const float *r, const float *gamma, const float *beta, float *y, int64_t rows,
                    int64_t width, float eps, const rowred_plan *plan, hipStream_t stream) {
  Call c;
  int st = check_call(ROWRED_OP_LAYERNORM_RESIDUAL, x, r, y, rows, width, false, true, eps, &c);
  if (st != ROWRED_OK || rows == 0 || width == 0) return st;
  st = attach_affine(&c, gamma, beta);
  if (st != ROWRED_OK) return st;
  rowred_plan p;
  if (plan) {
    p = *plan;
  } else {
    choose_plan(c, &p);
    if (p.chunks < 0) return ROWRED_ERR_UNSUPPORTED;  // affine rows wider than 6144 granules
  }
  st = finish_plan(c, &p);
  if (st != ROWRED_OK) return st;
  return run(c, p, eps, stream);
}

// ---------------------------------------------------------------------------
// Split rows (the _ws entry points).
// ---------------------------------------------------------------------------

// Window at the worst 16-byte phase: the chooser and the workspace size do
// not depend on where x starts.
int64_t worst_window(int64_t width) { return (width + 6) / 4; }

// Split geometry, from sweeps of every (threads, chunks) and policy at
// 64x1048576, 1024x131072, 256x262144, 4096x65536 (matrix outputs) and
// 16x4194304 (row sum), each call on buffers rotated through >= 2 GiB:
//   * 256 threads x 2 slots per segment is best or within 3% of it for the
//     normalisations, 512 x 2 for row sum / min-max (10% ahead of 256 x 2);
//   * the apply kernel wants streaming loads and stores (cached stores are
//     10-20% slower); walking the pairs backwards or in blocks of rows (so
//     that the second read finds the first in the last-level cache) did not
//     pay: each extra pass of the three kernels costs ~3 us of launch and
//     drain, and blocks of 64-256 MiB gained at most 3-8%.
// Narrow rows take smaller segments, down to 64 granules, until every row
// has a few; the first geometry that gives the chip rows * S >=
// kSplitTargetGroups workgroups is taken (segments wider than the row are
// skipped), else the smallest.
constexpr int64_t kSplitTargetGroups = 1024;
constexpr int kSplitGeometries[][2] = {{512, 2}, {256, 2}, {256, 1}, {128, 1}, {64, 1}};
constexpr int kNumSplitGeometries = sizeof(kSplitGeometries) / sizeof(kSplitGeometries[0]);

void choose_split(int op, int64_t rows, int64_t width, rowred_split_plan *p) {
  const int64_t w = worst_window(width);
  const bool scalar_out = op == ROWRED_OP_ROW_SUM || op == ROWRED_OP_ROW_MINMAX;
  int pick = kNumSplitGeometries - 1;
  for (int i = scalar_out ? 0 : 1; i < kNumSplitGeometries; ++i) {
    const int64_t G = (int64_t)kSplitGeometries[i][0] * kSplitGeometries[i][1];
    if (G > w) continue;
    if (rows * ((w + G - 1) / G) >= kSplitTargetGroups) {
      pick = i;
      break;
    }
  }
  *p = rowred_split_plan{};
  p->threads = kSplitGeometries[pick][0];
  p->chunks = kSplitGeometries[pick][1];
  p->policy = kPolicyNtLoads | kPolicyNtStores;
}

// Exchange geometry (one-kernel split rows), from sweeps of (threads, chunks)
// x policy at 64x1048576, 1024x131072, 256x262144, 4096x65536, 2048x131072,
// 1024x65536 and few-row shapes (7x1537, 16x32768, 64x65536, 8x65536), each
// call on buffers rotated through >= 2 GiB.  A workgroup pays a fixed
// latency (its loads, then the wait for its row's other segments) that only
// more bytes per workgroup amortise:
//   * the time a row's workgroups spend waiting for each other grows with the
//     segments per row S, at any segment size (2^26-element matrices,
//     softmax at 256 x 8: S = 8, 16, 32, 64, 128 take 93, 96, 106, 118, 140
//     us; 8 + 8 LDS slots: S = 8, 16, 32, 64, 128: 96, 97, 101, 109, 124 us),
//     so the segment grows with the row to keep S low;
//   * RMSNorm and softmax: 256 threads x 8 register slots up to 16 segments
//     (2 slots per lane were 1.5-2x slower), then 8 register + 8 LDS slots
//     (LDS_STRIPE) up to 64 (256x262144 softmax 106 -> 97 us, 128x524288
//     118 -> 101 us, RMSNorm 102 -> 95 and 115 -> 100 us); wider rows take
//     the three split kernels (32x2097152 softmax 121 us against 124 for
//     128 segments of 8 + 8);
//   * LayerNorm, whose x and r both take slots: 4 register + 4 LDS slots
//     (LDS_STRIPE; 10% faster than 256 x 4 registers at 1024x65536, 25% at
//     256x262144) up to 32 segments, then 8 + 8 up to 128 (64x1048576 194 ->
//     174 us, 32x2097152 211 -> 188 us), then 1024 x 4.
//   * rows narrower than two segments of the first geometry take the first
//     of 256 x 4, 256 x 2, 128 x 2, 64 x 2 whose segment is at most half the
//     row (else 64 x 1): few-row shapes are latency bound and gain from more,
//     shorter segments;
//   * streaming loads and stores, as everywhere on rows read once.
// `window`: the row's 16-byte granules (the x at hand's, or the worst phase's
// for sizing).  False when no geometry cuts the row into at most its
// max_segments.  Keeping a row's segments on one XCD was 25-60% slower
// everywhere.  kExchangeChosenSegments bounds the halved segments of calls
// with few workgroups (below).
constexpr int64_t kExchangeChosenSegments = 64;
struct ExchangeGeometry {
  int threads, chunks;
  bool lds;
  int max_segments;  // the widest row (in segments) the geometry is chosen for
};
constexpr ExchangeGeometry kExchangeWide[2][3] = {
    {{256, 8, true, 32}, {256, 16, true, 128}, {1024, 4, false, 64}},  // LayerNorm
    {{256, 8, false, 16}, {256, 16, true, 64}, {0, 0, false, 0}},      // RMSNorm, softmax
};
constexpr int kExchangeNarrow[][2] = {{256, 4}, {256, 2}, {128, 2}, {64, 2}, {64, 1}};

// rows: the call's row count; with no more (row, segment) workgroups than
// the 256 CUs the segment is halved to 256 x 4 where that keeps S <= 64
// (MI355X: LayerNorm 8x65536 11.5 -> 8.7 us, RMSNorm 16x32768 7.3 -> 5.6
// us; from 512 workgroups the larger segments stay ahead).  rows = 0 asks
// for the plan with the most segments any row count can get (workspace
// sizing).
bool choose_exchange(int op, int64_t rows, int64_t window, rowred_split_plan *p) {
  if (op > ROWRED_OP_SOFTMAX) return false;
  const int64_t w = window;
  const auto &wide = kExchangeWide[op == ROWRED_OP_LAYERNORM_RESIDUAL ? 0 : 1];
  int T = 0, C = 0;
  bool lds = false;
  if (w >= 2 * (int64_t)wide[0].threads * wide[0].chunks) {
    for (const auto &g : wide) {
      if (!g.threads) break;
      const int64_t G = (int64_t)g.threads * g.chunks;
      const int64_t S = (w + G - 1) / G;
      if (S <= g.max_segments && S <= g.threads) {
        T = g.threads;
        C = g.chunks;
        lds = g.lds;
        break;
      }
    }
    if (!T) return false;
    const int64_t G = (int64_t)T * C;
    const int64_t S = (w + G - 1) / G, S_half = (w + 1023) / 1024;
    if (rows * S <= 256 && S_half <= kExchangeChosenSegments && S_half <= 256) {
      T = 256;
      C = 4;
      lds = false;
    }
  } else {
    T = 64;
    C = 1;
    for (const auto &g : kExchangeNarrow) {
      if (2 * (int64_t)g[0] * g[1] <= w) {
        T = g[0];
        C = g[1];
        break;
      }
    }
  }
  *p = rowred_split_plan{};
  p->threads = T;
  p->chunks = C;
  p->policy = kPolicyExchange | kPolicyNtLoads | kPolicyNtStores | (lds ? kPolicyLdsStripe : 0);
  return true;
}

// The split plan of a _ws call: exchange where it applies, else the three
// split kernels.
void choose_ws_split(int op, int64_t rows, int64_t width, int64_t window, rowred_split_plan *p) {
  if (!choose_exchange(op, rows, window, p)) choose_split(op, rows, width, p);
}

// Validate an explicit or chosen split plan and fill its derived fields.
int finish_split(const Call &c, rowred_split_plan *p) {
  const int64_t T = p->threads;
  if (!is_pow2(T) || T < 64 || T > 1024) return ROWRED_ERR_INVALID_ARG;
  if (p->policy & ~kSplitPolicyAll) return ROWRED_ERR_INVALID_ARG;
  const bool exchange = (p->policy & kPolicyExchange) != 0;
  const bool lds = (p->policy & kPolicyLdsStripe) != 0;
  if (lds) {  // exchange kernels with part of the segment in LDS
    if (!exchange || c.op > ROWRED_OP_SOFTMAX || T != kXldsThreads || xlds_stripe_index(c.op, p->chunks) < 0)
      return ROWRED_ERR_INVALID_ARG;
  } else {
    if (p->chunks != 1 && p->chunks != 2 && p->chunks != 4 && !(exchange && p->chunks == 8))
      return ROWRED_ERR_INVALID_ARG;
    if (exchange && (T > exchange_max_threads(p->chunks) || !exchange_kernel_exists(c.op, p->chunks)))
      return ROWRED_ERR_INVALID_ARG;
  }
  if (exchange && ((p->policy & kPolicyReverse) || c.op > ROWRED_OP_SOFTMAX)) return ROWRED_ERR_INVALID_ARG;
  if (p->block_rows < 0 || p->wait_polls < 0 || p->reserved != 0) return ROWRED_ERR_INVALID_ARG;
  const int64_t G = T * p->chunks;
  const int64_t br = p->block_rows == 0 || p->block_rows > c.rows ? c.rows : p->block_rows;
  p->block_rows = br;
  p->window = c.window;
  p->segments = (c.window + G - 1) / G;
  // lane k of the workgroup reads segment k's slot
  if (exchange && (p->segments > kMaxExchangeSegments || p->segments > T)) return ROWRED_ERR_INVALID_ARG;
  if (p->segments > INT32_MAX || br > INT64_MAX / p->segments) return ROWRED_ERR_UNSUPPORTED;
  p->grid = br * p->segments;
  if (p->grid > INT32_MAX || p->grid * T > (int64_t)UINT32_MAX) return ROWRED_ERR_UNSUPPORTED;
  p->workspace_bytes = (p->grid + br) * 16;
  return ROWRED_OK;
}

// The S workgroups of a row wait for each other, so they must all be
// resident at once.  Workgroups reach each XCD in index order and a row's
// segments have consecutive indices, so the oldest unfinished row always
// has its segments dispatched as long as the device holds more than S of
// them; twice S leaves room for workgroups of the next row (and for other
// kernels that hold compute units for a while).  Needs the current device.
bool exchange_fits(int op, const rowred_split_plan &p) {
  return exchange_resident_groups(op, p.chunks, p.threads, p.policy) >= 2 * p.segments;
}

// A row plan with ROWRED_POLICY_EXCHANGE: LayerNorm, RMSNorm or softmax rows
// cut into segments of threads * chunks granules, one workgroup each, that
// swap their statistics through words in y's own row (the first 16-byte
// boundary of the row on; segment 0 writes its outputs over them last).
// lanes_per_row == threads; policy: EXCHANGE with NT_LOADS, NT_STORES and
// LDS_STRIPE as on split plans.  grid = rows * segments.  *sp (optional)
// receives the matching split plan.
int finish_row_exchange_plan(const Call &c, rowred_plan *p, rowred_split_plan *sp) {
  if (c.op > ROWRED_OP_SOFTMAX || p->lanes_per_row != p->threads || p->reserved != 0) return ROWRED_ERR_INVALID_ARG;
  if (p->policy & ~(kPolicyExchange | kPolicyNtLoads | kPolicyNtStores | kPolicyLdsStripe))
    return ROWRED_ERR_INVALID_ARG;
  rowred_split_plan q = rowred_split_plan{};
  q.threads = p->threads;
  q.chunks = p->chunks;
  q.policy = p->policy;
  const int st = finish_split(c, &q);  // the whole matrix in one launch (block_rows = rows)
  if (st != ROWRED_OK) return st;
  // the row's words end inside the row and inside segment 0's outputs; for
  // LayerNorm inside the granules of segment 0's first slot (which the row's
  // last workgroup stores)
  const bool ln = c.op == ROWRED_OP_LAYERNORM_RESIDUAL;
  const int64_t bytes = row_exchange_bytes(ln ? 2 : 1, q.segments);
  if (bytes > 16 * (int64_t)q.threads * (ln ? 1 : q.chunks) - 12 || bytes > 4 * c.width) return ROWRED_ERR_INVALID_ARG;
  p->rows_per_group = 1;
  p->window = c.window;
  p->vector_io = c.y_vec && (c.r == nullptr || c.r_vec) ? 1 : 0;
  p->grid = q.grid;
  if (sp) *sp = q;
  return ROWRED_OK;
}

// Run a row exchange plan: the row clear of each row's words in y, then the
// exchange kernel.  The device must hold twice a row's segments at once
// (ROWRED_ERR_UNSUPPORTED otherwise).
int run_row_exchange(const Call &c, const rowred_plan &plan, float eps, hipStream_t stream) {
  rowred_plan p = plan;
  rowred_split_plan q;
  const int st = finish_row_exchange_plan(c, &p, &q);
  if (st != ROWRED_OK) return st;
  if (!exchange_fits(c.op, q)) return ROWRED_ERR_UNSUPPORTED;
  SegArgs a;
  a.x = c.x;
  a.r = c.r;
  a.gamma = c.gamma;
  a.beta = c.beta;
  a.y = c.y;
  a.y2 = nullptr;
  a.ws = nullptr;
  a.ws_in_y = 1;
  a.rows = c.rows;
  a.width = (int32_t)c.width;
  a.segments = (int32_t)q.segments;
  a.lanes_log2 = ilog2(q.threads);
  a.seg_granules = q.threads * q.chunks;
  a.eps = eps;
  a.inv_width = 1.0f / (float)c.width;
  a.policy = q.policy;
  a.r_vec = c.r_vec ? 1 : 0;
  a.y_vec = c.y_vec ? 1 : 0;
  a.spin_limit = kExchangeSpinLimit;
  return launch_exchange(c.op, q.chunks, q.grid, q.threads, a, true, stream) != 0 ? ROWRED_ERR_HIP : ROWRED_OK;
}

// static_ws: the library's own workspace (rowred_static_ws), whose size is
// a limit of the library rather than an argument error.
int run_split(const Call &c, const rowred_split_plan &p, float eps, void *ws, size_t ws_bytes, bool static_ws,
              hipStream_t stream) {
  if (!ws || ((uintptr_t)ws & 15)) return ROWRED_ERR_INVALID_ARG;
  if ((int64_t)ws_bytes < p.workspace_bytes) return static_ws ? ROWRED_ERR_UNSUPPORTED : ROWRED_ERR_INVALID_ARG;
  // the workspace overlaps none of the operands
  const uintptr_t w0 = (uintptr_t)ws, w1 = w0 + (uintptr_t)p.workspace_bytes;
  auto hit = [&](const void *b, int64_t nb) {
    return b && nb > 0 && (uintptr_t)b < w1 && w0 < (uintptr_t)b + (uintptr_t)nb;
  };
  const int64_t mat = c.rows * c.width * 4;
  const bool scalar = c.op == ROWRED_OP_ROW_SUM || c.op == ROWRED_OP_ROW_MINMAX;
  const int64_t out_bytes = scalar ? c.rows * 4 : mat;
  if (hit(c.x, mat) || hit(c.r, mat) || hit(c.y, out_bytes) || hit(c.y2, c.rows * 4) || hit(c.gamma, c.width * 4) ||
      hit(c.beta, c.width * 4))
    return ROWRED_ERR_ALIAS;
  SegArgs a;
  a.gamma = c.gamma;
  a.beta = c.beta;
  a.ws = static_cast<double *>(ws);
  a.ws_in_y = 0;
  a.width = (int32_t)c.width;
  a.segments = (int32_t)p.segments;
  a.lanes_log2 = ilog2(p.threads);
  a.seg_granules = p.threads * p.chunks;
  a.eps = eps;
  a.inv_width = 1.0f / (float)c.width;
  a.policy = p.policy;
  a.r_vec = c.r_vec ? 1 : 0;
  a.y_vec = c.y_vec ? 1 : 0;
  a.spin_limit = p.wait_polls > 0 ? (uint32_t)p.wait_polls : kExchangeSpinLimit;
  // Row blocks run one after another; offsetting every operand by whole
  // rows keeps r and y at x's 16-byte phase.  The workspace is reused; the
  // exchange status word is cleared by the first block only.
  for (int64_t r0 = 0; r0 < c.rows; r0 += p.block_rows) {
    const int64_t n = c.rows - r0 < p.block_rows ? c.rows - r0 : p.block_rows;
    const int64_t e0 = r0 * c.width;
    a.x = c.x + e0;
    a.r = c.r ? c.r + e0 : nullptr;
    a.y = scalar ? c.y + r0 : c.y + e0;
    a.y2 = c.y2 ? c.y2 + r0 : nullptr;
    a.rows = n;
    // kernel operator = the public op: LayerNorm (any of r, gamma, beta) 0,
    // RMSNorm 1, softmax 2, row sum 3, row min/max 4
    const int err = (p.policy & kPolicyExchange)
                        ? launch_exchange(c.op, p.chunks, n * p.segments, p.threads, a, r0 == 0, stream)
                        : launch_split(c.op, p.chunks, n * p.segments, p.threads, a, stream);
    if (err != 0) return ROWRED_ERR_HIP;
  }
  return ROWRED_OK;
}

// Checks of a _ws call: those of the register-resident entry points without
// the width cap.  gamma / beta only with LayerNorm.
int check_ws_call(int op, const float *x, const float *r, const float *gamma, const float *beta, float *y, float *y2,
                  int64_t rows, int64_t width, float eps, Call *c) {
  if (op == ROWRED_OP_ROW_SUM || op == ROWRED_OP_ROW_MINMAX) {
    if (r || gamma || beta) return ROWRED_ERR_INVALID_ARG;
    return check_reduce_call(op, x, y, y2, rows, width, c, false);
  }
  if (op != ROWRED_OP_LAYERNORM_RESIDUAL && (r || gamma || beta)) return ROWRED_ERR_INVALID_ARG;
  if (y2) return ROWRED_ERR_INVALID_ARG;
  int st = check_call(op, x, r, y, rows, width, false, op_has_eps(op), eps, c, false);
  if (st != ROWRED_OK || rows == 0 || width == 0) return st;
  return op == ROWRED_OP_LAYERNORM_RESIDUAL ? attach_affine(c, gamma, beta) : ROWRED_OK;
}

// Rows beyond the register-resident window where the exchange kernels do
// not apply (row sum and min/max, or rows too wide): with at least this many
// rows the looped kernels (one workgroup per row, no workspace) fill the chip
// and beat the three split kernels (softmax 4096x65536: 0.88x the time,
// residual LayerNorm 1024x65536: 0.94x); with fewer the split kernels win,
// by up to 6x on 16 rows (measured on MI355X).  The exchange kernels beat
// both on matrix outputs (4096x65536 softmax: 0.79x the looped time).
constexpr int64_t kLoopedMinRows = 2048;

// A _ws call: the register-resident kernels when the row fits them, the
// exchange kernels for wider rows of the matrix operators, the looped
// kernels for many wide rows, else (or with an explicit split plan) the
// three split kernels.
int ws_entry(int op, const float *x, const float *r, const float *gamma, const float *beta, float *y, float *y2,
             int64_t rows, int64_t width, float eps, const rowred_split_plan *plan, void *ws, size_t ws_bytes,
             hipStream_t stream, bool static_ws = false) {
  Call c;
  int st = check_ws_call(op, x, r, gamma, beta, y, y2, rows, width, eps, &c);
  if (st != ROWRED_OK || rows == 0 || width == 0) return st;
  rowred_split_plan sp;
  bool exchange = !plan && c.window > kMaxWindow && choose_exchange(op, c.rows, c.window, &sp);
  if (exchange) {
    // the device must hold twice a row's segments at once (else: the other
    // paths below)
    st = finish_split(c, &sp);
    if (st != ROWRED_OK) return st;
    exchange = exchange_fits(op, sp);
  }
  if (!plan && !exchange && (c.window <= kMaxWindow || c.rows >= kLoopedMinRows)) {
    rowred_plan p;
    choose_plan(c, &p);
    if (p.chunks >= 0) {
      st = finish_plan(c, &p);
      if (st != ROWRED_OK) return st;
      return run(c, p, eps, stream);
    }
  }
  rowred_split_plan p;
  if (plan) {
    p = *plan;
  } else if (exchange) {
    p = sp;
  } else {
    choose_split(op, rows, width, &p);
  }
  st = finish_split(c, &p);
  if (st != ROWRED_OK) return st;
  if ((p.policy & kPolicyExchange) && !exchange_fits(op, p)) return ROWRED_ERR_UNSUPPORTED;
  if (static_ws) {  // the library's array, looked up only once a call needs it
    const int e = static_workspace(&ws);
    if (e != 0) return ROWRED_ERR_HIP;
    ws_bytes = (size_t)ROWRED_STATIC_WORKSPACE_BYTES;
  }
  return run_split(c, p, eps, ws, ws_bytes, static_ws, stream);
}

}  // namespace
}  // namespace rowred

using namespace rowred;

ROWRED_API int rowred_layernorm_residual(const float *x, const float *r, float *y, int64_t rows, int64_t width,
                                         float eps, hipStream_t stream) {
  return entry(ROWRED_OP_LAYERNORM_RESIDUAL, x, r, y, rows, width, eps, true, true, stream);
}

ROWRED_API int rowred_layernorm(const float *x, const float *r, const float *gamma, const float *beta, float *y,
                                int64_t rows, int64_t width, float eps, hipStream_t stream) {
  return layernorm_entry(x, r, gamma, beta, y, rows, width, eps, nullptr, stream);
}

ROWRED_API int rowred_layernorm_run_plan(const float *x, const float *r, const float *gamma, const float *beta,
                                         float *y, int64_t rows, int64_t width, float eps, const rowred_plan *plan,
                                         hipStream_t stream) {
  if (!plan) return ROWRED_ERR_INVALID_ARG;
  return layernorm_entry(x, r, gamma, beta, y, rows, width, eps, plan, stream);
}

ROWRED_API int rowred_row_sum(const float *x, float *out, int64_t rows, int64_t width, hipStream_t stream) {
  return row_reduce_entry(ROWRED_OP_ROW_SUM, x, out, nullptr, rows, width, nullptr, stream);
}

ROWRED_API int rowred_row_minmax(const float *x, float *out_min, float *out_max, int64_t rows, int64_t width,
                                 hipStream_t stream) {
  return row_reduce_entry(ROWRED_OP_ROW_MINMAX, x, out_min, out_max, rows, width, nullptr, stream);
}

ROWRED_API int rowred_row_reduce_run_plan(int op, const float *x, float *out0, float *out1, int64_t rows,
                                          int64_t width, const rowred_plan *plan, hipStream_t stream) {
  if (!plan) return ROWRED_ERR_INVALID_ARG;
  return row_reduce_entry(op, x, out0, out1, rows, width, plan, stream);
}

ROWRED_API int rowred_rmsnorm(const float *x, float *y, int64_t rows, int64_t width, float eps,
                              hipStream_t stream) {
  return entry(ROWRED_OP_RMSNORM, x, nullptr, y, rows, width, eps, false, true, stream);
}

ROWRED_API int rowred_softmax(const float *x, float *y, int64_t rows, int64_t width, hipStream_t stream) {
  return entry(ROWRED_OP_SOFTMAX, x, nullptr, y, rows, width, 0.0f, false, false, stream);
}

ROWRED_API int rowred_plan_query(int op, const float *x, const float *r, const float *y, int64_t rows,
                                 int64_t width, rowred_plan *out) {
  if (!out) return ROWRED_ERR_INVALID_ARG;
  Call c;
  const bool has_r = op == ROWRED_OP_LAYERNORM_RESIDUAL;  // LayerNorm: the residual is optional here
  int st = op == ROWRED_OP_ROW_SUM || op == ROWRED_OP_ROW_MINMAX
               ? check_reduce_call(op, x, const_cast<float *>(y), const_cast<float *>(r), rows, width, &c)
               : check_call(op, x, has_r ? r : nullptr, y, rows, width, false, false, 0.0f, &c);
  if (st != ROWRED_OK) return st;
  if (rows == 0 || width == 0) {
    *out = rowred_plan{0, 0, 0, 0, 0, 0, 0, 0, 0};
    return ROWRED_OK;
  }
  choose_plan(c, out);
  if (out->chunks < 0) return ROWRED_ERR_UNSUPPORTED;
  return finish_plan(c, out);
}

ROWRED_API int rowred_layernorm_plan_query(const float *x, const float *r, const float *gamma, const float *beta,
                                           const float *y, int64_t rows, int64_t width, rowred_plan *out) {
  if (!out) return ROWRED_ERR_INVALID_ARG;
  Call c;
  int st = check_call(ROWRED_OP_LAYERNORM_RESIDUAL, x, r, const_cast<float *>(y), rows, width, false, false, 0.0f,
                      &c);
  if (st != ROWRED_OK) return st;
  if (rows == 0 || width == 0) {
    *out = rowred_plan{0, 0, 0, 0, 0, 0, 0, 0, 0};
    return ROWRED_OK;
  }
  st = attach_affine(&c, gamma, beta);
  if (st != ROWRED_OK) return st;
  choose_plan(c, out);
  if (out->chunks < 0) return ROWRED_ERR_UNSUPPORTED;
  return finish_plan(c, out);
}

ROWRED_API int rowred_run_plan(int op, const float *x, const float *r, float *y, int64_t rows, int64_t width,
                               float eps, const rowred_plan *plan, hipStream_t stream) {
  if (!plan) return ROWRED_ERR_INVALID_ARG;
  Call c;
  const bool need_r = op == ROWRED_OP_LAYERNORM_RESIDUAL;
  int st = check_call(op, x, need_r ? r : nullptr, y, rows, width, need_r, op_has_eps(op), eps, &c);
  if (st != ROWRED_OK || rows == 0 || width == 0) return st;
  rowred_plan p = *plan;
  st = finish_plan(c, &p);
  if (st != ROWRED_OK) return st;
  return run(c, p, eps, stream);
}

ROWRED_API int rowred_workspace_size(int op, int64_t rows, int64_t width, size_t *bytes) {
  if (!bytes) return ROWRED_ERR_INVALID_ARG;
  if (op < 0 || op > ROWRED_OP_ROW_MINMAX || rows < 0 || width < 0) return ROWRED_ERR_INVALID_ARG;
  *bytes = 0;
  if (rows == 0 || width == 0) return ROWRED_OK;
  if (width > ROWRED_MAX_WIDTH || rows > INT64_MAX / width || rows * width > INT64_MAX / 4) return ROWRED_ERR_UNSUPPORTED;
  // enough for the three split kernels and for the exchange kernels at the
  // worst 16-byte phase of x.  (An x whose own window admits the exchange
  // kernels where the worst phase does not needs fewer, wider segments than
  // the three-kernel plan counted here.)
  rowred_split_plan p;
  choose_split(op, rows, width, &p);
  int64_t G = (int64_t)p.threads * p.chunks;
  int64_t S = (worst_window(width) + G - 1) / G;
  // every exchange plan a call of this width may run: the row count decides
  // between two, and rows = 0 gives the one with the most segments
  for (const int64_t rr : {rows, (int64_t)0}) {
    if (choose_exchange(op, rr, worst_window(width), &p)) {
      G = (int64_t)p.threads * p.chunks;
      const int64_t Sx = (worst_window(width) + G - 1) / G;
      S = Sx > S ? Sx : S;
    }
  }
  if (rows > INT64_MAX / 16 / (S + 1)) return ROWRED_ERR_UNSUPPORTED;
  *bytes = (size_t)(rows * (S + 1) * 16);
  return ROWRED_OK;
}

ROWRED_API int rowred_layernorm_ws(const float *x, const float *r, const float *gamma, const float *beta, float *y,
                                   int64_t rows, int64_t width, float eps, void *workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  return ws_entry(ROWRED_OP_LAYERNORM_RESIDUAL, x, r, gamma, beta, y, nullptr, rows, width, eps, nullptr, workspace,
                  workspace_bytes, stream);
}

ROWRED_API int rowred_rmsnorm_ws(const float *x, float *y, int64_t rows, int64_t width, float eps, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  return ws_entry(ROWRED_OP_RMSNORM, x, nullptr, nullptr, nullptr, y, nullptr, rows, width, eps, nullptr, workspace,
                  workspace_bytes, stream);
}

ROWRED_API int rowred_softmax_ws(const float *x, float *y, int64_t rows, int64_t width, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  return ws_entry(ROWRED_OP_SOFTMAX, x, nullptr, nullptr, nullptr, y, nullptr, rows, width, 0.0f, nullptr, workspace,
                  workspace_bytes, stream);
}

ROWRED_API int rowred_row_sum_ws(const float *x, float *out, int64_t rows, int64_t width, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  return ws_entry(ROWRED_OP_ROW_SUM, x, nullptr, nullptr, nullptr, out, nullptr, rows, width, 0.0f, nullptr,
                  workspace, workspace_bytes, stream);
}

ROWRED_API int rowred_row_minmax_ws(const float *x, float *out_min, float *out_max, int64_t rows, int64_t width,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream) {
  return ws_entry(ROWRED_OP_ROW_MINMAX, x, nullptr, nullptr, nullptr, out_min, out_max, rows, width, 0.0f, nullptr,
                  workspace, workspace_bytes, stream);
}

ROWRED_API int rowred_static_ws(int op, const float *x, const float *r, const float *gamma, const float *beta,
                                float *y, float *y2, int64_t rows, int64_t width, float eps, hipStream_t stream) {
  return ws_entry(op, x, r, gamma, beta, y, y2, rows, width, eps, nullptr, nullptr, 0, stream, true);
}

ROWRED_API int rowred_split_plan_query(int op, const float *x, int64_t rows, int64_t width,
                                       rowred_split_plan *plan) {
  if (!plan || op < 0 || op > ROWRED_OP_ROW_MINMAX || rows < 0 || width < 0) return ROWRED_ERR_INVALID_ARG;
  if (rows == 0 || width == 0) {
    *plan = rowred_split_plan{};
    return ROWRED_OK;
  }
  if (!x || ((uintptr_t)x & 3)) return ROWRED_ERR_INVALID_ARG;
  if (width > ROWRED_MAX_WIDTH || rows > INT64_MAX / width || rows * width > INT64_MAX / 4) return ROWRED_ERR_UNSUPPORTED;
  Call c;
  c.op = op;
  c.x = x;
  c.r = nullptr;
  c.y = nullptr;
  c.rows = rows;
  c.width = width;
  c.r_vec = c.y_vec = false;
  c.window = max_window(x, rows, width);
  if (plan->threads == 0) choose_ws_split(op, rows, width, c.window, plan);
  return finish_split(c, plan);
}

ROWRED_API int rowred_split_run_plan(int op, const float *x, const float *r, const float *gamma, const float *beta,
                                     float *y, float *y2, int64_t rows, int64_t width, float eps,
                                     const rowred_split_plan *plan, void *workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  if (!plan) return ROWRED_ERR_INVALID_ARG;
  return ws_entry(op, x, r, gamma, beta, y, y2, rows, width, eps, plan, workspace, workspace_bytes, stream);
}

ROWRED_API const char *rowred_status_string(int status) {
  switch (status) {
    case ROWRED_OK: return "ok";
    case ROWRED_ERR_INVALID_ARG: return "invalid argument (size, pointer, eps or plan)";
    case ROWRED_ERR_ALIAS: return "output overlaps an input";
    case ROWRED_ERR_UNSUPPORTED: return "size beyond the library's limits (width above ROWRED_MAX_WIDTH or launch grid too large)";
    case ROWRED_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

ROWRED_API int rowred_copy(const float *x, float *y, int64_t n, hipStream_t stream) {
  if (n < 0 || (n & 3)) return ROWRED_ERR_INVALID_ARG;
  if (n == 0) return ROWRED_OK;
  if (!x || !y || ((uintptr_t)x & 15) || ((uintptr_t)y & 15)) return ROWRED_ERR_INVALID_ARG;
  if (n > INT64_MAX / 4) return ROWRED_ERR_UNSUPPORTED;
  if (overlaps(x, y, n * 4)) return ROWRED_ERR_ALIAS;
  if ((n / 4 + 63) / 64 > INT32_MAX) return ROWRED_ERR_UNSUPPORTED;  // 64-lane workgroups, one slot per lane
  return launch_copy(x, y, n / 4, stream) == 0 ? ROWRED_OK : ROWRED_ERR_HIP;
}
