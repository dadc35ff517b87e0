// rowred_internal.h -- interface between the host entry points and the
// gfx950 kernels.  Not installed; not part of the C ABI.
#pragma once

#include <stdint.h>

#include "rowred.h"

namespace rowred {

// Kernel arguments, passed by value in the kernarg segment.
struct RowArgs {
  const float *x;      // rows x width input
  const float *r;      // residual (LayerNorm) or nullptr
  const float *gamma;  // LayerNorm scale per column or nullptr
  const float *beta;   // LayerNorm shift per column or nullptr
  float *y;            // rows x width output (row sum / row min: rows floats)
  float *y2;           // row max: rows floats
  int64_t rows;
  int32_t width;
  int32_t lanes_log2;  // log2(L)
  float eps;
  float inv_width;     // 1.0f / width, rounded to FP32
  int32_t policy;      // ROWRED_POLICY_* bits
  int32_t r_vec;       // 1: r shares x's address modulo 16 (16-byte loads)
  int32_t y_vec;       // 1: y shares x's address modulo 16 (16-byte stores)
  int32_t affine_vec;  // 1: rows start on 16-byte boundaries and gamma/beta are 16-byte aligned
  int32_t group_rows;  // flat kernels: rows per workgroup (P)
  int32_t affine_shift;  // 1: gamma / beta at another 16-byte phase than the rows (row kernels)
};

constexpr int kPolicyNtLoads = ROWRED_POLICY_NT_LOADS;
constexpr int kPolicyNtStores = ROWRED_POLICY_NT_STORES;
constexpr int kPolicyXcdRemap = ROWRED_POLICY_XCD_REMAP;
constexpr int kPolicyStageStores = ROWRED_POLICY_STAGE_STORES;
constexpr int kPolicyReload = ROWRED_POLICY_RELOAD;
constexpr int kPolicyLooped = ROWRED_POLICY_LOOPED;
constexpr int kPolicyLdsStripe = ROWRED_POLICY_LDS_STRIPE;
constexpr int kPolicyFlat = ROWRED_POLICY_FLAT;
constexpr int kPolicyOnline = ROWRED_POLICY_ONLINE;
constexpr int kPolicyCuGroups = ROWRED_POLICY_CU_GROUPS(15);  // the field's mask
constexpr int kPolicyAll = kPolicyNtLoads | kPolicyNtStores | kPolicyXcdRemap | kPolicyStageStores | kPolicyReload |
                           kPolicyLooped | kPolicyLdsStripe | kPolicyOnline | kPolicyCuGroups;
// LDS per compute unit (gfx950), and the LDS a register-kernel workgroup
// reserves so that at most n (1-14) share a CU: floor(160 KiB / n) rounded
// down to 1 KiB, less 256 bytes for the kernel's own partials -- (n + 1) such
// workgroups never fit.
constexpr size_t kLdsPerCu = 160 * 1024;
constexpr size_t cu_groups_lds_bytes(int n) { return (kLdsPerCu / n) / 1024 * 1024 - 256; }
// The per-phase reload variant exists for the three matrix operators (kernel
// ops 0-2) at up to 8 chunks.
constexpr int kMaxReloadChunks = 8;
constexpr bool reload_kernel_exists(int op, int chunks) { return op >= 0 && op <= 2 && chunks <= kMaxReloadChunks; }
// LayerNorm's reload kernels rebuild x + r as a pair in the last two phases;
// from 7 chunks on that needs the registers of a 512-thread workgroup.
constexpr int reload_max_threads_for(int op, int chunks) { return op == 0 && chunks >= 7 ? 512 : 1024; }
constexpr int kMaxStageThreads = 512;  // workgroup size the staged stores support
constexpr int kMaxStageChunks = 4;     // chunks per lane the staged stores are compiled for
// LDS for a staged workgroup: its rows span at most threads*chunks granules
// of the x window, plus the two partial granules at the run's ends.
constexpr size_t stage_lds_bytes(int chunks, int threads) { return ((size_t)threads * chunks + 2) * 16; }

// Kernel operator ids: the public operators (enum rowred_op) plus affine
// LayerNorm.
constexpr int kKernelOpLayerNormAffine = 5;
constexpr int kNumKernelOps = 6;

// Chunk counts for which kernels are instantiated (slots per lane).
constexpr int kChunkSet[] = {1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 16};
constexpr int kNumChunkSizes = sizeof(kChunkSet) / sizeof(kChunkSet[0]);
constexpr int kMaxWindow = 8192;  // 16-byte slots per row: 1024 lanes x 8 or 512 x 16

// Largest workgroup the kernel for (op, chunks) is compiled for: stripes of
// up to 8 slots fit the 128 VGPRs of a 1024-thread workgroup, except affine
// LayerNorm from 7 slots on, whose gamma/beta need the 256 VGPRs of 512.
constexpr int max_threads_for(int op, int chunks) {
  return chunks <= 8 && !(op == kKernelOpLayerNormAffine && chunks >= 7) ? 1024 : 512;
}
// Whether (op, chunks) is instantiated (affine LayerNorm stops at 12 slots:
// 16 would not fit its registers).
constexpr bool kernel_exists(int op, int chunks) { return !(op == kKernelOpLayerNormAffine && chunks > 12); }

// Enqueue one reduction kernel (op: a kernel operator id).  Returns the
// hipError_t of the launch (0 = success).  The caller has validated every
// argument.
int launch_rows(int op, int chunks, int64_t grid, int threads, const RowArgs &args,
                hipStream_t stream);

// Enqueue the looped kernel (rows wider than the register-resident window,
// ROWRED_POLICY_LOOPED): one workgroup of `threads` lanes per row, tiles of
// threads * chunks granules (chunks 2 or 4), grid = rows.
int launch_looped(int op, int chunks, int64_t rows, int threads, const RowArgs &args, hipStream_t stream);
// LayerNorm (plain, residual or affine) loops at 2 chunks only: its x and r
// tiles, two deep, need the registers.
constexpr bool looped_kernel_exists(int op, int chunks) {
  return chunks == 2 || (chunks == 4 && op != 0 && op != kKernelOpLayerNormAffine);
}

// Enqueue the LDS-stripe kernel (ROWRED_POLICY_LDS_STRIPE): RMSNorm (op 1)
// or softmax (op 2), one 1024-lane workgroup per row, chunks 5-16 (the first
// 4, from 9 chunks on 8, stay in registers).  grid = rows.
constexpr int kWideMinChunks = 5;
constexpr int kWideMaxChunks = 16;
constexpr int kWideMaxWindow = 1024 * kWideMaxChunks;
int launch_wide(int op, int chunks, int64_t rows, const RowArgs &args, hipStream_t stream);
// Rows wider than kWideMaxWindow (ROWRED_POLICY_LDS_STRIPE | ROWRED_POLICY_LOOPED,
// RMSNorm or softmax): the first kWideMaxWindow granules held as by the
// 16-chunk LDS-stripe kernel, the rest walked twice in tiles.  grid = rows.
int launch_wide_tail(int op, int64_t rows, const RowArgs &args, hipStream_t stream);
// LayerNorm's head in that kernel: x and r of 8 granules per lane (4 in
// registers, 4 in LDS).
constexpr int kLnTailHeadChunks = 8;

// Enqueue the flat kernel (ROWRED_POLICY_FLAT): RMSNorm (op 1) or softmax
// (op 2), rows of at least 4 elements, args.group_rows rows per workgroup of
// `threads` (64..512) lanes holding `chunks` (1, 2 or 4) granules each,
// args.lanes_log2 = log2 of the lanes that fold one row (<= 6).
constexpr int kFlatMaxThreads = 512;
constexpr size_t flat_lds_bytes(int chunks, int threads, int group_rows) {
  return (4 * (size_t)threads * chunks + 2 * ((size_t)group_rows + 1)) * 4;
}
int launch_flat(int op, int chunks, int64_t grid, int threads, const RowArgs &args, hipStream_t stream);

// Enqueue the streaming copy (n4 = number of 16-byte slots).
int launch_copy(const float *x, float *y, int64_t n4, hipStream_t stream);

// ---------------------------------------------------------------------------
// Split rows: a row's granule window is cut into segments of T*C granules,
// one workgroup of T threads per (row, segment).  A statistics kernel writes
// one record of two doubles per (row, segment) to the workspace; an apply
// kernel (matrix operators) merges its row's records in a fixed order,
// reads its segment again and writes it; a merge kernel (row sum, min/max)
// folds each row's records into the outputs.
// ---------------------------------------------------------------------------
struct SegArgs {
  const float *x;
  const float *r;
  const float *gamma;
  const float *beta;
  float *y;
  float *y2;
  double *ws;          // rows * segments records of two doubles, 16-byte aligned
  int64_t rows;
  int32_t width;
  int32_t segments;    // S
  int32_t lanes_log2;  // log2(T): all threads of a workgroup serve one segment
  int32_t seg_granules;  // G = T * C granules per segment
  float eps;
  float inv_width;
  int32_t policy;      // ROWRED_POLICY_NT_LOADS / NT_STORES (apply kernel), ROWRED_POLICY_REVERSE
  int32_t r_vec;
  int32_t y_vec;
  uint32_t spin_limit;  // exchange kernels: polls of one slot before a wait gives up
  int32_t ws_in_y;      // exchange kernels: 1 = the words live in each row of y (no workspace)
};

// Exchange words kept in y's own row (plain entry points, no workspace): from
// the row's first 16-byte boundary, `rounds * S` slots then one count of the
// segments done reading them; the last of them must end inside segment 0's
// outputs, which that segment writes last.
constexpr int64_t row_exchange_bytes(int rounds, int64_t segments) { return 15 + 8 * (rounds * segments + 1); }

// Polls of one exchange slot before the wait gives up (a second or so: each
// poll is a load that goes past the XCD's L2, then s_sleep 2).  An explicit
// split plan may set a smaller bound (rowred_split_plan.wait_polls), for
// tests of the give-up path.
constexpr uint32_t kExchangeSpinLimit = 1u << 20;

// Chunk counts (16-byte slots per lane) of the split kernels.
constexpr int kSplitChunkSet[] = {1, 2, 4};
constexpr int kNumSplitChunks = 3;
constexpr int kPolicyReverse = ROWRED_POLICY_REVERSE;
constexpr int kPolicyExchange = ROWRED_POLICY_EXCHANGE;
constexpr int kSplitPolicyAll =
    kPolicyNtLoads | kPolicyNtStores | kPolicyReverse | kPolicyExchange | ROWRED_POLICY_LDS_STRIPE;
// The segments of a row wait for each other in the exchange kernel, so all
// of a row's segments must fit on the chip at once.  Every CU holds at least
// one workgroup of any allowed size (launch bounds keep 1024-thread kernels
// within 128 VGPRs): 32 per XCD, 256 in all.  Dealt round robin over the 8
// XCDs, a row of at most 128 segments needs 16 per XCD.  Lane k reads
// segment k's slot, so S is also at most the workgroup's threads.
constexpr int kMaxExchangeSegments = 128;
// Exchange kernels: 1, 2, 4 or 8 slots per lane; 8 slots in workgroups of at
// most 512 threads (their registers), and not for LayerNorm, whose x, r and
// x + r pair at 8 slots outgrow the register file.
constexpr int kNumExchangeChunks = 4;
constexpr int exchange_max_threads(int chunks) { return chunks >= 8 ? 512 : 1024; }
constexpr bool exchange_kernel_exists(int op, int chunks) { return chunks != 8 || op != 0; }
// Exchange kernels with part of the segment in LDS (ROWRED_POLICY_LDS_STRIPE
// on a split plan): 256 threads; chunks 8 (4 in registers + 4 in LDS), 12
// (8 + 4) or 16 (8 + 8), for x and, LayerNorm, r alike.  -1: no such kernel.
constexpr int kXldsThreads = 256;
constexpr int kNumXldsStripes = 3;
constexpr int xlds_stripe_index(int op, int chunks) {
  return chunks == 8 ? 0 : chunks == 12 ? 1 : chunks == 16 ? 2 : -1;
}

// Enqueue the statistics kernel (op: LayerNorm 0, RMSNorm 1, softmax 2, row
// sum 3, row min/max 4) and then the apply (ops 0-2) or merge (ops 3-4)
// kernel.  grid = rows * segments.  Returns the first launch's hipError_t.
int launch_split(int op, int chunks, int64_t grid, int threads, const SegArgs &args, hipStream_t stream);

// One-kernel split rows (ROWRED_POLICY_EXCHANGE, ops 0-2): a clear kernel
// zeroes exchange_words() 64-bit words of the workspace, then one workgroup
// per (row, segment) keeps its segment in registers and swaps statistics
// with its row's other segments through those words.
// clear_status: also zero the status word (the first launch of a call; a
// call that runs in row blocks clears only the slots for the later blocks,
// so a give-up in an earlier block stays visible).
int64_t exchange_words(int op, int64_t rows, int64_t segments);
int launch_exchange(int op, int chunks, int64_t grid, int threads, const SegArgs &args, bool clear_status,
                    hipStream_t stream);
// Workgroups of the exchange kernel for (op, chunks, threads, policy) that
// the current device holds at once: its compute units times the kernel's
// occupancy per compute unit (cached per device and kernel).  0 on any HIP
// error.  A row's S segments wait for each other, so S must stay well below
// this.
int64_t exchange_resident_groups(int op, int chunks, int threads, int policy);

// The library's static workspace on the current device (rowred_static_ws):
// ROWRED_STATIC_WORKSPACE_BYTES, 256-byte aligned.  The first call on a
// device looks up that device's copy of the array; later calls reuse the
// address.  Returns the hipError_t of the lookup (0 = success).
int static_workspace(void **ptr);

}  // namespace rowred
