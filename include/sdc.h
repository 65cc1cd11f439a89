/*
 * sdc.h -- C ABI of libsdc.so, the MI355X (gfx950) integrity scan for
 * silent-data-corruption checks in data-parallel training.
 *
 * What the library computes comes from these pages:
 *   [BLOG] AWS Machine Learning Blog, "Detecting and recovering from silent
 *          data corruption on Amazon SageMaker HyperPod":
 *          "Compare by fingerprint"           -- the two 64-bit sums per tensor;
 *          "Check 1: NaN/Inf gradients, ..."   -- NaN/Inf detection;
 *          "Check 2: Ring replay, ..."         -- exact comparison of a replay
 *                                                 with the original;
 *          "Check 3: Weight fingerprints, ..." -- strict-majority comparison
 *                                                 of the replicas' tables.
 *   [AEGIS] review page of "Safeguarding LLM Training at Scale: Online SDC
 *          Detection and Insights from 35 Million GPU Hours", section "core
 *          method" (核心方法) item 4 -- the xorsum fingerprint, and the
 *          bitwise comparison of a result with its deterministic
 *          recomputation.
 *
 * Conventions shared by every entry point
 *   - Every function returns an int32_t status (SDC_OK or a negative SDC_ERR_*).
 *     No C++ exception or abort crosses the ABI.
 *   - "d_" arguments are device pointers (HIP device memory of the current
 *     device), "h_" arguments are host pointers.  The caller owns and allocates
 *     all device memory; the library allocates none.  Between calls it keeps
 *     only per-host-thread state (the last HIP error and a small host staging
 *     buffer of the compare calls' single device-to-host copy), per-device
 *     facts (the compute-unit count), and one static 256 KiB device array per
 *     GPU that only sdc_fingerprint_tensor_noalloc uses.
 *   - "stream" is a hipStream_t passed as void* (NULL = the null stream).
 *     Functions documented as asynchronous only enqueue work on that stream;
 *     their device outputs are valid once the stream reaches that point.
 *   - The fingerprints are arithmetic on unsigned 64-bit integers modulo 2^64
 *     over raw bit patterns (floating-point data are never converted), so
 *     every row is exact and independent of launch shape and scheduling.  The
 *     one floating-point result, sdc_sqnorm's squared norms, is summed in an
 *     order fixed by the plan.
 *   - Functions are thread-safe.  Two scans that write the same output rows
 *     must not run concurrently.
 *   - Launch shapes: scans of large items (list scans whose items average at
 *     least 512 KiB, single-tensor scans of at least 128 MiB) run one
 *     256-lane workgroup per CU; their launches reserve 96 KiB of dynamic LDS
 *     per workgroup (untouched) to hold the CU to one, so work on other
 *     streams shares those CUs only as far as LDS allows.  Results do not
 *     depend on the shape.
 */
#ifndef SDC_H
#define SDC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SDC_ABI_VERSION 2u

typedef void* sdc_stream_t; /* a hipStream_t */

/* Status codes. */
enum {
  SDC_OK = 0,
  SDC_ERR_INVALID = -1,   /* NULL where data is required, zero R/T, bad column mask, ... */
  SDC_ERR_DTYPE = -2,     /* unknown element type                                        */
  SDC_ERR_ALIGN = -3,     /* tensor pointer not aligned to its element size              */
  SDC_ERR_WORKSPACE = -4, /* plan / workspace buffer smaller than required               */
  SDC_ERR_HIP = -5,       /* a HIP runtime call failed; see sdc_last_hip_error()         */
  SDC_ERR_PLAN = -6,      /* plan buffer and plan info do not belong together            */
  SDC_ERR_RANGE = -7      /* a size exceeds what the library supports                   */
};

/* Element types.  Only the element width (1, 2, 4 or 8 bytes) and the
 * NaN/Inf encoding (for the nonfinite count) depend on the type; values are
 * never converted.  NaN/Inf: IEEE formats (F32, BF16, F16, F64, FP8_E5M2):
 * exponent field all ones; FP8_E4M3 (OCP "fn", no Inf): S.1111.111; the
 * "fnuz" fp8 formats (no Inf): 0x80; U* raw integers (also int8/bool, int16,
 * int32, int64 tensors): never. */
enum {
  SDC_F32 = 0, SDC_BF16 = 1, SDC_F16 = 2, SDC_F64 = 3, SDC_U8 = 4, SDC_FP8_E4M3 = 5,
  SDC_FP8_E5M2 = 6, SDC_FP8_E4M3FNUZ = 7, SDC_FP8_E5M2FNUZ = 8, SDC_U16 = 9, SDC_U32 = 10,
  SDC_U64 = 11
};

/* sdc_tensor.flags: SDC_FLAG_SIGNED widens 2- and 4-byte patterns with sign
 * extension before summing, which reproduces [BLOG]'s own fingerprint
 * function exactly (it views 1/2/4/8-byte elements as uint8/int16/int32/int64
 * and widens to int64); 1- and 8-byte elements are unaffected.  xorsum is then
 * the xor of the widened values.  Without the flag every pattern is
 * zero-extended. */
enum { SDC_FLAG_SIGNED = 1u };

/* Column mask bits for comparisons.  [BLOG] "Check 3" compares (sum, wsum);
 * SDC_COL_SUM | SDC_COL_WSUM reproduces exactly that comparison. */
enum {
  SDC_COL_SUM = 1u, SDC_COL_WSUM = 2u, SDC_COL_XOR = 4u, SDC_COL_NONFINITE = 8u,
  SDC_COL_ALL = 15u
};

/* One tensor of the list to scan.
 *   ptr    device pointer to numel contiguous elements (row-major, little-
 *          endian), aligned to the element size; NULL means a missing tensor
 *          (its row is all zero, [BLOG] "Compare by fingerprint").
 *   numel  number of elements (0 gives a zero row); numel * element size below 2^62.
 *   dtype  one of the SDC_* element types above.
 *   flags  0 or SDC_FLAG_SIGNED. */
typedef struct {
  const void* ptr;
  uint64_t numel;
  uint32_t dtype;
  uint32_t flags;
} sdc_tensor;

/* Fingerprint row of one tensor, x_i = raw bit pattern of element i widened
 * to 64 bits (zero-extended; sign-extended for 2-/4-byte elements under
 * SDC_FLAG_SIGNED), i = 0 .. numel-1:
 *   sum       = sum_i x_i                 mod 2^64   [BLOG] plain sum
 *   wsum      = sum_i (i+1) * x_i         mod 2^64   [BLOG] position-weighted sum
 *   xorsum    = xor_i x_i                            [AEGIS] xorsum
 *   nonfinite = #{i : element i is NaN or +-Inf in its type's encoding} */
typedef struct {
  uint64_t sum;
  uint64_t wsum;
  uint64_t xorsum;
  uint64_t nonfinite;
} sdc_row;

/* Host-side summary of a plan, filled by sdc_plan_build and passed back to
 * the scan calls (it carries the launch size, so no device read is needed). */
typedef struct {
  uint64_t magic;        /* identifies a plan built by sdc_plan_build            */
  uint64_t n_tensors;    /* number of descriptors = number of output rows        */
  uint64_t n_items;      /* work items (workgroup items + wave items)            */
  uint64_t n_small;      /* of which wave items: small tensors scanned whole by
                            a group of lanes of one wave                        */
  uint64_t n_split;      /* rows merged from several items (or missing/empty)    */
  uint64_t n_slots;      /* partial-row slots in the plan's scratch area         */
  uint64_t total_elems;  /* elements scanned per pass                            */
  uint64_t total_bytes;  /* bytes scanned per pass (the algorithmic traffic)     */
  uint64_t plan_bytes;   /* bytes of the device plan                             */
  uint64_t item_bytes;   /* bytes per work item (the chunk size used)            */
  uint64_t n_wave[4];    /* wave items by class: scanned by 64, 32, 16, 8 lanes   */
} sdc_plan_info;

/* Result of sdc_majority_compare ([BLOG] "Check 3"). */
typedef struct {
  int32_t diverged;            /* 1 if some tensor's replica rows are not all equal      */
  int32_t has_majority;        /* 0 if some differing tensor has no strict majority:
                                  then no replica is named (h_suspect is all zero)       */
  uint64_t n_diff;             /* number of differing tensors                            */
  uint64_t first_diff;         /* smallest differing tensor index, UINT64_MAX if none    */
  uint64_t first_no_majority;  /* smallest tensor without a strict majority, or UINT64_MAX */
} sdc_majority;

/* Single-bit-flip localisation of a differing row pair (see sdc_fingerprint_diff). */
typedef struct {
  uint64_t index; /* element index of the flipped bit, UINT64_MAX if the change is
                     not one bit flip */
  int32_t bit;    /* flipped bit (0 = least significant), -1 if none          */
  int32_t dir;    /* +1: bit is 0 in a and 1 in b; -1: 1 in a, 0 in b; 0: none */
} sdc_flip_hint;

/* ---- plans: a fixed tensor list scanned many times ------------------------
 * [BLOG] "Compare by fingerprint" fingerprints a tensor list by looping over
 * the tensors and, within each, over fixed-size chunks, adding each chunk's
 * sums into the tensor's row.  A plan is that loop laid out once on the host:
 * every tensor cut into work items (chunks of at most 4 MiB, each a
 * contiguous element range of one tensor), which the scan kernels process in
 * parallel; the chunks' sums combine exactly as in that loop (concatenation
 * identity W(A||B) = W(A) + W(B) + |A| S(B)).  Parameter pointers do not
 * change between training steps, so one plan serves every check. */

/* Device bytes needed for the plan of h_tensors[0..n) ([BLOG] "Compare by
 * fingerprint": the per-tensor chunk loop).  item_bytes is the work
 * item size in bytes (a multiple of 16, at most 4 MiB); 0 selects it
 * automatically: the largest power of two from 1 MiB down to 64 KiB that
 * still splits the list into at least 49152 items (else 64 KiB).  The rows do
 * not depend on it.  Host-only: no HIP call. */
int32_t sdc_plan_bytes(const sdc_tensor* h_tensors, uint64_t n, uint64_t item_bytes,
                       uint64_t* h_bytes);

/* [BLOG] "Compare by fingerprint" (the per-tensor chunk loop, laid out once):
 * packs the descriptors of h_tensors[0..n) into a work list and copies it into
 * d_plan (plan_bytes bytes of device memory owned by the caller).  The plan
 * also holds the scratch partial rows of tensors split over several work
 * items, so scans that use the same plan must not overlap in time.
 * SYNCHRONOUS: returns after the copy, ordered on stream, has completed.
 * h_info receives the host summary needed by the scan calls.  The plan stores
 * the tensors' device pointers: they must stay valid while the plan is used.
 * Errors: SDC_ERR_INVALID, SDC_ERR_DTYPE, SDC_ERR_ALIGN, SDC_ERR_RANGE,
 * SDC_ERR_WORKSPACE (plan_bytes too small), SDC_ERR_HIP. */
int32_t sdc_plan_build(const sdc_tensor* h_tensors, uint64_t n, uint64_t item_bytes,
                       void* d_plan, uint64_t plan_bytes, sdc_plan_info* h_info,
                       sdc_stream_t stream);

/* [BLOG] "Compare by fingerprint" (the per-tensor chunk loop, laid out once).
 * Host-only form of sdc_plan_build for inspection and testing: writes the
 * plan's descriptor part (everything but the scratch partial rows, i.e. the
 * first plan_bytes bytes it needs, at most sdc_plan_bytes) to host memory
 * h_plan and fills h_info.  No HIP call.  Layout of the image: a 64-byte
 * header {magic, n_tensors, n_items, n_split, n_slots, total_bytes,
 * item_bytes, n_small} (uint64 each); n_items 32-byte work items {addr u64,
 * start u64, len u32, row u32, slot u32, dtype | 0x100 if whole-tensor u32},
 * workgroup items first, then the n_small wave items (the n_wave[0..3] items
 * of each class in turn, each class ordered by element type); then n_split
 * 16-byte entries {row, first slot, slot count, 0} (uint32 each). */
int32_t sdc_plan_pack_host(const sdc_tensor* h_tensors, uint64_t n, uint64_t item_bytes,
                           void* h_plan, uint64_t plan_bytes, sdc_plan_info* h_info);

/* [BLOG] "Compare by fingerprint", [AEGIS] xorsum: writes d_out[k] = row of
 * tensor k for k < n_tensors (d_out: n_tensors * 32 bytes of device memory;
 * every row is written, previous contents do not matter).
 * ASYNCHRONOUS on stream: one launch for the wave items, one for the
 * workgroup items, then one merge launch for the rows of split (and
 * missing/empty) tensors.  Errors: SDC_ERR_INVALID,
 * SDC_ERR_PLAN, SDC_ERR_HIP. */
int32_t sdc_fingerprint_plan(const void* d_plan, const sdc_plan_info* h_info, sdc_row* d_out,
                             sdc_stream_t stream);

/* [BLOG] "Check 1": element-exact NaN/Inf count.  d_counts[k] (uint64 per
 * tensor, may be NULL) and *d_total receive the counts.  ASYNCHRONOUS.
 * Errors as sdc_fingerprint_plan. */
int32_t sdc_nonfinite(const void* d_plan, const sdc_plan_info* h_info, uint64_t* d_counts,
                      uint64_t* d_total, sdc_stream_t stream);

/* [BLOG] "Check 1", the norm-based form: d_sq[k] = sum of the squared values
 * of tensor k's elements (n_tensors doubles), *d_total = their sum, and
 * *d_flag (may be NULL) = 1 when *d_total rounded to fp32 is not finite --
 * exactly when an fp32 norm of these tensors would be NaN or Inf: any NaN or
 * Inf element, or a finite norm above ~1.8e19.  Values are decoded exactly
 * from each floating-point type (raw integer types contribute 0) and summed
 * in double in an order fixed by the plan, so results are bit-reproducible
 * for a given plan (a different item size may change the last bits).
 * ASYNCHRONOUS.  Uses the plan's scratch area, like a scan.  Errors as
 * sdc_fingerprint_plan. */
int32_t sdc_sqnorm(const void* d_plan, const sdc_plan_info* h_info, double* d_sq,
                   double* d_total, uint32_t* d_flag, sdc_stream_t stream);

/* [BLOG] "Compare by fingerprint": device workspace bytes of sdc_fingerprint
 * on this list (the plan's size with the automatic item size:
 * sdc_plan_bytes(h_tensors, n, 0)).  Host only;
 * errors as sdc_plan_bytes. */
int32_t sdc_fingerprint_ws_bytes(const sdc_tensor* h_tensors, uint64_t n, uint64_t* h_bytes);

/* [BLOG] "Compare by fingerprint" (rows of a tensor list), [AEGIS] xorsum, and
 * [BLOG] "Check 1" (the NaN/Inf count): one-shot form of sdc_plan_build +
 * sdc_fingerprint_plan; the rows are those of sdc_fingerprint_plan.  d_ws is a device
 * workspace of at least sdc_fingerprint_ws_bytes(h_tensors, n) bytes that
 * holds the plan.  The plan upload is synchronous; the scan is asynchronous
 * on stream.  The workspace must not be reused before the scan has completed. */
int32_t sdc_fingerprint(const sdc_tensor* h_tensors, uint64_t n, void* d_ws, uint64_t ws_bytes,
                        sdc_row* d_out, sdc_stream_t stream);

/* ---- one tensor, no plan ------------------------------------------------- */

/* [AEGIS] "core method" item 4 (the recompute check's scan): device
 * workspace bytes for sdc_fingerprint_tensor on *h_tensor with the same
 * item_bytes: 32 bytes per work item, at least 32.  With the automatic item
 * size the split of tensors of 128 MiB and more depends on the device's
 * compute-unit count; the size returned then holds on every gfx950 device
 * (at most 8 KiB more than one device needs).  Host only (no HIP call).
 * Errors as sdc_fingerprint_tensor's argument checks. */
int32_t sdc_tensor_ws_bytes(const sdc_tensor* h_tensor, uint64_t item_bytes, uint64_t* h_bytes);

/* Host-only view of the split sdc_fingerprint_tensor makes of *h_tensor on a
 * device with cu_count compute units (for inspection and testing; no HIP
 * call): *h_n_items work items of *h_item_bytes bytes each (the first may
 * also hold a misaligned head, the last may be shorter).  With item_bytes 0
 * (automatic), tensors of at least 128 MiB take a multiple of
 * min(cu_count, 256) items of at most 4 MiB (one per CU per pass); smaller
 * ones about 1024 items of 64 KiB to 1 MiB.  Errors: SDC_ERR_INVALID
 * (NULL outputs, cu_count 0), else as sdc_fingerprint_tensor's checks. */
int32_t sdc_tensor_split_host(const sdc_tensor* h_tensor, uint64_t item_bytes, uint32_t cu_count,
                              uint64_t* h_n_items, uint64_t* h_item_bytes);

/* [AEGIS] "core method" item 4: fingerprints of an original result and of its
 * deterministic recomputation, compared bit for bit; any difference is a
 * confirmed fault.  Scans ONE tensor without a plan (its work items follow
 * from its size; the split, and so the row, is that of the list scan) and
 * writes its row to d_out[0].  With d_ref != NULL (device, one row, e.g. the
 * row stored when the original was computed) the row is compared with
 * *d_ref under col_mask (SDC_COL_*), and a difference adds 1 to the device
 * counter *d_mismatch (required then; the caller clears it).
 *   h_tensor   host descriptor; ptr is a device pointer (NULL or numel 0: the
 *              zero row), aligned to the element size; flags: SDC_FLAG_SIGNED.
 *   item_bytes bytes per work item, a multiple of 16 up to 4 MiB; 0 = automatic
 *              (about 1024 items, 64 KiB to 1 MiB).  The row does not depend on it.
 *   d_ws       device workspace of at least sdc_tensor_ws_bytes bytes, not
 *              reused by the caller before the call's work has completed.
 * ASYNCHRONOUS on stream, with no host synchronisation and no host-to-device
 * copy, so it can run inside a backward pass.  Errors: SDC_ERR_INVALID (NULL
 * d_out / d_ws, d_ref without d_mismatch, bad mask or flags), SDC_ERR_DTYPE,
 * SDC_ERR_ALIGN, SDC_ERR_RANGE, SDC_ERR_WORKSPACE, SDC_ERR_HIP. */
int32_t sdc_fingerprint_tensor(const sdc_tensor* h_tensor, uint64_t item_bytes, void* d_ws,
                               uint64_t ws_bytes, const sdc_row* d_ref, uint32_t col_mask,
                               sdc_row* d_out, uint32_t* d_mismatch, sdc_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the scan of
 * sdc_fingerprint_tensor -- same arguments, same row, same compare -- without
 * a workspace.  The partial rows of the tensor's work items go to a static
 * device array of 8192 rows (256 KiB) that the library holds on every GPU it
 * runs on until the process ends; no device memory is allocated by the call.
 * Limit: the tensor's split must fit the array on every device -- at most
 * 8192 work items for an explicit item_bytes; with the automatic split
 * (item_bytes 0), tensors of up to 7935 * 4 MiB (about 31 GiB).  Larger ones
 * give SDC_ERR_RANGE before anything is queued.  All calls on one GPU share
 * the array: calls that overlap in time on one GPU (on different streams or
 * from different host threads) race and give wrong rows; calls in order on
 * one stream are safe (each call's items write their slots before its merge
 * reads them, so the array needs no clearing).  The first call on each device
 * looks up the array's device address (hipGetSymbolAddress, a runtime call
 * that is not stream work): a caller that captures graphs makes one call on
 * each device before capturing -- one on an empty tensor (numel 0, which
 * writes the zero row) is enough.  ASYNCHRONOUS on stream, like
 * sdc_fingerprint_tensor.  Errors as sdc_fingerprint_tensor, with
 * SDC_ERR_RANGE for a tensor beyond the limit or a current device index of 64
 * or more (the library keeps the array's address for devices 0..63). */
int32_t sdc_fingerprint_tensor_noalloc(const sdc_tensor* h_tensor, uint64_t item_bytes,
                                       const sdc_row* d_ref, uint32_t col_mask, sdc_row* d_out,
                                       uint32_t* d_mismatch, sdc_stream_t stream);

/* ---- comparisons of fingerprint tables ------------------------------------ */

/* Device workspace bytes for sdc_majority_compare with R replicas, T tensors. */
int32_t sdc_majority_ws_bytes(uint32_t R, uint64_t T, uint64_t* h_bytes);

/* [BLOG] "Check 3": strict-majority comparison of R replicas' tables.
 *   d_table  R*T rows, replica-major: row of replica r, tensor k at r*T + k
 *            (the layout a scan over the replicas' concatenated lists gives).
 *   col_mask columns compared (SDC_COL_*; nonzero, no other bits).
 * For each tensor whose R rows are not all equal: if one row value is held by
 * more than R/2 replicas, every replica whose row differs from it is named;
 * otherwise the tensor has no majority, and then no replica is named at all.
 *   h_res      receives the summary; h_suspect[R] receives 1 for a named
 *              replica, else 0.
 *   d_tensor_status  optional (NULL allowed), T bytes of device memory:
 *              0 = all equal, 1 = differs with a strict majority, 2 = no majority.
 *   d_ws       sdc_majority_ws_bytes(R, T) bytes of device workspace.
 * SYNCHRONOUS (waits for stream).  R == 1 never diverges.
 * Errors: SDC_ERR_INVALID (R == 0, T == 0, NULL, bad mask), SDC_ERR_WORKSPACE,
 * SDC_ERR_RANGE (R * T too large, or the R-byte host staging buffer could not
 * be allocated; nothing is queued then), SDC_ERR_HIP. */
int32_t sdc_majority_compare(const sdc_row* d_table, uint32_t R, uint64_t T, uint32_t col_mask,
                             void* d_ws, uint64_t ws_bytes, sdc_majority* h_res,
                             uint8_t* h_suspect, uint8_t* d_tensor_status, sdc_stream_t stream);

/* Device workspace bytes for sdc_fingerprint_diff over T rows reporting up to
 * idx_cap indices (an idx_cap above T counts as T: at most T rows differ). */
int32_t sdc_diff_ws_bytes(uint64_t T, uint64_t idx_cap, uint64_t* h_bytes);

/* [BLOG] "Check 2" (replay vs original) and the check after a restore:
 * indices k < T with d_a[k] != d_b[k] under col_mask.
 *   h_n_diff  receives the exact number of differing rows.
 *   h_idx     receives the first min(n_diff, idx_cap) of them, ascending.
 *   h_hints   (NULL allowed) receives, for each reported index, the single-bit-
 *             flip localisation: when X_a ^ X_b = 2^b, S_b - S_a = s * 2^b and
 *             W_b - W_a = s * (i+1) * 2^b with one sign s = +-1 and
 *             (i+1) * 2^b < 2^63, the change is one flip of bit b of element i.
 * SYNCHRONOUS.  Errors: SDC_ERR_INVALID, SDC_ERR_WORKSPACE, SDC_ERR_RANGE (T or
 * idx_cap >= 2^58, or the host staging of min(idx_cap, T) records could not be
 * allocated; nothing is queued then), SDC_ERR_HIP. */
int32_t sdc_fingerprint_diff(const sdc_row* d_a, const sdc_row* d_b, uint64_t T, uint32_t col_mask,
                             void* d_ws, uint64_t ws_bytes, uint64_t* h_n_diff, uint64_t* h_idx,
                             uint64_t idx_cap, sdc_flip_hint* h_hints, sdc_stream_t stream);

/* ---- ring replay audit ([BLOG] "Check 2: Ring replay, before the optimizer
 * step") --------------------------------------------------------------------
 * Every rank r replays the work of rank (r + offset) mod n.  The gathered table
 * holds, per rank, two results of `width` uint64 words each (for example the
 * loss bits followed by the gradient fingerprint rows): [r][0] = r's own
 * result, [r][1] = r's replay of its target.  Layout: rank-major,
 * d_table[(r*2 + j)*width + w]. */

/* Device workspace bytes for sdc_ring_compare (n ranks) and sdc_confirm_verdict. */
int32_t sdc_ring_ws_bytes(uint32_t n, uint64_t* h_bytes);

/* h_mismatch[r] = 1 when pair r, (target (r+offset) mod n, replayer r),
 * mismatches: the target's own result differs from r's replay in any word.
 * SYNCHRONOUS.  Errors: SDC_ERR_INVALID (n == 0, NULL), SDC_ERR_WORKSPACE,
 * SDC_ERR_RANGE, SDC_ERR_HIP. */
int32_t sdc_ring_compare(const uint64_t* d_table, uint32_t n, uint64_t width, uint32_t offset,
                         void* d_ws, uint64_t ws_bytes, uint8_t* h_mismatch, sdc_stream_t stream);

/* Host-only (no HIP call).  h_culprit[q] = 1 for every rank q that appears,
 * as target or replayer, in at least two mismatched pairs; h_ambiguous[r] = 1
 * for every mismatched pair r that contains no culprit (it needs
 * confirmation).  Errors: SDC_ERR_INVALID, SDC_ERR_RANGE (the n-entry host
 * work array could not be allocated). */
int32_t sdc_ring_localize(const uint8_t* h_mismatch, uint32_t n, uint32_t offset,
                          uint8_t* h_culprit, uint8_t* h_ambiguous);

/* Confirmation of an ambiguous pair ("Check 2", the case where only one of
 * a rank's two comparisons mismatches): a witness GPU on a third node and the
 * target itself replay the target's work once more.  d_witness, d_retry:
 * those two replays; d_original: the target's first own result; d_replay:
 * the replayer's replay of it; all `width` words of device memory.  Verdict,
 * per the verdict rows of [BLOG] "Decide what the alarm means": the replayer
 * computed wrong if the witness reproduces the original; otherwise, if the
 * witness sides with the replayer, the target was wrong -- persistent when
 * its retry reproduced its original, transient when its retry agrees with the
 * witness, else unclear; if the witness agrees with neither, unattributable.
 * d_ws: sdc_ring_ws_bytes(1) bytes.  SYNCHRONOUS. */
enum {
  SDC_VERDICT_REPLAYER_WRONG = 1, /* suspect: the replayer */
  SDC_VERDICT_PERSISTENT = 2,     /* suspect: the target   */
  SDC_VERDICT_TRANSIENT = 3,      /* suspect: the target   */
  SDC_VERDICT_UNCLEAR = 4,        /* suspect: the target   */
  SDC_VERDICT_UNATTRIBUTABLE = 5  /* no suspect            */
};
int32_t sdc_confirm_verdict(const uint64_t* d_witness, const uint64_t* d_retry,
                            const uint64_t* d_original, const uint64_t* d_replay, uint64_t width,
                            void* d_ws, uint64_t ws_bytes, int32_t* h_verdict,
                            sdc_stream_t stream);

/* ---- measurement ----------------------------------------------------------- */

/* Streaming-read reference (no passage of the pages defines it: it measures
 * the bandwidth the fingerprint scan is read against).  *d_sum = the sum
 * (mod 2^64) of the bytes/4 little-endian 32-bit words at d_buf, each
 * zero-extended -- for an fp32 buffer, the same value as the sum column of its
 * fingerprint.  The words are read with the scan's load structure (one
 * workgroup per 1 MiB, non-temporal 16-byte loads, a partial sum per
 * workgroup merged by a second one-workgroup launch) and one add per word, so
 * the call's rate is the chip's streaming-read rate for that structure.
 * d_buf: device memory, 16-byte aligned; bytes: a multiple of 4 (0 gives 0);
 * d_ws: sdc_read_sum_ws_bytes(bytes) bytes of device memory, 8-byte aligned,
 * caller-owned (no initial contents needed); d_sum: one device uint64_t.
 * ASYNCHRONOUS on `stream`; calls that share d_ws must not overlap.
 * Errors: SDC_ERR_INVALID (NULL, bytes % 4 != 0), SDC_ERR_ALIGN,
 * SDC_ERR_WORKSPACE, SDC_ERR_RANGE, SDC_ERR_HIP. */
int32_t sdc_read_sum_ws_bytes(uint64_t bytes, uint64_t* h_ws_bytes);
int32_t sdc_read_sum(const void* d_buf, uint64_t bytes, void* d_ws, uint64_t ws_bytes,
                     uint64_t* d_sum, sdc_stream_t stream);

/* ---- misc ------------------------------------------------------------------ */

/* Static text for a status code (not from the pages). */
const char* sdc_status_string(int32_t status);

/* The hipError_t of the last failed HIP call on this thread (0 if none; not
 * from the pages). */
int32_t sdc_last_hip_error(void);

/* SDC_ABI_VERSION of the library (not from the pages). */
uint32_t sdc_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif
