/*
 * sdc_oracle.h -- reference (oracle) implementation of the integrity scan.
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists so that tests, the smoke
 * check and the benchmark's CPU baseline can check the HIP path against a
 * plain, slow, obviously correct CPU computation.  It shares no code, header,
 * table or constant with the HIP library, and no product code path may call it.
 *
 * Everything here is single-threaded scalar C over uint64_t, taken directly
 * from the definitions on the pages:
 *
 *   "Detecting and recovering from silent data corruption on Amazon SageMaker
 *    HyperPod" (AWS Machine Learning Blog):
 *     - section "Compare by fingerprint": two 64-bit sums of the raw bit
 *       patterns per tensor, one plain and one weighted by 1-based position;
 *       a missing (None) tensor keeps a zero row.
 *     - section "Check 3: Weight fingerprints, after the optimizer step":
 *       a replica is named only when its copy differs from a strict majority.
 *     - section "Check 2: Ring replay, before the optimizer step": a replay's
 *       result is compared for exact equality with the original's.
 *     - section "Check 1: NaN/Inf gradients, ...": NaN/Inf detection.
 *   Review page of "Safeguarding LLM Training at Scale: Online SDC Detection
 *    and Insights from 35 Million GPU Hours" (AEGIS), section "core method"
 *    (核心方法), item 4: an xorsum fingerprint of an original result and of
 *    its deterministic recomputation.
 *
 * All functions return 0 on success and a negative ORACLE_E* code on bad
 * arguments.  All pointers are host pointers.
 */
#ifndef SDC_ORACLE_H
#define SDC_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  Only the element width and the NaN/Inf encoding matter;
 * values are never interpreted as numbers.  The U* types are raw integers
 * (never NaN/Inf). */
enum {
  ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F16 = 2, ORACLE_F64 = 3, ORACLE_U8 = 4,
  ORACLE_FP8_E4M3 = 5, ORACLE_FP8_E5M2 = 6, ORACLE_FP8_E4M3FNUZ = 7, ORACLE_FP8_E5M2FNUZ = 8,
  ORACLE_U16 = 9, ORACLE_U32 = 10, ORACLE_U64 = 11
};

/* Per-tensor flag: widen 2- and 4-byte patterns to 64 bits with sign
 * extension, as the pages' code does by viewing such elements as int16 and
 * int32 ("Compare by fingerprint"); 1-byte elements stay unsigned there
 * (a uint8 view) and 8-byte ones need no widening, so the flag does not
 * change them.  X is then the xor of the widened values. */
enum { ORACLE_SIGNED = 1 };

enum {
  ORACLE_OK = 0,
  ORACLE_EINVAL = -1,  /* NULL where data is required, zero column mask, R or T zero */
  ORACLE_EDTYPE = -2   /* unknown element type */
};

/* Column mask bits (which columns of a row take part in a comparison). */
enum {
  ORACLE_COL_SUM = 1u, ORACLE_COL_WSUM = 2u, ORACLE_COL_XOR = 4u, ORACLE_COL_NONFINITE = 8u,
  ORACLE_COL_ALL = 15u
};

/* One fingerprint row per tensor. */
typedef struct {
  uint64_t sum;       /* S = sum_i x_i                 (mod 2^64) */
  uint64_t wsum;      /* W = sum_i (i+1) * x_i         (mod 2^64) */
  uint64_t xorsum;    /* X = xor_i x_i                             */
  uint64_t nonfinite; /* NF = #{i : exponent field of x_i all ones} */
} oracle_row;

typedef struct {
  int32_t diverged;            /* some tensor's rows are not all equal        */
  int32_t has_majority;        /* every differing tensor has a strict majority */
  uint64_t n_diff;             /* number of differing tensors                  */
  uint64_t first_diff;         /* smallest differing tensor, or UINT64_MAX     */
  uint64_t first_no_majority;  /* smallest tensor with no majority, or UINT64_MAX */
} oracle_majority;

typedef struct {
  uint64_t index; /* element index of a single bit flip, UINT64_MAX if none fits */
  int32_t bit;    /* flipped bit, -1 if none                                      */
  int32_t dir;    /* +1: bit went 0->1 from a to b; -1: 1->0; 0: not a single flip */
} oracle_hint;

/* Width in bytes of one element, or 0 for an unknown type. */
uint32_t oracle_element_size(uint32_t dtype);

/* 1 if the raw pattern x (zero-extended) is NaN or +-Inf for dtype, else 0. */
int oracle_is_nonfinite(uint64_t x, uint32_t dtype);

/* Row of one tensor: data holds numel elements, contiguous, little-endian.
 * data == NULL or numel == 0 gives the zero row.  flags: ORACLE_SIGNED or 0. */
int oracle_fingerprint_ex(const void* data, uint64_t numel, uint32_t dtype, uint32_t flags,
                          oracle_row* out);
/* oracle_fingerprint_ex with flags 0 (zero-extended patterns). */
int oracle_fingerprint(const void* data, uint64_t numel, uint32_t dtype, oracle_row* out);

/* Rows of n tensors (ptrs[k], numels[k], dtypes[k]) into rows[0..n). */
int oracle_fingerprint_list(const void* const* ptrs, const uint64_t* numels,
                            const uint32_t* dtypes, uint64_t n, oracle_row* rows);

/* Non-finite count of each of n tensors, and their total. */
int oracle_nonfinite_list(const void* const* ptrs, const uint64_t* numels,
                          const uint32_t* dtypes, uint64_t n, uint64_t* counts,
                          uint64_t* total);

/* Strict-majority comparison of a replica-major table: row (r, k) is
 * table[r * T + k].  suspect[R] receives 1 for every named replica (all zero
 * when there is no majority somewhere); tensor_status[T] (may be NULL)
 * receives 0 = all equal, 1 = differs with a strict majority, 2 = no majority. */
int oracle_majority_compare(const oracle_row* table, uint32_t R, uint64_t T, uint32_t col_mask,
                            oracle_majority* res, uint8_t* suspect, uint8_t* tensor_status);

/* Single-bit-flip localisation for two rows of the same tensor. */
int oracle_flip_hint(const oracle_row* a, const oracle_row* b, oracle_hint* hint);

/* Tensors whose rows differ between tables a and b (length T): the exact count
 * in *n_diff, the first min(n_diff, cap) indices in ascending order in idx,
 * and (if hints != NULL) a flip hint for each of those indices. */
int oracle_fingerprint_diff(const oracle_row* a, const oracle_row* b, uint64_t T,
                            uint32_t col_mask, uint64_t* n_diff, uint64_t* idx, uint64_t cap,
                            oracle_hint* hints);

/* ---- squared norm ("Check 1: NaN/Inf gradients, ..."): the local gradient
 * norm is flagged when it is NaN or Inf in fp32 (which also catches finite
 * overflow of the squared sum). ------------------------------------------- */

/* Value of one element as a double, decoded from its type's bit layout
 * (raw integer types: 0, they carry no floating-point value). */
double oracle_value(uint64_t x, uint32_t dtype);

/* sum_i value_i^2 of one tensor, summed in index order in double. */
int oracle_sqnorm(const void* data, uint64_t numel, uint32_t dtype, double* out);

/* 1 when the squared sum, rounded to fp32, is not finite (NaN, Inf, or a
 * norm too large for fp32), else 0. */
int oracle_sqnorm_flag(double sq);

/* ---- ring replay audit ("Check 2: Ring replay, before the optimizer step") --
 * table: n ranks x 2 results x width uint64 words, rank-major.  Result 0 of
 * rank r is r's own result (loss bits and gradient fingerprints), result 1 is
 * r's replay of rank (r + offset) mod n.  Pair r = (target (r+offset) mod n,
 * replayer r) mismatches when the target's own result differs from the
 * replayer's replay in any word. */
int oracle_ring_pairs(const uint64_t* table, uint32_t n, uint64_t width, uint32_t offset,
                      uint8_t* mismatch);

/* Culprits are ranks that appear (as target or replayer) in at least two
 * mismatched pairs; a mismatched pair containing no culprit is ambiguous.
 * culprit[n] and ambiguous[n] (indexed like mismatch) receive 0/1. */
int oracle_ring_localize(const uint8_t* mismatch, uint32_t n, uint32_t offset, uint8_t* culprit,
                         uint8_t* ambiguous);

/* Verdict of a confirmation: a witness GPU on a third node and the target
 * itself (its retry) replay the target's work again.  original: the target's
 * first own result; replay: the replayer's replay of it.  All width words
 * long. */
enum {
  ORACLE_VERDICT_REPLAYER_WRONG = 1, /* suspect: the replayer */
  ORACLE_VERDICT_PERSISTENT = 2,     /* suspect: the target   */
  ORACLE_VERDICT_TRANSIENT = 3,      /* suspect: the target   */
  ORACLE_VERDICT_UNCLEAR = 4,        /* suspect: the target   */
  ORACLE_VERDICT_UNATTRIBUTABLE = 5  /* no suspect            */
};
int oracle_confirm_verdict(const uint64_t* witness, const uint64_t* retry, const uint64_t* original,
                           const uint64_t* replay, uint64_t width, int32_t* verdict);

#ifdef __cplusplus
}
#endif
#endif
