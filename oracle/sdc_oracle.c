/*
 * sdc_oracle.c -- reference (oracle) implementation.  TEST INFRASTRUCTURE ONLY:
 * only the tests, the smoke check and the benchmark's CPU-baseline leg load it.
 *
 * Plain single-threaded C.  Every quantity is a uint64_t, so all sums wrap
 * modulo 2^64 with defined behaviour.  No blocking, splitting, reordering or
 * vector tricks: each function walks its input once, in order, exactly as the
 * definition it cites reads.
 */
#include "sdc_oracle.h"

#include <math.h>
#include <stddef.h>
#include <string.h>

uint32_t oracle_element_size(uint32_t dtype) {
  switch (dtype) {
    case ORACLE_F32: case ORACLE_U32: return 4;
    case ORACLE_BF16: case ORACLE_F16: case ORACLE_U16: return 2;
    case ORACLE_F64: case ORACLE_U64: return 8;
    case ORACLE_U8: case ORACLE_FP8_E4M3: case ORACLE_FP8_E5M2:
    case ORACLE_FP8_E4M3FNUZ: case ORACLE_FP8_E5M2FNUZ: return 1;
    default: return 0;
  }
}

/* Raw bit pattern of element i, read byte by byte as little-endian and
 * zero-extended to 64 bits ("Compare by fingerprint": the sums run over the
 * elements' raw bit patterns; the unsigned reading is stated in the design
 * notes). */
static uint64_t load_bits(const unsigned char* base, uint64_t i, uint32_t esize) {
  const unsigned char* p = base + i * esize;
  uint64_t x = 0;
  for (uint32_t b = 0; b < esize; ++b) x |= (uint64_t)p[b] << (8u * b);
  return x;
}

/* NaN or +-Inf.  IEEE-style formats (binary32, bfloat16, binary16, binary64,
 * fp8 E5M2): the exponent field is all ones (every NaN payload and sign
 * counts).  fp8 E4M3 (OCP "fn"): no Inf, NaN is S.1111.111.  The "fnuz" fp8
 * formats: no Inf, the single NaN is 0x80.  Raw integer types: never. */
int oracle_is_nonfinite(uint64_t x, uint32_t dtype) {
  switch (dtype) {
    case ORACLE_F32: return (x & 0x7F800000ull) == 0x7F800000ull;
    case ORACLE_BF16: return (x & 0x7F80ull) == 0x7F80ull;
    case ORACLE_F16: return (x & 0x7C00ull) == 0x7C00ull;
    case ORACLE_F64: return (x & 0x7FF0000000000000ull) == 0x7FF0000000000000ull;
    case ORACLE_FP8_E4M3: return (x & 0x7Full) == 0x7Full;
    case ORACLE_FP8_E5M2: return (x & 0x7Cull) == 0x7Cull;
    case ORACLE_FP8_E4M3FNUZ: case ORACLE_FP8_E5M2FNUZ: return x == 0x80ull;
    default: return 0;
  }
}

/* The pattern x of a `esize`-byte element widened to 64 bits: sign-extended
 * for 2- and 4-byte elements when ORACLE_SIGNED is set, else zero-extended. */
static uint64_t widen(uint64_t x, uint32_t esize, uint32_t flags) {
  if ((flags & ORACLE_SIGNED) && (esize == 2 || esize == 4)) {
    uint64_t msb = 1ull << (8u * esize - 1u);
    if (x & msb) x |= ~((msb << 1) - 1u);
  }
  return x;
}

/* "Compare by fingerprint": S = sum of x_i, W = sum of (i+1)*x_i, both modulo
 * 2^64 with 1-based positions; a missing tensor keeps its zero row.
 * AEGIS review, "core method" item 4: X = xor of the x_i.
 * Nonfinite count: the element-exact form of the NaN/Inf test of "Check 1". */
int oracle_fingerprint_ex(const void* data, uint64_t numel, uint32_t dtype, uint32_t flags,
                          oracle_row* out) {
  if (out == NULL || (flags & ~(uint32_t)ORACLE_SIGNED) != 0) return ORACLE_EINVAL;
  uint32_t esize = oracle_element_size(dtype);
  if (esize == 0) return ORACLE_EDTYPE;
  uint64_t s = 0, w = 0, x = 0, nf = 0;
  if (data != NULL) {
    const unsigned char* base = (const unsigned char*)data;
    for (uint64_t i = 0; i < numel; ++i) {
      uint64_t raw = load_bits(base, i, esize);
      uint64_t v = widen(raw, esize, flags);
      s += v;
      w += (i + 1) * v;
      x ^= v;
      nf += (uint64_t)oracle_is_nonfinite(raw, dtype);
    }
  }
  out->sum = s;
  out->wsum = w;
  out->xorsum = x;
  out->nonfinite = nf;
  return ORACLE_OK;
}

int oracle_fingerprint(const void* data, uint64_t numel, uint32_t dtype, oracle_row* out) {
  return oracle_fingerprint_ex(data, numel, dtype, 0, out);
}

int oracle_fingerprint_list(const void* const* ptrs, const uint64_t* numels,
                            const uint32_t* dtypes, uint64_t n, oracle_row* rows) {
  if (n > 0 && (ptrs == NULL || numels == NULL || dtypes == NULL || rows == NULL))
    return ORACLE_EINVAL;
  for (uint64_t k = 0; k < n; ++k) {
    int rc = oracle_fingerprint(ptrs[k], numels[k], dtypes[k], &rows[k]);
    if (rc != ORACLE_OK) return rc;
  }
  return ORACLE_OK;
}

int oracle_nonfinite_list(const void* const* ptrs, const uint64_t* numels,
                          const uint32_t* dtypes, uint64_t n, uint64_t* counts,
                          uint64_t* total) {
  if (total == NULL) return ORACLE_EINVAL;
  if (n > 0 && (ptrs == NULL || numels == NULL || dtypes == NULL || counts == NULL))
    return ORACLE_EINVAL;
  uint64_t t = 0;
  for (uint64_t k = 0; k < n; ++k) {
    uint32_t esize = oracle_element_size(dtypes[k]);
    if (esize == 0) return ORACLE_EDTYPE;
    uint64_t c = 0;
    if (ptrs[k] != NULL) {
      const unsigned char* base = (const unsigned char*)ptrs[k];
      for (uint64_t i = 0; i < numels[k]; ++i)
        c += (uint64_t)oracle_is_nonfinite(load_bits(base, i, esize), dtypes[k]);
    }
    counts[k] = c;
    t += c;
  }
  *total = t;
  return ORACLE_OK;
}

static int rows_equal(const oracle_row* a, const oracle_row* b, uint32_t mask) {
  if ((mask & ORACLE_COL_SUM) && a->sum != b->sum) return 0;
  if ((mask & ORACLE_COL_WSUM) && a->wsum != b->wsum) return 0;
  if ((mask & ORACLE_COL_XOR) && a->xorsum != b->xorsum) return 0;
  if ((mask & ORACLE_COL_NONFINITE) && a->nonfinite != b->nonfinite) return 0;
  return 1;
}

/* "Check 3: Weight fingerprints, after the optimizer step": a tensor differs
 * when some replica's row is not equal to replica 0's.  For each differing
 * tensor the most common row is found; if it is held by no more than half of
 * the replicas there is no strict majority and no replica is named;
 * otherwise every replica whose row differs from it is named. */
int oracle_majority_compare(const oracle_row* table, uint32_t R, uint64_t T, uint32_t col_mask,
                            oracle_majority* res, uint8_t* suspect, uint8_t* tensor_status) {
  if (table == NULL || res == NULL || suspect == NULL || R == 0 || T == 0) return ORACLE_EINVAL;
  if ((col_mask & ORACLE_COL_ALL) == 0 || (col_mask & ~(uint32_t)ORACLE_COL_ALL) != 0)
    return ORACLE_EINVAL;
  res->diverged = 0;
  res->has_majority = 1;
  res->n_diff = 0;
  res->first_diff = UINT64_MAX;
  res->first_no_majority = UINT64_MAX;
  for (uint32_t r = 0; r < R; ++r) suspect[r] = 0;

  for (uint64_t k = 0; k < T; ++k) {
    int differs = 0;
    for (uint32_t r = 1; r < R; ++r)
      if (!rows_equal(&table[(uint64_t)r * T + k], &table[k], col_mask)) differs = 1;
    if (tensor_status != NULL) tensor_status[k] = 0;
    if (!differs) continue;

    res->diverged = 1;
    res->n_diff += 1;
    if (res->first_diff == UINT64_MAX) res->first_diff = k;

    /* Most common row: count, for every replica, how many replicas hold the
     * same row; keep the first replica with the largest count. */
    uint32_t best = 0, best_count = 0;
    for (uint32_t r = 0; r < R; ++r) {
      uint32_t c = 0;
      for (uint32_t q = 0; q < R; ++q)
        if (rows_equal(&table[(uint64_t)q * T + k], &table[(uint64_t)r * T + k], col_mask)) c++;
      if (c > best_count) { best_count = c; best = r; }
    }
    if (2ull * best_count <= (uint64_t)R) {
      res->has_majority = 0;
      if (res->first_no_majority == UINT64_MAX) res->first_no_majority = k;
      if (tensor_status != NULL) tensor_status[k] = 2;
      continue;
    }
    if (tensor_status != NULL) tensor_status[k] = 1;
    for (uint32_t r = 0; r < R; ++r)
      if (!rows_equal(&table[(uint64_t)r * T + k], &table[(uint64_t)best * T + k], col_mask))
        suspect[r] = 1;
  }
  /* A single tensor without a strict majority means no replica is named. */
  if (!res->has_majority)
    for (uint32_t r = 0; r < R; ++r) suspect[r] = 0;
  return ORACLE_OK;
}

/* A single flipped bit b at element i (0-based) moves S by +-2^b, W by
 * +-(i+1)*2^b with the same sign, and X by exactly 2^b.  This inverts that:
 * it is a consequence of the definitions of "Compare by fingerprint", not a
 * rule stated on the pages. */
int oracle_flip_hint(const oracle_row* a, const oracle_row* b, oracle_hint* hint) {
  if (a == NULL || b == NULL || hint == NULL) return ORACLE_EINVAL;
  hint->index = UINT64_MAX;
  hint->bit = -1;
  hint->dir = 0;
  uint64_t dx = a->xorsum ^ b->xorsum;
  if (dx == 0 || (dx & (dx - 1)) != 0) return ORACLE_OK; /* not exactly one bit */
  int bit = 0;
  while (((dx >> bit) & 1u) == 0) bit++;
  uint64_t ds = b->sum - a->sum;
  uint64_t dw = b->wsum - a->wsum;
  int dir;
  if (ds == dx) {
    dir = 1;
  } else if (ds == (uint64_t)0 - dx) {
    dir = -1;
    dw = (uint64_t)0 - dw;
  } else {
    return ORACLE_OK;
  }
  /* dw must equal (i+1) * 2^bit for some i >= 0 with (i+1) * 2^bit < 2^63.
   * Below that bound (met by any tensor of fewer than 2^32 elements of at
   * most 4 bytes) the inversion is unique; above it the sign is ambiguous. */
  if ((dw >> 63) != 0) return ORACLE_OK;
  uint64_t q = dw >> bit;
  if (q == 0 || (q << bit) != dw) return ORACLE_OK;
  hint->index = q - 1;
  hint->bit = bit;
  hint->dir = dir;
  return ORACLE_OK;
}

/* "Check 2: Ring replay": the replay is compared row by row, for exact
 * equality, with the original. */
int oracle_fingerprint_diff(const oracle_row* a, const oracle_row* b, uint64_t T,
                            uint32_t col_mask, uint64_t* n_diff, uint64_t* idx, uint64_t cap,
                            oracle_hint* hints) {
  if (n_diff == NULL || (T > 0 && (a == NULL || b == NULL)) || (cap > 0 && idx == NULL))
    return ORACLE_EINVAL;
  if ((col_mask & ORACLE_COL_ALL) == 0 || (col_mask & ~(uint32_t)ORACLE_COL_ALL) != 0)
    return ORACLE_EINVAL;
  uint64_t n = 0;
  for (uint64_t k = 0; k < T; ++k) {
    if (rows_equal(&a[k], &b[k], col_mask)) continue;
    if (n < cap) {
      idx[n] = k;
      if (hints != NULL) oracle_flip_hint(&a[k], &b[k], &hints[n]);
    }
    n++;
  }
  *n_diff = n;
  return ORACLE_OK;
}

static int words_equal(const uint64_t* a, const uint64_t* b, uint64_t width) {
  for (uint64_t i = 0; i < width; ++i)
    if (a[i] != b[i]) return 0;
  return 1;
}

/* "Check 2": every rank replays the rank `offset` positions ahead; pair r
 * mismatches when the target's own result and the replay are not equal. */
int oracle_ring_pairs(const uint64_t* table, uint32_t n, uint64_t width, uint32_t offset,
                      uint8_t* mismatch) {
  if (n == 0 || mismatch == NULL || (width > 0 && table == NULL)) return ORACLE_EINVAL;
  for (uint32_t r = 0; r < n; ++r) {
    uint32_t t = (uint32_t)(((uint64_t)r + offset) % n);
    const uint64_t* own_of_target = table + ((uint64_t)t * 2 + 0) * width;
    const uint64_t* replay_by_r = table + ((uint64_t)r * 2 + 1) * width;
    mismatch[r] = (uint8_t)!words_equal(own_of_target, replay_by_r, width);
  }
  return ORACLE_OK;
}

/* "Check 2": a rank seen in both of its comparisons (or more) is a culprit;
 * a mismatched pair with no culprit in it is left for confirmation. */
int oracle_ring_localize(const uint8_t* mismatch, uint32_t n, uint32_t offset, uint8_t* culprit,
                         uint8_t* ambiguous) {
  if (n == 0 || mismatch == NULL || culprit == NULL || ambiguous == NULL) return ORACLE_EINVAL;
  for (uint32_t r = 0; r < n; ++r) culprit[r] = 0;
  /* count appearances: pair r holds the target (r+offset) mod n and the replayer r */
  for (uint32_t q = 0; q < n; ++q) {
    uint32_t hits = 0;
    for (uint32_t r = 0; r < n; ++r) {
      if (!mismatch[r]) continue;
      uint32_t t = (uint32_t)(((uint64_t)r + offset) % n);
      if (t == q) hits++;
      if (r == q) hits++;
    }
    culprit[q] = (uint8_t)(hits >= 2);
  }
  for (uint32_t r = 0; r < n; ++r) {
    uint32_t t = (uint32_t)(((uint64_t)r + offset) % n);
    ambiguous[r] = (uint8_t)(mismatch[r] && !culprit[t] && !culprit[r]);
  }
  return ORACLE_OK;
}

/* "Check 2", confirmation, from the section's "Only one mismatches" case and
 * the verdict rows of "Decide what the alarm means".  Two GPUs replay the
 * target's work once more: a witness on a third node and the target itself
 * (its retry).  Four equalities decide: witness == original (the target's own
 * first result), witness == replay (the replayer's replay of that work),
 * retry == original, retry == witness.
 *   - The witness reproduces the original: the target was right, so the
 *     replaying GPU was wrong ("replayer computed wrong").
 *   - The witness sides with the replayer (and not with the original): the
 *     target was wrong.  It reproduced its own wrong answer: "persistent";
 *     its retry came out right, agreeing with the witness: "transient";
 *     otherwise the three results do not line up: "unclear".
 *   - The witness agrees with neither: nobody can be named ("unattributable").
 * Indexed by the four equalities as bits (1: witness == original, 2: witness
 * == replay, 4: retry == original, 8: retry == witness).  Where the witness
 * equals both, the original equals the replay, and the pair did not mismatch;
 * the first rule then still applies. */
static const int32_t kVerdictOf[16] = {
    /* 0b0000 */ ORACLE_VERDICT_UNATTRIBUTABLE, /* 0b0001 */ ORACLE_VERDICT_REPLAYER_WRONG,
    /* 0b0010 */ ORACLE_VERDICT_UNCLEAR,        /* 0b0011 */ ORACLE_VERDICT_REPLAYER_WRONG,
    /* 0b0100 */ ORACLE_VERDICT_UNATTRIBUTABLE, /* 0b0101 */ ORACLE_VERDICT_REPLAYER_WRONG,
    /* 0b0110 */ ORACLE_VERDICT_PERSISTENT,     /* 0b0111 */ ORACLE_VERDICT_REPLAYER_WRONG,
    /* 0b1000 */ ORACLE_VERDICT_UNATTRIBUTABLE, /* 0b1001 */ ORACLE_VERDICT_REPLAYER_WRONG,
    /* 0b1010 */ ORACLE_VERDICT_TRANSIENT,      /* 0b1011 */ ORACLE_VERDICT_REPLAYER_WRONG,
    /* 0b1100 */ ORACLE_VERDICT_UNATTRIBUTABLE, /* 0b1101 */ ORACLE_VERDICT_REPLAYER_WRONG,
    /* 0b1110 */ ORACLE_VERDICT_PERSISTENT,     /* 0b1111 */ ORACLE_VERDICT_REPLAYER_WRONG};

int oracle_confirm_verdict(const uint64_t* witness, const uint64_t* retry, const uint64_t* original,
                           const uint64_t* replay, uint64_t width, int32_t* verdict) {
  if (verdict == NULL ||
      (width > 0 && (witness == NULL || retry == NULL || original == NULL || replay == NULL)))
    return ORACLE_EINVAL;
  unsigned idx = (unsigned)words_equal(witness, original, width) |
                 (unsigned)words_equal(witness, replay, width) << 1 |
                 (unsigned)words_equal(retry, original, width) << 2 |
                 (unsigned)words_equal(retry, witness, width) << 3;
  *verdict = kVerdictOf[idx];
  return ORACLE_OK;
}

/* Decoding from the formats' definitions: (-1)^s * 2^(e - bias) * (1 + f)
 * for normal numbers, (-1)^s * 2^(1 - bias) * f for subnormals (e == 0),
 * with f the mantissa field over 2^(mantissa bits). */
static double decode(uint64_t x, int ebits, int mbits, int bias) {
  uint64_t m = x & ((1ull << mbits) - 1u);
  uint64_t e = (x >> mbits) & ((1ull << ebits) - 1u);
  int s = (int)((x >> (ebits + mbits)) & 1u);
  double f = (double)m / (double)(1ull << mbits);
  double v = (e == 0) ? ldexp(f, 1 - bias) : ldexp(1.0 + f, (int)e - bias);
  return s ? -v : v;
}

double oracle_value(uint64_t x, uint32_t dtype) {
  switch (dtype) {
    case ORACLE_F32: case ORACLE_BF16: case ORACLE_F16: case ORACLE_F64: case ORACLE_FP8_E5M2:
      if (oracle_is_nonfinite(x, dtype)) {  /* IEEE: mantissa 0 is Inf, else NaN */
        int mbits = dtype == ORACLE_F32 ? 23 : dtype == ORACLE_BF16 ? 7 : dtype == ORACLE_F16 ? 10
                  : dtype == ORACLE_F64 ? 52 : 2;
        int sbit = dtype == ORACLE_F32 ? 31 : dtype == ORACLE_F64 ? 63 : dtype == ORACLE_FP8_E5M2 ? 7 : 15;
        if ((x & ((1ull << mbits) - 1u)) != 0) return NAN;
        return ((x >> sbit) & 1u) ? -INFINITY : INFINITY;
      }
      break;
    case ORACLE_FP8_E4M3: case ORACLE_FP8_E4M3FNUZ: case ORACLE_FP8_E5M2FNUZ:
      if (oracle_is_nonfinite(x, dtype)) return NAN;  /* these formats have no Inf */
      break;
    default:
      return 0.0;
  }
  switch (dtype) {
    case ORACLE_F32: return decode(x, 8, 23, 127);
    case ORACLE_BF16: return decode(x, 8, 7, 127);
    case ORACLE_F16: return decode(x, 5, 10, 15);
    case ORACLE_F64: return decode(x, 11, 52, 1023);
    case ORACLE_FP8_E5M2: return decode(x, 5, 2, 15);
    case ORACLE_FP8_E4M3: return decode(x, 4, 3, 7);
    case ORACLE_FP8_E4M3FNUZ: return decode(x, 4, 3, 8);
    case ORACLE_FP8_E5M2FNUZ: return decode(x, 5, 2, 16);
    default: return 0.0;
  }
}

int oracle_sqnorm(const void* data, uint64_t numel, uint32_t dtype, double* out) {
  if (out == NULL) return ORACLE_EINVAL;
  uint32_t esize = oracle_element_size(dtype);
  if (esize == 0) return ORACLE_EDTYPE;
  double acc = 0.0;
  if (data != NULL) {
    const unsigned char* base = (const unsigned char*)data;
    for (uint64_t i = 0; i < numel; ++i) {
      double v = oracle_value(load_bits(base, i, esize), dtype);
      acc += v * v;
    }
  }
  *out = acc;
  return ORACLE_OK;
}

int oracle_sqnorm_flag(double sq) {
  float f = (float)sq;
  return !isfinite(f);
}
