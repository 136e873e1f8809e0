/*
 * oracle.c -- plain fp64 CPU reference for block-sparse masked attention.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code,
 * header, table or constant with the HIP library, and includes nothing from it.
 *
 * What it computes, and where the definition comes from:
 *
 *  - The attention definition: O = softmax(Q K^T * scale + B) V, with B = 0 on
 *    live pairs and -inf on masked ones, applied in four steps (score table,
 *    scale, add the mask bias, softmax then mix V). Page "SDPA replaces
 *    hand-written attention" (qiita GeneLab_999), section 1, the Attention
 *    equation and the four steps listed under it. Default scale 1/sqrt(E) is
 *    the caller's business; this function takes scale explicitly.
 *
 *  - The mask rules (all return "live"):
 *      causal:   q_idx >= kv_idx
 *      sliding:  q_idx >= kv_idx and q_idx - kv_idx < W
 *      document: q_idx >= kv_idx and doc[q_idx] == doc[kv_idx]
 *    Page "FlexAttention on Apple Silicon: block masks" (dreaming.press),
 *    sections "Mask 1: causal", "Mask 2: sliding-window causal",
 *    "Mask 3: document-packed".
 *    Variants on the same rules:
 *      causal, lower right:   q_idx + (S - L) >= kv_idx
 *      sliding, lower right:  with p = q_idx + (S - L): p >= kv_idx and p - kv_idx < W
 *    the causal triangle aligned to the bottom-right corner when L != S, so
 *    the last query sees every key (page "SDPA replaces hand-written
 *    attention" (qiita GeneLab_999), section 4, pitfall 3, causal_lower_right);
 *      document, bidirectional: doc[q_idx] == doc[kv_idx]
 *    the block-diagonal document mask without the causal part.
 *
 *  - The score_mod soft-cap s <- c * tanh(s / c), applied to the scaled score
 *    of every pair; the mask then removes dead pairs. Same page, section
 *    "Bonus: a score_mod for soft-capping" (score_mod changes the value, the
 *    mask decides liveness; sparsity from the mask, score_mod on survivors).
 *
 *  - A user-supplied dense boolean mask M [L][S] (kind DENSE): the pair is
 *    live exactly when M[i][j] is true, the boolean attn_mask convention of
 *    page "SDPA replaces hand-written attention" (qiita GeneLab_999),
 *    section 4, pitfall 1 (True keeps the pair); the pages build such masks
 *    densely for SDPA and skip blocks from them for FlexAttention (page
 *    "FlexAttention on MPS vs SDPA" (qiita kiarina), setup notes on the
 *    32768 x 32768 boolean mask). Its bit-packed form (oracle_pack_mask):
 *    row i holds W = 4 * ceil(S / 128) 32-bit words, bit b of word w is
 *    M[i][32 w + b], and bits at 32 w + b >= S are 0.
 *
 *  - Key padding: per batch entry b, only keys in [key_start[b], key_end[b])
 *    are kept, ANDed with the mask rule (padding keys never take weight).
 *    Page "SDPA replaces hand-written attention" (qiita GeneLab_999),
 *    section 4, pitfall 1 (a boolean mask's True keeps the pair; padded
 *    keys are dropped) and section 5 (padding ANDed with the causal mask,
 *    left padding in its test).
 *
 *  - A row with no live key yields O = 0 and logsumexp = -inf, the
 *    fully-masked-row behaviour that the SDPA page measures (section 4,
 *    pitfall 1, the "all rows masked" aside: zeros, not NaN).
 *
 *  - The 128x128 BlockMask: per query block, kv blocks with no live pair are
 *    skipped, blocks whose every pair is live are "full", the rest "partial".
 *    Page "FlexAttention on MPS vs SDPA" (qiita kiarina), data-flow section
 *    (BlockMask groups tokens into 128x128 blocks and skips unneeded blocks);
 *    "FlexAttention on Apple Silicon", closing section (only fully masked
 *    blocks can be skipped; causal leaves blocks partially live).
 *    Here each block is classified by brute force: every in-range pair is
 *    evaluated with the predicate and counted.
 *
 *  - The backward: gradients of the scalar sum(dO * O) with respect to q, k
 *    and v, with the attention matrix recomputed instead of stored (page
 *    "Flash Attention 2 and the IO bottleneck" (tcdigital), section on
 *    recomputation in backpropagation). Written out by the chain rule from
 *    the forward definition: with P the row softmax of the masked scores
 *    s' = mod(scale * q.k) (mod = identity, or c * tanh(. / c)),
 *      dV_j  = sum_i P_ij dO_i
 *      dP_ij = dO_i . v_j,   D_i = sum_j P_ij dP_ij
 *      dS'_ij = P_ij (dP_ij - D_i)
 *      dS_ij = dS'_ij * scale * mod'(scale q_i.k_j),  mod' = 1 - (s'/c)^2 or 1
 *      dQ_i = sum_j dS_ij k_j,   dK_j = sum_i dS_ij q_i
 *    Masked pairs have P = 0 and so no gradient; a row with no live key has
 *    P = 0 and contributes nothing.
 *
 * Arithmetic is fp64 throughout (libm exp, tanh, log). Rows are independent;
 * OpenMP spreads whole rows over threads and changes no arithmetic order
 * inside a row.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_NONE 0
#define ORACLE_CAUSAL 1
#define ORACLE_SLIDING 2
#define ORACLE_DOCUMENT 3
#define ORACLE_CAUSAL_LOWER_RIGHT 4
#define ORACLE_SLIDING_LOWER_RIGHT 5
#define ORACLE_DOCUMENT_BIDIRECTIONAL 6
#define ORACLE_DENSE 7

/* The mask predicate: 1 when query i may attend to key j, for L queries and
 * S keys (the lower-right kinds shift the query position by S - L; DENSE
 * reads the L x S byte mask, nonzero = live). */
static int live(int kind, int64_t window, const int32_t* doc, const uint8_t* dense, int64_t L,
                int64_t S, int64_t i, int64_t j) {
  switch (kind) {
    case ORACLE_DENSE:
      return dense[i * S + j] != 0;
    case ORACLE_NONE:
      return 1;
    case ORACLE_CAUSAL:
      return i >= j;
    case ORACLE_SLIDING:
      return i >= j && (i - j) < window;
    case ORACLE_DOCUMENT:
      return i >= j && doc[i] == doc[j];
    case ORACLE_CAUSAL_LOWER_RIGHT:
      return i + (S - L) >= j;
    case ORACLE_SLIDING_LOWER_RIGHT: {
      const int64_t p = i + (S - L);
      return p >= j && (p - j) < window;
    }
    case ORACLE_DOCUMENT_BIDIRECTIONAL:
      return doc[i] == doc[j];
    default:
      return 0;
  }
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Evaluate the predicate itself (used by the tests to count live pairs). */
int oracle_live(int kind, int64_t window, const int32_t* doc, const uint8_t* dense, int64_t L,
                int64_t S, int64_t i, int64_t j) {
  return live(kind, window, doc, dense, L, S, i, j);
}

/* Number of live pairs over [0,L) x [0,S). */
int64_t oracle_count_live(int kind, int64_t window, const int32_t* doc, const uint8_t* dense,
                          int64_t L, int64_t S) {
  int64_t total = 0;
#pragma omp parallel for reduction(+ : total) schedule(dynamic, 16)
  for (int64_t i = 0; i < L; ++i) {
    int64_t c = 0;
    for (int64_t j = 0; j < S; ++j) c += live(kind, window, doc, dense, L, S, i, j);
    total += c;
  }
  return total;
}

/*
 * Brute-force BlockMask. Outputs (caller-allocated, int32):
 *   kv_num[nq], kv_idx[nq*nk]         partial blocks, ascending, pad 0
 *   full_num[nq], full_idx[nq*nk]     full blocks, ascending, pad 0
 * with nq = ceil(L/bs), nk = ceil(S/bs). A block is full only when all
 * bs*bs of its pairs are in range and live. Returns 0, or -1 on bad sizes.
 */
int oracle_block_mask(int kind, int64_t window, const int32_t* doc, const uint8_t* dense, int64_t L,
                      int64_t S, int64_t bs, int32_t* kv_num, int32_t* kv_idx, int32_t* full_num,
                      int32_t* full_idx) {
  if (L < 0 || S < 0 || bs <= 0) return -1;
  int64_t nq = (L + bs - 1) / bs, nk = (S + bs - 1) / bs;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t qb = 0; qb < nq; ++qb) {
    int32_t np = 0, nf = 0;
    for (int64_t t = 0; t < nk; ++t) {
      kv_idx[qb * nk + t] = 0;
      full_idx[qb * nk + t] = 0;
    }
    for (int64_t kb = 0; kb < nk; ++kb) {
      int64_t count = 0;
      for (int64_t i = qb * bs; i < (qb + 1) * bs && i < L; ++i)
        for (int64_t j = kb * bs; j < (kb + 1) * bs && j < S; ++j)
          count += live(kind, window, doc, dense, L, S, i, j);
      if (count == 0) continue;
      if (count == bs * bs)
        full_idx[qb * nk + nf++] = (int32_t)kb;
      else
        kv_idx[qb * nk + np++] = (int32_t)kb;
    }
    kv_num[qb] = np;
    full_num[qb] = nf;
  }
  return 0;
}

/*
 * Bit-packed form of a dense L x S byte mask (nonzero = live): row i is
 * W = 4 * ceil(S / 128) words, bit b of word w = (dense[i][32 w + b] != 0),
 * 0 past S. bits: caller-allocated uint32 [L * W]. Returns 0, or -1 on bad
 * sizes.
 */
int oracle_pack_mask(const uint8_t* dense, int64_t L, int64_t S, uint32_t* bits) {
  if (L < 0 || S < 0) return -1;
  const int64_t W = 4 * ((S + 127) / 128);
  for (int64_t i = 0; i < L; ++i)
    for (int64_t w = 0; w < W; ++w) {
      uint32_t word = 0;
      for (int64_t b = 0; b < 32; ++b) {
        const int64_t j = 32 * w + b;
        if (j < S && dense[i * S + j] != 0) word |= (uint32_t)1 << b;
      }
      bits[i * W + w] = word;
    }
  return 0;
}

/*
 * Steps 1-3 for query row i of one (batch, head): s[j] = the scaled score
 * q_i.k_j * scale, soft-capped when softcap > 0, and -inf where the mask or
 * the kept key range [kept_lo, kept_hi) drops the pair. Returns the row max
 * (-inf when no key is live).
 */
static double row_scores(const double* qi, const double* kh, int64_t L, int64_t S, int64_t E,
                         int64_t i, int kind, int64_t window, const int32_t* doc,
                         const uint8_t* dense, double softcap, double scale, int64_t kept_lo,
                         int64_t kept_hi, double* s) {
  double m = -INFINITY;
  for (int64_t j = 0; j < S; ++j) {
    double dot = 0.0;
    for (int64_t e = 0; e < E; ++e) dot += qi[e] * kh[j * E + e];
    double sc = dot * scale;
    if (softcap > 0.0) sc = softcap * tanh(sc / softcap);
    if (!live(kind, window, doc, dense, L, S, i, j) || j < kept_lo || j >= kept_hi) sc = -INFINITY;
    s[j] = sc;
    if (sc > m) m = sc;
  }
  return m;
}

/*
 * Masked softmax attention, fp64, for a list of rows.
 *   q [B,H,L,E], k [B,H,S,E], v [B,H,S,Ev]: contiguous fp64.
 *   key_start, key_end: per batch entry [B], the kept key range [start, end),
 *   or NULL for no padding. dense: the L x S byte mask of kind DENSE (NULL
 *   otherwise).
 *   rows: flat row ids r = (b*H + h)*L + i, or NULL for all B*H*L rows.
 *   out [nrows, Ev], lse [nrows] (natural log; -inf for a row with no live key).
 *   softcap > 0 applies s <- softcap * tanh(s / softcap) to the scaled score.
 * Returns 0, or -1 on bad sizes / allocation failure.
 */
int oracle_attention(const double* q, const double* k, const double* v, int64_t B, int64_t H,
                     int64_t L, int64_t S, int64_t E, int64_t Ev, int kind, int64_t window,
                     const int32_t* doc, const uint8_t* dense, double softcap, double scale,
                     const int64_t* key_start,
                     const int64_t* key_end, const int64_t* rows, int64_t nrows, double* out,
                     double* lse) {
  if (B < 0 || H < 0 || L < 0 || S < 0 || E <= 0 || Ev <= 0) return -1;
  if (rows == NULL) nrows = B * H * L;
  int failed = 0;
#pragma omp parallel reduction(| : failed)
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
    if (s == NULL) failed = 1;
#pragma omp for schedule(dynamic, 8)
    for (int64_t n = 0; n < nrows; ++n) {
      if (s == NULL) continue;
      int64_t r = rows ? rows[n] : n;
      int64_t bh = r / L, i = r % L;
      /* Kept keys of this batch entry (whole range when no padding given). */
      const int64_t b = bh / H;
      const int64_t kept_lo = key_start ? key_start[b] : 0;
      const int64_t kept_hi = key_end ? key_end[b] : S;
      const double* qi = q + r * E;
      const double* kh = k + bh * S * E;
      const double* vh = v + bh * S * Ev;
      double* o = out + n * Ev;

      /* Step 1-3: scores, scale, score_mod, mask. */
      const double m = row_scores(qi, kh, L, S, E, i, kind, window, doc, dense, softcap, scale,
                                  kept_lo, kept_hi, s);
      /* Step 4: softmax, then mix V. */
      for (int64_t e = 0; e < Ev; ++e) o[e] = 0.0;
      if (m == -INFINITY) {
        lse[n] = -INFINITY;
        continue;
      }
      double l = 0.0;
      for (int64_t j = 0; j < S; ++j) {
        double w = exp(s[j] - m); /* exp(-inf) = 0 for masked pairs */
        l += w;
        if (w != 0.0)
          for (int64_t e = 0; e < Ev; ++e) o[e] += w * vh[j * Ev + e];
      }
      for (int64_t e = 0; e < Ev; ++e) o[e] /= l;
      lse[n] = m + log(l);
    }
    free(s);
  }
  return failed ? -1 : 0;
}

/* dS_ij = P_ij (dP_ij - D_i) * scale * mod', with mod' = 1 - (s'/c)^2 the
 * soft-cap's derivative at the capped score s' (1 without the soft-cap). */
static double dscore(double p, double dp, double D, double sp, double softcap, double scale) {
  double ds = p * (dp - D) * scale;
  if (softcap > 0.0) ds *= 1.0 - (sp / softcap) * (sp / softcap);
  return ds;
}

/*
 * Backward of oracle_attention (all rows): q [B,H,L,E], k, v [B,H,S,E], dout
 * [B,H,L,E] contiguous fp64 (K/V heads already expanded to H); outputs dq
 * [B,H,L,E], dk, dv [B,H,S,E]. Same mask arguments as oracle_attention.
 * Returns 0, or -1 on bad sizes / allocation failure.
 */
int oracle_attention_backward(const double* q, const double* k, const double* v, const double* dout,
                              int64_t B, int64_t H, int64_t L, int64_t S, int64_t E, int kind,
                              int64_t window, const int32_t* doc, const uint8_t* dense, double softcap,
                              double scale, const int64_t* key_start, const int64_t* key_end,
                              double* dq, double* dk, double* dv) {
  if (B < 0 || H < 0 || L < 0 || S < 0 || E <= 0) return -1;
  memset(dq, 0, sizeof(double) * (size_t)(B * H * L * E));
  memset(dk, 0, sizeof(double) * (size_t)(B * H * S * E));
  memset(dv, 0, sizeof(double) * (size_t)(B * H * S * E));
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
  for (int64_t bh = 0; bh < B * H; ++bh) {
    double* sp = (double*)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));  /* scores s' */
    double* p = (double*)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));   /* P */
    double* dp = (double*)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));  /* dP */
    if (sp == NULL || p == NULL || dp == NULL) {
      failed = 1;
      free(sp), free(p), free(dp);
      continue;
    }
    const int64_t b = bh / H;
    const int64_t kept_lo = key_start ? key_start[b] : 0;
    const int64_t kept_hi = key_end ? key_end[b] : S;
    const double* kh = k + bh * S * E;
    const double* vh = v + bh * S * E;
    double* dkh = dk + bh * S * E;
    double* dvh = dv + bh * S * E;
    for (int64_t i = 0; i < L; ++i) {
      const double* qi = q + (bh * L + i) * E;
      const double* doi = dout + (bh * L + i) * E;
      double* dqi = dq + (bh * L + i) * E;
      /* forward: masked scores and their softmax */
      const double m = row_scores(qi, kh, L, S, E, i, kind, window, doc, dense, softcap, scale,
                                  kept_lo, kept_hi, sp);
      if (m == -INFINITY) continue; /* no live key: P = 0, no gradient */
      double l = 0.0;
      for (int64_t j = 0; j < S; ++j) {
        p[j] = exp(sp[j] - m);
        l += p[j];
      }
      for (int64_t j = 0; j < S; ++j) p[j] /= l;
      /* dP and D */
      double D = 0.0;
      for (int64_t j = 0; j < S; ++j) {
        double t = 0.0;
        for (int64_t e = 0; e < E; ++e) t += doi[e] * vh[j * E + e];
        dp[j] = t;
        D += p[j] * t;
      }
      for (int64_t j = 0; j < S; ++j) {
        if (p[j] == 0.0) continue;
        const double ds = dscore(p[j], dp[j], D, sp[j], softcap, scale);
        for (int64_t e = 0; e < E; ++e) {
          dqi[e] += ds * kh[j * E + e];
          dkh[j * E + e] += ds * qi[e];
          dvh[j * E + e] += p[j] * doi[e];
        }
      }
    }
    free(sp), free(p), free(dp);
  }
  return failed ? -1 : 0;
}

/*
 * dq of oracle_attention_backward for a list of flat rows r = (b*H + h)*L + i
 * only (each needs just its own row of P): dq_rows [nrows, E]. Returns 0, or
 * -1 on bad sizes / allocation failure.
 */
int oracle_attention_backward_dq_rows(const double* q, const double* k, const double* v,
                                      const double* dout, int64_t B, int64_t H, int64_t L, int64_t S,
                                      int64_t E, int kind, int64_t window, const int32_t* doc,
                                      const uint8_t* dense, double softcap, double scale,
                                      const int64_t* key_start, const int64_t* key_end,
                                      const int64_t* rows, int64_t nrows, double* dq_rows) {
  if (B < 0 || H < 0 || L <= 0 || S < 0 || E <= 0 || nrows < 0) return -1;
  int failed = 0;
#pragma omp parallel reduction(| : failed)
  {
    double* sp = (double*)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
    double* p = (double*)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
    double* dp = (double*)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
    if (sp == NULL || p == NULL || dp == NULL) failed = 1;
#pragma omp for schedule(dynamic, 4)
    for (int64_t n = 0; n < nrows; ++n) {
      double* dqi = dq_rows + n * E;
      for (int64_t e = 0; e < E; ++e) dqi[e] = 0.0;
      if (sp == NULL || p == NULL || dp == NULL) continue;
      const int64_t r = rows[n], bh = r / L, i = r % L, b = bh / H;
      const double* qi = q + r * E;
      const double* doi = dout + r * E;
      const double* kh = k + bh * S * E;
      const double* vh = v + bh * S * E;
      const double m = row_scores(qi, kh, L, S, E, i, kind, window, doc, dense, softcap, scale,
                                  key_start ? key_start[b] : 0, key_end ? key_end[b] : S, sp);
      if (m == -INFINITY) continue;
      double l = 0.0, D = 0.0;
      for (int64_t j = 0; j < S; ++j) {
        p[j] = exp(sp[j] - m);
        l += p[j];
      }
      for (int64_t j = 0; j < S; ++j) {
        p[j] /= l;
        double t = 0.0;
        for (int64_t e = 0; e < E; ++e) t += doi[e] * vh[j * E + e];
        dp[j] = t;
        D += p[j] * t;
      }
      for (int64_t j = 0; j < S; ++j) {
        if (p[j] == 0.0) continue;
        const double ds = dscore(p[j], dp[j], D, sp[j], softcap, scale);
        for (int64_t e = 0; e < E; ++e) dqi[e] += ds * kh[j * E + e];
      }
    }
    free(sp), free(p), free(dp);
  }
  return failed ? -1 : 0;
}
