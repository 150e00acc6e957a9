/*
 * MSA reference oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU definition of MiniMax Sparse Attention
 * (MSA) decode and chunked prefill, used to check the HIP kernels.  It shares
 * no code with them.  Only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark may load it; the product path never does.
 *
 * What it computes follows "MiniMax wird dünn: M3-Attention anhand eines
 * einzigen Diagramms entschlüsselt" (atlascloud.ai), section 1 "Was das
 * Diagramm zeigt":
 *   Step 1 "Index-Branch": each GQA group owns index queries; one single-head
 *     index key is shared by all groups; token scores are Q_idx . K_idx^T;
 *     "Block Max Pool" keeps the top score per fixed-size block; TopK keeps
 *     the k best blocks per group (index lists I_1, I_2, ...).
 *   Step 2 "Sparse-Branch": every query head of a group attends, with plain
 *     softmax attention, to the real keys/values of its group's kept blocks
 *     only (Q1-Q3 use I_1, Q4-Q6 use I_2).
 * and the traeai.com summary of the M3 live session (highlight 1): the KV
 * cache stays real and uncompressed, selection is block-level, top-K small.
 *
 * The formulas on that page were lost; the readings taken here are:
 *   - the index score is the raw dot product, no scale or activation;
 *   - several index heads of a group are pooled by max, together with the
 *     tokens of the block (and, in prefill, the queries of the tile);
 *   - k counts the current ("own") block, which is always kept and not
 *     scored; only blocks strictly before it are eligible (causal limit);
 *   - blocks are ranked by (score descending, block index ascending);
 *   - query head j belongs to group j / (Hq / Hkv);
 *   - the index lists are returned sorted ascending, padded with -1;
 *   - optional per-group index keys (num_idx_k_heads = Hkv, the ablation of
 *     the single shared index-key head): group g scores its blocks against
 *     its own index-key head g; 0 or 1 means the one shared head;
 *   - optional forced blocks (section 2: the dropped sliding-window branch is
 *     probably replaced by an attention sink or local attention): the first
 *     sink_blocks blocks and the local_blocks blocks just before the own
 *     block are always kept and not ranked; they count toward k, so TopK
 *     chooses k-1-(number forced) of the remaining eligible blocks.
 *
 * Arithmetic: every bfloat16 input is widened exactly to double; products,
 * sums, exp and the softmax are double.  OpenMP runs independent units
 * (one block score, one selection, one query head) in parallel; each unit is
 * a plain loop in the order of the definition.
 *
 * Paged cache layout (page = one block of B tokens):
 *   k      [num_pages][Hkv][B][D]      keys, token-major
 *   v      [num_pages][Hkv][B][D]      values, token-major
 *   idx_k  [num_pages][Hk][B][d_i]     index keys, Hk = 1 (the single shared
 *                                      head) or Hkv (one head per group)
 *   block_table [batch][max_blocks]    logical block -> physical page
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

typedef struct {
  int32_t num_q_heads, num_kv_heads, head_dim;
  int32_t num_idx_heads, idx_dim;
  int32_t block_size, top_k;
  double softmax_scale;
  int32_t sink_blocks, local_blocks;  /* forced blocks (0, 0: none) */
  int32_t num_idx_k_heads;            /* 0 or 1: one shared head; Hkv: one per group */
} oracle_params;

typedef struct {
  const uint16_t *k, *v, *idx_k;
  const int32_t *block_table;
  int32_t num_pages, max_blocks;
} oracle_cache;

/* bfloat16 bits -> double, exact. */
static double bf(uint16_t h) {
  union { uint32_t u; float f; } x;
  x.u = (uint32_t)h << 16;
  return (double)x.f;
}

static int64_t page_of(const oracle_cache *c, int32_t seq, int64_t t, int32_t B) {
  return (int64_t)c->block_table[(int64_t)seq * c->max_blocks + t / B];
}

static double key_at(const oracle_params *p, const oracle_cache *c, int32_t seq,
                     int32_t g, int64_t t, int32_t d) {
  const int32_t B = p->block_size, D = p->head_dim, H = p->num_kv_heads;
  int64_t pg = page_of(c, seq, t, B);
  return bf(c->k[((pg * H + g) * B + t % B) * D + d]);
}

static double value_at(const oracle_params *p, const oracle_cache *c, int32_t seq,
                       int32_t g, int64_t t, int32_t d) {
  const int32_t B = p->block_size, D = p->head_dim, H = p->num_kv_heads;
  int64_t pg = page_of(c, seq, t, B);
  return bf(c->v[((pg * H + g) * B + t % B) * D + d]);
}

static int32_t idx_k_heads(const oracle_params *p) {
  return p->num_idx_k_heads > 1 ? p->num_idx_k_heads : 1;
}

static double index_key_at(const oracle_params *p, const oracle_cache *c,
                           int32_t seq, int32_t g, int64_t t, int32_t d) {
  const int32_t B = p->block_size, di = p->idx_dim, Hk = idx_k_heads(p);
  const int32_t head = Hk > 1 ? g : 0;
  int64_t pg = page_of(c, seq, t, B);
  return bf(c->idx_k[((pg * Hk + head) * B + t % B) * di + d]);
}

/*
 * Step 1 for one block: the largest index score Q_idx . K_idx^T over the index
 * heads of group g, the tokens of block b, and the query rows given
 * (queries [q0, q1) of idx_q, laid out [query][Hkv][n_i][d_i]).
 */
static double block_score(const oracle_params *p, const oracle_cache *c,
                          int32_t seq, const uint16_t *idx_q, int64_t q0,
                          int64_t q1, int32_t g, int64_t b) {
  const int32_t B = p->block_size, di = p->idx_dim, ni = p->num_idx_heads;
  const int32_t H = p->num_kv_heads;
  const int64_t nrows = (q1 - q0) * ni;
  /* widen the block's index keys and the query rows once */
  double *key = (double *)malloc(sizeof(double) * (size_t)B * di);
  double *qry = (double *)malloc(sizeof(double) * (size_t)(nrows > 0 ? nrows : 1) * di);
  for (int32_t r = 0; r < B; r++)
    for (int32_t d = 0; d < di; d++) key[r * di + d] = index_key_at(p, c, seq, g, b * B + r, d);
  for (int64_t i = q0; i < q1; i++)
    for (int32_t h = 0; h < ni; h++)
      for (int32_t d = 0; d < di; d++)
        qry[((i - q0) * ni + h) * di + d] = bf(idx_q[((i * H + g) * ni + h) * di + d]);
  double best = -INFINITY;
  for (int32_t r = 0; r < B; r++) {
    for (int64_t row = 0; row < nrows; row++) {
      double dot = 0.0;
      for (int32_t d = 0; d < di; d++) dot += qry[row * di + d] * key[r * di + d];
      if (dot > best) best = dot;
    }
  }
  free(key);
  free(qry);
  return best;
}

/*
 * TopK: the forced blocks among 0..own-1 (the first n_sink and the last
 * n_local before the own block) are kept unranked; of the other blocks before
 * the own block, keep k' = min(k-1-forced, how many there are), ranked by
 * (score descending, index ascending); plus the own block; sorted ascending,
 * padded with -1 up to k entries.  Chosen by repeated arg-max, the plainest
 * statement of "keep the k highest-scored".  Without forced blocks
 * k' = min(k-1, own).
 */
static void select_blocks(const double *score, int32_t own, int32_t k, int32_t n_sink,
                          int32_t n_local, int32_t *sel) {
  char *taken = (char *)calloc((size_t)(own > 0 ? own : 1), 1);
  int32_t n = 0, eligible = 0;
  for (int32_t b = 0; b < own; b++) {
    if (b < n_sink || b >= own - n_local) {
      taken[b] = 1;  /* forced: kept, never ranked */
      sel[n++] = b;
    } else {
      eligible++;
    }
  }
  int32_t kk = k - 1 - n;
  if (kk > eligible) kk = eligible;
  for (int32_t r = 0; r < kk; r++) {
    int32_t best = -1;
    for (int32_t b = 0; b < own; b++) {
      if (taken[b]) continue;
      if (best < 0 || score[b] > score[best]) best = b;  /* ties: lower index stays */
    }
    taken[best] = 1;
    sel[n++] = best;
  }
  free(taken);
  sel[n++] = own;
  for (int32_t i = 1; i < n; i++) {  /* insertion sort, ascending */
    int32_t x = sel[i], j = i - 1;
    while (j >= 0 && sel[j] > x) { sel[j + 1] = sel[j]; j--; }
    sel[j + 1] = x;
  }
  for (int32_t i = n; i < k; i++) sel[i] = -1;
}

/*
 * Step 2 for one query head: softmax(scale * q . K_t) weighted sum of V_t over
 * the tokens t of the kept blocks of group g with t <= last_pos.
 */
static void attend(const oracle_params *p, const oracle_cache *c, int32_t seq,
                   int32_t g, const uint16_t *qvec, const int32_t *sel,
                   int64_t last_pos, double *out) {
  const int32_t B = p->block_size, D = p->head_dim, k = p->top_k;
  int64_t ntok = 0;
  for (int32_t i = 0; i < k; i++) {
    if (sel[i] < 0) continue;
    int64_t lo = (int64_t)sel[i] * B, hi = lo + B;
    if (hi > last_pos + 1) hi = last_pos + 1;
    if (hi > lo) ntok += hi - lo;
  }
  int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)(ntok > 0 ? ntok : 1));
  double *z = (double *)malloc(sizeof(double) * (size_t)(ntok > 0 ? ntok : 1));
  int64_t n = 0;
  for (int32_t i = 0; i < k; i++) {
    if (sel[i] < 0) continue;
    int64_t lo = (int64_t)sel[i] * B, hi = lo + B;
    if (hi > last_pos + 1) hi = last_pos + 1;
    for (int64_t t = lo; t < hi; t++) tok[n++] = t;
  }
  double zmax = -INFINITY;
  for (int64_t i = 0; i < n; i++) {
    double dot = 0.0;
    for (int32_t d = 0; d < D; d++)
      dot += bf(qvec[d]) * key_at(p, c, seq, g, tok[i], d);
    z[i] = p->softmax_scale * dot;
    if (z[i] > zmax) zmax = z[i];
  }
  double den = 0.0;
  for (int64_t i = 0; i < n; i++) { z[i] = exp(z[i] - zmax); den += z[i]; }
  for (int32_t d = 0; d < D; d++) {
    double acc = 0.0;
    for (int64_t i = 0; i < n; i++) acc += z[i] * value_at(p, c, seq, g, tok[i], d);
    out[d] = acc / den;
  }
  free(tok);
  free(z);
}

static int check(const oracle_params *p, const oracle_cache *c) {
  if (!p || !c || !c->k || !c->v || !c->idx_k || !c->block_table) return -1;
  if (p->num_kv_heads < 1 || p->num_q_heads % p->num_kv_heads) return -1;
  if (p->block_size < 1 || p->top_k < 1 || p->head_dim < 1 || p->idx_dim < 1 ||
      p->num_idx_heads < 1)
    return -1;
  if (p->sink_blocks < 0 || p->local_blocks < 0 || p->sink_blocks + p->local_blocks > p->top_k - 1)
    return -1;
  if (p->num_idx_k_heads > 1 && p->num_idx_k_heads != p->num_kv_heads) return -1;
  return 0;
}

/*
 * Step 2 of decode for every query head of every sequence: head j of
 * sequence s attends to the tokens t <= seq_lens[s]-1 of the blocks listed in
 * sel[s][j / G] (the selection of its group).
 */
static void attend_decode_heads(const oracle_params *p, const oracle_cache *c,
                                const uint16_t *q, const int32_t *seq_lens, int32_t batch,
                                const int32_t *sel, double *out) {
  const int32_t H = p->num_kv_heads, Hq = p->num_q_heads, G = Hq / H;
  const int32_t D = p->head_dim, k = p->top_k;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int32_t s = 0; s < batch; s++)
    for (int32_t j = 0; j < Hq; j++) {
      int32_t g = j / G;
      attend(p, c, s, g, q + ((int64_t)s * Hq + j) * D, sel + ((int64_t)s * H + g) * k,
             (int64_t)seq_lens[s] - 1, out + ((int64_t)s * Hq + j) * D);
    }
}

int msa_oracle_max_threads(void) { return omp_get_max_threads(); }

/* Exported for the tests: the TopK rule on a given score vector. */
int msa_oracle_select(const double *score, int32_t own, int32_t k, int32_t *sel) {
  if (!sel || k < 1 || own < 0 || (own > 0 && !score)) return -1;
  select_blocks(score, own, k, 0, 0, sel);
  return 0;
}

/* The same with forced sink and local blocks. */
int msa_oracle_select_forced(const double *score, int32_t own, int32_t k, int32_t n_sink,
                             int32_t n_local, int32_t *sel) {
  if (!sel || k < 1 || own < 0 || (own > 0 && !score)) return -1;
  if (n_sink < 0 || n_local < 0 || n_sink + n_local > k - 1) return -1;
  select_blocks(score, own, k, n_sink, n_local, sel);
  return 0;
}

/*
 * Decode.  Sequence s holds seq_lens[s] tokens in the cache, the last of which
 * is the current token (its K/V/index key already appended).  Own block
 * c = (L-1)/B.
 *   q      [batch][Hq][D]            idx_q [batch][Hkv][n_i][d_i]
 *   out    [batch][Hq][D]            sel   [batch][Hkv][k]
 *   pooled [batch][Hkv][max_blocks]  (optional; -inf where not scored)
 */
int msa_oracle_decode(const oracle_params *p, const oracle_cache *c,
                      const uint16_t *q, const uint16_t *idx_q,
                      const int32_t *seq_lens, int32_t batch, double *out,
                      int32_t *sel, double *pooled) {
  if (check(p, c) || !q || !idx_q || !seq_lens || !out || !sel || batch < 1) return -1;
  const int32_t B = p->block_size, H = p->num_kv_heads;
  const int32_t k = p->top_k, MB = c->max_blocks;
  for (int32_t s = 0; s < batch; s++)
    if (seq_lens[s] < 1 || (int64_t)seq_lens[s] > (int64_t)MB * B) return -1;

  double *score = (double *)malloc(sizeof(double) * (size_t)batch * H * MB);
  for (int64_t i = 0; i < (int64_t)batch * H * MB; i++) score[i] = -INFINITY;

  /* Step 1: one block score per (sequence, group, eligible block). */
#pragma omp parallel for collapse(3) schedule(dynamic, 64)
  for (int32_t s = 0; s < batch; s++)
    for (int32_t g = 0; g < H; g++)
      for (int32_t b = 0; b < MB; b++) {
        int32_t own = (seq_lens[s] - 1) / B;
        if (b < own)
          score[((int64_t)s * H + g) * MB + b] =
              block_score(p, c, s, idx_q + (int64_t)s * H * p->num_idx_heads * p->idx_dim,
                          0, 1, g, b);
      }

  /* TopK per (sequence, group). */
  for (int32_t s = 0; s < batch; s++)
    for (int32_t g = 0; g < H; g++)
      select_blocks(score + ((int64_t)s * H + g) * MB, (seq_lens[s] - 1) / B, k,
                    p->sink_blocks, p->local_blocks, sel + ((int64_t)s * H + g) * k);

  /* Step 2 per query head. */
  attend_decode_heads(p, c, q, seq_lens, batch, sel, out);

  if (pooled) memcpy(pooled, score, sizeof(double) * (size_t)batch * H * MB);
  free(score);
  return 0;
}

/* Step 2 only, for a given selection (decode layout). */
int msa_oracle_attend_decode(const oracle_params *p, const oracle_cache *c,
                             const uint16_t *q, const int32_t *seq_lens,
                             int32_t batch, const int32_t *sel, double *out) {
  if (check(p, c) || !q || !seq_lens || !sel || !out || batch < 1) return -1;
  attend_decode_heads(p, c, q, seq_lens, batch, sel, out);
  return 0;
}

/*
 * Chunked prefill of one sequence: chunk_len new queries at positions
 * prior_len .. prior_len+chunk_len-1 (their keys are in the cache).  Tile tau
 * is the set of chunk queries inside absolute block c_tau = prior_len/B + tau;
 * it is scored and selected as one unit (its queries pooled like index heads)
 * with c_tau as its own block, and query i attends to tokens t <= prior_len+i
 * of the kept blocks.
 *   tiles: list of tile ids to compute (NULL = all); rows of other tiles in
 *          out/sel/pooled are left untouched.
 *   q [C][Hq][D], idx_q [C][Hkv][n_i][d_i], out [C][Hq][D],
 *   sel [num_tiles][Hkv][k], pooled [num_tiles][Hkv][max_blocks] (optional).
 */
static int prefill_impl(const oracle_params *p, const oracle_cache *c,
                        const uint16_t *q, const uint16_t *idx_q,
                        int32_t prior_len, int32_t chunk_len,
                        const int32_t *tiles, int32_t n_tiles, double *out,
                        int32_t *sel, const int32_t *given_sel, double *pooled) {
  if (check(p, c) || !q || !out || prior_len < 0 || chunk_len < 1) return -1;
  if (!given_sel && (!idx_q || !sel)) return -1;
  const int32_t B = p->block_size, H = p->num_kv_heads, Hq = p->num_q_heads;
  const int32_t G = Hq / H, D = p->head_dim, k = p->top_k, MB = c->max_blocks;
  const int64_t total = (int64_t)prior_len + chunk_len;
  if (total > (int64_t)MB * B) return -1;
  const int32_t first = prior_len / B;
  const int32_t num_tiles = (int32_t)((total + B - 1) / B) - first;
  int32_t nt = tiles ? n_tiles : num_tiles;
  int32_t *list = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nt > 0 ? nt : 1));
  for (int32_t i = 0; i < nt; i++) {
    list[i] = tiles ? tiles[i] : i;
    if (list[i] < 0 || list[i] >= num_tiles) { free(list); return -1; }
  }
  const int32_t *use_sel = given_sel;
  if (!given_sel) {
    double *score = (double *)malloc(sizeof(double) * (size_t)nt * H * MB);
    for (int64_t i = 0; i < (int64_t)nt * H * MB; i++) score[i] = -INFINITY;
#pragma omp parallel for collapse(3) schedule(dynamic, 16)
    for (int32_t u = 0; u < nt; u++)
      for (int32_t g = 0; g < H; g++)
        for (int32_t b = 0; b < MB; b++) {
          int32_t own = first + list[u];
          if (b >= own) continue;
          int64_t q0 = (int64_t)own * B - prior_len, q1 = q0 + B;
          if (q0 < 0) q0 = 0;
          if (q1 > chunk_len) q1 = chunk_len;
          score[((int64_t)u * H + g) * MB + b] = block_score(p, c, 0, idx_q, q0, q1, g, b);
        }
    for (int32_t u = 0; u < nt; u++)
      for (int32_t g = 0; g < H; g++) {
        select_blocks(score + ((int64_t)u * H + g) * MB, first + list[u], k, p->sink_blocks,
                      p->local_blocks, sel + ((int64_t)list[u] * H + g) * k);
        if (pooled)
          memcpy(pooled + ((int64_t)list[u] * H + g) * MB, score + ((int64_t)u * H + g) * MB,
                 sizeof(double) * (size_t)MB);
      }
    free(score);
    use_sel = sel;
  }
  /* Step 2 per (query of a listed tile, head). */
  int64_t nq = 0;
  for (int32_t u = 0; u < nt; u++) {
    int64_t q0 = (int64_t)(first + list[u]) * B - prior_len, q1 = q0 + B;
    if (q0 < 0) q0 = 0;
    if (q1 > chunk_len) q1 = chunk_len;
    nq += q1 - q0;
  }
  int64_t *qi = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nq > 0 ? nq : 1));
  int32_t *qt = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nq > 0 ? nq : 1));
  int64_t n = 0;
  for (int32_t u = 0; u < nt; u++) {
    int64_t q0 = (int64_t)(first + list[u]) * B - prior_len, q1 = q0 + B;
    if (q0 < 0) q0 = 0;
    if (q1 > chunk_len) q1 = chunk_len;
    for (int64_t i = q0; i < q1; i++) { qi[n] = i; qt[n] = list[u]; n++; }
  }
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
  for (int64_t r = 0; r < nq; r++)
    for (int32_t j = 0; j < Hq; j++) {
      int32_t g = j / G;
      attend(p, c, 0, g, q + (qi[r] * Hq + j) * D, use_sel + ((int64_t)qt[r] * H + g) * k,
             (int64_t)prior_len + qi[r], out + (qi[r] * Hq + j) * D);
    }
  free(qi);
  free(qt);
  free(list);
  return 0;
}

int msa_oracle_prefill(const oracle_params *p, const oracle_cache *c,
                       const uint16_t *q, const uint16_t *idx_q,
                       int32_t prior_len, int32_t chunk_len,
                       const int32_t *tiles, int32_t n_tiles, double *out,
                       int32_t *sel, double *pooled) {
  return prefill_impl(p, c, q, idx_q, prior_len, chunk_len, tiles, n_tiles, out,
                      sel, NULL, pooled);
}

/* Step 2 only, for a given selection sel [num_tiles][Hkv][k] (prefill). */
int msa_oracle_attend_prefill(const oracle_params *p, const oracle_cache *c,
                              const uint16_t *q, int32_t prior_len,
                              int32_t chunk_len, const int32_t *tiles,
                              int32_t n_tiles, const int32_t *sel, double *out) {
  if (!sel) return -1;
  return prefill_impl(p, c, q, NULL, prior_len, chunk_len, tiles, n_tiles, out,
                      NULL, sel, NULL);
}

/*
 * Step 1 for listed blocks only: out[i] = block score of blocks[i] for group g
 * of sequence seq, pooled over the query rows [q0, q1) of idx_q
 * ([query][Hkv][n_i][d_i]; decode: the sequence's own row, q0 = 0, q1 = 1).
 * Lets tests check single pooled scores of very long contexts.
 */
int msa_oracle_block_scores(const oracle_params *p, const oracle_cache *c, int32_t seq,
                            const uint16_t *idx_q, int32_t q0, int32_t q1, int32_t g,
                            const int32_t *blocks, int32_t n, double *out) {
  if (check(p, c) || !idx_q || !blocks || !out || q0 < 0 || q1 <= q0 || g < 0 ||
      g >= p->num_kv_heads || n < 0)
    return -1;
  for (int32_t i = 0; i < n; i++)
    if (blocks[i] < 0 || blocks[i] >= c->max_blocks) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t i = 0; i < n; i++)
    out[i] = block_score(p, c, seq, idx_q, q0, q1, g, blocks[i]);
  return 0;
}

/*
 * Cache append: the step before Step 1.  Every token brings its key and value
 * per KV head and its one index key (the index-key side has a single head,
 * section 1 "Schritt 1"; the real K/V are kept, section 2).  Token i of
 * sequence s sits at position t = start[s] + i and is stored in page
 * block_table[s][t / B], slot t % B, in the layouts above:
 *   k_new, v_new [batch][n_new][Hkv][D], idx_new [batch][n_new][Hk][d_i]
 *   (Hk index-key heads, 1 for the shared head).
 * The cache arrays are written in place; nothing else changes.
 */
int msa_oracle_append(const oracle_params *p, uint16_t *k, uint16_t *v, uint16_t *idx_k,
                      const int32_t *block_table, int32_t max_blocks, const uint16_t *k_new,
                      const uint16_t *v_new, const uint16_t *idx_new, const int32_t *start,
                      int32_t batch, int32_t n_new) {
  const int32_t B = p->block_size, D = p->head_dim, H = p->num_kv_heads, di = p->idx_dim;
  const int32_t Hk = idx_k_heads(p);
  if (batch < 1 || n_new < 1 || B < 1) return -1;
  for (int32_t s = 0; s < batch; ++s) {
    for (int32_t i = 0; i < n_new; ++i) {
      const int64_t t = (int64_t)start[s] + i;
      if (t < 0 || t >= (int64_t)max_blocks * B) return -1;
      const int64_t pg = block_table[(int64_t)s * max_blocks + t / B];
      const int64_t slot = t % B;
      const int64_t src = (int64_t)s * n_new + i;
      for (int32_t g = 0; g < H; ++g) {
        for (int32_t d = 0; d < D; ++d) {
          k[((pg * H + g) * B + slot) * D + d] = k_new[(src * H + g) * D + d];
          v[((pg * H + g) * B + slot) * D + d] = v_new[(src * H + g) * D + d];
        }
      }
      for (int32_t h = 0; h < Hk; ++h)
        for (int32_t d = 0; d < di; ++d)
          idx_k[((pg * Hk + h) * B + slot) * di + d] = idx_new[(src * Hk + h) * di + d];
    }
  }
  return 0;
}
