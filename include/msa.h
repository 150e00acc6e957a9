/*
 * msa.h -- C ABI of libmsa.so: MiniMax Sparse Attention (MSA) decode and
 * chunked prefill on AMD Instinct MI355X (gfx950).
 *
 * The operation is the attention block of "MiniMax wird dünn:
 * M3-Attention anhand eines einzigen Diagramms entschlüsselt"
 * (atlascloud.ai), section 1 "Was das Diagramm zeigt":
 *   Step 1 (index branch): each GQA group has index queries; a single index-key
 *     head is shared by every group; token scores are Q_idx . K_idx^T; "Block
 *     Max Pool" keeps the largest score of each fixed-size block; TopK keeps
 *     the k best blocks per group (index lists I_1, I_2, ...).
 *   Step 2 (sparse branch): every query head of a group runs plain softmax
 *     attention over the real, uncompressed keys/values of its group's kept
 *     blocks only (traeai.com summary of the M3 live session, highlight 1).
 * Parameters the page leaves open are fixed as follows: the index score is the
 * raw dot product; the index heads of a group (and, in prefill, the queries of
 * a tile) are pooled by max together with the block's tokens; k counts the
 * current block, which is always kept and never scored; only blocks before it
 * are eligible; ranking is by (score descending, block index ascending); query
 * head j belongs to group j / (num_q_heads / num_kv_heads).
 * Forced blocks (section 2 of the same page: NSA's sliding-window branch is
 * dropped, probably in favour of an attention sink or local attention): the
 * first sink_blocks blocks and the local_blocks blocks just before the own
 * block are always kept and never ranked; they count toward top_k, so TopK
 * chooses top_k - 1 - (number forced) of the other blocks before the own one.
 * sink_blocks = local_blocks = 0 is the plain method.
 * Per-group index keys (num_idx_k_heads = num_kv_heads) replace the page's
 * single shared index-key head by one head per KV group, each group scoring
 * against its own: an ablation of "K_idx hat nur einen Head"; the index
 * cache is then [num_pages][Hkv][B][d_i] and appended index keys carry Hkv
 * heads ([..][Hkv][d_i]).
 *
 * Conventions for every entry point
 * ---------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller; nothing is
 *   copied between host and device, nothing is allocated, the library keeps
 *   no pointer after returning, and no call synchronises.  Work is enqueued
 *   on `stream` (a hipStream_t; NULL = the default stream) in order.
 * - bf16 = IEEE bfloat16 stored as uint16; f32 = IEEE binary32.
 * - Arguments are validated on the host before anything is launched; a
 *   rejected call launches nothing and returns a negative msa_status;
 *   msa_last_error() then describes it (thread-local).  A failed launch
 *   returns MSA_ERR_HIP.  No C++ exception crosses this interface.
 * - Device-side data errors (a block-table entry outside [0, num_pages), a
 *   seq_len larger than max_blocks_per_seq * block_size) are not detected
 *   and give undefined results.
 * - Supported set: head_dim 128, idx_dim 64, block_size 64 or 128,
 *   1 <= top_k <= 64, num_idx_heads in {1, 2, 4, 8, 16},
 *   num_kv_heads * num_idx_heads <= 64, group size num_q_heads/num_kv_heads
 *   in 1..16.  Other values return MSA_ERR_UNSUPPORTED.  sink_blocks and
 *   local_blocks must be >= 0 with sink_blocks + local_blocks <= top_k - 1
 *   (else MSA_ERR_INVALID_ARGUMENT); num_idx_k_heads must be 0, 1 or
 *   num_kv_heads (else MSA_ERR_UNSUPPORTED).  The prefill calls also need
 *   block_size * num_idx_heads <= 512 (one tile's query x index-head rows in
 *   one workgroup), else MSA_ERR_UNSUPPORTED.
 *
 * Paged KV cache (one page holds one KV block of block_size tokens)
 * -----------------------------------------------------------------
 *   k      bf16 [num_pages][Hkv][B][D]   keys, token-major within a page
 *   v      bf16 [num_pages][Hkv][B][D]   values, token-major within a page
 *   idx_k  bf16 [num_pages][B][d_i]      the single shared index-key head
 *          ([num_pages][Hkv][B][d_i] with per-group index keys)
 *   block_table int32 [batch][max_blocks_per_seq]: logical block b of
 *          sequence s lives in page block_table[s*max_blocks_per_seq + b]
 * The caller has already written the current token's (decode) or the
 * chunk's (prefill) keys, values and index keys into the cache, for example
 * with msa_cache_append (msa_decode_append does it in the same pass).
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARGUMENT = -1, /* null pointer, inconsistent sizes      */
  MSA_ERR_UNSUPPORTED = -2,      /* valid but outside the supported set    */
  MSA_ERR_WORKSPACE = -3,        /* workspace missing or too small         */
  MSA_ERR_HIP = -4               /* a HIP launch or runtime call failed    */
} msa_status;

typedef struct {
  int32_t num_q_heads;   /* Hq                                            */
  int32_t num_kv_heads;  /* Hkv = number of GQA groups                    */
  int32_t head_dim;      /* D                                             */
  int32_t num_idx_heads; /* n_i index queries per group                   */
  int32_t idx_dim;       /* d_i                                           */
  int32_t block_size;    /* B tokens per block (= page)                   */
  int32_t top_k;         /* k kept blocks per group, own block included   */
  float softmax_scale;   /* applied to attention scores only, e.g. 1/sqrt(D) */
  int32_t sink_blocks;   /* blocks 0..sink_blocks-1 always kept (0: none)   */
  int32_t local_blocks;  /* the local_blocks blocks just before the own block
                            always kept (0: none)                          */
  int32_t num_idx_k_heads; /* index-key heads: 0 or 1 = the single shared head;
                              num_kv_heads = one per group (ablation)       */
} msa_params;

typedef struct {
  const void *k;              /* bf16 [num_pages][Hkv][B][D]  */
  const void *v;              /* bf16 [num_pages][Hkv][B][D]  */
  const void *idx_k;          /* bf16 [num_pages][B][d_i]     */
  const int32_t *block_table; /* int32 [batch][max_blocks_per_seq] */
  int32_t num_pages;
  int32_t max_blocks_per_seq;
} msa_paged_kv;

/* The same cache, writable: used by the calls that append tokens.  Layouts
 * and meaning as in msa_paged_kv. */
typedef struct {
  void *k;                    /* bf16 [num_pages][Hkv][B][D]  */
  void *v;                    /* bf16 [num_pages][Hkv][B][D]  */
  void *idx_k;                /* bf16 [num_pages][B][d_i]     */
  const int32_t *block_table; /* int32 [batch][max_blocks_per_seq] */
  int32_t num_pages;
  int32_t max_blocks_per_seq;
} msa_paged_kv_mut;

/* ------------------------------------------------------------ cache append
 * The step before the index branch: the keys, values and index keys of new
 * tokens are written into their pages ("MiniMax wird dünn", section 1,
 * Schritt 1: one index key per token, a single shared index-key head;
 * section 2: the real, uncompressed K/V stay in the cache).
 * Sequence s receives n_new >= 1 consecutive tokens at positions
 * start_pos[s] .. start_pos[s]+n_new-1 (token t goes to page
 * block_table[s][t/B], slot t%B, row t%B of the page's K and V).
 *   k_new     bf16 [batch][n_new][Hkv][D]
 *   v_new     bf16 [batch][n_new][Hkv][D]
 *   idx_k_new bf16 [batch][n_new][d_i]
 *   start_pos int32 [batch]  (device)
 * Only the slots of the new tokens are written.  Pages written for one
 * sequence must not be shared with another sequence in the same call.
 * Positions beyond max_blocks_per_seq*B are a device-side data error. */
msa_status msa_cache_append(const msa_params *params, const msa_paged_kv_mut *kv,
                            const void *k_new, const void *v_new,
                            const void *idx_k_new, const int32_t *start_pos,
                            int32_t batch, int32_t n_new, void *stream);

/* ------------------------------------------------------------------ decode
 * One decode step for a batch of sequences (Step 1 + TopK + Step 2).
 * Sequence s holds seq_lens[s] >= 1 tokens, the last being the current one;
 * its own block is c = (seq_lens[s]-1)/B; blocks 0..c-1 are scored.
 *   q        bf16 [batch][Hq][D]
 *   idx_q    bf16 [batch][Hkv][n_i][d_i]
 *   seq_lens int32 [batch]            (device)
 *   max_seq_len  host upper bound of seq_lens (sizes the launch grid; a
 *                smaller bound than a real length gives wrong results)
 *   out      f32 [batch][Hq][D]
 *   sel      int32 [batch][Hkv][top_k] or NULL: kept blocks, ascending,
 *            padded with -1
 *   workspace  device memory of at least msa_decode_workspace_bytes(); its
 *              contents on entry do not matter.  Calls that overlap in time
 *              must not share a workspace.
 */
size_t msa_decode_workspace_bytes(const msa_params *params, int32_t batch,
                                  int32_t max_blocks_per_seq);

msa_status msa_decode(const msa_params *params, const msa_paged_kv *kv,
                      const void *q, const void *idx_q, const int32_t *seq_lens,
                      int32_t batch, int32_t max_seq_len, float *out,
                      int32_t *sel, void *workspace, size_t workspace_bytes,
                      void *stream);

/* msa_decode with the current token's append fused in: the launch that
 * scores the index keys also writes each sequence's current token (position
 * seq_lens[s]-1) into its own block, which that launch never reads, before
 * the sparse branch reads it.  Same arguments and results as msa_decode on
 * a cache that already holds the token, plus
 *   k_new, v_new  bf16 [batch][Hkv][D]   (the current token's key and value)
 *   idx_k_new     bf16 [batch][d_i]      (its index key)
 * The cache's slots of the current tokens are written. */
msa_status msa_decode_append(const msa_params *params, const msa_paged_kv_mut *kv,
                             const void *k_new, const void *v_new,
                             const void *idx_k_new, const void *q,
                             const void *idx_q, const int32_t *seq_lens,
                             int32_t batch, int32_t max_seq_len, float *out,
                             int32_t *sel, void *workspace,
                             size_t workspace_bytes, void *stream);

/* msa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments and results as msa_decode, without the workspace: the kernels'
 * scratch is a static 32 MiB array of the library, one per GPU, held until
 * the process ends (its device address is looked up on the first call on
 * each device).  A call whose msa_decode_workspace_bytes() would exceed
 * 32 MiB returns MSA_ERR_WORKSPACE (at 64/8 heads and top_k 16 the 1M-token
 * single-sequence decode needs 0.8 MiB, 32 sequences of up to 512K tokens
 * 20.5 MiB).  Calls on one GPU share the array: calls that overlap in time
 * on one GPU race. */
msa_status msa_decode_noalloc(const msa_params *params, const msa_paged_kv *kv,
                              const void *q, const void *idx_q,
                              const int32_t *seq_lens, int32_t batch,
                              int32_t max_seq_len, float *out, int32_t *sel,
                              void *stream);

/* Step 1 of decode alone (index scores + block max pool):
 *   pooled f32 [batch][Hkv][max_blocks_per_seq]; entries b < c are written,
 *   the others are left untouched. */
msa_status msa_index_score_decode(const msa_params *params,
                                  const msa_paged_kv *kv, const void *idx_q,
                                  const int32_t *seq_lens, int32_t batch,
                                  int32_t max_seq_len, float *pooled,
                                  void *stream);

/* ----------------------------------------------------------------- prefill
 * One chunk of a single sequence: chunk_len >= 1 new queries at positions
 * prior_len .. prior_len+chunk_len-1 (their K/V/index keys already cached).
 * Tile t is the set of chunk queries inside absolute block
 * c_t = prior_len/B + t, for t in [0, num_tiles) with
 * num_tiles = ceil((prior_len+chunk_len)/B) - prior_len/B.  A tile is scored
 * as one unit (its queries pooled like index heads) with c_t as its own
 * block; query i attends to tokens <= prior_len + i of its tile's kept blocks.
 *   q      bf16 [chunk_len][Hq][D]
 *   idx_q  bf16 [chunk_len][Hkv][n_i][d_i]
 *   out    f32 [chunk_len][Hq][D]
 *   sel    int32 [num_tiles][Hkv][top_k] or NULL (ascending, -1 padded)
 * block_table row 0 is used; it must cover prior_len+chunk_len tokens.
 * Precision: every output row is within 2e-3 (max |error| / max |value| of
 * the row) of exact softmax attention over the kept blocks.  The sparse
 * attention forms P.V in IEEE half (P rounded to nearest-even half, V
 * converted exactly) when every kept block's largest |v| lies in
 * [2^-8, 2^15] (and is finite); otherwise a second
 * launch recomputes that workgroup's rows with P as two bf16 terms.  That
 * launch finds such workgroups by a NaN the first one leaves in `out`, so
 * `out` must not be read before the call's work on `stream` is done. */
size_t msa_prefill_workspace_bytes(const msa_params *params, int32_t prior_len,
                                   int32_t chunk_len,
                                   int32_t max_blocks_per_seq);

msa_status msa_prefill_chunk(const msa_params *params, const msa_paged_kv *kv,
                             const void *q, const void *idx_q,
                             int32_t prior_len, int32_t chunk_len, float *out,
                             int32_t *sel, void *workspace,
                             size_t workspace_bytes, void *stream);

/* ------------------------------------------------- batched prefill (varlen)
 * Chunks of `batch` sequences in one call, each with its own context: the
 * same computation as msa_prefill_chunk for every sequence s, with prior
 * length prior_lens[s], chunk length chunk_lens[s] and block-table row s.
 * The chunks' rows are packed sequence after sequence: sequence s owns rows
 * q_start[s] .. q_start[s]+chunk_lens[s]-1 of q, idx_q and out, where
 * q_start[s] = chunk_lens[0] + ... + chunk_lens[s-1].  Tiles are numbered the
 * same way (those of sequence 0 first), giving the rows of sel.
 *   q          bf16 [total_rows][Hq][D]
 *   idx_q      bf16 [total_rows][Hkv][n_i][d_i]
 *   prior_lens, chunk_lens       int32 [batch], device
 *   prior_lens_host, chunk_lens_host  int32 [batch], host copies of the
 *              same values (they size the launches; read during the call
 *              only)
 *   out        f32 [total_rows][Hq][D]
 *   sel        int32 [total_tiles][Hkv][top_k] or NULL
 * Each prior_lens[s] >= 0, chunk_lens[s] >= 1, and prior + chunk must fit
 * in max_blocks_per_seq blocks; batch <= 65535. */
size_t msa_prefill_varlen_workspace_bytes(const msa_params *params,
                                          const int32_t *prior_lens_host,
                                          const int32_t *chunk_lens_host,
                                          int32_t batch, int32_t max_blocks_per_seq);

msa_status msa_prefill_varlen(const msa_params *params, const msa_paged_kv *kv,
                              const void *q, const void *idx_q,
                              const int32_t *prior_lens, const int32_t *chunk_lens,
                              const int32_t *prior_lens_host,
                              const int32_t *chunk_lens_host, int32_t batch,
                              float *out, int32_t *sel, void *workspace,
                              size_t workspace_bytes, void *stream);

/* Step 1 of prefill alone: pooled f32 [num_tiles][Hkv][max_blocks_per_seq];
 * entries b < c_t are written, the others are left untouched. */
msa_status msa_index_score_prefill(const msa_params *params,
                                   const msa_paged_kv *kv, const void *idx_q,
                                   int32_t prior_len, int32_t chunk_len,
                                   float *pooled, void *stream);

/* TopK of prefill alone, from pooled scores as written by
 * msa_index_score_prefill: sel int32 [num_tiles][Hkv][top_k]. */
msa_status msa_block_topk_prefill(const msa_params *params,
                                  int32_t prior_len, int32_t chunk_len,
                                  int32_t max_blocks_per_seq,
                                  const float *pooled, int32_t *sel,
                                  void *stream);

/* Step 2 of prefill alone, for a given selection sel [num_tiles][Hkv][top_k]
 * (ascending, -1 padded, every entry <= its tile's own block). */
msa_status msa_sparse_attn_prefill(const msa_params *params,
                                   const msa_paged_kv *kv, const void *q,
                                   int32_t prior_len, int32_t chunk_len,
                                   const int32_t *sel, float *out,
                                   void *stream);

/* Text of the last non-OK status returned on this thread. */
const char *msa_last_error(void);

/* Library version string. */
const char *msa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H_ */
