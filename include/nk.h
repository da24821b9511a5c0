/*
 * nk.h -- ragged paged attention with fused RoPE + KV append, for AMD
 * Instinct MI355X (gfx950).  C ABI of libnk.so.
 *
 * Three operations on the forward path:
 *
 *   nk_rope_qk_write_paged     rotate Q and K with a (cos, sin) table, write
 *                              the rotated Q out and append rotated K and
 *                              plain V to a paged cache (Mojo docs,
 *                              generic_fused_qk_rope_bshd_paged_ragged_kernel_api,
 *                              "Args"; NumKong for Python, matrix-kernels page,
 *                              attention_rope);
 *   nk_ragged_paged_attention  ragged causal (optionally windowed) grouped-query
 *                              scaled-dot-product attention over that cache,
 *                              with a per-row log-sum-exp (NumKong matrix-kernels
 *                              page, "Attention with a Pre-Packed KV-Cache" and
 *                              attention_packed);
 *   nk_attention_lse_merge     merge of partial attention states by their
 *                              log-sum-exp (Algenta "Attention variant kernels",
 *                              "Flash attention's running state reproduces the
 *                              same softmax").
 *
 * Beside them: nk_ragged_paged_attention_band (any band of keys before and
 * after a row, plus attention-sink keys), nk_attention_pack (ragged K/V
 * token rows packed into the paged cache, NumKong attention_pack),
 * nk_ragged_paged_attention_backward (query, key and value gradients,
 * NumKong attention_packed_gradients) and nk_rope_qk_write_paged_mrope
 * (multimodal RoPE sections).
 *
 * Conventions for every call (after the NumKong python page, "GPU Tensors
 * through DLPack": no verb allocates, each GPU call queues its launches on
 * the given stream and returns before they finish):
 *
 *   - Pointers are DEVICE pointers unless the parameter is named *_host or
 *     is the cache descriptor itself (a host struct holding device pointers).
 *     Integer arrays are int32.
 *   - The caller owns every buffer, the workspace and the cache.  The library
 *     never allocates device memory, keeps no state between calls apart from
 *     per-device properties it caches (CU count, resident work-groups of the
 *     prefill kernel) and the optional profiling events below, and may be
 *     called from several host threads at once (profiling excepted).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work; they never synchronise.
 *   - Errors are returned as nk_status_t values, detected on the host before
 *     anything is launched.  There is no CPU fallback: an unsupported
 *     combination returns NK_ERR_UNSUPPORTED.  A failed launch returns
 *     NK_ERR_DEVICE.  Contents of device arrays are preconditions, not
 *     checked (see each call).
 *
 * Paged cache layout (one layer), nk_paged_kv_t:
 *
 *   K pages   [num_pages][num_kv_heads][head_dim/(32*NK)][page_size][32*NK],
 *             NK = 2 for e4m3 and 1 otherwise: within one page and head, K is
 *             stored in blocks of 32*NK dimensions, token after token; a
 *             token's row of a block is 4 runs of NK*8 elements, run g holding
 *             dims 8g..8g+7 of each of the block's NK 32-dim halves: element
 *             (dim d, token t) of a page is at
 *               ((d/(32*NK)) * page_size + t) * 32*NK + ((d%32)/8) * NK*8
 *               + ((d/32)%NK) * 8 + d%8
 *             (for bf16 and f32 simply [head_dim/32][page_size][32]; a run is
 *             what one lane of the 16x16x32 MFMA holds of NK K operands)
 *   V pages   [num_pages][num_kv_heads][page_size/16][head_dim/(16*NV)]
 *             [64][4*NV], NV = 4 / element bytes (f32 1, bf16 2, e4m3 4):
 *             within one page and head, each 16-token block is stored as
 *             runs of 16 bytes.  Run r = 16*g + l of dim group c holds the
 *             4 tokens 4g..4g+3 (of the block) of the dims 16*(c*NV + j) + l,
 *             j = 0..NV-1, dim-major within the run: element (dim d, token t)
 *             of a page is at
 *               ((t/16) * head_dim/(16*NV) + c) * 64 * 4*NV
 *               + (16*((t%16)/4) + d%16) * 4*NV + ((d/16)%NV) * 4 + t%4
 *             with c = (d/16)/NV.  (This is the order in which the 64 lanes
 *             of a wave hold a V^T operand of the 16x16x16 MFMA, so that one
 *             16-byte load per lane fetches NV operands.)
 *   scales    [num_pages][num_kv_heads][page_size] float32, K and V apart,
 *             only for NK_E4M3 caches: the stored code times its scale is the
 *             value
 *   page_table[s][p] (device, [num_seqs][page_table_stride]) is the physical
 *             page of logical slots p*page_size .. p*page_size+page_size-1 of
 *             sequence s.
 *
 * Supported: head_dim 64, 128 or 256; page_size 16 or 32; query heads a
 * multiple of KV heads.  Element types: f32 inputs with an f32 cache; bf16
 * inputs with a bf16 or e4m3 (OCP e4m3fn: bias 7, max 448, no Inf) cache.
 */
#ifndef NK_H_
#define NK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { NK_F32 = 0, NK_BF16 = 1, NK_E4M3 = 2 } nk_dtype_t;

/* NK_ROPE_HALF pairs dim i with dim i + rotary_dim/2 (rotate-half);
 * NK_ROPE_INTERLEAVED pairs dims 2i and 2i+1 (Mojo `interleaved`;
 * aria_kernel `rope` / `rope_half`); NK_ROPE_HALF_PROPORTIONAL pairs dim i
 * with dim i + head_dim/2 and rotates only the pairs i < rotary_dim/2, the
 * others passing unchanged (aria_kernel `rope_half_proportional`, p-RoPE;
 * the caller builds its table with the head_dim denominator).  In every
 * layout pair i reads table entry i. */
typedef enum {
  NK_ROPE_HALF = 0,
  NK_ROPE_INTERLEAVED = 1,
  NK_ROPE_HALF_PROPORTIONAL = 2
} nk_rope_layout_t;

typedef enum {
  NK_OK = 0,
  NK_ERR_INVALID_ARG = 1,   /* null pointer, negative size, inconsistent shape */
  NK_ERR_UNSUPPORTED = 2,   /* valid but not built: head_dim, page size, dtypes */
  NK_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required */
  NK_ERR_DEVICE = 4         /* a HIP launch or query failed */
} nk_status_t;

typedef struct nk_paged_kv {
  void *k_pages;               /* see layout above, element type `dtype` */
  void *v_pages;
  float *k_scales;             /* NK_E4M3 only, else NULL */
  float *v_scales;
  int32_t dtype;               /* nk_dtype_t of the stored elements */
  int32_t num_pages;
  int32_t page_size;           /* 16 or 32 */
  int32_t num_kv_heads;
  int32_t head_dim;            /* 64, 128 or 256 */
  const int32_t *page_table;   /* [num_seqs][page_table_stride] */
  int32_t page_table_stride;
} nk_paged_kv_t;

/*
 * nk_rope_qk_write_paged -- fused RoPE on Q and K plus append of K/V.
 *
 * Defined by the Mojo docs page generic_fused_qk_rope_bshd_paged_ragged_
 * kernel_api (one fused pass rotates Q and K and writes the rotated keys into
 * the paged cache; Args input_row_offsets, freqs_cis, position_ids, output;
 * parameter `interleaved`), extended to append V.
 *
 * For token t = q_offsets[s] + i (i < q_len(s) = q_offsets[s+1]-q_offsets[s]):
 *   slot  j   = kv_lens[s] - q_len(s) + i      (kv_lens counts keys AFTER
 *                                               this append)
 *   pos       = position_ids ? position_ids[t] : j
 *   each Q head and K head: the pairs of the first rotary_dim dims rotate by
 *   (c, s) = (freqs[pos][p][0], freqs[pos][p][1]):  x' = x c - y s,
 *   y' = x s + y c; dims >= rotary_dim are copied.  V is not rotated.
 *   q_out[t] = rotated Q (input dtype; may alias q).
 *   K and V rows go to page page_table[s][j / page_size], offset
 *   j % page_size, of every KV head.  For an NK_E4M3 cache each (token, kv
 *   head) row gets scale = absmax/448 and codes e4m3(x / scale), rounded to
 *   nearest even (an all-zero row stores scale 0 and zero codes).
 *
 * q      [total_tokens][num_q_heads][head_dim]   in_dtype (NK_F32 / NK_BF16)
 * k, v   [total_tokens][num_kv_heads][head_dim]  in_dtype
 * q_out  [total_tokens][num_q_heads][head_dim]   in_dtype
 * q_offsets [num_seqs+1], kv_lens [num_seqs], position_ids [total_tokens] or NULL
 * freqs  [max_pos][rotary_dim/2][2] float32 (cos, sin)
 * rotary_dim: multiple of 16, 16 <= rotary_dim <= head_dim.
 * Preconditions (not checked): q_offsets non-decreasing with
 * q_offsets[num_seqs] == total_tokens, q_len(s) <= kv_lens[s], the page
 * table covers ceil(kv_lens[s]/page_size) pages, 0 <= pos < max_pos.
 * Slots outside the appended ones are not touched.
 */
int nk_rope_qk_write_paged(const void *q, const void *k, const void *v, int32_t in_dtype,
                           void *q_out, const int32_t *q_offsets, const int32_t *kv_lens,
                           const int32_t *position_ids, const float *freqs, int32_t max_pos,
                           int32_t rotary_dim, int32_t layout, int32_t num_seqs,
                           int32_t total_tokens, int32_t num_q_heads,
                           const nk_paged_kv_t *cache, void *stream);

/*
 * nk_rope_qk_write_paged_mrope -- the same with M-RoPE sections.
 *
 * Mojo page, generic_fused_qk_rope_bshd_paged_ragged_kernel_api, parameter
 * mrope_section (the head dimension partitioned across modalities).  The
 * rotated pairs are split, in pair order, into num_sections sections of
 * section_pairs_host[s] pairs (host array; each a positive multiple of 8,
 * summing to rotary_dim/2); position_ids is [num_sections][total_tokens]
 * (device) and pair p of token t rotates by row
 * position_ids[section(p)][t] of the table.  num_sections 0 is
 * nk_rope_qk_write_paged (position_ids [total_tokens] or NULL); at most 4
 * sections (NK_ERR_INVALID_ARG beyond, or when the sections do not sum to
 * rotary_dim/2; NK_ERR_UNSUPPORTED for a section that is not a multiple of
 * 8 pairs).  Every other argument is as above.
 */
int nk_rope_qk_write_paged_mrope(const void *q, const void *k, const void *v, int32_t in_dtype,
                                 void *q_out, const int32_t *q_offsets, const int32_t *kv_lens,
                                 const int32_t *position_ids, int32_t num_sections,
                                 const int32_t *section_pairs_host, const float *freqs, int32_t max_pos,
                                 int32_t rotary_dim, int32_t layout, int32_t num_seqs,
                                 int32_t total_tokens, int32_t num_q_heads,
                                 const nk_paged_kv_t *cache, void *stream);

/*
 * nk_ragged_paged_attention -- causal (optionally windowed) GQA attention.
 *
 * NumKong matrix-kernels page, attention_packed: query row i of a segment
 * with q_len rows over kv_len keys sits at position p = i + kv_len - q_len
 * and sees keys lo..hi with hi = min(p, kv_len-1), lo = 0 if window_left < 0
 * else max(0, p - window_left) (window_left = w - 1 for a window of w keys);
 * rows that see no key return zeros and lse = -inf.  Query head h reads KV
 * head h / (num_q_heads / num_kv_heads).  With scores
 * s_j = softmax_scale * <q, K_j> (e4m3: K_j = code * scale):
 *   out[t][h] = sum_j exp(s_j - m) V_j / sum_j exp(s_j - m),  m = max_j s_j
 *   lse[t][h] = m + ln(sum_j exp(s_j - m))          (natural log, float32)
 *
 * q    [total_q][num_q_heads][head_dim] q_dtype; out the same, q_dtype.
 * lse  [total_q][num_q_heads] float32, or NULL.
 * q_offsets [num_seqs+1], kv_lens [num_seqs] (device).
 * max_q_len / max_kv_len: host upper bounds of q_len(s) / kv_lens[s]; they
 *   size the launch grids (rows beyond them are not computed).
 * kv_split_tokens: keys per split-KV chunk of a single-token (decode) row,
 *   a multiple of 32; 0 lets the library choose.  Rows of longer segments
 *   (prefill) are not split.
 * workspace: device scratch of at least nk_ragged_paged_attention_workspace_
 *   size(...) bytes with the same scalars (may be NULL when that is 0);
 *   contents need no initialisation and are garbage afterwards.
 * Supported: q_dtype NK_F32 with an NK_F32 cache, NK_BF16 with an NK_BF16
 *   or NK_E4M3 cache.
 */
int nk_ragged_paged_attention(const void *q, int32_t q_dtype, const int32_t *q_offsets,
                              const int32_t *kv_lens, const nk_paged_kv_t *cache,
                              float softmax_scale, int32_t window_left, void *out, float *lse,
                              int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                              int32_t max_kv_len, int32_t num_q_heads, int32_t kv_split_tokens,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * nk_ragged_paged_attention_band -- the same over a general band of keys.
 *
 * NumKong matrix-kernels page, attention_packed: the row at position p sees
 * the keys from p - keys_before through p + keys_after, each side unbounded
 * at None.  Here window_left = keys_before and window_right = keys_after,
 * -1 standing for None:
 *   hi = kv_len-1 if window_right < 0 else min(p + window_right, kv_len-1),
 *   lo as above.
 * window_right = 0 is causal (nk_ragged_paged_attention is this call with
 * window_right 0); window_right < -1 returns NK_ERR_INVALID_ARG.  A
 * single-token row sits at its segment's last key, so window_right does not
 * change it.
 *
 * sink_keys: Algenta "Ten named techniques, one scalar formula each",
 * streaming_llm_sink_score -- StreamingLLM attention keeps a segment's first
 * keys visible beside the window.  Here the row also sees keys
 * 0 .. sink_keys-1 that are not right of hi (they widen the band's left side
 * only); 0 = none; ignored when window_left = -1 (those keys are already in
 * the band); negative returns NK_ERR_INVALID_ARG.  Decode rows take the sink
 * keys as one extra split-KV chunk, which the workspace of every windowed
 * call reserves (nk_ragged_paged_attention_workspace_size covers it).
 * min_q_len: a host lower bound of q_len(s) over the batch's segments (0 when
 * unknown; must not exceed max_q_len, else NK_ERR_INVALID_ARG).  Single-token
 * (decode) rows and longer (prefill) rows run as separate launches; with
 * min_q_len >= 2 the batch holds no decode row and the call launches no
 * decode or merge kernel, as with max_q_len <= 1 it launches no prefill
 * kernel.  A segment shorter than min_q_len violates the precondition (its
 * rows may be left unwritten).
 * Every other argument, the workspace and the errors are those of
 * nk_ragged_paged_attention (which is this call with min_q_len 0).
 */
int nk_ragged_paged_attention_band(const void *q, int32_t q_dtype, const int32_t *q_offsets,
                                   const int32_t *kv_lens, const nk_paged_kv_t *cache,
                                   float softmax_scale, int32_t window_left, int32_t window_right,
                                   int32_t sink_keys, void *out, float *lse, int32_t num_seqs, int32_t total_q,
                                   int32_t min_q_len, int32_t max_q_len, int32_t max_kv_len, int32_t num_q_heads,
                                   int32_t kv_split_tokens, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * nk_ragged_paged_attention_noalloc -- nk_ragged_paged_attention_band without
 * a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The split-KV partials and the prefill work list live in a
 * static device array of NK_NOALLOC_SCRATCH_BYTES inside the library, one per
 * device, held from the first call on that device until the process ends.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine); on its first call on a device it looks the array's address up
 * and clears it with a fill kernel on `stream`.
 *
 * Every argument, result and error is that of nk_ragged_paged_attention_band;
 * a call whose nk_ragged_paged_attention_workspace_size exceeds
 * NK_NOALLOC_SCRATCH_BYTES returns NK_ERR_WORKSPACE before launching
 * anything.  All calls on one device share its array and it keeps the last
 * call's contents: calls that may overlap on one device (several streams or
 * host threads without ordering between them) race and must be serialised
 * by the caller.
 */
#define NK_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int nk_ragged_paged_attention_noalloc(const void *q, int32_t q_dtype, const int32_t *q_offsets,
                                      const int32_t *kv_lens, const nk_paged_kv_t *cache,
                                      float softmax_scale, int32_t window_left, int32_t window_right,
                                      int32_t sink_keys, void *out, float *lse, int32_t num_seqs,
                                      int32_t total_q, int32_t min_q_len, int32_t max_q_len, int32_t max_kv_len,
                                      int32_t num_q_heads, int32_t kv_split_tokens, void *stream);

/* Bytes of workspace nk_ragged_paged_attention needs for these scalars
 * (0 if none).  Pure host computation. */
size_t nk_ragged_paged_attention_workspace_size(int32_t q_dtype, int32_t cache_dtype,
                                                int32_t num_seqs, int32_t total_q,
                                                int32_t max_q_len, int32_t max_kv_len,
                                                int32_t num_q_heads, int32_t num_kv_heads,
                                                int32_t head_dim, int32_t window_left,
                                                int32_t kv_split_tokens);

/* The keys per split-KV chunk nk_ragged_paged_attention uses for these
 * scalars (resolves kv_split_tokens = 0).  Pure host computation. */
int32_t nk_ragged_paged_attention_split_tokens(int32_t num_seqs, int32_t max_kv_len,
                                               int32_t num_q_heads, int32_t num_kv_heads,
                                               int32_t head_dim, int32_t window_left,
                                               int32_t kv_split_tokens);

/*
 * nk_attention_lse_merge -- merge partial attention states.
 *
 * Algenta "Attention variant kernels", "Flash attention's running state
 * reproduces the same softmax" (running max, rescale by exp(old - new),
 * final divide), applied to whole chunks: for row r and head h, with
 * partials i in merge_offsets[r] .. merge_offsets[r+1]-1,
 *   M = max_i lse_i, w_i = exp(lse_i - M),
 *   out[r][h] = sum_i w_i partial_out[i][h] / sum_i w_i,
 *   lse_out[r][h] = M + ln(sum_i w_i);
 * a row whose partials are all -inf (or that has none) gets zeros and -inf.
 *
 * partial_out [n_part][num_heads][head_dim] float32 (normalised chunk outputs)
 * partial_lse [n_part][num_heads] float32, natural log, -inf = empty chunk
 * merge_offsets [num_rows+1] (device, non-decreasing)
 * out [num_rows][num_heads][head_dim] in out_dtype (NK_F32 or NK_BF16)
 * lse_out [num_rows][num_heads] float32 or NULL
 * head_dim: any multiple of 2 up to 512.
 */
int nk_attention_lse_merge(const float *partial_out, const float *partial_lse,
                           const int32_t *merge_offsets, int32_t num_rows, int32_t num_heads,
                           int32_t head_dim, void *out, int32_t out_dtype, float *lse_out,
                           void *stream);

/* Static description of a status code. */
const char *nk_status_string(int status);

/*
 * nk_attention_pack -- pack ragged K/V token matrices into the paged cache.
 *
 * NumKong matrix-kernels page, "Attention with a Pre-Packed KV-Cache" and
 * attention_pack (a pack built once, then read by many attention calls).
 * Input rows key_offsets[s] .. key_offsets[s+1]-1 form segment s's slot;
 * the first kept_s rows of the slot enter the pack, kept_s being
 * key_lengths[s] or, when key_lengths is NULL, the slot's size.
 * The pack is this library's paged cache: attention over it is
 * nk_ragged_paged_attention (or _band) with kv_lens = kv_lens_out, the
 * queries aligned to the end of each segment's kept keys.
 *
 *   k, v         device, in_dtype [rows][num_kv_heads][head_dim] row-major
 *                (rows >= key_offsets[num_seqs]); in_dtype NK_F32 for an
 *                NK_F32 cache, NK_BF16 for NK_BF16 and NK_E4M3 caches.
 *   key_offsets  device int32 [num_seqs + 1], non-decreasing: segment s's
 *                slot is rows key_offsets[s] .. key_offsets[s+1]-1.
 *   key_lengths  device int32 [num_seqs] or NULL (whole slots): kept keys,
 *                clamped to [0, slot size] and to max_key_len.
 *   cache        written: segment s takes the next ceil(kept/page_size)
 *                pages after those of segments 0..s-1 (pages 0, 1, ... in
 *                order), its page_table row lists them (entries past that
 *                count are left alone), and the kept tokens' K, V (and e4m3
 *                scales, absmax/448 per token and head, as the append
 *                step) are stored unrotated, rounded once to the cache type.
 *                Slots past a segment's last kept key are not written.
 *   kv_lens_out  device int32 [num_seqs]: the kept lengths.
 *   max_key_len  an upper bound of the kept lengths; the page table's
 *                stride must hold ceil(max_key_len / page_size) entries.
 * Precondition: num_pages >= sum over s of ceil(kept_s / page_size); with a
 * smaller cache, page ids are clamped to num_pages - 1 (no access out of
 * bounds, the contents unspecified).  Two kernels on `stream`, no
 * allocation, no synchronisation.  Errors: NK_ERR_INVALID_ARG (negative
 * sizes, null pointers, a table stride too small), NK_ERR_UNSUPPORTED
 * (dtype pair, head_dim, page_size), NK_ERR_DEVICE (launch failure).
 */
int nk_attention_pack(const void *k, const void *v, int32_t in_dtype, const int32_t *key_offsets,
                      const int32_t *key_lengths, const nk_paged_kv_t *cache, int32_t *kv_lens_out,
                      int32_t num_seqs, int32_t max_key_len, void *stream);

/*
 * nk_ragged_paged_attention_backward -- query, key and value gradients.
 *
 * NumKong matrix-kernels page, attention_packed_gradients: from the
 * forward's output, its gradient and its (tokens, heads) log-sum-exp, the
 * gradients of q, k and v under the same band.  With s_ij = scale * q_i.k_j
 * over the keys row i sees (window_left, window_right, sink_keys exactly as
 * nk_ragged_paged_attention_band) and P_ij = exp(s_ij - lse_i):
 *   dv_j = sum_i P_ij dout_i,  ds_ij = P_ij (dout_i.v_j - dout_i.out_i),
 *   dq_i = scale * sum_j ds_ij k_j,  dk_j = scale * sum_i ds_ij q_i,
 * each KV head's dk, dv summed over its query heads.
 *
 *   q, out, dout q_dtype [total_q][num_q_heads][head_dim]: the (rotated)
 *                queries the forward used, its output, the output gradient.
 *   lse          float32 [total_q][num_q_heads], the forward's.
 *   cache, q_offsets, kv_lens: as the forward (keys read from the pages).
 *   key_offsets  int32 [num_seqs + 1]: segment s's key j has its dk, dv at
 *                row key_offsets[s] + j (e.g. the offsets nk_attention_pack
 *                read the keys from); rows past kv_lens[s] are not written.
 *   dq           float32 [total_q][num_q_heads][head_dim].
 *   dk, dv       float32 [rows][num_kv_heads][head_dim]; every key of every
 *                segment is written (zeros when no row sees it).
 * The pages call these bf16 gradients yet take a float32 query-gradient
 * buffer; all three are float32 here (a bf16 copy is one rounding away).
 * Types: q_dtype NK_F32 with an NK_F32 cache, NK_BF16 with NK_BF16;
 * e4m3 caches return NK_ERR_UNSUPPORTED.  bf16 at head_dim 64 and 128 runs
 * on bf16 MFMA (the probabilities and dS rounded to bf16 for their products,
 * float32 accumulation); there, with two or more query heads per KV head,
 * the dk/dv rows are zeroed and then summed over head groups with float
 * atomic adds, so their last bits can differ from call to call.  Other cases
 * run in float32 throughout and are deterministic.  Up to four kernels on
 * `stream` (the MFMA path first stores dO.O per row and head in dq, which it
 * then overwrites with the gradient), no workspace, no allocation.  Errors as
 * nk_ragged_paged_attention_band.
 */
int nk_ragged_paged_attention_backward(const void *q, int32_t q_dtype, const int32_t *q_offsets,
                                       const int32_t *kv_lens, const nk_paged_kv_t *cache, float softmax_scale,
                                       int32_t window_left, int32_t window_right, int32_t sink_keys,
                                       const void *out, const void *dout, const float *lse,
                                       const int32_t *key_offsets, float *dq, float *dk, float *dv,
                                       int32_t num_seqs, int32_t total_q, int32_t max_kv_len,
                                       int32_t num_q_heads, void *stream);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int nk_version(void);

/*
 * Kernel timing (diagnostics).  nk_profile_enable takes a mask of kernel
 * families: NK_PROF_ROPE_WRITE ("rope_write"), NK_PROF_ATTN_DECODE
 * ("attn_decode"), NK_PROF_ATTN_PREFILL ("attn_prefill", which includes its
 * scheduling kernel), NK_PROF_ATTN_F32 ("attn_f32"), NK_PROF_LSE_MERGE
 * ("lse_merge"), NK_PROF_ATTENTION_PACK ("attention_pack", with its page
 * assignment kernel), NK_PROF_ATTN_BACKWARD ("attn_backward", both of its
 * kernels); NK_PROF_ALL selects every family and 0 turns timing off.
 * The kernels of a selected family are launched with a pair of HIP events
 * (hipExtLaunchKernel) that take the first kernel's dispatch start time and
 * the last one's end time on the call's stream; no marker packets are added
 * between kernels, but timestamped dispatches still cost the stream about a
 * microsecond, so a caller timing whole steps selects only the family it
 * needs.  nk_profile_read waits for the recorded events and returns the
 * summed milliseconds and the launch count of one family since the last
 * reset.  Events are created on first use and reused; this is the only state
 * the library keeps.  Not for concurrent use from several threads.
 */
#define NK_PROF_ROPE_WRITE 1
#define NK_PROF_ATTN_DECODE 2
#define NK_PROF_ATTN_PREFILL 4
#define NK_PROF_ATTN_F32 8
#define NK_PROF_LSE_MERGE 16
#define NK_PROF_ATTENTION_PACK 32
#define NK_PROF_ATTN_BACKWARD 64
#define NK_PROF_ALL 127
int nk_profile_enable(int family_mask);
int nk_profile_reset(void);
int nk_profile_read(const char *kernel, double *total_ms_host, int64_t *launches_host);

#ifdef __cplusplus
}
#endif

#endif /* NK_H_ */
