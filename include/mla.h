/*
 * mla.h — C ABI of the MI355X (gfx950) Multi-Head Latent Attention library.
 *
 * The library computes one attention layer of MLA decode (and chunked
 * prefill) over a compressed latent KV cache, in the weight-absorbed form:
 *
 *   cache row of token i   : [ c_i (d_latent) | k_pe_i (d_rope) ]
 *                            c_i = x_i W_DKV, k_pe_i = RoPE_i(x_i W_KR)
 *   query of token t       : c_Q = x_t W_DQ
 *                            q_lat[h] = c_Q (W_UQ[h] W_UK[h]^T)     merged
 *                            q_pe[h]  = RoPE_t(c_Q W_QR[h])
 *   score                  : s[h][i] = scale * (q_lat[h].c_i + q_pe[h].k_pe_i)
 *   latent head output     : o_lat[h] = sum_i softmax(s[h])_i c_i
 *   layer output           : y = sum_h o_lat[h] (W_UV[h] W_O[h])        merged
 *
 * Sources: one shared latent per token is cached (page "Latent Space Strikes
 * Again", "The Core Idea"; page "Multi-Head Latent Attention (MLA)", "The
 * construction"), the two merges W_UQ W_UK^T and W_UV W_O (same page, "Two
 * merges are where the compute win comes from"; page "How DeepSeek Rewrote
 * the Transformer", "The short version"), the decoupled RoPE key and query
 * (page "Multi-Head Latent Attention (MLA)", "The RoPE problem"; page
 * "Multi-Head Latent Attention: How DeepSeek Shrinks AI Memory", "How does
 * multi-head latent attention work?"), the causal mask and the
 * 1/sqrt(dim) scale (page "How DeepSeek Rewrote the Transformer", section 03),
 * and paged cache allocation (page "Multi-head Latent Attention (MLA): how
 * DeepSeek cuts KV cache memory", "Where MLA sits in the taxonomy").
 *
 * Conventions (all entry points)
 * ------------------------------
 * - Row-major tensors, row-vector convention (y = x W).
 * - Pointers are DEVICE pointers unless the comment says "host".  The
 *   caller owns and allocates every buffer (weights, absorbed weights, cache
 *   pool, page table, lengths, workspace, outputs); the library allocates no
 *   device memory and keeps no per-call state.
 * - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *   enqueues work on that stream and returns; no call synchronises.
 * - All host-visible argument checks happen before anything is enqueued; a
 *   failing check returns MLA_ERR_INVALID_ARG / MLA_ERR_UNSUPPORTED /
 *   MLA_ERR_WORKSPACE and enqueues nothing.  A failed launch returns
 *   MLA_ERR_HIP.  mla_last_error() returns a message for the last failure
 *   on the calling thread.  No C++ exception crosses this interface.
 * - Values that live on the device (lengths, positions, page ids) are
 *   checked by the kernels: an out-of-range value sets a bit in the
 *   workspace's error word (see mla_read_device_error) and the affected
 *   rows are skipped (append) or the affected outputs are set to NaN
 *   (attention); the kernels never read or write outside the buffers.
 * - dtype MLA_BF16: weights, x, cache rows and q are bf16; accumulation is
 *   fp32; o_lat and y are fp32.  dtype MLA_F32: everything fp32.
 * - Positions are 0-based token indices in the sequence.  RoPE rotates
 *   consecutive pairs (2j, 2j+1) by pos * rope_base^(-2j/d_rope).
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1,  /* null / misaligned pointer, bad size */
  MLA_ERR_UNSUPPORTED = -2,  /* dims or dtype the library has no kernel for */
  MLA_ERR_HIP = -3,          /* a HIP runtime call or launch failed */
  MLA_ERR_WORKSPACE = -4     /* workspace or absorbed buffer too small */
} mla_status;

typedef enum mla_dtype { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

/* How the absorbed weights are held (mla_dims.weight_form).
 *   MLA_WEIGHTS_MERGED: the two merges are precomputed, W_UQ[h] W_UK[h]^T
 *     (d_LQ x d_L per head) and W_UV[h] W_O[h] (d_L x d_model per head)
 *     (page "Multi-Head Latent Attention (MLA)", "Two merges are where the
 *     compute win comes from").
 *   MLA_WEIGHTS_FACTORED: the same products taken in two steps at run time,
 *     q_lat[h] = (c_Q W_UQ[h]) W_UK[h]^T and y = sum_h (o_lat[h] W_UV[h]) W_O[h]
 *     (page "Multi-Head Latent Attention (MLA)", "The construction": the
 *     factors themselves; per-head keys and values are still never formed).
 *     Fewer weight bytes per step when d_nope, d_v < d_L (the DeepSeek-V2
 *     shapes: 0.30 GB instead of 0.92 GB); the intermediate c_Q W_UQ[h] and
 *     o_lat[h] W_UV[h] are rounded to dtype.
 * Every entry point that takes `absorbed` follows dims->weight_form; the
 * attention itself (mla_attention) does not depend on it. */
typedef enum mla_weight_form { MLA_WEIGHTS_MERGED = 0, MLA_WEIGHTS_FACTORED = 1 } mla_weight_form;

/* Model dimensions of one MLA layer. */
typedef struct mla_dims {
  int32_t d_model;     /* token hidden width */
  int32_t n_heads;     /* H */
  int32_t d_latent;    /* d_L: shared KV latent width */
  int32_t d_q_latent;  /* d_LQ: query latent width */
  int32_t d_nope;      /* per-head non-positional key/query width */
  int32_t d_rope;      /* decoupled RoPE key/query width (even) */
  int32_t d_v;         /* per-head value width */
  int32_t dtype;       /* mla_dtype */
  float rope_base;     /* RoPE frequency base, e.g. 10000 */
  float softmax_scale; /* 0 => 1/sqrt(d_nope + d_rope) */
  int32_t weight_form; /* mla_weight_form (0 = merged) */
} mla_dims;

/* Raw (unmerged) weights, device, dtype, row-major with these shapes:
 *   W_DQ [d_model, d_LQ]      W_UQ [d_LQ, H, d_nope]   W_QR [d_LQ, H, d_rope]
 *   W_DKV[d_model, d_L]       W_KR [d_model, d_rope]
 *   W_UK [d_L, H, d_nope]     W_UV [d_L, H, d_v]       W_O  [H, d_v, d_model] */
typedef struct mla_raw_weights {
  const void *W_DQ, *W_UQ, *W_QR, *W_DKV, *W_KR, *W_UK, *W_UV, *W_O;
} mla_raw_weights;

/* Row formats of the latent cache.  The pages leave the bytes per cache
 * element open (page "Multi-Head Latent Attention: How DeepSeek Shrinks AI
 * Memory", "What did DeepSeek's papers actually report?": about 6 bits per
 * element in the served model; page "Multi-Head Latent Attention (MLA)",
 * "Against the alternatives": quantisation as a separate axis).
 *   MLA_ROWS_DTYPE: R elements of the layer dtype per row.
 *   MLA_ROWS_E4M3:  (bf16 layers) R E4M3 codes per row (OCP e4m3fn: sign,
 *     4 exponent bits with bias 7, 3 mantissa bits, largest finite 448),
 *     and one fp32 scale per row; the row's values are code * scale.  The
 *     library writes scale = 2^k with k the smallest integer such that the
 *     row's largest |value| <= 448 * 2^k (k >= -126; 1 for a zero row), and
 *     codes rounded to nearest, ties to even; every code * scale is then
 *     exactly a bf16 value, which is what the attention computes with. */
typedef enum mla_row_format { MLA_ROWS_DTYPE = 0, MLA_ROWS_E4M3 = 1 } mla_row_format;

/* Latent cache.  Row width R = d_latent + d_rope elements.
 * Contiguous (page_table == NULL): pool is [batch, s_max, R].
 * Paged: pool is [n_pages, page_size, R]; token t of sequence b lives in
 * page page_table[b * max_pages_per_seq + t / page_size], slot
 * t % page_size.  page_size must be a positive multiple of 32.
 * row_format MLA_ROWS_E4M3: pool elements are one-byte codes and `scales`
 * (4-byte aligned) holds one fp32 scale per row slot, laid out like the
 * rows ([batch, s_max] or [n_pages, page_size]); otherwise scales is
 * ignored.  The caller owns both buffers. */
typedef struct mla_cache {
  void *pool;
  const int32_t *page_table;
  int32_t page_size;
  int32_t n_pages;
  int32_t max_pages_per_seq;
  int32_t s_max;
  int32_t row_format; /* mla_row_format */
  float *scales;
} mla_cache;

/* Human-readable name of a status code (static string). */
const char *mla_status_str(int32_t status);

/* Message describing the last failure on the calling thread (static
 * thread-local buffer; empty if none). */
const char *mla_last_error(void);

/* Library version string. */
const char *mla_version(void);

/* Layout of the absorbed-weight buffer (host only, no device work).
 * The buffer holds four regions in the packed fragment order described
 * below, at byte offsets[i] with sizes bytes[i]; *total is the buffer size.
 * Merged form (one matrix per region):
 *   [0] W_DKVR : K = d_model,  N = R          [W_DKV | W_KR]
 *   [1] W_DQ   : K = d_model,  N = d_LQ
 *   [2] W_QC   : K = d_LQ,     N = H * R      column h*R + f:
 *                f <  d_L : (W_UQ[h] W_UK[h]^T)[:, f]   (merged, page
 *                           "Multi-Head Latent Attention (MLA)", "Two
 *                           merges", query side)
 *                f >= d_L : W_QR[:, h, f - d_L]
 *   [3] W_UVO  : K = H * d_L,  N = d_model    row h*d_L + c:
 *                (W_UV[h] W_O[h])[c, :]  (merged, output side)
 * Factored form: [0] and [1] as above; region [2] holds four matrices and
 * region [3] two, each starting at a 256-byte boundary in this order:
 *   [2] W_UQ  : K = d_LQ,   N = H * d_nope   column h*d_nope + f: W_UQ[:, h, f]
 *       W_QR  : K = d_LQ,   N = H * d_rope   column h*d_rope + f: W_QR[:, h, f]
 *       W_UKT : K = d_nope, N = H * d_L      column h*d_L + c:    W_UK[c, h, :]
 *       W_UK  : K = d_L,    N = H * d_nope   column h*d_nope + f: W_UK[:, h, f]
 *               (keys of the expanded prefill)
 *   [3] W_UV  : K = d_L,    N = H * d_v      column h*d_v + f:    W_UV[:, h, f]
 *       W_O   : K = H*d_v,  N = d_model      row h*d_v + f:       W_O[h, f, :]
 * Packed order of a logical K x N matrix W (y = x W): element (k, n) sits at
 *   ((k/KB) * (Np/16) + n/16) * 64*KPL + ((n%16) + 16*((k%KB)/KPL)) * KPL + k%KPL
 * with KB = 32, KPL = 8 for bf16 (KB = 4, KPL = 1 for fp32), Np = N rounded
 * up to 16 and K rounded up to KB; padding is zero.  Each 64*KPL block is
 * exactly one MFMA B-operand fragment (16 columns x KB rows), and the
 * fragments of neighbouring column tiles at one k-block are adjacent.
 * Offsets are 256-byte aligned. */
mla_status mla_absorbed_layout(const mla_dims *dims, size_t offsets[4], size_t bytes[4], size_t *total);

/* One-time weight absorption: fills `absorbed` (size from
 * mla_absorbed_layout, in dims->weight_form) from the raw weights (the
 * factored form only repacks them).  Products accumulate in fp32
 * and are rounded once to dtype.  Raw weights are only read. */
mla_status mla_absorb_weights(const mla_dims *dims, const mla_raw_weights *raw, void *absorbed,
                              size_t absorbed_bytes, void *stream);

/* Workspace bytes needed by mla_compress_append / mla_q_proj /
 * mla_attention / mla_decode / mla_out_proj for up to `batch` sequences of
 * `n_q` new tokens on the current device (host only).  A call with fewer
 * rows chooses its GEMMs' K splits so that their fp32 partials fit the
 * workspace it is given (the splits a call would choose on its own vary
 * with the row count).  The first 256 bytes
 * hold the device error word: zero the whole workspace once before first
 * use; later calls keep it sticky until mla_read_device_error clears it. */
mla_status mla_workspace_size(const mla_dims *dims, int32_t batch, int32_t n_q, size_t *bytes);

/* Whether a workspace of ws_bytes serves mla_compress_append, mla_q_proj,
 * mla_attention, mla_decode and mla_out_proj for batch x n_q rows (host
 * only; nothing is enqueued).  Returns MLA_OK, or the status those calls
 * return before enqueueing anything for that size (MLA_ERR_WORKSPACE when
 * the bytes do not fit, MLA_ERR_UNSUPPORTED when no GEMM configuration fits
 * the dims, MLA_ERR_INVALID_ARG for bad dims or sizes).  The workspace
 * pointer itself is not needed. */
mla_status mla_workspace_check(const mla_dims *dims, int32_t batch, int32_t n_q, size_t ws_bytes);

/* Reads (and clears) the device error word of a workspace; synchronises
 * `stream`.  *flags (host) receives a bit mask: 1 = position outside the
 * cache, 2 = page id outside [0, n_pages), 4 = kv_len outside
 * [n_q, capacity]. */
mla_status mla_read_device_error(void *workspace, int32_t *flags, void *stream);

/* Latent down-projection + RoPE + append (page "Latent Space Strikes
 * Again", step 1; page "How DeepSeek Rewrote the Transformer", section 07;
 * page "Multi-Head Latent Attention (MLA)", "The RoPE problem").
 *   x   [batch * n_q, d_model]  dtype   (token t of sequence b at row b*n_q+t)
 *   pos [batch] int32           position of each sequence's first new token
 * Writes the row [x W_DKV | RoPE_p(x W_KR)] of token t of sequence b to the
 * cache slot of position pos[b] + t (contiguous: pool[b][p]; paged: through
 * the page table).  Rows of other positions are not touched. */
mla_status mla_compress_append(const mla_dims *dims, const void *absorbed, const void *x, const int32_t *pos,
                               int32_t batch, int32_t n_q, const mla_cache *cache, void *workspace,
                               size_t ws_bytes, void *stream);

/* Writes given rows into the cache slots of positions pos[b] + t (token t
 * of sequence b), as mla_compress_append writes the rows it computes:
 * rounded to nearest even for a bf16 cache, copied for fp32, quantised as
 * described at mla_row_format for MLA_ROWS_E4M3.  For loading or converting
 * caches, and the reference point of the E4M3 quantiser.
 *   rows [batch * n_q, R] fp32 device; pos [batch] int32 device
 *   workspace: only its first 256 bytes, the device error word, are used
 *   (any workspace of this library, or a zeroed 256-byte buffer)
 * Positions outside the cache and page ids outside the pool set bits 1 and
 * 2 of the device error word and leave the slot untouched. */
mla_status mla_cache_store_rows(const mla_dims *dims, const float *rows, const int32_t *pos, int32_t batch,
                                int32_t n_q, const mla_cache *cache, void *workspace, size_t ws_bytes,
                                void *stream);

/* Query projection with the merged query weight (page "Multi-Head Latent
 * Attention (MLA)", "Two merges", query side; "The RoPE problem"), or in the
 * factored form c_Q W_UQ[h] (rounded to dtype) times W_UK[h]^T.
 *   x [batch * n_q, d_model] dtype; kv_len [batch] int32 (the n_q new tokens
 *   of sequence b sit at positions kv_len[b]-n_q .. kv_len[b]-1)
 *   q [batch * n_q, H, R] dtype out: [c_Q W_UQK[h] | RoPE(c_Q W_QR[h])] */
mla_status mla_q_proj(const mla_dims *dims, const void *absorbed, const void *x, const int32_t *kv_len,
                      int32_t batch, int32_t n_q, void *q, void *workspace, size_t ws_bytes, void *stream);

/* Attention over the latent cache from a projected query (scores straight
 * from the latents; causal inside the n_q new tokens).
 *   q      [batch * n_q, H, R] dtype  (layout of mla_q_proj)
 *   kv_len [batch] int32: visible rows of sequence b, including its n_q new
 *          rows (already appended); query t sees rows 0 .. kv_len-n_q+t
 *   o_lat  [batch * n_q, H, d_latent] fp32 out
 *   lse    [batch * n_q, H] fp32 out or NULL: natural-log log-sum-exp of
 *          the scaled scores of each query row and head
 * The work split depends only on kv_len, n_q and the device, so the same
 * logical cache gives bit-identical results whether paged or contiguous. */
mla_status mla_attention(const mla_dims *dims, const void *q, const int32_t *kv_len, int32_t batch, int32_t n_q,
                         const mla_cache *cache, float *o_lat, float *lse, void *workspace, size_t ws_bytes,
                         void *stream);

/* mla_attention for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels with the same arguments, except that the plan records
 * and split partials live in a library-owned scratch array of 96 MiB per
 * GPU (held from its first use on that GPU until the process ends) instead
 * of a caller workspace.  Nothing is allocated: no hipMalloc, hipFree or
 * allocating library call.
 *   dev_err  device int32, or NULL: the error bits of mla_read_device_error
 *            are OR-ed into it (the caller zeroes it); with NULL they go to
 *            a word in the scratch that nobody reads.
 * The split uses one work-group per CU, or fewer when the partials of that
 * many would not fit the scratch (batch * n_q * ceil(H / 128) above 127 at
 * d_latent 512); when not even 8 fit, returns MLA_ERR_WORKSPACE.  Every
 * call on a GPU shares that GPU's scratch: calls that overlap on one GPU
 * (two streams, two threads) race and must be serialised by the caller. */
mla_status mla_attention_noalloc(const mla_dims *dims, const void *q, const int32_t *kv_len, int32_t batch,
                                 int32_t n_q, const mla_cache *cache, float *o_lat, float *lse, int32_t *dev_err,
                                 void *stream);

/* mla_q_proj followed by mla_attention, with q kept in the workspace. */
mla_status mla_decode(const mla_dims *dims, const void *absorbed, const void *x, const int32_t *kv_len,
                      int32_t batch, int32_t n_q, const mla_cache *cache, float *o_lat, float *lse,
                      void *workspace, size_t ws_bytes, void *stream);

/* Absorbed output projection (page "Multi-Head Latent Attention (MLA)",
 * "Two merges", output side): y[n] = sum_h o_lat[n][h] W_UVO[h]; in the
 * factored form v[h] = o_lat[n][h] W_UV[h] (rounded to dtype), then
 * y[n] = sum_h v[h] W_O[h].
 *   o_lat [n_tok, H, d_latent] fp32;  y [n_tok, d_model] fp32 out.
 * For a bf16 layer with enough rows (the 256-row tiling), o_lat is first
 * rounded to bf16 into the workspace (the rounding every bf16 product
 * applies to it anyway); mla_workspace_size counts that region. */
mla_status mla_out_proj(const mla_dims *dims, const void *absorbed, const float *o_lat, int32_t n_tok, float *y,
                        void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes needed by mla_prefill_expanded for up to `batch`
 * sequences of `n_q` new tokens over a contiguous cache of s_max rows per
 * sequence (host only).  The first 256 bytes hold the device error word, as
 * in mla_workspace_size: zero the workspace once before first use. */
mla_status mla_prefill_workspace_size(const mla_dims *dims, int32_t batch, int32_t n_q, int32_t s_max,
                                      size_t *bytes);

/* Whether a workspace of ws_bytes serves mla_prefill_expanded for batch
 * sequences of n_q new tokens over a contiguous cache of s_max rows per
 * sequence (host only, as mla_workspace_check). */
mla_status mla_prefill_workspace_check(const mla_dims *dims, int32_t batch, int32_t n_q, int32_t s_max,
                                       size_t ws_bytes);

/* Chunked prefill in the expanded form (for long query chunks, where the
 * attention is bound by matrix throughput): every cached latent c_i is
 * up-projected to per-head keys k_i[h] = c_i W_UK[h] and values
 * v_i[h] = c_i W_UV[h]; each head runs causal softmax attention with the
 * query [c_Q W_UQ[h] | RoPE_t(c_Q W_QR[h])] against [k_i[h] | k_pe_i]; then
 * y = sum_h o[h] W_O[h] (page "How DeepSeek Rewrote the Transformer",
 * sections 03-04; page "Multi-Head Latent Attention (MLA)", "The
 * construction").  The same function as mla_decode + mla_out_proj.
 * Needs dims->weight_form == MLA_WEIGHTS_FACTORED, dtype bf16, d_nope =
 * d_v = 128, d_rope = 64 (else MLA_ERR_UNSUPPORTED) and a contiguous cache
 * (page_table NULL) into which the n_q new rows are already appended.
 *   x      [batch * n_q, d_model] bf16; kv_len [batch] int32 as in mla_attention
 *   y      [batch * n_q, d_model] fp32 out
 *   lse    [batch * n_q, H] fp32 out or NULL (natural log, scaled scores)
 * The per-head keys and values of all batch * s_max cache slots live in the
 * workspace (mla_prefill_workspace_size).  A kv_len outside [n_q, s_max]
 * sets error bit 4 and makes that sequence's outputs NaN. */
mla_status mla_prefill_expanded(const mla_dims *dims, const void *absorbed, const void *x, const int32_t *kv_len,
                                int32_t batch, int32_t n_q, const mla_cache *cache, float *y, float *lse,
                                void *workspace, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
