/*
 * mla.h -- weight-absorbed Multi-head Latent Attention (MLA) decode on AMD MI355X (gfx950).
 *
 * The operation.  MLA caches, per token, one d_c-wide latent c_kv instead of every head's
 * keys and values; per-head keys and values are the latent times the up-projections
 * W_UK and W_UV ("Operator Notes (1): MLA -- Multi-head Latent Attention at the Operator
 * Level", section 2).  A small RoPE key k_rope, shared by all heads, is cached beside the
 * latent, and the up-projections can be folded into the query side and the output side
 * ("multi-head latent attention" glossary entry, paragraph on the decoupled RoPE key);
 * by associativity the folded form gives the same attention result ("Multi-Head Latent
 * Attention and the compression of the KV cache", paragraph on mathematical
 * equivalence).  One decode step is three calls:
 *
 *   mla_absorb_q    q_lat[b,i,h,:] = q_nope[b,i,h,:] . W_UK[h]              (query side)
 *   mla_decode      s[t] = scale * (q_lat . c_kv[b,t] + q_rope . k_rope[b,t])
 *                   p = softmax over visible t;  o_lat = sum_t p[t] * c_kv[b,t]
 *                   (mla_decode_paged: the same over a block-table-indexed pool)
 *   mla_absorb_out  out[b,i,h,:] = o_lat[b,i,h,:] . W_UV[h]                  (output side)
 *
 * Conventions shared by every entry point.
 *   - Tensor arguments are DEVICE pointers to dense row-major arrays, shapes listed
 *     outermost first, aligned to 16 bytes.  Host arguments are marked "host".
 *   - Index names: B batch, s_q query tokens per sequence, n_h heads, d_h head width,
 *     d_c latent width, d_r RoPE-key width, T cache rows per sequence.
 *   - Dtypes: MLA_F32 (IEEE binary32), MLA_BF16 (bfloat16), MLA_FP8_E4M3 (OCP e4m3fn,
 *     latent cache only, with one float32 scale per token: value = e4m3(code) * scale).
 *   - Causality: seq_lens[b] counts cache rows INCLUDING the s_q new tokens; query i of
 *     sequence b sees rows 0 .. seq_lens[b] - s_q + i.  A query that sees no row gets
 *     o_lat = 0 and lse = -inf.
 *   - Ownership: the caller owns every buffer.  The library keeps no state (besides the
 *     static device array of mla_decode_noalloc), never allocates or frees device memory,
 *     and never synchronises: each call validates
 *     its arguments on the host, enqueues its kernels on `stream` (a hipStream_t passed
 *     as void*, NULL = the null stream) and returns.  Outputs must not alias inputs.
 *     The calls enqueue kernels only (no memset or copy), so a sequence of them can be
 *     captured into a HIP graph and replayed with the same buffers.
 *   - Errors: a status is returned; nothing is thrown or aborted across the ABI.  On any
 *     status other than MLA_OK nothing was enqueued, except MLA_ERR_HIP (a launch
 *     failed; mla_last_hip_error() gives the hipError_t of the calling thread).
 *   - Contracts not checked on the host (they live in device memory): s_q <= seq_lens[b]
 *     <= T (or <= max_seq_len when paged), and block-table entries are valid pool block
 *     indices for every row below seq_lens[b].  Rows at or past seq_lens[b] and table
 *     entries past the last used block are never read.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, bad scale, misaligned pointer */
  MLA_ERR_UNSUPPORTED = 2, /* valid, but no kernel for this dtype / shape combination */
  MLA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than mla_decode_workspace_bytes */
  MLA_ERR_HIP = 4          /* a HIP launch failed; see mla_last_hip_error() */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1, MLA_FP8_E4M3 = 2 } mla_dtype;

typedef struct {
  int32_t batch;         /* B   >= 1 */
  int32_t q_len;         /* s_q in [1, 8] */
  int32_t n_heads;       /* n_h >= 1 */
  int32_t d_head;        /* d_h >= 1 */
  int32_t d_latent;      /* d_c >= 1 */
  int32_t d_rope;        /* d_r >= 0 */
  float softmax_scale;   /* finite, > 0; multiplies the whole [latent | rope] dot product */
  int32_t split_tokens;  /* tokens per split of the context (split-K); 0 = library's choice.
                            On the matrix-core kernel the choice is balanced ranges: the
                            batch's 32-token tiles (from the device seq_lens) are cut into
                            equal contiguous ranges, one workgroup each, so ragged batches
                            keep every compute unit busy; elsewhere it is a fixed split
                            from max_seq_len.  Any value gives the same result up to
                            rounding; every plan is bitwise reproducible run to run for
                            the same lengths. */
  int32_t fp8_scores;    /* 0, 1 or 2.  1: the latent part of the score is an fp8 matrix
                            product: each row's 128-column slices of q_lat are rounded to
                            e4m3 with their own scale (max|x| / 448) and multiplied with the
                            cache codes as stored; the RoPE term, the softmax and the product
                            with V are unchanged.  Twice the matrix rate for the score, at
                            the cost of the query rounding.  Needs an MLA_FP8_E4M3 cache on
                            the matrix-core kernel (else MLA_ERR_UNSUPPORTED); taken by every
                            decode call (prefill requires 0).
                            Accuracy: the result is attention with that rounded query (to the
                            fp8 kernel bar of 2e-2), which is an approximation of the exact
                            result, outside its 6e-2 parity bar in general: each logit moves by
                            about 2^-4 of its size, so with logits of unit standard deviation
                            the output stays within a few 1e-2 of exact attention over long
                            contexts but the log-sum-exp of a sequence of a few tokens moves by
                            up to about 7e-2, and with logits 4x larger (peaked attention) the
                            output moves by several percent.
                            2: the score as with 1, and the product with V also an fp8 matrix
                            product on the cache codes as stored: each softmax weight times its
                            token's scale is rounded to e4m3 precision (4 significant bits,
                            nearest even; a power-of-two scale per row and 32 tokens keeps
                            every weight above 2^-13 of that block's largest in e4m3's normal
                            range), the normaliser sums the unrounded weights.  Same kernel
                            set and accuracy statement as 1, plus the weight rounding (about
                            2^-5 of each weight, averaging out over long contexts). */
} mla_dims;

/* Supported kernel set (anything else returns MLA_ERR_UNSUPPORTED):
 *   - every shape with all tensors MLA_F32, and with activations / weights in MLA_BF16
 *     and the latent cache in MLA_BF16 or MLA_FP8_E4M3 (general kernels);
 *   - d_c = 512, d_r = 64, activations MLA_BF16, cache MLA_BF16 or MLA_FP8_E4M3,
 *     s_q * n_h a multiple of 64 (for a bf16 cache, of 32), and one sequence's cache rows
 *     spanning less than 2 GiB (max_seq_len * 512 * bytes per code < 2^31): the
 *     matrix-core (MFMA) decode kernels, with row blocks of 64 query rows, or for a bf16
 *     cache of 128 (see mla_decode_plan for which).
 * Limits of every kernel: d_c <= 2048, d_r <= 512, s_q * n_h <= 65536, batch <= 65535,
 * n_heads <= 65535; a decode call uses at most 8192 context splits (an explicit
 * split_tokens that would need more returns MLA_ERR_UNSUPPORTED). */

/* ---- query-side absorption ---------------------------------------------------------
 * q_lat[b,i,h,c] = sum_j q_nope[b,i,h,j] * w_uk[h,j,c]   (fp32 accumulation)
 *   q_nope [B, s_q, n_h, d_h]   dtype q_dt
 *   w_uk   [n_h, d_h, d_c]      dtype w_dt  (w_uk[h,j,c] is the page's W_UK[c, h*d_h + j])
 *   q_lat  [B, s_q, n_h, d_c]   dtype out_dt (rounded to nearest-even)
 * q_dt, w_dt, out_dt are all MLA_F32 or all MLA_BF16. */
mla_status mla_absorb_q(const mla_dims* dims, const void* q_nope, mla_dtype q_dt,
                        const void* w_uk, mla_dtype w_dt, void* q_lat, mla_dtype out_dt,
                        void* stream);

/* ---- latent attention (contiguous cache) -------------------------------------------
 * For every (b, i, h): s[t] = softmax_scale * (q_lat[b,i,h,:] . c_kv[b,t,:]
 *                                              + q_rope[b,i,h,:] . k_rope[b,t,:]),
 * p = softmax of s over the visible rows, o_lat[b,i,h,:] = sum_t p[t] * c_kv[b,t,:],
 * lse[b,i,h] = log sum_t exp(s[t]) (natural log).  fp32 accumulation and softmax.
 *   q_lat   [B, s_q, n_h, d_c]  dtype q_dt
 *   q_rope  [B, s_q, n_h, d_r]  dtype q_dt  (may be NULL when d_r == 0)
 *   c_kv    [B, T, d_c]         dtype kv_dt
 *   kv_scale[B, T] float32      required iff kv_dt == MLA_FP8_E4M3, else NULL
 *   k_rope  [B, T, d_r]         dtype rope_dt (== q_dt; may be NULL when d_r == 0)
 *   T       host, rows per sequence in the cache arrays (their second dimension)
 *   seq_lens[B] int32           valid rows per sequence, or NULL (every sequence has T)
 *   o_lat   [B, s_q, n_h, d_c]  dtype o_dt (== q_dt)
 *   lse     [B, s_q, n_h] float32, or NULL
 *   workspace / workspace_bytes: device scratch of at least
 *           mla_decode_workspace_bytes(dims, kv_dt, T) bytes (may be NULL when that is 0);
 *           its contents on entry are irrelevant and on return unspecified. */
mla_status mla_decode(const mla_dims* dims, const void* q_lat, const void* q_rope, mla_dtype q_dt,
                      const void* c_kv, mla_dtype kv_dt, const float* kv_scale,
                      const void* k_rope, mla_dtype rope_dt, int32_t T, const int32_t* seq_lens,
                      void* o_lat, mla_dtype o_dt, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream);

/* ---- latent attention over a paged cache -------------------------------------------
 * Same result as mla_decode on the cache rebuilt from a block pool: logical row t of
 * sequence b is row (t % block_size) of pool block block_table[b, t / block_size].
 *   c_kv_pool     [n_blocks, block_size, d_c]  dtype kv_dt
 *   kv_scale_pool [n_blocks, block_size] f32   iff kv_dt == MLA_FP8_E4M3, else NULL
 *   k_rope_pool   [n_blocks, block_size, d_r]  dtype rope_dt
 *   block_table   [B, max_blocks_per_seq] int32
 *   seq_lens      [B] int32 (required)
 *   max_seq_len   host upper bound of seq_lens; block_size * max_blocks_per_seq must be
 *                 >= max_seq_len.  The work grid is sized from it.
 * Other arguments as mla_decode; workspace sized by mla_decode_workspace_bytes(dims,
 * kv_dt, max_seq_len).  With the same split_tokens the result is bitwise equal to
 * mla_decode on the gathered cache. */
mla_status mla_decode_paged(const mla_dims* dims, const void* q_lat, const void* q_rope,
                            mla_dtype q_dt, const void* c_kv_pool, mla_dtype kv_dt,
                            const float* kv_scale_pool, const void* k_rope_pool, mla_dtype rope_dt,
                            int32_t n_blocks, int32_t block_size, const int32_t* block_table,
                            int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                            void* o_lat, mla_dtype o_dt, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Bytes of device workspace mla_decode / mla_decode_paged need for this shape, cache dtype
 * and (maximum) context length; 0 when the chosen plan needs none.  Returns 0 as well for
 * arguments that mla_decode would reject (call mla_decode_plan to tell the cases apart). */
size_t mla_decode_workspace_bytes(const mla_dims* dims, mla_dtype kv_dt, int32_t max_seq_len);

/* Host-only: the split-K plan mla_decode would use.  Writes the number of context splits
 * and the tokens per split (host pointers, either may be NULL); for balanced ranges
 * (split_tokens == 0 on the matrix-core kernels) it writes the number of ranges per row
 * block and 0 tokens.  A bf16 cache takes row blocks of 128 query rows when max_seq_len is
 * at least 8192 (or when the rows are a multiple of 32 but not of 64), else of 64; the
 * environment variable MLA_DECODE_ROW_BLOCK=64 or =128, read on every plan, overrides the
 * length rule where that kernel applies.  bf16 row blocks of 64 run on the kernel with two
 * score waves per row block, or, with the environment variable MLA_DECODE_PAIR=0, on the
 * kernel with loader, score and output waves; both take the same plan.  An fp8 cache
 * takes 64.  The device's compute unit count (256 when no device is present) sets the
 * ranges.  No kernel launch. */
mla_status mla_decode_plan(const mla_dims* dims, mla_dtype kv_dt, int32_t max_seq_len,
                           int32_t* num_splits, int32_t* split_tokens);

/* ---- latent attention without allocation -------------------------------------------
 * For callers that cannot allocate device memory or pass a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments, result and
 * errors as mla_decode, minus the workspace: the partial results live in a static device
 * array of MLA_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds from the
 * library's first kernel launch there until the process ends.  The call allocates and frees
 * nothing; on its first call on a device it looks up that device's copy of the array.
 *   - Plans that need more than MLA_NOALLOC_SCRATCH_BYTES of workspace
 *     (mla_decode_workspace_bytes) return MLA_ERR_WORKSPACE before any HIP call.
 *   - Every call on one GPU shares that GPU's array: calls that overlap on one GPU (on
 *     different streams, or from different threads without ordering) race and give
 *     undefined results.  Calls ordered on one stream are safe.
 *   - Nothing in the array needs to start at zero (each call writes what it reads). */
#define MLA_NOALLOC_SCRATCH_BYTES (80u << 20)
mla_status mla_decode_noalloc(const mla_dims* dims, const void* q_lat, const void* q_rope,
                              mla_dtype q_dt, const void* c_kv, mla_dtype kv_dt, const float* kv_scale,
                              const void* k_rope, mla_dtype rope_dt, int32_t T,
                              const int32_t* seq_lens, void* o_lat, mla_dtype o_dt, float* lse,
                              void* stream);

/* ---- output-side absorption --------------------------------------------------------
 * out[b,i,h,j] = sum_c o_lat[b,i,h,c] * w_uv[h,c,j]   (fp32 accumulation)
 *   o_lat [B, s_q, n_h, d_c]  dtype in_dt
 *   w_uv  [n_h, d_c, d_h]     dtype w_dt  (w_uv[h,c,j] is the page's W_UV[c, h*d_h + j])
 *   out   [B, s_q, n_h, d_h]  dtype out_dt
 * in_dt, w_dt, out_dt are all MLA_F32 or all MLA_BF16. */
mla_status mla_absorb_out(const mla_dims* dims, const void* o_lat, mla_dtype in_dt,
                          const void* w_uv, mla_dtype w_dt, void* out, mla_dtype out_dt,
                          void* stream);

/* ---- latent attention and output absorption in one call ------------------------------
 * mla_decode (same arguments, o_dt = q_dt) followed by mla_absorb_out(dims, o_lat, q_dt,
 * w_uv, q_dt, out, q_dt, stream), with the same results bit for bit: o_lat, lse (if not
 * NULL) and out[B, s_q, n_h, d_h] are all written.  w_uv [n_h, d_c, d_h] as for
 * mla_absorb_out.  On the matrix-core kernels' default plan (balanced ranges, bf16, d_c =
 * 512, d_h a multiple of 64, fewer than 8 ranges per sequence on average) the merge of the
 * sequences cut by range boundaries runs inside the output absorption: one launch and one
 * round trip of the merged rows fewer (the output side of "Operator Notes (1): MLA",
 * section 2, o = attn . V then O; the split-K merge of the decode as in mla_decode).
 * Otherwise the two calls run one after the other.  workspace: as for mla_decode.  Errors
 * as for mla_decode, plus MLA_ERR_INVALID_ARG for a NULL or misaligned w_uv or out, all
 * before any launch. */
mla_status mla_decode_absorb_out(const mla_dims* dims, const void* q_lat, const void* q_rope, mla_dtype q_dt,
                                 const void* c_kv, mla_dtype kv_dt, const float* kv_scale, const void* k_rope,
                                 mla_dtype rope_dt, int32_t T, const int32_t* seq_lens, const void* w_uv,
                                 void* o_lat, float* lse, void* out, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* ---- cache write of the new tokens (the step before decode) ------------------------
 * The latent is the only KV state cached ("Operator Notes (1): MLA", section 2:
 * c_kv = x . W_DKV); next to it sits the small decoupled key that carries the rotary
 * position ("multi-head latent attention" glossary entry, paragraph on the decoupled RoPE
 * key).  For new token i (0 <= i < s_q) of sequence b, at position p = seq_lens[b] - s_q + i
 * (seq_lens counts the new tokens, as in decode):
 *   c[b,i,:]  = x[b,i,:] . w_dkv                        (d_c wide, fp32 accumulation)
 *   kr[b,i,:] = RoPE(x[b,i,:] . w_kr, p)                (d_r wide)
 * RoPE turns pair j of the vector by the angle p * rope_base^(-2j / d_r); the pairs are
 * (2j, 2j + 1) for MLA_ROPE_INTERLEAVED and (j, j + d_r / 2) for MLA_ROPE_HALF (the pages
 * name the rotation but print no formula; this is the standard rotary embedding).
 * Both are written to pool row  block_table[b, p / block_size] * block_size + p % block_size:
 *   c_kv_pool row   <- c: kv_dt MLA_BF16 rounds to nearest-even; MLA_F32 stores as is;
 *                      MLA_FP8_E4M3 stores the e4m3fn codes of c / s (nearest-even on the
 *                      magnitude) with s = max|c| / 448 (1 for an all-zero row), and
 *                      kv_scale_pool row <- s
 *   k_rope_pool row <- kr, in dtype x_dt
 *   x      [B, s_q, d_model]  dtype x_dt (MLA_BF16; MLA_F32 only with an MLA_F32 cache)
 *   w_dkv  [d_model, d_c]     dtype x_dt
 *   w_kr   [d_model, d_r]     dtype x_dt (may be NULL when d_r == 0)
 *   pools, block_table, seq_lens as for mla_decode_paged; s_q <= seq_lens[b] and the
 *   rows written must lie inside the pool (device-side contracts, not checked).
 *   d_r must be even.  workspace: at least mla_cache_append_workspace_bytes(dims, d_model)
 *   bytes of device scratch (fp32 split-K partial sums); contents irrelevant on entry.
 * Only the rows of the new tokens are written.  Errors as for mla_decode. */
typedef enum { MLA_ROPE_INTERLEAVED = 0, MLA_ROPE_HALF = 1 } mla_rope_pairing;

size_t mla_cache_append_workspace_bytes(const mla_dims* dims, int32_t d_model);
mla_status mla_cache_append(const mla_dims* dims, int32_t d_model, const void* x, const void* w_dkv,
                            const void* w_kr, mla_dtype x_dt, float rope_base, mla_rope_pairing pairing,
                            void* c_kv_pool, mla_dtype kv_dt, float* kv_scale_pool, void* k_rope_pool,
                            int32_t n_blocks, int32_t block_size, const int32_t* block_table,
                            int32_t max_blocks_per_seq, const int32_t* seq_lens, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Rotary embedding of the query's decoupled part, in place, with the positions above:
 *   q_rope[b,i,h,:] <- RoPE(q_rope[b,i,h,:], seq_lens[b] - s_q + i)
 *   q_rope [B, s_q, n_h, d_r]  dtype q_dt (MLA_BF16 or MLA_F32), d_r even; seq_lens [B]. */
mla_status mla_rope_query(const mla_dims* dims, void* q_rope, mla_dtype q_dt, const int32_t* seq_lens,
                          float rope_base, mla_rope_pairing pairing, void* stream);

/* ---- prefill (explicit form) --------------------------------------------------------
 * "Operator Notes (1): MLA", section 2 (restore K and V from the latent with the
 * up-projections, then scaled dot-product attention), with the decoupled RoPE key of the
 * glossary entry appended to every head's key.  For each sequence b of length
 * L = seq_lens[b] (NULL: T) the s_q = dims.q_len queries are its last s_q rows; query i sees
 * rows t <= L - s_q + i:
 *   K_h[t] = [ W_UK[h] c_kv[b,t] | k_rope[b,t] ],  V_h[t] = W_UV[h]^T c_kv[b,t]
 *   s = scale * (q_nope[b,i,h] . K_h[t][:128] + q_rope[b,i,h] . k_rope[b,t])
 *   out[b,i,h,:] = sum_t softmax(s)_t V_h[t],  lse[b,i,h] = log sum_t exp(s_t)
 * Shapes (all MLA_BF16, d_h = 128, d_c = 512, d_r = 64, any n_h <= 32767):
 *   q_nope [B, s_q, n_h, 128], q_rope [B, s_q, n_h, 64] (already rotated),
 *   c_kv [B, T, 512], k_rope [B, T, 64], w_uk [n_h, 128, 512], w_uv [n_h, 512, 128],
 *   out [B, s_q, n_h, 128], lse [B, s_q, n_h] f32 or NULL; 1 <= s_q <= T; seq_lens [B] device
 *   int32 with s_q <= L <= T (not validated: queries left without a visible row return 0
 *   and -inf).  dims.split_tokens is ignored; dims.fp8_scores must be 0.
 * workspace: at least mla_prefill_workspace_bytes(dims, T) bytes (256-byte aligned) of
 * device scratch, holding the concatenated weights and every cache row's decompressed key
 * and value (B * T * n_h * 512 bytes).  Other errors and the stream as for mla_decode. */
size_t mla_prefill_workspace_bytes(const mla_dims* dims, int32_t T);
mla_status mla_prefill(const mla_dims* dims, const void* q_nope, const void* q_rope, const void* c_kv,
                       const void* k_rope, int32_t T, const int32_t* seq_lens, const void* w_uk,
                       const void* w_uv, mla_dtype dt, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream);

/* ---- projections: query compression, output projection, folds ------------------------
 * y[m, n] = sum_k x[m, k] * w[k, n] (MLA_BF16 in and out, fp32 accumulation), row-major
 * x [M, K], w [K, N], y [M, N].  The weight-streaming products around the attention:
 * c_q = x W_DQ and the query up-projections ("Operator Notes (1): MLA", section 4), the
 * output projection O W_O (section 2), and products with folded weights.  K must be a
 * multiple of 256 and N of 64 (else MLA_ERR_UNSUPPORTED); 1 <= M <= 32 * 65535.  The
 * workspace (at least mla_linear_workspace_bytes(M, K, N) bytes, 16-byte aligned) holds
 * the fp32 partial sums of the 256-wide slices of K; contents irrelevant on entry. */
size_t mla_linear_workspace_bytes(int32_t M, int32_t K, int32_t N);

/* ---- output-side fold ----------------------------------------------------------------
 * w_uvo[h, c, :] = sum_j w_uv[h, c, j] * w_o[h * d_h + j, :]   (fp32 accumulation, bf16 out)
 *   w_uv  [n_h, d_c, d_h]       MLA_BF16 (the per-head layout mla_absorb_out takes)
 *   w_o   [n_h * d_h, d_model]  MLA_BF16 (the output projection W_O, row-major)
 *   w_uvo [n_h, d_c, d_model]   MLA_BF16
 * The value up-projection merged into the output projection ("Operator Notes (1): MLA",
 * sections 2 and 4; the glossary's paragraph on the decoupled RoPE key): afterwards
 * mla_linear(o_lat viewed as [M, n_h * d_c], w_uvo viewed as [n_h * d_c, d_model]) gives the
 * layer output O W_O without forming the per-head outputs O.  Run once per weight set.
 * d_h must be 128 or 512, d_model a multiple of 64, d_c <= 32 * 65535, dt MLA_BF16 (else
 * MLA_ERR_UNSUPPORTED); pointers 16-byte aligned (else MLA_ERR_INVALID_ARG). */
mla_status mla_fold_output_weights(const void* w_uv, const void* w_o, void* w_uvo, int32_t n_h, int32_t d_c,
                                   int32_t d_h, int32_t d_model, mla_dtype dt, void* stream);
mla_status mla_linear(const void* x, const void* w, void* y, int32_t M, int32_t K, int32_t N, mla_dtype dt,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ---- utilities -------------------------------------------------------------------- */

/* Copy rows of a block pool into a contiguous per-sequence array (the paged lookup alone):
 * dst[b, t, :] = pool[block_table[b, t / block_size], t % block_size, :] for t < seq_lens[b];
 * rows t >= seq_lens[b] (t < max_seq_len) are left untouched.  Rows are row_bytes wide
 * (a multiple of 4).  pool [n_blocks, block_size, row_bytes], dst [B, max_seq_len, row_bytes]. */
mla_status mla_gather_pages(const void* pool, int32_t n_blocks, int32_t block_size, int64_t row_bytes,
                            const int32_t* block_table, int32_t batch, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, int32_t max_seq_len, void* dst, void* stream);

/* Decode every e4m3fn code on the device exactly as the fp8 decode kernels do:
 * out[k] = value of code k as the general kernels convert it, out[256 + k] as the
 * matrix-core kernels convert it (to bf16), k = 0..255 (float32 [512]). */
mla_status mla_fp8_e4m3_table(float* out, void* stream);

/* Static description of a status code (never NULL). */
const char* mla_status_str(mla_status status);

/* hipError_t of the last MLA_ERR_HIP returned on the calling thread (0 if none). */
int mla_last_hip_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int mla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
