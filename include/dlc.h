/*
 * dlc.h - C ABI of the CSA/HCA compressed-attention hot path for AMD gfx950.
 *
 * The operations are those derived on the page "DeepSeek-V4 Hybrid Attention:
 * CSA and HCA from Scratch" (cited below as [Scratch] with its section):
 * the token-level KV compressor (CSA with overlapping 2m windows, HCA with
 * m' windows), lightning-indexer scoring with top-k over the CSA cache,
 * shared-KV multi-query attention over the k selected CSA entries, and
 * dense shared-KV attention over the HCA cache.  Argument names follow the
 * page's notation: n tokens, query position t, compressed width c, ratios m
 * and m', budget k, n_h query heads, n_h^I indexer heads of width c^I.
 *
 * Conventions for every call:
 *  - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees, copies to the host or synchronises; every call
 *    only enqueues kernels on `stream` (a hipStream_t; NULL is the default
 *    stream) and returns.
 *  - Arrays are row-major and contiguous unless a stride argument says
 *    otherwise; the batch index is outermost.  Strides count elements.
 *  - `dtype` is the storage type of the compressed entries, streams and
 *    queries (DLC_F32 or DLC_BF16).  Arithmetic always accumulates in fp32;
 *    outputs documented as float are fp32.
 *  - Return value: DLC_OK (0) or a negative dlc_status.  Arguments are
 *    validated on the host before anything is enqueued; on an error nothing
 *    is enqueued and dlc_last_error() describes the problem.  A failed launch
 *    returns DLC_E_HIP.  No exception or abort crosses this boundary.
 *  - Device-side values (query positions t, top-k indices and counts) are
 *    clamped by the kernels to the ranges the host validated, so malformed
 *    device data yields wrong numbers, never an out-of-bounds access.
 *  - The five calls and dlc_project hold no state and are reentrant (the
 *    only state in the library is the per-thread timing hook of the
 *    measurement section below).  Outputs are bitwise reproducible for
 *    identical inputs, shapes and device; a compressed entry has the same
 *    bits whether it was computed alone (i_end = i_begin + 1) or in a long
 *    range.
 */
#ifndef DLC_H
#define DLC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DLC_ABI_VERSION 1

typedef enum {
  DLC_OK = 0,
  DLC_E_INVAL = -1,       /* bad scalar argument or NULL required pointer */
  DLC_E_DTYPE = -2,       /* unsupported dtype */
  DLC_E_SHAPE = -3,       /* inconsistent sizes, strides or ranges */
  DLC_E_WORKSPACE = -4,   /* workspace missing or smaller than the *_ws query */
  DLC_E_HIP = -5,         /* a HIP runtime call or kernel launch failed */
  DLC_E_UNSUPPORTED = -6  /* valid request outside this build's limits */
} dlc_status;

typedef enum { DLC_F32 = 0, DLC_BF16 = 1 } dlc_dtype;

/* ABI version, status names and the last error of the calling thread. */
int dlc_abi_version(void);
const char* dlc_status_str(int status);
const char* dlc_last_error(void);

/*
 * csa_compress - CSA compressed entries i_begin .. i_end-1 ([Scratch] §4-§5).
 *
 * For entry i and column j: one softmax over the 2m logits
 *   Z^a[m*i + r][j] + B^a[r][j]        (r < m, current block)
 *   Z^b[m*(i-1) + r][j] + B^b[r][j]    (r < m, previous block; absent for i = 0)
 * then C^Comp[i][j] = sum of the weights times the matching C^a / C^b values.
 * The missing b-rows of entry 0 (the page pads them with -inf) get weight 0,
 * and so does any row whose logit Z + B is -inf (a -inf bias masks its row
 * position); a column whose logits are all -inf has no softmax and gives NaN.
 * The same call builds the indexer-key cache K^IComp from the indexer's own
 * four streams at width c := c^I ([Scratch] §6.4).
 *
 *  dtype          storage type of streams and output
 *  B, n, c, m     sequences, valid stream rows per sequence, width, ratio (m >= 1)
 *  Za, Zb, Ca, Cb streams; element (b, row, j) at X[b*batch_stride + row*ld + j]
 *  ld             row stride (>= c); batch_stride (>= (n-1)*ld + c when B > 1)
 *  Ba, Bb         fp32 [m][c] positional biases, or NULL for zeros
 *  i_begin,i_end  0 <= i_begin <= i_end <= n/m; entries outside are untouched
 *  Ccomp, cap     output [B][cap][c] (cap >= i_end); entry i of sequence b
 *                 at Ccomp[(b*cap + i)*c]
 * Decode appends one token row at a time; when (t+1) % m == 0 the caller
 * compresses the entry that row completes with i_begin = (t+1)/m - 1.
 */
int csa_compress(int dtype, int64_t B, int64_t n, int64_t c, int64_t m,
                 const void* Za, const void* Zb, const void* Ca, const void* Cb,
                 int64_t ld, int64_t batch_stride, const float* Ba, const float* Bb,
                 int64_t i_begin, int64_t i_end, void* Ccomp, int64_t cap, void* stream);

/*
 * hca_compress - HCA compressed entries ([Scratch] §10): one softmax per
 * column over the m' logits Z[m'*i + r][j] + Bias[r][j] of the
 * non-overlapping block i, then C^HCA[i][j] = sum_r S[r][j] * C[m'*i + r][j].
 * Arguments as for csa_compress with one stream pair (Z, C) and an fp32
 * [m'][c] Bias (NULL for zeros).
 */
int hca_compress(int dtype, int64_t B, int64_t n, int64_t c, int64_t m_prime,
                 const void* Z, const void* C, int64_t ld, int64_t batch_stride,
                 const float* Bias, int64_t i_begin, int64_t i_end,
                 void* Chca, int64_t cap, void* stream);

/*
 * csa_project_compress / hca_project_compress - the compressor's stream
 * projections ([Scratch] §3: Z^a = H W^{aZ}, C^a = H W^{aKV}, and the b- and
 * HCA streams alike) and its pooling (§4-§5, §10) in one pass: the projected
 * streams are never written.  The result equals dlc_project of each stream
 * (stored in bf16) followed by csa_compress / hca_compress with the same
 * biases and entry range, bit for bit, where n > 16 (with at most 16 rows
 * dlc_project takes its row-vector path, which adds the same fp32 products
 * in another order).
 *
 *  dtype          DLC_BF16 (hidden rows, weights and output)
 *  B, n, d        sequences, valid rows per sequence, hidden width (d % 8 == 0)
 *  H              hidden rows: row r of sequence b at H + b*h_bstride + r*ldh
 *                 (ldh >= d; ldh, h_bstride multiples of 8; 16-byte aligned)
 *  Wt*            per stream the weight transposed, [c][ldw] (channel j is
 *                 row j, its d weights contiguous; ldw >= d, ldw % 8 == 0,
 *                 16-byte aligned): csa takes Z^a, Z^b, C^a, C^b; hca Z, C
 *  c              width: a multiple of 32 (csa) or 64 (hca)
 *  m, m_prime     ratio: a divisor of 128 (csa: below 128)
 *  Ba, Bb, Bias   fp32 [m][c] positional biases, or NULL for zeros
 *  i_begin,i_end  0 <= i_begin <= i_end <= n/m; entries outside are untouched
 *  Ccomp/Chca,cap output [B][cap][c] bf16 (cap >= i_end)
 * Each workgroup projects a 128-row tile of every stream for one group of
 * channels and pools it in place; a CSA tile completes 128/m - 1 entries (one
 * block is shared with the next tile and projected twice).
 */
int csa_project_compress(int dtype, int64_t B, int64_t n, int64_t d, int64_t c, int64_t m,
                         const void* H, int64_t ldh, int64_t h_bstride,
                         const void* WtZa, const void* WtZb, const void* WtCa, const void* WtCb,
                         int64_t ldw, const float* Ba, const float* Bb, int64_t i_begin,
                         int64_t i_end, void* Ccomp, int64_t cap, void* stream);
int hca_project_compress(int dtype, int64_t B, int64_t n, int64_t d, int64_t c, int64_t m_prime,
                         const void* H, int64_t ldh, int64_t h_bstride, const void* WtZ,
                         const void* WtC, int64_t ldw, const float* Bias, int64_t i_begin,
                         int64_t i_end, void* Chca, int64_t cap, void* stream);

/*
 * csa_index_topk - lightning-indexer scores and top-k ([Scratch] §6.4, §7).
 *
 * For query (b, q) at position t = t[b][q], over the visible entries
 * s < min(floor(t/m), cap):
 *   I[s] = sum_h w^I[h] * ReLU(q^I[h] . K^I[s])     (no softmax, no scale)
 * then the k_eff = min(k, visible) largest scores, ranked by score
 * (descending) and then index (ascending); -0.0 ranks equal to +0.0.
 *
 *  qI      [B][n_q][n_hI][cI] in dtype (head h is columns h*cI ... of the
 *          up-projected latent, [Scratch] §6.2)
 *  wI      [B][n_q][n_hI] fp32 head weights
 *  KI,cap  [B][cap][cI] indexer-key cache in dtype
 *  t       DEVICE int64 [B][n_q] query positions, each in [0, t_max]
 *  t_max   host bound on t; floor(t_max/m) must not exceed cap
 *  idx     out int32 [B][n_q][k]: the selected entries in ascending order,
 *          padded with -1 after count entries
 *  count   out int32 [B][n_q]: k_eff
 *  scores  optional out fp32 [B][n_q][cap]: I[s] for visible s (others
 *          untouched), or NULL
 *  ws      workspace of at least csa_index_topk_ws(B, n_q, cap, k) bytes,
 *          256-byte aligned; its contents on entry do not matter for the
 *          result.  Each call leaves the first-digit histograms at its
 *          start (B*n_q*2048 words) at zero for the next call on the same
 *          workspace; a workspace that does not start that way (a new
 *          allocation, or one used for something else in between) is
 *          detected, and the call then counts the histograms again from
 *          the scores, which costs it one more pass over them.  Calls that
 *          share a workspace must not overlap.
 * Limits: 1 <= k <= 8192; bf16 with c^I in {32, 64, 128, 256} and n_hI <= 64
 * (the MFMA shapes), otherwise n_hI*cI <= 8192.
 * Many queries per sequence (a prefill chunk, n_q >= 64) run query-tiled
 * (bf16, c^I = 128: each key row then serves 64 queries) and stream the
 * cache in ranges of 32768 entries, each range's top-k folded into a running
 * top-k; the results are the same.  Their workspace grows with B*n_q*k and
 * B*n_q*32768, not with cap; a decode call (n_q < 64) keeps eight 4-byte
 * arrays per query and entry.
 */
size_t csa_index_topk_ws(int64_t B, int64_t n_q, int64_t cap, int64_t k);
int csa_index_topk(int dtype, int64_t B, int64_t n_q, int64_t n_hI, int64_t cI, int64_t m, int64_t k,
                   const void* qI, const float* wI, const void* KI, int64_t cap,
                   const int64_t* t, int64_t t_max, int32_t* idx, int32_t* count, float* scores,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * FP4 indexer ([Scratch] §6.4: the indexer's q . K products run in FP4;
 * §12: indexer FLOPs "in FP4").  The pages name no FP4 format; these calls
 * use OCP MXFP4: a row is cut into blocks of 32 elements, each block stores
 * one E8M0 scale byte e + 127 with e = floor(log2(max |x|)) - 2 (-127 for an
 * all-zero block) and 32 E2M1 codes (bit 3 sign, bits 0..2 the magnitude
 * index into {0, 0.5, 1, 1.5, 2, 3, 4, 6}), each x / 2^e rounded to the
 * nearest magnitude with ties to the even code, saturated at 6, zero stored
 * as code 0.  Element 2i is the low nibble of code byte i.
 *
 * mxfp4_quantize - quantize rows of width `width` (a multiple of 32):
 *  src     [B] batches of [rows][width] in dtype (DLC_F32 or DLC_BF16),
 *          batch b at src + b*src_bstride elements; 16-byte aligned
 *  codes   out [B] x [rows][width/2] bytes, batch b at codes + b*codes_bstride;
 *          16-byte aligned
 *  scales  out [B] x [rows][width/32] E8M0 bytes, batch b at
 *          scales + b*scales_bstride
 * Quantizing rows i_begin .. i_end-1 of a cache: pass src + i_begin*width,
 * codes + i_begin*width/2, scales + i_begin*width/32 and rows = i_end-i_begin.
 *
 * csa_index_topk_fp4 - csa_index_topk with q^I and K^I in MXFP4: the scores
 * are the formula of csa_index_topk on the dequantized operands, products
 * exact and sums in fp32 (v_mfma_scale_f32_16x16x128_f8f6f4), w^I in fp32.
 *  qI      [B][n_q][n_hI][cI] in dtype (DLC_F32 or DLC_BF16), quantized per
 *          head row inside the call (the same rule); 16-byte aligned
 *  KIc     [B][cap][cI/2] key code bytes (mxfp4_quantize of the K^I cache)
 *  KIs     [B][cap][cI/32] key scale bytes; 4-byte aligned
 *  ws      workspace of at least csa_index_topk_fp4_ws(B, n_q, n_hI, cI,
 *          cap, k) bytes, 256-byte aligned (it also holds the quantized
 *          queries); its contents on entry do not matter
 *  other arguments, outputs and ranking as for csa_index_topk.
 * Limits: cI in {128, 256}, n_hI <= 64, 1 <= k <= 8192; KIc 16-byte
 * aligned, KIs 4-byte aligned (DLC_E_INVAL otherwise).
 */
int mxfp4_quantize(int dtype, int64_t B, int64_t rows, int64_t width, const void* src, int64_t src_bstride,
                   uint8_t* codes, int64_t codes_bstride, uint8_t* scales, int64_t scales_bstride, void* stream);
size_t csa_index_topk_fp4_ws(int64_t B, int64_t n_q, int64_t n_hI, int64_t cI, int64_t cap, int64_t k);
int csa_index_topk_fp4(int dtype, int64_t B, int64_t n_q, int64_t n_hI, int64_t cI, int64_t m, int64_t k,
                       const void* qI, const float* wI, const uint8_t* KIc, const uint8_t* KIs, int64_t cap,
                       const int64_t* t, int64_t t_max, int32_t* idx, int32_t* count, float* scores,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * csa_attend - shared-KV multi-query attention over the selected CSA
 * entries ([Scratch] §8): for every head h,
 *   o[h] = sum_s softmax_s(scale * q[h] . C^Comp[s]) * C^Comp[s],
 *   lse[h] = log sum_s exp(scale * q[h] . C^Comp[s]),
 * over s = idx[b][q][0 .. count-1].  Key and value are the same entry.
 *
 *  q         [B][n_q][n_h][c] in dtype
 *  Ccomp,cap [B][cap][c] compressed cache in dtype
 *  idx,count as returned by csa_index_topk; indices outside [0, cap) and
 *            positions past min(count, k) are ignored
 *  scale     logit scale; <= 0 selects 1/sqrt(c)
 *  out       fp32 [B][n_q][n_h][c];  lse: fp32 [B][n_q][n_h] or NULL
 *  ws        at least csa_attend_ws(B, n_q, n_h, c, k) bytes, 256-byte aligned
 * An empty selection gives o = 0 and lse = -inf.
 * Limit: bf16 with c = 512 lists each split's rows in LDS, so k (plus n_win
 * for csa_attend_window) is at most 256 * 2048 = 524288; beyond that the call
 * returns DLC_E_UNSUPPORTED.
 */
size_t csa_attend_ws(int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t k);
int csa_attend(int dtype, int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t k,
               const void* q, const void* Ccomp, int64_t cap, const int32_t* idx, const int32_t* count,
               float scale, float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * csa_attend_noalloc - csa_attend for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments without the workspace, the same
 * kernels and bit-identical results.  Its split-K partials live in a static
 * device array of 32 MiB (33554432 bytes) that every device the library runs
 * on holds until the process ends; a shape whose csa_attend_ws(B, n_q, n_h, c,
 * k) exceeds that returns DLC_E_UNSUPPORTED before anything is enqueued.  The
 * call allocates and frees nothing.  All calls on one device share that
 * device's array: calls that overlap on one device (concurrent streams or
 * host threads) race and must be serialised by the caller.  Nothing in the
 * array needs to start at zero; each call writes every byte it reads.
 */
int csa_attend_noalloc(int dtype, int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t k,
                       const void* q, const void* Ccomp, int64_t cap, const int32_t* idx, const int32_t* count,
                       float scale, float* out, float* lse, void* stream);

/*
 * hca_attend - dense shared-KV attention over every visible HCA entry
 * s < min(floor(t/m'), cap) ([Scratch] §10 and the unified operator of §11,
 * whose top-k is a no-op for HCA).  Same formula, layouts and empty-case
 * rule as csa_attend; t and t_max as for csa_index_topk with m := m'.
 *  ws  at least hca_attend_ws(B, n_q, n_h, c, cap) bytes, 256-byte aligned
 */
size_t hca_attend_ws(int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t cap);
int hca_attend(int dtype, int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t m_prime,
               const void* q, const void* Chca, int64_t cap, const int64_t* t, int64_t t_max,
               float scale, float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * window_attend - the sliding-window branch ("From MHA, GQA to MLA, DSA,
 * HCA/CSA", §6.1 and §6.2, sliding window path): shared-KV attention of each
 * query over the raw window entries c^window_p = h_p W^{window,KV} of the
 * n_win most recent tokens p = max(0, t-n_win+1) .. t, with the same formula,
 * scale and empty-case rule as csa_attend.  The pages join these entries to
 * the compressed ones by concatenation before one attention; since softmax
 * sums over keys, that equals merging the two parts' outputs by their
 * log-sum-exp, which this call does when o_in is given.
 *
 *  Cwin    [B][ring][c] ring in dtype (ring >= n_win): the entry of token p
 *          is row p % ring.  Decode: ring = n_win, the caller writes the new
 *          token's row before the call.  Queries at several positions (a
 *          prefill chunk ending at token T) need every window inside the
 *          ring: ring >= n_win + (T - smallest t).
 *  t,t_max as for hca_attend; only rows of tokens in the window are read
 *  o_in, lse_in  optional fp32 [B][n_q][n_h][c] and [B][n_q][n_h]: the
 *          compressed branch's output (csa_attend or hca_attend).  When given,
 *          out / lse are the attention over both key sets; out may be o_in and
 *          lse may be lse_in (in place).  Both NULL: the window part alone.
 *  out     fp32 [B][n_q][n_h][c];  lse: fp32 [B][n_q][n_h] or NULL
 *  ws      at least window_attend_ws(B, n_q, n_h, c, n_win) bytes, 256-byte aligned
 */
size_t window_attend_ws(int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t n_win);
int window_attend(int dtype, int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t n_win,
                  const void* q, const void* Cwin, int64_t ring, const int64_t* t, int64_t t_max, float scale,
                  const float* o_in, const float* lse_in, float* out, float* lse,
                  void* ws, size_t ws_bytes, void* stream);

/*
 * csa_attend_window / hca_attend_window - csa_attend and hca_attend with the
 * layer's sliding-window branch joined in: one attention over the selected
 * (CSA) or visible (HCA) compressed entries followed by the window entries of
 * the ring, as the pages concatenate them (see window_attend).  The window
 * keys are a tail of the same key list, so both sets share the splits and the
 * combine; the result equals csa_attend (hca_attend) followed by window_attend
 * with o_in, up to rounding.  Arguments as for csa_attend / hca_attend plus
 * the ring Cwin [B][ring][c] (token p at row p % ring, ring >= n_win), n_win,
 * and, for the CSA form, the query positions t / t_max that place the window.
 */
size_t csa_attend_window_ws(int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t k, int64_t n_win);
int csa_attend_window(int dtype, int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t k,
                      const void* q, const void* Ccomp, int64_t cap, const int32_t* idx, const int32_t* count,
                      const void* Cwin, int64_t ring, int64_t n_win, const int64_t* t, int64_t t_max,
                      float scale, float* out, float* lse, void* ws, size_t ws_bytes, void* stream);
size_t hca_attend_window_ws(int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t cap, int64_t n_win);
int hca_attend_window(int dtype, int64_t B, int64_t n_q, int64_t n_h, int64_t c, int64_t m_prime,
                      const void* q, const void* Chca, int64_t cap, const int64_t* t, int64_t t_max,
                      const void* Cwin, int64_t ring, int64_t n_win, float scale, float* out, float* lse,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * attend_sink - per-head sink logits ([Scratch] §12 names them without a formula;
 * the reading: one logit z_h per head joins the attention's softmax as an
 * extra key whose value is the zero vector).  Applied in place to a finished
 * attention (the output and log-sum-exp of csa_attend, hca_attend or their
 * joined forms), which is exact:
 *   o'[h]   = o[h] * e^lse[h] / (e^lse[h] + e^z[h])
 *   lse'[h] = log(e^lse[h] + e^z[h])
 * An empty key set (lse = -inf, o = 0) gives o' = 0 and lse' = z.
 *  out  [rows][n_h][c] fp32, in place, 16-byte aligned (rows = B*n_q)
 *  lse  [rows][n_h] fp32, in place
 *  z    [n_h] fp32 sink logits (natural-log units, like lse)
 */
int attend_sink(int64_t rows, int64_t n_h, int64_t c, float* out, float* lse, const float* z, void* stream);

/*
 * dlc_project - dense projection out = A . W with fp32 accumulation, the
 * token projections that feed the compressor and the queries ([Scratch] §3:
 * C^a = H W^{aKV} and its siblings; §6.1-6.3 and §8: c^Q, q^I, w^I, q).
 *
 *  A    [M][K] rows with stride lda, in dtype
 *  Wt   the weight matrix W [K][N] stored transposed, Wt[N][K] with row
 *       stride ldw, in dtype
 *  out  [M][N] with row stride ldo, stored in out_dtype (DLC_F32 or dtype)
 *  ws   optional workspace of ws_bytes >= dlc_project_ws(dtype, M, N, K)
 *       bytes, or NULL.  It must be all zero before its first use; every
 *       call leaves it all zero again, so calls of any shape can reuse it
 *       (calls that share one workspace must not run at the same time).  A
 *       smaller non-NULL workspace returns DLC_E_WORKSPACE.
 *
 * bf16 with K, lda, ldw multiples of 8 and A, Wt 16-byte aligned runs on
 * MFMA: 128x128 output tiles, or at M <= 16 (a decode step's tokens) a
 * row-vector path that streams the weight rows (its cost is the read of
 * Wt).  With a workspace the row path also splits the k-range of a column
 * tile over several workgroups, which pays where N is small and K large;
 * the slices are added in a fixed order, so the result is bitwise the same
 * from call to call (but not the same bits as without the workspace).
 * Other cases run a VALU kernel.
 *
 * dlc_project_ws - the workspace bytes that let dlc_project split the
 * k-range at this shape (0: it never splits here, pass NULL).
 */
int dlc_project(int dtype, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                const void* Wt, int64_t ldw, void* out, int64_t ldo, int out_dtype,
                void* ws, size_t ws_bytes, void* stream);
size_t dlc_project_ws(int dtype, int64_t M, int64_t N, int64_t K);

/*
 * Measurement support (not part of the method).
 *
 * dlc_timing_arm - the next launch of `stage` on the calling thread records
 * the caller's HIP events `ev_begin` (before) and `ev_end` (after) on that
 * launch's stream, then disarms.  Where the stage is one kernel (marked
 * [kernel] below) the events are bound to that kernel's own dispatch
 * (hipExtLaunchKernel) and time the kernel alone; elsewhere they are
 * recorded around the stage's launches and also take in their dispatch
 * latency.  The events are hipEvent_t handles owned by the caller; NULL
 * events disarm the stage.  Stages:
 *   DLC_STAGE_INDEX_SCORES  the indexer score kernel of csa_index_topk (or _fp4) [kernel];
 *                           for a query-tiled call (n_q >= 64), which runs the cache range
 *                           by range, the whole indexer: every range's scores, selection
 *                           and merge
 *   DLC_STAGE_TOPK_SELECT   the selection kernel of csa_index_topk (or _fp4)
 *   DLC_STAGE_CSA_ATTEND    csa_attend (attention and combine kernels)
 *   DLC_STAGE_HCA_ATTEND    hca_attend (attention and combine kernels)
 *   DLC_STAGE_COMPRESS      csa_compress / hca_compress and the fused calls
 *   DLC_STAGE_WINDOW_ATTEND window_attend (attention and merge kernels)
 *   DLC_STAGE_READ          the kernel of dlc_read [kernel]
 *
 * dlc_copy - device-to-device copy kernel of `bytes` bytes (a multiple of
 * 16, both pointers 16-byte aligned); the reference for achievable HBM
 * bandwidth and for scaling hardware byte counters.
 */
enum {
  DLC_STAGE_INDEX_SCORES = 1,
  DLC_STAGE_TOPK_SELECT = 2,
  DLC_STAGE_CSA_ATTEND = 3,
  DLC_STAGE_HCA_ATTEND = 4,
  DLC_STAGE_COMPRESS = 5,
  DLC_STAGE_WINDOW_ATTEND = 6,
  DLC_STAGE_READ = 7
};
int dlc_timing_arm(int stage, void* ev_begin, void* ev_end);
int dlc_copy(void* dst, const void* src, size_t bytes, void* stream);
/* load forms of dlc_read */
#define DLC_READ_LDS 0   /* 1 KB per wave instruction straight to LDS (global_load_lds_dwordx4) */
#define DLC_READ_TILES 1 /* 16-byte register loads in the bf16 indexer's MFMA operand pattern */
/*
 * dlc_read - read-only kernel over `bytes` bytes of device memory at src
 * (16-byte aligned); each byte is loaded once and nothing is written.  The
 * reference that calibrates the read counters of kernels that load the same
 * way.  form DLC_READ_LDS: the FP4 indexer's key-stream form (bytes a
 * multiple of 1024).  form DLC_READ_TILES: the bf16 indexer's form (bytes a
 * multiple of 4096, read as 16-row tiles of 256-byte rows, lane l of a wave
 * loading row l%16 at byte 64*kt + 16*(l/16) for kt = 0..3).  Returns
 * DLC_E_INVAL for a NULL or misaligned src, a size that is not a multiple of
 * the form's unit or an unknown form.
 */
int dlc_read(const void* src, size_t bytes, int form, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DLC_H */
