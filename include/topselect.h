/*
 * topselect.h -- C ABI of the MI355X (gfx950) batched per-row vocabulary sampler.
 *
 * Three operations on fp32 logits laid out row-major as [rows, row_stride] (row r starts
 * at logits + r * row_stride; only the first `vocab` entries of a row are read):
 *
 *   ts_topk_select   deterministic top-k select with index-ordered ties;
 *   ts_topp_mask     softmax + top-p nucleus (probability-space predicate, row max kept);
 *   ts_sample_rows   Gumbel-max sampling over the kept set, log1p(-u) noise, Philox4x32-10.
 *
 * Sources (page title, then section):
 *   [DETK]   vLLM PR #55122 "[Kernel] Make persistent_topk deterministic" -- "Changes"
 *            (exact radix select, index-ordered ties, ascending-index output, per-CTA
 *            >/== counts prefix-summed in CTA order) and "Test plan" (short rows padded -1).
 *   [TOPP]   "Split top-p numerical reference and conservative gate" -- "Source basis"
 *            (predicate in probability space, keep the row maximum), "Independent binary64
 *            numerical reference" (canonical order, p taken after fp32 conversion, reaching
 *            p keeps), "Breakage probes" (non-finite inputs fail closed).
 *   [GUMBEL] prhub summary of vLLM PR #45996 -- "implementation breakdown" and "key source
 *            excerpts" (g = -log(-log1p(-u)), u clamped at the generator's minimum, per-row
 *            seed and temperature applied inside the kernel, max with its index).
 *   [LOGP]   RL-Kernel issue #332 "Deterministic SM90 linear_logp" -- "Integration"
 *            (transform order temperature -> top-k -> top-p) and "Contract constants"
 *            (padded / masked lanes contribute 0 mass; reduction shape independent of batch).
 *   [REJ]    mlxcel issue #901 -- "Task" (one launch for the batch with per-row parameters;
 *            masked, zero-probability entries are never sampled).
 *
 * Conventions shared by all three operations:
 *   - Every pointer argument except `workspace`'s size query is a DEVICE pointer unless
 *     noted. The caller owns all memory; the library never allocates, frees or copies to
 *     the host inside these calls.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*, NULL = the null
 *     stream): they enqueue kernels and return; they never synchronise.
 *   - rows == 0 (an empty batch) returns TS_OK at once once vocab and row_stride are valid:
 *     nothing is read or written and every pointer may be NULL.
 *   - Ordering of a row: by (logit descending, token id ascending); -0.0 and +0.0 are equal.
 *     Top-k ranks the raw fp32 logits; temperature enters only exp((x - max)/T) and the
 *     Gumbel score (x - max)/T + g.
 *   - Per-row parameters: k >= vocab means top-k off; p == 1.0f means top-p off; T == 0
 *     means greedy (the first token of the ordering). NULL parameter arrays mean: top_k
 *     off, top_p = 1, temperature = 1.
 *   - -inf logits are masked tokens (weight 0, never sampled). NaN or +inf logits, or a
 *     row of only -inf, reject the row (for ts_topk_select only NaN rejects).
 *   - Per-row problems are reported in row_status[r] (if row_status is non-NULL) and the
 *     row's outputs are poisoned (-1 ids, kept count 0, all-zero mask row); other rows are
 *     unaffected. Codes, by precedence: TS_ROW_NONFINITE, TS_ROW_BAD_K, TS_ROW_BAD_P,
 *     TS_ROW_BAD_T, TS_ROW_BAD_MINP.
 *   - Host-side argument errors return a negative TS_ERR_* code before anything is
 *     enqueued; ts_last_error() then holds a thread-local message.
 *   - Workspace: device memory of at least ts_workspace_bytes(op, rows, vocab, k_max)
 *     bytes, 256-byte aligned, owned by the caller. It needs no initialisation: every call
 *     writes what it later reads (per-wave chunk summaries, then candidate slices). With
 *     the default chunking it is no larger than the logits it covers (the 64 x 151936
 *     decode batch: 38.4 MB). One workspace serves one call at a time: calls that overlap
 *     on one workspace race.
 *   - Results are deterministic: the same inputs give the same output bytes on every
 *     call, independent of how rows are split over workgroups.
 */
#ifndef TOPSELECT_H_
#define TOPSELECT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes of the host API. */
#define TS_OK               0
#define TS_ERR_INVALID_ARG  (-1)   /* null pointer, rows < 0, vocab < 1, stride < vocab, ... */
#define TS_ERR_WORKSPACE    (-2)   /* workspace NULL, misaligned or smaller than required */
#define TS_ERR_UNSUPPORTED  (-3)   /* no HIP device, or the device is not gfx950 */
#define TS_ERR_LAUNCH       (-4)   /* a HIP launch failed; detail in ts_last_error() */

/* Per-row status codes written to row_status[r]. */
#define TS_ROW_OK           0
#define TS_ROW_NONFINITE    1      /* NaN or +inf logits, or every logit is -inf */
#define TS_ROW_BAD_K        2      /* k < 1, or (ts_topk_select) min(k, row_len) > k_max */
#define TS_ROW_BAD_P        3      /* p not in (0, 1] (NaN included) */
#define TS_ROW_BAD_T        4      /* temperature negative, NaN or infinite */
#define TS_ROW_BAD_MINP     5      /* min_p outside [0, 1] or NaN (the _minp entry points) */

/* Operation ids for ts_workspace_bytes. */
#define TS_OP_TOPK_SELECT   0
#define TS_OP_TOPP_MASK     1
#define TS_OP_SAMPLE_ROWS   2

/* Largest supported row length (ids are int32). */
#define TS_MAX_VOCAB        ((int64_t)1 << 30)

/*
 * Workspace size in bytes for one call of `op` on `rows` rows of `vocab` logits
 * (k_max is the ts_topk_select output width; ignored for the other ops). Returns 0 for
 * invalid sizes. Pure host function: needs no device.
 */
size_t ts_workspace_bytes(int op, int64_t rows, int64_t vocab, int32_t k_max);

/* Zero-fill a workspace (enqueued on `stream` as a fill kernel, no memset node). Optional:
 * the operations need no initialised workspace; this only makes its contents defined. */
int ts_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * ts_topk_select -- [DETK] "Changes": exact top-k by (value desc, index asc).
 *   keys        [rows, row_stride] fp32, read-only.
 *   k           [rows] int32, per-row k (>= 1). k >= row_len selects the whole row.
 *   k_max       width of out_idx; every row needs min(k[r], row_len) <= k_max.
 *   out_idx     [rows, k_max] int32, written: the selected ids in ASCENDING id order,
 *               then -1 in the unused slots ([DETK] "Test plan": short rows).
 *   row_status  [rows] int32 or NULL.
 */
int ts_topk_select(const float* keys, int64_t rows, int64_t row_len, int64_t row_stride,
                   const int32_t* k, int32_t k_max, int32_t* out_idx, int32_t* row_status,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * ts_topk_select_rows -- ts_topk_select for sparse-indexer rows of varying length ([DETK]
 * "Changes": filtered-row length clamping; "Test plan": short rows, -1 padding):
 *   lengths  [rows] int32 or NULL: only keys [0, n) of row r take part, n = lengths[r]
 *            clamped to [0, row_len]; NULL = row_len. A NaN at or past n is ignored. The
 *            row's k_eff = min(k[r], n) (status TS_ROW_BAD_K if it exceeds k_max); an empty
 *            row gives k_max slots of -1.
 *   order    TS_ORDER_INDEX: the selected ids ascending (as ts_topk_select);
 *            TS_ORDER_VALUE: in the row ordering itself, value descending then id ascending
 *            (the order a value-ordered top-k returns); needs k_max <= 8192.
 *   offsets  [rows] int32 or NULL: added to every emitted id of row r (the row's start in a
 *            ragged index space); the caller keeps offset + id within int32.
 * Other arguments and the workspace as for ts_topk_select (the workspace is sized with
 * TS_OP_TOPK_SELECT for row_len).
 */
#define TS_ORDER_INDEX 0
#define TS_ORDER_VALUE 1
int ts_topk_select_rows(const float* keys, int64_t rows, int64_t row_len, int64_t row_stride,
                        const int32_t* lengths, const int32_t* k, int32_t k_max, int order,
                        const int32_t* offsets, int32_t* out_idx, int32_t* row_status, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * ts_topp_mask -- [TOPP] "Source basis" and "Independent binary64 numerical reference":
 * temperature -> top-k -> top-p. With w_i = exp((x_i - max)/T) over the top-k set K and
 * Z = sum_K w, the kept set P is the shortest prefix of K (in the row ordering) whose
 * weight reaches p * Z (>=). P always holds the row maximum.
 *   top_k, top_p, temperature   [rows] or NULL. With top_k NULL (top-k off for every row)
 *               and top_p or min_p given, rows of more than 12288 logits with top-p or
 *               min-p on spread their work over the row's chunk workgroups (two extra
 *               launches: mass histograms, then the cut bin); the results are the same
 *               bytes as with a top_k array of k >= vocab, which keeps one workgroup per row.
 *   out_kept    [rows] int32: |P|.
 *   out_mask    [rows, vocab] uint8 or NULL: 1 for tokens in P, else 0 (dense, row pitch
 *               = vocab bytes).
 */
int ts_topp_mask(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride,
                 const int32_t* top_k, const float* top_p, const float* temperature,
                 int32_t* out_kept, uint8_t* out_mask, int32_t* row_status,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * ts_sample_rows -- [GUMBEL] "key source excerpts": one token per row,
 * argmax over P of (x_i - max)/T + g_i with g_i = -log(-log1p(-u_i)) in fp32 and the
 * lowest id winning exact ties; T == 0 returns the first token of the row ordering.
 *   seed        [rows] uint64, required: u_i comes from Philox4x32-10 (Salmon et al.,
 *               SC'11) with key (seed mod 2^32, seed div 2^32), counter (i div 4, r, 0, 0),
 *               output word i mod 4; u = fp32(word * 2^-32) clamped to [2^-32, 1 - 2^-24].
 *               r is the row's index within this call.
 *   out_token   [rows] int32.
 */
int ts_sample_rows(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride,
                   const int32_t* top_k, const float* top_p, const float* temperature,
                   const uint64_t* seed, int32_t* out_token, int32_t* row_status,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * ts_sample_rows_noalloc -- ts_sample_rows for callers that cannot allocate: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments and the
 * same results (byte for byte) as ts_sample_rows, without the workspace: the library keeps it
 * in a static device array of 16 MiB per GPU (held from the library's load until the process
 * ends), found once per device with hipGetSymbolAddress. The call allocates nothing. Its
 * candidate slices hold at most 256 candidates per wave; rows whose waves publish more
 * (massive ties) take the exact path, which gives the same bytes at a higher cost.
 * Limit: the batch must fit the scratch (about 8.4 KB per 8192-logit chunk of a row plus
 * 8.3 KB per row: the 64 x 151936 decode batch takes 11 MB); larger batches fail with
 * TS_ERR_INVALID_ARG and a message in ts_last_error, before any device work.
 * Calls that overlap on one GPU (other streams, other threads) share the one array and race;
 * serialise them. Nothing in the array needs to start at zero.
 */
int ts_sample_rows_noalloc(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride,
                           const int32_t* top_k, const float* top_p, const float* temperature,
                           const uint64_t* seed, int32_t* out_token, int32_t* row_status, void* stream);

/*
 * ts_sample_rows_logp -- ts_sample_rows plus the sampled token's log-probability under the
 * row's temperature-scaled distribution, [LOGP] "Design: the numeric contract" with
 * temperature applied in the epilogue ([LOGP] "Contract constants"): over the WHOLE row
 * (before top-k / top-p), m = max x, S = sum exp((x - m)/T), lse = m/T + log S,
 * logp = min(x_t/T - lse, 0) for the returned token t. -inf logits contribute 0 to S.
 *   out_token   [rows] int32, identical to what ts_sample_rows returns for the same inputs.
 *   out_logp    [rows] fp32, required.
 *   out_lse     [rows] fp32, or NULL.
 * S is accumulated per 2048-element wave slice (fp32 exponentials of the slice's elements
 * relative to its maximum, binary64 sums) and combined in slice order after rescaling to
 * the row maximum: the same bits for every call with the same vocabulary, independent of
 * the batch. Rows with a non-OK status get NaN in both outputs; greedy rows (T == 0) get
 * logp 0 and lse +inf. The workspace is the one sized for TS_OP_SAMPLE_ROWS.
 */
int ts_sample_rows_logp(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride,
                        const int32_t* top_k, const float* top_p, const float* temperature,
                        const uint64_t* seed, int32_t* out_token, float* out_logp, float* out_lse,
                        int32_t* row_status, void* workspace, size_t workspace_bytes, void* stream);

/*
 * ts_topp_mask_minp, ts_sample_rows_minp -- ts_topp_mask and ts_sample_rows with a min-p
 * step after top-p, in the pinned transform order temperature -> top-k -> top-p -> min-p
 * ([LOGP] "Integration", relay program with pinned order; [REJ] "Task": min-p on
 * probabilities). A token of the top-p set stays when its probability is at least
 * min_p[r] times the row's largest, i.e. when exp((x - max) / T) >= min_p[r]; the row maximum
 * always stays and the result is again a prefix of the row ordering (out_kept, out_mask and
 * the sampled token refer to it).
 *   min_p   [rows] fp32, required: 0 = off; outside [0, 1] or NaN -> TS_ROW_BAD_MINP.
 * The weight is the one the top-p step uses (an fp32 exp2 of a binary64 exponent, about
 * 1.6e-7 relative), so a token whose weight lies within that of min_p can fall on either
 * side. Rows that would take the full-row path (top-k and top-p off) take the exact
 * row-streaming path when min-p is on. Other arguments as for ts_topp_mask / ts_sample_rows.
 */
int ts_topp_mask_minp(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride,
                      const int32_t* top_k, const float* top_p, const float* temperature,
                      const float* min_p, int32_t* out_kept, uint8_t* out_mask, int32_t* row_status,
                      void* workspace, size_t workspace_bytes, void* stream);
int ts_sample_rows_minp(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride,
                        const int32_t* top_k, const float* top_p, const float* temperature,
                        const float* min_p, const uint64_t* seed, int32_t* out_token,
                        int32_t* row_status, void* workspace, size_t workspace_bytes, void* stream);

/*
 * ts_sample_rows_rejection -- sorting-free sampling by dual-pivot rejection ([REJ] mlxcel
 * issue #901 "Sorting-free top-k/top-p/min-p sampling with dual-pivot rejection kernels",
 * "Background": per round one candidate from a CDF scan over the tokens above the lower
 * bound, a second pivot halfway to the upper bound, counts and masses above both, accept or
 * shrink; "Task" item 2: a round cap with an exact fallback for the row).
 *
 * Support of row r: the first n tokens of the row ordering, n = min(k, n_p, n_m), where n_p
 * is the shortest prefix whose probability mass reaches top_p[r] over the WHOLE row (the
 * joint filter: top-k and top-p tested together against the full distribution, unlike
 * ts_sample_rows, whose top-p is taken over the top-k set) and n_m counts the tokens with
 * exp((x - max) / T) >= min_p[r]. The token is drawn with probability proportional to
 * exp((x - max) / T) on the support (masses as integers floor(w * 2^S), S = 63 - bitlen(vocab);
 * each round's random word is word 0 of Philox4x32-10 keyed by seed[r] at counter
 * (round, r, 1, 0), drawn against floor(word * mass / 2^32)). Equal logits rank by id.
 *   top_k, top_p, temperature, min_p   [rows] device arrays or NULL (off / 1 / 1 / 0);
 *                 T == 0 is greedy (the first token of the ordering).
 *   seed        [rows] u64, required.
 *   max_rounds  rejection rounds before the fallback, in [0, 64] (else TS_ERR_INVALID_ARG);
 *               a row that reaches it finds its support's last token by bisection over the
 *               row ordering and draws once over the support (the word of counter
 *               (max_rounds, r, 1, 0)).
 *   out_token   [rows] i32, required: the token, -1 for rejected rows.
 *   out_rounds  [rows] i32 or NULL: the accepting round (1-based), 0 for greedy or rejected
 *               rows, -1 when the fallback drew the token.
 *   row_status  [rows] i32 or NULL: as for ts_sample_rows_minp.
 * Needs no workspace: one 1024-thread workgroup per row reads the row from global memory
 * once per pass (two passes, then one per round). Weights are fp32-accurate (about 1.6e-7
 * relative), so a draw within that of a mass boundary may fall on either side.
 */
int ts_sample_rows_rejection(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride,
                             const int32_t* top_k, const float* top_p, const float* temperature,
                             const float* min_p, const uint64_t* seed, int32_t max_rounds,
                             int32_t* out_token, int32_t* out_rounds, int32_t* row_status,
                             void* stream);

/*
 * Diagnostic: the noise the sampler uses. For each tokens[j] of row `row` under `seed`,
 * writes the Philox word, u and g (all device arrays of n entries; any output may be NULL).
 */
int ts_gumbel_noise(uint64_t seed, int32_t row, const int32_t* tokens, int64_t n,
                    uint32_t* out_word, float* out_u, float* out_g, void* stream);
/*
 * Diagnostic: the sampler's word -> (u, g) map on given 32-bit words (device arrays of n
 * entries; either output may be NULL): u = fp32(word * 2^-32) clamped to [2^-32, 1 - 2^-24]
 * and g = -log(-log1p(-u)) ([GUMBEL] "implementation breakdown"), as ts_sample_rows uses them.
 */
int ts_noise_transform(const uint32_t* words, int64_t n, float* out_u, float* out_g, void* stream);
/*
 * Diagnostic: a plain streaming read of the n floats at x (device, 16-byte aligned), launched
 * with the sampling stream kernel's shape (256-thread workgroups, eight non-temporal 16-byte
 * loads per thread, all in flight before any is used): the read bandwidth that kernel is
 * measured against. out (device, 4 * ceil(n / 8192) floats) receives one fp32 partial sum per
 * wave; together they sum to the n floats (the stores keep the loads). Asynchronous on
 * `stream`; TS_ERR_INVALID_ARG for n < 0, a NULL or misaligned pointer.
 */
int ts_read_ceiling(const float* x, int64_t n, float* out, void* stream);

const char* ts_status_string(int status);  /* static string for a TS_* or TS_ROW_* code */
const char* ts_last_error(void);           /* thread-local detail of the last host error */

#ifdef __cplusplus
}
#endif
#endif /* TOPSELECT_H_ */
