/* topselect_testing.h -- test hooks of libtopselect.so, not part of the product interface.
 *
 * Callers: the library's own tests, which force each internal path of the kernels to check
 * that every path gives the same bytes. Nothing in the hot path needs these.
 */
#ifndef TOPSELECT_TESTING_H_
#define TOPSELECT_TESTING_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Test-only, bit-neutral path forcing. Each setting belongs to the calling thread: it
 * affects only the calls (and the ts_workspace_bytes results) of that thread, never another
 * thread's. With every knob at its default - the state of every thread that never calls
 * this - results and workspace sizes depend on the call arguments alone. Knobs:
 *   TS_KNOB_CHUNK_ELEMS   logits per stream-kernel chunk (0 = automatic, 8192 at most;
 *                         else a multiple of 64 in [64, 8192]): changes how a row is split
 *                         over workgroups. Also changes this thread's ts_workspace_bytes.
 *   TS_KNOB_FORCE_EXACT   1 = every top-k / top-p row takes the exact row-streaming path of
 *                         the row kernel instead of the certified candidate path.
 *   TS_KNOB_DIRECT        1 (default) = rows of at most 12288 logits run in the row kernel
 *                         alone, the row loaded straight into its LDS (one launch instead of
 *                         two); 0 = such rows also take the stream kernel. A forced chunk size
 *                         also turns it off.
 *   TS_KNOB_NUCLEUS_PASSES 1 = sampling calls without a top-k array always take the nucleus
 *                         passes for their top-p / min-p rows; 0 (default) = calls of at most
 *                         6,400,000 logits over rows of at most 100,000 take the split nucleus.
 * Every setting gives byte-identical results, with two exceptions under TS_KNOB_DIRECT: a
 * full-row sample (top-k and top-p off) rounds its perturbed scores in another order, so its
 * token can differ where two scores lie within a few fp32 ulps, and the LSE of
 * ts_sample_rows_logp can differ in its last bits. Returns the previous value, or -1 for an
 * unknown knob or an invalid value (the setting is then unchanged).
 */
#define TS_KNOB_CHUNK_ELEMS   1
#define TS_KNOB_FORCE_EXACT   2
#define TS_KNOB_DIRECT        3
#define TS_KNOB_NUCLEUS_PASSES 4
int64_t ts_debug_set(int knob, int64_t value);

#ifdef __cplusplus
}
#endif
#endif /* TOPSELECT_TESTING_H_ */
