"""CPU oracle (binary64) for the batched top-k / top-p / Gumbel-max sampling path.

TEST INFRASTRUCTURE ONLY: imported by tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``, never by the library itself. It shares no code,
header, table or constant generator with the HIP library.

Parity pins (see tests/test_oracle_*.py): brute-force ranks and subset enumeration on
V <= 16, closed forms (all-equal rows, two-token rows, dominant tokens, p = 1), library
cross-checks (numpy stable argsort, scipy logsumexp), an independent Philox4x32
implementation (Triton's CPU interpreter, when importable), the inverse Gumbel CDF, and
chi-square / z tests of the sampling law; for the rejection sampler, hand-worked
trajectories with injected random words and the law of the truncated distribution. No function here is "parity unpinned".
"""
from .philox import philox4x32, philox4x32_np, seed_key, token_words
from .rejection import RejectionResult, rejection_sample_row, rejection_sample_rows, round_word
from .sampler import (
    STATUS_BAD_K,
    STATUS_BAD_MINP,
    STATUS_BAD_P,
    STATUS_BAD_T,
    STATUS_NONFINITE,
    STATUS_OK,
    SampleResult,
    ToppResult,
    canonical_order,
    gumbel_argmax,
    gumbel_from_word,
    gumbel_noise,
    lse_logp_row,
    minp_filter,
    neumaier_first_reach,
    row_floats,
    sample_logp_rows,
    sample_minp_row,
    sample_rows_minp,
    sample_row,
    sample_rows,
    to_f32,
    ORDER_INDEX,
    ORDER_VALUE,
    topk_select,
    topk_select_row,
    topk_select_rows,
    topk_select_rows_row,
    topp_mask,
    topp_minp_mask,
    topp_minp_row,
    topp_row,
    uniform_from_word,
)
