"""Greedy verification of a speculative-decoding round, written as its definition.

ORACLE -- test infrastructure only (tests, smoke check, CPU-baseline leg of the
benchmark); shares no code with the library.

A round feeds the target model the last accepted token followed by k draft
tokens d_1 .. d_k, so the verification pass has M = k + 1 rows; row m holds
the target's state after the last accepted token (m = 0) or after draft m,
and its argmax t_m is the target's greedy choice for the next token.  Greedy
speculative decoding (Leviathan, Kalman and Matias, "Fast Inference from
Transformers via Speculative Decoding", 2023, the temperature-zero case)
accepts d_1, d_2, ... as long as each equals the target's choice before it,
d_{j+1} == t_j, and then commits the accepted drafts plus the target's
choice after them, t_L.  The author's post runs such rounds with k = 7 native
MTP drafts and counts the tokens committed per round (5.89 on its workload).
"""


def verify_greedy(idx, drafts):
    """idx: the M per-row argmax tokens t_0 .. t_{M-1}; drafts: d_1 .. d_{M-1}.

    Returns (L, committed): L accepted drafts and the L + 1 committed tokens."""
    idx = [int(v) for v in idx]
    drafts = [int(v) for v in drafts]
    assert len(drafts) == len(idx) - 1
    L = 0
    while L < len(drafts) and drafts[L] == idx[L]:
        L += 1
    return L, drafts[:L] + [idx[L]]
