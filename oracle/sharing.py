"""Which sequences of a batch share leading blocks, and how many positions.

Source: "vLLM PagedAttention and continuous batching", section "Sharing with
reference counts and copy-on-write": parallel samples and beams of one
prompt map the same physical blocks for the prompt; the last partial block
is copied before a write.  A kernel may read such positions once for all
the sequences that map them.

Definition written out (test infrastructure): the batch is cut into runs of
consecutive sequences; a run of two or more sequences whose first block is
the same physical block shares k * B positions, k = the number of leading
table entries all members agree on, capped at the shortest member's length
minus one and rounded down to a multiple of 16 (the processing granularity
of the kernels; the cap leaves every member the position this step writes);
other runs share nothing, and neighbouring runs that share nothing are one
run.
"""

from __future__ import annotations

from typing import List, Sequence, Tuple


def prefix_groups(tables: Sequence[Sequence[int]], lens: Sequence[int], B: int
                  ) -> Tuple[List[int], List[int], List[int]]:
    """Returns (group_start [n_groups + 1], group_len [n_groups], seq_group [S])."""
    S = len(lens)
    runs = []        # (first, end, shared)
    i = 0
    while i < S:
        j = i + 1
        if lens[i] > 0:
            while j < S and lens[j] > 0 and tables[j][0] == tables[i][0]:
                j += 1
        shared = 0
        if j - i >= 2:
            members = range(i, j)
            nb = min(-(-int(lens[m]) // B) for m in members)
            k = 0
            while k < nb and all(tables[m][k] == tables[i][k] for m in members):
                k += 1
            shared = min(k * B, min(int(lens[m]) for m in members) - 1)
            shared -= shared % 16
        if shared == 0 and runs and runs[-1][2] == 0:
            runs[-1] = (runs[-1][0], j, 0)
        else:
            runs.append((i, j, shared))
        i = j
    group_start = [r[0] for r in runs] + [S]
    group_len = [r[2] for r in runs]
    seq_group = [0] * S
    for g, (a, b, _) in enumerate(runs):
        for m in range(a, b):
            seq_group[m] = g
    return group_start, group_len, seq_group
