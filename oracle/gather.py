"""Stage 2b: assembling the selected documents' pooled rows (test infrastructure).

Source: neo-ai.one MSA article, 推論パイプライン (Fig. 3): only the selected
K̄/V̄ are loaded and concatenated with the local context; the content K̄/V̄ live
in host memory and are fetched on demand.

Reading taken: the selected documents' rows are concatenated in ascending doc
id order (attention is invariant to the order of memory rows, so one canonical
order is fixed for comparisons).  Pure indexing; no arithmetic.

Parity status: pinned (tests/test_oracle_gather.py): hand-written layouts whose
rows name their own index (ids out of order, adjacent documents, one-chunk
documents, the first and last document, no document) against the row lists
written out by hand.
"""

import numpy as np


def gather_rows(bank, doc_chunk_off, ids):
    """bank[N, ...], ids: selected doc ids of one query.  Returns the rows of
    the selected documents, ascending id order, and their count."""
    off = np.asarray(doc_chunk_off, dtype=np.int64)
    sel = sorted(int(i) for i in ids)
    if len(set(sel)) != len(sel):
        raise ValueError("duplicate doc id")
    parts = [bank[off[i]:off[i + 1]] for i in sel]
    if not parts:
        return bank[:0], 0
    out = np.concatenate(parts, axis=0)
    return out, out.shape[0]
