"""Pins of the oracle's stage 2b (assembling the selected documents' rows).

The neo-ai.one MSA article (推論パイプライン, Fig. 3) loads only the selected
documents' pooled K̄/V̄ and places them before the local context.  The oracle
fixes ascending document id as the canonical order.  Each bank row here holds
its own row index, so the expected output is the list of row numbers written
out by hand from the layout below; a wrong offset, a dropped or repeated
document, selection order instead of id order, or an off-by-one at a document
boundary changes that list.
"""

import numpy as np
import pytest

import oracle

# Hand-written layout: 7 documents over 16 chunk rows.
#   doc:    0       1    2   3        4     5   6
#   rows: [0,1,2] [3,4] [5] [6,7,8,9] [10] [11] [12,13,14,15]
OFF = [0, 3, 5, 6, 10, 11, 12, 16]


def _bank(n=16, width=3):
    """Row r holds (r, r + 0.25, r + 0.5, ...), so every element names its row."""
    return np.arange(n, dtype=np.float64)[:, None] + 0.25 * np.arange(width)[None, :]


def _rows(out):
    return [int(r) for r in out[:, 0]]


def test_out_of_order_ids_come_back_in_ascending_id_order():
    out, m = oracle.gather_rows(_bank(), OFF, [6, 1, 3])
    assert m == 2 + 4 + 4
    assert _rows(out) == [3, 4, 6, 7, 8, 9, 12, 13, 14, 15]


def test_adjacent_documents_are_contiguous_without_gap_or_overlap():
    out, m = oracle.gather_rows(_bank(), OFF, [3, 2, 4, 5])
    assert m == 1 + 4 + 1 + 1
    assert _rows(out) == [5, 6, 7, 8, 9, 10, 11]


def test_one_chunk_documents_and_the_first_and_last_document():
    out, m = oracle.gather_rows(_bank(), OFF, [5, 0, 2])
    assert m == 3 + 1 + 1
    assert _rows(out) == [0, 1, 2, 5, 11]
    out, m = oracle.gather_rows(_bank(), OFF, [6])
    assert m == 4 and _rows(out) == [12, 13, 14, 15]


def test_whole_rows_are_copied_unchanged():
    bank = _bank(width=5)
    out, _ = oracle.gather_rows(bank, OFF, [4, 1])
    np.testing.assert_array_equal(out, np.array([[r + 0.25 * j for j in range(5)]
                                                 for r in (3, 4, 10)]))


def test_trailing_axes_are_carried_along():
    # rows shaped like the pooled bank's [2][Hkv][d]
    bank = np.arange(16 * 2 * 2 * 3, dtype=np.float64).reshape(16, 2, 2, 3)
    out, m = oracle.gather_rows(bank, OFF, [1])
    assert m == 2 and out.shape == (2, 2, 2, 3)
    np.testing.assert_array_equal(out[0], bank[3])
    np.testing.assert_array_equal(out[1], bank[4])


def test_all_documents_give_the_whole_bank():
    out, m = oracle.gather_rows(_bank(), OFF, [6, 5, 4, 3, 2, 1, 0])
    assert m == 16 and _rows(out) == list(range(16))


def test_no_documents_give_no_rows():
    out, m = oracle.gather_rows(_bank(), OFF, [])
    assert m == 0 and out.shape == (0, 3)


def test_duplicate_id_is_rejected():
    with pytest.raises(ValueError):
        oracle.gather_rows(_bank(), OFF, [2, 2])
