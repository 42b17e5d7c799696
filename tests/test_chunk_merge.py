"""The chunked-key row check used by the longest-sequence GPU test: oracle
results on key chunks merged by the two-partition rule of "FlashAttention-1:
eliminating IO", section 10.2.2, must equal the oracle's rows on all keys at
once (causal, so row r sees keys 0..r), for chunk sizes that split rows in
every way (one chunk, ragged last chunk, a chunk per key)."""
import numpy as np
import pytest

import oracle
from _util import rows_by_key_chunks


@pytest.mark.parametrize("chunk", [1, 7, 64, 500])
def test_chunk_merge_equals_full_rows(chunk):
    rng = np.random.default_rng(3)
    N, d = 300, 16
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    q[5] *= 20  # a peaked row
    rows = [0, 1, 5, 63, 64, 150, 298, 299]
    scale = 0.3
    o_ref, lse_ref = oracle.attn_fwd_rows(q, k, v, rows, scale, True)
    o, lse = rows_by_key_chunks(q[rows], rows, scale, chunk, N,
                                lambda a, b: (k[a:b], v[a:b]))
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-13, atol=1e-13)
