"""The benchmark's closed-form work counts agree with the oracle's pair count
(CPU)."""

import numpy as np
import pytest

import oracle as O
from blockwise_causal_varlen_amd import inputs, workloads as W


@pytest.mark.parametrize("cp", [2, 4, 8])
def test_zigzag_pairs(cp):
    lens = [16 * cp, 2 * cp, 40 * cp]
    cu = np.cumsum([0] + lens)
    cu_l = cu // cp
    for r in range(cp):
        n = sum(O.count_visible_pairs(cu_l, cu_l, **O.zigzag_block_args(O.zigzag_step(r, s, cp)[1]))
                for s in range(cp))
        assert n == W.zigzag_rank_pairs(lens, cp)
        for s in range(cp):
            kind = O.zigzag_step(r, s, cp)[1]
            assert O.count_visible_pairs(cu_l, cu_l, **O.zigzag_block_args(kind)) == W.zigzag_step_pairs(lens, cp, s)


@pytest.mark.parametrize("window", [0, 37, 500])
@pytest.mark.parametrize("r", [0, 1, 3])
def test_kvp_pairs(window, r):
    s_q, goff, nb, bs, R = 50, 700, 20, 16, 4
    n_local = nb * bs
    want = O.count_visible_pairs([0, s_q], [0, n_local], causal=True, window=window, q_pos_offset=goff,
                                 kv_interleave=R, kv_rank=r, block_size=bs)
    assert W.kvp_rank_pairs(s_q, goff, n_local, R, r, bs, window) == want


def test_kvp_pairs_full_size_w0():
    """cfg4 at W=0: 1568 of 2048 local blocks per rank are (partly) visible."""
    tot = sum(W.kvp_rank_pairs(2048, 98304, 32768, 4, r, 16, 0) for r in range(4))
    assert tot == 203424768


def test_decode_bytes():
    k_lens = np.array([1, 2048, 7])
    b = W.decode_bytes(k_lens, 32, 4, 128)
    assert b == 2056 * 4 * 128 * 4 + 3 * 32 * 128 * 4 + 3 * 32 * 4 + 8 * 4
