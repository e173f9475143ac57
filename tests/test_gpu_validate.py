"""attn_validate_inputs on device contents (the checks [DEC]
`triton_varlen_attn_func` makes before a launch: monotone cu_seqlens, one query
per sequence for decode; plus block-table range and zig-zag divisibility).
Bad contents only ever reach the validator, never a launch path."""

import pytest
import torch

from blockwise_causal_varlen_amd import lib as L

pytestmark = pytest.mark.gpu
CONTENT = 12  # ATTN_ERR_CONTENT


def say(*a):
    print(*a, flush=True)


def status(fn):
    try:
        fn()
        return 0
    except L.AttnError as e:
        say(f"  -> {e}")
        return e.status


def test_validate_inputs_rejects_bad_contents(gpu_lib):
    dev = "cuda"
    q = torch.zeros(64, 4, 128, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(64, 2, 128, dtype=torch.bfloat16, device=dev)
    good = torch.tensor([0, 16, 48, 64], dtype=torch.int32)
    say("valid cu_seqlens")
    assert status(lambda: L.validate_inputs(q, k, good, good, 32, 32)) == 0
    say("cu_seqlens that decrease")
    bad = torch.tensor([0, 40, 24, 64], dtype=torch.int32)
    assert status(lambda: L.validate_inputs(q, k, bad, good, 64, 64)) == CONTENT
    assert status(lambda: L.validate_inputs(q, k, good, bad, 64, 64)) == CONTENT
    say("cu_seqlens that do not start at 0")
    assert status(lambda: L.validate_inputs(q, k, good + 1, good, 64, 64)) == CONTENT
    say("a document longer than max_seqlen")
    assert status(lambda: L.validate_inputs(q, k, good, good, 31, 64)) == CONTENT
    say("cu_seqlens past the end of the tensors")
    over = torch.tensor([0, 16, 48, 80], dtype=torch.int32)
    assert status(lambda: L.validate_inputs(q, k, over, over, 64, 64)) == CONTENT
    say("zig-zag: every document a multiple of 2 cp")
    assert status(lambda: L.validate_inputs(q, k, good, good, 32, 32, zigzag_cp=2)) == 0   # 16, 32, 16
    assert status(lambda: L.validate_inputs(q, k, good, good, 32, 32, zigzag_cp=3)) == CONTENT   # 16 % 6
    say("decode: one query per sequence")
    one = torch.arange(4, dtype=torch.int32)
    assert status(lambda: L.validate_inputs(q, k, one, good, 1, 32, one_query=1)) == 0
    assert status(lambda: L.validate_inputs(q, k, good, good, 32, 32, one_query=1)) == CONTENT
    say("paged keys: block-table entries within the cache's pages")
    cache = torch.zeros(6, 2, 16, 128, dtype=torch.bfloat16, device=dev)   # 6 pages of 16 rows
    kd, pstride = L.paged_desc(cache)
    cu_k = torch.tensor([0, 64], dtype=torch.int32)                         # 4 logical blocks used
    q1 = q[:8]
    cu_q = torch.tensor([0, 8], dtype=torch.int32)
    for table, want in (([5, 0, 3, 1], 0), ([5, 0, 6, 1], CONTENT), ([5, -1, 3, 1], CONTENT)):
        bt = torch.tensor(table, dtype=torch.int32, device=dev)
        m = L.mask(causal=True, block_size=16, max_blocks=4, page_stride=pstride, block_table=bt)
        say(f"  table {table}")
        assert status(lambda: L.validate_inputs(q1, None, cu_q, cu_k, 8, 64, m=m, k_desc=kd)) == want
