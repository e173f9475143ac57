"""Pins of the fp64 oracle against things other than itself.

Brute-force loops, closed forms, finite differences, a library routine
(torch SDPA on the CPU in fp64) and the facts the pages state
(tests/golden/page_facts.json). Every test here runs on the CPU.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
FACTS = json.load(open(os.path.join(HERE, "golden", "page_facts.json")))


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# --------------------------------------------------------------------------
# brute force: pure Python loops written from the definition, no numpy algebra
# --------------------------------------------------------------------------
def brute_forward(q, k, v, cu_q, cu_k, scale, causal=False, q_view="all", k_view="all", window=0,
                  q_off=0, k_off=0, R=0, r=0, bs=0):
    nq, hq, d = q.shape
    hkv = k.shape[1]
    out = [[[0.0] * d for _ in range(hq)] for _ in range(nq)]
    lse = [[-math.inf] * nq for _ in range(hq)]
    for doc in range(len(cu_q) - 1):
        qs, qe, ks, ke = cu_q[doc], cu_q[doc + 1], cu_k[doc], cu_k[doc + 1]
        for i in range(qs, qe):
            t = i - qs
            nqd = qe - qs
            if q_view == "front" and not t < nqd // 2:
                continue
            if q_view == "back" and not t >= nqd // 2:
                continue
            for h in range(hq):
                g = h * hkv // hq
                terms = []
                for j in range(ks, ke):
                    u = j - ks
                    nkd = ke - ks
                    if k_view == "front" and not u < nkd // 2:
                        continue
                    if k_view == "back" and not u >= nkd // 2:
                        continue
                    qp = q_off + t
                    kp = k_off + (((u // bs) * R + r) * bs + u % bs if R else u)
                    if causal and kp > qp:
                        continue
                    if window and kp <= qp - window:
                        continue
                    s = scale * sum(q[i, h, x] * k[j, g, x] for x in range(d))
                    terms.append((s, j))
                if not terms:
                    continue
                z = sum(math.exp(s) for s, _ in terms)
                lse[h][i] = math.log(z)
                for x in range(d):
                    out[i][h][x] = sum(math.exp(s) * v[j, g, x] for s, j in terms) / z
    return np.array(out), np.array(lse)


CASES = [
    dict(causal=True),
    dict(),
    dict(k_view="front"),
    dict(q_view="back"),
    dict(q_view="front", k_view="back"),
    dict(causal=True, window=3),
    dict(causal=True, q_off=40, k_off=0, R=3, r=1, bs=4),
    dict(causal=True, window=9, q_off=40, R=3, r=2, bs=4),
    dict(causal=True, q_off=5, k_off=2),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("gqa", [(2, 2), (4, 2), (4, 1)])
def test_forward_matches_brute_force(case, gqa):
    hq, hkv = gqa
    cu_q = [0, 6, 6, 16, 21]
    cu_k = [0, 6, 9, 19, 28] if "R" in case or "k_off" in case else cu_q
    q, k, v = rnd((cu_q[-1], hq, 5), 1), rnd((cu_k[-1], hkv, 5), 2), rnd((cu_k[-1], hkv, 5), 3)
    scale = 0.37
    ref_o, ref_l = brute_forward(q, k, v, cu_q, cu_k, scale, **case)
    kw = dict(causal=case.get("causal", False), q_view=case.get("q_view", "all"),
              k_view=case.get("k_view", "all"), window=case.get("window", 0),
              q_pos_offset=case.get("q_off", 0), k_pos_offset=case.get("k_off", 0),
              kv_interleave=case.get("R", 0), kv_rank=case.get("r", 0), block_size=case.get("bs", 0))
    o, l = O.block_forward(q, k, v, cu_q, cu_k, scale, chunk=4, **kw)
    assert np.array_equal(np.isfinite(l), np.isfinite(ref_l))
    fin = np.isfinite(ref_l)
    assert np.max(np.abs(l[fin] - ref_l[fin]), initial=0) < 1e-12
    assert np.max(np.abs(o - ref_o)) < 1e-12


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
def test_single_key_closed_form_from_page():
    f = FACTS["single_key_lse"]
    q = np.array(f["q"])[None, None, :]
    k = np.array(f["k"])[None, None, :]
    v = np.array(f["v"])[None, None, :]
    o, l = O.block_forward(q, k, v, [0, 1], [0, 1], f["scale"], causal=True)
    assert l[0, 0] == pytest.approx(f["lse"], abs=1e-15)
    assert np.allclose(o[0, 0], f["out"], atol=0)


def test_two_key_closed_form():
    # q=(1,0), keys e1,e2, values e1,e2, scale 1: scores (1, 0)
    q = np.array([[[1.0, 0.0]]])
    k = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    v = k.copy()
    o, l = O.block_forward(q, k, v, [0, 1], [0, 2], 1.0)
    e = math.e
    assert l[0, 0] == pytest.approx(math.log(e + 1), abs=1e-15)
    assert o[0, 0] == pytest.approx([e / (e + 1), 1 / (e + 1)], abs=1e-15)


def test_causal_three_token_closed_form():
    q = np.full((3, 1, 1), 2.0)
    k = np.array([0.0, 2.0, 4.0]).reshape(3, 1, 1)
    v = np.array([1.0, 10.0, 100.0]).reshape(3, 1, 1)
    o, l = O.block_forward(q, k, v, [0, 3], [0, 3], 0.5, causal=True)
    e2, e4 = math.exp(2), math.exp(4)
    assert l[0].tolist() == pytest.approx([0.0, math.log(1 + e2), math.log(1 + e2 + e4)], abs=1e-14)
    assert o[:, 0, 0].tolist() == pytest.approx(
        [1.0, (1 + 10 * e2) / (1 + e2), (1 + 10 * e2 + 100 * e4) / (1 + e2 + e4)], rel=1e-14)


def test_zero_query_gives_mean_and_log_count():
    cu = [0, 7, 12]
    k, v = rnd((12, 2, 4), 5), rnd((12, 2, 4), 6)
    q = np.zeros((12, 2, 4))
    o, l = O.block_forward(q, k, v, cu, cu, 0.7, causal=True)
    for doc in range(2):
        for i in range(cu[doc], cu[doc + 1]):
            n = i - cu[doc] + 1
            assert l[:, i] == pytest.approx([math.log(n)] * 2, abs=1e-14)
            assert np.allclose(o[i], v[cu[doc]:i + 1].mean(axis=0), atol=1e-14)


def test_identical_keys_uniform_weights():
    k = np.tile(rnd((1, 1, 8), 7), (9, 1, 1))
    q, v = rnd((9, 1, 8), 8), rnd((9, 1, 8), 9)
    o, _ = O.block_forward(q, k, v, [0, 9], [0, 9], 0.3)
    assert np.allclose(o[:, 0], np.broadcast_to(v[:, 0].mean(axis=0), (9, 8)), atol=1e-14)


def test_empty_row_zero_and_neg_inf():
    assert FACTS["empty_row"]["out"] == 0.0
    q, k, v = rnd((4, 2, 3), 1), rnd((4, 2, 3), 2), rnd((4, 2, 3), 3)
    # window 1 with offset puts every key after the query -> nothing visible for row 0
    o, l = O.block_forward(q, k, v, [0, 4], [0, 4], 1.0, causal=True, k_pos_offset=1)
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(l[:, 0]))
    assert np.all(np.isfinite(l[:, 1:]))


def test_sdpa_library_cross_check():
    """torch SDPA (fp64, CPU, explicit block-diagonal causal mask, GQA by
    repeat_interleave) agrees with the oracle."""
    cu = [0, 13, 20, 41]
    hq, hkv, d = 6, 2, 16
    q, k, v = rnd((41, hq, d), 11), rnd((41, hkv, d), 12), rnd((41, hkv, d), 13)
    mask = torch.zeros(41, 41, dtype=torch.bool)
    for a, b in zip(cu[:-1], cu[1:]):
        mask[a:b, a:b] = torch.tril(torch.ones(b - a, b - a, dtype=torch.bool))
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).repeat_interleave(hq // hkv, dim=1).permute(1, 0, 2)
    tv = torch.from_numpy(v).repeat_interleave(hq // hkv, dim=1).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.25)
    o, l = O.block_forward(q, k, v, cu, cu, 0.25, causal=True)
    assert np.max(np.abs(o - ref.permute(1, 0, 2).numpy())) < 1e-12
    s = torch.einsum("hid,hjd->hij", tq, tk) * 0.25
    s = s.masked_fill(~mask, -math.inf)
    assert np.max(np.abs(l - torch.logsumexp(s, dim=-1).numpy())) < 1e-12


# --------------------------------------------------------------------------
# merge algebra and the partition invariant
# --------------------------------------------------------------------------
def _partials(seed, n=10, h=3, d=4):
    rng = np.random.default_rng(seed)
    o = rng.standard_normal((n, h, d))
    l = rng.standard_normal((h, n)) * 3
    l[0, 2] = -np.inf
    return o, l


def test_merge_algebra():
    a, b, c = _partials(1), _partials(2), _partials(3)
    ab = O.merge(*a, *b)
    ba = O.merge(*b, *a)
    assert np.allclose(ab[0], ba[0], atol=1e-14) and np.allclose(ab[1], ba[1], atol=1e-14)
    abc1 = O.merge(*O.merge(*a, *b)[:2], *c)
    abc2 = O.merge(*a, *O.merge(*b, *c)[:2])
    assert np.allclose(abc1[0], abc2[0], atol=1e-13) and np.allclose(abc1[1], abc2[1], atol=1e-13)
    ident = (np.zeros_like(a[0]), np.full_like(a[1], -np.inf))
    ai = O.merge(*a, *ident)
    fin = np.isfinite(a[1])
    assert np.allclose(ai[0][fin.T], a[0][fin.T]) and np.array_equal(ai[1], a[1])
    aa = O.merge(*a, *a)
    assert np.allclose(aa[1][fin], a[1][fin] + math.log(2), atol=1e-14)
    assert np.allclose(aa[0][fin.T], a[0][fin.T], atol=1e-14)
    both = O.merge(np.ones((1, 1, 2)), np.array([[-np.inf]]), np.ones((1, 1, 2)), np.array([[-np.inf]]))
    assert np.all(both[0] == 0) and np.isneginf(both[1][0, 0])


def test_merge_sigma_is_sigmoid_and_sigmoid_form():
    a, b = _partials(4), _partials(5)
    out, lse, sig = O.merge(*a, *b)
    with np.errstate(over="ignore", invalid="ignore"):
        expect = 1.0 / (1.0 + np.exp(a[1] - b[1]))
    fin = np.isfinite(lse)
    assert np.allclose(sig[fin], expect[fin], atol=1e-14)
    # sigmoid form: out = out_a - sigma (out_a - out_b)
    sform = a[0] - sig.T[:, :, None] * (a[0] - b[0])
    assert np.allclose(out[fin.T], sform[fin.T], atol=1e-13)


@pytest.mark.parametrize("split", [0, 3, 7, 12])
def test_partition_merge_equals_union(split):
    cu = [0, 12, 20]
    q, k, v = rnd((20, 2, 6), 21), rnd((20, 2, 6), 22), rnd((20, 2, 6), 23)
    full = O.block_forward(q, k, v, cu, cu, 0.5, causal=True)
    pa = O.block_forward(q, k, v, cu, cu, 0.5, causal=True, k_range=(0, split))
    pb = O.block_forward(q, k, v, cu, cu, 0.5, causal=True, k_range=(split, 10 ** 9))
    o, l, _ = O.merge(*pa, *pb)
    assert np.max(np.abs(o - full[0])) < 1e-12 and np.max(np.abs(l - full[1])) < 1e-12


# --------------------------------------------------------------------------
# gradients: finite differences, block sums, the lse_grad negative case
# --------------------------------------------------------------------------
def _loss(q, k, v, dout, cu, scale):
    o, _ = O.full_attention(q, k, v, cu, scale)
    return float(np.sum(o * dout))


def test_gradients_finite_differences():
    cu = [0, 5, 11]
    hq, hkv, d = 4, 2, 3
    q, k, v = rnd((11, hq, d), 31), rnd((11, hkv, d), 32), rnd((11, hkv, d), 33)
    dout = rnd((11, hq, d), 34)
    scale = 0.6
    dq, dk, dv = O.attention_grads(dout, q, k, v, cu, scale)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in itertools.product(*map(range, x.shape)):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = _loss(args["q"], args["k"], args["v"], dout, cu, scale)
            args[name] = xm
            fm = _loss(args["q"], args["k"], args["v"], dout, cu, scale)
            num[idx] = (fp - fm) / (2 * h)
        err = np.max(np.abs(num - g)) / max(1.0, np.max(np.abs(g)))
        assert err < 1e-6, (name, err)


def _zz_inputs(lens, hq, hkv, d, cp, seed):
    cu = np.cumsum([0] + lens)
    S = cu[-1]
    q, k, v, do = rnd((S, hq, d), seed), rnd((S, hkv, d), seed + 1), rnd((S, hkv, d), seed + 2), rnd((S, hq, d), seed + 3)
    loc = lambda x: [O.zigzag_shard(x, cu, cp, r)[0] for r in range(cp)]
    return cu, q, k, v, do, loc(q), loc(k), loc(v), loc(do)


@pytest.mark.parametrize("cp", [1, 2, 4, 8])
def test_zigzag_forward_equals_full_attention(cp):
    lens = [16 * cp, 2 * cp, 6 * cp]
    cu, q, k, v, do, ql, kl, vl, _ = _zz_inputs(lens, 4, 2, 8, cp, 40 + cp)
    fo, fl = O.full_attention(q, k, v, cu, 0.4)
    outs, lses = [], []
    for r in range(cp):
        o, l = O.zigzag_forward(ql, kl, vl, cu, cp, r, 0.4)  # also checks the step rule
        outs.append(o)
        lses.append(l)
    go = O.zigzag_unshard(outs, cu, cp)
    gl = O.zigzag_unshard([l.T for l in lses], cu, cp).T
    assert np.max(np.abs(go - fo)) < 1e-10 and np.max(np.abs(gl - fl)) < 1e-10


@pytest.mark.parametrize("cp", [2, 4])
def test_zigzag_backward_sums_to_full_gradient_and_lse_grad_variant_does_not(cp):
    lens = [8 * cp, 4 * cp]
    cu, q, k, v, do, ql, kl, vl, dol = _zz_inputs(lens, 4, 2, 6, cp, 60 + cp)
    scale = 0.45
    gdq, gdk, gdv = O.attention_grads(do, q, k, v, cu, scale)
    dq_l, dk_l, dv_l = [None] * cp, [np.zeros_like(x) for x in kl], [np.zeros_like(x) for x in vl]
    for r in range(cp):
        o, l = O.zigzag_forward(ql, kl, vl, cu, cp, r, scale, check=False)
        dq, dk, dv = O.zigzag_backward(dol[r], ql, kl, vl, o, l, cu, cp, r, scale)
        dq_l[r] = dq
        for s in range(cp):
            dk_l[s] += dk[s]
            dv_l[s] += dv[s]
    for got, want in ((dq_l, gdq), (dk_l, gdk), (dv_l, gdv)):
        assert np.max(np.abs(O.zigzag_unshard(got, cu, cp) - want)) < 1e-10
    # negative: each block's backward fed its OWN block lse/out (lse_grad-style) is wrong
    cu_l = cu // cp
    r = cp - 1
    dq_bad = np.zeros_like(ql[r])
    for s in range(cp):
        src, kind = O.zigzag_step(r, s, cp)
        a = O.zigzag_block_args(kind)
        bo, bl = O.block_forward(ql[r], kl[src], vl[src], cu_l, cu_l, scale, **a)
        dq_bad += O.block_backward(dol[r], ql[r], kl[src], vl[src], bo, bl, cu_l, cu_l, scale, **a)[0]
    assert np.max(np.abs(dq_bad - dq_l[r])) > 1e-2


def test_zigzag_shard_roundtrip_and_ownership():
    for cp, key in ((2, "cp2"), (4, "cp4")):
        L = 2 * cp * 3
        x = np.arange(L)
        for r in range(cp):
            loc, cu_l = O.zigzag_shard(x, [0, L], cp, r)
            chunks = sorted(set(loc // 3))
            assert chunks == FACTS["zigzag_ownership"][key][str(r)]
            assert cu_l.tolist() == [0, L // cp]
        assert np.array_equal(O.zigzag_unshard([O.zigzag_shard(x, [0, L], cp, r)[0] for r in range(cp)], [0, L], cp), x)


def test_zigzag_rule_rejects_a_wrong_rule():
    """The rule check inside zigzag_forward catches a swapped block kind."""
    with pytest.raises(AssertionError):
        O.attention._check_zigzag_rule([0, 16], 2, 1, 0, "q_back")
    with pytest.raises(AssertionError):
        O.attention._check_zigzag_rule([0, 16], 2, 0, 1, "kv_front")


def _pairs(cu, cp, r, zigzag):
    cu_l = np.asarray(cu) // cp
    n = 0
    for s in range(cp):
        if zigzag:
            src, kind = O.zigzag_step(r, s, cp)
            n += O.count_visible_pairs(cu_l, cu_l, **O.zigzag_block_args(kind))
        elif s <= r:
            n += O.count_visible_pairs(cu_l, cu_l, causal=(s == 0))
    return n


@pytest.mark.parametrize("cp,ratio", [(2, 1.5), (4, 1.75), (8, 1.875)])
def test_load_balance_claim(cp, ratio):
    L = 2 * cp * 64
    cu = [0, L]
    zz = [_pairs(cu, cp, r, True) for r in range(cp)]
    ring = [_pairs(cu, cp, r, False) for r in range(cp)]
    assert len(set(zz)) == 1 and sum(zz) == L * (L + 1) // 2 == sum(ring)
    assert ring[-1] / np.mean(ring) == pytest.approx(ratio, rel=0.01)


def test_ring_forward_backward_equals_full():
    cp, S = 4, 32
    cu = [0, S, 2 * S]  # two sequences (a batch of 2), each sharded contiguously
    q, k, v, do = rnd((2 * S, 2, 4), 81), rnd((2 * S, 2, 4), 82), rnd((2 * S, 2, 4), 83), rnd((2 * S, 2, 4), 84)
    loc = lambda x: [O.ring_shard(x, cu, cp, r)[0] for r in range(cp)]
    ql, kl, vl, dol = loc(q), loc(k), loc(v), loc(do)
    fo, fl = O.full_attention(q, k, v, cu, 0.5)
    gdq, gdk, gdv = O.attention_grads(do, q, k, v, cu, 0.5)
    dk_acc = [np.zeros_like(x) for x in kl]
    dv_acc = [np.zeros_like(x) for x in vl]
    steps = FACTS["ring_causal_steps"]["cp4"]
    for r in range(cp):
        o, l = O.ring_forward(ql, kl, vl, cu, cp, r, 0.5)
        want = np.concatenate([fo[b * S + r * S // cp: b * S + (r + 1) * S // cp] for b in range(2)])
        assert np.max(np.abs(o - want)) < 1e-10
        assert [s for s, _ in steps[str(r)]] == [str(r - s) for s in range(r + 1)]
        dq, dk, dv = O.ring_backward(dol[r], ql, kl, vl, o, l, cu, cp, r, 0.5)
        wq = np.concatenate([gdq[b * S + r * S // cp: b * S + (r + 1) * S // cp] for b in range(2)])
        assert np.max(np.abs(dq - wq)) < 1e-10
        for s in range(cp):
            dk_acc[s] += dk[s]
            dv_acc[s] += dv[s]
    for s in range(cp):
        wk = np.concatenate([gdk[b * S + s * S // cp: b * S + (s + 1) * S // cp] for b in range(2)])
        assert np.max(np.abs(dk_acc[s] - wk)) < 1e-10


# --------------------------------------------------------------------------
# KV-parallel
# --------------------------------------------------------------------------
def test_round_robin_positions_from_page():
    f = FACTS["round_robin_positions"]
    for c in f["cases"]:
        assert int(O.key_position(c["local_token"], 0, f["R"], c["rank"], f["block_size"])) == c["global_position"]


def test_contiguous_offset_formula_from_page():
    """Moving the offset to the q side (kvp_q_offset) gives the same mask as
    keeping global key positions."""
    for c in FACTS["kvp_q_offset_contiguous"]["cases"]:
        off = -c["rank"] * c["local_kv_len"] + c["global_q_offset"]
        assert off == c["kvp_q_offset"]
        qpos = c["global_q_offset"] + np.arange(0, 4096, 97)
        kloc = np.arange(0, c["local_kv_len"], 131)
        a = O.visibility(qpos, c["rank"] * c["local_kv_len"] + kloc, True, 4096)
        b = O.visibility(qpos - c["global_q_offset"] + off, kloc, True, 4096)
        assert np.array_equal(a, b)


@pytest.mark.parametrize("window", [0, 37])
@pytest.mark.parametrize("seg", [0, 16, 40])
def test_kvp_merge_equals_global_attention(window, seg):
    R, nb, bs, hq, hkv, d, nq = 4, 6, 4, 4, 1, 5, 13
    rng = np.random.default_rng(90)
    kc = [rng.standard_normal((nb, hkv, bs, d)) for _ in range(R)]
    vc = [rng.standard_normal((nb, hkv, bs, d)) for _ in range(R)]
    tabs = [rng.permutation(nb).reshape(1, -1) for _ in range(R)]
    q = rng.standard_normal((nq, hq, d))
    gq_off = 70  # global KV = 96 tokens, queries at 70..82
    o, l, parts = O.kvp_forward(q, kc, vc, tabs, nb, seg, gq_off, window, 0.5)
    gk = O.kvp_global_kv(kc, tabs, nb)
    gv = O.kvp_global_kv(vc, tabs, nb)
    ro, rl = O.block_forward(q, gk, gv, [0, nq], [0, gk.shape[0]], 0.5, causal=True, window=window,
                             q_pos_offset=gq_off)
    assert np.max(np.abs(o - ro)) < 1e-12 and np.max(np.abs(l - rl)) < 1e-12
    # the same global cache distributed contiguously gives the same answer
    paged = lambda x: x.reshape(R * nb, bs, hkv, d).transpose(0, 2, 1, 3)  # [blocks, HKV, bs, D]
    ck = [paged(gk)[i * nb:(i + 1) * nb] for i in range(R)]
    cv = [paged(gv)[i * nb:(i + 1) * nb] for i in range(R)]
    ident = [np.arange(nb).reshape(1, -1)] * R
    co, cl, _ = O.kvp_forward(q, ck, cv, ident, nb, seg, gq_off, window, 0.5, interleave=False)
    assert np.max(np.abs(co - ro)) < 1e-12 and np.max(np.abs(cl - rl)) < 1e-12


def test_page_table_direction_from_page():
    """Logical block b of a rank's keys is read from physical page block_table[b]
    (hand-worked table with a table that is not its own inverse)."""
    f = FACTS["page_table_direction"]
    nb, bs, d = f["num_blocks"], f["block_size"], 3
    cache = np.zeros((nb, 2, bs, d))
    for p in range(nb):
        for o in range(bs):
            cache[p, :, o, :] = 10 * p + o  # the value names (page, offset)
    got = O.kvp_gather_pages(cache, np.array([f["block_table"]]), nb)
    assert got.shape == (nb * bs, 2, d)
    for c in f["logical_token_reads"]:
        assert np.all(got[c["logical_token"]] == 10 * c["page"] + c["offset"]), c


# --------------------------------------------------------------------------
# block backward under the position-map and window masks
# --------------------------------------------------------------------------
MASKED_BWD_CASES = [
    dict(causal=True, window=3),
    dict(causal=True, window=4, q_pos_offset=7, k_pos_offset=2),
    dict(causal=True, q_pos_offset=9, kv_interleave=3, kv_rank=1, block_size=2),
    dict(causal=True, window=6, q_pos_offset=11, kv_interleave=2, kv_rank=1, block_size=3),
    dict(q_view="back", k_view="front"),
]


@pytest.mark.parametrize("mask", MASKED_BWD_CASES)
def test_block_backward_finite_differences_under_masks(mask):
    """block_backward fed the block's own (out, lse) is the gradient of
    L = sum(dout * out) of block_forward under the same mask; central
    differences of L check every element of dq, dk and dv."""
    cu_q, cu_k = [0, 5, 12], [0, 6, 14]
    hq, hkv, d = 4, 2, 3
    q, k, v = rnd((12, hq, d), 131), rnd((14, hkv, d), 132), rnd((14, hkv, d), 133)
    dout = rnd((12, hq, d), 134)
    scale = 0.55
    out, lse = O.block_forward(q, k, v, cu_q, cu_k, scale, **mask)
    assert np.isfinite(lse).sum() > 0
    dq, dk, dv = O.block_backward(dout, q, k, v, out, lse, cu_q, cu_k, scale, **mask)

    def loss(q_, k_, v_):
        return float(np.sum(dout * O.block_forward(q_, k_, v_, cu_q, cu_k, scale, **mask)[0]))

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in itertools.product(*map(range, x.shape)):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = loss(args["q"], args["k"], args["v"])
            args[name] = xm
            fm = loss(args["q"], args["k"], args["v"])
            num[idx] = (fp - fm) / (2 * h)
        assert np.max(np.abs(g)) > 1e-3, name  # the mask leaves gradient to check
        err = np.max(np.abs(num - g)) / max(1.0, np.max(np.abs(g)))
        assert err < 1e-6, (name, mask, err)


@pytest.mark.parametrize("mask", MASKED_BWD_CASES[:4])
def test_block_backward_key_split_sums_to_whole_under_masks(mask):
    """With the merged (out, lse) of the whole key range, the backward of any
    split of the keys (k_range parts) sums to the backward of the whole."""
    cu_q, cu_k = [0, 9, 20], [0, 10, 23]
    hq, hkv, d = 4, 1, 4
    q, k, v = rnd((20, hq, d), 141), rnd((23, hkv, d), 142), rnd((23, hkv, d), 143)
    dout = rnd((20, hq, d), 144)
    out, lse = O.block_forward(q, k, v, cu_q, cu_k, 0.5, **mask)
    whole = O.block_backward(dout, q, k, v, out, lse, cu_q, cu_k, 0.5, **mask)
    parts = [O.block_backward(dout, q, k, v, out, lse, cu_q, cu_k, 0.5, k_range=rg, **mask)
             for rg in ((0, 3), (3, 8), (8, 100))]
    for i in range(3):
        assert np.max(np.abs(sum(p[i] for p in parts) - whole[i])) < 1e-12


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------
def test_decode_is_softmax_weighted_average():
    lens = [1, 5, 17, 2]
    cu = np.cumsum([0] + lens)
    q, k, v = rnd((4, 8, 6), 91), rnd((cu[-1], 2, 6), 92), rnd((cu[-1], 2, 6), 93)
    o, l = O.decode_forward(q, k, v, cu, 0.3)
    for i in range(4):
        for h in range(8):
            g = h // 4
            s = np.array([0.3 * float(np.dot(q[i, h], k[j, g])) for j in range(cu[i], cu[i + 1])])
            w = np.exp(s) / np.exp(s).sum()
            assert l[h, i] == pytest.approx(math.log(np.exp(s).sum()), abs=1e-13)
            assert np.allclose(o[i, h], (w[:, None] * v[cu[i]:cu[i + 1], g]).sum(0), atol=1e-13)
    os_, ls_ = O.decode_forward(q, k, v, cu, 0.3, seqs=[2])
    assert np.allclose(os_[2], o[2]) and np.all(os_[0] == 0)


# ----------------------------------------------------------------------------
# EAGLE-3 mixed attention (block 0 causal + TTT diagonal blocks)
# ----------------------------------------------------------------------------
def _eagle_case(seed, lens, hq, hkv, d, nblk):
    rng = np.random.default_rng(seed)
    n = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q = rng.standard_normal((n, hq, d))
    ks = [rng.standard_normal((n, hkv, d)) for _ in range(nblk)]
    vs = [rng.standard_normal((n, hkv, d)) for _ in range(nblk)]
    return q, ks, vs, cu


def _dense_masked_attention(q, keys, vals, mask, scale, grp):
    """Brute force: one dense masked softmax per head over an explicit key list."""
    n, hq, _ = q.shape
    out = np.zeros_like(q)
    lse = np.zeros((hq, n))
    for h in range(hq):
        g = h // grp
        s = scale * q[:, h, :] @ keys[:, g, :].T
        s = np.where(mask, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        lse[h] = (m[:, 0] + np.log(w.sum(axis=1)))
        out[:, h, :] = (w / w.sum(axis=1, keepdims=True)) @ vals[:, g, :]
    return out, lse


def test_eagle_equals_dense_augmented_keys():
    # The joint softmax equals a dense masked softmax over the concatenated key
    # list [block 0 rows | block 1 rows | ...] where query t sees the causal
    # block-0 keys of its document and key t of every later block.
    q, ks, vs, cu = _eagle_case(1, [5, 7, 4], 4, 2, 8, 4)
    n = q.shape[0]
    keys = np.concatenate(ks, axis=0)
    vals = np.concatenate(vs, axis=0)
    mask = np.zeros((n, n * len(ks)), dtype=bool)
    for qs, qe in O.doc_bounds(cu):
        for t in range(qs, qe):
            mask[t, qs:t + 1] = True
            for i in range(1, len(ks)):
                mask[t, i * n + t] = True
    scale = 0.3
    ref_o, ref_l = _dense_masked_attention(q, keys, vals, mask, scale, 2)
    out, lse = O.eagle_forward(q, ks, vs, cu, scale)
    assert np.allclose(out, ref_o, atol=1e-12) and np.allclose(lse, ref_l, atol=1e-12)


def test_eagle_without_diagonals_is_causal_attention():
    q, ks, vs, cu = _eagle_case(2, [6, 3], 2, 1, 8, 1)
    out, lse = O.eagle_forward(q, ks, vs, cu, 0.5)
    ro, rl = O.full_attention(q, ks[0], vs[0], cu, 0.5)
    assert np.allclose(out, ro, atol=1e-12) and np.allclose(lse, rl, atol=1e-12)


def test_eagle_is_block0_merged_with_diagonal_partials():
    # The pages' route: block 0's (out, lse) merged with each diagonal block's
    # partial (block_out = v_i[t], block_lse = scale <q_t, k_i[t]>).
    q, ks, vs, cu = _eagle_case(3, [4, 9], 4, 1, 8, 3)
    scale = 0.25
    out, lse = O.full_attention(q, ks[0], vs[0], cu, scale)
    for k, v in zip(ks[1:], vs[1:]):
        bl = scale * np.einsum("thd,thd->ht", q, np.repeat(k, 4, axis=1))
        bo = np.repeat(v, 4, axis=1)
        out, lse, _ = O.merge(out, lse, bo, bl)
    eo, el = O.eagle_forward(q, ks, vs, cu, scale)
    assert np.allclose(out, eo, atol=1e-12) and np.allclose(lse, el, atol=1e-12)


def test_eagle_grads_match_finite_differences():
    q, ks, vs, cu = _eagle_case(4, [3, 4], 2, 1, 4, 3)
    rng = np.random.default_rng(5)
    dout = rng.standard_normal(q.shape)
    scale = 0.7
    dq, dks, dvs = O.eagle_grads(dout, q, ks, vs, cu, scale)

    def loss(q_, ks_, vs_):
        return float(np.sum(dout * O.eagle_forward(q_, ks_, vs_, cu, scale)[0]))

    eps = 1e-6
    checks = [(q, dq, lambda x: (x, ks, vs))]
    for i in range(len(ks)):
        checks.append((ks[i], dks[i], lambda x, i=i: (q, ks[:i] + [x] + ks[i + 1:], vs)))
        checks.append((vs[i], dvs[i], lambda x, i=i: (q, ks, vs[:i] + [x] + vs[i + 1:])))
    for base, grad, build in checks:
        for idx in [(0, 0, 0), (2, 1 if base.shape[1] > 1 else 0, 3), (6, 0, 1)]:
            xp, xm = base.copy(), base.copy()
            xp[idx] += eps
            xm[idx] -= eps
            fd = (loss(*build(xp)) - loss(*build(xm))) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-6 * max(1.0, abs(fd)), (idx, fd, grad[idx])


# ----------------------------------------------------------------------------
# Ulysses all-to-all reshard
# ----------------------------------------------------------------------------
def test_ulysses_reshard_element_map_and_round_trip():
    uly, S, H, D = 4, 12, 8, 3
    # element value encodes (global row, head, d)
    full = (np.arange(S)[:, None, None] * 1000 + np.arange(H)[None, :, None] * 10
            + np.arange(D)[None, None, :]).astype(np.float64)
    locals_ = [full[r * S // uly:(r + 1) * S // uly] for r in range(uly)]
    heads = O.ulysses_seq_to_head(locals_, uly)
    for r in range(uly):
        assert heads[r].shape == (S, H // uly, D)
        for t in range(S):
            for j in range(H // uly):
                assert heads[r][t, j, 0] == t * 1000 + (r * (H // uly) + j) * 10
    back = O.ulysses_head_to_seq(heads, uly)
    for r in range(uly):
        assert np.array_equal(back[r], locals_[r])
    lse = np.arange(H)[:, None] * 100.0 + np.arange(S)[None, :]
    lloc = [lse[:, r * S // uly:(r + 1) * S // uly] for r in range(uly)]
    lh = O.ulysses_lse_seq_to_head(lloc, uly)
    for r in range(uly):
        assert lh[r].flags["C_CONTIGUOUS"]
        assert np.array_equal(lh[r], lse[r * (H // uly):(r + 1) * (H // uly)])
    lb = O.ulysses_lse_head_to_seq(lh, uly)
    for r in range(uly):
        assert np.array_equal(lb[r], lloc[r])
