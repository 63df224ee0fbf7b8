"""Pins of the float64 oracle against things other than itself: scalar brute force,
closed forms, invariants the pages state (associativity of per-slice results, FCP
paper Sec. 2.2; causal and non-causal masks, Sec. 2.2; GQA head groups, Sec. 2.2 and
Sec. 6.1), and central finite differences for the backward."""
import math

import numpy as np
import pytest

import fcp_workloads as W
import oracle
from tests import brute_force

TINY = [
    # seqlens, block, hq, hkv, d, causal
    ([5, 1, 9, 3], 4, 4, 2, 8, True),
    ([5, 1, 9, 3], 4, 4, 2, 8, False),
    ([7, 12], 5, 2, 1, 4, True),
    ([16], 4, 3, 3, 6, True),
]


def _inputs(wl, seed=0, which=("q", "k", "v", "do")):
    bits = W.make_host_inputs(wl, seed=seed, which=which)
    return {n: W.bf16_bits_to_f64(b) for n, b in bits.items()}


@pytest.mark.parametrize("case", TINY)
def test_forward_matches_brute_force(case):
    seqlens, b, hq, hkv, d, causal = case
    wl = W.custom(seqlens, b, hq, hkv, d, causal)
    x = _inputs(wl)
    idx = oracle.SeqIndex(wl)
    o, lse = oracle.forward(x["q"], x["k"], x["v"], idx)
    ref = brute_force.attention(x["q"], x["k"], x["v"], wl)
    rows = idx.owned_rows()
    for ri, r in enumerate(rows):
        for h in range(hq):
            ro, rl = ref[(int(r), h)]
            assert abs(lse[ri, h] - rl) <= 1e-12 * max(1.0, abs(rl))
            np.testing.assert_allclose(o[ri, h], ro, rtol=0, atol=1e-12)


def test_forward_matches_brute_force_with_scale_and_subset():
    wl = W.custom([6, 10], 4, 4, 2, 8, True, q_ids=[1, 3], kv_ids=[0, 1, 2, 3])
    x = _inputs(wl, seed=3)
    idx = oracle.SeqIndex(wl)
    o, lse = oracle.forward(x["q"], x["k"], x["v"], idx, scale=0.37)
    ref = brute_force.attention(x["q"], x["k"], x["v"], wl, scale=0.37)
    for ri, r in enumerate(idx.owned_rows()):
        for h in range(4):
            ro, rl = ref[(int(r), h)]
            assert abs(lse[ri, h] - rl) <= 1e-12
            np.testing.assert_allclose(o[ri, h], ro, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_zero_query_gives_uniform_weights(causal):
    """Q = 0: every visible key has weight 1/|V(i)|, so O_i is the mean of the visible
    values and LSE_i = ln |V(i)| (ln(i+1) causal, ln L non-causal)."""
    wl = W.custom([6, 3, 11], 4, 2, 1, 4, causal)
    x = _inputs(wl)
    q0 = np.zeros_like(x["q"])
    idx = oracle.SeqIndex(wl)
    o, lse = oracle.forward(q0, x["k"], x["v"], idx)
    for ri, r in enumerate(idx.owned_rows()):
        s, p = idx.q_row_seq[r], idx.q_row_pos[r]
        n = p + 1 if causal else wl.seqlens[s]
        krows = idx.kv_row_of_pos[s][:n]
        np.testing.assert_allclose(lse[ri], np.log(n), atol=1e-14)
        np.testing.assert_allclose(o[ri, 0], x["v"][krows, 0].mean(axis=0), atol=1e-14)


def test_single_visible_key():
    """The first query of a sequence under the causal mask sees only key 0:
    O = v_0 and LSE = q_0 . k_0 / sqrt(D)."""
    wl = W.custom([4, 5], 3, 2, 2, 8, True)
    x = _inputs(wl)
    idx = oracle.SeqIndex(wl)
    o, lse = oracle.forward(x["q"], x["k"], x["v"], idx)
    for ri, r in enumerate(idx.owned_rows()):
        if idx.q_row_pos[r] != 0:
            continue
        kr = idx.kv_row_of_pos[idx.q_row_seq[r]][0]
        for h in range(2):
            np.testing.assert_allclose(o[ri, h], x["v"][kr, h], atol=1e-15)
            assert abs(lse[ri, h] - x["q"][r, h] @ x["k"][kr, h] / math.sqrt(8)) < 1e-14


def test_constant_values_give_constant_output():
    wl = W.custom([9, 4], 4, 4, 2, 8, True)
    x = _inputs(wl)
    v = np.full_like(x["v"], -1.75)
    o, _ = oracle.forward(x["q"], x["k"], v, oracle.SeqIndex(wl))
    np.testing.assert_allclose(o, -1.75, atol=1e-14)


def test_key_shift_moves_lse_only():
    """k_j <- k_j + u: every score of query i moves by q_i.u*scale, so O is unchanged
    and LSE_i grows by that amount."""
    wl = W.custom([7, 5], 4, 2, 1, 8, False)
    x = _inputs(wl)
    u = np.linspace(-1, 1, 8)
    idx = oracle.SeqIndex(wl)
    o0, l0 = oracle.forward(x["q"], x["k"], x["v"], idx)
    o1, l1 = oracle.forward(x["q"], x["k"] + u, x["v"], idx)
    rows = idx.owned_rows()
    np.testing.assert_allclose(o1, o0, atol=1e-12)
    np.testing.assert_allclose(l1 - l0, x["q"][rows] @ u / math.sqrt(8), atol=1e-12)


def test_softmax_rows_sum_to_one():
    """With one-hot values (v_j = e_j, D >= keys) the output row is the softmax row:
    it sums to 1 and each entry is exp(S_ij - LSE_i)."""
    wl = W.custom([12], 4, 1, 1, 16, True)
    x = _inputs(wl)
    v = np.zeros_like(x["v"])
    for j in range(12):
        v[j, 0, j] = 1.0
    idx = oracle.SeqIndex(wl)
    o, lse = oracle.forward(x["q"], x["k"], v, idx)
    np.testing.assert_allclose(o[:, 0].sum(axis=1), 1.0, atol=1e-14)
    s = x["q"][:, 0] @ x["k"][:, 0].T / 4.0
    for i in range(12):
        np.testing.assert_allclose(o[i, 0, :i + 1], np.exp(s[i, :i + 1] - lse[i, 0]),
                                   atol=1e-14)
        assert np.all(o[i, 0, i + 1:] == 0.0)


@pytest.mark.parametrize("causal", [True, False])
def test_merged_partials_equal_unsplit(causal):
    """Associativity: any split of each sequence's keys into subsets, computed as
    partials and merged (any order, linear or tree), equals the unsplit result."""
    rng = np.random.default_rng(7)
    wl = W.custom([13, 6, 20], 5, 4, 2, 8, causal)
    x = _inputs(wl)
    idx = oracle.SeqIndex(wl)
    o_ref, l_ref = oracle.forward(x["q"], x["k"], x["v"], idx)
    rows = idx.owned_rows()
    for s, length in enumerate(wl.seqlens):
        sel = np.nonzero(idx.q_row_seq[rows] == s)[0]
        qr, qp = rows[sel], idx.q_row_pos[rows[sel]]
        labels = rng.integers(0, 3, size=length)
        parts = []
        for lab in range(3):
            kp = np.nonzero(labels == lab)[0]
            if len(kp) == 0:
                continue
            parts.append(oracle.partial(x["q"], x["k"], x["v"], qr, qp,
                                        idx.kv_row_of_pos[s][kp], kp, causal, 4, 2))
        order = rng.permutation(len(parts))
        o_m, l_m = oracle.merge([parts[i][1] for i in order], [parts[i][0] for i in order])
        np.testing.assert_allclose(o_m, o_ref[sel], atol=1e-13)
        np.testing.assert_allclose(l_m, l_ref[sel], atol=1e-13)
        if len(parts) == 3:  # tree merge: (0,1) then with 2
            o01, l01 = oracle.merge([parts[0][1], parts[1][1]], [parts[0][0], parts[1][0]])
            o_t, l_t = oracle.merge([l01, parts[2][1]], [o01, parts[2][0]])
            np.testing.assert_allclose(o_t, o_ref[sel], atol=1e-13)
            np.testing.assert_allclose(l_t, l_ref[sel], atol=1e-13)


def test_merge_identity_and_empty_partials():
    rng = np.random.default_rng(1)
    o = rng.standard_normal((5, 3, 4))
    lse = rng.standard_normal((5, 3))
    o1, l1 = oracle.merge([lse], [o])
    np.testing.assert_allclose(o1, o, atol=1e-15)
    np.testing.assert_allclose(l1, lse, atol=1e-15)
    empty_l = np.full((5, 3), -np.inf)
    o2, l2 = oracle.merge([lse, empty_l], [o, np.zeros_like(o)])
    np.testing.assert_allclose(o2, o, atol=1e-15)
    np.testing.assert_allclose(l2, lse, atol=1e-15)
    o3, l3 = oracle.merge([empty_l, empty_l], [np.zeros_like(o), np.zeros_like(o)])
    assert np.all(np.isneginf(l3)) and np.all(o3 == 0.0)


def test_partial_with_no_visible_key_is_empty():
    wl = W.custom([8], 8, 2, 1, 4, True)
    x = _inputs(wl)
    # queries 0..3 against keys 5..7: nothing visible for queries 0..3 under causality
    o, lse = oracle.partial(x["q"], x["k"], x["v"], np.arange(4), np.arange(4),
                            np.arange(5, 8), np.arange(5, 8), True, 2, 1)
    assert np.all(np.isneginf(lse)) and np.all(o == 0.0)


def test_causal_row_equals_noncausal_prefix():
    """Causal query i equals non-causal attention over the prefix [0..i]."""
    wl = W.custom([11], 4, 2, 1, 8, True)
    x = _inputs(wl)
    o, lse = oracle.forward(x["q"], x["k"], x["v"], oracle.SeqIndex(wl))
    for i in range(11):
        pre = W.custom([i + 1], 16, 2, 1, 8, False)
        idx = oracle.SeqIndex(pre)
        op, lp = oracle.forward(x["q"][:i + 1], x["k"][:i + 1], x["v"][:i + 1], idx)
        np.testing.assert_allclose(o[i], op[i], atol=1e-13)
        np.testing.assert_allclose(lse[i], lp[i], atol=1e-13)


def test_noncausal_invariant_to_kv_permutation():
    wl = W.custom([10], 10, 2, 2, 8, False)
    x = _inputs(wl)
    perm = np.random.default_rng(2).permutation(10)
    idx = oracle.SeqIndex(wl)
    o0, l0 = oracle.forward(x["q"], x["k"], x["v"], idx)
    idx.kv_row_of_pos[0] = idx.kv_row_of_pos[0][perm]
    k2, v2 = x["k"].copy(), x["v"].copy()
    k2[perm], v2[perm] = x["k"], x["v"]  # key at position p now sits in row perm[p]
    o1, l1 = oracle.forward(x["q"], k2, v2, idx)
    np.testing.assert_allclose(o1, o0, atol=1e-13)
    np.testing.assert_allclose(l1, l0, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    """Contiguous head groups: query head h reads KV head h // G, the same as MHA with
    every KV head repeated G times in place."""
    wl = W.custom([9, 5], 4, 6, 2, 8, True)
    x = _inputs(wl)
    o, lse = oracle.forward(x["q"], x["k"], x["v"], oracle.SeqIndex(wl))
    mha = W.custom([9, 5], 4, 6, 6, 8, True)
    k6, v6 = np.repeat(x["k"], 3, axis=1), np.repeat(x["v"], 3, axis=1)
    om, lm = oracle.forward(x["q"], k6, v6, oracle.SeqIndex(mha))
    np.testing.assert_allclose(o, om, atol=1e-14)
    np.testing.assert_allclose(lse, lm, atol=1e-14)


@pytest.mark.parametrize("causal", [True, False])
def test_backward_matches_finite_differences(causal):
    """Central differences (step 1e-6) of L = sum_i <dO_i, O_i> agree with the analytic
    gradients to 1e-6 relative."""
    wl = W.custom([5, 3], 4, 4, 2, 4, causal)
    x = _inputs(wl)
    idx = oracle.SeqIndex(wl)
    rows = idx.owned_rows()
    dq, dk, dv = oracle.backward(x["q"], x["k"], x["v"], x["do"], idx)

    def loss(q, k, v):
        o, _ = oracle.forward(q, k, v, idx)
        return float((o * x["do"][rows]).sum())

    eps = 1e-6
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        base = x[name]
        num = np.zeros_like(base)
        for pos in np.ndindex(base.shape):
            args = {n: x[n] for n in ("q", "k", "v")}
            plus, minus = base.copy(), base.copy()
            plus[pos] += eps
            minus[pos] -= eps
            args[name] = plus
            lp = loss(args["q"], args["k"], args["v"])
            args[name] = minus
            lm = loss(args["q"], args["k"], args["v"])
            num[pos] = (lp - lm) / (2 * eps)
        err = np.abs(num - grad).max() / max(np.abs(grad).max(), 1e-30)
        assert err <= 1e-6, (name, err)


def test_backward_sums():
    """Rows of dS sum to zero, so sum_j dK_j = 0 per sequence and KV head; rows of P sum
    to one, so sum_j dV_j equals the sum of dO over the group's query heads."""
    wl = W.custom([9, 14, 4], 5, 4, 2, 8, True)
    x = _inputs(wl)
    idx = oracle.SeqIndex(wl)
    dq, dk, dv = oracle.backward(x["q"], x["k"], x["v"], x["do"], idx)
    for s in range(3):
        krows = idx.kv_row_of_pos[s]
        qrows = np.nonzero(idx.q_row_seq == s)[0]
        for g in range(2):
            np.testing.assert_allclose(dk[krows, g].sum(axis=0), 0.0, atol=1e-12)
            np.testing.assert_allclose(dv[krows, g].sum(axis=0),
                                       x["do"][qrows, 2 * g:2 * g + 2].sum(axis=(0, 1)),
                                       atol=1e-12)


def test_dq_rows_matches_full_backward():
    wl = W.custom([9, 14, 4], 5, 4, 2, 8, True)
    x = _inputs(wl)
    idx = oracle.SeqIndex(wl)
    dq, _, _ = oracle.backward(x["q"], x["k"], x["v"], x["do"], idx)
    rows = np.array([0, 3, 10, 22, 26])
    np.testing.assert_allclose(oracle.dq_rows(x["q"], x["k"], x["v"], x["do"], idx, rows),
                               dq[rows], atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_dkv_rows_matches_full_backward(causal):
    wl = W.custom([9, 14, 4], 5, 4, 2, 8, causal)
    x = _inputs(wl)
    idx = oracle.SeqIndex(wl)
    _, dk, dv = oracle.backward(x["q"], x["k"], x["v"], x["do"], idx)
    rows = np.array([0, 4, 8, 9, 15, 22, 23, 26])
    sk, sv = oracle.dkv_rows(x["q"], x["k"], x["v"], x["do"], idx, rows)
    np.testing.assert_allclose(sk, dk[rows], atol=1e-13)
    np.testing.assert_allclose(sv, dv[rows], atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_dkv_keys_matches_full_backward(causal):
    """dkv_keys (one forward per query, requested key columns only) against the full
    backward, whose gradients are pinned by finite differences above; with a head subset
    equal to one KV head's group, that KV head's rows are exact and the others zero."""
    wl = W.custom([9, 14, 4], 5, 4, 2, 8, causal)
    x = _inputs(wl)
    idx = oracle.SeqIndex(wl)
    _, dk, dv = oracle.backward(x["q"], x["k"], x["v"], x["do"], idx)
    rows = np.array([26, 0, 4, 8, 9, 15, 22, 23])
    sk, sv = oracle.dkv_keys(x["q"], x["k"], x["v"], x["do"], idx, rows)
    np.testing.assert_allclose(sk, dk[rows], atol=1e-13)
    np.testing.assert_allclose(sv, dv[rows], atol=1e-13)
    hk, hv = oracle.dkv_keys(x["q"], x["k"], x["v"], x["do"], idx, rows, heads=[2, 3])
    np.testing.assert_allclose(hk[:, 1], dk[rows, 1], atol=1e-13)
    np.testing.assert_allclose(hv[:, 1], dv[rows, 1], atol=1e-13)
    assert not hk[:, 0].any() and not hv[:, 0].any()


def test_dkv_keys_single_head_equals_masked_upstream_gradient():
    """Zeroing dO on every query head but one makes the other heads contribute nothing
    (dS = P (dP - Delta) with dP = Delta = 0): the full backward with that dO equals
    dkv_keys restricted to the one head."""
    wl = W.custom([9, 14, 4], 5, 4, 2, 8, True)
    x = _inputs(wl)
    idx = oracle.SeqIndex(wl)
    do1 = np.zeros_like(x["do"])
    do1[:, 3] = x["do"][:, 3]
    _, dk, dv = oracle.backward(x["q"], x["k"], x["v"], do1, idx)
    rows = np.arange(wl.kv_rows)
    hk, hv = oracle.dkv_keys(x["q"], x["k"], x["v"], x["do"], idx, rows, heads=[3])
    np.testing.assert_allclose(hk, dk, atol=1e-13)
    np.testing.assert_allclose(hv, dv, atol=1e-13)


def test_backward_head_subset_is_a_selection():
    """backward(heads=...) returns the all-heads dQ on those heads (zero elsewhere), and
    dK/dV of a KV head whose whole group is selected equal the all-heads result."""
    wl = W.custom([9, 14, 4], 5, 4, 2, 8, True)
    x = _inputs(wl)
    idx = oracle.SeqIndex(wl)
    dq, dk, dv = oracle.backward(x["q"], x["k"], x["v"], x["do"], idx)
    sq, sk, sv = oracle.backward(x["q"], x["k"], x["v"], x["do"], idx, heads=[2, 3])
    np.testing.assert_allclose(sq[:, 2:], dq[:, 2:], atol=1e-13)
    assert not sq[:, :2].any() and not sk[:, 0].any() and not sv[:, 0].any()
    np.testing.assert_allclose(sk[:, 1], dk[:, 1], atol=1e-13)
    np.testing.assert_allclose(sv[:, 1], dv[:, 1], atol=1e-13)
