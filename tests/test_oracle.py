"""Pins of the CPU oracle against facts that do not come from the oracle.

Each check is chosen so that a plausible slip in oracle/attn_oracle.c (a
dropped scale, a wrong mask direction, a transposed operand, a missing max
shift, a wrong log base, a wrong sign in the softmax gradient) fails at least
one of them:

* closed forms: equal scores -> O is the mean of the visible V rows and
  LSE = ln |A_i|; one dominant score -> O copies that V row;
* invariants: rows of P sum to one (O of a constant V), LSE equals a direct
  long-double log-sum-exp, linearity and shift of V, joint key/value
  permutation, causal row i equals non-causal attention on the prefix [0, i];
* brute force for S <= 16: an independent long-double implementation that
  materialises the whole score matrix and exponentiates without max shift,
  and whose gradient uses the softmax Jacobian diag(p) - p p^T;
* central finite differences of L = sum(dO * O) for all three gradients;
* gradient identities: dQ = 0 when all keys are equal, dK = 0 and dV uniform
  when Q = 0, linearity of every gradient in dO;
* the sampled-row / sampled-column entry points equal the full ones;
* hand-worked examples (tests/golden/hand_worked_examples.json): scores that
  are logarithms of small integers, so that P, O, LSE and every gradient are
  simple closed forms derived by hand in that file.

The pages print no worked example, so no fixture value comes from them.
"""
import math

import numpy as np
import pytest

import attn_inputs as gen
import golden_worked
import oracle

rng = np.random.default_rng(1234)
LD = np.longdouble


def rand(*shape, s=1.0):
    return rng.standard_normal(shape) * s


# ---------------------------------------------------------------- brute force
def brute_forward(q, k, v, scale, causal):
    """Long double, whole S x S matrix, exp without max shift."""
    q, k, v = q.astype(LD), k.astype(LD), v.astype(LD)
    S = q.shape[0]
    s = (q @ k.T) * LD(scale)
    e = np.exp(s)
    if causal:
        e = e * np.tril(np.ones((S, S), dtype=LD))
    z = e.sum(axis=1, keepdims=True)
    p = e / z
    return p @ v, np.log(z[:, 0]), p


def brute_backward(q, k, v, do, scale, causal):
    _, _, p = brute_forward(q, k, v, scale, causal)
    q, k, v, do = q.astype(LD), k.astype(LD), v.astype(LD), do.astype(LD)
    dp = do @ v.T
    ds = np.empty_like(dp)
    for i in range(q.shape[0]):
        jac = np.diag(p[i]) - np.outer(p[i], p[i])
        ds[i] = jac @ dp[i]
    return LD(scale) * ds @ k, LD(scale) * ds.T @ q, p.T @ do


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S,d", [(1, 4), (5, 3), (16, 8), (13, 16)])
def test_forward_matches_brute_force(S, d, causal):
    q, k, v = rand(S, d), rand(S, d), rand(S, d)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attention_forward(q, k, v, scale, causal)
    ob, lseb, _ = brute_forward(q, k, v, scale, causal)
    np.testing.assert_allclose(o, ob.astype(np.float64), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lseb.astype(np.float64), rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S,d", [(1, 4), (6, 3), (16, 8)])
def test_backward_matches_brute_force(S, d, causal):
    q, k, v, do = rand(S, d), rand(S, d), rand(S, d), rand(S, d)
    scale = 0.7
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale, causal)
    bq, bk, bv = brute_backward(q, k, v, do, scale, causal)
    for a, b in ((dq, bq), (dk, bk), (dv, bv)):
        np.testing.assert_allclose(a, b.astype(np.float64), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("causal", [False, True])
def test_equal_scores_give_mean_of_visible_v(causal):
    S, d = 37, 8
    q = np.zeros((S, d))
    k, v = rand(S, d), rand(S, d)
    o, lse = oracle.attention_forward(q, k, v, 0.125, causal)
    for i in range(S):
        n = i + 1 if causal else S
        np.testing.assert_allclose(o[i], v[:n].mean(axis=0), rtol=0, atol=1e-13)
        assert abs(lse[i] - math.log(n)) < 1e-13


def test_dominant_score_copies_that_v_row():
    S, d = 24, 24
    k = np.eye(S, d) * 3.0                        # orthogonal keys
    v = rand(S, d)
    target = rng.permutation(S)
    q = 40.0 * k[target] / 3.0                      # s_i,target = 40*3*scale... large
    scale = 1.0
    o, lse = oracle.attention_forward(q, k, v, scale, False)
    np.testing.assert_allclose(o, v[target], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.full(S, 120.0), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one_and_lse_is_logsumexp(causal):
    S, d = 29, 12
    q, k = rand(S, d, s=2.0), rand(S, d)
    scale = 1 / math.sqrt(d)
    c = rand(d)
    o, lse = oracle.attention_forward(q, k, np.tile(c, (S, 1)), scale, causal)
    np.testing.assert_allclose(o, np.tile(c, (S, 1)), rtol=0, atol=1e-13)
    s = (q.astype(LD) @ k.T.astype(LD)) * LD(scale)
    for i in range(S):
        n = i + 1 if causal else S
        ref = np.log(np.sum(np.exp(s[i, :n])))
        assert abs(lse[i] - float(ref)) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_linear_and_shift_in_v(causal):
    S, d = 21, 6
    q, k, v = rand(S, d), rand(S, d), rand(S, d)
    a, c = -2.5, rand(d)
    o, _ = oracle.attention_forward(q, k, v, 0.4, causal)
    o2, _ = oracle.attention_forward(q, k, a * v + c, 0.4, causal)
    np.testing.assert_allclose(o2, a * o + c, rtol=0, atol=1e-12)


def test_joint_key_value_permutation_noncausal():
    S, d = 19, 7
    q, k, v = rand(S, d), rand(S, d), rand(S, d)
    perm = rng.permutation(S)
    o, lse = oracle.attention_forward(q, k, v, 0.3, False)
    o2, lse2 = oracle.attention_forward(q, k[perm], v[perm], 0.3, False)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-13)


def test_causal_row_is_noncausal_prefix():
    S, d = 17, 5
    q, k, v = rand(S, d), rand(S, d), rand(S, d)
    oc, lc = oracle.attention_forward(q, k, v, 0.5, True)
    for i in range(S):
        on, ln = oracle.attention_forward(q[: i + 1], k[: i + 1], v[: i + 1], 0.5, False)
        np.testing.assert_allclose(oc[i], on[i], rtol=0, atol=1e-13)
        assert abs(lc[i] - ln[i]) < 1e-13
    # row 0 sees only key 0
    np.testing.assert_allclose(oc[0], v[0], rtol=0, atol=1e-15)
    assert abs(lc[0] - 0.5 * float(q[0] @ k[0])) < 1e-13


def test_batched_heads_are_independent():
    B, H, S, d = 2, 3, 9, 4
    q, k, v = rand(B, H, S, d), rand(B, H, S, d), rand(B, H, S, d)
    o, lse = oracle.attention_forward(q, k, v, 0.6, True, nthreads=4)
    for b in range(B):
        for h in range(H):
            o1, l1 = oracle.attention_forward(q[b, h], k[b, h], v[b, h], 0.6, True, nthreads=1)
            np.testing.assert_array_equal(o[b, h], o1)
            np.testing.assert_array_equal(lse[b, h], l1)


# ---------------------------------------------------------------- gradients
def _loss(q, k, v, do, scale, causal):
    o, _ = oracle.attention_forward(q, k, v, scale, causal, nthreads=1)
    return float(np.sum(do * o))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S,d", [(5, 3), (8, 4)])
def test_backward_matches_central_differences(S, d, causal):
    q, k, v, do = rand(S, d), rand(S, d), rand(S, d), rand(S, d)
    scale = 0.8
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale, causal, nthreads=1)
    h = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.empty_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], do, scale, causal)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], do, scale, causal)
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=0, atol=2e-8 * max(1.0, np.abs(num).max()),
                                   err_msg=f"d{name}")


@pytest.mark.parametrize("causal", [False, True])
def test_equal_keys_give_zero_dq(causal):
    S, d = 11, 6
    q, v, do = rand(S, d), rand(S, d), rand(S, d)
    k = np.tile(rand(d), (S, 1))
    dq, _, _ = oracle.attention_backward(q, k, v, do, 0.9, causal)
    np.testing.assert_allclose(dq, 0.0, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_zero_dk_and_uniform_dv(causal):
    S, d = 10, 5
    q = np.zeros((S, d))
    k, v, do = rand(S, d), rand(S, d), rand(S, d)
    _, dk, dv = oracle.attention_backward(q, k, v, do, 0.9, causal)
    np.testing.assert_allclose(dk, 0.0, rtol=0, atol=1e-13)
    ref = np.zeros((S, d))
    for i in range(S):
        n = i + 1 if causal else S
        ref[:n] += do[i] / n
    np.testing.assert_allclose(dv, ref, rtol=0, atol=1e-13)


def test_gradients_linear_in_do():
    S, d = 9, 4
    q, k, v, d1, d2 = (rand(S, d) for _ in range(5))
    g1 = oracle.attention_backward(q, k, v, d1, 0.5, True)
    g2 = oracle.attention_backward(q, k, v, d2, 0.5, True)
    g3 = oracle.attention_backward(q, k, v, 2.0 * d1 - 3.0 * d2, 0.5, True)
    for a, b, c in zip(g1, g2, g3):
        np.testing.assert_allclose(c, 2.0 * a - 3.0 * b, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- sampled entry points
@pytest.mark.parametrize("causal", [False, True])
def test_sampled_rows_and_columns_equal_full(causal):
    S, d = 70, 8
    q, k, v, do = rand(S, d), rand(S, d), rand(S, d), rand(S, d)
    scale = 1 / math.sqrt(d)
    o, lse = oracle.attention_forward(q, k, v, scale, causal)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale, causal)
    rows = np.array([0, 1, 33, 69, 5])
    o_r, l_r = oracle.forward_rows(q, k, v, rows, scale, causal, nthreads=3)
    np.testing.assert_allclose(o_r, o[rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(l_r, lse[rows], rtol=0, atol=1e-14)
    dq_r = oracle.backward_dq_rows(q, k, v, do, rows, scale, causal, nthreads=2)
    np.testing.assert_allclose(dq_r, dq[rows], rtol=0, atol=1e-13)
    cols = np.array([0, 69, 40, 2])
    dk_c, dv_c = oracle.backward_dkdv_cols(q, k, v, do, cols, scale, causal, nthreads=5)
    np.testing.assert_allclose(dk_c, dk[cols], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv_c, dv[cols], rtol=0, atol=1e-13)


# ---------------------------------------------------------------- input generator
def test_splitmix64_reference_values():
    # SplitMix64 with state 0: the first outputs quoted with the generator's
    # published definition (Vigna's reference splitmix64.c, seed 0).
    got = gen.splitmix64(0, 0, 3)
    assert [int(x) for x in got] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.concatenate([gen.normal_f32(99, 100000) * 7.0,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 65504.0, 0.0,
                                  -0.0, 1e-30, 3.0e38], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(gen.f32_to_bf16_bits(x), ref)
    back = gen.bf16_bits_to_f64(ref)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_normal_draws_are_standard_normal():
    x = gen.normal_f32(0xFA000010, 1 << 20).astype(np.float64)
    assert abs(x.mean()) < 5e-3
    assert abs(x.std() - 1.0) < 5e-3
    # 4th moment of N(0,1) is 3
    assert abs(np.mean(x ** 4) - 3.0) < 0.05
    # chunked generation is the same stream as one shot
    y = gen.normal_f32(0xFA000010, 1001, chunk=100)
    np.testing.assert_array_equal(y, gen.normal_f32(0xFA000010, 1001))


# ------------------------------------------------------- hand-worked examples
@pytest.mark.parametrize("d", [2, 5])
def test_hand_worked_examples(d):
    for c in golden_worked.cases(d):
        o, lse = oracle.attention_forward(c["q"], c["k"], c["v"], c["scale"], c["causal"])
        dq, dk, dv = oracle.attention_backward(c["q"], c["k"], c["v"], c["do"], c["scale"], c["causal"])
        for got, t in ((o, "o"), (lse, "lse"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
            assert np.abs(got - c[t]).max() <= 1e-13, (c["name"], t, got, c[t])
