"""The largest sequence the library accepts: S = 2^22, d = 128, causal.

At this size the per-head byte offsets reach their 32-bit limits: Q, K, V, O
and dO rows end at 2^30 bytes, the fp32 dQ at 2^31.  One head runs the
forward and the default backward; the oracle checks, on sampled query rows,
O and LSE (forward_rows) and dQ (backward_dq_rows).  dK and dV of the last
keys are checked exactly too: under the causal mask only the last m queries
see the last m keys, so their gradients follow from those m rows alone, with
P and D formed from the oracle's O and LSE of the rows (the textbook
backward restricted to them).  Tolerances as in test_gpu_parity.py.
"""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

S, D = 1 << 22, 128
O_MAX, LSE_MAX, G_REL = 2e-2, 1e-3, 5e-2


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the -m gpu tests need an MI355X")
    import exact_attention_39_amd as m
    m.load_library()
    return m


def host64(t):
    return t.float().cpu().numpy().astype(np.float64)


def test_max_sequence_length_causal(fa):
    say(f"[max S] B=1 H=1 S={S} d={D} causal: inputs")
    gen = torch.Generator(device="cuda").manual_seed(2026)
    q, k, v, do = (torch.randn((1, 1, S, D), generator=gen, device="cuda").to(torch.bfloat16) for _ in range(4))
    scale = D ** -0.5
    say("[max S] forward")
    o, lse = fa.forward(q, k, v, causal=True, scale=scale)
    say("[max S] backward")
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=True, scale=scale)
    torch.cuda.synchronize()
    for t, nm in ((o, "O"), (lse, "LSE"), (dq, "dQ"), (dk, "dK"), (dv, "dV")):
        assert torch.isfinite(t.float()).all(), f"{nm} has non-finite values"

    say("[max S] oracle on sampled rows")
    Q, K, V, dO = (host64(t[0, 0]) for t in (q, k, v, do))
    rows = np.array([0, 1, 2, 255, 256, S // 2 - 1, S // 2, S - 257, S - 256, S - 3, S - 2, S - 1], dtype=np.int64)
    idx = torch.from_numpy(rows).cuda()
    o_ref, l_ref = oracle.forward_rows(Q, K, V, rows, scale, True)
    err_o = np.abs(host64(o[0, 0, idx]) - o_ref).max()
    err_l = np.abs(lse[0, 0, idx].double().cpu().numpy() - l_ref).max()
    assert err_o <= O_MAX, f"O max err {err_o:.3e}"
    assert err_l <= LSE_MAX, f"LSE max err {err_l:.3e}"
    gq = oracle.backward_dq_rows(Q, K, V, dO, rows, scale, True)
    rel = np.abs(dq[0, 0, idx].double().cpu().numpy() - gq).max() / np.abs(gq).max()
    assert rel <= G_REL, f"dQ rel err {rel:.3e}"

    say("[max S] dK, dV of the last keys")
    m = 8
    tail = np.arange(S - m, S, dtype=np.int64)
    o_t, l_t = oracle.forward_rows(Q, K, V, tail, scale, True)
    Qt, Kt, Vt, dOt = Q[tail], K[tail], V[tail], dO[tail]
    P = np.exp(scale * (Qt @ Kt.T) - l_t[:, None]) * np.tril(np.ones((m, m)))  # row i sees tail keys <= i
    Dt = np.sum(dOt * o_t, axis=1)
    dS = P * (dOt @ Vt.T - Dt[:, None])
    gk, gv = scale * dS.T @ Qt, P.T @ dOt
    tidx = torch.from_numpy(tail).cuda()
    for g, ref, nm in ((dk, gk, "dK"), (dv, gv, "dV")):
        rel = np.abs(host64(g[0, 0, tidx]) - ref).max() / np.abs(ref).max()
        assert rel <= G_REL, f"{nm} of the last keys: rel err {rel:.3e}"
