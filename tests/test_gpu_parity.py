"""GPU parity of the HIP path (through the C ABI) against the CPU fp64 oracle.

Tolerances (fixed by the attention target, written here once):
  O     max |O - O_ref| <= 2e-2 and mean |O - O_ref| <= 2e-3
  LSE   max |LSE - LSE_ref| <= 1e-3
  dQ, dK, dV   max |g - g_ref| / max |g_ref| <= 5e-2  (per tensor);
               where g_ref is identically zero, max |g| <= 1e-4

Both sides see the same bf16 inputs from attn_inputs (seeded SplitMix64 +
Box-Muller, rounded to bf16); the oracle widens them exactly to fp64.
Small shapes are compared element by element over whole tensors; the
workload shapes are compared on sampled query rows (O, LSE, dQ) and sampled
key rows (dK, dV) that the oracle computes one by one.
"""
import sys

import numpy as np
import pytest

import attn_inputs as gen
import golden_worked
import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX, G_REL = 2e-2, 2e-3, 1e-3, 5e-2
G_ABS_ZERO = 1e-4  # for gradients that are exactly zero


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the -m gpu tests need an MI355X")
    import exact_attention_39_amd as m
    m.load_library()
    return m


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_to_np64(t):
    return t.float().cpu().numpy().astype(np.float64)


def rand_bits(shape, seed, scale=1.0):
    x = gen.normal_f32(seed, int(np.prod(shape))).reshape(shape) * np.float32(scale)
    return gen.f32_to_bf16_bits(x)


def check_o(o, ref, what):
    err = np.abs(o - ref)
    assert err.max() <= O_MAX and err.mean() <= O_MEAN, f"{what}: O max {err.max():.3e} mean {err.mean():.3e}"


def check_lse(l, ref, what):
    err = np.abs(l - ref).max()
    assert err <= LSE_MAX, f"{what}: LSE max err {err:.3e}"


def check_grad(g, ref, what):
    peak = np.abs(ref).max()
    if peak == 0.0:
        # degenerate case (e.g. S = 1: one key, so dS = 0 and dQ = dK = 0
        # exactly); the relative form is undefined, bound the rounding noise
        # absolutely instead.
        assert np.abs(g).max() <= G_ABS_ZERO, f"{what}: max |g| {np.abs(g).max():.3e} for a zero gradient"
        return 0.0
    rel = np.abs(g - ref).max() / peak
    assert rel <= G_REL, f"{what}: rel err {rel:.3e}"
    return rel


def run_fwd(fa, qb, kb, vb, causal, scale, opts=None):
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale, opts=opts)
    torch.cuda.synchronize()
    return q, k, v, o, lse


# ------------------------------------------------------------------ whole tensors, small shapes
SMALL = [
    # (B, H, S, d, causal)  -- several tiles and ragged tails
    (1, 2, 256, 64, False),
    (1, 2, 256, 64, True),
    (2, 3, 300, 128, False),
    (2, 3, 300, 128, True),
    (1, 1, 1, 128, False),
    (1, 1, 1, 64, True),
    (1, 2, 130, 64, True),
    (1, 1, 129, 128, True),
    (1, 2, 64, 128, False),
    (1, 1, 515, 128, True),
    (1, 1, 200, 64, False),
]


@pytest.mark.parametrize("B,H,S,d,causal", SMALL)
def test_small_forward_backward_full_tensors(fa, B, H, S, d, causal):
    say(f"[small] B={B} H={H} S={S} d={d} causal={causal}")
    shape = (B, H, S, d)
    seed = 1000 + S * 7 + d + int(causal)
    qb, kb, vb, db = (rand_bits(shape, seed + i) for i in range(4))
    scale = 1.0 / np.sqrt(d)
    q, k, v, o, lse = run_fwd(fa, qb, kb, vb, causal, scale)
    Q, K, V, dO = (gen.bf16_bits_to_f64(x) for x in (qb, kb, vb, db))
    o_ref, lse_ref = oracle.attention_forward(Q, K, V, scale, causal)
    check_o(bf16_to_np64(o), o_ref, "fwd")
    check_lse(lse.cpu().numpy().astype(np.float64), lse_ref, "fwd")
    do = to_dev(db)
    gq, gk, gv = oracle.attention_backward(Q, K, V, dO, scale, causal)
    got = []
    for stored in (False, True):
        dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=causal, scale=scale,
                                 opts=fa.Options(stored_ds=stored))
        torch.cuda.synchronize()
        what = "stored dS" if stored else "recomputed dS"
        check_grad(dq.cpu().numpy().astype(np.float64), gq, f"{what} dQ")
        check_grad(bf16_to_np64(dk), gk, f"{what} dK")
        check_grad(bf16_to_np64(dv), gv, f"{what} dV")
        got.append((dk, dv))
    # the dK/dV kernel runs the same arithmetic whether or not it also stores dS
    assert torch.equal(got[0][0], got[1][0]) and torch.equal(got[0][1], got[1][1])


# B*H a multiple of the XCD count (8): fa_bwd takes the single-pass backward
FUSED_SMALL = [
    (1, 8, 300, 128, False),
    (1, 8, 300, 128, True),
    (2, 4, 515, 64, True),
    (2, 4, 515, 64, False),
    (1, 8, 1, 128, True),
    (1, 16, 33, 128, False),
    (1, 8, 256, 128, True),
    (1, 8, 257, 64, True),
    (1, 8, 700, 128, False),
]


def sync_error_word(ws, B, H, S):
    """The error word of the single-pass backward's sync area in the workspace."""
    off = (8 * B * H * S + 255) // 256 * 256
    return int(ws.view(torch.int32)[off // 4 + 16].item())


@pytest.mark.parametrize("B,H,S,d,causal", FUSED_SMALL)
def test_fused_backward_full_tensors(fa, B, H, S, d, causal):
    """The single-pass backward (dQ summed over key blocks in turn) against
    the oracle on whole tensors, several key blocks and ragged tails; the
    split backward on the same inputs too, and the error word stays 0."""
    say(f"[fused] B={B} H={H} S={S} d={d} causal={causal}")
    shape = (B, H, S, d)
    seed = 5000 + S * 7 + d + int(causal) + H
    qb, kb, vb, db = (rand_bits(shape, seed + i) for i in range(4))
    scale = 1.0 / np.sqrt(d)
    q, k, v, o, lse = run_fwd(fa, qb, kb, vb, causal, scale)
    do = to_dev(db)
    Q, K, V, dO = (gen.bf16_bits_to_f64(x) for x in (qb, kb, vb, db))
    gq, gk, gv = oracle.attention_backward(Q, K, V, dO, scale, causal)
    ws = torch.empty(max(1, fa.fa_bwd_workspace_bytes(B, H, S, d) // 4), dtype=torch.float32, device="cuda")
    for fused in (True, False):
        dq = torch.empty((B, H, S, d), dtype=torch.float32, device="cuda")
        dk, dv = torch.empty_like(q), torch.empty_like(q)
        fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, scale, causal, ws, opts=fa.Options(fused_backward=fused))
        torch.cuda.synchronize()
        if fused:
            assert sync_error_word(ws, B, H, S) == 0, "a turn wait of the single-pass backward expired"
        what = "fused" if fused else "split"
        check_grad(dq.cpu().numpy().astype(np.float64), gq, f"{what} dQ")
        check_grad(bf16_to_np64(dk), gk, f"{what} dK")
        check_grad(bf16_to_np64(dv), gv, f"{what} dV")


def test_fused_backward_repeatable_and_matches_split(fa):
    """Two single-pass runs agree bit for bit (fixed order of the dQ sums);
    against the split backward the gradients agree to fp32/bf16 rounding."""
    say("[fused] repeatability")
    shape = (1, 16, 2500, 128)
    qb, kb, vb, db = (rand_bits(shape, 8100 + i) for i in range(4))
    scale = 1.0 / np.sqrt(128)
    for causal in (False, True):
        q, k, v, o, lse = run_fwd(fa, qb, kb, vb, causal, scale)
        do = to_dev(db)
        fused = fa.Options(fused_backward=True)
        g1 = fa.backward(q, k, v, o, lse, do, causal=causal, scale=scale, opts=fused)
        g2 = fa.backward(q, k, v, o, lse, do, causal=causal, scale=scale, opts=fused)
        gs = fa.backward(q, k, v, o, lse, do, causal=causal, scale=scale)
        torch.cuda.synchronize()
        for a, b, c_, nm in zip(g1, g2, gs, ("dQ", "dK", "dV")):
            assert torch.equal(a, b), f"{nm} of the single-pass backward differs between runs (causal={causal})"
            a64, c64 = a.float().cpu().numpy(), c_.float().cpu().numpy()
            rel = np.abs(a64 - c64).max() / np.abs(c64).max()
            assert rel <= 2e-2, f"{nm}: single-pass vs split rel diff {rel:.3e} (causal={causal})"


@pytest.mark.parametrize("d", [64, 128])
def test_hand_worked_examples(fa, d):
    """The hand-derived closed forms of tests/golden/hand_worked_examples.json,
    padded to head dimension d; every input value is exact in bf16."""
    for c in golden_worked.cases(d):
        say(f"[golden] {c['name']} d={d}")
        bits = {t: gen.f32_to_bf16_bits(c[t].astype(np.float32))[None, None] for t in ("q", "k", "v", "do")}
        for t, b in bits.items():
            assert np.array_equal(gen.bf16_bits_to_f64(b)[0, 0], c[t]), (c["name"], t)
        q, k, v, o, lse = run_fwd(fa, bits["q"], bits["k"], bits["v"], c["causal"], c["scale"])
        check_o(bf16_to_np64(o)[0, 0], c["o"], c["name"])
        check_lse(lse.cpu().numpy().astype(np.float64)[0, 0], c["lse"], c["name"])
        dq, dk, dv = fa.backward(q, k, v, o, lse, to_dev(bits["do"]), causal=c["causal"], scale=c["scale"])
        torch.cuda.synchronize()
        check_grad(dq.cpu().numpy().astype(np.float64)[0, 0], c["dq"], c["name"] + " dQ")
        check_grad(bf16_to_np64(dk)[0, 0], c["dk"], c["name"] + " dK")
        check_grad(bf16_to_np64(dv)[0, 0], c["dv"], c["name"] + " dV")


def test_smoke_workload_forward(fa):
    """fp32 host draws -> bf16 device, B=1 H=2 S=256 d=64, non-causal, all elements."""
    name = "smoke_d64_s256"
    say(f"[workload] {name}")
    w = gen.WORKLOADS[name]
    bits = gen.workload_inputs(name, ("q", "k", "v"))
    scale = gen.default_scale(w["d"])
    _, _, _, o, lse = run_fwd(fa, bits["q"], bits["k"], bits["v"], False, scale)
    Q, K, V = (gen.bf16_bits_to_f64(bits[t]) for t in "qkv")
    o_ref, lse_ref = oracle.attention_forward(Q, K, V, scale, False)
    check_o(bf16_to_np64(o), o_ref, name)
    check_lse(lse.cpu().numpy().astype(np.float64), lse_ref, name)


def test_empty_inputs_launch_nothing(fa):
    say("[edge] empty inputs")
    for shape in [(1, 1, 0, 128), (0, 4, 64, 64), (2, 0, 64, 128)]:
        q = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
        o, lse = fa.forward(q, q, q, causal=True)
        dq, dk, dv = fa.backward(q, q, q, o, lse, q, causal=True)
        torch.cuda.synchronize()
        assert o.shape == shape and lse.shape == shape[:3] and dq.shape == shape


@pytest.mark.parametrize("d", [64, 128])
def test_forward_repeatable_and_rescale_options_agree(fa, d):
    say(f"[ab] tau / poly options d={d}")
    B, H, S = 1, 4, 1024
    shape = (B, H, S, d)
    qb = rand_bits(shape, 77, scale=3.0)  # large scores: the running max moves often
    kb, vb = rand_bits(shape, 78), rand_bits(shape, 79)
    scale = 1.0 / np.sqrt(d)
    Q, K, V = (gen.bf16_bits_to_f64(x) for x in (qb, kb, vb))
    refs = {c: oracle.attention_forward(Q, K, V, scale, c) for c in (False, True)}
    for tau, poly, deg in [(8.0, 0, 3), (0.0, 0, 3), (8.0, 1, 3), (8.0, 2, 3), (8.0, 2, 5), (2.0, 1, 5)]:
        opts = fa.Options(tau, poly, deg)
        for causal in (False, True):
            _, _, _, o, lse = run_fwd(fa, qb, kb, vb, causal, scale, opts)
            what = f"tau={tau} poly={poly}/8 deg={deg} causal={causal}"
            check_o(bf16_to_np64(o), refs[causal][0], what)
            check_lse(lse.cpu().numpy().astype(np.float64), refs[causal][1], what)
            _, _, _, o2, lse2 = run_fwd(fa, qb, kb, vb, causal, scale, opts)
            assert torch.equal(o, o2) and torch.equal(lse, lse2), f"{what}: not repeatable"


def test_reference_max_paths(fa):
    """The forward forms P against the running reference max first and takes
    row maxima only when a partial row sum exceeds 2^tau.  Equal scores (Q =
    0: every P is 1, so with tau = 2 every tile takes the row-max path and no
    row moves) must give the closed form, mean of V over the allowed keys and
    LSE = log(count); keys whose scores jump by more than tau in the last tile
    must move the reference there."""
    say("[ab] reference-max paths")
    B, H, S, d = 1, 2, 700, 128
    shape = (B, H, S, d)
    scale = 1.0 / np.sqrt(d)
    kb, vb = rand_bits(shape, 91), rand_bits(shape, 92)
    V = gen.bf16_bits_to_f64(vb)
    zero = np.zeros(shape, dtype=np.uint16)  # bf16 +0.0
    for tau in (8.0, 2.0, 0.0):
        for causal in (False, True):
            _, _, _, o, lse = run_fwd(fa, zero, kb, vb, causal, scale, fa.Options(tau))
            cnt = np.arange(1, S + 1, dtype=np.float64) if causal else np.full(S, float(S))
            o_ref = (np.cumsum(V, axis=2) / cnt[:, None]) if causal else np.broadcast_to(V.mean(axis=2, keepdims=True), shape)
            what = f"Q=0 tau={tau} causal={causal}"
            check_o(bf16_to_np64(o), o_ref, what)
            check_lse(lse.cpu().numpy().astype(np.float64), np.broadcast_to(np.log(cnt), (B, H, S)), what)
    # late jump: keys S-50.. get +96 on every raw score (12 in log2 units)
    q = gen.bf16_bits_to_f64(rand_bits(shape, 93)).astype(np.float32)
    k = gen.bf16_bits_to_f64(kb).astype(np.float32)
    q[..., 0] = 8.0
    k[..., : S - 50, 0] = 0.0
    k[..., S - 50:, 0] = 12.0
    qb2, kb2 = gen.f32_to_bf16_bits(q), gen.f32_to_bf16_bits(k)
    Q2, K2 = gen.bf16_bits_to_f64(qb2), gen.bf16_bits_to_f64(kb2)
    for tau in (8.0, 2.0):
        for causal in (False, True):
            o_ref, l_ref = oracle.attention_forward(Q2, K2, V, scale, causal)
            _, _, _, o, lse = run_fwd(fa, qb2, kb2, vb, causal, scale, fa.Options(tau))
            what = f"late jump tau={tau} causal={causal}"
            check_o(bf16_to_np64(o), o_ref, what)
            check_lse(lse.cpu().numpy().astype(np.float64), l_ref, what)


def test_device_exp2_polynomial(fa):
    say("[exp2] device polynomial")
    x = np.concatenate([np.linspace(-126.0, 0.0, 1 << 20), np.linspace(0.0, 8.0, 1 << 16),
                        np.arange(-126, 9, dtype=np.float64)]).astype(np.float32)
    xd = torch.from_numpy(x).cuda()
    for deg in (3, 5):
        y = torch.empty_like(xd)
        fa.fa_exp2_poly(xd, y, deg)
        torch.cuda.synchronize()
        ref = np.exp2(x.astype(np.float64))
        rel = np.abs(y.cpu().numpy().astype(np.float64) / ref - 1.0).max()
        assert rel <= 2e-4, (deg, rel)
    low = torch.tensor([-np.inf, -127.0, -200.0], dtype=torch.float32, device="cuda")
    y = torch.empty_like(low)
    fa.fa_exp2_poly(low, y, 3)
    torch.cuda.synchronize()
    assert torch.all(y == 0)


# ------------------------------------------------------------------ workload shapes, sampled
def sample_rows(S, extra=()):
    rng = np.random.default_rng(S)
    base = {0, 1, 31, 32, 63, 64, 127, 128, 129, S // 2, S - 129, S - 128, S - 65, S - 64, S - 2, S - 1}
    base |= set(int(x) for x in rng.integers(0, S, 24))
    base |= set(extra)
    return np.array(sorted(r for r in base if 0 <= r < S), dtype=np.int64)


_WORKLOAD_CACHE = {}


def workload_bits(name):
    """All four tensors of a workload, generated once per test session."""
    if name not in _WORKLOAD_CACHE:
        _WORKLOAD_CACHE.clear()  # keep one workload resident at a time
        _WORKLOAD_CACHE[name] = gen.workload_inputs(name, ("q", "k", "v", "do"))
    return _WORKLOAD_CACHE[name]


def head_f64(bits, b, h):
    return gen.bf16_bits_to_f64(bits[b, h])


WORKLOAD_FWD = [
    ("fwd_b4_h16_s4096", False),
    ("causal_boost_b2_h16_s8192", True),
    ("causal_fwdbwd_b2_h16_s16384", True),
    ("long_b1_h16_s32768", False),
    ("long_b1_h16_s32768", True),
]


@pytest.mark.parametrize("name,causal", WORKLOAD_FWD)
def test_workload_forward_sampled(fa, name, causal):
    say(f"[workload fwd] {name} causal={causal}")
    w = gen.WORKLOADS[name]
    bits = workload_bits(name)
    scale = gen.default_scale(w["d"])
    _, _, _, o, lse = run_fwd(fa, bits["q"], bits["k"], bits["v"], causal, scale)
    S = w["S"]
    boosted = range(0, S, 64) if w["boost"] else ()
    rows = sample_rows(S, extra=list(boosted)[:: max(1, len(boosted) // 16)] if boosted else ())
    heads = [(0, 0), (w["B"] - 1, w["H"] - 1)]
    for b, h in heads:
        Q, K, V = (head_f64(bits[t], b, h) for t in "qkv")
        o_ref, l_ref = oracle.forward_rows(Q, K, V, rows, scale, causal)
        o_g = bf16_to_np64(o[b, h, torch.from_numpy(rows).cuda()])
        l_g = lse[b, h, torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
        check_o(o_g, o_ref, f"{name} head ({b},{h})")
        check_lse(l_g, l_ref, f"{name} head ({b},{h})")


@pytest.mark.parametrize("name,causal", [("fwd_b4_h16_s4096", False), ("causal_boost_b2_h16_s8192", True)])
def test_workload_forward_full_tensors(fa, name, causal):
    """Every element of O and LSE of the two forward-only workloads against the
    oracle's full forward (its cost, 5.5e11 and 2.8e11 fp64 FLOP, is seconds),
    so the O mean-abs criterion runs over all elements."""
    say(f"[workload fwd full] {name} causal={causal}")
    w = gen.WORKLOADS[name]
    bits = workload_bits(name)
    scale = gen.default_scale(w["d"])
    _, _, _, o, lse = run_fwd(fa, bits["q"], bits["k"], bits["v"], causal, scale)
    Q, K, V = (gen.bf16_bits_to_f64(bits[t]) for t in "qkv")
    o_ref, l_ref = oracle.attention_forward(Q, K, V, scale, causal)
    del Q, K, V
    check_o(bf16_to_np64(o), o_ref, f"{name} all elements")
    check_lse(lse.cpu().numpy().astype(np.float64), l_ref, f"{name} all elements")


WORKLOAD_BWD = [
    ("fwd_b4_h16_s4096", False),
    ("causal_boost_b2_h16_s8192", True),  # every 64th query row x8: peaked rows
    ("causal_fwdbwd_b2_h16_s16384", True),
    ("long_b1_h16_s32768", False),
    ("long_b1_h16_s32768", True),
]


BWD_VARIANTS = {"split": dict(), "single-pass": dict(fused_backward=True), "stored dS": dict(stored_ds=True)}


@pytest.mark.parametrize("name,causal", WORKLOAD_BWD)
def test_workload_backward_sampled(fa, name, causal):
    """The three backward variants (split with recomputed dS, single-pass,
    split with stored dS) in the launch configuration bench.py times:
    sampled dQ rows of every head (cheap for the oracle: S*d work per row)
    and sampled dK/dV key rows of the first, a middle and the last head
    (each needs the full softmax of its head)."""
    say(f"[workload bwd] {name} causal={causal}")
    w = gen.WORKLOADS[name]
    bits = workload_bits(name)
    scale = gen.default_scale(w["d"])
    q, k, v, o, lse = run_fwd(fa, bits["q"], bits["k"], bits["v"], causal, scale)
    do = to_dev(bits["do"])
    S, B, H = w["S"], w["B"], w["H"]
    rows = sample_rows(S)
    idx = torch.from_numpy(rows).cuda()
    cols = np.array(sorted({0, 1, 127, 128, S // 3, S // 2, S - 129, S - 128, S - 1}), dtype=np.int64)
    cidx = torch.from_numpy(cols).cuda()
    got = {}
    for var, kw in BWD_VARIANTS.items():
        say(f"[workload bwd]   {var}")
        dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=causal, scale=scale, opts=fa.Options(**kw))
        torch.cuda.synchronize()
        got[var] = (dq[:, :, idx].cpu().numpy().astype(np.float64), bf16_to_np64(dk[:, :, cidx]),
                    bf16_to_np64(dv[:, :, cidx]))
        del dq, dk, dv
        torch.cuda.empty_cache()  # the stored dS of the 32k workloads is 16-32 GiB
    for b in range(B):
        for h in range(H):
            Q, K, V, dO = (head_f64(bits[t], b, h) for t in ("q", "k", "v", "do"))
            gq = oracle.backward_dq_rows(Q, K, V, dO, rows, scale, causal)
            for var in BWD_VARIANTS:
                check_grad(got[var][0][b, h], gq, f"{name} dQ rows head ({b},{h}) {var}")
    for b, h in sorted({(0, 0), (B // 2, H // 2), (B - 1, H - 1)}):
        Q, K, V, dO = (head_f64(bits[t], b, h) for t in ("q", "k", "v", "do"))
        gk, gv = oracle.backward_dkdv_cols(Q, K, V, dO, cols, scale, causal)
        for var in BWD_VARIANTS:
            check_grad(got[var][1][b, h], gk, f"{name} dK cols head ({b},{h}) {var}")
            check_grad(got[var][2][b, h], gv, f"{name} dV cols head ({b},{h}) {var}")


@pytest.mark.parametrize("B,H,S,d,causal", [(2, 3, 3000, 64, False), (2, 3, 3000, 64, True),
                                             (1, 2, 8300, 64, False), (1, 2, 5000, 128, True),
                                             (1, 2, 9000, 128, False)])
def test_ragged_sampled(fa, B, H, S, d, causal):
    """Multi-tile sizes with ragged tails (S not a multiple of 64 or 256),
    both head dimensions: sampled forward rows, dQ rows, dK/dV columns of two
    heads against the oracle.  Non-causal S >= 8192 takes the wide dQ shape
    (256 queries per workgroup)."""
    say(f"[ragged] B={B} H={H} S={S} d={d} causal={causal}")
    shape = (B, H, S, d)
    qb, kb, vb, dob = (rand_bits(shape, 7500 + i) for i in range(4))
    scale = 1.0 / np.sqrt(d)
    q, k, v, o, lse = run_fwd(fa, qb, kb, vb, causal, scale)
    grads = {st: fa.backward(q, k, v, o, lse, to_dev(dob), causal=causal, scale=scale,
                             opts=fa.Options(stored_ds=st)) for st in (False, True)}
    torch.cuda.synchronize()
    rows = sample_rows(S)
    cols = np.array(sorted({0, 1, 127, 128, S // 3, S // 2, S - 129, S - 128, S - 1}), dtype=np.int64)
    idx, cidx = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    for b, h in ((0, 0), (B - 1, H - 1)):
        Q, K, V, dO = (gen.bf16_bits_to_f64(x[b, h]) for x in (qb, kb, vb, dob))
        o_ref, l_ref = oracle.forward_rows(Q, K, V, rows, scale, causal)
        check_o(bf16_to_np64(o[b, h, idx]), o_ref, f"d={d} O rows head ({b},{h})")
        check_lse(lse[b, h, idx].cpu().numpy().astype(np.float64), l_ref, f"d={d} LSE rows head ({b},{h})")
        gq = oracle.backward_dq_rows(Q, K, V, dO, rows, scale, causal)
        gk, gv = oracle.backward_dkdv_cols(Q, K, V, dO, cols, scale, causal)
        for st, (dq, dk, dv) in grads.items():
            what = f"d={d} stored_ds={st}"
            check_grad(dq[b, h, idx].cpu().numpy().astype(np.float64), gq, f"{what} dQ rows head ({b},{h})")
            check_grad(bf16_to_np64(dk[b, h, cidx]), gk, f"{what} dK cols head ({b},{h})")
            check_grad(bf16_to_np64(dv[b, h, cidx]), gv, f"{what} dV cols head ({b},{h})")


def test_backward_is_bitwise_repeatable(fa):
    """Every gradient element is written once (no atomics): two runs agree bit for bit."""
    say("[determinism] backward twice")
    shape = (2, 4, 1000, 128)
    qb, kb, vb, db = (rand_bits(shape, 500 + i) for i in range(4))
    scale = 1.0 / np.sqrt(128)
    for causal in (False, True):
        q, k, v, o, lse = run_fwd(fa, qb, kb, vb, causal, scale)
        do = to_dev(db)
        for stored in (False, True):
            opts = fa.Options(stored_ds=stored)
            g1 = fa.backward(q, k, v, o, lse, do, causal=causal, scale=scale, opts=opts)
            g2 = fa.backward(q, k, v, o, lse, do, causal=causal, scale=scale, opts=opts)
            torch.cuda.synchronize()
            for a, b, nm in zip(g1, g2, ("dQ", "dK", "dV")):
                assert torch.equal(a, b), f"{nm} differs between runs (causal={causal}, stored_ds={stored})"


@pytest.mark.parametrize("B,H,S,d,causal", [(1, 3, 1100, 128, False), (2, 2, 1100, 128, True),
                                             (1, 2, 777, 64, False), (1, 3, 2049, 64, True)])
def test_stored_ds_steps_match_recompute(fa, B, H, S, d, causal):
    """The stored-dS path through its C-ABI steps (preprocess, dK/dV writing
    dS into the workspace, dQ reading it back) against the recomputing
    steps on the same inputs: dK and dV bitwise equal, dQ equal to the
    rounding of the bf16 dS (both compute dS = P (dP - D) from the same
    inputs, in transposed orientations); and the dQ of the stored path
    against the oracle on sampled rows."""
    say(f"[stored dS steps] B={B} H={H} S={S} d={d} causal={causal}")
    shape = (B, H, S, d)
    qb, kb, vb, db = (rand_bits(shape, 9100 + S + i) for i in range(4))
    scale = 1.0 / np.sqrt(d)
    q, k, v, o, lse = run_fwd(fa, qb, kb, vb, causal, scale)
    do = to_dev(db)
    res = {}
    for stored in (False, True):
        opts = fa.Options(stored_ds=stored)
        nb = fa.fa_bwd_workspace_bytes(B, H, S, d, causal, opts)
        ws = torch.full(((nb + 3) // 4,), float("nan"), dtype=torch.float32, device="cuda")
        dq = torch.empty((B, H, S, d), dtype=torch.float32, device="cuda")
        dk, dv = torch.empty_like(q), torch.empty_like(q)
        fa.fa_bwd_preprocess(o, do, lse, ws)
        fa.fa_bwd_dkdv(q, k, v, do, dk, dv, scale, causal, ws, opts=opts)
        fa.fa_bwd_dq(q, k, v, do, dq, scale, causal, ws, opts=opts)
        torch.cuda.synchronize()
        res[stored] = (dq, dk, dv)
    assert torch.equal(res[False][1], res[True][1]) and torch.equal(res[False][2], res[True][2])
    a, b = res[False][0].double(), res[True][0].double()
    assert torch.isfinite(b).all()
    rel = float((a - b).abs().max() / a.abs().max())
    assert rel <= 1e-3, f"dQ from stored dS vs recomputed: rel diff {rel:.3e}"
    rows = sample_rows(S)
    idx = torch.from_numpy(rows).cuda()
    for bb, h in ((0, 0), (B - 1, H - 1)):
        Q, K, V, dO = (gen.bf16_bits_to_f64(x[bb, h]) for x in (qb, kb, vb, db))
        gq = oracle.backward_dq_rows(Q, K, V, dO, rows, scale, causal)
        check_grad(res[True][0][bb, h, idx].cpu().numpy().astype(np.float64), gq, f"stored dS dQ head ({bb},{h})")


@pytest.mark.parametrize("B,H,S,d,causal", [(2, 3, 777, 128, False), (2, 3, 777, 128, True),
                                             (1, 5, 1000, 64, True)])
def test_stored_ds_head_groups_are_bitwise_the_single_launch(fa, B, H, S, d, causal):
    """With a workspace between fa_bwd_workspace_bytes_min and the full size,
    fa_bwd runs the stored-dS backward in groups of heads (one head; four
    heads); every head computes exactly as in the single launch."""
    say(f"[stored dS groups] B={B} H={H} S={S} d={d} causal={causal}")
    shape = (B, H, S, d)
    qb, kb, vb, db = (rand_bits(shape, 9300 + S + i) for i in range(4))
    scale = 1.0 / np.sqrt(d)
    q, k, v, o, lse = run_fwd(fa, qb, kb, vb, causal, scale)
    do = to_dev(db)
    on = fa.Options(stored_ds=True)
    full = fa.fa_bwd_workspace_bytes(B, H, S, d, causal, on)
    least = fa.fa_bwd_workspace_bytes_min(B, H, S, d, causal, on)
    base = fa.fa_bwd_workspace_bytes(B, H, S, d)
    per_head = least - base
    out = []
    for nbytes in (full, least, base + 4 * per_head + 100):
        ws = torch.full(((nbytes + 3) // 4,), float("nan"), dtype=torch.float32, device="cuda")
        dq = torch.empty((B, H, S, d), dtype=torch.float32, device="cuda")
        dk, dv = torch.empty_like(q), torch.empty_like(q)
        fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, scale, causal, ws, opts=on)
        torch.cuda.synchronize()
        out.append((dq, dk, dv))
    for grouped in out[1:]:
        for a, b, nm in zip(out[0], grouped, ("dQ", "dK", "dV")):
            assert torch.equal(a, b), f"{nm}: head groups differ from the single launch"
    Q, K, V, dO = (gen.bf16_bits_to_f64(x) for x in (qb, kb, vb, db))
    gq, gk, gv = oracle.attention_backward(Q, K, V, dO, scale, causal)
    check_grad(out[1][0].cpu().numpy().astype(np.float64), gq, "grouped stored dS dQ")
    check_grad(bf16_to_np64(out[1][1]), gk, "grouped stored dS dK")
    check_grad(bf16_to_np64(out[1][2]), gv, "grouped stored dS dV")


def test_options_do_not_mix_across_threads(fa):
    """Options travel with each call.  Two host threads launch forwards with
    different options on their own streams at the same time; every result is
    bitwise the one that option set gives alone (the polynomial exp2 and the
    max-first order change the rounding, so a mixed-up call would show)."""
    import threading
    say("[threads] per-call options")
    shape = (1, 4, 1024, 128)
    qb, kb, vb = (rand_bits(shape, 300 + i, scale=2.0) for i in range(3))
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    scale = 1.0 / np.sqrt(128)
    sets = [fa.Options(8.0, 0, 3), fa.Options(0.0, 2, 5), fa.Options(2.0, 1, 3, False)]
    ref = []
    for opts in sets:
        o, lse = fa.forward(q, k, v, causal=True, scale=scale, opts=opts)
        torch.cuda.synchronize()
        ref.append((o.clone(), lse.clone()))
    assert not torch.equal(ref[0][0], ref[1][0]), "option sets must give distinguishable bits"
    errors = []

    def worker(t):
        opts = sets[t]
        st = torch.cuda.Stream()
        try:
            for _ in range(20):
                o, lse = fa.forward(q, k, v, causal=True, scale=scale, opts=opts, stream=st)
                st.synchronize()
                if not (torch.equal(o, ref[t][0]) and torch.equal(lse, ref[t][1])):
                    errors.append(t)
        except Exception as e:  # pragma: no cover - reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(len(sets))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors


def test_backward_on_a_side_stream(fa):
    """backward() allocates its outputs and workspace on the stream it
    launches on.  With the kernels queued on a side stream and new
    allocations made on the current stream before any synchronisation, the
    gradients are bitwise those of a run on the current stream."""
    say("[stream] backward on a side stream")
    shape = (2, 4, 2000, 128)
    qb, kb, vb, db = (rand_bits(shape, 400 + i) for i in range(4))
    scale = 1.0 / np.sqrt(128)
    q, k, v, o, lse = run_fwd(fa, qb, kb, vb, True, scale)
    do = to_dev(db)
    ref = fa.backward(q, k, v, o, lse, do, causal=True, scale=scale)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        got = fa.backward(q, k, v, o, lse, do, causal=True, scale=scale, stream=side)
        # allocations and writes on the current stream while the side stream still runs
        junk = [torch.full((fa.fa_bwd_workspace_bytes(*shape) // 4,), 7.0, device="cuda") for _ in range(4)]
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        del junk
        for a, b, nm in zip(got, ref, ("dQ", "dK", "dV")):
            assert torch.equal(a, b), f"{nm} differs on the side stream"


# ------------------------------------------------------------------ packed variable-length forward
VARLEN = [
    # (sequence lengths, H, d, causal): empty, one-token, ragged and multi-tile sequences
    ([0, 1, 37, 129, 256, 300, 515, 64], 3, 128, False),
    ([0, 1, 37, 129, 256, 300, 515, 64], 3, 128, True),
    ([200, 0, 131, 1], 2, 64, True),
    ([1000, 17], 4, 128, True),
]


def varlen_case(lens, H, d, seed):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    qb, kb, vb = (rand_bits((total, H, d), seed + i) for i in range(3))
    return cu, total, qb, kb, vb


def seq_f64(bits, a, b):
    """Tokens a..b-1 of a [total, H, d] bf16 tensor as an oracle [1, H, L, d] array."""
    return np.ascontiguousarray(gen.bf16_bits_to_f64(bits[a:b]).transpose(1, 0, 2)[None])


@pytest.mark.parametrize("lens,H,d,causal", VARLEN)
def test_varlen_forward_matches_oracle_per_sequence(fa, lens, H, d, causal):
    say(f"[varlen] lens={lens} H={H} d={d} causal={causal}")
    cu, total, qb, kb, vb = varlen_case(lens, H, d, 7000 + d + int(causal) + len(lens))
    scale = 1.0 / np.sqrt(d)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    cu_d = torch.from_numpy(cu).cuda()
    o, lse = fa.forward_varlen(q, k, v, cu_d, max(lens), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_np, lse_np = bf16_to_np64(o), lse.cpu().numpy().astype(np.float64)
    for s in range(len(lens)):
        a, b = int(cu[s]), int(cu[s + 1])
        if a == b:
            continue
        o_ref, lse_ref = oracle.attention_forward(seq_f64(qb, a, b), seq_f64(kb, a, b), seq_f64(vb, a, b),
                                                  scale, causal)
        check_o(o_np[a:b].transpose(1, 0, 2), o_ref[0], f"varlen seq {s} (len {b - a})")
        check_lse(lse_np[:, a:b], lse_ref[0], f"varlen seq {s} (len {b - a})")


@pytest.mark.parametrize("d", [64, 128])
def test_varlen_softmax_options(fa, d):
    """The packed forward under the other softmax options (max-first order,
    hybrid exponentials) against the oracle, per sequence."""
    lens, H = [300, 0, 131, 1, 77], 2
    cu, total, qb, kb, vb = varlen_case(lens, H, d, 7300 + d)
    scale = 1.0 / np.sqrt(d)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    cu_d = torch.from_numpy(cu).cuda()
    for tau, poly, deg in [(0.0, 2, 5), (2.0, 1, 3)]:
        for causal in (False, True):
            say(f"[varlen options] d={d} tau={tau} poly={poly}/8 deg={deg} causal={causal}")
            o, lse = fa.forward_varlen(q, k, v, cu_d, max(lens), causal=causal, scale=scale,
                                       opts=fa.Options(tau, poly, deg))
            torch.cuda.synchronize()
            o_np, lse_np = bf16_to_np64(o), lse.cpu().numpy().astype(np.float64)
            for sq in range(len(lens)):
                a, b = int(cu[sq]), int(cu[sq + 1])
                if a == b:
                    continue
                o_ref, lse_ref = oracle.attention_forward(seq_f64(qb, a, b), seq_f64(kb, a, b),
                                                          seq_f64(vb, a, b), scale, causal)
                what = f"varlen seq {sq} tau={tau} poly={poly} deg={deg} causal={causal}"
                check_o(o_np[a:b].transpose(1, 0, 2), o_ref[0], what)
                check_lse(lse_np[:, a:b], lse_ref[0], what)


def test_varlen_equals_dense_forward_bitwise(fa):
    """Each sequence of a packed batch gives bit for bit what the dense
    [1, H, L, d] forward gives: the same kernel, only the addressing differs."""
    lens, H, d = [300, 1, 129, 640], 2, 128
    say(f"[varlen vs dense] lens={lens}")
    cu, total, qb, kb, vb = varlen_case(lens, H, d, 7100)
    scale = 1.0 / np.sqrt(d)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    cu_d = torch.from_numpy(cu).cuda()
    for causal in (False, True):
        o, lse = fa.forward_varlen(q, k, v, cu_d, max(lens), causal=causal, scale=scale)
        for s in range(len(lens)):
            a, b = int(cu[s]), int(cu[s + 1])
            qs, ks, vs = (t[a:b].transpose(0, 1).unsqueeze(0).contiguous() for t in (q, k, v))
            od, lsed = fa.forward(qs, ks, vs, causal=causal, scale=scale)
            torch.cuda.synchronize()
            assert torch.equal(o[a:b], od[0].transpose(0, 1)), f"O of sequence {s} (causal={causal})"
            assert torch.equal(lse[:, a:b], lsed[0]), f"LSE of sequence {s} (causal={causal})"


def test_varlen_clamps_offsets(fa):
    """Offsets below 0 or past total are clamped (to 0 and total): the batch
    then splits as [0, 30), [30, 30), [30, total)."""
    H, d, total = 2, 128, 100
    say("[varlen clamp] cu = [-5, 30, 30, 250], total 100")
    qb, kb, vb = (rand_bits((total, H, d), 7200 + i) for i in range(3))
    cu_d = torch.tensor([-5, 30, 30, 250], dtype=torch.int32).cuda()
    scale = 1.0 / np.sqrt(d)
    o, lse = fa.forward_varlen(to_dev(qb), to_dev(kb), to_dev(vb), cu_d, 128, causal=True, scale=scale)
    torch.cuda.synchronize()
    o_np, lse_np = bf16_to_np64(o), lse.cpu().numpy().astype(np.float64)
    for a, b in ((0, 30), (30, 100)):
        o_ref, lse_ref = oracle.attention_forward(seq_f64(qb, a, b), seq_f64(kb, a, b), seq_f64(vb, a, b),
                                                  scale, True)
        check_o(o_np[a:b].transpose(1, 0, 2), o_ref[0], f"clamped [{a}, {b})")
        check_lse(lse_np[:, a:b], lse_ref[0], f"clamped [{a}, {b})")


def test_varlen_many_sequences_and_work_order(fa):
    """More than 64 sequences (the work-item search walks the offsets in
    chunks of 64), zero-length ones among them, in no particular order; the
    longest-first and reversed work orders give the same bits."""
    rng = np.random.default_rng(7300)
    lens = [int(x) for x in rng.integers(0, 600, 150)]
    lens[3] = lens[77] = 0
    H, d = 2, 64
    say(f"[varlen many] {len(lens)} sequences, {sum(lens)} tokens")
    cu, total, qb, kb, vb = varlen_case(lens, H, d, 7300)
    scale = 1.0 / np.sqrt(d)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    cu_d = torch.from_numpy(cu).cuda()
    for causal in (False, True):
        o, lse = fa.forward_varlen(q, k, v, cu_d, max(lens), causal=causal, scale=scale,
                                   opts=fa.Options(longest_first=True))
        o2, lse2 = fa.forward_varlen(q, k, v, cu_d, max(lens), causal=causal, scale=scale,
                                     opts=fa.Options(longest_first=False))
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(lse, lse2), f"work order changed the result (causal={causal})"
        o_np, lse_np = bf16_to_np64(o), lse.cpu().numpy().astype(np.float64)
        for si in range(len(lens)):
            a, b = int(cu[si]), int(cu[si + 1])
            if a == b:
                continue
            o_ref, lse_ref = oracle.attention_forward(seq_f64(qb, a, b), seq_f64(kb, a, b), seq_f64(vb, a, b),
                                                      scale, causal)
            check_o(o_np[a:b].transpose(1, 0, 2), o_ref[0], f"seq {si} (len {b - a}, causal={causal})")
            check_lse(lse_np[:, a:b], lse_ref[0], f"seq {si} (len {b - a}, causal={causal})")


def test_varlen_rows_past_max_seqlen_untouched(fa):
    """max_seqlen below a sequence's length: the launch covers
    ceil(max_seqlen / 256) query blocks per sequence; rows past them keep
    what the output held, rows before them are exact."""
    lens, H, d, maxlen = [700, 100], 2, 128, 300   # 2 blocks: rows 0..511 of sequence 0
    say(f"[varlen max_seqlen] lens={lens} max_seqlen={maxlen}")
    cu, total, qb, kb, vb = varlen_case(lens, H, d, 7400)
    scale = 1.0 / np.sqrt(d)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    cu_d = torch.from_numpy(cu).cuda()
    for causal in (False, True):
        o = torch.full((total, H, d), 1024.0, device="cuda").to(torch.bfloat16)
        lse = torch.full((H, total), -7.0, device="cuda")
        fa.fa_fwd_varlen(q, k, v, o, lse, cu_d, maxlen, scale, causal)
        torch.cuda.synchronize()
        o_np, lse_np = bf16_to_np64(o), lse.cpu().numpy().astype(np.float64)
        assert np.all(o_np[512:700] == 1024.0) and np.all(lse_np[:, 512:700] == -7.0), "rows past the blocks written"
        for a, b, rows in ((0, 700, 512), (700, 800, 100)):
            o_ref, lse_ref = oracle.attention_forward(seq_f64(qb, a, b), seq_f64(kb, a, b), seq_f64(vb, a, b),
                                                      scale, causal)
            check_o(o_np[a:a + rows].transpose(1, 0, 2), o_ref[0][:, :rows], f"[{a}, {b}) causal={causal}")
            check_lse(lse_np[:, a:a + rows], lse_ref[0][:, :rows], f"[{a}, {b}) causal={causal}")


def test_varlen_prefill_workload_sampled(fa):
    """The packed prefill batch that bench.py --varlen times, in the same
    launch configuration: sampled rows of the shortest, the longest and a
    middle sequence, first and last head, against the oracle."""
    name = "prefill_varlen_h16_d128"
    w = gen.VARLEN_WORKLOADS[name]
    say(f"[varlen workload] {name}")
    lens, bits = gen.varlen_inputs(name)
    _WORKLOAD_CACHE.clear()
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    H, d = w["H"], w["d"]
    scale = gen.default_scale(d)
    q, k, v = (to_dev(bits[t]) for t in ("q", "k", "v"))
    o, lse = fa.forward_varlen(q, k, v, torch.from_numpy(cu).cuda(), int(lens.max()), causal=w["causal"],
                               scale=scale)
    torch.cuda.synchronize()
    order = np.argsort(lens)
    for s in (int(order[0]), int(order[len(order) // 2]), int(order[-1])):
        a, b = int(cu[s]), int(cu[s + 1])
        rows = sample_rows(b - a)
        for h in (0, H - 1):
            Q, K, V = (gen.bf16_bits_to_f64(bits[t][a:b, h]) for t in ("q", "k", "v"))
            o_ref, l_ref = oracle.forward_rows(Q, K, V, rows, scale, w["causal"])
            idx = torch.from_numpy(rows + a).cuda()
            check_o(bf16_to_np64(o[idx, h]), o_ref, f"{name} seq {s} head {h}")
            check_lse(lse[h, idx].cpu().numpy().astype(np.float64), l_ref, f"{name} seq {s} head {h}")


def test_causal_block_order_does_not_change_results(fa):
    """Longest-first and shortest-first block orders run the same arithmetic
    per block: forward and backward agree bit for bit."""
    say("[causal order] lpt on/off")
    shape = (1, 3, 700, 128)
    qb, kb, vb, db = (rand_bits(shape, 600 + i) for i in range(4))
    scale = 1.0 / np.sqrt(128)
    for stored in (False, True):
        out = []
        for lpt in (True, False):
            opts = fa.Options(longest_first=lpt, stored_ds=stored)
            q, k, v, o, lse = run_fwd(fa, qb, kb, vb, True, scale, opts)
            g = fa.backward(q, k, v, o, lse, to_dev(db), causal=True, scale=scale, opts=opts)
            torch.cuda.synchronize()
            out.append((o, lse) + tuple(g))
        for a, b, nm in zip(out[0], out[1], ("O", "LSE", "dQ", "dK", "dV")):
            assert torch.equal(a, b), f"{nm} depends on the causal block order (stored_ds={stored})"
