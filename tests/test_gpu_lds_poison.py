"""Barrier discipline of the LDS stages, checked with the LDS-poison build.

libfa_poison.so is libfa.so compiled with -DFA_LDS_POISON: every direct
memory-to-LDS copy first fills its destination with all-ones bytes (NaN as
fp32 and bf16) and waits for that write before the copy is issued.  If any
wave read a stage while another wave refilled it, or before its copy had
landed, it would read NaN (or a half-filled tile) and the result would
change.  The arithmetic of the two builds is the same, so every output of
every kernel family must agree bit for bit between them: forward (both
masks, both head dimensions, ragged tails), packed varlen forward, and the
three backward variants (recomputed dS, stored dS, single pass).
"""
import contextlib
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
POISON = os.path.join(ROOT, "exact_attention_39_amd", "libfa_poison.so")


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the -m gpu tests need an MI355X")
    import exact_attention_39_amd as m
    m.load_library()
    if not os.path.exists(POISON):
        pytest.fail("libfa_poison.so is not built: run __graft_entry__.build()")
    return m


@contextlib.contextmanager
def library(fa, path):
    """Route the binding to another build of the library for the duration."""
    saved = (fa._lib, fa.LIB_PATH)
    fa._lib, fa.LIB_PATH = None, path
    try:
        fa.load_library()
        yield
    finally:
        torch.cuda.synchronize()
        fa._lib, fa.LIB_PATH = saved


def randn(shape, seed, scale=1.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16).cuda()


def both_builds(fa, fn):
    """fn() under libfa.so, then under libfa_poison.so; results as tuples."""
    normal = tuple(t.clone() for t in fn())
    torch.cuda.synchronize()
    with library(fa, POISON):
        poisoned = tuple(t.clone() for t in fn())
    return normal, poisoned


def assert_same(normal, poisoned, what):
    for i, (a, b) in enumerate(zip(normal, poisoned)):
        assert torch.equal(a, b), f"{what}: output {i} differs under LDS poison"
        assert not torch.isnan(b.float()).any(), f"{what}: output {i} has NaN under LDS poison"


@pytest.mark.parametrize("B,H,S,d,causal", [(1, 3, 1000, 128, False), (2, 2, 777, 128, True),
                                             (1, 4, 1300, 64, False), (1, 2, 2049, 64, True),
                                             (1, 8, 515, 128, True)])
def test_forward_and_backward_variants_under_poison(fa, B, H, S, d, causal):
    print(f"[poison] B={B} H={H} S={S} d={d} causal={causal}", flush=True)
    shape = (B, H, S, d)
    q, k, v, do = (randn(shape, 40 + i) for i in range(4))
    scale = d ** -0.5

    def fwd():
        return fa.forward(q, k, v, causal=causal, scale=scale)

    n, p = both_builds(fa, fwd)
    assert_same(n, p, "forward")
    o, lse = n
    variants = {"recomputed dS": fa.Options(), "stored dS": fa.Options(stored_ds=True)}
    if (B * H) % 8 == 0:
        variants["single pass"] = fa.Options(fused_backward=True)
    for name, opts in variants.items():
        def bwd():
            return fa.backward(q, k, v, o, lse, do, causal=causal, scale=scale, opts=opts)
        n, p = both_builds(fa, bwd)
        assert_same(n, p, f"backward, {name}")


def test_varlen_forward_under_poison(fa):
    print("[poison] varlen", flush=True)
    lens = [0, 1, 300, 1000, 64, 515]
    H, d = 3, 128
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
    total, mx = int(sum(lens)), max(lens)
    q, k, v = (randn((total, H, d), 70 + i) for i in range(3))
    for causal in (False, True):
        def fwd():
            return fa.forward_varlen(q, k, v, cu, mx, causal=causal)
        n, p = both_builds(fa, fwd)
        assert_same(n, p, f"varlen forward causal={causal}")
