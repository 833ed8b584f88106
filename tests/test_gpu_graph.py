"""The attention path under HIP graph capture.

Every entry point only enqueues kernels on the caller's stream: no
allocation, no synchronisation, no memset (the preprocess kernel clears the
sync words itself).  So a forward + backward sequence can be captured once
and replayed.  The test captures fa_fwd, fa_bwd (default and stored dS) and
fa_bwd_noalloc into one graph, then replays it three times with new inputs
written eagerly between the replays (and a synchronisation after each), and
requires every replay to equal, bit for bit, the same calls made eagerly on
those inputs.
"""
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the -m gpu tests need an MI355X")
    import exact_attention_39_amd as m
    m.load_library()
    return m


def randn_(t, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    t.copy_(torch.randn(t.shape, generator=g).to(torch.bfloat16))


@pytest.mark.parametrize("causal", [False, True])
def test_forward_backward_graph_replays_match_eager(fa, causal):
    print(f"[graph] causal={causal}", flush=True)
    B, H, S, d = 1, 8, 1100, 128
    scale = d ** -0.5
    shape = (B, H, S, d)
    dev = "cuda"
    q, k, v, do = (torch.empty(shape, dtype=torch.bfloat16, device=dev) for _ in range(4))
    stored = fa.Options(stored_ds=True)

    def buffers():
        o = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
        grads = [(torch.empty(shape, dtype=torch.float32, device=dev), torch.empty(shape, dtype=torch.bfloat16,
                  device=dev), torch.empty(shape, dtype=torch.bfloat16, device=dev)) for _ in range(3)]
        return o, lse, grads

    ws_default = torch.empty(fa.fa_bwd_workspace_bytes(B, H, S, d) // 4 + 1, dtype=torch.float32, device=dev)
    ws_stored = torch.empty(fa.fa_bwd_workspace_bytes(B, H, S, d, causal, stored) // 4 + 1,
                            dtype=torch.float32, device=dev)

    def run(bufs):
        o, lse, grads = bufs
        fa.fa_fwd(q, k, v, o, lse, scale, causal)
        fa.fa_bwd(q, k, v, o, lse, do, *grads[0], scale, causal, ws_default)
        fa.fa_bwd(q, k, v, o, lse, do, *grads[1], scale, causal, ws_stored, opts=stored)
        fa.fa_bwd_noalloc(q, k, v, o, lse, do, *grads[2], scale, causal)

    def flat(bufs):
        o, lse, grads = bufs
        return [o, lse] + [t for g in grads for t in g]

    for t, seed in zip((q, k, v, do), (1, 2, 3, 4)):
        randn_(t, seed)
    captured = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        run(captured)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(captured)
    torch.cuda.synchronize()

    eager = buffers()
    for replay in range(3):
        for t, seed in zip((q, k, v, do), (10 * replay + 11, 10 * replay + 12, 10 * replay + 13, 10 * replay + 14)):
            randn_(t, seed)  # new inputs, written eagerly
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        run(eager)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(flat(captured), flat(eager))):
            assert torch.equal(a, b), f"replay {replay}: output {i} differs from the eager calls"
        assert not torch.isnan(captured[0].float()).any()
