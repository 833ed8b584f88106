"""The C-ABI library without a GPU: it loads, exports every function that
include/fa.h declares, and rejects malformed calls before touching the GPU
(argument checks run on the host, ahead of any HIP call)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def lib():
    import exact_attention_39_amd as fa
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libfa.so is not built: run __graft_entry__.build()")
    return fa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_status_string"} <= set(names)
    nm = subprocess.check_output(["nm", "-D", "--defined-only", os.path.join(ROOT, "exact_attention_39_amd", "libfa.so")],
                                 text=True)
    exported = {l.split()[-1] for l in nm.splitlines() if " T " in l}
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_poison_build_exports_the_same_symbols():
    """The LDS-poison debug build (libfa_poison.so) is the same library."""
    path = os.path.join(ROOT, "exact_attention_39_amd", "libfa_poison.so")
    if not os.path.exists(path):
        pytest.fail("libfa_poison.so is not built: run __graft_entry__.build()")
    nm = subprocess.check_output(["nm", "-D", "--defined-only", path], text=True)
    exported = {l.split()[-1] for l in nm.splitlines() if " T " in l}
    assert set(declared_functions()) <= exported


def test_status_strings(lib):
    for code in range(5):
        assert lib.fa_status_string(code).decode().startswith("FA_")


NULL = None
A = ctypes.c_void_p(0x10000)   # aligned fake device addresses (never dereferenced: calls fail first)
MIS = ctypes.c_void_p(0x10008)


def fwd(lib, B=1, H=1, S=128, d=128, scale=0.088, causal=0, ptrs=None):
    p = ptrs or [A, A, A, A, A]
    return lib.fa_fwd(*p, B, H, S, d, ctypes.c_float(scale), causal, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), 1), (dict(H=-2), 1), (dict(S=-5), 1), (dict(d=96), 2), (dict(d=256), 2),
    (dict(scale=0.0), 1), (dict(scale=-1.0), 1), (dict(scale=float("nan")), 1), (dict(scale=float("inf")), 1),
    (dict(causal=2), 1), (dict(causal=-1), 1), (dict(S=(1 << 22) + 1), 1),
])
def test_forward_rejects_bad_arguments(lib, kw, code):
    assert fwd(lib, **kw) == code


def test_forward_rejects_null_and_misaligned(lib):
    assert fwd(lib, ptrs=[A, A, A, NULL, A]) == 1
    assert fwd(lib, ptrs=[A, MIS, A, A, A]) == 1
    assert fwd(lib, ptrs=[A, A, A, A, MIS]) == 1


def test_empty_calls_are_ok_without_gpu(lib):
    assert fwd(lib, S=0, ptrs=[NULL] * 5) == 0
    assert fwd(lib, B=0, ptrs=[NULL] * 5) == 0
    ws = lib.fa_bwd_workspace_bytes(1, 1, 0, 128)
    assert ws == 0
    assert lib.fa_bwd(*([NULL] * 9), 1, 1, 0, 128, ctypes.c_float(0.1), 1, NULL, 0, NULL) == 0


def test_backward_checks(lib):
    # -D and LSE*log2 e (8 bytes per row, rounded up to 256), then the sync words of the
    # single-pass backward: 32 + 8 * B*H * ceil(S / 32) int32, rounded up to 256 bytes
    def ws_bytes(bh, S):
        return (8 * bh * S + 255) // 256 * 256 + ((32 + 8 * bh * -(-S // 32)) * 4 + 255) // 256 * 256
    assert lib.fa_bwd_workspace_bytes(2, 3, 100, 128) == ws_bytes(6, 100) == 4864 + 1024
    assert lib.fa_bwd_workspace_bytes(1, 16, 32768, 128) == ws_bytes(16, 32768)
    assert lib.fa_bwd_workspace_bytes(1, 1, 128, 128) == 1280
    p9 = [A] * 9
    # workspace too small (needs 1280 bytes)
    assert lib.fa_bwd(*p9, 1, 1, 128, 128, ctypes.c_float(0.1), 0, A, 1276, NULL) == 1
    # null workspace
    assert lib.fa_bwd(*p9, 1, 1, 128, 128, ctypes.c_float(0.1), 0, NULL, 1024, NULL) == 1
    # misaligned dQ
    p = list(p9)
    p[6] = MIS
    assert lib.fa_bwd(*p, 1, 1, 128, 128, ctypes.c_float(0.1), 0, A, 1280, NULL) == 1
    assert lib.fa_bwd(*p9, 1, 1, 128, 64 + 1, ctypes.c_float(0.1), 0, A, 1280, NULL) == 2
    assert lib.fa_bwd_dkdv(*([A] * 6), 1, 1, 128, 128, ctypes.c_float(0.1), 3, NULL, A, 1280, NULL) == 1
    assert lib.fa_bwd_dkdv(*([A] * 5), MIS, 1, 1, 128, 128, ctypes.c_float(0.1), 0, NULL, A, 1280, NULL) == 1
    assert lib.fa_bwd_dq(*([A] * 4), MIS, 1, 1, 128, 128, ctypes.c_float(0.1), 0, NULL, A, 1280, NULL) == 1
    assert lib.fa_bwd_dq(*([A] * 5), 1, 1, 128, 128, ctypes.c_float(0.0), 0, NULL, A, 1280, NULL) == 1
    assert lib.fa_bwd_preprocess(A, MIS, A, 1, 1, 128, 128, A, 1280, NULL) == 1
    assert lib.fa_bwd_preprocess(A, A, NULL, 1, 1, 128, 128, A, 1280, NULL) == 1
    assert lib.fa_bwd_preprocess(A, A, A, 1, 1, 128, 128, A, 4, NULL) == 1


def test_default_options(lib):
    import exact_attention_39_amd as fa
    o = lib.fa_default_options()
    assert (o.rescale_tau, o.poly_eighths, o.poly_degree, o.longest_first, o.fused_backward,
            o.stored_ds) == (8.0, 0, 3, 1, 0, 0)
    assert ctypes.sizeof(fa.Options) == 24
    assert repr(fa.default_options()) == repr(fa.Options())


@pytest.mark.parametrize("fields", [(-1.0, 0, 3, 1, 1, 0), (float("nan"), 0, 3, 1, 1, 0), (65.0, 0, 3, 1, 1, 0),
                                    (8.0, 3, 3, 1, 1, 0), (8.0, -1, 3, 1, 1, 0), (8.0, 1, 4, 1, 1, 0),
                                    (8.0, 0, 3, 2, 1, 0), (8.0, 0, 3, 1, 2, 0), (8.0, 0, 3, 1, -1, 0),
                                    (8.0, 0, 3, 1, 0, 2), (8.0, 0, 3, 1, 0, -1),
                                    (8.0, 0, 3, 1, 1, 1)])  # single-pass and stored dS exclude each other
def test_options_out_of_range_are_rejected_by_every_entry_point(lib, fields):
    """Per-call options are validated on the host, before any HIP call: every
    entry point that takes them returns FA_ERR_INVALID for a bad field."""
    import exact_attention_39_amd as fa
    o = fa.Options()
    o.rescale_tau, o.poly_eighths, o.poly_degree, o.longest_first, o.fused_backward, o.stored_ds = fields
    po = ctypes.byref(o)
    f = ctypes.c_float
    assert lib.fa_fwd_opt(A, A, A, A, A, 1, 1, 128, 128, f(0.1), 0, po, NULL) == 1
    assert lib.fa_fwd_varlen(A, A, A, A, A, A, 2, 2, 300, 200, 128, f(0.1), 0, po, NULL) == 1
    assert lib.fa_bwd_opt(*([A] * 9), 1, 1, 128, 128, f(0.1), 0, po, A, 1024, NULL) == 1
    assert lib.fa_bwd_dkdv(*([A] * 6), 1, 1, 128, 128, f(0.1), 0, po, A, 1024, NULL) == 1
    assert lib.fa_bwd_dq(*([A] * 5), 1, 1, 128, 128, f(0.1), 0, po, A, 1024, NULL) == 1
    # bad options are rejected even for empty calls (nothing else is looked at)
    assert lib.fa_fwd_opt(*([NULL] * 5), 1, 1, 0, 128, f(0.1), 0, po, NULL) == 1
    assert lib.fa_bwd_workspace_bytes_opt(1, 1, 128, 128, 0, po) == 0


def ds_tiles(S, causal):
    """32 KB tiles of the stored dS per head: one per (256-key block, 64-query
    iteration) that the mask keeps, causal: iterations i >= 4 kb."""
    nkb, nqi = -(-S // 256), -(-S // 64)
    return sum(nqi - (4 * kb if causal else 0) for kb in range(nkb))


@pytest.mark.parametrize("B,H,S,d", [(1, 1, 1, 64), (2, 3, 100, 128), (1, 2, 300, 128), (1, 16, 32768, 128),
                                     (2, 16, 16384, 128), (1, 4, 4099, 64)])
def test_stored_ds_workspace(lib, B, H, S, d):
    """With stored_ds the workspace is the default one plus the dS tiles;
    a workspace of the default size is refused on the host by every step
    that reads or writes dS."""
    import exact_attention_39_amd as fa
    f = ctypes.c_float
    base = lib.fa_bwd_workspace_bytes(B, H, S, d)
    on = fa.Options(stored_ds=True)
    for causal in (0, 1):
        assert lib.fa_bwd_workspace_bytes_opt(B, H, S, d, causal, NULL) == base
        assert lib.fa_bwd_workspace_bytes_opt(B, H, S, d, causal, ctypes.byref(fa.Options())) == base
        need = lib.fa_bwd_workspace_bytes_opt(B, H, S, d, causal, ctypes.byref(on))
        assert need == base + B * H * ds_tiles(S, causal) * 32768
        assert fa.fa_bwd_workspace_bytes(B, H, S, d, bool(causal), on) == need
        po = ctypes.byref(on)
        least = lib.fa_bwd_workspace_bytes_min(B, H, S, d, causal, po)
        assert least == base + ds_tiles(S, causal) * 32768  # one head's dS: heads run in groups
        assert lib.fa_bwd_workspace_bytes_min(B, H, S, d, causal, NULL) == base
        assert lib.fa_bwd_opt(*([A] * 9), B, H, S, d, f(0.1), causal, po, A, least - 16, NULL) == 1
        assert lib.fa_bwd_dkdv(*([A] * 6), B, H, S, d, f(0.1), causal, po, A, base, NULL) == 1
        assert lib.fa_bwd_dq(*([A] * 5), B, H, S, d, f(0.1), causal, po, A, base, NULL) == 1
    # the causal layout keeps about half the tiles
    if S >= 4096:
        assert 0.49 < ds_tiles(S, True) / ds_tiles(S, False) < 0.52
    assert lib.fa_bwd_workspace_bytes_opt(B, H, 0, d, 0, ctypes.byref(on)) == 0


def test_options_are_read_once_per_call_no_shared_state(lib):
    """The library holds no tuning state: a call with NULL options behaves as
    the defaults whatever other calls passed before (here: a valid non-default
    set, then an invalid one, then NULL on an empty call)."""
    import exact_attention_39_amd as fa
    f = ctypes.c_float
    odd = fa.Options(0.0, 2, 5, False)
    assert lib.fa_fwd_opt(*([NULL] * 5), 1, 1, 0, 128, f(0.1), 0, ctypes.byref(odd), NULL) == 0
    bad = fa.Options(8.0, 7, 3, True)
    assert lib.fa_fwd_opt(*([NULL] * 5), 1, 1, 0, 128, f(0.1), 0, ctypes.byref(bad), NULL) == 1
    assert lib.fa_fwd_opt(*([NULL] * 5), 1, 1, 0, 128, f(0.1), 0, NULL, NULL) == 0
    assert "fa_set_softmax_options" not in declared_functions()
    assert "fa_set_causal_order" not in declared_functions()


def test_exp2_poly_validation(lib):
    assert lib.fa_exp2_poly(NULL, NULL, -1, 3, NULL) == 1
    assert lib.fa_exp2_poly(NULL, NULL, 0, 3, NULL) == 0
    assert lib.fa_exp2_poly(A, A, 16, 4, NULL) == 1


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    import exact_attention_39_amd as fa
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        fa.forward(q, q, q)


def fwd_varlen(lib, nseq=2, H=2, total=300, max_seqlen=200, d=128, scale=0.088, causal=0, ptrs=None, cu=A):
    p = ptrs or [A, A, A, A, A]
    return lib.fa_fwd_varlen(*p, cu, nseq, H, total, max_seqlen, d, ctypes.c_float(scale), causal, NULL, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(nseq=-1), 1), (dict(H=-1), 1), (dict(total=-3), 1), (dict(max_seqlen=-1), 1),
    (dict(d=80), 2), (dict(scale=0.0), 1), (dict(scale=float("nan")), 1), (dict(causal=2), 1),
    (dict(max_seqlen=(1 << 22) + 1), 1),
    # row offsets of one (sequence, head) must stay below 2^32
    (dict(total=1 << 20, H=16), 1),
    # the furthest query block: max_seqlen rounded up to 256 rows, at H*d*2 bytes per row
    (dict(total=300, max_seqlen=(1 << 22), H=8, d=128), 1),
    # one sequence of 2,796,202 tokens at H = 12, d = 64: total * H * d * 2 < 2^32, but the key/value
    # tile copies reach 192 rows past the end, whose offsets would wrap onto the first rows
    (dict(nseq=1, total=2796202, max_seqlen=2796202, H=12, d=64), 1),
])
def test_varlen_forward_rejects_bad_arguments(lib, kw, code):
    assert fwd_varlen(lib, **kw) == code


def test_varlen_offset_bound_is_tight(lib):
    """The largest accepted packed batch has every row offset the kernel forms
    below 2^32: reach = max(round_up(max_seqlen, 256), total + 192) rows of
    H*d*2 bytes.  One token more is rejected (fake pointers: a call that passes
    the checks would launch, so only the rejected side runs here)."""
    H, d = 12, 64
    pitch = H * d * 2
    total_ok = (1 << 32) // pitch - 192
    assert (total_ok + 192) * pitch <= (1 << 32) < (total_ok + 193) * pitch
    assert fwd_varlen(lib, nseq=1, total=total_ok + 1, max_seqlen=total_ok + 1, H=H, d=d) == 1
    maxlen_bad = (1 << 32) // pitch // 256 * 256 + 1     # rounds up past the limit
    assert fwd_varlen(lib, nseq=1, total=100, max_seqlen=maxlen_bad, H=H, d=d) == 1


def test_varlen_forward_null_misaligned_and_empty(lib):
    assert fwd_varlen(lib, cu=NULL) == 1
    assert fwd_varlen(lib, cu=ctypes.c_void_p(0x10002)) == 1      # cu_seqlens not 4-byte aligned
    assert fwd_varlen(lib, ptrs=[A, A, MIS, A, A]) == 1
    assert fwd_varlen(lib, ptrs=[A, A, A, A, NULL]) == 1
    # empty calls: nothing to compute, nothing dereferenced
    assert fwd_varlen(lib, nseq=0, ptrs=[NULL] * 5, cu=NULL) == 0
    assert fwd_varlen(lib, total=0, ptrs=[NULL] * 5, cu=NULL) == 0
    assert fwd_varlen(lib, max_seqlen=0, ptrs=[NULL] * 5, cu=NULL) == 0
    assert fwd_varlen(lib, H=0, ptrs=[NULL] * 5, cu=NULL) == 0


def test_varlen_binding_checks_shapes():
    torch = pytest.importorskip("torch")
    import exact_attention_39_amd as fa
    q = torch.zeros(10, 2, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 4, 10], dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        fa.forward_varlen(q, q, q, cu, 6)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus N > 1 exits with a message, before
    touching the GPU."""
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "not supported" in r.stderr and r.stdout == ""


def test_noalloc_backward_host_checks(lib):
    """fa_bwd_noalloc rejects a workspace larger than its static array
    (FA_ERR_TOO_LARGE = 4), and malformed calls, on the host before any HIP
    call; empty calls are no-ops."""
    import exact_attention_39_amd as fa
    f = ctypes.c_float
    p9 = [A] * 9
    # about 9 bytes of workspace per (b, h, query row): the largest S for B = H = 1
    S_max = max(S for S in range(1800000, 1900000, 32) if lib.fa_bwd_workspace_bytes(1, 1, S, 128) <= fa.NOALLOC_SCRATCH_BYTES)
    assert lib.fa_bwd_workspace_bytes(1, 1, S_max + 32, 128) > fa.NOALLOC_SCRATCH_BYTES
    assert lib.fa_bwd_noalloc(*p9, 1, 1, S_max + 32, 128, f(0.1), 0, NULL) == 4
    assert lib.fa_bwd_noalloc(*p9, 2, 16, 65537, 128, f(0.1), 1, NULL) == 4
    assert lib.fa_bwd_noalloc(*p9, 1, 1, 128, 96, f(0.1), 0, NULL) == 2
    assert lib.fa_bwd_noalloc(*p9, 1, 1, 128, 128, f(0.0), 0, NULL) == 1
    assert lib.fa_bwd_noalloc(*p9, 1, 1, 128, 128, f(0.1), 2, NULL) == 1
    p = list(p9)
    p[6] = MIS
    assert lib.fa_bwd_noalloc(*p, 1, 1, 128, 128, f(0.1), 0, NULL) == 1
    p[6] = NULL
    assert lib.fa_bwd_noalloc(*p, 1, 1, 128, 128, f(0.1), 0, NULL) == 1
    assert lib.fa_bwd_noalloc(*([NULL] * 9), 1, 1, 0, 128, f(0.1), 0, NULL) == 0
    assert "scratch" in lib.fa_status_string(4).decode()
