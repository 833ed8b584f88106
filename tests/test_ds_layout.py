"""Model of the stored-dS layout, on the CPU.

With the stored-dS backward the dK/dV kernel writes its bf16 dS tiles to the
workspace and the dQ kernel gathers them into LDS and reads them back with
transposing LDS reads.  This model replays both kernels' index arithmetic
(as written in csrc/fa_bwd.hip) on byte arrays:
  * tile indices: every (head, 256-key block, 64-query iteration) the mask
    keeps gets one tile, each written exactly once, all inside the buffer
    whose size the library reports, and the dQ kernel reads only tiles the
    dK/dV kernel wrote (ragged S, causal and not);
  * data movement: values dS[key][query] stored from the dK/dV kernel's
    accumulator layout, copied by the dQ kernel's 16-byte gathers into its
    swizzled LDS rows, and read by ds_read_b64_tr_b16 (the semantics stated
    in fa_common.h) arrive in every lane's MFMA B operand as
    dS[key of k position p][query of the lane's column], for every wave,
    lane, k-step and key tile;
  * the transposing reads of a half wave touch 64 distinct LDS banks.
Planted mistakes (a wrong swizzle, a wrong unit order) are shown to fail.
"""
import numpy as np
import pytest

KB, QI = 256, 64  # keys per dK/dV block, queries per iteration


def tiles_per_head(nkb, nqi, causal):
    return nkb * nqi - 2 * nkb * (nkb - 1) if causal else nkb * nqi


def ds_tile(bh, kb, i, nkb, nqi, causal):
    head = bh * tiles_per_head(nkb, nqi, causal)
    if causal:
        return head + kb * nqi - 2 * kb * (kb - 1) + (i - 4 * kb)
    return head + kb * nqi + i


@pytest.mark.parametrize("S", [1, 63, 64, 65, 255, 256, 257, 300, 515, 1000, 4099])
@pytest.mark.parametrize("causal", [False, True])
def test_tiles_written_once_and_read_only_when_written(S, causal):
    BH = 3
    nkb, nqi = -(-S // KB), -(-S // QI)
    total = BH * tiles_per_head(nkb, nqi, causal)
    written = {}
    for bh in range(BH):
        for kb in range(nkb):
            for i in range(4 * kb if causal else 0, nqi):  # the dK/dV kernel's iterations
                t = ds_tile(bh, kb, i, nkb, nqi, causal)
                assert 0 <= t < total and t not in written
                written[t] = (bh, kb, i)
    assert len(written) == total
    for bh in range(BH):
        for qb in range(-(-S // 256)):  # the dQ kernel's 256-query blocks
            kv_end = min(S, qb * 256 + 256) if causal else S
            for kt in range(-(-kv_end // 64)):
                for k in range(4):
                    i = 4 * qb + k
                    if i < nqi:
                        assert written.get(ds_tile(bh, kt >> 2, i, nkb, nqi, causal)) == (bh, kt >> 2, i)


# ---------------------------------------------------------------- data movement of one tile
def store_tile(ds, unit_order=lambda qh, t, h: (2 * qh + t) * 2 + h):
    """The dK/dV kernel's stores of one 256-key x 64-query tile: wave w, lane
    (n, h), query half qh, k-step t write 8 bf16 (queries 16 t + 4 h + 0..3
    and 16 t + 8 + 4 h + 0..3 of the half, key 32 w + n) at byte
    ((2 qh + t) * 8 + w) * 1024 + lane * 16.  Values are integer codes
    key * 64 + query, one per 2-byte slot."""
    buf = np.full(32768 // 2, -1, dtype=np.int64)
    for w in range(8):
        for lane in range(64):
            n, h = lane & 31, lane >> 5
            for qh in range(2):
                for t in range(2):
                    u = unit_order(qh, t, h)
                    base = ((u >> 1) * 8 + w) * 1024 + ((u & 1) * 32 + n) * 16
                    for j in range(8):
                        g, e = 2 * t + (j >> 2), j & 3
                        q = 32 * qh + 8 * g + 4 * h + e
                        buf[base // 2 + j] = ds[32 * w + n, q]
    return buf


def gather_chunk(buf, kt, swz=lambda r: ((r >> 1) & 1) << 2):
    """The dQ kernel's copies of one 64-query chunk: LDS row r (key
    (kt % 4) * 64 + r), physical 16-byte chunk pc <- logical chunk
    pc ^ swz(r) = unit (2 qh + t) * 2 + h of that key."""
    lds = np.full((64, 64), -1, dtype=np.int64)  # [row][2-byte slot]
    for r in range(64):
        kk = (kt & 3) * 64 + r
        for pc in range(8):
            lc = pc ^ swz(r)
            src = (((lc >> 1) * 8 + (kk >> 5)) * 2 + (lc & 1)) * 512 + (kk & 31) * 16
            lds[r, pc * 8:(pc + 1) * 8] = buf[src // 2:src // 2 + 8]
    return lds


def b_operand(lds, qh, ks, swz=lambda r: ((r >> 1) & 1) << 2):
    """The B operand (dS^T, 8 keys x the lane's query) of k-step ks for every
    lane, through two ds_read_b64_tr_b16 per lane."""
    out = np.zeros((64, 8), dtype=np.int64)
    for s2 in range(2):
        w4 = {}
        for lane in range(64):  # addressing: 4 bf16 per lane
            h, tq, L = lane >> 5, (lane >> 4) & 1, lane & 15
            row = 16 * ks + 8 * h + 4 * s2 + (L >> 2)
            byte = ((((qh << 2) ^ swz(row)) >> 2) << 6) | (tq << 5) | ((L & 1) << 4) | (((L >> 1) & 1) << 3)
            w4[lane] = lds[row, byte // 2:byte // 2 + 4]
        for lane in range(64):  # delivery: lane i of a 16-lane group
            g0, i = lane & ~15, lane & 15
            for j in range(4):
                out[lane, 4 * s2 + j] = w4[g0 + (i >> 2) + 4 * j][i & 3]
    return out


def banks_of_half_wave(qh, ks, s2, half, swz=lambda r: ((r >> 1) & 1) << 2):
    banks = []
    for lane in range(32 * half, 32 * half + 32):
        h, tq, L = lane >> 5, (lane >> 4) & 1, lane & 15
        row = 16 * ks + 8 * h + 4 * s2 + (L >> 2)
        byte = ((((qh << 2) ^ swz(row)) >> 2) << 6) | (tq << 5) | ((L & 1) << 4) | (((L >> 1) & 1) << 3)
        addr = row * 128 + byte
        banks += [(addr // 4) % 64, (addr // 4 + 1) % 64]
    return banks


def check_tile(swz=None, unit_order=None):
    ds = np.arange(256)[:, None] * 64 + np.arange(64)[None, :]  # code key * 64 + query
    kw = {} if unit_order is None else {"unit_order": unit_order}
    buf = store_tile(ds, **kw)
    assert (buf >= 0).all(), "the stores must cover the tile"
    sw = {} if swz is None else {"swz": swz}
    for kt in range(4):
        lds = gather_chunk(buf, kt, **sw)
        for qh in range(2):
            for ks in range(4):
                b = b_operand(lds, qh, ks, **sw)
                for lane in range(64):
                    h = lane >> 5
                    keys = (kt & 3) * 64 + 16 * ks + 8 * h + np.arange(8)
                    want = keys * 64 + 32 * qh + (lane & 31)
                    if not np.array_equal(b[lane], want):
                        return False
    return True


def test_dq_operands_are_the_stored_ds():
    assert check_tile()


def test_transposing_reads_are_free_of_bank_conflicts():
    for qh in range(2):
        for ks in range(4):
            for s2 in range(2):
                for half in range(2):
                    assert len(set(banks_of_half_wave(qh, ks, s2, half))) == 64


def test_planted_mistakes_are_caught():
    # without the half swap the data still arrives (the reads apply the same
    # swizzle), but rows r and r + 2 of a half wave share banks
    assert len(set(banks_of_half_wave(0, 0, 0, 0, swz=lambda r: 0))) < 64
    # a swizzle applied on one side only scrambles the operand
    ds = np.arange(256)[:, None] * 64 + np.arange(64)[None, :]
    lds = gather_chunk(store_tile(ds), 0, swz=lambda r: 0)  # copied without the swap
    b = b_operand(lds, 0, 0)                               # read with it
    assert not np.array_equal(b[0], np.arange(8) * 64)
    # units stored in another order
    assert not check_tile(unit_order=lambda qh, t, h: (2 * qh + h) * 2 + t)
