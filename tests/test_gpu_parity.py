"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle, at
sizes the oracle finishes in seconds: several tiles, ragged token and
vocabulary tails, multi-chunk backward, both payload paths, full-row mode.

Bars: per-token |dL| <= 1e-4 + 1e-3|L|; gradients max|d| <= 2e-3 max|ref|;
compaction, gather and scatter bit-exact; exact zeros where the method gives
exact zeros (unmasked rows, self-distillation).
"""
import copy

import numpy as np
import pytest

import lm_head_reverse_amd as R
import synth
from gpu_util import bf16, f32, host, oracle_full, say, torch_dev, u8
from oracle import rkl_oracle as O
from tolerances import assert_grad_close, assert_loss_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tdev():
    torch, dev = torch_dev()
    R.lib()
    return torch, dev


# ------------------------------------------------------------------ compaction

def _masks():
    rng = np.random.default_rng(0)
    yield "empty", np.zeros(0, np.uint8)
    yield "one_on", np.ones(1, np.uint8)
    yield "one_off", np.zeros(1, np.uint8)
    yield "bern0.3_T1000", (rng.random(1000) < 0.3).astype(np.uint8)
    yield "all_T2049", np.ones(2049, np.uint8)
    yield "none_T5000", np.zeros(5000, np.uint8)
    m = np.zeros((2, 16384), np.uint8)
    m[:, -2048:] = 1
    yield "last2048_T32768", m.reshape(-1)
    yield "bytes_T3001", rng.integers(0, 3, 3001).astype(np.uint8) * 77


@pytest.mark.parametrize("name,mask", list(_masks()), ids=[n for n, _ in _masks()])
def test_compact_rows_bitexact(tdev, name, mask):
    torch, dev = tdev
    say("compact", name, mask.shape)
    idx, n = R.compact_rows(u8(mask, dev))
    want = O.compact_rows(mask)
    assert n == want.shape[0]
    assert np.array_equal(host(idx), want)


def test_gather_scatter_bitexact(tdev):
    torch, dev = tdev
    rng = np.random.default_rng(1)
    T = 777
    mask = (rng.random(T) < 0.4).astype(np.uint8)
    idx_np = O.compact_rows(mask)
    idx = torch.from_numpy(idx_np).to(dev)
    for shape, kind in (((T, 192), "bf16"), ((T,), "f32"), ((T, 3), "f32"), ((T, 2048), "bf16")):
        say("gather/scatter", shape, kind)
        if kind == "bf16":
            bits = rng.integers(0, 65536, size=shape, dtype=np.uint16)
            src = bf16(bits, dev)
            ref = bits
        else:
            ref = rng.standard_normal(shape).astype(np.float32)
            src = f32(ref, dev)
        g = R.gather_rows(src, idx)
        gh = host(g.view(torch.int16)).view(np.uint16) if kind == "bf16" else host(g)
        assert np.array_equal(gh.view(np.uint8), O.gather_rows(ref, idx_np).view(np.uint8))
        back = R.scatter_rows(g, idx, T)
        bh = host(back.view(torch.int16)).view(np.uint16) if kind == "bf16" else host(back)
        assert np.array_equal(bh.view(np.uint8), O.scatter_rows(O.gather_rows(ref, idx_np), idx_np, T).view(np.uint8))


# ------------------------------------------------------------------ logits path (both sides as logits)

def test_logits_both_sides_tiny(tdev):
    """64 positions, V = 1024, N(0, 2^2) logits, Bernoulli(0.7) mask."""
    torch, dev = tdev
    case = synth.config("c1")
    T, V = case.T, case.V
    say("c1 logits tiny", T, V)
    mask = u8(case.mask, dev)
    zs_all, zt_all = f32(case.z_s, dev), f32(case.z_t, dev)
    idx, N = R.compact_rows(mask)
    zs, zt = R.gather_rows(zs_all, idx), R.gather_rows(zt_all, idx)
    loss, stats = R.forward_logits(zt, z_s=zs)
    dz = R.backward_logits(zt, stats, z_s=zs)
    loss_pos = host(R.scatter_rows(loss, idx, T))
    torch.cuda.synchronize()

    rows = O.compact_rows(case.mask)
    inp, (L, ls, lt), b = oracle_full(case, rows, want_dz=True)
    assert_loss_close(loss_pos[rows], L)
    assert np.all(loss_pos[case.mask == 0] == 0.0)
    assert_loss_close(host(stats)[:, 0], ls, "lse_s")
    assert_loss_close(host(stats)[:, 1], lt, "lse_t")
    assert_grad_close(host(dz), b["dz"], "dz")

    # full-row mode over all T positions: unmasked rows exactly zero, masked rows identical
    say("c1 full-row")
    loss_f, stats_f = R.forward_logits(zt_all, z_s=zs_all, row_mask=mask)
    dz_f = R.backward_logits(zt_all, stats_f, z_s=zs_all, row_mask=mask)
    lf, dzf = host(loss_f), host(dz_f)
    assert np.array_equal(lf[rows], host(loss))
    assert np.all(lf[case.mask == 0] == 0.0)
    assert np.array_equal(dzf[rows], host(dz))
    assert np.all(dzf[case.mask == 0] == 0.0)


# ------------------------------------------------------------------ hidden-state path

def _run_hidden(case, dev, g=None, teacher_logits=False, full_row=False):
    """Compaction -> gather -> forward -> backward through the binding."""
    torch = __import__("torch")
    mask = u8(case.mask, dev)
    idx, N = R.compact_rows(mask)
    if full_row:
        idx = torch.arange(case.T, dtype=torch.int32, device=dev)
        N = case.T
    hs = R.gather_rows(bf16(case.h_s, dev), idx)
    Ws = bf16(case.W_s, dev)
    gg = None if g is None else R.gather_rows(f32(g, dev), idx)
    rm = mask if full_row else None
    if teacher_logits:
        zt = R.gather_rows(f32(case.z_t, dev), idx)
        loss, stats = R.forward_logits(zt, h_s=hs, W_s=Ws, row_mask=rm)
        dh, dW = R.backward_logits(zt, stats, h_s=hs, W_s=Ws, grad_loss=gg, row_mask=rm)
    else:
        ht = R.gather_rows(bf16(case.h_t, dev), idx)
        Wt = bf16(case.W_t, dev)
        loss, stats = R.forward_hidden(hs, Ws, ht, Wt, row_mask=rm)
        dh, dW = R.backward_hidden(hs, Ws, ht, Wt, stats, grad_loss=gg, row_mask=rm)
    torch.cuda.synchronize()
    return host(idx), host(loss), host(stats), host(dh), host(dW)


def _check_against_oracle(case, out, g=None):
    idx, loss, stats, dh, dW = out
    rows = O.compact_rows(case.mask)
    assert np.array_equal(idx, rows)
    gr = None if g is None else g[rows]
    inp, (L, ls, lt), b = oracle_full(case, rows, gr)
    assert_loss_close(loss, L)
    assert_loss_close(stats[:, 2], L, "stats L")
    assert_loss_close(stats[:, 0], ls, "lse_s")
    if case.h_t is not None:
        assert_loss_close(stats[:, 1], lt, "lse_t")
    assert_grad_close(dh, b["dh"], "dh")
    assert_grad_close(dW, b["dW"], "dW")


def _random_shapes(n=12, seed=2024):
    """Seeded random shapes: T in [1, 700], V in [1, 6000] (tails of every
    size, including V < one 256-row tile), widths multiples of 64 up to 512,
    mask densities from 0.05 to 1."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        T = int(rng.integers(1, 701))
        V = int(rng.choice([int(rng.integers(1, 257)), int(rng.integers(257, 6001))]))
        Hs, Ht = (64 * int(rng.integers(1, 9)) for _ in range(2))
        p = float(rng.choice([0.05, 0.3, 0.7, 1.0]))
        out.append((i, T, V, Hs, Ht, p))
    return out


@pytest.mark.parametrize("i,T,V,Hs,Ht,p", _random_shapes())
def test_random_shapes_both_payloads(tdev, i, T, V, Hs, Ht, p):
    """Seeded random shapes through both payloads (the teacher as hidden
    states, and as the fp32 rounding of its logits) against the oracle."""
    torch, dev = tdev
    case = synth.random_case(5000 + i, T=T, V=V, Hs=Hs, Ht=Ht, p_mask=p, with_grad=True)
    if int(case.mask.sum()) == 0:
        case.mask[T // 2] = 1
    say("random shape", i, T, V, Hs, Ht, p)
    _check_against_oracle(case, _run_hidden(case, dev, g=case.grad), g=case.grad)
    lg = copy.copy(case)
    lg.z_t = O.project_f32(case.h_t, case.W_t)
    lg.h_t = lg.W_t = None
    say("random shape, teacher logits", i)
    idx, loss, stats, dh, dW = _run_hidden(lg, dev, g=lg.grad, teacher_logits=True)
    rows = O.compact_rows(lg.mask)
    inp, (L, ls, lt), b = oracle_full(lg, rows, lg.grad[rows])
    assert_loss_close(loss, L, "loss (teacher logits)")
    assert_grad_close(dh, b["dh"], "dh (teacher logits)")
    assert_grad_close(dW, b["dW"], "dW (teacher logits)")


def test_hidden_small(tdev):
    """B=2, S=129, Hs=Ht=256, V=8192, response spans from random offsets."""
    torch, dev = tdev
    case = synth.config("c2")
    say("c2 hidden small", case.T, case.V, case.Hs)
    _check_against_oracle(case, _run_hidden(case, dev))


@pytest.mark.parametrize("T,V,Hs,Ht", [(300, 1000, 128, 192), (129, 257, 64, 64), (517, 2053, 192, 128)])
def test_hidden_ragged_with_grad(tdev, T, V, Hs, Ht):
    """Ragged N and V tails, unequal widths, an upstream per-token gradient."""
    torch, dev = tdev
    case = synth.random_case(10 + T, T=T, V=V, Hs=Hs, Ht=Ht, p_mask=0.5, with_grad=True)
    say("ragged hidden", T, V, Hs, Ht)
    _check_against_oracle(case, _run_hidden(case, dev, g=case.grad), g=case.grad)


def test_hidden_multi_chunk_backward(tdev, monkeypatch):
    """V = 140000 spans three 65536-column dh segments (the last one ragged):
    one backward chunk by default at this N, three chunks of 65536 columns
    when the chunk width is forced.  Both match the oracle, and bit for bit
    each other: dh's sum is split at the same segment boundaries either way
    (the chunk plan depends on N, the result must not)."""
    torch, dev = tdev
    case = synth.random_case(31, T=150, V=140000, Hs=64, Ht=64, p_mask=0.6, with_grad=True)
    say("multi-chunk", case.T, case.V)
    one = _run_hidden(case, dev, g=case.grad)
    _check_against_oracle(case, one, g=case.grad)
    monkeypatch.setenv("RKL_VOCAB_CHUNK", "65536")
    three = _run_hidden(case, dev, g=case.grad)
    for a, b, what in zip(three[1:], one[1:], ("loss", "stats", "dh", "dW")):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), what


@pytest.mark.parametrize("orders", [("1,1", "1,1", "1", "1", "1"), ("3,5", "7,2", "3", "3", "2"),
                                    ("64,64", "2,3", "64", "64", "1000")],
                         ids=["one_by_one", "ragged_panels", "oversized"])
def test_tile_order_and_grouping_do_not_change_results(tdev, monkeypatch, orders):
    """The workgroup orders (the fused kernels' panel sizes GS x TG, the dh
    GEMM's column tiles per panel), the vocabulary tiles per backward
    workgroup and the forward splits per workgroup only reorder independent
    work: results are bitwise those of the default settings, for ragged token
    and vocabulary tails (Hs = 640: five dh column tiles, so panels of 3
    leave a ragged last panel; 20 forward splits, so groups of 2 and of all
    of them)."""
    torch, dev = tdev
    case = synth.random_case(77, T=700, V=5003, Hs=640, Ht=192, p_mask=0.8, with_grad=True)
    say("orders", orders, case.T, case.V)
    ref = _run_hidden(case, dev, g=case.grad)
    fo, bo, bt, dp, sp = orders
    monkeypatch.setenv("RKL_FWD_ORDER", fo)
    monkeypatch.setenv("RKL_BWD_ORDER", bo)
    monkeypatch.setenv("RKL_BWD_TILES", bt)
    monkeypatch.setenv("RKL_DH_PANEL", dp)
    monkeypatch.setenv("RKL_FWD_SPLITS_PER_WG", sp)
    got = _run_hidden(case, dev, g=case.grad)
    for a, b, what in zip(got[1:], ref[1:], ("loss", "stats", "dh", "dW")):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), what


@pytest.mark.parametrize("tiles", [1, 5, 40])
def test_forward_split_sizes(tdev, monkeypatch, tiles):
    """Vocabulary tiles per forward split (1: one split per 256-row tile; 5: a
    ragged last split; 40: one split over the whole vocabulary): the split
    plan changes only the order of the log-sum-exp merges, so every setting
    matches the oracle."""
    torch, dev = tdev
    monkeypatch.setenv("RKL_FWD_TILES", str(tiles))
    case = synth.random_case(79, T=300, V=9001, Hs=128, Ht=192, p_mask=0.7, with_grad=True)
    say("forward split", tiles, case.T, case.V)
    _check_against_oracle(case, _run_hidden(case, dev, g=case.grad), g=case.grad)


@pytest.mark.parametrize("chunk", [256, 768])
def test_narrow_backward_chunks(tdev, monkeypatch, chunk):
    """Backward vocabulary chunks of 256 and 768 columns over V = 3001: many
    chunks, the last ragged and past V (the clamped dh variant)."""
    torch, dev = tdev
    monkeypatch.setenv("RKL_VOCAB_CHUNK", str(chunk))
    case = synth.random_case(78, T=300, V=3001, Hs=128, Ht=64, p_mask=0.6, with_grad=True)
    say("chunk", chunk, case.T, case.V)
    _check_against_oracle(case, _run_hidden(case, dev, g=case.grad), g=case.grad)


@pytest.mark.parametrize("V", [3000, 1001])
def test_student_hidden_teacher_logits(tdev, V):
    """Teacher logits payload with the student projected; V = 1001 takes the unvectorised z_t reads."""
    torch, dev = tdev
    case = synth.random_case(40 + V, T=200, V=V, Hs=128, Ht=0, teacher_logits=True, p_mask=0.7, with_grad=True)
    say("teacher logits", case.T, V)
    _check_against_oracle(case, _run_hidden(case, dev, g=case.grad, teacher_logits=True), g=case.grad)


@pytest.mark.parametrize("V", [3000, 1001])
def test_logits_read_through_row_index(tdev, V):
    """z_rows: reading the logits rows through an index gives, bit for bit,
    the results of the same rows gathered first -- for the compacted rows, a
    shuffled order with repeats, and indices outside [0, T) (read as the
    clamped row) -- with the student as hidden states (the tiled kernels;
    V = 1001 takes the unvectorised z_t reads) and as logits (row kernels).
    Several 128-token tiles with a ragged last one (N = 300 of T = 400)."""
    torch, dev = tdev
    T = 400
    case = synth.random_case(70 + V, T=T, V=V, Hs=128, Ht=0, teacher_logits=True, p_mask=0.7, with_grad=True)
    zs_case = synth.random_case(80 + V, T=T, V=V, Hs=0, Ht=0, student_logits=True, teacher_logits=True)
    rng = np.random.default_rng(V)
    idx_c = O.compact_rows(case.mask).astype(np.int32)
    idx_s = rng.integers(0, T, size=300).astype(np.int32)
    idx_o = idx_s.copy()
    idx_o[::7] = T + 5
    idx_o[3::11] = -2
    zt_all = f32(case.z_t, dev)
    Ws = bf16(case.W_s, dev)
    zs_all, zt2_all = f32(zs_case.z_s, dev), f32(zs_case.z_t, dev)
    for name, idx in (("compacted", idx_c), ("shuffled", idx_s), ("out of range", idx_o)):
        say("logits through z_rows", name, V, idx.shape[0])
        clamped = np.clip(idx, 0, T - 1).astype(np.int32)
        rows = torch.from_numpy(idx).to(dev)
        crow = torch.from_numpy(clamped).to(dev)
        hs = R.gather_rows(bf16(case.h_s, dev), crow)
        g = R.gather_rows(f32(case.grad, dev), crow)
        # student projected
        zt = R.gather_rows(zt_all, crow)
        ref = R.forward_logits(zt, h_s=hs, W_s=Ws)
        ref_b = R.backward_logits(zt, ref[1], h_s=hs, W_s=Ws, grad_loss=g)
        got = R.forward_logits(zt_all, h_s=hs, W_s=Ws, z_rows=rows)
        got_b = R.backward_logits(zt_all, got[1], h_s=hs, W_s=Ws, grad_loss=g, z_rows=rows)
        for a, b, what in zip(got + got_b, ref + ref_b, ("loss", "stats", "dh", "dW")):
            assert np.array_equal(host(a).view(np.uint32), host(b).view(np.uint32)), (name, what)
        # student as logits
        zs, zt2 = R.gather_rows(zs_all, crow), R.gather_rows(zt2_all, crow)
        ref = R.forward_logits(zt2, z_s=zs)
        ref_dz = R.backward_logits(zt2, ref[1], z_s=zs, grad_loss=g)
        got = R.forward_logits(zt2_all, z_s=zs_all, z_rows=rows)
        got_dz = R.backward_logits(zt2_all, got[1], z_s=zs_all, grad_loss=g, z_rows=rows)
        for a, b, what in zip(got + (got_dz,), ref + (ref_dz,), ("loss", "stats", "dz")):
            assert np.array_equal(host(a).view(np.uint32), host(b).view(np.uint32)), (name, what)


def test_logits_payload_equals_hidden_payload(tdev):
    """Teacher logits = fp32 rounding of h_t W_t^T: both payload paths agree."""
    torch, dev = tdev
    case = synth.random_case(50, T=160, V=4000, Hs=128, Ht=128, p_mask=0.8)
    say("logits == hidden", case.T, case.V)
    hid = _run_hidden(case, dev)
    case.z_t = O.project_f32(case.h_t, case.W_t)
    lg = _run_hidden(case, dev, teacher_logits=True)
    assert_loss_close(lg[1], hid[1], "loss logits vs hidden")
    assert_grad_close(lg[3], hid[3], "dh logits vs hidden")
    assert_grad_close(lg[4], hid[4], "dW logits vs hidden")


def test_full_row_equals_compact(tdev):
    """Full-row mode (all T rows projected, mask applied in the epilogues) gives
    bit-identical loss and dh on masked rows, exact zeros elsewhere."""
    torch, dev = tdev
    case = synth.config("c2")
    say("full-row vs compact", case.T)
    c = _run_hidden(case, dev)
    f = _run_hidden(case, dev, full_row=True)
    rows = c[0]
    m = case.mask != 0
    assert np.array_equal(f[1][rows], c[1])
    assert np.all(f[1][~m] == 0.0)
    assert np.array_equal(f[2][rows], c[2])
    assert np.array_equal(f[3][rows], c[3])
    assert np.all(f[3][~m] == 0.0)
    assert_grad_close(f[4], c[4], "dW full-row vs compact")


@pytest.mark.parametrize("T,V,Hs,chunk", [(700, 5003, 640, None), (300, 40000, 128, None), (260, 5003, 256, "768"),
                                           (129, 16385, 192, "16384")])
def test_dh_split_by_segment_is_bitwise_the_same(tdev, monkeypatch, T, V, Hs, chunk):
    """The dh GEMM split into one workgroup per (tile, vocabulary segment)
    plus an in-order reduce gives dh (and everything else) bit for bit as the
    one-workgroup-per-tile GEMM: one and several segments per chunk, chunks
    that do not start on a segment boundary (768 columns), a segment of one
    column past 16384, several accumulated chunks."""
    torch, dev = tdev
    case = synth.random_case(300 + T, T=T, V=V, Hs=Hs, Ht=64, p_mask=0.8, with_grad=True)
    if chunk:
        monkeypatch.setenv("RKL_VOCAB_CHUNK", chunk)
    say("dh split by segment", T, V, Hs, chunk)
    monkeypatch.setenv("RKL_DH_SPLIT", "0")
    ref = _run_hidden(case, dev, g=case.grad)
    monkeypatch.setenv("RKL_DH_SPLIT", "1")
    got = _run_hidden(case, dev, g=case.grad)
    for a, b, what in zip(got[1:], ref[1:], ("loss", "stats", "dh", "dW")):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), what
    if not chunk:
        _check_against_oracle(case, got, g=case.grad)


@pytest.mark.parametrize("T,V,Hs", [(500, 5003, 192), (1400, 3001, 512), (129, 1000, 64)])
def test_late_w_copy_is_bitwise_the_same(tdev, monkeypatch, T, V, Hs):
    """The dz kernel's fp16 copy of W_s made after the stream from the k-tile
    loaded again (the default when a workgroup converts at most one k-tile)
    gives dh, dW (and everything else) bit for bit as the copy made from the
    stream's own stage; ragged vocabulary tails and widths included."""
    torch, dev = tdev
    case = synth.random_case(600 + T, T=T, V=V, Hs=Hs, Ht=Hs, p_mask=0.8, with_grad=True)
    say("late W copy", T, V, Hs)
    monkeypatch.setenv("RKL_LATE_W16", "0")
    ref = _run_hidden(case, dev, g=case.grad)
    monkeypatch.setenv("RKL_LATE_W16", "1")
    got = _run_hidden(case, dev, g=case.grad)
    for a, b, what in zip(got[1:], ref[1:], ("loss", "stats", "dh", "dW")):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), what


@pytest.mark.parametrize("splits_per_wg", [None, "2", "1000"])
def test_self_distillation_is_exactly_zero(tdev, monkeypatch, splits_per_wg):
    """Bit-identical teacher: every loss and gradient entry is exactly zero,
    also when a forward workgroup folds and merges several vocabulary splits
    in turn (V = 3000: four splits)."""
    torch, dev = tdev
    case = synth.random_case(60, T=100, V=3000, Hs=128, Ht=128, p_mask=0.9)
    case.h_t, case.W_t = case.h_s, case.W_s
    if splits_per_wg:
        monkeypatch.setenv("RKL_FWD_SPLITS_PER_WG", splits_per_wg)
    say("self-distillation small, forward splits per workgroup", splits_per_wg)
    idx, loss, stats, dh, dW = _run_hidden(case, dev)
    assert np.all(loss == 0.0)
    assert np.all(dh == 0.0) and np.all(dW == 0.0)


def test_bitwise_deterministic(tdev):
    torch, dev = tdev
    case = synth.random_case(70, T=300, V=5000, Hs=128, Ht=64, p_mask=0.5)
    say("determinism")
    a = _run_hidden(case, dev)
    b = _run_hidden(case, dev)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_empty_mask(tdev):
    torch, dev = tdev
    case = synth.random_case(80, T=40, V=600, Hs=64, Ht=64, p_mask=0.0)
    say("empty mask")
    mask = u8(case.mask, dev)
    idx, N = R.compact_rows(mask)
    assert N == 0
    hs = R.gather_rows(bf16(case.h_s, dev), idx)
    ht = R.gather_rows(bf16(case.h_t, dev), idx)
    Ws, Wt = bf16(case.W_s, dev), bf16(case.W_t, dev)
    loss, stats = R.forward_hidden(hs, Ws, ht, Wt)
    assert loss.shape == (0,)
    assert np.all(host(R.scatter_rows(loss, idx, case.T)) == 0.0)
    dh, dW = R.backward_hidden(hs, Ws, ht, Wt, stats)
    assert dh.shape == (0, 64) and np.all(host(dW) == 0.0)
    prev = torch.full((600, 64), 3.5, device=dev)
    _, dW2 = R.backward_hidden(hs, Ws, ht, Wt, stats, dW=prev, accumulate_dW=True)
    assert np.all(host(dW2) == 3.5)


def test_accumulate_dW(tdev):
    torch, dev = tdev
    case = synth.random_case(90, T=120, V=1500, Hs=128, Ht=128, p_mask=0.6)
    say("accumulate dW")
    mask = u8(case.mask, dev)
    idx, N = R.compact_rows(mask)
    hs = R.gather_rows(bf16(case.h_s, dev), idx)
    ht = R.gather_rows(bf16(case.h_t, dev), idx)
    Ws, Wt = bf16(case.W_s, dev), bf16(case.W_t, dev)
    loss, stats = R.forward_hidden(hs, Ws, ht, Wt)
    _, dW = R.backward_hidden(hs, Ws, ht, Wt, stats)
    base = np.random.default_rng(3).standard_normal((1500, 128)).astype(np.float32)
    _, dW2 = R.backward_hidden(hs, Ws, ht, Wt, stats, dW=f32(base, dev), accumulate_dW=True)
    assert np.array_equal(host(dW2), base + host(dW))


@pytest.mark.parametrize("T,V", [(1, 1), (3, 1), (2, 2), (5, 63), (1, 300)])
def test_tiny_vocabulary_and_single_rows(tdev, T, V):
    """Vocabularies far below one 256-row tile (down to V = 1) and batches of
    one row: clamped rows and padded columns everywhere.  With V = 1 both
    distributions are the point mass: L and every gradient are 0 in exact
    arithmetic (the oracle gives exact zeros), so the relative gradient bar
    does not apply; the GPU values must be zero up to fp32 rounding of the
    log-sum-exps (exp of the max entry is 1 only to within an ulp)."""
    torch, dev = tdev
    case = synth.random_case(200 + 10 * T + V, T=T, V=V, Hs=64, Ht=128, p_mask=1.0, with_grad=True)
    say("tiny vocabulary", T, V)
    out = _run_hidden(case, dev, g=case.grad)
    if V > 1:
        _check_against_oracle(case, out, g=case.grad)
        return
    idx, loss, stats, dh, dW = out
    assert np.array_equal(idx, np.arange(T))
    assert np.all(np.abs(loss) <= 1e-6)
    # z_s of the single entry: lse_s equals it up to rounding
    z_s = O.project(O.widen_bf16(case.h_s), O.widen_bf16(case.W_s))
    assert np.allclose(stats[:, 0], z_s[:, 0], rtol=1e-5, atol=1e-5)
    assert np.max(np.abs(dh)) <= 1e-6 and np.max(np.abs(dW)) <= 1e-6


def test_token_mean_gradient_large_vocab(tdev):
    """Upstream gradient 1/N with V = 60000: dz values around g/V must keep
    their precision in the scaled fp16 workspace."""
    torch, dev = tdev
    case = synth.random_case(95, T=400, V=60000, Hs=128, Ht=64, p_mask=0.75)
    rows = O.compact_rows(case.mask)
    case.grad = np.full(case.T, 1.0 / rows.shape[0], np.float32)
    say("token-mean gradient, V=60000")
    _check_against_oracle(case, _run_hidden(case, dev, g=case.grad), g=case.grad)
