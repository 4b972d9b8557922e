"""Chunked linear + cross-entropy (ce_linear_cross_entropy) on the GPU, through
the C ABI, against the FP64 oracle (oracle.linear_ce).

Inputs sit on a grid (h = k/8, |k| <= 4; W = m/64, |m| <= 8) so that every
partial sum of h W^T is a multiple of 2^-9 below 2^17 and thus exact in FP32
whatever the GEMM's summation order: the library's logits then equal the
oracle's (FP32, then BF16 by nearest even) bit for bit, and the stated
cross-entropy bar applies to the loss.  The logits have a standard deviation
of about 0.08 sqrt(D).

Every test runs under each GEMM choice: "native" (the library's MFMA
kernel, ce_gemm.hip, for BF16 heads whose rows are 16-byte multiples),
"library" (hipBLASLt) and "auto" (the default: the native kernel for dh and
dW, the library for the logits); the plan query confirms which products ran
natively.  Both engines accumulate in FP32, so the same bars hold for all.

Gradient bars, derived from the cross-entropy bar (the library's G differs
from the exact G by at most r_G |G| + a_G per element: 2^-8 and 1e-7 for
BF16, 1e-5 and 1e-8 for FP32) and from FP32 accumulation over K terms
(gamma_K = K 2^-24):
  dh_id: (r_G + gamma_V) sum_j |G_ij||W_jd| + a_G sum_j |W_jd|, plus the output
         rounding rho |ref| (rho = 2^-8 for BF16, 2^-23 for FP32);
  dW_jd: (r_G + gamma_N) sum_i |G_ij||h_id| + a_G sum_i |h_id| + 2^-23 |ref|.
"""
import math

import numpy as np
import pytest
import torch

import vocab_cross_entropy_amd as vce
from gpu_util import GRAD_TOL, assert_loss, orc, say

pytestmark = pytest.mark.gpu

ENGINES = ["native", "library", "auto"]


def expected_plan(h, w, gemm):
    """The products the native kernel takes: all three for BF16 with 16-byte rows under "native", dh and dW
    under "auto"."""
    D = h.shape[1]
    ok = (h.dtype == torch.bfloat16 and D % 8 == 0 and max(h.stride(0), D) % 8 == 0 and w.stride(0) % 8 == 0
          and h.data_ptr() % 16 == 0 and w.data_ptr() % 16 == 0)
    return 0 if not ok else {"native": 7, "auto": 6}.get(gemm, 0)


def grid_inputs(N, D, V, dtype, seed, ignore_frac=0.2):
    g = torch.Generator().manual_seed(seed)
    h = (torch.randint(-4, 5, (N, D), generator=g).double() / 8).to(dtype)
    w = (torch.randint(-8, 9, (V, D), generator=g).double() / 64).to(dtype)
    t = torch.randint(0, V, (N,), generator=g)
    k = int(round(ignore_frac * N))
    if k:
        t[torch.randperm(N, generator=g)[:k]] = -100
    return h, w, t


def _bars(dtype):
    r_g, a_g = GRAD_TOL[dtype]
    return r_g, a_g, (2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -23)


def check_dh(got, ref, G, w, dtype, what):
    r_g, a_g, rho = _bars(dtype)
    V = w.shape[0]
    W = np.abs(w.double().numpy())
    A = np.abs(G) @ W
    B = np.broadcast_to(W.sum(axis=0), ref.shape)
    tol = (r_g + V * 2.0 ** -24) * A + a_g * B
    tol = tol + rho * (np.abs(ref) + tol)
    err = np.abs(got - ref)
    bad = ~(err <= tol)
    assert not bad.any(), f"{what}: dh off at {bad.sum()} elements, max err {err.max():.3e}, max tol {tol.max():.3e}"


def check_dw(got, ref, G, h, dtype, what, out_rho=2.0 ** -23):
    """``out_rho``: the output's own rounding (FP32 accumulator; 2^-8 once cast to BF16)."""
    r_g, a_g, _ = _bars(dtype)
    N = h.shape[0]
    H = np.abs(h.double().numpy())
    A = np.abs(G).T @ H
    B = np.broadcast_to(H.sum(axis=0), ref.shape)
    tol = (r_g + N * 2.0 ** -24) * A + a_g * B
    tol = tol + out_rho * (np.abs(ref) + tol)
    err = np.abs(got - ref)
    bad = ~(err <= tol)
    assert not bad.any(), f"{what}: dW off at {bad.sum()} elements, max err {err.max():.3e}"


def run_linear(h, w, t, alpha, reduce, g=None, chunk_rows=0, smoothing="all", want_dh=True, want_dw=True,
               dw0=None, h_pad=0, gemm="auto"):
    """Device copies (h optionally inside a wider buffer: row stride D + h_pad), the call, results on the host."""
    N, D = h.shape
    hd_full = torch.zeros((N, D + h_pad), dtype=h.dtype)
    hd_full[:, :D] = h
    hd = hd_full.cuda()[:, :D]
    wd, td = w.cuda(), t.cuda()
    if g is None:
        gd = None
    elif reduce in ("none", False):
        gd = torch.as_tensor(np.asarray(g, dtype=np.float32)).cuda()
    else:
        gd = torch.tensor([float(g)], dtype=torch.float32, device="cuda")
    dw = None
    if dw0 is not None:
        dw = torch.as_tensor(dw0, dtype=torch.float32).cuda()
    assert vce.ce_linear_gemm_plan(hd, wd, gemm) == expected_plan(hd, wd, gemm)
    loss, dh, dwo, n = vce.ce_linear_cross_entropy(hd, wd, td, alpha, reduce, grad_out=gd, chunk_rows=chunk_rows,
                                                   smoothing=smoothing, want_dh=want_dh, want_dw=want_dw, dw=dw,
                                                   accumulate_dw=dw0 is not None, gemm=gemm)
    torch.cuda.synchronize()
    return (loss.cpu().double().numpy(), None if dh is None else dh.cpu().double().numpy(),
            None if dwo is None else dwo.cpu().double().numpy(), int(n.item()))


def check_linear(h, w, t, alpha, reduce, g=None, chunk_rows=0, smoothing="all", what="", **kw):
    N, D = h.shape
    V = w.shape[0]
    say(f"[linear] {what} N={N} D={D} V={V} {h.dtype} a={alpha} {reduce} {smoothing} chunk={chunk_rows} "
        f"gemm={kw.get('gemm', 'auto')}")
    loss, dh, dw, n = run_linear(h, w, t, alpha, reduce, g, chunk_rows, smoothing, **kw)
    o = orc()
    n_ref = int((t != -100).sum())
    assert n == n_ref
    g_or = None if g is None else (float(g) if reduce not in ("none", False) else np.asarray(g, np.float64))
    ref_rows, ref_dh, ref_dw, G = o.linear_ce(h, w, t, alpha, reduce_loss=reduce, g=g_or, smoothing=smoothing,
                                              want_g=True)
    if reduce in ("none", False):
        assert_loss(loss, ref_rows, f"{what} loss rows")
        ign = t.numpy() == -100
        assert np.all(loss[ign] == 0.0)
    else:
        ref = o.reduce(ref_rows, reduce, n_ref)
        if reduce in ("mean", True) and n_ref == 0:
            assert math.isnan(loss[0]) and math.isnan(ref)
        else:
            assert_loss([loss[0]], [ref], f"{what} {reduce}")
    if dh is not None:
        check_dh(dh, ref_dh, G, w, h.dtype, what)
        ign = t.numpy() == -100
        assert np.all(dh[ign] == 0.0), "ignored rows' dh must be 0"
    if dw is not None:
        dw0 = kw.get("dw0")
        check_dw(dw - (0.0 if dw0 is None else np.asarray(dw0, np.float64)), ref_dw, G, h, h.dtype, what)
    return loss, dh, dw


CASES = [(dt, red, sm) for dt in (torch.bfloat16, torch.float32) for red in ("none", "mean", "sum")
         for sm in ("all", "others")]


@pytest.mark.parametrize("gemm", ENGINES)
@pytest.mark.parametrize("dtype,reduce,smoothing", CASES,
                         ids=[f"{'bf16' if c[0] == torch.bfloat16 else 'f32'}-{c[1]}-{c[2]}" for c in CASES])
def test_linear_chunks_of_32(dtype, reduce, smoothing, gemm):
    """100 rows in chunks of 32, 32, 32 and 4; V = 4099 (ragged rows; the
    native dh product's K tail), D = 96 (the logits product's K tail)."""
    h, w, t = grid_inputs(100, 96, 4099, dtype, seed=5)
    g = np.linspace(-1.0, 2.0, 100) if reduce == "none" else 0.8
    check_linear(h, w, t, 0.1, reduce, g=g, chunk_rows=32, smoothing=smoothing, what="chunks of 32", gemm=gemm)


@pytest.mark.parametrize("gemm", ENGINES)
@pytest.mark.parametrize("chunk_rows", [0, 1, 7, 64, 100, 1000])
def test_linear_chunk_sizes(chunk_rows, gemm):
    """One chunk, one row per chunk, ragged chunks, more rows per chunk than rows."""
    h, w, t = grid_inputs(64, 64, 3001, torch.bfloat16, seed=11)
    check_linear(h, w, t, 0.1, "mean", chunk_rows=chunk_rows, what=f"chunk {chunk_rows}", gemm=gemm)


@pytest.mark.parametrize("gemm", ENGINES)
def test_linear_partial_outputs_and_accumulation(gemm):
    """dh only, dW only, dW added to an existing gradient, and a strided h."""
    h, w, t = grid_inputs(40, 64, 2048, torch.bfloat16, seed=13)
    check_linear(h, w, t, 0.0, "sum", chunk_rows=16, want_dw=False, what="dh only", gemm=gemm)
    check_linear(h, w, t, 0.0, "sum", chunk_rows=16, want_dh=False, what="dW only", gemm=gemm)
    rng = np.random.default_rng(3)
    dw0 = rng.standard_normal((2048, 64)).astype(np.float32)
    check_linear(h, w, t, 0.0, "sum", chunk_rows=16, dw0=dw0, what="dW accumulated", gemm=gemm)
    check_linear(h, w, t, 0.1, "mean", chunk_rows=16, h_pad=24, what="strided h", gemm=gemm)


@pytest.mark.parametrize("gemm", ENGINES)
def test_linear_short_rows_and_small_heads(gemm):
    """V = 7 (the fused kernel's FP64 path for short rows), D = 1, all rows of a chunk ignored."""
    h, w, t = grid_inputs(20, 8, 7, torch.float32, seed=17)
    check_linear(h, w, t, 0.3, "mean", chunk_rows=8, smoothing="others", what="V=7", gemm=gemm)
    h, w, t = grid_inputs(12, 1, 500, torch.bfloat16, seed=19)
    check_linear(h, w, t, 0.1, "none", g=np.ones(12), chunk_rows=5, what="D=1", gemm=gemm)
    h, w, t = grid_inputs(12, 32, 500, torch.bfloat16, seed=23, ignore_frac=0.0)
    t[4:8] = -100
    check_linear(h, w, t, 0.1, "mean", chunk_rows=4, what="an all-ignored chunk", gemm=gemm)
    h, w, t = grid_inputs(20, 8, 13, torch.bfloat16, seed=43)
    check_linear(h, w, t, 0.2, "sum", chunk_rows=3, what="V=13, D=8", gemm=gemm)


@pytest.mark.parametrize("gemm", ENGINES)
def test_linear_tile_edges(gemm):
    """Sizes around the native kernel's 256 x 256 x 64 tiles and its even
    k-tile count: K = D of 64, 128 and 192 (one, two and three k-tiles),
    V one past and one short of a tile, chunks of 255, 256 and 257 rows."""
    for N, D, V, chunk in [(300, 64, 257, 256), (257, 128, 511, 255), (520, 192, 768, 257), (64, 448, 1000, 0)]:
        h, w, t = grid_inputs(N, D, V, torch.bfloat16, seed=N + D)
        check_linear(h, w, t, 0.1, "mean", chunk_rows=chunk, what=f"tile edges N={N} D={D} V={V}", gemm=gemm)


def test_linear_many_tiles():
    """More logits tiles than compute units, in a count that is not a multiple of 8: 3 x 157 = 471 tiles of
    256 x 256 over 2 k-tiles, which the native kernel's persistent form deals to the 8 XCDs in runs of 59
    and 58 tiles, each workgroup taking one or two; the dW product over 12 k-tiles and 157 row blocks."""
    h, w, t = grid_inputs(768, 128, 40001, torch.bfloat16, seed=71)
    check_linear(h, w, t, 0.1, "mean", chunk_rows=768, what="many tiles", gemm="native")


def test_linear_split_dh():
    """dh of chunks with fewer output tiles than half the compute units: the native kernel splits the
    vocabulary (K = 8192, 128 k-tiles) over FP32 partial planes in the head's GEMM scratch (2 tiles of 256 x
    256 per chunk of 256 rows, so 128 splits of one k-tile) and sums them in a fixed order."""
    h, w, t = grid_inputs(512, 512, 8192, torch.bfloat16, seed=73)
    check_linear(h, w, t, 0.1, "sum", chunk_rows=256, what="split dh", gemm="native")


def test_linear_no_rows():
    h = torch.empty((0, 32), dtype=torch.bfloat16, device="cuda")
    w = torch.ones((100, 32), dtype=torch.bfloat16, device="cuda")
    t = torch.empty((0,), dtype=torch.int64, device="cuda")
    dw = torch.full((100, 32), 5.0, device="cuda")
    loss, dh, dwo, n = vce.ce_linear_cross_entropy(h, w, t, 0.1, "mean", dw=dw)
    ls, _, _, _ = vce.ce_linear_cross_entropy(h, w, t, 0.1, "sum", want_dw=False)
    lr, _, _, _ = vce.ce_linear_cross_entropy(h, w, t, 0.1, "none", want_dw=False)  # an empty loss[0]
    torch.cuda.synchronize()
    assert lr.numel() == 0
    assert int(n.item()) == 0 and math.isnan(loss.item()) and ls.item() == 0.0
    assert torch.count_nonzero(dwo).item() == 0, "no rows: dW is zero"


@pytest.mark.parametrize("gemm", ENGINES)
def test_linear_full_size(gemm):
    """The 4 x 2048-row head of a 4096-wide model onto 128000 BF16 columns in
    the automatic chunks (4096 rows), against the oracle's blocked head over
    every row: the mean against the oracle's mean over all rows, every row's
    loss (an unreduced call), dW element by element on 16 sampled hidden
    columns (all 128000 vocabulary rows of each) within the derived bar, and
    dh on sampled rows (the oracle's own loops)."""
    N, D, V = 8192, 4096, 128000
    say("[linear] generating the full-size grid inputs")
    h, w, t = grid_inputs(N, D, V, torch.bfloat16, seed=29, ignore_frac=0.05)
    n_all = int((t != -100).sum())
    loss, dh, dw, n = run_linear(h, w, t, 0.1, "mean", gemm=gemm)
    assert n == n_all
    o = orc()
    rng = np.random.default_rng(1)
    cols = np.unique(np.concatenate([[0, 1, D - 1], rng.choice(D, 13, replace=False)]))
    habs = np.abs(h.double().numpy()[:, cols])
    acc = [np.zeros((V, cols.size))]

    def bar_terms(rows, G):  # sum_i |G_ij| |h_id| over the rows, for the dW bar
        acc[0] += np.abs(G).T @ habs[rows]

    say("[linear] oracle over every row (blocked head)")
    ref_rows, ref_dw = o.linear_ce_blocked(h, w, t, 0.1, reduce_loss="mean", n_valid=n_all, dw_cols=cols,
                                           on_block=bar_terms)
    assert_loss([loss[0]], [o.mean_loss(ref_rows, n_all)], "full size mean")
    rl, _, _, _ = run_linear(h, w, t, 0.1, "none", want_dh=False, want_dw=False, gemm=gemm)
    assert_loss(rl, ref_rows, "full size loss rows")
    assert np.all(rl[t.numpy() == -100] == 0.0)
    # dW: (r_G + gamma_N) sum_i |G||h| + a_G sum_i |h| + the FP32 output's rounding
    r_g, a_g, _ = _bars(torch.bfloat16)
    tol = (r_g + N * 2.0 ** -24) * acc[0] + a_g * np.broadcast_to(habs.sum(axis=0), ref_dw.shape)
    tol = tol + 2.0 ** -23 * (np.abs(ref_dw) + tol)
    got = dw[:, cols]
    err = np.abs(got - ref_dw)
    bad = ~(err <= tol)
    assert not bad.any(), f"full size dW: {bad.sum()} elements off, max err {err.max():.3e}"
    rows = np.array([0, 1, 1023, 1024, 4097, 8191] + list(rng.choice(N, 6, replace=False)))
    say(f"[linear] oracle dh on {len(rows)} sampled rows")
    hs, ts = h[rows].contiguous(), t[rows].contiguous()
    _, ref_dh, _, G = o.linear_ce(hs, w, ts, 0.1, reduce_loss="mean", n_valid=n_all, want_dw=False, want_g=True)
    check_dh(dh[rows], ref_dh, G, w, torch.bfloat16, "full size sampled dh")


@pytest.mark.parametrize("gemm", ENGINES)
@pytest.mark.parametrize("reduce", ["mean", "sum", "none"])
def test_linear_autograd(reduce, gemm):
    """linear_cross_entropy: the loss and, after backward with upstream 0.5
    (per-row weights for per-row losses), h.grad and W.grad (FP32 dW cast to
    BF16 by autograd) against the oracle."""
    h, w, t = grid_inputs(48, 64, 3001, torch.bfloat16, seed=31)
    say(f"[linear autograd] {reduce}")
    hd = h.cuda().requires_grad_(True)
    wd = w.cuda().requires_grad_(True)
    loss = vce.linear_cross_entropy(hd, wd, t.cuda(), 0.1, reduce, chunk_rows=16, gemm=gemm)
    gw = np.linspace(-1.0, 2.0, 48) if reduce == "none" else 0.5
    if reduce == "none":
        loss.backward(torch.as_tensor(gw, dtype=torch.float32, device="cuda"))
    else:
        (0.5 * loss).backward()
    torch.cuda.synchronize()
    o = orc()
    ref_rows, ref_dh, ref_dw, G = o.linear_ce(h, w, t, 0.1, reduce_loss=reduce, g=gw, want_g=True)
    if reduce == "none":
        assert_loss(loss.detach().cpu().numpy(), ref_rows, "autograd rows")
    else:
        assert_loss([loss.item()], [o.reduce(ref_rows, reduce, int((t != -100).sum()))], f"autograd {reduce}")
    assert hd.grad.dtype == torch.bfloat16 and wd.grad.dtype == torch.bfloat16
    check_dh(hd.grad.double().cpu().numpy(), ref_dh, G, w, torch.bfloat16, "autograd h.grad")
    check_dw(wd.grad.double().cpu().numpy(), ref_dw, G, h, torch.bfloat16, "autograd W.grad", out_rho=2.0 ** -8)


def test_linear_autograd_trains_a_head():
    """A few SGD steps on a head through linear_cross_entropy lower the loss
    (hidden states fixed, the weight learns; FP32)."""
    g = torch.Generator().manual_seed(37)
    h = torch.randn((256, 32), generator=g).cuda()
    t = torch.randint(0, 500, (256,), generator=g).cuda()
    w = (torch.randn((500, 32), generator=g) * 0.05).cuda().requires_grad_(True)
    losses = []
    for _ in range(20):
        loss = vce.linear_cross_entropy(h, w, t, 0.0, "mean", chunk_rows=64)
        w.grad = None
        loss.backward()
        with torch.no_grad():
            w -= 2.0 * w.grad
        losses.append(loss.item())
    assert losses[-1] < 0.8 * losses[0], losses


@pytest.mark.parametrize("gemm", ENGINES)
def test_linear_graph_replays(gemm):
    """A captured ce_linear_cross_entropy (GEMMs, one fused call per chunk,
    count and finish kernels) replays bit-identically to the eager call: each
    chunk's fused call takes its tag from the workspace's epoch, which every
    call advances, so replays never see an earlier call's words."""
    h, w, t = grid_inputs(64, 64, 3001, torch.bfloat16, seed=41)
    hd, wd, td = h.cuda(), w.cuda(), t.cuda()
    nb, _ = vce.ce_linear_workspace_bytes(hd, wd, "mean", 16, 0.1)
    ws = vce.ce_workspace_init(torch.empty(nb, dtype=torch.uint8, device="cuda"))
    loss = torch.empty(1, device="cuda")
    dh = torch.empty_like(hd)
    dw = torch.empty((3001, 64), device="cuda")
    n = torch.empty(1, dtype=torch.int32, device="cuda")

    def call():
        vce.ce_linear_cross_entropy(hd, wd, td, 0.1, "mean", loss=loss, n_valid=n, dh=dh, dw=dw, ws=ws,
                                    chunk_rows=16, gemm=gemm)

    say("[linear graph] eager reference")
    call()
    torch.cuda.synchronize()
    ref = (loss.clone(), dh.clone(), dw.clone())
    say("[linear graph] capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"[linear graph] replay {rep}")
        loss.fill_(float("nan"))
        dh.zero_()
        dw.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(loss.view(torch.int32), ref[0].view(torch.int32)), f"replay {rep}: loss"
        assert torch.equal(dh.view(torch.int16), ref[1].view(torch.int16)), f"replay {rep}: dh"
        assert torch.equal(dw.view(torch.int32), ref[2].view(torch.int32)), f"replay {rep}: dW"
        if rep == 0:
            call()  # an eager call on the same workspace between replays
            torch.cuda.synchronize()
    vce.ce_workspace_check(ws)


def test_linear_after_tuning():
    """ce_linear_tune picks each GEMM's algorithm by timing; the call then
    still meets the bar (ragged last chunk, dh and dW)."""
    h, w, t = grid_inputs(72, 64, 3001, torch.bfloat16, seed=43)
    hd, wd = h.cuda(), w.cuda()
    say("[linear tune] timing candidates")
    vce.ce_linear_tune(hd, wd, "mean", chunk_rows=32)
    check_linear(h, w, t, 0.1, "mean", chunk_rows=32, what="after tuning")


def test_linear_from_two_host_threads():
    """Two host threads run the chunked head at the same time, each on its own
    stream and workspace (sharing the library's per-device GEMM handle and
    plans); each result equals the same call made alone."""
    import threading

    cases = [grid_inputs(48, 64, 3001, torch.bfloat16, seed=s) for s in (91, 92)]
    refs = [run_linear(h, w, t, 0.1, "mean", chunk_rows=16) for h, w, t in cases]
    errors = []

    def worker(i):
        try:
            h, w, t = cases[i]
            stream = torch.cuda.Stream()
            hd, wd, td = h.cuda(), w.cuda(), t.cuda()
            torch.cuda.synchronize()
            with torch.cuda.stream(stream):
                for _ in range(10):
                    loss, dh, dw, n = vce.ce_linear_cross_entropy(hd, wd, td, 0.1, "mean", chunk_rows=16)
                    stream.synchronize()
                    got = (loss.cpu().double().numpy(), dh.cpu().double().numpy(), dw.cpu().double().numpy())
                    if not all(np.array_equal(a, b) for a, b in zip(got, refs[i][:3])):
                        errors.append(f"thread {i}: result differs")
                        return
        except Exception as e:  # reported below
            errors.append(f"thread {i}: {e!r}")

    say("[linear] two host threads")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
