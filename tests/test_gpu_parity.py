"""GPU parity of libmuon (through its C ABI) against the float64 oracle.

Tolerances (relative Frobenius error of the update / polar output):
  fp32 path  <= 1e-4;  bf16 matrix-core path <= 3e-2;
  long-side row norms agree within 1e-2 (bf16);  momentum <= 1e-6 (relative).
Weights W' are checked against the oracle's W - lr V, rounded to the stored
type: elementwise within half an ulp of each of the two rounded values plus
lr times the update's own difference from the oracle (bounded by the V
test); they are also checked exactly against the update the same call
returned (W' == round(W - lr V)).
Inputs come from the seeded generators; the oracle reads the stored tensors.
"""
import math
import sys

import numpy as np
import pytest
import torch

import muon_newton_schulz_update_amd as mu
from muon_newton_schulz_update_amd import inputs as gen
from oracle import muon_oracle as O

pytestmark = pytest.mark.gpu

FP32_TOL, BF16_TOL, ROW_TOL, MOM_TOL = 1e-4, 3e-2, 1e-2, 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def f64(t):
    return t.detach().float().cpu().double().numpy()


def rel(a, b):
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


def row_agree(a, b):
    """max relative difference of long-side row norms."""
    if a.shape[0] < a.shape[1]:
        a, b = a.T, b.T
    na, nb = np.linalg.norm(a, axis=1), np.linalg.norm(b, axis=1)
    mask = nb > 1e-6 * nb.max()
    return float(np.max(np.abs(na[mask] / nb[mask] - 1))) if mask.any() else 0.0


def ocfg(cfg: mu.MuonConfig) -> O.OracleConfig:
    return O.OracleConfig(ns_steps=cfg.ns_steps, ns_a=cfg.ns_a, ns_b=cfg.ns_b, ns_c=cfg.ns_c,
                          ns_eps=float(np.float32(cfg.ns_eps)), pp_iterations=cfg.pp_iterations,
                          pp_beta=cfg.pp_beta, pp_eps=float(np.float32(cfg.pp_eps)),
                          mu=float(np.float32(cfg.mu)), nesterov=bool(cfg.nesterov),
                          power_steps=cfg.power_steps, contra=float(np.float32(cfg.contra)),
                          target_uw=float(np.float32(cfg.target_uw)), lr=float(np.float32(cfg.lr)),
                          momentum="sgd" if cfg.flags & mu.MUON_FLAG_SGD_MOMENTUM else "ema",
                          wide_rows=bool(cfg.flags & mu.MUON_FLAG_WIDE_ROWS))


def weight_add_ok(W0, V, W1, cfg):
    """W1 == round(W0 - lr V): within one ulp of the stored type (the kernel
    may fuse the multiply-add, so fp32 is allowed the product's rounding too)."""
    lr = np.float32(cfg.lr)
    want = (W0.float() - lr * V.float()).to(W0.dtype).float()
    diff = (W1.float() - want).abs()
    # fp32 rounding of the two terms (fused or not), plus one ulp of the stored type
    tol = (W0.float().abs() + lr * V.float().abs()) * 2.0 ** -22
    if W0.dtype == torch.bfloat16:
        tol = tol + want.abs() * 2.0 ** -7
    return bool((diff <= tol + 1e-30).all())


def rne_bf16(x64):
    return torch.from_numpy(np.asarray(x64, dtype=np.float32)).to(torch.bfloat16)


def _ulp(x, dtype):
    """Spacing of the stored type at |x| (the gap to the next representable
    value away from zero; subnormal spacing at 0)."""
    ax = np.abs(x.astype(np.float64))
    e = np.floor(np.log2(np.maximum(ax, np.finfo(np.float32).tiny)))
    mant = 7 if dtype == torch.bfloat16 else 23
    return np.exp2(np.maximum(e, -126) - mant)


def weight_vs_oracle(case, W0, W1, V, Vo, cfg):
    """W' against the oracle's parameter step W - lr V_oracle.

    W' = round(W - lr V) with V the library's update, so elementwise
      |W' - round(W - lr V_oracle)| <= ulp(W')/2 + ulp(want)/2 + lr |V - V_oracle|
    plus fp32 rounding of the product and the difference (ulp at each
    value's own binade; round-to-nearest puts a value at most half its ulp
    from the exact one). The V term is the update's own difference from the
    oracle, which the V test bounds. The share of elements within one ulp
    outright is printed: it depends on the inputs (elements where |W'| is so
    small that lr |V - V_oracle| is above its ulp fall outside)."""
    lr = float(np.float32(cfg.lr))
    w0 = f64(W0)
    exact = w0 - lr * Vo
    want = torch.from_numpy(exact.astype(np.float32)).to(W0.dtype).double().numpy()
    got = f64(W1)
    ulp_w, ulp_g = _ulp(want, W0.dtype), _ulp(got, W0.dtype)
    diff = np.abs(got - want)
    bound = 0.5 * (ulp_w + ulp_g) + lr * np.abs(f64(V) - Vo) + (np.abs(w0) + lr * np.abs(Vo)) * 2.0 ** -22
    frac = float(np.mean(diff <= ulp_w))
    say(f"  {case}: W' vs oracle: {frac * 100:.3f} % within 1 ulp, max diff/bound "
        f"{float(np.max(diff / bound)):.3f}")
    assert bool(np.all(diff <= bound)), case


def check_update(case, G, M0, W0, M1, V, W1, cfg, tol, rows_tol=None):
    """Compare one matrix's outputs with the oracle."""
    oc = ocfg(cfg)
    Mo, Vo, Wo = O.muon_update(f64(G), f64(M0), None if W0 is None else f64(W0), oc)
    e_v = rel(f64(V), Vo)
    e_m = rel(f64(M1), Mo)
    say(f"  {case}: {tuple(G.shape)} {G.dtype} rel(V)={e_v:.2e} rel(M)={e_m:.2e}")
    assert e_v <= tol, (case, e_v)
    assert e_m <= MOM_TOL, (case, e_m)
    if rows_tol is not None:
        assert row_agree(f64(V), Vo) <= rows_tol, case
    if W0 is not None:
        # the parameter add is exact given the returned update: W' = round(W - lr V)
        assert weight_add_ok(W0, V, W1, cfg), case
        weight_vs_oracle(case, W0, W1, V, Vo, cfg)
    return e_v


def run_update(dev, mats, cfg=None, out_dtype=torch.float32, handle=None):
    """mats: list of (G, M, W-or-None) on the device. Returns (M1, V, W1) lists and the originals."""
    cfg = cfg or mu.default_config()
    G = [g for g, _, _ in mats]
    M0 = [m.clone() for _, m, _ in mats]
    W0 = [None if w is None else w.clone() for _, _, w in mats]
    M = [m.clone() for _, m, _ in mats]
    W = [None if w is None else w.clone() for _, _, w in mats]
    V = [torch.empty(g.shape, device=dev, dtype=out_dtype) for g in G]
    have_w = any(w is not None for w in W)
    mu.muon_update(G, M, W if have_w else None, cfg, update_out=V, handle=handle)
    torch.cuda.synchronize()
    return G, M0, W0, M, V, W


# ---------------------------------------------------------------------------
# ns_polar
# ---------------------------------------------------------------------------
ODD = [(1, 1), (1, 7), (7, 1), (5, 5), (33, 517), (517, 33), (255, 257), (300, 700), (4096, 1), (1, 4096)]


def test_ns_polar_fp32_odd_shapes(dev):
    say("ns_polar fp32 odd shapes (one batched call)")
    xs = [gen.custom_matrix(s, 100 + i, dev)[0] for i, s in enumerate(ODD)]
    outs = mu.ns_polar(xs)
    torch.cuda.synchronize()
    for x, u in zip(xs, outs):
        e = rel(f64(u), O.newton_schulz(f64(x)))
        say(f"  {tuple(x.shape)} rel={e:.2e}")
        assert e <= FP32_TOL


def test_ns_polar_bf16(dev):
    say("ns_polar bf16")
    shapes = [(300, 700), (768, 768), (700, 300), (40, 1000)]
    xs = [gen.custom_matrix(s, 200 + i, dev, grad_dtype=torch.bfloat16, grad_sd=1e-3)[0]
          for i, s in enumerate(shapes)]
    outs = mu.ns_polar(xs, [torch.empty(x.shape, device=dev, dtype=torch.float32) for x in xs])
    torch.cuda.synchronize()
    for x, u in zip(xs, outs):
        want = O.newton_schulz(f64(x))
        e = rel(f64(u), want)
        say(f"  {tuple(x.shape)} rel={e:.2e} rows={row_agree(f64(u), want):.2e}")
        assert e <= BF16_TOL
        assert row_agree(f64(u), want) <= ROW_TOL


def test_ns_polar_aliasing_and_ld(dev):
    say("ns_polar in-place and ld > cols")
    x = gen.custom_matrix((130, 300), 300, dev)[0]
    want = O.newton_schulz(f64(x))
    y = x.clone()
    mu.ns_polar([y], [y])                                   # out aliases in
    big = torch.zeros((130, 512), device=dev)
    big[:, 100:400] = x
    view = big[:, 100:400]                                  # ld = 512
    out_big = torch.full((130, 320), 7.0, device=dev)
    mu.ns_polar([view], [out_big[:, :300]])
    torch.cuda.synchronize()
    assert rel(f64(y), want) <= FP32_TOL
    assert rel(f64(out_big[:, :300]), want) <= FP32_TOL
    assert bool((out_big[:, 300:] == 7.0).all())            # nothing outside the view written


@pytest.mark.parametrize("dtype,tol", [(torch.float32, FP32_TOL), (torch.bfloat16, BF16_TOL)])
def test_ns_polar_classic_five_step(dev, dtype, tol):
    """The earlier 5-step recipe (Track-1 page) through the same engine."""
    say(f"ns_polar classic 5-step recipe {dtype}")
    cfg = mu.make_config(ns_steps=5, ns_a=3.4445, ns_b=-4.7750, ns_c=2.0315)
    xs = [gen.custom_matrix(s, 250 + i, dev, grad_dtype=dtype, grad_sd=1e-3)[0]
          for i, s in enumerate([(200, 600), (600, 200), (384, 384)])]
    outs = mu.ns_polar(xs, [torch.empty(x.shape, device=dev) for x in xs], cfg=cfg)
    torch.cuda.synchronize()
    for x, u in zip(xs, outs):
        e = rel(f64(u), O.ns5_classic(f64(x), 5, np.float32(3.4445), np.float32(-4.7750), np.float32(2.0315)))
        say(f"  {tuple(x.shape)} rel={e:.2e}")
        assert e <= tol


# ---------------------------------------------------------------------------
# aurora_orthogonalize
# ---------------------------------------------------------------------------
def test_aurora_fp32(dev):
    say("aurora fp32 pp=2 beta=0.5")
    shapes = [(33, 517), (517, 33), (256, 1024), (600, 200), (96, 96)]
    xs = [gen.custom_matrix(s, 400 + i, dev)[0] for i, s in enumerate(shapes)]
    outs = mu.aurora_orthogonalize(xs)
    torch.cuda.synchronize()
    for x, u in zip(xs, outs):
        e = rel(f64(u), O.aurora_orthogonalize(f64(x)))
        say(f"  {tuple(x.shape)} rel={e:.2e}")
        assert e <= FP32_TOL


@pytest.mark.parametrize("pp,beta", [(1, 0.5), (3, 0.5), (2, 0.25), (2, 1.0), (0, 0.5)])
def test_aurora_fp32_options(dev, pp, beta):
    say(f"aurora fp32 pp={pp} beta={beta}")
    x = gen.custom_matrix((384, 160), 500 + pp * 10 + int(beta * 4), dev)[0]
    cfg = mu.make_config(pp_iterations=pp, pp_beta=beta)
    u = mu.aurora_orthogonalize([x], cfg=cfg)[0]
    torch.cuda.synchronize()
    e = rel(f64(u), O.aurora_orthogonalize(f64(x), pp, beta))
    say(f"  rel={e:.2e}")
    assert e <= FP32_TOL


def test_aurora_bf16(dev):
    say("aurora bf16")
    shapes = [(256, 1024), (1024, 256), (512, 512), (768, 3072)]
    xs = [gen.custom_matrix(s, 600 + i, dev, grad_dtype=torch.bfloat16, grad_sd=1e-3)[0]
          for i, s in enumerate(shapes)]
    outs = mu.aurora_orthogonalize(xs, [torch.empty(x.shape, device=dev) for x in xs])
    torch.cuda.synchronize()
    for x, u in zip(xs, outs):
        want = O.aurora_orthogonalize(f64(x))
        e, r = rel(f64(u), want), row_agree(f64(u), want)
        say(f"  {tuple(x.shape)} rel={e:.2e} rows={r:.2e}")
        assert e <= BF16_TOL and r <= ROW_TOL


# ---------------------------------------------------------------------------
# muon_update
# ---------------------------------------------------------------------------
def test_ns_polar_misaligned_bf16_view(dev):
    say("ns_polar on a bf16 view with an odd column offset and odd ld")
    x = gen.custom_matrix((140, 260), 310, dev, grad_dtype=torch.bfloat16)[0]
    want = O.newton_schulz(f64(x))
    big = torch.full((140, 267), 3.0, device=dev, dtype=torch.bfloat16)
    view = big[:, 1:261]                                    # 2-byte offset, ld = 267
    view.copy_(x)
    out_big = torch.full((140, 263), 7.0, device=dev, dtype=torch.bfloat16)
    out = out_big[:, 3:263]
    mu.ns_polar([view], [out])
    torch.cuda.synchronize()
    e = rel(f64(out), want)
    say(f"  rel={e:.2e}")
    assert e <= BF16_TOL
    assert torch.equal(view, x) and bool((big[:, 0] == 3.0).all()) and bool((big[:, 261:] == 3.0).all())
    assert bool((out_big[:, :3] == 7.0).all())


@pytest.mark.parametrize("aligned", [True, False])
def test_update_strided_caller_buffers(dev, aligned):
    """G, M, W and update_out as row-strided views: 16-byte aligned rows take
    the vector path of the streaming kernels with ld != cols; an odd column
    offset and odd ld take the element-wise path. Nothing outside a view
    may change."""
    say(f"muon_update on strided {'aligned' if aligned else 'misaligned'} caller views")
    pad, off = (16, 8) if aligned else (5, 1)
    cases = [((200, 300), torch.bfloat16, BF16_TOL), ((300, 200), torch.float32, FP32_TOL)]
    views, bigs, ref = [], [], []
    for i, (shape, dt, _) in enumerate(cases):
        g, m, w = gen.custom_matrix(shape, 1200 + i, dev, grad_dtype=dt, weight_dtype=dt)
        r, c = shape
        bg = torch.full((r, c + pad), 3.0, device=dev, dtype=dt)
        bm = torch.full((r, c + pad), 5.0, device=dev, dtype=torch.float32)
        bw = torch.full((r, c + pad), 6.0, device=dev, dtype=dt)
        bv = torch.full((r, c + pad), 7.0, device=dev, dtype=torch.float32)
        vg, vm, vw, vv = (b[:, off:off + c] for b in (bg, bm, bw, bv))
        vg.copy_(g); vm.copy_(m); vw.copy_(w)
        views.append((vg, vm, vw, vv)); bigs.append((bg, bm, bw, bv)); ref.append((g, m.clone(), w.clone()))
    mu.muon_update([v[0] for v in views], [v[1] for v in views], [v[2] for v in views], mu.default_config(),
                   update_out=[v[3] for v in views])
    torch.cuda.synchronize()
    for i, (shape, dt, tol) in enumerate(cases):
        vg, vm, vw, vv = views[i]
        g, m0, w0 = ref[i]
        check_update(f"strided[{i}]", g, m0, w0, vm, vv, vw, mu.default_config(), tol)
        assert torch.equal(vg, g), "the grad is read-only"
        c = shape[1]
        for b, fill in zip(bigs[i], (3.0, 5.0, 6.0, 7.0)):
            outside = torch.cat([b[:, :off], b[:, off + c:]], dim=1)
            assert bool((outside == fill).all()), "a write landed outside a view"


@pytest.mark.parametrize("tile", [128, 256])
def test_engine_tile_sizes(dev, tile, monkeypatch):
    """Both engine tile edges on odd, padded shapes (launches this small
    choose 128 by default; 256 is forced here), fp32 and bf16, through
    ns_polar and the Aurora path of muon_update. A fresh handle builds its
    plans with the forced size."""
    say(f"engine forced to {tile}x{tile} tiles")
    monkeypatch.setenv("MUON_NS_TILE", str(tile))
    h = mu.Handle(dev.index)
    try:
        shapes = [(33, 517), (300, 700), (517, 33), (260, 260)]
        for dt, tol in ((torch.float32, FP32_TOL), (torch.bfloat16, BF16_TOL)):
            xs = [gen.custom_matrix(sh, 1300 + i, dev, grad_dtype=dt)[0] for i, sh in enumerate(shapes)]
            outs = mu.ns_polar(xs, handle=h)
            torch.cuda.synchronize()
            for x, o in zip(xs, outs):
                e = rel(f64(o), O.newton_schulz(f64(x)))
                say(f"  ns_polar {tuple(x.shape)} {dt} rel={e:.2e}")
                assert e <= tol
        mats = [gen.custom_matrix((384, 130), 1320, dev, grad_dtype=torch.bfloat16, weight_dtype=torch.bfloat16),
                gen.custom_matrix((130, 600), 1321, dev)]
        G, M0, W0, M, V, W = run_update(dev, mats, handle=h)
        check_update("tile-bf16", G[0], M0[0], W0[0], M[0], V[0], W[0], mu.default_config(), BF16_TOL, ROW_TOL)
        check_update("tile-fp32", G[1], M0[1], W0[1], M[1], V[1], W[1], mu.default_config(), FP32_TOL)
    finally:
        h.close()


def test_engine_layouts_and_tiles_agree_bitwise(dev, monkeypatch):
    """Every output element's K sum runs inside one wave in the same k
    order whatever the workgroup layout or tile edge, so the 4-wave
    128 x 128 layout (MUON_NS_VARIANT=1), forced 256-tiles and forced
    128-tiles give the default's bits exactly: a check of each refill
    schedule (the 256-tile one, with four or eight loads per operand and
    wave, and the 128-tile one) against the others. Rectangular matrices
    with blocks (s >= 512) and squares, bf16 and fp32, in one update."""
    say("engine layouts and tile edges agree bitwise")
    mats = [gen.custom_matrix(sh, 1350 + i, dev, grad_dtype=dt, weight_dtype=dt)
            for i, (sh, dt) in enumerate([((600, 1300), torch.bfloat16), ((1300, 520), torch.bfloat16),
                                          ((512, 512), torch.bfloat16), ((300, 700), torch.float32),
                                          ((520, 1030), torch.float32)])]
    results = {}
    for name, env in (("default", {}), ("4-wave 256", {"MUON_NS_VARIANT": "1", "MUON_NS_TILE": "256"}),
                      ("8-wave 256", {"MUON_NS_TILE": "256"}), ("128", {"MUON_NS_TILE": "128"})):
        for k in ("MUON_NS_VARIANT", "MUON_NS_TILE"):
            monkeypatch.delenv(k, raising=False)
        for k, v in env.items():
            monkeypatch.setenv(k, v)
        h = mu.Handle(dev.index)
        try:
            results[name] = run_update(dev, mats, handle=h)[3:]
        finally:
            h.close()
    base = results["default"]
    for name, res in results.items():
        for i in range(len(mats)):
            for a, b in zip(res, base):
                assert same_bits(a[i], b[i]), (name, i)
        say(f"  {name}: bitwise equal to the default")


def test_side_stream_matches_one_stream(dev, monkeypatch):
    """On small sets the Newton-Schulz passes run as two chains of launches
    on two streams: the one-iteration matrices (squares, and rectangular
    matrices whose short side is under 512, which carry Aurora and so feed
    the D update after the pass) beside those with blocks, or, in a pass
    with only one of the two kinds, two halves of it (here: squares only;
    blocked rectangles only, split in both Aurora passes; squares beside
    blocked rectangles in the first pass, the rectangles split in the
    second). The call's stream waits for the second one at the end of each
    pass. Two
    calls in a row (the fork and join events are reused, the second call
    reads the first one's momenta and weights) give the one-stream bits
    (MUON_NS_SIDE=0, no split) exactly, by default and with the second
    stream forced on; the default's second step is checked against the
    oracle too."""
    say("second stream of small sets against one stream")
    batches = {
        "mixed": [((600, 1300), torch.bfloat16), ((768, 768), torch.bfloat16), ((300, 700), torch.bfloat16),
                  ((700, 300), torch.float32), ((520, 1030), torch.float32), ((256, 256), torch.float32)],
        "squares": [((768, 768), torch.bfloat16)] * 5 + [((512, 512), torch.float32)] * 2,
        "blocked": [((600, 1300), torch.bfloat16), ((1300, 600), torch.bfloat16), ((768, 2304), torch.bfloat16)],
        "squares and blocked": [((768, 768), torch.bfloat16)] * 3 + [((768, 3072), torch.bfloat16),
                                                                      ((3072, 768), torch.bfloat16)],
    }
    for bname, spec in batches.items():
        mats = [gen.custom_matrix(sh, 1380 + 10 * len(bname) + i, dev, grad_dtype=dt, weight_dtype=dt)
                for i, (sh, dt) in enumerate(spec)]
        results = {}
        for name, env in (("one stream", "0"), ("default", None), ("forced", "1")):
            monkeypatch.delenv("MUON_NS_SIDE", raising=False)
            if env is not None:
                monkeypatch.setenv("MUON_NS_SIDE", env)
            h = mu.Handle(dev.index)
            try:
                G = [g for g, _, _ in mats]
                M = [m.clone() for _, m, _ in mats]
                W = [w.clone() for _, _, w in mats]
                V = [torch.empty(g.shape, device=dev) for g in G]
                mu.muon_update(G, M, W, mu.default_config(), update_out=V, handle=h)
                M1 = [m.clone() for m in M]
                W1 = [w.clone() for w in W]
                mu.muon_update(G, M, W, mu.default_config(), update_out=V, handle=h)
                torch.cuda.synchronize()
                results[name] = (M1, W1, M, W, V)
            finally:
                h.close()
        base = results["one stream"]
        for name, res in results.items():
            for a, b in zip(res, base):
                for i in range(len(mats)):
                    assert same_bits(a[i], b[i]), (bname, name, i)
            say(f"  {bname}, {name}: bitwise equal to one stream over two calls")
        M1, W1, M, W, V = results["default"]
        for i, (g, _, _) in enumerate(mats):
            tol = BF16_TOL if g.dtype == torch.bfloat16 else FP32_TOL
            check_update(f"{bname}[{i}]", g, M1[i], W1[i], M[i], V[i], W[i], mu.default_config(), tol)


@pytest.mark.parametrize("block", [1, 2, 3, 8])
def test_engine_block_lengths(dev, block, monkeypatch):
    """Rectangular matrices run Newton-Schulz in blocks of iterations on the
    short side (Gram, short-side products, one X' = Q X per block); the block
    length is forced here (MUON_NS_BLOCK, read when a fresh handle builds its
    plans): 1 is the plain iteration, 8 longer than the default, 3 leaves a
    shorter last block of 12 iterations and of the classic 5. ns_polar,
    aurora_orthogonalize and muon_update, fp32 and bf16, odd shapes."""
    say(f"engine with {block}-iteration blocks")
    monkeypatch.setenv("MUON_NS_BLOCK", str(block))
    h = mu.Handle(dev.index)
    try:
        shapes = [(33, 517), (300, 700), (517, 33), (260, 260)]
        for dt, tol in ((torch.float32, FP32_TOL), (torch.bfloat16, BF16_TOL)):
            xs = [gen.custom_matrix(sh, 2800 + i, dev, grad_dtype=dt)[0] for i, sh in enumerate(shapes)]
            for name, cfg, ref in (("ns_polar", None, lambda x: O.newton_schulz(x)),
                                   ("classic ns", mu.make_config(ns_steps=5, ns_a=3.4445, ns_b=-4.7750,
                                                                 ns_c=2.0315),
                                    lambda x: O.ns5_classic(x, 5, np.float32(3.4445), np.float32(-4.7750),
                                                            np.float32(2.0315)))):
                outs = mu.ns_polar(xs, [torch.empty(x.shape, device=dev) for x in xs], cfg=cfg, handle=h)
                torch.cuda.synchronize()
                for x, o in zip(xs, outs):
                    e = rel(f64(o), ref(f64(x)))
                    say(f"  {name} {tuple(x.shape)} {dt} rel={e:.2e}")
                    assert e <= tol
            outs = mu.aurora_orthogonalize(xs, [torch.empty(x.shape, device=dev) for x in xs], handle=h)
            torch.cuda.synchronize()
            for x, o in zip(xs, outs):
                want = O.aurora_orthogonalize(f64(x))
                e = rel(f64(o), want)
                say(f"  aurora {tuple(x.shape)} {dt} rel={e:.2e}")
                assert e <= tol
                if dt == torch.bfloat16:
                    assert row_agree(f64(o), want) <= ROW_TOL
        mats = [gen.custom_matrix((384, 130), 2820, dev, grad_dtype=torch.bfloat16, weight_dtype=torch.bfloat16),
                gen.custom_matrix((130, 600), 2821, dev), gen.custom_matrix((200, 200), 2822, dev)]
        G, M0, W0, M, V, W = run_update(dev, mats, handle=h)
        check_update("block-bf16", G[0], M0[0], W0[0], M[0], V[0], W[0], mu.default_config(), BF16_TOL, ROW_TOL)
        check_update("block-fp32", G[1], M0[1], W0[1], M[1], V[1], W[1], mu.default_config(), FP32_TOL)
        check_update("block-square", G[2], M0[2], W0[2], M[2], V[2], W[2], mu.default_config(), FP32_TOL)
    finally:
        h.close()


@pytest.mark.parametrize("dtype,tol", [(torch.float32, FP32_TOL), (torch.bfloat16, BF16_TOL)])
def test_update_ragged_columns_mixed_lanes(dev, dtype, tol):
    """Column counts whose last 8-column chunk is partial, so one wave holds
    lanes on the vector path, a lane on the element-wise path and idle
    lanes (cross-lane sums must wait until they rejoin); rows not a
    multiple of the 8-row wave batch."""
    say(f"muon_update with ragged columns, {dtype}")
    shapes = [(37, 260), (260, 37), (70, 1030), (1030, 70), (9, 515)]
    mats = [gen.custom_matrix(sh, 1400 + i, dev, grad_dtype=dtype, weight_dtype=dtype)
            for i, sh in enumerate(shapes)]
    G, M0, W0, M, V, W = run_update(dev, mats)
    for i in range(len(shapes)):
        check_update(f"ragged[{i}]", G[i], M0[i], W0[i], M[i], V[i], W[i], mu.default_config(), tol,
                     ROW_TOL if dtype == torch.bfloat16 else None)


def test_calls_follow_the_current_stream(dev):
    """The binding hands torch's current stream to the handle (muon_set_stream
    when it changes): a call on a side stream, then one back on the default
    stream, each ordered after the work that produced its inputs."""
    say("muon_update on a side stream, then on the default stream")
    side = torch.cuda.Stream(device=dev)   # default priority
    cfg = mu.default_config()
    shapes = [(200, 90), (90, 200)]
    for rnd, stream in enumerate([side, torch.cuda.current_stream(dev)]):
        with torch.cuda.stream(stream):
            mats = [gen.custom_matrix(sh, 1700 + 10 * rnd + i, dev, weight_sd=1.0) for i, sh in enumerate(shapes)]
            G, M0, W0, M, V, W = run_update(dev, mats, cfg)
        for i in range(len(shapes)):
            check_update(f"stream{rnd}[{i}]", G[i], M0[i], W0[i], M[i], V[i], W[i], cfg, FP32_TOL)


def test_workspace_allocation_failure_leaves_handle_usable(dev):
    """A workspace larger than the device (40 matrices of 16384 x 65536 bf16,
    about 440 GB of workspace) fails in hipMalloc: MUON_ERR_ALLOC with a
    message, nothing enqueued, and the same handle then runs a normal call."""
    say("workspace allocation failure")
    h = mu.Handle(dev.index)
    try:
        with pytest.raises(mu.LibMuonError) as ei:
            h.reserve([(16384, 65536, torch.bfloat16)] * 40)
        assert ei.value.status == -4 and "workspace allocation" in str(ei.value)
        x = gen.custom_matrix((96, 200), 1500, dev)[0]
        out = mu.ns_polar([x], handle=h)[0]
        torch.cuda.synchronize()
        assert rel(f64(out), O.newton_schulz(f64(x))) <= FP32_TOL
    finally:
        h.close()


def test_entry_points_reject_shared_buffers(dev):
    """A written buffer that shares memory with another buffer of the call is
    rejected before anything is enqueued: the buffers keep their values. An
    in-place polar call and momenta that are column slices of one parent
    buffer are accepted and match the oracle."""
    say("entry points reject shared written buffers")
    g, m, w = gen.custom_matrix((64, 96), 1600, dev)
    g0, m0, w0 = g.clone(), m.clone(), w.clone()
    pw = torch.zeros((72, 96), device=dev)          # weight = rows 0..63, update_out = rows 8..71
    pw[:64].copy_(w)
    cases = [
        ("momentum is the grad", dict(grads=[g], moms=[g], weights=[w])),
        ("weight is the momentum", dict(grads=[g], moms=[m], weights=[m])),
        ("update_out overlaps the weight", dict(grads=[g], moms=[m], weights=[pw[:64]], out=[pw[8:]])),
    ]
    for name, c in cases:
        with pytest.raises(mu.LibMuonError) as ei:
            mu.muon_update(c["grads"], c["moms"], c["weights"], update_out=c.get("out"))
        assert ei.value.status == -1 and "share memory" in str(ei.value), (name, str(ei.value))
    x = torch.zeros((64, 96), device=dev)
    with pytest.raises(mu.LibMuonError) as ei:
        mu.ns_polar([g, m], [x, x])                  # two outputs in one buffer
    assert ei.value.status == -1 and "share memory" in str(ei.value), str(ei.value)
    torch.cuda.synchronize()
    assert torch.equal(g, g0) and torch.equal(m, m0) and torch.equal(w, w0), "a rejected call changed a buffer"
    assert torch.equal(pw[:64], w0) and bool((pw[64:] == 0).all()) and bool((x == 0).all())
    # momenta as column slices of one parent, weights likewise: accepted
    parent_m = torch.empty((64, 192), device=dev)
    parent_w = torch.empty((64, 192), device=dev)
    g2, m2, w2 = gen.custom_matrix((64, 96), 1601, dev)
    parent_m[:, :96].copy_(m); parent_m[:, 96:].copy_(m2)
    parent_w[:, :96].copy_(w); parent_w[:, 96:].copy_(w2)
    M = [parent_m[:, :96], parent_m[:, 96:]]
    W = [parent_w[:, :96], parent_w[:, 96:]]
    V = [torch.empty((64, 96), device=dev), torch.empty((64, 96), device=dev)]
    mu.muon_update([g, g2], M, W, update_out=V)
    torch.cuda.synchronize()
    for i, (gi, mi, wi) in enumerate([(g0, m0, w0), (g2, m2, w2)]):
        check_update(f"slices[{i}]", gi, mi, wi, M[i], V[i], W[i], mu.default_config(), FP32_TOL)


def test_profile_counts_and_flops(dev):
    """The library's own profile (what bench.py's roofline divides): for a
    256 x 256 bf16 square (one pass of 12 single iterations: GRAM, SQ, BX)
    and a 600 x 2048 bf16 matrix (two Aurora passes of three 4-iteration
    blocks: GRAM, 4 SQ, 9 SYM products in 7 launches, two of them a pair of
    independent products, BX), 36 + 78 engine launches, the algorithmic
    flops 12 * 4 s^3 and 2 * 3 * (3 s^2 L + 13 s^3), the counted flops
    (4 s^2 L + 2 s^3 per iteration and pass), positive times, and the
    streaming bytes of the momentum pass; twice that after a second step.
    The first pass runs the two matrices' chains on two streams; the
    classes' times are wall time covered (overlap counted once), so
    together they fit inside the call's own time."""
    say("profile counts and flops")
    mats = [gen.custom_matrix((256, 256), 3300, dev, grad_dtype=torch.bfloat16, weight_dtype=torch.bfloat16),
            gen.custom_matrix((600, 2048), 3301, dev, grad_dtype=torch.bfloat16, weight_dtype=torch.bfloat16)]
    h = mu.Handle(dev.index)
    try:
        h.profile_reset()
        h.profile_enable(True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run_update(dev, mats, handle=h)
        e1.record()
        torch.cuda.synchronize()
        wall = e0.elapsed_time(e1)
        p1 = h.profile_read()
        run_update(dev, mats, handle=h)
        p2 = h.profile_read()
        h.profile_enable(False)
    finally:
        h.close()
    sq, s, L = 256.0, 600.0, 2048.0
    algo = 12 * 4 * sq ** 3 + 2 * 3 * (3 * s * s * L + 13 * s ** 3)
    counted = 12 * (4 * sq ** 3 + 2 * sq ** 3) + 2 * 12 * (4 * s * s * L + 2 * s ** 3)
    say(f"  launches {p1['gemm_launches']}, engine {p1['gemm_ms']:.3f} ms, stream {p1['stream_ms']:.3f} ms")
    assert p1["gemm_launches"] == 36 + 78
    assert p1["gemm_algorithmic_flop"] == pytest.approx(algo, rel=1e-12)
    assert p1["gemm_counted_flop"] == pytest.approx(counted, rel=1e-12)
    assert p1["gemm_ms"] > 0 and p1["stream_ms"] > 0 and p1["aux_ms"] > 0
    say(f"  classes {p1['gemm_ms'] + p1['stream_ms'] + p1['aux_ms']:.3f} ms of the call's {wall:.3f} ms")
    assert p1["gemm_ms"] + p1["stream_ms"] + p1["aux_ms"] <= wall * 1.001 + 0.01
    assert p1["stream_bytes"] >= (256 * 256 + 600 * 2048) * (2 + 8 + 2)   # at least the momentum pass
    assert p2["gemm_launches"] == 2 * p1["gemm_launches"]
    assert p2["gemm_algorithmic_flop"] == pytest.approx(2 * algo, rel=1e-12)
    assert p2["stream_bytes"] == pytest.approx(2 * p1["stream_bytes"], rel=1e-12)


def test_roctx_ranges_leave_results_unchanged(dev, monkeypatch):
    """MUON_ROCTX=1 at handle creation wraps each phase of a call in a ROCTx
    range (rocprofv3 --marker-trace shows them); the results are the bits
    of a handle without them."""
    say("ROCTx phase ranges")
    mats = [gen.custom_matrix(sh, 3400 + i, dev, grad_dtype=torch.bfloat16, weight_dtype=torch.bfloat16)
            for i, sh in enumerate([(600, 2048), (256, 256)])]
    out = {}
    for on in ("0", "1"):
        monkeypatch.setenv("MUON_ROCTX", on)
        h = mu.Handle(dev.index)
        try:
            out[on] = run_update(dev, mats, handle=h)[3:]
        finally:
            h.close()
    for a, b in zip(out["0"], out["1"]):
        for x, y in zip(a, b):
            assert same_bits(x, y)


def same_bits(a, b):
    """Bitwise equality (torch.equal is False wherever a NaN sits)."""
    it = {2: torch.int16, 4: torch.int32}[a.element_size()]
    return a.dtype == b.dtype and torch.equal(a.view(it), b.view(it))


def test_check_finite_flag(dev):
    """MUON_FLAG_CHECK_FINITE: a NaN or Inf in any input (grad, momentum or
    weight of an update; the input of a polar call) makes the call return
    MUON_ERR_NONFINITE naming the first such matrix, with every caller buffer
    as it was; the handle stays usable. Clean inputs give the same bits as
    without the flag. Without the flag a non-finite input reaches only its
    own matrix: the others keep the bits of a clean run."""
    say("non-finite input check")
    shapes = [(300, 700), (640, 257), (256, 256), (33, 517)]
    base = [gen.custom_matrix(sh, 3100 + i, dev, grad_dtype=torch.bfloat16 if i % 2 else torch.float32,
                              weight_dtype=torch.bfloat16 if i % 2 else torch.float32)
            for i, sh in enumerate(shapes)]
    cfg0 = mu.default_config()
    cfgc = mu.make_config(flags=mu.MUON_FLAG_CHECK_FINITE)
    _, _, _, Mr, Vr, Wr = run_update(dev, base, cfg0)
    _, _, _, Mc, Vc, Wc = run_update(dev, base, cfgc)
    for i in range(len(shapes)):
        assert torch.equal(Mc[i], Mr[i]) and torch.equal(Vc[i], Vr[i]) and torch.equal(Wc[i], Wr[i]), i
    # one bad element per case: (matrix, which input, row, col, value); the
    # last rows and columns of ragged matrices and a misaligned view included
    cases = [(1, "g", 639, 256, float("nan")), (0, "m", 0, 0, float("inf")),
             (3, "w", 32, 516, float("-inf")), (2, "g", 128, 77, float("nan"))]
    for mi, which, r, c, val in cases:
        mats = [(g.clone(), m.clone(), w.clone()) for g, m, w in base]
        k = {"g": 0, "m": 1, "w": 2}[which]
        mats[mi][k][r, c] = val
        if mi == 2:   # the grad through a view with a 2-element offset (not 16-byte aligned)
            pad = torch.zeros((256, 258), device=dev, dtype=mats[2][0].dtype)
            pad[:, 2:] = mats[2][0]
            mats[2] = (pad[:, 2:], mats[2][1], mats[2][2])
        before = [(g.clone(), m.clone(), w.clone()) for g, m, w in mats]
        V = [torch.full(g.shape, 7.0, device=dev) for g, _, _ in mats]
        with pytest.raises(mu.LibMuonError) as ei:
            mu.muon_update([g for g, _, _ in mats], [m for _, m, _ in mats], [w for _, _, w in mats], cfgc,
                           update_out=V)
        torch.cuda.synchronize()
        assert ei.value.status == -8 and f"matrix {mi} " in str(ei.value), (which, str(ei.value))
        for (g, m, w), (g0, m0, w0), v in zip(mats, before, V):
            assert same_bits(g, g0) and same_bits(m, m0) and same_bits(w, w0) and bool((v == 7.0).all())
        say(f"  {which}[{mi}] ({r}, {c}) = {val}: refused, nothing written")
    # polar input
    xs = [gen.custom_matrix(sh, 3150 + i, dev)[0] for i, sh in enumerate(shapes[:2])]
    xs[1][5, 250] = float("nan")
    outs = [torch.full(x.shape, 3.0, device=dev) for x in xs]
    with pytest.raises(mu.LibMuonError) as ei:
        mu.ns_polar(xs, outs, cfg=cfgc)
    torch.cuda.synchronize()
    assert ei.value.status == -8 and "matrix 1 " in str(ei.value)
    assert all(bool((o == 3.0).all()) for o in outs)
    # the handle still works; without the flag the NaN stays in its matrix
    mats = [(g.clone(), m.clone(), w.clone()) for g, m, w in base]
    mats[1][0][10, 10] = float("nan")
    _, _, _, Mn, Vn, Wn = run_update(dev, mats, cfg0)
    assert not bool(torch.isfinite(Vn[1]).all())
    for i in (0, 2, 3):
        assert torch.equal(Mn[i], Mr[i]) and torch.equal(Vn[i], Vr[i]) and torch.equal(Wn[i], Wr[i]), i


def test_update_single_fp32_256x1024(dev):
    say("muon_update single_fp32_256x1024")
    g, m, w = gen.make_matrix(gen.WORKLOADS["single_fp32_256x1024"], 0, dev)
    G, M0, W0, M, V, W = run_update(dev, [(g, m, w)])
    check_update("single_fp32", G[0], M0[0], W0[0], M[0], V[0], W[0], mu.default_config(), FP32_TOL)


def test_update_mixed_batch_bf16(dev):
    say("muon_update mixed bf16 batch with ragged shapes")
    shapes = [(512, 256), (256, 512), (384, 384), (300, 129), (129, 300)]
    mats = [gen.custom_matrix(s, 700 + i, dev, grad_dtype=torch.bfloat16, grad_sd=1e-3, mom_sd=1e-3,
                              weight_dtype=torch.bfloat16) for i, s in enumerate(shapes)]
    G, M0, W0, M, V, W = run_update(dev, mats)
    for i in range(len(shapes)):
        check_update(f"mixed[{i}]", G[i], M0[i], W0[i], M[i], V[i], W[i], mu.default_config(), BF16_TOL, ROW_TOL)


def test_update_many_small_matrices(dev):
    """1500 small matrices of 1500 distinct shapes (733 tall, 735 wide, 32
    square, 1 to 48 on a side) in one call: the planner's per-launch block lists and tile lists
    at a batch size far beyond the named workloads, every matrix checked."""
    say("muon_update 1500 small matrices in one call")
    shapes = [(1 + (7 * i) % 48, 1 + (11 * i + 3 + i // 48) % 48) for i in range(1500)]   # 1500 distinct
    mats = [gen.custom_matrix(sh, 5000 + i, dev, weight_sd=1.0) for i, sh in enumerate(shapes)]
    G, M0, W0, M, V, W = run_update(dev, mats)
    cfg = mu.default_config()
    oc = ocfg(cfg)
    worst = 0.0
    for i in range(len(shapes)):
        Mo, Vo, Wo = O.muon_update(f64(G[i]), f64(M0[i]), f64(W0[i]), oc)
        e = rel(f64(V[i]), Vo)
        worst = max(worst, e)
        assert e <= FP32_TOL, (i, shapes[i], e)
        assert rel(f64(M[i]), Mo) <= MOM_TOL, i
        assert weight_add_ok(W0[i], V[i], W[i], cfg), i
    say(f"  worst rel(V) over 1500 matrices {worst:.2e}")


@pytest.mark.parametrize("dtype,tol", [(torch.float32, FP32_TOL), (torch.bfloat16, BF16_TOL)])
def test_update_power_step_forms(dev, dtype, tol):
    """The power step's forms in one call: the fused X^T X v pass for 1 to 6
    chunks of 2048 columns (up to its 12288-column limit), and the X v, X^T u
    kernels for a matrix past that limit and for one with ragged rows."""
    say(f"muon_update power-step forms {dtype}")
    shapes = [(70, 2000), (130, 4000), (70, 6000), (200, 8000), (64, 10000), (96, 12288), (40, 12304), (50, 3001)]
    mats = [gen.custom_matrix(sh, 2100 + i, dev, grad_dtype=dtype, grad_sd=1e-3, mom_sd=1e-3, weight_dtype=dtype)
            for i, sh in enumerate(shapes)]
    G, M0, W0, M, V, W = run_update(dev, mats)
    for i in range(len(shapes)):
        check_update(f"power[{shapes[i]}]", G[i], M0[i], W0[i], M[i], V[i], W[i], mu.default_config(), tol)


def test_update_mixed_dtypes_in_one_call(dev):
    say("muon_update fp32 and bf16 matrices in one call")
    a = gen.custom_matrix((200, 90), 800, dev)
    b = gen.custom_matrix((90, 200), 801, dev, grad_dtype=torch.bfloat16, weight_dtype=torch.bfloat16)
    G, M0, W0, M, V, W = run_update(dev, [a, b])
    check_update("fp32", G[0], M0[0], W0[0], M[0], V[0], W[0], mu.default_config(), FP32_TOL)
    check_update("bf16", G[1], M0[1], W0[1], M[1], V[1], W[1], mu.default_config(), BF16_TOL)


def test_update_floor_forced(dev):
    say("muon_update with the u/w floor firing (W ~ N(0,1))")
    g, m, w = gen.custom_matrix((160, 480), 900, dev, weight_sd=1.0)
    G, M0, W0, M, V, W = run_update(dev, [(g, m, w)])
    check_update("floor", G[0], M0[0], W0[0], M[0], V[0], W[0], mu.default_config(), FP32_TOL)
    ratio = torch.linalg.norm(V[0].double()) / torch.linalg.norm(W0[0].double())
    assert float(ratio) == pytest.approx(0.35, rel=1e-4)


FUSED_TAIL_CASES = {
    "default": dict(), "contra0": dict(contra=0.0), "contra1": dict(contra=1.0), "pp0": dict(pp_iterations=0),
    "ns_steps1": dict(ns_steps=1), "no_weight_floor": dict(target_uw=0.0),
}


@pytest.mark.parametrize("case", list(FUSED_TAIL_CASES))
def test_fused_tail_matches_reduction_pass(dev, monkeypatch, case):
    """bf16 muon_update with the fused tail (||U||^2, <U, X> and the parts of
    sigma = ||X v|| taken in the final product's epilogue, ||W||^2 in the
    momentum pass) against the tail's own reduction pass and last X v
    (MUON_FUSED_TAIL=0, a new handle): the same update up to the float32
    order of those sums, both within the bf16 tolerance of the oracle. Tall,
    wide, square and ragged matrices, one without a weight, one whose floor
    fires (W ~ N(0,1)), and an fp32 matrix (never fused) in the same call."""
    say(f"fused tail against the reduction pass: {case}")
    cfg = mu.default_config()
    for k, v in FUSED_TAIL_CASES[case].items():
        setattr(cfg, k, v)
    shapes = [(384, 200), (200, 520), (256, 256), (130, 61), (61, 130), (96, 300)]
    mats = [gen.custom_matrix(sh, 4400 + i, dev, grad_dtype=torch.bfloat16, grad_sd=1e-3, mom_sd=1e-3,
                              weight_dtype=torch.bfloat16, weight_sd=1.0 if i == 5 else 0.02)
            for i, sh in enumerate(shapes)]
    mats[1] = (mats[1][0], mats[1][1], None)
    mats.append(gen.custom_matrix((90, 200), 4410, dev))
    runs = []
    for fused in ("1", "0"):
        monkeypatch.setenv("MUON_FUSED_TAIL", fused)
        h = mu.Handle(dev.index)
        try:
            runs.append(run_update(dev, mats, cfg=cfg, handle=h))
        finally:
            h.close()
    monkeypatch.delenv("MUON_FUSED_TAIL")
    (G, M0, W0, M, V, W), (_, _, _, Mr, Vr, Wr) = runs
    for i in range(len(mats)):
        d = rel(f64(V[i]), f64(Vr[i]))
        say(f"  [{i}] {tuple(G[i].shape)} {G[i].dtype}: fused vs reduction pass rel(V)={d:.2e}")
        if G[i].dtype == torch.float32:
            assert torch.equal(V[i], Vr[i]) and torch.equal(W[i], Wr[i]), i   # same path either way
        else:
            assert d <= 2e-5, (i, d)
        assert torch.equal(M[i], Mr[i]), i
        tol = FP32_TOL if G[i].dtype == torch.float32 else BF16_TOL
        check_update(f"fused[{i}]", G[i], M0[i], W0[i], M[i], V[i], W[i], cfg, tol)
    if cfg.target_uw > 0:
        ratio = torch.linalg.norm(V[5].double()) / torch.linalg.norm(W0[5].double())
        assert float(ratio) == pytest.approx(float(np.float32(cfg.target_uw)), rel=1e-4)


@pytest.mark.parametrize("case", ["default", "pp0", "classic"])
def test_x0_direct_matches_prologue_copy(dev, monkeypatch, case):
    """bf16 matrices whose sides are multiples of 256 read the stored blended
    update in place of a prologue copy (the default): a tall one's first
    X' = Q X of each pass reads it as X0^T and applies the prologue's scale D
    to its output columns (the prologue writes only X0); a square or wide one
    without the preconditioner reads it as X0 in its pass's first Gram,
    scaled by scale^2 (the prologue writes only X0^T). Against both copies
    written by the prologue (MUON_TALL_X0=0, a new handle) they differ only
    by the copy's bf16 rounding (relative 1e-2 allowed); both are within the
    bf16 tolerance of the oracle. Blocks of four iterations (short side 512
    and 768) and single ones (256), Aurora, plain NS (pp 0) and the classic
    recipe; a wide Aurora matrix is never affected and must agree bit for
    bit."""
    say(f"X0 or X0^T read from the blended update: {case}")
    cfg = mu.make_config("classic") if case == "classic" else mu.default_config()
    if case == "pp0":
        cfg.pp_iterations = 0
    shapes = [(1024, 256), (768, 512), (2048, 768), (512, 1024), (512, 512)]
    mats = [gen.custom_matrix(sh, 4600 + i, dev, grad_dtype=torch.bfloat16, grad_sd=1e-3, mom_sd=1e-3,
                              weight_dtype=torch.bfloat16) for i, sh in enumerate(shapes)]
    runs = []
    for direct in ("1", "0"):
        monkeypatch.setenv("MUON_TALL_X0", direct)
        h = mu.Handle(dev.index)
        try:
            runs.append(run_update(dev, mats, cfg=cfg, handle=h))
        finally:
            h.close()
    monkeypatch.delenv("MUON_TALL_X0")
    (G, M0, W0, M, V, W), (_, _, _, Mr, Vr, Wr) = runs
    for i, sh in enumerate(shapes):
        d = rel(f64(V[i]), f64(Vr[i]))
        say(f"  [{i}] {sh}: direct vs prologue copy rel(V)={d:.2e}")
        if sh[0] >= sh[1] or cfg.pp_iterations == 0:
            assert d <= 1e-2, (i, d)
        else:
            assert torch.equal(V[i], Vr[i]) and torch.equal(W[i], Wr[i]), i
        assert torch.equal(M[i], Mr[i]), i
        check_update(f"x0n[{i}]", G[i], M0[i], W0[i], M[i], V[i], W[i], cfg, BF16_TOL)


OPTIONS = {
    "contra0": dict(contra=0.0), "contra1": dict(contra=1.0), "nesterov0": dict(nesterov=0),
    "pp0": dict(pp_iterations=0), "pp1": dict(pp_iterations=1), "pp3": dict(pp_iterations=3),
    "beta1": dict(pp_beta=1.0), "no_weight_floor": dict(target_uw=0.0), "ns_steps1": dict(ns_steps=1),
    "ns_steps20": dict(ns_steps=20), "power1": dict(power_steps=1), "power9": dict(power_steps=9),
    "mu0": dict(mu=0.0), "mu0p5": dict(mu=0.5), "lr0": dict(lr=0.0),
}


@pytest.mark.parametrize("opt", list(OPTIONS))
def test_update_options(dev, opt):
    """Each configuration field away from its default (pp 1 is the row-
    normalised Muon baseline the Aurora page compares against)."""
    say(f"muon_update option {opt}")
    over = OPTIONS[opt]
    cfg = mu.make_config(**over)
    i = list(OPTIONS).index(opt)
    g, m, w = gen.custom_matrix((260, 140) if i % 2 == 0 else (140, 260), 1000 + i, dev, weight_sd=1.0)
    G, M0, W0, M, V, W = run_update(dev, [(g, m, w)], cfg)
    check_update(opt, G[0], M0[0], W0[0], M[0], V[0], W[0], cfg, FP32_TOL)


@pytest.mark.parametrize("dtype,tol", [(torch.float32, FP32_TOL), (torch.bfloat16, BF16_TOL)])
def test_update_classic_recipe(dev, dtype, tol):
    """The classic five-step Muon recipe through muon_update: momentum from
    the warm-up at step 123, NS5, sqrt(max(1, rows/cols)), lr 0.04, no
    Aurora, Contra or floor."""
    say(f"muon_update classic recipe {dtype}")
    cfg = mu.make_config("classic", mu=mu.momentum_warmup(123))
    shapes = [(384, 128), (128, 384), (256, 256), (300, 77)]
    mats = [gen.custom_matrix(s, 1300 + i, dev, grad_dtype=dtype, grad_sd=1e-3, mom_sd=1e-3, weight_dtype=dtype)
            for i, s in enumerate(shapes)]
    G, M0, W0, M, V, W = run_update(dev, mats, cfg)
    for i in range(len(shapes)):
        check_update(f"classic[{i}]", G[i], M0[i], W0[i], M[i], V[i], W[i], cfg, tol)


@pytest.mark.parametrize("dtype,tol", [(torch.float32, FP32_TOL), (torch.bfloat16, BF16_TOL)])
def test_update_classic_warmup_sequence(dev, dtype, tol):
    """Three consecutive classic steps from a zero buffer at warm-up steps 0,
    100 and 200 (mu 0.85, 0.87, 0.89), the momentum carried in HBM from call
    to call and in float64 by the oracle: the SGD-momentum buffer and each
    step's update against the oracle. The two momentum forms part here (the
    buffer by about 1 / (1 - mu), the direction through the changing mu)."""
    say(f"muon_update classic warm-up sequence {dtype}")
    shapes = [(384, 128), (128, 384), (256, 256)]
    mats = [gen.custom_matrix(s, 1900 + i, dev, grad_dtype=dtype, grad_sd=1e-3, weight_dtype=dtype)
            for i, s in enumerate(shapes)]
    M = [torch.zeros(s, device=dev) for s in shapes]
    W = [w.clone() for _, _, w in mats]
    Mo = [np.zeros(s) for s in shapes]
    Me = [np.zeros(s) for s in shapes]        # the moving-average form, for contrast
    for k, step in enumerate((0, 100, 200)):
        cfg = mu.make_config("classic", mu=mu.momentum_warmup(step))
        assert cfg.flags == mu.MUON_FLAG_SGD_MOMENTUM
        G = [gen.custom_matrix(s, 1950 + 10 * k + i, dev, grad_dtype=dtype, grad_sd=1e-3)[0]
             for i, s in enumerate(shapes)]
        W0 = [w.clone() for w in W]
        V = [torch.empty(s, device=dev) for s in shapes]
        mu.muon_update(G, M, W, cfg, update_out=V)
        torch.cuda.synchronize()
        oc = ocfg(cfg)
        for i in range(len(shapes)):
            Mo[i], Vo, _ = O.muon_update(f64(G[i]), Mo[i], f64(W0[i]), oc)
            Me[i], _ = O.momentum_step(f64(G[i]), Me[i], oc.mu, True, "ema")
            e_v, e_m, e_ema = rel(f64(V[i]), Vo), rel(f64(M[i]), Mo[i]), rel(f64(M[i]), Me[i])
            say(f"  step {step} {shapes[i]}: rel(V)={e_v:.2e} rel(M)={e_m:.2e}")
            assert e_v <= tol and e_m <= MOM_TOL and e_ema > 0.1
            assert weight_add_ok(W0[i], V[i], W[i], cfg)
            weight_vs_oracle(f"warmup{step}[{i}]", W0[i], W[i], V[i], Vo, cfg)


@pytest.mark.parametrize("dtype,tol", [(torch.float32, FP32_TOL), (torch.bfloat16, BF16_TOL)])
def test_aurora_wide_rows_option(dev, dtype, tol):
    """MUON_FLAG_WIDE_ROWS: a wide matrix equilibrated on its own rows
    (target 1), tall and square ones as before; through aurora_orthogonalize
    (pp 1, 2, 3) and muon_update, with ragged and multi-tile shapes."""
    say(f"aurora on a wide matrix's own rows, {dtype}")
    shapes = [(100, 700), (300, 1030), (700, 100), (256, 256), (33, 517)]
    xs = [gen.custom_matrix(s, 2600 + i, dev, grad_dtype=dtype, grad_sd=1e-3)[0] for i, s in enumerate(shapes)]
    for pp in (1, 2, 3):
        cfg = mu.make_config(pp_iterations=pp, flags=mu.MUON_FLAG_WIDE_ROWS)
        outs = mu.aurora_orthogonalize(xs, [torch.empty(x.shape, device=dev) for x in xs], cfg=cfg)
        torch.cuda.synchronize()
        for x, u in zip(xs, outs):
            want = O.aurora_orthogonalize(f64(x), pp, 0.5, wide_rows=True)
            e = rel(f64(u), want)
            say(f"  pp={pp} {tuple(x.shape)} rel={e:.2e}")
            assert e <= tol
            if x.shape[0] < x.shape[1] and pp == 1:
                # not the default (column) equilibration: much farther from it
                # than from the wide-row oracle
                assert rel(f64(u), O.aurora_orthogonalize(f64(x), 1, 0.5)) > max(2 * tol, 10 * e)
    cfg = mu.make_config(flags=mu.MUON_FLAG_WIDE_ROWS)
    mats = [gen.custom_matrix(s, 2650 + i, dev, grad_dtype=dtype, grad_sd=1e-3, mom_sd=1e-3, weight_dtype=dtype)
            for i, s in enumerate(shapes)]
    G, M0, W0, M, V, W = run_update(dev, mats, cfg)
    for i in range(len(shapes)):
        check_update(f"wide_rows[{i}]", G[i], M0[i], W0[i], M[i], V[i], W[i], cfg, tol)


def test_fp8_first_gram_option(dev):
    """MUON_FLAG_FP8_GRAM (research option): the first Gram of each pass of
    bf16 matrices that run blocks reads an fp8 copy of X0. Against the oracle
    at the bf16 bar (row norms too); against the same call without the option
    it differs (fp8 was used) by about the bf16 rounding level; fp32 and
    square matrices, which do not take it, are bitwise unchanged."""
    say("fp8 first Gram option")
    shapes = [(600, 2048), (2048, 600), (520, 1030), (512, 512)]
    cfg8 = mu.make_config(flags=mu.MUON_FLAG_FP8_GRAM)
    cfg0 = mu.default_config()
    mats = [gen.custom_matrix(sh, 2900 + i, dev, grad_dtype=torch.bfloat16, grad_sd=1e-3, mom_sd=1e-3,
                              weight_dtype=torch.bfloat16) for i, sh in enumerate(shapes)]
    mats.append(gen.custom_matrix((300, 700), 2950, dev))          # fp32: not taken
    G, M0, W0, M8, V8, W8 = run_update(dev, mats, cfg8)
    _, _, _, M0b, V0, W0b = run_update(dev, mats, cfg0)
    for i, sh in enumerate(shapes + [(300, 700)]):
        tol = BF16_TOL if i < len(shapes) else FP32_TOL
        check_update(f"fp8gram[{sh}]", G[i], M0[i], W0[i], M8[i], V8[i], W8[i], cfg8, tol,
                     ROW_TOL if i < len(shapes) else None)
        d = rel(f64(V8[i]), f64(V0[i]))
        say(f"  {sh}: rel(fp8 option vs without) = {d:.2e}")
        if i < 3:
            assert 0 < d < 2e-2, (sh, d)
        else:
            assert torch.equal(V8[i], V0[i]), sh                 # square / fp32: unchanged
    for name, fn, ref in (("ns_polar", mu.ns_polar, lambda x: O.newton_schulz(x)),
                          ("aurora", mu.aurora_orthogonalize, lambda x: O.aurora_orthogonalize(x))):
        xs = [gen.custom_matrix(sh, 2960 + i, dev, grad_dtype=torch.bfloat16, grad_sd=1e-3)[0]
              for i, sh in enumerate(shapes[:3])]
        outs = fn(xs, [torch.empty(x.shape, device=dev) for x in xs], cfg=cfg8)
        torch.cuda.synchronize()
        for x, o in zip(xs, outs):
            want = ref(f64(x))
            e, r = rel(f64(o), want), row_agree(f64(o), want)
            say(f"  {name} {tuple(x.shape)} fp8 first Gram: rel={e:.2e} rows={r:.2e}")
            assert e <= BF16_TOL and r <= ROW_TOL


def test_overlapping_rows_rejected(dev):
    """An expanded momentum (stride(0) = 0: every row the same memory) is
    rejected before anything is enqueued and stays untouched."""
    say("muon_update rejects a momentum whose rows overlap")
    g, m, w = gen.custom_matrix((64, 96), 2700, dev)
    row = torch.full((1, 96), 0.25, device=dev)
    with pytest.raises(mu.LibMuonError) as ei:
        mu.muon_update([g], [row.expand(64, 96)], [w])
    assert ei.value.status == -3, str(ei.value)
    with pytest.raises(mu.LibMuonError) as ei:
        mu.ns_polar([g], [torch.zeros(1, 96, device=dev).expand(64, 96)])
    assert ei.value.status == -3
    torch.cuda.synchronize()
    assert bool((row == 0.25).all())


# ---------------------------------------------------------------------------
# size limits: long side 65536, short side 16384, 2^30 elements
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape,dtype,tol", [((256, 65536), torch.bfloat16, BF16_TOL),
                                             ((65536, 256), torch.float32, FP32_TOL)])
def test_update_max_long_side(dev, shape, dtype, tol):
    """The full step at the longest side the library accepts, dense random
    inputs, every element checked against the oracle."""
    say(f"muon_update at the long-side limit {shape} {dtype}")
    mats = [gen.custom_matrix(shape, 1400, dev, grad_dtype=dtype, grad_sd=1e-3, mom_sd=1e-3, weight_dtype=dtype)]
    G, M0, W0, M, V, W = run_update(dev, mats)
    check_update("max_long", G[0], M0[0], W0[0], M[0], V[0], W[0], mu.default_config(), tol, ROW_TOL)


def test_ns_polar_max_short_side_and_elements(dev):
    """ns_polar on a 16384 x 65536 bf16 matrix (short-side limit, 2^30
    elements) with one nonzero v_i per row in distinct columns: X = D P with
    D diagonal and P a partial permutation, so every Gram is diagonal and the
    exact result keeps the support, with values sign(v_i) p^12(|v_i| / (||v|| + 1e-7))."""
    rows, cols = 16384, 65536
    say(f"ns_polar at the short-side / element limit {rows}x{cols} bf16")
    gcpu = torch.Generator().manual_seed(1500)
    col = torch.randperm(cols, generator=gcpu)[:rows]
    mag = torch.pow(10.0, -3.0 * torch.rand(rows, generator=gcpu, dtype=torch.float64))
    sgn = torch.where(torch.rand(rows, generator=gcpu) < 0.5, -1.0, 1.0).double()
    v = (sgn * mag).to(torch.bfloat16)                      # stored values are the ground truth
    x = torch.zeros((rows, cols), device=dev, dtype=torch.bfloat16)
    ridx = torch.arange(rows, device=dev)
    x[ridx, col.to(dev)] = v.to(dev)
    out = torch.empty_like(x)
    mu.ns_polar([x], [out])
    torch.cuda.synchronize()
    del x
    # support kept exactly
    nz = int(torch.count_nonzero(out))
    got = out[ridx, col.to(dev)].double().cpu().numpy()
    assert nz == rows and bool((got != 0).all()), nz
    # closed form on the support
    vv = v.double().numpy()
    t = np.abs(vv) / (np.linalg.norm(vv) + 1e-7)
    for _ in range(12):
        t = 2.0 * t - 1.5 * t ** 3 + 0.5 * t ** 5
    want = np.sign(vv) * t
    e_f = rel(got, want)
    e_max = float(np.max(np.abs(got - want) / np.abs(want)))
    say(f"  rel(Frobenius)={e_f:.2e} max elementwise rel={e_max:.2e}")
    assert e_f <= BF16_TOL and e_max <= 5e-2


def test_update_zero_and_empty(dev):
    say("muon_update zero and empty matrices")
    z = torch.zeros((64, 200), device=dev)
    wz = torch.full((64, 200), 0.5, device=dev)
    e = torch.zeros((0, 5), device=dev)
    G, M0, W0, M, V, W = run_update(dev, [(z, z.clone(), wz), (e, e.clone(), e.clone())])
    assert bool(torch.isfinite(V[0]).all()) and float(V[0].abs().max()) == 0.0
    assert torch.equal(W[0], wz) and float(M[0].abs().max()) == 0.0


def test_update_power_restart(dev):
    """Rows summing to zero: the all-ones start vector is annihilated and the
    power iteration restarts from the largest column."""
    say("muon_update power-iteration restart")
    base = torch.tensor([[1.0, -1.0, 0.0, 0.0], [2.0, 0.0, -2.0, 0.0], [0.0, 3.0, 0.0, -3.0],
                         [1.0, 1.0, -1.0, -1.0], [0.0, 0.0, 4.0, -4.0], [2.0, -1.0, -1.0, 0.0]])
    g = base.repeat(1, 16).to(dev)              # 6 x 64, every row sums to zero
    m = torch.zeros_like(g)
    w = 0.02 * torch.ones_like(g)
    G, M0, W0, M, V, W = run_update(dev, [(g, m, w)])
    check_update("restart", G[0], M0[0], W0[0], M[0], V[0], W[0], mu.default_config(), FP32_TOL)


def test_update_resume_equals_uninterrupted(dev):
    """The library keeps no state between calls: two steps on one handle equal
    step 1, momentum and weights saved to the host, a fresh handle, the state
    restored and step 2, bit for bit."""
    say("muon_update: step k, save, reload, step k+1 == uninterrupted")
    shapes = [(300, 140), (140, 300), (256, 256)]
    first = [gen.custom_matrix(sh, 2400 + i, dev, grad_dtype=torch.bfloat16, grad_sd=1e-3, mom_sd=1e-3,
                               weight_dtype=torch.bfloat16) for i, sh in enumerate(shapes)]
    second = [gen.custom_matrix(sh, 2500 + i, dev, grad_dtype=torch.bfloat16, grad_sd=1e-3)[0]
              for i, sh in enumerate(shapes)]
    g1 = [g for g, _, _ in first]
    # uninterrupted: both steps on one handle
    h = mu.Handle(dev.index)
    try:
        M = [m.clone() for _, m, _ in first]
        W = [w.clone() for _, _, w in first]
        V = [torch.empty(sh, device=dev) for sh in shapes]
        mu.muon_update(g1, M, W, update_out=V, handle=h)
        mu.muon_update(second, M, W, update_out=V, handle=h)
        torch.cuda.synchronize()
    finally:
        h.close()
    # interrupted: step 1, save to the host, new handle, restore, step 2
    ha = mu.Handle(dev.index)
    try:
        Ma = [m.clone() for _, m, _ in first]
        Wa = [w.clone() for _, _, w in first]
        mu.muon_update(g1, Ma, Wa, handle=ha)
        torch.cuda.synchronize()
        saved = ([t.cpu() for t in Ma], [t.cpu() for t in Wa])
    finally:
        ha.close()
    del Ma, Wa
    hb = mu.Handle(dev.index)
    try:
        Mb = [t.to(dev) for t in saved[0]]
        Wb = [t.to(dev) for t in saved[1]]
        Vb = [torch.empty(sh, device=dev) for sh in shapes]
        mu.muon_update(second, Mb, Wb, update_out=Vb, handle=hb)
        torch.cuda.synchronize()
    finally:
        hb.close()
    for i in range(len(shapes)):
        assert torch.equal(M[i], Mb[i]), i
        assert torch.equal(W[i], Wb[i]), i
        assert torch.equal(V[i], Vb[i]), i


def test_update_deterministic(dev):
    say("muon_update bitwise determinism")
    mats = [gen.custom_matrix(s, 1100 + i, dev, grad_dtype=torch.bfloat16, weight_dtype=torch.bfloat16)
            for i, s in enumerate([(300, 500), (512, 512)])]
    r1 = run_update(dev, mats)
    r2 = run_update(dev, mats)
    for a, b in zip(r1[4] + r1[3] + r1[5], r2[4] + r2[3] + r2[5]):
        assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# the named workloads, in the configuration the benchmark times
# ---------------------------------------------------------------------------
def _workload_run(dev, name, sample, big_oracle=()):
    w = gen.WORKLOADS[name]
    cfg = mu.make_config(**dict(w.config))
    grads, moms, weights = gen.make_batch(name, dev)
    say(f"workload {name}: {len(grads)} matrices")
    mats = list(zip(grads, moms, weights if weights is not None else [None] * len(grads)))
    G, M0, W0, M, V, W = run_update(dev, mats, cfg, out_dtype=torch.float32)
    # elementwise outputs the oracle computes one by one: momentum on sampled
    # rows of every matrix; every update finite; W' = round(W - lr V) exactly
    for i in range(len(G)):
        r = G[i].shape[0]
        rows = sorted({0, r // 3, r // 2, r - 1})
        mo, _ = O.momentum_nesterov(f64(G[i][rows]), f64(M0[i][rows]), float(np.float32(cfg.mu)),
                                    bool(cfg.nesterov))
        assert rel(f64(M[i][rows]), mo) <= MOM_TOL, i
        assert bool(torch.isfinite(V[i]).all()), i
        if W0[i] is not None:
            assert weight_add_ok(W0[i], V[i], W[i], cfg), i
    # whole-matrix oracle on a sample
    for i in list(sample) + list(big_oracle):
        check_update(f"{name}[{i}]", G[i], M0[i], W0[i], M[i], V[i], W[i], cfg, BF16_TOL, ROW_TOL)
    return cfg, grads, moms, weights, V


def test_workload_ns_48x768sq(dev):
    _workload_run(dev, "ns_48x768sq_bf16", sample=[0, 17, 47])


def test_workload_gpt2_124m(dev):
    _workload_run(dev, "gpt2_124m_matrices", sample=[0, 4, 5, 70, 71])


def test_workload_llama3p8b_layer(dev):
    # every matrix of the layer against the oracle: q, o (3072^2, square
    # short-circuit), k, v (1024x3072), up (12288x3072) and down (3072x12288,
    # wide, at the fused power pass's 12288-column limit)
    _workload_run(dev, "llama3p8b_layer", sample=[1, 2], big_oracle=[0, 3, 4, 5])


def test_workload_llama3p8b_all_layers(dev):
    # one matrix of each shape against the oracle, from layers 0, 13 and 27:
    # k (1), q (78), up (82), k (164), down (167)
    cfg, grads, moms, weights, V = _workload_run(dev, "llama3p8b_all_layers", sample=[1, 164],
                                                 big_oracle=[78, 82, 167])
    # batching independence: a matrix run alone gives the same bits as inside the 168-matrix batch
    w = gen.WORKLOADS["llama3p8b_all_layers"]
    for i in (0, 101, 167):
        g, m, wt = gen.make_matrix(w, i, dev)
        v = torch.empty(g.shape, device=dev)
        mu.muon_update([g], [m], [wt], cfg, update_out=[v])
        torch.cuda.synchronize()
        say(f"  batch independence [{i}] {tuple(g.shape)}")
        assert torch.equal(v, V[i]), i
