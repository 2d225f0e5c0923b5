"""muon_update_static (the entry point that allocates nothing) against
muon_update through the C ABI: identical results on two calls in a row, the
second with a smaller batch; the oracle bar on each; a batch beyond the
static scratch rejected before anything runs; no device allocation."""
import numpy as np
import pytest
import torch

import muon_newton_schulz_update_amd as mu
from muon_newton_schulz_update_amd import inputs as gen
from oracle import muon_oracle as O

from test_gpu_parity import BF16_TOL, FP32_TOL, ROW_TOL, check_update, f64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _pair(dev, mats, cfg, h):
    """The same batch through muon_update and muon_update_static on fresh
    copies of the state; returns both results and the originals."""
    G = [g for g, _, _ in mats]
    M0 = [m.clone() for _, m, _ in mats]
    W0 = [w.clone() for _, _, w in mats]
    out = []
    for fn in (mu.muon_update, mu.muon_update_static):
        M = [m.clone() for m in M0]
        W = [w.clone() for w in W0]
        V = [torch.empty(g.shape, device=dev) for g in G]
        fn(G, M, W, cfg, update_out=V, handle=h)
        torch.cuda.synchronize()
        out.append((M, V, W))
    return G, M0, W0, out


def test_static_entry_point_matches_muon_update(dev):
    say("muon_update_static vs muon_update, two calls in a row (the second smaller)")
    h = mu.Handle(dev.index)
    try:
        cfg = mu.default_config()
        calls = [
            [((384, 130), torch.bfloat16, 1), ((130, 600), torch.float32, 2), ((256, 256), torch.bfloat16, 3),
             ((1024, 768), torch.bfloat16, 4)],
            [((96, 200), torch.float32, 5), ((64, 64), torch.bfloat16, 6)],
        ]
        for k, batch in enumerate(calls):
            mats = [gen.custom_matrix(sh, 3000 + 10 * k + i, dev, grad_dtype=dt, grad_sd=1e-3, mom_sd=1e-3,
                                      weight_dtype=dt) for sh, dt, i in batch]
            G, M0, W0, ((Ma, Va, Wa), (Ms, Vs, Ws)) = _pair(dev, mats, cfg, h)
            for i, (sh, dt, _) in enumerate(batch):
                assert torch.equal(Ma[i], Ms[i]) and torch.equal(Va[i], Vs[i]) and torch.equal(Wa[i], Ws[i]), \
                    (k, sh)
                tol = BF16_TOL if dt == torch.bfloat16 else FP32_TOL
                check_update(f"static call {k} {sh}", G[i], M0[i], W0[i], Ms[i], Vs[i], Ws[i], cfg, tol,
                             ROW_TOL if dt == torch.bfloat16 else None)
    finally:
        h.close()


def test_static_entry_point_allocates_nothing_and_rejects_large(dev):
    say("muon_update_static: device free memory unchanged; too-large batch rejected")
    h = mu.Handle(dev.index)
    try:
        warm = [gen.custom_matrix((64, 96), 3100, dev)]
        mu.muon_update_static([g for g, _, _ in warm], [m for _, m, _ in warm], [w for _, _, w in warm], handle=h)
        torch.cuda.synchronize()
        mats = [gen.custom_matrix((300, 200), 3101, dev), gen.custom_matrix((200, 512), 3102, dev)]
        G = [g for g, _, _ in mats]
        M = [m for _, m, _ in mats]
        W = [w for _, _, w in mats]
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info(dev)[0]
        mu.muon_update_static(G, M, W, handle=h)        # new shapes: a new plan, no workspace growth
        torch.cuda.synchronize()
        free1 = torch.cuda.mem_get_info(dev)[0]
        assert free1 == free0, (free0, free1)
        # beyond the 64 MiB scratch: rejected, nothing written
        g, m, w = gen.custom_matrix((3072, 12288), 3103, dev, grad_dtype=torch.bfloat16, weight_dtype=torch.bfloat16)
        m0, w0 = m.clone(), w.clone()
        with pytest.raises(mu.LibMuonError) as ei:
            mu.muon_update_static([g], [m], [w], handle=h)
        assert ei.value.status == -7 and "static scratch" in str(ei.value), str(ei.value)
        torch.cuda.synchronize()
        assert torch.equal(m, m0) and torch.equal(w, w0)
    finally:
        h.close()
