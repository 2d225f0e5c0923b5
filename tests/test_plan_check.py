"""Host-only checks of the planner's launch plans (libmuon
`muon_debug_check_plan`, no device needed): every workspace region inside
the workspace and disjoint from the others, every Newton-Schulz product tile
inside its matrix's padded tile grid and in the list of that matrix's pass,
chain and element type, every tile a product needs listed exactly once,
each chain's matrices of one block length, and consistent streaming lists.
Edge shapes, the named workloads, and seeded random batches over the shape
space the library accepts, every call kind, and the options that change
plans: Aurora pass count, wide rows, the fp8 first Gram, and a forced block
length or tile edge."""
import os
import random

import pytest
import torch

import muon_newton_schulz_update_amd as mu

EDGE = [(1, 1), (1, 7), (7, 1), (5, 5), (33, 517), (517, 33), (255, 257), (256, 256), (257, 256),
        (511, 2048), (512, 2048), (513, 2047), (768, 768), (1024, 3072), (3072, 12288), (12288, 3072),
        (16384, 65536), (65536, 16384), (65536, 256), (1, 65536), (65536, 1), (0, 5), (5, 0)]
KINDS = ("update", "polar", "aurora")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mu.library_path()):
        pytest.skip("libmuon.so not built")
    return mu.load_library()


def check(kind, shapes, cfg=None):
    rc, msg = mu.debug_check_plan(kind, shapes, cfg)
    assert rc == 0, (kind, shapes[:6], msg)


def test_edge_shapes_alone_and_together(lib):
    for kind in KINDS:
        for dt in (torch.float32, torch.bfloat16):
            for r, c in EDGE:
                check(kind, [(r, c, dt)])
            check(kind, [(r, c, dt) for r, c in EDGE])
        check(kind, [(r, c, dt) for r, c in EDGE for dt in (torch.float32, torch.bfloat16)])
        check(kind, [])


def test_named_workloads(lib):
    """The benchmark's shape sets, and sets of 3072 x 3072 squares alone and
    beside a few blocked rectangles (lists of thousands of 256-tiles)."""
    from muon_newton_schulz_update_amd import inputs as gen
    for name, w in gen.WORKLOADS.items():
        dt = w.grad_dtype
        check("update", [(r, c, dt) for r, c in w.shapes])
    check("polar", [(3072, 3072, torch.bfloat16)] * 56)
    check("update", [(3072, 3072, torch.bfloat16)] * 56 + [(3072, 12288, torch.bfloat16)] * 3)


def rand_shape(rng):
    u = rng.random()
    if u < 0.3:
        return rng.randint(1, 64), rng.randint(1, 64)
    if u < 0.6:
        return rng.randint(1, 2048), rng.randint(1, 2048)
    if u < 0.85:
        r, c = rng.randint(256, 4096), rng.randint(256, 16384)
        return (r, c) if rng.random() < 0.5 else (c, r)
    return rng.choice(EDGE)


def test_random_batches_and_options(lib, monkeypatch):
    rng = random.Random(20261203)
    for trial in range(300):
        monkeypatch.delenv("MUON_NS_TILE", raising=False)
        monkeypatch.delenv("MUON_NS_BLOCK", raising=False)
        if rng.random() < 0.3:
            monkeypatch.setenv("MUON_NS_TILE", rng.choice(["128", "256"]))
        if rng.random() < 0.3:
            monkeypatch.setenv("MUON_NS_BLOCK", str(rng.randint(1, 8)))
        flags = 0
        if rng.random() < 0.3:
            flags |= mu.MUON_FLAG_WIDE_ROWS
        if rng.random() < 0.3:
            flags |= mu.MUON_FLAG_FP8_GRAM
        cfg = mu.make_config("classic" if rng.random() < 0.15 else "aurora", flags=flags,
                             pp_iterations=rng.choice([0, 1, 2, 3]))
        shapes = [(*rand_shape(rng), rng.choice([torch.float32, torch.bfloat16]))
                  for _ in range(rng.randint(1, 40))]
        check(rng.choice(KINDS), shapes, cfg)


def test_rejects_shapes_past_the_limits(lib):
    for bad in [(16385, 65536), (65537, 8), (8, 65537)]:
        rc, _ = mu.debug_check_plan("update", [(*bad, torch.float32)])
        assert rc == -3, bad
