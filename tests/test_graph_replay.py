"""GPU: the three entry points captured in one HIP graph (torch.cuda.graph), replayed several times
with eager work and synchronizations between the replays; every replay must equal the eager
result bit for bit (the kernels are deterministic and use no memset), and the eager result is
checked against the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def pe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vlm_vision_patch_amd
    return vlm_vision_patch_amd


def make(seed, shape, dtype, dist="normal", bound=1.0):
    return workloads.random_tensor(shape, seed=seed, dtype=dtype, dist=dist, bound=bound)


def test_graph_replays_match_eager(pe):
    print("[case] graph replay: PatchEmbed (split-k and large tiles), fused add, merger LayerNorm", flush=True)
    P, E = 14, 1280
    K = 3 * 2 * P * P
    w = make(5000, (E, 3, 2, P, P), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    b = make(5001, (E,), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    x1 = make(5002, (1, 3, 16 * P, 64 * P), torch.bfloat16)      # one image, 1024 patches
    x2 = make(5003, (8, 3, 32 * P, 32 * P), torch.bfloat16)      # 8 images, 8192 patches
    g1, g2 = [[1, 16, 64]], [[1, 32, 32]] * 8
    pos = (make(5004, (1024, E), torch.float32) * 0.02).to(torch.bfloat16)
    gam = (1 + 0.1 * make(5005, (E,), torch.float32)).to(torch.bfloat16)
    bet = (0.1 * make(5006, (E,), torch.float32)).to(torch.bfloat16)
    mod = pe.PatchEmbed(w.to(DEV), b.to(DEV), order="merge")
    d1, d2, dpos = x1.to(DEV), x2.to(DEV), pos.to(DEV)
    dg, db = gam.to(DEV), bet.to(DEV)
    o1 = torch.empty(1024, E, dtype=torch.bfloat16, device=DEV)
    o2 = torch.empty(8192, E, dtype=torch.bfloat16, device=DEV)
    o3 = torch.empty(1024, E, dtype=torch.bfloat16, device=DEV)
    y = torch.empty(8192, E, dtype=torch.bfloat16, device=DEV)

    def step():
        mod(d1, g1, [1], out=o1)
        mod(d2, g2, [1] * 8, out=o2)
        mod(d1, g1, [1], out=o3, add=dpos)
        pe.layer_norm(o2, dg, db, 1e-6, out=y)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (o1, o2, o3, y)]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for rep in range(4):
        for t in (o1, o2, o3, y):
            t.fill_(float("nan"))            # eager work between replays; replays must rewrite it all
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, e in zip(("image", "batch", "add", "layernorm"), (o1, o2, o3, y), eager):
            assert torch.equal(t, e), "replay %d: %s differs from the eager result" % (rep, name)
    del g
    mod.close()

    # the eager results themselves, against the oracle
    r1 = oracle.forward(x1, w, b, grid=g1, frames=[1], order="merge")
    r3 = oracle.forward(x1, w, b, grid=g1, frames=[1], order="merge", addend=pos)
    for got, ref, what in ((eager[0], r1, "image"), (eager[2], r3, "add")):
        gd = got.double().cpu().numpy()
        assert np.all(np.abs(gd - ref) <= 1e-3 + 1e-2 * np.abs(ref)), what
    rows = np.arange(0, 8192, 97)
    r2 = oracle.forward(x2, w, b, grid=g2, frames=[1] * 8, order="merge", rows=rows)
    gd = eager[1][torch.as_tensor(rows, device=DEV)].double().cpu().numpy()
    assert np.all(np.abs(gd - r2) <= 1e-3 + 1e-2 * np.abs(r2)), "batch"
    # (the LayerNorm's parity against the oracle is in test_layernorm_parity.py)
