"""The decode layer replayed from a captured HIP graph matches eager
execution on every replay (the layer records no memset nodes: its
accumulators are cleared by a fill kernel). Replays are interleaved with
eager work and synchronisations."""
import numpy as np
import pytest

from tests._helpers import rand, to_dev

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rank_decomposed_linear_amd import binding
    from rank_decomposed_linear_amd import workloads as W
    r = np.random.Generator(np.random.PCG64(11))
    ranks = {"q": 192, "k": 128, "v": 128, "o": 192, "gate": 256, "up": 256, "down": 256}
    shp = W.LayerShape(512, 8, 2, 128, 1024, tuple((p, ranks[p]) for p in W.PROJECTIONS), "bf16",
                       500000.0)
    # factors and caches drawn directly in the library's storage (transposed,
    # operand tiles): random values in any order are random values
    facs = {p: (to_dev(rand(r, (shp.rank(p), m), 0.05, "bf16")),
                to_dev(rand(r, (n, shp.rank(p)), 0.05, "bf16")))
            for p, (m, n) in shp.shapes().items()}
    layer = binding.DecomposedLayer(facs, shp.hidden, shp.n_q, shp.n_kv, shp.head_dim, shp.ffn,
                                    shp.rope_theta)
    Bsz, L_max = 16, 320
    x = to_dev(rand(r, (Bsz, 1, 512), 1.0, "bf16"))
    ck = to_dev(rand(r, (Bsz, L_max, 128), 1.0, "bf16"))
    cv = to_dev(rand(r, (Bsz, 128, L_max), 1.0, "bf16"))
    past = to_dev(np.array(r.integers(0, L_max - 1, size=Bsz), np.int32))
    ws = torch.empty(layer.workspace_bytes(Bsz, 1, L_max), dtype=torch.uint8, device="cuda:0")
    y = torch.empty_like(x)
    layer.forward(x, ck, cv, past, y=y, ws=ws)
    torch.cuda.synchronize()
    eager = y.float().clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(x, ck, cv, past, y=y, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x, ck, cv, past, y=y, ws=ws)
    scale = eager.abs().max().item()
    for i in range(4):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        err = (y.float() - eager).abs().max().item()
        assert err <= 1e-2 * scale, (i, err)
        # eager work between replays
        layer.forward(x, ck, cv, past, y=y, ws=ws)
        torch.cuda.synchronize()
