"""The decode layer replayed from a captured HIP graph reproduces eager
execution bit for bit on every replay (the layer records no memset nodes: its
accumulators are cleared by a fill kernel). Replays are interleaved with
eager work and synchronisations. The forward pass is deterministic: split
partial sums are added in split order, so repeated steps on the same inputs
give identical bits."""
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
    for i in range(4):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.float(), eager), (i, (y.float() - eager).abs().max().item())
        # eager work between replays
        layer.forward(x, ck, cv, past, y=y, ws=ws)
        torch.cuda.synchronize()


def test_decode_step_is_bitwise_repeatable():
    """Full 8B decode step (batch 16, 1025 positions): the GEMVs split K and
    attention splits the context, and the last arriving workgroup adds the
    partials in split order; two steps on the same inputs must agree bit for
    bit (y and the f32 residual stream x2), as must the appended cache rows."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rank_decomposed_linear_amd import binding
    from rank_decomposed_linear_amd import workloads as W
    w = W.LLAMA3_8B_C40_DECODE
    print(f"{w.name}: two steps on the same inputs", flush=True)
    weights, inp = W.draw(w)
    shp = w.shape
    facs = {p: (to_dev(W.to_library_factor(a)), to_dev(W.to_library_factor(b)))
            for p, (a, b) in weights.factors.items()}
    layer = binding.DecomposedLayer(facs, shp.hidden, shp.n_q, shp.n_kv, shp.head_dim, shp.ffn,
                                    shp.rope_theta, shp.rms_eps)
    x = to_dev(inp.x)
    ck = to_dev(W.to_library_key_cache(inp.ck))
    cv = to_dev(W.to_library_value_cache(inp.cv))
    past = to_dev(inp.past_lens)
    outs = []
    for _ in range(3):
        x2 = torch.empty(inp.x.shape, dtype=torch.float32, device="cuda:0")
        y = layer.forward(x, ck, cv, past, x2_out=x2)
        torch.cuda.synchronize()
        outs.append((y.clone(), x2.clone(), ck.clone(), cv.clone()))
    for i in (1, 2):
        for a, b, nm in zip(outs[0], outs[i], ("y", "x2", "ck", "cv")):
            assert torch.equal(a, b), (i, nm)
