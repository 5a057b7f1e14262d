"""dl_lowrank_linear_static (the allocation-free variant of
dl_lowrank_linear, whose workspace is the library's static device scratch)
against dl_lowrank_linear with a caller workspace, through the C ABI: the
same kernels on the same plan, so the outputs must agree bit for bit. Two
calls in a row per path, the second on a smaller input, so the second call
runs on scratch left over from the first; both are also compared with the
fp64 oracle. Sizes beyond the scratch are rejected before any device work."""
import numpy as np
import pytest

from oracle import ref
from rank_decomposed_linear_amd import workloads as W
from tests._helpers import TOL, f64, rand, relerr, to_dev, to_host

pytestmark = pytest.mark.gpu

# (name, dtype, m, k, n, M first call, M second call): the GEMV path (M <= 64,
# split-K partials and counters in the scratch), the GEMM path (bf16
# intermediate in the scratch) and the f32 path
CASES = [
    ("gemv_bf16", "bf16", 1024, 512, 2048, 48, 8),
    ("gemm_bf16", "bf16", 512, 256, 640, 300, 130),
    ("f32", "f32", 40, 24, 56, 5, 3),
]


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from rank_decomposed_linear_amd import binding
    binding.load()
    return binding


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_static_scratch_matches_caller_workspace(B, case):
    import torch
    name, dt, m, k, n, M1, M2 = case
    r = np.random.Generator(np.random.PCG64(sum(map(ord, name))))
    A = rand(r, (m, k), 0.05, dt)
    Bf = rand(r, (k, n), 0.05, dt)
    At, Bt = to_dev(W.to_library_factor(A)), to_dev(W.to_library_factor(Bf))
    for M in (M1, M2):
        print(f"static scratch {name}: M={M} m={m} k={k} n={n}", flush=True)
        x = rand(r, (M, m), 1.0, dt)
        xd = to_dev(x)
        y_static = B.lowrank_linear_static(xd, At, Bt)
        y_ws = B.lowrank_linear(xd, At, Bt)
        torch.cuda.synchronize()
        assert torch.equal(y_static, y_ws), (name, M)
        want = ref.lowrank_linear(f64(x), f64(A), f64(Bf))
        assert relerr(to_host(y_static), want) <= TOL[dt], (name, M)


def test_static_scratch_rejects_oversize(B):
    import torch
    from rank_decomposed_linear_amd import binding
    M, m, k, n = 4096, 4096, 4096, 64
    need = binding.load().dl_lowrank_linear_workspace(M, m, k, n, binding.DL_BF16)
    assert need > binding.STATIC_SCRATCH_BYTES
    x = torch.zeros((M, m), dtype=torch.bfloat16, device="cuda:0")
    At = torch.zeros((k, m), dtype=torch.bfloat16, device="cuda:0")
    Bt = torch.zeros((n, k), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(binding.DLError) as e:
        binding.lowrank_linear_static(x, At, Bt)
    assert e.value.status == 4 and "static scratch" in str(e.value)
