"""dobb_step_noalloc (the step with the library's static per-GPU scratch, for callers that cannot
allocate) against dobb_step, the entry point with a caller workspace: the same kernels, so the
results are equal bit for bit.  Two calls in a row, the second on a smaller input, so the second
runs on scratch the first left behind; the sizes cover the rows kernels (nb <= 128), the wide
kernels (nb = 400, basis planes in the scratch), a bf16 basis (its fp32 copy in the scratch) and
column-l2 (coefficients and column sums in the scratch)."""
import numpy as np
import pytest
import torch

import workload

pytestmark = pytest.mark.gpu
dobb = pytest.importorskip("block_diagonal_eigenbasis_amd")
DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _case(m, n, nb, seed, qdt=torch.float32):
    rng = np.random.default_rng(seed)
    Q = torch.tensor(np.stack([workload.haar(nb, rng) for _ in range(n // nb)]), dtype=torch.float32,
                     device=DEV).to(qdt)
    W = torch.tensor(0.02 * rng.standard_normal((m, n)), dtype=torch.float32, device=DEV)
    G = torch.tensor(rng.standard_normal((m, n)), dtype=torch.float32, device=DEV)
    M = torch.tensor(rng.standard_normal((m, n)), dtype=torch.float32, device=DEV)
    return W, G, M, Q


def _both(m, n, nb, seed, norm, qdt=torch.float32):
    W, G, M, Q = _case(m, n, nb, seed, qdt)
    hp = dobb.make_hparams(2.5e-3, 0.1, 0.9, 0.2, norm=norm)
    out = []
    for fn in (dobb.dobb_step, dobb.dobb_step_noalloc):
        W1, M1 = W.clone(), M.clone()
        U = torch.empty(m, n, device=DEV)
        C = torch.empty(m, n, device=DEV)
        fn(W1, G, M1, Q, nb, hp, U_out=U, C_out=C)
        torch.cuda.synchronize()
        out.append((W1, M1, U, C))
    for a, b, name in zip(out[0], out[1], "WMUC"):
        assert torch.equal(a, b), f"{name} differs ({m}x{n}, nb={nb})"


@pytest.mark.parametrize("first,second,norm,qdt", [
    ((1600, 6400, 400), (300, 800, 400), dobb.DOBB_NORM_SIGN, torch.float32),
    ((4800, 1600, 100), (130, 400, 100), dobb.DOBB_NORM_SIGN, torch.float32),
    ((2048, 1024, 128), (96, 256, 128), dobb.DOBB_NORM_SIGN, torch.bfloat16),
    ((1024, 1024, 64), (200, 128, 64), dobb.DOBB_NORM_COL_L2, torch.float32),
])
def test_noalloc_step_equals_workspace_step_twice(first, second, norm, qdt):
    print(f"noalloc {first} then {second} norm={norm} {qdt}", flush=True)
    _both(*first, seed=1, norm=norm, qdt=qdt)
    _both(*second, seed=2, norm=norm, qdt=qdt)


def test_noalloc_refuses_a_shape_beyond_its_scratch():
    W, G, M, Q = (torch.zeros(1, device=DEV),) * 4
    W = torch.zeros(11008, 4096, device=DEV, dtype=torch.bfloat16)
    G = torch.zeros_like(W)
    M = torch.zeros(11008, 4096, device=DEV)
    Q = torch.zeros(32, 128, 128, device=DEV)
    with pytest.raises(dobb.DobbError) as e:
        dobb.dobb_step_noalloc(W, G, M, Q, 128, dobb.make_hparams(0.1, 0, 0.9, 0.2, norm=dobb.DOBB_NORM_COL_L2))
    assert e.value.status == dobb.DOBB_ERR_WORKSPACE
