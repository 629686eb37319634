"""The optimizer layer over libdobb.so against the entry points it drives (MI355X only).

* DobbGroup with streams=2 runs the weights whose blocks have at most 128 columns and the wider ones
  on two streams; its fused refresh_step must leave W, M, A and Q bit for bit where the one-stream
  accumulate -> refresh -> step sequence leaves them (every kernel is deterministic, and the grouped
  forms equal the single calls, test_gpu_parity.py).
* The torch.optim wrapper follows the cadence of the Dobb paper (Tables 14, 15 and 17: capture on
  refresh iterations only, from the first micro-batch; an exact first refresh, warm-started orthogonal
  iteration with k = 1 afterwards; the moment EMA starting from the first capture). The test replays
  that cadence with the single-matrix entry points and compares bit for bit.
"""
import numpy as np
import pytest
import torch

import workload

pytestmark = pytest.mark.gpu
dobb = pytest.importorskip("block_diagonal_eigenbasis_amd")
from block_diagonal_eigenbasis_amd.optimizer import Dobb, DobbGroup, default_update_scale  # noqa: E402

DEV = "cuda"
RNG = np.random.default_rng


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def t32(x):
    return torch.as_tensor(np.ascontiguousarray(x), dtype=torch.float32, device=DEV)


SHAPES = [(96, 256, 64), (64, 512, 256), (128, 256, 128), (80, 400, 200), (48, 96, 48)]


@pytest.mark.parametrize("norm,wdt", [("sign", torch.float32), ("col_l2", torch.float32), ("sign", torch.bfloat16)])
def test_two_streams_match_one_stream(norm, wdt):
    print(f"two streams: norm={norm} W={wdt}", flush=True)
    rng = RNG(91)
    N = 512
    Ws = [t32(0.02 * rng.standard_normal((m, n))).to(wdt) for m, n, _ in SHAPES]
    Gs = [t32(rng.standard_normal((m, n))).to(wdt) for m, n, _ in SHAPES]
    xs = [t32(workload.activations(N, n, 0.15, rng)).to(torch.bfloat16) for _, n, _ in SHAPES]
    nm = dobb.DOBB_NORM_COL_L2 if norm == "col_l2" else dobb.DOBB_NORM_SIGN
    g1, g2 = [DobbGroup([w.clone() for w in Ws], [nb for _, _, nb in SHAPES], grads=Gs, n_tokens=N,
                        weight_decay=0.1, momentum=0.9, norm=nm, streams=s) for s in (1, 2)]
    assert len(g1._parts) == 1 and len(g2._parts) == 2
    assert sorted(g2._parts[0].idx + g2._parts[1].idx) == list(range(len(SHAPES)))
    for g in (g1, g2):
        g.accumulate(xs, 0.0)
        g.refresh(dobb.DOBB_REFRESH_EXACT, 0, warm_start=False)
        g.step()
    for it in range(3):
        print(f"two streams: iteration {it}", flush=True)
        g1.accumulate(xs, 0.9)
        g1.refresh(dobb.DOBB_REFRESH_ORTH_ITER, 1)
        g1.step()
        g2.refresh_step(xs, 0.9, dobb.DOBB_REFRESH_ORTH_ITER, 1)
    g2.set_streams(1)                                        # back to one part, the state kept
    assert len(g2._parts) == 1
    g1.step()
    g2.step()
    torch.cuda.synchronize()
    for name in ("W", "M", "A", "Q"):
        for i, (a, b) in enumerate(zip(getattr(g1, name), getattr(g2, name))):
            assert torch.equal(a, b), f"{name}[{i}] differs"


def test_refresh_step_grows_the_workspace_for_more_tokens():
    rng = RNG(92)
    shapes = SHAPES[:2]
    Ws = [t32(0.02 * rng.standard_normal((m, n))) for m, n, _ in shapes]
    Gs = [t32(rng.standard_normal((m, n))) for m, n, _ in shapes]
    g = DobbGroup(Ws, [nb for _, _, nb in shapes], grads=Gs, n_tokens=16, streams=2)
    As = [torch.zeros_like(a) for a in g.A]
    xs = [t32(workload.activations(3000, n, 0.15, rng)) for _, n, _ in shapes]
    g.refresh_step(xs, 0.0, dobb.DOBB_REFRESH_EXACT, 0, warm_start=False)
    for x, A, (_, _, nb) in zip(xs, As, shapes):
        dobb.dobb_accumulate_moment(x, A, nb)
    torch.cuda.synchronize()
    assert g.n_tokens == 3000
    for a, b in zip(g.A, As):
        assert torch.equal(a, b)


@pytest.mark.parametrize("streams", [1, 2])
def test_optimizer_cadence_matches_entry_points(streams):
    rng = RNG(93)
    dims = [(96, 256), (64, 512), (48, 128)]          # blocks=2: nb = 128, 256, 64
    mods = [torch.nn.Linear(n, m, bias=False).to(DEV) for m, n in dims]
    params = [mod.weight for mod in mods]
    with torch.no_grad():
        for p in params:
            p.copy_(t32(0.02 * rng.standard_normal(tuple(p.shape))))
    lr, wd, mu, T, beta = 2.5e-3, 0.1, 0.9, 2, 0.9
    opt = Dobb(params, lr=lr, weight_decay=wd, momentum=mu, blocks=2, refresh_period=T, orth_iters=1, beta=beta,
               streams=streams)
    hooks = opt.attach_capture_hooks(mods)
    nbs = [n // 2 for _, n in dims]
    W_ref = [p.detach().clone() for p in params]
    M_ref = [torch.zeros(m, n, device=DEV) for m, n in dims]
    A_ref = [torch.zeros(n // nb, nb, nb, device=DEV) for (_, n), nb in zip(dims, nbs)]
    Q_ref = [torch.eye(nb, device=DEV).expand(n // nb, nb, nb).contiguous() for (_, n), nb in zip(dims, nbs)]
    hps = [dobb.make_hparams(lr, wd, mu, default_update_scale(m, n)) for m, n in dims]
    refreshed = False
    for t in range(5):
        print(f"optimizer cadence: streams={streams} t={t}", flush=True)
        captures = opt.wants_capture()
        assert captures == (t % T == 0)
        xs = [t32(workload.activations(256, n, 0.15, rng)) for _, n in dims]
        with torch.no_grad():
            for mod, x in zip(mods, xs):
                mod(x)
                mod(t32(rng.standard_normal(tuple(x.shape))))   # a second micro-batch: not captured
        grads = [t32(rng.standard_normal((m, n))) for m, n in dims]
        for p, g in zip(params, grads):
            p.grad = g
        opt.step()
        if captures:
            for i, nb in enumerate(nbs):
                dobb.dobb_accumulate_moment(xs[i], A_ref[i], nb, beta if refreshed else 0.0)
                if refreshed:
                    dobb.dobb_refresh_basis(A_ref[i], Q_ref[i], dobb.DOBB_REFRESH_ORTH_ITER, iters=1, warm_start=True)
                else:
                    dobb.dobb_refresh_basis(A_ref[i], Q_ref[i], dobb.DOBB_REFRESH_EXACT, warm_start=False)
            refreshed = True
        for i, nb in enumerate(nbs):
            dobb.dobb_step(W_ref[i], grads[i], M_ref[i], Q_ref[i], nb, hps[i])
    torch.cuda.synchronize()
    for h in hooks:
        h.remove()
    g = opt._group
    for i in range(len(dims)):
        assert torch.equal(params[i].detach(), W_ref[i]), f"W[{i}]"
        assert torch.equal(g.M[i], M_ref[i]), f"M[{i}]"
        assert torch.equal(g.A[i], A_ref[i]), f"A[{i}]"
        assert torch.equal(g.Q[i], Q_ref[i]), f"Q[{i}]"


def test_lr_scheduler_and_param_groups_take_effect():
    """lr, weight decay and momentum are read from param_groups at every step: a StepLR schedule
    halving lr each step, and a second group with its own weight decay, match the entry points
    called with those values, bit for bit."""
    rng = RNG(94)
    dims = [(96, 256), (64, 128)]
    params = [torch.nn.Parameter(t32(0.02 * rng.standard_normal((m, n)))) for m, n in dims]
    opt = Dobb([{"params": [params[0]]}, {"params": [params[1]], "weight_decay": 0.3}], lr=4e-3,
               weight_decay=0.1, momentum=0.9, blocks=2, refresh_period=1000)
    sched = torch.optim.lr_scheduler.StepLR(opt, step_size=1, gamma=0.5)
    W_ref = [p.detach().clone() for p in params]
    M_ref = [torch.zeros(m, n, device=DEV) for m, n in dims]
    Q_ref = [torch.eye(n // 2, device=DEV).expand(2, n // 2, n // 2).contiguous() for _, n in dims]
    lr = 4e-3
    for t in range(4):
        grads = [t32(rng.standard_normal((m, n))) for m, n in dims]
        for p, g in zip(params, grads):
            p.grad = g
        if t == 2:
            opt.param_groups[1]["momentum"] = 0.5
        opt.step()
        sched.step()
        for i, (m, n) in enumerate(dims):
            wd = 0.1 if i == 0 else 0.3
            mu = 0.5 if (i == 1 and t >= 2) else 0.9
            hp = dobb.make_hparams(lr, wd, mu, default_update_scale(m, n))
            dobb.dobb_step(W_ref[i], grads[i], M_ref[i], Q_ref[i], n // 2, hp)
        lr *= 0.5
    torch.cuda.synchronize()
    for i in range(len(dims)):
        assert torch.equal(params[i].detach(), W_ref[i]), f"W[{i}]"


def test_mixed_dtypes_are_split_per_call():
    """A set mixing fp32 and bf16 weights, activations and gradients (as under autocast): every
    grouped call is issued per dtype, and each weight ends bit for bit where the single-matrix entry
    points leave it."""
    rng = RNG(95)
    shapes = [(96, 256, 64), (64, 128, 64), (80, 256, 128), (48, 128, 32)]
    wdts = [torch.float32, torch.bfloat16, torch.float32, torch.bfloat16]
    xdts = [torch.bfloat16, torch.float32, torch.float32, torch.bfloat16]
    gdts = [torch.float32, torch.float32, torch.bfloat16, torch.bfloat16]
    Ws = [t32(0.02 * rng.standard_normal((m, n))).to(d) for (m, n, _), d in zip(shapes, wdts)]
    Gs = [t32(rng.standard_normal((m, n))).to(d) for (m, n, _), d in zip(shapes, gdts)]
    xs = [t32(workload.activations(300 + 50 * i, n, 0.15, rng)).to(d)
          for i, ((_, n, _), d) in enumerate(zip(shapes, xdts))]
    g = DobbGroup([w.clone() for w in Ws], [nb for _, _, nb in shapes], grads=Gs, weight_decay=0.1, momentum=0.9)
    assert len(g._parts) == 2
    g.accumulate(xs, 0.0)
    g.refresh(dobb.DOBB_REFRESH_EXACT, 0, warm_start=False)
    g.step()
    g.refresh_step(xs, 0.9, dobb.DOBB_REFRESH_ORTH_ITER, 1)
    for i, (m, n, nb) in enumerate(shapes):
        W = Ws[i].clone()
        M = torch.zeros(m, n, device=DEV)
        A = torch.zeros(n // nb, nb, nb, device=DEV)
        Q = torch.empty_like(A)
        hp = dobb.make_hparams(2.5e-3, 0.1, 0.9, default_update_scale(m, n))
        dobb.dobb_accumulate_moment(xs[i], A, nb, 0.0)
        dobb.dobb_refresh_basis(A, Q, dobb.DOBB_REFRESH_EXACT)
        dobb.dobb_step(W, Gs[i], M, Q, nb, hp)
        dobb.dobb_accumulate_moment(xs[i], A, nb, 0.9)
        dobb.dobb_refresh_basis(A, Q, dobb.DOBB_REFRESH_ORTH_ITER, iters=1, warm_start=True)
        dobb.dobb_step(W, Gs[i], M, Q, nb, hp)
        torch.cuda.synchronize()
        assert torch.equal(g.W[i], W), f"W[{i}]"
        assert torch.equal(g.A[i], A) and torch.equal(g.Q[i], Q) and torch.equal(g.M[i], M), f"state {i}"


def test_capture_all_micro_batches_and_bf16_basis():
    """capture="all" (Table 17) pools every micro-batch of a refresh iteration into one capture;
    basis_dtype=bf16 (Table 18) keeps Q in bf16.  Both match the entry points bit for bit."""
    rng = RNG(96)
    dims = [(96, 256), (64, 512)]
    mods = [torch.nn.Linear(n, m, bias=False).to(DEV) for m, n in dims]
    params = [mod.weight for mod in mods]
    with torch.no_grad():
        for p in params:
            p.copy_(t32(0.02 * rng.standard_normal(tuple(p.shape))))
    opt = Dobb(params, lr=2.5e-3, weight_decay=0.1, momentum=0.9, blocks=2, refresh_period=2, capture="all",
               basis_dtype=torch.bfloat16)
    hooks = opt.attach_capture_hooks(mods)
    nbs = [n // 2 for _, n in dims]
    W_ref = [p.detach().clone() for p in params]
    M_ref = [torch.zeros(m, n, device=DEV) for m, n in dims]
    A_ref = [torch.zeros(n // nb, nb, nb, device=DEV) for (_, n), nb in zip(dims, nbs)]
    Q_ref = [torch.eye(nb, device=DEV, dtype=torch.bfloat16).expand(n // nb, nb, nb).contiguous()
             for (_, n), nb in zip(dims, nbs)]
    refreshed = False
    for t in range(4):
        captures = opt.wants_capture()
        mbs = [[t32(workload.activations(128, n, 0.15, rng)) for _, n in dims] for _ in range(3)]
        with torch.no_grad():
            for mb in mbs:
                for mod, x in zip(mods, mb):
                    mod(x)
        grads = [t32(rng.standard_normal((m, n))) for m, n in dims]
        for p, gr in zip(params, grads):
            p.grad = gr
        opt.step()
        for i, nb in enumerate(nbs):
            if captures:
                x_all = torch.cat([mb[i] for mb in mbs], 0)
                dobb.dobb_accumulate_moment(x_all, A_ref[i], nb, 0.9 if refreshed else 0.0)
                mode = dobb.DOBB_REFRESH_ORTH_ITER if refreshed else dobb.DOBB_REFRESH_EXACT
                dobb.dobb_refresh_basis(A_ref[i], Q_ref[i], mode, iters=1 if refreshed else 0, warm_start=refreshed)
            m, n = dims[i]
            dobb.dobb_step(W_ref[i], grads[i], M_ref[i], Q_ref[i], nb,
                           dobb.make_hparams(2.5e-3, 0.1, 0.9, default_update_scale(m, n)))
        refreshed = refreshed or captures
    torch.cuda.synchronize()
    for h in hooks:
        h.remove()
    g = opt._group
    for i in range(len(dims)):
        assert g.Q[i].dtype == torch.bfloat16
        assert torch.equal(params[i].detach(), W_ref[i]), f"W[{i}]"
        assert torch.equal(g.A[i], A_ref[i]) and torch.equal(g.Q[i], Q_ref[i]), f"state {i}"


def test_dobb_g_optimizer_captures_output_gradients():
    """basis="output_gradient" (Dobb-G, Tables 12-13): backward hooks capture each weight's output
    gradient on refresh iterations, the moments and bases live on the output axis (blocks of rows),
    and the step is dobb_step_g; bit for bit equal to those entry points called in turn."""
    rng = RNG(97)
    dims = [(128, 96), (64, 256)]           # (m, n); blocks=2: nb = 64, 32 rows
    mods = [torch.nn.Linear(n, m, bias=False).to(DEV) for m, n in dims]
    params = [mod.weight for mod in mods]
    with torch.no_grad():
        for p in params:
            p.copy_(t32(0.02 * rng.standard_normal(tuple(p.shape))))
    opt = Dobb(params, lr=2.5e-3, weight_decay=0.1, momentum=0.9, blocks=2, refresh_period=2,
               basis="output_gradient")
    hooks = opt.attach_capture_hooks(mods)
    nbs = [m // 2 for m, _ in dims]
    W_ref = [p.detach().clone() for p in params]
    M_ref = [torch.zeros(m, n, device=DEV) for m, n in dims]
    A_ref = [torch.zeros(2, nb, nb, device=DEV) for nb in nbs]
    P_ref = [torch.eye(nb, device=DEV).expand(2, nb, nb).contiguous() for nb in nbs]
    refreshed = False
    for t in range(4):
        captures = opt.wants_capture()
        xs = [t32(workload.activations(200, n, 0.15, rng)) for _, n in dims]
        dys = [t32(workload.activations(200, m, 0.15, rng)) for m, _ in dims]
        for p in params:
            p.grad = None
        for mod, x, dy in zip(mods, xs, dys):
            (mod(x) * dy).sum().backward()            # the output gradient is dy
        grads = [p.grad.detach().clone() for p in params]
        opt.step()
        for i, nb in enumerate(nbs):
            m, n = dims[i]
            if captures:
                dobb.dobb_accumulate_moment(dys[i], A_ref[i], nb, 0.9 if refreshed else 0.0)
                mode = dobb.DOBB_REFRESH_ORTH_ITER if refreshed else dobb.DOBB_REFRESH_EXACT
                dobb.dobb_refresh_basis(A_ref[i], P_ref[i], mode, iters=1 if refreshed else 0, warm_start=refreshed)
            dobb.dobb_step_g(W_ref[i], grads[i], M_ref[i], P_ref[i], nb,
                             dobb.make_hparams(2.5e-3, 0.1, 0.9, 0.2 * (max(m, n) / n) ** 0.5))
        refreshed = refreshed or captures
    torch.cuda.synchronize()
    for h in hooks:
        h.remove()
    g = opt._group
    for i in range(len(dims)):
        assert g.A[i].shape == (2, nbs[i], nbs[i])
        assert torch.equal(params[i].detach(), W_ref[i]), f"W[{i}]"
        assert torch.equal(g.A[i], A_ref[i]) and torch.equal(g.Q[i], P_ref[i]), f"state {i}"


@pytest.mark.parametrize("streams", [1, 2])
def test_graph_replay_matches_eager_steps(streams):
    """refresh_step captured into a HIP graph: each replay, with eager work and synchronisations
    between the replays, leaves W, M, A and Q bitwise equal to a twin group stepped eagerly."""
    print(f"graph replay: streams={streams}", flush=True)
    rng = RNG(97)
    N = 512
    Ws = [t32(0.02 * rng.standard_normal((m, n))) for m, n, _ in SHAPES]
    Gs = [t32(rng.standard_normal((m, n))) for m, n, _ in SHAPES]
    xs = [t32(workload.activations(N, n, 0.15, rng)).to(torch.bfloat16) for _, n, _ in SHAPES]
    eager, graphed = [DobbGroup([w.clone() for w in Ws], [nb for _, _, nb in SHAPES], grads=Gs, n_tokens=N,
                                weight_decay=0.1, momentum=0.9, streams=streams) for _ in range(2)]
    for g in (eager, graphed):
        g.accumulate(xs, 0.0)
        g.refresh(dobb.DOBB_REFRESH_EXACT, 0, warm_start=False)
        g.refresh_step(xs, 0.9, dobb.DOBB_REFRESH_ORTH_ITER, 1)
    graph = graphed.capture_refresh_step(xs, 0.9, dobb.DOBB_REFRESH_ORTH_ITER, 1)
    torch.cuda.synchronize()
    for g1, g2 in ((eager.W, graphed.W), (eager.A, graphed.A)):   # capturing ran nothing
        for a, b in zip(g1, g2):
            assert torch.equal(a, b)
    for it in range(4):
        eager.refresh_step(xs, 0.9, dobb.DOBB_REFRESH_ORTH_ITER, 1)
        graph.replay()
        noise = torch.randn(4096, device=DEV)          # eager work between the replays
        assert torch.isfinite(noise.sum()).item()
        torch.cuda.synchronize()
        for name in ("W", "M", "A", "Q"):
            for i, (a, b) in enumerate(zip(getattr(eager, name), getattr(graphed, name))):
                assert torch.equal(a, b), (it, name, i)
