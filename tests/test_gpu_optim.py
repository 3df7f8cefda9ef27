"""GPU parity of the paged AdamW step of the adapter parameters against the
fp64 oracle: the state in device memory (one launch) and paged out to pinned
host memory (chunks through a device staging buffer, copies on a second
stream or on the compute stream), single and repeated steps, ragged sizes
that leave a tail of n % 4 and several staging chunks.

Tolerances (fp32 arithmetic against fp64): m and v within 1e-6 normwise;
the parameter's change p_new - p_old within 1e-4 normwise of its largest
magnitude (the change is ~lr, while p's own fp32 rounding is ~1e-9); the
bf16 copy is torch's round-to-nearest-even of the fp32 result."""

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qn():
    import bit_nf4_quantized_16_amd as qn

    assert torch.cuda.is_available()
    return qn


def _state(n, seed):
    g = torch.Generator().manual_seed(seed)
    p = torch.randn(n, generator=g) * 0.02
    grad = torch.randn(n, generator=g) * torch.exp(torch.randn(n, generator=g) * 2.0) * 1e-3
    m = torch.randn(n, generator=g) * 1e-3
    v = torch.rand(n, generator=g) * 1e-6
    return p, grad, m, v


def _normwise(got, want):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    return float(np.max(np.abs(got - want)) / max(np.max(np.abs(want)), 1e-300))


def _check(p0, p, m, v, po, mo, vo):
    assert _normwise(m, mo) <= 1e-6
    assert _normwise(v, vo) <= 1e-6
    du, duo = np.asarray(p, np.float64) - p0, po - p0
    assert _normwise(du, duo) <= 1e-4


HP = dict(lr=2e-4, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)


def _f32(x):
    # the call takes its hyperparameters as fp32 values: the oracle gets the
    # same values (1 - fl32(0.999) differs from 1 - 0.999 by 1.3e-5 relative)
    return float(np.float32(x))


def _oracle_steps(p, g_list, m, v, t0):
    po, mo, vo = p.double().numpy(), m.double().numpy(), v.double().numpy()
    for i, g in enumerate(g_list):
        po, mo, vo = oracle.adamw_step(po, g.double().numpy(), mo, vo, t0 + i, _f32(HP["lr"]), _f32(HP["betas"][0]),
                                       _f32(HP["betas"][1]), _f32(HP["eps"]), _f32(HP["weight_decay"]))
    return po, mo, vo


@pytest.mark.parametrize("n", [1, 3, 4, 1000, (1 << 20) + 5])
@pytest.mark.parametrize("t", [1, 7])
def test_device_state_step(qn, n, t):
    p, g, m, v = _state(n, seed=n + t)
    P, G, M, V = (x.cuda() for x in (p, g, m, v))
    P16 = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    qn.paged_adamw_step(P, G, M, V, t, param_bf16=P16, **HP)
    torch.cuda.synchronize()
    po, mo, vo = _oracle_steps(p, [g], m, v, t)
    _check(p.double().numpy(), P.cpu(), M.cpu(), V.cpu(), po, mo, vo)
    assert torch.equal(P16, P.to(torch.bfloat16))


@pytest.mark.parametrize("mode,two_streams", [("direct", False), ("staged", True), ("staged", False)])
@pytest.mark.parametrize("n", [1000, 3 * (1 << 21) + 77])
def test_paged_state_equals_device_state(qn, monkeypatch, n, mode, two_streams):
    """State in pinned host memory, updated in place over the host link
    (default) or staged through device buffers in chunks: three steps in a
    row give the device-state results bit for bit (the same kernel per
    element) and the oracle's within the tolerances; the host copies hold the
    updated state afterwards."""
    if mode == "staged":
        monkeypatch.setenv("QLORA_NF4_ADAMW_PAGING", "staged")
    p, _, m, v = _state(n, seed=3 * n)
    grads = [_state(n, seed=100 + i)[1] for i in range(3)]
    Pd, Md, Vd = p.cuda(), m.cuda(), v.cuda()
    Ph = p.cuda()
    Mh, Vh = m.clone().pin_memory(), v.clone().pin_memory()
    cs = torch.cuda.Stream() if two_streams else None
    for i, g in enumerate(grads):
        G = g.cuda()
        qn.paged_adamw_step(Pd, G, Md, Vd, 1 + i, **HP)
        qn.paged_adamw_step(Ph, G, Mh, Vh, 1 + i, copy_stream=cs, **HP)
    torch.cuda.synchronize()
    assert torch.equal(Ph, Pd)
    assert torch.equal(Mh, Md.cpu()) and torch.equal(Vh, Vd.cpu())
    po, mo, vo = _oracle_steps(p, grads, m, v, 1)
    _check(p.double().numpy(), Ph.cpu(), Mh, Vh, po, mo, vo)


@pytest.mark.parametrize("mode", ["direct", "staged"])
def test_paged_step_orders_with_the_compute_stream(qn, monkeypatch, mode):
    """Work queued on the compute stream before the call (the gradient) is
    seen by the update (and, staged, by the copies on the copy stream), and
    work queued after it sees the state updated in host memory."""
    if mode == "staged":
        monkeypatch.setenv("QLORA_NF4_ADAMW_PAGING", "staged")
    n = 2 * (1 << 21) + 9
    p, g, m, v = _state(n, seed=11)
    P, Mh, Vh = p.cuda(), m.clone().pin_memory(), v.clone().pin_memory()
    G = torch.zeros(n, device="cuda")
    cs = torch.cuda.Stream()
    torch.cuda._sleep(2_000_000)  # keep the compute stream busy before the gradient lands
    G.copy_(g.cuda(non_blocking=True))
    qn.paged_adamw_step(P, G, Mh, Vh, 1, copy_stream=cs, **HP)
    Mc = torch.empty(n, device="cuda")
    Mc.copy_(Mh, non_blocking=True)  # queued after the step on the compute stream
    torch.cuda.synchronize()
    po, mo, vo = _oracle_steps(p, [g], m, v, 1)
    _check(p.double().numpy(), P.cpu(), Mh, Vh, po, mo, vo)
    assert torch.equal(Mc.cpu(), Mh)


def test_unpinned_or_mixed_state_is_refused(qn):
    n = 64
    P, G = torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    with pytest.raises(qn.QLoraError):
        qn.paged_adamw_step(P, G, torch.zeros(n), torch.zeros(n), 1)  # pageable host memory
    with pytest.raises(qn.QLoraError):
        qn.paged_adamw_step(P, G, torch.zeros(n, device="cuda"), torch.zeros(n).pin_memory(), 1)


def test_device_state_step_replays_in_a_graph(qn):
    """Device-resident state: the step is one kernel launch and can be
    captured; three replays equal three eager steps (the step number is
    fixed at capture, so the replays repeat step 5's bias correction)."""
    n = 50_000
    p, g, m, v = _state(n, seed=21)
    P1, M1, V1, G = p.cuda(), m.cuda(), v.cuda(), g.cuda()
    P2, M2, V2 = p.cuda(), m.cuda(), v.cuda()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        qn.paged_adamw_step(P2, G, M2, V2, 5, **HP)  # warm-up, then restore
    torch.cuda.current_stream().wait_stream(s)
    P2.copy_(P1)
    M2.copy_(M1)
    V2.copy_(V1)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        qn.paged_adamw_step(P2, G, M2, V2, 5, **HP)
    for _ in range(3):
        qn.paged_adamw_step(P1, G, M1, V1, 5, **HP)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(P1, P2) and torch.equal(M1, M2) and torch.equal(V1, V2)
