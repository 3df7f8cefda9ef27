"""The library's calls captured in a HIP graph (torch.cuda.graph) and replayed:
every replay, with unrelated eager work and synchronizations between the
replays, must give the eager results bit for bit. The captured step covers
quantization with double quantization, the forward and backward GEMM path
with split rank projections (their arrival counters must work when a launch
is replayed with the same token) and the decode GEMV."""

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qn():
    import bit_nf4_quantized_16_amd as qn

    assert torch.cuda.is_available()
    return qn


def test_graph_replay_matches_eager(qn):
    N = K = 5120
    T, r = 256, 16
    W = workloads.normal_weight(N, K, 0.02, seed=31).cuda()
    case = workloads.lora_case("graph", W.cpu(), T, r, 32.0, 1 / K, 0.05, seed=31)
    X, dY, A, B = (t.cuda() for t in (case.X, case.dY, case.A, case.B))
    X1 = X[:1].contiguous()
    s = case.scale

    def step():
        w = qn.quantize_weight(W)
        Y, U = qn.qlora_linear_fwd(w, X, A, B, s)
        dX, dA, dB = qn.qlora_linear_bwd(w, X, dY, A, B, s, U=U)
        y1, _ = qn.qlora_linear_fwd(w, X1, A, B, s)
        return [w.packed, w.c8, w.dq_scale, w.dq_mean, Y, U, dX, dA, dB, y1]

    eager = [t.clone() for t in step()]
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = step()
    other = workloads.normal_weight(1024, 2048, 0.02, seed=32).cuda()
    for rep in range(3):
        qn.quantize_weight(other)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, eager)):
            assert torch.equal(a, b), "replay %d: output %d differs from the eager run" % (rep, i)


@pytest.mark.parametrize("split_bwd", [False, True])
def test_two_stream_graph_matches_serial(qn, split_bwd):
    # weights quantized on a second stream while the first runs the layer of
    # the previous weight (event waits in between), captured and replayed;
    # split_bwd: dX on the first stream, dA and dB by a second backward call
    # on the other stream once the forward is done (the benchmark's step)
    Ws = [workloads.normal_weight(1024, 2048, 0.02, seed=40 + i).cuda() for i in range(3)]
    case = workloads.lora_case("streams", Ws[0].cpu(), 96, 16, 32.0, 1 / 2048, 0.05, seed=40)
    X, dY, A, B = (t.cuda() for t in (case.X, case.dY, case.A, case.B))
    s = case.scale

    def serial():
        outs = []
        for W in Ws:
            w = qn.quantize_weight(W)
            Y, U = qn.qlora_linear_fwd(w, X, A, B, s)
            outs += [w.packed, Y, U, *qn.qlora_linear_bwd(w, X, dY, A, B, s, U=U)]
        return outs

    side = torch.cuda.Stream()

    def two_streams():
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        ws, evs = [], []
        with torch.cuda.stream(side):
            for W in Ws:
                ws.append(qn.quantize_weight(W))
                ev = torch.cuda.Event()
                ev.record(side)
                evs.append(ev)
        outs = []
        for w, ev in zip(ws, evs):
            main.wait_event(ev)
            Y, U = qn.qlora_linear_fwd(w, X, A, B, s)
            if not split_bwd:
                outs += [w.packed, Y, U, *qn.qlora_linear_bwd(w, X, dY, A, B, s, U=U)]
                continue
            done = torch.cuda.Event()
            done.record(main)
            dX, _, _ = qn.qlora_linear_bwd(w, X, dY, A, B, s, U=U, need_da=False, need_db=False)
            side.wait_event(done)
            with torch.cuda.stream(side):
                _, dA, dB = qn.qlora_linear_bwd(w, X, dY, A, B, s, U=U, need_dx=False)
            outs += [w.packed, Y, U, dX, dA, dB]
        main.wait_stream(side)
        return outs

    ref = [t.clone() for t in serial()]
    warm = torch.cuda.Stream()
    warm.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(warm):
        two_streams()
    torch.cuda.current_stream().wait_stream(warm)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = two_streams()
    for rep in range(3):
        qn.quantize_weight(Ws[1])  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a, b), "replay %d: output %d differs from the serial run" % (rep, i)


def test_two_stream_graph_with_grouped_backward(qn):
    # the benchmark's step shape: three layers, the first two reading the same
    # X; weights quantized on the second stream, forwards on the first, then
    # the third layer's backward and the first two's grouped backward (dX on
    # the first stream, dA and dB by a second call on the other), captured
    # and replayed against the same calls made serially on one stream
    Ws = [workloads.normal_weight(n, 2048, 0.02, seed=50 + i).cuda() for i, n in enumerate((1024, 1024, 512))]
    cases = [workloads.lora_case("g%d" % i, W.cpu(), 96, 16, 32.0, 1 / 2048, 0.05, seed=50 + i)
             for i, W in enumerate(Ws)]
    X = cases[0].X.cuda()
    dYs = [c.dY.cuda() for c in cases]
    As = [c.A.cuda() for c in cases]
    Bs = [c.B.cuda() for c in cases]
    s = cases[0].scale

    def serial():
        ws = [qn.quantize_weight(W) for W in Ws]
        fw = [qn.qlora_linear_fwd(w, X, As[i], Bs[i], s) for i, w in enumerate(ws)]
        outs = [t for Y, U in fw for t in (Y, U)]
        outs += list(qn.qlora_linear_bwd(ws[2], X, dYs[2], As[2], Bs[2], s, U=fw[2][1]))
        dX, dA, dB = qn.qlora_linear_bwd_group(ws[:2], X, dYs[:2], As[:2], Bs[:2], s, Us=[fw[0][1], fw[1][1]])
        return outs + [dX, *dA, *dB]

    side = torch.cuda.Stream()

    def two_streams():
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        ws, evs = [], []
        with torch.cuda.stream(side):
            for W in Ws:
                ws.append(qn.quantize_weight(W))
                ev = torch.cuda.Event()
                ev.record(side)
                evs.append(ev)
        fw = []
        for i, (w, ev) in enumerate(zip(ws, evs)):
            main.wait_event(ev)
            Y, U = qn.qlora_linear_fwd(w, X, As[i], Bs[i], s)
            done = torch.cuda.Event()
            done.record(main)
            fw.append((Y, U, done))
        dX2, _, _ = qn.qlora_linear_bwd(ws[2], X, dYs[2], As[2], Bs[2], s, U=fw[2][1], need_da=False, need_db=False)
        side.wait_event(fw[2][2])
        with torch.cuda.stream(side):
            _, dA2, dB2 = qn.qlora_linear_bwd(ws[2], X, dYs[2], As[2], Bs[2], s, U=fw[2][1], need_dx=False)
        grp = (ws[:2], X, dYs[:2], As[:2], Bs[:2], s)
        Us = [fw[0][1], fw[1][1]]
        dX, _, _ = qn.qlora_linear_bwd_group(*grp, Us=Us, need_da=False, need_db=False)
        side.wait_event(fw[1][2])
        with torch.cuda.stream(side):
            _, dA, dB = qn.qlora_linear_bwd_group(*grp, Us=Us, need_dx=False)
        main.wait_stream(side)
        return [t for Y, U, _ in fw for t in (Y, U)] + [dX2, dA2, dB2, dX, *dA, *dB]

    ref = [t.clone() for t in serial()]
    warm = torch.cuda.Stream()
    warm.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(warm):
        two_streams()
    torch.cuda.current_stream().wait_stream(warm)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = two_streams()
    for rep in range(3):
        qn.quantize_weight(Ws[1])  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a, b), "replay %d: output %d differs from the serial run" % (rep, i)


@pytest.mark.parametrize("spin", [None, "1"])
@pytest.mark.parametrize("T", [1, 16])
def test_decode_graph_replays_with_new_inputs(qn, monkeypatch, T, spin):
    """A captured decode call (the GEMV hands U over in tagged words in its
    workspace, and a replay reuses the launch's tag, mixed with an epoch
    word that a kernel recorded before the launch advances): replays with
    new x give the eager results for that x. With QLORA_NF4_GEMV_SPIN=1 the
    row workgroups give up waiting for the shared U almost at once and
    compute it themselves, while the U workgroups' stores land late: no
    replay may take those for its own."""
    if spin is not None:
        monkeypatch.setenv("QLORA_NF4_GEMV_SPIN", spin)
    N, K, r = 4096, 4096, 16
    W = workloads.normal_weight(N, K, 0.02, seed=41).cuda()
    case = workloads.lora_case("graph_decode", W.cpu(), T, r, 32.0, 1 / K, 0.05, seed=41)
    A, B = case.A.cuda(), case.B.cuda()
    w = qn.quantize_weight(W)
    X = torch.empty(T, K, dtype=torch.bfloat16, device="cuda")
    xs = [workloads.bf16_normal((T, K), 1.0, seed=50 + i).cuda() for i in range(4)]
    X.copy_(xs[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        qn.qlora_linear_fwd(w, X, A, B, case.scale)  # warm-up before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        Y, U = qn.qlora_linear_fwd(w, X, A, B, case.scale)
    for rep in range(1, 7):
        X.copy_(xs[rep % 4])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        Ye, Ue = qn.qlora_linear_fwd(w, xs[rep % 4], A, B, case.scale)
        torch.cuda.synchronize()
        assert torch.equal(Y, Ye) and torch.equal(U, Ue), "replay %d differs from the eager call" % rep


@pytest.mark.parametrize("spin", [None, "1"])
def test_grouped_decode_graph_replays_with_new_inputs(qn, monkeypatch, spin):
    """The grouped decode call captured once: each layer keeps its own tagged
    words in its slice of the workspace; every replay with a new x gives
    the eager single-layer results (also when the row workgroups give up
    waiting for U almost at once)."""
    if spin is not None:
        monkeypatch.setenv("QLORA_NF4_GEMV_SPIN", spin)
    T, K, r = 1, 4096, 16
    ws, As, Bs = [], [], []
    for i, N in enumerate((4096, 1024, 1024)):
        W = workloads.normal_weight(N, K, 0.02, seed=60 + i)
        case = workloads.lora_case("graph_group%d" % i, W, T, r, 32.0, 1 / K, 0.05, seed=60 + i)
        ws.append(qn.quantize_weight(W.cuda()))
        As.append(case.A.cuda())
        Bs.append(case.B.cuda())
    s = case.scale
    X = torch.empty(T, K, dtype=torch.bfloat16, device="cuda")
    xs = [workloads.bf16_normal((T, K), 1.0, seed=70 + i).cuda() for i in range(4)]
    X.copy_(xs[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        qn.qlora_linear_fwd_group(ws, X, As, Bs, s)  # warm-up before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = qn.qlora_linear_fwd_group(ws, X, As, Bs, s)
    for rep in range(1, 4):
        X.copy_(xs[rep])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, w in enumerate(ws):
            Ye, Ue = qn.qlora_linear_fwd(w, xs[rep], As[i], Bs[i], s)
            torch.cuda.synchronize()
            assert torch.equal(outs[i][0], Ye) and torch.equal(outs[i][1], Ue), "replay %d, layer %d" % (rep, i)
