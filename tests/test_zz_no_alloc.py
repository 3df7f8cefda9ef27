"""The forward entry point that allocates nothing (qlora_linear_fwd_noalloc,
for callers that cannot allocate device memory): on the same inputs it gives
qlora_linear_fwd's Y and U bit for bit (same kernels, same launch plan), on
two calls in a row with the second smaller, while the library's scratch
array keeps the first call's contents; and a decode call captured into a
graph and replayed with new x gives the eager results each time."""

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qn():
    import bit_nf4_quantized_16_amd as qn

    assert torch.cuda.is_available()
    return qn


def _case(qn, N, K, T, r, seed):
    W = workloads.normal_weight(N, K, 0.02, seed=seed)
    c = workloads.lora_case("noalloc_N%dK%dT%dr%d" % (N, K, T, r), W, T, r, 2.0 * r, 1 / K, 0.05, seed=seed + 1)
    w = qn.quantize_weight(W.cuda())
    return w, c.X.cuda(), c.A.cuda(), c.B.cuda(), c.scale


# (first call, second smaller call): N, K, T, r
PAIRS = [
    # decode GEMV: U's tagged words and the epoch word live in the scratch
    ((4096, 4096, 16, 16), (1024, 4096, 1, 8)),
    ((11008, 4096, 5, 64), (264, 1088, 3, 5)),
    # GEMM: bf16 s U staging, the projection's split partials and, for the
    # 4096 x 11008 weight at T = 1024, 64 MiB of split-K partials
    ((4096, 11008, 1024, 16), (520, 1088, 40, 16)),
    ((520, 1088, 300, 70), (264, 192, 17, 5)),
    # GEMM with U computed inside its launch (7B gate at T = 1024, r = 16):
    # the tagged U words live in the scratch
    ((11008, 4096, 1024, 16), (1024, 512, 300, 8)),
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_equals_workspace_entry(qn, first, second):
    for i, (N, K, T, r) in enumerate((first, second)):
        print("noalloc call %d: N=%d K=%d T=%d r=%d" % (i, N, K, T, r), flush=True)
        w, X, A, B, s = _case(qn, N, K, T, r, seed=N + K + T + r)
        Y0, U0 = qn.qlora_linear_fwd(w, X, A, B, s)
        Y1, U1 = qn.qlora_linear_fwd_noalloc(w, X, A, B, s)
        torch.cuda.synchronize()
        assert torch.equal(Y0, Y1), "call %d: Y differs" % i
        assert torch.equal(U0, U1), "call %d: U differs" % i


def test_noalloc_rank_zero_needs_no_scratch(qn):
    w, X, _, _, _ = _case(qn, 264, 1024, 3, 8, seed=5)
    Y0, _ = qn.qlora_linear_fwd(w, X)
    Y1, U1 = qn.qlora_linear_fwd_noalloc(w, X)
    torch.cuda.synchronize()
    assert U1 is None and torch.equal(Y0, Y1)


@pytest.mark.parametrize("T", [1, 16])
def test_noalloc_decode_graph_replays_with_new_inputs(qn, T):
    N, K, r = 4096, 4096, 16
    w, X0, A, B, s = _case(qn, N, K, T, r, seed=77)
    X = torch.empty_like(X0)
    xs = [workloads.bf16_normal((T, K), 1.0, seed=90 + i).cuda() for i in range(4)]
    X.copy_(xs[0])
    Y = torch.empty(T, N, dtype=torch.bfloat16, device="cuda")
    U = torch.empty(T, r, dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        qn.qlora_linear_fwd_noalloc(w, X, A, B, s, out=Y, U_out=U)  # first call on the GPU: outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qn.qlora_linear_fwd_noalloc(w, X, A, B, s, out=Y, U_out=U)
    for rep in range(1, 5):
        X.copy_(xs[rep % 4])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        Ye, Ue = qn.qlora_linear_fwd(w, xs[rep % 4], A, B, s)
        torch.cuda.synchronize()
        assert torch.equal(Y, Ye) and torch.equal(U, Ue), "replay %d differs from the eager call" % rep
