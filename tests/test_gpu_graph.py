"""tile_gemm_run is enqueue-only (no allocation, no synchronisation), so it can
be captured into a HIP graph and replayed: the split between preparing work
once and replaying it that "Rust Compute Kernels" describes (section "Why
scoped graph capture helps borrowing").

Each replay is checked against the fp64 CPU oracle (the 1e-5 * |A|.|B| rule,
exact for integer inputs) and bitwise against an eager run of the same
operands, with eager work and synchronisation between replays, and with the
captured inputs rewritten in place between replays (a graph keeps its
pointers, not their contents).
"""

import numpy as np
import pytest

import oracle
import tile_partitioned_dense_amd as tg
from tile_partitioned_dense_amd import synth

from gpu_helpers import host_out

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    with tg.TileGemm(0) as gg:
        yield gg


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def _bits(C):
    return C.view(torch.int32) if C.dtype == torch.float32 else C.view(torch.int16)


def _oracle_check(out, A, Bs, bcol, dt, integer):
    C64, D64 = oracle.gemm(A, Bs.T if bcol else Bs)
    bf16 = dt == torch.bfloat16
    if integer:
        return oracle.check_exact(out, C64, bf16)
    return oracle.check_bf16(out, C64, D64) if bf16 else oracle.check_f32(out, C64, D64)


@pytest.mark.parametrize("M,N,K,bcol,dt", [
    (700, 904, 296, False, torch.float32),    # tile kernel, several tiles, K tail
    (700, 904, 296, True, torch.bfloat16),
    (16, 2048, 512, False, torch.bfloat16),   # skinny kernel
    (16, 2048, 512, True, torch.float32),     # stream kernel
    (256, 256, 256, False, torch.float32),    # the launch-bound 256^3 shape (K-split)
])
def test_capture_and_replay(g, M, N, K, bcol, dt):
    print(f"[graph {M}x{N}x{K} bcol={bcol} {dt}]", flush=True)
    versions, host = [], []
    for v in range(3):
        dist = "int3" if v == 2 else "normal"     # the third version is integer-valued
        A = synth.draw(M, K, dist, 500 + v)
        Bs = synth.draw(N, K, dist, 600 + v) if bcol else synth.draw(K, N, dist, 600 + v)
        versions.append((_dev(A), _dev(Bs)))
        host.append((A, Bs))
    A = versions[0][0].clone()
    Bs = versions[0][1].clone()
    B = Bs.t() if bcol else Bs

    def eager(i):
        Ai, Bi = versions[i]
        out = torch.empty((M, N), dtype=dt, device="cuda")
        g(Ai, Bi.t() if bcol else Bi, out)
        torch.cuda.synchronize()
        return out

    refs = [eager(i) for i in range(3)]
    C = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g(A, B, C)                     # warm-up on the capturing stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g(A, B, C)
    torch.cuda.synchronize()
    for rep in range(6):
        i = rep % 3
        A.copy_(versions[i][0])
        Bs.copy_(versions[i][1])
        C.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        rep_ok = _oracle_check(host_out(C), *host[i], bcol, dt, integer=(i == 2))
        assert rep_ok.ok, f"replay {rep} (version {i}) against the oracle: {rep_ok}"
        assert torch.equal(_bits(C), _bits(refs[i])), f"replay {rep} differs from the eager run"
        _ = (refs[i].float() * 2).sum().item()   # unrelated eager work between replays


def test_capture_and_replay_epilogue_and_mx(g):
    """The fused-epilogue and MX entry points are enqueue-only too: captured
    once, replayed with rewritten inputs, each replay equal to an eager run."""
    print("[graph epilogue + mx]", flush=True)
    M, N, K = 300, 520, 256
    A_np = [synth.draw(M, K, "normal", 700 + v) for v in range(2)]
    B_np = [synth.draw(K, N, "normal", 710 + v, K ** -0.5) for v in range(2)]
    mx_ops = [(synth.draw_mx(M, K, "normal", 720 + v), synth.draw_mx(N, K, "normal", 730 + v))
              for v in range(2)]
    bias = torch.from_numpy(synth.draw_bias(N, 740)).cuda()
    A, B = _dev(A_np[0]), _dev(B_np[0])
    (a8, sa), (b8, sb) = mx_ops[0]
    Am, Bm = torch.from_numpy(a8).cuda(), torch.from_numpy(b8).cuda()
    Sa, Sb = torch.from_numpy(sa).cuda(), torch.from_numpy(sb).cuda()
    C1 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    C2 = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")

    def work():
        g(A, B, C1, bias=bias, act=tg.Act.SILU)
        g.mx(Am, Bm, C2, Sa, Sb, bias=bias, act=tg.Act.RELU)

    def load(v):
        A.copy_(_dev(A_np[v])); B.copy_(_dev(B_np[v]))
        (a8, sa), (b8, sb) = mx_ops[v]
        Am.copy_(torch.from_numpy(a8)); Bm.copy_(torch.from_numpy(b8))
        Sa.copy_(torch.from_numpy(sa)); Sb.copy_(torch.from_numpy(sb))

    refs = []
    for v in range(2):
        load(v)
        work()
        torch.cuda.synchronize()
        refs.append((C1.clone(), C2.clone()))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    torch.cuda.synchronize()
    for rep in range(4):
        v = rep % 2
        load(v)
        C1.fill_(float("nan")); C2.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(C1), _bits(refs[v][0])), f"epilogue replay {rep}"
        assert torch.equal(_bits(C2), _bits(refs[v][1])), f"mx replay {rep}"
        _ = (refs[v][1] * 2).sum().item()
