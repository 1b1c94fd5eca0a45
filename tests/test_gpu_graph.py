"""tile_gemm_run is enqueue-only (no allocation, no synchronisation), so it can
be captured into a HIP graph and replayed: the split between preparing work
once and replaying it that "Rust Compute Kernels" describes (section "Why
scoped graph capture helps borrowing").

Each replay is checked against an eager run of the same operands, with eager
work and synchronisation between replays, and with the captured inputs
rewritten in place between replays (a graph keeps its pointers, not their
contents).
"""

import numpy as np
import pytest

import tile_partitioned_dense_amd as tg
from tile_partitioned_dense_amd import synth

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


@pytest.mark.parametrize("M,N,K,bcol,dt", [
    (700, 904, 296, False, torch.float32),    # tile kernel, several tiles, K tail
    (700, 904, 296, True, torch.bfloat16),
    (16, 2048, 512, False, torch.bfloat16),   # skinny kernel
])
def test_capture_and_replay(g, M, N, K, bcol, dt):
    print(f"[graph {M}x{N}x{K} bcol={bcol} {dt}]", flush=True)
    versions = []
    for v in range(3):
        A = synth.draw(M, K, "normal", 500 + v)
        Bs = synth.draw(N, K, "normal", 600 + v) if bcol else synth.draw(K, N, "normal", 600 + v)
        versions.append((_dev(A), _dev(Bs)))
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
        assert torch.equal(_bits(C), _bits(refs[i])), f"replay {rep} differs from the eager run"
        _ = (refs[i].float() * 2).sum().item()   # unrelated eager work between replays
