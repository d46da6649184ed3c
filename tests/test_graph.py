"""The library's calls inside a captured HIP graph (torch.cuda.CUDAGraph):
every replay, with other eager work and synchronisations in between, gives
exactly the eager result.  The library enqueues kernels only (no memsets,
no allocation), so capture needs nothing from it beyond the stream it is
handed.
"""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import flashattention_forward_07_amd as fa  # noqa: E402


def _replays_match(run, outs, n_replays=4):
    """Capture run() on a side stream, then replay it several times with
    eager work between the replays and compare with the eager result."""
    run()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    for t in outs:
        t.fill_(float("nan"))
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device="cuda")
    for i in range(n_replays):
        for t in outs:
            t.fill_(float("nan"))
        scratch.mul_(1.0001)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip(outs, eager):
            assert torch.equal(t, e), f"replay {i} differs from the eager result"


@pytest.mark.parametrize("N", [100, 1000])
def test_fwd_in_graph(N):
    print(f"case graph fwd N={N}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(21)
    B, H, d = 2, 4, 128
    q, k, v = (torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).cuda() for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")

    def run():
        fa.fa_fwd(q, k, v, o, lse, B, H, N, d, 1.0 / math.sqrt(d), True, fa.FA_DTYPE_BF16,
                  torch.cuda.current_stream())

    _replays_match(run, [o, lse])


def test_varlen_in_graph():
    print("case graph varlen", flush=True)
    g = torch.Generator(device="cpu").manual_seed(22)
    lens = [5, 300, 77, 1024]
    cu_np = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, d = int(cu_np[-1]), 2, 64
    q, k, v = (torch.randn(T, H, d, generator=g).to(torch.bfloat16).cuda() for _ in range(3))
    cu = torch.from_numpy(cu_np).cuda()
    o = torch.empty_like(q)
    lse = torch.empty(T, H, dtype=torch.float32, device="cuda")

    def run():
        fa.fa_fwd_varlen(q, k, v, o, lse, cu, len(lens), max(lens), H, d, 0.125, True,
                         fa.FA_DTYPE_BF16, torch.cuda.current_stream())

    _replays_match(run, [o, lse])


def test_decode_in_graph():
    """Split-KV decode: two kernels and a workspace whose partial results
    are rewritten on every replay."""
    print("case graph decode", flush=True)
    g = torch.Generator(device="cpu").manual_seed(23)
    B, H, Nq, Nk, d = 2, 8, 2, 5000, 128
    q = torch.randn(B, H, Nq, d, generator=g).to(torch.bfloat16).cuda()
    k, v = (torch.randn(B, H, Nk, d, generator=g).to(torch.bfloat16).cuda() for _ in range(2))
    o = torch.empty_like(q)
    lse = torch.empty(B, H, Nq, dtype=torch.float32, device="cuda")
    need = fa.fa_decode_workspace_bytes(B, H, Nq, Nk, d, 8)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def run():
        fa.fa_decode_fwd(q, k, v, o, lse, ws, need, B, H, Nq, Nk, d, 1.0 / math.sqrt(d), True,
                         fa.FA_DTYPE_BF16, 8, torch.cuda.current_stream())

    _replays_match(run, [o, lse])
