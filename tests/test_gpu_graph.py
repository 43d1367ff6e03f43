"""The routing step inside a HIP graph, and two steps on concurrent streams.

Every entry point allocates nothing, keeps no state and enqueues only kernels
on the caller's stream (no memset, no host synchronisation), so a whole step
-- route, map, FP8 expand, reduce -- can be captured once and replayed.  Each
replay is compared bit for bit with the eager step, with eager steps on other
inputs (and host synchronisations) in between.  Two independent steps issued
at once on two streams (default priority) give the same bits as run one after
the other.
"""
import pytest
import torch

from moe_routing_amd import synth

pytestmark = pytest.mark.gpu

tk = pytest.importorskip("moe_routing_amd")

T, E, K, H = 4096, 256, 8, 2048


class Step:
    """Inputs and preallocated outputs of one routing step."""

    def __init__(self, seed: int, dev, reduce: str = "tk_reduce"):
        self.reduce = getattr(tk, reduce)
        g = torch.Generator().manual_seed(seed)
        self.logits = torch.randn((T, E), generator=g).to(dev)
        self.bias = (torch.rand(E, generator=g) * 0.2 - 0.1).to(dev)
        self.x = torch.randn((T, H), generator=g).to(torch.bfloat16).to(dev)
        self.y = torch.randn((T * K, H), generator=g).to(torch.bfloat16).to(dev)
        self.opts = tk.RouteOpts(**synth.v3_gate(0)["route"])
        self.idx = torch.empty((T, K), dtype=torch.int32, device=dev)
        self.w = torch.empty((T, K), dtype=torch.float32, device=dev)
        self.counts = torch.empty(E, dtype=torch.int32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        self.pos = torch.empty((T, K), dtype=torch.int32, device=dev)
        self.row_src = torch.empty(T * K, dtype=torch.int32, device=dev)
        self.ws = torch.empty(max(tk.tk_map_workspace_bytes(T, K, E), 16), dtype=torch.uint8,
                              device=dev)
        self.xq = torch.empty((T * K, H), dtype=torch.uint8, device=dev)
        self.sc = torch.empty((T * K, H // 128), dtype=torch.float32, device=dev)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    def run(self):
        tk.tk_route(self.logits, self.bias, K, self.opts, self.idx, self.w)
        tk.tk_map(self.idx, E, 0, E, self.counts, self.offsets, self.pos, self.row_src, self.ws)
        tk.tk_expand_quant(self.x, self.pos, tk.TK_EXPAND_FP8_E4M3_1X128, T * K, self.xq, self.sc)
        self.reduce(self.y, self.pos, self.w, self.out)

    def outputs(self):
        return [self.idx, self.w, self.counts, self.offsets, self.pos, self.row_src, self.xq,
                self.sc, self.out]

    def snapshot(self):
        return [t.clone() for t in self.outputs()]


def _same(a, b):
    return all(torch.equal(u, v) for u, v in zip(a, b))


# both combines: at T=4096, H=2048 tk_reduce_dense takes its staged form (16 tokens per workgroup, one launch)
@pytest.mark.parametrize("reduce", ["tk_reduce", "tk_reduce_dense"])
def test_step_replays_from_a_graph(reduce):
    dev = torch.device("cuda:0")
    s = Step(1, dev, reduce)
    other = Step(2, dev, reduce)
    s.run()
    torch.cuda.synchronize()
    ref = s.snapshot()
    for t in s.outputs():
        t.zero_()
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on the capture stream's side
        s.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        s.run()
    for replay in range(3):
        for t in s.outputs():
            t.zero_()
        other.run()                        # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert _same(s.outputs(), ref), f"replay {replay} differs from the eager step"


@pytest.mark.parametrize("reduce", ["tk_reduce", "tk_reduce_dense"])
def test_two_steps_on_concurrent_streams(reduce):
    dev = torch.device("cuda:0")
    a, b = Step(3, dev, reduce), Step(4, dev, reduce)
    a.run()
    b.run()
    torch.cuda.synchronize()
    ref_a, ref_b = a.snapshot(), b.snapshot()
    for t in a.outputs() + b.outputs():
        t.zero_()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(2):
        with torch.cuda.stream(s1):
            a.run()
        with torch.cuda.stream(s2):
            b.run()
    torch.cuda.synchronize()
    assert _same(a.outputs(), ref_a)
    assert _same(b.outputs(), ref_b)


def test_dense_combine_in_launches_replays_from_a_graph():
    # k=8, H=7168: tk_reduce_dense issues one launch per round of workgroups;
    # T=9000 -> three launches (256 + 256 + 238 workgroups of 12 tokens), all
    # captured in the graph and replayed in order
    dev = torch.device("cuda:0")
    t9, h9 = 9000, 7168
    g = torch.Generator(device=dev)
    g.manual_seed(9)
    y = torch.randn((t9 * K, h9), generator=g, device=dev).to(torch.bfloat16)
    pos = torch.randperm(t9 * K, generator=g, device=dev).to(torch.int32).view(t9, K)
    w = torch.rand((t9, K), generator=g, device=dev)
    out = torch.empty((t9, h9), dtype=torch.bfloat16, device=dev)
    tk.tk_reduce_dense(y, pos, w, out)
    torch.cuda.synchronize()
    ref = out.clone()
    other = Step(5, dev, "tk_reduce_dense")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        tk.tk_reduce_dense(y, pos, w, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        tk.tk_reduce_dense(y, pos, w, out)
    for replay in range(3):
        out.zero_()
        other.run()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {replay} differs from the eager call"
