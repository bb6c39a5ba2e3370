"""The forward captured in a HIP graph and replayed: routing, the expert
forward (staged pair, or the fused Mega launch whose tickets and readiness
counters the planner launch clears on every call) and the combine.  Each
replay runs after eager work on the same buffers and must give the eager
result bit for bit (the path records no memset nodes; every buffer it
clears is cleared by a kernel)."""
import pytest
import torch

from tests._harness import banner, make_inputs, run_forward

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from mixture_experts_routed_03_amd import binding
    binding.lib()
    assert torch.cuda.is_available()
    return binding


@pytest.mark.parametrize("pipeline,prec", [("staged", "bf16"), ("mega", "bf16"),
                                           ("mega", "mxfp8")])
def test_forward_graph_replays_match_eager(B, pipeline, prec):
    banner(f"graph replay {pipeline} {prec}")
    T, D, F, E, K = 300, 512, 256, 12, 3
    lay = make_inputs(T, D, F, E, K, prec, zipf=1.1, seed=90)
    layer = B.MoeLayer(T, D, F, E, K, prec)
    if prec == "mxfp8":
        layer.prepare(lay["w13"], lay["w2"])
    fwd = layer.forward_mega if pipeline == "mega" else layer.forward
    y_graph = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")

    def body():
        layer.route(lay["ids"])
        fwd(lay["x"], lay["w13"], lay["w2"])
        layer.combine(lay["scores"], y_graph)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up off the capture
        body()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    torch.cuda.synchronize()

    def eager():   # the same pipeline, eagerly, on the same workspaces
        y = torch.empty_like(y_graph)
        layer.route(lay["ids"])
        fwd(lay["x"], lay["w13"], lay["w2"])
        layer.combine(lay["scores"], y)
        torch.cuda.synchronize()
        return y

    ref = eager()
    for i in range(3):
        y_graph.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_graph, ref), f"replay {i}"
        # eager work on the same workspaces between replays (the other
        # pipeline too, which writes h2 and the route slots from other XCDs)
        assert torch.equal(eager(), ref)
        run_forward(layer, lay)
        torch.cuda.synchronize()
    assert layer.status()[0] == 0


@pytest.mark.parametrize("mega", [False, True])
def test_training_step_graph_replays_match_eager(B, mega):
    """Forward and backward captured in one graph (BF16; with mega, the fused
    backward, whose tickets and per-block counters the backward's planner
    launch clears on every call): every replay, with eager steps between,
    gives the eager step's gradients bit for bit."""
    banner(f"graph replay training step, fused backward={mega}")
    T, D, F, E, K = 300, 512, 256, 12, 3
    lay = make_inputs(T, D, F, E, K, "bf16", zipf=1.1, seed=91, training=True)
    layer = B.MoeLayer(T, D, F, E, K, "bf16", training=True)
    flags = B.BWD_MEGA if mega else 0
    dev = "cuda"
    y = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    grads = [torch.empty((T, D), dtype=torch.bfloat16, device=dev),
             torch.empty((E, 2 * F, D), dtype=torch.bfloat16, device=dev),
             torch.empty((E, D, F), dtype=torch.bfloat16, device=dev),
             torch.empty((T, K), dtype=torch.float32, device=dev)]

    def step(out):
        layer.route(lay["ids"])
        layer.forward(lay["x"], lay["w13"], lay["w2"])
        layer.combine(lay["scores"], y)
        layer.backward(lay["x"], lay["scores"], lay["dy"], lay["w13"], lay["w2"], out[0], out[1],
                       out[2], out[3], flags=flags)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up off the capture
        step(grads)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(grads)
    torch.cuda.synchronize()

    def eager():
        out = [torch.empty_like(t) for t in grads]
        step(out)
        torch.cuda.synchronize()
        return out

    ref = eager()
    for i in range(3):
        for t in grads:
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for name, u, v in zip(("dx", "dw13", "dw2", "ds"), grads, ref):
            assert torch.equal(u, v), (i, name)
        got = eager()
        for u, v in zip(got, ref):
            assert torch.equal(u, v)
    assert layer.status()[0] == 0
