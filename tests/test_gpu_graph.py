"""The layer (forward, and forward + backward) captured in a HIP graph.

Nothing in the library allocates, synchronises or issues a memset, so a
whole layer call can be captured.  Each graph is replayed several times with
unrelated eager work and synchronisations in between, and every replay must
reproduce the eager result bit for bit (the layer is deterministic).
"""
import numpy as np
import pytest

from gpu_cases import SMALL

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from sparse_mixture_experts_rmsnorm_amd import binding as B  # noqa: E402
from sparse_mixture_experts_rmsnorm_amd import synth  # noqa: E402
from sparse_mixture_experts_rmsnorm_amd.layer import MoELayer  # noqa: E402


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    return "cuda"


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _capture(fn):
    """Warm up on a side stream, then capture fn into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name", ["mixtral_small_drops", "finegrained_small", "bcsr_small",
                                  "atomic_small", "mixtral_small_mxfp8", "bcsr_small_mxfp8",
                                  "persistent_tiles"])
def test_forward_graph_replay(name, dev):
    _say(f"[gpu] graph replay forward {name}")
    wl = SMALL[name]
    inp = synth.make_numpy(wl)
    params = {k: synth.to_device(v, dev) for k, v in inp.items()}
    layer = MoELayer(wl, params, dev)
    x = params["x"]
    ws = layer.alloc_workspace(wl.T)
    stats = torch.zeros(4, dtype=torch.int32, device=dev)
    eager = layer.forward(x, ws=ws, stats=stats).clone()
    eager_stats = stats.clone()
    out = torch.empty_like(x)
    g = _capture(lambda: layer.forward(x, out=out, ws=ws, stats=stats))
    # unrelated eager work between replays: another batch through the same
    # layer on its own workspace
    x2 = torch.randn(x.shape, device=dev).to(x.dtype)
    ws2 = layer.alloc_workspace(wl.T)
    for i in range(3):
        out.zero_()
        stats.zero_()
        other = layer.forward(x2, ws=ws2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(eager)), i
        assert torch.equal(stats, eager_stats), i
        del other


def test_train_step_graph_replay(dev):
    _say("[gpu] graph replay forward + backward")
    wl = SMALL["finegrained_small"]
    inp = synth.make_numpy(wl)
    params = {k: synth.to_device(v, dev) for k, v in inp.items()}
    layer = MoELayer(wl, params, dev, train=True)
    x = params["x"]
    ws = layer.alloc_workspace(wl.T)
    bws = torch.empty(layer.backward_workspace_size(wl.T), dtype=torch.uint8, device=dev)
    rng = np.random.default_rng(3)
    dout = synth.to_device(synth._to_bf16_bits(rng.standard_normal((wl.T, wl.d)).astype(np.float32)), dev)
    layer.forward(x, ws=ws)
    eager = {k: v.clone() for k, v in layer.backward(x, dout, ws, bws=bws).items()}
    out = torch.empty_like(x)
    grads = {k: torch.empty_like(v) for k, v in eager.items()}

    def step():
        layer.forward(x, out=out, ws=ws)
        layer.backward(x, dout, ws, bws=bws, grads=grads)

    g = _capture(step)
    for i in range(3):
        for v in grads.values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in eager.items():
            assert torch.equal(_bits(grads[k]), _bits(v)), (i, k)
