"""Bit-exact routing against the oracle's own routing, at the real shapes.

The routing decision takes floating-point logits to integers, so the GPU and
the oracle can only be required to agree where the logits leave no doubt.
Here every fp32 sum is exact in any order: token rows are +-1, router
weights are small integers times 2^-6, and some router columns are copies of
others, so exact ties occur on every token and must go to the lower expert
index ("Mixture of Experts (MoE)" glossary, top-k gating: the k highest
scores; ties to the lower index is this library's rule).  A bias row skews
the load so that the capacity rule (glossary, expert capacity) drops slots.

On these inputs the selected ids, per-expert counts, offsets, positions,
row order and the dropped set of the whole layer (moe_layer_forward, the
launch configuration the benchmark times) must equal the oracle's routing
from its own float64 logits for every token, with no exceptions.
"""
import numpy as np
import pytest

import oracle as O
from gpu_cases import record

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from sparse_mixture_experts_rmsnorm_amd import binding as B  # noqa: E402
from sparse_mixture_experts_rmsnorm_amd import synth  # noqa: E402
from sparse_mixture_experts_rmsnorm_amd.layer import MoELayer  # noqa: E402
from sparse_mixture_experts_rmsnorm_amd.workloads import WORKLOADS  # noqa: E402

# (workload, duplicated router columns, bias integers in units of 2^-6)
CASES = {
    "mixtral_bf16": ([(0, 1), (4, 5)], [40, 40, 0, -20, 10, 10, -40, 0]),
    "finegrained_bf16": ([(2 * j, 2 * j + 1) for j in range(8)], "zipf"),
    "variable_bcsr_bf16": ([(0, 1), (6, 7)], [60, 60, -30, 0, 20, -64, 10, 10]),
}


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", list(CASES))
def test_integer_exact_routing(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"[gpu] integer-exact routing {name}", flush=True)
    B.lib()
    wl = WORKLOADS[name].scaled(bias="none")
    dup, bias = CASES[name]
    if isinstance(bias, str):
        bias = synth.zipf_bias_int(wl.E, wl.zipf_s, wl.seed)
    ints = synth.make_integer_routing(wl.T, wl.d, wl.E, wl.seed, dup, bias)
    dev = "cuda"
    params = synth.make_torch(wl, dev)
    params["x"] = synth.to_device(ints["x"], dev)
    params["w_router"] = synth.to_device(ints["w_router"], dev)
    layer = MoELayer(wl, params, dev)
    ws = layer.alloc_workspace(wl.T)
    stats = torch.zeros(4, dtype=torch.int32, device=dev)
    layer.forward(params["x"], ws=ws, stats=stats)
    torch.cuda.synchronize()
    rt = layer.routing(wl.T, ws)
    ids = rt["ids"].cpu().numpy()

    # the oracle's own routing from float64 logits
    x = ints["x"]
    r_ref = O.rmsnorm_scale(x, wl.eps)
    l_ref = O.router_logits(x, None, r_ref, ints["w_router"], None)
    own = O.select_topk(l_ref, wl.k)
    srt = -np.sort(-l_ref, axis=1)
    ties = int(np.sum(np.any(srt[:, :wl.k] == srt[:, 1:wl.k + 1], axis=1)))
    cap = O.capacity(wl.T, wl.k, wl.E, wl.cf)
    disp = O.dispatch(own, wl.E, cap, wl.pad)
    print(f"  {name}: tokens with exact ties in the top k+1: {ties}, dropped {disp['dropped']}, "
          f"loads {disp['counts'].min()}..{disp['counts'].max()} (capacity {cap})", flush=True)
    assert ties > 0                      # the ties really are there
    if wl.cf > 0:
        assert disp["dropped"] > 0       # and so are the drops

    bad = int(np.sum(np.any(ids != own, axis=1)))
    print(f"  {name}: tokens whose ids differ from the oracle's: {bad}", flush=True)
    record(f"integer-exact routing {name}", id_mismatch=bad, tie_tokens=ties,
           dropped=int(disp["dropped"]))
    assert bad == 0
    assert np.array_equal(rt["counts"].cpu().numpy(), disp["counts"])
    assert np.array_equal(rt["offsets"].cpu().numpy(), disp["offsets"])
    assert np.array_equal(rt["pos"].cpu().numpy(), disp["pos"])
    row_token = rt["row_token"].cpu().numpy()
    assert np.array_equal(row_token[:disp["rows"]], disp["row_token"])
    assert np.all(row_token[disp["rows"]:] == -1)
    st = stats.cpu().numpy()
    assert st[0] == disp["rows"] and st[1] == disp["dropped"] and st[2] == disp["max_load"]
    assert st[3] == 0
    # the gates on these logits: every r is the same, so the gate values are
    # fixed by the integer sums; fp32 against float64 within 1e-5
    g_ref = O.gates(l_ref, own, wl.renorm)
    assert np.max(np.abs(rt["w"].cpu().numpy() - g_ref)) < 1e-5
