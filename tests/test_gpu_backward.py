"""GPU parity of the backward pass (moe_layer_backward) against the oracle.

The forward runs with save_for_backward on the GPU; the oracle's backward is
evaluated on the GPU's own routing (ids), as in the forward parity tests.
Every gradient (dx, dgamma, router weight and bias, routed and shared
expert weights) is compared as max|gpu - ref| / max|ref|.

Tolerance: the bf16 bound of the forward, 2e-2 of the largest magnitude
per gradient tensor.  The backward's GEMM operands are bf16 (dout scaled by
the gate, r xhat, the saved h and pre-activations, the pre-activation
gradients) with fp32 accumulation, and dx is stored in bf16; each rounding
is at most 2^-9 relative, so even compounded over the two GEMM stages the
error stays an order of magnitude inside the bound.  The measured errors are
printed and kept in the session summary.
"""
import numpy as np
import pytest

import oracle as O
from gpu_cases import SMALL, f64, oracle_params, record, rel_err

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from sparse_mixture_experts_rmsnorm_amd import binding as B  # noqa: E402
from sparse_mixture_experts_rmsnorm_amd import synth  # noqa: E402
from sparse_mixture_experts_rmsnorm_amd.layer import MoELayer  # noqa: E402

TOL_BWD = 2e-2

CASES = {
    "mixtral_small_drops": SMALL["mixtral_small_drops"],          # SwiGLU, bias, drops
    "gelu_gamma_switch": SMALL["gelu_gamma_switch"],              # gain, k = 1
    "gelu_tanh_dense_mixture": SMALL["gelu_tanh_dense_mixture"],  # k = E
    "bcsr_small": SMALL["bcsr_small"],                            # BCSR (padded rows)
    "finegrained_small": SMALL["finegrained_small"],              # E = 64, shared SwiGLU
    "swiglu_full_softmax": SMALL["mixtral_small"].scaled(name="swiglu_full_softmax", renorm=0,
                                                         gamma=True, bias="normal", ffn=384,
                                                         T=333, seed=21),
}


def _say(*a):
    print(*a, flush=True)


def pack_w13(dw1, dw3, sizes):
    """The pages' first-linear gradients [d, F] in the packed w13_t layout."""
    if dw3 is None:
        return dw1.T
    d, F = dw1.shape
    out = np.empty((2 * F, d))
    k = np.arange(2 * F)
    grp, sel, c = k // 64, (k % 64) // 32, k % 32
    f = grp * 32 + c
    out[sel == 0] = dw1[:, f[sel == 0]].T
    out[sel == 1] = dw3[:, f[sel == 1]].T
    return out


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    return "cuda"


@pytest.mark.parametrize("name", list(CASES))
def test_backward_parity(name, dev):
    _say(f"[gpu] backward parity {name}")
    wl = CASES[name]
    inp = synth.make_numpy(wl)
    params = {k: synth.to_device(v, dev) for k, v in inp.items()}
    layer = MoELayer(wl, params, dev, train=True)
    x = params["x"]
    ws = layer.alloc_workspace(wl.T)
    layer.forward(x, ws=ws)
    rng = np.random.default_rng(wl.seed + 7)
    dout_np = synth._to_bf16_bits(rng.standard_normal((wl.T, wl.d)).astype(np.float32))
    dout = synth.to_device(dout_np, dev)
    g1 = layer.backward(x, dout, ws)
    torch.cuda.synchronize()
    ids = layer.routing(wl.T, ws)["ids"].cpu().numpy()
    # a second backward on the same saved state gives the same bits
    g2 = layer.backward(x, dout, ws)
    torch.cuda.synchronize()
    for key in g1:
        assert torch.equal(g1[key].view(torch.int16) if g1[key].dtype == torch.bfloat16 else g1[key],
                           g2[key].view(torch.int16) if g2[key].dtype == torch.bfloat16 else g2[key]), key

    p = oracle_params(wl, inp)
    ref = O.layer_backward(p, inp["x"], dout_np, ids_override=ids)
    got = {k: (f64(synth.to_host(v)) if v.dtype == torch.bfloat16 else v.cpu().numpy().astype(np.float64))
           for k, v in g1.items()}
    checks = [("dx", ref["dx"]), ("dw_router", ref["dw_router"].T),
              ("dw13", pack_w13(ref["dw1"], ref["dw3"], wl.sizes)), ("dw2", ref["dw2"])]
    if "dbias" in got:
        checks.append(("dbias", ref["dbias"]))
    if "dgamma" in got:
        checks.append(("dgamma", ref["dgamma"]))
    if "dws13" in got:
        checks += [("dws13", pack_w13(ref["dws1"], ref["dws3"], [wl.shared_ffn])),
                   ("dws2", ref["dws2"])]
    errs = {k: rel_err(got[k], v) for k, v in checks}
    _say("  " + ", ".join(f"{k} {e:.2e}" for k, e in errs.items()))
    for k, e in errs.items():
        assert e <= TOL_BWD, (k, e)
    # dx without the residual's identity term (whose bf16 rounding in dx
    # would otherwise hide the error of the expert, router and norm terms)
    layer.desc.residual = 0
    g0 = layer.backward(x, dout, ws)
    layer.desc.residual = 1
    torch.cuda.synchronize()
    ref0 = O.layer_backward(dict(p, residual=False), inp["x"], dout_np, ids_override=ids)
    e0 = rel_err(f64(synth.to_host(g0["dx"])), ref0["dx"])
    _say(f"  dx without the residual {e0:.2e}")
    record(f"backward {name}", **errs, dx_no_residual=e0)
    assert e0 <= TOL_BWD


def test_backward_argument_checks(dev):
    wl = SMALL["mixtral_small"]
    inp = synth.make_numpy(wl)
    params = {k: synth.to_device(v, dev) for k, v in inp.items()}
    inference = MoELayer(wl, params, dev)
    assert B.lib().moe_layer_backward_workspace_size(B.C.byref(inference.desc), wl.T) == 0
    assert "save_for_backward" in B.last_error()
    layer = MoELayer(wl, params, dev, train=True)
    ws = layer.alloc_workspace(wl.T)
    small = torch.empty(16, dtype=torch.uint8, device=dev)
    with pytest.raises(B.MoeError, match="forward workspace"):
        layer.backward(params["x"], params["x"], small)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["mixtral_bf16", "finegrained_bf16"])
def test_backward_fullsize(name, dev):
    """The backward at the full workload sizes, in the configuration the
    benchmark times.  Checked on what the oracle can compute in pieces: dx of
    sampled tokens (with and without the residual), and the routed and shared
    expert weight gradients on sampled hidden units of a few experts (the FFN
    is separable over hidden units).  The router and gain gradients sum every
    token's expert outputs; they are checked at the small sizes above."""
    from sparse_mixture_experts_rmsnorm_amd.workloads import WORKLOADS
    _say(f"[gpu] full-size backward {name}")
    wl = WORKLOADS[name]
    params = synth.make_torch(wl, dev)
    layer = MoELayer(wl, params, dev, train=True)
    x = params["x"]
    ws = layer.alloc_workspace(wl.T)
    layer.forward(x, ws=ws)
    gen = torch.Generator(device=dev).manual_seed(wl.seed + 7)
    dout = torch.randn((wl.T, wl.d), generator=gen, device=dev).to(torch.bfloat16)
    g = layer.backward(x, dout, ws)
    layer.desc.residual = 0
    g0 = layer.backward(x, dout, ws, grads={k: torch.empty_like(v) for k, v in g.items()})
    layer.desc.residual = 1
    torch.cuda.synchronize()
    ids = layer.routing(wl.T, ws)["ids"].cpu().numpy()
    inp = {k: synth.to_host(v) for k, v in params.items()}
    dout_np = synth.to_host(dout)
    p = oracle_params(wl, inp)
    rng = np.random.default_rng(wl.seed)
    tok = np.sort(rng.choice(wl.T, size=12, replace=False))
    _say(f"  oracle: dx of {len(tok)} tokens")
    ref = O.layer_backward(p, inp["x"], dout_np, ids_override=ids, tokens=tok)
    ref0 = O.layer_backward(dict(p, residual=False), inp["x"], dout_np, ids_override=ids, tokens=tok)
    e_dx = rel_err(f64(synth.to_host(g["dx"]))[tok], ref["dx"])
    e_dx0 = rel_err(f64(synth.to_host(g0["dx"]))[tok], ref0["dx"])
    # expert weight gradients on sampled units
    foff = wl.f_offsets
    sw = wl.act == "swiglu"
    dw13 = g["dw13"].cpu().numpy()
    dw2 = g["dw2"].cpu().numpy()
    errs = []
    for e in (0, wl.E - 1):
        units = np.sort(rng.choice(wl.sizes[e], size=32, replace=False))
        _say(f"  oracle: expert {e}, {len(units)} units")
        u = O.expert_unit_grads(p, inp["x"], dout_np, ids, e, units)
        f = foff[e] + units
        rows1 = 2 * foff[e] + (units // 32) * 64 + units % 32 if sw else f
        errs.append(rel_err(dw13[rows1], u["dw1"].T))
        if sw:
            errs.append(rel_err(dw13[rows1 + 32], u["dw3"].T))
        errs.append(rel_err(dw2[f], u["dw2"]))
    if wl.shared_ffn:
        units = np.sort(rng.choice(wl.shared_ffn, size=32, replace=False))
        x64 = f64(inp["x"])
        r = O.rmsnorm_scale(x64, wl.eps)
        ssw = wl.shared_act == "swiglu"
        b = O.ffn_backward(x64, r, f64(inp["ws1"])[:, units], f64(inp["ws2"])[units, :],
                           wl.shared_act, f64(dout_np), f64(inp["ws3"])[:, units] if ssw else None)
        dws13 = g["dws13"].cpu().numpy()
        rows1 = (units // 32) * 64 + units % 32 if ssw else units
        errs.append(rel_err(dws13[rows1], b["dw1"].T))
        if ssw:
            errs.append(rel_err(dws13[rows1 + 32], b["dw3"].T))
        errs.append(rel_err(g["dws2"].cpu().numpy()[units], b["dw2"]))
    _say(f"  {name}: dx {e_dx:.2e}, dx without residual {e_dx0:.2e}, "
         f"sampled weight gradients max {max(errs):.2e}")
    record(f"full-size backward {name}", dx=e_dx, dx_no_residual=e_dx0, dw_sampled=max(errs))
    assert e_dx <= TOL_BWD and e_dx0 <= TOL_BWD
    assert max(errs) <= TOL_BWD


def test_backward_empty_experts_and_tiny_batch(dev):
    """Experts that receive no rows get exactly zero weight gradients (their
    weight-gradient tiles have K = 0), a batch smaller than one tile works,
    and T = 0 is a no-op."""
    _say("[gpu] backward: empty experts, tiny batch, T = 0")
    wl = SMALL["mixtral_small"].scaled(name="tiny_bwd", T=9, E=8, k=2, bias="normal", seed=23)
    inp = synth.make_numpy(wl)
    b = np.asarray(O.as_f64(inp["bias"]), dtype=np.float32) if inp.get("bias") is not None else None
    bias = np.zeros(wl.E, dtype=np.float32) if b is None else b.copy()
    bias[[3, 6]] = -1e4                       # never selected (k < E)
    inp["bias"] = bias
    params = {k: synth.to_device(v, dev) for k, v in inp.items()}
    layer = MoELayer(wl, params, dev, train=True)
    x = params["x"]
    ws = layer.alloc_workspace(wl.T)
    layer.forward(x, ws=ws)
    rng = np.random.default_rng(5)
    dout_np = synth._to_bf16_bits(rng.standard_normal((wl.T, wl.d)).astype(np.float32))
    g = layer.backward(x, synth.to_device(dout_np, dev), ws)
    torch.cuda.synchronize()
    ids = layer.routing(wl.T, ws)["ids"].cpu().numpy()
    assert not np.isin(ids, [3, 6]).any()
    foff = wl.f_offsets
    dw13 = g["dw13"].cpu().numpy()
    dw2 = g["dw2"].cpu().numpy()
    for e in (3, 6):
        assert not dw13[2 * foff[e]:2 * foff[e + 1]].any()
        assert not dw2[foff[e]:foff[e + 1]].any()
    p = oracle_params(wl, inp)
    ref = O.layer_backward(p, inp["x"], dout_np, ids_override=ids)
    assert rel_err(f64(synth.to_host(g["dx"])), ref["dx"]) <= TOL_BWD
    assert rel_err(dw13, pack_w13(ref["dw1"], ref["dw3"], wl.sizes)) <= TOL_BWD
    assert rel_err(dw2, ref["dw2"]) <= TOL_BWD
    # T = 0
    x0 = x[:0]
    ws0 = layer.alloc_workspace(0)
    layer.forward(x0, ws=ws0)
    g0 = layer.backward(x0, x0, ws0)
    torch.cuda.synchronize()
    assert g0["dx"].numel() == 0
