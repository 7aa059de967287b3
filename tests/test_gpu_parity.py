"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Integer results (ids, counts, offsets, permutation, dropped set, topology)
must match bit-exactly; floating-point outputs within max|gpu-ref|/max|ref|
of 1e-3 (fp32) or 2e-2 (bf16).  Routing follows a stage-wise protocol: the
top-k decision is checked bit-exactly on the GPU's own logits, then every
later stage is compared on the GPU's ids.
"""
import numpy as np
import pytest

import oracle as O
from gpu_cases import (SMALL, TOL, check_ids_against_reference, f64, oracle_params, record,
                       rel_err)

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
    B.lib()   # fail loudly if the library is missing
    return "cuda"


def _setup(name, dev):
    wl = SMALL[name]
    inp = synth.make_numpy(wl)
    params = {k: synth.to_device(v, dev) for k, v in inp.items()}
    layer = MoELayer(wl, params, dev)
    return wl, inp, params, layer


def _gpu_logits(wl, layer, params, r):
    """Run the router alone with its logits output (fp32)."""
    T = wl.T
    x = params["xg"] if "xg" in params else params["x"]
    E = wl.E if wl.router == "dense" else wl.Nr + wl.Nc
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    ids = torch.empty((T, wl.k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, wl.k), dtype=torch.float32, device=x.device)
    nws = B.router_workspace_size(layer.desc.router, T)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=x.device)
    B.router_topk(layer.desc.router, x, wl.k, wl.renorm, ids, w, r_in=r, logits=logits, ws=ws)
    return logits, ids, w


def _standalone_dispatch(rt, E, cap, pad, dev):
    """moe_dispatch on a layer's ids / gates / r; returns its outputs by name."""
    T, k = rt["ids"].shape
    R = B.rows_max(T, k, E, cap, pad)
    i32, f32 = dict(dtype=torch.int32, device=dev), dict(dtype=torch.float32, device=dev)
    out = dict(counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
               pos=torch.empty((T, k), **i32), row_token=torch.empty(R, **i32),
               row_r=torch.empty(R, **f32), row_w=torch.empty(R, **f32),
               row_expert=torch.empty(R, **i32))
    stats = torch.zeros(4, **i32)
    ws = torch.empty(max(B.dispatch_workspace_size(T, k, E), 1), dtype=torch.uint8, device=dev)
    B.dispatch(rt["ids"], rt["w"], rt["r"], E, cap, pad, R, out, stats=stats, ws=ws)
    torch.cuda.synchronize()
    return dict(out, stats=stats)


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_parity(name, dev):
    _say(f"[gpu] layer parity {name}")
    wl, inp, params, layer = _setup(name, dev)
    x = params["x"]
    ws = layer.alloc_workspace(wl.T)
    stats = torch.zeros(4, dtype=torch.int32, device=dev)
    out = layer.forward(x, ws=ws, stats=stats)
    torch.cuda.synchronize()
    rt = layer.routing(wl.T, ws)
    ids = rt["ids"].cpu().numpy()
    w = rt["w"].cpu().numpy()
    r = rt["r"].cpu().numpy()
    p = oracle_params(wl, inp)

    # r: RMSNorm statistic
    r_ref = O.rmsnorm_scale(inp["x"], wl.eps)
    assert rel_err(r, r_ref) < 1e-5

    # router: bit-exact selection on the GPU's logits, logits within tolerance
    if wl.gamma:
        xg = torch.empty_like(x)
        B.rmsnorm_stats(x, wl.eps, torch.empty(wl.T, device=dev), gamma=params["gamma"], xg=xg)
        params["xg"] = xg
    logits, ids2, w2 = _gpu_logits(wl, layer, params, rt["r"])
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    assert np.array_equal(ids2.cpu().numpy(), ids)          # the same decision twice
    if wl.router == "dense":
        assert np.array_equal(O.select_topk(lg, wl.k), ids)
        if wl.gamma and wl.dtype == "bf16":
            # with a gain the router reads x * gamma stored as bf16 (the
            # product of two bf16 values is exact in fp32, so the rounding is
            # the oracle's): bit-exact, then the logits on that operand
            xg_ref = O.f64_to_bf16_bits(O.as_f64(inp["x"]) * O.as_f64(inp["gamma"]))
            assert np.array_equal(synth.to_host(params["xg"]), xg_ref)
            l_ref = O.router_logits(xg_ref, None, r_ref, inp["w_router"], inp.get("bias"))
        else:
            l_ref = O.router_logits(inp["x"], inp.get("gamma"), r_ref, inp["w_router"],
                                    inp.get("bias"))
        e_l = rel_err(lg, l_ref)
        assert e_l < (1e-5 if wl.dtype == "f32" else 1e-4), e_l
        g_ref = O.gates(lg.astype(np.float64), ids, wl.renorm)
        assert rel_err(w, g_ref) < 1e-5
        # against the oracle's own routing: only near-ties may differ
        check_ids_against_reference(ids, O.select_topk(l_ref, wl.k), -np.sort(-l_ref, axis=1),
                                    wl.k, 1e-5 * np.max(np.abs(l_ref)))
    else:
        s1, s2 = lg[:, :wl.Nr], lg[:, wl.Nr:]
        sel, sc = O.cartesian_topk(s1, s2, wl.k)               # float32 sums, as the kernel
        assert np.array_equal(sel, ids)
        s1r, s2r = O.cartesian_scores(inp["x"], inp.get("gamma"), r_ref, inp["k_rows"], inp["k_cols"])
        assert rel_err(lg, np.hstack([s1r, s2r])) < 1e-4
        own, own_sc = O.cartesian_topk(s1r, s2r, wl.k)
        top = O.cartesian_topk(s1r, s2r, wl.k + 1)[1]
        check_ids_against_reference(ids, own, top, wl.k, 1e-5 * np.max(np.abs(own_sc[:, 0])))
        e = np.exp(sc.astype(np.float64) - sc[:, :1])
        assert rel_err(w, e / e.sum(axis=1, keepdims=True)) < 1e-5

    # dispatch on the GPU's ids: bit-exact.  A layer of atomic experts reads
    # its routing by token and runs no dispatch: the standalone dispatch (the
    # expert-sorted task list) is checked on the same ids instead.
    E = wl.E if wl.router == "dense" else wl.Nr * wl.Nc
    cap = O.capacity(wl.T, wl.k, E, wl.cf)
    disp = O.dispatch(ids, E, cap, wl.pad)
    st = stats.cpu().numpy()
    if wl.expert_kind == "atomic":
        assert st[0] == wl.T * wl.k and st[1] == 0 and st[2] == -1 and st[3] == 0
        rt = _standalone_dispatch(rt, E, cap, wl.pad, dev)
    assert np.array_equal(rt["counts"].cpu().numpy(), disp["counts"])
    assert np.array_equal(rt["offsets"].cpu().numpy(), disp["offsets"])
    pos = rt["pos"].cpu().numpy()
    assert np.array_equal(pos, disp["pos"])
    rows = disp["rows"]
    row_token = rt["row_token"].cpu().numpy()
    assert np.array_equal(row_token[:rows], disp["row_token"])
    assert np.all(row_token[rows:] == -1)
    kept = pos >= 0
    row_w = rt["row_w"].cpu().numpy()
    row_r = rt["row_r"].cpu().numpy()
    assert np.array_equal(row_w[pos[kept]], w[kept])
    assert np.array_equal(row_r[pos[kept]], r[np.nonzero(kept)[0]])
    if "stats" in rt:
        st = rt["stats"].cpu().numpy()
    assert st[0] == rows and st[1] == disp["dropped"] and st[2] == disp["max_load"] and st[3] == 0

    # whole layer on the GPU's routing
    ref = O.layer_forward(p, inp["x"], ids_override=ids)
    out_np = f64(synth.to_host(out))
    tol = TOL[wl.dtype]
    e_out = rel_err(out_np, ref["out"])
    # the experts alone (no residual): the bf16 rounding of x + moe would
    # otherwise hide the expert path's own error
    layer.desc.residual = 0
    moe = layer.forward(x, ws=ws)
    layer.desc.residual = 1
    torch.cuda.synchronize()
    p0 = dict(p, residual=False)
    ref0 = O.layer_forward(p0, inp["x"], ids_override=ids)
    moe_np = f64(synth.to_host(moe))
    e_moe = rel_err(moe_np, ref0["out"])
    _say(f"  {name}: rel err out {e_out:.2e}, experts only {e_moe:.2e}, dropped {disp['dropped']}")
    record(f"layer {name}", out=e_out, experts_only=e_moe, dropped=int(disp["dropped"]))
    assert e_out <= tol
    assert e_moe <= tol
    if wl.quant != "none":
        # MXFP8 experts: the oracle's MXFP8 layer is much closer than its
        # unquantised one (the quantisation really happens, and as specified)
        ref_fp = O.layer_forward(dict(p0, quant=None), inp["x"], ids_override=ids)
        e_fp = rel_err(moe_np, ref_fp["out"])
        _say(f"  {name}: experts only vs the unquantised oracle {e_fp:.2e}")
        assert e_moe < 0.5 * e_fp
    # fully dropped tokens pass through bit-exactly (and get exactly 0 without the
    # residual) -- unless always-on shared experts add to every token
    gone = np.all(pos < 0, axis=1)
    if gone.any() and not wl.shared_ffn:
        xb = synth.to_host(x)
        assert np.array_equal(synth.to_host(out)[gone], xb[gone])
        assert np.all(f64(synth.to_host(moe))[gone] == 0)


def test_side_stream_forward(dev):
    """The layer run on a side stream, with its output and workspace left to
    the wrapper, gives the bits of the run on the current stream; the
    side stream's buffers are reused by later work on that stream while
    the default stream is kept busy."""
    _say("[gpu] forward on a side stream")
    wl, inp, params, layer = _setup("mixtral_small_drops", dev)
    x = params["x"]
    ref = layer.forward(x).clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        o = layer.forward(x, stream=side)
        o.record_stream(side)
        with torch.cuda.stream(side):
            outs.append(o.clone())
        # unrelated work on the default stream meanwhile
        torch.randn(1 << 20, device=dev).sum()
    side.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("name", ["mixtral_small_drops", "finegrained_small", "atomic_small"])
def test_determinism(name, dev):
    _say(f"[gpu] determinism {name}")
    wl, inp, params, layer = _setup(name, dev)
    ws = layer.alloc_workspace(wl.T)
    a = layer.forward(params["x"], ws=ws).clone()
    ra = {k: v.clone() for k, v in layer.routing(wl.T, ws).items() if torch.is_tensor(v)}
    b = layer.forward(params["x"], ws=ws)
    rb = layer.routing(wl.T, ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
    for k, v in ra.items():
        assert torch.equal(v, rb[k]), k


@pytest.mark.parametrize("E,k,cap,pad,T", [(8, 2, 5, 1, 40), (8, 2, 1000, 128, 300),
                                           (64, 6, 30, 1, 1000), (5, 3, 2, 4, 1),
                                           (256, 8, 7, 1, 513), (3000, 4, 10 ** 6, 1, 777),
                                           (16, 4, 6000, 1, 20000),
                                           (1 << 20, 32, 10 ** 6, 1, 300),
                                           # 16384 slots in groups padded to 128 rows;
                                           # 256 experts at k=6 with a ragged T
                                           (8, 2, 8192, 128, 8192), (256, 6, 40, 1, 2730),
                                           # 2048 experts: a count table of 4 chunks that
                                           # the rank launch scans itself (one thread
                                           # per expert), and one of 18 chunks (over
                                           # 2^15 entries) that takes the separate scan
                                           (2048, 2, 50, 1, 1000), (2048, 2, 50, 1, 4500)])
def test_dispatch_bit_exact(E, k, cap, pad, T, dev):
    _check_dispatch(E, k, cap, pad, T, 256, "bf16", dev)


# rows of 2 KB and more: the rank launch copies them itself (its blocks split
# each chunk's rows; the last chunk's blocks zero the padding rows)
@pytest.mark.parametrize("E,k,cap,pad,T,d,xdt", [(8, 2, 5, 1, 40, 1024, "bf16"),
                                                 (64, 6, 30, 1, 1000, 1024, "bf16"),
                                                 (8, 2, 8192, 128, 8192, 2048, "bf16"),
                                                 (16, 4, 6000, 1, 3000, 512, "f32")])
def test_dispatch_gather_wide_rows(E, k, cap, pad, T, d, xdt, dev):
    _check_dispatch(E, k, cap, pad, T, d, xdt, dev)


def _check_dispatch(E, k, cap, pad, T, d, xdt, dev):
    _say(f"[gpu] dispatch E={E} k={k} cap={cap} pad={pad} T={T} d={d} {xdt}")
    rng = np.random.default_rng(E + k + T)
    # skewed ids (many ties in token order), distinct within a token
    pop = rng.zipf(1.3, size=E * 4) % E
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        ch = []
        while len(ch) < k:
            e = int(pop[rng.integers(0, len(pop))]) if rng.random() < 0.7 else int(rng.integers(0, E))
            if e not in ch:
                ch.append(e)
        ids[t] = ch
    w = rng.random((T, k)).astype(np.float32)
    r = rng.random(T).astype(np.float32)
    capc = min(cap, T)
    R = B.rows_max(T, k, E, capc, pad)
    out = dict(counts=torch.empty(E, dtype=torch.int32, device=dev),
               offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
               pos=torch.empty((T, k), dtype=torch.int32, device=dev),
               row_token=torch.empty(max(R, 1), dtype=torch.int32, device=dev),
               row_r=torch.empty(max(R, 1), dtype=torch.float32, device=dev),
               row_w=torch.empty(max(R, 1), dtype=torch.float32, device=dev),
               row_expert=torch.empty(max(R, 1), dtype=torch.int32, device=dev))
    if xdt == "bf16":
        xb = O.f64_to_bf16_bits(rng.standard_normal((T, d)))
        x = synth.to_device(xb, dev)
    else:
        xb = rng.standard_normal((T, d)).astype(np.float32)
        x = torch.from_numpy(xb).to(dev)
    x_perm = torch.empty((max(R, 1), d), dtype=x.dtype, device=dev) if E <= 2048 else None
    stats = torch.zeros(4, dtype=torch.int32, device=dev)
    ws = torch.empty(B.dispatch_workspace_size(T, k, E), dtype=torch.uint8, device=dev)
    B.dispatch(torch.from_numpy(ids).to(dev), torch.from_numpy(w).to(dev), torch.from_numpy(r).to(dev),
               E, capc, pad, R, out, x=x if x_perm is not None else None, x_perm=x_perm,
               stats=stats, ws=ws)
    torch.cuda.synchronize()
    ref = O.dispatch(ids, E, capc, pad)
    assert np.array_equal(out["counts"].cpu().numpy(), ref["counts"])
    assert np.array_equal(out["offsets"].cpu().numpy(), ref["offsets"])
    assert np.array_equal(out["pos"].cpu().numpy(), ref["pos"])
    rows = ref["rows"]
    rtok = out["row_token"].cpu().numpy()
    assert np.array_equal(rtok[:rows], ref["row_token"])
    assert np.all(rtok[rows:R] == -1)
    rex = out["row_expert"].cpu().numpy()[:rows]
    valid = ref["row_token"] >= 0
    exp_of_row = np.repeat(np.arange(E), np.diff(ref["offsets"]))
    assert np.array_equal(rex[valid], exp_of_row[valid]) and np.all(rex[~valid] == -1)
    pos = ref["pos"]
    kept = pos >= 0
    assert np.array_equal(out["row_w"].cpu().numpy()[pos[kept]], w[kept])
    assert np.array_equal(out["row_r"].cpu().numpy()[pos[kept]], r[np.nonzero(kept)[0]])
    st = stats.cpu().numpy()
    assert st[0] == rows and st[1] == ref["dropped"] and st[2] == ref["max_load"] and st[3] == 0
    if x_perm is not None:
        xp = synth.to_host(x_perm)[:rows] if xdt == "bf16" else x_perm.cpu().numpy()[:rows]
        want = np.where(ref["row_token"][:, None] >= 0, xb[np.maximum(ref["row_token"], 0)], 0)
        assert np.array_equal(xp, want.astype(xb.dtype))


def test_dispatch_counts_bad_ids(dev):
    _say("[gpu] dispatch with out-of-range ids")
    T, k, E = 50, 2, 8
    ids = np.tile(np.array([[0, 1]], dtype=np.int32), (T, 1))
    ids[3, 1] = 9
    ids[7, 0] = -2
    R = B.rows_max(T, k, E, T, 1)
    out = {n: torch.empty(sz, dtype=torch.int32, device=dev) for n, sz in
           [("counts", E), ("offsets", E + 1), ("pos", (T, k)), ("row_token", R)]}
    out["row_r"] = torch.empty(R, device=dev)
    out["row_w"] = torch.empty(R, device=dev)
    stats = torch.zeros(4, dtype=torch.int32, device=dev)
    ws = torch.empty(B.dispatch_workspace_size(T, k, E), dtype=torch.uint8, device=dev)
    B.dispatch(torch.from_numpy(ids).to(dev), torch.ones((T, k), device=dev), torch.ones(T, device=dev),
               E, T, 1, R, out, stats=stats, ws=ws)
    torch.cuda.synchronize()
    pos = out["pos"].cpu().numpy()
    assert pos[3, 1] == -1 and pos[7, 0] == -1
    assert stats.cpu().numpy()[3] == 2
    assert out["counts"].cpu().numpy()[:2].tolist() == [T - 1, T - 1]


def test_topology_matches_oracle(dev):
    _say("[gpu] BCSR topology")
    sizes = [2048] + [1024] * 7
    lay = O.expert_layout([(1, 2048), (7, 1024)], 8, 128)
    tb = [5, 0, 2, 9, 1, 1, 3, 4]
    offsets = np.concatenate([[0], np.cumsum(np.array(tb) * 128)]).astype(np.int32)
    rows_max = int(offsets[-1]) + 3 * 128
    ref = O.bcsr_topology(offsets, lay["size_blocks"], lay["block_offsets"], 128)
    nnz_max = B.topology_nnz_max(rows_max, 128, sizes)
    ro = torch.full((rows_max // 128 + 1,), -7, dtype=torch.int32, device=dev)
    ci = torch.full((nnz_max,), -7, dtype=torch.int32, device=dev)
    nnz = torch.zeros(1, dtype=torch.int32, device=dev)
    t = lambda a: torch.tensor(a, dtype=torch.int32, device=dev)  # noqa: E731
    B.build_topology(t(offsets), t(lay["size_blocks"]), t(lay["block_offsets"]), 8, 128, rows_max,
                     ro, ci, nnz)
    torch.cuda.synchronize()
    n = int(nnz.item())
    assert n == ref["nnz"]
    rb = ref["block_rows"]
    assert np.array_equal(ro.cpu().numpy()[:rb + 1], ref["row_offsets"])
    assert np.all(ro.cpu().numpy()[rb + 1:] == n)
    assert np.array_equal(ci.cpu().numpy()[:n], ref["column_indices"])


def test_empty_batch(dev):
    _say("[gpu] T = 0")
    wl, inp, params, layer = _setup("mixtral_small", dev)
    x = params["x"][:0]
    out = layer.forward(x)
    torch.cuda.synchronize()
    assert out.shape == (0, wl.d)


@pytest.mark.parametrize("renorm", [1, 0])
def test_cartesian_topk_ties(dev, renorm):
    """Key tables with repeated columns: many rows / columns score exactly alike
    and many pair sums tie, so every selection decides ties by index."""
    _say(f"[gpu] Cartesian top-k with exact ties, renorm={renorm}")
    rng = np.random.default_rng(77)
    T, d, Nr, Nc, k = 300, 256, 128, 128, 8
    base_r = rng.standard_normal((d, 16)).astype(np.float32) * 0.05
    base_c = rng.standard_normal((d, 8)).astype(np.float32) * 0.05
    kr = np.ascontiguousarray(base_r[:, rng.permutation(np.arange(Nr) % 16)])
    kc = np.ascontiguousarray(base_c[:, rng.permutation(np.arange(Nc) % 8)])
    x = rng.standard_normal((T, d)).astype(np.float32)
    to_bf16 = lambda a: torch.from_numpy(a).to(dev).to(torch.bfloat16)  # noqa: E731
    keys_t = torch.empty((Nr + Nc, d), dtype=torch.bfloat16, device=dev)
    B.pack_transpose(to_bf16(kr), keys_t[:Nr])
    B.pack_transpose(to_bf16(kc), keys_t[Nr:])
    R = B.RouterDesc()
    R.kind, R.E, R.Nr, R.Nc, R.keys_t = B.ROUTER_CARTESIAN, Nr * Nc, Nr, Nc, keys_t.data_ptr()
    xb = to_bf16(x)
    logits = torch.empty((T, Nr + Nc), dtype=torch.float32, device=dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    r = torch.empty(T, dtype=torch.float32, device=dev)
    ws = torch.empty(max(B.router_workspace_size(R, T), 1), dtype=torch.uint8, device=dev)
    B.router_topk(R, xb, k, renorm, ids, w, r_out=r, logits=logits, ws=ws)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    s1, s2 = lg[:, :Nr], lg[:, Nr:]
    # the ties are really there: 16 distinct row scores and 8 distinct column scores
    assert max(len(np.unique(s1[t])) for t in range(T)) <= 16
    assert max(len(np.unique(s2[t])) for t in range(T)) <= 8
    sel, sc = O.cartesian_topk(s1, s2, k)
    assert np.array_equal(ids.cpu().numpy(), sel)
    got = w.cpu().numpy().astype(np.float64)
    if renorm:
        e = np.exp(sc.astype(np.float64) - sc[:, :1])
        ref = e / e.sum(axis=1, keepdims=True)
    else:
        full = s1.astype(np.float64)[:, :, None] + s2.astype(np.float64)[:, None, :]
        m = full.reshape(T, -1).max(axis=1)
        z = np.exp(full.reshape(T, -1) - m[:, None]).sum(axis=1)
        ref = np.exp(sc.astype(np.float64) - m[:, None]) / z[:, None]
    assert rel_err(got, ref) < 1e-5


@pytest.mark.parametrize("E,k,renorm,T", [(8, 2, 1, 333), (64, 6, 0, 333), (160, 40, 1, 333),
                                          (32, 4, 1, 8200), (64, 6, 1, 16400)])
def test_dense_topk_ties(dev, E, k, renorm, T):
    """Router columns repeated: logits tie exactly and the top-k must take the
    lower expert index first, in slot order (logit descending)."""
    _say(f"[gpu] dense router top-k with exact ties E={E} k={k} renorm={renorm} T={T}")
    rng = np.random.default_rng(E * 100 + k)
    d = 256
    distinct = max(2, E // 4)
    base = rng.standard_normal((d, distinct)).astype(np.float32) * 0.05
    wr = np.ascontiguousarray(base[:, rng.permutation(np.arange(E) % distinct)])
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr_t = torch.empty((E, d), dtype=torch.bfloat16, device=dev)
    B.pack_transpose(torch.from_numpy(wr).to(dev).to(torch.bfloat16), wr_t)
    R = B.RouterDesc()
    R.kind, R.E, R.wr_t = B.ROUTER_DENSE, E, wr_t.data_ptr()
    xb = torch.from_numpy(x).to(dev).to(torch.bfloat16)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    r = torch.empty(T, dtype=torch.float32, device=dev)
    ws = torch.empty(max(B.router_workspace_size(R, T), 1), dtype=torch.uint8, device=dev)
    B.router_topk(R, xb, k, renorm, ids, w, r_out=r, logits=logits, ws=ws)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    assert max(len(np.unique(lg[t])) for t in range(T)) <= distinct
    sel = O.select_topk(lg, k)
    assert np.array_equal(ids.cpu().numpy(), sel)
    assert rel_err(w.cpu().numpy(), O.gates(lg.astype(np.float64), sel, renorm)) < 1e-5


def _dense_router(dev, E, d, dtype, seed):
    rng = np.random.default_rng(seed)
    wr = (rng.standard_normal((d, E)) * 0.05).astype(np.float32)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    wr_t = torch.empty((E, d), dtype=tdt, device=dev)
    B.pack_transpose(torch.from_numpy(wr).to(dev).to(tdt), wr_t)
    R = B.RouterDesc()
    R.kind, R.E, R.wr_t = B.ROUTER_DENSE, E, wr_t.data_ptr()
    return R, wr_t, rng, tdt


@pytest.mark.parametrize("dtype,E,k,renorm,noisy", [
    ("bf16", 8, 2, 1, False), ("bf16", 8, 2, 1, True), ("bf16", 64, 6, 0, True),
    ("bf16", 160, 40, 1, True), ("f32", 24, 3, 1, True), ("f32", 24, 3, 0, False)])
def test_router_stats_and_noise(dev, dtype, E, k, renorm, noisy):
    """Noise top-k and the routing statistics against the oracle on the GPU's
    own (noisy) logits; the statistics are bit-identical run to run."""
    _say(f"[gpu] router statistics dtype={dtype} E={E} k={k} renorm={renorm} noise={noisy}")
    T, d = 1000, 256
    R, keep, rng, tdt = _dense_router(dev, E, d, dtype, 5000 + E + k)
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(dev).to(tdt)
    noise = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).to(dev) if noisy else None
    std = 0.7 if noisy else 0.0
    ws = torch.empty(max(B.router_workspace_size(R, T), 1), dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)

    def run(with_noise):
        logits = torch.empty((T, E), **f32)
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), **f32)
        r = torch.empty(T, **f32)
        ps, gs, aux = torch.empty(E, **f32), torch.empty(E, **f32), torch.empty(3, **f32)
        ex = B.router_extras(noise=noise if with_noise else None, noise_std=std, prob_sum=ps,
                             gate_sum=gs, aux=aux)
        B.router_topk(R, x, k, renorm, ids, w, r_out=r, logits=logits, ws=ws, extras=ex)
        torch.cuda.synchronize()
        return [t.cpu().numpy() for t in (logits, ids, w, ps, gs, aux)]

    lg, ids, w, ps, gs, aux = run(noisy)
    if noisy:
        clean = run(False)[0]
        assert rel_err(lg, clean.astype(np.float64) + std * noise.cpu().numpy()) < 1e-6
    assert np.array_equal(ids, O.select_topk(lg, k))
    assert rel_err(w, O.gates(lg.astype(np.float64), ids, renorm)) < 1e-5
    st = O.router_stats(lg.astype(np.float64), ids, w, np.bincount(ids.ravel(), minlength=E))
    assert rel_err(ps, st["prob_sum"]) < 1e-5
    assert rel_err(gs, st["gate_sum"]) < 1e-5
    assert np.allclose(aux, st["aux"], rtol=1e-4, atol=1e-6), (aux, st["aux"])
    again = run(noisy)
    for a, b in zip((ps, gs, aux), again[3:]):
        assert np.array_equal(a, b)


def test_router_extras_rejected(dev):
    _say("[gpu] router extras: unsupported requests")
    T, d, E = 64, 256, 8
    R, keep, rng, tdt = _dense_router(dev, E, d, "bf16", 1)
    x = torch.zeros((T, d), dtype=tdt, device=dev)
    ids = torch.empty((T, E), dtype=torch.int32, device=dev)
    w = torch.empty((T, E), dtype=torch.float32, device=dev)
    r = torch.empty(T, dtype=torch.float32, device=dev)
    aux = torch.empty(3, dtype=torch.float32, device=dev)
    ws = torch.empty(max(B.router_workspace_size(R, T), 1), dtype=torch.uint8, device=dev)
    ex = B.router_extras(aux=aux, noise_std=float("nan"))
    with pytest.raises(B.MoeError):
        B.router_topk(R, x, 2, 1, ids, w, r_out=r, ws=ws, extras=ex)


def test_layer_router_extras(dev):
    """The layer forward with noise and statistics: its routing equals the
    router's own on the same noisy logits, and the statistics match it."""
    _say("[gpu] layer forward with router noise and statistics")
    wl, inp, params, layer = _setup("mixtral_small", dev)
    x = params["x"]
    T, E = wl.T, wl.E
    g = torch.Generator(device=dev).manual_seed(3)
    noise = torch.randn((T, E), generator=g, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    ps, gs, aux = torch.empty(E, **f32), torch.empty(E, **f32), torch.empty(3, **f32)
    ex = B.router_extras(noise=noise, noise_std=0.5, prob_sum=ps, gate_sum=gs, aux=aux)
    ws = layer.alloc_workspace(T)
    layer.forward(x, ws=ws, router_extras=ex)
    torch.cuda.synchronize()
    rt = layer.routing(T, ws)
    ids, w = rt["ids"].cpu().numpy(), rt["w"].cpu().numpy()
    # the router alone, same noise, with its logits
    logits = torch.empty((T, E), **f32)
    ids2 = torch.empty_like(rt["ids"])
    w2 = torch.empty_like(rt["w"])
    rws = torch.empty(max(B.router_workspace_size(layer.desc.router, T), 1), dtype=torch.uint8,
                      device=dev)
    B.router_topk(layer.desc.router, x, wl.k, wl.renorm, ids2, w2, r_in=rt["r"], logits=logits,
                  ws=rws, extras=B.router_extras(noise=noise, noise_std=0.5))
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    assert np.array_equal(ids2.cpu().numpy(), ids)
    assert np.array_equal(ids, O.select_topk(lg, wl.k))
    st = O.router_stats(lg.astype(np.float64), ids, w, np.bincount(ids.ravel(), minlength=E))
    assert rel_err(ps.cpu().numpy(), st["prob_sum"]) < 1e-5
    assert rel_err(gs.cpu().numpy(), st["gate_sum"]) < 1e-5
    assert np.allclose(aux.cpu().numpy(), st["aux"], rtol=1e-4, atol=1e-6)


def test_atomic_schedules_agree(dev):
    """Atomic experts through moe_expert_gemm: the expert-centric two-phase
    schedule (on the dispatch's task list) and the token-centric single pass
    (ids, w, r only) give the same bits, and match the oracle."""
    _say("[gpu] atomic experts: expert-centric == token-centric")
    wl, inp, params, layer = _setup("atomic_small", dev)
    ws = layer.alloc_workspace(wl.T)
    layer.forward(params["x"], ws=ws)
    torch.cuda.synchronize()
    rt = layer.routing(wl.T, ws)
    E = wl.Nr * wl.Nc
    full = _standalone_dispatch(rt, E, wl.T, 1, dev)
    full.update(ids=rt["ids"], w=rt["w"], r=rt["r"])
    X = layer.desc.experts
    R = B.rows_max(wl.T, wl.k, E, wl.T, 1)
    nws = B.expert_workspace_size(X, B.MOE_BF16, wl.d, wl.T, wl.k, R)
    ews = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    x = params["x"]
    y_ec = torch.empty_like(x)
    y_tc = torch.empty_like(x)
    B.expert_gemm(X, B.MOE_BF16, wl.d, B.make_routing(wl.T, wl.k, E, R, 1, full), x, y_ec, ews)
    tok = dict(ids=rt["ids"], w=rt["w"], r=rt["r"])
    B.expert_gemm(X, B.MOE_BF16, wl.d, B.make_routing(wl.T, wl.k, E, R, 1, tok), x, y_tc, ews)
    torch.cuda.synchronize()
    assert torch.equal(y_ec.view(torch.int16), y_tc.view(torch.int16))
    ids = rt["ids"].cpu().numpy()
    ref = O.atomic_experts_token_centric(O.as_f64(inp["x"]), rt["r"].cpu().numpy().astype(np.float64),
                                         ids, rt["w"].cpu().numpy().astype(np.float64),
                                         O.as_f64(inp["W"]), O.as_f64(inp["V"]))
    assert rel_err(f64(synth.to_host(y_tc)), ref) < TOL["bf16"]


def test_atomic_counts_bad_ids(dev):
    """Atomic expert ids outside [0, N) given to moe_expert_gemm are dropped
    (no row read) and counted in stats.errors, in both schedules; the result
    equals the same routing with those slots removed."""
    _say("[gpu] atomic experts with out-of-range ids")
    wl, inp, params, layer = _setup("atomic_small", dev)
    ws = layer.alloc_workspace(wl.T)
    layer.forward(params["x"], ws=ws)
    torch.cuda.synchronize()
    rt = layer.routing(wl.T, ws)
    E = wl.Nr * wl.Nc
    ids = rt["ids"].cpu().numpy().copy()
    bad = [(3, 1, E), (7, 0, -2), (11, wl.k - 1, 2 ** 31 - 1), (12, 4, E + 12345)]
    for t, j, v in bad:
        ids[t, j] = v
    ids_d = torch.from_numpy(ids).to(dev)
    w = rt["w"].clone()
    X = layer.desc.experts
    R = B.rows_max(wl.T, wl.k, E, wl.T, 1)
    ews = torch.empty(max(B.expert_workspace_size(X, B.MOE_BF16, wl.d, wl.T, wl.k, R), 1),
                      dtype=torch.uint8, device=dev)
    x = params["x"]
    # token-centric: ids, w, r only
    st_tc = torch.zeros(4, dtype=torch.int32, device=dev)
    y_tc = torch.empty_like(x)
    tok = dict(ids=ids_d, w=w, r=rt["r"])
    B.expert_gemm(X, B.MOE_BF16, wl.d, B.make_routing(wl.T, wl.k, E, R, 1, tok), x, y_tc, ews,
                  stats=st_tc)
    # expert-centric: the dispatch drops (and counts) the bad ids itself
    full = _standalone_dispatch(dict(rt, ids=ids_d, w=w), E, wl.T, 1, dev)
    full.update(ids=ids_d, w=w, r=rt["r"])
    st_ec = torch.zeros(4, dtype=torch.int32, device=dev)
    y_ec = torch.empty_like(x)
    B.expert_gemm(X, B.MOE_BF16, wl.d, B.make_routing(wl.T, wl.k, E, R, 1, full), x, y_ec, ews,
                  stats=st_ec)
    # the same routing with the bad slots' gates set to zero (ids in range)
    ids_ok = ids.copy()
    w_ok = w.cpu().numpy().copy()
    for t, j, _ in bad:
        ids_ok[t, j] = 0
        w_ok[t, j] = 0.0
    y_ok = torch.empty_like(x)
    ok = dict(ids=torch.from_numpy(ids_ok).to(dev), w=torch.from_numpy(w_ok).to(dev), r=rt["r"])
    B.expert_gemm(X, B.MOE_BF16, wl.d, B.make_routing(wl.T, wl.k, E, R, 1, ok), x, y_ok, ews)
    torch.cuda.synchronize()
    assert int(st_tc.cpu()[3]) == len(bad)
    assert int(st_ec.cpu()[3]) == 0 and int(full["stats"].cpu()[3]) == len(bad)
    assert torch.equal(y_tc.view(torch.int16), y_ec.view(torch.int16))
    assert torch.equal(y_tc.view(torch.int16), y_ok.view(torch.int16))
    ref = O.atomic_experts_token_centric(O.as_f64(inp["x"]), rt["r"].cpu().numpy().astype(np.float64),
                                         ids_ok, w_ok.astype(np.float64), O.as_f64(inp["W"]),
                                         O.as_f64(inp["V"]))
    assert rel_err(f64(synth.to_host(y_tc)), ref) < TOL["bf16"]


def _mx_pack_input():
    """bf16 rows that exercise the MXFP8 conversion: random magnitudes over
    a wide exponent range, and rows of special blocks (all zero, -0, the
    E8M0 clamp at -127, saturation above 448, round-half-even ties in the
    normal and the subnormal range)."""
    rng = np.random.default_rng(21)
    R, K = 67, 1120                                  # ragged: K = 2 x 512 + 96, R % 4 = 3
    v = rng.standard_normal((R, K)).astype(np.float32)
    v *= np.exp2(rng.integers(-30, 30, size=(R, K // 32, 1))).repeat(32, axis=2).reshape(R, K)
    v[0, :32] = 0.0
    v[0, 32:64] = -0.0
    v[0, 64:96] = np.float32(2.0 ** -125) * rng.standard_normal(32).astype(np.float32)  # clamp
    v[0, 96:128] = np.float32(2.0 ** -131)           # bf16 subnormals under the clamp
    # amax 256 (scale 2^0): ties 1 + 1/16 (-> 1), 1 + 3/16 (-> 1.25), 3 * 2^-10 (-> 2^-8),
    # 2^-10 (-> 0), 464 is not reachable (amax < 512 maps to < 512); 448 and 480 saturate
    v[1, :32] = 256.0
    v[1, 1:8] = [1.0625, 1.1875, 3 * 2.0 ** -10, 2.0 ** -10, -1.0625, 5 * 2.0 ** -10, 2.0 ** -6]
    v[1, 32:64] = 480.0                              # scale 2^0, elements at 480 -> 448
    v[1, 40] = 500.0
    v[1, 64:96] = np.float32(2.0 ** 120)             # large exponents
    v[1, 96:128] = -np.float32(2.0 ** -100)
    # every midpoint between neighbouring E4M3 codes and the bf16 values just
    # below and above it, both signs, in blocks whose largest element 256 sets
    # the scale (rows 2-4: block exponents 0, -20 and +10); all exactly bf16
    tests = _e4m3_midpoint_values()
    per = 31
    for row, t in ((2, 0), (3, -20), (4, 10)):
        for b in range(0, len(tests), per):
            blk = b // per
            chunk = tests[b:b + per]
            v[row, 32 * blk] = 256.0 * 2.0 ** t
            v[row, 32 * blk + 1:32 * blk + 1 + len(chunk)] = chunk * 2.0 ** t
            v[row, 32 * blk + 1 + len(chunk):32 * (blk + 1)] = 0.0
    return synth._to_bf16_bits(v)


def _e4m3_midpoint_values():
    """The midpoint between each pair of neighbouring positive E4M3 values
    (codes 0..126; normals have 3 mantissa bits, subnormals step 2^-9), the
    bf16 values one unit below and above it, and the negatives of all."""
    def value(c):
        e, m = (c >> 3) & 15, c & 7
        return m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
    out = []
    for c in range(126):
        mid = 0.5 * (value(c) + value(c + 1))
        ulp = 2.0 ** (np.floor(np.log2(mid)) - 7)     # bf16 unit at mid
        out += [mid, mid - ulp, mid + ulp]
    out = np.array(out, dtype=np.float64)
    return np.concatenate([out, -out]).astype(np.float32)


def test_pack_mxfp8_bit_exact(dev):
    """moe_pack_mxfp8 (the quantiser of the MXFP8 path) against the oracle's
    OCP MX conversion: codes and E8M0 scales bit-exact."""
    _say("[gpu] MXFP8 pack: codes and scales bit-exact")
    bits = _mx_pack_input()
    R, K = bits.shape
    src = synth.to_device(bits, dev)
    codes = torch.full((R, K), 0xAA, dtype=torch.uint8, device=dev)
    scales = torch.full((R, K // 32), 0xAA, dtype=torch.uint8, device=dev)
    B.pack_mxfp8(src, codes, scales)
    torch.cuda.synchronize()
    c_ref, s_ref = O.mx_quantize(O.as_f64(bits), axis=1)
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    bad = np.argwhere(c != c_ref)
    assert len(bad) == 0, (bad[:8], c[tuple(bad[0])], c_ref[tuple(bad[0])])
    assert np.array_equal(s, s_ref)
    # a strided source and destination (a column window of a wider matrix)
    c2 = torch.zeros((R, K + 64), dtype=torch.uint8, device=dev)
    s2 = torch.zeros((R, K // 32 + 4), dtype=torch.uint8, device=dev)
    wide = synth.to_device(np.hstack([bits, bits[:, :64]]), dev)
    B.pack_mxfp8(wide[:, :K], c2[:, :K], s2[:, :K // 32])
    torch.cuda.synchronize()
    assert np.array_equal(c2[:, :K].cpu().numpy(), c_ref)
    assert np.array_equal(s2[:, :K // 32].cpu().numpy(), s_ref)
    assert not c2[:, K:].any() and not s2[:, K // 32:].any()


@pytest.mark.parametrize("name", ["mixtral_small", "mixtral_small_mxfp8", "bcsr_small_mxfp8"])
def test_w2_row_stride(dev, name):
    """A padded row stride of w2_t (w2_ld) changes where the second linear
    reads its weights, not what it computes: the layer output is bit-identical
    with w2_t repacked at another stride (bf16: dense -> padded by 64
    elements; MXFP8, which the layer pads by 256 bytes: padded -> dense, and
    -> padded by 4 KB)."""
    _say(f"[gpu] w2_ld restride: {name}")
    wl, inp, params, layer = _setup(name, dev)
    x = params["x"]
    ref = layer.forward(x).clone()
    X = layer.desc.experts
    F = sum(wl.sizes)
    d = wl.d
    eb = 1 if wl.quant == "mxfp8" else 2
    ld0 = X.w2_ld or F
    old = [t for t in layer._keep if hasattr(t, "data_ptr") and t.data_ptr() == X.w2_t][0]
    cur = old.view(torch.uint8).view(d, ld0 * eb)[:, :F * eb]
    pads = [0, 4096] if wl.quant == "mxfp8" else [128]
    for pad in pads:
        w = torch.zeros((d, F * eb + pad), dtype=torch.uint8, device=dev)
        w[:, :F * eb] = cur
        X.w2_t, X.w2_ld = w.data_ptr(), (F * eb + pad) // eb if pad else 0
        out = layer.forward(x)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), pad
    X.w2_t, X.w2_ld = old.data_ptr(), (ld0 if ld0 != F else 0)


def test_pack_mxfp8_weights_layout(dev):
    """moe_pack_mxfp8_weights (the expert weights' quantiser): the oracle's
    OCP MX codes bit-exact, and its E8M0 scales bit-exact in the stage-major
    layout the expert GEMMs read: byte j % 4 of row r's word in K stage j // 4,
    at 4 ((j // 4) R + r) + j % 4."""
    _say("[gpu] MXFP8 weight pack: codes and stage-major scales bit-exact")
    bits = np.ascontiguousarray(_mx_pack_input()[:, :1024])      # R = 67, K = 8 stages
    R, K = bits.shape
    src = synth.to_device(bits, dev)
    codes = torch.full((R, K), 0xAA, dtype=torch.uint8, device=dev)
    scales = torch.full((K // 128, R, 4), 0xAA, dtype=torch.uint8, device=dev)
    B.pack_mxfp8_weights(src, codes, scales)
    torch.cuda.synchronize()
    c_ref, s_ref = O.mx_quantize(O.as_f64(bits), axis=1)          # scales [R, K / 32]
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    got = scales.cpu().numpy()
    for j in range(K // 32):
        assert np.array_equal(got[j // 4, :, j % 4], s_ref[:, j]), j


@pytest.mark.parametrize("d,T", [(384, 77), (256, 300), (1536, 40), (4096, 33)])
def test_dense_router_k_splits(dev, d, T):
    """bf16 router with each workgroup shape (the K range of d split over 4,
    8 or 16 waves, chosen by d): r, logits, ids and gates against the oracle
    on the same bf16 inputs, with a token count that leaves a partial block."""
    _say(f"[gpu] dense bf16 router d={d} T={T}")
    E, k = 24, 3
    R, keep, rng, tdt = _dense_router(dev, E, d, "bf16", 7000 + d)
    xb = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(dev).to(tdt)
    bias = torch.from_numpy(rng.standard_normal(E).astype(np.float32) * 0.1).to(dev)
    R.bias = bias.data_ptr()
    f32 = dict(dtype=torch.float32, device=dev)
    logits, w, r = torch.empty((T, E), **f32), torch.empty((T, k), **f32), torch.empty(T, **f32)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    ws = torch.empty(max(B.router_workspace_size(R, T), 1), dtype=torch.uint8, device=dev)
    B.router_topk(R, xb, k, 1, ids, w, r_out=r, logits=logits, ws=ws, eps=1e-6)
    torch.cuda.synchronize()
    x64 = xb.float().cpu().numpy().astype(np.float64)
    wr64 = keep.float().cpu().numpy().astype(np.float64).T          # [d, E]
    r_ref = O.rmsnorm_scale(x64, 1e-6)
    assert rel_err(r.cpu().numpy(), r_ref) < 1e-5
    lg = logits.cpu().numpy()
    ref = O.router_logits(x64, None, r_ref, wr64, bias.cpu().numpy())
    assert np.abs(lg - ref).max() < 1e-4 * np.abs(ref).max() + 1e-6
    got_ids = ids.cpu().numpy()
    assert np.array_equal(got_ids, O.select_topk(lg, k))
    assert rel_err(w.cpu().numpy(), O.gates(lg.astype(np.float64), got_ids, 1)) < 1e-5
