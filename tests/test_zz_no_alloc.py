"""moe_dispatch_noalloc: the dispatch on the library's static scratch (for
callers that cannot allocate) against moe_dispatch with a caller-supplied
workspace, through the C ABI.

Each case runs two calls of the allocation-free entry point in a row on one
stream, the second with a smaller input, so the second call finds the first
call's contents in the shared scratch; both must give exactly the outputs
of moe_dispatch on the same inputs (integer outputs, gathered rows and the
carried r / gate values bit for bit), and those equal the oracle's dispatch.
"""
import numpy as np
import pytest

import oracle as O

torch = pytest.importorskip("torch")

from sparse_mixture_experts_rmsnorm_amd import binding as B  # noqa: E402


def _case(T, k, E, d, seed):
    rng = np.random.default_rng(seed)
    if E <= 4096:
        # k distinct experts per token, skewed towards low ids so capacity bites
        score = rng.standard_normal((T, E)) - 0.15 * np.log1p(np.arange(E))[None, :]
        ids = np.argsort(-score, axis=1, kind="stable")[:, :k].astype(np.int32)
    else:
        # many experts: uniform ids, a few slots from a small range so that
        # experts are shared between tokens
        ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
        ids[:, :4] = rng.integers(0, 4096, size=(T, 4))
    w = rng.random((T, k)).astype(np.float32)
    r = (0.5 + rng.random(T)).astype(np.float32)
    x = rng.standard_normal((T, d)).astype(np.float32)
    return ids, w, r, x


def _outputs(T, k, E, R, d, dev):
    i32, f32 = dict(dtype=torch.int32, device=dev), dict(dtype=torch.float32, device=dev)
    return dict(counts=torch.full((E,), -7, **i32), offsets=torch.full((E + 1,), -7, **i32),
                pos=torch.full((T, k), -7, **i32), row_token=torch.full((R,), -7, **i32),
                row_r=torch.full((R,), -7.0, **f32), row_w=torch.full((R,), -7.0, **f32),
                row_expert=torch.full((R,), -7, **i32),
                x_perm=torch.full((R, d), -7.0, dtype=torch.bfloat16, device=dev),
                stats=torch.full((4,), -7, **i32))


def _run(fn_noalloc, ids, w, r, x, E, cap, pad, dev):
    T, k = ids.shape
    d = x.shape[1]
    R = B.rows_max(T, k, E, cap, pad)
    o = _outputs(T, k, E, R, d, dev)
    args = (torch.from_numpy(ids).to(dev), torch.from_numpy(w).to(dev),
            torch.from_numpy(r).to(dev), E, cap, pad, R)
    xd = torch.from_numpy(x).to(dev).to(torch.bfloat16)
    if fn_noalloc:
        B.dispatch_noalloc(*args, o, x=xd, x_perm=o["x_perm"], stats=o["stats"])
    else:
        ws = torch.empty(max(B.dispatch_workspace_size(T, k, E), 1), dtype=torch.uint8, device=dev)
        B.dispatch(*args, o, x=xd, x_perm=o["x_perm"], stats=o["stats"], ws=ws)
        o["_ws"] = ws
    o["_x"] = xd
    return o


# (T, k, E, capacity, pad, d): a first call, then a smaller second one
PAIRS = {
    "dense_capacity": ((4096, 2, 8, 1280, 1, 512), (700, 2, 8, 150, 1, 256)),
    "dense_bcsr_pad": ((3000, 6, 64, 3000, 128, 256), (129, 6, 64, 129, 128, 256)),
    "radix_2e20": ((2048, 32, 1 << 20, 2048, 1, 256), (300, 32, 1 << 20, 300, 1, 256)),
}


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(PAIRS))
def test_noalloc_dispatch_matches_dispatch(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"[gpu] moe_dispatch_noalloc {name}", flush=True)
    B.lib()
    dev = "cuda"
    cases = []
    for i, (T, k, E, cap, pad, d) in enumerate(PAIRS[name]):
        assert B.dispatch_workspace_size(T, k, E) <= B.NOALLOC_SCRATCH_BYTES
        cases.append((_case(T, k, E, d, 100 + i), E, cap, pad))
    # two allocation-free calls in a row on one stream, then the references
    got = [_run(True, *c[0], c[1], c[2], c[3], dev) for c in cases]
    ref = [_run(False, *c[0], c[1], c[2], c[3], dev) for c in cases]
    torch.cuda.synchronize()
    for (inp, E, cap, pad), g, rf in zip(cases, got, ref):
        ids = inp[0]
        disp = O.dispatch(ids, E, min(cap, ids.shape[0]), pad)
        for key in ("counts", "offsets", "pos", "row_token", "row_expert", "stats"):
            assert torch.equal(g[key], rf[key]), key
        for key in ("row_r", "row_w"):
            assert torch.equal(g[key].view(torch.int32), rf[key].view(torch.int32)), key
        assert torch.equal(g["x_perm"].view(torch.int16), rf["x_perm"].view(torch.int16))
        assert np.array_equal(g["counts"].cpu().numpy(), disp["counts"])
        assert np.array_equal(g["offsets"].cpu().numpy(), disp["offsets"])
        assert np.array_equal(g["pos"].cpu().numpy(), disp["pos"])
        rows = disp["rows"]
        assert np.array_equal(g["row_token"].cpu().numpy()[:rows], disp["row_token"])
        st = g["stats"].cpu().numpy()
        assert st[0] == rows and st[1] == disp["dropped"] and st[3] == 0
        # the gathered rows are the tokens' rows (zeros on padding rows)
        xp = g["x_perm"].cpu()
        tok = g["row_token"].cpu()
        live = tok[:rows] >= 0
        assert torch.equal(xp[:rows][live].view(torch.int16),
                           g["_x"].cpu()[tok[:rows][live].long()].view(torch.int16))


@pytest.mark.gpu
def test_noalloc_rejects_sizes_beyond_the_scratch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    dev = "cuda"
    T, k, E = 65536, 32, 1 << 20
    need = B.dispatch_workspace_size(T, k, E)
    assert need > B.NOALLOC_SCRATCH_BYTES
    o = _outputs(4, k, 8, 8, 256, dev)   # never written: the call is refused on the host
    ids = torch.zeros((4, k), dtype=torch.int32, device=dev)
    with pytest.raises(B.MoeError) as ei:
        B.lib()
        B.check(B.lib().moe_dispatch_noalloc(
            B.ptr(ids), B.ptr(o["row_w"]), B.ptr(o["row_r"]), None, B.MOE_BF16, T, 0, E, k, T, 1,
            T * k, B.ptr(o["counts"]), B.ptr(o["offsets"]), B.ptr(o["pos"]),
            B.ptr(o["row_token"]), B.ptr(o["row_r"]), B.ptr(o["row_w"]), None, None, None,
            B.stream_handle()))
    assert ei.value.code == -5          # MOE_EWORKSPACE
    assert str(need) in str(ei.value) and str(B.NOALLOC_SCRATCH_BYTES) in str(ei.value)
    torch.cuda.synchronize()
    assert torch.all(o["counts"] == -7)
