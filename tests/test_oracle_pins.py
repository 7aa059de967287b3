"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a worked
example printed on the pages (tests/golden/), a closed form, an identity, a
special case that reduces to a textbook computation, or brute force on tiny
inputs.  No GPU is needed.
"""
import itertools
import json
import math
from pathlib import Path

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax, ndtr

import oracle as O

GOLD = Path(__file__).parent / "golden"


def _rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- bf16 format

def test_bf16_rounding_known_values():
    vals = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.0,
                     1.0 + 2.0 ** -8 + 2.0 ** -20, 3.140625, 0.0, -0.0])
    bits = O.f64_to_bf16_bits(vals)
    # 1+2^-8 is halfway between 1 and 1+2^-7: ties to the even mantissa (1.0);
    # 1+3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even).
    assert [hex(int(b)) for b in bits] == ["0x3f80", "0x3f80", "0x3f82", "0xc000",
                                          "0x3f81", "0x4049", "0x0", "0x8000"]
    assert O.bf16_to_f64(np.array([0x3F80, 0x4049, 0xC000], np.uint16)).tolist() == [1.0, 3.140625, -2.0]


def test_bf16_roundtrip_exact():
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)  # finite positive patterns
    assert np.array_equal(O.f64_to_bf16_bits(O.bf16_to_f64(bits)), bits)


# ---------------------------------------------------------------- capacity

def test_capacity_table():
    for c in json.loads((GOLD / "capacity.json").read_text())["cases"]:
        assert O.capacity(c["T"], c["k"], c["E"], c["cf"]) == c["capacity"], c


def test_capacity_is_smallest_integer_bound():
    rng = _rng(1)
    for _ in range(300):
        T = int(rng.integers(0, 5000))
        k = int(rng.integers(1, 9))
        E = int(rng.integers(1, 100))
        a = int(rng.integers(1, 64))
        C = O.capacity(T, k, E, a / 16.0)               # cf = a/16 is exact in binary
        # smallest integer C with 16*E*C >= T*k*a, clamped to T
        c0 = -(-(T * k * a) // (16 * E))
        assert C == min(c0, T)
        assert 16 * E * C >= min(T * k * a, 16 * E * T)


# ---------------------------------------------------------------- RMSNorm / r-scale

def test_rmsnorm_closed_forms():
    x = np.array([[3.0, 4.0], [2.0, 2.0], [0.0, 0.0]])
    r = O.rmsnorm_scale(x, 0.0 + 1e-6)
    assert r[0] == pytest.approx(1.0 / math.sqrt(12.5 + 1e-6), rel=1e-15)
    assert r[1] == pytest.approx(1.0 / math.sqrt(4.0 + 1e-6), rel=1e-15)
    assert r[2] == pytest.approx(1.0 / math.sqrt(1e-6), rel=1e-15)
    # scale invariance (eps = 0) and unit RMS of the normalised output
    z = _rng(2).standard_normal((5, 33))
    assert np.allclose(O.rmsnorm_scale(7.5 * z, 0.0), O.rmsnorm_scale(z, 0.0) / 7.5, rtol=1e-14)
    y = O.rmsnorm(z, None, 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-14)
    g = _rng(3).standard_normal(33)
    assert np.allclose(O.rmsnorm(z, g, 0.0), y * g, rtol=1e-14)


def test_r_scale_epilogue_equals_unfused_rmsnorm():
    rng = _rng(4)
    x = rng.standard_normal((40, 64))
    gamma = 1 + 0.1 * rng.standard_normal(64)
    w = 0.02 * rng.standard_normal((64, 6))
    b = rng.standard_normal(6)
    r = O.rmsnorm_scale(x, 1e-6)
    fused = O.router_logits(x, gamma, r, w, b)
    unfused = O.router_logits_unfused(x, gamma, 1e-6, w, b)
    assert np.max(np.abs(fused - unfused)) <= 1e-12 * np.max(np.abs(unfused))


# ---------------------------------------------------------------- top-k and gates

def _brute_topk(l, k):
    """Best ordered k-tuple of distinct experts by the key sequence (l desc, e asc)."""
    best, best_key = None, None
    for perm in itertools.permutations(range(len(l)), k):
        key = [(l[e], -e) for e in perm]
        if best_key is None or key > best_key:
            best, best_key = perm, key
    return list(best)


def test_topk_bruteforce_with_ties():
    rng = _rng(5)
    for E in range(1, 7):
        for k in range(1, E + 1):
            l = rng.integers(-2, 3, size=(12, E)).astype(np.float64)  # many exact ties
            ids = O.select_topk(l, k)
            for t in range(l.shape[0]):
                assert ids[t].tolist() == _brute_topk(l[t].tolist(), k)


def test_topk_crafted_ties_go_to_lower_index():
    assert O.select_topk(np.array([[1.0, 3.0, 3.0, 2.0]]), 2).tolist() == [[1, 2]]
    assert O.select_topk(np.array([[5.0, 5.0, 5.0, 5.0]]), 3).tolist() == [[0, 1, 2]]
    assert O.select_topk(np.array([[0.0, -0.0, 1.0]]), 2).tolist() == [[2, 0]]
    assert O.select_topk(np.array([[-1.0, -3.0, -2.0]]), 1).tolist() == [[0]]


def test_gates_properties():
    rng = _rng(6)
    l = rng.standard_normal((30, 8)) * 3
    for k in (1, 2, 5, 8):
        ids = O.select_topk(l, k)
        g = O.gates(l, ids, renorm=1)
        assert np.allclose(g.sum(axis=1), 1.0, rtol=1e-14)
        assert np.all(np.diff(g, axis=1) <= 0)           # slot 0 is the best
        full = np.take_along_axis(sp_softmax(l, axis=1), ids.astype(np.int64), axis=1)
        assert np.allclose(O.gates(l, ids, renorm=0), full, rtol=1e-13)
    ids = O.select_topk(l, 8)
    assert np.allclose(O.gates(l, ids, 1), O.gates(l, ids, 0), rtol=1e-13)
    assert np.all(O.gates(l, O.select_topk(l, 1), 1) == 1.0)


# ---------------------------------------------------------------- dispatch

def _dispatch_brute(ids, E, cap, pad):
    T, k = ids.shape
    rank = np.zeros((T, k), int)
    for t in range(T):
        for j in range(k):
            rank[t, j] = sum(1 for t2 in range(t) for j2 in range(k) if ids[t2, j2] == ids[t, j])
    counts = [int((ids == e).sum()) for e in range(E)]
    kept = [min(c, cap) for c in counts]
    offs = [0]
    for e in range(E):
        offs.append(offs[-1] + -(-kept[e] // pad) * pad)
    pos = np.where(rank < cap, np.array(offs)[ids] + rank, -1)
    return counts, kept, offs, rank, pos


@pytest.mark.parametrize("cap,pad", [(1, 1), (3, 1), (100, 1), (2, 4), (100, 8)])
def test_dispatch_bruteforce(cap, pad):
    rng = _rng(7 + cap + pad)
    T, E, k = 40, 5, 2
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    d = O.dispatch(ids, E, cap, pad)
    counts, kept, offs, rank, pos = _dispatch_brute(ids, E, cap, pad)
    assert d["counts"].tolist() == counts and sum(counts) == T * k
    assert d["kept"].tolist() == kept
    assert d["offsets"].tolist() == offs
    assert np.array_equal(d["rank"], rank)
    assert np.array_equal(d["pos"], pos)
    assert set(zip(*np.nonzero(d["pos"] < 0))) == set(zip(*np.nonzero(rank >= cap)))
    p = d["pos"][d["pos"] >= 0]
    assert len(set(p.tolist())) == len(p)                          # injective
    for e in range(E):
        rows = d["row_token"][offs[e]:offs[e] + kept[e]]
        assert np.all(np.diff(rows) > 0)                          # token order
        assert np.all(d["row_token"][offs[e] + kept[e]:offs[e + 1]] == -1)   # padding
        assert all(e in ids[t] for t in rows)                     # rows chose e
    assert d["dropped"] == int((rank >= cap).sum())


# ---------------------------------------------------------------- variable sizes / BCSR

def test_expert_layout_worked_example():
    g = json.loads((GOLD / "variable_experts_layout.json").read_text())
    lay = O.expert_layout([tuple(s) for s in g["expert_sizes_spec"]], g["num_experts"], g["block_size"])
    assert lay["sizes"] == g["expert_sizes"]
    assert lay["offsets"] == g["expert_offsets"]
    assert lay["total"] == g["total_expert_width"]
    assert [g["n_embd"], lay["total"]] == g["w1_shape"]
    assert lay["offsets"][0:2] == g["w1_columns_expert0"]
    assert lay["offsets"][1:3] == g["w1_columns_expert1"]
    assert lay["size_blocks"][:3] == g["expert_size_blocks_prefix"]
    assert lay["block_offsets"][:3] == g["expert_block_offsets_prefix"]
    with pytest.raises(ValueError):
        O.expert_layout([(1, 2048), (6, 1024)], 8)
    # sizes are rounded up to the block
    assert O.expert_layout([(2, 100), (1, 129)], 3, 128)["sizes"] == [128, 128, 256]


def test_topology_worked_example():
    g = json.loads((GOLD / "variable_experts_layout.json").read_text())
    lay = O.expert_layout([tuple(s) for s in g["expert_sizes_spec"]], 8, 128)
    tb = [2, 1, 0, 3, 1, 1, 1, 2]                      # token blocks per expert
    offsets = [0]
    for n in tb:
        offsets.append(offsets[-1] + 128 * n)
    topo = O.bcsr_topology(offsets, lay["size_blocks"], lay["block_offsets"], 128)
    assert topo["block_rows"] == sum(tb)
    assert topo["nnz"] == sum(n * s for n, s in zip(tb, lay["size_blocks"]))
    # first row block belongs to the 2048-wide expert: 16 column blocks 0..15
    ro, ci = topo["row_offsets"], topo["column_indices"]
    assert ci[ro[0]:ro[1]].tolist() == list(range(16))
    assert ci[ro[1]:ro[2]].tolist() == list(range(16))
    assert ci[ro[2]:ro[3]].tolist() == list(range(16, 24))       # expert 1
    assert ci[ro[3]:ro[4]].tolist() == list(range(32, 40))       # expert 3 (expert 2 empty)
    assert np.all(np.diff(ro) == np.repeat(lay["size_blocks"], tb))


def test_topology_output_offsets_regression():
    g = json.loads((GOLD / "output_offsets_regression.json").read_text())
    sizes = g["expert_sizes"]
    B = g["block_size"]
    lay = O.expert_layout([(1, s) for s in sizes], len(sizes), B)
    small = [g["token_blocks_small_total"] // 31] * 31
    small[-1] += g["token_blocks_small_total"] - sum(small)
    tb = small + [g["token_blocks_large"]]
    offsets = [0]
    for n in tb:
        offsets.append(offsets[-1] + B * n)
    topo = O.bcsr_topology(offsets, lay["size_blocks"], lay["block_offsets"], B)
    large = len(sizes) - 1
    assert topo["output_offsets"][large] == g["expected_large_output_offset"]
    assert topo["output_offsets"][large] != g["buggy_large_output_offset"]
    assert topo["nnz"] == g["token_blocks_small_total"] + 4 * g["token_blocks_large"]
    first = topo["row_offsets"][sum(small)]
    assert topo["column_indices"][first:first + 4].tolist() == [31, 32, 33, 34]


@pytest.mark.parametrize("act,sizes", [("gelu", [256, 128, 384]), ("swiglu", [128, 256, 128]),
                                       ("gelu", [256, 256, 256])])
def test_bcsr_walk_equals_per_expert_dense(act, sizes):
    rng = _rng(8)
    T, d, E, k, B = 70, 64, 3, 2, 128
    x = rng.standard_normal((T, d))
    F = sum(sizes)
    w1 = 0.05 * rng.standard_normal((d, F))
    w3 = 0.05 * rng.standard_normal((d, F)) if act == "swiglu" else None
    w2 = 0.05 * rng.standard_normal((F, d))
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    disp = O.dispatch(ids, E, T, B)
    lay = O.expert_layout([(1, s) for s in sizes], E, B)
    topo = O.bcsr_topology(disp["offsets"], lay["size_blocks"], lay["block_offsets"], B)
    r = O.rmsnorm_scale(x, 1e-6)
    rt = disp["row_token"]
    x_perm = np.where(rt[:, None] >= 0, x[np.maximum(rt, 0)], 0.0)
    r_perm = np.where(rt >= 0, r[np.maximum(rt, 0)], 0.0)
    y_bcsr = O.bcsr_expert_ffn(x_perm, r_perm, topo, w1, w2, act, B, w3)
    valid = rt >= 0
    e_of_row = np.searchsorted(disp["offsets"], np.nonzero(valid)[0], side="right") - 1
    y_dense = O.grouped_expert_ffn(x_perm[valid], r_perm[valid], e_of_row, w1, w2,
                                   lay["offsets"], act, w3)
    assert np.allclose(y_bcsr[valid], y_dense, rtol=1e-12, atol=1e-14)
    assert np.all(y_bcsr[~valid] == 0)


# ---------------------------------------------------------------- activations

def test_activation_values():
    assert O.gelu(0.0) == 0.0
    assert float(O.gelu(1.0)) == pytest.approx(float(ndtr(1.0)), rel=1e-15)
    assert float(O.gelu(1.0)) == pytest.approx(0.8413447460685429, rel=1e-15)
    assert float(O.gelu(-1.0)) == pytest.approx(-0.15865525393145707, rel=1e-14)
    assert float(O.gelu(40.0)) == 40.0 and float(O.gelu(-40.0)) == pytest.approx(0.0, abs=1e-300)
    assert float(O.silu(1.0)) == pytest.approx(0.7310585786300049, rel=1e-15)
    assert float(O.silu(0.0)) == 0.0
    assert float(O.gelu_tanh(1.0)) == pytest.approx(0.8411919906082768, rel=1e-12)


# ---------------------------------------------------------------- whole-layer special cases

def _layer(rng, T, d, E, k, f, act, cf=0.0, renorm=1, gamma=False, bias=False):
    p = dict(k=k, eps=1e-6, renorm=renorm, cf=cf, act=act, residual=True,
             w_router=0.3 * rng.standard_normal((d, E)),
             bias=rng.standard_normal(E) if bias else None,
             gamma=(1 + 0.1 * rng.standard_normal(d)) if gamma else None,
             w1=0.05 * rng.standard_normal((d, E * f)),
             w2=0.05 * rng.standard_normal((E * f, d)),
             f_offsets=[e * f for e in range(E + 1)])
    if act == "swiglu":
        p["w3"] = 0.05 * rng.standard_normal((d, E * f))
    return p


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_k_equals_E_is_dense_softmax_mixture(act):
    rng = _rng(9)
    T, d, E, f = 25, 32, 4, 48
    p = _layer(rng, T, d, E, E, f, act, gamma=True, bias=True)
    x = rng.standard_normal((T, d))
    res = O.layer_forward(p, x)
    xn = O.rmsnorm(x, p["gamma"], 1e-6)
    prob = sp_softmax(xn @ p["w_router"] + p["bias"], axis=1)
    dense = x.copy()
    for e in range(E):
        sl = slice(e * f, (e + 1) * f)
        a = xn @ p["w1"][:, sl]
        h = (a / (1 + np.exp(-a))) * (xn @ p["w3"][:, sl]) if act == "swiglu" else a * ndtr(a)
        dense += prob[:, e:e + 1] * (h @ p["w2"][sl, :])
    assert np.max(np.abs(res["out"] - dense)) <= 1e-12 * np.max(np.abs(dense))


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_single_expert_is_dense_ffn(act):
    rng = _rng(10)
    T, d, f = 30, 48, 64
    p = _layer(rng, T, d, 1, 1, f, act)
    x = rng.standard_normal((T, d))
    res = O.layer_forward(p, x)
    assert np.all(res["w"] == 1.0)
    xn = O.rmsnorm(x, None, 1e-6)
    a = xn @ p["w1"]
    h = (a / (1 + np.exp(-a))) * (xn @ p["w3"]) if act == "swiglu" else a * ndtr(a)
    ref = x + h @ p["w2"]
    assert np.max(np.abs(res["out"] - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_fully_dropped_tokens_pass_through_bit_exactly():
    rng = _rng(11)
    T, d, E, k = 64, 32, 4, 2
    p = _layer(rng, T, d, E, k, 32, "gelu", cf=0.25)       # capacity 8 per expert
    xb = O.f64_to_bf16_bits(rng.standard_normal((T, d)))
    for faithful in (False, True):
        res = O.layer_forward(p, xb, faithful=faithful)
        assert res["capacity"] == 8
        gone = np.all(res["pos"] < 0, axis=1)
        assert gone.sum() > 0
        assert np.array_equal(res["out"][gone], O.bf16_to_f64(xb[gone]))
        kept_any = ~gone
        assert not np.array_equal(res["out"][kept_any], O.bf16_to_f64(xb[kept_any]))


def test_shared_experts_concatenate():
    rng = _rng(12)
    T, d, f = 20, 32, 40
    x = rng.standard_normal((T, d))
    r = O.rmsnorm_scale(x, 1e-6)
    a1, a3, a2 = (0.05 * rng.standard_normal(s) for s in [(d, f), (d, f), (f, d)])
    b1, b3, b2 = (0.05 * rng.standard_normal(s) for s in [(d, f), (d, f), (f, d)])
    two = O.ffn(x, r, a1, a2, "swiglu", a3) + O.ffn(x, r, b1, b2, "swiglu", b3)
    one = O.ffn(x, r, np.hstack([a1, b1]), np.vstack([a2, b2]), "swiglu", np.hstack([a3, b3]))
    assert np.allclose(two, one, rtol=1e-12, atol=1e-15)


def test_uniform_sizes_through_variable_spec_match_uniform():
    a = O.expert_layout([(8, 1024)], 8, 128)
    b = O.expert_layout(None, 8, 128, default_size=1024)
    assert a == b


# ---------------------------------------------------------------- Cartesian router / atomic experts

@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_cartesian_two_stage_equals_bruteforce(dtype):
    rng = _rng(13)
    T, Nr, Nc, k = 24, 32, 32, 8
    s1 = rng.standard_normal((T, Nr)).astype(dtype)
    s2 = rng.standard_normal((T, Nc)).astype(dtype)
    a, sa = O.cartesian_topk(s1, s2, k)
    b, sb = O.cartesian_topk_bruteforce(s1, s2, k)
    assert np.array_equal(a, b) and np.array_equal(sa, sb)
    # integer scores: many exact ties, ties go to the lower flat index
    s1 = rng.integers(-2, 3, (T, 6)).astype(dtype)
    s2 = rng.integers(-2, 3, (T, 5)).astype(dtype)
    for kk in (1, 4, 9):
        assert np.array_equal(O.cartesian_topk(s1, s2, kk)[0], O.cartesian_topk_bruteforce(s1, s2, kk)[0])


def test_cartesian_scores_are_row_plus_column():
    rng = _rng(14)
    T, d, Nr, Nc = 5, 16, 4, 3
    x = rng.standard_normal((T, d))
    Kr, Kc = rng.standard_normal((d, Nr)), rng.standard_normal((d, Nc))
    r = O.rmsnorm_scale(x, 1e-6)
    s1, s2 = O.cartesian_scores(x, None, r, Kr, Kc)
    xn = O.rmsnorm(x, None, 1e-6)
    for i in range(Nr):
        for j in range(Nc):
            # score of expert n = i*Nc + j, against a dense router with the concatenated key
            assert np.allclose(s1[:, i] + s2[:, j], xn @ (Kr[:, i] + Kc[:, j]), rtol=1e-12)


def test_atomic_all_experts_is_dense_gelu_ffn():
    rng = _rng(15)
    T, d, Nr, Nc = 10, 24, 4, 4
    N = Nr * Nc
    x = rng.standard_normal((T, d))
    W, V = 0.3 * rng.standard_normal((N, d)), 0.3 * rng.standard_normal((N, d))
    r = O.rmsnorm_scale(x, 1e-6)
    ids = np.tile(np.arange(N), (T, 1))
    g = sp_softmax(rng.standard_normal((T, N)), axis=1)
    routed = O.atomic_experts_token_centric(x, r, ids, g, W, V)
    xn = O.rmsnorm(x, None, 1e-6)
    a = xn @ W.T
    dense = (g * a * ndtr(a)) @ V
    assert np.allclose(routed, dense, rtol=1e-12, atol=1e-14)


def test_atomic_expert_centric_equals_token_centric():
    rng = _rng(16)
    T, d, N, k = 30, 16, 20, 5
    x = rng.standard_normal((T, d))
    W, V = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    r = O.rmsnorm_scale(x, 1e-6)
    ids = np.stack([rng.choice(N, size=k, replace=False) for _ in range(T)])
    g = sp_softmax(rng.standard_normal((T, k)), axis=1)
    a = O.atomic_experts_token_centric(x, r, ids, g, W, V)
    b = O.atomic_experts_expert_centric(x, r, ids, g, W, V)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13)


def test_cartesian_layer_matches_bruteforce_routing():
    rng = _rng(17)
    T, d, Nr, Nc, k = 12, 32, 8, 8, 6
    p = dict(router="cartesian", k=k, eps=1e-6, act="gelu", residual=True,
             k_rows=rng.standard_normal((d, Nr)), k_cols=rng.standard_normal((d, Nc)),
             W=0.2 * rng.standard_normal((Nr * Nc, d)), V=0.2 * rng.standard_normal((Nr * Nc, d)),
             ws1=0.05 * rng.standard_normal((d, 40)), ws2=0.05 * rng.standard_normal((40, d)),
             shared_act="gelu")
    x = rng.standard_normal((T, d))
    res = O.layer_forward(p, x)
    xn = O.rmsnorm(x, None, 1e-6)
    full = np.stack([(xn @ p["k_rows"])[:, i:i + 1] + xn @ p["k_cols"] for i in range(Nr)], axis=1)
    full = full.reshape(T, Nr * Nc)
    for t in range(T):
        # definition: the k best flat ids by (score desc, id asc), by a plain sort
        assert res["ids"][t].tolist() == sorted(range(Nr * Nc), key=lambda n: (-full[t, n], n))[:k]
    gg = sp_softmax(np.take_along_axis(full, res["ids"], axis=1), axis=1)
    assert np.allclose(res["w"], gg, rtol=1e-12)
    a = xn @ p["ws1"]
    shared = (a * ndtr(a)) @ p["ws2"]
    routed = np.stack([sum(gg[t, j] * O.gelu(xn[t] @ p["W"][n]) * p["V"][n]
                           for j, n in enumerate(res["ids"][t])) for t in range(T)])
    assert np.allclose(res["out"], x + shared + routed, rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------- routing statistics / noisy top-k

def test_squared_cv_closed_forms():
    assert O.squared_cv(np.full(8, 3.0)) == 0.0
    # all mass on one of E experts: CV^2 = E - 1
    for E in (2, 8, 64):
        v = np.zeros(E)
        v[3 % E] = 5.0
        assert abs(O.squared_cv(v) - (E - 1)) < 1e-12
    # two levels a, b over halves: CV^2 = ((a - b) / (a + b))^2
    a, b = 3.0, 1.0
    assert abs(O.squared_cv(np.array([a] * 4 + [b] * 4)) - ((a - b) / (a + b)) ** 2) < 1e-15
    assert np.isnan(O.squared_cv(np.zeros(4)))


def test_router_stats_uniform_and_collapsed():
    T, E, k = 50, 8, 2
    # equal logits: every expert gets T / E probability mass, CV^2 = 0
    st = O.router_stats(np.zeros((T, E)), np.tile(np.arange(k), (T, 1)), np.full((T, k), 0.5))
    assert np.allclose(st["prob_sum"], T / E, rtol=0, atol=1e-12)
    assert abs(st["aux"][0]) < 1e-24
    # one expert dominates every token: the mass is all on it, CV^2 = E - 1
    l = np.full((T, E), -800.0)
    l[:, 5] = 0.0
    st = O.router_stats(l, np.tile([5, 0], (T, 1)), np.tile([1.0, 0.0], (T, 1)))
    assert abs(st["prob_sum"][5] - T) < 1e-9 and abs(st["aux"][0] - (E - 1)) < 1e-9
    assert st["gate_sum"][5] == T and abs(st["aux"][1] - (E - 1)) < 1e-12
    assert np.isnan(st["aux"][2])


def test_router_stats_sums_and_scatter():
    rng = np.random.default_rng(11)
    T, E, k = 40, 16, 3
    l = rng.standard_normal((T, E))
    ids = O.select_topk(l, k)
    w = O.gates(l, ids, 1)
    counts = np.bincount(ids.ravel(), minlength=E)
    st = O.router_stats(l, ids, w, counts)
    # every token's probabilities and renormalised gates sum to one
    assert abs(st["prob_sum"].sum() - T) < 1e-9
    assert abs(st["gate_sum"].sum() - T) < 1e-9
    # the gate sum scatters each slot's weight to its expert (checked by expert)
    for e in range(E):
        assert abs(st["gate_sum"][e] - w[ids == e].sum()) < 1e-12
    # full-softmax mass of expert e equals the column sum of exp(l - m) / z
    p = np.exp(l - l.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    assert np.allclose(st["prob_sum"], p.sum(0), rtol=1e-13)
    assert abs(st["aux"][2] - counts.var() / counts.mean() ** 2) < 1e-12


def test_noisy_logits_flip_selection():
    l = np.array([[1.0, 0.5, -1.0]])
    n = np.array([[0.0, 1.0, 0.0]])
    assert O.select_topk(O.noisy_logits(l, n, 0.0), 1)[0, 0] == 0
    assert O.select_topk(O.noisy_logits(l, n, 1.0), 1)[0, 0] == 1       # 0.5 + 1 > 1
    assert O.select_topk(O.noisy_logits(l, n, 0.4), 1)[0, 0] == 0       # 0.9 < 1
    assert np.array_equal(O.noisy_logits(l, n, 2.5), l + 2.5 * n)


# ---------------------------------------------------------------- MXFP8 (OCP MX v1.0, E4M3 elements)

def test_e4m3_code_table():
    codes = np.arange(256, dtype=np.uint8)
    v = O.e4m3_decode(codes)
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.sum(np.isnan(v)) == 2
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0          # largest finite
    assert v[0x38] == 1.0 and v[0x08] == 2.0 ** -6          # 1.0, smallest normal
    assert v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9  # subnormals
    assert v[0x00] == 0.0 and np.signbit(v[0x80])
    fin = ~np.isnan(v)
    assert np.array_equal(O.e4m3_encode(v[fin]), codes[fin])
    # the finite values are distinct except +-0, and symmetric
    pos = np.sort(v[fin & ~np.signbit(v)])
    assert len(np.unique(pos)) == 127 and np.all(np.diff(pos) > 0)
    assert np.array_equal(np.sort(-v[fin & np.signbit(v)]), np.sort(v[fin & ~np.signbit(v)]))


def test_e4m3_round_is_nearest_even_on_the_grid():
    grid = O.e4m3_decode(np.arange(256, dtype=np.uint8))
    ok = ~np.isnan(grid)
    gv, gc = grid[ok], np.arange(256)[ok]
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(4000) * 50, rng.standard_normal(2000) * 0.01,
                        (gv[:-1] + np.roll(gv, -1)[:-1]) / 2])      # include midpoints
    v = v[np.abs(v) <= 448]
    got = O.e4m3_round(v)
    for x, y in zip(v, got):
        dist = np.abs(gv - x)
        best = np.nonzero(dist == dist.min())[0]
        if len(best) > 1:          # a tie: the even mantissa (code bit 0 clear) wins
            best = [b for b in best if gc[b] % 2 == 0 and np.signbit(gv[b]) == np.signbit(x)] or best
        assert y == gv[best[0]] or (y == 0 and gv[best[0]] == 0), (x, y, gv[best])


def test_e4m3_saturation_and_ties():
    r = O.e4m3_round
    assert r(470.0) == 448.0 and r(-1000.0) == -448.0 and r(464.0) == 448.0
    assert r(1.0625) == 1.0 and r(1.1875) == 1.25            # ties to the even mantissa
    assert r(2.0 ** -10) == 0.0 and r(3 * 2.0 ** -10) == 2 * 2.0 ** -9


def test_mx_block_scale_closed_form():
    # a block whose largest magnitude lies in [2^j, 2^(j+1)) gets scale 2^(j - 8)
    for j in (-20, -3, 0, 5, 40):
        v = np.zeros(32)
        v[7] = 1.5 * 2.0 ** j
        v[3] = -0.25 * 2.0 ** j
        c, s = O.mx_quantize(v)
        assert s.tolist() == [j - 8 + 127]
        deq = O.mx_dequantize(c, s)
        assert deq[7] == 1.5 * 2.0 ** j and deq[3] == -0.25 * 2.0 ** j
    c, s = O.mx_quantize(np.zeros(64))
    assert s.tolist() == [0, 0] and not c.any()


def test_mx_quantize_matches_brute_force():
    rng = np.random.default_rng(9)
    v = rng.standard_normal((4, 96)) * np.exp2(rng.integers(-6, 6, size=(4, 1)))
    c, s = O.mx_quantize(v, axis=1)
    deq = O.mx_dequantize(c, s, axis=1)
    grid = O.e4m3_decode(np.arange(256, dtype=np.uint8))
    grid = np.unique(grid[~np.isnan(grid)])
    for i in range(4):
        for b in range(3):
            blk = v[i, 32 * b:32 * b + 32]
            e = int(np.floor(np.log2(np.abs(blk).max())))
            scale = 2.0 ** (e - 8)
            assert s[i, b] == e - 8 + 127
            for x, y in zip(blk, deq[i, 32 * b:32 * b + 32]):
                t = min(abs(x) / scale, 448.0)
                near = grid[np.argmin(np.abs(grid - t))]
                assert abs(abs(y) / scale - t) <= abs(near - t) + 1e-15
    # quantisation along axis 0 is the same as along axis 1 of the transpose
    c0, s0 = O.mx_quantize(v.T, axis=0)
    assert np.array_equal(c0, c.T) and np.array_equal(s0, s.T)


def test_mx_ffn_reduces_to_dense_on_grid_values():
    """Inputs already exact in MXFP8 pass the quantisers unchanged, so the MX
    FFN equals the plain FFN on them (the hidden layer is also put on the grid
    by making the second linear act on an exact hidden value: GELU of 0 = 0)."""
    rng = np.random.default_rng(4)
    d, f, T = 64, 64, 5
    on_grid = lambda a, ax: O.mx_qdq(a, axis=ax)  # noqa: E731
    x = on_grid(rng.standard_normal((T, d)), 1)
    w1 = on_grid(rng.standard_normal((d, f)) * 0.1, 0)
    w2 = on_grid(rng.standard_normal((f, d)) * 0.1, 0)
    r = np.ones(T)
    a = x @ w1
    h = O.gelu(a)
    ref = O.mx_qdq(h, axis=1) @ w2
    assert np.allclose(O.ffn_mxfp8(x, r, w1, w2, "gelu"), ref, rtol=0, atol=1e-12)
    # and MX quantisation error stays within the E4M3 bound relative to block max
    full = O.ffn(x, r, w1, w2, "gelu")
    assert np.max(np.abs(O.ffn_mxfp8(x, r, w1, w2, "gelu") - full)) < 0.1 * np.max(np.abs(full))


def _e4m3_positive_grid():
    """Every finite non-negative E4M3 value, from the bit fields: exponent 0
    is subnormal m * 2^-9, otherwise (1 + m/8) * 2^(e-7); S.1111.111 is NaN."""
    vals = [m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
            for e in range(16) for m in range(8) if not (e == 15 and m == 7)]
    return np.array(sorted(set(vals)))


def _mx_grid_operand(rng, shape, axis, grid, s_lo, s_hi):
    """(Q, A): Q lies on the MXFP8 grid along `axis` (each block of 32 shares
    a power-of-two scale 2^s, s drawn from [s_lo, s_hi), and holds E4M3 values
    in [32, 416] times 2^s, its largest in [288, 416] so that
    floor(log2 max) = s + 8); A = Q plus a perturbation of
    at most a fifth of each element's quantum, so MXFP8 quantisation of A along
    `axis` gives back exactly Q (the perturbation keeps every block's binade of
    the maximum and stays inside each element's rounding interval)."""
    normal = grid[(grid >= 32.0) & (grid <= 416.0)]
    big = grid[(grid >= 288.0) & (grid <= 416.0)]
    q = np.moveaxis(rng.choice(normal, size=shape) * rng.choice([-1.0, 1.0], size=shape), axis, -1)
    nb = q.shape[-1] // 32
    qb = q.reshape(q.shape[:-1] + (nb, 32))
    flat = qb.reshape(-1, 32)
    at = rng.integers(0, 32, size=flat.shape[0])
    flat[np.arange(flat.shape[0]), at] = rng.choice(big, size=flat.shape[0]) * \
        rng.choice([-1.0, 1.0], size=flat.shape[0])
    s = rng.integers(s_lo, s_hi, size=qb.shape[:-1])
    qb = flat.reshape(qb.shape) * np.exp2(s)[..., None]
    quantum = np.exp2(np.floor(np.log2(np.abs(qb))) - 3.0)
    a = qb + 0.2 * rng.uniform(-1.0, 1.0, size=qb.shape) * quantum
    back = lambda t: np.moveaxis(t.reshape(q.shape), -1, axis)  # noqa: E731
    return back(qb), back(a)


def _bruteforce_qdq_rows(h, grid):
    """MXFP8 quantise-dequantise along axis 1 by brute force: per block of 32
    the scale is 2^(floor(log2 max|v|) - 8); each element goes to the nearest
    grid value of |v| / scale (clamped to 448), with its sign."""
    out = np.empty_like(h)
    for i in range(h.shape[0]):
        for b in range(h.shape[1] // 32):
            blk = h[i, 32 * b:32 * b + 32]
            scale = 2.0 ** (math.floor(math.log2(np.max(np.abs(blk)))) - 8)
            t = np.minimum(np.abs(blk) / scale, 448.0)
            near = grid[np.argmin(np.abs(grid[None, :] - t[:, None]), axis=1)]
            out[i, 32 * b:32 * b + 32] = np.sign(blk) * near * scale
    return out


def _mx_ffn_case(act, seed):
    """Operands off the MXFP8 grid whose quantised values are known by
    construction, r far from 1 and not a power of two, and the expected
    output of the MXFP8 expert FFN built from those values by hand: x rows
    quantised along d, w1 / w3 along d (per column), r on the first linear's
    accumulator, SiLU(gate) * up (or GELU), h quantised along f, w2 along f."""
    rng = _rng(seed)
    grid = _e4m3_positive_grid()
    T, d, f = 6, 64, 96
    # blocks of x at 2^-3 .. 2^1, of the weights at 2^-8 .. 2^-4, so the hidden
    # pre-activations are O(1) and blocks of one row differ in scale
    qx, x = _mx_grid_operand(rng, (T, d), 1, grid, -11, -7)
    q1, w1 = _mx_grid_operand(rng, (d, f), 0, grid, -16, -12)
    q3, w3 = _mx_grid_operand(rng, (d, f), 0, grid, -16, -12)
    q2, w2 = _mx_grid_operand(rng, (f, d), 0, grid, -16, -12)
    r = rng.uniform(0.55, 1.45, size=T)
    a = r[:, None] * (qx @ q1)
    if act == "swiglu":
        h = a / (1.0 + np.exp(-a)) * (r[:, None] * (qx @ q3))
    else:
        h = 0.5 * a * (1.0 + np.vectorize(math.erf)(a / math.sqrt(2.0)))
    ref = _bruteforce_qdq_rows(h, grid) @ q2
    return dict(x=x, r=r, w1=w1, w3=w3 if act == "swiglu" else None, w2=w2, ref=ref)


def _mx_ffn_mutant(kind):
    """Plausible mistakes in the MXFP8 FFN, each a copy of the composition
    with one step changed (planted on the CPU only, to show the pin sees it)."""
    def run(xhat, r, w1, w2, act, w3=None):
        r = np.asarray(r, dtype=np.float64)[:, None]
        if kind == "r_before_quant":
            xq = O.mx_qdq(r * xhat, axis=1)
            a = xq @ O.mx_qdq(w1, axis=0)
            u = None if w3 is None else xq @ O.mx_qdq(w3, axis=0)
        else:
            xq = O.mx_qdq(xhat, axis=1)
            a = r * (xq @ O.mx_qdq(w1, axis=0))
            w3q = {"w3_unquantised": lambda w: w, "w3_wrong_axis": lambda w: O.mx_qdq(w, axis=1),
                   "w1_wrong_axis": lambda w: O.mx_qdq(w, axis=0)}[kind](w3) if w3 is not None else None
            if kind == "w1_wrong_axis":
                a = r * (xq @ O.mx_qdq(w1, axis=1))
            u = None if w3q is None else r * (xq @ w3q)
        h = O.silu(a) * u if act == "swiglu" else O.gelu(a)
        return O.mx_qdq(h, axis=1) @ O.mx_qdq(w2, axis=0)
    return run


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_mx_ffn_matches_hand_built_quantised_product(act):
    """The MXFP8 expert FFN with r != 1 equals the product built by hand from
    operand values known to be the MXFP8 quantisation of the inputs; each
    plausible misplacement of a quantiser or of r misses it by orders of
    magnitude more than the oracle does."""
    c = _mx_ffn_case(act, 31 if act == "swiglu" else 32)
    den = np.max(np.abs(c["ref"]))
    err = lambda fn: float(np.max(np.abs(fn(c["x"], c["r"], c["w1"], c["w2"], act, c["w3"])  # noqa: E731
                                        - c["ref"])) / den)
    e0 = err(O.ffn_mxfp8)
    assert e0 < 1e-12
    mutants = ["r_before_quant", "w1_wrong_axis"]
    if act == "swiglu":
        mutants += ["w3_unquantised", "w3_wrong_axis"]
    for kind in mutants:
        em = err(_mx_ffn_mutant(kind))
        assert em > 2e-3, (kind, em)


# ---------------------------------------------------------------- backward pass

def test_activation_derivatives_match_finite_differences():
    z = np.linspace(-6.0, 6.0, 241)
    h = 1e-5
    for f, df in ((O.gelu, O.gelu_grad), (O.gelu_tanh, O.gelu_tanh_grad), (O.silu, O.silu_grad)):
        fd = (f(z + h) - f(z - h)) / (2 * h)
        assert np.max(np.abs(df(z) - fd)) < 1e-8
    # textbook values: GELU'(0) = SiLU'(0) = 1/2, GELU'(z) = Phi(z) + z phi(z)
    assert O.gelu_grad(0.0) == 0.5 and O.silu_grad(0.0) == 0.5 and O.gelu_tanh_grad(0.0) == 0.5
    assert abs(O.gelu_grad(1.0) - (ndtr(1.0) + math.exp(-0.5) / math.sqrt(2 * math.pi))) < 1e-15


def _bwd_case(act, renorm, gamma, bias, shared, cf, k, seed):
    rng = _rng(seed)
    T, d, E, f = 7, 8, 4, 16
    p = dict(k=k, eps=1e-6, renorm=renorm, cf=cf, act=act, residual=True, pad=1,
             gamma=(1.0 + 0.1 * rng.standard_normal(d)) if gamma else None,
             router="dense", w_router=rng.standard_normal((d, E)),
             bias=rng.standard_normal(E) if bias else None,
             w1=0.5 * rng.standard_normal((d, E * f)), w2=0.5 * rng.standard_normal((E * f, d)),
             w3=0.5 * rng.standard_normal((d, E * f)) if act == "swiglu" else None,
             f_offsets=[i * f for i in range(E + 1)])
    if shared:
        p.update(ws1=0.5 * rng.standard_normal((d, 2 * f)), ws2=0.5 * rng.standard_normal((2 * f, d)),
                 shared_act=act, ws3=0.5 * rng.standard_normal((d, 2 * f)) if act == "swiglu" else None)
    x = rng.standard_normal((T, d))
    G = rng.standard_normal((T, d))
    return p, x, G


@pytest.mark.parametrize("act,renorm,gamma,bias,shared,cf,k,seed", [
    ("gelu", 1, True, True, False, 0.75, 2, 1),       # drops, gain, bias
    ("swiglu", 0, False, False, True, 0.0, 2, 2),      # full-softmax gates, shared experts
    ("gelu_tanh", 1, True, False, True, 0.0, 4, 3),    # k = E
    ("swiglu", 1, True, True, False, 0.5, 1, 4),       # switch routing with drops
])
def test_layer_backward_matches_finite_differences(act, renorm, gamma, bias, shared, cf, k, seed):
    """Every gradient of the oracle's backward against central differences
    of the oracle's forward (the routing frozen at the forward's own ids; the
    selection and the capacity rule are piecewise constant)."""
    p, x, G = _bwd_case(act, renorm, gamma, bias, shared, cf, k, seed)
    base = O.layer_forward(p, x)
    ids = base["ids"]
    grads = O.layer_backward(p, x, G, ids_override=ids)
    assert np.array_equal(grads["ids"], ids)
    if cf > 0:
        assert np.any(grads["pos"] < 0)               # the case really drops slots
    h = 1e-6

    def loss(pp, xx):
        return float(np.sum(O.layer_forward(pp, xx, ids_override=ids)["out"] * G))

    def fd(name):
        if name == "x":
            v = x
        else:
            v = p[name]
        g = np.zeros_like(v)
        for idx in np.ndindex(v.shape):
            vp, vm = v.copy(), v.copy()
            vp[idx] += h
            vm[idx] -= h
            if name == "x":
                g[idx] = (loss(p, vp) - loss(p, vm)) / (2 * h)
            else:
                g[idx] = (loss(dict(p, **{name: vp}), x) - loss(dict(p, **{name: vm}), x)) / (2 * h)
        return g

    pairs = [("x", "dx"), ("w_router", "dw_router"), ("w1", "dw1"), ("w2", "dw2")]
    if gamma:
        pairs.append(("gamma", "dgamma"))
    if bias:
        pairs.append(("bias", "dbias"))
    if act == "swiglu":
        pairs.append(("w3", "dw3"))
    if shared:
        pairs += [("ws1", "dws1"), ("ws2", "dws2")] + ([("ws3", "dws3")] if act == "swiglu" else [])
    for name, gname in pairs:
        num = fd(name)
        ana = grads[gname]
        scale = max(np.max(np.abs(num)), 1e-3)
        assert np.max(np.abs(ana - num)) < 1e-6 * scale, (name, np.max(np.abs(ana - num)), scale)


def test_gates_backward_special_cases():
    rng = _rng(9)
    l = rng.standard_normal((5, 6))
    # k = E with renorm: the gates are the full softmax in selection order, so
    # both readings give the same logit gradient (the softmax Jacobian)
    ids = O.select_topk(l, 6)
    dg = rng.standard_normal((5, 6))
    a = O.gates_backward(l, ids, 1, dg)
    b = O.gates_backward(l, ids, 0, dg)
    assert np.allclose(a, b, atol=1e-14)
    P = sp_softmax(l, axis=1)
    dP = np.zeros_like(l)
    np.put_along_axis(dP, ids.astype(np.int64), dg, axis=1)
    J = np.einsum("te,ef->tef", P, np.eye(6)) - np.einsum("te,tf->tef", P, P)
    assert np.allclose(a, np.einsum("tef,te->tf", J, dP), atol=1e-14)
    # switch routing (k = 1, renorm): the gate is identically 1, so no gradient
    ids1 = O.select_topk(l, 1)
    assert np.all(O.gates_backward(l, ids1, 1, rng.standard_normal((5, 1))) == 0)
    # the logit gradient of renormalised gates sums to zero per token (shift invariance)
    ids2 = O.select_topk(l, 3)
    assert np.allclose(O.gates_backward(l, ids2, 1, rng.standard_normal((5, 3))).sum(axis=1), 0,
                       atol=1e-14)


def test_backward_token_subset_and_unit_slices_agree_with_the_whole():
    """The two restrictions the full-size GPU tests use: layer_backward on a
    token subset returns those tokens' rows of the full computation, and
    expert_unit_grads returns the units' slices of the full weight gradients."""
    p, x, G = _bwd_case("swiglu", 0, True, True, True, 0.75, 2, 5)
    ids = O.layer_forward(p, x)["ids"]
    full = O.layer_backward(p, x, G, ids_override=ids)
    tok = np.array([0, 3, 6])
    part = O.layer_backward(p, x, G, ids_override=ids, tokens=tok)
    for key in ("dx", "dxhat", "dr", "dg", "dl"):
        assert np.allclose(part[key], full[key][tok], rtol=1e-12, atol=1e-14), key
    assert "dw1" not in part and "dw_router" not in part
    units = np.array([1, 5, 15])
    for e in range(4):
        u = O.expert_unit_grads(p, x, G, ids, e, units)
        cols = p["f_offsets"][e] + units
        assert np.allclose(u["dw1"], full["dw1"][:, cols], rtol=1e-12, atol=1e-14)
        assert np.allclose(u["dw3"], full["dw3"][:, cols], rtol=1e-12, atol=1e-14)
        assert np.allclose(u["dw2"], full["dw2"][cols, :], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- work precision

@pytest.mark.parametrize("kind", ["dense_swiglu_shared", "cartesian_atomic"])
def test_float32_work_precision_matches_float64(kind):
    """The float32 work precision (used only to time the CPU baseline) computes
    the same layer: outputs within float32 rounding of the float64 default,
    the same routing except at near-ties, and float64 is the default."""
    rng = _rng(41)
    T, d = 40, 64
    x = rng.standard_normal((T, d)).astype(np.float32)
    if kind == "dense_swiglu_shared":
        E, f, k = 6, 96, 2
        p = dict(k=k, eps=1e-6, renorm=1, cf=1.0, act="swiglu", residual=True, pad=1,
                 router="dense", w_router=0.1 * rng.standard_normal((d, E)), bias=None,
                 w1=0.1 * rng.standard_normal((d, E * f)), w3=0.1 * rng.standard_normal((d, E * f)),
                 w2=0.1 * rng.standard_normal((E * f, d)), f_offsets=[f * e for e in range(E + 1)],
                 ws1=0.1 * rng.standard_normal((d, 64)), ws3=0.1 * rng.standard_normal((d, 64)),
                 ws2=0.1 * rng.standard_normal((64, d)), shared_act="swiglu")
    else:
        Nr = Nc = 16
        k = 8
        p = dict(k=k, eps=1e-6, renorm=1, act="gelu", residual=True, router="cartesian",
                 k_rows=0.2 * rng.standard_normal((d, Nr)), k_cols=0.2 * rng.standard_normal((d, Nc)),
                 W=0.2 * rng.standard_normal((Nr * Nc, d)), V=0.2 * rng.standard_normal((Nr * Nc, d)),
                 ws1=0.1 * rng.standard_normal((d, 64)), ws2=0.1 * rng.standard_normal((64, d)),
                 shared_act="gelu")
    p = {key: (v.astype(np.float32) if isinstance(v, np.ndarray) else v) for key, v in p.items()}
    ref = O.layer_forward(p, x)
    assert ref["out"].dtype == np.float64
    with O.work_precision(np.float32):
        got = O.layer_forward(p, x)
    assert got["out"].dtype == np.float32
    assert O.layer_forward(p, x)["out"].dtype == np.float64       # restored on exit
    err = np.max(np.abs(got["out"] - ref["out"])) / np.max(np.abs(ref["out"]))
    assert err < 1e-5, err
    assert np.array_equal(got["ids"], ref["ids"])
