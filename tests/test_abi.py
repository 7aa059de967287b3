"""The C-ABI library loads, exports every declared entry point, and its host
logic (capacity, row bounds, argument checks) behaves -- no GPU needed.

Only calls that return before touching the HIP runtime are made here: the
host-side capacity / size functions and argument-validation error paths.
"""
import ctypes as C
import json
import re
from pathlib import Path

import numpy as np
import pytest

import oracle as O
from sparse_mixture_experts_rmsnorm_amd import binding as B

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "moe.h"

pytestmark = pytest.mark.skipif(not B.LIB_PATH.exists(),
                                reason="libmoe_mi355x.so not built (run __graft_entry__.build())")


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = B.lib()
    names = declared_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/moe.h but not exported"
    assert set(names) == set(B.EXPORTED)


def test_version():
    assert "gfx950" in B.version()


def test_capacity_matches_oracle_table():
    for c in json.loads((ROOT / "tests/golden/capacity.json").read_text())["cases"]:
        assert B.capacity(c["T"], c["k"], c["E"], c["cf"]) == c["capacity"], c


def test_capacity_matches_oracle_random():
    rng = np.random.default_rng(0)
    for _ in range(2000):
        T = int(rng.integers(0, 1 << 20))
        k = int(rng.integers(1, 65))
        E = int(rng.integers(1, 1 << 12))
        cf = float(rng.choice([rng.uniform(0.01, 4.0), rng.integers(1, 80) / 16.0, 1.1, 0.1, 1.0]))
        assert B.capacity(T, k, E, cf) == O.capacity(T, k, E, cf), (T, k, E, cf)
    assert B.capacity(-1, 2, 8, 1.0) == -1
    assert B.capacity(10, 0, 8, 1.0) == -1
    assert B.capacity(10, 2, 8, float("nan")) == -1
    assert B.capacity(10, 2, 8, float("inf")) == 10


def test_rows_max():
    assert B.rows_max(4096, 2, 8, 1280, 1) == 8192
    assert B.rows_max(4096, 2, 8, 1000, 1) == 8000
    assert B.rows_max(8192, 2, 8, 8192, 128) == 16384 + 8 * 127
    assert B.rows_max(10, 2, 8, 10, 0) == -1


def _err(rc):
    return rc, B.last_error()


def test_argument_errors_are_reported_without_touching_the_gpu():
    lib = B.lib()
    # pack: bad dtype, NULL pointers, in place
    rc, msg = _err(lib.moe_pack_transpose(None, 7, 4, 4, None, None))
    assert rc == -3 and "dtype" in msg
    rc, msg = _err(lib.moe_pack_transpose(None, 1, 4, 4, None, None))
    assert rc == -1
    rc, _ = _err(lib.moe_pack_transpose(C.c_void_p(16), 1, 4, 4, C.c_void_p(16), None))
    assert rc == -1
    # SwiGLU pack: sizes must be multiples of 32
    sizes = B.i64_array([48, 64])
    rc, msg = _err(lib.moe_pack_swiglu(C.c_void_p(16), C.c_void_p(32), 1, 64, sizes, 2,
                                       C.c_void_p(64), None))
    assert rc == -2 and "multiples of 32" in msg
    # router: k > E, E too large, Cartesian constraints
    R = B.RouterDesc(kind=0, E=8, wr_t=16)
    rc, msg = _err(lib.moe_router_topk(C.byref(R), C.c_void_p(16), 1, 10, 256, None, 1e-6,
                                       C.c_void_p(16), 9, 1, C.c_void_p(16), C.c_void_p(16), None,
                                       None, 0, None))
    assert rc == -1 and "k must be" in msg
    R.E = 300
    rc, _ = _err(lib.moe_router_topk(C.byref(R), C.c_void_p(16), 1, 10, 256, None, 1e-6,
                                     C.c_void_p(16), 2, 1, C.c_void_p(16), C.c_void_p(16), None,
                                     None, 0, None))
    assert rc == -4
    Rc = B.RouterDesc(kind=1, E=64 * 64, Nr=64, Nc=64, keys_t=16)
    rc, msg = _err(lib.moe_router_topk(C.byref(Rc), C.c_void_p(16), 1, 10, 256, None, 1e-6,
                                       C.c_void_p(16), 8, 1, C.c_void_p(16), C.c_void_p(16), None,
                                       None, 0, None))
    assert rc == -2 and "multiple of 256" in msg
    # dispatch: rows_max too small, radix path with a capacity limit, no workspace
    P = C.c_void_p(16)
    rc, msg = _err(lib.moe_dispatch(P, P, P, None, 1, 100, 0, 8, 2, 100, 1, 10, P, P, P, P, P, P,
                                    None, None, None, P, 1 << 20, None))
    assert rc == -2 and "rows_max" in msg
    rc, msg = _err(lib.moe_dispatch(P, P, P, None, 1, 100, 0, 1 << 20, 2, 50, 1, 200, P, P, P, P,
                                    P, P, None, None, None, P, 1 << 20, None))
    assert rc == -4 and "radix" in msg
    rc, msg = _err(lib.moe_dispatch(P, P, P, None, 1, 100, 0, 8, 2, 100, 1, 200, P, P, P, P, P, P,
                                    None, None, None, None, 0, None))
    assert rc == -5
    # topology: rows_max not a multiple of the block
    rc, _ = _err(lib.moe_build_topology(P, P, P, 8, 128, 1000, P, P, P, None))
    assert rc == -2
    # combine: d not filling 16-byte vectors
    rc, _ = _err(lib.moe_combine(P, P, P, None, 1, 4, 12, 2, P, None))
    assert rc == -2


def test_expert_descriptor_checks():
    lib = B.lib()
    sizes = B.i64_array([384, 256])
    X = B.ExpertsDesc(kind=0, act=0, E=2, ffn_sizes=C.cast(sizes, C.POINTER(C.c_int64)),
                      ffn_offsets=16, w13_t=16, w2_t=16)
    # GELU bf16 needs ffn sizes that are multiples of 256
    assert lib.moe_expert_workspace_size(C.byref(X), 1, 512, 100, 2, 200) == 0
    X.act = 2     # SwiGLU: multiples of 128 suffice
    assert lib.moe_expert_workspace_size(C.byref(X), 1, 512, 100, 2, 200) > 0
    X.act = 5
    assert lib.moe_expert_workspace_size(C.byref(X), 1, 512, 100, 2, 200) == 0
    X.act = 2
    assert lib.moe_expert_workspace_size(C.byref(X), 1, 500, 100, 2, 200) == 0   # d % 256
    # MXFP8: scales required, bf16 grouped or BCSR, ffn sizes multiples of 128
    n_bf16 = lib.moe_expert_workspace_size(C.byref(X), 1, 512, 100, 2, 200)
    X.quant = B.QUANT_MXFP8
    assert lib.moe_expert_workspace_size(C.byref(X), 1, 512, 100, 2, 200) == 0
    assert "w13_scale" in B.last_error()
    X.w13_scale, X.w2_scale = 16, 16
    n_mx = lib.moe_expert_workspace_size(C.byref(X), 1, 512, 100, 2, 200)
    assert n_mx > 0 and n_mx != n_bf16
    assert lib.moe_expert_workspace_size(C.byref(X), 0, 512, 100, 2, 200) == 0   # f32
    X.kind = 1
    assert lib.moe_expert_workspace_size(C.byref(X), 1, 512, 100, 2, 200) == 0   # BCSR, block 0
    assert "block" in B.last_error()
    X.block, X.size_blocks, X.block_offsets = 128, 16, 16
    assert lib.moe_expert_workspace_size(C.byref(X), 1, 512, 100, 2, 256) > 0    # MXFP8 BCSR
    X.kind, X.block, X.size_blocks, X.block_offsets = 0, 0, None, None
    # w2_ld: 0 (dense) or a stride >= F in whole 16-byte units
    X.w2_ld = 512                                                                 # < F = 640
    assert lib.moe_expert_workspace_size(C.byref(X), 1, 512, 100, 2, 200) == 0
    assert "w2_ld" in B.last_error()
    X.w2_ld = 648                                                                 # MXFP8: 648 B
    assert lib.moe_expert_workspace_size(C.byref(X), 1, 512, 100, 2, 200) == 0
    X.w2_ld = 656
    assert lib.moe_expert_workspace_size(C.byref(X), 1, 512, 100, 2, 200) > 0
    X.quant, X.w2_ld = 0, 644                                                     # bf16: 1288 B
    assert lib.moe_expert_workspace_size(C.byref(X), 1, 512, 100, 2, 200) == 0
    X.w2_ld = 648
    assert lib.moe_expert_workspace_size(C.byref(X), 1, 512, 100, 2, 200) > 0
    X.quant, X.w2_ld = B.QUANT_MXFP8, 0
    sizes2 = B.i64_array([320, 256])
    X.ffn_sizes = C.cast(sizes2, C.POINTER(C.c_int64))
    assert lib.moe_expert_workspace_size(C.byref(X), 1, 512, 100, 2, 200) == 0
    assert "multiples of 128" in B.last_error()
    X.quant = 7
    X.ffn_sizes = C.cast(sizes, C.POINTER(C.c_int64))
    assert lib.moe_expert_workspace_size(C.byref(X), 1, 512, 100, 2, 200) == 0
    assert "quant" in B.last_error()


def test_mxfp8_pack_argument_checks():
    lib = B.lib()
    P = C.c_void_p(256)
    rc, msg = _err(lib.moe_pack_mxfp8(P, 4, 48, 48, P, 48, P, 2, None))
    assert rc == -2 and "K % 32" in msg
    rc, msg = _err(lib.moe_pack_mxfp8(P, 4, 64, 60, P, 64, P, 2, None))
    assert rc == -2 and "strides" in msg
    rc, _ = _err(lib.moe_pack_mxfp8(None, 4, 64, 64, P, 64, P, 2, None))
    assert rc == -1
    rc, msg = _err(lib.moe_pack_mxfp8(C.c_void_p(264), 4, 64, 64, P, 64, P, 2, None))
    assert rc == -1 and "aligned" in msg
    assert lib.moe_pack_mxfp8(None, 0, 64, 64, None, 64, None, 2, None) == 0   # nothing to do


def test_mxfp8_weight_pack_argument_checks():
    lib = B.lib()
    P = C.c_void_p(256)
    rc, msg = _err(lib.moe_pack_mxfp8_weights(P, 4, 96, 96, P, 96, P, None))
    assert rc == -2 and "K % 128" in msg                    # stage-major words need K % 128
    rc, msg = _err(lib.moe_pack_mxfp8_weights(P, 4, 128, 124, P, 128, P, None))
    assert rc == -2 and "strides" in msg
    rc, msg = _err(lib.moe_pack_mxfp8_weights(P, 4, 128, 128, P, 120, P, None))
    assert rc == -2 and "strides" in msg
    rc, _ = _err(lib.moe_pack_mxfp8_weights(P, 4, 128, 128, P, 128, None, None))
    assert rc == -1
    rc, msg = _err(lib.moe_pack_mxfp8_weights(C.c_void_p(264), 4, 128, 128, P, 128, P, None))
    assert rc == -1 and "aligned" in msg
    rc, msg = _err(lib.moe_pack_mxfp8_weights(P, 1 << 26, 1 << 12, 1 << 12, P, 1 << 12, P, None))
    assert rc == -2 and "2 GiB" in msg
    assert lib.moe_pack_mxfp8_weights(None, 0, 128, 128, None, 128, None, None) == 0


def test_layer_workspace_validation():
    lib = B.lib()
    assert lib.moe_layer_workspace_size(None, 10) == 0
    sizes = B.i64_array([256] * 5)
    L = B.LayerDesc(d=512, dtype=1, eps=1e-6, k=2, renorm=1, capacity_factor=1.25, residual=1)
    L.router = B.RouterDesc(kind=0, E=4, wr_t=16)
    L.experts = B.ExpertsDesc(kind=0, act=2, E=4, ffn_sizes=C.cast(sizes, C.POINTER(C.c_int64)),
                              ffn_offsets=16, w13_t=16, w2_t=16)
    n = lib.moe_layer_workspace_size(C.byref(L), 1000)
    assert n > 1000 * 512 * 2
    L.experts.E = 5
    assert lib.moe_layer_workspace_size(C.byref(L), 1000) == 0
    assert "router E" in B.last_error()
