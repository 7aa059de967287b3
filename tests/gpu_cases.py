"""Shared helpers of the GPU parity tests: workload cases, oracle parameters,
error metrics.  Inputs come from the seeded generator; expected values come
only from the oracle."""
from __future__ import annotations

import numpy as np

import oracle as O
from sparse_mixture_experts_rmsnorm_amd.workloads import WORKLOADS, Workload

# Small layers the oracle finishes in seconds; each spans several GEMM tiles
# (256 features x 128 rows) with ragged tails, and together they cover every
# router / expert kind, drops, empty experts, a gain, k = 1 and k = E.
SMALL = {
    "tiny_fp32": WORKLOADS["tiny_fp32"],
    "fp32_swiglu_drops": Workload("fp32_swiglu_drops", T=100, d=128, E=4, k=2, dtype="f32",
                                  act="swiglu", ffn=128, cf=0.75, bias="normal", seed=16),
    "mixtral_small_drops": Workload("mixtral_small_drops", T=300, d=512, E=8, k=2, act="swiglu",
                                    ffn=384, cf=1.0, bias="normal", seed=11),
    "mixtral_small": Workload("mixtral_small", T=700, d=512, E=8, k=2, act="swiglu", ffn=640,
                              cf=1.25, seed=17),
    "gelu_gamma_switch": Workload("gelu_gamma_switch", T=257, d=256, E=4, k=1, act="gelu",
                                  ffn=512, cf=2.0, gamma=True, seed=12),
    "gelu_tanh_dense_mixture": Workload("gelu_tanh_dense_mixture", T=130, d=256, E=4, k=4,
                                        act="gelu_tanh", ffn=256, cf=0.0, seed=18),
    "bcsr_small": Workload("bcsr_small", T=600, d=256, E=4, k=2, act="gelu",
                           expert_sizes=((1, 512), (3, 256)), bias="normal", expert_kind="bcsr",
                           seed=13),
    # BCSR under a skewed router (Zipf bias): token-block counts 3, 1, 1, 0, 4, 1 per
    # expert, so the walk pairs blocks, leaves lone last blocks and skips an empty expert
    "bcsr_skew": Workload("bcsr_skew", T=500, d=256, E=6, k=2, act="gelu",
                          expert_sizes=((2, 512), (4, 256)), bias="zipf", zipf_s=0.8,
                          expert_kind="bcsr", seed=40),
    "finegrained_small": Workload("finegrained_small", T=500, d=256, E=64, k=6, act="swiglu",
                                  ffn=128, cf=1.5, bias="zipf", shared_ffn=256, seed=14),
    "mixtral_small_mxfp8": Workload("mixtral_small_mxfp8", T=700, d=512, E=8, k=2,
                                    act="swiglu", ffn=640, cf=1.25, quant="mxfp8", seed=19),
    "gelu_mxfp8_split": Workload("gelu_mxfp8_split", T=333, d=256, E=4, k=2, act="gelu",
                                 ffn=512, cf=1.0, bias="normal", shared_ffn=256,
                                 shared_act="gelu", quant="mxfp8", seed=20),
    "mxfp8_tiny": Workload("mxfp8_tiny", T=13, d=256, E=8, k=2, act="gelu", ffn=256, cf=0.0,
                           quant="mxfp8", seed=22),
    "atomic_small": Workload("atomic_small", T=200, d=512, E=128 * 128, k=8, act="gelu",
                             router="cartesian", Nr=128, Nc=128, expert_kind="atomic",
                             shared_ffn=512, shared_act="gelu", seed=15),
    # more tiles than compute units in both expert GEMMs (512 and ~400 with the
    # second one split), so each persistent workgroup runs several tiles and
    # issues the next tile's first loads before its epilogue
    "persistent_tiles": Workload("persistent_tiles", T=4096, d=512, E=8, k=2, act="swiglu",
                                 ffn=2048, cf=1.25, seed=23),
    # ffn a multiple of 256 and few tiles: a K split would fill the second
    # GEMM's last round, so that round's tiles are cut into K pieces whose
    # fp32 partials the fixup kernel sums in part order
    "split4_small": Workload("split4_small", T=600, d=512, E=8, k=2, act="swiglu", ffn=512,
                             cf=1.25, seed=24),
    # one expert, k = 1: every token's gate is 1 and the layer is a dense FFN
    "single_expert": Workload("single_expert", T=300, d=256, E=1, k=1, act="gelu", ffn=512,
                              cf=0.0, seed=25),
    # a wide model: K of 8192 in the router and the first GEMM (128 stages),
    # 32 output tiles in the second
    "wide_d": Workload("wide_d", T=96, d=8192, E=4, k=2, act="swiglu", ffn=256, cf=1.5,
                       seed=26),
    # MXFP8 operands on the block-sparse (BCSR) walk: 128-row token blocks,
    # variable expert sizes
    "bcsr_small_mxfp8": Workload("bcsr_small_mxfp8", T=600, d=256, E=4, k=2, act="gelu",
                                 expert_sizes=((1, 512), (3, 256)), bias="normal",
                                 expert_kind="bcsr", quant="mxfp8", seed=27),
}

# max |gpu - ref| / max |ref| per output tensor
TOL = {"f32": 1e-3, "bf16": 2e-2}

# measured errors of this session's parity tests, printed at the end of the
# run by the terminal-summary hook in conftest.py
RESULTS: list = []


def record(test: str, **errs) -> None:
    """Keep the measured errors of one parity case for the session summary."""
    RESULTS.append((test, errs))


def rel_err(gpu, ref) -> float:
    """max |gpu - ref| / max |ref| (the absolute error when ref is all zero)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not ref.size:
        return 0.0
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(gpu - ref)) / (den if den > 0 else 1.0))


def oracle_params(wl: Workload, inp: dict) -> dict:
    p = dict(k=wl.k, eps=wl.eps, renorm=wl.renorm, cf=wl.cf, act=wl.act, residual=True,
             gamma=inp.get("gamma"), pad=wl.pad)
    if wl.router == "cartesian":
        p.update(router="cartesian", k_rows=inp["k_rows"], k_cols=inp["k_cols"], W=inp["W"],
                 V=inp["V"])
    else:
        p.update(router="dense", w_router=inp["w_router"], bias=inp.get("bias"), w1=inp["w1"],
                 w3=inp.get("w3"), w2=inp["w2"], f_offsets=wl.f_offsets)
    if wl.quant != "none":
        p.update(quant=wl.quant)
    if wl.shared_ffn:
        p.update(ws1=inp["ws1"], ws3=inp.get("ws3"), ws2=inp["ws2"], shared_act=wl.shared_act)
    return p


def f64(a) -> np.ndarray:
    return O.as_f64(a)


def near_tie_tokens(ref_sorted: np.ndarray, k: int, tau: float) -> np.ndarray:
    """Tokens whose reference scores, sorted in descending order, have two
    neighbours among the first k+1 closer than tau: there the k selected ids
    or their order are decided by rounding, not by the scores."""
    m = min(k + 1, ref_sorted.shape[1])
    gaps = ref_sorted[:, :m - 1] - ref_sorted[:, 1:m]
    return np.nonzero(np.any(gaps < tau, axis=1))[0]


def check_ids_against_reference(ids_gpu, ids_ref, ref_sorted, k, tau, what=""):
    """ids_gpu must equal ids_ref on every token except near-ties (step 4 of
    the routing protocol); returns (mismatches, near-tie tokens)."""
    bad = np.nonzero(np.any(np.asarray(ids_gpu) != np.asarray(ids_ref), axis=1))[0]
    near = near_tie_tokens(ref_sorted, k, tau)
    unexplained = np.setdiff1d(bad, near)
    print(f"  {what}ids against the oracle's own routing: {len(bad)} differ, "
          f"{len(near)} near-ties under tau={tau:.3e}", flush=True)
    assert len(unexplained) == 0, unexplained[:10]
    return len(bad), len(near)
