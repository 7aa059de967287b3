"""Plain CPU oracle for the forward pass of one sparse MoE FFN layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test-suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP path.

Everything is computed in float64 from the exact values of the inputs (bf16
inputs arrive as uint16 bit patterns and are widened exactly).  Loops, sorts
and matrix products are the plain definitions; nothing is blocked, fused or
reordered beyond what the cited passage states.

Sources (web pages; cited by title and section):
  [CODA]   "CODA for sparse MoEs" thread (digg.com/tech/6tc58j9c) -- the
           paragraphs on the RMSNorm r-scale commuted across the GEMM into its
           epilogue, the router fusion, and dispatch carrying the r-scale.
  [GLOSS]  "Mixture of Experts (MoE)" glossary (inferensys.com) -- entries on
           experts, the gating network, top-k / switch routing, expert
           capacity, and fused MoE kernels.
  [VAREXP] "Variable-size experts" nanoMOE implementation notes
           (hbfreed.com) -- sections 2 (offset calculation, buffers, weight
           allocation), 3 (indices kernel), the output-array-indexing bug fix,
           and 4 (topology construction).
  [OMNI]   "OmniMoE" technical summary (gist.science, Italian) -- section 2.1
           (atomic experts, dynamic expert assembly, shared dense MLP) and
           section 2.2 (Cartesian-product router, expert-centric scheduling).

Readings taken where the pages are silent:
  * RMSNorm is x * (mean(x^2) + eps)^-1/2 * gamma, eps inside the root.
  * The r-scale multiplies the accumulator of every GEMM that consumes the
    normed activation (router, W1, W3) before bias / activation; never W2.
  * Top-k compares the post-scale, post-bias logits; ties go to the lower
    expert index; slots are ordered by descending logit.
  * Gate = softmax over the k selected logits (renorm=1) or the full-softmax
    probability (renorm=0).
  * Noise top-k adds noise_std * (caller-supplied N(0,1) draws) to the logits
    before selection; gates and statistics use the noisy logits.
  * The load-balancing auxiliary loss is the squared coefficient of
    variation (population variance / mean^2) across experts of the summed
    full-softmax router probabilities.
  * Capacity = ceil(T*k*cf/E) computed exactly, clamped to [0, T]; cf <= 0
    means "no limit" (= T).  Within an expert, tokens are kept in token order.
  * Dropped slots contribute zero; kept gates are not renormalised.  The
    layer output includes the residual x, so a fully dropped token passes
    through unchanged.
  * GELU is the exact erf form (a tanh form is available by flag).
  * SwiGLU: w1 is the gate (SiLU), w3 the up projection, w2 the down
    projection; no FFN biases.
  * Cartesian expert n = i*Nc + j scores s1[i] + s2[j]; both sub-tables see
    the full r-scaled input.  Atomic gates are a softmax over the k selected
    scores.

Parity status: every function here is pinned by tests in
tests/test_oracle_pins.py (closed forms, special cases, brute force, the
worked examples printed in [VAREXP]).  The numeric output values of a whole
layer are not printed anywhere on the pages, so tolerance parity against this
float64 oracle is the check for the floating-point outputs.
"""
from __future__ import annotations

import contextlib
import math
from fractions import Fraction

import numpy as np
from scipy.special import erf

__all__ = [
    "bf16_to_f64", "f64_to_bf16_bits", "as_f64", "work_precision",
    "capacity", "rmsnorm_scale", "rmsnorm", "router_logits", "router_logits_unfused",
    "E4M3_MAX", "MX_BLOCK", "e4m3_decode", "e4m3_round", "e4m3_encode", "mx_quantize",
    "mx_dequantize", "mx_qdq", "ffn_mxfp8",
    "select_topk", "gates", "noisy_logits", "router_probabilities", "squared_cv", "router_stats",
    "dispatch", "expert_layout", "bcsr_topology",
    "gelu", "gelu_tanh", "silu", "ffn", "grouped_expert_ffn", "bcsr_expert_ffn",
    "cartesian_scores", "cartesian_topk", "cartesian_topk_bruteforce",
    "atomic_experts_token_centric", "atomic_experts_expert_centric",
    "combine", "layer_forward",
    "gelu_grad", "gelu_tanh_grad", "silu_grad", "ffn_backward", "gates_backward", "layer_backward",
    "expert_unit_grads",
]


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly to float64.

    A bf16 value is the upper 16 bits of an IEEE float32, so shifting the
    pattern into the high half of a 32-bit word gives the float32 exactly.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round to float32 (nearest-even), then to bf16 (nearest-even); return bits.

    This is the storage rounding of the bf16 path: the GPU holds an fp32
    accumulator and stores it as bf16 with round-to-nearest-even.
    """
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        rounded = np.where(nan, np.uint16(0x7FC0), rounded)
    return rounded


def as_f64(a) -> np.ndarray | None:
    """float64 view of an input tensor: uint16 means bf16 bits, else a float."""
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_to_f64(a)
    return a.astype(np.float64)


# Work precision of the forward pass's floating-point arithmetic.  Every
# test runs the default, float64.  work_precision(np.float32) switches the
# products and sums of the forward (RMSNorm, router, expert and shared FFNs,
# Cartesian scores, atomic experts, combine) to float32 -- the precision the
# benchmark's CPU baseline is timed in; the definitions are the same, and the
# integer decisions (top-k, capacity, dispatch) and the MXFP8 quantiser keep
# their own precision.
_WORK = [np.float64]


@contextlib.contextmanager
def work_precision(dtype):
    """Run the enclosed forward-pass calls in `dtype` (np.float32 or np.float64)."""
    if dtype not in (np.float32, np.float64):
        raise ValueError("work precision must be float32 or float64")
    prev = _WORK[0]
    _WORK[0] = dtype
    try:
        yield
    finally:
        _WORK[0] = prev


def _wd():
    return _WORK[0]


def _aw(a) -> np.ndarray | None:
    """An input tensor in the work precision: uint16 means bf16 bits (widened
    exactly), else a float."""
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(_wd())
    return a.astype(_wd())


# --------------------------------------------------------------------------
# [GLOSS] expert capacity
# --------------------------------------------------------------------------

def capacity(T: int, k: int, E: int, cf: float) -> int:
    """Expert capacity from the [GLOSS] expert-capacity entry.

    The entry gives batch*sequence*k/num_experts*capacity_factor as a real
    number.  It is rounded up (so the theoretical minimum load always fits)
    and clamped to T (an expert can receive at most one slot per token).
    The product is evaluated exactly with rationals: cf is the exact binary
    value of the float given.  cf <= 0 means no capacity limit.
    """
    if T < 0 or k <= 0 or E <= 0:
        raise ValueError("bad capacity arguments")
    if cf <= 0:
        return int(T)
    exact = Fraction(T) * Fraction(k) * Fraction(cf) / Fraction(E)
    c = math.ceil(exact)
    return int(min(max(c, 0), T))


# --------------------------------------------------------------------------
# [CODA] RMSNorm and the r-scale
# --------------------------------------------------------------------------

def rmsnorm_scale(x: np.ndarray, eps: float) -> np.ndarray:
    """Per-token RMSNorm statistic r[t] = (mean_i x[t,i]^2 + eps)^(-1/2).

    [CODA]: the normalisation is a per-row scale by this statistic, which is
    what gets commuted across the following GEMM into its epilogue.
    """
    x = _aw(x)
    return 1.0 / np.sqrt(np.mean(x * x, axis=1) + eps)


def rmsnorm(x: np.ndarray, gamma, eps: float) -> np.ndarray:
    """Unfused RMSNorm output x * r[:,None] * gamma (the textbook form)."""
    x = _aw(x)
    r = rmsnorm_scale(x, eps)
    y = x * r[:, None]
    g = _aw(gamma)
    return y if g is None else y * g[None, :]


def _xhat(x, gamma):
    x = _aw(x)
    g = _aw(gamma)
    return x if g is None else x * g[None, :]


def router_logits(x, gamma, r, w_router, bias=None) -> np.ndarray:
    """Router logits with the r-scale in the epilogue ([CODA] router fusion).

    l[t,e] = r[t] * (xhat[t] . W_r[:,e]) + b[e], xhat = x * gamma.  The GEMM
    runs on the un-normalised input; the statistic is applied to its output
    right before the top-k.  ([GLOSS] gating network: a linear layer giving
    one logit per expert.)
    """
    acc = _xhat(x, gamma) @ _aw(w_router)
    logits = np.asarray(r, dtype=_wd())[:, None] * acc
    if bias is not None:
        logits = logits + _aw(bias)[None, :]
    return logits


def router_logits_unfused(x, gamma, eps, w_router, bias=None) -> np.ndarray:
    """The same logits the textbook way: RMSNorm first, then the GEMM."""
    logits = rmsnorm(x, gamma, eps) @ _aw(w_router)
    if bias is not None:
        logits = logits + _aw(bias)[None, :]
    return logits


# --------------------------------------------------------------------------
# [CODA] low precision: MXFP8 (OCP Microscaling Formats v1.0: blocks of 32
# elements sharing an E8M0 power-of-two scale, elements in FP8 E4M3)
# --------------------------------------------------------------------------

E4M3_MAX = 448.0          # largest finite E4M3 value, 1.75 * 2^8
E4M3_EMAX = 8             # exponent of the largest normal
MX_BLOCK = 32


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code (sign, 4 exponent bits with bias 7, 3 mantissa
    bits; exponent 0 is subnormal m * 2^-9; S.1111.111 is NaN; no infinities)."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def e4m3_round(v) -> np.ndarray:
    """Nearest E4M3 value, ties to even, magnitudes above 448 saturated to
    448 (the MX conversion clamps to the largest normal).  float64 in, out."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e2 = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(e2 - 1, -6)                 # exponent of the binade; subnormals share 2^-6's
    quantum = np.exp2(e - 3.0)                  # 3 mantissa bits
    q = np.rint(a / quantum) * quantum          # rint: ties to even
    q = np.minimum(q, E4M3_MAX)
    return np.copysign(q, v)


def e4m3_encode(v) -> np.ndarray:
    """E4M3 code of values already on the E4M3 grid (|v| <= 448)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    sign = np.where(np.signbit(v), 0x80, 0)
    _, e2 = np.frexp(np.where(a > 0, a, 1.0))
    e = e2 - 1
    sub = a < 2.0 ** -6
    m_sub = np.rint(a / 2.0 ** -9)
    ebits = np.where(sub, 0, e + 7)
    m = np.where(sub, m_sub, np.rint((a / np.exp2(e) - 1.0) * 8.0))
    return (sign | (ebits.astype(np.int64) << 3) | m.astype(np.int64)).astype(np.uint8)


def mx_quantize(v, axis: int = -1):
    """MXFP8 quantisation of v along `axis` in blocks of 32 (the length along
    axis must be a multiple of 32).  Per block: shared exponent
    s = floor(log2(max |v|)) - 8, clamped to [-127, 127] (s = -127 for an
    all-zero block); elements P = e4m3_round(v / 2^s).  Returns (codes uint8
    shaped like v, scale codes uint8 = s + 127 with the axis length / 32)."""
    v = np.moveaxis(np.asarray(v, dtype=np.float64), axis, -1)
    n = v.shape[-1]
    if n % MX_BLOCK:
        raise ValueError("length along the axis must be a multiple of 32")
    b = v.reshape(v.shape[:-1] + (n // MX_BLOCK, MX_BLOCK))
    amax = np.abs(b).max(axis=-1)
    _, e2 = np.frexp(np.where(amax > 0, amax, 1.0))
    s = np.where(amax > 0, (e2 - 1) - E4M3_EMAX, -127)
    s = np.clip(s, -127, 127)
    p = e4m3_round(b / np.exp2(s)[..., None])
    codes = e4m3_encode(p).reshape(v.shape)
    return np.moveaxis(codes, -1, axis), np.moveaxis((s + 127).astype(np.uint8), -1, axis)


def mx_dequantize(codes, scales, axis: int = -1) -> np.ndarray:
    """Values of MXFP8 data: element value times its block's 2^(scale - 127)."""
    c = np.moveaxis(np.asarray(codes), axis, -1)
    sc = np.moveaxis(np.asarray(scales, dtype=np.int64), axis, -1)
    x = np.exp2(np.repeat(sc - 127, MX_BLOCK, axis=-1).astype(np.float64))
    return np.moveaxis(e4m3_decode(c) * x, -1, axis)


def mx_qdq(v, axis: int = -1) -> np.ndarray:
    """Quantise to MXFP8 along `axis` and return the represented values."""
    c, sc = mx_quantize(v, axis)
    return mx_dequantize(c, sc, axis)


# --------------------------------------------------------------------------
# [GLOSS] top-k gating
# --------------------------------------------------------------------------

def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Top-k expert ids per token ([GLOSS] top-k gating / switch routing).

    The k highest logits, ordered by (logit descending, expert index
    ascending): a stable sort of the negated logits puts equal values in
    index order.  k=1 is switch routing.  Returns int32 [T, k].
    """
    logits = np.asarray(logits)
    E = logits.shape[1]
    if not 1 <= k <= E:
        raise ValueError("k must be in [1, E]")
    order = np.argsort(-logits, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def gates(logits: np.ndarray, ids: np.ndarray, renorm: int = 1) -> np.ndarray:
    """Gate weight of each selected slot ([GLOSS]: weighted sum by score).

    renorm=1: softmax over the k selected logits.  renorm=0: the full softmax
    probability of the selected expert.  float64 [T, k].
    """
    l = np.asarray(logits, dtype=np.float64)
    sel = np.take_along_axis(l, ids.astype(np.int64), axis=1)
    if renorm:
        m = sel.max(axis=1, keepdims=True)
        e = np.exp(sel - m)
        return e / e.sum(axis=1, keepdims=True)
    m = l.max(axis=1, keepdims=True)
    z = np.exp(l - m).sum(axis=1, keepdims=True)
    return np.exp(sel - m) / z


# --------------------------------------------------------------------------
# [GLOSS] noise top-k gating; load balancing and its auxiliary loss;
# [CODA] metrics computed in epilogues
# --------------------------------------------------------------------------

def noisy_logits(logits, noise, noise_std: float) -> np.ndarray:
    """Logits with tunable Gaussian noise added before selection ([GLOSS]
    gating network: noise top-k).  `noise` holds standard-normal draws
    [T, E] supplied by the caller; `noise_std` scales them.  Selection,
    gates and the routing statistics all use the noisy logits.  float64.
    """
    return np.asarray(logits, dtype=np.float64) + float(noise_std) * np.asarray(noise, dtype=np.float64)


def router_probabilities(logits) -> np.ndarray:
    """The router's probability distribution over all E experts per token:
    softmax of the (post-scale, post-bias) logits.  float64 [T, E]."""
    l = np.asarray(logits, dtype=np.float64)
    m = l.max(axis=1, keepdims=True)
    e = np.exp(l - m)
    return e / e.sum(axis=1, keepdims=True)


def squared_cv(v) -> float:
    """Squared coefficient of variation across experts: population variance
    over the squared mean ([GLOSS] load balancing / auxiliary loss).  NaN
    when the mean is zero."""
    v = np.asarray(v, dtype=np.float64)
    mean = v.mean()
    if mean == 0:
        return float("nan")
    return float(((v - mean) ** 2).mean() / mean ** 2)


def router_stats(logits, ids, w, counts=None) -> dict:
    """Per-expert routing statistics and the load-balancing quantities.

    prob_sum[e] = sum over tokens of the router probability of e (full
    softmax); gate_sum[e] = sum over tokens of the gate weight given to e in
    the selected slots; aux = [CV^2(prob_sum), CV^2(gate_sum), CV^2(counts)]
    (the last NaN without counts).  The squared CV of the routing
    probability mass per expert is the auxiliary load loss the glossary
    names; the other two are the same statistic of the gates actually used
    and of the hard per-expert load.
    """
    l = np.asarray(logits, dtype=np.float64)
    T, E = l.shape
    prob_sum = router_probabilities(l).sum(axis=0)
    gate_sum = np.zeros(E, dtype=np.float64)
    ids = np.asarray(ids)
    w = np.asarray(w, dtype=np.float64)
    for t in range(T):
        for j in range(ids.shape[1]):
            gate_sum[ids[t, j]] += w[t, j]
    aux = [squared_cv(prob_sum), squared_cv(gate_sum),
           squared_cv(counts) if counts is not None else float("nan")]
    return {"prob_sum": prob_sum, "gate_sum": gate_sum, "aux": np.array(aux)}


# --------------------------------------------------------------------------
# dispatch: histogram, capacity rule, stable permutation
# --------------------------------------------------------------------------

def dispatch(ids: np.ndarray, E: int, cap: int, pad: int = 1) -> dict:
    """Expert-contiguous permutation of the (token, slot) assignments.

    counts[e]  number of slots choosing e ([GLOSS] capacity: the load before
               the rule is applied);
    rank(t,j)  number of earlier tokens that chose the same expert -- tokens
               keep their order inside an expert ([OMNI] 2.2 sorts tasks by
               token id within each expert group);
    kept[e]    min(counts[e], cap): slots with rank >= cap are dropped;
    offsets    exclusive prefix sum of kept, each rounded up to a multiple of
               pad (pad=128 is the block padding of the [VAREXP] BCSR path);
    pos(t,j)   offsets[e] + rank, or -1 when dropped;
    row_token  the token of every row, -1 for padding rows.

    The rank is taken from a stable sort of the flat slot list (token-major
    order); the tests pin it with an O(T^2) count.
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    order = np.argsort(flat, kind="stable")
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
    rank_sorted = np.arange(flat.size, dtype=np.int64) - starts[flat[order]]
    rank = np.empty(flat.size, dtype=np.int64)
    rank[order] = rank_sorted
    rank = rank.reshape(T, k)
    kept = np.minimum(counts, cap)
    padded = ((kept + pad - 1) // pad) * pad
    offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)
    keep = rank < cap
    pos = np.where(keep, offsets[ids] + rank, -1)
    rows = int(offsets[-1])
    row_token = np.full(rows, -1, dtype=np.int64)
    row_slot = np.full(rows, -1, dtype=np.int64)
    tt, jj = np.nonzero(keep)
    row_token[pos[tt, jj]] = tt
    row_slot[pos[tt, jj]] = jj
    return dict(counts=counts, kept=kept, offsets=offsets, rank=rank, pos=pos,
                row_token=row_token, row_slot=row_slot, rows=rows,
                dropped=int((~keep).sum()), max_load=int(counts.max() if E else 0))


# --------------------------------------------------------------------------
# [VAREXP] variable-size experts and the BCSR topology
# --------------------------------------------------------------------------

def expert_layout(expert_sizes, num_experts: int, block: int = 128,
                  default_size: int | None = None) -> dict:
    """Per-expert widths, column offsets and block buffers ([VAREXP] sec. 2).

    expert_sizes is the [(count, size), ...] spec; counts must sum to the
    number of experts; each size is rounded up to a multiple of the block.
    None means uniform experts of default_size.
    """
    if expert_sizes is None:
        if default_size is None:
            raise ValueError("uniform layout needs default_size")
        sizes = [default_size] * num_experts
    else:
        if sum(c for c, _ in expert_sizes) != num_experts:
            raise ValueError("sum of counts in expert_sizes must equal num_experts")
        sizes = []
        for count, size in expert_sizes:
            sizes.extend([((size + block - 1) // block) * block] * count)
    offsets = [0]
    for s in sizes:
        offsets.append(offsets[-1] + s)
    return dict(sizes=sizes, offsets=offsets, total=offsets[-1],
                size_blocks=[s // block for s in sizes],
                block_offsets=[o // block for o in offsets])


def bcsr_topology(offsets, size_blocks, block_offsets, block: int = 128) -> dict:
    """Block-sparse (BCSR) topology of the expert FFN ([VAREXP] sec. 3-4).

    Rows of the permuted activation come in blocks of `block`; expert e owns
    tb_e = (offsets[e+1]-offsets[e])/block token blocks (offsets padded to
    the block).  Every token block of expert e connects to the sb_e column
    blocks of e's slice of W1, whose first column block is block_offsets[e].
    Each expert writes its column indices at output_offsets[e], the exclusive
    prefix sum of tb_e*sb_e (the bug-fix section: never a uniform stride).
    row_offsets is the CSR row pointer over token blocks.
    """
    offsets = [int(o) for o in offsets]
    E = len(offsets) - 1
    tb = []
    for e in range(E):
        n = offsets[e + 1] - offsets[e]
        if n % block:
            raise ValueError("offsets must be padded to the block size")
        tb.append(n // block)
    out_off = [0]
    for e in range(E):
        out_off.append(out_off[-1] + tb[e] * int(size_blocks[e]))
    nnz = out_off[-1]
    column_indices = [0] * nnz
    row_offsets = [0]
    for e in range(E):
        for y in range(tb[e]):
            for c in range(int(size_blocks[e])):
                column_indices[out_off[e] + y * int(size_blocks[e]) + c] = int(block_offsets[e]) + c
            row_offsets.append(row_offsets[-1] + int(size_blocks[e]))
    return dict(token_blocks=tb, output_offsets=out_off[:-1], nnz=nnz,
                row_offsets=np.array(row_offsets, dtype=np.int64),
                column_indices=np.array(column_indices, dtype=np.int64),
                block_rows=len(row_offsets) - 1)


# --------------------------------------------------------------------------
# activations and FFNs
# --------------------------------------------------------------------------

def _float(z) -> np.ndarray:
    """z as a float array: float32 stays float32 (the float32 work
    precision), everything else becomes float64."""
    z = np.asarray(z)
    return z if z.dtype == np.float32 else z.astype(np.float64)


def gelu(z):
    """Exact GELU: z * Phi(z) = z/2 * (1 + erf(z/sqrt 2))."""
    z = _float(z)
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def gelu_tanh(z):
    """tanh approximation of GELU."""
    z = _float(z)
    return 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def silu(z):
    z = _float(z)
    return z / (1.0 + np.exp(-z))


def _act(name):
    return {"gelu": gelu, "gelu_tanh": gelu_tanh}[name]


def ffn(xhat, r, w1, w2, act: str, w3=None, faithful: bool = False):
    """One expert FFN on r-scaled rows ([GLOSS] experts; [CODA] epilogue).

    GELU form:   act(r * (xhat @ w1)) @ w2
    SwiGLU form: (silu(r * (xhat @ w1)) * (r * (xhat @ w3))) @ w2
    With faithful=True the hidden activation is rounded to bf16, the storage
    point of the bf16 path.
    """
    xhat = np.asarray(xhat, dtype=_wd())
    r = np.asarray(r, dtype=_wd())[:, None]
    a = r * (xhat @ w1)
    if act == "swiglu":
        h = silu(a) * (r * (xhat @ w3))
    else:
        h = _act(act)(a)
    if faithful:
        h = bf16_to_f64(f64_to_bf16_bits(h))
    return h @ w2


def ffn_mxfp8(xhat, r, w1, w2, act: str, w3=None):
    """One expert FFN with MXFP8 operands ([CODA]: low-precision conversions
    at the epilogues).  The activation rows are quantised along d before the
    first linear and the weights along their K dimension (w1 / w3 per column
    along d, w2 per column along f); r multiplies the first linear's
    accumulator as in the bf16 path; the hidden activation is quantised along
    f (blocks of 32 features) before the second linear.
    """
    xq = mx_qdq(np.asarray(xhat, dtype=np.float64), axis=1)
    r = np.asarray(r, dtype=np.float64)[:, None]
    a = r * (xq @ mx_qdq(w1, axis=0))
    if act == "swiglu":
        h = silu(a) * (r * (xq @ mx_qdq(w3, axis=0)))
    else:
        h = _act(act)(a)
    return mx_qdq(h, axis=1) @ mx_qdq(w2, axis=0)


def grouped_expert_ffn(xhat_rows, r_rows, e_of_row, w1, w2, f_offsets, act,
                       w3=None, faithful=False, quant=None):
    """Per-row expert FFN output for rows that each name their expert.

    w1, w3 are [d, sum f] and w2 is [sum f, d]; expert e owns columns
    f_offsets[e]:f_offsets[e+1] of w1/w3 and the same rows of w2 ([VAREXP]
    sec. 2, weight allocation).  Weights may be bf16 bit patterns; only the
    slices of experts that have rows are widened to float64.
    """
    d = np.asarray(w2).shape[1]
    out = np.zeros((len(e_of_row), d), dtype=_wd())
    for e in np.unique(e_of_row):
        m = e_of_row == e
        lo, hi = int(f_offsets[e]), int(f_offsets[e + 1])
        w3e = None if w3 is None else _aw(np.asarray(w3)[:, lo:hi])
        if quant == "mxfp8":
            out[m] = ffn_mxfp8(xhat_rows[m], r_rows[m], _aw(np.asarray(w1)[:, lo:hi]),
                               _aw(np.asarray(w2)[lo:hi, :]), act, w3e)
        else:
            out[m] = ffn(xhat_rows[m], r_rows[m], _aw(np.asarray(w1)[:, lo:hi]),
                         _aw(np.asarray(w2)[lo:hi, :]), act, w3e, faithful)
    return out


def bcsr_expert_ffn(x_perm, row_r, topo, w1, w2, act, block=128, w3=None):
    """The expert FFN walked block by block over the BCSR topology.

    SDD: for each nonzero block (token block rb, column block cb),
    h[rb, cb] = act(r * x_perm[rb] @ w1[:, cb]).  DSD: y[rb] = sum over the
    row's nonzero blocks of h[rb, cb] @ w2[cb, :].  ([VAREXP]: the sparse
    products run over the topology; the topology is the only change.)
    Returns y (no gate) for every permuted row.
    """
    x_perm = np.asarray(x_perm, dtype=np.float64)
    row_r = np.asarray(row_r, dtype=np.float64)
    R, d = x_perm.shape
    y = np.zeros((R, w2.shape[1]), dtype=np.float64)
    ro, ci = topo["row_offsets"], topo["column_indices"]
    for rb in range(topo["block_rows"]):
        rows = slice(rb * block, (rb + 1) * block)
        xr = x_perm[rows]
        rr = row_r[rows][:, None]
        for idx in range(int(ro[rb]), int(ro[rb + 1])):
            cols = slice(int(ci[idx]) * block, (int(ci[idx]) + 1) * block)
            a = rr * (xr @ w1[:, cols])
            if act == "swiglu":
                hb = silu(a) * (rr * (xr @ w3[:, cols]))
            else:
                hb = _act(act)(a)
            y[rows] += hb @ w2[cols, :]
    return y


# --------------------------------------------------------------------------
# [OMNI] Cartesian-product router and atomic experts
# --------------------------------------------------------------------------

def cartesian_scores(x, gamma, r, k_rows, k_cols):
    """Row and column scores of the [OMNI] 2.2 Cartesian router.

    s1 = r * (xhat @ K_r) over the Nr row keys, s2 = r * (xhat @ K_c) over
    the Nc column keys; expert n = i*Nc + j scores s1[i] + s2[j].
    """
    xh = _xhat(x, gamma)
    r = np.asarray(r, dtype=_wd())[:, None]
    return r * (xh @ _aw(k_rows)), r * (xh @ _aw(k_cols))


def _topk_lex(v: np.ndarray, k: int) -> np.ndarray:
    return np.argsort(-v, kind="stable")[:k]


def cartesian_topk(s1, s2, k: int):
    """Top-k over the Nr x Nc grid in two stages.

    The best k rows of s1 and the best k columns of s2 give k*k candidate
    pairs; the answer is the top k of those by (score desc, n asc).  This
    equals the top k of the whole grid (a pair with a row outside the row
    top-k is beaten by k pairs in the same column), except where rounding of
    the sum creates a tie that reorders; the tests check it against the
    brute force.  Scores are summed in the precision of the inputs, so the
    oracle takes the same decision as a float32 kernel given float32 scores.
    Returns (ids int64 [T,k], scores [T,k]).
    """
    s1 = np.asarray(s1)
    s2 = np.asarray(s2)
    T, Nr = s1.shape
    Nc = s2.shape[1]
    ids = np.empty((T, k), dtype=np.int64)
    sc = np.empty((T, k), dtype=s1.dtype)
    for t in range(T):
        I = _topk_lex(s1[t], k)
        J = _topk_lex(s2[t], k)
        cand_n = (I[:, None] * Nc + J[None, :]).reshape(-1)
        cand_s = (s1[t][I][:, None] + s2[t][J][None, :]).reshape(-1)
        # lexicographic (score desc, n asc)
        order = np.lexsort((cand_n, -cand_s))[:k]
        ids[t] = cand_n[order]
        sc[t] = cand_s[order]
    return ids, sc


def cartesian_topk_bruteforce(s1, s2, k: int):
    """Top-k of all Nr*Nc scores (definition; for small token subsets)."""
    s1 = np.asarray(s1)
    s2 = np.asarray(s2)
    T = s1.shape[0]
    ids = np.empty((T, k), dtype=np.int64)
    sc = np.empty((T, k), dtype=s1.dtype)
    for t in range(T):
        full = (s1[t][:, None] + s2[t][None, :]).reshape(-1)
        order = _topk_lex(full, k)
        ids[t] = order
        sc[t] = full[order]
    return ids, sc


def atomic_experts_token_centric(xhat, r, ids, g, W, V, act="gelu"):
    """Routed branch of [OMNI] 2.1, token by token (dynamic expert assembly).

    For token t, its k atomic experts' rows W[n], V[n] are gathered into a
    token-specific block; routed[t] = sum_j g[t,j] * act(r_t * xhat_t.W[n_j]) * V[n_j].
    Only the gathered rows are widened (to the work precision).
    """
    xhat = np.asarray(xhat, dtype=_wd())
    r = np.asarray(r, dtype=_wd())
    T = xhat.shape[0]
    out = np.zeros((T, np.asarray(V).shape[1]), dtype=_wd())
    f = _act(act)
    for t in range(T):
        Wt = _aw(np.asarray(W)[ids[t]])      # [k, d] assembled block
        Vt = _aw(np.asarray(V)[ids[t]])
        a = np.asarray(g[t], dtype=_wd()) * f(r[t] * (Wt @ xhat[t]))
        out[t] = a @ Vt
    return out


def atomic_experts_expert_centric(xhat, r, ids, g, W, V, act="gelu"):
    """The same branch in the [OMNI] 2.2 expert-centric order.

    All (token, expert) tasks form one flat list, grouped by expert id and
    sorted by token id within each group; each expert's rows are used for
    all of its tasks before moving on.  Sums are collected per token.
    """
    xhat = np.asarray(xhat, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    W = as_f64(W) if not (isinstance(W, np.ndarray) and W.dtype == np.float64) else W
    V = as_f64(V) if not (isinstance(V, np.ndarray) and V.dtype == np.float64) else V
    T, k = ids.shape
    tok = np.repeat(np.arange(T), k)
    exp_ = np.asarray(ids, dtype=np.int64).reshape(-1)
    gg = np.asarray(g, dtype=np.float64).reshape(-1)
    order = np.lexsort((tok, exp_))            # by expert, then token
    out = np.zeros((T, V.shape[1]), dtype=np.float64)
    f = _act(act)
    i = 0
    n_tasks = len(order)
    while i < n_tasks:
        n = exp_[order[i]]
        j = i
        while j < n_tasks and exp_[order[j]] == n:
            j += 1
        ts = tok[order[i:j]]
        a = gg[order[i:j]] * f(r[ts] * (xhat[ts] @ W[n]))
        for t_, a_ in zip(ts, a):
            out[t_] += a_ * V[n]
        i = j
    return out


# --------------------------------------------------------------------------
# combine and the whole layer
# --------------------------------------------------------------------------

def combine(x, shared, slot_out, pos, residual=True):
    """out[t] = x[t] + shared[t] + sum over kept slots of the gated expert output.

    slot_out[t, j] holds g * FFN(x_t) for slot j; dropped slots (pos < 0)
    contribute nothing, so a token with every slot dropped returns x (or 0
    without the residual) -- [GLOSS] capacity: dropped tokens pass through.
    """
    x = _aw(x)
    T, d = x.shape
    out = x.copy() if residual else np.zeros_like(x)
    if shared is not None:
        out = out + shared
    keep = np.asarray(pos) >= 0
    for j in range(keep.shape[1]):
        out = out + np.where(keep[:, j:j + 1], slot_out[:, j, :], 0.0)
    return out


def _shared_ffn(xh, r, p, faithful):
    act = p.get("shared_act", "swiglu" if p.get("ws3") is not None else "gelu")
    return ffn(xh, r, _aw(p["ws1"]), _aw(p["ws2"]), act,
               _aw(p.get("ws3")), faithful)


def layer_forward(p: dict, x, ids_override=None, tokens=None, faithful=False) -> dict:
    """The whole MoE FFN layer forward (the pass the four pages describe).

    p holds: k, eps, renorm, cf, act, gamma, residual, and either
      router 'dense': w_router [d,E], bias [E] or None, expert weights
        w1 [d,sum f], w3 (SwiGLU) and w2 [sum f,d], f_offsets [E+1]
      router 'cartesian': k_rows [d,Nr], k_cols [d,Nc], atomic W, V [N,d]
    plus optional shared-expert weights ws1, ws3, ws2 (always active, gate 1),
    and quant='mxfp8' for routed experts with MXFP8 operands (ffn_mxfp8).

    ids_override replaces the selected ids (the stage-wise protocol: compare
    downstream stages on the GPU's own routing).  tokens restricts the FFN
    and combine to a subset of tokens (routing and ranks still use all T).
    faithful=True rounds h, the gated expert outputs, the shared output and
    the layer output to bf16 at the storage points of the bf16 path.
    """
    x64 = _aw(x)
    T, d = x64.shape
    k = int(p["k"])
    eps = float(p["eps"])
    gamma = p.get("gamma")
    r = rmsnorm_scale(x64, eps)
    xh = _xhat(x64, gamma)
    res = dict(r=r)
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    rnd = (lambda a: bf16_to_f64(f64_to_bf16_bits(a))) if faithful else (lambda a: a)

    if p.get("router", "dense") == "cartesian":
        s1, s2 = cartesian_scores(x64, gamma, r, p["k_rows"], p["k_cols"])
        res["s1"], res["s2"] = s1, s2
        if ids_override is None:
            ids, sc = cartesian_topk(s1, s2, k)
        else:
            ids = np.asarray(ids_override, dtype=np.int64)
            Nc = s2.shape[1]
            sc = np.take_along_axis(s1, ids // Nc, axis=1) + np.take_along_axis(s2, ids % Nc, axis=1)
        m = sc.max(axis=1, keepdims=True)
        ee = np.exp(sc - m)
        g = ee / ee.sum(axis=1, keepdims=True)
        res.update(ids=ids, w=g)
        routed = atomic_experts_token_centric(xh[tok], r[tok], ids[tok], g[tok],
                                              p["W"], p["V"], p.get("act", "gelu"))
        shared = _shared_ffn(xh[tok], r[tok], p, faithful) if p.get("ws1") is not None else None
        if shared is not None:
            shared = rnd(shared)
        routed = rnd(routed)
        out = x64[tok].copy() if p.get("residual", True) else np.zeros((len(tok), d))
        if shared is not None:
            out = out + shared
        out = out + routed
        res.update(routed=routed, shared=shared, out=rnd(out), tokens=tok)
        return res

    logits = router_logits(x64, gamma, r, p["w_router"], p.get("bias"))
    E = logits.shape[1]
    ids = select_topk(logits, k) if ids_override is None else np.asarray(ids_override)
    g = gates(logits, ids, int(p.get("renorm", 1)))
    cap = capacity(T, k, E, float(p.get("cf", 0.0)))
    disp = dispatch(ids, E, cap, int(p.get("pad", 1)))
    res.update(logits=logits, ids=ids.astype(np.int32), w=g, capacity=cap, **disp)

    w1, w2, w3 = p["w1"], p["w2"], p.get("w3")
    foff = np.asarray(p["f_offsets"], dtype=np.int64)
    act = p["act"]
    pos = disp["pos"][tok]
    slot_out = np.zeros((len(tok), k, d), dtype=_wd())
    tt, jj = np.nonzero(pos >= 0)
    if len(tt):
        e_rows = np.asarray(ids)[tok[tt], jj].astype(np.int64)
        y = grouped_expert_ffn(xh[tok[tt]], r[tok[tt]], e_rows, w1, w2, foff, act, w3, faithful,
                               quant=p.get("quant"))
        slot_out[tt, jj] = rnd(g[tok[tt], jj][:, None] * y)
    shared = _shared_ffn(xh[tok], r[tok], p, faithful) if p.get("ws1") is not None else None
    if shared is not None:
        shared = rnd(shared)
    out = combine(x64[tok], shared, slot_out, pos, p.get("residual", True))
    res.update(slot_out=slot_out, shared=shared, out=rnd(out), tokens=tok)
    return res


# --------------------------------------------------------------------------
# The backward pass ([CODA]: the RMSNorm backward is fused into the backward
# of the linear that consumed the normed input, and needs the saved r;
# [VAREXP] validation list: forward / backward and gradient checks)
# --------------------------------------------------------------------------

def gelu_grad(z):
    """d/dz of the exact GELU: Phi(z) + z * phi(z)."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * (1.0 + erf(z / math.sqrt(2.0))) + z * np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def gelu_tanh_grad(z):
    """d/dz of the tanh form: with u = c (z + 0.044715 z^3),
    0.5 (1 + tanh u) + 0.5 z (1 - tanh^2 u) c (1 + 3 * 0.044715 z^2)."""
    z = np.asarray(z, dtype=np.float64)
    c = math.sqrt(2.0 / math.pi)
    t = np.tanh(c * (z + 0.044715 * z ** 3))
    return 0.5 * (1.0 + t) + 0.5 * z * (1.0 - t * t) * c * (1.0 + 3.0 * 0.044715 * z * z)


def silu_grad(z):
    """d/dz of z * sigmoid(z): sigmoid(z) (1 + z (1 - sigmoid(z)))."""
    z = np.asarray(z, dtype=np.float64)
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def ffn_backward(xhat, r, w1, w2, act: str, dy, w3=None) -> dict:
    """Gradients of the rows' FFN outputs y = ffn(xhat, r, ...) for the
    upstream gradient dy of y: with a = r (xhat w1) (and u = r (xhat w3)),
    h = act(a) (or silu(a) u), y = h w2:
      dw2 = h^T dy,  dh = dy w2^T,
      da = dh act'(a)  (SwiGLU: da = dh u silu'(a), du = dh silu(a)),
      dw1 = (r xhat)^T da  (dw3 = (r xhat)^T du),
      dxhat = r (da w1^T + du w3^T),
      dr = sum over units of (xhat w1) da + (xhat w3) du.
    """
    xhat = np.asarray(xhat, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)[:, None]
    dy = np.asarray(dy, dtype=np.float64)
    z1 = xhat @ w1
    a = r * z1
    out = {}
    if act == "swiglu":
        z3 = xhat @ w3
        u = r * z3
        h = silu(a) * u
    else:
        h = _act(act)(a)
    out["dw2"] = h.T @ dy
    dh = dy @ w2.T
    rx = r * xhat
    if act == "swiglu":
        da = dh * u * silu_grad(a)
        du = dh * silu(a)
        out["dw3"] = rx.T @ du
        out["dxhat"] = r * (da @ w1.T + du @ w3.T)
        out["dr"] = np.sum(z1 * da + z3 * du, axis=1)
    else:
        grad = {"gelu": gelu_grad, "gelu_tanh": gelu_tanh_grad}[act]
        da = dh * grad(a)
        out["dxhat"] = r * (da @ w1.T)
        out["dr"] = np.sum(z1 * da, axis=1)
    out["dw1"] = rx.T @ da
    return out


def gates_backward(logits, ids, renorm: int, dg) -> np.ndarray:
    """Gradient of the router logits from the gradient of the gates (the
    selection itself is piecewise constant).  renorm=1, g = softmax of the k
    selected logits: dl[sel_j] = g_j (dg_j - sum_i g_i dg_i).  renorm=0,
    g_j = P[sel_j] with P the full softmax:
    dl[e] = P[e] (sum over j with sel_j = e of dg_j - sum_j P[sel_j] dg_j)."""
    l = np.asarray(logits, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    dg = np.asarray(dg, dtype=np.float64)
    T, E = l.shape
    dl = np.zeros((T, E))
    g = gates(l, ids, renorm)
    rows = np.arange(T)[:, None]
    if renorm:
        s = np.sum(g * dg, axis=1, keepdims=True)
        np.add.at(dl, (np.broadcast_to(rows, ids.shape), ids), g * (dg - s))
    else:
        m = l.max(axis=1, keepdims=True)
        P = np.exp(l - m)
        P /= P.sum(axis=1, keepdims=True)
        s = np.sum(g * dg, axis=1, keepdims=True)
        np.add.at(dl, (np.broadcast_to(rows, ids.shape), ids), dg)
        dl = P * (dl - s)
    return dl


def layer_backward(p: dict, x, dout, ids_override=None, tokens=None) -> dict:
    """Gradients of layer_forward's output for the upstream gradient dout
    (dense router, routed grouped experts, shared experts).

    Returns dx, dgamma (with a gain), dw_router [d, E], dbias [E], dw1,
    dw3, dw2 (routed, the pages' layouts), dws1, dws3, dws2 (shared) and the
    intermediate dg [T, k] (gates), dl [T, E] (logits), dxhat, dr.
    The chain: dropped slots get no gradient; top-k selection and the
    capacity rule are piecewise constant; the router logit is
    l = r (xhat w_router) + b; the RMSNorm backward uses the saved r:
    with xhat = x gamma and r = (mean x^2 + eps)^-1/2,
    dx = dout + gamma dxhat - (r^3 / d) dr x  and  dgamma = sum_t dxhat x.

    tokens (optional) restricts the computation to those tokens' own
    gradients: dx, dxhat, dr, dg and dl of the tokens (in that order); the
    weight gradients, which sum over every token, are then not returned.
    The routing (selection, capacity, positions) still covers all tokens.
    """
    if p.get("router", "dense") != "dense":
        raise NotImplementedError("the backward covers the dense router")
    if p.get("quant"):
        raise NotImplementedError("the backward covers unquantised experts")
    x64 = as_f64(x)
    G = as_f64(dout)
    T, d = x64.shape
    k = int(p["k"])
    eps = float(p["eps"])
    gamma = as_f64(p.get("gamma"))
    r = rmsnorm_scale(x64, eps)
    xh = _xhat(x64, p.get("gamma"))
    wr = as_f64(p["w_router"])
    bias = p.get("bias")
    logits = router_logits(x64, p.get("gamma"), r, wr, bias)
    E = logits.shape[1]
    ids = select_topk(logits, k) if ids_override is None else np.asarray(ids_override)
    renorm = int(p.get("renorm", 1))
    g = gates(logits, ids, renorm)
    cap = capacity(T, k, E, float(p.get("cf", 0.0)))
    pos = dispatch(ids, E, cap, int(p.get("pad", 1)))["pos"]

    act = p["act"]
    # weights stay in their stored form; each expert's slices are widened
    # to float64 when used
    w1, w2, w3 = np.asarray(p["w1"]), np.asarray(p["w2"]), p.get("w3")
    w3 = None if w3 is None else np.asarray(w3)
    foff = np.asarray(p["f_offsets"], dtype=np.int64)
    dxh = np.zeros((T, d))
    dr = np.zeros(T)
    dg = np.zeros((T, k))
    sub = tokens is not None
    res = {} if sub else dict(dw1=np.zeros(w1.shape), dw2=np.zeros(w2.shape),
                              dw3=None if w3 is None else np.zeros(w3.shape))
    tok = np.arange(T) if not sub else np.asarray(tokens, dtype=np.int64)
    keep = np.zeros(T, dtype=bool)
    keep[tok] = True
    tt, jj = np.nonzero((pos >= 0) & keep[:, None])
    e_rows = np.asarray(ids)[tt, jj].astype(np.int64)
    for e in np.unique(e_rows):
        m = e_rows == e
        ts, js = tt[m], jj[m]
        lo, hi = int(foff[e]), int(foff[e + 1])
        w1e, w2e = as_f64(w1[:, lo:hi]), as_f64(w2[lo:hi, :])
        w3e = None if w3 is None else as_f64(w3[:, lo:hi])
        y = ffn(xh[ts], r[ts], w1e, w2e, act, w3e)
        dg[ts, js] = np.sum(G[ts] * y, axis=1)
        b = ffn_backward(xh[ts], r[ts], w1e, w2e, act, g[ts, js][:, None] * G[ts], w3e)
        np.add.at(dxh, ts, b["dxhat"])
        np.add.at(dr, ts, b["dr"])
        if not sub:
            res["dw1"][:, lo:hi] += b["dw1"]
            res["dw2"][lo:hi, :] += b["dw2"]
            if w3 is not None:
                res["dw3"][:, lo:hi] += b["dw3"]
    if p.get("ws1") is not None:
        sact = p.get("shared_act", "swiglu" if p.get("ws3") is not None else "gelu")
        b = ffn_backward(xh[tok], r[tok], as_f64(p["ws1"]), as_f64(p["ws2"]), sact, G[tok],
                         as_f64(p.get("ws3")))
        dxh[tok] += b["dxhat"]
        dr[tok] += b["dr"]
        res.update(dws1=b["dw1"], dws2=b["dw2"], dws3=b.get("dw3"))
    dl = np.zeros((T, E))
    dl[tok] = gates_backward(logits[tok], np.asarray(ids)[tok], renorm, dg[tok])
    z = xh[tok] @ wr
    res["dw_router"] = (r[:, None] * xh).T @ dl
    res["dbias"] = dl.sum(axis=0)
    dxh[tok] += r[tok, None] * (dl[tok] @ wr.T)
    dr[tok] += np.sum(z * dl[tok], axis=1)
    dx = G.copy() if p.get("residual", True) else np.zeros_like(G)
    dx += (dxh * gamma if gamma is not None else dxh) - (r ** 3 / d)[:, None] * dr[:, None] * x64
    res.update(dx=dx[tok], dgamma=None if gamma is None else np.sum(dxh * x64, axis=0),
               dg=dg[tok], dl=dl[tok], dxhat=dxh[tok], dr=dr[tok],
               ids=np.asarray(ids, dtype=np.int32), pos=pos, tokens=tok)
    if sub:
        for key in ("dw1", "dw2", "dw3", "dws1", "dws2", "dws3", "dw_router", "dbias", "dgamma"):
            res.pop(key, None)
    return res


def expert_unit_grads(p: dict, x, dout, ids, e: int, units) -> dict:
    """Weight gradients of routed expert e restricted to some of its hidden
    units: dw1[:, units], dw3[:, units], dw2[units, :] summed over all of the
    expert's kept rows.  The FFN is separable over hidden units (each unit's
    pre-activation, activation and down-projection row involve only that
    unit), so this is the same computation as layer_backward on the units'
    slices of the weights."""
    x64 = as_f64(x)
    G = as_f64(dout)
    T, d = x64.shape
    k = int(p["k"])
    r = rmsnorm_scale(x64, float(p["eps"]))
    xh = _xhat(x64, p.get("gamma"))
    logits = router_logits(x64, p.get("gamma"), r, as_f64(p["w_router"]), p.get("bias"))
    E = logits.shape[1]
    ids = np.asarray(ids)
    g = gates(logits, ids, int(p.get("renorm", 1)))
    cap = capacity(T, k, E, float(p.get("cf", 0.0)))
    pos = dispatch(ids, E, cap, int(p.get("pad", 1)))["pos"]
    foff = np.asarray(p["f_offsets"], dtype=np.int64)
    cols = int(foff[e]) + np.asarray(units, dtype=np.int64)
    tt, jj = np.nonzero((pos >= 0) & (ids == e))
    w1e = as_f64(np.asarray(p["w1"])[:, cols])
    w2e = as_f64(np.asarray(p["w2"])[cols, :])
    w3e = None if p.get("w3") is None else as_f64(np.asarray(p["w3"])[:, cols])
    b = ffn_backward(xh[tt], r[tt], w1e, w2e, p["act"], g[tt, jj][:, None] * G[tt], w3e)
    return dict(dw1=b["dw1"], dw2=b["dw2"], dw3=b.get("dw3"))
