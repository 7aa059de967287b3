"""ctypes binding of libmoe_mi355x.so (argument marshalling only).

Every step of the layer runs in the HIP kernels behind the C ABI declared in
include/moe.h.  PyTorch provides device memory and the current stream; this
module turns tensors into pointers, fills the C descriptors and raises on a
non-zero return code with the library's own message.  There is no other
code path: if the shared library is missing, every call raises.
"""
from __future__ import annotations

import ctypes as C
from pathlib import Path

LIB_PATH = Path(__file__).resolve().with_name("libmoe_mi355x.so")

MOE_F32, MOE_BF16 = 0, 1
ACT = {"gelu": 0, "gelu_tanh": 1, "swiglu": 2}
ROUTER_DENSE, ROUTER_CARTESIAN = 0, 1
EXPERTS_GROUPED, EXPERTS_BCSR, EXPERTS_ATOMIC = 0, 1, 2
QUANT_NONE, QUANT_MXFP8 = 0, 1
STAGES = ["router", "dispatch", "plan", "gemm1", "gemm2", "shared", "combine"]

EXPORTED = [
    "moe_last_error", "moe_version", "moe_capacity", "moe_rows_max", "moe_pack_transpose",
    "moe_pack_swiglu", "moe_pack_mxfp8", "moe_pack_mxfp8_weights", "moe_rmsnorm_stats", "moe_router_workspace_size", "moe_router_topk",
    "moe_router_topk_ex",
    "moe_dispatch_workspace_size", "moe_dispatch", "moe_topology_nnz_max", "moe_build_topology",
    "moe_expert_workspace_size", "moe_expert_gemm", "moe_shared_workspace_size", "moe_shared_ffn",
    "moe_combine", "moe_layer_workspace_size", "moe_layer_forward", "moe_layer_routing",
    "moe_timer_create", "moe_timer_destroy", "moe_timer_reset", "moe_timer_stage_ms",
    "moe_layer_backward_workspace_size", "moe_layer_backward", "moe_dispatch_noalloc",
]
# size of the static scratch behind moe_dispatch_noalloc (MOE_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 8 << 20


class RouterDesc(C.Structure):
    _fields_ = [("kind", C.c_int), ("E", C.c_int64), ("wr_t", C.c_void_p), ("bias", C.c_void_p),
                ("Nr", C.c_int64), ("Nc", C.c_int64), ("keys_t", C.c_void_p)]


class ExpertsDesc(C.Structure):
    _fields_ = [("kind", C.c_int), ("act", C.c_int), ("E", C.c_int64),
                ("ffn_sizes", C.POINTER(C.c_int64)), ("ffn_offsets", C.c_void_p),
                ("w13_t", C.c_void_p), ("w2_t", C.c_void_p), ("w2_ld", C.c_int64),
                ("W", C.c_void_p), ("V", C.c_void_p),
                ("block", C.c_int), ("size_blocks", C.c_void_p), ("block_offsets", C.c_void_p),
                ("row_offsets", C.c_void_p), ("column_indices", C.c_void_p),
                ("quant", C.c_int), ("w13_scale", C.c_void_p), ("w2_scale", C.c_void_p),
                ("w2_fk", C.c_void_p), ("w13_dk", C.c_void_p)]


class Routing(C.Structure):
    _fields_ = [("T", C.c_int64), ("k", C.c_int), ("E", C.c_int64), ("rows_max", C.c_int64),
                ("pad", C.c_int), ("ids", C.c_void_p), ("w", C.c_void_p), ("r", C.c_void_p),
                ("counts", C.c_void_p), ("offsets", C.c_void_p), ("pos", C.c_void_p),
                ("row_token", C.c_void_p), ("row_r", C.c_void_p), ("row_w", C.c_void_p),
                ("row_expert", C.c_void_p)]


class RouterExtras(C.Structure):
    _fields_ = [("noise", C.c_void_p), ("noise_std", C.c_float), ("prob_sum", C.c_void_p),
                ("gate_sum", C.c_void_p), ("aux", C.c_void_p)]


class LayerDesc(C.Structure):
    _fields_ = [("d", C.c_int64), ("dtype", C.c_int), ("gamma", C.c_void_p), ("eps", C.c_float),
                ("router", RouterDesc), ("k", C.c_int), ("renorm", C.c_int),
                ("capacity_factor", C.c_double), ("experts", ExpertsDesc),
                ("shared", C.POINTER(ExpertsDesc)), ("residual", C.c_int), ("timer", C.c_void_p),
                ("router_extras", C.POINTER(RouterExtras)), ("save_for_backward", C.c_int)]


class LayerGrads(C.Structure):
    _fields_ = [("dx", C.c_void_p), ("dgamma", C.c_void_p), ("dw_router", C.c_void_p),
                ("dbias", C.c_void_p), ("dw13", C.c_void_p), ("dw2", C.c_void_p),
                ("dws13", C.c_void_p), ("dws2", C.c_void_p)]


class Stats(C.Structure):
    _fields_ = [("rows", C.c_int32), ("dropped", C.c_int32), ("max_load", C.c_int32),
                ("errors", C.c_int32)]


_LIB = None


def lib() -> C.CDLL:
    """Load the shared library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH.name} is not built: run __graft_entry__.build() "
                               "(hipcc for gfx950) first")
        L = C.CDLL(str(LIB_PATH))
        P, I, I64, SZ, F, D = C.c_void_p, C.c_int, C.c_int64, C.c_size_t, C.c_float, C.c_double
        sig = {
            "moe_last_error": (C.c_char_p, []),
            "moe_version": (C.c_char_p, []),
            "moe_capacity": (I64, [I64, I, I64, D]),
            "moe_rows_max": (I64, [I64, I, I64, I64, I]),
            "moe_pack_transpose": (I, [P, I, I64, I64, P, P]),
            "moe_pack_swiglu": (I, [P, P, I, I64, C.POINTER(I64), I64, P, P]),
            "moe_pack_mxfp8": (I, [P, I64, I64, I64, P, I64, P, I64, P]),
            "moe_pack_mxfp8_weights": (I, [P, I64, I64, I64, P, I64, P, P]),
            "moe_rmsnorm_stats": (I, [P, I, I64, I64, P, F, P, P, P]),
            "moe_router_workspace_size": (SZ, [C.POINTER(RouterDesc), I64]),
            "moe_router_topk": (I, [C.POINTER(RouterDesc), P, I, I64, I64, P, F, P, I, I, P, P, P,
                                    P, SZ, P]),
            "moe_router_topk_ex": (I, [C.POINTER(RouterDesc), P, I, I64, I64, P, F, P, I, I, P, P,
                                       P, C.POINTER(RouterExtras), P, SZ, P]),
            "moe_dispatch_workspace_size": (SZ, [I64, I, I64]),
            "moe_dispatch": (I, [P, P, P, P, I, I64, I64, I64, I, I64, I, I64, P, P, P, P, P, P, P,
                                 P, P, P, SZ, P]),
            "moe_dispatch_noalloc": (I, [P, P, P, P, I, I64, I64, I64, I, I64, I, I64, P, P, P, P,
                                         P, P, P, P, P, P]),
            "moe_topology_nnz_max": (I64, [I64, I, C.POINTER(I64), I64]),
            "moe_build_topology": (I, [P, P, P, I64, I, I64, P, P, P, P]),
            "moe_expert_workspace_size": (SZ, [C.POINTER(ExpertsDesc), I, I64, I64, I, I64]),
            "moe_expert_gemm": (I, [C.POINTER(ExpertsDesc), I, I64, C.POINTER(Routing), P, P, P,
                                    P, SZ, P]),
            "moe_shared_workspace_size": (SZ, [C.POINTER(ExpertsDesc), I, I64, I64]),
            "moe_shared_ffn": (I, [C.POINTER(ExpertsDesc), I, I64, I64, P, P, P, P, SZ, P]),
            "moe_combine": (I, [P, P, P, P, I, I64, I64, I, P, P]),
            "moe_layer_workspace_size": (SZ, [C.POINTER(LayerDesc), I64]),
            "moe_layer_forward": (I, [C.POINTER(LayerDesc), P, I64, P, P, P, SZ, P]),
            "moe_layer_routing": (I, [C.POINTER(LayerDesc), I64, P, SZ, C.POINTER(Routing)]),
            "moe_layer_backward_workspace_size": (SZ, [C.POINTER(LayerDesc), I64]),
            "moe_layer_backward": (I, [C.POINTER(LayerDesc), P, I64, P, P, SZ,
                                       C.POINTER(LayerGrads), P, SZ, P]),
            "moe_timer_create": (I, [C.POINTER(P), I]),
            "moe_timer_destroy": (I, [P]),
            "moe_timer_reset": (I, [P]),
            "moe_timer_stage_ms": (I, [P, I, C.POINTER(D), C.POINTER(I)]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"moe error {code}: {msg}")
        self.code = code


def check(rc: int) -> None:
    if rc != 0:
        raise MoeError(rc, lib().moe_last_error().decode())


def last_error() -> str:
    return lib().moe_last_error().decode()


# ---------------------------------------------------------------- tensor helpers

def ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def stream_handle(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def i64_array(vals):
    arr = (C.c_int64 * len(vals))(*[int(v) for v in vals])
    return arr


# ---------------------------------------------------------------- host functions

def capacity(T: int, k: int, E: int, cf: float) -> int:
    return int(lib().moe_capacity(T, k, E, float(cf)))


def rows_max(T: int, k: int, E: int, cap: int, pad: int) -> int:
    return int(lib().moe_rows_max(T, k, E, cap, pad))


def version() -> str:
    return lib().moe_version().decode()


# ---------------------------------------------------------------- stage calls

def pack_transpose(src, dst, stream=None) -> None:
    K, N = src.shape
    assert tuple(dst.shape) == (N, K) and src.is_contiguous() and dst.is_contiguous()
    check(lib().moe_pack_transpose(ptr(src), dtype_code(src), K, N, ptr(dst), stream_handle(stream)))


def pack_swiglu(w1, w3, ffn_sizes, dst, stream=None) -> None:
    d, F = w1.shape
    assert tuple(dst.shape) == (2 * F, d)
    arr = i64_array(ffn_sizes)
    check(lib().moe_pack_swiglu(ptr(w1), ptr(w3), dtype_code(w1), d, arr, len(ffn_sizes), ptr(dst),
                                stream_handle(stream)))


def pack_mxfp8(src, codes, scales, stream=None) -> None:
    """MXFP8 codes [R, K] (uint8) and E8M0 block scales [R, K/32] (uint8) of
    the rows of a bf16 matrix src [R, K]."""
    R, K = src.shape
    assert src.stride(1) == 1 and codes.stride(1) == 1 and scales.stride(1) == 1
    assert tuple(codes.shape) == (R, K) and tuple(scales.shape) == (R, K // 32)
    check(lib().moe_pack_mxfp8(ptr(src), R, K, src.stride(0), ptr(codes), codes.stride(0),
                               ptr(scales), scales.stride(0), stream_handle(stream)))


def pack_mxfp8_weights(src, codes, scales, stream=None) -> None:
    """MXFP8 codes [R, K] (uint8) and E8M0 block scales, stage-major
    [K/128, R, 4] (uint8), of a packed bf16 weight matrix src [R, K]: the
    layout the expert descriptor's w13_scale / w2_scale hold."""
    R, K = src.shape
    assert src.stride(1) == 1 and codes.stride(1) == 1 and scales.is_contiguous()
    assert tuple(codes.shape) == (R, K) and tuple(scales.shape) == (K // 128, R, 4)
    check(lib().moe_pack_mxfp8_weights(ptr(src), R, K, src.stride(0), ptr(codes), codes.stride(0),
                                       ptr(scales), stream_handle(stream)))


def rmsnorm_stats(x, eps, r, gamma=None, xg=None, stream=None) -> None:
    T, d = x.shape
    check(lib().moe_rmsnorm_stats(ptr(x), dtype_code(x), T, d, ptr(gamma), float(eps), ptr(r),
                                  ptr(xg), stream_handle(stream)))


def router_topk(router: RouterDesc, x, k, renorm, ids, w, r_in=None, r_out=None, eps=1e-6,
                logits=None, ws=None, stream=None, extras: "RouterExtras | None" = None) -> None:
    T, d = x.shape
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    ex = C.byref(extras) if extras is not None else None
    check(lib().moe_router_topk_ex(C.byref(router), ptr(x), dtype_code(x), T, d, ptr(r_in),
                                   float(eps), ptr(r_out), k, renorm, ptr(ids), ptr(w), ptr(logits),
                                   ex, ptr(ws), nbytes, stream_handle(stream)))


def router_extras(noise=None, noise_std=0.0, prob_sum=None, gate_sum=None, aux=None) -> RouterExtras:
    """Noise top-k input and routing-statistics outputs (device tensors or None)."""
    ex = RouterExtras()
    ex.noise, ex.noise_std = ptr(noise), float(noise_std)
    ex.prob_sum, ex.gate_sum, ex.aux = ptr(prob_sum), ptr(gate_sum), ptr(aux)
    return ex


def router_workspace_size(router: RouterDesc, T: int) -> int:
    return int(lib().moe_router_workspace_size(C.byref(router), T))


def dispatch_workspace_size(T: int, k: int, E: int) -> int:
    return int(lib().moe_dispatch_workspace_size(T, k, E))


def dispatch(ids, w, r, E, cap, pad, rows_max_, out: dict, x=None, x_perm=None, stats=None,
             ws=None, stream=None, dtype=None) -> None:
    T, k = ids.shape
    d = 0 if x is None else x.shape[1]
    dt = dtype_code(x) if x is not None else (MOE_BF16 if dtype is None else dtype)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    check(lib().moe_dispatch(ptr(ids), ptr(w), ptr(r), ptr(x), dt, T, d, E, k, cap, pad, rows_max_,
                             ptr(out["counts"]), ptr(out["offsets"]), ptr(out["pos"]),
                             ptr(out["row_token"]), ptr(out["row_r"]), ptr(out["row_w"]),
                             ptr(out.get("row_expert")), ptr(x_perm), ptr(stats), ptr(ws), nbytes,
                             stream_handle(stream)))


def dispatch_noalloc(ids, w, r, E, cap, pad, rows_max_, out: dict, x=None, x_perm=None,
                     stats=None, stream=None, dtype=None) -> None:
    """moe_dispatch_noalloc: moe_dispatch on the library's static scratch."""
    T, k = ids.shape
    d = 0 if x is None else x.shape[1]
    dt = dtype_code(x) if x is not None else (MOE_BF16 if dtype is None else dtype)
    check(lib().moe_dispatch_noalloc(ptr(ids), ptr(w), ptr(r), ptr(x), dt, T, d, E, k, cap, pad,
                                     rows_max_, ptr(out["counts"]), ptr(out["offsets"]),
                                     ptr(out["pos"]), ptr(out["row_token"]), ptr(out["row_r"]),
                                     ptr(out["row_w"]), ptr(out.get("row_expert")), ptr(x_perm),
                                     ptr(stats), stream_handle(stream)))


def topology_nnz_max(rows_max_: int, block: int, ffn_sizes) -> int:
    return int(lib().moe_topology_nnz_max(rows_max_, block, i64_array(ffn_sizes), len(ffn_sizes)))


def build_topology(offsets, size_blocks, block_offsets, E, block, rows_max_, row_offsets,
                   column_indices, nnz, stream=None) -> None:
    check(lib().moe_build_topology(ptr(offsets), ptr(size_blocks), ptr(block_offsets), E, block,
                                   rows_max_, ptr(row_offsets), ptr(column_indices), ptr(nnz),
                                   stream_handle(stream)))


def combine(y, pos, residual, shared, T, d, k, out, stream=None) -> None:
    check(lib().moe_combine(ptr(y), ptr(pos), ptr(residual), ptr(shared), dtype_code(out), T, d, k,
                            ptr(out), stream_handle(stream)))


def make_routing(T, k, E, rows_max_, pad, t: dict) -> Routing:
    rt = Routing()
    rt.T, rt.k, rt.E, rt.rows_max, rt.pad = T, k, E, rows_max_, pad
    for name in ("ids", "w", "r", "counts", "offsets", "pos", "row_token", "row_r", "row_w",
                 "row_expert"):
        setattr(rt, name, ptr(t.get(name)))
    return rt


def expert_workspace_size(desc: ExpertsDesc, dtype: int, d: int, T: int, k: int, rows_max_: int) -> int:
    return int(lib().moe_expert_workspace_size(C.byref(desc), dtype, d, T, k, rows_max_))


def expert_gemm(desc: ExpertsDesc, dtype: int, d: int, routing: Routing, x_in, y, ws,
                stream=None, stats=None) -> None:
    check(lib().moe_expert_gemm(C.byref(desc), dtype, d, C.byref(routing), ptr(x_in), ptr(y),
                                ptr(stats), ptr(ws), ws.numel() * ws.element_size(),
                                stream_handle(stream)))


def shared_workspace_size(desc: ExpertsDesc, dtype: int, d: int, T: int) -> int:
    return int(lib().moe_shared_workspace_size(C.byref(desc), dtype, d, T))


def shared_ffn(desc: ExpertsDesc, xhat, r, s, ws, stream=None) -> None:
    T, d = xhat.shape
    check(lib().moe_shared_ffn(C.byref(desc), dtype_code(xhat), d, T, ptr(xhat), ptr(r), ptr(s),
                               ptr(ws), ws.numel() * ws.element_size(), stream_handle(stream)))


# ---------------------------------------------------------------- timer

class StageTimer:
    """hipEvent timing of each stage of moe_layer_forward (library-side)."""

    def __init__(self, max_calls: int):
        h = C.c_void_p()
        check(lib().moe_timer_create(C.byref(h), max_calls))
        self.handle = h

    def reset(self) -> None:
        check(lib().moe_timer_reset(self.handle))

    def stage_ms(self, stage: str) -> tuple[float, int]:
        tot = C.c_double()
        n = C.c_int()
        check(lib().moe_timer_stage_ms(self.handle, STAGES.index(stage), C.byref(tot), C.byref(n)))
        return tot.value, n.value

    def close(self) -> None:
        if self.handle:
            lib().moe_timer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
