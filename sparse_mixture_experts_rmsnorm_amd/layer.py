"""One MoE FFN layer on the GPU: weight packing, descriptors, workspace.

A thin owner of device buffers around the C ABI: it packs the weights once
(moe_pack_transpose / moe_pack_swiglu / moe_pack_mxfp8_weights), fills the
moe_layer_desc and calls moe_layer_forward.  No arithmetic of the layer
happens here.
"""
from __future__ import annotations

import ctypes as C

from . import binding as B
from .workloads import Workload

# Row padding (bytes) of the MXFP8 second-linear weight codes.
MX_W2_PAD = 256


class MoELayer:
    def __init__(self, wl: Workload, params: dict, device="cuda", train: bool = False):
        """train=True: the forward keeps what backward() needs, and the
        expert descriptors carry the backward's weight layouts."""
        import torch
        self.wl = wl
        self.train = train
        self.device = device
        self.tdtype = torch.float32 if wl.dtype == "f32" else torch.bfloat16
        self.dtype = B.MOE_F32 if wl.dtype == "f32" else B.MOE_BF16
        d = wl.d
        keep = []
        desc = B.LayerDesc()
        desc.d = d
        desc.dtype = self.dtype
        desc.gamma = B.ptr(params.get("gamma"))
        keep.append(params.get("gamma"))
        desc.eps = wl.eps
        desc.k = wl.k
        desc.renorm = wl.renorm
        desc.capacity_factor = wl.cf
        desc.residual = 1
        desc.timer = None
        desc.save_for_backward = 1 if train else 0

        def empty(*shape):
            return torch.empty(shape, dtype=self.tdtype, device=device)

        # router
        R = desc.router
        if wl.router == "cartesian":
            R.kind = B.ROUTER_CARTESIAN
            R.E = wl.Nr * wl.Nc
            R.Nr, R.Nc = wl.Nr, wl.Nc
            keys_t = empty(wl.Nr + wl.Nc, d)
            B.pack_transpose(params["k_rows"], keys_t[: wl.Nr])
            B.pack_transpose(params["k_cols"], keys_t[wl.Nr:])
            R.keys_t = keys_t.data_ptr()
            keep.append(keys_t)
        else:
            R.kind = B.ROUTER_DENSE
            R.E = wl.E
            wr_t = empty(wl.E, d)
            B.pack_transpose(params["w_router"], wr_t)
            R.wr_t = wr_t.data_ptr()
            keep.append(wr_t)
            bias = params.get("bias")
            if bias is not None:
                bias = bias.to(device=device, dtype=torch.float32).contiguous()
                R.bias = bias.data_ptr()
                keep.append(bias)
        # routed experts
        X = desc.experts
        self._fill_experts(X, wl, params, keep, "w1", "w3", "w2", wl.sizes, wl.act,
                           {"grouped": B.EXPERTS_GROUPED, "bcsr": B.EXPERTS_BCSR,
                            "atomic": B.EXPERTS_ATOMIC}[wl.expert_kind], wl.quant)
        # shared experts
        self.shared_desc = None
        if wl.shared_ffn:
            S = B.ExpertsDesc()
            self._fill_experts(S, wl, params, keep, "ws1", "ws3", "ws2", [wl.shared_ffn],
                               wl.shared_act, B.EXPERTS_GROUPED)
            self.shared_desc = S
            desc.shared = C.pointer(S)
        self.desc = desc
        self._keep = keep
        torch.cuda.current_stream().synchronize()

    def _fill_experts(self, X, wl, params, keep, n1, n3, n2, sizes, act, kind, quant="none"):
        import torch
        d = wl.d
        X.kind = kind
        X.act = B.ACT[act]
        if kind == B.EXPERTS_ATOMIC:
            X.E = wl.Nr * wl.Nc
            X.W = params["W"].data_ptr()
            X.V = params["V"].data_ptr()
            keep += [params["W"], params["V"]]
            return
        E = len(sizes)
        X.E = E
        F = sum(sizes)
        arr = B.i64_array(sizes)
        keep.append(arr)
        X.ffn_sizes = C.cast(arr, C.POINTER(C.c_int64))
        off = [0]
        for s in sizes:
            off.append(off[-1] + s)
        foff = torch.tensor(off, dtype=torch.int32, device=self.device)
        X.ffn_offsets = foff.data_ptr()
        keep.append(foff)
        if act == "swiglu":
            w13 = torch.empty((2 * F, d), dtype=self.tdtype, device=self.device)
            B.pack_swiglu(params[n1], params[n3], sizes, w13)
        else:
            w13 = torch.empty((F, d), dtype=self.tdtype, device=self.device)
            B.pack_transpose(params[n1], w13)
        w2t = torch.empty((d, F), dtype=self.tdtype, device=self.device)
        B.pack_transpose(params[n2], w2t)
        if quant == "mxfp8":
            # E4M3 codes + E8M0 block scales along K of each packed row (the
            # scales stage-major, as the expert GEMMs read them).  The code
            # rows of the second linear (F bytes, a multiple of 128) get
            # MX_W2_PAD bytes of row padding (w2_ld): with F a multiple of a
            # large power of two, the rows one K step of a weight tile reads
            # would all start on the same low address bits, which measured
            # markedly slower.
            packed = []
            for w, pad in ((w13, 0), (w2t, MX_W2_PAD)):
                R, K = w.shape
                q = torch.empty((R, K + pad), dtype=torch.uint8, device=self.device)
                sc = torch.empty((K // 128, R, 4), dtype=torch.uint8, device=self.device)
                B.pack_mxfp8_weights(w, q[:, :K], sc)
                packed.append((q, sc))
            torch.cuda.current_stream().synchronize()
            (w13, s13), (w2t, s2) = packed
            X.w2_ld = F + MX_W2_PAD
            X.quant = B.QUANT_MXFP8
            X.w13_scale = s13.data_ptr()
            X.w2_scale = s2.data_ptr()
            keep += [s13, s2]
        X.w13_t = w13.data_ptr()
        X.w2_t = w2t.data_ptr()
        keep += [w13, w2t]
        if self.train:
            # backward layouts: the pages' w2 [F, d] as given, w13_t transposed
            w2fk = params[n2].contiguous()
            w13dk = torch.empty((d, w13.shape[0]), dtype=self.tdtype, device=self.device)
            B.pack_transpose(w13, w13dk)
            X.w2_fk = w2fk.data_ptr()
            X.w13_dk = w13dk.data_ptr()
            keep += [w2fk, w13dk]
        X.block = 128
        if kind == B.EXPERTS_BCSR:
            sb = torch.tensor([s // 128 for s in sizes], dtype=torch.int32, device=self.device)
            bo = torch.tensor([o // 128 for o in off], dtype=torch.int32, device=self.device)
            X.size_blocks = sb.data_ptr()
            X.block_offsets = bo.data_ptr()
            keep += [sb, bo]

    # ------------------------------------------------------------ calls

    def workspace_size(self, T: int) -> int:
        n = int(B.lib().moe_layer_workspace_size(C.byref(self.desc), T))
        if n == 0:
            raise B.MoeError(-1, B.last_error() or "invalid layer descriptor")
        return n

    def alloc_workspace(self, T: int):
        import torch
        return torch.empty(self.workspace_size(T), dtype=torch.uint8, device=self.device)

    def forward(self, x, out=None, ws=None, stats=None, timer: B.StageTimer | None = None,
                stream=None, router_extras: B.RouterExtras | None = None):
        """moe_layer_forward on `stream` (torch's current stream by default).

        An `out` or `ws` left to this wrapper is allocated from the pool of
        the stream the layer runs on, so the caching allocator cannot hand
        the workspace (freed when this returns) to another stream while the
        layer's kernels still use it.  Buffers the caller passes are the
        caller's to keep alive until the stream has finished with them."""
        import contextlib

        import torch
        T = x.shape[0]
        ctx = torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()
        with ctx:
            if out is None:
                out = torch.empty_like(x)
            if ws is None:
                ws = self.alloc_workspace(T)
        self.desc.timer = None if timer is None else timer.handle
        if router_extras is not None:
            self.desc.router_extras = C.pointer(router_extras)
        try:
            B.check(B.lib().moe_layer_forward(C.byref(self.desc), B.ptr(x), T, B.ptr(out),
                                              B.ptr(stats), B.ptr(ws), ws.numel(),
                                              B.stream_handle(stream)))
        finally:
            self.desc.timer = None
            self.desc.router_extras = None
        return out

    def backward_workspace_size(self, T: int) -> int:
        n = int(B.lib().moe_layer_backward_workspace_size(C.byref(self.desc), T))
        if n == 0:
            raise B.MoeError(-1, B.last_error() or "invalid layer descriptor for the backward")
        return n

    def backward(self, x, dout, ws, bws=None, grads: dict | None = None, stream=None) -> dict:
        """Gradients for dout = dL/d(out) of the last forward on ws (fp32
        weight gradients in the forward's packed layouts; dx in x's dtype).
        Buffers left to the wrapper come from the pool of the stream the
        backward runs on (as in forward)."""
        import contextlib

        import torch
        if not self.train:
            raise RuntimeError("the layer was built without train=True")
        wl, d, T = self.wl, self.wl.d, x.shape[0]
        dev = x.device
        ctx = torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()
        with ctx:
            if bws is None:
                bws = torch.empty(self.backward_workspace_size(T), dtype=torch.uint8, device=dev)
            if grads is None:
                f32 = dict(dtype=torch.float32, device=dev)
                E = wl.E
                F = sum(wl.sizes)
                P = 2 * F if wl.act == "swiglu" else F
                grads = dict(dx=torch.empty_like(x), dw_router=torch.empty((E, d), **f32),
                             dw13=torch.empty((P, d), **f32), dw2=torch.empty((F, d), **f32))
                if self.desc.router.bias:
                    grads["dbias"] = torch.empty(E, **f32)
                if self.desc.gamma:
                    grads["dgamma"] = torch.empty(d, **f32)
                if wl.shared_ffn:
                    Ps = 2 * wl.shared_ffn if wl.shared_act == "swiglu" else wl.shared_ffn
                    grads["dws13"] = torch.empty((Ps, d), **f32)
                    grads["dws2"] = torch.empty((wl.shared_ffn, d), **f32)
        g = B.LayerGrads()
        for name in ("dx", "dgamma", "dw_router", "dbias", "dw13", "dw2", "dws13", "dws2"):
            setattr(g, name, B.ptr(grads.get(name)))
        B.check(B.lib().moe_layer_backward(C.byref(self.desc), B.ptr(x), T, B.ptr(dout), B.ptr(ws),
                                           ws.numel(), C.byref(g), B.ptr(bws), bws.numel(),
                                           B.stream_handle(stream)))
        return grads

    def routing(self, T: int, ws) -> dict:
        """Views into the workspace of the routing of the last forward."""
        import torch
        rt = B.Routing()
        B.check(B.lib().moe_layer_routing(C.byref(self.desc), T, B.ptr(ws), ws.numel(),
                                          C.byref(rt)))
        base = ws.data_ptr()
        k, E, R = rt.k, rt.E, rt.rows_max

        def view(p, n, dt):
            nbytes = n * torch.empty(0, dtype=dt).element_size()
            o = p - base
            return ws[o:o + nbytes].view(dt)

        i32, f32 = torch.int32, torch.float32
        return dict(
            ids=view(rt.ids, T * k, i32).view(T, k), w=view(rt.w, T * k, f32).view(T, k),
            r=view(rt.r, T, f32), counts=view(rt.counts, E, i32),
            offsets=view(rt.offsets, E + 1, i32), pos=view(rt.pos, T * k, i32).view(T, k),
            row_token=view(rt.row_token, R, i32), row_r=view(rt.row_r, R, f32),
            row_w=view(rt.row_w, R, f32), row_expert=view(rt.row_expert, R, i32),
            rows_max=R, pad=rt.pad)
