"""Device memory holder for one layer's weights (PyTorch tensors).

Uploads the arrays of a layer (the dict layout written by the seeded input
generator: GGUF-like NVFP4 bytes or BF16 bits) and repacks NVFP4 matrices
into the runtime layout with the library's own repack kernel.  Builds the
moe_layer_desc / moe_layer_weights structs the C entry points take.
"""
import numpy as np
import torch

from . import (MOE_W_BF16, MOE_W_NVFP4, moe_decode_layer, moe_decode_wait_status, moe_decode_workspace_bytes,
               moe_layer_desc, moe_layer_weights, moe_prefill_layer, moe_prefill_workspace_bytes, moe_repack_nvfp4)


class DeviceLayer:
    """One layer resident in device memory, in the library's runtime layout."""

    def __init__(self, layer, device="cuda", nan_count=None):
        self.device = torch.device(device)
        H, I, Is, E = layer["hidden"], layer["inter"], layer["shared_inter"], layer["n_experts"]
        self.wtype = MOE_W_NVFP4 if layer["wtype"] == "nvfp4" else MOE_W_BF16
        self.desc = moe_layer_desc(hidden=H, inter=I, shared_inter=Is, n_experts=E,
                                   top_k=layer["top_k"] if E > 0 else 0, wtype=self.wtype,
                                   norm_eps=float(layer.get("eps", 1e-6)))
        self.t = {}
        dev = self.device

        def u8(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8).reshape(-1)).to(dev)

        def u16(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16).reshape(-1)).to(dev)

        def f32(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32).reshape(-1)).to(dev)

        self.nan_count = nan_count if nan_count is not None else torch.zeros(1, dtype=torch.int32, device=dev)

        def repacked(a, rows, cols, n):
            src = u8(a)
            dst = torch.empty_like(src)
            moe_repack_nvfp4(src, dst, rows, cols, n, self.nan_count)
            return dst

        if E > 0:
            self.t["router_w"] = u16(layer["router_w"])
            if layer.get("router_b") is not None:
                self.t["router_b"] = f32(layer["router_b"])
            if self.wtype == MOE_W_NVFP4:
                self.t["w_gate"] = repacked(layer["w_gate"], I, H, E)
                self.t["w_up"] = repacked(layer["w_up"], I, H, E)
                self.t["w_down"] = repacked(layer["w_down"], H, I, E)
                self.t["w_scale"] = f32(layer["w_scale"])
            else:
                self.t["w_gate"] = u16(layer["w_gate"])
                self.t["w_up"] = u16(layer["w_up"])
                self.t["w_down"] = u16(layer["w_down"])
        if Is > 0:
            if self.wtype == MOE_W_NVFP4:
                self.t["sh_gate"] = repacked(layer["sh_gate"], Is, H, 1)
                self.t["sh_up"] = repacked(layer["sh_up"], Is, H, 1)
                self.t["sh_down"] = repacked(layer["sh_down"], H, Is, 1)
                self.t["sh_scale"] = f32(layer["sh_scale"])
            else:
                self.t["sh_gate"] = u16(layer["sh_gate"])
                self.t["sh_up"] = u16(layer["sh_up"])
                self.t["sh_down"] = u16(layer["sh_down"])
        if layer.get("norm_gain") is not None:
            self.t["norm_gain"] = u16(layer["norm_gain"])
        self.residual = int(layer.get("residual", 0))
        self.weights = self.make_weights()

    def make_weights(self):
        w = moe_layer_weights()
        for name, _ in moe_layer_weights._fields_:
            v = self.t.get(name)
            setattr(w, name, None if v is None else v.data_ptr())
        return w

    # -- convenience wrappers over the C entry points ------------------------
    def workspace(self, max_batch=8):
        n = moe_decode_workspace_bytes(self.desc, max_batch)
        return torch.zeros(n, dtype=torch.uint8, device=self.device)

    def decode(self, x, ws=None, residual=None, want_topk=True, stream=None):
        """x: int16 tensor [B, H] of BF16 bits on the device -> (y, idx, w).
        The call's wait status word is copied into self.status (see
        wait_status())."""
        B = x.shape[0]
        if ws is None:
            ws = self.workspace(B)
        y = torch.empty_like(x)
        k = self.desc.top_k if self.desc.n_experts > 0 else 0
        idx = torch.empty((B, max(k, 1)), dtype=torch.int32, device=self.device) if want_topk else None
        w = torch.empty((B, max(k, 1)), dtype=torch.float32, device=self.device) if want_topk else None
        moe_decode_layer(self.desc, self.weights, x, B, self.residual if residual is None else residual, y,
                         idx if k else None, w if k else None, ws, ws.numel(), stream)
        if not hasattr(self, "status"):
            self.status = torch.zeros(1, dtype=torch.int32, device=self.device)
        moe_decode_wait_status(ws, self.status, stream)
        return y, idx, w

    def wait_status(self):
        """The last decode call's wait status (0: no wait gave up); syncs."""
        return int(self.status.item())

    def prefill(self, x, ws=None, residual=None, stream=None):
        T = x.shape[0]
        if ws is None:
            ws = torch.zeros(moe_prefill_workspace_bytes(self.desc, T), dtype=torch.uint8, device=self.device)
        y = torch.empty_like(x)
        k = self.desc.top_k if self.desc.n_experts > 0 else 0
        idx = torch.empty((T, max(k, 1)), dtype=torch.int32, device=self.device)
        w = torch.empty((T, max(k, 1)), dtype=torch.float32, device=self.device)
        moe_prefill_layer(self.desc, self.weights, x, T, self.residual if residual is None else residual, y,
                          idx if k else None, w if k else None, ws, ws.numel(), stream)
        return y, idx, w
