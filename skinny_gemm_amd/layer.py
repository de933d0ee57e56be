"""Device-side holders for the C ABI: upload canonical arrays, prepack, size
workspaces, call forward.  Allocation and copies only (PyTorch tensors);
all arithmetic runs in the library's kernels.
"""

from __future__ import annotations

import numpy as np
import torch

from . import (layer_desc, qmatrix_desc, prepacked_size, prepack, prepack_scales, workspace_size, forward_ex,
               forward_plan,
               linear_prepacked_size, linear_prepack, linear, linear_workspace_size, unpack_codes,
               linear_unpack_codes)

TORCH_ACT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def to_device_bits(a: np.ndarray, dtype: str = None, device="cuda") -> torch.Tensor:
    """uint16 bit patterns -> a device tensor of that dtype (bf16/f16), or uint8 bytes."""
    if a is None:
        return None
    if a.dtype == np.float32:  # f32 activations are carried as values
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    if a.dtype == np.uint8:
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)
    return t.view(TORCH_ACT[dtype]) if dtype else t


def bits_of(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16/f16 tensor; float32 values of an f32 one."""
    if t.dtype == torch.float32:
        return t.detach().contiguous().cpu().numpy()
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class MoeLayer:
    """One prepacked MoE layer on the current device."""

    def __init__(self, E, H, I, act_dtype, fc1, fc2, arrays: dict, device="cuda", activation="swiglu"):
        self.E, self.H, self.I, self.act_dtype = E, H, I, act_dtype
        self.desc = layer_desc(E, H, I, act_dtype, fc1, fc2, activation)
        self.device = device
        dev = {k: to_device_bits(arrays[k], None, device) for k in
               ("fc1_codes", "fc1_scales", "fc1_biases", "fc2_codes", "fc2_scales", "fc2_biases")}
        self.packed = torch.empty(prepacked_size(self.desc), dtype=torch.uint8, device=device)
        prepack(self.desc, dev["fc1_codes"], dev["fc1_scales"], dev["fc1_biases"], dev["fc2_codes"],
                dev["fc2_scales"], dev["fc2_biases"], self.packed)
        del dev
        # optional per-expert output biases of FC1 [E][FC1 rows] and FC2 [E][H]
        self.fc1_bias = to_device_bits(arrays.get("fc1_expert_bias"), None, device)
        self.fc2_bias = to_device_bits(arrays.get("fc2_expert_bias"), None, device)

    @classmethod
    def from_spec(cls, spec, arrays, device="cuda"):
        return cls(spec.E, spec.H, spec.I, spec.act_dtype,
                   (spec.fc1.fmt, spec.fc1.block, spec.fc1.scale_dtype),
                   (spec.fc2.fmt, spec.fc2.block, spec.fc2.scale_dtype), arrays, device,
                   getattr(spec, "activation", "swiglu"))

    def update_scales(self, arrays: dict, stream=None):
        """Runtime scales: new fc1/fc2 scales (and affine biases), codes kept."""
        dev = {k: to_device_bits(arrays[k], None, self.device) for k in
               ("fc1_scales", "fc1_biases", "fc2_scales", "fc2_biases")}
        prepack_scales(self.desc, dev["fc1_scales"], dev["fc1_biases"], dev["fc2_scales"], dev["fc2_biases"],
                       self.packed, stream=stream)
        torch.cuda.synchronize()  # the device copies of the sources are freed on return
        del dev

    def workspace(self, T: int, top_k: int) -> torch.Tensor:
        return torch.empty(max(workspace_size(self.desc, T, top_k), 256), dtype=torch.uint8,
                           device=self.device)

    def forward(self, x: torch.Tensor, logits: torch.Tensor, top_k: int, y=None, ws=None,
                path="auto", debug=False, stream=None, events=None, topk_weights="renormalized",
                workspace_limit=0, swiglu=None):
        T = x.shape[0]
        if y is None:
            y = torch.empty((T, self.H), dtype=TORCH_ACT[self.act_dtype], device=self.device)
        if ws is None:
            ws = self.workspace(T, top_k) if not workspace_limit else torch.empty(
                max(forward_plan(self.desc, T, top_k, path, topk_weights, workspace_limit)["workspace_bytes"], 256),
                dtype=torch.uint8, device=self.device)
        dbg = {}
        if debug:
            dbg["h"] = torch.full((T * top_k, self.I), float("nan"), dtype=torch.float32, device=self.device)
            dbg["ids"] = torch.full((T, top_k), -1, dtype=torch.int32, device=self.device)
            dbg["w"] = torch.full((T, top_k), float("nan"), dtype=torch.float32, device=self.device)
            if not workspace_limit:  # per-expert counts need a single tile
                dbg["counts"] = torch.full((self.E,), -1, dtype=torch.int32, device=self.device)
        forward_ex(self.desc, self.packed, x, logits, T, top_k, y, ws, stream=stream, path=path,
                   h_out=dbg.get("h"), ids_out=dbg.get("ids"), w_out=dbg.get("w"),
                   counts_out=dbg.get("counts"), events=events, fc1_bias=self.fc1_bias,
                   fc2_bias=self.fc2_bias, topk_weights=topk_weights, workspace_limit=workspace_limit,
                   swiglu=swiglu)
        return (y, dbg) if debug else y

    def unpack(self, which: int) -> torch.Tensor:
        rows, cols = (self.desc.fc1.rows, self.H) if which == 1 else (self.H, self.I)
        out = torch.empty((self.E, rows, cols), dtype=torch.int8, device=self.device)
        unpack_codes(self.desc, self.packed, which, out)
        return out


class QLinear:
    """One prepacked dense quantized matrix W [N][K]."""

    def __init__(self, fmt, block, scale_dtype, N, K, codes, scales, biases, device="cuda"):
        self.N, self.K = N, K
        self.desc = qmatrix_desc(fmt, block, scale_dtype, N, K)
        self.device = device
        c = to_device_bits(codes, None, device)
        s = to_device_bits(scales, None, device)
        b = to_device_bits(biases, None, device)
        self.packed = torch.empty(linear_prepacked_size(self.desc), dtype=torch.uint8, device=device)
        linear_prepack(self.desc, c, s, b, self.packed)
        del c, s, b

    def workspace(self, M: int) -> torch.Tensor:
        return torch.empty(max(linear_workspace_size(self.desc, M), 256), dtype=torch.uint8, device=self.device)

    def __call__(self, x: torch.Tensor, x_dtype: str, y=None, ws=None, path="auto", stream=None):
        M = x.shape[0]
        if y is None:
            y = torch.empty((M, self.N), dtype=TORCH_ACT[x_dtype], device=self.device)
        if ws is None:
            ws = self.workspace(M)
        linear(self.desc, self.packed, x, x_dtype, M, y, ws, path=path, stream=stream)
        return y

    def unpack(self) -> torch.Tensor:
        out = torch.empty((self.N, self.K), dtype=torch.int8, device=self.device)
        linear_unpack_codes(self.desc, self.packed, out)
        return out
