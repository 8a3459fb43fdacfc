"""Copy one layer's seeded numpy inputs into device tensors.

bf16 arrays arrive as uint16 bit patterns and are reinterpreted, not
converted, so the device holds exactly the values the oracle decodes.
"""
from __future__ import annotations

import numpy as np
import torch


def _bf16(a: np.ndarray, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def elem_tensor(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    if dtype == "bf16":
        return _bf16(a, device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def to_device(inp: dict, device="cuda", weights: bool = True) -> dict:
    dev = torch.device(device)
    d = dict(
        logits=torch.from_numpy(np.ascontiguousarray(inp["logits"])).to(dev),
        is_visual=torch.from_numpy(np.ascontiguousarray(inp["is_visual"])).to(dev),
        entropy_w=torch.from_numpy(np.ascontiguousarray(inp["entropy_w"])).to(dev),
        modality=torch.from_numpy(np.ascontiguousarray(inp["modality"])).to(dev),
        sim=torch.from_numpy(np.ascontiguousarray(inp["sim"])).to(dev),
        prot=torch.from_numpy(np.ascontiguousarray(inp["prot"])).to(dev),
    )
    if weights:
        d["x"] = elem_tensor(inp["x"], inp["dtype"], dev)
        d["w13"] = elem_tensor(inp["w13"], inp["dtype"], dev)
        d["w2"] = elem_tensor(inp["w2"], inp["dtype"], dev)
    return d


def torch_elem_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def y_to_f64(y: torch.Tensor) -> np.ndarray:
    """Exact fp64 values of a device result (bf16 or fp32)."""
    return y.detach().float().cpu().numpy().astype(np.float64)
