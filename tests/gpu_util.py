"""Helpers for the GPU parity tests: run the HIP path through the C ABI on
seeded inputs and compare with the CPU oracle.

Tolerances on the layer output y (values of the oracle in fp64):
  bf16: element by element, |dy| <= min(1e-2, 1e-2 max|y|) + 2e-2 |y|:
        the stated bar 1e-2 + 2e-2 |y|, with the absolute floor cut to 1%
        of the largest output when y is small (y of the Qwen-shaped layer
        is itself ~1e-2).  The GPU rounds h and the expert output rows to
        bf16 (relative 2^-9 each) and y once more, so its error is a few
        2^-9 of the row scale.
  fp32: |dy| <= 1e-5 + 1e-5 |y|.
Gates (fp32 on the GPU, fp64 in the oracle): |dg| <= 1e-7 + 1e-5 |g|.
"""
from __future__ import annotations

import math
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def load_binding():
    """Import the binding; build the library first only if nothing is built."""
    from mixture_experts_layer_macs_amd import build as _build
    if not os.path.exists(_build.LIB):
        _build.build()
    from mixture_experts_layer_macs_amd import binding
    return binding


def say(msg: str):
    print(f"[gpu-test] {msg}", flush=True)


def run_gpu_layer(inp: dict, tokens_out=True, fused=None):
    """Run the layer on the GPU through the C ABI; return host numpy copies of
    everything.  fused: True = one moe_routing_fused launch, False = the four
    separate routing calls, None = the layer's default (fused when the batch
    is decode-sized)."""
    import torch
    from mixture_experts_layer_macs_amd import binding as B
    from mixture_experts_layer_macs_amd.staging import to_device, torch_elem_dtype

    d = to_device(inp, "cuda", weights=tokens_out)
    T, H, N, k, I, R = inp["T"], inp["H"], inp["N"], inp["k"], inp["I"], inp["R"]
    lay = B.Layer(T, H, N, k, I, R, torch_elem_dtype(inp["dtype"]))
    if tokens_out:
        lay.forward(d["logits"], d["x"], d["w13"], d["w2"], d["is_visual"],
                    d["entropy_w"], d["modality"], d["sim"], d["prot"],
                    inp["kprime"], inp["rho"], inp["gamma"], inp["lam"],
                    inp["group"], fused=fused)
    else:
        lay.routing(d["logits"], d["is_visual"], d["entropy_w"], d["modality"],
                    d["sim"], d["prot"], inp["kprime"], inp["rho"],
                    inp["gamma"], inp["lam"], inp["group"], fused=fused)
    torch.cuda.synchronize()
    c = lambda t: t.detach().cpu().numpy()
    out = dict(topk_ids=c(lay.topk_ids), gates=c(lay.topk_gates),
               fallback_ids=c(lay.fallback_ids),
               slot_sere=c(lay.slot_sere) if inp["kprime"] else c(lay.topk_ids),
               slot_expert=c(lay.cap["slot_out"]), flags=c(lay.cap["flags"]),
               load_q=c(lay.cap["load_q"]), cap_q=c(lay.cap["cap_q"]),
               stats=c(lay.cap["stats"]), r_v=float(c(lay.cap["r_v"])[0]),
               expert_offsets=c(lay.disp["expert_offsets"]),
               row_token=c(lay.disp["row_token"]),
               row_slot=c(lay.disp["row_slot"]),
               slot_row=c(lay.disp["slot_row"]))
    if tokens_out:
        out["y"] = lay.y.detach().float().cpu().numpy().astype(np.float64)
    return out


def assert_routing_equal(g: dict, rt: dict, inp: dict):
    """Bit-exact comparison of every integer routing output."""
    T, k, N = inp["T"], inp["k"], inp["N"]
    np.testing.assert_array_equal(g["topk_ids"], rt["topk_ids"], "topk_ids")
    if inp["R"]:
        np.testing.assert_array_equal(g["fallback_ids"], rt["fallback_ids"],
                                      "fallback_ids")
    np.testing.assert_allclose(g["gates"], rt["gates"], rtol=1e-5, atol=1e-7,
                               err_msg="gates")
    np.testing.assert_array_equal(g["slot_sere"], rt["slot_sere"], "slot_sere")
    np.testing.assert_array_equal(g["slot_expert"], rt["slot_expert"],
                                  "slot_expert")
    np.testing.assert_array_equal(g["flags"], rt["flags"], "flags")
    np.testing.assert_array_equal(g["load_q"], rt["load_q"], "load_q")
    if rt["cap_q"] is None:
        assert (g["cap_q"] == np.iinfo(np.int64).max).all()
    else:
        np.testing.assert_array_equal(g["cap_q"], rt["cap_q"], "cap_q")
    assert g["r_v"] == rt["r_v"], ("r_v", g["r_v"], rt["r_v"])
    assert g["stats"][0] == rt["w_all"] and g["stats"][1] == rt["w_vis"]
    assert g["stats"][2] == rt["dropped"] and g["stats"][3] == rt["macs_rerouted"]
    M = int(rt["expert_offsets"][-1])
    np.testing.assert_array_equal(g["expert_offsets"], rt["expert_offsets"],
                                  "expert_offsets")
    np.testing.assert_array_equal(g["row_token"][:M], rt["row_token"], "row_token")
    np.testing.assert_array_equal(g["row_slot"][:M], rt["row_slot"], "row_slot")
    np.testing.assert_array_equal(g["slot_row"], rt["slot_row"], "slot_row")


def assert_y_close(y_gpu: np.ndarray, y_ref: np.ndarray, dtype: str):
    err = np.abs(y_gpu - y_ref)
    ref = np.abs(y_ref)
    if dtype == "f32":
        bound = 1e-5 + 1e-5 * ref
    else:
        bound = np.minimum(1e-2, 1e-2 * ref.max()) + 2e-2 * ref
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(
            f"y mismatch at {i}: gpu={y_gpu[i]} ref={y_ref[i]} "
            f"({int(bad.sum())} of {err.size} over bound; "
            f"max|dy|/max|y| = {err.max() / max(ref.max(), 1e-300):.3e})")
    say(f"y ok: max|dy| = {err.max():.3e}, max|y| = {ref.max():.3e}, "
        f"max|dy|/max|y| = {err.max() / max(ref.max(), 1e-300):.3e}")


needs_gpu = pytest.mark.skipif(not gpu_available(), reason="needs a GPU")
