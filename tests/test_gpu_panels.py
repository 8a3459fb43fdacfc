"""The panel weight layout (moe_pack_weights) through the C ABI.

1. The packed tensors hold each element where the layout puts it: the
   expected packed matrix is built here from the row layout by reshapes
   and a transpose (tile-order rows cut into panels of 128, each panel
   stored as blocks of 64 K elements in MFMA operand order), independent of
   the kernel's index arithmetic, and compared bit for bit.
2. The expert FFN on packed weights equals the FFN on the row layout bit for
   bit on every kernel path the two layouts share (16-row panels, decode
   tiles of both heights, 256-row down tiles, reductions of 4096 and more,
   prefill tiles), since only the addresses of the weight loads differ.
   Decode batches of a few rows per expert take the GEMV on packed weights
   (fp32 sums in another order): there the packed result agrees with the
   row layout to the bf16 bound, and its three entry points bit for bit.
3. A whole layer on packed weights matches the oracle to the bf16 bound.
"""
import numpy as np
import pytest
import torch

from gpu_util import (assert_routing_equal, assert_y_close, load_binding,
                      needs_gpu, say)
from mixture_experts_layer_macs_amd import configs, synth
from mixture_experts_layer_macs_amd.staging import to_device, torch_elem_dtype
from oracle import moe_oracle as O

pytestmark = [pytest.mark.gpu, needs_gpu]


def _panels_expected(w, gate_up):
    """Row layout [N, R, K] -> packed flat [N, R*K] (numpy)."""
    N, R, K = w.shape
    if gate_up:                       # tile order: per 16 h columns, 16 gate
        I = R // 2                    # rows then the 16 matching up rows
        gate = w[:, :I].reshape(N, I // 16, 16, K)
        up = w[:, I:].reshape(N, I // 16, 16, K)
        w = np.stack([gate, up], axis=2).reshape(N, R, K)
    # [N, P, G, r, b, kk, half, e] -> [N, P, b, G, kk, half, r, e]
    p = w.reshape(N, R // 128, 4, 32, K // 64, 4, 2, 8)
    p = p.transpose(0, 1, 4, 2, 5, 6, 3, 7)
    return np.ascontiguousarray(p).reshape(N, R * K)


@pytest.mark.parametrize("N,H,I", [(3, 256, 128), (2, 768, 384), (1, 4096, 256)])
def test_pack_layout(N, H, I):
    B = load_binding()
    say(f"pack layout N={N} H={H} I={I}")
    g = torch.Generator(device="cuda")
    g.manual_seed(N * 1000 + H + I)
    w13 = torch.randn((N, 2 * I, H), device="cuda", generator=g).bfloat16()
    w2 = torch.randn((N, H, I), device="cuda", generator=g).bfloat16()
    p13, p2 = B.moe_pack_weights(w13, w2)
    only2 = B.moe_pack_weights(w2=w2)[1]
    torch.cuda.synchronize()
    bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy()
    np.testing.assert_array_equal(bits(p13).reshape(N, -1),
                                  _panels_expected(bits(w13), True))
    np.testing.assert_array_equal(bits(p2).reshape(N, -1),
                                  _panels_expected(bits(w2), False))
    np.testing.assert_array_equal(bits(only2), bits(p2))


def _mid(**kw):
    base = configs.MM_PREFILL.with_(name="mid_bf16", T=600, H=512, N=16, k=4,
                                    I=256, gamma=1.0, R=4, group=16)
    return base.with_(**kw)


PATH_CASES = [
    # name, workload, both layouts on the same kernels
    # decode tiles (device-chosen heights), 256-row down tiles
    ("qwen3_decode_b128", configs.QWEN3_DECODE, True),
    # few active experts after SERE: one wave of tiles, 128-row down tiles
    ("sweep_b128_k2", configs.SWEEP_LAYER.with_(T=128, kprime=2), True),
    ("sweep_b32", configs.SWEEP_LAYER.with_(T=32, kprime=0), True),
    # packed: the decode GEMV (both halves); rows: 16-row weight panels
    ("sweep_b1", configs.SWEEP_LAYER.with_(T=1, kprime=1), False),
    ("sweep_b4", configs.SWEEP_LAYER.with_(T=4, kprime=0), False),
    # packed: 16-row panels for the K = 4096 half, the GEMV for the other
    ("skinny_h4096", _mid(T=3, H=4096, I=512, k=2), False),
    ("skinny_i4096", _mid(T=2, H=512, I=4096), False),
    # reductions of 4096 and more on the decode tiles
    ("mixtral_decode_t64", configs.MIXTRAL_DECODE, True),
    # prefill tiles, ragged tails, 6 panels of 64-wide K blocks
    ("mid_prefill", _mid(), True),
    ("mid_prefill_h768_i384", _mid(H=768, I=384, T=300), True),
]


@pytest.mark.parametrize("name,wl,same", PATH_CASES, ids=[c[0] for c in PATH_CASES])
def test_panels_ffn_equals_row_layout(name, wl, same):
    B = load_binding()
    say(f"panels ffn {name} T={wl.T} H={wl.H} N={wl.N} k={wl.k} I={wl.I}")
    inp = synth.make_inputs(wl, 0)
    d = to_device(inp, "cuda", weights=True)
    lay = B.Layer(wl.T, wl.H, wl.N, wl.k, wl.I, wl.R, torch_elem_dtype(wl.dtype))
    lay.routing(d["logits"], d["is_visual"], d["entropy_w"], d["modality"],
                d["sim"], d["prot"], wl.kprime, wl.rho, wl.gamma, wl.lam,
                wl.group)
    rt, off = lay.disp["row_token"], lay.disp["expert_offsets"]
    ws = B.new_workspace(B.moe_ffn_workspace_size(wl.T, wl.N, wl.k, wl.H, wl.I,
                                                  torch.bfloat16), d["x"].device)
    ref = B.moe_expert_ffn(d["x"], rt, off, d["w13"], d["w2"], wl.k, ws)
    p13, p2 = B.moe_pack_weights(d["w13"], d["w2"])
    out = torch.full_like(ref, float("nan"))
    B.moe_expert_ffn(d["x"], rt, off, p13, p2, wl.k, ws, out, panels=True)
    # the two halves called separately, and the no-allocation entry point
    h = torch.empty((wl.T * wl.k, wl.I), dtype=torch.bfloat16, device="cuda")
    out2 = torch.full_like(ref, float("nan"))
    B.moe_ffn_gate_up(d["x"], rt, off, p13, wl.k, h, panels=True)
    B.moe_ffn_down(h, off, p2, wl.T, wl.k, out2, panels=True)
    torch.cuda.synchronize()
    M = int(off[-1].item())
    assert M > 0
    bits = lambda t: t[:M].contiguous().view(torch.int16)
    a = bits(out)
    assert torch.equal(a, bits(out2))
    if wl.T * wl.k * wl.I * 2 <= B.FFN_NOALLOC_MAX_BYTES:
        out3 = torch.full_like(ref, float("nan"))
        B.moe_expert_ffn_noalloc(d["x"], rt, off, p13, p2, wl.k, out3, panels=True)
        torch.cuda.synchronize()
        assert torch.equal(a, bits(out3))
    if same:
        assert torch.equal(bits(ref), a)
        say(f"  {M} rows bit-identical")
    else:
        f64 = lambda t: t[:M].float().cpu().numpy().astype(np.float64)
        assert_y_close(f64(out), f64(ref), "bf16")
        say(f"  {M} rows: packed entry points bit-identical, rows to the bf16 bound")


@pytest.mark.parametrize("name,wl", [
    ("qwen3_decode_b128", configs.QWEN3_DECODE),
    ("sweep_b1_vis05_k2", configs.SWEEP_LAYER.with_(T=1, kprime=2)),
    ("mid_prefill", _mid()),
], ids=lambda v: v if isinstance(v, str) else "")
def test_layer_on_panels_matches_oracle(name, wl):
    B = load_binding()
    say(f"layer on panels {name}")
    inp = synth.make_inputs(wl, 1)
    rt = O.layer_routing(inp)
    d = to_device(inp, "cuda", weights=True)
    p13, p2 = B.moe_pack_weights(d["w13"], d["w2"])
    lay = B.Layer(wl.T, wl.H, wl.N, wl.k, wl.I, wl.R, torch.bfloat16)
    lay.forward(d["logits"], d["x"], p13, p2, d["is_visual"], d["entropy_w"],
                d["modality"], d["sim"], d["prot"], wl.kprime, wl.rho,
                wl.gamma, wl.lam, wl.group, panels=True)
    torch.cuda.synchronize()
    M = int(lay.disp["expert_offsets"][-1].item())
    np.testing.assert_array_equal(lay.disp["expert_offsets"].cpu().numpy(),
                                  rt["expert_offsets"])
    assert M == int(rt["expert_offsets"][-1])
    y = lay.y.float().cpu().numpy().astype(np.float64)
    assert_y_close(y, O.layer_outputs(inp, rt), "bf16")
