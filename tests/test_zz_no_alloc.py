"""moe_expert_ffn_noalloc against moe_expert_ffn through the C ABI.

The no-allocation entry point runs the same kernels with h in the library's
fixed device buffer instead of a caller workspace, so its expert output rows
must equal those of moe_expert_ffn bit for bit.  Each case makes two calls in
a row on one GPU, the second with a smaller batch (the buffer keeps the
first call's contents), and the decode and tiny fp32 shapes cover the
weight-streaming, 16-row panel and fp32 paths.
"""
import numpy as np
import pytest
import torch

from gpu_util import load_binding, needs_gpu, say
from mixture_experts_layer_macs_amd import configs, synth
from mixture_experts_layer_macs_amd.staging import to_device, torch_elem_dtype

pytestmark = [pytest.mark.gpu, needs_gpu]


def _routed(wl, seed):
    """Device inputs and the dispatch maps of one seeded layer."""
    B = load_binding()
    inp = synth.make_inputs(wl, seed)
    d = to_device(inp, "cuda", weights=True)
    lay = B.Layer(wl.T, wl.H, wl.N, wl.k, wl.I, wl.R, torch_elem_dtype(wl.dtype))
    lay.routing(d["logits"], d["is_visual"], d["entropy_w"], d["modality"],
                d["sim"], d["prot"], wl.kprime, wl.rho, wl.gamma, wl.lam,
                wl.group)
    return B, d, lay.disp["row_token"], lay.disp["expert_offsets"]


def _compare(wl, seed):
    say(f"noalloc ffn {wl.name} seed={seed} T={wl.T} H={wl.H} N={wl.N} "
        f"k={wl.k} I={wl.I} {wl.dtype}")
    B, d, row_token, offsets = _routed(wl, seed)
    ws = B.new_workspace(B.moe_ffn_workspace_size(wl.T, wl.N, wl.k, wl.H, wl.I,
                                                  d["x"].dtype),
                         d["x"].device)
    ref = B.moe_expert_ffn(d["x"], row_token, offsets, d["w13"], d["w2"], wl.k, ws)
    out = torch.full_like(ref, float("nan"))
    B.moe_expert_ffn_noalloc(d["x"], row_token, offsets, d["w13"], d["w2"],
                             wl.k, out)
    torch.cuda.synchronize()
    M = int(offsets[-1].item())
    assert M > 0
    # bit-identical rows (compared as raw bits; rows past M are not written)
    a = ref[:M].contiguous().view(torch.int16 if ref.dtype == torch.bfloat16
                                  else torch.int32)
    b = out[:M].contiguous().view(a.dtype)
    assert torch.equal(a, b), "no-allocation rows differ from moe_expert_ffn"
    say(f"  {M} rows bit-identical")


PAIRS = [
    # (first call, second call with a smaller batch)
    ("qwen3_decode", configs.QWEN3_DECODE, configs.QWEN3_DECODE.with_(T=5)),
    ("sweep_b256_then_b32", configs.SWEEP_LAYER.with_(T=256, kprime=2),
     configs.SWEEP_LAYER.with_(T=32, kprime=0)),
    ("tiny_f32", configs.TINY_F32, configs.TINY_F32.with_(T=37)),
]


@pytest.mark.parametrize("name,first,second", PAIRS, ids=[p[0] for p in PAIRS])
def test_noalloc_ffn_matches_workspace_ffn(name, first, second):
    _compare(first, 0)
    _compare(second, 1)


def test_noalloc_ffn_refuses_more_than_its_buffer():
    B = load_binding()
    wl = configs.QWEN3_DECODE
    T = B.FFN_NOALLOC_MAX_BYTES // (wl.k * wl.I * 2) + 1
    N = wl.k                  # the fewest experts a top-k layer can have
    x = torch.zeros((T, wl.H), dtype=torch.bfloat16, device="cuda")
    w13 = torch.zeros((N, 2 * wl.I, wl.H), dtype=torch.bfloat16, device="cuda")
    w2 = torch.zeros((N, wl.H, wl.I), dtype=torch.bfloat16, device="cuda")
    rt = torch.zeros(T * wl.k, dtype=torch.int32, device="cuda")
    off = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError, match="MOE_ESCRATCH"):
        B.moe_expert_ffn_noalloc(x, rt, off, w13, w2, wl.k)
