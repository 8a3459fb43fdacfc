"""The decode GEMV path of the expert FFN (packed weights, a few token rows
per expert) through the C ABI, against the oracle's fp64 expert FFN.

The dispatch maps are built by the oracle's dispatch from slot assignments
drawn here, so every case controls how many rows each expert gets: one row,
a token with two slots on one expert, every slot on one expert (more rows
than one workgroup's chunk, so several workgroups share an expert's weight
group), and every reduction length the path takes (K = 256, 512, 768, 1024, 2048 for
the gate-up and the down projections).  Each dispatch row of h and of the
output is compared with the fp64 value to the bf16 bound; the fused and the
no-allocation entry points give the same bits as the two halves called
separately; the row-layout kernels (tile MFMA) agree to the same bound.

moe_expert_ffn_combine (the combine folded into the down GEMV) is checked
against moe_expert_ffn + moe_combine bit for bit -- out_rows and y -- with
dropped slots, tokens or whole batches with every slot dropped, and shapes
that take the two-call path, over two calls in a row on one workspace whose
arrival tickets must be zero again after each; y also against the oracle's
combine of the same rows.
"""
import numpy as np
import pytest
import torch

from gpu_util import assert_y_close, load_binding, needs_gpu, say
from mixture_experts_layer_macs_amd import synth
from mixture_experts_layer_macs_amd.staging import elem_tensor
from oracle import moe_oracle as O

pytestmark = [pytest.mark.gpu, needs_gpu]

CASES = [
    # name, T, H, N, k, I, slot assignment (at most 16 dispatch rows: the
    # GEMV; the last two cases, with more, check the tile kernels the same way)
    ("b1_qwen3_shape", 1, 2048, 128, 8, 768, "spread"),
    ("b2_qwen3_shape", 2, 2048, 128, 8, 768, "spread"),
    ("k256_two_rows_each", 2, 256, 8, 8, 256, "all"),
    ("k512_k1024", 3, 512, 4, 4, 1024, "spread"),
    ("k768_k512", 4, 768, 4, 4, 512, "spread"),
    ("one_expert_16_rows", 8, 1024, 4, 2, 768, "one"),
    ("k2048_both", 4, 2048, 3, 2, 2048, "spread"),
    ("repeated_expert_in_token", 5, 256, 5, 3, 512, "repeat"),
    # 16 tokens: gate-up on the tile kernels (more tokens than are staged
    # whole), down on the GEMV
    ("t16_k1_down_only", 16, 512, 4, 1, 256, "repeat"),
    ("b8_qwen3_shape_tiles", 8, 2048, 128, 8, 768, "spread"),
    ("one_expert_64_rows_tiles", 8, 512, 8, 8, 256, "one"),
]


def _slots(T, N, k, mode, rng):
    if mode == "spread":
        return np.stack([rng.permutation(N)[:k] for _ in range(T)]).astype(np.int32)
    if mode == "all":           # every token on experts 0..k-1
        return np.tile(np.arange(k, dtype=np.int32), (T, 1))
    if mode == "one":           # every slot on expert 1
        return np.full((T, k), 1, dtype=np.int32)
    return rng.integers(0, N, size=(T, k)).astype(np.int32)  # repeats allowed


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gemv_rows_match_oracle(case):
    name, T, H, N, k, I, mode = case
    B = load_binding()
    say(f"gemv {name} T={T} H={H} N={N} k={k} I={I} slots={mode}")
    rng = np.random.default_rng(7000 + CASES.index(case))
    slot = _slots(T, N, k, mode, rng)
    offsets, row_token, _, _ = O.dispatch(slot, N)
    M = int(offsets[-1])
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    w13 = synth.f32_to_bf16_bits(0.02 * rng.standard_normal((N, 2 * I, H), dtype=np.float32))
    w2 = synth.f32_to_bf16_bits(0.02 * rng.standard_normal((N, H, I), dtype=np.float32))
    dev = torch.device("cuda")
    xd, w13d, w2d = (elem_tensor(a, "bf16", dev) for a in (x, w13, w2))
    off_d = torch.from_numpy(offsets).to(dev)
    rt_d = torch.from_numpy(np.ascontiguousarray(row_token)).to(dev)
    p13, p2 = B.moe_pack_weights(w13d, w2d)

    h = torch.full((T * k, I), float("nan"), dtype=torch.bfloat16, device=dev)
    out = torch.full((T * k, H), float("nan"), dtype=torch.bfloat16, device=dev)
    B.moe_ffn_gate_up(xd, rt_d, off_d, p13, k, h, panels=True)
    B.moe_ffn_down(h, off_d, p2, T, k, out, panels=True)
    # the fused and the no-allocation entry points: the same kernels
    ws = B.new_workspace(B.moe_ffn_workspace_size(T, N, k, H, I, torch.bfloat16), dev)
    out_f = torch.full_like(out, float("nan"))
    B.moe_expert_ffn(xd, rt_d, off_d, p13, p2, k, ws, out_f, panels=True)
    out_n = torch.full_like(out, float("nan"))
    B.moe_expert_ffn_noalloc(xd, rt_d, off_d, p13, p2, k, out_n, panels=True)
    # the row layout (tile kernels)
    out_r = B.moe_expert_ffn(xd, rt_d, off_d, w13d, w2d, k, ws)
    torch.cuda.synchronize()

    bits = lambda t: t[:M].contiguous().view(torch.int16)
    assert torch.equal(bits(out), bits(out_f)), "fused entry point differs"
    assert torch.equal(bits(out), bits(out_n)), "no-allocation entry point differs"

    # fp64 reference, expert by expert
    x64 = O.decode(x, "bf16")
    h_ref = np.empty((M, I))
    y_ref = np.empty((M, H))
    for e in range(N):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r0 == r1:
            continue
        xe = x64[row_token[r0:r1]]
        a13 = O.decode(w13[e], "bf16")
        g, u = xe @ a13[:I].T, xe @ a13[I:].T
        h_ref[r0:r1] = O.silu(g) * u
        y_ref[r0:r1] = O.expert_ffn(xe, a13, O.decode(w2[e], "bf16"))
    f64 = lambda t: t[:M].float().cpu().numpy().astype(np.float64)
    assert_y_close(f64(h), h_ref, "bf16")
    assert_y_close(f64(out), y_ref, "bf16")
    assert_y_close(f64(out_r), y_ref, "bf16")
    say(f"  {M} rows within the bf16 bound")


COMBINE_CASES = [
    # name, T, H, N, k, I, slot assignment, share of slots dropped, packed
    ("b1_qwen3_shape", 1, 2048, 128, 8, 768, "spread", 0.0, True),
    ("b2_qwen3_some_dropped", 2, 2048, 128, 8, 768, "spread", 0.3, True),
    ("one_expert_16_rows", 8, 1024, 4, 2, 768, "one", 0.0, True),
    ("repeated_expert_dropped", 5, 256, 5, 3, 512, "repeat", 0.4, True),
    ("t16_k1", 16, 512, 4, 1, 256, "repeat", 0.2, True),
    ("k2048_down", 4, 512, 3, 2, 2048, "spread", 0.0, True),
    ("every_slot_dropped", 2, 512, 8, 4, 256, "spread", 1.0, True),
    # two calls: more rows than the GEMV takes (streamed down tiles, with
    # tokens whose every slot is dropped), and the row layout
    ("b8_qwen3_shape_stream", 8, 2048, 128, 8, 768, "spread", 0.1, True),
    ("b64_dropped_tokens_stream", 64, 1024, 16, 4, 512, "spread", 0.5, True),
    ("b8_qwen3_shape_rows", 8, 2048, 128, 8, 768, "spread", 0.1, False),
    ("b2_rows_layout", 2, 512, 8, 4, 256, "spread", 0.0, False),
]


@pytest.mark.parametrize("case", COMBINE_CASES, ids=[c[0] for c in COMBINE_CASES])
def test_ffn_combine_matches_two_calls(case):
    name, T, H, N, k, I, mode, drop, packed = case
    B = load_binding()
    say(f"ffn+combine {name} T={T} H={H} N={N} k={k} I={I} drop={drop}")
    rng = np.random.default_rng(7100 + COMBINE_CASES.index(case))
    dev = torch.device("cuda")
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    w13 = synth.f32_to_bf16_bits(0.02 * rng.standard_normal((N, 2 * I, H), dtype=np.float32))
    w2 = synth.f32_to_bf16_bits(0.02 * rng.standard_normal((N, H, I), dtype=np.float32))
    xd, w13d, w2d = (elem_tensor(a, "bf16", dev) for a in (x, w13, w2))
    if packed:
        w13d, w2d = B.moe_pack_weights(w13d, w2d)
    ws = B.new_workspace(B.moe_ffn_combine_workspace_size(T, N, k, H, I, torch.bfloat16), dev)
    ws_two = B.new_workspace(B.moe_ffn_workspace_size(T, N, k, H, I, torch.bfloat16), dev)
    # two calls on the same workspace: the second keeps fewer slots
    for call, dropped in enumerate((drop, min(1.0, drop + 0.25))):
        slot = _slots(T, N, k, mode, rng)
        slot[rng.random((T, k)) < dropped] = -1
        offsets, row_token, _, slot_row = O.dispatch(slot, N)
        M = int(offsets[-1])
        gates = rng.uniform(0.01, 1.0, (T, k)).astype(np.float32)
        off_d = torch.from_numpy(offsets).to(dev)
        rt = np.zeros(T * k, dtype=np.int32)  # rows past M are not read
        rt[:M] = row_token
        rt_d = torch.from_numpy(rt).to(dev)
        sr_d = torch.from_numpy(slot_row).to(dev)
        g_d = torch.from_numpy(gates).to(dev)

        rows_f = torch.full((T * k, H), float("nan"), dtype=torch.bfloat16, device=dev)
        y_f = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=dev)
        B.moe_expert_ffn_combine(xd, rt_d, off_d, w13d, w2d, sr_d, g_d, k, ws, rows_f, y_f,
                                 panels=packed)
        rows_2 = torch.full_like(rows_f, float("nan"))
        B.moe_expert_ffn(xd, rt_d, off_d, w13d, w2d, k, ws_two, rows_2, panels=packed)
        y_2 = B.moe_combine(rows_2, sr_d, g_d)
        torch.cuda.synchronize()

        bits = lambda t: t.contiguous().view(torch.int16)
        assert torch.equal(bits(rows_f[:M]), bits(rows_2[:M])), f"call {call}: out_rows differ"
        assert torch.equal(bits(y_f), bits(y_2)), f"call {call}: y differs from moe_combine"
        tickets = ws[: (H // 32) * 4].view(torch.int32)
        assert int(tickets.abs().sum().item()) == 0, f"call {call}: tickets not back to zero"
        rows64 = rows_f[:M].float().cpu().numpy().astype(np.float64)
        y_ref = O.combine(range(T), slot, slot_row, gates.astype(np.float64), rows64, H)
        assert_y_close(y_f.float().cpu().numpy().astype(np.float64), y_ref, "bf16")
        say(f"  call {call}: {M} rows kept, y equal to the two calls")
