"""The C-ABI library without a GPU: it builds, loads, exports every entry
point that include/moe_macs.h declares, answers workspace queries, and
rejects bad arguments on the host before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_macs.h")


@pytest.fixture(scope="module")
def lib():
    from mixture_experts_layer_macs_amd import build
    if not os.path.exists(build.LIB):
        build.build()
    return ctypes.CDLL(build.LIB)


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_path():
    names = declared()
    for n in ("moe_route", "moe_sere_reroute", "moe_capacity_assign",
              "moe_dispatch", "moe_expert_ffn", "moe_combine"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared():
        assert hasattr(lib, name), name


def test_binding_covers_every_symbol():
    from mixture_experts_layer_macs_amd import binding  # loads on CPU too
    assert set(binding._SIGS) == set(declared())


def test_workspace_queries(lib):
    for fn in ("moe_capacity_workspace_size", "moe_dispatch_workspace_size"):
        f = getattr(lib, fn)
        f.restype = ctypes.c_size_t
        small, big = f(128, 128, 8), f(8192, 128, 8)
        assert 0 < small < big
        assert f(0, 128, 8) > 0 and f(-1, 128, 8) == 0
    f = lib.moe_ffn_workspace_size
    f.restype = ctypes.c_size_t
    assert f(128, 128, 8, 2048, 768, 1) >= 128 * 8 * 768 * 2
    assert f(128, 128, 8, 2048, 768, 0) >= 128 * 8 * 768 * 4


def test_host_side_argument_errors(lib):
    P = ctypes.c_void_p
    fake = P(0x1000)   # never dereferenced: every call below fails its checks
    lib.moe_route.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                              ctypes.c_int, P, P, P, P]
    assert lib.moe_route(fake, 4, 0, 1, 0, fake, fake, None, None) == -1  # N<1
    assert lib.moe_route(fake, 4, 8, 9, 0, fake, fake, None, None) == -1  # k>N
    assert lib.moe_route(fake, 4, 8, 2, 7, fake, fake, fake, None) == -1  # R>N-k
    assert lib.moe_route(fake, 4, 2048, 2, 0, fake, fake, None, None) == -1
    assert lib.moe_route(None, 4, 8, 2, 0, fake, fake, None, None) == -1
    assert lib.moe_route(fake, 4, 8, 2, 2, fake, fake, None, None) == -1
    assert lib.moe_route(None, 0, 8, 2, 0, None, None, None, None) == 0   # T=0
    lib.moe_sere_reroute.argtypes = [P, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                     P, P, P, P, P]
    assert lib.moe_sere_reroute(fake, 4, 8, 2, 3, 0.5, fake, fake, fake, fake, None) == -1
    assert lib.moe_sere_reroute(fake, 4, 8, 2, 0, 0.5, fake, fake, fake, fake, None) == -1
    assert lib.moe_sere_reroute(fake, 4, 8, 2, 1, 0.5, fake, None, fake, fake, None) == -1
    D = ctypes.c_double
    lib.moe_capacity_assign.argtypes = (
        [P] * 6 + [ctypes.c_int] * 5 + [D, D] + [P] * 7 + [ctypes.c_size_t, P])
    args = [fake] * 6 + [4, 8, 2, 2, 8, 1.0, 1.0] + [fake] * 7
    assert lib.moe_capacity_assign(*args, 0, None) == -1        # workspace short
    bad_group = [fake] * 6 + [4, 8, 2, 2, 0, 1.0, 1.0] + [fake] * 7
    assert lib.moe_capacity_assign(*bad_group, 1 << 20, None) == -1
    bad_gamma = [fake] * 6 + [4, 8, 2, 2, 8, float("nan"), 1.0] + [fake] * 7
    assert lib.moe_capacity_assign(*bad_gamma, 1 << 20, None) == -1
    lib.moe_expert_ffn.argtypes = ([P] * 5 + [ctypes.c_int] * 6 + [P, P,
                                   ctypes.c_size_t, P])
    # bf16 needs H % 256 == 0 and I % 128 == 0
    assert lib.moe_expert_ffn(fake, fake, fake, fake, fake, 4, 8, 2, 200, 768,
                              1, fake, fake, 1 << 30, None) == -2
    assert lib.moe_expert_ffn(fake, fake, fake, fake, fake, 4, 8, 2, 2048, 768,
                              7, fake, fake, 1 << 30, None) == -2   # dtype
    lib.moe_ffn_combine_workspace_size.restype = ctypes.c_size_t
    lib.moe_ffn_workspace_size.restype = ctypes.c_size_t
    ws_c = lib.moe_ffn_combine_workspace_size(4, 8, 2, 2048, 768, 2)
    ws_f = lib.moe_ffn_workspace_size(4, 8, 2, 2048, 768, 2)
    assert ws_c == ws_f + 256     # 64 ticket words, then h
    lib.moe_expert_ffn_combine.argtypes = ([P] * 7 + [ctypes.c_int] * 6 +
                                           [P, P, P, ctypes.c_size_t, P])
    args = [fake] * 7 + [4, 8, 2, 2048, 768, 2, fake, fake, fake]
    assert lib.moe_expert_ffn_combine(*args, ws_c - 1, None) == -1   # workspace short
    args = [fake] * 5 + [None, fake] + [4, 8, 2, 2048, 768, 2, fake, fake, fake]
    assert lib.moe_expert_ffn_combine(*args, ws_c, None) == -1       # no slot_row
    args = [fake] * 7 + [4, 8, 2, 2048, 768, 5, fake, fake, fake]
    assert lib.moe_expert_ffn_combine(*args, 1 << 30, None) == -2    # dtype
    args = [fake] * 7 + [4, 8, 2, 4, 4, 0, fake, fake, fake]
    assert lib.moe_expert_ffn_combine(*args, 1 << 30, None) == -2    # f32, H % 8
    lib.moe_combine.argtypes = [P, P, P] + [ctypes.c_int] * 4 + [P, P]
    assert lib.moe_combine(fake, fake, fake, 4, 2, 100, 1, fake, None) == -2
    assert lib.moe_combine(None, fake, fake, 4, 2, 64, 1, fake, None) == -1


def test_host_side_errors_fused_and_entropy(lib):
    """The fused routing launch and the entropy producer reject bad
    arguments on the host and report shapes they do not cover."""
    P, I_, F, D, SZ = (ctypes.c_void_p, ctypes.c_int, ctypes.c_float,
                       ctypes.c_double, ctypes.c_size_t)
    fake = P(0x1000)
    lib.moe_routing_workspace_size.restype = SZ
    lib.moe_routing_workspace_size.argtypes = [I_] * 4
    assert lib.moe_routing_workspace_size(128, 128, 8, 8) > 0
    assert lib.moe_routing_workspace_size(4096, 128, 8, 8) == 0   # tail too big
    lib.moe_routing_fused.argtypes = ([P] * 6 + [I_] * 5 + [F, I_, D, D] +
                                      [P] * 15 + [SZ, P])
    big = [fake] * 6 + [4096, 128, 8, 8, 2, 0.5, 128, 1.0, 1.0] + [fake] * 15
    assert lib.moe_routing_fused(*big, 1 << 20, None) == -2       # MOE_EUNSUP
    bad_kp = [fake] * 6 + [16, 128, 8, 8, 9, 0.5, 128, 1.0, 1.0] + [fake] * 15
    assert lib.moe_routing_fused(*bad_kp, 1 << 20, None) == -1    # K' > k
    short = [fake] * 6 + [16, 128, 8, 8, 2, 0.5, 128, 1.0, 1.0] + [fake] * 15
    assert lib.moe_routing_fused(*short, 0, None) == -1           # workspace
    lib.moe_entropy_workspace_size.restype = SZ
    lib.moe_entropy_workspace_size.argtypes = [I_]
    assert lib.moe_entropy_workspace_size(8192) > 8192 * 4
    lib.moe_entropy_weights.argtypes = [P, P, I_, I_, I_, F, F, P, P, P, SZ, P]
    assert lib.moe_entropy_weights(fake, fake, 4, 64, 7, 1.0, 1e-6, fake, None,
                                   fake, 1 << 20, None) == -2     # dtype
    assert lib.moe_entropy_weights(fake, fake, 4, 64, 1, 1.0, -1.0, fake, None,
                                   fake, 1 << 20, None) == -1     # eps < 0
    assert lib.moe_entropy_weights(fake, None, 4, 64, 1, 1.0, 1e-6, fake, None,
                                   fake, 1 << 20, None) == -1
    assert lib.moe_entropy_weights(fake, fake, 4, 64, 1, 1.0, 1e-6, fake, None,
                                   fake, 8, None) == -1           # workspace
    assert lib.moe_entropy_weights(None, None, 0, 64, 1, 1.0, 1e-6, None, None,
                                   None, 0, None) == 0            # T = 0


def test_router_host_checks_and_workspace(lib):
    """moe_router_topk: shape limits and the workspace query (the split of
    the H axis for short batches needs room for the partial scores)."""
    P, I_, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    f = lib.moe_router_workspace_size
    f.restype = SZ
    f.argtypes = [I_] * 4
    # one control word per 32-token tile; short batches add partial scores
    assert f(8192, 128, 2048, 1) == 256 * 4
    assert f(128, 128, 2048, 1) >= 4 * 8 * 32 * 128 * 4
    assert f(128, 128, 2048, 0) == 256            # fp32: no split
    assert f(128, 128, 2000, 1) == 0              # bf16 needs H % 64 == 0
    assert f(-1, 128, 2048, 1) == 0
    fake = P(0x1000)
    lib.moe_router_topk.argtypes = [P, P] + [I_] * 6 + [P] * 5 + [SZ, P]
    def call(T=4, N=128, H=2048, k=8, R=8, dt=1, logits=None, fb=fake, ws=fake,
             nbytes=1 << 20, x=fake):
        return lib.moe_router_topk(x, fake, T, N, H, k, R, dt, logits, fake,
                                   fake, fb, ws, nbytes, None)
    assert call(N=0) == -1 and call(k=129) == -1 and call(R=121) == -1
    assert call(N=300) == -2                      # fused top-k covers N <= 256
    assert call(H=100) == -2                      # bf16: H % 64
    assert call(H=102, dt=0) == -2                # fp32: H % 4
    assert call(dt=5) == -2
    assert call(fb=None) == -1                    # R > 0 needs fallback_ids
    assert call(ws=None) == -1
    assert call(nbytes=16) == -1                  # workspace too small
    assert call(x=None) == -1
    assert call(T=0, x=None, ws=None) == 0        # T = 0: nothing to do


def test_similarity_host_checks(lib):
    P, I_, SZ, LL = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_longlong
    f = lib.moe_similarity_workspace_size
    f.restype = SZ
    f.argtypes = [I_, LL, I_]
    assert f(128, 256 * 2048, 1) >= 128 * 128 * 8
    assert f(128, 100, 1) == 0            # bf16 needs D % 64 == 0
    assert f(200, 64, 1) == 0             # N <= 128
    assert f(8, 100, 0) > 0               # fp32: any D
    lib.moe_expert_similarity.argtypes = [P, I_, LL, I_, P, P, SZ, P]
    fake = P(0x1000)
    call = lib.moe_expert_similarity
    assert call(fake, 0, 64, 1, fake, fake, 1 << 20, None) == -1
    assert call(fake, 8, 0, 1, fake, fake, 1 << 20, None) == -1
    assert call(fake, 8, 100, 1, fake, fake, 1 << 20, None) == -2
    assert call(fake, 200, 64, 1, fake, fake, 1 << 20, None) == -2
    assert call(fake, 8, 64, 7, fake, fake, 1 << 20, None) == -2
    assert call(None, 8, 64, 1, fake, fake, 1 << 20, None) == -1
    assert call(fake, 8, 64, 1, fake, fake, 8, None) == -1    # workspace short


def test_noalloc_ffn_host_checks(lib):
    P = ctypes.c_void_p
    fake = P(0x1000)   # never dereferenced: every call below fails its checks
    f = lib.moe_expert_ffn_noalloc
    f.argtypes = [P] * 5 + [ctypes.c_int] * 6 + [P, P]
    ws = lib.moe_ffn_workspace_size
    ws.restype = ctypes.c_size_t
    limit = 32 << 20
    # 8192 tokens of the 2048 x 768 shape need 96 MiB of bf16 h: refused
    assert ws(8192, 128, 8, 2048, 768, 1) > limit
    assert f(fake, fake, fake, fake, fake, 8192, 128, 8, 2048, 768, 1, fake,
             None) == -4
    # the largest batch that fits (2730 tokens: 33 546 240 bytes of h) is
    # accepted by the size check (not called here: it would launch); one
    # token more is refused
    T_max = limit // (8 * 768 * 2)
    assert ws(T_max, 128, 8, 2048, 768, 1) <= limit
    assert ws(T_max + 1, 128, 8, 2048, 768, 1) > limit
    assert f(fake, fake, fake, fake, fake, T_max + 1, 128, 8, 2048, 768, 1,
             fake, None) == -4
    # the usual shape and argument checks come first
    assert f(fake, fake, fake, fake, fake, 4, 8, 2, 200, 768, 1, fake,
             None) == -2
    assert f(fake, fake, fake, fake, fake, 4, 8, 9, 2048, 768, 1, fake,
             None) == -1
    assert f(None, None, None, None, None, 0, 8, 2, 2048, 768, 1, None,
             None) == 0                                    # T = 0: nothing


def test_pack_weights_host_checks(lib):
    P = ctypes.c_void_p
    a, b, c, d = P(0x1000), P(0x2000), P(0x3000), P(0x4000)  # never touched
    f = lib.moe_pack_weights
    f.argtypes = [P, P] + [ctypes.c_int] * 4 + [P, P, P]
    assert f(a, b, 8, 2048, 768, 0, c, d, None) == -2         # fp32: no panels
    assert f(a, b, 8, 2048, 768, 2, c, d, None) == -2         # already packed
    assert f(a, b, 8, 2000, 768, 1, c, d, None) == -2         # H % 256
    assert f(a, b, 8, 2048, 700, 1, c, d, None) == -2         # I % 128
    assert f(a, b, 0, 2048, 768, 1, c, d, None) == -1         # no experts
    assert f(a, b, 8, 2048, 768, 1, None, d, None) == -1      # w13 unpaired
    assert f(a, None, 8, 2048, 768, 1, c, d, None) == -1      # w2 unpaired
    assert f(a, b, 8, 2048, 768, 1, a, d, None) == -1         # in place
    assert f(a, b, 8, 2048, 768, 1, c, b, None) == -1
    # the FFN calls accept the packed format code with the bf16 shape rules
    g = lib.moe_expert_ffn_noalloc
    g.argtypes = [P] * 5 + [ctypes.c_int] * 6 + [P, P]
    assert g(a, a, a, a, a, 4, 8, 2, 200, 768, 2, a, None) == -2
    assert g(a, a, a, a, a, 4, 8, 2, 2048, 768, 3, a, None) == -2  # unknown
    assert g(None, None, None, None, None, 0, 8, 2, 2048, 768, 2, None,
             None) == 0
