"""The C ABI without a GPU: the library loads, exports every function that
include/moe.h declares, and rejects bad arguments on the host before it
enqueues anything.  Every call below fails its argument checks, so no kernel
is ever launched."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = range(5)
F32, BF16 = 0, 1
FAKE = 0x10000  # 16-byte aligned stand-in address; only ever passed to calls that fail their checks
MISALIGNED = 0x10002


@pytest.fixture(scope="module")
def L():
    import moe_layer_amd
    return moe_layer_amd.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(moe_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("moe_route", "moe_permute", "moe_grouped_gemm", "moe_combine", "moe_repack_ep_to_tp",
              "moe_repack_tp_to_ep", "moe_dispatch", "moe_switch_init", "moe_switch_step",
              "moe_switch_crossover", "moe_schedule_requests"):
        assert n in names


def test_library_exports_every_declared_function(L):
    import moe_layer_amd
    for name in declared_functions():
        assert hasattr(L, name), name
        assert name in moe_layer_amd.EXPORTED


def test_version_and_status_strings(L):
    assert L.moe_abi_version() == 8
    for s in range(5):
        assert L.moe_status_str(s).decode().startswith(
            ["MOE_OK", "MOE_EINVAL", "MOE_EUNSUPPORTED", "MOE_EWORKSPACE", "MOE_EHIP"][s])
    assert b"unknown" in L.moe_status_str(99)


def test_workspace_size(L):
    up = L.moe_workspace_bytes(5, 256, 8, 66, 2048, 1408, BF16)
    down = L.moe_workspace_bytes(6, 256, 8, 66, 2048, 1408, BF16)
    a = 256 * 8 * 1408 * 2
    assert up > 0 and up == down and up % 256 == 0  # one layout serves both halves
    assert L.moe_workspace_bytes(2, 256, 8, 66, 2048, 1408, BF16) == a + up
    # a of 3*3*40*4 = 1440 bytes is padded to 1536 before the split-item region
    assert L.moe_workspace_bytes(2, 3, 3, 4, 256, 40, F32) == 1536 + L.moe_workspace_bytes(
        5, 3, 3, 4, 256, 40, F32)
    assert L.moe_workspace_bytes(0, 256, 8, 66, 2048, 1408, BF16) == 0
    assert L.moe_workspace_bytes(2, 0, 8, 66, 2048, 1408, BF16) == 0
    assert L.moe_workspace_bytes(5, 256, 8, 0, 2048, 1408, BF16) == 0
    # grows with the batch, independent of the device
    assert L.moe_workspace_bytes(5, 2048, 8, 16, 4096, 1536, BF16) > L.moe_workspace_bytes(
        5, 8, 8, 16, 4096, 1536, BF16)


def route(L, x=FAKE, wg=FAKE, b=None, T=4, H=256, E=8, k=2, renorm=1, ns=0, dt=BF16,
          lo=FAKE, ids=FAKE, w=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return L.moe_route(x, wg, b, T, H, E, k, renorm, ns, dt, lo, ids, w, ws, ws_bytes, None)


def route_permute(L, T=4, H=256, E=8, k=2, g_begin=0, n_groups=8, counts=FAKE, ws=FAKE, ws_bytes=1 << 30,
                  x=FAKE):
    return L.moe_route_permute(x, FAKE, None, T, H, E, k, 1, 0, BF16, FAKE, FAKE, FAKE, g_begin, n_groups,
                               counts, FAKE, FAKE, FAKE, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=9), MOE_EINVAL),                 # k > E
    (dict(k=0), MOE_EINVAL),
    (dict(T=-1), MOE_EINVAL),
    (dict(dt=7), MOE_EINVAL),
    (dict(x=None), MOE_EINVAL),
    (dict(ids=None), MOE_EINVAL),
    (dict(x=MISALIGNED), MOE_EINVAL),
    (dict(E=513, k=8), MOE_EUNSUPPORTED),
    (dict(E=64, k=33), MOE_EUNSUPPORTED),
    (dict(k=2, ns=63), MOE_EUNSUPPORTED),    # k + n_shared > 64
    (dict(H=100), MOE_EUNSUPPORTED),         # not whole 64-byte K chunks
    (dict(H=1 << 20), MOE_EUNSUPPORTED),     # rows over 1 MiB
    (dict(T=(1 << 27) + 1, k=8), MOE_EUNSUPPORTED),      # T * kk over 2^30 pairs
    (dict(T=1 << 30, E=512, k=1), MOE_EUNSUPPORTED),      # 2^30 pairs, but over 2^31 blocks
    (dict(ws=None), MOE_EWORKSPACE),
    (dict(ws=MISALIGNED), MOE_EWORKSPACE),
    (dict(ws_bytes=0), MOE_EWORKSPACE),
])
def test_route_rejects(L, kw, status):
    assert route(L, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(g_begin=-1), MOE_EINVAL),
    (dict(n_groups=0), MOE_EINVAL),
    (dict(n_groups=513), MOE_EUNSUPPORTED),
    (dict(counts=None), MOE_EINVAL),
    (dict(ws_bytes=16), MOE_EWORKSPACE),
    (dict(x=None), MOE_EINVAL),
    (dict(T=(1 << 29) + 1), MOE_EUNSUPPORTED),   # T * kk over 2^30 pairs
])
def test_route_permute_rejects(L, kw, status):
    assert route_permute(L, **kw) == status


def route_permute_noalloc(L, T=4, H=256, E=8, k=2, g_begin=0, n_groups=8, counts=FAKE, x=FAKE):
    return L.moe_route_permute_noalloc(x, FAKE, None, T, H, E, k, 1, 0, BF16, FAKE, FAKE, FAKE, g_begin,
                                       n_groups, counts, FAKE, FAKE, FAKE, None)


@pytest.mark.parametrize("kw,status", [
    (dict(g_begin=-1), MOE_EINVAL),
    (dict(n_groups=513), MOE_EUNSUPPORTED),
    (dict(counts=None), MOE_EINVAL),
    (dict(x=None), MOE_EINVAL),
    (dict(k=9), MOE_EINVAL),
    (dict(E=513), MOE_EUNSUPPORTED),
    # 2^22 + 1 token-tile counters need more than the 16 MiB fixed scratch
    (dict(T=1 << 26, k=8), MOE_EWORKSPACE),
])
def test_route_permute_noalloc_rejects(L, kw, status):
    assert route_permute_noalloc(L, **kw) == status


def test_route_workspace_size(L):
    small = L.moe_route_workspace_bytes(8, 4096, 128, BF16)
    big = L.moe_route_workspace_bytes(2048, 4096, 128, BF16)
    assert small >= 256 and small % 256 == 0
    assert big >= (2048 // 16 + 1) * 4
    assert L.moe_route_workspace_bytes(0, 4096, 128, BF16) == 0


def test_empty_batch_is_a_no_op(L):
    assert route(L, T=0, x=None, lo=None, ids=None, w=None, ws=None, ws_bytes=0) == MOE_OK
    assert L.moe_combine(None, None, None, 0, 8, 256, BF16, None, None) == MOE_OK
    assert L.moe_grouped_gemm(None, None, None, 0, 8, 16, None, None, 256, 128, BF16, None, None, 0,
                              None) == MOE_OK


@pytest.mark.parametrize("args,status", [
    ((FAKE, 4, 0, 0, 8), MOE_EINVAL),        # kk = 0
    ((FAKE, 4, 65, 0, 8), MOE_EINVAL),       # kk > 64
    ((FAKE, 4, 2, -1, 8), MOE_EINVAL),       # negative window
    ((FAKE, 4, 2, 0, 0), MOE_EINVAL),        # no groups
    ((FAKE, 4, 2, 0, 513), MOE_EUNSUPPORTED),
    ((None, 4, 2, 0, 8), MOE_EINVAL),
])
def test_permute_rejects(L, args, status):
    assert L.moe_permute(*args, FAKE, FAKE, FAKE, FAKE, None) == status


def test_permute_rejects_null_outputs(L):
    assert L.moe_permute(FAKE, 4, 2, 0, 8, None, FAKE, FAKE, FAKE, None) == MOE_EINVAL
    assert L.moe_permute(FAKE, 4, 2, 0, 8, FAKE, FAKE, FAKE, MISALIGNED + 1, None) == MOE_EINVAL


def gg(L, T=4, kk=2, G=8, H=256, I=128, dt=BF16, ws=FAKE, ws_bytes=1 << 30, w13=FAKE, x=FAKE):
    return L.moe_grouped_gemm(x, FAKE, FAKE, T, kk, G, w13, FAKE, H, I, dt, FAKE, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(ws_bytes=4 * 2 * 128 * 2 - 1), MOE_EWORKSPACE),
    (dict(ws=None), MOE_EWORKSPACE),
    (dict(ws=MISALIGNED), MOE_EWORKSPACE),
    (dict(I=120), MOE_EUNSUPPORTED),          # bf16 I must be whole 64-byte chunks (I % 32)
    (dict(H=240), MOE_EUNSUPPORTED),
    (dict(G=600), MOE_EUNSUPPORTED),
    (dict(H=0), MOE_EINVAL),
    (dict(w13=None), MOE_EINVAL),
    (dict(w13=MISALIGNED), MOE_EINVAL),
    (dict(dt=3), MOE_EINVAL),
])
def test_grouped_gemm_rejects(L, kw, status):
    assert gg(L, **kw) == status


def test_expert_halves_reject(L):
    up = lambda **kw: L.moe_expert_up(FAKE, FAKE, FAKE, 4, 2, 8, FAKE, 256, 128, BF16, kw.get("a", FAKE),
                                      kw.get("ws", FAKE), kw.get("ws_bytes", 1 << 30), None)
    assert up(a=None) == MOE_EINVAL
    assert up(ws=None) == MOE_EWORKSPACE
    assert up(ws=MISALIGNED) == MOE_EWORKSPACE
    assert up(ws_bytes=16) == MOE_EWORKSPACE
    assert L.moe_expert_down(FAKE, FAKE, 4, 2, 8, FAKE, 256, 100, BF16, FAKE, FAKE, 1 << 30,
                             None) == MOE_EUNSUPPORTED
    assert L.moe_expert_down(FAKE, FAKE, 4, 2, 8, FAKE, 256, 128, BF16, FAKE, None, 1 << 30,
                             None) == MOE_EWORKSPACE


def test_combine_rejects(L):
    assert L.moe_combine(FAKE, FAKE, FAKE, 4, 0, 256, BF16, FAKE, None) == MOE_EINVAL
    assert L.moe_combine(FAKE, FAKE, FAKE, 4, 2, 260, BF16, FAKE, None) == MOE_EUNSUPPORTED
    assert L.moe_combine(FAKE, None, FAKE, 4, 2, 256, BF16, FAKE, None) == MOE_EINVAL
    assert L.moe_combine(MISALIGNED, FAKE, FAKE, 4, 2, 256, BF16, FAKE, None) == MOE_EINVAL
    assert L.moe_combine(FAKE, FAKE, MISALIGNED, 4, 2, 256, BF16, FAKE, None) == MOE_EINVAL
    assert L.moe_combine(FAKE, FAKE, None, 4, 2, 260, BF16, FAKE, None) == MOE_EUNSUPPORTED


def disp(L, x=FAKE, ids=FAKE, T=4, kk=2, H=256, E_l=2, P=4, dt=BF16, counts=FAKE, offsets=FAKE,
         order=FAKE, pos=FAKE, send_x=FAKE, send_ids=FAKE):
    return L.moe_dispatch(x, ids, T, kk, H, E_l, P, dt, counts, offsets, order, pos, send_x, send_ids,
                          None)


@pytest.mark.parametrize("kw,status", [
    (dict(kk=0), MOE_EINVAL),
    (dict(kk=65), MOE_EINVAL),
    (dict(E_l=0), MOE_EINVAL),
    (dict(P=0), MOE_EINVAL),
    (dict(P=513), MOE_EUNSUPPORTED),
    (dict(E_l=1 << 30, P=4), MOE_EUNSUPPORTED),   # expert ids past 2^31
    (dict(T=-1), MOE_EINVAL),
    (dict(H=0), MOE_EINVAL),
    (dict(H=260), MOE_EUNSUPPORTED),           # bf16 rows must be whole 16-byte vectors
    (dict(dt=2), MOE_EINVAL),
    (dict(counts=None), MOE_EINVAL),
    (dict(offsets=MISALIGNED), MOE_EINVAL),
    (dict(x=None), MOE_EINVAL),
    (dict(x=MISALIGNED), MOE_EINVAL),
    (dict(send_x=MISALIGNED + 4), MOE_EINVAL),
    (dict(send_ids=None), MOE_EINVAL),
    (dict(order=MISALIGNED + 1), MOE_EINVAL),
    (dict(ids=FAKE + 4), MOE_EINVAL),          # the id sweep reads 16-byte vectors
])
def test_dispatch_rejects(L, kw, status):
    assert disp(L, **kw) == status


def ptrs(*vals):
    return (ctypes.c_void_p * len(vals))(*vals)


def test_repack_rejects(L):
    d = ptrs(FAKE, FAKE)
    assert L.moe_repack_ep_to_tp(FAKE, FAKE, 2, 256, 100, 3, BF16, d, d, None) == MOE_EINVAL  # I % P
    assert L.moe_repack_ep_to_tp(FAKE, FAKE, 2, 256, 128, 0, BF16, d, d, None) == MOE_EINVAL
    assert L.moe_repack_ep_to_tp(FAKE, FAKE, 2, 256, 8 * 65, 65, BF16, d, d, None) == MOE_EUNSUPPORTED
    assert L.moe_repack_ep_to_tp(FAKE, FAKE, 2, 256, 12, 2, BF16, d, d, None) == MOE_EUNSUPPORTED  # 6*2 B
    assert L.moe_repack_ep_to_tp(FAKE, FAKE, 2, 256, 128, 2, BF16, ptrs(FAKE, None), d, None) == MOE_EINVAL
    assert L.moe_repack_ep_to_tp(FAKE, FAKE, 2, 256, 128, 2, BF16, ptrs(FAKE, MISALIGNED), d,
                                 None) == MOE_EINVAL
    assert L.moe_repack_ep_to_tp(None, FAKE, 2, 256, 128, 2, BF16, d, d, None) == MOE_EINVAL


def test_repack_tp_to_ep_rejects(L):
    d = ptrs(FAKE, FAKE)
    assert L.moe_repack_tp_to_ep(d, d, 2, 256, 100, 3, BF16, FAKE, FAKE, None) == MOE_EINVAL  # I % P
    assert L.moe_repack_tp_to_ep(d, d, 2, 256, 128, 0, BF16, FAKE, FAKE, None) == MOE_EINVAL
    assert L.moe_repack_tp_to_ep(d, d, 2, 256, 8 * 65, 65, BF16, FAKE, FAKE, None) == MOE_EUNSUPPORTED
    assert L.moe_repack_tp_to_ep(d, d, 2, 256, 12, 2, BF16, FAKE, FAKE, None) == MOE_EUNSUPPORTED  # 6*2 B
    assert L.moe_repack_tp_to_ep(ptrs(FAKE, None), d, 2, 256, 128, 2, BF16, FAKE, FAKE, None) == MOE_EINVAL
    assert L.moe_repack_tp_to_ep(d, ptrs(MISALIGNED, FAKE), 2, 256, 128, 2, BF16, FAKE, FAKE, None) == MOE_EINVAL
    assert L.moe_repack_tp_to_ep(None, d, 2, 256, 128, 2, BF16, FAKE, FAKE, None) == MOE_EINVAL
    assert L.moe_repack_tp_to_ep(d, d, 2, 256, 128, 2, BF16, None, FAKE, None) == MOE_EINVAL
    assert L.moe_repack_tp_to_ep(d, d, 2, 256, 128, 2, BF16, FAKE, MISALIGNED, None) == MOE_EINVAL


def test_schedule_rejects(L):
    sch = lambda **kw: L.moe_schedule_requests(
        kw.get("tok", FAKE), kw.get("nt", 100), kw.get("off", FAKE), kw.get("nr", 10), kw.get("cl", FAKE),
        kw.get("V", 1000), kw.get("E", 8), kw.get("sc", FAKE), FAKE, FAKE, kw.get("ws", FAKE),
        kw.get("wsb", 1 << 20), None)
    assert sch(E=0) == MOE_EINVAL
    assert sch(E=65) == MOE_EUNSUPPORTED
    assert sch(nt=1 << 25) == MOE_EUNSUPPORTED
    assert sch(V=0) == MOE_EINVAL
    assert sch(nr=-1) == MOE_EINVAL
    assert sch(nr=0) == MOE_OK                       # nothing to do, nothing launched
    assert sch(off=None) == MOE_EINVAL
    assert sch(tok=None) == MOE_EINVAL
    assert sch(sc=MISALIGNED) == MOE_EINVAL
    assert sch(ws=None) == MOE_EWORKSPACE
    assert sch(wsb=4) == MOE_EWORKSPACE
    assert L.moe_schedule_workspace_bytes(10, 8) == 256
    assert L.moe_schedule_workspace_bytes(0, 8) == 0
