"""C-ABI checks that need no GPU: the library loads, exports what include/m3.h
declares, plans chunks exactly, and rejects bad arguments before any HIP call.

Pointers here are fake, 16-byte aligned addresses: every call below fails
validation, which never dereferences them.
"""
import ctypes
import math
import os
import re

import pytest

from mamba_ssm_scan_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIB_PATH):
        from mamba_ssm_scan_amd import build
        build.build()
    return bd.load()


def header_functions():
    text = open(os.path.join(ROOT, "include", "m3.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(m3_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert set(names) == set(bd.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version(lib):
    assert lib.m3_abi_version() == 1
    assert lib.m3_status_string(0) == b"ok"
    assert lib.m3_status_string(6) == b"HIP runtime error"


def _dims(b=1, L=100, H=4, G=1, P=8, N=16):
    return bd.dims(b, L, H, G, P, N)


@pytest.mark.parametrize("L", [0, 1, 15, 16, 17, 64, 127, 128, 129, 2048, 32768, 33024])
@pytest.mark.parametrize("chunk", [1, 3, 16, 64, 100, 4096])
def test_plan_integers(lib, L, chunk):
    p = bd.plan(_dims(L=L), 1, chunk, bd.M3_F32)
    n = math.ceil(L / chunk)
    assert p.n_chunks == n
    assert p.last_chunk_len == (0 if L == 0 else L - (n - 1) * chunk)
    assert 1 <= p.segments
    assert p.segments * p.chunks_per_segment >= n
    assert (p.segments - 1) * p.chunks_per_segment < max(n, 1)


def test_plan_generic_workspace(lib):
    d = _dims(b=3, H=4, P=8, N=16)
    p = bd.plan(d, 2, 16, bd.M3_F32)
    assert p.path == bd.M3_PATH_GENERIC
    assert p.workspace_bytes >= 3 * 4 * 16 * 8 * 4
    assert lib.m3_prefill_workspace_size(ctypes.byref(d), 2, 16, bd.M3_F32) == p.workspace_bytes


@pytest.mark.parametrize("N,P,R,io,path", [
    (128, 64, 1, "bf16", "MFMA"), (128, 64, 4, "bf16", "MFMA"), (128, 64, 3, "bf16", "MFMA"),
    (128, 64, 5, "bf16", "MFMA"), (120, 64, 5, "bf16", "GENERIC"), (128, 72, 6, "bf16", "GENERIC"),
    (256, 64, 1, "bf16", "MFMA"), (128, 64, 8, "bf16", "MFMA"), (256, 32, 6, "bf16", "SCAN"),
    (256, 64, 8, "bf16", "SCAN"), (128, 32, 8, "bf16", "SCAN"), (128, 64, 7, "bf16", "MFMA"),
    (64, 64, 6, "bf16", "SCAN"), (128, 64, 6, "bf16", "MFMA"),
    (256, 64, 3, "bf16", "MFMA"), (512, 64, 4, "bf16", "MFMA"), (520, 64, 1, "bf16", "GENERIC"),
    (128, 64, 9, "bf16", "GENERIC"), (272, 64, 1, "bf16", "MFMA"), (128, 72, 1, "bf16", "MFMA"),
    (120, 64, 1, "bf16", "MFMA"), (64, 64, 2, "bf16", "MFMA"), (8, 64, 4, "bf16", "MFMA"),
    (64, 64, 3, "bf16", "MFMA"), (64, 32, 1, "bf16", "MFMA"), (100, 64, 1, "bf16", "GENERIC"),
    (128, 36, 1, "bf16", "GENERIC"), (128, 1024, 2, "bf16", "MFMA"), (128, 1032, 1, "bf16", "GENERIC"),
    (256, 64, 8, "f32", "GENERIC")])
def test_plan_path_choice(lib, N, P, R, io, path):
    """Which kernel family takes a shape; the token-walk path needs no workspace."""
    p = bd.plan(_dims(b=2, H=4, P=P, N=N), R, 64, bd.M3_BF16 if io == "bf16" else bd.M3_F32)
    assert p.path == getattr(bd, "M3_PATH_" + path)
    if path == "SCAN":
        assert p.workspace_bytes == 0 and p.segments == 1
    if path == "MFMA" and R > 4:  # chunks of at most 32 tokens, no sequence segments
        assert p.segments == 1 and p.n_chunks == (100 + 31) // 32 and p.last_chunk_len == 100 - 3 * 32


FAKE = 1 << 40  # never dereferenced


def _call(lib, d, R=1, chunk=16, io=bd.M3_F32, **over):
    # disjoint fake regions, 1 GiB apart
    names = ["x", "dt", "A", "omega", "lam", "B", "C", "D", "h0", "y", "h_out", "cB", "cx", "ws"]
    ptr = {n: FAKE + i * (1 << 30) for i, n in enumerate(names)}
    ptr["h0"] = ptr["cB"] = ptr["cx"] = None
    ptr["ws"] = None
    ptr.update(over)
    v = lambda n: None if ptr[n] is None else ctypes.c_void_p(ptr[n])
    ws_bytes = over.get("ws_bytes", 0)
    dp = None if d is None else ctypes.byref(d)
    st = lib.m3_prefill(v("x"), v("dt"), v("A"), v("omega"), v("lam"), v("B"), v("C"), v("D"), R, chunk,
                        v("h0"), v("y"), v("h_out"), dp, io, v("cB"), v("cx"), v("ws"), ws_bytes, None)
    return st, lib.m3_last_error().decode()


def test_prefill_argument_errors(lib):
    assert _call(lib, None)[0] == 1
    assert _call(lib, _dims(N=15))[0] == 1                       # odd state dim
    assert _call(lib, _dims(N=0))[0] == 1
    assert _call(lib, _dims(H=4, G=3))[0] == 1                   # G does not divide H
    assert _call(lib, _dims(), R=0)[0] == 1
    assert _call(lib, _dims(), chunk=0)[0] == 1
    assert _call(lib, _dims(), chunk=4097)[0] == 5
    assert _call(lib, _dims(), io=7)[0] == 3
    st, msg = _call(lib, _dims(), x=None)
    assert st == 1 and "x" in msg
    assert _call(lib, _dims(), cB=FAKE + 50 * (1 << 30))[0] == 1  # carry_B without carry_x
    st, msg = _call(lib, _dims(), B=FAKE + 5 * (1 << 30) + 8)
    assert st == 4 and "B" in msg                                  # misaligned
    st, msg = _call(lib, _dims(), y=FAKE + 16)                     # y inside x
    assert st == 1 and "overlaps x" in msg
    st, msg = _call(lib, _dims(), h_out=FAKE + 6 * (1 << 30) + 32)  # h_out inside C
    assert st == 1 and "h_out" in msg
    # the generic path needs a workspace
    st, msg = _call(lib, _dims())
    assert st == 7, msg
    d = _dims()
    need = lib.m3_prefill_workspace_size(ctypes.byref(d), 1, 16, bd.M3_F32)
    st, msg = _call(lib, d, ws=FAKE + 20 * (1 << 30), ws_bytes=need - 1)
    assert st == 7
    st, msg = _call(lib, d, ws=FAKE + 20 * (1 << 30) + 16, ws_bytes=need)
    assert st == 4 and "workspace" in msg


def test_prefill_fused_argument_errors(lib):
    """m3_prefill_fused: m3_prefill's checks, plus dt_bias (16-byte aligned, not under y)."""
    d = _dims()
    v = ctypes.c_void_p

    def call(dtb=None, y=FAKE + 9 * (1 << 30), x=FAKE):
        return lib.m3_prefill_fused(v(x) if x else None, v(FAKE + (1 << 30)), v(dtb) if dtb else None,
                                    v(FAKE + (2 << 30)), None, None, v(FAKE + (5 << 30)), v(FAKE + (6 << 30)),
                                    v(FAKE + (7 << 30)), 1, 16, None, v(y), None, ctypes.byref(d), bd.M3_F32, None,
                                    None, None, 0, None)
    assert call(x=None) == 1
    assert call(dtb=FAKE + 14 * (1 << 30) + 8) == 4                      # misaligned bias
    assert "dt_bias" in lib.m3_last_error().decode()
    assert call(dtb=FAKE + 9 * (1 << 30) + 64) == 1                      # bias inside y
    assert "dt_bias" in lib.m3_last_error().decode()
    assert call(dtb=FAKE + 14 * (1 << 30)) == 7                          # valid: the generic path needs a workspace


def test_noalloc_rejects_before_any_launch(lib):
    """m3_prefill_noalloc: same argument checks as m3_prefill; sizes whose workspace
    exceeds the fixed scratch are refused (M3_EWORKSPACE) before any HIP call."""
    assert lib.m3_noalloc_scratch_bytes() == 32 << 20
    def call(d, R=1, chunk=64, io=bd.M3_BF16, x=FAKE):
        return lib.m3_prefill_noalloc(x, FAKE + (1 << 30), FAKE + (2 << 30), None, None, FAKE + (3 << 30),
                                      FAKE + (4 << 30), FAKE + (5 << 30), R, chunk, None, FAKE + (6 << 30), None,
                                      ctypes.byref(d), io, None, None, None)
    assert call(_dims(N=15)) == 1
    assert call(_dims(), x=None) == 1
    # N 256 takes two row passes whose fp32 partial outputs need b*L*H*R*P*4 bytes: 48 MiB here
    d = bd.dims(1, 8192, 24, 1, 64, 256)
    assert lib.m3_prefill_workspace_size(ctypes.byref(d), 1, 64, bd.M3_BF16) > (32 << 20)
    assert call(d) == 7
    assert "scratch" in lib.m3_last_error().decode()


def test_prefill_check_without_segments_needs_no_gpu(lib):
    """m3_prefill_check returns M3_OK at once (no HIP call) when the plan has one segment,
    and rejects bad sizes like the other entry points."""
    d = bd.dims(4, 2048, 64, 1, 64, 128)
    assert bd.plan(d, 4, 64, bd.M3_BF16).segments == 1
    assert lib.m3_prefill_check(ctypes.byref(d), 4, 64, bd.M3_BF16, None, 0, None) == 0
    assert lib.m3_prefill_check(ctypes.byref(_dims(N=15)), 1, 64, bd.M3_BF16, None, 0, None) == 1
    assert lib.m3_status_string(8) == b"a sequence-segment look-back gave up; outputs not valid"
    # a segmented plan with a workspace smaller than the plan's is refused before any HIP call
    d4 = bd.dims(1, 32768, 64, 1, 64, 128)
    p4 = bd.plan(d4, 4, 64, bd.M3_BF16)
    assert p4.segments > 1
    assert lib.m3_prefill_check(ctypes.byref(d4), 4, 64, bd.M3_BF16, ctypes.c_void_p(FAKE),
                                p4.workspace_bytes - 1, None) == 7


def test_prefill_empty_batch_is_a_no_op(lib):
    # b = 0: valid, nothing to launch
    assert _call(lib, _dims(b=0))[0] == 0


def test_decode_argument_errors(lib):
    st = bd.M3DecodeState()
    d = _dims()
    f = lambda i: ctypes.c_void_p(FAKE + i * (1 << 30))
    assert lib.m3_decode_state_init(None, ctypes.byref(d), 1, 0, f(0), f(1), f(2), None, None, None, 0, None) == 1
    bad = _dims(N=9)
    assert lib.m3_decode_state_init(ctypes.byref(st), ctypes.byref(bad), 1, 0, f(0), f(1), f(2), None, None, None,
                                    0, None) == 1
    assert lib.m3_decode_state_init(ctypes.byref(st), ctypes.byref(d), 1, 0, f(0), f(1), f(2), None, f(3), None,
                                    0, None) == 1          # B_last without x_last
    assert lib.m3_decode_state_init(ctypes.byref(st), ctypes.byref(d), 1, 0, f(0), f(1), f(2), None, None, None,
                                    -1, None) == 1
    assert lib.m3_decode_state_init(ctypes.byref(st), ctypes.byref(d), 1, 0, ctypes.c_void_p(FAKE + 4), f(1), f(2),
                                    None, None, None, 0, None) == 4
    # a state bound by hand (no HIP call): a step with another rank is a shape error
    st.h, st.carry_B, st.carry_x, st.t = FAKE, FAKE + (1 << 30), FAKE + 2 * (1 << 30), 5
    st.dims, st.R, st.io_dtype = d, 2, 0
    args = [f(10 + i) for i in range(8)]
    assert lib.m3_decode_step(ctypes.byref(st), *args, 1, f(30), None) == 2
    assert lib.m3_decode_step(ctypes.byref(st), *args[:7], None, 2, f(30), None) == 1   # D NULL
    assert lib.m3_decode_step(ctypes.byref(st), *args, 2, ctypes.c_void_p(FAKE + 10 * (1 << 30) + 64), None) == 1
    assert st.t == 5                                  # failed steps do not advance the counter
    # the fused step: the same checks, plus its prologue arguments
    fused = lambda R=2, eps=1e-6, D=f(17), dtb=None: lib.m3_decode_step_fused(
        ctypes.byref(st), f(10), f(11), dtb, f(12), f(13), f(14), f(15), f(16), None, None, None, None,
        ctypes.c_float(eps), D, R, f(30), None)
    assert fused(R=1) == 2
    assert fused(eps=-1.0) == 1
    assert fused(D=None) == 1
    assert fused(dtb=ctypes.c_void_p(FAKE + 8)) == 4
    big = bd.M3DecodeState()
    big.h, big.carry_B, big.carry_x, big.t = FAKE, FAKE + (1 << 30), FAKE + 2 * (1 << 30), 0
    big.dims, big.R, big.io_dtype = _dims(N=4096), 4, 0  # R * N = 16384 rows of LDS: unsupported
    assert lib.m3_decode_step_fused(ctypes.byref(big), f(10), f(11), None, f(12), f(13), f(14), f(15), f(16), None,
                                    None, None, None, ctypes.c_float(1e-6), f(17), 4, f(30), None) == 5
    assert st.t == 5 and big.t == 0


def test_carry_bytes(lib):
    # B: two slots [2][b][G][R][N] (to a 16-byte boundary), then a 32-bit parity word per (b, h);
    # x: [b][H][R][P]
    d = _dims(b=3, H=4, G=2, P=8, N=16)
    assert lib.m3_decode_carry_bytes(ctypes.byref(d), 2, bd.M3_BF16, 0) == 2 * 3 * 2 * 2 * 16 * 2 + 3 * 4 * 4
    assert lib.m3_decode_carry_bytes(ctypes.byref(d), 2, bd.M3_BF16, 1) == 3 * 4 * 2 * 8 * 2
    d = _dims(b=1, H=3, G=1, P=8, N=2)   # slots of 2 * 1 * 1 * 1 * 2 * 4 = 16 bytes (f32)
    assert lib.m3_decode_carry_bytes(ctypes.byref(d), 1, bd.M3_F32, 0) == 16 + 3 * 4
    d = _dims(b=1, H=3, G=1, P=8, N=2)   # 8 bytes of bf16 slots, padded to 16
    assert lib.m3_decode_carry_bytes(ctypes.byref(d), 1, bd.M3_BF16, 0) == 16 + 3 * 4


def test_plan_segments_for_few_heads(lib):
    # b*H = 64 walks over 512 chunks: split into segments so every CU has one
    d = bd.dims(1, 32768, 64, 1, 64, 128)
    p = bd.plan(d, 4, 64, bd.M3_BF16)
    assert p.path == bd.M3_PATH_MFMA
    assert p.segments == 4 and p.chunks_per_segment == 128
    assert p.workspace_bytes >= 2 * 64 * 4 * 128 * 64 * 4
    # enough walks already: one segment, no workspace
    p1 = bd.plan(bd.dims(4, 2048, 64, 1, 64, 128), 4, 64, bd.M3_BF16)
    assert p1.segments == 1 and p1.workspace_bytes == 0
    # the R=1 kernel walks whole sequences
    assert bd.plan(d, 1, 64, bd.M3_BF16).segments == 1


def test_omega_lambda_may_be_null(lib):
    # omega NULL (omega = 0) and lambda NULL (lambda = 1) pass validation: the
    # prefill call gets as far as the workspace check, the decode step as far as
    # the overlap check (both run before any HIP call)
    st, msg = _call(lib, _dims(), omega=None, lam=None)
    assert st == 7, msg
    s = bd.M3DecodeState()
    s.h, s.carry_B, s.carry_x, s.t = FAKE, FAKE + (1 << 30), FAKE + 2 * (1 << 30), 0
    s.dims, s.R, s.io_dtype = _dims(), 1, 0
    f = lambda i: ctypes.c_void_p(FAKE + i * (1 << 30))
    y_in_x = ctypes.c_void_p(FAKE + 10 * (1 << 30) + 64)
    assert lib.m3_decode_step(ctypes.byref(s), f(10), f(11), f(12), None, None, f(15), f(16), f(17), 1,
                              y_in_x, None) == 1
    assert "y_t overlaps" in lib.m3_last_error().decode()


def _prologue(lib, d, R=1, io=bd.M3_F32, ntok=10, eps=1e-6, **over):
    names = ["B_raw", "C_raw", "B_weight", "B_bias", "C_weight", "C_bias", "dt_raw", "dt_bias", "lambda_raw",
             "B", "C", "dt", "lambda"]
    ptr = {n: FAKE + i * (1 << 30) for i, n in enumerate(names)}
    ptr.update(over)
    v = lambda n: None if ptr[n] is None else ctypes.c_void_p(ptr[n])
    dp = None if d is None else ctypes.byref(d)
    st = lib.m3_prologue(dp, R, io, ntok, v("B_raw"), v("C_raw"), v("B_weight"), v("B_bias"), v("C_weight"),
                         v("C_bias"), ctypes.c_float(eps), v("dt_raw"), v("dt_bias"), v("lambda_raw"), v("B"), v("C"),
                         v("dt"), v("lambda"), None)
    return st, lib.m3_last_error().decode()


def test_prologue_argument_errors(lib):
    assert _prologue(lib, None)[0] == 1
    assert _prologue(lib, _dims(N=7))[0] == 1
    assert _prologue(lib, _dims(), R=0)[0] == 1
    assert _prologue(lib, _dims(), io=9)[0] == 3
    assert _prologue(lib, _dims(), ntok=-1)[0] == 1
    assert _prologue(lib, _dims(), eps=-1.0)[0] == 1
    assert _prologue(lib, _dims(), eps=float("nan"))[0] == 1
    st, msg = _prologue(lib, _dims(), B=None)                      # B_raw without B
    assert st == 1 and "B_raw" in msg
    st, msg = _prologue(lib, _dims(), dt_raw=None)                 # dt without dt_raw
    assert st == 1 and "dt" in msg
    st, msg = _prologue(lib, _dims(), C_raw=None, C=None)          # C weight without C
    assert st == 1 and "C_weight" in msg
    st, msg = _prologue(lib, _dims(), dt_raw=None, dt=None)        # dt_bias without dt
    assert st == 1 and "dt_bias" in msg
    st, msg = _prologue(lib, _dims(), C=FAKE + 1 * (1 << 30) + 8)  # misaligned
    assert st == 4 and "C" in msg
    st, msg = _prologue(lib, _dims(), B=FAKE + 16)                 # B inside B_raw, not in place
    assert st == 1 and "B overlaps B_raw" in msg
    st, msg = _prologue(lib, _dims(), dt=FAKE + 8 * (1 << 30))     # dt on lambda_raw
    assert st == 1 and "dt overlaps lambda_raw" in msg
    st, msg = _prologue(lib, _dims(), lam=None, **{"lambda": FAKE + 11 * (1 << 30)})  # lambda on dt
    assert st == 1 and "overlaps" in msg


def test_prologue_in_place_and_empty_pass_checks(lib):
    # outputs on their own inputs are allowed; with ntok = 0 nothing is launched
    same = {"B": FAKE, "C": FAKE + (1 << 30), "dt": FAKE + 6 * (1 << 30), "lambda": FAKE + 8 * (1 << 30)}
    assert _prologue(lib, _dims(), ntok=0, **same)[0] == 0
    assert _prologue(lib, _dims(), ntok=0)[0] == 0
    # nothing given at all is a valid no-op
    none = {n: None for n in ["B_raw", "C_raw", "B_weight", "B_bias", "C_weight", "C_bias", "dt_raw", "dt_bias",
                              "lambda_raw", "B", "C", "dt", "lambda"]}
    assert _prologue(lib, _dims(), **none)[0] == 0


def _backward(lib, d, R=1, io=bd.M3_F32, ws_bytes=None, **over):
    names = ["x", "dt", "A", "omega", "lam", "B", "C", "D", "h0", "cB", "cx", "dy", "dh", "dx", "dB", "dC", "ddt",
             "dlam", "dA", "domega", "dD", "dh0", "dcB", "dcx", "ws"]
    ptr = {n: FAKE + i * (1 << 30) for i, n in enumerate(names)}
    ptr["h0"] = ptr["cB"] = ptr["cx"] = ptr["dh"] = ptr["dcB"] = ptr["dcx"] = None
    ptr.update(over)
    v = lambda n: None if ptr[n] is None else ctypes.c_void_p(ptr[n])
    if ws_bytes is None:
        ws_bytes = 0 if d is None else lib.m3_prefill_backward_workspace_size(ctypes.byref(d), R)
    dp = None if d is None else ctypes.byref(d)
    st = lib.m3_prefill_backward(v("x"), v("dt"), v("A"), v("omega"), v("lam"), v("B"), v("C"), v("D"), R, v("h0"),
                                 v("cB"), v("cx"), v("dy"), v("dh"), v("dx"), v("dB"), v("dC"), v("ddt"), v("dlam"),
                                 v("dA"), v("domega"), v("dD"), v("dh0"), v("dcB"), v("dcx"), dp, io, v("ws"),
                                 ws_bytes, None)
    return st, lib.m3_last_error().decode()


def test_backward_argument_errors(lib):
    d = _dims()
    assert lib.m3_prefill_backward_workspace_size(ctypes.byref(d), 1) > 0
    assert lib.m3_prefill_backward_workspace_size(ctypes.byref(_dims(N=256)), 1) == 0   # unsupported
    assert _backward(lib, None)[0] == 1
    assert _backward(lib, _dims(N=256))[0] == 5
    assert _backward(lib, _dims(P=65))[0] == 5
    assert _backward(lib, _dims(), R=5)[0] == 5
    assert _backward(lib, _dims(P=7), io=bd.M3_BF16)[0] == 5                  # odd P with bf16
    st, msg = _backward(lib, _dims(), dy=None)
    assert st == 1 and "dy" in msg
    st, msg = _backward(lib, _dims(), cB=FAKE + 40 * (1 << 30))
    assert st == 1 and "carry" in msg
    st, msg = _backward(lib, _dims(), dcB=FAKE + 40 * (1 << 30), dcx=FAKE + 41 * (1 << 30))
    assert st == 1 and "without a carry" in msg
    st, msg = _backward(lib, _dims(), dB=FAKE + 14 * (1 << 30) + 8)
    assert st == 4 and "dB" in msg
    st, msg = _backward(lib, _dims(), dC=FAKE + 14 * (1 << 30))          # dC on dB
    assert st == 1 and "overlaps" in msg
    st, msg = _backward(lib, _dims(), dx=FAKE + 16)                      # dx inside x
    assert st == 1 and "dx overlaps x" in msg
    st, msg = _backward(lib, _dims(), ws_bytes=16)
    assert st == 7 and "workspace" in msg
    # no tokens: valid, nothing launched
    assert _backward(lib, _dims(b=0))[0] == 0


def _mixer_weights(**over):
    names = ["W_x", "W_z", "W_B", "W_C", "W_dt", "W_lambda", "W_out", "B_weight", "B_bias", "C_weight", "C_bias",
             "dt_bias", "A", "omega", "D"]
    ptr = {n: FAKE + (60 + i) * (1 << 30) for i, n in enumerate(names)}
    ptr.update({k: v for k, v in over.items() if k in ptr})
    return bd.M3MixerWeights(over.get("d_model", 64), *[ptr[n] for n in names], over.get("eps", 1e-6))


def test_mixer_argument_errors(lib):
    """Every check of m3_mixer_prefill / m3_mixer_decode_step runs before the mixer object is used."""
    d = _dims(b=2, L=10, H=2, P=16, N=32)
    need = lib.m3_mixer_workspace_size(ctypes.byref(d), 1, 64, 64)
    assert need > 0
    assert lib.m3_mixer_workspace_size(ctypes.byref(_dims(N=15)), 1, 64, 64) == 0
    assert lib.m3_mixer_workspace_size(ctypes.byref(d), 1, 64, 0) == 0
    ws, u, out = ctypes.c_void_p(FAKE + 90 * (1 << 30)), ctypes.c_void_p(FAKE + 91 * (1 << 30)), \
        ctypes.c_void_p(FAKE + 92 * (1 << 30))

    def pre(w, dims=d, ws_bytes=need):
        st = lib.m3_mixer_prefill(None, None if w is None else ctypes.byref(w), ctypes.byref(dims), 1, 64, u, out,
                                  None, None, None, ws, ws_bytes, None)
        return st, lib.m3_last_error().decode()

    assert pre(None)[0] == 1
    st, msg = pre(_mixer_weights(W_x=None))
    assert st == 1 and "W_x" in msg
    assert pre(_mixer_weights(d_model=0))[0] == 1
    assert pre(_mixer_weights(eps=-1.0))[0] == 1
    assert pre(_mixer_weights(), dims=_dims(N=15))[0] == 1
    st, msg = pre(_mixer_weights(), ws_bytes=need - 1)
    assert st == 7 and "workspace" in msg
    st, msg = pre(_mixer_weights())                     # everything else valid
    assert st == 1 and "mixer" in msg
    # decode step: the state is checked first
    st = lib.m3_mixer_decode_step(None, ctypes.byref(_mixer_weights()), None, u, out, ws, need, None)
    assert st == 1 and "state" in lib.m3_last_error().decode()
    s = bd.M3DecodeState()
    s.R, s.io_dtype, s.dims = 1, bd.M3_F32, _dims(b=2, L=1, H=2, P=16, N=32)
    assert lib.m3_mixer_decode_step(None, ctypes.byref(_mixer_weights()), ctypes.byref(s), u, out, ws, need,
                                    None) == 3
