"""Host-only checks of the C ABI: the library loads, exports what include/kda.h
declares, and rejects bad arguments before touching the GPU (no compute calls)."""
import ctypes
import os
import subprocess

import pytest

import gated_delta_rule_chunk_amd as kda

FAKE = ctypes.c_void_p(0x1000)     # never dereferenced: every call below is rejected on the host


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIB_PATH):
        from gated_delta_rule_chunk_amd import _build
        _build.build()
    return kda.load_library()


def test_exports_every_declared_symbol(lib):
    names = kda.declared_symbols()
    assert set(names) == {"kda_chunk_fwd", "kda_chunk_fwd_prologue", "kda_recurrent_step", "kda_short_conv",
                          "kda_recurrent_step_prologue", "kda_recurrent_step_conv", "kda_chunk_bwd_conv",
                          "kda_chunk_fwd_split_prologue", "kda_prologue",
                          "kda_chunk_bwd_conv_workspace_bytes",
                          "kda_short_conv_step", "kda_chunk_bwd", "kda_chunk_bwd_workspace_bytes",
                          "kda_chunk_fwd_split", "kda_chunk_fwd_split_workspace_bytes",
                          "kda_chunk_fwd_split_static", "kda_chunk_fwd_conv", "kda_chunk_fwd_conv_workspace_bytes",
                          "kda_chunk_bwd_prologue", "kda_chunk_bwd_prologue_workspace_bytes",
                          "kda_short_conv_bwd", "kda_short_conv_bwd_workspace_bytes",
                          "kda_status_string", "kda_last_error_message", "kda_device_check",
                          "kda_set_wait_limit"}
    out = subprocess.run(["nm", "-D", "--defined-only", kda.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_status_strings(lib):
    assert lib.kda_status_string(0) == b"KDA_OK"
    assert lib.kda_status_string(1) == b"KDA_ERR_INVALID_ARG"
    assert lib.kda_status_string(2) == b"KDA_ERR_UNSUPPORTED"
    assert lib.kda_status_string(3) == b"KDA_ERR_HIP"
    assert lib.kda_status_string(4) == b"KDA_ERR_DEVICE"


def test_set_wait_limit_rejects_negative(lib):
    assert lib.kda_set_wait_limit(-1) == kda.KDA_ERR_INVALID_ARG
    assert "polls" in lib.kda_last_error_message().decode()
    assert lib.kda_set_wait_limit(1 << 22) == kda.KDA_OK


def _fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s0=None, cu=None, B=1, T=64, H=2, Dk=128,
             Dv=128, N=1, chunk=64, scale=1.0, dtype=kda.KDA_BF16, o=ctypes.c_void_p(0x2000),
             sT=None, stream=None)
    a.update(kw)
    return lib.kda_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["cu"], a["B"],
                             a["T"], a["H"], a["Dk"], a["Dv"], a["N"], a["chunk"], a["scale"],
                             a["dtype"], a["o"], a["sT"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), kda.KDA_ERR_INVALID_ARG, "non-NULL"),
    (dict(T=0, q=None, B=0), kda.KDA_ERR_INVALID_ARG, "B >= 1"),
    (dict(o=None), kda.KDA_ERR_INVALID_ARG, "non-NULL"),
    (dict(B=0), kda.KDA_ERR_INVALID_ARG, "B >= 1"),
    (dict(T=-1), kda.KDA_ERR_INVALID_ARG, "T >= 0"),
    (dict(H=0), kda.KDA_ERR_INVALID_ARG, "H >= 1"),
    (dict(Dk=96), kda.KDA_ERR_UNSUPPORTED, "head dims"),
    (dict(Dv=256), kda.KDA_ERR_UNSUPPORTED, "head dims"),
    (dict(chunk=48), kda.KDA_ERR_UNSUPPORTED, "chunk_size"),
    # the bf16 d=128 matrix-core kernel runs 16-row chunks only: other explicit lengths are refused
    (dict(chunk=64), kda.KDA_ERR_UNSUPPORTED, "16-row chunks"),
    (dict(chunk=32), kda.KDA_ERR_UNSUPPORTED, "16-row chunks"),
    (dict(dtype=7), kda.KDA_ERR_UNSUPPORTED, "dtype"),
    (dict(N=2), kda.KDA_ERR_INVALID_ARG, "N must equal B"),
    (dict(cu=FAKE, B=2, N=2), kda.KDA_ERR_INVALID_ARG, "B == 1"),
    (dict(cu=FAKE, N=0), kda.KDA_ERR_INVALID_ARG, "N >= 1"),
    (dict(o=FAKE), kda.KDA_ERR_INVALID_ARG, "alias"),
])
def test_chunk_fwd_rejects_before_launch(lib, kw, status, needle):
    st = _fwd(lib, **kw)
    assert st == status
    assert needle in lib.kda_last_error_message().decode()


def _pro(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=FAKE, lb=-5.0, eps=1e-6,
             s0=None, cu=None, B=1, T=64, H=2, Dk=128, Dv=128, N=1, chunk=0, scale=1.0,
             dtype=kda.KDA_BF16, o=ctypes.c_void_p(0x2000), sT=None, stream=None)
    a.update(kw)
    return lib.kda_chunk_fwd_prologue(a["q"], a["k"], a["v"], a["g"], a["beta"], a["A_log"], a["dt_bias"],
                                      a["lb"], a["eps"], a["s0"], a["cu"], a["B"], a["T"], a["H"], a["Dk"],
                                      a["Dv"], a["N"], a["chunk"], a["scale"], a["dtype"], a["o"], a["sT"],
                                      a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(A_log=None), kda.KDA_ERR_INVALID_ARG, "A_log"),
    (dict(dt_bias=None), kda.KDA_ERR_INVALID_ARG, "dt_bias"),
    (dict(lb=0.0), kda.KDA_ERR_INVALID_ARG, "gate_lower_bound"),
    (dict(lb=float("nan")), kda.KDA_ERR_INVALID_ARG, "gate_lower_bound"),
    (dict(lb=float("-inf")), kda.KDA_ERR_INVALID_ARG, "gate_lower_bound"),
    (dict(eps=0.0), kda.KDA_ERR_INVALID_ARG, "l2_eps"),
    (dict(eps=float("nan")), kda.KDA_ERR_INVALID_ARG, "l2_eps"),
    (dict(q=None), kda.KDA_ERR_INVALID_ARG, "non-NULL"),
    (dict(Dk=96), kda.KDA_ERR_UNSUPPORTED, "head dims"),
    (dict(N=2), kda.KDA_ERR_INVALID_ARG, "N must equal B"),
    (dict(o=FAKE), kda.KDA_ERR_INVALID_ARG, "alias"),
    (dict(chunk=64), kda.KDA_ERR_UNSUPPORTED, "16-row chunks"),
])
def test_chunk_fwd_prologue_rejects_before_launch(lib, kw, status, needle):
    st = _pro(lib, **kw)
    assert st == status
    msg = lib.kda_last_error_message().decode()
    assert needle in msg and msg.startswith("kda_chunk_fwd_prologue")


def _step(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, cache=FAKE, slots=None, n_slots=4, Nb=4, H=2,
             Dk=128, Dv=128, scale=1.0, dtype=kda.KDA_BF16, o=ctypes.c_void_p(0x2000), stream=None)
    a.update(kw)
    return lib.kda_recurrent_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cache"], a["slots"],
                                  a["n_slots"], a["Nb"], a["H"], a["Dk"], a["Dv"], a["scale"],
                                  a["dtype"], a["o"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(cache=None), kda.KDA_ERR_INVALID_ARG, "non-NULL"),
    (dict(Nb=-1), kda.KDA_ERR_INVALID_ARG, "Nb >= 0"),
    (dict(H=0), kda.KDA_ERR_INVALID_ARG, "H >= 1"),
    (dict(Dk=8), kda.KDA_ERR_UNSUPPORTED, "head dims"),
    (dict(dtype=5), kda.KDA_ERR_UNSUPPORTED, "dtype"),
    (dict(Nb=5), kda.KDA_ERR_INVALID_ARG, "n_slots"),
    (dict(o=FAKE), kda.KDA_ERR_INVALID_ARG, "alias"),
])
def test_recurrent_step_rejects_before_launch(lib, kw, status, needle):
    st = _step(lib, **kw)
    assert st == status
    assert needle in lib.kda_last_error_message().decode()


def _step_prologue(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=FAKE, lb=-5.0, eps=1e-6, cache=FAKE,
             slots=None, n_slots=4, Nb=4, H=2, Dk=128, Dv=128, scale=1.0, dtype=kda.KDA_BF16,
             o=ctypes.c_void_p(0x2000), stream=None)
    a.update(kw)
    return lib.kda_recurrent_step_prologue(a["q"], a["k"], a["v"], a["g"], a["beta"], a["A_log"], a["dt_bias"],
                                           a["lb"], a["eps"], a["cache"], a["slots"], a["n_slots"], a["Nb"],
                                           a["H"], a["Dk"], a["Dv"], a["scale"], a["dtype"], a["o"], a["stream"])


def _step_conv(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, wq=ctypes.c_void_p(0x3000), wk=ctypes.c_void_p(0x4000),
             wv=ctypes.c_void_p(0x5000), cq=ctypes.c_void_p(0x6000), ck=ctypes.c_void_p(0x7000),
             cv=ctypes.c_void_p(0x8000), act=1, g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=FAKE, lb=-5.0, eps=1e-6,
             cache=FAKE, slots=None, n_slots=4, Nb=4, H=2, Dk=128, Dv=128, scale=1.0, dtype=kda.KDA_BF16,
             o=ctypes.c_void_p(0x2000), stream=None)
    a.update(kw)
    return lib.kda_recurrent_step_conv(a["q"], a["k"], a["v"], a["wq"], a["wk"], a["wv"], a["cq"], a["ck"], a["cv"],
                                       a["act"], a["g"], a["beta"], a["A_log"], a["dt_bias"], a["lb"], a["eps"],
                                       a["cache"], a["slots"], a["n_slots"], a["Nb"], a["H"], a["Dk"], a["Dv"],
                                       a["scale"], a["dtype"], a["o"], a["stream"])


STEP_RAW_CASES = [
    (dict(cache=None), kda.KDA_ERR_INVALID_ARG, "non-NULL"),
    (dict(Nb=5), kda.KDA_ERR_INVALID_ARG, "n_slots"),
    (dict(Dv=48), kda.KDA_ERR_UNSUPPORTED, "head dims"),
    (dict(o=FAKE), kda.KDA_ERR_INVALID_ARG, "alias"),
    (dict(A_log=None), kda.KDA_ERR_INVALID_ARG, "A_log"),
    (dict(dt_bias=None), kda.KDA_ERR_INVALID_ARG, "dt_bias"),
    (dict(lb=0.0), kda.KDA_ERR_INVALID_ARG, "gate_lower_bound"),
    (dict(lb=float("-inf")), kda.KDA_ERR_INVALID_ARG, "gate_lower_bound"),
    (dict(eps=0.0), kda.KDA_ERR_INVALID_ARG, "l2_eps"),
    (dict(eps=float("nan")), kda.KDA_ERR_INVALID_ARG, "l2_eps"),
]


@pytest.mark.parametrize("kw,status,needle", STEP_RAW_CASES)
def test_recurrent_step_prologue_rejects_before_launch(lib, kw, status, needle):
    assert _step_prologue(lib, **kw) == status
    msg = lib.kda_last_error_message().decode()
    assert needle in msg and msg.startswith("kda_recurrent_step_prologue")


@pytest.mark.parametrize("kw,status,needle", STEP_RAW_CASES + [
    (dict(act=2), kda.KDA_ERR_INVALID_ARG, "activation"),
    (dict(wk=None), kda.KDA_ERR_INVALID_ARG, "non-NULL"),
    (dict(cv=None), kda.KDA_ERR_INVALID_ARG, "non-NULL"),
    (dict(wv=ctypes.c_void_p(0x5004)), kda.KDA_ERR_INVALID_ARG, "aligned"),
    (dict(ck=ctypes.c_void_p(0x6000)), kda.KDA_ERR_INVALID_ARG, "distinct"),
    (dict(cq=FAKE), kda.KDA_ERR_INVALID_ARG, "distinct"),
    (dict(cv=ctypes.c_void_p(0x2000)), kda.KDA_ERR_INVALID_ARG, "alias"),
])
def test_recurrent_step_conv_rejects_before_launch(lib, kw, status, needle):
    assert _step_conv(lib, **kw) == status
    msg = lib.kda_last_error_message().decode()
    assert needle in msg and msg.startswith("kda_recurrent_step_conv")


def test_empty_work_is_ok_without_launch(lib):
    assert _step_prologue(lib, Nb=0, q=None, A_log=None) == kda.KDA_OK
    assert _step_conv(lib, Nb=0, wq=None, cq=None) == kda.KDA_OK
    assert _step(lib, Nb=0) == kda.KDA_OK
    assert lib.kda_last_error_message() == b""


def test_binding_refuses_cpu_tensors(lib):
    import torch
    x = torch.zeros(1, 4, 2, 16)
    with pytest.raises(ValueError, match="GPU"):
        kda.chunk_fwd(x, x, x, x, torch.zeros(1, 4, 2))


def _conv(lib, **kw):
    a = dict(x=FAKE, w=FAKE, s_in=None, cu=None, B=1, T=64, C=1024, N=1, act=1, dtype=kda.KDA_BF16,
             y=ctypes.c_void_p(0x2000), s_out=None, stream=None)
    a.update(kw)
    return lib.kda_short_conv(a["x"], a["w"], a["s_in"], a["cu"], a["B"], a["T"], a["C"], a["N"], a["act"],
                              a["dtype"], a["y"], a["s_out"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(x=None), kda.KDA_ERR_INVALID_ARG, "non-NULL"),
    (dict(w=None), kda.KDA_ERR_INVALID_ARG, "non-NULL"),
    (dict(C=1020), kda.KDA_ERR_UNSUPPORTED, "multiple of 8"),
    (dict(act=2), kda.KDA_ERR_INVALID_ARG, "activation"),
    (dict(dtype=9), kda.KDA_ERR_UNSUPPORTED, "dtype"),
    (dict(N=3), kda.KDA_ERR_INVALID_ARG, "N must equal B"),
    (dict(cu=FAKE, B=2, N=2), kda.KDA_ERR_INVALID_ARG, "B == 1"),
    (dict(y=FAKE), kda.KDA_ERR_INVALID_ARG, "alias"),
    (dict(B=0), kda.KDA_ERR_INVALID_ARG, "B >= 1"),
])
def test_short_conv_rejects_before_launch(lib, kw, status, needle):
    assert _conv(lib, **kw) == status
    assert needle in lib.kda_last_error_message().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(cache=None), kda.KDA_ERR_INVALID_ARG, "non-NULL"),
    (dict(C=12), kda.KDA_ERR_UNSUPPORTED, "multiple of 8"),
    (dict(Nb=5), kda.KDA_ERR_INVALID_ARG, "n_slots"),
    (dict(act=-1), kda.KDA_ERR_INVALID_ARG, "activation"),
    (dict(y=FAKE), kda.KDA_ERR_INVALID_ARG, "alias"),
])
def test_short_conv_step_rejects_before_launch(lib, kw, status, needle):
    a = dict(x=FAKE, w=FAKE, cache=FAKE, slots=None, n_slots=4, Nb=4, C=1024, act=1, dtype=kda.KDA_BF16,
             y=ctypes.c_void_p(0x2000), stream=None)
    a.update(kw)
    st = lib.kda_short_conv_step(a["x"], a["w"], a["cache"], a["slots"], a["n_slots"], a["Nb"], a["C"], a["act"],
                                 a["dtype"], a["y"], a["stream"])
    assert st == status
    assert needle in lib.kda_last_error_message().decode()


def test_short_conv_step_empty_is_ok(lib):
    st = lib.kda_short_conv_step(None, None, None, None, 0, 0, 1024, 1, kda.KDA_BF16, None, None)
    assert st == kda.KDA_OK


def test_chunk_bwd_workspace_bytes(lib):
    # per 16-row chunk slot and head: a float32 [Dk,Dv] state, and the chunk's
    # T, P and KK (3 x 16 x 16 floats)
    def expect(slots, H, Dk, Dv):
        return slots * H * (Dk * Dv + 768) * 4
    assert kda.chunk_bwd_workspace_bytes(1, 4096, 96, 128, 128, 1, False) == expect(256, 96, 128, 128)
    assert kda.chunk_bwd_workspace_bytes(2, 17, 3, 64, 32, 2, False) == expect(4, 3, 64, 32)
    assert kda.chunk_bwd_workspace_bytes(1, 100, 2, 16, 16, 5, True) == expect(100 // 16 + 5, 2, 16, 16)
    assert kda.chunk_bwd_workspace_bytes(1, 0, 2, 16, 16, 1, False) == 0
    assert kda.chunk_bwd_workspace_bytes(0, 10, 2, 16, 16, 1, False) == 0


def test_chunk_bwd_packed_slots_never_overlap():
    # Sequence n's chunks use slots [cu[n] // 16 + n, ... + ceil(len / 16)); the
    # ranges of consecutive sequences must not overlap and must fit the count.
    import numpy as np
    rng = np.random.default_rng(0)
    for _ in range(200):
        lens = rng.integers(0, 70, size=int(rng.integers(1, 9)))
        cu = np.concatenate([[0], np.cumsum(lens)])
        T, N = int(cu[-1]), len(lens)
        total = T // 16 + N
        used = set()
        for n in range(N):
            base = int(cu[n]) // 16 + n
            for c in range((int(lens[n]) + 15) // 16):
                assert base + c not in used and base + c < total
                used.add(base + c)


def _bwd(lib, **kw):
    W = ctypes.c_void_p(0x3000)
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s0=None, cu=None, do=FAKE, dfin=None, B=1, T=64, H=2,
             Dk=128, Dv=128, N=1, scale=1.0, dtype=kda.KDA_BF16, ws=W, wsb=1 << 30,
             dq=ctypes.c_void_p(0x4000), dk=ctypes.c_void_p(0x5000), dv=ctypes.c_void_p(0x6000),
             dg=ctypes.c_void_p(0x7000), db=ctypes.c_void_p(0x8000), d0=None, stream=None)
    a.update(kw)
    return lib.kda_chunk_bwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["cu"], a["do"], a["dfin"],
                             a["B"], a["T"], a["H"], a["Dk"], a["Dv"], a["N"], a["scale"], a["dtype"], a["ws"],
                             a["wsb"], a["dq"], a["dk"], a["dv"], a["dg"], a["db"], a["d0"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(do=None), kda.KDA_ERR_INVALID_ARG, "non-NULL"),
    (dict(dg=None), kda.KDA_ERR_INVALID_ARG, "non-NULL"),
    (dict(B=0), kda.KDA_ERR_INVALID_ARG, "B >= 1"),
    (dict(Dk=96), kda.KDA_ERR_UNSUPPORTED, "head dims"),
    (dict(dtype=7), kda.KDA_ERR_UNSUPPORTED, "dtype"),
    (dict(cu=FAKE, B=2, N=1), kda.KDA_ERR_INVALID_ARG, "B == 1"),
    (dict(N=2), kda.KDA_ERR_INVALID_ARG, "N must equal B"),
    (dict(wsb=4 * 2 * (128 * 128 + 768) * 4 - 1), kda.KDA_ERR_INVALID_ARG, "workspace"),
    (dict(ws=None), kda.KDA_ERR_INVALID_ARG, "workspace"),
    (dict(dq=FAKE), kda.KDA_ERR_INVALID_ARG, "alias"),
    (dict(dv=ctypes.c_void_p(0x3000)), kda.KDA_ERR_INVALID_ARG, "alias"),
])
def test_chunk_bwd_rejects_before_launch(lib, kw, status, needle):
    st = _bwd(lib, **kw)
    assert st == status
    assert needle in lib.kda_last_error_message().decode()


def _split(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s0=None, cu=None, B=1, T=4096, H=12, Dk=128, Dv=128, N=1,
             chunk=0, scale=1.0, dtype=kda.KDA_BF16, seg=8, ws=ctypes.c_void_p(1 << 40), wsb=1 << 34,
             o=ctypes.c_void_p(0x2000), sT=None, stream=None)
    a.update(kw)
    return lib.kda_chunk_fwd_split(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["cu"], a["B"], a["T"],
                                   a["H"], a["Dk"], a["Dv"], a["N"], a["chunk"], a["scale"], a["dtype"], a["seg"],
                                   a["ws"], a["wsb"], a["o"], a["sT"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(seg=0), kda.KDA_ERR_INVALID_ARG, "segments"),
    (dict(seg=5000), kda.KDA_ERR_INVALID_ARG, "segments"),
    (dict(ws=None), kda.KDA_ERR_INVALID_ARG, "workspace"),
    (dict(wsb=1000), kda.KDA_ERR_INVALID_ARG, "workspace"),
    (dict(o=ctypes.c_void_p((1 << 40) + 4096)), kda.KDA_ERR_INVALID_ARG, "overlap"),
    (dict(Dk=96), kda.KDA_ERR_UNSUPPORTED, "head dims"),
    (dict(o=None), kda.KDA_ERR_INVALID_ARG, "non-NULL"),
    (dict(B=2, N=1), kda.KDA_ERR_INVALID_ARG, "N must equal B"),
    (dict(chunk=64), kda.KDA_ERR_UNSUPPORTED, "16-row chunks"),
])
def test_chunk_fwd_split_rejects_before_launch(lib, kw, status, needle):
    st = _split(lib, **kw)
    assert st == status
    assert needle in lib.kda_last_error_message().decode()


def test_chunk_fwd_split_workspace_bytes(lib):
    import torch
    assert kda.chunk_fwd_split_workspace_bytes(1, 4096, 12, 128, 128, 1, torch.bfloat16, 1) == 0
    assert kda.chunk_fwd_split_workspace_bytes(1, 0, 12, 128, 128, 1, torch.bfloat16, 8) == 0
    a = kda.chunk_fwd_split_workspace_bytes(1, 4096, 12, 128, 128, 1, torch.bfloat16, 8)
    b = kda.chunk_fwd_split_workspace_bytes(1, 4096, 12, 128, 128, 1, torch.float32, 8)
    # three fp32 states per segment and head (identity then A, B, entry states) and the segment
    # offsets; the bf16 d=128 path adds the A pass's bf16 outputs, one row of Dk per token and head
    states = 3 * 8 * 12 * 128 * 128 * 4
    assert states <= b < states + 4096
    assert a == b + 4096 * 12 * 128 * 2
    c = kda.chunk_fwd_split_workspace_bytes(1, 4096, 12, 64, 64, 1, torch.bfloat16, 8)
    assert 3 * 8 * 12 * 64 * 64 * 4 <= c < 3 * 8 * 12 * 64 * 64 * 4 + 4096


def _bwd_pro(lib, **kw):
    W = ctypes.c_void_p(0x3000)
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A=ctypes.c_void_p(0x9000), b=ctypes.c_void_p(0xA000),
             lb=-5.0, eps=1e-6, s0=None, cu=None, do=FAKE, dfin=None, B=1, T=64, H=2, Dk=128, Dv=128, N=1,
             scale=1.0, dtype=kda.KDA_BF16, ws=W, wsb=1 << 34, dq=ctypes.c_void_p(0x4000),
             dk=ctypes.c_void_p(0x5000), dv=ctypes.c_void_p(0x6000), dg=ctypes.c_void_p(0x7000),
             db=ctypes.c_void_p(0x8000), dA=ctypes.c_void_p(0xB000), dbias=ctypes.c_void_p(0xC000), d0=None,
             stream=None)
    a.update(kw)
    return lib.kda_chunk_bwd_prologue(a["q"], a["k"], a["v"], a["g"], a["beta"], a["A"], a["b"], a["lb"], a["eps"],
                                      a["s0"], a["cu"], a["do"], a["dfin"], a["B"], a["T"], a["H"], a["Dk"],
                                      a["Dv"], a["N"], a["scale"], a["dtype"], a["ws"], a["wsb"], a["dq"], a["dk"],
                                      a["dv"], a["dg"], a["db"], a["dA"], a["dbias"], a["d0"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(A=None), kda.KDA_ERR_INVALID_ARG, "A_log"),
    (dict(dbias=None), kda.KDA_ERR_INVALID_ARG, "ddt_bias"),
    (dict(lb=0.0), kda.KDA_ERR_INVALID_ARG, "gate_lower_bound"),
    (dict(eps=0.0), kda.KDA_ERR_INVALID_ARG, "l2_eps"),
    (dict(do=None), kda.KDA_ERR_INVALID_ARG, "non-NULL"),
    (dict(Dk=96), kda.KDA_ERR_UNSUPPORTED, "head dims"),
    (dict(N=2), kda.KDA_ERR_INVALID_ARG, "N must equal B"),
    (dict(wsb=100), kda.KDA_ERR_INVALID_ARG, "workspace"),
    (dict(dq=FAKE), kda.KDA_ERR_INVALID_ARG, "alias"),
    (dict(dA=ctypes.c_void_p(0x9000)), kda.KDA_ERR_INVALID_ARG, "alias"),
])
def test_chunk_bwd_prologue_rejects_before_launch(lib, kw, status, needle):
    st = _bwd_pro(lib, **kw)
    assert st == status
    assert needle in lib.kda_last_error_message().decode()


def test_chunk_bwd_prologue_workspace_bytes(lib):
    core = kda.chunk_bwd_workspace_bytes(1, 4096, 96, 128, 128, 1, False)
    total = kda.chunk_bwd_prologue_workspace_bytes(1, 4096, 96, 128, 128, 1, False)
    rows = 4096 * 96
    assert total >= core + rows * (3 * 128 + 1 + 2 * 128) * 4 + 2 * 64 * 96 * 128 * 4
    assert kda.chunk_bwd_prologue_workspace_bytes(1, 0, 96, 128, 128, 1, False) == 0


def _conv_bwd(lib, **kw):
    a = dict(x=FAKE, w=ctypes.c_void_p(0x9000), s0=None, cu=None, dy=ctypes.c_void_p(0xA000), dfin=None, B=1, T=64,
             C=256, N=1, act=1, dtype=kda.KDA_BF16, ws=ctypes.c_void_p(0x3000), wsb=1 << 30,
             dx=ctypes.c_void_p(0x4000), dw=ctypes.c_void_p(0x5000), dst=None, stream=None)
    a.update(kw)
    return lib.kda_short_conv_bwd(a["x"], a["w"], a["s0"], a["cu"], a["dy"], a["dfin"], a["B"], a["T"], a["C"],
                                  a["N"], a["act"], a["dtype"], a["ws"], a["wsb"], a["dx"], a["dw"], a["dst"],
                                  a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(w=None), kda.KDA_ERR_INVALID_ARG, "weight"),
    (dict(dy=None), kda.KDA_ERR_INVALID_ARG, "non-NULL"),
    (dict(C=12), kda.KDA_ERR_UNSUPPORTED, "multiple of 8"),
    (dict(act=2), kda.KDA_ERR_INVALID_ARG, "activation"),
    (dict(N=2), kda.KDA_ERR_INVALID_ARG, "N must equal B"),
    (dict(wsb=10), kda.KDA_ERR_INVALID_ARG, "workspace"),
    (dict(dx=FAKE), kda.KDA_ERR_INVALID_ARG, "alias"),
])
def test_short_conv_bwd_rejects_before_launch(lib, kw, status, needle):
    st = _conv_bwd(lib, **kw)
    assert st == status
    assert needle in lib.kda_last_error_message().decode()


def test_short_conv_bwd_workspace_bytes(lib):
    # one partial of C x 4 floats per 256 tokens
    assert lib.kda_short_conv_bwd_workspace_bytes(1, 4096, 12288) == 16 * 12288 * 4 * 4
    assert lib.kda_short_conv_bwd_workspace_bytes(2, 65, 8) == 1 * 8 * 4 * 4
    assert lib.kda_short_conv_bwd_workspace_bytes(1, 257, 8) == 2 * 8 * 4 * 4
    assert lib.kda_short_conv_bwd_workspace_bytes(1, 0, 8) == 0


def _split_static(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s0=None, cu=None, B=1, T=4096, H=12, Dk=128, Dv=128, N=1,
             chunk=0, scale=1.0, dtype=kda.KDA_BF16, seg=8, o=ctypes.c_void_p(0x2000), sT=None, stream=None)
    a.update(kw)
    return lib.kda_chunk_fwd_split_static(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["cu"], a["B"],
                                          a["T"], a["H"], a["Dk"], a["Dv"], a["N"], a["chunk"], a["scale"],
                                          a["dtype"], a["seg"], a["o"], a["sT"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    # 3 fp32 states of 64 KiB per (segment, head), plus the A pass's bf16 outputs:
    # 96 heads x 8 segments at T=4096 need 252 MB > 128 MiB
    (dict(H=96), kda.KDA_ERR_UNSUPPORTED, "static scratch holds 134217728"),
    (dict(seg=0), kda.KDA_ERR_INVALID_ARG, "segments"),
    (dict(o=None), kda.KDA_ERR_INVALID_ARG, "non-NULL"),
    (dict(chunk=64), kda.KDA_ERR_UNSUPPORTED, "16-row chunks"),
])
def test_chunk_fwd_split_static_rejects_before_launch(lib, kw, status, needle):
    st = _split_static(lib, **kw)
    assert st == status
    msg = lib.kda_last_error_message().decode()
    assert needle in msg and msg.startswith("kda_chunk_fwd_split_static")


def test_split_static_scratch_size_matches_header():
    text = open(kda.HEADER_PATH).read()
    assert "#define KDA_SPLIT_STATIC_SCRATCH_BYTES ((size_t)128 << 20)" in text
    assert kda.SPLIT_STATIC_SCRATCH_BYTES == 128 << 20


def _conv_fwd(lib, **kw):
    a = dict(xq=FAKE, xk=FAKE, xv=FAKE, wq=FAKE, wk=FAKE, wv=FAKE, sq=None, sk=None, sv=None, act=1, g=FAKE,
             beta=FAKE, A_log=FAKE, dt_bias=FAKE, lb=-5.0, eps=1e-6, s0=None, cu=None, B=1, T=64, H=2, Dk=128,
             Dv=128, N=1, chunk=0, scale=1.0, dtype=kda.KDA_BF16, ws=ctypes.c_void_p(1 << 40), wsb=1 << 30,
             o=ctypes.c_void_p(0x2000), sT=None, oq=None, ok=None, ov=None, stream=None)
    a.update(kw)
    return lib.kda_chunk_fwd_conv(a["xq"], a["xk"], a["xv"], a["wq"], a["wk"], a["wv"], a["sq"], a["sk"], a["sv"],
                                  a["act"], a["g"], a["beta"], a["A_log"], a["dt_bias"], a["lb"], a["eps"], a["s0"],
                                  a["cu"], a["B"], a["T"], a["H"], a["Dk"], a["Dv"], a["N"], a["chunk"], a["scale"],
                                  a["dtype"], a["ws"], a["wsb"], a["o"], a["sT"], a["oq"], a["ok"], a["ov"],
                                  a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(xq=None), kda.KDA_ERR_INVALID_ARG, "non-NULL"),
    (dict(wk=None), kda.KDA_ERR_INVALID_ARG, "conv taps"),
    (dict(act=2), kda.KDA_ERR_INVALID_ARG, "activation"),
    (dict(A_log=None), kda.KDA_ERR_INVALID_ARG, "A_log"),
    (dict(lb=0.0), kda.KDA_ERR_INVALID_ARG, "gate_lower_bound"),
    (dict(eps=0.0), kda.KDA_ERR_INVALID_ARG, "l2_eps"),
    (dict(ws=None), kda.KDA_ERR_INVALID_ARG, "workspace"),
    (dict(wsb=100), kda.KDA_ERR_INVALID_ARG, "workspace"),
    (dict(o=ctypes.c_void_p((1 << 40) + 64)), kda.KDA_ERR_INVALID_ARG, "overlap"),
    (dict(Dk=96), kda.KDA_ERR_UNSUPPORTED, "head dims"),
    (dict(chunk=64), kda.KDA_ERR_UNSUPPORTED, "16-row chunks"),
])
def test_chunk_fwd_conv_rejects_before_launch(lib, kw, status, needle):
    st = _conv_fwd(lib, **kw)
    assert st == status
    msg = lib.kda_last_error_message().decode()
    assert needle in msg and msg.startswith("kda_chunk_fwd_conv")


def test_chunk_fwd_conv_workspace_bytes():
    import torch
    # fused path (bf16, d=128, bound >= -5): convolved q and k in bf16
    assert kda.chunk_fwd_conv_workspace_bytes(1, 4096, 96, 128, 128, torch.bfloat16, -5.0) == 2 * 4096 * 96 * 128 * 2
    # other paths: the three convolved projections in the input dtype
    assert kda.chunk_fwd_conv_workspace_bytes(1, 100, 4, 64, 32, torch.float32, -5.0) == 100 * 4 * (2 * 64 + 32) * 4
    assert kda.chunk_fwd_conv_workspace_bytes(1, 100, 4, 128, 128, torch.bfloat16, -6.0) == 100 * 4 * 384 * 2
    assert kda.chunk_fwd_conv_workspace_bytes(1, 0, 4, 128, 128, torch.bfloat16, -5.0) == 0



def _bwd_conv(lib, **kw):
    P = ctypes.c_void_p
    a = dict(xq=FAKE, xk=FAKE, xv=FAKE, wq=P(0x3000), wk=P(0x4000), wv=P(0x5000), sq=None, sk=None, sv=None, act=1,
             g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=FAKE, lb=-5.0, eps=1e-6, s0=None, cu=None, d_o=FAKE,
             dfin=None, dcq=None, dck=None, dcv=None, B=1, T=64, H=2, Dk=128, Dv=128, N=1, scale=1.0,
             dtype=kda.KDA_BF16, ws=P(0x100000), wsb=1 << 40, dxq=P(0x6000), dxk=P(0x7000), dxv=P(0x8000),
             dwq=P(0x9000), dwk=P(0xa000), dwv=P(0xb000), dsq=None, dsk=None, dsv=None, dg=P(0xc000),
             db=P(0xd000), dA=P(0xe000), ddt=P(0xf000), ds0=None, stream=None)
    a.update(kw)
    return lib.kda_chunk_bwd_conv(*a.values())


@pytest.mark.parametrize("kw,status,needle", [
    (dict(act=2), kda.KDA_ERR_INVALID_ARG, "activation"),
    (dict(wk=None), kda.KDA_ERR_INVALID_ARG, "taps"),
    (dict(dwv=None), kda.KDA_ERR_INVALID_ARG, "taps"),
    (dict(wq=ctypes.c_void_p(0x3008)), kda.KDA_ERR_INVALID_ARG, "aligned"),
    (dict(xv=None), kda.KDA_ERR_INVALID_ARG, "non-NULL"),
    (dict(dA=None), kda.KDA_ERR_INVALID_ARG, "dA_log"),
    (dict(lb=0.0), kda.KDA_ERR_INVALID_ARG, "gate_lower_bound"),
    (dict(eps=-1.0), kda.KDA_ERR_INVALID_ARG, "l2_eps"),
    (dict(Dk=8), kda.KDA_ERR_UNSUPPORTED, "head dims"),
    (dict(N=2), kda.KDA_ERR_INVALID_ARG, "N must equal B"),
    (dict(wsb=16), kda.KDA_ERR_INVALID_ARG, "workspace"),
    (dict(dg=FAKE), kda.KDA_ERR_INVALID_ARG, "alias"),
    (dict(dxq=ctypes.c_void_p(0x100000)), kda.KDA_ERR_INVALID_ARG, "alias"),
])
def test_chunk_bwd_conv_rejects_before_launch(lib, kw, status, needle):
    assert _bwd_conv(lib, **kw) == status
    msg = lib.kda_last_error_message().decode()
    assert needle in msg and msg.startswith("kda_chunk_bwd_conv")


def test_chunk_bwd_conv_workspace_covers_its_parts(lib):
    B, T, H, D, N = 1, 4096, 96, 128, 1
    need = lib.kda_chunk_bwd_conv_workspace_bytes(B, T, H, D, D, N, 0, kda.KDA_BF16)
    parts = 3 * B * T * H * D * (2 + 4) + max(lib.kda_chunk_bwd_prologue_workspace_bytes(B, T, H, D, D, N, 0),
                                              lib.kda_short_conv_bwd_workspace_bytes(B, T, H * D))
    assert parts <= need <= parts + 8 * 256
    assert lib.kda_chunk_bwd_conv_workspace_bytes(B, 0, H, D, D, N, 0, kda.KDA_BF16) == 0


def test_autograd_entry_points_import_without_a_gpu():
    from gated_delta_rule_chunk_amd import autograd as kag
    for name in ("chunk_kda", "chunk_kda_prologue", "chunk_kda_conv"):
        assert callable(getattr(kag, name))



def _prologue(lib, **kw):
    P = ctypes.c_void_p
    a = dict(q=FAKE, k=FAKE, g=FAKE, beta=FAKE, A_log=P(0x3000), dt_bias=P(0x4000), lb=-5.0, eps=1e-6, B=1, T=8,
             H=2, Dk=128, dtype=kda.KDA_BF16, qo=P(0x5000), ko=P(0x6000), go=P(0x7000), bo=P(0x8000), stream=None)
    a["q"], a["k"], a["g"], a["beta"] = P(0x1000), P(0x1100), P(0x1200), P(0x1300)
    a.update(kw)
    return lib.kda_prologue(*a.values())


@pytest.mark.parametrize("kw,status,needle", [
    (dict(A_log=None), kda.KDA_ERR_INVALID_ARG, "non-NULL"),
    (dict(ko=None), kda.KDA_ERR_INVALID_ARG, "non-NULL"),
    (dict(lb=0.5), kda.KDA_ERR_INVALID_ARG, "gate_lower_bound"),
    (dict(eps=0.0), kda.KDA_ERR_INVALID_ARG, "l2_eps"),
    (dict(Dk=48), kda.KDA_ERR_UNSUPPORTED, "head dims"),
    (dict(dtype=3), kda.KDA_ERR_UNSUPPORTED, "dtype"),
    (dict(H=0), kda.KDA_ERR_INVALID_ARG, "H >= 1"),
    (dict(ko=ctypes.c_void_p(0x1000)), kda.KDA_ERR_INVALID_ARG, "its own input"),
    (dict(go=ctypes.c_void_p(0x5000)), kda.KDA_ERR_INVALID_ARG, "distinct"),
    (dict(bo=ctypes.c_void_p(0x3000)), kda.KDA_ERR_INVALID_ARG, "its own input"),
])
def test_prologue_rejects_before_launch(lib, kw, status, needle):
    assert _prologue(lib, **kw) == status
    msg = lib.kda_last_error_message().decode()
    assert needle in msg and msg.startswith("kda_prologue")


def test_prologue_in_place_and_empty_are_accepted_without_launch(lib):
    # T = 0: nothing to launch, so no GPU is needed even for an in-place call
    P = ctypes.c_void_p
    assert _prologue(lib, T=0, qo=P(0x1000), ko=P(0x1100), go=P(0x1200), bo=P(0x1300)) == kda.KDA_OK
