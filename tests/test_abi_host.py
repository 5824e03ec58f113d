"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point declared in include/kda.h, and rejects bad arguments before
launching anything."""
import ctypes
import os
import re
import subprocess

import pytest

import gated_delta_rule_12_amd as kda
from tests.conftest import ROOT

HDR = os.path.join(ROOT, "include", "kda.h")
FAKE = 0x100000          # 256-byte aligned, never dereferenced: every call below fails validation


def declared_symbols():
    src = open(HDR).read()
    return sorted(set(re.findall(r"KDA_API\s+[\w\s\*]*?\b(kda_\w+)\s*\(", src)))


def test_header_declares_the_abi():
    assert declared_symbols() == sorted(kda.EXPORTED)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", kda.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, re.M))
    for name in declared_symbols():
        assert name in exported, name
        assert hasattr(kda.lib(), name)


def test_header_compiles_as_c():
    src = f'#include "{HDR}"\nint main(void) {{ return (int)sizeof(kda_status); }}\n'
    r = subprocess.run(["gcc", "-x", "c", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-"],
                       input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_status_strings():
    names = [kda.kda_status_string(i) for i in range(5)]
    assert names == ["KDA_SUCCESS", "KDA_ERROR_INVALID_VALUE", "KDA_ERROR_NOT_SUPPORTED",
                     "KDA_ERROR_WORKSPACE_TOO_SMALL", "KDA_ERROR_LAUNCH"]
    assert kda.kda_status_string(99) == "KDA_ERROR_UNKNOWN"


def test_workspace_size_plan():
    f = kda.kda_chunk_fwd_workspace_bytes
    n = f(2, 4096, 8, 128, 128, False, 0, 64, kda.KDA_DTYPE_BF16)
    gh = 2 * 64 * 8
    per = 64 * 128 * 2 * 3 + 6 * 16 * 32 * 2 + 128 * 64 * 2 + 128 * 4   # qh, w, ktt, p (6 fragments), ut (fp16), gam
    assert gh * per <= n < gh * per + 64 * 1024
    assert f(2, 4096, 8, 128, 128, False, 0, 64, kda.KDA_DTYPE_F32) > n
    # packed: chunk capacity is ceil(T/64) + N
    nv = f(1, 1000, 4, 64, 64, True, 10, 64, kda.KDA_DTYPE_BF16)
    assert nv > f(1, 1000, 4, 64, 64, False, 0, 64, kda.KDA_DTYPE_BF16)
    # unsupported combinations report 0
    assert f(1, 256, 1, 96, 64, False, 0, 64, kda.KDA_DTYPE_BF16) == 0
    assert f(1, 256, 1, 64, 64, False, 0, 96, kda.KDA_DTYPE_BF16) == 0
    # chunk sizes 32 and 128 take the generic path, with its own record
    assert f(1, 256, 1, 64, 64, False, 0, 32, kda.KDA_DTYPE_BF16) > 0
    assert f(1, 256, 1, 64, 64, False, 0, 128, kda.KDA_DTYPE_BF16) > 0
    # the backward runs at C = 64 only
    fb = kda.kda_chunk_bwd_workspace_bytes
    assert fb(1, 256, 1, 64, 64, False, 0, 64, kda.KDA_DTYPE_BF16) > 0
    assert fb(1, 256, 1, 64, 64, False, 0, 32, kda.KDA_DTYPE_BF16) == 0
    assert fb(1, 256, 1, 64, 64, False, 0, 128, kda.KDA_DTYPE_BF16) == 0
    assert f(2, 256, 1, 64, 64, True, 3, 64, kda.KDA_DTYPE_BF16) == 0
    assert f(1, 1 << 31, 1, 64, 64, False, 0, 64, kda.KDA_DTYPE_BF16) == 0


@pytest.mark.parametrize("C", [32, 128])
@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_generic_record_size(C, Dk, Dv):
    """One more chunk adds H generic records: Gamma.Q, Kt, W, b (C x d_k each),
    U (C x d_v) and P (C x C) in fp32, gamma (d_k fp32), and at C = 128 the
    state entering the chunk (d_k x d_v) and U' (C x d_v) for the output
    pass, fp16 with 16-bit activations and fp32 otherwise (at C = 32 the
    chain writes the output itself and the record ends at gamma); up to the
    256-byte alignment steps of the regions that grow."""
    H = 3
    f = kda.kda_chunk_fwd_workspace_bytes
    for act, se in ((kda.KDA_DTYPE_F32, 4), (kda.KDA_DTYPE_BF16, 2)):
        r = (4 * C * Dk + C * Dv + C * C + Dk) * 4 + ((Dk * Dv + C * Dv) * se if C == 128 else 0)
        r = (r + 255) // 256 * 256
        diff = f(1, 10 * C, H, Dk, Dv, False, 0, C, act) - f(1, 9 * C, H, Dk, Dv, False, 0, C, act)
        assert abs(diff - H * r) <= 4 * 256, (act, diff, H * r)


def _chunk(**over):
    L = kda.lib()
    a = dict(q=FAKE, k=FAKE, v=FAKE, alpha=FAKE, beta=FAKE, s0=None, sT=None, cu=None, N=0,
             o=FAKE, B=1, T=128, H=2, Dk=64, Dv=64, C=64, act=kda.KDA_DTYPE_BF16,
             out=kda.KDA_DTYPE_BF16, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(over)
    return L.kda_chunk_fwd(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["s0"], a["sT"],
                           a["cu"], a["N"], a["o"], a["B"], a["T"], a["H"], a["Dk"], a["Dv"],
                           a["C"], a["act"], a["out"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_bwd_record_size_matches_the_header(Dk, Dv):
    """One more chunk adds H records of the size include/kda.h states, and 8
    bytes per head for the general-form list and flags (up to a 256-byte
    alignment step of each of the three regions that grow)."""
    C, H = 64, 3
    rec = {kda.KDA_DTYPE_F32: (3 * C * Dk + 3 * C * Dv + 2 * Dk * Dv + 2 * C * C + Dk) * 4,
           kda.KDA_DTYPE_BF16: 14 * C * Dk + 8 * C * Dv + 4 * Dk * Dv + 6 * C * C + 4 * Dk}
    for act, r in rec.items():
        r = (r + 255) // 256 * 256
        fb = kda.kda_chunk_bwd_workspace_bytes
        diff = fb(1, 10 * C, H, Dk, Dv, False, 0, C, act) - fb(1, 9 * C, H, Dk, Dv, False, 0, C, act)
        assert abs(diff - H * (r + 8)) <= 3 * 256, (act, diff, H * (r + 8))


def test_chunk_fwd_argument_errors():
    assert _chunk(q=None) == kda.KDA_ERROR_INVALID_VALUE
    assert _chunk(o=None) == kda.KDA_ERROR_INVALID_VALUE
    assert _chunk(k=FAKE + 8) == kda.KDA_ERROR_INVALID_VALUE          # misaligned
    assert _chunk(beta=FAKE + 2) == kda.KDA_ERROR_INVALID_VALUE
    assert _chunk(T=-1) == kda.KDA_ERROR_INVALID_VALUE
    assert _chunk(H=0) == kda.KDA_ERROR_INVALID_VALUE
    assert _chunk(Dk=96) == kda.KDA_ERROR_NOT_SUPPORTED
    assert _chunk(Dv=32) == kda.KDA_ERROR_NOT_SUPPORTED
    assert _chunk(C=96) == kda.KDA_ERROR_NOT_SUPPORTED
    assert _chunk(C=16) == kda.KDA_ERROR_NOT_SUPPORTED
    assert _chunk(act=7) == kda.KDA_ERROR_INVALID_VALUE
    assert _chunk(act=kda.KDA_DTYPE_F32, out=kda.KDA_DTYPE_BF16) == kda.KDA_ERROR_NOT_SUPPORTED
    assert _chunk(cu=FAKE, B=2, N=3) == kda.KDA_ERROR_INVALID_VALUE
    assert _chunk(cu=FAKE, N=-1) == kda.KDA_ERROR_INVALID_VALUE
    assert _chunk(ws=None) == kda.KDA_ERROR_INVALID_VALUE
    assert _chunk(ws=FAKE + 16) == kda.KDA_ERROR_INVALID_VALUE
    assert _chunk(wsb=100) == kda.KDA_ERROR_WORKSPACE_TOO_SMALL
    assert _chunk(B=1 << 20, T=1 << 12) == kda.KDA_ERROR_NOT_SUPPORTED   # > 2^31 token rows


def _chunk_gated(gate_kind, gate=FAKE, **over):
    L = kda.lib()
    a = dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, s0=None, sT=None, cu=None, N=0,
             o=FAKE, B=1, T=128, H=2, Dk=64, Dv=64, C=64, act=kda.KDA_DTYPE_BF16,
             out=kda.KDA_DTYPE_BF16, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(over)
    return L.kda_chunk_fwd_gated(a["q"], a["k"], a["v"], gate, gate_kind, a["beta"], a["s0"],
                                 a["sT"], a["cu"], a["N"], a["o"], a["B"], a["T"], a["H"],
                                 a["Dk"], a["Dv"], a["C"], a["act"], a["out"], a["ws"], a["wsb"],
                                 a["stream"])


def test_gated_entry_points_argument_errors():
    assert _chunk_gated(3) == kda.KDA_ERROR_INVALID_VALUE                       # unknown form
    assert _chunk_gated(kda.KDA_GATE_SOFTPLUS_BF16, gate=None) == kda.KDA_ERROR_INVALID_VALUE
    assert _chunk_gated(kda.KDA_GATE_ALPHA, gate=FAKE + 8) == kda.KDA_ERROR_INVALID_VALUE
    assert _chunk_gated(kda.KDA_GATE_SOFTPLUS_BF16, gate=FAKE + 4) == kda.KDA_ERROR_INVALID_VALUE
    assert _chunk_gated(kda.KDA_GATE_SCALAR, gate=FAKE + 2) == kda.KDA_ERROR_INVALID_VALUE
    assert _chunk_gated(kda.KDA_GATE_SCALAR, Dk=96) == kda.KDA_ERROR_NOT_SUPPORTED
    assert _chunk_gated(kda.KDA_GATE_SCALAR, B=0, q=None, k=None, v=None, beta=None, o=None,
                        ws=None, gate=None) == kda.KDA_SUCCESS
    L = kda.lib()
    st = L.kda_recurrent_step_gated(FAKE, FAKE, FAKE, FAKE + 4, kda.KDA_GATE_SOFTPLUS_BF16, FAKE,
                                    FAKE, FAKE, 4, 2, 128, 128, kda.KDA_DTYPE_BF16,
                                    kda.KDA_DTYPE_F32, None)
    assert st == kda.KDA_ERROR_INVALID_VALUE
    st = L.kda_recurrent_step_gated(FAKE, FAKE, FAKE, FAKE, 5, FAKE, FAKE, FAKE, 4, 2, 128, 128,
                                    kda.KDA_DTYPE_BF16, kda.KDA_DTYPE_F32, None)
    assert st == kda.KDA_ERROR_INVALID_VALUE
    st = L.kda_recurrent_step_gated(FAKE, FAKE, FAKE, FAKE, kda.KDA_GATE_SCALAR, FAKE, FAKE,
                                    FAKE, 1 << 29, 4, 128, 128, kda.KDA_DTYPE_BF16,
                                    kda.KDA_DTYPE_F32, None)
    assert st == kda.KDA_ERROR_NOT_SUPPORTED                                    # N * H >= 2^30


def test_chunk_fwd_nothing_to_do_launches_nothing():
    # zero sequences: success without touching the device
    assert _chunk(B=0, q=None, k=None, v=None, alpha=None, beta=None, o=None, ws=None) == 0
    assert _chunk(cu=FAKE, N=0, T=0, ws=None) == 0


def _step(**over):
    L = kda.lib()
    a = dict(q=FAKE, k=FAKE, v=FAKE, alpha=FAKE, beta=FAKE, state=FAKE, o=FAKE, N=4, H=2,
             Dk=128, Dv=128, act=kda.KDA_DTYPE_BF16, out=kda.KDA_DTYPE_F32, stream=None)
    a.update(over)
    return L.kda_recurrent_step(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["state"],
                                a["o"], a["N"], a["H"], a["Dk"], a["Dv"], a["act"], a["out"],
                                a["stream"])


def test_recurrent_step_argument_errors():
    assert _step(state=None) == kda.KDA_ERROR_INVALID_VALUE
    assert _step(q=FAKE + 4) == kda.KDA_ERROR_INVALID_VALUE
    assert _step(N=-1) == kda.KDA_ERROR_INVALID_VALUE
    assert _step(Dk=32) == kda.KDA_ERROR_NOT_SUPPORTED
    assert _step(act=kda.KDA_DTYPE_F32, out=kda.KDA_DTYPE_BF16) == kda.KDA_ERROR_NOT_SUPPORTED
    assert _step(out=5) == kda.KDA_ERROR_INVALID_VALUE
    assert _step(N=0) == kda.KDA_SUCCESS


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(kda, "_lib", None)
    monkeypatch.setattr(kda, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        kda.lib()


def _chunk_static(**over):
    L = kda.lib()
    a = dict(q=FAKE, k=FAKE, v=FAKE, gate=FAKE, g=kda.KDA_GATE_ALPHA, beta=FAKE, s0=None, sT=None,
             cu=None, N=0, o=FAKE, B=1, T=128, H=2, Dk=64, Dv=64, C=64, act=kda.KDA_DTYPE_BF16,
             out=kda.KDA_DTYPE_BF16, stream=None)
    a.update(over)
    return L.kda_chunk_fwd_static(a["q"], a["k"], a["v"], a["gate"], a["g"], a["beta"], a["s0"],
                                  a["sT"], a["cu"], a["N"], a["o"], a["B"], a["T"], a["H"],
                                  a["Dk"], a["Dv"], a["C"], a["act"], a["out"], a["stream"])


def test_static_entry_point_limit_and_argument_errors():
    """The static-workspace forward checks its arguments like the others and
    rejects a problem whose workspace exceeds KDA_STATIC_WORKSPACE_BYTES before
    touching any GPU (this host has none)."""
    f = kda.kda_chunk_fwd_workspace_bytes
    hdr = open(HDR).read()
    assert re.search(r"#define KDA_STATIC_WORKSPACE_BYTES \(64u << 20\)", hdr)
    assert kda.KDA_STATIC_WORKSPACE_BYTES == 64 << 20
    # 32 heads x 64 chunks of bf16 records needs about 144 MiB: rejected
    assert f(1, 4096, 32, 128, 128, False, 0, 64, kda.KDA_DTYPE_BF16) > kda.KDA_STATIC_WORKSPACE_BYTES
    assert _chunk_static(T=4096, H=32, Dk=128, Dv=128) == kda.KDA_ERROR_WORKSPACE_TOO_SMALL
    assert _chunk_static(q=None) == kda.KDA_ERROR_INVALID_VALUE
    assert _chunk_static(k=FAKE + 8) == kda.KDA_ERROR_INVALID_VALUE
    assert _chunk_static(C=96) == kda.KDA_ERROR_NOT_SUPPORTED
    assert _chunk_static(g=9) == kda.KDA_ERROR_INVALID_VALUE
    assert _chunk_static(B=0, q=None, k=None, v=None, gate=None, beta=None, o=None) == kda.KDA_SUCCESS


def test_binding_rejects_bad_tensors_before_the_call():
    """The Python binding refuses host tensors, wrong dtypes and wrong shapes
    (the kernels read raw memory)."""
    import torch
    q = torch.zeros(1, 8, 2, 64)
    with pytest.raises(ValueError, match="GPU"):
        kda.kda_chunk_fwd(q, q, q, q, torch.zeros(1, 8, 2))
    with pytest.raises(ValueError, match="GPU"):
        kda.kda_chunk_fwd_static(q, q, q, q, torch.zeros(1, 8, 2))
    with pytest.raises(ValueError, match="GPU"):
        kda.kda_recurrent_step(q[0], q[0], q[0], q[0], torch.zeros(8, 2), torch.zeros(8, 2, 64, 64))
    with pytest.raises(ValueError, match="unknown gate"):
        kda._gate_spec("sigmoid", (1, 8, 2), 64)
    assert kda._gate_spec("scalar", (1, 8, 2), 64) == (torch.float32, (1, 8, 2))
    assert kda._gate_spec("softplus", (1, 8, 2), 64) == (torch.bfloat16, (1, 8, 2, 64))
