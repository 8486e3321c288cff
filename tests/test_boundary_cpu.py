"""The C-ABI library on a machine without a GPU: it loads, exports every
function include/moe_ffn.h declares, and rejects bad arguments on the host
before touching the device (no compute calls are made here)."""
import ctypes
import os
import re

import pytest

from mixture_experts_ffn_top_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ffn.h")

S = {n: i for i, n in enumerate(moe.STATUS)}
FAKE = 0x7F0000000000  # never dereferenced: every case below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) == 31, names
    lib = moe.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(moe._SIGS) == set(names)


def test_status_strings():
    lib = moe.lib()
    for i, n in enumerate(moe.STATUS):
        assert lib.moe_status_string(i).decode() == n
    assert lib.moe_status_string(99).decode() == "MOE_ERROR_UNKNOWN"


def test_route_validation():
    f = moe.lib().moe_route
    assert f(FAKE, 0, 4, 8, 0, 1, FAKE, FAKE + 4096, None) == S["MOE_ERROR_ARGUMENT"]
    assert f(FAKE, 0, 4, 8, 9, 1, FAKE, FAKE + 4096, None) == S["MOE_ERROR_ARGUMENT"]
    assert f(FAKE, 0, -1, 8, 2, 1, FAKE, FAKE + 4096, None) == S["MOE_ERROR_SHAPE"]
    assert f(FAKE, 0, 4, 0, 1, 1, FAKE, FAKE + 4096, None) == S["MOE_ERROR_SHAPE"]
    assert f(FAKE, 7, 4, 8, 2, 1, FAKE, FAKE + 4096, None) == S["MOE_ERROR_DTYPE"]
    assert f(FAKE, 0, 4, 1025, 2, 1, FAKE, FAKE + 4096, None) == S["MOE_ERROR_UNSUPPORTED"]
    assert f(FAKE, 0, 2**31, 8, 2, 1, FAKE, FAKE + 4096, None) == S["MOE_ERROR_UNSUPPORTED"]
    assert f(None, 0, 4, 8, 2, 1, FAKE, FAKE + 4096, None) == S["MOE_ERROR_NULL_POINTER"]
    # T = 0 is a no-op, even with NULL pointers
    assert f(None, 0, 0, 8, 2, 1, None, None, None) == S["MOE_SUCCESS"]
    # weights output overlapping the logits
    assert f(FAKE, 0, 4, 8, 2, 1, FAKE + 8192, FAKE + 16, None) == S["MOE_ERROR_ARGUMENT"]


def test_dispatch_validation():
    f = moe.lib().moe_dispatch
    ws_need = moe.lib().moe_dispatch_workspace_size(64, 2, 8)
    assert ws_need > 0
    args = lambda **kw: dict(dict(idx=FAKE, T=64, k=2, E=8, x=FAKE + 2**20, dt=2, H=128, xd=FAKE + 2**21,  # noqa: E731
                                  off=FAKE + 2**22, sor=FAKE + 2**23, ros=FAKE + 2**24,
                                  ws=FAKE + 2**25, wsb=ws_need), **kw)

    def call(**kw):
        a = args(**kw)
        return f(a["idx"], a["T"], a["k"], a["E"], a["x"], a["dt"], a["H"], a["xd"], a["off"],
                 a["sor"], a["ros"], a["ws"], a["wsb"], None)

    assert call(k=0) == S["MOE_ERROR_ARGUMENT"]
    assert call(H=-8) == S["MOE_ERROR_SHAPE"]
    assert call(H=100) == S["MOE_ERROR_UNSUPPORTED"]
    assert call(dt=5) == S["MOE_ERROR_DTYPE"]
    assert call(off=None) == S["MOE_ERROR_NULL_POINTER"]
    assert call(x=None) == S["MOE_ERROR_NULL_POINTER"]
    assert call(wsb=ws_need - 1) == S["MOE_ERROR_WORKSPACE"]
    assert call(ws=FAKE + 2**25 + 8) == S["MOE_ERROR_WORKSPACE"]
    assert call(ws=None) == S["MOE_ERROR_WORKSPACE"]
    assert call(sor=FAKE + 2**24 + 64) == S["MOE_ERROR_ARGUMENT"]  # overlaps row_of_slot


def test_experts_validation():
    lib = moe.lib()
    f = lib.moe_experts_forward_dispatched
    need = lib.moe_experts_workspace_size(128, 8, 128, 256, 2)
    assert need > 128 * 256 * 2
    base = [FAKE, FAKE + 2**20, 128, 8, 128, 256, FAKE + 2**21, FAKE + 2**22, FAKE + 2**23, 2,
            FAKE + 2**24, FAKE + 2**26, need, None]

    def call(i=None, v=None):
        a = list(base)
        if i is not None:
            a[i] = v
        return f(*a)

    assert call(4, 0) == S["MOE_ERROR_SHAPE"]
    assert call(4, 132) == S["MOE_ERROR_UNSUPPORTED"]
    assert call(5, 260) == S["MOE_ERROR_UNSUPPORTED"]
    assert call(3, 2000) == S["MOE_ERROR_UNSUPPORTED"]
    assert call(9, 3) == S["MOE_ERROR_DTYPE"]
    assert call(8, None) == S["MOE_ERROR_NULL_POINTER"]
    assert call(12, need - 256) == S["MOE_ERROR_WORKSPACE"]
    assert call(10, FAKE + 2**21 + 512) == S["MOE_ERROR_ARGUMENT"]  # expert_out inside w_gate
    assert call(2, 0) == S["MOE_SUCCESS"]  # no rows: no-op


def test_combine_and_norm_validation():
    lib = moe.lib()
    c = lib.moe_combine
    assert c(FAKE, FAKE + 2**20, FAKE + 2**21, 0, 16, 0, 64, 2, FAKE + 2**22, None) == S["MOE_ERROR_SHAPE"]
    assert c(FAKE, FAKE + 2**20, FAKE + 2**21, 9, 16, 2, 64, 2, FAKE + 2**22, None) == S["MOE_ERROR_DTYPE"]
    assert c(FAKE, FAKE + 2**20, FAKE + 2**21, 0, 16, 2, 60, 2, FAKE + 2**22, None) == S["MOE_ERROR_UNSUPPORTED"]
    # an fp32 row of 2^29 elements is 2 GiB: past the 32-bit range of a row's buffer resource
    assert c(FAKE, FAKE + 2**20, FAKE + 2**21, 0, 1, 1, 2**29, 0, FAKE + 2**22, None) == S["MOE_ERROR_UNSUPPORTED"]
    assert c(FAKE, FAKE + 2**20, FAKE + 2**21, 0, 1, 1, 2**28, 0, FAKE + 2**22, None) != S["MOE_ERROR_UNSUPPORTED"]
    assert c(FAKE, FAKE + 2**20, FAKE + 2**21, 0, 16, 2, 64, 2, FAKE + 64, None) == S["MOE_ERROR_ARGUMENT"]
    n = lib.moe_combine_add_rmsnorm
    args = [FAKE, FAKE + 2**20, FAKE + 2**21, 0, None, FAKE + 2**22, FAKE + 2**23, 1e-6, 16, 2, 64,
            2, FAKE + 2**24, FAKE + 2**25, FAKE + 2**26, None]
    for eps in (0.0, -1.0, float("inf"), float("nan")):
        a = list(args)
        a[7] = eps
        assert n(*a) == S["MOE_ERROR_ARGUMENT"], eps
    a = list(args)
    a[10] = 40000
    assert n(*a) == S["MOE_ERROR_UNSUPPORTED"]
    a = list(args)
    a[13] = FAKE + 2**24 + 64  # x_out overlaps y
    assert n(*a) == S["MOE_ERROR_ARGUMENT"]


def test_forward_validation_and_workspace_query():
    lib = moe.lib()
    q = lib.moe_forward_workspace_size
    need = q(4096, 4096, 14336, 8, 2, 2, 0)
    # h [T*k, I] and expert_out [T*k, H] in bf16 dominate
    assert need >= 4096 * 2 * (14336 + 4096) * 2
    assert q(4, 128, 256, 8, 9, 2, 0) == 0
    f = lib.moe_forward
    # x, logits, logits_dt, T, H, I, E, k, renorm, wg, wu, wd, dt, out, indices_out, weights_out,
    # offsets_out, ws, ws_bytes, stage_events, stream
    base = [FAKE, FAKE + 2**20, 0, 64, 128, 256, 8, 2, 1, FAKE + 2**21, FAKE + 2**22, FAKE + 2**23,
            0, FAKE + 2**24, None, None, None, FAKE + 2**26, q(64, 128, 256, 8, 2, 0, 0), None, None]

    def call(i=None, v=None):
        a = list(base)
        if i is not None:
            a[i] = v
        return f(*a)

    assert call(7, 9) == S["MOE_ERROR_ARGUMENT"]
    assert call(12, 4) == S["MOE_ERROR_DTYPE"]
    assert call(5, 250) == S["MOE_ERROR_UNSUPPORTED"]
    assert call(18, 10) == S["MOE_ERROR_WORKSPACE"]
    assert call(0, None) == S["MOE_ERROR_NULL_POINTER"]
    assert call(3, 0) == S["MOE_SUCCESS"]
    assert call(13, FAKE + 64) == S["MOE_ERROR_ARGUMENT"]  # out overlaps x
    assert call(16, FAKE + 2**24 + 64) == S["MOE_ERROR_ARGUMENT"]  # offsets_out overlaps out
    assert call(16, FAKE + 2**26 + 256) == S["MOE_ERROR_ARGUMENT"]  # offsets_out inside the workspace


def test_grouped_route_validation():
    f = moe.lib().moe_route_sigmoid_grouped
    # logits, dt, T, E, bias, k, groups, selected, top_two, renorm, scale, idx, w, stream
    base = [FAKE, 0, 4, 256, None, 8, 8, 4, 1, 1, 2.5, FAKE + 2**20, FAKE + 2**21, None]

    def call(**kw):
        a = list(base)
        names = ["logits", "dt", "T", "E", "bias", "k", "groups", "sel", "two", "renorm", "scale"]
        for n, v in kw.items():
            a[names.index(n)] = v
        return f(*a)

    assert call(groups=3) == S["MOE_ERROR_ARGUMENT"]        # does not divide E
    assert call(groups=256) == S["MOE_ERROR_ARGUMENT"]      # more than 128 groups
    assert call(groups=0) == S["MOE_ERROR_ARGUMENT"]
    assert call(sel=0) == S["MOE_ERROR_ARGUMENT"]
    assert call(sel=9) == S["MOE_ERROR_ARGUMENT"]
    assert call(k=65) == S["MOE_ERROR_ARGUMENT"]            # more than 64
    assert call(k=33, sel=1) == S["MOE_ERROR_ARGUMENT"]     # more than the kept experts
    assert call(E=128, groups=128, k=4) == S["MOE_ERROR_ARGUMENT"]  # top-two with one expert a group
    for sc in (0.0, -1.0, float("inf"), float("nan")):
        assert call(scale=sc) == S["MOE_ERROR_ARGUMENT"], sc
    assert call(E=2048, groups=8) == S["MOE_ERROR_UNSUPPORTED"]
    assert call(dt=7) == S["MOE_ERROR_DTYPE"]
    assert call(logits=None) == S["MOE_ERROR_NULL_POINTER"]
    assert call(T=0, logits=None) == S["MOE_SUCCESS"]
    assert call(bias=FAKE + 2**20 + 8) == S["MOE_ERROR_ARGUMENT"]  # bias overlaps indices
    g = moe.lib().moe_forward_sigmoid_grouped
    q = moe.lib().moe_forward_workspace_size(64, 128, 256, 16, 4, 2, 0)
    fb = [FAKE, FAKE + 2**20, 0, 64, 128, 256, 16, None, 4, 4, 2, 1, 1, 1.0, FAKE + 2**21,
          FAKE + 2**22, FAKE + 2**23, 2, FAKE + 2**24, None, None, None, FAKE + 2**26, q, None, None]
    a = list(fb)
    a[9] = 5  # groups must divide E = 16
    assert g(*a) == S["MOE_ERROR_ARGUMENT"]
    a = list(fb)
    a[13] = 0.0
    assert g(*a) == S["MOE_ERROR_ARGUMENT"]
    a = list(fb)
    a[3] = 0
    assert g(*a) == S["MOE_SUCCESS"]


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(moe, "_LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="missing"):
        moe.lib()


def test_quant_validation():
    f = moe.lib().moe_experts_forward_dispatched_quant
    need = moe.lib().moe_experts_quant_workspace_size(64, 16, 512, 384, 2)
    # x, offsets, rows, E, H, I, wg, wu, wd, bits, groups, sg, su, sd, og, ou, od, dt, out, ws, wsb, stream
    base = [FAKE, FAKE + 2**20, 64, 16, 512, 384, FAKE + 2**21, FAKE + 2**22, FAKE + 2**23, 8, 1,
            FAKE + 2**24, FAKE + 2**25, FAKE + 2**26, None, None, None, 2, FAKE + 2**27, FAKE + 2**28, need, None]

    def call(i=None, v=None, **kw):
        a = list(base)
        if i is not None:
            a[i] = v
        return f(*a)

    assert call(9, 5) == S["MOE_ERROR_ARGUMENT"]          # bits
    assert call(10, 3) == S["MOE_ERROR_ARGUMENT"]         # groups does not divide 384? 512 % 3
    assert call(10, 4) == S["MOE_ERROR_ARGUMENT"]         # per-group with INT8
    assert call(17, 0) == S["MOE_ERROR_UNSUPPORTED"]      # fp32
    assert call(2, 65) == S["MOE_ERROR_UNSUPPORTED"]      # rows > 4 * E: not a decode batch
    a = list(base)
    a[9], a[10] = 4, 2                                    # INT4, 2 groups: 512/2 and 384/2 not multiples of 128
    assert f(*a) == S["MOE_ERROR_UNSUPPORTED"]
    assert call(11, None) == S["MOE_ERROR_NULL_POINTER"]  # scale missing
    assert call(20, need - 1) == S["MOE_ERROR_WORKSPACE"]
    assert call(2, 0) == S["MOE_SUCCESS"]
    a = list(base)
    a[4], a[5] = 65536, 65536                             # one expert's INT8 codes: 4 GiB
    assert f(*a) == S["MOE_ERROR_UNSUPPORTED"]


def test_training_validation():
    lib = moe.lib()
    # router weights: logits, logits_dt, indices, idx_dt, T, E, k, scoring, normalize, scale, weights, stream
    f = lib.moe_router_weights
    ok = [FAKE, 0, FAKE + 2**20, 0, 4, 8, 2, 0, 1, 1.0, FAKE + 2**21, None]

    def call(fn, base, i, v):
        a = list(base)
        a[i] = v
        return fn(*a)
    assert call(f, ok, 6, 0) == S["MOE_ERROR_ARGUMENT"]       # top_k 0
    assert call(f, ok, 6, 9) == S["MOE_ERROR_ARGUMENT"]       # top_k > E
    assert call(f, ok, 7, 2) == S["MOE_ERROR_ARGUMENT"]       # unknown scoring
    assert call(f, ok, 9, 0.0) == S["MOE_ERROR_ARGUMENT"]     # scale must be > 0
    assert call(f, ok, 9, float("inf")) == S["MOE_ERROR_ARGUMENT"]
    assert call(f, ok, 3, 3) == S["MOE_ERROR_DTYPE"]          # index dtype
    assert call(f, ok, 1, 5) == S["MOE_ERROR_DTYPE"]
    assert call(f, ok, 5, 1025) == S["MOE_ERROR_UNSUPPORTED"]
    assert call(f, ok, 10, None) == S["MOE_ERROR_NULL_POINTER"]
    assert call(f, ok, 10, FAKE + 8) == S["MOE_ERROR_ARGUMENT"]  # output overlaps the logits
    assert call(f, ok, 4, 0) == S["MOE_SUCCESS"]
    a = list(ok)
    a[5], a[6] = 128, 65
    assert f(*a) == S["MOE_ERROR_ARGUMENT"]                    # top_k > 64
    g = lib.moe_router_backward
    okb = [FAKE, 0, FAKE + 2**20, 0, FAKE + 2**21, 4, 8, 2, 1, 0, 1.0, FAKE + 2**22, None]
    assert call(g, okb, 4, None) == S["MOE_ERROR_NULL_POINTER"]  # grad_weights
    assert call(g, okb, 11, None) == S["MOE_ERROR_NULL_POINTER"]
    assert call(g, okb, 11, FAKE + 2**20 + 4) == S["MOE_ERROR_ARGUMENT"]  # overlaps the indices
    # combine backward: y, ros, w, w_dt, go, T, k, H, dt, dexp, dw, stream
    c = lib.moe_combine_backward
    okc = [FAKE, FAKE + 2**20, FAKE + 2**21, 0, FAKE + 2**22, 4, 2, 64, 8, 2, FAKE + 2**23, FAKE + 2**24, None]
    assert call(c, okc, 7, 60) == S["MOE_ERROR_UNSUPPORTED"]
    assert call(c, okc, 9, 9) == S["MOE_ERROR_DTYPE"]
    assert call(c, okc, 8, 9) == S["MOE_ERROR_SHAPE"]           # rows > T * top_k
    assert call(c, okc, 11, None) == S["MOE_ERROR_NULL_POINTER"]
    assert call(c, okc, 10, FAKE + 16) == S["MOE_ERROR_ARGUMENT"]
    assert call(c, okc, 5, 0) == S["MOE_ERROR_SHAPE"]            # rows 8 > 0 * 2
    a = list(okc)
    a[5], a[8] = 0, 0
    assert c(*a) == S["MOE_SUCCESS"]
    d = lib.moe_dispatch_backward
    okd = [FAKE, FAKE + 2**20, 4, 2, 64, 8, 2, FAKE + 2**21, None]
    assert call(d, okd, 7, FAKE + 64) == S["MOE_ERROR_ARGUMENT"]
    assert call(d, okd, 3, 0) == S["MOE_ERROR_SHAPE"]
    assert call(d, okd, 5, -1) == S["MOE_ERROR_SHAPE"]
    a = list(okd)
    a[2], a[5] = 0, 0
    assert d(*a) == S["MOE_SUCCESS"]
    # experts training forward / backward
    need_f = lib.moe_experts_forward_training_workspace_size(64, 8, 512, 384, 2)
    need_b = lib.moe_experts_backward_workspace_size(64, 8, 512, 384, 2)
    assert need_f > 0 and need_b >= 64 * 384 * 2 * 2
    assert lib.moe_experts_backward_workspace_size(64, 8, 512, 384, 0) == 0  # fp32 unsupported
    assert lib.moe_experts_training_cache_size(64, 384, 2) == 64 * 3 * 384 * 2
    ft = lib.moe_experts_forward_training
    okf = [FAKE, FAKE + 2**20, 64, 8, 512, 384, FAKE + 2**24, FAKE + 2**25, FAKE + 2**26, 2,
           FAKE + 2**27, FAKE + 2**28, FAKE + 2**29, need_f, None]
    assert call(ft, okf, 9, 0) == S["MOE_ERROR_UNSUPPORTED"]
    assert call(ft, okf, 5, 380) == S["MOE_ERROR_UNSUPPORTED"]
    assert call(ft, okf, 11, None) == S["MOE_ERROR_NULL_POINTER"]
    assert call(ft, okf, 13, need_f - 1) == S["MOE_ERROR_WORKSPACE"]
    assert call(ft, okf, 12, FAKE + 2**29 + 8) == S["MOE_ERROR_WORKSPACE"]  # misaligned
    assert call(ft, okf, 11, FAKE + 2**27 + 64) == S["MOE_ERROR_ARGUMENT"]  # cache overlaps expert_out
    assert call(ft, okf, 2, 0) == S["MOE_SUCCESS"]
    assert call(ft, okf, 4, (1 << 22) + 8) == S["MOE_ERROR_UNSUPPORTED"]   # H past 2^22
    assert call(ft, okf, 5, (1 << 21) + 8) == S["MOE_ERROR_UNSUPPORTED"]   # 2I past 2^22
    bw = lib.moe_experts_backward
    okw = [FAKE, FAKE + 2**20, 64, 8, 512, 384, FAKE + 2**24, FAKE + 2**25, FAKE + 2**26, 2,
           FAKE + 2**27, FAKE + 2**28, FAKE + 2**29, FAKE + 2**31, FAKE + 2**32, FAKE + 2**33,
           FAKE + 2**34, need_b, None]
    assert call(bw, okw, 9, 0) == S["MOE_ERROR_UNSUPPORTED"]
    assert call(bw, okw, 14, None) == S["MOE_ERROR_NULL_POINTER"]
    assert call(bw, okw, 17, need_b - 1) == S["MOE_ERROR_WORKSPACE"]
    assert call(bw, okw, 14, FAKE + 2**31 + 4) == S["MOE_ERROR_ARGUMENT"]  # dup overlaps dgate


def test_gemm_operands_of_2_gib_are_unsupported():
    """The bf16 / f16 expert GEMMs address operands with 32-bit byte offsets:
    every entry point that reaches them rejects, before any device query, an
    operand of 2^31 bytes or more, and accepts the same shape one size step
    below (the call then fails later, on the fake pointers, with another
    status). fp32 experts use 64-bit addressing and are not limited."""
    lib = moe.lib()
    U = S["MOE_ERROR_UNSUPPORTED"]
    ws = FAKE + 2**40

    def experts(rows, H, I_, dt=2):
        return lib.moe_experts_forward_dispatched(FAKE, FAKE + 2**38, rows, 8, H, I_, FAKE + 2**39,
                                                  FAKE + 2**41, FAKE + 2**42, dt, FAKE + 2**43, ws,
                                                  2**44, None)

    # h [rows, I]: 131072 rows of the Mixtral expert width (3.76 GB) against 65536 (1.88 GB)
    assert experts(131072, 4096, 14336) == U
    assert experts(65536, 4096, 14336) != U
    assert experts(131072, 4096, 14336, dt=1) == U    # f16 too
    assert experts(131072, 4096, 14336, dt=0) != U    # fp32: 64-bit pointers
    # x_disp [rows, H]: 16384 rows of 65536 elements is exactly 2^31 bytes
    assert experts(16384, 65536, 8) == U
    assert experts(16383, 65536, 8) != U
    # one expert's weight matrix [I, H]: 32768 x 32768 bf16 is 2^31 bytes
    assert experts(8, 32768, 32768) == U
    assert experts(8, 32768, 32760) != U
    # a 256-row fp32 output tile of H = 2^21 columns
    assert experts(1, 2**21, 8) == U
    assert experts(1, 2**21 - 8, 8) != U

    def gate_up(rows, div, H, I_):
        return lib.moe_experts_gate_up(FAKE, FAKE + 2**38, div, FAKE + 2**37, rows, 8, H, I_, FAKE + 2**39,
                                       FAKE + 2**41, 2, FAKE + 2**43, ws, 2**44, None)

    # token rows read through the map: ceil(rows / div) rows of x
    assert gate_up(131072, 8, 65536, 8) == U
    assert gate_up(131072, 9, 65536, 8) != U

    def down(rows, H, I_):
        return lib.moe_experts_down(FAKE, FAKE + 2**38, rows, 8, H, I_, FAKE + 2**39, 2, FAKE + 2**43, ws,
                                    2**44, None)

    assert down(131072, 4096, 14336) == U
    assert down(65536, 4096, 14336) != U

    def forward(T, k, H, I_, grouped=False):
        if grouped:
            return lib.moe_forward_sigmoid_grouped(FAKE, FAKE + 2**36, 0, T, H, I_, 8, None, k, 1, 1, 0, 1,
                                                   1.0, FAKE + 2**39, FAKE + 2**41, FAKE + 2**42, 2,
                                                   FAKE + 2**43, None, None, None, ws, 2**45, None, None)
        return lib.moe_forward(FAKE, FAKE + 2**36, 0, T, H, I_, 8, k, 1, FAKE + 2**39, FAKE + 2**41,
                               FAKE + 2**42, 2, FAKE + 2**43, None, None, None, ws, 2**45, None, None)

    assert forward(65536, 2, 4096, 14336) == U          # h = 131072 x 14336 bf16
    assert forward(32768, 2, 4096, 14336) != U
    assert forward(65536, 2, 4096, 14336, grouped=True) == U
    assert forward(32768, 2, 4096, 14336, grouped=True) != U
    assert forward(16384, 1, 65536, 8) == U             # x [T, H] read by the gate/up GEMM
    assert forward(16383, 1, 65536, 8) != U

    # the experts' training forward runs the same GEMMs
    def train(rows, H, I_):
        return lib.moe_experts_forward_training(FAKE, FAKE + 2**38, rows, 8, H, I_, FAKE + 2**39,
                                                FAKE + 2**41, FAKE + 2**42, 2, FAKE + 2**43, FAKE + 2**44,
                                                ws, 2**45, None)

    assert train(131072, 4096, 14336) == U
    assert train(65536, 4096, 14336) != U


def test_forward_noalloc_validation():
    """moe_forward_noalloc checks its arguments like moe_forward, before it
    looks up the device or its scratch array."""
    f = moe.lib().moe_forward_noalloc
    # x, logits, logits_dt, T, H, I, E, k, renorm, wg, wu, wd, dt, out, idx, w, offs, events, stream
    base = [FAKE, FAKE + 2**20, 0, 64, 128, 256, 8, 2, 1, FAKE + 2**21, FAKE + 2**22, FAKE + 2**23,
            2, FAKE + 2**24, None, None, None, None, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)

    assert call(7, 9) == S["MOE_ERROR_ARGUMENT"]     # top_k > E
    assert call(4, 0) == S["MOE_ERROR_SHAPE"]
    assert call(2, 7) == S["MOE_ERROR_DTYPE"]        # logits dtype
    assert call(6, 2000) == S["MOE_ERROR_UNSUPPORTED"]
    assert call(3, 0) == S["MOE_SUCCESS"]            # no tokens: nothing to do


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU's share; asked for several it exits with status 2 and says so,
    before importing torch or touching a device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
