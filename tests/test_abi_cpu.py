"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects invalid arguments on the host before any HIP call
(the format's error catalogue: nuvec-core "invalid_arguments_are_rejected",
"gather_qmm_selects_batches")."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moegq.h")


@pytest.fixture(scope="module")
def L():
    import moe_expert_gathered_amd as m
    if not os.path.exists(m.library_path):
        pytest.fail("libmoegq.so not built (run `python -m moe_expert_gathered_amd.build`)")
    return m.lib()


def header_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moegq_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    syms = header_symbols()
    assert len(syms) >= 15
    for s in syms:
        assert hasattr(L, s), s


def test_status_strings_and_version(L):
    assert L.moegq_version().startswith(b"moegq")
    for code in range(0, -12, -1):
        assert L.moegq_status_string(code) != b"unknown status"


FAKE = ctypes.c_void_p(0x100000)       # never dereferenced: every call below fails validation


def gq(L, **kw):
    a = dict(x=FAKE, x_dtype=0, X=4, M=1, K=256, w=FAKE, w_dtype=5, s=FAKE, b=FAKE, E=8, N=64,
             lhs=None, lhs_div=1, rhs=FAKE, idx_dtype=4, P=4, sorted=0, transpose=1, gs=64, bits=4,
             out=FAKE, ws=None, wsb=0)
    a.update(kw)
    return L.moegq_gather_qmm(a["x"], a["x_dtype"], a["X"], a["M"], a["K"], a["w"], a["w_dtype"], a["s"], a["b"],
                              a["E"], a["N"], a["lhs"], a["lhs_div"], a["rhs"], a["idx_dtype"], a["P"], a["sorted"],
                              a["transpose"], a["gs"], a["bits"], a["out"], a["ws"], a["wsb"], None)


def test_gather_qmm_error_catalogue(L):
    import moe_expert_gathered_amd as m
    assert gq(L, gs=48) == -3                       # group size 48
    assert gq(L, bits=7) == -2                      # bits 7
    assert gq(L, bits=3, K=96) == -4                # 3 bits: the format's checks (vector-unit route)
    assert gq(L, bits=6, gs=48) == -3
    assert gq(L, bits=0) == -2 and gq(L, bits=9) == -2
    assert gq(L, K=96) == -4                        # K not divisible by the group size
    assert gq(L, x_dtype=m.I32) == -5               # integer activations
    assert gq(L, x_dtype=m.F64) == -5               # f64 activations
    assert gq(L, x_dtype=m.F32, K=96) == -4         # f32 activations take the same format checks
    assert gq(L, w_dtype=m.F32) == -5               # packed weights must be u32
    assert gq(L, idx_dtype=m.F32) == -5             # float indices
    assert gq(L, transpose=0, N=96) == -4           # without the transpose the groups run along N
    assert gq(L, transpose=0, N=64, gs=128) == -4
    # the vector-unit route's K split needs its workspace
    assert gq(L, transpose=0, X=1, P=1, N=4096, K=4096) == -7
    assert gq(L, x_dtype=m.F16, X=1, P=1, N=64, K=8192) == -7
    assert gq(L, rhs=None) == -1
    assert gq(L, x=ctypes.c_void_p(0x100008)) == -11
    assert gq(L, lhs_div=0) == -4
    assert gq(L, lhs_div=1, X=2) == -4              # pair rows past x's batch
    assert gq(L, M=40) == -7                        # tile route needs a workspace
    assert gq(L, sorted=1, P=128, X=128) == -7      # grouped route needs a workspace
    # empty products launch nothing and succeed, even with null pointers
    assert gq(L, P=0, x=None, w=None, out=None, rhs=None) == 0
    assert gq(L, M=0, x=None, out=None) == 0


def test_gather_qmm_workspace_query(L):
    import moe_expert_gathered_amd as m
    q = L.moegq_gather_qmm_workspace_bytes
    # vector route: [splits, P, M, N] fp32 partial sums
    # transpose=0, one pair, 4096 x 4096 4-bit: 2 column strips (workgroup items)
    # -> 64 splits of 64 rows
    assert q(1, 1, 1, 4096, 4096, m.BF16, 0, 4, 0) == 64 * 4096 * 4
    # float16, transposed, N = 64, K = 8192: 16 row blocks (wave items) -> 4 splits of 256 words
    assert q(1, 1, 1, 64, 8192, m.F16, 1, 4, 0) == 4 * 64 * 4
    # enough work items: no split, no workspace
    assert q(4096, 8, 1, 64, 256, m.F32, 1, 4, 0) == 0
    # bf16 with the transpose: the existing routes
    assert q(8, 8, 1, 64, 256, m.BF16, 1, 4, 0) == 0
    assert q(8, 8, 4, 64, 256, m.BF16, 1, 4, 0) == 0
    assert q(8, 8, 40, 64, 256, m.BF16, 1, 4, 0) == L.moegq_workspace_bytes(m.OP_GATHER_QMM, 8, 8, 40, 0)
    assert q(0, 8, 1, 64, 256, m.BF16, 1, 4, 0) == 0
    # every width of the format has a workspace size on the vector route
    assert q(1, 1, 1, 4096, 4096, m.BF16, 1, 3, 0) > 0
    assert q(1, 1, 1, 4096, 4096, m.BF16, 1, 7, 0) == 0
    # the gate/up variant rejects the vector route
    p = FAKE
    assert L.moegq_gather_qmm_glu(p, m.F32, 4, 1, 256, p, p, p, p, p, p, 8, 64, None, 1, p, 4, 4, 0, 64, 4, p,
                                  None, 0, None) == -6


def test_gather_qmm_mx_validates(L):
    import moe_expert_gathered_amd as m
    p = FAKE
    mx = lambda **kw: L.moegq_gather_qmm_mx(*[kw.get(k, v) for k, v in (
        ("x", p), ("xd", 0), ("X", 4), ("M", 1), ("K", 256), ("w", p), ("s", p), ("E", 8), ("N", 64), ("lhs", None),
        ("div", 1), ("rhs", p), ("idt", 4), ("P", 4), ("tr", 1), ("mode", 2), ("out", p), ("ws", None), ("wsb", 0),
        ("st", None))])
    assert mx(mode=0) == -2 and mx(mode=3) == -2     # only mxfp4 (1) and mxfp8 (2)
    assert mx(K=200) == -4                            # blocks of 32 along the packed axis
    assert mx(tr=0, N=48) == -4
    assert mx(xd=m.F64) == -5 and mx(idt=m.F32) == -5
    assert mx(rhs=None) == -1 and mx(s=None) == -1
    assert mx(P=0, x=None, w=None, s=None, out=None, rhs=None) == 0
    assert mx(X=1, P=1, N=4096, K=4096, tr=0) == -7  # the K split needs its workspace
    q = L.moegq_gather_qmm_mx_workspace_bytes
    assert q(1, 1, 4096, 4096, 0, 2) == 64 * 4096 * 4 and q(1, 1, 4096, 4096, 0, 5) == 0
    assert q(4096, 1, 64, 256, 1, 1) == 0


def test_other_entry_points_validate(L):
    p = FAKE
    # affine_qmm: inner-size / group checks
    assert L.moegq_affine_qmm(p, 0, 3, 63, p, 5, p, p, 16, 1, 64, 4, None, p, None) == -4
    assert L.moegq_affine_qmm(p, 3, 3, 64, p, 5, p, p, 16, 1, 64, 4, None, p, None) == -5
    assert L.moegq_affine_qmm(None, 0, 0, 64, None, 5, None, None, 16, 1, 64, 4, None, None, None) == 0
    # switch_glu
    args = [p, 4, 256, 128, 8, p, 2] + [p] * 9
    assert L.moegq_switch_glu(*args, 64, 4, 1, 0, 0, p, None, None, 0, None) == -7   # no workspace
    assert L.moegq_switch_glu(*args, 64, 4, 2, 0, 0, p, None, None, 0, None) == -1   # sorted needs inv
    assert L.moegq_switch_glu(*args, 64, 4, 1, 0, 48, p, None, None, 0, None) == -4  # bm
    assert L.moegq_switch_glu(*args, 64, 4, 7, 0, 0, p, None, None, 0, None) == -4   # mode
    assert L.moegq_switch_glu(p, 0, 256, 128, 8, p, 2, *[p] * 9, 64, 4, 1, 0, 0, p, None, None, 0, None) == 0
    # combine
    assert L.moegq_moe_combine(p, None, p, None, 4, 8, 12, p, None) == -4           # H % 8
    assert L.moegq_moe_combine(None, None, None, None, 0, 8, 16, None, None) == 0
    assert L.moegq_moe_combine_unfused(p, None, p, None, 4, 8, 16, p, None, 0, None) == -7
    # sort / schedule
    assert L.moegq_sort_pairs(p, 2, 4, 8, 16, None, None, None, p, p, p, None, 0, None) == -5  # float idx
    assert L.moegq_sort_pairs(p, 4, 4, 8, 2000, None, None, None, p, p, p, None, 0, None) == -6
    assert L.moegq_sort_pairs(p, 4, 4, 8, 16, None, None, None, p, p, p, None, 0, None) == -7  # no workspace
    assert L.moegq_sort_pairs(None, 4, 0, 8, 16, None, None, None, p, p, p, None, 0, None) == -1
    assert L.moegq_schedule_tiles(p, 4, 33, 16, 0, p, 3, p, None) == -7            # capacity
    assert L.moegq_schedule_tiles(p, 4, 33, 24, 0, p, 100, p, None) == -4          # bm
    assert L.moegq_selfcheck(None, 0, None) == -7
    # whole prefill layer
    lay = lambda T, H, I, ws, wsb, sh=p: L.moegq_moe_prefill(p, T, H, I, 8, p, 2, p, *[p] * 9, sh, *[p] * 11,
                                                               64, 4, p, ws, wsb, None)
    assert lay(64, 1024, 512, None, 0) == -7                                        # no workspace
    assert lay(64, 256, 96, None, 0) == -4                                          # I % 64
    assert lay(64, 320, 512, p, 1 << 30) == -6                                      # H % 128
    assert lay(64, 1024, 128, p, 1 << 30) == -6                                     # I % (8 * 64)
    assert lay(0, 256, 128, None, 0) == 0
    assert L.moegq_moe_combine_gated(p, None, p, None, p, 4, 8, 16, p, None) == -1  # shared required
    # unquantized gather_mm
    assert L.moegq_gather_mm(p, 4, 1, 100, p, 8, 16, None, 1, p, 4, 0, p, None, 0, None) == -4      # K % 8
    assert L.moegq_gather_mm(p, 4, 1, 128, p, 8, 16, None, 1, None, 4, 0, p, None, 0, None) == -1   # no rhs
    assert L.moegq_gather_mm(p, 4, 1, 128, p, 8, 16, None, 0, p, 4, 0, p, None, 0, None) == -4      # lhs_div
    assert L.moegq_gather_mm(p, 2, 1, 128, p, 8, 16, None, 1, p, 4, 0, p, None, 0, None) == -4      # x rows
    assert L.moegq_gather_mm(p, 4, 3, 96, p, 8, 16, None, 1, p, 4, 0, p, p, 1 << 20, None) == -6    # M > 1, K % 128
    assert L.moegq_gather_mm(None, 4, 1, 128, None, 8, 16, None, 1, None, 0, 0, None, None, 0, None) == 0
    # router
    assert L.moegq_route(p, 4, 2000, 8, p, p, None) == -4                           # E > 1024
    assert L.moegq_route(p, 4, 16, 17, p, p, None) == -4                            # top_k > E
    assert L.moegq_route(p, 4, 256, 65, p, p, None) == -4                           # top_k > 64
    assert L.moegq_route(p, 4, 256, 0, p, p, None) == -4
    assert L.moegq_route(None, 4, 256, 8, p, p, None) == -1
    assert L.moegq_route(None, 0, 256, 8, None, None, None) == 0


def test_workspace_sizes(L):
    import moe_expert_gathered_amd as m
    assert m.workspace_bytes(m.OP_SWITCH_GLU_DECODE, 8, 288, 2048) >= 8 * 2048 * 2
    big = m.workspace_bytes(m.OP_SWITCH_GLU_SORTED, 16384, 256, 512, 16)
    assert big >= 16384 * 512 * 2 + 3 * 16384 * 4
    assert m.workspace_bytes(m.OP_SWITCH_GLU_SORTED, 16384, 256, 512, 0) == big
    assert m.workspace_bytes(99, 1, 1, 1, 0) == 0
    assert m.workspace_bytes(m.OP_SORT_PAIRS, 16384, 256, 0, 0) >= 16 * 256 * 4
    lay = m.moe_prefill_workspace_bytes(2048, 8, 256, 2048, 512, True)
    # h and y for the routed and shared rows, the fp16 activations
    assert lay >= (16384 + 2048) * (512 + 2048) * 2 + 2048 * 2048 * 2
    assert m.moe_prefill_workspace_bytes(2048, 8, 256, 2048, 512, False) < lay
    assert m.workspace_bytes(m.OP_GATHER_MM, 100, 8, 3, 0) >= 12 * 100       # per-pair tiles
    assert m.workspace_bytes(m.OP_GATHER_MM, 4096, 64, 1, 0) >= 4 * 65 + 12 * (4096 // 64)
    assert m.switch_glu_mode(1, 8, 288) == m.MODE_DECODE
    assert m.switch_glu_mode(2048, 8, 256) == m.MODE_SORTED


def test_no_cpu_fallback(tmp_path, monkeypatch):
    """The binding refuses to run without the library (no silent fallback)."""
    import importlib
    import moe_expert_gathered_amd as m
    monkeypatch.setattr(m, "library_path", str(tmp_path / "missing.so"))
    monkeypatch.setattr(m, "_LIB", None)
    with pytest.raises(ImportError):
        m.lib()
    importlib.reload(m)


def _mat(E, N, K, bits=4, gs=64, wdt=None):
    import torch
    lead = (E,) if E else ()
    return (torch.zeros(lead + (N, K * bits // 32), dtype=wdt or torch.int32),
            torch.zeros(lead + (N, K // gs), dtype=torch.bfloat16),
            torch.zeros(lead + (N, K // gs), dtype=torch.bfloat16))


def test_binding_rejects_wrong_dtypes_and_shapes():
    """The layer wrappers check dtypes and shapes before any launch (the C
    entry points take raw pointers): int64 indices (as torch.topk returns),
    float32 scores or activations, mismatched index and score shapes, and
    weights of the wrong size raise ValueError, here on host tensors."""
    import torch
    import moe_expert_gathered_amd as m
    T, H, I, E, k = 4, 256, 128, 8, 2
    x = torch.zeros((T, H), dtype=torch.bfloat16)
    idx = torch.zeros((T, k), dtype=torch.int32)
    sc = torch.zeros((T, k), dtype=torch.bfloat16)
    ex = (_mat(E, I, H), _mat(E, I, H), _mat(E, H, I))

    def raises(fn, *a, **kw):
        with pytest.raises(ValueError):
            fn(*a, **kw)

    for fn in (m.moe_decode, m.moe_prefill):
        raises(fn, x, idx.long(), sc, *ex)                           # int64 indices
        raises(fn, x, idx, sc.float(), *ex)                          # fp32 scores
        raises(fn, x.float(), idx, sc, *ex)                          # fp32 activations
        raises(fn, x, idx, sc[:, :1], *ex)                           # scores shape
        raises(fn, x, idx, sc, _mat(E, I, H + 64), *ex[1:])          # gate K mismatch
        raises(fn, x, idx, sc, ex[0], ex[1], _mat(E, H, I, bits=8))  # down packed for 8 bits, called with 4
        # the right arguments pass every check and stop only at the device check
        with pytest.raises(ValueError, match="device tensors"):
            fn(x, idx, sc, *ex)
    raises(m.moe_decode, x, idx, sc, *ex, shared=torch.zeros((T, H + 8), dtype=torch.bfloat16))
    raises(m.switch_glu, x, idx.long(), *ex)
    raises(m.switch_glu, x, idx, *ex, y=torch.zeros((T * k, H), dtype=torch.float32))
    y = torch.zeros((T * k, H), dtype=torch.bfloat16)
    raises(m.moe_combine, y, idx.reshape(-1).long(), sc)             # int64 inverse permutation
    raises(m.moe_combine, y, None, sc.float())
    raises(m.moe_combine, y[: T * k - 1], None, sc)                  # too few expert rows
    raises(m.moe_combine_unfused, y, None, sc, torch.zeros((T, H), dtype=torch.float32))
    raises(m.moe_combine_gated, y, None, sc, torch.zeros((T, H), dtype=torch.bfloat16),
           torch.zeros(T + 1, dtype=torch.bfloat16))
    raises(m.sort_pairs, idx.long(), E)
    raises(m.affine_qmm, x, *_mat(0, I, H, gs=32))                   # scales for group size 32, called with 64
    raises(m.affine_qmm, x, *_mat(0, I, H), residual=torch.zeros((T, I), dtype=torch.float32))
    raises(m.gather_qmm_glu, x, _mat(E, I, H), _mat(E, I, H), torch.zeros(T * k, dtype=torch.int64))
    raises(m.rms_norm, x, torch.zeros(H + 1, dtype=torch.bfloat16))
    raises(m.gather_mm, x.float(), torch.zeros((E, I, H), dtype=torch.bfloat16), idx.reshape(-1))


def test_prefill_layout_query(L):
    """The host-side layout query of the whole-layer workspace: pieces in
    order, 256-byte aligned, inside the workspace size, with the schedule
    parameters (128/32-row tiles, 4 column blocks at inter 512)."""
    import moe_expert_gathered_amd as m
    for T, shared in ((1, True), (2048, True), (4123, False)):
        lay = m.moe_prefill_layout(T, 8, 256, 2048, 512, shared)
        o = list(lay["offsets"].values())
        assert o == sorted(o) and all(v % 256 == 0 for v in o)
        assert o[-1] + 2 * (8 * T + 2 * T) * 2048 <= m.moe_prefill_workspace_bytes(T, 8, 256, 2048, 512, shared)
        assert (lay["big"], lay["small"], lay["col_blocks"]) == (128, 32, 4)
        assert lay["slots"] > 0 and min(lay["caps"]) > 0
    off = (ctypes.c_int64 * 9)()
    caps = (ctypes.c_int64 * 2)()
    par = (ctypes.c_int32 * 4)()
    assert L.moegq_moe_prefill_layout(4, 8, 2000, 2048, 512, 1, off, caps, par) == -6
    assert L.moegq_moe_prefill_layout(4, 8, 256, 2048, 512, 1, None, caps, par) == -1
    assert L.moegq_moe_prefill_layout(-1, 8, 256, 2048, 512, 1, off, caps, par) == -4
