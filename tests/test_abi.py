"""The C ABI loads and rejects bad arguments on the host (CPU only, no launches).

Every case here returns from the library's argument checks before any HIP
call, so it runs without a GPU.
"""
import ctypes
import subprocess

import pytest

from head_latent_attention_laga_amd import _lib
from head_latent_attention_laga_amd.build import LIB

OK, INVALID, UNSUPPORTED, ALIGN, HIP, WORKSPACE = range(6)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def v3(**kw):
    d = dict(B=1, S=512, n_h=128, sp_size=8, sp_rank=0, d_kv=512, d_nope=128, d_rope=64, d_v=128,
             dtype=_lib.LAGA_BF16, precision=_lib.LAGA_OPERANDS_SPLIT)
    d.update(kw)
    return _lib.make_dims(**d)


def tiny(**kw):
    d = dict(B=1, S=256, n_h=2, sp_size=1, sp_rank=0, d_kv=64, d_nope=32, d_rope=16, d_v=32,
             dtype=_lib.LAGA_F32, precision=0)
    d.update(kw)
    return _lib.make_dims(**d)


FAKE = ctypes.c_void_p(1 << 20)     # 16-byte aligned, never dereferenced
MISALIGNED = ctypes.c_void_p((1 << 20) + 4)


def test_exports_every_header_function(lib):
    names = _lib.header_functions()
    assert set(names) >= {"laga_latent_norm", "laga_kv_up", "laga_attn_fwd", "laga_attn_bwd",
                          "laga_attn_bwd_workspace_bytes", "laga_status_string", "laga_kv_elem_bytes"}
    syms = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    for n in names:
        assert getattr(lib, n) is not None
        assert f" T {n}\n" in syms, n


def test_status_strings(lib):
    for s in range(6):
        assert lib.laga_status_string(s).decode().startswith(_lib.STATUS[s])


def test_kv_lo_shift_matches_header():
    import re
    text = open(_lib.HEADER).read()
    m = re.search(r"#define\s+LAGA_KV_LO_SHIFT\s+(\d+)", text)
    assert m and int(m.group(1)) == _lib.LAGA_KV_LO_SHIFT


def test_kv_elem_bytes():
    assert _lib.kv_elem_bytes(tiny()) == 4
    assert _lib.kv_elem_bytes(v3(precision=_lib.LAGA_OPERANDS_FP16)) == 2
    assert _lib.kv_elem_bytes(v3(precision=_lib.LAGA_OPERANDS_SPLIT)) == 3
    assert _lib.kv_elem_bytes(v3(d_kv=256)) == 0


@pytest.mark.parametrize("bad,code", [
    (dict(B=0), INVALID), (dict(S=0), INVALID), (dict(n_h=0), INVALID), (dict(sp_size=0), INVALID),
    (dict(n_h=12, sp_size=8), INVALID), (dict(sp_rank=8), INVALID), (dict(sp_rank=-1), INVALID),
    (dict(eps=0.0), INVALID), (dict(dtype=7), INVALID), (dict(precision=3), INVALID),
    (dict(d_kv=256), UNSUPPORTED), (dict(d_rope=32), UNSUPPORTED), (dict(d_v=64), UNSUPPORTED),
    (dict(dtype=_lib.LAGA_F32), UNSUPPORTED), (dict(S=1 << 23), UNSUPPORTED),
])
def test_dims_rejected_before_launch(lib, bad, code):
    d = v3(**bad)
    assert lib.laga_latent_norm(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None) == code
    assert lib.laga_kv_up(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None) == code
    assert lib.laga_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == code
    assert lib.laga_attn_bwd_workspace_bytes(ctypes.byref(d)) == 0
    args = [FAKE] * 17 + [ctypes.c_size_t(1 << 40), None]
    assert lib.laga_attn_bwd(ctypes.byref(d), *args) == code
    assert lib.laga_absorbed_fwd(ctypes.byref(d), *([FAKE] * 9), None) == code


def test_null_dims(lib):
    assert lib.laga_attn_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == INVALID
    assert lib.laga_attn_bwd_workspace_bytes(None) == 0


@pytest.mark.parametrize("slot", range(6))
def test_null_and_misaligned_pointers(lib, slot):
    d = v3()
    args = [FAKE] * 6
    args[slot] = None
    assert lib.laga_attn_fwd(ctypes.byref(d), *args, None) == INVALID
    args[slot] = MISALIGNED
    assert lib.laga_attn_fwd(ctypes.byref(d), *args, None) == ALIGN


@pytest.mark.parametrize("slot", range(9))
def test_absorbed_null_and_misaligned_pointers(lib, slot):
    d = v3()
    args = [FAKE] * 9
    args[slot] = None
    assert lib.laga_absorbed_fwd(ctypes.byref(d), *args, None) == INVALID
    args[slot] = MISALIGNED
    assert lib.laga_absorbed_fwd(ctypes.byref(d), *args, None) == ALIGN


def test_absorbed_form_needs_bf16_v3_dims(lib):
    assert lib.laga_absorbed_fwd(ctypes.byref(tiny()), *([FAKE] * 9), None) == UNSUPPORTED
    assert lib.laga_absorbed_fwd(None, *([FAKE] * 9), None) == INVALID


def test_backward_argument_checks(lib):
    d = v3()
    need = lib.laga_attn_bwd_workspace_bytes(ctypes.byref(d))
    assert need > 0
    args = [FAKE] * 17
    assert lib.laga_attn_bwd(ctypes.byref(d), *args, ctypes.c_size_t(need - 1), None) == WORKSPACE
    a2 = list(args)
    a2[16] = None  # workspace pointer
    assert lib.laga_attn_bwd(ctypes.byref(d), *a2, ctypes.c_size_t(need), None) == WORKSPACE
    a3 = list(args)
    a3[4] = None
    assert lib.laga_attn_bwd(ctypes.byref(d), *a3, ctypes.c_size_t(need), None) == INVALID
    a4 = list(args)
    a4[10] = MISALIGNED
    assert lib.laga_attn_bwd(ctypes.byref(d), *a4, ctypes.c_size_t(need), None) == ALIGN
    # the backward needs the fp32-class K/V of a split-operand forward
    d16 = v3(precision=_lib.LAGA_OPERANDS_FP16)
    assert lib.laga_attn_bwd(ctypes.byref(d16), *args, ctypes.c_size_t(1 << 40), None) == UNSUPPORTED


def test_fused_forward_checks_on_the_host(lib):
    """laga_attn_fwd_fused: fp16 operands at the bf16 V3 dims only, and every
    pointer, alignment and workspace check before any HIP call."""
    d = v3(precision=_lib.LAGA_OPERANDS_FP16)
    need = lib.laga_attn_fwd_fused_workspace_bytes(ctypes.byref(d))
    assert need > 0
    assert lib.laga_attn_fwd_fused_workspace_bytes(ctypes.byref(v3())) == 0          # split operands
    assert lib.laga_attn_fwd_fused_workspace_bytes(ctypes.byref(tiny())) == 0        # float32 dims
    assert lib.laga_attn_fwd_fused_workspace_bytes(ctypes.byref(v3(S=0))) == 0       # invalid dims
    args = [FAKE] * 7
    ok = (FAKE, ctypes.c_size_t(need), None)
    assert lib.laga_attn_fwd_fused(ctypes.byref(v3()), *args, *ok) == UNSUPPORTED
    assert lib.laga_attn_fwd_fused(ctypes.byref(tiny()), *args, *ok) == UNSUPPORTED
    assert lib.laga_attn_fwd_fused(None, *args, *ok) == INVALID
    for slot in range(7):
        a = list(args)
        a[slot] = None
        assert lib.laga_attn_fwd_fused(ctypes.byref(d), *a, *ok) == INVALID
        a[slot] = MISALIGNED
        assert lib.laga_attn_fwd_fused(ctypes.byref(d), *a, *ok) == ALIGN
    assert lib.laga_attn_fwd_fused(ctypes.byref(d), *args, FAKE, ctypes.c_size_t(need - 1), None) == WORKSPACE
    assert lib.laga_attn_fwd_fused(ctypes.byref(d), *args, None, ctypes.c_size_t(need), None) == WORKSPACE
    assert lib.laga_attn_fwd_fused(ctypes.byref(d), *args, MISALIGNED, ctypes.c_size_t(need), None) == ALIGN


def test_fused_workspace_is_linear_in_the_sequence_beyond_split_tiles(lib):
    def ws(S, **kw):
        return lib.laga_attn_fwd_fused_workspace_bytes(ctypes.byref(v3(S=S, precision=_lib.LAGA_OPERANDS_FP16, **kw)))
    a, b, c = ws(8192), ws(12288), ws(16384)
    assert b - a == c - b > 0
    assert c < 200e6
    # S=4096: half of its 16 query tiles run as two tasks each; their partials
    # (2 x 256 rows x 132 floats per tile and head) come on top of the linear part.
    assert ws(4096) - (a - (b - a)) == 8 * 16 * 2 * 256 * 132 * 4


def test_absorbed_backward_checks_on_the_host(lib):
    d = v3()
    need = lib.laga_absorbed_bwd_workspace_bytes(ctypes.byref(d))
    assert need > 0
    assert lib.laga_absorbed_bwd_workspace_bytes(ctypes.byref(tiny())) == 0
    args = [FAKE] * 12
    ok = (FAKE, ctypes.c_size_t(need), None)
    assert lib.laga_absorbed_bwd(ctypes.byref(tiny()), *args, *ok) == UNSUPPORTED
    assert lib.laga_absorbed_bwd(None, *args, *ok) == INVALID
    for slot in (0, 3, 6, 11):
        a = list(args)
        a[slot] = None
        assert lib.laga_absorbed_bwd(ctypes.byref(d), *a, *ok) == INVALID
        a[slot] = MISALIGNED
        assert lib.laga_absorbed_bwd(ctypes.byref(d), *a, *ok) == ALIGN
    # Smaller workspaces run with smaller chunks, down to 32-token chunks.
    least = lib.laga_absorbed_bwd_min_workspace_bytes(ctypes.byref(d))
    assert 0 < least < need
    assert lib.laga_absorbed_bwd_min_workspace_bytes(ctypes.byref(tiny())) == 0
    assert lib.laga_absorbed_bwd(ctypes.byref(d), *args, FAKE, ctypes.c_size_t(least - 1), None) == WORKSPACE
    assert lib.laga_absorbed_bwd(ctypes.byref(d), *args, None, ctypes.c_size_t(need), None) == WORKSPACE


def test_absorbed_backward_workspace_sizes():
    """Default and minimum workspaces: at S=16384, 16 heads the default holds 1 GiB
    of chunk buffers beside the per-row planes; the minimum (32-token chunks) is
    linear in S."""
    def sizes(S):
        d = _lib.make_dims(1, S, 128, 8, 0, 512, 128, 64, 128, _lib.LAGA_BF16, 0)
        return _lib.absorbed_bwd_workspace_bytes(d), _lib.absorbed_bwd_min_workspace_bytes(d)
    full, least = sizes(16384)
    assert 3.3e9 < full < 3.8e9
    assert full - least > 0.9e9
    m1, m2, m3 = (sizes(S)[1] for S in (4096, 8192, 12288))
    assert abs((m3 - m2) - (m2 - m1)) < 1e6


def test_noalloc_scratch_size_matches_header():
    import re
    text = open(_lib.HEADER).read()
    m = re.search(r"#define\s+LAGA_NOALLOC_SCRATCH_BYTES\s+\(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.LAGA_NOALLOC_SCRATCH_BYTES


def test_noalloc_backward_checks_on_the_host(lib):
    """The allocation-free backward rejects, before any HIP call, problems whose
    workspace exceeds its static scratch and every argument laga_attn_bwd rejects."""
    cap = _lib.LAGA_NOALLOC_SCRATCH_BYTES
    args = [FAKE] * 16
    fits = v3(S=4096, n_h=128, sp_size=8)
    big = v3(S=8192, n_h=128, sp_size=8)
    assert lib.laga_attn_bwd_workspace_bytes(ctypes.byref(fits)) <= cap
    assert lib.laga_attn_bwd_workspace_bytes(ctypes.byref(big)) > cap
    assert lib.laga_attn_bwd_noalloc(ctypes.byref(big), *args, None) == WORKSPACE
    assert lib.laga_attn_bwd_noalloc(ctypes.byref(v3(S=1024, n_h=128, sp_size=1)), *args, None) == WORKSPACE
    a3 = list(args)
    a3[4] = None
    assert lib.laga_attn_bwd_noalloc(ctypes.byref(fits), *a3, None) == INVALID
    a4 = list(args)
    a4[10] = MISALIGNED
    assert lib.laga_attn_bwd_noalloc(ctypes.byref(fits), *a4, None) == ALIGN
    assert lib.laga_attn_bwd_noalloc(ctypes.byref(v3(precision=_lib.LAGA_OPERANDS_FP16)), *args, None) == UNSUPPORTED
    assert lib.laga_attn_bwd_noalloc(ctypes.byref(v3(S=0)), *args, None) == INVALID
    assert lib.laga_attn_bwd_noalloc(None, *args, None) == INVALID


def test_workspace_grows_with_sequence(lib):
    a = lib.laga_attn_bwd_workspace_bytes(ctypes.byref(v3(S=1024)))
    b = lib.laga_attn_bwd_workspace_bytes(ctypes.byref(v3(S=2048)))
    assert b > a > 0
    assert lib.laga_attn_bwd_workspace_bytes(ctypes.byref(tiny())) > 0


def test_workspace_is_linear_in_the_sequence(lib):
    # No S x S quantity is stored: the workspace is an affine function of the
    # token count (a per-token part plus the fixed dW_kv_b partial sums), far
    # below the fp16 score matrix of a single head once S is large.
    def ws(S, B=1, **kw):
        return lib.laga_attn_bwd_workspace_bytes(ctypes.byref(v3(S=S, B=B, **kw)))
    a, b, c = ws(8192), ws(16384), ws(32768)
    per_token = (c - b) / 16384
    assert abs((b - a) / 8192 - per_token) <= 1e-3 * per_token
    assert ws(131072) < 6 * 2**30                       # 4.9 GiB at S = 128K (16 local heads)
    assert ws(131072) < 131072 * 131072 * 2 / 4         # a quarter of one head's fp16 score matrix
    assert ws(16384) < 0.7 * 2**30
    assert ws(4096, B=4) == ws(16384) or abs(ws(4096, B=4) - ws(16384)) < 2**20  # only the token count matters
    t = tiny(S=300)
    assert lib.laga_attn_bwd_workspace_bytes(ctypes.byref(t)) > 0
