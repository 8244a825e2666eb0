"""CPU checks of the C ABI: the library loads, exports every function the header
declares, and rejects bad arguments on the host before touching a device."""
import ctypes
import subprocess

import pytest


@pytest.fixture(scope="module")
def jb():
    from gated_delta_rule_jetblock_amd import jetblock
    return jetblock


def test_exports_every_declared_function(jb):
    names = jb.declared_functions()
    assert {"jb_prefill", "jb_decode_step", "jb_prefill_workspace_size", "jb_decode_workspace_size",
            "jb_gen_taps", "jb_gen_conv", "jb_prologue", "jb_decode_update", "jb_project",
            "jb_project_workspace_size", "jb_prefill_from_x", "jb_prefill_from_x_workspace_size"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", jb.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        getattr(jb.library(), n)  # resolvable through ctypes


def test_version_and_status_strings(jb):
    assert jb.version() >= 10000
    lib = jb.library()
    assert lib.jb_status_string(0) == b"JB_OK"
    assert lib.jb_status_string(3) == b"JB_ERR_WORKSPACE"
    assert lib.jb_status_string(99) == b"JB_ERR_UNKNOWN"


def _ws(jb, shape):
    n = ctypes.c_size_t(0)
    st = jb.library().jb_prefill_workspace_size(ctypes.byref(shape), ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("field,value,status", [
    ("dk", 48, 2), ("dv", 96, 2), ("gen_hidden", 16, 2), ("taps", 3, 2), ("chunk", 32, 2),
    ("d_model", 100, 2), ("H", 0, 2), ("H", 33, 2), ("B", 0, 1), ("B", 65536, 2), ("T", -1, 1), ("io_dtype", 7, 1),
    ("flags", 1, 1),
])
def test_shape_validation(jb, field, value, status):
    s = jb.make_shape(1, 100, 2, 32, 64, 128)
    setattr(s, field, value)
    st, _ = _ws(jb, s)
    assert st == status, (field, st, jb.last_error())
    assert field in jb.last_error() or "flags" in jb.last_error()


def test_workspace_sizes(jb):
    st, n1 = _ws(jb, jb.make_shape(1, 65536, 12, 96, 256, 1536))
    assert st == 0 and n1 >= 65536 * 12 * 16
    st, n2 = _ws(jb, jb.make_shape(1, 65536, 12, 96, 256, 1536, flags=jb.flag_segment(1024)))
    assert st == 0 and n2 == ((65536 * 12 * 16 + 255) // 256) * 256  # one segment: taps only
    n = ctypes.c_size_t(0)
    assert jb.library().jb_decode_workspace_size(ctypes.byref(jb.make_shape(256, 1, 12, 96, 256, 1536)),
                                                 ctypes.byref(n)) == 0
    assert n.value == 0  # the fused decode step keeps its intermediates on chip
    assert jb.library().jb_decode_workspace_size(ctypes.byref(jb.make_shape(4, 2, 12, 96, 256, 1536)),
                                                 ctypes.byref(n)) == 1


def test_prefill_rejects_before_launch(jb):
    """Null, misaligned and undersized arguments come back as status codes; none of these
    calls reaches the HIP runtime (this machine may have no GPU)."""
    lib = jb.library()
    s = jb.make_shape(1, 64, 2, 32, 64, 128)
    P = ctypes.c_void_p
    fake = P(0x10000)  # never dereferenced: validation fails first
    args = [fake] * 15
    # x = NULL
    a = list(args); a[0] = None
    assert lib.jb_prefill(ctypes.byref(s), *a, fake, 1 << 30, None) == 1
    assert "x is NULL" in jb.last_error()
    # misaligned q
    a = list(args); a[1] = P(0x10004)
    assert lib.jb_prefill(ctypes.byref(s), *a, fake, 1 << 30, None) == 1
    assert "q is not 16-byte aligned" in jb.last_error()
    # alpha only needs 4-byte alignment: a 4-aligned alpha passes that check and the
    # call then fails on the workspace size
    a = list(args); a[4] = P(0x10004)
    assert lib.jb_prefill(ctypes.byref(s), *a, fake, 0, None) == 3
    # workspace too small
    assert lib.jb_prefill(ctypes.byref(s), *args, fake, 16, None) == 3
    assert "workspace" in jb.last_error()
    # all-fp32 mode at a shape whose tiles do not fit in LDS
    s32 = jb.make_shape(1, 64, 2, 96, 256, 128, io_dtype=jb.JB_F32)
    assert lib.jb_prefill(ctypes.byref(s32), *args, fake, 1 << 30, None) == 2


def test_decode_rejects_before_launch(jb):
    lib = jb.library()
    s = jb.make_shape(8, 1, 2, 32, 64, 128)
    fake = ctypes.c_void_p(0x10000)
    args = [fake] * 15
    a = list(args); a[0] = None  # S_in
    assert lib.jb_decode_step(ctypes.byref(s), *a, fake, 1 << 20, None) == 1
    assert "S_in is NULL" in jb.last_error()
    a = list(args); a[8] = ctypes.c_void_p(0x10002)  # alpha_t only 2-byte aligned
    assert lib.jb_decode_step(ctypes.byref(s), *a, None, 0, None) == 1
    a = list(args); a[4] = ctypes.c_void_p(0x10008)  # x_t not 16-byte aligned
    assert lib.jb_decode_step(ctypes.byref(s), *a, None, 0, None) == 1
    s.T = 2
    assert lib.jb_decode_step(ctypes.byref(s), *args, fake, 1 << 20, None) == 1
    s.T = 1
    s.dk = 80
    assert lib.jb_decode_step(ctypes.byref(s), *args, fake, 1 << 20, None) == 2


def test_binding_refuses_host_tensors(jb):
    import torch
    x = torch.zeros(1, 4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        jb.gen_taps(x, torch.zeros(32, 128, dtype=torch.bfloat16), torch.zeros(8, 32, dtype=torch.bfloat16), H=2)


def test_projection_entries_reject_before_launch(jb):
    lib = jb.library()
    n = ctypes.c_size_t(0)
    s = jb.make_shape(1, 64, 2, 32, 64, 128)
    n.value = 1
    assert lib.jb_project_workspace_size(ctypes.byref(s), ctypes.byref(n)) == 0 and n.value == 0  # none needed
    assert lib.jb_prefill_from_x_workspace_size(ctypes.byref(s), ctypes.byref(n)) == 0
    # q, k, v (bf16) and the two gates (fp32) of the 64 tokens, plus the prefill's taps
    assert n.value >= 64 * 2 * (2 * 32 + 64) * 2 + 2 * 64 * 2 * 4 + 64 * 2 * 4 * 4
    s32 = jb.make_shape(1, 64, 2, 32, 64, 128, io_dtype=jb.JB_F32)
    assert lib.jb_project_workspace_size(ctypes.byref(s32), ctypes.byref(n)) == 2  # bf16 inputs only
    fake = ctypes.c_void_p(0x10000)
    args = [fake] * 18
    a = list(args); a[0] = None  # x
    assert lib.jb_project(ctypes.byref(s), *a, fake, 1 << 30, None) == 1
    assert "x is NULL" in jb.last_error()
    a = list(args); a[2] = ctypes.c_void_p(0x10008)  # Wk misaligned
    assert lib.jb_project(ctypes.byref(s), *a, fake, 1 << 30, None) == 1
    pargs = [fake] * 17
    assert lib.jb_prefill_from_x(ctypes.byref(s), *pargs, fake, 16, None) == 3
    assert lib.jb_prefill_from_x(ctypes.byref(s32), *pargs, fake, 1 << 30, None) == 2


def test_static_entries_reject_before_launch(jb):
    """jb_prefill_static / jb_decode_step_static: unsupported shapes, mixed caches, bad
    pointers and small workspaces come back as status codes before any launch."""
    lib = jb.library()
    n = ctypes.c_size_t(0)
    s = jb.make_shape(1, 64, 2, 32, 64, 128)
    assert lib.jb_prefill_static_workspace_size(ctypes.byref(s), ctypes.byref(n)) == 0
    assert n.value == 0  # one segment: no workspace
    sseg = jb.make_shape(1, 4096, 2, 32, 64, 128, flags=jb.flag_segment(8))
    assert lib.jb_prefill_static_workspace_size(ctypes.byref(sseg), ctypes.byref(n)) == 0
    assert n.value >= 8 * 2 * (2 * 32 * 64 + 32 * 32) * 4  # Mstart, Dsum, Phi of 8 segments
    s_bad = jb.make_shape(1, 64, 2, 32, 128, 128)  # (32, 128) is not built for the static block
    assert lib.jb_prefill_static_workspace_size(ctypes.byref(s_bad), ctypes.byref(n)) == 2
    s32 = jb.make_shape(1, 64, 2, 32, 64, 128, io_dtype=jb.JB_F32)
    assert lib.jb_prefill_static_workspace_size(ctypes.byref(s32), ctypes.byref(n)) == 2
    fake = ctypes.c_void_p(0x10000)
    args = [fake] * 17
    a = list(args); a[0] = None  # q
    assert lib.jb_prefill_static(ctypes.byref(s), *a, None, 0, None) == 1
    assert "q is NULL" in jb.last_error()
    a = list(args); a[5] = ctypes.c_void_p(0x10004)  # wq misaligned
    assert lib.jb_prefill_static(ctypes.byref(s), *a, None, 0, None) == 1
    a = list(args); a[10] = None  # cache_k_in NULL but the other two set
    assert lib.jb_prefill_static(ctypes.byref(s), *a, None, 0, None) == 1
    assert "all set or all NULL" in jb.last_error()
    assert lib.jb_prefill_static(ctypes.byref(sseg), *args, fake, 16, None) == 3
    d = jb.make_shape(8, 1, 2, 32, 64, 128)
    dargs = [fake] * 17
    a = list(dargs); a[4] = None  # cache_v_in
    assert lib.jb_decode_step_static(ctypes.byref(d), *a, None) == 1
    assert "cache_v_in is NULL" in jb.last_error()
    a = list(dargs); a[14] = None  # wk
    assert lib.jb_decode_step_static(ctypes.byref(d), *a, None) == 1
    d.T = 3
    assert lib.jb_decode_step_static(ctypes.byref(d), *dargs, None) == 1


def test_varlen_entries_reject_before_launch(jb):
    lib = jb.library()
    n = ctypes.c_size_t(0)
    s = jb.make_shape(4, 1000, 2, 32, 64, 128)   # 4 sequences, the longest 1000 tokens
    assert lib.jb_prefill_varlen_workspace_size(ctypes.byref(s), 2500, ctypes.byref(n)) == 0
    assert n.value >= 2500 * 2 * 16              # the taps of the packed rows
    assert lib.jb_prefill_varlen_workspace_size(ctypes.byref(s), 4001, ctypes.byref(n)) == 1  # > B * T
    assert "total_tokens" in jb.last_error()
    assert lib.jb_prefill_varlen_workspace_size(ctypes.byref(s), -1, ctypes.byref(n)) == 1
    fake = ctypes.c_void_p(0x10000)
    args = [fake] * 16
    a = list(args); a[0] = None  # cu_seqlens
    assert lib.jb_prefill_varlen(ctypes.byref(s), 2500, *a, fake, 1 << 30, None) == 1
    assert "cu_seqlens is NULL" in jb.last_error()
    a = list(args); a[0] = ctypes.c_void_p(0x10002)  # cu_seqlens not 4-byte aligned
    assert lib.jb_prefill_varlen(ctypes.byref(s), 2500, *a, fake, 1 << 30, None) == 1
    a = list(args); a[2] = None  # q
    assert lib.jb_prefill_varlen(ctypes.byref(s), 2500, *a, fake, 1 << 30, None) == 1
    assert lib.jb_prefill_varlen(ctypes.byref(s), 2500, *args, fake, 16, None) == 3  # workspace too small


def test_backward_entries_reject_before_launch(jb):
    lib = jb.library()
    n = ctypes.c_size_t(0)
    s = jb.make_shape(2, 200, 2, 32, 64, 128)
    assert lib.jb_backward_workspace_size(ctypes.byref(s), ctypes.byref(n)) == 0 and n.value > 2 * 200 * 2 * 64 * 8
    s_bad = jb.make_shape(2, 200, 2, 32, 128, 128)   # (32, 128) not built for the backward pass
    assert lib.jb_backward_workspace_size(ctypes.byref(s_bad), ctypes.byref(n)) == 2
    s32 = jb.make_shape(2, 200, 2, 32, 64, 128, io_dtype=jb.JB_F32)
    assert lib.jb_backward_workspace_size(ctypes.byref(s32), ctypes.byref(n)) == 2
    sflag = jb.make_shape(2, 200, 2, 32, 64, 128, flags=jb.flag_segment(2))
    assert lib.jb_backward_workspace_size(ctypes.byref(sflag), ctypes.byref(n)) == 1
    fake = ctypes.c_void_p(0x10000)
    args = [fake] * 27
    a = list(args); a[12] = None  # dout
    assert lib.jb_backward(ctypes.byref(s), *a, fake, 1 << 34, None) == 1
    assert "dout is NULL" in jb.last_error()
    a = list(args); a[25] = None  # dS0
    assert lib.jb_backward(ctypes.byref(s), *a, fake, 1 << 34, None) == 1
    assert lib.jb_backward(ctypes.byref(s), *args, fake, 16, None) == 3   # workspace too small
