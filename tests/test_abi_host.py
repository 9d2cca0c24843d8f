"""C-ABI host checks that need no GPU: the library loads, exports every entry
point declared in include/gdn.h, and rejects malformed arguments before any
HIP call (so these calls are safe without a device)."""
import ctypes
import os
import re

import pytest

from gated_deltanet_linear_rule_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def _lib():
    if not os.path.exists(B.lib_path()):
        pytest.fail("libgdn.so is not built (run python -m gated_deltanet_linear_rule_amd.build)")
    return B.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_header_declares_the_abi():
    assert _declared_functions() == ["gdn_abi_version", "gdn_decode_slots", "gdn_decode_step", "gdn_decode_tokens",
                                     "gdn_decode_tokens_raw", "gdn_last_error", "gdn_prefill", "gdn_prefill_affine",
                                     "gdn_prefill_affine_ws", "gdn_prefill_raw", "gdn_prefill_raw_ws",
                                     "gdn_prefill_snapshots", "gdn_prefill_snapshots_ws", "gdn_prefill_static",
                                     "gdn_prefill_workspace_size", "gdn_prefill_ws", "gdn_status_string"]


def test_library_exports_every_declared_symbol():
    L = _lib()
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_library_exports_only_the_abi():
    """No stray C symbols: the dynamic table holds the declared gdn_* functions."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", B.lib_path()], capture_output=True, text=True).stdout
    exported = sorted({ln.split()[-1] for ln in out.splitlines() if " T gdn_" in ln})
    assert exported == _declared_functions()


def test_abi_version_and_status_strings():
    assert B.gdn_abi_version() == 2
    seen = set()
    for st in range(5):
        s = B.status_string(st)
        assert s and s not in seen
        seen.add(s)
    assert B.status_string(99) == "unknown status"


def _shape(**kw):
    d = dict(num_seqs=1, num_tokens=64, num_qk_heads=2, num_v_heads=2, head_dim_k=64, head_dim_v=64,
             dtype=B.GDN_DTYPE_BF16)
    d.update(kw)
    return B.GdnShape(d["num_seqs"], d["num_tokens"], d["num_qk_heads"], d["num_v_heads"],
                      d["head_dim_k"], d["head_dim_v"], d["dtype"])


FAKE = 1 << 20   # non-NULL, 16-byte aligned host-side stand-in (never dereferenced)


def _prefill(shape, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, init=None, cu=None, out=FAKE, fin=None)
    p.update(ptrs)
    c = ctypes.c_void_p
    L = _lib()
    rc = L.gdn_prefill(ctypes.byref(shape) if shape is not None else None, c(p["q"]), c(p["k"]), c(p["v"]),
                       c(p["g"]), c(p["beta"]), c(p["init"]), c(p["cu"]), c(p["out"]), c(p["fin"]), None)
    return rc, L.gdn_last_error().decode()


def _decode(shape, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, state=FAKE, out=FAKE)
    p.update(ptrs)
    c = ctypes.c_void_p
    L = _lib()
    rc = L.gdn_decode_step(ctypes.byref(shape), c(p["q"]), c(p["k"]), c(p["v"]), c(p["g"]), c(p["beta"]),
                           c(p["state"]), c(p["out"]), None)
    return rc, L.gdn_last_error().decode()


@pytest.mark.parametrize("shape_kw,ptrs,status,msg", [
    (None, {}, B.GDN_ERROR_INVALID_VALUE, "shape is NULL"),
    (dict(num_seqs=-1), {}, B.GDN_ERROR_INVALID_VALUE, "negative"),
    (dict(num_tokens=-5), {}, B.GDN_ERROR_INVALID_VALUE, "negative"),
    (dict(num_qk_heads=0), {}, B.GDN_ERROR_INVALID_VALUE, "positive"),
    (dict(num_qk_heads=3, num_v_heads=4), {}, B.GDN_ERROR_INVALID_VALUE, "multiple"),
    (dict(dtype=7), {}, B.GDN_ERROR_INVALID_VALUE, "dtype"),
    (dict(head_dim_k=96), {}, B.GDN_ERROR_NOT_SUPPORTED, "head dims"),
    (dict(head_dim_v=256), {}, B.GDN_ERROR_NOT_SUPPORTED, "head dims"),
    (dict(num_seqs=0, num_tokens=3), {}, B.GDN_ERROR_INVALID_VALUE, "without sequences"),
    (dict(num_seqs=3, num_tokens=64), {}, B.GDN_ERROR_INVALID_VALUE, "multiple of num_seqs"),
    ({}, dict(q=None), B.GDN_ERROR_INVALID_VALUE, "q is NULL"),
    ({}, dict(out=None), B.GDN_ERROR_INVALID_VALUE, "out is NULL"),
    ({}, dict(beta=None), B.GDN_ERROR_INVALID_VALUE, "beta is NULL"),
    ({}, dict(k=FAKE + 2), B.GDN_ERROR_INVALID_VALUE, "aligned"),
    ({}, dict(g=FAKE + 2), B.GDN_ERROR_INVALID_VALUE, "aligned"),
    ({}, dict(init=FAKE + 8), B.GDN_ERROR_INVALID_VALUE, "aligned"),
    ({}, dict(cu=FAKE + 1), B.GDN_ERROR_INVALID_VALUE, "aligned"),
    ({}, dict(init=FAKE, fin=FAKE + 4096), B.GDN_ERROR_INVALID_VALUE, "overlap"),
])
def test_prefill_rejects_bad_arguments_before_any_hip_call(shape_kw, ptrs, status, msg):
    rc, err = _prefill(None if shape_kw is None else _shape(**shape_kw), **ptrs)
    assert rc == status and msg in err, (rc, err)


def test_prefill_with_nothing_to_do_succeeds_without_a_device():
    rc, err = _prefill(_shape(num_seqs=0, num_tokens=0), q=None, k=None, v=None, g=None, beta=None, out=None)
    assert rc == B.GDN_SUCCESS and err == ""


@pytest.mark.parametrize("shape_kw,ptrs,status,msg", [
    (dict(num_seqs=4, num_tokens=5), {}, B.GDN_ERROR_INVALID_VALUE, "num_tokens == num_seqs"),
    (dict(num_seqs=4, num_tokens=4), dict(state=None), B.GDN_ERROR_INVALID_VALUE, "state is NULL"),
    (dict(num_seqs=4, num_tokens=4), dict(state=FAKE + 4), B.GDN_ERROR_INVALID_VALUE, "aligned"),
    (dict(num_seqs=4, num_tokens=4, head_dim_k=32), {}, B.GDN_ERROR_NOT_SUPPORTED, "head dims"),
])
def test_decode_rejects_bad_arguments(shape_kw, ptrs, status, msg):
    rc, err = _decode(_shape(**shape_kw), **ptrs)
    assert rc == status and msg in err, (rc, err)


def _decode_tokens(shape, T, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, state=FAKE, out=FAKE, ts=None)
    p.update(ptrs)
    c = ctypes.c_void_p
    L = _lib()
    rc = L.gdn_decode_tokens(ctypes.byref(shape), T, c(p["q"]), c(p["k"]), c(p["v"]), c(p["g"]), c(p["beta"]),
                             c(p["state"]), c(p["out"]), c(p["ts"]), None)
    return rc, L.gdn_last_error().decode()


# state of 4 sequences x 2 heads x 64 x 64 fp32 = 128 KiB
@pytest.mark.parametrize("shape_kw,T,ptrs,status,msg", [
    (dict(num_seqs=4, num_tokens=12), 0, {}, B.GDN_ERROR_INVALID_VALUE, "tokens_per_seq must be positive"),
    (dict(num_seqs=4, num_tokens=12), -3, {}, B.GDN_ERROR_INVALID_VALUE, "tokens_per_seq must be positive"),
    (dict(num_seqs=4, num_tokens=13), 3, {}, B.GDN_ERROR_INVALID_VALUE, "num_seqs * tokens_per_seq"),
    (dict(num_seqs=4, num_tokens=12), 3, dict(state=None), B.GDN_ERROR_INVALID_VALUE, "state is NULL"),
    (dict(num_seqs=4, num_tokens=12), 3, dict(v=None), B.GDN_ERROR_INVALID_VALUE, "v is NULL"),
    (dict(num_seqs=4, num_tokens=12), 3, dict(ts=FAKE + 8), B.GDN_ERROR_INVALID_VALUE, "aligned"),
    (dict(num_seqs=4, num_tokens=12), 3, dict(ts=FAKE + 65536), B.GDN_ERROR_INVALID_VALUE, "overlaps"),
    (dict(num_seqs=4, num_tokens=12), 3, dict(ts=FAKE - 3 * 131072 + 16), B.GDN_ERROR_INVALID_VALUE, "overlaps"),
    (dict(num_seqs=4, num_tokens=12, head_dim_v=96), 3, {}, B.GDN_ERROR_NOT_SUPPORTED, "head dims"),
])
def test_decode_tokens_rejects_bad_arguments(shape_kw, T, ptrs, status, msg):
    rc, err = _decode_tokens(_shape(**shape_kw), T, **ptrs)
    assert rc == status and msg in err, (rc, err)


def test_decode_tokens_with_nothing_to_do_succeeds_without_a_device():
    rc, err = _decode_tokens(_shape(num_seqs=0, num_tokens=0), 4, q=None, k=None, v=None, g=None, beta=None,
                             state=None, out=None)
    assert rc == B.GDN_SUCCESS and err == ""


def _decode_slots(shape, T, pool_slots, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, pool=FAKE, idx=FAKE, out=FAKE, ts=None)
    p.update(ptrs)
    c = ctypes.c_void_p
    L = _lib()
    rc = L.gdn_decode_slots(ctypes.byref(shape), T, c(p["q"]), c(p["k"]), c(p["v"]), c(p["g"]), c(p["beta"]),
                            c(p["pool"]), pool_slots, c(p["idx"]), c(p["out"]), c(p["ts"]), None)
    return rc, L.gdn_last_error().decode()


@pytest.mark.parametrize("T,pool,ptrs,status,msg", [
    (1, 8, dict(idx=None), B.GDN_ERROR_INVALID_VALUE, "slot_idx is NULL"),
    (1, 8, dict(idx=FAKE + 2), B.GDN_ERROR_INVALID_VALUE, "aligned"),
    (1, -1, {}, B.GDN_ERROR_INVALID_VALUE, "negative pool_slots"),
    (1, 8, dict(pool=None), B.GDN_ERROR_INVALID_VALUE, "state is NULL"),
    (2, 8, {}, B.GDN_ERROR_INVALID_VALUE, "num_seqs * tokens_per_seq"),
    (1, 8, dict(ts=FAKE + 7 * 32768), B.GDN_ERROR_INVALID_VALUE, "overlaps"),
])
def test_decode_slots_rejects_bad_arguments(T, pool, ptrs, status, msg):
    rc, err = _decode_slots(_shape(num_seqs=4, num_tokens=4), T, pool, **ptrs)
    assert rc == status and msg in err, (rc, err)


def test_decode_slots_with_an_empty_pool_succeeds_without_a_device():
    rc, err = _decode_slots(_shape(num_seqs=4, num_tokens=4), 1, 0, pool=None)
    assert rc == B.GDN_SUCCESS and err == ""


def _prefill_snapshots(shape, chunks, snaps):
    c = ctypes.c_void_p
    L = _lib()
    rc = L.gdn_prefill_snapshots(ctypes.byref(shape), c(FAKE), c(FAKE), c(FAKE), c(FAKE), c(FAKE), None, None,
                                 c(FAKE), None, chunks, c(snaps) if snaps else None, None)
    return rc, L.gdn_last_error().decode()


@pytest.mark.parametrize("chunks,snaps,status,msg", [
    (2, None, B.GDN_ERROR_INVALID_VALUE, "snapshots is NULL"),
    (0, FAKE, B.GDN_ERROR_INVALID_VALUE, "snapshot_chunks must be positive"),
    (-4, FAKE, B.GDN_ERROR_INVALID_VALUE, "snapshot_chunks must be positive"),
    (2, FAKE + 4, B.GDN_ERROR_INVALID_VALUE, "aligned"),
])
def test_prefill_snapshots_rejects_bad_arguments(chunks, snaps, status, msg):
    rc, err = _prefill_snapshots(_shape(), chunks, snaps)
    assert rc == status and msg in err, (rc, err)


def test_raw_entry_points_apply_the_same_argument_checks():
    c = ctypes.c_void_p
    L = _lib()
    rc = L.gdn_prefill_raw(ctypes.byref(_shape(num_qk_heads=3, num_v_heads=4)), c(FAKE), c(FAKE), c(FAKE), c(FAKE),
                           c(FAKE), None, None, c(FAKE), None, None)
    assert rc == B.GDN_ERROR_INVALID_VALUE and "multiple" in L.gdn_last_error().decode()
    rc = L.gdn_decode_tokens_raw(ctypes.byref(_shape(num_seqs=4, num_tokens=12)), 3, c(FAKE), c(FAKE), c(FAKE),
                                 None, c(FAKE), c(FAKE), c(FAKE), None, None)
    assert rc == B.GDN_ERROR_INVALID_VALUE and "g is NULL" in L.gdn_last_error().decode()


def test_prefill_workspace_size_host_paths():
    L = _lib()
    n = ctypes.c_size_t(123)
    assert L.gdn_prefill_workspace_size(ctypes.byref(_shape()), 0, None) == B.GDN_ERROR_INVALID_VALUE
    assert L.gdn_prefill_workspace_size(None, 0, ctypes.byref(n)) == B.GDN_ERROR_INVALID_VALUE and n.value == 0
    rc = L.gdn_prefill_workspace_size(ctypes.byref(_shape(num_seqs=3, num_tokens=64)), 0, ctypes.byref(n))
    assert rc == B.GDN_ERROR_INVALID_VALUE and "not packed" in L.gdn_last_error().decode()
    n.value = 123
    rc = L.gdn_prefill_workspace_size(ctypes.byref(_shape(num_seqs=0, num_tokens=0)), B.GDN_WS_PACKED,
                                      ctypes.byref(n))
    assert rc == B.GDN_SUCCESS and n.value == 0


@pytest.mark.parametrize("flags,msg", [(8, "unknown workspace flags"), (1 << 31, "unknown workspace flags"),
                                       (B.GDN_WS_RAW | B.GDN_WS_AFFINE, "exclude each other")])
def test_prefill_workspace_size_rejects_bad_flags(flags, msg):
    L = _lib()
    n = ctypes.c_size_t(123)
    assert L.gdn_prefill_workspace_size(ctypes.byref(_shape()), flags, ctypes.byref(n)) == B.GDN_ERROR_INVALID_VALUE
    assert msg in L.gdn_last_error().decode() and n.value == 0


def _ws_call(name, shape, ws, nbytes, **kw):
    """One of the caller-workspace prefill forms with host-side stand-in pointers."""
    c = ctypes.c_void_p
    L = _lib()
    w = (c(ws) if ws else None, nbytes, None)
    if name == "gdn_prefill_affine_ws":
        rc = L.gdn_prefill_affine_ws(ctypes.byref(shape), c(FAKE), c(FAKE), c(FAKE), c(FAKE), None,
                                     c(kw.get("m", FAKE)), c(kw.get("b", FAKE + (1 << 22))), *w)
    elif name == "gdn_prefill_snapshots_ws":
        rc = L.gdn_prefill_snapshots_ws(ctypes.byref(shape), c(FAKE), c(FAKE), c(FAKE), c(FAKE), c(FAKE), None, None,
                                        c(FAKE), None, kw.get("chunks", 2), c(kw.get("snaps", FAKE)), *w)
    else:
        rc = getattr(L, name)(ctypes.byref(shape), c(FAKE), c(FAKE), c(FAKE), c(FAKE), c(FAKE), None, None, c(FAKE),
                              None, *w)
    return rc, L.gdn_last_error().decode()


WS_FORMS = ["gdn_prefill_ws", "gdn_prefill_raw_ws", "gdn_prefill_snapshots_ws", "gdn_prefill_affine_ws"]


@pytest.mark.parametrize("name", WS_FORMS)
@pytest.mark.parametrize("ws,status,msg", [
    (None, B.GDN_ERROR_INVALID_VALUE, "workspace is NULL"),
    (FAKE + 16, B.GDN_ERROR_INVALID_VALUE, "aligned"),
])
def test_prefill_ws_forms_reject_bad_workspace(name, ws, status, msg):
    rc, err = _ws_call(name, _shape(), ws, 1 << 20)
    assert rc == status and msg in err, (name, rc, err)


@pytest.mark.parametrize("name", WS_FORMS)
def test_prefill_ws_forms_apply_the_prefill_checks(name):
    rc, err = _ws_call(name, _shape(num_qk_heads=3, num_v_heads=4), FAKE, 1 << 20)
    assert rc == B.GDN_ERROR_INVALID_VALUE and "multiple" in err
    rc, err = _ws_call(name, _shape(num_seqs=0, num_tokens=0), FAKE, 0)
    assert rc == B.GDN_SUCCESS and err == ""


def test_prefill_ws_forms_check_their_own_arguments():
    rc, err = _ws_call("gdn_prefill_snapshots_ws", _shape(), FAKE, 1 << 20, snaps=0)
    assert rc == B.GDN_ERROR_INVALID_VALUE and "snapshots is NULL" in err
    rc, err = _ws_call("gdn_prefill_snapshots_ws", _shape(), FAKE, 1 << 20, chunks=0)
    assert rc == B.GDN_ERROR_INVALID_VALUE and "snapshot_chunks must be positive" in err
    rc, err = _ws_call("gdn_prefill_affine_ws", _shape(), FAKE, 1 << 20, b=FAKE + 1024)
    assert rc == B.GDN_ERROR_INVALID_VALUE and "overlap" in err
    rc, err = _ws_call("gdn_prefill_affine_ws", _shape(), FAKE, 1 << 20, m=0)
    assert rc == B.GDN_ERROR_INVALID_VALUE and "transition is NULL" in err


def test_prefill_static_applies_the_prefill_checks_before_any_hip_call():
    c = ctypes.c_void_p
    L = _lib()
    rc = L.gdn_prefill_static(ctypes.byref(_shape(num_qk_heads=3, num_v_heads=4)), c(FAKE), c(FAKE), c(FAKE),
                              c(FAKE), c(FAKE), None, None, c(FAKE), None, None)
    assert rc == B.GDN_ERROR_INVALID_VALUE and "multiple" in L.gdn_last_error().decode()
    rc = L.gdn_prefill_static(ctypes.byref(_shape()), c(FAKE), c(FAKE + 2), c(FAKE), c(FAKE), c(FAKE), None, None,
                              c(FAKE), None, None)
    assert rc == B.GDN_ERROR_INVALID_VALUE and "aligned" in L.gdn_last_error().decode()
    rc = L.gdn_prefill_static(ctypes.byref(_shape(num_seqs=0, num_tokens=0)), None, None, None, None, None, None,
                              None, None, None, None)
    assert rc == B.GDN_SUCCESS


def test_library_changes_no_pool_setting():
    """The library never sets an attribute of a memory pool (a process-wide setting)."""
    src = open(os.path.join(ROOT, "gated_deltanet_linear_rule_amd", "csrc", "gdn_api.cpp")).read()
    assert "hipMemPoolSetAttribute" not in src and "hipDeviceSetMemPool" not in src


def _affine(shape, m, b):
    c = ctypes.c_void_p
    L = _lib()
    rc = L.gdn_prefill_affine(ctypes.byref(shape), c(FAKE), c(FAKE), c(FAKE), c(FAKE), None,
                              c(m) if m else None, c(b) if b else None, None)
    return rc, L.gdn_last_error().decode()


@pytest.mark.parametrize("m,b,status,msg", [
    (None, FAKE, B.GDN_ERROR_INVALID_VALUE, "transition is NULL"),
    (FAKE, None, B.GDN_ERROR_INVALID_VALUE, "offset is NULL"),
    (FAKE, FAKE + 1024, B.GDN_ERROR_INVALID_VALUE, "overlap"),
    (FAKE + 8, FAKE + (1 << 22), B.GDN_ERROR_INVALID_VALUE, "aligned"),
])
def test_prefill_affine_rejects_bad_arguments(m, b, status, msg):
    rc, err = _affine(_shape(), m, b)
    assert rc == status and msg in err, (rc, err)


def test_prefill_affine_applies_the_shape_checks():
    rc, err = _affine(_shape(num_qk_heads=3, num_v_heads=4), FAKE, FAKE + (1 << 22))
    assert rc == B.GDN_ERROR_INVALID_VALUE and "multiple" in err


def test_binding_fails_loudly_without_the_library(monkeypatch):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "_LIB_PATH", "/nonexistent/libgdn.so")
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()


def test_product_path_does_not_touch_the_oracle():
    """No file of the library imports, links or loads the oracle."""
    pkg = os.path.join(ROOT, "gated_deltanet_linear_rule_amd")
    pat = re.compile(r"\b(from|import)\s+oracle\b|c_oracle|gdn_oracle|libgdn_oracle")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                assert not pat.search(open(os.path.join(dirpath, f)).read()), f
