"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/ssu.h declares, agrees with the header on struct layouts, and rejects
bad arguments on the host (every such path returns before any HIP call)."""
import ctypes
import os
import re
import subprocess

import pytest

from linear_rnn_recurrent_amd import ssu as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssu.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(S.LIB_PATH):
        from linear_rnn_recurrent_amd import build
        build.build()
    return S.load_library()


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^(?:ssu_status|const char \*|int32_t|int64_t)\s*(ssu_\w+)\s*\(", text,
                      re.M)


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert set(names) == set(S.EXPORTS), set(names) ^ set(S.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    nm = subprocess.run(["nm", "-D", "--defined-only", S.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r" T (ssu_\w+)$", nm, re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_library_links_hip_runtime_only():
    ldd = subprocess.run(["ldd", S.LIB_PATH], capture_output=True, text=True).stdout
    assert "amdhip64" in ldd
    assert "torch" not in ldd and "python" not in ldd


def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "sz.c"
    src.write_text('#include "ssu.h"\n#include <stdio.h>\n#include <stddef.h>\n'
                   'int main(void){printf("%zu %zu %zu %zu\\n", sizeof(ssu_dims),'
                   ' offsetof(ssu_dims, state_row_stride), sizeof(ssu_state_spec),'
                   ' offsetof(ssu_state_spec, shape));return 0;}\n')
    exe = tmp_path / "sz"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert got == [ctypes.sizeof(S.ssu_dims), S.ssu_dims.state_row_stride.offset,
                   ctypes.sizeof(S.ssu_state_spec), S.ssu_state_spec.shape.offset]


def test_version(lib):
    assert lib.ssu_version() == 10200


# ---------------------------------------------------------------------------
# Host-side validation (no GPU needed: nothing reaches the HIP runtime)
# ---------------------------------------------------------------------------
FAKE = 0x100000  # a 16-byte aligned non-null pointer value, never dereferenced


def dims(**kw):
    d = dict(batch=2, nheads=4, dim=16, dstate=16, ngroups=1, pool_rows=4, state_row_stride=0,
             state_dtype=0, io_dtype=0, bc_dtype=0, reserved=0)
    d.update(kw)
    return S.ssu_dims(**d)


def decode(lib, d, **ptrs):
    p = dict(x=FAKE, A=FAKE, B=FAKE, C=FAKE, dt=FAKE, dt_bias=None, D=None, z=None,
             state=FAKE, out=FAKE, idx=None)
    p.update(ptrs)
    return lib.ssu_decode(None if d is None else ctypes.byref(d), p["x"], p["A"], p["B"],
                          p["C"], p["dt"], p["dt_bias"], p["D"], p["z"], p["state"], p["out"],
                          1, p["idx"], None)


def err(lib):
    return lib.ssu_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(reserved=1), 1, "reserved"),
    (dict(batch=-1), 1, "batch"),
    (dict(nheads=0), 1, "> 0"),
    (dict(dim=0), 1, "> 0"),
    (dict(ngroups=3), 1, "multiple of ngroups"),
    (dict(pool_rows=0), 1, "pool_rows"),
    (dict(dstate=24), 2, "dstate"),
    (dict(dstate=512), 2, "dstate"),
    (dict(dim=5000), 2, "dim"),
    (dict(state_dtype=7), 2, "dtype"),
    (dict(io_dtype=3), 2, "dtype"),
    (dict(state_row_stride=100), 1, "state_row_stride"),
    (dict(state_row_stride=4 * 16 * 16 + 1), 1, "multiple of 16"),
    (dict(batch=5), 1, "pool_rows"),
])
def test_decode_rejects_bad_dims(lib, kw, status, needle):
    assert decode(lib, dims(**kw)) == status
    assert needle in err(lib)


def test_decode_null_dims_and_pointers(lib):
    assert decode(lib, None) == 1 and "dims is NULL" in err(lib)
    for name in ("x", "A", "B", "C", "dt", "state", "out"):
        assert decode(lib, dims(), **{name: None}) == 1
        assert f"'{name}'" in err(lib)
    assert decode(lib, dims(), x=FAKE + 2) == 1 and "4-byte aligned" in err(lib)
    assert decode(lib, dims(), z=FAKE + 2) == 1 and "aligned" in err(lib)
    assert decode(lib, dims(), B=FAKE + 4) == 1 and "16-byte aligned" in err(lib)
    assert decode(lib, dims(), state=FAKE + 8) == 1 and "16-byte aligned" in err(lib)
    assert decode(lib, dims(), idx=FAKE + 2) == 1 and "'state_indices'" in err(lib)
    assert decode(lib, dims(io_dtype=2), x=FAKE + 1) == 1 and "2-byte aligned" in err(lib)


def test_decode_empty_batch_is_a_noop(lib):
    assert decode(lib, dims(batch=0), x=None, state=None) == 0
    assert err(lib) == ""


def test_decode_indices_lift_the_pool_rows_bound(lib):
    # batch 5 > pool_rows 4 is fine with indices; it then fails on the next check (null x),
    # which proves the bound was not applied and no launch happened.
    assert decode(lib, dims(batch=5), idx=FAKE, x=None) == 1 and "'x'" in err(lib)


def prefill(lib, d, seq_len=8, stash=(None, None, None, None), **ptrs):
    p = dict(x=FAKE, A=FAKE, B=FAKE, C=FAKE, dt=FAKE, state=FAKE, out=FAKE)
    p.update(ptrs)
    return lib.ssu_prefill(ctypes.byref(d), seq_len, p["x"], p["A"], p["B"], p["C"], p["dt"],
                           None, None, None, p["state"], p["out"], 1, None, None, *stash, None)


def test_prefill_validation(lib):
    assert prefill(lib, dims(), seq_len=-1) == 1 and "seq_len" in err(lib)
    assert prefill(lib, dims(), stash=(FAKE, None, None, None)) == 1 and "all four" in err(lib)
    assert prefill(lib, dims(), stash=(FAKE, FAKE, FAKE, None)) == 1
    assert prefill(lib, dims(), seq_len=0, x=None) == 0
    assert prefill(lib, dims(), x=None) == 1 and "'x'" in err(lib)
    assert prefill(lib, dims(dstate=48)) == 2


def replay(lib, d, seq_len=4, active=2, ids=None, max_accept=0, **ptrs):
    p = dict(state=FAKE, dA=FAKE, u=FAKE, B=FAKE, dt=FAKE, acc=FAKE, idx=None)
    p.update(ptrs)
    return lib.ssu_replay(ctypes.byref(d), seq_len, p["state"], p["dA"], p["u"], p["B"],
                          p["dt"], p["acc"], p["idx"], active, ids, max_accept, None)


def test_replay_validation(lib):
    assert replay(lib, dims(), active=3) == 1 and "active_batch" in err(lib)
    assert replay(lib, dims(), active=-1) == 1
    assert replay(lib, dims(batch=8, pool_rows=4), active=6) == 1 and "pool_rows" in err(lib)
    assert replay(lib, dims(), seq_len=-2) == 1
    assert replay(lib, dims(), active=0, state=None) == 0
    for name in ("state", "dA", "u", "B", "dt", "acc"):
        assert replay(lib, dims(), **{name: None}) == 1, name


def test_replay_node_id_validation(lib):
    assert replay(lib, dims(), ids=FAKE, max_accept=0) == 1 and "max_accept_len" in err(lib)
    assert replay(lib, dims(), ids=FAKE, max_accept=-3) == 1 and "max_accept_len" in err(lib)
    # ignored without ids: fails later on the null state, not on max_accept_len
    assert replay(lib, dims(), max_accept=-3, state=None) == 1 and "'state'" in err(lib)
    assert replay(lib, dims(), ids=FAKE + 2, max_accept=4) == 1
    assert "'accepted_node_ids'" in err(lib) and "4-byte aligned" in err(lib)


def tree(lib, d, num_nodes=8, stash=(None, None, None, None), ws=FAKE, ws_bytes=1 << 30, **ptrs):
    p = dict(x=FAKE, A=FAKE, B=FAKE, C=FAKE, dt=FAKE, state=FAKE, out=FAKE, par=FAKE,
             dep=None, idx=None)
    p.update(ptrs)
    return lib.ssu_tree_verify(ctypes.byref(d), num_nodes, p["x"], p["A"], p["B"], p["C"],
                               p["dt"], None, None, None, p["state"], p["out"], 1, p["idx"],
                               p["par"], p["dep"], *stash, ws, ws_bytes, None)


def test_tree_verify_validation(lib):
    assert tree(lib, dims(), num_nodes=-1) == 1 and "num_nodes" in err(lib)
    assert tree(lib, dims(), num_nodes=129) == 1 and "num_nodes" in err(lib)
    assert tree(lib, dims(), stash=(FAKE, FAKE, None, FAKE)) == 1 and "all four" in err(lib)
    assert tree(lib, dims(), num_nodes=0, x=None) == 0 and err(lib) == ""
    assert tree(lib, dims(batch=0), x=None) == 0
    for name in ("x", "A", "B", "C", "dt", "state", "out", "par"):
        assert tree(lib, dims(), **{name: None}) == 1, name
    assert tree(lib, dims(), par=None) == 1 and "'parent_ids'" in err(lib)
    assert tree(lib, dims(), dep=FAKE + 1) == 1 and "'depths'" in err(lib)
    assert tree(lib, dims(), C=FAKE + 8) == 1 and "16-byte aligned" in err(lib)
    assert tree(lib, dims(), stash=(FAKE, FAKE, FAKE + 4, FAKE)) == 1 and "'replay_B'" in err(lib)
    assert tree(lib, dims(batch=5)) == 1 and "pool_rows" in err(lib)
    assert tree(lib, dims(dstate=48)) == 2
    assert tree(lib, dims(), ws=None) == 1 and "'workspace'" in err(lib)
    assert tree(lib, dims(), ws=FAKE + 4) == 1 and "'workspace'" in err(lib)
    d = dims()
    need = lib.ssu_tree_workspace_bytes(ctypes.byref(d), 8)
    assert need == 4 * d.batch * d.ngroups * 64 == S.tree_workspace_bytes(d.batch, d.ngroups, 8)
    assert tree(lib, d, ws_bytes=need - 4) == 1 and "workspace_bytes" in err(lib)
    assert lib.ssu_tree_workspace_bytes(ctypes.byref(d), 129) == -1
    assert lib.ssu_tree_workspace_bytes(None, 8) == -1


def test_tree_noalloc_refuses_beyond_its_scratch_on_the_host(lib):
    # B65 G1 M128 needs 4 * 65 * 128^2 bytes > SSU_TREE_SCRATCH_BYTES: refused
    # before any HIP call (fake pointers are never dereferenced)
    d = dims(batch=65, pool_rows=65, dim=64, dstate=64, nheads=2)
    p = [FAKE] * 8
    rc = lib.ssu_tree_verify_noalloc(ctypes.byref(d), 128, p[0], p[1], p[2], p[3], p[4], None,
                                     None, None, p[5], p[6], 1, None, p[7], None, None, None,
                                     None, None, None)
    assert rc == 1 and "scratch" in err(lib)
    assert S.TREE_SCRATCH_BYTES == 4 * 64 * 128 * 128


def spec_array(specs):
    arr = (S.ssu_state_spec * max(len(specs), 1))()
    for i, (kind, layer, shape, dt) in enumerate(specs):
        arr[i].kind, arr[i].layer, arr[i].rank, arr[i].dtype = kind, layer, len(shape), dt
        for k, s in enumerate(shape):
            arr[i].shape[k] = s
    return arr


def test_pool_bytes_per_slot(lib):
    specs = [(0, 0, (80, 64, 128), 0), (1, 0, (8192, 3), 2), (0, 1, (7,), 3)]
    out = ctypes.c_size_t()
    assert lib.ssu_pool_bytes_per_slot(spec_array(specs), 3, ctypes.byref(out)) == 0
    assert out.value == 80 * 64 * 128 * 4 + 8192 * 3 * 2 + 7
    assert lib.ssu_pool_bytes_per_slot(spec_array([]), 0, ctypes.byref(out)) == 0
    assert out.value == 0


@pytest.mark.parametrize("specs,needle", [
    ([(0, -1, (4,), 0)], "negative layer"),
    ([(0, 0, (4, 0), 0)], "non-positive"),
    ([(0, 0, (4,), 9)], "dtype"),
    ([(0, 0, (4,), 0), (1, 0, (4,), 0), (0, 0, (8,), 0)], "repeats"),
])
def test_pool_rejects_bad_specs(lib, specs, needle):
    out = ctypes.c_size_t()
    assert lib.ssu_pool_bytes_per_slot(spec_array(specs), len(specs), ctypes.byref(out)) == 1
    assert needle in err(lib)
    h = ctypes.c_void_p(123)
    assert lib.ssu_pool_alloc(spec_array(specs), len(specs), 4, None, None, 0, None,
                              ctypes.byref(h)) == 1
    assert h.value is None


def test_pool_rank_checks(lib):
    arr = spec_array([(0, 0, (4,), 0)])
    arr[0].rank = 5
    out = ctypes.c_size_t()
    assert lib.ssu_pool_bytes_per_slot(arr, 1, ctypes.byref(out)) == 1 and "rank" in err(lib)


def test_empty_pool_needs_no_device(lib):
    """slot_count == 0 allocates nothing, so the whole lifecycle runs on the host."""
    specs = [(0, 0, (80, 64, 128), 0), (1, 0, (128, 3), 2)]
    h = ctypes.c_void_p()
    assert lib.ssu_pool_alloc(spec_array(specs), 2, 0, b"rsm", None, 0, None, ctypes.byref(h)) == 0
    n, sc = ctypes.c_int32(), ctypes.c_int32()
    assert lib.ssu_pool_info(h, ctypes.byref(n), ctypes.byref(sc)) == 0
    assert (n.value, sc.value) == (2, 0)
    idx = ctypes.c_int32()
    assert lib.ssu_pool_find_state(h, 1, 0, ctypes.byref(idx)) == 0 and idx.value == 1
    assert lib.ssu_pool_find_state(h, 1, 5, ctypes.byref(idx)) == 0 and idx.value == -1
    b = ctypes.c_size_t()
    assert lib.ssu_pool_state_bytes_per_slot(h, 1, ctypes.byref(b)) == 0 and b.value == 768
    assert lib.ssu_pool_state_bytes_per_slot(h, 2, ctypes.byref(b)) == 1
    p = ctypes.c_void_p(1)
    assert lib.ssu_pool_state_ptr(h, 0, ctypes.byref(p)) == 0 and p.value is None
    assert lib.ssu_pool_clear_slot(h, -1, None) == 0          # nothing to clear
    assert lib.ssu_pool_clear_slot(h, 0, None) == 1 and "slot" in err(lib)
    assert lib.ssu_pool_clear_slot(h, -2, None) == 1
    ptrs = (ctypes.c_void_p * 2)(FAKE, FAKE)
    sizes = (ctypes.c_size_t * 2)(80 * 64 * 128 * 4, 768)
    assert lib.ssu_pool_capture(h, 0, ptrs, sizes, 2, None) == 1 and "slot" in err(lib)
    assert "pool 'rsm'" in err(lib)  # the pool's name prefixes its diagnostics
    assert lib.ssu_pool_restore(h, 0, ptrs, sizes, 2, None) == 1 and "slot" in err(lib)
    assert lib.ssu_pool_free(h) == 0
    assert lib.ssu_pool_free(None) == 0


def test_pool_slab_bytes_aligns_every_state(lib):
    # 1000 and 7 bytes per slot: 3 slots -> 3000 (3072 aligned) + 21 (256 aligned)
    specs = [(0, 0, (250,), 0), (1, 0, (7,), 3)]
    out = ctypes.c_size_t()
    assert lib.ssu_pool_slab_bytes(spec_array(specs), 2, 3, ctypes.byref(out)) == 0
    assert out.value == 3072 + 256
    assert lib.ssu_pool_slab_bytes(spec_array(specs), 2, 0, ctypes.byref(out)) == 0
    assert out.value == 0
    assert lib.ssu_pool_slab_bytes(spec_array(specs), 2, -1, ctypes.byref(out)) == 1
    assert lib.ssu_pool_slab_bytes(spec_array([(0, 0, (0,), 0)]), 1, 3, ctypes.byref(out)) == 1


def test_pool_caller_slab_checks_before_any_device_call(lib):
    specs = [(0, 0, (250,), 0), (1, 0, (7,), 3)]
    h = ctypes.c_void_p(123)
    # misaligned, then too small: rejected on the host, no pool returned
    assert lib.ssu_pool_alloc(spec_array(specs), 2, 3, b"p", FAKE + 16, 4096, None,
                              ctypes.byref(h)) == 1
    assert "aligned" in err(lib) and "pool 'p'" in err(lib) and h.value is None
    assert lib.ssu_pool_alloc(spec_array(specs), 2, 3, b"p", FAKE, 3327, None,
                              ctypes.byref(h)) == 1
    assert "3328" in err(lib) and h.value is None
    # zero slots in a caller slab: a valid pool that uses and owns no memory
    assert lib.ssu_pool_alloc(spec_array(specs), 2, 0, b"p", FAKE, 0, None, ctypes.byref(h)) == 0
    owns = ctypes.c_int32(7)
    assert lib.ssu_pool_owns_memory(h, ctypes.byref(owns)) == 0 and owns.value == 0
    assert lib.ssu_pool_free(h) == 0


def test_pool_spec_getters_and_name(lib):
    specs = [(0, 3, (80, 64, 128), 0), (1, 3, (128, 3), 2), (0, 4, (5,), 3)]
    h = ctypes.c_void_p()
    assert lib.ssu_pool_alloc(spec_array(specs), 3, 0, b"layers-3-4", None, 0, None,
                              ctypes.byref(h)) == 0
    name = ctypes.c_char_p()
    assert lib.ssu_pool_name(h, ctypes.byref(name)) == 0 and name.value == b"layers-3-4"
    owns = ctypes.c_int32()
    assert lib.ssu_pool_owns_memory(h, ctypes.byref(owns)) == 0 and owns.value == 1
    sp = S.ssu_state_spec()
    for i, (kind, layer, shape, dt) in enumerate(specs):
        assert lib.ssu_pool_spec(h, i, ctypes.byref(sp)) == 0
        assert (sp.kind, sp.layer, sp.rank, sp.dtype) == (kind, layer, len(shape), dt)
        assert tuple(sp.shape[:sp.rank]) == shape
    assert lib.ssu_pool_spec(h, 3, ctypes.byref(sp)) == 1 and "layers-3-4" in err(lib)
    assert lib.ssu_pool_spec(h, -1, ctypes.byref(sp)) == 1
    n = ctypes.c_int32()
    assert lib.ssu_pool_specs(h, None, 0, ctypes.byref(n)) == 0 and n.value == 3
    arr = (S.ssu_state_spec * 2)()
    assert lib.ssu_pool_specs(h, arr, 2, ctypes.byref(n)) == 0 and n.value == 3
    assert [(a.kind, a.layer) for a in arr] == [(0, 3), (1, 3)]
    assert lib.ssu_pool_specs(h, None, 2, ctypes.byref(n)) == 1
    assert lib.ssu_pool_free(h) == 0
    # unnamed pool: empty name, "pool" in diagnostics
    assert lib.ssu_pool_alloc(spec_array(specs), 3, 0, None, None, 0, None, ctypes.byref(h)) == 0
    assert lib.ssu_pool_name(h, ctypes.byref(name)) == 0 and name.value == b""
    assert lib.ssu_pool_free(h) == 0


def test_null_pool_arguments(lib):
    assert lib.ssu_pool_clear(None, None) == 1
    assert lib.ssu_pool_clear_slot(None, 0, None) == 1
    assert lib.ssu_pool_info(None, None, None) == 1
    assert lib.ssu_pool_alloc(spec_array([]), 0, 0, None, None, 0, None, None) == 1
    assert lib.ssu_pool_spec(None, 0, None) == 1
    assert lib.ssu_pool_specs(None, None, 0, None) == 1
    assert lib.ssu_pool_name(None, None) == 1
    assert lib.ssu_pool_owns_memory(None, None) == 1
    assert lib.ssu_pool_copy_slot_from(None, None, 0, 0, None) == 1


def test_python_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="not found"):
        S.load_library(str(tmp_path / "missing.so"))


def test_replay_layers_validation(lib):
    def call(d, num_layers=3, active=2, layers=FAKE, acc=FAKE, ids=None, max_accept=0, seq_len=4):
        return lib.ssu_replay_layers(ctypes.byref(d), seq_len, layers, num_layers, acc, None,
                                     active, ids, max_accept, None)
    assert call(dims(), num_layers=-1) == 1 and "num_layers" in err(lib)
    assert call(dims(), num_layers=70000) == 1 and "num_layers" in err(lib)
    assert call(dims(), active=3) == 1 and "active_batch" in err(lib)
    assert call(dims(), ids=FAKE, max_accept=0) == 1 and "max_accept_len" in err(lib)
    assert call(dims(), num_layers=0, layers=None) == 0 and err(lib) == ""
    assert call(dims(), seq_len=0, layers=None) == 0
    assert call(dims(), layers=None) == 1 and "'layers'" in err(lib)
    assert call(dims(), layers=FAKE + 4) == 1 and "aligned" in err(lib)
    assert call(dims(), acc=None) == 1 and "'accepted_lengths'" in err(lib)
    assert call(dims(dstate=48)) == 2


def test_state_clear_layers_validation(lib):
    def call(num_layers=2, rows=4, slot=1, rb=64, cb=10, layers=FAKE):
        return lib.ssu_state_clear_layers(layers, num_layers, rows, slot, rb, cb, None)
    assert call(num_layers=-1) == 1 and "num_layers" in err(lib)
    assert call(rows=-1) == 1 and "resident_rows" in err(lib)
    assert call(slot=4) == 1 and "slot" in err(lib)
    assert call(slot=-2) == 1 and "slot" in err(lib)
    assert call(rb=-1) == 1 and "row byte" in err(lib)
    assert call(layers=None) == 1 and "'layers'" in err(lib)
    assert call(num_layers=0, layers=None) == 0
    assert call(rows=0, slot=-1, layers=None) == 0


def test_row_movement_validation(lib):
    g = lambda rr=4, rs=0, as_=0, idx=FAKE, batch=2, rb=64, res=FAKE, act=FAKE: lib.ssu_state_gather(
        res, rr, rs, act, as_, idx, batch, rb, None)
    assert g(rr=-1) == 1 and "row count" in err(lib)
    assert g(batch=70000) == 1 and "batch" in err(lib)
    assert g(rb=-1) == 1 and "row_bytes" in err(lib)
    assert g(rs=32) == 1 and "stride" in err(lib)
    assert g(idx=None) == 1 and "'state_indices'" in err(lib)
    assert g(batch=0, res=None) == 0 and g(rb=0, res=None) == 0
    assert lib.ssu_state_scatter(FAKE, 0, FAKE, 4, 0, None, 2, 64, None) == 1
    p = lambda batch=3, rows=4, nby=0, by=None, ws=FAKE, homes=FAKE: lib.ssu_state_pack(
        FAKE, rows, 0, 64, homes, batch, by, nby, ws, None)
    assert p(batch=5) == 1 and "pool_rows" in err(lib)
    assert p(nby=4) == 1 and "n_bystanders" in err(lib)
    assert p(nby=1) == 1 and "'bystanders'" in err(lib)
    assert p(ws=None) == 1 and "'workspace'" in err(lib)
    assert p(homes=None) == 1 and "'homes'" in err(lib)
    assert p(batch=0, ws=None) == 0
    assert lib.ssu_state_unpack(FAKE, 4, 0, 64, FAKE, 3, None, 0, None, None) == 1


def test_gdn_decode_validation(lib):
    need = 4 * 2 * (2 * 2 * 128 + 4 * 128 + 2 * 4 * 1)  # hidden 64: one 256-row chunk

    def call(hq=2, hv=4, d=128, w=4, rs=0, w_ba=FAKE, hs=FAKE, batch=2, ws=FAKE, ws_bytes=need):
        dd = S.ssu_gdn_dims(batch, 64, hq, hv, d, w, 4, 1, rs, 3 * (2 * hq + hv) * d, 3, 1)
        return lib.ssu_gdn_decode(ctypes.byref(dd), hs, w_ba, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  ctypes.c_float(0.0), FAKE, FAKE, FAKE, ws, ws_bytes, None)
    assert call(hv=3) == 1 and "multiple" in err(lib)
    assert call(hq=1, hv=3) == 2 and "{1, 2, 4, 8}" in err(lib)
    assert call(hq=1, hv=16) == 2
    assert call(d=96) == 2 and "head_dim" in err(lib)
    assert call(w=9) == 2 and "conv_width" in err(lib)
    assert call(rs=4 * 128 * 128 - 4) == 1 and "ssm_row_stride" in err(lib)
    assert call(w_ba=FAKE + 2) == 1 and "'w_ba'" in err(lib)
    assert call(hq=128, hv=512) == 2 and "256" in err(lib)
    assert call(ws=None) == 1 and "'workspace'" in err(lib)
    assert call(ws=FAKE + 8) == 1 and "'workspace'" in err(lib)
    assert call(ws_bytes=need - 4) == 1 and "workspace_bytes" in err(lib)
    assert call(hs=None) == 1 and "'hidden_states'" in err(lib)
    assert call(batch=0, hs=None, w_ba=None, ws=None) == 0
    dd = S.ssu_gdn_dims(2, 64, 2, 4, 128, 4, 4, 1, 0, 0, 0, 0)
    assert lib.ssu_gdn_workspace_bytes(ctypes.byref(dd)) == need
    assert lib.ssu_gdn_workspace_bytes(None) == -1
