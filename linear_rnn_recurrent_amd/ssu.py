"""Python binding of libssu (ctypes). Argument marshalling only.

Each function takes torch tensors that live on the GPU, checks that their
shapes agree (the C library cannot see shapes), and calls the C entry point of
the same name on torch's current stream. All computation happens in the HIP
kernels of libssu.so; there is no fallback. If the library has not been built
the first call raises RuntimeError (build it with
`python -m linear_rnn_recurrent_amd.build`).
"""
import ctypes
import os
from typing import Optional, Sequence

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libssu.so")

SSU_OK, SSU_EINVAL, SSU_ENOTSUP, SSU_EHIP, SSU_ENOMEM = 0, 1, 2, 3, 4
SSU_F32, SSU_F16, SSU_BF16, SSU_U8 = 0, 1, 2, 3
_DT = {torch.float32: SSU_F32, torch.float16: SSU_F16, torch.bfloat16: SSU_BF16,
       torch.uint8: SSU_U8}

EXPORTS = ("ssu_decode", "ssu_prefill", "ssu_replay", "ssu_tree_verify",
           "ssu_tree_verify_noalloc", "ssu_replay_layers",
           "ssu_state_clear_layers", "ssu_state_gather", "ssu_state_scatter", "ssu_state_pack",
           "ssu_state_unpack", "ssu_gdn_decode", "ssu_gdn_workspace_bytes", "ssu_tree_workspace_bytes",
           "ssu_pool_bytes_per_slot", "ssu_pool_slab_bytes", "ssu_pool_spec", "ssu_pool_specs",
           "ssu_pool_name", "ssu_pool_owns_memory",
           "ssu_pool_alloc", "ssu_pool_free", "ssu_pool_info", "ssu_pool_state_ptr",
           "ssu_pool_state_bytes_per_slot", "ssu_pool_find_state", "ssu_pool_clear",
           "ssu_pool_clear_slot", "ssu_pool_capture", "ssu_pool_restore",
           "ssu_pool_copy_slot_from", "ssu_last_error", "ssu_version")


class SsuError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"[ssu status {status}] {msg}")
        self.status = status


class ssu_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("nheads", ctypes.c_int32), ("dim", ctypes.c_int32),
                ("dstate", ctypes.c_int32), ("ngroups", ctypes.c_int32),
                ("pool_rows", ctypes.c_int32), ("state_row_stride", ctypes.c_int64),
                ("state_dtype", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("bc_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class ssu_replay_layer(ctypes.Structure):
    _fields_ = [("state", ctypes.c_void_p), ("replay_dA", ctypes.c_void_p),
                ("replay_u", ctypes.c_void_p), ("replay_B", ctypes.c_void_p),
                ("replay_dt", ctypes.c_void_p)]


class ssu_state_layer(ctypes.Structure):
    _fields_ = [("recurrent_state", ctypes.c_void_p), ("conv_state", ctypes.c_void_p)]


class ssu_gdn_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("conv_width", ctypes.c_int32),
                ("pool_rows", ctypes.c_int32), ("use_qk_l2norm", ctypes.c_int32),
                ("ssm_row_stride", ctypes.c_int64), ("conv_slot_stride", ctypes.c_int64),
                ("conv_chan_stride", ctypes.c_int64), ("conv_tap_stride", ctypes.c_int64)]


class ssu_state_spec(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("layer", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("shape", ctypes.c_int64 * 4)]


_LIB = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32


def load_library(path: Optional[str] = None):
    """Load libssu.so (once) and declare the C signatures."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libssu.so not found at {p}: build it with "
                           "`python -m linear_rnn_recurrent_amd.build`")
    lib = ctypes.CDLL(p)
    D = ctypes.POINTER(ssu_dims)
    S = ctypes.POINTER(ssu_state_spec)
    sig = {
        "ssu_decode": [D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _P],
        "ssu_prefill": [D, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _P,
                        _P, _P, _P, _P, _P],
        "ssu_replay": [D, _I32, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _I32, _P],
        "ssu_tree_verify": [D, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P,
                            _P, _P, _P, _P, _P, ctypes.c_int64, _P],
        "ssu_tree_verify_noalloc": [D, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P,
                                    _P, _P, _P, _P, _P, _P, _P],
        "ssu_replay_layers": [D, _I32, _P, _I32, _P, _P, _I32, _P, _I32, _P],
        "ssu_state_clear_layers": [_P, _I32, _I32, _I32, ctypes.c_int64, ctypes.c_int64, _P],
        "ssu_state_gather": [_P, _I32, ctypes.c_int64, _P, ctypes.c_int64, _P, _I32,
                             ctypes.c_int64, _P],
        "ssu_state_scatter": [_P, ctypes.c_int64, _P, _I32, ctypes.c_int64, _P, _I32,
                              ctypes.c_int64, _P],
        "ssu_state_pack": [_P, _I32, ctypes.c_int64, ctypes.c_int64, _P, _I32, _P, _I32, _P, _P],
        "ssu_gdn_decode": [ctypes.POINTER(ssu_gdn_dims), _P, _P, _P, _P, _P, _P, _P, _P,
                           ctypes.c_float, _P, _P, _P, _P, ctypes.c_int64, _P],
        "ssu_state_unpack": [_P, _I32, ctypes.c_int64, ctypes.c_int64, _P, _I32, _P, _I32, _P, _P],
        "ssu_pool_bytes_per_slot": [S, _I32, ctypes.POINTER(ctypes.c_size_t)],
        "ssu_pool_slab_bytes": [S, _I32, _I32, ctypes.POINTER(ctypes.c_size_t)],
        "ssu_pool_alloc": [S, _I32, _I32, ctypes.c_char_p, _P, ctypes.c_size_t, _P,
                           ctypes.POINTER(_P)],
        "ssu_pool_spec": [_P, _I32, S],
        "ssu_pool_specs": [_P, S, _I32, ctypes.POINTER(_I32)],
        "ssu_pool_name": [_P, ctypes.POINTER(ctypes.c_char_p)],
        "ssu_pool_owns_memory": [_P, ctypes.POINTER(_I32)],
        "ssu_pool_free": [_P],
        "ssu_pool_info": [_P, ctypes.POINTER(_I32), ctypes.POINTER(_I32)],
        "ssu_pool_state_ptr": [_P, _I32, ctypes.POINTER(_P)],
        "ssu_pool_state_bytes_per_slot": [_P, _I32, ctypes.POINTER(ctypes.c_size_t)],
        "ssu_pool_find_state": [_P, _I32, _I32, ctypes.POINTER(_I32)],
        "ssu_pool_clear": [_P, _P],
        "ssu_pool_clear_slot": [_P, _I32, _P],
        "ssu_pool_capture": [_P, _I32, ctypes.POINTER(_P), ctypes.POINTER(ctypes.c_size_t),
                             _I32, _P],
        "ssu_pool_restore": [_P, _I32, ctypes.POINTER(_P), ctypes.POINTER(ctypes.c_size_t),
                             _I32, _P],
        "ssu_pool_copy_slot_from": [_P, _P, _I32, _I32, _P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int32
    lib.ssu_tree_workspace_bytes.argtypes = [D, _I32]
    lib.ssu_tree_workspace_bytes.restype = ctypes.c_int64
    lib.ssu_gdn_workspace_bytes.argtypes = [ctypes.POINTER(ssu_gdn_dims)]
    lib.ssu_gdn_workspace_bytes.restype = ctypes.c_int64
    lib.ssu_last_error.argtypes = []
    lib.ssu_last_error.restype = ctypes.c_char_p
    lib.ssu_version.argtypes = []
    lib.ssu_version.restype = ctypes.c_int32
    if path is None:
        _LIB = lib
    return lib


def _check(status):
    if status != SSU_OK:
        raise SsuError(status, load_library().ssu_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    if stream is not None:
        return ctypes.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _dev(t, name, dtypes=None, shape=None):
    _need(t.is_cuda, f"{name} must be a GPU tensor")
    if dtypes is not None:
        _need(t.dtype in dtypes, f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if shape is not None:
        _need(tuple(t.shape) == tuple(shape), f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _dense(t, name, dtypes=None, shape=None):
    _dev(t, name, dtypes, shape)
    _need(t.is_contiguous(), f"{name} must be contiguous")
    return t


_FLOAT = (torch.float32, torch.float16, torch.bfloat16)


def _state_geometry(state, nheads, dim, dstate):
    """state: [rows, nheads, dim, dstate] with dense rows; stride(0) may be padded."""
    _dev(state, "state", _FLOAT)
    _need(state.dim() == 4 and tuple(state.shape[1:]) == (nheads, dim, dstate),
          f"state has shape {tuple(state.shape)}, expected [rows, {nheads}, {dim}, {dstate}]")
    st = state.stride()
    _need(st[3] == 1 and st[2] == dstate and st[1] == dim * dstate,
          "state rows must be dense ([nheads, dim, dstate] contiguous)")
    _need(st[0] >= nheads * dim * dstate or state.shape[0] == 1, "state row stride too small")
    stride = st[0] if state.shape[0] > 1 else nheads * dim * dstate
    return state.shape[0], stride


def _dims(batch, nheads, dim, dstate, ngroups, pool_rows, row_stride, state_dtype,
          io_dtype, bc_dtype):
    return ssu_dims(batch, nheads, dim, dstate, ngroups, pool_rows, row_stride,
                    _DT[state_dtype], _DT[io_dtype], _DT[bc_dtype], 0)


def _opt_idx(t, name, n):
    if t is None:
        return None
    return _dense(t, name, (torch.int32,), (n,))


def ssu_decode(x, A, B, C, dt, state, out, *, dt_bias=None, D=None, z=None,
               dt_softplus=True, state_indices=None, stream=None):
    """One decode step; updates `state` in place and writes `out`.

    x, z, out [batch, nheads, dim]; A, dt_bias, D [nheads] fp32; dt [batch, nheads] fp32;
    B, C [batch, ngroups, dstate]; state [rows, nheads, dim, dstate];
    state_indices [batch] int32 (negative = padding row).
    """
    lib = load_library()
    _dense(x, "x", _FLOAT)
    _need(x.dim() == 3, "x must be [batch, nheads, dim]")
    batch, nheads, dim = x.shape
    _dense(B, "B", _FLOAT)
    _need(B.dim() == 3 and B.shape[0] == batch, "B must be [batch, ngroups, dstate]")
    ngroups, dstate = B.shape[1], B.shape[2]
    _dense(C, "C", (B.dtype,), B.shape)
    _dense(A, "A", (torch.float32,), (nheads,))
    _dense(dt, "dt", (torch.float32,), (batch, nheads))
    if dt_bias is not None:
        _dense(dt_bias, "dt_bias", (torch.float32,), (nheads,))
    if D is not None:
        _dense(D, "D", (torch.float32,), (nheads,))
    if z is not None:
        _dense(z, "z", (x.dtype,), x.shape)
    _dense(out, "out", (x.dtype,), x.shape)
    rows, stride = _state_geometry(state, nheads, dim, dstate)
    _opt_idx(state_indices, "state_indices", batch)
    d = _dims(batch, nheads, dim, dstate, ngroups, rows, stride, state.dtype, x.dtype, B.dtype)
    with torch.cuda.device(x.device):
        _check(lib.ssu_decode(ctypes.byref(d), _ptr(x), _ptr(A), _ptr(B), _ptr(C), _ptr(dt),
                              _ptr(dt_bias), _ptr(D), _ptr(z), _ptr(state), _ptr(out),
                              1 if dt_softplus else 0, _ptr(state_indices),
                              _stream(x.device, stream)))
    return out


def ssu_prefill(x, A, B, C, dt, state, out, *, dt_bias=None, D=None, z=None,
                dt_softplus=True, context_lengths=None, state_indices=None,
                replay_dA=None, replay_u=None, replay_B=None, replay_dt=None, stream=None):
    """All seq_len tokens in one launch.

    x, z, out [batch, seq_len, nheads, dim]; dt [batch, seq_len, nheads];
    B, C [batch, seq_len, ngroups, dstate]; context_lengths [batch] int32.
    Replay stash (fp32, all four or none): replay_dA, replay_dt [batch, seq_len, nheads],
    replay_u [batch, seq_len, nheads, dim], replay_B [batch, seq_len, ngroups, dstate].
    """
    lib = load_library()
    _dense(x, "x", _FLOAT)
    _need(x.dim() == 4, "x must be [batch, seq_len, nheads, dim]")
    batch, seq_len, nheads, dim = x.shape
    _dense(B, "B", _FLOAT)
    _need(B.dim() == 4 and tuple(B.shape[:2]) == (batch, seq_len),
          "B must be [batch, seq_len, ngroups, dstate]")
    ngroups, dstate = B.shape[2], B.shape[3]
    _dense(C, "C", (B.dtype,), B.shape)
    _dense(A, "A", (torch.float32,), (nheads,))
    _dense(dt, "dt", (torch.float32,), (batch, seq_len, nheads))
    if dt_bias is not None:
        _dense(dt_bias, "dt_bias", (torch.float32,), (nheads,))
    if D is not None:
        _dense(D, "D", (torch.float32,), (nheads,))
    if z is not None:
        _dense(z, "z", (x.dtype,), x.shape)
    _dense(out, "out", (x.dtype,), x.shape)
    rows, stride = _state_geometry(state, nheads, dim, dstate)
    _opt_idx(state_indices, "state_indices", batch)
    _opt_idx(context_lengths, "context_lengths", batch)
    stash = (replay_dA, replay_u, replay_B, replay_dt)
    if any(s is not None for s in stash):
        _dense(replay_dA, "replay_dA", (torch.float32,), (batch, seq_len, nheads))
        _dense(replay_dt, "replay_dt", (torch.float32,), (batch, seq_len, nheads))
        _dense(replay_u, "replay_u", (torch.float32,), x.shape)
        _dense(replay_B, "replay_B", (torch.float32,), B.shape)
    d = _dims(batch, nheads, dim, dstate, ngroups, rows, stride, state.dtype, x.dtype, B.dtype)
    with torch.cuda.device(x.device):
        _check(lib.ssu_prefill(ctypes.byref(d), seq_len, _ptr(x), _ptr(A), _ptr(B), _ptr(C),
                               _ptr(dt), _ptr(dt_bias), _ptr(D), _ptr(z), _ptr(state),
                               _ptr(out), 1 if dt_softplus else 0, _ptr(context_lengths),
                               _ptr(state_indices), *[_ptr(s) for s in stash],
                               _stream(x.device, stream)))
    return out


def ssu_replay(state, replay_dA, replay_u, replay_B, replay_dt, accepted_lengths, *,
               state_indices=None, active_batch=None, accepted_node_ids=None, stream=None):
    """Apply accepted stashed tokens to the state, in place.

    replay_dA, replay_dt [batch, seq_len, nheads]; replay_u [batch, seq_len, nheads, dim];
    replay_B [batch, seq_len, ngroups, dstate]; accepted_lengths, state_indices [batch] int32.
    accepted_node_ids [batch, max_accept_len] int32: token t of row b is stash entry
    accepted_node_ids[b, t] (default: entry t). Rows b >= active_batch (default batch)
    are never read.
    """
    lib = load_library()
    _dense(replay_dA, "replay_dA", (torch.float32,))
    _need(replay_dA.dim() == 3, "replay_dA must be [batch, seq_len, nheads]")
    batch, seq_len, nheads = replay_dA.shape
    _dense(replay_u, "replay_u", (torch.float32,))
    _need(replay_u.dim() == 4 and tuple(replay_u.shape[:3]) == (batch, seq_len, nheads),
          "replay_u must be [batch, seq_len, nheads, dim]")
    dim = replay_u.shape[3]
    _dense(replay_B, "replay_B", (torch.float32,))
    _need(replay_B.dim() == 4 and tuple(replay_B.shape[:2]) == (batch, seq_len),
          "replay_B must be [batch, seq_len, ngroups, dstate]")
    ngroups, dstate = replay_B.shape[2], replay_B.shape[3]
    _dense(replay_dt, "replay_dt", (torch.float32,), (batch, seq_len, nheads))
    _dense(accepted_lengths, "accepted_lengths", (torch.int32,), (batch,))
    _opt_idx(state_indices, "state_indices", batch)
    max_accept = 0
    if accepted_node_ids is not None:
        _dense(accepted_node_ids, "accepted_node_ids", (torch.int32,))
        _need(accepted_node_ids.dim() == 2 and accepted_node_ids.shape[0] == batch,
              "accepted_node_ids must be [batch, max_accept_len]")
        max_accept = accepted_node_ids.shape[1]
    rows, stride = _state_geometry(state, nheads, dim, dstate)
    if active_batch is None:
        active_batch = batch
    d = _dims(batch, nheads, dim, dstate, ngroups, rows, stride, state.dtype, torch.float32,
              torch.float32)
    with torch.cuda.device(state.device):
        _check(lib.ssu_replay(ctypes.byref(d), seq_len, _ptr(state), _ptr(replay_dA),
                              _ptr(replay_u), _ptr(replay_B), _ptr(replay_dt),
                              _ptr(accepted_lengths), _ptr(state_indices), int(active_batch),
                              _ptr(accepted_node_ids), int(max_accept),
                              _stream(state.device, stream)))


def _tree_dims(x, A, B, C, dt, state, out, parent_ids, depths, dt_bias, D, z, state_indices,
               stash):
    """Shape checks of a tree-verify call; returns (dims, num_nodes)."""
    _dense(x, "x", _FLOAT)
    _need(x.dim() == 4, "x must be [batch, num_nodes, nheads, dim]")
    batch, num_nodes, nheads, dim = x.shape
    _dense(B, "B", _FLOAT)
    _need(B.dim() == 4 and tuple(B.shape[:2]) == (batch, num_nodes),
          "B must be [batch, num_nodes, ngroups, dstate]")
    ngroups, dstate = B.shape[2], B.shape[3]
    _dense(C, "C", (B.dtype,), B.shape)
    _dense(A, "A", (torch.float32,), (nheads,))
    _dense(dt, "dt", (torch.float32,), (batch, num_nodes, nheads))
    _dense(parent_ids, "parent_ids", (torch.int32,), (batch, num_nodes))
    if depths is not None:
        _dense(depths, "depths", (torch.int32,), (batch, num_nodes))
    if dt_bias is not None:
        _dense(dt_bias, "dt_bias", (torch.float32,), (nheads,))
    if D is not None:
        _dense(D, "D", (torch.float32,), (nheads,))
    if z is not None:
        _dense(z, "z", (x.dtype,), x.shape)
    _dense(out, "out", (x.dtype,), x.shape)
    rows, stride = _state_geometry(state, nheads, dim, dstate)
    _opt_idx(state_indices, "state_indices", batch)
    replay_dA, replay_u, replay_B, replay_dt = stash
    if any(s is not None for s in stash):
        _dense(replay_dA, "replay_dA", (torch.float32,), (batch, num_nodes, nheads))
        _dense(replay_dt, "replay_dt", (torch.float32,), (batch, num_nodes, nheads))
        _dense(replay_u, "replay_u", (torch.float32,), x.shape)
        _dense(replay_B, "replay_B", (torch.float32,), B.shape)
    return _dims(batch, nheads, dim, dstate, ngroups, rows, stride, state.dtype, x.dtype,
                 B.dtype), num_nodes


def ssu_tree_verify(x, A, B, C, dt, state, out, parent_ids, *, depths=None, dt_bias=None,
                    D=None, z=None, dt_softplus=True, state_indices=None, replay_dA=None,
                    replay_u=None, replay_B=None, replay_dt=None, workspace=None, stream=None):
    """Every node of a draft tree per batch row, from the read-only committed state.

    x, z, out [batch, num_nodes, nheads, dim]; dt [batch, num_nodes, nheads];
    B, C [batch, num_nodes, ngroups, dstate]; parent_ids, depths [batch, num_nodes] int32.
    Replay stash (fp32, all four or none) in the ssu_prefill layouts with the node axis.
    workspace: a uint8 GPU tensor of at least tree_workspace_bytes(...) bytes (allocated
    here when None).
    """
    lib = load_library()
    stash = (replay_dA, replay_u, replay_B, replay_dt)
    d, num_nodes = _tree_dims(x, A, B, C, dt, state, out, parent_ids, depths, dt_bias, D, z,
                              state_indices, stash)
    if workspace is None:
        need = max(int(lib.ssu_tree_workspace_bytes(ctypes.byref(d), num_nodes)), 16)
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _dense(workspace, "workspace", (torch.uint8,))
    with torch.cuda.device(x.device):
        _check(lib.ssu_tree_verify(ctypes.byref(d), num_nodes, _ptr(x), _ptr(A), _ptr(B),
                                   _ptr(C), _ptr(dt), _ptr(dt_bias), _ptr(D), _ptr(z),
                                   _ptr(state), _ptr(out), 1 if dt_softplus else 0,
                                   _ptr(state_indices), _ptr(parent_ids), _ptr(depths),
                                   *[_ptr(s) for s in stash], _ptr(workspace),
                                   workspace.numel(), _stream(x.device, stream)))
    return out


def ssu_tree_verify_noalloc(x, A, B, C, dt, state, out, parent_ids, *, depths=None,
                            dt_bias=None, D=None, z=None, dt_softplus=True, state_indices=None,
                            replay_dA=None, replay_u=None, replay_B=None, replay_dt=None,
                            stream=None):
    """ssu_tree_verify without a workspace: the library's per-GPU scratch of
    SSU_TREE_SCRATCH_BYTES holds the B.C dots, so nothing is allocated (for
    code under graph capture). Calls that overlap on one GPU race on it."""
    lib = load_library()
    stash = (replay_dA, replay_u, replay_B, replay_dt)
    d, num_nodes = _tree_dims(x, A, B, C, dt, state, out, parent_ids, depths, dt_bias, D, z,
                              state_indices, stash)
    with torch.cuda.device(x.device):
        _check(lib.ssu_tree_verify_noalloc(ctypes.byref(d), num_nodes, _ptr(x), _ptr(A), _ptr(B),
                                           _ptr(C), _ptr(dt), _ptr(dt_bias), _ptr(D), _ptr(z),
                                           _ptr(state), _ptr(out), 1 if dt_softplus else 0,
                                           _ptr(state_indices), _ptr(parent_ids), _ptr(depths),
                                           *[_ptr(s) for s in stash], _stream(x.device, stream)))
    return out


TREE_SCRATCH_BYTES = 4194304  # SSU_TREE_SCRATCH_BYTES of include/ssu.h


def tree_workspace_bytes(batch, ngroups, num_nodes):
    """Bytes of the workspace ssu_tree_verify needs (no GPU needed)."""
    return 4 * batch * ngroups * num_nodes * num_nodes


def _device_table(structs, device):
    """Pack ctypes structs into one device buffer (a uint8 tensor)."""
    n = len(structs)
    size = ctypes.sizeof(structs[0]) if n else 0
    raw = bytearray(size * n)
    for i, st in enumerate(structs):
        ctypes.memmove((ctypes.c_char * size).from_buffer(raw, i * size), ctypes.addressof(st), size)
    host = torch.frombuffer(raw, dtype=torch.uint8) if n else torch.empty(0, dtype=torch.uint8)
    return host.to(device)


class ReplayLayerTable:
    """Device array of per-layer replay buffers for ssu_replay_layers.

    states[i] [rows, nheads, dim, dstate]; dAs[i], dts[i] [batch, seq_len, nheads];
    us[i] [batch, seq_len, nheads, dim]; Bs[i] [batch, seq_len, ngroups, dstate] (fp32).
    Every layer has the same shapes and dtypes. Keeps the tensors alive."""

    def __init__(self, states, dAs, us, Bs, dts):
        n = len(states)
        _need(n > 0 and all(len(v) == n for v in (dAs, us, Bs, dts)), "one entry per layer")
        s0, a0, u0, b0 = states[0], dAs[0], us[0], Bs[0]
        for i in range(n):
            _need(states[i].dtype == s0.dtype and states[i].shape == s0.shape and
                  states[i].stride() == s0.stride(), "every layer's state has the same geometry")
            _dense(dAs[i], "replay_dA", (torch.float32,), a0.shape)
            _dense(dts[i], "replay_dt", (torch.float32,), a0.shape)
            _dense(us[i], "replay_u", (torch.float32,), u0.shape)
            _dense(Bs[i], "replay_B", (torch.float32,), b0.shape)
        _need(a0.dim() == 3 and u0.dim() == 4 and b0.dim() == 4, "stash shapes")
        self.batch, self.seq_len, self.nheads = a0.shape
        self.dim = u0.shape[3]
        self.ngroups, self.dstate = b0.shape[2], b0.shape[3]
        self.rows, self.stride = _state_geometry(s0, self.nheads, self.dim, self.dstate)
        self.state_dtype = s0.dtype
        self.keep = (states, dAs, us, Bs, dts)
        self.num_layers = n
        self.device = s0.device
        self.table = _device_table([ssu_replay_layer(states[i].data_ptr(), dAs[i].data_ptr(),
                                                     us[i].data_ptr(), Bs[i].data_ptr(),
                                                     dts[i].data_ptr()) for i in range(n)],
                                   self.device)


def ssu_replay_layers(table: ReplayLayerTable, accepted_lengths, *, state_indices=None,
                      active_batch=None, accepted_node_ids=None, stream=None):
    """ssu_replay for every layer of `table` in one launch (shared accepted
    lengths, state indices and node ids)."""
    lib = load_library()
    _dense(accepted_lengths, "accepted_lengths", (torch.int32,), (table.batch,))
    _opt_idx(state_indices, "state_indices", table.batch)
    max_accept = 0
    if accepted_node_ids is not None:
        _dense(accepted_node_ids, "accepted_node_ids", (torch.int32,))
        _need(accepted_node_ids.dim() == 2 and accepted_node_ids.shape[0] == table.batch,
              "accepted_node_ids must be [batch, max_accept_len]")
        max_accept = accepted_node_ids.shape[1]
    if active_batch is None:
        active_batch = table.batch
    d = _dims(table.batch, table.nheads, table.dim, table.dstate, table.ngroups, table.rows,
              table.stride, table.state_dtype, torch.float32, torch.float32)
    with torch.cuda.device(table.device):
        _check(lib.ssu_replay_layers(ctypes.byref(d), table.seq_len, _ptr(table.table),
                                     table.num_layers, _ptr(accepted_lengths),
                                     _ptr(state_indices), int(active_batch),
                                     _ptr(accepted_node_ids), int(max_accept),
                                     _stream(table.device, stream)))


class StateLayerTable:
    """Device array of per-layer {recurrent, conv} state buffers for
    ssu_state_clear_layers. Entries may be None (that buffer is skipped)."""

    def __init__(self, recurrent, conv):
        _need(len(recurrent) == len(conv) and len(recurrent) > 0, "one entry per layer")
        self.keep = (recurrent, conv)
        self.num_layers = len(recurrent)
        dev = next(t.device for t in list(recurrent) + list(conv) if t is not None)
        self.device = dev
        self.table = _device_table([ssu_state_layer(0 if r is None else r.data_ptr(),
                                                    0 if c is None else c.data_ptr())
                                    for r, c in zip(recurrent, conv)], dev)


def ssu_state_clear_layers(table: StateLayerTable, resident_rows, slot, recurrent_row_bytes,
                           conv_row_bytes, stream=None):
    """Zero row `slot` (or every row, slot -1) of both states of every layer."""
    lib = load_library()
    with torch.cuda.device(table.device):
        _check(lib.ssu_state_clear_layers(_ptr(table.table), table.num_layers, int(resident_rows),
                                          int(slot), int(recurrent_row_bytes),
                                          int(conv_row_bytes), _stream(table.device, stream)))


def _rows(t, name):
    """(rows, row_bytes, row stride in bytes) of a tensor whose leading dim is the row."""
    _dev(t, name)
    _need(t.dim() >= 1, f"{name} needs a leading row dimension")
    inner = t[0] if t.shape[0] > 0 else t.new_empty(t.shape[1:])
    _need(inner.is_contiguous(), f"{name} rows must be dense")
    row_bytes = inner.numel() * t.element_size()
    stride = t.stride(0) * t.element_size() if t.shape[0] > 1 else row_bytes
    return t.shape[0], row_bytes, stride


def ssu_state_gather(resident, active, state_indices, stream=None):
    """active[b] = resident[state_indices[b]]; a negative index gives a zero row."""
    lib = load_library()
    rr, rb, rs = _rows(resident, "resident")
    ar, ab, ast = _rows(active, "active")
    _need(rb == ab and resident.dtype == active.dtype, "resident and active rows must match")
    _dense(state_indices, "state_indices", (torch.int32,), (ar,))
    with torch.cuda.device(active.device):
        _check(lib.ssu_state_gather(_ptr(resident), rr, rs, _ptr(active), ast,
                                    _ptr(state_indices), ar, rb, _stream(active.device, stream)))


def ssu_state_scatter(active, resident, state_indices, stream=None):
    """resident[state_indices[b]] = active[b] for non-negative indices."""
    lib = load_library()
    rr, rb, rs = _rows(resident, "resident")
    ar, ab, ast = _rows(active, "active")
    _need(rb == ab and resident.dtype == active.dtype, "resident and active rows must match")
    _dense(state_indices, "state_indices", (torch.int32,), (ar,))
    with torch.cuda.device(active.device):
        _check(lib.ssu_state_scatter(_ptr(active), ast, _ptr(resident), rr, rs,
                                     _ptr(state_indices), ar, rb, _stream(active.device, stream)))


def pack_workspace_bytes(pool, batch, n_bystanders):
    """Bytes of the workspace ssu_state_pack / ssu_state_unpack need (pool: any
    tensor whose leading dimension is the row)."""
    row_bytes = int(torch.Size(pool.shape[1:]).numel()) * pool.element_size()
    return (batch + n_bystanders) * row_bytes


def _pack_call(fn, pool, homes, bystanders, workspace, stream):
    lib = load_library()
    rows, rb, rs = _rows(pool, "pool")
    _dense(homes, "homes", (torch.int32,))
    _need(homes.dim() == 1, "homes must be 1-D")
    nb = 0
    if bystanders is not None:
        _dense(bystanders, "bystanders", (torch.int32,))
        nb = bystanders.numel()
    _dev(workspace, "workspace")
    _need(workspace.numel() * workspace.element_size() >= (homes.numel() + nb) * rb,
          "workspace too small")
    with torch.cuda.device(pool.device):
        _check(getattr(lib, fn)(_ptr(pool), rows, rs, rb, _ptr(homes), homes.numel(),
                                _ptr(bystanders) if nb else None, nb, _ptr(workspace),
                                _stream(pool.device, stream)))


def ssu_state_pack(pool, homes, workspace, bystanders=None, stream=None):
    """Slots [0, len(homes)) of `pool` get the rows homes[b] held (all read first);
    bystander rows are saved in `workspace` for ssu_state_unpack."""
    _pack_call("ssu_state_pack", pool, homes, bystanders, workspace, stream)


def ssu_state_unpack(pool, homes, workspace, bystanders=None, stream=None):
    """Slots [0, len(homes)) go back to their homes; bystanders are restored."""
    _pack_call("ssu_state_unpack", pool, homes, bystanders, workspace, stream)


def ssu_gdn_decode(hidden_states, w_ba, mixed_qkv, conv_weight, conv_bias, conv_state, A_log,
                   dt_bias, scale, ssm_state, state_indices, *, num_q_heads, use_qk_l2norm=True,
                   out=None, workspace=None, stream=None):
    """Fused gated-delta-rule decode step (one token per batch entry) over paged
    conv / ssm pools, both updated in place. conv_state: a [P, qkv_dim, W-1]
    view of any strides (a dense pool, or the transposed view of a
    [P, W-1, qkv_dim] pool). workspace: a uint8 GPU tensor of at least
    gdn_workspace_bytes(...) bytes (allocated here when None). Returns
    out [B, 1, HV, D] (bf16)."""
    lib = load_library()
    bf = (torch.bfloat16,)
    _dense(hidden_states, "hidden_states", bf)
    B, hidden = hidden_states.shape
    _dense(w_ba, "w_ba", bf)
    _need(w_ba.dim() == 2 and w_ba.shape[0] == hidden and w_ba.shape[1] % 2 == 0,
          "w_ba must be [hidden, 2*HV]")
    hv = w_ba.shape[1] // 2
    hq = int(num_q_heads)
    _need(hq > 0 and hv % hq == 0, "num_v_heads must be a multiple of num_q_heads")
    _dense(conv_weight, "conv_weight", bf)
    qkv, width = conv_weight.shape
    _need(qkv % (2 * hq + hv) == 0, "qkv_dim must be (2*Hq + HV)*D")
    d = qkv // (2 * hq + hv)
    _dense(mixed_qkv, "mixed_qkv", bf, (B, qkv))
    _dense(conv_bias, "conv_bias", bf, (qkv,))
    _dev(conv_state, "conv_state", bf)
    _need(conv_state.dim() == 3 and tuple(conv_state.shape[1:]) == (qkv, width - 1),
          "conv_state must be a [P, qkv_dim, W-1] view")
    _dense(A_log, "A_log", (torch.float32,), (hv,))
    _dense(dt_bias, "dt_bias", bf, (hv,))
    _dev(ssm_state, "ssm_state", (torch.float32,))
    _need(ssm_state.dim() == 4 and tuple(ssm_state.shape[1:]) == (hv, d, d),
          "ssm_state must be [P, HV, D, D]")
    st = ssm_state.stride()
    _need(st[3] == 1 and st[2] == d and st[1] == d * d, "ssm_state rows must be dense")
    _need(ssm_state.shape[0] == conv_state.shape[0], "both pools have the same slots")
    _dense(state_indices, "state_indices", (torch.int32,), (B,))
    if out is None:
        out = torch.empty((B, 1, hv, d), dtype=torch.bfloat16, device=hidden_states.device)
    _dense(out, "out", bf, (B, 1, hv, d))
    cs = conv_state.stride()
    dims = ssu_gdn_dims(B, hidden, hq, hv, d, width, ssm_state.shape[0],
                        1 if use_qk_l2norm else 0,
                        st[0] if ssm_state.shape[0] > 1 else hv * d * d, cs[0], cs[1], cs[2])
    sc = 0.0 if scale is None else float(scale)
    need = int(lib.ssu_gdn_workspace_bytes(ctypes.byref(dims)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=hidden_states.device)
    _dense(workspace, "workspace", (torch.uint8,))
    with torch.cuda.device(hidden_states.device):
        _check(lib.ssu_gdn_decode(ctypes.byref(dims), _ptr(hidden_states), _ptr(w_ba),
                                  _ptr(mixed_qkv), _ptr(conv_weight), _ptr(conv_bias),
                                  _ptr(conv_state), _ptr(A_log), _ptr(dt_bias), sc,
                                  _ptr(ssm_state), _ptr(state_indices), _ptr(out),
                                  _ptr(workspace), workspace.numel(),
                                  _stream(hidden_states.device, stream)))
    return out


def gdn_workspace_bytes(batch, hidden, num_q_heads, num_v_heads, head_dim):
    """Bytes of the workspace ssu_gdn_decode needs (no GPU needed)."""
    d = ssu_gdn_dims(batch, hidden, num_q_heads, num_v_heads, head_dim, 1, 1, 1, 0, 0, 0, 0)
    return int(load_library().ssu_gdn_workspace_bytes(ctypes.byref(d)))


# ---------------------------------------------------------------------------
# Recurrent-state pool
# ---------------------------------------------------------------------------
class DeviceArray:
    """Non-owning view of pool memory: enough of the tensor protocol for the SSU
    entry points (data_ptr, shape, stride, dtype, device) plus
    __cuda_array_interface__ for zero-copy interop."""

    _TYPESTR = {torch.float32: "<f4", torch.float16: "<f2", torch.bfloat16: "<V2",
                torch.uint8: "|u1"}

    def __init__(self, ptr, shape, dtype, device, owner):
        self._ptr, self.shape, self.dtype, self.device = ptr, tuple(shape), dtype, device
        self._owner = owner  # keeps the pool alive
        st, acc = [], 1
        for s in reversed(self.shape):
            st.append(acc)
            acc *= s
        self._stride = tuple(reversed(st))
        self.is_cuda = True

    def data_ptr(self):
        return self._ptr

    def stride(self):
        return self._stride

    def dim(self):
        return len(self.shape)

    @property
    def __cuda_array_interface__(self):
        return {"shape": self.shape, "typestr": self._TYPESTR[self.dtype],
                "data": (self._ptr, False), "version": 3, "strides": None}


class SsuPool:
    """Handle of an ssu_pool: one zeroed [slot_count] + shape slab per spec.

    specs: sequence of (kind, layer, shape, dtype) with dtype a torch dtype
    (float32, float16, bfloat16 or uint8). name: the pool's name in the
    library's diagnostics. base: None (the library allocates the slabs) or a
    uint8 GPU tensor of at least slab_bytes(specs, slot_count) bytes, 256-byte
    aligned, in which the states are laid out (the pool then owns no memory and
    keeps a reference to the tensor).
    """

    def __init__(self, specs: Sequence, slot_count: int, *, name=None, base=None, stream=None,
                 device=None):
        self._lib = load_library()
        if base is not None:
            _dense(base, "base", (torch.uint8,))
            device = base.device if device is None else device
        self.device = (torch.device("cuda", torch.cuda.current_device()) if device is None
                       else torch.device(device))
        arr = self._spec_array(specs)
        self.specs = [(kind, layer, tuple(int(v) for v in shape), dtype)
                      for (kind, layer, shape, dtype) in specs]
        self._base = base
        self._h = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            _check(self._lib.ssu_pool_alloc(arr, len(specs), slot_count,
                                            None if name is None else name.encode(),
                                            _ptr(base) if base is not None else None,
                                            0 if base is None else base.numel(),
                                            _stream(self.device, stream), ctypes.byref(self._h)))
        self.slot_count = slot_count

    @staticmethod
    def _spec_array(specs):
        arr = (ssu_state_spec * max(len(specs), 1))()
        for i, (kind, layer, shape, dtype) in enumerate(specs):
            shape = tuple(int(v) for v in shape)
            _need(1 <= len(shape) <= 4, "spec shape must have 1..4 entries")
            arr[i].kind, arr[i].layer, arr[i].rank = kind, layer, len(shape)
            arr[i].dtype = _DT.get(dtype, 99)
            for k, v in enumerate(shape):
                arr[i].shape[k] = v
        return arr

    @staticmethod
    def bytes_per_slot(specs):
        lib = load_library()
        out = ctypes.c_size_t()
        _check(lib.ssu_pool_bytes_per_slot(SsuPool._spec_array(specs), len(specs),
                                           ctypes.byref(out)))
        return out.value

    @staticmethod
    def slab_bytes(specs, slot_count):
        """Bytes a caller slab (`base`) must hold for these specs and slots."""
        lib = load_library()
        out = ctypes.c_size_t()
        _check(lib.ssu_pool_slab_bytes(SsuPool._spec_array(specs), len(specs), slot_count,
                                       ctypes.byref(out)))
        return out.value

    @property
    def name(self):
        p = ctypes.c_char_p()
        _check(self._lib.ssu_pool_name(self._h, ctypes.byref(p)))
        return p.value.decode()

    @property
    def owns_memory(self):
        o = ctypes.c_int32()
        _check(self._lib.ssu_pool_owns_memory(self._h, ctypes.byref(o)))
        return bool(o.value)

    def spec(self, i):
        """(kind, layer, shape, dtype) of state i, as the library holds it."""
        sp = ssu_state_spec()
        _check(self._lib.ssu_pool_spec(self._h, i, ctypes.byref(sp)))
        return self._spec_tuple(sp)

    def specs_from_library(self):
        n = ctypes.c_int32()
        _check(self._lib.ssu_pool_specs(self._h, None, 0, ctypes.byref(n)))
        arr = (ssu_state_spec * max(n.value, 1))()
        _check(self._lib.ssu_pool_specs(self._h, arr, n.value, ctypes.byref(n)))
        return [self._spec_tuple(arr[i]) for i in range(n.value)]

    @staticmethod
    def _spec_tuple(sp):
        dt = {v: k for k, v in _DT.items()}[sp.dtype]
        return (sp.kind, sp.layer, tuple(int(sp.shape[k]) for k in range(sp.rank)), dt)

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            _check(self._lib.ssu_pool_free(self._h))
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def num_states(self):
        n, s = ctypes.c_int32(), ctypes.c_int32()
        _check(self._lib.ssu_pool_info(self._h, ctypes.byref(n), ctypes.byref(s)))
        return n.value

    def state_bytes_per_slot(self, i):
        out = ctypes.c_size_t()
        _check(self._lib.ssu_pool_state_bytes_per_slot(self._h, i, ctypes.byref(out)))
        return out.value

    def find_state(self, kind, layer):
        out = ctypes.c_int32()
        _check(self._lib.ssu_pool_find_state(self._h, kind, layer, ctypes.byref(out)))
        return out.value

    def state(self, i):
        """DeviceArray view of state i, shaped [slot_count] + spec shape."""
        p = ctypes.c_void_p()
        _check(self._lib.ssu_pool_state_ptr(self._h, i, ctypes.byref(p)))
        kind, layer, shape, dtype = self.specs[i]
        return DeviceArray(p.value or 0, (self.slot_count,) + shape, dtype, self.device, self)

    def clear(self, stream=None):
        _check(self._lib.ssu_pool_clear(self._h, _stream(self.device, stream)))

    def clear_slot(self, slot, stream=None):
        _check(self._lib.ssu_pool_clear_slot(self._h, slot, _stream(self.device, stream)))

    def capture(self, slot, dst=None, stream=None):
        """Copy one slot of every state into `dst` (list of GPU tensors, allocated
        here when None) and return it."""
        if dst is None:
            dst = [torch.empty((1,) + shape, dtype=dtype, device=self.device)
                   for (_, _, shape, dtype) in self.specs]
        n = len(dst)
        ptrs = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in dst])
        sizes = (ctypes.c_size_t * max(n, 1))(*[t.numel() * t.element_size() for t in dst])
        _check(self._lib.ssu_pool_capture(self._h, slot, ptrs, sizes, n,
                                          _stream(self.device, stream)))
        return dst

    def restore(self, saved, slot, stream=None):
        n = len(saved)
        ptrs = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in saved])
        sizes = (ctypes.c_size_t * max(n, 1))(*[t.numel() * t.element_size() for t in saved])
        _check(self._lib.ssu_pool_restore(self._h, slot, ptrs, sizes, n,
                                          _stream(self.device, stream)))

    def copy_slot_from(self, source: "SsuPool", dst_slot, src_slot, stream=None):
        _check(self._lib.ssu_pool_copy_slot_from(self._h, source._h, dst_slot, src_slot,
                                                 _stream(self.device, stream)))
