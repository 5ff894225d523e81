"""fp64 CPU oracle for the selective state update (numpy front end over ssu_oracle.c).

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg are the only callers.  The HIP library never imports, links
or calls anything here, and nothing here imports the HIP library.

All arrays are float64 (int32 for index arrays) in the layouts of the
TensorRT-Edge-LLM "Selective State Update" page (invokeSelectiveStateUpdate
shape list; invokeSelectiveStateUpdatePrefill; MambaReplayLayerInfo):

  decode : x [b,h,d]  B,C [b,g,n]  dt [b,h]  z/out [b,h,d]
  prefill: x [b,t,h,d]  B,C [b,t,g,n]  dt [b,t,h]  z/out [b,t,h,d]
  replay : dA,DT [b,t,h]  u [b,t,h,d]  Bst [b,t,g,n]  node_ids [b, max_accept_len]
  tree   : prefill layouts with the node axis in place of t; parent_ids and
           depths [b, num_nodes] (invokeSelectiveStateUpdateDDTree)
  layers : lists of per-layer states / stashes (invokeMambaReplayReconstructBatched,
           invokeMambaStateClear)
  gdn    : the fused gated-delta-rule decode step of FlashInfer's
           gdn_fused_decode_step page (gdn_oracle.c)
  state  : [rows, h, d, n], or a flat buffer with `row_stride` elements per row

`state`, `out` and the stash arrays are updated in place.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None
_F64P = ctypes.POINTER(ctypes.c_double)
_I32P = ctypes.POINTER(ctypes.c_int32)


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        lib.oracle_ssu_decode.argtypes = [i32] * 5 + [i64] + [_F64P] * 10 + [i32, _I32P]
        lib.oracle_ssu_prefill.argtypes = ([i32] * 6 + [i64] + [_F64P] * 10 + [i32, _I32P, _I32P]
                                           + [_F64P] * 5)
        lib.oracle_ssu_replay.argtypes = ([i32] * 6 + [i64] + [_F64P] * 5 + [_I32P] * 3
                                          + [i32])
        lib.oracle_ssu_tree.argtypes = ([i32] * 6 + [i64] + [_F64P] * 10 + [i32] + [_I32P] * 3
                                        + [_F64P] * 5)
        for f in (lib.oracle_ssu_decode, lib.oracle_ssu_prefill, lib.oracle_ssu_replay,
                  lib.oracle_ssu_tree):
            f.restype = None
        lib.oracle_gdn_decode.argtypes = ([i32] * 6 + [_F64P] * 5 + [_F64P] + [i64] * 3
                                          + [_F64P] * 2 + [ctypes.c_double] + [_F64P] + [i64]
                                          + [_I32P, i32, _F64P])
        lib.oracle_gdn_decode.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int32
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int32]
        lib.oracle_set_num_threads.restype = None
        _LIB = lib
    return _LIB


def _f64(a, name, writable=False):
    if a is None:
        return None, None
    if not isinstance(a, np.ndarray) or a.dtype != np.float64 or not a.flags.c_contiguous:
        if writable:
            raise TypeError(f"{name} must be a C-contiguous float64 ndarray (updated in place)")
        a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(_F64P)


def _i32(a):
    if a is None:
        return None, None
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(_I32P)


def _row_stride(state, nheads, dim, dstate, row_stride):
    tile = nheads * dim * dstate
    if row_stride in (None, 0):
        row_stride = tile
    if row_stride < tile:
        raise ValueError("row_stride smaller than one pool row")
    return row_stride


def decode(x, A, B, C, dt, state, out, *, dt_bias=None, D=None, z=None,
           dt_softplus=True, state_indices=None, row_stride=None):
    batch, nheads, dim = x.shape
    ngroups, dstate = B.shape[1], B.shape[2]
    rs = _row_stride(state, nheads, dim, dstate, row_stride)
    keep = [_f64(v, k) for k, v in (("x", x), ("A", A), ("B", B), ("C", C), ("dt", dt),
                                     ("dt_bias", dt_bias), ("D", D), ("z", z))]
    st = _f64(state, "state", True)
    ot = _f64(out, "out", True)
    ix = _i32(state_indices)
    _lib().oracle_ssu_decode(batch, nheads, dim, dstate, ngroups, rs,
                             *[k[1] for k in keep[:8]], st[1], ot[1],
                             1 if dt_softplus else 0, ix[1])


def prefill(x, A, B, C, dt, state, out, *, dt_bias=None, D=None, z=None,
            dt_softplus=True, context_lengths=None, state_indices=None,
            stash=None, row_stride=None):
    """stash: None or dict of float64 arrays 'dA', 'u', 'B', 'dt' (filled in)."""
    batch, seq_len, nheads, dim = x.shape
    ngroups, dstate = B.shape[2], B.shape[3]
    rs = _row_stride(state, nheads, dim, dstate, row_stride)
    keep = [_f64(v, k) for k, v in (("x", x), ("A", A), ("B", B), ("C", C), ("dt", dt),
                                     ("dt_bias", dt_bias), ("D", D), ("z", z))]
    st = _f64(state, "state", True)
    ot = _f64(out, "out", True)
    cl = _i32(context_lengths)
    ix = _i32(state_indices)
    if stash is not None:
        sd = [_f64(stash[k], "stash " + k, True) for k in ("dA", "u", "B", "dt")]
        scratch = np.empty(batch * nheads * dim * dstate, dtype=np.float64)
        sp = [s[1] for s in sd] + [scratch.ctypes.data_as(_F64P)]
    else:
        sp = [None] * 5
    _lib().oracle_ssu_prefill(batch, seq_len, nheads, dim, dstate, ngroups, rs,
                              *[k[1] for k in keep[:8]], st[1], ot[1],
                              1 if dt_softplus else 0, cl[1], ix[1], *sp)


def replay(state, dA, u, Bst, DT, accepted_lengths, *, state_indices=None,
           active_batch=None, row_stride=None, node_ids=None):
    """node_ids: None (token t is stash entry t) or int32 [b, max_accept_len]."""
    nb, seq_len, nheads = dA.shape
    dim = u.shape[3]
    ngroups, dstate = Bst.shape[2], Bst.shape[3]
    if active_batch is None:
        active_batch = nb
    rs = _row_stride(state, nheads, dim, dstate, row_stride)
    keep = [_f64(v, k) for k, v in (("dA", dA), ("u", u), ("B", Bst), ("DT", DT))]
    st = _f64(state, "state", True)
    ac = _i32(accepted_lengths)
    ix = _i32(state_indices)
    ni = _i32(node_ids)
    max_accept = 0 if node_ids is None else ni[0].shape[1]
    _lib().oracle_ssu_replay(active_batch, seq_len, nheads, dim, dstate, ngroups, rs,
                             st[1], *[k[1] for k in keep], ac[1], ix[1], ni[1], max_accept)


def replay_layers(states, stashes, accepted_lengths, *, state_indices=None, active_batch=None,
                  node_ids=None, row_stride=None):
    """Replay of every layer (TensorRT-Edge-LLM "Selective State Update" page,
    invokeMambaReplayReconstructBatched: the MambaReplayLayerInfo replay for each of
    numLayers layers, with acceptedLengths, stateIndices, activeBatchSize and
    acceptedNodeIds shared by all layers). states[i] is updated in place; stashes[i]
    is a dict with 'dA', 'u', 'B', 'dt'."""
    for st, S in zip(states, stashes):
        replay(st, S["dA"], S["u"], S["B"], S["dt"], accepted_lengths,
               state_indices=state_indices, active_batch=active_batch, row_stride=row_stride,
               node_ids=node_ids)


def clear_layers(recurrent, conv, resident_rows, slot, recurrent_row_bytes, conv_row_bytes):
    """Zero resident row `slot`, or every row when slot == -1, of the recurrent and
    the conv state of every layer (same page, MambaStateLayerInfo and
    invokeMambaStateClear). Buffers are uint8 arrays of resident_rows rows of the
    given byte count (None: absent); updated in place."""
    for bufs, rb in ((recurrent, recurrent_row_bytes), (conv, conv_row_bytes)):
        for buf in bufs:
            if buf is None or rb == 0:
                continue
            if slot == -1:
                buf[: resident_rows * rb] = 0
            else:
                buf[slot * rb:(slot + 1) * rb] = 0


def gather(resident, state_indices):
    """Active rows from a pool (TensorRT-Edge-LLM "Selective State Update" page,
    invokeMambaStateGather): row b is resident[state_indices[b]]; a negative index
    (padding, FlashInfer gdn_fused_decode_step page, state_indices) gives zeros."""
    out = np.zeros((len(state_indices),) + resident.shape[1:], dtype=resident.dtype)
    for b, r in enumerate(state_indices):
        if r >= 0:
            out[b] = resident[r]
    return out


def scatter(active, resident, state_indices):
    """invokeMambaStateScatter (same page): resident[state_indices[b]] = active[b] for
    non-negative indices; `resident` is updated in place."""
    for b, r in enumerate(state_indices):
        if r >= 0:
            resident[r] = active[b]


def pack(pool, homes, bystanders):
    """activateStep (Smile "Class DeltaNetStatePool" page): every source row is read
    first, then slot b of the pool gets the row homes[b] held; the bystander rows
    (live rows of other requests with homes in [0, B)) are saved and returned."""
    src = [pool[h].copy() for h in homes]
    saved = [pool[r].copy() for r in bystanders]
    for b, row in enumerate(src):
        pool[b] = row
    return saved


def unpack(pool, homes, bystanders, saved):
    """scatterActive (same page): working slots [0, B) go back to their homes (all
    slots read first), then the saved bystander rows are put back."""
    slots = [pool[b].copy() for b in range(len(homes))]
    for b, h in enumerate(homes):
        pool[h] = slots[b]
    for r, row in zip(bystanders, saved):
        pool[r] = row


def gdn_decode(hidden_states, w_ba, mixed_qkv, conv_weight, conv_bias, conv_state, A_log,
               dt_bias, scale, ssm_state, state_indices, *, num_q_heads, use_qk_l2norm=True,
               out=None, conv_strides=None, ssm_row_stride=None):
    """Fused gated-delta-rule decode step (FlashInfer "flashinfer.gdn_fused_decode_step"
    page; formulas in oracle/gdn_oracle.c). Shapes: hidden_states [B, hidden],
    w_ba [hidden, 2 HV], mixed_qkv [B, (2 Hq + HV) D], conv_weight [qkv_dim, W],
    conv_bias [qkv_dim], conv_state [P, qkv_dim, W-1] (or a flat buffer with
    conv_strides = (slot, channel, tap) element strides), A_log / dt_bias [HV],
    ssm_state [P, HV, D, D] (V-major, K-last). conv_state, ssm_state and out
    ([B, 1, HV, D]) are updated in place; out is returned."""
    B, hidden = hidden_states.shape
    hv = w_ba.shape[1] // 2
    hq = num_q_heads
    dhead = conv_weight.shape[0] // (2 * num_q_heads + hv)
    width = conv_weight.shape[1]
    keep = [_f64(v, k) for k, v in (("hidden_states", hidden_states), ("w_ba", w_ba),
                                     ("mixed_qkv", mixed_qkv), ("conv_weight", conv_weight),
                                     ("conv_bias", conv_bias), ("A_log", A_log),
                                     ("dt_bias", dt_bias))]
    cs = _f64(conv_state, "conv_state", True)
    st = _f64(ssm_state, "ssm_state", True)
    if out is None:
        out = np.zeros((B, 1, hv, dhead))
    ot = _f64(out, "out", True)
    if conv_strides is None:
        conv_strides = (conv_state.shape[1] * conv_state.shape[2], conv_state.shape[2], 1)
    if scale is None or scale == 0.0:
        scale = 1.0 / np.sqrt(dhead)
    ix = _i32(state_indices)
    row_stride = hv * dhead * dhead if ssm_row_stride is None else int(ssm_row_stride)
    _lib().oracle_gdn_decode(B, hidden, hq, hv, dhead, width, keep[0][1], keep[1][1], keep[2][1],
                             keep[3][1], keep[4][1], cs[1], *[int(x) for x in conv_strides],
                             keep[5][1], keep[6][1], float(scale), st[1], row_stride, ix[1],
                             1 if use_qk_l2norm else 0, ot[1])
    return out


MAX_NODES = 128


def tree(x, A, B, C, dt, state, out, parent_ids, *, depths=None, dt_bias=None, D=None, z=None,
         dt_softplus=True, state_indices=None, stash=None, row_stride=None):
    """Tree verify: x [b,n,h,d], B/C [b,n,g,s], dt [b,n,h], parent_ids/depths [b,n].

    `state` is only read. stash: None or dict of float64 arrays 'dA', 'u', 'B',
    'dt' (filled in for every node of every live row)."""
    batch, num_nodes, nheads, dim = x.shape
    if num_nodes > MAX_NODES:
        raise ValueError(f"a draft tree holds at most {MAX_NODES} nodes")
    ngroups, dstate = B.shape[2], B.shape[3]
    rs = _row_stride(state, nheads, dim, dstate, row_stride)
    keep = [_f64(v, k) for k, v in (("x", x), ("A", A), ("B", B), ("C", C), ("dt", dt),
                                     ("dt_bias", dt_bias), ("D", D), ("z", z))]
    st = _f64(state, "state")
    ot = _f64(out, "out", True)
    ix = _i32(state_indices)
    pa = _i32(parent_ids)
    dp = _i32(depths)
    scratch = np.empty(batch * nheads * (dim * dstate + dim), dtype=np.float64)
    if stash is not None:
        sd = [_f64(stash[k], "stash " + k, True) for k in ("dA", "u", "B", "dt")]
        sp = [s[1] for s in sd]
    else:
        sp = [None] * 4
    _lib().oracle_ssu_tree(batch, num_nodes, nheads, dim, dstate, ngroups, rs,
                           *[k[1] for k in keep[:8]], st[1], ot[1], 1 if dt_softplus else 0,
                           ix[1], pa[1], dp[1], *sp, scratch.ctypes.data_as(_F64P))


def num_threads():
    """OpenMP threads the oracle's loops run on."""
    return int(_lib().oracle_num_threads())


def set_num_threads(n):
    """Thread count of the oracle's OpenMP loops in this thread's later calls."""
    _lib().oracle_set_num_threads(int(n))
