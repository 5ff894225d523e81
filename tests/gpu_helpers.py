"""Shared helpers for the GPU parity tests (not a test module)."""
import numpy as np
import torch

import oracle
from linear_rnn_recurrent_amd import ssu_decode, ssu_prefill, ssu_replay, ssu_tree_verify

# Tolerances: max|got - ref| <= tol * (1 + |ref|), elementwise.
TOL_F32 = 2e-5      # fp32 state and fp32 outputs
TOL_LOW = 1e-2      # fp16/bf16 state, fp16/bf16 outputs


def tol_for(dtype):
    return TOL_F32 if dtype == torch.float32 else TOL_LOW


def f64(t):
    if t is None:
        return None
    if t.is_floating_point():
        return t.detach().cpu().double().numpy()
    return t.detach().cpu().numpy()


def gpu(t):
    return None if t is None else t.cuda()


def assert_close(got, ref, tol, what, scale=None):
    """max|got - ref| <= tol * (1 + scale) elementwise; scale defaults to |ref|
    (a caller may pass the magnitude of each value's terms instead, which bounds
    the rounding of a sum whose terms cancel)."""
    got = f64(got) if isinstance(got, torch.Tensor) else got
    err = np.abs(got - ref)
    bound = tol * (1.0 + (np.abs(ref) if scale is None else scale))
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err / bound, 0)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements outside "
                             f"{tol}*(1+|ref|); worst at {i}: got {got[i]!r} ref {ref[i]!r}")


def assert_bitwise(a, b, what):
    a = a.detach().cpu()
    b = b.detach().cpu()
    assert a.dtype == b.dtype and a.shape == b.shape, what
    va = a.contiguous().view(torch.uint8) if a.element_size() > 0 else a
    vb = b.contiguous().view(torch.uint8)
    if not torch.equal(va, vb):
        raise AssertionError(f"{what}: not bitwise identical")


def misaligned(t):
    """The values of a 16-bit tensor on the GPU, 2 bytes past a 16-byte boundary.

    The matrix-core prefill reads x with 16-byte vector loads and is chosen only
    for 16-byte aligned x; this routes a 16-bit prefill to the VALU kernel."""
    assert t.element_size() == 2
    buf = torch.empty(t.numel() + 8, dtype=t.dtype, device="cuda")
    v = buf[1:1 + t.numel()].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 == 2
    return v


def run_decode(w, state=None, out=None, **over):
    T = {k: gpu(v) for k, v in w.tensors.items()}
    T.update(over)
    st = T["state"] if state is None else state
    if out is None:
        out = torch.full_like(T["x"], float("nan"))
    ssu_decode(T["x"], T["A"], T["B"], T["C"], T["dt"], st, out, dt_bias=T["dt_bias"],
               D=T["D"], z=T["z"], dt_softplus=w.dt_softplus, state_indices=T["state_indices"])
    return st, out


def oracle_decode(w, **over):
    a = {k: f64(v) for k, v in w.tensors.items()}
    a.update(over)
    st = a["state"].copy()
    out = np.zeros(a["x"].shape)
    oracle.decode(a["x"], a["A"], a["B"], a["C"], a["dt"], st, out, dt_bias=a["dt_bias"],
                  D=a["D"], z=a["z"], dt_softplus=w.dt_softplus,
                  state_indices=a["state_indices"])
    return st, out


def run_prefill(w, stash=False, **over):
    T = {k: gpu(v) for k, v in w.tensors.items()}
    T.update(over)
    out = torch.full_like(T["x"], float("nan"))
    st = T["state"]
    S = {}
    if stash:
        b, t, h, d = T["x"].shape
        S = {"replay_dA": torch.full((b, t, h), float("nan"), device="cuda"),
             "replay_dt": torch.full((b, t, h), float("nan"), device="cuda"),
             "replay_u": torch.full((b, t, h, d), float("nan"), device="cuda"),
             "replay_B": torch.full(tuple(T["B"].shape), float("nan"), device="cuda")}
    ssu_prefill(T["x"], T["A"], T["B"], T["C"], T["dt"], st, out, dt_bias=T["dt_bias"],
                D=T["D"], z=T["z"], dt_softplus=w.dt_softplus,
                context_lengths=T["context_lengths"], state_indices=T["state_indices"], **S)
    return st, out, S


def oracle_prefill(w, stash=False, **over):
    a = {k: f64(v) for k, v in w.tensors.items()}
    a.update(over)
    st = a["state"].copy()
    out = np.zeros(a["x"].shape)
    S = None
    if stash:
        b, t, h, d = a["x"].shape
        S = {"dA": np.full((b, t, h), np.nan), "dt": np.full((b, t, h), np.nan),
             "u": np.full((b, t, h, d), np.nan), "B": np.full(a["B"].shape, np.nan)}
    oracle.prefill(a["x"], a["A"], a["B"], a["C"], a["dt"], st, out, dt_bias=a["dt_bias"],
                   D=a["D"], z=a["z"], dt_softplus=w.dt_softplus,
                   context_lengths=a["context_lengths"], state_indices=a["state_indices"],
                   stash=S)
    return st, out, S


def oracle_prefill_magnitude(w):
    """The oracle's prefill of |state|, |x|, |B|, |C|, |D| and |z| with the same
    decays and dt': every state entry and output as the sum of the magnitudes of
    its terms (silu(|z|) >= |silu(z)|), the scale of fp32 rounding in any order
    of evaluation where the terms cancel."""
    a = {k: f64(v) for k, v in w.tensors.items()}
    for k in ("state", "x", "B", "C", "D", "z"):
        if a.get(k) is not None:
            a[k] = np.abs(a[k])
    st = a["state"].copy()
    out = np.zeros(a["x"].shape)
    oracle.prefill(a["x"], a["A"], a["B"], a["C"], a["dt"], st, out, dt_bias=a["dt_bias"],
                   D=a["D"], z=a["z"], dt_softplus=w.dt_softplus,
                   context_lengths=a["context_lengths"], state_indices=a["state_indices"])
    return st, out


def run_replay(w, **over):
    T = {k: gpu(v) for k, v in w.tensors.items()}
    T.update(over)
    ssu_replay(T["state"], T["replay_dA"], T["replay_u"], T["replay_B"], T["replay_dt"],
               T["accepted_lengths"], state_indices=T["state_indices"],
               active_batch=w.active_batch, accepted_node_ids=T.get("node_ids"))
    return T["state"]


def oracle_replay(w, **over):
    a = {k: f64(v) for k, v in w.tensors.items()}
    a.update(over)
    st = a["state"].copy()
    oracle.replay(st, a["replay_dA"], a["replay_u"], a["replay_B"], a["replay_dt"],
                  a["accepted_lengths"], state_indices=a["state_indices"],
                  active_batch=w.active_batch, node_ids=a.get("node_ids"))
    return st


def _nan_stash(b, m, h, d, bshape, device):
    return {"replay_dA": torch.full((b, m, h), float("nan"), device=device),
            "replay_dt": torch.full((b, m, h), float("nan"), device=device),
            "replay_u": torch.full((b, m, h, d), float("nan"), device=device),
            "replay_B": torch.full(tuple(bshape), float("nan"), device=device)}


def run_tree(w, stash=False, **over):
    T = {k: gpu(v) for k, v in w.tensors.items()}
    T.update(over)
    out = torch.full_like(T["x"], float("nan"))
    b, m, h, d = T["x"].shape
    S = _nan_stash(b, m, h, d, T["B"].shape, "cuda") if stash else {}
    ssu_tree_verify(T["x"], T["A"], T["B"], T["C"], T["dt"], T["state"], out, T["parent_ids"],
                    depths=T["depths"], dt_bias=T["dt_bias"], D=T["D"], z=T["z"],
                    dt_softplus=w.dt_softplus, state_indices=T["state_indices"], **S)
    return T["state"], out, S


def oracle_tree(w, stash=False, **over):
    a = {k: f64(v) for k, v in w.tensors.items()}
    a.update(over)
    out = np.zeros(a["x"].shape)
    S = None
    if stash:
        b, m, h, d = a["x"].shape
        S = {"dA": np.full((b, m, h), np.nan), "dt": np.full((b, m, h), np.nan),
             "u": np.full((b, m, h, d), np.nan), "B": np.full(a["B"].shape, np.nan)}
    oracle.tree(a["x"], a["A"], a["B"], a["C"], a["dt"], a["state"], out, a["parent_ids"],
                depths=a["depths"], dt_bias=a["dt_bias"], D=a["D"], z=a["z"],
                dt_softplus=w.dt_softplus, state_indices=a["state_indices"], stash=S)
    return out, S


def touched_rows(idx, n_rows):
    if idx is None:
        return np.arange(n_rows)
    idx = f64(idx)
    return np.unique(idx[idx >= 0])


def untouched_rows(idx, pool_rows, batch):
    rows = np.ones(pool_rows, dtype=bool)
    rows[touched_rows(idx, batch)] = False
    return np.nonzero(rows)[0]
