"""Seeded synthetic inputs for the selective state update.

This module only draws random numbers and casts them to storage dtypes; it
holds none of the update's arithmetic.  Both the HIP path (through the tests
and the benchmark) and the fp64 oracle consume exactly the tensors it returns:
the oracle sees them upcast to float64, which is exact for fp32/fp16/bf16.

Value recipe (per head h, per batch row b, per token t):
  A[h]       = -exp(U(ln 1, ln 16))                     fp32
  dt_bias[h] = log(expm1(U(1e-3, 0.1)))                 fp32  (softplus^-1 of U)
  dt         ~ N(0, std 0.5)                            fp32
  D[h]       ~ N(0, 1)                                  fp32
  x, z       ~ N(0, 1)                                  io dtype
  B, C       ~ N(0, std bc_std)                         bc dtype
  state      ~ N(0, 1) or zeros                         state dtype
Replay stash (the stash a verify prefill would have written):
  DT         = exp(U(ln 4e-4, ln 0.33))                 fp32  (range of dt' above)
  dA         = A[h] * DT, rounded once to fp32          fp32  (log-decay)
  u          ~ N(0, 1), replayB ~ N(0, std 1/sqrt(dstate))
Values are drawn in float64 (float32 for the large state pools), rounded to
fp32, then cast on the CPU by torch (round to nearest even) to bf16/fp16.
Draft trees (one per batch row, nodes in topological order, node 0 a root):
  'random': node n > 0 hangs under a uniformly drawn earlier node whose depth
            is below max_depth - 1 (a random recursive tree, depth ~ ln n);
  'chain' : parent n - 1 (a linear draft); 'star': every node a root.
  depths  : the exact hop count of every node, unless a test overrides it.
"""
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class Workload:
    """One batch of inputs.  `kind` is 'decode', 'prefill', 'replay' or 'tree'."""
    name: str
    kind: str
    dims: Dict[str, int]
    tensors: Dict[str, Optional[torch.Tensor]]
    dt_softplus: bool = True
    active_batch: Optional[int] = None
    notes: Dict[str, str] = field(default_factory=dict)

    def __getitem__(self, k):
        return self.tensors[k]


def _t(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DTYPES[dtype])


def _head_params(rng, nheads):
    A = -np.exp(rng.uniform(np.log(1.0), np.log(16.0), nheads))
    dt_bias = np.log(np.expm1(rng.uniform(1e-3, 0.1, nheads)))
    D = rng.standard_normal(nheads)
    return A, dt_bias, D


def _pool(rng, shape, dtype, zero=False):
    if zero:
        return torch.zeros(shape, dtype=DTYPES[dtype])
    a = rng.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    return torch.from_numpy(a).to(DTYPES[dtype])


def decode_workload(*, batch, nheads, dim, dstate, ngroups, pool_rows, seed,
                    state_dtype="f32", io_dtype="bf16", bc_dtype="bf16",
                    bc_std=None, indices="perm", n_live=None, with_z=True,
                    with_D=True, with_bias=True, dt_softplus=True,
                    zero_state=False, name="decode"):
    """indices: 'perm' (unique rows of the pool), 'none' (row = b), or an int list.
    n_live: keep the first n_live indices, pad the rest with -1."""
    rng = np.random.default_rng(seed)
    if bc_std is None:
        bc_std = 1.0
    A, dt_bias, D = _head_params(rng, nheads)
    state = _pool(rng, (pool_rows, nheads, dim, dstate), state_dtype, zero_state)
    x = rng.standard_normal((batch, nheads, dim))
    z = rng.standard_normal((batch, nheads, dim))
    Bm = rng.standard_normal((batch, ngroups, dstate)) * bc_std
    Cm = rng.standard_normal((batch, ngroups, dstate)) * bc_std
    dt = rng.standard_normal((batch, nheads)) * 0.5
    if isinstance(indices, str) and indices == "perm":
        idx = rng.permutation(pool_rows)[:batch].astype(np.int32)
    elif isinstance(indices, str) and indices == "none":
        idx = None
    else:
        idx = np.asarray(indices, dtype=np.int32)
    if idx is not None and n_live is not None:
        idx = idx.copy()
        idx[n_live:] = -1
    T = {
        "x": _t(x, io_dtype), "z": _t(z, io_dtype) if with_z else None,
        "B": _t(Bm, bc_dtype), "C": _t(Cm, bc_dtype), "dt": _t(dt, "f32"),
        "A": _t(A, "f32"), "dt_bias": _t(dt_bias, "f32") if with_bias else None,
        "D": _t(D, "f32") if with_D else None, "state": state,
        "state_indices": None if idx is None else torch.from_numpy(idx),
    }
    dims = dict(batch=batch, nheads=nheads, dim=dim, dstate=dstate, ngroups=ngroups,
                pool_rows=pool_rows, seq_len=1)
    return Workload(name, "decode", dims, T, dt_softplus)


def prefill_workload(*, batch, seq_len, nheads, dim, dstate, ngroups, pool_rows, seed,
                     state_dtype="f32", io_dtype="bf16", bc_dtype="bf16", bc_std=None,
                     ctx=("uniform", 1, None), indices="perm", n_live=None,
                     with_z=True, with_D=True, with_bias=True, dt_softplus=True,
                     zero_state=False, name="prefill"):
    """ctx: ('uniform', lo, hi) inclusive (hi None -> seq_len), ('none',), or a list."""
    rng = np.random.default_rng(seed)
    if bc_std is None:
        bc_std = 1.0
    A, dt_bias, D = _head_params(rng, nheads)
    state = _pool(rng, (pool_rows, nheads, dim, dstate), state_dtype, zero_state)
    x = rng.standard_normal((batch, seq_len, nheads, dim))
    z = rng.standard_normal((batch, seq_len, nheads, dim))
    Bm = rng.standard_normal((batch, seq_len, ngroups, dstate)) * bc_std
    Cm = rng.standard_normal((batch, seq_len, ngroups, dstate)) * bc_std
    dt = rng.standard_normal((batch, seq_len, nheads)) * 0.5
    if ctx[0] == "uniform":
        hi = seq_len if ctx[2] is None else ctx[2]
        cl = rng.integers(ctx[1], hi + 1, batch).astype(np.int32)
    elif ctx[0] == "none":
        cl = None
    else:
        cl = np.asarray(ctx, dtype=np.int32)
    if isinstance(indices, str) and indices == "perm":
        idx = rng.permutation(pool_rows)[:batch].astype(np.int32)
    elif isinstance(indices, str) and indices == "none":
        idx = None
    else:
        idx = np.asarray(indices, dtype=np.int32)
    if idx is not None and n_live is not None:
        idx = idx.copy()
        idx[n_live:] = -1
    T = {
        "x": _t(x, io_dtype), "z": _t(z, io_dtype) if with_z else None,
        "B": _t(Bm, bc_dtype), "C": _t(Cm, bc_dtype), "dt": _t(dt, "f32"),
        "A": _t(A, "f32"), "dt_bias": _t(dt_bias, "f32") if with_bias else None,
        "D": _t(D, "f32") if with_D else None, "state": state,
        "context_lengths": None if cl is None else torch.from_numpy(cl),
        "state_indices": None if idx is None else torch.from_numpy(idx),
    }
    dims = dict(batch=batch, nheads=nheads, dim=dim, dstate=dstate, ngroups=ngroups,
                pool_rows=pool_rows, seq_len=seq_len)
    return Workload(name, "prefill", dims, T, dt_softplus)


def replay_workload(*, active_batch, seq_len, nheads, dim, dstate, ngroups, pool_rows,
                    seed, state_dtype="f32", accepted=("uniform", 0, None),
                    indices="perm", n_live=None, stash_batch=None, name="replay"):
    """stash_batch: leading extent of the stash and accepted arrays (>= active_batch);
    entries at or beyond active_batch are filled with poison values."""
    rng = np.random.default_rng(seed)
    nb = active_batch if stash_batch is None else stash_batch
    A, _, _ = _head_params(rng, nheads)
    state = _pool(rng, (pool_rows, nheads, dim, dstate), state_dtype)
    DT = np.exp(rng.uniform(np.log(4e-4), np.log(0.33), (nb, seq_len, nheads))).astype(np.float32)
    dA = (A.astype(np.float32)[None, None, :] * DT).astype(np.float32)
    u = rng.standard_normal((nb, seq_len, nheads, dim))
    Bst = rng.standard_normal((nb, seq_len, ngroups, dstate)) / np.sqrt(dstate)
    if accepted[0] == "uniform":
        hi = seq_len if accepted[2] is None else accepted[2]
        acc = rng.integers(accepted[1], hi + 1, nb).astype(np.int32)
    else:
        acc = np.asarray(accepted, dtype=np.int32)
    if nb > active_batch:
        acc[active_batch:] = 1 << 30   # poison: must never be read
    if isinstance(indices, str) and indices == "perm":
        idx = rng.permutation(pool_rows)[:nb].astype(np.int32)
    elif isinstance(indices, str) and indices == "none":
        idx = None
    else:
        idx = np.asarray(indices, dtype=np.int32)
    if idx is not None and n_live is not None:
        idx = idx.copy()
        idx[n_live:] = -1
    T = {
        "state": state, "replay_dA": _t(dA, "f32"), "replay_u": _t(u, "f32"),
        "replay_B": _t(Bst, "f32"), "replay_dt": _t(DT, "f32"),
        "accepted_lengths": torch.from_numpy(acc),
        "state_indices": None if idx is None else torch.from_numpy(idx),
        "A": _t(A, "f32"),
    }
    dims = dict(batch=active_batch, nheads=nheads, dim=dim, dstate=dstate, ngroups=ngroups,
                pool_rows=pool_rows, seq_len=seq_len)
    return Workload(name, "replay", dims, T, False, active_batch=active_batch)


def random_tree(rng, num_nodes, shape="random", max_depth=None):
    """Parent ids and depths (hops to the root) of one draft tree."""
    parents = np.full(num_nodes, -1, dtype=np.int32)
    depth = np.zeros(num_nodes, dtype=np.int32)
    for n in range(1, num_nodes):
        if shape == "star":
            continue
        if shape == "chain":
            p = n - 1
        else:
            ok = np.arange(n) if max_depth is None else np.nonzero(depth[:n] < max_depth - 1)[0]
            p = int(ok[rng.integers(ok.size)])
        parents[n] = p
        depth[n] = depth[p] + 1
    return parents, depth


def tree_workload(*, batch, num_nodes, nheads, dim, dstate, ngroups, pool_rows, seed,
                  state_dtype="f32", io_dtype="bf16", bc_dtype="bf16", bc_std=None,
                  shape="random", max_depth=None, indices="perm", n_live=None,
                  with_z=False, with_D=True, with_bias=True, dt_softplus=True,
                  with_depths=True, name="tree"):
    """Tree-verify inputs: per-node tensors in the prefill layouts (the node axis
    in place of the token axis) and int32 parent_ids / depths [batch, num_nodes].
    shape: 'random', 'chain', 'star' or a [batch, num_nodes] parent-id array."""
    rng = np.random.default_rng(seed)
    if bc_std is None:
        bc_std = 1.0
    A, dt_bias, D = _head_params(rng, nheads)
    state = _pool(rng, (pool_rows, nheads, dim, dstate), state_dtype)
    x = rng.standard_normal((batch, num_nodes, nheads, dim))
    z = rng.standard_normal((batch, num_nodes, nheads, dim))
    Bm = rng.standard_normal((batch, num_nodes, ngroups, dstate)) * bc_std
    Cm = rng.standard_normal((batch, num_nodes, ngroups, dstate)) * bc_std
    dt = rng.standard_normal((batch, num_nodes, nheads)) * 0.5
    if isinstance(shape, str):
        trees = [random_tree(rng, num_nodes, shape, max_depth) for _ in range(batch)]
        par = np.stack([t[0] for t in trees]) if batch else np.zeros((0, num_nodes), np.int32)
        dep = np.stack([t[1] for t in trees]) if batch else np.zeros((0, num_nodes), np.int32)
    else:
        par = np.asarray(shape, dtype=np.int32).reshape(batch, num_nodes)
        dep = np.zeros_like(par)
        for b in range(batch):
            for n in range(num_nodes):
                p = par[b, n]
                dep[b, n] = dep[b, p] + 1 if 0 <= p < n else 0
    if isinstance(indices, str) and indices == "perm":
        idx = rng.permutation(pool_rows)[:batch].astype(np.int32)
    elif isinstance(indices, str) and indices == "none":
        idx = None
    else:
        idx = np.asarray(indices, dtype=np.int32)
    if idx is not None and n_live is not None:
        idx = idx.copy()
        idx[n_live:] = -1
    T = {
        "x": _t(x, io_dtype), "z": _t(z, io_dtype) if with_z else None,
        "B": _t(Bm, bc_dtype), "C": _t(Cm, bc_dtype), "dt": _t(dt, "f32"),
        "A": _t(A, "f32"), "dt_bias": _t(dt_bias, "f32") if with_bias else None,
        "D": _t(D, "f32") if with_D else None, "state": state,
        "state_indices": None if idx is None else torch.from_numpy(idx),
        "parent_ids": torch.from_numpy(np.ascontiguousarray(par)),
        "depths": torch.from_numpy(np.ascontiguousarray(dep)) if with_depths else None,
    }
    dims = dict(batch=batch, nheads=nheads, dim=dim, dstate=dstate, ngroups=ngroups,
                pool_rows=pool_rows, seq_len=num_nodes, num_nodes=num_nodes)
    return Workload(name, "tree", dims, T, dt_softplus)


# ---------------------------------------------------------------------------
# The five benchmark configurations.
# ---------------------------------------------------------------------------
CONFIG_NAMES = {
    0: "tiny decode B2 H4 Dm16 N16 G1, fp32 pool P4",
    1: "Mamba2-2.7B-shaped decode B64 H80 Dm64 N128 G1, fp32 pool P256",
    2: "prefill B8 T512 H80 Dm64 N128 G1, ctx~U[64,512], fp32 pool P64 (zeros)",
    3: "padded decode B128 (97 live) H64 Dm64 N128 G8, fp16 pool P160",
    4: "MTP replay active32/48 T4 H80 Dm64 N128 G1, fp32 pool P48",
}


def config(i: int, seed: Optional[int] = None) -> Workload:
    s = i if seed is None else seed
    if i == 0:
        return decode_workload(batch=2, nheads=4, dim=16, dstate=16, ngroups=1, pool_rows=4,
                               seed=s, state_dtype="f32", io_dtype="f32", bc_dtype="f32",
                               bc_std=1.0, indices=[2, 0], name=CONFIG_NAMES[0])
    if i == 1:
        return decode_workload(batch=64, nheads=80, dim=64, dstate=128, ngroups=1,
                               pool_rows=256, seed=s, state_dtype="f32", io_dtype="bf16",
                               bc_dtype="bf16", bc_std=1.0 / np.sqrt(128), name=CONFIG_NAMES[1])
    if i == 2:
        return prefill_workload(batch=8, seq_len=512, nheads=80, dim=64, dstate=128,
                                ngroups=1, pool_rows=64, seed=s, state_dtype="f32",
                                io_dtype="bf16", bc_dtype="bf16", bc_std=1.0 / np.sqrt(128),
                                ctx=("uniform", 64, 512), zero_state=True,
                                name=CONFIG_NAMES[2])
    if i == 3:
        return decode_workload(batch=128, nheads=64, dim=64, dstate=128, ngroups=8,
                               pool_rows=160, seed=s, state_dtype="f16", io_dtype="bf16",
                               bc_dtype="bf16", bc_std=1.0 / np.sqrt(128), n_live=97,
                               name=CONFIG_NAMES[3])
    if i == 4:
        return replay_workload(active_batch=32, seq_len=4, nheads=80, dim=64, dstate=128,
                               ngroups=1, pool_rows=48, seed=s, state_dtype="f32",
                               accepted=("uniform", 0, 4), name=CONFIG_NAMES[4])
    raise ValueError(f"no configuration {i}")


# A Mamba2-2.7B-shaped layer stack for the layer-batched calls: 64 layers, and a
# conv-state row of (d_inner + 2 ngroups dstate) channels x (d_conv - 1) taps in bf16.
STACK_LAYERS = 64
STACK_CONV_ROW_BYTES = (5120 + 2 * 128) * 3 * 2
LAYERS_NAME = {
    6: "MTP replay of the config-4 batch (active32/48 T4 H80 Dm64 N128 G1, fp32) on each of "
       "64 layers, one launch",
    7: "clear of one resident slot of 64 layers (fp32 recurrent rows H80 Dm64 N128 + bf16 conv "
       "rows 5376 x 3), one launch",
}

def gdn_workload(*, batch, hidden, num_q_heads, num_v_heads, head_dim, conv_width, pool_rows,
                 seed, indices="perm", n_live=None, conv_layout="ds", use_qk_l2norm=True,
                 scale=None, ssm_std=0.1, name="gdn"):
    """Inputs of the fused gated-delta-rule decode step (bf16 activations and
    conv pool, fp32 A_log and ssm pool). conv_layout 'ds': conv_state is the
    dense [P, qkv_dim, W-1] pool; 'sd': the pool holds [P, W-1, qkv_dim] rows and
    conv_state is its transposed view."""
    rng = np.random.default_rng(seed)
    hq, hv, d, w = num_q_heads, num_v_heads, head_dim, conv_width
    qkv = (2 * hq + hv) * d
    bf = lambda a: _t(a, "bf16")
    hs = rng.standard_normal((batch, hidden))
    w_ba = rng.standard_normal((hidden, 2 * hv)) / np.sqrt(hidden)
    mixed = rng.standard_normal((batch, qkv))
    conv_w = rng.standard_normal((qkv, w)) / np.sqrt(w)
    conv_b = rng.standard_normal(qkv) * 0.1
    A_log = np.log(rng.uniform(1.0, 16.0, hv))
    dt_bias = np.log(np.expm1(rng.uniform(1e-3, 0.1, hv)))
    if conv_layout == "ds":
        conv_state = bf(rng.standard_normal((pool_rows, qkv, w - 1)))
    else:
        conv_state = bf(rng.standard_normal((pool_rows, w - 1, qkv))).transpose(1, 2)
    ssm = torch.from_numpy((rng.standard_normal((pool_rows, hv, d, d)) * ssm_std).astype(np.float32))
    if isinstance(indices, str) and indices == "perm":
        idx = rng.permutation(pool_rows)[:batch].astype(np.int32)
    else:
        idx = np.asarray(indices, dtype=np.int32)
    if n_live is not None:
        idx = idx.copy()
        idx[n_live:] = -1
    T = {"hidden_states": bf(hs), "w_ba": bf(w_ba), "mixed_qkv": bf(mixed), "conv_weight": bf(conv_w),
         "conv_bias": bf(conv_b), "conv_state": conv_state, "A_log": _t(A_log, "f32"),
         "dt_bias": bf(dt_bias), "ssm_state": ssm, "state_indices": torch.from_numpy(idx)}
    dims = dict(batch=batch, hidden=hidden, num_q_heads=hq, num_v_heads=hv, head_dim=d,
                conv_width=w, pool_rows=pool_rows, use_qk_l2norm=use_qk_l2norm, scale=scale)
    return Workload(name, "gdn", dims, T, True)


GDN_NAME = ("GDN fused decode B64 hidden2048 Hq16 HV32 D128 W4 (Qwen3-Next-shaped linear "
            "attention layer), fp32 ssm pool P256, bf16 conv pool")


def gdn_config(seed: int = 9) -> Workload:
    """Fused gated-delta-rule decode at a Qwen3-Next-shaped linear-attention layer."""
    return gdn_workload(batch=64, hidden=2048, num_q_heads=16, num_v_heads=32, head_dim=128,
                        conv_width=4, pool_rows=256, seed=seed, name=GDN_NAME)


GATHER_NAME = ("gather of the config-1 batch: 64 rows of H80 Dm64 N128 fp32 (2.6 MB each) from "
               "the 256-row pool into a contiguous active batch")

TREE_NAME = ("tree verify B16 M128 (random draft tree, depth < 16) H80 Dm64 N128 G1, "
             "fp32 pool P64")


def tree_config(seed: int = 5, num_nodes: int = 128) -> Workload:
    """Tree-verify workload: 16 requests, each with a random draft tree of the
    full 128-node verify budget, on the decode model shape (H80 Dm64 N128 G1)."""
    return tree_workload(batch=16, num_nodes=num_nodes, nheads=80, dim=64, dstate=128,
                         ngroups=1, pool_rows=64, seed=seed, state_dtype="f32",
                         io_dtype="bf16", bc_dtype="bf16", bc_std=1.0 / np.sqrt(128),
                         shape="random", max_depth=16, with_z=False, name=TREE_NAME)


def rotation_index_sets(pool_rows: int, batch: int, seed: int):
    """Disjoint index sets that together cover the whole pool (one per step)."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(pool_rows).astype(np.int32)
    return [torch.from_numpy(perm[i:i + batch].copy())
            for i in range(0, pool_rows - batch + 1, batch)]
