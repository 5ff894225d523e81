#!/usr/bin/env python3
"""Throughput of the selective state update on one MI355X.

Default workload: decode of the Mamba2-2.7B-shaped batch (B=64, H=80, dim=64,
dstate=128, G=1, fp32 state, bf16 x/z/B/C/out) over a 256-row fp32 pool
(671 MB). One step is one ssu_decode launch over 64 rows; consecutive steps use
four disjoint 64-row index sets that together cover the pool, so every step
streams state rows the previous three steps did not touch and the 256 MB
last-level cache cannot serve them.

    python bench.py [--steps K] [--warmup W] [--config {1,2,3,4,5,6,7,8,9}]

--config 2/3/4/5 time prefill / padded decode / MTP replay / tree verify
(prefill: --operands f16 or f32 for fp16 or fp32 x/z/B/C instead of bf16,
--stash with the replay stash)
(16 requests with 128-node draft trees, replay stash on) instead; 6 and 7 the
layer-batched calls over a 64-layer stack: the MTP replay of config 4 for every
layer in one launch, and the clear of one resident slot (recurrent and conv
rows) of every layer in one launch; 8 the gather of the config-1 batch's 64 pool
rows into a contiguous active batch; 9 the fused gated-delta-rule decode step
of a Qwen3-Next-shaped linear-attention layer (B=64, hidden 2048, Hq 16, HV 32,
D 128, conv width 4) over a 256-slot pool, steps rotating disjoint 64-slot
index sets as in the default. The other pools
are smaller than the last-level cache, so the steps rotate over replicas of
the pool (and, for prefill, of every input) that together exceed it; every
configuration is timed as back-to-back launches on one stream.

The K timed steps are captured once as a HIP graph and replayed (--no-graph
launches them one by one from Python instead, which leaves gaps for kernels
shorter than the binding's per-call host time).

Prints one JSON line: value = algorithmic GB/s (bytes the method must move,
each element counted once, divided by the average launch time measured with
HIP events on the launch stream), plus token*head updates/s, the roofline
object of the timed kernel (HBM for every configuration; prefill and tree
verify also report their rate on the bf16 matrix cores they run on), the
flushed protocol (--flushed launches timed one by one, each after a 1 GiB
scratch write that evicts the last-level cache: median, p10, p90) with a
device-to-device copy rate as context, and the fp64 oracle's throughput on
the host (cpu_baseline: all threads and one thread, CPU model; a reported
baseline, not a target).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak (the instruction the
                                 # prefill and tree kernels issue)
MFMA_F32_PEAK_TFLOPS = 157.3     # dense fp32 matrix-core peak (context only)
FLUSH_BYTES = 1 << 30            # scratch written before each individually timed launch


def metric_name():
    return "state-update GB/s and % of HBM peak; token·head updates/s (B=64 decode)"


def esize(t):
    return t.element_size()


def decode_bytes(T, live):
    """Algorithmic bytes of one decode launch (element counted once; B/C per group)."""
    b, h, d = T["x"].shape
    g, n = T["B"].shape[1], T["B"].shape[2]
    s_s, s_x = esize(T["state"]), esize(T["x"])
    s_z = esize(T["z"]) if T["z"] is not None else 0
    per_live = h * d * n * 2 * s_s + h * d * (s_x + s_z) + 2 * g * n * esize(T["B"]) + 4 * h
    return live * per_live + b * h * d * s_x + 12 * h + 4 * b


def prefill_bytes(T, L, stash=False):
    """Algorithmic bytes of one prefill launch. With the replay stash the state is
    only read, and the fp32 stash (A dt', dt', x, B) is written for every token
    position (zero past the context)."""
    b, t, h, d = T["x"].shape
    g, n = T["B"].shape[2], T["B"].shape[3]
    s_s, s_x = esize(T["state"]), esize(T["x"])
    per_tok = h * d * (2 * s_x + (s_x if T["z"] is not None else 0)) + 2 * g * n * esize(T["B"]) + 4 * h
    total = 0
    for Lb in L:
        total += h * d * n * (1 if stash else 2) * s_s + int(Lb) * per_tok
        total += (t - int(Lb)) * h * d * s_x
        if stash:
            total += t * (8 * h + 4 * h * d + 4 * g * n)
    return total + 12 * h + 8 * b


def replay_bytes(T, k_rows):
    h = T["replay_dA"].shape[2]
    d = T["replay_u"].shape[3]
    g, n = T["replay_B"].shape[2], T["replay_B"].shape[3]
    s_s = esize(T["state"])
    total = 0
    for k in k_rows:
        if k > 0:
            total += h * d * n * 2 * s_s + k * (4 * h * d + 4 * g * n + 8 * h)
    return total + 8 * len(k_rows)


def tree_bytes(T, stash=True):
    """Algorithmic bytes of one tree-verify launch: committed state of every live
    row, every node's x, B, C, dt, parent id, depth and output, and the stash."""
    b, m, h, d = T["x"].shape
    g, n = T["B"].shape[2], T["B"].shape[3]
    live = int((T["state_indices"] >= 0).sum().item()) if T["state_indices"] is not None else b
    s_x = esize(T["x"])
    per_node = h * d * 2 * s_x + (h * d * s_x if T["z"] is not None else 0) \
        + 2 * g * n * esize(T["B"]) + 4 * h + 8
    st = 4 * h * d + 4 * g * n + 8 * h if stash else 0
    return live * h * d * n * esize(T["state"]) + b * m * per_node + live * m * st + 12 * h


def gdn_bytes(T, live):
    """Algorithmic bytes of one fused gated-delta-rule decode launch: weights once,
    per live entry its activations, conv-pool taps (read and written) and the
    HV x D x D fp32 state (read and written); out for every entry."""
    B, hidden = T["hidden_states"].shape
    qkv, w = T["conv_weight"].shape
    P, hv, d, _ = T["ssm_state"].shape
    e = esize(T["hidden_states"])
    once = (T["w_ba"].numel() + T["conv_weight"].numel() + qkv) * e + hv * (4 + e)
    per = (hidden + qkv) * e + 2 * qkv * (w - 1) * e + 2 * hv * d * d * 4
    return once + live * per + B * (4 + hv * d * e)


def prefill_mm_fmas(T, L, chunk=32):
    """FMAs of the chunked closed form the bf16 prefill evaluates: per token and
    head S . C and the state update (dim x dstate each); per chunk the in-chunk
    B . C dots (per group) and Q . X terms (per head) over token pairs j <= t."""
    b, t, h, d = T["x"].shape
    g, n = T["B"].shape[2], T["B"].shape[3]
    idx = T["state_indices"].cpu().tolist() if T["state_indices"] is not None else list(range(b))
    f = 0
    for r, Lb in enumerate(L):
        if idx[r] < 0:
            continue
        for t0 in range(0, int(Lb), chunk):
            nv = min(chunk, int(Lb) - t0)
            pairs = nv * (nv + 1) // 2
            f += h * (2 * nv * d * n + pairs * d) + g * pairs * n
    return f


def prefill_method_flops(T, L):
    """Flops of the method itself, 5 per state element and token (decay multiply,
    the B dt' x FMA and the C dot FMA), over the live rows' tokens."""
    b, t, h, d = T["x"].shape
    n = T["B"].shape[3]
    idx = T["state_indices"].cpu().tolist() if T["state_indices"] is not None else list(range(b))
    return 5 * h * d * n * sum(int(Lb) for r, Lb in enumerate(L) if idx[r] >= 0)


def tree_lane_ops(T):
    """FMAs of the closed form the tree kernel evaluates: S0 . C per (node, row)
    plus, per path entry, one dstate-long B . C dot and one x term per row."""
    import numpy as np
    b, m, h, d = T["x"].shape
    n = T["B"].shape[3]
    par = T["parent_ids"].cpu().numpy()
    dep = T["depths"].cpu().numpy() if T["depths"] is not None else None
    idx = T["state_indices"].cpu().numpy() if T["state_indices"] is not None else np.arange(b)
    ops = 0
    for r in range(b):
        if idx[r] < 0:
            continue
        entries = 0
        for node in range(m):
            cap = node if dep is None else int(dep[r, node])
            j, hops = node, 0
            while hops < cap and 0 <= par[r, j] < j:
                j, hops = int(par[r, j]), hops + 1
            entries += hops + 1
        ops += h * (m * d * n + entries * (n + d))
    return ops


def source_hash(*names):
    hsh = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "linear_rnn_recurrent_amd", "csrc", n), "rb") as f:
            hsh.update(f.read())
    return hsh.hexdigest()[:16]


def measured_traffic(kernel_key, src_hash):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(kind, w, seconds, bytes_per_call, units_per_call, stash=False):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload."""
    import numpy as np
    import oracle

    from linear_rnn_recurrent_amd import inputs as inputs_mod
    a = {k: (None if v is None else (v.double().numpy() if v.is_floating_point() else v.numpy()))
         for k, v in w.tensors.items()}
    scale = 1.0   # fraction of one step's work a call does
    if kind == "decode":
        idx = a["state_indices"]
        live = idx[idx >= 0]
        st = a["state"][live].copy()                # compact pool of the addressed rows
        remap = np.full(idx.shape, -1, dtype=np.int32)
        remap[idx >= 0] = np.arange(live.size, dtype=np.int32)
        out = np.zeros(a["x"].shape)

        def call():
            oracle.decode(a["x"], a["A"], a["B"], a["C"], a["dt"], st, out, dt_bias=a["dt_bias"],
                          D=a["D"], z=a["z"], dt_softplus=w.dt_softplus, state_indices=remap)
        sample = f"the full {a['x'].shape[0]}-row batch of this workload"
    elif kind == "prefill":
        st = a["state"].copy()
        out = np.zeros(a["x"].shape)
        b, t, h, d = a["x"].shape
        S = ({"dA": np.zeros((b, t, h)), "dt": np.zeros((b, t, h)), "u": np.zeros((b, t, h, d)),
              "B": np.zeros(a["B"].shape)} if stash else None)

        def call():
            oracle.prefill(a["x"], a["A"], a["B"], a["C"], a["dt"], st, out, dt_bias=a["dt_bias"],
                           D=a["D"], z=a["z"], dt_softplus=w.dt_softplus,
                           context_lengths=a["context_lengths"], state_indices=a["state_indices"],
                           stash=S)
        sample = "the full prefill batch of this workload" + (", replay stash on" if stash else "")
    elif kind == "tree":
        out = np.zeros(a["x"].shape)
        b, m, h, d = a["x"].shape
        S = {"dA": np.zeros((b, m, h)), "dt": np.zeros((b, m, h)), "u": np.zeros((b, m, h, d)),
             "B": np.zeros(a["B"].shape)}

        def call():
            oracle.tree(a["x"], a["A"], a["B"], a["C"], a["dt"], a["state"], out, a["parent_ids"],
                        depths=a["depths"], dt_bias=a["dt_bias"], D=a["D"], z=a["z"],
                        dt_softplus=w.dt_softplus, state_indices=a["state_indices"], stash=S)
        sample = "the full tree batch of this workload"
    elif kind == "gdn":
        idx = a["state_indices"]
        live = idx[idx >= 0]
        st = a["ssm_state"][live].copy()            # compact pools of the addressed slots
        cs = a["conv_state"][live].copy()
        remap = np.full(idx.shape, -1, dtype=np.int32)
        remap[idx >= 0] = np.arange(live.size, dtype=np.int32)

        def call():
            oracle.gdn_decode(a["hidden_states"], a["w_ba"], a["mixed_qkv"], a["conv_weight"],
                              a["conv_bias"], cs, a["A_log"], a["dt_bias"], w.dims["scale"], st,
                              remap, num_q_heads=w.dims["num_q_heads"],
                              use_qk_l2norm=w.dims["use_qk_l2norm"])
        sample = f"the full {idx.shape[0]}-entry batch of this workload"
    elif kind == "gather":
        idx = a["state_indices"]
        pool = a["state"]

        def call():
            oracle.gather(pool, idx)
        sample = "the full 64-row gather of this workload"
    elif kind == "clear_layers":
        nl = 4
        rows = a["state"].shape[0]
        rec_rb = a["state"][0].size * 4
        conv_rb = inputs_mod.STACK_CONV_ROW_BYTES
        recs = [np.ones(rows * rec_rb, dtype=np.uint8) for _ in range(nl)]
        convs = [np.ones(rows * conv_rb, dtype=np.uint8) for _ in range(nl)]
        slot = [0]

        def call():
            oracle.clear_layers(recs, convs, rows, slot[0] % rows, rec_rb, conv_rb)
            slot[0] += 1
        sample = f"{nl} of the {inputs_mod.STACK_LAYERS} layers per call"
        scale = nl / inputs_mod.STACK_LAYERS
    else:
        st = a["state"].copy()
        reps = 1 if kind == "replay" else 2
        stacks = [st] + [st.copy() for _ in range(reps - 1)]

        def call():
            for s_ in stacks:
                oracle.replay(s_, a["replay_dA"], a["replay_u"], a["replay_B"], a["replay_dt"],
                              a["accepted_lengths"], state_indices=a["state_indices"],
                              active_batch=w.active_batch)
        if kind == "replay":
            sample = "the full replay batch of this workload"
        else:
            sample = f"{reps} of the {inputs_mod.STACK_LAYERS} layers per call"
            scale = reps / inputs_mod.STACK_LAYERS
    def timed(limit):
        calls, t0 = 0, time.perf_counter()
        while True:
            call()
            calls += 1
            el = time.perf_counter() - t0
            if el >= limit:
                return calls, el

    threads = oracle.num_threads()
    calls, el = timed(seconds)
    gbs = bytes_per_call * scale * calls / el / 1e9
    # the same sample on one thread (a single call at least)
    oracle.set_num_threads(1)
    try:
        calls1, el1 = timed(seconds / 3)
    finally:
        oracle.set_num_threads(threads)
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{sample}, {calls} call(s) in {el:.1f} s (fp64, OpenMP)",
            "cpu_model": cpu_model(),
            "token_head_updates_per_s": units_per_call * scale * calls / el,
            "single_thread": {"value": round(bytes_per_call * scale * calls1 / el1 / 1e9, 4),
                              "unit": "GB/s", "calls": calls1, "seconds": round(el1, 2)}}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def flushed_launches(step, first, n, warm, dev):
    """Per-launch times (us) of n steps, each preceded by a write of FLUSH_BYTES
    of scratch outside its event pair, so that no step finds its data in the
    last-level cache; warm untimed flushed steps first."""
    import torch
    scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    evs = []
    for i in range(warm + n):
        scratch.fill_(float(i))
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        step(first + i)
        b.record()
        if i >= warm:
            evs.append((a, b))
    torch.cuda.synchronize()
    del scratch
    return sorted(a.elapsed_time(b) * 1e3 for a, b in evs)


def copy_bandwidth(dev, nbytes=1 << 30, reps=10):
    """Device-to-device copy rate (bytes read + written per second): the
    achievable streaming rate on this machine, as context for the HBM peak."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    return 2 * nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", type=int, default=1, choices=[1, 2, 3, 4, 5, 6, 7, 8, 9])
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--prewarm-ms", type=float, default=300.0,
                    help="untimed launches before the warm-up steps, to reach steady clocks")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the timed steps one by one from Python instead of one HIP graph")
    ap.add_argument("--flushed", type=int, default=100,
                    help="after the graph-timed steps, time this many launches one by one, each "
                         "after a 1 GiB scratch write (median, p10, p90); 0 skips it")
    ap.add_argument("--operands", choices=["bf16", "f16", "f32"], default="bf16",
                    help="config 2: the dtype of x/z/B/C/out (bf16 as the workload states; fp16 "
                         "also runs on the matrix cores, fp32 on the VALU kernel)")
    ap.add_argument("--stash", action="store_true", help="config 2: prefill with the replay stash")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the timed steps, one plain device copy of this many MiB "
                         "(a known-size kernel for scaling memory-traffic counters)")
    args = ap.parse_args()
    if args.config != 2 and (args.operands != "bf16" or args.stash):
        ap.error("--operands and --stash apply to --config 2 (prefill) only")
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the selective state update needs no collective, "
              "so only --gpus 1 is supported", file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_rnn_recurrent_amd import (ReplayLayerTable, StateLayerTable, inputs, load_library,
                                          gdn_workspace_bytes, tree_workspace_bytes,
                                          ssu_decode, ssu_gdn_decode,
                                          ssu_prefill,
                                          ssu_replay, ssu_replay_layers, ssu_state_clear_layers,
                                          ssu_state_gather, ssu_tree_verify)

    load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.config == 5:
        w, name = inputs.tree_config(), inputs.TREE_NAME
    elif args.config in (6, 7):
        w, name = inputs.config(4), inputs.LAYERS_NAME[args.config]
    elif args.config == 8:
        w, name = inputs.config(1), inputs.GATHER_NAME
    elif args.config == 9:
        w, name = inputs.gdn_config(), inputs.GDN_NAME
    else:
        w, name = inputs.config(args.config), inputs.CONFIG_NAMES[args.config]
    if args.operands != "bf16":  # config 2 with the same values in another dtype
        dt_ = {"f16": torch.float16, "f32": torch.float32}[args.operands]
        for k in ("x", "z", "B", "C"):
            if w.tensors[k] is not None:
                w.tensors[k] = w.tensors[k].to(dt_)
        name += f"; {args.operands} x/z/B/C/out"
    if args.stash:
        name += "; replay stash on (state read-only)"
    T = {k: (None if v is None else v.to(dev)) for k, v in w.tensors.items()}
    stream = torch.cuda.current_stream(dev)

    def replicas(names, n):
        """n copies of the named tensors (replica 0 is the original)."""
        reps = [T]
        for _ in range(n - 1):
            r = dict(T)
            for k in names:
                if T[k] is not None:
                    r[k] = T[k].clone()
            reps.append(r)
        return reps

    matrix = None
    if args.config in (1, 3):
        kind = "decode"
        B = T["x"].shape[0]
        if args.config == 1:
            idx_sets = [s.to(dev) for s in inputs.rotation_index_sets(w.dims["pool_rows"], B, seed=1)]
            reps = [dict(T, state_indices=ix) for ix in idx_sets]
            rot = "steps rotate 4 disjoint 64-row index sets over the pool"
        else:
            reps = replicas(["state"], 4)
            rot = "steps rotate 4 replicas of the pool"
        live = int((reps[0]["state_indices"] >= 0).sum().item())
        nbytes = decode_bytes(T, live)
        units = live * T["x"].shape[1]
        out = torch.empty_like(T["x"])

        def step(i):
            R = reps[i % len(reps)]
            ssu_decode(R["x"], R["A"], R["B"], R["C"], R["dt"], R["state"], out,
                       dt_bias=R["dt_bias"], D=R["D"], z=R["z"], dt_softplus=w.dt_softplus,
                       state_indices=R["state_indices"])
        src = source_hash("ssu_decode_impl.h", "ssu_device.h")
        kkey = f"decode_config{args.config}"
        bound, peak, unit = "hbm", HBM_PEAK_GBS, "GB/s"
    elif args.config == 2:
        kind = "prefill"
        L = T["context_lengths"].clamp(0, T["x"].shape[1]).cpu().tolist()
        nbytes = prefill_bytes(T, L, args.stash)
        units = sum(L) * T["x"].shape[2]
        reps = replicas(["x", "z", "B", "C", "dt", "state"], 4)
        outs = [torch.empty_like(T["x"]) for _ in reps]
        rot = "steps rotate 4 replicas of the pool and of every input and output"
        stashes = [{}] * len(reps)
        if args.stash:
            b_, t_, h_, d_ = T["x"].shape
            stashes = [{"replay_dA": torch.empty((b_, t_, h_), device=dev),
                        "replay_dt": torch.empty((b_, t_, h_), device=dev),
                        "replay_u": torch.empty((b_, t_, h_, d_), device=dev),
                        "replay_B": torch.empty(tuple(T["B"].shape), device=dev)} for _ in reps]

        def step(i):
            R = reps[i % len(reps)]
            ssu_prefill(R["x"], R["A"], R["B"], R["C"], R["dt"], R["state"], outs[i % len(reps)],
                        dt_bias=R["dt_bias"], D=R["D"], z=R["z"], dt_softplus=w.dt_softplus,
                        context_lengths=R["context_lengths"], state_indices=R["state_indices"],
                        **stashes[i % len(reps)])
        src = source_hash("ssu_prefill_impl.h", "ssu_prefill_mm.h", "ssu_rowblock.h", "ssu_device.h",
                          "ssu_dpp.h")
        kkey = "prefill_config2"
        if args.operands != "bf16" or args.stash:  # each variant has its own counter record
            kkey += f"_{args.operands}" + ("_stash" if args.stash else "")
        if args.operands != "f32":
            matrix = {"flops_per_step": prefill_method_flops(T, L),
                      "flops": "the method's own: 5 per state element and token",
                      "closed_form_fmas_per_step": prefill_mm_fmas(T, L), "dtype": args.operands}
        bound, peak, unit = "hbm", HBM_PEAK_GBS, "GB/s"
    elif args.config == 5:
        kind = "tree"
        b, m, h, d = T["x"].shape
        nbytes = tree_bytes(T)
        units = int((T["state_indices"] >= 0).sum().item()) * m * h
        reps = replicas(["x", "B", "C", "dt", "state"], 3)
        for R in reps:
            R["out"] = torch.empty_like(T["x"])
            R["S"] = {"replay_dA": torch.empty((b, m, h), device=dev),
                      "replay_dt": torch.empty((b, m, h), device=dev),
                      "replay_u": torch.empty((b, m, h, d), device=dev),
                      "replay_B": torch.empty(tuple(T["B"].shape), device=dev)}
        rot = "steps rotate 3 replicas of the pool, of every input and of the outputs and stash"
        tws = torch.empty(tree_workspace_bytes(b, T["B"].shape[2], m), dtype=torch.uint8,
                          device=dev)

        def step(i):
            R = reps[i % len(reps)]
            ssu_tree_verify(R["x"], R["A"], R["B"], R["C"], R["dt"], R["state"], R["out"],
                            R["parent_ids"], depths=R["depths"], dt_bias=R["dt_bias"], D=R["D"],
                            z=R["z"], dt_softplus=w.dt_softplus, state_indices=R["state_indices"],
                            workspace=tws, **R["S"])
        src = source_hash("ssu_tree_impl.h", "ssu_dpp.h", "ssu_device.h")
        kkey = "tree_config5"
        fmas = tree_lane_ops(T)
        matrix = {"flops_per_step": 2 * fmas,
                  "flops": "the closed form's: S0.C per node and one B.C dot and x term per "
                           "path entry",
                  "closed_form_fmas_per_step": fmas}
        bound, peak, unit = "hbm", HBM_PEAK_GBS, "GB/s"
    elif args.config == 6:
        kind = "replay_layers"
        nl = inputs.STACK_LAYERS
        acc = T["accepted_lengths"][: w.active_batch].cpu()
        idx = T["state_indices"][: w.active_batch].cpu()
        k_rows = [min(int(a), T["replay_dA"].shape[1]) if int(i) >= 0 else 0
                  for a, i in zip(acc, idx)]
        nbytes = nl * replay_bytes(T, k_rows)
        units = nl * sum(k_rows) * T["replay_dA"].shape[2]
        # every layer its own pool and stash (copies of the config-4 tensors)
        table = ReplayLayerTable([T["state"].clone() for _ in range(nl)],
                                 [T["replay_dA"].clone() for _ in range(nl)],
                                 [T["replay_u"].clone() for _ in range(nl)],
                                 [T["replay_B"].clone() for _ in range(nl)],
                                 [T["replay_dt"].clone() for _ in range(nl)])
        rot = f"one launch replays all {nl} layers ({nl} separate pools, 8 GB in all)"

        def step(i):
            ssu_replay_layers(table, T["accepted_lengths"], state_indices=T["state_indices"],
                              active_batch=w.active_batch)
        src = source_hash("ssu_replay.hip", "ssu_device.h")
        kkey = "replay_layers_config6"
        bound, peak, unit = "hbm", HBM_PEAK_GBS, "GB/s"
    elif args.config == 7:
        kind = "clear_layers"
        nl = inputs.STACK_LAYERS
        rows = T["state"].shape[0]
        rec_rb = T["state"][0].numel() * T["state"].element_size()
        conv_rb = inputs.STACK_CONV_ROW_BYTES
        recs = [torch.ones_like(T["state"]) for _ in range(nl)]
        convs = [torch.ones(rows * conv_rb, dtype=torch.uint8, device=dev) for _ in range(nl)]
        table = StateLayerTable(recs, convs)
        nbytes = nl * (rec_rb + conv_rb)
        units = nl
        rot = f"one launch clears one slot of all {nl} layers; steps rotate over the {rows} slots"

        def step(i):
            ssu_state_clear_layers(table, rows, i % rows, rec_rb, conv_rb)
        src = source_hash("ssu_pool_kernels.hip", "ssu_device.h")
        kkey = "clear_layers_config7"
        bound, peak, unit = "hbm", HBM_PEAK_GBS, "GB/s"
    elif args.config == 8:
        kind = "gather"
        B = T["x"].shape[0]
        idx_sets = [s.to(dev) for s in inputs.rotation_index_sets(w.dims["pool_rows"], B, seed=1)]
        active = torch.empty((B,) + tuple(T["state"].shape[1:]), device=dev)
        row_bytes = T["state"][0].numel() * T["state"].element_size()
        nbytes = 2 * B * row_bytes
        units = B
        rot = "steps rotate 4 disjoint 64-row index sets over the pool"

        def step(i):
            ssu_state_gather(T["state"], active, idx_sets[i % len(idx_sets)])
        src = source_hash("ssu_pool_kernels.hip", "ssu_device.h")
        kkey = "gather_config8"
        bound, peak, unit = "hbm", HBM_PEAK_GBS, "GB/s"
    elif args.config == 9:
        kind = "gdn"
        B = T["hidden_states"].shape[0]
        idx_sets = [s.to(dev) for s in inputs.rotation_index_sets(w.dims["pool_rows"], B, seed=1)]
        nbytes = gdn_bytes(T, B)
        units = B * w.dims["num_v_heads"]
        out = torch.empty((B, 1, w.dims["num_v_heads"], w.dims["head_dim"]), dtype=torch.bfloat16,
                          device=dev)
        ws = torch.empty(gdn_workspace_bytes(B, w.dims["hidden"], w.dims["num_q_heads"],
                                             w.dims["num_v_heads"], w.dims["head_dim"]),
                         dtype=torch.uint8, device=dev)
        rot = "steps rotate 4 disjoint 64-slot index sets over both pools"

        def step(i):
            ssu_gdn_decode(T["hidden_states"], T["w_ba"], T["mixed_qkv"], T["conv_weight"],
                           T["conv_bias"], T["conv_state"], T["A_log"], T["dt_bias"],
                           w.dims["scale"], T["ssm_state"], idx_sets[i % len(idx_sets)],
                           num_q_heads=w.dims["num_q_heads"],
                           use_qk_l2norm=w.dims["use_qk_l2norm"], out=out, workspace=ws)
        src = source_hash("ssu_gdn.hip", "ssu_dpp.h", "ssu_device.h")
        kkey = "gdn_config9"
        bound, peak, unit = "hbm", HBM_PEAK_GBS, "GB/s"
    else:
        kind = "replay"
        acc = T["accepted_lengths"][: w.active_batch].cpu()
        idx = T["state_indices"][: w.active_batch].cpu()
        k_rows = [min(int(a), T["replay_dA"].shape[1]) if int(i) >= 0 else 0
                  for a, i in zip(acc, idx)]
        nbytes = replay_bytes(T, k_rows)
        units = sum(k_rows) * T["replay_dA"].shape[2]
        reps = replicas(["state"], 8)
        rot = "steps rotate 8 replicas of the pool"

        def step(i):
            R = reps[i % len(reps)]
            ssu_replay(R["state"], R["replay_dA"], R["replay_u"], R["replay_B"], R["replay_dt"],
                       R["accepted_lengths"], state_indices=R["state_indices"],
                       active_batch=w.active_batch)
        src = source_hash("ssu_replay.hip", "ssu_device.h")
        kkey = "replay_config4"
        bound, peak, unit = "hbm", HBM_PEAK_GBS, "GB/s"

    # Bring the GPU to its steady clocks before the W warm-up steps: a few
    # milliseconds of launches are not enough for the clocks to ramp.
    t_pre = time.perf_counter()
    n_pre = 0
    while (time.perf_counter() - t_pre) * 1e3 < args.prewarm_ms:
        for _ in range(20):
            step(n_pre)
            n_pre += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] config {args.config} ({kind}) warmed up, timing {args.steps} steps",
          file=sys.stderr, flush=True)

    graph = None
    if not args.no_graph:
        # The K timed steps as one HIP graph: launches go back to back with no
        # host work between them, as in a captured serving loop.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                step(args.warmup + i)
        torch.cuda.synchronize()
        graph.replay()                      # untimed: first replay uploads the graph
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream(dev)

    wall0 = time.perf_counter()
    # back-to-back launches on one stream; events recorded on that same stream
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    wall = time.perf_counter() - wall0

    ms = total_ms / args.steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    achieved = gbs
    traffic = measured_traffic(kkey, src)
    rec = {
        "metric": metric_name(),
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": name + "; " + rot,
                   "kernel": kind, "algorithmic_bytes_per_step": nbytes,
                   "token_head_updates_per_step": units},
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "token_head_updates_per_s": round(units / (ms * 1e-3), 1),
        "roofline": {"bound": bound, "achieved": round(achieved, 3), "peak": round(peak, 3),
                     "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic},
        "launch": "eager" if graph is None else "hip graph of the K steps",
        "wall_s_timed": round(wall, 3),
        "prewarm": {"ms": args.prewarm_ms, "launches": n_pre},
    }
    if matrix is not None:
        # the matrix cores these kernels run on: bf16 MFMA (fp32 operands are split
        # into bf16 terms); neither this roof nor HBM binds them
        tf = matrix["flops_per_step"] / (ms * 1e-3) / 1e12
        cf = 2.0 * matrix["closed_form_fmas_per_step"] / (ms * 1e-3) / 1e12
        rec["roofline_matrix_cores"] = {
            "dtype": matrix.get("dtype", "bf16"), "flops": matrix["flops"], "achieved": round(tf, 3),
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "closed_form_fp32_equivalent": {"achieved": round(cf, 3),
                                            "peak_fp32_mfma": MFMA_F32_PEAK_TFLOPS,
                                            "frac": round(cf / MFMA_F32_PEAK_TFLOPS, 4)}}
    if args.flushed > 0:
        print(f"[bench] {args.flushed} launches, each after a {FLUSH_BYTES >> 30} GiB scratch write",
              file=sys.stderr, flush=True)
        us = flushed_launches(step, args.warmup + args.steps, args.flushed, 10, dev)
        pick = lambda q: us[min(len(us) - 1, int(round(q * (len(us) - 1))))]
        med = pick(0.5)
        rec["flushed"] = {"launches": len(us), "flush_bytes": FLUSH_BYTES,
                          "median_us": round(med, 2), "p10_us": round(pick(0.1), 2),
                          "p90_us": round(pick(0.9), 2),
                          "median_gbs": round(nbytes / (med * 1e-6) / 1e9, 1),
                          "median_hbm_frac": round(nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        rec["d2d_copy_gbs"] = round(copy_bandwidth(dev), 1)
    if args.copy_mib > 0:
        cal_src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        cal_dst = torch.empty_like(cal_src)
        torch.cuda.synchronize()
        cal_dst.copy_(cal_src)
        torch.cuda.synchronize()
        rec["copy_calibration_bytes"] = cal_src.numel() * 4
        del cal_src, cal_dst
    if not args.no_cpu_baseline:
        print(f"[bench] timing the fp64 oracle for about {args.cpu_seconds:.0f} s",
              file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(kind, w, args.cpu_seconds, nbytes, units, args.stash)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
