"""Second, independent scalar oracle in pure Python (tiny shapes only).

TEST INFRASTRUCTURE ONLY: imported by tests/ alone.  It is written apart from
oracle/ssu_oracle.c (no shared code, different loop structure) so that the two
can be checked against each other by brute force on small inputs.

Definitions followed (TensorRT-Edge-LLM "Selective State Update" page):
  * mamba_ssm::invokeSelectiveStateUpdate, "Computes":
      new_state = state * exp(A * dt) + B * dt * x
      output    = sum_i new_state_i * C_i + D * x, then * silu(z) if z is given
  * invokeSelectiveStateUpdatePrefill: all seq_len tokens in order; with the
    replay stash the committed state stays read-only.
  * MambaReplayLayerInfo: replay the first acceptedLengths[b] stashed tokens;
    invokeMambaReplayReconstructBatched: optionally through acceptedNodeIds.
  * invokeSelectiveStateUpdateDDTree: every node's output after the recurrence
    along its ancestor path.  Here the path's state is written in its unrolled
    form (products of the decays along the path), not replayed step by step,
    so that this file and the C oracle reach the tree outputs by different
    formulas.
  * FlashInfer "flashinfer.gdn_fused_decode_step": the fused gated-delta-rule
    decode step (readings as in oracle/gdn_oracle.c). Here the output is formed
    from the expanded update, o = alpha (S q) + delta (k . q), and the prediction
    as alpha (S k), instead of from the updated state row, so the two oracles
    reach the outputs by different formulas.
Padding rows (negative index) follow the FlashInfer gdn_fused_decode_step page,
parameter state_indices.

Every argument is a numpy float64/int32 array (or None) in the layouts of the
C oracle; every loop below runs over Python scalars.
"""
import math


def _sp(v):
    # softplus(v) = log(1 + e^v) evaluated without overflow
    if v > 0:
        return v + math.log1p(math.exp(-v))
    return math.log1p(math.exp(v))


def _gate(zv):
    return zv * (1.0 / (1.0 + math.exp(-zv)))


def _dt_proc(raw, bias, softplus):
    v = float(raw) + (0.0 if bias is None else float(bias))
    return _sp(v) if softplus else v


def _row(idx, b):
    return b if idx is None else int(idx[b])


def decode(x, A, B, C, dt, state, out, dt_bias=None, D=None, z=None,
           dt_softplus=True, state_indices=None):
    """x [b,h,d]; B,C [b,g,n]; dt [b,h]; state [rows,h,d,n]; out [b,h,d]."""
    nb, nh, nd = x.shape
    ng, ns = B.shape[1], B.shape[2]
    per_group = nh // ng
    for b in range(nb):
        r = _row(state_indices, b)
        for h in range(nh):
            if r < 0:
                for d in range(nd):
                    out[b, h, d] = 0.0
                continue
            grp = h // per_group
            dtp = _dt_proc(dt[b, h], None if dt_bias is None else dt_bias[h], dt_softplus)
            dec = math.exp(float(A[h]) * dtp)
            for d in range(nd):
                xv = float(x[b, h, d])
                total = 0.0
                for n in range(ns):
                    new = float(state[r, h, d, n]) * dec + float(B[b, grp, n]) * dtp * xv
                    state[r, h, d, n] = new
                    total += new * float(C[b, grp, n])
                if D is not None:
                    total += float(D[h]) * xv
                if z is not None:
                    total *= _gate(float(z[b, h, d]))
                out[b, h, d] = total


def prefill(x, A, B, C, dt, state, out, dt_bias=None, D=None, z=None,
            dt_softplus=True, context_lengths=None, state_indices=None,
            stash=None):
    """x [b,t,h,d]; B,C [b,t,g,n]; dt [b,t,h]; out [b,t,h,d].

    stash: None or dict with arrays 'dA' [b,t,h], 'u' [b,t,h,d], 'B' [b,t,g,n],
    'dt' [b,t,h] that are filled in while the state is left untouched.
    """
    nb, nt, nh, nd = x.shape
    ng, ns = B.shape[2], B.shape[3]
    per_group = nh // ng
    for b in range(nb):
        r = _row(state_indices, b)
        length = nt if context_lengths is None else min(max(int(context_lengths[b]), 0), nt)
        if r < 0:
            for t in range(nt):
                for h in range(nh):
                    for d in range(nd):
                        out[b, t, h, d] = 0.0
            continue
        for h in range(nh):
            grp = h // per_group
            # a private copy of this head's state for the whole sequence
            s = [[float(state[r, h, d, n]) for n in range(ns)] for d in range(nd)]
            for t in range(nt):
                if t >= length:
                    for d in range(nd):
                        out[b, t, h, d] = 0.0
                    if stash is not None:
                        stash['dA'][b, t, h] = 0.0
                        stash['dt'][b, t, h] = 0.0
                        for d in range(nd):
                            stash['u'][b, t, h, d] = 0.0
                        for n in range(ns):
                            stash['B'][b, t, grp, n] = 0.0
                    continue
                dtp = _dt_proc(dt[b, t, h], None if dt_bias is None else dt_bias[h], dt_softplus)
                dec = math.exp(float(A[h]) * dtp)
                for d in range(nd):
                    xv = float(x[b, t, h, d])
                    total = 0.0
                    for n in range(ns):
                        s[d][n] = s[d][n] * dec + float(B[b, t, grp, n]) * dtp * xv
                        total += s[d][n] * float(C[b, t, grp, n])
                    if D is not None:
                        total += float(D[h]) * xv
                    if z is not None:
                        total *= _gate(float(z[b, t, h, d]))
                    out[b, t, h, d] = total
                if stash is not None:
                    stash['dA'][b, t, h] = float(A[h]) * dtp
                    stash['dt'][b, t, h] = dtp
                    for d in range(nd):
                        stash['u'][b, t, h, d] = float(x[b, t, h, d])
                    for n in range(ns):
                        stash['B'][b, t, grp, n] = float(B[b, t, grp, n])
            if stash is None:
                for d in range(nd):
                    for n in range(ns):
                        state[r, h, d, n] = s[d][n]


def replay(state, dA, u, Bst, DT, accepted_lengths, state_indices=None,
           active_batch=None, node_ids=None):
    """dA, DT [b,t,h]; u [b,t,h,d]; Bst [b,t,g,n]; state [rows,h,d,n];
    node_ids None or [b, max_accept_len] (stash entry of each accepted token)."""
    nb_stash, nt, nh = dA.shape
    nd = u.shape[3]
    ng, ns = Bst.shape[2], Bst.shape[3]
    per_group = nh // ng
    nb = nb_stash if active_batch is None else active_batch
    for b in range(nb):
        r = _row(state_indices, b)
        cap = nt if node_ids is None else node_ids.shape[1]
        steps = min(int(accepted_lengths[b]), cap)
        if r < 0 or steps <= 0:
            continue
        order = []
        for t in range(steps):
            pos = t if node_ids is None else int(node_ids[b, t])
            if not 0 <= pos < nt:
                break
            order.append(pos)
        for h in range(nh):
            grp = h // per_group
            for t in order:
                dec = math.exp(float(dA[b, t, h]))
                for d in range(nd):
                    for n in range(ns):
                        state[r, h, d, n] = (float(state[r, h, d, n]) * dec
                                             + float(Bst[b, t, grp, n]) * float(DT[b, t, h])
                                             * float(u[b, t, h, d]))


def ancestors(parent_ids, depths, b, node):
    """Nodes whose tokens the recurrence of `node` runs over, node first, then
    its parent, and so on: at most depths[b, node] hops (any number without
    depths), ending at a negative parent id or one not smaller than the node
    it belongs to."""
    chain = [node]
    limit = node if depths is None else int(depths[b, node])
    while len(chain) <= limit:
        nxt = int(parent_ids[b, chain[-1]])
        if nxt < 0 or nxt >= chain[-1]:
            break
        chain.append(nxt)
    return chain


def tree(x, A, B, C, dt, state, out, parent_ids, depths=None, dt_bias=None, D=None, z=None,
         dt_softplus=True, state_indices=None, stash=None):
    """Tree verify. x, z, out [b,m,h,d]; B, C [b,m,g,n]; dt [b,m,h]; parent_ids,
    depths [b,m]. state [rows,h,d,n] is read only.

    For a node whose chain (node first) is c_0 .. c_k with decays a_i and inputs
    dt'_i x_i B_i, the state after the chain is
        (a_0 a_1 ... a_k) S0 + sum_i (a_0 ... a_{i-1}) dt'_i x_i B_i^T
    and the node's output is C_0 . state + D x_0, gated by silu(z_0)."""
    nb, nm, nh, nd = x.shape
    ng, ns = B.shape[2], B.shape[3]
    per_group = nh // ng
    for b in range(nb):
        r = _row(state_indices, b)
        if r < 0:
            for m in range(nm):
                for h in range(nh):
                    for d in range(nd):
                        out[b, m, h, d] = 0.0
            continue
        for h in range(nh):
            grp = h // per_group
            bias = None if dt_bias is None else dt_bias[h]
            dtp = [_dt_proc(dt[b, m, h], bias, dt_softplus) for m in range(nm)]
            dec = [math.exp(float(A[h]) * v) for v in dtp]
            for m in range(nm):
                chain = ancestors(parent_ids, depths, b, m)
                for d in range(nd):
                    total = 0.0
                    for n in range(ns):
                        later = 1.0   # product of the decays of the chain nodes after c_i
                        acc = 0.0
                        for c in chain:
                            acc += later * dtp[c] * float(x[b, c, h, d]) * float(B[b, c, grp, n])
                            later *= dec[c]
                        acc += later * float(state[r, h, d, n])
                        total += acc * float(C[b, m, grp, n])
                    if D is not None:
                        total += float(D[h]) * float(x[b, m, h, d])
                    if z is not None:
                        total *= _gate(float(z[b, m, h, d]))
                    out[b, m, h, d] = total
                if stash is not None:
                    stash['dA'][b, m, h] = float(A[h]) * dtp[m]
                    stash['dt'][b, m, h] = dtp[m]
                    for d in range(nd):
                        stash['u'][b, m, h, d] = float(x[b, m, h, d])
                    for n in range(ns):
                        stash['B'][b, m, grp, n] = float(B[b, m, grp, n])


def gdn_decode(hidden_states, w_ba, mixed_qkv, conv_weight, conv_bias, conv_state, A_log,
               dt_bias, scale, ssm_state, state_indices, num_q_heads, use_qk_l2norm=True):
    """Returns out [B, 1, HV, D]; conv_state [P, qkv, W-1] and ssm_state
    [P, HV, D, D] are updated in place."""
    nb, hidden = hidden_states.shape
    hv = w_ba.shape[1] // 2
    hq = num_q_heads
    qkv, width = conv_weight.shape
    dh = qkv // (2 * hq + hv)
    if scale is None or scale == 0.0:
        scale = 1.0 / math.sqrt(dh)
    out = [[[[0.0] * dh for _ in range(hv)]] for _ in range(nb)]
    for b in range(nb):
        s = int(state_indices[b])
        if s < 0:
            continue
        proj = [sum(float(hidden_states[b, i]) * float(w_ba[i, j]) for i in range(hidden))
                for j in range(2 * hv)]
        ch = []
        for c in range(qkv):
            taps = [float(conv_state[s, c, j]) for j in range(width - 1)]
            taps.append(float(mixed_qkv[b, c]))
            pre = float(conv_bias[c]) + sum(taps[j] * float(conv_weight[c, j]) for j in range(width))
            ch.append(pre / (1.0 + math.exp(-pre)))
            for j in range(width - 1):
                conv_state[s, c, j] = taps[j + 1]
        heads_q = [ch[h * dh:(h + 1) * dh] for h in range(hq)]
        heads_k = [ch[(hq + h) * dh:(hq + h + 1) * dh] for h in range(hq)]
        if use_qk_l2norm:
            heads_q = [[e / math.sqrt(sum(t * t for t in x) + 1e-6) for e in x] for x in heads_q]
            heads_k = [[e / math.sqrt(sum(t * t for t in x) + 1e-6) for e in x] for x in heads_k]
        heads_q = [[e * scale for e in x] for x in heads_q]
        for h in range(hv):
            q = heads_q[h // (hv // hq)]
            k = heads_k[h // (hv // hq)]
            v = ch[(2 * hq + h) * dh:(2 * hq + h + 1) * dh]
            beta = 1.0 / (1.0 + math.exp(-proj[h]))
            sp = _sp(proj[hv + h] + float(dt_bias[h]))
            alpha = math.exp(-math.exp(float(A_log[h])) * sp)
            kq = sum(k[i] * q[i] for i in range(dh))
            for vi in range(dh):
                row = [float(ssm_state[s, h, vi, i]) for i in range(dh)]
                sk = sum(row[i] * k[i] for i in range(dh))
                sq = sum(row[i] * q[i] for i in range(dh))
                delta = beta * (v[vi] - alpha * sk)
                out[b][0][h][vi] = alpha * sq + delta * kq
                for i in range(dh):
                    ssm_state[s, h, vi, i] = alpha * row[i] + delta * k[i]
    return out
