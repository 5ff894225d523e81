"""The decay-handling branches of both prefill kernels are reached by the GPU
strong-decay tests: checked on the CPU by taking the kernels' branch decisions
on those tests' own inputs.

The rescaled VALU recurrence (8-token chunks, fp32) keeps the running product
P_t of the decays exp(A dt') and, when a chunk's P_t would leave [1e-30, 1e30],
either renormalises once before the chunk (every in-chunk prefix product stays
in range), or walks the chunk token by token, restarting the product at a
token (its decay in range) or applying a decay below 1e-30 directly. The
matrix-core kernel (32-token chunks) forms Q entry by entry in a chunk where a
4-token quad spans more than 2^64 of decay. The decisions below follow those
rules in the kernels' own precision (fp32 decays and products, the in-chunk
products in the VALU kernel's scan order); the GPU tests then compare every
case with the fp64 oracle.
"""
import numpy as np
import pytest

from test_gpu_strong_decay import strong_prefill_workload

TC_VALU = 8
TC_MM = 32
LO, HI = np.float32(1e-30), np.float32(1e30)


def _inside(v):
    return (v >= LO) & (v <= HI)


def _lengths(w):
    return np.clip(w["context_lengths"].numpy(), 0, w.dims["seq_len"]).astype(int)


def _dtp(w):
    # these workloads have softplus off and no dt_bias: dt' = dt
    assert not w.dims.get("dt_softplus", False) and w.tensors.get("dt_bias") is None
    return w["dt"].numpy().astype(np.float32)


def valu_branches(w):
    """Counts of VALU-kernel chunks that renormalise once, chunks walked token by
    token, and tokens whose decay is applied directly."""
    A = w["A"].numpy().astype(np.float32)
    dt = _dtp(w)
    n = {"once": 0, "walk": 0, "direct": 0, "plain": 0}
    for b, L in enumerate(_lengths(w)):
        for h in range(w.dims["nheads"]):
            pcarry = np.float32(1.0)
            for t0 in range(0, L, TC_VALU):
                nt = min(TC_VALU, L - t0)
                a = np.ones(TC_VALU, np.float32)
                a[:nt] = np.exp(A[h] * dt[b, t0:t0 + nt, h])
                pre = a.copy()  # inclusive scan, steps 1, 2, 4 as the kernel's shuffles
                d = 1
                while d < TC_VALU:
                    prev = pre.copy()
                    pre[d:] = prev[d:] * prev[:-d]
                    d *= 2
                P = pcarry * pre
                if _inside(P).all():
                    n["plain"] += 1
                elif _inside(pre).all():
                    n["once"] += 1
                    P = pre
                else:
                    n["walk"] += 1
                    pr = pcarry
                    for t in range(TC_VALU):
                        cand = np.float32(pr * a[t])
                        pt = cand
                        if not _inside(cand):
                            if _inside(a[t]):
                                pt = a[t]
                            else:
                                n["direct"] += 1
                                pt = np.float32(1.0)
                        P[t] = pt
                        pr = pt
                pcarry = P[-1]
    return n


def mm_branches(w):
    """Counts of matrix-core chunks whose Q is formed per entry (a quad spans more
    than 2^64 of decay) and per quad."""
    A = w["A"].numpy().astype(np.float32)
    dt = _dtp(w)
    n = {"per_entry": 0, "per_quad": 0}
    for b, L in enumerate(_lengths(w)):
        for h in range(w.dims["nheads"]):
            for t0 in range(0, L, TC_MM):
                nt = min(TC_MM, L - t0)
                a = np.zeros(TC_MM, np.float32)
                a[:nt] = A[h] * dt[b, t0:t0 + nt, h]
                l2 = np.cumsum(a, dtype=np.float32) * np.float32(1.4426950408889634)
                span = np.abs(np.repeat(l2[::4], 4) - l2)
                n["per_entry" if (span > 64).any() else "per_quad"] += 1
    return n


# the inputs of the GPU tests that run on the VALU kernel (fp32 operands, or
# fp16 operands placed off alignment), and of those on the matrix cores
VALU_CASES = [dict(io="f32", bc="f32"), dict(io="f16", bc="f16"), dict(io="f32", bc="bf16"),
              dict(io="f32", bc="f32", state_dtype="f16", seed=62),
              dict(io="f32", bc="f32", seed=63),
              dict(io="f32", bc="f32", seed=64, seq_len=1100)]
MM_CASES = [dict(io="bf16", bc="bf16"), dict(io="f16", bc="f16"),
            dict(io="bf16", bc="bf16", state_dtype="f16", seed=62),
            dict(io="f16", bc="f16", state_dtype="f16", seed=62)]


@pytest.mark.parametrize("case", VALU_CASES, ids=lambda c: "-".join(f"{k}={v}" for k, v in c.items()))
def test_valu_prefill_inputs_reach_every_decay_branch(case):
    n = valu_branches(strong_prefill_workload(**case))
    assert n["plain"] > 0 and n["once"] > 0 and n["walk"] > 0 and n["direct"] > 0, n


@pytest.mark.parametrize("case", MM_CASES, ids=lambda c: "-".join(f"{k}={v}" for k, v in c.items()))
def test_matrix_core_prefill_inputs_reach_both_q_forms(case):
    n = mm_branches(strong_prefill_workload(**case))
    assert n["per_entry"] > 0 and n["per_quad"] > 0, n
