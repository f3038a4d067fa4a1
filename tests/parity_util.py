"""Helpers shared by the GPU parity tests: run the HIP path through the C-ABI binding,
run the fp64 oracle on the same bf16 inputs, and compare element by element."""
import math

import numpy as np

import synthetic_inputs as si

# Tolerances of the target: O, dQ, dK, dV within relative L2 5e-3 and max abs 2e-2;
# LSE within 1e-4 absolute.
REL_L2 = 5e-3
MAX_ABS = 2e-2
LSE_ABS = 1e-4


def to_device(arrs):
    import torch
    return {n: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda() for n, a in arrs.items()}


def gpu_run(arrs, scale, backward=True, stream=None):
    """Runs attn_fwd (and attn_bwd_dq, attn_bwd_dkv) on device copies of the bf16 inputs.
    Returns numpy float64 copies of every output (o widened from bf16)."""
    import torch
    import causal_gqa_flash_amd as cg
    x = to_device(arrs)
    o, lse = cg.attn_fwd(x["q"], x["k"], x["v"], scale=scale, stream=stream)
    out = dict(o=o, lse=lse)
    if backward:
        delta, dq = cg.attn_bwd_dq(x["q"], x["k"], x["v"], o, x["do"], lse, scale=scale, stream=stream)
        dk, dv = cg.attn_bwd_dkv(x["q"], x["k"], x["v"], x["do"], lse, delta, scale=scale, stream=stream)
        out.update(delta=delta, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {n: t.float().cpu().numpy().astype(np.float64) for n, t in out.items()}


def oracle_run(arrs, scale, backward=True):
    import oracle
    f = {n: oracle.bf16_to_f64(a) for n, a in arrs.items()}
    if backward:
        return oracle.attn_bwd(f["q"], f["k"], f["v"], f["do"], scale)
    o, lse = oracle.attn_fwd(f["q"], f["k"], f["v"], scale)
    return dict(o=o, lse=lse)


def compare(name, got, want, rel_l2=REL_L2, max_abs=MAX_ABS):
    """Returns (ok, message). The message names the first element whose absolute error
    exceeds max_abs (as index tuple), the relative L2 error and the largest error."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    if got.size == 0:
        return True, f"{name}: empty"
    if not np.all(np.isfinite(got)):
        bad = np.argwhere(~np.isfinite(got))[0]
        return False, f"{name}: non-finite value at {tuple(bad)}"
    err = np.abs(got - want)
    denom = np.linalg.norm(want)
    rel = np.linalg.norm(got - want) / denom if denom > 0 else np.linalg.norm(got - want)
    mx = float(err.max())
    first = ""
    if mx > max_abs:
        first = f" first failing index {tuple(np.argwhere(err > max_abs)[0])}"
    ok = (rel <= rel_l2 if rel_l2 is not None else True) and mx <= max_abs
    return ok, f"{name}: rel_l2={rel:.3e} max_abs={mx:.3e}{first}"


def check_all(got, want, keys=("o", "lse", "dq", "dk", "dv"), inputs=None):
    msgs, ok = [], True
    for k in keys:
        if k not in got:
            continue
        if k == "lse":
            good, m = compare(k, got[k], want[k], rel_l2=None, max_abs=LSE_ABS)
        else:
            good, m = compare(k, got[k], want[k])
        ok &= good
        msgs.append(m)
    return ok, "; ".join(msgs)


def slice_outputs(out, Hq, Hkv, b, g):
    """The outputs of one (batch, kv head) slice of full-size results."""
    G = Hq // Hkv
    r = {}
    for n, a in out.items():
        if n in ("lse", "delta"):
            r[n] = a[b:b + 1, g * G:(g + 1) * G, :]
        elif n in ("o", "dq"):
            r[n] = a[b:b + 1, :, g * G:(g + 1) * G, :]
        else:
            r[n] = a[b:b + 1, :, g:g + 1, :]
    return r


def workload_scale(d):
    return float(np.float32(1.0 / math.sqrt(d)))
