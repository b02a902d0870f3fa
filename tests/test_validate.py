"""CPATTN_VALIDATE=1: the calls (the multi-block gradient call per block)
copy the position arrays to the host and reject ones that do not ascend
(CPATTN_ERR_UNSORTED), and a planned document call (forward or gradient)
recomputes its plan and rejects a different one (CPATTN_ERR_RANGE), before
anything is enqueued.
The setting is read once per process, so the checks run in a child process
started with it set."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r'''
import torch
import context_long_sequence_amd as cp

dev = "cuda"
lq, lk, hq, d = 64, 96, 2, 64
g = torch.Generator().manual_seed(3)
q = torch.randn((lq, hq, d), generator=g).to(torch.bfloat16).to(dev)
k = torch.randn((lk, hq, d), generator=g).to(torch.bfloat16).to(dev)
v = torch.randn((lk, hq, d), generator=g).to(torch.bfloat16).to(dev)
o = torch.empty((lq, hq, d), dtype=torch.bfloat16, device=dev)
lse = torch.empty((hq, lq), dtype=torch.float32, device=dev)
qp = torch.arange(100, 100 + lq, dtype=torch.int32, device=dev)
kp = torch.arange(60, 60 + lk, dtype=torch.int32, device=dev)
bad_q = qp.clone(); bad_q[10], bad_q[11] = qp[11], qp[10]
bad_k = kp.clone(); bad_k[50], bad_k[51] = kp[51], kp[50]
cu = torch.tensor([0, 80, 200], dtype=torch.int32, device=dev)
bad_cu = torch.tensor([0, 120, 80, 200], dtype=torch.int32, device=dev)

def status(fn):
    try:
        fn()
        torch.cuda.synchronize()
        return "OK"
    except cp.CpattnError as e:
        return cp.STATUS.get(e.status, str(e.status))

print("fwd sorted", status(lambda: cp.cpattn_partial(q, k, v, qp, kp, o, lse)))
print("fwd q unsorted", status(lambda: cp.cpattn_partial(q, k, v, bad_q, kp, o, lse)))
print("fwd k unsorted", status(lambda: cp.cpattn_partial(q, k, v, qp, bad_k, o, lse)))
print("varlen cu unsorted", status(lambda: cp.cpattn_varlen_partial(q, k, v, qp, kp, bad_cu, o, lse)))
print("varlen sorted", status(lambda: cp.cpattn_varlen_partial(q, k, v, qp, kp, cu, o, lse)))
plan = cp.cpattn_varlen_plan(qp.cpu().numpy(), kp.cpu().numpy(), cu.cpu().numpy(), hq, hq, d)
other = cp.cpattn_varlen_plan(qp.cpu().numpy(), (kp + 7).cpu().numpy(), cu.cpu().numpy(), hq, hq, d)
print("varlen plan", status(lambda: cp.cpattn_varlen_partial(q, k, v, qp, kp, cu, o, lse,
                                                              plan=torch.from_numpy(plan).to(dev))))
print("varlen other plan", status(lambda: cp.cpattn_varlen_partial(q, k, v, qp, kp, cu, o, lse,
                                                                    plan=torch.from_numpy(other).to(dev))))
cp.cpattn_partial(q, k, v, qp, kp, o, lse)
delta = torch.empty((hq, lq), dtype=torch.float32, device=dev)
cp.cpattn_bwd_delta(o, q, delta)
dq = torch.empty((lq, hq, d), dtype=torch.float32, device=dev)
dk = torch.empty((lk, hq, d), dtype=torch.float32, device=dev)
dv = torch.empty((lk, hq, d), dtype=torch.float32, device=dev)
print("bwd sorted", status(lambda: cp.cpattn_partial_bwd(q, k, v, q, qp, kp, lse, delta, dq, dk, dv)))
print("bwd k unsorted", status(lambda: cp.cpattn_partial_bwd(q, k, v, q, qp, bad_k, lse, delta, dq, dk, dv)))
print("bwd cu unsorted", status(lambda: cp.cpattn_partial_bwd(q, k, v, q, qp, kp, lse, delta, dq, dk, dv,
                                                              cu_seqlens=bad_cu)))
bplan = cp.cpattn_varlen_bwd_plan(qp.cpu().numpy(), kp.cpu().numpy(), cu.cpu().numpy(), hq, hq)
bother = torch.from_numpy(bplan[::-1].copy()).to(dev)
bplan = torch.from_numpy(bplan).to(dev)
print("bwd plan", status(lambda: cp.cpattn_partial_bwd(q, k, v, q, qp, kp, lse, delta, dq, dk, dv, cu_seqlens=cu,
                                                       plan=bplan)))
print("bwd other plan", status(lambda: cp.cpattn_partial_bwd(q, k, v, q, qp, kp, lse, delta, dq, dk, dv,
                                                             cu_seqlens=cu, plan=bother)))
dk2, dv2 = torch.empty_like(dk), torch.empty_like(dv)
print("bwd multi sorted", status(lambda: cp.cpattn_partial_bwd_multi(q, [k, k], [v, v], q, qp, [kp, kp], lse, delta,
                                                                     dq, [dk, dk2], [dv, dv2])))
print("bwd multi k unsorted", status(lambda: cp.cpattn_partial_bwd_multi(q, [k, k], [v, v], q, qp, [kp, bad_k], lse,
                                                                         delta, dq, [dk, dk2], [dv, dv2])))
'''


def test_validate_rejects_unsorted_positions():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    env = dict(os.environ, CPATTN_VALIDATE="1", PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    r = subprocess.run([sys.executable, "-c", SCRIPT], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=240)
    print(r.stdout)
    assert r.returncode == 0, r.stderr[-2000:]
    got = dict(line.rsplit(" ", 1) for line in r.stdout.strip().splitlines())
    assert got == {
        "fwd sorted": "OK",
        "fwd q unsorted": "ERR_UNSORTED",
        "fwd k unsorted": "ERR_UNSORTED",
        "varlen cu unsorted": "ERR_UNSORTED",
        "varlen sorted": "OK",
        "varlen plan": "OK",
        "varlen other plan": "ERR_RANGE",
        "bwd sorted": "OK",
        "bwd k unsorted": "ERR_UNSORTED",
        "bwd cu unsorted": "ERR_UNSORTED",
        "bwd plan": "OK",
        "bwd other plan": "ERR_RANGE",
        "bwd multi sorted": "OK",
        "bwd multi k unsorted": "ERR_UNSORTED",
    }, got
