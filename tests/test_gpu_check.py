"""csa2_check_index (the device-side check of index rows) and debug mode.

* On the oracle-exact outputs of the Full and Reindex calls (ragged
  visibility, an empty row, a long context) every row passes.
* Rows altered on the host (out of order, out of range, a hole, a missing or
  extra entry, a position outside the pool, a pool not ascending or too
  long) are each counted exactly once.
* With CSA2_DEBUG=1 (a child process: the flag is read when the library
  loads) correct calls return CSA2_OK and a Reindex call given a pool that
  is not ascending returns CSA2_ERR_DEBUG without writing its Top-K."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import fp4_kv_cache_e4m3_amd as csa2
from tests.parity import dev, host

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def inputs(seed, B, Qn, T, HI=8, DI=128):
    rng = np.random.default_rng(seed)
    iq = rng.integers(-8, 9, size=(B * Qn, HI, DI), dtype=np.int8)
    iw = rng.integers(1, 9, size=(B * Qn, HI)).astype(np.float32)
    ik = rng.integers(-8, 9, size=(B, T, DI), dtype=np.int8)
    return [dev(a) for a in (iq, iw, ik)]


def run(args, pool, topk, mode):
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    csa2.check_index(args, pool, topk, mode, bad)
    return int(host(bad)[0])


def full(args, nq):
    ws = torch.empty(max(256, csa2.index_workspace_size(args)), dtype=torch.uint8, device="cuda")
    pool = torch.full((nq, 2048), -7, dtype=torch.int32, device="cuda")
    topk = torch.full((nq, 512), -7, dtype=torch.int32, device="cuda")
    csa2.index_full(args, pool, topk, ws)
    return pool, topk, ws


@pytest.mark.parametrize("B,Qn,T", [(2, 3, 20011), (1, 2, 1 << 19), (3, 1, 300)])
def test_check_passes_full_and_reindex_outputs(B, Qn, T):
    iq, iw, ik = inputs(B + Qn + T, B, Qn, T)
    nq = B * Qn
    nv = dev(np.array([T, 0, 9, 513, T - 1, 4097][:nq], dtype=np.int32)) if nq > 1 else None
    args = csa2.index_args(iq, iw, ik, Qn, nv)
    pool, topk, ws = full(args, nq)
    assert run(args, pool, topk, 0) == 0
    assert run(args, None, topk, 0) == 0                    # without the pool
    assert run(args, pool, None, 2) == 0
    iq2, iw2, _ = inputs(B + Qn + T + 1, B, Qn, T)
    args2 = csa2.index_args(iq2, iw2, ik, Qn, nv)
    rtopk = torch.full((nq, 512), -7, dtype=torch.int32, device="cuda")
    csa2.index_reindex(args2, pool, rtopk, ws)
    assert run(args2, pool, rtopk, 1) == 0


def ref_bad(pool_row, topk_row, nv, mode):
    """The contract of csa2_check_index for one query, restated on the host:
    the number of failing rows (pool, Top-K) it must report."""
    nb = (nv + 7) // 8
    bad = 0
    pc, npos = 0, 0
    if pool_row is not None:
        v = [int(x) for x in pool_row]
        lead = [x for x in v if x >= 0]
        pc = len(lead)
        ok = all(x >= 0 or x == -1 for x in v) and v[:pc] == lead and v[pc:] == [-1] * (len(v) - pc)
        ok = ok and all(a < b for a, b in zip(lead, lead[1:]))
        if mode == 0:
            ok = ok and all(x < nb for x in lead) and pc == min(2048, nb)
        npos = sum(min(8, nv - 8 * x) for x in lead if x < nb)
        bad += not ok
    if mode != 2:
        v = [int(x) for x in topk_row]
        lead = [x for x in v if x >= 0]
        tc = len(lead)
        ok = all(x >= 0 or x == -1 for x in v) and v[:tc] == lead and v[tc:] == [-1] * (len(v) - tc)
        ok = ok and all(a < b for a, b in zip(lead, lead[1:])) and all(x < nv for x in lead)
        if pool_row is not None:
            blocks = set(int(x) for x in pool_row[:pc])
            ok = ok and all(x // 8 in blocks for x in lead)
        if mode == 0:
            ok = ok and tc == min(512, nv)
        if mode == 1:
            ok = ok and tc == min(512, npos)
        bad += not ok
    return bad


def test_check_counts_each_altered_row_once():
    B, Qn, T = 1, 12, 30011
    iq, iw, ik = inputs(5, B, Qn, T)
    args = csa2.index_args(iq, iw, ik, Qn)
    pool, topk, _ = full(args, B * Qn)
    p, t = host(pool).copy(), host(topk).copy()
    t[0, [10, 11]] = t[0, [11, 10]]                         # out of order
    t[1, 5] = T + 3                                          # out of range
    t[2, 7] = -1                                             # a hole
    t[3, 511] = -1                                           # one entry short
    out = sorted(set(range(0, T, 8)) - set(int(x) * 8 for x in p[4] if x >= 0))[0]
    t[4] = np.sort(np.append(t[4][:511], out))               # a position outside the pool, in order
    t[5, 3] = t[5, 2]                                        # a repeated position
    p[6, [0, 1]] = p[6, [1, 0]]                              # pool out of order
    used = set(int(x) // 8 for x in t[7])                    # pool one block short (one no Top-K entry uses)
    k = next(i for i in range(2048) if int(p[7, i]) not in used)
    p[7] = np.append(np.delete(p[7], k), -1)
    p[8, 100] = -5                                           # pool: a bad sentinel
    for mode, pp, tt in ((0, p, t), (2, p, None), (0, None, t), (0, host(pool), t), (0, p, host(topk))):
        want = sum(ref_bad(None if pp is None else pp[q], None if tt is None else tt[q], T, mode) for q in range(12))
        got = run(args, None if pp is None else dev(pp), None if tt is None else dev(tt), mode)
        assert got == want, (mode, got, want)
    # every altered row is caught, the others pass
    per_row = [ref_bad(p[q], t[q], T, 0) for q in range(12)]
    assert all(per_row[q] > 0 for q in range(9)) and per_row[9:] == [0, 0, 0]
    assert run(args, dev(p), dev(t), 0) == sum(per_row)


def test_debug_mode_reports_a_bad_pool():
    script = r"""
import sys
sys.path.insert(0, %r)
import numpy as np, torch
import fp4_kv_cache_e4m3_amd as csa2
from fp4_kv_cache_e4m3_amd import _binding as B
rng = np.random.default_rng(3)
iq = torch.from_numpy(rng.integers(-8, 9, size=(4, 8, 128), dtype=np.int8)).cuda()
iw = torch.from_numpy(rng.integers(1, 9, size=(4, 8)).astype(np.float32)).cuda()
ik = torch.from_numpy(rng.integers(-8, 9, size=(2, 5003, 128), dtype=np.int8)).cuda()
args = csa2.index_args(iq, iw, ik, 2)
ws = torch.empty(max(256, csa2.index_workspace_size(args)), dtype=torch.uint8, device="cuda")
pool = torch.full((4, 2048), -1, dtype=torch.int32, device="cuda")
topk = torch.full((4, 512), -1, dtype=torch.int32, device="cuda")
lib = B.load()
print("full", lib.csa2_index_full(B.ctypes.byref(args), B._ptr(pool), B._ptr(topk), B._ptr(ws), ws.numel(), None))
print("reindex", lib.csa2_index_reindex(B.ctypes.byref(args), B._ptr(pool), B._ptr(topk), B._ptr(ws), ws.numel(), None))
bad = pool.clone()
bad[1, :2] = bad[1, :2].flip(0)
before = topk.clone()
print("bad", lib.csa2_index_reindex(B.ctypes.byref(args), B._ptr(bad), B._ptr(topk), B._ptr(ws), ws.numel(), None))
torch.cuda.synchronize()
print("untouched", bool(torch.equal(before, topk)))
""" % ROOT
    env = dict(os.environ, CSA2_DEBUG="1")
    r = subprocess.run([sys.executable, "-c", script], env=env, capture_output=True, text=True, timeout=180)
    assert r.returncode == 0, r.stderr[-2000:]
    out = dict(line.split() for line in r.stdout.strip().splitlines())
    assert out == {"full": "0", "reindex": "0", "bad": "7", "untouched": "True"}, r.stdout
