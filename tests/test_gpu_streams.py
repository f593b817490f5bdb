"""The C ABI is thread-safe and calls on different streams are independent
(include/vimscan.h): two host threads, each with its own stream, inputs,
output and workspace, call the scan at once; each result must equal the
same call made alone, bit for bit."""
import threading

import pytest
import torch

from gpu_util import say, upload
from vision_mamba_selective_amd import workloads as wlm

pytestmark = pytest.mark.gpu


def make_case(seed):
    wl = wlm.WORKLOADS[1].with_(batch=4, dim=40, seqlen=300, seed=seed)
    return wl, upload(wlm.make_inputs(wl, random_A=True, random_D=True))


def call(t, y, ws):
    import vision_mamba_selective_amd as vms
    return vms.vim_scan_bidir(t["u"], t["delta"], t["z"], t["B"], t["C"], t["A"], t["Dskip"],
                              t["dt_bias"], out=y, workspace=ws)


def test_two_threads_two_streams():
    import vision_mamba_selective_amd as vms
    cases = [make_case(s) for s in (101, 202)]
    bufs = []
    for wl, t in cases:
        y = torch.empty_like(t["u"])
        ws = torch.empty(vms.workspace_bytes(0, wl.batch, wl.dim, wl.seqlen, torch.bfloat16),
                         dtype=torch.uint8, device="cuda")
        bufs.append((y, ws))
    alone = []
    for (wl, t), (y, ws) in zip(cases, bufs):
        alone.append(call(t, y, ws).clone())
    torch.cuda.synchronize()

    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            (wl, t), (y, ws) = cases[i], bufs[i]
            with torch.cuda.stream(s):
                for _ in range(20):
                    call(t, y, ws)
            s.synchronize()
        except Exception as e:   # reported by the main thread
            errors.append(e)

    for (y, _) in bufs:
        y.fill_(float("nan"))
    torch.cuda.synchronize()
    th = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for x in th:
        x.start()
    for x in th:
        x.join()
    assert not errors, errors
    for i, (y, _) in enumerate(bufs):
        assert torch.equal(y, alone[i]), "thread %d: result differs from the call made alone" % i
    say("  two threads on two streams: both results equal the calls made alone")

