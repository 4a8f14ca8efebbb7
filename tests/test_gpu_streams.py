"""One library handle used from several HIP streams at once.

The C ABI's handle is immutable after ssm_scan_create and every call only
enqueues work on the stream it is given, so calls on different streams may
overlap on the device.  This runs a row-parallel Mamba-1 scan (bf16), a
time-split Mamba-1 scan (float32, with its workspace) and an SSD call on four
streams at once, three rounds in a row, and checks every output bitwise
against the same calls run one after another on one stream (the kernels are
deterministic).
"""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mamba_selective_scan_ssm_amd as ssm
    ssm.load_library()
    return ssm


def mamba1_call(ssm, seed, b, d, n, L, dtype):
    cfg = synth.Mamba1Config("streams", b, d, n, L, dtype, 0.0, 0.5, delta_bias=True, gate=True)
    x = synth.mamba1_inputs(cfg, seed=seed)
    t = {k: (None if v is None else
             synth.to_device(v, dtype if k in ("u", "delta", "z", "B", "C") else "f32", "cuda"))
         for k, v in x.items()}

    def run():
        return ssm.selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"],
                                      z=t["z"], delta_bias=t["delta_bias"])
    return run


def ssd_call(ssm, seed):
    s = synth.ssd_inputs(synth.SSD_CONFIGS["ssd"], seed=seed, batch=2, seqlen=1024, nheads=8,
                         headdim=64, dstate=128, ngroups=1)
    t = {k: synth.to_device(v, "bf16" if k in ("x", "dt", "B", "C") else "f32", "cuda")
         for k, v in s.items()}

    def run():
        return ssm.ssd_chunk_scan(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"],
                                  dt_bias=t["dt_bias"], chunk_size=256)
    return run


def test_concurrent_streams_match_serial(lib):
    print("case four streams: mamba1 bf16 x2, mamba1 f32 time split, ssd", flush=True)
    calls = [mamba1_call(lib, 61, 4, 1024, 16, 1024, "bf16"),
             mamba1_call(lib, 62, 4, 1024, 16, 1024, "bf16"),
             mamba1_call(lib, 63, 1, 256, 16, 2048, "f32"),   # time split, workspace
             ssd_call(lib, 64)]
    torch.cuda.synchronize()
    serial = [tuple(o.clone() for o in f()) for f in calls]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in calls]
    cur = torch.cuda.current_stream()
    for s in streams:
        s.wait_stream(cur)
    for rnd in range(3):
        outs = [None] * len(calls)
        for i, (f, s) in enumerate(zip(calls, streams)):
            with torch.cuda.stream(s):
                outs[i] = f()
        torch.cuda.synchronize()
        for i, (got, ref) in enumerate(zip(outs, serial)):
            for g, r in zip(got, ref):
                assert torch.equal(g, r), f"round {rnd}: call {i} differs from its serial run"
        print(f"  round {rnd}: all {len(calls)} calls bitwise equal", flush=True)
