"""GPU parity of the chunked (SSD) scan on seeded random shapes:
ssd_chunk_scan_fwd (and its initial-state form) against the fp64
sequential oracle, every y and final_state entry.

Cases are drawn once from a fixed seed over the boundary's limits: headdim
1..128 and dstate 1..256 (tile sizes and the zero-padded sizes between
them), chunk 64 / 128 / 256, one or several groups, ragged sequence
lengths, softplus on and off, with and without an initial state.
Tolerance as in test_gpu_ssd.py (2e-2 relative, bf16 inputs).
"""
import numpy as np
import pytest

import oracle
import synth
from test_gpu_ssd import check

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

HEADDIMS = (1, 7, 16, 32, 33, 64, 80, 100, 128)
DSTATES = (1, 5, 16, 32, 48, 64, 100, 128, 200, 256)
SEQLENS = (1, 17, 64, 65, 200, 256, 257, 700)
MAX_WORK = 40_000_000  # batch * seqlen * nheads * headdim * dstate (oracle time)


def draw_cases(n_cases, seed=20261205):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n_cases:
        b = int(rng.integers(1, 4))
        L = int(rng.choice(SEQLENS))
        g = int(rng.choice((1, 1, 2, 3)))
        h = g * int(rng.integers(1, 4))
        p = int(rng.choice(HEADDIMS))
        n = int(rng.choice(DSTATES))
        if b * L * h * p * n > MAX_WORK:
            continue
        cases.append(dict(shape=(b, L, h, p, n, g), chunk=int(rng.choice((64, 128, 256))),
                          softplus=bool(rng.integers(0, 4) > 0),
                          h0=bool(rng.integers(0, 3) == 0), seed=int(rng.integers(0, 1 << 30))))
    return cases


CASES = draw_cases(32)


def case_id(c):
    b, L, h, p, n, g = c["shape"]
    return (f"b{b}L{L}h{h}P{p}N{n}g{g}Q{c['chunk']}{'' if c['softplus'] else '-nosp'}"
            f"{'-h0' if c['h0'] else ''}")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mamba_selective_scan_ssm_amd as ssm
    ssm.load_library()
    return ssm


@pytest.mark.parametrize("case", CASES, ids=[case_id(c) for c in CASES])
def test_random_ssd_case(lib, case):
    b, L, h, p, n, g = case["shape"]
    print(f"case random ssd {case_id(case)} seed={case['seed']}", flush=True)
    s = synth.ssd_inputs(synth.SSD_CONFIGS["ssd"], seed=case["seed"], batch=b, seqlen=L,
                         nheads=h, headdim=p, dstate=n, ngroups=g)
    if not case["softplus"]:
        # dt is then the step size as given: keep it positive, as softplus would
        s["dt"] = synth.round_bf16(np.abs(s["dt"]).astype(np.float32))
        s["dt_bias"] = None
    h0 = (np.random.default_rng(case["seed"] + 1).standard_normal((b, h, p, n)).astype(np.float32)
          if case["h0"] else None)
    dev = "cuda"
    t = {k: (None if v is None else
             synth.to_device(v, "bf16" if k in ("x", "dt", "B", "C") else "f32", dev))
         for k, v in s.items()}
    y, fs = lib.ssd_chunk_scan(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"],
                               dt_bias=t["dt_bias"], dt_softplus=case["softplus"],
                               chunk_size=case["chunk"],
                               initial_state=None if h0 is None else torch.from_numpy(h0).to(dev))
    torch.cuda.synchronize()
    ry, rf = oracle.ssd_scan(**s, dt_softplus=case["softplus"],
                             initial_state=None if h0 is None else h0.astype(np.float64))
    check("y", synth.to_host_f64(y), ry)
    check("final_state", synth.to_host_f64(fs), rf)
