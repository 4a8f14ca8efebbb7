"""GPU parity of the backward pass on seeded random shapes and options:
ssm_selective_scan_bwd / ssm_selective_scan_bwd_grouped (through the
allocating binding) against the fp64 oracle's backward, every gradient.

Cases are drawn once from a fixed seed: sizes across the kernels' tile
edges, every dstate tier (1..64), one group, whole-workgroup groups, small
groups and per-channel B, C (the shared-B/C and the per-row kernels), both
dtypes, gate / bias / softplus on and off, initial state and dlast on and
off, batches small enough for the time split.  Tolerances as in
test_gpu_bwd.py (1e-4 float32, 2e-2 bf16, relative to each gradient's
size).
"""
import numpy as np
import pytest

from test_gpu_bwd import compare, run_case

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DIMS = (1, 5, 16, 33, 64, 100, 128, 192, 256, 320)
SEQLENS = (1, 7, 16, 31, 32, 33, 64, 100, 257, 700, 1100)
MAX_UPDATES = 6_000_000  # batch * dim * seqlen * dstate per case (oracle time)


def draw_cases(n_cases, seed=20261204):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n_cases:
        b = int(rng.integers(1, 4))
        d = int(rng.choice(DIMS))
        lo, hi = ((1, 4), (5, 8), (9, 16), (9, 16), (17, 32), (33, 64))[int(rng.integers(0, 6))]
        n = int(rng.integers(lo, hi + 1))
        L = int(rng.choice(SEQLENS))
        if b * d * L * n > MAX_UPDATES:
            continue
        rpw = 256 if n <= 4 else 128 if n <= 8 else 64
        whole = [g for g in range(2, d + 1) if d % g == 0 and (d // g) % rpw == 0]
        small = [g for g in range(2, d + 1) if d % g == 0 and (d // g) % rpw != 0]
        kind = int(rng.integers(0, 4))
        if kind == 1 and whole:
            G = int(rng.choice(whole))
        elif kind == 2 and small:
            G = int(rng.choice(small))
        elif kind == 3 and d > 1:
            G = d
        else:
            G = 1
        softplus = bool(rng.integers(0, 4) > 0)
        cases.append(dict(shape=(b, d, n, L), groups=G,
                          dtype="bf16" if rng.integers(0, 2) else "f32",
                          gate=bool(rng.integers(0, 2)),
                          bias=softplus and bool(rng.integers(0, 2)),
                          softplus=softplus, h0=bool(rng.integers(0, 2)),
                          dlast=bool(rng.integers(0, 2)), seed=int(rng.integers(0, 1 << 30))))
    return cases


CASES = draw_cases(40)


def case_id(c):
    b, d, n, L = c["shape"]
    return (f"b{b}d{d}n{n}L{L}g{c['groups']}-{c['dtype']}{'-z' if c['gate'] else ''}"
            f"{'-bias' if c['bias'] else ''}{'' if c['softplus'] else '-nosp'}"
            f"{'-h0' if c['h0'] else ''}{'-dlast' if c['dlast'] else ''}")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mamba_selective_scan_ssm_amd as ssm
    ssm.load_library()
    return ssm


@pytest.mark.parametrize("case", CASES, ids=[case_id(c) for c in CASES])
def test_random_backward_case(lib, case):
    b, d, n, L = case["shape"]
    print(f"case random bwd {case_id(case)} seed={case['seed']}", flush=True)
    g, ref = run_case(lib, case["seed"], b, d, n, L, case["dtype"], case["gate"], case["bias"],
                      case["softplus"], case["h0"], case["dlast"],
                      case["groups"] if case["groups"] > 1 else 0)
    compare(g, ref, case["dtype"], case["gate"], case["bias"], case["h0"])
