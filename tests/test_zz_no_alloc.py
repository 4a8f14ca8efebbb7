"""GPU test of ssm_selective_scan_fwd_noalloc (the entry point that allocates
nothing: its time-split aggregates live in the library's per-GPU scratch
array) against ssm_selective_scan_fwd_ws with a caller-allocated workspace,
through the C ABI.  Both run the same kernels with the same plan, so their
outputs must be bitwise equal; the calls are made back to back, the second
on a smaller input, so a stale scratch from the first call would show."""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 32 << 20


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mamba_selective_scan_ssm_amd as ssm
    ssm.load_library()
    return ssm


def inputs(seed, b, d, n, L, dtype, h0=False):
    cfg = synth.Mamba1Config("noalloc", b, d, n, L, dtype, 0.0, 0.5, delta_bias=True, gate=True,
                             use_D=True)
    x = synth.mamba1_inputs(cfg, seed=seed)
    t = {k: (None if v is None else synth.to_device(v, dtype if k in ("u", "delta", "z", "B", "C")
                                                     else "f32", "cuda"))
         for k, v in x.items()}
    if h0:
        t["h0"] = torch.from_numpy(
            np.random.default_rng(seed).standard_normal((b, d, n)).astype(np.float32)).cuda()
    else:
        t["h0"] = None
    return t


def args_of(t):
    return (t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], True,
            t["h0"])


def outputs(t, fill):
    b, d, _ = t["u"].shape
    n = t["A"].shape[1]
    return (torch.full_like(t["u"], fill),
            torch.full((b, d, n), fill, dtype=torch.float32, device="cuda"))


CASES = [  # two no-allocation calls in a row: the second on a smaller input
    [((1, 256, 16, 2048), "f32", False), ((1, 64, 8, 700), "bf16", False)],
    [((2, 1536, 16, 2048), "f32", True), ((1, 40, 64, 500), "bf16", True)],
    [((8, 4096, 16, 64), "bf16", False), ((1, 130, 3, 1000), "bf16", False)],
]


@pytest.mark.parametrize("pair", CASES)
def test_noalloc_matches_workspace_entry(lib, pair):
    ins, refs, sizes = [], [], []
    for i, ((b, d, n, L), dtype, h0) in enumerate(pair):
        t = inputs(500 + 7 * i + n, b, d, n, L, dtype, h0)
        nbytes = lib.ssm_selective_scan_fwd_workspace_size(b, d, n, L)
        print(f"case noalloc call {i}: {(b, d, n, L)} {dtype} h0={h0}, "
              f"time-split workspace {nbytes} bytes", flush=True)
        assert nbytes <= SCRATCH_BYTES
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda") if nbytes else None
        y0, s0 = outputs(t, 0.0)
        lib.ssm_selective_scan_fwd_ws(*args_of(t), y0, s0, ws)
        ins.append(t)
        refs.append((y0, s0))
        sizes.append(t["u"].numel())
    assert sizes[1] < sizes[0]
    torch.cuda.synchronize()
    # the two no-allocation calls back to back on the current stream
    got = []
    for t in ins:
        y1, s1 = outputs(t, float("nan"))
        lib.ssm_selective_scan_fwd_noalloc(*args_of(t), y1, s1)
        got.append((y1, s1))
    torch.cuda.synchronize()
    for i, ((y0, s0), (y1, s1)) in enumerate(zip(refs, got)):
        assert torch.equal(y0, y1), f"call {i}: y differs from the workspace entry point"
        assert torch.equal(s0, s1), f"call {i}: last_state differs from the workspace entry point"


def test_noalloc_matches_workspace_entry_per_row(lib):
    """B, C per channel (the per-row kernels, cut in time): two no-allocation
    calls in a row, the second smaller, against the workspace entry point."""
    cases = [((1, 256, 16, 2048), "f32"), ((1, 40, 48, 700), "bf16")]
    ins, refs = [], []
    for i, ((b, d, n, L), dtype) in enumerate(cases):
        t = inputs(900 + i, b, d, n, L, dtype)
        rng = np.random.default_rng(901 + i)
        for k in ("B", "C"):
            v = rng.standard_normal((b, d, n, L)).astype(np.float32)
            t[k] = synth.to_device(synth.round_bf16(v) if dtype == "bf16" else v, dtype, "cuda")
        nbytes = lib.ssm_selective_scan_fwd_workspace_size(b, d, n, L, ngroups=d)
        print(f"case noalloc per channel call {i}: {(b, d, n, L)} {dtype}, "
              f"time-split workspace {nbytes} bytes", flush=True)
        assert 0 < nbytes <= SCRATCH_BYTES
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        y0, s0 = outputs(t, 0.0)
        lib.ssm_selective_scan_fwd_ws(*args_of(t), y0, s0, ws)
        ins.append(t)
        refs.append((y0, s0))
    torch.cuda.synchronize()
    got = []
    for t in ins:
        y1, s1 = outputs(t, float("nan"))
        lib.ssm_selective_scan_fwd_noalloc(*args_of(t), y1, s1)
        got.append((y1, s1))
    torch.cuda.synchronize()
    for i, ((y0, s0), (y1, s1)) in enumerate(zip(refs, got)):
        assert torch.equal(y0, y1), f"call {i}: y differs from the workspace entry point"
        assert torch.equal(s0, s1), f"call {i}: last_state differs from the workspace entry point"


def test_scratch_holds_every_plan(lib):
    """The real planner's workspace for a sweep of shapes fits the scratch,
    shared B, C and per row (one group per channel, groups of 3 channels)."""
    worst = 0
    for n in (1, 4, 8, 16, 33, 64):
        for b in (1, 2, 3, 16):
            for d in (1, 64, 66, 256, 1002, 1536, 4098):
                for L in (128, 1000, 4096, 1 << 20):
                    for g in (1, d, d // 3 if d % 3 == 0 else 1):
                        worst = max(worst, lib.ssm_selective_scan_fwd_workspace_size(
                            b, d, n, L, ngroups=g))
    print(f"  largest planned workspace {worst} bytes", flush=True)
    assert 0 < worst <= SCRATCH_BYTES
