"""GPU parity: ssd_chunk_scan_fwd (Mamba-2 chunked form, HIP through the C
ABI) against the fp64 sequential oracle on the same seeded inputs.

bf16 inputs; tolerance per element |gpu - ref| <= 2e-2 * (|ref| + rms(ref))
and norm-wise relative error <= 2e-2, for y and final_state.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REL = 2e-2


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mamba_selective_scan_ssm_amd as ssm
    ssm.load_library()
    return ssm


def check(name, got, ref):
    got = np.asarray(got, np.float64).reshape(ref.shape)
    err = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    rel_l2 = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    worst = float((err / (REL * (np.abs(ref) + rms))).max())
    print(f"  {name}: max_abs={err.max():.3e} max|ref|={np.abs(ref).max():.3e} rms={rms:.3e} "
          f"rel_l2={rel_l2:.3e} worst/bound={worst:.3f}", flush=True)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    assert worst <= 1.0, f"{name}: element error {worst:.3f}x the bound"
    assert rel_l2 <= REL, f"{name}: relative L2 error {rel_l2:.3e}"


def run(ssm, s, chunk, softplus=True):
    dev = "cuda"
    t = {k: (None if v is None else
             synth.to_device(v, "bf16" if k in ("x", "dt", "B", "C") else "f32", dev))
         for k, v in s.items()}
    y, fs = ssm.ssd_chunk_scan(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"],
                               dt_bias=t["dt_bias"], dt_softplus=softplus, chunk_size=chunk)
    torch.cuda.synchronize()
    return synth.to_host_f64(y), synth.to_host_f64(fs)


def compare(ssm, s, chunk, label, softplus=True):
    print(f"case {label}", flush=True)
    yg, fg = run(ssm, s, chunk, softplus)
    ry, rf = oracle.ssd_scan(**s, dt_softplus=softplus)
    check("y", yg, ry)
    check("final_state", fg, rf)


CASES = [  # (batch, seqlen, nheads, headdim, dstate, ngroups, chunk)
    (1, 64, 2, 32, 32, 1, 64),
    (2, 300, 4, 64, 64, 2, 128),
    (1, 256, 3, 128, 128, 1, 256),
    (2, 1000, 2, 64, 256, 1, 64),
    (1, 777, 6, 64, 128, 3, 256),
    (3, 129, 2, 32, 128, 2, 64),
    (2, 4096, 32, 32, 64, 1, 256),   # several heads per workgroup
    (1, 2048, 16, 64, 128, 2, 128),
    (1, 300, 2, 128, 256, 1, 128),   # the largest head and state (documented limits)
    (2, 200, 4, 32, 256, 2, 64),
    (1, 513, 2, 128, 32, 1, 256),
]


@pytest.mark.parametrize("case", CASES)
def test_ssd_shapes(lib, case):
    b, L, h, p, n, g, q = case
    s = synth.ssd_inputs(synth.SSD_CONFIGS["ssd"], seed=50 + L, batch=b, seqlen=L, nheads=h,
                         headdim=p, dstate=n, ngroups=g)
    compare(lib, s, q, f"ssd {case}")


ODD = [  # (batch, seqlen, nheads, headdim, dstate, ngroups, chunk): sizes between the tiles
    (1, 200, 2, 64, 16, 1, 64),      # dstate 16 -> tile 32
    (2, 300, 4, 32, 48, 2, 128),     # dstate 48 -> 64, two groups
    (1, 513, 3, 64, 100, 1, 256),    # dstate 100 -> 128, ragged tail
    (2, 130, 2, 16, 128, 1, 64),     # headdim 16 -> 32
    (1, 260, 2, 80, 64, 2, 128),     # headdim 80 -> 128
    (1, 77, 3, 1, 1, 3, 64),         # headdim 1, dstate 1, one head per group
    (1, 400, 2, 100, 200, 1, 128),   # headdim 100 -> 128, dstate 200 -> 256
]


@pytest.mark.parametrize("case", ODD)
def test_ssd_odd_sizes(lib, case):
    """headdim 1..128 and dstate 1..256 off the tile sizes (zero-padded
    copies in the workspace): every y and final_state entry."""
    b, L, h, p, n, g, q = case
    s = synth.ssd_inputs(synth.SSD_CONFIGS["ssd"], seed=60 + L + p + n, batch=b, seqlen=L,
                         nheads=h, headdim=p, dstate=n, ngroups=g)
    compare(lib, s, q, f"ssd odd sizes {case}")


def test_ssd_odd_sizes_initial_state_in_place(lib):
    """An off-tile shape from a given state, updated in place."""
    b, L, h, p, n, g, q = 2, 300, 4, 48, 40, 2, 128
    print("case ssd odd sizes, initial state in place", flush=True)
    s = synth.ssd_inputs(synth.SSD_CONFIGS["ssd"], seed=71, batch=b, seqlen=L, nheads=h,
                         headdim=p, dstate=n, ngroups=g)
    init = np.random.default_rng(72).standard_normal((b, h, p, n)).astype(np.float32)
    dev = "cuda"
    t = {k: (None if v is None else
             synth.to_device(v, "bf16" if k in ("x", "dt", "B", "C") else "f32", dev))
         for k, v in s.items()}
    state = torch.from_numpy(init).to(dev)
    y = torch.empty_like(t["x"])
    ws = torch.empty(lib.ssd_chunk_scan_workspace_size(b, L, h, p, n, g, q), dtype=torch.uint8,
                     device=dev)
    lib.ssd_chunk_scan_fwd_with_state(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"],
                                      t["dt_bias"], True, state, y, state, ws, q)
    torch.cuda.synchronize()
    ry, rf = oracle.ssd_scan(**s, initial_state=init.astype(np.float64))
    check("y", synth.to_host_f64(y), ry)
    check("final_state", synth.to_host_f64(state), rf)


def test_ssd_nullable_and_softplus_off(lib):
    s = synth.ssd_inputs(synth.SSD_CONFIGS["ssd"], seed=7, batch=2, seqlen=200, nheads=2,
                         headdim=64, dstate=64, ngroups=1)
    s["D"] = None
    s["dt_bias"] = None
    s["dt"] = np.abs(s["dt"]).astype(np.float32) * np.float32(0.05)
    s["dt"] = synth.round_bf16(s["dt"])
    compare(lib, s, 64, "no D, no bias, softplus off", softplus=False)


def test_ssd_config_full(lib):
    """The SSD workload (batch 4, seqlen 4096, 24 heads, headdim 64, dstate
    128, 1 group, chunk 256): every y and final_state entry."""
    cfg = synth.SSD_CONFIGS["ssd"]
    compare(lib, synth.ssd_inputs(cfg, seed=4), cfg.chunk, "ssd full")


def test_ssd_repeatable(lib):
    s = synth.ssd_inputs(synth.SSD_CONFIGS["ssd"], seed=9, batch=1, seqlen=512, nheads=4,
                         headdim=64, dstate=128, ngroups=1)
    y1, f1 = run(lib, s, 256)
    y2, f2 = run(lib, s, 256)
    assert np.array_equal(y1, y2) and np.array_equal(f1, f2)


@pytest.mark.parametrize("case", [(2, 300, 4, 64, 64, 2, 128), (1, 512, 6, 64, 128, 1, 256),
                                  (2, 200, 2, 32, 32, 1, 64),
                                  (1, 300, 3, 128, 128, 1, 128),  # heads run as two of 64
                                  (2, 260, 2, 128, 256, 2, 256),  # ... as four of 32
                                  (1, 200, 2, 64, 256, 1, 64)])   # ... as two of 32
def test_ssd_initial_state(lib, case):
    """S starts at a given state; every y and final_state entry.  Heads wider
    than the kernels' tiles are split into narrower heads, the initial and
    final states included."""
    b, L, h, p, n, g, q = case
    print(f"case ssd initial state {case}", flush=True)
    s = synth.ssd_inputs(synth.SSD_CONFIGS["ssd"], seed=80 + L, batch=b, seqlen=L, nheads=h,
                         headdim=p, dstate=n, ngroups=g)
    init = np.random.default_rng(L).standard_normal((b, h, p, n)).astype(np.float32)
    dev = "cuda"
    t = {k: (None if v is None else
             synth.to_device(v, "bf16" if k in ("x", "dt", "B", "C") else "f32", dev))
         for k, v in s.items()}
    y, fs = lib.ssd_chunk_scan(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"],
                               dt_bias=t["dt_bias"], chunk_size=q,
                               initial_state=torch.from_numpy(init).to(dev))
    torch.cuda.synchronize()
    ry, rf = oracle.ssd_scan(**s, initial_state=init.astype(np.float64))
    check("y", synth.to_host_f64(y), ry)
    check("final_state", synth.to_host_f64(fs), rf)


@pytest.mark.parametrize("k", [256, 300])
def test_ssd_scan_in_pieces(lib, k):
    """Two calls, the second from the first's final_state (updated in place),
    match the oracle's single scan; cut at a chunk boundary and inside a chunk."""
    b, L, h, p, n, g, q = 1, 600, 4, 64, 128, 1, 256
    print(f"case ssd pieces k={k}", flush=True)
    s = synth.ssd_inputs(synth.SSD_CONFIGS["ssd"], seed=90, batch=b, seqlen=L, nheads=h,
                         headdim=p, dstate=n, ngroups=g)
    dev = "cuda"
    t = {kk: (None if v is None else
              synth.to_device(v, "bf16" if kk in ("x", "dt", "B", "C") else "f32", dev))
         for kk, v in s.items()}
    state = torch.empty((b, h, p, n), dtype=torch.float32, device=dev)
    ys = []
    for i, (t0, t1) in enumerate(((0, k), (k, L))):
        part = {kk: (v[:, t0:t1].contiguous() if kk in ("x", "dt", "B", "C") else v)
                for kk, v in t.items()}
        yp = torch.empty_like(part["x"])
        nb = lib.ssd_chunk_scan_workspace_size(b, t1 - t0, h, p, n, g, q)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        lib.ssd_chunk_scan_fwd_with_state(part["x"], part["dt"], part["A"], part["B"], part["C"],
                                          part["D"], part["dt_bias"], True,
                                          state if i else None, yp, state, ws, q)
        ys.append(yp)
    torch.cuda.synchronize()
    y = torch.cat(ys, dim=1)
    ry, rf = oracle.ssd_scan(**s)
    check("y", synth.to_host_f64(y), ry)
    check("final_state", synth.to_host_f64(state), rf)


# ---------------------------------------------------------------------------
# Decode step (ssd_state_update)
# ---------------------------------------------------------------------------

def step_inputs(s, t):
    """Token t of a sequence in the decode layouts."""
    return {"x": s["x"][:, t], "dt": s["dt"][:, t], "B": s["B"][:, t], "C": s["C"][:, t]}


@pytest.mark.parametrize("shape,dtype", [
    ((2, 4, 64, 128, 2), "bf16"), ((2, 4, 64, 128, 2), "f32"), ((1, 3, 32, 30, 1), "f32"),
    ((1, 2, 128, 256, 1), "bf16"), ((3, 6, 16, 5, 3), "f32")])
def test_ssd_state_update_one_step(lib, shape, dtype):
    """One token from a given state equals the oracle's scan of a one-token
    sequence started from that state: y and the new state."""
    b, h, p, n, g = shape
    print(f"case ssd step {shape} {dtype}", flush=True)
    s = synth.ssd_inputs(synth.SSD_CONFIGS["ssd"], seed=120 + n, batch=b, seqlen=1, nheads=h,
                         headdim=p, dstate=n, ngroups=g)
    if dtype == "f32":
        s = {k: (None if v is None else np.asarray(v, np.float32)) for k, v in s.items()}
    init = np.random.default_rng(n).standard_normal((b, h, p, n)).astype(np.float32)
    dev = "cuda"
    one = step_inputs(s, 0)
    t = {k: synth.to_device(v, dtype, dev) for k, v in one.items()}
    f = {k: (None if s[k] is None else synth.to_device(s[k], "f32", dev))
         for k in ("A", "D", "dt_bias")}
    state = torch.from_numpy(init).to(dev)
    y = torch.empty_like(t["x"])
    lib.ssd_state_update(state, t["x"], t["dt"], f["A"], t["B"], t["C"], f["D"], f["dt_bias"],
                         True, y)
    torch.cuda.synchronize()
    ry, rf = oracle.ssd_scan(**s, initial_state=init.astype(np.float64))
    check("y", synth.to_host_f64(y), ry[:, 0])
    check("state", synth.to_host_f64(state), rf)


def test_ssd_decode_loop_matches_scan(lib):
    """48 tokens decoded one at a time from a zero state: every token's y and
    the final state against the oracle's scan of the whole sequence."""
    b, L, h, p, n, g = 2, 48, 4, 64, 128, 1
    print("case ssd decode loop", flush=True)
    s = synth.ssd_inputs(synth.SSD_CONFIGS["ssd"], seed=131, batch=b, seqlen=L, nheads=h,
                         headdim=p, dstate=n, ngroups=g)
    dev = "cuda"
    f = {k: (None if s[k] is None else synth.to_device(s[k], "f32", dev))
         for k in ("A", "D", "dt_bias")}
    state = torch.zeros((b, h, p, n), dtype=torch.float32, device=dev)
    ys = []
    for tt in range(L):
        t = {k: synth.to_device(np.ascontiguousarray(v), "bf16", dev)
             for k, v in step_inputs(s, tt).items()}
        y = torch.empty_like(t["x"])
        lib.ssd_state_update(state, t["x"], t["dt"], f["A"], t["B"], t["C"], f["D"],
                             f["dt_bias"], True, y)
        ys.append(y)
    torch.cuda.synchronize()
    yg = torch.stack(ys, dim=1)
    ry, rf = oracle.ssd_scan(**s)
    check("y", synth.to_host_f64(yg), ry)
    check("final_state", synth.to_host_f64(state), rf)
