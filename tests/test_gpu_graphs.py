"""HIP-graph capture of the entry points.  Each call is captured once into a
graph and replayed several times; before each replay new input values are
copied into the captured tensors, the eager call on those inputs gives the
reference, the outputs are overwritten with NaN, and unrelated eager work
runs.  Every replay must equal the eager call bit for bit: the library
enqueues only kernel launches (no allocation, no memset, no host-side state
between calls), so a captured call stays valid for new input values."""
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


def mamba1_values(seed, b, d, n, L, dtype, h0):
    cfg = synth.Mamba1Config("graph", b, d, n, L, dtype, 0.0, 0.5, delta_bias=True, gate=True,
                             use_D=True)
    x = synth.mamba1_inputs(cfg, seed=seed)
    t = {k: synth.to_device(v, dtype if k in ("u", "delta", "z", "B", "C") else "f32", "cuda")
         for k, v in x.items() if v is not None}
    rng = np.random.default_rng(seed)
    if h0:
        t["h0"] = torch.from_numpy(rng.standard_normal((b, d, n)).astype(np.float32)).cuda()
    t["dy"] = synth.to_device(synth.round_bf16(rng.standard_normal((b, d, L)).astype(np.float32))
                              if dtype == "bf16" else
                              rng.standard_normal((b, d, L)).astype(np.float32), dtype, "cuda")
    t["dlast"] = torch.from_numpy(rng.standard_normal((b, d, n)).astype(np.float32)).cuda()
    return t


def check_replays(call, inputs, outputs, new_values, replays=3):
    """Capture call() once, then for each replay: copy new input values into
    the captured tensors, run call() eagerly for the reference, overwrite the
    outputs with NaN, do unrelated eager work, replay, compare bitwise."""
    call()  # eager warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    scratch = torch.randn(512, 512, device="cuda")
    for r in range(replays):
        vals = new_values(r)
        for k, t in inputs.items():
            t.copy_(vals[k])
        call()
        torch.cuda.synchronize()
        ref = [o.clone() for o in outputs]
        for o in outputs:
            o.fill_(float("nan"))
        scratch = (scratch @ scratch).tanh_()  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outputs, ref)):
            assert torch.equal(o, e), f"replay {r}: output {i} differs from the eager call"


FWD = [  # (batch, dim, dstate, seqlen, dtype, entry): the time split, and not
    ((1, 256, 16, 2048), "f32", "ws"),       # 64 segments (workspace)
    ((2, 320, 8, 1500), "bf16", "noalloc"),  # segments in the library's scratch
    ((8, 1024, 16, 192), "bf16", "ws"),      # enough rows: no split
    ((1, 64, 40, 600), "f32", "plain"),      # 17..64 states without a workspace
]


@pytest.mark.parametrize("case", FWD)
def test_forward_graph_replays(lib, case):
    (b, d, n, L), dtype, entry = case
    print(f"case graph fwd {case}", flush=True)
    base = mamba1_values(500, b, d, n, L, dtype, h0=(entry != "plain"))
    keys = ("u", "delta", "A", "B", "C", "D", "z", "delta_bias") + (("h0",) if "h0" in base else ())
    inp = {k: base[k] for k in keys}
    y = torch.empty_like(inp["u"])
    ls = torch.empty((b, d, n), dtype=torch.float32, device="cuda")
    nb = lib.ssm_selective_scan_fwd_workspace_size(b, d, n, L)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    if entry == "ws":
        assert (nb > 0) == (b * d < 4096), "the split plan is not the one this case exercises"

    def call():
        a = (inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
             inp["delta_bias"], True)
        if entry == "ws":
            lib.ssm_selective_scan_fwd_ws(*a, inp.get("h0"), y, ls, ws if nb else None)
        elif entry == "noalloc":
            lib.ssm_selective_scan_fwd_noalloc(*a, inp.get("h0"), y, ls)
        else:
            lib.ssm_selective_scan_fwd(*a, y, ls)

    def new_values(r):
        v = mamba1_values(501 + r, b, d, n, L, dtype, h0=("h0" in inp))
        return {k: v[k] for k in inp}

    check_replays(call, inp, (y, ls), new_values)


BWD = [  # (batch, dim, dstate, seqlen, dtype)
    ((1, 128, 16, 1024), "f32"),   # split in time (few rows)
    ((4, 512, 16, 160), "bf16"),   # no split
    ((1, 64, 33, 300), "f32"),     # blocks of 16 states
]


@pytest.mark.parametrize("case", BWD)
def test_backward_graph_replays(lib, case):
    (b, d, n, L), dtype = case
    print(f"case graph bwd {case}", flush=True)
    base = mamba1_values(600, b, d, n, L, dtype, h0=True)
    keys = ("u", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0", "dy", "dlast")
    inp = {k: base[k] for k in keys}
    f32 = dict(dtype=torch.float32, device="cuda")
    du, dd, dz = (torch.empty_like(inp["u"]) for _ in range(3))
    dA = torch.empty((d, n), **f32)
    dB, dC = torch.empty((b, n, L), **f32), torch.empty((b, n, L), **f32)
    dD, dbias = torch.empty((d,), **f32), torch.empty((d,), **f32)
    dh0 = torch.empty((b, d, n), **f32)
    ws = torch.empty(lib.ssm_selective_scan_bwd_workspace_size(b, d, n, L), dtype=torch.uint8,
                     device="cuda")

    def call():
        lib.ssm_selective_scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"],
                                   inp["D"], inp["z"], inp["delta_bias"], True, inp["h0"],
                                   inp["dy"], inp["dlast"], du, dd, dA, dB, dC, dD, dz, dbias,
                                   dh0, ws)

    def new_values(r):
        v = mamba1_values(601 + r, b, d, n, L, dtype, h0=True)
        return {k: v[k] for k in inp}

    check_replays(call, inp, (du, dd, dA, dB, dC, dD, dz, dbias, dh0), new_values)


BWD_ROWS = [  # (batch, dim, dstate, seqlen, ngroups, dtype): B, C per row
    ((1, 64, 16, 1024, 64), "f32"),   # per channel, split in time
    ((2, 30, 20, 150, 10), "bf16"),   # groups of 3 channels (per-row dB, dC summed)
]


@pytest.mark.parametrize("case", BWD_ROWS)
def test_per_row_backward_graph_replays(lib, case):
    (b, d, n, L, G), dtype = case
    print(f"case graph bwd per-row {case}", flush=True)

    def values(seed):
        v = mamba1_values(seed, b, d, n, L, dtype, h0=True)
        rng = np.random.default_rng(seed + 7)
        for k in ("B", "C"):
            x = rng.standard_normal((b, G, n, L)).astype(np.float32)
            v[k] = synth.to_device(synth.round_bf16(x) if dtype == "bf16" else x, dtype, "cuda")
        return v

    base = values(800)
    keys = ("u", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0", "dy", "dlast")
    inp = {k: base[k] for k in keys}
    f32 = dict(dtype=torch.float32, device="cuda")
    du, dd, dz = (torch.empty_like(inp["u"]) for _ in range(3))
    dA = torch.empty((d, n), **f32)
    dB, dC = torch.empty((b, G, n, L), **f32), torch.empty((b, G, n, L), **f32)
    dD, dbias = torch.empty((d,), **f32), torch.empty((d,), **f32)
    dh0 = torch.empty((b, d, n), **f32)
    ws = torch.empty(lib.ssm_selective_scan_bwd_grouped_workspace_size(b, d, n, L, G),
                     dtype=torch.uint8, device="cuda")

    def call():
        lib.ssm_selective_scan_bwd_grouped(
            inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
            inp["delta_bias"], True, inp["h0"], inp["dy"], inp["dlast"], du, dd, dA, dB, dC, dD,
            dz, dbias, dh0, ws)

    def new_values(r):
        v = values(801 + r)
        return {k: v[k] for k in inp}

    check_replays(call, inp, (du, dd, dA, dB, dC, dD, dz, dbias, dh0), new_values)


SSD = [  # (batch, seqlen, heads, headdim, dstate, chunk)
    (1, 600, 4, 64, 128, 256),
    (2, 300, 2, 80, 96, 128),   # off-tile sizes: the zero-padded copies
]


@pytest.mark.parametrize("case", SSD)
def test_ssd_graph_replays(lib, case):
    b, L, h, p, n, q = case
    print(f"case graph ssd {case}", flush=True)
    cfg = synth.SSD_CONFIGS["ssd"]

    def values(seed):
        s = synth.ssd_inputs(cfg, seed=seed, batch=b, seqlen=L, nheads=h, headdim=p, dstate=n,
                             ngroups=1)
        return {k: synth.to_device(v, "bf16" if k in ("x", "dt", "B", "C") else "f32", "cuda")
                for k, v in s.items() if v is not None}

    inp = values(700)
    y = torch.empty_like(inp["x"])
    fs = torch.empty((b, h, p, n), dtype=torch.float32, device="cuda")
    ws = torch.empty(lib.ssd_chunk_scan_workspace_size(b, L, h, p, n, 1, q), dtype=torch.uint8,
                     device="cuda")

    def call():
        lib.ssd_chunk_scan_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp.get("D"),
                               inp.get("dt_bias"), True, y, fs, ws, q)

    check_replays(call, inp, (y, fs), lambda r: values(701 + r))
