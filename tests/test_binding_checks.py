"""CPU tests of the Python binding's argument checks.

The C ABI receives only pointers and sizes, and the binding takes the sizes
from the tensors' shapes, so every tensor's dtype and shape must be checked
against those sizes before the library is called: a tensor smaller than the
sizes say would be read (or written) past its end on the device.  These
tests pass mismatched CPU tensors and check that ValueError is raised before
the library is loaded (load_library is replaced by a function that fails).
"""
import pytest

torch = pytest.importorskip("torch")

import mamba_selective_scan_ssm_amd as ssm  # noqa: E402


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def refuse(*a, **k):
        raise AssertionError("the library was reached before the argument checks")
    monkeypatch.setattr(ssm, "load_library", refuse)
    monkeypatch.setattr(ssm, "get_handle", refuse)


def mamba1(dtype=torch.bfloat16, b=2, d=8, n=4, L=16, groups=None):
    f32 = torch.float32
    bc = (b, n, L) if groups is None else (b, groups, n, L)
    t = dict(u=torch.zeros(b, d, L, dtype=dtype), delta=torch.zeros(b, d, L, dtype=dtype),
             A=torch.zeros(d, n, dtype=f32), B=torch.zeros(bc, dtype=dtype),
             C=torch.zeros(bc, dtype=dtype), D=torch.zeros(d, dtype=f32),
             z=torch.zeros(b, d, L, dtype=dtype), delta_bias=torch.zeros(d, dtype=f32),
             y=torch.zeros(b, d, L, dtype=dtype), last_state=torch.zeros(b, d, n, dtype=f32))
    return t


def call_fwd(t):
    ssm.ssm_selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                               t["delta_bias"], True, t["y"], t["last_state"])


def test_well_formed_call_reaches_the_device_check():
    with pytest.raises(ValueError, match="device tensor"):
        call_fwd(mamba1())


@pytest.mark.parametrize("name,bad", [
    ("delta", lambda t: t["delta"].float()),             # fp32 delta with bf16 u
    ("A", lambda t: t["A"].bfloat16()),                  # A must be float32
    ("B", lambda t: t["B"][:, :3].contiguous()),         # fewer states than A
    ("C", lambda t: t["C"][..., :8].contiguous()),       # shorter than seqlen
    ("z", lambda t: t["z"][:1].contiguous()),            # wrong batch
    ("D", lambda t: t["D"].bfloat16()),
    ("delta_bias", lambda t: t["delta_bias"][:4].contiguous()),
    ("y", lambda t: t["y"].float()),                     # output dtype
    ("last_state", lambda t: t["last_state"][:, :, :2].contiguous()),
])
def test_mamba1_mismatch_rejected(name, bad):
    t = mamba1()
    t[name] = bad(t)
    with pytest.raises(ValueError, match=name):
        call_fwd(t)


def test_mamba1_unsupported_dtype():
    t = mamba1()
    for k in ("u", "delta", "z", "y", "B", "C"):
        t[k] = t[k].half()
    with pytest.raises(ValueError, match="float32 or bfloat16"):
        call_fwd(t)


def test_grouped_layout_and_divisibility():
    t = mamba1(groups=3, d=8)  # 3 groups do not divide 8 channels
    with pytest.raises(ValueError, match="ngroups"):
        ssm.ssm_selective_scan_fwd_grouped(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"],
                                           t["z"], t["delta_bias"], True, None, t["y"],
                                           t["last_state"])
    t = mamba1()  # three-dimensional B through the grouped entry point
    with pytest.raises(ValueError, match="ngroups"):
        ssm.ssm_selective_scan_fwd_grouped(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"],
                                           t["z"], t["delta_bias"], True, None, t["y"],
                                           t["last_state"])


def test_initial_state_shape():
    t = mamba1()
    h0 = torch.zeros(2, 8, 3)
    with pytest.raises(ValueError, match="initial_state"):
        ssm.ssm_selective_scan_fwd_with_state(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"],
                                              t["z"], t["delta_bias"], True, h0, t["y"],
                                              t["last_state"])


def test_workspace_dtype():
    t = mamba1()
    ws = torch.zeros(16, dtype=torch.float32)
    with pytest.raises(ValueError, match="workspace"):
        ssm.ssm_selective_scan_fwd_ws(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                                      t["delta_bias"], True, None, t["y"], t["last_state"], ws)


def test_state_update_checks():
    f32 = torch.float32
    b, d, n = 2, 8, 4
    args = dict(state=torch.zeros(b, d, n), u=torch.zeros(b, d), delta=torch.zeros(b, d),
                A=torch.zeros(d, n), B=torch.zeros(b, n), C=torch.zeros(b, n),
                D=torch.zeros(d), z=torch.zeros(b, d), delta_bias=torch.zeros(d),
                y=torch.zeros(b, d))

    def call(a):
        ssm.ssm_selective_state_update(a["state"], a["u"], a["delta"], a["A"], a["B"], a["C"],
                                       a["D"], a["z"], a["delta_bias"], True, a["y"])
    with pytest.raises(ValueError, match="device tensor"):
        call(args)
    for k, v in (("state", torch.zeros(b, d, n - 1)), ("B", torch.zeros(b, n + 1)),
                 ("delta", torch.zeros(b, d, dtype=torch.bfloat16)),
                 ("A", torch.zeros(d, n, dtype=torch.float64))):
        a = dict(args, **{k: v})
        with pytest.raises(ValueError, match=k):
            call(a)
    assert args["state"].dtype == f32


def ssd(b=1, L=64, h=4, p=8, n=16, g=2, dtype=torch.bfloat16):
    f32 = torch.float32
    return dict(x=torch.zeros(b, L, h, p, dtype=dtype), dt=torch.zeros(b, L, h, dtype=dtype),
                A=torch.zeros(h, dtype=f32), B=torch.zeros(b, L, g, n, dtype=dtype),
                C=torch.zeros(b, L, g, n, dtype=dtype), D=torch.zeros(h, dtype=f32),
                dt_bias=torch.zeros(h, dtype=f32), y=torch.zeros(b, L, h, p, dtype=dtype),
                final_state=torch.zeros(b, h, p, n, dtype=f32),
                ws=torch.zeros(256, dtype=torch.uint8))


def call_ssd(t):
    ssm.ssd_chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["dt_bias"], True,
                           t["y"], t["final_state"], t["ws"], 64)


def test_ssd_well_formed_call_reaches_the_device_check():
    with pytest.raises(ValueError, match="device tensor"):
        call_ssd(ssd())


@pytest.mark.parametrize("name,bad", [
    ("dt", lambda t: t["dt"].float()),                   # fp32 dt with bf16 x
    ("A", lambda t: t["A"][:3].contiguous()),
    ("C", lambda t: t["C"][:, :, :1].contiguous()),      # groups differ from B
    ("D", lambda t: t["D"].double()),
    ("y", lambda t: t["y"][:, :32].contiguous()),
    ("final_state", lambda t: t["final_state"][..., :8].contiguous()),
    ("workspace", lambda t: t["ws"].float()),
])
def test_ssd_mismatch_rejected(name, bad):
    t = ssd()
    key = "ws" if name == "workspace" else name
    t[key] = bad(t)
    with pytest.raises(ValueError, match=name):
        call_ssd(t)


def test_backward_checks():
    t = mamba1(dtype=torch.float32)
    b, d, L = t["u"].shape
    n = t["A"].shape[1]
    f32 = torch.float32
    g = dict(dy=torch.zeros(b, d, L), du=torch.zeros(b, d, L), ddelta=torch.zeros(b, d, L),
             dA=torch.zeros(d, n), dB=torch.zeros(b, n, L), dC=torch.zeros(b, n, L),
             dD=torch.zeros(d), dz=torch.zeros(b, d, L), ddelta_bias=torch.zeros(d),
             ws=torch.zeros(64, dtype=torch.uint8))

    def call(gg):
        ssm.ssm_selective_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                                   t["delta_bias"], True, None, gg["dy"], None, gg["du"],
                                   gg["ddelta"], gg["dA"], gg["dB"], gg["dC"], gg["dD"], gg["dz"],
                                   gg["ddelta_bias"], None, gg["ws"])
    with pytest.raises(ValueError, match="device tensor"):
        call(g)
    for k, v in (("dB", torch.zeros(b, n, L - 1)), ("dA", torch.zeros(d, n, dtype=torch.bfloat16)),
                 ("dy", torch.zeros(b, d, L, dtype=torch.bfloat16)), ("dz", None)):
        with pytest.raises(ValueError, match=k):
            call(dict(g, **{k: v}))
    assert g["dA"].dtype == f32
