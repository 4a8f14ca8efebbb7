"""C-ABI boundary tests that need no GPU: the library loads, exports every
symbol the header declares, and rejects invalid arguments before any HIP call
(the exercise spec's Definition of Done: batch=0 is invalid but must not
crash)."""
import ctypes
import os
import re

import pytest

import mamba_selective_scan_ssm_amd as ssm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_scan.h")

# Fake, 16-byte aligned, never dereferenced device addresses.
P = [0x10000000 * (i + 1) for i in range(16)]


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_\w+|ssd_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ssm.load_library()
    declared = header_functions()
    assert set(declared) == set(ssm.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    for code in (0, 1, 2, 3):
        assert ssm.status_string(code)
    assert "unknown" in ssm.status_string(99)


def scan(handle=None, u=P[0], delta=P[1], A=P[2], B=P[3], C=P[4], D=None, z=None, bias=None,
         y=P[5], ls=None, batch=2, dim=4, dstate=4, seqlen=8, dtype=ssm.SSM_F32):
    lib = ssm.load_library()
    st = lib.ssm_selective_scan_fwd(handle, u, delta, A, B, C, D, z, bias, 1, y, ls,
                                    batch, dim, dstate, seqlen, dtype, None)
    return st, ssm.ssm_last_error_message()


@pytest.mark.parametrize("field,value,word", [
    ("batch", 0, "batch"), ("batch", -3, "batch"), ("dim", 0, "dim"),
    ("seqlen", 0, "seqlen"), ("dstate", 0, "dstate")])
def test_nonpositive_sizes_rejected(field, value, word):
    st, msg = scan(**{field: value})
    assert st == ssm.SSM_ERR_INVALID_ARG
    assert word in msg


def test_limits_and_enums():
    st, msg = scan(dstate=65)
    assert st == ssm.SSM_ERR_UNSUPPORTED and "dstate" in msg
    st, msg = scan(dtype=7)
    assert st == ssm.SSM_ERR_INVALID_ARG and "dtype" in msg


@pytest.mark.parametrize("name", ["u", "delta", "A", "B", "C", "y"])
def test_required_pointers(name):
    st, msg = scan(**{name: None})
    assert st == ssm.SSM_ERR_INVALID_ARG and f"{name} is NULL" in msg


def test_misaligned_and_overlapping_pointers():
    st, msg = scan(u=P[0] + 4)
    assert st == ssm.SSM_ERR_INVALID_ARG and "aligned" in msg
    st, msg = scan(y=P[0])          # y aliases u
    assert st == ssm.SSM_ERR_INVALID_ARG and "overlaps" in msg
    st, msg = scan(ls=P[5] + 16)    # last_state inside y
    assert st == ssm.SSM_ERR_INVALID_ARG and "overlap" in msg


def test_null_handle_is_last_check():
    st, msg = scan(D=P[6], z=P[7], bias=P[8], ls=P[9])
    assert st == ssm.SSM_ERR_INVALID_ARG and "handle" in msg


def ssd_ws(batch=2, seqlen=64, nheads=4, headdim=64, dstate=32, ngroups=1, chunk=64):
    lib = ssm.load_library()
    n = ctypes.c_size_t(123)
    st = lib.ssd_chunk_scan_workspace_size(None, batch, seqlen, nheads, headdim, dstate,
                                           ngroups, chunk, ctypes.byref(n))
    return st, ssm.ssm_last_error_message(), n.value


def test_ssd_shape_checks():
    assert ssd_ws()[0] == ssm.SSM_ERR_INVALID_ARG            # valid shape, NULL handle
    assert "handle" in ssd_ws()[1]
    assert ssd_ws(nheads=6, ngroups=4)[0] == ssm.SSM_ERR_INVALID_ARG
    assert ssd_ws(chunk=100)[0] == ssm.SSM_ERR_UNSUPPORTED
    # any headdim 1..128 and dstate 1..256 (the documented limits) is valid
    for hd, ds in ((48, 32), (1, 1), (16, 100), (80, 16), (128, 256), (127, 255)):
        st, msg, _ = ssd_ws(headdim=hd, dstate=ds)
        assert st == ssm.SSM_ERR_INVALID_ARG and "handle" in msg, (hd, ds, msg)
    assert ssd_ws(headdim=129)[0] == ssm.SSM_ERR_UNSUPPORTED
    assert ssd_ws(dstate=257)[0] == ssm.SSM_ERR_UNSUPPORTED
    assert ssd_ws(batch=0)[0] == ssm.SSM_ERR_INVALID_ARG
    assert ssd_ws(batch=0)[2] == 0


def test_create_rejects_bad_arguments():
    lib = ssm.load_library()
    assert lib.ssm_scan_create(None, 0) == ssm.SSM_ERR_INVALID_ARG
    assert lib.ssm_scan_destroy(None) == ssm.SSM_OK


def scan_h0(h0, ls, y=P[5], handle=None):
    lib = ssm.load_library()
    st = lib.ssm_selective_scan_fwd_with_state(handle, P[0], P[1], P[2], P[3], P[4], None, None,
                                               None, 1, h0, y, ls, 2, 4, 4, 8, ssm.SSM_F32, None)
    return st, ssm.ssm_last_error_message()


def test_initial_state_rules():
    # in place (initial_state == last_state) passes every check up to the handle
    st, msg = scan_h0(P[9], P[9])
    assert st == ssm.SSM_ERR_INVALID_ARG and "handle" in msg
    st, msg = scan_h0(P[9], P[10])
    assert st == ssm.SSM_ERR_INVALID_ARG and "handle" in msg
    st, msg = scan_h0(P[9] + 4, P[10])       # misaligned
    assert st == ssm.SSM_ERR_INVALID_ARG and "initial_state" in msg and "aligned" in msg
    st, msg = scan_h0(P[9] + 16, P[9])       # partial overlap with last_state
    assert st == ssm.SSM_ERR_INVALID_ARG and "initial_state" in msg
    st, msg = scan_h0(P[5], P[10])           # overlaps y
    assert st == ssm.SSM_ERR_INVALID_ARG and "initial_state" in msg


def ssd_h0(init, fs):
    lib = ssm.load_library()
    st = lib.ssd_chunk_scan_fwd_with_state(None, P[0], P[1], P[2], P[3], P[4], None, None, 1,
                                           init, P[5], fs, P[6], 1 << 30, 2, 64, 4, 64, 32, 1, 64,
                                           ssm.SSM_BF16, None)
    return st, ssm.ssm_last_error_message()


def test_ssd_initial_state_rules():
    st, msg = ssd_h0(P[9], P[9])             # in place
    assert st == ssm.SSM_ERR_INVALID_ARG and "handle" in msg
    st, msg = ssd_h0(P[9] + 32, P[9])        # partial overlap with final_state
    assert st == ssm.SSM_ERR_INVALID_ARG and "initial_state" in msg
    st, msg = ssd_h0(P[9] + 8, P[10])        # misaligned
    assert st == ssm.SSM_ERR_INVALID_ARG and "aligned" in msg


def step(state=P[9], u=P[0], delta=P[1], A=P[2], B=P[3], C=P[4], y=P[5], batch=2, dim=4,
         dstate=16, dtype=ssm.SSM_F32):
    lib = ssm.load_library()
    st = lib.ssm_selective_state_update(None, state, u, delta, A, B, C, None, None, None, 1, y,
                                        batch, dim, dstate, dtype, None)
    return st, ssm.ssm_last_error_message()


def test_state_update_checks():
    st, msg = step()
    assert st == ssm.SSM_ERR_INVALID_ARG and "handle" in msg
    assert step(batch=0)[0] == ssm.SSM_ERR_INVALID_ARG
    assert step(dstate=65)[0] == ssm.SSM_ERR_UNSUPPORTED
    st, msg = step(state=None)
    assert st == ssm.SSM_ERR_INVALID_ARG and "state is NULL" in msg
    st, msg = step(state=P[5])               # state aliases y
    assert st == ssm.SSM_ERR_INVALID_ARG and "overlap" in msg
    st, msg = step(state=P[9] + 4)           # misaligned
    assert st == ssm.SSM_ERR_INVALID_ARG and "aligned" in msg


def step_grouped(ngroups, dim=4):
    lib = ssm.load_library()
    st = lib.ssm_selective_state_update_grouped(None, P[9], P[0], P[1], P[2], P[3], P[4], None,
                                                None, None, 1, P[5], 2, dim, 16, ngroups,
                                                ssm.SSM_F32, None)
    return st, ssm.ssm_last_error_message()


def test_grouped_state_update_checks():
    """ngroups must divide dim; a valid grouped call stops at the handle."""
    for g in (1, 2, 4):
        st, msg = step_grouped(g)
        assert st == ssm.SSM_ERR_INVALID_ARG and "handle" in msg, (g, msg)
    for g in (0, 3, -1):
        st, msg = step_grouped(g)
        assert st == ssm.SSM_ERR_INVALID_ARG and "ngroups" in msg, (g, msg)


def scan_grouped(ngroups, B=P[3], C=P[4], y=P[5], dim=4, seqlen=8):
    lib = ssm.load_library()
    st = lib.ssm_selective_scan_fwd_grouped(None, P[0], P[1], P[2], B, C, None, None, None, 1,
                                            None, y, None, 2, dim, 4, seqlen, ngroups,
                                            ssm.SSM_F32, None)
    return st, ssm.ssm_last_error_message()


def test_grouped_rules():
    for g in (1, 2, 4):  # divisors of dim pass every check up to the handle
        st, msg = scan_grouped(g)
        assert st == ssm.SSM_ERR_INVALID_ARG and "handle" in msg, (g, msg)
    for g in (0, -1, 3, 8):
        st, msg = scan_grouped(g)
        assert st == ssm.SSM_ERR_INVALID_ARG and "ngroups" in msg, (g, msg)
    # B spans batch * ngroups * dstate * seqlen elements: with 4 groups of
    # 4 states, B (2*4*4*8 floats = 1 KiB) reaches an output 512 bytes on
    st, msg = scan_grouped(4, y=P[3] + 512)
    assert st == ssm.SSM_ERR_INVALID_ARG and "overlap" in msg, msg
    st, msg = scan_grouped(1, y=P[3] + 512)  # one group: 512 bytes, no overlap
    assert st == ssm.SSM_ERR_INVALID_ARG and "handle" in msg, msg


def ssd_step(batch=2, nheads=4, headdim=8, dstate=16, ngroups=2, state=P[9], y=P[10], x=P[0]):
    lib = ssm.load_library()
    st = lib.ssd_state_update(None, state, x, P[1], P[2], P[3], P[4], None, None, 1, y,
                              batch, nheads, headdim, dstate, ngroups, ssm.SSM_F32, None)
    return st, ssm.ssm_last_error_message()


def test_ssd_state_update_rules():
    st, msg = ssd_step()
    assert st == ssm.SSM_ERR_INVALID_ARG and "handle" in msg, msg
    for kw in ({"batch": 0}, {"nheads": -1}, {"headdim": 0}, {"dstate": 0}, {"ngroups": 0}):
        st, msg = ssd_step(**kw)
        assert st == ssm.SSM_ERR_INVALID_ARG and "sizes" in msg, (kw, msg)
    st, msg = ssd_step(ngroups=3)
    assert st == ssm.SSM_ERR_INVALID_ARG and "ngroups" in msg, msg
    st, msg = ssd_step(dstate=257)
    assert st == ssm.SSM_ERR_UNSUPPORTED and "dstate" in msg, msg
    st, msg = ssd_step(state=None)
    assert st == ssm.SSM_ERR_INVALID_ARG and "state" in msg, msg
    st, msg = ssd_step(y=P[0] + 16)  # overlaps x
    assert st == ssm.SSM_ERR_INVALID_ARG and "overlap" in msg, msg
    st, msg = ssd_step(state=P[9] + 4)
    assert st == ssm.SSM_ERR_INVALID_ARG and "aligned" in msg, msg


def test_noalloc_entry_checks_arguments_before_the_handle():
    lib = ssm.load_library()
    st = lib.ssm_selective_scan_fwd_noalloc(None, P[0], P[1], P[2], P[3], P[4], None, None, None,
                                            1, None, P[5], None, 0, 4, 4, 8, 1, ssm.SSM_F32,
                                            None)
    assert st == ssm.SSM_ERR_INVALID_ARG and "batch" in ssm.ssm_last_error_message()
    st = lib.ssm_selective_scan_fwd_noalloc(None, P[0], P[1], P[2], P[3], P[4], None, None, None,
                                            1, None, P[5], None, 2, 4, 4, 8, 1, ssm.SSM_F32,
                                            None)
    assert st == ssm.SSM_ERR_INVALID_ARG and "handle" in ssm.ssm_last_error_message()


def test_noalloc_scratch_bound_covers_every_plan():
    """The scratch of the no-allocation entry point (32 MiB) holds the
    aggregates of every time-split plan on a 256-CU device: the planner's
    rule replayed here over a sweep of shapes (split only below 4 waves per
    CU, at most ceil(12 CUs / waves) and 64 segments, segments of whole
    chunks)."""
    import math
    cus, limit = 256, 32 << 20
    worst = 0
    for dstate in (1, 4, 5, 8, 9, 16, 17, 33, 64):
        lpc = 1 if dstate <= 4 else 2 if dstate <= 8 else 4
        T = 16 if dstate <= 4 else 32
        rpb = 256 // lpc
        for batch in (1, 2, 3, 7, 16, 64):
            for dim in (1, 63, 64, 65, 200, 256, 1000, 1536, 4095, 4096, 16384):
                waves = batch * math.ceil(dim / rpb) * 4
                if waves >= 4 * cus:
                    continue
                for seqlen in (8 * T, 1000, 4096, 1 << 20):
                    chunks = math.ceil(seqlen / T)
                    if chunks < 8:
                        continue
                    want = min(math.ceil(12 * cus / waves), chunks, 64)
                    if want <= 1:
                        continue
                    seg_len = math.ceil(math.ceil(seqlen / want) / T) * T
                    nseg = math.ceil(seqlen / seg_len)
                    if nseg <= 1:
                        continue
                    worst = max(worst, (nseg - 1) * batch * dim * dstate * 8)
    assert 0 < worst < limit, worst


def bwd_grouped(ngroups, dim=256, dstate=16, handle=None, dB=P[13]):
    lib = ssm.load_library()
    st = lib.ssm_selective_scan_bwd_grouped(
        handle, P[0], P[1], P[2], P[3], P[4], None, None, None, 1, None, P[5], None,
        P[6], P[7], P[8], dB, P[9], None, None, None, None, P[10], 1 << 20,
        2, dim, dstate, 8, ngroups, ssm.SSM_F32, None)
    return st, ssm.ssm_last_error_message()


def test_grouped_backward_rules():
    """Groups must divide dim; any such group count is accepted: whole
    workgroups of the shared-B/C kernels (64 channels at dstate 9..64, 128 at
    5..8, 256 at 1..4), or the per-row kernels for smaller groups down to one
    channel.  (Without a handle every valid call stops at the handle check.)"""
    for g, dim, n in ((1, 256, 16), (2, 256, 16), (4, 256, 16), (2, 256, 8), (1, 100, 4),
                      (2, 128, 64), (8, 256, 16), (4, 256, 8), (2, 256, 4), (256, 256, 16),
                      (3, 300, 48)):
        st, msg = bwd_grouped(g, dim, n)
        assert st == ssm.SSM_ERR_INVALID_ARG and "handle" in msg, (g, dim, n, msg)
    for g, dim, n in ((3, 256, 16), (0, 256, 16)):
        st, msg = bwd_grouped(g, dim, n)
        assert st == ssm.SSM_ERR_INVALID_ARG and "ngroups" in msg, (g, msg)
    n = ctypes.c_size_t(1)
    lib = ssm.load_library()
    st = lib.ssm_selective_scan_bwd_grouped_workspace_size(None, 2, 256, 16, 8, 8,
                                                           ctypes.byref(n))
    assert st == ssm.SSM_ERR_INVALID_ARG and n.value == 0
