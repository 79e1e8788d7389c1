"""The C ABI without a GPU: the library loads, exports what include/sscan.h declares,
and rejects bad arguments before anything touches the device."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sscan.h")


def _build_module():
    # by path: importing the package loads libsscan.so, which may not exist yet
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_sscan_build", os.path.join(ROOT, "selective_state_space_77_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def lib():
    hb = _build_module()
    if not os.path.exists(hb.LIB):
        hb.build()
    import selective_state_space_77_amd as s
    return s.lib


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sscan_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert _declared() == ["sscan_backward", "sscan_forward", "sscan_forward_from_state",
                           "sscan_forward_fused", "sscan_forward_noalloc", "sscan_forward_plan", "sscan_last_error",
                           "sscan_ssd_forward",
                           "sscan_ssd_step", "sscan_status_string", "sscan_step", "sscan_step_fused",
                           "sscan_version"]


def test_every_declared_symbol_is_exported(lib):
    hb = _build_module()
    out = subprocess.run(["nm", "-D", "--defined-only", hb.LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (sscan_\w+)", out))
    for name in _declared():
        assert name in exported, name
        assert hasattr(lib, name)


def test_version_and_status_strings(lib):
    assert lib.sscan_version() == 1
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.sscan_status_string(code)
    assert lib.sscan_status_string(7) == b"unknown status"


def _fwd(lib, **kw):
    a = dict(x=0x1000, delta=0x2000, A=0x3000, B=0x4000, C=0x5000, D=None, y=0x6000, hs=None,
             batch=1, L=4, dim=2, N=3, io=0)
    a.update(kw)
    return lib.sscan_forward(a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["y"], a["hs"],
                             a["batch"], a["L"], a["dim"], a["N"], a["io"], None)


def test_forward_validation_happens_before_any_device_work(lib):
    # fake, never-dereferenced addresses far apart: only validation runs
    assert _fwd(lib, x=None) == -1
    assert _fwd(lib, y=None) == -1
    assert _fwd(lib, A=None) == -1
    assert _fwd(lib, batch=-1) == -2
    assert _fwd(lib, L=1 << 62, dim=1 << 20) == -2
    assert _fwd(lib, N=0) == -3
    assert _fwd(lib, N=17) == -3
    assert _fwd(lib, io=2) == -3
    assert _fwd(lib, y=0x1000) == -4              # y == x
    assert _fwd(lib, y=0x2010) == -4              # y overlaps delta
    assert _fwd(lib, hs=0x4004) == -4             # final_state overlaps B
    assert _fwd(lib, hs=0x6008) == -4             # final_state overlaps y
    assert b"overlap" in lib.sscan_last_error()


def test_empty_inputs_need_no_pointers_and_launch_nothing(lib):
    assert _fwd(lib, x=None, delta=None, B=None, C=None, y=None, batch=0) == 0
    assert _fwd(lib, x=None, delta=None, y=None, dim=0, A=None) == 0
    assert _fwd(lib, x=None, delta=None, y=None, dim=0, A=None, B=None) == -1  # B still non-empty


def test_initial_state_validation(lib):
    f = lib.sscan_forward_from_state
    args = lambda h0, hs, **kw: (kw.get("x", 0x1000), 0x2000, 0x3000, 0x4000, 0x5000, None, h0, 0x6000,
                                 hs, 1, 4, 2, 3, 0, None)
    assert f(*args(0x20000, 0x20000)) == -4          # initial_state == final_state
    assert f(*args(0x20004, 0x20000)) == -4          # initial_state overlaps final_state
    assert f(*args(0x6004, None)) == -4              # initial_state overlaps y
    assert b"initial_state" in lib.sscan_last_error()
    assert f(*args(0x20000, None, x=None)) == -1     # required pointers still checked
    # empty batch: nothing to do, initial_state may be NULL (A still required: dim > 0)
    assert lib.sscan_forward_from_state(None, None, 0x3000, None, None, None, None, None, None,
                                        0, 4, 2, 3, 0, None) == 0


def _bwd(lib, **kw):
    a = dict(x=0x1000, delta=0x2000, A=0x3000, B=0x4000, C=0x5000, D=None, h0=None, dy=0x7000,
             dhT=None, dx=0x8000, dd=0x9000, dA=0xA000, dB=0xB000, dC=0xC000, dD=None, dh0=None,
             batch=1, L=4, dim=2, N=3, io=0)
    a.update(kw)
    return lib.sscan_backward(a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["h0"], a["dy"],
                              a["dhT"], a["dx"], a["dd"], a["dA"], a["dB"], a["dC"], a["dD"], a["dh0"],
                              a["batch"], a["L"], a["dim"], a["N"], a["io"], None)


def test_backward_validation(lib):
    # fake, never-dereferenced addresses: only validation runs
    for name in ("x", "delta", "A", "B", "C", "dy", "dx", "dd", "dA", "dB", "dC"):
        assert _bwd(lib, **{name: None}) == -1, name
    assert _bwd(lib, L=-1) == -2
    assert _bwd(lib, L=1 << 50, dim=1 << 20) == -2
    assert _bwd(lib, N=0) == -3
    assert _bwd(lib, N=17) == -3
    assert _bwd(lib, io=5) == -3
    assert _bwd(lib, dim=(1 << 24) + 1) == -3
    assert _bwd(lib, dx=0x1000) == -4                      # dx == x
    assert _bwd(lib, dd=0x7004) == -4                      # ddelta overlaps dy
    assert _bwd(lib, dC=0xB010) == -4                      # dC overlaps dB (fp32, 48 bytes)
    assert _bwd(lib, dh0=0x20000, dhT=0x20008) == -4       # dinitial_state overlaps dfinal_state
    assert _bwd(lib, dD=0x3004) == -4                      # dDskip overlaps A
    assert b"overlap" in lib.sscan_last_error()
    # dB/dC are fp32 whatever io_dtype is: with bf16 inputs (B: 24 bytes) a dC 32
    # bytes after dB still overlaps it
    assert _bwd(lib, io=1, dC=0xB020) == -4


def _fwd_fused(lib, **kw):
    a = dict(x=0x1000, w=0x20000, cb=None, K=4, act=0, csi=None, dr=0x2000, db=None, A=0x3000,
             B=0x4000, C=0x5000, D=None, h0=None, y=0x6000, hs=None, cso=None,
             batch=1, L=4, dim=2, N=3, io=0)
    a.update(kw)
    return lib.sscan_forward_fused(a["x"], a["w"], a["cb"], a["K"], a["act"], a["csi"], a["dr"], a["db"],
                                   a["A"], a["B"], a["C"], a["D"], a["h0"], a["y"], a["hs"], a["cso"],
                                   a["batch"], a["L"], a["dim"], a["N"], a["io"], None)


def test_forward_fused_validation(lib):
    assert _fwd_fused(lib, K=0) == -3
    assert _fwd_fused(lib, K=5) == -3
    assert _fwd_fused(lib, act=2) == -3
    assert _fwd_fused(lib, w=None) == -1
    assert _fwd_fused(lib, dr=None) == -1
    assert _fwd_fused(lib, batch=-1) == -2
    assert _fwd_fused(lib, cso=0x1004) == -4                 # conv_state_out overlaps x
    assert _fwd_fused(lib, csi=0x30000, cso=0x30008) == -4   # conv_state_out overlaps conv_state_in
    assert b"conv_state_out" in lib.sscan_last_error()
    assert _fwd_fused(lib, y=0x20004) == -4                  # y overlaps conv_weight (2 x 4 fp32)
    assert _fwd_fused(lib, cso=0x20010) == -4                # conv_state_out overlaps conv_weight
    # K = 1 has no carried inputs: conv_state pointers may then be anything disjoint
    assert _fwd_fused(lib, K=1, y=None) == -1


def _step_fused(lib, **kw):
    a = dict(st=0x10000, cs=0x40000, x=0x1000, w=0x20000, cb=None, K=4, act=1, dr=0x2000, db=None,
             A=0x3000, B=0x4000, C=0x5000, D=None, y=0x6000, batch=2, dim=3, N=4, io=1)
    a.update(kw)
    return lib.sscan_step_fused(a["st"], a["cs"], a["x"], a["w"], a["cb"], a["K"], a["act"], a["dr"],
                                a["db"], a["A"], a["B"], a["C"], a["D"], a["y"], a["batch"], a["dim"],
                                a["N"], a["io"], None)


def test_step_fused_validation(lib):
    assert _step_fused(lib, cs=None) == -1           # d_conv > 1 needs the carried inputs
    assert _step_fused(lib, w=None) == -1
    assert _step_fused(lib, K=0) == -3
    assert _step_fused(lib, K=9) == -3
    assert _step_fused(lib, act=-1) == -3
    assert _step_fused(lib, cs=0x10010) == -4        # conv_state overlaps state
    assert _step_fused(lib, cs=0x2002) == -4         # conv_state overlaps delta_raw_t
    assert b"conv_state" in lib.sscan_last_error()
    assert _step_fused(lib, batch=0, st=None, cs=None, x=None, dr=None, B=None, C=None, y=None) == 0


def _ssd(lib, **kw):
    a = dict(x=0x100000, d=0x200000, A=0x300000, B=0x400000, C=0x500000, D=None, h0=None, y=0x600000,
             hs=None, batch=1, L=8, H=4, P=64, G=2, N=64, io=1)
    a.update(kw)
    return lib.sscan_ssd_forward(a["x"], a["d"], a["A"], a["B"], a["C"], a["D"], a["h0"], a["y"], a["hs"],
                                 a["batch"], a["L"], a["H"], a["P"], a["G"], a["N"], a["io"], None)


def test_ssd_validation(lib):
    assert _ssd(lib, P=32) == -3
    assert _ssd(lib, N=16) == -3
    assert _ssd(lib, io=3) == -3
    assert _ssd(lib, G=3) == -2                 # heads not a multiple of groups
    assert _ssd(lib, G=0) == -2
    assert _ssd(lib, L=-1) == -2
    assert _ssd(lib, x=None) == -1
    assert _ssd(lib, C=None) == -1
    assert _ssd(lib, y=0x100010) == -4          # y overlaps x
    assert _ssd(lib, hs=0x300008) == -4         # final state overlaps A
    assert _ssd(lib, batch=0, x=None, d=None, B=None, C=None, y=None) == 0


def _ssd_step(lib, **kw):
    # batch 2, 4 heads of 64 channels, 2 groups, N = 64, bf16: x_t 1 KiB, state 128 KiB
    a = dict(st=0x1000000, x=0x10000, d=0x20000, A=0x30000, B=0x40000, C=0x50000, D=None, y=0x60000,
             batch=2, H=4, P=64, G=2, N=64, io=1)
    a.update(kw)
    return lib.sscan_ssd_step(a["st"], a["x"], a["d"], a["A"], a["B"], a["C"], a["D"], a["y"], a["batch"],
                              a["H"], a["P"], a["G"], a["N"], a["io"], None)


def test_ssd_step_validation(lib):
    assert _ssd_step(lib, P=32) == -3
    assert _ssd_step(lib, N=16) == -3
    assert _ssd_step(lib, io=2) == -3
    assert _ssd_step(lib, G=3) == -2             # heads not a multiple of groups
    assert _ssd_step(lib, batch=-1) == -2
    assert _ssd_step(lib, st=None) == -1
    assert _ssd_step(lib, B=None) == -1
    assert _ssd_step(lib, y=None) == -1
    assert _ssd_step(lib, y=0x10100) == -4       # y_t overlaps x_t
    assert _ssd_step(lib, st=0x40000) == -4      # state overlaps B_t
    assert _ssd_step(lib, D=0x1000100) == -4     # Dskip inside the state
    assert _ssd_step(lib, batch=0, st=None, x=None, d=None, B=None, C=None, y=None) == 0


def _step(lib, **kw):
    a = dict(st=0x10000, x=0x1000, delta=0x2000, A=0x3000, B=0x4000, C=0x5000, D=None, y=0x6000,
             batch=2, dim=3, N=4, io=1)
    a.update(kw)
    return lib.sscan_step(a["st"], a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["y"],
                          a["batch"], a["dim"], a["N"], a["io"], None)


def test_step_validation(lib):
    assert _step(lib, st=None) == -1
    assert _step(lib, C=None) == -1
    assert _step(lib, dim=-3) == -2
    assert _step(lib, N=32) == -3
    assert _step(lib, io=-1) == -3
    assert _step(lib, st=0x1004) == -4           # state overlaps x_t
    assert _step(lib, y=0x10010) == -4           # y_t overlaps state
    assert _step(lib, y=0x3000) == -4            # y_t overlaps A
    assert _step(lib, batch=0, st=None, x=None, delta=None, B=None, C=None, y=None) == 0


def test_python_binding_rejects_host_tensors():
    import torch
    import selective_state_space_77_amd as s
    x = torch.zeros(1, 4, 2)
    with pytest.raises(ValueError):
        s.forward(x, x.clone(), torch.zeros(2, 3), torch.zeros(1, 4, 3), torch.zeros(1, 4, 3))
    with pytest.raises(TypeError):
        s.forward(x.double(), x.double(), torch.zeros(2, 3), torch.zeros(1, 4, 3).double(),
                  torch.zeros(1, 4, 3).double())


def test_python_binding_checks_output_shapes_before_any_device_work():
    """An output buffer of the wrong shape would be written past its end by the
    kernels; the binding refuses it (host tensors reach the shape check first)."""
    import torch
    import selective_state_space_77_amd as s
    x = torch.zeros(1, 4, 2)
    A, B = torch.zeros(2, 3), torch.zeros(1, 4, 3)
    with pytest.raises(ValueError, match="y must have shape"):
        s.forward(x, x.clone(), A, B, B.clone(), y=torch.zeros(1, 3, 2))
    with pytest.raises(ValueError, match="y_t must have shape"):
        s.step(torch.zeros(1, 2, 3), torch.zeros(1, 2), torch.zeros(1, 2), A, torch.zeros(1, 3),
               torch.zeros(1, 3), y_t=torch.zeros(1, 1))
    with pytest.raises(ValueError, match="y must have shape"):
        xs = torch.zeros(1, 4, 2, 64)
        Bs = torch.zeros(1, 4, 1, 64)
        s.ssd_forward(xs, torch.zeros(1, 4, 2), torch.zeros(2), Bs, Bs.clone(), y=torch.zeros(1, 4, 2, 32))
    with pytest.raises(ValueError, match="Dskip must have shape"):
        s.step_fused(torch.zeros(1, 2, 3), torch.zeros(1, 3, 2), torch.zeros(1, 2), torch.zeros(2, 4),
                     torch.zeros(1, 2), A, torch.zeros(1, 3), torch.zeros(1, 3), Dskip=torch.zeros(5))


def test_product_package_does_not_reference_the_oracle():
    pkg = os.path.join(ROOT, "selective_state_space_77_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in src.lower(), f
