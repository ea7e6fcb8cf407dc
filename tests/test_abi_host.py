"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments with the documented status codes
before any HIP call (no GPU needed: no compute call is made)."""
import ctypes
import re
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "ssd_mi355x.h"

OK, NULL, SHAPE, UNSUP, WS, ALIGN, HIP, ALIAS = range(8)


def _declared():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_\w+|ssm_step\w*)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import mamba_ssd_scan_02_amd as ssd
    return ssd.load()


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("ssd_forward", "ssm_step", "ssd_forward_workspace_bytes", "ssd_status_str",
              "ssd_abi_version", "ssd_chunk_cumsum", "ssd_chunk_state", "ssd_chunk_cumsum_state",
              "ssd_forward_gated",
              "ssd_state_passing",
              "ssd_state_scan", "ssd_chunk_scan", "ssd_forward_zoh", "ssd_chunk_cumsum_zoh",
              "ssm_step_zoh", "ssd_layer_in", "ssd_layer_out", "ssd_state_passing_seg",
              "ssd_state_passing_seg_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    import mamba_ssd_scan_02_amd as ssd
    out = subprocess.run(["nm", "-D", "--defined-only", str(ssd.library_path())],
                         capture_output=True, text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for n in _declared():
        assert n in exported, n
        assert hasattr(lib, n)


def test_version_and_status_strings(lib):
    assert lib.ssd_abi_version() == 8
    for s in range(8):
        assert lib.ssd_status_str(s)
    assert lib.ssd_status_str(99) == b"unknown status"


def test_workspace_bytes(lib):
    import mamba_ssd_scan_02_amd as ssd
    import torch
    n = lib.ssd_forward_workspace_bytes(4, 8192, 80, 64, 128, 1, 256, 1)
    regions = ssd.workspace_regions(4, 8192, 80, 64, 128, 256, torch.bfloat16)
    assert n == regions["total"]
    nc = 32
    # cs, dtc fp32; S and Hin in the storage type (bf16)
    assert n >= 4 * 80 * nc * 256 * 4 * 2 + 4 * 80 * nc * 64 * 128 * 2 * 2
    n = lib.ssd_forward_workspace_bytes(1, 256, 1, 16, 16, 1, 64, 0)
    assert n == ssd.workspace_regions(1, 256, 1, 16, 16, 64, torch.float32)["total"]
    assert lib.ssd_forward_workspace_bytes(4, 8192, 80, 64, 128, 3, 256, 1) == 0   # H % G
    assert lib.ssd_forward_workspace_bytes(4, 8192, 80, 64, 128, 1, 512, 1) == 0   # chunk
    assert lib.ssd_forward_workspace_bytes(1, 8, 1, 256, 16, 1, 8, 0) == 0         # P too big
    assert lib.ssd_forward_workspace_bytes(1, 8, 1, 16, 16, 1, 8, 7) == 0          # dtype
    assert lib.ssd_forward_workspace_bytes(0, 8, 1, 16, 16, 1, 8, 0) == 0


def _fwd(lib, **over):
    a = dict(batch=1, seqlen=64, nheads=2, headdim=16, dstate=16, ngroups=1, chunk=64, dtype=0,
             x=0x1000, dt=0x2000, A=0x3000, B=0x4000, C=0x5000, D=None, init=None, y=0x100000,
             final=None, ws=0x200000, wsb=1 << 30, stream=None)
    a.update(over)
    P = ctypes.c_void_p
    return lib.ssd_forward(a["batch"], a["seqlen"], a["nheads"], a["headdim"], a["dstate"],
                           a["ngroups"], a["chunk"], a["dtype"], P(a["x"]), P(a["dt"]), P(a["A"]),
                           P(a["B"]), P(a["C"]), P(a["D"]), P(a["init"]), P(a["y"]), P(a["final"]),
                           P(a["ws"]), a["wsb"], P(a["stream"]))


def test_forward_argument_errors(lib):
    assert _fwd(lib, batch=0) == SHAPE
    assert _fwd(lib, seqlen=-1) == SHAPE
    assert _fwd(lib, nheads=3, ngroups=2) == SHAPE
    assert _fwd(lib, chunk=0) == SHAPE
    assert _fwd(lib, chunk=300) == UNSUP
    assert _fwd(lib, headdim=129) == UNSUP
    assert _fwd(lib, dtype=5) == UNSUP
    assert _fwd(lib, x=None) == NULL
    assert _fwd(lib, y=None) == NULL
    assert _fwd(lib, ws=None) == WS
    assert _fwd(lib, wsb=16) == WS
    assert _fwd(lib, x=0x1008) == ALIGN
    assert _fwd(lib, dt=0x2002) == ALIGN
    assert _fwd(lib, y=0x1000) == ALIAS            # y on top of x
    assert _fwd(lib, ws=0x1000) == ALIAS           # workspace on top of x
    # y or the workspace on top of A or D
    assert _fwd(lib, y=0x3000) == ALIAS
    assert _fwd(lib, D=0x6000, y=0x6000) == ALIAS
    assert _fwd(lib, ws=0x3000) == ALIAS
    assert _fwd(lib, D=0x6000, ws=0x6000) == ALIAS
    # final_state on any input but init_state, on y or on the workspace
    for name, addr in (("x", 0x1000), ("dt", 0x2000), ("A", 0x3000), ("B", 0x4000),
                       ("C", 0x5000)):
        assert _fwd(lib, final=addr) == ALIAS, name
    assert _fwd(lib, D=0x6000, final=0x6000) == ALIAS
    assert _fwd(lib, final=0x100000) == ALIAS      # on y
    assert _fwd(lib, final=0x200000) == ALIAS      # on the workspace
    # (final_state on init_state is allowed: tests/test_gpu_forward.py runs it)


def test_noalloc_rejects_before_any_call(lib):
    """ssd_forward_noalloc refuses sizes whose workspace exceeds its scratch
    array, bad sizes and missing pointers before any GPU call."""
    P = ctypes.c_void_p
    p = P(0x10000)
    assert lib.ssd_forward_workspace_bytes(4, 8192, 80, 64, 128, 1, 256, 1) > 64 << 20
    assert lib.ssd_forward_noalloc(4, 8192, 80, 64, 128, 1, 256, 1, p, p, p, p, p, None, None, p,
                                   None, None) == WS
    assert lib.ssd_forward_noalloc(0, 64, 2, 64, 128, 1, 256, 1, p, p, p, p, p, None, None, p,
                                   None, None) == SHAPE
    assert lib.ssd_forward_noalloc(1, 64, 2, 64, 128, 1, 512, 1, p, p, p, p, p, None, None, p,
                                   None, None) == UNSUP
    assert lib.ssd_forward_noalloc(1, 64, 2, 64, 128, 1, 256, 1, None, p, p, p, p, None, None, p,
                                   None, None) == NULL


def test_step_argument_errors(lib):
    P = ctypes.c_void_p

    def step(**over):
        a = dict(batch=1, nheads=2, headdim=16, dstate=16, ngroups=1, dtype=0, state=0x100000,
                 x=0x1000, dt=0x2000, A=0x3000, B=0x4000, C=0x5000, D=None, y=0x6000)
        a.update(over)
        return lib.ssm_step(a["batch"], a["nheads"], a["headdim"], a["dstate"], a["ngroups"],
                            a["dtype"], P(a["state"]), P(a["x"]), P(a["dt"]), P(a["A"]),
                            P(a["B"]), P(a["C"]), P(a["D"]), P(a["y"]), None)

    assert step(batch=0) == SHAPE
    assert step(nheads=3, ngroups=2) == SHAPE
    assert step(dstate=2048) == UNSUP
    assert step(dtype=9) == UNSUP
    assert step(state=None) == NULL
    assert step(state=0x100004) == ALIGN
    assert step(y=0x100000) == ALIAS


def test_stage_argument_errors(lib):
    P = ctypes.c_void_p
    assert lib.ssd_chunk_cumsum(1, 64, 2, 0, P(0x1000), P(0x2000), P(0x3000), P(0x4000), None) == SHAPE
    assert lib.ssd_chunk_cumsum(1, 64, 2, 512, P(0x1000), P(0x2000), P(0x3000), P(0x4000), None) == UNSUP
    assert lib.ssd_chunk_cumsum(1, 64, 2, 64, None, P(0x2000), P(0x3000), P(0x4000), None) == NULL
    assert lib.ssd_chunk_state(1, 64, 2, 64, 128, 1, 64, 1, P(0x1000), None, P(0x10), P(0x20),
                               P(0x4000), None) == NULL
    assert lib.ssd_state_passing(1, 64, 2, 64, 128, 64, 1, P(0x1000), P(0x2000), None, P(0x3008),
                                 None, None) == ALIGN
    # the one-pass state stage exists for bf16, P = 64, N = 128, chunk 128 or
    # 256 with heads that pair up in a group, else chunk 256 (no call below
    # passes its checks: none may reach a launch)
    assert lib.ssd_state_scan(1, 64, 2, 64, 128, 1, 64, 1, P(0x1000), P(0x2000), P(0x10), P(0x20),
                              None, P(0x4000), None, None) == UNSUP
    assert lib.ssd_state_scan(1, 64, 3, 64, 128, 1, 128, 1, P(0x1000), P(0x2000), P(0x10), P(0x20),
                              None, P(0x4000), None, None) == UNSUP
    assert lib.ssd_state_scan(1, 64, 2, 64, 128, 1, 256, 0, P(0x1000), P(0x2000), P(0x10), P(0x20),
                              None, P(0x4000), None, None) == UNSUP
    assert lib.ssd_state_scan(1, 64, 2, 32, 128, 1, 256, 1, P(0x1000), P(0x2000), P(0x10), P(0x20),
                              None, P(0x4000), None, None) == UNSUP
    assert lib.ssd_state_scan(1, 64, 2, 64, 128, 1, 256, 1, P(0x1000), None, P(0x10), P(0x20),
                              None, P(0x4000), None, None) == NULL
    assert lib.ssd_state_scan(1, 64, 2, 64, 128, 1, 256, 1, P(0x1000), P(0x2000), P(0x10), P(0x20),
                              None, P(0x4008), None, None) == ALIGN
    assert lib.ssd_state_scan(1, 64, 3, 64, 128, 2, 256, 1, P(0x1000), P(0x2000), P(0x10), P(0x20),
                              None, P(0x4000), None, None) == SHAPE
    assert lib.ssd_chunk_scan(1, 64, 2, 64, 128, 1, 64, 1, P(0x1000), P(0x2000), P(0x3000),
                              P(0x10), P(0x20), P(0x8000), None, P(0x1000), None) == ALIAS


def test_stage_outputs_must_not_overlap_inputs(lib):
    """Each stage call refuses an output on top of an input or of another
    output before any launch (every call below would otherwise reach a
    launch, so a missed check shows up as a HIP error, not as ALIAS)."""
    P = ctypes.c_void_p
    M = 1 << 24                      # arrays 16 MiB apart: none of them overlaps another
    a = [P((k + 1) * M) for k in range(12)]
    # batch 1, 512 tokens, 4 heads, P 64, N 128, 1 group, chunk 256, bf16:
    # x 256 KB, B/C 128 KB, dt 8 KB, cs/dtc rows 8 KB, S/Hin 128 KB, fp32 state 128 KB
    dims = (1, 512, 4, 64, 128, 1, 256, 1)
    cum = lambda dt, A, cs, dtc: lib.ssd_chunk_cumsum(1, 512, 4, 256, dt, A, cs, dtc, None)
    assert cum(a[0], a[1], a[0], a[3]) == ALIAS                   # cs on dt
    assert cum(a[0], a[1], a[2], P(a[1].value + 8)) == ALIAS      # dtc inside A's 16 bytes
    assert cum(a[0], a[1], a[2], P(a[2].value + 4096)) == ALIAS   # dtc on cs
    st = lambda x, B, cs, dtc, S: lib.ssd_chunk_state(*dims, x, B, cs, dtc, S, None)
    assert st(a[0], a[1], a[2], a[3], P(a[0].value + 65536)) == ALIAS   # S inside x
    assert st(a[0], a[1], a[2], a[3], a[3]) == ALIAS                    # S on dtc
    cst = lambda x, B, dt, A, cs, dtc, S: lib.ssd_chunk_cumsum_state(*dims, x, B, dt, A, cs, dtc,
                                                                      S, None)
    assert cst(a[0], a[1], a[2], a[3], a[4], a[5], a[1]) == ALIAS     # S on B
    assert cst(a[0], a[1], a[2], a[3], a[4], a[4], a[6]) == ALIAS     # dtc on cs
    sp = lambda S, cs, init, Hin, fin: lib.ssd_state_passing(1, 512, 4, 64, 128, 256, 1, S, cs,
                                                             init, Hin, fin, None)
    assert sp(a[0], a[1], a[2], a[0], a[4]) == ALIAS                  # Hin on S
    assert sp(a[0], a[1], a[2], a[3], a[3]) == ALIAS                  # final on Hin
    assert sp(a[0], a[1], a[2], a[3], a[1]) == ALIAS                  # final on cs
    assert sp(a[0], a[1], a[2], a[2], a[4]) == ALIAS                  # Hin on init
    ws = lib.ssd_state_passing_seg_workspace_bytes(1, 4, 64, 128, 2)
    seg = lambda S, Hin, fin, w: lib.ssd_state_passing_seg(1, 512, 4, 64, 128, 256, 2, 1, S, a[1],
                                                           None, Hin, fin, w, ws, None)
    assert seg(a[0], a[3], a[4], a[0]) == ALIAS                       # workspace on S
    assert seg(a[0], a[3], a[4], a[3]) == ALIAS                       # workspace on Hin
    scan = lambda x, B, cs, dtc, init, Hin, fin: lib.ssd_state_scan(*dims, x, B, cs, dtc, init,
                                                                     Hin, fin, None)
    assert scan(a[0], a[1], a[2], a[3], a[4], a[1], a[6]) == ALIAS    # Hin on B
    assert scan(a[0], a[1], a[2], a[3], a[4], a[5], a[2]) == ALIAS    # final on cs
    cscan = lambda y, Hin, D: lib.ssd_chunk_scan(*dims, a[0], a[1], a[2], a[3], a[4], Hin, D, y,
                                                 None)
    assert cscan(a[5], a[5], None) == ALIAS                           # y on Hin
    assert cscan(a[3], a[5], None) == ALIAS                           # y on cs
    assert cscan(a[6], a[5], a[6]) == ALIAS                           # y on D


def test_layer_argument_errors(lib):
    P = ctypes.c_void_p

    def lin(**over):
        a = dict(batch=1, seqlen=64, nheads=2, headdim=8, dstate=8, ngroups=1, K=4, dtype=1,
                 xbc=0x10000, w=0x20000, b=None, dtr=0x30000, dtb=None, x=0x40000, B=0x50000,
                 C=0x60000, dt=0x70000)
        a.update(over)
        return lib.ssd_layer_in(a["batch"], a["seqlen"], a["nheads"], a["headdim"], a["dstate"],
                                a["ngroups"], a["K"], a["dtype"], P(a["xbc"]), P(a["w"]),
                                P(a["b"]), P(a["dtr"]), P(a["dtb"]), P(a["x"]), P(a["B"]),
                                P(a["C"]), P(a["dt"]), None)

    assert lin(seqlen=0) == SHAPE
    assert lin(nheads=3, ngroups=2) == SHAPE
    assert lin(batch=70000) == SHAPE
    assert lin(K=0) == UNSUP and lin(K=9) == UNSUP
    assert lin(dtype=4) == UNSUP
    assert lin(xbc=None) == NULL and lin(dt=None) == NULL and lin(w=None) == NULL
    assert lin(x=0x40001) == ALIGN
    assert lin(dtr=0x30002) == ALIGN
    assert lin(x=0x10000) == ALIAS                 # x on top of xbc
    assert lin(C=0x50000) == ALIAS                 # C on top of B
    assert lin(dt=0x30000) == ALIAS                # dt on top of dt_raw
    assert lib.ssd_layer_out(0, 1, P(0x1000), P(0x2000), P(0x3000), None) == SHAPE
    assert lib.ssd_layer_out(16, 3, P(0x1000), P(0x2000), P(0x3000), None) == UNSUP
    assert lib.ssd_layer_out(16, 1, P(0x1000), None, P(0x3000), None) == NULL
    assert lib.ssd_layer_out(16, 1, P(0x1001), P(0x2000), P(0x3000), None) == ALIGN
    assert lib.ssd_layer_out(16, 1, P(0x1000), P(0x2000), P(0x2010), None) == ALIAS   # out on z
    assert lib.ssd_layer_out(16, 1, P(0x1000), P(0x2000), P(0x1010), None) == ALIAS   # part of y


def test_segmented_state_passing_argument_errors(lib):
    P = ctypes.c_void_p
    need = lib.ssd_state_passing_seg_workspace_bytes(1, 2, 64, 128, 4)
    # two state buffers of 2 x 4 x 64 x 128 fp32 plus the decays, 256-byte rounded
    assert need == 2 * (2 * 4 * 64 * 128 * 4) + 256
    assert lib.ssd_state_passing_seg_workspace_bytes(1, 2, 64, 128, 0) == 0

    def seg(**over):
        a = dict(nseg=4, S=0x100000, cs=0x2000, init=None, Hin=0x400000, fin=None, ws=0x800000,
                 wsb=need)
        a.update(over)
        return lib.ssd_state_passing_seg(1, 1024, 2, 64, 128, 256, a["nseg"], 1, P(a["S"]),
                                         P(a["cs"]), P(a["init"]), P(a["Hin"]), P(a["fin"]),
                                         P(a["ws"]), a["wsb"], None)

    assert seg(nseg=0) == SHAPE
    assert seg(S=None) == NULL
    assert seg(ws=None) == WS
    assert seg(wsb=need - 1) == WS
    assert seg(ws=0x800010) == ALIGN
    assert seg(Hin=0x400008) == ALIGN
    # more segments than chunks act as one per chunk (4 here): the same workspace suffices
    assert lib.ssd_state_passing_seg_workspace_bytes(1, 2, 64, 128, 4) == need


def test_plain_c_caller(tmp_path):
    """The header compiles as C99 and a C program linked against the library
    gets the documented results from the calls that need no GPU."""
    import shutil
    import mamba_ssd_scan_02_amd as ssd
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not available")
    root = Path(__file__).resolve().parents[1]
    libdir = ssd.library_path().parent
    exe = tmp_path / "abi_smoke"
    cmd = ["gcc", "-std=c99", "-D__HIP_PLATFORM_AMD__", f"-I{root / 'include'}",
           "-I/opt/rocm/include", str(root / "tests" / "c" / "abi_smoke.c"), "-o", str(exe),
           f"-L{libdir}", "-lssd_mi355x", f"-Wl,-rpath,{libdir}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "abi_smoke: ok" in out.stdout


def test_two_level_stage_argument_errors(lib):
    """The two-level stage calls accept only the shapes the forward runs them
    at (bf16, P = 64, N = 128, chunk 256, an even head count per group) and
    run lengths 1 .. 65536; every error returns before any launch."""
    import mamba_ssd_scan_02_amd as ssd
    import torch
    P = ctypes.c_void_p
    M = 1 << 24
    a = [P((k + 1) * M) for k in range(12)]
    ok = (1, 512, 4, 64, 128, 1, 256, 1)

    def sr(dims=ok, K=2, ptrs=None):
        q = ptrs or a[:9]
        return lib.ssd_chunk_state_runs(*dims, K, *q, None)

    assert sr(dims=(1, 512, 4, 64, 128, 1, 256, 0)) == UNSUP        # fp32
    assert sr(dims=(1, 512, 4, 64, 128, 1, 128, 1)) == UNSUP        # chunk 128
    assert sr(dims=(1, 512, 3, 64, 128, 1, 256, 1)) == UNSUP        # odd heads per group
    assert sr(dims=(1, 512, 4, 32, 128, 1, 256, 1)) == UNSUP        # P = 32
    assert sr(K=0) == SHAPE and sr(K=65537) == SHAPE
    assert sr(ptrs=[a[0], None] + a[2:9]) == NULL
    assert sr(ptrs=a[:6] + [P(a[6].value + 8)] + a[7:9]) == ALIGN   # T 8-byte aligned
    rp = lambda K=2, T=a[0], Hr=a[3], fin=None: lib.ssd_run_passing(1, 512, 4, 64, 128, 256, 1, K, T,
                                                                    a[1], None, Hr, fin, None)
    assert rp(K=0) == SHAPE
    assert rp(T=None) == NULL
    assert rp(Hr=a[0]) == ALIAS                                     # Hr on T
    cs = lambda K=2, y=a[10], T=a[5]: lib.ssd_chunk_scan_runs(*ok, K, a[0], a[1], a[2], a[3], a[4],
                                                              T, a[6], a[7], None, y, None)
    assert cs(K=0) == SHAPE
    assert cs(T=None) == NULL
    assert cs(y=a[6]) == ALIAS                                      # y on Hr
    # the run length the forward uses: 0 where it keeps the per-chunk stages
    assert ssd.forward_run_chunks(1, 512, 4, 64, 128, 1, 256, torch.bfloat16) == 0
    assert ssd.forward_run_chunks(4, 8192, 80, 64, 128, 1, 256, torch.float32) == 0
    assert ssd.forward_run_chunks(4, 8192, 80, 64, 128, 1, 128, torch.bfloat16) == 0
    K = ssd.forward_run_chunks(4, 8192, 80, 64, 128, 1, 256, torch.bfloat16)
    assert K in (2, 4, 8, 16)
    # the workspace covers both layouts
    n = lib.ssd_forward_workspace_bytes(1, 1, 2, 64, 128, 1, 256, 1)
    assert n >= 2 * 256 * 4 * 2 + 2 * 64 * 128 * 2
