"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments with the documented codes before
touching the HIP runtime (fake, never-dereferenced device addresses are used).

The ABI layer is also built on its own with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer, with recording stubs in place of the kernel
launchers (tests/host_abi_check.cpp), and run here: every error path, the launch
sequence of accepted calls, the KDA_TRACE plan line, and the kernels' 32-bit
per-lane offset formula at the ABI's size limits."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")
LIBPATH = os.path.join(ROOT, "gated_delta_rule_107_amd", "libkda.so")
CSRC = os.path.join(ROOT, "gated_delta_rule_107_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

needs_lib = pytest.mark.skipif(not os.path.exists(LIBPATH), reason="libkda.so not built")

OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, WS, HIP, ALIAS = range(9)
F32, BF16 = 0, 1


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIBPATH):
        pytest.skip("libkda.so not built")
    import gated_delta_rule_107_amd as g
    return g.lib()


# ------------------------------------------------------------------ sanitized host build of the ABI layer

@pytest.fixture(scope="module")
def host_check(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("g++ or the HIP headers are missing")
    exe = str(tmp_path_factory.mktemp("host_abi") / "host_abi_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include", f"-I{CSRC}",
           os.path.join(ROOT, "tests", "host_abi_check.cpp"), os.path.join(CSRC, "kda_api.cpp"),
           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


def _run_host_check(exe, *args, env=None):
    e = dict(os.environ)
    e.pop("KDA_TRACE", None)
    e.update(env or {})
    e.setdefault("ASAN_OPTIONS", "abort_on_error=0:halt_on_error=1")
    e.setdefault("UBSAN_OPTIONS", "print_stacktrace=1:halt_on_error=1")
    return subprocess.run([exe, *args], capture_output=True, text=True, env=e, timeout=120)


def test_abi_layer_under_sanitizers(host_check):
    r = _run_host_check(host_check)
    assert r.returncode == 0 and "ok: 0 failed checks" in r.stdout, r.stdout[-4000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]


def test_trace_prints_the_resolved_plan(host_check):
    r = _run_host_check(host_check, "trace", env={"KDA_TRACE": "1"})
    assert r.returncode == 0, r.stderr[-4000:]
    line = [ln for ln in r.stderr.splitlines() if ln.startswith("kda_chunk_fwd_noalloc:")]
    assert len(line) == 1, r.stderr
    for field in ("B=1", "T=4096", "H=16", "n_segments=16", "seg_len=256", "dv_block=128",
                  "workspace=50331648", "launches=segment-pass-1,scan,segment-pass-2"):
        assert field in line[0], (field, line[0])
    quiet = _run_host_check(host_check, "trace")
    assert "kda_chunk_fwd" not in quiet.stderr


def _plan_shapes(n, seed=20261203):
    """Seeded random problems over the supported set (B, H up to 9 x 300, T log-uniform up to 2^20,
    the ABI's size bounds kept), plus edge cases around the segment and compute-unit thresholds."""
    import numpy as np
    rng = np.random.default_rng(seed)
    out = [(1, T, H, 128, 128, 64, BF16) for T in (0, 1, 63, 64, 65, 192, 255, 256, 257, 4096)
           for H in (1, 16, 32, 48, 64, 100, 128, 129, 255, 256, 257)]
    out += [(2, 81920, 2, 64, 64, 64, BF16), (2, 78720, 2, 64, 64, 64, BF16), (1, 1 << 20, 32, 128, 128, 64, BF16)]
    while len(out) < n:
        dt = int(rng.integers(0, 2))
        dk, dv = (int(x) for x in rng.choice([16, 32, 64, 128], 2))
        chunk = int(rng.choice([16, 32, 64]))
        if dt == F32 and chunk * dk > 4096:
            continue
        B, H = int(rng.integers(1, 10)), int(rng.integers(1, 301))
        T = int(np.exp(rng.uniform(0, np.log(1 << 20)))) if rng.random() < 0.95 else 0
        if B * T > 1 << 22:
            continue
        out.append((B, T, H, dk, dv, chunk, dt))
    return out


def test_default_plans_are_well_formed(host_check):
    """For ~3,000 problems, the default plan as kda_chunk_fwd executes it (recorded by the host
    build's stub launchers): the segments tile [0, T) in whole chunks of at least two, the launch
    sequence matches the plan's form, no launch has more workgroups than the 256 compute units hold
    in one round (unless the units alone exceed them), segments are used exactly when at most half
    of the compute units would otherwise be busy and the sequence has eight chunks, the workspace
    matches, and passing the returned plan back explicitly executes identically."""
    shapes = _plan_shapes(3000)
    stdin = "".join(" ".join(map(str, s)) + "\n" for s in shapes)
    e = dict(os.environ)
    e.pop("KDA_TRACE", None)
    r = subprocess.run([host_check, "plans"], input=stdin, capture_output=True, text=True, env=e, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    lines = r.stdout.splitlines()
    assert len(lines) == len(shapes)
    bad = []
    for (B, T, H, dk, dv, chunk, dt), line in zip(shapes, lines):
        head, dflt, copy = line.split(" |")
        status, need, nseg, dvb, seg0 = (int(x) for x in head.split())
        copy_launches, status2 = copy.split()[:-1], int(copy.split()[-1])
        L = [x.split(":") for x in dflt.split()]
        what = [x[0] for x in L]
        f = [[int(v) for v in x[1:]] for x in L]          # mode seg_lo seg_cnt seg_cnt1 n_seg seg_len seg0_len dvb B
        units, nch = B * H, -(-T // chunk)
        why = []
        if status or status2:
            why.append(f"status {status} / {status2}")
        elif dflt.split() != copy_launches:
            why.append("explicit copy differs")
        elif dvb != dv:
            why.append(f"dv_block {dvb}")
        elif (nseg > 1) != (units <= 128 and nch >= 8):
            why.append(f"{nseg} segments for {units} units, {nch} chunks")
        elif nseg == 1:
            if what != ["chunk"] or f[0][:3] != [0, 0, 1] or need or seg0:
                why.append("one-pass launch")
        else:
            seg_len = f[0][5]
            if need != B * H * nseg * (2 * dk * dv + dk * dk) * 4:
                why.append(f"workspace {need}")
            if seg_len % chunk or seg0 % chunk or seg_len < 2 * chunk:
                why.append(f"segment lengths {seg0} / {seg_len}")
            if seg0 == 0:
                if not (nseg - 1) * seg_len < T <= nseg * seg_len:
                    why.append(f"{nseg} x {seg_len} does not tile T")
                if what != ["pass1", "scan", "chunk"] or f[0][:3] != [1, 0, nseg - 1] or f[1][1] != 0 \
                        or f[2][:3] != [0, 0, nseg]:
                    why.append("segmented launches")
            else:
                if not (0 < seg0 < T and seg0 + (nseg - 2) * seg_len < T <= seg0 + (nseg - 1) * seg_len):
                    why.append(f"lead form {seg0} + {nseg - 1} x {seg_len} does not tile T")
                if what != ["lead", "scan", "chunk"] or f[0][3] != nseg - 2 or f[1][1] != 1 or f[2][1:3] != [1, nseg - 1]:
                    why.append("lead-form launches")
            wgs = {"pass1": lambda x: x[2], "chunk": lambda x: x[2], "lead": lambda x: 1 + x[3]}
            most = max(units * wgs[w](x) for w, x in zip(what, f) if w in wgs)
            if most > 256:
                why.append(f"a launch of {most} workgroups")
        if why:
            bad.append(((B, T, H, dk, dv, chunk, dt), why, line[:200]))
    assert not bad, bad[:10]


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert {"kda_chunk_fwd", "kda_decode_step", "kda_decode_verify", "kda_decode_commit", "kda_status_str",
            "kda_last_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings(lib):
    assert lib.kda_abi_version() == 2
    for code in range(9):
        assert lib.kda_status_str(code).decode() not in ("", "unknown status")
    assert lib.kda_status_str(99) == b"unknown status"
    assert lib.kda_status_str(-1) == b"unknown status"


# fake device addresses: 16-byte aligned, far apart, never dereferenced
A = [0x10000000 * (i + 1) for i in range(12)]


def call_chunk(lib, **kw):
    import gated_delta_rule_107_amd as g
    args = dict(q=A[0], k=A[1], v=A[2], la=A[3], beta=A[4], S0=None, o=A[6], S_T=A[7],
                B=1, T=64, H=2, dk=16, dv=16, chunk=16, dt=F32, plan=g.Plan(1, 0), ws=None, wsb=0)
    args.update(kw)
    plan = ctypes.byref(args["plan"]) if args["plan"] is not None else None
    return lib.kda_chunk_fwd(args["q"], args["k"], args["v"], args["la"], args["beta"], args["S0"], args["o"],
                             args["S_T"], args["B"], args["T"], args["H"], args["dk"], args["dv"], args["chunk"],
                             args["dt"], plan, args["ws"], args["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(o=None), NULL), (dict(S_T=None), NULL), (dict(beta=None), NULL),
    (dict(B=0), SHAPE), (dict(H=0), SHAPE), (dict(T=-1), SHAPE),
    (dict(dt=7), DTYPE),
    (dict(dk=24), UNSUP), (dict(dv=256), UNSUP), (dict(chunk=128), UNSUP), (dict(chunk=8), UNSUP),
    (dict(dk=128, chunk=64, dt=F32), UNSUP), (dict(H=1 << 17, dk=128), UNSUP),
    (dict(q=A[0] + 4), ALIGN), (dict(S_T=A[7] + 8), ALIGN),
    (dict(o=A[0]), ALIAS), (dict(o=A[4] + 256), ALIAS), (dict(S_T=A[1]), ALIAS),
    (dict(S0=A[7] + 16), ALIAS),
])
def test_chunk_fwd_rejects(lib, kw, code):
    assert call_chunk(lib, **kw) == code
    assert lib.kda_last_error().decode() != ""


def test_chunk_fwd_plan_errors(lib):
    import gated_delta_rule_107_amd as g
    assert call_chunk(lib, plan=g.Plan(1, 24)) == UNSUP            # not a multiple of 16
    assert call_chunk(lib, plan=g.Plan(1, 32)) == UNSUP            # does not divide dv=16
    assert call_chunk(lib, plan=g.Plan(-1, 16)) == UNSUP
    # segments need a workspace
    r = call_chunk(lib, B=1, T=256, H=1, dk=32, dv=32, chunk=16, dt=BF16, plan=g.Plan(4, 32))
    assert r == WS


def test_chunk_fwd_checkpoint_errors(lib):
    import gated_delta_rule_107_amd as g

    def plan_ck(ptr, stride):
        p = g.Plan(1, 0)
        p.state_ckpt, p.ckpt_stride = ptr, stride
        return p
    assert call_chunk(lib, plan=plan_ck(A[9], 24)) == UNSUP        # not a multiple of chunk 16
    assert call_chunk(lib, plan=plan_ck(A[9], 0)) == UNSUP
    assert call_chunk(lib, plan=plan_ck(A[9], -32)) == UNSUP
    assert call_chunk(lib, plan=plan_ck(A[9] + 4, 32)) == ALIGN
    assert call_chunk(lib, plan=plan_ck(A[6], 32)) == ALIAS        # overlaps o
    assert call_chunk(lib, plan=plan_ck(A[7], 32)) == ALIAS        # overlaps S_T
    with pytest.raises(g.KdaError) as e:                           # the binding's own check
        import torch
        x = torch.zeros(1)
        g.chunk_fwd(x, x, x, x, x, ckpt_stride=24, chunk=16)
    assert e.value.code in (2, 5)


def test_chunk_fwd_packed_sequence_errors(lib):
    import gated_delta_rule_107_amd as g

    def plan_cu(n, nseg=1, ck=None):
        p = g.Plan(nseg, 0)
        p.cu_seqlens, p.n_seqs = A[10], n
        if ck:
            p.state_ckpt, p.ckpt_stride = ck, 32
        return p
    assert call_chunk(lib, B=2, plan=plan_cu(3)) == SHAPE           # packed means one batch row
    assert call_chunk(lib, plan=plan_cu(0)) == SHAPE
    assert call_chunk(lib, plan=plan_cu(3, nseg=2)) == WS           # segments need the workspace
    assert call_chunk(lib, plan=plan_cu(3, ck=A[9])) == UNSUP       # no checkpoints
    p = plan_cu(3)
    p.cu_seqlens = A[10] + 2
    assert call_chunk(lib, plan=p) == ALIGN


def test_plan_and_workspace_queries(lib):
    import gated_delta_rule_107_amd as g
    import torch
    # one (b,h) per workgroup already covers 256 compute units: no segments
    p = g.default_plan(8, 8192, 32, 128, 128, 64, torch.bfloat16)
    assert p.n_segments == 1 and p.dv_block == 128
    assert g.workspace_bytes(8, 8192, 32, 128, 128, 64, torch.bfloat16) == 0
    # one long sequence: segments give the parallelism
    p = g.default_plan(1, 1 << 20, 32, 128, 128, 64, torch.bfloat16)
    assert p.n_segments >= 8
    nb = g.workspace_bytes(1, 1 << 20, 32, 128, 128, 64, torch.bfloat16, p)
    assert nb == 32 * p.n_segments * (2 * 128 * 128 + 128 * 128) * 4
    # explicit plan is honoured; short sequences cap the number of segments
    p = g.Plan(4, 64)
    assert g.workspace_bytes(1, 1024, 2, 128, 128, 64, torch.bfloat16, p) == 2 * 4 * 3 * 128 * 128 * 4
    p = g.default_plan(1, 64, 1, 128, 128, 64, torch.bfloat16)
    assert p.n_segments == 1
    with pytest.raises(g.KdaError) as e:
        g.default_plan(1, 64, 1, 100, 128, 64, torch.bfloat16)
    assert e.value.code == UNSUP


@pytest.mark.parametrize("kw,code", [
    (dict(state=None), NULL), (dict(o=None), NULL), (dict(N=0), SHAPE), (dict(dt=3), DTYPE),
    (dict(dk=48), UNSUP), (dict(flags=4), UNSUP), (dict(q=A[1] + 2), ALIGN), (dict(o=A[0]), ALIAS),
    (dict(q=A[0] + 64), ALIAS),
])
def test_decode_step_rejects(lib, kw, code):
    args = dict(state=A[0], q=A[1], k=A[2], v=A[3], la=A[4], beta=A[5], o=A[6], N=4, H=2, dk=16, dv=16, dt=BF16,
                flags=0)
    args.update(kw)
    r = lib.kda_decode_step(args["state"], args["q"], args["k"], args["v"], args["la"], args["beta"], args["o"],
                            args["N"], args["H"], args["dk"], args["dv"], args["dt"], args["flags"], None)
    assert r == code


def decode_multi_args(**kw):
    args = dict(state=A[0], q=A[1], k=A[2], v=A[3], la=A[4], beta=A[5], o=A[6], n_accept=A[7], N=4, n=3, H=2,
                dk=16, dv=16, dt=BF16, flags=0)
    args.update(kw)
    return args


@pytest.mark.parametrize("kw,code", [
    (dict(o=None), NULL), (dict(n=0), SHAPE), (dict(N=1 << 20, n=1 << 12), SHAPE), (dict(flags=0xFFFFFFFF), UNSUP),
    (dict(dv=8), UNSUP), (dict(o=A[6] + 8), ALIGN),
    (dict(o=A[1] + 32), ALIAS),                      # o overlaps q of the 3 draft tokens
    (dict(state=A[6]), ALIAS),                       # o overlaps the (read-only) state
])
def test_decode_verify_rejects(lib, kw, code):
    a = decode_multi_args(**kw)
    r = lib.kda_decode_verify(a["state"], a["q"], a["k"], a["v"], a["la"], a["beta"], a["o"], a["N"], a["n"],
                              a["H"], a["dk"], a["dv"], a["dt"], a["flags"], None)
    assert r == code


@pytest.mark.parametrize("kw,code", [
    (dict(n_accept=None), NULL), (dict(state=None), NULL), (dict(n=-1), SHAPE), (dict(dt=9), DTYPE),
    (dict(n_accept=A[7] + 2), ALIGN), (dict(n_accept=A[0] + 64), ALIAS), (dict(beta=A[0] + 16), ALIAS),
])
def test_decode_commit_rejects(lib, kw, code):
    a = decode_multi_args(**kw)
    r = lib.kda_decode_commit(a["state"], a["q"], a["k"], a["v"], a["la"], a["beta"], a["n_accept"], a["N"],
                              a["n"], a["H"], a["dk"], a["dv"], a["dt"], a["flags"], None)
    assert r == code


def test_input_flag_errors(lib):
    import gated_delta_rule_107_amd as g
    p = g.Plan(1, 0)
    p.flags = 4                                                      # unknown bit
    assert call_chunk(lib, plan=p) == UNSUP
    assert "flags" in lib.kda_last_error().decode()
    with pytest.raises(g.KdaError) as e:                             # the binding's own check
        g._flags(7, False)
    assert e.value.code == UNSUP
    assert g._flags(g.GATE_LOGITS, True) == g.FLAG_GATE_LOGITS | g.FLAG_QK_L2NORM


@needs_lib
def test_python_binding_rejects_cpu_tensors():
    import gated_delta_rule_107_amd as g
    import torch
    q = torch.zeros(1, 16, 1, 16)
    with pytest.raises(g.KdaError):
        g.chunk_fwd(q, q, q, q, torch.zeros(1, 16, 1))
