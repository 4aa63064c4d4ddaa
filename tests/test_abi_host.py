"""Host-side checks of the C ABI: loading, exported symbols, validation and
workspace sizing.  Validation runs before anything is enqueued, so these
calls need no GPU; no call here reaches a kernel launch."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")
HEADERS = [HEADER, os.path.join(ROOT, "include", "dspark_instr.h")]


@pytest.fixture(scope="module")
def ds():
    from draft_sampling_verification_markov_amd import dspark
    if not os.path.exists(dspark.LIB_PATH):
        from draft_sampling_verification_markov_amd import build
        build.build()
    dspark.load()
    return dspark


def _declared(headers=HEADERS):
    text = "".join(open(h).read() for h in headers)
    return sorted(set(re.findall(r"\b(dspark_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert _declared([HEADER]) == sorted(["dspark_draft", "dspark_schedule", "dspark_schedule_async",
                                          "dspark_schedule_fixed", "dspark_schedule_threshold", "dspark_sts_fit",
                                          "dspark_sts_workspace_bytes", "dspark_verify", "dspark_workspace_bytes",
                                          "dspark_status_string", "dspark_rnn_workspace_bytes", "dspark_draft_rnn",
                                          "dspark_verify_rnn", "dspark_schedule_noalloc"])
    # instrumentation, outside the step's contract
    assert _declared([HEADERS[1]]) == ["dspark_debug_check_inputs", "dspark_debug_flags",
                                       "dspark_debug_force_barrier_timeout", "dspark_draft_path",
                                       "dspark_draft_timed", "dspark_probe_draws"]


def test_status_codes_are_the_contract(ds):
    # the five codes of the boundary's contract keep their values; the pointer
    # error is appended after them
    text = open(HEADER).read()
    codes = {m.group(1): int(m.group(2)) for m in re.finditer(r"DSPARK_(OK|E_[A-Z]+)\s*=\s*(-?\d+)", text)}
    assert codes == {"OK": 0, "E_INVALID": -1, "E_DTYPE": -2, "E_UNSUPPORTED": -3, "E_WORKSPACE": -4,
                     "E_LAUNCH": -5, "E_POINTER": -6}
    assert (ds.OK, ds.E_INVALID, ds.E_DTYPE, ds.E_UNSUPPORTED, ds.E_WORKSPACE, ds.E_LAUNCH, ds.E_POINTER) == \
        (0, -1, -2, -3, -4, -5, -6)
    assert ds.status_string(-5) == "kernel launch failed"
    assert ds.status_string(-6) == "null or misaligned pointer argument"


@pytest.mark.parametrize("debug", [False, True], ids=["libdspark", "libdspark_debug"])
def test_library_exports_every_declared_symbol(ds, debug):
    path = ds.DEBUG_LIB_PATH if debug else ds.LIB_PATH
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True)
    exported = set(re.findall(r"\sT\s(dspark_\w+)", out.stdout))
    for name in _declared():
        assert name in exported, name
        assert hasattr(ds.load(debug), name)
    assert set(ds.SYMBOLS) == set(_declared())
    # one roctx range per ABI call
    undefined = subprocess.run(["nm", "-D", "--undefined-only", path], capture_output=True, text=True,
                               check=True).stdout
    assert "roctxRangePushA" in undefined and "roctxRangePop" in undefined


def test_debug_entry_points(ds):
    # the ordinary library has no debug checks; the debug library validates
    # before touching a device
    plain, debug = ds.load(False), ds.load(True)
    flags = ctypes.c_uint32()
    assert plain.dspark_debug_flags(ctypes.byref(flags), 0) == ds.E_UNSUPPORTED
    assert plain.dspark_debug_check_inputs(ctypes.byref(_P(ds)), None, None, None, None, None) == ds.E_UNSUPPORTED
    assert plain.dspark_debug_force_barrier_timeout(1) == ds.E_UNSUPPORTED
    assert debug.dspark_debug_force_barrier_timeout(0) == ds.OK
    assert debug.dspark_debug_flags(None, 0) == ds.E_POINTER
    assert debug.dspark_debug_check_inputs(None, None, None, None, None, None) == ds.E_POINTER
    assert debug.dspark_debug_check_inputs(ctypes.byref(_P(ds, B=0)), None, None, None, None, None) == ds.E_INVALID
    assert debug.dspark_debug_check_inputs(ctypes.byref(_P(ds)), ctypes.c_void_p(0x1008), None, None, None,
                                           None) == ds.E_POINTER
    assert (ds.DEBUG_LOGITS, ds.DEBUG_FACTORS, ds.DEBUG_IDS, ds.DEBUG_SCHEDULE_INPUT, ds.DEBUG_OUTPUT,
            ds.DEBUG_BARRIER_TIMEOUT) == (1, 2, 4, 8, 16, 32)


def test_header_compiles_as_c():
    src = ('#include "dspark.h"\n#include "dspark_instr.h"\n'
           'int main(void){ dspark_problem p; (void)p; return (int)sizeof(dspark_problem); }\n')
    r = subprocess.run(["gcc", "-x", "c", "-std=c99", "-fsyntax-only", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", "-"], input=src, text=True,
                       capture_output=True)
    assert r.returncode == 0, r.stderr


def test_problem_struct_layout(ds):
    assert ctypes.sizeof(ds.Problem) == 48
    assert ds.Problem.seed.offset == 40


def _P(ds, **kw):
    base = dict(B=256, K=16, V=151936, r=256, d=4096)
    base.update(kw)
    return ds.Problem.make(base["B"], base["K"], base["V"], base["r"], base["d"],
                           kw.get("logits", "bf16"), kw.get("weights", "bf16"), kw.get("hidden", "bf16"),
                           kw.get("T_s", 1.0), 0)


def test_workspace_bytes(ds):
    P = _P(ds)
    n = ds.workspace_bytes(P)
    G = 238   # 1,187 chunks: 238 workgroups of at most 5
    nseg = (151936 + 8191) // 8192
    assert n >= 256 * G * 16 + 256 * 16 * nseg * 8
    assert n % 256 == 0
    assert ds.workspace_bytes(_P(ds, B=1024, K=32)) > n
    assert ds.workspace_bytes(_P(ds, V=100)) == 0          # V % 8 != 0
    assert ds.workspace_bytes(_P(ds, r=48)) == 0           # unsupported rank


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), -1), (dict(K=0), -1), (dict(K=65), -1), (dict(V=4), -1), (dict(V=1004), -1),
    (dict(d=0), -1), (dict(d=12), -1), (dict(r=0), -1), (dict(B=65537), -1), (dict(B=32768, K=64), -1),
    (dict(T_s=0.0), -1), (dict(T_s=float("inf")), -1), (dict(T_s=float("nan")), -1),
    (dict(r=48), -3), (dict(r=512), -3), (dict(r=128, weights="f32"), -3),
])
def test_draft_rejects_bad_problems(ds, kw, code):
    lib = ds.load()
    P = _P(ds, **kw)
    st = lib.dspark_draft(ctypes.byref(P), *([None] * 5), ctypes.c_float(0), *([None] * 8), 0, None)
    assert st == code, ds.status_string(st)


def test_draft_schedule_arguments(ds):
    # an unknown schedule is rejected before anything else; the schedule query
    # rejects what dspark_draft rejects and reports the per-position schedule
    # where the persistent one cannot apply or is slower (256 rows of fp32
    # logits, rank 128, 257 rows)
    lib = ds.load()
    P = _P(ds)
    for bad in (-1, 3, 7):
        st = lib.dspark_draft_timed(ctypes.byref(P), *([None] * 5), ctypes.c_float(0), *([None] * 8), 0, None,
                                    None, 0, bad)
        assert st == ds.E_INVALID, ds.status_string(st)
    # event counts: 0 without events, else 2 or 2 + 2K
    ev = (ctypes.c_void_p * 40)()
    for n, events in ((2, None), (0, ev), (3, ev), (2 + 2 * 16 + 2, ev)):
        st = lib.dspark_draft_timed(ctypes.byref(P), *([None] * 5), ctypes.c_float(0), *([None] * 8), 0, None,
                                    events, n, 0)
        assert st == ds.E_INVALID, (n, ds.status_string(st))
    assert lib.dspark_draft_path(ctypes.byref(_P(ds, B=0))) == ds.E_INVALID
    assert lib.dspark_draft_path(ctypes.byref(_P(ds, r=48))) == ds.E_UNSUPPORTED
    for kw in (dict(logits="f32"), dict(r=128), dict(B=257)):
        assert lib.dspark_draft_path(ctypes.byref(_P(ds, **kw))) == ds.DRAFT_PER_POSITION
    assert (ds.DRAFT_AUTO, ds.DRAFT_PER_POSITION, ds.DRAFT_PERSISTENT) == (0, 1, 2)


def test_bad_dtype_code(ds):
    lib = ds.load()
    P = _P(ds)
    P.hidden_dtype = 7
    st = lib.dspark_schedule(ctypes.byref(P), None, None, None, None, None, 0, None)
    assert st == ds.E_DTYPE


def test_null_and_misaligned_pointers(ds):
    lib = ds.load()
    P = _P(ds, B=4, K=2, V=1024, r=32, d=64)
    fake = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(14)]
    st = lib.dspark_draft(ctypes.byref(P), None, *fake[:4], ctypes.c_float(0), *fake[4:11], None, 0, None)
    assert st == ds.E_POINTER
    # misaligned logits (not 16-byte aligned)
    st = lib.dspark_draft(ctypes.byref(P), ctypes.c_void_p(0x1004), *fake[:4], ctypes.c_float(0), *fake[4:11],
                          ctypes.c_void_p(0x10000), 1 << 20, None)
    assert st == ds.E_POINTER
    st = lib.dspark_verify(ctypes.byref(P), *fake[:9], None, *fake[10:14], ctypes.c_void_p(0x10000), 1 << 20, None)
    assert st == ds.E_POINTER
    st = lib.dspark_schedule(ctypes.byref(P), None, fake[0], fake[1], fake[2], ctypes.c_void_p(0x10000), 1 << 20,
                             None)
    assert st == ds.E_POINTER
    # the asynchronous scheduler: missing lagged survivals, then a misaligned count buffer
    st = lib.dspark_schedule_async(ctypes.byref(P), None, *fake[:4], ctypes.c_void_p(0x10000), 1 << 20, None)
    assert st == ds.E_POINTER
    st = lib.dspark_schedule_async(ctypes.byref(P), *fake[:3], ctypes.c_void_p(0x1002), fake[4],
                                   ctypes.c_void_p(0x10000), 1 << 20, None)
    assert st == ds.E_POINTER


def test_baseline_schedulers_validate(ds):
    lib = ds.load()
    P = _P(ds, B=4, K=3, V=1024, r=32, d=64)
    fake = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(3)]
    assert lib.dspark_schedule_fixed(ctypes.byref(P), -1, fake[0], fake[1], None) == ds.E_INVALID
    assert lib.dspark_schedule_fixed(ctypes.byref(P), 4, fake[0], fake[1], None) == ds.E_INVALID
    assert lib.dspark_schedule_fixed(ctypes.byref(P), 2, None, fake[1], None) == ds.E_POINTER
    assert lib.dspark_schedule_fixed(ctypes.byref(P), 2, ctypes.c_void_p(0x1001), fake[1], None) == ds.E_POINTER
    assert lib.dspark_schedule_threshold(ctypes.byref(P), fake[0], ctypes.c_float(float("nan")), fake[1], fake[2],
                                         None) == ds.E_INVALID
    assert lib.dspark_schedule_threshold(ctypes.byref(P), None, ctypes.c_float(0.5), fake[1], fake[2],
                                         None) == ds.E_POINTER


def test_rnn_validation(ds):
    lib = ds.load()
    P = _P(ds)
    assert ds.rnn_workspace_bytes(P) == ds.workspace_bytes(P) + ((256 * 16 * 3 * 256 * 4 + 255) // 256) * 256
    f = [ctypes.c_void_p(0x10000 * (i + 1)) for i in range(24)]
    ws = ctypes.c_void_p(0x40000000)
    need = ds.rnn_workspace_bytes(P)

    def draft(P, wsb=need, **kw):
        a = list(f[:9]) + [ctypes.c_float(0.0)] + list(f[9:16]) + [kw.get("state", f[17])]
        return lib.dspark_draft_rnn(ctypes.byref(P), *a, ws, wsb, None)
    # fp32 logits or hidden states, or r not a multiple of 32: no RNN kernels
    assert draft(_P(ds, logits="f32")) == ds.E_UNSUPPORTED
    assert draft(_P(ds, hidden="f32")) == ds.E_UNSUPPORTED
    assert draft(_P(ds, r=16)) == ds.E_UNSUPPORTED
    assert draft(P, state=None) == ds.E_POINTER
    assert draft(P, state=ctypes.c_void_p(0x10008)) == ds.E_POINTER
    assert draft(P, wsb=ds.workspace_bytes(P)) == ds.E_WORKSPACE  # the Markov size lacks the gate region

    def verify(P, state):
        a = list(f[:8]) + [state] + list(f[8:14])
        return lib.dspark_verify_rnn(ctypes.byref(P), *a, ws, ds.workspace_bytes(P), None)
    assert verify(P, None) == ds.E_POINTER
    assert verify(_P(ds, weights="f32"), f[20]) == ds.E_UNSUPPORTED


def test_sts_validation(ds):
    lib = ds.load()
    assert lib.dspark_sts_workspace_bytes(1000, 16, 129, 15) > 16 * 1000 * 8
    for bad in [(-1, 4, 8, 15), (10, 0, 8, 15), (10, 4, 0, 15), (10, 4, 8, 0), (10, 4, 8, 17), (10, 4, 5000, 15)]:
        assert lib.dspark_sts_workspace_bytes(*bad) == 0
    f = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(10)]
    ws = ctypes.c_void_p(0x100000)
    need = lib.dspark_sts_workspace_bytes(10, 4, 8, 15)
    ok = dict(M=10, K=4, c=f[0], a=f[1], n=f[2], g=f[3], G=8, nb=15, t=f[4], i=f[5], ef=f[6], er=f[7])

    def call(**kw):
        a = {**ok, **kw}
        return lib.dspark_sts_fit(a["M"], a["K"], a["c"], a["a"], a["n"], a["g"], a["G"], a["nb"], a["t"], a["i"],
                                  a["ef"], a["er"], kw.get("ws", ws), kw.get("wsb", need), None)
    assert call(nb=17) == ds.E_INVALID
    assert call(K=0) == ds.E_INVALID
    assert call(g=None) == ds.E_POINTER
    assert call(c=None) == ds.E_POINTER
    assert call(t=ctypes.c_void_p(0x1004)) == ds.E_POINTER   # float64 output needs 8-byte alignment
    assert call(ws=None) == ds.E_WORKSPACE
    assert call(wsb=need - 1) == ds.E_WORKSPACE
    assert call(ws=ctypes.c_void_p(0x100010)) == ds.E_WORKSPACE


def test_workspace_checks(ds):
    lib = ds.load()
    P = _P(ds, B=4, K=2, V=1024, r=32, d=64)
    need = ds.workspace_bytes(P)
    fake = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(4)]
    for ws, nbytes in ((None, need), (ctypes.c_void_p(0x10080), need), (ctypes.c_void_p(0x10000), need - 1)):
        st = lib.dspark_schedule(ctypes.byref(P), *fake, ws, nbytes, None)
        assert st == ds.E_WORKSPACE
        st = lib.dspark_schedule_async(ctypes.byref(P), fake[0], *fake, ws, nbytes, None)
        assert st == ds.E_WORKSPACE


def test_status_strings(ds):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert ds.status_string(code) and ds.status_string(code) != "unknown status"
    assert ds.status_string(42) == "unknown status"


def test_binding_refuses_host_tensors(ds):
    torch = pytest.importorskip("torch")
    P = _P(ds, B=1, K=1, V=8, r=16, d=8)
    t = torch.zeros(8)
    with pytest.raises(ValueError, match="device"):
        ds.schedule(P, t, t, t, t, t)
