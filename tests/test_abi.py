"""Host-side checks of libm3.so: it loads, exports every function the header
declares, and rejects every broken geometry rule before any HIP call (these
calls run on a CPU-only host: validation never initialises the runtime)."""

import ctypes
import os
import subprocess

import pytest

import selective_state_space_mamba3_amd as m3
from selective_state_space_mamba3_amd import _binding as bd
from abi_rules import MIMO_BAD, PRE_BAD, PRE_BASE, SISO_BAD, SSM_BASE

INVALID = bd.M3_ERR_INVALID_ARGUMENT
FAKE = 0x1000  # never dereferenced: every call below is rejected by validation


def _lib():
    try:
        return m3.lib()
    except ImportError as e:  # pragma: no cover
        pytest.fail(str(e))


def test_library_exports_every_header_function():
    names = m3.header_functions()
    assert set(names) >= {"m3_preprocess", "m3_siso_fwd", "m3_mimo_fwd", "m3_siso_step", "m3_set_scan_segments",
                          "m3_mimo_step", "m3_siso_bwd", "m3_preprocess_bwd", "m3_siso_fwd_packed",
                          "m3_mimo_bwd", "m3_mimo_bwd_workspace_bytes",
                          "m3_siso_bwd_workspace_bytes", "m3_last_error", "m3_siso_fwd_workspace_bytes",
                          "m3_mimo_fwd_workspace_bytes", "m3_version"}
    L = _lib()
    for n in names:
        assert hasattr(L, n), f"libm3.so does not export {n}"
    out = subprocess.run(["nm", "-D", "--defined-only", m3.LIB_PATH], capture_output=True, text=True)
    exported = {ln.split()[-1] for ln in out.stdout.splitlines() if ln.strip()}
    assert set(names) <= exported
    assert L.m3_version().decode().startswith("m3 ")


def _ssm(**kw):
    base = dict(SSM_BASE)
    base.update(kw)
    return bd.SsmConfig(**base)


def _siso_call(cfg, ptrs=None, ws=FAKE, ws_bytes=1 << 40):
    L = _lib()
    p = ptrs if ptrs is not None else [FAKE] * 11
    return L.m3_siso_fwd(*p, bd.c_ssm(cfg), FAKE, ws, ws_bytes, None)




@pytest.mark.parametrize("bad,rule", SISO_BAD)
def test_siso_rejects_broken_geometry(bad, rule):
    assert _siso_call(_ssm(**bad)) == INVALID
    msg = m3.last_error()
    assert msg.startswith("m3_siso_fwd: ") and rule in msg, msg


def test_siso_rejects_flags_and_null_operands():
    L = _lib()
    c = bd.c_ssm(_ssm())
    c.has_z = 2
    assert L.m3_siso_fwd(*[FAKE] * 11, c, FAKE, FAKE, 1 << 40, None) == INVALID
    assert "flag has_z is 2" in m3.last_error()
    for i in range(11):
        p = [FAKE] * 11
        p[i] = None
        st = _siso_call(_ssm(), p)
        if i == 7:  # angle
            assert st == INVALID and "angle" in m3.last_error()
        else:
            assert st == INVALID and "NULL" in m3.last_error()
    # angle may be NULL only without rotary pairs; then the call passes validation, so only
    # check the error text of the other case here (a valid call would launch a kernel)
    assert L.m3_siso_fwd(*[FAKE] * 11, bd.c_ssm(_ssm()), None, FAKE, 1 << 40, None) == INVALID


def test_u32_element_count_limit():
    # B*L*H*P = 2^32 exceeds the u32 element-count limit
    cfg = _ssm(batch_size=1 << 12, sequence_length=1 << 12, num_heads=2, num_groups=1,
               head_dim=128, state_size=16, num_rope_angles=0)
    assert _siso_call(cfg) == INVALID
    assert "the x / z / out element count does not fit in u32" in m3.last_error()


def test_workspace_rule():
    cfg = _ssm(batch_size=1, num_heads=1, num_groups=1, sequence_length=8192, head_dim=64,
               state_size=128, num_rope_angles=32)
    need = m3.siso_fwd_workspace_bytes(cfg)
    assert need > 0  # one (batch, head) over a long sequence is split into segments
    assert _siso_call(cfg, ws=None, ws_bytes=0) == INVALID
    assert "workspace" in m3.last_error()
    assert _siso_call(cfg, ws=FAKE, ws_bytes=need - 1) == INVALID
    # a broken configuration reports zero workspace
    assert m3.siso_fwd_workspace_bytes(_ssm(batch_size=0)) == 0


def test_scan_segment_override():
    # the plan override changes the segment count, and with it the summary
    # workspace, on this thread only; 0 restores the automatic plan
    cfg = _ssm(batch_size=1, num_heads=1, num_groups=1, sequence_length=4096, head_dim=64,
               state_size=128, num_rope_angles=32)
    auto = m3.siso_fwd_workspace_bytes(cfg)
    with m3.scan_segments(1):
        assert m3.siso_fwd_workspace_bytes(cfg) == 0
    with m3.scan_segments(3):
        three = m3.siso_fwd_workspace_bytes(cfg)
    with m3.scan_segments(5):
        five = m3.siso_fwd_workspace_bytes(cfg)
    assert 0 < three < five
    assert m3.siso_fwd_workspace_bytes(cfg) == auto
    import threading
    seen = {}
    with m3.scan_segments(1):
        th = threading.Thread(target=lambda: seen.setdefault("ws", m3.siso_fwd_workspace_bytes(cfg)))
        th.start()
        th.join()
    assert seen["ws"] == auto


def test_noalloc_rules():
    # same validation as m3_siso_fwd, and a clear refusal (before any HIP
    # call) when the plan's workspace exceeds the fixed 64 MiB scratch
    L = _lib()
    for bad, rule in SISO_BAD:
        assert L.m3_siso_fwd_noalloc(*[FAKE] * 11, bd.c_ssm(_ssm(**bad)), FAKE, None) == INVALID
        msg = m3.last_error()
        assert msg.startswith("m3_siso_fwd_noalloc: ") and rule in msg, msg
    big = _ssm(batch_size=1, num_heads=1, num_groups=1, sequence_length=64000, head_dim=128,
               state_size=128, num_rope_angles=32)
    with m3.scan_segments(2000):
        need = m3.siso_fwd_workspace_bytes(big)
        assert need > 64 << 20
        assert L.m3_siso_fwd_noalloc(*[FAKE] * 11, bd.c_ssm(big), FAKE, None) == bd.M3_ERR_UNSUPPORTED
    assert "fixed scratch holds 67108864" in m3.last_error()




@pytest.mark.parametrize("bad,rule", MIMO_BAD)
def test_mimo_rejects_broken_geometry(bad, rule):
    L = _lib()
    c = bd.c_ssm(_ssm(mimo_rank=2))
    for k, v in bad.items():
        setattr(c, k, int(v))
    assert L.m3_mimo_fwd(*[FAKE] * 15, c, FAKE, FAKE, 1 << 40, None) == INVALID
    msg = m3.last_error()
    assert msg.startswith("m3_mimo_fwd: ") and rule in msg, msg


def test_mimo_lifts_the_pn_cap_and_checks_pointers():
    L = _lib()
    # P*N = 128*128 > 4096 is accepted by validation; the NULL norm_weight is what fails
    cfg = _ssm(mimo_rank=4, head_dim=128, state_size=128, has_output_norm=True)
    p = [FAKE] * 15
    p[14] = None
    assert L.m3_mimo_fwd(*p, bd.c_ssm(cfg), FAKE, FAKE, 1 << 40, None) == INVALID
    assert "norm_weight" in m3.last_error()


def test_step_rules():
    L = _lib()
    cfg = _ssm(sequence_length=2)
    args = [FAKE] * 15
    assert L.m3_siso_step(*args, bd.c_ssm(cfg), FAKE, None) == INVALID
    assert "sequence_length is 2; a decode step takes exactly one token" in m3.last_error()
    for i in (11, 13, 14):  # ssm_state, k_state, v_state
        a = list(args)
        a[i] = None
        assert L.m3_siso_step(*a, bd.c_ssm(_ssm(sequence_length=1)), FAKE, None) == INVALID
    a = list(args)
    a[12] = None  # angle_state with A > 0
    assert L.m3_siso_step(*a, bd.c_ssm(_ssm(sequence_length=1)), FAKE, None) == INVALID
    assert L.m3_siso_step(*args, bd.c_ssm(_ssm(sequence_length=1, mimo_rank=2)), FAKE, None) == INVALID


def test_mimo_step_rules():
    L = _lib()
    args = [FAKE] * 19
    one = _ssm(sequence_length=1, mimo_rank=2)
    assert L.m3_mimo_step(*args, bd.c_ssm(_ssm(sequence_length=2, mimo_rank=2)), FAKE, None) == INVALID
    assert "sequence_length is 2; a decode step takes exactly one token" in m3.last_error()
    for i in (15, 17, 18):  # ssm_state, k_state, v_state
        a = list(args)
        a[i] = None
        assert L.m3_mimo_step(*a, bd.c_ssm(one), FAKE, None) == INVALID
    a = list(args)
    a[16] = None  # angle_state with A > 0
    assert L.m3_mimo_step(*a, bd.c_ssm(one), FAKE, None) == INVALID
    a = list(args)
    a[14] = None  # norm_weight must be valid even without the norm
    assert L.m3_mimo_step(*a, bd.c_ssm(one), FAKE, None) == INVALID
    for rank in (0, 9):
        assert L.m3_mimo_step(*args, bd.c_ssm(_ssm(sequence_length=1, mimo_rank=rank)), FAKE, None) == INVALID
    assert L.m3_mimo_step(*args, bd.c_ssm(one), None, None) == INVALID  # out


def _pre(**kw):
    base = dict(PRE_BASE)
    base.update(kw)
    return bd.PreprocessConfig(**base)




@pytest.mark.parametrize("bad,rule", PRE_BAD)
def test_preprocess_rejects_broken_config(bad, rule):
    L = _lib()
    assert L.m3_preprocess(FAKE, FAKE, 16, bd.c_pre(_pre(**bad)), *[FAKE] * 8, None) == INVALID
    msg = m3.last_error()
    assert msg.startswith("m3_preprocess: ") and rule in msg, msg


def test_preprocess_rejects_empty_rows_and_nulls():
    L = _lib()
    assert L.m3_preprocess(FAKE, FAKE, 0, bd.c_pre(_pre()), *[FAKE] * 8, None) == INVALID
    assert "rows is 0" in m3.last_error()
    for i in range(10):
        p = [FAKE] * 10
        p[i] = None
        assert L.m3_preprocess(p[0], p[1], 16, bd.c_pre(_pre()), *p[2:], None) == INVALID


@pytest.mark.parametrize("bad,rule", SISO_BAD)
def test_siso_bwd_rejects_broken_geometry(bad, rule):
    L = _lib()
    cfg = bd.c_ssm(_ssm(**bad))
    assert L.m3_siso_bwd(*[FAKE] * 12, cfg, *[FAKE] * 11, FAKE, 1 << 40, None) == INVALID
    msg = m3.last_error()
    assert msg.startswith("m3_siso_bwd: ") and rule in msg, msg
    assert L.m3_siso_bwd_workspace_bytes(cfg) == 0


def test_siso_bwd_rules():
    L = _lib()
    cfg = _ssm()
    c = bd.c_ssm(cfg)
    need = L.m3_siso_bwd_workspace_bytes(c)
    # theta, two [BH, nc, P, N] state buffers, two [B, L, H, N] adjoints, ... (B2 L8 H4 P16 N32 A8)
    assert need >= 4 * (2 * 2 * 4 * 1 * 16 * 32 + 2 * 2 * 8 * 4 * 32)
    for i in range(23):  # every operand and gradient except angle / d_angle
        if i in (8, 19):
            continue
        p = [FAKE] * 23
        p[i] = None
        assert L.m3_siso_bwd(*p[:12], c, *p[12:], FAKE, need, None) == INVALID, i
    for i in (8, 19):  # angle, d_angle with A > 0
        p = [FAKE] * 23
        p[i] = None
        assert L.m3_siso_bwd(*p[:12], c, *p[12:], FAKE, need, None) == INVALID
    assert L.m3_siso_bwd(*[FAKE] * 12, c, *[FAKE] * 11, FAKE, need - 1, None) == INVALID
    assert "workspace" in m3.last_error()
    assert L.m3_siso_bwd(*[FAKE] * 12, c, *[FAKE] * 11, None, need, None) == INVALID
    big = bd.c_ssm(_ssm(num_heads=256, num_groups=1, state_size=128, num_rope_angles=8))  # 256 heads share a group
    assert L.m3_siso_bwd(*[FAKE] * 12, big, *[FAKE] * 11, FAKE, 1 << 40, None) == bd.M3_ERR_UNSUPPORTED
    assert "LDS" in m3.last_error()
    assert L.m3_siso_bwd_workspace_bytes(big) > 0


def test_mimo_bwd_rules():
    L = _lib()
    cfg = bd.c_ssm(_ssm(mimo_rank=3, has_output_norm=True))
    need = L.m3_mimo_bwd_workspace_bytes(cfg)
    assert need > 0
    call = lambda p, c, ws=FAKE, nb=need: L.m3_mimo_bwd(*p[:16], c, *p[16:], ws, nb, None)
    for i in range(31):  # every operand and gradient except angle (8) and d_angle (23)
        if i in (8, 23):
            continue
        p = [FAKE] * 31
        p[i] = None
        assert call(p, cfg) == INVALID, i
    for i in (8, 23):
        p = [FAKE] * 31
        p[i] = None
        assert call(p, cfg) == INVALID
    assert call([FAKE] * 31, cfg, nb=need - 1) == INVALID
    assert "workspace" in m3.last_error()
    assert call([FAKE] * 31, cfg, ws=None) == INVALID
    for bad, rule in MIMO_BAD[:4]:
        assert call([FAKE] * 31, bd.c_ssm(_ssm(**bad))) == INVALID, bad
        assert rule in m3.last_error()
        assert L.m3_mimo_bwd_workspace_bytes(bd.c_ssm(_ssm(**bad))) == 0
    big = bd.c_ssm(_ssm(num_heads=256, num_groups=1, state_size=128, mimo_rank=4))
    assert call([FAKE] * 31, big, nb=1 << 40) == bd.M3_ERR_UNSUPPORTED


@pytest.mark.parametrize("bad,rule", PRE_BAD)
def test_preprocess_bwd_rejects_broken_config(bad, rule):
    L = _lib()
    assert L.m3_preprocess_bwd(FAKE, FAKE, 16, bd.c_pre(_pre(**bad)), *[FAKE] * 8, FAKE, FAKE, None) == INVALID
    msg = m3.last_error()
    assert msg.startswith("m3_preprocess_bwd: ") and rule in msg, msg


def test_preprocess_bwd_null_rules():
    L = _lib()
    assert L.m3_preprocess_bwd(FAKE, FAKE, 0, bd.c_pre(_pre()), *[FAKE] * 8, FAKE, FAKE, None) == INVALID
    for i in (0, 1, 10, 11):  # projected, dt_bias, d_projected, d_dt_bias
        p = [FAKE] * 12
        p[i] = None
        assert L.m3_preprocess_bwd(p[0], p[1], 16, bd.c_pre(_pre()), *p[2:], None) == INVALID


def _packed_pre(cfg, **kw):
    base = dict(inner_size=cfg.num_heads * cfg.head_dim, state_size=cfg.state_size, num_heads=cfg.num_heads,
                num_rope_angles=cfg.num_rope_angles, num_groups=cfg.num_groups or cfg.num_heads, mimo_rank=1,
                epsilon=1e-5, dt_min=1e-3, dt_max=0.1, a_floor=1e-4)
    base.update(kw)
    return bd.PreprocessConfig(**base)


def test_siso_fwd_packed_rules():
    L = _lib()
    cfg = _ssm()
    pc = _packed_pre(cfg)
    need = L.m3_siso_fwd_packed_workspace_bytes(bd.c_pre(pc), bd.c_ssm(cfg))
    rows = cfg.batch_size * cfg.sequence_length
    assert need >= 4 * rows * (2 * cfg.num_groups * cfg.state_size + 2 * cfg.num_heads)
    call = lambda p, c, s, ws=FAKE, nb=need: L.m3_siso_fwd_packed(*p, bd.c_pre(c), bd.c_ssm(s), FAKE, ws, nb, None)
    for bad, rule in ((dict(inner_size=cfg.num_heads * cfg.head_dim + 4), "inner_size 68 differs from num_heads * head_dim = 64"),
                      (dict(state_size=16), "state_size is 16 in the preprocess config but 32 in the scan config"),
                      (dict(num_heads=2), "num_heads is 2 in the preprocess config but 4"),
                      (dict(num_rope_angles=4), "num_rope_angles is 4 in the preprocess config but 8"),
                      (dict(num_groups=1), "num_groups is 1 in the preprocess config but 2"),
                      (dict(mimo_rank=2), "the preprocess config has mimo_rank 2"), (dict(epsilon=0.0), "epsilon is 0")):
        assert call([FAKE] * 5, _packed_pre(cfg, **bad), cfg) == INVALID, bad
        msg = m3.last_error()
        assert msg.startswith("m3_siso_fwd_packed: ") and rule in msg, msg
        assert L.m3_siso_fwd_packed_workspace_bytes(bd.c_pre(_packed_pre(cfg, **bad)), bd.c_ssm(cfg)) == 0
    for bad, rule in SISO_BAD:
        assert call([FAKE] * 5, pc, _ssm(**bad)) == INVALID
        assert rule in m3.last_error()
    for i in range(5):
        p = [FAKE] * 5
        p[i] = None
        assert call(p, pc, cfg) == INVALID
    assert call([FAKE] * 5, pc, cfg, ws=None) == INVALID
    assert call([FAKE] * 5, pc, cfg, nb=need - 1) == INVALID
    assert "workspace" in m3.last_error()
    # num_groups 0 in the scan config resolves to one group per head
    cfg0 = _ssm(num_groups=0)
    assert L.m3_siso_fwd_packed_workspace_bytes(bd.c_pre(_packed_pre(cfg0)), bd.c_ssm(cfg0)) > 0


def test_error_is_thread_local_and_cleared():
    import threading
    _siso_call(_ssm(batch_size=0))
    seen = {}

    def other():
        seen["msg"] = m3.last_error()
    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["msg"] == ""
    assert m3.last_error() != ""


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(bd, "_LIB", None)
    monkeypatch.setattr(bd, "LIB_PATH", str(tmp_path / "libm3.so"))
    with pytest.raises(ImportError):
        bd.lib()


def test_validation_does_not_initialise_hip():
    # A rejected call in a fresh process must not touch the GPU runtime: the
    # process may have no device at all.
    code = (
        "import ctypes, sys\n"
        f"L = ctypes.CDLL({m3.LIB_PATH!r})\n"
        "class C(ctypes.Structure):\n"
        "    _fields_ = [(n, ctypes.c_uint32) for n in 'abcdefghijk']\n"
        "c = C(0, 8, 4, 1, 16, 32, 8, 1, 1, 1, 0)\n"
        "r = L.m3_siso_fwd(*([ctypes.c_void_p(4096)] * 11), c, ctypes.c_void_p(4096), None,"
        " ctypes.c_size_t(0), None)\n"
        "sys.exit(0 if r == 1 else 3)\n")
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1")
    assert subprocess.run(["python", "-c", code], env=env).returncode == 0
