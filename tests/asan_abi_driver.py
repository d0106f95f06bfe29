"""Drive the host-side paths of a libm3 build through ctypes: every broken
rule of every entry point, the workspace queries, the segment override, the
allocation-free entry point's size refusal, and the thread-local error text
from several threads at once.  No call gets past validation, so no HIP work
is launched and no GPU is needed.

Run as `python asan_abi_driver.py LIB` with the AddressSanitizer runtime
preloaded (tests/test_abi_asan.py does this): any heap or stack error in the
C ABI layer then ends the process with the sanitizer's report.  Imports
neither torch nor the package, so that only the library runs instrumented.
"""

import ctypes
import sys
import threading

from abi_rules import MIMO_BAD, PRE_BAD, PRE_BASE, PRE_FIELDS, SISO_BAD, SSM_BASE, SSM_FIELDS

INVALID, UNSUPPORTED = 1, 2
P = ctypes.c_void_p
FAKE = P(0x1000)  # never dereferenced: validation rejects every call first
BIG = ctypes.c_size_t(1 << 40)


class CSsm(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in SSM_FIELDS]


class CPre(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in PRE_FIELDS[:6]] + [(n, ctypes.c_float) for n in PRE_FIELDS[6:]]


def ssm(**kw):
    d = dict(SSM_BASE)
    d.update(kw)
    return CSsm(*[int(d[f]) for f in SSM_FIELDS])


def pre(**kw):
    d = dict(PRE_BASE)
    d.update(kw)
    return CPre(*[int(d[f]) for f in PRE_FIELDS[:6]], *[float(d[f]) for f in PRE_FIELDS[6:]])


def main(path):
    L = ctypes.CDLL(path)
    L.m3_last_error.restype = ctypes.c_char_p
    L.m3_version.restype = ctypes.c_char_p
    for n in ("m3_siso_fwd_workspace_bytes", "m3_mimo_fwd_workspace_bytes", "m3_siso_bwd_workspace_bytes",
              "m3_mimo_bwd_workspace_bytes", "m3_siso_fwd_packed_workspace_bytes"):
        getattr(L, n).restype = ctypes.c_size_t
    L.m3_set_scan_segments.argtypes = [ctypes.c_uint32]
    L.m3_set_scan_segments.restype = None
    checks = 0

    def expect(status, want, prefix, rule):
        nonlocal checks
        msg = L.m3_last_error().decode()
        assert status == want and msg.startswith(prefix + ": ") and rule in msg, (status, msg, rule)
        checks += 1

    assert L.m3_version().decode().startswith("m3 ")
    for bad, rule in SISO_BAD:
        c = ssm(**bad)
        expect(L.m3_siso_fwd(*[FAKE] * 11, c, FAKE, FAKE, BIG, None), INVALID, "m3_siso_fwd", rule)
        expect(L.m3_siso_fwd_noalloc(*[FAKE] * 11, c, FAKE, None), INVALID, "m3_siso_fwd_noalloc", rule)
        expect(L.m3_siso_bwd(*[FAKE] * 12, c, *[FAKE] * 11, FAKE, BIG, None), INVALID, "m3_siso_bwd", rule)
        assert L.m3_siso_fwd_workspace_bytes(c) == 0 and L.m3_siso_bwd_workspace_bytes(c) == 0
    for bad, rule in MIMO_BAD:
        c = ssm(mimo_rank=2)
        for k, v in bad.items():
            setattr(c, k, int(v))
        expect(L.m3_mimo_fwd(*[FAKE] * 15, c, FAKE, FAKE, BIG, None), INVALID, "m3_mimo_fwd", rule)
        assert L.m3_mimo_fwd_workspace_bytes(c) == 0
    for bad, rule in PRE_BAD:
        expect(L.m3_preprocess(FAKE, FAKE, ctypes.c_uint32(16), pre(**bad), *[FAKE] * 8, None), INVALID,
               "m3_preprocess", rule)
    expect(L.m3_siso_step(*[FAKE] * 15, ssm(sequence_length=2), FAKE, None), INVALID, "m3_siso_step",
           "a decode step takes exactly one token")
    # the u32 element-count rule, and a workspace one byte short
    wide = ssm(batch_size=1 << 12, sequence_length=1 << 12, num_heads=2, num_groups=1, head_dim=128,
               state_size=16, num_rope_angles=0)
    expect(L.m3_siso_fwd(*[FAKE] * 11, wide, FAKE, FAKE, BIG, None), INVALID, "m3_siso_fwd",
           "element count does not fit in u32")
    long_seq = ssm(batch_size=1, num_heads=1, num_groups=1, sequence_length=8192, head_dim=64, state_size=128,
                   num_rope_angles=32)
    need = L.m3_siso_fwd_workspace_bytes(long_seq)
    assert need > 0
    expect(L.m3_siso_fwd(*[FAKE] * 11, long_seq, FAKE, FAKE, ctypes.c_size_t(need - 1), None), INVALID,
           "m3_siso_fwd", "workspace")
    # segment override: many plans, then the fixed-scratch refusal
    for n in (1, 2, 3, 7, 64, 255, 2000):
        L.m3_set_scan_segments(n)
        L.m3_siso_fwd_workspace_bytes(long_seq)
        L.m3_mimo_fwd_workspace_bytes(ssm(mimo_rank=4, sequence_length=4096, head_dim=64, state_size=128,
                                          num_rope_angles=32, num_heads=2, num_groups=1))
    big = ssm(batch_size=1, num_heads=1, num_groups=1, sequence_length=64000, head_dim=128, state_size=128,
              num_rope_angles=32)
    expect(L.m3_siso_fwd_noalloc(*[FAKE] * 11, big, FAKE, None), UNSUPPORTED, "m3_siso_fwd_noalloc",
           "fixed scratch holds 67108864")
    L.m3_set_scan_segments(0)
    # the packed call's workspace query over both configurations
    assert L.m3_siso_fwd_packed_workspace_bytes(pre(), ssm(num_groups=1, num_heads=4, head_dim=16,
                                                           state_size=16, num_rope_angles=4)) >= 0

    # thread-local error text: each thread sees its own last message
    errors = []

    def worker(i):
        try:
            for _ in range(200):
                bad, rule = SISO_BAD[i % len(SISO_BAD)]
                st = L.m3_siso_fwd(*[FAKE] * 11, ssm(**bad), FAKE, FAKE, BIG, None)
                msg = L.m3_last_error().decode()
                assert st == INVALID and rule in msg, msg
        except AssertionError as e:  # pragma: no cover
            errors.append(str(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]
    print(f"asan driver: {checks} rule checks and 8 x 200 threaded calls passed", flush=True)


if __name__ == "__main__":
    main(sys.argv[1])
