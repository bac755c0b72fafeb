"""The decode merge's publication order, pinned on the compiled code (CPU:
hipcc cross-compiles gfx950).

A decode work-group publishes its split record with agent-coherent (sc1)
stores and then takes a ticket with a relaxed agent-scope atomic; the last
arrival reads every record.  Relaxed atomics to different addresses carry
no ordering in the language's memory model, so the order rests on the
code the compiler emits: the record stores complete (a wait on the vector
memory counter) and the work-group meets at a barrier before the ticket
atomic is issued.  This test reads the gfx950 assembly of every decode
kernel instance and checks exactly that, so a compiler that moved the
ticket ahead of the stores, or dropped the wait, fails here instead of
racing on the GPU (where the poisoned-record determinism tests would catch
it only when the race shows)."""

import os
import re
import shutil
import subprocess

import pytest

from kv_cache_duo_amd import build as b

HIPCC = b.hipcc()


def _kernels(asm: str):
    """(name, body lines) of every decode_kernel instance."""
    out = []
    for m in re.finditer(r"^(_Z\w*decode_kernel\w*):.*?$(.*?)^\.Lfunc_end", asm, re.S | re.M):
        out.append((m.group(1), m.group(2).splitlines()))
    return out


def _target(inst: str):
    """(scalar base, offset) of a global access with a scalar base, else None."""
    m = re.search(r"(s\[\d+:\d+\])(?:\s+offset:(\d+))?", inst)
    return (m.group(1), int(m.group(2) or 0)) if m else None


@pytest.fixture(scope="module")
def decode_asm(tmp_path_factory):
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "decode.s"
    cmd = [HIPCC, *b.COMMON, "--cuda-device-only", "-S", "-x", "hip", os.path.join(b.CSRC, "decode.hip"),
           "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def test_record_stores_complete_before_every_ticket(decode_asm):
    kernels = _kernels(decode_asm)
    assert len(kernels) >= 16, "expected every decode_kernel instance"
    checked = 0
    for name, lines in kernels:
        last_store = None
        last_ticket = None  # (scalar base, offset) of the latest ticket atomic
        for i, ln in enumerate(lines):
            t = ln.strip()
            if t.startswith("global_store") and re.search(r"\bsc1\b", t):
                if _target(t) is not None and _target(t) == last_ticket:
                    continue  # the last arrival resetting that ticket: no record
                last_store = i
            elif t.startswith("global_atomic_add"):
                last_ticket = _target(t)
                if last_store is None:
                    continue  # a row claim, before any record
                between = [x.strip() for x in lines[last_store + 1:i]]
                waits = [x for x in between if x.startswith("s_waitcnt") and ("vmcnt(0)" in x or x == "s_waitcnt 0")]
                bar = [j for j, x in enumerate(between) if x == "s_barrier"]
                assert waits and bar, f"{name}: ticket atomic at line {i} without wait + barrier after the records"
                last_wait = max(j for j, x in enumerate(between) if x in waits)
                assert last_wait < max(bar), f"{name}: the barrier before the ticket precedes the store wait"
                checked += 1
    assert checked >= len(kernels), "every instance has at least one ticket after its record stores"


def test_no_fences_in_decode(decode_asm):
    """No L2 write-back or invalidate: agent-scope fences would add them (and
    cost far more than the merge)."""
    for name, lines in _kernels(decode_asm):
        body = "\n".join(lines)
        assert "buffer_wbl2" not in body and "buffer_inv" not in body, name
