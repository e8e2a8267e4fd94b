"""The cross-workgroup publication order, checked in the gfx950 code the
compiler makes for it (CPU: hipcc -S, no GPU).

The single-launch kernels (la_fused.hip: the causal look-back; la_forward_bf16.hip:
the non-causal state / reduce / output hand-overs) publish data with
device-scope (sc1) buffer stores and announce it with a 64-bit flag store;
readers poll the flag and then load the data with sc1 buffer loads.  That
order rests on the instructions the compiler emits, not on language-level
fences, so these tests read the assembly of the library's own sources and
check, in every instantiation of those kernels:

- each flag store (global_store_dwordx2 ... sc1) follows a workgroup
  barrier, with no sc1 data store between that barrier and the flag, and an
  s_waitcnt vmcnt(0) between the last sc1 data store before the barrier and
  the barrier (the data has reached the device coherence point before any
  thread can set the flag);
- each sc1 data load follows an s_waitcnt vmcnt(0) issued after the last
  flag poll (global_load_dwordx2 ... sc1) before it, so the poll's value is
  known (and branched on) before the data is requested;
- the protocol is present at all: flag stores, sc1 data stores and sc1 data
  loads appear in every instantiation.

A compiler that dropped the sc1 bits, moved a flag store above the data's
completion or hoisted a data load above the poll fails here."""
import os
import re
import subprocess

import pytest

from linear_attention_phi_amd import build as labuild

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "linear_attention_phi_amd", "csrc")

FLAG = re.compile(r"^global_store_dwordx2\b.*\bsc1\b")
DSTORE = re.compile(r"^buffer_store_dword\S*\b.*\bsc1\b")
DLOAD = re.compile(r"^buffer_load_dword\S*\b.*\bsc1\b")
POLL = re.compile(r"^global_load_dwordx2\b.*\bsc1\b")


def _assembly(src, tmp_path):
    hipcc = labuild._hipcc()
    if not os.path.exists(hipcc):
        pytest.skip("hipcc is not installed")
    out = str(tmp_path / (os.path.basename(src) + ".s"))
    flags = [f for f in labuild._flags() if f != "-fPIC"] + ["--cuda-device-only", "-S"]
    res = subprocess.run([hipcc, *flags, os.path.join(CSRC, src), "-o", out], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return open(out).read()


def _kernels(text, stem):
    """Instruction lists (stripped lines) of the kernels whose symbol contains stem."""
    cur, out = None, {}
    for line in text.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            cur = m.group(1) if stem in m.group(1) else None
            if cur:
                out[cur] = []
            continue
        if cur is not None:
            s = line.strip()
            out[cur].append(s)
            if s.startswith("s_endpgm"):
                cur = None
    return out


def _violations(ins):
    errs = []
    flags = [i for i, s in enumerate(ins) if FLAG.match(s)]
    for i in flags:
        b = max((j for j in range(i) if ins[j].startswith("s_barrier")), default=None)
        if b is None:
            errs.append(f"flag store at {i}: no barrier before it")
            continue
        if any(DSTORE.match(ins[j]) for j in range(b, i)):
            errs.append(f"flag store at {i}: an sc1 data store between the barrier at {b} and the flag")
        s = max((j for j in range(b) if DSTORE.match(ins[j])), default=None)
        if s is not None and not any(ins[j].startswith("s_waitcnt") and "vmcnt(0)" in ins[j] for j in range(s, b)):
            errs.append(f"flag store at {i}: no vmcnt(0) between the sc1 data store at {s} and the barrier at {b}")
    loads = [i for i, s in enumerate(ins) if DLOAD.match(s)]
    for i in loads:
        p = max((j for j in range(i) if POLL.match(ins[j])), default=None)
        if p is not None and not any(ins[j].startswith("s_waitcnt") and "vmcnt(0)" in ins[j] for j in range(p, i)):
            errs.append(f"sc1 data load at {i}: no vmcnt(0) after the flag poll at {p}")
    counts = (len(flags), sum(1 for s in ins if DSTORE.match(s)), len(loads))
    return counts, errs


@pytest.mark.parametrize("src, stem, ninst", [("la_fused.hip", "k_causal_fused", 12),
                                              ("la_forward_bf16.hip", "k_fwd_one", 3)])
def test_publication_order_in_assembly(tmp_path, src, stem, ninst):
    kernels = _kernels(_assembly(src, tmp_path), stem)
    assert len(kernels) == ninst, sorted(kernels)
    for name, ins in kernels.items():
        (nflag, nstore, nload), errs = _violations(ins)
        assert nflag > 0 and nstore > 0 and nload > 0, (name, nflag, nstore, nload)
        assert not errs, (name, errs[:5])


def test_checker_rejects_a_misordered_flag():
    """The checks themselves: a flag store moved above the data's completion,
    and a data load moved above the poll's wait, are reported."""
    good = ["buffer_store_dwordx4 v[0:3], v4, s[0:3], 0 offen sc1", "s_waitcnt vmcnt(0)", "s_barrier",
            "global_store_dwordx2 v0, v[2:3], s[4:5] sc1", "global_load_dwordx2 v[6:7], v0, s[4:5] sc1",
            "s_waitcnt vmcnt(0)", "s_cbranch_scc1 .LBB0_1", "buffer_load_dwordx4 v[8:11], v4, s[0:3], 0 offen sc1"]
    assert _violations(good) == ((1, 1, 1), [])
    no_wait = [s for s in good[:3] if s != "s_waitcnt vmcnt(0)"] + good[3:]
    assert _violations(no_wait)[1]
    early_flag = [good[0], good[3], good[1], good[2]] + good[4:]
    assert _violations(early_flag)[1]
    early_load = good[:5] + [good[7], good[5], good[6]]
    assert _violations(early_load)[1]
