"""The gfx950 machine code never touches the destination of an LDS read that
may still be in flight.

Some kernels read k-major fragments with ``ds_read_b64_tr_b16`` written as
inline assembly, so that the compiler does not make those reads wait for the
direct-to-LDS loads in flight. The compiler's wait insertion does not see such
a read either: the kernel source issues ``s_waitcnt lgkmcnt(0)`` itself before
the fragments are used. Nothing in the source stops the compiler from placing a
register copy of a fragment (to assemble a 4-register MFMA operand, say)
between the read and that wait, and the hardware does not interlock a VGPR
whose LDS read has not returned: such a copy would take a stale value. This
test disassembles the built code objects and proves, over each function's
control-flow graph, that every instruction that reads or writes the
destination registers of an LDS read comes after a wait that has retired it.

The model: LDS operations return in issue order, and ``s_waitcnt lgkmcnt(N)``
retires every LDS operation that has at least N younger LDS operations (scalar
memory loads only make that wait stricter). A planted missing wait must be
found, so the check is not vacuous. Runs on the CPU over what the build wrote.
"""
import collections
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OBJ = os.path.join(ROOT, "mma_fragment_layouts_amd", "_build")
LLVM = os.environ.get("ROCM_PATH", "/opt/rocm") + "/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
CAP = 64  # younger-op counts saturate here; lgkmcnt's field is far smaller

_REG = re.compile(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out.update((m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
        else:
            out.add((m.group(4), int(m.group(5))))
    return frozenset(out)


def _parse(listing):
    """{function: [instruction dicts]} from llvm-objdump -d text."""
    funcs, cur = collections.OrderedDict(), None
    for line in listing.splitlines():
        m = re.match(r"^[0-9a-f]+ <(.*)>:", line)
        if m:
            cur = funcs.setdefault(m.group(1), [])
            continue
        if cur is None or "//" not in line:
            continue
        code, comment = line.split("//", 1)
        code = code.strip()
        am = re.match(r"\s*([0-9A-F]+):", comment)
        if not code or not am:
            continue
        tm = re.search(r"<(.*)\+0x([0-9a-f]+)>", comment)
        mn, _, ops = code.partition(" ")
        cur.append({"addr": int(am.group(1), 16), "mn": mn, "ops": ops.strip(), "text": code,
                    "tgt": (tm.group(1), int(tm.group(2), 16)) if tm else None})
    return funcs


def _hazards(name, ins):
    """Instructions that touch the destination of a possibly outstanding LDS read."""
    base = ins[0]["addr"]
    at = {x["addr"]: i for i, x in enumerate(ins)}
    succ = []
    for i, x in enumerate(ins):
        s, mn = [], x["mn"]
        if mn.startswith("s_cbranch") or mn == "s_branch":
            if x["tgt"] and x["tgt"][0] == name:
                s.append(at[base + x["tgt"][1]])
            if mn != "s_branch" and i + 1 < len(ins):
                s.append(i + 1)
        elif mn not in ("s_endpgm", "s_setpc_b64") and i + 1 < len(ins):
            s.append(i + 1)
        succ.append(s)
    # state: LDS op address -> (destination registers, fewest younger LDS ops on any path)
    state_in = [None] * len(ins)
    state_in[0] = {}
    work = collections.deque([0])
    found = {}
    while work:
        i = work.popleft()
        x, st = ins[i], dict(state_in[i])
        if x["mn"] == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", x["ops"])
            if m:
                st = {k: v for k, v in st.items() if v[1] < int(m.group(1))}
        else:
            touched = _regs(x["ops"])
            for k, (dest, _) in st.items():
                if dest & touched:
                    found[x["addr"]] = (x["text"], k)
            if x["mn"].startswith("ds_"):
                st = {k: (d, min(y + 1, CAP)) for k, (d, y) in st.items()}
                writes = x["mn"].startswith(("ds_write", "ds_store"))
                st[x["addr"]] = (frozenset() if writes or not x["ops"] else _regs(x["ops"].split(",")[0]), 0)
        for j in succ[i]:
            old = state_in[j]
            new = dict(st) if old is None else dict(old)
            if old is not None:
                for k, v in st.items():
                    new[k] = (v[0], min(v[1], new[k][1])) if k in new else v
            if new != old:
                state_in[j] = new
                work.append(j)
    return found


@pytest.fixture(scope="module")
def listings(tmp_path_factory):
    tmp_path = tmp_path_factory.mktemp("isa")
    tools = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump")]
    if not all(os.path.exists(t) for t in tools):
        pytest.skip("LLVM tools of the ROCm install not found")
    if not os.path.isdir(OBJ):
        pytest.skip("library not built (run the build first)")
    objcopy, bundler, objdump = tools
    out = {}
    for f in sorted(os.listdir(OBJ)):
        if not f.endswith(".o"):
            continue
        fat, co = tmp_path / (f + ".fatbin"), tmp_path / (f + ".co")
        r = subprocess.run([objcopy, "--dump-section=.hip_fatbin=" + str(fat), os.path.join(OBJ, f)],
                           capture_output=True)
        if r.returncode != 0:  # host-only translation unit
            continue
        subprocess.run([bundler, "--unbundle", "--type=o", "--input=" + str(fat), "--targets=" + TARGET,
                        "--output=" + str(co)], check=True, capture_output=True)
        out[f] = subprocess.run([objdump, "-d", "--mcpu=gfx950", str(co)], check=True,
                                capture_output=True, text=True).stdout
    if not out:
        pytest.skip("no device code objects under the build folder")
    return out


def test_no_use_of_outstanding_lds_reads(listings):
    tr_reads, bad = 0, []
    for f, text in listings.items():
        tr_reads += text.count("ds_read_b64_tr_b16")
        for name, ins in _parse(text).items():
            if ins:
                bad += [(f, name, hex(a), t, hex(k)) for a, (t, k) in _hazards(name, ins).items()]
    assert tr_reads > 0, "no transpose reads found: the check would be vacuous"
    assert not bad, "\n".join(map(str, bad[:20]))


def test_planted_missing_wait_is_found(listings):
    """Drop, in one function, the first full LDS wait after its transpose reads:
    the analysis must then report a hazard in that function."""
    for text in listings.values():
        for name, ins in _parse(text).items():
            first = next((i for i, x in enumerate(ins) if x["mn"] == "ds_read_b64_tr_b16"), None)
            if first is None:
                continue
            wait = next(i for i in range(first, len(ins))
                        if ins[i]["mn"] == "s_waitcnt" and "lgkmcnt(0)" in ins[i]["ops"])
            planted = [dict(x) for x in ins]
            planted[wait] = dict(planted[wait], mn="s_nop", ops="0", text="s_nop 0")
            assert not _hazards(name, ins)
            assert _hazards(name, planted), name
            return
    pytest.fail("no function with transpose reads")
