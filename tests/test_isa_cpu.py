"""Instruction order of the dot kernel with x in LDS, checked in the built
library.

That kernel waits for its buffer-to-LDS copies of x by counting: after the
copies each wave issues exactly CW * V loads of W, then s_waitcnt
vmcnt(CW * V) (loads complete in issue order) and a barrier.  The count is
only right while the compiler keeps that order.  This test disassembles the
gfx950 code object of every instantiation in libskinny_gemm.so (our own
build) and checks, between the last x copy and the first barrier after it:
no branch, every W load issued before the first vmcnt wait, and that wait no
larger than the loads issued after the last copy (the x copies have all
landed when it returns).  It also checks that no instantiation touches
scratch memory (register spills) and that the instantiations present are
exactly those the register bound admits.

The LDS-ring kernels (the tiled, whole-row and their FP8 forms) wait for a
stage the same way: the loop's s_waitcnt vmcnt must equal the loads of the
NS - 2 stages issued after it, which holds while each iteration issues the
same number of buffer-to-LDS loads and nothing else touches vmcnt in the
loop, and the prologue issues NS - 1 stages.  Those are checked for every
instantiation too.
"""
import os
import re
import struct
import subprocess
import tempfile

import pytest

import latency_skinny_gemm_amd as skg
from latency_skinny_gemm_amd import build as lib_build

LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
NAME = re.compile(r"^[0-9a-f]+ <(_ZN3skg11dotx_kernelILi(\d+)ELi(\d+)ELi(\d+)E\S*)>:\s*$")


def _gfx950_objects(fatbin):
    """The gfx950 code objects of a .hip_fatbin section (one offload bundle
    per compiled source: magic, entry count, then offset, size, triple)."""
    out, i = [], fatbin.find(MAGIC)
    while i >= 0:
        (n,) = struct.unpack_from("<Q", fatbin, i + 24)
        q = i + 32
        for _ in range(n):
            off, size, tl = struct.unpack_from("<QQQ", fatbin, q)
            q += 24
            triple = fatbin[q:q + tl].decode()
            q += tl
            if triple.endswith("gfx950"):
                out.append(fatbin[i + off:i + off + size])
        i = fatbin.find(MAGIC, i + 1)
    return out


RING = re.compile(r"^_ZN3skg(\d+)(rows_kernel|fp8_rows_kernel|tiled_kernel|fp8_tiled_kernel)I((?:L[ib]\d+E)+)E")


def _disassemble_all():
    """{mangled name: [(offset, text, branch target offset or None)]} over
    every gfx950 code object of the built library."""
    with tempfile.TemporaryDirectory() as d:
        fb = os.path.join(d, "fatbin")
        subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section",
                        f".hip_fatbin={fb}", skg.library_path()], check=True)
        funcs = {}
        for n, co in enumerate(_gfx950_objects(open(fb, "rb").read())):
            path = os.path.join(d, f"co{n}.o")
            open(path, "wb").write(co)
            dis = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", path],
                                 check=True, capture_output=True, text=True).stdout
            cur, start = None, 0
            for line in dis.splitlines():
                m = re.match(r"^([0-9a-f]+) <(\S+)>:\s*$", line)
                if m:
                    cur, start = m.group(2), int(m.group(1), 16)
                    funcs[cur] = []
                    continue
                if cur is not None and line.startswith("\t"):
                    text, _, comment = line.partition("//")
                    addr = re.match(r"\s*([0-9A-Fa-f]+):", comment)
                    if addr is None:  # the "..." that stands for a run of zero words
                        continue
                    tgt = re.search(r"<[^>+]*\+0x([0-9a-f]+)>", comment)
                    funcs[cur].append((int(addr.group(1), 16) - start, text.strip(),
                                       int(tgt.group(1), 16) if tgt else None))
    return funcs


@pytest.fixture(scope="module")
def all_functions():
    for tool in ("llvm-objcopy", "llvm-objdump"):
        if not os.path.exists(os.path.join(LLVM, tool)):
            pytest.skip(f"{tool} not installed")
    if not os.path.exists(skg.library_path()):
        lib_build.build()
    return _disassemble_all()


@pytest.fixture(scope="module")
def functions():
    """{(M, CW, V): [(offset, text, branch target offset or None)]}"""
    for tool in ("llvm-objcopy", "llvm-objdump"):
        if not os.path.exists(os.path.join(LLVM, tool)):
            pytest.skip(f"{tool} not installed")
    if not os.path.exists(skg.library_path()):
        lib_build.build()
    with tempfile.TemporaryDirectory() as d:
        fb = os.path.join(d, "fatbin")
        subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section",
                        f".hip_fatbin={fb}", skg.library_path()], check=True)
        objs = [o for o in _gfx950_objects(open(fb, "rb").read()) if b"dotx_kernel" in o]
        assert len(objs) == 1, "expected one code object holding the x-in-LDS dot kernels"
        co = os.path.join(d, "dot.co")
        open(co, "wb").write(objs[0])
        dis = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", co],
                             check=True, capture_output=True, text=True).stdout
    funcs, cur, start = {}, None, 0
    for line in dis.splitlines():
        m = NAME.match(line)
        if m:
            cur = (int(m.group(2)), int(m.group(3)), int(m.group(4)))
            start = int(line.split()[0], 16)
            funcs[cur] = []
            continue
        if re.match(r"^[0-9a-f]+ <", line):
            cur = None
        elif cur is not None and line.startswith("\t"):
            text, _, comment = line.partition("//")
            addr = re.match(r"\s*([0-9A-Fa-f]+):", comment)
            if addr is None:  # the "..." that stands for a run of zero words
                continue
            tgt = re.search(r"<[^>+]*\+0x([0-9a-f]+)>", comment)
            funcs[cur].append((int(addr.group(1), 16) - start, text.strip(),
                               int(tgt.group(1), 16) if tgt else None))
    return funcs


def _built(M, CW, V):
    # the register bound of the kernel (CW * V W vectors, one step's x
    # vectors, CW * M sums, addressing) and vmcnt's 6 bits
    return CW in (1, 2, 4) and CW * V * 4 + 4 * M + CW * M + 16 <= 224 and CW * V < 64


def test_instantiations_are_those_the_bound_admits(functions):
    want = {(M, CW, V) for M in range(1, 17) for CW in (1, 2, 4) for V in (4, 6, 8, 12, 14, 16)
            if _built(M, CW, V)}
    assert set(functions) == want


def _is_branch(text):
    return text.startswith(("s_branch", "s_cbranch", "s_setpc", "s_swappc"))


def test_w_loads_sit_between_x_copies_and_the_wait(functions):
    for (M, CW, V), ins in sorted(functions.items()):
        tag = f"dotx M={M} CW={CW} V={V}"
        texts = [t for _, t, _ in ins]
        offs = [o for o, _, _ in ins]
        assert not any(t.startswith("scratch_") for t in texts), f"{tag}: spills to scratch"
        copies = [k for k, t in enumerate(texts) if t.startswith("buffer_load") and t.endswith(" lds")]
        assert copies, f"{tag}: no buffer-to-LDS copy"
        s = copies[-1]
        bar = next(k for k in range(s, len(texts)) if texts[k].startswith("s_barrier"))
        wait, issued, first_w = None, 0, None
        for k in range(s + 1, bar):
            t = texts[k]
            if t.startswith(("buffer_load", "global_load")):
                issued += 1
                first_w = k if first_w is None else first_w
            m = re.match(r"s_waitcnt\b.*\bvmcnt\((\d+)\)", t)
            if m:
                wait = (k, int(m.group(1)))
                break
        assert wait is not None and first_w is not None, f"{tag}: no W loads and vmcnt wait"
        # past the last copy only backward branches into the copy region
        for k in range(s + 1, bar):
            if _is_branch(texts[k]):
                assert ins[k][2] is not None and ins[k][2] <= offs[s], \
                    f"{tag}: branch at +{offs[k]:#x} out of the load sequence"
        # no branch lands among the W loads or between the wait and the
        # barrier: every path to the barrier issues all of them, then waits
        for _, t, tgt in ins:
            if tgt is not None and _is_branch(t):
                assert not (offs[first_w] < tgt <= offs[bar]), \
                    f"{tag}: branch into the load sequence at +{tgt:#x}"
        assert wait[1] <= issued, f"{tag}: vmcnt({wait[1]}) with only {issued} loads after the copies"
        assert issued == CW * V and wait[1] == CW * V, f"{tag}: {issued} loads, vmcnt({wait[1]})"


def _is_vmem(text):
    return text.startswith(("buffer_", "global_", "flat_", "scratch_")) and \
        not text.startswith(("buffer_inv", "buffer_wbl2"))


def _is_epilogue_operand_load(text):
    # a load of the bias or a per-tensor scale into a VGPR, issued before
    # the ring (ahead of the epilogue that uses it); an older load only makes
    # the ring's in-order vmcnt waits stricter
    return re.match(r"buffer_load_(ushort|dword) v\d+, ", text) is not None and \
        not text.endswith(" lds")


def _ring_params(name):
    m = RING.match(name)
    args = [int(v) for v in re.findall(r"L[ib](\d+)E", m.group(3))]
    family = m.group(2)
    ns = args[2] if family in ("rows_kernel", "fp8_rows_kernel") else args[3]
    return family, args, ns


def _barrier_follows(texts, j):
    """An s_barrier after j, with no memory op, wait or branch in between."""
    for q in range(j + 1, len(texts)):
        if texts[q] == "s_barrier":
            return True
        if _is_vmem(texts[q]) or _is_branch(texts[q]) or texts[q].startswith(("s_waitcnt", "ds_")):
            return False
    return False


def _blocks(ins):
    """Basic blocks: {start index: (end index exclusive, successor start indices)}."""
    offs = [o for o, _, _ in ins]
    at = {o: k for k, o in enumerate(offs)}
    leaders = {0}
    for k, (o, t, tgt) in enumerate(ins):
        if _is_branch(t) or t.startswith("s_endpgm"):
            if k + 1 < len(ins):
                leaders.add(k + 1)
            if tgt is not None:
                leaders.add(at[tgt])
    starts = sorted(leaders)
    blocks = {}
    for a, b in zip(starts, starts[1:] + [len(ins)]):
        o, t, tgt = ins[b - 1]
        if t.startswith("s_endpgm"):
            succ = []
        elif t.startswith("s_branch"):
            succ = [at[tgt]]
        elif t.startswith("s_cbranch"):
            succ = [at[tgt]] + ([b] if b < len(ins) else [])
        elif t.startswith(("s_setpc", "s_swappc")):
            raise AssertionError("indirect branch")
        else:
            succ = [b] if b < len(ins) else []
        blocks[a] = (b, succ)
    return blocks


def _check_ring(ins, ns, tag):
    texts = [t for _, t, _ in ins]
    offs = [o for o, _, _ in ins]
    assert not any(t.startswith("scratch_") for t in texts), f"{tag}: spills to scratch"
    # the ring loop: the innermost back-edge whose body holds a vmcnt wait
    # followed by a barrier (other backward branches are out-of-line blocks
    # or the epilogue's loops)
    loops = []
    for k, (o, t, tgt) in enumerate(ins):
        if _is_branch(t) and tgt is not None and tgt < o:
            head = offs.index(tgt)
            waits = [j for j in range(head, k + 1)
                     if re.match(r"s_waitcnt\b.*\bvmcnt\(\d+\)", texts[j]) and _barrier_follows(texts, j)]
            if waits:
                loops.append((k - head, head, k, waits))
    assert loops, f"{tag}: no ring loop"
    _, head, back, waits = min(loops)
    # inside the loop: no branch but the latch (the back-edge, which may be
    # preceded by a conditional exit with only arithmetic after it), no
    # vector memory op but the ring's buffer-to-LDS loads
    for j in range(head, back):
        if _is_branch(texts[j]):
            exits = ins[j][2] is not None and ins[j][2] > offs[back]
            plain = not any(_is_vmem(t) or _is_branch(t) or
                            t.startswith(("ds_", "s_waitcnt", "s_barrier", "s_load", "s_buffer",
                                          "s_store", "s_dcache"))
                            for t in texts[j + 1:back])
            assert exits and plain, f"{tag}: branch inside the ring loop at +{offs[j]:#x}"
        if _is_vmem(texts[j]):
            assert texts[j].startswith("buffer_load") and texts[j].endswith(" lds"), \
                f"{tag}: '{texts[j]}' inside the ring loop"

    # each wait is followed, before the next wait or the back-edge, by the
    # stage's loads; all segments issue the same count, and nothing is issued
    # between the loop head and the first wait
    assert not any(_is_vmem(texts[j]) for j in range(head, waits[0])), f"{tag}: loads before the wait"
    ends = waits[1:] + [back]
    per = {sum(1 for j in range(w, e) if _is_vmem(texts[j])) for w, e in zip(waits, ends)}
    assert len(per) == 1, f"{tag}: iterations issue {per} loads"
    lpw = per.pop()
    assert lpw > 0
    for w in waits:
        x = int(re.search(r"vmcnt\((\d+)\)", texts[w]).group(1))
        assert x == (ns - 2) * lpw, f"{tag}: vmcnt({x}) with {lpw} loads a stage, NS = {ns}"
    # the prologue: on every path from the entry to the loop head, exactly
    # NS - 1 stages of ring loads and no other vector memory op but the
    # epilogue's operand loads (bias, scales) into VGPRs
    blocks = _blocks(ins)
    want = (ns - 1) * lpw
    # the blocks from which the loop head is reachable without entering the loop
    pred = {}
    for a, (_, succ) in blocks.items():
        for b in succ:
            pred.setdefault(b, []).append(a)
    reach, todo = {head}, [head]
    while todo:
        b = todo.pop()
        for a in pred.get(b, []):
            if a not in reach and not (head <= a <= back):
                reach.add(a)
                todo.append(a)
    assert 0 in reach, f"{tag}: the entry does not reach the ring loop"
    # prologue blocks on a cycle among themselves: loops before the ring (the
    # FP8 MX scale copies); the ring's own NS - 1 stages are straight-line
    def on_cycle(a):
        todo, seen_c = list(blocks[a][1]), set()
        while todo:
            b = todo.pop()
            if b == a:
                return True
            if b in seen_c or b not in reach or b == head:
                continue
            seen_c.add(b)
            todo.extend(blocks[b][1])
        return False
    cyclic = {a for a in reach if a != head and on_cycle(a)}
    seen, todo, arrive = set(), [(0, 0)], set()
    while todo:
        a, n = todo.pop()
        if (a, n) in seen:
            continue
        seen.add((a, n))
        assert n <= want, f"{tag}: a prologue path issues more than {want} loads"
        if a == head:
            arrive.add(n)
            continue
        end, succ = blocks[a]
        m = n
        for j in range(a, end):
            if _is_vmem(texts[j]):
                if _is_epilogue_operand_load(texts[j]) and a not in cyclic:
                    continue
                assert texts[j].startswith("buffer_load") and texts[j].endswith(" lds"), \
                    f"{tag}: '{texts[j]}' before the ring loop"
                if a not in cyclic:
                    m += 1
                else:
                    # other copies to LDS (the MX scale bytes) must precede the
                    # path's first ring load: the wait for the first stage
                    # then covers them
                    assert m == 0, f"{tag}: a copy to LDS after the ring's first load"
        for b in succ:
            if b in reach:  # other edges never reach the ring
                todo.append((b, m))
    assert arrive == {want}, f"{tag}: paths reach the ring with {sorted(arrive)} loads, want {want}"


def test_ring_kernels_wait_for_their_stage(all_functions):
    seen = {}
    for name, ins in sorted(all_functions.items()):
        if not RING.match(name):
            continue
        family, args, ns = _ring_params(name)
        seen[family] = seen.get(family, 0) + 1
        _check_ring(ins, ns, f"{family}<{', '.join(map(str, args))}>")
    assert set(seen) == {"rows_kernel", "fp8_rows_kernel", "tiled_kernel", "fp8_tiled_kernel"}, seen


def test_no_kernel_uses_scratch():
    # every kernel of the library keeps its state in registers and LDS: a
    # register spill shows as a private segment in the code object metadata
    for tool in ("llvm-objcopy", "llvm-readelf"):
        if not os.path.exists(os.path.join(LLVM, tool)):
            pytest.skip(f"{tool} not installed")
    if not os.path.exists(skg.library_path()):
        lib_build.build()
    with tempfile.TemporaryDirectory() as d:
        fb = os.path.join(d, "fatbin")
        subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section",
                        f".hip_fatbin={fb}", skg.library_path()], check=True)
        kernels, spilled = 0, []
        for n, co in enumerate(_gfx950_objects(open(fb, "rb").read())):
            path = os.path.join(d, f"co{n}.o")
            open(path, "wb").write(co)
            notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", path],
                                   check=True, capture_output=True, text=True).stdout
            names = re.findall(r"\.symbol:\s+(\S+)", notes)
            sizes = re.findall(r"\.private_segment_fixed_size:\s+(\d+)", notes)
            assert len(names) == len(sizes), "one private segment size per kernel"
            kernels += len(names)
            spilled += [nm for nm, sz in zip(names, sizes) if int(sz) > 0]
    assert kernels > 1000 and not spilled, spilled[:5]
