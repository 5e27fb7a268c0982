"""Structure of the SNAC kernels in the gfx950 assembly (CPU only: hipcc
cross-compiles).

A persistent kernel whose loop contains barriers must leave that loop on a
wave-uniform branch. If the compiler instead builds a divergent loop (lanes
leave one at a time through `s_andn2_b64 exec, exec, ...`), lanes other than
the one that claims the next task re-read a stale ticket and never leave:
the kernel cannot terminate. The SNAC loop is written so that every branch
around a barrier is uniform; this test keeps it that way."""

import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "reduce_atom_03_amd", "csrc", "k_snac.hip")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("isa") / "k_snac.s"
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-x", "hip", "--cuda-device-only", "-S",
           SRC, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(r.stderr[-2000:])
    return out.read_text()


def _kernels(text):
    """(name, body) of every persistent k_snac kernel in the assembly."""
    out = []
    for m in re.finditer(r"^(_Z\S*k_snac\S*):", text, re.M):
        if "k_snac_tagged" in m.group(1):
            continue
        end = text.find("s_endpgm", m.end())
        out.append((m.group(1), text[m.end():end]))
    return out


def _tagged_kernels(text):
    """(name, whole body) of every k_snac_tagged kernel (small calls on the
    tagged ring)."""
    out = []
    for m in re.finditer(r"^(_Z\S*k_snac_tagged\S*):", text, re.M):
        end = text.find(".Lfunc_end", m.end())
        out.append((m.group(1), text[m.end():end]))
    return out


def test_every_snac_kernel_is_present(asm):
    names = [n for n, _ in _kernels(asm)]
    # 4 pipeline depths x 2 workgroup bounds (256, 512 lanes) x 2 element
    # types (the unit of the element-wise path)
    assert sum("StageCopy" in n for n in names) == 16
    # 2 dtypes x P = 1..16 x 2 workgroup bounds
    assert sum("StageReduce" in n for n in names) == 64


def _loops(body):
    """[start, end) character ranges of the loops in a kernel body: from a
    label to a later branch back to it."""
    labels = {m.group(1): m.start() for m in re.finditer(r"^(\.LBB\w+):", body, re.M)}
    out = []
    for m in re.finditer(r"^\s*s_(?:cbranch_\w+|branch)\s+(\.LBB\w+)", body, re.M):
        start = labels.get(m.group(1))
        if start is not None and start < m.start():
            out.append((start, m.end()))
    return out


def test_no_divergent_loop_exit(asm):
    """Lanes may leave a loop one at a time (the element-wise loops over a
    segment's elements do), but never a loop that contains a barrier: the
    innermost loop around every divergent exit (`s_andn2_b64 exec, exec`)
    holds no s_barrier."""
    for name, body in _kernels(asm):
        assert "s_barrier" in body
        loops = _loops(body)
        assert loops, f"{name}: no loop found"
        for m in re.finditer(r"s_andn2_b64\s+exec,\s*exec", body):
            around = [(a, b) for a, b in loops if a <= m.start() < b]
            if not around:
                continue
            a, b = min(around, key=lambda r: r[1] - r[0])
            assert "s_barrier" not in body[a:b], \
                f"{name}: a loop with barriers exits on a divergent branch"


def test_the_task_loop_is_uniform(asm):
    """The loop that claims tasks (the outermost one, holding the barriers)
    exits on a scalar condition, not on the exec mask."""
    for name, body in _kernels(asm):
        loops = [r for r in _loops(body) if "s_barrier" in body[r[0]:r[1]]]
        assert loops, name
        a, b = max(loops, key=lambda r: r[1] - r[0])
        branch = body[a:b].rstrip().splitlines()[-1]
        assert re.match(r"\s*s_(cbranch_scc[01]|branch)\b", branch), (name, branch)


def test_no_scratch(asm):
    for m in re.finditer(r"\.name:\s+(\S*k_snac\S*)\n(?:.*\n)*?\s+\.private_segment_fixed_size:\s+(\d+)", asm):
        assert int(m.group(2)) == 0, m.group(1)


def test_ring_hand_off_needs_no_l2_maintenance(asm):
    """The ring is read and written only with agent-coherent (sc1) buffer
    operations, so no SNAC kernel writes back or invalidates an L2. Inputs
    are read with ordinary global loads; outputs are written with buffer
    stores whose policy is an immediate: nt (streaming, the default) or
    none (ATOM_F_NO_NT), both present, never sc0 or sc1."""
    for name, body in _kernels(asm):
        assert not re.search(r"buffer_wbl2|buffer_inv", body), name
        loads = re.findall(r"^\s*(buffer_load_\w+[^\n]*)", body, re.M)
        stores = re.findall(r"^\s*(buffer_store_dwordx4[^\n]*)", body, re.M)
        narrow = re.findall(r"^\s*(buffer_store_(?:short|dword)\b[^\n]*)", body, re.M)
        assert loads, f"{name}: no ring loads"
        assert narrow, f"{name}: no element-wise ring stores"
        for op in loads + narrow:
            assert re.search(r"\bsc1\b", op), f"{name}: ring access without sc1: {op}"
        ring = [op for op in stores if re.search(r"\bsc1\b", op)]
        outs = [op for op in stores if not re.search(r"\bsc1\b", op)]
        assert ring, f"{name}: no ring stores"
        assert any(re.search(r"\bnt\b", op) for op in outs), f"{name}: no streaming output store"
        assert any(not re.search(r"\bnt\b", op) for op in outs), f"{name}: no ordinary output store"
        for op in outs:
            assert not re.search(r"\bsc0\b", op), f"{name}: output store with sc0: {op}"


def test_producer_waits_for_its_stores_before_notify(asm):
    """Each wave waits for vmcnt(0) after its last ring store and before the
    barrier that precedes the `ready` increment."""
    for name, body in _kernels(asm):
        last_store = max(m.end() for m in re.finditer(r"buffer_store_\w+[^\n]*\bsc1\b", body))
        rest = body[last_store:]
        wait = re.search(r"s_waitcnt vmcnt\(0\)", rest)
        barrier = re.search(r"s_barrier", rest)
        assert wait and barrier and wait.start() < barrier.start(), name


def test_every_tagged_kernel_is_present(asm):
    names = [n for n, _ in _tagged_kernels(asm)]
    assert sum("StageCopy" in n for n in names) == 1
    # 2 dtypes x P = 1..16, built for up to 512 lanes
    assert sum("StageReduce" in n for n in names) == 32


def _blocks(body):
    """(label line, instructions) of each basic block; the compiler marks a
    block that belongs to a loop in its label's comment ("Loop Header",
    "in Loop: Header=...", "Parent Loop ...")."""
    out, cur = [], None
    for line in body.splitlines():
        if re.match(r"^\.LBB\w+:", line):
            cur = [line, []]
            out.append(cur)
        elif cur is not None:
            cur[1].append(line)
    return out


def test_tagged_kernels_have_no_barrier_in_a_loop(asm):
    """The tagged kernel's waves poll on their own: the only barriers (the
    test hooks' jitter and clock stamps) sit in blocks that belong to no
    loop, so a wave that leaves a loop early can never hold up another at a
    barrier."""
    for name, body in _tagged_kernels(asm):
        assert "s_barrier" in body, name
        for label, ins in _blocks(body):
            if "Loop" in label:
                assert not any("s_barrier" in i for i in ins), f"{name}: a barrier inside a loop: {label}"


def test_tagged_words_are_agent_coherent(asm):
    """Every access to the tagged ring is a 64-bit agent-scope (sc1) load or
    store (single-copy atomic: a word and its tag are seen together; written
    through the L2, never read from a stale L2 line), the error word's too;
    no L2 write-back or invalidation; no ring (buffer) loads at all. Inputs
    are read with streaming loads, outputs written with stores without sc0
    or sc1."""
    for name, body in _tagged_kernels(asm):
        assert not re.search(r"buffer_wbl2|buffer_inv|buffer_load", body), name
        pairs = re.findall(r"^\s*(global_(?:load|store)_dwordx2[^\n]*)", body, re.M)
        assert any("load" in op for op in pairs) and any("store" in op for op in pairs), name
        for op in pairs + re.findall(r"^\s*(global_(?:load|store)_dword\s[^\n]*)", body, re.M):
            assert re.search(r"\bsc1\b", op), f"{name}: tag or error access without sc1: {op}"
        for op in re.findall(r"^\s*(global_load_dwordx4[^\n]*)", body, re.M):
            assert re.search(r"\bnt\b", op), f"{name}: input load that is not streaming: {op}"
        for op in re.findall(r"^\s*((?:buffer|global)_store_(?:dwordx4|short)[^\n]*)", body, re.M):
            assert not re.search(r"\bsc[01]\b", op), f"{name}: output store with sc0/sc1: {op}"
