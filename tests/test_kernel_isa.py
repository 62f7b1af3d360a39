"""The compiled kernels keep their tile copies in flight.

The compiler adds waits of its own in front of LDS reads and barriers, and
some of its rules turn copies that the loops mean to keep in flight into a
wait for everything. These tests compile the prefill and split-KV sources
to gfx950 assembly with the library's own flags and check the hot blocks:

* the prefill main block (the Sᵀ and PV MFMAs of a step) holds no
  `s_waitcnt vmcnt(0)` — its tile copies stay in flight until the next
  step's explicit wait — and its LDS operand waits are graded (some
  `lgkmcnt(N)` with N > 0), so operand reads issued ahead stay in flight;
* in the head-dim-128 prefill (two wave groups in ping-pong) each block
  holding a softmax slot and an MFMA slot keeps them apart: every
  exponential before the slot barrier, every MFMA after it (the compiler
  is free to move arithmetic across a barrier; explicit register pins stop
  it);
* the split-KV loop that keeps its copy ring full (two waves over a paged
  cache, the verify shape) reads no tile right behind a full drain
  (`s_waitcnt vmcnt(0) lgkmcnt(0)` in front of a `ds_read`): each tile read
  waits only through the loop's explicit wait. (The other split kernels
  drain at each tile on purpose.)

Needs only hipcc (no GPU); compiling both sources takes about a minute.
"""

import concurrent.futures as cf
import os
import re
import subprocess

import pytest

from gqa_flash_attention_amd import build

PREFILL_D128 = "_ZN5gqafa11attn_kernelILi128ELi8ELi64ELi1ELi3ELb0ELb0ELi2ELi0ELb0ELb0EEEvNS_8AttnArgsE"
PREFILL_D128_MASK = "_ZN5gqafa11attn_kernelILi128ELi4ELi64ELi1ELi2ELb0ELb0ELi2ELi2ELb0ELb0EEEvNS_8AttnArgsE"
SPLIT_D128_PAGED_TWO_WAVES = "_ZN5gqafa11attn_kernelILi128ELi2ELi32ELi1ELi2ELb1ELb1ELi2ELi0ELb0ELb0EEEvNS_8AttnArgsE"


def _asm(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, src.replace(".hip", ".s"))
    cmd = [build.HIPCC, *[f for f in build.FLAGS if f != "-fPIC"], "--cuda-device-only", "-S",
           os.path.join(build.CSRC, src), "-o", out]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        pytest.fail(f"hipcc failed for {src}:\n{p.stderr[-4000:]}")
    return open(out).read()


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not found")
    d = str(tmp_path_factory.mktemp("isa"))
    with cf.ThreadPoolExecutor(2) as ex:
        pre, spl = ex.map(lambda s: _asm(s, d), ["fa_prefill.hip", "fa_split_d128.hip"])
    return {"prefill": pre, "split": spl}


def _function(text: str, name: str) -> list[str]:
    lines = text.split("\n")
    start = next(i for i, l in enumerate(lines) if l.startswith(name + ":"))
    end = next(i for i in range(start, len(lines)) if lines[i].startswith(".Lfunc_end"))
    return lines[start:end]


def _blocks(body: list[str]) -> list[list[str]]:
    """Instruction lists of the basic blocks, in order."""
    blocks, cur = [], []
    for line in body:
        if re.match(r"^\.LBB\S+:", line):
            blocks.append(cur)
            cur = []
        elif line.startswith("\t") and not line.strip().startswith((";", ".")):
            cur.append(line.strip())
    blocks.append(cur)
    return blocks


def _loop(body: list[str]) -> list[str]:
    """Lines of the largest loop (a backward branch's span)."""
    labels = {}
    for i, line in enumerate(body):
        m = re.match(r"^(\.LBB\S+):", line)
        if m:
            labels[m.group(1)] = i
    best = None
    for i, line in enumerate(body):
        m = re.search(r"s_cbranch_\w+\s+(\.LBB\S+)|s_branch\s+(\.LBB\S+)", line)
        if m:
            tgt = m.group(1) or m.group(2)
            if tgt in labels and labels[tgt] < i and (best is None or i - labels[tgt] > best[1] - best[0]):
                best = (labels[tgt], i)
    assert best is not None, "no loop found"
    return body[best[0]:best[1] + 1]


@pytest.mark.parametrize("kernel", [PREFILL_D128, PREFILL_D128_MASK], ids=["ping_pong", "masked"])
def test_prefill_main_block_keeps_copies_and_reads_in_flight(asm, kernel):
    blocks = [b for b in _blocks(_function(asm["prefill"], kernel))
              if sum(i.startswith("v_mfma") for i in b) >= 32]
    assert blocks, "prefill main block (32 MFMAs) not found"
    for b in blocks:
        waits = [i for i in b if i.startswith("s_waitcnt")]
        assert not any(re.search(r"vmcnt\(0\)", w) for w in waits[:-1]), \
            "a tile-copy drain inside the prefill main block"
        graded = [w for w in waits if re.search(r"lgkmcnt\(([1-9]\d*)\)", w)]
        assert graded, "prefill operand reads wait for all LDS reads (lgkmcnt(0) only)"


def test_ping_pong_slots_stay_apart(asm):
    """In the ping-pong loop every stretch between two workgroup barriers is
    one slot: softmax work (exponentials, on the fast path or its rare
    fallback) or MFMA work, never both; one of each per ring position."""
    loop = [l.strip() for l in _loop(_function(asm["prefill"], PREFILL_D128))
            if l.startswith("\t") and not l.strip().startswith((";", "."))]
    segs, cur = [], []
    for ins in loop:
        if ins.startswith("s_barrier"):
            segs.append(cur)
            cur = []
        else:
            cur.append(ins)
    # the loop may be laid out rotated: its last stretch continues its first
    segs[0] = cur + segs[0]
    n_exp = [sum(i.startswith("v_exp") for i in g) for g in segs]
    n_mfma = [sum(i.startswith("v_mfma") for i in g) for g in segs]
    assert not any(e and m for e, m in zip(n_exp, n_mfma)), "softmax and MFMA work mixed inside one slot"
    assert sum(m >= 32 for m in n_mfma) == 3, "one MFMA slot (32 MFMAs) per ring position expected"
    assert sum(e >= 32 for e in n_exp) == 3, "one softmax slot (32 exponentials) per ring position expected"


def test_split_loop_reads_tiles_without_full_drain(asm):
    """Some barrier of the loop (the one handing a landed tile over) is
    reached from the ring's partial wait, vmcnt(N > 0), with no full drain
    in between; a fenced barrier would put a vmcnt(0) in front of each."""
    loop = [l.strip() for l in _loop(_function(asm["split"], SPLIT_D128_PAGED_TWO_WAVES))
            if l.startswith("\t") and not l.strip().startswith((";", "."))]
    last_vm, at_barrier = None, []
    for ins in loop:
        m = re.match(r"s_waitcnt\s.*vmcnt\((\d+)\)", ins)
        if m:
            last_vm = int(m.group(1))
        elif ins.startswith("s_barrier"):
            at_barrier.append(last_vm)
    assert at_barrier, "no barrier in the two-wave split loop"
    assert any(v is not None and v > 0 for v in at_barrier), \
        f"every barrier of the split loop follows a full drain: {at_barrier}"
