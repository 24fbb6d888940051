"""Checks on the gfx950 code the attention kernels compile to (CPU only:
hipcc cross-compiles without a GPU).

* The loads into LDS are issued from inline asm that sets M0 itself. That
  is only sound while nothing else in those kernels uses M0, so every M0
  access must be an `s_mov_b32 m0, sN` directly followed by the
  `buffer_load_dwordx4 ... lds` it serves.
* The attention kernels must not touch scratch memory inside a loop: a
  spill in the key loop costs far more than it saves. A few spilled words
  outside the loops (values that live across the key loop but are not used
  in it) cost nothing measurable and are allowed, up to 64 bytes.
* The dK/dV kernel's query loop copies nothing out of AGPRs: its
  accumulators live there, pinned by an asm MFMA (the loop may also keep
  fragments in AGPRs; it only never copies them back to VGPRs).
* The compiler's hazard checks do not see into that asm MFMA, so the code
  around it is checked here, over the kernel's control flow: no write of one
  of its operands (accumulator AGPRs, A and B VGPRs) within the 2 wait
  states before it, and no access to its accumulator AGPRs within the 19
  wait states after it (the distance a 16-pass MFMA result needs; another
  such MFMA accumulating into the same registers excepted).
* Inside the key and query loops (the loops that issue MFMAs), a wait on
  the vector-memory counter may only come right before a barrier. The tile
  loads into LDS are inline asm the compiler does not count, so a wait it
  inserts for a load it does see (say, of Q) would also wait for the tiles
  loaded ahead. (Loops without MFMAs, such as the copy of a block-sparse
  row's kept-block list before the first tile load, are not concerned.)
"""
import os
import re
import subprocess

import pytest

from long_sequence_head_amd import build as B

SOURCES = ["attn_fwd.hip", "attn_bwd.hip", "attn_bwd_dq.hip"]


def _hipcc():
    try:
        return B.hipcc()
    except RuntimeError:
        return None


@pytest.fixture(scope="module", params=SOURCES)
def asm(request, tmp_path_factory):
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    src = request.param
    out = tmp_path_factory.mktemp("asm") / (src + ".s")
    cmd = [cc] + [f for f in B.common_flags() if f not in ("-fPIC",)] + \
        B.FILE_FLAGS.get(src, []) + ["-S", "--cuda-device-only", os.path.join(B.CSRC, src),
                                     "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _functions(text):
    parts = re.split(r"\n(?=_ZN3lsh\S+:)", text)
    return {p.split(":", 1)[0]: p for p in parts if p.startswith("_ZN3lsh")}


def _code_lines(body):
    return [l.strip() for l in body.split("\n")
            if l.strip() and not l.strip().startswith(";") and not l.strip().startswith(".")]


def test_m0_only_feeds_lds_loads(asm):
    funcs = _functions(asm)
    assert any(k in n for n in funcs for k in ("attn_fwd_bf16", "attn_bwd_dkdv", "attn_bwd_dq"))
    for name, body in funcs.items():
        lines = _code_lines(body)
        for i, l in enumerate(lines):
            if not re.search(r"\bm0\b", l):
                continue
            assert re.fullmatch(r"s_mov_b32 m0, s\d+", l), (name, l)
            nxt = lines[i + 1] if i + 1 < len(lines) else ""
            assert nxt.startswith("buffer_load_dwordx4") and nxt.endswith(" lds"), (name, l, nxt)


def _loops(lines):
    """(header, back-edge) line ranges of the loops the compiler annotated."""
    labels = {l.split(":")[0]: i for i, l in enumerate(lines) if re.match(r"^\.LBB\d+_\d+:", l)}
    out = []
    for i, l in enumerate(lines):
        m = re.search(r"s_c?branch\S*\s+(\.LBB\d+_\d+)", l)
        if m and m.group(1) in labels and labels[m.group(1)] < i and \
                "Loop Header" in lines[labels[m.group(1)]]:
            out.append((labels[m.group(1)], i))
    return out


def _attention_bodies(asm):
    funcs = _functions(asm)
    bodies = {n: b.split("\n") for n, b in funcs.items()
              if re.search(r"attn_(fwd|bwd)\w*_kernel", n) and "empty" not in n}
    assert bodies, "no attention kernels found"
    return bodies


def test_attention_kernels_do_not_spill_in_loops(asm):
    sizes = dict(re.findall(r"\.set (_ZN3lsh\S*attn_(?:fwd|bwd)\S*)\.private_seg_size, (\d+)", asm))
    assert sizes, "no attention kernels found"
    for name, size in sizes.items():
        assert int(size) <= 64, (name, size)
    for name, lines in _attention_bodies(asm).items():
        for a, b in _loops(lines):
            bad = [l.strip() for l in lines[a:b + 1] if "scratch_" in l or "buffer_store" in l]
            assert not bad, (name, bad[:3])


def test_vmcnt_waits_in_loops_only_before_barriers(asm):
    for name, lines in _attention_bodies(asm).items():
        loops = _loops(lines)
        if re.search(r"bf16|dkdv|bwd_dq", name):   # the kernels with a key or query loop
            assert loops, (name, "no loop found")
        for a, b in loops:
            code = [l.split(";")[0].strip() for l in lines[a:b + 1]]
            code = [l for l in code if l]
            if not any(l.startswith("v_mfma") for l in code):
                continue
            for i, l in enumerate(code):
                if l.startswith("s_waitcnt") and "vmcnt" in l:
                    # the next instruction, skipping labels and the scalar
                    # branch bookkeeping of the wait's own if/else, is the
                    # barrier
                    rest = [x for x in code[i + 1:i + 10]
                            if not re.match(r"\.LBB\d+_\d+:", x) and not x.split()[0].startswith(
                                ("s_branch", "s_cbranch", "s_mov_b64", "s_andn2_b64", "s_and_b64",
                                 "s_waitcnt"))]
                    assert rest and rest[0] == "s_barrier", (name, l, code[i + 1:i + 4])


def test_dkdv_loop_reads_no_agprs(asm):
    """The dK/dV kernel keeps its accumulators in AGPRs through an asm MFMA
    and every other MFMA result in VGPRs, so its query loop must not copy
    values out of AGPRs (each `v_accvgpr_read` there is a VALU instruction
    the elementwise step would pay for). The rest of the kernel may: the
    accumulators are copied out after the loop, and the hazards of those
    copies are checked by test_dkdv_asm_mfma_hazard_distances."""
    bodies = {n: l for n, l in _attention_bodies(asm).items() if "dkdv" in n}
    if not bodies:
        pytest.skip("no dK/dV kernel in this file")
    for name, lines in bodies.items():
        loops = _loops(lines)
        assert loops, (name, "no loop found")
        for a, b in loops:
            bad = [l.strip() for l in lines[a:b + 1] if "v_accvgpr_read" in l]
            assert not bad, (name, len(bad), bad[:3])
            mfma = [l for l in lines[a:b + 1] if "v_mfma_f32_32x32x16_bf16" in l]
            assert any(re.search(r"v_mfma\S*\s+a\[", l) for l in mfma), (name, "no AGPR accumulator")


_AREG = re.compile(r"\ba\[(\d+):(\d+)\]|\ba(\d+)\b")
_VREG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def _regset(rx, text):
    out = set()
    for m in rx.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _blocks(lines):
    """Basic blocks of a function body: lists of instruction strings, with
    successor indices (fall-through and branch targets)."""
    code = [l.split(";")[0].strip() for l in lines]
    code = [l for l in code if l and (not l.startswith(".") or re.match(r"^\.LBB\d+_\d+:", l))]
    blocks, labels, cur = [], {}, []
    for l in code:
        if re.match(r"^\.LBB\d+_\d+:", l):
            if cur:
                blocks.append(cur)
            cur = []
            labels[l[:-1]] = len(blocks)
            continue
        cur.append(l)
        if l.startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
            blocks.append(cur)
            cur = []
    if cur:
        blocks.append(cur)
    # labels point at the block that starts after them
    succ = []
    for i, b in enumerate(blocks):
        s_ = set()
        last = b[-1] if b else ""
        m = re.match(r"s_c?branch\S*\s+(\.LBB\d+_\d+)", last)
        if m and m.group(1) in labels:
            s_.add(labels[m.group(1)])
        if not last.startswith(("s_branch", "s_endpgm", "s_setpc")) and i + 1 < len(blocks):
            s_.add(i + 1)
        succ.append(s_)
    pred = [set() for _ in blocks]
    for i, s_ in enumerate(succ):
        for j in s_:
            pred[j].add(i)
    return blocks, succ, pred


def _wait_states(ins):
    m = re.match(r"s_nop\s+(\d+)", ins)
    return int(m.group(1)) + 1 if m else 1


def _dst(ins):
    parts = ins.split(None, 1)
    return parts[1].split(",")[0] if len(parts) > 1 else ""


def _asm_mfma_hazards(lines, before=2, after=19):
    blocks, succ, pred = _blocks(lines)
    found = []
    for bi, blk in enumerate(blocks):
        for ii, ins in enumerate(blk):
            if not (ins.startswith("v_mfma") and _dst(ins).startswith("a[")):
                continue
            acc = _regset(_AREG, _dst(ins))
            srcs = _regset(_VREG, ins.split(",", 1)[1])
            # backwards: writes of an operand within `before` wait states
            stack = [(bi, ii - 1, 0)]
            seen = set()
            while stack:
                b, i, ws = stack.pop()
                while i >= 0 and ws < before:
                    p_ = blocks[b][i]
                    if p_.startswith("v_") or p_.startswith("ds_read") or p_.startswith("buffer_load"):
                        d = _dst(p_)
                        if (_regset(_AREG, d) & acc) or (p_.startswith("v_") and _regset(_VREG, d) & srcs):
                            found.append(("write before", ws, p_, ins))
                    ws += _wait_states(p_)
                    i -= 1
                if ws < before:
                    for pb in pred[b]:
                        if (pb, ws) not in seen:
                            seen.add((pb, ws))
                            stack.append((pb, len(blocks[pb]) - 1, ws))
            # forwards: accesses of the accumulators within `after` wait states
            stack = [(bi, ii + 1, 0)]
            seen = set()
            while stack:
                b, i, ws = stack.pop()
                while i < len(blocks[b]) and ws < after:
                    n_ = blocks[b][i]
                    same_chain = n_.startswith("v_mfma") and _regset(_AREG, _dst(n_)) == acc
                    if not same_chain and _regset(_AREG, n_) & acc:
                        found.append(("access after", ws, ins, n_))
                    ws += _wait_states(n_)
                    i += 1
                if ws < after and i >= len(blocks[b]):
                    for sb in succ[b]:
                        if (sb, ws) not in seen:
                            seen.add((sb, ws))
                            stack.append((sb, 0, ws))
    return found


def test_dkdv_asm_mfma_hazard_distances(asm):
    bodies = {n: l for n, l in _attention_bodies(asm).items() if "dkdv" in n}
    if not bodies:
        pytest.skip("no dK/dV kernel in this file")
    for name, lines in bodies.items():
        n_asm = sum(1 for l in lines if re.search(r"v_mfma\S*\s+a\[", l))
        assert n_asm > 0, (name, "no asm MFMA found")
        bad = _asm_mfma_hazards(lines)
        assert not bad, (name, len(bad), bad[:4])
