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
* The dK/dV kernel's query loop copies nothing out of AGPRs: only its
  accumulators live there, pinned by an asm MFMA.
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
    the elementwise step would pay for)."""
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
