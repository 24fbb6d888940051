"""Checks on the gfx950 code the attention kernels compile to (CPU only:
hipcc cross-compiles without a GPU).

* The loads into LDS are issued from inline asm that sets M0 itself. That
  is only sound while nothing else in those kernels uses M0, so every M0
  access must be an `s_mov_b32 m0, sN` directly followed by the
  `buffer_load_dwordx4 ... lds` it serves.
* The attention kernels must not spill to scratch: a spill in the key loop
  costs far more than it saves.
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


def test_attention_kernels_do_not_spill(asm):
    sizes = dict(re.findall(r"\.set (_ZN3lsh\S*attn_(?:fwd|bwd)\S*)\.private_seg_size, (\d+)", asm))
    assert sizes, "no attention kernels found"
    for name, size in sizes.items():
        assert int(size) == 0, (name, size)
