"""Source checks of the kernel's cross-task publication rule (CPU only).

Values that one task writes and another task reads, possibly on another XCD whose L2 is not
coherent with the writer's, must be written with agent-scope stores (pub(), st_relaxed,
st_relaxed64 or atomics): the notify that follows them is a relaxed atomic preceded by a
vmcnt(0) wait, with no L2 write-back, so a plain store left in the writer's L2 would be a
silent race.  These checks scan megakernel.hip for plain stores into the published arrays.
"""
import os
import re

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "..", "moe_groupgemm_amd", "csrc", "megakernel.hip")

# Workspace arrays read by tasks other than their writer (out is read only after the kernel
# ends, trace only by the host, so both may be written with plain stores).
PUBLISHED = ("h", "y", "yp", "perm", "inv", "amt", "logits", "topk_idx", "topk_w", "tile_hist",
             "hist", "indptr", "mt_base", "mt_expert", "mt_row0", "mt_rows", "qslots", "ev_logit", "ev_exp",
             "ev_h", "ev_d", "red_ctr", "ctl")


def _strip_comments(src):
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    return re.sub(r"//[^\n]*", " ", src)


def plain_stores(src):
    """(line, text) of every plain store into a published array, directly or through a
    non-const pointer initialised from one."""
    code = _strip_comments(src)
    arr = "|".join(PUBLISHED)
    assign = r"\s*=(?!=)"
    pats = [re.compile(r"P\.(?:%s)\s*\[[^\]]*\]%s" % (arr, assign)),
            re.compile(r"\*\s*\([^;]*\bP\.(?:%s)\b[^;]*\)%s" % (arr, assign))]
    alias = re.compile(r"(?<!const )MK_G\s+(?!const\b)[\w\s]*?\*\s*(\w+)\s*=\s*(?:\([^)]*\)\s*)?P\.(?:%s)\b" % arr)
    for name in set(alias.findall(code)):
        n = re.escape(name)
        pats += [re.compile(r"\b%s\s*\[[^\]]*\]%s" % (n, assign)),
                 re.compile(r"(?:^|[;{}])\s*\*\s*%s\b%s" % (n, assign)),
                 re.compile(r"\*\s*\(\s*[^;]*\b%s\b[^;]*\)%s" % (n, assign))]
    hits = []
    for i, line in enumerate(code.split("\n"), 1):
        if any(p.search(line) for p in pats):
            hits.append((i, line.strip()))
    return hits


def test_published_arrays_use_agent_scope_stores():
    with open(SRC) as fh:
        hits = plain_stores(fh.read())
    assert not hits, "plain stores into published arrays:\n" + "\n".join(f"  line {i}: {t}" for i, t in hits)


@pytest.mark.parametrize("snippet", [
    "P.perm[i] = v;",
    "*(MK_G uint32_t *)(P.h + (size_t)row * P.f + col) = hv;",
    "MK_G float *ys = P.yp + o;\n ys[j] = acc;",
    "MK_G int *q = (MK_G int *)P.inv;\n *q = 3;",
])
def test_scanner_finds_planted_plain_stores(snippet):
    assert plain_stores(snippet), snippet


@pytest.mark.parametrize("snippet", [
    "pub(P.perm + i, v);",
    "if (P.perm[i] == v) x = 1;",
    "const MK_G int *src = P.tile_hist + t;\n int v = src[3];",
    "*(MK_G u32x2 *)(P.out + o) = w;",
    "st_relaxed64(P.qslots + s, tag);",
])
def test_scanner_accepts_agent_scope_stores_and_reads(snippet):
    assert not plain_stores(snippet), snippet
