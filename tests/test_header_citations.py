"""The boundary's declarations cite the passage that defines each operation.

Every entry point of include/shannonic.h that performs a step of the method carries, in
the comment above its declaration, the paper section of the Shannonic talk notes it
implements ("Preprocessing" 4.1, "Runtime encoding/decoding" 4.2, "Theorem 1" 4, the
section-5 metrics).  Size queries and messages carry none; an entry point for callers
that cannot allocate names those callers instead.
"""
from __future__ import annotations

import os
import re

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "shannonic.h")

# size queries, messages and plain data movement: no step of the method
UTILITY = {"sh_version", "sh_status_string", "sh_device_table_bytes", "sh_encode_bound",
           "sh_encode_workspace", "sh_build_tables_workspace",
           "sh_build_tables_batch_workspace", "sh_encode_batch_workspace",
           "sh_decode_stream_staging", "sh_tables_from_bytes", "sh_tables_from_device"}


def _declarations():
    """(name, comment block above it) for every function the header declares; functions
    declared back to back under one comment share it."""
    text = open(HEADER).read()
    body = text[text.index("extern \"C\" {"):]
    out = []
    comment = ""
    pos = 0
    token = re.compile(r"/\*.*?\*/|^[a-z_][^;{}]*?\b(sh_[a-z0-9_]+)\s*\([^;]*\);", re.S | re.M)
    for m in token.finditer(body):
        if m.group(0).startswith("/*"):
            comment = m.group(0)
        else:
            out.append((m.group(1), comment))
        pos = m.end()
    return out


def test_every_declaration_is_found():
    names = [n for n, _ in _declarations()]
    for must in ("sh_build_tables", "sh_encode", "sh_decode", "sh_stats", "sh_encode_batch",
                 "sh_decode_batch", "sh_build_tables_batch", "sh_histogram"):
        assert must in names


def test_every_method_entry_point_cites_a_section():
    missing = []
    for name, comment in _declarations():
        if name in UTILITY:
            continue
        cites = re.search(r"\bsections?\s+\d", comment) is not None
        no_alloc = "cannot allocate" in comment
        if not (cites or no_alloc):
            missing.append(name)
    assert not missing, f"no passage cited above: {missing}"
