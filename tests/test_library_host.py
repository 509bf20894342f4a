"""CPU checks of the HIP library: it loads without a GPU, exports every entry
point include/medusa.h declares, and its host-only tree construction (the
ancestor bitmask that the attention kernel consumes) equals the oracle's."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from medusa_tree_verification_amd import _lib, synth
from oracle import tree as otree

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "medusa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(medusa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmedusa_amd.so is not built; run __graft_entry__.build()")
    return _lib.load()


def test_header_declares_the_four_stages():
    names = declared_functions()
    for n in ["medusa_heads", "medusa_tree_candidates", "medusa_tree_attention",
              "medusa_accept_paths", "medusa_tree_create", "medusa_last_error"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if " T " in l)
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    # and the binding declares exactly those
    assert sorted(_lib.SIGNATURES) == declared_functions()


def test_version(lib):
    assert b"gfx950" in lib.medusa_version()


def _build_host(parent, rank, kpd):
    from medusa_tree_verification_amd import api
    return api.tree_build_host(parent, rank, kpd)


TREES = [("chain", synth.chain_tree(5), (1,) * 5),
         ("cart232", synth.cartesian_tree((2, 3, 2)), (2, 3, 2))]
for _name in synth.WORKLOAD_ORDER:
    _w = synth.WORKLOADS[_name]
    TREES.append((_name, synth.cost_ordered_tree(_w.topk, _w.T), _w.topk))
for _s in range(4):
    TREES.append((f"random{_s}", synth.random_tree(200, (8, 8, 6, 4, 3), _s), (8, 8, 6, 4, 3)))


@pytest.mark.parametrize("name,pr,kpd", TREES, ids=[t[0] for t in TREES])
def test_host_mask_equals_oracle(lib, name, pr, kpd):
    parent, rank = pr
    mask, depth = _build_host(parent, rank, kpd)
    vis = otree.visible_bruteforce(parent)
    np.testing.assert_array_equal(mask, otree.bitmask_rows(vis))
    np.testing.assert_array_equal(depth, otree.depth_of(parent))


BAD = [
    ("root parent", [0, 0], [0, 0], [3, 2]),
    ("parent after child", [-1, 2, 0], [0, 0, 1], [3, 2]),
    ("duplicate rank", [-1, 0, 0], [0, 1, 1], [3, 2]),
    ("rank too large", [-1, 0, 1], [0, 0, 2], [3, 2]),
    ("too deep", [-1, 0, 1, 2], [0, 0, 0, 0], [3, 2]),
    ("negative k", [-1, 0], [0, 0], [0, 2]),
]


@pytest.mark.parametrize("what,parent,rank,kpd", BAD, ids=[b[0] for b in BAD])
def test_host_rejects_invalid_trees_like_the_oracle(lib, what, parent, rank, kpd):
    from medusa_tree_verification_amd import api
    with pytest.raises(api.MedusaError) as ei:
        api.tree_build_host(parent, rank, kpd)
    assert ei.value.code == api.EINVAL
    if what != "negative k":
        with pytest.raises(ValueError):
            otree.validate(parent, rank, kpd)


def test_tree_size_limit(lib):
    from medusa_tree_verification_amd import api
    parent = [-1] + [0] * 256
    with pytest.raises(api.MedusaError):
        api.tree_build_host(parent, list(range(257)), [32])
