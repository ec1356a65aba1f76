"""Plant plausible mistakes in the block manager oracle and check the pins see them.

Each mutant is ``oracle/block_manager.py`` with one edit: copy-on-write
skipped or miscounted, references not counted, shared blocks freed, the free
stack used as a queue, table lists aliased, a batch that is not all or
nothing, a reversed or unchecked block copy.  It is loaded as a fresh module
and run through the pool pins of ``test_block_pool.py``: the page's
copy-on-write example step by step and with data, invariants after random
operations, the all-or-nothing batch and the block copy.  Every mutant must
fail at least one of them.
"""
import os
import types

import pytest

import oracle.block_manager as bm
import test_block_pool as pins

SRC = bm.__file__

MUTANTS = {
    "cow_write_in_place": ("elif self.refcount[table[j]] > 1:", "elif False:"),
    "cow_shared_count_kept": ("                self.refcount[shared] -= 1\n", ""),
    "fork_no_refcount": ("            self.refcount[b] += 1\n", "            pass\n"),
    "release_frees_shared": ("            if self.refcount[b] == 0:\n                self.free.append(b)",
                             "            self.free.append(b)"),
    "free_queue_not_stack": ("b = self.free.pop()", "b = self.free.pop(0)"),
    "needed_ignores_copy": ("cow = 1 if room > 0 and self.refcount[table[-1]] > 1 else 0", "cow = 0"),
    "room_off_by_one": ("room = len(table) * self.B - L", "room = len(table) * self.B - L + 1"),
    "fork_aliases_table": ("self.tables[child] = list(self.tables[parent])",
                           "self.tables[child] = self.tables[parent]"),
    "batch_not_atomic": ("trial = copy.deepcopy(self)", "trial = self"),
    "copy_reversed": ("kc[d] = src_k[s]", "kc[s] = src_k[d]"),
    "copy_no_skip": (" if 0 <= s < NB and 0 <= d < NB and s != d]", "]"),
}


def _module(name=None):
    """The oracle's source, with mutant ``name`` applied, as a new module whose
    OutOfBlocks is the real one (so the pins recognise the error)."""
    with open(SRC) as f:
        src = f.read()
    if name is not None:
        old, new = MUTANTS[name]
        assert src.count(old) == 1, f"mutant {name}: pattern not unique"
        src = src.replace(old, new)
    mod = types.ModuleType(f"block_manager_{name or 'plain'}")
    exec(compile(src, os.path.basename(SRC), "exec"), mod.__dict__)
    mod.OutOfBlocks = bm.OutOfBlocks
    return mod


def _battery(mod):
    """Names of the pins that fail (an exception from the mutant is a fail)."""
    runs = {
        "cow_example": lambda: pins.cow_example_checks(mod.BlockManager),
        "cow_example_data": lambda: pins.cow_example_data_checks(mod.BlockManager, mod.copy_blocks),
        "random_ops": lambda: [pins.random_ops_checks(mod.BlockManager, seed) for seed in range(3)],
        "batch": lambda: pins.batch_checks(mod.BlockManager),
        "copy": lambda: pins.copy_checks(mod.copy_blocks),
    }
    failed = []
    for name, run in runs.items():
        try:
            run()
        except (Exception, pytest.fail.Exception):   # an assertion or pytest.raises
            failed.append(name)                       # miss, or the mutant breaking
    return failed


def test_unmutated_block_manager_passes_battery():
    assert _battery(_module()) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_block_manager_mutant_is_caught(name):
    assert _battery(_module(name)), f"mutant {name} passed every pin"
