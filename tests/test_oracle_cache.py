"""Pins of the paged-cache append oracle (CPU). The oracle's loop is checked
against the pools that the input generator builds with its own vectorised
scatter, against itself split in two batches, and by what must not change;
planted mistakes in copies of the oracle must each fail a pin."""
import importlib
import types

import numpy as np
import pytest

import fa_inputs as fi

oracle_cache = importlib.import_module("oracle.cache")


def _cases():
    # (lengths, split points): a sequence of 0, 1, 15, 16, 17 and 100 tokens
    return [([0, 1, 15, 16, 17, 100], [0, 1, 7, 16, 1, 55]),
            ([33, 2, 64], [32, 0, 63])]


def _empty_like_pool(x, fill):
    return np.full_like(x.k_pool, fill)


def pin_append_all_builds_generator_pool(mod):
    """Appending every token to empty sequences reproduces the generator's
    pool (its tail slots hold the fill value)."""
    for lens, _ in _cases():
        x = fi.paged(lens, 4, 2, 8, "f32", seed=3, permute=True)
        lens = np.asarray(lens)
        pool = mod.append(_empty_like_pool(x, 0.0), x.k_seq, x.cu_k, x.page_table,
                          np.zeros(len(lens), np.int32))
        if not np.array_equal(pool, x.k_pool):
            return False
    return True


def pin_two_batches_equal_one(mod):
    """Appending the first part of every sequence, then the rest after the
    new lengths, equals appending everything at once."""
    for lens, split in _cases():
        x = fi.paged(lens, 4, 2, 8, "f32", seed=4, permute=True)
        lens, split = np.asarray(lens), np.asarray(split)
        first = np.concatenate([x.k_seq[x.cu_k[s]:x.cu_k[s] + split[s]] for s in range(len(lens))])
        rest = np.concatenate([x.k_seq[x.cu_k[s] + split[s]:x.cu_k[s + 1]] for s in range(len(lens))])
        cu1 = np.concatenate([[0], np.cumsum(split)]).astype(np.int32)
        cu2 = np.concatenate([[0], np.cumsum(lens - split)]).astype(np.int32)
        pool = mod.append(_empty_like_pool(x, 0.0), first, cu1, x.page_table, np.zeros(len(lens), np.int32))
        pool = mod.append(pool, rest, cu2, x.page_table, split.astype(np.int32))
        if not np.array_equal(pool, x.k_pool):
            return False
    return True


def pin_only_new_slots_change(mod):
    """Exactly the T_new addressed slots change; every other slot keeps its
    value (a NaN-filled pool keeps its NaNs elsewhere)."""
    lens, split = _cases()[0]
    x = fi.paged(lens, 4, 2, 8, "f32", seed=5, permute=True)
    before = np.full_like(x.k_pool, np.nan)
    new = np.arange(sum(lens) * 16, dtype=np.float32).reshape(sum(lens), 2, 8) + 1.0
    after = mod.append(before, new, x.cu_k, x.page_table, np.zeros(len(lens), np.int32))
    changed = ~np.isnan(after[..., 0, 0])
    return int(changed.sum()) == sum(lens) and np.all(np.isnan(after[~changed]))


def pin_gather_inverts_append(mod):
    """Reading each sequence back through its page table gives its rows in
    order."""
    lens, _ = _cases()[1]
    x = fi.paged(lens, 4, 2, 8, "f32", seed=6, permute=True)
    for s in range(len(lens)):
        got = mod.gather(x.k_pool, x.page_table, lens[s], s)
        if not np.array_equal(got, x.k_seq[x.cu_k[s]:x.cu_k[s + 1]]):
            return False
    return True


PINS = [pin_append_all_builds_generator_pool, pin_two_batches_equal_one, pin_only_new_slots_change,
        pin_gather_inverts_append]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_cache_oracle_pins(pin):
    assert pin(oracle_cache)


def _mutant(old, new):
    src = open(oracle_cache.__file__).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("cache_mutant")
    exec(compile(src.replace(old, new), "cache_mutant", "exec"), mod.__dict__)
    return mod


MUTATIONS = {
    "position ignores the existing length": ("pos = base + (i - int(cu_new[s]))", "pos = i - int(cu_new[s])"),
    "position off by one": ("pos = base + (i - int(cu_new[s]))", "pos = base + (i - int(cu_new[s])) + 1"),
    "wrong page size": ("page_table[s][pos // PAGE_SIZE])\n            out", "page_table[s][pos // 8])\n            out"),
    "slot taken from the batch index": ("out[page, pos % PAGE_SIZE] = new_rows[i]", "out[page, i % PAGE_SIZE] = new_rows[i]"),
    "rows of the wrong sequence": ("out[page, pos % PAGE_SIZE] = new_rows[i]", "out[page, pos % PAGE_SIZE] = new_rows[i - int(cu_new[s])]"),
    "pool not copied": ("out = np.array(pool, copy=True)", "out = np.zeros_like(pool)"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_cache_mistake_is_caught(name):
    mut = _mutant(*MUTATIONS[name])
    failed = []
    for pin in PINS:
        try:
            ok = pin(mut)
        except Exception:
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"no pin caught: {name}"
