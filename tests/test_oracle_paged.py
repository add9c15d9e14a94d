"""Pin of the paged-ContextKV oracle: with the context scattered over pages
in a random order (spare pages and the rows past the context NaN), it must
reproduce the dense oracle bitwise, whatever the page size.  Copies of the
page gather with planted mistakes must fail that comparison."""
import inspect
import textwrap

import numpy as np
import pytest

from oracle import oracle as O
from shared_prefix_beam_amd import inputs as I


def _case(seed):
    return I.custom(B=3, Hq=8, Hkv=4, D=64, W=[5, 2, 7], ctx_len=[77, 16, 130],
                    beam_len=[2, 1, 3], seed=seed)


def _paged_vs_dense(gather, page_size, seed):
    inp = _case(seed)
    pg = I.to_paged(inp, page_size, seed=seed + 1)
    k, v = gather(pg.k_pages, pg.v_pages, pg.page_table, page_size, inp.ctx_len, inp.ctx_cap)
    a = O.decode_attn_inputs(inp)
    b = O.decode_attn(inp.q, k, v, inp.ctx_len, inp.beam_k, inp.beam_v, inp.beam_path,
                      inp.beam_len, inp.row_offset, scale=inp.scale)
    return np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("page_size", [16, 32, 64, 256])
def test_paged_oracle_equals_dense(page_size):
    assert _paged_vs_dense(O.gather_pages, page_size, seed=page_size)


def test_paged_entry_point_matches_gather():
    inp = _case(9)
    pg = I.to_paged(inp, 32, seed=10)
    a = O.decode_attn_inputs(inp)
    b = O.decode_attn_paged(inp.q, pg.k_pages, pg.v_pages, pg.page_table, 32, inp.ctx_len,
                            inp.beam_k, inp.beam_v, inp.beam_path, inp.beam_len,
                            inp.row_offset, ctx_cap=inp.ctx_cap, scale=inp.scale)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


MUTANTS = [
    ("page and offset swapped", "k[b, j] = k_pages[page, j % page_size]",
     "k[b, j] = k_pages[page, (j // page_size) % page_size]"),
    ("table row of request 0", "page = int(page_table[b, j // page_size])",
     "page = int(page_table[0, j // page_size])"),
    ("logical page off by one", "page = int(page_table[b, j // page_size])",
     "page = int(page_table[b, (j + 1) // page_size])"),
    ("V from the K pool", "v[b, j] = v_pages[page, j % page_size]",
     "v[b, j] = k_pages[page, j % page_size]"),
]


@pytest.mark.parametrize("name,orig,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_gather_mutant_is_rejected(name, orig, bad):
    src = textwrap.dedent(inspect.getsource(O.gather_pages))
    assert orig in src
    ns = {"np": np}
    exec(src.replace(orig, bad, 1), ns)
    broken = ns["gather_pages"]
    rejected = False
    for page_size in (16, 32):
        try:
            ok = _paged_vs_dense(broken, page_size, seed=page_size + 3)
        except (IndexError, ValueError):
            ok = False
        rejected |= not ok
    assert rejected, f"no comparison rejects '{name}'"
