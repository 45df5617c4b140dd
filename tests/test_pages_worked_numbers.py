"""The oracle's accounting against the numbers the pages print (tests/golden)."""
import json
import math
import os

import pytest

from oracle import pkv_oracle as O

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_worked_numbers.json")))


def test_kv_bytes_of_a_7b_request_and_batch():
    g = GOLDEN["kv_bytes_7b"]
    b = O.kv_cache_bytes(g["layers"], g["heads"], g["head_dim"], g["tokens"], g["elem_bytes"])
    # the page rounds to one decimal (2.1 GB) and then multiplies the rounded figure (67 GB)
    assert round(b / 1e9, 1) == g["printed_request_gb"]
    assert math.isclose(g["batch"] * b / 1e9, g["printed_batch_gb"], rel_tol=0.03)


def test_static_padding_waste():
    g = GOLDEN["static_padding"]
    assert round(O.static_padding_waste(g["mean_len"], g["max_len"]), 2) == g["printed_waste"]


@pytest.mark.parametrize("case", GOLDEN["paged_waste"]["cases"])
def test_paged_tail_waste_is_within_one_block(case):
    n, printed_bound = case
    P = GOLDEN["paged_waste"]["block_size"]
    assert P / n == pytest.approx(printed_bound)
    waste = (O.paged_slots_reserved(n, P) - n) / n
    assert 0 <= waste <= P / n
    # and the allocator model reserves exactly that many slots
    a = O.BlockAllocatorModel(200, P)
    s = a.create()
    a.append_slots(s, n)
    assert len(a.block_table(s)) * P == O.paged_slots_reserved(n, P)


def test_preallocation_waste():
    g = GOLDEN["paged_waste"]
    assert round(O.preallocation_waste(g["prealloc_len"], g["prealloc_max"]), 2) == g["printed_prealloc_waste"]


def test_copy_on_write_saving():
    g = GOLDEN["cow_saving"]
    saved = O.cow_saving_bytes(g["n_requests"], g["shared_tokens"], g["kb_per_token"] * 1024)
    assert round(saved / 2 ** 20, 1) == g["printed_mb"]
