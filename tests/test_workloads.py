"""The seeded generators: deterministic, within the stated distributions."""
import math

import numpy as np

from workloads import WORKLOADS, make_scenario, round_to_bits, ValueStream, F16, BF16, F32


def test_tiny_matches_the_pages_example_order():
    sc = make_scenario(WORKLOADS["tiny_fp32"])
    assert list(sc.free_order[:5]) == [5, 12, 3, 9, 0]
    assert sorted(sc.free_order) == list(range(16))
    assert sc.setup == [("add", 0, 10), ("add", 1, 7)]


def test_scenarios_are_deterministic():
    for w in WORKLOADS.values():
        a = make_scenario(w, batch=min(w.batch, 16))
        b = make_scenario(w, batch=min(w.batch, 16))
        assert a.setup == b.setup and np.array_equal(a.free_order, b.free_order)
        assert a.growth == b.growth


def test_length_ranges():
    lens = make_scenario(WORKLOADS["mha7b_fp16"]).lengths_before
    assert len(lens) == 64 and min(lens.values()) >= 128 and max(lens.values()) <= 2048
    lens = make_scenario(WORKLOADS["gqa70b_bf16"]).lengths_before
    assert min(lens.values()) >= 256 and max(lens.values()) <= 4096
    sc = make_scenario(WORKLOADS["long_splitk_bf16"])
    assert min(sc.lengths_before.values()) >= 32768 and max(sc.lengths_before.values()) <= 131072
    total = sum(-(-(n + 1) // 32) for n in sc.lengths_before.values())
    assert sc.num_blocks == math.ceil(1.1 * total)


def test_prefix_share_structure():
    sc = make_scenario(WORKLOADS["prefix_share_fp16"])
    adds = [op for op in sc.setup if op[0] == "add"]
    forks = [op for op in sc.setup if op[0] == "fork"]
    assert len(adds) == 32 and len(forks) == 32 * 7
    assert all(1024 + 1 <= n <= 1024 + 15 for _, _, n in adds)
    assert all(1024 + 16 <= n <= 1024 + 512 for n in sc.lengths_before.values())


def test_rounding_to_storage_types():
    x = np.array([1.0, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11], dtype=np.float32)
    assert round_to_bits(x, F16).tolist() == [0x3C00, 0x3C00, 0x3C02]        # ties to even
    y = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -9], dtype=np.float32)
    assert round_to_bits(y, BF16).tolist() == [0x3F80, 0x3F82, 0x3F81]       # ties to even; 0.75 ulp up
    assert round_to_bits(x[:1], F32).tolist() == [0x3F800000]


def test_value_stream_is_reproducible():
    a = ValueStream(5, F16, 0.1).draw(3, 4)
    b = ValueStream(5, F16, 0.1).draw(3, 4)
    assert a.dtype == np.uint16 and np.array_equal(a, b)
