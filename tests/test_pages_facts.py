"""The launch facts and the throughput formula the pages print.

The pages give no output values for any GEMM input, so the oracle cannot be
pinned to a worked example; these fixtures pin the host-side arithmetic the
pages do print: the ceil-div tile grid, the K-loop trip count, the shared
memory ring size and the TFLOPS formula.
"""
import json
import os

import pytest

import workloads

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))


def _cdiv(a, b):
    return -(-a // b)


def test_hopper_lowering_launch_shape():
    f = FACTS["hopper_lowering"]
    t = f["tile_inferred"]
    assert _cdiv(f["N"], t["block_N"]) == f["grid_x"]
    assert _cdiv(f["M"], t["block_M"]) == f["grid_y"]
    assert _cdiv(f["K"], t["block_K"]) == f["k_iterations"]
    assert t["block_M"] * t["block_K"] == f["a_slot_elems"]
    assert t["block_K"] * t["block_N"] == f["b_slot_elems"]
    ring = f["stages"] * (f["a_slot_elems"] + f["b_slot_elems"]) * f["elem_bytes"]
    assert ring == f["dyn_smem_bytes"]


def test_sm100_example_grid_and_tflops_formula():
    f = FACTS["sm100_example"]
    assert (_cdiv(f["N"], f["block_N"]), _cdiv(f["M"], f["block_M"])) == (16, 32)
    latency_ms = 0.25
    want = 2 * f["M"] * f["N"] * f["K"] / (latency_ms / 1e3) / 1e12
    assert workloads.tflops(f["M"], f["N"], f["K"], latency_ms / 1e3) == pytest.approx(want, rel=1e-15)
    assert want == pytest.approx(1099.511627776, rel=1e-12)
