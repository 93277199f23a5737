"""The selection budget the pages fix (tests/golden/page_constants.json) is what every workload uses."""
import json
import os

from kv_reuse_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


def test_page_constants_used_by_every_workload():
    with open(GOLDEN, encoding="utf-8") as f:
        c = json.load(f)
    for w in wl.WORKLOADS.values():
        assert w.top_k == c["top_k"] and w.window == c["window"]
