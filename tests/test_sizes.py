"""Shape pins against the size statements of the pages (tests/golden/page_sizes.txt)."""
import os

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _facts():
    d = {}
    for line in open(os.path.join(GOLD, "page_sizes.txt")):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":")
        d[k.strip()] = float(v)
    return d


def blob_bytes(H, I, group):
    nib = 3 * H * I // 2
    if group == 0:
        sc = (2 * I + H) * 4
    else:
        sc = (2 * I * (H // group) + H * (I // group)) * 4
    return nib + sc


def test_expert_size_pins_intermediate():
    f = _facts()
    H = int(f["hidden"])
    b = blob_bytes(H, 2048, 0)
    assert b == 18_915_328
    # "about 19 MB" per expert: within 1 MB, and the neighbouring power-of-two
    # intermediate sizes are far off
    assert abs(b / 1e6 - f["expert_mb_approx"]) < 1.0
    assert abs(blob_bytes(H, 1024, 0) / 1e6 - f["expert_mb_approx"]) > 5
    assert abs(blob_bytes(H, 4096, 0) / 1e6 - f["expert_mb_approx"]) > 5


def test_routed_bytes_per_token():
    f = _facts()
    per_token = f["moe_layers"] * f["top_k"] * blob_bytes(int(f["hidden"]), 2048, 0)
    assert abs(per_token / 1e9 - f["routed_gb_per_token_approx"]) < 1.0


def test_gs64_blob():
    assert blob_bytes(6144, 2048, 64) == 21_233_664
