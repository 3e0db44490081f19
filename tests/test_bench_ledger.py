"""The benchmark's algorithmic byte ledger against the pages' per-token accounting
(TileLang tutorial ch. 38, section 1.2: k x d x b bytes per token and direction) and the
combine's extra weight bytes.  CPU only."""

import bench


def test_dispatch_payload_bytes_match_the_pages_per_token_figures(golden):
    g = golden["byte_ledger"]
    k, H = g["k"], g["hidden"]
    for fp8, key in ((False, "bf16_dispatch_bytes_per_token"), (True, "fp8_dispatch_bytes_per_token")):
        led = bench.ledger(T=1, K=k, H=H, rows=k, pad=0, fp8=fp8, zero_padding=True)
        sf = 4 * (H // 128) if fp8 else 0
        payload = led["dispatch_write"] - k * 12 - k * sf  # minus row metadata and fp8 scales
        assert payload == g[key]


def test_combine_bytes_include_the_weights(golden):
    g = golden["byte_ledger"]
    k, H = g["k"], g["hidden"]
    led = bench.ledger(T=1, K=k, H=H, rows=k, pad=0, fp8=False, zero_padding=True)
    # read k expert rows plus, per slot, its weight (4 B) and its row index (4 B)
    assert led["combine_read"] == g["bf16_dispatch_bytes_per_token"] + 8 * k
    # the page's 86040 counts the k rows plus 4 B of weight per slot
    assert led["combine_read"] - 4 * k == g["bf16_combine_bytes_per_token_with_weights"]


def test_padding_rows_cost_only_with_zero_padding():
    a = bench.ledger(T=10, K=2, H=512, rows=20, pad=12, fp8=False, zero_padding=True)
    b = bench.ledger(T=10, K=2, H=512, rows=20, pad=12, fp8=False, zero_padding=False)
    assert a["dispatch_write"] - b["dispatch_write"] == 12 * 512 * 2
    assert a["combine"] == b["combine"]
