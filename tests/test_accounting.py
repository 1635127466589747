"""Byte accounting of the measured workloads (CPU only).

The benchmark's KV bytes per step decide its headline rate, so they are
pinned here against the page formats and the workload shapes, each figure
derived from first principles rather than re-typed from bench.py:

* one (page, KV head) of the 8-bit format: 64 x 256 key codes, 256 x 64 value
  codes, 64 FP32 token factors, 256 FP32 channel factors, 256 FP32 value
  scales ("Model quantization" page, "An 8-bit page format shaped for its
  kernel");
* one BF16 (page, KV head): 64 tokens x 256 channels x (K, V) x 2 bytes;
* the history per token of the modelled stack (16 layers x 4 KV heads x 256
  channels x K and V in BF16) is 64 KiB, so 128,000 tokens are 8,388,608,000
  bytes: the about 8.4 GB per generated token that exact decode moves over
  PCIe at 128K in the "Model quantization" page's headline figures.
"""
import bench
from quantized_paged_kv_akv_amd import configs, inputs


def test_page_formats():
    codes = 64 * 256 + 256 * 64          # int8 K and V codes
    scales = (64 + 256 + 256) * 4        # k_tok, k_chan, v_chan as FP32
    assert bench.PAGE_INT8_BYTES == codes + scales == 35_072
    assert bench.PAGE_BF16_BYTES == 64 * 256 * 2 * 2 == 65_536
    # the 8-bit page is a little over half the BF16 page (codes are half, scales add ~7%)
    assert abs(bench.PAGE_INT8_BYTES / bench.PAGE_BF16_BYTES - 0.535) < 1e-3


def test_history_bytes_per_token_match_the_quoted_figure():
    w = configs.ALL["ctx128k"]()
    per_token = w.layers * w.num_kv_heads * 256 * 2 * 2
    assert per_token == 65_536
    assert 128_000 * per_token == 8_388_608_000


def test_ctx128k_step_bytes():
    w = configs.ALL["ctx128k"]()
    plan = inputs.plan_pools(w)
    assert plan.n8 == [2032] and plan.win_tokens == [1024]   # 131,072 tokens = 2032 + 16 full pages
    b = bench.step_kv_bytes(plan, w.num_kv_heads)
    assert b["int8"] == 2032 * 4 * 35_072
    assert b["window"] == 16 * 4 * 65_536
    assert b["int8"] + b["window"] == 289_259_520                 # one layer of the hybrid step
    assert w.layers * (b["int8"] + b["window"]) == 4_628_152_320  # the 16-layer step
    assert b["bf16_all"] == 2048 * 4 * 65_536 == 536_870_912
    assert w.layers * b["bf16_all"] == 8_589_934_592
    # bytes the hybrid tier does not move per token when staged from the host
    assert w.layers * (b["bf16_all"] - b["int8"] - b["window"]) == 3_961_782_272


def test_ctx32k_step_bytes():
    w = configs.ALL["ctx32k"]()
    plan = inputs.plan_pools(w)
    assert plan.n8 == [496] and plan.win_tokens == [1024]
    b = bench.step_kv_bytes(plan, w.num_kv_heads)
    assert w.layers * (b["int8"] + b["window"]) == 1_180_434_432


def test_tile_order_transpose_matches_the_header_formula():
    """The benchmark's transpose of tile-ordered key codes back to token-major
    order equals indexing by the byte offsets include/akv.h states."""
    import numpy as np

    t = np.arange(64)[:, None]
    d = np.arange(256)[None, :]
    off = ((4 * (d // 64) + (t // 4) % 4) * 64 + 16 * ((d // 16) % 4) + 4 * (t // 16) + t % 4) * 16 + d % 16
    assert sorted(off.reshape(-1).tolist()) == list(range(16384))
    tiled = np.random.default_rng(0).integers(-127, 128, size=(3, 2, 16384)).astype(np.int8)
    ref = tiled[..., off.reshape(-1)].reshape(3, 2, 64, 256)
    got = bench.tile_order_to_token_major(tiled.reshape(3, 2, 4, 4, 4, 4, 4, 16)).reshape(3, 2, 64, 256)
    assert np.array_equal(got, ref)
