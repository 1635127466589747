"""The seeded input generator: BF16 rounding agrees with torch's
round-to-nearest-even conversion (ties included), draws are reproducible,
and the tier split follows the page-boundary reading."""
import numpy as np
import torch

from quantized_paged_kv_akv_amd import configs, inputs


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(7)
    x = r.standard_normal(200_000).astype(np.float32) * np.float32(1e3)
    # exact ties: low half 0x8000 under even and odd kept bits, and near-ties
    hi = r.integers(0x0080, 0x7F00, 4000).astype(np.uint32) << np.uint32(16)
    ties = np.concatenate([hi | np.uint32(0x8000), hi | np.uint32(0x7FFF), hi | np.uint32(0x8001),
                           (hi | np.uint32(0x18000)), hi]).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.array([0.0, -0.0, 1.0, 65504.0, 3.0e38], np.float32)])
    ours = inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_draws_are_reproducible_and_split_on_page_boundaries():
    w = configs.tiny()
    a, b = inputs.make_layer_np(w, 0), inputs.make_layer_np(w, 0)
    assert np.array_equal(a["k_pool"], b["k_pool"]) and np.array_equal(a["q"], b["q"])
    c = inputs.make_layer_np(w, 1)
    assert not np.array_equal(a["k_pool"], c["k_pool"])
    plan = a["plan"]
    # 512 tokens, 256-token window: 4 full int8 pages, the window starts on a page boundary
    assert plan.n8 == [4] and plan.win_tokens == [256]
    w2 = configs.ctx128k()
    n8, win = w2.split(0)
    assert n8 == 2032 and win == 1024 and n8 * 64 + win == 131072
