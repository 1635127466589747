"""The synthetic decode workloads.

Shapes: 4 KV heads with 6 query heads each (24 query heads), head_dim 256,
page 64 tokens, 16 attention layers; the recent window stays BF16 and every
full page older than it is int8.  The tiny workload is the one the float64
oracle finishes in well under a second.
"""
from __future__ import annotations

from .inputs import Workload, draw_lengths

SIGMA = 1.0 / 16.0  # softmax scale 1/sqrt(256)


def tiny() -> Workload:
    # 1 sequence, 1 KV head, 2 query heads; 512 tokens = 4 int8 pages + 256-token window
    return Workload("tiny", 0, batch=1, layers=1, num_kv_heads=1, group=2, lengths=(512,),
                    window=256, outlier_frac=0.0, permute=False)


def ctx32k() -> Workload:
    return Workload("ctx32k", 1, batch=1, layers=16, num_kv_heads=4, group=6, lengths=(32768,),
                    window=1024, outlier_frac=0.02, permute=False)


def ctx128k() -> Workload:
    # 131,072 tokens = 2032 int8 pages + 16 BF16 window pages
    return Workload("ctx128k", 2, batch=1, layers=16, num_kv_heads=4, group=6, lengths=(131072,),
                    window=1024, outlier_frac=0.02, permute=False)


def batched() -> Workload:
    # 32 requests; 16 lengths drawn uniformly from [4096, 16384], each shared by a
    # pair of requests so pairs have equal page counts (two-owner mode)
    return Workload("batched", 3, batch=32, layers=16, num_kv_heads=4, group=6,
                    lengths=draw_lengths(3, 16, 4096, 16384), window=512, outlier_frac=0.02,
                    permute=True)


def staged128k() -> Workload:
    return Workload("staged128k", 4, batch=1, layers=16, num_kv_heads=4, group=6,
                    lengths=(131072,), window=1024, outlier_frac=0.02, permute=False)


ALL = {f.__name__: f for f in (tiny, ctx32k, ctx128k, batched, staged128k)}
