"""CPU oracle of the load-balanced MoE token path.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg; never by the product path.
"""
from .path import (SOFTMAX, SIGMOID, UNSPECIFIED, route_topk, load_matrix,  # noqa: F401
                   imbalance, capacity, plan_balance, plan_quota, replicas_per_rank,
                   align_sort, dispatch,
                   dispatch_rows, combine, bf16_to_f64, prefetch_slots,
                   prefetch_weights, f32_to_bf16_rne, combine_bwd, dispatch_bwd, reduce_grad)
