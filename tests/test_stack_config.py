"""The stack workload's layer list is the oracle's cyclic schedule (CPU only)."""

import oracle
from inputs import STACK_CONFIGS


def test_stack_layers_follow_the_cyclic_schedule():
    cfg = STACK_CONFIGS["sst_cycle_sr"]
    assert list(cfg.layers) == oracle.cyclic_schedule(len(cfg.layers), (16, 32, 64))
    for M, _ in cfg.layers:
        assert cfg.Hg % M == 0 and cfg.Wg % M == 0
