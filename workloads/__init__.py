"""Seeded synthetic inputs for paged decode attention.

This package draws random numbers and lays them out; it computes nothing the
attention method itself computes.  Both the test oracle and the GPU library
consume what it produces, and neither side's arithmetic lives here.
"""
from .synth import (  # noqa: F401
    DecodeBatch,
    CONFIGS,
    make_config,
    make_decode_batch,
    relayout,
)
from .groups import (  # noqa: F401
    GROUP_CONFIGS,
    GroupedBatch,
    TreeBatch,
    make_group_config,
    make_tree_batch,
    make_tree_config,
    make_grouped_batch,
    random_group_tables,
    tables_from_blocks,
    token_blocks,
)
