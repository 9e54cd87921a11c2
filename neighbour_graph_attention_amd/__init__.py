"""Neighbour-graph attention hot path on MI355X (gfx950).

Python face of libnga.so, the C-ABI library declared in include/nga.h:

* ``nl_build``: O(N) cell-list neighbour rows under periodic boundaries;
* ``edge_csr``: those rows as a destination CSR with image shifts;
* ``block_attn_forward``: block-dense multi-head attention through the CSR;
* ``local_attn_forward``: LocalAtten, one query per centre over its edges;
* ``pair_attn_forward``: the same attention by the ragged pair-axis route, a
  measured comparator;
* ``block_gather`` / ``block_scatter``: the padded per-centre block on its own;
* ``nl_build_static``: ``nl_build`` without a workspace, for callers that
  cannot allocate.

Importing the package loads the library and fails loudly if it has not been
built (``neighbour_graph_attention_amd._build.build()``).
"""
from ._lib import (  # noqa: F401
    EXPORTS,
    NGA_F32,
    NGA_F32_SPLIT16,
    NGA_F64,
    ROW_CAP,
    NGAError,
    StepGraph,
    Workspace,
    attn_plan,
    attn_variant,
    block_attn_forward,
    block_attn_workspace_bytes,
    block_gather,
    block_scatter,
    check_status,
    edge_csr,
    load,
    nl_build,
    local_attn_forward,
    nl_build_batch,
    nl_build_static,
    nl_build_workspace_bytes,
    nl_max_displacement,
    nl_refine,
    pair_attn_forward,
    pair_attn_workspace_bytes,
    strerror,
    sync_status,
)

load()
