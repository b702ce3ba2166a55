"""Plain CPU oracle for the ZeRO-3 shard step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It
shares no code with the HIP library (no kernels, headers, helpers or tables);
it is a slow, obviously correct restatement of what the pages define, kept
in fp32/fp64 numpy so that a reader can check it against the pages by eye.

Pages cited (short tags used in every docstring here):

* [codex]  "03 · ZeRO-3: parameter sharding and the all-gather schedule",
           a chapter of the DeepSpeed reference on ai-reference-codex.pages.dev.
           Sections 1-8 (3.1 zero.Init; 5.2 fetch / all_gather_coalesced;
           5.3 release / persistence threshold; 6.1 optimizer initialisation;
           6.2 gradient reduce paths; 6.3 the per-sub-group step).
* [csdn]   "DeepSpeed ZeRO Stage 3: parameter partitioning ..." on
           adg.csdn.net.  Sections "core algorithm" steps 1-4 and the
           "worked example" (4 GPUs, a 2-layer model of 4 units).
* [llmnex] "ZeRO-3 core flow: the setting that also shards the parameters"
           on llmnex.top.  Sections 1 (what is sharded, the 120 GB table),
           2 (per-layer flow), 3 (communication), 4 (neighbours, pitfalls).

Modules:

* ``zero3``  -- the oracle proper: layout, partition, gather pack/unpack,
  reduce-scatter (contiguous path, and the non-contiguous path's send-side
  pack and owner-side reduce), shard-aware grad norm, fused Adam + cast.
* ``brute``  -- pure-Python per-element loops for tiny inputs, used only to
  pin ``zero3`` (a second, differently structured derivation).
* ``coordinator`` -- the trace-driven fetch/release coordinator as a
  step-by-step simulation (imported as ``oracle.coordinator``).

Parity status of each function is stated in its docstring; every function
has an independent pin.  (The decoupled weight-decay branch of
``adam_step``, which the pages never mention and every workload leaves at
weight_decay = 0, is pinned against torch.optim.AdamW, a zero-gradient
closed form and the per-element brute force.)
"""

from .zero3 import (  # noqa: F401
    FP16,
    BF16,
    AdamHParams,
    Layout,
    ParamSlot,
    adam_scalars,
    adam_step,
    bucket_sizes,
    dense_reference_step,
    from_f32,
    gather_buckets,
    grad_norm_finalize,
    grad_norm_partial,
    init_state,
    make_layout,
    pack,
    padding_mask,
    partition,
    reduce_buckets,
    reduce_scatter,
    scatter_pack,
    scatter_reduce,
    sub_groups,
    to_f32,
    unpack,
    wire,
)
