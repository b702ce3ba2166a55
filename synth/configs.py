"""Workload shapes of the shard-step configurations.

Each configuration is a list of named parameter shapes in module
registration order (ds_id = position in that order), a 16-bit dtype, the
number of data-parallel ranks N, the persistence threshold, bucket and
sub-group sizes, Adam hyperparameters and the gradient distribution.

* ``c0``  the 4-unit, 4-GPU worked example of the csdn page (its "worked
          example" section), as four scalar parameters.
* ``c0b`` the same example as one 4-element parameter.
* ``c1``  toy 2-layer model, N = 4, fp16, 2,608 elements.
* ``c2``  GPT-2-small-shaped parameter set (124,439,808), bf16, N = 8.
* ``c3``  one Llama-3-8B decoder layer (218,112,000), bf16, N = 8.
* ``c4``  the full Llama-3-8B-shaped set (8,030,261,248), bf16, N = 8:
          one GPU's 1/8 share is the measured workload.
* ``c5``  ragged 7.5B GPT-style set (7,461,217,053), fp16, N = 64: width
          4095 so that no 2-D tensor's size divides by 64 (padding forced).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Tuple


@dataclass(frozen=True)
class ParamSpec:
    name: str
    shape: Tuple[int, ...]

    @property
    def numel(self) -> int:
        n = 1
        for s in self.shape:
            n *= s
        return n


@dataclass(frozen=True)
class Config:
    name: str
    title: str
    dtype: str                      # "fp16" | "bf16"
    world_size: int
    threshold: int                  # param_persistence_threshold (elements)
    params: Tuple[ParamSpec, ...]
    prefetch_bucket_size: int       # gather bucket limit (full elements)
    reduce_bucket_size: int         # gradient bucket limit (full elements)
    sub_group_size: int             # per-rank shard elements per sub-group
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    max_norm: float = 1.0
    steps: int = 10
    weight_std: float = 0.02
    grad_std: float = 1e-3
    outlier_prob: float = 0.0       # per element, per virtual rank
    outlier_mult: float = 100.0
    seed: int = 0
    config_id: int = 0
    parity_ranks: Tuple[int, ...] = (0,)
    bench_rank: int = 0

    @property
    def ds_ids(self) -> List[int]:
        return list(range(len(self.params)))

    @property
    def numels(self) -> List[int]:
        return [p.numel for p in self.params]

    @property
    def total_params(self) -> int:
        return sum(self.numels)


def _gpt2_small() -> Tuple[ParamSpec, ...]:
    d, v, ctx, L = 768, 50257, 1024, 12
    ps = [ParamSpec("wte", (v, d)), ParamSpec("wpe", (ctx, d))]
    for i in range(L):
        h = f"h.{i}."
        ps += [
            ParamSpec(h + "ln_1.weight", (d,)), ParamSpec(h + "ln_1.bias", (d,)),
            ParamSpec(h + "attn.c_attn.weight", (d, 3 * d)), ParamSpec(h + "attn.c_attn.bias", (3 * d,)),
            ParamSpec(h + "attn.c_proj.weight", (d, d)), ParamSpec(h + "attn.c_proj.bias", (d,)),
            ParamSpec(h + "ln_2.weight", (d,)), ParamSpec(h + "ln_2.bias", (d,)),
            ParamSpec(h + "mlp.c_fc.weight", (d, 4 * d)), ParamSpec(h + "mlp.c_fc.bias", (4 * d,)),
            ParamSpec(h + "mlp.c_proj.weight", (4 * d, d)), ParamSpec(h + "mlp.c_proj.bias", (d,)),
        ]
    ps += [ParamSpec("ln_f.weight", (d,)), ParamSpec("ln_f.bias", (d,))]
    return tuple(ps)


def _llama_layer(prefix: str, d=4096, kv=1024, ffn=14336) -> List[ParamSpec]:
    return [
        ParamSpec(prefix + "self_attn.q_proj.weight", (d, d)),
        ParamSpec(prefix + "self_attn.k_proj.weight", (kv, d)),
        ParamSpec(prefix + "self_attn.v_proj.weight", (kv, d)),
        ParamSpec(prefix + "self_attn.o_proj.weight", (d, d)),
        ParamSpec(prefix + "mlp.gate_proj.weight", (ffn, d)),
        ParamSpec(prefix + "mlp.up_proj.weight", (ffn, d)),
        ParamSpec(prefix + "mlp.down_proj.weight", (d, ffn)),
        ParamSpec(prefix + "input_layernorm.weight", (d,)),
        ParamSpec(prefix + "post_attention_layernorm.weight", (d,)),
    ]


def _llama3_8b() -> Tuple[ParamSpec, ...]:
    vocab, d = 128256, 4096
    ps = [ParamSpec("model.embed_tokens.weight", (vocab, d))]
    for i in range(32):
        ps += _llama_layer(f"model.layers.{i}.")
    ps += [ParamSpec("model.norm.weight", (d,)), ParamSpec("lm_head.weight", (vocab, d))]
    return tuple(ps)


def _ragged_7p5b() -> Tuple[ParamSpec, ...]:
    d, ffn, v, ctx, L = 4095, 16383, 50257, 2048, 36
    ps = [ParamSpec("wte", (v, d)), ParamSpec("wpe", (ctx, d))]
    for i in range(L):
        h = f"h.{i}."
        ps += [
            ParamSpec(h + "ln_1.weight", (d,)), ParamSpec(h + "ln_1.bias", (d,)),
            ParamSpec(h + "attn.c_attn.weight", (d, 3 * d)), ParamSpec(h + "attn.c_attn.bias", (3 * d,)),
            ParamSpec(h + "attn.c_proj.weight", (d, d)), ParamSpec(h + "attn.c_proj.bias", (d,)),
            ParamSpec(h + "ln_2.weight", (d,)), ParamSpec(h + "ln_2.bias", (d,)),
            ParamSpec(h + "mlp.c_fc.weight", (d, ffn)), ParamSpec(h + "mlp.c_fc.bias", (ffn,)),
            ParamSpec(h + "mlp.c_proj.weight", (ffn, d)), ParamSpec(h + "mlp.c_proj.bias", (d,)),
        ]
    ps += [ParamSpec("ln_f.weight", (d,)), ParamSpec("ln_f.bias", (d,))]
    return tuple(ps)


CONFIGS: Dict[str, Config] = {
    "c0": Config(
        name="c0", title="worked example: 4 scalar params, N=4", dtype="fp16",
        world_size=4, threshold=0,
        params=tuple(ParamSpec(n, (1,)) for n in ("l1_w1", "l1_w2", "l2_w1", "l2_w2")),
        prefetch_bucket_size=int(5e7), reduce_bucket_size=int(5e6), sub_group_size=int(1e9),
        steps=1, config_id=0, parity_ranks=(0, 1, 2, 3)),
    "c0b": Config(
        name="c0b", title="worked example: one 4-element param, N=4", dtype="fp16",
        world_size=4, threshold=0, params=(ParamSpec("w", (4,)),),
        prefetch_bucket_size=int(5e7), reduce_bucket_size=int(5e6), sub_group_size=int(1e9),
        steps=1, config_id=10, parity_ranks=(0, 1, 2, 3)),
    "c1": Config(
        name="c1", title="toy 2-layer model, N=4, fp16", dtype="fp16", world_size=4, threshold=0,
        params=(ParamSpec("l1.weight", (64, 32)), ParamSpec("l1.bias", (32,)),
                ParamSpec("l2.weight", (32, 16)), ParamSpec("l2.bias", (16,))),
        prefetch_bucket_size=int(5e7), reduce_bucket_size=int(5e6), sub_group_size=int(1e9),
        steps=3, config_id=1, parity_ranks=(0, 1, 2, 3)),
    "c2": Config(
        name="c2", title="GPT-2-small-shaped set, N=8, bf16", dtype="bf16", world_size=8,
        threshold=int(1e5), params=_gpt2_small(),
        prefetch_bucket_size=int(5e7), reduce_bucket_size=int(5e6), sub_group_size=int(1e9),
        config_id=2, parity_ranks=(0, 7)),
    "c3": Config(
        name="c3", title="one Llama-3-8B decoder layer, N=8, bf16", dtype="bf16", world_size=8,
        threshold=int(1e5), params=tuple(_llama_layer("layer.")),
        prefetch_bucket_size=int(5e7), reduce_bucket_size=int(5e6), sub_group_size=int(1e9),
        outlier_prob=0.01, config_id=3, parity_ranks=(0, 7)),
    "c4": Config(
        name="c4", title="Llama-3-8B-shaped set, N=8, bf16, one rank's share", dtype="bf16",
        world_size=8, threshold=int(1e5), params=_llama3_8b(),
        prefetch_bucket_size=int(5e7), reduce_bucket_size=int(5e6), sub_group_size=int(1e9),
        outlier_prob=0.01, config_id=4, parity_ranks=(0, 7)),
    "c5": Config(
        name="c5", title="ragged 7.5B GPT-style set (width 4095), N=64, fp16", dtype="fp16",
        world_size=64, threshold=int(1e5), params=_ragged_7p5b(),
        prefetch_bucket_size=int(5e7), reduce_bucket_size=int(5e7), sub_group_size=int(1e9),
        config_id=5, parity_ranks=(0, 63), bench_rank=63),
}


def get_config(name: str) -> Config:
    return CONFIGS[name]
