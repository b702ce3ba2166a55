"""Module structure and per-step module order of the workloads (for the
fetch/release coordinator).  Shapes only: no arithmetic of the method.

A module owns the parameters whose names share its prefix (the name
without its last dotted component, e.g. ``model.layers.3.mlp.up_proj``).
The forward pass runs modules in execution order -- for a Llama decoder
layer: input norm, q, k, v, o, post-attention norm, gate, up, down; for a
GPT-2 block: ln_1, c_attn, c_proj, ln_2, c_fc, c_proj -- and a GPT-style
model's output head is its token embedding again (tied weights), so that
module runs twice.  Backward fetches the forward's modules in reverse order.
"""

from __future__ import annotations

from typing import Dict, List, Tuple

from .configs import Config


def _module_name(param_name: str) -> str:
    if "." in param_name:
        return param_name.rsplit(".", 1)[0]
    return param_name.split("_")[0]


def module_table(cfg: Config) -> Tuple[List[str], List[List[int]]]:
    """Module names in registration order and each module's ds_ids."""
    names: List[str] = []
    params: Dict[str, List[int]] = {}
    for d, p in enumerate(cfg.params):
        m = _module_name(p.name)
        if m not in params:
            names.append(m)
            params[m] = []
        params[m].append(d)
    return names, [params[m] for m in names]


_LLAMA_ORDER = ("input_layernorm", "self_attn.q_proj", "self_attn.k_proj", "self_attn.v_proj",
                "self_attn.o_proj", "post_attention_layernorm", "mlp.gate_proj", "mlp.up_proj",
                "mlp.down_proj")


def forward_order(cfg: Config) -> List[int]:
    names, _ = module_table(cfg)
    idx = {n: i for i, n in enumerate(names)}
    if "model.embed_tokens" in idx or any(n.startswith("layer.") for n in names):
        out = []
        if "model.embed_tokens" in idx:
            out.append(idx["model.embed_tokens"])
        layers = sorted({n.rsplit(".", 2)[0] if n.startswith("model.layers.") else "layer"
                         for n in names if n.startswith("model.layers.") or n.startswith("layer.")},
                        key=lambda s: int(s.split(".")[2]) if s.startswith("model.layers.") else 0)
        for lay in layers:
            for part in _LLAMA_ORDER:
                key = (lay + "." + part) if lay != "layer" else ("layer." + part)
                if key in idx:
                    out.append(idx[key])
        for tail in ("model.norm", "lm_head"):
            if tail in idx:
                out.append(idx[tail])
        assert sorted(out) == list(range(len(names))), "every module runs once"
        return out
    if "wte" in idx:        # GPT-style: embeddings, blocks, final norm, tied head
        return list(range(len(names))) + [idx["wte"]]
    return list(range(len(names)))


def step_order(cfg: Config) -> List[int]:
    """The modules fetched in one training step: forward, then backward."""
    f = forward_order(cfg)
    return f + f[::-1]
