"""Workload definitions: unit parameter shapes, rank counts, layouts and AdamW
hyper-parameters for the synthetic FSDP workloads.

This module holds shapes and constants only.  It contains none of the
method's arithmetic and is shared by the oracle tests, the GPU tests and the
benchmark.

Sources (the pages describing the method):
  * "FSDP Training Step Walkthrough" (astro-wiki), "Setup": a 2-layer toy whose
    layers each hold one weight vector of length 4, sharded over 2 ranks.
  * "FSDP Transformer Block Sharding Example" (astro-wiki), "Model definition":
    a TransformerBlock with hidden 512, 8 heads, ffn 2048 -- W_Q/W_K/W_V/W_O
    [512, 512], W_up [512, 2048], W_down [2048, 512], two LayerNorm scales of
    512 -- and a 12-layer model built from it; "FSDP1 (FlatParameter)": the six
    linear weights flattened in the order W_Q, W_K, ..., W_down.
  * "FSDP2 parameter all-gather, gradient reduce-scatter and memory peak"
    (zwjcode), section 04: torch.optim.AdamW over all parameters.

Reading taken where the pages are silent: inside a block the parameter order
is W_Q, W_K, W_V, W_O, W_up, W_down, norm1, norm2 (the linears in the order
the FlatParameter example flattens them, the LayerNorm scales last).  The
AdamW hyper-parameters lr=1e-3, betas (0.9, 0.999), eps=1e-8, wd=0.01 apply
to every workload.
"""

from __future__ import annotations

PER_PARAM = "per_param"   # FSDP2: every parameter split along dim 0
FLAT = "flat"             # FSDP1: one padded 1-D FlatParameter per unit

ADAMW = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)

# Transformer block of hidden 512 / ffn 2048.
BLOCK_512 = [
    ("W_Q", (512, 512)),
    ("W_K", (512, 512)),
    ("W_V", (512, 512)),
    ("W_O", (512, 512)),
    ("W_up", (512, 2048)),
    ("W_down", (2048, 512)),
    ("norm1", (512,)),
    ("norm2", (512,)),
]

# The six linear weights of the same block: the FlatParameter example.
LINEARS_512 = [p for p in BLOCK_512 if not p[0].startswith("norm")]


def block_4096(i: int):
    """One block of hidden 4096, ffn 14336, grouped-query K/V of 1024 rows."""
    return [
        (f"b{i}.Wq", (4096, 4096)),
        (f"b{i}.Wk", (1024, 4096)),
        (f"b{i}.Wv", (1024, 4096)),
        (f"b{i}.Wo", (4096, 4096)),
        (f"b{i}.w1", (14336, 4096)),
        (f"b{i}.w2", (4096, 14336)),
        (f"b{i}.w3", (14336, 4096)),
        (f"b{i}.norm1", (4096,)),
        (f"b{i}.norm2", (4096,)),
    ]


GROUP_4096 = [p for i in range(4) for p in block_4096(i)]

# Each workload: a list of FSDP units (each a list of (name, shape)), the
# number of virtual ranks R, the layout, dtypes, grad scale and step count.
#   grad_sigma: per-rank gradients are N(0, grad_sigma) (then rounded to bf16
#   when grad_dtype is bf16).
WORKLOADS = {
    "toy_2layer_r2": dict(
        cid=0, units=[[("W1", (4,))], [("W2", (4,))]], R=2, layout=PER_PARAM,
        grad_dtype="f32", param_dtype="f32", grad_sigma=1.0, steps=3,
        master_init="normal"),
    "block512_r4": dict(
        cid=1, units=[BLOCK_512], R=4, layout=PER_PARAM,
        grad_dtype="bf16", param_dtype="bf16", grad_sigma=1e-3, steps=3,
        master_init="fan_in"),
    "block512_flat_r4": dict(
        cid=2, units=[LINEARS_512], R=4, layout=FLAT,
        grad_dtype="bf16", param_dtype="bf16", grad_sigma=1e-3, steps=3,
        master_init="fan_in"),
    "block512_r3": dict(
        cid=3, units=[BLOCK_512], R=3, layout=PER_PARAM,
        grad_dtype="bf16", param_dtype="bf16", grad_sigma=1e-3, steps=3,
        master_init="fan_in"),
    "block512_flat_r3": dict(
        cid=4, units=[BLOCK_512], R=3, layout=FLAT,
        grad_dtype="bf16", param_dtype="bf16", grad_sigma=1e-3, steps=3,
        master_init="fan_in"),
    "model12_r8": dict(
        cid=5, units=[BLOCK_512] * 12, R=8, layout=PER_PARAM,
        grad_dtype="bf16", param_dtype="bf16", grad_sigma=1e-3, steps=3,
        master_init="fan_in"),
    "model12_flat_r8": dict(
        cid=6, units=[BLOCK_512] * 12, R=8, layout=FLAT,
        grad_dtype="bf16", param_dtype="bf16", grad_sigma=1e-3, steps=3,
        master_init="fan_in"),
    # the same 12-layer model wrapped at other granularities (the FSDP unit
    # decides what one all-gather covers): the whole model as one unit, two
    # or four blocks per unit, and one unit per parameter
    "model12_whole_r8": dict(
        cid=8, units=[[(f"l{i}.{n}", s) for i in range(12) for n, s in BLOCK_512]], R=8,
        layout=PER_PARAM, grad_dtype="bf16", param_dtype="bf16", grad_sigma=1e-3, steps=3,
        master_init="fan_in"),
    "model12_pair_r8": dict(
        cid=10, units=[[(f"l{2 * i + j}.{n}", sh) for j in range(2) for n, sh in BLOCK_512]
                       for i in range(6)], R=8, layout=PER_PARAM, grad_dtype="bf16",
        param_dtype="bf16", grad_sigma=1e-3, steps=3, master_init="fan_in"),
    "model12_quad_r8": dict(
        cid=11, units=[[(f"l{4 * i + j}.{n}", sh) for j in range(4) for n, sh in BLOCK_512]
                       for i in range(3)], R=8, layout=PER_PARAM, grad_dtype="bf16",
        param_dtype="bf16", grad_sigma=1e-3, steps=3, master_init="fan_in"),
    "model12_perparam_r8": dict(
        cid=9, units=[[p] for _ in range(12) for p in BLOCK_512], R=8, layout=PER_PARAM,
        grad_dtype="bf16", param_dtype="bf16", grad_sigma=1e-3, steps=3, master_init="fan_in"),
    "group4096_flat_r8": dict(
        cid=7, units=[GROUP_4096], R=8, layout=FLAT,
        grad_dtype="bf16", param_dtype="bf16", grad_sigma=1e-3, steps=3,
        master_init="fan_in"),
}


def shapes_of(unit):
    return [tuple(s) for _, s in unit]


def numel_of(shape) -> int:
    n = 1
    for d in shape:
        n *= int(d)
    return n
