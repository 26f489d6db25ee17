"""Unit shapes of the synthetic workloads (Llama-shaped FSDP units).

One FSDP unit per transformer block, as in [FSDP-math, "The sharding unit:
FlatParameter and the wrapping policy"] (one wrapped block = one
FlatParameter) and the 7B-on-8-GPUs worked example on the same page
(32 block units). Shapes are row-major (out_features, in_features); tensor
order inside a unit is the order listed here.
"""

from __future__ import annotations

TINY = [  # two-layer MLP unit, 525,568 params
    ("W1", (256, 1024)), ("b1", (1024,)), ("W2", (1024, 256)), ("b2", (256,)),
]


def llama_block(hidden: int, ffn: int, kv: int | None = None):
    kv = hidden if kv is None else kv
    return [
        ("q", (hidden, hidden)), ("k", (kv, hidden)), ("v", (kv, hidden)),
        ("o", (hidden, hidden)),
        ("gate", (ffn, hidden)), ("up", (ffn, hidden)), ("down", (hidden, ffn)),
        ("norm1", (hidden,)), ("norm2", (hidden,)),
    ]


def llama_root(hidden: int, vocab: int = 32000):
    """Outermost unit: untied embedding, final norm, lm_head."""
    return [("embed", (vocab, hidden)), ("norm", (hidden,)), ("lm_head", (vocab, hidden))]


BLK7 = llama_block(4096, 11008)              # 202,383,360 params
ROOT7 = llama_root(4096)                     # 262,148,096 params
BLK70 = llama_block(8192, 28672, kv=1024)    # 855,654,400 params (GQA k/v)
ROOT70 = llama_root(8192)                    # 524,296,192 params


def shapes(unit):
    return [s for _, s in unit]


def full7b_units():
    return [BLK7] * 32 + [ROOT7]


def full70b_units():
    return [BLK70] * 80 + [ROOT70]


# The five workloads: (name, description). Sizes and hyper-parameters are
# fixed here; the GPU tests and the bench read them from this table.
ADAMW = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
MASTER_SIGMA = 0.02
GRAD_SIGMA = 1e-3

WORKLOADS = {
    "tiny": dict(config=0, units=[TINY], F=4, rank=1, steps=3),
    "blk7": dict(config=1, units=[BLK7], F=8, rank=0, steps=3),
    "full7b": dict(config=2, units=full7b_units(), F=8, rank=0, steps=1),
    "sweep": dict(config=3, units=[BLK7], Fs=[1, 2, 4, 8, 16, 64], padded_Fs=[7, 11, 13],
                  outliers=True, steps=1),
    "full70b": dict(config=4, units=full70b_units(), F=8, rank=0, steps=1),
}
