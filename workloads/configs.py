"""Model shapes and named synthetic workloads.

A shape is the seven-value model configuration of the curta-core inference
core ("The inference core" page, section "WebAssembly exports": the
configuration is seven u32 values), taken in the order dim, hidden, layers,
heads, kv_heads, vocab, context.  The pages do not list that order; it is
the header order of the llama2.c checkpoints the converter reads.

A workload adds what one batch of independent runs needs: how many runs,
how many prompt ids each run is fed, the max-tokens limit, the temperature
and the seeds from which every weight byte and prompt id is drawn.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Shape:
    dim: int
    hidden: int
    layers: int
    heads: int
    kv_heads: int
    vocab: int
    context: int

    @property
    def head_size(self) -> int:
        return self.dim // self.heads

    @property
    def kv_dim(self) -> int:
        return self.kv_heads * self.head_size

    def as_tuple(self):
        return (self.dim, self.hidden, self.layers, self.heads, self.kv_heads,
                self.vocab, self.context)


@dataclass(frozen=True)
class Workload:
    name: str
    shape: Shape
    runs: int            # independent runs in one batch
    prompt: int          # prompt ids fed to each run
    max_tokens: int      # tokens each run may generate
    temperature_q16: int = 0
    blob_seed: int = 1000
    ids_seed: int = 2000
    run_seed: int = 42   # sampler seed of run r is run_seed + r
    note: str = ""

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of the build.  Sizes follow the descriptions of the
# models and batches they stand in for; weights and ids are synthetic.
TINY = Workload(
    name="tiny-1L-d64",
    shape=Shape(64, 172, 1, 4, 4, 512, 32),
    runs=1, prompt=16, max_tokens=16, blob_seed=1000, ids_seed=2000,
    note="1 layer, dim 64, 4x16 heads, FFN 172, vocab 512, context 32")

M1B = Workload(
    name="1.1B-shaped-d2048-L22",
    shape=Shape(2048, 5632, 22, 32, 32, 32000, 2048),
    runs=32, prompt=128, max_tokens=128, blob_seed=1002, ids_seed=2002,
    note="22 layers, dim 2048, 32x64 heads, FFN 5632, vocab 32000")

M7B = Workload(
    name="7B-shaped-d4096-L32",
    shape=Shape(4096, 11008, 32, 32, 32, 32000, 4096),
    runs=64, prompt=512, max_tokens=256, blob_seed=1003, ids_seed=2003,
    note="32 layers, dim 4096, 32x128 heads, FFN 11008, vocab 32000")

LONG8K = Workload(
    name="long-context-8k-d2048-L16",
    shape=Shape(2048, 5632, 16, 16, 16, 32000, 8192),
    runs=16, prompt=7936, max_tokens=256, blob_seed=1004, ids_seed=2004,
    note="16 layers, dim 2048, 16x128 heads, FFN 5632, context 8192")

# The standalone matrix-row sweep: one 4096x4096 matrix, batches of inputs.
ROW_SWEEP_ROWS = 4096
ROW_SWEEP_COLS = 4096
ROW_SWEEP_BATCHES = (1, 8, 32, 128)
ROW_SWEEP_SEED = 1001

# Small shapes used by the parity tests: several tiles and ragged tails,
# grouped-query attention, odd hidden sizes.
SMALL_SHAPES = {
    "tiny": TINY.shape,
    "gqa": Shape(96, 200, 2, 6, 2, 300, 40),
    "ragged": Shape(160, 392, 2, 5, 5, 1000, 48),
    "wide": Shape(256, 704, 2, 4, 4, 2048, 64),
    "h8": Shape(64, 128, 1, 8, 4, 64, 24),
    # wide enough that the row kernel splits the columns of every matrix
    "split": Shape(1024, 2816, 2, 8, 4, 700, 24),
    # the longest and the shortest heads of the vector attention path, grouped
    "h256": Shape(512, 1024, 2, 2, 1, 500, 40),
    "h4": Shape(32, 96, 1, 8, 2, 200, 24),
}


def by_name(name: str) -> Workload:
    for w in (TINY, M1B, M7B, LONG8K):
        if w.name == name:
            return w
    raise KeyError(name)
