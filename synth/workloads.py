"""The five workloads: simulated rank count W and bf16 parameter shapes.

Shapes are those of one decoder layer (or block) of the named model families;
gradients of each (rank, parameter) pair are separate tensors, as autograd
leaves them.
"""
from dataclasses import dataclass, field
from typing import List, Tuple

Shape = Tuple[int, ...]


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    world: int
    shapes: List[Shape] = field(hash=False)
    names: List[str] = field(hash=False)
    sigma: float
    outliers: bool = False

    @property
    def nparams(self) -> int:
        return len(self.shapes)

    def numel(self, p: int) -> int:
        n = 1
        for d in self.shapes[p]:
            n *= d
        return n


def _tiny():
    shapes = [(7, 5), (16,), (33, 8), (3, 3, 4)]
    return Workload(0, "tiny", 4, shapes, ["p0", "p1", "p2", "p3"], sigma=1.0)


def _llama(index, name, hidden, kv, ffn):
    named = [
        ("q_proj", (hidden, hidden)),
        ("k_proj", (kv, hidden)),
        ("v_proj", (kv, hidden)),
        ("o_proj", (hidden, hidden)),
        ("gate_proj", (ffn, hidden)),
        ("up_proj", (ffn, hidden)),
        ("down_proj", (hidden, ffn)),
        ("input_layernorm", (hidden,)),
        ("post_attention_layernorm", (hidden,)),
    ]
    return named


def _llama8b():
    named = _llama(1, "llama3.1-8b-layer", 4096, 1024, 14336)
    return Workload(1, "llama3.1-8b-layer", 8, [s for _, s in named], [n for n, _ in named], sigma=1e-3)


def _llama70b():
    named = _llama(2, "llama3.1-70b-layer", 8192, 1024, 28672)
    return Workload(2, "llama3.1-70b-layer", 8, [s for _, s in named], [n for n, _ in named], sigma=1e-3,
                    outliers=True)


def _qwen3_moe():
    named = [
        ("q_proj", (4096, 2048)),
        ("k_proj", (512, 2048)),
        ("v_proj", (512, 2048)),
        ("o_proj", (2048, 4096)),
        ("router", (128, 2048)),
    ]
    for e in range(128):
        named += [
            (f"experts.{e}.gate_proj", (768, 2048)),
            (f"experts.{e}.up_proj", (768, 2048)),
            (f"experts.{e}.down_proj", (2048, 768)),
        ]
    named += [
        ("q_norm", (128,)),
        ("k_norm", (128,)),
        ("input_layernorm", (2048,)),
        ("post_attention_layernorm", (2048,)),
    ]
    return Workload(3, "qwen3-30b-a3b-moe-layer", 8, [s for _, s in named], [n for n, _ in named], sigma=1e-3)


def _wan22_block():
    h, f = 5120, 13824
    named = []
    for attn in ("self_attn", "cross_attn"):
        for proj in ("q", "k", "v", "o"):
            named += [(f"{attn}.{proj}.weight", (h, h)), (f"{attn}.{proj}.bias", (h,))]
    named += [
        ("ffn.0.weight", (f, h)),
        ("ffn.0.bias", (f,)),
        ("ffn.2.weight", (h, f)),
        ("ffn.2.bias", (h,)),
        ("norm1", (h,)),
        ("norm2", (h,)),
        ("norm3", (h,)),
        ("modulation", (6, h)),
    ]
    return Workload(4, "wan2.2-dit-block", 8, [s for _, s in named], [n for n, _ in named], sigma=1e-3)


def _equal16(index, name, side):
    """The shape class of the reduce-scatter latency table of "The Endgame of
    FSDP Communication" (Table 8): 16 bf16 gradients and 32 or 128 MiB of
    fp32 output per rank at W = 8.  The pages give no tensor shapes; these are
    16 equal square tensors of that total: side 2048 gives 16 x 256 rows x
    2048 = 8 Mi fp32 elements (32 MiB) per rank, side 4096 gives 128 MiB."""
    shapes = [(side, side)] * 16
    return Workload(index, name, 8, shapes, [f"grad{i}" for i in range(16)], sigma=1e-3)


WORKLOADS = {w.name: w for w in (_tiny(), _llama8b(), _llama70b(), _qwen3_moe(), _wan22_block())}
WORKLOAD_ORDER = ["tiny", "llama3.1-8b-layer", "llama3.1-70b-layer", "qwen3-30b-a3b-moe-layer", "wan2.2-dit-block"]

# Context shapes: not among the graded workloads above, for comparisons with
# the pages' own latency tables.
CONTEXT_WORKLOADS = {w.name: w for w in (_equal16(5, "equal16-32mib", 2048), _equal16(6, "equal16-128mib", 4096))}


def workload(name: str) -> Workload:
    if name in WORKLOADS:
        return WORKLOADS[name]
    if name in CONTEXT_WORKLOADS:
        return CONTEXT_WORKLOADS[name]
    raise KeyError(f"unknown workload {name!r}; known: {', '.join(WORKLOAD_ORDER + list(CONTEXT_WORKLOADS))}")
