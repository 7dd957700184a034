"""The workloads the all-reduce is measured and checked on.

Shapes follow the pages' workloads:
  - Baidu Ring-Allreduce article, paragraph after the overlap one: a language
    model of about 300 million parameters, a 1.2 GB gradient, 40 GPUs.
  - IBM DDL blog / "[论文解读] PowerAI DDL", ABSTRACT; Sony article
    throughout: ResNet-50 on ImageNet.
  - Sony article, "2D-Torus All-reduce": GPUs on a logical 2D grid;
    "训练设置": FP16 gradient exchange.
The gradient values are synthetic (see synth.h); no dataset or trained
weights are involved.  ResNet-50's parameter tensors are not listed on the
pages; they are derived here from the standard architecture (7x7 stem, four
stages of 3/4/6/3 bottleneck blocks of widths 64/128/256/512 with expansion
4, a 1x1 projection on each stage's first block, every conv followed by a
batch norm with weight and bias, a 2048x1000 classifier with bias).
"""
from dataclasses import dataclass, field
from typing import List, Optional, Tuple


def resnet50_param_sizes():
    """(name, element count) of ResNet-50's 161 parameter tensors, in
    registration (forward) order."""
    out = []

    def conv(name, cin, cout, k):
        out.append((name + ".weight", cout * cin * k * k))

    def bn(name, c):
        out.append((name + ".weight", c))
        out.append((name + ".bias", c))

    conv("conv1", 3, 64, 7)
    bn("bn1", 64)
    cin = 64
    for stage, (blocks, width) in enumerate(zip((3, 4, 6, 3), (64, 128, 256, 512))):
        cout = width * 4
        for b in range(blocks):
            pre = f"layer{stage + 1}.{b}"
            conv(pre + ".conv1", cin, width, 1)
            bn(pre + ".bn1", width)
            conv(pre + ".conv2", width, width, 3)
            bn(pre + ".bn2", width)
            conv(pre + ".conv3", width, cout, 1)
            bn(pre + ".bn3", cout)
            if b == 0:
                conv(pre + ".downsample.0", cin, cout, 1)
                bn(pre + ".downsample.1", cout)
            cin = cout
    out.append(("fc.weight", 2048 * 1000))
    out.append(("fc.bias", 1000))
    return out


def resnet50_mixed_typed_buckets():
    """Typed buckets (byte offset, count, dtype) of a mixed-precision
    ResNet-50 gradient: the convolution and fc weights in binary16, the
    BatchNorm weights and biases and the fc bias in binary32.  Tensors are
    packed in registration order (every size is a multiple of 8 elements, so
    every offset is a multiple of 16 bytes) and issued output layer first.
    Returns (buckets, nbytes)."""
    out, at = [], 0
    for name, cnt in resnet50_param_sizes():
        f32 = ".bn" in name or name.startswith("bn") or "downsample.1" in name \
            or name.endswith(".bias")
        dt = "f32" if f32 else "f16"
        out.append((at, cnt, dt))
        at += cnt * (4 if f32 else 2)
    return out[::-1], at


def reverse_layer_buckets(sizes):
    """One bucket per tensor, tensors laid out in registration order, buckets
    issued in reverse (output layer first)."""
    offs, o = [], 0
    for s in sizes:
        offs.append(o)
        o += s
    return [(offs[i], sizes[i]) for i in reversed(range(len(sizes)))]


def equal_buckets_reversed(n, nb):
    assert n % nb == 0
    s = n // nb
    return [(i * s, s) for i in reversed(range(nb))]


@dataclass
class Workload:
    name: str
    P: int
    n: int
    dtype: str                 # "f32" | "f16"
    op: str                    # "sum" | "mean"
    topo: str                  # "ring" | "multiring" | "torus2d"
    k: int = 1
    rows: int = 0
    cols: int = 0
    dist: str = "normal"
    sigma: float = 1.0
    seed: int = 0
    buckets: Optional[List[Tuple[int, int]]] = None   # issue order
    side_stream: bool = False
    description: str = ""

    def bucket_list(self):
        return self.buckets if self.buckets is not None else [(0, self.n)]

    @property
    def esize(self):
        return 4 if self.dtype == "f32" else 2

    def fused_bytes(self):
        """Algorithmic HBM bytes of one all-reduce at the floor: every rank's
        input read once and its result written once."""
        return 2 * self.P * self.n * self.esize

    def stepwise_bytes(self):
        """Bytes of the step-by-step schedule: (P-1) reduce-scatter steps of
        3 L s and (P-1) all-gather steps of 2 L s per segment of L elements."""
        return 5 * (self.P - 1) * self.n * self.esize


_RN50 = [s for _, s in resnet50_param_sizes()]
_RN50_N = sum(_RN50)

WORKLOADS = {
    w.name: w for w in [
        Workload("ring_p4_1m_sum", P=4, n=1 << 20, dtype="f32", op="sum",
                 topo="ring", dist="uniform", seed=1,
                 description="ring, 4 ranks, 2^20 fp32, uniform[-1,1), sum"),
        Workload("ring_p8_300m_mean", P=8, n=300_000_000, dtype="f32", op="mean",
                 topo="ring", dist="normal", sigma=1e-3, seed=2,
                 description="ring, 8 ranks, 300M fp32 (1.2 GB gradient), mean"),
        Workload("multiring_k4_p16_resnet50", P=16, n=_RN50_N, dtype="f32",
                 op="mean", topo="multiring", k=4, dist="normal", sigma=1e-3,
                 seed=3, buckets=reverse_layer_buckets(_RN50),
                 description="4 rings, 16 ranks, ResNet-50 fp32 gradient, "
                             "161 tensor buckets output layer first, mean"),
        Workload("torus_4x4_resnet50_f16", P=16, n=_RN50_N, dtype="f16",
                 op="mean", topo="torus2d", rows=4, cols=4, dist="normal",
                 sigma=1e-2, seed=4,
                 description="2D torus 4x4, ResNet-50 fp16 gradient (fp32 math), "
                             "mean"),
        Workload("ring_p40_300m_64b", P=40, n=300_000_000, dtype="f32", op="mean",
                 topo="ring", dist="normal", sigma=1e-3, seed=5,
                 buckets=equal_buckets_reversed(300_000_000, 64), side_stream=True,
                 description="ring, 40 ranks, 300M fp32 each (48 GB), 64 equal "
                             "buckets issued last-first on a side stream"),
    ]
}
