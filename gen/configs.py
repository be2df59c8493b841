"""Workload shapes for the MoE expert-cache step (seeded, synthetic).

Shapes follow the models the FreeToken edge-MoE write-up serves ("Why personal
MoE is hard": DeepSeek-V4-Flash has 43 MoE layers, 6 of 256 routed experts per
token; evaluation setup: Qwen3.6-35B-A3B in BF16, DeepSeek-V4-Flash as native
MXFP4 expert blocks; mechanism attribution: 8192-token prefill chunks).
"""
from dataclasses import dataclass, replace

F32, BF16, MXFP4 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", BF16: "bf16", MXFP4: "mxfp4"}


@dataclass(frozen=True)
class Workload:
    name: str
    L: int            # MoE layers
    E: int            # experts per layer
    k: int            # routed experts per token
    H: int            # hidden size
    I: int            # expert intermediate size
    wdtype: int       # expert weight dtype (F32 / BF16 / MXFP4)
    slots: int        # GPU cache slots C
    K: int            # victim candidates per step
    T: int = 1        # tokens per decode step
    steps: int = 64   # decode steps
    p: float = 0.5    # step-to-step routing overlap
    bp: int = 1000    # expert transfer bandwidth BP (MB/s, integer)
    bh: int = 1000    # host-side expert processing bandwidth BH (MB/s, integer)
    sigma: float = 0.02
    seed: int = 20260817

    @property
    def act_bf16(self):
        return self.wdtype != F32

    @property
    def expert_bytes(self):
        n = self.H * self.I
        if self.wdtype == F32:
            return 3 * n * 4
        if self.wdtype == BF16:
            return 3 * n * 2
        return 3 * (n // 2) + 3 * (n // 32)

    def with_(self, **kw):
        return replace(self, **kw)


def budget_slots(L, E, budget_bp):
    """Slots for a budget given in basis points of all L*E experts (floor)."""
    return (budget_bp * L * E) // 10000


TINY = Workload("tiny", L=1, E=16, k=2, H=256, I=128, wdtype=F32, slots=8, K=2, T=1, steps=64,
                p=0.5, bp=500, bh=1000, seed=20260817 + 1)
QWEN_DECODE = Workload("qwen35b_a3b_decode", L=40, E=256, k=8, H=2048, I=512, wdtype=BF16,
                       slots=budget_slots(40, 256, 3000), K=8, T=1, steps=1024, p=0.6,
                       bp=1000, bh=1000, seed=20260817 + 2)
QWEN_PREFILL = Workload("qwen35b_a3b_prefill", L=40, E=256, k=8, H=2048, I=512, wdtype=BF16,
                        slots=0, K=8, T=8192, steps=1, p=0.0, seed=20260817 + 3)
DSV4_DECODE = Workload("dsv4_flash_decode", L=43, E=256, k=6, H=4096, I=2048, wdtype=MXFP4,
                       slots=budget_slots(43, 256, 2500), K=6, T=1, steps=1024, p=0.6,
                       bp=300, bh=1000, seed=20260817 + 4)
STRESS = Workload("dsv4_flash_stress", L=43, E=256, k=6, H=4096, I=2048, wdtype=MXFP4,
                  slots=4096, K=64, T=16, steps=256, p=0.6, bp=1000, bh=1000,
                  seed=20260817 + 5)

ALL = [TINY, QWEN_DECODE, QWEN_PREFILL, DSV4_DECODE, STRESS]
