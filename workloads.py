"""Seeded synthetic inputs shaped like the workloads of the vLLM pages.

This module only draws random numbers and plants special values; it holds
none of the method's arithmetic (no maxima, no argmax, no acceptance), so the
oracle and the HIP path can both be fed from it.

Shapes follow the pages:
  * draft-side get_top_tokens on a 151936-token vocabulary padded to 152064
    and split over 2 ranks (vLLM PR #39419, "Current Issue" and the fused
    get_top_tokens of PR #62604, "Purpose" item 2);
  * greedy verification of 24 requests x (K=3 drafts + 1 bonus row) over a
    200064-token vocabulary at TP4 (PR #62604, "Results": 24 requests x 4
    tokens per decode step);
  * a 4096-row stress batch over the same vocabulary at 8 ranks;
  * the edge cases of PR #62604 "Test Plan": vocabularies 1000 and 50257,
    shards narrower than a block, NaN rows, all -inf rows, planted ties
    across shard edges, unaligned padding, empty batches, placeholder drafts.
No dataset and no trained model is involved: logits are normal draws.

Draft tokens depend on the target argmax, which is the method's output, so
this module does not build them.  It returns a *plan* per draft position
(1 = copy the target token, 0 = take the uniform draw, -1 = placeholder) and
the uniform draws; ``compose_drafts`` applies a plan to target tokens that the
caller obtained elsewhere.
"""
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import torch

# A planted maximum: normal draws in fp32 stay far below it (|z| < 6), and it
# is exact in bf16.
PLANT = 64.0


@dataclass
class Workload:
    name: str
    logits: torch.Tensor            # [rows, ld], float32 or bfloat16
    vocab: int                      # V, valid columns
    shard_width: int                # W
    n_shards: int                   # S; the padded width is S*W <= ld
    blocks: List[int]               # block sizes to exercise
    n_req: int = 0                  # verification requests (0: none)
    k: int = 0                      # drafts per request
    draft_plan: Optional[torch.Tensor] = None    # int8 [R][K]: 1 target, 0 uniform, -1 placeholder
    draft_uniform: Optional[torch.Tensor] = None  # int32 [R][K], uniform over [0, V)
    notes: Dict[str, object] = field(default_factory=dict)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal_rows(n_rows: int, width: int, sigma: float, seed: int, device="cpu",
                 dtype=torch.bfloat16, chunk: int = 256, scale: float = 1.0) -> torch.Tensor:
    """sigma * N(0,1) * scale in fp32, cast (round-to-nearest-even) to dtype, chunk by chunk."""
    out = torch.empty((n_rows, width), dtype=dtype, device=device)
    g = _gen(seed, device)
    for r0 in range(0, n_rows, chunk):
        r1 = min(n_rows, r0 + chunk)
        z = torch.randn((r1 - r0, width), generator=g, device=device, dtype=torch.float32)
        z.mul_(sigma)
        if scale != 1.0:
            z.mul_(scale)
        out[r0:r1] = z.to(dtype)
    return out


def _draft_plan(n_req: int, k: int, p: float, vocab: int, seed: int):
    g = _gen(seed, "cpu")
    plan = (torch.rand((n_req, k), generator=g) < p).to(torch.int8)
    uniform = torch.randint(0, vocab, (n_req, k), generator=g, dtype=torch.int64).to(torch.int32)
    return plan, uniform


def compose_drafts(target_ids: torch.Tensor, plan: torch.Tensor, uniform: torch.Tensor) -> torch.Tensor:
    """Drafts [R][K] from target tokens [R][K(+1)] and a plan: copy, uniform draw or -1."""
    k = plan.shape[1]
    tgt = target_ids[:, :k].to(torch.int32).cpu()
    plan = plan.cpu()
    out = torch.where(plan == 1, tgt, uniform.cpu().to(torch.int32))
    return torch.where(plan == -1, torch.full_like(out, -1), out)


def synthetic_counts(n_req: int, k_max: int, seed: int, p_real: float = 0.25) -> torch.Tensor:
    """Synthetic accept counts int32 [R]: -1 (real acceptance) with probability
    p_real, otherwise a uniform draw from [0, k_max + 2] (so that counts past
    the draft count occur too).  The acceptance itself is not computed here."""
    g = _gen(seed, "cpu")
    counts = torch.randint(0, k_max + 3, (n_req,), generator=g, dtype=torch.int64)
    real = torch.rand(n_req, generator=g) < p_real
    return torch.where(real, torch.full_like(counts, -1), counts).to(torch.int32)


def config1() -> Workload:
    """4 rows x vocab 1000 fp32 ~N(0,1), one shard, block 256; rows 1 and 3 carry a
    planted exact tie of the row maximum at ids 17 and 903."""
    x = _normal_rows(4, 1000, 1.0, seed=1001, dtype=torch.float32)
    for r in (1, 3):
        x[r, 17] = PLANT
        x[r, 903] = PLANT
    return Workload("argmax_v1000_fp32", x, 1000, 1000, 1, [256])


def config2(device="cpu") -> Workload:
    """32 rows x vocab 151936 bf16 ~N(0,2)/0.7 padded to 152064 with +inf, 2 shards
    of 76032 columns, block 8192 (draft-side get_top_tokens)."""
    v, w, s = 151936, 76032, 2
    x = _normal_rows(32, s * w, 2.0, seed=1002, device=device, scale=1.0 / 0.7)
    x[:, v:] = float("inf")
    return Workload("top_tokens_v151936_bf16_tp2", x, v, w, s, [8192])


def config3(device="cpu") -> Workload:
    """24 requests x (K=3 drafts + 1 bonus) = 96 rows x vocab 200064 bf16 ~N(0,3),
    4 shards of 50016; drafts copy the target with p=0.7; blocks 8192 / 1024."""
    v, w, s, r, k = 200064, 50016, 4, 24, 3
    x = _normal_rows(r * (k + 1), v, 3.0, seed=1003, device=device)
    plan, uni = _draft_plan(r, k, 0.7, v, seed=2003)
    return Workload("verify_v200064_bf16_tp4_r24_k3", x, v, w, s, [8192, 1024], r, k, plan, uni)


def config4(device="cpu", n_rows: int = 4096, seed: int = 1004,
            dtype=torch.bfloat16) -> Workload:
    """n_rows x vocab 200064 bf16 ~N(0,3), 8 shards of 25008; verification of
    682 requests x (K=5 + 1) rows (the last 4 rows are not referenced), drafts copy
    the target with p=0.4; blocks 8192 / 1024.  dtype=torch.float32 gives the
    same values uncast (the fp32 variant of the workload)."""
    v, w, s, k = 200064, 25008, 8, 5
    r = n_rows // (k + 1)
    x = _normal_rows(n_rows, v, 3.0, seed=seed, device=device, dtype=dtype)
    plan, uni = _draft_plan(r, k, 0.4, v, seed=seed + 1000)
    tag = "fp32" if dtype == torch.float32 else "bf16"
    return Workload(f"stress_v200064_{tag}_tp8_n{n_rows}", x, v, w, s, [8192, 1024], r, k, plan,
                    uni)


# ---------------------------------------------------------------------------
# Edge cases
# ---------------------------------------------------------------------------

def _bits_f32(v: int) -> float:
    return torch.tensor([v], dtype=torch.int64).to(torch.int32).view(torch.float32).item()


def _set_bits(x: torch.Tensor, r: int, c: int, fp32_bits: int):
    """Plant an exact bit pattern (given as fp32 bits; bf16 keeps the top half)."""
    if x.dtype == torch.float32:
        x.view(torch.int32)[r, c] = torch.tensor(fp32_bits, dtype=torch.int64).to(torch.int32)
    else:
        h = (fp32_bits >> 16) & 0xFFFF
        x.view(torch.int16)[r, c] = torch.tensor(h, dtype=torch.int64).to(torch.int16)


NEG_NAN_PAYLOAD = 0xFFC12300   # -NaN with a payload (survives bf16 truncation: 0xFFC1)
POS_NAN = 0x7FC00000
POS_NAN_PAYLOAD = 0x7FA10000   # signalling-pattern NaN with payload (bf16 0x7FA1)
NEG_ZERO = 0x80000000
POS_ZERO = 0x00000000
POS_INF = 0x7F800000
NEG_INF = 0xFF800000
F32_MIN_SUB = 0x00000001       # smallest fp32 subnormal
BF16_MIN_SUB = 0x00010000      # smallest bf16 subnormal, as fp32 bits


EDGE_ROW_NAMES = [
    "all_-inf_nan_padding", "all_-inf_inf_padding", "one_nan", "nans_in_several_shards",
    "nan_only_at_last_valid", "tie_across_edge_0_1", "tie_across_last_edge",
    "three_way_cross_shard_tie", "max_at_id_0", "max_at_last_valid", "neg_zero_pos_zero_max",
    "pos_inf_twice", "subnormal_max", "neg_nan_before_pos_nan", "tie_across_block_edge",
    "random",
]


def edge_case(vocab: int, n_shards: int, dtype, seed: int) -> Workload:
    """16 planted rows over vocab V split into S shards of W = ceil(V/S); padding
    columns [V, S*W) hold NaN (row 1: +inf), and must never be chosen."""
    w = -(-vocab // n_shards)
    ld = n_shards * w
    g = _gen(seed, "cpu")
    x = (torch.randn((16, ld), generator=g) * 1.0).to(dtype)
    x[:, vocab:] = float("nan")

    def pick(lo, hi):
        return int(torch.randint(lo, hi, (1,), generator=g).item())

    # 0, 1: every valid column -inf
    x[0, :vocab] = float("-inf")
    x[1, :vocab] = float("-inf")
    x[1, vocab:] = float("inf")
    # 2: one NaN
    _set_bits(x, 2, pick(0, vocab), POS_NAN)
    # 3: NaNs in several shards (one per shard that holds valid columns)
    for s in range(n_shards):
        lo, hi = s * w, min((s + 1) * w, vocab)
        if lo < hi:
            _set_bits(x, 3, pick(lo, hi), NEG_NAN_PAYLOAD if s % 2 else POS_NAN_PAYLOAD)
    # 4: NaN only at the last valid column
    _set_bits(x, 4, vocab - 1, POS_NAN)
    # 5: tie across the edge between shards 0 and 1
    x[5, w - 1] = PLANT
    x[5, min(w, vocab - 1)] = PLANT
    # 6: tie across the last shard edge
    e = (n_shards - 1) * w
    x[6, min(e - 1, vocab - 1)] = PLANT
    x[6, min(e, vocab - 1)] = PLANT
    # 7: three-way tie in three different shards (last, middle, first)
    for s in (n_shards - 1, n_shards // 2, 0):
        lo, hi = s * w, min((s + 1) * w, vocab)
        x[7, pick(lo, hi)] = PLANT
    # 8, 9: maximum at the first / last valid column
    x[8, 0] = PLANT
    x[9, vocab - 1] = PLANT
    # 10: every value negative except a -0 and a +0 (the -0 first)
    x[10, :vocab] = -(x[10, :vocab].float().abs() + 1.0).to(dtype)
    a, b = sorted((pick(0, vocab // 2), pick(vocab // 2, vocab)))
    _set_bits(x, 10, a, NEG_ZERO)
    _set_bits(x, 10, b, POS_ZERO)
    # 11: +inf twice
    a, b = pick(0, vocab), pick(0, vocab)
    _set_bits(x, 11, a, POS_INF)
    _set_bits(x, 11, b, POS_INF)
    # 12: every value negative, the maximum a subnormal, a smaller subnormal earlier
    x[12, :vocab] = -(x[12, :vocab].float().abs() + 1.0).to(dtype)
    sub = F32_MIN_SUB if dtype == torch.float32 else BF16_MIN_SUB
    a, b = sorted((pick(0, vocab // 2), pick(vocab // 2, vocab)))
    _set_bits(x, 12, a, sub)
    _set_bits(x, 12, b, 2 * sub)
    # 13: a -NaN with payload before a +NaN
    a, b = sorted((pick(0, vocab // 2), pick(vocab // 2, vocab)))
    _set_bits(x, 13, a, NEG_NAN_PAYLOAD)
    _set_bits(x, 13, b, POS_NAN)
    # 14: tie across a global block edge (1024) inside the row
    c = 1024 if vocab > 1025 else 512
    x[14, c - 1] = PLANT
    x[14, c] = PLANT
    # 15: plain normal draws
    name = f"edge_v{vocab}_s{n_shards}_{'fp32' if dtype == torch.float32 else 'bf16'}"
    return Workload(name, x, vocab, w, n_shards, [8192, 1024, 256],
                    notes={"row_names": EDGE_ROW_NAMES})


def edge_cases() -> List[Workload]:
    out = []
    i = 0
    for vocab, s in ((50257, 3), (1000, 8)):
        for dt in (torch.float32, torch.bfloat16):
            out.append(edge_case(vocab, s, dt, seed=1500 + i))
            i += 1
    return out


# Draft plans for the edge cases (1 = copy the target, 0 = uniform draw,
# -1 = placeholder).  With 16 rows, K=1 gives 8 requests and K=5 gives 2; K=5
# is run once per variant.
EDGE_PLANS = {
    1: [[[1], [-1], [0], [0], [1], [-1], [1], [0]]],
    5: [
        [[1, 1, 1, 1, 1], [-1, -1, -1, -1, -1]],
        [[1, 1, -1, -1, -1], [1, 1, 0, 1, 1]],
        [[-1, 1, 1, 1, 1], [1, 1, 1, 1, 0]],
        [[0, 0, 0, 0, 0], [1, 1, 1, 0, -1]],
    ],
}


def edge_verify_plans(k: int, vocab: int, seed: int = 2500):
    """[(plan int8 [R][K], uniform int32 [R][K])] for K in {1, 5}.  Where the plan
    says 0 the draft is a uniform draw, except that in the first variant's
    fourth K=1 request and in the fourth K=5 variant's first request it is an id
    past the vocabulary (V+7), which can never match."""
    g = _gen(seed + k, "cpu")
    out = []
    for vi, rows in enumerate(EDGE_PLANS[k]):
        plan = torch.tensor(rows, dtype=torch.int8)
        uniform = torch.randint(0, vocab, plan.shape, generator=g, dtype=torch.int64).to(torch.int32)
        if k == 1 and vi == 0:
            uniform[3, 0] = vocab + 7
        if k == 5 and vi == 3:
            uniform[0, :] = vocab + 7
        out.append((plan, uniform))
    return out
