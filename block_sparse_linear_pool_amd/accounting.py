"""FLOP and byte accounting of the SLA2 forward, per kernel of libsla2.so.

Counts only: nothing here computes any part of the method. Used by bench.py for the
full-attention-equivalent rate and the roofline fractions.

Full-attention-equivalent work is 4 B H N^2 d FLOP per call (QK^T and PV of dense
attention over the padded N, no softmax). The sparse kernel's algorithmic work is
4 * 128 * 64 * d FLOP per kept (query block, key block) pair. Byte counts are the
compulsory (algorithmic) HBM traffic of each kernel: every input read once, every
output written once; gathers that a cache can serve are not counted.
"""

from __future__ import annotations

import dataclasses

MI355X_PEAK = {
    "hbm_gbs": 8000.0,          # HBM3E, GB/s
    "mfma_i8_fp8_tflops": 5000.0,  # dense INT8 / FP8 MFMA
    "mfma_bf16_tflops": 2500.0,
    "fp64_tflops": 78.6,
    "mfma_fp32_tflops": 157.3,  # dense fp32 MFMA
}

KERNELS_FORWARD = ("pool", "colmean", "project", "score_topk", "kv_prep", "linear_total", "attn")
KERNELS_WITH_MASK = ("pool", "colmean", "mask_to_list", "kv_prep", "linear_total", "attn")
# sla2_router_soft: pool here writes block sums only (no Q codes)
KERNELS_SOFT_ROUTER = ("pool_sums", "colmean", "project", "score_soft")
# sla2_forward_sla1 (the earlier SLA mix): identity projections, alpha = 1 fill, O += O_l Wo
KERNELS_SLA1 = ("pool", "colmean", "project", "score_topk", "fill", "kv_prep", "linear_total",
                "attn", "sla1_mix")
# sla2_backward (mask given): the forward's linear precompute, the transposed mask, then the
# gradient kernels; dk_center is the column mean and the subtraction together
KERNELS_BACKWARD = ("pool_k", "colmean", "kv_prep", "linear_total", "mask_to_list", "key_lists",
                    "key_plan", "bwd_prep", "bwd_lin_q", "dh_total", "bwd_q", "bwd_kv_extra",
                    "bwd_kv", "dk_center")


@dataclasses.dataclass
class Problem:
    B: int
    H: int
    N: int
    kb: int
    d: int = 128
    in_bytes: int = 2            # bf16 inputs
    kv_main_pairs: int | None = None   # backward: kept pairs done by bwd_kv (rest: bwd_kv_extra)

    @property
    def BH(self):
        return self.B * self.H

    @property
    def nqb(self):
        return self.N // 128

    @property
    def nkb(self):
        return self.N // 64

    @property
    def E(self):                 # elements of one [B, H, N, d] tensor
        return self.BH * self.N * self.d

    @property
    def pairs(self):             # kept (query block, key block) pairs
        return self.BH * self.nqb * self.kb

    @property
    def sparsity(self):
        return 1.0 - self.kb / self.nkb


def full_attention_flops(p: Problem) -> float:
    return 4.0 * p.BH * p.N * p.N * p.d


def sparse_flops(p: Problem) -> float:
    return 4.0 * 128 * 64 * p.d * p.pairs


def linear_flops(p: Problem) -> float:
    """phi(K)^T V per key block plus phi(Q) H per query block: 4 N d^2 per head."""
    return 2.0 * p.BH * p.N * p.d * p.d + 2.0 * p.BH * p.N * p.d * p.d


def call_min_bytes(p: Problem) -> float:
    """Algorithmic-minimum HBM bytes of one forward call: Q, K, V read once, K read a second
    time for its column mean, O written in fp32, and the per-key-block h_j^T (bf16) and z_j
    (fp32) written once and read once."""
    return (3 * p.E * p.in_bytes + p.E * p.in_bytes + p.E * 4
            + 2 * p.BH * p.nkb * (p.d * p.d * 2 + p.d * 4))


def whole_call_frac(p: Problem, seconds: float) -> float:
    """Whole-call roofline fraction: the larger of the sparse branch's matrix time at the
    dense INT8/FP8 peak and the minimum bytes' time at the HBM peak, over the call's time."""
    t_mfma = sparse_flops(p) / (MI355X_PEAK["mfma_i8_fp8_tflops"] * 1e12)
    t_hbm = call_min_bytes(p) / (MI355X_PEAK["hbm_gbs"] * 1e9)
    return max(t_mfma, t_hbm) / seconds


def full_attention_backward_flops(p: Problem) -> float:
    """Dense attention backward: five N x N x d products (S, dP, dV, dK, dQ), 10 B H N^2 d."""
    return 10.0 * p.BH * p.N * p.N * p.d


def kernel_bytes(p: Problem, name: str) -> float:
    """Compulsory HBM bytes of one launch of kernel `name`."""
    E, BH, d = p.E, p.BH, p.d
    np_ = (p.nkb + 7) // 8
    if name == "pool_k":
        # K read; fp64 block sums written
        return E * p.in_bytes + BH * p.nkb * d * 8
    if name == "bwd_prep":
        # K, dO (and Q, V if fp32) read; bf16 K_s, alpha dO (and Q, V if fp32) written
        copies = 2 if p.in_bytes == 2 else 4
        return (E * p.in_bytes + E * 4 + (0 if p.in_bytes == 2 else 2 * E * p.in_bytes)
                + copies * E * 2)
    if name == "bwd_lin_q":
        # Q, dO read (and h_j, z_j once), dQ, bf16 dH_i^T and dZ_i written
        return (E * p.in_bytes + E * 4 + BH * p.nkb * (d * d * 2 + d * 4) + E * 4
                + BH * p.nqb * (d * d * 2 + d * 4))
    if name == "dh_total":
        return BH * p.nqb * (d * d * 2 + d * 4) + BH * (d * d + d) * 4
    if name == "bwd_q":
        # Q, dO, K, V read once; dQ read and written; row statistics written
        return E * p.in_bytes + E * 4 + 2 * E * p.in_bytes + 2 * E * 4 + BH * p.N * 8
    if name == "bwd_kv":
        # K, V, Q, dO, row statistics, dH_i^T read once; dK_s, dV written
        return (3 * E * p.in_bytes + E * 4 + BH * p.N * 8 + BH * p.nqb * d * d * 2
                + 2 * E * 4)
    if name == "dk_center":
        return 2 * E * 4 + BH * p.nkb * d * 4
    if name == "pool":
        # Q, K read; fp64 block sums, INT8 Q codes and scales written
        return 2 * E * p.in_bytes + BH * (p.nqb + p.nkb) * d * 8 + E + BH * p.nqb * 4
    if name == "pool_sums":
        # Q, K read; fp64 block sums written
        return 2 * E * p.in_bytes + BH * (p.nqb + p.nkb) * d * 8
    if name == "score_soft":
        # fp32 A and B read; the fp32 soft mask and lambda written
        return BH * p.nqb * d * 4 + BH * p.nkb * d * 4 + BH * p.nqb * p.nkb * 4 + BH * p.nqb * 4
    if name == "score_topk":
        # fp32 A and B read; mask, lists and counts written
        return (BH * p.nqb * d * 4 + BH * p.nkb * d * 4 + BH * p.nqb * p.nkb
                + BH * p.nqb * (p.kb + 1) * 4)
    if name == "project":
        # fp64 block sums read (keys and queries), fp32 B and A written
        return BH * (p.nkb + p.nqb) * d * (8 + 4)
    if name == "sla1_mix":
        # O_l and O read, O written
        return 3 * E * 4
    if name == "kv_prep":
        # K, V read; INT8 K_s and E4M3 V codes + scales, bf16 h_j^T, z_j, partials written
        return (2 * E * p.in_bytes + 2 * E + BH * p.nkb * 8 + BH * p.nkb * (d * d * 2 + d * 4)
                + BH * np_ * (d * d + d) * 4)
    if name == "linear_total":
        return BH * np_ * (d * d + d) * 4 + BH * (d * d + d) * 4
    if name == "attn":
        # Qhat, Khat + Vhat once, Q (phi), h_j^T + z_j once, H_tot/Z_tot, O written
        return (E + 2 * E + E * p.in_bytes + BH * p.nkb * (d * d * 2 + d * 4)
                + BH * (d * d + d) * 4 + E * 4)
    return 0.0


def kernel_flops(p: Problem, name: str) -> float:
    if name == "mask_grad":
        # stage-1 router gradient: S, delta V^T and phi(Q) phi(K_s)^T for every block pair
        return 3 * 2.0 * 128 * 64 * p.d * p.BH * p.nqb * p.nkb
    if name == "attn":
        # INT8/FP8 sparse-branch work only: the linear branch's bf16 phi(Q) H product
        # (4 N d^2 per head) is reported separately by linear_flops()
        return sparse_flops(p)
    if name in ("score_topk", "score_soft"):
        # the logits A B^T
        return 2.0 * p.BH * p.nqb * p.nkb * p.d
    if name == "project":
        # B = Kbar_s Wk and A = Qbar Wq
        return 2.0 * p.BH * (p.nkb + p.nqb) * p.d * p.d
    if name in ("kv_prep", "sla1_mix"):
        return 2.0 * p.BH * p.N * p.d * p.d
    if name == "bwd_lin_q":
        # num = a H_i, da = dnum H_i^T, dH_i = a^T dnum: 6 N d^2 per head
        return 6.0 * p.BH * p.N * p.d * p.d
    if name == "bwd_q":
        # per kept pair: S and P V (pass 1), S, dP and dS K (pass 2)
        return 5 * 2.0 * 128 * 64 * p.d * p.pairs
    if name in ("bwd_kv", "bwd_kv_extra"):
        # per kept pair: S, dP, P^T dO_s, dS^T Q; per key block (bwd_kv) phi dh_j and V dh_j^T
        main = p.pairs if p.kv_main_pairs is None else p.kv_main_pairs
        if name == "bwd_kv_extra":
            return 4 * 2.0 * 128 * 64 * p.d * (p.pairs - main)
        return 4 * 2.0 * 128 * 64 * p.d * main + 4.0 * p.BH * p.N * p.d * p.d
    return 0.0


def kernel_bound(name: str) -> str:
    """Roofline a kernel is priced against: attn on the INT8/FP8 matrix peak, the backward's
    matrix kernels on the bf16 matrix peak, the router's fp32 projections and logits on the
    fp32 matrix peak, everything else on HBM bandwidth."""
    if name == "attn":
        return "mfma"
    if name in ("bwd_q", "bwd_kv", "bwd_kv_extra", "bwd_lin_q"):
        return "mfma_bf16"
    if name in ("score_topk", "score_soft", "project"):
        return "mfma_fp32"
    return "hbm"
