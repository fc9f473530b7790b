"""The seeded synthetic workloads and their tensors.

Every tensor of layer `l` is keyed by (seed, tensor id, l, batch, row), so a
slice generated on the host equals the same slice generated on the device.
Recipes (stated once here, used by tests, smoke and bench):
  indexer keys   k8[B][L][128]   N(0,1) -> bf16 -> E4M3 with a per-key scale
                 (amax/448); optionally a planted subset shifted by +3 sigma
  indexer query  q8[B][T][32][128] same quantisation, one scale per (t, head)
  head weights   w[B][T][32]     U(0,1)
  attn query     q[B][T][64][576] N(0,1) bf16
  latent KV      kv[B][L][576]   N(0,1) bf16, or E4M3 + per-row scale
For MTP draft reuse, draft step s uses attention query layer s and the
indexer inputs, keys and KV of layer 0.
"""
from dataclasses import dataclass

import numpy as np

from . import (ATT_HEADS, IDX_DIM, IDX_HEADS, KV_DIM, T_ATT_Q, T_IDX_KEY, T_IDX_Q, T_IDX_W,
               T_KV, dev_bf16_rows, dev_fp8_rows, dev_uniform_rows, host_bf16_rows,
               host_fp8_rows, host_uniform_rows)

SCHED_GROUP4, SCHED_GLM52, SCHED_ALL_FULL = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    T: int
    L: int
    n_layers: int
    sched: int = SCHED_GROUP4
    kv_fp8: bool = False
    plant_permyriad: int = 0
    prefix: int = -1  # >= 0: causal chunk, vis_len[t] = prefix + t + 1
    mtp_steps: int = 0
    k: int = 2048
    sm_scale: float = 1.0 / 24.0  # 1/sqrt(576)

    def vis_len(self):
        if self.prefix < 0:
            return np.full((self.B, self.T), self.L, np.int32)
        v = self.prefix + 1 + np.arange(self.T, dtype=np.int64)
        return np.broadcast_to(v.astype(np.int32), (self.B, self.T)).copy()

    def indexer_layer(self, l):
        """layer whose indexer inputs / keys / KV a layer or draft step reads"""
        return 0 if self.mtp_steps else l

    def full_layers(self):
        if self.mtp_steps:
            return [0]
        if self.sched == SCHED_GROUP4:
            return [l for l in range(self.n_layers) if l % 4 == 0]
        if self.sched == SCHED_GLM52:
            return [l for l in range(self.n_layers) if l < 2 or (l - 2) % 4 == 0]
        return list(range(self.n_layers))


WORKLOADS = {
    # tiny single IndexShare group, 4 decode queries of one sequence
    "tiny": Workload("tiny-group-L8192", seed=1, B=1, T=4, L=8192, n_layers=4),
    # decode, one 4-layer group, 1% planted +3 sigma keys per sequence
    "decode128k": Workload("decode-B32-L131072-group4", seed=2, B=32, T=1, L=131072,
                           n_layers=4, plant_permyriad=100),
    # chunked prefill: 4096 queries at the end of a 131072-position cache
    "prefill": Workload("prefill-T4096-L131072-group4", seed=3, B=1, T=4096, L=131072,
                        n_layers=4, prefix=131072 - 4096),
    # the 78-layer schedule at 1M with FP8 latent KV
    "decode1m": Workload("decode-B2-L1048576-78layers-fp8kv", seed=4, B=2, T=1, L=1 << 20,
                         n_layers=78, sched=SCHED_GLM52, kv_fp8=True),
    # MTP draft reuse, 7 draft steps on one shared layer
    "mtp1m": Workload("mtp-B8-L1048576-7steps-fp8kv", seed=5, B=8, T=1, L=1 << 20, n_layers=7,
                      kv_fp8=True, mtp_steps=7),
    # MTP verify: 1 + 5 draft tokens per sequence scored in one pass, causal
    # among themselves (vis_len = L - 6 + t + 1), one 4-layer group
    "verify128k": Workload("verify-B32-T6-L131072-group4", seed=6, B=32, T=6, L=131072,
                           n_layers=4, plant_permyriad=100, prefix=131072 - 6),
}


# ------------------------------------------------------------------ host side
def host_indexer(w: Workload, layer, b0=0, nb=None, with_keys=True, key_r0=0, key_nr=None):
    nb = w.B - b0 if nb is None else nb
    q8, qs = host_fp8_rows(w.seed, T_IDX_Q, layer, w.T * IDX_HEADS, IDX_DIM, 0, b0, nb, 0,
                           w.T * IDX_HEADS)
    wt = host_uniform_rows(w.seed, T_IDX_W, layer, IDX_HEADS, b0, nb, 0, w.T)
    d = {"q8": q8.reshape(nb, w.T, IDX_HEADS, IDX_DIM), "q_scale": qs.reshape(nb, w.T, IDX_HEADS),
         "w": wt.reshape(nb, w.T, IDX_HEADS)}
    if with_keys:
        key_nr = w.L - key_r0 if key_nr is None else key_nr
        k8, ks = host_fp8_rows(w.seed, T_IDX_KEY, layer, w.L, IDX_DIM, w.plant_permyriad, b0, nb,
                               key_r0, key_nr)
        d["k8"], d["k_scale"] = k8, ks
    return d


def host_attn_q(w: Workload, layer, b0=0, nb=None):
    nb = w.B - b0 if nb is None else nb
    q = host_bf16_rows(w.seed, T_ATT_Q, layer, KV_DIM, b0, nb, 0, w.T * ATT_HEADS)
    return q.reshape(nb, w.T, ATT_HEADS, KV_DIM)


def host_kv(w: Workload, layer, b0=0, nb=None, r0=0, nr=None):
    """(kv, kv_scale): bf16 bits [nb][nr][576] and None, or E4M3 codes and scales"""
    nb = w.B - b0 if nb is None else nb
    nr = w.L - r0 if nr is None else nr
    if w.kv_fp8:
        return host_fp8_rows(w.seed, T_KV, layer, w.L, KV_DIM, 0, b0, nb, r0, nr)
    return host_bf16_rows(w.seed, T_KV, layer, KV_DIM, b0, nb, r0, nr), None


def host_kv_rows(w: Workload, layer, b, positions):
    """KV rows of batch b at arbitrary positions, as a dense [1][L'] slice where
    L' = len(positions); returns (kv, kv_scale)"""
    kv = np.empty((1, len(positions), KV_DIM), np.uint8 if w.kv_fp8 else np.uint16)
    sc = np.empty((1, len(positions)), np.float32) if w.kv_fp8 else None
    for i, s in enumerate(positions):
        a, c = host_kv(w, layer, b, 1, int(s), 1)
        kv[0, i] = a[0, 0]
        if sc is not None:
            sc[0, i] = c[0, 0]
    return kv, sc


# ---------------------------------------------------------------- device side
def dev_indexer(w: Workload, layer, device, keys=True):
    import torch
    B, T = w.B, w.T
    d = {
        "q8": torch.empty((B, T, IDX_HEADS, IDX_DIM), dtype=torch.uint8, device=device),
        "q_scale": torch.empty((B, T, IDX_HEADS), dtype=torch.float32, device=device),
        "w": torch.empty((B, T, IDX_HEADS), dtype=torch.float32, device=device),
    }
    dev_fp8_rows(w.seed, T_IDX_Q, layer, T * IDX_HEADS, IDX_DIM, 0, 0, B, 0, T * IDX_HEADS,
                 d["q8"], d["q_scale"])
    dev_uniform_rows(w.seed, T_IDX_W, layer, IDX_HEADS, 0, B, 0, T, d["w"])
    if keys:
        d["k8"] = torch.empty((B, w.L, IDX_DIM), dtype=torch.uint8, device=device)
        d["k_scale"] = torch.empty((B, w.L), dtype=torch.float32, device=device)
        dev_fp8_rows(w.seed, T_IDX_KEY, layer, w.L, IDX_DIM, w.plant_permyriad, 0, B, 0, w.L,
                     d["k8"], d["k_scale"])
    return d


def dev_attn_q(w: Workload, layer, device):
    import torch
    q = torch.empty((w.B, w.T, ATT_HEADS, KV_DIM), dtype=torch.bfloat16, device=device)
    dev_bf16_rows(w.seed, T_ATT_Q, layer, KV_DIM, 0, w.B, 0, w.T * ATT_HEADS, q)
    return q


def dev_kv(w: Workload, layer, device):
    import torch
    if w.kv_fp8:
        kv = torch.empty((w.B, w.L, KV_DIM), dtype=torch.uint8, device=device)
        sc = torch.empty((w.B, w.L), dtype=torch.float32, device=device)
        dev_fp8_rows(w.seed, T_KV, layer, w.L, KV_DIM, 0, 0, w.B, 0, w.L, kv, sc)
        return kv, sc
    kv = torch.empty((w.B, w.L, KV_DIM), dtype=torch.bfloat16, device=device)
    dev_bf16_rows(w.seed, T_KV, layer, KV_DIM, 0, w.B, 0, w.L, kv)
    return kv, None
