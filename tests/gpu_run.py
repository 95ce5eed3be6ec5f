"""Runs a synthetic workload through the HIP library (C ABI via the binding)
and returns host numpy arrays shaped like the oracle's results."""
import sys

import numpy as np
import torch

import verified_sparse_attention_amd as vsa


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class GpuCase:
    """Device copies of one workload plus a reusable Decoder."""

    def __init__(self, w, want_idx=True, device="cuda:0"):
        self.w = w
        dev = torch.device(device)
        self.q = w.q.to(dev)
        self.k = w.k_cache.to(dev)
        self.v = w.v_cache.to(dev)
        self.bt = w.block_table.to(dev)
        self.sl = w.seq_lens.to(dev)
        self.proj = w.proj.to(dev) if w.proj is not None else None
        self.kt = vsa.project_keys(self.k, self.proj) if w.cfg["predictor"] == 1 else None
        self.dec = vsa.Decoder(self.q, self.k, self.v, self.bt, self.sl, vsa.Config.from_dict(w.cfg),
                               max_seq_len=w.max_seq_len, k_lowrank=self.kt, proj=self.proj,
                               want_idx=want_idx)

    def run(self, seed=None):
        if seed is not None:
            self.dec.set_seed(seed)
        self.dec()
        torch.cuda.synchronize()
        r = dict(out=self.dec.out.cpu().numpy(), lse=self.dec.lse.cpu().numpy(),
                 counts=self.dec.counts.cpu().numpy(),
                 stats=self.dec.stats.cpu().numpy().view(np.uint64), z32=self.dec.z_used)
        if self.dec.idx is not None:
            r["idx"] = self.dec.idx.cpu().numpy()
        return r
