"""Runs a synthetic workload through the HIP library (C ABI via the binding)
and returns host numpy arrays shaped like the oracle's results."""
import sys

import numpy as np
import torch

import verified_sparse_attention_amd as vsa


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def device_alias(t):
    """Device address of a pinned host tensor (hipHostGetDevicePointer), or None
    when the memory is not mapped for the device."""
    import ctypes as C
    rt = C.CDLL("libamdhip64.so.7")
    rt.hipHostGetDevicePointer.argtypes = [C.POINTER(C.c_void_p), C.c_void_p, C.c_uint]
    p = C.c_void_p()
    if rt.hipHostGetDevicePointer(C.byref(p), C.c_void_p(t.data_ptr()), 0) != 0:
        return None
    return p.value


class GpuCase:
    """Device copies of one workload plus a reusable Decoder."""

    def __init__(self, w, want_idx=True, device="cuda:0", kv_host=False):
        """kv_host: K and V stay in pinned (device-mapped) host memory; the
        low-rank keys (or key signatures) are made from a device copy and kept in HBM."""
        self.w = w
        dev = torch.device(device)
        self.q = w.q.to(dev)
        self.bt = w.block_table.to(dev)
        self.sl = w.seq_lens.to(dev)
        self.proj = w.proj.to(dev) if w.proj is not None else None
        kd = w.k_cache.to(dev)
        self.kt = vsa.project_keys(kd, self.proj) if w.cfg["predictor"] == 1 else None
        self.ks = vsa.sign_keys(kd, self.proj) if w.cfg["predictor"] == 2 else None
        if kv_host:
            torch.cuda.synchronize()
            del kd
            self.k = w.k_cache.pin_memory()
            self.v = w.v_cache.pin_memory()
            # the kernels take the host addresses: they must be the device's too
            for t in (self.k, self.v):
                if device_alias(t) != t.data_ptr():
                    raise RuntimeError("pinned host memory is not mapped at the same address on the device")
        else:
            self.k = kd
            self.v = w.v_cache.to(dev)
        self.dec = vsa.Decoder(self.q, self.k, self.v, self.bt, self.sl, vsa.Config.from_dict(w.cfg),
                               max_seq_len=w.max_seq_len, k_lowrank=self.kt, proj=self.proj,
                               want_idx=want_idx, want_group_counts=True, k_sig=self.ks)

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
        r["gcounts"] = self.dec.group_counts.cpu().numpy()
        if self.dec.num_stats is not None:
            r["num_stats"] = self.dec.num_stats.cpu().numpy()
        return r
