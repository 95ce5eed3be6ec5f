"""vattn_decode_noalloc (the library's static device scratch instead of a
workspace argument) against vattn_decode with a caller workspace: two calls in
a row, the second with a smaller input, each bit-identical to the existing
entry point on the same inputs and seed (index sets, counts, statistics, out,
lse)."""
import ctypes as C

import numpy as np
import pytest

import synthetic

pytestmark = pytest.mark.gpu

KEYS = ("idx", "counts", "stats", "out", "lse")


def _outputs(dec):
    return dict(idx=dec.idx.cpu().numpy(), counts=dec.counts.cpu().numpy(),
                stats=dec.stats.cpu().numpy().view(np.uint64), out=dec.out.cpu().numpy(),
                lse=dec.lse.cpu().numpy())


def _pair(w, seed):
    """(noalloc, workspace) results of one decode of workload w."""
    import torch
    import verified_sparse_attention_amd as vsa
    from tests.gpu_run import log
    dev = torch.device("cuda:0")
    q, bt, sl = w.q.to(dev), w.block_table.to(dev), w.seq_lens.to(dev)
    k, v = w.k_cache.to(dev), w.v_cache.to(dev)
    proj = w.proj.to(dev) if w.proj is not None else None
    kt = vsa.project_keys(k, proj) if w.cfg["predictor"] == 1 else None
    res = []
    for noalloc in (True, False):
        cfg = vsa.Config.from_dict(dict(w.cfg, seed=seed))
        dec = vsa.Decoder(q, k, v, bt, sl, cfg, max_seq_len=w.max_seq_len, k_lowrank=kt, proj=proj,
                          want_idx=True, noalloc=noalloc)
        log("[noalloc] %s noalloc=%s B=%d L=%s scratch need %d bytes"
            % (w.name, noalloc, w.B, w.seq_lens.tolist()[:4], dec.ws_bytes))
        dec()
        torch.cuda.synchronize()
        res.append(_outputs(dec))
    return res


def test_noalloc_matches_workspace_entry_point_twice():
    import verified_sparse_attention_amd as vsa
    big = synthetic.llama8b_32k(B=2, name="llama8b_32k_b2")
    small = synthetic.make(name="small_ragged", B=3, Hq=16, Hkv=4, d=128, seq_lens=(5000, 2500, 777),
                           kv_dtype="bf16", recipe="outlier", predictor=1, rank=32, sinks=32, window=64,
                           topk_ppm=25000, shuffle=True, data_seed=11)
    for w, seed in ((big, 3), (small, 4)):  # second call: smaller input, scratch holds the first's contents
        got, want = _pair(w, seed)
        for key in KEYS:
            assert np.array_equal(got[key], want[key]), (w.name, key)
    assert vsa.load().vattn_decode_noalloc is not None


def test_noalloc_rejects_oversized_before_any_launch():
    import verified_sparse_attention_amd as vsa
    lib = vsa.load()
    inp = vsa.vattn_inputs(256, 256, 256, 256, 256, 256, 256, 64, 32, 8, 128, 1024, 65536, 16384,
                           vsa.BF16, 1, None)
    cfg = vsa.Config(sinks=64, window=64, topk_ppm=20000, rank=32).to_c()
    assert lib.vattn_workspace_size(C.byref(inp), C.byref(cfg)) > vsa.NOALLOC_SCRATCH_BYTES
    outs = vsa.vattn_outputs(256, 256, None, 0, None, None, None, 0.0)
    assert lib.vattn_decode_noalloc(C.byref(inp), C.byref(cfg), C.byref(outs), None) == 5  # VATTN_E_WORKSPACE
