"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, rejects bad arguments with the documented status before any
launch, sizes its workspace, and computes the same fp32 z as the oracle."""
import ctypes as C
import os
import re
import subprocess

import pytest

import oracle
import verified_sparse_attention_amd as vsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vattn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(vsa.LIB_PATH):
        from verified_sparse_attention_amd import build
        build.build()
    return vsa.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vattn_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(vsa.EXPORTS)
    nm = subprocess.run(["nm", "-D", "--defined-only", vsa.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r"\bT (vattn_[a-z_0-9]+)$", nm, flags=re.M))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def _inputs(**kw):
    a = dict(q=256, k_cache=256, v_cache=256, k_lowrank=256, proj=256, block_table=256,
             seq_lens=256, B=2, Hq=8, Hkv=2, d=128, max_blocks=64, num_blocks=128,
             max_seq_len=1000, kv_dtype=vsa.BF16)
    a.update(kw)
    return vsa.vattn_inputs(**a)


def _cfg(**kw):
    c = vsa.Config(sinks=16, window=16, topk_ppm=25000, rank=32)
    for k, v in kw.items():
        setattr(c, k, v)
    return c.to_c()


def _decode(lib, inp, cfg, outs=None, ws=None, ws_bytes=1 << 40):
    if outs is None:
        outs = vsa.vattn_outputs(256, 256, None, 0, None, None, None, 0.0)
    return lib.vattn_decode(C.byref(inp) if inp is not None else None,
                            C.byref(cfg) if cfg is not None else None,
                            C.byref(outs) if outs is not None else None,
                            C.c_void_p(ws) if ws is not None else None, ws_bytes, None)


BAD = [
    ("hq_not_multiple", dict(Hq=6, Hkv=4), {}, 2),
    ("gqa_16", dict(Hq=32, Hkv=2), {}, 6),
    ("d_96", dict(d=96), {}, 6),
    ("seq_0", dict(max_seq_len=0), {}, 2),
    ("seq_huge", dict(max_seq_len=(1 << 20) + 1, max_blocks=70000), {}, 2),
    ("blocks_short", dict(max_blocks=10), {}, 2),
    ("dtype", dict(kv_dtype=7), {}, 3),
    ("neg_sinks", {}, dict(sinks=-1), 4),
    ("ppm", {}, dict(topk_ppm=2000000), 4),
    ("base_ppm0", {}, dict(base_ppm=0), 4),
    ("eps0", {}, dict(eps=0.0), 4),
    ("delta1", {}, dict(delta=1.0), 4),
    ("predictor", {}, dict(predictor=5), 4),
    ("proj_heads", dict(proj_heads=3), {}, 2),  # neither one basis nor one per KV head
    ("rank", {}, dict(rank=24), 6),
    ("rank_gt_d", dict(d=64), dict(rank=128), 6),
    ("hash_rank", {}, dict(predictor=2, rank=16), 6),  # signatures have 32 bits
]


@pytest.mark.parametrize("name,ikw,ckw,code", BAD, ids=[b[0] for b in BAD])
def test_rejects_bad_arguments(lib, name, ikw, ckw, code):
    inp, cfg = _inputs(**ikw), _cfg(**ckw)
    assert _decode(lib, inp, cfg) == code
    assert lib.vattn_workspace_size(C.byref(inp), C.byref(cfg)) == 0


def test_null_and_workspace_errors(lib):
    inp, cfg = _inputs(), _cfg()
    assert _decode(lib, None, cfg) == 1
    assert _decode(lib, inp, None) == 1
    assert lib.vattn_decode(C.byref(inp), C.byref(cfg), None, None, 0, None) == 1
    outs = vsa.vattn_outputs(None, 256, None, 0, None, None, None, 0.0)
    assert _decode(lib, inp, cfg, outs=outs) == 1
    assert _decode(lib, _inputs(k_lowrank=None), cfg, ws=256) == 1
    assert _decode(lib, _inputs(q=None), cfg, ws=256) == 1
    # idx capacity below max_seq_len
    outs = vsa.vattn_outputs(256, 256, 256, 999, None, None, None, 0.0)
    assert _decode(lib, inp, cfg, outs=outs, ws=256) == 2
    # misaligned q
    assert _decode(lib, _inputs(q=260), cfg, ws=256) == 2
    need = lib.vattn_workspace_size(C.byref(inp), C.byref(cfg))
    assert need > 0
    assert _decode(lib, inp, cfg, ws=None) == 5
    assert _decode(lib, inp, cfg, ws=256, ws_bytes=need - 1) == 5
    assert _decode(lib, inp, cfg, ws=256 + 64, ws_bytes=need) == 5
    # project_keys argument checks
    P = C.c_void_p
    assert lib.vattn_project_keys(None, 1, P(256), P(256), 4, 2, 128, 32, 1, None) == 1
    assert lib.vattn_project_keys(P(256), 3, P(256), P(256), 4, 2, 128, 32, 1, None) == 3
    assert lib.vattn_project_keys(P(256), 1, P(256), P(256), 4, 2, 128, 24, 1, None) == 6
    assert lib.vattn_project_keys(P(256), 1, P(256), P(256), 0, 2, 128, 32, 1, None) == 2
    assert lib.vattn_project_keys(P(256), 1, P(256), P(256), 4, 2, 128, 32, 3, None) == 2  # proj_heads


def test_append_kv_argument_checks(lib):
    P = C.c_void_p
    ok = dict(k_new=P(256), v_new=P(256), pos=P(256), bt=P(256), B=4, mb=8, kc=P(256), vc=P(256),
              kt=P(256), proj=P(256), dt=1, nb=32, Hkv=2, d=128, r=32, ph=1)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.vattn_append_kv(a["k_new"], a["v_new"], a["pos"], a["bt"], a["B"], a["mb"], a["kc"],
                                   a["vc"], a["kt"], a["proj"], a["dt"], a["nb"], a["Hkv"], a["d"], a["r"],
                                   a["ph"], None)
    assert call(k_new=None) == 1
    assert call(pos=None) == 1
    assert call(kt=None) == 1          # projection without an output
    assert call(dt=5) == 3
    assert call(B=0) == 2
    assert call(Hkv=0) == 2
    assert call(d=96) == 6
    assert call(r=24) == 6
    assert call(d=64, r=128) == 6     # rank above the head dim
    assert call(kc=P(260)) == 2        # misaligned
    assert call(ph=3) == 2             # neither one basis nor one per KV head


def test_hash_predictor_argument_checks(lib):
    P = C.c_void_p
    cfg = _cfg(predictor=2, rank=32)
    inp = _inputs(k_sig=256)
    need = lib.vattn_workspace_size(C.byref(inp), C.byref(cfg))
    assert need > 0
    assert _decode(lib, _inputs(k_sig=None), cfg, ws=256) == 1
    assert _decode(lib, _inputs(k_sig=256, proj=None), cfg, ws=256) == 1
    assert _decode(lib, _inputs(k_sig=264), cfg, ws=256) == 2  # misaligned signatures
    assert _decode(lib, inp, cfg, ws=256, ws_bytes=need - 1) == 5

    def sign(**kw):
        a = dict(k=P(256), dt=1, proj=P(256), ks=P(256), nb=4, Hkv=2, d=128, ph=1)
        a.update(kw)
        return lib.vattn_sign_keys(a["k"], a["dt"], a["proj"], a["ks"], a["nb"], a["Hkv"], a["d"], a["ph"], None)
    assert sign(k=None) == 1 and sign(proj=None) == 1 and sign(ks=None) == 1
    assert sign(dt=3) == 3
    assert sign(d=96) == 6
    assert sign(nb=0) == 2
    assert sign(ph=3) == 2
    assert sign(ks=P(260)) == 2

    def app(**kw):
        a = dict(kn=P(256), vn=P(256), pos=P(256), bt=P(256), B=2, mb=4, kc=P(256), vc=P(256), ks=P(256),
                 proj=P(256), dt=1, nb=8, Hkv=2, d=128, ph=1)
        a.update(kw)
        return lib.vattn_append_kv_sig(a["kn"], a["vn"], a["pos"], a["bt"], a["B"], a["mb"], a["kc"], a["vc"],
                                       a["ks"], a["proj"], a["dt"], a["nb"], a["Hkv"], a["d"], a["ph"], None)
    assert app(ks=None) == 1 and app(proj=None) == 1 and app(kn=None) == 1
    assert app(dt=2) == 3
    assert app(B=0) == 2
    assert app(ph=5) == 2
    assert app(d=80) == 6
    assert app(ks=P(264)) == 2


def test_key_gram_argument_checks(lib):
    P = C.c_void_p
    ws = lib.vattn_key_gram_workspace_size(2, 4, 128, 10000)
    assert ws > 0 and ws % 256 == 0
    assert lib.vattn_key_gram_workspace_size(2, 4, 96, 10000) == 0
    assert lib.vattn_key_gram_workspace_size(2, 4, 128, (1 << 20) + 1) == 0
    assert lib.vattn_key_gram_workspace_size(2, 4, 128, 20000) >= ws

    def call(**kw):
        a = dict(k=P(256), dt=1, bt=P(256), sl=P(256), B=2, mb=700, nb=1400, Hkv=4, d=128, msl=10000,
                 gram=P(256), ws=P(256), wsb=ws)
        a.update(kw)
        return lib.vattn_key_gram(a["k"], a["dt"], a["bt"], a["sl"], a["B"], a["mb"], a["nb"], a["Hkv"], a["d"],
                                  a["msl"], a["gram"], a["ws"], a["wsb"], None)
    assert call(k=None) == 1
    assert call(gram=None) == 1
    assert call(dt=7) == 3
    assert call(dt=0) == 6            # fp32 caches: bf16 only
    assert call(d=96) == 6
    assert call(B=0) == 2
    assert call(mb=10) == 2           # block table shorter than max_seq_len
    assert call(k=P(264)) == 2        # misaligned
    assert call(ws=None) == 5
    assert call(wsb=ws - 1) == 5


def test_read_probe_argument_checks(lib):
    lib.vattn_read_probe.restype = C.c_int
    lib.vattn_read_probe.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p]
    P = C.c_void_p
    assert lib.vattn_read_probe(None, 256, P(256), None) == 1
    assert lib.vattn_read_probe(P(256), 256, None, None) == 1
    assert lib.vattn_read_probe(P(256), 0, P(256), None) == 2
    assert lib.vattn_read_probe(P(256), 100, P(256), None) == 2      # not a multiple of 16
    assert lib.vattn_read_probe(P(264), 256, P(256), None) == 2      # misaligned buffer


def test_workspace_size_monotone(lib):
    cfg = _cfg()
    prev = 0
    for L in (16, 100, 1000, 5000, 32768, 131072):
        inp = _inputs(max_seq_len=L, max_blocks=(L + 15) // 16)
        n = lib.vattn_workspace_size(C.byref(inp), C.byref(cfg))
        assert n >= prev and n % 256 == 0
        prev = n
    a = lib.vattn_workspace_size(C.byref(_inputs(B=1)), C.byref(cfg))
    b = lib.vattn_workspace_size(C.byref(_inputs(B=4)), C.byref(cfg))
    assert b > a


def test_z_matches_oracle_and_status_strings(lib):
    for delta in (0.5, 0.2, 0.1, 0.05, 0.02, 0.01, 1e-3, 1e-6, 0.9):
        assert lib.vattn_z_from_delta(delta) == oracle.z_for_delta(delta)
    assert lib.vattn_z_from_delta(0.0) != lib.vattn_z_from_delta(0.0)  # NaN
    for code, name in vsa.STATUS.items():
        assert lib.vattn_status_string(code).decode().startswith(name)


def test_profiled_entry_point_argument_checks(lib):
    inp, cfg = _inputs(), _cfg()
    outs = vsa.vattn_outputs(256, 256, None, 0, None, None, None, 0.0)
    ne = vsa.NUM_STAGES + 1
    ev = (C.c_void_p * ne)(*([256] * ne))
    f = lib.vattn_decode_profiled
    assert f(C.byref(inp), C.byref(cfg), C.byref(outs), None, 0, None, None, ne) == 1
    assert f(C.byref(inp), C.byref(cfg), C.byref(outs), None, 0, None, ev, ne - 1) == 2
    ev0 = (C.c_void_p * ne)(*([256] * (ne - 1) + [None]))
    assert f(C.byref(inp), C.byref(cfg), C.byref(outs), None, 0, None, ev0, ne) == 1
    assert f(C.byref(inp), C.byref(cfg), C.byref(outs), None, 0, None, ev, ne) == 5
    assert len(vsa.STAGES) == vsa.NUM_STAGES
    text = open(HEADER).read()
    assert re.search(r"#define VATTN_NUM_STAGES %d\b" % vsa.NUM_STAGES, text)


# ---------------------------------------------------------------------------
# Binding checks: dtypes and shapes the C ABI cannot see behind raw pointers
# (a wrong one would make the kernels read past a buffer).  CPU tensors: every
# check fails before any device work.
# ---------------------------------------------------------------------------
def _tensors(**over):
    import torch
    B, Hq, Hkv, d, nb, r = 2, 8, 2, 128, 20, 32
    t = dict(q=torch.zeros(B, Hq, d), k_cache=torch.zeros(nb, Hkv, 16, d, dtype=torch.bfloat16),
             v_cache=torch.zeros(nb, Hkv, 16, d, dtype=torch.bfloat16),
             block_table=torch.zeros(B, 10, dtype=torch.int32), seq_lens=torch.zeros(B, dtype=torch.int32),
             k_lowrank=torch.zeros(nb, Hkv, 16, r, dtype=torch.int16), proj=torch.zeros(d, r),
             k_sig=None)
    t.update(over)
    return t


@pytest.mark.parametrize("over,cfg_kw,msg", [
    (lambda torch: dict(q=torch.zeros(2, 8, 128, dtype=torch.bfloat16)), {}, "q must be float32"),
    (lambda torch: dict(q=torch.zeros(2, 8, 64)), {}, "k_cache must be"),
    (lambda torch: dict(proj=torch.zeros(128, 16)), {}, "proj must have 32 columns"),
    (lambda torch: dict(proj=torch.zeros(64, 32)), {}, "proj must have d = 128"),
    (lambda torch: dict(proj=torch.zeros(3, 128, 32)), {}, "Hkv = 2"),
    (lambda torch: dict(k_lowrank=torch.zeros(20, 2, 16, 16, dtype=torch.int16)), {}, "r = 32"),
    (lambda torch: dict(k_lowrank=torch.zeros(19, 2, 16, 32, dtype=torch.int16)), {}, "matching k_cache"),
    (lambda torch: dict(block_table=torch.zeros(2, 10, dtype=torch.int64)), {}, "block_table must be int32"),
    (lambda torch: dict(seq_lens=torch.zeros(2, dtype=torch.int64)), {}, "seq_lens must be int32"),
    (lambda torch: dict(v_cache=torch.zeros(20, 2, 16, 128)), {}, "v_cache must match"),
    (lambda torch: dict(k_lowrank=None), {}, "needs k_lowrank and proj"),
    (lambda torch: dict(k_sig=torch.zeros(20, 2, 15, dtype=torch.int32)), {"predictor": vsa.PRED_HASH},
     "k_sig must be"),
    (lambda torch: dict(), {"predictor": vsa.PRED_HASH}, "needs k_sig and proj"),
])
def test_binding_rejects_bad_tensors(over, cfg_kw, msg):
    import torch
    t = _tensors(**over(torch))
    cfg = vsa.Config(**dict(dict(sinks=16, window=16, rank=32), **cfg_kw))
    with pytest.raises(ValueError, match=msg):
        vsa.make_inputs(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["seq_lens"], 160,
                        k_lowrank=t["k_lowrank"], proj=t["proj"], k_sig=t["k_sig"], cfg=cfg)


def test_binding_accepts_good_tensors():
    t = _tensors()
    inp = vsa.make_inputs(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["seq_lens"], 160,
                          k_lowrank=t["k_lowrank"], proj=t["proj"], cfg=vsa.Config(rank=32))
    assert (inp.B, inp.Hq, inp.Hkv, inp.d, inp.max_blocks, inp.num_blocks) == (2, 8, 2, 128, 10, 20)
    with pytest.raises(ValueError, match="shorter than max_seq_len"):
        vsa.make_inputs(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["seq_lens"], 161,
                        k_lowrank=t["k_lowrank"], proj=t["proj"], cfg=vsa.Config(rank=32))


def test_binding_rejects_bad_maintenance_tensors():
    import torch
    t = _tensors()
    B, Hkv, d = 2, 2, 128
    k_new = torch.zeros(B, Hkv, d, dtype=torch.bfloat16)
    pos = torch.zeros(B, dtype=torch.int32)
    with pytest.raises(ValueError, match="k_new must be"):
        vsa.append_kv(k_new.float(), k_new, pos, t["block_table"], t["k_cache"], t["v_cache"])
    with pytest.raises(ValueError, match="pos must be int32"):
        vsa.append_kv(k_new, k_new, pos.long(), t["block_table"], t["k_cache"], t["v_cache"])
    with pytest.raises(ValueError, match="k_lowrank must be"):
        vsa.append_kv(k_new, k_new, pos, t["block_table"], t["k_cache"], t["v_cache"],
                      k_lowrank=torch.zeros(20, 2, 16, 16, dtype=torch.int16), proj=t["proj"])
    with pytest.raises(ValueError, match="k_sig must be"):
        vsa.append_kv_sig(k_new, k_new, pos, t["block_table"], t["k_cache"], t["v_cache"],
                          torch.zeros(20, 2, 16, dtype=torch.int64), t["proj"])
    with pytest.raises(ValueError, match="proj must be"):
        vsa.project_keys(t["k_cache"], torch.zeros(64, 32))
    with pytest.raises(ValueError, match="k_lowrank must be"):
        vsa.project_keys(t["k_cache"], t["proj"], k_lowrank=torch.zeros(20, 2, 16, 16, dtype=torch.int16))
    with pytest.raises(ValueError, match="k_sig must be"):
        vsa.sign_keys(t["k_cache"], t["proj"], k_sig=torch.zeros(20, 2, 16, dtype=torch.int16))
    with pytest.raises(ValueError, match="seq_lens must be int32"):
        vsa.key_gram(t["k_cache"], t["block_table"], t["seq_lens"].long(), 160)


def test_guarantee_field(lib):
    inp = _inputs()
    for bad in (-1, 2):
        assert lib.vattn_workspace_size(C.byref(inp), C.byref(_cfg(guarantee=bad))) == 0
        assert _decode(lib, inp, _cfg(guarantee=bad)) == 4  # VATTN_E_CFG
    den = lib.vattn_workspace_size(C.byref(inp), C.byref(_cfg(guarantee=0)))
    out = lib.vattn_workspace_size(C.byref(inp), C.byref(_cfg(guarantee=1)))
    assert out > den > 0  # the output-level mode's V-row lists and numerator partials
