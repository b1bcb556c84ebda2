"""C-ABI checks that need no GPU: the library loads, exports every entry point
the headers in include/ declare, and rejects bad arguments before launching anything
(no pointer is dereferenced on the host, so fake device addresses are safe)."""
import ctypes as C
import glob
import os
import re

import pytest

import block_drafting_sd_amd as sd
from block_drafting_sd_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

FAKE = 1 << 20        # 16-byte aligned, never dereferenced by validation
ODD = FAKE + 8        # not 16-byte aligned


def _declared():
    txt = "\n".join(open(h).read() for h in HEADERS)
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(sd_[a-z_0-9]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from block_drafting_sd_amd import build
        build.build()
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) >= {"sd_draft_attn", "sd_lm_head_probs", "sd_verify"}
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_status_strings_and_version(lib):
    for s in range(7):
        assert lib.sd_status_str(s)
    assert lib.sd_status_str(99) == b"unknown status"
    assert sd.sd_version() == "0.1.0"


@pytest.mark.parametrize("batch,hkv,total,split", [
    (16, 8, 16 * 131072, 32768),     # 16 x 128K: 512 prefix items of 32K tokens
    (16, 8, 16 * 32768, 8192),       # 16 x 32K: 512 items of 8K (32K would leave 128)
    (64, 8, 64 * 4096, 4096),        # 64 x 4K: at most the mean prefix
    (128, 8, 3_430_000, 16384),      # ragged mix, mean ~26.8K: the mean caps it
    (64, 8, 64 * 3000, 2048),        # mean 3000 < 4096
    (1, 1, 512, 2048),               # tiny: the 2048-token floor
])
def test_automatic_attention_split(lib, batch, hkv, total, split):
    """The automatic split (largest power of two in [2048, 32768] tokens with
    at least 512 prefix items and at most the mean prefix) sizes the
    workspace exactly as the explicit split does, and unlike its neighbours."""
    auto = lib.sd_draft_attn_workspace_size(batch, 4 * hkv, hkv, 128, 16, total, 0)
    assert auto == lib.sd_draft_attn_workspace_size(batch, 4 * hkv, hkv, 128, 16, total, split)
    for other in (split // 2, split * 2):
        if 2048 <= other <= 32768 and total // other != total // split:
            assert auto != lib.sd_draft_attn_workspace_size(batch, 4 * hkv, hkv, 128, 16, total,
                                                             other)


def test_workspace_sizes(lib):
    n = lib.sd_draft_attn_workspace_size(16, 32, 8, 128, 16, 16 * 131072, 0)
    # fp32 partials (64 rows x 128 dims) of every prefix item at the automatic
    # split for 16 x 128K prefixes (32768 tokens)
    assert n > 16 * 131072 // 32768 * 8 * 64 * 128 * 4
    assert lib.sd_draft_attn_workspace_size(0, 32, 8, 128, 16, 1, 0) == 0
    assert lib.sd_draft_attn_workspace_size(1, 32, 8, 128, 0, 1, 0) == 0
    # more than 64 query rows per (request, KV head): items of 128 rows
    n5 = lib.sd_draft_attn_workspace_size(16, 40, 8, 128, 16, 16 * 131072, 0)
    assert n5 > 2 * n - 2 * 4096
    assert lib.sd_lm_head_workspace_size(256, 151936) >= 256 * (-(-151936 // 128)) * 16
    assert lib.sd_lm_head_workspace_size(0, 10) == 0
    assert lib.sd_verify_workspace_size(16, 256, 272, 151936) > 0
    assert lib.sd_verify_workspace_size(16, 256, 0, 151936) == 0


def _attn(lib, **kw):
    a = dict(q=FAKE, k_blk=FAKE, v_blk=FAKE, k_cache=FAKE, v_cache=FAKE, page_table=FAKE,
             ctx_len=FAKE, q_off=FAKE, batch=2, total_q=8, max_draft_k=4, num_pages=10,
             max_pages=5, page_size=16, hq=8, hkv=2, d=128, max_total_ctx=100, split=0,
             scale=0.088, mask=0, window=0, sum_k=None, sum_v=None, n_sum=0, out=FAKE, ws=FAKE,
             ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.sd_draft_attn(a["q"], a["k_blk"], a["v_blk"], a["k_cache"], a["v_cache"],
                             a["page_table"], a["ctx_len"], a["q_off"], a["batch"],
                             a["total_q"], a["max_draft_k"], a["num_pages"], a["max_pages"],
                             a["page_size"], a["hq"], a["hkv"], a["d"], a["max_total_ctx"],
                             a["split"], a["scale"], a["mask"], a["window"], a["sum_k"],
                             a["sum_v"], a["n_sum"], a["out"], a["ws"], a["ws_bytes"],
                             a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(page_table=None), 1), (dict(out=None), 1),
    (dict(batch=0), 2), (dict(page_size=32), 2), (dict(d=96), 2), (dict(hq=6, hkv=4), 2),
    (dict(max_draft_k=33), 2),            # group 4 * 33 > 128 query rows
    (dict(hq=16, hkv=2, max_draft_k=17), 2),   # group 8 * 17 > 128
    (dict(split=100), 2), (dict(scale=float("inf")), 2), (dict(scale=0.0), 2), (dict(q=ODD), 2),
    (dict(mask=2), 2), (dict(window=-1), 2), (dict(n_sum=65, sum_k=FAKE, sum_v=FAKE), 2),
    (dict(n_sum=16), 1), (dict(n_sum=16, sum_k=FAKE), 1), (dict(n_sum=16, sum_k=ODD, sum_v=FAKE), 2),
    (dict(ws=None), 3), (dict(ws_bytes=10), 3),
    (dict(total_q=0), 0),                 # nothing to do: returns before launching
    (dict(total_q=0, mask=1, window=256, n_sum=16, sum_k=FAKE, sum_v=FAKE), 0),
])
def test_draft_attn_validation(lib, kw, status):
    assert _attn(lib, **kw) == status


def test_noalloc_rejects_before_any_device_call(lib):
    """The no-allocation attention validates like sd_draft_attn and refuses a
    call whose scratch exceeds its fixed array, all before it touches a
    device (so these run without a GPU)."""
    cap = lib.sd_draft_attn_noalloc_max_scratch()
    assert cap == 128 << 20
    def call(**kw):
        a = dict(q=FAKE, batch=2, total_q=8, max_draft_k=4, hq=8, hkv=2, max_total_ctx=100)
        a.update(kw)
        return lib.sd_draft_attn_noalloc(a["q"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                         a["batch"], a["total_q"], a["max_draft_k"], 10, 5, 16,
                                         a["hq"], a["hkv"], 128, a["max_total_ctx"], 0, 0.088,
                                         0, 0, None, None, 0, FAKE, None)
    assert call(q=None) == 1
    assert call(max_draft_k=33) == 2
    # 16 x 2M tokens of prefix need far more partials than the array holds
    big = 16 * (1 << 21)
    assert lib.sd_draft_attn_workspace_size(16, 32, 8, 128, 16, big, 0) > cap
    assert call(batch=16, hq=32, hkv=8, max_draft_k=16, max_total_ctx=big) == 6
    assert lib.sd_status_str(6).startswith(b"the call needs more scratch")


def _sum(lib, **kw):
    a = dict(u=FAKE, k_cache=FAKE, v_cache=FAKE, page_table=FAKE, ctx_len=FAKE, acc=FAKE,
             batch=2, num_pages=10, max_pages=5, page_size=16, hkv=2, d=128, n_sum=16,
             scale=0.088, z=FAKE, c=FAKE, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return lib.sd_summary_update(a["u"], a["k_cache"], a["v_cache"], a["page_table"],
                                 a["ctx_len"], a["acc"], a["batch"], a["num_pages"],
                                 a["max_pages"], a["page_size"], a["hkv"], a["d"], a["n_sum"],
                                 a["scale"], a["z"], a["c"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(u=None), 1), (dict(z=None), 1), (dict(c=None), 1), (dict(ctx_len=None), 1),
    (dict(batch=0), 2), (dict(d=96), 2), (dict(n_sum=0), 2), (dict(n_sum=65), 2),
    (dict(page_size=8), 2), (dict(scale=-1.0), 2), (dict(k_cache=ODD), 2), (dict(u=ODD), 2),
    # an initialisation needs the workspace
    (dict(acc=None, ws=None), 3), (dict(acc=None, ws_bytes=16), 3), (dict(acc=None, ws=ODD), 3),
])
def test_summary_update_validation(lib, kw, status):
    assert _sum(lib, **kw) == status


def test_summary_workspace_size(lib):
    """A fold needs no workspace; an initialisation keeps a (max, sum,
    S x D values) fp32 partial state per slot: 1,024 waves walk the
    concatenated (request, KV head) rows and the piece of pair p that wave w
    covers goes to slot p + w, so 1,024 + B * Hkv slots, each array rounded
    up to 256 bytes."""
    size = lib.sd_summary_workspace_size

    def expect(batch, hkv, s, d):
        parts = (1024 + batch * hkv) * s
        return -(-parts * 8 // 256) * 256 + -(-parts * d * 4 // 256) * 256

    for args in ((2, 2, 16, 128, 5), (16, 8, 16, 128, 8192), (128, 8, 16, 128, 8192),
                 (3, 1, 5, 64, 100)):
        assert size(*args, 16) == expect(*args[:4])
    assert size(0, 2, 16, 128, 4096, 16) == 0 and size(2, 2, 16, 128, 4096, 8) == 0


def _lm(lib, **kw):
    a = dict(hidden=FAKE, w=FAKE, M=16, H=256, V=1024, q_off=FAKE, batch=1, req=FAKE, seed=1,
             vmap=None, w_rows=0, greedy=0, logits=FAKE, lse=FAKE, tok=FAKE, ws=FAKE,
             ws_bytes=1 << 40)
    a.update(kw)
    return lib.sd_lm_head_probs(a["hidden"], a["w"], a["M"], a["H"], a["V"], a["q_off"],
                                a["batch"], a["req"], a["seed"], a["vmap"], a["w_rows"],
                                a["greedy"], a["logits"], a["lse"], a["tok"], a["ws"],
                                a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=None), 1), (dict(req=None), 1), (dict(tok=None), 1),
    (dict(M=0), 2), (dict(H=100), 2), (dict(H=0), 2), (dict(V=0), 2), (dict(logits=ODD), 2),
    (dict(greedy=2), 2), (dict(vmap=FAKE, w_rows=0), 2),
    (dict(ws=None), 3), (dict(ws_bytes=1), 3),
])
def test_lm_head_validation(lib, kw, status):
    assert _lm(lib, **kw) == status


def _vf(lib, **kw):
    a = dict(target=FAKE, t_off=FAKE, draft=FAKE, lse=None, tok=FAKE, q_off=FAKE, batch=2,
             total_q=8, R=10, V=1024, vinv=None, v_draft=0, greedy=0, req=FAKE, seed=3,
             acc=FAKE, nxt=FAKE, ratio=None, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return lib.sd_verify(a["target"], a["t_off"], a["draft"], a["lse"], a["tok"], a["q_off"],
                         a["batch"], a["total_q"], a["R"], a["V"], a["vinv"], a["v_draft"],
                         a["greedy"], a["req"], a["seed"], a["acc"], a["nxt"], a["ratio"],
                         a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(target=None), 1), (dict(acc=None), 1), (dict(draft=None), 1),
    (dict(batch=0), 2), (dict(R=0), 2), (dict(V=0), 2),
    (dict(greedy=-1), 2), (dict(vinv=FAKE, v_draft=100), 1),        # pruned needs draft_lse
    (dict(vinv=FAKE, v_draft=0, lse=FAKE), 2),
    (dict(ws=None), 3), (dict(ws_bytes=5), 3),
])
def test_verify_validation(lib, kw, status):
    assert _vf(lib, **kw) == status


def test_python_binding_rejects_cpu_dtype_mismatch():
    import torch
    x = torch.zeros(4, 4, dtype=torch.float32)
    with pytest.raises(TypeError):
        sd.sd_lm_head_probs(x, x, torch.zeros(2, dtype=torch.int32),
                            torch.zeros(1, dtype=torch.int32), 0)


def _sch(lib, **kw):
    a = dict(c=FAKE, e=FAKE, wc=FAKE, we=FAKE, bu=None, wo=FAKE, bo=None, cs=None, cb=None,
             n=4, dh=64, r=32, K=6, dcap=FAKE, dlat=FAKE, ndb=3, vcap=FAKE, vlat=FAKE, nvb=2,
             N=4, logits=FAKE, scores=FAKE, dlen=FAKE, qoff=None, budget=FAKE, obj=None, ws=FAKE,
             ws_bytes=1 << 40)
    a.update(kw)
    return lib.sd_schedule_draft(a["c"], a["e"], a["wc"], a["we"], a["bu"], a["wo"], a["bo"],
                                 a["cs"], a["cb"], a["n"], a["dh"], a["r"], a["K"], a["dcap"],
                                 a["dlat"], a["ndb"], a["vcap"], a["vlat"], a["nvb"], a["N"],
                                 a["logits"], a["scores"], a["dlen"], a["qoff"], a["budget"],
                                 a["obj"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(c=None), 1), (dict(wo=None), 1), (dict(dcap=None), 1), (dict(budget=None), 1),
    (dict(n=0), 2), (dict(n=1025), 2), (dict(K=0), 2), (dict(K=33), 2),
    (dict(n=200, K=32), 2),               # n K > 4096 entries
    (dict(dh=40), 2), (dict(r=8), 2), (dict(ndb=0), 2), (dict(N=-1), 2), (dict(c=ODD), 2),
    (dict(ws=None), 3), (dict(ws_bytes=8), 3),
])
def test_schedule_draft_validation(lib, kw, status):
    assert _sch(lib, **kw) == status


def _schv(lib, **kw):
    a = dict(h=FAKE, ws_=FAKE, ep=FAKE, w=FAKE, bias=1.0, temp=None, anchor=FAKE, tok=FAKE,
             qoff=FAKE, budget=FAKE, n=4, rows=24, H=64, m=16, V=100, K=6, p=FAKE, s=FAKE,
             vlen=FAKE, toff=None, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return lib.sd_schedule_verify(a["h"], a["ws_"], a["ep"], a["w"], a["bias"], a["temp"],
                                  a["anchor"], a["tok"], a["qoff"], a["budget"], a["n"],
                                  a["rows"], a["H"], a["m"], a["V"], a["K"], a["p"], a["s"],
                                  a["vlen"], a["toff"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(h=None), 1), (dict(qoff=None), 1), (dict(budget=None), 1), (dict(vlen=None), 1),
    (dict(n=0), 2), (dict(rows=0), 2), (dict(rows=4097), 2), (dict(H=40), 2), (dict(m=8), 2),
    (dict(V=0), 2), (dict(K=33), 2), (dict(bias=float("nan")), 2), (dict(h=ODD), 2),
    (dict(ws=None), 3), (dict(ws_bytes=8), 3),
])
def test_schedule_verify_validation(lib, kw, status):
    assert _schv(lib, **kw) == status


def _mk(lib, **kw):
    a = dict(z=FAKE, lse=FAKE, tok=FAKE, anchor=FAKE, wc=FAKE, ec=FAKE, alpha=1.0, bias=None,
             greedy=0, qoff=FAKE, batch=2, M=8, V=1000, r=32, k=4, req=FAKE, seed=5, ws=FAKE,
             ws_bytes=1 << 40)
    a.update(kw)
    return lib.sd_markov_sample(a["z"], a["lse"], a["tok"], a["anchor"], a["wc"], a["ec"],
                                a["alpha"], a["bias"], a["greedy"], a["qoff"], a["batch"], a["M"],
                                a["V"], a["r"], a["k"], a["req"], a["seed"], a["ws"], a["ws_bytes"],
                                None)


@pytest.mark.parametrize("kw,status", [
    (dict(z=None), 1), (dict(anchor=None), 1), (dict(wc=None), 1), (dict(req=None), 1),
    (dict(batch=0), 2), (dict(M=-1), 2), (dict(V=0), 2), (dict(r=0), 2), (dict(r=24), 2),
    (dict(k=-1), 2), (dict(k=5000), 2), (dict(wc=ODD), 2), (dict(ec=ODD), 2),
    (dict(alpha=float("inf")), 2), (dict(alpha=float("nan")), 2), (dict(greedy=2), 2),
    (dict(ws=None), 3), (dict(ws_bytes=16), 3), (dict(ws=ODD), 3),
    (dict(M=0), 0), (dict(k=0), 0), (dict(k=0, ws=None), 0),          # nothing to launch
])
def test_markov_validation(lib, kw, status):
    assert _mk(lib, **kw) == status


def test_markov_workspace_size(lib):
    # (max, sum exp) per workgroup and a 64-bit draw cell per (position, request)
    assert lib.sd_markov_workspace_size(16, 151936, 16) >= 16 * 16 * (512 * 8 + 8)
    assert lib.sd_markov_workspace_size(3, 1000, 5) >= 3 * 5 * (8 * 8 + 8)
    assert lib.sd_markov_workspace_size(0, 10, 1) == 0
    assert lib.sd_markov_workspace_size(1, 10, 0) == 0


@pytest.mark.parametrize("args,status", [
    ((None, 10, 1.0, -0.3, FAKE), 1), ((FAKE, 10, 1.0, -0.3, None), 1),
    ((FAKE, 0, 1.0, -0.3, FAKE), 2), ((FAKE, 10, 0.0, -0.3, FAKE), 2),
    ((FAKE, 10, float("nan"), -0.3, FAKE), 2), ((FAKE, 10, 1.0, float("inf"), FAKE), 2),
])
def test_log_prior_bias_validation(lib, args, status):
    assert lib.sd_log_prior_bias(*args, None) == status


def test_probe_validation(lib):
    assert lib.sd_probe_read(None, 64, FAKE, None) == 1
    assert lib.sd_probe_read(FAKE, 64, None, None) == 1
    assert lib.sd_probe_read(FAKE, 8, FAKE, None) == 2
    assert lib.sd_probe_read(ODD, 64, FAKE, None) == 2
    assert lib.sd_probe_mfma(0, FAKE, None) == 2
    assert lib.sd_probe_mfma(10, None, None) == 1
    assert lib.sd_probe_mfma_flops(1) == 512 * 4 * 8 * 2 * 32 * 32 * 16
    assert lib.sd_probe_mfma_flops(0) == 0


def test_python_binding_checks_array_lengths():
    # device arrays are never read on the host: the binding checks lengths
    import torch
    bf, i32 = torch.bfloat16, torch.int32
    z = torch.zeros(8, 100)
    w = torch.zeros(100, 16, dtype=bf)
    q_off = torch.tensor([0, 4, 8], dtype=i32)
    with pytest.raises(ValueError, match="anchor_tokens"):
        sd.sd_markov_sample(z, torch.zeros(1, dtype=i32), w, w, q_off, torch.zeros(2, dtype=i32),
                            1, max_draft_k=4)
    with pytest.raises(ValueError, match="req_id"):
        sd.sd_markov_sample(z, torch.zeros(2, dtype=i32), w, w, q_off, torch.zeros(1, dtype=i32),
                            1, max_draft_k=4)
    h = torch.zeros(8, 64, dtype=bf)
    wv = torch.zeros(100, 64, dtype=bf)
    with pytest.raises(ValueError, match="req_id"):
        sd.sd_lm_head_probs(h, wv, q_off, torch.zeros(1, dtype=i32), 0)
    with pytest.raises(ValueError, match="lse"):
        sd.sd_lm_head_probs(h, wv, q_off, torch.zeros(2, dtype=i32), 0, lse=torch.zeros(3))


def test_python_binding_checks_verify_draft_rows():
    # without a vocabulary map the library reads draft rows with the target's
    # row length, so shorter or longer rows must be refused before the call
    import torch
    i32 = torch.int32
    tl = torch.zeros(3, 100)
    t_off = torch.tensor([0, 3], dtype=i32)
    q_off = torch.tensor([0, 2], dtype=i32)
    tok = torch.zeros(2, dtype=i32)
    rid = torch.zeros(1, dtype=i32)
    with pytest.raises(ValueError, match="V = 100"):
        sd.sd_verify(tl, t_off, torch.zeros(2, 320), None, tok, q_off, rid, 0)
    with pytest.raises(ValueError, match="V = 100"):
        sd.sd_verify(tl, t_off, torch.zeros(2, 50), torch.zeros(2), tok, q_off, rid, 0)
    with pytest.raises(ValueError, match="draft_lse"):
        sd.sd_verify(tl, t_off, torch.zeros(2, 50), None, tok, q_off, rid, 0,
                     draft_vocab_inv=torch.full((100,), -1, dtype=i32))
    with pytest.raises(ValueError, match="draft_lse"):
        sd.sd_verify(tl, t_off, torch.zeros(2, 50), torch.zeros(1), tok, q_off, rid, 0,
                     draft_vocab_inv=torch.full((100,), -1, dtype=i32))
    with pytest.raises(ValueError, match="total_q"):
        sd.sd_verify(tl, t_off, torch.zeros(200), None, tok, q_off, rid, 0)


def test_bench_refuses_several_gpus():
    import json
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]
