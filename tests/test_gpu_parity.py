"""GPU parity: the HIP path against the fp64 oracle, element by element.

Tolerances (stated for bf16 inputs): max |O - O_ref| <= 2e-2 and
max |lse - lse_ref| <= 1e-3; the same bar is applied to the fp32-input path.
Rows where both lse values are -inf agree.
"""
import math
import sys

import numpy as np
import pytest
import torch

import attention_forward_attn_amd as A
import oracle
import synth

pytestmark = pytest.mark.gpu

TOL_O = 2e-2
TOL_LSE = 1e-3


def announce(msg):
    sys.stderr.write(f"[gpu-case] {msg}\n")
    sys.stderr.flush()


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _lse_err(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        d = np.where(same_inf, 0.0, np.abs(a - b))
    return float(np.nan_to_num(d, nan=np.inf).max()) if d.size else 0.0


def _o_err(a, b):
    d = np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))
    return float(np.nan_to_num(d, nan=np.inf).max()) if d.size else 0.0


def run_dense(inp, *, causal, scale, poison=True, stream=None):
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    sk = inp["sinks"].cuda() if inp["sinks"] is not None else None
    B, H, Tq, _ = q.shape
    out = torch.full((B, H, Tq, v.shape[-1]), float("nan"), dtype=q.dtype, device="cuda")
    lse = torch.full((B, H, Tq), float("nan"), dtype=torch.float32, device="cuda")
    A.dense(q, k, v, causal=causal, scale=scale, sinks=sk, out=out, lse=lse, stream=stream)
    torch.cuda.synchronize()
    return out, lse


def check_dense_full(inp, *, causal, scale, label):
    announce(f"dense {label} q{tuple(inp['q'].shape)} k{tuple(inp['k'].shape)} v{tuple(inp['v'].shape)} "
             f"causal={causal} sinks={inp['sinks'] is not None}")
    out, lse = run_dense(inp, causal=causal, scale=scale)
    ro, rl = oracle.dense_attention(inp["q"], inp["k"], inp["v"], scale=scale, causal=causal,
                                    sinks=inp["sinks"])
    eo, el = _o_err(_np(out), ro), _lse_err(_np(lse), rl)
    assert eo <= TOL_O and el <= TOL_LSE, f"{label}: max|dO|={eo:.3e} max|dlse|={el:.3e}"
    return eo, el


# ------------------------------------------------------------------ small shapes, full outputs
HEAD_DIMS = [(64, 64), (128, 128), (192, 128), (256, 256), (512, 512)]


@pytest.mark.parametrize("dqk,dv", HEAD_DIMS)
@pytest.mark.parametrize("causal", [True, False])
def test_dense_bf16_head_dims(dqk, dv, causal):
    # T = 200: several 64/128-row tiles and several key blocks, ragged in both
    inp = synth.randn_dense(2, 4, 2, 200, 200, dqk, dv, dtype="bf16", sinks=False, seed=dqk + dv)
    check_dense_full(inp, causal=causal, scale=1 / math.sqrt(dqk), label=f"bf16 d{dqk}/{dv}")


@pytest.mark.parametrize("dqk,dv", HEAD_DIMS)
def test_dense_bf16_sinks(dqk, dv):
    inp = synth.randn_dense(1, 8, 2, 150, 150, dqk, dv, dtype="bf16", sinks=True, seed=7 + dqk)
    check_dense_full(inp, causal=True, scale=1 / math.sqrt(dqk), label=f"sinks d{dqk}")


@pytest.mark.parametrize("Tk", [1, 32, 33, 65, 97, 129])
@pytest.mark.parametrize("causal", [True, False])
def test_dense_d512_few_key_blocks(Tk, causal):
    """The 512-wide kernel keeps up to two K blocks and one V block in flight ahead of
    the block it reads: one to five 32-key blocks, whole and ragged, cover its prologue
    and the steps where fewer loads are pending."""
    inp = synth.randn_dense(1, 16, 1, 40, Tk, 512, 512, dtype="bf16", sinks=True, seed=900 + Tk)
    check_dense_full(inp, causal=causal, scale=1 / math.sqrt(512), label=f"d512 Tk{Tk}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_dense_f32_split(d, causal):
    inp = synth.randn_dense(1, 4, 1, 150, 150, d, d, dtype="f32", seed=11 + d)
    check_dense_full(inp, causal=causal, scale=1 / math.sqrt(d), label=f"f32 d{d}")


@pytest.mark.parametrize("g,Hkv,T", [(1, 3, 70), (4, 2, 5), (8, 1, 17), (64, 1, 3), (16, 2, 1)])
def test_gqa_fold_packed_rows(g, Hkv, T):
    """Small Tq: rows of several heads share one workgroup tile (folded view)."""
    inp = synth.randn_dense(2, g * Hkv, Hkv, T, T, 128, 128, dtype="bf16", sinks=True, seed=100 + g)
    check_dense_full(inp, causal=True, scale=1 / math.sqrt(128), label=f"fold g{g}")


@pytest.mark.parametrize("Tq,Tk", [(1, 300), (37, 300), (300, 37), (130, 129), (64, 64)])
@pytest.mark.parametrize("sinks", [False, True])
def test_causal_bottom_right_unequal_lengths(Tq, Tk, sinks):
    inp = synth.randn_dense(1, 8, 2, Tq, Tk, 128, 128, dtype="bf16", sinks=sinks, seed=Tq * 1000 + Tk)
    check_dense_full(inp, causal=True, scale=1 / math.sqrt(128), label=f"Tq{Tq} Tk{Tk}")


@pytest.mark.parametrize("sinks", [False, True])
def test_no_keys(sinks):
    inp = synth.randn_dense(1, 4, 2, 9, 0, 64, 64, dtype="bf16", sinks=sinks, seed=5)
    announce(f"dense Tk=0 sinks={sinks}")
    out, lse = run_dense(inp, causal=False, scale=0.125)
    assert torch.all(out.float() == 0)
    if sinks:
        assert torch.allclose(lse.cpu(), inp["sinks"].repeat_interleave(1).view(1, 4, 1).expand(1, 4, 9))
    else:
        assert torch.all(torch.isneginf(lse))


def test_no_queries_launches_nothing():
    inp = synth.randn_dense(1, 4, 2, 0, 16, 64, 64, dtype="bf16", seed=6)
    announce("dense Tq=0")
    A.reset_dispatch_counts()
    out, lse = A.dense(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), causal=True)
    torch.cuda.synchronize()
    assert out.numel() == 0 and lse.numel() == 0
    assert A.dispatch_count("dense_bf16_d64") == 0


def test_strided_bshd_view():
    """A BSHD tensor passed as a strided BHSD view gives the same result."""
    inp = synth.randn_dense(2, 8, 2, 96, 96, 128, 128, dtype="bf16", seed=21)
    announce("dense strided BSHD view")
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    qs, ks, vs = (x.transpose(1, 2).contiguous().transpose(1, 2) for x in (q, k, v))
    assert qs.stride(-1) == 1 and not qs.is_contiguous()
    o1, l1 = A.dense(q, k, v, causal=True)
    o2, l2 = A.dense(qs, ks, vs, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_streams_default_and_side():
    """The legacy NULL stream and a side stream both work (stream 0 is valid)."""
    inp = synth.randn_dense(1, 4, 1, 128, 128, 64, 64, dtype="bf16", seed=31)
    announce("dense on NULL stream and on a side stream")
    o0, l0 = run_dense(inp, causal=True, scale=0.125, stream=torch.cuda.default_stream())
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o1, l1 = run_dense(inp, causal=True, scale=0.125, stream=s)
    s.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


# ------------------------------------------------------------------ sparse, small
@pytest.mark.parametrize("Hq,sinks", [(64, False), (64, True), (16, False)])
def test_sparse_small(Hq, sinks):
    Sq, N, topk = 7, 300, 100
    inp = synth.randn_sparse(Sq, Hq, N, 512, topk, seed=40 + Hq, sinks=sinks)
    idx = inp["idx"].clone()
    idx[0, 5] = -1           # skipped
    idx[1, 0] = N + 5        # out of range: skipped
    idx[2, 7] = idx[2, 8]    # duplicate: counted twice
    idx[3, :] = -1           # a query with no valid key
    announce(f"sparse Sq={Sq} Hq={Hq} N={N} topk={topk} sinks={sinks}")
    q, kv, ix = inp["q"].cuda(), inp["kv"].cuda(), idx.cuda()
    sk = inp["sinks"].cuda() if sinks else None
    out, lse = A.sparse_topk(q, kv, ix, d_v=512, sinks=sk)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_topk_attention(inp["q"], inp["kv"], idx, d_v=512, scale=1 / math.sqrt(512),
                                          sinks=inp["sinks"])
    eo, el = _o_err(_np(out), ro), _lse_err(_np(lse), rl)
    assert eo <= TOL_O and el <= TOL_LSE, f"sparse: max|dO|={eo:.3e} max|dlse|={el:.3e}"


# ------------------------------------------------------------------ the five workloads
def _sample_rows(B, H, Tq, rng, n_rand=24):
    ts = sorted({0, 1, 2, 31, 32, 63, 64, 127, 128, 129, Tq // 2, Tq - 129, Tq - 2, Tq - 1}
                | set(rng.integers(0, Tq, n_rand).tolist()))
    ts = [t for t in ts if 0 <= t < Tq]
    hs = sorted({0, H - 1, H // 2} | set(rng.integers(0, H, 3).tolist()))
    return [(b, h, t) for b in range(B) for h in hs for t in ts]


def test_workload_tiny_full():
    s = synth.spec(1)
    inp = synth.make(1)
    check_dense_full(inp, causal=True, scale=s.scale, label="tiny (fp32, B1 H4 Hkv1 T128 d64)")


@pytest.mark.parametrize("n", [2, 3, 4])
def test_workload_dense_full(n):
    """The benchmark's launch of workload n (same planner, same kernel, same tile
    order) compared with the oracle on every output element."""
    s = synth.spec(n)
    inp = synth.make(n)
    announce(f"workload {s.name}: B{s.B} H{s.H} Hkv{s.Hkv} T{s.Tq} d{s.d_qk}/{s.d_v} sinks={s.sinks}")
    A.reset_dispatch_counts()
    out, lse = run_dense(inp, causal=True, scale=s.scale)
    path = A.plan_dense(s.B, s.H, s.Hkv, s.Tq, s.Tk, s.d_qk, s.d_v, sinks=s.sinks)["path"]
    assert A.dispatch_count(path) == 1
    # every element written (outputs were poisoned with NaN)
    assert not torch.isnan(out).any().item() and not torch.isnan(lse).any().item()
    # run-to-run bitwise determinism
    out2, lse2 = run_dense(inp, causal=True, scale=s.scale)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    del out2, lse2
    ro, rl = oracle.dense_attention(inp["q"], inp["k"], inp["v"], scale=s.scale, causal=True, sinks=inp["sinks"])
    go, gl = _np(out), _np(lse)
    eo, el = _o_err(go, ro), _lse_err(gl, rl)
    where = np.unravel_index(int(np.argmax(np.abs(go - ro))), go.shape)
    announce(f"workload {s.name}: all {go.size} outputs, max|dO|={eo:.3e} at {tuple(int(x) for x in where)} "
             f"max|dlse|={el:.3e}")
    assert eo <= TOL_O and el <= TOL_LSE


def test_fold_with_xcd_order_full():
    """Token-major GQA fold (g = 4) with the XCD-chunked tile order (B*Hkv = 16, a
    multiple of 8): the combination the gqa workload launches, at a size whose
    every output the oracle checks."""
    inp = synth.randn_dense(2, 32, 8, 512, 512, 128, 128, dtype="bf16", seed=2512)
    p = A.plan_dense(2, 32, 8, 512, 512, 128, 128)
    assert p["fold_g"] == 4 and p["path"] == "dense_bf16_d128"
    check_dense_full(inp, causal=True, scale=1 / math.sqrt(128), label="fold g4 + xcd order, B2 H32/8 T512")


@pytest.mark.parametrize("B,H,Hkv,T,dqk,dv", [(1, 8, 8, 700, 192, 128), (2, 64, 8, 300, 64, 64),
                                              (4, 8, 4, 257, 256, 256)])
def test_xcd_order_other_dims_full(B, H, Hkv, T, dqk, dv):
    """XCD-chunked order (B*Hkv a multiple of 8) on the other kernels: one head per kv head
    (row blocks aligned to heads) and folded groups."""
    inp = synth.randn_dense(B, H, Hkv, T, T, dqk, dv, dtype="bf16", sinks=True, seed=B * H + T)
    check_dense_full(inp, causal=True, scale=1 / math.sqrt(dqk), label=f"xcd order B{B} H{H}/{Hkv} d{dqk}")


def test_workload_sparse_queries():
    """The benchmark's sparse launch at full size; 1024 of its 13312 queries (the
    first and last 256 and 512 more drawn at random) against the oracle."""
    s = synth.spec(5)
    inp = synth.make(5)
    announce(f"workload sparse: Sq{s.Sq} Hq{s.Hq} N{s.N} d{s.d_qk} topk{s.topk}")
    q, kv, ix = inp["q"].cuda(), inp["kv"].cuda(), inp["idx"].cuda()
    out = torch.full((s.Sq, s.Hq, s.d_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((s.Sq, s.Hq), float("nan"), dtype=torch.float32, device="cuda")
    A.reset_dispatch_counts()
    A.sparse_topk(q, kv, ix, d_v=s.d_v, scale=s.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    assert A.dispatch_count("sparse_bf16_d512") == 1 and A.dispatch_count("dense_bf16_d512") == 0
    assert not torch.isnan(out).any().item() and not torch.isnan(lse).any().item()
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    A.sparse_topk(q, kv, ix, d_v=s.d_v, scale=s.scale, out=out2, lse=lse2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    del out2, lse2
    rng = np.random.default_rng(5)
    middle = rng.choice(np.arange(256, s.Sq - 256), 512, replace=False).tolist()
    qs = sorted(set(range(256)) | set(range(s.Sq - 256, s.Sq)) | set(middle))
    assert len(qs) == 1024
    ro, rl = oracle.sparse_topk_attention(inp["q"], inp["kv"], inp["idx"], d_v=s.d_v, scale=s.scale,
                                          queries=qs)
    go, gl = _np(out[qs]), _np(lse[qs])
    eo, el = _o_err(go, ro), _lse_err(gl, rl)
    announce(f"workload sparse: {len(qs)} queries, max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= TOL_O and el <= TOL_LSE


@pytest.mark.parametrize("topk", [4096, 4097, 9000])
def test_sparse_index_segments(topk):
    """Index lists longer than the kernel's LDS index buffer (4096 entries) are
    read in segments: exactly one segment, one entry more, and three segments."""
    inp = synth.randn_sparse(3, 64, 12000, 512, topk, seed=topk)
    idx = inp["idx"].clone()
    idx[0, 4096 % topk] = -1     # a skipped entry in the second segment (or the first)
    idx[1, topk - 1] = idx[1, 0]  # a duplicate across segments
    announce(f"sparse segments topk={topk}")
    out, lse = A.sparse_topk(inp["q"].cuda(), inp["kv"].cuda(), idx.cuda(), d_v=512)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_topk_attention(inp["q"], inp["kv"], idx, d_v=512, scale=1 / math.sqrt(512))
    eo, el = _o_err(_np(out), ro), _lse_err(_np(lse), rl)
    assert eo <= TOL_O and el <= TOL_LSE, f"topk {topk}: max|dO|={eo:.3e} max|dlse|={el:.3e}"


# ------------------------------------------------------------------ seeded random sweeps
def _sweep_cases(n, seed):
    """Shapes drawn at random (seeded): head dims, GQA group, lengths with
    ragged tails on every tile size, causal and sink switches."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dqk, dv = HEAD_DIMS[i % len(HEAD_DIMS)]
        Hkv = int(rng.integers(1, 3))
        g = int(rng.choice([1, 2, 4, 8]))
        Tq = int(rng.integers(1, 300))
        Tk = Tq if rng.random() < 0.5 else int(rng.integers(1, 300))
        cases.append(dict(B=int(rng.integers(1, 3)), H=g * Hkv, Hkv=Hkv, Tq=Tq, Tk=Tk, dqk=int(dqk), dv=int(dv),
                          causal=bool(rng.random() < 0.7), sinks=bool(rng.random() < 0.3), seed=1000 * seed + i))
    return cases


@pytest.mark.parametrize("case", _sweep_cases(12, 7), ids=lambda c: (
    f"B{c['B']}H{c['H']}/{c['Hkv']}T{c['Tq']}x{c['Tk']}d{c['dqk']}/{c['dv']}"
    f"{'c' if c['causal'] else 'n'}{'s' if c['sinks'] else ''}"))
def test_dense_random_sweep(case):
    c = case
    inp = synth.randn_dense(c["B"], c["H"], c["Hkv"], c["Tq"], c["Tk"], c["dqk"], c["dv"], dtype="bf16",
                            sinks=c["sinks"], seed=c["seed"])
    check_dense_full(inp, causal=c["causal"], scale=1 / math.sqrt(c["dqk"]), label=f"sweep {c}")


@pytest.mark.parametrize("seed", [3, 4, 5, 6])
def test_sparse_random_sweep(seed):
    rng = np.random.default_rng(seed)
    Sq, Hq = int(rng.integers(1, 6)), int(rng.choice([8, 16, 32, 64]))
    N, topk = int(rng.integers(64, 400)), int(rng.integers(1, 300))
    sinks = bool(rng.random() < 0.5)
    inp = synth.randn_sparse(Sq, Hq, N, 512, min(topk, N), seed=500 + seed, sinks=sinks)
    idx = inp["idx"].clone()
    # a few skipped (-1) and out-of-range entries at random positions
    flat = idx.view(-1)
    pos = torch.from_numpy(rng.choice(flat.numel(), size=min(5, flat.numel()), replace=False))
    flat[pos[: len(pos) // 2]] = -1
    flat[pos[len(pos) // 2:]] = N + 7
    announce(f"sparse sweep Sq={Sq} Hq={Hq} N={N} topk={idx.shape[1]} sinks={sinks}")
    sk = inp["sinks"].cuda() if sinks else None
    out, lse = A.sparse_topk(inp["q"].cuda(), inp["kv"].cuda(), idx.cuda(), d_v=512, sinks=sk)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_topk_attention(inp["q"], inp["kv"], idx, d_v=512, scale=1 / math.sqrt(512),
                                          sinks=inp["sinks"])
    eo, el = _o_err(_np(out), ro), _lse_err(_np(lse), rl)
    assert eo <= TOL_O and el <= TOL_LSE, f"sparse sweep: max|dO|={eo:.3e} max|dlse|={el:.3e}"


@pytest.mark.parametrize("d_v,Hq,topk,sinks", [(128, 64, 500, False), (256, 64, 500, True), (384, 64, 500, True),
                                               (256, 16, 5000, False), (384, 64, 97, False)])
def test_sparse_value_prefix(d_v, Hq, topk, sinks):
    """V = the first d_v columns of each gathered 512-wide pool row (d_v < d_qk): the
    kernel path of that width runs and matches the oracle's prefix reading."""
    Sq, N = 5, 6000
    inp = synth.randn_sparse(Sq, Hq, N, 512, topk, seed=d_v + topk, sinks=sinks)
    idx = inp["idx"].clone()
    idx[0, 3] = -1
    idx[1, topk - 1] = N + 1
    idx[2, 1] = idx[2, 0]
    announce(f"sparse value prefix d_v={d_v} Hq={Hq} topk={topk} sinks={sinks}")
    A.reset_dispatch_counts()
    out, lse = A.sparse_topk(inp["q"].cuda(), inp["kv"].cuda(), idx.cuda(), d_v=d_v,
                             sinks=inp["sinks"].cuda() if sinks else None)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (Sq, Hq, d_v)
    assert A.dispatch_count(f"sparse_bf16_d512_v{d_v}") == 1 and A.dispatch_count("sparse_bf16_d512") == 0
    ro, rl = oracle.sparse_topk_attention(inp["q"], inp["kv"], idx, d_v=d_v, scale=1 / math.sqrt(512),
                                          sinks=inp["sinks"])
    eo, el = _o_err(_np(out), ro), _lse_err(_np(lse), rl)
    assert eo <= TOL_O and el <= TOL_LSE, f"d_v {d_v}: max|dO|={eo:.3e} max|dlse|={el:.3e}"
