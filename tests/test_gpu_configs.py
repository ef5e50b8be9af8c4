"""GPU parity at the five workloads' full sizes, in the launch configuration the benchmark times.

The fp64 oracle cannot redo every full-size workload within a test, so each
one is checked on outputs the oracle computes one by one (sampled rows, heads,
keys or (batch, head) pairs), plus properties that hold at any size and are
checked on every head:

* a causal self-attention row 0 sees only key 0: O_0 = v_0 exactly and
  LSE_0 = c q_0 . k_0;
* softmax rows sum to one, so sum_j dV_j = sum of dO over rows that see a key,
  and the shift invariance of softmax gives sum_j dK_j = 0.

Bounds (absolute): O 1e-2, dQ/dK/dV 2e-2, LSE 1e-3.  At long context the
outputs are small (|O| ~ 1e-2), so an all-zero output would pass the absolute
bounds: the LSE bound, the relative Frobenius error (< 1e-2 for O, < 2e-2 for
gradients) and the sum rules are the discriminating checks.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_blockwise_attention_attn_amd import binding as B
from exact_blockwise_attention_attn_amd import shard
from seeded_inputs import TREE_DECODE, VARLEN_PACKED, WORKLOADS, bf16_bits_to_f32, normal_bf16, normal_f32, tree_nodes
from tests.gpu_util import check, log, rel_fro, row0_pin, sum_rule, to_np, verify

pytestmark = pytest.mark.gpu


def _gen(w, tid, S, H):
    bits = normal_bf16(w.wid, tid, w.B, (S, H, w.D), threads=16)
    dev = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return bits, dev


def _f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def _runs(n, starts, length):
    return [(s, min(n, s + length)) for s in starts]


@pytest.fixture(scope="module")
def shard_inputs():
    w = WORKLOADS["shard_fwd_128k"]
    log("generating shard_fwd_128k inputs")
    qb, q = _gen(w, 0, w.S_q, w.H_q)
    kb, k = _gen(w, 1, w.S_k, w.H_kv)
    vb, v = _gen(w, 2, w.S_k, w.H_kv)
    dob, do = _gen(w, 3, w.S_q, w.H_q)
    return w, (qb, kb, vb, dob), (q, k, v, do)


def test_shard_fwd_128k(shard_inputs):
    w, (qb, kb, vb, _), (q, k, v, _) = shard_inputs
    log("shard_fwd_128k: 32 chunks of 4096, accumulate epilogue")
    o, lse, o_run = shard.shard_forward(q, k, v, w.chunk, q_pos0=w.q_pos0, causal=True)
    log("shard_fwd_128k: per-chunk partials + one sequential merge")
    o2, lse2, _ = shard.shard_forward_partials(q, k, v, w.chunk, q_pos0=w.q_pos0, causal=True)
    log("shard_fwd_128k: fused chunk table, one launch")
    o3, lse3 = shard.shard_forward_fused(q, k, v, w.chunk, q_pos0=w.q_pos0, causal=True)
    torch.cuda.synchronize()
    assert o.shape == (1, 4096, 32, 128) and o.dtype == torch.bfloat16
    # Sampled rows of every head against the oracle.  Keys past the shard's last
    # position are invisible to every query; the oracle sees them all anyway.
    runs = _runs(w.S_q, [0, 1000, 2048, 4080], 16)
    o_np, l_np, o2_np, l2_np, o3_np, l3_np = to_np(o), to_np(lse), to_np(o2), to_np(lse2), to_np(o3), to_np(lse3)
    errs = {"O": 0.0, "LSE": 0.0}
    rms_o = []
    for h in range(w.H_q):
        kh, vh = _f64(kb[0, :, h]), _f64(vb[0, :, h])
        for a, e in runs:
            O_ref, L_ref = oracle.attention_head(_f64(qb[0, a:e, h]), kh, vh, w.scale, True, w.q_pos0 + a, 0)
            for got_o, got_l in ((o_np, l_np), (o2_np, l2_np), (o3_np, l3_np)):
                errs["O"] = max(errs["O"], np.abs(got_o[0, a:e, h] - O_ref).max())
                errs["LSE"] = max(errs["LSE"], np.abs(got_l[0, h, a:e] - L_ref).max())
            rms_o.append(np.sqrt(np.mean(O_ref ** 2)))
    rms = float(np.mean(rms_o))
    log(f"  sampled {len(runs) * 16 * w.H_q} rows: max|err| O {errs['O']:.3e} (rms(O) {rms:.3e}, "
        f"max|err| / rms {errs['O'] / rms:.3e}), LSE {errs['LSE']:.3e}")
    assert errs["O"] <= 1e-2 and errs["LSE"] <= 1e-3
    assert errs["O"] / rms <= 5e-2, "error not small relative to the output's scale"


@pytest.fixture(scope="module")
def shard_bwd(shard_inputs):
    w, (qb, kb, vb, dob), (q, k, v, do) = shard_inputs
    log("shard_bwd_128k: forward, then per-chunk backward from the saved O/LSE")
    o, lse, _ = shard.shard_forward(q, k, v, w.chunk, q_pos0=w.q_pos0, causal=True)
    dq, dk, dv = shard.shard_backward(q, k, v, o, do, lse, w.chunk, q_pos0=w.q_pos0, causal=True)
    log("shard_bwd_128k: fused chunk table (attn_bwd_chunks)")
    fq, fk, fv = shard.shard_backward_fused(q, k, v, o, do, lse, w.chunk, q_pos0=w.q_pos0, causal=True)
    torch.cuda.synchronize()
    return w, (o, lse, dq, dk, dv), (fq, fk, fv)


def test_shard_bwd_128k(shard_inputs, shard_bwd):
    w, _, (q, k, v, do) = shard_inputs
    _, (o, lse, dq, dk, dv), (fq, fk, fv) = shard_bwd
    assert torch.equal(fk, dk) and torch.equal(fv, dv), "fused dK/dV differ from the per-chunk calls"
    e = (fq.float() - dq.float()).abs().max().item()
    log(f"  max|dQ fused - dQ chained| {e:.3e} (max|dQ| {dq.float().abs().max().item():.3e})")
    assert e <= 2e-3
    last = w.q_pos0 + w.S_q  # keys at or after this position are invisible to the shard
    assert torch.all(dk[:, last:] == 0) and torch.all(dv[:, last:] == 0)
    # Sum rules on every head (fp64 sums of the bf16 outputs).
    assert sum_rule("dK", dk[:, :last], 0.0) < 1e-2
    assert sum_rule("dV", dv[:, :last], do.double().sum(1)) < 1e-2


# Heads checked in full against the oracle (restricted to the visible keys).
SHARD_HEADS = [0, 7, 19, 31]


@pytest.mark.parametrize("h", SHARD_HEADS)
def test_shard_bwd_128k_oracle_head(shard_inputs, shard_bwd, h):
    w, (qb, kb, vb, dob), _ = shard_inputs
    _, (o, lse, dq, dk, dv), _ = shard_bwd
    last = w.q_pos0 + w.S_q
    log(f"  oracle forward + backward, head {h}")
    qh, doh = _f64(qb[0, :, h]), _f64(dob[0, :, h])
    kh, vh = _f64(kb[0, :last, h]), _f64(vb[0, :last, h])
    O_ref, L_ref = oracle.attention_head(qh, kh, vh, w.scale, True, w.q_pos0, 0)
    dq_r, dk_r, dv_r = oracle.attention_backward_head(qh, kh, vh, O_ref, doh, L_ref, w.scale, True, w.q_pos0, 0)
    verify(f"h{h}", {"LSE": lse[0, h], "O": o[0, :, h], "dQ": dq[0, :, h], "dK": dk[0, :last, h],
                     "dV": dv[0, :last, h]},
           {"LSE": L_ref, "O": O_ref, "dQ": dq_r, "dK": dk_r, "dV": dv_r})


def test_fp32_s256_4chunks():
    """The fp32 workload in full: Q, K, V, dO [256, 64] fp32, four key chunks of 64, non-causal.
    Forward chunk by chunk (fused accumulate, and per-chunk partials merged sequentially and as
    a tree), backward chunk by chunk from the final (O, LSE); every output against the oracle at
    the graded bounds and at 1e-4, the fp32 self-check."""
    w = WORKLOADS["fp32_s256_4chunks"]
    log("fp32_s256_4chunks: generating inputs")
    x = [normal_f32(w.wid, t, 0, (w.S_q, w.H_q, w.D))[None] for t in range(4)]
    q, k, v, do = (torch.from_numpy(a).cuda() for a in x)
    qh, kh, vh, doh = (a.astype(np.float64) for a in x)
    O_ref, L_ref = oracle.attention(qh, kh, vh, w.scale, w.causal)
    dq_r, dk_r, dv_r = oracle.attention_backward(qh, kh, vh, O_ref, doh, L_ref, w.scale, w.causal)
    o, lse, o_run = shard.shard_forward(q, k, v, w.chunk, causal=w.causal)
    parts = [shard.shard_forward_partials(q, k, v, w.chunk, causal=w.causal, tree=t) for t in (False, True)]
    dq, dk, dv = shard.shard_backward(q, k, v, o, do, lse, w.chunk, causal=w.causal)
    torch.cuda.synchronize()
    for bound in (None, 1e-4):
        for name, got, ref, tol in (("O", o, O_ref, 1e-2), ("O running", o_run, O_ref, 1e-2),
                                    ("O merged sequential", parts[0][0], O_ref, 1e-2),
                                    ("O merged tree", parts[1][0], O_ref, 1e-2), ("LSE", lse, L_ref, 1e-3),
                                    ("dQ", dq, dq_r, 2e-2), ("dK", dk, dk_r, 2e-2), ("dV", dv, dv_r, 2e-2)):
            check(f"{name} (bound {bound or tol})", got, ref, bound or tol)


def test_varlen_packed_70k():
    """The packed variable-length workload at its benchmarked size: 16 causal sequences of
    512 k tokens (k = 1..16), H = 32, d = 128.  Every sequence and head: row 0 equals v_0 and
    the two gradient sum rules; two (sequence, head) pairs in full against the oracle."""
    H, D, wid = VARLEN_PACKED["H"], VARLEN_PACKED["D"], VARLEN_PACKED["wid"]
    lens = [VARLEN_PACKED["unit"] * k for k in VARLEN_PACKED["k"]]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, mx = int(cu[-1]), max(lens)
    log(f"varlen_packed_70k: {len(lens)} sequences, {T} tokens")
    bits = [normal_bf16(wid, t, 1, (T, H, D), threads=16)[0] for t in range(4)]
    q, k, v, do = (torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda() for b in bits)
    cud = torch.from_numpy(cu).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    B.attn_fwd_varlen(q, k, v, o, lse, cud, cud, mx, mx, causal=True, balanced=True)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dq_acc = torch.empty((T, H, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.attn_bwd_workspace_size(len(lens), H, mx), dtype=torch.uint8, device="cuda")
    B.attn_bwd_varlen(q, k, v, o, do, lse, ws, dq_acc, dk, dv, cud, cud, mx, mx, dq=dq, causal=True,
                      compute_delta=True, dq_overwrite=True, finalize_dq=True, balanced=True)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(D)
    starts = torch.from_numpy(cu[:-1].astype(np.int64)).cuda()
    assert torch.equal(o[starts], v[starts]), "row 0 of every sequence must equal its v_0 exactly"
    lse0 = np.einsum("shd,shd->sh", _f64(bits[0][cu[:-1]]), _f64(bits[1][cu[:-1]])) * scale
    check("LSE row 0, every sequence and head", lse[starts], lse0, 1e-3)
    worst_k = worst_v = 0.0
    for a, e in zip(cu[:-1], cu[1:]):
        worst_k = max(worst_k, _sum_rule_quiet(dk[a:e][None], 0.0))
        worst_v = max(worst_v, _sum_rule_quiet(dv[a:e][None], do[a:e][None].double().sum(1)))
    log(f"  sum rules over 16 sequences x 32 heads: dK {worst_k:.3e}, dV {worst_v:.3e}")
    assert worst_k < 1e-2 and worst_v < 1e-2
    for s, h in ((4, 3), (6, 30)):  # a 512-token and a 2048-token sequence
        a, e = int(cu[s]), int(cu[s + 1])
        log(f"  oracle forward + backward for sequence {s} ({e - a} tokens), head {h}")
        qh, kh, vh, doh = (_f64(b[a:e, h]) for b in bits)
        O_ref, L_ref = oracle.attention_head(qh, kh, vh, scale, True)
        check("O", o[a:e, h], O_ref, 1e-2)
        check("LSE", lse[a:e, h], L_ref, 1e-3)
        dq_r, dk_r, dv_r = oracle.attention_backward_head(qh, kh, vh, O_ref, doh, L_ref, scale, True)
        for name, got, ref in (("dQ", dq[a:e, h], dq_r), ("dK", dk[a:e, h], dk_r), ("dV", dv[a:e, h], dv_r)):
            check(name, got, ref, 2e-2)
            err = rel_fro(got, ref)
            log(f"    {name} relative Frobenius error {err:.3e}")
            assert err < 2e-2


def test_tree_decode_64q():
    """The tree decode workload at its benchmarked size: 64 queries under a 32K-token root, 8 children
    of 4K, 8 leaves of 512 each, GQA 32/8.  Every query against split-KV decode of its materialised
    path; sampled (query, head) pairs against the oracle over the path's keys."""
    T = TREE_DECODE
    nodes = tree_nodes(T)
    nq = T["children"] * T["leaves"]
    L = T["root"] + T["children"] * (T["child_len"] + T["leaves"] * T["leaf_len"])
    Hq, Hkv, D = T["H_q"], T["H_kv"], T["D"]
    log(f"tree_decode_64q: {nq} queries, {len(nodes)} nodes, {L} cached tokens")
    qb_ = normal_bf16(T["wid"], 0, 1, (nq, Hq, D))[0]
    kb_ = normal_bf16(T["wid"], 1, 1, (L, Hkv, D), threads=16)[0]
    vb_ = normal_bf16(T["wid"], 2, 1, (L, Hkv, D), threads=16)[0]
    q, kc, vc = (torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda() for b in (qb_, kb_, vb_))
    ks, kl, qs, qe = zip(*nodes)
    ws = torch.empty(B.attn_decode_tree_workspace_size(q, kc, kv_start=ks, kv_len=kl, q_begin=qs, q_end=qe),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty((nq, Hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((nq, Hq), dtype=torch.float32, device="cuda")
    B.attn_decode_tree(q, kc, vc, o, lse, ws, kv_start=ks, kv_len=kl, q_begin=qs, q_end=qe)
    paths = [np.concatenate([np.arange(s, s + n) for s, n, b, e in nodes if b <= i < e]) for i in range(nq)]
    idx = torch.from_numpy(np.stack(paths)).cuda()
    o2, l2 = torch.empty_like(o), torch.empty_like(lse)
    ws2 = torch.empty(B.attn_decode_workspace_size(nq, Hq, D, 16), dtype=torch.uint8, device="cuda")
    B.attn_decode_splitkv(q, kc[idx], vc[idx], o2, l2, ws2, n_splits=16)
    torch.cuda.synchronize()
    check("O vs split-KV decode of the paths, all queries", o, to_np(o2), 1e-2)
    check("LSE vs split-KV decode of the paths, all queries", lse, to_np(l2), 1e-3)
    G = Hq // Hkv
    scale = 1 / math.sqrt(D)
    for i, h in ((0, 0), (37, 17), (63, 31)):
        r = paths[i]
        O_ref, L_ref = oracle.attention_head(_f64(qb_[i:i + 1, h]), _f64(kb_[r, h // G]), _f64(vb_[r, h // G]), scale)
        check(f"query {i} head {h} O", o[i, h], O_ref[0], 1e-2)
        check(f"query {i} head {h} LSE", lse[i, h], L_ref[0], 1e-3)


def _sum_rule_quiet(grads, target):
    s = grads.double().sum(1)
    a = grads.double().abs().sum(1)
    return ((s - target).abs() / a.clamp_min(1e-30)).max().item()


def test_decode_gqa_128k():
    w = WORKLOADS["decode_gqa_128k"]
    log("decode_gqa_128k: generating the 8 GiB KV cache")
    qbits = normal_bf16(w.wid, 0, w.B, (w.H_q, w.D))
    q = torch.from_numpy(qbits.view(np.int16)).view(torch.bfloat16).cuda()
    kb, kc = _gen(w, 1, w.S_k, w.H_kv)
    vb, vc = _gen(w, 2, w.S_k, w.H_kv)
    o = torch.empty((w.B, w.H_q, w.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H_q), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.attn_decode_workspace_size(w.B, w.H_q, w.D, w.n_chunks), dtype=torch.uint8, device="cuda")
    log("decode_gqa_128k: 64 splits + tree merge")
    B.attn_decode_splitkv(q, kc, vc, o, lse, ws, n_splits=w.n_chunks)
    torch.cuda.synchronize()
    o_np, l_np = to_np(o), to_np(lse)
    G = w.H_q // w.H_kv
    err_o = err_l = 0.0
    for b in range(w.B):
        g = (3 * b) % w.H_kv
        heads = list(range(g * G, g * G + G))
        O_ref, L_ref = oracle.attention_head(_f64(qbits[b, heads]), _f64(kb[b, :, g]), _f64(vb[b, :, g]), w.scale)
        err_o = max(err_o, np.abs(o_np[b, heads] - O_ref).max())
        err_l = max(err_l, np.abs(l_np[b, heads] - L_ref).max())
    log(f"  16 (b, kv head) pairs: max|err| O {err_o:.3e}, LSE {err_l:.3e}")
    assert err_o <= 1e-2 and err_l <= 1e-3

    # The uneven-length call the benchmark also times: sequence b holds 8192 k
    # keys, k a permutation of 1..16, so most of its 64 splits are empty.
    lens = [8192 * k for k in (5, 12, 1, 16, 9, 3, 14, 7, 11, 2, 15, 6, 10, 4, 13, 8)]
    log("decode_gqa_128k: uneven lengths, 64 splits + tree merge")
    B.attn_decode_splitkv(q, kc, vc, o, lse, ws, n_splits=w.n_chunks,
                          seqlens=torch.tensor(lens, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    o_np, l_np = to_np(o), to_np(lse)
    err_o = err_l = 0.0
    for b in range(w.B):
        g = (5 * b + 1) % w.H_kv
        heads = list(range(g * G, g * G + G))
        n = lens[b]
        O_ref, L_ref = oracle.attention_head(_f64(qbits[b, heads]), _f64(kb[b, :n, g]), _f64(vb[b, :n, g]), w.scale)
        err_o = max(err_o, np.abs(o_np[b, heads] - O_ref).max())
        err_l = max(err_l, np.abs(l_np[b, heads] - L_ref).max())
    log(f"  uneven lengths, 16 (b, kv head) pairs: max|err| O {err_o:.3e}, LSE {err_l:.3e}")
    assert err_o <= 1e-2 and err_l <= 1e-3


@pytest.fixture(scope="module")
def causal32k():
    w = WORKLOADS["causal_fwdbwd_32k"]
    log("causal_fwdbwd_32k: generating inputs")
    qb, q = _gen(w, 0, w.S_q, w.H_q)
    kb, k = _gen(w, 1, w.S_k, w.H_kv)
    vb, v = _gen(w, 2, w.S_k, w.H_kv)
    dob, do = _gen(w, 3, w.S_q, w.H_q)
    log("causal_fwdbwd_32k: balanced forward + backward (the benchmark's launch configuration)")
    o, lse = shard.causal_attention_forward(q, k, v, balanced=True)
    dq, dk, dv = shard.causal_attention_backward(q, k, v, o, do, lse, balanced=True)
    torch.cuda.synchronize()
    return w, (qb, kb, vb, dob), (q, k, v, do), (o, lse, dq, dk, dv)


def test_causal_fwdbwd_32k(causal32k):
    w, (qb, kb, vb, dob), (q, k, v, do), (o, lse, dq, dk, dv) = causal32k
    # Row 0 of every (b, h) sees only key 0.
    row0_pin(o[:, 0], v[:, 0], lse[:, :, 0], _f64(qb[:, 0]), _f64(kb[:, 0]), w.scale)
    # Sum rules on every (b, h).
    assert sum_rule("dK", dk, 0.0) < 1e-2
    assert sum_rule("dV", dv, do.double().sum(1)) < 1e-2
    # Sampled rows of a head the full checks below do not cover.
    for a, e in _runs(w.S_q, [0, 5000, 20000, 32752], 16):
        O_ref, L_ref = oracle.attention_head(_f64(qb[1, a:e, 13]), _f64(kb[1, :e, 13]), _f64(vb[1, :e, 13]),
                                             w.scale, True, a, 0)
        verify(f"(1,13) rows {a}..{e}", {"O": o[1, a:e, 13], "LSE": lse[1, 13, a:e]}, {"O": O_ref, "LSE": L_ref})


# (batch, head) pairs checked in full against the oracle: every batch, four heads.
C5_PAIRS = [(b, h) for b in (0, 1) for h in (0, 7, 19, 31)]


@pytest.mark.parametrize("b,h", C5_PAIRS)
def test_causal_fwdbwd_32k_oracle_pair(causal32k, b, h):
    w, (qb, kb, vb, dob), _, (o, lse, dq, dk, dv) = causal32k
    log(f"  oracle forward + backward for (b={b}, h={h})")
    qh, kh, vh, doh = (_f64(x[b, :, h]) for x in (qb, kb, vb, dob))
    O_ref, L_ref = oracle.attention_head(qh, kh, vh, w.scale, True)
    dq_r, dk_r, dv_r = oracle.attention_backward_head(qh, kh, vh, O_ref, doh, L_ref, w.scale, True)
    verify(f"({b},{h})", {"LSE": lse[b, h], "O": o[b, :, h], "dQ": dq[b, :, h], "dK": dk[b, :, h], "dV": dv[b, :, h]},
           {"LSE": L_ref, "O": O_ref, "dQ": dq_r, "dK": dk_r, "dV": dv_r})
