"""GPU parity at small sizes: every entry point against the fp64 oracle, element by element.

Shapes span several tiles and ragged tails, causal offsets that make rows fully
visible, diagonal or fully masked, grouped heads, empty inputs, chunked
accumulation, both merge orders and decode splits.  Bounds: O 1e-2 and
dQ/dK/dV 2e-2, each times max(1, max|oracle|) because bf16 output rounding
alone is relative; LSE 1e-3 absolute.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_blockwise_attention_attn_amd import binding as B
from exact_blockwise_attention_attn_amd import shard
from seeded_inputs import normal_f32
from tests.gpu_util import check, log, seq_tensor, to_np

pytestmark = pytest.mark.gpu

O_TOL, G_TOL, L_TOL = 1e-2, 2e-2, 1e-3

# (Sq, Sk, D, causal, q_pos0, k_pos0, B, Hq, Hkv, dtype, balanced)
FWD_CASES = [
    (1, 1, 128, False, 0, 0, 1, 1, 1, "bf16", False),
    (2, 17, 64, False, 0, 0, 1, 2, 2, "bf16", False),
    (17, 63, 128, True, 0, 0, 1, 1, 1, "bf16", False),
    (63, 64, 128, True, 10, 0, 2, 2, 1, "bf16", False),
    (64, 65, 64, False, 0, 0, 1, 3, 3, "bf16", False),
    (65, 129, 128, True, 64, 0, 2, 4, 2, "bf16", False),
    (129, 255, 128, True, 0, 100, 1, 2, 2, "bf16", False),  # rows 0..99 see nothing
    (255, 300, 128, False, 0, 0, 1, 8, 1, "bf16", False),
    (200, 200, 128, True, 0, 0, 2, 2, 2, "bf16", True),
    (300, 257, 64, True, 500, 0, 1, 2, 2, "bf16", False),  # every row sees every key
    (1024, 2048, 128, True, 1024, 0, 1, 2, 2, "bf16", False),
    (513, 513, 128, True, 0, 0, 1, 1, 1, "bf16", True),
    (5, 0, 128, False, 0, 0, 1, 1, 1, "bf16", False),  # no keys: identity
    (100, 77, 64, True, 5, 0, 1, 2, 2, "f32", False),
    (64, 256, 128, False, 0, 0, 1, 1, 1, "f32", False),
    (70, 90, 64, True, 0, 30, 2, 2, 1, "f32", False),
]


def _ids(cases):
    return ["-".join(str(x) for x in c) for c in cases]


def _inputs(wid, Bn, Sq, Sk, Hq, Hkv, D, dtype):
    q, qh = seq_tensor(wid, 0, Bn, Sq, Hq, D, dtype)
    k, kh = seq_tensor(wid, 1, Bn, Sk, Hkv, D, dtype)
    v, vh = seq_tensor(wid, 2, Bn, Sk, Hkv, D, dtype)
    return (q, k, v), (qh, kh, vh)


@pytest.mark.parametrize("case", FWD_CASES, ids=_ids(FWD_CASES))
def test_fwd_partial(case):
    Sq, Sk, D, causal, qp, kp, Bn, Hq, Hkv, dtype, bal = case
    log(f"fwd {case}")
    (q, k, v), (qh, kh, vh) = _inputs(101, Bn, Sq, Sk, Hq, Hkv, D, dtype)
    scale = 1 / math.sqrt(D)
    O_ref, L_ref = oracle.attention(qh, kh, vh, scale, causal, qp, kp)
    for odt in (torch.float32, torch.bfloat16) if dtype == "bf16" else (torch.float32,):
        o = torch.full((Bn, Sq, Hq, D), float("nan"), dtype=odt, device="cuda")
        lse = torch.full((Bn, Hq, Sq), float("nan"), dtype=torch.float32, device="cuda")
        B.attn_fwd_partial(q, k, v, o, lse, q_pos0=qp, k_pos0=kp, causal=causal, balanced=bal)
        torch.cuda.synchronize()
        check(f"O ({odt})", o, O_ref, O_TOL, scale_by_max=True)
        check("LSE", lse, L_ref, L_TOL)


def test_fwd_strided_views_and_scale():
    """Non-contiguous [B, S, H, D] views (a head slice of a wider tensor) and an explicit scale."""
    log("fwd strided")
    (q, k, v), (qh, kh, vh) = _inputs(102, 2, 96, 150, 6, 6, 128, "bf16")
    qs, ks, vs = q[:, :, 1:4], k[:, :, 2:5], v[:, :, 3:6]
    o = torch.empty((2, 96, 3, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((2, 3, 96), dtype=torch.float32, device="cuda")
    B.attn_fwd_partial(qs, ks, vs, o, lse, causal=True, q_pos0=60, scale=0.05)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(qh[:, :, 1:4], kh[:, :, 2:5], vh[:, :, 3:6], 0.05, True, 60, 0)
    check("O", o, O_ref, O_TOL, scale_by_max=True)
    check("LSE", lse, L_ref, L_TOL)


def _oracle_over_chunks(qh, chunks, scale, causal, q_pos0):
    """Oracle attention over a list of (k, v, pos0) chunks: each chunk on its own, then merged."""
    parts = []
    for kh, vh, pos0 in chunks:
        if kh.shape[1] == 0:
            continue
        O, L = oracle.attention(qh, kh, vh, scale, causal, q_pos0, pos0)
        parts.append((O, np.transpose(L, (0, 2, 1))))
    if not parts:
        Bn, Sq, Hq, D = qh.shape
        return np.zeros((Bn, Sq, Hq, D)), np.full((Bn, Hq, Sq), -np.inf)
    O, L = oracle.merge(parts)
    return O, np.transpose(L, (0, 2, 1))


# (B, Sq, Hq, Hkv, D, chunk lengths, chunk positions, q_pos0, causal, balanced)
FUSED_CASES = [
    # contiguous chunks, ragged lengths, an empty chunk, causal with a partly visible diagonal
    (1, 200, 2, 2, 128, (64, 100, 0, 37), (0, 64, 164, 164), 100, True, False),
    # chunks out of position order, grouped heads, head_dim 64
    (2, 130, 4, 2, 64, (129, 200), (1000, 0), 1100, True, False),
    # non-causal, one long chunk
    (1, 64, 2, 1, 128, (300,), (0,), 0, False, False),
    # a chunk entirely after every query (skipped) and one every query sees
    (1, 96, 2, 2, 128, (128, 64), (5000, 0), 200, True, True),
    # the shard layout: 8 chunks of 64 keys, queries in the middle of the range
    (1, 256, 2, 2, 128, (64,) * 8, tuple(64 * i for i in range(8)), 192, True, True),
    # the most chunks a table takes (64): ragged lengths 0..69 at consecutive positions, the
    # queries' diagonal inside the range, so chunks are fully visible, partly visible and skipped
    (1, 128, 2, 2, 128, tuple((37 * i) % 70 for i in range(64)),
     tuple(sum((37 * j) % 70 for j in range(i)) for i in range(64)), 1000, True, True),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=_ids(FUSED_CASES))
def test_fwd_chunks_fused(case):
    """One launch over a chunk table against the oracle over the same chunks, for fp32 and
    bf16 outputs; with ACCUMULATE the chunks merge into a running result from an earlier call."""
    Bn, Sq, Hq, Hkv, D, lens, pos, qp, causal, bal = case
    log(f"fwd chunks {case}")
    q, qh = seq_tensor(109, 0, Bn, Sq, Hq, D, "bf16")
    chunks, chunks_h = [], []
    for c, L in enumerate(lens):
        k, kh = seq_tensor(109, 10 + 2 * c, Bn, L, Hkv, D, "bf16")
        v, vh = seq_tensor(109, 11 + 2 * c, Bn, L, Hkv, D, "bf16")
        chunks.append((k, v))
        chunks_h.append((kh, vh, pos[c]))
    scale = 1 / math.sqrt(D)
    O_ref, L_ref = _oracle_over_chunks(qh, chunks_h, scale, causal, qp)
    ks, vs = [k for k, _ in chunks], [v for _, v in chunks]
    for odt in (torch.float32, torch.bfloat16):
        o = torch.full((Bn, Sq, Hq, D), float("nan"), dtype=odt, device="cuda")
        lse = torch.full((Bn, Hq, Sq), float("nan"), dtype=torch.float32, device="cuda")
        B.attn_fwd_chunks(q, ks, vs, o, lse, chunk_pos0=pos, q_pos0=qp, causal=causal, balanced=bal)
        torch.cuda.synchronize()
        check(f"O ({odt})", o, O_ref, O_TOL, scale_by_max=True)
        check("LSE", lse, L_ref, L_TOL)
    # ACCUMULATE: a running result over extra keys at other positions, then the chunk table.
    ke, keh = seq_tensor(109, 90, Bn, 77, Hkv, D, "bf16")
    ve, veh = seq_tensor(109, 91, Bn, 77, Hkv, D, "bf16")
    o = torch.empty((Bn, Sq, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((Bn, Hq, Sq), dtype=torch.float32, device="cuda")
    B.attn_fwd_partial(q, ke, ve, o, lse, q_pos0=qp, k_pos0=-500, causal=causal)
    of = torch.empty((Bn, Sq, Hq, D), dtype=torch.bfloat16, device="cuda")
    B.attn_fwd_chunks(q, ks, vs, o, lse, chunk_pos0=pos, q_pos0=qp, causal=causal, accumulate=True, o_final=of)
    torch.cuda.synchronize()
    O_acc, L_acc = _oracle_over_chunks(qh, [(keh, veh, -500)] + chunks_h, scale, causal, qp)
    check("O accumulate", o, O_acc, O_TOL, scale_by_max=True)
    check("O final bf16", of, O_acc, O_TOL, scale_by_max=True)
    check("LSE accumulate", lse, L_acc, L_TOL)


def test_fwd_chunks_matches_chained_partials():
    """The fused call and chained attn_fwd_partial(ACCUMULATE) calls over the same chunks agree."""
    log("fwd chunks vs chained")
    Bn, Sq, H, D = 1, 160, 2, 128
    q, _ = seq_tensor(110, 0, Bn, Sq, H, D, "bf16")
    k, _ = seq_tensor(110, 1, Bn, 640, H, D, "bf16")
    v, _ = seq_tensor(110, 2, Bn, 640, H, D, "bf16")
    bounds = [(0, 128), (128, 300), (300, 640)]
    ks, vs = [k[:, a:e] for a, e in bounds], [v[:, a:e] for a, e in bounds]
    o1 = torch.empty((Bn, Sq, H, D), dtype=torch.float32, device="cuda")
    l1 = torch.empty((Bn, H, Sq), dtype=torch.float32, device="cuda")
    B.attn_fwd_chunks(q, ks, vs, o1, l1, chunk_pos0=[a for a, _ in bounds], q_pos0=400, causal=True)
    _, l2, o2 = shard.shard_forward(q, k, v, 128, q_pos0=400, causal=True)
    torch.cuda.synchronize()
    check("O fused vs chained", o1, to_np(o2), O_TOL, scale_by_max=True)
    check("LSE fused vs chained", l1, to_np(l2), L_TOL)


# (Sq, Sk, chunk, causal, q_pos0, Hq, Hkv, D, dtype)
CHUNK_CASES = [
    (256, 256, 64, False, 0, 1, 1, 64, "f32"),
    (128, 1000, 128, True, 600, 2, 2, 128, "bf16"),
    (300, 700, 100, True, 350, 4, 1, 128, "bf16"),
    (64, 512, 64, True, 0, 2, 2, 64, "bf16"),
]


@pytest.mark.parametrize("case", CHUNK_CASES, ids=_ids(CHUNK_CASES))
def test_chunked_forward_and_merge(case):
    """Chunk by chunk with the fused accumulate epilogue, and per-chunk partials merged
    sequentially and as a tree, all against the unchunked oracle."""
    Sq, Sk, chunk, causal, qp, Hq, Hkv, D, dtype = case
    log(f"chunked {case}")
    (q, k, v), (qh, kh, vh) = _inputs(103, 1, Sq, Sk, Hq, Hkv, D, dtype)
    scale = 1 / math.sqrt(D)
    O_ref, L_ref = oracle.attention(qh, kh, vh, scale, causal, qp, 0)
    o, lse, o_run = shard.shard_forward(q, k, v, chunk, q_pos0=qp, causal=causal)
    torch.cuda.synchronize()
    check("O accumulate", o, O_ref, O_TOL, scale_by_max=True)
    check("O running fp32", o_run, O_ref, O_TOL, scale_by_max=True)
    check("LSE accumulate", lse, L_ref, L_TOL)
    for tree in (False, True):
        o2, l2, _ = shard.shard_forward_partials(q, k, v, chunk, q_pos0=qp, causal=causal, tree=tree)
        torch.cuda.synchronize()
        check(f"O merged tree={tree}", o2, O_ref, O_TOL, scale_by_max=True)
        check(f"LSE merged tree={tree}", l2, L_ref, L_TOL)


@pytest.mark.parametrize("n,tree,D", [(1, False, 128), (2, True, 64), (5, True, 128), (17, False, 128),
                                      (64, True, 128), (100, True, 64)])
def test_merge_kernel(n, tree, D):
    log(f"merge n={n} tree={tree} D={D}")
    Bn, S, H = 2, 37, 3
    rng = np.random.default_rng([104, n, D])
    O = rng.standard_normal((n, Bn, S, H, D)).astype(np.float32)
    L = (3 * rng.standard_normal((n, Bn, H, S))).astype(np.float32)
    L[:, 0, 0, :5] = -np.inf  # rows with no key in any part
    if n > 1:
        L[1] = -np.inf  # an empty part
        O[1] = 0.0
    O[np.isinf(L).transpose(0, 1, 3, 2)] = 0.0
    O_ref, L_ref = (oracle.merge_tree if tree else oracle.merge)(
        [(O[c], L[c].transpose(0, 2, 1)) for c in range(n)])
    L_ref = L_ref.transpose(0, 2, 1)
    o_parts = torch.from_numpy(O).cuda()
    l_parts = torch.from_numpy(L).cuda()
    for odt in (torch.float32, torch.bfloat16):
        o = torch.empty((Bn, S, H, D), dtype=odt, device="cuda")
        lse = torch.empty((Bn, H, S), dtype=torch.float32, device="cuda")
        B.attn_merge_lse(o_parts, l_parts, o, lse, tree=tree)
        torch.cuda.synchronize()
        check(f"merge O {odt}", o, O_ref, 1e-5 if odt == torch.float32 else O_TOL, scale_by_max=True)
        check("merge LSE", lse, L_ref, 1e-5)
    # Output aliasing part 0 (documented as allowed).
    B.attn_merge_lse(o_parts, l_parts, o_parts[0], l_parts[0], tree=tree)
    torch.cuda.synchronize()
    check("merge O aliased", o_parts[0], O_ref, 1e-5, scale_by_max=True)
    check("merge LSE aliased", l_parts[0], L_ref, 1e-5)



def test_merge_pair_separate_buffers():
    """The two-pointer form: two partials in separately allocated buffers merged through a part stride equal
    to their distance (positive or negative), bit for bit as the same two parts stacked in one array."""
    log("merge of two separate buffers")
    Bn, S, H, D = 2, 45, 3, 128
    rng = np.random.default_rng(123)
    mk = lambda *sh: torch.from_numpy(rng.standard_normal(sh).astype(np.float32)).cuda()
    o_a, o_b = mk(Bn, S, H, D), mk(Bn, S, H, D)
    l_a, l_b = 3 * mk(Bn, H, S), 3 * mk(Bn, H, S)
    l_b[0, 1, :7] = -float("inf")  # part b sees no key for these rows
    o_b[0, :7, 1] = 0.0
    for (x, lx), (y, ly) in (((o_a, l_a), (o_b, l_b)), ((o_b, l_b), (o_a, l_a))):
        for tree in (False, True):
            o1, l1 = torch.empty_like(o_a), torch.empty_like(l_a)
            B.attn_merge_lse_pair(x, lx, y, ly, o1, l1, tree=tree)
            o2, l2 = torch.empty_like(o_a), torch.empty_like(l_a)
            B.attn_merge_lse(torch.stack([x, y]), torch.stack([lx, ly]), o2, l2, tree=tree)
            torch.cuda.synchronize()
            assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert o_a.data_ptr() != o_b.data_ptr()  # so one of the two orders above has a negative part stride
    O_ref, L_ref = oracle.merge([(to_np(o_a), to_np(l_a).transpose(0, 2, 1)), (to_np(o_b), to_np(l_b).transpose(0, 2, 1))])
    o1, l1 = torch.empty_like(o_a), torch.empty_like(l_a)
    B.attn_merge_lse_pair(o_a, l_a, o_b, l_b, o1, l1)
    torch.cuda.synchronize()
    check("pair merge O", o1, O_ref, 1e-5, scale_by_max=True)
    check("pair merge LSE", l1, L_ref.transpose(0, 2, 1), 1e-5)


# (Sq, Sk, D, causal, q_pos0, k_pos0, B, Hq, Hkv, dtype, balanced)
BWD_CASES = [
    (1, 1, 128, False, 0, 0, 1, 1, 1, "bf16", False),
    (17, 63, 64, True, 0, 0, 1, 2, 2, "bf16", False),
    (65, 129, 128, True, 64, 0, 2, 4, 2, "bf16", False),
    (129, 255, 128, True, 0, 100, 1, 2, 2, "bf16", False),
    (200, 200, 128, True, 0, 0, 2, 2, 2, "bf16", True),
    (255, 64, 128, False, 0, 0, 1, 4, 1, "bf16", False),
    (300, 257, 64, True, 500, 0, 1, 2, 2, "bf16", False),
    (257, 257, 128, True, 0, 0, 1, 1, 1, "bf16", True),
    (100, 77, 64, True, 5, 0, 1, 2, 2, "f32", False),
    (64, 130, 128, False, 0, 0, 1, 2, 1, "f32", False),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=_ids(BWD_CASES))
def test_bwd(case):
    Sq, Sk, D, causal, qp, kp, Bn, Hq, Hkv, dtype, bal = case
    log(f"bwd {case}")
    (q, k, v), (qh, kh, vh) = _inputs(105, Bn, Sq, Sk, Hq, Hkv, D, dtype)
    do, doh = seq_tensor(105, 3, Bn, Sq, Hq, D, dtype)
    scale = 1 / math.sqrt(D)
    O_ref, L_ref = oracle.attention(qh, kh, vh, scale, causal, qp, kp)
    dq_ref, dk_ref, dv_ref = oracle.attention_backward(qh, kh, vh, O_ref, doh, L_ref, scale, causal, qp, kp)
    o = torch.empty_like(q)
    lse = torch.empty((Bn, Hq, Sq), dtype=torch.float32, device="cuda")
    B.attn_fwd_partial(q, k, v, o, lse, q_pos0=qp, k_pos0=kp, causal=causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dq_acc = torch.full((Bn, Sq, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.full((B.attn_bwd_workspace_size(Bn, Hq, Sq) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    B.attn_bwd(q, k, v, o, do, lse, ws, dq_acc, dk, dv, dq=dq, q_pos0=qp, k_pos0=kp, causal=causal,
               compute_delta=True, dq_overwrite=True, finalize_dq=True, balanced=bal)
    torch.cuda.synchronize()
    check("dQ", dq, dq_ref, G_TOL, scale_by_max=True)
    check("dK", dk, dk_ref, G_TOL, scale_by_max=True)
    check("dV", dv, dv_ref, G_TOL, scale_by_max=True)
    # Workspace layout: per (b, h), Sq_pad rows of LSE*log2(e) then Sq_pad rows of -delta.
    sq_pad = (Sq + 63) // 64 * 64
    st = ws[: Bn * Hq * 2 * sq_pad].view(Bn, Hq, 2, sq_pad).cpu().double().numpy()
    check("-delta", st[:, :, 1, :Sq], -np.einsum("bshd,bshd->bhs", doh, O_ref), G_TOL, scale_by_max=True)
    l2_ref = np.where(np.isneginf(L_ref), np.inf, L_ref * math.log2(math.e))
    check("lse*log2e", st[:, :, 0, :Sq], l2_ref, L_TOL * math.log2(math.e))
    assert np.all(st[:, :, 0, Sq:] == np.inf) and np.all(st[:, :, 1, Sq:] == 0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_chunked(dtype):
    """Per-chunk backward with the final LSE: dQ accumulated over chunks, dK/dV per chunk."""
    Sq, Sk, chunk, qp, H, D = 160, 600, 128, 400, 2, 64 if dtype == "f32" else 128
    log(f"bwd chunked {dtype}")
    (q, k, v), (qh, kh, vh) = _inputs(106, 1, Sq, Sk, H, H, D, dtype)
    do, doh = seq_tensor(106, 3, 1, Sq, H, D, dtype)
    scale = 1 / math.sqrt(D)
    O_ref, L_ref = oracle.attention(qh, kh, vh, scale, True, qp, 0)
    dq_ref, dk_ref, dv_ref = oracle.attention_backward(qh, kh, vh, O_ref, doh, L_ref, scale, True, qp, 0)
    o, lse, _ = shard.shard_forward(q, k, v, chunk, q_pos0=qp, causal=True)
    dq, dk, dv = shard.shard_backward(q, k, v, o, do, lse, chunk, q_pos0=qp, causal=True)
    torch.cuda.synchronize()
    check("dQ", dq, dq_ref, G_TOL, scale_by_max=True)
    check("dK", dk, dk_ref, G_TOL, scale_by_max=True)
    check("dV", dv, dv_ref, G_TOL, scale_by_max=True)
    assert torch.all(dk[:, Sq + qp:] == 0) and torch.all(dv[:, Sq + qp:] == 0), "invisible keys got gradient"


@pytest.mark.parametrize("case", FUSED_CASES, ids=_ids(FUSED_CASES))
def test_bwd_chunks_fused(case):
    """One call over a chunk table against the oracle's per-chunk backward from the global O and
    LSE: dK/dV of every chunk (zeros for a chunk no query sees), dQ summed over the chunks, also
    added to a running dq_acc without DQ_OVERWRITE."""
    Bn, Sq, Hq, Hkv, D, lens, pos, qp, causal, bal = case
    log(f"bwd chunks {case}")
    q, qh = seq_tensor(111, 0, Bn, Sq, Hq, D, "bf16")
    do, doh = seq_tensor(111, 1, Bn, Sq, Hq, D, "bf16")
    ks, vs, chunks_h = [], [], []
    for c, L in enumerate(lens):
        k, kh = seq_tensor(111, 10 + 2 * c, Bn, L, Hkv, D, "bf16")
        v, vh = seq_tensor(111, 11 + 2 * c, Bn, L, Hkv, D, "bf16")
        ks.append(k)
        vs.append(v)
        chunks_h.append((kh, vh, pos[c]))
    scale = 1 / math.sqrt(D)
    O_ref, L_ref = _oracle_over_chunks(qh, chunks_h, scale, causal, qp)
    dq_ref = np.zeros(qh.shape)
    dkv_ref = []
    for kh, vh, p0 in chunks_h:
        a, bk, bv = oracle.attention_backward(qh, kh, vh, O_ref, doh, L_ref, scale, causal, qp, p0)
        dq_ref += a
        dkv_ref.append((bk, bv))
    o = torch.empty((Bn, Sq, Hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((Bn, Hq, Sq), dtype=torch.float32, device="cuda")
    B.attn_fwd_chunks(q, ks, vs, o, lse, chunk_pos0=pos, q_pos0=qp, causal=causal)
    dks = [torch.full_like(k, float("nan")) for k in ks]
    dvs = [torch.full_like(v, float("nan")) for v in vs]
    dq = torch.full_like(q, float("nan"))
    dq_acc = torch.full((Bn, Sq, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.full((B.attn_bwd_workspace_size(Bn, Hq, Sq) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    B.attn_bwd_chunks(q, ks, vs, o, do, lse, ws, dq_acc, dks, dvs, chunk_pos0=pos, dq=dq, q_pos0=qp, causal=causal,
                      compute_delta=True, dq_overwrite=True, finalize_dq=True, balanced=bal)
    torch.cuda.synchronize()
    check("dQ", dq, dq_ref, G_TOL, scale_by_max=True)
    check("dQ acc", dq_acc, dq_ref, G_TOL, scale_by_max=True)
    for c, ((bk, bv), dk, dv) in enumerate(zip(dkv_ref, dks, dvs)):
        check(f"dK[{c}]", dk, bk, G_TOL, scale_by_max=True)
        check(f"dV[{c}]", dv, bv, G_TOL, scale_by_max=True)
        if not np.any(bk) and not np.any(bv) and lens[c] > 0:
            assert torch.all(dk == 0) and torch.all(dv == 0), f"chunk {c} is invisible but got gradient"
    # Accumulate into a running dq_acc, statistics reused from the first call.
    base = torch.randn((Bn, Sq, Hq, D), dtype=torch.float32, device="cuda", generator=torch.Generator("cuda").manual_seed(3))
    dq_acc2 = base.clone()
    B.attn_bwd_chunks(q, ks, vs, o, do, lse, ws, dq_acc2, dks, dvs, chunk_pos0=pos, dq=dq, q_pos0=qp, causal=causal,
                      finalize_dq=True, balanced=bal)
    torch.cuda.synchronize()
    check("dQ acc added", dq_acc2 - base, dq_ref, G_TOL, scale_by_max=True)
    check("dQ from added acc", dq, (base.cpu().double().numpy() + dq_ref), G_TOL, scale_by_max=True)


def test_bwd_chunks_matches_chained_calls():
    """The fused call and chained attn_bwd calls over the same chunks: identical dK/dV (the same
    per-tile arithmetic), dQ equal up to the order of the fp32 additions across chunks."""
    log("bwd chunks vs chained")
    Bn, Sq, H, D, chunk, qp = 2, 192, 2, 128, 96, 300
    Sk = 600
    (q, k, v), _ = _inputs(112, Bn, Sq, Sk, H, H, D, "bf16")
    do, _ = seq_tensor(112, 3, Bn, Sq, H, D, "bf16")
    o, lse, _ = shard.shard_forward(q, k, v, chunk, q_pos0=qp, causal=True)
    dq1, dk1, dv1 = shard.shard_backward(q, k, v, o, do, lse, chunk, q_pos0=qp, causal=True)
    dq2, dk2, dv2 = shard.shard_backward_fused(q, k, v, o, do, lse, chunk, q_pos0=qp, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dk1, dk2) and torch.equal(dv1, dv2)
    err = (dq1.float() - dq2.float()).abs().max().item()
    log(f"  max|dQ chained - dQ fused| = {err:.3e} (max|dQ| {dq1.float().abs().max().item():.3e})")
    assert err <= 1e-2 * max(1.0, dq1.float().abs().max().item())


# (per-sequence (len_q, len_k), Hq, Hkv, D, causal, balanced)
VARLEN_CASES = [
    # equal lengths as in packed training, including an empty and a one-token sequence
    (((200, 200), (1, 1), (0, 0), (130, 130), (64, 64)), 2, 2, 128, True, False),
    # queries at the end of longer key sequences, grouped heads, head_dim 64
    (((17, 300), (128, 129), (65, 65)), 4, 2, 64, True, True),
    # more queries than keys: the first len_q - len_k queries see nothing
    (((100, 60), (33, 200)), 2, 1, 128, True, False),
    # non-causal
    (((77, 250), (256, 3)), 2, 2, 128, False, False),
]


def _varlen_inputs(wid, lens, Hq, Hkv, D):
    """Packed [total, heads, D] bf16 tensors and per-sequence fp64 views, plus offsets."""
    cu_q = np.concatenate([[0], np.cumsum([a for a, _ in lens])]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum([b for _, b in lens])]).astype(np.int32)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    q, qh = seq_tensor(wid, 0, 1, tq, Hq, D, "bf16")
    k, kh = seq_tensor(wid, 1, 1, tk, Hkv, D, "bf16")
    v, vh = seq_tensor(wid, 2, 1, tk, Hkv, D, "bf16")
    do, doh = seq_tensor(wid, 3, 1, tq, Hq, D, "bf16")
    dev = [x[0] for x in (q, k, v, do)]
    host = [x[0] for x in (qh, kh, vh, doh)]
    return dev, host, torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda(), cu_q, cu_k


@pytest.mark.parametrize("case", VARLEN_CASES, ids=_ids(VARLEN_CASES))
def test_varlen_fwd_bwd(case):
    """Packed variable-length batch, forward and backward, against the oracle run on each
    sequence alone with its queries at the end of its keys."""
    lens, Hq, Hkv, D, causal, bal = case
    log(f"varlen {case}")
    (q, k, v, do), (qh, kh, vh, doh), cuq, cuk, cu_q, cu_k = _varlen_inputs(113, lens, Hq, Hkv, D)
    mq, mk = max(a for a, _ in lens), max(b for _, b in lens)
    scale = 1 / math.sqrt(D)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    o = torch.full((tq, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((tq, Hq), float("nan"), dtype=torch.float32, device="cuda")
    B.attn_fwd_varlen(q, k, v, o, lse, cuq, cuk, mq, mk, causal=causal, balanced=bal)
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    dq_acc = torch.full((tq, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.full((B.attn_bwd_workspace_size(len(lens), Hq, mq) // 4,), float("nan"), dtype=torch.float32,
                    device="cuda")
    B.attn_bwd_varlen(q, k, v, o, do, lse, ws, dq_acc, dk, dv, cuq, cuk, mq, mk, dq=dq, causal=causal,
                      compute_delta=True, dq_overwrite=True, finalize_dq=True, balanced=bal)
    torch.cuda.synchronize()
    for s, (a0, a1, b0, b1) in enumerate(zip(cu_q[:-1], cu_q[1:], cu_k[:-1], cu_k[1:])):
        if a1 == a0 and b1 == b0:
            continue
        qs, ks, vs, dos = qh[None, a0:a1], kh[None, b0:b1], vh[None, b0:b1], doh[None, a0:a1]
        qp = int(b1 - b0) - int(a1 - a0)
        O_ref, L_ref = oracle.attention(qs, ks, vs, scale, causal, qp, 0)
        dq_r, dk_r, dv_r = oracle.attention_backward(qs, ks, vs, O_ref, dos, L_ref, scale, causal, qp, 0)
        check(f"seq {s} O", o[a0:a1], O_ref[0], O_TOL, scale_by_max=True)
        check(f"seq {s} LSE", lse[a0:a1], L_ref[0].T, L_TOL)
        check(f"seq {s} dQ", dq[a0:a1], dq_r[0], G_TOL, scale_by_max=True)
        check(f"seq {s} dQ acc", dq_acc[a0:a1], dq_r[0], G_TOL, scale_by_max=True)
        check(f"seq {s} dK", dk[b0:b1], dk_r[0], G_TOL, scale_by_max=True)
        check(f"seq {s} dV", dv[b0:b1], dv_r[0], G_TOL, scale_by_max=True)


# (n_queries, Hq, Hkv, D, cache_len, nodes as (kv_start, kv_len, q_begin, q_end), root first)
def _chain_tree():
    """20 queries under a chain of 70 short nodes, a node with no keys, one leaf per query and a
    2100-key node (two segments) over queries 5..14."""
    nodes, s = [], 0
    for j in range(70):
        n = 16 + j % 5
        nodes.append((s, n, 0, 20))
        s += n
    nodes.append((s, 0, 0, 20))
    for i in range(20):
        nodes.append((s, 33, i, i + 1))
        s += 33
    nodes.append((s, 2100, 5, 15))
    s += 2100
    return (20, 16, 2, 128, s, tuple(nodes))


TREE_CASES = [
    # root, two inner nodes, five leaves (one with no keys)
    (5, 8, 2, 128, 1700, ((0, 1000, 0, 5), (1000, 300, 0, 3), (1300, 10, 3, 5), (1310, 90, 0, 1), (1400, 1, 1, 2),
                          (1401, 0, 2, 3), (1401, 99, 3, 4), (1500, 200, 4, 5))),
    # a root shared by 300 queries (several query tiles per node) and three uneven branches
    (300, 4, 4, 64, 6500, ((0, 5000, 0, 300), (5000, 500, 0, 100), (5500, 500, 100, 250), (6000, 500, 250, 300))),
    # a query no node covers
    (3, 2, 1, 128, 64, ((0, 64, 0, 2),)),
    # GQA group of 8 (a packed tile of 20 queries x 8 heads, leaves with 8 live rows); 93 table
    # segments, more than 64 of them on every query's path
    _chain_tree(),
    # d = 64 with GQA 4: 70 queries x 4 heads = 280 packed rows under the root (three tiles)
    (70, 8, 2, 64, 3000, ((0, 2500, 0, 70), (2500, 300, 0, 35), (2800, 200, 35, 70))),
    # the most nodes a tree takes (256): a 9,000-key root over 255 queries and one 10-key leaf
    # per query.  Cut into 2,048-key segments the nodes need 260 table entries, so the host
    # doubles the segment length until they fit (16,384 keys: 256 entries).
    (255, 4, 2, 128, 9000 + 255 * 10, ((0, 9000, 0, 255),) + tuple((9000 + 10 * i, 10, i, i + 1) for i in range(255))),
]


@pytest.mark.parametrize("case", TREE_CASES, ids=[f"tree{i}" for i in range(len(TREE_CASES))])
def test_decode_tree(case):
    """Tree-structured decode against the oracle over each query's path (the concatenated keys
    of the nodes that cover it); the first tree also against split-KV decode of the
    materialised per-query caches."""
    nq, Hq, Hkv, D, L, nodes = case
    log(f"tree decode {nq} queries, {len(nodes)} nodes")
    q, qh = seq_tensor(114, 0, 1, nq, Hq, D, "bf16")
    kc, kh = seq_tensor(114, 1, 1, L, Hkv, D, "bf16")
    vc, vh = seq_tensor(114, 2, 1, L, Hkv, D, "bf16")
    q, qh, kc, kh, vc, vh = q[0], qh[0], kc[0], kh[0], vc[0], vh[0]
    scale = 1 / math.sqrt(D)
    ks, kl, qb, qe = zip(*nodes)
    need = B.attn_decode_tree_workspace_size(q, kc, kv_start=ks, kv_len=kl, q_begin=qb, q_end=qe)
    ws = torch.empty(max(1, need), dtype=torch.uint8, device="cuda")
    o = torch.full((nq, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((nq, Hq), float("nan"), dtype=torch.float32, device="cuda")
    B.attn_decode_tree(q, kc, vc, o, lse, ws, kv_start=ks, kv_len=kl, q_begin=qb, q_end=qe)
    torch.cuda.synchronize()
    G = Hq // Hkv
    O_ref = np.zeros((nq, Hq, D))
    L_ref = np.full((nq, Hq), -np.inf)
    paths = []
    for i in range(nq):
        rows = np.concatenate([np.arange(s, s + n) for s, n, b, e in nodes if b <= i < e] + [np.zeros(0, int)])
        paths.append(rows)
        for h in range(Hq):
            O_ref[i, h], L_ref[i, h] = (x[0] for x in oracle.attention_head(qh[i:i + 1, h], kh[rows, h // G],
                                                                            vh[rows, h // G], scale))
    check("O", o, O_ref, O_TOL, scale_by_max=True)
    check("LSE", lse, L_ref, L_TOL)
    if case is TREE_CASES[0]:
        P = max(len(r) for r in paths)
        kp = torch.zeros((nq, P, Hkv, D), dtype=torch.bfloat16, device="cuda")
        vp = torch.zeros_like(kp)
        for i, r in enumerate(paths):
            idx = torch.from_numpy(r).cuda()
            kp[i, :len(r)] = kc[idx]
            vp[i, :len(r)] = vc[idx]
        lens = torch.tensor([len(r) for r in paths], dtype=torch.int32, device="cuda")
        o2 = torch.empty_like(o)
        l2 = torch.empty_like(lse)
        ws2 = torch.empty(B.attn_decode_workspace_size(nq, Hq, D, 4), dtype=torch.uint8, device="cuda")
        B.attn_decode_splitkv(q, kp, vp, o2, l2, ws2, n_splits=4, seqlens=lens)
        torch.cuda.synchronize()
        check("O vs split-KV decode of the paths", o, to_np(o2), O_TOL, scale_by_max=True)
        check("LSE vs split-KV decode of the paths", lse, to_np(l2), L_TOL)


def test_bwd_deterministic():
    log("bwd determinism")
    (q, k, v), _ = _inputs(107, 1, 300, 300, 2, 2, 128, "bf16")
    do, _ = seq_tensor(107, 3, 1, 300, 2, 128, "bf16")
    o, lse = shard.causal_attention_forward(q, k, v)
    r1 = shard.causal_attention_backward(q, k, v, o, do, lse)
    r2 = shard.causal_attention_backward(q, k, v, o, do, lse)
    # The DETERMINISTIC flag is accepted and changes nothing.
    dq, dk, dv = (torch.empty_like(x) for x in (q, k, v))
    dq_acc = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    ws = shard.bwd_workspace(1, 2, 300, q.device)
    B.attn_bwd(q, k, v, o, do, lse, ws, dq_acc, dk, dv, dq=dq, causal=True, compute_delta=True,
               dq_overwrite=True, finalize_dq=True, balanced=True, deterministic=True)
    torch.cuda.synchronize()
    for a, b, c in zip(r1, r2, (dq, dk, dv)):
        assert torch.equal(a, b)
        assert torch.equal(a, c)


def test_debug_sync_same_results(monkeypatch):
    """ATTN_DEBUG_SYNC only adds a wait: forward, backward and decode results are unchanged bit for bit."""
    log("ATTN_DEBUG_SYNC")
    (q, k, v), _ = _inputs(108, 1, 200, 200, 2, 2, 128, "bf16")
    do, _ = seq_tensor(108, 3, 1, 200, 2, 128, "bf16")

    def run():
        o, lse = shard.causal_attention_forward(q, k, v)
        grads = shard.causal_attention_backward(q, k, v, o, do, lse)
        qd = q[:, 0].contiguous()  # [1, 2, 128] decode queries over the cache k, v
        od = torch.empty_like(qd)
        ld = torch.empty((1, 2), dtype=torch.float32, device=q.device)
        ws = torch.empty(B.attn_decode_workspace_size(1, 2, 128, 4), dtype=torch.uint8, device=q.device)
        B.attn_decode_splitkv(qd, k, v, od, ld, ws, n_splits=4)
        torch.cuda.synchronize()
        return (o, lse, *grads, od, ld)

    ref = run()
    monkeypatch.setenv("ATTN_DEBUG_SYNC", "1")
    got = run()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


def test_log_line(monkeypatch, capfd):
    """ATTN_LOG writes one line per enqueued call, naming the call and its sizes."""
    (q, k, v), _ = _inputs(108, 1, 70, 90, 2, 1, 64, "bf16")
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, 70), dtype=torch.float32, device="cuda")
    monkeypatch.setenv("ATTN_LOG", "1")
    B.attn_fwd_partial(q, k, v, o, lse, causal=True)
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    assert "[attn] attn_fwd_partial dtype=1 batch=1 heads_q=2 heads_kv=1 seqlen_q=70 seqlen_k=90 head_dim=64 causal=1" in err


def test_nan_propagates_where_visible():
    """A NaN in one key row reaches exactly the rows that see that key (causal), and no other output
    changes: rows before it are bitwise equal to the clean run (hidden keys are masked out, never read
    into the softmax)."""
    log("NaN propagation")
    (q, k, v), _ = _inputs(115, 1, 192, 192, 2, 2, 128, "bf16")
    o0, l0 = shard.causal_attention_forward(q, k, v)
    j = 100
    k2 = k.clone()
    k2[0, j, 1, 5] = float("nan")
    o1, l1 = shard.causal_attention_forward(q, k2, v)
    torch.cuda.synchronize()
    # head 1, rows i >= j see key j: all NaN; rows before it and head 0 are unchanged bit for bit.
    assert torch.isnan(o1[0, j:, 1]).all() and torch.isnan(l1[0, 1, j:]).all()
    assert torch.equal(o1[0, :j, 1], o0[0, :j, 1]) and torch.equal(l1[0, 1, :j], l0[0, 1, :j])
    assert torch.equal(o1[0, :, 0], o0[0, :, 0]) and torch.equal(l1[0, 0], l0[0, 0])



def test_nan_propagates_other_paths():
    """The same rule on the fp32 forward, the fused chunk table, the LSE merge and split-KV decode: a NaN
    reaches the outputs that depend on it and changes nothing else bit for bit."""
    log("NaN propagation: fp32 forward, chunks, merge, decode")
    j = 100
    # fp32 forward, causal.
    (q, k, v), _ = _inputs(116, 1, 192, 192, 2, 2, 64, "f32")
    o0, l0 = torch.empty_like(q), torch.empty((1, 2, 192), dtype=torch.float32, device="cuda")
    B.attn_fwd_partial(q, k, v, o0, l0, causal=True)
    k2 = k.clone()
    k2[0, j, 1, 5] = float("nan")
    o1, l1 = torch.empty_like(q), torch.empty_like(l0)
    B.attn_fwd_partial(q, k2, v, o1, l1, causal=True)
    torch.cuda.synchronize()
    assert torch.isnan(o1[0, j:, 1]).all() and torch.isnan(l1[0, 1, j:]).all()
    assert torch.equal(o1[0, :j, 1], o0[0, :j, 1]) and torch.equal(l1[0, 1, :j], l0[0, 1, :j])
    assert torch.equal(o1[0, :, 0], o0[0, :, 0]) and torch.equal(l1[0, 0], l0[0, 0])

    # Fused chunk table: two chunks of 96 keys at positions 0 and 96; the NaN is global key 100.
    (q, k, v), _ = _inputs(117, 1, 192, 192, 2, 2, 128, "bf16")
    ks, vs = [k[:, :96], k[:, 96:]], [v[:, :96], v[:, 96:]]
    k2 = k.clone()
    k2[0, j, 1, 5] = float("nan")
    ks2 = [k2[:, :96], k2[:, 96:]]
    outs = []
    for kk in (ks, ks2):
        o = torch.empty((1, 192, 2, 128), dtype=torch.float32, device="cuda")
        lse = torch.empty((1, 2, 192), dtype=torch.float32, device="cuda")
        B.attn_fwd_chunks(q, kk, vs, o, lse, chunk_pos0=[0, 96], q_pos0=0, causal=True)
        outs.append((o, lse))
    torch.cuda.synchronize()
    (o0, l0), (o1, l1) = outs
    assert torch.isnan(o1[0, j:, 1]).all() and torch.isnan(l1[0, 1, j:]).all()
    assert torch.equal(o1[0, :j, 1], o0[0, :j, 1]) and torch.equal(l1[0, 1, :j], l0[0, 1, :j])
    assert torch.equal(o1[0, :, 0], o0[0, :, 0]) and torch.equal(l1[0, 0], l0[0, 0])

    # LSE merge: a NaN LSE in one part poisons exactly its row, also next to an empty (-inf) part.
    rng = np.random.default_rng(118)
    O = torch.from_numpy(rng.standard_normal((3, 1, 20, 2, 64)).astype(np.float32)).cuda()
    L = torch.from_numpy(rng.standard_normal((3, 1, 2, 20)).astype(np.float32)).cuda()
    L[1, 0, 0, 3] = -float("inf")
    O[1, 0, 3, 0] = 0.0
    L2 = L.clone()
    L2[2, 0, 1, 7] = float("nan")
    L2[0, 0, 0, 3] = float("nan")  # row (h 0, s 3): NaN beside an empty part
    for tree in (False, True):
        res = []
        for LL in (L, L2):
            o = torch.empty((1, 20, 2, 64), dtype=torch.float32, device="cuda")
            lse = torch.empty((1, 2, 20), dtype=torch.float32, device="cuda")
            B.attn_merge_lse(O, LL, o, lse, tree=tree)
            res.append((o, lse))
        torch.cuda.synchronize()
        (o0, l0), (o1, l1) = res
        bad = torch.zeros((2, 20), dtype=torch.bool, device="cuda")
        bad[1, 7] = bad[0, 3] = True
        assert torch.isnan(l1[0][bad]).all() and torch.isnan(o1[0].permute(1, 0, 2)[bad]).all()
        assert torch.equal(l1[0][~bad], l0[0][~bad])
        assert torch.equal(o1[0].permute(1, 0, 2)[~bad], o0[0].permute(1, 0, 2)[~bad])

    # Split-KV decode (GQA 4 -> 2): a NaN key of kv head 1 in sequence 0 reaches query heads 2 and 3 of
    # sequence 0; with that sequence cut before the key, nothing changes.
    q, _ = seq_tensor(119, 0, 2, 1, 4, 128, "bf16")
    kc, _ = seq_tensor(119, 1, 2, 1000, 2, 128, "bf16")
    vc, _ = seq_tensor(119, 2, 2, 1000, 2, 128, "bf16")
    q = q[:, 0]
    kc2 = kc.clone()
    kc2[0, 500, 1, 3] = float("nan")
    ws = torch.empty(B.attn_decode_workspace_size(2, 4, 128, 8), dtype=torch.uint8, device="cuda")
    for lens in (None, [400, 1000]):
        sl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
        res = []
        for kk in (kc, kc2):
            o = torch.empty((2, 4, 128), dtype=torch.bfloat16, device="cuda")
            lse = torch.empty((2, 4), dtype=torch.float32, device="cuda")
            B.attn_decode_splitkv(q, kk, vc, o, lse, ws, n_splits=8, seqlens=sl)
            torch.cuda.synchronize()
            res.append((o, lse))
        (o0, l0), (o1, l1) = res
        if lens is None:
            assert torch.isnan(o1[0, 2:]).all() and torch.isnan(l1[0, 2:]).all()
            assert torch.equal(o1[0, :2], o0[0, :2]) and torch.equal(l1[0, :2], l0[0, :2])
            assert torch.equal(o1[1], o0[1]) and torch.equal(l1[1], l0[1])
        else:
            assert torch.equal(o1, o0) and torch.equal(l1, l0)



def test_check_finite_reports(monkeypatch):
    """ATTN_CHECK_FINITE: clean calls return normally with unchanged results; a NaN input makes the call that
    writes the first non-finite output fail with ATTN_ERR_NONFINITE, naming the tensor and the index."""
    log("ATTN_CHECK_FINITE")
    (q, k, v), _ = _inputs(120, 1, 192, 192, 2, 2, 128, "bf16")
    do, _ = seq_tensor(120, 3, 1, 192, 2, 128, "bf16")
    o0, l0 = shard.causal_attention_forward(q, k, v)
    g0 = shard.causal_attention_backward(q, k, v, o0, do, l0)
    torch.cuda.synchronize()
    monkeypatch.setenv("ATTN_CHECK_FINITE", "1")
    # Clean inputs (fully masked rows give LSE -inf, which is allowed): no error, same bits.
    o1, l1 = shard.causal_attention_forward(q, k, v)
    g1 = shard.causal_attention_backward(q, k, v, o1, do, l1)
    for a, b in zip((o0, l0, *g0), (o1, l1, *g1)):
        assert torch.equal(a, b)
    lm = torch.empty((1, 2, 192), dtype=torch.float32, device="cuda")
    om = torch.empty((1, 192, 2, 128), dtype=torch.float32, device="cuda")
    B.attn_fwd_partial(q, k, v, om, lm, q_pos0=0, k_pos0=150, causal=True)  # rows 0..149 see no key
    assert torch.isinf(lm[0, :, :150]).all()
    # A NaN key (row 100, head 1): the forward reports o at the first row that sees it.
    k2 = k.clone()
    k2[0, 100, 1, 5] = float("nan")
    with pytest.raises(B.AttnError) as ei:
        shard.causal_attention_forward(q, k2, v)
    assert ei.value.status == B.ATTN_ERR_NONFINITE
    assert "attn_fwd_partial: non-finite value in o at (batch, seq, head, dim) = (0, 100, 1, 0)" in str(ei.value)
    # A NaN in dout (row 7, head 0): the backward reports dq_acc at the first row that holds one.
    do2 = do.clone()
    do2[0, 7, 0, 3] = float("nan")
    with pytest.raises(B.AttnError) as ei:
        shard.causal_attention_backward(q, k, v, o0, do2, l0)
    assert ei.value.status == B.ATTN_ERR_NONFINITE
    assert "attn_bwd: non-finite value in dq_acc at (batch, seq, head, dim) = (0, 7, 0, 0)" in str(ei.value)
    # Decode over a cache with one NaN value element (key 30, head 0, dim 9): o of query head 0 at dim 9.
    qd = q[:, 0].contiguous()
    v2 = v.clone()
    v2[0, 30, 0, 9] = float("nan")
    od = torch.empty_like(qd)
    ld = torch.empty((1, 2), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.attn_decode_workspace_size(1, 2, 128, 4), dtype=torch.uint8, device="cuda")
    with pytest.raises(B.AttnError) as ei:
        B.attn_decode_splitkv(qd, k, v2, od, ld, ws, n_splits=4)
    assert "attn_decode_splitkv: non-finite value in o at (batch, head, dim) = (0, 0, 9)" in str(ei.value)
    monkeypatch.delenv("ATTN_CHECK_FINITE")


# (B, Hq, Hkv, L, D, n_splits, seqlens)
DECODE_CASES = [
    (2, 8, 2, 1000, 128, 8, None),
    (3, 4, 4, 37, 128, 4, [1, 20, 37]),
    (2, 16, 2, 2048 + 17, 128, 16, None),
    (1, 2, 1, 5000, 64, 7, None),
    (2, 4, 1, 64, 128, 64, [0, 64]),
    (1, 32, 8, 16384, 128, 64, None),
    (2, 6, 2, 300, 128, 1, [300, 150]),
    # Ragged lengths (empty, one key, mid-split cut), a split length of 65 keys
    # (a last tile of one key), and 64 splits over many (batch, head) items.
    (4, 8, 8, 4133, 128, 64, [0, 1, 2000, 4133]),
    (2, 16, 4, 8192, 64, 128, [8192, 777]),
    # Deep merge trees: the most splits the boundary takes (10 levels, most of
    # them empty), more splits than keys, and split counts that carry an odd
    # node up at several levels.
    (2, 8, 2, 1500, 128, 1024, [1500, 3]),
    (1, 4, 1, 37, 64, 100, None),
    (2, 4, 2, 999, 128, 1000, None),
    (1, 8, 2, 700, 128, 5, [700]),
    # Uneven lengths run as equal-key work units (stream-K) when B * n_splits <= 1024:
    # units that span many short sequences and empty ones, every sequence empty,
    # lengths past the cache (clamped to it), the largest unit count with one long
    # sequence (about 1000 pieces in one merge tree) next to a one-key one, and
    # 64 sequences of random lengths.
    (8, 8, 2, 3000, 128, 4, [5, 0, 3000, 17, 1, 2999, 64, 0]),
    (5, 4, 1, 1000, 64, 2, [0, 0, 0, 0, 0]),
    (3, 8, 2, 500, 128, 16, [600, 0, 499]),
    (2, 8, 2, 4096, 128, 512, [4096, 1]),
    (1, 8, 2, 10000, 128, 1024, [10000]),
    (64, 4, 4, 256, 128, 16, [int(x) for x in np.random.default_rng(3).integers(0, 257, 64)]),
    (16, 32, 8, 2048, 64, 64, [128 * k for k in (5, 12, 1, 16, 9, 3, 14, 7, 11, 2, 15, 6, 10, 4, 13, 8)]),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=_ids(DECODE_CASES))
def test_decode(case):
    Bn, Hq, Hkv, L, D, ns, lens = case
    log(f"decode {case}")
    q, qh = seq_tensor(108, 0, Bn, 1, Hq, D, "bf16")
    kc, kh = seq_tensor(108, 1, Bn, L, Hkv, D, "bf16")
    vc, vh = seq_tensor(108, 2, Bn, L, Hkv, D, "bf16")
    q, qh = q[:, 0], qh[:, 0]
    scale = 1 / math.sqrt(D)
    # Lengths are clamped to [0, L] by the library; the oracle takes the clamped ones.
    O_ref, L_ref = oracle.decode(qh, kh, vh, scale, seqlens=None if lens is None else [min(x, L) for x in lens])
    o = torch.empty((Bn, Hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((Bn, Hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.attn_decode_workspace_size(Bn, Hq, D, ns), dtype=torch.uint8, device="cuda")
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    B.attn_decode_splitkv(q, kc, vc, o, lse, ws, n_splits=ns, seqlens=sl)
    torch.cuda.synchronize()
    check("decode O", o, O_ref, O_TOL, scale_by_max=True)
    check("decode LSE", lse, L_ref, L_TOL)


def test_fp32_s256_four_chunks():
    """The fp32 workload: S=256, d=64, keys in 4 chunks of 64 merged by LSE weighting, and its backward."""
    log("fp32 S=256 4 chunks")
    q, qh = seq_tensor(1, 0, 1, 256, 1, 64, "f32")
    k, kh = seq_tensor(1, 1, 1, 256, 1, 64, "f32")
    v, vh = seq_tensor(1, 2, 1, 256, 1, 64, "f32")
    do, doh = seq_tensor(1, 3, 1, 256, 1, 64, "f32")
    O_ref, L_ref = oracle.attention(qh, kh, vh, 1 / 8)
    dq_ref, dk_ref, dv_ref = oracle.attention_backward(qh, kh, vh, O_ref, doh, L_ref, 1 / 8)
    for mode in ("accumulate", "partials", "tree"):
        if mode == "accumulate":
            o, lse, _ = shard.shard_forward(q, k, v, 64)
        else:
            o, lse, _ = shard.shard_forward_partials(q, k, v, 64, tree=mode == "tree")
        torch.cuda.synchronize()
        check(f"O {mode}", o, O_ref, 1e-5)
        check(f"LSE {mode}", lse, L_ref, 1e-5)
    dq, dk, dv = shard.shard_backward(q, k, v, o, do, lse, 64)
    torch.cuda.synchronize()
    check("dQ", dq, dq_ref, 1e-5)
    check("dK", dk, dk_ref, 1e-5)
    check("dV", dv, dv_ref, 1e-5)
