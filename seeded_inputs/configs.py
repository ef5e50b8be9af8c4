"""The five workloads, as plain data.

Each entry records shapes, dtype, chunking and global positions only.  The
workload ids double as the first component of every seed.

* ``fp32_s256_4chunks``: one head, S=256, d=64, fp32, keys in 4 chunks of 64,
  non-causal, forward + backward.
* ``shard_fwd_128k``: one rank's forward share of a 131072-token causal
  sequence: 4096 queries at global offset 65536, 32 heads, d=128, bf16, keys
  in 32 chunks of 4096 processed in order.
* ``shard_bwd_128k``: the backward of that shard, dK/dV per key chunk, dQ for
  the shard, from the saved output and row log-sum-exp.
* ``decode_gqa_128k``: 16 sequences, one query each, 32 query heads over 8
  key/value heads, 131072 cached keys, 64 splits merged by a binary tree.
* ``causal_fwdbwd_32k``: causal self-attention, B=2, H=32, S=32768, d=128,
  forward + backward, 16 chunks of 2048 with each work unit pairing query
  chunk u with chunk 15-u.
"""

from __future__ import annotations

import dataclasses
import math


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    dtype: str  # "f32" or "bf16"
    B: int
    H_q: int
    H_kv: int
    S_q: int
    S_k: int
    D: int
    causal: bool
    q_pos0: int = 0
    k_pos0: int = 0
    n_chunks: int = 1  # key chunks (forward/backward) or decode splits
    decode: bool = False
    balanced: bool = False

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def chunk(self) -> int:
        return self.S_k // self.n_chunks


WORKLOADS = {
    "fp32_s256_4chunks": Workload(
        wid=1, name="fp32_s256_4chunks", dtype="f32", B=1, H_q=1, H_kv=1,
        S_q=256, S_k=256, D=64, causal=False, n_chunks=4),
    "shard_fwd_128k": Workload(
        wid=2, name="shard_fwd_128k", dtype="bf16", B=1, H_q=32, H_kv=32,
        S_q=4096, S_k=131072, D=128, causal=True, q_pos0=65536, k_pos0=0,
        n_chunks=32),
    # The backward shares the forward's tensors, so it draws with the same id.
    "shard_bwd_128k": Workload(
        wid=2, name="shard_bwd_128k", dtype="bf16", B=1, H_q=32, H_kv=32,
        S_q=4096, S_k=131072, D=128, causal=True, q_pos0=65536, k_pos0=0,
        n_chunks=32),
    "decode_gqa_128k": Workload(
        wid=4, name="decode_gqa_128k", dtype="bf16", B=16, H_q=32, H_kv=8,
        S_q=1, S_k=131072, D=128, causal=False, n_chunks=64, decode=True),
    "causal_fwdbwd_32k": Workload(
        wid=5, name="causal_fwdbwd_32k", dtype="bf16", B=2, H_q=32, H_kv=32,
        S_q=32768, S_k=32768, D=128, causal=True, n_chunks=16, balanced=True),
}

# Packed variable-length batch: causal sequences of unit * k tokens for each k
# in the order given (every k in 1..16 once), H heads of dimension D.
VARLEN_PACKED = {"wid": 6, "name": "varlen_packed_70k", "unit": 512,
                 "k": (7, 2, 12, 16, 1, 9, 4, 14, 6, 11, 3, 15, 8, 13, 5, 10), "H": 32, "D": 128}

# Tree-structured decode: a root segment shared by every query, `children`
# child segments, each with `leaves` leaf segments; one query per leaf (in
# depth-first order), GQA with H_q query heads over H_kv key/value heads.
TREE_DECODE = {"wid": 7, "name": "tree_decode_64q", "root": 32768, "children": 8, "child_len": 4096, "leaves": 8,
               "leaf_len": 512, "H_q": 32, "H_kv": 8, "D": 128}


def tree_nodes(t):
    """(kv_start, kv_len, q_begin, q_end) of every node of a TREE_DECODE-style tree, root first."""
    nodes = [(0, t["root"], 0, t["children"] * t["leaves"])]
    base = t["root"]
    for c in range(t["children"]):
        nodes.append((base + c * t["child_len"], t["child_len"], c * t["leaves"], (c + 1) * t["leaves"]))
    base += t["children"] * t["child_len"]
    for i in range(t["children"] * t["leaves"]):
        nodes.append((base + i * t["leaf_len"], t["leaf_len"], i, i + 1))
    return nodes

