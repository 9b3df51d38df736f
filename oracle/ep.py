"""CPU oracle of the expert-parallel data movement around the padding-free layer.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product library never imports,
links or runs anything in this directory, and this module imports nothing from
the product package.

Plain definitions in numpy and Python loops, written for checking, not speed:

* Expert parallelism ("5.4 MoE模型在分布式训练中的应用", section 专家并行:
  数据流 and All-to-All通信步骤): G ranks, rank q holds the E/G consecutive
  experts [q*E/G, (q+1)*E/G).  Dispatch sends each rank the rows routed to its
  experts; compute runs the local experts; combine sends the results back.
  The X-MoE article (adg.csdn.net), section 2.1.1 "PFT数据结构创新", sends the
  Padding-Free Token rows with an alltoallv and no padding: the rows for a rank
  are then a contiguous run of the expert-sorted buffer.
* Redundancy-Bypassing Dispatch, stage 1 (X-MoE article, section 2.2.1
  "分层冗余消除算法", Pilot Token选择): experts map to nodes by integer division
  by the experts per node; a token's k destinations are deduplicated per node;
  the pilots are the (token, node) pairs.

Readings where the pages leave the layout open (each listed in the design
notes): the receiver lays its rows out expert-major (local expert, then source
rank, then the source's own row order) so that its grouped GEMM sees each local
expert's rows contiguously; pilots are listed by node, then token, like the
Padding-Free Token buffer is listed by expert, then token.
"""
from __future__ import annotations

from typing import Dict

import numpy as np


def ep_send_plan(tokens_per_expert, G: int) -> Dict[str, np.ndarray]:
    """Rows a rank's Padding-Free Token buffer sends to each of G ranks.

    send_counts[q] = sum of tokens_per_expert over rank q's experts;
    send_displs[q] = rows before rank q's run (send_displs[G] = all rows)."""
    tpe = [int(v) for v in np.asarray(tokens_per_expert).reshape(-1)]
    E = len(tpe)
    if G < 1 or E % G:
        raise ValueError("E must be a multiple of G")
    el = E // G
    counts = []
    for q in range(G):
        c = 0
        for e in range(q * el, (q + 1) * el):
            c += tpe[e]
        counts.append(c)
    displs = [0]
    for c in counts:
        displs.append(displs[-1] + c)
    return {"send_counts": np.array(counts, np.int32), "send_displs": np.array(displs, np.int32)}


def ep_recv_plan(recv_counts) -> Dict[str, np.ndarray]:
    """Regrouping of the rows one rank receives.

    recv_counts[s, e]: rows source rank s sends for local expert e.  The rows
    arrive source-major (source s, then its experts ascending, then its own row
    order within the expert) and are laid out expert-major (local expert e,
    then source s, then the same row order).  Returns local_to_recv[m] (the
    arrival index of expert-major row m), its inverse recv_to_local,
    local_offsets [E_local + 1] and recv_displs [G + 1]."""
    C = np.asarray(recv_counts, dtype=np.int64)
    if C.ndim != 2 or (C < 0).any():
        raise ValueError("recv_counts must be a [G, E_local] matrix of counts")
    G, el = C.shape
    arrival = []
    for s in range(G):
        for e in range(el):
            for i in range(int(C[s, e])):
                arrival.append((s, e, i))
    n = len(arrival)
    # expert-major order: sort the arrival indices by (expert, source, row)
    local_to_recv = sorted(range(n), key=lambda a: (arrival[a][1], arrival[a][0], arrival[a][2]))
    recv_to_local = [0] * n
    for m, a in enumerate(local_to_recv):
        recv_to_local[a] = m
    local_offsets = [sum(1 for a in arrival if a[1] < e) for e in range(el + 1)]
    recv_displs = [sum(1 for a in arrival if a[0] < s) for s in range(G + 1)]
    return {"local_to_recv": np.array(local_to_recv, np.int32), "recv_to_local": np.array(recv_to_local, np.int32),
            "local_offsets": np.array(local_offsets, np.int32), "recv_displs": np.array(recv_displs, np.int32)}


def rbd_pilots(topk_ids, E: int, experts_per_node: int) -> Dict[str, np.ndarray]:
    """Pilot tokens of Redundancy-Bypassing Dispatch, stage 1.

    node(e) = e // experts_per_node; pilots = {(token, node(e)) : e among the
    token's k experts}, listed by node, then token.  Returns pilot_token_ids,
    pilot_node_ids, node_counts [N], node_offsets [N + 1] and slot_to_pilot
    [T*k] (the pilot that carries slot (t, j) to its expert's node)."""
    ids = np.asarray(topk_ids)
    T, k = ids.shape
    if experts_per_node < 1 or E % experts_per_node:
        raise ValueError("E must be a multiple of experts_per_node")
    N = E // experts_per_node
    pilots = set()
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if not 0 <= e < E:
                raise ValueError("expert id out of range")
            pilots.add((e // experts_per_node, t))
    order = sorted(pilots)
    where = {p: i for i, p in enumerate(order)}
    node_counts = [sum(1 for p in order if p[0] == nd) for nd in range(N)]
    node_offsets = [0]
    for c in node_counts:
        node_offsets.append(node_offsets[-1] + c)
    slot_to_pilot = [where[(int(ids[t, j]) // experts_per_node, t)] for t in range(T) for j in range(k)]
    return {"pilot_token_ids": np.array([p[1] for p in order], np.int32),
            "pilot_node_ids": np.array([p[0] for p in order], np.int32),
            "node_counts": np.array(node_counts, np.int32), "node_offsets": np.array(node_offsets, np.int32),
            "slot_to_pilot": np.array(slot_to_pilot, np.int32)}
