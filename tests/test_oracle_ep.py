"""Pins of the expert-parallel and pilot-token oracles (CPU only).

Each check ties the oracle to something other than itself: a brute-force
enumeration from the routing, the special cases where the operation reduces to
a known one, and invariants that a dropped term, a swapped key or a wrong
index would break."""
import numpy as np
import pytest

import oracle as orc
from oracle import ep

import workloads


def _routing(T, E, k, seed):
    ids, w = workloads.random_topk(T, E, k, seed=seed)
    return ids.numpy(), w.numpy()


@pytest.mark.parametrize("T,E,k,G,seed", [(37, 8, 2, 2, 0), (200, 16, 4, 4, 1), (64, 12, 3, 3, 2), (5, 4, 4, 4, 3)])
def test_send_plan_counts_rows_by_rank(T, E, k, G, seed):
    ids, w = _routing(T, E, k, seed)
    pft = orc.build_pft(ids, w, E)
    plan = ep.ep_send_plan(pft["tokens_per_expert"], G)
    el = E // G
    # brute force: count the buffer's rows whose expert belongs to each rank
    rank_of_row = pft["expert_ids"] // el
    np.testing.assert_array_equal(plan["send_counts"], np.bincount(rank_of_row, minlength=G))
    # the runs are the buffer's contiguous expert blocks
    np.testing.assert_array_equal(plan["send_displs"], pft["expert_offsets"][::el])
    assert plan["send_displs"][-1] == T * k


def test_send_plan_rejects_uneven_split():
    with pytest.raises(ValueError):
        ep.ep_send_plan(np.ones(10, np.int32), 4)


@pytest.mark.parametrize("G,el,seed", [(1, 5, 0), (4, 1, 1), (3, 4, 2), (8, 8, 3)])
def test_recv_plan_is_the_expert_major_permutation(G, el, seed):
    rng = np.random.default_rng(seed)
    C = rng.integers(0, 6, size=(G, el))
    C[rng.random((G, el)) < 0.2] = 0  # empty (source, expert) blocks
    plan = ep.ep_recv_plan(C)
    n = int(C.sum())
    l2r, r2l = plan["local_to_recv"], plan["recv_to_local"]
    # a bijection and its inverse
    assert sorted(l2r.tolist()) == list(range(n))
    np.testing.assert_array_equal(l2r[r2l], np.arange(n))
    # brute force: label every arrival (source, expert, row), then check the
    # expert-major rows visit the labels in (expert, source, row) order
    labels = [(s, e, i) for s in range(G) for e in range(el) for i in range(C[s, e])]
    keyed = [(labels[a][1], labels[a][0], labels[a][2]) for a in l2r]
    assert keyed == sorted(keyed)
    np.testing.assert_array_equal(np.diff(plan["local_offsets"]), C.sum(axis=0))
    np.testing.assert_array_equal(np.diff(plan["recv_displs"]), C.sum(axis=1))
    if G == 1 or el == 1:  # source-major and expert-major coincide
        np.testing.assert_array_equal(l2r, np.arange(n))


@pytest.mark.parametrize("T,E,k,G,seed", [(40, 8, 2, 2, 5), (120, 16, 4, 4, 6)])
def test_emulated_exchange_gives_each_expert_its_rows(T, E, k, G, seed):
    """Emulate the alltoallv on the CPU: every rank's expert-major rows must be
    exactly the (source, token) pairs routed to each of its experts, sources
    ascending, tokens ascending within a source."""
    el = E // G
    routes = [_routing(T, E, k, seed + 17 * s) for s in range(G)]
    pfts = [orc.build_pft(ids, w, E) for ids, w in routes]
    plans = [ep.ep_send_plan(p["tokens_per_expert"], G) for p in pfts]
    for q in range(G):
        # what q receives from s: s's rows for q's experts, tagged (s, token, expert)
        recv = []
        C = np.zeros((G, el), np.int64)
        for s in range(G):
            a, b = plans[s]["send_displs"][q], plans[s]["send_displs"][q + 1]
            recv += [(s, int(pfts[s]["token_ids"][r]), int(pfts[s]["expert_ids"][r])) for r in range(a, b)]
            C[s] = pfts[s]["tokens_per_expert"][q * el:(q + 1) * el]
        plan = ep.ep_recv_plan(C)
        local = [recv[a] for a in plan["local_to_recv"]]
        for e in range(el):
            got = local[plan["local_offsets"][e]:plan["local_offsets"][e + 1]]
            want = [(s, t, q * el + e) for s in range(G) for t in range(T)
                    if q * el + e in routes[s][0][t]]
            assert got == want


@pytest.mark.parametrize("T,E,k,P,seed", [(50, 8, 2, 2, 0), (300, 16, 4, 4, 1), (64, 64, 6, 8, 2), (33, 12, 5, 3, 3)])
def test_pilots_deduplicate_per_node(T, E, k, P, seed):
    ids, _ = _routing(T, E, k, seed)
    out = ep.rbd_pilots(ids, E, P)
    N = E // P
    # brute force count: a token sends one pilot per distinct node among its experts
    per_token = [len({int(e) // P for e in ids[t]}) for t in range(T)]
    assert out["node_offsets"][-1] == sum(per_token)
    for t in range(T):
        assert np.count_nonzero(out["pilot_token_ids"] == t) == per_token[t]
    # listed by node, then token, with the node's run at its offsets
    key = out["pilot_node_ids"].astype(np.int64) * T + out["pilot_token_ids"]
    assert (np.diff(key) > 0).all()
    for nd in range(N):
        run = out["pilot_node_ids"][out["node_offsets"][nd]:out["node_offsets"][nd + 1]]
        assert (run == nd).all()
    np.testing.assert_array_equal(np.diff(out["node_offsets"]), out["node_counts"])
    # every slot's pilot carries its token to its expert's node
    s2p = out["slot_to_pilot"].reshape(T, k)
    np.testing.assert_array_equal(out["pilot_token_ids"][s2p], np.repeat(np.arange(T)[:, None], k, axis=1))
    np.testing.assert_array_equal(out["pilot_node_ids"][s2p], ids // P)


def test_pilots_special_cases():
    T, E, k = 70, 16, 4
    ids, w = _routing(T, E, k, 9)
    # one expert per node: nothing to deduplicate, the pilots are the buffer's rows
    one = ep.rbd_pilots(ids, E, 1)
    pft = orc.build_pft(ids, w, E)
    np.testing.assert_array_equal(one["pilot_token_ids"], pft["token_ids"])
    np.testing.assert_array_equal(one["node_counts"], pft["tokens_per_expert"])
    np.testing.assert_array_equal(one["slot_to_pilot"], pft["slot_to_row"])
    # a single node: one pilot per token, in token order
    single = ep.rbd_pilots(ids, E, E)
    np.testing.assert_array_equal(single["pilot_token_ids"], np.arange(T))
    np.testing.assert_array_equal(single["slot_to_pilot"].reshape(T, k), np.repeat(np.arange(T)[:, None], k, 1))
    with pytest.raises(ValueError):
        ep.rbd_pilots(ids, E, 5)
