"""Pins of the oracle's tree-shaped speculation (verify_tree / commit_tree).

A draft tree whose every draft hangs off the previous one is the linear draft chain,
so it must reproduce verify / commit exactly.  For a branching tree, draft t's output
must equal the last output of a linear verify fed only the drafts on t's root-to-node
path, and committing a path must leave the same state and the same committed ring
records as verifying and committing that path as a linear chain.
"""
import numpy as np
import pytest

from oracle import ReplayOracle
from synth import accept_counts, draft_inputs, draft_tree, get_workload, initial_state


def _wl(kind, dtype="bf16"):
    name = {"gdn": "gdn_b256", "kda": "kda_b256"}.get(kind, "m2_verify_b512")
    return get_workload(name).replace(name="tree", batch=5, n_heads=4, n_qk_heads=2 if kind != "mamba2" else 4,
                                      dv=6, dk=32, in_dtype=dtype)


def _pick(drafts, i, order):
    """Drafts of sequence i reordered as a one-sequence linear draft batch."""
    return {k: (None if v is None else v[i:i + 1, order]) for k, v in drafts.items()}


@pytest.mark.parametrize("kind", ["mamba2", "gdn", "kda"])
def test_chain_tree_is_the_linear_verify(kind):
    wl = _wl(kind)
    T = wl.t_max
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    lin, tree = ReplayOracle(wl, seqs, S0), ReplayOracle(wl, seqs, S0)
    chain = np.tile(np.arange(-1, T - 1, dtype=np.int32), (wl.batch, 1))
    for s in range(6):
        d = draft_inputs(wl, s, seqs, T)
        o_lin = lin.verify(d, T)
        o_tree = tree.verify_tree(d, T, chain)
        assert np.array_equal(o_lin, o_tree)
        a = accept_counts(wl, s, T)
        path = np.where(np.arange(T)[None, :] < a[:, None], np.arange(T)[None, :], -1).astype(np.int32)
        lin.commit(a, T)
        tree.commit_tree(path, a, T)
        assert np.array_equal(lin.S, tree.S)
        assert np.array_equal(lin.n_committed, tree.n_committed)
        for f in lin.ring:
            assert np.array_equal(lin.ring[f], tree.ring[f])
        lin.flush(wl.L)
        tree.flush(wl.L)
    assert not lin.err and not tree.err


@pytest.mark.parametrize("kind", ["mamba2", "gdn", "kda"])
def test_tree_outputs_follow_root_to_node_paths(kind):
    wl = _wl(kind)
    T = wl.t_max
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    tree = ReplayOracle(wl, seqs, S0)
    for s in range(4):
        parent, path, a = draft_tree(wl, s, T)
        d = draft_inputs(wl, 100 + s, seqs, T)
        O = tree.verify_tree(d, T, parent)
        for i in seqs:
            paths = ReplayOracle.tree_paths(parent[i])
            for t in range(T):
                one = ReplayOracle(wl.replace(batch=1), [i], tree.S[i:i + 1].astype(np.float32))
                # S is carried exactly in float64 here: start the linear reference from it
                one.S = tree.S[i:i + 1].copy()
                o_lin = one.verify(_pick(d, i, paths[t]), len(paths[t]))
                assert np.array_equal(O[i, t], o_lin[0, -1])
        tree.commit_tree(path, a, T)
        tree.flush(wl.L)
    assert not tree.err


@pytest.mark.parametrize("kind", ["mamba2", "gdn", "kda"])
def test_tree_commit_compacts_the_accepted_path(kind):
    """After commit_tree the committed window holds exactly the accepted path's records in
    consecutive slots, and S is the state after that path: the same as verifying the path
    as a linear chain and committing all of it."""
    wl = _wl(kind, dtype="fp32")
    T = wl.t_max
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    tree = ReplayOracle(wl, seqs, S0)
    for s in range(5):
        parent, path, a = draft_tree(wl, s, T)
        d = draft_inputs(wl, 200 + s, seqs, T)
        h0 = tree.n_committed - tree.n_ckpt
        tree.verify_tree(d, T, parent)
        S_before = tree.S.copy()
        nc0 = tree.n_committed.copy()
        tree.commit_tree(path, a, T)
        for i in seqs:
            lin = ReplayOracle(wl.replace(batch=1), [i])
            lin.S = S_before[i:i + 1].copy()
            k = int(a[i])
            if k:
                lin.verify(_pick(d, i, list(path[i, :k])), k)
                lin.commit(np.array([k]), k)
            assert np.array_equal(lin.S[0], tree.S[i])
            C = wl.capacity
            for j in range(k):
                slot = int((nc0[i] + j) % C)
                for f in ("alpha", "v", "k", "q") + (("beta",) if kind != "mamba2" else ()):
                    src = d[f][i, int(path[i, j])]
                    assert np.array_equal(tree.ring[f][i, slot], src)
            assert tree.n_committed[i] == nc0[i] + k
            assert h0[i] + T <= C
        tree.flush(wl.L)
    assert not tree.err


def test_invalid_trees_and_paths_are_contract_errors():
    wl = _wl("mamba2")
    T = wl.t_max
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    orc = ReplayOracle(wl, seqs, S0)
    d = draft_inputs(wl, 0, seqs, T)
    parent = np.tile(np.array([-1, 0, 0, 1], np.int32), (wl.batch, 1))
    parent[1, 2] = 2                    # a draft cannot be its own parent
    parent[2, 3] = -2                   # nor point before the committed head
    O = orc.verify_tree(d, T, parent)
    assert orc.err
    assert np.isnan(O[1]).all() and np.isnan(O[2]).all() and np.isfinite(O[0]).all()
    orc.err = False
    S = orc.S.copy()
    path = np.full((wl.batch, T), -1, np.int32)
    path[0, :2] = [0, 2]                # 2 is a child of 0: valid
    path[3, :2] = [1, 0]                # 1 is not a root
    path[4, :2] = [0, 3]                # 3 is a child of 1, not of 0
    a = np.array([2, 0, 0, 2, 2], np.int32)
    orc.commit_tree(path, a, T)
    assert orc.err
    assert orc.n_committed.tolist() == [2, 0, 0, 0, 0]
    assert np.array_equal(orc.S[3], S[3]) and np.array_equal(orc.S[4], S[4])
