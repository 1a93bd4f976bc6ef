"""Seeded input generators: shapes, determinism and block-route structure."""

import numpy as np
import torch

from workloads import config_doc_lens, make_config, make_custom, qsa_routes


def test_config1_shapes_and_seed():
    a = make_config(1)
    b = make_config(1)
    assert a.T == 256 and a.q.shape == (256, 16, 576) and a.kv.shape == (256, 576)
    assert a.q_idx.shape == (256, 4, 64) and a.k_idx.shape == (256, 64) and a.w.shape == (256, 4)
    assert a.sink.shape == (16,) and a.sink.dtype == torch.float32
    assert a.q.dtype == torch.bfloat16 and a.topk == 64
    assert torch.equal(a.q.view(torch.int16), b.q.view(torch.int16))
    assert abs(a.scale - 1.0 / 24.0) < 1e-15
    # N(0,1)/sqrt(dim): std close to 1/24 for q, 1/sqrt(64) for the indexer q
    assert abs(a.q.float().std().item() - 1 / 24) < 2e-3
    assert abs(a.q_idx.float().std().item() - 1 / 8) < 5e-3


def test_config3_doc_lengths_seeded():
    lens = config_doc_lens(3)
    assert lens == config_doc_lens(3) and len(lens) == 8
    assert all(512 <= x <= 4096 for x in lens)
    assert config_doc_lens(4) == [65536] and config_doc_lens(5) == [8192] * 4


def _check_routes(routes, doc_lens):
    origin = 0
    for L in doc_lens:
        for p in range(L):
            row = routes[origin + p]
            groups = row.reshape(-1, 4)
            seen = set()
            tail_seen = False
            n_groups_used = 0
            for g in groups:
                valid = g[g >= 0]
                if len(valid) == 0:
                    assert np.all(g == -1)
                    tail_seen = tail_seen or False
                    continue
                n_groups_used += 1
                # -1 only as a suffix inside a group, ids consecutive
                nv = len(valid)
                assert np.all(g[:nv] >= 0) and np.all(g[nv:] == -1)
                assert np.all(np.diff(valid) == 1)
                loc = valid - origin
                assert loc[0] % 4 == 0 and loc.min() >= 0 and loc.max() <= p
                if nv < 4 or loc[-1] == p:
                    # the causal tail group [4*(p//4) .. p]
                    assert loc[0] == 4 * (p // 4) and loc[-1] == p
                    tail_seen = True
                else:
                    assert loc[-1] < 4 * (p // 4)  # complete causal block
                for x in valid:
                    assert x not in seen
                    seen.add(int(x))
            assert tail_seen
            assert n_groups_used == min(p // 4, groups.shape[0] - 1) + 1
        origin += L


def test_qsa_routes_structure():
    doc_lens = [70, 13, 600]
    routes = qsa_routes(doc_lens, 64, np.random.default_rng(3))
    assert routes.shape == (sum(doc_lens), 64) and routes.dtype == np.int32
    _check_routes(routes, doc_lens)


def test_config5_like_custom_routes():
    wl = make_custom([40, 33], H=12, D_qk=256, D_v=256, shared_kv=False, H_idx=0, topk=32,
                     scale=1 / 16, sink=False, seed=5, routes_width=32, value_std=1 / 16)
    assert wl.v.shape == (73, 256) and wl.routes.shape == (73, 32)
    _check_routes(wl.routes.numpy(), [40, 33])
