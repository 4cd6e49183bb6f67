"""HIP graph capture of the compression step (through torch.cuda.CUDAGraph).

A captured rkv_compress is replayed several times on new inputs copied into
its fixed buffers, with the program's own eager work and synchronisations
between replays; every replay must equal an eager call on the same inputs,
bit for bit (the kernels' arithmetic does not depend on scheduling). The
decode loop with captured compressions must leave the same caches as the
eager loop.
"""
import numpy as np
import pytest

import parity as par
from synth import dense_case_host
from synth.decode_gen import DecodeStream

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rkv():
    import torch
    assert torch.cuda.is_available(), "gpu tests need a GPU"
    import decode_kv_cache_03_amd as mod
    return mod


CASES = [
    # (N, B, w, G, dtype, units, select_group, variant)
    (1152, 1024, 8, 4, "bf16", 16, 1, {}),                    # fused kernel
    (300, 200, 8, 2, "f32", 4, 1, {}),                        # statistics pass + team kernel
    (700, 512, 8, 5, "bf16", 8, 4, {}),                       # shared selection: three launches
    (700, 512, 8, 5, "bf16", 4, 1, dict(symmetric=True, pool="mean")),
]


@pytest.mark.parametrize("case", CASES, ids=[f"N{c[0]}-{c[4]}-g{c[6]}-{len(c[7])}v" for c in CASES])
def test_captured_compress_replays_match_eager(rkv, case):
    import torch
    n, b, w, g, dt, units, group, var = case
    cases = [dense_case_host(71 + r, 1, 1, units, g, n, b, w, 0.1, dt, 0.4, 0.02) for r in range(4)]
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    K = torch.empty((units, n, 128), dtype=tdt, device="cuda")
    V, Q = torch.empty_like(K), torch.empty((units, g, w, 128), dtype=tdt, device="cuda")
    Ko = torch.empty((units, b, 128), dtype=tdt, device="cuda")
    Vo = torch.empty_like(Ko)
    kept = torch.empty((units, b), dtype=torch.int32, device="cuda")
    ws = torch.empty(rkv.workspace_size(units, n, g, w, b, dt, select_group=group),
                     dtype=torch.uint8, device="cuda")

    def load(c):
        K.copy_(par.to_device(c.K, dt))
        V.copy_(par.to_device(c.V, dt))
        Q.copy_(par.to_device(c.Q, dt))

    def call():
        rkv.compress(K, V, Q, b, w, 0.1, K_out=Ko, V_out=Vo, kept_idx=kept, workspace=ws,
                     select_group=group, **var)

    load(cases[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for r in (1, 0, 2, 3, 1):
        load(cases[r])
        Ko.fill_(0)
        kept.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        got = (kept.clone(), Ko.clone(), Vo.clone())
        ref = rkv.compress(K, V, Q, b, w, 0.1, select_group=group, **var)   # eager, own outputs
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref.kept_idx), f"replay on inputs {r}: kept differs"
        assert par.bits_equal(got[1], ref.K_out) and par.bits_equal(got[2], ref.V_out), \
            f"replay on inputs {r}: rows differ"
        # and the eager result is the oracle's (checked on one unit per replay)
        c = cases[r]
        u = r % units
        if group == 1:
            from oracle import rkv_oracle as orc
            ref_o = orc.compress_head(c.K[u], c.V[u], c.Q[u], b, w, 0.1, **var)
            par.assert_tau_valid(got[0][u].cpu().numpy(), ref_o["Z"], n, b, w, f"replay {r}")


def test_decode_loop_with_graphs_matches_eager_loop(rkv):
    import torch
    from decode_kv_cache_03_amd.decode_loop import DecodeLoop
    batch, layers, kv_heads, gqa = 2, 2, 2, 2
    B, w, dl, steps = 64, 8, 24, 400       # 24 % 8 != 0: the query ring moves between events
    stream = DecodeStream(9, batch, layers, kv_heads, gqa, steps, coverage=0.4, max_back=64)
    eager = DecodeLoop(stream.units, gqa, kv_budget=B, window_size=w, divide_length=dl)
    graphed = DecodeLoop(stream.units, gqa, kv_budget=B, window_size=w, divide_length=dl,
                         use_graph=True)
    for t in range(steps):
        k, v, q = stream.rows(t)
        a = eager.append(k, v, q)
        g = graphed.append(k, v, q)
        assert a == g
        if a:
            torch.cuda.synchronize()
            assert torch.equal(eager.last_kept, graphed.last_kept), f"step {t}"
    torch.cuda.synchronize()
    assert eager.events == graphed.events == (steps - B - dl) // dl + 1
    assert par.bits_equal(eager.K, graphed.K) and par.bits_equal(eager.V, graphed.V)
    assert graphed._graphs[0] is not None and graphed._graphs[1] is not None
