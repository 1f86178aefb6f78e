"""Graph capture of one DSA step: every replay must reproduce the eager results.

The benchmark replays a captured HIP graph of its timed steps; this test
captures `indexer -> top-k -> sparse MLA` (or the fused indexer + top-k call
and sparse MLA) once and replays it three times with other eager GPU work and
host synchronisation in between, comparing each replay bit for bit with the
eager run (every stage is deterministic).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from dsa_workloads import generate, small_config  # noqa: E402
from tests import parity  # noqa: E402

pytestmark = pytest.mark.gpu


def _snapshot(step):
    torch.cuda.synchronize()
    return {
        "logits": step.logits.cpu().numpy().copy() if step.logits is not None else None,
        "topk": step.topk_idx.cpu().numpy().copy(),
        "out": step.out.float().cpu().numpy().copy(),
        "lse": step.lse.cpu().numpy().copy(),
    }


@pytest.mark.parametrize("lens,q_lens,mla_kind,forcing,fused", [
    ([3000, 700, 5000, 64], (), "bf16", (0, 0), False),
    ([9000], (), "bf16", (0, 0), False),
    ([3000, 700, 5000], (), "fp8", (4, 32), False),          # fp8 latent cache, init/local forcing
    ([2500, 2100], (2, 2), "bf16", (0, 0), False),           # multi-token decode
    ([3000, 700, 9000, 20000], (), "bf16", (2, 16), True),   # fused indexer + top-k, forcing
    ([9000, 2500], (3, 2), "bf16", (0, 0), True),            # fused, multi-token decode
], ids=["decode", "long_row", "fp8_forced", "mtp", "fused", "fused_mtp"])
def test_graph_replays_match_eager(lens, q_lens, mla_kind, forcing, fused):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from dsa_workloads.device import make_step
    cfg = small_config(f"graph_{len(lens)}_{mla_kind}", seed=211, lens=lens, q_lens=q_lens, mla_kind=mla_kind)
    print(f"\n[graph] {cfg.name}: lens {lens} q_lens {q_lens} forcing {forcing}", flush=True)
    wl = generate(cfg)
    step = make_step(wl, fused=fused)
    step.num_init_tokens, step.num_local_tokens = forcing
    step.run()
    want = _snapshot(step)
    vis = parity.visible_of(wl)                         # per query row (multi-token rows see fewer keys)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.run()

    scratch = torch.empty(1 << 20, device="cuda")
    for r in range(3):
        # clobber every output, run unrelated eager work, then replay
        if step.logits is not None:
            step.logits.fill_(float("nan"))
        step.topk_idx.fill_(-7)
        step.out.fill_(float("nan"))
        step.lse.fill_(float("nan"))
        scratch.uniform_()
        _ = (scratch * 2.0).sum().item()
        graph.replay()
        got = _snapshot(step)
        for t, n in enumerate(vis):
            if want["logits"] is not None:
                assert np.array_equal(got["logits"][t, :n], want["logits"][t, :n]), f"replay {r}: logits row {t}"
        assert np.array_equal(got["topk"], want["topk"]), f"replay {r}: top-k"
        assert np.array_equal(got["out"], want["out"], equal_nan=True), f"replay {r}: attention output"
        assert np.array_equal(got["lse"], want["lse"], equal_nan=True), f"replay {r}: lse"
        print(f"[graph] replay {r} identical", flush=True)
