"""The decode step captured as a HIP graph (as the measurement replays it)
gives the eager step's results, replay after replay, with eager work and
synchronisations between the replays: pools and attention output compared
bit for bit (the step's kernels are deterministic and idempotent: the same
slots receive the same rows, copies re-copy unchanged sources)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from workloads import config_workload  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from paged_attention_slot_amd import lib
    lib()


@pytest.mark.parametrize("name", ["qwen3-0.6b-layer", "shared-prefix-cow", "tiny"])
def test_graph_replays_match_eager(name):
    from paged_attention_slot_amd.runtime import DecodeStep, to_host_bits
    wl = config_workload(name)
    say(f"  case {name}: N={wl.num_seqs} B={wl.block_size} dtype={wl.dtype}")
    step = DecodeStep(wl, layers=2)
    step.step(0)
    torch.cuda.synchronize()
    want = (to_host_bits(step.out).copy(), to_host_bits(step.k_caches[0]),
            to_host_bits(step.v_caches[0]))
    assert int(step.cow_pairs.shape[0]) == (48 if name == "shared-prefix-cow" else 0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.step(0)
    for r in range(4):
        step.out.zero_()                  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (to_host_bits(step.out), to_host_bits(step.k_caches[0]),
               to_host_bits(step.v_caches[0]))
        say(f"  replay {r}")
        for a, b, what in zip(got, want, ("out", "k pool", "v pool")):
            assert np.array_equal(a, b), f"replay {r}: {what} differs"
