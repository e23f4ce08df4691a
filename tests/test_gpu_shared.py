"""GPU parity of pkv_attention_decode_shared (shared prefix read once per group)
through the C ABI against the oracle's decode attention (the definition: the
groups change which reads serve which positions, not the result).

Cases: the 176-sequence shared-prefix configuration (one group, 2048 shared
tokens) in the launch configuration its measurement times; small families with
prefixes ending inside a block, forks, several groups, group sizes beyond one
row block, head dims 64/128, group sizes G of 1 to 16; hand-built tables where
members are shorter than the shared blocks, empty sequences, a grid bound
(max_group_size) below a group's size, and a suffix-length hint too small (the
extra partitions are folded in).  Every case prints its shape first."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle.attention import attention_decode, to_f64  # noqa: E402
from oracle.replay import run_step  # noqa: E402
from oracle.shared import prefix_groups  # noqa: E402
from tests.parity import assert_gate  # noqa: E402
from workloads import config_workload, shared_prefix_workload  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from paged_attention_slot_amd import lib
    lib()


def run_wl(wl, groups_expected=None):
    from paged_attention_slot_amd.runtime import DecodeStep, to_host_bits
    say(f"  case {wl.name}: N={wl.num_seqs} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} "
        f"D={wl.head_dim} B={wl.block_size} seed={wl.seed}")
    step = DecodeStep(wl)
    step.copy()
    step.write()
    gs, pl, mg, mp, ms = step.shared_groups()
    say(f"  groups={pl.numel()} max_group={mg} max_prefix={mp} max_suffix={ms}")
    if groups_expected is not None:
        assert (gs.cpu().tolist(), pl.cpu().tolist()) == groups_expected
    step.attention_shared()
    torch.cuda.synchronize()
    got = to_f64(to_host_bits(step.out))
    ost = run_step(wl, keep_values=False)
    s0, p0 = prefix_groups(ost.block_tables, ost.seq_lens, wl.block_size)
    assert np.array_equal(s0, gs.cpu().numpy()) and np.array_equal(p0, pl.cpu().numpy())
    return got, ost.attention(), step


def test_shared_prefix_config_full():
    wl = config_workload("shared-prefix-cow")
    got, ref, _ = run_wl(wl, ([0, 176], [2048]))
    say("  gate", assert_gate(got, ref, "bf16", "shared-prefix-cow"))


@pytest.mark.parametrize("hint", [0, 2000], ids=["no-hint", "long-hint"])
def test_two_kernel_form_on_the_config(hint):
    """Without a suffix hint, or with one past what the prefix workgroups walk
    themselves, the step takes the two-kernel form (suffix pieces through the
    workspace, then the prefix kernel's combine): every element against the
    oracle, as the one-launch form."""
    from paged_attention_slot_amd import ops
    from paged_attention_slot_amd.runtime import to_host_bits
    wl = config_workload("shared-prefix-cow")
    got, ref, step = run_wl(wl, ([0, 176], [2048]))
    gs, pl, mg, mp, _ = step.shared_groups()
    n = ops.shared_workspace_bytes(wl.num_seqs, wl.num_q_heads, pl.numel(), mg, mp, hint,
                                   step.max_seq_len, step.k_caches[0])
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device=step.q.device)
    out = torch.empty_like(step.q)
    ops.attention_decode_shared(step.q, step.k_caches[0], step.v_caches[0], step.block_tables,
                                step.seq_lens, wl.scale, gs, pl, mg, mp, hint, out=out,
                                max_seq_len=step.max_seq_len, workspace=ws)
    torch.cuda.synchronize()
    two = to_f64(to_host_bits(out))
    say("  gate", assert_gate(two, ref, "bf16", f"two-kernel form, hint {hint}"))
    assert_gate(got, ref, "bf16", "one-launch form")


FAMILIES = [  # prefix, suffix lens, forking parents, samples, Hq, Hkv, D, B
    (64, [3, 16, 7, 1, 12, 30, 9], 4, 4, 16, 4, 128, 16),
    (40, [3, 9, 1, 20, 33], 2, 3, 8, 8, 128, 16),      # prefix ends inside a block
    (512, [100, 1, 37, 250], 1, 2, 32, 8, 128, 32),
    (96, [5, 8, 13] * 12, 0, 1, 16, 1, 128, 8),         # 36 members x G = 16: many row blocks
    (130, [4, 70, 9], 1, 3, 12, 4, 64, 64),
    (33, [1, 2, 3, 4, 5, 6, 7, 8, 9, 10], 3, 2, 2, 2, 64, 8),
]


@pytest.mark.parametrize("prefix,suffix,fp,spf,Hq,Hkv,D,B", FAMILIES, ids=lambda v: str(v))
def test_families(prefix, suffix, fp, spf, Hq, Hkv, D, B):
    wl = shared_prefix_workload(prefix_tokens=prefix, suffix_lens=suffix, forking_parents=fp,
                                samples_per_fork=spf, num_q_heads=Hq, num_kv_heads=Hkv,
                                head_dim=D, block_size=B, dtype="bf16", seed=prefix + B,
                                name=f"family-p{prefix}")
    # pools sized for block-aligned prefixes; a partial prefix block is
    # copied once per sharer
    extra = len(suffix) + 8
    wl.num_blocks += extra
    wl.free_order = np.random.default_rng(prefix).permutation(wl.num_blocks).astype(np.int32)
    got, ref, _ = run_wl(wl)
    assert_gate(got, ref, "bf16", wl.name)


@pytest.mark.parametrize("scale", [-0.0884, 0.0, 0.75], ids=["negative", "zero", "sharp"])
def test_family_with_unusual_scales(scale):
    """The caller's scale as it comes on both kernels of the read-once path
    (the prefix walk's two row groups, the suffix walks, the combine of their
    states): negative, zero and large enough that the references move."""
    wl = shared_prefix_workload(prefix_tokens=512, suffix_lens=[100, 1, 37, 250, 64, 3],
                                forking_parents=2, samples_per_fork=3, num_q_heads=32,
                                num_kv_heads=8, head_dim=128, block_size=32, dtype="bf16", seed=91,
                                name="family-scale")
    wl.scale = scale
    wl.num_blocks += 16
    wl.free_order = np.random.default_rng(91).permutation(wl.num_blocks).astype(np.int32)
    got, ref, _ = run_wl(wl)
    say("  gate", assert_gate(got, ref, "bf16", f"scale {scale}"))


def hand_case(tables, lens, Hq, Hkv, D, B, nb, seed):
    from paged_attention_slot_amd import ops
    rng = np.random.default_rng(seed)

    def bf(shape):
        u = rng.normal(0, 1, shape).astype(np.float32).view(np.uint32)
        return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    kp, vp = bf((nb, B, Hkv, D)), bf((nb, B, Hkv, D))
    q = bf((len(lens), Hq, D))
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)  # noqa: E731
    tables = np.asarray(tables, np.int32)
    lens = np.asarray(lens, np.int32)
    ref = attention_decode(q, kp, vp, tables, lens, 1 / np.sqrt(D))
    return ops, (t(q), t(kp), t(vp), torch.from_numpy(tables).to(dev),
                 torch.from_numpy(lens).to(dev)), ref


def test_members_shorter_than_the_shared_blocks_and_empty_sequences():
    """Sequences 0-2 hold the same three blocks with 40, 33 and 48 tokens (the
    shared prefix of 48 tokens is longer than two of them); sequence 3 is
    empty; 4-5 share one block, then differ (sequence 4 has 74 positions
    after it: more than one suffix partition of 64)."""
    from paged_attention_slot_amd.runtime import to_host_bits
    B = 16
    tables = [[5, 7, 9, -1, -1, -1]] * 3 + [[-1] * 6, [2, 3, 4, 8, 10, 11],
                                            [2, 6, -1, -1, -1, -1]]
    lens = [40, 33, 48, 0, 90, 20]
    ops, (q, kp, vp, tb, ln), ref = hand_case(tables, lens, 8, 2, 128, B, 12, 11)
    starts, plens, mg, mp, ms = ops.prefix_groups(np.asarray(tables, np.int32),
                                                  np.asarray(lens, np.int32), B)
    assert starts.tolist() == [0, 3, 4, 6] and plens.tolist() == [48, 0, 16] and ms == 74
    for bound, hint, name in ((mg, ms, "grid fits"), (1, ms, "groups beyond the grid share nothing"),
                              (mg, 1, "suffix hint too small: extra partitions folded in")):
        say(f"  hand case: max_group_size={bound} max_suffix_len={hint} ({name})")
        out = ops.attention_decode_shared(q, kp, vp, tb, ln, 1 / np.sqrt(128),
                                          torch.from_numpy(starts).cuda(),
                                          torch.from_numpy(plens).cuda(), bound, mp, hint,
                                          max_seq_len=96)
        torch.cuda.synchronize()
        got = to_f64(to_host_bits(out))
        assert_gate(got, ref, "bf16", name)
        assert not got[3].any()


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (8, 2)])
def test_groups_of_more_than_64_members_of_varying_lengths(Hq, Hkv):
    """100 sequences on the same three blocks with lengths 20..48 (the shortest
    at member 90, in the second row block for G = 1): every member masks at
    its own length, and each row block's common limit is its own shortest
    member's."""
    from paged_attention_slot_amd.runtime import to_host_bits
    B, n = 16, 100
    rng = np.random.default_rng(21)
    lens = rng.integers(24, 49, n).astype(np.int32)
    lens[90] = 20
    tables = [[5, 7, 9]] * n
    ops, (q, kp, vp, tb, ln), ref = hand_case(tables, lens, Hq, Hkv, 128, B, 12, 12)
    starts, plens, mg, mp, ms = ops.prefix_groups(np.asarray(tables, np.int32), lens, B)
    say(f"  case {n} members Hq={Hq} Hkv={Hkv}: groups={starts.tolist()} prefix={plens.tolist()}")
    out = ops.attention_decode_shared(q, kp, vp, tb, ln, 1 / np.sqrt(128),
                                      torch.from_numpy(starts).cuda(),
                                      torch.from_numpy(plens).cuda(), mg, mp, ms, max_seq_len=48)
    torch.cuda.synchronize()
    assert_gate(to_f64(to_host_bits(out)), ref, "bf16", f"{n} members")


def test_matches_the_plain_decode_kernel_on_the_config():
    """Both entry points on the same pools: each within the gate of the
    oracle, and within twice the gate of each other."""
    from paged_attention_slot_amd.runtime import to_host_bits
    wl = config_workload("shared-prefix-cow")
    got, ref, step = run_wl(wl)
    step.attention()
    torch.cuda.synchronize()
    plain = to_f64(to_host_bits(step.out))
    assert_gate(plain, ref, "bf16", "plain decode")
    assert np.max(np.abs(got - plain)) < 2 * (2e-3 + 2 ** -8)


# -- one-byte caches (pkv_attention_decode_shared_quant) ------------------------

@pytest.mark.parametrize("kind", ["fp8_e4m3", "int8"])
@pytest.mark.parametrize("fam", [0, 1, 2], ids=["forks", "partial-prefix", "large-groups"])
def test_quantized_families(kind, fam):
    from oracle.replay import run_step_quant
    from paged_attention_slot_amd.runtime import DecodeStep, to_host_bits
    prefix, suffix, fp, spf, Hq, Hkv, D, B = [FAMILIES[0], FAMILIES[1], FAMILIES[3]][fam]
    wl = shared_prefix_workload(prefix_tokens=prefix, suffix_lens=suffix, forking_parents=fp,
                                samples_per_fork=spf, num_q_heads=Hq, num_kv_heads=Hkv,
                                head_dim=D, block_size=B, dtype="bf16", seed=prefix + B + 1,
                                name=f"family-p{prefix}-{kind}")
    wl.num_blocks += len(suffix) + 8
    wl.free_order = np.random.default_rng(prefix).permutation(wl.num_blocks).astype(np.int32)
    ks, vs = (0.5, 2.0) if kind == "fp8_e4m3" else (1.0, 1.0)
    say(f"  case {wl.name}: N={wl.num_seqs} Hq={Hq} Hkv={Hkv} B={B} scales={ks},{vs}")
    step = DecodeStep(wl, kv_dtype=kind, k_scale=ks, v_scale=vs)
    step.copy()
    step.write()
    step.attention_shared()
    torch.cuda.synchronize()
    got = to_f64(to_host_bits(step.out))
    ost = run_step_quant(wl, kind, ks, vs)
    assert_gate(got, ost.attention(), "bf16", wl.name)


def test_shared_prefix_config_full_fp8():
    from oracle.replay import run_step_quant
    from paged_attention_slot_amd.runtime import DecodeStep, to_host_bits
    wl = config_workload("shared-prefix-cow")
    say(f"  case {wl.name} fp8_e4m3: N={wl.num_seqs}")
    step = DecodeStep(wl, kv_dtype="fp8_e4m3")
    step.copy()
    step.write()
    step.attention_shared()
    torch.cuda.synchronize()
    got = to_f64(to_host_bits(step.out))
    ost = run_step_quant(wl, "fp8_e4m3")
    say("  gate", assert_gate(got, ost.attention(), "bf16", "shared-prefix-cow fp8"))
