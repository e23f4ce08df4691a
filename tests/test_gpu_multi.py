"""GPU parity of pkv_attention_multi (several new query tokens per sequence)
against the fp64 oracle attention_multi, through the C ABI.

Pools, block tables and queries are drawn here (bf16 values, shuffled block
ids, padded tables); every case prints its shapes and seed before running."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle.attention import attention_decode, attention_multi, to_f64  # noqa: E402
from tests.parity import assert_gate  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from paged_attention_slot_amd import lib
    lib()


def bf16_bits(x):
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def case(seed, lens, nq, Hq, Hkv, D, B, extra_blocks=5):
    rng = np.random.default_rng(seed)
    N = len(lens)
    maxb = max(1, max(-(-L // B) for L in lens))
    need = sum(-(-L // B) for L in lens)
    nb = need + extra_blocks
    perm = rng.permutation(nb).astype(np.int32)
    tables = np.full((N, maxb), -1, np.int32)
    k = 0
    for s, L in enumerate(lens):
        for b in range(-(-L // B)):
            tables[s, b] = perm[k]
            k += 1
    kp = bf16_bits(rng.normal(0, 1, (nb, B, Hkv, D)))
    vp = bf16_bits(rng.normal(0, 1, (nb, B, Hkv, D)))
    offs = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    q = bf16_bits(rng.normal(0, 1, (int(offs[-1]), Hq, D)))
    return q, offs, kp, vp, tables, np.asarray(lens, np.int32)


def run_case(seed, lens, nq, Hq, Hkv, D, B, pt=0, scale=None):
    from paged_attention_slot_amd import ops
    say(f"  case seed={seed} N={len(lens)} Hq={Hq} Hkv={Hkv} D={D} B={B} pt={pt} "
        f"lens={lens[:6]} nq={nq[:6]}")
    q, offs, kp, vp, tables, lens_a = case(seed, lens, nq, Hq, Hkv, D, B)
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    out = ops.attention_multi(dev_bf16(q), torch.from_numpy(offs).cuda(), dev_bf16(kp),
                              dev_bf16(vp), torch.from_numpy(tables).cuda(),
                              torch.from_numpy(lens_a).cuda(), scale, max(nq),
                              max_seq_len=int(max(lens)), partition_tokens=pt)
    torch.cuda.synchronize()
    got = to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16))
    ref = attention_multi(q, offs, kp, vp, tables, lens_a, scale)
    return got, ref, (q, offs, kp, vp, tables, lens_a)


SHAPES = [  # Hq, Hkv, D, B
    (16, 8, 128, 16), (32, 8, 128, 16), (64, 8, 128, 32), (8, 8, 128, 8), (16, 1, 128, 16),
    (64, 1, 128, 16), (12, 4, 64, 64), (6, 2, 64, 16), (32, 1, 64, 8),
]


@pytest.mark.parametrize("Hq,Hkv,D,B", SHAPES, ids=lambda v: str(v))
def test_chunks_of_mixed_sizes(Hq, Hkv, D, B):
    lens = [40, 1, 77, 300, 17, 5, 130]
    nq = [40, 1, 9, 33, 16, 8, 2]          # a whole prompt, decode, chunks, more queries than history
    got, ref, _ = run_case(300 + Hq + D + B, lens, nq, Hq, Hkv, D, B)
    say("  gate", assert_gate(got, ref, "bf16", "multi"))
    assert not got[sum(nq[:5]):sum(nq[:5]) + 3].any()   # positions -3..-1 of sequence 5


@pytest.mark.parametrize("Hq,Hkv,D,B", [(32, 8, 128, 16), (12, 4, 64, 32), (16, 16, 128, 8)],
                         ids=lambda v: str(v))
def test_long_prefill_chunks(Hq, Hkv, D, B):
    """Prefill-shaped chunks (hundreds of query tokens per sequence: workgroups
    of four waves with two 16-row blocks each, ragged last query block, a
    group size of 3 whose rows straddle tokens) against the oracle."""
    lens = [512, 700, 301, 64]
    nq = [512, 200, 301, 13]
    got, ref, _ = run_case(700 + Hq + D, lens, nq, Hq, Hkv, D, B)
    say("  gate", assert_gate(got, ref, "bf16", "prefill chunks"))


@pytest.mark.parametrize("scale", [-0.0884, 0.0, 0.75], ids=["negative", "zero", "sharp"])
@pytest.mark.parametrize("Hq,Hkv,D,B", [(32, 8, 128, 16), (12, 4, 64, 32), (16, 16, 128, 8)],
                         ids=lambda v: str(v))
def test_chunks_with_unusual_scales(Hq, Hkv, D, B, scale):
    """The caller's scale as it comes (negative, zero, large enough that the
    running references move often) on prefill-shaped chunks and single
    queries: the four-wave direct-load walk, the register-staged walks and the
    one-wave walk, against the oracle."""
    lens = [512, 700, 301, 64, 9]
    nq = [512, 200, 301, 13, 1]
    got, ref, _ = run_case(800 + Hq + D, lens, nq, Hq, Hkv, D, B, scale=scale)
    say("  gate", assert_gate(got, ref, "bf16", f"chunks scale {scale}"))


@pytest.mark.parametrize("pt", [32, 64, 256])
@pytest.mark.parametrize("Hq,Hkv", [(16, 8), (64, 8), (32, 32)])
def test_partitions_match_oracle(pt, Hq, Hkv):
    lens = [700, 33, 1000, 64]
    nq = [12, 33, 5, 1]
    got, ref, _ = run_case(400 + pt + Hq, lens, nq, Hq, Hkv, 128, 16, pt=pt)
    assert_gate(got, ref, "bf16", f"multi pt={pt}")


@pytest.mark.parametrize("pt", [32, 96])
def test_equal_shares_fold_partitions(pt, tuning):
    """More (query block, KV head, partition) items than the GPU holds at
    once: each workgroup takes an equal share of one history (cut at tiles,
    not at partitions) and folds it into one piece; a row merges the pieces of
    the shares that start at or before its causal limit."""
    tuning("PKV_ATTN_PARTS_PER_WG", 0)
    lens = [7500, 33, 6000, 2047, 1, 500, 7000, 4096]
    nq = [2, 1, 2, 1, 1, 2, 2, 1]
    got, ref, _ = run_case(900 + pt, lens, nq, 64, 8, 128, 16, pt=pt)
    say("  gate", assert_gate(got, ref, "bf16", f"equal shares pt={pt}"))


def test_automatic_split_on_a_long_history():
    lens = [20000, 3000]
    nq = [4, 4]
    got, ref, _ = run_case(501, lens, nq, 64, 8, 128, 32)
    assert_gate(got, ref, "bf16", "long history")


def test_empty_sequences_and_single_queries():
    lens = [10, 50, 0, 33]
    nq = [0, 1, 0, 1]
    got, ref, data = run_case(502, lens, nq, 16, 4, 128, 16)
    assert_gate(got, ref, "bf16", "sparse")
    q, offs, kp, vp, tables, lens_a = data
    # one query per sequence is decode attention
    dec = attention_decode(q, kp, vp, tables[[1, 3]], lens_a[[1, 3]], 1 / np.sqrt(128))
    assert np.allclose(ref, dec, rtol=0, atol=1e-12)


def test_bench_configuration_sampled():
    """The multi-token measurement's own launch (qwen3-0.6b layer, 4 tokens per
    sequence, automatic partitions, library-sized workspace) on sampled
    sequences: shortest, longest and four drawn ones, each against the oracle
    over that sequence's blocks."""
    import ctypes

    from paged_attention_slot_amd import lib, ops
    from paged_attention_slot_amd.runtime import DecodeStep, to_host_bits
    from workloads import config_workload, multi_queries
    wl = config_workload("qwen3-0.6b-layer")
    say(f"  case {wl.name} + 4 query tokens: N={wl.num_seqs} seed={wl.seed}")
    step = DecodeStep(wl)
    step.copy()
    step.write()
    qh, offs = multi_queries(wl, 4)
    total = int(offs[-1])
    need = lib().pkv_attention_multi_workspace_bytes(
        wl.num_seqs, wl.num_q_heads, total, 4, step.max_seq_len, 0,
        ctypes.byref(ops.geom_of(step.k_cache)))
    ws = torch.empty(max(int(need), 16), dtype=torch.uint8, device="cuda")
    out = ops.attention_multi(dev_bf16(qh), torch.from_numpy(offs).cuda(), step.k_cache,
                              step.v_cache, step.block_tables, step.seq_lens, wl.scale, 4,
                              max_seq_len=step.max_seq_len, workspace=ws)
    torch.cuda.synchronize()
    got_all = to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16))
    lens = wl.seq_lens
    rng = np.random.default_rng(7)
    sample = sorted({int(np.argmin(lens)), int(np.argmax(lens)),
                     *rng.choice(wl.num_seqs, 4, replace=False).tolist()})
    for s in sample:
        L = int(lens[s])
        nb = -(-L // wl.block_size)
        ids = torch.from_numpy(step.block_tables_h[s, :nb].astype(np.int64)).cuda()
        kp = to_host_bits(step.k_cache.index_select(0, ids))
        vp = to_host_bits(step.v_cache.index_select(0, ids))
        q = qh[offs[s]:offs[s + 1]]
        ref = attention_multi(q, np.asarray([0, q.shape[0]], np.int32), kp, vp,
                              np.arange(nb, dtype=np.int32)[None], np.asarray([L], np.int32),
                              wl.scale)
        assert_gate(got_all[offs[s]:offs[s + 1]], ref, "bf16", f"bench multi seq {s} L={L}")


# -- one-byte caches (pkv_attention_multi_quant) -------------------------------

def quant_case(seed, lens, nq, Hq, Hkv, B, kind, scale_kv=(1.0, 1.0)):
    """Codes drawn with the oracle's encoders from N(0, 1) values (FP8 with
    per-tensor scales: the encoded value is x / scale); INT8 with per-(slot,
    head) scales.  Slots past each history hold NaN scales (never read into
    an output)."""
    from oracle import quant
    D = 128
    q, offs, kp, vp, tables, lens_a = case(seed, lens, nq, Hq, Hkv, D, B)
    rng = np.random.default_rng(seed + 1)
    nb = kp.shape[0]
    x_k = rng.normal(0, 1, (nb, B, Hkv, D)).astype(np.float32)
    x_v = rng.normal(0, 1, (nb, B, Hkv, D)).astype(np.float32)
    if kind == quant.FP8:
        ks, vs = scale_kv
        return q, offs, quant.e4m3_encode(x_k / ks), quant.e4m3_encode(x_v / vs), tables, \
            lens_a, dict(k_scale=ks, v_scale=vs)
    kc, ksc = quant.int8_quantize_rows(x_k)
    vc, vsc = quant.int8_quantize_rows(x_v)
    ksc, vsc = ksc.reshape(nb * B, Hkv), vsc.reshape(nb * B, Hkv)
    used = np.zeros(nb * B, bool)
    for s, L in enumerate(lens_a):
        t = np.arange(int(L))
        used[tables[s, t // B].astype(np.int64) * B + t % B] = True
    ksc[~used] = np.nan
    vsc[~used] = np.nan
    return q, offs, kc, vc, tables, lens_a, dict(k_scales=ksc, v_scales=vsc)


@pytest.mark.parametrize("kind", ["fp8_e4m3", "int8"])
@pytest.mark.parametrize("Hq,Hkv,B,pt", [(16, 8, 16, 0), (32, 8, 16, 64), (64, 8, 32, 0),
                                          (8, 8, 8, 32), (16, 1, 16, 0)])
def test_quantized_caches_match_oracle(kind, Hq, Hkv, B, pt):
    from oracle import quant
    from paged_attention_slot_amd import ops
    lens = [40, 1, 77, 300, 17, 5, 130]
    nq = [40, 1, 9, 33, 16, 8, 2]
    scales = (0.5, 2.0) if kind == quant.FP8 else (1.0, 1.0)
    say(f"  case {kind} Hq={Hq} Hkv={Hkv} B={B} pt={pt} scales={scales}")
    q, offs, kc, vc, tables, lens_a, sc = quant_case(600 + Hq + B, lens, nq, Hq, Hkv, B, kind,
                                                     scales)
    dev = torch.device("cuda:0")
    tdt = torch.float8_e4m3fn if kind == quant.FP8 else torch.int8
    kt = torch.from_numpy(kc).to(dev).view(tdt)
    vt = torch.from_numpy(vc).to(dev).view(tdt)
    kw = {}
    if kind == quant.FP8:
        kw = dict(k_scale=sc["k_scale"], v_scale=sc["v_scale"])
    else:
        kw = dict(k_scales=torch.from_numpy(sc["k_scales"]).to(dev),
                  v_scales=torch.from_numpy(sc["v_scales"]).to(dev))
    scale = 1.0 / np.sqrt(128)
    out = ops.attention_multi(dev_bf16(q), torch.from_numpy(offs).to(dev), kt, vt,
                              torch.from_numpy(tables).to(dev), torch.from_numpy(lens_a).to(dev),
                              scale, max(nq), max_seq_len=int(max(lens)), partition_tokens=pt,
                              **kw)
    torch.cuda.synchronize()
    got = to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16))
    ref = quant.attention_multi_quant(q, offs, kc, vc, tables, lens_a, scale, kind, **sc)
    say("  gate", assert_gate(got, ref, "bf16", f"multi {kind}"))
