"""GPU parity of multi-token (causal) paged attention against the CPU
oracle ("LLM inference basics and vLLM internals" §5/§6: prefill chunks and
the tokens left after a prefix-cache hit).  Bars as for decode: max-abs
2e-2 (bf16 / fp16 KV), 6e-2 (fp8 KV); one-token chunks must equal the decode
kernel bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import pools

pkv = pytest.importorskip("paged_kv_cache_51_amd")

pytestmark = pytest.mark.gpu

DEV = "cuda"
D = 128
SCALE = float(np.float32(1.0 / np.sqrt(D)))
TOL = {oracle.BF16: 2e-2, oracle.FP16: 2e-2, oracle.FP8: 6e-2}


def log(*a):
    print(*a, flush=True)


def dev16(bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if dtype == oracle.BF16 else torch.float16).to(DEV)


def devi(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def case(lengths, q_lens, H, Hkv, bs, kv, qdt, seed=0, ks=1.0, vs=1.0):
    _, r_perm, _, r_val = workloads.streams(seed)
    tabs = workloads.build_tables(lengths, bs, r_perm)
    kb = [workloads.normal_bits(r_val, (int(c), Hkv, D), qdt) for c in lengths]
    vb = [workloads.normal_bits(r_val, (int(c), Hkv, D), qdt) for c in lengths]
    kp, vp = pools.write_contiguous(kb, vb, tabs.block_tables, tabs.context_lens, Hkv, D, bs,
                                    tabs.num_blocks, kv, qdt, ks, vs)
    qs = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    q = workloads.normal_bits(r_val, (int(qs[-1]), H, D), qdt)
    return tabs, kp, vp, qs, q


def gpu_prefill(tabs, kp, vp, qs, q, qdt, kv, Hkv, bs, ks=1.0, vs=1.0, max_q=None):
    qt = dev16(q, qdt)
    out = torch.full_like(qt, float("nan"))
    ql = np.diff(qs)
    pkv.paged_attention_prefill(out, qt, torch.from_numpy(kp).to(DEV), torch.from_numpy(vp).to(DEV),
                                devi(tabs.block_tables), devi(tabs.context_lens), devi(qs),
                                int(ql.max()) if max_q is None else max_q,
                                int(tabs.context_lens.max()), Hkv, bs, kv, SCALE, ks, vs)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def check(got, want, kv, what):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - want)
    log(f"  {what}: max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
    assert err.max() <= TOL[kv], what


@pytest.mark.parametrize("kv,qdt,bs", [(oracle.BF16, oracle.BF16, 16), (oracle.FP16, oracle.FP16, 32),
                                       (oracle.FP8, oracle.BF16, 16), (oracle.FP8, oracle.FP16, 32)])
@pytest.mark.parametrize("H,Hkv", [(12, 2), (28, 4), (8, 8), (32, 2), (16, 2)])
def test_prefill_tiny(kv, qdt, bs, H, Hkv):
    G = H // Hkv
    tile = 16 // G
    lengths = [5, 17, 64, 130, 40, 1]
    # q_len: fresh prefill, ragged vs the tile, exactly a tile, many tiles, 1
    q_lens = [5, tile + 1, tile, 37, 3 * tile - 1, 1]
    ks, vs = (0.02, 0.03) if kv == oracle.FP8 else (1.0, 1.0)
    log(f"prefill tiny kv={kv} q={qdt} bs={bs} G={G} tile={tile}")
    tabs, kp, vp, qs, q = case(lengths, q_lens, H, Hkv, bs, kv, qdt, seed=G, ks=ks, vs=vs)
    want = oracle.paged_prefill(q, qdt, kp, vp, kv, tabs.block_tables, tabs.context_lens, qs,
                                Hkv, bs, SCALE, ks, vs)
    got = gpu_prefill(tabs, kp, vp, qs, q, qdt, kv, Hkv, bs, ks, vs)
    check(got, want, kv, f"G={G}")


def test_prefill_tokens_before_context_start_are_zero():
    lengths = [3, 20]
    q_lens = [6, 4]                                # seq 0: 3 tokens precede its context
    tabs, kp, vp, qs, q = case(lengths, q_lens, 8, 2, 16, oracle.BF16, oracle.BF16, seed=2)
    got = gpu_prefill(tabs, kp, vp, qs, q, oracle.BF16, oracle.BF16, 2, 16)
    want = oracle.paged_prefill(q, oracle.BF16, kp, vp, oracle.BF16, tabs.block_tables,
                                tabs.context_lens, qs, 2, 16, SCALE)
    assert np.array_equal(got[:3], np.zeros((3, 8, D)))
    check(got, want, oracle.BF16, "early tokens")


def test_prefill_staged_form_tokens_before_context_start_are_zero():
    """More than 4 query tiles (the staged kernel), with a chunk
    longer than its sequence's context."""
    lengths = [3, 40]
    q_lens = [40, 30]                              # seq 0: 37 tokens precede its context
    tabs, kp, vp, qs, q = case(lengths, q_lens, 8, 2, 16, oracle.BF16, oracle.BF16, seed=4)
    got = gpu_prefill(tabs, kp, vp, qs, q, oracle.BF16, oracle.BF16, 2, 16)
    want = oracle.paged_prefill(q, oracle.BF16, kp, vp, oracle.BF16, tabs.block_tables,
                                tabs.context_lens, qs, 2, 16, SCALE)
    assert np.array_equal(got[:37], np.zeros((37, 8, D)))
    check(got, want, oracle.BF16, "early tokens, staged form")


@pytest.mark.parametrize("kv,qdt,bs", [(oracle.BF16, oracle.BF16, 16), (oracle.FP16, oracle.FP16, 32),
                                       (oracle.FP8, oracle.BF16, 32), (oracle.FP8, oracle.FP16, 16)])
@pytest.mark.parametrize("H,Hkv", [(28, 4), (8, 8), (16, 2), (20, 4)])
def test_prefill_medium(kv, qdt, bs, H, Hkv):
    """Contexts of several hundred keys: many unit pairs walked without masks,
    odd and even unit counts, the diagonal pairs masked; chunks ragged
    against the wave tiles."""
    G = H // Hkv
    lengths = [700, 333, 1025, 96]
    q_lens = [300, 77, 512, 96]
    ks, vs = (0.02, 0.03) if kv == oracle.FP8 else (1.0, 1.0)
    log(f"prefill medium kv={kv} q={qdt} bs={bs} G={G}")
    tabs, kp, vp, qs, q = case(lengths, q_lens, H, Hkv, bs, kv, qdt, seed=10 + G, ks=ks, vs=vs)
    want = oracle.paged_prefill(q, qdt, kp, vp, kv, tabs.block_tables, tabs.context_lens, qs,
                                Hkv, bs, SCALE, ks, vs)
    got = gpu_prefill(tabs, kp, vp, qs, q, qdt, kv, Hkv, bs, ks, vs)
    check(got, want, kv, f"G={G}")


@pytest.mark.parametrize("H,Hkv", [(28, 4), (7, 1), (12, 3), (16, 2)])
def test_prefill_work_order_tied_lengths(H, Hkv):
    """The staged form takes sequences longest context first: equal context
    lengths (ranked by index), a sequence count that leaves the last band of
    sequences partial for every H_kv, and chunks of many sizes."""
    lengths = [300, 300, 128, 700, 300, 700, 45, 128, 128, 900, 45, 300, 5]
    q_lens = [300, 40, 128, 99, 17, 700, 45, 1, 64, 250, 3, 120, 5]
    log(f"prefill work order H={H} Hkv={Hkv}")
    tabs, kp, vp, qs, q = case(lengths, q_lens, H, Hkv, 16, oracle.BF16, oracle.BF16, seed=31 + Hkv)
    want = oracle.paged_prefill(q, oracle.BF16, kp, vp, oracle.BF16, tabs.block_tables, tabs.context_lens,
                                qs, Hkv, 16, SCALE)
    got = gpu_prefill(tabs, kp, vp, qs, q, oracle.BF16, oracle.BF16, Hkv, 16)
    check(got, want, oracle.BF16, f"H={H} Hkv={Hkv}")


def test_prefill_many_sequences_keep_their_order():
    """More sequences than the staged form ranks (512): they run in their own
    order, with the same results."""
    rng = np.random.default_rng(5)
    S = 520
    lengths = rng.integers(12, 80, S)
    q_lens = np.minimum(lengths, rng.integers(1, 40, S))
    log(f"prefill {S} sequences")
    tabs, kp, vp, qs, q = case(lengths.tolist(), q_lens.tolist(), 28, 4, 16, oracle.BF16, oracle.BF16, seed=41)
    want = oracle.paged_prefill(q, oracle.BF16, kp, vp, oracle.BF16, tabs.block_tables, tabs.context_lens,
                                qs, 4, 16, SCALE)
    got = gpu_prefill(tabs, kp, vp, qs, q, oracle.BF16, oracle.BF16, 4, 16)
    check(got, want, oracle.BF16, f"S={S}")


@pytest.mark.parametrize("scale", [-SCALE, 0.0, 4.0 * SCALE])
def test_prefill_staged_form_any_scale(scale):
    """The staged form applies the scale after the row maxima: a negative
    scale (query signs flipped), a zero scale (uniform weights over the
    keys each token sees) and a large one agree with the oracle."""
    lengths = [300, 77, 130]
    q_lens = [120, 77, 33]
    log(f"prefill staged scale={scale}")
    tabs, kp, vp, qs, q = case(lengths, q_lens, 28, 4, 16, oracle.BF16, oracle.BF16, seed=51)
    want = oracle.paged_prefill(q, oracle.BF16, kp, vp, oracle.BF16, tabs.block_tables, tabs.context_lens,
                                qs, 4, 16, scale)
    qt = dev16(q, oracle.BF16)
    out = torch.full_like(qt, float("nan"))
    pkv.paged_attention_prefill(out, qt, torch.from_numpy(kp).to(DEV), torch.from_numpy(vp).to(DEV),
                                devi(tabs.block_tables), devi(tabs.context_lens), devi(qs), int(max(q_lens)),
                                int(max(lengths)), 4, 16, oracle.BF16, scale, 1.0, 1.0)
    torch.cuda.synchronize()
    check(out.float().cpu().numpy().astype(np.float64), want, oracle.BF16, f"scale={scale}")


@pytest.mark.parametrize("qdt,bs", [(oracle.BF16, 16), (oracle.FP16, 32)])
def test_prefill_fp8_independent_of_max_context(qdt, bs):
    """fp8 pools in the staged form (widened to the query type by the stage
    writer): the result equals the oracle and does not depend on the
    maximum context passed (a longer table and maximum context over the
    same short sequences give the same bits)."""
    lengths = [700, 333, 1025, 96]
    q_lens = [300, 77, 512, 96]
    ks, vs = 0.02, 0.03
    tabs, kp, vp, qs, q = case(lengths, q_lens, 16, 2, bs, oracle.FP8, qdt, seed=61, ks=ks, vs=vs)
    want = oracle.paged_prefill(q, qdt, kp, vp, oracle.FP8, tabs.block_tables, tabs.context_lens, qs,
                                2, bs, SCALE, ks, vs)
    wide = 20000 // bs + 1
    bt = np.zeros((len(lengths), wide), dtype=np.int32)
    bt[:, :tabs.block_tables.shape[1]] = tabs.block_tables
    outs = []
    for max_ctx, table in [(int(max(lengths)), tabs.block_tables), (20000, bt)]:
        qt = dev16(q, qdt)
        out = torch.full_like(qt, float("nan"))
        pkv.paged_attention_prefill(out, qt, torch.from_numpy(kp).to(DEV), torch.from_numpy(vp).to(DEV),
                                    devi(table), devi(tabs.context_lens), devi(qs), int(max(q_lens)), max_ctx,
                                    2, bs, oracle.FP8, SCALE, ks, vs)
        torch.cuda.synchronize()
        outs.append(out.float().cpu().numpy().astype(np.float64))
        check(outs[-1], want, oracle.FP8, f"max_ctx={max_ctx}")
    assert np.array_equal(outs[0], outs[1])


def test_prefill_fp8_long_context_widened():
    """One sequence of 17,000 keys (fp8) with a chunk of 24 new tokens,
    beside a short one."""
    lengths = [17000, 90]
    q_lens = [24, 90]
    ks, vs = 0.02, 0.03
    log("prefill fp8 17K context")
    tabs, kp, vp, qs, q = case(lengths, q_lens, 16, 2, 16, oracle.FP8, oracle.BF16, seed=71, ks=ks, vs=vs)
    want = oracle.paged_prefill(q, oracle.BF16, kp, vp, oracle.FP8, tabs.block_tables, tabs.context_lens,
                                qs, 2, 16, SCALE, ks, vs)
    got = gpu_prefill(tabs, kp, vp, qs, q, oracle.BF16, oracle.FP8, 2, 16, ks, vs)
    check(got, want, oracle.FP8, "17K fp8")


@pytest.mark.parametrize("G,Hkv", [(3, 2), (5, 1), (9, 2), (12, 1), (16, 1), (7, 3)])
def test_prefill_group_sizes_packed_columns(G, Hkv):
    """Group sizes whose (token, head) pairs do not fill 16-column tiles with
    whole tokens: the staged form packs them across token boundaries, so a
    wave starts mid-token and its tokens' causal limits differ per column.
    Seeded random chunk and context lengths, each dtype pair."""
    r = np.random.default_rng(100 + G * 10 + Hkv)
    S = 5
    lengths = r.integers(40, 420, S)
    q_lens = np.minimum(lengths, r.integers(1, 160, S))
    q_lens[0] = lengths[0]                          # one chunk that is the whole context
    kv, qdt, bs = [(oracle.BF16, oracle.BF16, 16), (oracle.FP16, oracle.FP16, 32),
                   (oracle.FP8, oracle.BF16, 16)][G % 3]
    ks, vs = (0.02, 0.03) if kv == oracle.FP8 else (1.0, 1.0)
    log(f"prefill G={G} Hkv={Hkv} kv={kv} lengths={lengths.tolist()} q_lens={q_lens.tolist()}")
    tabs, kp, vp, qs, q = case(lengths.tolist(), q_lens.tolist(), G * Hkv, Hkv, bs, kv, qdt,
                               seed=200 + G, ks=ks, vs=vs)
    want = oracle.paged_prefill(q, qdt, kp, vp, kv, tabs.block_tables, tabs.context_lens, qs,
                                Hkv, bs, SCALE, ks, vs)
    got = gpu_prefill(tabs, kp, vp, qs, q, qdt, kv, Hkv, bs, ks, vs)
    check(got, want, kv, f"G={G}")


@pytest.mark.parametrize("kv,qdt,bs", [(oracle.BF16, oracle.BF16, 16), (oracle.FP8, oracle.FP16, 16)])
def test_prefill_repeatable(kv, qdt, bs):
    """Two launches on the same inputs give the same bits: every step of the
    kernel is a fixed function of its inputs (no timing-dependent reads)."""
    lengths = [700, 333, 1025, 96]
    q_lens = [300, 77, 512, 96]
    ks, vs = (0.02, 0.03) if kv == oracle.FP8 else (1.0, 1.0)
    tabs, kp, vp, qs, q = case(lengths, q_lens, 28, 4, bs, kv, qdt, seed=21, ks=ks, vs=vs)
    runs = [gpu_prefill(tabs, kp, vp, qs, q, qdt, kv, 4, bs, ks, vs) for _ in range(3)]
    assert np.array_equal(runs[0], runs[1]) and np.array_equal(runs[0], runs[2])


def test_prefill_empty_chunks_and_max_query_len_above_need():
    lengths = [30, 9, 50]
    q_lens = [0, 4, 0]
    tabs, kp, vp, qs, q = case(lengths, q_lens, 8, 2, 16, oracle.BF16, oracle.BF16, seed=3)
    got = gpu_prefill(tabs, kp, vp, qs, q, oracle.BF16, oracle.BF16, 2, 16, max_q=40)
    want = oracle.paged_prefill(q, oracle.BF16, kp, vp, oracle.BF16, tabs.block_tables,
                                tabs.context_lens, qs, 2, 16, SCALE)
    check(got, want, oracle.BF16, "empty chunks")


@pytest.mark.parametrize("kv", [oracle.BF16, oracle.FP8])
def test_prefill_staged_form_empty_chunks(kv):
    # the staged form (13+ query tiles) with sequences that have no new
    # tokens among them: they take part in the length ranking, and their
    # workgroups have no columns; one chunk is its whole context
    lengths = [30, 260, 50, 90, 7, 400]
    q_lens = [0, 200, 0, 90, 0, 150]
    tabs, kp, vp, qs, q = case(lengths, q_lens, 28, 4, 16, kv, oracle.BF16, seed=11)
    log(f"staged empty chunks kv={kv} lengths={lengths} q_lens={q_lens}")
    got = gpu_prefill(tabs, kp, vp, qs, q, oracle.BF16, kv, 4, 16, max_q=300)
    want = oracle.paged_prefill(q, oracle.BF16, kp, vp, kv, tabs.block_tables,
                                tabs.context_lens, qs, 4, 16, SCALE)
    check(got, want, kv, "staged form, empty chunks")


@pytest.mark.parametrize("kv", [oracle.BF16, oracle.FP8])
def test_one_token_chunks_equal_decode_bitwise(kv):
    """q_len = 1 everywhere: the multi-token kernel is the decode kernel."""
    c, tabs, _, r_val = workloads.make("qwen15b")
    Hkv, H, bs = c.num_kv_heads, c.num_heads, c.block_size
    ks = vs = 0.05 if kv == oracle.FP8 else 1.0
    kb = [workloads.normal_bits(r_val, (int(x), Hkv, D), oracle.BF16) for x in tabs.context_lens]
    vb = [workloads.normal_bits(r_val, (int(x), Hkv, D), oracle.BF16) for x in tabs.context_lens]
    S = len(tabs.context_lens)
    qb = workloads.normal_bits(r_val, (S, H, D), oracle.BF16)
    kp, vp = pools.write_contiguous(kb, vb, tabs.block_tables, tabs.context_lens, Hkv, D, bs,
                                    tabs.num_blocks, kv, oracle.BF16, ks, vs)
    mc = int(tabs.context_lens.max())
    q = dev16(qb, oracle.BF16)
    kd, vd = torch.from_numpy(kp).to(DEV), torch.from_numpy(vp).to(DEV)
    bt, cl = devi(tabs.block_tables), devi(tabs.context_lens)
    a = torch.full_like(q, float("nan"))
    # the four-wave decode form (the multi-token kernel runs four waves)
    pkv.paged_attention_decode(a, q, kd, vd, bt, cl, mc, Hkv, bs, kv, SCALE, ks, vs,
                               partition_tokens=-(-mc // bs) * bs, num_blocks=tabs.num_blocks,
                               impl=pkv.IMPL_MFMA)
    b = torch.full_like(q, float("nan"))
    pkv.paged_attention_prefill(b, q, kd, vd, bt, cl, devi(np.arange(S + 1)), 1, mc, Hkv, bs, kv,
                                SCALE, ks, vs)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_prefill_chunk_at_7b_shape_sampled():
    """A chunked-prefill step of the 7B shape (28 q / 4 kv heads): 8
    sequences, 2-6K tokens of context each, the last 256 of them new; the
    oracle checks sampled rows (first, tile edges, last) of every sequence."""
    r = np.random.default_rng(12)
    lengths = [int(x) for x in r.integers(2048, 6144, 8)]
    q_lens = [256] * 8
    H, Hkv, bs = 28, 4, 16
    log("prefill 7B-shape chunk")
    _, r_perm, _, _ = workloads.streams(12)
    tabs = workloads.build_tables(lengths, bs, r_perm)
    nbytes = pkv.layer_pool_bytes(tabs.num_blocks, Hkv, D, bs, oracle.BF16)
    kd = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    vd = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    workloads.device_fill_normal(kd, oracle.BF16, 51)
    workloads.device_fill_normal(vd, oracle.BF16, 52)
    qs = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    g = torch.Generator(device=DEV)
    g.manual_seed(13)
    qt = torch.randn(int(qs[-1]), H, D, generator=g, device=DEV).to(torch.bfloat16)
    out = torch.full_like(qt, float("nan"))
    pkv.paged_attention_prefill(out, qt, kd, vd, devi(tabs.block_tables), devi(tabs.context_lens),
                                devi(qs), 256, int(max(lengths)), Hkv, bs, oracle.BF16, SCALE)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    rows = sorted({int(qs[s]) + j for s in range(8) for j in (0, 1, 2, 127, 128, 255)})
    qb = qt.cpu().view(torch.int16).numpy().view(np.uint16)
    # the oracle for the sampled rows: one-row chunks placed at each row's position
    sub_q, sub_ctx, sub_bt = [], [], []
    for row in rows:
        s = int(np.searchsorted(qs, row, side="right") - 1)
        pos = lengths[s] - q_lens[s] + (row - int(qs[s]))
        sub_q.append(qb[row])
        sub_ctx.append(pos + 1)                    # a one-token chunk at position pos
        sub_bt.append(tabs.block_tables[s])
    want = oracle.paged_prefill(np.stack(sub_q), oracle.BF16, kd.cpu().numpy(), vd.cpu().numpy(),
                                oracle.BF16, np.stack(sub_bt), np.array(sub_ctx, np.int32),
                                np.arange(len(rows) + 1, dtype=np.int32), Hkv, bs, SCALE)
    check(got[rows], want, oracle.BF16, f"{len(rows)} sampled rows")
