"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on identical
seeded inputs.  Tolerances: max-abs 2e-2 for bf16 I/O, 1e-5 for fp32 I/O; caches and
int4 codes bit-exact."""

import numpy as np
import pytest

from mixed_head_kv_amd import inputs as I
from oracle import attention as OA
from oracle import int4 as OQ

from parity_util import (TOL, compare, device_synth, fill_stack, guard_violations, host_history, oracle_decode_steps,
                         oracle_rows,
                         oracle_rows_threaded, q_rows, run_layer, say, to_f64)

pytestmark = pytest.mark.gpu


def W(name, seed, hq, hkv, D, io, S, R, ctx, steps, nr, fmt="same", layers=1, fixed=None):
    return I.Workload(name, seed, layers, hq, hkv, D, io, fmt, S, R, ctx, 0, steps, nr, fixed)


SMALL = {
    "mha_bf16": W("mha_bf16", 11, 8, 8, 128, "bf16", 8, 32, 557, 20, 3),
    "gqa_bf16": W("gqa_bf16", 12, 16, 4, 128, "bf16", 4, 64, 1024, 12, 2),
    "mha_f32_d128": W("mha_f32_d128", 13, 4, 4, 128, "f32", 2, 16, 300, 9, 2),
    "gqa_bf16_d64": W("gqa_bf16_d64", 14, 8, 2, 64, "bf16", 0, 8, 200, 7, 1),
    "mha_f32_d64_nosink": W("mha_f32_d64_nosink", 15, 2, 2, 64, "f32", 0, 1, 70, 5, 1),
    "all_streaming_bf16": W("all_streaming_bf16", 16, 4, 2, 128, "bf16", 16, 48, 400, 6, 0),
    "all_retrieval_bf16": W("all_retrieval_bf16", 17, 4, 2, 128, "bf16", 16, 48, 400, 6, 2),
    "nosink_r1_bf16": W("nosink_r1_bf16", 18, 8, 4, 128, "bf16", 0, 1, 300, 5, 1),
    # a window longer than one decode split (2048 slots): streaming decode in two splits
    # with a merge, staged prefill over a 2304-row window, the ring wrapped
    "long_window_bf16": W("long_window_bf16", 19, 8, 4, 128, "bf16", 4, 2300, 3000, 12, 2),
    # group sizes that pack 1 (G = 3) and 2 (G = 6: three workgroups per KV head) query
    # heads into a prefill workgroup
    "gqa3_bf16": W("gqa3_bf16", 24, 12, 4, 128, "bf16", 4, 64, 700, 6, 2),
    "gqa6_bf16": W("gqa6_bf16", 25, 12, 2, 128, "bf16", 4, 64, 700, 6, 1),
}
CHUNKS = {
    "mha_bf16": [100, 156, 1, 300],
    "gqa_bf16": [257, 255, 512],
    "mha_f32_d128": [64, 1, 235],
    "gqa_bf16_d64": [3, 197],
    "mha_f32_d64_nosink": [70],
    "all_streaming_bf16": [40, 360],
    "all_retrieval_bf16": [400],
    "nosink_r1_bf16": [37, 263],
    "long_window_bf16": [1000, 1900, 100],
    "gqa3_bf16": [129, 400, 71],
    "gqa6_bf16": [300, 93, 1, 200],
}


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_device_synth_matches_host_generator(torch_cuda, dtype):
    w = W("synth", 99, 4, 2, 64, dtype, 1, 1, 10, 0, 1)
    say(f"synth {dtype}")
    got = device_synth(w, 3, "k", 5, 77).cpu()
    ref = I.synth(99, 3, "k", 5, 77, 2, 64, dtype)
    if dtype == "bf16":
        got = got.view(torch_cuda.int16).numpy().view(np.uint16)
    else:
        got = got.numpy()
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("via", ["append", "prefill"])
@pytest.mark.parametrize("name", ["mha_bf16", "gqa_bf16", "mha_f32_d128", "gqa_bf16_d64"])
def test_append_then_read_is_bit_exact(torch_cuda, name, via):
    """Cache contents after the chunks went in through kv_append or through prefill (whose
    retrieval rows are written by the chunk staging launch, ragged chunk edges included)
    and a few decode steps (whose append is fused into the decode launch)."""
    w = SMALL[name]
    chunks = CHUNKS[name]
    say(f"{via}/read {name} chunks={chunks}")
    kv, _, _, total = run_layer(w, chunks, 0 if via == "append" else 3, append_only_chunks=via == "append")
    mask = w.mask(0)
    for which, kind in ((0, "k"), (1, "v")):
        hist = host_history(w, 0, kind, total)
        for g in range(w.n_kv_heads):
            if mask[g]:
                got = to_f64(kv.read(0, g, which, 0, total))
                assert np.array_equal(got, hist[:, g]), (kind, g)
            else:
                last = total - 1
                held = [p for p in range(total) if p < w.sink or last - p < w.recent]
                for p in held:
                    got = to_f64(kv.read(0, g, which, p, 1))
                    assert np.array_equal(got[0], hist[p, g]), (kind, g, p)


@pytest.mark.parametrize("via", ["append", "decode"])
def test_int4_append_codes_and_dequant_are_bit_exact(torch_cuda, via):
    """int4 codes, (scale, zero) and dequantised values after kv_append chunks, or after
    decode steps (which quantise their token inside the decode launch, 8-row V code
    blocks filled one row per step and the streaming ring wrapped)."""
    w = W("int4", 21, 8, 4, 128, "bf16", 4, 32, 0, 0, 2, fmt="int4")
    chunks, steps = ([3, 50, 8, 1, 100, 9], 0) if via == "append" else ([3, 50, 8], 45)
    total = sum(chunks) + steps
    w = w.scaled(context=sum(chunks), decode_steps=steps)
    say(f"int4 {via} chunks={chunks} steps={steps}")
    kv, _, _, _ = run_layer(w, chunks, steps, append_only_chunks=True)
    mask = w.mask(0)
    for which, kind in ((0, "k"), (1, "v")):
        raw = I.synth(w.seed, 0, kind, 0, total, w.n_kv_heads, 128, "bf16")
        codes, s, z = OQ.quantize(raw)
        deq = OQ.dequantize(codes, s, z)
        for g in range(w.n_kv_heads):
            pos = list(range(total)) if mask[g] else [p for p in range(total) if p < w.sink or total - 1 - p < w.recent]
            for a in ([pos] if mask[g] else [[p] for p in pos]):
                c_dev, m_dev = kv.read_int4(0, g, which, a[0], len(a))
                c_dev = c_dev.cpu().numpy()
                m_dev = m_dev.cpu().numpy().view(np.uint16)
                assert np.array_equal(c_dev, codes[a, g]), (kind, g, a[0])
                assert np.array_equal(m_dev[:, 0], s[a, g].view(np.uint16)), (kind, g, "scale")
                assert np.array_equal(m_dev[:, 1], z[a, g].view(np.uint16)), (kind, g, "zero")
                x = kv.read(0, g, which, a[0], len(a)).cpu().numpy()
                assert np.array_equal(x.view(np.uint32), deq[a, g].view(np.uint32)), (kind, g, "dequant")


@pytest.mark.parametrize("name", list(SMALL))
def test_prefill_and_decode_match_oracle(torch_cuda, name):
    w = SMALL[name]
    chunks = CHUNKS[name]
    say(f"prefill+decode {name} chunks={chunks} steps={w.decode_steps}")
    kv, pre, dec, total = run_layer(w, chunks, w.decode_steps)
    L = sum(chunks)
    ref = oracle_rows(w, 0, np.arange(total), total)
    compare(f"{name} prefill", to_f64(pre), ref[:L], TOL[w.io_dtype])
    compare(f"{name} decode", to_f64(dec), ref[L:], TOL[w.io_dtype])
    assert kv.length(0) == total


@pytest.mark.parametrize("name", ["gqa_bf16", "mha_bf16"])
def test_poisoned_workspace_is_cleared_by_init(torch_cuda, name):
    """Whole tiles are read past the valid length and weighted by zero; init must clear
    the workspace so stale NaN bit patterns can never reach the math."""
    from mixed_head_kv_amd import binding as B
    w = SMALL[name]
    chunks = CHUNKS[name]
    say(f"poisoned workspace {name}")
    kv = B.DuoKV.for_workload(w)
    B.duo_kv_free(kv.h)
    kv.workspace.fill_(255)
    kv.h = B.duo_kv_init(kv.cfg, kv.workspace)
    kv, pre, dec, total = run_layer(w, chunks, w.decode_steps, kv=kv)
    L = sum(chunks)
    ref = oracle_rows(w, 0, np.arange(total), total)
    compare(f"{name} prefill (poisoned)", to_f64(pre), ref[:L], TOL[w.io_dtype])
    compare(f"{name} decode (poisoned)", to_f64(dec), ref[L:], TOL[w.io_dtype])


@pytest.mark.parametrize("name", ["mha_bf16", "gqa_bf16", "all_retrieval_bf16", "gqa6_bf16"])
def test_split_key_prefill_matches_oracle(torch_cuda, monkeypatch, name):
    """Query blocks whose key range is split over two workgroups (merged by the last to
    finish) give the same result; forced on small ragged chunks here."""
    monkeypatch.setenv("DUO_PREFILL_SPLIT", "2")
    w = SMALL[name]
    chunks = CHUNKS[name]
    say(f"split prefill {name} chunks={chunks}")
    kv, pre, dec, total = run_layer(w, chunks, 2)
    L = sum(chunks)
    ref = oracle_rows(w, 0, np.arange(total), total)
    compare(f"{name} split prefill", to_f64(pre), ref[:L], TOL[w.io_dtype])
    compare(f"{name} split decode", to_f64(dec), ref[L:], TOL[w.io_dtype])


def test_int4_decode_matches_oracle(torch_cuda):
    w = W("int4_gqa", 22, 8, 4, 128, "bf16", 4, 32, 700, 10, 2, fmt="int4")
    say("int4 decode")
    kv, _, dec, total = run_layer(w, [300, 400], w.decode_steps, append_only_chunks=True)
    ref = oracle_rows(w, 0, np.arange(700, total), total)
    compare("int4 decode", to_f64(dec), ref, TOL["bf16"])


def test_decode_without_new_kv_uses_appended_token(torch_cuda):
    import torch
    w = SMALL["gqa_bf16"]
    say("decode with NULL k/v")
    kv, _, _, total = run_layer(w, [200], 0)
    q = device_synth(w, 0, "q", 0, 203)
    k = device_synth(w, 0, "k", 0, 203)
    v = device_synth(w, 0, "v", 0, 203)
    kv.append(0, k[200:203], v[200:203])
    out = kv.decode(0, q[202])
    torch.cuda.synchronize()
    ref = oracle_rows(w, 0, [202], 203)
    compare("null-kv decode", to_f64(out)[None], ref, TOL["bf16"])


def test_tiny_workload_exact_config(torch_cuda):
    """4 heads (0 and 2 retrieval), head_dim 64, fp32, 512-token causal prefill, 16 decode steps."""
    w = I.WORKLOADS["tiny_mha_f32_512"]
    say("tiny_mha_f32_512")
    kv, pre, dec, total = run_layer(w, [512], 16)
    ref = oracle_rows(w, 0, np.arange(total), total)
    compare("tiny prefill", to_f64(pre), ref[:512], TOL["f32"])
    compare("tiny decode", to_f64(dec), ref[512:], TOL["f32"])


@pytest.mark.parametrize("split", [None, "2"])
@pytest.mark.parametrize("name", ["gqa_bf16", "mha_bf16"])
def test_outputs_are_bitwise_repeatable(torch_cuda, monkeypatch, name, split):
    """Same inputs, same bits, including when query blocks are split over two workgroups
    (merged in split order whichever finishes last); 8-wavefront (GQA) and 4-wavefront
    (MHA) prefill workgroups."""
    if split:
        monkeypatch.setenv("DUO_PREFILL_SPLIT", split)
    w = SMALL[name]
    say(f"repeatability {name} split={split}")
    runs = [run_layer(w, CHUNKS[name], 5) for _ in range(3)]
    for _, p, d, _ in runs[1:]:
        assert torch_cuda.equal(runs[0][1], p) and torch_cuda.equal(runs[0][2], d)


def test_failed_calls_leave_state_unchanged(torch_cuda):
    from mixed_head_kv_amd import binding as B
    w = SMALL["mha_bf16"].scaled(context=64, decode_steps=0)
    say("error paths")
    kv = B.DuoKV.for_workload(w)
    k = device_synth(w, 0, "k", 0, 65)
    v = device_synth(w, 0, "v", 0, 65)
    q = device_synth(w, 0, "q", 0, 65)
    kv.prefill(0, q[:60], k[:60], v[:60])
    with pytest.raises(B.DuoError) as e:
        kv.prefill(0, q[:5], k[:5], v[:5])
    assert e.value.code == B.DUO_E_CAPACITY and kv.length(0) == 60
    with pytest.raises(B.DuoError) as e:
        B.duo_decode(kv.h, 0, q[0], k[0], None, q[1])
    assert e.value.code == B.DUO_E_STATE and kv.length(0) == 60
    with pytest.raises(B.DuoError) as e:
        B.duo_prefill(kv.h, 1, q, k, v, 4, q)
    assert e.value.code == B.DUO_E_INVALID
    for n in (0, -3):  # empty and negative token counts: rejected, nothing changes
        with pytest.raises(B.DuoError) as e:
            B.duo_prefill(kv.h, 0, q, k, v, n, q)
        assert e.value.code == B.DUO_E_INVALID and kv.length(0) == 60
        with pytest.raises(B.DuoError) as e:
            B.duo_kv_append(kv.h, 0, k, v, n)
        assert e.value.code == B.DUO_E_INVALID and kv.length(0) == 60
    with pytest.raises(B.DuoError) as e:
        kv.read(0, int(np.nonzero(~w.mask(0))[0][0]), 0, 20, 1)  # evicted from a streaming cache
    assert e.value.code == B.DUO_E_INVALID
    kv.prefill(0, q[60:64], k[60:64], v[60:64])
    assert kv.length(0) == 64


def test_injected_faults_leave_state_unchanged(torch_cuda, monkeypatch):
    """DUO_FAULT_INJECT makes each named call fail with DUO_E_HIP after validation and
    before any launch: the binding raises it, lengths and caches are unchanged, and the
    same calls succeed once the variable is cleared (outputs against the oracle)."""
    import torch
    from mixed_head_kv_amd import binding as B
    w = SMALL["gqa_bf16"].scaled(context=300, decode_steps=3)
    say("injected faults")
    kv = B.DuoKV.for_workload(w)
    total = 300 + 3
    q = device_synth(w, 0, "q", 0, total)
    k = device_synth(w, 0, "k", 0, total)
    v = device_synth(w, 0, "v", 0, total)
    pre = [kv.prefill(0, q[:200], k[:200], v[:200])]
    snap = kv.workspace.clone()
    monkeypatch.setenv("DUO_FAULT_INJECT", "duo_prefill,duo_kv_append,duo_decode,duo_decode_static,duo_kv_read,"
                                           "duo_prefill_seq,duo_kv_append_seq")
    out = torch.zeros_like(q[:100])
    calls = [lambda: B.duo_prefill(kv.h, 0, q[200:], k[200:], v[200:], 100, out),
             lambda: B.duo_prefill_seq(kv.h, 0, 0, q[200:], k[200:], v[200:], 100, out),
             lambda: B.duo_kv_append(kv.h, 0, k[200:], v[200:], 100),
             lambda: B.duo_kv_append_seq(kv.h, 0, 0, k[200:], v[200:], 100),
             lambda: B.duo_decode(kv.h, 0, q[200], k[200], v[200], out[0]),
             lambda: B.duo_decode_static(kv.h, 0, q[200], k[200], v[200], out[0]),
             lambda: kv.read(0, int(np.nonzero(w.mask(0))[0][0]), 0, 0, 10)]  # a retrieval head
    for call in calls:
        with pytest.raises(B.DuoError) as e:
            call()
        assert e.value.code == B.DUO_E_HIP and "fault injected" in str(e.value)
    torch.cuda.synchronize()
    assert kv.length(0) == 200 and torch.equal(kv.workspace, snap) and not out.any()
    monkeypatch.delenv("DUO_FAULT_INJECT")
    pre.append(kv.prefill(0, q[200:300], k[200:300], v[200:300]))
    dec = torch.stack([kv.decode(0, q[t], k[t], v[t]) for t in range(300, total)])
    torch.cuda.synchronize()
    ref = oracle_rows(w, 0, np.arange(total), total)
    compare("after injected faults, prefill", to_f64(torch.cat(pre)), ref[:300], TOL["bf16"])
    compare("after injected faults, decode", to_f64(dec), ref[300:], TOL["bf16"])


@pytest.mark.parametrize("name", ["gqa_bf16", "mha_bf16", "int4"])
def test_resume_from_a_saved_workspace_or_replayed_appends(torch_cuda, name):
    """Checkpoint and resume: after the prefill (int4: appends) and two decode steps the
    state is saved (workspace bytes and the per-sequence lengths).  The next decode steps
    on the original handle, on a handle attached to a copy of the saved bytes
    (duo_kv_attach), and on a fresh handle refilled by appending the same tokens are
    bitwise equal, and match the oracle."""
    import torch
    from mixed_head_kv_amd import binding as B
    if name == "int4":
        w = W("int4_resume", 26, 8, 4, 128, "bf16", 4, 32, 394, 6, 2, fmt="int4")
        chunks, append_only = [150, 244], True
    else:
        w, chunks, append_only = SMALL[name], CHUNKS[name], False
    L = sum(chunks)
    total = L + w.decode_steps
    say(f"resume {name}: {L} tokens, {w.decode_steps} decode steps")
    kv = B.DuoKV.for_workload(w)
    Q, K, V = (device_synth(w, 0, kind, 0, total) for kind in ("q", "k", "v"))
    t = 0
    for T in chunks:
        if append_only:
            kv.append(0, K[t:t + T], V[t:t + T])
        else:
            kv.prefill(0, Q[t:t + T], K[t:t + T], V[t:t + T])
        t += T
    for t in range(L, L + 2):
        kv.decode(0, Q[t], K[t], V[t])
    torch.cuda.synchronize()
    saved, lengths = kv.workspace.clone(), kv.lengths()
    assert lengths == [L + 2]

    def rest(h):
        return torch.stack([h.decode(0, Q[t], K[t], V[t]) for t in range(L + 2, total)])

    out_a = rest(kv)
    resumed = B.DuoKV.attach(kv, saved.clone(), lengths)
    out_b = rest(resumed)
    replayed = B.DuoKV.for_workload(w)
    replayed.append(0, K[:L + 2], V[:L + 2])
    out_c = rest(replayed)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b), "attached handle differs"
    assert torch.equal(out_a, out_c), "replayed appends differ"
    assert resumed.lengths() == replayed.lengths() == [total]
    compare(f"resume {name}", to_f64(out_a), oracle_rows(w, 0, np.arange(L + 2, total), total), TOL["bf16"])
    resumed.close()
    replayed.close()


@pytest.mark.parametrize("hq", [16, 4])
def test_planted_needles_dominate_like_the_oracle(torch_cuda, hq):
    """Planted needles: queries share one direction u; two retrieval-cache keys (positions
    123 and 517) and one sink key (position 2) are large multiples of u, so once visible
    they outweigh every other key by ~40-60 in log2 units.  The running maximum must jump
    far past its slack mid-sequence (prefill and decode), and the outputs must match the
    oracle on every row and head (hq = 16: 8-wavefront prefill workgroups; 4: MHA)."""
    import torch
    from mixed_head_kv_amd import binding as B
    from oracle import attention as OA
    hkv, D, S, R, L, steps = 4, 128, 4, 64, 700, 4
    total = L + steps
    g = torch.Generator().manual_seed(5)
    u = torch.randn(D, generator=g)
    q = (u + 0.1 * torch.randn(total, hq, D, generator=g)).to(torch.bfloat16)
    k = torch.randn(total, hkv, D, generator=g)
    v = torch.randn(total, hkv, D, generator=g)
    unit = u / u.norm()
    for pos, alpha in ((2, 40.0), (123, 40.0), (517, 60.0)):
        k[pos] = alpha * unit
    k, v = k.to(torch.bfloat16), v.to(torch.bfloat16)
    mask = np.array([[1, 0, 1, 0]], dtype=np.uint8)
    say(f"needles hq={hq}")
    kv = B.DuoKV(1, hq, hkv, D, S, R, total, mask)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    pre = [kv.prefill(0, qd[a:b], kd[a:b], vd[a:b]) for a, b in ((0, 300), (300, L))]
    dec = [kv.decode(0, qd[t], kd[t], vd[t]) for t in range(L, total)]
    torch.cuda.synchronize()
    got = np.concatenate([to_f64(torch.cat(pre)), to_f64(torch.stack(dec))])
    ref = OA.layer_attention(q.double().numpy(), np.arange(total), k.double().numpy(), v.double().numpy(),
                             mask[0].astype(bool), S, R)
    compare(f"needles hq={hq}", got, ref, TOL["bf16"])
    kv.close()


def test_launch_log_reports_the_plan_and_changes_nothing(torch_cuda, monkeypatch, capfd):
    """DUO_LOG=1: init, prefill and every decode step write one line of launch parameters
    to stderr (here 8-wavefront workgroups of 4 heads x 64 queries); the outputs are the
    unlogged run's, bit for bit."""
    w = SMALL["gqa_bf16"]
    say("launch log")
    _, pre0, dec0, _ = run_layer(w, [300], 2)
    torch_cuda.cuda.synchronize()
    capfd.readouterr()
    monkeypatch.setenv("DUO_LOG", "1")
    _, pre1, dec1, _ = run_layer(w, [300], 2)
    torch_cuda.cuda.synchronize()
    lines = [ln for ln in capfd.readouterr().err.splitlines() if ln.startswith("duo: ")]
    assert sum(ln.startswith("duo: init") for ln in lines) == 1, lines
    pre_lines = [ln for ln in lines if ln.startswith("duo: prefill t0=0 tokens=300")]
    assert len(pre_lines) == 1 and "workgroups of 8 wavefronts (4 heads x 64 queries)" in pre_lines[0], lines
    assert sum(ln.startswith("duo: duo_decode layer=0 t=30") for ln in lines) == 2, lines
    assert torch_cuda.equal(pre0, pre1) and torch_cuda.equal(dec0, dec1)


def test_guard_band_check_sees_a_stray_write(torch_cuda):
    """The guard bands sit between the workspace's regions and hold the pattern after
    init and after work; a byte written into one (here from the host side, the way a
    kernel writing past its region would) is reported."""
    from mixed_head_kv_amd import binding as B
    w = SMALL["gqa_bf16"].scaled(context=200, decode_steps=2)
    say("guard bands")
    kv, _, _, _ = run_layer(w, [198], 2)
    offs = B.duo_kv_guard_bands(kv.h)
    assert offs == sorted(offs) and len(set(offs)) == len(offs)
    assert all(o % 256 == 0 and o + B.DUO_GUARD_BYTES <= kv.nbytes for o in offs)
    assert len(offs) == 4 * w.n_layers + 5  # K and V of both cache kinds per layer; scratch, counters, staging
    assert guard_violations(kv) == []
    o = offs[len(offs) // 2] + 77
    saved = int(kv.workspace[o])
    kv.workspace[o] = saved ^ 0x40
    assert guard_violations(kv) == [o - 77]
    kv.workspace[o] = saved
    assert guard_violations(kv) == []


def test_llama2_7b_mha_32k_layer(torch_cuda):
    """32 heads (8 retrieval), head_dim 128, bf16, 8 prefill chunks of 4096 and 128 decode
    steps.  Every prefill and every decode output of every head is checked."""
    w = I.WORKLOADS["llama2_7b_mha_32k"]
    say("llama2_7b_mha_32k")
    chunks = [w.prefill_chunk] * (w.context // w.prefill_chunk)
    kv, pre, dec, total = run_layer(w, chunks, w.decode_steps)
    got = np.concatenate([to_f64(pre), to_f64(dec)], 0)
    say("  oracle: every row of every head")
    ref = oracle_rows_threaded(w, 0, np.arange(total), total)
    compare("32k prefill (every row)", got[:w.context], ref[:w.context], TOL["bf16"])
    compare("32k decode (every step)", got[w.context:], ref[w.context:], TOL["bf16"])


def test_llama3_8b_gqa_128k_layer(torch_cuda):
    """32 query / 8 KV heads (4 retrieval), head_dim 128, bf16, 16 prefill chunks of 8192
    and 256 decode steps.  Checked, all heads: every decode step; prefill rows: the whole
    first chunk, the last 256 rows of the last chunk, +-R rows around every chunk
    boundary, and 256 seeded rows per chunk."""
    w = I.WORKLOADS["llama3_8b_gqa_128k"]
    say("llama3_8b_gqa_128k")
    chunks = [w.prefill_chunk] * (w.context // w.prefill_chunk)
    kv, pre, dec, total = run_layer(w, chunks, w.decode_steps)
    rng = np.random.default_rng(1)
    rows = set(range(w.prefill_chunk)) | set(range(w.context - 256, w.context))
    for c in range(len(chunks)):
        a, b = c * w.prefill_chunk, (c + 1) * w.prefill_chunk
        rows |= set(range(max(0, a - w.recent), min(w.context, a + w.recent)))
        rows |= set(rng.integers(a, b, 256).tolist())
    rows = np.array(sorted(rows))
    say(f"  oracle: {len(rows)} prefill rows and {w.decode_steps} decode steps, all heads")
    ref = oracle_rows_threaded(w, 0, np.concatenate([rows, np.arange(w.context, total)]), total)
    compare("128k decode (every step)", to_f64(dec), ref[len(rows):], TOL["bf16"])
    compare("128k prefill (sampled rows)", to_f64(pre[rows]), ref[:len(rows)], TOL["bf16"])
    assert np.isfinite(to_f64(dec)).all() and np.isfinite(to_f64(pre)).all()


@pytest.mark.parametrize("name", ["mha", "gqa"])
def test_one_call_prefill_of_a_long_prompt(torch_cuda, name):
    """A whole prompt in one prefill call: 32768 tokens of the 32K MHA layer (8 of 32 heads
    retrieval; 256 query blocks per head, the streaming heads' keys staged in 8 passes
    inside the call) or 16384 tokens of a GQA layer with 4 query heads per KV head
    (8-wavefront workgroups), then 4 decode steps.  Checked, all heads: every decode step;
    prefill rows: the first and last 256, +-R rows around every 4096-row staging pass, and
    512 seeded rows."""
    w = {
        "mha": W("oneshot_mha", 81, 32, 32, 128, "bf16", 64, 256, 32768 + 4, 4, 8),
        "gqa": W("oneshot_gqa", 82, 32, 8, 128, "bf16", 64, 256, 16384 + 4, 4, 4),
    }[name]
    L = w.context - w.decode_steps
    say(f"one-call prefill {name}: {L} tokens")
    kv, pre, dec, total = run_layer(w, [L], w.decode_steps)
    rng = np.random.default_rng(7)
    rows = set(range(256)) | set(range(L - 256, L)) | set(rng.integers(0, L, 512).tolist())
    for a in range(4096, L, 4096):
        rows |= set(range(a - w.recent, min(L, a + w.recent)))
    rows = np.array(sorted(rows))
    say(f"  oracle: {len(rows)} prefill rows and {w.decode_steps} decode steps, all heads")
    ref = oracle_rows_threaded(w, 0, np.concatenate([rows, np.arange(L, total)]), total)
    compare(f"one-call {name} decode", to_f64(dec), ref[len(rows):], TOL["bf16"])
    compare(f"one-call {name} prefill (sampled rows)", to_f64(pre[rows]), ref[:len(rows)], TOL["bf16"])
    assert np.isfinite(to_f64(pre)).all()


STACK_LAYERS = (0, 15, 31)


def _stack_decode_check(torch_cuda, name, steps):
    """Fill every layer to the workload's context with kv_append, decode `steps` tokens
    through all 32 layers; layers 0, 15 and 31 are checked on every KV head (all query
    heads) at every step, every other layer finite at every step."""
    from mixed_head_kv_amd.binding import DuoKV
    w = I.WORKLOADS[name].scaled(decode_steps=steps)
    say(f"{name}: fill {w.n_layers} layers x {w.context} tokens")
    kv = DuoKV.for_workload(w)
    fill_stack(w, kv)
    outs = {l: [] for l in STACK_LAYERS}
    qs = {l: [] for l in STACK_LAYERS}
    for s in range(steps):
        t = w.context + s
        for layer in range(w.n_layers):
            q = device_synth(w, layer, "q", t, 1)[0]
            k = device_synth(w, layer, "k", t, 1)[0]
            v = device_synth(w, layer, "v", t, 1)[0]
            o = kv.decode(layer, q, k, v)
            if layer in outs:
                outs[layer].append(to_f64(o))
                qs[layer].append(q.cpu().view(torch_cuda.int16).numpy().view(np.uint16))
            else:
                assert torch_cuda.isfinite(o.float()).all(), (layer, s)
    kv.close()
    for layer in STACK_LAYERS:
        say(f"  oracle: layer {layer}, all 8 KV heads, {steps} steps")
        ref = oracle_decode_steps(w, layer, w.context, steps, list(range(w.n_kv_heads)), np.stack(qs[layer]))
        got = np.stack(outs[layer])  # [steps, Hq, D]
        refa = np.stack([ref[h] for h in range(w.n_q_heads)], 1)
        compare(f"{name} layer {layer} decode ({steps} steps)", got, refa, TOL["bf16"])


def test_llama3_8b_gqa_32layer_1m_stack(torch_cuda):
    """32-layer GQA stack, 1,048,576-token bf16 caches filled by kv_append, 8 decode
    steps through all layers."""
    _stack_decode_check(torch_cuda, "llama3_8b_gqa_32layer_1m", 8)


def test_llama3_8b_gqa_32layer_int4_3p3m_stack(torch_cuda):
    """32-layer GQA stack, 3,300,000-token int4 caches (quantised by kv_append), 8 decode
    steps through all layers."""
    _stack_decode_check(torch_cuda, "llama3_8b_gqa_32layer_int4_3p3m", 8)


def _ramped_inputs(w, total, growth):
    """Seeded Q, K, V with every key scaled by 1 + growth * t / total (bf16-rounded on the
    host): scores grow along the sequence, so the running maximum keeps rising."""
    ramp = (1.0 + growth * np.arange(total) / total)[:, None, None].astype(np.float32)
    qf = I.values_f32(w.seed, 0, np.arange(total * w.n_q_heads * w.head_dim, dtype=np.uint64))
    kf = I.values_f32(w.seed, 1, np.arange(total * w.n_kv_heads * w.head_dim, dtype=np.uint64))
    vf = I.values_f32(w.seed, 2, np.arange(total * w.n_kv_heads * w.head_dim, dtype=np.uint64))
    q = I.f32_to_bf16_bits(qf.reshape(total, w.n_q_heads, w.head_dim))
    k = I.f32_to_bf16_bits(kf.reshape(total, w.n_kv_heads, w.head_dim) * ramp)
    v = I.f32_to_bf16_bits(vf.reshape(total, w.n_kv_heads, w.head_dim))
    return q, k, v


@pytest.mark.parametrize("split", [None, "2"])
def test_growing_scores_exercise_the_rescale(torch_cuda, monkeypatch, split):
    """Keys grow 5x in magnitude along the sequence, so the running max outgrows the
    reference by more than the lazy-rescale slack many times (prefill, split-key prefill
    and decode); results must still match the oracle."""
    import torch
    from mixed_head_kv_amd.binding import DuoKV
    if split:
        monkeypatch.setenv("DUO_PREFILL_SPLIT", split)
    w = W("ramp_gqa", 31, 16, 4, 128, "bf16", 4, 64, 1536, 6, 2)
    chunks = [512, 1024]
    total = sum(chunks) + w.decode_steps
    say(f"growing scores split={split}")
    q, k, v = _ramped_inputs(w, total, 4.0)
    dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    Q, K, V = dev(q), dev(k), dev(v)
    kv = DuoKV.for_workload(w)
    pre, t = [], 0
    for T in chunks:
        pre.append(kv.prefill(0, Q[t:t + T], K[t:t + T], V[t:t + T]))
        t += T
    dec = []
    for _ in range(w.decode_steps):
        dec.append(kv.decode(0, Q[t], K[t], V[t]))
        t += 1
    torch.cuda.synchronize()
    up = lambda a: OA.upcast(a, "bf16")
    ref = OA.layer_attention(up(q), np.arange(total), up(k), up(v), w.mask(0), w.sink, w.recent)
    L = sum(chunks)
    compare("ramp prefill", to_f64(torch.cat(pre, 0)), ref[:L], TOL["bf16"])
    compare("ramp decode", to_f64(torch.stack(dec, 0)), ref[L:], TOL["bf16"])


@pytest.mark.parametrize("chunks", [[350, 4550], [4900]])
def test_streaming_prefill_over_several_staged_launches(torch_cuda, chunks):
    """A chunk longer than one staged launch (4096 queries) of the streaming heads: the
    second launch's window starts inside the first launch's queries (and, for the later
    chunk, reaches back into the constant-length cache).  Every streaming-head output is
    checked; retrieval heads on 96 sampled rows plus the launch boundary."""
    w = W("long_chunk", 41, 8, 4, 128, "bf16", 4, 300, sum(chunks), 2, 1)
    say(f"staged streaming prefill chunks={chunks}")
    kv, pre, dec, total = run_layer(w, chunks, w.decode_steps)
    L = sum(chunks)
    G = w.group
    mask = w.mask(0)
    str_heads = [h for h in range(w.n_q_heads) if not mask[h // G]]
    ret_heads = [h for h in range(w.n_q_heads) if mask[h // G]]
    ref = oracle_rows(w, 0, np.arange(L), total, heads=str_heads)
    compare("staged streaming prefill (all rows)", to_f64(pre)[:, str_heads], ref[:, str_heads], TOL["bf16"])
    boundary = chunks[0] + 4096 if len(chunks) > 1 else 4096
    rows = np.unique(np.concatenate([np.random.default_rng(5).integers(0, L, 96),
                                     np.arange(boundary - 4, boundary + 4)]))
    ref_r = oracle_rows(w, 0, rows, total, heads=ret_heads)
    compare("staged prefill retrieval heads (sampled)", to_f64(pre[rows])[:, ret_heads], ref_r[:, ret_heads],
            TOL["bf16"])
    ref_d = oracle_rows(w, 0, np.arange(L, total), total)
    compare("decode after staged prefill", to_f64(dec), ref_d, TOL["bf16"])


def _batched_run(w, B_, chunks, steps, append_only=False):
    """Prefill (or append) and decode B_ sequences together; sequence b's data is the
    workload reseeded with seed + 100 b (the retrieval heads are fixed, so all sequences
    share one configuration)."""
    import torch
    from mixed_head_kv_amd.binding import DuoKV
    ws = [w.scaled(seed=w.seed + 100 * b) for b in range(B_)]
    total = sum(chunks) + steps
    Q = torch.stack([device_synth(x, 0, "q", 0, total) for x in ws])
    K = torch.stack([device_synth(x, 0, "k", 0, total) for x in ws])
    V = torch.stack([device_synth(x, 0, "v", 0, total) for x in ws])
    kv = DuoKV.for_workload(w, batch=B_)
    pre, t = [], 0
    for T in chunks:
        sl = slice(t, t + T)
        if append_only:
            kv.append(0, K[:, sl].contiguous(), V[:, sl].contiguous())
        else:
            pre.append(kv.prefill(0, Q[:, sl].contiguous(), K[:, sl].contiguous(), V[:, sl].contiguous()))
        t += T
    dec = []
    for _ in range(steps):
        dec.append(kv.decode(0, Q[:, t].contiguous(), K[:, t].contiguous(), V[:, t].contiguous()))
        t += 1
    torch.cuda.synchronize()
    return ws, kv, (torch.cat(pre, 1) if pre else None), torch.stack(dec, 1), total


@pytest.mark.parametrize("name", ["gqa_bf16", "mha_bf16", "mha_f32_d128", "int4", "long_chunk", "long_chunk_g4"])
def test_batched_sequences_match_oracle(torch_cuda, name):
    """Several sequences in one handle: every sequence's prefill and decode outputs and its
    caches checked against the oracle on that sequence's own data (long_chunk: two
    sequences, one chunk of 4600 tokens, so the streaming heads take two staged launches;
    long_chunk_g4 the same with 4 query heads per KV head: an 8-wavefront main launch, a
    4-wavefront streaming-only launch and the caches' update in a launch of its own)."""
    B_ = 3
    if name == "int4":
        w = W("int4_b", 23, 8, 4, 128, "bf16", 4, 32, 400, 6, 2, fmt="int4", fixed=(0, 3))
        chunks, append_only = [150, 250], True
    elif name == "long_chunk":
        w = W("long_chunk_b", 42, 8, 4, 128, "bf16", 4, 300, 4600, 2, 1, fixed=(1,))
        chunks, append_only, B_ = [4600], False, 2
    elif name == "long_chunk_g4":
        w = W("long_chunk_g4_b", 43, 16, 4, 128, "bf16", 4, 300, 4600, 2, 1, fixed=(2,))
        chunks, append_only, B_ = [4600], False, 2
    else:
        base = SMALL[name]
        w = base.scaled(fixed_retrieval=tuple(int(g) for g in np.flatnonzero(base.mask(0))))
        chunks, append_only = CHUNKS[name], False
    say(f"batched {name} B={B_} chunks={chunks} steps={w.decode_steps}")
    ws, kv, pre, dec, total = _batched_run(w, B_, chunks, w.decode_steps, append_only)
    L = sum(chunks)
    tol = TOL[w.io_dtype]
    for b, wb in enumerate(ws):
        ref = oracle_rows(wb, 0, np.arange(0 if pre is not None else L, total), total)
        if pre is not None:
            compare(f"batched {name} seq {b} prefill", to_f64(pre[b]), ref[:L], tol)
            compare(f"batched {name} seq {b} decode", to_f64(dec[b]), ref[L:], tol)
        else:
            compare(f"batched {name} seq {b} decode", to_f64(dec[b]), ref, tol)
        if name != "int4":
            hist = host_history(wb, 0, "k", total)
            g = int(np.flatnonzero(wb.mask(0))[0])
            got = to_f64(kv.read(0, g, 0, 0, total, b=b))
            assert np.array_equal(got, hist[:, g]), (name, b, "retrieval K cache")


@pytest.mark.parametrize("name", ["gqa_bf16", "mha_bf16"])
def test_batched_split_key_prefill_matches_oracle(torch_cuda, monkeypatch, name):
    """Three sequences with every query block's keys split over two workgroups (forced):
    the split partials and arrival counters of each sequence's blocks are kept apart, on
    8-wavefront (GQA) and 4-wavefront (MHA) workgroups."""
    monkeypatch.setenv("DUO_PREFILL_SPLIT", "2")
    base = SMALL[name]
    w = base.scaled(fixed_retrieval=tuple(int(g) for g in np.flatnonzero(base.mask(0))))
    chunks = CHUNKS[name]
    say(f"batched split {name}")
    ws, kv, pre, dec, total = _batched_run(w, 3, chunks, 2)
    L = sum(chunks)
    for b, wb in enumerate(ws):
        ref = oracle_rows(wb, 0, np.arange(total), total)
        compare(f"batched split {name} seq {b} prefill", to_f64(pre[b]), ref[:L], TOL["bf16"])
        compare(f"batched split {name} seq {b} decode", to_f64(dec[b]), ref[L:], TOL["bf16"])


def test_llama2_7b_mha_32k_full_attention_layer(torch_cuda):
    """The full-attention baseline on the same kernels (all 32 heads retrieval) at the 32K
    shape: 8 prefill chunks of 4096 and 16 decode steps.  Every decode output is checked;
    prefill rows are sampled (the first and last 16 rows of every chunk and 16 seeded rows
    per chunk)."""
    base = I.WORKLOADS["llama2_7b_mha_32k"]
    w = base.scaled(name="llama2_7b_mha_32k_full_attention", n_retrieval=base.n_kv_heads, fixed_retrieval=None,
                    decode_steps=16)
    assert w.mask(0).all()
    say("llama2_7b_mha_32k, full attention")
    chunks = [w.prefill_chunk] * (w.context // w.prefill_chunk)
    kv, pre, dec, total = run_layer(w, chunks, w.decode_steps)
    rng = np.random.default_rng(2)
    rows = set()
    for c in range(len(chunks)):
        a, b = c * w.prefill_chunk, (c + 1) * w.prefill_chunk
        rows |= set(range(a, a + 16)) | set(range(b - 16, b)) | set(rng.integers(a, b, 16).tolist())
    rows = np.array(sorted(rows))
    ref_dec = oracle_rows(w, 0, np.arange(w.context, total), total)
    compare("32k full-attention decode", to_f64(dec), ref_dec, TOL["bf16"])
    ref_pre = oracle_rows(w, 0, rows, total)
    compare("32k full-attention prefill (sampled rows)", to_f64(pre[rows]), ref_pre, TOL["bf16"])


VARLEN = {
    # name: (workload, per-sequence lengths before decoding; 0 = the first decode step
    # is the sequence's first token)
    "mha_bf16": (W("mha_bf16_var", 31, 8, 8, 128, "bf16", 8, 32, 1801, 6, 3, fixed=(0, 2, 5)),
                 [0, 1, 40, 1200, 613, 1800]),
    "gqa_bf16": (W("gqa_bf16_var", 32, 16, 4, 128, "bf16", 4, 64, 2101, 5, 2, fixed=(1, 3)), [700, 2100, 3]),
    "mha_f32_d128": (W("mha_f32_var", 33, 4, 4, 128, "f32", 2, 16, 501, 5, 2, fixed=(0, 3)), [5, 500, 0, 200]),
    "int4": (W("int4_var", 34, 8, 4, 128, "bf16", 4, 32, 1501, 5, 2, fmt="int4", fixed=(0, 3)), [90, 1500, 513]),
}


@pytest.mark.parametrize("name", list(VARLEN))
def test_varlen_batch_decode_matches_oracle(torch_cuda, name):
    """Sequences of different lengths in one handle: each filled by the per-sequence
    calls (prefill, or two appends for int4), then decode steps for the whole batch with
    every sequence's token at its own position, then one decode without new K/V after a
    per-sequence append.  Every sequence's outputs are checked against the oracle on its
    own data (sequence b: the workload reseeded with seed + 100 b), and its length and
    caches too.  The short sequences leave the long ones' later key splits empty."""
    import torch
    from mixed_head_kv_amd import binding as B
    w, lens = VARLEN[name]
    Bn, steps = len(lens), w.decode_steps
    ws = [w.scaled(seed=w.seed + 100 * b) for b in range(Bn)]
    say(f"varlen {name} lengths={lens} steps={steps}")
    kv = B.DuoKV.for_workload(w, batch=Bn)
    tol = TOL[w.io_dtype]
    data, pre = [], {}
    for b, (wb, L) in enumerate(zip(ws, lens)):
        q, k, v = (device_synth(wb, 0, x, 0, L + steps + 1) for x in "qkv")
        data.append((q, k, v))
        if L == 0:
            continue
        if w.kv_format == "int4":
            h = L // 2
            if h:
                kv.append_seq(0, b, k[:h].contiguous(), v[:h].contiguous())
            kv.append_seq(0, b, k[h:L].contiguous(), v[h:L].contiguous())
        else:
            pre[b] = kv.prefill_seq(0, b, q[:L].contiguous(), k[:L].contiguous(), v[:L].contiguous())
    torch.cuda.synchronize()
    assert [kv.length_seq(0, b) for b in range(Bn)] == lens
    with pytest.raises(B.DuoError) as e:
        kv.length(0)
    assert e.value.code == B.DUO_E_STATE
    dec = []
    for s in range(steps):
        qs, ks, vs = (torch.stack([data[b][i][lens[b] + s] for b in range(Bn)]) for i in range(3))
        dec.append(kv.decode(0, qs, ks, vs))
    # one more token per sequence by the per-sequence append, then a decode that reads it
    for b in range(Bn):
        t = lens[b] + steps
        kv.append_seq(0, b, data[b][1][t:t + 1].contiguous(), data[b][2][t:t + 1].contiguous())
    last = kv.decode(0, torch.stack([data[b][0][lens[b] + steps] for b in range(Bn)]))
    torch.cuda.synchronize()
    dec = torch.stack(dec, 1)
    rng = np.random.default_rng(5)
    for b, wb in enumerate(ws):
        L, total = lens[b], lens[b] + steps + 1
        assert kv.length_seq(0, b) == total
        ref = oracle_rows(wb, 0, np.arange(L, total), total)
        compare(f"varlen {name} seq {b} decode", to_f64(dec[b]), ref[:steps], tol)
        compare(f"varlen {name} seq {b} decode without new K/V", to_f64(last[b])[None], ref[steps:], tol)
        if b in pre:
            rows = np.unique(np.concatenate([np.arange(min(L, 8)), np.arange(max(0, L - 8), L),
                                             rng.integers(0, L, 16)]))
            compare(f"varlen {name} seq {b} prefill", to_f64(pre[b])[rows], oracle_rows(wb, 0, rows, total), tol)
        if w.kv_format != "int4":
            mask = wb.mask(0)
            g = int(np.flatnonzero(mask)[0])
            hist = host_history(wb, 0, "k", total)
            assert np.array_equal(to_f64(kv.read(0, g, 0, 0, total, b=b)), hist[:, g]), (name, b, "retrieval K")
            gs = int(np.flatnonzero(~mask)[0])
            n = min(w.recent, total)
            assert np.array_equal(to_f64(kv.read(0, gs, 0, total - n, n, b=b)), hist[total - n:, gs]), \
                (name, b, "streaming K window")


def test_varlen_batch_limits(torch_cuda):
    """Differing lengths in one decode launch take at most 32 sequences; a refused call
    changes nothing, and equal lengths are served at any batch size."""
    import torch
    from mixed_head_kv_amd import binding as B
    w = W("varlen_limit", 35, 4, 2, 128, "bf16", 2, 8, 40, 0, 1, fixed=(0,))
    say("varlen limits, batch 33")
    kv = B.DuoKV.for_workload(w, batch=33)
    k, v, q = (device_synth(w, 0, x, 0, 2) for x in "kvq")
    kv.append_seq(0, 0, k[:1].contiguous(), v[:1].contiguous())
    # every sequence holds the same data: position 0 appended, position 1 decoded
    qs, ks, vs = (x[1].expand(33, -1, -1).contiguous() for x in (q, k, v))
    with pytest.raises(B.DuoError) as e:
        kv.decode(0, qs, ks, vs)
    assert e.value.code == B.DUO_E_UNSUPPORTED
    assert [kv.length_seq(0, b) for b in range(33)] == [1] + [0] * 32
    for b in range(1, 33):
        kv.append_seq(0, b, k[:1].contiguous(), v[:1].contiguous())
    assert kv.length(0) == 1
    out = kv.decode(0, qs, ks, vs)
    torch.cuda.synchronize()
    ref = oracle_rows(w, 0, [1], 2)
    for b in range(33):
        compare(f"batch 33 seq {b}", to_f64(out[b])[None], ref, TOL["bf16"])
    with pytest.raises(B.DuoError) as e:
        kv.length_seq(0, 33)
    assert e.value.code == B.DUO_E_INVALID


DUAL = {
    # name: (workload with every KV head a retrieval head, chunks)
    "gqa_sink4": (W("dual_gqa", 41, 16, 4, 128, "bf16", 4, 64, 1024, 3, 4), [257, 255, 512]),
    "mha_sink64": (W("dual_mha", 42, 8, 8, 128, "bf16", 64, 256, 1700, 3, 8), [700, 1000]),
    "nosink": (W("dual_nosink", 43, 4, 2, 128, "bf16", 0, 8, 300, 2, 2), [37, 263]),
    "long_chunk": (W("dual_long", 44, 4, 2, 128, "bf16", 16, 128, 4700, 2, 2), [4600, 100]),
    # the 128K layer's shape and chunk (4 query heads per KV head: 8-wavefront workgroups)
    "gqa_8192": (W("dual_gqa_8192", 45, 32, 8, 128, "bf16", 64, 256, 8292, 2, 8), [8192, 100]),
}


@pytest.mark.parametrize("name", list(DUAL))
def test_prefill_dual_outputs_match_oracle(torch_cuda, name):
    """Head identification: every head's full causal output and its sinks + window output
    over the same keys, chunk by chunk, against the oracle with every head labelled
    retrieval and with every head labelled streaming; then decode steps on the caches the
    call filled (full attention)."""
    import torch
    from mixed_head_kv_amd.binding import DuoKV
    w, chunks = DUAL[name]
    assert w.mask(0).all()
    L = sum(chunks)
    total = L + w.decode_steps
    say(f"dual prefill {name} chunks={chunks}")
    Q, K, V = (device_synth(w, 0, x, 0, total) for x in "qkv")
    kv = DuoKV.for_workload(w)
    full, strm, t = [], [], 0
    for T in chunks:
        sl = slice(t, t + T)
        f, s = kv.prefill_dual(0, Q[sl].contiguous(), K[sl].contiguous(), V[sl].contiguous())
        full.append(f)
        strm.append(s)
        t += T
    dec = [kv.decode(0, Q[t + i], K[t + i], V[t + i]) for i in range(w.decode_steps)]
    torch.cuda.synchronize()
    rows = np.arange(total)
    Kh, Vh = host_history(w, 0, "k", total), host_history(w, 0, "v", total)
    Qh = OA.upcast(q_rows(w, 0, rows), w.io_dtype)
    ones, zeros = np.ones(w.n_kv_heads, bool), np.zeros(w.n_kv_heads, bool)
    ref_full = OA.layer_attention(Qh, rows, Kh, Vh, ones, w.sink, w.recent)
    ref_strm = OA.layer_attention(Qh[:L], rows[:L], Kh, Vh, zeros, w.sink, w.recent)
    # the two references are far apart past the first sink + window rows, so each output
    # is checked against its own definition
    assert np.abs(ref_full[w.sink + w.recent:L] - ref_strm[w.sink + w.recent:]).max() > 10 * TOL["bf16"]
    compare(f"{name} full", to_f64(torch.cat(full)), ref_full[:L], TOL["bf16"])
    compare(f"{name} streaming", to_f64(torch.cat(strm)), ref_strm, TOL["bf16"])
    compare(f"{name} decode after", to_f64(torch.stack(dec)), ref_full[L:], TOL["bf16"])
    assert kv.length(0) == total


def test_prefill_dual_needs_full_caches(torch_cuda):
    from mixed_head_kv_amd import binding as B
    w = SMALL["gqa_bf16"]
    kv = B.DuoKV.for_workload(w)
    q = device_synth(w, 0, "q", 0, 8)
    k = device_synth(w, 0, "k", 0, 8)
    with pytest.raises(B.DuoError) as e:
        kv.prefill_dual(0, q, k, k)
    assert e.value.code == B.DUO_E_STATE and kv.length(0) == 0


def test_int4_decode_at_32m_context_periodic_history(torch_cuda):
    """One Llama-3-8B-shaped layer (32 query heads, 8 KV heads, 4 of them retrieval, sink
    64 + recent 256) holding an int4 cache of 2^25 tokens, ten times the pages' longest
    context: the history repeats one 65536-token block (appended 512 times), so the
    oracle checks every head exactly through the periodic form of the softmax; then two
    decode steps whose tokens continue the period."""
    import torch
    from mixed_head_kv_amd.binding import DuoKV
    P, ctx = 1 << 16, 1 << 25
    w = W("int4_32m", 51, 32, 8, 128, "bf16", 64, 256, ctx, 2, 4, fmt="int4", fixed=(0, 2, 5, 7))
    say("int4 decode at 2^25 tokens (periodic history)")
    kv = DuoKV.for_workload(w)
    K, V = device_synth(w, 0, "k", 0, P), device_synth(w, 0, "v", 0, P)
    for _ in range(ctx // P):
        kv.append(0, K, V)
    torch.cuda.synchronize()
    assert kv.length(0) == ctx
    outs = []
    for t in (ctx, ctx + 1):
        q = device_synth(w, 0, "q", t, 1)[0]
        outs.append(kv.decode(0, q, K[t % P], V[t % P]))
    torch.cuda.synchronize()
    Kp, Vp = host_history(w, 0, "k", P), host_history(w, 0, "v", P)
    mask, G = w.mask(0), w.group
    for t, o in zip((ctx, ctx + 1), outs):
        qh = OA.upcast(q_rows(w, 0, [t]), w.io_dtype)[0]
        ref = np.stack([OA.head_attention_periodic(qh[h], t, Kp[:, h // G], Vp[:, h // G], bool(mask[h // G]),
                                                   w.sink, w.recent) for h in range(w.n_q_heads)])
        compare(f"int4 2^25 decode t={t}", to_f64(o), ref, TOL["bf16"])



def test_per_sequence_prefill_with_a_chunk_over_one_staging_pass(torch_cuda):
    """A batch of two where one sequence takes a 4600-token chunk by itself (its streaming
    heads need two staged launches, and the streaming caches are updated in a launch of
    their own) and the other a short one; then decode steps for both at their own
    positions."""
    import torch
    from mixed_head_kv_amd.binding import DuoKV
    w = W("seq_long", 45, 8, 4, 128, "bf16", 4, 300, 4600, 3, 1, fixed=(2,))
    lens = [4600, 120]
    ws = [w.scaled(seed=w.seed + 100 * b) for b in range(2)]
    say(f"per-sequence prefill lengths={lens}")
    kv = DuoKV.for_workload(w, batch=2)
    data, pre = [], []
    for b, (wb, L) in enumerate(zip(ws, lens)):
        q, k, v = (device_synth(wb, 0, x, 0, L + w.decode_steps) for x in "qkv")
        data.append((q, k, v))
        pre.append(kv.prefill_seq(0, b, q[:L].contiguous(), k[:L].contiguous(), v[:L].contiguous()))
    dec = []
    for s in range(w.decode_steps):
        qs, ks, vs = (torch.stack([data[b][i][lens[b] + s] for b in range(2)]) for i in range(3))
        dec.append(kv.decode(0, qs, ks, vs))
    torch.cuda.synchronize()
    dec = torch.stack(dec, 1)
    rng = np.random.default_rng(3)
    for b, wb in enumerate(ws):
        L, total = lens[b], lens[b] + w.decode_steps
        rows = np.unique(np.concatenate([np.arange(min(L, 16)), np.arange(max(0, L - 16), L),
                                         rng.integers(0, L, 48), np.arange(4090, 4110) if L > 4110 else []]))
        rows = rows.astype(np.int64)
        compare(f"seq {b} prefill", to_f64(pre[b])[rows], oracle_rows(wb, 0, rows, total), TOL["bf16"])
        compare(f"seq {b} decode", to_f64(dec[b]), oracle_rows(wb, 0, np.arange(L, total), total), TOL["bf16"])



@pytest.mark.parametrize("G", [8, 16])
def test_wide_query_groups_match_oracle(torch_cuda, G):
    """GQA groups of 8 and 16 query heads per KV head (16 fills every column of the decode
    products): prefill over two chunks, then decode steps, bf16 and int4 caches."""
    for fmt in ("same", "int4"):
        hkv = 2
        w = W(f"group{G}_{fmt}", 60 + G, hkv * G, hkv, 128, "bf16", 4, 48, 600, 4, 1, fmt=fmt, fixed=(1,))
        say(f"group {G} {fmt}")
        chunks = [333, 267]
        kv, pre, dec, total = run_layer(w, chunks, w.decode_steps, append_only_chunks=fmt == "int4")
        L = sum(chunks)
        ref = oracle_rows(w, 0, np.arange(0 if pre is not None else L, total), total)
        if pre is not None:
            compare(f"G={G} {fmt} prefill", to_f64(pre), ref[:L], TOL["bf16"])
            compare(f"G={G} {fmt} decode", to_f64(dec), ref[L:], TOL["bf16"])
        else:
            compare(f"G={G} {fmt} decode", to_f64(dec), ref, TOL["bf16"])


def test_wide_query_groups_over_long_split_chunks(torch_cuda):
    """8 query heads per KV head (two 4-head groups per KV head in 8-wavefront prefill
    workgroups, both groups' blocks dispatched to one XCD) over chunks of 4096 and 2048
    tokens, whose query blocks split their keys over two workgroups: every prefill row and
    decode step of every head against the oracle."""
    w = W("group8_long", 68, 16, 2, 128, "bf16", 64, 256, 6144 + 4, 4, 1, fixed=(0,))
    chunks = [4096, 2048]
    say("group 8 long split chunks")
    kv, pre, dec, total = run_layer(w, chunks, w.decode_steps)
    L = sum(chunks)
    ref = oracle_rows_threaded(w, 0, np.arange(total), total)
    compare("G=8 long prefill (every row)", to_f64(pre), ref[:L], TOL["bf16"])
    compare("G=8 long decode", to_f64(dec), ref[L:], TOL["bf16"])


@pytest.mark.parametrize("name", ["mha64_bf16", "gqa64x2_f32_d64"])
def test_most_kv_heads_match_oracle(torch_cuda, name):
    """The largest head count the library accepts (64 KV heads): a bf16 MHA layer whose
    retrieval heads' decode runs in three splits (1100 keys), and an fp32 head_dim 64 layer
    with two query heads per KV head (128 query heads; vector-ALU kernels)."""
    w = {
        "mha64_bf16": W("mha64_bf16", 70, 64, 64, 128, "bf16", 8, 96, 1100, 3, 16),
        "gqa64x2_f32_d64": W("gqa64x2_f32_d64", 71, 128, 64, 64, "f32", 4, 40, 300, 2, 20),
    }[name]
    chunks = {"mha64_bf16": [700, 400], "gqa64x2_f32_d64": [300]}[name]
    say(f"64 KV heads: {name}")
    kv, pre, dec, total = run_layer(w, chunks, w.decode_steps)
    L = sum(chunks)
    ref = oracle_rows(w, 0, np.arange(total), total)
    compare(f"{name} prefill", to_f64(pre), ref[:L], TOL[w.io_dtype])
    compare(f"{name} decode", to_f64(dec), ref[L:], TOL[w.io_dtype])
