"""Every workload at full size, through the layer-step bench.py times.

bench.LayerStep builds the step the bench captures: the same entry points
(the planned, fused pa_decode_append; the planned pa_decode_cascade with its
append arrays; pa_kv_append + planned decode + pa_prefill_chunk for the mixed
batch; pa_decode_multi for draft verification), the same partition sizes and
a pa_decode_plan launch inside the captured region.  Here the pools start
without the step's new tokens (the step's own append writes them) and with
every unowned byte NaN.  Three layer-steps over two layer copies are
captured in one graph, as the bench captures its timed steps; after each
replay, with other work and synchronisations between replays, every output
row is compared with the fp64 oracle and every byte of both layer copies
with oracle_append's pool (llm-infer, "What It Does": the captured decode
step writes the KV cache and runs attention; all five workloads must match
the oracle)."""

import numpy as np
import pytest
import torch

import bench
from oracle import paged_attention as opa
from tests.gpu_helpers import TOL, as_f64, host, max_abs_err, oracle_pool

pytestmark = pytest.mark.gpu


def _reference(w, spec, kp, vp):
    """(decode rows or None, prefill / draft-token rows or None), fp64."""
    dec = pre = None
    if spec or w.num_chunks:
        pre = opa.oracle_prefill(host(w.q_prefill), w.q_dtype, w.query_start_loc, kp, vp,
                                 w.cache_dtype, w.chunk_block_tables, w.chunk_context_lens,
                                 w.scale, w.k_scale, w.v_scale, w.block_size)
    if not spec:
        dec = opa.oracle_decode(host(w.q), w.q_dtype, kp, vp, w.cache_dtype, w.block_tables,
                                w.context_lens, w.scale, w.k_scale, w.v_scale, w.block_size)
    return dec, pre


@pytest.mark.parametrize("name", bench.workload_names())
def test_bench_step_full_size_every_row_every_replay(name):
    print("full-size bench step:", name, flush=True)
    w, ps, spec = bench.make_workload(name, None, "cuda")
    ls = bench.LayerStep(w, ps, spec, "cuda", layer_copies=2, fill_new=False, poison=True)
    torch.cuda.synchronize()
    g = bench.capture(lambda: [ls.step(layer, 0) for layer in range(3)], torch.cuda.Stream())
    torch.cuda.synchronize()

    kp, vp = oracle_pool(w)
    dec, pre = _reference(w, spec, kp, vp)
    kd = torch.from_numpy(kp.view(np.uint8)).to("cuda")
    vd = torch.from_numpy(vp.view(np.uint8)).to("cuda")
    del kp, vp
    tol = TOL[w.cache_dtype]
    for rep in range(2):
        ls.out.fill_(float("nan"))
        if ls.has_prefill:
            ls.outp.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if spec:
            err = max_abs_err(as_f64(ls.out), pre)
            assert err <= tol, "draft rows, replay %d: %g" % (rep, err)
        else:
            err = max_abs_err(as_f64(ls.out), dec)
            assert err <= tol, "decode rows, replay %d: %g" % (rep, err)
            if ls.has_prefill:
                err = max_abs_err(as_f64(ls.outp), pre)
                assert err <= tol, "prefill rows, replay %d: %g" % (rep, err)
        for i, pool in enumerate(ls.pools):
            assert torch.equal(pool.k.view(torch.uint8).flatten(), kd.flatten()), \
                "K pool of layer copy %d, replay %d" % (i, rep)
            assert torch.equal(pool.v.view(torch.uint8).flatten(), vd.flatten()), \
                "V pool of layer copy %d, replay %d" % (i, rep)
        x = torch.randn(1024, 1024, device="cuda")
        (x @ x).sum().item()


@pytest.mark.parametrize("name", ["qwen2.5-3b-bf16-decode-b64", "long-context-bf16-splitk-b8",
                                  "mixed-chunked-prefill-fp8kv"])
def test_bench_step_is_batch_invariant_at_full_size(name):
    """The planned decode step gives every sequence the same bits when the
    batch around it is reordered (which moves every cut between
    wavefronts): infer-lab, batched decode == sequential decode."""
    import copy
    print("batch invariance:", name, flush=True)
    w, ps, spec = bench.make_workload(name, None, "cuda")
    ls = bench.LayerStep(w, ps, spec, "cuda", layer_copies=1)
    ls.step(0, 0)
    torch.cuda.synchronize()
    full = ls.out.clone()
    del ls
    assert np.all(w.context_lens > 0)         # one new token per sequence, in order
    for perm in (np.arange(w.batch)[::-1].copy(), np.random.default_rng(1).permutation(w.batch)):
        w2 = copy.copy(w)
        w2.context_lens = w.context_lens[perm]
        w2.block_tables = w.block_tables[perm]
        w2.q = w.q[torch.as_tensor(perm, device="cuda")]
        w2.new_rows = np.concatenate([w.new_rows[:w.batch][perm], w.new_rows[w.batch:]])
        w2.new_slots = np.concatenate([w.new_slots[:w.batch][perm], w.new_slots[w.batch:]])
        ls2 = bench.LayerStep(w2, ps, spec, "cuda", layer_copies=1)
        ls2.step(0, 0)
        torch.cuda.synchronize()
        assert torch.equal(ls2.out, full[torch.as_tensor(perm, device="cuda")])
        del ls2
