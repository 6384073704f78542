"""Capture of a whole decode step in a HIP graph (through torch.cuda.graph)
and its replay. The calls' launch grids depend only on their dims, and the
balanced split's counters return to zero by themselves, so a captured step
replays without any host work. Every replay is checked against the float64
oracle (every row of every layer at bucket 8; sampled rows of the first and
last layers at bucket 256) and bit for bit against the eager result, with
eager work and synchronisations between replays."""

import math

import numpy as np
import pytest
import torch

import paged_kv_cache_55_amd as pk
import workloads as wl
from parity import compare, gpu_out_f64, oracle_config5_rows, oracle_step

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16)


@pytest.mark.parametrize("partition", [0, 512])
@pytest.mark.parametrize("bucket", [8, 256])
def test_replay_of_32_layer_step(bucket, partition):
    spec = wl.config5_spec(bucket)
    bt = torch.from_numpy(spec.block_tables).cuda()
    lens = torch.from_numpy(spec.seq_lens).cuda()
    layers = [wl.config5_layer(spec, layer, "cuda") for layer in range(spec.layers)]
    outs = [torch.empty_like(q) for q, _, _ in layers]
    if bucket <= 8:
        checked = {layer: list(range(bucket)) for layer in range(spec.layers)}
    else:
        rng = np.random.default_rng(bucket + partition)
        rows = sorted(rng.choice(spec.n_real, size=14, replace=False).tolist()
                      + [spec.n_real - 1, bucket - 1])
        checked = {0: rows, spec.layers - 1: rows}
    print(f"graph bucket {bucket} split {partition}: oracle on {len(checked)} layers",
          flush=True)
    refs = {layer: oracle_config5_rows(spec, *layers[layer], rows)
            for layer, rows in checked.items()}

    def check_oracle(tag):
        for layer, rows in checked.items():
            compare(gpu_out_f64(outs[layer], rows), refs[layer], spec.seq_lens[rows], "bf16")
    q0, k0, _ = layers[0]
    dims = pk.make_dims(spec.bucket, 32, 8, 128, bt.shape[1], k0.shape[0], pk.PA_BF16,
                        partition, "mfma")
    ws = torch.zeros(max(pk.pa_decode_workspace_bytes(dims), 1), dtype=torch.uint8,
                     device="cuda")
    scale = 1.0 / math.sqrt(128)

    def step():
        for (q, k, v), o in zip(layers, outs):
            pk.pa_decode(q, k, v, bt, lens, scale, o, partition_tokens=partition,
                         kernel="mfma", workspace=ws)

    step()
    torch.cuda.synchronize()
    check_oracle("eager")
    ref = [o.clone() for o in outs]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = wl.random_case(601, 5, 32, 8, 128, "bf16", max_len=900).to("cuda")
    for replay in range(4):
        for o in outs:
            o.fill_(7.0)  # eager fill kernel between replays
        g.replay()
        torch.cuda.synchronize()
        check_oracle(f"replay {replay}")
        for layer, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(_bits(o), _bits(r)), f"replay {replay} layer {layer}"
        # an unrelated eager call on its own workspace between replays
        pk.pa_decode(other.q, other.k_pool, other.v_pool, other.block_tables, other.seq_lens,
                     other.scale, partition_tokens=0, kernel="mfma")
        torch.cuda.synchronize()


def test_replay_of_write_then_decode_step():
    """The 8B batch's two-call step (append, then decode) as one graph:
    every replay's output matches the oracle's append-then-decode, and the
    pools and output after a replay match a fresh eager run bit for bit."""
    c = wl.config2()
    oracle_out, _, _ = oracle_step(c)
    eager = c.to("cuda")
    out_e = torch.empty_like(eager.q)
    dims = pk.make_dims(c.num_seqs, 32, 8, 128, c.max_blocks_per_seq, c.num_blocks,
                        pk.PA_BF16, 0, "mfma")
    ws = torch.zeros(pk.pa_decode_workspace_bytes(dims), dtype=torch.uint8, device="cuda")

    def step(d, out):
        pk.pa_write_kv(d.k_new, d.v_new, d.slot_mapping, d.k_pool, d.v_pool)
        pk.pa_decode(d.q, d.k_pool, d.v_pool, d.block_tables, d.seq_lens, c.scale, out,
                     partition_tokens=0, kernel="mfma", workspace=ws)

    step(eager, out_e)
    torch.cuda.synchronize()

    d = c.to("cuda")
    out = torch.empty_like(d.q)
    g = torch.cuda.CUDAGraph()
    k0, v0 = d.k_pool.clone(), d.v_pool.clone()
    with torch.cuda.graph(g):
        step(d, out)
    for replay in range(3):
        d.k_pool.copy_(k0)  # back to the pre-step pools (eager copy kernels)
        d.v_pool.copy_(v0)
        out.fill_(3.0)
        g.replay()
        torch.cuda.synchronize()
        compare(gpu_out_f64(out), oracle_out, c.seq_lens.numpy(), "bf16")
        assert torch.equal(_bits(out), _bits(out_e)), f"replay {replay}"
        assert torch.equal(_bits(d.k_pool), _bits(eager.k_pool))
        assert torch.equal(_bits(d.v_pool), _bits(eager.v_pool))
