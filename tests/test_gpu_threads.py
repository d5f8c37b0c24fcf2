"""Calls from several host threads at once, each on its own stream, must give
exactly the results of the same calls made one at a time: the library keeps no
shared mutable state beyond per-thread caches (RoPE frequency tables, rocBLAS
handles) and the per-device CU count."""

import threading

import numpy as np
import pytest
import torch

import zero_shot_rope_attention_amd as jl
from zero_shot_rope_attention_amd.inputs import make_layer, make_qkv

from gpu_helpers import to_device

pytestmark = pytest.mark.gpu


def _jobs():
    jobs = []
    for i, (n_kv, base, big_l) in enumerate([(3000, 1e4, 512), (2048, 1e6, 256), (1500, 5e5, 1024), (4096, 1e4, 900)]):
        qb, kb, vb = make_qkv(800 + i, 1, 300, n_kv, 8, 2, 128)
        q, k, v = to_device(qb), to_device(kb), to_device(vb)
        qd = q[:, -1:].contiguous()
        x, w_qkv, w_o, gq, gk = (to_device(a) for a in make_layer(850 + i, 1, 64, 256, 4, 2))
        jobs.append(dict(q=q, k=k, v=v, qd=qd, base=base, big_l=big_l, n_kv=n_kv, layer=(x, w_qkv, w_o, gq, gk)))
    return jobs


def _run(job, stream):
    with torch.cuda.stream(stream):
        q, k, v, qd = job["q"], job["k"], job["v"], job["qd"]
        out = torch.empty_like(q)
        ws = torch.empty(jl.jl_bifocal_prefill_workspace_size(1, job["n_kv"], 2), dtype=torch.uint8, device="cuda:0")
        jl.jl_bifocal_prefill_ws(q, k, v, out, None, job["big_l"], 64, job["base"], ws, stream=stream.cuda_stream)
        od = torch.empty_like(qd)
        wsd = torch.empty(jl.jl_bifocal_decode_workspace_size(1, job["n_kv"], 8, 2), dtype=torch.uint8, device="cuda:0")
        jl.jl_bifocal_decode(qd, k, v, od, None, job["big_l"], 64, job["base"], wsd, stream=stream.cuda_stream)
        x, w_qkv, w_o, gq, gk = job["layer"]
        kc = torch.zeros((1, 64, 2, 128), dtype=torch.bfloat16, device="cuda:0")
        vc = torch.zeros_like(kc)
        lo = torch.empty_like(x)
        wsl = torch.empty(jl.jl_qwen3_layer_workspace_size(1, 64, 64, 4, 2), dtype=torch.uint8, device="cuda:0")
        jl.jl_qwen3_attention_layer(x, w_qkv, gq, gk, w_o, lo, kc, vc, wsl, bifocal=True, pretrained_window=16,
                                    local_window=8, rope_base=job["base"], stream=stream.cuda_stream)
        stream.synchronize()
        return [t.view(torch.int16).cpu().numpy() for t in (out, od, lo, kc)]


def test_concurrent_threads_match_serial_calls():
    jobs = _jobs()
    print(f"threads: {len(jobs)} jobs, serial then concurrent", flush=True)
    serial = [_run(j, torch.cuda.Stream()) for j in jobs]
    results = [None] * len(jobs)
    errors = []

    def worker(i):
        try:
            for _ in range(3):
                results[i] = _run(jobs[i], torch.cuda.Stream())
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    for i in range(len(jobs)):
        for a, b in zip(serial[i], results[i]):
            assert np.array_equal(a, b), f"job {i} differs from its serial run"
