"""The allocation-free decode entry point against the decode that takes a workspace.

jl_bifocal_decode_noalloc keeps its chunk partials in a device array the library
holds per GPU; jl_bifocal_decode takes the caller's workspace.  Both run the same
kernels with the same chunking, so their results must be equal bit for bit: on
two calls in a row (the second with a smaller cache and batch, over the array the
first one left behind), for g > 1 and g = 1.
"""

import numpy as np
import pytest
import torch

import oracle
import zero_shot_rope_attention_amd as jl
from zero_shot_rope_attention_amd.inputs import bf16_bits_to_f64, make_qkv

from gpu_helpers import assert_parity, to_device, to_f64

pytestmark = pytest.mark.gpu


def _both(wid, b, n_kv, hq, hkv, big_l, w, base):
    qb, kb, vb = make_qkv(wid, b, 1, n_kv, hq, hkv, 128)
    q, k, v = to_device(qb), to_device(kb), to_device(vb)
    print(f"no-alloc decode wid={wid} B={b} n_kv={n_kv} Hq={hq} Hkv={hkv} L={big_l} W={w} "
          f"g={jl.jl_group_factor(n_kv, big_l)}", flush=True)
    out_a, out_b = torch.empty_like(q), torch.empty_like(q)
    lse_a = torch.empty((b, hq, 1), dtype=torch.float32, device="cuda:0")
    lse_b = torch.empty_like(lse_a)
    jl.jl_bifocal_decode_noalloc(q, k, v, out_a, lse_a, big_l, w, base)
    ws = torch.empty(jl.jl_bifocal_decode_workspace_size(b, n_kv, hq, hkv), dtype=torch.uint8, device="cuda:0")
    jl.jl_bifocal_decode(q, k, v, out_b, lse_b, big_l, w, base, ws)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    assert torch.equal(lse_a, lse_b)
    return (qb, kb, vb), to_f64(out_a)


def test_noalloc_decode_matches_the_workspace_decode_twice():
    # a larger call first, then a smaller one over the array it left behind
    (qb, kb, vb), out = _both(900, 2, 70000, 32, 8, 32768, 4096, 1e6)           # g = 3
    ro, _ = oracle.bifocal_decode(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb), 32768, 4096, 1e6)
    assert_parity(out, ro, "no-alloc decode, first call")
    (qb, kb, vb), out = _both(901, 1, 5000, 8, 2, 1024, 256, 1e4)               # g = 5, fewer chunks
    ro, _ = oracle.bifocal_decode(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb), 1024, 256, 1e4)
    assert_parity(out, ro, "no-alloc decode, second call")


def test_noalloc_decode_plain_length_and_workload_shape():
    _both(902, 1, 3000, 16, 4, 4096, 512, 1e6)                                  # g = 1: the plain kernels
    _both(903, 1, 131072, 32, 8, 32768, 4096, 1e6)                              # the 128K decode


def test_noalloc_decode_under_graph_capture():
    # The callers this entry point is for: a HIP graph captures several decode
    # calls (different caches, shared library array), and every replay -- with
    # the program's own eager work and synchronisations between replays -- must
    # give bit for bit the eager results.  The path records no memset.
    b, hq, hkv, big_l, w, base = 1, 32, 8, 32768, 4096, 1e6
    lengths = (65536, 40000, 131072, 32768)
    caches = []
    for i, n in enumerate(lengths):
        qb, kb, vb = make_qkv(910 + i, b, 1, n, hq, hkv, 128)
        caches.append((to_device(qb), to_device(kb), to_device(vb)))
    print(f"no-alloc decode under graph capture: lengths {lengths}", flush=True)
    eager = []
    for q, k, v in caches:
        o = torch.empty_like(q)
        l_ = torch.empty((b, hq, 1), dtype=torch.float32, device="cuda:0")
        jl.jl_bifocal_decode_noalloc(q, k, v, o, l_, big_l, w, base)
        eager.append((o, l_))
    torch.cuda.synchronize()
    outs = [(torch.empty_like(q), torch.empty((b, hq, 1), dtype=torch.float32, device="cuda:0"))
            for q, _, _ in caches]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for (q, k, v), (o, l_) in zip(caches, outs):
                jl.jl_bifocal_decode_noalloc(q, k, v, o, l_, big_l, w, base)  # on the capturing stream
    torch.cuda.synchronize()
    for rep in range(3):
        for o, l_ in outs:
            o.zero_()
            l_.zero_()
        # eager work on the array between replays: the graph must not depend on what it held
        q, k, v = caches[rep % len(caches)]
        jl.jl_bifocal_decode_noalloc(q, k, v, torch.empty_like(q), None, big_l, w, base)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for (o, l_), (eo, el) in zip(outs, eager):
            assert torch.equal(o.view(torch.int16), eo.view(torch.int16)), f"replay {rep}"
            assert torch.equal(l_, el), f"replay {rep}"
