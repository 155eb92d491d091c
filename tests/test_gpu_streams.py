"""The mixed step with the prefill chunks and the decode on two streams.

Both calls only read the cache once the write is done, so a caller may run
them concurrently: the write on its stream, then the prefill on a second
stream that waits for the write, and the decode on the first.  Every call
enqueues on the stream it is given, so the outputs must equal the same step
run in sequence on one stream, bit for bit (the sequential step itself is
held to the oracle in test_gpu_graph.py)."""
import pytest
import torch

import paged_kv_cache_422_amd as pa
import workloads as W
from tests.gpu_util import DEV

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("P", [32, 128], ids=["two-pass", "on-chip"])
def test_mixed_step_on_two_streams_matches_one(P):
    print(f"mixed step on two streams, partitions of {P}", flush=True)
    w = W.mixed(num_decode=192, chunk=160, cached=96, lmin=16, lmax=900)
    kc0, vc0, k_new, v_new, q_dec, q_pre = w.make_tensors(DEV)
    sm = torch.from_numpy(w.slot_mapping).to(DEV)
    pbt = torch.from_numpy(w.prefill_bt).to(DEV)
    qsl = torch.from_numpy(w.q_start_loc).to(DEV)
    psl = torch.from_numpy(w.prefill_seq_lens).to(DEV)
    dbt = torch.from_numpy(w.decode_bt).to(DEV)
    dctx = torch.from_numpy(w.decode_lens).to(DEV)
    ws = torch.empty(max(pa.decode_workspace_size(w.num_decode, w.num_q_heads, w.head_dim, w.max_model_len, P,
                                                  w.num_kv_heads), 1), dtype=torch.uint8, device=DEV)
    kc, vc = kc0.clone(), vc0.clone()
    out_pre, out_dec = torch.empty_like(q_pre), torch.empty_like(q_dec)

    def write():
        pa.write_kv(k_new, v_new, kc, vc, sm)

    def prefill():
        pa.prefill_chunk(out_pre, q_pre, kc, vc, pbt, qsl, psl, w.prefill_chunk,
                         w.prefill_cached + w.prefill_chunk, w.scale)

    def decode():
        pa.decode(out_dec, q_dec, kc, vc, dbt, dctx, w.max_model_len, w.scale, P, ws)

    write()
    prefill()
    decode()
    torch.cuda.synchronize()
    want = [t.clone() for t in (kc, vc, out_pre, out_dec)]

    side = torch.cuda.Stream()
    written = torch.cuda.Event()
    for r in range(3):
        kc.copy_(kc0)
        vc.copy_(vc0)
        out_pre.fill_(float("nan"))
        out_dec.fill_(float("nan"))
        write()
        written.record()
        side.wait_event(written)
        with torch.cuda.stream(side):
            prefill()
        decode()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for got, ref in zip((kc, vc, out_pre, out_dec), want):
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"round {r}"
