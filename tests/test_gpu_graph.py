"""The mixed step (slot-mapped write, prefill chunks, split-KV decode with
its partitions merged by a second kernel, or on chip in one pass) captured
into a HIP graph: the eager step matches the fp64 oracle, and every replay,
with the program's own eager work and synchronisations in between,
reproduces the eager step bit for bit.  All three calls enqueue on the
caller's stream, take their workspace from the caller and never allocate or
set memory, so they can be captured."""
import pytest
import torch

import paged_kv_cache_422_amd as pa
import workloads as W
from oracle import attention as A
from oracle import kv_cache as KC
from tests.gpu_util import DEV, assert_close, bits

pytestmark = pytest.mark.gpu


# Contexts up to 900 tokens: 32-token partitions (29 of them) are more than
# the single pass's LDS holds, so the merge pass runs; 128-token partitions
# (8) are merged on chip.
@pytest.mark.parametrize("P,merge", [(32, pa.MERGE_TWO_PASS), (128, pa.MERGE_ON_CHIP)],
                         ids=["two-pass", "on-chip"])
def test_mixed_step_graph_replays_match_eager(P, merge):
    print(f"graph capture of the mixed step, partitions of {P}", flush=True)
    w = W.mixed(num_decode=192, chunk=160, cached=96, lmin=16, lmax=900)
    kc0, vc0, k_new, v_new, q_dec, q_pre = w.make_tensors(DEV)
    sm = torch.from_numpy(w.slot_mapping).to(DEV)
    pbt = torch.from_numpy(w.prefill_bt).to(DEV)
    qsl = torch.from_numpy(w.q_start_loc).to(DEV)
    psl = torch.from_numpy(w.prefill_seq_lens).to(DEV)
    dbt = torch.from_numpy(w.decode_bt).to(DEV)
    dctx = torch.from_numpy(w.decode_lens).to(DEV)
    assert pa.decode_plan(w.num_decode, w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_model_len, P)[1] == merge
    ws = torch.empty(pa.decode_workspace_size(w.num_decode, w.num_q_heads, w.head_dim, w.max_model_len, P,
                                              w.num_kv_heads), dtype=torch.uint8, device=DEV)
    assert ws.numel() > 0
    kc, vc = kc0.clone(), vc0.clone()
    out_pre, out_dec = torch.empty_like(q_pre), torch.empty_like(q_dec)

    def step():
        pa.write_kv(k_new, v_new, kc, vc, sm)
        pa.prefill_chunk(out_pre, q_pre, kc, vc, pbt, qsl, psl, w.prefill_chunk,
                         w.prefill_cached + w.prefill_chunk, w.scale)
        pa.decode(out_dec, q_dec, kc, vc, dbt, dctx, w.max_model_len, w.scale, P, ws)

    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (kc, vc, out_pre, out_dec)]

    # The eager step against the oracle: the write bit for bit, prefill and
    # decode within tolerance (so every replay below is held to it too).
    kh, vh = bits(kc0), bits(vc0)
    KC.write_kv(kh, vh, bits(k_new), bits(v_new), w.slot_mapping, 16)
    assert (bits(kc).view('u2') == kh.view('u2')).all() and (bits(vc).view('u2') == vh.view('u2')).all()
    assert_close(out_pre, A.prefill(bits(q_pre), kh, vh, w.prefill_bt, w.q_start_loc, w.prefill_seq_lens,
                                    w.scale, w.dtype), what=f"eager prefill, P={P}")
    assert_close(out_dec, A.decode(bits(q_dec), kh, vh, w.decode_bt, w.decode_lens, w.scale, w.dtype),
                 what=f"eager decode, P={P}")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                           # warm-up off the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()

    other = torch.empty_like(out_dec)
    for r in range(4):
        kc.copy_(kc0)                                    # eager work between replays
        vc.copy_(vc0)
        out_pre.fill_(float("nan"))
        out_dec.fill_(float("nan"))
        pa.decode(other, q_dec, kc0, vc0, dbt, dctx, w.max_model_len, w.scale, 0,
                  torch.empty(1, dtype=torch.uint8, device=DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, ref in zip((kc, vc, out_pre, out_dec), want):
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {r}"
