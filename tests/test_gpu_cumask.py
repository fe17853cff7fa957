"""The nano-batch schedule's CU-masked second stream
(ns_sched.cu_mask_frac: the attention nano-ops' stream created with
hipExtStreamCreateWithCUMask on a fraction of the compute units, NanoFlow
review, "The part that is harder than it looks": the resource share R given
to the memory-bound nano-ops).  Restricting where the attention runs changes
no result: overlapped on the masked stream = the same split run serially,
bit for bit, eager and graph-replayed."""
import pytest
import torch

from decode_step_06_amd import ns
from decode_step_06_amd.configs import ModelShape, Workload
from gpu_helpers import Case, say

pytestmark = pytest.mark.gpu

SMALL = ModelShape("small", 2, 256, 8, 2, 64, 512, 1000, True, "bf16")


@pytest.mark.skip(reason="CU-masked second stream switched off: on its first GPU run (fraction 0.4) the step "
                         "returned and the engine's destroy then waited on the masked stream until the test's "
                         "time limit; cause not found, so ns_engine_create rejects cu_mask_frac != 0")
@pytest.mark.parametrize("frac", [0.4, 1.0])
def test_cu_masked_attention_stream_equals_serial(frac):
    w = Workload("cm", SMALL, 6, ctx_range=(1, 200), prefill_chunks=(40, 25))
    rows, qrows = (30, 41), (16, 16, 16, 23)
    c = Case(w, max_tokens=80, sched=ns.make_sched(nano_rows=rows, qkv_rows=qrows, overlap=True, cu_mask_frac=frac))
    try:
        say(f"  CU mask fraction {frac}: overlapped step")
        over = c.step().cpu()
        # the same split on the caller's stream (the mask is fixed at creation)
        ns.ns_engine_set_sched(c.h.eng, ns.make_sched(nano_rows=rows, qkv_rows=qrows))
        c.reset_cache()
        serial = c.step().cpu()
        torch.testing.assert_close(over, serial, rtol=0, atol=0)
        ns.ns_engine_set_sched(c.h.eng, ns.make_sched(nano_rows=rows, qkv_rows=qrows, overlap=True))
        out = torch.empty_like(over).cuda()
        stream = torch.cuda.Stream()
        g = ns.ns_graph_capture(c.h.eng, c.batch.n_rows, out.data_ptr(), stream)
        try:
            for _ in range(2):
                c.reset_cache()
                ns.ns_graph_replay(g, c.ns_batch(), stream)
                stream.synchronize()
                torch.testing.assert_close(out.cpu(), serial, rtol=0, atol=0)
        finally:
            ns.ns_graph_destroy(g)
    finally:
        c.close()

