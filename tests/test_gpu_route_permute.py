"""GPU routing and grouping against the oracle, bit for bit, across the routing kernels (one
wave per token; one 16-lane row per token from 16384 tokens) and the permute's code paths:
the atomic-free one-workgroup permute (at most 8192 slots and 63 local experts; chunk
prefixes over one or two wave-wide passes), the one-workgroup permute with a one-wave
bucket scan (more slots, at most 63 local experts) or the block scan (64 to 256 local
experts), several rounds of 1024 slots, and the chunked multi-workgroup permute (more than
16384 slots or more than 256 local experts; ballot-ranked chunks for at most 63 local
experts, over several wave-wide passes of the chunk scan)."""
import numpy as np
import pytest

from moe_expert_layer_amd import synth
from oracle import moe_oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests import gpu_util as G
    from moe_expert_layer_amd import binding as B

CASES = [  # tokens, experts, local_begin, local, topk
    (100, 64, 0, 63, 4),      # 64 buckets: atomic-free permute, bucket boundary
    (600, 64, 5, 50, 8),      # 4800 slots = 75 chunks: the chunk prefix carries into a second pass
    (1024, 64, 3, 40, 8),     # 8192 slots = 128 chunks: largest atomic-free case
    (1025, 64, 3, 40, 8),     # 8200 slots: one-workgroup permute with the one-wave bucket scan
    (100, 128, 10, 64, 4),    # 65 buckets: block scan, boundary
    (700, 256, 0, 256, 8),    # 257 buckets: largest one-workgroup case, several rounds
    (2048, 64, 3, 40, 8),     # 16384 slots exactly: sixteen rounds
    (2049, 64, 3, 40, 8),     # one slot more: chunked permute
    (64, 1024, 500, 300, 16), # 301 buckets: chunked permute
    (33000, 64, 3, 40, 8),    # 264000 slots = 258 chunks of 1024: the chunk scan carries over five passes
    (8192, 64, 3, 40, 8),     # 65536 slots = 64 chunks exactly
    (8193, 64, 3, 40, 8),     # 65 chunks, the last one of 8 slots
    # 16384 tokens or more: routing with one 16-lane row per token (1, 2 and 8 keys per lane)
    (16384, 16, 0, 16, 4),
    (16400, 32, 0, 20, 3),
    (16384, 100, 10, 40, 16),
    (1, 8, 0, 8, 1),          # a single slot
    (512, 32, 0, 32, 4),      # the oai share's routing shape
    (1024, 8, 0, 8, 8),       # every expert taken
    (257, 33, 1, 30, 5),      # expert count not a multiple of 4
    (256, 64, 0, 63, 16),     # largest k
    (128, 256, 0, 32, 8),     # the decode share's routing shape
    (1000, 16, 0, 16, 8),
]


@pytest.mark.parametrize("T,E,e0,EL,k", CASES)
def test_route_permute_bit_exact(T, E, e0, EL, k):
    G.say(f"[route] T={T} E={E} e0={e0} EL={EL} k={k}")
    rng = np.random.default_rng(T * 7 + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, ::5] = np.round(logits[:, ::5])  # exact ties
    w = synth.shrink(synth.workload("tiny"), tokens=T, num_experts=E, local_begin=e0, num_local=EL, topk=k)
    d = B.desc_from_workload(w)
    ws = B.alloc_workspace(d)
    i32 = lambda *s: torch.empty(s, dtype=torch.int32, device="cuda")
    ids, tw = i32(T, k), torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts, offsets, r2s, s2r = i32(EL), i32(EL + 1), i32(T * k), i32(T * k)
    r2s.fill_(-7)
    B.moe_route_permute(d, torch.from_numpy(logits).cuda(), ids, tw, counts, offsets, r2s, s2r, ws)
    torch.cuda.synchronize()
    rid, rw = O.route(logits, k)
    rc, ro, rr, rs = O.permute(rid, e0, EL)
    got = {"topk_ids": ids.cpu().numpy(), "topk_w": tw.cpu().numpy(), "counts": counts.cpu().numpy(),
           "offsets": offsets.cpu().numpy(), "row_to_slot": r2s.cpu().numpy(), "slot_to_row": s2r.cpu().numpy()}
    G.check_routing(got, {"topk_ids": rid, "topk_w": rw, "counts": rc, "offsets": ro, "row_to_slot": rr,
                          "slot_to_row": rs})
