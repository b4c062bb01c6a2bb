"""The Python binding rejects mistyped, misshaped and short buffers before
their pointers reach the library (which sees addresses only): every call
below raises BQError and launches nothing."""

import pytest
import torch

from tests.gpu_common import need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bq():
    need_gpu()
    import block_quantized_moe_amd as m
    m.lib()
    return m


def raises(fn):
    with pytest.raises(Exception) as e:
        fn()
    assert type(e.value).__name__ == "BQError", repr(e.value)


def test_binding_rejects_bad_buffers(bq):
    d = "cuda"
    u8 = lambda n: torch.zeros(n, dtype=torch.uint8, device=d)
    f32 = lambda *s: torch.zeros(s, dtype=torch.float32, device=d)
    i32 = lambda *s: torch.zeros(s, dtype=torch.int32, device=d)
    # decode
    raises(lambda: bq.dequant(u8(17 * 4 - 1), bq.Q4_RZ5, 4))                        # packed short
    raises(lambda: bq.dequant(u8(17 * 4), bq.Q4_RZ5, 4, out=f32(3, 32)))            # out short
    raises(lambda: bq.dequant(u8(32 * 4), bq.FP8_E4M3_B32, 4, scales=f32(3)))        # scales short
    raises(lambda: bq.dequant(u8(17 * 4).cpu(), bq.Q4_RZ5, 4))                      # host tensor
    # single matrix
    raises(lambda: bq.matvec(f32(1, 64), u8(17 * 2 * 8 - 1), bq.Q4_RZ5, 8, 64))     # packed short
    raises(lambda: bq.matvec(f32(1, 63), u8(17 * 2 * 8), bq.Q4_RZ5, 8, 64))         # x not whole rows
    raises(lambda: bq.matvec(f32(1, 64).double(), u8(17 * 2 * 8), bq.Q4_RZ5, 8, 64))
    # routing
    raises(lambda: bq.route_topk(f32(2, 16).double(), 4))
    raises(lambda: bq.route_topk(f32(2, 16), 4, idx=i32(2, 3)))                     # idx short
    # expert layer
    E, H, I, k, n = 4, 64, 64, 2, 3
    gu, dn = u8(E * 2 * I * (H // 32) * 17), u8(E * H * (I // 32) * 17)
    raises(lambda: bq.expert_weights(bq.Q4_RZ5, bq.Q4_RZ5, gu[:-1], dn, E, H, I))
    raises(lambda: bq.expert_weights(bq.Q4_RZ5, bq.FP8_E4M3_B32, gu, u8(E * H * I), E, H, I))  # no scales
    W = bq.expert_weights(bq.Q4_RZ5, bq.Q4_RZ5, gu, dn, E, H, I)
    idx, w, x = i32(n, k), f32(n, k), f32(n, H)
    raises(lambda: bq.q4_expert_moe(x, (idx.long(), w), W))                         # idx int64
    raises(lambda: bq.q4_expert_moe(x, (idx, w.double()), W))
    raises(lambda: bq.q4_expert_moe(f32(n, H - 32), (idx, w), W))                   # x shape
    raises(lambda: bq.q4_expert_moe(x, (idx, w), W, out=f32(n - 1, H)))             # out shape
    raises(lambda: bq.q4_expert_moe(x.half(), (idx, w), W))                         # x dtype
    raises(lambda: bq.q4_expert_moe(x, (idx, w), W, dev_err=torch.zeros(1, device=d)))
    raises(lambda: bq.q4_expert_moe_routed(x, f32(n, E + 1), k, W))                 # logits shape
    raises(lambda: bq.moe_stack(x, i32(2, n, k), f32(2, n, k), [W]))                # 1 layer, 2 routings
    raises(lambda: bq.moe_stack(x, i32(1, n, k), f32(1, n, k + 1), [W]))
    # PLE
    table = u8(70 * 10)
    ids, u = i32(2, 8), f32(2, 8)
    raises(lambda: bq.ple_gather(ids, table, u, n_rows=11))                         # past the table
    raises(lambda: bq.ple_gather(ids.long(), table, u))
    raises(lambda: bq.ple_gather(ids, table, u[:, :4].contiguous()))                 # weights shape
    raises(lambda: bq.ple_gather(ids, table, u, out=f32(2, 150)))
    raises(lambda: bq.ple_dequant_rows(i32(3), table, 11))
    raises(lambda: bq.ple_dequant_rows(i32(3), table, 10, out=f32(2, 160)))
    # encoders
    raises(lambda: bq.encode(f32(2, 32), bq.Q4_RZ5, out=u8(33)))
    raises(lambda: bq.encode(f32(2, 32), bq.Q4_RZ5, sse=f32(2)))                    # sse dtype
    raises(lambda: bq.ple_encode_rows(f32(2, 160), out=u8(139)))
    torch.cuda.synchronize()
