"""msa_decode_static (the decode entry point that allocates nothing) against
msa_decode on the same inputs, through the C ABI: two calls in a row, the
second on a smaller batch, each bit for bit equal to msa_decode's outputs."""
import numpy as np
import pytest
import torch

import synth
from tests import parity

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import decode_msa_index_amd as msa


def _static_outputs(dw, with_scores):
    w = dw.w
    scores = torch.full_like(dw.scores, 7.0) if with_scores else None
    topk = torch.full_like(dw.topk, -7)
    out = torch.full_like(dw.out, 3.0)
    lse = torch.full_like(dw.lse, 5.0)
    msa.decode_static(dw.p, dw.index_q, dw.ik_data, dw.ik_scales, dw.q, dw.kv_data,
                      dw.kv_scales, dw.block_table, dw.seq_lens, dw.q_pos, scores, topk, out,
                      lse)
    torch.cuda.synchronize()
    return scores, topk, out, lse


@pytest.mark.parametrize("kv", [synth.FP8, synth.NVFP4])
def test_static_scratch_decode_equals_workspace_decode(kv):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    big = synth.make("static-a", seed=301 + kv, seq_lens=[20000, 9000, 3000, 700, 65536],
                     q_dtype=synth.BF16, kv_dtype=kv, plant_per_seq=2)
    small = synth.make("static-b", seed=302 + kv, seq_lens=[5000, 129], q_dtype=synth.BF16,
                       kv_dtype=kv, plant_per_seq=1)
    for w, with_scores in ((big, False), (small, True)):
        dw = parity.DeviceWorkload(w)
        dw.decode(with_scores=True)
        torch.cuda.synchronize()
        ref = (dw.scores.clone(), dw.topk.clone(), dw.out.clone(), dw.lse.clone())
        print(f"[no-alloc] {w.name}: msa_decode_static, block_scores "
              f"{'given' if with_scores else 'NULL'}", flush=True)
        scores, topk, out, lse = _static_outputs(dw, with_scores)
        if with_scores:
            assert torch.equal(scores.view(torch.int32), ref[0].view(torch.int32))
        assert torch.equal(topk, ref[1])
        assert torch.equal(out.view(torch.int16), ref[2].view(torch.int16))
        assert torch.equal(lse.view(torch.int32), ref[3].view(torch.int32))
        assert msa.workspace_status(None) == 0


def test_static_scratch_key_block_chunk():
    """A 640-row prefill chunk small enough for the static scratch (G = 1,
    top-4: its key-block lists and partials take about 10.8 MB after the
    4.3 MB split zone), then a small decode batch on the same scratch: each
    bit for bit equal to msa_decode."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    R = 640
    qp = np.arange(3000 - R, 3000).astype(np.int32)
    chunk = synth.make("static-k2q", seed=311, seq_lens=[3000], rows_per_seq=R, q_pos=qp,
                       num_q_heads=16, num_groups=1, q_dtype=synth.BF16, kv_dtype=synth.FP8,
                       plant_per_seq=2, top_k=4)
    small = synth.make("static-c", seed=312, seq_lens=[5000, 129], q_dtype=synth.BF16,
                       kv_dtype=synth.FP8, plant_per_seq=1)
    for w in (chunk, small):
        dw = parity.DeviceWorkload(w)
        assert msa.workspace_bytes(dw.p, msa.OP_DECODE) <= (16 << 20)
        dw.decode(with_scores=True)
        torch.cuda.synchronize()
        ref = (dw.topk.clone(), dw.out.clone(), dw.lse.clone())
        print(f"[no-alloc] {w.name}: msa_decode_static", flush=True)
        _, topk, out, lse = _static_outputs(dw, False)
        assert torch.equal(topk, ref[0])
        assert torch.equal(out.view(torch.int16), ref[1].view(torch.int16))
        assert torch.equal(lse.view(torch.int32), ref[2].view(torch.int32))
        assert msa.workspace_status(None) == 0


def test_static_scratch_rejects_problems_beyond_its_size():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    p = msa.Problem(num_seqs=1, rows_per_seq=4096, max_blocks_per_seq=544,
                    num_phys_blocks=544)
    need = msa.workspace_bytes(p, msa.OP_DECODE)
    assert need > (16 << 20)
    with pytest.raises(msa.MsaError) as e:
        msa.decode_static(p, 0x1000, 0x1000, None, 0x1000, 0x1000, None, 0x1000, 0x1000,
                          0x1000, None, 0x1000, 0x1000, None)
    assert e.value.status == 3 and "msa_decode_static" in e.value.detail
