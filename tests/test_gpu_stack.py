"""Whole-stack workload: 64 synthetic decoder blocks x (qkv, o, gate_up, down).

Each (block, layer type) has its own weight substream (layer index 4*block +
type); one activation tensor per layer type is shared by all blocks.  Decode runs
at b = 16, prefill with a 2048-token chunk.  Every layer is checked on sampled
outputs against the CPU oracle (64 random rows x all 16 decode tokens; 64 rows x
64 random prefill tokens, int32 accumulators bit-exact); blocks 0, 31 and 63 are
checked on every decode output and on all rows of 256 prefill tokens.

The oracle's inputs come from `synth` only: sampled code rows from the numpy
generator, whole layers from its torch twin (pinned equal to the numpy one in
tests/test_synth.py) because generating 180 M codes in numpy takes ~20 s.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from gpu_common import REL_TOL, announce, bf16_dev, dev, to_dev

pytestmark = pytest.mark.gpu

TYPES = [("qkv", 5120, 10240), ("o", 5120, 5120), ("gate_up", 5120, 34816), ("down", 17408, 5120)]
BLOCKS = 64
FULL_BLOCKS = (0, 31, 63)
B_DEC, M_PRE = 16, 2048
SAMPLE_ROWS, SAMPLE_TOKENS, FULL_TOKENS = 64, 64, 256


def _rows_codes(L, rows):
    return np.concatenate([L.codes(int(r), 1) for r in rows])


@pytest.mark.timeout(1200)
def test_stack64_decode_and_prefill():
    import torch
    import quantized_gemv_gemm_amd as tl

    d = dev()
    rng = np.random.default_rng(4)
    for ti, (name, K, N) in enumerate(TYPES):
        # activations of this layer type (shared by the 64 blocks)
        xd_bits = synth.activations(0, 4, ti, B_DEC, K)
        xp_bits = synth.activations(0, 4, len(TYPES) + ti, M_PRE, K)
        xr_dec = tl.hadamard_blk(bf16_dev(xd_bits, d))
        ws = torch.empty((tl.gemv_workspace_size(B_DEC, K, N),), dtype=torch.uint8, device=d)
        tl.gemv_prepare(xr_dec, ws)
        xq_d, sx_d = tl.quant_act_int8(tl.hadamard_blk(bf16_dev(xp_bits, d)))
        y_dec = torch.empty((B_DEC, N), dtype=torch.float32, device=d)
        y_pre = torch.empty((M_PRE, N), dtype=torch.float32, device=d)
        acc = torch.empty((M_PRE, N), dtype=torch.int32, device=d)

        # oracle activations: decode rotation in binary64; prefill tokens sampled
        xr_ref = oracle.rotate_exact(synth.bf16_bits_to_f32(xd_bits))
        tok_full = np.sort(rng.choice(M_PRE, FULL_TOKENS, replace=False))
        xp_f = synth.bf16_bits_to_f32(xp_bits[tok_full])
        xq_ref, sx_ref = oracle.quant_act_int8(oracle.rotate_exact(xp_f).astype(np.float32))
        torch.cuda.synchronize()
        got_xq = xq_d[torch.from_numpy(tok_full).to(d)].cpu().numpy()
        assert np.array_equal(got_xq, xq_ref), f"{name}: int8 activations differ"
        assert np.array_equal(sx_d.cpu().numpy()[tok_full], sx_ref)

        for blk in range(BLOCKS):
            layer = 4 * blk + ti
            announce(f"stack64 {name} block {blk} (layer {layer}) K={K} N={N}")
            L = synth.LayerInputs(0, 4, layer, K, N)
            scales = L.scales()
            codes_d = L.codes_torch(d)
            scales_d = to_dev(scales, d)
            packed, q, rs = tl.pack_weights(codes_d, scales_d)
            tl.gemv_prepared(ws, B_DEC, K, packed, scales_d, y_dec)
            tl.gemm_int8_rescale(xq_d, sx_d, packed, q, rs, out=y_pre, acc_out=acc)
            torch.cuda.synchronize()

            q_ref, rs_ref, _ = oracle.decompose_scales(scales)
            assert np.array_equal(q.cpu().numpy(), q_ref) and np.array_equal(rs.cpu().numpy(), rs_ref)
            if blk in FULL_BLOCKS:
                codes = codes_d.cpu().numpy()
                y_ref = oracle.gemv_ternary(xr_ref, codes, scales)
                assert oracle.rel_fro(y_dec.cpu().numpy(), y_ref) <= REL_TOL, (name, blk)
                tsel = torch.from_numpy(tok_full).to(d)
                acc_ref = oracle.gemm_int8_acc(xq_ref, codes, q_ref)
                assert np.array_equal(acc[tsel].cpu().numpy().astype(np.int64), acc_ref), (name, blk)
                e = oracle.rel_fro(y_pre[tsel].cpu().numpy(), oracle.rescale(acc_ref, rs_ref, sx_ref))
                assert e <= REL_TOL, (name, blk, e)
            else:
                rows = np.sort(rng.choice(N, SAMPLE_ROWS, replace=False))
                tpos = np.sort(rng.choice(FULL_TOKENS, SAMPLE_TOKENS, replace=False))
                codes_r = _rows_codes(L, rows)
                y_ref = oracle.gemv_ternary(xr_ref, codes_r, scales[rows])
                rsel = torch.from_numpy(rows).to(d)
                assert oracle.rel_fro(y_dec[:, rsel].cpu().numpy(), y_ref) <= REL_TOL, (name, blk)
                acc_ref = oracle.gemm_int8_acc(xq_ref[tpos], codes_r, q_ref[rows])
                tsel = torch.from_numpy(tok_full[tpos]).to(d)
                got = acc[tsel][:, rsel].cpu().numpy().astype(np.int64)
                assert np.array_equal(got, acc_ref), (name, blk)
                e = oracle.rel_fro(y_pre[tsel][:, rsel].cpu().numpy(),
                                   oracle.rescale(acc_ref, rs_ref[rows], sx_ref[tpos]))
                assert e <= REL_TOL, (name, blk, e)
            del packed, q, rs, codes_d, scales_d
