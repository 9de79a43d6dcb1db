"""select_tokens against the oracle (explainer section 3, cross-loop token-sparse updates):
change scores within 1e-4 relative of the fp64 oracle, the kept set bit-exact when the
oracle ranks the GPU's own fp32 scores (ties to the lower index), identical untaught sets
where the k-th and (k+1)-th scores are gapped, nesting, and the lists feeding
kv_encode_loop directly, with planes bit-exact against an oracle cache built from the same
active sets."""
import math

import numpy as np
import pytest
import torch

import oracle as orc
import quantized_kv_attention_amd as qkv
from gpu_helpers import compare_planes, say, to_dev_bf16
from quantized_kv_attention_amd import cache as qcache
from quantized_kv_attention_amd import synth

pytestmark = pytest.mark.gpu


def run_select(Hc, Hp, n, k, act_prev=None, n_prev=None, split=0):
    """Hc, Hp: uint16 [B, n, dm] host; act_prev int32 [B, ld] host or None."""
    B = Hc.shape[0]
    hc, hp = to_dev_bf16(Hc), to_dev_bf16(Hp)
    score = torch.zeros((B, n), dtype=torch.float32, device="cuda")
    out = torch.full((B, k), -5, dtype=torch.int32, device="cuda")
    nout = torch.zeros(B, dtype=torch.int32, device="cuda")
    nbef = torch.zeros(B, dtype=torch.int32, device="cuda")
    ws = torch.zeros(qkv.token_workspace_bytes(B, k), dtype=torch.uint8, device="cuda")
    ap = None if act_prev is None else torch.from_numpy(np.ascontiguousarray(act_prev)).cuda()
    npv = None if n_prev is None else torch.from_numpy(np.ascontiguousarray(n_prev, np.int32)).cuda()
    qkv.select_tokens(hc, hp, n, k, score, out, nout, ws, ap, npv, split, nbef)
    torch.cuda.synchronize()
    return score.cpu().numpy(), out.cpu().numpy(), nout.cpu().numpy(), nbef.cpu().numpy(), out


def check_against_oracle(Hc, Hp, n, k, prev_mask, got, label):
    """prev_mask: bool [B, n] or None.  Returns the kept masks [B, n]."""
    score, out, nout, nbef, _ = got
    B = Hc.shape[0]
    kept = np.zeros((B, n), bool)
    gapped = 0
    for b in range(B):
        pm = None if prev_mask is None else prev_mask[b]
        ref = orc.token_change(orc.bf16_bits_to_f32(Hc[b]), orc.bf16_bits_to_f32(Hp[b]), pm)
        fin = np.isfinite(ref)
        assert np.array_equal(np.isneginf(score[b]), np.isneginf(ref)), f"{label}: -inf pattern b={b}"
        np.testing.assert_allclose(score[b][fin], ref[fin], rtol=1e-4, atol=0, err_msg=f"{label}: scores b={b}")
        # teacher-forced: the oracle ranks the GPU's fp32 scores
        idx_tf = orc.select_tokens(orc.bf16_bits_to_f32(Hc[b]), orc.bf16_bits_to_f32(Hp[b]), pm, k,
                                   scores_f32=score[b])
        assert nout[b] == idx_tf.size, f"{label}: count b={b}"
        assert np.array_equal(out[b, :nout[b]], idx_tf), f"{label}: kept tokens b={b}"
        if pm is not None:
            assert pm[out[b, :nout[b]]].all(), f"{label}: not nested b={b}"
        # untaught: identical where the k-th and (k+1)-th oracle scores are gapped
        idx_u = orc.select_tokens(orc.bf16_bits_to_f32(Hc[b]), orc.bf16_bits_to_f32(Hp[b]), pm, k)
        top = np.sort(ref[fin])[::-1]
        if idx_u.size < top.size and top[idx_u.size - 1] - top[idx_u.size] > 1e-3 * top[idx_u.size - 1]:
            gapped += 1
            assert np.array_equal(idx_u, idx_tf), f"{label}: gapped untaught selection b={b}"
        kept[b, out[b, :nout[b]]] = True
    say(f"  {label}: kept {nout.tolist()}, gapped sequences asserted identical: {gapped}")
    return kept


@pytest.mark.parametrize("n,dm,B", [(256, 64, 2), (3000, 256, 3), (32768, 2048, 1)])
def test_nested_selection_loops_3_and_4(n, dm, B):
    w = synth.WORKLOADS["tiny"]
    H = [np.stack([synth.gen_hidden(w, dm, n, b)[r] for b in range(B)]) for r in range(w.R)]
    k3, k4 = math.ceil(0.25 * n), math.ceil(0.10 * n)
    say(f"select_tokens n={n} dm={dm} B={B}: loop 3 keeps {k3}, loop 4 keeps {k4}")
    # loop 3: ranks every token (loop 2 was dense) by the change of loop 2
    g3 = run_select(H[1], H[0], n, k3)
    m3 = check_against_oracle(H[1], H[0], n, k3, None, g3, "loop 3")
    # loop 4: ranks loop 3's active tokens by the change of loop 3
    ld = k3
    ap = np.zeros((B, ld), np.int32)
    for b in range(B):
        ap[b, :m3[b].sum()] = np.nonzero(m3[b])[0]
    g4 = run_select(H[2], H[1], n, k4, ap, m3.sum(1), split=n // 2)
    m4 = check_against_oracle(H[2], H[1], n, k4, m3, g4, "loop 4")
    for b in range(B):
        assert g4[3][b] == int(np.sum(np.nonzero(m4[b])[0] < n // 2)), "count below the split"
    # k above the preceding set keeps exactly that set
    g5 = run_select(H[3], H[2], n, min(n, 2 * k4), np.pad(np.stack([np.nonzero(m)[0] for m in m4]).astype(np.int32),
                                                        ((0, 0), (0, 0))), m4.sum(1))
    for b in range(B):
        assert np.array_equal(g5[1][b, :g5[2][b]], np.nonzero(m4[b])[0])
    # the same over more than one compaction pass (8192 entries each): k above loop 3's set
    k6 = min(n, k3 + 8192 + 7)
    g6 = run_select(H[3], H[2], n, k6, ap, m3.sum(1), split=n // 3)
    for b in range(B):
        assert np.array_equal(g6[1][b, :g6[2][b]], np.nonzero(m3[b])[0])
        assert g6[3][b] == int(np.sum(np.nonzero(m3[b])[0] < n // 3)), "count below the split"


def test_ties_and_zero_states():
    n, dm = 300, 64
    Hp = np.zeros((1, n, dm), np.float32)
    Hp[0, :, 0] = 1.0
    Hc = Hp.copy()
    Hc[0, ::3, 1] = 0.5           # a hundred equal changes
    Hp[0, 7] = 0.0                # zero previous states: +inf with a change, 0 without
    Hc[0, 7] = 0.0
    Hc[0, 7, 3] = 1.0
    Hp[0, 8] = 0.0
    Hc[0, 8] = 0.0
    Hcb, Hpb = synth.bf16_round_bits(Hc), synth.bf16_round_bits(Hp)
    g = run_select(Hcb, Hpb, n, 40)
    check_against_oracle(Hcb, Hpb, n, 40, None, g, "ties")
    assert g[1][0, 0] == 0 and 7 in g[1][0, :40] and np.isinf(g[0][0, 7]) and g[0][0, 8] == 0.0


def test_selected_lists_feed_the_encoder():
    """The kept lists go to kv_encode_loop as they are (body part counted by n_before); the
    planes equal those of an oracle cache built with the same active sets."""
    w = synth.WORKLOADS["tiny"]
    B, n, dm = 2, 700, 128
    w = synth.Workload("tokens", B, 2, 64, n, 4, [0.3, 0.1, 0.05], [1, 1, 0.25, 0.10], 2, 0.10, 1, 20261001)
    H = [np.stack([synth.gen_hidden(w, dm, n, b)[r] for b in range(B)]) for r in range(w.R)]
    nb = qkv.body_len(n)
    k3, k4 = math.ceil(0.25 * n), math.ceil(0.10 * n)
    _, _, n3, nb3, out3 = run_select(H[1], H[0], n, k3, split=nb)
    m3 = np.zeros((B, n), bool)
    o3 = out3.cpu().numpy()
    for b in range(B):
        m3[b, o3[b, :n3[b]]] = True
    _, _, n4, nb4, out4 = run_select(H[2], H[1], n, k4, o3, n3, split=nb)
    m4 = np.zeros((B, n), bool)
    o4 = out4.cpu().numpy()
    for b in range(B):
        m4[b, o4[b, :n4[b]]] = True
    act = [np.ones((B, n), bool), np.ones((B, n), bool), m3, m4]
    K, V = [], []
    for r in range(w.R):
        K.append(np.zeros((B, w.H, n, w.d), np.uint16))
        V.append(np.zeros((B, w.H, n, w.d), np.uint16))
    for b in range(B):
        for h in range(w.H):
            kk, vv = synth.gen_head_kv(w, b, h, act, n)
            for r in range(w.R):
                K[r][b, h], V[r][b, h] = kk[r], vv[r]
    cap = 768
    g = qcache.LayerCache(B, w.H, w.d, w.R, cap)
    Kd = [to_dev_bf16(x) for x in K]
    Vd = [to_dev_bf16(x) for x in V]
    for r in range(w.R):
        if r < 2:
            qkv.kv_encode_loop(g, r + 1, 0, nb, k_src=Kd[r][:, :, :nb].contiguous(), v_src=Vd[r][:, :, :nb].contiguous())
            continue
        out, cnt = (out3, nb3) if r == 2 else (out4, nb4)
        # rows of the kept body tokens, in list order (gathered with torch; the list itself is
        # passed to the encoder unchanged)
        ks = torch.zeros((B, w.H, nb, w.d), dtype=torch.bfloat16, device="cuda")
        vs = torch.zeros_like(ks)
        for b in range(B):
            c = int(cnt[b])
            rows = out[b, :c].long()
            ks[b, :, :c] = Kd[r][b].index_select(1, rows)
            vs[b, :, :c] = Vd[r][b].index_select(1, rows)
        cnt_d = torch.from_numpy(np.ascontiguousarray(cnt, np.int32)).cuda()
        qkv.kv_encode_loop(g, r + 1, 0, nb, out, cnt_d, ks, vs)
    torch.cuda.synchronize()
    oc = orc.OracleCache(B, w.H, w.d, w.R, cap)
    oc.prefill(K, V, act)
    compare_planes(g, oc, range(w.H), range(w.H))
    say(f"  encoder fed by select_tokens: planes bit-exact (body {nb}, kept {n3.tolist()} / {n4.tolist()})")
