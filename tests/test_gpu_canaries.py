"""Out-of-bounds guards on the device outputs: every buffer an entry point writes sits between
two 4 KB guard regions filled with a sentinel byte, and after the calls every guard byte is
unchanged (a write past either end of any output would show here even when the values the
parity tests compare are right)."""
import dataclasses

import numpy as np
import pytest
import torch

import quantized_kv_attention_amd as qkv
from gpu_helpers import Pair, say, to_dev_bf16
from quantized_kv_attention_amd import synth

pytestmark = pytest.mark.gpu

GB = 4096      # guard bytes on each side (keeps the 16-byte alignment the entry points check)
SENT = 0xA5


class Guarded:
    """A zeroed device tensor of `shape` inside a sentinel-filled byte buffer."""

    def __init__(self, shape, dtype, name):
        self.name = name
        nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.nbytes = nbytes
        self.buf = torch.full((nbytes + 2 * GB,), SENT, dtype=torch.uint8, device="cuda")
        self.t = self.buf[GB:GB + nbytes].view(dtype).view(shape)
        self.t.zero_()

    def check(self):
        lo = self.buf[:GB].cpu().numpy()
        hi = self.buf[GB + self.nbytes:].cpu().numpy()
        bad_lo = np.nonzero(lo != SENT)[0]
        bad_hi = np.nonzero(hi != SENT)[0]
        assert bad_lo.size == 0, f"{self.name}: {bad_lo.size} guard bytes before the buffer changed"
        assert bad_hi.size == 0, f"{self.name}: {bad_hi.size} guard bytes after the buffer changed"


@pytest.mark.parametrize("d,H,n", [(128, 3, 1000), (64, 2, 3000)])
def test_decode_step_outputs_stay_in_bounds(d, H, n):
    w = dataclasses.replace(synth.WORKLOADS["ctx4k"] if d == 128 else synth.WORKLOADS["tiny"], H=H)
    p = Pair(w, n=n, extra=70)
    b = p.bufs
    g = {}
    for name in ("o", "o_f32", "scores", "lse", "idx", "p_sel", "mass", "ws"):
        t = getattr(b, name)
        g[name] = Guarded(tuple(t.shape), t.dtype, name)
        setattr(b, name, g[name].t)
    p.run_gpu_loopwise(p.queries(0), w.n_dense, w.k_cols(n))
    for step in range(66):   # across a tail flush (fused into the attention calls)
        p.append(step)
    p.run_gpu_loopwise(p.queries(1), w.n_dense, w.k_cols(p.gpu.n_ctx))
    torch.cuda.synchronize()
    for x in g.values():
        x.check()
    say(f"  d={d} H={H} n={n}: {len(g)} guarded outputs intact")


def test_token_selection_outputs_stay_in_bounds():
    B, n, dm = 2, 3000, 256
    w = synth.WORKLOADS["tiny"]
    H = [np.stack([synth.gen_hidden(w, dm, n, bb)[r] for bb in range(B)]) for r in range(2)]
    k = 750
    score = Guarded((B, n), torch.float32, "score")
    out = Guarded((B, k), torch.int32, "act_out")
    nout = Guarded((B,), torch.int32, "n_act_out")
    nbef = Guarded((B,), torch.int32, "n_before")
    ws = Guarded((qkv.token_workspace_bytes(B, k),), torch.uint8, "ws")
    qkv.select_tokens(to_dev_bf16(H[1]), to_dev_bf16(H[0]), n, k, score.t, out.t, nout.t, ws.t, None, None, 1500,
                      nbef.t)
    torch.cuda.synchronize()
    for x in (score, out, nout, nbef, ws):
        x.check()


def test_gather_and_prefill_outputs_stay_in_bounds():
    L = qkv.lib()
    B, Hh, d, ld = 1, 2, 128, 700
    g = torch.Generator(device="cuda").manual_seed(5)
    src = (torch.randn((B, Hh, ld, d), generator=g, device="cuda")).to(torch.bfloat16)
    qpos = torch.tensor(np.sort(np.random.default_rng(1).choice(ld, 133, replace=False)).astype(np.int32)[None],
                        device="cuda")
    cpos = torch.tensor(np.stack([np.sort(np.random.default_rng(2 + h).choice(ld, 77, replace=False))
                                  for h in range(Hh)]).astype(np.int32)[None], device="cuda")
    nq, nc = qpos.shape[1], cpos.shape[2]
    ldt = ((nc + 31) // 32) * 32
    bufs = {}
    for name, idx, tr, shape in (("q", qpos, 0, (B, Hh, nq, d)), ("q0", qpos, 0, (B, Hh, nq, d)),
                                 ("k", cpos, 0, (B, Hh, nc, d)), ("k0", cpos, 0, (B, Hh, nc, d)),
                                 ("vt", cpos, 1, (B, Hh, d, ldt)), ("v0t", cpos, 1, (B, Hh, d, ldt))):
        dst = Guarded(shape, torch.bfloat16, f"gather {name}")
        per_head = 1 if idx.dim() == 3 else 0
        st = L.kv_gather_rows(qkv._ptr(src), B, Hh, ld, d, qkv._ptr(idx), idx.shape[-1], per_head, tr,
                              qkv._ptr(dst.t), None)
        assert st == 0, qkv.strerror(st)
        bufs[name] = dst
    lse0 = torch.zeros((B, Hh, nq), device="cuda")
    o0 = torch.zeros((B, Hh, nq, d), device="cuda")
    o32 = Guarded((B, Hh, nq, d), torch.float32, "o_f32")
    o16 = Guarded((B, Hh, nq, d), torch.bfloat16, "o")
    mass = Guarded((B, Hh, nq), torch.float32, "mass")
    qkv.attn_prefill_sparse(bufs["q"].t, bufs["q0"].t, qpos, lse0, o0, bufs["k"].t, bufs["k0"].t, bufs["vt"].t,
                            bufs["v0t"].t, cpos, 0.088, o32.t, o16.t, mass.t)
    torch.cuda.synchronize()
    for x in list(bufs.values()) + [o32, o16, mass]:
        x.check()


def test_export_plane_outputs_stay_in_bounds():
    w = dataclasses.replace(synth.WORKLOADS["ctx4k"], H=2)
    p = Pair(w, n=1000, extra=8)
    c = p.gpu
    L = qkv.lib()
    for loop, n_slots in ((1, 896), (3, 100), (4, 37)):
        d = c.d
        outs = [Guarded((n_slots, d), torch.uint8, "kc"), Guarded((n_slots, d), torch.uint8, "vc"),
                Guarded(((n_slots + 63) // 64, d), torch.float32, "ks"),
                Guarded(((n_slots + 63) // 64, d), torch.float32, "kz"),
                Guarded((n_slots, d // 64), torch.float32, "vs"), Guarded((n_slots, d // 64), torch.float32, "vz")]
        import ctypes
        st = L.qkv_export_plane(ctypes.byref(c.desc), loop, 0, 1, n_slots, *[qkv._ptr(x.t) for x in outs], None)
        assert st == 0, qkv.strerror(st)
        torch.cuda.synchronize()
        for x in outs:
            x.check()
