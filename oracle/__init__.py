"""Plain CPU oracle for quantized cross-loop decode attention (FlashLoop).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the HIP path (``quantized_kv_attention_amd``) and never imports it.

The arithmetic lives in ``oracle.c`` (fp64 attention, exact fp32 codec); this module
marshals numpy arrays into it and keeps the per-loop cache state of one layer the
way the pages describe it:

* project page, The Method, STEP 01: inactive tokens keep the previous loop's K/V;
* project page, STEP 03, and flozi.net explainer section 3: loop 1 is stored as an
  INT4 base, each later loop as the INT4 residual against the previous loop's
  *reconstruction*, for active tokens only; keys per channel over 64 tokens, values
  per token over 64 channels; the most recent tokens stay in BF16;
* project page, STEP 02, and explainer section 3: sparse loops pick the top-K columns
  of the preceding loop's distribution, cache their mass m, and correct the preceding
  output for those columns only;
* PyPI page, Configuration: dense loops 1-2, 4-bit, group 64, 64-token BF16 tail.

Readings taken where the pages are silent (geometry of the BF16 tail, K grouping
over stored rows, the splice formula) are stated next to the code that takes them.
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import build as _build

GROUP = 64
TAIL_MIN = 64

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        L = ctypes.CDLL(path)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        i32p = ctypes.POINTER(ctypes.c_int32)
        L.orc_quantize_group.argtypes = [f32p, ctypes.c_int, ctypes.c_long, ctypes.c_int, u8p, ctypes.c_long, f32p,
                                         f32p]
        L.orc_quantize_group.restype = None
        L.orc_dequant.argtypes = [ctypes.c_uint8, ctypes.c_float, ctypes.c_float]
        L.orc_dequant.restype = ctypes.c_float
        L.orc_encode_rows.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, f32p, f32p, u8p, f32p,
                                      f32p, f32p]
        L.orc_encode_rows.restype = None
        L.orc_attend_dense.argtypes = [ctypes.c_int, ctypes.c_int, f32p, ctypes.c_double, f32p, f32p, f64p, f64p, f64p]
        L.orc_attend_dense.restype = None
        L.orc_select.argtypes = [ctypes.c_int, f32p, ctypes.c_double, ctypes.c_int, i32p, f64p, f64p]
        L.orc_select.restype = ctypes.c_int
        L.orc_attend_sparse.argtypes = [ctypes.c_int, ctypes.c_int, f32p, ctypes.c_double, f32p, f32p, f32p,
                                        i32p, ctypes.c_int, f64p, ctypes.c_double, f64p, ctypes.c_double, f64p, f64p]
        L.orc_attend_sparse.restype = None
        L.orc_token_change.argtypes = [ctypes.c_int, ctypes.c_int, f32p, f32p, u8p, f64p]
        L.orc_token_change.restype = None
        L.orc_prefill_sparse.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, f32p, f32p, i32p, f64p, f64p,
                                         f32p, f32p, f32p, f32p, i32p, ctypes.c_double, f64p, f64p]
        L.orc_prefill_sparse.restype = None
        L.orc_rebuild_plane.argtypes = [ctypes.c_int, ctypes.c_int, i32p, u8p, f32p, f32p, u8p, f32p, f32p,
                                        ctypes.c_int, f32p, f32p]
        L.orc_rebuild_plane.restype = None
        _lib = L
    return _lib


def _p(a, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly (bf16 is the top half of fp32)."""
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to bf16, nearest-even, via fp32 (the output format of the attention)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


# ----------------------------------------------------------------------------------
# Codec (explainer section 3: asymmetric INT4, group 64; 2-bit codes for the residual
# precision setting of the project page's "Main Results" sweep)
# ----------------------------------------------------------------------------------
def quantize_group(x: np.ndarray, bits: int = 4):
    x = np.ascontiguousarray(x, dtype=np.float32)
    m = x.shape[0]
    codes = np.zeros(m, np.uint8)
    s = np.zeros(1, np.float32)
    z = np.zeros(1, np.float32)
    lib().orc_quantize_group(_p(x, ctypes.c_float), m, 1, int(bits), _p(codes, ctypes.c_uint8), 1,
                             _p(s, ctypes.c_float), _p(z, ctypes.c_float))
    return codes, s[0], z[0]


def dequant(codes: np.ndarray, s, z) -> np.ndarray:
    L = lib()
    c = np.asarray(codes, np.uint8)
    out = np.empty(c.shape, np.float32)
    for i, v in np.ndenumerate(c):
        out[i] = L.orc_dequant(int(v), float(np.float32(s)), float(np.float32(z)))
    return out


def encode_rows(X: np.ndarray, P, is_key: bool, bits: int = 4):
    """Encode one call's stored rows (ascending positions) of one (sequence, head):
    X - P quantized with `bits`-bit codes (P None: X itself).

    Returns codes [nrows,d] u8, s, z (keys: [ceil(nrows/64), d]; values: [nrows, d/64])
    and the new reconstruction R [nrows, d] f32.
    """
    X = np.ascontiguousarray(X, dtype=np.float32)
    nrows, d = X.shape
    codes = np.zeros((nrows, d), np.uint8)
    if is_key:
        ng = (nrows + GROUP - 1) // GROUP
        s = np.zeros((ng, d), np.float32)
        z = np.zeros((ng, d), np.float32)
    else:
        s = np.zeros((nrows, d // GROUP), np.float32)
        z = np.zeros((nrows, d // GROUP), np.float32)
    R = np.zeros((nrows, d), np.float32)
    if nrows == 0:
        return codes, s, z, R
    Pp = None
    if P is not None:
        P = np.ascontiguousarray(P, dtype=np.float32)
        Pp = _p(P, ctypes.c_float)
    lib().orc_encode_rows(nrows, d, 1 if is_key else 0, int(bits), _p(X, ctypes.c_float), Pp,
                          _p(codes, ctypes.c_uint8), _p(s, ctypes.c_float), _p(z, ctypes.c_float),
                          _p(R, ctypes.c_float))
    return codes, s, z, R


# ----------------------------------------------------------------------------------
# Attention, selection, splice
# ----------------------------------------------------------------------------------
def attend_dense(q, K, V, sm: float = 1.0):
    q = np.ascontiguousarray(q, np.float32)
    K = np.ascontiguousarray(K, np.float32)
    V = np.ascontiguousarray(V, np.float32)
    n, d = K.shape
    o = np.zeros(d, np.float64)
    sc = np.zeros(n, np.float64)
    lse = np.zeros(1, np.float64)
    lib().orc_attend_dense(n, d, _p(q, ctypes.c_float), float(sm), _p(K, ctypes.c_float),
                           _p(V, ctypes.c_float), _p(o, ctypes.c_double), _p(sc, ctypes.c_double),
                           _p(lse, ctypes.c_double))
    return o, sc, float(lse[0])


def select(scores_f32, lse: float, k: int):
    s = np.ascontiguousarray(scores_f32, np.float32)
    n = s.shape[0]
    kk = max(0, min(int(k), n))
    idx = np.zeros(max(kk, 1), np.int32)
    p = np.zeros(max(kk, 1), np.float64)
    m = np.zeros(1, np.float64)
    got = lib().orc_select(n, _p(s, ctypes.c_float), float(lse), int(k), _p(idx, ctypes.c_int32),
                           _p(p, ctypes.c_double), _p(m, ctypes.c_double))
    return idx[:got].copy(), p[:got].copy(), float(m[0])


def attend_sparse(q, Kr, Vr, Vrm1, idx, p_sel, mass: float, o_prev, lse: float, scores, sm: float = 1.0):
    """Returns (o^(r) f64 [d], updated copy of scores f64 [n])."""
    q = np.ascontiguousarray(q, np.float32)
    Kr = np.ascontiguousarray(Kr, np.float32)
    Vr = np.ascontiguousarray(Vr, np.float32)
    Vrm1 = np.ascontiguousarray(Vrm1, np.float32)
    idx = np.ascontiguousarray(idx, np.int32)
    p_sel = np.ascontiguousarray(p_sel, np.float64)
    o_prev = np.ascontiguousarray(o_prev, np.float64)
    sc = np.array(scores, dtype=np.float64, copy=True)
    n, d = Kr.shape
    o = np.zeros(d, np.float64)
    k = idx.shape[0]
    if k == 0:
        idx = np.zeros(1, np.int32)
        p_sel = np.zeros(1, np.float64)
    lib().orc_attend_sparse(n, d, _p(q, ctypes.c_float), float(sm), _p(Kr, ctypes.c_float),
                            _p(Vr, ctypes.c_float), _p(Vrm1, ctypes.c_float), _p(idx, ctypes.c_int32), k,
                            _p(p_sel, ctypes.c_double), float(mass), _p(o_prev, ctypes.c_double),
                            float(lse), _p(sc, ctypes.c_double), _p(o, ctypes.c_double))
    return o, sc


# ----------------------------------------------------------------------------------
# Token selection (explainer section 3, cross-loop token-sparse updates; project page
# STEP 01): rank the tokens active in the preceding loop by their normalized hidden-state
# change and keep the top k; the kept set is the next loop's active set.
# ----------------------------------------------------------------------------------
def token_change(H_cur, H_prev, act_prev=None):
    """fp64 score per token: ||H_cur - H_prev|| / ||H_prev|| (see orc_token_change); -inf
    for tokens outside act_prev (bool [n], None = every token)."""
    Hc = np.ascontiguousarray(H_cur, np.float32)
    Hp = np.ascontiguousarray(H_prev, np.float32)
    n, dm = Hc.shape
    out = np.zeros(n, np.float64)
    a = None if act_prev is None else np.ascontiguousarray(act_prev, np.uint8)
    lib().orc_token_change(n, dm, _p(Hc, ctypes.c_float), _p(Hp, ctypes.c_float),
                           None if a is None else _p(a, ctypes.c_uint8), _p(out, ctypes.c_double))
    return out


def select_tokens(H_cur, H_prev, act_prev, k: int, scores_f32=None):
    """The next loop's active tokens, ascending: the min(k, |act_prev|) tokens of act_prev
    with the largest change score, ties to the lower index.  The ranking key is the score
    rounded to fp32, or `scores_f32` when given (to compare on identical scores)."""
    sc = token_change(H_cur, H_prev, act_prev).astype(np.float32) if scores_f32 is None else \
        np.asarray(scores_f32, np.float32)
    n_prev = int(np.asarray(act_prev).sum()) if act_prev is not None else sc.shape[0]
    kk = min(int(k), n_prev)
    idx, _, _ = select(sc, 0.0, kk)
    return idx


# ----------------------------------------------------------------------------------
# Prefill-side sparse loop over compact buffers (project page, The Method, after STEP 03;
# STEP 02; explainer section 3): active query rows against one selected column set.
# ----------------------------------------------------------------------------------
def prefill_sparse(Q, Q0, qpos, lse0, O0, K, V, K0, V0, cpos, sm: float = 1.0):
    """Returns (O f64 [nq, d], mass f64 [nq]); see orc_prefill_sparse."""
    f = lambda a: np.ascontiguousarray(a, np.float32)
    Q, Q0, K, V, K0, V0 = f(Q), f(Q0), f(K), f(V), f(K0), f(V0)
    qpos = np.ascontiguousarray(qpos, np.int32)
    cpos = np.ascontiguousarray(cpos, np.int32)
    lse0 = np.ascontiguousarray(lse0, np.float64)
    O0 = np.ascontiguousarray(O0, np.float64)
    nq, d = Q.shape
    nc = K.shape[0]
    O = np.zeros((nq, d), np.float64)
    mass = np.zeros(nq, np.float64)
    if nc == 0:
        K = V = K0 = V0 = np.zeros((1, d), np.float32)
        cpos = np.zeros(1, np.int32)
    lib().orc_prefill_sparse(nq, nc, d, _p(Q, ctypes.c_float), _p(Q0, ctypes.c_float), _p(qpos, ctypes.c_int32),
                             _p(lse0, ctypes.c_double), _p(O0, ctypes.c_double), _p(K, ctypes.c_float),
                             _p(V, ctypes.c_float), _p(K0, ctypes.c_float), _p(V0, ctypes.c_float),
                             _p(cpos, ctypes.c_int32), float(sm), _p(O, ctypes.c_double), _p(mass, ctypes.c_double))
    return O, mass


# ----------------------------------------------------------------------------------
# Geometry of the BF16 tail.  Reading: the tail holds the most recent T tokens with
# 64 <= T < 128 once the context has 64 tokens; when it would reach 128 the oldest 64
# are encoded as one group (PyPI Configuration "64-token BF16 residual tail";
# explainer section 3 "64 most-recent tokens kept BF16").
# ----------------------------------------------------------------------------------
def body_len(n: int) -> int:
    return GROUP * ((n - TAIL_MIN) // GROUP) if n >= TAIL_MIN else 0


class PlaneRecord:
    """Codes and metadata of one (sequence, head, loop), slot by slot, exactly as stored.

    Each encode call starts at a slot that is a multiple of 64; its last group is padded
    to 64 slots (codes 0, value metadata 0, position -1).
    """

    def __init__(self, d: int):
        self.d = d
        self.kc = np.zeros((0, d), np.uint8)
        self.vc = np.zeros((0, d), np.uint8)
        self.ks = np.zeros((0, d), np.float32)
        self.kz = np.zeros((0, d), np.float32)
        self.vs = np.zeros((0, d // GROUP), np.float32)
        self.vz = np.zeros((0, d // GROUP), np.float32)
        self.pos = np.zeros((0,), np.int32)

    def append(self, pos, kc, ks, kz, vc, vs, vz):
        n = len(pos)
        npad = ((n + GROUP - 1) // GROUP) * GROUP
        pad = npad - n
        d = self.d
        self.pos = np.concatenate([self.pos, np.asarray(pos, np.int32), np.full(pad, -1, np.int32)])
        self.kc = np.concatenate([self.kc, kc, np.zeros((pad, d), np.uint8)])
        self.vc = np.concatenate([self.vc, vc, np.zeros((pad, d), np.uint8)])
        self.ks = np.concatenate([self.ks, ks])
        self.kz = np.concatenate([self.kz, kz])
        self.vs = np.concatenate([self.vs, vs, np.zeros((pad, d // GROUP), np.float32)])
        self.vz = np.concatenate([self.vz, vz, np.zeros((pad, d // GROUP), np.float32)])


class OracleCache:
    """One layer's cross-loop K/V state for B sequences x H heads x R loops.

    Khat[r], Vhat[r] hold the loop-(r+1) reconstruction of every cached position
    (float32 [B, H, cap, d]): quantized chain for body positions, exact BF16 values in
    the tail.  act[r] is the loop's active-token mask per sequence ([B, cap] bool).

    Codec variants (the project page's "Main Results" precision sweep; the explainer's
    sections 4 and 5):
      residual_bits  bits of the residual planes of loops >= 2 (4, or 2); loop 1's base
                     is always 4-bit;
      full_state     True: every loop stores its own K/V quantized with 4-bit codes, not a
                     residual (the "Per-loop KIVI4" ablation row); an inactive row still
                     keeps the previous loop's reconstruction.
    """

    def __init__(self, B: int, H: int, d: int, R: int, cap: int, residual_bits: int = 4,
                 full_state: bool = False):
        assert residual_bits in (2, 4) and not (full_state and residual_bits != 4)
        self.residual_bits, self.full_state = residual_bits, full_state
        self.B, self.H, self.d, self.R, self.cap = B, H, d, R, cap
        self.n = 0
        self.nb = 0
        self.Khat = [np.zeros((B, H, cap, d), np.float32) for _ in range(R)]
        self.Vhat = [np.zeros((B, H, cap, d), np.float32) for _ in range(R)]
        self.Kin = [np.zeros((B, H, cap, d), np.float32) for _ in range(R)]  # loop inputs X^(r)
        self.Vin = [np.zeros((B, H, cap, d), np.float32) for _ in range(R)]
        self.act = [np.zeros((B, cap), bool) for _ in range(R)]
        self.planes = [[[PlaneRecord(d) for _ in range(R)] for _ in range(H)] for _ in range(B)]

    # -- encode positions [p0, p1) of every loop, in loop order (STEP 03) ------------
    def _encode_range(self, p0: int, p1: int):
        for r in range(self.R):
            for b in range(self.B):
                rows = p0 + np.nonzero(self.act[r][b, p0:p1])[0]
                for h in range(self.H):
                    out = {}
                    for name, Xin, Xhat in (("k", self.Kin, self.Khat), ("v", self.Vin, self.Vhat)):
                        X = Xin[r][b, h, rows]
                        P = None if (r == 0 or self.full_state) else Xhat[r - 1][b, h, rows]
                        bits = 4 if (r == 0 or self.full_state) else self.residual_bits
                        codes, s, z, Rc = encode_rows(X, P, is_key=(name == "k"), bits=bits)
                        out[name] = (codes, s, z)
                        # active rows: new reconstruction; inactive rows keep loop r-1's
                        if r > 0:
                            Xhat[r][b, h, p0:p1] = Xhat[r - 1][b, h, p0:p1]
                        Xhat[r][b, h, rows] = Rc
                    self.planes[b][h][r].append(rows, *out["k"], *out["v"])

    def _set_tail(self, p0: int, p1: int):
        """Tail positions keep this loop's exact BF16 value if active, else loop r-1's."""
        for r in range(self.R):
            for b in range(self.B):
                a = self.act[r][b, p0:p1]
                for X, Xin in ((self.Khat, self.Kin), (self.Vhat, self.Vin)):
                    src = Xin[r][b, :, p0:p1]
                    if r > 0:
                        src = np.where(a[None, :, None], src, X[r - 1][b, :, p0:p1])
                    X[r][b, :, p0:p1] = src

    def prefill(self, K, V, act):
        """K[r], V[r]: uint16 bf16 bits [B,H,n,d]; act[r]: bool [B,n] (loop-r active set)."""
        n = K[0].shape[2]
        for r in range(self.R):
            self.Kin[r][:, :, :n] = bf16_bits_to_f32(K[r])
            self.Vin[r][:, :, :n] = bf16_bits_to_f32(V[r])
            self.act[r][:, :n] = act[r]
        self.n = n
        self.nb = body_len(n)
        if self.nb > 0:
            self._encode_range(0, self.nb)
        self._set_tail(self.nb, n)

    def append(self, k_new, v_new):
        """Adds one generated token (active in every loop) at position n.

        If the tail would reach 128 tokens, its oldest 64 are first encoded, loop by loop.
        k_new[r], v_new[r]: uint16 bf16 bits [B,H,d].
        """
        t = self.n
        nb_new = body_len(t + 1)
        if nb_new > self.nb:
            self._encode_range(self.nb, nb_new)
            self.nb = nb_new
        for r in range(self.R):
            self.Kin[r][:, :, t] = bf16_bits_to_f32(k_new[r])
            self.Vin[r][:, :, t] = bf16_bits_to_f32(v_new[r])
            self.act[r][:, t] = True
        self.n = t + 1
        self._set_tail(t, t + 1)

    # -- reconstruction from the stored planes (the chain dequantisation of a decode step) --
    def rebuild(self, b: int, h: int):
        """Per loop, K and V reconstructions [n, d] of (b, h) rebuilt from the stored plane
        records alone (the loop's BF16 tail rows for tail positions), as a reader of the
        stored cache does each step: base plus residuals, or the last plane storing a
        position in the full-state codec."""
        n, d = self.n, self.d
        Ks, Vs = [], []
        Kx = np.zeros((self.cap, d), np.float32)
        Vx = np.zeros((self.cap, d), np.float32)
        for r in range(self.R):
            rec = self.planes[b][h][r]
            ns = rec.pos.size
            if ns:
                first = 1 if (r == 0 or self.full_state) else 0
                if first and r > 0:
                    Kx, Vx = Kx.copy(), Vx.copy()   # positions the plane does not store keep loop r-1
                lib().orc_rebuild_plane(ns, d, _p(rec.pos, ctypes.c_int32), _p(np.ascontiguousarray(rec.kc), ctypes.c_uint8),
                                        _p(np.ascontiguousarray(rec.ks), ctypes.c_float),
                                        _p(np.ascontiguousarray(rec.kz), ctypes.c_float),
                                        _p(np.ascontiguousarray(rec.vc), ctypes.c_uint8),
                                        _p(np.ascontiguousarray(rec.vs), ctypes.c_float),
                                        _p(np.ascontiguousarray(rec.vz), ctypes.c_float), first,
                                        _p(Kx, ctypes.c_float), _p(Vx, ctypes.c_float))
            Kr, Vr = Kx[:n].copy(), Vx[:n].copy()
            # tail rows: the loop's BF16 values (an inactive token holds loop r-1's)
            Kr[self.nb:n] = self.Khat[r][b, h, self.nb:n]
            Vr[self.nb:n] = self.Vhat[r][b, h, self.nb:n]
            Ks.append(Kr)
            Vs.append(Vr)
            Kx, Vx = Kx.copy(), Vx.copy()
        return Ks, Vs

    # -- one decode step over all loops (PyPI Configuration: dense loops, then sparse) --
    def step(self, q, n_dense: int, k: int, sm: float = 1.0, threads: int = 1, teacher=None,
             from_planes: bool = False):
        """Runs loops 1..R for query q[r] (uint16 bf16 bits [B,H,d]).

        Loops 1..n_dense are dense; later loops select k columns from the scores left by
        the preceding loop (spliced scores if it was sparse) and apply the sparse update.
        The selection key is the preceding scores rounded to fp32.  ``teacher`` may
        supply, per loop, the fp32 scores/lse to select from (to compare selection and
        splice on identical inputs).

        Returns a list over loops of dicts with o (f64 [B,H,d]), scores (f64 [B,H,n]),
        lse (f64 [B,H]) and, for sparse loops, idx/p_sel/mass.  from_planes: every head first
        rebuilds its reconstructions from the stored planes (rebuild), as a reader of the
        stored cache does, instead of taking the ones kept at encode time (same values).
        """
        B, H, d, n = self.B, self.H, self.d, self.n
        out = []
        state = {}

        def run_head(bh):
            b, h = bh
            res = []
            scores = lse = o_prev = None
            if from_planes:
                KK, VV = self.rebuild(b, h)
            for r in range(self.R):
                qf = bf16_bits_to_f32(q[r][b, h])
                Kr = KK[r] if from_planes else self.Khat[r][b, h, :n]
                Vr = VV[r] if from_planes else self.Vhat[r][b, h, :n]
                if r < n_dense:
                    o, scores, lse = attend_dense(qf, Kr, Vr, sm)
                    res.append(dict(o=o, scores=scores.copy(), lse=lse))
                else:
                    if teacher is not None and teacher[r] is not None:
                        sel_scores = teacher[r]["scores"][b, h, :n]
                        sel_lse = float(teacher[r]["lse"][b, h])
                        o_in = teacher[r]["o_prev"][b, h]
                        sc_in = np.asarray(sel_scores, np.float64)
                    else:
                        sel_scores = scores.astype(np.float32)
                        sel_lse = float(np.float32(lse))
                        o_in = o_prev
                        sc_in = scores
                    idx, p_sel, mass = select(sel_scores, sel_lse, k)
                    Vprev = VV[r - 1] if from_planes else self.Vhat[r - 1][b, h, :n]
                    o, scores = attend_sparse(qf, Kr, Vr, Vprev, idx, p_sel, mass, o_in, sel_lse, sc_in, sm)
                    lse = sel_lse
                    res.append(dict(o=o, scores=scores.copy(), lse=lse, idx=idx, p_sel=p_sel, mass=mass))
                o_prev = o
            state[bh] = res

        heads = [(b, h) for b in range(B) for h in range(H)]
        if threads > 1:
            with ThreadPoolExecutor(threads) as ex:
                list(ex.map(run_head, heads))
        else:
            for bh in heads:
                run_head(bh)
        for r in range(self.R):
            o = np.zeros((B, H, d))
            sc = np.zeros((B, H, n))
            lse = np.zeros((B, H))
            rec = dict(o=o, scores=sc, lse=lse)
            sparse = r >= n_dense
            if sparse:
                rec["idx"] = [[None] * H for _ in range(B)]
                rec["p_sel"] = [[None] * H for _ in range(B)]
                rec["mass"] = np.zeros((B, H))
            for (b, h) in heads:
                e = state[(b, h)][r]
                o[b, h] = e["o"]
                sc[b, h] = e["scores"]
                lse[b, h] = e["lse"]
                if sparse:
                    rec["idx"][b][h] = e["idx"]
                    rec["p_sel"][b][h] = e["p_sel"]
                    rec["mass"][b, h] = e["mass"]
            out.append(rec)
        return out
