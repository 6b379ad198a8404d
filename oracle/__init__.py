"""float64 CPU oracle for the ReplaySSM Mamba-2 decode step -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this package. The GPU
library and its Python binding never import it; the two share no code. Inputs are the exact fp32
values the GPU sees; every result is float64.

Functions (all arrays numpy, C-contiguous):
  step(S, x, B, C, dt, A, D) -> y              O1, one token, S (float64) updated in place
  spec_stepwise(S, T, x, B, C, dt, A, D, acc)  O5, the per-draft definition of spec decoding
  Replay(...)                                  O3 + O4, the replay form and its pointer machine
  bf16_encode / e4m3_encode_tiles / e4m3_encode_at / e4m3_decode / bf16_decode    O7
  mxfp4_encode / mxfp4_decode / mx_scale_code / e2m1_encode_scaled / e2m1_decode   O7 (MXFP4)
  philox4x32_10 / f16_encode / f16_decode      R8: the fp16 master's rounding and its random stream
  gdn_step(S, q, k, v, alpha, beta) -> o       O1g, one Gated DeltaNet token (oracle_gdn.c)
  gdn_spec_stepwise(...)                       O5g, per-draft spec decoding on GDN
  GDNReplay(...)                               O3g + O4, the GDN replay form and pointer machine
  mixer_edge / mixer_gate / silu / softplus    M1: the Mamba-2 mixer edges (oracle_mixer.c)
  MixerStepwise(...) / MixerReplay(...)        edge + O1 / O5 + gate; edge + replay form + gate

Pinning (what each function is checked against, independent of itself) is in tests/test_oracle_*.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_u32p = np.ctypeslib.ndpointer(np.uint32, flags="C_CONTIGUOUS")
_i = ctypes.c_int
_sz = ctypes.c_size_t


def lib():
    """Load liboracle.so, building it first if it is missing or older than its source. The
    environment variable RSSM_ORACLE_LIB names another build to load instead (the sanitizer
    build of the tests)."""
    global _lib
    if _lib is None:
        path = os.environ.get("RSSM_ORACLE_LIB")
        if not path:
            path = _LIB_PATH
            srcs = [os.path.join(_HERE, f) for f in ("oracle.c", "oracle_gdn.c", "oracle_mixer.c")]
            if not os.path.exists(path) or any(os.path.getmtime(path) < os.path.getmtime(f) for f in srcs):
                _build.build()
        L = ctypes.CDLL(path)
        L.oracle_step.argtypes = [_i] * 5 + [_f64p, _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _f64p]
        L.oracle_step.restype = None
        L.oracle_silu.argtypes = [ctypes.c_double]
        L.oracle_silu.restype = ctypes.c_double
        L.oracle_softplus.argtypes = [ctypes.c_double]
        L.oracle_softplus.restype = ctypes.c_double
        L.oracle_mixer_edge.argtypes = [_i] * 6 + [_f32p] * 10
        L.oracle_mixer_edge.restype = None
        L.oracle_mixer_gate.argtypes = [_sz, _f64p, _f32p, _f64p]
        L.oracle_mixer_gate.restype = None
        L.oracle_spec_stepwise.argtypes = [_i] * 6 + [_f64p, _f32p, _f32p, _f32p, _f32p, _f32p,
                                                      _f32p, _i32p, _f64p]
        L.oracle_spec_stepwise.restype = _i
        L.oracle_bf16_encode.argtypes = [ctypes.c_float]
        L.oracle_bf16_encode.restype = ctypes.c_uint16
        L.oracle_encode_bf16.argtypes = [_f32p, _u16p, _sz]
        L.oracle_encode_e4m3_tiles.argtypes = [_f32p, _u8p, _f32p, _sz, _sz]
        L.oracle_encode_e4m3_at.argtypes = [_f32p, _u8p, _sz, ctypes.c_float]
        L.oracle_e4m3_encode_sr.argtypes = [ctypes.c_float, ctypes.c_uint32]
        L.oracle_e4m3_encode_sr.restype = ctypes.c_uint8
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_float
        L.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_decode.restype = ctypes.c_float
        L.oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e2m1_decode.restype = ctypes.c_float
        L.oracle_encode_e2m1_scaled.argtypes = [_f64p, _u8p, _sz]
        L.oracle_mx_scale_code.argtypes = [_f32p, _sz]
        L.oracle_mx_scale_code.restype = ctypes.c_uint8
        L.oracle_encode_mxfp4.argtypes = [_f32p, _u8p, _u8p, _sz]
        L.oracle_decode_mxfp4.argtypes = [_u8p, _u8p, _f64p, _sz]
        L.oracle_replay_create.argtypes = [_i] * 8 + [_f32p, _f32p, _f32p, _i, ctypes.c_uint32]
        L.oracle_philox4x32_10.argtypes = [_u32p, _u32p, _u32p]
        L.oracle_f16_decode.argtypes = [ctypes.c_uint16]
        L.oracle_f16_decode.restype = ctypes.c_float
        L.oracle_encode_f16.argtypes = [_f32p, _u16p, _sz, _i, ctypes.c_void_p]
        L.oracle_replay_create.restype = ctypes.c_void_p
        L.oracle_replay_set_seq_ids.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)]
        L.oracle_replay_set_seq_ids.restype = None
        L.oracle_replay_destroy.argtypes = [ctypes.c_void_p]
        L.oracle_replay_step.argtypes = [ctypes.c_void_p, _f32p, _f32p, _f32p, _f32p, _f64p]
        L.oracle_replay_step.restype = _i
        L.oracle_replay_verify.argtypes = [ctypes.c_void_p, _i, _f32p, _f32p, _f32p, _f32p, _f64p]
        L.oracle_replay_verify.restype = _i
        L.oracle_replay_rollback.argtypes = [ctypes.c_void_p, _i32p]
        L.oracle_replay_rollback.restype = _i
        L.oracle_replay_flush.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_replay_flush.restype = _i
        L.oracle_replay_set_checkpoint.argtypes = [ctypes.c_void_p, _f32p, ctypes.c_void_p, _i]
        L.oracle_replay_set_checkpoint.restype = _i
        L.oracle_replay_master_fp8.argtypes = [ctypes.c_void_p, _u8p, _f32p]
        L.oracle_replay_master_fp8.restype = _i
        L.oracle_replay_set_master_fp8.argtypes = [ctypes.c_void_p, _u8p, _f32p, ctypes.c_void_p, _i]
        L.oracle_replay_set_master_fp8.restype = _i
        L.oracle_replay_pointers.argtypes = [ctypes.c_void_p, _i32p, _i32p]
        L.oracle_replay_checkpoint.argtypes = [ctypes.c_void_p, _f64p]
        L.oracle_replay_read_copy.argtypes = [ctypes.c_void_p, _f64p]
        L.oracle_replay_materialize.argtypes = [ctypes.c_void_p, _f64p]
        L.oracle_threads.restype = _i
        L.oracle_set_threads.argtypes = [_i]
        L.oracle_set_threads.restype = None
        L.oracle_gdn_step.argtypes = [_i] * 5 + [_f64p] + [_f32p] * 5 + [_f64p]
        L.oracle_gdn_spec_stepwise.argtypes = [_i] * 6 + [_f64p] + [_f32p] * 5 + [_i32p, _f64p]
        L.oracle_gdn_spec_stepwise.restype = _i
        L.oracle_gdn_create.argtypes = [_i] * 7 + [_f32p, _i]
        L.oracle_gdn_replay_read_copy.argtypes = [ctypes.c_void_p, _f64p]
        L.oracle_gdn_replay_read_copy.restype = None
        L.oracle_gdn_create.restype = ctypes.c_void_p
        L.oracle_gdn_destroy.argtypes = [ctypes.c_void_p]
        L.oracle_gdn_replay_step.argtypes = [ctypes.c_void_p] + [_f32p] * 5 + [_f64p]
        L.oracle_gdn_replay_step.restype = _i
        L.oracle_gdn_replay_verify.argtypes = [ctypes.c_void_p, _i] + [_f32p] * 5 + [_f64p]
        L.oracle_gdn_replay_verify.restype = _i
        L.oracle_gdn_replay_rollback.argtypes = [ctypes.c_void_p, _i32p]
        L.oracle_gdn_replay_rollback.restype = _i
        L.oracle_gdn_replay_flush.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_gdn_replay_flush.restype = _i
        L.oracle_gdn_replay_set_checkpoint.argtypes = [ctypes.c_void_p, _f32p]
        L.oracle_gdn_replay_set_checkpoint.restype = _i
        L.oracle_gdn_replay_pointers.argtypes = [ctypes.c_void_p, _i32p, _i32p]
        L.oracle_gdn_replay_checkpoint.argtypes = [ctypes.c_void_p, _f64p]
        L.oracle_gdn_replay_materialize.argtypes = [ctypes.c_void_p, _f64p]
        _lib = L
    return _lib


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS or the cores available)."""
    return int(lib().oracle_threads())


def set_threads(n: int) -> None:
    """Use n OpenMP threads from now on (timing the oracle on a given core count)."""
    lib().oracle_set_threads(int(n))


def step(S, x, B, C, dt, A, D):
    """O1 for one token. S: float64 [Bt,H,P,N], updated in place. Returns y float64 [Bt,H,P]."""
    assert S.dtype == np.float64 and S.flags.c_contiguous
    Bt, H, P, N = S.shape
    G = B.shape[1]
    y = np.empty((Bt, H, P), np.float64)
    lib().oracle_step(Bt, H, P, N, G, S, _f32(x), _f32(B), _f32(C), _f32(dt), _f32(A), _f32(D), y)
    return y


def spec_stepwise(S, T, x, B, C, dt, A, D, accepted):
    """O5: all T draft outputs from the committed state S (float64, updated to the accepted
    prefix). Inputs carry the draft index second: x [Bt,T,H,P], B/C [Bt,T,G,N], dt [Bt,T,H]."""
    Bt, H, P, N = S.shape
    G = B.shape[2]
    y = np.empty((Bt, T, H, P), np.float64)
    acc = np.ascontiguousarray(accepted, dtype=np.int32)
    rc = lib().oracle_spec_stepwise(Bt, H, P, N, G, T, S, _f32(x), _f32(B), _f32(C), _f32(dt),
                                    _f32(A), _f32(D), acc, y)
    if rc != 0:
        raise ValueError("accepted count outside [0, T]")
    return y


READ_FP32, READ_BF16, READ_FP8, READ_MXFP4 = 0, 1, 2, 3
MASTER_FP32, MASTER_FP16, MASTER_FP16_SR, MASTER_FP8, MASTER_FP8_SR = 0, 1, 2, 3, 4


class Replay:
    """O3 + O4: the replay form (checkpoint + records) with its pointer and flush machine."""

    def __init__(self, S0, A, D, G, L, Tmax=1, read_prec=READ_FP32, master_prec=MASTER_FP32, seed=0,
                 seq_ids=None):
        """seq_ids: the batch index each row of S0 stands for (default 0..Bt-1); it enters only
        the stochastic-rounding counter, so rows sampled from a larger batch round as there."""
        S0 = _f32(S0)
        self.Bt, self.H, self.P, self.N = S0.shape
        self.G, self.L, self.Tmax = G, L, Tmax
        self._h = lib().oracle_replay_create(self.Bt, self.H, self.P, self.N, G, L, Tmax,
                                             read_prec, S0, _f32(A), _f32(D), int(master_prec), int(seed))
        if not self._h:
            raise ValueError("invalid replay configuration")
        if seq_ids is not None:
            ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
            if ids.shape != (self.Bt,) or np.any(ids < 0):
                raise ValueError("seq_ids must hold Bt non-negative indices")
            lib().oracle_replay_set_seq_ids(self._h, ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))

    def __del__(self):
        if getattr(self, "_h", None):
            lib().oracle_replay_destroy(self._h)
            self._h = None

    def step(self, x, B, C, dt):
        y = np.empty((self.Bt, self.H, self.P), np.float64)
        if lib().oracle_replay_step(self._h, _f32(x), _f32(B), _f32(C), _f32(dt), y) != 0:
            raise RuntimeError("oracle replay: step rejected by the state machine")
        return y

    def verify(self, T, x, B, C, dt):
        y = np.empty((self.Bt, T, self.H, self.P), np.float64)
        if lib().oracle_replay_verify(self._h, T, _f32(x), _f32(B), _f32(C), _f32(dt), y) != 0:
            raise RuntimeError("oracle replay: verify rejected by the state machine")
        return y

    def rollback(self, accepted):
        acc = np.ascontiguousarray(accepted, dtype=np.int32)
        if lib().oracle_replay_rollback(self._h, acc) != 0:
            raise RuntimeError("oracle replay: rollback rejected by the state machine")

    def flush(self, seq_mask=None):
        if seq_mask is None:
            rc = lib().oracle_replay_flush(self._h, None)
        else:
            m = np.ascontiguousarray(seq_mask, dtype=np.int32)
            rc = lib().oracle_replay_flush(self._h, m.ctypes.data_as(ctypes.c_void_p))
        if rc != 0:
            raise RuntimeError("oracle replay: flush rejected by the state machine")

    def set_checkpoint(self, S, rows=None):
        """Continue from fp32 checkpoint values (taken as they are; records and pointers stay),
        with the read copy re-encoded from them: S [Bt,H,P,N] for every sequence, or S
        [len(rows),H,P,N] for the sequences listed in rows."""
        S = _f32(S)
        n = self.Bt if rows is None else len(rows)
        if S.shape != (n, self.H, self.P, self.N):
            raise ValueError("checkpoint shape mismatch")
        if rows is None:
            rc = lib().oracle_replay_set_checkpoint(self._h, S, None, n)
        else:
            idx = np.ascontiguousarray(rows, dtype=np.int32)
            rc = lib().oracle_replay_set_checkpoint(self._h, S, idx.ctypes.data_as(ctypes.c_void_p), n)
        if rc != 0:
            raise RuntimeError("oracle replay: set_checkpoint while a verify is pending, or a bad row")

    def fp8_master(self):
        """fp8 master (reading R9): E4M3FN codes uint8 [Bt,H,P,N] and fp32 scales
        [Bt,H,ceil(P/64)] (one per block of 64 rows)."""
        codes = np.empty((self.Bt, self.H, self.P, self.N), np.uint8)
        scales = np.empty((self.Bt, self.H, (self.P + 63) // 64), np.float32)
        if lib().oracle_replay_master_fp8(self._h, codes, scales) != 0:
            raise RuntimeError("oracle replay: not an fp8 master")
        return codes, scales

    def set_master_fp8(self, codes, scales, rows=None):
        """fp8 master: continue from codes [n,H,P,N] times scales [n,H,ceil(P/64)] (exact), for
        every sequence or for the sequences listed in rows (records and pointers stay)."""
        n = self.Bt if rows is None else len(rows)
        codes = np.ascontiguousarray(codes, np.uint8)
        scales = _f32(scales)
        if codes.shape != (n, self.H, self.P, self.N) or scales.shape != (n, self.H, (self.P + 63) // 64):
            raise ValueError("fp8 master shape mismatch")
        idx = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
        rc = lib().oracle_replay_set_master_fp8(self._h, codes, scales,
                                                None if idx is None else idx.ctypes.data_as(ctypes.c_void_p), n)
        if rc != 0:
            raise RuntimeError("oracle replay: set_master_fp8 while a verify is pending, a bad row, or not fp8")

    def pointers(self):
        pos = np.empty(self.Bt, np.int32)
        ck = np.empty(self.Bt, np.int32)
        lib().oracle_replay_pointers(self._h, pos, ck)
        return pos, ck

    def _state(self, fn):
        out = np.empty((self.Bt, self.H, self.P, self.N), np.float64)
        fn(self._h, out)
        return out

    def checkpoint(self):
        return self._state(lib().oracle_replay_checkpoint)

    def read_copy(self):
        return self._state(lib().oracle_replay_read_copy)

    def materialize(self):
        return self._state(lib().oracle_replay_materialize)


def bf16_encode(a):
    a = _f32(a)
    out = np.empty(a.shape, np.uint16)
    lib().oracle_encode_bf16(a.reshape(-1), out.reshape(-1), a.size)
    return out


def bf16_decode(codes):
    return (np.asarray(codes, np.uint16).astype(np.uint32) << 16).view(np.float32)


def e4m3_encode_tiles(a, tile_elems):
    """Per-tile scaled e4m3 encode (read-copy reading R6). Returns (codes uint8, scales f32)."""
    a = _f32(a).reshape(-1)
    ntiles = a.size // tile_elems
    codes = np.empty(a.size, np.uint8)
    scales = np.empty(ntiles, np.float32)
    lib().oracle_encode_e4m3_tiles(a, codes, scales, ntiles, tile_elems)
    return codes, scales


def e4m3_encode_rows(a):
    """The fp8 read copy of states a [..., P, N] (reading R6): one scale per block of 64
    consecutive rows p. Returns (codes uint8 [..., P, N], scales f32 [..., ceil(P/64)])."""
    a = _f32(a)
    P, N = a.shape[-2], a.shape[-1]
    lead = a.shape[:-2]
    flat = a.reshape(-1, P, N)
    nblk = (P + 63) // 64
    codes = np.empty(flat.shape, np.uint8)
    scales = np.empty((flat.shape[0], nblk), np.float32)
    for kb in range(nblk):
        p0, p1 = 64 * kb, min(64 * kb + 64, P)
        blk = np.ascontiguousarray(flat[:, p0:p1, :])
        c, sc = e4m3_encode_tiles(blk, (p1 - p0) * N)
        codes[:, p0:p1, :] = c.reshape(blk.shape)
        scales[:, kb] = sc
    return codes.reshape(a.shape), scales.reshape(*lead, nblk)


def e4m3_encode_at(a, inv_scale=1.0):
    a = _f32(a)
    out = np.empty(a.shape, np.uint8)
    lib().oracle_encode_e4m3_at(a.reshape(-1), out.reshape(-1), a.size, float(inv_scale))
    return out


def e4m3_encode_sr(a, r16):
    """E4M3FN codes (uint8) of fp32 values already divided by their scale, rounded
    stochastically with the 16-bit random integers r16 (reading R9)."""
    a = _f32(a).reshape(-1)
    r = np.asarray(r16, np.uint32).reshape(-1)
    assert r.size == a.size
    return np.array([lib().oracle_e4m3_encode_sr(float(x), int(y)) for x, y in zip(a, r)], np.uint8)


def e4m3_decode_table():
    """float32 value of each of the 256 codes (NaN for the two NaN codes)."""
    return np.array([lib().oracle_e4m3_decode(c) for c in range(256)], np.float32)


def e2m1_decode(code):
    """Value of a 4-bit OCP FP4 E2M1 code."""
    return float(lib().oracle_e2m1_decode(int(code) & 15))


def e2m1_encode_scaled(v):
    """E2M1 codes (uint8, one per value) of values already divided by their block scale."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_encode_e2m1_scaled(v.reshape(-1), out.reshape(-1), v.size)
    return out


def mx_scale_code(block):
    """E8M0 scale code of one block of values (reading R7)."""
    b = _f32(block).reshape(-1)
    return int(lib().oracle_mx_scale_code(b, b.size))


def mxfp4_encode(a):
    """MXFP4 encode along the last axis (a multiple of 32). Returns (codes uint8 [..., n/2],
    scales uint8 [..., n/32]): element 2i in the low nibble of byte i."""
    a = _f32(a)
    assert a.shape[-1] % 32 == 0
    nb = a.size // 32
    codes = np.empty(a.shape[:-1] + (a.shape[-1] // 2,), np.uint8)
    scales = np.empty(a.shape[:-1] + (a.shape[-1] // 32,), np.uint8)
    lib().oracle_encode_mxfp4(a.reshape(-1), codes.reshape(-1), scales.reshape(-1), nb)
    return codes, scales


def mxfp4_decode(codes, scales):
    """float64 values of MXFP4 codes [..., n/2] with scales [..., n/32]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    nb = scales.size
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), np.float64)
    lib().oracle_decode_mxfp4(codes.reshape(-1), scales.reshape(-1), out.reshape(-1), nb)
    return out


# --------------------------------------------------------------------------------------------
# Gated DeltaNet (oracle_gdn.c). Shapes: H value heads of Dv, G key heads of Dk; q, k [Bt,G,Dk];
# v [Bt,H,Dv]; alpha, beta [Bt,H]; state [Bt,H,Dv,Dk]; o [Bt,H,Dv].
# --------------------------------------------------------------------------------------------
def gdn_step(S, q, k, v, alpha, beta):
    """O1g for one token. S float64 [Bt,H,Dv,Dk], updated in place. Returns o float64 [Bt,H,Dv]."""
    assert S.dtype == np.float64 and S.flags.c_contiguous
    Bt, H, Dv, Dk = S.shape
    G = q.shape[1]
    o = np.empty((Bt, H, Dv), np.float64)
    lib().oracle_gdn_step(Bt, H, G, Dv, Dk, S, _f32(q), _f32(k), _f32(v), _f32(alpha), _f32(beta), o)
    return o


def gdn_spec_stepwise(S, T, q, k, v, alpha, beta, accepted):
    """O5g: all T draft outputs from the committed state S (updated to the accepted prefix).
    Inputs carry the draft index second: q, k [Bt,T,G,Dk], v [Bt,T,H,Dv], alpha, beta [Bt,T,H]."""
    Bt, H, Dv, Dk = S.shape
    G = q.shape[2]
    o = np.empty((Bt, T, H, Dv), np.float64)
    acc = np.ascontiguousarray(accepted, dtype=np.int32)
    rc = lib().oracle_gdn_spec_stepwise(Bt, H, G, Dv, Dk, T, S, _f32(q), _f32(k), _f32(v), _f32(alpha),
                                        _f32(beta), acc, o)
    if rc != 0:
        raise ValueError("accepted count outside [0, T]")
    return o


class GDNReplay:
    """O3g + O4: the GDN replay form (checkpoint + records, backward sweep) and its pointer machine."""

    def __init__(self, S0, G, L, Tmax=1, read_prec=READ_FP32):
        """read_prec READ_BF16 / READ_FP8 / READ_MXFP4: the checkpoint product of replayed
        outputs reads a copy of the checkpoint in that format (reading G4); READ_FP32: the
        checkpoint itself."""
        S0 = _f32(S0)
        self.Bt, self.H, self.Dv, self.Dk = S0.shape
        self.G, self.L, self.Tmax, self.read_prec = G, L, Tmax, read_prec
        self._h = lib().oracle_gdn_create(self.Bt, self.H, G, self.Dv, self.Dk, L, Tmax, S0, int(read_prec))
        if not self._h:
            raise ValueError("invalid GDN replay configuration")

    def __del__(self):
        if getattr(self, "_h", None):
            lib().oracle_gdn_destroy(self._h)
            self._h = None

    def step(self, q, k, v, alpha, beta):
        o = np.empty((self.Bt, self.H, self.Dv), np.float64)
        if lib().oracle_gdn_replay_step(self._h, _f32(q), _f32(k), _f32(v), _f32(alpha), _f32(beta), o) != 0:
            raise RuntimeError("oracle GDN replay: step rejected by the state machine")
        return o

    def verify(self, T, q, k, v, alpha, beta):
        o = np.empty((self.Bt, T, self.H, self.Dv), np.float64)
        if lib().oracle_gdn_replay_verify(self._h, T, _f32(q), _f32(k), _f32(v), _f32(alpha), _f32(beta), o) != 0:
            raise RuntimeError("oracle GDN replay: verify rejected by the state machine")
        return o

    def rollback(self, accepted):
        acc = np.ascontiguousarray(accepted, dtype=np.int32)
        if lib().oracle_gdn_replay_rollback(self._h, acc) != 0:
            raise RuntimeError("oracle GDN replay: rollback rejected by the state machine")

    def flush(self, seq_mask=None):
        if seq_mask is None:
            rc = lib().oracle_gdn_replay_flush(self._h, None)
        else:
            m = np.ascontiguousarray(seq_mask, dtype=np.int32)
            rc = lib().oracle_gdn_replay_flush(self._h, m.ctypes.data_as(ctypes.c_void_p))
        if rc != 0:
            raise RuntimeError("oracle GDN replay: flush rejected by the state machine")

    def set_checkpoint(self, S):
        """Continue from the fp32 checkpoint S [Bt,H,Dv,Dk] (taken as it is; records and pointers
        stay), with the read copy re-encoded from it."""
        S = _f32(S)
        if S.shape != (self.Bt, self.H, self.Dv, self.Dk):
            raise ValueError("checkpoint shape mismatch")
        if lib().oracle_gdn_replay_set_checkpoint(self._h, S) != 0:
            raise RuntimeError("oracle GDN replay: set_checkpoint while a verify is pending")

    def pointers(self):
        pos = np.empty(self.Bt, np.int32)
        ck = np.empty(self.Bt, np.int32)
        lib().oracle_gdn_replay_pointers(self._h, pos, ck)
        return pos, ck

    def _state(self, fn):
        out = np.empty((self.Bt, self.H, self.Dv, self.Dk), np.float64)
        fn(self._h, out)
        return out

    def checkpoint(self):
        return self._state(lib().oracle_gdn_replay_checkpoint)

    def read_copy(self):
        """The decoded bf16 read copy (float64), or None without one."""
        return self._state(lib().oracle_gdn_replay_read_copy) if self.read_prec else None

    def materialize(self):
        return self._state(lib().oracle_gdn_replay_materialize)


def philox4x32_10(ctr, key):
    """Philox4x32-10 of one 4-word counter and 2-word key (uint32 sequences) -> 4 uint32 words."""
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.empty(4, np.uint32)
    lib().oracle_philox4x32_10(c, k, out)
    return out


def f16_encode(a, r16=None):
    """fp16 codes (uint16) of fp32 values: nearest even, or stochastic with 16-bit randoms r16."""
    a = _f32(a)
    out = np.empty(a.shape, np.uint16)
    if r16 is None:
        lib().oracle_encode_f16(a.reshape(-1), out.reshape(-1), a.size, 0, None)
    else:
        r = np.ascontiguousarray(r16, dtype=np.uint32).reshape(-1)
        assert r.size == a.size
        lib().oracle_encode_f16(a.reshape(-1), out.reshape(-1), a.size, 1, r.ctypes.data_as(ctypes.c_void_p))
    return out


def f16_decode(codes):
    codes = np.asarray(codes, np.uint16)
    return np.array([lib().oracle_f16_decode(int(c)) for c in codes.reshape(-1)], np.float32).reshape(codes.shape)


# ---- Mamba-2 mixer edges (oracle_mixer.c) --------------------------------------------------------
def silu(v):
    return float(lib().oracle_silu(float(v)))


def softplus(v):
    return float(lib().oracle_softplus(float(v)))


def mixer_edge(hist, xbc, dt_raw, conv_w, conv_b, dt_bias, H, P, G, N):
    """One token of the input edge. hist: float32 [Bt, K-1, CD] raw history (oldest first),
    updated in place; xbc [Bt, CD]; dt_raw [Bt, H]; conv_w [CD, K]; conv_b [CD]; dt_bias [H].
    Returns x [Bt,H,P], B, C [Bt,G,N], dt [Bt,H] (float32)."""
    assert hist.dtype == np.float32 and hist.flags.c_contiguous
    Bt, CD = xbc.shape
    K = conv_w.shape[1]
    assert CD == H * P + 2 * G * N and hist.shape == (Bt, K - 1, CD)
    x = np.empty((Bt, H, P), np.float32)
    B = np.empty((Bt, G, N), np.float32)
    C = np.empty((Bt, G, N), np.float32)
    dt = np.empty((Bt, H), np.float32)
    h = hist if K > 1 else np.zeros(1, np.float32)
    lib().oracle_mixer_edge(Bt, H, P, N, G, K, h, _f32(xbc), _f32(dt_raw), _f32(conv_w), _f32(conv_b),
                            _f32(dt_bias), x, B, C, dt)
    return x, B, C, dt


def mixer_gate(y, z):
    """o = y * silu(z); y float64, z float32 of the same shape."""
    y = np.ascontiguousarray(y, np.float64)
    o = np.empty_like(y)
    lib().oracle_mixer_gate(y.size, y.reshape(-1), _f32(z).reshape(-1), o.reshape(-1))
    return o


class MixerStepwise:
    """The truth for the fused mixer step: the input edge, O1 (or O5 for drafts), the gate.
    S0 float32 [Bt,H,P,N]; hist0 float32 [Bt,K-1,CD] (zeros for a fresh sequence)."""

    def __init__(self, S0, hist0, A, D, conv_w, conv_b, dt_bias, G):
        self.S = np.ascontiguousarray(S0, np.float64)
        self.hist = np.ascontiguousarray(hist0, np.float32).copy()
        self.A, self.D, self.w, self.b, self.bias, self.G = A, D, conv_w, conv_b, dt_bias, G
        _, self.H, self.P, self.N = self.S.shape

    def edge(self, hist, xbc, dt_raw):
        return mixer_edge(hist, xbc, dt_raw, self.w, self.b, self.bias, self.H, self.P, self.G, self.N)

    def step(self, xbc, z, dt_raw, with_y=False):
        """The gated output o; with with_y, (y, o): the SSM output before the gate as well."""
        x, B, C, dt = self.edge(self.hist, xbc, dt_raw)
        self.last_edge = (x, B, C, dt)   # this token's SSM inputs, as the edge formed them
        y = step(self.S, x, B, C, dt, self.A, self.D)
        o = mixer_gate(y, z)
        return (y, o) if with_y else o

    def spec(self, T, xbc, z, dt_raw, accepted):
        """All T draft outputs (xbc [Bt,T,CD], z [Bt,T,H,P], dt_raw [Bt,T,H]); the state and the
        history then advance by the accepted prefix of each sequence."""
        Bt = xbc.shape[0]
        tent = self.hist.copy()
        ins = [self.edge(tent, np.ascontiguousarray(xbc[:, i]), np.ascontiguousarray(dt_raw[:, i])) for i in range(T)]
        x, B, C, dt = (np.ascontiguousarray(np.stack([t[j] for t in ins], axis=1)) for j in range(4))
        y = spec_stepwise(self.S, T, x, B, C, dt, self.A, self.D, accepted)
        for b in range(Bt):
            for i in range(int(accepted[b])):
                one = self.hist[b:b + 1]
                mixer_edge(one, np.ascontiguousarray(xbc[b:b + 1, i]), np.ascontiguousarray(dt_raw[b:b + 1, i]),
                           self.w, self.b, self.bias, self.H, self.P, self.G, self.N)
                self.hist[b:b + 1] = one
        return mixer_gate(y, z)


class MixerReplay:
    """The replay form with the mixer edges: the same edge and gate around Replay (O3 + O4). The
    conv history follows the committed tokens, so a rollback cuts it back with the records."""

    def __init__(self, S0, hist0, A, D, conv_w, conv_b, dt_bias, G, L, Tmax=1, read_prec=READ_FP32,
                 master_prec=MASTER_FP32, seed=0, seq_ids=None):
        self.rep = Replay(S0, A, D, G, L, Tmax, read_prec, master_prec, seed, seq_ids)
        self.hist = np.ascontiguousarray(hist0, np.float32).copy()
        self.w, self.b, self.bias, self.G = conv_w, conv_b, dt_bias, G
        self.H, self.P, self.N = self.rep.H, self.rep.P, self.rep.N
        self._drafts = None

    def step(self, xbc, z, dt_raw):
        x, B, C, dt = mixer_edge(self.hist, xbc, dt_raw, self.w, self.b, self.bias, self.H, self.P, self.G, self.N)
        return mixer_gate(self.rep.step(x, B, C, dt), z)

    def verify(self, T, xbc, z, dt_raw):
        tent = self.hist.copy()
        ins = [mixer_edge(tent, np.ascontiguousarray(xbc[:, i]), np.ascontiguousarray(dt_raw[:, i]), self.w,
                          self.b, self.bias, self.H, self.P, self.G, self.N) for i in range(T)]
        x, B, C, dt = (np.ascontiguousarray(np.stack([t[j] for t in ins], axis=1)) for j in range(4))
        self._drafts = (T, np.ascontiguousarray(xbc), np.ascontiguousarray(dt_raw))
        return mixer_gate(self.rep.verify(T, x, B, C, dt), z)

    def rollback(self, accepted):
        self.rep.rollback(accepted)
        T, xbc, dt_raw = self._drafts
        for b in range(self.hist.shape[0]):
            for i in range(int(accepted[b])):
                one = self.hist[b:b + 1]
                mixer_edge(one, np.ascontiguousarray(xbc[b:b + 1, i]), np.ascontiguousarray(dt_raw[b:b + 1, i]),
                           self.w, self.b, self.bias, self.H, self.P, self.G, self.N)
                self.hist[b:b + 1] = one
        self._drafts = None

    def set_checkpoint(self, S, rows=None):
        self.rep.set_checkpoint(S, rows)

    def pointers(self):
        return self.rep.pointers()

    def checkpoint(self):
        return self.rep.checkpoint()

    def materialize(self):
        return self.rep.materialize()
