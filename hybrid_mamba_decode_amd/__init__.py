"""Python binding of libreplayssm.so, the ReplaySSM Mamba-2 decode-step library for MI355X.

Argument marshalling only: every step of the decode path runs in the library's HIP kernels.
PyTorch supplies device memory (the caller's tensors and the layer workspace) and streams.

The module-level functions carry the C ABI's names (``replayssm_step``, ``replayssm_flush``,
``replayssm_spec_verify``, ``replayssm_rollback``, ``conventional_step``, ...); ``ReplaySSM`` is
a small object around one layer handle. There is no CPU fallback: importing this package raises
if the built library is missing.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libreplayssm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python hybrid_mamba_decode_amd/build.py` "
        "(hipcc, gfx950). There is no fallback implementation.")

_lib = ctypes.CDLL(LIB_PATH)

RSSM_OK, RSSM_E_INVAL, RSSM_E_WORKSPACE, RSSM_E_HIP, RSSM_E_STATE, RSSM_E_UNSUPPORTED = 0, -1, -2, -3, -4, -5
READ_FP32, READ_BF16, READ_FP8_E4M3, READ_MXFP4 = 0, 1, 2, 3
_PREC_NAMES = {"fp32": READ_FP32, "bf16": READ_BF16, "fp8": READ_FP8_E4M3, "fp8_e4m3": READ_FP8_E4M3,
               "mxfp4": READ_MXFP4, "fp4": READ_MXFP4}
MASTER_FP32, MASTER_FP16, MASTER_FP16_SR, MASTER_FP8, MASTER_FP8_SR = 0, 1, 2, 3, 4
_MASTER_NAMES = {"fp32": MASTER_FP32, "fp16": MASTER_FP16, "fp16_sr": MASTER_FP16_SR, "fp8": MASTER_FP8,
                 "fp8_sr": MASTER_FP8_SR}

EXPORTED = (
    "replayssm_workspace_bytes", "replayssm_workspace_layout", "replayssm_create", "replayssm_destroy",
    "replayssm_load_state", "replayssm_step", "replayssm_flush", "replayssm_spec_verify",
    "replayssm_rollback", "replayssm_set_lockstep", "replayssm_get_pointers", "replayssm_check",
    "replayssm_materialize_state", "replayssm_set_mixer", "replayssm_load_conv_state",
    "replayssm_materialize_conv_state", "replayssm_mixer_step", "replayssm_mixer_spec_verify",
    "conventional_step", "conventional_mixer_step", "snapshot_spec_verify", "snapshot_commit",
    "snapshot_spec_step", "replayssm_status_string",
)
GDN_EXPORTED = (
    "gdnreplay_workspace_bytes", "gdnreplay_workspace_layout", "gdnreplay_create", "gdnreplay_destroy",
    "gdnreplay_load_state", "gdnreplay_step", "gdnreplay_flush", "gdnreplay_spec_verify",
    "gdnreplay_rollback", "gdnreplay_set_lockstep", "gdnreplay_get_pointers", "gdnreplay_check",
    "gdnreplay_materialize_state", "gdn_conventional_step", "gdn_snapshot_spec_verify",
)


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "nheads", "headdim", "dstate", "ngroups", "buffer_len", "max_draft", "read_prec",
        "store_C", "master_prec", "sr_seed", "d_conv")]


class Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "master", "read_copy", "scale", "ring_x", "ring_B", "ring_C", "ring_dt", "conv_ring", "pos",
        "ckpt_pos", "counters", "flag", "total")]


class GDNConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "nheads", "nkheads", "dv", "dk", "buffer_len", "max_draft", "read_prec")]


class GDNLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "master", "read_copy", "scale", "ring_k", "ring_v", "ring_a", "ring_b", "pos", "ckpt_pos", "counters",
        "flag", "total")]


_vp = ctypes.c_void_p
_cfgp = ctypes.POINTER(Config)
_gcfgp = ctypes.POINTER(GDNConfig)
_i32 = ctypes.c_int32
_sig = {
    "replayssm_workspace_bytes": (ctypes.c_size_t, [_cfgp]),
    "replayssm_workspace_layout": (ctypes.c_int, [_cfgp, ctypes.POINTER(Layout)]),
    "replayssm_create": (ctypes.c_int, [_cfgp, _vp, ctypes.c_size_t, _vp, _vp, ctypes.POINTER(_vp)]),
    "replayssm_destroy": (ctypes.c_int, [_vp]),
    "replayssm_load_state": (ctypes.c_int, [_vp, _vp, _vp]),
    "replayssm_step": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "replayssm_flush": (ctypes.c_int, [_vp, _vp, _vp]),
    "replayssm_spec_verify": (ctypes.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "replayssm_rollback": (ctypes.c_int, [_vp, _vp, _vp]),
    "replayssm_set_lockstep": (ctypes.c_int, [_vp, ctypes.c_int]),
    "replayssm_get_pointers": (ctypes.c_int, [_vp, _vp, _vp, _vp]),
    "replayssm_check": (ctypes.c_int, [_vp, _vp]),
    "replayssm_materialize_state": (ctypes.c_int, [_vp, _vp, _vp]),
    "replayssm_set_mixer": (ctypes.c_int, [_vp, _vp, _vp, _vp]),
    "replayssm_load_conv_state": (ctypes.c_int, [_vp, _vp, _vp]),
    "replayssm_materialize_conv_state": (ctypes.c_int, [_vp, _vp, _vp]),
    "replayssm_mixer_step": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp]),
    "replayssm_mixer_spec_verify": (ctypes.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _vp]),
    "conventional_mixer_step": (ctypes.c_int, [_cfgp, _vp, _vp, _i32] + [_vp] * 9 + [_vp]),
    "conventional_step": (ctypes.c_int, [_cfgp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "snapshot_spec_verify": (ctypes.c_int, [_cfgp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "snapshot_commit": (ctypes.c_int, [_cfgp, _vp, _vp, _i32, _vp]),
    "snapshot_spec_step": (ctypes.c_int, [_cfgp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "replayssm_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "gdnreplay_workspace_bytes": (ctypes.c_size_t, [_gcfgp]),
    "gdnreplay_workspace_layout": (ctypes.c_int, [_gcfgp, ctypes.POINTER(GDNLayout)]),
    "gdnreplay_create": (ctypes.c_int, [_gcfgp, _vp, ctypes.c_size_t, ctypes.POINTER(_vp)]),
    "gdnreplay_destroy": (ctypes.c_int, [_vp]),
    "gdnreplay_load_state": (ctypes.c_int, [_vp, _vp, _vp]),
    "gdnreplay_step": (ctypes.c_int, [_vp] + [_vp] * 6 + [_vp]),
    "gdnreplay_flush": (ctypes.c_int, [_vp, _vp, _vp]),
    "gdnreplay_spec_verify": (ctypes.c_int, [_vp, _i32] + [_vp] * 6 + [_vp]),
    "gdnreplay_rollback": (ctypes.c_int, [_vp, _vp, _vp]),
    "gdnreplay_set_lockstep": (ctypes.c_int, [_vp, ctypes.c_int]),
    "gdnreplay_get_pointers": (ctypes.c_int, [_vp, _vp, _vp, _vp]),
    "gdnreplay_check": (ctypes.c_int, [_vp, _vp]),
    "gdnreplay_materialize_state": (ctypes.c_int, [_vp, _vp, _vp]),
    "gdn_conventional_step": (ctypes.c_int, [_gcfgp, _vp] + [_vp] * 6 + [_vp]),
    "gdn_snapshot_spec_verify": (ctypes.c_int, [_gcfgp, _vp, _vp, _i32] + [_vp] * 6 + [_vp]),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class ReplaySSMError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {_lib.replayssm_status_string(status).decode()} (status {status})")


def _check(status, what):
    if status != RSSM_OK:
        raise ReplaySSMError(status, what)


def _ptr(t, dtype=torch.float32, name="tensor"):
    """Device pointer of a contiguous CUDA tensor of the given dtype (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def make_config(batch, nheads, headdim, dstate, ngroups, buffer_len=16, max_draft=1,
                read_prec="fp32", store_C=True, master_prec="fp32", sr_seed=0, d_conv=0):
    rp = _PREC_NAMES[read_prec] if isinstance(read_prec, str) else int(read_prec)
    mp = _MASTER_NAMES[master_prec] if isinstance(master_prec, str) else int(master_prec)
    return Config(batch, nheads, headdim, dstate, ngroups, buffer_len, max_draft, rp, int(bool(store_C)), mp,
                  int(sr_seed), int(d_conv))


def conv_dim(cfg) -> int:
    """Channels of the in-projection's xBC: H*P + 2*G*N."""
    return cfg.nheads * cfg.headdim + 2 * cfg.ngroups * cfg.dstate


def _expect(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


# ---- C ABI, by name -------------------------------------------------------------------------

def replayssm_workspace_bytes(cfg: Config) -> int:
    return int(_lib.replayssm_workspace_bytes(ctypes.byref(cfg)))


def replayssm_workspace_layout(cfg: Config) -> Layout:
    lay = Layout()
    _check(_lib.replayssm_workspace_layout(ctypes.byref(cfg), ctypes.byref(lay)), "replayssm_workspace_layout")
    return lay


def replayssm_create(cfg: Config, workspace: torch.Tensor, A: torch.Tensor, D: torch.Tensor):
    h = _vp()
    _check(_lib.replayssm_create(ctypes.byref(cfg), _ptr(workspace, torch.uint8, "workspace"),
                                 workspace.numel(), _ptr(A, name="A"), _ptr(D, name="D"),
                                 ctypes.byref(h)), "replayssm_create")
    return h


def replayssm_destroy(h):
    _check(_lib.replayssm_destroy(h), "replayssm_destroy")


def replayssm_load_state(h, state, stream=None):
    _check(_lib.replayssm_load_state(h, _ptr(state, name="state"), _stream(stream)), "replayssm_load_state")


def replayssm_step(h, x, B, C, dt, y, stream=None):
    _check(_lib.replayssm_step(h, _ptr(x, name="x"), _ptr(B, name="B"), _ptr(C, name="C"),
                               _ptr(dt, name="dt"), _ptr(y, name="y"), _stream(stream)), "replayssm_step")


def replayssm_flush(h, seq_mask=None, stream=None):
    _check(_lib.replayssm_flush(h, _ptr(seq_mask, torch.int32, "seq_mask"), _stream(stream)), "replayssm_flush")


def replayssm_spec_verify(h, T, x, B, C, dt, y, stream=None):
    _check(_lib.replayssm_spec_verify(h, int(T), _ptr(x, name="x"), _ptr(B, name="B"), _ptr(C, name="C"),
                                      _ptr(dt, name="dt"), _ptr(y, name="y"), _stream(stream)),
           "replayssm_spec_verify")


def replayssm_rollback(h, accepted, stream=None):
    _check(_lib.replayssm_rollback(h, _ptr(accepted, torch.int32, "accepted"), _stream(stream)),
           "replayssm_rollback")


def replayssm_set_lockstep(h, enable):
    _check(_lib.replayssm_set_lockstep(h, int(bool(enable))), "replayssm_set_lockstep")


def replayssm_get_pointers(h, batch, stream=None):
    pos = (ctypes.c_int32 * max(batch, 1))()
    ck = (ctypes.c_int32 * max(batch, 1))()
    _check(_lib.replayssm_get_pointers(h, ctypes.cast(pos, _vp), ctypes.cast(ck, _vp), _stream(stream)),
           "replayssm_get_pointers")
    return list(pos)[:batch], list(ck)[:batch]


def replayssm_check(h, stream=None):
    return int(_lib.replayssm_check(h, _stream(stream)))


def replayssm_materialize_state(h, out, stream=None):
    _check(_lib.replayssm_materialize_state(h, _ptr(out, name="out"), _stream(stream)),
           "replayssm_materialize_state")


def _check_token_shapes(cfg, x, B, C, dt, lead=()):
    Bt, H, P, N, G = cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups
    _expect(x, (Bt, *lead, H, P), "x")
    _expect(B, (Bt, *lead, G, N), "B")
    _expect(C, (Bt, *lead, G, N), "C")
    _expect(dt, (Bt, *lead, H), "dt")


def conventional_step(cfg: Config, state, x, B, C, dt, A, D, y, stream=None):
    _check_token_shapes(cfg, x, B, C, dt)
    _expect(state, (cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate), "state")
    _expect(y, (cfg.batch, cfg.nheads, cfg.headdim), "y")
    _expect(A, (cfg.nheads,), "A")
    _expect(D, (cfg.nheads,), "D")
    _check(_lib.conventional_step(ctypes.byref(cfg), _ptr(state, name="state"), _ptr(x, name="x"),
                                  _ptr(B, name="B"), _ptr(C, name="C"), _ptr(dt, name="dt"),
                                  _ptr(A, name="A"), _ptr(D, name="D"), _ptr(y, name="y"),
                                  _stream(stream)), "conventional_step")


def snapshot_spec_verify(cfg: Config, slots, cur, T, x, B, C, dt, A, D, y, stream=None):
    _check_token_shapes(cfg, x, B, C, dt, (T,))
    _expect(slots, (cfg.batch, T + 1, cfg.nheads, cfg.headdim, cfg.dstate), "slots")
    _expect(cur, (cfg.batch,), "cur")
    _expect(y, (cfg.batch, T, cfg.nheads, cfg.headdim), "y")
    _expect(A, (cfg.nheads,), "A")
    _expect(D, (cfg.nheads,), "D")
    _check(_lib.snapshot_spec_verify(ctypes.byref(cfg), _ptr(slots, name="slots"),
                                     _ptr(cur, torch.int32, "cur"), int(T), _ptr(x, name="x"),
                                     _ptr(B, name="B"), _ptr(C, name="C"), _ptr(dt, name="dt"),
                                     _ptr(A, name="A"), _ptr(D, name="D"), _ptr(y, name="y"),
                                     _stream(stream)), "snapshot_spec_verify")


def snapshot_commit(cfg: Config, cur, accepted, T, stream=None):
    _expect(cur, (cfg.batch,), "cur")
    _expect(accepted, (cfg.batch,), "accepted")
    _check(_lib.snapshot_commit(ctypes.byref(cfg), _ptr(cur, torch.int32, "cur"),
                                _ptr(accepted, torch.int32, "accepted"), int(T), _stream(stream)),
           "snapshot_commit")


def snapshot_spec_step(cfg: Config, slots, cur, T, x, B, C, dt, A, D, y, accepted, stream=None):
    """snapshot_spec_verify then snapshot_commit, as one call of the C ABI."""
    _check_token_shapes(cfg, x, B, C, dt, (T,))
    _expect(slots, (cfg.batch, T + 1, cfg.nheads, cfg.headdim, cfg.dstate), "slots")
    _expect(cur, (cfg.batch,), "cur")
    _expect(y, (cfg.batch, T, cfg.nheads, cfg.headdim), "y")
    _expect(A, (cfg.nheads,), "A")
    _expect(D, (cfg.nheads,), "D")
    _expect(accepted, (cfg.batch,), "accepted")
    _check(_lib.snapshot_spec_step(ctypes.byref(cfg), _ptr(slots, name="slots"), _ptr(cur, torch.int32, "cur"),
                                   int(T), _ptr(x, name="x"), _ptr(B, name="B"), _ptr(C, name="C"),
                                   _ptr(dt, name="dt"), _ptr(A, name="A"), _ptr(D, name="D"), _ptr(y, name="y"),
                                   _ptr(accepted, torch.int32, "accepted"), _stream(stream)), "snapshot_spec_step")


def replayssm_set_mixer(h, conv_w, conv_b, dt_bias):
    _check(_lib.replayssm_set_mixer(h, _ptr(conv_w, name="conv_w"), _ptr(conv_b, name="conv_b"),
                                    _ptr(dt_bias, name="dt_bias")), "replayssm_set_mixer")


def replayssm_load_conv_state(h, hist=None, stream=None):
    _check(_lib.replayssm_load_conv_state(h, _ptr(hist, name="hist"), _stream(stream)), "replayssm_load_conv_state")


def replayssm_materialize_conv_state(h, out, stream=None):
    _check(_lib.replayssm_materialize_conv_state(h, _ptr(out, name="out"), _stream(stream)),
           "replayssm_materialize_conv_state")


def replayssm_mixer_step(h, xbc, z, dt_raw, o, stream=None):
    _check(_lib.replayssm_mixer_step(h, _ptr(xbc, name="xbc"), _ptr(z, name="z"), _ptr(dt_raw, name="dt_raw"),
                                     _ptr(o, name="o"), _stream(stream)), "replayssm_mixer_step")


def replayssm_mixer_spec_verify(h, T, xbc, z, dt_raw, o, stream=None):
    _check(_lib.replayssm_mixer_spec_verify(h, int(T), _ptr(xbc, name="xbc"), _ptr(z, name="z"),
                                            _ptr(dt_raw, name="dt_raw"), _ptr(o, name="o"), _stream(stream)),
           "replayssm_mixer_spec_verify")


def conventional_mixer_step(cfg: Config, state, conv_ring, t, xbc, z, dt_raw, A, D, conv_w, conv_b, dt_bias, o,
                            stream=None):
    Bt, H, P, K, CD = cfg.batch, cfg.nheads, cfg.headdim, cfg.d_conv, conv_dim(cfg)
    _expect(state, (Bt, H, P, cfg.dstate), "state")
    _expect(conv_ring, (Bt, K, CD), "conv_ring")
    _expect(xbc, (Bt, CD), "xbc")
    _expect(z, (Bt, H, P), "z")
    _expect(dt_raw, (Bt, H), "dt_raw")
    _expect(o, (Bt, H, P), "o")
    _check(_lib.conventional_mixer_step(ctypes.byref(cfg), _ptr(state, name="state"), _ptr(conv_ring, name="conv_ring"),
                                        int(t), _ptr(xbc, name="xbc"), _ptr(z, name="z"), _ptr(dt_raw, name="dt_raw"),
                                        _ptr(A, name="A"), _ptr(D, name="D"), _ptr(conv_w, name="conv_w"),
                                        _ptr(conv_b, name="conv_b"), _ptr(dt_bias, name="dt_bias"), _ptr(o, name="o"),
                                        _stream(stream)), "conventional_mixer_step")


def replayssm_status_string(status: int) -> str:
    return _lib.replayssm_status_string(int(status)).decode()


# ---- one layer as an object -------------------------------------------------------------------

class ReplaySSM:
    """One Mamba-2 layer's decode state kept as checkpoint + record ring, on one GPU.

    The workspace (fp32 master, read copy, ring, pointers) is one uint8 CUDA tensor owned here.
    """

    def __init__(self, batch, nheads, headdim, dstate, ngroups, A, D, buffer_len=16, max_draft=1,
                 read_prec="fp32", store_C=True, master_prec="fp32", sr_seed=0, d_conv=0, device="cuda"):
        self.cfg = make_config(batch, nheads, headdim, dstate, ngroups, buffer_len, max_draft,
                               read_prec, store_C, master_prec, sr_seed, d_conv)
        nbytes = replayssm_workspace_bytes(self.cfg)
        if nbytes == 0:
            raise ReplaySSMError(RSSM_E_INVAL, "replayssm_workspace_bytes")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        if self.workspace.data_ptr() % 256:
            raise RuntimeError("workspace allocation is not 256-byte aligned")
        self.A = A.contiguous()
        self.D = D.contiguous()
        self.layout = replayssm_workspace_layout(self.cfg)
        self.handle = replayssm_create(self.cfg, self.workspace, self.A, self.D)
        self.batch, self.nheads, self.headdim, self.dstate, self.ngroups = batch, nheads, headdim, dstate, ngroups
        self.buffer_len, self.max_draft = buffer_len, max_draft

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:  # at interpreter exit the module's globals may be gone
            _lib.replayssm_destroy(h)
            self.handle = None

    # shapes
    def _tok(self, lead=()):
        Bt, H, P, N, G = self.batch, self.nheads, self.headdim, self.dstate, self.ngroups
        return ((Bt, *lead, H, P), (Bt, *lead, G, N), (Bt, *lead, G, N), (Bt, *lead, H))

    def load_state(self, state, stream=None):
        _expect(state, (self.batch, self.nheads, self.headdim, self.dstate), "state")
        replayssm_load_state(self.handle, state, stream)

    def step(self, x, B, C, dt, y=None, stream=None):
        for t, s, n in zip((x, B, C, dt), self._tok(), "xBCd"):
            _expect(t, s, n)
        if y is None:
            y = torch.empty_like(x)
        _expect(y, self._tok()[0], "y")
        replayssm_step(self.handle, x, B, C, dt, y, stream)
        return y

    def flush(self, seq_mask=None, stream=None):
        replayssm_flush(self.handle, seq_mask, stream)

    def spec_verify(self, x, B, C, dt, y=None, stream=None):
        T = x.shape[1]
        for t, s, n in zip((x, B, C, dt), self._tok((T,)), "xBCd"):
            _expect(t, s, n)
        if y is None:
            y = torch.empty_like(x)
        _expect(y, self._tok((T,))[0], "y")
        replayssm_spec_verify(self.handle, T, x, B, C, dt, y, stream)
        return y

    def rollback(self, accepted, stream=None):
        _expect(accepted, (self.batch,), "accepted")
        replayssm_rollback(self.handle, accepted, stream)

    def set_lockstep(self, enable):
        replayssm_set_lockstep(self.handle, enable)

    def get_pointers(self, stream=None):
        return replayssm_get_pointers(self.handle, self.batch, stream)

    def check(self, stream=None):
        return replayssm_check(self.handle, stream)

    def materialize_state(self, out=None, stream=None):
        if out is None:
            out = torch.empty((self.batch, self.nheads, self.headdim, self.dstate),
                              dtype=torch.float32, device=self.workspace.device)
        _expect(out, (self.batch, self.nheads, self.headdim, self.dstate), "out")
        replayssm_materialize_state(self.handle, out, stream)
        return out

    # mixer edges (d_conv > 0)
    def set_mixer(self, conv_w, conv_b, dt_bias):
        """conv_w [CD, K], conv_b [CD], dt_bias [H]; kept referenced by this object."""
        CD, K = conv_dim(self.cfg), self.cfg.d_conv
        _expect(conv_w, (CD, K), "conv_w")
        _expect(conv_b, (CD,), "conv_b")
        _expect(dt_bias, (self.nheads,), "dt_bias")
        self._mixer = (conv_w.contiguous(), conv_b.contiguous(), dt_bias.contiguous())
        replayssm_set_mixer(self.handle, *self._mixer)

    def load_conv_state(self, hist=None, stream=None):
        if hist is not None:
            _expect(hist, (self.batch, self.cfg.d_conv - 1, conv_dim(self.cfg)), "hist")
        replayssm_load_conv_state(self.handle, hist, stream)

    def materialize_conv_state(self, out=None, stream=None):
        if out is None:
            out = torch.empty((self.batch, self.cfg.d_conv - 1, conv_dim(self.cfg)), dtype=torch.float32,
                              device=self.workspace.device)
        _expect(out, (self.batch, self.cfg.d_conv - 1, conv_dim(self.cfg)), "out")
        replayssm_materialize_conv_state(self.handle, out, stream)
        return out

    def mixer_step(self, xbc, z, dt_raw, o=None, stream=None):
        _expect(xbc, (self.batch, conv_dim(self.cfg)), "xbc")
        _expect(z, (self.batch, self.nheads, self.headdim), "z")
        _expect(dt_raw, (self.batch, self.nheads), "dt_raw")
        if o is None:
            o = torch.empty_like(z)
        _expect(o, (self.batch, self.nheads, self.headdim), "o")
        replayssm_mixer_step(self.handle, xbc, z, dt_raw, o, stream)
        return o

    def mixer_spec_verify(self, xbc, z, dt_raw, o=None, stream=None):
        T = xbc.shape[1]
        _expect(xbc, (self.batch, T, conv_dim(self.cfg)), "xbc")
        _expect(z, (self.batch, T, self.nheads, self.headdim), "z")
        _expect(dt_raw, (self.batch, T, self.nheads), "dt_raw")
        if o is None:
            o = torch.empty_like(z)
        _expect(o, (self.batch, T, self.nheads, self.headdim), "o")
        replayssm_mixer_spec_verify(self.handle, T, xbc, z, dt_raw, o, stream)
        return o

    # workspace views (inspection)
    def region(self, name, dtype, shape):
        off = getattr(self.layout, name)
        n = 1
        for s in shape:
            n *= s
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return self.workspace[off:off + nbytes].view(dtype).view(*shape)

    def master(self):
        """The checkpoint as stored: float32, float16 for an fp16 master, or for an fp8 master its
        E4M3FN codes uint8 [Bt,H,P,N] in row-major order (a reordered copy of the chunked codes;
        the per-head scales are `scales()`)."""
        Bt, H, P, N = self.batch, self.nheads, self.headdim, self.dstate
        if self.cfg.master_prec in (MASTER_FP8, MASTER_FP8_SR):
            raw = self.region("master", torch.uint8, (Bt, H, N // 16, P, 16))
            return raw.permute(0, 1, 3, 2, 4).contiguous().view(Bt, H, P, N)
        dt = torch.float32 if self.cfg.master_prec == MASTER_FP32 else torch.float16
        return self.region("master", dt, (Bt, H, P, N))

    def read_copy(self):
        """The read copy in row-major order: bf16 bits int16 [Bt,H,P,N], fp8 codes uint8
        [Bt,H,P,N], MXFP4 code bytes uint8 [Bt,H,P,N/2]. bf16 is a view of the workspace; the fp8
        and MXFP4 copies are stored per head as 16-byte chunks in chunk-column-major order
        ([N/VEC][P] chunks, see replayssm.h), so this returns a reordered copy."""
        Bt, H, P, N = self.batch, self.nheads, self.headdim, self.dstate
        if self.cfg.read_prec == READ_BF16:
            return self.region("read_copy", torch.int16, (Bt, H, P, N))
        if self.cfg.read_prec in (READ_FP8_E4M3, READ_MXFP4):
            row_bytes = N if self.cfg.read_prec == READ_FP8_E4M3 else N // 2
            raw = self.region("read_copy", torch.uint8, (Bt, H, row_bytes // 16, P, 16))
            return raw.permute(0, 1, 3, 2, 4).contiguous().view(Bt, H, P, row_bytes)
        return None

    def scales(self):
        """fp8 copy or fp8 master: fp32 scales [Bt,H,ceil(P/64)], one per block of 64 rows;
        MXFP4: E8M0 block-scale bytes [Bt,H,P,N/32]."""
        if self.cfg.read_prec == READ_MXFP4:
            return self.region("scale", torch.uint8, (self.batch, self.nheads, self.headdim, self.dstate // 32))
        return self.region("scale", torch.float32, (self.batch, self.nheads, (self.headdim + 63) // 64))

    def pointer_arrays(self):
        return (self.region("pos", torch.int32, (self.batch,)),
                self.region("ckpt_pos", torch.int32, (self.batch,)))


# ---- Gated DeltaNet layers (gdnreplay.h) ------------------------------------------------------

def make_gdn_config(batch, nheads, nkheads, dv, dk, buffer_len=16, max_draft=1, read_prec="fp32"):
    rp = _PREC_NAMES[read_prec] if isinstance(read_prec, str) else int(read_prec)
    return GDNConfig(batch, nheads, nkheads, dv, dk, buffer_len, max_draft, rp)


def gdnreplay_workspace_bytes(cfg: GDNConfig) -> int:
    return int(_lib.gdnreplay_workspace_bytes(ctypes.byref(cfg)))


def gdnreplay_workspace_layout(cfg: GDNConfig) -> GDNLayout:
    lay = GDNLayout()
    _check(_lib.gdnreplay_workspace_layout(ctypes.byref(cfg), ctypes.byref(lay)), "gdnreplay_workspace_layout")
    return lay


def gdnreplay_create(cfg: GDNConfig, workspace: torch.Tensor):
    h = _vp()
    _check(_lib.gdnreplay_create(ctypes.byref(cfg), _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                 ctypes.byref(h)), "gdnreplay_create")
    return h


def gdnreplay_destroy(h):
    _check(_lib.gdnreplay_destroy(h), "gdnreplay_destroy")


def gdnreplay_load_state(h, state, stream=None):
    _check(_lib.gdnreplay_load_state(h, _ptr(state, name="state"), _stream(stream)), "gdnreplay_load_state")


def _gio(q, k, v, alpha, beta, o):
    return (_ptr(q, name="q"), _ptr(k, name="k"), _ptr(v, name="v"), _ptr(alpha, name="alpha"),
            _ptr(beta, name="beta"), _ptr(o, name="o"))


def gdnreplay_step(h, q, k, v, alpha, beta, o, stream=None):
    _check(_lib.gdnreplay_step(h, *_gio(q, k, v, alpha, beta, o), _stream(stream)), "gdnreplay_step")


def gdnreplay_flush(h, seq_mask=None, stream=None):
    _check(_lib.gdnreplay_flush(h, _ptr(seq_mask, torch.int32, "seq_mask"), _stream(stream)), "gdnreplay_flush")


def gdnreplay_spec_verify(h, T, q, k, v, alpha, beta, o, stream=None):
    _check(_lib.gdnreplay_spec_verify(h, int(T), *_gio(q, k, v, alpha, beta, o), _stream(stream)),
           "gdnreplay_spec_verify")


def gdnreplay_rollback(h, accepted, stream=None):
    _check(_lib.gdnreplay_rollback(h, _ptr(accepted, torch.int32, "accepted"), _stream(stream)), "gdnreplay_rollback")


def gdnreplay_set_lockstep(h, enable):
    _check(_lib.gdnreplay_set_lockstep(h, int(bool(enable))), "gdnreplay_set_lockstep")


def gdnreplay_get_pointers(h, batch, stream=None):
    pos = (ctypes.c_int32 * max(batch, 1))()
    ck = (ctypes.c_int32 * max(batch, 1))()
    _check(_lib.gdnreplay_get_pointers(h, ctypes.cast(pos, _vp), ctypes.cast(ck, _vp), _stream(stream)),
           "gdnreplay_get_pointers")
    return list(pos)[:batch], list(ck)[:batch]


def gdnreplay_check(h, stream=None):
    return int(_lib.gdnreplay_check(h, _stream(stream)))


def gdnreplay_materialize_state(h, out, stream=None):
    _check(_lib.gdnreplay_materialize_state(h, _ptr(out, name="out"), _stream(stream)), "gdnreplay_materialize_state")


def _check_gdn_tokens(cfg, q, k, v, alpha, beta, o, lead=()):
    Bt, H, G, Dv, Dk = cfg.batch, cfg.nheads, cfg.nkheads, cfg.dv, cfg.dk
    _expect(q, (Bt, *lead, G, Dk), "q")
    _expect(k, (Bt, *lead, G, Dk), "k")
    _expect(v, (Bt, *lead, H, Dv), "v")
    _expect(alpha, (Bt, *lead, H), "alpha")
    _expect(beta, (Bt, *lead, H), "beta")
    _expect(o, (Bt, *lead, H, Dv), "o")


def gdn_conventional_step(cfg: GDNConfig, state, q, k, v, alpha, beta, o, stream=None):
    _check_gdn_tokens(cfg, q, k, v, alpha, beta, o)
    _expect(state, (cfg.batch, cfg.nheads, cfg.dv, cfg.dk), "state")
    _check(_lib.gdn_conventional_step(ctypes.byref(cfg), _ptr(state, name="state"), *_gio(q, k, v, alpha, beta, o),
                                      _stream(stream)), "gdn_conventional_step")


def gdn_snapshot_spec_verify(cfg: GDNConfig, slots, cur, T, q, k, v, alpha, beta, o, stream=None):
    _check_gdn_tokens(cfg, q, k, v, alpha, beta, o, (T,))
    _expect(slots, (cfg.batch, T + 1, cfg.nheads, cfg.dv, cfg.dk), "slots")
    _expect(cur, (cfg.batch,), "cur")
    _check(_lib.gdn_snapshot_spec_verify(ctypes.byref(cfg), _ptr(slots, name="slots"), _ptr(cur, torch.int32, "cur"),
                                         int(T), *_gio(q, k, v, alpha, beta, o), _stream(stream)),
           "gdn_snapshot_spec_verify")


class GDNReplay:
    """One Gated DeltaNet layer's decode state kept as checkpoint + record ring, on one GPU."""

    def __init__(self, batch, nheads, nkheads, dv, dk, buffer_len=16, max_draft=1, read_prec="fp32", device="cuda"):
        self.cfg = make_gdn_config(batch, nheads, nkheads, dv, dk, buffer_len, max_draft, read_prec)
        nbytes = gdnreplay_workspace_bytes(self.cfg)
        if nbytes == 0:
            raise ReplaySSMError(RSSM_E_INVAL, "gdnreplay_workspace_bytes")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        if self.workspace.data_ptr() % 256:
            raise RuntimeError("workspace allocation is not 256-byte aligned")
        self.layout = gdnreplay_workspace_layout(self.cfg)
        self.handle = gdnreplay_create(self.cfg, self.workspace)
        self.batch, self.nheads, self.nkheads, self.dv, self.dk = batch, nheads, nkheads, dv, dk
        self.buffer_len, self.max_draft = buffer_len, max_draft

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:  # at interpreter exit the module's globals may be gone
            _lib.gdnreplay_destroy(h)
            self.handle = None

    def load_state(self, state, stream=None):
        _expect(state, (self.batch, self.nheads, self.dv, self.dk), "state")
        gdnreplay_load_state(self.handle, state, stream)

    def step(self, q, k, v, alpha, beta, o=None, stream=None):
        if o is None:
            o = torch.empty_like(v)
        _check_gdn_tokens(self.cfg, q, k, v, alpha, beta, o)
        gdnreplay_step(self.handle, q, k, v, alpha, beta, o, stream)
        return o

    def flush(self, seq_mask=None, stream=None):
        gdnreplay_flush(self.handle, seq_mask, stream)

    def spec_verify(self, q, k, v, alpha, beta, o=None, stream=None):
        T = q.shape[1]
        if o is None:
            o = torch.empty_like(v)
        _check_gdn_tokens(self.cfg, q, k, v, alpha, beta, o, (T,))
        gdnreplay_spec_verify(self.handle, T, q, k, v, alpha, beta, o, stream)
        return o

    def rollback(self, accepted, stream=None):
        _expect(accepted, (self.batch,), "accepted")
        gdnreplay_rollback(self.handle, accepted, stream)

    def set_lockstep(self, enable):
        gdnreplay_set_lockstep(self.handle, enable)

    def get_pointers(self, stream=None):
        return gdnreplay_get_pointers(self.handle, self.batch, stream)

    def check(self, stream=None):
        return gdnreplay_check(self.handle, stream)

    def materialize_state(self, out=None, stream=None):
        if out is None:
            out = torch.empty(self.batch, self.nheads, self.dv, self.dk, device=self.workspace.device)
        _expect(out, (self.batch, self.nheads, self.dv, self.dk), "out")
        gdnreplay_materialize_state(self.handle, out, stream)
        return out

    def master(self):
        off = self.layout.master
        n = self.batch * self.nheads * self.dv * self.dk
        return self.workspace[off:off + 4 * n].view(torch.float32).view(self.batch, self.nheads, self.dv, self.dk)

    def read_copy(self):
        """The read copy in row-major order (value rows of Dk key columns): bf16 bits int16
        [Bt,H,Dv,Dk] (a view of the workspace), fp8 codes uint8 [Bt,H,Dv,Dk] or MXFP4 code bytes
        uint8 [Bt,H,Dv,Dk/2] (reordered copies of the chunked codes); None with fp32 reads."""
        Bt, H, Dv, Dk = self.batch, self.nheads, self.dv, self.dk
        off = self.layout.read_copy
        if self.cfg.read_prec == READ_BF16:
            return self.workspace[off:off + 2 * Bt * H * Dv * Dk].view(torch.int16).view(Bt, H, Dv, Dk)
        if self.cfg.read_prec in (READ_FP8_E4M3, READ_MXFP4):
            row_bytes = Dk if self.cfg.read_prec == READ_FP8_E4M3 else Dk // 2
            raw = self.workspace[off:off + Bt * H * Dv * row_bytes].view(Bt, H, row_bytes // 16, Dv, 16)
            return raw.permute(0, 1, 3, 2, 4).contiguous().view(Bt, H, Dv, row_bytes)
        return None

    def scales(self):
        """fp8: fp32 scales [Bt,H,ceil(Dv/64)]; MXFP4: E8M0 block-scale bytes [Bt,H,Dv,Dk/32];
        None otherwise."""
        Bt, H, Dv, Dk = self.batch, self.nheads, self.dv, self.dk
        off = self.layout.scale
        if self.cfg.read_prec == READ_FP8_E4M3:
            nb = (Dv + 63) // 64
            return self.workspace[off:off + 4 * Bt * H * nb].view(torch.float32).view(Bt, H, nb)
        if self.cfg.read_prec == READ_MXFP4:
            return self.workspace[off:off + Bt * H * Dv * Dk // 32].view(Bt, H, Dv, Dk // 32)
        return None

    def pointer_arrays(self):
        def region(off, n):
            return self.workspace[off:off + 4 * n].view(torch.int32)
        return region(self.layout.pos, self.batch), region(self.layout.ckpt_pos, self.batch)
