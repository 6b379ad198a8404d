"""C-ABI checks that need no GPU: the library loads, exports every function the header declares,
sizes and lays out the workspace, and rejects bad arguments and state-machine misuse on the host
before any HIP call (batch 0 makes every accepted call a no-op, so nothing is launched)."""
import ctypes
import os
import re

import pytest

import hybrid_mamba_decode_amd as rs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "replayssm.h")
FAKE = 0x10000  # a 256-byte-aligned fake device address; never dereferenced in these tests


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(rs._lib, n), f"{n} declared in replayssm.h but not exported"
    assert set(names) == set(rs.EXPORTED)


def cfg(**kw):
    base = dict(batch=0, nheads=128, headdim=64, dstate=128, ngroups=8, buffer_len=16, max_draft=1,
                read_prec="fp32", store_C=True)
    base.update(kw)
    return rs.make_config(**base)


def test_workspace_layout_serving_shape():
    c = cfg(batch=256)
    lay = rs.replayssm_workspace_layout(c)
    Bt, H, P, N, G, L = 256, 128, 64, 128, 8, 16
    assert lay.master == 0
    assert lay.read_copy == Bt * H * P * N * 4                 # fp32 reads: no copy
    assert lay.ring_B - lay.ring_x == Bt * H * L * P * 4
    assert lay.ring_C - lay.ring_B == Bt * G * L * N * 4
    assert lay.ring_dt - lay.ring_C == Bt * G * L * N * 4
    assert lay.total == rs.replayssm_workspace_bytes(c)
    for name in ("master", "read_copy", "scale", "ring_x", "ring_B", "ring_C", "ring_dt", "pos",
                 "ckpt_pos", "counters", "flag"):
        assert getattr(lay, name) % 256 == 0
    c8 = cfg(batch=256, read_prec="fp8")
    l8 = rs.replayssm_workspace_layout(c8)
    assert l8.scale - l8.read_copy == Bt * H * P * N           # one byte per element
    assert l8.ring_x - l8.scale == Bt * H * 4
    c4 = cfg(batch=256, read_prec="mxfp4", headdim=100)
    l4 = rs.replayssm_workspace_layout(c4)
    assert l4.scale - l4.read_copy == Bt * H * 100 * N // 2     # two codes per byte
    assert l4.ring_x - l4.scale == Bt * H * 100 * N // 32       # one E8M0 byte per 32 values
    cb = cfg(batch=256, read_prec="bf16", store_C=False)
    lb = rs.replayssm_workspace_layout(cb)
    assert lb.scale - lb.read_copy == Bt * H * P * N * 2
    assert lb.ring_C == lb.ring_dt                               # no C in the records
    ch = cfg(batch=256, master_prec="fp16_sr", read_prec="bf16")
    lh = rs.replayssm_workspace_layout(ch)
    assert lh.read_copy - lh.master == Bt * H * P * N * 2          # fp16 master
    assert lh.scale - lh.read_copy == Bt * H * P * N * 2
    assert lh.total < lb.total + Bt * H * P * N * 4
    for m in ("fp8", "fp8_sr"):                                     # fp8 master: its own read copy
        l8m = rs.replayssm_workspace_layout(cfg(batch=256, master_prec=m))
        assert l8m.read_copy - l8m.master == Bt * H * P * N           # one code byte per value
        assert l8m.scale == l8m.read_copy                             # no second copy
        assert l8m.ring_x - l8m.scale == Bt * H * 4                   # fp32 scale per head (P <= 64)
    l8w = rs.replayssm_workspace_layout(cfg(batch=256, read_prec="fp8", headdim=100))
    assert l8w.ring_x - l8w.scale == Bt * H * 2 * 4                   # two 64-row blocks per head


@pytest.mark.parametrize("kw,status", [
    (dict(dstate=48), rs.RSSM_E_UNSUPPORTED),
    (dict(dstate=512), rs.RSSM_E_UNSUPPORTED),
    (dict(headdim=66), rs.RSSM_E_INVAL),
    (dict(headdim=260), rs.RSSM_E_UNSUPPORTED),
    (dict(nheads=6, ngroups=4), rs.RSSM_E_INVAL),
    (dict(buffer_len=0), rs.RSSM_E_INVAL),
    (dict(buffer_len=4, max_draft=5), rs.RSSM_E_INVAL),
    (dict(buffer_len=65), rs.RSSM_E_UNSUPPORTED),
    (dict(buffer_len=16, max_draft=9), rs.RSSM_E_UNSUPPORTED),
    (dict(read_prec=4), rs.RSSM_E_INVAL),
    (dict(read_prec="mxfp4", dstate=16), rs.RSSM_E_UNSUPPORTED),
    (dict(batch=-1), rs.RSSM_E_INVAL),
    (dict(store_C=2), rs.RSSM_E_INVAL),
    (dict(master_prec=5), rs.RSSM_E_INVAL),
    (dict(master_prec="fp8", read_prec="bf16"), rs.RSSM_E_INVAL),
    (dict(master_prec="fp8_sr", read_prec="fp8"), rs.RSSM_E_INVAL),
    (dict(master_prec=-1), rs.RSSM_E_INVAL),
    (dict(d_conv=1), rs.RSSM_E_INVAL),
    (dict(d_conv=-1), rs.RSSM_E_INVAL),
    (dict(d_conv=5), rs.RSSM_E_UNSUPPORTED),
    (dict(d_conv=4, buffer_len=64), rs.RSSM_E_UNSUPPORTED),
])
def test_invalid_configs_rejected(kw, status):
    c = cfg(**kw)
    if kw.get("store_C") == 2:
        c.store_C = 2
    assert rs.replayssm_workspace_bytes(c) == 0
    h = ctypes.c_void_p()
    st = rs._lib.replayssm_create(ctypes.byref(c), FAKE, 1 << 40, FAKE, FAKE, ctypes.byref(h))
    assert st == status
    assert not h.value


def test_workspace_errors():
    c = cfg(batch=4)
    need = rs.replayssm_workspace_bytes(c)
    h = ctypes.c_void_p()
    create = rs._lib.replayssm_create
    assert create(ctypes.byref(c), None, need, FAKE, FAKE, ctypes.byref(h)) == rs.RSSM_E_WORKSPACE
    assert create(ctypes.byref(c), FAKE + 16, need, FAKE, FAKE, ctypes.byref(h)) == rs.RSSM_E_WORKSPACE
    assert create(ctypes.byref(c), FAKE, need - 1, FAKE, FAKE, ctypes.byref(h)) == rs.RSSM_E_WORKSPACE
    assert create(ctypes.byref(c), FAKE, need, None, FAKE, ctypes.byref(h)) == rs.RSSM_E_INVAL
    assert create(ctypes.byref(c), FAKE, need, FAKE, FAKE, None) == rs.RSSM_E_INVAL
    assert create(ctypes.byref(c), FAKE, need, FAKE, FAKE, ctypes.byref(h)) == rs.RSSM_OK
    assert rs._lib.replayssm_destroy(h) == rs.RSSM_OK
    assert rs._lib.replayssm_destroy(None) == rs.RSSM_OK


def _handle(**kw):
    c = cfg(**kw)
    h = ctypes.c_void_p()
    assert rs._lib.replayssm_create(ctypes.byref(c), FAKE, rs.replayssm_workspace_bytes(c), FAKE, FAKE,
                                    ctypes.byref(h)) == rs.RSSM_OK
    return h


def test_state_machine_on_host():
    """Batch 0: every accepted call is a no-op on the device, so the host state machine can be
    driven completely without a GPU. Empty arrays may be NULL at batch 0."""
    L = rs._lib
    h = _handle(max_draft=4)
    io = [FAKE] * 5
    assert L.replayssm_step(h, *io, None) == rs.RSSM_E_STATE            # before load_state
    assert L.replayssm_spec_verify(h, 2, *io, None) == rs.RSSM_E_STATE
    assert L.replayssm_load_state(h, None, None) == rs.RSSM_OK          # batch 0: nothing launched
    assert L.replayssm_step(h, *io, None) == rs.RSSM_OK
    assert L.replayssm_step(h, None, None, None, None, None, None) == rs.RSSM_OK
    assert L.replayssm_step(h, FAKE + 4, FAKE, FAKE, FAKE, FAKE, None) == rs.RSSM_E_INVAL  # misaligned
    assert L.replayssm_rollback(h, FAKE, None) == rs.RSSM_E_STATE         # no verify pending
    assert L.replayssm_spec_verify(h, 0, *io, None) == rs.RSSM_E_INVAL
    assert L.replayssm_spec_verify(h, 5, *io, None) == rs.RSSM_E_INVAL    # T > max_draft
    assert L.replayssm_spec_verify(h, 4, *io, None) == rs.RSSM_OK
    assert L.replayssm_spec_verify(h, 2, *io, None) == rs.RSSM_E_STATE    # verify twice
    assert L.replayssm_step(h, *io, None) == rs.RSSM_E_STATE              # step while pending
    assert L.replayssm_flush(h, None, None) == rs.RSSM_E_STATE            # flush while pending
    assert L.replayssm_rollback(h, FAKE + 2, None) == rs.RSSM_E_INVAL     # misaligned counts
    assert L.replayssm_rollback(h, FAKE, None) == rs.RSSM_OK
    assert L.replayssm_rollback(h, FAKE, None) == rs.RSSM_E_STATE
    assert L.replayssm_flush(h, None, None) == rs.RSSM_OK
    assert L.replayssm_flush(h, FAKE + 2, None) == rs.RSSM_E_INVAL
    assert L.replayssm_materialize_state(h, FAKE + 8, None) == rs.RSSM_E_INVAL
    assert L.replayssm_materialize_state(h, FAKE, None) == rs.RSSM_OK
    assert L.replayssm_set_lockstep(h, 2) == rs.RSSM_E_INVAL
    assert L.replayssm_set_lockstep(None, 0) == rs.RSSM_E_INVAL
    assert L.replayssm_set_lockstep(h, 0) == rs.RSSM_OK
    assert L.replayssm_step(h, *io, None) == rs.RSSM_OK
    assert L.replayssm_set_lockstep(h, 1) == rs.RSSM_OK
    assert L.replayssm_destroy(h) == rs.RSSM_OK


def test_pointer_validation_before_state():
    """With a non-empty batch, NULL or misaligned device arrays are rejected before any state or
    device work (the handle here is never loaded, so valid arguments stop at RSSM_E_STATE)."""
    L = rs._lib
    h = _handle(batch=2, max_draft=2)
    io = [FAKE] * 5
    assert L.replayssm_load_state(h, None, None) == rs.RSSM_E_INVAL
    assert L.replayssm_load_state(h, FAKE + 4, None) == rs.RSSM_E_INVAL
    for i in range(5):
        bad = list(io)
        bad[i] = None
        assert L.replayssm_step(h, *bad, None) == rs.RSSM_E_INVAL
        assert L.replayssm_spec_verify(h, 2, *bad, None) == rs.RSSM_E_INVAL
        bad[i] = FAKE + 8
        assert L.replayssm_step(h, *bad, None) == rs.RSSM_E_INVAL
    assert L.replayssm_step(h, *io, None) == rs.RSSM_E_STATE
    assert L.replayssm_spec_verify(h, 3, *io, None) == rs.RSSM_E_INVAL
    assert L.replayssm_spec_verify(h, 2, *io, None) == rs.RSSM_E_STATE
    assert L.replayssm_rollback(h, None, None) == rs.RSSM_E_INVAL
    assert L.replayssm_rollback(h, FAKE, None) == rs.RSSM_E_STATE
    assert L.replayssm_materialize_state(h, None, None) == rs.RSSM_E_INVAL
    assert L.replayssm_flush(h, None, None) == rs.RSSM_E_STATE
    assert L.replayssm_destroy(h) == rs.RSSM_OK


def test_baselines_validate():
    L = rs._lib
    c = cfg()
    args = [FAKE] * 8
    assert L.conventional_step(ctypes.byref(c), *args, None) == rs.RSSM_OK
    bad = cfg(dstate=24)
    assert L.conventional_step(ctypes.byref(bad), *args, None) == rs.RSSM_E_UNSUPPORTED
    assert L.conventional_step(None, *args, None) == rs.RSSM_E_INVAL
    assert L.conventional_step(ctypes.byref(c), None, *args[1:], None) == rs.RSSM_OK      # batch 0
    c1 = cfg(batch=1)
    assert L.conventional_step(ctypes.byref(c1), None, *args[1:], None) == rs.RSSM_E_INVAL
    assert L.conventional_step(ctypes.byref(c1), FAKE + 4, *args[1:], None) == rs.RSSM_E_INVAL
    assert L.snapshot_spec_verify(ctypes.byref(c), FAKE, FAKE, 4, *([FAKE] * 7), None) == rs.RSSM_OK
    assert L.snapshot_spec_verify(ctypes.byref(c), FAKE, FAKE, 0, *([FAKE] * 7), None) == rs.RSSM_E_INVAL
    assert L.snapshot_spec_verify(ctypes.byref(c), FAKE, FAKE, 9, *([FAKE] * 7), None) == rs.RSSM_E_INVAL
    assert L.snapshot_commit(ctypes.byref(c), FAKE, FAKE, 4, None) == rs.RSSM_OK
    assert L.snapshot_commit(ctypes.byref(c1), FAKE, None, 4, None) == rs.RSSM_E_INVAL
    assert L.snapshot_spec_verify(ctypes.byref(c1), None, FAKE, 4, *([FAKE] * 7), None) == rs.RSSM_E_INVAL


def test_snapshot_spec_step_validates_before_launch():
    """The one-call snapshot baseline checks every argument of both halves before any launch."""
    L = rs._lib
    c, c1 = cfg(), cfg(batch=1)
    args = [FAKE] * 7                                  # x, B, C, dt, A, D, y
    assert L.snapshot_spec_step(ctypes.byref(c), FAKE, FAKE, 4, *args, FAKE, None) == rs.RSSM_OK   # batch 0
    assert L.snapshot_spec_step(ctypes.byref(c), FAKE, FAKE, 0, *args, FAKE, None) == rs.RSSM_E_INVAL
    assert L.snapshot_spec_step(ctypes.byref(c), FAKE, FAKE, 9, *args, FAKE, None) == rs.RSSM_E_INVAL
    assert L.snapshot_spec_step(ctypes.byref(c1), FAKE, FAKE, 4, *args, None, None) == rs.RSSM_E_INVAL
    assert L.snapshot_spec_step(ctypes.byref(c1), FAKE, FAKE, 4, *args, FAKE + 2, None) == rs.RSSM_E_INVAL
    assert L.snapshot_spec_step(ctypes.byref(c1), FAKE, None, 4, *args, FAKE, None) == rs.RSSM_E_INVAL
    assert L.snapshot_spec_step(ctypes.byref(c1), FAKE + 4, FAKE, 4, *args, FAKE, None) == rs.RSSM_E_INVAL
    assert L.snapshot_spec_step(ctypes.byref(cfg(dstate=24)), FAKE, FAKE, 4, *args, FAKE, None) == \
        rs.RSSM_E_UNSUPPORTED
    assert L.snapshot_spec_step(None, FAKE, FAKE, 4, *args, FAKE, None) == rs.RSSM_E_INVAL


def _shape_only(cls, **attrs):
    """An instance carrying shapes only (no handle, no workspace): enough for the binding's
    argument checks, which all run before the first library call."""
    obj = object.__new__(cls)
    obj.handle = None
    for k, v in attrs.items():
        setattr(obj, k, v)
    return obj


def test_binding_rejects_wrong_output_shapes():
    """Caller-supplied outputs of the wrong shape raise ValueError before any library call (an
    undersized buffer would otherwise let a kernel write past its end)."""
    import torch
    Bt, H, P, N, G, T, K = 2, 4, 16, 32, 2, 3, 4
    lay = _shape_only(rs.ReplaySSM, batch=Bt, nheads=H, headdim=P, dstate=N, ngroups=G,
                      cfg=rs.make_config(Bt, H, P, N, G, max_draft=T, d_conv=K))
    e = torch.empty
    tok = (e(Bt, H, P), e(Bt, G, N), e(Bt, G, N), e(Bt, H))
    with pytest.raises(ValueError, match="y has shape"):
        lay.step(*tok, y=e(Bt, H, P - 4))
    drafts = (e(Bt, T, H, P), e(Bt, T, G, N), e(Bt, T, G, N), e(Bt, T, H))
    with pytest.raises(ValueError, match="y has shape"):
        lay.spec_verify(*drafts, y=e(Bt, H, P))
    with pytest.raises(ValueError, match="out has shape"):
        lay.materialize_state(out=e(Bt, H, P, N // 2))
    CD = rs.conv_dim(lay.cfg)
    with pytest.raises(ValueError, match="o has shape"):
        lay.mixer_step(e(Bt, CD), e(Bt, H, P), e(Bt, H), o=e(Bt, H, P - 1))
    with pytest.raises(ValueError, match="o has shape"):
        lay.mixer_spec_verify(e(Bt, T, CD), e(Bt, T, H, P), e(Bt, T, H), o=e(Bt, T, H, P + 1))
    with pytest.raises(ValueError, match="out has shape"):
        lay.materialize_conv_state(out=e(Bt, K, CD))
    gl = _shape_only(rs.GDNReplay, batch=Bt, nheads=H, nkheads=G, dv=P, dk=N,
                     cfg=rs.make_gdn_config(Bt, H, G, P, N, max_draft=T))
    with pytest.raises(ValueError, match="out has shape"):
        gl.materialize_state(out=e(Bt, H, P, N - 1))
    q = e(Bt, G, N)
    with pytest.raises(ValueError, match="o has shape"):
        gl.step(q, q, e(Bt, H, P), e(Bt, H), e(Bt, H), o=e(Bt, H, P // 2))
    slots, cur = e(Bt, T + 1, H, P, N), e(Bt, dtype=torch.int32)
    A = e(H)
    with pytest.raises(ValueError, match="y has shape"):
        rs.snapshot_spec_step(lay.cfg, slots, cur, T, *drafts, A, A, e(Bt, T, H, P - 4), cur)
    with pytest.raises(ValueError, match="accepted has shape"):
        rs.snapshot_spec_step(lay.cfg, slots, cur, T, *drafts, A, A, e(Bt, T, H, P), e(Bt + 1, dtype=torch.int32))


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(rs.replayssm_status_string(s), str) and rs.replayssm_status_string(s)


# ---- Gated DeltaNet ABI (gdnreplay.h) ---------------------------------------------------------
GDN_HEADER = os.path.join(ROOT, "include", "gdnreplay.h")


def test_every_gdn_symbol_is_exported():
    text = re.sub(r"/\*.*?\*/", "", open(GDN_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                                  text, re.M)))
    assert len(names) >= 14
    for n in names:
        assert hasattr(rs._lib, n), f"{n} declared in gdnreplay.h but not exported"
    assert set(names) == set(rs.GDN_EXPORTED)


def gcfg(**kw):
    base = dict(batch=0, nheads=32, nkheads=16, dv=128, dk=128, buffer_len=16, max_draft=1)
    base.update(kw)
    return rs.make_gdn_config(**base)


def test_gdn_workspace_layout():
    c = gcfg(batch=256)
    lay = rs.gdnreplay_workspace_layout(c)
    Bt, H, G, Dv, Dk, L = 256, 32, 16, 128, 128, 16
    assert lay.master == 0 and lay.ring_k == Bt * H * Dv * Dk * 4
    assert lay.ring_v - lay.ring_k == Bt * G * L * Dk * 4
    assert lay.ring_a - lay.ring_v == Bt * H * L * Dv * 4
    assert lay.ring_b - lay.ring_a == Bt * H * L * 4
    assert lay.total == rs.gdnreplay_workspace_bytes(c)
    for name in ("master", "ring_k", "ring_v", "ring_a", "ring_b", "pos", "ckpt_pos", "counters", "flag"):
        assert getattr(lay, name) % 256 == 0
    assert lay.read_copy == lay.scale == lay.ring_k                     # fp32 reads: no copy
    lb = rs.gdnreplay_workspace_layout(gcfg(batch=256, read_prec="bf16"))
    assert lb.scale - lb.read_copy == Bt * H * Dv * Dk * 2                # bf16 copy
    assert lb.ring_k == lb.scale
    l8 = rs.gdnreplay_workspace_layout(gcfg(batch=256, read_prec="fp8"))
    assert l8.scale - l8.read_copy == Bt * H * Dv * Dk                    # one byte per value
    assert l8.ring_k - l8.scale == Bt * H * ((Dv + 63) // 64) * 4         # a scale per 64 value rows
    l4 = rs.gdnreplay_workspace_layout(gcfg(batch=256, read_prec="mxfp4"))
    assert l4.scale - l4.read_copy == Bt * H * Dv * Dk // 2               # two codes per byte
    assert l4.ring_k - l4.scale == Bt * H * Dv * Dk // 32                 # an E8M0 byte per 32 values


@pytest.mark.parametrize("kw,status", [
    (dict(dk=48), rs.RSSM_E_UNSUPPORTED),
    (dict(dk=512), rs.RSSM_E_UNSUPPORTED),
    (dict(dv=66), rs.RSSM_E_INVAL),
    (dict(dv=260), rs.RSSM_E_UNSUPPORTED),
    (dict(nheads=6, nkheads=4), rs.RSSM_E_INVAL),
    (dict(buffer_len=0), rs.RSSM_E_INVAL),
    (dict(buffer_len=4, max_draft=5), rs.RSSM_E_INVAL),
    (dict(buffer_len=65), rs.RSSM_E_UNSUPPORTED),
    (dict(buffer_len=16, max_draft=9), rs.RSSM_E_UNSUPPORTED),
    (dict(batch=-1), rs.RSSM_E_INVAL),
    (dict(read_prec=4), rs.RSSM_E_INVAL),
    (dict(read_prec=-1), rs.RSSM_E_INVAL),
    (dict(read_prec="mxfp4", dk=16), rs.RSSM_E_UNSUPPORTED),
])
def test_gdn_invalid_configs_rejected(kw, status):
    c = gcfg(**kw)
    assert rs.gdnreplay_workspace_bytes(c) == 0
    h = ctypes.c_void_p()
    assert rs._lib.gdnreplay_create(ctypes.byref(c), FAKE, 1 << 40, ctypes.byref(h)) == status
    assert not h.value


def test_gdn_state_machine_on_host():
    L = rs._lib
    c = gcfg(max_draft=4)
    h = ctypes.c_void_p()
    need = rs.gdnreplay_workspace_bytes(c)
    assert L.gdnreplay_create(ctypes.byref(c), None, need, ctypes.byref(h)) == rs.RSSM_E_WORKSPACE
    assert L.gdnreplay_create(ctypes.byref(c), FAKE + 16, need, ctypes.byref(h)) == rs.RSSM_E_WORKSPACE
    assert L.gdnreplay_create(ctypes.byref(c), FAKE, need, ctypes.byref(h)) == rs.RSSM_OK
    io = [FAKE] * 6
    assert L.gdnreplay_step(h, *io, None) == rs.RSSM_E_STATE              # before load_state
    assert L.gdnreplay_load_state(h, None, None) == rs.RSSM_OK            # batch 0: nothing launched
    assert L.gdnreplay_step(h, *io, None) == rs.RSSM_OK
    assert L.gdnreplay_step(h, FAKE + 4, *io[1:], None) == rs.RSSM_E_INVAL  # misaligned
    assert L.gdnreplay_rollback(h, FAKE, None) == rs.RSSM_E_STATE          # no verify pending
    assert L.gdnreplay_spec_verify(h, 0, *io, None) == rs.RSSM_E_INVAL
    assert L.gdnreplay_spec_verify(h, 5, *io, None) == rs.RSSM_E_INVAL     # T > max_draft
    assert L.gdnreplay_spec_verify(h, 4, *io, None) == rs.RSSM_OK
    assert L.gdnreplay_spec_verify(h, 2, *io, None) == rs.RSSM_E_STATE     # verify twice
    assert L.gdnreplay_step(h, *io, None) == rs.RSSM_E_STATE               # step while pending
    assert L.gdnreplay_flush(h, None, None) == rs.RSSM_E_STATE
    assert L.gdnreplay_rollback(h, FAKE + 2, None) == rs.RSSM_E_INVAL
    assert L.gdnreplay_rollback(h, FAKE, None) == rs.RSSM_OK
    assert L.gdnreplay_flush(h, None, None) == rs.RSSM_OK
    assert L.gdnreplay_materialize_state(h, FAKE + 8, None) == rs.RSSM_E_INVAL
    assert L.gdnreplay_destroy(h) == rs.RSSM_OK
    assert L.gdnreplay_destroy(None) == rs.RSSM_OK


def test_gdn_pointer_validation_before_state():
    L = rs._lib
    c = gcfg(batch=2, max_draft=2)
    h = ctypes.c_void_p()
    assert L.gdnreplay_create(ctypes.byref(c), FAKE, rs.gdnreplay_workspace_bytes(c), ctypes.byref(h)) == rs.RSSM_OK
    io = [FAKE] * 6
    assert L.gdnreplay_load_state(h, None, None) == rs.RSSM_E_INVAL
    for i in range(6):
        bad = list(io)
        bad[i] = None
        assert L.gdnreplay_step(h, *bad, None) == rs.RSSM_E_INVAL
        assert L.gdnreplay_spec_verify(h, 2, *bad, None) == rs.RSSM_E_INVAL
    assert L.gdnreplay_step(h, *io, None) == rs.RSSM_E_STATE
    assert L.gdn_conventional_step(ctypes.byref(c), None, *io, None) == rs.RSSM_E_INVAL
    assert L.gdn_conventional_step(ctypes.byref(gcfg()), FAKE, *io, None) == rs.RSSM_OK   # batch 0
    assert L.gdn_snapshot_spec_verify(ctypes.byref(c), FAKE, FAKE, 9, *io, None) == rs.RSSM_E_INVAL
    assert L.gdnreplay_destroy(h) == rs.RSSM_OK


def test_mixer_layout():
    Bt, H, P, N, G, K, T = 4, 8, 64, 128, 2, 4, 3
    CD = H * P + 2 * G * N
    lay = rs.replayssm_workspace_layout(cfg(batch=Bt, nheads=H, ngroups=G, d_conv=K, max_draft=T))
    assert lay.conv_ring % 256 == 0
    assert lay.pos - lay.conv_ring == -(-Bt * (K - 1 + T) * CD * 4 // 256) * 256   # R = K - 1 + T slots
    plain = rs.replayssm_workspace_layout(cfg(batch=Bt, nheads=H, ngroups=G))
    assert plain.pos == plain.conv_ring                                           # no ring without edges
    assert rs.conv_dim(cfg(nheads=H, ngroups=G)) == CD


def test_mixer_entry_points_on_host():
    """Host-side rules of the mixer calls (batch 0, fake pointers; nothing reaches the GPU)."""
    L = rs._lib
    plain = _handle()
    mix = _handle(d_conv=4, max_draft=2)
    io = [FAKE] * 4
    assert L.replayssm_set_mixer(plain, FAKE, FAKE, FAKE) == rs.RSSM_E_INVAL       # no edges on this handle
    assert L.replayssm_mixer_step(plain, *io, None) == rs.RSSM_E_INVAL
    assert L.replayssm_load_conv_state(plain, None, None) == rs.RSSM_E_INVAL
    assert L.replayssm_mixer_step(mix, *io, None) == rs.RSSM_E_STATE             # parameters not given
    assert L.replayssm_set_mixer(mix, None, FAKE, FAKE) == rs.RSSM_E_INVAL
    assert L.replayssm_set_mixer(mix, FAKE, FAKE + 2, FAKE) == rs.RSSM_E_INVAL   # misaligned
    assert L.replayssm_set_mixer(mix, FAKE, FAKE, FAKE) == rs.RSSM_OK
    assert L.replayssm_mixer_step(mix, *io, None) == rs.RSSM_E_STATE             # before load_state
    assert L.replayssm_load_conv_state(mix, None, None) == rs.RSSM_E_STATE
    assert L.replayssm_load_state(mix, None, None) == rs.RSSM_OK
    assert L.replayssm_load_conv_state(mix, None, None) == rs.RSSM_OK
    assert L.replayssm_mixer_step(mix, *io, None) == rs.RSSM_OK
    assert L.replayssm_mixer_step(mix, FAKE + 2, FAKE, FAKE, FAKE, None) == rs.RSSM_E_INVAL
    assert L.replayssm_step(mix, *([FAKE] * 5), None) == rs.RSSM_E_INVAL         # plain calls refused
    assert L.replayssm_spec_verify(mix, 2, *([FAKE] * 5), None) == rs.RSSM_E_INVAL
    assert L.replayssm_mixer_spec_verify(plain, 2, *io, None) == rs.RSSM_E_INVAL
    assert L.replayssm_mixer_spec_verify(mix, 3, *io, None) == rs.RSSM_E_INVAL     # T > max_draft
    assert L.replayssm_mixer_spec_verify(mix, 2, *io, None) == rs.RSSM_OK
    assert L.replayssm_mixer_step(mix, *io, None) == rs.RSSM_E_STATE              # verify pending
    assert L.replayssm_load_conv_state(mix, None, None) == rs.RSSM_E_STATE
    assert L.replayssm_rollback(mix, FAKE, None) == rs.RSSM_OK
    assert L.replayssm_materialize_conv_state(mix, FAKE, None) == rs.RSSM_OK
    assert L.replayssm_materialize_conv_state(mix, FAKE + 2, None) == rs.RSSM_E_INVAL
    for h in (plain, mix):
        assert L.replayssm_destroy(h) == rs.RSSM_OK


def test_conventional_mixer_argument_checks():
    L = rs._lib
    c = cfg(d_conv=4)
    args = [FAKE] * 9            # xbc, z, dt_raw, A, D, conv_w, conv_b, dt_bias, o
    assert L.conventional_mixer_step(ctypes.byref(c), FAKE, FAKE, 0, *args, None) == rs.RSSM_OK   # batch 0
    assert L.conventional_mixer_step(ctypes.byref(c), FAKE, FAKE, -1, *args, None) == rs.RSSM_E_INVAL
    c0 = cfg()
    assert L.conventional_mixer_step(ctypes.byref(c0), FAKE, FAKE, 0, *args, None) == rs.RSSM_E_INVAL
    c5 = cfg(d_conv=5)
    assert L.conventional_mixer_step(ctypes.byref(c5), FAKE, FAKE, 0, *args, None) == rs.RSSM_E_UNSUPPORTED
    bad = list(args)
    bad[5] = None                                                                     # conv_w NULL
    assert L.conventional_mixer_step(ctypes.byref(c), FAKE, FAKE, 0, *bad, None) == rs.RSSM_E_INVAL
