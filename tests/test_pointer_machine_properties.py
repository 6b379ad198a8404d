"""Property tests of the pointer and flush machine (reading R2/R5 of oracle.c) over random
buffer lengths, draft limits and operation streams (hypothesis).

The oracle's replay machine (with one 1x1x1 head: only its pointers matter) is run against a
plain integer model written here from the rules: a standard step commits one record and flushes
the sequence when more than L - T_max records are pending; a verify of T <= T_max drafts leaves
the pointers alone; its rollback commits the accepted prefix (0..T) and then flushes under the
same rule; an explicit flush folds every pending record of the selected sequences. Properties:
the two agree on (pos, ckpt_pos) of every sequence after every operation; 0 <= pos - ckpt_pos
<= L - T_max between calls; ckpt_pos never moves backwards and only ever jumps to pos; the
machine rejects a second verify, a rollback without one and accept counts above T.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle

Bt = 3


def _machine(L, Tmax):
    z = np.zeros((Bt, 1, 1, 1), np.float32)
    return oracle.Replay(z, np.array([-1.0], np.float32), np.zeros(1, np.float32), 1, L, Tmax)


ops = st.lists(
    st.one_of(
        st.tuples(st.just("step")),
        st.tuples(st.just("spec"), st.integers(1, 8), st.lists(st.integers(0, 8), min_size=Bt, max_size=Bt)),
        st.tuples(st.just("flush"), st.lists(st.booleans(), min_size=Bt, max_size=Bt)),
    ),
    min_size=1, max_size=40)


@settings(max_examples=150, deadline=None)
@given(L=st.integers(1, 16), tdiv=st.integers(0, 7), stream=ops)
def test_pointer_machine_matches_the_rules(L, tdiv, stream):
    Tmax = 1 + tdiv % min(L, 8)
    lim = L - Tmax
    m = _machine(L, Tmax)
    pos = [0] * Bt
    ck = [0] * Bt
    one = [np.zeros((Bt, 1, 1), np.float32)] * 3 + [np.zeros((Bt, 1), np.float32)]
    for op in stream:
        if op[0] == "step":
            m.step(*one)
            for b in range(Bt):
                pos[b] += 1
                if pos[b] - ck[b] > lim:
                    ck[b] = pos[b]
        elif op[0] == "spec":
            T = 1 + (op[1] - 1) % Tmax
            acc = np.array([a % (T + 1) for a in op[2]], np.int32)
            drafts = [np.zeros((Bt, T, 1, 1), np.float32)] * 3 + [np.zeros((Bt, T, 1), np.float32)]
            m.verify(T, *drafts)
            with pytest.raises(RuntimeError):
                m.verify(T, *drafts)                       # a second verify is refused
            if T < 8:
                with pytest.raises(RuntimeError):
                    m.rollback(np.full(Bt, T + 1, np.int32))  # an accept count above T is refused
            m.rollback(acc)
            for b in range(Bt):
                pos[b] += int(acc[b])
                if pos[b] - ck[b] > lim:
                    ck[b] = pos[b]
        else:
            mask = np.array(op[1], np.int32)
            m.flush(mask)
            for b in range(Bt):
                if mask[b]:
                    ck[b] = pos[b]
        got_pos, got_ck = m.pointers()
        assert list(got_pos) == pos and list(got_ck) == ck, op
        for b in range(Bt):
            assert 0 <= pos[b] - ck[b] <= lim
    with pytest.raises(RuntimeError):
        m.rollback(np.zeros(Bt, np.int32))                  # no verify pending


@settings(max_examples=60, deadline=None)
@given(L=st.integers(1, 32), steps=st.integers(1, 100))
def test_standard_decoding_flushes_every_L_steps(L, steps):
    """Standard decoding (T_max = 1): the checkpoint moves exactly on the steps whose append fills
    the buffer, t = L-1, 2L-1, ... (0-based), to pos; count = (t+1) mod L after step t."""
    m = _machine(L, 1)
    one = [np.zeros((Bt, 1, 1), np.float32)] * 3 + [np.zeros((Bt, 1), np.float32)]
    for t in range(steps):
        _, ck_before = m.pointers()
        m.step(*one)
        pos, ck = m.pointers()
        assert np.all(pos == t + 1)
        assert np.all(pos - ck == (t + 1) % L)
        assert np.all(ck != ck_before) == ((t + 1) % L == 0)
