"""Watchdog of the step kernel's bounded waits (include/mk.h, mk_set_spin_limit).

A stage of the per-op path launched on its own (mk_debug_stage) waits for
inputs that its producers never wrote in this step: an unsatisfiable wait.
With a small spin limit every wave must give up, the error record must name
the wait (code 1, the stage's opcode), the grid must drain (the call returns
and the device stays usable), and decoding afterwards must again match the
oracle: the aborted launch leaves nothing that a later step takes for data."""
import numpy as np
import pytest

import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu

OP_ATTENTION, OP_RMS_LM_HEAD = 2, 7


@pytest.mark.parametrize("multikernel", [False, True], ids=["megakernel", "multikernel"])
def test_unsatisfiable_wait_reports_and_recovers(multikernel):
    shape = synth.TINY
    w = synth.make_weights(shape)
    B, max_seq = 2, 32
    dec = H.GpuDecoder(shape, w, B, max_seq)
    mk, torch = dec.mk, dec.torch
    try:
        prompt = synth.make_prompts(shape.vocab, B, 12)
        run = H.Run([], [], [])

        def step(i):
            toks, pos = prompt[:, i], np.full(B, i, dtype=np.int32)
            run.tokens.append(toks.copy())
            run.positions.append(pos.copy())
            run.logits.append(dec.step(toks, pos, multikernel))

        for i in range(4):
            step(i)
        n_layers = shape.n_layers
        for stage, op in [(1, OP_ATTENTION), (6 * n_layers, OP_RMS_LM_HEAD)]:
            mk.mk_set_spin_limit(dec.h, 2000)
            dec.tokens.copy_(torch.as_tensor(prompt[:, 4].astype(np.int32)))
            dec.positions.fill_(4)
            mk.mk_debug_stage(dec.h, stage, dec.tokens, dec.positions, dec.kv, dec.logits, mk.current_stream())
            torch.cuda.synchronize()
            err = mk.mk_get_device_error(dec.h)
            assert err is not None and err.code == 1, "the bounded wait did not report"
            assert err.opcode == op, (err.opcode, op)
            assert mk.mk_get_device_error(dec.h) is None, "reading the record clears it"
            mk.mk_set_spin_limit(dec.h, 0)
        for i in range(4, 12):  # position 4 is decoded for real now
            step(i)
    finally:
        dec.close()
    ref = H.oracle_replay(shape, w, B, max_seq, run)
    stats = H.compare(run, ref, "after watchdog")
    print("watchdog", "multikernel" if multikernel else "megakernel", stats)
