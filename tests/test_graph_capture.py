"""The default fills inside a HIP graph: captured once on a stream, replayed several times.

Each fill is kernel launches on the caller's stream; the default f64 normal fill keeps no
per-device state beyond its constant tables and records no event, so a sequence of fills
captures as kernel nodes.  Per-device state is created on a fill's first call, which
allocates, so every fill runs once eagerly before the capture.  The replays are separated
by eager work that overwrites the outputs, and every replay is checked against the oracle
(graph nodes that reset memory have misbehaved on replays after the first on this
hardware; these fills have none)."""
import numpy as np
import pytest
import torch

import bulk_fills_amd as tk
import oracle
import tk_inputs
from gpu_harness import assert_bits_equal, log

pytestmark = pytest.mark.gpu

PK = 0x0123456789ABCDEF


def test_captured_fills_replay_to_the_oracle():
    n = (1 << 20) + 3
    dev = torch.device("cuda")
    u32 = torch.empty(n, dtype=torch.int32, device=dev)
    f64 = torch.empty(n, dtype=torch.float64, device=dev)
    xh = tk_inputs.normal_x(n)
    x = torch.from_numpy(xh).to(dev)
    y = torch.empty(n, dtype=torch.float32, device=dev)
    mask = torch.empty(n, dtype=torch.uint8, device=dev)
    ch = torch.empty(n, dtype=torch.int32, device=dev)
    ph = torch.empty(n, dtype=torch.int32, device=dev)
    w = tk_inputs.zipf_weights()
    table = tk.tk_alias_create(w)
    q, al, _ = oracle.alias_build(w)

    want_u32 = oracle.fill_u32(1, 3, n)
    want_f64, path = oracle.fill_normal_f64(2, 1, n, with_path=True)
    want_y, want_mask = oracle.dropout_f32(tk_inputs.DROPOUT_KEY, 5, xh, tk_inputs.DROPOUT_P)
    want_ch = oracle.fill_choice_u32(4, 0, n, q, al)
    want_ph = oracle.philox_fill_u32(PK, 1, n)  # a start that straddles Philox blocks

    def fills():
        tk.tk_fill_u32(1, 3, n, u32)
        tk.tk_fill_normal_f64(2, 1, n, f64)
        tk.tk_dropout_f32(tk_inputs.DROPOUT_KEY, 5, n, tk_inputs.DROPOUT_P, x, y, mask)
        tk.tk_fill_choice_u32(4, 0, n, table, ch)
        tk.tk_philox_fill_u32(PK, 1, n, ph)

    def check(what):
        torch.cuda.synchronize()
        assert_bits_equal(u32.cpu().numpy().view(np.uint32), want_u32, f"{what}: u32")
        got = f64.cpu().numpy()
        exact = path != 2
        assert_bits_equal(got[exact], want_f64[exact], f"{what}: normal_f64")
        if (~exact).any():
            assert np.max(np.abs(got[~exact] / want_f64[~exact] - 1)) <= 1e-12, f"{what}: normal_f64 tail"
        assert_bits_equal(y.cpu().numpy(), want_y, f"{what}: dropout y")
        assert_bits_equal(mask.cpu().numpy(), want_mask, f"{what}: dropout mask")
        assert_bits_equal(ch.cpu().numpy().view(np.uint32), want_ch, f"{what}: choice")
        assert_bits_equal(ph.cpu().numpy().view(np.uint32), want_ph, f"{what}: philox")

    log("graph: eager fills (create the per-device state)")
    fills()
    check("eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fills()
    for r in range(4):
        for t in (u32, f64, y, mask, ch, ph):  # eager work between the replays
            t.zero_()
        torch.cuda.synchronize()
        log(f"graph: replay {r}")
        g.replay()
        check(f"replay {r}")
    del g
