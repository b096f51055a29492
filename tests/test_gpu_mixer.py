"""GPU parity of the mixer block (m3_mixer_prefill / m3_mixer_decode_step) against
the fp64 block oracle (oracle/mixer.py, bf16 storage points made explicit).

The block's projections run as hipBLASLt GEMMs with fp32 accumulation; the
oracle sums in fp64 and rounds at the same storage points, so a few bf16
roundings can land on the other side of a tie and the rest of the block carries
that. Bar: 2e-2 max-relative error per sequence (the recurrence's bf16 bar),
for the block output and the final state.
"""
import numpy as np
import pytest
import torch

from oracle import mixer as omix
from mamba_ssm_scan_amd import binding, inputs
from tests.util import f64, to_dev

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _rel_per_batch(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    g = got.reshape(got.shape[0], -1)
    r = ref.reshape(ref.shape[0], -1)
    return float((np.abs(g - r).max(axis=1) / np.abs(r).max(axis=1)).max())


def _weights(**kw):
    w = inputs.mixer_inputs(**kw)
    return w, to_dev(w)


CASES = [
    # b, L, d_model, H, G, P, N, R, path
    (2, 70, 64, 2, 1, 16, 32, 1, "MFMA"),    # chunked recurrence, rows and columns zero-padded, ragged chunk
    (1, 100, 128, 2, 1, 64, 128, 1, "MFMA"),  # chunked R 1 kernel
    (2, 65, 96, 2, 2, 64, 128, 4, "MFMA"),    # chunked R 4, one B, C group per head
    (1, 40, 64, 3, 1, 32, 64, 5, "SCAN"),     # rank 5: the token-walk recurrence
    (1, 40, 64, 3, 1, 32, 64, 3, "MFMA"),     # rank 3 on the R 4 kernel
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_mixer_prefill_matches_oracle(case):
    b, L, dm, H, G, P, N, R, path = case
    print(f"mixer prefill case {case}", flush=True)
    w, d = _weights(batch=b, seqlen=L, d_model=dm, heads=H, groups=G, headdim=P, dstate=N, rank=R, wid=600 + L)
    assert binding.plan(binding.dims(b, L, H, G, P, N), R, 64, binding.M3_BF16).path == \
        getattr(binding, "M3_PATH_" + path)
    m = binding.Mixer(d)
    out, h = m.prefill(d["u"], h_out=True)
    torch.cuda.synchronize()
    ref, h_ref, _ = omix.forward(w, w["u"])
    e_out, e_h = _rel_per_batch(f64(out), ref), _rel_per_batch(f64(h), h_ref)
    print(f"  out {e_out:.2e}, h_out {e_h:.2e}", flush=True)
    assert e_out <= TOL and e_h <= TOL


@pytest.mark.parametrize("R,N,P", [(1, 128, 64), (4, 128, 64), (2, 32, 16)])
def test_mixer_prefill_then_decode(R, N, P):
    """A prefill of 40 tokens hands its state to the decode state; 6 decode steps follow;
    against the oracle block over all 46 tokens."""
    b, L, k, dm, H = 2, 46, 40, 64, 2
    print(f"mixer prefill {k} + decode {L - k}, R {R}, N {N}, P {P}", flush=True)
    w, d = _weights(batch=b, seqlen=L, d_model=dm, heads=H, groups=1, headdim=P, dstate=N, rank=R, wid=650 + R)
    m = binding.Mixer(d)
    st = m.decode_state(b)
    out_pre, _ = m.prefill(d["u"][:, :k].contiguous(), state=st)
    assert st.t == k
    outs = [m.decode_step(st, d["u"][:, t].contiguous()) for t in range(k, L)]
    torch.cuda.synchronize()
    got = torch.cat([out_pre, torch.stack(outs, 1)], 1)
    ref, h_ref, _ = omix.forward(w, w["u"])
    e_out, e_h = _rel_per_batch(f64(got), ref), _rel_per_batch(f64(st.h), h_ref)
    e_dec = _rel_per_batch(f64(torch.stack(outs, 1)), ref[:, k:])
    print(f"  out {e_out:.2e} (decode part {e_dec:.2e}), state {e_h:.2e}", flush=True)
    assert e_out <= TOL and e_dec <= TOL and e_h <= TOL


def test_mixer_zero_gate_and_h0():
    """W_z = 0 closes the gate exactly (out == 0); a given h0 reaches h_out."""
    b, L, dm, H, P, N, R = 1, 20, 64, 2, 16, 32, 1
    w, d = _weights(batch=b, seqlen=L, d_model=dm, heads=H, groups=1, headdim=P, dstate=N, rank=R, wid=690)
    d["W_z"] = torch.zeros_like(d["W_z"])
    w["W_z"] = d["W_z"].cpu()
    h0 = torch.randn((b, H, N, P), generator=torch.Generator().manual_seed(5)) * 0.1
    m = binding.Mixer(d)
    out, h = m.prefill(d["u"], h0=h0.cuda(), h_out=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
    _, h_ref, _ = omix.forward(w, w["u"], h0=h0)
    assert _rel_per_batch(f64(h), h_ref) <= TOL


def test_mixer_decode_batch_over_128():
    """Batch 130 decode steps (projection GEMMs with 130 rows, more decode workgroups than
    CUs): 3 prefill tokens, then 2 steps, against the oracle."""
    b, L, k, dm, H, P, N, R = 130, 5, 3, 64, 2, 16, 32, 2
    print("mixer decode at batch 130", flush=True)
    w, d = _weights(batch=b, seqlen=L, d_model=dm, heads=H, groups=1, headdim=P, dstate=N, rank=R, wid=695)
    m = binding.Mixer(d)
    st = m.decode_state(b)
    out_pre, _ = m.prefill(d["u"][:, :k].contiguous(), state=st)
    outs = [m.decode_step(st, d["u"][:, t].contiguous()) for t in range(k, L)]
    torch.cuda.synchronize()
    ref, h_ref, _ = omix.forward(w, w["u"])
    e_dec = _rel_per_batch(f64(torch.stack(outs, 1)), ref[:, k:])
    e_h = _rel_per_batch(f64(st.h), h_ref)
    print(f"  decode out {e_dec:.2e}, state {e_h:.2e}", flush=True)
    assert e_dec <= TOL and e_h <= TOL
