"""The encoder on a stream of its own beside a decode-like load on another.

Serving stacks schedule the encoder on a side stream next to the language
model's decode (TRT-LLM's "Multimodal Encoder Side Stream", (1) SERVICEABILITY
JOIN of the "Kimi-Audio-7B-Instruct" record). What must hold: the encoder's
output under load meets the bf16 bar against the oracle and is the same bits
as alone, the load's result is unchanged too, and the overlap measurement in
bench.py returns a consistent record.
"""
import os
import sys

import pytest
import torch

import oracle
import synth
from tests import parity
from synth.decode_load import DecodeLoad, DecodeShape

pytestmark = pytest.mark.gpu

DEV = "cuda"
SMALL_LOAD = DecodeShape(layers=4, hidden=1024, kv_dim=256, inter=2816, tokens=16)


@pytest.fixture(scope="module")
def encoder():
    import audio_encoder_tower_amd as aenc
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    w = synth.get_workload("whisper_large_b1")
    w = w.replace(geom=w.geom.replace(batch=4, n_layers=2, n_frames=1000), init="perturbed")
    W = synth.make_weights(w)
    enc = aenc.Encoder(w.geom, {k: torch.from_numpy(v).to(DEV).to(torch.bfloat16) for k, v in W.items()})
    mel_np = synth.make_mel(w)
    mel = torch.from_numpy(mel_np).to(DEV).to(torch.bfloat16)
    want = oracle.encode(w.geom, W, mel_np)
    yield w, enc, mel, want
    enc.close()


def test_outputs_unchanged_under_concurrent_load(encoder):
    w, enc, mel, want = encoder
    load = DecodeLoad(SMALL_LOAD)
    ref_enc = enc.forward(mel).clone()
    ref_dec = load.step().clone()
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs, decs = [], []
    for _ in range(3):
        o = torch.empty_like(ref_enc)
        enc.forward(mel, out=o, stream=sa)        # the encoder's stream
        with torch.cuda.stream(sb):               # the decode stream, unsynchronised with it
            for _ in range(4):
                d = load.step()
            decs.append(d)
        outs.append(o)
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert torch.equal(o, ref_enc)
        m = parity.assert_bf16_parity(o.double().cpu().numpy(), want, f"forward {i} under load")
    print("under load vs oracle", m)
    for d in decs:
        assert torch.equal(d, ref_dec)


def test_overlap_record(encoder):
    w, enc, mel, want = encoder
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    out = torch.empty(enc.out_shape, dtype=enc.out_dtype, device=DEV)
    rec = bench.side_stream_leg(enc, mel, None, out, audio_s=40.0, n_enc=2, gate_forwards=2, shape=SMALL_LOAD)
    assert rec["encoder_forwards"] == 2 and rec["decode_steps"] >= 1
    for k in ("encoder_alone_ms", "decode_alone_ms", "concurrent_ms"):
        assert rec[k] > 0
    # the concurrent run ends when its later stream ends
    assert rec["concurrent_ms"] == max(rec["encoder_done_ms"], rec["decode_done_ms"])
    assert rec["speedup_vs_serial"] == pytest.approx(
        (rec["encoder_alone_ms"] + rec["decode_alone_ms"]) / rec["concurrent_ms"], rel=1e-3)
    torch.cuda.synchronize()
    assert torch.equal(out, enc.forward(mel))
    parity.assert_bf16_parity(out.double().cpu().numpy(), want, "output after the overlap record")
