"""The allocation-free frame loop: tts_run_frames_noalloc (exchange buffers in the library's static
scratch array, frames launched one by one) against tts_run_frames (exchange buffers in the
context's workspace, the captured frame graph), through the C ABI, on two calls in a row, the
second with fewer frames, for bf16 and E4M3 weights. Both paths run the same kernels on the same
inputs, so codes and the logits after them must be identical bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

from autoregressive_tts_decode_amd import config, synth, tts

pytestmark = pytest.mark.gpu
GREEDY = config.GREEDY.as_dict()


def _bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


@pytest.mark.parametrize("name", ["1.7b", "1.7b-fp8"])
def test_noalloc_frames_equal_the_graph_frames(name):
    assert torch.cuda.is_available(), "the gpu tests need a HIP device"
    d = torch.device("cuda:0")
    model = config.MODELS[name]
    w = synth.make_weights(model, 0)
    dw = tts.weights_to_device(w, model, d)
    dec = tts.TTSDecoder(model, 1, 64, 32)
    dec.load_weights(dw)
    assert dec.exec_mode() == (tts.EXEC_PERSISTENT, tts.PERSISTENT_CODEPRED | tts.PERSISTENT_TALKER)
    lib = tts.load_library()
    ids = torch.from_numpy(synth.random_ids(16, model.text_vocab, seed=7)).to(d)
    greedy = tts.sampling_struct(GREEDY)
    probe = torch.full((1,), 11, dtype=torch.int32, device=d)
    a = torch.zeros((1, 15), dtype=torch.int32, device=d)
    Va = model.codepred.vocab
    for F in (8, 3):  # two calls in a row, the second with fewer frames
        print(f"{name} frames {F}: graph", flush=True)
        ref = torch.full((1, 32, 16), -1, dtype=torch.int32, device=d)
        al_ref = torch.zeros((1, 15, Va), dtype=torch.float32, device=d)
        dec.prefill(ids)
        dec.run_frames(F, GREEDY, GREEDY, None, ref)
        dec.codepred_frame(probe, GREEDY, None, a, logits=al_ref)
        torch.cuda.synchronize()
        prog_ref = dec.progress()
        print(f"{name} frames {F}: noalloc", flush=True)
        got = torch.full((1, 32, 16), -1, dtype=torch.int32, device=d)
        al_got = torch.zeros((1, 15, Va), dtype=torch.float32, device=d)
        dec.prefill(ids)
        rc = lib.tts_run_frames_noalloc(dec.ctx, F, ctypes.byref(greedy), ctypes.byref(greedy), None, got.data_ptr())
        assert rc == tts.TTS_OK, lib.tts_last_error(dec.ctx)
        assert dec.progress() == prog_ref
        dec.codepred_frame(probe, GREEDY, None, a, logits=al_got)
        torch.cuda.synchronize()
        assert dec.device_status() == 0
        np.testing.assert_array_equal(got.cpu().numpy(), ref.cpu().numpy())
        np.testing.assert_array_equal(_bits(al_got.cpu().numpy()), _bits(al_ref.cpu().numpy()))
    # what it does not run: sampled acoustic tokens, or the per-op kernels
    sampled = tts.sampling_struct(config.ACOUSTIC_SAMPLED.as_dict())
    u = torch.zeros((1, 32, 16), dtype=torch.float32, device=d)
    got = torch.zeros((1, 32, 16), dtype=torch.int32, device=d)
    dec.prefill(ids)
    assert lib.tts_run_frames_noalloc(dec.ctx, 1, ctypes.byref(greedy), ctypes.byref(sampled), u.data_ptr(),
                                      got.data_ptr()) == tts.TTS_E_UNSUPPORTED
    dec.set_exec_mode(tts.EXEC_KERNELS)
    assert lib.tts_run_frames_noalloc(dec.ctx, 1, ctypes.byref(greedy), ctypes.byref(greedy), None,
                                      got.data_ptr()) == tts.TTS_E_UNSUPPORTED
    dec.close()
    del dw
    torch.cuda.empty_cache()
