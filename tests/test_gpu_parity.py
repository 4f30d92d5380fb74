"""GPU parity: the HIP path (through the C ABI) against the oracle.

Bars (per step, per stream):
  * logits: max|dlogit| <= tol * max|logit|, tol = 1e-4 for the fp32 model,
    1e-2 for the bf16 models;
  * greedy tokens: the GPU's own argmax equals the oracle's wherever the
    oracle's top-2 margin exceeds 0.05 (near ties are counted, not compared);
  * sampled tokens: equal given the same uniforms, except draws whose
    boundary lies within the model's logit tolerance (counted): the GPU
    draws from its own logits, which may differ from the oracle's by up to
    that tolerance.
End-to-end comparisons are teacher-forced with the oracle's codes: random
weights leave many greedy steps near a tie, so free-running streams part
ways within a few frames. A free-running GPU run is checked the other way
round: the oracle, teacher-forced along the GPU's own codes, must find each
non-exempt code to be its argmax. For the fp32 model a step is near a tie
when its top-2 margin is at most 2e-4 max|logit| (twice its logit bar).
"""
import numpy as np
import pytest
import torch

from autoregressive_tts_decode_amd import config, synth, tts
from oracle import OracleModel
from oracle.decoder import linear
from oracle.sampler import sample_token
from parity_util import (MIN_CHECKED, rowwise_rel_err, greedy_agreement, top2_margin, sample_exempt, check_free_running,
                         check_stop_masking)

pytestmark = pytest.mark.gpu
GREEDY = config.GREEDY.as_dict()
SEM = config.SEMANTIC_SAMPLED.as_dict()
AC = config.ACOUSTIC_SAMPLED.as_dict()


def dev():
    assert torch.cuda.is_available(), "the gpu tests need a HIP device"
    return torch.device("cuda:0")


def make_decoder(model, batch, cap, frames, weights):
    dw = tts.weights_to_device(weights, model, dev())
    dec = tts.TTSDecoder(model, batch, cap, frames)
    dec.load_weights(dw)
    return dec, dw


def teacher_forced(dec, model, ids, ref_codes, frames, logits_out=True, lengths=None):
    """GPU prefill (ragged when lengths is given) + per-frame CodePredictor (forced) + Talker step
    on the oracle's codes."""
    d = dev()
    B = ids.shape[0]
    Vs, Va = model.talker.vocab, model.codepred.vocab
    sem = torch.zeros((frames, B, Vs), dtype=torch.float32, device=d)
    acl = torch.zeros((frames, B, 15, Va), dtype=torch.float32, device=d)
    own = torch.zeros((frames, B, 15), dtype=torch.int32, device=d)
    codes = torch.from_numpy(np.ascontiguousarray(ref_codes)).to(d)
    rows = [codes[:, t].contiguous() for t in range(frames)]
    sems = [codes[:, t, 0].contiguous() for t in range(frames)]
    forced = [codes[:, t, 1:].contiguous() for t in range(frames)]
    if lengths is None:
        dec.prefill(torch.from_numpy(ids).to(d), sem[0])
    else:
        dec.prefill_ragged(torch.from_numpy(np.ascontiguousarray(ids)).to(d), lengths, sem[0])
    for t in range(frames):
        if t > 0:
            dec.talker_step(rows[t - 1], sem[t])
        dec.codepred_frame(sems[t], GREEDY, None, own[t], forced=forced[t], logits=acl[t])
    torch.cuda.synchronize()
    return (sem.cpu().numpy().transpose(1, 0, 2), acl.cpu().numpy().transpose(1, 0, 2, 3),
            own.cpu().numpy().transpose(1, 0, 2))


def stream_teacher_forced(dec, model, ids, lookahead, ref_codes, frames):
    """Streaming decode on the GPU with the oracle's codes fed forward: prefill of the first
    `lookahead` ids, then every Talker step adds the next text id (-1 once the text is used up)."""
    d = dev()
    B, n = ids.shape
    Vs, Va = model.talker.vocab, model.codepred.vocab
    sem = torch.zeros((frames, B, Vs), dtype=torch.float32, device=d)
    acl = torch.zeros((frames, B, 15, Va), dtype=torch.float32, device=d)
    own = torch.zeros((frames, B, 15), dtype=torch.int32, device=d)
    codes = torch.from_numpy(np.ascontiguousarray(ref_codes)).to(d)
    text = [None] + [torch.from_numpy(ids[:, lookahead + t - 1].astype(np.int32) if lookahead + t - 1 < n
                                      else np.full(B, -1, np.int32)).to(d) for t in range(1, frames)]
    dec.prefill(torch.from_numpy(np.ascontiguousarray(ids[:, :lookahead])).to(d), sem[0])
    for t in range(frames):
        if t > 0:
            dec.talker_step(codes[:, t - 1].contiguous(), sem[t], text_ids=text[t])
        dec.codepred_frame(codes[:, t, 0].contiguous(), GREEDY, None, own[t], forced=codes[:, t, 1:].contiguous(), logits=acl[t])
    torch.cuda.synchronize()
    return (sem.cpu().numpy().transpose(1, 0, 2), acl.cpu().numpy().transpose(1, 0, 2, 3),
            own.cpu().numpy().transpose(1, 0, 2))


def check_step_parity(model, ref, got_sem, got_ac, got_tok, tol):
    e_sem = rowwise_rel_err(got_sem, ref["sem_logits"])
    e_ac = rowwise_rel_err(got_ac, ref["ac_logits"])
    assert e_sem.max() <= tol, f"semantic logits rel err {e_sem.max():.3e} > {tol}"
    assert e_ac.max() <= tol, f"acoustic logits rel err {e_ac.max():.3e} > {tol}"
    n, ex, bad = greedy_agreement(got_tok, ref["ac_logits"], rel=tol if model.weight_dtype == "fp32" else None)
    assert not bad, f"{len(bad)} greedy acoustic mismatches on non-exempt steps (of {n}; {ex} exempt): {bad[:5]}"
    return e_sem.max(), e_ac.max(), n, ex


# ----------------------------------------------------------------------------- tiny fp32 model

@pytest.fixture(scope="module")
def tiny():
    wl = config.WORKLOADS["tiny"]
    w = synth.make_weights(wl.model, wl.weight_seed)
    orc = OracleModel(w, wl.model.as_dict(), np.float64)
    ids = synth.make_text_ids(wl)
    u = synth.make_uniforms(wl)
    ref = orc.generate(ids, wl.frames, GREEDY, GREEDY, u)
    dec, dw = make_decoder(wl.model, 1, wl.prefill_len + wl.frames + 8, wl.frames + 8, w)
    return dict(wl=wl, w=w, orc=orc, ids=ids, u=u, ref=ref, dec=dec, dw=dw)


def test_tiny_teacher_forced_step_parity(tiny):
    wl = tiny["wl"]
    sem, ac, tok = teacher_forced(tiny["dec"], wl.model, tiny["ids"], tiny["ref"]["codes"], wl.frames)
    es, ea, n, ex = check_step_parity(wl.model, tiny["ref"], sem, ac, tok, 1e-4)
    print(f"tiny: sem rel err {es:.2e}, ac rel err {ea:.2e}, greedy checked {n}, exempt {ex}")


def test_tiny_run_frames_greedy_checked_by_the_oracle(tiny):
    wl, dec = tiny["wl"], tiny["dec"]
    d = dev()
    codes = torch.full((1, wl.frames + 8, 16), -1, dtype=torch.int32, device=d)
    dec.prefill(torch.from_numpy(tiny["ids"]).to(d))
    dec.run_frames(wl.frames, GREEDY, GREEDY, None, codes)
    got = codes.cpu().numpy()[:, : wl.frames]
    n, ex = check_free_running(tiny["orc"], tiny["ids"], got, wl.frames, GREEDY, "tiny free-running", rel=1e-4)
    assert dec.progress() == (wl.prefill_len + wl.frames, wl.frames)
    np.testing.assert_array_equal(got, tiny["ref"]["codes"])  # no near tie at all on this input
    print(f"tiny free-running: {n} codes checked, {ex} near ties; equal to the oracle's own free run")


def test_tiny_graph_replay_equals_eager_and_is_deterministic(tiny):
    wl, dec = tiny["wl"], tiny["dec"]
    d = dev()
    F = 6
    ids = torch.from_numpy(tiny["ids"]).to(d)
    u = torch.from_numpy(synth.random_uniforms((1, wl.frames + 8, 16), seed=9)).to(d)
    for sem_cfg, ac_cfg in [(GREEDY, GREEDY), (SEM, AC)]:
        runs = []
        for _ in range(2):
            codes = torch.zeros((1, wl.frames + 8, 16), dtype=torch.int32, device=d)
            dec.prefill(ids)
            dec.run_frames(F, sem_cfg, ac_cfg, u, codes)
            torch.cuda.synchronize()
            runs.append(codes.cpu().numpy()[:, :F])
        np.testing.assert_array_equal(runs[0], runs[1])
        # eager: the same frames through tts_sample / tts_codepred_frame / tts_talker_step
        logits = torch.zeros((1, wl.model.talker.vocab), dtype=torch.float32, device=d)
        hist = torch.zeros((1, wl.model.talker.vocab), dtype=torch.uint8, device=d)
        s = torch.zeros((1,), dtype=torch.int32, device=d)
        a = torch.zeros((1, 15), dtype=torch.int32, device=d)
        eager = np.zeros((1, F, 16), np.int32)
        dec.prefill(ids, logits)
        for t in range(F):
            dec.sample(logits, sem_cfg, u[:, t, 0].contiguous(), s, history=hist)
            dec.codepred_frame(s, ac_cfg, u[:, t, 1:].contiguous(), a)
            row = torch.cat([s.view(1, 1), a], dim=1).contiguous()
            dec.talker_step(row, logits)
            torch.cuda.synchronize()
            eager[:, t] = row.cpu().numpy()
        np.testing.assert_array_equal(eager, runs[0])


def test_tiny_sampled_frames_teacher_forced(tiny):
    """Sampling with the pages' controls, draws compared given the same uniforms."""
    wl, orc, dec = tiny["wl"], tiny["orc"], tiny["dec"]
    d = dev()
    F = wl.frames
    u = synth.random_uniforms((1, F, 16), seed=17)
    ref = orc.generate(tiny["ids"], F, SEM, AC, u, sampler_dtype=np.float32)
    codes = ref["codes"]
    Vs, Va = wl.model.talker.vocab, wl.model.codepred.vocab
    ud = torch.from_numpy(u).to(d)
    logits = torch.zeros((1, Vs), dtype=torch.float32, device=d)
    s = torch.zeros((1,), dtype=torch.int32, device=d)
    own = torch.zeros((1, 15), dtype=torch.int32, device=d)
    acl = torch.zeros((1, 15, Va), dtype=torch.float32, device=d)
    hist_np = np.zeros((1, Vs), bool)
    dec.prefill(torch.from_numpy(tiny["ids"]).to(d), logits)
    checked = exempt = 0
    for t in range(F):
        if t > 0:
            dec.talker_step(torch.from_numpy(codes[:, t - 1]).to(d).contiguous(), logits)
        hist = torch.from_numpy(hist_np.astype(np.uint8)).to(d)
        dec.sample(logits, SEM, ud[:, t, 0].contiguous(), s, history=hist)
        dec.codepred_frame(torch.from_numpy(codes[:, t, 0]).to(d).contiguous(), AC, ud[:, t, 1:].contiguous(), own,
                           forced=torch.from_numpy(codes[:, t, 1:]).to(d).contiguous(), logits=acl)
        torch.cuda.synchronize()
        lg = ref["sem_logits"][0, t]
        if sample_exempt(lg, SEM, float(u[0, t, 0]), hist_np[0], rel=1e-4):
            exempt += 1
        else:
            checked += 1
            assert int(s.item()) == codes[0, t, 0], f"semantic draw differs at frame {t}"
        got_ac = own.cpu().numpy()[0]
        for j in range(15):
            if sample_exempt(ref["ac_logits"][0, t, j], AC, float(u[0, t, 1 + j]), rel=1e-4):
                exempt += 1
            else:
                checked += 1
                assert got_ac[j] == codes[0, t, 1 + j], f"acoustic draw {j + 1} differs at frame {t}"
        hist_np[0, codes[0, t, 0]] = True
    assert checked > MIN_CHECKED * (checked + exempt)
    print(f"tiny sampled: {checked} draws equal, {exempt} exempt")


def test_tiny_split_attention_over_long_context():
    """Positions past one 64-position attention split (ragged last split)."""
    model = config.TINY
    w = synth.make_weights(model, 3)
    orc = OracleModel(w, model.as_dict(), np.float64)
    ids = synth.random_ids(150, model.text_vocab, seed=4)
    F = 5
    ref = orc.generate(ids, F, GREEDY, GREEDY, np.zeros((1, F, 16), np.float32))
    dec, _ = make_decoder(model, 1, 160, 8, w)
    sem, ac, tok = teacher_forced(dec, model, ids, ref["codes"], F)
    check_step_parity(model, ref, sem, ac, tok, 1e-4)


def test_tiny_64_streams_take_64_position_attention_splits():
    """64 streams of 2 KV heads make 128 (stream, head) pairs, so the decode attention runs
    64-position splits; a 150-id prompt spans three of them with a ragged last one, merged by the
    last block to arrive. Every stream must still equal its own oracle run."""
    model = config.TINY
    w = synth.make_weights(model, 5)
    orc = OracleModel(w, model.as_dict(), np.float64)
    B, F = 64, 2
    ids = synth.random_ids(150, model.text_vocab, seed=9, batch=B)
    ref = orc.generate(ids, F, GREEDY, GREEDY, np.zeros((B, F, 16), np.float32))
    dec, _ = make_decoder(model, B, 160, 4, w)
    sem, ac, tok = teacher_forced(dec, model, ids, ref["codes"], F)
    es, ea, n, ex = check_step_parity(model, ref, sem, ac, tok, 1e-4)
    print(f"tiny 64 streams: sem rel err {es:.2e}, ac rel err {ea:.2e}, greedy checked {n}, exempt {ex}")
    dec.close()


def test_0p6b_32_streams_attend_past_128_positions_in_one_block_per_pair():
    """32 streams of 8 KV heads (256 pairs, enough blocks to fill the chip) attend in one block per
    (stream, KV head) over the whole context, with no split and no merge; after a 132-id prompt the
    decode steps attend over 133 and 134 positions. Logits of both frames of every stream within
    the bf16 bar of the oracle. (Splits and their merge: the 64-stream and long-context tests.)"""
    model = config.MODELS["0.6b"]
    w = synth.make_weights(model, 0)
    B, F = 32, 2
    ids = synth.random_ids(132, model.text_vocab, seed=19, batch=B)
    print("0.6b 32 streams: oracle", flush=True)
    orc = OracleModel(w, model.as_dict(), np.float32)
    ref = orc.generate(ids, F, GREEDY, GREEDY, np.zeros((B, F, 16), np.float32))
    del orc
    print("0.6b 32 streams: decoder", flush=True)
    dec, dw = make_decoder(model, B, 136, 4, w)
    sem, ac, tok = teacher_forced(dec, model, ids, ref["codes"], F)
    es, ea, n, ex = check_step_parity(model, ref, sem, ac, tok, 1e-2)
    print(f"0.6b 32 streams: sem rel err {es:.2e}, ac rel err {ea:.2e}, greedy checked {n}, exempt {ex}")
    dec.close()
    del dw
    torch.cuda.empty_cache()


def test_tiny_batched_streams_are_independent():
    """B lockstep streams: each equals its own single-stream run."""
    model = config.TINY
    w = synth.make_weights(model, 0)
    orc = OracleModel(w, model.as_dict(), np.float64)
    B, F = 3, 4
    ids = synth.random_ids(20, model.text_vocab, seed=8, batch=B)
    ref = orc.generate(ids, F, GREEDY, GREEDY, np.zeros((B, F, 16), np.float32))
    dec, _ = make_decoder(model, B, 32, 8, w)
    sem, ac, tok = teacher_forced(dec, model, ids, ref["codes"], F)
    check_step_parity(model, ref, sem, ac, tok, 1e-4)


# ----------------------------------------------------------------------------- sampler

@pytest.mark.parametrize("V", [3072, 2048, 512, 37])
def test_sampler_on_uploaded_logits_matches_oracle(tiny, V):
    dec = tiny["dec"]
    d = dev()
    B = 64
    L = synth.random_logits((B, V), 2.0, seed=V)
    u = synth.random_uniforms((B,), seed=V + 1)
    hist = synth.random_uniforms((B, V), seed=V + 2) < 0.05
    cfgs = [GREEDY, SEM, AC, dict(AC, top_p=0.8), dict(AC, top_k=0), dict(SEM, top_k=7, temperature=0.5)]
    Ld, ud = torch.from_numpy(L).to(d), torch.from_numpy(u).to(d)
    for cfg in cfgs:
        out = torch.zeros((B,), dtype=torch.int32, device=d)
        hd = torch.from_numpy(hist.astype(np.uint8)).to(d)
        dec.sample(Ld, cfg, ud, out, history=hd)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        ex = 0
        for b in range(B):
            want = sample_token(L[b], cfg, float(u[b]), hist[b], dtype=np.float32)
            if got[b] != want:
                assert cfg["do_sample"] and sample_exempt(L[b], cfg, float(u[b]), hist[b], rel=1e-5), (cfg, b, got[b], want)
                ex += 1
        assert ex <= 2
        # the drawn id is marked in the history
        hn = hd.cpu().numpy()
        assert all(hn[b, got[b]] == 1 for b in range(B))


def test_sampler_top_k_ties_keep_the_lowest_ids(tiny):
    """Five equal largest logits at ids 40, 2, 90, 11, 7 with top_k = 3: the kept set is the
    lowest ids {2, 7, 11} (order logit desc, id asc), equally weighted, so uniforms 0.1, 0.5 and
    0.9 draw 2, 7 and 11; with top_k = 1 every draw is id 2. Both equal the oracle's sampler."""
    d = dev()
    V = 300
    row = -5.0 + 0.1 * synth.random_logits((1, V), 1.0, seed=77)[0]
    row[[40, 2, 90, 11, 7]] = 4.0
    L = np.repeat(row[None, :].astype(np.float32), 3, axis=0)
    u = np.array([0.1, 0.5, 0.9], np.float32)
    for k, want in ((3, [2, 7, 11]), (1, [2, 2, 2])):
        cfg = dict(do_sample=True, top_k=k, top_p=1.0, temperature=1.0, repetition_penalty=1.0)
        out = torch.zeros((3,), dtype=torch.int32, device=d)
        tiny["dec"].sample(torch.from_numpy(L).to(d), cfg, torch.from_numpy(u).to(d), out)
        torch.cuda.synchronize()
        got = out.cpu().numpy().tolist()
        assert got == want, (k, got)
        assert got == [sample_token(L[b], cfg, float(u[b]), None, dtype=np.float32) for b in range(3)]


def test_sampler_greedy_ties_pick_the_lowest_id(tiny):
    d = dev()
    L = np.zeros((4, 300), np.float32)
    L[0, [5, 9, 200]] = 3.0
    L[1, :] = -1.0
    L[2, 299] = 1.0
    L[3, [0, 299]] = 2.0
    out = torch.zeros((4,), dtype=torch.int32, device=d)
    tiny["dec"].sample(torch.from_numpy(L).to(d), GREEDY, None, out)
    torch.cuda.synchronize()
    assert out.cpu().numpy().tolist() == [5, 0, 299, 0]


# ----------------------------------------------------------------------------- error paths on a live context

def test_error_paths_leave_the_context_usable(tiny):
    wl = tiny["wl"]
    d = dev()
    dec = tts.TTSDecoder(wl.model, 1, 40, 4)
    codes = torch.zeros((1, 16), dtype=torch.int32, device=d)
    with pytest.raises(tts.TTSError) as e:
        dec.talker_step(codes)
    assert e.value.code == tts.TTS_E_STATE
    with pytest.raises(tts.TTSError) as e:
        dec.prefill(torch.zeros((1, 4), dtype=torch.int32, device=d))
    assert e.value.code == tts.TTS_E_STATE  # no weights yet
    bad = dict(tiny["dw"])
    bad["talker.lm_head"] = bad["talker.lm_head"][:-1].contiguous()
    with pytest.raises(tts.TTSError) as e:
        dec.load_weights(bad)
    assert e.value.code == tts.TTS_E_SHAPE
    missing = {k: v for k, v in tiny["dw"].items() if k != "cp.heads"}
    with pytest.raises(tts.TTSError) as e:
        dec.load_weights(missing)
    assert e.value.code == tts.TTS_E_SHAPE
    dec.load_weights(tiny["dw"])
    with pytest.raises(tts.TTSError) as e:
        dec.prefill(torch.zeros((1, 41), dtype=torch.int32, device=d))
    assert e.value.code == tts.TTS_E_CAPACITY
    with pytest.raises(tts.TTSError) as e:
        dec.prefill(torch.zeros((2, 4), dtype=torch.int32, device=d))
    assert e.value.code == tts.TTS_E_ARG
    dec.prefill(torch.zeros((1, 30), dtype=torch.int32, device=d))
    fr = torch.zeros((1, 4, 16), dtype=torch.int32, device=d)
    with pytest.raises(tts.TTSError) as e:
        dec.run_frames(5, GREEDY, GREEDY, None, fr)
    assert e.value.code == tts.TTS_E_CAPACITY
    with pytest.raises(tts.TTSError) as e:
        dec.run_frames(1, dict(SEM, temperature=0.0), GREEDY, torch.zeros((1, 4, 16), device=d), fr)
    assert e.value.code == tts.TTS_E_ARG
    with pytest.raises(tts.TTSError) as e:
        dec.run_frames(1, SEM, GREEDY, None, fr)
    assert e.value.code == tts.TTS_E_ARG
    dec.run_frames(4, GREEDY, GREEDY, None, fr)
    assert dec.progress() == (34, 4)
    with pytest.raises(tts.TTSError) as e:
        dec.run_frames(1, GREEDY, GREEDY, None, fr)
    assert e.value.code == tts.TTS_E_CAPACITY
    torch.cuda.synchronize()
    assert fr.cpu().numpy().max() < wl.model.codepred.vocab
    dec.reset()
    assert dec.progress() == (0, 0)
    dec.close()


def test_error_paths_of_stop_ragged_and_text_stream(tiny):
    """The stop id, ragged prefill and text stream validate their arguments before anything is
    enqueued, and a rejected call leaves the context usable."""
    wl = tiny["wl"]
    d = dev()
    dec = tts.TTSDecoder(wl.model, 2, 40, 4)
    dec.load_weights(tiny["dw"])
    stop = torch.zeros((2,), dtype=torch.int32, device=d)
    with pytest.raises(tts.TTSError) as e:
        dec.set_stop(wl.model.talker.vocab, stop)
    assert e.value.code == tts.TTS_E_ARG
    with pytest.raises(tts.TTSError) as e:
        dec.set_stop(3, None)
    assert e.value.code == tts.TTS_E_ARG
    ids = torch.zeros((2, 8), dtype=torch.int32, device=d)
    for bad in ([0, 8], [9, 8]):
        with pytest.raises(tts.TTSError) as e:
            dec.prefill_ragged(ids, bad)
        assert e.value.code == tts.TTS_E_SHAPE
    text = torch.zeros((2, 4), dtype=torch.int32, device=d)
    assert dec.lib.tts_set_text_stream(dec.ctx, text.data_ptr(), 0, 0) == tts.TTS_E_ARG  # ids with n_text < 1
    with pytest.raises(tts.TTSError) as e:
        dec.set_text_stream(text, -1)
    assert e.value.code == tts.TTS_E_ARG
    dec.set_stop(3, stop)
    torch.cuda.synchronize()
    assert (stop.cpu().numpy() == -1).all()
    dec.prefill_ragged(ids, [8, 3])
    fr = torch.zeros((2, 4, 16), dtype=torch.int32, device=d)
    dec.run_frames(2, GREEDY, GREEDY, None, fr)
    torch.cuda.synchronize()
    assert dec.progress() == (10, 2)
    dec.set_stop(-1)
    dec.close()


# ----------------------------------------------------------------------------- bf16 models

@pytest.fixture(scope="module", params=["0.6b", "1.7b"])
def bf16_model(request):
    model = config.MODELS[request.param]
    w = synth.make_weights(model, 0)
    return request.param, model, w


@pytest.mark.parametrize("mode", ["persistent", "kernels"])
def test_bf16_teacher_forced_step_parity(bf16_model, mode):
    """Both CodePredictor executions against the oracle: the persistent XCD-split
    kernel (the default at batch 1 with greedy acoustic tokens) and the per-op kernels."""
    name, model, w = bf16_model
    orc = OracleModel(w, model.as_dict(), np.float32)
    ids = synth.random_ids(16, model.text_vocab, seed=1)
    F = 3
    ref = orc.generate(ids, F, GREEDY, GREEDY, np.zeros((1, F, 16), np.float32))
    del orc
    dec, dw = make_decoder(model, 1, 64 + 240, 240, w)
    _, supported = dec.exec_mode()
    assert supported == tts.PERSISTENT_CODEPRED | tts.PERSISTENT_TALKER, f"{name}: both persistent kernels should support this config"
    dec.set_exec_mode(tts.EXEC_PERSISTENT if mode == "persistent" else tts.EXEC_KERNELS)
    assert dec.exec_mode()[0] == (tts.EXEC_PERSISTENT if mode == "persistent" else tts.EXEC_KERNELS)
    print(f"{name} {mode}: running", flush=True)
    sem, ac, tok = teacher_forced(dec, model, ids, ref["codes"], F)
    assert dec.device_status() == 0
    es, ea, n, ex = check_step_parity(model, ref, sem, ac, tok, 1e-2)
    print(f"{name} {mode}: sem rel err {es:.2e}, ac rel err {ea:.2e}, greedy checked {n}, exempt {ex}")
    dec.close()
    del dw
    torch.cuda.empty_cache()


def test_bf16_run_frames_greedy_both_modes_checked_by_the_oracle(bf16_model):
    """The captured frame graph, free-running, with the persistent kernels and with the per-op
    kernels; the oracle, teacher-forced along each run's own codes, must find every non-exempt
    code to be its argmax."""
    name, model, w = bf16_model
    F = 8
    ids = synth.random_ids(16, model.text_vocab, seed=3)
    orc = OracleModel(w, model.as_dict(), np.float32)
    dec, dw = make_decoder(model, 1, 64, F + 4, w)
    d = dev()
    for mode in (tts.EXEC_PERSISTENT, tts.EXEC_KERNELS):
        dec.set_exec_mode(mode)
        codes = torch.full((1, F + 4, 16), -1, dtype=torch.int32, device=d)
        dec.prefill(torch.from_numpy(ids).to(d))
        dec.run_frames(F, GREEDY, GREEDY, None, codes)
        assert dec.device_status() == 0
        got = codes.cpu().numpy()[:, :F]
        n, ex = check_free_running(orc, ids, got, F, GREEDY, f"{name} mode {mode}")
        print(f"{name} mode {mode}: {n} codes checked against the oracle, {ex} near ties", flush=True)
    del orc
    dec.close()
    del dw
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- FP8 (E4M3) weights

@pytest.fixture(scope="module", params=["0.6b-fp8", "1.7b-fp8"])
def fp8_model(request):
    model = config.MODELS[request.param]
    w = synth.make_weights(model, 0)
    return request.param, model, w


@pytest.mark.parametrize("mode", ["persistent", "kernels"])
def test_fp8_teacher_forced_step_parity(fp8_model, mode):
    """Weight-only E4M3 decode against the oracle run on the matrices the codes and row scales
    stand for, on the persistent kernels (the default: the Talker step with E4M3 tiles widened to
    bf16 for the MFMAs, the CodePredictor frame with E4M3 rows in its register buffers, row scales
    applied to each row's sum) and on the per-op kernels; the prompt runs on the MFMA GEMMs. Both
    sides compute in fp32 from the same weights, so the bf16 models' bar applies."""
    name, model, w = fp8_model
    orc = OracleModel(w, model.as_dict(), np.float32)
    ids = synth.random_ids(16, model.text_vocab, seed=1)
    F = 3
    ref = orc.generate(ids, F, GREEDY, GREEDY, np.zeros((1, F, 16), np.float32))
    del orc
    dec, dw = make_decoder(model, 1, 64 + 240, 240, w)
    default, supported = dec.exec_mode()
    assert supported == tts.PERSISTENT_CODEPRED | tts.PERSISTENT_TALKER and default == tts.EXEC_PERSISTENT, \
        "E4M3 weights: both persistent kernels"
    dec.set_exec_mode(tts.EXEC_PERSISTENT if mode == "persistent" else tts.EXEC_KERNELS)
    assert dec.prefill_mode() == tts.PREFILL_GEMM
    print(f"{name} {mode}: running", flush=True)
    sem, ac, tok = teacher_forced(dec, model, ids, ref["codes"], F)
    assert dec.device_status() == 0
    es, ea, n, ex = check_step_parity(model, ref, sem, ac, tok, 1e-2)
    print(f"{name} {mode}: sem rel err {es:.2e}, ac rel err {ea:.2e}, greedy checked {n}, exempt {ex}")
    dec.close()
    del dw
    torch.cuda.empty_cache()


def test_fp8_frame_graph_greedy_checked_by_the_oracle():
    """The captured frame graph on E4M3 weights, free-running: the oracle, teacher-forced along the
    run's own codes, must find every non-exempt code to be its argmax."""
    model = config.MODELS["0.6b-fp8"]
    w = synth.make_weights(model, 0)
    F = 8
    ids = synth.random_ids(16, model.text_vocab, seed=3)
    orc = OracleModel(w, model.as_dict(), np.float32)
    dec, dw = make_decoder(model, 1, 64, F + 4, w)
    d = dev()
    codes = torch.full((1, F + 4, 16), -1, dtype=torch.int32, device=d)
    dec.prefill(torch.from_numpy(ids).to(d))
    dec.run_frames(F, GREEDY, GREEDY, None, codes)
    assert dec.device_status() == 0
    got = codes.cpu().numpy()[:, :F]
    n, ex = check_free_running(orc, ids, got, F, GREEDY, "0.6b-fp8 frame graph")
    del orc
    print(f"0.6b-fp8 frame graph: {n} codes checked against the oracle, {ex} near ties", flush=True)
    dec.close()
    del dw
    torch.cuda.empty_cache()


def test_fp8_batched_streams_take_the_gemm_route():
    """16 lockstep streams of the 0.6B E4M3 model: every projection has 16 or more rows, so the
    decode runs its projections as MFMA GEMMs on the widened codes (split K, row scales at the
    output). Teacher-forced logits of every stream within the bar, greedy tokens equal."""
    model = config.MODELS["0.6b-fp8"]
    w = synth.make_weights(model, 0)
    B, n, F = 16, 8, 2
    ids = synth.random_ids(n, model.text_vocab, seed=21, batch=B)
    orc = OracleModel(w, model.as_dict(), np.float32)
    ref = orc.generate(ids, F, GREEDY, GREEDY, np.zeros((B, F, 16), np.float32))
    del orc
    dec, dw = make_decoder(model, B, n + F + 2, F + 2, w)
    print("0.6b-fp8 x16: running", flush=True)
    sem, ac, tok = teacher_forced(dec, model, ids, ref["codes"], F)
    es, ea, n_, ex = check_step_parity(model, ref, sem, ac, tok, 1e-2)
    print(f"0.6b-fp8 x16: sem rel err {es:.2e}, ac rel err {ea:.2e}, greedy checked {n_}, exempt {ex}")
    dec.close()
    del dw
    torch.cuda.empty_cache()


def test_fp8_load_weights_checks_scales_and_dtypes():
    """An E4M3 context wants every matrix as uint8 with its fp32 '.scale', gains and tables as bf16."""
    model = config.MODELS["0.6b-fp8"]
    w = synth.make_weights(model, 0)
    dw = tts.weights_to_device(w, model, dev())
    dec = tts.TTSDecoder(model, 1, 64, 8)
    missing = dict(dw)
    del missing["talker.layers.3.wo.scale"]
    with pytest.raises(RuntimeError, match="wo.scale"):
        dec.load_weights(missing)
    wrong = dict(dw)
    wrong["talker.layers.0.attn_norm"] = dw["talker.layers.0.attn_norm"].float()
    with pytest.raises(RuntimeError, match="dtype"):
        dec.load_weights(wrong)
    dec.load_weights(dw)
    dec.close()


# ----------------------------------------------------------------------------- streaming text

def test_tiny_streaming_text_teacher_forced_and_frame_graph(tiny):
    """Streaming text conditioning: prefill of 4 of 12 ids, one text row per Talker step, none
    once the text is used up (frames 9..15), eager steps and the captured frame graph."""
    wl, dec = tiny["wl"], tiny["dec"]
    ids = synth.random_ids(12, wl.model.text_vocab, seed=31)
    L, F = 4, wl.frames
    ref = tiny["orc"].generate(ids, F, GREEDY, GREEDY, tiny["u"], text_lookahead=L)
    sem, ac, tok = stream_teacher_forced(dec, wl.model, ids, L, ref["codes"], F)
    es, ea, n, ex = check_step_parity(wl.model, ref, sem, ac, tok, 1e-4)
    print(f"tiny streaming: sem rel err {es:.2e}, ac rel err {ea:.2e}, greedy checked {n}, exempt {ex}", flush=True)
    d = dev()
    text = torch.from_numpy(ids.astype(np.int32)).to(d)
    codes = torch.full((1, F + 8, 16), -1, dtype=torch.int32, device=d)
    dec.set_text_stream(text, L)
    try:
        dec.prefill(torch.from_numpy(np.ascontiguousarray(ids[:, :L])).to(d))
        dec.run_frames(F, GREEDY, GREEDY, None, codes)
        torch.cuda.synchronize()
    finally:
        dec.set_text_stream(None)
    got = codes.cpu().numpy()[:, :F]
    n, ex = check_free_running(tiny["orc"], ids, got, F, GREEDY, "tiny streaming frame graph", rel=1e-4, text_lookahead=L)
    print(f"tiny streaming frame graph: {n} codes checked against the oracle, {ex} near ties")


def test_bf16_streaming_text_teacher_forced_and_frame_graph(bf16_model):
    """Streaming text on the bf16 models with the persistent kernels (the default path): 4 of 6 ids
    in the prefill, text rows on frames 1 and 2, none after; then the frame graph free-running."""
    name, model, w = bf16_model
    ids = synth.random_ids(6, model.text_vocab, seed=32)
    L, F = 4, 4
    orc = OracleModel(w, model.as_dict(), np.float32)
    ref = orc.generate(ids, F, GREEDY, GREEDY, np.zeros((1, F, 16), np.float32), text_lookahead=L)
    dec, dw = make_decoder(model, 1, 64, 16, w)
    assert dec.exec_mode()[0] == tts.EXEC_PERSISTENT
    print(f"{name} streaming: running", flush=True)
    sem, ac, tok = stream_teacher_forced(dec, model, ids, L, ref["codes"], F)
    assert dec.device_status() == 0
    es, ea, n, ex = check_step_parity(model, ref, sem, ac, tok, 1e-2)
    print(f"{name} streaming: sem rel err {es:.2e}, ac rel err {ea:.2e}, greedy checked {n}, exempt {ex}", flush=True)
    d = dev()
    text = torch.from_numpy(ids.astype(np.int32)).to(d)
    codes = torch.full((1, 16, 16), -1, dtype=torch.int32, device=d)
    dec.set_text_stream(text, L)
    dec.prefill(torch.from_numpy(np.ascontiguousarray(ids[:, :L])).to(d))
    dec.run_frames(8, GREEDY, GREEDY, None, codes)
    assert dec.device_status() == 0
    got = codes.cpu().numpy()[:, :8]
    n, ex = check_free_running(orc, ids, got, 8, GREEDY, f"{name} streaming frame graph", text_lookahead=L)
    del orc
    print(f"{name} streaming frame graph: {n} codes checked against the oracle, {ex} near ties")
    dec.close()
    del dw
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- ragged prompts, stop id

def test_tiny_ragged_prompts_teacher_forced():
    """Three streams with prompts of 12, 7 and 1 ids in one lockstep batch: each must decode as the
    oracle's stream decoding alone from position 0."""
    model = config.TINY
    w = synth.make_weights(model, 0)
    orc = OracleModel(w, model.as_dict(), np.float64)
    ids = np.concatenate([synth.random_ids(12, model.text_vocab, seed=s) for s in (51, 52, 53)])
    lengths, F = [12, 7, 1], 6
    u = synth.random_uniforms((3, F, 16), seed=54)
    ref = orc.generate(ids, F, GREEDY, GREEDY, u, lengths=lengths)
    dec, dw = make_decoder(model, 3, 12 + F + 4, F + 4, w)
    sem, ac, tok = teacher_forced(dec, model, ids, ref["codes"], F, lengths=lengths)
    es, ea, n, ex = check_step_parity(model, ref, sem, ac, tok, 1e-4)
    print(f"tiny ragged: sem rel err {es:.2e}, ac rel err {ea:.2e}, greedy checked {n}, exempt {ex}")
    dec.close()


@pytest.mark.parametrize("prefill", ["gemm", "steps"])
def test_0p6b_ragged_prompts_teacher_forced(prefill):
    model = config.MODELS["0.6b"]
    w = synth.make_weights(model, 0)
    ids = np.concatenate([synth.random_ids(16, model.text_vocab, seed=s) for s in (55, 56, 57)])
    lengths, F = [16, 9, 4], 3
    orc = OracleModel(w, model.as_dict(), np.float32)
    ref = orc.generate(ids, F, GREEDY, GREEDY, np.zeros((3, F, 16), np.float32), lengths=lengths)
    del orc
    dec, dw = make_decoder(model, 3, 64, 8, w)
    dec.set_prefill_mode(tts.PREFILL_GEMM if prefill == "gemm" else tts.PREFILL_STEPS)
    print(f"0.6b ragged {prefill}: running", flush=True)
    sem, ac, tok = teacher_forced(dec, model, ids, ref["codes"], F, lengths=lengths)
    es, ea, n, ex = check_step_parity(model, ref, sem, ac, tok, 1e-2)
    print(f"0.6b ragged {prefill}: sem rel err {es:.2e}, ac rel err {ea:.2e}, greedy checked {n}, exempt {ex}")
    dec.close()
    del dw
    torch.cuda.empty_cache()


def test_tiny_stop_id_in_the_frame_graph():
    """Greedy frame graph with a stop id that stream 1 draws at frame 3: stop frames and masked
    codes equal the oracle's, the other streams run on."""
    model = config.TINY
    w = synth.make_weights(model, 0)
    orc = OracleModel(w, model.as_dict(), np.float64)
    ids = np.concatenate([synth.random_ids(10, model.text_vocab, seed=s) for s in (61, 62, 63)])
    F = 10
    u = np.zeros((3, F, 16), np.float32)
    free = orc.generate(ids, F, GREEDY, GREEDY, u)
    eos = int(free["codes"][1, 3, 0])
    ref = orc.generate(ids, F, GREEDY, GREEDY, u, eos_id=eos)
    assert ref["stop"][1] >= 0
    d = dev()
    dec, dw = make_decoder(model, 3, 10 + F + 4, F + 4, w)
    stop = torch.full((dec_max_batch(dec),), 7, dtype=torch.int32, device=d)
    dec.set_stop(eos, stop)
    codes = torch.full((3, F + 4, 16), -7, dtype=torch.int32, device=d)
    dec.prefill(torch.from_numpy(ids).to(d))
    dec.run_frames(F, GREEDY, GREEDY, None, codes)
    torch.cuda.synchronize()
    got = codes.cpu().numpy()[:, :F]
    stops = stop.cpu().numpy()[:3]
    upto = check_stop_masking(got, stops, eos, "tiny stop")
    n, ex = check_free_running(orc, ids, got, F, GREEDY, "tiny stop", rel=1e-4, upto=upto)
    np.testing.assert_array_equal(stops, ref["stop"])  # no near tie on this input: the oracle's stops
    print(f"tiny stop id {eos}: stop frames {stops} (oracle {ref['stop']}), {n} codes checked, {ex} near ties")
    dec.set_stop(-1)
    dec.close()


def test_0p6b_stop_id_with_the_persistent_kernels():
    """The stop id through the frame graph on the persistent kernels: the id is the semantic token
    the same run draws at frame 4 without a stop, so the stop fires (at its first draw); the codes
    up to it are checked by the oracle teacher-forced along them."""
    model = config.MODELS["0.6b"]
    w = synth.make_weights(model, 0)
    ids = synth.random_ids(12, model.text_vocab, seed=64)
    F = 8
    d = dev()
    dec, dw = make_decoder(model, 1, 64, 16, w)
    assert dec.exec_mode()[0] == tts.EXEC_PERSISTENT
    free = torch.full((1, 16, 16), -7, dtype=torch.int32, device=d)
    dec.prefill(torch.from_numpy(ids).to(d))
    dec.run_frames(F, GREEDY, GREEDY, None, free)
    eos = int(free.cpu().numpy()[0, 4, 0])
    stop = torch.full((dec_max_batch(dec),), 7, dtype=torch.int32, device=d)
    dec.set_stop(eos, stop)
    codes = torch.full((1, 16, 16), -7, dtype=torch.int32, device=d)
    dec.prefill(torch.from_numpy(ids).to(d))
    dec.run_frames(F, GREEDY, GREEDY, None, codes)
    assert dec.device_status() == 0
    got = codes.cpu().numpy()[:, :F]
    stops = stop.cpu().numpy()[:1]
    upto = check_stop_masking(got, stops, eos, "0.6b stop")
    first = int(np.nonzero(free.cpu().numpy()[0, :F, 0] == eos)[0][0])
    assert int(stops[0]) == first, f"stop at {int(stops[0])}, the free run first draws {eos} at {first}"
    np.testing.assert_array_equal(got[0, :first], free.cpu().numpy()[0, :first])
    orc = OracleModel(w, model.as_dict(), np.float32)
    n, ex = check_free_running(orc, ids, got, F, GREEDY, "0.6b stop", upto=upto)
    del orc
    print(f"0.6b stop id {eos}: stop frame {int(stops[0])}, {n} codes checked against the oracle, {ex} near ties")
    dec.close()
    del dw
    torch.cuda.empty_cache()


def dec_max_batch(dec):
    return dec.max_batch


def test_1p7b_long_context_logits_at_2255_positions():
    """Full long-utterance length: 2255 positions through the split attention.
    The oracle computes the last position by the cache-free whole-sequence pass."""
    model = config.M17B
    w = synth.make_weights(model, 0)
    n = 2255
    print("long context: weights ready", flush=True)
    ids = synth.random_ids(n, model.text_vocab, seed=5)
    dec, dw = make_decoder(model, 1, n + 1, 4, w)
    d = dev()
    got = torch.zeros((1, model.talker.vocab), dtype=torch.float32, device=d)
    dec.prefill(torch.from_numpy(ids).to(d), got)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    dec.close()
    del dw
    torch.cuda.empty_cache()
    print("long context: GPU prefill done; oracle whole-sequence pass", flush=True)
    orc = OracleModel(w, model.as_dict(), np.float32)
    X = orc.embed_text[ids[0]][None]
    hT = orc.full_forward("talker", X)[:, -1]
    ref = linear(hT, orc.lm_head)
    err = rowwise_rel_err(got, ref).max()
    assert err <= 1e-2, err
    if top2_margin(ref[0]) > 0.05:
        assert int(np.argmax(got[0])) == int(np.argmax(ref[0]))
    print(f"1.7b at 2255 positions: rel err {err:.2e}")


def test_1p7b_persistent_talker_step_at_2255_positions():
    """The persistent Talker step at the full long-utterance length: position 2254 after a 2254-id
    prefill, fed one frame of codes, so its attention splits 2255 positions over the 32 ranks of
    each XCD. The oracle runs the whole sequence (text rows, then the frame's code-embedding sum)
    through its cache-free pass."""
    model = config.M17B
    w = synth.make_weights(model, 0)
    n = 2254
    ids = synth.random_ids(n, model.text_vocab, seed=6)
    codes = np.concatenate([synth.random_ids(1, model.talker.vocab, seed=7),
                            synth.random_ids(15, model.codepred.vocab, seed=8)], axis=1)
    print("persistent talker long context: weights ready", flush=True)
    dec, dw = make_decoder(model, 1, n + 2, 4, w)
    assert dec.exec_mode() == (tts.EXEC_PERSISTENT, tts.PERSISTENT_CODEPRED | tts.PERSISTENT_TALKER)
    d = dev()
    got = torch.zeros((1, model.talker.vocab), dtype=torch.float32, device=d)
    dec.prefill(torch.from_numpy(ids).to(d))
    dec.talker_step(torch.from_numpy(codes).to(d), got)
    torch.cuda.synchronize()
    assert dec.device_status() == 0
    assert dec.progress() == (n + 1, 0)
    got = got.cpu().numpy()
    dec.close()
    del dw
    torch.cuda.empty_cache()
    print("persistent talker long context: GPU step done; oracle whole-sequence pass", flush=True)
    orc = OracleModel(w, model.as_dict(), np.float32)
    X = np.concatenate([orc.embed_text[ids[0]], orc.embed_sum(codes)], axis=0)[None]
    ref = linear(orc.full_forward("talker", X)[:, -1], orc.lm_head)
    err = rowwise_rel_err(got, ref).max()
    assert err <= 1e-2, err
    if top2_margin(ref[0]) > 0.05:
        assert int(np.argmax(got[0])) == int(np.argmax(ref[0]))
    print(f"1.7b persistent talker step at position 2254: rel err {err:.2e}")


def test_1p7b_x32_sampled_streams_teacher_forced():
    """The 32-stream 1.7B configuration with the pages' sampling controls: 32 independent lockstep
    streams (semantic: top-k 50, T 0.9, repetition penalty 1.05; acoustic: the same without the
    penalty), each with its own ids, history and uniforms. Logits of every stream and step within
    the bf16 bar; every non-exempt draw equal to the oracle's given the same uniforms. The prefill is
    shortened to 8 ids so the fp32 oracle runs 32 streams in seconds."""
    model = config.M17B
    w = synth.make_weights(model, 0)
    B, n, F = 32, 8, 2
    ids = synth.random_ids(n, model.text_vocab, seed=9, batch=B)
    u = synth.random_uniforms((B, F, 16), seed=10)
    orc = OracleModel(w, model.as_dict(), np.float32)
    print("x32: oracle run", flush=True)
    ref = orc.generate(ids, F, SEM, AC, u, sampler_dtype=np.float32)
    del orc
    codes = ref["codes"]
    Vs, Va = model.talker.vocab, model.codepred.vocab
    dec, dw = make_decoder(model, B, n + F + 2, F + 2, w)
    d = dev()
    ud = torch.from_numpy(u).to(d)
    logits = torch.zeros((B, Vs), dtype=torch.float32, device=d)
    s = torch.zeros((B,), dtype=torch.int32, device=d)
    own = torch.zeros((B, 15), dtype=torch.int32, device=d)
    acl = torch.zeros((B, 15, Va), dtype=torch.float32, device=d)
    hist_np = np.zeros((B, Vs), bool)
    dec.prefill(torch.from_numpy(ids).to(d), logits)
    checked = exempt = 0
    worst = 0.0
    for t in range(F):
        if t > 0:
            dec.talker_step(torch.from_numpy(codes[:, t - 1]).to(d).contiguous(), logits)
        hist = torch.from_numpy(hist_np.astype(np.uint8)).to(d)
        dec.sample(logits, SEM, ud[:, t, 0].contiguous(), s, history=hist)
        dec.codepred_frame(torch.from_numpy(codes[:, t, 0]).to(d).contiguous(), AC, ud[:, t, 1:].contiguous(), own,
                           forced=torch.from_numpy(codes[:, t, 1:]).to(d).contiguous(), logits=acl)
        torch.cuda.synchronize()
        sl, al = logits.cpu().numpy(), acl.cpu().numpy()
        e_s = rowwise_rel_err(sl, ref["sem_logits"][:, t]).max()
        e_a = rowwise_rel_err(al, ref["ac_logits"][:, t]).max()
        assert e_s <= 1e-2 and e_a <= 1e-2, f"frame {t}: logits rel err {e_s:.2e} / {e_a:.2e}"
        worst = max(worst, e_s, e_a)
        got_s, got_a = s.cpu().numpy(), own.cpu().numpy()
        for b in range(B):
            if sample_exempt(ref["sem_logits"][b, t], SEM, float(u[b, t, 0]), hist_np[b], rel=1e-4):
                exempt += 1
            else:
                checked += 1
                assert got_s[b] == codes[b, t, 0], f"semantic draw differs: stream {b} frame {t}"
            for j in range(15):
                if sample_exempt(ref["ac_logits"][b, t, j], AC, float(u[b, t, 1 + j]), rel=1e-4):
                    exempt += 1
                else:
                    checked += 1
                    assert got_a[b, j] == codes[b, t, 1 + j], f"acoustic draw {j + 1} differs: stream {b} frame {t}"
            hist_np[b, codes[b, t, 0]] = True
    dec.close()
    del dw
    torch.cuda.empty_cache()
    assert checked > MIN_CHECKED * (checked + exempt)
    print(f"1.7b x32 sampled: logits rel err <= {worst:.2e}; {checked} draws equal, {exempt} exempt")


@pytest.mark.parametrize("name,B", [("0.6b", 2), ("1.7b", 2), ("0.6b-fp8", 2), ("1.7b", 1), ("1.7b-fp8", 1)])
def test_gemm_prefill_matches_step_prefill_and_oracle(name, B):
    """The prompt pass as MFMA GEMMs (chunks of 64 positions, a ragged last chunk) against the
    one-position-at-a-time path and the oracle: logits after the prompt and after one Talker step on
    the same codes (which reads the KV cache both prefills wrote). 2 streams: chunks of 128 and 72
    rows (row tiles); 1 stream: chunks of 64 and 36 rows (the split-K route of few rows)."""
    model = config.MODELS[name]
    w = synth.make_weights(model, 0)
    n = 100
    ids = synth.random_ids(n, model.text_vocab, seed=11, batch=B)
    codes = np.concatenate([synth.random_ids(1, model.talker.vocab, seed=12, batch=B),
                            synth.random_ids(15, model.codepred.vocab, seed=13, batch=B)], axis=1)
    dec, dw = make_decoder(model, B, n + 4, 4, w)
    d = dev()
    got = {}
    for mode in (tts.PREFILL_GEMM, tts.PREFILL_STEPS):
        dec.set_prefill_mode(mode)
        assert dec.prefill_mode() == mode
        l0 = torch.zeros((B, model.talker.vocab), dtype=torch.float32, device=d)
        l1 = torch.zeros_like(l0)
        dec.prefill(torch.from_numpy(ids).to(d), l0)
        dec.talker_step(torch.from_numpy(codes).to(d), l1)
        torch.cuda.synchronize()
        got[mode] = (l0.cpu().numpy(), l1.cpu().numpy())
    dec.close()
    del dw
    torch.cuda.empty_cache()
    orc = OracleModel(w, model.as_dict(), np.float32)
    X = np.concatenate([orc.embed_text[ids], orc.embed_sum(codes)[:, None]], axis=1)  # [B, n + 1, Ht]
    hs = orc.full_forward("talker", X)
    ref0, ref1 = linear(hs[:, n - 1], orc.lm_head), linear(hs[:, n], orc.lm_head)
    for mode, (g0, g1) in got.items():
        e0, e1 = rowwise_rel_err(g0, ref0).max(), rowwise_rel_err(g1, ref1).max()
        assert e0 <= 1e-2 and e1 <= 1e-2, (mode, e0, e1)
        for g, r in ((g0, ref0), (g1, ref1)):
            n_, ex, bad = greedy_agreement(np.argmax(g, axis=-1), r)
            assert not bad, (mode, bad)
        print(f"{name} x{B} prefill mode {mode}: rel err after prompt {e0:.2e}, after one step {e1:.2e}")
    e = rowwise_rel_err(got[tts.PREFILL_GEMM][1], got[tts.PREFILL_STEPS][1]).max()
    print(f"{name} x{B}: GEMM vs step prefill, step logits rel diff {e:.2e}")


# ----------------------------------------------------------------------------- reproducibility

def _bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


@pytest.mark.parametrize("name", ["1.7b", "1.7b-fp8"])
def test_1p7b_persistent_decode_is_bitwise_reproducible(name):
    """Two runs of the same 1.7B batch-1 work give identical bits, with bf16 and with E4M3 weights:
    the MFMA prompt pass, eight frames of the captured graph on both persistent kernels, then an
    eager CodePredictor frame and Talker step (every sum has a fixed order; split-K partials are
    added in slice order)."""
    model = config.MODELS[name]
    w = synth.make_weights(model, 0)
    dec, dw = make_decoder(model, 1, 64, 16, w)
    assert dec.exec_mode()[0] == tts.EXEC_PERSISTENT and dec.prefill_mode() == tts.PREFILL_GEMM
    d = dev()
    ids = torch.from_numpy(synth.random_ids(16, model.text_vocab, seed=5)).to(d)
    Vs, Va = model.talker.vocab, model.codepred.vocab
    runs = []
    for _ in range(2):
        l0 = torch.zeros((1, Vs), dtype=torch.float32, device=d)
        codes = torch.full((1, 16, 16), -1, dtype=torch.int32, device=d)
        al = torch.zeros((1, 15, Va), dtype=torch.float32, device=d)
        a = torch.zeros((1, 15), dtype=torch.int32, device=d)
        sl = torch.zeros((1, Vs), dtype=torch.float32, device=d)
        dec.prefill(ids, l0)
        dec.run_frames(8, GREEDY, GREEDY, None, codes)
        s = codes[:, 7, 0].contiguous()
        dec.codepred_frame(s, GREEDY, None, a, logits=al)
        dec.talker_step(torch.cat([s.view(1, 1), a], dim=1).contiguous(), sl)
        torch.cuda.synchronize()
        assert dec.device_status() == 0
        runs.append([x.cpu().numpy() for x in (l0, codes, al, a, sl)])
    for name, x, y in zip(("prompt logits", "codes", "acoustic logits", "acoustic codes", "semantic logits"), *runs):
        np.testing.assert_array_equal(_bits(x), _bits(y), err_msg=name)
    dec.close()
    del dw
    torch.cuda.empty_cache()


def test_0p6b_persistent_frame_graph_equals_eager_bitwise():
    """The captured frame graph on the persistent kernels and the same frames issued eagerly
    (tts_sample, tts_codepred_frame, tts_talker_step) give identical codes and identical logits
    after them."""
    model = config.MODELS["0.6b"]
    w = synth.make_weights(model, 0)
    dec, dw = make_decoder(model, 1, 64, 16, w)
    assert dec.exec_mode()[0] == tts.EXEC_PERSISTENT
    d = dev()
    F = 5
    ids = torch.from_numpy(synth.random_ids(16, model.text_vocab, seed=6)).to(d)
    Vs, Va = model.talker.vocab, model.codepred.vocab
    probe = torch.full((1,), 7, dtype=torch.int32, device=d)
    a = torch.zeros((1, 15), dtype=torch.int32, device=d)
    # graph
    codes = torch.full((1, 16, 16), -1, dtype=torch.int32, device=d)
    alg = torch.zeros((1, 15, Va), dtype=torch.float32, device=d)
    dec.prefill(ids)
    dec.run_frames(F, GREEDY, GREEDY, None, codes)
    dec.codepred_frame(probe, GREEDY, None, a, logits=alg)
    torch.cuda.synchronize()
    # eager
    logits = torch.zeros((1, Vs), dtype=torch.float32, device=d)
    s = torch.zeros((1,), dtype=torch.int32, device=d)
    eager = np.zeros((1, F, 16), np.int32)
    dec.prefill(ids, logits)
    for t in range(F):
        dec.sample(logits, GREEDY, None, s)
        dec.codepred_frame(s, GREEDY, None, a)
        row = torch.cat([s.view(1, 1), a], dim=1).contiguous()
        dec.talker_step(row, logits)
        torch.cuda.synchronize()
        eager[:, t] = row.cpu().numpy()
    ale = torch.zeros((1, 15, Va), dtype=torch.float32, device=d)
    dec.codepred_frame(probe, GREEDY, None, a, logits=ale)
    torch.cuda.synchronize()
    assert dec.device_status() == 0
    np.testing.assert_array_equal(codes.cpu().numpy()[:, :F], eager)
    np.testing.assert_array_equal(_bits(alg.cpu().numpy()), _bits(ale.cpu().numpy()))
    dec.close()
    del dw
    torch.cuda.empty_cache()


def test_1p7b_x32_sampled_runs_are_reproducible():
    """32 sampled 1.7B streams (the batched decode: split-K MFMA GEMMs whose K slices are added in
    slice order, the radix-select sampler): two runs give identical codes and identical logits."""
    model = config.MODELS["1.7b"]
    w = synth.make_weights(model, 0)
    B, n, F = 32, 8, 3
    ids = torch.from_numpy(synth.random_ids(n, model.text_vocab, seed=21, batch=B)).to(dev())
    u = torch.from_numpy(synth.random_uniforms((B, F + 2, 16), seed=22)).to(dev())
    dec, dw = make_decoder(model, B, n + F + 4, F + 2, w)
    d = dev()
    Va = model.codepred.vocab
    runs = []
    for _ in range(2):
        codes = torch.full((B, F + 2, 16), -1, dtype=torch.int32, device=d)
        al = torch.zeros((B, 15, Va), dtype=torch.float32, device=d)
        a = torch.zeros((B, 15), dtype=torch.int32, device=d)
        dec.prefill(ids)
        dec.run_frames(F, SEM, AC, u, codes)
        dec.codepred_frame(codes[:, F - 1, 0].contiguous(), AC, u[:, F, 1:].contiguous(), a, logits=al)
        torch.cuda.synchronize()
        runs.append([x.cpu().numpy() for x in (codes, al, a)])
    for name, x, y in zip(("codes", "acoustic logits", "acoustic codes"), *runs):
        np.testing.assert_array_equal(_bits(x), _bits(y), err_msg=name)
    dec.close()
    del dw
    torch.cuda.empty_cache()
