"""Sampled acoustic tokens inside the persistent CodePredictor kernel ("qwen3-tts-hip" README,
section "Library Usage": the subtalker sampling controls top_k, top_p and temperature, on by
default). At batch 1 with top_k in 1..64 the kernel draws each acoustic id itself (the 2048 logits
gathered by every workgroup, a radix select for top-k, top-p and the inverse CDF in one wave);
other top_k values take the per-op sampler.

Three kinds of check:
  * the draw against the oracle's sampler applied to the kernel's own logits (float32 decision):
    equal wherever the draw is not within 1e-6 of a CDF step (rounding of exp and of the running
    sum); ties of equal logits at the top-k cut are not exempt, so rows of a head made identical
    check that the lowest ids are kept;
  * logits and draws against the oracle model, teacher-forced (logits within the bf16 bar, draws
    equal wherever the oracle's draw is not within 1e-4 of a boundary or of a near tie in the kept
    order, see parity_util.sample_exempt);
  * a free-running sampled frame graph checked by the oracle along its own codes, and run twice
    with equal codes.
"""
import numpy as np
import pytest
import torch

from autoregressive_tts_decode_amd import config, synth, tts
from oracle.decoder import OracleModel
from oracle.sampler import sample_token
from parity_util import MIN_CHECKED, rowwise_rel_err, sample_exempt

pytestmark = pytest.mark.gpu
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


def near_cdf_step(logits_row, cfg, u, rel=1e-6):
    """True when u * sum lies within rel * sum of a running sum of the oracle's draw."""
    _, det = sample_token(np.asarray(logits_row, np.float32), cfg, u, None, dtype=np.float32, return_detail=True)
    cum = det["cum"].astype(np.float64)
    return bool(np.min(np.abs(cum - float(det["target"]))) < rel * cum[-1])


def check_draws_on_own_logits(logits, draws, cfg, u, what):
    """Each of the 15 draws against the oracle sampler on the same logits; returns (equal, exempt)."""
    eq = ex = 0
    for j in range(15):
        if near_cdf_step(logits[j], cfg, float(u[j])):
            ex += 1
            continue
        want = sample_token(np.asarray(logits[j], np.float32), cfg, float(u[j]), None, dtype=np.float32)
        assert draws[j] == want, f"{what}: acoustic draw {j + 1} is {draws[j]}, the oracle sampler draws {want}"
        eq += 1
    return eq, ex


def tied_heads(w, model):
    """Head 1 (acoustic 1): every row equal to row 0, so all 2048 logits tie. Head 2: row r equal
    to row r % 30, so each of 30 values ties about 68 ids and the top-k cut falls inside a tie."""
    w = dict(w)
    h = np.array(w["cp.heads"], copy=True)
    h[0] = h[0, 0][None, :]
    h[1] = h[1, np.arange(h.shape[1]) % 30]
    w["cp.heads"] = h
    if "cp.heads.scale" in w:
        s = np.array(w["cp.heads.scale"], copy=True)
        s[0] = s[0, 0]
        s[1] = s[1, np.arange(s.shape[1]) % 30]
        w["cp.heads.scale"] = s
    return w


CFGS = [
    ("pages' acoustic default", AC),
    ("k 64, T 0.7, top-p 0.8", dict(AC, top_k=64, temperature=0.7, top_p=0.8)),
    ("k 1", dict(AC, top_k=1)),
    ("k 7, T 1.3, top-p 0.5", dict(AC, top_k=7, temperature=1.3, top_p=0.5)),
    ("k 100 (per-op sampler)", dict(AC, top_k=100)),
    ("k 0 = all ids (per-op sampler)", dict(AC, top_k=0, temperature=1.1)),
]


@pytest.mark.parametrize("name", ["0.6b", "0.6b-fp8"])
def test_in_kernel_sampler_matches_the_oracle_sampler_on_its_own_logits(name):
    model = config.MODELS[name]
    w = tied_heads(synth.make_weights(model, 0), model)
    dec, dw = make_decoder(model, 1, 64, 8, w)
    assert dec.exec_mode()[0] == tts.EXEC_PERSISTENT
    d = dev()
    Va = model.codepred.vocab
    ids = torch.from_numpy(synth.random_ids(16, model.text_vocab, seed=21)).to(d)
    forced = torch.from_numpy(synth.random_ids(15, Va, seed=22)).to(d).view(1, 15).contiguous()
    sem = torch.tensor([5], dtype=torch.int32, device=d)
    dec.prefill(ids)
    total_eq = total_ex = 0
    for c, (label, cfg) in enumerate(CFGS):
        for rep in range(2):
            u_np = synth.random_uniforms((1, 15), seed=100 + 10 * c + rep)
            u = torch.from_numpy(u_np).to(d)
            own = torch.full((1, 15), -1, dtype=torch.int32, device=d)
            acl = torch.zeros((1, 15, Va), dtype=torch.float32, device=d)
            print(f"{name} {label} rep {rep}", flush=True)
            dec.codepred_frame(sem, cfg, u, own, forced=forced, logits=acl)
            torch.cuda.synchronize()
            assert dec.device_status() == 0
            lg = acl.cpu().numpy()[0]
            if rep == 0 and c == 0:
                assert np.all(lg[0] == lg[0, 0]), "identical head rows must give identical logits"
                assert np.sum(lg[1] == lg[1].max()) >= 60, "the top-k cut of head 2 must fall inside a tie"
            eq, ex = check_draws_on_own_logits(lg, own.cpu().numpy()[0], cfg, u_np[0], f"{name} {label} rep {rep}")
            total_eq += eq
            total_ex += ex
            if cfg["top_k"] == 1:
                np.testing.assert_array_equal(own.cpu().numpy()[0], np.argmax(lg, axis=-1))
    assert total_eq > 0.9 * (total_eq + total_ex)
    print(f"{name}: {total_eq} draws equal to the oracle sampler on the kernel's logits, {total_ex} at a CDF step")
    dec.close()
    del dw
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["1.7b", "1.7b-fp8"])
def test_sampled_codepred_teacher_forced_against_the_oracle(name):
    model = config.MODELS[name]
    w = synth.make_weights(model, 0)
    orc = OracleModel(w, model.as_dict(), np.float32)
    ids = synth.random_ids(16, model.text_vocab, seed=31)
    F = 3
    u = synth.random_uniforms((1, F, 16), seed=32)
    print(f"{name}: oracle run", flush=True)
    ref = orc.generate(ids, F, SEM, AC, u, sampler_dtype=np.float32)
    del orc
    codes = ref["codes"]
    dec, dw = make_decoder(model, 1, 64, 8, w)
    assert dec.exec_mode()[0] == tts.EXEC_PERSISTENT
    d = dev()
    Vs, Va = model.talker.vocab, model.codepred.vocab
    ud = torch.from_numpy(u).to(d)
    logits = torch.zeros((1, Vs), dtype=torch.float32, device=d)
    own = torch.zeros((1, 15), dtype=torch.int32, device=d)
    acl = torch.zeros((1, 15, Va), dtype=torch.float32, device=d)
    dec.prefill(torch.from_numpy(ids).to(d), logits)
    checked = exempt = own_eq = 0
    worst = 0.0
    for t in range(F):
        if t > 0:
            dec.talker_step(torch.from_numpy(codes[:, t - 1]).to(d).contiguous(), logits)
        print(f"{name}: frame {t}", flush=True)
        dec.codepred_frame(torch.from_numpy(codes[:, t, 0]).to(d).contiguous(), AC, ud[:, t, 1:].contiguous(), own,
                           forced=torch.from_numpy(codes[:, t, 1:]).to(d).contiguous(), logits=acl)
        torch.cuda.synchronize()
        assert dec.device_status() == 0
        al = acl.cpu().numpy()[0]
        e = rowwise_rel_err(al, ref["ac_logits"][0, t]).max()
        assert e <= 1e-2, f"frame {t}: acoustic logits rel err {e:.2e}"
        worst = max(worst, e)
        got = own.cpu().numpy()[0]
        own_eq += check_draws_on_own_logits(al, got, AC, u[0, t, 1:], f"{name} frame {t}")[0]
        for j in range(15):
            if sample_exempt(ref["ac_logits"][0, t, j], AC, float(u[0, t, 1 + j]), rel=1e-4):
                exempt += 1
            else:
                checked += 1
                assert got[j] == codes[0, t, 1 + j], f"frame {t}: acoustic draw {j + 1} differs from the oracle's"
    assert checked > MIN_CHECKED * (checked + exempt)
    print(f"{name}: logits rel err <= {worst:.2e}; {checked} draws equal to the oracle's, {exempt} exempt; "
          f"{own_eq} equal to the oracle sampler on the kernel's logits")
    dec.close()
    del dw
    torch.cuda.empty_cache()


def test_sampled_frame_graph_checked_by_the_oracle_and_reproducible():
    """The pages' default decode (semantic and acoustic tokens sampled) as a captured frame graph
    with both persistent kernels: the oracle, teacher-forced along the run's own codes, draws the
    same token at every non-exempt step; a second run gives the same codes bit for bit."""
    model = config.M17B
    w = synth.make_weights(model, 0)
    F = 6
    ids = synth.random_ids(16, model.text_vocab, seed=41)
    u = synth.random_uniforms((1, F + 2, 16), seed=42)
    dec, dw = make_decoder(model, 1, 64, F + 2, w)
    assert dec.exec_mode()[0] == tts.EXEC_PERSISTENT
    d = dev()
    ud = torch.from_numpy(u).to(d)
    runs = []
    for rep in range(2):
        print(f"1.7b sampled frame graph: run {rep}", flush=True)
        codes = torch.full((1, F + 2, 16), -1, dtype=torch.int32, device=d)
        dec.prefill(torch.from_numpy(ids).to(d))
        dec.run_frames(F, SEM, AC, ud, codes)
        torch.cuda.synchronize()
        assert dec.device_status() == 0
        runs.append(codes.cpu().numpy()[:, :F])
    np.testing.assert_array_equal(runs[0], runs[1])
    dec.close()
    del dw
    torch.cuda.empty_cache()
    got = runs[0]
    print("1.7b sampled frame graph: oracle along the run's codes", flush=True)
    orc = OracleModel(w, model.as_dict(), np.float32)
    ref = orc.generate(ids, F, SEM, AC, u, teacher=got, sampler_dtype=np.float32)
    del orc
    hist = np.zeros(model.talker.vocab, bool)
    checked = exempt = 0
    for t in range(F):
        if sample_exempt(ref["sem_logits"][0, t], SEM, float(u[0, t, 0]), hist, rel=1e-4):
            exempt += 1
        else:
            checked += 1
            assert got[0, t, 0] == ref["codes"][0, t, 0], f"frame {t}: semantic draw differs from the oracle's"
        for j in range(15):
            if sample_exempt(ref["ac_logits"][0, t, j], AC, float(u[0, t, 1 + j]), rel=1e-4):
                exempt += 1
            else:
                checked += 1
                assert got[0, t, 1 + j] == ref["codes"][0, t, 1 + j], f"frame {t}: acoustic draw {j + 1} differs"
        hist[got[0, t, 0]] = True
    assert checked > MIN_CHECKED * (checked + exempt)
    print(f"1.7b sampled frame graph: {checked} draws equal to the oracle's, {exempt} exempt; two runs equal")
