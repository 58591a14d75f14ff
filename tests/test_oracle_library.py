"""Pins of the oracles against independent implementations of the same model
in a library (transformers' Qwen3-ASR audio encoder, multimodal projector and
feature extractor, and its Qwen3 text model), run in float64 on the CPU with
the same random weights.  The library is not the pages: it is evidence that
the readings the oracle takes where the pages are open (tail chunks zero-padded
to 100 frames before the stem, windows of 104 tokens per clip, LayerNorm eps
1e-5, erf GELU, PE restarting per chunk, proj1 d -> d, RMSNorm eps 1e-6,
rotate-half RoPE) are the ones an independent implementation of the same
checkpoint takes, and it catches arithmetic slips that composing pinned parts
could miss.  The oracles do not import it; only these tests do."""
import numpy as np
import pytest

import oracle as O
import oracle.thinker as TH
import synth
import synth.thinker as ST

tr = pytest.importorskip("transformers")
torch = pytest.importorskip("torch")


def _t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def _encoder_pair(dims, W):
    """The library's encoder and projector with the oracle's weights."""
    from transformers.models.qwen3_asr.configuration_qwen3_asr import Qwen3ASRConfig, Qwen3ASREncoderConfig
    from transformers.models.qwen3_asr.modeling_qwen3_asr import Qwen3ASREncoder, Qwen3ASRMultiModalProjector
    ec = Qwen3ASREncoderConfig(num_mel_bins=128, encoder_layers=dims.n_layers, encoder_attention_heads=dims.n_heads,
                               encoder_ffn_dim=dims.ffn_dim, d_model=dims.d_model, output_dim=dims.output_dim,
                               downsample_hidden_size=dims.conv_channels, n_window=50,
                               n_window_infer=100 * dims.window_chunks)
    ec._attn_implementation = "eager"
    enc = Qwen3ASREncoder(ec).double().eval()
    proj = Qwen3ASRMultiModalProjector(Qwen3ASRConfig(audio_config=ec.to_dict())).double().eval()
    sd = {"conv2d1.weight": W["conv1_w"], "conv2d1.bias": W["conv1_b"], "conv2d2.weight": W["conv2_w"],
          "conv2d2.bias": W["conv2_b"], "conv2d3.weight": W["conv3_w"], "conv2d3.bias": W["conv3_b"],
          "conv_out.weight": W["conv_out_w"], "ln_post.weight": W["post_ln_w"], "ln_post.bias": W["post_ln_b"]}
    names = {"ln1": "self_attn_layer_norm", "q": "self_attn.q_proj", "k": "self_attn.k_proj",
             "v": "self_attn.v_proj", "o": "self_attn.out_proj", "ln2": "final_layer_norm", "fc1": "fc1", "fc2": "fc2"}
    for l in range(dims.n_layers):
        for ours, theirs in names.items():
            sd[f"layers.{l}.{theirs}.weight"] = W[f"layers.{l}.{ours}_w"]
            sd[f"layers.{l}.{theirs}.bias"] = W[f"layers.{l}.{ours}_b"]
    missing, unexpected = enc.load_state_dict({k: _t(v) for k, v in sd.items()}, strict=False)
    assert not unexpected and all("positional" in m for m in missing), (missing, unexpected)
    proj.load_state_dict({"linear_1.weight": _t(W["proj1_w"]), "linear_1.bias": _t(W["proj1_b"]),
                          "linear_2.weight": _t(W["proj2_w"]), "linear_2.bias": _t(W["proj2_b"])})
    return enc, proj


def _library_encode(enc, proj, mels):
    """Packed batch through the library: log-mel [128, F_i] per clip, time
    axis zero-padded to a common multiple of 100 frames with a frame mask."""
    T = max(m.shape[1] for m in mels)
    T = (T + 99) // 100 * 100
    feats = np.zeros((len(mels), 128, T))
    mask = np.zeros((len(mels), T), dtype=np.int64)
    for i, m in enumerate(mels):
        feats[i, :, :m.shape[1]] = m
        mask[i, :m.shape[1]] = 1
    with torch.no_grad():
        h = enc(input_features=_t(feats), input_features_mask=torch.from_numpy(mask)).last_hidden_state
        return proj(h).numpy()


@pytest.mark.parametrize("window_chunks", [8, 2])
def test_encoder_matches_transformers_qwen3_asr(window_chunks):
    """Whole encoder forward from the normalised log-mel to the projected
    output, packed batch of clips with tail chunks of 37, 1 and 75 frames, an
    exact 2-chunk clip and a 9-chunk clip (two windows), against the library
    in float64.  Its position table is computed in float32 (rows 0..12), so
    the outputs agree to float32 rounding of the PE, not to fp64 rounding."""
    import dataclasses
    dims = dataclasses.replace(synth.DIMS_TINY, conv_channels=8, d_model=64, n_layers=2, n_heads=1, ffn_dim=128,
                               output_dim=32, window_chunks=window_chunks)
    W = O.as_f64(synth.make_weights(dims, 400 + window_chunks))
    lens = [16000 * 9 + 160 * 37 + 11, 201, 32000, 16000 * 6 + 160 * 75]
    clips = [synth.speech_like_clip(n, [401, i]).astype(np.float64) for i, n in enumerate(lens)]
    mels = [O.log_mel(x) for x in clips]
    ref = np.concatenate([np.concatenate([v for _, v in sorted(
        O.encode_clip(x, W, dims.n_layers, dims.n_heads, window_chunks=window_chunks, mel=m).items())])
        for x, m in zip(clips, mels)])
    enc, proj = _encoder_pair(dims, W)
    got = _library_encode(enc, proj, mels)
    assert got.shape == ref.shape == (sum(O.clip_num_tokens(n) for n in lens), dims.output_dim)
    err = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
    assert err.max() < 3e-7, err.max()          # measured <= 5e-8
    # reading B (stem on the m frames of a tail chunk) is what the library does not do
    refB = np.concatenate([np.concatenate([v for _, v in sorted(
        O.encode_clip(x, W, dims.n_layers, dims.n_heads, window_chunks=window_chunks, mel=m, tail="B").items())])
        for x, m in zip(clips, mels)])
    errB = np.linalg.norm(got - refB, axis=1) / np.linalg.norm(refB, axis=1)
    assert errB.max() > 100 * err.max(), (errB.max(), err.max())   # only the last row of a tail chunk differs


def test_front_end_matches_transformers_qwen3_asr_extractor():
    """The Qwen3-ASR feature extractor (torch.stft with centred reflection,
    periodic Hann, Slaney mel, 1e-10 floor, log10, max - 8, (x + 4) / 4, the
    last frame dropped) on clips it does not pad (min_length 0, no mel-axis
    padding): within the float32 tolerance the OneSpeech page states (3e-5)."""
    from transformers.models.qwen3_asr.feature_extraction_qwen3_asr import Qwen3ASRFeatureExtractor
    fe = Qwen3ASRFeatureExtractor(min_length=0)
    for i, n in enumerate((16000 * 7 + 123, 201, 16000 * 2 + 160 * 37 + 99)):
        x = synth.speech_like_clip(n, [402, i])
        f = fe(x, sampling_rate=16000, padding="longest", n_window=0, return_tensors="np")["input_features"][0]
        r = O.log_mel(x.astype(np.float64))
        assert f.shape == r.shape
        assert np.abs(f - r).max() <= 3e-5


def test_thinker_matches_transformers_qwen3():
    """Splice + prefill of a prompt through the library's Qwen3 text model
    (RMSNorm eps 1e-6, per-head q/k RMSNorm, rotate-half RoPE with base 1e6,
    GQA 4/2, SwiGLU, no bias, logits from the tied embedding) in float64,
    prompts with 40, 0 and 130 spliced states."""
    from transformers import Qwen3Config, Qwen3Model
    d = ST.ThinkerDims(hidden=256, n_layers=2, n_q_heads=4, n_kv_heads=2, ffn_dim=384, vocab=500, dtype="f32")
    W = {k: v.astype(np.float64) for k, v in ST.make_weights(d, 403).items()}
    cfg = Qwen3Config(vocab_size=d.vocab, hidden_size=d.hidden, intermediate_size=d.ffn_dim,
                      num_hidden_layers=d.n_layers, num_attention_heads=d.n_q_heads,
                      num_key_value_heads=d.n_kv_heads, head_dim=d.head_dim, rms_norm_eps=1e-6,
                      rope_parameters={"rope_type": "default", "rope_theta": 1e6}, attention_bias=False,
                      tie_word_embeddings=True, max_position_embeddings=4096)
    cfg._attn_implementation = "eager"
    model = Qwen3Model(cfg).double().eval()
    sd = {"embed_tokens.weight": W["embed"], "norm.weight": W["out_norm"]}
    names = {"attn_norm": "input_layernorm", "q_w": "self_attn.q_proj", "k_w": "self_attn.k_proj",
             "v_w": "self_attn.v_proj", "o_w": "self_attn.o_proj", "q_norm": "self_attn.q_norm",
             "k_norm": "self_attn.k_norm", "ffn_norm": "post_attention_layernorm", "gate_w": "mlp.gate_proj",
             "up_w": "mlp.up_proj", "down_w": "mlp.down_proj"}
    for l in range(d.n_layers):
        for ours, theirs in names.items():
            sd[f"layers.{l}.{theirs}.weight"] = W[f"layers.{l}.{ours}"]
    missing, unexpected = model.load_state_dict({k: _t(v) for k, v in sd.items()}, strict=False)
    assert not unexpected and not [m for m in missing if "rotary" not in m], (missing, unexpected)
    for i, n_audio in enumerate((40, 0, 130)):
        ids, off = ST.make_prompt(n_audio, d.vocab, [404, i])
        audio = ST.make_audio_states(n_audio, d.hidden, [405, i]).astype(np.float64)
        rh, rg = TH.prefill_prompt(ids, audio, off, W, d.n_layers, d.n_q_heads, d.n_kv_heads)
        with torch.no_grad():
            emb = model.embed_tokens(torch.from_numpy(ids.astype(np.int64)))
            if n_audio:
                emb[off:off + n_audio] = _t(audio)
            h = model(inputs_embeds=emb[None]).last_hidden_state[0]
            g = h[-1] @ model.embed_tokens.weight.T
        # the library computes the RoPE frequencies in float32: agreement to ~1e-7 relative
        assert np.abs(h.numpy() - rh).max() <= 2e-6 * np.abs(rh).max()
        assert np.abs(g.numpy() - rg).max() <= 2e-6 * np.abs(rg).max()
