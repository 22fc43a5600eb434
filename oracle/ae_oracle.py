"""CPU oracle for the flow-matching action-expert denoise loop (fp64, numpy).

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module. The product library
never calls it, and it shares no code with the GPU path: it decodes bf16 and
FP8 itself, and it computes every step plainly, in float64, with numpy's
matmul as the only library primitive.

Sources (page title, then section):

* "DM0.5: high-performance embodied VLA and OpenDM guide" (the DM0.5 guide):
  section 5.1 (prefix encoded once into a KV cache), section 5.2 (action
  expert modules: action_in_proj, time_mlp_in/out, prefix KV, action_out_proj,
  built on the Gemma3 text stack), section 5.3 (linear flow path, velocity
  target, Euler integration, 10 steps, action chunk), section 6.3 (FP8 E4M3
  with scales).
* "Realtime-VLA FLASH" article, section 02 (interpolate a draft with noise at
  several flow times, evaluate the expert's velocity there, rebuild endpoints,
  compare with the draft) and section 03 (delta-prefix acceptance at all
  verification times, fall back on length 0; a gripper switch in the candidate
  chunk forces the full path).

Readings where the pages are silent or garbled (listed with reasons in the
design notes):

* Time runs from 0 (noise) to 1 (action): x_t = (1 - t) eps + t a, the exact
  velocity is a - eps, and Euler steps x <- x + (1/N) v(x, k/N), k = 0..N-1.
  The DM0.5 guide writes the path with noise at t = 1 and prints the update
  as x_{t-dt} = x_t + v dt; both describe the same integration under
  t -> 1 - t, v -> -v.
* Time embedding: [sin | cos] of 2 pi t / p_i with periods geometric from
  4e-3 to 4, then time_mlp_in -> SiLU -> time_mlp_out, added to every
  action_in_proj row.
* Decoder block (Gemma-style, pre-norm): RMSNorm (eps inside the root, gain
  multiplies), GQA attention of the suffix rows over [prefix KV ; suffix KV]
  with no mask among the suffix rows, half-split RoPE at positions P + i on
  the suffix q and k (prefix K is used as cached), scale 1/sqrt(head_dim),
  GeGLU MLP with the tanh GELU, residual adds. Decoder linears have no bias;
  action_in/out and time_mlp_in/out have biases.
* Verification: one noise draw shared by all tau; endpoint a_hat = x + (1 - tau) v;
  Euclidean distance per chunk row over all action dims; strict < delta.
* Prefix prefill (DM0.5 guide 5.1): the VLM's Gemma blocks over the prefix token embeddings
  with full attention among the prefix tokens (a prefix is seen whole), RoPE at 0..P-1, no
  embedding scale or logit softcap; each layer's K (rotated) and V form the cache.
* Draft model (FLASH section 03: one Gemma block and a linear action head, learnable action
  queries over the current image features, one pass): the block's sequence is [features ;
  queries]; queries attend to all of it, RoPE positions 0..P-1 for the features and P.. for the
  queries; the head is the final RMSNorm then a linear map with bias. Features enter as tokens of
  the block's width.
* Time-modulated expert (time_mode 1; the guide derives a per-layer conditioning signal from the
  time MLP and leaves its form open): per layer a linear map of
  temb gives (scale, shift, gate) for each of the two sublayers, norm -> norm * (1 + scale) +
  shift, residual += gate * sublayer; the final norm gets (scale, shift) the same way; temb is
  then not added to the action tokens. QK-norm (qk_norm 1, Gemma3 text stack): RMSNorm of q and
  k per head over head_dim with gains q_norm / k_norm, before RoPE; the cached prefix K is used
  as given.
"""
import numpy as np

# ----------------------------------------------------------------------------
# storage-format decoders (own implementation, from the format definitions)
# ----------------------------------------------------------------------------


def decode_bf16(bits):
    """bf16 bit patterns (uint16) -> float64: the 16 bits are the top half of an IEEE binary32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN payloads are kept as NaN
        return u32.view(np.float32).astype(np.float64)


def _e4m3_value(code):
    """OCP FP8 E4M3 (e4m3fn) code -> value: 1 sign, 4 exponent (bias 7), 3 mantissa bits.

    Exponent 0 is subnormal (m/8 * 2^-6); exponent 15 with mantissa 7 is NaN;
    there is no infinity, so exponent 15 with mantissa 0..6 is a normal number.
    """
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return np.nan
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3(codes):
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode(arr, dtype, scale=None):
    """Storage array -> float64. fp8 rows are multiplied by their per-row scale."""
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return decode_bf16(arr)
    if dtype == "fp8":
        return decode_e4m3(arr) * np.asarray(scale, np.float64)[:, None]
    raise ValueError(dtype)


def dequantize_weights(cfg, W):
    """Decode every tensor of a weight dict (workload storage formats) to float64."""
    out = {}
    for name, arr in W.items():
        if name.endswith(".scale"):
            continue
        if arr.dtype == np.float32:
            out[name] = arr.astype(np.float64)
        elif name.split(".")[-1] in ("wg", "wu", "wd"):
            out[name] = decode(arr, cfg.mlp_dtype, W.get(name + ".scale"))
        else:
            out[name] = decode(arr, cfg.weight_dtype)
    return out


# ----------------------------------------------------------------------------
# elementwise pieces
# ----------------------------------------------------------------------------


def silu(x):
    return x / (1.0 + np.exp(-x))


def gelu_tanh(x):
    """GELU, tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))


def rmsnorm(x, gain, eps):
    """x / sqrt(mean(x^2) + eps) * gain over the last axis."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * gain


def linear(x, w, b=None):
    """x @ w^T (+ b); w is [out][in]."""
    y = x @ w.T
    return y if b is None else y + b


# ----------------------------------------------------------------------------
# time embedding (DM0.5 guide 5.2: time_mlp_in / time_mlp_out)
# ----------------------------------------------------------------------------

MIN_PERIOD = 4e-3
MAX_PERIOD = 4.0


def sinusoid(t, width):
    """phi(t): first half sin(2 pi t / p_i), second half cos(2 pi t / p_i),
    p_i = MIN_PERIOD * (MAX_PERIOD / MIN_PERIOD) ** (i / (width/2 - 1))."""
    half = width // 2
    frac = np.arange(half, dtype=np.float64) / (half - 1)
    period = MIN_PERIOD * (MAX_PERIOD / MIN_PERIOD) ** frac
    ang = 2.0 * np.pi * float(t) / period
    return np.concatenate([np.sin(ang), np.cos(ang)])


def time_embedding(Wd, t, width):
    """temb(t) = W_out silu(W_in phi(t) + b_in) + b_out."""
    hid = silu(linear(sinusoid(t, width), Wd["time_in_w"], Wd["time_in_b"]))
    return linear(hid, Wd["time_out_w"], Wd["time_out_b"])


# ----------------------------------------------------------------------------
# rotary position embedding and attention
# ----------------------------------------------------------------------------


def rope(x, positions, base):
    """Rotate pairs (d, d + dh/2) of the last axis by pos * base^(-2d/dh).

    x: [..., n_pos, n_heads, dh]; positions: [n_pos].
    """
    dh = x.shape[-1]
    half = dh // 2
    inv_freq = base ** (-2.0 * np.arange(half, dtype=np.float64) / dh)
    ang = np.asarray(positions, np.float64)[:, None] * inv_freq[None, :]  # [n_pos][half]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x1 * sin + x2 * cos], axis=-1)


def attention(q, k, v):
    """softmax(q k^T / sqrt(dh)) v per query head, GQA head map kv = head * n_kv // n_q.

    q: [n_rows][n_q][dh]; k, v: [n_keys][n_kv][dh] -> [n_rows][n_q][dh].
    """
    n_q, dh = q.shape[1], q.shape[2]
    n_kv = k.shape[1]
    out = np.empty_like(q)
    for hq in range(n_q):
        hk = hq * n_kv // n_q
        s = q[:, hq, :] @ k[:, hk, :].T / np.sqrt(dh)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, hq, :] = p @ v[:, hk, :]
    return out


# ----------------------------------------------------------------------------
# the action expert (velocity field) and its two uses
# ----------------------------------------------------------------------------


def layer_modulation(cfg, Wd, l, temb):
    """Per-layer scale/shift/gate taken linearly from temb (DM0.5 guide 5.2, which derives a per-layer
    conditioning signal from the time MLP without fixing its form): (scale1, shift1, gate1, scale2,
    shift2, gate2), each [w], for the attention and MLP sublayers."""
    return np.split(linear(temb, Wd[f"layers.{l}.w_mod"], Wd[f"layers.{l}.b_mod"]), 6)


def decoder_layer(cfg, Wd, l, h, k_pre, v_pre, mod=None):
    """One Gemma-style block over one sequence. h: [H][w]; k_pre, v_pre: [P][n_kv][dh].

    mod (time-modulated expert): (scale, shift, gate) per sublayer; the normalised input becomes
    rmsnorm(h) * (1 + scale) + shift and the sublayer output enters the residual times gate.
    With cfg.qk_norm, q and k are RMS-normalised per head over head_dim (gains q_norm, k_norm)
    before RoPE, as in the Gemma3 text stack the guide builds the expert on.
    """
    p = f"layers.{l}."
    H = h.shape[0]
    nq, nkv, dh = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    n = rmsnorm(h, Wd[p + "ln1"], cfg.rms_eps)
    if mod is not None:
        n = n * (1.0 + mod[0]) + mod[1]
    q = linear(n, Wd[p + "wq"]).reshape(H, nq, dh)
    k = linear(n, Wd[p + "wk"]).reshape(H, nkv, dh)
    v = linear(n, Wd[p + "wv"]).reshape(H, nkv, dh)
    if cfg.qk_norm:
        q = rmsnorm(q, Wd[p + "q_norm"], cfg.rms_eps)
        k = rmsnorm(k, Wd[p + "k_norm"], cfg.rms_eps)
    pos = cfg.prefix_len + np.arange(H)
    q = rope(q, pos, cfg.rope_base)
    k = rope(k, pos, cfg.rope_base)
    o = attention(q, np.concatenate([k_pre, k], axis=0), np.concatenate([v_pre, v], axis=0))
    a = linear(o.reshape(H, nq * dh), Wd[p + "wo"])
    h = h + (a if mod is None else mod[2] * a)
    n2 = rmsnorm(h, Wd[p + "ln2"], cfg.rms_eps)
    if mod is not None:
        n2 = n2 * (1.0 + mod[3]) + mod[4]
    u = gelu_tanh(linear(n2, Wd[p + "wg"])) * linear(n2, Wd[p + "wu"])
    m = linear(u, Wd[p + "wd"])
    return h + (m if mod is None else mod[5] * m)


def velocity(cfg, Wd, kv_k, kv_v, x, t):
    """v_theta(x_t, t | c) for one sequence (DM0.5 guide 5.2).

    x: [H][A] float64, t: scalar flow time, kv_k / kv_v: [L][P][n_kv][dh] float64.
    cfg.time_mode 0: temb is added to every action_in_proj row; 1: temb modulates every layer's
    norms and residual branches and the final norm (final scale and shift from final_mod).
    """
    temb = time_embedding(Wd, t, cfg.width)
    h = linear(x, Wd["action_in_w"], Wd["action_in_b"])
    if not cfg.time_mode:
        h = h + temb[None, :]
    for l in range(cfg.n_layers):
        mod = layer_modulation(cfg, Wd, l, temb) if cfg.time_mode else None
        h = decoder_layer(cfg, Wd, l, h, kv_k[l], kv_v[l], mod)
    n = rmsnorm(h, Wd["final_ln"], cfg.rms_eps)
    if cfg.time_mode:
        scale, shift = np.split(linear(temb, Wd["final_mod_w"], Wd["final_mod_b"]), 2)
        n = n * (1.0 + scale) + shift
    return linear(n, Wd["action_out_w"], Wd["action_out_b"])


def euler_integrate(x0, steps, vfield):
    """Integrate dx/dt = vfield(x, t) from t = 0 to t = 1 in ``steps`` uniform Euler steps.

    The field is evaluated at t_k = k / steps, k = 0 .. steps-1 (never at t = 1).
    """
    x = np.array(x0, dtype=np.float64)
    dt = 1.0 / steps
    for k in range(steps):
        x = x + dt * vfield(x, k * dt)
    return x


def denoise(cfg, Wd, kv_k, kv_v, noise, steps):
    """Noise [H][A] -> action chunk [H][A] for one robot with its own prefix cache."""
    return euler_integrate(noise, steps, lambda x, t: velocity(cfg, Wd, kv_k, kv_v, x, t))


def denoise_batch(cfg, Wd, kvs, noise, steps):
    """Robots are independent: robot r uses cache kvs[r] = (K, V) and noise[r]."""
    return np.stack([denoise(cfg, Wd, kvs[r][0], kvs[r][1], noise[r], steps) for r in range(noise.shape[0])])


def interpolate(draft, noise, taus):
    """x_j = (1 - tau_j) eps + tau_j d: the draft placed on the linear flow path at each tau_j."""
    taus = np.asarray(taus, np.float64)[:, None, None]
    return (1.0 - taus) * np.asarray(noise, np.float64)[None] + taus * np.asarray(draft, np.float64)[None]


def gripper_switch(draft, gripper_dim):
    """1 if the gripper channel changes sign between two consecutive chunk rows, else 0."""
    if gripper_dim < 0:
        return 0
    g = np.asarray(draft, np.float64)[:, gripper_dim]
    return int(np.any(g[1:] * g[:-1] < 0))


def accept_from_distances(D, delta, switch):
    """Longest prefix k with D[j, i] < delta for all i < k and all j; 0 when switch is set."""
    ok = np.all(np.asarray(D) < delta, axis=0)
    accept = 0
    while accept < ok.shape[0] and ok[accept]:
        accept += 1
    return 0 if switch else accept


def accept_from_velocity(draft, x_tau, v_tau, taus, delta, gripper_dim):
    """FLASH acceptance given the expert velocity at each verification time.

    a_hat_j = x_j + (1 - tau_j) v_j; D[j, i] = || a_hat_j[i] - d[i] ||_2;
    accept = longest prefix k with D[j, i] < delta for all i < k and all j,
    forced to 0 when the draft contains a gripper switch.
    Returns (accept, switch, D).
    """
    taus = np.asarray(taus, np.float64)
    a_hat = x_tau + (1.0 - taus)[:, None, None] * v_tau
    D = np.sqrt(np.sum((a_hat - np.asarray(draft, np.float64)[None]) ** 2, axis=-1))
    switch = gripper_switch(draft, gripper_dim)
    return accept_from_distances(D, delta, switch), switch, D


def verify(cfg, Wd, kv_k, kv_v, draft, noise, taus, delta):
    """Speculative verification of one draft chunk against the expert (FLASH section 03)."""
    x_tau = interpolate(draft, noise, taus)
    v_tau = np.stack([velocity(cfg, Wd, kv_k, kv_v, x_tau[j], float(taus[j])) for j in range(len(taus))])
    return accept_from_velocity(draft, x_tau, v_tau, taus, delta, cfg.gripper_dim)


def dual_path_round(cfg, Wd, kv_k, kv_v, draft, noise_verify, taus, delta, noise_full, steps):
    """One round of the dual-path runtime (FLASH section 03): the fast path verifies the draft;
    when the accepted prefix is empty (a gripper switch in the draft forces that), the round falls
    back to the full path, the denoise loop from noise_full. Returns (actions, accept, switch,
    full_path): the draft on the fast path, the denoised chunk on the full path."""
    accept, switch, _ = verify(cfg, Wd, kv_k, kv_v, draft, noise_verify, taus, delta)
    if accept == 0:
        return denoise(cfg, Wd, kv_k, kv_v, noise_full, steps), accept, switch, 1
    return np.asarray(draft, np.float64), accept, switch, 0


def draft_feature_kv(cfg, Wd, feats):
    """K/V that the draft block's attention reads for the image features (FLASH section 03, draft action
    generation): the block's own RMSNorm and k / v projections of each feature token, K rotated at the
    token's position 0..P-1. feats: [P][w] -> (k, v) each [P][n_kv][dh]."""
    P = feats.shape[0]
    n = rmsnorm(np.asarray(feats, np.float64), Wd["layers.0.ln1"], cfg.rms_eps)
    k = linear(n, Wd["layers.0.wk"]).reshape(P, cfg.n_kv_heads, cfg.head_dim)
    v = linear(n, Wd["layers.0.wv"]).reshape(P, cfg.n_kv_heads, cfg.head_dim)
    return rope(k, np.arange(P), cfg.rope_base), v


def draft_chunk(cfg, Wd, feats):
    """Candidate chunk of the draft model (FLASH section 03): one Gemma block over [image features ;
    learnable action queries] with every query attending to every feature and every query, then the
    final RMSNorm and a linear action head on the query rows. Only the queries' rows are needed, so the
    features enter as cached K/V (draft_feature_kv) and the queries as the suffix rows at positions
    P .. P+H-1. feats: [P][w] -> chunk [H][A]."""
    k_pre, v_pre = draft_feature_kv(cfg, Wd, feats)
    h = decoder_layer(cfg, Wd, 0, np.asarray(Wd["queries"], np.float64), k_pre, v_pre)
    return linear(rmsnorm(h, Wd["final_ln"], cfg.rms_eps), Wd["action_out_w"], Wd["action_out_b"])


def prefill_kv(cfg, Wd, emb):
    """Per-layer prefix K/V cache from the prefix token embeddings (DM0.5 guide 5.1: the prefix is
    encoded once by the VLM into a KV cache every step reuses): the VLM's Gemma blocks over the P
    prefix tokens, every token attending to every prefix token, RoPE at positions 0..P-1. Returns
    K (rotated, as the expert uses it) and V, each [L][P][n_kv][dh]. emb: [P][w]."""
    P = emb.shape[0]
    nq, nkv, dh = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    pos = np.arange(P)
    h = np.asarray(emb, np.float64)
    ks, vs = [], []
    for l in range(cfg.n_layers):
        p = f"layers.{l}."
        n = rmsnorm(h, Wd[p + "ln1"], cfg.rms_eps)
        q = rope(linear(n, Wd[p + "wq"]).reshape(P, nq, dh), pos, cfg.rope_base)
        k = rope(linear(n, Wd[p + "wk"]).reshape(P, nkv, dh), pos, cfg.rope_base)
        v = linear(n, Wd[p + "wv"]).reshape(P, nkv, dh)
        ks.append(k)
        vs.append(v)
        h = h + linear(attention(q, k, v).reshape(P, nq * dh), Wd[p + "wo"])
        n2 = rmsnorm(h, Wd[p + "ln2"], cfg.rms_eps)
        h = h + linear(gelu_tanh(linear(n2, Wd[p + "wg"])) * linear(n2, Wd[p + "wu"]), Wd[p + "wd"])
    return np.stack(ks), np.stack(vs)


def decode_kv(cfg, k, v):
    return decode(k, cfg.kv_dtype), decode(v, cfg.kv_dtype)
