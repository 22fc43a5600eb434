"""ctypes binding of the C-ABI in include/ae.h (argument marshalling only).

Every step of the denoise loop and of verification runs in the HIP library
``libae.so``; this module only turns numpy arrays into the plain pointers and
structs that the C-ABI takes. There is no fallback: if the library is missing
or a call fails, it raises.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libae.so")

AE_OK = 0
ERRORS = {-1: "AE_ERR_INVALID_ARG", -2: "AE_ERR_UNSUPPORTED", -3: "AE_ERR_NOT_READY", -4: "AE_ERR_OOM", -5: "AE_ERR_HIP"}
DTYPES = {"f32": 0, "bf16": 1, "fp8": 2}
EXPORTS = ("ae_create", "ae_load_prefix_kv", "ae_denoise", "ae_denoise_async", "ae_denoise_static", "ae_verify", "ae_verify_async", "ae_round",
           "ae_draft", "ae_prefill", "ae_prefill_to_slot",
           "ae_destroy", "ae_last_error", "ae_last_gpu_ms", "ae_kernel_times")


class AEError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


class ae_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "n_layers", "width", "n_q_heads", "n_kv_heads", "head_dim", "mlp_dim", "action_dim", "horizon",
        "prefix_len", "max_batch", "max_taus")] + [("rope_base", ctypes.c_float), ("rms_eps", ctypes.c_float)] + [
        (n, ctypes.c_int) for n in ("weight_dtype", "mlp_dtype", "kv_dtype", "gripper_dim", "time_mode", "qk_norm",
                                    "draft", "prefill")]


class ae_layer_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "ln1", "wq", "wk", "wv", "wo", "ln2", "wg", "wu", "wd", "wg_scale", "wu_scale", "wd_scale",
        "w_mod", "b_mod", "q_norm", "k_norm")]


class ae_weights(ctypes.Structure):
    _fields_ = [("time_in_w", ctypes.c_void_p), ("time_in_b", ctypes.c_void_p),
                ("time_out_w", ctypes.c_void_p), ("time_out_b", ctypes.c_void_p),
                ("action_in_w", ctypes.c_void_p), ("action_in_b", ctypes.c_void_p),
                ("layers", ctypes.POINTER(ae_layer_weights)),
                ("final_ln", ctypes.c_void_p), ("action_out_w", ctypes.c_void_p), ("action_out_b", ctypes.c_void_p),
                ("final_mod_w", ctypes.c_void_p), ("final_mod_b", ctypes.c_void_p), ("queries", ctypes.c_void_p)]


class ae_kernel_stat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int), ("total_ms", ctypes.c_float)]


_lib = None


def load_library(path=LIB_PATH):
    """Load libae.so and declare the prototypes. Raises OSError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError(f"{path} is missing: build it first (python -c 'import __graft_entry__; __graft_entry__.build()')")
    lib = ctypes.CDLL(path)
    P, I, F, V = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, None
    protos = {
        "ae_create": (I, [ctypes.POINTER(ae_config), ctypes.POINTER(ae_weights), ctypes.POINTER(P)]),
        "ae_load_prefix_kv": (I, [P, I, P, P]),
        "ae_denoise": (I, [P, I, P, I, P]),
        "ae_denoise_async": (I, [P, I, P, I, P, P]),
        "ae_denoise_static": (I, [P, I, P, I, P, P]),
        "ae_verify": (I, [P, I, P, P, P, I, F, P, P, P]),
        "ae_verify_async": (I, [P, I, P, P, P, I, F, P, P, P, P]),
        "ae_round": (I, [P, I, P, P, P, I, F, P, I, P, P, P, P]),
        "ae_draft": (I, [P, P, P]),
        "ae_prefill": (I, [P, P, P, P]),
        "ae_prefill_to_slot": (I, [P, P, P, I]),
        "ae_destroy": (V, [P]),
        "ae_last_error": (ctypes.c_char_p, [P]),
        "ae_last_gpu_ms": (I, [P, ctypes.POINTER(F)]),
        "ae_kernel_times": (I, [P, I, I, I, I, ctypes.POINTER(ae_kernel_stat), I, ctypes.POINTER(I)]),
    }
    for name, (res, args) in protos.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def make_config(cfg):
    """ae_config from any object with the config attribute names (dtype names "f32" | "bf16" | "fp8")."""
    return ae_config(
        n_layers=cfg.n_layers, width=cfg.width, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
        head_dim=cfg.head_dim, mlp_dim=cfg.mlp_dim, action_dim=cfg.action_dim, horizon=cfg.horizon,
        prefix_len=cfg.prefix_len, max_batch=cfg.max_batch, max_taus=cfg.max_taus, rope_base=cfg.rope_base,
        rms_eps=cfg.rms_eps, weight_dtype=DTYPES[cfg.weight_dtype], mlp_dtype=DTYPES[cfg.mlp_dtype],
        kv_dtype=DTYPES[cfg.kv_dtype], gripper_dim=cfg.gripper_dim, time_mode=getattr(cfg, "time_mode", 0),
        qk_norm=getattr(cfg, "qk_norm", 0), draft=getattr(cfg, "draft", 0), prefill=getattr(cfg, "prefill", 0))


class ActionExpert:
    """One library handle: weights resident on the current HIP device.

    ``weights`` maps the tensor names of include/ae.h (``layers.{l}.wq`` ...) to
    host arrays in their storage format: float32, uint16 bf16 bit patterns or
    uint8 E4M3 codes with ``<name>.scale`` float32 per-row scales.
    """

    def __init__(self, cfg, weights):
        self.lib = load_library()
        self.cfg = cfg
        keep = []

        def p(name):
            a = weights.get(name)
            if a is None:
                return None
            a = np.ascontiguousarray(a)
            keep.append(a)
            return a.ctypes.data

        L = cfg.n_layers
        layers = (ae_layer_weights * L)()
        for l in range(L):
            pre = f"layers.{l}."
            for f in ("ln1", "wq", "wk", "wv", "wo", "ln2", "wg", "wu", "wd", "w_mod", "b_mod", "q_norm", "k_norm"):
                setattr(layers[l], f, p(pre + f))
            for f in ("wg", "wu", "wd"):
                setattr(layers[l], f + "_scale", p(pre + f + ".scale"))
        w = ae_weights(time_in_w=p("time_in_w"), time_in_b=p("time_in_b"), time_out_w=p("time_out_w"),
                       time_out_b=p("time_out_b"), action_in_w=p("action_in_w"), action_in_b=p("action_in_b"),
                       layers=layers, final_ln=p("final_ln"), action_out_w=p("action_out_w"),
                       action_out_b=p("action_out_b"), final_mod_w=p("final_mod_w"), final_mod_b=p("final_mod_b"),
                       queries=p("queries"))
        self._cfg = make_config(cfg)
        h = ctypes.c_void_p()
        rc = self.lib.ae_create(ctypes.byref(self._cfg), ctypes.byref(w), ctypes.byref(h))
        if rc != AE_OK:
            raise AEError(rc, self.lib.ae_last_error(None).decode())
        self.h = h

    def _check(self, rc):
        if rc != AE_OK:
            raise AEError(rc, self.lib.ae_last_error(self.h).decode())

    def close(self):
        if getattr(self, "h", None):
            self.lib.ae_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def load_prefix_kv(self, slot, k, v):
        dt = np.float32 if self.cfg.kv_dtype == "f32" else np.uint16
        k, v = _c(k, dt), _c(v, dt)
        self._check(self.lib.ae_load_prefix_kv(self.h, slot, _ptr(k), _ptr(v)))

    def denoise(self, noise, steps):
        noise = _c(noise, np.float32)
        out = np.empty_like(noise)
        self._check(self.lib.ae_denoise(self.h, noise.shape[0], _ptr(noise), steps, _ptr(out)))
        return out

    def denoise_async(self, batch, d_noise, steps, d_out, stream=None):
        """Device-pointer variant (ints from e.g. torch ``tensor.data_ptr()``)."""
        self._check(self.lib.ae_denoise_async(self.h, batch, ctypes.c_void_p(d_noise), steps,
                                              ctypes.c_void_p(d_out), ctypes.c_void_p(stream) if stream else None))

    def denoise_static(self, batch, d_noise, steps, d_out, stream=None):
        """ae_denoise_static: as denoise_async, with the pass's scratch in the library's static
        device array instead of the handle's buffers (no allocation)."""
        self._check(self.lib.ae_denoise_static(self.h, batch, ctypes.c_void_p(d_noise), steps,
                                               ctypes.c_void_p(d_out), ctypes.c_void_p(stream) if stream else None))

    def verify(self, slot, draft, noise, taus, delta, want_dist=True):
        draft, noise, taus = _c(draft, np.float32), _c(noise, np.float32), _c(taus, np.float32)
        acc, sw = ctypes.c_int(), ctypes.c_int()
        dist = np.empty((len(taus), self.cfg.horizon), np.float32) if want_dist else None
        self._check(self.lib.ae_verify(self.h, slot, _ptr(draft), _ptr(noise), _ptr(taus), len(taus),
                                       ctypes.c_float(delta), ctypes.byref(acc), ctypes.byref(sw), _ptr(dist)))
        return acc.value, sw.value, dist

    def verify_async(self, slot, d_draft, d_noise, d_taus, n_tau, delta, d_accept, d_switch, d_dist=None, stream=None):
        self._check(self.lib.ae_verify_async(
            self.h, slot, ctypes.c_void_p(d_draft), ctypes.c_void_p(d_noise), ctypes.c_void_p(d_taus), n_tau,
            ctypes.c_float(delta), ctypes.c_void_p(d_accept), ctypes.c_void_p(d_switch),
            ctypes.c_void_p(d_dist) if d_dist else None, ctypes.c_void_p(stream) if stream else None))

    def round(self, slot, draft, noise_verify, taus, delta, noise_full, steps):
        """One dual-path round: (actions [H][A], accept_len, gripper_switch, full_path)."""
        draft, nv, taus, nf = (_c(draft, np.float32), _c(noise_verify, np.float32), _c(taus, np.float32),
                               _c(noise_full, np.float32))
        out = np.empty_like(draft)
        acc, sw, full = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        self._check(self.lib.ae_round(self.h, slot, _ptr(draft), _ptr(nv), _ptr(taus), len(taus), ctypes.c_float(delta),
                                      _ptr(nf), steps, _ptr(out), ctypes.byref(acc), ctypes.byref(sw),
                                      ctypes.byref(full)))
        return out, acc.value, sw.value, full.value

    def draft(self, features):
        """Candidate chunk [H][A] of a draft-model handle from image features [P][w]."""
        features = _c(features, np.float32)
        out = np.empty((self.cfg.horizon, self.cfg.action_dim), np.float32)
        self._check(self.lib.ae_draft(self.h, _ptr(features), _ptr(out)))
        return out

    def prefill(self, emb):
        """Per-layer prefix (K, V) [L][P][n_kv][dh] in kv_dtype storage from embeddings [P][w]."""
        emb = _c(emb, np.float32)
        c = self.cfg
        dt = np.float32 if c.kv_dtype == "f32" else np.uint16
        k = np.empty((c.n_layers, c.horizon, c.n_kv_heads, c.head_dim), dt)
        v = np.empty_like(k)
        self._check(self.lib.ae_prefill(self.h, _ptr(emb), _ptr(k), _ptr(v)))
        return k, v

    def prefill_to_slot(self, emb, expert, slot):
        """Run this prefill stack over embeddings [P][w] and copy every layer's K/V on the device into
        prefix slot `slot` of the expert handle `expert` (an ActionExpert)."""
        emb = _c(emb, np.float32)
        self._check(self.lib.ae_prefill_to_slot(self.h, _ptr(emb), expert.h, slot))

    def last_gpu_ms(self):
        ms = ctypes.c_float()
        self._check(self.lib.ae_last_gpu_ms(self.h, ctypes.byref(ms)))
        return ms.value

    def kernel_times(self, mode, batch, steps, iters):
        stats = (ae_kernel_stat * 64)()
        n = ctypes.c_int()
        self._check(self.lib.ae_kernel_times(self.h, mode, batch, steps, iters, stats, 64, ctypes.byref(n)))
        return [(stats[i].name.decode(), stats[i].launches, stats[i].total_ms) for i in range(n.value)]
