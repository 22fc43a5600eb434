/*
 * ae.h -- C-ABI of the MI355X (gfx950) flow-matching action-expert library.
 *
 * What it computes. A VLM prefix (images, text, robot state) is encoded once
 * into a per-layer key/value cache; each of N Euler steps then runs only the
 * action suffix of the expert: action_in_proj plus a sinusoidal time
 * embedding through time_mlp_in / time_mlp_out, L Gemma-style decoder blocks
 * (RMSNorm, grouped-query attention of the suffix rows over
 * [cached prefix KV ; suffix KV] with rotary positions, GeGLU MLP), a final
 * RMSNorm and action_out_proj giving the velocity v, then x += dt * v.
 *   - "DM0.5: high-performance embodied VLA and OpenDM guide", section 5.1
 *     (prefix once, KV cache reused by every step), section 5.2 (suffix
 *     modules), section 5.3 (flow-matching path and Euler sampling, 10 steps,
 *     action chunk), section 6.3 (FP8 E4M3 MLP weights with scales),
 *     section 6.5 (fixed shapes, static buffers, one graph replay).
 *   - "Realtime-VLA FLASH" article, sections 02-03: speculative verification
 *     of a draft chunk at several flow times in one batched pass, endpoint
 *     reconstruction, delta-prefix acceptance, gripper-switch fallback.
 *
 * Conventions (the pages leave these open; the library and its tests use them):
 *   - time runs 0 (noise) -> 1 (action); step k evaluates v at t_k = k/N and
 *     applies x += (1/N) v; the velocity is never evaluated at t = 1;
 *   - time embedding phi(t) = [sin(2 pi t / p_i) | cos(2 pi t / p_i)],
 *     p_i geometric from 4e-3 to 4 over width/2 entries; temb =
 *     time_out(silu(time_in(phi))) is added to every action_in_proj row;
 *   - RMSNorm y = x / sqrt(mean(x^2) + eps) * gain; GELU is the tanh form;
 *   - RoPE rotates pairs (d, d + head_dim/2) by pos * base^(-2d/head_dim), suffix
 *     row i sits at position prefix_len + i; the cached prefix K is used as given;
 *   - suffix rows see every prefix key and every suffix key of their own
 *     sequence (no mask); scale 1/sqrt(head_dim); query head h reads kv head
 *     h * n_kv_heads / n_q_heads;
 *   - decoder linears have no bias; action_in/out and time_mlp_in/out do.
 *
 * Layouts. Every matrix is row-major [out][in]. bf16 tensors are uint16 bit
 * patterns; fp8 tensors are OCP E4M3 (e4m3fn) bytes with one fp32 scale per
 * output row (value = scale[row] * e4m3(code)). Gains and biases are fp32.
 * Prefix caches are [n_layers][prefix_len][n_kv_heads][head_dim] in kv_dtype.
 * Action chunks are [batch][horizon][action_dim] fp32.
 *
 * Ownership. Device memory belongs to the library. Host buffers belong to the
 * caller and are only read (or written) during the call. Weights and caches
 * are copied; the caller may free them after the call returns.
 *
 * Errors. Every int-returning call returns AE_OK (0) or a negative AE_ERR_*
 * code and never throws; ae_last_error() describes the last failure. On error
 * the outputs are not written. A bounded wait inside a kernel that gave up
 * (data of another workgroup never arrived: not all of the launch was resident)
 * does not fail a synchronous call: it restores the exchange buffers and repeats
 * its pass with launches that have no in-kernel waits, and returns that pass's
 * outputs. An asynchronous call cannot repeat its pass: the next call on the
 * handle reports AE_ERR_HIP (the outputs of the asynchronous passes since the last
 * successful call are invalid) and restores the buffers. A handle is not re-entrant: calls on one
 * handle must not overlap. Separate handles are independent.
 */
#ifndef AE_H_
#define AE_H_

#ifdef __cplusplus
extern "C" {
#endif

#define AE_OK 0
#define AE_ERR_INVALID_ARG (-1)  /* null pointer, bad size, out-of-range slot/batch/steps */
#define AE_ERR_UNSUPPORTED (-2)  /* shape or dtype combination the kernels do not cover */
#define AE_ERR_NOT_READY (-3)    /* a prefix slot used before ae_load_prefix_kv */
#define AE_ERR_OOM (-4)          /* device allocation failed */
#define AE_ERR_HIP (-5)          /* a HIP runtime call failed (no device, launch error, ...) */

enum ae_dtype { AE_F32 = 0, AE_BF16 = 1, AE_FP8_E4M3 = 2 };

typedef struct ae_config {
  int n_layers;     /* L decoder blocks (1..1024) */
  int width;        /* hidden size w (multiple of 256, <= 65536) */
  int n_q_heads;    /* query heads (n_q_heads * head_dim a multiple of 256; <= 1024) */
  int n_kv_heads;   /* key/value heads (divides n_q_heads; <= 1024) */
  int head_dim;     /* dh: 32, 64, 128 or 256 */
  int mlp_dim;      /* GeGLU inner size F (multiple of 256, <= 2^20) */
  int action_dim;   /* A (1..64) */
  int horizon;      /* H chunk rows (1..256; a prefill stack: 1..1024 tokens) */
  int prefix_len;   /* P cached prefix tokens (0..2^20) */
  int max_batch;    /* prefix slots = robots advanced together by ae_denoise (1..4096) */
  int max_taus;     /* verification times per ae_verify call (0..64; 0 disables ae_verify) */
  float rope_base;  /* e.g. 10000 */
  float rms_eps;    /* e.g. 1e-6 (>= 0) */
  int weight_dtype; /* AE_F32 | AE_BF16: q/k/v/o, action in/out, time MLP */
  int mlp_dtype;    /* AE_F32 | AE_BF16 | AE_FP8_E4M3: gate / up / down; AE_F32 exactly when
                       weight_dtype is AE_F32 */
  int kv_dtype;     /* prefix cache: equal to weight_dtype */
  int gripper_dim;  /* action dim holding the +-1 gripper channel, -1 = none */
  int time_mode;    /* 0: temb added to every action_in_proj row; 1: per-layer time modulation
                       (see ae_layer_weights.w_mod; bf16 weights and MLP; ae_verify / ae_round form
                       each verification time's modulation vectors inside the pass) */
  int qk_norm;      /* 1: RMSNorm of q and k per head over head_dim (gains q_norm, k_norm)
                       before RoPE; the cached prefix K is used as given */
  int draft;        /* 1: a draft model for ae_draft ("Realtime-VLA FLASH" article, section 03:
                       one Gemma block and a linear action head; learnable action queries read the
                       current image features): n_layers 1, prefix_len = image tokens, max_batch 1,
                       max_taus 0, time_mode 0, qk_norm 0, bf16; the time MLP and action_in weights
                       are unused (may be NULL), ae_weights.queries is required */
  int prefill;      /* 1: a prefix-prefill stack for ae_prefill ("DM0.5" guide, section 5.1: the
                       prefix is encoded once into the per-layer KV cache): horizon = prefix tokens
                       (<= 1024), prefix_len 0, max_batch 1, max_taus 0, bf16 attention weights
                       (MLP bf16 or fp8), no modulation or QK-norm; only the decoder blocks are used */
} ae_config;

/* One decoder block. wq [n_q*dh][w], wk/wv [n_kv*dh][w], wo [w][n_q*dh],
 * wg/wu [F][w], wd [w][F]; *_scale are fp32 per output row, fp8 only (NULL otherwise).
 * time_mode 1 ("DM0.5" guide, section 5.2, where the time MLP conditions every layer; the
 * linear scale/shift/gate form is this library's reading): w_mod [6w][w] (weight_dtype) and
 * b_mod [6w] map temb to
 * (scale1, shift1, gate1, scale2, shift2, gate2); the attention input is
 * rmsnorm(h)*ln1*(1 + scale1) + shift1 and h += gate1 * o_proj(...), likewise for the MLP
 * with the second triple. qk_norm 1: q_norm, k_norm [dh] fp32 gains. Unused pointers NULL. */
typedef struct ae_layer_weights {
  const float* ln1;
  const void* wq;
  const void* wk;
  const void* wv;
  const void* wo;
  const float* ln2;
  const void* wg;
  const void* wu;
  const void* wd;
  const float* wg_scale;
  const float* wu_scale;
  const float* wd_scale;
  const void* w_mod;
  const float* b_mod;
  const float* q_norm;
  const float* k_norm;
} ae_layer_weights;

/* time_in_w/time_out_w [w][w], action_in_w [w][A], action_out_w [A][w], all host pointers.
 * time_mode 1: final_mod_w [2w][w] and final_mod_b [2w] give (scale, shift) of the final norm
 * from temb: rmsnorm(h)*final_ln*(1 + scale) + shift; NULL otherwise. */
typedef struct ae_weights {
  const void* time_in_w;
  const float* time_in_b;
  const void* time_out_w;
  const float* time_out_b;
  const void* action_in_w;
  const float* action_in_b;
  const ae_layer_weights* layers; /* n_layers entries */
  const float* final_ln;
  const void* action_out_w;
  const float* action_out_b;
  const void* final_mod_w;
  const float* final_mod_b;
  const float* queries;       /* draft 1: learnable action queries [H][w] fp32; NULL otherwise */
} ae_weights;

typedef struct ae_handle ae_handle;

/* Validate cfg, allocate device memory on the current HIP device, pack and
 * upload the weights (host pointers; copied). *out receives the handle.
 * The shape contract is fixed for the handle's lifetime (DM0.5 guide 6.1 and
 * 6.5: fixed image count, token length and chunk shape). Returns
 * AE_ERR_INVALID_ARG / AE_ERR_UNSUPPORTED before touching the GPU when cfg is
 * not covered, AE_ERR_HIP if no device is usable, AE_ERR_OOM on allocation failure.
 * Read here from the environment, once, for the handle's lifetime (all optional):
 *   AE_FUSED=0         batch-1 denoise passes use one launch per phase instead of the
 *                      persistent step kernel (one launch per Euler step);
 *   AE_ATTN_CORESIDENT=0  attention key splits merge in a separate launch instead of
 *                      inside the attention launch;
 *   AE_EXCH_POLL=0     split-K partials meet through arrival tickets instead of being
 *                      polled;
 *   AE_SPLITK=<o>,<d>  split-K factors (1..4) of o_proj and down in passes of one
 *                      64-token group (default 4,4; lowered to what divides K);
 *   AE_TILED=<mask>    GEMM roles (bit 0 qkv, 1 o_proj, 2 gate/up, 3 down) that may take
 *                      the token-tiled kernel when a pass has 128 or more tokens (0xf);
 *   AE_TILED_SHAPE=0..3  force one tiled shape wherever it fits;
 *   AE_ATTN_XCD=0      attention workgroups of one sequence not grouped on one XCD when
 *                      a pass has 8 or more sequences;
 *   AE_WAIT_TICKS=<n>  bound of every in-kernel wait in ticks of the 100 MHz clock
 *                      (default 2e6 = 20 ms; 0 makes every wait give up at once);
 *   AE_GRAPH=0         passes enqueue their launches directly instead of replaying a
 *                      captured graph (same kernels, same arguments, same results).
 * The persistent step kernel and the in-kernel exchanges assume every workgroup of
 * their launch is resident at once (one workgroup per compute unit). ae_create asks
 * the runtime's occupancy calculator (hipOccupancyMaxActiveBlocksPerMultiprocessor)
 * for each kernel that may wait: the step kernel, the split attention kernels and the
 * split-K GEMM kernels of the handle's dtypes; a kernel with no workgroup per compute
 * unit is never launched in a form that waits. When another
 * process or stream holds compute units, a bounded wait gives up, sets a host-visible
 * flag, and the call repeats its pass with launches that wait for nothing inside a
 * kernel (see Errors); after three such passes in a row a handle stops trying the
 * step kernel. */
int ae_create(const ae_config* cfg, const ae_weights* w, ae_handle** out);

/* Copy one robot's prefix cache into slot (0 <= slot < max_batch). k and v are
 * host [n_layers][prefix_len][n_kv_heads][head_dim] in kv_dtype, keys already
 * position-rotated by the prefix encoder (DM0.5 guide 5.1). Synchronous. */
int ae_load_prefix_kv(ae_handle* h, int slot, const void* k, const void* v);

/* Denoise `batch` robots (slots 0..batch-1) from host noise [batch][H][A]
 * with `steps` uniform Euler steps (DM0.5 guide 5.3); writes the host action
 * chunks [batch][H][A]. Synchronous. The first call for a new (steps, batch)
 * builds and captures a graph of the whole step loop (slow, once). */
int ae_denoise(ae_handle* h, int batch, const float* noise, int steps, float* actions_out);

/* Same as ae_denoise with device pointers (d_noise, d_actions_out: device
 * [batch][H][A] fp32), enqueued on `stream` (a hipStream_t; NULL = the
 * library's own stream). Returns after enqueueing; the caller synchronises. */
int ae_denoise_async(ae_handle* h, int batch, const float* d_noise, int steps, float* d_actions_out,
                     void* stream);

/* Bytes of the static device scratch behind ae_denoise_static (64 MiB per device). */
#define AE_STATIC_SCRATCH_BYTES (64u << 20)

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): ae_denoise_async with
 * every activation, partial, counter and time table of the pass taken from one
 * file-scope device array of AE_STATIC_SCRATCH_BYTES (each device holds its own
 * copy until the process ends) instead of the handle's buffers. The call makes
 * no hipMalloc / hipFree / allocating library call and no hipMemsetAsync: it
 * enqueues on `stream` (NULL = the library's stream) a clear kernel over the
 * bytes the pass uses, the step-time table, the time MLP, the copy of d_noise
 * in, the denoise pass (one launch per phase, no waits inside a kernel, so no
 * pass ever needs repeating) and the copy out to d_actions_out (device
 * [batch][H][A] fp32); it returns after enqueueing. Every call on a device
 * shares that device's array and it keeps the last call's contents: calls
 * that overlap on one device (two streams, two handles) race and their outputs
 * are undefined. AE_ERR_INVALID_ARG, before anything is enqueued, when the
 * pass needs more than AE_STATIC_SCRATCH_BYTES (about 20 MB per Pi0-shaped
 * robot at 10 steps: three fit, four do not); AE_ERR_UNSUPPORTED for a time-modulated
 * expert (its modulation tables are built in allocated memory); otherwise the
 * errors of ae_denoise_async. The result equals ae_denoise_async's within the
 * bf16 tolerance of the path (its batch-1 passes run the persistent step
 * kernel, whose sums are split differently). */
int ae_denoise_static(ae_handle* h, int batch, const float* d_noise, int steps, float* d_actions_out,
                      void* stream);

/* Speculative verification of a draft chunk against the expert (Realtime-VLA
 * FLASH, sections 02-03). Host inputs: draft [H][A], noise [H][A] (one draw
 * shared by every tau), taus [n_tau] in [0, 1). The expert velocity v_j is
 * evaluated at x_j = (1 - tau_j) noise + tau_j draft for all j in one batched
 * pass over prefix slot `slot`; endpoints a_j = x_j + (1 - tau_j) v_j;
 * D[j][i] = ||a_j[i] - draft[i]||_2. *accept_len = longest k with D[j][i] < delta
 * for all i < k and all j, forced to 0 when *gripper_switch = 1 (the gripper
 * channel changes sign between consecutive rows). dist_out (nullable) receives
 * D [n_tau][H]. Synchronous. Requires 1 <= n_tau <= max_taus. A time-modulated
 * expert (time_mode 1) conditions sequence j on tau_j alone: its layer and final-norm
 * modulation vectors are computed from temb(tau_j) at the start of the pass. */
int ae_verify(ae_handle* h, int slot, const float* draft, const float* noise, const float* taus, int n_tau,
              float delta, int* accept_len, int* gripper_switch, float* dist_out);

/* Same as ae_verify with device pointers for every array (d_dist_out
 * nullable), enqueued on `stream` (NULL = the library's stream). */
int ae_verify_async(ae_handle* h, int slot, const float* d_draft, const float* d_noise, const float* d_taus,
                    int n_tau, float delta, int* d_accept_len, int* d_gripper_switch, float* d_dist_out,
                    void* stream);

/* One round of the dual-path runtime ("Realtime-VLA FLASH" article, section 03:
 * dual-path inference and phase-aware fallback). The fast path is ae_verify of
 * `draft` on prefix slot `slot` at the n_tau flow times `taus` with the noise
 * `noise_verify` and threshold `delta`. When its accepted prefix is empty -- which
 * a gripper switch in the draft forces -- the round falls back to the full path:
 * the denoise loop of `steps` uniform Euler steps (as ae_denoise, for this slot)
 * from `noise_full`.
 * Host buffers: draft, noise_verify, noise_full, actions_out [H][A] fp32;
 * taus [n_tau]. actions_out receives the draft on the fast path (its first
 * *accept_len rows are the accepted ones) and the denoised chunk on the full
 * path; *full_path is 0 or 1. Synchronous: the host reads the verification's
 * decision before the full path is launched. ae_last_gpu_ms then covers the
 * round on the device timeline, from the verification's start to the end of
 * the last pass it ran (the host decision included). The first round of a
 * (n_tau, steps, slot) shape captures its graphs (slow). Errors as ae_verify,
 * plus AE_ERR_INVALID_ARG for steps outside 1..1000; on error the outputs are
 * not written. */
int ae_round(ae_handle* h, int slot, const float* draft, const float* noise_verify, const float* taus, int n_tau,
             float delta, const float* noise_full, int steps, float* actions_out, int* accept_len,
             int* gripper_switch, int* full_path);

/* The draft model's candidate chunk ("Realtime-VLA FLASH" article, section 03, draft action
 * generation) on a handle created with draft = 1. `features` is host [prefix_len][width] fp32:
 * the current image features, as tokens of the block's width. The block's sequence is
 * [features ; queries]: the features' K/V (RMSNorm ln1, k/v projections, K rotated at positions
 * 0..prefix_len-1) are written to prefix slot 0, then the query rows run the block at positions
 * prefix_len.. with every query attending to every feature and query, then final_ln and the
 * action head (action_out_w, action_out_b). chunk_out: host [horizon][action_dim] fp32.
 * Synchronous; ae_last_gpu_ms covers the device pass (features already uploaded). The first call
 * captures the graph. AE_ERR_UNSUPPORTED on a handle that is not a draft model. */
int ae_draft(ae_handle* h, const float* features, float* chunk_out);

/* The per-layer prefix KV cache from the prefix token embeddings, on a handle created with
 * prefill = 1 ("DM0.5" guide, section 5.1). emb: host [horizon][width] fp32. The handle's
 * decoder blocks run over the horizon tokens with every token attending to every token and RoPE
 * at positions 0..horizon-1. k_out, v_out: host [n_layers][horizon][n_kv_heads][head_dim] in
 * kv_dtype, K rotated -- the layout and convention ae_load_prefix_kv takes, for an expert whose
 * n_layers, n_kv_heads and head_dim match. Synchronous; ae_last_gpu_ms covers the device pass.
 * AE_ERR_UNSUPPORTED on a handle that is not a prefill stack. */
int ae_prefill(ae_handle* h, const float* emb, void* k_out, void* v_out);

/* ae_prefill with the cache left on the device: the prefill stack h runs over emb (host
 * [horizon][width] fp32) and its per-layer K/V are copied device to device into prefix slot
 * `slot` of the expert handle `expert` (the packed layout ae_load_prefix_kv builds; no host
 * round trip). The expert's prefix_len must equal h's horizon and its n_layers, n_kv_heads,
 * head_dim and kv_dtype must match h's, else AE_ERR_UNSUPPORTED; both handles on one device.
 * Marks the slot loaded. Synchronous (h's stream drained before return); ae_last_gpu_ms(h) covers
 * the prefill pass. */
int ae_prefill_to_slot(ae_handle* h, const float* emb, ae_handle* expert, int slot);

/* Free every device resource of the handle. NULL is a no-op. */
void ae_destroy(ae_handle* h);

/* Text of the last error on this handle ("" if none); h == NULL gives the
 * last ae_create failure of this thread. Valid until the next call. */
const char* ae_last_error(const ae_handle* h);

/* GPU time in ms of the last synchronous ae_denoise / ae_verify graph replay,
 * measured with HIP events around the launch on the library's stream. */
int ae_last_gpu_ms(const ae_handle* h, float* ms);

/* Per-kernel timing of one ae_denoise pass (mode bit 0 clear: slots
 * 0..batch-1, `steps` Euler steps) or one ae_verify pass (bit 0 set: the slot
 * and inputs of the last ae_verify call, batch = n_tau).
 *   bit 1 clear (isolated): for each kernel, a graph holding every launch of
 *     that kernel in the pass, back to back, is replayed `iters` times between
 *     two HIP events on the library's stream;
 *   bit 1 set (in place): the pass is launched eagerly in its normal order,
 *     `iters` times after one warm-up pass, with a start/stop event pair bound
 *     to every dispatch (hipExtLaunchKernel), so each launch is timed by its
 *     own execution in the cache state the full pass gives it.
 * Writes up to max_stats entries {kernel name, launches (per pass x iters),
 * total ms} in launch order and the number written to *n_stats. Leaves the
 * activation buffers in an unspecified state (the next call reinitialises them). */
typedef struct ae_kernel_stat {
  char name[48];
  int launches;
  float total_ms;
} ae_kernel_stat;
int ae_kernel_times(ae_handle* h, int mode, int batch, int steps, int iters, ae_kernel_stat* stats,
                    int max_stats, int* n_stats);

#ifdef __cplusplus
}
#endif
#endif /* AE_H_ */
