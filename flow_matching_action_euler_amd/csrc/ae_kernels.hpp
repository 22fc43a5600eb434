// Device code of the action-expert denoise loop for gfx950 (CDNA4).
//
// One Euler step of the suffix (DM0.5 guide, sections 5.2-5.3) runs as:
//   in_proj   : h = x W_in^T + b_in + temb(t)                      (tiny, FMA)
//   per layer : qkv  = rmsnorm(h) W_qkv^T, RoPE on q/k             (qkv_rope_kernel)      
//               attn = softmax(q [Kp;k]^T / sqrt(dh)) [Vp;v]        (attn_kernel + attn_merge)
//               h   += o W_o^T                                       (o_proj_resid_kernel)
//               u    = gelu(rmsnorm(h) W_g^T) * (rmsnorm(h) W_u^T)  (gate_up_geglu_kernel)  
//               h   += u W_d^T                                       (down_resid_kernel)
//   out_proj  : v = rmsnorm(h) W_out^T + b_out; x += dt v          (out_proj_euler_kernel)
//
// RMSNorm is never a pass of its own. A producer of h (in_proj or a
// residual epilogue) writes h in fp32, a copy hb = h * gain_next in the
// activation type, and per-16-channel partial sums of h^2. The consumer
// GEMM multiplies hb by its weights and scales each output row by
// 1/sqrt(sum/width + eps): rmsnorm(h) W^T = diag(1/rms) (h * g) W^T.
//
// Weights are packed at create time into MFMA lane order: tile (16 output
// rows) x k-block (32 inputs) is 64 lanes x 8 contiguous elements, lane l
// holding row l%16 and inputs (l/16)*8 .. +8, so one wave's 16-byte (bf16)
// or 8-byte (fp8) loads read one contiguous block. The same lane map feeds
// v_mfma_f32_16x16x32_bf16 (A = weights, B = activations^T); fp8 weights
// are widened to bf16 in registers (exact) and scaled per output row in the
// epilogue; fp32 weights use 8 v_mfma_f32_16x16x4f32, one per element slot.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ae {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

enum WType { WT_BF16 = 0, WT_FP8 = 1, WT_F32 = 2 };
enum AType { AT_BF16 = 0, AT_F32 = 1 };
enum Epi { EPI_QKV = 0, EPI_RESID = 1, EPI_GEGLU = 2, EPI_OUT = 3 };

constexpr int TOKG = 64;   // tokens per workgroup (4 MFMA column tiles of 16)

constexpr int KBLK = 32;   // inputs per k-block

// Activations passed between kernels (hb, o, u: M_pad tokens x K inputs) are stored in the
// MFMA B-operand order of the GEMM that reads them: [K/32][M_pad/16][64 lanes][8], lane =
// 16 * (k % 32 / 8) + token % 16, element k % 8 (bf16 and fp32 alike). A wave then loads
// each 16-token x 32-input fragment as one contiguous run straight into registers.
__device__ __forceinline__ size_t act_idx(int tok, int k, int ntt) {
  return ((((size_t)(k >> 5) * ntt + (tok >> 4)) * 64 + (((k & 31) >> 3) << 4) + (tok & 15)) << 3) + (k & 7);
}

// ------------------------------------------------------------------ small helpers

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  // round to nearest even (finite inputs)
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int AT> struct Act;
template <> struct Act<AT_BF16> {
  typedef uint16_t T;
  __device__ static __forceinline__ float ld(const T* p, size_t i) { return bf16_to_f32(p[i]); }
  __device__ static __forceinline__ void st(T* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};
template <> struct Act<AT_F32> {
  typedef float T;
  __device__ static __forceinline__ float ld(const T* p, size_t i) { return p[i]; }
  __device__ static __forceinline__ void st(T* p, size_t i, float v) { p[i] = v; }
};

__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint2 w) {
  f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false);
  f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
  f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false);
  f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
  // every E4M3 value is exact in bf16: keep the top 16 bits
  uint4 r;
  r.x = (__float_as_uint(a[0]) >> 16) | (__float_as_uint(a[1]) & 0xffff0000u);
  r.y = (__float_as_uint(b[0]) >> 16) | (__float_as_uint(b[1]) & 0xffff0000u);
  r.z = (__float_as_uint(c[0]) >> 16) | (__float_as_uint(c[1]) & 0xffff0000u);
  r.w = (__float_as_uint(d[0]) >> 16) | (__float_as_uint(d[1]) & 0xffff0000u);
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ float gelu_tanh(float x) {
  const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
  float u = k0 * (x + 0.044715f * x * x * x);
  return 0.5f * x * (1.0f + tanhf(u));
}
// The same function through 0.5 (1 + tanh u) = 1 / (1 + exp(-2u)): one exp2 and one reciprocal
// (relative error ~1e-6, far inside the bf16 rounding of its output)
__device__ __forceinline__ float gelu_tanh_fast(float x) {
  const float k2 = -2.f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
  const float e = __builtin_amdgcn_exp2f(k2 * (x + 0.044715f * x * x * x));
  return x * __builtin_amdgcn_rcpf(1.f + e);
}

// ------------------------------------------------------------------ L2 prefetch of the next kernel's operands
//
// A kernel's working set arrives from HBM about 2 us after it asks; the same
// bytes already in its XCD's L2 arrive in a fraction of that, and L2 contents
// survive kernel boundaries. A GEMM whose HBM traffic is over once its main
// loop is done (no split-K exchange follows) therefore touches, one dword per
// 128-byte line, what the next kernel will read while it reduces and runs its
// epilogue, placing each line in the L2 of the XCD where the consumer
// workgroup will run (workgroup i of a launch runs on XCD i % 8). A fixed
// number of touches per thread, no branch: unused slots reread a line of the
// kernel's own weights.
struct Prefetch {
  const char* base;         // kind 1: first region; kind 2: next kernel's packed weights
  const char* base2;        // kind 1: second region
  const char* dummy;        // a line this kernel reads anyway
  unsigned long long bytes; // kind 1: bytes of each region
  int kind;                 // 0: none, 1: whole regions into every XCD's L2, 2: next GEMM's weights
  int next_groups, next_S, NT, KB, frag_bytes;  // kind 2: next launch's tiling
  int kb_lead;              // kind 2: leading k-blocks of each tile's k-range to place (0: all)
};

// The touched values stay in registers until prefetch_done: combining them any earlier would
// make the wave wait for HBM at the next scheduling boundary (a barrier), mid-kernel.
template <int NL> struct PfVals { int v[NL]; };

template <int NL>
__device__ __forceinline__ PfVals<NL> prefetch_issue(const Prefetch& pf, unsigned wg, unsigned n_wg, unsigned tid, unsigned nthr) {
  const unsigned c8 = n_wg >= 8 ? n_wg / 8 : 1;  // this launch's workgroups per XCD
  const unsigned xcd = wg % 8, j0 = wg / 8;
  const bool wg_ok = pf.kind != 0 && wg < c8 * 8;
  PfVals<NL> out;
#pragma unroll
  for (int k = 0; k < NL; ++k) {
    const unsigned L = tid + nthr * k;  // this workgroup's k-th touch slot
    bool ok = wg_ok;
    const char* a1;
    if (pf.kind == 1) {  // every XCD gets every line: the c8 workgroups of an XCD interleave them
      const unsigned long long lines1 = pf.bytes / 128;
      const unsigned long long Lg = j0 + (unsigned long long)c8 * L;
      ok = ok && Lg < 2 * lines1;
      a1 = Lg < lines1 ? pf.base + Lg * 128 : pf.base2 + (Lg - lines1) * 128;
    } else {  // the lines of next-launch workgroups i = xcd + 8 (j0 + m c8), m = 0, 1, ...
      const unsigned kbs = pf.KB / max(pf.next_S, 1);
      const unsigned kbl = pf.kb_lead > 0 && (unsigned)pf.kb_lead < kbs ? (unsigned)pf.kb_lead : kbs;
      const unsigned lpt = max(kbl * pf.frag_bytes / 128, 1u);  // lines per tile range
      const unsigned lpw = max(pf.NT, 1) * lpt;                 // lines per next workgroup
      const unsigned m = L / lpw, r = L % lpw;
      const unsigned i = xcd + 8 * (j0 + m * c8);
      ok = ok && pf.kind == 2 && i < (unsigned)(pf.next_groups * pf.next_S);
      const unsigned g = i % max(pf.next_groups, 1), sp = i / max(pf.next_groups, 1);
      const unsigned long long off =
          ((unsigned long long)(g * pf.NT + r / lpt) * pf.KB + (unsigned long long)sp * kbs) * pf.frag_bytes +
          (unsigned long long)(r % lpt) * 128;
      a1 = pf.base + off;
    }
    out.v[k] = *(const int*)(ok ? a1 : pf.dummy);
  }
  return out;
}

// Consume the prefetch values (call once, at the end): forces their completion, nothing else.
template <int NL>
__device__ __forceinline__ void prefetch_done(const PfVals<NL>& p) {
  int acc = 0;
#pragma unroll
  for (int k = 0; k < NL; ++k) acc ^= p.v[k];
  asm volatile("" ::"v"(acc));
}

// ------------------------------------------------------------------ GEMM

struct GemmArgs {
  const void* w;        // packed weights [n_tiles][KB][64][8]
  const float* wscale;  // fp8: scale per packed channel (tile*16 + c); else null
  const void* x;        // activations in fragment order (act_idx), gain-scaled, not normalised
  const float* ssp_in;  // [g_in][M_pad] partial sums of h^2 (null: no RMS scaling)
  int g_in;
  float inv_width;      // 1 / width of the normalised vector
  float eps;
  int M, M_pad, K, S;   // rows, padded rows, inputs, k-splits
  int n_zt, zpw;        // 64-token groups in all, and per workgroup (grid z = ceil(n_zt / zpw); zpw = 1 if S > 1)
  int passes;           // k-passes per wave: K/32/S = passes * GW * KPW
  float* part;          // split-K partials [S][n_z][n_groups][NT*64*16], EXCH_EMPTY between launches
  unsigned* counters;   // [n_z][n_groups], zero between launches (arrival tickets)
  int exch_poll;        // 1: every workgroup is resident at once; split S-1 polls the others' partials
  int poll_delay;       // ~0.2 us steps split S-1 waits before its first poll (the partials' flight time)
  unsigned* err;        // set if a poll gave up (host-visible)
  unsigned long long wait;  // constant-clock ticks (100 MHz) a poll waits before it gives up
  // EPI_QKV
  void* q_out; void* k_out; void* v_out;   // attention operands in fragment order (see the attention section)
  const float* rope_cs;                    // [H][dh/2][2] cos, sin at positions P + t
  int n_q, n_kv, dh, H;
  int n_qt;                                // 16-row query tiles per (sequence, kv head)
  int nbs;                                 // 32-key suffix blocks per (sequence, kv head)
  // EPI_RESID
  float* h;              // [M_pad][N] residual, updated in place
  void* hb;              // h * gain_next for the next consumer, fragment order (act_idx)
  const float* gain_next;
  float* ssp_out;        // [N/16][M_pad]
  int N;                 // logical outputs
  // EPI_GEGLU
  void* u_out;           // fragment order (act_idx)
  // EPI_OUT
  const float* bias;     // [A]
  float* xio;            // denoise: x [M_pad][A] updated in place; verify: v out
  int A;
  float dt;              // > 0: x += dt * v; 0: store v
  // EPI_OUT of a verification pass (vx non-null; FLASH article, section 03, parallel verification):
  // the endpoints x + (1 - tau) v, their distances to the draft and the accepted length are formed here
  const float* vx;       // [n_tau * H][A] the interpolated points the velocities are taken at
  const float* draft;    // [H][A]
  const float* taus;     // [n_tau] (sequence j of the pass is flow time taus[j])
  const float* vparams;  // [0] = delta
  float* vpart;          // [ceil(A / 16)][M_pad] per 16-dim tile: sums of squared endpoint errors
  unsigned* vcount;      // arrival ticket, zero between launches
  int v_epi;             // epilogues of the launch (output tile groups x token groups)
  int gripper_dim;       // < 0: none
  float* dist;           // [n_tau][H] distances
  int* accept;           // accepted length
  int* gswitch;          // 1 when the draft's gripper column changes sign between rows
  Prefetch pf;           // next kernel's operands to place in L2 (QKV and gate/up launches only)
  int tn_blocks, tm_blocks;  // token-tiled launches: channel and token panels of the output
  // time-modulated expert and QK-norm (null when off; 64-token kernel only)
  const float* shift_bias;  // EPI_QKV / EPI_GEGLU: W . shift per packed channel, added after the 1/rms scaling
  const float* res_gate;    // EPI_RESID: gate per output channel on the sublayer's output
  const float* qk_gain;     // EPI_QKV: QK-norm gain per packed q/k channel (applied before RoPE)
  float* qk_ssp;            // EPI_QKV: [q and k tiles][M_pad] sums of squares of the q/k channels of a tile
  // modulation per sequence (a verification pass of a time-modulated expert: each flow time has its
  // own vectors): row r takes sequence r / mod_rows's vectors, ms_* elements apart; 0: one set for all
  int mod_rows;
  size_t ms_gain, ms_shift, ms_gate, ms_bias;
};

constexpr int GW = 8;         // waves per GEMM workgroup
constexpr int GTHREADS = GW * 64;

// Device-coherent publication of one value: the store writes through to the
// point of coherence (sc1), so workgroups on other XCDs read it without any
// L2 write-back or invalidation (a device-scope fence costs microseconds).
__device__ __forceinline__ void st_coherent(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ float ld_coherent(const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ unsigned ldu_coherent(const unsigned* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
// Wait until this thread's outstanding memory operations have completed.
__device__ __forceinline__ void wait_mem() { __builtin_amdgcn_s_waitcnt(0); }

// 16-byte device-coherent (sc1) buffer accesses: partials exchanged between
// workgroups of one launch, possibly on different XCDs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ void st16_coherent(__amdgpu_buffer_rsrc_t r, unsigned byte_off, float4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, byte_off, 0, 0x10);
}
__device__ __forceinline__ float ld_coherent_buf(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0x10));
}
__device__ __forceinline__ f32x4 ld16_coherent(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0x10));
}
__device__ __forceinline__ void st4_coherent(__amdgpu_buffer_rsrc_t r, unsigned byte_off, unsigned v) {
  __builtin_amdgcn_raw_buffer_store_b32((int)v, r, byte_off, 0, 0x10);
}

// Partials exchanged inside one launch (split-K tiles, attention key splits) go
// to buffers that hold EXCH_EMPTY in every word between launches. A consumer
// polls the words it needs until none holds it, so it sees each partial arrive
// in the data itself: the producer neither waits for its stores to be
// acknowledged nor takes a counter, which saves two dependent round trips
// across XCDs. The consumer then writes EXCH_EMPTY back over what it read
// (complete before the next launch starts). EXCH_EMPTY is a NaN that no
// arithmetic on finite inputs produces; a word is tested on its own, so a
// 16-byte store seen half-written still reads as not arrived.
constexpr unsigned EXCH_EMPTY = 0xffffffffu;
constexpr unsigned long long EXCH_WAIT = 2000000;  // default wait: constant-clock ticks (100 MHz: 20 ms) before a poll gives up
__device__ __forceinline__ bool exch_arrived(float v) { return __float_as_uint(v) != EXCH_EMPTY; }
__device__ __forceinline__ bool exch_arrived(f32x4 v) {
  return exch_arrived(v[0]) && exch_arrived(v[1]) && exch_arrived(v[2]) && exch_arrived(v[3]);
}
__device__ __forceinline__ void st16_empty(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
  __builtin_amdgcn_raw_buffer_store_b128(i32x4{-1, -1, -1, -1}, r, byte_off, 0, 0x10);
}


// One 16x16 tile x 32-input block of MFMA work in the lane map described above.
template <int WT, int AT> struct Frag;
template <int WT> struct Frag<WT, AT_BF16> {
  typedef bf16x8 A;
  typedef bf16x8 B;
  __device__ static __forceinline__ A load_a(const void* w, size_t blk, int lane) {
    if constexpr (WT == WT_FP8) return fp8x8_to_bf16x8(((const uint2*)w)[blk * 64 + lane]);
    else return __builtin_bit_cast(bf16x8, ((const uint4*)w)[blk * 64 + lane]);
  }
  __device__ static __forceinline__ B load_b(const uint16_t* p) { return __builtin_bit_cast(bf16x8, *(const uint4*)p); }
  __device__ static __forceinline__ f32x4 mma(const A& a, const B& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
struct f32x8 { float4 lo, hi; };
template <int WT> struct Frag<WT, AT_F32> {
  typedef f32x8 A;
  typedef f32x8 B;
  __device__ static __forceinline__ A load_a(const void* w, size_t blk, int lane) {
    const float4* p = (const float4*)w + (blk * 64 + lane) * 2;
    return A{p[0], p[1]};
  }
  __device__ static __forceinline__ B load_b(const float* p) { return B{((const float4*)p)[0], ((const float4*)p)[1]}; }
  __device__ static __forceinline__ f32x4 mma(const A& a, const B& b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.x, b.lo.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.y, b.lo.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.z, b.lo.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.w, b.lo.w, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.x, b.hi.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.y, b.hi.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.z, b.hi.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.w, b.hi.w, c, 0, 0, 0);
    return c;
  }
};

// LDS bytes of the GEMM kernels: the cross-wave reduction, the reduced tile,
// inverse RMS and RMS partials.
template <int AT, int NT, int KPW>
constexpr size_t gemm_lds_size() {
  // reduction tiles, summed tile, 1/rms, h^2 partials, ticket; at least 81 KB so that a compute
  // unit holds one workgroup and a launch of up to 256 workgroups spreads over all of them
  constexpr size_t need = (size_t)GW * NT * 1024 * 4 + (size_t)NT * 1024 * 4 + 64 * 4 + 512 * 4 + 16;
  return need > 81 * 1024 ? need : 81 * 1024;
}

// End of a verification pass (FLASH article, section 03: a prefix of the draft is accepted while every
// flow time reconstructs it within delta): each output-projection epilogue has stored, per 16-dim tile
// and row, the sum of squared endpoint errors with write-through stores; it counts its arrival, and
// the last one forms D[j][i] = sqrt(sum over tiles, in tile order), writes the distances, and takes the
// accepted length (first row rejected at some flow time: D >= delta or NaN; H when none, 0 when the
// draft's gripper column changes sign between two rows) and the switch flag with one ballot per wave.
// Rows up to GTHREADS; n_tau * H <= M.
__device__ __forceinline__ void verify_tail(const GemmArgs& a, unsigned* ticket, int* wsh) {
  wait_mem();  // this workgroup's partial stores have been acknowledged
  __syncthreads();
  if (threadIdx.x == 0) {
    *ticket = __hip_atomic_fetch_add(a.vcount, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (*ticket == (unsigned)a.v_epi - 1) __hip_atomic_store(a.vcount, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (*ticket != (unsigned)a.v_epi - 1) return;
  const int H = a.H, n_tau = a.M / H, n_tiles = (a.A + 15) / 16, i = threadIdx.x;
  const int lane = i & 63, wave = i >> 6;
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.vpart);
  const bool row = i < H;
  const int gd = a.gripper_dim;
  const bool g_row = gd >= 0 && i > 0 && row;
  const float g_cur = a.draft[g_row ? (size_t)i * a.A + gd : 0], g_prev = a.draft[g_row ? (size_t)(i - 1) * a.A + gd : 0];
  const float delta = a.vparams[0];
  bool bad = false;
  for (int j0 = 0; j0 < n_tau; j0 += 4) {
    float s[4][4];  // [flow time][tile]: every load of the group in flight before the sums
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bool in = row && j0 + q < n_tau && t < n_tiles;
        s[q][t] = ld_coherent_buf(rp, in ? (unsigned)((t * a.M_pad + (j0 + q) * H + i) * 4) : 0u);
      }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (row && j0 + q < n_tau) {
        float sum = s[q][0];
        for (int t = 1; t < n_tiles; ++t) sum += s[q][t];
        const float D = sqrtf(sum);
        a.dist[(size_t)(j0 + q) * H + i] = D;
        bad = bad || !(D < delta);
      }
  }
  const unsigned long long mb = __ballot(row && bad), mf = __ballot(g_row && g_cur * g_prev < 0.f);
  if (lane == 0) {
    wsh[wave] = mb ? wave * 64 + (__ffsll((long long)mb) - 1) : H;
    wsh[GW + wave] = mf != 0ull;
  }
  __syncthreads();
  if (i == 0) {
    int first = H, flip = 0;
    for (int w = 0; w < GW; ++w) {
      first = min(first, wsh[w]);
      flip |= wsh[GW + w];
    }
    *a.accept = flip ? 0 : first;
    *a.gswitch = flip;
  }
}

// Y = X W^T over the workgroup's channel tiles [g*NT, g*NT+NT), k-split s and
// token group z (64 rows), then the epilogue EPI. Block = 8 waves. In each
// pass wave w owns KPW consecutive k-blocks: it issues its weight fragments
// and the matching 4 x KPW activation fragments (each one contiguous run, see
// act_idx) straight into registers, then runs the MFMAs; no LDS staging.
// The 8 partial tiles are summed in LDS.
template <int WT, int AT, int EPI, int NT, int KPW, bool LOOP>
__device__ __forceinline__ void gemm_body(const GemmArgs& a) {
  typedef typename Act<AT>::T XT;
  typedef Frag<WT, AT> F;
  constexpr size_t REDB = (size_t)GW * NT * 1024 * 4;
  extern __shared__ __attribute__((aligned(16))) float smem[];  // no static LDS: keeps 16-byte accesses aligned
  float* red = smem;                                          // [GW][NT][64][16] cross-wave reduction
  float* res = (float*)((char*)smem + REDB);                  // [NT][64][16]
  float* inv_rms = res + NT * 1024;                           // [64]
  float* ssq8 = inv_rms + 64;                                 // [8][64]
  unsigned* ticket = (unsigned*)(ssq8 + 512);                 // split-K arrival ticket

  const int g = blockIdx.x, s = blockIdx.y;
  const int n_groups = gridDim.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int KB = a.K / KBLK;
  const bool has_ssp = a.ssp_in != nullptr;

  const int ntt = a.M_pad / 16;
  // pass p: wave w owns k-blocks kb0 .. kb0 + KPW
  auto issue_w = [&](int p, typename F::A (&wa)[NT][KPW]) {
    const int kb0 = s * (KB / a.S) + (p * GW + wave) * KPW;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int j = 0; j < KPW; ++j) wa[nt][j] = F::load_a(a.w, ((size_t)g * NT + nt) * KB + kb0 + j, lane);
  };
  // activation fragments of token group z, unconditional: the padding tokens of the last group
  // are in bounds (buffers hold M_pad rows) and only reach output columns that are never stored
  // (tokens are MFMA columns, nothing mixes across them); a per-lane condition here made the
  // compiler wait for each load before issuing the next
  auto issue_x = [&](int p, int z, typename F::B (&xb)[KPW][4]) {
    const int kb0 = s * (KB / a.S) + (p * GW + wave) * KPW;
    const XT* xg = (const XT*)a.x + ((size_t)z * 4 * 64 + lane) * 8;  // this lane's slot of token tile 4z
#pragma unroll
    for (int j = 0; j < KPW; ++j)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) xb[j][tt] = F::load_b(xg + ((size_t)(kb0 + j) * ntt + tt) * 512);
  };
  f32x4 acc[NT][4];
  auto compute = [&](const typename F::A (&wa)[NT][KPW], const typename F::B (&xb)[KPW][4]) {
#pragma unroll
    for (int j = 0; j < KPW; ++j)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt][tt] = F::mma(wa[nt][j], xb[j][tt], acc[nt][tt]);
  };

  PfVals<2> pf_acc{};
  // token group z (the zi-th of this workgroup); true when the workgroup has nothing more to do
  // (a split-K producer that handed over its partial)
  typename F::A wa0[NT][KPW];  // LOOP: the first pass's weights, kept for every token group
  auto group = [&](const int z, const int zi) __attribute__((always_inline)) -> bool {
    const int tok0 = z * TOKG;
    // epilogue operands of this workgroup's channels (reloaded per token group: L2 hits)
    float gn[2 * NT];  // EPI_RESID: next gain; EPI_OUT: bias
#pragma unroll
    for (int i = 0; i < 2 * NT; ++i) {
      const int e = threadIdx.x + GTHREADS * i;
      const int n = (int)((size_t)g * NT + (e >> 10)) * 16 + (e & 15);
      const int sq = a.mod_rows ? min(tok0 + ((e >> 4) & 63), a.M - 1) / a.mod_rows : 0;
      gn[i] = 0.f;
      if constexpr (EPI == EPI_RESID) gn[i] = a.gain_next[sq * a.ms_gain + n];
      else if constexpr (EPI == EPI_OUT) gn[i] = a.bias[sq * a.ms_bias + (n < a.A ? n : 0)];
    }
    // fp8 weights: the per-row scale of each epilogue element, loaded now
    float psc[2 * NT];
#pragma unroll
    for (int i = 0; i < 2 * NT; ++i) {
      const int e = threadIdx.x + GTHREADS * i;
      psc[i] = WT == WT_FP8 ? a.wscale[((size_t)g * NT + (e >> 10)) * 16 + (e & 15)] : 1.f;
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) acc[nt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // partial sums of h^2 (thread -> token t & 63, groups (t >> 6) + 8 i), the residual or x
    // (element e = t + 512 i -> (nt = e / 1024, token (e / 16) % 64, channel e % 16)) and the
    // RoPE (cos, sin) of the 8 head dims this thread rotates (thread -> token (t >> 1) % 64,
    // pair g % (dh/16); threads past 128 repeat addresses: L1 hits): loaded right after the
    // first pass's activations (loads retire in order, so the MFMAs do not wait for them). The
    // loads are unconditional (clamped or fallback addresses, masked at use): a conditional load
    // let the compiler wait for it before the main loads were issued, and so did a 64-bit offset
    // product for ssv (its register pair overlapped a load in flight), hence 32-bit offsets there.
    float ssv[8];
    const float* sp = has_ssp ? a.ssp_in + tok0 + (threadIdx.x & 63) : (const float*)a.w;
    float pre0[2 * NT];  // EPI_RESID: h; EPI_OUT: x (denoise), the interpolated point (verification)
    float vom[2 * NT], vdr[2 * NT];  // verification: 1 - tau of the row's sequence, the draft's value
    float4 cs_pre[4];
    {
      typename F::A wa[NT][KPW];
      typename F::B xb[KPW][4];
      if constexpr (!LOOP) issue_w(0, wa);
      issue_x(0, z, xb);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int gi = (threadIdx.x >> 6) + 8 * i;
        ssv[i] = sp[(has_ssp && gi < a.g_in) ? gi * a.M_pad : 0];
      }
#pragma unroll
      for (int i = 0; i < 2 * NT; ++i) {
        const int e = threadIdx.x + GTHREADS * i;
        const int tok = min(tok0 + ((e >> 4) & 63), a.M - 1);
        const int n = (int)((size_t)g * NT + (e >> 10)) * 16 + (e & 15);
        pre0[i] = 0.f;
        if constexpr (EPI == EPI_RESID) pre0[i] = a.h[(size_t)tok * a.N + n];
        else if constexpr (EPI == EPI_OUT) {
          const bool ver = a.vx != nullptr;
          const int nn = n < a.A ? n : 0;
          const float* xs = a.dt > 0.f ? a.xio : ver ? a.vx : a.bias;
          pre0[i] = xs[xs == a.bias ? 0 : (size_t)tok * a.A + nn];
          vom[i] = 1.f - (ver ? a.taus : a.bias)[ver ? tok / a.H : 0];
          vdr[i] = (ver ? a.draft : a.bias)[ver ? (size_t)(tok % a.H) * a.A + nn : 0];
        }
      }
      if constexpr (EPI == EPI_QKV) {
        const int tok = min(tok0 + ((threadIdx.x >> 1) & (TOKG - 1)), a.M - 1);
        const float4* csp = (const float4*)a.rope_cs + ((size_t)(tok % a.H) * (a.dh / 2) + (g % (a.dh / 16)) * 8) / 2;
#pragma unroll
        for (int j = 0; j < 4; ++j) cs_pre[j] = csp[j];
      }
      __builtin_amdgcn_sched_barrier(0);  // every load of the pass in flight before the first MFMA
      if constexpr (LOOP) compute(wa0, xb);
      else compute(wa, xb);
    }
    for (int p = 1; p < a.passes; ++p) {
      typename F::A wa[NT][KPW];
      typename F::B xb[KPW][4];
      issue_w(p, wa);
      issue_x(p, z, xb);
      __builtin_amdgcn_sched_barrier(0);
      compute(wa, xb);
    }

    // next kernel's operands into L2 while this one reduces and runs its epilogue (no
    // split-K exchange in these roles, so nothing below waits on memory before the end)
    if constexpr (EPI == EPI_QKV || EPI == EPI_GEGLU)
      if (zi == 0)
        pf_acc = prefetch_issue<2>(a.pf, blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z),
                                   gridDim.x * gridDim.y * gridDim.z, threadIdx.x, GTHREADS);
    float ssq = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ssq += (has_ssp && (int)(threadIdx.x >> 6) + 8 * i < a.g_in) ? ssv[i] : 0.f;
    if (a.ssp_in != nullptr)
      for (int gi = (threadIdx.x >> 6) + 64; gi < a.g_in; gi += 8) ssq += sp[(size_t)gi * a.M_pad];  // width > 1024
    // cross-wave reduction: red[wave][nt][tt][channel quad][token % 16][4], so the 16 lanes of a
    // write phase cover 256 consecutive bytes (no bank conflicts); res is [nt][token][channel]
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        *(f32x4*)(red + ((((wave * NT + nt) * 4 + tt) * 4 + (lane >> 4)) * 16 + (lane & 15)) * 4) = acc[nt][tt];
    ssq8[threadIdx.x] = ssq;
    __syncthreads();
    // NT * 256 quads over 512 threads; quad qd = ((nt * 4 + tt) * 4 + cq) * 16 + t
#pragma unroll
    for (int i = 0; i < (NT + 1) / 2; ++i) {
      const int qd = threadIdx.x + GTHREADS * i;
      if (qd < NT * 256) {
        f32x4 sum = *(const f32x4*)(red + qd * 4);
#pragma unroll
        for (int w = 1; w < GW; ++w) sum += *(const f32x4*)(red + w * NT * 1024 + qd * 4);
        const int nt = qd >> 8, tt = (qd >> 6) & 3, cq = (qd >> 4) & 3, t = qd & 15;
        *(f32x4*)(res + nt * 1024 + (tt * 16 + t) * 16 + cq * 4) = sum;
      }
    }
    if (threadIdx.x < TOKG) {
      float r = 1.f;
      if (a.ssp_in != nullptr) {
        float t8 = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) t8 += ssq8[q * 64 + threadIdx.x];
        r = rsqrtf(t8 * a.inv_width + a.eps);
      }
      inv_rms[threadIdx.x] = r;
    }
    __syncthreads();

    if (a.S > 1) {  // one token group (zpw = 1)
      const int n_z = a.n_zt;
      const int tile_elems = NT * 1024;
      const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.part);
      auto poff = [&](int ss, int qd) {
        return (unsigned)(((((size_t)ss * n_z + z) * n_groups + g) * tile_elems + qd * 4) * 4);
      };
      if (a.exch_poll) {
        // split-K, all workgroups resident: splits 0..S-2 publish their partial write-through and
        // leave; split S-1 (the highest workgroup ids of the tile) adds them as they land, in split
        // order (deterministic), and empties them
        if (s != a.S - 1) {
#pragma unroll
          for (int i = 0; i < (NT + 1) / 2; ++i) {
            const int qd = threadIdx.x + GTHREADS * i;
            if (qd < NT * 256) st16_coherent(rp, poff(s, qd), *(const float4*)(res + qd * 4));
          }
          // this workgroup's HBM reads are over while split S-1 still merges: place the next
          // GEMM's weights in L2 (producers are workgroup ids below n_groups * (S-1) * n_z)
          if (a.pf.kind == 2)
            prefetch_done(prefetch_issue<2>(a.pf, blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z),
                                            gridDim.x * (gridDim.y - 1) * gridDim.z, threadIdx.x, GTHREADS));
          return true;
        }
        bool gave_up = false;
        for (int d = 0; d < a.poll_delay; ++d) __builtin_amdgcn_s_sleep(8);
#pragma unroll
        for (int i = 0; i < (NT + 1) / 2; ++i) {
          const int qd = threadIdx.x + GTHREADS * i;
          if (qd < NT * 256) {
            f32x4 v[3];
            const unsigned long long t_end = wall_clock64() + a.wait;
            for (;;) {
              bool ok = true;
#pragma unroll
              for (int ss = 0; ss < 3; ++ss) {
                v[ss] = ss < a.S - 1 ? ld16_coherent(rp, poff(ss, qd)) : f32x4{0.f, 0.f, 0.f, 0.f};
                ok = ok && exch_arrived(v[ss]);
              }
              if (ok) break;
              if (wall_clock64() > t_end) { gave_up = true; break; }
              __builtin_amdgcn_s_sleep(1);
            }
            const f32x4 own = *(const f32x4*)(res + qd * 4);
            const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
            f32x4 sum = v[0] + (a.S == 2 ? own : v[1]);
            sum = sum + (a.S == 3 ? own : v[2]);
            sum = sum + (a.S == 4 ? own : zero);
            *(f32x4*)(res + qd * 4) = sum;
#pragma unroll
            for (int ss = 0; ss < 3; ++ss)
              if (ss < a.S - 1) st16_empty(rp, poff(ss, qd));
          }
        }
        if (gave_up) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __syncthreads();
      } else {
        // split-K, more workgroups than fit at once: publish the partial, count arrivals; the
        // last arriver of (z, g) sums the S partials in split order and empties them
#pragma unroll
        for (int i = 0; i < (NT + 1) / 2; ++i) {
          const int qd = threadIdx.x + GTHREADS * i;
          if (qd < NT * 256) st16_coherent(rp, poff(s, qd), *(const float4*)(res + qd * 4));
        }
        wait_mem();
        __syncthreads();
        unsigned* cnt = a.counters + z * n_groups + g;
        if (threadIdx.x == 0) {
          *ticket = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (*ticket == (unsigned)a.S - 1) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (*ticket != (unsigned)a.S - 1) return true;
#pragma unroll
        for (int i = 0; i < (NT + 1) / 2; ++i) {
          const int qd = threadIdx.x + GTHREADS * i;
          if (qd < NT * 256) {
            f32x4 v[4];
#pragma unroll
            for (int ss = 0; ss < 4; ++ss)
              v[ss] = ss < a.S ? ld16_coherent(rp, poff(ss, qd)) : f32x4{0.f, 0.f, 0.f, 0.f};
            *(f32x4*)(res + qd * 4) = ((v[0] + v[1]) + v[2]) + v[3];
#pragma unroll
            for (int ss = 0; ss < 4; ++ss)
              if (ss < a.S) st16_empty(rp, poff(ss, qd));
          }
        }
        __syncthreads();
      }
    }

    if constexpr (EPI == EPI_QKV) {
      // q and k tiles: thread -> (token, half of the tile's 16 channels) = 8 consecutive head dims,
      // rotated and stored as one 16-byte run of a fragment row
      const int tiles_per_head = a.dh / 16, half = a.dh / 2;
      const int q_tiles = a.n_q * tiles_per_head, k_tiles = a.n_kv * tiles_per_head;
      const int t_in = (int)g;  // one tile per workgroup
      if (t_in < q_tiles + k_tiles) {
        const int tl = threadIdx.x >> 1, hf = threadIdx.x & 1, tok = tok0 + tl;
        if (threadIdx.x < 2 * TOKG && tok < a.M) {
          const bool is_q = t_in < q_tiles;
          const int tt2 = is_q ? t_in : t_in - q_tiles;
          const int head = tt2 / tiles_per_head, pair = tt2 % tiles_per_head;
          const int sq = tok / a.H, t = tok % a.H;
          const float ir = inv_rms[tl];
          const float* rr = res + tl * 16;
          float xs[16];  // the tile's 16 channels of this token: dims pair*8 + c, then + dh/2
#pragma unroll
          for (int c = 0; c < 16; ++c) xs[c] = rr[c] * ir;
          if (a.shift_bias) {
            const float* sb = a.shift_bias + (a.mod_rows ? (size_t)(tok / a.mod_rows) * a.ms_shift : 0) + t_in * 16;
#pragma unroll
            for (int c = 0; c < 16; ++c) xs[c] += sb[c];
          }
          if (a.qk_gain) {  // QK-norm: this tile's share of the head's sum of squares, then the gains
            float sq2 = 0.f;
#pragma unroll
            for (int c = 0; c < 16; ++c) sq2 += xs[c] * xs[c];
            if (hf == 0) a.qk_ssp[(size_t)t_in * a.M_pad + tok] = sq2;
#pragma unroll
            for (int c = 0; c < 16; ++c) xs[c] *= a.qk_gain[t_in * 16 + c];
          }
          float out[8];
#pragma unroll
          for (int j = 0; j < 8; j += 2) {
            const float4 cs2 = cs_pre[j / 2];  // (cos, sin) of dims pair*8 + j and + j + 1
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const float cs_c = u ? cs2.z : cs2.x, cs_s = u ? cs2.w : cs2.y;
              const float x1 = xs[j + u], x2 = xs[8 + j + u];  // dims d and d + dh/2
              out[j + u] = hf ? x1 * cs_s + x2 * cs_c : x1 * cs_c - x2 * cs_s;
            }
          }
          const int dfull = hf * half + pair * 8;
          const int nkb = a.dh / KBLK, lgrp = ((dfull % KBLK) >> 3) << 4, kb = dfull / KBLK;
          size_t off;
          if (is_q) {  // query B fragments: row r = j*H + t of the tile, dims kb*32 + (lane/16)*8
            const int gq = a.n_q / a.n_kv, gg = head / gq, r = (head % gq) * a.H + t;
            off = ((((size_t)sq * a.n_kv + gg) * a.n_qt + r / 16) * nkb + kb) * 512 + (lgrp + (r & 15)) * 8;
          } else {     // key A fragments of 32-key block t/32, keys in the order the attention expects
            const int kk = t & 31, kt = (kk & 7) >> 2, m = 4 * (kk >> 3) + (kk & 3);
            off = (((((size_t)sq * a.n_kv + head) * a.nbs + (t >> 5)) * 2 + kt) * nkb + kb) * 512 + (lgrp + m) * 8;
          }
          XT* dst = (XT*)(is_q ? a.q_out : a.k_out) + off;
          if constexpr (AT == AT_BF16) {
            uint4 v;
            v.x = (uint32_t)f32_to_bf16(out[0]) | ((uint32_t)f32_to_bf16(out[1]) << 16);
            v.y = (uint32_t)f32_to_bf16(out[2]) | ((uint32_t)f32_to_bf16(out[3]) << 16);
            v.z = (uint32_t)f32_to_bf16(out[4]) | ((uint32_t)f32_to_bf16(out[5]) << 16);
            v.w = (uint32_t)f32_to_bf16(out[6]) | ((uint32_t)f32_to_bf16(out[7]) << 16);
            *(uint4*)dst = v;
          } else {
            ((float4*)dst)[0] = make_float4(out[0], out[1], out[2], out[3]);
            ((float4*)dst)[1] = make_float4(out[4], out[5], out[6], out[7]);
          }
        }
        return false;
      }
    }
    // ---------------- epilogues: element e -> (nt = e / 1024, token tl = (e / 16) % 64, channel c = e % 16)
#pragma unroll
    for (int i = 0; i < 2 * NT; ++i) {
      const int e = threadIdx.x + GTHREADS * i;
      const int nt = e >> 10, tl = (e >> 4) & 63, c = e & 15;
      const size_t tile = (size_t)g * NT + nt;
      const int tok = tok0 + tl;
      const bool valid = tok < a.M;
      if constexpr (EPI == EPI_GEGLU) {
        if (nt & 1) continue;
      }
      const size_t msq = a.mod_rows ? (size_t)(min(tok, a.M - 1) / a.mod_rows) : 0;  // modulation set of this row
      float val = res[e] * inv_rms[tl];
      if constexpr (WT == WT_FP8) val *= psc[i];
      if constexpr (EPI == EPI_QKV || EPI == EPI_GEGLU)
        if (a.shift_bias) val += a.shift_bias[msq * a.ms_shift + tile * 16 + c];
      if constexpr (EPI == EPI_QKV) {
        // v tiles only (q and k tiles took the vectorised path above): value A fragments (of V^T)
        // of block t/32: dims dt*16 + lane%16, keys (lane/16)*8 + e
        const int col = ((int)tile - (a.n_q + a.n_kv) * (a.dh / 16)) * 16 + c;
        if (valid) {
          const int sq = tok / a.H, t = tok % a.H, hd = col / a.dh, d = col % a.dh, kk = t & 31;
          const size_t fr = ((((size_t)sq * a.n_kv + hd) * a.nbs + (t >> 5)) * (a.dh / 16) + d / 16);
          Act<AT>::st((XT*)a.v_out, fr * 512 + (((kk >> 3) << 4) + (d & 15)) * 8 + (kk & 7), val);
        }
      } else if constexpr (EPI == EPI_RESID) {
        const int n = (int)tile * 16 + c;
        float hn = 0.f;
        if (valid) {
          hn = pre0[i] + (a.res_gate ? a.res_gate[msq * a.ms_gate + n] * val : val);
          a.h[(size_t)tok * a.N + n] = hn;
          Act<AT>::st((XT*)a.hb, act_idx(tok, n, a.M_pad / 16), hn * gn[i]);
        }
        float sq = hn * hn;
        sq += __shfl_xor(sq, 1, 16);
        sq += __shfl_xor(sq, 2, 16);
        sq += __shfl_xor(sq, 4, 16);
        sq += __shfl_xor(sq, 8, 16);
        if (c == 0) a.ssp_out[tile * a.M_pad + tok] = sq;
      } else if constexpr (EPI == EPI_GEGLU) {
        float up = res[e + 1024] * inv_rms[tl];
        if constexpr (WT == WT_FP8) up *= psc[(i + 2) & (2 * NT - 1)];  // the up tile of this gate element
        if (a.shift_bias) up += a.shift_bias[msq * a.ms_shift + (tile + 1) * 16 + c];
        const int f = (int)(tile / 2) * 16 + c;
        if (valid) Act<AT>::st((XT*)a.u_out, act_idx(tok, f, a.M_pad / 16), gelu_tanh(val) * up);
      } else {  // EPI_OUT: bias (gn) and x (pre0) were loaded before the MFMAs
        const int n = (int)tile * 16 + c;
        const float v = val + gn[i];
        if (valid && n < a.A) a.xio[(size_t)tok * a.A + n] = a.dt > 0.f ? pre0[i] + a.dt * v : v;
        if (a.vx) {  // the squared endpoint error summed over the tile's 16 dims (16 lanes), device-scope
          float d2 = 0.f;
          if (valid && n < a.A) {
            const float d = pre0[i] + vom[i] * v - vdr[i];
            d2 = d * d;
          }
          d2 += __shfl_xor(d2, 1, 16);
          d2 += __shfl_xor(d2, 2, 16);
          d2 += __shfl_xor(d2, 4, 16);
          d2 += __shfl_xor(d2, 8, 16);
          if (c == 0 && valid)
            st4_coherent(make_rsrc(a.vpart), (unsigned)((tile * a.M_pad + tok) * 4), __float_as_uint(d2));
        }
      }
    }
    if constexpr (EPI == EPI_OUT) {
      if (a.vx) verify_tail(a, ticket, (int*)red);
    }
    return false;
  };
  // The passes below reach the weight panel (this workgroup's channel tiles, the k-range of split s)
  // one pass at a time, each waiting out HBM for the lines it is the first on its XCD to read. The
  // workgroups of the gridDim.z token-group rows share the panel (on one XCD: the row stride is a
  // multiple of 8 when n_groups * S is); each first touches its share of the panel's lines, one dword
  // per 128-byte line, at most two loads per thread, consumed at the end (loads complete in order: the
  // first pass's wait covers them). Only with several token-group rows (verification: o_proj 7.1 ->
  // 6.7 us, down 10.7 -> 10.0 us): with one (batch-1 passes) the touches duplicate the previous
  // kernel's L2 placement of these weights and made the launch-per-phase chunk 6.94 -> 7.33 ms.
  int tch[2] = {0, 0};
  if (gridDim.z > 1) {
    constexpr size_t FB = WT == WT_FP8 ? 512 : WT == WT_F32 ? 2048 : 1024;  // bytes per fragment
    const int kbs = KB / a.S;
    const unsigned lpt = (unsigned)(kbs * FB / 128), wl = NT * lpt;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const unsigned L = blockIdx.z + gridDim.z * (threadIdx.x + GTHREADS * i);
      if (L < wl)
        tch[i] = *(const int*)((const char*)a.w + (((size_t)g * NT + L / lpt) * KB + (size_t)s * kbs) * FB +
                               (size_t)(L % lpt) * 128);
    }
  }
  // LOOP = false: one token group per workgroup (zpw = 1) in straight-line code: at a loop head
  // the compiler waits for every load in flight, which would hold up the first pass
  if constexpr (LOOP) {
    // the first group peeled off, so that its MFMAs wait for their own loads only
    const int z0 = blockIdx.z * a.zpw;  // < n_zt: the grid holds ceil(n_zt / zpw) rows
    issue_w(0, wa0);
    if (!group(z0, 0))
      for (int zi = 1; zi < a.zpw; ++zi) {
        const int z = z0 + zi;
        if (z >= a.n_zt || group(z, zi)) break;
      }
  } else if (group(blockIdx.z, 0)) {
    asm volatile("" ::"v"(tch[0] ^ tch[1]));
    return;
  }
  asm volatile("" ::"v"(tch[0] ^ tch[1]));
  prefetch_done(pf_acc);
}

// One entry point per role, so that profiles name the phase: same body,
// the epilogue and tiles-per-workgroup fixed by the role.
enum Role { R_QKV_ROPE = 0, R_O_PROJ = 1, R_GATE_UP = 2, R_DOWN = 3, R_OUT_PROJ = 4 };
template <int ROLE> struct RoleTraits;
template <> struct RoleTraits<R_QKV_ROPE> { static constexpr int EPI = EPI_QKV, NT = 1; };
template <> struct RoleTraits<R_O_PROJ> { static constexpr int EPI = EPI_RESID, NT = 1; };
template <> struct RoleTraits<R_GATE_UP> { static constexpr int EPI = EPI_GEGLU, NT = 2; };
template <> struct RoleTraits<R_DOWN> { static constexpr int EPI = EPI_RESID, NT = 1; };
template <> struct RoleTraits<R_OUT_PROJ> { static constexpr int EPI = EPI_OUT, NT = 1; };

#define AE_GEMM_ENTRY(NAME, ROLE)                                                                         \
  template <int WT, int AT, int KPW, bool LOOP>                                                           \
  __global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(1, 2))) void NAME(GemmArgs a) {   \
    gemm_body<WT, AT, RoleTraits<ROLE>::EPI, RoleTraits<ROLE>::NT, KPW, LOOP>(a);                        \
  }
AE_GEMM_ENTRY(qkv_rope_kernel, R_QKV_ROPE)
AE_GEMM_ENTRY(o_proj_resid_kernel, R_O_PROJ)
AE_GEMM_ENTRY(gate_up_geglu_kernel, R_GATE_UP)
AE_GEMM_ENTRY(down_resid_kernel, R_DOWN)
AE_GEMM_ENTRY(out_proj_euler_kernel, R_OUT_PROJ)
#undef AE_GEMM_ENTRY

template <int ROLE, int WT, int AT, int KPW, bool LOOP>
constexpr void (*gemm_entry())(GemmArgs) {
  if constexpr (ROLE == R_QKV_ROPE) return qkv_rope_kernel<WT, AT, KPW, LOOP>;
  else if constexpr (ROLE == R_O_PROJ) return o_proj_resid_kernel<WT, AT, KPW, LOOP>;
  else if constexpr (ROLE == R_GATE_UP) return gate_up_geglu_kernel<WT, AT, KPW, LOOP>;
  else if constexpr (ROLE == R_DOWN) return down_resid_kernel<WT, AT, KPW, LOOP>;
  else return out_proj_euler_kernel<WT, AT, KPW, LOOP>;
}

// ------------------------------------------------------------------ GEMM, many tokens

// For a few hundred tokens and more (verification passes, batched robots, prefill) a workgroup
// owns an output tile of TN = 64*WN channels x TM = 64*WM tokens, so that each operand byte it
// brings in feeds TM (weights) or TN (activations) outputs; the kernel above re-reads every
// activation in each 16- or 32-channel group. The 8 waves are WN x WM x WK: wave (wn, wm, wk)
// accumulates the 64 x 64 sub-tile (wn, wm) (4 x 4 MFMA tiles) over the k-blocks of its k-group
// wk (one k-block of each chunk); with WK > 1 the partial sub-tiles meet in LDS and each wave
// finishes 1/WK of the tiles. Operands go from global memory straight into LDS as whole fragments
// in the packed order (lane-major, so fragment reads are conflict-free), several chunks in flight;
// each wave holds the fragments of two chunks in registers, so the MFMAs of one chunk run while the
// next chunk's fragments are read. bf16 activations; bf16 weights, or E4M3 weights (the MLP roles)
// kept as bytes in LDS (512-byte fragments), widened to bf16 (exact) after the fragment read and
// scaled per output channel in the epilogue. (Staging through registers and LDS stores, the form
// this replaced, cost the prefill 4%: 6.73 -> 6.44 ms per pass once its E4M3 weights loaded direct.)
template <int WN, int WM, int WK>
struct TileCfg {
  static_assert(WN * WM * WK == GW, "8 waves");
  static constexpr int NT = 4 * WN, MT = 4 * WM;                   // 16-channel, 16-token tiles
  static constexpr int CK = WK;                                    // k-blocks per chunk: one per k-group
  static constexpr int NA = NT * CK, NB = MT * CK;                 // fragments per chunk
  static constexpr int LOADS = (NA + NB) / GW;                     // 16-byte loads per thread
  static constexpr size_t CHUNK = (size_t)(NA + NB) * 1024;
  // shapes that share fragments between waves stage them in LDS; with bf16 weights NBUF chunk
  // buffers are filled straight from global memory, NBUF - 1 chunks in flight
  static constexpr bool SHARED = !(WN == 1 && WM == 1);
  static constexpr int NBUF = !SHARED ? 2 : (int)((144 * 1024) / CHUNK) < 3 ? 3 : (int)((144 * 1024) / CHUNK);
  // operand buffers; with WK > 1 they then hold the 8 waves' partial sub-tiles (16 KB each)
  static constexpr size_t OPER = (size_t)NBUF * CHUNK > 2 * CHUNK ? (size_t)NBUF * CHUNK : 2 * CHUNK;
  static constexpr size_t STAGE = WK > 1 && OPER < (size_t)GW * 16384 ? (size_t)GW * 16384 : OPER;
  static constexpr int GPT = GTHREADS / (MT * 16);                 // RMS partial groups per token
  static constexpr int NRD = 64 / GPT;                             // RMS partial loads per thread
  static constexpr size_t LDS = STAGE + (size_t)MT * 16 * 4 + GTHREADS * 4;
  static_assert(NA % GW == 0 && NB % GW == 0 && 2 * CHUNK <= 128 * 1024 && LDS <= 160 * 1024, "chunk shape");
};
constexpr int TILED_MAX_GIN = 128;  // RMS partial groups the prologue reads (width <= 2048)
template <int WT> struct TiledWReg { typedef i32x4 T; };   // one lane's share of a weight fragment
template <> struct TiledWReg<WT_FP8> { typedef i32x2 T; };

// Wait until at most N of this wave's vector memory operations are outstanding and its LDS
// operations are done, then meet the workgroup. Loads return in order, so this waits for every
// load but the N youngest, including loads that write LDS directly.
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int EPI, int WN, int WM, int WK, int WT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(1, 2))) void gemm_tiled_kernel(GemmArgs a) {
  typedef TileCfg<WN, WM, WK> C;
  typedef typename TiledWReg<WT>::T WR;
  static_assert(WT == WT_BF16 || (WT == WT_FP8 && EPI != EPI_QKV), "E4M3 weights: MLP roles");
  constexpr int LW = C::NA / GW, LX = C::NB / GW;  // weight / activation loads per thread
  // E4M3 weight fragments stay 512-byte runs in LDS (widened to bf16 after the fragment read):
  // a quarter fewer LDS bytes stored and read per step than widening them before the store
  constexpr size_t AFB = WT == WT_FP8 ? 512 : 1024, CHUNKB = (size_t)C::NA * AFB + (size_t)C::NB * 1024;
  extern __shared__ __attribute__((aligned(16))) float smem[];
  char* stage = (char*)smem;                                  // [2][CHUNK] operands; then partials
  float* inv_rms = (float*)(stage + C::STAGE);                // [TM]
  float* ssq = inv_rms + C::MT * 16;                          // [512]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;  // wave: scalar
  const int wk = wave % WK, wn = (wave / WK) % WN, wm = wave / (WK * WN);
  const int KB = a.K / KBLK, ntt = a.M_pad / 16;

  // workgroup i runs on XCD i % 8: each XCD takes a contiguous run of output tiles in
  // channel-major order, so the workgroups that share a weight panel share one L2
  const int T = a.tn_blocks * a.tm_blocks;
  const int xcd = blockIdx.x & 7;
  const int item = xcd * (T >> 3) + min(xcd, T & 7) + (int)(blockIdx.x >> 3);
  const int nb = item / a.tm_blocks, mb = item % a.tm_blocks;
  const int ct0 = nb * C::NT, tt0 = mb * C::MT;  // first 16-channel tile, first 16-token tile

  // The chunk loads below reach each line of the operand panels one chunk at a time, and the first
  // reader of a line on this XCD waits out HBM (or another XCD's write-back). In the one-tile shape
  // (o_proj, down) the workgroups sharing this weight panel (one per token panel, rank mb) and this
  // activation panel (one per channel panel, rank nb) therefore first touch their share of it, one
  // dword per 128-byte line, at most two loads per thread each, when the panel is small enough to
  // stay in L2 (512 KB); the values are consumed after the loop (loads complete in order: the first
  // chunk's wait covers them). Measured at batch 16: o_proj 12.5 -> 11.6 us, down 19.9 -> 18.3 us;
  // the shapes that stage shared fragments in LDS got slower with it (gate/up 19.0 -> 20.8 us).
  int tch[4] = {0, 0, 0, 0};
  if constexpr (!C::SHARED) {
    constexpr size_t AFB_ = WT == WT_FP8 ? 512 : 1024;
    const unsigned wl = (unsigned)((size_t)C::NT * KB * AFB_ / 128);  // weight panel lines, contiguous
    const char* wpan = (const char*)a.w + (size_t)ct0 * KB * AFB_;
    if (wl <= 4096) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const unsigned L = mb + a.tm_blocks * (threadIdx.x + GTHREADS * i);
        if (L < wl) tch[i] = *(const int*)(wpan + (size_t)L * 128);
      }
    }
    // activation panel: per k-block a run of MT 1 KB fragments (token tiles tt0 .. ntt - 1 of it exist)
    const int mt_ok = min(C::MT, ntt - tt0);
    const unsigned rl = (unsigned)mt_ok * 8, xl = rl * KB;
    if (xl <= 4096) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const unsigned L = nb + a.tn_blocks * (threadIdx.x + GTHREADS * i);
        if (L < xl)
          tch[2 + i] = *(const int*)((const char*)a.x + ((size_t)(L / rl) * ntt + tt0) * 1024 + (size_t)(L % rl) * 128);
      }
    }
  }

  // weight fragments [ct][kk] and activation fragments [kk][tt] of the packed operands; the token
  // tiles past the buffer's rows read its last tile (their outputs are never stored)
  const WR* wsrc = (const WR*)a.w;
  const i32x4* xsrc = (const i32x4*)a.x;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragments of this wave's k-block of the chunk in LDS buffer b, and their 16 MFMAs
  auto rd = [&](bf16x8 (&af)[4], bf16x8 (&bf)[4], int b) __attribute__((always_inline)) {
    const char* buf = stage + b * CHUNKB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const char* src = buf + (size_t)((wn * 4 + i) * C::CK + wk) * AFB + lane * (AFB / 64);
      if constexpr (WT == WT_FP8) {
        const i32x2 v = *(const i32x2*)src;
        af[i] = fp8x8_to_bf16x8(make_uint2(v[0], v[1]));
      } else {
        af[i] = *(const bf16x8*)src;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bf[j] = *(const bf16x8*)(buf + C::NA * AFB + (size_t)(wk * C::MT + wm * 4 + j) * 1024 + lane * 16);
  };
  auto mm = [&](const bf16x8 (&af)[4], const bf16x8 (&bf)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
  };

  // 1/rms of this tile's tokens from the producer's partial sums of h^2 (QKV, gate/up):
  // thread -> token t % TM, partial groups t / TM + GPT * q; clamped loads, masked sums
  auto rms_partial = [&]() __attribute__((always_inline)) {
    if constexpr (EPI == EPI_QKV || EPI == EPI_GEGLU) {
      const int tl = threadIdx.x % (C::MT * 16), g0 = threadIdx.x / (C::MT * 16);
      const float* sp = a.ssp_in + min(tt0 * 16 + tl, a.M_pad - 1);
      float sum = 0.f;
      for (int q0 = 0; q0 < a.g_in; q0 += C::GPT * C::NRD) {  // 64 groups a pass (width 1024 per pass)
        float sv[C::NRD];
  #pragma unroll
        for (int q = 0; q < C::NRD; ++q) sv[q] = sp[(size_t)min(q0 + g0 + C::GPT * q, a.g_in - 1) * a.M_pad];
  #pragma unroll
        for (int q = 0; q < C::NRD; ++q) sum += q0 + g0 + C::GPT * q < a.g_in ? sv[q] : 0.f;
      }
      ssq[threadIdx.x] = sum;
    }
  };
  auto rms_final = [&]() __attribute__((always_inline)) {  // after a barrier
    if constexpr (EPI == EPI_QKV || EPI == EPI_GEGLU) {
      if (threadIdx.x < C::MT * 16) {
        float t = 0.f;
  #pragma unroll
        for (int q = 0; q < C::GPT; ++q) t += ssq[q * C::MT * 16 + threadIdx.x];
        inv_rms[threadIdx.x] = rsqrtf(t * a.inv_width + a.eps);
      }
    }
  };
  const int nc = KB / C::CK;
  bf16x8 fa_d[4], fb_d[4], ga_d[4], gb_d[4];  // the LDS-staged shapes' fragments of two chunks
  if constexpr (WN == 1 && WM == 1) {
    // one 64 x 64 tile per workgroup, one k-group per wave: no fragment is shared between waves,
    // so each wave loads its own straight into registers (three k-blocks in flight) and the loop
    // has no LDS traffic and no barrier; LDS only meets the k-groups' partial tiles afterwards
    auto ld = [&](bf16x8 (&af)[4], bf16x8 (&bf)[4], int c) __attribute__((always_inline)) {
      const int kb = min(c, nc - 1) * WK + wk;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const WR v = wsrc[((size_t)(ct0 + i) * KB + kb) * 64 + lane];
        if constexpr (WT == WT_FP8) af[i] = fp8x8_to_bf16x8(make_uint2(v[0], v[1]));
        else af[i] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = __builtin_bit_cast(bf16x8, xsrc[((size_t)kb * ntt + min(tt0 + j, ntt - 1)) * 64 + lane]);
    };
    bf16x8 a0[4], b0[4], a1[4], b1[4], a2[4], b2[4];
    ld(a0, b0, 0);
    ld(a1, b1, 1);
    ld(a2, b2, 2);
    rms_partial();
    __syncthreads();
    rms_final();
    for (int c = 0; c < nc; c += 3) {
      mm(a0, b0);
      ld(a0, b0, c + 3);
      if (c + 1 < nc) mm(a1, b1);
      ld(a1, b1, c + 4);
      if (c + 2 < nc) mm(a2, b2);
      ld(a2, b2, c + 5);
    }
  } else if constexpr (WT == WT_BF16 || WT == WT_FP8) {
    // Operands go from global memory straight into LDS: one global_load_lds_dwordx4 of a wave writes
    // a whole 1 KB fragment (lane l's 16 bytes at l * 16), so no register carries them and no LDS
    // store is issued; an E4M3 weight fragment (512 bytes) takes two dword loads (bytes l * 4 and
    // 256 + l * 4). Chunk c goes to buffer c % NBUF and D = NBUF - 1 chunks are in flight; a
    // wave waits for its own loads of a chunk (vmcnt), and the barrier after that makes every
    // wave's loads of it visible. Fragments of the next chunk are read from LDS into registers while
    // the MFMAs of the current one run (the LDS reads hide under the MFMAs).
    constexpr int AL = WT == WT_FP8 ? 2 : 1;  // loads per weight fragment
    // (E4M3 chunks are smaller than the bf16 ones the stage is sized for; filling it with more of them
    // measured the same on the prefill)
    constexpr int NB_ = C::NBUF, D = NB_ - 1, LPC = AL * LW + LX;
    static_assert((D - 1) * LPC < 64 && (size_t)NB_ * CHUNKB <= C::STAGE, "chunk buffers");
    const char* wb = (const char*)a.w;
    const char* xb = (const char*)a.x;
    auto dma = [&](int c) __attribute__((always_inline)) {
      char* dst = stage + (size_t)(c % NB_) * CHUNKB;
#pragma unroll
      for (int i = 0; i < LW; ++i) {
        const int f = wave + GW * i;
        const size_t frag = (size_t)(ct0 + f / C::CK) * KB + c * C::CK + f % C::CK;
        if constexpr (WT == WT_FP8) {
          const char* src = wb + frag * 512 + lane * 4;
          __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)(dst + (size_t)f * 512),
                                           4, 0, 0);
          __builtin_amdgcn_global_load_lds((const void*)(src + 256),
                                           (__attribute__((address_space(3))) void*)(dst + (size_t)f * 512 + 256), 4, 0, 0);
        } else {
          const char* src = wb + (frag * 64 + lane) * 16;
          __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)(dst + (size_t)f * 1024),
                                           16, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < LX; ++i) {
        const int f = wave + GW * i;
        const char* src = xb + (((size_t)(c * C::CK + f / C::MT) * ntt + min(tt0 + f % C::MT, ntt - 1)) * 64 + lane) * 16;
        __builtin_amdgcn_global_load_lds((const void*)src,
                                         (__attribute__((address_space(3))) void*)(dst + (size_t)C::NA * AFB + (size_t)f * 1024),
                                         16, 0, 0);
      }
    };
    // issue chunk `last` (when it exists) and wait until chunk last - D + 1 has landed everywhere: D - 1
    // chunks of this wave's loads may stay in flight; with nothing issued, wait for all of them
    auto issue_wait = [&](int last) __attribute__((always_inline)) {
      if (last < nc) {
        dma(last);
        vm_wait_barrier<(D - 1) * LPC>();
      } else {
        vm_wait_barrier<0>();
      }
    };
#pragma unroll
    for (int c = 0; c < D - 1; ++c)
      if (c < nc) dma(c);
    rms_partial();           // its loads are the youngest: the compiler's wait for them waits for these too
    issue_wait(D - 1);       // chunk 0 landed
    rms_final();
    rd(fa_d, fb_d, 0);
    issue_wait(D);           // chunk 1 landed; every wave's reads of buffer 0 are done
    // step c: chunk c's fragments in registers; read chunk c + 1's, MFMAs of chunk c, then chunk
    // c + D + 1 into buffer c % NBUF (chunk c's, read before the last barrier)
    auto dstep = [&](int c, const bf16x8 (&fc)[4], const bf16x8 (&gc)[4], bf16x8 (&fn)[4], bf16x8 (&gn)[4])
                     __attribute__((always_inline)) {
      rd(fn, gn, (c + 1) % NB_);
      mm(fc, gc);
      issue_wait(c + D + 1);
    };
    int c = 0;
    for (; c + 2 <= nc; c += 2) {
      dstep(c, fa_d, fb_d, ga_d, gb_d);
      dstep(c + 1, ga_d, gb_d, fa_d, fb_d);
    }
    if (c < nc) dstep(c, fa_d, fb_d, ga_d, gb_d);
  }

  asm volatile("" ::"v"(tch[0] ^ tch[1] ^ tch[2] ^ tch[3]));  // the touches, long since in
  // partial sub-tiles of the WK k-groups meet in LDS: [wave][tile q = 4 i + j][lane][4]
  if constexpr (WK > 1) {
    __syncthreads();  // every wave is done reading the operand stage
    float* red = (float*)stage;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) *(f32x4*)(red + (((size_t)wave * 16 + i * 4 + j) * 64 + lane) * 4) = acc[i][j];
    __syncthreads();
  }
  // the sum of tile (i, j) of this wave's sub-tile over the k-groups, in k-group order
  auto tile_sum = [&](int i, int j) __attribute__((always_inline)) -> f32x4 {
    if constexpr (WK == 1) {
      return acc[i][j];
    } else {
      const float* red = (const float*)stage;
      f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int g = 0; g < WK; ++g) {
        const int w = (wm * WN + wn) * WK + g;
        v += *(const f32x4*)(red + (((size_t)w * 16 + i * 4 + j) * 64 + lane) * 4);
      }
      return v;
    }
  };

  // ---------------- epilogues: lane -> token tt*16 + lane % 16, channels 4 (lane / 16) + v of a tile
  const int cq = lane >> 4, tq = lane & 15;
  if constexpr (EPI == EPI_GEGLU) {
    // gate tile 2p and up tile 2p + 1 hold the same 16 outputs f
#pragma unroll
    for (int u = 0; u < 8 / WK; ++u) {
      const int pq = wk + WK * u, p = pq >> 2, j = pq & 3;
      f32x4 gv = tile_sum(2 * p, j), uv = tile_sum(2 * p + 1, j);
      if constexpr (WT == WT_FP8) {  // per-channel scales of the gate and up rows
        const int ch = (ct0 + wn * 4 + 2 * p) * 16 + cq * 4;
        gv *= *(const f32x4*)(a.wscale + ch);
        uv *= *(const f32x4*)(a.wscale + ch + 16);
      }
      const int tl = (wm * 4 + j) * 16 + tq, tok = tt0 * 16 + tl;
      const float ir = inv_rms[tl];
      const int f = ((ct0 + wn * 4) / 2 + p) * 16 + cq * 4;
      f32x4 g2 = gv * ir, u2 = uv * ir;
      if (a.shift_bias) {  // time-modulated expert: W . shift of the row's sequence, after the 1/rms scaling
        const float* sb = a.shift_bias + (a.mod_rows ? (size_t)(min(tok, a.M - 1) / a.mod_rows) * a.ms_shift : 0) +
                          (ct0 + wn * 4 + 2 * p) * 16 + cq * 4;
        g2 += *(const f32x4*)sb;
        u2 += *(const f32x4*)(sb + 16);
      }
      if (tok < a.M) {
        uint2 o;
        o.x = (uint32_t)f32_to_bf16(gelu_tanh_fast(g2[0]) * u2[0]) | ((uint32_t)f32_to_bf16(gelu_tanh_fast(g2[1]) * u2[1]) << 16);
        o.y = (uint32_t)f32_to_bf16(gelu_tanh_fast(g2[2]) * u2[2]) | ((uint32_t)f32_to_bf16(gelu_tanh_fast(g2[3]) * u2[3]) << 16);
        *(uint2*)((uint16_t*)a.u_out + act_idx(tok, f, ntt)) = o;
      }
    }
  } else if constexpr (EPI == EPI_RESID) {
    // groups of up to 8 tiles: their residual rows are loaded before any is stored
    constexpr int PER = 16 / WK, GRP = PER < 8 ? PER : 8;
#pragma unroll
    for (int u0 = 0; u0 < PER; u0 += GRP) {
      float4 hv[GRP], gv[GRP];
      f32x4 val[GRP];
#pragma unroll
      for (int u = 0; u < GRP; ++u) {
        const int q = wk + WK * (u0 + u), i = q >> 2, j = q & 3;
        const int tok = tt0 * 16 + (wm * 4 + j) * 16 + tq;
        const int n = (ct0 + wn * 4 + i) * 16 + cq * 4;
        // time-modulated expert: the next gain and this sublayer's residual gate of the row's sequence
        const size_t msq = a.mod_rows ? (size_t)(min(tok, a.M - 1) / a.mod_rows) : 0;
        hv[u] = *(const float4*)(a.h + (size_t)min(tok, a.M - 1) * a.N + n);
        gv[u] = *(const float4*)(a.gain_next + msq * a.ms_gain + n);
        val[u] = tile_sum(i, j);
        if constexpr (WT == WT_FP8) val[u] *= *(const f32x4*)(a.wscale + n);  // per-channel scales
        if (a.res_gate) val[u] *= *(const f32x4*)(a.res_gate + msq * a.ms_gate + n);
      }
#pragma unroll
      for (int u = 0; u < GRP; ++u) {
        const int q = wk + WK * (u0 + u), i = q >> 2, j = q & 3;
        const int tok = tt0 * 16 + (wm * 4 + j) * 16 + tq;
        const int tile = ct0 + wn * 4 + i, n = tile * 16 + cq * 4;
        const bool valid = tok < a.M;
        float4 hn = make_float4(0.f, 0.f, 0.f, 0.f);
        if (valid) {
          hn = make_float4(hv[u].x + val[u][0], hv[u].y + val[u][1], hv[u].z + val[u][2], hv[u].w + val[u][3]);
          *(float4*)(a.h + (size_t)tok * a.N + n) = hn;
          uint2 o;
          o.x = (uint32_t)f32_to_bf16(hn.x * gv[u].x) | ((uint32_t)f32_to_bf16(hn.y * gv[u].y) << 16);
          o.y = (uint32_t)f32_to_bf16(hn.z * gv[u].z) | ((uint32_t)f32_to_bf16(hn.w * gv[u].w) << 16);
          *(uint2*)((uint16_t*)a.hb + act_idx(tok, n, ntt)) = o;
        }
        float sq = hn.x * hn.x + hn.y * hn.y + hn.z * hn.z + hn.w * hn.w;
        sq += __shfl_xor(sq, 16);
        sq += __shfl_xor(sq, 32);
        if (cq == 0 && tok < a.M_pad) a.ssp_out[(size_t)tile * a.M_pad + tok] = sq;
      }
    }
  } else {  // EPI_QKV
    const int tph = a.dh / 16, half = a.dh / 2, nkb = a.dh / KBLK;
    const int q_tiles = a.n_q * tph, k_tiles = a.n_kv * tph, gq = a.n_q / a.n_kv;
    // this lane's 4 tokens (one per token tile j): sequence and chunk row, divided once
    int sqj[4], tj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tok = min(tt0 * 16 + (wm * 4 + j) * 16 + tq, a.M - 1);
      sqj[j] = tok / a.H;
      tj[j] = tok - sqj[j] * a.H;
    }
    constexpr int PER = 16 / WK, GRP = PER < 4 ? PER : 4;
#pragma unroll
    for (int u0 = 0; u0 < PER; u0 += GRP) {
      // (cos, sin) of the 4 head dims this lane rotates, for each tile of the group
      float4 cs[GRP][2];
#pragma unroll
      for (int u = 0; u < GRP; ++u) {
        const int q = wk + WK * (u0 + u), i = q >> 2, j = q & 3;
        const int tin = ct0 + wn * 4 + i, pair = (tin < q_tiles ? tin : tin - q_tiles) % tph;  // wave-uniform
        const float4* cp = (const float4*)(a.rope_cs + ((size_t)tj[j] * half + pair * 8 + 4 * (cq & 1)) * 2);
        cs[u][0] = cp[0];
        cs[u][1] = cp[1];
      }
#pragma unroll
      for (int u = 0; u < GRP; ++u) {
        const int q = wk + WK * (u0 + u), i = q >> 2, j = q & 3;
        const int tl = (wm * 4 + j) * 16 + tq, tok = tt0 * 16 + tl;
        const int tin = ct0 + wn * 4 + i;  // wave-uniform
        const float ir = inv_rms[tl];
        const f32x4 v = tile_sum(i, j);
        const bool valid = tok < a.M;
        const int sq = sqj[j], t = tj[j];
        float x[4], xp[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = v[e] * ir;
        if (a.shift_bias) {  // time-modulated expert: W . shift of the row's sequence
          const f32x4 sb = *(const f32x4*)(a.shift_bias + (a.mod_rows ? (size_t)sq * a.ms_shift : 0) + tin * 16 + cq * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] += sb[e];
        }
        if (a.qk_gain && tin < q_tiles + k_tiles) {  // QK-norm (wave-uniform): the tile's share of its head's
          // sum of squares for this token (its 16 channels sit in lanes tq + 16 cq), then the per-dim gains
          float s2 = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
          s2 += __shfl_xor(s2, 16);
          s2 += __shfl_xor(s2, 32);
          if (cq == 0 && valid) a.qk_ssp[(size_t)tin * a.M_pad + tok] = s2;
          const f32x4 qg = *(const f32x4*)(a.qk_gain + tin * 16 + cq * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] *= qg[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) xp[e] = __shfl_xor(x[e], 32);  // channel c +- 8: the other half of the rotation pair
        if (tin < q_tiles + k_tiles) {
          const bool is_q = tin < q_tiles;
          const int tt2 = is_q ? tin : tin - q_tiles, head = tt2 / tph, pair = tt2 - head * tph;
          const int hf = cq >> 1;
          const float c4[4] = {cs[u][0].x, cs[u][0].z, cs[u][1].x, cs[u][1].z};
          const float s4[4] = {cs[u][0].y, cs[u][0].w, cs[u][1].y, cs[u][1].w};
          float out[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            out[e] = hf ? xp[e] * s4[e] + x[e] * c4[e] : x[e] * c4[e] - xp[e] * s4[e];
          const int dfull = hf * half + pair * 8;
          const int lgrp = ((dfull % KBLK) >> 3) << 4, kb = dfull / KBLK;
          size_t off;
          if (is_q) {
            const int gg = head / gq, rr = (head - gg * gq) * a.H + t;
            off = ((((size_t)sq * a.n_kv + gg) * a.n_qt + (rr >> 4)) * nkb + kb) * 512 + (lgrp + (rr & 15)) * 8;
          } else {
            const int kk = t & 31, kt = (kk & 7) >> 2, m = 4 * (kk >> 3) + (kk & 3);
            off = (((((size_t)sq * a.n_kv + head) * a.nbs + (t >> 5)) * 2 + kt) * nkb + kb) * 512 + (lgrp + m) * 8;
          }
          if (valid) {
            uint2 o;
            o.x = (uint32_t)f32_to_bf16(out[0]) | ((uint32_t)f32_to_bf16(out[1]) << 16);
            o.y = (uint32_t)f32_to_bf16(out[2]) | ((uint32_t)f32_to_bf16(out[3]) << 16);
            *(uint2*)((uint16_t*)(is_q ? a.q_out : a.k_out) + off + 4 * (cq & 1)) = o;
          }
        } else if (valid) {
          // value A fragments (of V^T) of key block t/32: dims dt*16 + lane%16, keys (lane/16)*8 + e;
          // this tile is head dims (tv % tph)*16 .. +16 of kv head tv / tph
          const int tv = tin - q_tiles - k_tiles, hd = tv / tph, d16 = tv - hd * tph;
          const int kk = t & 31;
          const size_t fr = (((size_t)sq * a.n_kv + hd) * a.nbs + (t >> 5)) * (a.dh / 16) + d16;
          uint16_t* vp = (uint16_t*)a.v_out + fr * 512 + (((kk >> 3) << 4) + cq * 4) * 8 + (kk & 7);
#pragma unroll
          for (int e = 0; e < 4; ++e) vp[e * 8] = f32_to_bf16(x[e]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ attention

// Attention operands live in MFMA fragment order, one 1 KB (bf16) or 2 KB (fp32)
// contiguous run per fragment, so every load instruction of a wave reads whole
// cache lines (scattered 16-byte pieces of 16 rows cost several times more):
//   Q  [seq][kv head][16-row tile][dh/32][64 lanes][8]: lane = (d%32/8)*16 + row%16,
//      row r = j*H + t for query head g*gq + j and chunk row t;
//   K  [..][32-key block][2][dh/32][64][8]: half kt, lane = (d%32/8)*16 + m holds key
//      8*(m/4) + 4*kt + m%4 of the block, so that the S^T accumulators of a lane
//      cover keys 8*(lane/16) .. +8 of the block in order;
//   V  [..][32-key block][dh/16][64][8]: lane = (key/8)*16 + d%16, element key%8
//      (the A operand of O^T = V^T P^T over the same 8 keys).
// The prefix cache is packed this way at load time, per slot and layer, with
// ceil(P/32) blocks (keys past P zero); the suffix operands are written in
// this order by the QKV epilogue with ceil(H/32) blocks per sequence.
struct AttnArgs {
  const void* q;          // packed queries
  const void* ks;         // packed suffix K
  const void* vs;         // packed suffix V
  const void* kcache;     // packed prefix K [slot][L][n_kv][nbp][2][dh/32][64][8]
  const void* vcache;     // packed prefix V [slot][L][n_kv][nbp][dh/16][64][8]
  const int* seq_slot;    // prefix slot of each sequence; null: sequence s uses slot slot0 + s (no load)
  int slot0;
  size_t slot_stride, layer_off;  // elements (same for K and V)
  int P, H, n_q, n_kv, dh;
  int nbp, nbs;           // 32-key prefix / suffix blocks
  int ntt;                // 16-token tiles of o (fragment order, act_idx)
  int n_qt;               // 16-row query tiles per (sequence, kv head)
  int n_split;            // key splits (workgroups) per query tile
  float scale_log2;       // log2(e) / sqrt(dh)
  float* opart;           // [zz][qt][split][16][dh] split partials, EXCH_EMPTY between launches
  float* mlpart;          // [zz][qt][split][16][2]  (row max in log2 units, row sum), same
  unsigned* err;          // set if a co-resident merge poll gave up (host-visible)
  unsigned long long wait;  // constant-clock ticks (100 MHz) a merge poll waits before it gives up
  int coresident;         // 1: every workgroup is resident at once; splits merge in-kernel
  void* o;                // output, fragment order (act_idx)
  // QK-norm: per (q or k tile, token) sums of squares of the raw projections written by the QKV
  // epilogue ([q tiles, then k tiles][qk_mpad]); a score is scaled by 1/rms of its query head row and,
  // for suffix keys, of its key (the cached prefix keys come normalised)
  const float* qk_ssp;
  int qk_mpad;
  float qk_inv_dh, qk_eps;
  // 1: workgroup i (on XCD i % 8) takes the i-th of a contiguous run of (sequence, query tile, split)
  // items per XCD, so the workgroups reading one sequence's K/V share one L2 (many sequences)
  int xcd_group;
  // 1 (passes over several sequences): each workgroup first touches its share of its sequence's prefix
  // K/V lines, one dword per 128-byte line, so that all of them are asked from HBM at once
  int touch;
};

constexpr int ATT_ROWS = 16;   // query rows per workgroup
constexpr int ATT_KB = 32;     // keys per wave block
// Two shapes: splits that merge inside the launch give each of 8 waves one key block
// (measured: 4 waves x 7 splits read less per compute unit but lose more to the larger
// exchange); otherwise 8 waves walk up to 4 blocks each (a split covers 32 blocks).
constexpr int ATT_WAVES_SPLIT = 8, ATT_IT_SPLIT = 1;
constexpr int ATT_WAVES_WHOLE = 8, ATT_IT_WHOLE = 4;
constexpr int ATT_IT_MID = 2;  // co-resident splits of 8 waves x 2 blocks when 1-block splits would not fit

constexpr int ATT_QKN_KEYS = 256;  // suffix keys the QK-norm scales are staged for (horizon <= 256)
template <int DH, int NW, bool QKN = false>
constexpr size_t attn_lds_size() {  // per-wave O and (m, l), the query tile (fp32 at most); QK-norm scales
  return (size_t)NW * ATT_ROWS * (DH + 4) * 4 + (size_t)NW * ATT_ROWS * 2 * 4 + (size_t)ATT_ROWS * DH * 4 +
         (QKN ? (size_t)(ATT_ROWS + ATT_QKN_KEYS) * 4 : 0);
}

// Attention of suffix query rows over [prefix ; suffix] keys. Grid (n_split,
// n_qt, n_seq * n_kv), block = NW waves. A query tile is 16 rows; GQA folds the
// gq heads of a kv head into rows, so each key is read once per tile. The key
// blocks of a split (prefix blocks first, then the sequence's suffix blocks)
// are dealt to the NW waves round robin; a wave runs an online softmax over its
// blocks. S^T = K Q^T leaves per lane 8 scores of one row that are exactly the
// B operand of O^T = V^T P^T, so the softmax stays in registers. Loads are
// pipelined without extra registers: a block's K fragments are reissued for
// the next block as soon as its S^T is done, its V fragments as soon as its
// O^T is done. The waves merge (m, l, O) in LDS; with one split the workgroup
// writes o, with several it stores its partial for attn_merge.
// TPW = 2 (bf16, one split, no QK-norm): the workgroup takes query tiles 2y and 2y + 1 of its
// sequence, 4 waves each; the waves of the two tiles walk the same key blocks in the same order, so
// the second reader of each K/V fragment finds it in the compute unit's L1 and a sequence's K/V
// crosses from L2 once per pair of tiles (and the launch is one round of half as many workgroups).
template <int AT, int DH, int ATT_IT, int NW, bool QKN = false, int TPW = 1>
__global__ __launch_bounds__(NW * 64) void attn_kernel(AttnArgs a) {
  static_assert(TPW == 1 || (TPW == 2 && !QKN && AT == AT_BF16), "two query tiles: bf16 without QK-norm");
  constexpr int NWT = NW / TPW;    // waves per query tile
  typedef typename Act<AT>::T XT;
  typedef Frag<WT_BF16, AT> F;
  constexpr int NKB = DH / KBLK;   // 32-dim blocks of a head
  constexpr int NDT = DH / 16;     // 16-dim tiles of a head
  constexpr int LDO = DH + 4;      // LDS row stride of a wave's O (floats)
  constexpr int FR = 512;          // elements per fragment (64 lanes x 8)
  extern __shared__ __attribute__((aligned(16))) float att_smem[];
  float* Ow = att_smem;                                    // [waves][16][LDO]
  float* MLw = Ow + NW * ATT_ROWS * LDO;                   // [waves][16][2]
  XT* Qs = (XT*)(MLw + NW * ATT_ROWS * 2);                 // [NKB][64][8] query fragments
  float* rq_s = (float*)((char*)Qs + (size_t)ATT_ROWS * DH * 4);  // QK-norm: 1/rms of the 16 query rows
  float* rk_s = rq_s + ATT_ROWS;                                  // and of the suffix keys

  int split = blockIdx.x, qt = blockIdx.y, zz = blockIdx.z;
  if (a.xcd_group) {
    const int T = gridDim.x * gridDim.y * gridDim.z;
    const int L = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z), xcd = L & 7;
    const int item = xcd * (T >> 3) + min(xcd, T & 7) + (L >> 3);
    split = item % gridDim.x;
    qt = (item / gridDim.x) % gridDim.y;
    zz = item / (gridDim.x * gridDim.y);
  }
  const int s = zz / a.n_kv, g = zz % a.n_kv;
  const int gq = a.n_q / a.n_kv;
  const int R = gq * a.H;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;  // wave: scalar
  const int qt0 = qt * TPW, tq = wave / NWT, wv = wave % NWT;  // this wave's tile qt0 + tq
  const int slot = a.seq_slot ? a.seq_slot[s] : a.slot0 + s;
  const int nb = a.nbp + a.nbs;
  const int bps = (nb + a.n_split - 1) / a.n_split;         // blocks per split
  const int b_begin = split * bps, b_end = min(nb, b_begin + bps);
  const size_t pre_base = (size_t)slot * a.slot_stride + a.layer_off + (size_t)g * a.nbp * (2 * NKB * FR);
  const size_t suf_base = ((size_t)s * a.n_kv + g) * a.nbs * (2 * NKB * FR);
  // fragment base and valid keys of block b (a prefix or a suffix block)
  auto block_src = [&](int b, const XT*& kf, const XT*& vf, int& n_valid) {
    if (b < a.nbp) {
      const size_t base = pre_base + (size_t)b * (2 * NKB * FR);
      kf = (const XT*)a.kcache + base;
      vf = (const XT*)a.vcache + base;
      n_valid = min(ATT_KB, a.P - b * ATT_KB);
    } else {
      const size_t base = suf_base + (size_t)(b - a.nbp) * (2 * NKB * FR);
      kf = (const XT*)a.ks + base;
      vf = (const XT*)a.vs + base;
      n_valid = min(ATT_KB, a.H - (b - a.nbp) * ATT_KB);
    }
  };
  const XT* qf = (const XT*)a.q + (((size_t)s * a.n_kv + g) * a.n_qt) * NKB * FR;  // the sequence's first tile

  // Several sequences: the blocks below reach each wave one at a time (a block's loads go out once the
  // previous block's are in), and the first reader of a line of the sequence's prefix waits out HBM
  // latency for it, block after block. The workgroups of one (sequence, kv head) therefore touch its
  // prefix K and V first, line by line (rank split + n_split * tile of n_split * tiles), so that every
  // line is asked for at once and the chained loads find them in L2. The values are only consumed after
  // the block loop (loads complete in order: the first block's wait covers them).
  int tch[2] = {0, 0};
  if (a.touch) {
    const unsigned n_grp = gridDim.x * gridDim.y, rk = split + gridDim.x * qt;
    const unsigned lines = (unsigned)((size_t)a.nbp * 2 * NKB * FR * sizeof(XT) / 128);  // of K (and of V)
    const char* kb0 = (const char*)((const XT*)a.kcache + pre_base);
    const char* vb0 = (const char*)((const XT*)a.vcache + pre_base);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const unsigned L = rk + n_grp * (threadIdx.x + NW * 64 * i);
      if (L < 2 * lines) tch[i] = *(const int*)((L < lines ? kb0 : vb0) + (size_t)(L % lines) * 128);
    }
  }

  // the query tile(s) go to LDS once (the same for every wave and block): their loads are issued
  // first, the LDS stores wait only for them while the K/V loads below stay in flight; a second
  // tile past the sequence's last one reads the last one (its rows are never stored)
  constexpr int QVEC = 16 / sizeof(XT);  // elements per 16-byte vector
  constexpr int QNV1 = NKB * FR / QVEC, QNV = TPW * QNV1;
  constexpr int QIT = (QNV + NW * 64 - 1) / (NW * 64);
  static_assert((size_t)QNV * 16 <= (size_t)ATT_ROWS * DH * 4, "query tiles fit their LDS region");
  i32x4 qtmp[QIT];
#pragma unroll
  for (int i = 0; i < QIT; ++i) {
    const int e = threadIdx.x + NW * 64 * i;
    const int tile = min(qt0 + e / QNV1, a.n_qt - 1);
    qtmp[i] = e < QNV ? *(const i32x4*)(qf + (size_t)tile * NKB * FR + (e % QNV1) * QVEC) : i32x4{0, 0, 0, 0};
  }
  __builtin_amdgcn_sched_barrier(0);
  // this wave's blocks: b_begin + wave + NW it for it < ATT_IT (the runtime keeps a split within
  // ATT_IT blocks per wave); a slot past the split's end reads the split's first block, masked.
  // The loop is unrolled with no data-dependent branch so every wait covers exactly the loads it needs.
  const XT* kfs[ATT_IT];
  const XT* vfs[ATT_IT];
  int nvs[ATT_IT];
#pragma unroll
  for (int it = 0; it < ATT_IT; ++it) {
    const int bb = b_begin + wv + NWT * it;
    block_src(bb < b_end ? bb : b_begin, kfs[it], vfs[it], nvs[it]);
    if (bb >= b_end) nvs[it] = 0;
  }
  typename F::A ka[2][NKB];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) ka[kt][kb] = F::load_b(kfs[0] + (kt * NKB + kb) * FR + lane * 8);
  typename F::A va[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) va[dt] = F::load_b(vfs[0] + dt * FR + lane * 8);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < QIT; ++i) {
    const int e = threadIdx.x + NW * 64 * i;
    if (e < QNV) *(i32x4*)(Qs + e * QVEC) = qtmp[i];
  }
  if constexpr (QKN) {
    // thread -> (row or key, one of the head's dh/16 tiles); a row's 16 lanes sum its tiles' partials
    const int tph = DH / 16, q_tiles = a.n_q * tph;
    for (int idx = threadIdx.x; idx < (ATT_ROWS + a.nbs * ATT_KB) * 16; idx += NW * 64) {
      const int r = idx >> 4, i = idx & 15;
      float v = 0.f;
      if (r < ATT_ROWS) {
        const int rg = qt * ATT_ROWS + r;
        if (rg < R && i < tph) {
          const int head = g * gq + rg / a.H, t = rg % a.H;
          v = a.qk_ssp[(size_t)(head * tph + i) * a.qk_mpad + s * a.H + t];
        }
      } else {
        const int key = r - ATT_ROWS;
        if (key < a.H && i < tph) v = a.qk_ssp[(size_t)(q_tiles + g * tph + i) * a.qk_mpad + s * a.H + key];
      }
      v += __shfl_xor(v, 1, 16);
      v += __shfl_xor(v, 2, 16);
      v += __shfl_xor(v, 4, 16);
      v += __shfl_xor(v, 8, 16);
      if (i == 0) rq_s[r] = rsqrtf(v * a.qk_inv_dh + a.qk_eps);  // rk_s[key] = rq_s[ATT_ROWS + key]
    }
  }
  __syncthreads();  // query tile staged

  const int k8 = 8 * (lane >> 4);
  const float row_scale = QKN ? a.scale_log2 * rq_s[lane & 15] : a.scale_log2;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int it = 0; it < ATT_IT; ++it) {
    // S^T: sacc[kt][v] = score(block key 8*(lane/16) + 4*kt + v, row lane%16)
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const typename F::B qb = F::load_b(Qs + (tq * NKB + kb) * FR + lane * 8);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) sacc[kt] = F::mma(ka[kt][kb], qb, sacc[kt]);
    }
    __builtin_amdgcn_sched_barrier(0);  // ka consumed before the next block's K overwrites it
    if (it + 1 < ATT_IT) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) ka[kt][kb] = F::load_b(kfs[it + 1] + (kt * NKB + kb) * FR + lane * 8);
    }
    __builtin_amdgcn_sched_barrier(0);
    // online softmax over this block for row lane%16
    const int n_valid = nvs[it];
    float mb = -INFINITY;
    // QK-norm: a suffix block's keys carry 1/rms of their own (prefix keys come normalised)
    const int bb_it = b_begin + wv + NWT * it, sk0 = (bb_it - a.nbp) * ATT_KB + k8;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float f = row_scale;
        if constexpr (QKN)
          if (bb_it >= a.nbp && k8 + 4 * kt + v < n_valid) f *= rk_s[sk0 + 4 * kt + v];
        const float sv = (k8 + 4 * kt + v < n_valid) ? sacc[kt][v] * f : -INFINITY;
        sacc[kt][v] = sv;
        mb = fmaxf(mb, sv);
      }
    mb = fmaxf(mb, __shfl_xor(mb, 16));
    mb = fmaxf(mb, __shfl_xor(mb, 32));
    const float m_new = fmaxf(m_run, mb);
    const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
    float lb = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float p = (m_new == -INFINITY) ? 0.f : exp2f(sacc[kt][v] - m_new);
        sacc[kt][v] = p;
        lb += p;
      }
    lb += __shfl_xor(lb, 16);
    lb += __shfl_xor(lb, 32);
    l_run = l_run * alpha + lb;
    m_run = m_new;
    typename F::B pb;
    if constexpr (AT == AT_BF16) {
      pb = bf16x8{(__bf16)sacc[0][0], (__bf16)sacc[0][1], (__bf16)sacc[0][2], (__bf16)sacc[0][3],
                  (__bf16)sacc[1][0], (__bf16)sacc[1][1], (__bf16)sacc[1][2], (__bf16)sacc[1][3]};
    } else {
      pb = typename F::B{make_float4(sacc[0][0], sacc[0][1], sacc[0][2], sacc[0][3]),
                         make_float4(sacc[1][0], sacc[1][1], sacc[1][2], sacc[1][3])};
    }
    // O^T = alpha O^T + V^T P^T: element (dim dt*16 + 4*(lane/16) + v, row lane%16)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = F::mma(va[dt], pb, oacc[dt] * alpha);
    __builtin_amdgcn_sched_barrier(0);  // va consumed before the next block's V overwrites it
    if (it + 1 < ATT_IT) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) va[dt] = F::load_b(vfs[it + 1] + dt * FR + lane * 8);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  asm volatile("" ::"v"(tch[0] ^ tch[1]));  // the touches, long since in
  // this wave's (m, l, O) to LDS: O[row lane%16][dt*16 + 4*(lane/16) + v]
  float* ow = Ow + (size_t)wave * ATT_ROWS * LDO + (lane & 15) * LDO + 4 * (lane >> 4);
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) *(f32x4*)(ow + dt * 16) = oacc[dt];
  if (lane < 16) *(float2*)(MLw + (wave * ATT_ROWS + lane) * 2) = make_float2(m_run, l_run);
  __syncthreads();

  // ---- merge the waves: thread -> (row, 4-dim chunk) pairs q = t + 64 NW i; a wave reads whole
  // 1 KB rows of the wave partials, so the LDS reads have no bank conflicts
  constexpr int CPR = DH / 4;                              // 16-byte chunks per row
  constexpr int NTH = NW * 64;
  constexpr int PPT = (TPW * ATT_ROWS * CPR + NTH - 1) / NTH;  // pairs per thread
  const int c4 = threadIdx.x % CPR;                        // same chunk for every pair of a thread
  if constexpr (TPW > 1) {
    // two tiles, one split: each pair merged from its tile's waves and stored at once
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int q = threadIdx.x + NTH * i;
      const int row2 = q / CPR, row = row2 % ATT_ROWS, w0 = (row2 / ATT_ROWS) * NWT;
      const int tile = qt0 + row2 / ATT_ROWS, r = tile * ATT_ROWS + row;
      if (q >= TPW * ATT_ROWS * CPR || tile >= a.n_qt || r >= R) continue;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NWT; ++w) M = fmaxf(M, MLw[((w0 + w) * ATT_ROWS + row) * 2]);
      float L = 0.f;
      f32x4 O = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < NWT; ++w) {
        const float mw = MLw[((w0 + w) * ATT_ROWS + row) * 2];
        const float wt = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
        L += wt * MLw[((w0 + w) * ATT_ROWS + row) * 2 + 1];
        O += wt * *(const f32x4*)(Ow + ((size_t)(w0 + w) * ATT_ROWS + row) * LDO + 4 * c4);
      }
      const int tok = s * a.H + r % a.H, col = (g * gq + r / a.H) * DH + 4 * c4;
      const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) Act<AT>::st((XT*)a.o, act_idx(tok, col + j, a.ntt), O[j] * inv);
    }
    return;
  }
  float Mq[PPT], Lq[PPT];
  f32x4 Oq[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int q = threadIdx.x + NTH * i;
    const int row = q < ATT_ROWS * CPR ? q / CPR : 0;
    float mw[NW], lw[NW];
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float2 ml = *(const float2*)(MLw + (w * ATT_ROWS + row) * 2);
      mw[w] = ml.x;
      lw[w] = ml.y;
      M = fmaxf(M, ml.x);
    }
    float L = 0.f;
    f32x4 O = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = (mw[w] == -INFINITY) ? 0.f : exp2f(mw[w] - M);
      L += wt * lw[w];
      O += wt * *(const f32x4*)(Ow + ((size_t)w * ATT_ROWS + row) * LDO + 4 * c4);
    }
    Mq[i] = M;
    Lq[i] = L;
    Oq[i] = O;
  }

  auto pair_row = [&](int i) { return (int)(threadIdx.x + NTH * i) / CPR; };
  auto pair_ok = [&](int i) { return (int)(threadIdx.x + NTH * i) < ATT_ROWS * CPR; };
  if (a.n_split == 1) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int r = qt * ATT_ROWS + pair_row(i);
      if (pair_ok(i) && r < R) {
        const int tok = s * a.H + r % a.H, col = (g * gq + r / a.H) * DH + 4 * c4;
        const float inv = Lq[i] > 0.f ? 1.f / Lq[i] : 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) Act<AT>::st((XT*)a.o, act_idx(tok, col + j, a.ntt), Oq[i][j] * inv);
      }
    }
    return;
  }

  // partial rows are row-major [dims]; (m, l) per row
  const size_t tile = (size_t)zz * a.n_qt + qt;
  const size_t prow = (tile * a.n_split + split) * ATT_ROWS;  // this split's first partial row
  if (!a.coresident) {
    // ---- several splits: store this split's partial; attn_merge combines them after the launch boundary
#pragma unroll
    for (int i = 0; i < PPT; ++i)
      if (pair_ok(i)) {
        *(f32x4*)(a.opart + (prow + pair_row(i)) * DH + 4 * c4) = Oq[i];
        if (c4 == 0) *(float2*)(a.mlpart + (prow + pair_row(i)) * 2) = make_float2(Mq[i], Lq[i]);
      }
    return;
  }

  // ---- co-resident splits: publish the partial write-through (a wave stores whole 1 KB rows,
  // the 16 rows' (m, l) go out as one 128-byte run); split c then merges rows [c * rps, +rps)
  // of the tile from every split's partial as the words land (see EXCH_EMPTY) and empties
  // them. A row's consumer threads share one wave, whose polls end together.
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.opart), rm = make_rsrc(a.mlpart);
  float2* MLs = (float2*)Qs;  // merged (m, l) per row; the query tile is dead by now
#pragma unroll
  for (int i = 0; i < PPT; ++i)
    if (pair_ok(i)) {
      st16_coherent(ro, (unsigned)(((prow + pair_row(i)) * DH + 4 * c4) * 4),
                    make_float4(Oq[i][0], Oq[i][1], Oq[i][2], Oq[i][3]));
      if (c4 == 0) MLs[pair_row(i)] = make_float2(Mq[i], Lq[i]);
    }
  __syncthreads();
  if (threadIdx.x < ATT_ROWS)
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, MLs[threadIdx.x]), rm,
                                          (unsigned)((prow + threadIdx.x) * 8), 0, 0x10);
  const int rps = (ATT_ROWS + a.n_split - 1) / a.n_split;
  constexpr int TPC = DH / 4;            // consumer threads per row, one 16-byte chunk each
  constexpr int RPP = NW * 64 / TPC;     // rows per pass
  const int kc = threadIdx.x % TPC;
  const int dim = 4 * kc;
  bool gave_up = false;
  for (int rb = 0; rb < rps; rb += RPP) {
    const int rl = rb + (int)threadIdx.x / TPC, rr = split * rps + rl;
    if (rl >= rps || rr >= ATT_ROWS) continue;
    const int r2 = qt * ATT_ROWS + rr;
    float M2 = -INFINITY, L2 = 0.f;
    float4 O2 = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c0 = 0; c0 < a.n_split; c0 += 8) {
      const int nc = min(8, a.n_split - c0);
      float2 ml[8];
      f32x4 oc[8];
      auto moff = [&](int c) { return (unsigned)(((tile * a.n_split + c) * ATT_ROWS + rr) * 8); };
      auto ooff = [&](int c) { return (unsigned)((((tile * a.n_split + c) * ATT_ROWS + rr) * DH + kc * 4) * 4); };
      const unsigned long long t_end = wall_clock64() + a.wait;
      for (;;) {
        bool ok = true;
#pragma unroll
        for (int c = 0; c < 8; ++c)
          if (c < nc) {
            ml[c] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rm, moff(c0 + c), 0, 0x10));
            oc[c] = ld16_coherent(ro, ooff(c0 + c));
            ok = ok && exch_arrived(ml[c].x) && exch_arrived(ml[c].y) && exch_arrived(oc[c]);
          }
        if (__all(ok)) break;
        if (wall_clock64() > t_end) { gave_up = true; break; }
        __builtin_amdgcn_s_sleep(1);
      }
      float Mn = M2;
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (c < nc) Mn = fmaxf(Mn, ml[c].x);
      const float sc = (M2 == -INFINITY) ? 0.f : exp2f(M2 - Mn);
      L2 *= sc;
      O2.x *= sc; O2.y *= sc; O2.z *= sc; O2.w *= sc;
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (c < nc) {
          const float wt = (ml[c].x == -INFINITY) ? 0.f : exp2f(ml[c].x - Mn);
          L2 += wt * ml[c].y;
          O2.x += wt * oc[c][0]; O2.y += wt * oc[c][1]; O2.z += wt * oc[c][2]; O2.w += wt * oc[c][3];
        }
      M2 = Mn;
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (c < nc) {
          st16_empty(ro, ooff(c0 + c));
          if (kc == 0) __builtin_amdgcn_raw_buffer_store_b64(i32x2{-1, -1}, rm, moff(c0 + c), 0, 0x10);
        }
    }
    if (r2 < R) {
      const int tok = s * a.H + r2 % a.H, col = (g * gq + r2 / a.H) * DH + dim;
      const float inv = L2 > 0.f ? 1.f / L2 : 0.f;
      Act<AT>::st((XT*)a.o, act_idx(tok, col, a.ntt), O2.x * inv);
      Act<AT>::st((XT*)a.o, act_idx(tok, col + 1, a.ntt), O2.y * inv);
      Act<AT>::st((XT*)a.o, act_idx(tok, col + 2, a.ntt), O2.z * inv);
      Act<AT>::st((XT*)a.o, act_idx(tok, col + 3, a.ntt), O2.w * inv);
    }
  }
  if (gave_up) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Merge of the key-split partials of attn_kernel: o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// Grid (n_qt, n_seq * n_kv), block = 16 rows x TPR threads, each DPT consecutive dims; the
// partials of up to 8 splits are loaded at once, in split order (deterministic).
template <int AT, int DH>
__global__ __launch_bounds__(256) void attn_merge(AttnArgs a) {
  typedef typename Act<AT>::T XT;
  constexpr int DPT = DH / 16 >= 4 ? DH / 16 : 4;
  constexpr int TPR = DH / DPT;
  const int qt = blockIdx.x, zz = blockIdx.y;
  if ((int)threadIdx.x >= ATT_ROWS * TPR) return;
  const int row = threadIdx.x / TPR, d0 = (threadIdx.x % TPR) * DPT;
  const int s = zz / a.n_kv, g = zz % a.n_kv, gq = a.n_q / a.n_kv;
  const int r = qt * ATT_ROWS + row;
  const size_t tile = (size_t)zz * a.n_qt + qt;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.opart), rm = make_rsrc(a.mlpart);
  float M = -INFINITY, L = 0.f, O[DPT];
#pragma unroll
  for (int i = 0; i < DPT; ++i) O[i] = 0.f;
  for (int c0 = 0; c0 < a.n_split; c0 += 8) {
    float mc[8], lc[8];
    float4 oc[8][DPT / 4];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int sp = c0 + c < a.n_split ? c0 + c : 0;
      const float2 ml = *(const float2*)(a.mlpart + ((tile * a.n_split + sp) * ATT_ROWS + row) * 2);
      mc[c] = c0 + c < a.n_split ? ml.x : -INFINITY;
      lc[c] = ml.y;
      const float* src = a.opart + ((tile * a.n_split + sp) * ATT_ROWS + row) * DH + d0;
#pragma unroll
      for (int i = 0; i < DPT / 4; ++i) oc[c][i] = *(const float4*)(src + 4 * i);
    }
    float Mn = M;
#pragma unroll
    for (int c = 0; c < 8; ++c) Mn = fmaxf(Mn, mc[c]);
    const float sc = (M == -INFINITY) ? 0.f : exp2f(M - Mn);
    L *= sc;
#pragma unroll
    for (int i = 0; i < DPT; ++i) O[i] *= sc;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float wt = (mc[c] == -INFINITY) ? 0.f : exp2f(mc[c] - Mn);
      L += wt * lc[c];
#pragma unroll
      for (int i = 0; i < DPT / 4; ++i) {
        O[4 * i] += wt * oc[c][i].x; O[4 * i + 1] += wt * oc[c][i].y;
        O[4 * i + 2] += wt * oc[c][i].z; O[4 * i + 3] += wt * oc[c][i].w;
      }
    }
    M = Mn;
    // the partials read (rows past the last query row too) go back to EXCH_EMPTY
#pragma unroll
    for (int c = 0; c < 8; ++c)
      if (c0 + c < a.n_split) {
        const size_t pi = (tile * a.n_split + c0 + c) * ATT_ROWS + row;
#pragma unroll
        for (int i = 0; i < DPT / 4; ++i) st16_empty(ro, (unsigned)((pi * DH + d0 + 4 * i) * 4));
        if (d0 == 0) {
          st4_coherent(rm, (unsigned)(pi * 2 * 4), EXCH_EMPTY);
          st4_coherent(rm, (unsigned)(pi * 2 * 4 + 4), EXCH_EMPTY);
        }
      }
  }
  if (r >= gq * a.H) return;
  const int tok = s * a.H + r % a.H, col = (g * gq + r / a.H) * DH + d0;
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int i = 0; i < DPT; ++i) Act<AT>::st((XT*)a.o, act_idx(tok, col + i, a.ntt), O[i] * inv);
}

// ------------------------------------------------------------------ in_proj, time embedding, verify

// h = x W_in^T + b_in + temb[seq]; writes h, hb = h * gain, ssp partial sums.
// grid (width/64, M_pad/16); block 256: channel n = bx*64 + t%64, tokens by*16 + (t/64)*4 + i.
// x rows and W_in rows of the block are staged in LDS with independent loads.
template <int WT_IN, int AT>
__global__ __launch_bounds__(256) void in_proj_kernel(const float* x, const void* w_in, const float* b_in,
                                                      const float* temb, int temb_stride, int M, int M_pad,
                                                      int A, int H, int width, float* h, void* hb,
                                                      const float* gain, size_t gain_stride, float* ssp) {
  typedef typename Act<AT>::T XT;
  __shared__ float xs[16][65];
  __shared__ float ws[64][65];
  const int n0 = blockIdx.x * 64, t0 = blockIdx.y * 16;
#pragma unroll 4
  for (int e = threadIdx.x; e < 16 * A; e += 256) {
    const int r = e / A, k = e % A, tok = t0 + r;
    xs[r][k] = tok < M ? x[(size_t)tok * A + k] : 0.f;
  }
#pragma unroll 8
  for (int e = threadIdx.x; e < 64 * A; e += 256) {
    const int r = e / A, k = e % A;
    const size_t idx = (size_t)(n0 + r) * A + k;
    ws[r][k] = (WT_IN == WT_BF16) ? bf16_to_f32(((const uint16_t*)w_in)[idx]) : ((const float*)w_in)[idx];
  }
  const int nl = threadIdx.x & 63, n = n0 + nl;
  const float bias = b_in[n];
  float tv[4], gn[4];  // per row: its sequence's temb and norm gain (gain_stride 0: one gain for all rows)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tok = t0 + (threadIdx.x >> 6) * 4 + i;
    tv[i] = tok < M ? temb[(size_t)(tok / H) * temb_stride + n] : 0.f;
    gn[i] = gain[(size_t)(min(tok, M - 1) / H) * gain_stride + n];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = (threadIdx.x >> 6) * 4 + i, tok = t0 + rl;
    float acc = 0.f;
    const bool valid = tok < M;
    if (valid) {
      acc = bias + tv[i];
      for (int k = 0; k < A; ++k) acc += xs[rl][k] * ws[nl][k];
      h[(size_t)tok * width + n] = acc;
      Act<AT>::st((XT*)hb, act_idx(tok, n, M_pad / 16), acc * gn[i]);
    }
    float sq = acc * acc;
    sq += __shfl_xor(sq, 1, 16);
    sq += __shfl_xor(sq, 2, 16);
    sq += __shfl_xor(sq, 4, 16);
    sq += __shfl_xor(sq, 8, 16);
    if ((threadIdx.x & 15) == 0 && tok < M_pad) ssp[(size_t)(n / 16) * M_pad + tok] = sq;
  }
}

// t[k] = k / steps, the Euler step times (rounded from fp64, as the host computes them).
__global__ void step_times_kernel(float* t, int steps) {
  for (int k = threadIdx.x; k < steps; k += blockDim.x) t[k] = (float)((double)k / (double)steps);
}

// v in every 32-bit word of n16 16-byte units (a clear that graph capture records as a kernel).
__global__ void fill16_kernel(uint4* p, size_t n16, unsigned v) {
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n16; e += (size_t)gridDim.x * blockDim.x)
    p[e] = make_uint4(v, v, v, v);
}

// phi(t) for n_t times: [sin(2 pi t / p_i) | cos(2 pi t / p_i)], p_i geometric 4e-3 .. 4 (fp64 math).
__global__ void sinusoid_kernel(const float* t, int width, float* phi) {
  const int it = blockIdx.y;
  const int half = width / 2;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < half; i += gridDim.x * blockDim.x) {
    double frac = (half > 1) ? (double)i / (double)(half - 1) : 0.0;
    double period = 4e-3 * pow(4.0 / 4e-3, frac);
    double ang = 2.0 * 3.14159265358979323846 * (double)t[it] / period;
    phi[(size_t)it * width + i] = (float)sin(ang);
    phi[(size_t)it * width + half + i] = (float)cos(ang);
  }
}

// y[it][n] = act(W[n] . x[it] + b[n]); one wave per output row. act: 0 none, 1 silu.
// y[step][ch] = sum_k W(ch, k) x[step][k] (+ add[ch] for ch < n_add) over packed bf16 weights
// [n_tiles][KB][64][8] (the GEMMs' operand order: lane (k%32/8)*16 + ch%16 holds inputs k..k+7 of
// channel ch). Grid (tiles, steps), one workgroup per 16-channel tile. It builds the time-modulated
// expert's per-step biases W . shift, once per step count, outside the step loop.
__global__ __launch_bounds__(256) void packed_gemv_kernel(const uint16_t* w, int KB, const float* x, int x_stride,
                                                          const float* add, int n_add, float* y, int y_stride) {
  __shared__ float part[16][16];
  const int tile = blockIdx.x, step = blockIdx.y, c = threadIdx.x & 15, grp = threadIdx.x >> 4;
  const float* xs = x + (size_t)step * x_stride;
  float acc = 0.f;
  for (int kb = grp; kb < KB; kb += 16)
    for (int q = 0; q < 4; ++q) {
      const uint16_t* f = w + (((size_t)tile * KB + kb) * 64 + q * 16 + c) * 8;
      for (int e = 0; e < 8; ++e) acc += bf16_to_f32(f[e]) * xs[kb * 32 + q * 8 + e];
    }
  part[grp][c] = acc;
  __syncthreads();
  if (threadIdx.x < 16) {
    float sum = 0.f;
    for (int g = 0; g < 16; ++g) sum += part[g][threadIdx.x];
    const int ch = tile * 16 + threadIdx.x;
    y[(size_t)step * y_stride + ch] = sum + ((add && ch < n_add) ? add[ch] : 0.f);
  }
}

// Rows x [M][w] fp32 as a GEMM input: hb = x * gain in fragment order (act_idx, M_pad / 16 token
// tiles, bf16), the per-16-channel partial sums of x^2 [w/16][M_pad] the consumer's 1/rms needs,
// and optionally x itself into the fp32 residual h [M_pad][w]. Padding rows are zero. Grid
// (w / 16 / 4, M_pad / 64); thread -> (token, 16-channel group).
__global__ __launch_bounds__(256) void stage_rows_kernel(const float* x, int M, int Mp, int w, const float* gain,
                                                         float* h_out, uint16_t* hb, float* ssp) {
  const int grp = blockIdx.x * 4 + (threadIdx.x >> 6), tok = blockIdx.y * 64 + (threadIdx.x & 63);
  if (grp * 16 >= w || tok >= Mp) return;
  float ss = 0.f;
  for (int c = 0; c < 16; ++c) {
    const int k = grp * 16 + c;
    const float v = tok < M ? x[(size_t)tok * w + k] : 0.f;
    ss += v * v;
    if (h_out) h_out[(size_t)tok * w + k] = v;
    hb[act_idx(tok, k, Mp / 16)] = f32_to_bf16(v * gain[k]);
  }
  ssp[(size_t)grp * Mp + tok] = ss;
}

// g[step][i] = gain[i] * (1 + scale[step][i]): a modulated norm's gain for one step
__global__ void mod_gain_kernel(const float* gain, const float* scale, int scale_stride, int w, float* g) {
  const int step = blockIdx.y, i = blockIdx.x * 256 + threadIdx.x;
  if (i < w) g[(size_t)step * w + i] = gain[i] * (1.f + scale[(size_t)step * scale_stride + i]);
}

// y[it][n] = act(W[n] . x[it] + b[n]) for it < n_t; act: 0 none, 1 silu. One wave per output row n,
// 4 consecutive inputs per lane per 256-input step (K is a multiple of 256), the weight row read once
// for every 8 inputs x[it] (their dot products accumulate side by side), then one wave reduction each.
template <int WT_>
__global__ __launch_bounds__(256) void gemv_kernel(const void* w, const float* b, const float* x, int K, int N,
                                                   int act, float* y, int n_t) {
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (n >= N) return;
  for (int it0 = 0; it0 < n_t; it0 += 8) {
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.f;
    for (int k = lane * 4; k < K; k += 256) {
      float wv[4];
      if constexpr (WT_ == WT_BF16) {
        const uint2 p = *(const uint2*)((const uint16_t*)w + (size_t)n * K + k);
        wv[0] = bf16_to_f32((uint16_t)(p.x & 0xffffu));
        wv[1] = bf16_to_f32((uint16_t)(p.x >> 16));
        wv[2] = bf16_to_f32((uint16_t)(p.y & 0xffffu));
        wv[3] = bf16_to_f32((uint16_t)(p.y >> 16));
      } else {
        const float4 p = *(const float4*)((const float*)w + (size_t)n * K + k);
        wv[0] = p.x; wv[1] = p.y; wv[2] = p.z; wv[3] = p.w;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (it0 + j < n_t) {
          const float4 xv = *(const float4*)(x + (size_t)(it0 + j) * K + k);
          acc[j] += wv[0] * xv.x + wv[1] * xv.y + wv[2] * xv.z + wv[3] * xv.w;
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v = acc[j];
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
      if (lane == 0 && it0 + j < n_t) {
        v += b[n];
        if (act == 1) v = v / (1.f + expf(-v));
        y[(size_t)(it0 + j) * N + n] = v;
      }
    }
  }
}

// The start of a verification pass in one launch: rows y < n_tau of the grid write phi(tau_y) as
// sinusoid_kernel does, row n_tau writes x_j = (1 - tau_j) noise + tau_j draft into rows j*H + i.
__global__ void verify_start_kernel(const float* draft, const float* noise, const float* taus, int n_tau, int H, int A,
                                    float* x, int width, float* phi) {
  const int it = blockIdx.y;
  if (it < n_tau) {
    const int half = width / 2;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < half; i += gridDim.x * blockDim.x) {
      double frac = (half > 1) ? (double)i / (double)(half - 1) : 0.0;
      double period = 4e-3 * pow(4.0 / 4e-3, frac);
      double ang = 2.0 * 3.14159265358979323846 * (double)taus[it] / period;
      phi[(size_t)it * width + i] = (float)sin(ang);
      phi[(size_t)it * width + half + i] = (float)cos(ang);
    }
    return;
  }
  const int total = n_tau * H * A;
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < total; e += gridDim.x * blockDim.x) {
    int j = e / (H * A), ia = e % (H * A);
    float tau = taus[j];
    x[e] = (1.f - tau) * noise[ia] + tau * draft[ia];
  }
}

// ------------------------------------------------------------------ modulation vectors of a verification pass
// A time-modulated expert's verification pass (one flow time per sequence) forms every layer's
// modulation vectors from the flow times' temb inside the pass, in three launches over job tables
// built at create: the linear maps of temb, the modulated norm gains, and the shift biases W . shift.

// y[it][n] = W[n] . x[it] + b[n] for it < n_t, job blockIdx.y, bf16 weights. One wave per 4 output rows
// (grid.x = N / 16 for 4 waves): every 256-input step loads each input's 4 values once for the 4 rows
// and each row's 4 weights once for 4 inputs (inputs 4 at a time), then one wave reduction per sum.
struct GemvJob {
  const uint16_t* w;
  const float* b;
  const float* x;
  float* y;
  int K, N;
};
__global__ __launch_bounds__(256) void gemv_jobs_kernel(const GemvJob* jobs, int n_t) {
  const GemvJob jb = jobs[blockIdx.y];
  const int n0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 4;
  const int lane = threadIdx.x & 63;
  if (n0 >= jb.N) return;
  for (int it0 = 0; it0 < n_t; it0 += 4) {
    float acc[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[r][j] = 0.f;
    for (int k = lane * 4; k < jb.K; k += 256) {
      float4 xv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xv[j] = it0 + j < n_t ? *(const float4*)(jb.x + (size_t)(it0 + j) * jb.K + k) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint2 p = *(const uint2*)(jb.w + (size_t)(n0 + r) * jb.K + k);
        const float w0 = bf16_to_f32((uint16_t)(p.x & 0xffffu)), w1 = bf16_to_f32((uint16_t)(p.x >> 16));
        const float w2 = bf16_to_f32((uint16_t)(p.y & 0xffffu)), w3 = bf16_to_f32((uint16_t)(p.y >> 16));
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[r][j] += w0 * xv[j].x + w1 * xv[j].y + w2 * xv[j].z + w3 * xv[j].w;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float v = acc[r][j];
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
        if (lane == 0 && it0 + j < n_t) jb.y[(size_t)(it0 + j) * jb.N + n0 + r] = v + jb.b[n0 + r];
      }
  }
}

// g[it][i] = gain[i] (1 + scale[it][i]) for it < n_t, job blockIdx.z (grid (w / 256, n_t, jobs))
struct GainJob {
  const float* gain;
  const float* scale;
  float* g;
  int scale_stride;
};
__global__ void mod_gain_jobs_kernel(const GainJob* jobs, int w) {
  const GainJob jb = jobs[blockIdx.z];
  const int it = blockIdx.y, i = blockIdx.x * 256 + threadIdx.x;
  if (i < w) jb.g[(size_t)it * w + i] = jb.gain[i] * (1.f + jb.scale[(size_t)it * jb.scale_stride + i]);
}

// y[it][ch] = sum_k W(ch, k) x[it][k] (+ add[ch] for ch < n_add) over packed bf16 weights (the layout
// packed_gemv_kernel reads) for it < n_t, job blockIdx.y, tiles 8 blockIdx.x .. + 8. Thread -> (k-group
// wave, lane = 16 q + c): for each of its k-blocks it loads the 8 inputs k-block * 32 + 8 q .. + 8 of 4
// rows once and reuses them for the 8 tiles' pieces of channel c, so input loads do not outnumber weight
// loads; partial sums meet across q by shuffles and across the 4 waves in LDS.
struct PackedGemvJob {
  const uint16_t* w;
  const float* x;
  const float* add;
  float* y;
  int KB, tiles, x_stride, y_stride, n_add;
};
constexpr int PGJ_TILES = 8;
constexpr int PGJ_ROWS = 4;
__global__ __launch_bounds__(256) void packed_gemv_jobs_kernel(const PackedGemvJob* jobs, int n_t) {
  __shared__ float part[4][PGJ_TILES][PGJ_ROWS][16];
  const PackedGemvJob jb = jobs[blockIdx.y];
  const int t0 = blockIdx.x * PGJ_TILES;
  if (t0 >= jb.tiles) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, q = lane >> 4, c = lane & 15;
  for (int it0 = 0; it0 < n_t; it0 += PGJ_ROWS) {
    float acc[PGJ_TILES][PGJ_ROWS];
#pragma unroll
    for (int u = 0; u < PGJ_TILES; ++u)
#pragma unroll
      for (int j = 0; j < PGJ_ROWS; ++j) acc[u][j] = 0.f;
    for (int kb = wave; kb < jb.KB; kb += 4) {
      float xv[PGJ_ROWS][8];
#pragma unroll
      for (int j = 0; j < PGJ_ROWS; ++j) {
        const int row = min(it0 + j, n_t - 1);
        const float* xs = jb.x + (size_t)row * jb.x_stride + kb * 32 + q * 8;
        const float4 x0 = *(const float4*)xs, x1 = *(const float4*)(xs + 4);
        xv[j][0] = x0.x; xv[j][1] = x0.y; xv[j][2] = x0.z; xv[j][3] = x0.w;
        xv[j][4] = x1.x; xv[j][5] = x1.y; xv[j][6] = x1.z; xv[j][7] = x1.w;
      }
#pragma unroll
      for (int u = 0; u < PGJ_TILES; ++u) {
        const int tile = min(t0 + u, jb.tiles - 1);
        const uint4 p = *(const uint4*)(jb.w + (((size_t)tile * jb.KB + kb) * 64 + lane) * 8);
        const uint32_t pw[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float w0 = bf16_to_f32((uint16_t)(pw[e] & 0xffffu)), w1 = bf16_to_f32((uint16_t)(pw[e] >> 16));
#pragma unroll
          for (int j = 0; j < PGJ_ROWS; ++j) acc[u][j] += w0 * xv[j][2 * e] + w1 * xv[j][2 * e + 1];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < PGJ_TILES; ++u)
#pragma unroll
      for (int j = 0; j < PGJ_ROWS; ++j) {
        float v = acc[u][j];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (q == 0) part[wave][u][j][c] = v;
      }
    __syncthreads();
    for (int o = threadIdx.x; o < PGJ_TILES * PGJ_ROWS * 16; o += 256) {  // (tile u, row j, channel) sums over the waves
      const int u = o >> 6, j = (o >> 4) & 3, cc = o & 15;
      if (t0 + u < jb.tiles && it0 + j < n_t) {
        const float sum = part[0][u][j][cc] + part[1][u][j][cc] + part[2][u][j][cc] + part[3][u][j][cc];
        const int ch = (t0 + u) * 16 + cc;
        jb.y[(size_t)(it0 + j) * jb.y_stride + ch] = sum + ((jb.add && ch < jb.n_add) ? jb.add[ch] : 0.f);
      }
    }
    __syncthreads();
  }
}

// Per-call verification parameters, written on the stream so a captured graph reads them.
__global__ void set_verify_params_kernel(int* slots, int n_tau, int slot, float* params, float delta) {
  if (threadIdx.x < n_tau) slots[threadIdx.x] = slot;
  if (threadIdx.x == 0) params[0] = delta;
}

__global__ void copy_f32_kernel(const float* src, float* dst, int n) {
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < n; e += gridDim.x * blockDim.x) dst[e] = src[e];
}

}  // namespace ae
