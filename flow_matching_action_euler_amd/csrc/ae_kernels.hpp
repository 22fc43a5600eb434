// Device code of the action-expert denoise loop for gfx950 (CDNA4).
//
// One Euler step of the suffix (DM0.5 guide, sections 5.2-5.3) runs as:
//   in_proj   : h = x W_in^T + b_in + temb(t)                      (tiny, FMA)
//   per layer : qkv  = rmsnorm(h) W_qkv^T, RoPE on q/k             (gemm_kernel<EPI_QKV>)
//               attn = softmax(q [Kp;k]^T / sqrt(dh)) [Vp;v]        (attn_kernel + attn_combine)
//               h   += o W_o^T                                       (gemm_kernel<EPI_RESID>)
//               u    = gelu(rmsnorm(h) W_g^T) * (rmsnorm(h) W_u^T)  (gemm_kernel<EPI_GEGLU>)
//               h   += u W_d^T                                       (gemm_kernel<EPI_RESID>)
//   out_proj  : v = rmsnorm(h) W_out^T + b_out; x += dt v          (gemm_kernel<EPI_OUT>)
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

enum WType { WT_BF16 = 0, WT_FP8 = 1, WT_F32 = 2 };
enum AType { AT_BF16 = 0, AT_F32 = 1 };
enum Epi { EPI_QKV = 0, EPI_RESID = 1, EPI_GEGLU = 2, EPI_OUT = 3 };

constexpr int TOKG = 64;   // tokens per workgroup (4 MFMA column tiles of 16)
constexpr int KBLK = 32;   // inputs per k-block

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

// ------------------------------------------------------------------ GEMM

struct GemmArgs {
  const void* w;        // packed weights [n_tiles][KB][64][8]
  const float* wscale;  // fp8: scale per packed channel (tile*16 + c); else null
  const void* x;        // activations [M_pad][K], gain-scaled, not normalised
  const float* ssp_in;  // [g_in][M_pad] partial sums of h^2 (null: no RMS scaling)
  int g_in;
  float inv_width;      // 1 / width of the normalised vector
  float eps;
  int M, M_pad, K, S;   // rows, padded rows, inputs, k-splits
  int ldx;              // row stride of x in elements (K plus a 128-byte pad)
  int ldo;              // row stride of the activation written by the epilogue
  float* part;          // split-K partials [S][n_z][n_groups][NT*64*16]
  unsigned* counters;   // [n_z][n_groups], zero between launches
  // EPI_QKV
  void* q_out; void* k_out; void* v_out;   // [M_pad][n_q*dh], [M_pad][n_kv*dh] x2
  const float* rope_cs;                    // [H][dh/2][2] cos, sin at positions P + t
  int n_q, n_kv, dh, H;
  int ldkv;                                // row stride of the suffix k / v buffers
  // EPI_RESID
  float* h;              // [M_pad][N] residual, updated in place
  void* hb;              // [M_pad][N] copy h * gain_next for the next consumer
  const float* gain_next;
  float* ssp_out;        // [N/16][M_pad]
  int N;                 // logical outputs
  // EPI_GEGLU
  void* u_out;           // [M_pad][F]
  // EPI_OUT
  const float* bias;     // [A]
  float* xio;            // denoise: x [M_pad][A] updated in place; verify: v out
  int A;
  float dt;              // > 0: x += dt * v; 0: store v
};

// Load the weight fragment of (tile, kb) for this lane as MFMA A operand.
template <int WT>
__device__ __forceinline__ void load_w(const void* w, size_t tile, int KB, int kb, int lane, bf16x8& a, f32x4& f0, f32x4& f1) {
  size_t idx = ((tile * KB + kb) * 64 + lane);
  if constexpr (WT == WT_BF16) {
    a = __builtin_bit_cast(bf16x8, ((const uint4*)w)[idx]);
  } else if constexpr (WT == WT_FP8) {
    a = fp8x8_to_bf16x8(((const uint2*)w)[idx]);
  } else {
    const float4* p = (const float4*)w + idx * 2;
    float4 u = p[0], v = p[1];
    f0 = f32x4{u.x, u.y, u.z, u.w};
    f1 = f32x4{v.x, v.y, v.z, v.w};
  }
}

// Device-coherent publication of one value: the store writes through to the
// point of coherence (sc1), so workgroups on other XCDs read it without any
// L2 write-back or invalidation.
__device__ __forceinline__ void st_coherent(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ float ld_coherent(const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
// Wait until this thread's outstanding memory operations have completed.
__device__ __forceinline__ void wait_mem() { __builtin_amdgcn_s_waitcnt(0); }

// Reduce 4 waves' accumulators (+ split-K partials) into LDS res[NT][64][16] and
// return whether this workgroup runs the epilogue.
template <int NT>
__device__ __forceinline__ bool gemm_reduce(const GemmArgs& a, f32x4 (&acc)[NT][4], float* red, float* res,
                                            int g, int s, int z, int n_groups) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // each wave writes its accumulators: red[wave][nt][tok 64][c 16]
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        int c = 4 * (lane >> 4) + v, tok = tt * 16 + (lane & 15);
        red[((wave * NT + nt) * TOKG + tok) * 16 + c] = acc[nt][tt][v];
      }
  __syncthreads();
  const int tile_elems = NT * TOKG * 16;
  for (int e = threadIdx.x; e < tile_elems; e += 256)
    res[e] = red[e] + red[tile_elems + e] + red[2 * tile_elems + e] + red[3 * tile_elems + e];
  __syncthreads();
  if (a.S == 1) return true;
  // split-K: publish the partial (write-through), count arrivals; the last
  // arriver of (z, g) sums the S partials in split order (deterministic).
  const int n_z = gridDim.z;
  float* mine = a.part + (((size_t)s * n_z + z) * n_groups + g) * tile_elems;
#pragma unroll
  for (int i = 0; i < NT * 4; ++i) st_coherent(mine + threadIdx.x + 256 * i, res[threadIdx.x + 256 * i]);
  wait_mem();
  __syncthreads();
  __shared__ unsigned ticket;
  unsigned* cnt = a.counters + z * n_groups + g;
  if (threadIdx.x == 0) {
    ticket = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (ticket == (unsigned)a.S - 1) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (ticket != (unsigned)a.S - 1) return false;
#pragma unroll
  for (int i = 0; i < NT * 4; ++i) {
    const int e = threadIdx.x + 256 * i;
    float v[4];
#pragma unroll
    for (int ss = 0; ss < 4; ++ss)
      v[ss] = ss < a.S ? ld_coherent(a.part + (((size_t)ss * n_z + z) * n_groups + g) * tile_elems + e) : 0.f;
    res[e] = ((v[0] + v[1]) + v[2]) + v[3];
  }
  __syncthreads();
  return true;
}

// Y = X W^T over the workgroup's channel tiles [g*NT, g*NT+NT), k-split s and
// token group z, then the epilogue EPI. Block = 256 threads (4 waves); wave w
// takes a contiguous run of at most KBW k-blocks per pass and issues every
// weight and activation fragment of the pass before its first MFMA, so a
// wave has (NT + 4) * KBW 16-byte loads in flight.
template <int WT, int AT, int EPI, int NT, int KBW>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
  typedef typename Act<AT>::T XT;
  extern __shared__ float smem[];
  float* red = smem;                        // [4][NT][64][16]
  float* res = smem + 4 * NT * TOKG * 16;   // [NT][64][16]
  float* inv_rms = res + NT * TOKG * 16;    // [64]

  const int g = blockIdx.x, s = blockIdx.y, z = blockIdx.z;
  const int n_groups = gridDim.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int KB = a.K / KBLK;
  const int kb_per = KB / a.S;
  const int per_wave = (kb_per + 3) / 4;
  const int kw0 = s * kb_per + wave * per_wave;
  const int kw1 = min(s * kb_per + kb_per, kw0 + per_wave);
  const int tok0 = z * TOKG;
  const int tt_n = min(4, (a.M_pad - tok0) / 16);
  const XT* X = (const XT*)a.x;

  // partial sums of h^2 for token (t & 63), groups (t >> 6) + 4 i: loads issued now, summed after the MFMAs
  float ssq = 0.f;
  if (a.ssp_in != nullptr) {
    const int tok = tok0 + (threadIdx.x & 63);
    if (tok < a.M_pad) {
#pragma unroll 16
      for (int gi = threadIdx.x >> 6; gi < a.g_in; gi += 4) ssq += a.ssp_in[(size_t)gi * a.M_pad + tok];
    }
  }

  f32x4 acc[NT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[nt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int xrow = lane & 15, xk = (lane >> 4) * 8;
  for (int kp = kw0; kp < kw1; kp += KBW) {
    if constexpr (AT == AT_BF16) {
      bf16x8 wa[NT][KBW];
      bf16x8 xb[4][KBW];
      f32x4 d0, d1;
#pragma unroll
      for (int j = 0; j < KBW; ++j)
        if (kp + j < kw1)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) load_w<WT>(a.w, (size_t)g * NT + nt, KB, kp + j, lane, wa[nt][j], d0, d1);
#pragma unroll
      for (int j = 0; j < KBW; ++j)
        if (kp + j < kw1)
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
            if (tt < tt_n)
              xb[tt][j] = __builtin_bit_cast(bf16x8, *(const uint4*)(X + (size_t)(tok0 + tt * 16 + xrow) * a.ldx + (kp + j) * KBLK + xk));
#pragma unroll
      for (int j = 0; j < KBW; ++j)
        if (kp + j < kw1)
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
            if (tt < tt_n)
#pragma unroll
              for (int nt = 0; nt < NT; ++nt)
                acc[nt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[nt][j], xb[tt][j], acc[nt][tt], 0, 0, 0);
    } else {
      for (int kb = kp; kb < min(kw1, kp + KBW); ++kb) {
        bf16x8 dummy;
        f32x4 wf0[NT], wf1[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) load_w<WT>(a.w, (size_t)g * NT + nt, KB, kb, lane, dummy, wf0[nt], wf1[nt]);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          if (tt < tt_n) {
            const float* xp = (const float*)X + (size_t)(tok0 + tt * 16 + xrow) * a.ldx + kb * KBLK + xk;
            float4 u = ((const float4*)xp)[0], v = ((const float4*)xp)[1];
            float bx[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              float wx[8] = {wf0[nt][0], wf0[nt][1], wf0[nt][2], wf0[nt][3], wf1[nt][0], wf1[nt][1], wf1[nt][2], wf1[nt][3]};
#pragma unroll
              for (int jj = 0; jj < 8; ++jj)
                acc[nt][tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(wx[jj], bx[jj], acc[nt][tt], 0, 0, 0);
            }
          }
        }
      }
    }
  }

  // inverse RMS of this group's tokens: sum the producer's partial sums loaded above
  {
    float* part4 = red;  // [4][64], red is free again after gemm_reduce's first barrier
    __syncthreads();
    part4[threadIdx.x] = ssq;
    __syncthreads();
    if (threadIdx.x < TOKG) {
      float r = 1.f;
      if (a.ssp_in != nullptr) {
        float t4 = part4[threadIdx.x] + part4[64 + threadIdx.x] + part4[128 + threadIdx.x] + part4[192 + threadIdx.x];
        r = rsqrtf(t4 * a.inv_width + a.eps);
      }
      inv_rms[threadIdx.x] = r;
    }
    __syncthreads();
  }
  if (!gemm_reduce<NT>(a, acc, red, res, g, s, z, n_groups)) return;

  // ---------------- epilogues: thread -> (channel c = t%16, tokens t/16 + 16 i)
  const int c = threadIdx.x & 15;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const size_t tile = (size_t)g * NT + nt;
    if constexpr (EPI == EPI_GEGLU) {
      if (nt & 1) continue;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tl = (threadIdx.x >> 4) + 16 * i;
      const int tok = tok0 + tl;
      const bool valid = tok < a.M;
      float val = res[(nt * TOKG + tl) * 16 + c] * inv_rms[tl];
      if constexpr (WT == WT_FP8) {
        if constexpr (EPI != EPI_GEGLU) val *= a.wscale[tile * 16 + c];
      }
      if constexpr (EPI == EPI_QKV) {
        // packed tiles: q heads, then k heads (RoPE pairs d, d+dh/2 share a tile), then v
        const int tiles_per_head = a.dh / 16;
        const int q_tiles = a.n_q * tiles_per_head, k_tiles = a.n_kv * tiles_per_head;
        const int half = a.dh / 2;
        int t_in = (int)tile;
        if (t_in < q_tiles + k_tiles) {
          const bool is_q = t_in < q_tiles;
          const int tt2 = is_q ? t_in : t_in - q_tiles;
          const int head = tt2 / tiles_per_head, pair = tt2 % tiles_per_head;
          const int d = pair * 8 + (c & 7);
          float partner = res[(nt * TOKG + tl) * 16 + (c ^ 8)] * inv_rms[tl];
          const int t = tok % a.H;
          float cs = a.rope_cs[((size_t)t * half + d) * 2 + 0];
          float sn = a.rope_cs[((size_t)t * half + d) * 2 + 1];
          float out;
          int dfull;
          if (c < 8) { out = val * cs - partner * sn; dfull = d; }
          else { out = partner * sn + val * cs; dfull = half + d; }
          if (valid) {
            if (is_q) Act<AT>::st((XT*)a.q_out, (size_t)tok * a.ldo + head * a.dh + dfull, out);
            else Act<AT>::st((XT*)a.k_out, (size_t)tok * a.ldkv + head * a.dh + dfull, out);
          }
        } else {
          const int col = (t_in - q_tiles - k_tiles) * 16 + c;
          if (valid) Act<AT>::st((XT*)a.v_out, (size_t)tok * a.ldkv + col, val);
        }
      } else if constexpr (EPI == EPI_RESID) {
        const int n = (int)tile * 16 + c;
        float hn = 0.f;
        if (valid) {
          hn = a.h[(size_t)tok * a.N + n] + val;
          a.h[(size_t)tok * a.N + n] = hn;
          Act<AT>::st((XT*)a.hb, (size_t)tok * a.ldo + n, hn * a.gain_next[n]);
        }
        float sq = hn * hn;
        sq += __shfl_xor(sq, 1, 16);
        sq += __shfl_xor(sq, 2, 16);
        sq += __shfl_xor(sq, 4, 16);
        sq += __shfl_xor(sq, 8, 16);
        if (c == 0 && tok < a.M_pad) a.ssp_out[tile * a.M_pad + tok] = sq;
      } else if constexpr (EPI == EPI_GEGLU) {
        float up = res[((nt + 1) * TOKG + tl) * 16 + c] * inv_rms[tl];
        if constexpr (WT == WT_FP8) {
          val *= a.wscale[tile * 16 + c];
          up *= a.wscale[(tile + 1) * 16 + c];
        }
        const int f = (int)(tile / 2) * 16 + c;
        if (valid) Act<AT>::st((XT*)a.u_out, (size_t)tok * a.ldo + f, gelu_tanh(val) * up);
      } else {  // EPI_OUT
        const int n = (int)tile * 16 + c;
        if (valid && n < a.A) {
          float v = val + a.bias[n];
          if (a.dt > 0.f) a.xio[(size_t)tok * a.A + n] += a.dt * v;
          else a.xio[(size_t)tok * a.A + n] = v;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ attention

struct AttnArgs {
  const void* q;          // [M_pad][n_q*dh] (rotated)
  const void* ks;         // suffix keys [M_pad][n_kv*dh] (rotated)
  const void* vs;         // suffix values
  const void* kcache;     // prefix K, slot-major [slots][L][P][n_kv][dh]
  const void* vcache;
  const int* seq_slot;    // prefix slot of each sequence
  size_t slot_stride;     // elements per slot
  size_t layer_off;       // elements to this layer inside a slot
  int P, H, n_q, n_kv, dh, KC;
  int ldq, ldkv, ldo;     // row strides of q, suffix k/v and the output o
  int n_qt, n_chunks;
  float scale_log2;       // log2(e) / sqrt(dh)
  float* opart;           // [z][qt][chunk][64][dh]
  float* mlpart;          // [z][qt][chunk][64][2]  (running max in log2 units, sum)
};

// One workgroup: 64 query rows (of one sequence and kv head; rows r = j*H + t
// for query head j of the group) against one chunk of KC keys of
// [prefix ; suffix]. Writes the chunk's softmax partials (m, l, O).
template <int AT>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  typedef typename Act<AT>::T XT;
  extern __shared__ unsigned char smem_raw[];
  const int dh = a.dh, KC = a.KC;
  const int ldk = dh + (AT == AT_BF16 ? 8 : 4);    // padded row strides (elements)
  const int ldv = KC + (AT == AT_BF16 ? 8 : 4);
  const int ldp = KC + (AT == AT_BF16 ? 8 : 4);
  XT* Ks = (XT*)smem_raw;                 // [KC][ldk]
  XT* VT = Ks + (size_t)KC * ldk;         // [dh][ldv]
  XT* Ps = VT + (size_t)dh * ldv;         // [64][ldp]

  const int chunk = blockIdx.x, qt = blockIdx.y, zz = blockIdx.z;
  const int s = zz / a.n_kv, g = zz % a.n_kv;
  const int gq = a.n_q / a.n_kv;           // query heads per kv head
  const int R = gq * a.H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j0 = chunk * KC;
  const int n_keys = a.P + a.H;
  const XT* kc = (const XT*)a.kcache + (size_t)a.seq_slot[s] * a.slot_stride + a.layer_off;
  const XT* vc = (const XT*)a.vcache + (size_t)a.seq_slot[s] * a.slot_stride + a.layer_off;
  const XT* ks = (const XT*)a.ks;
  const XT* vs = (const XT*)a.vs;

  // stage K rows and V^T of this chunk (zeros past the last key), 16 bytes per load
  constexpr int VE = 16 / sizeof(XT);
  const int vpr = dh / VE;
#pragma unroll 8
  for (int e = threadIdx.x; e < KC * vpr; e += 256) {
    const int kr = e / vpr, d0 = (e % vpr) * VE;
    const int j = j0 + kr;
    uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
    if (j < a.P) {
      const size_t off = ((size_t)j * a.n_kv + g) * dh + d0;
      kv = *(const uint4*)(kc + off);
      vv = *(const uint4*)(vc + off);
    } else if (j < n_keys) {
      const size_t off = (size_t)(s * a.H + (j - a.P)) * a.ldkv + (size_t)g * dh + d0;
      kv = *(const uint4*)(ks + off);
      vv = *(const uint4*)(vs + off);
    }
    *(uint4*)(Ks + (size_t)kr * ldk + d0) = kv;
    const XT* vp = (const XT*)&vv;
#pragma unroll
    for (int i = 0; i < VE; ++i) VT[(size_t)(d0 + i) * ldv + kr] = vp[i];
  }
  __syncthreads();

  // this wave's 16 query rows
  const int r_lane = qt * 64 + wave * 16 + (lane & 15);
  const bool r_ok = r_lane < R;
  const int jh = r_ok ? r_lane / a.H : 0, t = r_ok ? r_lane % a.H : 0;
  const XT* qrow = (const XT*)a.q + (size_t)(s * a.H + t) * a.ldq + (size_t)(g * gq + jh) * dh;
  const int kofs = (lane >> 4) * 8;

  // S = Q K^T for KC keys: KC/16 column tiles
  const int n_kt = KC / 16;
  f32x4 sacc[8];  // KC <= 128
  for (int kt = 0; kt < 8; ++kt) sacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (AT == AT_BF16) {
    bf16x8 qa[8];  // dh <= 256: all query fragments of this lane, loaded before the first MFMA
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
      if (kb < dh / KBLK)
        qa[kb] = r_ok ? __builtin_bit_cast(bf16x8, *(const uint4*)(qrow + kb * KBLK + kofs))
                      : __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
      if (kb < dh / KBLK)
        for (int kt = 0; kt < n_kt; ++kt) {
          bf16x8 kb8 = __builtin_bit_cast(bf16x8, *(const uint4*)(Ks + (size_t)(kt * 16 + (lane & 15)) * ldk + kb * KBLK + kofs));
          sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kb], kb8, sacc[kt], 0, 0, 0);
        }
  } else {
    for (int kb = 0; kb < dh / KBLK; ++kb) {
      float qa[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) qa[jj] = r_ok ? (float)qrow[kb * KBLK + kofs + jj] : 0.f;
      for (int kt = 0; kt < n_kt; ++kt) {
        const XT* kp = Ks + (size_t)(kt * 16 + (lane & 15)) * ldk + kb * KBLK + kofs;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[jj], (float)kp[jj], sacc[kt], 0, 0, 0);
      }
    }
  }
  // softmax partials over this chunk: lane holds rows 4*(lane/16)+v, key kt*16 + lane%16
  float m[4], l[4];
  for (int v = 0; v < 4; ++v) {
    float mx = -INFINITY;
    for (int kt = 0; kt < n_kt; ++kt) {
      int j = j0 + kt * 16 + (lane & 15);
      float sv = (j < n_keys) ? sacc[kt][v] * a.scale_log2 : -INFINITY;
      sacc[kt][v] = sv;
      mx = fmaxf(mx, sv);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 1, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 2, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 4, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 8, 16));
    m[v] = mx;
    float sum = 0.f;
    for (int kt = 0; kt < n_kt; ++kt) {
      float p = (mx == -INFINITY) ? 0.f : exp2f(sacc[kt][v] - mx);
      int prow = wave * 16 + 4 * (lane >> 4) + v;
      Act<AT>::st(Ps, (size_t)prow * ldp + kt * 16 + (lane & 15), p);
      sum += p;
    }
    sum += __shfl_xor(sum, 1, 16);
    sum += __shfl_xor(sum, 2, 16);
    sum += __shfl_xor(sum, 4, 16);
    sum += __shfl_xor(sum, 8, 16);
    l[v] = sum;
  }
  __syncthreads();

  // O = P V: dh/16 column tiles, KC/32 k-blocks
  float* op = a.opart + ((((size_t)zz * a.n_qt + qt) * a.n_chunks + chunk) * 64) * dh;
  float* mlp = a.mlpart + ((((size_t)zz * a.n_qt + qt) * a.n_chunks + chunk) * 64) * 2;
  const int prow_a = wave * 16 + (lane & 15);
  for (int dt = 0; dt < dh / 16; ++dt) {
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kb = 0; kb < KC / KBLK; ++kb) {
      if constexpr (AT == AT_BF16) {
        bf16x8 pa = __builtin_bit_cast(bf16x8, *(const uint4*)(Ps + (size_t)prow_a * ldp + kb * KBLK + kofs));
        bf16x8 vb = __builtin_bit_cast(bf16x8, *(const uint4*)(VT + (size_t)(dt * 16 + (lane & 15)) * ldv + kb * KBLK + kofs));
        o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, o, 0, 0, 0);
      } else {
        const XT* pp = Ps + (size_t)prow_a * ldp + kb * KBLK + kofs;
        const XT* vp = VT + (size_t)(dt * 16 + (lane & 15)) * ldv + kb * KBLK + kofs;
        for (int jj = 0; jj < 8; ++jj) o = __builtin_amdgcn_mfma_f32_16x16x4f32((float)pp[jj], (float)vp[jj], o, 0, 0, 0);
      }
    }
    for (int v = 0; v < 4; ++v) {
      int row = wave * 16 + 4 * (lane >> 4) + v;
      op[(size_t)row * dh + dt * 16 + (lane & 15)] = o[v];
    }
  }
  if ((lane & 15) == 0) {
    for (int v = 0; v < 4; ++v) {
      int row = wave * 16 + 4 * (lane >> 4) + v;
      mlp[row * 2 + 0] = m[v];
      mlp[row * 2 + 1] = l[v];
    }
  }
}

// Combine the chunks of one query row: o = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c.
// grid (R rows, n_seq * n_kv); block = dh threads (<= 256).
template <int AT>
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a, void* o_out) {
  typedef typename Act<AT>::T XT;
  const int r = blockIdx.x, zz = blockIdx.y;
  const int s = zz / a.n_kv, g = zz % a.n_kv;
  const int gq = a.n_q / a.n_kv;
  const int qt = r / 64, row = r % 64;
  const int d = threadIdx.x;
  if (d >= a.dh) return;
  const size_t base = ((size_t)zz * a.n_qt + qt) * a.n_chunks;
  // batches of 16 chunks, all loads of a batch in flight, online rescaling between batches
  float M = -INFINITY, num = 0.f, den = 0.f;
  for (int c0 = 0; c0 < a.n_chunks; c0 += 16) {
    float mc[16], lc[16], oc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = c0 + i;
      if (c < a.n_chunks) {
        mc[i] = a.mlpart[((base + c) * 64 + row) * 2];
        lc[i] = a.mlpart[((base + c) * 64 + row) * 2 + 1];
        oc[i] = a.opart[((base + c) * 64 + row) * a.dh + d];
      } else {
        mc[i] = -INFINITY; lc[i] = 0.f; oc[i] = 0.f;
      }
    }
    float Mn = M;
#pragma unroll
    for (int i = 0; i < 16; ++i) Mn = fmaxf(Mn, mc[i]);
    const float sc = (M == -INFINITY) ? 0.f : exp2f(M - Mn);
    num *= sc;
    den *= sc;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float wgt = (mc[i] == -INFINITY) ? 0.f : exp2f(mc[i] - Mn);
      num += wgt * oc[i];
      den += wgt * lc[i];
    }
    M = Mn;
  }
  const int jh = r / a.H, t = r % a.H;
  const size_t tok = (size_t)s * a.H + t;
  Act<AT>::st((XT*)o_out, tok * a.ldo + (size_t)(g * gq + jh) * a.dh + d, num / den);
}

// ------------------------------------------------------------------ in_proj, time embedding, verify

// h = x W_in^T + b_in + temb[seq]; writes h, hb = h * gain, ssp partial sums.
// grid (width/64, M_pad/16); block 256: channel n = bx*64 + t%64, tokens by*16 + (t/64)*4 + i.
// x rows and W_in rows of the block are staged in LDS with independent loads.
template <int WT_IN, int AT>
__global__ __launch_bounds__(256) void in_proj_kernel(const float* x, const void* w_in, const float* b_in,
                                                      const float* temb, int temb_stride, int M, int M_pad,
                                                      int A, int H, int width, float* h, void* hb, int ldh,
                                                      const float* gain, float* ssp) {
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
  const float bias = b_in[n], gn = gain[n];
  float tv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tok = t0 + (threadIdx.x >> 6) * 4 + i;
    tv[i] = tok < M ? temb[(size_t)(tok / H) * temb_stride + n] : 0.f;
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
      Act<AT>::st((XT*)hb, (size_t)tok * ldh + n, acc * gn);
    }
    float sq = acc * acc;
    sq += __shfl_xor(sq, 1, 16);
    sq += __shfl_xor(sq, 2, 16);
    sq += __shfl_xor(sq, 4, 16);
    sq += __shfl_xor(sq, 8, 16);
    if ((threadIdx.x & 15) == 0 && tok < M_pad) ssp[(size_t)(n / 16) * M_pad + tok] = sq;
  }
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
template <int WT_>
__global__ __launch_bounds__(256) void gemv_kernel(const void* w, const float* b, const float* x, int K, int N,
                                                   int act, float* y) {
  const int it = blockIdx.y;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (n >= N) return;
  float acc = 0.f;
  for (int k = lane; k < K; k += 64) {
    float wv = (WT_ == WT_BF16) ? bf16_to_f32(((const uint16_t*)w)[(size_t)n * K + k]) : ((const float*)w)[(size_t)n * K + k];
    acc += wv * x[(size_t)it * K + k];
  }
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) {
    float v = acc + b[n];
    if (act == 1) v = v / (1.f + expf(-v));
    y[(size_t)it * N + n] = v;
  }
}

// x_j = (1 - tau_j) noise + tau_j draft into rows j*H + i.
__global__ void interp_kernel(const float* draft, const float* noise, const float* taus, int n_tau, int H, int A, float* x) {
  const int total = n_tau * H * A;
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < total; e += gridDim.x * blockDim.x) {
    int j = e / (H * A), ia = e % (H * A);
    float tau = taus[j];
    x[e] = (1.f - tau) * noise[ia] + tau * draft[ia];
  }
}

// Endpoints, distances, prefix scan and gripper check (one workgroup).
__global__ __launch_bounds__(256) void verify_kernel(const float* x, const float* v, const float* draft, const float* taus,
                                                     int n_tau, int H, int A, const float* params, int gripper_dim,
                                                     float* dist_out, int* accept_out, int* switch_out) {
  extern __shared__ float dsh[];  // [n_tau][H]
  const float delta = params[0];
  for (int e = threadIdx.x; e < n_tau * H; e += blockDim.x) {
    int j = e / H, i = e % H;
    float om = 1.f - taus[j];
    float acc = 0.f;
    for (int k = 0; k < A; ++k) {
      size_t idx = ((size_t)j * H + i) * A + k;
      float diff = x[idx] + om * v[idx] - draft[(size_t)i * A + k];
      acc += diff * diff;
    }
    float dd = sqrtf(acc);
    dsh[e] = dd;
    if (dist_out) dist_out[e] = dd;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int sw = 0;
    if (gripper_dim >= 0)
      for (int i = 1; i < H; ++i)
        if (draft[(size_t)i * A + gripper_dim] * draft[(size_t)(i - 1) * A + gripper_dim] < 0.f) sw = 1;
    int acc = 0;
    while (acc < H) {
      bool ok = true;
      for (int j = 0; j < n_tau; ++j) ok = ok && (dsh[j * H + acc] < delta);
      if (!ok) break;
      ++acc;
    }
    *accept_out = sw ? 0 : acc;
    *switch_out = sw;
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
