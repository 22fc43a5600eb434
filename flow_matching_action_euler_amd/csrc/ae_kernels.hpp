// Device code of the action-expert denoise loop for gfx950 (CDNA4).
//
// One Euler step of the suffix (DM0.5 guide, sections 5.2-5.3) runs as:
//   in_proj   : h = x W_in^T + b_in + temb(t)                      (tiny, FMA)
//   per layer : qkv  = rmsnorm(h) W_qkv^T, RoPE on q/k             (qkv_rope_kernel)      
//               attn = softmax(q [Kp;k]^T / sqrt(dh)) [Vp;v]        (attn_kernel + attn_combine)
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

enum WType { WT_BF16 = 0, WT_FP8 = 1, WT_F32 = 2 };
enum AType { AT_BF16 = 0, AT_F32 = 1 };
enum Epi { EPI_QKV = 0, EPI_RESID = 1, EPI_GEGLU = 2, EPI_OUT = 3 };

constexpr int TOKG = 64;   // tokens per workgroup (4 MFMA column tiles of 16)

// Optional phase timestamps (compile with -DAE_TRACE): thread 0 of every
// workgroup records the 100 MHz wall clock at numbered points of a kernel.
#ifdef AE_TRACE
__device__ unsigned long long ae_trace_buf[8][2048][8];  // [kernel kind][workgroup][point]
#define AE_TR(i)                                                                                         \
  do {                                                                                                   \
    if (threadIdx.x == 0) {                                                                              \
      const unsigned wg_ = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);               \
      if (wg_ < 2048) ae_trace_buf[a.trace_id & 7][wg_][i] = wall_clock64();                             \
    }                                                                                                    \
  } while (0)
#define AE_TRC(i)                                                                                        \
  do {                                                                                                   \
    if (threadIdx.x == 0) {                                                                              \
      const unsigned wg_ = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);               \
      if (wg_ < 2048) ae_trace_buf[a.trace_id & 7][wg_][i] = clock64();                                  \
    }                                                                                                    \
  } while (0)
#else
#define AE_TR(i) do { } while (0)
#define AE_TRC(i) do { } while (0)
#endif
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
  const void* x;        // activations [rows][ldx], gain-scaled, not normalised
  const float* ssp_in;  // [g_in][M_pad] partial sums of h^2 (null: no RMS scaling)
  int g_in;
  float inv_width;      // 1 / width of the normalised vector
  float eps;
  int M, M_pad, K, S;   // rows, padded rows, inputs, k-splits
  int passes;           // k-passes per wave: K/32/S = passes * GW * KPW
  int ldx;              // row stride of x in elements (K plus a 128-byte pad)
  int ldo;              // row stride of the activation written by the epilogue
  float* part;          // split-K partials [S][n_z][n_groups][NT*64*16]
  unsigned* counters;   // [n_z][n_groups], zero between launches
  // EPI_QKV
  void* q_out; void* k_out; void* v_out;   // [rows][ldo], [rows][ldkv] x2
  const float* rope_cs;                    // [H][dh/2][2] cos, sin at positions P + t
  int n_q, n_kv, dh, H;
  int ldkv;                                // row stride of the suffix k buffer
  int ldvt;                                // row stride of the transposed suffix v buffer
  // EPI_RESID
  float* h;              // [M_pad][N] residual, updated in place
  void* hb;              // [rows][ldo] copy h * gain_next for the next consumer
  const float* gain_next;
  float* ssp_out;        // [N/16][M_pad]
  int N;                 // logical outputs
  // EPI_GEGLU
  void* u_out;           // [rows][ldo]
  // EPI_OUT
  const float* bias;     // [A]
  float* xio;            // denoise: x [M_pad][A] updated in place; verify: v out
  int A;
  float dt;              // > 0: x += dt * v; 0: store v
  int trace_id;          // kernel kind for the optional phase trace
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

// LDS bytes of the GEMM kernels: per-wave activation staging (reused for the
// cross-wave reduction), the reduced tile, inverse RMS and RMS partials.
template <int AT, int NT, int KPW>
constexpr size_t gemm_lds_size() {
  constexpr size_t RS = KPW * KBLK * (AT == AT_BF16 ? 2 : 4) + 16;
  constexpr size_t stage = (size_t)GW * 64 * RS;
  constexpr size_t red = (size_t)GW * NT * 1024 * 4;
  return (stage > red ? stage : red) + (size_t)NT * 1024 * 4 + 64 * 4 + 512 * 4 + 16;
}

// Y = X W^T over the workgroup's channel tiles [g*NT, g*NT+NT), k-split s and
// token group z (64 rows), then the epilogue EPI. Block = 8 waves. In each
// pass wave w owns KPW consecutive k-blocks: it issues its weight fragments
// and the 64 x (KPW*32) activation slice as whole 128-byte lines (half the
// L2 requests of fragment-shaped loads), parks the slice in its own LDS
// region and reads the MFMA B fragments from there. No predication:
// activation buffers hold whole 64-row groups. The 8 partial tiles are summed
// in LDS.
template <int WT, int AT, int EPI, int NT, int KPW>
__device__ __forceinline__ void gemm_body(const GemmArgs& a) {
  typedef typename Act<AT>::T XT;
  typedef Frag<WT, AT> F;
  constexpr int RB = KPW * KBLK * (int)sizeof(XT);  // bytes of one staged row slice
  constexpr int RS = RB + 16;                        // LDS row stride
  constexpr int LPR = RB / 16;                       // lanes per row in a 16-byte load
  constexpr int RPI = 64 / LPR;                      // rows per load instruction
  constexpr int NI = 64 / RPI;                       // load instructions per slice
  constexpr size_t STAGE = (size_t)GW * 64 * RS;
  constexpr size_t REDB = (size_t)GW * NT * 1024 * 4;
  extern __shared__ __attribute__((aligned(16))) float smem[];  // no static LDS: keeps 16-byte accesses aligned
  float* red = smem;                                          // [GW][NT][64][16], reuses the staging area
  float* res = (float*)((char*)smem + (STAGE > REDB ? STAGE : REDB));  // [NT][64][16]
  float* inv_rms = res + NT * 1024;                           // [64]
  float* ssq8 = inv_rms + 64;                                 // [8][64]
  unsigned* ticket = (unsigned*)(ssq8 + 512);                 // split-K arrival ticket

  AE_TR(0);
  AE_TRC(6);
  const int g = blockIdx.x, s = blockIdx.y, z = blockIdx.z;
  const int n_groups = gridDim.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int KB = a.K / KBLK;
  const int tok0 = z * TOKG;

  // partial sums of h^2: thread -> token t & 63, groups (t >> 6) + 8 i; loaded now, summed after the MFMAs
  float ssv[8];
  const float* sp = a.ssp_in + tok0 + (threadIdx.x & 63);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int gi = (threadIdx.x >> 6) + 8 * i;
    ssv[i] = (a.ssp_in != nullptr && gi < a.g_in) ? sp[(size_t)gi * a.M_pad] : 0.f;
  }

  // epilogue operands that do not depend on the product, loaded before the main loads:
  // element e = t + 512 i -> (nt = e / 1024, token (e / 16) % 64, channel e % 16)
  float pre0[2 * NT], pre1[2 * NT];
#pragma unroll
  for (int i = 0; i < 2 * NT; ++i) {
    const int e = threadIdx.x + GTHREADS * i;
    const int nt = e >> 10, tl = (e >> 4) & 63, c = e & 15;
    const size_t tile = (size_t)g * NT + nt;
    const int tok = tok0 + tl;
    pre0[i] = 0.f;
    pre1[i] = 0.f;
    if constexpr (EPI == EPI_RESID) {
      if (tok < a.M) pre0[i] = a.h[(size_t)tok * a.N + tile * 16 + c];
      pre1[i] = a.gain_next[tile * 16 + c];
    } else if constexpr (EPI == EPI_QKV) {
      const int tiles_per_head = a.dh / 16, half = a.dh / 2;
      const int t_in = (int)tile;
      if (t_in < (a.n_q + a.n_kv) * tiles_per_head) {
        const int pair = (t_in % tiles_per_head);
        const float2 cs = *(const float2*)(a.rope_cs + ((size_t)(tok % a.H) * half + pair * 8 + (c & 7)) * 2);
        pre0[i] = cs.x;
        pre1[i] = cs.y;
      }
    }
  }

  f32x4 acc[NT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[nt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  unsigned char* xs = (unsigned char*)smem + (size_t)wave * 64 * RS;
  const int lr = lane / LPR, lc = lane % LPR;
  const char* xg = (const char*)a.x + ((size_t)(tok0 + lr) * a.ldx) * sizeof(XT) + lc * 16;
  const size_t xrow_step = (size_t)RPI * a.ldx * sizeof(XT);
  const unsigned char* xf = xs + (lane & 15) * RS + (lane >> 4) * 8 * sizeof(XT);
  for (int p = 0; p < a.passes; ++p) {
    const int kb0 = s * (KB / a.S) + (p * GW + wave) * KPW;
    typename F::A wa[NT][KPW];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int j = 0; j < KPW; ++j) wa[nt][j] = F::load_a(a.w, ((size_t)g * NT + nt) * KB + kb0 + j, lane);
    i32x4 xr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) xr[i] = *(const i32x4*)(xg + i * xrow_step + (size_t)kb0 * KBLK * sizeof(XT));
    __builtin_amdgcn_sched_barrier(0);  // keep every load of the pass in flight before the first LDS store
#pragma unroll
    for (int i = 0; i < NI; ++i) *(i32x4*)(xs + (size_t)(i * RPI + lr) * RS + lc * 16) = xr[i];
#pragma unroll
    for (int j = 0; j < KPW; ++j)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        typename F::B xb = F::load_b((const XT*)(xf + (size_t)tt * 16 * RS + j * KBLK * sizeof(XT)));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt][tt] = F::mma(wa[nt][j], xb, acc[nt][tt]);
      }
  }

  AE_TR(1);
  float ssq = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ssq += ssv[i];
  if (a.ssp_in != nullptr)
    for (int gi = (threadIdx.x >> 6) + 64; gi < a.g_in; gi += 8) ssq += sp[(size_t)gi * a.M_pad];  // width > 1024
  __syncthreads();  // every wave is done with its staging region before it becomes the reduction buffer
  // cross-wave reduction: red[wave][nt][tok][c], one 16-byte write per (nt, tt) per lane
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      *(f32x4*)(red + ((wave * NT + nt) * TOKG + tt * 16 + (lane & 15)) * 16 + 4 * (lane >> 4)) = acc[nt][tt];
  ssq8[threadIdx.x] = ssq;
  __syncthreads();
  // quads of 4 consecutive elements: NT * 256 quads over 512 threads
#pragma unroll
  for (int i = 0; i < (NT + 1) / 2; ++i) {
    const int qd = threadIdx.x + GTHREADS * i;
    if (qd < NT * 256) {
      f32x4 sum = *(const f32x4*)(red + qd * 4);
#pragma unroll
      for (int w = 1; w < GW; ++w) sum += *(const f32x4*)(red + w * NT * 1024 + qd * 4);
      *(f32x4*)(res + qd * 4) = sum;
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

  AE_TR(2);
  if (a.S > 1) {
    // split-K: publish the partial (write-through), count arrivals; the last
    // arriver of (z, g) sums the S partials in split order (deterministic).
    const int n_z = gridDim.z;
    const int tile_elems = NT * 1024;
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.part);
#pragma unroll
    for (int i = 0; i < (NT + 1) / 2; ++i) {
      const int qd = threadIdx.x + GTHREADS * i;
      if (qd < NT * 256)
        st16_coherent(rp, (unsigned)(((((size_t)s * n_z + z) * n_groups + g) * tile_elems + qd * 4) * 4),
                      *(const float4*)(res + qd * 4));
    }
    wait_mem();
    __syncthreads();
    unsigned* cnt = a.counters + z * n_groups + g;
    if (threadIdx.x == 0) {
      *ticket = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (*ticket == (unsigned)a.S - 1) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (*ticket != (unsigned)a.S - 1) return;
#pragma unroll
    for (int i = 0; i < (NT + 1) / 2; ++i) {
      const int qd = threadIdx.x + GTHREADS * i;
      if (qd < NT * 256) {
        f32x4 v[4];
#pragma unroll
        for (int ss = 0; ss < 4; ++ss)
          v[ss] = ss < a.S ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                 rp, (unsigned)(((((size_t)ss * n_z + z) * n_groups + g) * tile_elems + qd * 4) * 4), 0, 0x10))
                           : f32x4{0.f, 0.f, 0.f, 0.f};
        *(f32x4*)(res + qd * 4) = ((v[0] + v[1]) + v[2]) + v[3];
      }
    }
    __syncthreads();
  }

  AE_TR(3);
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
    float val = res[e] * inv_rms[tl];
    if constexpr (WT == WT_FP8) val *= a.wscale[tile * 16 + c];
    if constexpr (EPI == EPI_QKV) {
      // packed tiles: q heads, then k heads (RoPE pairs d, d+dh/2 share a tile), then v
      const int tiles_per_head = a.dh / 16;
      const int q_tiles = a.n_q * tiles_per_head, k_tiles = a.n_kv * tiles_per_head;
      const int half = a.dh / 2;
      const int t_in = (int)tile;
      if (t_in < q_tiles + k_tiles) {
        const bool is_q = t_in < q_tiles;
        const int tt2 = is_q ? t_in : t_in - q_tiles;
        const int head = tt2 / tiles_per_head, pair = tt2 % tiles_per_head;
        const int d = pair * 8 + (c & 7);
        const float partner = res[e ^ 8] * inv_rms[tl];
        const float2 cs = make_float2(pre0[i], pre1[i]);
        float out;
        int dfull;
        if (c < 8) { out = val * cs.x - partner * cs.y; dfull = d; }
        else { out = partner * cs.y + val * cs.x; dfull = half + d; }
        if (valid) {
          if (is_q) Act<AT>::st((XT*)a.q_out, (size_t)tok * a.ldo + head * a.dh + dfull, out);
          else Act<AT>::st((XT*)a.k_out, (size_t)tok * a.ldkv + head * a.dh + dfull, out);
        }
      } else {
        // suffix values transposed: [seq][kv head][dh][ldvt]
        const int col = (t_in - q_tiles - k_tiles) * 16 + c;
        if (valid)
          Act<AT>::st((XT*)a.v_out, ((size_t)(tok / a.H) * a.n_kv * a.dh + col) * a.ldvt + tok % a.H, val);
      }
    } else if constexpr (EPI == EPI_RESID) {
      const int n = (int)tile * 16 + c;
      float hn = 0.f;
      if (valid) {
        hn = pre0[i] + val;
        a.h[(size_t)tok * a.N + n] = hn;
        Act<AT>::st((XT*)a.hb, (size_t)tok * a.ldo + n, hn * pre1[i]);
      }
      float sq = hn * hn;
      sq += __shfl_xor(sq, 1, 16);
      sq += __shfl_xor(sq, 2, 16);
      sq += __shfl_xor(sq, 4, 16);
      sq += __shfl_xor(sq, 8, 16);
      if (c == 0) a.ssp_out[tile * a.M_pad + tok] = sq;
    } else if constexpr (EPI == EPI_GEGLU) {
      float up = res[e + 1024] * inv_rms[tl];
      if constexpr (WT == WT_FP8) up *= a.wscale[(tile + 1) * 16 + c];
      const int f = (int)(tile / 2) * 16 + c;
      if (valid) Act<AT>::st((XT*)a.u_out, (size_t)tok * a.ldo + f, gelu_tanh(val) * up);
    } else {  // EPI_OUT
      const int n = (int)tile * 16 + c;
      if (valid && n < a.A) {
        const float v = val + a.bias[n];
        if (a.dt > 0.f) a.xio[(size_t)tok * a.A + n] += a.dt * v;
        else a.xio[(size_t)tok * a.A + n] = v;
      }
    }
  }
#ifdef AE_TRACE
  wait_mem();
  AE_TR(4);
  AE_TRC(7);
#endif
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
  template <int WT, int AT, int KPW>                                                                      \
  __global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(1, 2))) void NAME(GemmArgs a) {   \
    gemm_body<WT, AT, RoleTraits<ROLE>::EPI, RoleTraits<ROLE>::NT, KPW>(a);                              \
  }
AE_GEMM_ENTRY(qkv_rope_kernel, R_QKV_ROPE)
AE_GEMM_ENTRY(o_proj_resid_kernel, R_O_PROJ)
AE_GEMM_ENTRY(gate_up_geglu_kernel, R_GATE_UP)
AE_GEMM_ENTRY(down_resid_kernel, R_DOWN)
AE_GEMM_ENTRY(out_proj_euler_kernel, R_OUT_PROJ)
#undef AE_GEMM_ENTRY

template <int ROLE, int WT, int AT, int KPW>
constexpr void (*gemm_entry())(GemmArgs) {
  if constexpr (ROLE == R_QKV_ROPE) return qkv_rope_kernel<WT, AT, KPW>;
  else if constexpr (ROLE == R_O_PROJ) return o_proj_resid_kernel<WT, AT, KPW>;
  else if constexpr (ROLE == R_GATE_UP) return gate_up_geglu_kernel<WT, AT, KPW>;
  else if constexpr (ROLE == R_DOWN) return down_resid_kernel<WT, AT, KPW>;
  else return out_proj_euler_kernel<WT, AT, KPW>;
}

// ------------------------------------------------------------------ attention

struct AttnArgs {
  const void* q;          // [rows][ldq] (rotated)
  const void* ks;         // suffix keys [rows][ldkv] (rotated)
  const void* vsT;        // suffix values transposed [seq][n_kv][dh][ldvt]
  const void* kcache;     // prefix K [slots][L][P][n_kv][dh]
  const void* vcacheT;    // prefix V transposed [slots][L][n_kv][dh][ldp]
  const int* seq_slot;    // prefix slot of each sequence
  size_t kslot_stride, klayer_off;  // elements
  size_t vslot_stride, vlayer_off;  // elements
  int P, H, n_q, n_kv, dh, KC;
  int ldq, ldkv, ldvt, ldp, ldo;
  int n_qt, n_chunks;
  float scale_log2;       // log2(e) / sqrt(dh)
  float* opart;           // [z][qt][chunk][64][dh]
  float* mlpart;          // [z][qt][chunk][64][2]  (row max in log2 units, row sum)
  unsigned* qt_counter;   // [z][qt] arrival counters (monotonic) for the fused combine
  unsigned* err;          // set when a fused-combine wait times out
  void* o;                // [rows][ldo] output
  int fused;              // 1: combine inside the kernel (whole grid co-resident)
  int p_aligned;          // prefix_len is a multiple of the 16-byte vector width
  int trace_id;
};

// Combine the chunk partials of one query row r (of sequence s, kv head g) for dims d:
// o = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c, 16 chunks per batch, all loads of a batch in flight.
template <int AT, bool COHERENT>
__device__ __forceinline__ void attn_combine_row(const AttnArgs& a, int zz, int qt, int row, int d, int s, int g) {
  typedef typename Act<AT>::T XT;
  const size_t base = ((size_t)zz * a.n_qt + qt) * a.n_chunks;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.opart), rm = make_rsrc(a.mlpart);
  float M = -INFINITY, num = 0.f, den = 0.f;
  for (int c0 = 0; c0 < a.n_chunks; c0 += 16) {
    float mc[16], lc[16], oc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = c0 + i;
      if (c < a.n_chunks) {
        const size_t mi = ((base + c) * 64 + row) * 2, oi = ((base + c) * 64 + row) * a.dh + d;
        if constexpr (COHERENT) {
          mc[i] = ld_coherent_buf(rm, (unsigned)(mi * 4));
          lc[i] = ld_coherent_buf(rm, (unsigned)(mi * 4 + 4));
          oc[i] = ld_coherent_buf(ro, (unsigned)(oi * 4));
        } else {
          mc[i] = a.mlpart[mi];
          lc[i] = a.mlpart[mi + 1];
          oc[i] = a.opart[oi];
        }
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
  const int gq = a.n_q / a.n_kv;
  const int r = qt * 64 + row;
  const int jh = r / a.H, t = r % a.H;
  Act<AT>::st((XT*)a.o, (size_t)(s * a.H + t) * a.ldo + (size_t)(g * gq + jh) * a.dh + d, num / den);
}

// One workgroup: 64 query rows (4 waves x 16; row r = j*H + t is query head
// g*gq + j, chunk row t of one sequence) against one chunk of KC keys of
// [prefix ; suffix]. S^T = K Q^T puts 16 keys x 16 rows in each MFMA tile,
// so a lane's accumulators hold 8 keys of one row per 32-key block: they are
// the B operand of O^T = V^T P^T directly (k index permuted identically for
// V^T), and the softmax never leaves registers. K and V^T are staged in LDS
// with 16-byte loads (V is cached transposed). The chunk's partial (m, l, O)
// is written write-through; with fused = 1 the n_chunks workgroups of a
// query tile then meet at a counter and each combines a share of the rows.
template <int AT, int KC, int DH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void attn_kernel(AttnArgs a) {
  typedef typename Act<AT>::T XT;
  typedef Frag<WT_BF16, AT> F;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];  // no static LDS: aligned 16-byte accesses
  constexpr int dh = DH;
  constexpr int VE = 16 / sizeof(XT);      // elements per 16-byte vector
  constexpr int ldk = DH + VE;             // padded LDS row strides (elements)
  constexpr int ldv = KC + VE;
  XT* Ks = (XT*)smem_raw;                  // [KC][ldk]
  XT* VT = Ks + (size_t)KC * ldk;          // [dh][ldv]

  AE_TR(0);
  const int chunk = blockIdx.x, qt = blockIdx.y, zz = blockIdx.z;
  const int s = zz / a.n_kv, g = zz % a.n_kv;
  const int gq = a.n_q / a.n_kv;
  const int R = gq * a.H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j0 = chunk * KC;
  const int n_keys = a.P + a.H;
  const int slot = a.seq_slot[s];
  const XT* kc = (const XT*)a.kcache + (size_t)slot * a.kslot_stride + a.klayer_off;
  const XT* vcT = (const XT*)a.vcacheT + (size_t)slot * a.vslot_stride + a.vlayer_off + (size_t)g * DH * a.ldp;
  const XT* ks = (const XT*)a.ks;
  const XT* vsT = (const XT*)a.vsT + ((size_t)s * a.n_kv + g) * dh * a.ldvt;

  // query fragments (B operand of S^T): row r of this lane, 8 inputs per 32-block
  const int r_lane = qt * 64 + wave * 16 + (lane & 15);
  const bool r_ok = r_lane < R;
  const int jh = r_ok ? r_lane / a.H : 0, t_lane = r_ok ? r_lane % a.H : 0;
  const XT* qrow = (const XT*)a.q + (size_t)(s * a.H + t_lane) * a.ldq + (size_t)(g * gq + jh) * dh + (lane >> 4) * 8;
  typename F::B qb[8];
#pragma unroll
  for (int kb = 0; kb < 8; ++kb)
    if (kb < dh / KBLK) qb[kb] = r_ok ? F::load_b(qrow + kb * KBLK) : typename F::B();

  // stage K rows [j0, j0+KC) and V^T columns: every global load of the thread is
  // issued before the first LDS store (one memory round trip). Sources are
  // selected, not branched on: key indices are clamped into range and keys
  // past the last one are zeroed after the load.
  constexpr int vpr = DH / VE, kpr = KC / VE;
  constexpr int KIT = KC * vpr / 256, VIT = DH * kpr / 256;  // vectors per thread
  static_assert(KIT >= 1 && VIT >= 1 && KIT <= 8 && VIT <= 8, "attention tile shape");
  i32x4 kreg[KIT], vreg[VIT];
#pragma unroll
  for (int i = 0; i < KIT; ++i) {
    const int e = threadIdx.x + 256 * i;
    const int kr = e / vpr, d0 = (e % vpr) * VE, j = j0 + kr;
    const int jc = min(j, n_keys - 1);
    const XT* src = jc < a.P ? kc + ((size_t)jc * a.n_kv + g) * DH + d0
                             : ks + (size_t)(s * a.H + (jc - a.P)) * a.ldkv + (size_t)g * DH + d0;
    kreg[i] = *(const i32x4*)src;
  }
  if (a.p_aligned) {  // every 16-byte key vector lies wholly in the prefix or wholly in the suffix
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int e = threadIdx.x + 256 * i;
      const int d = e / kpr, jb = j0 + (e % kpr) * VE;
      const int jc = min(jb, a.P + a.ldvt - VE);  // suffix rows are zero-padded to ldvt
      const XT* src = jc < a.P ? vcT + (size_t)d * a.ldp + jc : vsT + (size_t)d * a.ldvt + (jc - a.P);
      vreg[i] = *(const i32x4*)src;
    }
  } else {
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int e = threadIdx.x + 256 * i;
      const int d = e / kpr, jb = j0 + (e % kpr) * VE;
      XT tmp[VE];
#pragma unroll
      for (int t = 0; t < VE; ++t) {
        const int j = jb + t;
        tmp[t] = j < a.P ? vcT[(size_t)d * a.ldp + j] : (j < n_keys ? vsT[(size_t)d * a.ldvt + (j - a.P)] : (XT)0);
      }
      vreg[i] = *(const i32x4*)tmp;
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // all staging loads in flight before the first LDS store
#pragma unroll
  for (int i = 0; i < KIT; ++i) {
    const int e = threadIdx.x + 256 * i;
    const int kr = e / vpr;
    const i32x4 z = {0, 0, 0, 0};
    *(i32x4*)(Ks + (size_t)kr * ldk + (e % vpr) * VE) = (j0 + kr < n_keys) ? kreg[i] : z;
  }
#pragma unroll
  for (int i = 0; i < VIT; ++i) {
    const int e = threadIdx.x + 256 * i;
    const int jb = j0 + (e % kpr) * VE;
    const i32x4 z = {0, 0, 0, 0};
    *(i32x4*)(VT + (size_t)(e / kpr) * ldv + (e % kpr) * VE) = (jb < n_keys) ? vreg[i] : z;
  }
  __syncthreads();
  AE_TR(1);

  // S^T tiles: sacc[kt][v] = score(key kt*16 + 4*(lane/16) + v, row lane%16)
  const int n_kt = KC / 16;
  f32x4 sacc[8];
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) sacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    if (kt < n_kt) {
      const XT* kp = Ks + (size_t)(kt * 16 + (lane & 15)) * ldk + (lane >> 4) * 8;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
        if (kb < dh / KBLK) {
          typename F::A ka;
          if constexpr (AT == AT_BF16) ka = __builtin_bit_cast(bf16x8, *(const uint4*)(kp + kb * KBLK));
          else ka = typename F::A{((const float4*)(kp + kb * KBLK))[0], ((const float4*)(kp + kb * KBLK))[1]};
          sacc[kt] = F::mma(ka, qb[kb], sacc[kt]);
        }
    }
  }
  AE_TR(2);
  // softmax over this chunk's keys for row lane%16: reduce over kt, v and the 4 lane groups
  float m = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 8; ++kt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = j0 + kt * 16 + 4 * (lane >> 4) + v;
      const float sv = (kt < n_kt && j < n_keys) ? sacc[kt][v] * a.scale_log2 : -INFINITY;
      sacc[kt][v] = sv;
      m = fmaxf(m, sv);
    }
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  float lsum = 0.f;
#pragma unroll
  for (int kt = 0; kt < 8; ++kt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float p = (m == -INFINITY) ? 0.f : exp2f(sacc[kt][v] - m);
      sacc[kt][v] = p;
      lsum += p;
    }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);

  // O^T = V^T P^T: dims dt*16 + lane%16 (A from LDS, keys permuted like the B operand), rows lane%16
  const int q4 = 4 * (lane >> 4);
  f32x4 oacc[16];
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb2 = 0; kb2 < 4; ++kb2) {
    if (kb2 < KC / KBLK) {
      typename F::B pb;
      if constexpr (AT == AT_BF16) {
        pb = bf16x8{(__bf16)sacc[2 * kb2][0], (__bf16)sacc[2 * kb2][1], (__bf16)sacc[2 * kb2][2], (__bf16)sacc[2 * kb2][3],
                    (__bf16)sacc[2 * kb2 + 1][0], (__bf16)sacc[2 * kb2 + 1][1], (__bf16)sacc[2 * kb2 + 1][2],
                    (__bf16)sacc[2 * kb2 + 1][3]};
      } else {
        pb = typename F::B{make_float4(sacc[2 * kb2][0], sacc[2 * kb2][1], sacc[2 * kb2][2], sacc[2 * kb2][3]),
                           make_float4(sacc[2 * kb2 + 1][0], sacc[2 * kb2 + 1][1], sacc[2 * kb2 + 1][2], sacc[2 * kb2 + 1][3])};
      }
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) {
        if (dt < dh / 16) {
          const XT* vp = VT + (size_t)(dt * 16 + (lane & 15)) * ldv + kb2 * KBLK + q4;
          typename F::A va;
          if constexpr (AT == AT_BF16) {
            const uint2 lo = *(const uint2*)vp, hi = *(const uint2*)(vp + 16);
            va = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
          } else {
            va = typename F::A{*(const float4*)vp, *(const float4*)(vp + 16)};
          }
          oacc[dt] = F::mma(va, pb, oacc[dt]);
        }
      }
    }
  }

  AE_TR(3);
  // publish the chunk partial: row lane%16 holds dims dt*16 + q4 .. +4
  const int prow = wave * 16 + (lane & 15);
  const size_t pidx = ((size_t)zz * a.n_qt + qt) * a.n_chunks + chunk;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.opart), rm = make_rsrc(a.mlpart);
  if (a.fused) {  // read by other workgroups of this launch: write through
#pragma unroll
    for (int dt = 0; dt < dh / 16; ++dt)
      st16_coherent(ro, (unsigned)(((pidx * 64 + prow) * dh + dt * 16 + q4) * 4),
                    make_float4(oacc[dt][0], oacc[dt][1], oacc[dt][2], oacc[dt][3]));
    if (lane < 16) {
      __hip_atomic_store(a.mlpart + (pidx * 64 + prow) * 2, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.mlpart + (pidx * 64 + prow) * 2 + 1, lsum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {  // read by the combine kernel after the launch boundary
#pragma unroll
    for (int dt = 0; dt < dh / 16; ++dt)
      *(f32x4*)(a.opart + (pidx * 64 + prow) * dh + dt * 16 + q4) = oacc[dt];
    if (lane < 16) *(float2*)(a.mlpart + (pidx * 64 + prow) * 2) = make_float2(m, lsum);
  }
#ifdef AE_TRACE
  wait_mem();
  AE_TR(4);
#endif
  if (!a.fused) return;

  // fused combine: wait for the n_chunks workgroups of this query tile (bounded spin)
  wait_mem();
  __syncthreads();
  int* go = (int*)(VT + (size_t)dh * ldv);  // one int past the staged tiles
  if (threadIdx.x == 0) {
    unsigned* cnt = a.qt_counter + (size_t)zz * a.n_qt + qt;
    const unsigned old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned target = (old / a.n_chunks + 1) * a.n_chunks;
    int ok = 0;
    for (int it = 0; it < (1 << 22); ++it) {
      if ((int)(ldu_coherent(cnt) - target) >= 0) { ok = 1; break; }
      __builtin_amdgcn_s_sleep(1);
    }
    if (!ok) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *go = ok;
  }
  __syncthreads();
  AE_TR(5);
  if (!*go) return;
  // this workgroup's share of the tile: units (row, 4 dims), strided over the n_chunks workgroups
  const int rows_here = min(64, R - qt * 64);
  const int units = rows_here * (dh / 4);
  const size_t base = ((size_t)zz * a.n_qt + qt) * a.n_chunks;
  for (int u = chunk * 256 + threadIdx.x; u < units; u += a.n_chunks * 256) {
    const int row = u / (dh / 4), d4 = (u % (dh / 4)) * 4;
    float M = -INFINITY;
    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
    float den = 0.f;
    for (int c0 = 0; c0 < a.n_chunks; c0 += 16) {
      float mc[16], lc[16];
      float4 oc[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = c0 + i;
        if (c < a.n_chunks) {
          const size_t mi = ((base + c) * 64 + row) * 2, oi = ((base + c) * 64 + row) * dh + d4;
          mc[i] = ld_coherent_buf(rm, (unsigned)(mi * 4));
          lc[i] = ld_coherent_buf(rm, (unsigned)(mi * 4 + 4));
          oc[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(ro, (unsigned)(oi * 4), 0, 0x10));
        } else {
          mc[i] = -INFINITY; lc[i] = 0.f; oc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
      float Mn = M;
#pragma unroll
      for (int i = 0; i < 16; ++i) Mn = fmaxf(Mn, mc[i]);
      const float sc = (M == -INFINITY) ? 0.f : exp2f(M - Mn);
      num.x *= sc; num.y *= sc; num.z *= sc; num.w *= sc;
      den *= sc;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float wgt = (mc[i] == -INFINITY) ? 0.f : exp2f(mc[i] - Mn);
        num.x += wgt * oc[i].x; num.y += wgt * oc[i].y; num.z += wgt * oc[i].z; num.w += wgt * oc[i].w;
        den += wgt * lc[i];
      }
      M = Mn;
    }
    const int r = qt * 64 + row;
    const int jr = r / a.H, tr = r % a.H;
    XT* op = (XT*)a.o + (size_t)(s * a.H + tr) * a.ldo + (size_t)(g * gq + jr) * dh + d4;
    const float inv = 1.f / den;
    Act<AT>::st(op, 0, num.x * inv);
    Act<AT>::st(op, 1, num.y * inv);
    Act<AT>::st(op, 2, num.z * inv);
    Act<AT>::st(op, 3, num.w * inv);
  }
#ifdef AE_TRACE
  wait_mem();
  AE_TR(6);
#endif
}

// Separate combine (grid not co-resident): grid (R rows, n_seq * n_kv); block = dh threads.
template <int AT>
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a) {
  const int r = blockIdx.x, zz = blockIdx.y;
  if ((int)threadIdx.x >= a.dh) return;
  attn_combine_row<AT, false>(a, zz, r / 64, r % 64, threadIdx.x, zz / a.n_kv, zz % a.n_kv);
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
