// One Euler step of a batch-1 pass as ONE persistent launch (DM0.5 guide, section 6.4: fuse the
// suffix into few kernels with few temporary write-backs; section 6.5: one graph replay per request).
//
// A grid of one workgroup per compute unit, all resident at once, runs every phase of the step:
//   in_proj -> per layer [QKV + RoPE -> attention key splits -> split merge -> o_proj + residual ->
//   gate/up + GeGLU -> down + residual] -> out_proj + Euler update.
// There is no launch boundary and no grid barrier between phases. A producer stores its output with
// device-scope (write-through) stores into buffers that hold EXCH_EMPTY in every word; a consumer
// polls the MFMA operand fragments it needs with device-scope loads until no word of a valid lane
// holds EXCH_EMPTY, and then uses exactly what it polled. Measured on the part: a store is visible to
// such a poll ~0.4 us after it is issued; an acknowledged store plus an arrival counter and a plain
// read costs about 1 us more per dependency than polling the data itself.
//
// Buffers. Every activation a phase polls lives in a per-layer block of an activation ring; two
// rings alternate between consecutive launches, and each launch writes EXCH_EMPTY over the ring the
// previous launch used (that launch has ended, the next one has not begun), spread over the
// workgroups at the start of each layer. Attention split partials alternate the same way (two sets,
// the other emptied in the same reset phases). The residual h of a (16-channel tile, 16-token tile) never leaves the workgroup that
// owns it: in_proj, o_proj and down give the same workgroup the same tile, which keeps h in LDS.
//
// Work split (G workgroups; workgroup g runs on XCD g % 8). The token-split phases give the ntp
// (= token tiles rounded up to 1, 2 or 4) workgroups that share a weight tile the same XCD, so the
// tile is fetched from HBM once per XCD and the other reads hit that XCD's L2:
//   in_proj, o_proj, down, out_proj : unit = (16-channel tile, one token tile)
//   QKV                             : unit = (up to 3 tiles, one token tile)
//   gate/up                         : unit = (2 gate/up tile pairs, up to 2 token tiles)
//   attention                       : unit = (key split, 16-row query tile, kv head), one 32-key
//                                     block per wave; the splits of a tile meet in a merge unit
// Inside a unit the 8 waves split K; each wave loads its weight fragments with plain loads before it
// polls its activation fragments, and the partial tiles meet in LDS.
//
// Every poll is bounded (wait_ticks of the 100 MHz clock) and also watches an abort word: a wait
// that gives up sets abort (and a host-visible flag), and every workgroup then leaves at its next
// poll, so the launch always ends; the host restores the buffers and repeats the pass with launches
// that have no in-kernel waits.
#pragma once
#include "ae_kernels.hpp"

namespace ae {

struct FusedLayer {
  const uint16_t* qkv;   // packed QKV weights [qkv tiles][w/32][64][8] bf16 (RoPE-paired q/k tiles, then v)
  const uint16_t* o;     // packed o_proj weights [w/16][nq*dh/32][64][8]
  const void* gu;        // packed gate/up weights, gate and up tiles interleaved (bf16 or E4M3 bytes)
  const void* d;         // packed down weights [w/16][F/32][64][8]
  const float* gu_s;     // E4M3: scale per packed gate/up channel; else null
  const float* d_s;      // E4M3: scale per down output channel; else null
  const float* ln2;      // gain of the MLP norm (applied by the o_proj epilogue)
  const float* g_next;   // gain of the next norm (next layer's ln1, or the final norm)
  const uint16_t* kc;    // this layer's packed prefix K of slot 0 (a pass on slot s adds FusedArgs::slot_off)
  const uint16_t* vc;    // and V
  const float* qk_gain;  // QK-norm: gain per packed q/k channel; else null
};

struct FusedArgs {
  const FusedLayer* layers;
  int L, w, F, nq, nkv, dh, H, P, A;
  int ntt;               // 16-token tiles of the chunk (activation buffers hold ntt * 16 rows)
  int ntp;               // ntt rounded up to 1, 2 or 4
  int G;                 // workgroups
  float eps, inv_w;
  float* x;              // [H][A] fp32 chunk: read by in_proj, updated by out_proj
  const uint16_t* w_in;  // action_in_proj [w][A] bf16 row-major
  const float* b_in;
  const float* temb;     // [w] this step's time embedding
  const float* ln1_0;    // first layer's norm gain
  const uint16_t* w_out; // packed action_out_proj [out tiles][w/32][64][8]
  const float* b_out;
  int out_tiles;
  float dt;
  const float* rope_cs;  // [H][dh/2][2] (cos, sin) at positions P + t
  int n_qt, nbp, nbs, n_split, n_att;  // attention: query tiles, prefix / suffix 32-key blocks, key splits, units
  float scale_log2;
  float* part_o;         // [L][n_att][16][dh] split partials of this launch (EXCH_EMPTY before it)
  float* part_ml;        // [L][n_att][16][2]
  float* part_o_other;   // the partials of the previous launch, emptied here (as the other ring)
  float* part_ml_other;
  char* ring;            // this launch's activation ring: (L + 1) blocks of layer_bytes
  char* ring_other;      // the ring of the previous launch, emptied here
  unsigned layer_bytes;
  unsigned off_ssp, off_q, off_k, off_v, off_o, off_hb2, off_ssp2, off_u;  // byte offsets in a block (hb_in at 0)
  unsigned* abort;       // device word: set when a wait gave up
  unsigned* host_flag;   // host-visible copy of abort
  unsigned long long wait_ticks;
  size_t slot_off;       // elements from slot 0's prefix cache to the pass's slot
  // time-modulated expert (null otherwise; DM0.5 guide, section 5.2): this step's vectors of layer l at
  // base + l * stride: norm gains ln1 (1 + scale1) and ln2 (1 + scale2), the shift biases of QKV and
  // gate/up in their packed channel order, the modulation rows [6w] (gates at 2w and 5w), the final gain
  const float* m_g1;
  const float* m_g2;
  const float* m_bqkv;
  const float* m_bgu;
  const float* m_mod;
  const float* m_gf;
  size_t m_sw, m_sqkv, m_sgu, m_smod;
  // QK-norm: byte offset in a ring block of the per-tile sums of squares of q and k ([(nq + nkv) dh/16]
  // [ntt * 16] fp32), 0 without QK-norm
  unsigned off_qks;
  float qk_inv_dh, qk_eps;
};

constexpr int FW = 8;            // waves per workgroup
constexpr int FT = FW * 64;
constexpr int F_QKV_NT = 3;      // QKV tiles a workgroup computes in one pass
constexpr int F_SLOTS = 2;       // residual tiles a workgroup can own
constexpr int F_NQ = 8;          // (tile, token tile) pairs of one pass at most (gate/up: 4 x 2)

template <int DH>
constexpr size_t fused_scratch_bytes() {
  constexpr size_t att = attn_lds_size<DH, FW, false>();
  constexpr size_t gemm = (size_t)FW * F_NQ * 1024 + (size_t)F_NQ * 1024 + 64 * 4 + FW * 64 * 4;
  return att > gemm ? att : gemm;
}
// after the scratch: the residual slots, the abort word (16 bytes), QK-norm's 1/rms of the 16 query rows
// and of each wave's 32 suffix keys
constexpr size_t F_QKN_FLOATS = ATT_ROWS + FW * ATT_KB;
template <int DH>
constexpr size_t fused_lds_bytes() { return fused_scratch_bytes<DH>() + (size_t)F_SLOTS * 1024 + 16 + F_QKN_FLOATS * 4; }

// ------------------------------------------------------------------ polling

// Workgroup barrier for LDS only. __syncthreads() also orders global memory for the workgroup, so the
// compiler makes every wave wait there until its outstanding global stores are acknowledged -- after
// the device-scope (write-through) stores of an epilogue that is a fabric round trip. No wave of this
// kernel reads global data another wave of its workgroup wrote except through a poll, so the LDS
// operations completing is all a barrier has to wait for.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ bool is_empty4(i32x4 v) { return v[0] == -1 || v[1] == -1 || v[2] == -1 || v[3] == -1; }

__device__ __forceinline__ void fused_give_up(const FusedArgs& a) {
  __hip_atomic_store(a.abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(a.host_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// One wave loads N 16-byte pieces (this lane's piece i at byte offset off(i) of buffer r) with
// device-scope loads until no dword of a piece with need(i) holds EXCH_EMPTY in any lane; pieces
// without need are returned as zeros. off and need are recomputed per poll (cheaper than holding
// them in registers). False when the wait gave up or another workgroup's did.
// While the data is far from ready only the first piece of each lane is polled (1 KB per wave instead of
// the whole operand set), so that waiting workgroups do not crowd the fabric the producers need.
// With lead (an LDS word; every wave of the workgroup calls together), only wave 0 polls its first
// piece while the others wait at a barrier: an eighth of the polling traffic.
template <int N, class Off, class Need>
__device__ __forceinline__ bool poll16(__amdgpu_buffer_rsrc_t r, Off off, Need need, i32x4 (&v)[N], const FusedArgs& a,
                                       int* lead = nullptr) {
  const unsigned long long t_end = wall_clock64() + a.wait_ticks;
  if constexpr (N > 1) {
    const bool poll_first = !lead || __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0;
    bool first_ok = true;
    if (poll_first) for (;;) {
      const i32x4 w0 = __builtin_amdgcn_raw_buffer_load_b128(r, off(0), 0, 0x10);
      const unsigned ab = __hip_atomic_load(a.abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__all(!need(0) || !is_empty4(w0))) break;
      if (ab != 0u || wall_clock64() > t_end) {
        if (ab == 0u) fused_give_up(a);
        first_ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (lead) {
      if (poll_first && (threadIdx.x & 63) == 0) *lead = first_ok ? 0 : 1;
      lds_barrier();
      first_ok = *lead == 0;
    }
    if (!first_ok) return false;
  }
  for (;;) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(r, off(i), 0, 0x10);
    const unsigned ab = __hip_atomic_load(a.abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool ok = true;
#pragma unroll
    for (int i = 0; i < N; ++i) ok = ok && (!need(i) || !is_empty4(v[i]));
    if (__all(ok)) break;
    if (ab != 0u || wall_clock64() > t_end) {
      if (ab == 0u) fused_give_up(a);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (!need(i)) v[i] = i32x4{0, 0, 0, 0};
  return true;
}

// The same for N 4-byte words (RMS partial sums).
template <int N>
__device__ __forceinline__ bool poll4(__amdgpu_buffer_rsrc_t r, const unsigned (&off)[N], const bool (&need)[N],
                                      float (&v)[N], const FusedArgs& a) {
  const unsigned long long t_end = wall_clock64() + a.wait_ticks;
  for (;;) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off[i], 0, 0x10));
    const unsigned ab = __hip_atomic_load(a.abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool ok = true;
#pragma unroll
    for (int i = 0; i < N; ++i) ok = ok && (!need[i] || __float_as_uint(v[i]) != EXCH_EMPTY);
    if (__all(ok)) break;
    if (ab != 0u || wall_clock64() > t_end) {
      if (ab == 0u) fused_give_up(a);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (!need[i]) v[i] = 0.f;
  return true;
}

__device__ __forceinline__ void st8_coherent(__amdgpu_buffer_rsrc_t r, unsigned byte_off, uint2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, v), r, byte_off, 0, 0x10);
}
__device__ __forceinline__ void st16u_coherent(__amdgpu_buffer_rsrc_t r, unsigned byte_off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, byte_off, 0, 0x10);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// ------------------------------------------------------------------ work split

// Token-split phase with TS token groups: workgroup -> (token group tg, tile group gid); the TS
// workgroups of a tile group are on one XCD (g % 8). Tiles of the workgroup: gid + n_groups * i.
struct TokSplit {
  int tg, gid, n_groups;
};
__device__ __forceinline__ TokSplit tok_split(int G, int TS) {
  const int wg = blockIdx.x, xcd = wg & 7, r = wg >> 3;
  return TokSplit{r % TS, (r / TS) * 8 + xcd, G / TS};
}

// ------------------------------------------------------------------ GEMM pass of a unit

template <int WT> struct FWReg { typedef i32x4 T; };
template <> struct FWReg<WT_FP8> { typedef i32x2 T; };
template <int WT>
__device__ __forceinline__ bf16x8 to_bf16x8(typename FWReg<WT>::T v) {
  if constexpr (WT == WT_FP8) return fp8x8_to_bf16x8(make_uint2((unsigned)v[0], (unsigned)v[1]));
  else return __builtin_bit_cast(bf16x8, v);
}

// acc[t][j] = sum over this wave's k-blocks kb = wave * KBW + i of W(tile[t], kb) X(kb, token tile tt[j]).
// Weights packed [tiles][KB][64][8]; activations in fragment order (act_idx, ntt token tiles) at byte
// offset x_off of the ring, polled. tile[t] < 0 or tt[j] < 0: nothing (zeros). Lanes of tokens >= M
// are not waited for and read as zeros.
// With RMS, the same poll also takes this wave's share of the producer's per-16-channel sums of h^2 over
// the TT*16 tokens of tt[0] .. (consecutive tiles; [w/16][ntt*16] at ssp_off, 16-byte pieces of 4 tokens:
// piece wave*64 + lane), and inv_rms receives 1/rms of each token (through ssq in LDS).
template <int WT, int KBW, int NT, int TT, bool RMS = false>
__device__ __forceinline__ bool unit_mma(int tid, const FusedArgs& a, const void* w, const int (&tile)[NT], int KB,
                                         __amdgpu_buffer_rsrc_t rr, unsigned x_off, const int (&tt)[TT], int M,
                                         f32x4 (&acc)[NT][TT], unsigned ssp_off = 0, float* ssq = nullptr,
                                         float* inv_rms = nullptr, int* lead = nullptr) {
  typedef typename FWReg<WT>::T WR;
  const int wave = tid >> 6, lane = tid & 63;
  const int kb0 = wave * KBW;
  WR wr[NT][KBW];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < KBW; ++i) {
      const size_t e = ((size_t)(tile[t] >= 0 ? tile[t] : 0) * KB + kb0 + i) * 64 + lane;
      wr[t][i] = ((const WR*)w)[e];
    }
  constexpr int NX = KBW * TT, QPG = TT * 4;  // activation pieces; 4-token quads per channel group
  const int ng = a.w / 16, Mp = a.ntt * 16;
  const int g_rms = (wave * 64 + lane) / QPG, q_rms = lane % QPG;  // this lane's RMS piece
  auto off = [&](int q) {
    if (RMS && q == NX) return ssp_off + (unsigned)((((g_rms < ng ? g_rms : 0) * Mp) + tt[0] * 16 + q_rms * 4) * 4);
    const int i = q / TT, j = q % TT, tj = tt[j] >= 0 ? tt[j] : 0;
    return x_off + (unsigned)((((kb0 + i) * a.ntt + tj) * 64 + lane) * 16);
  };
  auto need = [&](int q) {
    if (RMS && q == NX) return g_rms < ng && tt[q_rms / 4] >= 0;  // a piece of an absent token tile: nothing
    const int j = q % TT;
    return tt[j] >= 0 && tt[j] * 16 + (lane & 15) < M;
  };
  i32x4 xv[NX + (RMS ? 1 : 0)];
  const bool ok = poll16<NX + (RMS ? 1 : 0)>(rr, off, need, xv, a, lead);
  if constexpr (RMS) {
    // sum this wave's channel groups per 4-token quad (lanes q_rms, q_rms + QPG, ...), then the waves in LDS
    f32x4 r = __builtin_bit_cast(f32x4, xv[NX]);
#pragma unroll
    for (int sh = QPG; sh < 64; sh <<= 1) {
      r[0] += __shfl_xor(r[0], sh);
      r[1] += __shfl_xor(r[1], sh);
      r[2] += __shfl_xor(r[2], sh);
      r[3] += __shfl_xor(r[3], sh);
    }
    if (lane < QPG) *(f32x4*)(ssq + wave * 64 + lane * 4) = r;
    lds_barrier();
    if (tid < TT * 16) {
      float t = 0.f;
#pragma unroll
      for (int q = 0; q < FW; ++q) t += ssq[q * 64 + tid];
      inv_rms[tid] = rsqrtf(t * a.inv_w + a.eps);
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < TT; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (!ok) return false;
#pragma unroll
  for (int i = 0; i < KBW; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const bf16x8 av = to_bf16x8<WT>(wr[t][i]);
#pragma unroll
      for (int j = 0; j < TT; ++j)
        acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, xv[i * TT + j]), acc[t][j], 0, 0, 0);
    }
  return true;
}

// Partial tiles of the 8 waves -> res[q][64 lanes][4] (MFMA layout: lane -> token lane % 16, channels
// 4 (lane / 16) + v) in LDS. Ends with a barrier.
template <int NQ>
__device__ __forceinline__ void unit_reduce(int tid, const f32x4 (&accq)[NQ], float* red, float* res) {
  const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int q = 0; q < NQ; ++q) *(f32x4*)(red + ((wave * NQ + q) * 64 + lane) * 4) = accq[q];
  lds_barrier();
  for (int e = tid; e < NQ * 64; e += FT) {
    f32x4 s = *(const f32x4*)(red + e * 4);
#pragma unroll
    for (int wv = 1; wv < FW; ++wv) s += *(const f32x4*)(red + (wv * NQ * 64 + e) * 4);
    *(f32x4*)(res + e * 4) = s;
  }
  lds_barrier();
}

// MFMA-layout index of (channel c, token t) of a 16 x 16 tile
__device__ __forceinline__ int mfma_idx(int c, int t) { return ((c >> 2) * 16 + t) * 4 + (c & 3); }

// Residual epilogue: slot (LDS, MFMA layout) += val (already in slot when add is null); then
// hb = h * gain in fragment order and the tile's partial sums of h^2, stored device-scope.
__device__ __forceinline__ void resid_store(int tid, const FusedArgs& a, const float* slot, int tile, int tt, const float* gain,
                                            __amdgpu_buffer_rsrc_t rr, unsigned hb_off, unsigned ssp_off) {
  const int t = tid;
  if (t < 64) {  // (token, channel quad) -> 4 channels, one 8-byte store
    const int tok = t & 15, cq = t >> 4, tg = tt * 16 + tok;
    if (tg < a.H) {
      const int n0 = tile * 16 + cq * 4;
      const float4 h = *(const float4*)(slot + (cq * 16 + tok) * 4);
      const float4 g = *(const float4*)(gain + n0);
      const uint2 o = make_uint2(pack_bf16x2(h.x * g.x, h.y * g.y), pack_bf16x2(h.z * g.z, h.w * g.w));
      st8_coherent(rr, hb_off + (unsigned)(act_idx(tg, n0, a.ntt) * 2), o);
    }
  } else if (t < 80) {  // every row of the token tile (padding rows hold h = 0), so 4-token pieces are whole
    const int tok = t - 64, tg = tt * 16 + tok;
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const float h = slot[mfma_idx(c, tok)];
      s += h * h;
    }
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(s), rr, ssp_off + (unsigned)((tile * a.ntt * 16 + tg) * 4), 0, 0x10);
  }
}

// ------------------------------------------------------------------ the step kernel

// Every phase rebuilds its context from the kernel's argument segment through a pointer the compiler
// cannot see through (an empty asm takes and returns it), so no argument or derived value is held in
// registers from one phase into the next: each phase allocates its registers as if it ran alone,
// without the call and register save cost of out-of-line phase functions. The segment (and the
// per-layer table) are read in the constant address space: scalar loads, and never reloaded after a
// store (through a plain pointer every store could alias them, and each reload costs a memory round
// trip on the phase's critical path).
typedef const __attribute__((address_space(4))) FusedArgs* ConstArgs;
typedef const __attribute__((address_space(4))) FusedLayer* ConstLayers;
typedef const __attribute__((address_space(4))) unsigned long long* ConstWords;

// A struct of scalars and pointers read from the constant address space, word by word (scalar loads).
template <class T>
__device__ __forceinline__ T load_const(ConstWords p) {
  static_assert(sizeof(T) % 8 == 0, "whole 8-byte words");
  unsigned long long w[sizeof(T) / 8];
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 8); ++i) w[i] = p[i];
  T r;
  __builtin_memcpy(&r, w, sizeof(T));
  return r;
}

template <int DH, int MT, int KW, int KO, int KF>
struct FusedStep {
  const FusedArgs& a;
  char* lds;
  float* red;
  float* res;
  float* inv_rms;
  float* ssq;
  float* slots;
  int* lds_abort;
  __amdgpu_buffer_rsrc_t rr;
  int tid;  // tid, opaque to the compiler: nothing derived from it is shared between phases

  __device__ __forceinline__ FusedStep(const FusedArgs& args, char* smem) : a(args), lds(smem) {
    tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    red = (float*)smem;
    res = red + FW * F_NQ * 256;
    inv_rms = res + F_NQ * 256;
    ssq = inv_rms + 64;
    slots = (float*)(smem + fused_scratch_bytes<DH>());
    lds_abort = (int*)(slots + F_SLOTS * 256);
    rr = make_rsrc(a.ring);
  }

  __device__ unsigned blk(int l) const { return (unsigned)l * a.layer_bytes; }


  // A phase result: every thread of the workgroup leaves together when any wave's wait gave up.
  __device__ bool settle(bool ok) {
    if (!ok) *lds_abort = 1;
    lds_barrier();
    return *lds_abort == 0;
  }

  // EXCH_EMPTY over this workgroup's share of block l of the other launch's ring and of layer l of the
  // other launch's attention partials (plain stores: the other launch's polls read memory after this
  // launch has ended)
  __device__ void reset_other(int l) {
    const uint4 e4 = make_uint4(EXCH_EMPTY, EXCH_EMPTY, EXCH_EMPTY, EXCH_EMPTY);
    {
      const unsigned n16 = a.layer_bytes / 16, per = (n16 + a.G - 1) / a.G;
      uint4* dst = (uint4*)(a.ring_other + (size_t)l * a.layer_bytes);
      const unsigned e0 = blockIdx.x * per, e1 = min(e0 + per, n16);
      for (unsigned e = e0 + tid; e < e1; e += FT) dst[e] = e4;
    }
    if (l < a.L) {
      const size_t rows = (size_t)a.n_att * ATT_ROWS;
      const unsigned n16 = (unsigned)(rows * a.dh / 4), per = (n16 + a.G - 1) / a.G;
      uint4* dst = (uint4*)(a.part_o_other + (size_t)l * rows * a.dh);
      const unsigned e0 = blockIdx.x * per, e1 = min(e0 + per, n16);
      for (unsigned e = e0 + tid; e < e1; e += FT) dst[e] = e4;
      const unsigned m16 = (unsigned)(rows * 2 / 4), mper = (m16 + a.G - 1) / a.G;  // (m, l) pairs, 16 bytes = 2 rows
      uint4* mdst = (uint4*)(a.part_ml_other + (size_t)l * rows * 2);
      const unsigned m0 = blockIdx.x * mper, m1 = min(m0 + mper, m16);
      for (unsigned e = m0 + tid; e < m1; e += FT) mdst[e] = e4;
    }
  }

  // ---- in_proj: h = x W_in^T + b_in + temb for (tile, token tile); h stays in the slot
  __device__ void phase_in() {
    const TokSplit ts = tok_split(a.G, a.ntp);
    const int tt = ts.tg;
    if (tt >= a.ntt) return;
    for (int i = 0, tile = ts.gid; tile < a.w / 16 && i < F_SLOTS; ++i, tile += ts.n_groups) {
      float* slot = slots + i * 256;
      if (tid < 256) {
        const int e = tid, ln = e >> 2, c = ((ln >> 4) << 2) + (e & 3), tok = ln & 15, tg = tt * 16 + tok;
        const int n = tile * 16 + c;
        float h = 0.f;
        if (tg < a.H) {
          h = a.b_in[n] + a.temb[n];
          const float* xr = a.x + (size_t)tg * a.A;
          const uint16_t* wr = a.w_in + (size_t)n * a.A;
          for (int k = 0; k < a.A; ++k) h += xr[k] * bf16_to_f32(wr[k]);
        }
        slot[e] = h;
      }
      lds_barrier();
      resid_store(tid, a, slot, tile, tt, a.m_g1 ? a.m_g1 : a.ln1_0, rr, blk(0), blk(0) + a.off_ssp);
    }
  }

  // ---- QKV + RoPE for (up to 3 tiles, one token tile): q, k, v in the attention's fragment orders
  __device__ bool phase_qkv(int l) {
    const FusedLayer Ly = load_const<FusedLayer>((ConstWords)(a.layers + l));
    const TokSplit ts = tok_split(a.G, a.ntp);
    const int tt = ts.tg;
    const int n_tiles = (a.nq + 2 * a.nkv) * a.dh / 16;
    if (tt >= a.ntt) return true;
    const int ttv[1] = {tt};
    for (int t0 = ts.gid; t0 < n_tiles; t0 += F_QKV_NT * ts.n_groups) {
      int tile[F_QKV_NT];
#pragma unroll
      for (int t = 0; t < F_QKV_NT; ++t) tile[t] = t0 + t * ts.n_groups < n_tiles ? t0 + t * ts.n_groups : -1;
      f32x4 acc[F_QKV_NT][1];
      const bool ok = unit_mma<WT_BF16, KW, F_QKV_NT, 1, true>(tid, a, Ly.qkv, tile, a.w / 32, rr, blk(l), ttv, a.H, acc,
                                                               blk(l) + a.off_ssp, ssq, inv_rms, lds_abort + 1);
      f32x4 accq[F_QKV_NT];
#pragma unroll
      for (int t = 0; t < F_QKV_NT; ++t) accq[t] = acc[t][0];
      if (!settle(ok)) return false;
      unit_reduce<F_QKV_NT>(tid, accq, red, res);
#pragma unroll
      for (int t = 0; t < F_QKV_NT; ++t)
        if (tile[t] >= 0) qkv_epilogue(l, tile[t], tt, res + t * 256, Ly.qk_gain);
      lds_barrier();
    }
    return true;
  }

  __device__ void qkv_epilogue(int l, int tin, int tt, const float* r, const float* qk_gain) {
    const int dh = a.dh, tph = dh / 16, half = dh / 2, nkb = dh / KBLK;
    const int q_tiles = a.nq * tph, k_tiles = a.nkv * tph, gq = a.nq / a.nkv;
    const int t = tid;
    const float* sb = a.m_bqkv ? a.m_bqkv + (size_t)l * a.m_sqkv + tin * 16 : nullptr;  // shift bias of the tile
    if (tin < q_tiles + k_tiles) {
      if (t >= 32) return;
      const int tok = t >> 1, hf = t & 1, tg = tt * 16 + tok;  // (token, half of the tile's channels)
      if (tg >= a.H) return;
      const bool is_q = tin < q_tiles;
      const int tt2 = is_q ? tin : tin - q_tiles, head = tt2 / tph, pair = tt2 % tph;
      const float ir = inv_rms[tok];
      float xs[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) xs[c] = r[mfma_idx(c, tok)] * ir + (sb ? sb[c] : 0.f);
      if (qk_gain) {  // QK-norm: the tile's share of the head's sum of squares, then the gains (before RoPE)
        float sq2 = 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c) sq2 += xs[c] * xs[c];
        if (hf == 0)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(sq2), rr,
                                                blk(l) + a.off_qks + (unsigned)(((size_t)tin * a.ntt * 16 + tg) * 4), 0, 0x10);
#pragma unroll
        for (int c = 0; c < 16; ++c) xs[c] *= qk_gain[tin * 16 + c];
      }
      const float4* csp = (const float4*)(a.rope_cs + ((size_t)tg * half + pair * 8) * 2);
      float out[8];
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const float4 cs2 = csp[j / 2];  // (cos, sin) of dims pair*8 + j and + j + 1
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const float cc = u ? cs2.z : cs2.x, ss = u ? cs2.w : cs2.y;
          const float x1 = xs[j + u], x2 = xs[8 + j + u];
          out[j + u] = hf ? x1 * ss + x2 * cc : x1 * cc - x2 * ss;
        }
      }
      const int dfull = hf * half + pair * 8;
      const int lgrp = ((dfull % KBLK) >> 3) << 4, kb = dfull / KBLK;
      unsigned off;
      if (is_q) {
        const int gg = head / gq, rq = (head % gq) * a.H + tg;
        off = a.off_q + (unsigned)(((((size_t)gg * a.n_qt + (rq >> 4)) * nkb + kb) * 512 + (lgrp + (rq & 15)) * 8) * 2);
      } else {
        const int kk = tg & 31, kt = (kk & 7) >> 2, m = 4 * (kk >> 3) + (kk & 3);
        off = a.off_k + (unsigned)((((((size_t)head * a.nbs + (tg >> 5)) * 2 + kt) * nkb + kb) * 512 + (lgrp + m) * 8) * 2);
      }
      const uint4 o = make_uint4(pack_bf16x2(out[0], out[1]), pack_bf16x2(out[2], out[3]), pack_bf16x2(out[4], out[5]),
                                 pack_bf16x2(out[6], out[7]));
      st16u_coherent(rr, blk(l) + off, o);
    } else {
      // value tile: thread -> (dim c, 8-key group kq8) -> 8 keys of one dim, one 16-byte store; keys past
      // H in a group that has a valid key are written as zeros
      if (t >= 32) return;
      const int c = t & 15, g8 = t >> 4, t0 = tt * 16 + g8 * 8;
      if (t0 >= a.H) return;
      const int tv = tin - q_tiles - k_tiles, hd = tv / tph, d16 = tv % tph;
      float vv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tok = g8 * 8 + e;
        vv[e] = t0 + e < a.H ? r[mfma_idx(c, tok)] * inv_rms[tok] + (sb ? sb[c] : 0.f) : 0.f;
      }
      const size_t fr = ((size_t)hd * a.nbs + (t0 >> 5)) * tph + d16;
      const unsigned off = a.off_v + (unsigned)((fr * 512 + ((((t0 & 31) >> 3) << 4) + c) * 8) * 2);
      const uint4 o = make_uint4(pack_bf16x2(vv[0], vv[1]), pack_bf16x2(vv[2], vv[3]), pack_bf16x2(vv[4], vv[5]),
                                 pack_bf16x2(vv[6], vv[7]));
      st16u_coherent(rr, blk(l) + off, o);
    }
  }

  // ---- attention units: unit -> (split, query tile, kv head). The i-th unit of this workgroup, or -1.
  __device__ int att_unit_of(int i) const {
    const int upsp = a.n_qt * a.nkv;
    const int xps = a.n_split <= 8 ? 8 / a.n_split : 0;
    if (xps > 0 && (upsp + xps - 1) / xps <= a.G / 8) {
      // split s on XCDs s*xps .. +xps, so the workgroups reading a split's K/V share L2s
      const int xcd = blockIdx.x & 7, r = blockIdx.x >> 3, s = xcd / xps;
      const int j = r * xps + xcd % xps;
      return i == 0 && s < a.n_split && j < upsp ? s * upsp + j : -1;
    }
    const int u = blockIdx.x + i * a.G;
    return u < a.n_att ? u : -1;
  }
  __device__ bool att_nth(int l, int i) {
    const int u = att_unit_of(i);
    return u < 0 ? true : att_unit(l, u);
  }
  __device__ bool merge_nth(int l, int i) {
    const int u = att_unit_of(i);
    return u < 0 ? true : merge_unit(l, u);
  }

  // Attention of one unit over its split's key blocks (one 32-key block per wave): prefix K/V with
  // plain loads issued first, the query tile and suffix K/V polled; the unit's (O, m, l) partial is
  // published device-scope for the merge.
  __device__ bool att_unit(int l, int u) {
    const FusedLayer Ly = load_const<FusedLayer>((ConstWords)(a.layers + l));
    constexpr int NKB = DH / KBLK, NDT = DH / 16, LDO = DH + 4, FR = 512;
    const int upsp = a.n_qt * a.nkv;
    const int split = u / upsp, qt = (u % upsp) / a.nkv, g = u % a.nkv;
    const int gq = a.nq / a.nkv, R = gq * a.H;
    const int wave = tid >> 6, lane = tid & 63;
    float* Ow = (float*)lds;
    float* MLw = Ow + FW * ATT_ROWS * LDO;
    uint16_t* Qs = (uint16_t*)(MLw + FW * ATT_ROWS * 2);
    const int nb = a.nbp + a.nbs, bps = (nb + a.n_split - 1) / a.n_split;
    const int b_begin = split * bps, b_end = min(nb, b_begin + bps);
    const int bb = b_begin + wave;
    const bool has = bb < b_end, pre = has && bb < a.nbp;
    const int n_valid = !has ? 0 : pre ? min(ATT_KB, a.P - bb * ATT_KB) : min(ATT_KB, a.H - (bb - a.nbp) * ATT_KB);
    typedef bf16x8 B8;
    constexpr int NKV = 2 * NKB + NDT;  // K fragments [kt][kb], then V fragments [dt]
    i32x4 kv[NKV];
    bool ok = true;
    if (pre) {  // a prefix block: plain loads (a wave with no block of the split loads nothing)
      const uint16_t* kf = Ly.kc + a.slot_off + ((size_t)g * a.nbp + bb) * (2 * NKB * FR);
      const uint16_t* vf = Ly.vc + a.slot_off + ((size_t)g * a.nbp + bb) * (2 * NKB * FR);
#pragma unroll
      for (int i = 0; i < 2 * NKB; ++i) kv[i] = *(const i32x4*)(kf + i * FR + lane * 8);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) kv[2 * NKB + dt] = *(const i32x4*)(vf + dt * FR + lane * 8);
    }
    // the query tile: thread e -> 16 bytes at e * 16 of the tile ([NKB][64][8]), row = lane % 16
    {
      constexpr int QV = NKB * 64;  // 16-byte pieces
      const unsigned qoff = blk(l) + a.off_q + (unsigned)(((size_t)g * a.n_qt + qt) * NKB * FR * 2);
      for (int e0 = 0; e0 < QV; e0 += FT) {
        const int e = e0 + (int)tid;
        i32x4 v[1];
        ok = poll16<1>(
                 rr, [&](int) { return qoff + (unsigned)((e < QV ? e : 0) * 16); },
                 [&](int) { return e < QV && qt * ATT_ROWS + (e & 15) < R; }, v, a) &&
             ok;
        if (e < QV) *(i32x4*)(Qs + e * 8) = v[0];
      }
    }
    if (has && !pre) {  // suffix block: poll its K and V fragments
      const int sb = bb - a.nbp;
      const unsigned koff = blk(l) + a.off_k + (unsigned)((((size_t)g * a.nbs + sb) * 2 * NKB * FR) * 2);
      const unsigned voff = blk(l) + a.off_v + (unsigned)((((size_t)g * a.nbs + sb) * NDT * FR) * 2);
      const int m = lane & 15;
      // K piece i = kt * NKB + kb holds key 8 (m / 4) + 4 kt + m % 4 of the block; a V piece holds keys
      // 8 (lane / 16) .. + 8, written whole (zeros past H) when its first key is valid
      ok = poll16<NKV>(
               rr,
               [&](int i) {
                 return i < 2 * NKB ? koff + (unsigned)((i * FR + lane * 8) * 2)
                                    : voff + (unsigned)(((i - 2 * NKB) * FR + lane * 8) * 2);
               },
               [&](int i) { return i < 2 * NKB ? 8 * (m >> 2) + 4 * (i / NKB) + (m & 3) < n_valid : (lane >> 4) * 8 < n_valid; },
               kv, a) &&
           ok;
    }
    // QK-norm: 1/rms of the 16 query rows and of this wave's suffix keys, from the QKV tiles' sums of
    // squares (prefix keys come normalised)
    float* rq_s = (float*)(lds + fused_scratch_bytes<DH>() + (size_t)F_SLOTS * 1024 + 16);
    float* rk_s = rq_s + ATT_ROWS + wave * ATT_KB;
    if (a.off_qks) {
      constexpr int TPH = DH / 16;
      static_assert(TPH <= 16, "16 lanes per query row");
      const int Mp = a.ntt * 16, q_tiles = a.nq * TPH;
      if (tid < ATT_ROWS * 16) {  // thread -> (row, tile of the row's head)
        const int row = tid >> 4, i = tid & 15, rg = qt * ATT_ROWS + row;
        const bool need = rg < R && i < TPH;
        const int head = g * gq + (rg < R ? rg / a.H : 0), t = rg < R ? rg % a.H : 0;
        float v[1];
        ok = poll4<1>(rr, {blk(l) + a.off_qks + (unsigned)((((size_t)head * TPH + (need ? i : 0)) * Mp + t) * 4)}, {need}, v, a) &&
             ok;
        float sum = v[0];
        sum += __shfl_xor(sum, 1);
        sum += __shfl_xor(sum, 2);
        sum += __shfl_xor(sum, 4);
        sum += __shfl_xor(sum, 8);
        if (i == 0) rq_s[row] = rg < R ? rsqrtf(sum * a.qk_inv_dh + a.qk_eps) : 0.f;
      }
      if (has && !pre) {  // lane -> (key lane % 32, tiles 8 (lane / 32) ..): 8 partial sums each
        const int kk = lane & 31, t = (bb - a.nbp) * ATT_KB + kk, i0 = (lane >> 5) * 8;
        const bool kv_ok = t < a.H;
        float v[8];
        unsigned offs[8];
        bool needs[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          needs[j] = kv_ok && i0 + j < TPH;
          offs[j] = blk(l) + a.off_qks +
                    (unsigned)((((size_t)q_tiles + g * TPH + (needs[j] ? i0 + j : 0)) * Mp + (kv_ok ? t : 0)) * 4);
        }
        ok = poll4<8>(rr, offs, needs, v, a) && ok;
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) sum += v[j];
        sum += __shfl_xor(sum, 32);
        if (lane < ATT_KB) rk_s[kk] = kv_ok ? rsqrtf(sum * a.qk_inv_dh + a.qk_eps) : 0.f;
      }
    }
    if (!settle(ok)) return false;
    if (has) {
    // S^T = K Q^T, online softmax over the block, O^T = V^T P^T (as the stand-alone attention)
    const int k8 = 8 * (lane >> 4);
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const B8 qb = *(const B8*)(Qs + kb * FR + lane * 8);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(B8, kv[kt * NKB + kb]), qb, sacc[kt], 0, 0, 0);
    }
    float mb = -INFINITY;
    const float row_scale = a.off_qks ? a.scale_log2 * rq_s[lane & 15] : a.scale_log2;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float f = row_scale;
        if (a.off_qks && !pre && k8 + 4 * kt + v < n_valid) f *= rk_s[k8 + 4 * kt + v];
        const float sv = (k8 + 4 * kt + v < n_valid) ? sacc[kt][v] * f : -INFINITY;
        sacc[kt][v] = sv;
        mb = fmaxf(mb, sv);
      }
    mb = fmaxf(mb, __shfl_xor(mb, 16));
    mb = fmaxf(mb, __shfl_xor(mb, 32));
    float lb = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float p = (mb == -INFINITY) ? 0.f : exp2f(sacc[kt][v] - mb);
        sacc[kt][v] = p;
        lb += p;
      }
    lb += __shfl_xor(lb, 16);
    lb += __shfl_xor(lb, 32);
    const B8 pb = B8{(__bf16)sacc[0][0], (__bf16)sacc[0][1], (__bf16)sacc[0][2], (__bf16)sacc[0][3],
                     (__bf16)sacc[1][0], (__bf16)sacc[1][1], (__bf16)sacc[1][2], (__bf16)sacc[1][3]};
    f32x4 oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(B8, kv[2 * NKB + dt]), pb, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    float* ow = Ow + (size_t)wave * ATT_ROWS * LDO + (lane & 15) * LDO + 4 * (lane >> 4);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) *(f32x4*)(ow + dt * 16) = oacc[dt];
    if (lane < 16) *(float2*)(MLw + (wave * ATT_ROWS + lane) * 2) = make_float2(mb, lb);
    } else if (lane < 16) {  // no block: m = -inf marks the wave's O (never written) as absent
      *(float2*)(MLw + (wave * ATT_ROWS + lane) * 2) = make_float2(-INFINITY, 0.f);
    }
    lds_barrier();
    // merge the waves: thread -> (row, 16-byte chunk), published as this unit's partial
    constexpr int CPR = DH / 4;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.part_o), rm = make_rsrc(a.part_ml);
    const size_t prow = ((size_t)l * a.n_att + u) * ATT_ROWS;
    for (int q = tid; q < ATT_ROWS * CPR; q += FT) {
      const int row = q / CPR, c4 = q % CPR;
      float M = -INFINITY;
#pragma unroll
      for (int wv = 0; wv < FW; ++wv) M = fmaxf(M, MLw[(wv * ATT_ROWS + row) * 2]);
      float Lsum = 0.f;
      f32x4 O = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int wv = 0; wv < FW; ++wv) {
        const float mw = MLw[(wv * ATT_ROWS + row) * 2];
        if (mw != -INFINITY) {
          const float wt = exp2f(mw - M);
          Lsum += wt * MLw[(wv * ATT_ROWS + row) * 2 + 1];
          O += wt * *(const f32x4*)(Ow + ((size_t)wv * ATT_ROWS + row) * LDO + 4 * c4);
        }
      }
      st16_coherent(ro, (unsigned)(((prow + row) * DH + 4 * c4) * 4), make_float4(O[0], O[1], O[2], O[3]));
      if (c4 == 0)
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, make_float2(M, Lsum)), rm, (unsigned)((prow + row) * 8), 0, 0x10);
    }
    lds_barrier();
    return true;
  }

  // Merge of one unit's share of its query tile (rows split * rps .. + rps) from every split's partial;
  // o in fragment order (act_idx), four dims per 8-byte store.
  __device__ bool merge_unit(int l, int u) {
    const int upsp = a.n_qt * a.nkv;
    const int split = u / upsp, rest = u % upsp, qt = rest / a.nkv, g = rest % a.nkv;
    const int gq = a.nq / a.nkv, R = gq * a.H;
    const int rps = (ATT_ROWS + a.n_split - 1) / a.n_split;
    constexpr int TPC = DH / 4, RPP = FT / TPC;
    const int kc = tid % TPC;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.part_o), rm = make_rsrc(a.part_ml);
    bool ok = true;
    for (int rb = 0; rb < rps; rb += RPP) {
      const int rl = rb + (int)tid / TPC, rr2 = split * rps + rl;
      const bool act = rl < rps && rr2 < ATT_ROWS;
      float M2 = -INFINITY, L2 = 0.f;
      f32x4 O2 = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int c0 = 0; c0 < a.n_split; c0 += 8) {
        const int nc = min(8, a.n_split - c0);
        float2 ml[8];
        f32x4 oc[8];
        auto unit_of = [&](int c) { return (c0 + c) * upsp + rest; };
        auto moff = [&](int c) { return (unsigned)((((size_t)l * a.n_att + unit_of(c)) * ATT_ROWS + (act ? rr2 : 0)) * 8); };
        auto ooff = [&](int c) {
          return (unsigned)(((((size_t)l * a.n_att + unit_of(c)) * ATT_ROWS + (act ? rr2 : 0)) * DH + kc * 4) * 4);
        };
        const unsigned long long t_end = wall_clock64() + a.wait_ticks;
        for (;;) {
          bool okp = true;
#pragma unroll
          for (int c = 0; c < 8; ++c)
            if (c < nc) {
              ml[c] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rm, moff(c), 0, 0x10));
              oc[c] = ld16_coherent(ro, ooff(c));
              okp = okp && (!act || (exch_arrived(ml[c].x) && exch_arrived(ml[c].y) && exch_arrived(oc[c])));
            }
          const unsigned ab = __hip_atomic_load(a.abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (__all(okp)) break;
          if (ab != 0u || wall_clock64() > t_end) {
            if (ab == 0u) fused_give_up(a);
            ok = false;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        if (!ok) break;
        float Mn = M2;
#pragma unroll
        for (int c = 0; c < 8; ++c)
          if (c < nc) Mn = fmaxf(Mn, ml[c].x);
        const float sc = (M2 == -INFINITY) ? 0.f : exp2f(M2 - Mn);
        L2 *= sc;
        O2 *= sc;
#pragma unroll
        for (int c = 0; c < 8; ++c)
          if (c < nc) {
            const float wt = (ml[c].x == -INFINITY) ? 0.f : exp2f(ml[c].x - Mn);
            L2 += wt * ml[c].y;
            O2 += wt * oc[c];
          }
        M2 = Mn;
      }
      if (!ok) break;
      const int r2 = qt * ATT_ROWS + rr2;
      if (act && r2 < R) {
        const int tok = r2 % a.H, col = (g * gq + r2 / a.H) * DH + 4 * kc;
        const float inv = L2 > 0.f ? 1.f / L2 : 0.f;
        const uint2 o = make_uint2(pack_bf16x2(O2[0] * inv, O2[1] * inv), pack_bf16x2(O2[2] * inv, O2[3] * inv));
        st8_coherent(rr, blk(l) + a.off_o + (unsigned)(act_idx(tok, col, a.ntt) * 2), o);
      }
      // the partials read stay as they are: the next launch (which uses the other partial buffers)
      // writes the empty pattern over them
    }
    return settle(ok);
  }

  // ---- o_proj + residual for (tile, token tile); hb2 = h * ln2 and its RMS partials
  __device__ bool phase_oproj(int l) {
    const FusedLayer Ly = load_const<FusedLayer>((ConstWords)(a.layers + l));
    const TokSplit ts = tok_split(a.G, a.ntp);
    const int tt = ts.tg;
    if (tt >= a.ntt) return true;
    const int ttv[1] = {tt};
    for (int i = 0, tile = ts.gid; tile < a.w / 16 && i < F_SLOTS; ++i, tile += ts.n_groups) {
      const int tl[1] = {tile};
      f32x4 acc[1][1];
      const bool ok = unit_mma<WT_BF16, KO, 1, 1>(tid, a, Ly.o, tl, a.nq * a.dh / 32, rr, blk(l) + a.off_o, ttv, a.H, acc,
                                                  0, nullptr, nullptr, lds_abort + 1);
      if (!settle(ok)) return false;
      const f32x4 accq[1] = {acc[0][0]};
      unit_reduce<1>(tid, accq, red, res);
      float* slot = slots + i * 256;
      const float* gate = a.m_mod ? a.m_mod + (size_t)l * a.m_smod + 2 * a.w : nullptr;  // time modulation
      if (tid < 256) {
        const int ln = tid >> 2, c = ((ln >> 4) << 2) + (tid & 3);
        slot[tid] += gate ? gate[tile * 16 + c] * res[tid] : res[tid];
      }
      lds_barrier();
      resid_store(tid, a, slot, tile, tt, a.m_g2 ? a.m_g2 + (size_t)l * a.m_sw : Ly.ln2, rr, blk(l) + a.off_hb2,
                  blk(l) + a.off_ssp2);
    }
    return true;
  }

  // ---- gate/up + GeGLU for (2 tile pairs, a group of token tiles); u in fragment order
  __device__ bool phase_gu(int l) {
    const FusedLayer Ly = load_const<FusedLayer>((ConstWords)(a.layers + l));
    const int TS = a.ntp >= 2 ? a.ntp / 2 : 1, tgn = a.ntp / TS;  // token groups, token tiles per group (<= 2)
    const TokSplit ts = tok_split(a.G, TS);
    const int n_pairs = a.F / 16;
    int ttv[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int tj = ts.tg * tgn + j;
      ttv[j] = j < tgn && tj < a.ntt ? tj : -1;
    }
    if (ttv[0] < 0) return true;
    for (int p0 = ts.gid; p0 < n_pairs; p0 += 2 * ts.n_groups) {
      const int p1 = p0 + ts.n_groups;
      const int tile[4] = {2 * p0, 2 * p0 + 1, p1 < n_pairs ? 2 * p1 : -1, p1 < n_pairs ? 2 * p1 + 1 : -1};
      f32x4 acc[4][2];
      const bool ok = unit_mma<MT, KW, 4, 2, true>(tid, a, Ly.gu, tile, a.w / 32, rr, blk(l) + a.off_hb2, ttv, a.H, acc,
                                                   blk(l) + a.off_ssp2, ssq, inv_rms, lds_abort + 1);
      if (!settle(ok)) return false;
      f32x4 accq[8];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 2; ++j) accq[t * 2 + j] = acc[t][j];
      unit_reduce<8>(tid, accq, red, res);
      // thread -> (pair pp, token tile j, token, channel quad) -> 4 features, one 8-byte store
      if (tid < 256) {
        const int e = tid, tok = e & 15, cq = (e >> 4) & 3, j = (e >> 6) & 1, pp = e >> 7;
        const int p = pp ? p1 : p0;
        if (ttv[j] >= 0 && (pp == 0 || p1 < n_pairs)) {
          const int tg = ttv[j] * 16 + tok;
          if (tg < a.H) {
            const float ir = inv_rms[j * 16 + tok];
            const float* gr = res + ((pp * 2 + 0) * 2 + j) * 256;
            const float* ur = res + ((pp * 2 + 1) * 2 + j) * 256;
            float4 gv = *(const float4*)(gr + (cq * 16 + tok) * 4), uv = *(const float4*)(ur + (cq * 16 + tok) * 4);
            if constexpr (MT == WT_FP8) {
              const float4 sg = *(const float4*)(Ly.gu_s + (size_t)(2 * p) * 16 + cq * 4);
              const float4 su = *(const float4*)(Ly.gu_s + (size_t)(2 * p + 1) * 16 + cq * 4);
              gv = make_float4(gv.x * sg.x, gv.y * sg.y, gv.z * sg.z, gv.w * sg.w);
              uv = make_float4(uv.x * su.x, uv.y * su.y, uv.z * su.z, uv.w * su.w);
            }
            gv = make_float4(gv.x * ir, gv.y * ir, gv.z * ir, gv.w * ir);
            uv = make_float4(uv.x * ir, uv.y * ir, uv.z * ir, uv.w * ir);
            if (a.m_bgu) {  // time modulation: the shift biases of the gate and up channels
              const float* sb = a.m_bgu + (size_t)l * a.m_sgu;
              const float4 bg = *(const float4*)(sb + (size_t)(2 * p) * 16 + cq * 4);
              const float4 bu = *(const float4*)(sb + (size_t)(2 * p + 1) * 16 + cq * 4);
              gv = make_float4(gv.x + bg.x, gv.y + bg.y, gv.z + bg.z, gv.w + bg.w);
              uv = make_float4(uv.x + bu.x, uv.y + bu.y, uv.z + bu.z, uv.w + bu.w);
            }
            const uint2 o = make_uint2(pack_bf16x2(gelu_tanh_fast(gv.x) * uv.x, gelu_tanh_fast(gv.y) * uv.y),
                                       pack_bf16x2(gelu_tanh_fast(gv.z) * uv.z, gelu_tanh_fast(gv.w) * uv.w));
            st8_coherent(rr, blk(l) + a.off_u + (unsigned)(act_idx(tg, p * 16 + cq * 4, a.ntt) * 2), o);
          }
        }
      }
      lds_barrier();
    }
    return true;
  }

  // ---- down + residual for (tile, token tile); hb_in of the next layer (or the final norm's input)
  __device__ bool phase_down(int l) {
    const FusedLayer Ly = load_const<FusedLayer>((ConstWords)(a.layers + l));
    const TokSplit ts = tok_split(a.G, a.ntp);
    const int tt = ts.tg;
    if (tt >= a.ntt) return true;
    const int ttv[1] = {tt};
    for (int i = 0, tile = ts.gid; tile < a.w / 16 && i < F_SLOTS; ++i, tile += ts.n_groups) {
      const int tl[1] = {tile};
      f32x4 acc[1][1];
      const bool ok = unit_mma<MT, KF, 1, 1>(tid, a, Ly.d, tl, a.F / 32, rr, blk(l) + a.off_u, ttv, a.H, acc, 0, nullptr,
                                             nullptr, lds_abort + 1);
      if (!settle(ok)) return false;
      const f32x4 accq[1] = {acc[0][0]};
      unit_reduce<1>(tid, accq, red, res);
      float* slot = slots + i * 256;
      const float* gate = a.m_mod ? a.m_mod + (size_t)l * a.m_smod + 5 * a.w : nullptr;  // time modulation
      if (tid < 256) {
        const int ln = tid >> 2, c = ((ln >> 4) << 2) + (tid & 3);
        float v = res[tid];
        if constexpr (MT == WT_FP8) v *= Ly.d_s[tile * 16 + c];
        slot[tid] += gate ? gate[tile * 16 + c] * v : v;
      }
      lds_barrier();
      const float* gn = !a.m_g1 ? Ly.g_next : l + 1 < a.L ? a.m_g1 + (size_t)(l + 1) * a.m_sw : a.m_gf;
      resid_store(tid, a, slot, tile, tt, gn, rr, blk(l + 1), blk(l + 1) + a.off_ssp);
    }
    return true;
  }

  // ---- out_proj + Euler update for (output tile, token tile): x += dt (rmsnorm(h) W_out^T + b_out)
  __device__ bool phase_out() {
    const TokSplit ts = tok_split(a.G, a.ntp);
    const int tt = ts.tg;
    if (tt >= a.ntt || ts.gid >= a.out_tiles) return true;
    const int ttv[1] = {tt};
    const int tl[1] = {ts.gid};
    f32x4 acc[1][1];
    const bool ok = unit_mma<WT_BF16, KW, 1, 1, true>(tid, a, a.w_out, tl, a.w / 32, rr, blk(a.L), ttv, a.H, acc,
                                                      blk(a.L) + a.off_ssp, ssq, inv_rms);
    if (!settle(ok)) return false;
    const f32x4 accq[1] = {acc[0][0]};
    unit_reduce<1>(tid, accq, red, res);
    if (tid < 256) {
      const int e = tid, ln = e >> 2, c = ((ln >> 4) << 2) + (e & 3), tok = ln & 15, tg = tt * 16 + tok;
      const int n = ts.gid * 16 + c;
      if (tg < a.H && n < a.A) {
        const float v = res[e] * inv_rms[tok] + a.b_out[n];
        a.x[(size_t)tg * a.A + n] += a.dt * v;
      }
    }
    return true;
  }

};

#define AE_FUSED_PHASE(NAME, CALL)                                                                      \
  template <int DH, int MT, int KW, int KO, int KF>                                                     \
  __device__ __forceinline__ bool NAME(const FusedArgs& args, char* lds, int l, int u) {                \
    FusedStep<DH, MT, KW, KO, KF> s(args, lds);                                                         \
    return CALL;                                                                                        \
  }
AE_FUSED_PHASE(fphase_in, (s.phase_in(), true))
AE_FUSED_PHASE(fphase_qkv, s.phase_qkv(l))
AE_FUSED_PHASE(fphase_att, s.att_nth(l, u))
AE_FUSED_PHASE(fphase_merge, s.merge_nth(l, u))
AE_FUSED_PHASE(fphase_oproj, s.phase_oproj(l))
AE_FUSED_PHASE(fphase_gu, s.phase_gu(l))
AE_FUSED_PHASE(fphase_down, s.phase_down(l))
AE_FUSED_PHASE(fphase_out, s.phase_out())
AE_FUSED_PHASE(fphase_reset, (s.reset_other(l), true))
#undef AE_FUSED_PHASE

template <int DH, int MT, int KW, int KO, int KF>
__global__ __launch_bounds__(FT) __attribute__((amdgpu_waves_per_eu(1, 2))) void fused_step_kernel(FusedArgs a) {
  extern __shared__ __attribute__((aligned(16))) char fsm[];
  int* lds_abort = (int*)(fsm + fused_scratch_bytes<DH>() + (size_t)F_SLOTS * 1024);
  if (threadIdx.x == 0) *lds_abort = __hip_atomic_load(a.abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
  __syncthreads();
  if (*lds_abort) return;
  fphase_in<DH, MT, KW, KO, KF>(a, fsm, 0, 0);
  const int n_layers = a.L;
  int n_units = 0;  // this workgroup's attention units (at most 4)
  {
    FusedStep<DH, MT, KW, KO, KF> s(a, fsm);
    while (n_units < 4 && s.att_unit_of(n_units) >= 0) ++n_units;
  }
  for (int l = 0; l < n_layers; ++l) {
    fphase_reset<DH, MT, KW, KO, KF>(a, fsm, l, 0);
    if (!fphase_qkv<DH, MT, KW, KO, KF>(a, fsm, l, 0)) return;
    for (int i = 0; i < n_units; ++i)
      if (!fphase_att<DH, MT, KW, KO, KF>(a, fsm, l, i)) return;
    for (int i = 0; i < n_units; ++i)
      if (!fphase_merge<DH, MT, KW, KO, KF>(a, fsm, l, i)) return;
    if (!fphase_oproj<DH, MT, KW, KO, KF>(a, fsm, l, 0)) return;
    if (!fphase_gu<DH, MT, KW, KO, KF>(a, fsm, l, 0)) return;
    if (!fphase_down<DH, MT, KW, KO, KF>(a, fsm, l, 0)) return;
  }
  if (!fphase_out<DH, MT, KW, KO, KF>(a, fsm, 0, 0)) return;
  fphase_reset<DH, MT, KW, KO, KF>(a, fsm, n_layers, 0);
}

// EXCH_EMPTY over n16 16-byte units (a whole activation ring; the partial buffers)
__global__ void fill_empty_kernel(uint4* p, size_t n16) {
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n16; e += (size_t)gridDim.x * blockDim.x)
    p[e] = make_uint4(EXCH_EMPTY, EXCH_EMPTY, EXCH_EMPTY, EXCH_EMPTY);
}

}  // namespace ae
