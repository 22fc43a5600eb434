// Host runtime of the action-expert library: implements include/ae.h.
//
// ae_create validates the shape contract, packs the weights into MFMA lane
// order and uploads them once; ae_load_prefix_kv fills a prefix slot;
// ae_denoise / ae_verify copy their small inputs into static device buffers
// and replay one captured hipGraph of the whole pass (DM0.5 guide, section
// 6.5: static buffers, fixed step count, one replay per request). Graphs are
// cached per (mode, steps or n_tau, batch).
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/ae.h"
#include "ae_host.hpp"
#include "ae_kernels.hpp"
#include "ae_fused.hpp"

using namespace ae;

namespace {

thread_local std::string g_create_error;

// Dispatch-bound timing events: when `start` is set, the next AE_LAUNCH binds
// this pair to its dispatch (hipExtLaunchKernel records the kernel's own start
// and end) and clears it.
struct DispatchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
thread_local DispatchEvents t_dispatch_ev;

#define AE_LAUNCH(kernel, grid, block, lds, st, ...)                                               \
  do {                                                                                             \
    if (t_dispatch_ev.start) {                                                                     \
      hipExtLaunchKernelGGL(kernel, grid, block, (std::uint32_t)(lds), st, t_dispatch_ev.start,    \
                            t_dispatch_ev.stop, 0, __VA_ARGS__);                                   \
      t_dispatch_ev = DispatchEvents{};                                                            \
    } else {                                                                                       \
      hipLaunchKernelGGL(kernel, grid, block, lds, st, __VA_ARGS__);                               \
    }                                                                                              \
  } while (0)

// Kernel filter and per-dispatch timing for ae_kernel_times. An enqueue pass
// launches only the kernels named `only` (all of them when empty) and records
// the names it meets; with `pairs` set, every launch gets the next event pair.
struct Timer {
  std::string only;
  int count = 0;
  std::vector<std::string> seen;
  std::vector<hipEvent_t>* pairs = nullptr;  // 2 per launch: start, stop
  std::vector<std::string> launched;         // name of each timed launch, in order
  bool overflow = false;
  bool take(const char* name) {
    if (std::find(seen.begin(), seen.end(), name) == seen.end()) seen.push_back(name);
    if (!only.empty() && only != name) return false;
    ++count;
    if (pairs) {
      size_t i = launched.size();
      if (2 * i + 1 < pairs->size()) {
        t_dispatch_ev.start = (*pairs)[2 * i];
        t_dispatch_ev.stop = (*pairs)[2 * i + 1];
        launched.push_back(name);
      } else {
        overflow = true;
      }
    }
    return true;
  }
};

using ae_host::dtype_size;

struct PhaseCfg {
  int S;  // k-splits
};

}  // namespace

// Split-K factor of each GEMM role when a pass has one token group (at most 4; pick() lowers it to what
// divides the role's k-blocks). AE_SPLITK=<o>,<down> sets the o_proj and down factors at ae_create.
struct Splits {
  int qkv = 1, o = 4, gu = 1, down = 4, out = 1;
};

struct ae_handle {
  ae_config c{};
  int dev = 0;
  hipStream_t stream = nullptr;
  std::string err;
  int at = AT_BF16;      // activation type
  int wt = WT_BF16;      // attention / projection weight type
  int mt = WT_BF16;      // MLP weight type
  int M_max = 0, Mp_max = 0;
  std::vector<void*> allocs;

  // weights (device)
  void *time_in_w = nullptr, *time_out_w = nullptr, *action_in_w = nullptr, *action_out_p = nullptr;
  float *time_in_b = nullptr, *time_out_b = nullptr, *action_in_b = nullptr, *action_out_b = nullptr;
  std::vector<void*> qkv_p, o_p, gu_p, d_p;
  std::vector<float*> gu_s, d_s;   // fp8 scales in packed order
  std::vector<float*> ln1, ln2;
  float* final_ln = nullptr;
  int qkv_tiles = 0, gu_tiles = 0, out_tiles = 0;

  // activations and scratch
  float *x = nullptr, *h = nullptr, *ssp_a = nullptr, *ssp_b = nullptr, *vout = nullptr;
  void *hb = nullptr, *o = nullptr, *u = nullptr;
  void *q = nullptr, *ks = nullptr, *vs = nullptr;  // attention operands of the suffix, fragment order
  float* part = nullptr;
  size_t part_floats = 0;
  unsigned* counters = nullptr;
  size_t n_counters = 0;
  float *opart = nullptr, *mlpart = nullptr;
  size_t opart_floats = 0, mlpart_floats = 0;
  unsigned long long wait_ticks = EXCH_WAIT;  // bound of every in-kernel wait (100 MHz ticks)
  unsigned* flag_host = nullptr;    // pinned host word, set by a kernel whose bounded wait gave up
  unsigned* flag_dev = nullptr;     // its device address
  // capture variant of the pass being enqueued: 0 = the persistent step kernel where eligible,
  // 1 = one launch per phase, 2 = one launch per phase with no in-kernel waits (no co-resident
  // exchanges: the pass a failed one is repeated with)
  int variant = 0;
  bool eager = false;               // AE_GRAPH=0: passes enqueue their launches instead of replaying a graph
  Splits sk;                        // split-K factors of the launch-per-phase GEMMs
  // persistent step kernel (batch-1 denoise)
  bool fused_ok = false;            // shape, dtypes, occupancy and AE_FUSED allow it
  std::string fused_why;            // why not, when fused_ok is false
  int fused_fail = 0;               // consecutive passes whose persistent launch gave up
  void (*fused_fn)(FusedArgs) = nullptr;
  size_t fused_lds = 0;
  FusedLayer* fused_layers = nullptr;  // device [L]
  char* ring[2] = {nullptr, nullptr};  // activation rings of alternating launches
  unsigned layer_bytes = 0, off_ssp = 0, off_q = 0, off_k = 0, off_v = 0, off_o = 0, off_hb2 = 0, off_ssp2 = 0, off_u = 0;
  unsigned off_qks = 0;              // QK-norm partials in a ring block (0: none)
  float *fpart_o = nullptr, *fpart_ml = nullptr;
  size_t fpart_o_floats = 0, fpart_ml_floats = 0;
  unsigned* abort_dev = nullptr;
  int f_nsplit = 0, f_natt = 0;
  int n_qt = 0, nbp = 0, nbs = 0;  // 16-row query tiles, 32-key prefix / suffix blocks
  int n_cu = 0;
  void* static_scratch = nullptr;   // device address of this device's `scratch` array (ae_denoise_static)
  std::string static_err;           // why it is null
  // in-kernel partial exchanges (read from AE_ATTN_CORESIDENT / AE_EXCH_POLL at creation, 0 = off):
  // attention key splits merged by co-resident workgroups, split-K partials polled by split S-1
  bool coresident_attn = true, poll_splitk = true;
  int occ_attn = 0, occ_gemm = 0, occ_fused = 0;  // workgroups per CU of the kernels that may wait in-kernel
  int tiled_roles = 0xf;  // GEMM roles (bit per Role) that may take the token-tiled kernel
  int tiled_force = -1;   // token-tiled shape forced for every GEMM it fits (tests)
  bool attn_xcd = true;   // attention workgroups of one sequence grouped on one XCD (8+ sequences)
  float* rope_cs = nullptr;
  void *kcache = nullptr, *vcache = nullptr;
  size_t slot_elems = 0;     // elements of one slot's packed K (and V) cache
  std::vector<int> slot_ready;
  int* verify_slots = nullptr;
  // verify inputs / outputs
  float *draft = nullptr, *vnoise = nullptr, *taus = nullptr, *temb_tau = nullptr, *phi = nullptr, *hid = nullptr,
        *dist = nullptr, *params = nullptr;
  int *accept = nullptr, *gswitch = nullptr;
  float* vpart = nullptr;       // [out tiles][Mp_max] the verification's squared endpoint errors per 16-dim tile
  unsigned* vcount = nullptr;   // its arrival ticket (zero between launches)
  bool verify_head = false;     // set while a verification pass is enqueued: the head forms its distances
  std::map<int, float*> temb_steps;  // steps -> [steps][width]
  // time-modulated expert (time_mode 1) and QK-norm
  std::vector<void*> w_mod;          // [6w][w] row-major per layer (weight dtype)
  std::vector<float*> b_mod;         // [6w]
  void* final_mod_w = nullptr;       // [2w][w]
  float* final_mod_b = nullptr;      // [2w]
  std::vector<float*> qk_gain;       // QK-norm gains per packed q/k channel, per layer
  float* qk_ssp = nullptr;           // [q and k tiles][Mp] per-tile sums of squares of q and k
  float* zero_w = nullptr;           // [w] zeros: the additive temb of a modulated expert
  // draft model: the queries staged as block input rows, image features and their staging, RoPE of 0..P-1
  float *q_h0 = nullptr, *q_ssp0 = nullptr, *feat = nullptr, *feat_ssp = nullptr, *rope_feat = nullptr;
  void *q_hb0 = nullptr, *feat_hb = nullptr;
  // prefill stack: every layer's K and V in the cache blocks' layout, [L][n_kv][nbs][32 keys x dh]
  void *pf_k = nullptr, *pf_v = nullptr;
  size_t pf_layer_elems = 0;
  struct ModTable {
    float* mod = nullptr;                   // [L][steps][6w]: scale1 shift1 gate1 scale2 shift2 gate2
    float *g1 = nullptr, *g2 = nullptr;     // [L][steps][w]: ln1 (1 + scale1), ln2 (1 + scale2)
    float *bqkv = nullptr, *bgu = nullptr;  // [L][steps][tiles * 16], packed order: W . shift
    float *fmod = nullptr, *gf = nullptr, *bout = nullptr;  // [steps][2w], [steps][w], [steps][out tiles * 16]
  };
  std::map<int, ModTable> mod_steps;
  ModTable mod_tau;  // time-modulated expert with max_taus > 0: the verification times' vectors, filled per pass
  GemvJob* mt_gemv = nullptr;          // and the job tables that fill it: L + 1 linear maps of temb,
  GainJob* mt_gain = nullptr;          // 2 L + 1 modulated gains,
  PackedGemvJob* mt_shift = nullptr;   // 2 L + 1 shift biases
  int mt_max_n = 0, mt_max_tiles = 0;
  std::map<std::tuple<int, int, int>, hipGraphExec_t> graphs;
  float last_ms = 0.f;
  hipEvent_t ev0 = nullptr, ev1 = nullptr, ev_round = nullptr;
  // inputs of the last call per mode, for ae_kernel_times
  int last_verify_slot = 0;
  float last_delta = 0.f;
};

namespace {

int fail(ae_handle* h, int code, const std::string& msg) {
  if (h) h->err = msg;
  else g_create_error = msg;
  return code;
}

#define HIP_TRY(h, expr)                                                                  \
  do {                                                                                    \
    hipError_t e_ = (expr);                                                               \
    if (e_ != hipSuccess) {                                                               \
      return fail(h, e_ == hipErrorOutOfMemory ? AE_ERR_OOM : AE_ERR_HIP,                 \
                  std::string(#expr) + ": " + hipGetErrorString(e_));                     \
    }                                                                                     \
  } while (0)

int dalloc(ae_handle* h, void** p, size_t bytes) {
  if (bytes == 0) bytes = 16;
  hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess) return fail(h, AE_ERR_OOM, "hipMalloc(" + std::to_string(bytes) + "): " + hipGetErrorString(e));
  h->allocs.push_back(*p);
  e = hipMemset(*p, 0, bytes);
  if (e != hipSuccess) return fail(h, AE_ERR_HIP, std::string("hipMemset: ") + hipGetErrorString(e));
  return AE_OK;
}

template <class T>
int dalloc_t(ae_handle* h, T** p, size_t count) {
  return dalloc(h, (void**)p, count * sizeof(T));
}

// The split partial buffers hold EXCH_EMPTY in every word between launches (all bytes 0xff);
// the GEMM arrival tickets hold zero. Synchronous.
int reset_exchange(ae_handle* h) {
  HIP_TRY(h, hipDeviceSynchronize());
  if (h->part) HIP_TRY(h, hipMemset(h->part, 0xff, h->part_floats * sizeof(float)));
  for (int r = 0; r < 2; ++r)
    if (h->ring[r]) HIP_TRY(h, hipMemset(h->ring[r], 0xff, (size_t)(h->c.n_layers + 1) * h->layer_bytes));
  if (h->fpart_o) HIP_TRY(h, hipMemset(h->fpart_o, 0xff, h->fpart_o_floats * sizeof(float)));
  if (h->fpart_ml) HIP_TRY(h, hipMemset(h->fpart_ml, 0xff, h->fpart_ml_floats * sizeof(float)));
  if (h->abort_dev) HIP_TRY(h, hipMemset(h->abort_dev, 0, sizeof(unsigned)));
  if (h->opart) HIP_TRY(h, hipMemset(h->opart, 0xff, h->opart_floats * sizeof(float)));
  if (h->mlpart) HIP_TRY(h, hipMemset(h->mlpart, 0xff, h->mlpart_floats * sizeof(float)));
  if (h->counters) HIP_TRY(h, hipMemset(h->counters, 0, h->n_counters * sizeof(unsigned)));
  HIP_TRY(h, hipDeviceSynchronize());
  if (h->flag_host) __atomic_store_n(h->flag_host, 0u, __ATOMIC_RELEASE);
  return AE_OK;
}

int upload(ae_handle* h, void** dst, const void* src, size_t bytes) {
  int rc = dalloc(h, dst, bytes);
  if (rc) return rc;
  HIP_TRY(h, hipMemcpy(*dst, src, bytes, hipMemcpyHostToDevice));
  return AE_OK;
}

// Pack rows (row_ptr[p] = source row of packed channel p, or null for a zero row)
// of K elements of size es into [tiles][K/32][64 lanes][8].
using ae_host::pack_rows;

// ae_create's checks of the config and the weight pointers (ae_host::validate_config), as an AE_* code
// with the reason for ae_last_error.
int validate(const ae_config* c, const ae_weights* w) {
  std::string why;
  const int rc = ae_host::validate_config(c, w, why);
  return rc ? fail(nullptr, rc, why) : AE_OK;
}

PhaseCfg pick(int KB, int want, int n_z) {
  int S = n_z == 1 ? std::min(std::max(want, 1), 4) : 1;  // the split-K reduction sums at most 4 partials
  while (S > 1 && (KB % S || (KB / S) % GW)) --S;
  return {S};
}

template <int WT, int AT, int ROLE, int KPW>
hipError_t launch_gemm_k(GemmArgs a, int n_groups, int n_z, hipStream_t st) {
  if (!a.pf.dummy) a.pf.dummy = (const char*)a.w;  // unused prefetch slots reread the kernel's own weights
  constexpr size_t lds = gemm_lds_size<AT, RoleTraits<ROLE>::NT, KPW>();
  const dim3 grid(n_groups, a.S, (a.n_zt + a.zpw - 1) / a.zpw);
  if (a.zpw > 1) AE_LAUNCH((gemm_entry<ROLE, WT, AT, KPW, true>()), grid, dim3(GTHREADS), lds, st, a);
  else AE_LAUNCH((gemm_entry<ROLE, WT, AT, KPW, false>()), grid, dim3(GTHREADS), lds, st, a);
  return hipGetLastError();
}

// Pick k-blocks per wave per pass (largest of 4, 2, 1 dividing the split) and launch.
template <int WT, int AT, int ROLE>
hipError_t launch_gemm(GemmArgs a, int n_groups, int n_z, hipStream_t st) {
  const int kb_split = a.K / KBLK / a.S;
  if constexpr (AT == AT_BF16) {  // fp32 staging of 4 k-blocks per wave would not fit in LDS
    if (kb_split % (GW * 4) == 0) { a.passes = kb_split / (GW * 4); return launch_gemm_k<WT, AT, ROLE, 4>(a, n_groups, n_z, st); }
  }
  if (kb_split % (GW * 2) == 0) { a.passes = kb_split / (GW * 2); return launch_gemm_k<WT, AT, ROLE, 2>(a, n_groups, n_z, st); }
  a.passes = kb_split / GW;
  return launch_gemm_k<WT, AT, ROLE, 1>(a, n_groups, n_z, st);
}

template <int WT, int AT, int ROLE, int KPW>
hipError_t set_gemm_attr_k() {
  const int lds = (int)gemm_lds_size<AT, RoleTraits<ROLE>::NT, KPW>();
  hipError_t e = hipFuncSetAttribute((const void*)gemm_entry<ROLE, WT, AT, KPW, false>(),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute((const void*)gemm_entry<ROLE, WT, AT, KPW, true>(), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
}
template <int WT, int AT, int ROLE>
hipError_t set_gemm_attr() {
  hipError_t e = hipSuccess;
  if constexpr (AT == AT_BF16) e = set_gemm_attr_k<WT, AT, ROLE, 4>();
  if (e == hipSuccess) e = set_gemm_attr_k<WT, AT, ROLE, 2>();
  if (e == hipSuccess) e = set_gemm_attr_k<WT, AT, ROLE, 1>();
  return e;
}
// Token-tiled GEMM shapes (WN, WM, WK): output tile 64 WN channels x 64 WM tokens, WK k-groups.
constexpr int N_TILED = 4;
template <int SH> struct TiledShape;
template <> struct TiledShape<0> { typedef TileCfg<4, 2, 1> C; };
template <> struct TiledShape<1> { typedef TileCfg<2, 2, 2> C; };
template <> struct TiledShape<2> { typedef TileCfg<2, 1, 4> C; };
template <> struct TiledShape<3> { typedef TileCfg<1, 1, 8> C; };
constexpr int tiled_nt(int sh) { return sh == 0 ? 16 : sh == 3 ? 4 : 8; }  // 16-channel tiles
constexpr int tiled_mt(int sh) { return sh == 0 || sh == 1 ? 8 : 4; }      // 16-token tiles
constexpr int tiled_ck(int sh) {
  return sh == 0 ? TiledShape<0>::C::CK : sh == 1 ? TiledShape<1>::C::CK : sh == 2 ? TiledShape<2>::C::CK : TiledShape<3>::C::CK;
}
static_assert(tiled_nt(0) == TiledShape<0>::C::NT && tiled_mt(0) == TiledShape<0>::C::MT, "shape 0");
static_assert(tiled_nt(1) == TiledShape<1>::C::NT && tiled_mt(1) == TiledShape<1>::C::MT, "shape 1");
static_assert(tiled_nt(2) == TiledShape<2>::C::NT && tiled_mt(2) == TiledShape<2>::C::MT, "shape 2");
static_assert(tiled_nt(3) == TiledShape<3>::C::NT && tiled_mt(3) == TiledShape<3>::C::MT, "shape 3");

template <int EPI, int WT, int WN, int WM, int WK>
hipError_t launch_tiled_k(const GemmArgs& a, hipStream_t st, bool set_attr) {
  typedef TileCfg<WN, WM, WK> C;
  if (set_attr)
    return hipFuncSetAttribute((const void*)gemm_tiled_kernel<EPI, WN, WM, WK, WT>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS);
  AE_LAUNCH((gemm_tiled_kernel<EPI, WN, WM, WK, WT>), dim3(a.tn_blocks * a.tm_blocks), dim3(GTHREADS), C::LDS, st, a);
  return hipGetLastError();
}
template <int EPI, int WT = WT_BF16>
hipError_t launch_tiled(int shape, const GemmArgs& a, hipStream_t st, bool set_attr) {
  switch (shape) {
    case 0: return launch_tiled_k<EPI, WT, 4, 2, 1>(a, st, set_attr);
    case 1: return launch_tiled_k<EPI, WT, 2, 2, 2>(a, st, set_attr);
    case 2: return launch_tiled_k<EPI, WT, 2, 1, 4>(a, st, set_attr);
    default: return launch_tiled_k<EPI, WT, 1, 1, 8>(a, st, set_attr);
  }
}
hipError_t set_tiled_attrs() {
  hipError_t e = hipSuccess;
  for (int sh = 0; sh < N_TILED && e == hipSuccess; ++sh) {
    GemmArgs a{};
    e = launch_tiled<EPI_QKV>(sh, a, nullptr, true);
    if (e == hipSuccess) e = launch_tiled<EPI_RESID>(sh, a, nullptr, true);
    if (e == hipSuccess) e = launch_tiled<EPI_GEGLU>(sh, a, nullptr, true);
    if (e == hipSuccess) e = launch_tiled<EPI_RESID, WT_FP8>(sh, a, nullptr, true);
    if (e == hipSuccess) e = launch_tiled<EPI_GEGLU, WT_FP8>(sh, a, nullptr, true);
  }
  return e;
}

hipError_t set_all_gemm_attrs() {
  hipError_t e = hipSuccess;
  auto acc = [&](hipError_t r) { if (e == hipSuccess) e = r; };
  acc(set_gemm_attr<WT_F32, AT_F32, R_QKV_ROPE>()); acc(set_gemm_attr<WT_F32, AT_F32, R_O_PROJ>());
  acc(set_gemm_attr<WT_F32, AT_F32, R_GATE_UP>()); acc(set_gemm_attr<WT_F32, AT_F32, R_DOWN>());
  acc(set_gemm_attr<WT_F32, AT_F32, R_OUT_PROJ>());
  acc(set_gemm_attr<WT_BF16, AT_BF16, R_QKV_ROPE>()); acc(set_gemm_attr<WT_BF16, AT_BF16, R_O_PROJ>());
  acc(set_gemm_attr<WT_BF16, AT_BF16, R_GATE_UP>()); acc(set_gemm_attr<WT_BF16, AT_BF16, R_DOWN>());
  acc(set_gemm_attr<WT_BF16, AT_BF16, R_OUT_PROJ>());
  acc(set_gemm_attr<WT_FP8, AT_BF16, R_GATE_UP>()); acc(set_gemm_attr<WT_FP8, AT_BF16, R_DOWN>());
  acc(set_tiled_attrs());
  return e;
}

// Workgroups of fn (threads each, lds bytes of dynamic LDS) one compute unit holds at once, from the
// runtime's occupancy calculator (registers, LDS, waves); 0 when the query fails.
int blocks_per_cu(const void* fn, int threads, size_t lds) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, threads, lds) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return nb;
}
// The kernels that may wait inside a launch for other workgroups of it assume every workgroup is
// resident at once, one per compute unit (the runtime sizes their grids to at most the CU count):
// the smallest occupancy among the split attention kernels of this head size ...
template <int AT, int IT, bool QKN>
int attn_split_occ_k(int dh) {
  constexpr int NW = ATT_WAVES_SPLIT;
  switch (dh) {
    case 32: return blocks_per_cu((const void*)attn_kernel<AT, 32, IT, NW, QKN>, NW * 64, attn_lds_size<32, NW, QKN>());
    case 64: return blocks_per_cu((const void*)attn_kernel<AT, 64, IT, NW, QKN>, NW * 64, attn_lds_size<64, NW, QKN>());
    case 128: return blocks_per_cu((const void*)attn_kernel<AT, 128, IT, NW, QKN>, NW * 64, attn_lds_size<128, NW, QKN>());
    default: return blocks_per_cu((const void*)attn_kernel<AT, 256, IT, NW, QKN>, NW * 64, attn_lds_size<256, NW, QKN>());
  }
}
template <int AT, bool QKN>
int attn_split_occ(int dh) { return std::min(attn_split_occ_k<AT, ATT_IT_SPLIT, QKN>(dh), attn_split_occ_k<AT, ATT_IT_MID, QKN>(dh)); }
// ... and among the one-group GEMM kernels of a role (their split-K partials are polled in-kernel)
template <int WT, int AT, int ROLE, int KPW>
int gemm_occ_k() {
  return blocks_per_cu((const void*)gemm_entry<ROLE, WT, AT, KPW, false>(), GTHREADS, gemm_lds_size<AT, RoleTraits<ROLE>::NT, KPW>());
}
template <int WT, int AT, int ROLE>
int gemm_occ() {
  int nb = std::min(gemm_occ_k<WT, AT, ROLE, 2>(), gemm_occ_k<WT, AT, ROLE, 1>());
  if constexpr (AT == AT_BF16) nb = std::min(nb, gemm_occ_k<WT, AT, ROLE, 4>());
  return nb;
}

// k-splits per GEMM phase (qkv, o, gate/up, down, out) for one token group (measured for Pi0:
// o_proj and down gain from 4 splits, the others from none)

// Key splits when each of nw waves walks `it` blocks of ATT_KB keys.
int attn_splits(int n_blocks, int it, int nw) { return std::max(1, (n_blocks + it * nw - 1) / (it * nw)); }

// Attention kernels are instantiated per (activation type, head_dim, blocks per wave, waves).
template <int AT, int IT, int NW, bool QKN>
hipError_t attn_dispatch_qkn(int dh, bool set_attr, dim3 grid, hipStream_t st, const AttnArgs& aa) {
  const void* fn = nullptr;
  size_t lds = 0;
  switch (dh) {
    case 32: fn = (const void*)attn_kernel<AT, 32, IT, NW, QKN>; lds = attn_lds_size<32, NW, QKN>(); break;
    case 64: fn = (const void*)attn_kernel<AT, 64, IT, NW, QKN>; lds = attn_lds_size<64, NW, QKN>(); break;
    case 128: fn = (const void*)attn_kernel<AT, 128, IT, NW, QKN>; lds = attn_lds_size<128, NW, QKN>(); break;
    case 256: fn = (const void*)attn_kernel<AT, 256, IT, NW, QKN>; lds = attn_lds_size<256, NW, QKN>(); break;
    default: return hipErrorInvalidValue;
  }
  if (set_attr) return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  switch (dh) {
    case 32: AE_LAUNCH((attn_kernel<AT, 32, IT, NW, QKN>), grid, dim3(NW * 64), lds, st, aa); break;
    case 64: AE_LAUNCH((attn_kernel<AT, 64, IT, NW, QKN>), grid, dim3(NW * 64), lds, st, aa); break;
    case 128: AE_LAUNCH((attn_kernel<AT, 128, IT, NW, QKN>), grid, dim3(NW * 64), lds, st, aa); break;
    default: AE_LAUNCH((attn_kernel<AT, 256, IT, NW, QKN>), grid, dim3(NW * 64), lds, st, aa); break;
  }
  return hipGetLastError();
}
// QK-norm scaling is a separate instantiation (bf16 only), so the plain kernel is untouched by it
template <int AT, int IT, int NW>
hipError_t attn_dispatch_it(int dh, bool set_attr, dim3 grid, hipStream_t st, const AttnArgs& aa) {
  if constexpr (AT == AT_BF16) {
    if (set_attr) {
      hipError_t e = attn_dispatch_qkn<AT, IT, NW, false>(dh, true, grid, st, aa);
      return e != hipSuccess ? e : attn_dispatch_qkn<AT, IT, NW, true>(dh, true, grid, st, aa);
    }
    if (aa.qk_ssp) return attn_dispatch_qkn<AT, IT, NW, true>(dh, false, grid, st, aa);
  }
  return attn_dispatch_qkn<AT, IT, NW, false>(dh, set_attr, grid, st, aa);
}
template <int AT>
hipError_t attn_dispatch(int dh, bool set_attr, int split_it, dim3 grid, hipStream_t st, const AttnArgs& aa) {
  if (set_attr) {
    hipError_t e = attn_dispatch_it<AT, ATT_IT_SPLIT, ATT_WAVES_SPLIT>(dh, true, grid, st, aa);
    if (e == hipSuccess) e = attn_dispatch_it<AT, ATT_IT_MID, ATT_WAVES_SPLIT>(dh, true, grid, st, aa);
    return e != hipSuccess ? e : attn_dispatch_it<AT, ATT_IT_WHOLE, ATT_WAVES_WHOLE>(dh, true, grid, st, aa);
  }
  if (split_it == ATT_IT_MID) return attn_dispatch_it<AT, ATT_IT_MID, ATT_WAVES_SPLIT>(dh, false, grid, st, aa);
  return split_it ? attn_dispatch_it<AT, ATT_IT_SPLIT, ATT_WAVES_SPLIT>(dh, false, grid, st, aa)
                  : attn_dispatch_it<AT, ATT_IT_WHOLE, ATT_WAVES_WHOLE>(dh, false, grid, st, aa);
}

// Two query tiles per workgroup (bf16, one split, no QK-norm): 4 waves per tile x up to 7 blocks each
// (896 keys; more blocks per wave spill registers at head_dim 256).
constexpr int ATT_IT_PAIR = 7;
template <int DH>
hipError_t attn_pair_k(bool set_attr, dim3 grid, hipStream_t st, const AttnArgs& aa) {
  constexpr size_t lds = attn_lds_size<DH, ATT_WAVES_WHOLE, false>();
  if (set_attr)
    return hipFuncSetAttribute((const void*)attn_kernel<AT_BF16, DH, ATT_IT_PAIR, ATT_WAVES_WHOLE, false, 2>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  AE_LAUNCH((attn_kernel<AT_BF16, DH, ATT_IT_PAIR, ATT_WAVES_WHOLE, false, 2>), grid, dim3(ATT_WAVES_WHOLE * 64), lds, st, aa);
  return hipGetLastError();
}
hipError_t attn_pair_dispatch(int dh, bool set_attr, dim3 grid, hipStream_t st, const AttnArgs& aa) {
  switch (dh) {
    case 32: return attn_pair_k<32>(set_attr, grid, st, aa);
    case 64: return attn_pair_k<64>(set_attr, grid, st, aa);
    case 128: return attn_pair_k<128>(set_attr, grid, st, aa);
    default: return attn_pair_k<256>(set_attr, grid, st, aa);
  }
}

template <int AT>
hipError_t attn_merge_dispatch(int dh, dim3 grid, hipStream_t st, const AttnArgs& aa) {
  switch (dh) {
    case 32: AE_LAUNCH((attn_merge<AT, 32>), grid, dim3(256), 0, st, aa); break;
    case 64: AE_LAUNCH((attn_merge<AT, 64>), grid, dim3(256), 0, st, aa); break;
    case 128: AE_LAUNCH((attn_merge<AT, 128>), grid, dim3(256), 0, st, aa); break;
    default: AE_LAUNCH((attn_merge<AT, 256>), grid, dim3(256), 0, st, aa); break;
  }
  return hipGetLastError();
}

// How the attention covers the keys: n_split workgroups per query tile and blocks per wave.
// Splits of 8 waves x one block merge in-kernel when every workgroup of the launch fits on
// the device at once (one per compute unit); otherwise 8 waves walk up to 4 blocks each and
// longer contexts fall back to attn_merge.
struct AttnPlan {
  int n_split, split_it, coresident;  // split_it: blocks per wave of a split plan (0: whole tile)
  int pair;                           // whole tile, two query tiles per workgroup
};
AttnPlan attn_plan(const ae_handle* h, int n_seq) {
  const int nb = h->nbp + h->nbs, zz = n_seq * h->c.n_kv_heads;
  const int ns = attn_splits(nb, ATT_IT_SPLIT, ATT_WAVES_SPLIT);
  const bool may_wait = h->coresident_attn && h->variant != 2;
  if (may_wait && ns >= 2 && ns <= 16 && ns * h->n_qt * zz <= h->n_cu) return {ns, ATT_IT_SPLIT, 1};
  // several sequences (verification): splits of 2 blocks per wave, if those fit on the device at once
  const int nm = attn_splits(nb, ATT_IT_MID, ATT_WAVES_SPLIT);
  if (may_wait && nm >= 2 && nm <= 16 && nm * h->n_qt * zz <= h->n_cu)
    return {nm, ATT_IT_MID, 1, 0};
  const int nw = attn_splits(nb, ATT_IT_WHOLE, ATT_WAVES_WHOLE);
  // many sequences (a launch of more than one round): two query tiles per workgroup share each K/V load
  const bool pair = nw == 1 && h->at == AT_BF16 && !h->c.qk_norm && nb <= ATT_IT_PAIR * ATT_WAVES_WHOLE / 2 &&
                    h->n_qt * zz > h->n_cu;
  return {nw, 0, 0, pair ? 1 : 0};
}

// Steps of ~0.2 us that a split-K consumer sleeps before its first poll, so that the poll
// finds the other splits' partials landed instead of costing a second round trip (measured
// for Pi0: 1 step saves 0.16 ms per chunk, 2-6 steps less).
constexpr int POLL_DELAY = 1;

// Token-tiled shape for a GEMM role over n_tiles 16-channel tiles, K inputs and M tokens, or
// -1 for the kernel above: one token group, fp32 operands, E4M3 weights outside the MLP roles,
// an RMS input wider than the tiled prologue reads, no shape dividing the tiles and k-blocks, or
// the role switched off
// (AE_TILED, a bit per role; AE_TILED_SHAPE forces one shape wherever it fits). Among the
// shapes that fit, the one with the least modelled time:
// rounds of workgroups over the compute units x (the larger of its MFMA clocks and its operand
// bytes at 64 B per clock per compute unit, + ~2 us per round). A shape whose launch would fill
// under half the compute units is not taken (measured: slower than the kernel above there).
int tiled_shape(const ae_handle* h, int role, int n_tiles, int K, int M, int Mp, int* tn_blocks, int* tm_blocks) {
  if (role == R_OUT_PROJ || !((h->tiled_roles >> role) & 1) || Mp / TOKG < 2 || h->n_cu <= 0) return -1;
  const int wt = (role == R_GATE_UP || role == R_DOWN) ? h->mt : h->wt;
  if (h->at != AT_BF16 || (wt != WT_BF16 && !(wt == WT_FP8 && (role == R_GATE_UP || role == R_DOWN)))) return -1;
  if ((role == R_QKV_ROPE || role == R_GATE_UP) && h->c.width / 16 > TILED_MAX_GIN) return -1;
  const int tok_tiles = (M + 15) / 16;
  int best = -1;
  double best_cost = 0;
  for (int sh = 0; sh < N_TILED; ++sh) {
    if (h->tiled_force >= 0 && sh != h->tiled_force) continue;
    const int nt = tiled_nt(sh), mt = tiled_mt(sh);
    if (n_tiles % nt || (K / KBLK) % tiled_ck(sh)) continue;
    const int nb = n_tiles / nt, mb = (tok_tiles + mt - 1) / mt;
    if (h->tiled_force < 0 && 2 * nb * mb < h->n_cu) continue;  // under half the compute units: the kernel above wins
    const double mfma = (double)nt * 16 * mt * 16 * K * 2 / 4096, bytes = (double)(nt + mt) * 16 * K * 2 / 64;
    const double cost = (double)((nb * mb + h->n_cu - 1) / h->n_cu) * (std::max(mfma, bytes) + 5000);
    if (best < 0 || cost < best_cost) { best = sh; best_cost = cost; *tn_blocks = nb; *tm_blocks = mb; }
  }
  return best;
}
bool uses_tiled(const ae_handle* h, int role, int n_tiles, int K, int M, int Mp) {
  int tn, tm;
  return tiled_shape(h, role, n_tiles, K, M, Mp, &tn, &tm) >= 0;
}

struct Dispatch {
  // one launcher per role bound to the handle's dtypes (fp8 weights: MLP roles only)
  static hipError_t gemm(ae_handle* h, int role, GemmArgs a, int n_groups, int n_z, hipStream_t st) {
    // token groups per workgroup: enough that the launch fits one round of compute units
    // (each workgroup then loads its weights once for all its groups); split-K: one group
    if (a.S == 1) {
      const int nt = role == R_GATE_UP ? 2 : 1;
      const int sh = tiled_shape(h, role, n_groups * nt, a.K, a.M, a.M_pad, &a.tn_blocks, &a.tm_blocks);
      if (sh >= 0) {
        const bool fp8 = (role == R_GATE_UP || role == R_DOWN) && h->mt == WT_FP8;
        switch (role) {
          case R_QKV_ROPE: return launch_tiled<EPI_QKV>(sh, a, st, false);
          case R_GATE_UP: return fp8 ? launch_tiled<EPI_GEGLU, WT_FP8>(sh, a, st, false)
                                     : launch_tiled<EPI_GEGLU>(sh, a, st, false);
          default: return fp8 && role == R_DOWN ? launch_tiled<EPI_RESID, WT_FP8>(sh, a, st, false)
                                                : launch_tiled<EPI_RESID>(sh, a, st, false);
        }
      }
    }
    a.n_zt = n_z;
    a.zpw = 1;
    if (a.S == 1 && n_z > 1 && h->n_cu > 0) {
      const int gz = std::max(1, std::min(n_z, h->n_cu / std::max(n_groups, 1)));
      a.zpw = (n_z + gz - 1) / gz;
    }
    // one workgroup per CU fits them all (and the pass may wait inside a kernel)
    a.exch_poll = h->poll_splitk && h->variant != 2 && (long long)n_groups * a.S * n_z <= h->n_cu;
    a.poll_delay = POLL_DELAY;
    a.err = h->flag_dev;
    a.wait = h->wait_ticks;
    if (h->at == AT_F32) {
      switch (role) {
        case R_QKV_ROPE: return launch_gemm<WT_F32, AT_F32, R_QKV_ROPE>(a, n_groups, n_z, st);
        case R_O_PROJ: return launch_gemm<WT_F32, AT_F32, R_O_PROJ>(a, n_groups, n_z, st);
        case R_GATE_UP: return launch_gemm<WT_F32, AT_F32, R_GATE_UP>(a, n_groups, n_z, st);
        case R_DOWN: return launch_gemm<WT_F32, AT_F32, R_DOWN>(a, n_groups, n_z, st);
        default: return launch_gemm<WT_F32, AT_F32, R_OUT_PROJ>(a, n_groups, n_z, st);
      }
    }
    if (h->mt == WT_FP8 && role == R_GATE_UP) return launch_gemm<WT_FP8, AT_BF16, R_GATE_UP>(a, n_groups, n_z, st);
    if (h->mt == WT_FP8 && role == R_DOWN) return launch_gemm<WT_FP8, AT_BF16, R_DOWN>(a, n_groups, n_z, st);
    switch (role) {
      case R_QKV_ROPE: return launch_gemm<WT_BF16, AT_BF16, R_QKV_ROPE>(a, n_groups, n_z, st);
      case R_O_PROJ: return launch_gemm<WT_BF16, AT_BF16, R_O_PROJ>(a, n_groups, n_z, st);
      case R_GATE_UP: return launch_gemm<WT_BF16, AT_BF16, R_GATE_UP>(a, n_groups, n_z, st);
      case R_DOWN: return launch_gemm<WT_BF16, AT_BF16, R_DOWN>(a, n_groups, n_z, st);
      default: return launch_gemm<WT_BF16, AT_BF16, R_OUT_PROJ>(a, n_groups, n_z, st);
    }
  }
};

#define LAUNCH_CHECK(h, name, expr)                                                          \
  do {                                                                                       \
    if (!tm || tm->take(name)) {                                                             \
      expr;                                                                                  \
      hipError_t e_ = hipGetLastError();                                                     \
      if (e_ != hipSuccess) return fail(h, AE_ERR_HIP, std::string(name) + ": " + hipGetErrorString(e_)); \
      t_dispatch_ev = DispatchEvents{};                                                      \
    }                                                                                        \
  } while (0)

// Which kernels place the next kernel's operands in L2 (bit 0: QKV -> the attention's prefix
// K/V, bit 1: gate/up -> down weights, bit 3: o_proj's split-K producers -> gate/up weights,
// bit 4: down's split-K producers -> the next layer's QKV weights). Measured for Pi0 per chunk:
// bit 0 saves 0.32 ms, bit 4 0.19 ms, bit 3 (half of each k-range) 0.1 ms, bit 1 0.04 ms (it
// moves ~1.3 us per layer from down to gate/up). The attention placing o_proj's weights
// costs it ~1 us per launch (its exchange shares the memory path) and is not offered.
constexpr int PREFETCH_MASK = 1 | 2 | 8 | 16;

// Leading k-blocks of each gate/up tile that o_proj's producers place in L2 (bit 3): half the
// k-range, so that the prefetch ends within o_proj's own tail (measured for Pi0: all of it
// lengthens o_proj as much as it shortens gate/up; 12-16 of 32 blocks gain 0.1 ms per chunk).
int prefetch_gu_lead(int kb) { return kb / 2; }

// Leading k-blocks of each down tile that gate/up places in L2 (bit 1; 0 = all of them).
constexpr int PREFETCH_DOWN_LEAD = 0;

// One velocity pass over M = n_seq * H rows in h->x (temb per sequence from
// temb[seq * temb_stride]); dt > 0 updates x in place, dt == 0 writes h->vout.
// Step k of a `steps`-step denoise of a time-modulated expert: where its modulation vectors live
// (per_seq: a verification pass, sequence j of the pass takes row j of the table; k = 0)
struct StepMod {
  const ae_handle::ModTable* t;
  int k, steps;
  bool per_seq = false;
};

int enqueue_velocity(ae_handle* h, int n_seq, const float* temb, int temb_stride, const int* seq_slot, int slot0, float dt,
                     hipStream_t st, Timer* tm, const StepMod* sm = nullptr, bool from_h = false, bool head = true) {
  const ae_config& c = h->c;
  const int H = c.horizon, A = c.action_dim, w = c.width, F = c.mlp_dim;
  const int nq = c.n_q_heads, nkv = c.n_kv_heads, dh = c.head_dim;
  const int M = n_seq * H, Mp = (M + TOKG - 1) / TOKG * TOKG, n_z = Mp / TOKG;
  const size_t nqkv = (size_t)h->qkv_tiles * 16, ngu = (size_t)h->gu_tiles * 16, nout = (size_t)h->out_tiles * 16;
  // per-(layer, step) vector of a modulation table
  auto modp = [&](const float* base, size_t per, int l) { return base + ((size_t)l * sm->steps + sm->k) * per; };
  const float* temb_in = sm ? h->zero_w : temb;  // a modulated expert adds no temb to the tokens
  const int temb_in_stride = sm ? 0 : temb_stride;
  const float* g_first = sm ? modp(sm->t->g1, w, 0) : h->ln1[0];
  const bool mseq = sm && sm->per_seq;  // each sequence its own modulation vectors, one table row apart

  // from_h: the block input rows are already in h / hb / ssp_a (the draft model's queries)
  if (!from_h) LAUNCH_CHECK(h, "in_proj", {
    if (h->at == AT_F32)
      AE_LAUNCH((in_proj_kernel<WT_F32, AT_F32>), dim3(w / 64, Mp / 16), dim3(256), 0, st, h->x, h->action_in_w,
                         h->action_in_b, temb_in, temb_in_stride, M, Mp, A, H, w, h->h, h->hb, g_first, mseq ? (size_t)w : 0, h->ssp_a);
    else
      AE_LAUNCH((in_proj_kernel<WT_BF16, AT_BF16>), dim3(w / 64, Mp / 16), dim3(256), 0, st, h->x, h->action_in_w,
                         h->action_in_b, temb_in, temb_in_stride, M, Mp, A, H, w, h->h, h->hb, g_first, mseq ? (size_t)w : 0, h->ssp_a);
  });

  const int gq = nq / nkv, R = gq * H;
  AttnArgs aa{};
  aa.q = h->q; aa.ks = h->ks; aa.vs = h->vs; aa.kcache = h->kcache; aa.vcache = h->vcache;
  aa.seq_slot = seq_slot;
  aa.slot0 = slot0;
  aa.slot_stride = h->slot_elems;
  aa.P = c.prefix_len; aa.H = H; aa.n_q = nq; aa.n_kv = nkv; aa.dh = dh;
  aa.nbp = h->nbp; aa.nbs = h->nbs; aa.ntt = Mp / 16;
  aa.n_qt = h->n_qt;
  const AttnPlan plan = attn_plan(h, n_seq);
  aa.n_split = plan.n_split;
  aa.coresident = plan.coresident;
  aa.xcd_group = n_seq * nkv >= 8 && !plan.coresident && h->attn_xcd;
  aa.touch = n_seq >= 2;  // several sequences: each touches its prefix K/V into L2 first
  aa.err = h->flag_dev;
  aa.wait = h->wait_ticks;
  aa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)dh));
  aa.opart = h->opart; aa.mlpart = h->mlpart; aa.o = h->o;
  if (c.qk_norm) {
    aa.qk_ssp = h->qk_ssp; aa.qk_mpad = Mp;
    aa.qk_inv_dh = 1.f / (float)dh; aa.qk_eps = c.rms_eps;
  }

  for (int l = 0; l < c.n_layers; ++l) {
    GemmArgs g{};
    g.inv_width = 1.f / (float)w; g.eps = c.rms_eps; g.M = M; g.M_pad = Mp;
    g.part = h->part; g.counters = h->counters;
    if (mseq) {  // gains, gates and shift biases of row r from sequence r / H's table row
      g.mod_rows = H; g.ms_gain = w; g.ms_gate = 6 * (size_t)w;
    }
    // --- norm1 + QKV + RoPE
    {
      GemmArgs a = g;
      a.w = h->qkv_p[l]; a.x = h->hb;
      a.ssp_in = h->ssp_a; a.g_in = w / 16; a.K = w;
      a.S = pick(w / 32, h->sk.qkv, n_z).S;
      if ((PREFETCH_MASK & 1) && n_seq == 1 && !seq_slot && h->slot_elems) {  // this layer's prefix K/V (one robot)
        const size_t kes = dtype_size(c.kv_dtype), lay = (size_t)nkv * h->nbp * ATT_KB * dh;
        const size_t off = ((size_t)slot0 * h->slot_elems + (size_t)l * lay) * kes;
        a.pf.kind = 1; a.pf.bytes = lay * kes;
        a.pf.base = (const char*)h->kcache + off; a.pf.base2 = (const char*)h->vcache + off;
      }
      a.q_out = h->q; a.k_out = h->ks; a.v_out = h->vs; a.n_qt = h->n_qt; a.nbs = h->nbs; a.rope_cs = h->rope_cs;
      if (c.prefill) {  // this layer's K and V are written straight into the stack's output cache
        const size_t off = l * h->pf_layer_elems * dtype_size(c.kv_dtype);
        a.k_out = (char*)h->pf_k + off; a.v_out = (char*)h->pf_v + off;
        aa.ks = a.k_out; aa.vs = a.v_out;
      }
      a.n_q = nq; a.n_kv = nkv; a.dh = dh; a.H = H;
      if (sm) a.shift_bias = modp(sm->t->bqkv, nqkv, l);
      a.ms_shift = nqkv;
      if (c.qk_norm) { a.qk_gain = h->qk_gain[l]; a.qk_ssp = h->qk_ssp; }
      LAUNCH_CHECK(h, "qkv_rope", (void)Dispatch::gemm(h, R_QKV_ROPE, a, h->qkv_tiles, n_z, st));
    }
    // --- attention over [prefix ; suffix]
    aa.layer_off = (size_t)l * nkv * h->nbp * ATT_KB * dh;
    const dim3 attn_grid(aa.n_split, plan.pair ? (aa.n_qt + 1) / 2 : aa.n_qt, n_seq * nkv);
    LAUNCH_CHECK(h, "attn", {
      if (plan.pair) (void)attn_pair_dispatch(dh, false, attn_grid, st, aa);
      else if (h->at == AT_BF16) (void)attn_dispatch<AT_BF16>(dh, false, plan.split_it, attn_grid, st, aa);
      else (void)attn_dispatch<AT_F32>(dh, false, plan.split_it, attn_grid, st, aa);
    });
    if (aa.n_split > 1 && !aa.coresident) {
      LAUNCH_CHECK(h, "attn_merge", {
        if (h->at == AT_BF16) (void)attn_merge_dispatch<AT_BF16>(dh, dim3(aa.n_qt, n_seq * nkv), st, aa);
        else (void)attn_merge_dispatch<AT_F32>(dh, dim3(aa.n_qt, n_seq * nkv), st, aa);
      });
    }
    // --- o_proj + residual; hb <- h * ln2
    {
      GemmArgs a = g;
      a.w = h->o_p[l]; a.x = h->o; a.ssp_in = nullptr; a.K = nq * dh;
      a.S = pick(nq * dh / 32, h->sk.o, n_z).S;
      a.h = h->h; a.hb = h->hb; a.gain_next = sm ? modp(sm->t->g2, w, l) : h->ln2[l]; a.ssp_out = h->ssp_b; a.N = w;
      if (sm) a.res_gate = modp(sm->t->mod, 6 * (size_t)w, l) + 2 * w;
      if ((PREFETCH_MASK & 8) && !uses_tiled(h, R_GATE_UP, h->gu_tiles, w, M, Mp)) {  // gate/up's weights, tiled as gate/up is launched below
        a.pf.kind = 2; a.pf.base = (const char*)h->gu_p[l];
        a.pf.next_groups = h->gu_tiles / 2; a.pf.next_S = pick(w / 32, h->sk.gu, n_z).S; a.pf.NT = 2; a.pf.KB = w / KBLK;
        a.pf.frag_bytes = h->mt == WT_F32 ? 2048 : h->mt == WT_BF16 ? 1024 : 512;
        a.pf.kb_lead = prefetch_gu_lead(w / KBLK / a.pf.next_S);
      }
      LAUNCH_CHECK(h, "o_proj_resid", (void)Dispatch::gemm(h, R_O_PROJ, a, w / 16, n_z, st));
    }
    // --- norm2 + gate/up + GeGLU
    {
      GemmArgs a = g;
      a.w = h->gu_p[l]; a.wscale = h->gu_s[l]; a.x = h->hb;
      a.ssp_in = h->ssp_b; a.g_in = w / 16; a.K = w;
      a.S = pick(w / 32, h->sk.gu, n_z).S; a.u_out = h->u; a.N = F;
      if (sm) a.shift_bias = modp(sm->t->bgu, ngu, l);
      a.ms_shift = ngu;
      if ((PREFETCH_MASK & 2) && !uses_tiled(h, R_DOWN, w / 16, F, M, Mp)) {  // down's weights, tiled as down is launched below
        a.pf.kind = 2; a.pf.base = (const char*)h->d_p[l];
        a.pf.next_groups = w / 16; a.pf.next_S = pick(F / 32, h->sk.down, n_z).S; a.pf.NT = 1; a.pf.KB = F / KBLK;
        a.pf.frag_bytes = h->mt == WT_F32 ? 2048 : h->mt == WT_BF16 ? 1024 : 512;
        a.pf.kb_lead = PREFETCH_DOWN_LEAD;
      }
      LAUNCH_CHECK(h, "gate_up_geglu", (void)Dispatch::gemm(h, R_GATE_UP, a, h->gu_tiles / 2, n_z, st));
    }
    // --- down + residual; hb <- h * next gain
    {
      GemmArgs a = g;
      a.w = h->d_p[l]; a.wscale = h->d_s[l]; a.x = h->u; a.ssp_in = nullptr; a.K = F;
      a.S = pick(F / 32, h->sk.down, n_z).S;
      a.h = h->h; a.hb = h->hb;
      a.gain_next = (l + 1 < c.n_layers) ? (sm ? modp(sm->t->g1, w, l + 1) : h->ln1[l + 1])
                                         : (sm ? sm->t->gf + (size_t)sm->k * w : h->final_ln ? h->final_ln : h->ln1[0]);
      if (sm) a.res_gate = modp(sm->t->mod, 6 * (size_t)w, l) + 5 * w;
      a.ssp_out = h->ssp_a; a.N = w;
      if ((PREFETCH_MASK & 16) && l + 1 < c.n_layers && !uses_tiled(h, R_QKV_ROPE, h->qkv_tiles, w, M, Mp)) {  // the next layer's QKV weights
        a.pf.kind = 2; a.pf.base = (const char*)h->qkv_p[l + 1];
        a.pf.next_groups = h->qkv_tiles; a.pf.next_S = pick(w / 32, h->sk.qkv, n_z).S; a.pf.NT = 1; a.pf.KB = w / KBLK;
        a.pf.frag_bytes = h->wt == WT_F32 ? 2048 : 1024;
      }
      LAUNCH_CHECK(h, "down_resid", (void)Dispatch::gemm(h, R_DOWN, a, w / 16, n_z, st));
    }
  }
  // --- final norm + action_out_proj (+ Euler update)
  if (head) {
    GemmArgs a{};
    a.inv_width = 1.f / (float)w; a.eps = c.rms_eps; a.M = M; a.M_pad = Mp;
    a.part = h->part; a.counters = h->counters;
    a.w = h->action_out_p; a.x = h->hb; a.ssp_in = h->ssp_a; a.g_in = w / 16; a.K = w;
    a.S = pick(w / 32, h->sk.out, n_z).S;
    a.bias = sm ? sm->t->bout + (size_t)sm->k * nout : h->action_out_b; a.A = A; a.dt = dt; a.xio = dt > 0.f ? h->x : h->vout;
    if (mseq) { a.mod_rows = H; a.ms_bias = nout; }
    if (h->verify_head) {  // the endpoints, distances and accepted length in the epilogue
      a.H = H; a.vx = h->x; a.draft = h->draft; a.taus = h->taus; a.vparams = h->params;
      a.vpart = h->vpart; a.vcount = h->vcount; a.v_epi = h->out_tiles * n_z; a.gripper_dim = c.gripper_dim;
      a.dist = h->dist; a.accept = h->accept; a.gswitch = h->gswitch;
    }
    LAUNCH_CHECK(h, "out_proj_euler", (void)Dispatch::gemm(h, R_OUT_PROJ, a, h->out_tiles, n_z, st));
  }
  return AE_OK;
}

// temb for n_t times in device array t_dev -> out [n_t][width].
// The time MLP over the n_t sinusoid rows in h->phi -> out [n_t][width].
int enqueue_time_mlp(ae_handle* h, int n_t, float* out, hipStream_t st, Timer* tm) {
  const int w = h->c.width;
  if (h->at == AT_F32) {
    LAUNCH_CHECK(h, "time_mlp_in", AE_LAUNCH(gemv_kernel<WT_F32>, dim3(w / 4), dim3(256), 0, st, h->time_in_w, h->time_in_b, h->phi, w, w, 1, h->hid, n_t));
    LAUNCH_CHECK(h, "time_mlp_out", AE_LAUNCH(gemv_kernel<WT_F32>, dim3(w / 4), dim3(256), 0, st, h->time_out_w, h->time_out_b, h->hid, w, w, 0, out, n_t));
  } else {
    LAUNCH_CHECK(h, "time_mlp_in", AE_LAUNCH(gemv_kernel<WT_BF16>, dim3(w / 4), dim3(256), 0, st, h->time_in_w, h->time_in_b, h->phi, w, w, 1, h->hid, n_t));
    LAUNCH_CHECK(h, "time_mlp_out", AE_LAUNCH(gemv_kernel<WT_BF16>, dim3(w / 4), dim3(256), 0, st, h->time_out_w, h->time_out_b, h->hid, w, w, 0, out, n_t));
  }
  return AE_OK;
}

int enqueue_temb(ae_handle* h, const float* t_dev, int n_t, float* out, hipStream_t st, Timer* tm) {
  const int w = h->c.width;
  LAUNCH_CHECK(h, "time_sinusoid", AE_LAUNCH(sinusoid_kernel, dim3(std::max(1, w / 2 / 256), n_t), dim3(256), 0, st, t_dev, w, h->phi));
  return enqueue_time_mlp(h, n_t, out, st, tm);
}

// The modulation vectors of every (layer, step) of a `steps`-step denoise of a time-modulated
// expert, built once per step count from the step times' temb: the linear maps of temb, the
// modulated norm gains, and the shift biases W . shift in the consumers' packed channel order.
int alloc_mod_table(ae_handle* h, int steps, ae_handle::ModTable& t) {
  const ae_config& c = h->c;
  const int w = c.width, L = c.n_layers;
  const size_t nqkv = (size_t)h->qkv_tiles * 16, ngu = (size_t)h->gu_tiles * 16, nout = (size_t)h->out_tiles * 16;
  int rc = dalloc_t(h, &t.mod, (size_t)L * steps * 6 * w);
  if (!rc) rc = dalloc_t(h, &t.g1, (size_t)L * steps * w);
  if (!rc) rc = dalloc_t(h, &t.g2, (size_t)L * steps * w);
  if (!rc) rc = dalloc_t(h, &t.bqkv, (size_t)L * steps * nqkv);
  if (!rc) rc = dalloc_t(h, &t.bgu, (size_t)L * steps * ngu);
  if (!rc) rc = dalloc_t(h, &t.fmod, (size_t)steps * 2 * w);
  if (!rc) rc = dalloc_t(h, &t.gf, (size_t)steps * w);
  if (!rc) rc = dalloc_t(h, &t.bout, (size_t)steps * nout);
  return rc;
}

// Fill rows 0 .. n - 1 of table t (laid out for `steps` rows per layer) from the n time embeddings
// temb [n][w]: no allocation and no synchronisation, so that a verification graph can hold it.
int enqueue_mod_table(ae_handle* h, const ae_handle::ModTable& t, int steps, int n, const float* temb, hipStream_t st,
                      Timer* tm) {
  const ae_config& c = h->c;
  const int w = c.width, L = c.n_layers;
  const size_t nqkv = (size_t)h->qkv_tiles * 16, ngu = (size_t)h->gu_tiles * 16, nout = (size_t)h->out_tiles * 16;
  const dim3 gw((w + 255) / 256, n);
  for (int l = 0; l < L; ++l) {
    float* m = t.mod + (size_t)l * steps * 6 * w;
    LAUNCH_CHECK(h, "mod_rows", AE_LAUNCH(gemv_kernel<WT_BF16>, dim3(6 * w / 4), dim3(256), 0, st, h->w_mod[l], h->b_mod[l],
                                         temb, w, 6 * w, 0, m, n));
    LAUNCH_CHECK(h, "mod_gain", AE_LAUNCH(mod_gain_kernel, gw, dim3(256), 0, st, h->ln1[l], m, 6 * w, w,
                                         t.g1 + (size_t)l * steps * w));
    LAUNCH_CHECK(h, "mod_gain", AE_LAUNCH(mod_gain_kernel, gw, dim3(256), 0, st, h->ln2[l], m + 3 * w, 6 * w, w,
                                         t.g2 + (size_t)l * steps * w));
    LAUNCH_CHECK(h, "mod_shift", AE_LAUNCH(packed_gemv_kernel, dim3(h->qkv_tiles, n), dim3(256), 0, st,
                                          (const uint16_t*)h->qkv_p[l], w / KBLK, m + w, 6 * w, nullptr, 0,
                                          t.bqkv + (size_t)l * steps * nqkv, (int)nqkv));
    LAUNCH_CHECK(h, "mod_shift", AE_LAUNCH(packed_gemv_kernel, dim3(h->gu_tiles, n), dim3(256), 0, st,
                                          (const uint16_t*)h->gu_p[l], w / KBLK, m + 4 * w, 6 * w, nullptr, 0,
                                          t.bgu + (size_t)l * steps * ngu, (int)ngu));
  }
  LAUNCH_CHECK(h, "mod_rows", AE_LAUNCH(gemv_kernel<WT_BF16>, dim3(2 * w / 4), dim3(256), 0, st, h->final_mod_w,
                                       h->final_mod_b, temb, w, 2 * w, 0, t.fmod, n));
  LAUNCH_CHECK(h, "mod_gain", AE_LAUNCH(mod_gain_kernel, gw, dim3(256), 0, st, h->final_ln, t.fmod, 2 * w, w, t.gf));
  LAUNCH_CHECK(h, "mod_shift", AE_LAUNCH(packed_gemv_kernel, dim3(h->out_tiles, n), dim3(256), 0, st,
                                        (const uint16_t*)h->action_out_p, w / KBLK, t.fmod + w, 2 * w, h->action_out_b,
                                        c.action_dim, t.bout, (int)nout));
  return AE_OK;
}

// The job tables of a verification pass's modulation vectors (mod_tau, from temb_tau), built once.
int setup_mod_tau_jobs(ae_handle* h) {
  const ae_config& c = h->c;
  const int w = c.width, L = c.n_layers, S = c.max_taus;
  const ae_handle::ModTable& t = h->mod_tau;
  const size_t nqkv = (size_t)h->qkv_tiles * 16, ngu = (size_t)h->gu_tiles * 16, nout = (size_t)h->out_tiles * 16;
  std::vector<GemvJob> gj;
  std::vector<GainJob> nj;
  std::vector<PackedGemvJob> pj;
  for (int l = 0; l < L; ++l) {
    float* m = t.mod + (size_t)l * S * 6 * w;
    gj.push_back({(const uint16_t*)h->w_mod[l], h->b_mod[l], h->temb_tau, m, w, 6 * w});
    nj.push_back({h->ln1[l], m, t.g1 + (size_t)l * S * w, 6 * w});
    nj.push_back({h->ln2[l], m + 3 * w, t.g2 + (size_t)l * S * w, 6 * w});
    pj.push_back({(const uint16_t*)h->qkv_p[l], m + w, nullptr, t.bqkv + (size_t)l * S * nqkv, w / KBLK, h->qkv_tiles,
                  6 * w, (int)nqkv, 0});
    pj.push_back({(const uint16_t*)h->gu_p[l], m + 4 * w, nullptr, t.bgu + (size_t)l * S * ngu, w / KBLK, h->gu_tiles,
                  6 * w, (int)ngu, 0});
  }
  gj.push_back({(const uint16_t*)h->final_mod_w, h->final_mod_b, h->temb_tau, t.fmod, w, 2 * w});
  nj.push_back({h->final_ln, t.fmod, t.gf, 2 * w});
  pj.push_back({(const uint16_t*)h->action_out_p, t.fmod + w, h->action_out_b, t.bout, w / KBLK, h->out_tiles, 2 * w,
                (int)nout, c.action_dim});
  h->mt_max_n = 6 * w;
  h->mt_max_tiles = std::max({h->qkv_tiles, h->gu_tiles, h->out_tiles});
  int rc = upload(h, (void**)&h->mt_gemv, gj.data(), gj.size() * sizeof(GemvJob));
  if (!rc) rc = upload(h, (void**)&h->mt_gain, nj.data(), nj.size() * sizeof(GainJob));
  if (!rc) rc = upload(h, (void**)&h->mt_shift, pj.data(), pj.size() * sizeof(PackedGemvJob));
  return rc;
}

// mod_tau rows 0 .. n - 1 from temb_tau: three launches over the job tables
int enqueue_mod_tau(ae_handle* h, int n, hipStream_t st, Timer* tm) {
  const int w = h->c.width, L = h->c.n_layers;
  LAUNCH_CHECK(h, "mod_rows", AE_LAUNCH(gemv_jobs_kernel, dim3(h->mt_max_n / 16, L + 1), dim3(256), 0, st, h->mt_gemv, n));
  LAUNCH_CHECK(h, "mod_gain", AE_LAUNCH(mod_gain_jobs_kernel, dim3((w + 255) / 256, n, 2 * L + 1), dim3(256), 0, st,
                                       h->mt_gain, w));
  LAUNCH_CHECK(h, "mod_shift", AE_LAUNCH(packed_gemv_jobs_kernel, dim3((h->mt_max_tiles + PGJ_TILES - 1) / PGJ_TILES, 2 * L + 1), dim3(256), 0, st,
                                        h->mt_shift, n));
  return AE_OK;
}

int build_mod_table(ae_handle* h, int steps, const float* temb) {
  ae_handle::ModTable t;
  int rc = alloc_mod_table(h, steps, t);
  if (!rc) rc = enqueue_mod_table(h, t, steps, steps, temb, h->stream, nullptr);
  if (rc) return rc;
  HIP_TRY(h, hipStreamSynchronize(h->stream));
  h->mod_steps[steps] = t;
  return AE_OK;
}

int get_temb_steps(ae_handle* h, int steps, float** out) {
  auto it = h->temb_steps.find(steps);
  if (it != h->temb_steps.end()) { *out = it->second; return AE_OK; }
  const int w = h->c.width;
  float* buf = nullptr;
  int rc = dalloc_t(h, &buf, (size_t)steps * w);
  if (rc) return rc;
  std::vector<float> ts(steps);
  for (int k = 0; k < steps; ++k) ts[k] = (float)((double)k / steps);
  // the sinusoid/hidden scratch holds max(steps, max_taus) rows
  float *tdev = nullptr, *phi = nullptr, *hid = nullptr;
  rc = dalloc_t(h, &tdev, steps); if (rc) return rc;
  rc = dalloc_t(h, &phi, (size_t)steps * w); if (rc) return rc;
  rc = dalloc_t(h, &hid, (size_t)steps * w); if (rc) return rc;
  HIP_TRY(h, hipMemcpy(tdev, ts.data(), steps * sizeof(float), hipMemcpyHostToDevice));
  float* save_phi = h->phi; float* save_hid = h->hid;
  h->phi = phi; h->hid = hid;
  rc = enqueue_temb(h, tdev, steps, buf, h->stream, nullptr);
  h->phi = save_phi; h->hid = save_hid;
  if (rc) return rc;
  HIP_TRY(h, hipStreamSynchronize(h->stream));
  h->temb_steps[steps] = buf;
  if (h->c.time_mode) {
    rc = build_mod_table(h, steps, buf);
    if (rc) return rc;
  }
  *out = buf;
  return AE_OK;
}

// The persistent step kernel of batch-1 denoise passes: the instantiation for the handle's shapes
// and dtypes, every workgroup of its grid resident at once (one per compute unit), the activation
// rings, the attention split partials and the per-layer table. fused_ok stays false, and the passes
// take one launch per phase, when any of it does not hold.
int setup_fused(ae_handle* h) {
  const ae_config& c = h->c;
  const int w = c.width, F = c.mlp_dim, nq = c.n_q_heads, nkv = c.n_kv_heads, dh = c.head_dim, H = c.horizon;
  const int L = c.n_layers;
  auto no = [&](const char* why) {
    h->fused_why = why;
    return AE_OK;
  };
  if (c.draft || c.prefill || c.weight_dtype != AE_BF16 || c.kv_dtype != AE_BF16 ||
      (c.mlp_dtype != AE_BF16 && c.mlp_dtype != AE_FP8_E4M3))
    return no("model variant or dtypes");
  if (H > 64 || c.prefix_len < 1 || h->n_cu < 32 || h->n_cu % 32) return no("horizon, prefix or compute-unit count");
  // instantiated shapes: head_dim 256, width 1024, n_q_heads * head_dim 2048, mlp_dim 4096
  const bool fp8 = c.mlp_dtype == AE_FP8_E4M3;
  if (dh == 256 && w == 1024 && nq * dh == 2048 && F == 4096) {
    h->fused_fn = fp8 ? fused_step_kernel<256, WT_FP8, 4, 8, 16> : fused_step_kernel<256, WT_BF16, 4, 8, 16>;
    h->fused_lds = fused_lds_bytes<256>();
  } else {
    return no("shapes without an instantiation");
  }
  const int ntt = (H + 15) / 16, ntp = ntt <= 1 ? 1 : ntt <= 2 ? 2 : 4, G = h->n_cu;
  const int nb = h->nbp + h->nbs;
  // key splits of 4 blocks (half the waves of a unit busy, half the K/V bytes per workgroup of 8-block
  // splits: measured for Pi0, 7 splits of 4 blocks take 0.685 ms per step, 4 splits of 7 blocks 0.694 ms),
  // as long as every unit still has a workgroup of its own
  h->f_nsplit = (nb + FW - 1) / FW;
  const int ns4 = (nb + 3) / 4;
  if (ns4 <= FW && ns4 * h->n_qt * nkv <= G) h->f_nsplit = std::max(h->f_nsplit, ns4);
  h->f_natt = h->f_nsplit * h->n_qt * nkv;
  if (w / 16 > F_SLOTS * (G / ntp) || h->f_natt > 4 * G || h->out_tiles > G / ntp || h->nbp < 1)
    return no("work split does not fit the grid");
  // a failed query leaves its error for the next hipGetLastError: read it back here
  const hipError_t ea = hipFuncSetAttribute((const void*)h->fused_fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                            (int)h->fused_lds);
  (void)hipGetLastError();
  if (ea != hipSuccess) return no("dynamic LDS attribute refused");
  // one workgroup per compute unit: its threads, registers (2 waves per SIMD: at most 256 VGPRs) and
  // LDS must fit one compute unit (the kernel's own attributes against the device's)
  hipFuncAttributes fat{};
  int lds_cu = 0;
  const hipError_t ef = hipFuncGetAttributes(&fat, (const void*)h->fused_fn);
  const hipError_t ed = hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, h->dev);
  (void)hipGetLastError();
  if (ef != hipSuccess || ed != hipSuccess) return no("kernel or device attribute query failed");
  if (fat.maxThreadsPerBlock < FT || fat.numRegs > 256 || fat.localSizeBytes > 0 ||
      fat.sharedSizeBytes + h->fused_lds > (size_t)lds_cu)
    return no("a workgroup does not fit a compute unit");
  h->occ_fused = blocks_per_cu((const void*)h->fused_fn, FT, h->fused_lds);
  if (h->occ_fused < 1) return no("the occupancy calculator puts no workgroup on a compute unit");
  // one block of the ring per layer (and one for the final norm's input), each buffer 256-byte aligned
  const size_t Mp = (size_t)ntt * 16;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return (unsigned)o;
  };
  take(Mp * w * 2);  // hb_in: the layer's input rows * ln1, fragment order
  h->off_ssp = take((size_t)(w / 16) * Mp * 4);
  h->off_q = take((size_t)nkv * h->n_qt * ATT_ROWS * dh * 2);
  h->off_k = take((size_t)nkv * h->nbs * ATT_KB * dh * 2);
  h->off_v = take((size_t)nkv * h->nbs * ATT_KB * dh * 2);
  h->off_o = take(Mp * nq * dh * 2);
  h->off_hb2 = take(Mp * w * 2);
  h->off_ssp2 = take((size_t)(w / 16) * Mp * 4);
  h->off_u = take(Mp * F * 2);
  if (c.qk_norm) h->off_qks = take((size_t)(nq + nkv) * (dh / 16) * Mp * 4);
  h->layer_bytes = (unsigned)off;
  for (int r = 0; r < 2; ++r) {
    const int rc = dalloc(h, (void**)&h->ring[r], (size_t)(L + 1) * off);
    if (rc) return rc;
  }
  // two sets of attention partials, used by alternating launches as the rings are
  h->fpart_o_floats = 2 * (size_t)L * h->f_natt * ATT_ROWS * dh;
  h->fpart_ml_floats = 2 * (size_t)L * h->f_natt * ATT_ROWS * 2;
  int rc = dalloc_t(h, &h->fpart_o, h->fpart_o_floats);
  if (!rc) rc = dalloc_t(h, &h->fpart_ml, h->fpart_ml_floats);
  if (!rc) rc = dalloc_t(h, &h->abort_dev, 1);
  if (rc) return rc;
  std::vector<FusedLayer> ly(L);
  const size_t lay = (size_t)nkv * h->nbp * ATT_KB * dh;  // elements of one layer of a slot's packed cache
  for (int l = 0; l < L; ++l) {
    ly[l].qkv = (const uint16_t*)h->qkv_p[l];
    ly[l].o = (const uint16_t*)h->o_p[l];
    ly[l].gu = h->gu_p[l];
    ly[l].d = h->d_p[l];
    ly[l].gu_s = h->gu_s[l];
    ly[l].d_s = h->d_s[l];
    ly[l].ln2 = h->ln2[l];
    ly[l].g_next = l + 1 < L ? h->ln1[l + 1] : h->final_ln;
    ly[l].kc = (const uint16_t*)h->kcache + (size_t)l * lay;
    ly[l].vc = (const uint16_t*)h->vcache + (size_t)l * lay;
    ly[l].qk_gain = c.qk_norm ? h->qk_gain[l] : nullptr;
  }
  rc = upload(h, (void**)&h->fused_layers, ly.data(), L * sizeof(FusedLayer));
  if (rc) return rc;
  h->fused_ok = true;
  return AE_OK;
}

// The batch-1 denoise as `steps` launches of the persistent step kernel (one per Euler step) on
// prefix slot slot0. Launch k polls activation ring k % 2 and empties ring (k + 1) % 2, which the
// previous launch used; ring 0 is empty when a pass starts, so a pass with an odd step count ends
// with a fill of ring 0 (its last launch used it).
int enqueue_fused(ae_handle* h, int steps, const float* temb, hipStream_t st, Timer* tm, int slot0) {
  const ae_config& c = h->c;
  FusedArgs fa{};
  fa.layers = h->fused_layers;
  fa.L = c.n_layers; fa.w = c.width; fa.F = c.mlp_dim; fa.nq = c.n_q_heads; fa.nkv = c.n_kv_heads; fa.dh = c.head_dim;
  fa.H = c.horizon; fa.P = c.prefix_len; fa.A = c.action_dim;
  fa.ntt = (c.horizon + 15) / 16;
  fa.ntp = fa.ntt <= 1 ? 1 : fa.ntt <= 2 ? 2 : 4;
  fa.G = h->n_cu;
  fa.eps = c.rms_eps; fa.inv_w = 1.f / (float)c.width;
  fa.x = h->x;
  fa.w_in = (const uint16_t*)h->action_in_w; fa.b_in = h->action_in_b; fa.ln1_0 = h->ln1[0];
  fa.w_out = (const uint16_t*)h->action_out_p; fa.b_out = h->action_out_b; fa.out_tiles = h->out_tiles;
  fa.dt = 1.f / (float)steps;
  fa.rope_cs = h->rope_cs;
  fa.n_qt = h->n_qt; fa.nbp = h->nbp; fa.nbs = h->nbs; fa.n_split = h->f_nsplit; fa.n_att = h->f_natt;
  fa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)c.head_dim));
  fa.part_o = h->fpart_o; fa.part_ml = h->fpart_ml;
  fa.layer_bytes = h->layer_bytes;
  fa.off_ssp = h->off_ssp; fa.off_q = h->off_q; fa.off_k = h->off_k; fa.off_v = h->off_v; fa.off_o = h->off_o;
  fa.off_hb2 = h->off_hb2; fa.off_ssp2 = h->off_ssp2; fa.off_u = h->off_u;
  fa.abort = h->abort_dev; fa.host_flag = h->flag_dev; fa.wait_ticks = h->wait_ticks;
  fa.slot_off = (size_t)slot0 * h->slot_elems;
  fa.off_qks = h->off_qks;
  fa.qk_inv_dh = 1.f / (float)c.head_dim;
  fa.qk_eps = c.rms_eps;
  const ae_handle::ModTable* mt = nullptr;  // time modulation: this step count's table
  if (c.time_mode) {
    auto it = h->mod_steps.find(steps);
    if (it == h->mod_steps.end()) return fail(h, AE_ERR_HIP, "modulation table missing for this step count");
    mt = &it->second;
    const size_t w = c.width;
    fa.m_sw = (size_t)steps * w;
    fa.m_sqkv = (size_t)steps * h->qkv_tiles * 16;
    fa.m_sgu = (size_t)steps * h->gu_tiles * 16;
    fa.m_smod = (size_t)steps * 6 * w;
  }
  for (int k = 0; k < steps; ++k) {
    fa.temb = temb + (size_t)k * c.width;
    if (mt) {  // step k's vectors; the tokens get no temb, the head this step's bias
      const size_t w = c.width;
      fa.temb = h->zero_w;
      fa.m_g1 = mt->g1 + (size_t)k * w;
      fa.m_g2 = mt->g2 + (size_t)k * w;
      fa.m_bqkv = mt->bqkv + (size_t)k * h->qkv_tiles * 16;
      fa.m_bgu = mt->bgu + (size_t)k * h->gu_tiles * 16;
      fa.m_mod = mt->mod + (size_t)k * 6 * w;
      fa.m_gf = mt->gf + (size_t)k * w;
      fa.b_out = mt->bout + (size_t)k * h->out_tiles * 16;
    }
    fa.ring = h->ring[k & 1];
    fa.ring_other = h->ring[(k + 1) & 1];
    fa.part_o = h->fpart_o + (k & 1) * (h->fpart_o_floats / 2);
    fa.part_ml = h->fpart_ml + (k & 1) * (h->fpart_ml_floats / 2);
    fa.part_o_other = h->fpart_o + ((k + 1) & 1) * (h->fpart_o_floats / 2);
    fa.part_ml_other = h->fpart_ml + ((k + 1) & 1) * (h->fpart_ml_floats / 2);
    LAUNCH_CHECK(h, "fused_step", AE_LAUNCH(h->fused_fn, dim3(h->n_cu), dim3(FT), h->fused_lds, st, fa));
  }
  if (steps & 1) {  // the last launch used ring 0 and partial set 0: the next call starts on them
    const size_t n16 = (size_t)(c.n_layers + 1) * h->layer_bytes / 16;
    LAUNCH_CHECK(h, "fill_empty", AE_LAUNCH(fill_empty_kernel, dim3(1024), dim3(256), 0, st, (uint4*)h->ring[0], n16));
    LAUNCH_CHECK(h, "fill_empty", AE_LAUNCH(fill_empty_kernel, dim3(1024), dim3(256), 0, st, (uint4*)h->fpart_o,
                                            h->fpart_o_floats / 2 / 4));
    LAUNCH_CHECK(h, "fill_empty", AE_LAUNCH(fill_empty_kernel, dim3(1024), dim3(256), 0, st, (uint4*)h->fpart_ml,
                                            h->fpart_ml_floats / 2 / 4));
  }
  return AE_OK;
}

int enqueue_denoise(ae_handle* h, int batch, int steps, float* temb, hipStream_t st, Timer* tm, int slot0 = 0) {
  if (batch == 1 && h->variant == 0 && h->fused_ok) return enqueue_fused(h, steps, temb, st, tm, slot0);
  const float dt = 1.f / (float)steps;
  for (int k = 0; k < steps; ++k) {
    // robot b uses prefix slot b: no slot table (the attention then reads no slot from memory)
    StepMod sm{nullptr, k, steps};
    if (h->c.time_mode) {
      auto it = h->mod_steps.find(steps);
      if (it == h->mod_steps.end()) return fail(h, AE_ERR_HIP, "modulation table missing for this step count");
      sm.t = &it->second;
    }
    int rc = enqueue_velocity(h, batch, temb + (size_t)k * h->c.width, 0, nullptr, slot0, dt, st, tm,
                              h->c.time_mode ? &sm : nullptr);
    if (rc) return rc;
  }
  return AE_OK;
}

int enqueue_verify(ae_handle* h, int n_tau, hipStream_t st, Timer* tm) {
  const ae_config& c = h->c;
  const int H = c.horizon, A = c.action_dim;
  // x_j and phi(tau_j) in one launch, then the time MLP
  LAUNCH_CHECK(h, "verify_start", AE_LAUNCH(verify_start_kernel, dim3(std::max((n_tau * H * A + 255) / 256, std::max(1, c.width / 2 / 256)), n_tau + 1),
                                             dim3(256), 0, st, h->draft, h->vnoise, h->taus, n_tau, H, A, h->x, c.width,
                                             h->phi));
  int rc = enqueue_time_mlp(h, n_tau, h->temb_tau, st, tm);
  if (rc) return rc;
  StepMod sm{&h->mod_tau, 0, std::max(1, c.max_taus), true};
  if (c.time_mode) {  // each flow time's modulation vectors, from its temb
    rc = enqueue_mod_tau(h, n_tau, st, tm);
    if (rc) return rc;
  }
  h->verify_head = true;  // the output projection forms the distances and the accepted length
  rc = enqueue_velocity(h, n_tau, h->temb_tau, c.width, h->verify_slots, 0, 0.f, st, tm, c.time_mode ? &sm : nullptr);
  h->verify_head = false;
  return rc;
}

// The draft model's pass: stage the image features (h->feat) as GEMM input rows, write their K/V
// through the block's own k/v projections (K rotated at positions 0..P-1) into prefix slot 0, put
// the staged queries into h / hb / ssp_a, then the block and the head over the query rows.
int enqueue_draft(ae_handle* h, hipStream_t st, Timer* tm) {
  const ae_config& c = h->c;
  const int w = c.width, P = c.prefix_len, H = c.horizon, nq = c.n_q_heads, nkv = c.n_kv_heads, dh = c.head_dim;
  const int Pp = (P + TOKG - 1) / TOKG * TOKG, Mp = (H + TOKG - 1) / TOKG * TOKG;
  LAUNCH_CHECK(h, "draft_stage_features", AE_LAUNCH(stage_rows_kernel, dim3(w / 64, Pp / 64), dim3(256), 0, st, h->feat,
                                                    P, Pp, w, h->ln1[0], (float*)nullptr, (uint16_t*)h->feat_hb,
                                                    h->feat_ssp));
  {
    // the k and v tiles of the packed QKV weights only (no query tiles): n_q = 0 makes every tile of
    // the launch a key tile, then value tiles, in the QKV epilogue
    const int tph = dh / 16, KB = w / KBLK;
    GemmArgs a{};
    a.w = (const uint16_t*)h->qkv_p[0] + (size_t)nq * tph * KB * 512;
    a.x = h->feat_hb; a.ssp_in = h->feat_ssp; a.g_in = w / 16;
    a.inv_width = 1.f / (float)w; a.eps = c.rms_eps;
    a.M = P; a.M_pad = Pp; a.K = w; a.S = 1;
    a.part = h->part; a.counters = h->counters;
    a.n_q = 0; a.n_kv = nkv; a.dh = dh; a.H = P; a.nbs = h->nbp; a.n_qt = 0;
    a.rope_cs = h->rope_feat;
    a.k_out = h->kcache; a.v_out = h->vcache;  // slot 0, layer 0: the cache's own block layout
    LAUNCH_CHECK(h, "draft_feature_kv", (void)Dispatch::gemm(h, R_QKV_ROPE, a, 2 * nkv * tph, Pp / TOKG, st));
  }
  HIP_TRY(h, hipMemcpyAsync(h->h, h->q_h0, (size_t)Mp * w * 4, hipMemcpyDeviceToDevice, st));
  HIP_TRY(h, hipMemcpyAsync(h->hb, h->q_hb0, (size_t)Mp * w * (h->at == AT_F32 ? 4 : 2), hipMemcpyDeviceToDevice, st));
  HIP_TRY(h, hipMemcpyAsync(h->ssp_a, h->q_ssp0, (size_t)(w / 16) * Mp * 4, hipMemcpyDeviceToDevice, st));
  return enqueue_velocity(h, 1, nullptr, 0, nullptr, 0, 0.f, st, tm, nullptr, true);
}

// The prefill stack's pass: the embeddings (h->feat) staged as the block input rows (h, hb and the
// RMS partials), then the blocks with every token attending to every token (the whole prefix is
// the "suffix" of a prefix-free pass); each layer's K/V is copied out as its QKV kernel writes it.
int enqueue_prefill(ae_handle* h, hipStream_t st, Timer* tm) {
  const ae_config& c = h->c;
  const int w = c.width, H = c.horizon, Mp = (H + TOKG - 1) / TOKG * TOKG;
  LAUNCH_CHECK(h, "prefill_stage", AE_LAUNCH(stage_rows_kernel, dim3(w / 64, Mp / 64), dim3(256), 0, st, h->feat, H, Mp,
                                             w, h->ln1[0], h->h, (uint16_t*)h->hb, h->ssp_a));
  return enqueue_velocity(h, 1, nullptr, 0, nullptr, 0, 0.f, st, tm, nullptr, true, false);
}

// The capture variant a call starts with: the persistent step kernel unless it gave up on three
// passes in a row (the device is shared, say), then one launch per phase.
int pref_variant(const ae_handle* h) { return h->fused_fail >= 3 ? 1 : 0; }

int get_graph(ae_handle* h, int mode, int a, int b, hipGraphExec_t* out, int variant) {
  auto key = std::make_tuple(mode + 16 * variant, a, b);
  auto it = h->graphs.find(key);
  if (it != h->graphs.end()) { *out = it->second; return AE_OK; }
  // mode 0: denoise (a steps, b robots on slots 0..b-1); 1: verify (a flow times);
  // 2: denoise of one robot on prefix slot b (a steps); 3: the draft model's pass; 4: prefill
  float* temb = nullptr;
  if (mode == 0 || mode == 2) {
    int rc = get_temb_steps(h, a, &temb);
    if (rc) return rc;
  }
  HIP_TRY(h, hipStreamBeginCapture(h->stream, hipStreamCaptureModeThreadLocal));
  h->variant = variant;
  int rc = mode == 0   ? enqueue_denoise(h, b, a, temb, h->stream, nullptr)
           : mode == 2 ? enqueue_denoise(h, 1, a, temb, h->stream, nullptr, b)
           : mode == 3 ? enqueue_draft(h, h->stream, nullptr)
           : mode == 4 ? enqueue_prefill(h, h->stream, nullptr)
                       : enqueue_verify(h, a, h->stream, nullptr);
  h->variant = 0;
  hipGraph_t graph = nullptr;
  hipError_t e = hipStreamEndCapture(h->stream, &graph);
  if (rc) { if (graph) hipGraphDestroy(graph); return rc; }
  if (e != hipSuccess) return fail(h, AE_ERR_HIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(e));
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  hipGraphDestroy(graph);
  if (e != hipSuccess) return fail(h, AE_ERR_HIP, std::string("hipGraphInstantiate: ") + hipGetErrorString(e));
  h->graphs[key] = exec;
  *out = exec;
  return AE_OK;
}

// A pass of `mode` (as in get_graph): its captured graph, replayed by launch_pass, or on an eager
// handle (AE_GRAPH=0) the same launches enqueued by launch_pass directly on its stream.
struct Pass {
  hipGraphExec_t g = nullptr;
  int mode = 0, a = 0, b = 0, variant = 0;
};

int get_pass(ae_handle* h, int mode, int a, int b, Pass* p, int variant) {
  *p = Pass{nullptr, mode, a, b, variant};
  if (!h->eager) return get_graph(h, mode, a, b, &p->g, variant);
  float* temb = nullptr;
  return mode == 0 || mode == 2 ? get_temb_steps(h, a, &temb) : AE_OK;  // built before the pass, as for a graph
}

int launch_pass(ae_handle* h, const Pass& p, hipStream_t st) {
  if (p.g) {
    HIP_TRY(h, hipGraphLaunch(p.g, st));
    return AE_OK;
  }
  float* temb = nullptr;
  if (p.mode == 0 || p.mode == 2) {
    const int rc = get_temb_steps(h, p.a, &temb);
    if (rc) return rc;
  }
  h->variant = p.variant;
  const int rc = p.mode == 0   ? enqueue_denoise(h, p.b, p.a, temb, st, nullptr)
                 : p.mode == 2 ? enqueue_denoise(h, 1, p.a, temb, st, nullptr, p.b)
                 : p.mode == 3 ? enqueue_draft(h, st, nullptr)
                 : p.mode == 4 ? enqueue_prefill(h, st, nullptr)
                               : enqueue_verify(h, p.a, st, nullptr);
  h->variant = 0;
  return rc;
}

}  // namespace

// =====================================================================================
// Scratch of the no-allocation entry point (ae_denoise_static): every activation, partial, counter
// and time table of one pass, carved from this file-scope array. Each device holds its own copy
// from the load of the code object to the end of the process. Host code never passes the array's
// name to a kernel or a copy (on the host it is a stand-in, not a device address): it uses the
// address hipGetSymbolAddress returns, looked up once per device with that device current.
static __device__ __align__(256) unsigned char scratch[AE_STATIC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_addr;  // per device ordinal: the address of `scratch` there

// The device address of `scratch` on h's device (the current one, at ae_create).
int scratch_address(ae_handle* h) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr.size() <= (size_t)h->dev) g_scratch_addr.resize((size_t)h->dev + 1, nullptr);
  if (!g_scratch_addr[h->dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      h->static_err = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
      return AE_ERR_HIP;
    }
    g_scratch_addr[h->dev] = p;
  }
  h->static_scratch = g_scratch_addr[h->dev];
  return AE_OK;
}

// Byte offsets in `scratch` of one ae_denoise_static pass over `batch` robots and `steps` steps:
// the buffers a handle allocates for its passes, sized for this batch (the kernels index them by the
// pass's own padded token count), plus the step-time table and its time-MLP staging.
struct StaticLayout {
  size_t x, h, hb, ssp_a, ssp_b, q, ks, vs, o, u, part, counters, opart, mlpart, qk_ssp, t, phi, hid, temb;
  size_t total;
};

StaticLayout static_layout(const ae_handle* h, int batch, int steps) {
  const ae_config& c = h->c;
  const int w = c.width, A = c.action_dim, F = c.mlp_dim, nq = c.n_q_heads, nkv = c.n_kv_heads, dh = c.head_dim;
  const size_t M = (size_t)batch * c.horizon, Mp = (M + TOKG - 1) / TOKG * TOKG, n_z = Mp / TOKG;
  const size_t aes = h->at == AT_F32 ? 4 : 2;
  StaticLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (std::max<size_t>(bytes, 16) + 255) / 256 * 256;
    return o;
  };
  L.x = take(Mp * A * 4);
  L.h = take(Mp * w * 4);
  L.hb = take(Mp * w * aes);
  L.ssp_a = take((size_t)(w / 16) * Mp * 4);
  L.ssp_b = take((size_t)(w / 16) * Mp * 4);
  L.q = take((size_t)batch * nkv * h->n_qt * ATT_ROWS * dh * aes);
  L.ks = take((size_t)batch * nkv * h->nbs * ATT_KB * dh * aes);
  L.vs = take((size_t)batch * nkv * h->nbs * ATT_KB * dh * aes);
  L.o = take(Mp * nq * dh * aes);
  L.u = take(Mp * F * aes);
  const size_t maxg = std::max({(size_t)h->qkv_tiles, (size_t)(w / 16), (size_t)h->gu_tiles, (size_t)h->out_tiles});
  L.part = take(4 * maxg * 2 * TOKG * 16 * n_z * 4);
  L.counters = take(maxg * n_z * 4);
  const int nb = h->nbp + h->nbs;
  const size_t n_split = std::max(attn_splits(nb, ATT_IT_SPLIT, ATT_WAVES_SPLIT), attn_splits(nb, ATT_IT_WHOLE, ATT_WAVES_WHOLE));
  const size_t zz = (size_t)batch * nkv;
  L.opart = take(zz * h->n_qt * n_split * ATT_ROWS * dh * 4);
  L.mlpart = take(zz * h->n_qt * n_split * ATT_ROWS * 2 * 4);
  L.qk_ssp = c.qk_norm ? take((size_t)(nq + nkv) * dh / 16 * Mp * 4) : 0;
  L.t = take((size_t)steps * 4);
  L.phi = take((size_t)steps * w * 4);
  L.hid = take((size_t)steps * w * 4);
  L.temb = take((size_t)steps * w * 4);
  L.total = off;
  return L;
}

// The handle's per-pass buffers and capture variant, set aside while a pass runs in the static
// scratch and put back when the call returns (on every path).
class PassBuffers {
 public:
  explicit PassBuffers(ae_handle* h)
      : h_(h), x_(h->x), h_buf_(h->h), ssp_a_(h->ssp_a), ssp_b_(h->ssp_b), part_(h->part), opart_(h->opart),
        mlpart_(h->mlpart), qk_ssp_(h->qk_ssp), phi_(h->phi), hid_(h->hid), hb_(h->hb), o_(h->o), u_(h->u),
        q_(h->q), ks_(h->ks), vs_(h->vs), counters_(h->counters), variant_(h->variant) {}
  ~PassBuffers() {
    h_->x = x_; h_->h = h_buf_; h_->ssp_a = ssp_a_; h_->ssp_b = ssp_b_; h_->part = part_; h_->opart = opart_;
    h_->mlpart = mlpart_; h_->qk_ssp = qk_ssp_; h_->phi = phi_; h_->hid = hid_; h_->hb = hb_; h_->o = o_;
    h_->u = u_; h_->q = q_; h_->ks = ks_; h_->vs = vs_; h_->counters = counters_; h_->variant = variant_;
  }
  PassBuffers(const PassBuffers&) = delete;
  PassBuffers& operator=(const PassBuffers&) = delete;

 private:
  ae_handle* h_;
  float *x_, *h_buf_, *ssp_a_, *ssp_b_, *part_, *opart_, *mlpart_, *qk_ssp_, *phi_, *hid_;
  void *hb_, *o_, *u_, *q_, *ks_, *vs_;
  unsigned* counters_;
  int variant_;
};

}  // namespace

extern "C" {

int ae_create(const ae_config* cfg, const ae_weights* wts, ae_handle** out) {
  g_create_error.clear();
  if (!out) return fail(nullptr, AE_ERR_INVALID_ARG, "null output handle pointer");
  *out = nullptr;
  int rc = validate(cfg, wts);
  if (rc) return rc;
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess || ndev == 0) return fail(nullptr, AE_ERR_HIP, "no HIP device available");

  ae_handle* h = new ae_handle();
  h->c = *cfg;
  const ae_config& c = h->c;
  if (hipGetDevice(&h->dev) != hipSuccess) { delete h; return fail(nullptr, AE_ERR_HIP, "hipGetDevice failed"); }
  if (hipDeviceGetAttribute(&h->n_cu, hipDeviceAttributeMultiprocessorCount, h->dev) != hipSuccess) h->n_cu = 0;
  if (const char* e = getenv("AE_ATTN_CORESIDENT")) h->coresident_attn = atoi(e) != 0;
  if (const char* e = getenv("AE_EXCH_POLL")) h->poll_splitk = atoi(e) != 0;
  if (const char* e = getenv("AE_TILED")) h->tiled_roles = (int)strtol(e, nullptr, 0);
  if (const char* e = getenv("AE_TILED_SHAPE")) h->tiled_force = atoi(e);
  if (const char* e = getenv("AE_ATTN_XCD")) h->attn_xcd = atoi(e) != 0;
  if (const char* e = getenv("AE_WAIT_TICKS")) h->wait_ticks = strtoull(e, nullptr, 0);
  if (const char* e = getenv("AE_GRAPH")) h->eager = atoi(e) == 0;
  if (const char* e = getenv("AE_SPLITK")) {
    int so = 0, sd = 0;
    if (sscanf(e, "%d,%d", &so, &sd) == 2 && so >= 1 && so <= 4 && sd >= 1 && sd <= 4) {
      h->sk.o = so;
      h->sk.down = sd;
    }
  }
  bool want_fused = true;
  if (const char* e = getenv("AE_FUSED")) want_fused = atoi(e) != 0;
  if (hipStreamCreateWithFlags(&h->stream, hipStreamNonBlocking) != hipSuccess) { delete h; return fail(nullptr, AE_ERR_HIP, "hipStreamCreate failed"); }
  hipEventCreate(&h->ev0);
  hipEventCreate(&h->ev1);
  hipEventCreate(&h->ev_round);
  h->at = c.weight_dtype == AE_F32 ? AT_F32 : AT_BF16;
  h->wt = c.weight_dtype == AE_F32 ? WT_F32 : WT_BF16;
  h->mt = c.mlp_dtype == AE_F32 ? WT_F32 : c.mlp_dtype == AE_BF16 ? WT_BF16 : WT_FP8;
  if ((h->at == AT_BF16 ? attn_dispatch<AT_BF16>(cfg->head_dim, true, false, dim3(), nullptr, AttnArgs{})
                        : attn_dispatch<AT_F32>(cfg->head_dim, true, false, dim3(), nullptr, AttnArgs{})) != hipSuccess ||
      (h->at == AT_BF16 && attn_pair_dispatch(cfg->head_dim, true, dim3(), nullptr, AttnArgs{}) != hipSuccess) ||
      set_all_gemm_attrs() != hipSuccess) {
    std::string m = "hipFuncSetAttribute failed";
    ae_destroy(h);
    return fail(nullptr, AE_ERR_HIP, m);
  }
  // in-kernel waits only where the occupancy calculator puts at least one workgroup on every compute unit
  {
    int occ_a, occ_g;
    if (h->at == AT_F32) {
      occ_a = attn_split_occ<AT_F32, false>(cfg->head_dim);
      occ_g = std::min(std::min(gemm_occ<WT_F32, AT_F32, R_QKV_ROPE>(), gemm_occ<WT_F32, AT_F32, R_O_PROJ>()),
                       std::min(gemm_occ<WT_F32, AT_F32, R_GATE_UP>(), gemm_occ<WT_F32, AT_F32, R_DOWN>()));
    } else {
      occ_a = cfg->qk_norm ? attn_split_occ<AT_BF16, true>(cfg->head_dim) : attn_split_occ<AT_BF16, false>(cfg->head_dim);
      occ_g = std::min(gemm_occ<WT_BF16, AT_BF16, R_QKV_ROPE>(), gemm_occ<WT_BF16, AT_BF16, R_O_PROJ>());
      occ_g = std::min(occ_g, h->mt == WT_FP8 ? std::min(gemm_occ<WT_FP8, AT_BF16, R_GATE_UP>(), gemm_occ<WT_FP8, AT_BF16, R_DOWN>())
                                              : std::min(gemm_occ<WT_BF16, AT_BF16, R_GATE_UP>(), gemm_occ<WT_BF16, AT_BF16, R_DOWN>()));
    }
    h->occ_attn = occ_a;
    h->occ_gemm = occ_g;
    if (occ_a < 1) h->coresident_attn = false;
    if (occ_g < 1) h->poll_splitk = false;
  }

  const int w = c.width, A = c.action_dim, F = c.mlp_dim, nq = c.n_q_heads, nkv = c.n_kv_heads, dh = c.head_dim;
  const int L = c.n_layers, H = c.horizon, P = c.prefix_len;
  const size_t wes = dtype_size(c.weight_dtype), mes = dtype_size(c.mlp_dtype), kes = dtype_size(c.kv_dtype);
  const int aes = h->at == AT_F32 ? 4 : 2;
  h->M_max = std::max(c.max_batch, std::max(1, c.max_taus)) * H;
  h->Mp_max = (h->M_max + TOKG - 1) / TOKG * TOKG;
  const int Mp = h->Mp_max;
  std::string msg;
#define TRY(x) do { int r_ = (x); if (r_) { msg = h->err; ae_destroy(h); return fail(nullptr, r_, msg); } } while (0)

  // ---- small weights (row-major, used by the time MLP and in_proj kernels)
  if (!c.draft && !c.prefill) {
    TRY(upload(h, &h->time_in_w, wts->time_in_w, (size_t)w * w * wes));
    TRY(upload(h, (void**)&h->time_in_b, wts->time_in_b, (size_t)w * 4));
    TRY(upload(h, &h->time_out_w, wts->time_out_w, (size_t)w * w * wes));
    TRY(upload(h, (void**)&h->time_out_b, wts->time_out_b, (size_t)w * 4));
    TRY(upload(h, &h->action_in_w, wts->action_in_w, (size_t)w * A * wes));
    TRY(upload(h, (void**)&h->action_in_b, wts->action_in_b, (size_t)w * 4));
  }
  h->out_tiles = (A + 15) / 16;
  if (!c.prefill) {  // the head (a prefill stack has none)
    TRY(upload(h, (void**)&h->action_out_b, wts->action_out_b, (size_t)A * 4));
    TRY(upload(h, (void**)&h->final_ln, wts->final_ln, (size_t)w * 4));
    std::vector<unsigned char> buf;
    pack_rows(ae_host::plain_rows(wts->action_out_w, A, w, wes, h->out_tiles * 16), w, wes, buf);
    TRY(upload(h, &h->action_out_p, buf.data(), buf.size()));
  }
  // ---- decoder layers, packed
  h->qkv_tiles = (nq + 2 * nkv) * dh / 16;
  h->gu_tiles = 2 * F / 16;
  for (int l = 0; l < L; ++l) {
    const ae_layer_weights& Lw = wts->layers[l];
    std::vector<unsigned char> buf;
    // q heads, k heads: tile = 8 channels d..d+7 and their RoPE partners d+dh/2..; then v
    pack_rows(ae_host::qkv_rows(Lw.wq, Lw.wk, Lw.wv, nq, nkv, dh, w, wes), w, wes, buf);
    void* p = nullptr;
    TRY(upload(h, &p, buf.data(), buf.size()));
    h->qkv_p.push_back(p);
    pack_rows(ae_host::plain_rows(Lw.wo, w, nq * dh, wes), nq * dh, wes, buf);
    TRY(upload(h, &p, buf.data(), buf.size()));
    h->o_p.push_back(p);
    // gate/up interleaved by 16-row tiles (their E4M3 scales likewise)
    std::vector<float> gus;
    if (c.mlp_dtype == AE_FP8_E4M3)
      for (int j = 0; j < F / 16; ++j) {
        for (int cc = 0; cc < 16; ++cc) gus.push_back(Lw.wg_scale[j * 16 + cc]);
        for (int cc = 0; cc < 16; ++cc) gus.push_back(Lw.wu_scale[j * 16 + cc]);
      }
    pack_rows(ae_host::gate_up_rows(Lw.wg, Lw.wu, F, w, mes), w, mes, buf);
    TRY(upload(h, &p, buf.data(), buf.size()));
    h->gu_p.push_back(p);
    pack_rows(ae_host::plain_rows(Lw.wd, w, F, mes), F, mes, buf);
    TRY(upload(h, &p, buf.data(), buf.size()));
    h->d_p.push_back(p);
    float *gs = nullptr, *ds = nullptr;
    if (c.mlp_dtype == AE_FP8_E4M3) {
      TRY(upload(h, (void**)&gs, gus.data(), gus.size() * 4));
      TRY(upload(h, (void**)&ds, Lw.wd_scale, (size_t)w * 4));
    }
    h->gu_s.push_back(gs);
    h->d_s.push_back(ds);
    float *g1 = nullptr, *g2 = nullptr;
    TRY(upload(h, (void**)&g1, Lw.ln1, (size_t)w * 4));
    TRY(upload(h, (void**)&g2, Lw.ln2, (size_t)w * 4));
    h->ln1.push_back(g1);
    h->ln2.push_back(g2);
    if (c.time_mode) {
      void* wm = nullptr;
      float* bm = nullptr;
      TRY(upload(h, &wm, Lw.w_mod, (size_t)6 * w * w * wes));
      TRY(upload(h, (void**)&bm, Lw.b_mod, (size_t)6 * w * 4));
      h->w_mod.push_back(wm);
      h->b_mod.push_back(bm);
    }
    if (c.qk_norm) {  // gains in the packed q/k channel order (tile = dims p*8.. and their RoPE partners)
      std::vector<float> gq;
      auto head_gains = [&](const float* gain, int nh) {
        for (int hh = 0; hh < nh; ++hh)
          for (int pp = 0; pp < dh / 16; ++pp)
            for (int cc = 0; cc < 16; ++cc) gq.push_back(gain[ae_host::rope_tile_dim(dh, pp, cc)]);
      };
      head_gains(Lw.q_norm, nq);
      head_gains(Lw.k_norm, nkv);
      float* gd = nullptr;
      TRY(upload(h, (void**)&gd, gq.data(), gq.size() * 4));
      h->qk_gain.push_back(gd);
    }
  }
  if (c.time_mode) {
    TRY(upload(h, &h->final_mod_w, wts->final_mod_w, (size_t)2 * w * w * wes));
    TRY(upload(h, (void**)&h->final_mod_b, wts->final_mod_b, (size_t)2 * w * 4));
    TRY(dalloc_t(h, &h->zero_w, (size_t)w));
    if (c.max_taus > 0) TRY(alloc_mod_table(h, c.max_taus, h->mod_tau));
  }
  if (c.qk_norm) TRY(dalloc_t(h, &h->qk_ssp, (size_t)(nq + nkv) * dh / 16 * Mp));
  // ---- activations and scratch (padding rows stay zero)
  TRY(dalloc_t(h, &h->x, (size_t)Mp * A));
  TRY(dalloc_t(h, &h->vout, (size_t)Mp * A));
  TRY(dalloc_t(h, &h->h, (size_t)Mp * w));
  // activations between kernels in the GEMMs' fragment order (act_idx): Mp tokens x K inputs
  TRY(dalloc(h, &h->hb, (size_t)Mp * w * aes));
  TRY(dalloc_t(h, &h->ssp_a, (size_t)(w / 16) * Mp));
  TRY(dalloc_t(h, &h->ssp_b, (size_t)(w / 16) * Mp));
  {
    const size_t seqs = (size_t)std::max(c.max_batch, std::max(1, c.max_taus));
    h->n_qt = (nq / nkv * H + ATT_ROWS - 1) / ATT_ROWS;
    h->nbs = (H + ATT_KB - 1) / ATT_KB;
    h->nbp = (P + ATT_KB - 1) / ATT_KB;
    TRY(dalloc(h, &h->q, seqs * nkv * h->n_qt * ATT_ROWS * dh * aes));
    TRY(dalloc(h, &h->ks, seqs * nkv * h->nbs * ATT_KB * dh * aes));
    TRY(dalloc(h, &h->vs, seqs * nkv * h->nbs * ATT_KB * dh * aes));
  }
  TRY(dalloc(h, &h->o, (size_t)Mp * nq * dh * aes));
  TRY(dalloc(h, &h->u, (size_t)Mp * F * aes));
  {
    const int n_z = (Mp + TOKG - 1) / TOKG;
    size_t maxg = std::max({(size_t)h->qkv_tiles, (size_t)(w / 16), (size_t)h->gu_tiles, (size_t)h->out_tiles});
    h->part_floats = 4 * maxg * 2 * TOKG * 16 * (size_t)n_z;
    TRY(dalloc_t(h, &h->part, h->part_floats));
    h->n_counters = maxg * n_z;
    TRY(dalloc_t(h, &h->counters, h->n_counters));
    const int R = nq / nkv * H;
    const size_t n_qt = (R + ATT_ROWS - 1) / ATT_ROWS;
    const int nb = (P + ATT_KB - 1) / ATT_KB + (H + ATT_KB - 1) / ATT_KB;
    const size_t n_split = std::max(attn_splits(nb, ATT_IT_SPLIT, ATT_WAVES_SPLIT), attn_splits(nb, ATT_IT_WHOLE, ATT_WAVES_WHOLE));
    const size_t n_zz = (size_t)std::max(c.max_batch, std::max(1, c.max_taus)) * nkv;
    h->opart_floats = n_zz * n_qt * n_split * ATT_ROWS * dh;
    h->mlpart_floats = n_zz * n_qt * n_split * ATT_ROWS * 2;
    TRY(dalloc_t(h, &h->opart, h->opart_floats));
    TRY(dalloc_t(h, &h->mlpart, h->mlpart_floats));
    if (hipHostMalloc((void**)&h->flag_host, sizeof(unsigned), hipHostMallocMapped) != hipSuccess ||
        hipHostGetDevicePointer((void**)&h->flag_dev, h->flag_host, 0) != hipSuccess) {
      ae_destroy(h);
      return fail(nullptr, AE_ERR_HIP, "pinned host flag allocation failed");
    }
    *h->flag_host = 0;
  }
  {
    std::vector<float> cs((size_t)H * (dh / 2) * 2);
    for (int t = 0; t < H; ++t)
      for (int d = 0; d < dh / 2; ++d) {
        double ang = (double)(P + t) * std::pow((double)c.rope_base, -2.0 * d / dh);
        cs[((size_t)t * (dh / 2) + d) * 2 + 0] = (float)std::cos(ang);
        cs[((size_t)t * (dh / 2) + d) * 2 + 1] = (float)std::sin(ang);
      }
    TRY(upload(h, (void**)&h->rope_cs, cs.data(), cs.size() * 4));
  }
  h->slot_elems = (size_t)L * nkv * h->nbp * ATT_KB * dh;
  TRY(dalloc(h, &h->kcache, h->slot_elems * c.max_batch * kes));
  TRY(dalloc(h, &h->vcache, h->slot_elems * c.max_batch * kes));
  h->slot_ready.assign(c.max_batch, 0);
  const int ntau = std::max(1, c.max_taus);
  TRY(dalloc_t(h, &h->verify_slots, ntau));
  TRY(dalloc_t(h, &h->draft, (size_t)H * A));
  TRY(dalloc_t(h, &h->vnoise, (size_t)H * A));
  TRY(dalloc_t(h, &h->taus, ntau));
  TRY(dalloc_t(h, &h->temb_tau, (size_t)ntau * w));
  TRY(dalloc_t(h, &h->phi, (size_t)ntau * w));
  TRY(dalloc_t(h, &h->hid, (size_t)ntau * w));
  TRY(dalloc_t(h, &h->dist, (size_t)ntau * H));
  TRY(dalloc_t(h, &h->params, 4));
  TRY(dalloc_t(h, &h->accept, 1));
  TRY(dalloc_t(h, &h->gswitch, 1));
  TRY(dalloc_t(h, &h->vpart, (size_t)h->out_tiles * Mp));
  TRY(dalloc_t(h, &h->vcount, 4));
  if (c.draft) {
    // the queries as the block's input rows (fixed: staged once), the feature buffers, and the RoPE
    // table of the feature positions 0..P-1
    const int Pp = (P + TOKG - 1) / TOKG * TOKG;
    float* qrows = nullptr;
    TRY(upload(h, (void**)&qrows, wts->queries, (size_t)H * w * 4));
    TRY(dalloc_t(h, &h->q_h0, (size_t)Mp * w));
    TRY(dalloc(h, &h->q_hb0, (size_t)Mp * w * aes));
    TRY(dalloc_t(h, &h->q_ssp0, (size_t)(w / 16) * Mp));
    hipLaunchKernelGGL(stage_rows_kernel, dim3(w / 64, Mp / 64), dim3(256), 0, h->stream, qrows, H, Mp, w, h->ln1[0],
                       h->q_h0, (uint16_t*)h->q_hb0, h->q_ssp0);
    TRY(dalloc_t(h, &h->feat, (size_t)P * w));
    TRY(dalloc(h, &h->feat_hb, (size_t)Pp * w * aes));
    TRY(dalloc_t(h, &h->feat_ssp, (size_t)(w / 16) * Pp));
    std::vector<float> cs((size_t)P * (dh / 2) * 2);
    for (int t = 0; t < P; ++t)
      for (int d = 0; d < dh / 2; ++d) {
        double ang = (double)t * std::pow((double)c.rope_base, -2.0 * d / dh);
        cs[((size_t)t * (dh / 2) + d) * 2 + 0] = (float)std::cos(ang);
        cs[((size_t)t * (dh / 2) + d) * 2 + 1] = (float)std::sin(ang);
      }
    TRY(upload(h, (void**)&h->rope_feat, cs.data(), cs.size() * 4));
    if (hipGetLastError() != hipSuccess) { ae_destroy(h); return fail(nullptr, AE_ERR_HIP, "query staging launch failed"); }
  }
  if (c.prefill) {  // the embeddings, and every layer's suffix K/V (the cache blocks' layout)
    TRY(dalloc_t(h, &h->feat, (size_t)H * w));
    h->pf_layer_elems = (size_t)nkv * h->nbs * ATT_KB * dh;
    TRY(dalloc(h, &h->pf_k, (size_t)L * h->pf_layer_elems * kes));
    TRY(dalloc(h, &h->pf_v, (size_t)L * h->pf_layer_elems * kes));
  }
  if (c.time_mode && c.max_taus > 0) TRY(setup_mod_tau_jobs(h));
  if (want_fused) TRY(setup_fused(h));
  (void)scratch_address(h);  // a failure is reported by ae_denoise_static
  TRY(reset_exchange(h));
  if (hipDeviceSynchronize() != hipSuccess) { ae_destroy(h); return fail(nullptr, AE_ERR_HIP, "device sync after upload failed"); }
#undef TRY
  *out = h;
  return AE_OK;
}

int ae_load_prefix_kv(ae_handle* h, int slot, const void* k, const void* v) {
  if (!h) return AE_ERR_INVALID_ARG;
  if (!k || !v) return fail(h, AE_ERR_INVALID_ARG, "null cache pointer");
  if (slot < 0 || slot >= h->c.max_batch) return fail(h, AE_ERR_INVALID_ARG, "slot out of range");
  const ae_config& c = h->c;
  const size_t es = dtype_size(c.kv_dtype);
  const size_t bytes = h->slot_elems * es;
  if (bytes) {
    // repack into the attention's fragment order: per layer and kv head, 32-key blocks; keys past
    // prefix_len stay zero
    std::vector<unsigned char> kp, vp;
    ae_host::repack_prefix_kv((const unsigned char*)k, (const unsigned char*)v, c.n_layers, c.prefix_len, c.n_kv_heads,
                              c.head_dim, h->nbp, es, kp, vp);
    HIP_TRY(h, hipMemcpy((char*)h->kcache + slot * bytes, kp.data(), bytes, hipMemcpyHostToDevice));
    HIP_TRY(h, hipMemcpy((char*)h->vcache + slot * bytes, vp.data(), bytes, hipMemcpyHostToDevice));
  }
  h->slot_ready[slot] = 1;
  return AE_OK;
}

// A kernel whose bounded wait gave up (not every workgroup of its launch was resident, say) sets the
// host-visible flag. A synchronous call that finds it set after its pass waits for the device,
// restores every exchange buffer and repeats the pass with launches that wait for nothing inside a
// kernel (variant 2); its outputs are then those of the repeated pass. An asynchronous call cannot
// repeat its pass: the next call on the handle finds the flag and reports it (failed_async).
static bool take_failure(ae_handle* h) {
  if (!h->flag_host || !__atomic_load_n(h->flag_host, __ATOMIC_ACQUIRE)) return false;
  reset_exchange(h);
  return true;
}

static int failed_async(ae_handle* h) {
  if (!take_failure(h)) return AE_OK;
  ++h->fused_fail;
  return fail(h, AE_ERR_HIP,
              "an earlier asynchronous pass on this handle gave up waiting for another workgroup of its launch "
              "(not all were resident); the outputs of the asynchronous passes enqueued since the last successful "
              "call are invalid; the exchange buffers are restored");
}

static int check_denoise(ae_handle* h, int batch, int steps) {
  if (!h) return AE_ERR_INVALID_ARG;
  if (h->c.draft) return fail(h, AE_ERR_UNSUPPORTED, "a draft-model handle runs ae_draft only");
  if (h->c.prefill) return fail(h, AE_ERR_UNSUPPORTED, "a prefill handle runs ae_prefill only");
  if (batch < 1 || batch > h->c.max_batch) return fail(h, AE_ERR_INVALID_ARG, "batch out of range");
  if (steps < 1 || steps > 1000) return fail(h, AE_ERR_INVALID_ARG, "steps out of range (1..1000)");
  for (int b = 0; b < batch; ++b)
    if (!h->slot_ready[b]) return fail(h, AE_ERR_NOT_READY, "prefix slot " + std::to_string(b) + " not loaded");
  return AE_OK;
}

// Count the outcome of a pass that used the persistent step kernel.
static void note_fused(ae_handle* h, int variant, int batch, bool failed) {
  if (variant != 0 || batch != 1 || !h->fused_ok) return;
  h->fused_fail = failed ? h->fused_fail + 1 : 0;
}

int ae_denoise_async(ae_handle* h, int batch, const float* d_noise, int steps, float* d_actions_out, void* stream) {
  int rc = check_denoise(h, batch, steps);
  if (rc) return rc;
  if (!d_noise || !d_actions_out) return fail(h, AE_ERR_INVALID_ARG, "null pointer");
  rc = failed_async(h);
  if (rc) return rc;
  hipStream_t st = stream ? (hipStream_t)stream : h->stream;
  Pass g;
  rc = get_pass(h, 0, steps, batch, &g, pref_variant(h));
  if (rc) return rc;
  const size_t bytes = (size_t)batch * h->c.horizon * h->c.action_dim * sizeof(float);
  HIP_TRY(h, hipMemcpyAsync(h->x, d_noise, bytes, hipMemcpyDeviceToDevice, st));
  rc = launch_pass(h, g, st);
  if (rc) return rc;
  HIP_TRY(h, hipMemcpyAsync(d_actions_out, h->x, bytes, hipMemcpyDeviceToDevice, st));
  return AE_OK;
}

int ae_denoise(ae_handle* h, int batch, const float* noise, int steps, float* actions_out) {
  int rc = check_denoise(h, batch, steps);
  if (rc) return rc;
  if (!noise || !actions_out) return fail(h, AE_ERR_INVALID_ARG, "null pointer");
  rc = failed_async(h);
  if (rc) return rc;
  const size_t bytes = (size_t)batch * h->c.horizon * h->c.action_dim * sizeof(float);
  std::vector<float> tmp(bytes / sizeof(float));
  for (int variant = pref_variant(h);; variant = 2) {
    Pass g;
    rc = get_pass(h, 0, steps, batch, &g, variant);
    if (rc) return rc;
    HIP_TRY(h, hipMemcpyAsync(h->x, noise, bytes, hipMemcpyHostToDevice, h->stream));
    HIP_TRY(h, hipEventRecord(h->ev0, h->stream));
    rc = launch_pass(h, g, h->stream);
    if (rc) return rc;
    HIP_TRY(h, hipEventRecord(h->ev1, h->stream));
    HIP_TRY(h, hipMemcpyAsync(tmp.data(), h->x, bytes, hipMemcpyDeviceToHost, h->stream));
    HIP_TRY(h, hipStreamSynchronize(h->stream));
    const bool failed = take_failure(h);
    note_fused(h, variant, batch, failed);
    if (!failed || variant == 2) break;
  }
  HIP_TRY(h, hipEventElapsedTime(&h->last_ms, h->ev0, h->ev1));
  memcpy(actions_out, tmp.data(), bytes);
  return AE_OK;
}

int ae_denoise_static(ae_handle* h, int batch, const float* d_noise, int steps, float* d_actions_out, void* stream) {
  int rc = check_denoise(h, batch, steps);
  if (rc) return rc;
  if (!d_noise || !d_actions_out) return fail(h, AE_ERR_INVALID_ARG, "null pointer");
  if (h->c.time_mode)
    return fail(h, AE_ERR_UNSUPPORTED, "a time-modulated expert builds its modulation tables per step count in "
                                       "allocated memory: use ae_denoise_async");
  if (!h->static_scratch) return fail(h, AE_ERR_HIP, h->static_err);
  const StaticLayout L = static_layout(h, batch, steps);
  if (L.total > (size_t)AE_STATIC_SCRATCH_BYTES)
    return fail(h, AE_ERR_INVALID_ARG, "batch " + std::to_string(batch) + " x " + std::to_string(steps) +
                                           " steps needs " + std::to_string(L.total) +
                                           " bytes of scratch; the static scratch holds " +
                                           std::to_string((size_t)AE_STATIC_SCRATCH_BYTES) + " (ae_denoise_async has no such limit)");
  hipStream_t st = stream ? (hipStream_t)stream : h->stream;
  Timer* tm = nullptr;
  char* base = (char*)h->static_scratch;
  PassBuffers keep(h);
  h->x = (float*)(base + L.x); h->h = (float*)(base + L.h); h->hb = base + L.hb;
  h->ssp_a = (float*)(base + L.ssp_a); h->ssp_b = (float*)(base + L.ssp_b);
  h->q = base + L.q; h->ks = base + L.ks; h->vs = base + L.vs; h->o = base + L.o; h->u = base + L.u;
  h->part = (float*)(base + L.part); h->counters = (unsigned*)(base + L.counters);
  h->opart = (float*)(base + L.opart); h->mlpart = (float*)(base + L.mlpart);
  h->qk_ssp = h->c.qk_norm ? (float*)(base + L.qk_ssp) : nullptr;
  h->phi = (float*)(base + L.phi); h->hid = (float*)(base + L.hid);
  // launches that wait for nothing inside a kernel: nothing can give up, so nothing is repeated
  h->variant = 2;
  // the previous call's contents (any handle, any size) go: padding rows and counters start at zero
  LAUNCH_CHECK(h, "static_clear", AE_LAUNCH(fill16_kernel, dim3(1024), dim3(256), 0, st, (uint4*)base, L.total / 16, 0u));
  float* t = (float*)(base + L.t);
  float* temb = (float*)(base + L.temb);
  LAUNCH_CHECK(h, "step_times", AE_LAUNCH(step_times_kernel, dim3(1), dim3(256), 0, st, t, steps));
  rc = enqueue_temb(h, t, steps, temb, st, tm);
  if (rc) return rc;
  const size_t bytes = (size_t)batch * h->c.horizon * h->c.action_dim * sizeof(float);
  HIP_TRY(h, hipMemcpyAsync(h->x, d_noise, bytes, hipMemcpyDeviceToDevice, st));
  rc = enqueue_denoise(h, batch, steps, temb, st, tm);
  if (rc) return rc;
  HIP_TRY(h, hipMemcpyAsync(d_actions_out, h->x, bytes, hipMemcpyDeviceToDevice, st));
  return AE_OK;
}

static int check_verify(ae_handle* h, int slot, int n_tau) {
  if (!h) return AE_ERR_INVALID_ARG;
  if (h->c.max_taus < 1) return fail(h, AE_ERR_UNSUPPORTED, "handle created with max_taus = 0");
  if (h->c.draft) return fail(h, AE_ERR_UNSUPPORTED, "a draft-model handle runs ae_draft only");
  if (h->c.prefill) return fail(h, AE_ERR_UNSUPPORTED, "a prefill handle runs ae_prefill only");
  if (n_tau < 1 || n_tau > h->c.max_taus) return fail(h, AE_ERR_INVALID_ARG, "n_tau out of range");
  if (slot < 0 || slot >= h->c.max_batch) return fail(h, AE_ERR_INVALID_ARG, "slot out of range");
  if (!h->slot_ready[slot]) return fail(h, AE_ERR_NOT_READY, "prefix slot not loaded");
  return AE_OK;
}

static int verify_common(ae_handle* h, int slot, int n_tau, float delta, hipStream_t st, hipMemcpyKind kind,
                         const float* draft, const float* noise, const float* taus) {
  const size_t ha = (size_t)h->c.horizon * h->c.action_dim * sizeof(float);
  HIP_TRY(h, hipMemcpyAsync(h->draft, draft, ha, kind, st));
  HIP_TRY(h, hipMemcpyAsync(h->vnoise, noise, ha, kind, st));
  HIP_TRY(h, hipMemcpyAsync(h->taus, taus, n_tau * sizeof(float), kind, st));
  hipLaunchKernelGGL(set_verify_params_kernel, dim3(1), dim3(64), 0, st, h->verify_slots, n_tau, slot, h->params, delta);
  HIP_TRY(h, hipGetLastError());
  h->last_verify_slot = slot;
  h->last_delta = delta;
  return AE_OK;
}

int ae_verify_async(ae_handle* h, int slot, const float* d_draft, const float* d_noise, const float* d_taus, int n_tau,
                    float delta, int* d_accept_len, int* d_gripper_switch, float* d_dist_out, void* stream) {
  int rc = check_verify(h, slot, n_tau);
  if (rc) return rc;
  if (!d_draft || !d_noise || !d_taus || !d_accept_len || !d_gripper_switch) return fail(h, AE_ERR_INVALID_ARG, "null pointer");
  rc = failed_async(h);
  if (rc) return rc;
  hipStream_t st = stream ? (hipStream_t)stream : h->stream;
  Pass g;
  rc = get_pass(h, 1, n_tau, 1, &g, pref_variant(h));
  if (rc) return rc;
  rc = verify_common(h, slot, n_tau, delta, st, hipMemcpyDeviceToDevice, d_draft, d_noise, d_taus);
  if (rc) return rc;
  rc = launch_pass(h, g, st);
  if (rc) return rc;
  HIP_TRY(h, hipMemcpyAsync(d_accept_len, h->accept, sizeof(int), hipMemcpyDeviceToDevice, st));
  HIP_TRY(h, hipMemcpyAsync(d_gripper_switch, h->gswitch, sizeof(int), hipMemcpyDeviceToDevice, st));
  if (d_dist_out)
    HIP_TRY(h, hipMemcpyAsync(d_dist_out, h->dist, (size_t)n_tau * h->c.horizon * sizeof(float), hipMemcpyDeviceToDevice, st));
  return AE_OK;
}

// The verification pass on the library's stream, repeated with no in-kernel waits if a wait gave up;
// the inputs are on the device already (verify_common). Reads back the decision (and D).
static int run_verify(ae_handle* h, int n_tau, int* acc, int* sw, float* dist) {
  for (int variant = pref_variant(h);; variant = 2) {
    Pass g;
    int rc = get_pass(h, 1, n_tau, 1, &g, variant);
    if (rc) return rc;
    HIP_TRY(h, hipEventRecord(h->ev0, h->stream));
    rc = launch_pass(h, g, h->stream);
    if (rc) return rc;
    HIP_TRY(h, hipEventRecord(h->ev1, h->stream));
    HIP_TRY(h, hipMemcpyAsync(acc, h->accept, sizeof(int), hipMemcpyDeviceToHost, h->stream));
    HIP_TRY(h, hipMemcpyAsync(sw, h->gswitch, sizeof(int), hipMemcpyDeviceToHost, h->stream));
    if (dist) HIP_TRY(h, hipMemcpyAsync(dist, h->dist, (size_t)n_tau * h->c.horizon * sizeof(float), hipMemcpyDeviceToHost, h->stream));
    HIP_TRY(h, hipStreamSynchronize(h->stream));
    if (!take_failure(h) || variant == 2) return AE_OK;
  }
}

int ae_verify(ae_handle* h, int slot, const float* draft, const float* noise, const float* taus, int n_tau, float delta,
              int* accept_len, int* gripper_switch, float* dist_out) {
  int rc = check_verify(h, slot, n_tau);
  if (rc) return rc;
  if (!draft || !noise || !taus || !accept_len || !gripper_switch) return fail(h, AE_ERR_INVALID_ARG, "null pointer");
  for (int j = 0; j < n_tau; ++j)
    if (!(taus[j] >= 0.f && taus[j] < 1.f)) return fail(h, AE_ERR_INVALID_ARG, "tau must lie in [0, 1)");
  rc = failed_async(h);
  if (rc) return rc;
  rc = verify_common(h, slot, n_tau, delta, h->stream, hipMemcpyHostToDevice, draft, noise, taus);
  if (rc) return rc;
  int acc = 0, sw = 0;
  std::vector<float> d((size_t)n_tau * h->c.horizon);
  rc = run_verify(h, n_tau, &acc, &sw, d.data());
  if (rc) return rc;
  HIP_TRY(h, hipEventElapsedTime(&h->last_ms, h->ev0, h->ev1));
  *accept_len = acc;
  *gripper_switch = sw;
  if (dist_out) memcpy(dist_out, d.data(), d.size() * sizeof(float));
  return AE_OK;
}

int ae_round(ae_handle* h, int slot, const float* draft, const float* noise_verify, const float* taus, int n_tau,
             float delta, const float* noise_full, int steps, float* actions_out, int* accept_len, int* gripper_switch,
             int* full_path) {
  int rc = check_verify(h, slot, n_tau);
  if (rc) return rc;
  if (steps < 1 || steps > 1000) return fail(h, AE_ERR_INVALID_ARG, "steps out of range (1..1000)");
  if (!draft || !noise_verify || !taus || !noise_full || !actions_out || !accept_len || !gripper_switch || !full_path)
    return fail(h, AE_ERR_INVALID_ARG, "null pointer");
  for (int j = 0; j < n_tau; ++j)
    if (!(taus[j] >= 0.f && taus[j] < 1.f)) return fail(h, AE_ERR_INVALID_ARG, "tau must lie in [0, 1)");
  rc = failed_async(h);
  if (rc) return rc;
  // both graphs exist before the round starts (the first round of a shape captures them)
  Pass gv, gd;
  const int var = pref_variant(h);
  rc = get_pass(h, 1, n_tau, 1, &gv, var);
  if (rc) return rc;
  rc = slot == 0 ? get_pass(h, 0, steps, 1, &gd, var) : get_pass(h, 2, steps, slot, &gd, var);
  if (rc) return rc;
  rc = verify_common(h, slot, n_tau, delta, h->stream, hipMemcpyHostToDevice, draft, noise_verify, taus);
  if (rc) return rc;
  const size_t ha = (size_t)h->c.horizon * h->c.action_dim * sizeof(float);
  // fast path: the verification pass, then the host reads the decision
  int acc = 0, sw = 0;
  HIP_TRY(h, hipEventRecord(h->ev_round, h->stream));
  rc = run_verify(h, n_tau, &acc, &sw, nullptr);
  if (rc) return rc;
  // an empty accepted prefix (a gripper switch forces it) falls back to the full denoise loop
  const int full = acc == 0;
  std::vector<float> out(ha / sizeof(float));
  if (full) {
    for (int variant = var;; variant = 2) {
      if (variant != var) {
        rc = slot == 0 ? get_pass(h, 0, steps, 1, &gd, variant) : get_pass(h, 2, steps, slot, &gd, variant);
        if (rc) return rc;
      }
      HIP_TRY(h, hipMemcpyAsync(h->x, noise_full, ha, hipMemcpyHostToDevice, h->stream));
      HIP_TRY(h, hipEventRecord(h->ev0, h->stream));
      rc = launch_pass(h, gd, h->stream);
      if (rc) return rc;
      HIP_TRY(h, hipEventRecord(h->ev1, h->stream));
      HIP_TRY(h, hipMemcpyAsync(out.data(), h->x, ha, hipMemcpyDeviceToHost, h->stream));
      HIP_TRY(h, hipStreamSynchronize(h->stream));
      const bool failed = take_failure(h);
      note_fused(h, variant, 1, failed);
      if (!failed || variant == 2) break;
    }
  } else {
    memcpy(out.data(), draft, ha);
  }
  // the round on the device timeline: verification, the host decision and the full pass if any
  HIP_TRY(h, hipEventElapsedTime(&h->last_ms, h->ev_round, h->ev1));
  memcpy(actions_out, out.data(), ha);
  *accept_len = acc;
  *gripper_switch = sw;
  *full_path = full;
  return AE_OK;
}

int ae_draft(ae_handle* h, const float* features, float* chunk_out) {
  if (!h) return AE_ERR_INVALID_ARG;
  if (!h->c.draft) return fail(h, AE_ERR_UNSUPPORTED, "not a draft-model handle (ae_config.draft = 0)");
  if (!features || !chunk_out) return fail(h, AE_ERR_INVALID_ARG, "null pointer");
  int rc = failed_async(h);
  if (rc) return rc;
  const ae_config& c = h->c;
  const size_t bytes = (size_t)c.horizon * c.action_dim * sizeof(float);
  std::vector<float> tmp(bytes / sizeof(float));
  for (int variant = 0;; variant = 2) {
    Pass g;
    rc = get_pass(h, 3, 0, 0, &g, variant);
    if (rc) return rc;
    HIP_TRY(h, hipMemcpyAsync(h->feat, features, (size_t)c.prefix_len * c.width * 4, hipMemcpyHostToDevice, h->stream));
    HIP_TRY(h, hipEventRecord(h->ev0, h->stream));
    rc = launch_pass(h, g, h->stream);
    if (rc) return rc;
    HIP_TRY(h, hipEventRecord(h->ev1, h->stream));
    HIP_TRY(h, hipMemcpyAsync(tmp.data(), h->vout, bytes, hipMemcpyDeviceToHost, h->stream));
    HIP_TRY(h, hipStreamSynchronize(h->stream));
    if (!take_failure(h) || variant == 2) break;
  }
  HIP_TRY(h, hipEventElapsedTime(&h->last_ms, h->ev0, h->ev1));
  h->slot_ready[0] = 1;
  memcpy(chunk_out, tmp.data(), bytes);
  return AE_OK;
}

// The prefill stack's pass over host embeddings emb, on the library's stream, repeated with no
// in-kernel waits if a wait gave up; every layer's K/V is then in pf_k / pf_v.
static int run_prefill(ae_handle* h, const float* emb) {
  const ae_config& c = h->c;
  for (int variant = 0;; variant = 2) {
    Pass g;
    int rc = get_pass(h, 4, 0, 0, &g, variant);
    if (rc) return rc;
    HIP_TRY(h, hipMemcpyAsync(h->feat, emb, (size_t)c.horizon * c.width * 4, hipMemcpyHostToDevice, h->stream));
    HIP_TRY(h, hipEventRecord(h->ev0, h->stream));
    rc = launch_pass(h, g, h->stream);
    if (rc) return rc;
    HIP_TRY(h, hipEventRecord(h->ev1, h->stream));
    HIP_TRY(h, hipStreamSynchronize(h->stream));
    if (!take_failure(h) || variant == 2) break;
  }
  HIP_TRY(h, hipEventElapsedTime(&h->last_ms, h->ev0, h->ev1));
  return AE_OK;
}

int ae_prefill_to_slot(ae_handle* h, const float* emb, ae_handle* expert, int slot) {
  if (!h || !expert) return AE_ERR_INVALID_ARG;
  if (!h->c.prefill) return fail(h, AE_ERR_UNSUPPORTED, "not a prefill handle (ae_config.prefill = 0)");
  if (!emb) return fail(h, AE_ERR_INVALID_ARG, "null pointer");
  const ae_config& c = h->c;
  const ae_config& e = expert->c;
  if (expert->c.prefill || expert->c.draft) return fail(h, AE_ERR_UNSUPPORTED, "the target is not an expert handle");
  if (slot < 0 || slot >= e.max_batch) return fail(h, AE_ERR_INVALID_ARG, "slot out of range");
  if (e.prefix_len != c.horizon || e.n_layers != c.n_layers || e.n_kv_heads != c.n_kv_heads ||
      e.head_dim != c.head_dim || e.kv_dtype != c.kv_dtype || expert->dev != h->dev)
    return fail(h, AE_ERR_UNSUPPORTED,
                "expert prefix_len, n_layers, n_kv_heads, head_dim, kv_dtype and device must match the prefill stack");
  // the two layouts coincide: [L][n_kv][32-key blocks][block fragments], ceil(P/32) blocks, keys
  // past P zero in both (never written here, zeroed at allocation)
  const size_t bytes = expert->slot_elems * dtype_size(e.kv_dtype);
  if (bytes != (size_t)c.n_layers * h->pf_layer_elems * dtype_size(c.kv_dtype))
    return fail(h, AE_ERR_UNSUPPORTED, "cache layouts differ");
  int rc = failed_async(h);
  if (rc) return rc;
  rc = run_prefill(h, emb);
  if (rc) return rc;
  HIP_TRY(h, hipMemcpyAsync((char*)expert->kcache + slot * bytes, h->pf_k, bytes, hipMemcpyDeviceToDevice, h->stream));
  HIP_TRY(h, hipMemcpyAsync((char*)expert->vcache + slot * bytes, h->pf_v, bytes, hipMemcpyDeviceToDevice, h->stream));
  HIP_TRY(h, hipStreamSynchronize(h->stream));
  expert->slot_ready[slot] = 1;
  return AE_OK;
}

int ae_prefill(ae_handle* h, const float* emb, void* k_out, void* v_out) {
  if (!h) return AE_ERR_INVALID_ARG;
  if (!h->c.prefill) return fail(h, AE_ERR_UNSUPPORTED, "not a prefill handle (ae_config.prefill = 0)");
  if (!emb || !k_out || !v_out) return fail(h, AE_ERR_INVALID_ARG, "null pointer");
  int rc = failed_async(h);
  if (rc) return rc;
  const ae_config& c = h->c;
  const int L = c.n_layers, P = c.horizon, nkv = c.n_kv_heads, dh = c.head_dim, nkb = dh / 32, nbs = h->nbs;
  const size_t es = dtype_size(c.kv_dtype), all = (size_t)L * h->pf_layer_elems * es;
  rc = run_prefill(h, emb);
  if (rc) return rc;
  std::vector<unsigned char> kp(all), vp(all);
  HIP_TRY(h, hipMemcpy(kp.data(), h->pf_k, all, hipMemcpyDeviceToHost));
  HIP_TRY(h, hipMemcpy(vp.data(), h->pf_v, all, hipMemcpyDeviceToHost));
  // from the cache blocks' fragment order back to [L][P][n_kv][dh] (the inverse of ae_load_prefix_kv)
  unsigned char* ko = (unsigned char*)k_out;
  unsigned char* vo = (unsigned char*)v_out;
  for (int l = 0; l < L; ++l)
    for (int j = 0; j < P; ++j)
      for (int g2 = 0; g2 < nkv; ++g2) {
        const size_t blk = (size_t)l * h->pf_layer_elems + ((size_t)g2 * nbs + j / 32) * 32 * dh;
        const int kk = j % 32, kt = (kk & 7) >> 2, m = 4 * (kk >> 3) + (kk & 3);
        const size_t drow = (((size_t)l * P + j) * nkv + g2) * dh;
        for (int d = 0; d < dh; ++d) {
          const size_t kidx = blk + ((size_t)(kt * nkb + d / 32) * 64 + ((d % 32) / 8) * 16 + m) * 8 + (d & 7);
          const size_t vidx = blk + ((size_t)(d / 16) * 64 + (kk / 8) * 16 + (d & 15)) * 8 + (kk & 7);
          memcpy(ko + (drow + d) * es, &kp[kidx * es], es);
          memcpy(vo + (drow + d) * es, &vp[vidx * es], es);
        }
      }
  return AE_OK;
}

void ae_destroy(ae_handle* h) {
  if (!h) return;
  if (h->stream) hipStreamSynchronize(h->stream);
  for (auto& kv : h->graphs) hipGraphExecDestroy(kv.second);
  for (void* p : h->allocs) hipFree(p);
  if (h->flag_host) hipHostFree(h->flag_host);
  if (h->ev0) hipEventDestroy(h->ev0);
  if (h->ev1) hipEventDestroy(h->ev1);
  if (h->ev_round) hipEventDestroy(h->ev_round);
  if (h->stream) hipStreamDestroy(h->stream);
  delete h;
}

const char* ae_last_error(const ae_handle* h) { return h ? h->err.c_str() : g_create_error.c_str(); }

int ae_last_gpu_ms(const ae_handle* h, float* ms) {
  if (!h || !ms) return AE_ERR_INVALID_ARG;
  *ms = h->last_ms;
  return AE_OK;
}

}  // extern "C"

namespace {
// The pass launched eagerly in its normal order (so each kernel sees the cache
// state and neighbours it has inside the graph), with a start/stop event pair
// bound to every dispatch: the kernel's own execution time, summed per name
// over `iters` passes.
template <class Enq>
int kernel_times_in_place(ae_handle* h, Enq& enqueue, const std::vector<std::string>& names, int iters,
                          ae_kernel_stat* stats, int max_stats, int* n_stats) {
  // count the pass's launches: a capture that is never instantiated
  int n_launch = 0;
  {
    Timer probe;
    HIP_TRY(h, hipStreamBeginCapture(h->stream, hipStreamCaptureModeThreadLocal));
    int rc = enqueue(&probe);
    hipGraph_t g0 = nullptr;
    hipError_t e = hipStreamEndCapture(h->stream, &g0);
    if (g0) hipGraphDestroy(g0);
    if (rc) return rc;
    if (e != hipSuccess) return fail(h, AE_ERR_HIP, std::string("in-place timing (launch count): ") + hipGetErrorString(e));
    n_launch = probe.count;
  }
  std::vector<hipEvent_t> ev;
  auto cleanup = [&]() { for (hipEvent_t x : ev) hipEventDestroy(x); };
  hipError_t e = hipSuccess;
  ev.reserve(2 * (size_t)n_launch);
  for (int i = 0; i < 2 * n_launch && e == hipSuccess; ++i) {
    hipEvent_t x;
    e = hipEventCreate(&x);
    if (e == hipSuccess) ev.push_back(x);
  }
  if (e != hipSuccess) { cleanup(); return fail(h, AE_ERR_HIP, std::string("in-place timing events: ") + hipGetErrorString(e)); }
  std::vector<double> tot(names.size(), 0.0);
  std::vector<int> cnt(names.size(), 0);
  for (int it = 0; it <= iters && e == hipSuccess; ++it) {  // pass 0 warms up
    Timer tm;
    tm.pairs = &ev;
    int rc = enqueue(&tm);
    t_dispatch_ev = DispatchEvents{};
    if (rc) { hipStreamSynchronize(h->stream); cleanup(); return rc; }
    if (tm.overflow) { hipStreamSynchronize(h->stream); cleanup(); return fail(h, AE_ERR_HIP, "in-place timing: launch count changed"); }
    e = hipStreamSynchronize(h->stream);
    for (size_t i = 0; i < tm.launched.size() && e == hipSuccess && it > 0; ++i) {
      float ms = 0.f;
      e = hipEventElapsedTime(&ms, ev[2 * i], ev[2 * i + 1]);
      size_t k = std::find(names.begin(), names.end(), tm.launched[i]) - names.begin();
      if (e == hipSuccess && k < names.size()) { tot[k] += ms; ++cnt[k]; }
    }
  }
  cleanup();
  if (e != hipSuccess) return fail(h, AE_ERR_HIP, std::string("in-place timing: ") + hipGetErrorString(e));
  int n = 0;
  for (size_t k = 0; k < names.size() && n < max_stats; ++k) {
    memset(stats[n].name, 0, sizeof(stats[n].name));
    strncpy(stats[n].name, names[k].c_str(), sizeof(stats[n].name) - 1);
    stats[n].launches = cnt[k];
    stats[n].total_ms = (float)tot[k];
    ++n;
  }
  *n_stats = n;
  return AE_OK;
}
}  // namespace

static int kernel_times_impl(ae_handle* h, int mode, int batch, int steps, int iters, ae_kernel_stat* stats,
                             int max_stats, int* n_stats) {
  const bool in_place = (mode & 2) != 0;
  mode &= 1;
  int rc;
  if (mode == 0) {
    rc = check_denoise(h, batch, steps);
    if (rc) return rc;
  } else {
    rc = check_verify(h, h->last_verify_slot, batch);
    if (rc) return rc;
  }
  float* temb = nullptr;
  if (mode == 0) { rc = get_temb_steps(h, steps, &temb); if (rc) return rc; }
  h->variant = pref_variant(h);
  auto enqueue = [&](Timer* tm) {
    return mode == 0 ? enqueue_denoise(h, batch, steps, temb, h->stream, tm) : enqueue_verify(h, batch, h->stream, tm);
  };
  // kernel names in launch order: a pass under capture that launches nothing
  std::vector<std::string> names;
  {
    Timer probe;
    probe.only = "\x01";
    HIP_TRY(h, hipStreamBeginCapture(h->stream, hipStreamCaptureModeThreadLocal));
    rc = enqueue(&probe);
    hipGraph_t g0 = nullptr;
    hipError_t e = hipStreamEndCapture(h->stream, &g0);
    if (g0) hipGraphDestroy(g0);
    if (rc) return rc;
    if (e != hipSuccess) return fail(h, AE_ERR_HIP, std::string("kernel timing capture: ") + hipGetErrorString(e));
    names = probe.seen;
  }
  if (in_place) return kernel_times_in_place(h, enqueue, names, iters, stats, max_stats, n_stats);
  // per kernel: one graph holding every launch of that kernel in the pass, back to back,
  // replayed `iters` times between two HIP events on the library's stream
  int n = 0;
  for (const std::string& nm : names) {
    if (n >= max_stats) break;
    Timer tm;
    tm.only = nm;
    HIP_TRY(h, hipStreamBeginCapture(h->stream, hipStreamCaptureModeThreadLocal));
    rc = enqueue(&tm);
    hipGraph_t g = nullptr;
    hipError_t e = hipStreamEndCapture(h->stream, &g);
    if (rc) { if (g) hipGraphDestroy(g); return rc; }
    if (e != hipSuccess) return fail(h, AE_ERR_HIP, std::string("kernel timing capture: ") + hipGetErrorString(e));
    hipGraphExec_t ge = nullptr;
    e = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
    hipGraphDestroy(g);
    if (e != hipSuccess) return fail(h, AE_ERR_HIP, std::string("kernel timing instantiate: ") + hipGetErrorString(e));
    float ms = 0.f;
    e = hipGraphLaunch(ge, h->stream);
    if (e == hipSuccess) e = hipEventRecord(h->ev0, h->stream);
    for (int it = 0; it < iters && e == hipSuccess; ++it) e = hipGraphLaunch(ge, h->stream);
    if (e == hipSuccess) e = hipEventRecord(h->ev1, h->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(h->stream);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, h->ev0, h->ev1);
    hipGraphExecDestroy(ge);
    if (e != hipSuccess) return fail(h, AE_ERR_HIP, std::string("kernel timing: ") + hipGetErrorString(e));
    memset(stats[n].name, 0, sizeof(stats[n].name));
    strncpy(stats[n].name, nm.c_str(), sizeof(stats[n].name) - 1);
    stats[n].launches = tm.count * iters;
    stats[n].total_ms = ms;
    ++n;
  }
  *n_stats = n;
  return AE_OK;
}

extern "C" {

int ae_kernel_times(ae_handle* h, int mode, int batch, int steps, int iters, ae_kernel_stat* stats, int max_stats,
                    int* n_stats) {
  if (!h || !stats || !n_stats || iters < 1 || mode < 0 || mode > 3) return AE_ERR_INVALID_ARG;
  const int rc = kernel_times_impl(h, mode, batch, steps, iters, stats, max_stats, n_stats);
  // a graph of one kernel's launches alone can leave partials that no launch consumed
  hipStreamSynchronize(h->stream);
  const int rc2 = reset_exchange(h);
  return rc ? rc : rc2;
}


}  // extern "C"
