// Host-side parts of the library that touch no device: the config and weight checks of ae_create, the
// row tables and the packing of weight matrices into MFMA fragment order, and the repacking of a prefix
// K/V cache into the attention's block layout. Plain C++ (no HIP), so that a host build with address
// and undefined-behaviour sanitizers can run it.
#pragma once
#include <cstddef>
#include <cstring>
#include <string>
#include <algorithm>
#include <vector>

#include "../../include/ae.h"

namespace ae_host {

inline size_t dtype_size(int dt) { return dt == AE_F32 ? 4 : dt == AE_BF16 ? 2 : 1; }

// AE_OK, or the error code of the first violated condition with its description in why.
inline int validate_config(const ae_config* c, const ae_weights* w, std::string& why) {
  auto fail = [&why](int code, const char* msg) {
    why = msg;
    return code;
  };
  if (!c || !w) return fail(AE_ERR_INVALID_ARG, "null config or weights");
  if (c->n_layers < 1 || c->width <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
      c->mlp_dim <= 0 || c->action_dim <= 0 || c->horizon <= 0 || c->prefix_len < 0 || c->max_batch < 1 ||
      c->max_taus < 0 || c->max_taus > 64 || !(c->rms_eps >= 0.f) || !(c->rope_base > 0.f))
    return fail(AE_ERR_INVALID_ARG, "non-positive size in ae_config");
  // bounds that keep every size product below are far inside int and size_t
  if (c->n_layers > 1024 || c->width > 65536 || c->n_q_heads > 1024 || c->n_kv_heads > 1024 || c->mlp_dim > (1 << 20) ||
      c->action_dim > 65536 || c->horizon > 65536 || c->prefix_len > (1 << 20) || c->max_batch > 4096)
    return fail(AE_ERR_UNSUPPORTED, "size beyond the library's range (layers <= 1024, width <= 65536, heads <= 1024, "
                                    "mlp_dim <= 2^20, prefix_len <= 2^20, max_batch <= 4096)");
  if (c->n_q_heads % c->n_kv_heads) return fail(AE_ERR_INVALID_ARG, "n_kv_heads must divide n_q_heads");
  if (c->gripper_dim >= c->action_dim || c->gripper_dim < -1) return fail(AE_ERR_INVALID_ARG, "gripper_dim out of range");
  for (int d : {c->weight_dtype, c->mlp_dtype, c->kv_dtype})
    if (d != AE_F32 && d != AE_BF16 && d != AE_FP8_E4M3) return fail(AE_ERR_INVALID_ARG, "unknown dtype");
  if (c->width % 256 || (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256) ||
      c->mlp_dim % 256 || (c->n_q_heads * c->head_dim) % 256)
    return fail(AE_ERR_UNSUPPORTED,
                "width, mlp_dim and n_q_heads*head_dim must be multiples of 256; head_dim one of 32, 64, 128, 256");
  if (c->action_dim > 64 || c->horizon > (c->prefill == 1 ? 1024 : 256))
    return fail(AE_ERR_UNSUPPORTED, "action_dim <= 64 and horizon <= 256 (prefill: <= 1024 tokens)");
  if (c->weight_dtype == AE_FP8_E4M3) return fail(AE_ERR_UNSUPPORTED, "fp8 is supported for the MLP only");
  if (c->kv_dtype != c->weight_dtype) return fail(AE_ERR_UNSUPPORTED, "kv_dtype must equal weight_dtype");
  if (c->weight_dtype == AE_F32 && c->mlp_dtype != AE_F32)
    return fail(AE_ERR_UNSUPPORTED, "fp32 attention weights need fp32 MLP weights");
  if (c->weight_dtype == AE_BF16 && c->mlp_dtype == AE_F32)
    return fail(AE_ERR_UNSUPPORTED, "bf16 attention weights need bf16 or fp8 MLP weights");
  if (c->draft != 0 && c->draft != 1) return fail(AE_ERR_INVALID_ARG, "draft is 0 or 1");
  if (c->prefill != 0 && c->prefill != 1) return fail(AE_ERR_INVALID_ARG, "prefill is 0 or 1");
  if (c->prefill) {
    if (c->draft || c->prefix_len != 0 || c->max_batch != 1 || c->max_taus != 0 || c->time_mode || c->qk_norm ||
        c->weight_dtype != AE_BF16 || c->mlp_dtype == AE_F32)
      return fail(AE_ERR_UNSUPPORTED,
                  "a prefill stack has prefix_len 0, max_batch 1, max_taus 0, bf16 attention weights, no modulation or QK-norm");
    if (!w->layers) return fail(AE_ERR_INVALID_ARG, "null weight pointer");
  } else if (c->draft) {
    if (c->n_layers != 1 || c->max_batch != 1 || c->max_taus != 0 || c->time_mode || c->qk_norm ||
        c->weight_dtype != AE_BF16 || c->mlp_dtype != AE_BF16 || c->prefix_len < 1)
      return fail(AE_ERR_UNSUPPORTED,
                  "a draft model has 1 layer, max_batch 1, max_taus 0, bf16 weights, no modulation or QK-norm, prefix_len >= 1");
    if (!w->queries || !w->layers || !w->final_ln || !w->action_out_w || !w->action_out_b)
      return fail(AE_ERR_INVALID_ARG, "null weight pointer");
  } else if (!w->time_in_w || !w->time_in_b || !w->time_out_w || !w->time_out_b || !w->action_in_w || !w->action_in_b ||
             !w->layers || !w->final_ln || !w->action_out_w || !w->action_out_b) {
    return fail(AE_ERR_INVALID_ARG, "null weight pointer");
  }
  if ((c->time_mode != 0 && c->time_mode != 1) || (c->qk_norm != 0 && c->qk_norm != 1))
    return fail(AE_ERR_INVALID_ARG, "time_mode and qk_norm are 0 or 1");
  if ((c->time_mode || c->qk_norm) && (c->weight_dtype != AE_BF16 || c->mlp_dtype != AE_BF16))
    return fail(AE_ERR_UNSUPPORTED, "time modulation and QK-norm are built for bf16 weights and MLP");
  if (c->time_mode && (!w->final_mod_w || !w->final_mod_b))
    return fail(AE_ERR_INVALID_ARG, "time_mode 1 needs final_mod_w and final_mod_b");
  for (int l = 0; l < c->n_layers; ++l) {
    const ae_layer_weights& L = w->layers[l];
    if (!L.ln1 || !L.wq || !L.wk || !L.wv || !L.wo || !L.ln2 || !L.wg || !L.wu || !L.wd)
      return fail(AE_ERR_INVALID_ARG, "null layer weight pointer");
    if (c->mlp_dtype == AE_FP8_E4M3 && (!L.wg_scale || !L.wu_scale || !L.wd_scale))
      return fail(AE_ERR_INVALID_ARG, "fp8 MLP needs per-row scales");
    if (c->time_mode && (!L.w_mod || !L.b_mod)) return fail(AE_ERR_INVALID_ARG, "time_mode 1 needs w_mod and b_mod");
    if (c->qk_norm && (!L.q_norm || !L.k_norm)) return fail(AE_ERR_INVALID_ARG, "qk_norm 1 needs q_norm and k_norm");
  }
  return AE_OK;
}



// Pack rows (row_ptr[p] = first byte of packed channel p's K inputs, or null for a zero row) of elements
// of es bytes into [tiles][K/32][64 lanes][8]: lane (k % 32 / 8) * 16 + (channel % 16) of k-block k / 32
// holds inputs k .. k + 7 of its channel (the MFMA A-operand order of a 16 x 32 tile).
inline void pack_rows(const std::vector<const unsigned char*>& row_ptr, int K, size_t es, std::vector<unsigned char>& out) {
  const int tiles = (int)row_ptr.size() / 16, KB = K / 32;
  out.assign((size_t)tiles * KB * 64 * 8 * es, 0);
  for (int t = 0; t < tiles; ++t)
    for (int kb = 0; kb < KB; ++kb)
      for (int lane = 0; lane < 64; ++lane) {
        const unsigned char* src = row_ptr[(size_t)t * 16 + (lane & 15)];
        unsigned char* dst = out.data() + (((size_t)t * KB + kb) * 64 + lane) * 8 * es;
        if (src) memcpy(dst, src + ((size_t)kb * 32 + (lane >> 4) * 8) * es, 8 * es);
      }
}

// Head-dim order of the packed q / k tiles: tile p of a head holds dims p*8 .. p*8+7 and their RoPE
// partners dh/2 + p*8 .. (channel cc of the tile -> dim), so one tile carries both halves of each pair.
inline int rope_tile_dim(int dh, int p, int cc) { return cc < 8 ? p * 8 + cc : dh / 2 + p * 8 + (cc - 8); }

// Row tables of the packed QKV weights ([nq heads of q tiles][nkv heads of k tiles][v rows]), the
// o_proj, the gate/up (16-row gate and up tiles interleaved) and the down weights; es bytes per element.
inline std::vector<const unsigned char*> qkv_rows(const void* wq, const void* wk, const void* wv, int nq, int nkv, int dh,
                                                 int w, size_t es) {
  std::vector<const unsigned char*> rows;
  rows.reserve((size_t)(nq + 2 * nkv) * dh);
  auto head_rows = [&](const void* base, int nh) {
    for (int hh = 0; hh < nh; ++hh)
      for (int p = 0; p < dh / 16; ++p)
        for (int cc = 0; cc < 16; ++cc)
          rows.push_back((const unsigned char*)base + ((size_t)hh * dh + rope_tile_dim(dh, p, cc)) * w * es);
  };
  head_rows(wq, nq);
  head_rows(wk, nkv);
  for (int r = 0; r < nkv * dh; ++r) rows.push_back((const unsigned char*)wv + (size_t)r * w * es);
  return rows;
}
inline std::vector<const unsigned char*> plain_rows(const void* wm, int n_rows, int K, size_t es, int padded_rows = 0) {
  std::vector<const unsigned char*> rows(std::max(n_rows, padded_rows), nullptr);
  for (int r = 0; r < n_rows; ++r) rows[r] = (const unsigned char*)wm + (size_t)r * K * es;
  return rows;
}
inline std::vector<const unsigned char*> gate_up_rows(const void* wg, const void* wu, int F, int w, size_t es) {
  std::vector<const unsigned char*> rows;
  rows.reserve((size_t)2 * F);
  for (int j = 0; j < F / 16; ++j) {
    for (int cc = 0; cc < 16; ++cc) rows.push_back((const unsigned char*)wg + ((size_t)j * 16 + cc) * w * es);
    for (int cc = 0; cc < 16; ++cc) rows.push_back((const unsigned char*)wu + ((size_t)j * 16 + cc) * w * es);
  }
  return rows;
}

// One robot's prefix cache (host [L][P][nkv][dh], es bytes per element) in the attention's block layout:
// per layer and kv head, nbp blocks of 32 keys; in a block, K as two 16-key halves of MFMA A fragments
// ([kt][dh/32][64][8], key 8 (m/4) + 4 kt + m % 4 on lane row m) and V as B fragments over keys
// ([dh/16][64][8], 8 keys per lane). Keys past P stay zero. kp and vp receive L*nkv*nbp*32*dh elements.
inline void repack_prefix_kv(const unsigned char* ksrc, const unsigned char* vsrc, int L, int P, int nkv, int dh, int nbp,
                             size_t es, std::vector<unsigned char>& kp, std::vector<unsigned char>& vp) {
  const size_t elems = (size_t)L * nkv * nbp * 32 * dh;
  kp.assign(elems * es, 0);
  vp.assign(elems * es, 0);
  const int nkb = dh / 32;
  for (int l = 0; l < L; ++l)
    for (int j = 0; j < P; ++j)
      for (int g = 0; g < nkv; ++g) {
        const size_t blk = (((size_t)l * nkv + g) * nbp + j / 32) * 32 * dh;  // block base (elements)
        const int kk = j % 32, kt = (kk & 7) >> 2, m = 4 * (kk >> 3) + (kk & 3);
        const size_t srow = (((size_t)l * P + j) * nkv + g) * dh;
        for (int d = 0; d < dh; ++d) {
          const size_t kidx = blk + ((size_t)(kt * nkb + d / 32) * 64 + ((d % 32) / 8) * 16 + m) * 8 + (d & 7);
          const size_t vidx = blk + ((size_t)(d / 16) * 64 + (kk / 8) * 16 + (d & 15)) * 8 + (kk & 7);
          memcpy(&kp[kidx * es], ksrc + (srow + d) * es, es);
          memcpy(&vp[vidx * es], vsrc + (srow + d) * es, es);
        }
      }
}

}  // namespace ae_host
