// Host code of libae (config checks, weight packing, prefix-cache repacking: csrc/ae_host.hpp) run under
// AddressSanitizer and UndefinedBehaviorSanitizer on varied shapes, each result checked against the
// operand layouts it must produce:
//   - v_mfma_f32_16x16x32_bf16's A operand: lane l of a 16 x 32 tile holds row l % 16, inputs
//     (l / 16) * 8 .. + 7 of the 32 (pack_rows, row tables of QKV / gate-up);
//   - RoPE pairs (d, d + dh/2) in one packed q/k tile (qkv_rows);
//   - the attention's K block: A fragments of 16 keys (key 8 (m / 4) + 4 kt + m % 4 on row m), and
//     its V block: B fragments holding 8 consecutive keys per lane (repack_prefix_kv);
//   - validate_config's codes for configs the library covers, rejects, or could overflow on.
// Prints "ok" and exits 0, or names the first mismatch and exits 1.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>

#include "../../flow_matching_action_euler_amd/csrc/ae_host.hpp"

static int g_fail = 0;
#define CHECK(cond, ...)                   \
  do {                                     \
    if (!(cond)) {                         \
      if (!g_fail) printf(__VA_ARGS__);    \
      g_fail = 1;                          \
    }                                      \
  } while (0)

static void check_pack_rows(std::mt19937& rng) {
  for (int it = 0; it < 40; ++it) {
    const int tiles = 1 + (int)(rng() % 4), KB = 1 + (int)(rng() % 5), K = KB * 32;
    const size_t es = (size_t)1 << (rng() % 3);
    std::vector<std::vector<unsigned char>> src(tiles * 16);
    std::vector<const unsigned char*> rows(tiles * 16, nullptr);
    for (int r = 0; r < tiles * 16; ++r) {
      if (rng() % 7 == 0) continue;  // a zero row
      src[r].resize(K * es);
      for (auto& b : src[r]) b = (unsigned char)(1 + rng() % 255);
      rows[r] = src[r].data();
    }
    std::vector<unsigned char> out;
    ae_host::pack_rows(rows, K, es, out);
    CHECK(out.size() == (size_t)tiles * KB * 64 * 8 * es, "pack_rows size\n");
    for (int t = 0; t < tiles; ++t)
      for (int kb = 0; kb < KB; ++kb)
        for (int lane = 0; lane < 64; ++lane)
          for (int j = 0; j < 8; ++j) {
            const int row = t * 16 + lane % 16, k = kb * 32 + (lane / 16) * 8 + j;
            for (size_t b = 0; b < es; ++b) {
              const unsigned char got = out[((((size_t)t * KB + kb) * 64 + lane) * 8 + j) * es + b];
              const unsigned char want = rows[row] ? src[row][k * es + b] : 0;
              CHECK(got == want, "pack_rows tile %d kb %d lane %d j %d\n", t, kb, lane, j);
            }
          }
  }
}

static void check_qkv_rows() {
  for (int dh : {32, 64, 128, 256})
    for (int nkv : {1, 2}) {
      const int nq = 2 * nkv, w = 64;
      std::vector<unsigned char> wq((size_t)nq * dh * w), wk((size_t)nkv * dh * w), wv((size_t)nkv * dh * w);
      const auto rows = ae_host::qkv_rows(wq.data(), wk.data(), wv.data(), nq, nkv, dh, w, 1);
      CHECK(rows.size() == (size_t)(nq + 2 * nkv) * dh, "qkv_rows count\n");
      // every q and k head: each dim once; tile p pairs dims p*8+c with dh/2+p*8+c
      for (int part = 0; part < 2; ++part) {
        const int nh = part ? nkv : nq;
        const unsigned char* base = part ? wk.data() : wq.data();
        const size_t off = part ? (size_t)nq * dh : 0;
        for (int hh = 0; hh < nh; ++hh) {
          std::vector<int> seen(dh, 0);
          for (int p = 0; p < dh / 16; ++p)
            for (int c = 0; c < 16; ++c) {
              const long d = (long)((rows[off + (size_t)hh * dh + p * 16 + c] - base) / w) - (long)hh * dh;
              CHECK(d >= 0 && d < dh, "qkv_rows dim out of the head\n");
              if (d >= 0 && d < dh) ++seen[d];
              if (c < 8) {
                const long d2 = (long)((rows[off + (size_t)hh * dh + p * 16 + c + 8] - base) / w) - (long)hh * dh;
                CHECK(d2 == d + dh / 2, "qkv_rows RoPE pair dh %d tile %d channel %d\n", dh, p, c);
              }
            }
          for (int d = 0; d < dh; ++d) CHECK(seen[d] == 1, "qkv_rows dim %d seen %d times\n", d, seen[d]);
        }
      }
      for (int r = 0; r < nkv * dh; ++r)
        CHECK(rows[(size_t)(nq + nkv) * dh + r] == wv.data() + (size_t)r * w, "qkv_rows v row %d\n", r);
    }
}

static void check_gate_up_rows() {
  const int F = 64, w = 32;
  std::vector<unsigned char> wg(F * w), wu(F * w);
  const auto rows = ae_host::gate_up_rows(wg.data(), wu.data(), F, w, 1);
  CHECK(rows.size() == (size_t)2 * F, "gate_up_rows count\n");
  for (int j = 0; j < F / 16; ++j)
    for (int c = 0; c < 16; ++c) {
      CHECK(rows[j * 32 + c] == wg.data() + (size_t)(j * 16 + c) * w, "gate row\n");
      CHECK(rows[j * 32 + 16 + c] == wu.data() + (size_t)(j * 16 + c) * w, "up row\n");
    }
}

static void check_repack(std::mt19937& rng) {
  for (int it = 0; it < 12; ++it) {
    const int L = 1 + (int)(rng() % 2), nkv = 1 + (int)(rng() % 3), dh = 32 << (rng() % 3), P = 1 + (int)(rng() % 100);
    const int nbp = (P + 31) / 32;
    const size_t n = (size_t)L * P * nkv * dh;
    std::vector<uint32_t> k(n), v(n);  // es = 4: element e holds e + 1 (K) and e + 1 + n (V)
    for (size_t e = 0; e < n; ++e) {
      k[e] = (uint32_t)(e + 1);
      v[e] = (uint32_t)(e + 1 + n);
    }
    std::vector<unsigned char> kp, vp;
    ae_host::repack_prefix_kv((const unsigned char*)k.data(), (const unsigned char*)v.data(), L, P, nkv, dh, nbp, 4, kp, vp);
    const size_t elems = (size_t)L * nkv * nbp * 32 * dh;
    CHECK(kp.size() == elems * 4 && vp.size() == elems * 4, "repack size\n");
    const uint32_t* K = (const uint32_t*)kp.data();
    const uint32_t* V = (const uint32_t*)vp.data();
    const int nkb = dh / 32;
    for (int l = 0; l < L; ++l)
      for (int g = 0; g < nkv; ++g)
        for (int b = 0; b < nbp; ++b) {
          const size_t blk = (((size_t)l * nkv + g) * nbp + b) * 32 * dh;
          auto src = [&](const std::vector<uint32_t>& s, int key, int d) -> uint32_t {
            const int j = b * 32 + key;
            return j < P ? s[(((size_t)l * P + j) * nkv + g) * dh + d] : 0u;
          };
          // K: fragment [kt][kb], lane ln: row m = ln % 16 is key 8 (m/4) + 4 kt + m % 4, dims kb*32 + (ln/16)*8 + e
          for (int kt = 0; kt < 2; ++kt)
            for (int kb = 0; kb < nkb; ++kb)
              for (int ln = 0; ln < 64; ++ln)
                for (int e = 0; e < 8; ++e) {
                  const int m = ln % 16, key = 8 * (m / 4) + 4 * kt + m % 4, d = kb * 32 + (ln / 16) * 8 + e;
                  const uint32_t got = K[blk + (((size_t)kt * nkb + kb) * 64 + ln) * 8 + e];
                  CHECK(got == src(k, key, d), "repack K l %d g %d block %d kt %d kb %d lane %d\n", l, g, b, kt, kb, ln);
                }
          // V: fragment [dt], lane ln: dim dt*16 + ln % 16, keys (ln/16)*8 + e
          for (int dt = 0; dt < dh / 16; ++dt)
            for (int ln = 0; ln < 64; ++ln)
              for (int e = 0; e < 8; ++e) {
                const int key = (ln / 16) * 8 + e, d = dt * 16 + ln % 16;
                const uint32_t got = V[blk + ((size_t)dt * 64 + ln) * 8 + e];
                CHECK(got == src(v, key, d), "repack V l %d g %d block %d dt %d lane %d\n", l, g, b, dt, ln);
              }
        }
  }
}

static void check_validate() {
  // one layer of dummy (non-null) pointers; the checks never read through them
  static float dummy[4];
  ae_layer_weights lw{};
  lw.ln1 = lw.ln2 = dummy;
  lw.wq = lw.wk = lw.wv = lw.wo = lw.wg = lw.wu = lw.wd = dummy;
  lw.wg_scale = lw.wu_scale = lw.wd_scale = dummy;
  std::vector<ae_layer_weights> layers(4, lw);
  ae_weights w{};
  w.time_in_w = w.time_out_w = w.action_in_w = w.action_out_w = dummy;
  w.time_in_b = w.time_out_b = w.action_in_b = w.action_out_b = w.final_ln = dummy;
  w.layers = layers.data();
  ae_config base{};
  base.n_layers = 2; base.width = 256; base.n_q_heads = 4; base.n_kv_heads = 1; base.head_dim = 64;
  base.mlp_dim = 1024; base.action_dim = 8; base.horizon = 8; base.prefix_len = 64; base.max_batch = 1;
  base.max_taus = 0; base.rope_base = 10000.f; base.rms_eps = 1e-6f; base.weight_dtype = AE_F32;
  base.mlp_dtype = AE_F32; base.kv_dtype = AE_F32; base.gripper_dim = -1;
  std::string why;
  CHECK(ae_host::validate_config(&base, &w, why) == AE_OK, "a covered config is rejected: %s\n", why.c_str());
  CHECK(ae_host::validate_config(nullptr, &w, why) == AE_ERR_INVALID_ARG, "null config\n");
  struct Case { void (*set)(ae_config&); int code; };
  const Case cases[] = {
      {[](ae_config& c) { c.width = 0; }, AE_ERR_INVALID_ARG},
      {[](ae_config& c) { c.n_kv_heads = 3; }, AE_ERR_INVALID_ARG},
      {[](ae_config& c) { c.gripper_dim = 8; }, AE_ERR_INVALID_ARG},
      {[](ae_config& c) { c.max_taus = 65; }, AE_ERR_INVALID_ARG},
      {[](ae_config& c) { c.rope_base = 0.f; }, AE_ERR_INVALID_ARG},
      {[](ae_config& c) { c.width = 200; }, AE_ERR_UNSUPPORTED},
      {[](ae_config& c) { c.head_dim = 48; }, AE_ERR_UNSUPPORTED},
      {[](ae_config& c) { c.action_dim = 65; }, AE_ERR_UNSUPPORTED},
      {[](ae_config& c) { c.horizon = 257; }, AE_ERR_UNSUPPORTED},
      {[](ae_config& c) { c.weight_dtype = 7; }, AE_ERR_INVALID_ARG},
      {[](ae_config& c) { c.kv_dtype = AE_BF16; }, AE_ERR_UNSUPPORTED},
      {[](ae_config& c) { c.mlp_dtype = AE_FP8_E4M3; }, AE_ERR_UNSUPPORTED},
      // sizes whose products overflow int: rejected before any product is formed
      {[](ae_config& c) { c.n_q_heads = INT_MAX; c.n_kv_heads = 1; }, AE_ERR_UNSUPPORTED},
      {[](ae_config& c) { c.width = INT_MAX - 255; }, AE_ERR_UNSUPPORTED},
      {[](ae_config& c) { c.mlp_dim = INT_MAX; }, AE_ERR_UNSUPPORTED},
      {[](ae_config& c) { c.n_layers = INT_MAX; }, AE_ERR_UNSUPPORTED},
      {[](ae_config& c) { c.prefix_len = INT_MAX; }, AE_ERR_UNSUPPORTED},
      {[](ae_config& c) { c.max_batch = INT_MAX; }, AE_ERR_UNSUPPORTED},
  };
  int i = 0;
  for (const Case& cs : cases) {
    ae_config c = base;
    cs.set(c);
    const int rc = ae_host::validate_config(&c, &w, why);
    CHECK(rc == cs.code, "validate case %d: code %d, expected %d (%s)\n", i, rc, cs.code, why.c_str());
    ++i;
  }
  ae_weights wn = w;
  wn.layers = nullptr;
  CHECK(ae_host::validate_config(&base, &wn, why) == AE_ERR_INVALID_ARG, "null layers\n");
}

int main() {
  std::mt19937 rng(1234);
  check_pack_rows(rng);
  check_qkv_rows();
  check_gate_up_rows();
  check_repack(rng);
  check_validate();
  if (g_fail) return 1;
  printf("ok\n");
  return 0;
}
