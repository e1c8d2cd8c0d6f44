// Host-side checks of the GDLA C ABI, built with AddressSanitizer and UndefinedBehaviorSanitizer
// over the library's host code (the device code is built as usual).  It drives the argument
// validation and workspace planning of every entry point, on the CPU:
//   1. gdla_workspace_bytes over every op, over the layers the library serves and over a seeded
//      sweep of edge-valued sizes (negative, zero, odd, huge), with properties of the result;
//   2. every entry point with one argument made invalid at a time: the documented status comes
//      back and gdla_last_error says why (so the check ran before any launch);
//   3. only when the process sees no GPU: valid argument sets with a workspace large enough, which
//      pass validation and planning and then fail at the first HIP runtime call;
//   4. the value layout of the prefill attention (key order inside each 32-key group).
// The pointers handed in are never dereferenced by host code; on a machine with a GPU part 3 is
// skipped so that no fake pointer can reach a copy or a kernel.
#include "gdla.h"
// the value layout shared by the expansion GEMM's store and the prefill attention's PV operand
#include "../attention_gdla_prefill_decode_amd/csrc/fast_paths.h"

#include <hip/hip_runtime_api.h>

#include <limits.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <random>
#include <thread>
#include <vector>

static int g_failures = 0;
static int g_checks = 0;

static void expect(bool ok, const char *what, ...) {
  ++g_checks;
  if (ok) return;
  ++g_failures;
  va_list ap;
  va_start(ap, what);
  fprintf(stderr, "FAIL: ");
  vfprintf(stderr, what, ap);
  fprintf(stderr, "\n");
  va_end(ap);
}

// ---------------------------------------------------------------------------------------------
// Layers: the 4096-wide, 80-head layer (64 signal + 16 noise heads over 16 KV heads, latents
// 1024 / 512, heads 128 + 64), and a small fp32 layer that takes the generic kernels.
static gdla_dims big_layer(gdla_dtype dt = GDLA_BF16, int32_t window = 0) {
  gdla_dims d{};
  d.d_model = 4096; d.n_heads = 80; d.n_signal = 64; d.n_noise = 16; d.n_kv_heads = 16;
  d.d_q_latent = 1024; d.d_kv_latent = 512; d.d_head = 128; d.d_rope = 64; d.window = window;
  d.rms_eps = 1e-6f; d.rope_theta = 10000.f; d.softmax_scale = 0.f; d.dtype = dt;
  return d;
}

static gdla_dims small_layer(gdla_dtype dt = GDLA_F32) {
  gdla_dims d{};
  d.d_model = 64; d.n_heads = 8; d.n_signal = 6; d.n_noise = 2; d.n_kv_heads = 2;
  d.d_q_latent = 32; d.d_kv_latent = 16; d.d_head = 8; d.d_rope = 4; d.window = 0;
  d.rms_eps = 1e-6f; d.rope_theta = 10000.f; d.softmax_scale = 0.f; d.dtype = dt;
  return d;
}

// Aligned stand-in addresses: never dereferenced by the library's host code.
static void *fake(uintptr_t k) { return (void *)(uintptr_t)(0x100000000ull + (k << 12)); }

static gdla_weights fake_weights() {
  gdla_weights w{};
  w.w_qa = fake(1); w.gamma_q = fake(2); w.w_qc = fake(3); w.w_qr = fake(4); w.w_dkv = fake(5);
  w.w_kr = fake(6); w.gamma_kv = fake(7); w.w_uk = fake(8); w.w_uv = fake(9); w.w_lambda = fake(10);
  w.w_gate = fake(11); w.w_o = fake(12);
  return w;
}

static gdla_grads fake_grads() {
  gdla_grads g{};
  float **f = &g.dx;
  for (int i = 0; i < 13; ++i) f[i] = (float *)fake(20 + i);
  return g;
}

// A heap copy of exactly B positions, so that a read past the caller's array is an ASan report.
struct Pos {
  int32_t *p = nullptr;
  explicit Pos(const std::vector<int32_t> &v) {
    p = (int32_t *)malloc(sizeof(int32_t) * (v.empty() ? 1 : v.size()));
    if (!v.empty()) memcpy(p, v.data(), sizeof(int32_t) * v.size());
  }
  ~Pos() { free(p); }
  Pos(const Pos &) = delete;
  Pos &operator=(const Pos &) = delete;
};

static bool last_error_set() {
  const char *e = gdla_last_error();
  return e && e[0] != 0 && strnlen(e, 4096) < 256;
}

// ---------------------------------------------------------------------------------------------
// 1. Workspace planning.
static void check_workspace_planning() {
  const int ops[] = {GDLA_OP_PREFILL, GDLA_OP_DECODE, GDLA_OP_APPEND, GDLA_OP_PREFILL_PAGED, GDLA_OP_BACKWARD};
  const gdla_dims layers[] = {big_layer(), big_layer(GDLA_BF16, 4096), big_layer(GDLA_F32), small_layer(),
                              small_layer(GDLA_BF16)};
  std::mt19937 rng(20261203);
  for (const gdla_dims &d : layers) {
    for (int op : ops) {
      const int32_t Bs[] = {1, 2, 3, 64};
      const int32_t Ts[] = {1, 4, 16, 17, 33, 256, 1000};
      for (int32_t B : Bs)
        for (int32_t T : Ts) {
          if (op == GDLA_OP_BACKWARD && (int64_t)B * T > 4096) continue;
          const int32_t max_len = op == GDLA_OP_BACKWARD ? T : T + 2000;
          const size_t bound = gdla_workspace_bytes(&d, op, B, T, nullptr, max_len);
          const bool decode_too_many = op == GDLA_OP_DECODE && T > GDLA_MAX_DECODE_TOKENS;
          expect(decode_too_many ? bound == 0 : bound > 0, "op %d B %d T %d: bound %zu", op, B, T, bound);
          expect(bound % 256 == 0, "op %d: %zu not a multiple of 256", op, bound);
          if (op == GDLA_OP_BACKWARD || decode_too_many) continue;
          // with positions, no more than the bound for any positions (header of gdla_workspace_bytes)
          std::vector<int32_t> v((size_t)B);
          for (int trial = 0; trial < 3; ++trial) {
            for (auto &p : v) p = (int32_t)(rng() % (uint32_t)(max_len - T + 1));
            Pos pos(v);
            const size_t n = gdla_workspace_bytes(&d, op, B, T, pos.p, max_len);
            expect(n > 0 && n <= bound, "op %d B %d T %d: %zu with positions, bound %zu", op, B, T, n, bound);
          }
          // a position past the end gives 0
          v.assign((size_t)B, 0);
          v[(size_t)B - 1] = max_len - T + 1;
          Pos bad(v);
          expect(gdla_workspace_bytes(&d, op, B, T, bad.p, max_len) == 0, "op %d: position past max_len", op);
          v[(size_t)B - 1] = -1;
          Pos neg(v);
          expect(gdla_workspace_bytes(&d, op, B, T, neg.p, max_len) == 0, "op %d: negative position", op);
        }
    }
  }
  // Edge-valued sizes: every combination that check_dims accepts must plan without overflow or
  // out-of-bounds access; the rest must return 0.  (pos is NULL here: the sizes run far beyond
  // any array worth allocating.)
  const int32_t edge[] = {-1, 0, 1, 2, 3, 7, 8, 16, 32, 64, 128, 256, 257, 1024, 4096, 65536, 1 << 20, INT32_MAX};
  const int n_edge = (int)(sizeof(edge) / sizeof(edge[0]));
  int accepted = 0;
  for (int trial = 0; trial < 20000; ++trial) {
    gdla_dims d = (rng() & 1) ? big_layer() : small_layer((rng() & 1) ? GDLA_BF16 : GDLA_F32);
    int32_t *fields = &d.d_model;  // the ten int32 size fields, in declaration order
    const int n_mut = 1 + (int)(rng() % 3);
    for (int k = 0; k < n_mut; ++k) fields[rng() % 10] = edge[rng() % n_edge];
    if (rng() % 8 == 0) d.rms_eps = (rng() & 1) ? -1.f : __builtin_nanf("");
    if (rng() % 8 == 0) d.rope_theta = (rng() & 1) ? 0.f : __builtin_inff();
    if (rng() % 16 == 0) d.dtype = (gdla_dtype)(rng() % 4);
    const int op = (int)(rng() % 7) - 1;
    const int32_t B = edge[rng() % n_edge], T = edge[rng() % n_edge], max_len = edge[rng() % n_edge];
    const size_t n = gdla_workspace_bytes(&d, op, B, T, nullptr, max_len);
    if (n) {
      ++accepted;
      expect(n % 256 == 0, "sweep: %zu not a multiple of 256", n);
      expect(B > 0 && T > 0 && T <= max_len, "sweep: accepted B %d T %d max_len %d", B, T, max_len);
    }
  }
  expect(accepted > 100, "sweep accepted only %d requests", accepted);
  expect(gdla_workspace_bytes(nullptr, GDLA_OP_PREFILL, 1, 1, nullptr, 8) == 0, "NULL dims");
  const gdla_dims big = big_layer();
  expect(gdla_workspace_bytes(&big, GDLA_OP_PREFILL, 65536, 65536, nullptr, 65536) == 0,
         "B T above 2^30 rows is refused");
  expect(gdla_prepared_weights_bytes(&big) > 0, "prepared weights of the bf16 layer");
  const gdla_dims f32 = big_layer(GDLA_F32);
  expect(gdla_prepared_weights_bytes(&f32) == 0, "no prepared weights for fp32 layers");
  expect(gdla_prepared_weights_bytes(nullptr) == 0, "prepared weights of NULL dims");
}

// ---------------------------------------------------------------------------------------------
// 2. One invalid argument at a time.
struct Args {
  gdla_dims d = big_layer();
  gdla_weights w = fake_weights();
  gdla_grads g = fake_grads();
  const void *x = fake(40);
  void *cache = fake(41);
  void *out = fake(42);
  void *ws = fake(43);
  void *prepared = fake(44);
  const int32_t *doc = (const int32_t *)fake(45);
  const void *dout = fake(46);
  size_t ws_bytes = (size_t)1 << 50;
  size_t prepared_bytes = (size_t)1 << 40;
  int32_t B = 2, T = 4, max_len = 4096;
  std::vector<int32_t> pos{0, 100};
  gdla_paged_cache pc{fake(47), (const int32_t *)fake(48), 1024, 32, 128};
  bool null_dims = false, null_w = false, null_pos = false, null_cache = false, null_grads = false;
};

enum Entry { PREFILL, PREFILL_PREPARED, PREFILL_PACKED, PREFILL_PAGED, DECODE, DECODE_NOALLOC, DECODE_TOKENS,
             DECODE_PAGED, APPEND, APPEND_PAGED, BACKWARD, PREPARE, N_ENTRIES };
static const char *entry_name[N_ENTRIES] = {"prefill", "prefill_prepared", "prefill_packed", "prefill_paged",
                                            "decode", "decode_noalloc", "decode_tokens", "decode_paged",
                                            "latent_append", "latent_append_paged", "backward", "prepare_weights"};

static gdla_status call(Entry e, const Args &a) {
  Pos pos(a.pos);
  const gdla_dims *d = a.null_dims ? nullptr : &a.d;
  const gdla_weights *w = a.null_w ? nullptr : &a.w;
  const int32_t *p = a.null_pos ? nullptr : pos.p;
  void *cache = a.null_cache ? nullptr : a.cache;
  const gdla_paged_cache *pc = a.null_cache ? nullptr : &a.pc;
  const hipStream_t s = nullptr;
  switch (e) {
    case PREFILL: return gdla_prefill(d, w, a.x, a.B, a.T, p, cache, a.max_len, a.out, a.ws, a.ws_bytes, nullptr, s);
    case PREFILL_PREPARED:
      return gdla_prefill_prepared(d, w, a.prepared, a.prepared_bytes, a.x, a.B, a.T, p, cache, a.max_len, a.out,
                                   a.ws, a.ws_bytes, nullptr, s);
    case PREFILL_PACKED:
      return gdla_prefill_packed(d, w, a.x, a.B, a.T, p, a.doc, cache, a.max_len, a.out, a.ws, a.ws_bytes, nullptr, s);
    case PREFILL_PAGED: return gdla_prefill_paged(d, w, a.x, a.B, a.T, p, pc, a.out, a.ws, a.ws_bytes, nullptr, s);
    case DECODE: return gdla_decode(d, w, a.x, a.B, p, cache, a.max_len, a.out, a.ws, a.ws_bytes, nullptr, s);
    case DECODE_NOALLOC: return gdla_decode_noalloc(d, w, a.x, a.B, p, cache, a.max_len, a.out, nullptr, s);
    case DECODE_TOKENS:
      return gdla_decode_tokens(d, w, a.x, a.B, a.T, p, cache, a.max_len, a.out, a.ws, a.ws_bytes, nullptr, s);
    case DECODE_PAGED: return gdla_decode_paged(d, w, a.x, a.B, a.T, p, pc, a.out, a.ws, a.ws_bytes, nullptr, s);
    case APPEND: return gdla_latent_append(d, w, a.x, a.B, a.T, p, cache, a.max_len, a.ws, a.ws_bytes, s);
    case APPEND_PAGED: return gdla_latent_append_paged(d, w, a.x, a.B, a.T, p, pc, a.ws, a.ws_bytes, s);
    case BACKWARD:
      return gdla_backward(d, w, a.x, a.B, a.T, a.doc, a.dout, a.null_grads ? nullptr : &a.g, a.ws, a.ws_bytes,
                           nullptr, s);
    case PREPARE: return gdla_prepare_weights(d, w, a.prepared, a.prepared_bytes, s);
    default: return GDLA_OK;
  }
}

static bool takes_T(Entry e) { return e != DECODE && e != DECODE_NOALLOC && e != PREPARE; }
static bool takes_pos(Entry e) { return e != BACKWARD && e != PREPARE; }
static bool takes_ws(Entry e) { return e != DECODE_NOALLOC && e != PREPARE; }
static bool paged(Entry e) { return e == PREFILL_PAGED || e == DECODE_PAGED || e == APPEND_PAGED; }

static void expect_status(Entry e, const Args &a, gdla_status want, const char *what) {
  const gdla_status got = call(e, a);
  expect(got == want, "%s, %s: %s, expected %s (%s)", entry_name[e], what, gdla_status_string(got),
         gdla_status_string(want), gdla_last_error());
  if (want != GDLA_OK) expect(last_error_set(), "%s, %s: no error text", entry_name[e], what);
}

static Args base_args(Entry e) {
  Args a;
  if (e == DECODE || e == DECODE_NOALLOC) {
    a.pos = {4095, 17};
    a.T = 1;
  }
  if (e == DECODE_TOKENS || e == DECODE_PAGED) a.pos = {4092, 17};
  if (e == BACKWARD) a.T = 300;
  return a;
}

static void check_validation() {
  for (int ei = 0; ei < N_ENTRIES; ++ei) {
    const Entry e = (Entry)ei;
    Args a;
    a = base_args(e); a.null_dims = true;
    expect_status(e, a, GDLA_ERR_INVALID_ARG, "NULL dims");
    a = base_args(e); a.d.n_noise = 15;
    expect_status(e, a, GDLA_ERR_INVALID_ARG, "n_signal + n_noise != n_heads");
    a = base_args(e); a.d.d_rope = 63;
    expect_status(e, a, GDLA_ERR_INVALID_ARG, "odd d_rope");
    a = base_args(e); a.d.rms_eps = __builtin_nanf("");
    expect_status(e, a, GDLA_ERR_INVALID_ARG, "NaN rms_eps");
    a = base_args(e); a.d.dtype = (gdla_dtype)7;
    expect_status(e, a, GDLA_ERR_INVALID_ARG, "unknown dtype");
    a = base_args(e); a.d.d_head = 512;
    expect_status(e, a, GDLA_ERR_UNSUPPORTED, "d_head 512");
    a = base_args(e); a.null_w = true;
    expect_status(e, a, GDLA_ERR_INVALID_ARG, "NULL weights");
    a = base_args(e); a.w.w_dkv = nullptr;
    expect_status(e, a, GDLA_ERR_INVALID_ARG, "NULL w_dkv");
    a = base_args(e); a.w.w_o = (const char *)a.w.w_o + 2;
    expect_status(e, a, GDLA_ERR_INVALID_ARG, "misaligned w_o");
    if (e == PREPARE) {
      a = base_args(e); a.prepared_bytes = gdla_prepared_weights_bytes(&a.d) - 1;
      expect_status(e, a, GDLA_ERR_WORKSPACE, "prepared buffer one byte short");
      a = base_args(e); a.prepared = (char *)a.prepared + 16;
      expect_status(e, a, GDLA_ERR_INVALID_ARG, "misaligned prepared buffer");
      a = base_args(e); a.d = big_layer(GDLA_F32);
      expect_status(e, a, GDLA_ERR_UNSUPPORTED, "fp32 layer");
      continue;
    }
    a = base_args(e); a.x = nullptr;
    expect_status(e, a, GDLA_ERR_INVALID_ARG, "NULL x");
    a = base_args(e); a.x = (const char *)a.x + 4;
    expect_status(e, a, GDLA_ERR_INVALID_ARG, "misaligned x");
    a = base_args(e); a.B = -1;
    expect_status(e, a, GDLA_ERR_INVALID_ARG, "negative B");
    if (takes_T(e)) {
      a = base_args(e); a.T = -3;
      expect_status(e, a, GDLA_ERR_INVALID_ARG, "negative T");
    }
    if (e == DECODE_TOKENS || e == DECODE_PAGED) {
      a = base_args(e); a.T = GDLA_MAX_DECODE_TOKENS + 1;
      expect_status(e, a, GDLA_ERR_INVALID_ARG, "T above GDLA_MAX_DECODE_TOKENS");
    }
    if (takes_pos(e)) {
      a = base_args(e); a.null_pos = true;
      expect_status(e, a, GDLA_ERR_INVALID_ARG, "NULL pos_host");
      a = base_args(e); a.pos[1] = -5;
      expect_status(e, a, GDLA_ERR_OUT_OF_RANGE, "negative position");
      a = base_args(e); a.pos[1] = 4096 - a.T + 1;
      expect_status(e, a, GDLA_ERR_OUT_OF_RANGE, "position + T past the cache");
      a = base_args(e); a.null_cache = true;
      expect_status(e, a, GDLA_ERR_INVALID_ARG, "NULL cache");
    }
    if (!paged(e) && takes_pos(e)) {
      a = base_args(e); a.cache = (char *)a.cache + 8;
      expect_status(e, a, GDLA_ERR_INVALID_ARG, "misaligned cache");
      a = base_args(e); a.max_len = 0;
      expect_status(e, a, GDLA_ERR_INVALID_ARG, "max_len 0");
    }
    if (paged(e)) {
      a = base_args(e); a.pc.page_rows = 48;
      expect_status(e, a, GDLA_ERR_INVALID_ARG, "page_rows not a multiple of 32");
      a = base_args(e); a.pc.max_blocks = INT32_MAX / 16;
      expect_status(e, a, GDLA_ERR_INVALID_ARG, "max_blocks * page_rows beyond int32");
      a = base_args(e); a.pc.block_table = (const int32_t *)((const char *)a.pc.block_table + 2);
      expect_status(e, a, GDLA_ERR_INVALID_ARG, "misaligned block_table");
      a = base_args(e); a.pc.n_pages = 0;
      expect_status(e, a, GDLA_ERR_INVALID_ARG, "no pages");
    }
    if (takes_ws(e)) {
      a = base_args(e);
      const int op = e == BACKWARD ? GDLA_OP_BACKWARD
                     : e == PREFILL_PAGED ? GDLA_OP_PREFILL_PAGED
                     : (e == APPEND || e == APPEND_PAGED) ? GDLA_OP_APPEND
                     : (e == DECODE || e == DECODE_TOKENS || e == DECODE_PAGED) ? GDLA_OP_DECODE
                     : GDLA_OP_PREFILL;
      Pos pos(a.pos);
      const int32_t max_len = paged(e) ? a.pc.max_blocks * a.pc.page_rows : e == BACKWARD ? a.T : a.max_len;
      const size_t need = gdla_workspace_bytes(&a.d, op, a.B, a.T, e == BACKWARD ? nullptr : pos.p, max_len);
      expect(need > 0, "%s: workspace size", entry_name[e]);
      a.ws_bytes = need - 1;
      expect_status(e, a, GDLA_ERR_WORKSPACE, "workspace one byte short");
      a = base_args(e); a.ws = (char *)a.ws + 64;
      expect_status(e, a, GDLA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
      a = base_args(e); a.ws = nullptr;
      expect_status(e, a, GDLA_ERR_INVALID_ARG, "NULL workspace");
    }
    if (e == PREFILL_PACKED) {
      a = base_args(e); a.doc = nullptr;
      expect_status(e, a, GDLA_ERR_INVALID_ARG, "NULL doc_start");
      a = base_args(e); a.doc = (const int32_t *)((const char *)a.doc + 2);
      expect_status(e, a, GDLA_ERR_INVALID_ARG, "misaligned doc_start");
    }
    if (e == PREFILL_PREPARED) {
      a = base_args(e); a.prepared_bytes = 1024;
      expect_status(e, a, GDLA_ERR_WORKSPACE, "prepared buffer too small");
      a = base_args(e); a.prepared = nullptr;
      expect_status(e, a, GDLA_ERR_INVALID_ARG, "NULL prepared");
    }
    if (e == BACKWARD) {
      a = base_args(e); a.null_grads = true;
      expect_status(e, a, GDLA_ERR_INVALID_ARG, "NULL grads");
      a = base_args(e); a.g.dw_uv = nullptr;
      expect_status(e, a, GDLA_ERR_INVALID_ARG, "NULL dw_uv");
      a = base_args(e); a.g.dgamma_kv = nullptr;
      expect_status(e, a, GDLA_ERR_INVALID_ARG, "NULL dgamma_kv with gamma_kv");
      a = base_args(e); a.dout = nullptr;
      expect_status(e, a, GDLA_ERR_INVALID_ARG, "NULL dout");
      a = base_args(e); a.doc = (const int32_t *)((const char *)a.doc + 1);
      expect_status(e, a, GDLA_ERR_INVALID_ARG, "misaligned doc_start");
    }
    if (e == DECODE_NOALLOC) {
      // more sequences than the static scratch holds: refused before anything runs
      a = base_args(e);
      a.B = 4096;
      a.pos.assign(4096, 100);
      expect_status(e, a, GDLA_ERR_WORKSPACE, "decode beyond the static scratch");
    }
    // nothing to do: OK without touching any pointer
    a = base_args(e); a.B = 0; a.x = nullptr; a.ws = nullptr; a.ws_bytes = 0; a.pos.clear();
    if (e != DECODE_NOALLOC) expect_status(e, a, GDLA_OK, "B = 0");
  }
  // more rows or positions than the library serves: refused, never wrapped
  Args a;
  a.B = 65536; a.T = 65536; a.max_len = 65536; a.pos.assign(65536, 0);
  expect_status(PREFILL, a, GDLA_ERR_UNSUPPORTED, "B T above 2^30 rows");
  a.T = 32768;
  a.g = fake_grads();
  expect_status(BACKWARD, a, GDLA_ERR_UNSUPPORTED, "B T at 2^31 rows");
  Args m;
  m.max_len = (1 << 30) + 1;
  expect_status(PREFILL, m, GDLA_ERR_UNSUPPORTED, "max_len above 2^30");
  expect_status(DECODE, m, GDLA_ERR_UNSUPPORTED, "max_len above 2^30");
}

// The value layout: vt_key inverts vt_slot; every aligned group of 32 keys maps onto itself and
// every aligned run of 4 keys onto 4 consecutive positions (the GEMM stores them with one 8-byte
// write); and the PV operand's k-slot 8 g + e (lane group g, element e) of a 32-key group holds
// key 16 (e / 4) + 4 g + e % 4, the order in which the 16 x 16 score blocks leave the keys.
static void check_value_layout() {
  for (int k = 0; k < 1 << 16; ++k) {
    const int p = gdla::vt_slot(k);
    expect(gdla::vt_key(p) == k, "vt_key(vt_slot(%d)) = %d", k, gdla::vt_key(p));
    expect(p / 32 == k / 32, "key %d leaves its 32-group (position %d)", k, p);
    if (k % 4) expect(p == gdla::vt_slot(k - k % 4) + k % 4, "keys %d..%d not consecutive", k - k % 4, k);
  }
  for (int g = 0; g < 4; ++g)
    for (int e = 0; e < 8; ++e) {
      const int key = 16 * (e / 4) + 4 * g + e % 4;
      expect(gdla::vt_slot(key) == 8 * g + e, "operand slot %d holds key %d", 8 * g + e, key);
    }
}

// The error text is per thread: a failure on one thread leaves another thread's text alone.
static void check_error_text_per_thread() {
  gdla_dims bad = big_layer();
  bad.n_noise = 15;
  expect(gdla_workspace_bytes(&bad, GDLA_OP_PREFILL, 1, 1, nullptr, 8) == 0, "bad dims");
  std::string mine = gdla_last_error();
  std::string theirs = "unset";
  std::thread t([&] { theirs = gdla_last_error(); });
  t.join();
  expect(!mine.empty() && theirs.empty(), "error text per thread: '%s' / '%s'", mine.c_str(), theirs.c_str());
}

// ---------------------------------------------------------------------------------------------
// 3. Valid calls on a machine without a GPU: validation and planning pass, the first HIP call fails.
static void check_valid_calls_without_gpu() {
  int n = 0;
  const hipError_t e = hipGetDeviceCount(&n);
  if (e == hipSuccess && n > 0) {
    printf("a GPU is visible: valid-argument calls skipped\n");
    return;
  }
  for (int ei = 0; ei < N_ENTRIES; ++ei) {
    const Entry en = (Entry)ei;
    Args a = base_args(en);
    if (en == PREFILL_PREPARED || en == PREPARE) a.prepared_bytes = gdla_prepared_weights_bytes(&a.d);
    const gdla_status got = call(en, a);
    expect(got == GDLA_ERR_HIP, "%s without a GPU: %s (%s)", entry_name[en], gdla_status_string(got),
           gdla_last_error());
  }
  // the small fp32 layer (generic kernels) and the windowed layer
  for (const gdla_dims &d : {small_layer(), big_layer(GDLA_BF16, 64)}) {
    for (int ei = 0; ei < N_ENTRIES; ++ei) {
      const Entry en = (Entry)ei;
      if (en == PREPARE || en == PREFILL_PREPARED) continue;
      Args a = base_args(en);
      a.d = d;
      expect(call(en, a) == GDLA_ERR_HIP, "%s (second layer) without a GPU: %s", entry_name[en], gdla_last_error());
    }
  }
}

int main() {
  check_workspace_planning();
  check_validation();
  check_error_text_per_thread();
  check_value_layout();
  check_valid_calls_without_gpu();
  printf("%d checks, %d failures\n", g_checks, g_failures);
  if (g_failures == 0) printf("all checks passed\n");
  return g_failures ? 1 : 0;
}
