// Host-side argument checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_abi_sanitized.py builds and runs
// it on the CPU).  Every size query is fed edge values of every shape field, one field at a
// time and in seeded random combinations, and every entry point is called with arguments
// its host checks must reject.  Nothing here may reach a kernel launch: the pointers are
// host integers that are never dereferenced, and the program refuses to call entry points
// if it finds a GPU.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "specfold.h"

namespace {

int g_failures = 0;

#define EXPECT(cond, ...)                                  \
  do {                                                     \
    if (!(cond)) {                                         \
      ++g_failures;                                        \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                        \
      fprintf(stderr, "\n");                               \
    }                                                      \
  } while (0)

const int kInts[] = {INT_MIN, -129, -1, 0, 1, 2, 3, 63, 64, 96, 127, 128, 129, 256, 1000,
                     1024, 1025, 3584, 16384, 16385, 32768, 32896, 131072, 131200,
                     1 << 24, (1 << 24) + 1, 1 << 30, INT_MAX - 127, INT_MAX};
const float kFloats[] = {-1.f, -0.f, 0.f, 1e-45f, 1e-6f, 1.f, 1e6f, FLT_MAX, INFINITY,
                         -INFINITY, NAN};
constexpr int kNI = sizeof(kInts) / sizeof(kInts[0]);
constexpr int kNF = sizeof(kFloats) / sizeof(kFloats[0]);

specfold_shape base_shape() {
  specfold_shape s{};
  s.num_nodes = 16; s.block = 32; s.hidden = 3584; s.n_q_heads = 28; s.n_kv_heads = 4;
  s.head_dim = 128; s.ffn = 18944; s.prefix_len = 512; s.rms_eps = 1e-6f;
  s.dtype = SPECFOLD_BF16; s.rope_theta = 0.f;
  return s;
}

// Size queries on one shape: either rejected with a message, or sizes that hold the
// layer's buffers with every intermediate inside.
void check_sizes(const specfold_shape& s) {
  const size_t ws = specfold_layer_workspace_bytes(&s);
  if (ws == 0) {
    EXPECT(specfold_last_error()[0] != 0, "rejected shape without a message");
    EXPECT(specfold_stack_workspace_bytes(&s) == 0, "stack size of a rejected shape");
    return;
  }
  const size_t S = (size_t)s.num_nodes * s.block;
  const size_t eb = s.dtype == SPECFOLD_BF16 ? 2 : 4;
  EXPECT(ws >= S * s.hidden * eb * 4 + S * s.ffn * eb, "workspace %zu too small", ws);
  EXPECT(specfold_stack_workspace_bytes(&s) == ws + S * s.hidden * eb, "stack workspace");
  for (int which = -1; which <= 4; ++which) {
    int64_t ld = -7;
    const size_t off = specfold_workspace_offset(&s, which, &ld);
    if (which < 0 || which > 3) {
      EXPECT(off == SIZE_MAX, "bad tensor id %d accepted", which);
    } else {
      const int64_t cols = which == 0 ? (int64_t)(s.n_q_heads + 2 * s.n_kv_heads) * s.head_dim
                           : which == 1 ? (int64_t)s.n_q_heads * s.head_dim
                                        : (int64_t)s.hidden;
      EXPECT(off < ws && off % 256 == 0 && ld >= cols, "tensor %d at %zu ld %lld", which, off,
             (long long)ld);
    }
  }
  for (int vocab : {INT_MIN, -1, 0, 1, 152064, 1 << 24, (1 << 24) + 1, INT_MAX}) {
    const size_t lw = specfold_lm_head_workspace_bytes(&s, vocab);
    if (vocab < 1 || vocab > (1 << 24)) EXPECT(lw == 0, "vocab %d accepted", vocab);
    else EXPECT(lw >= S * s.hidden * eb, "LM head workspace %zu", lw);
  }
}

void fuzz_shapes() {
  const specfold_shape b = base_shape();
  check_sizes(b);
  int32_t specfold_shape::*fields[] = {&specfold_shape::num_nodes, &specfold_shape::block,
                                       &specfold_shape::hidden, &specfold_shape::n_q_heads,
                                       &specfold_shape::n_kv_heads, &specfold_shape::head_dim,
                                       &specfold_shape::ffn, &specfold_shape::prefix_len,
                                       &specfold_shape::dtype};
  for (auto f : fields)
    for (int v : kInts) {
      specfold_shape s = b;
      s.*f = v;
      check_sizes(s);
    }
  for (float v : kFloats) {
    specfold_shape s = b;
    s.rms_eps = v;
    check_sizes(s);
    s = b;
    s.rope_theta = v;
    check_sizes(s);
  }
  // seeded random combinations (64-bit LCG)
  uint64_t x = 0x9e3779b97f4a7c15ull;
  auto next = [&](int n) {
    x = x * 6364136223846793005ull + 1442695040888963407ull;
    return (int)((x >> 33) % (uint64_t)n);
  };
  for (int it = 0; it < 20000; ++it) {
    specfold_shape s = b;
    for (auto f : fields)
      if (next(3) == 0) s.*f = kInts[next(kNI)];
    if (next(4) == 0) s.rms_eps = kFloats[next(kNF)];
    if (next(4) == 0) s.rope_theta = kFloats[next(kNF)];
    if (next(2) == 0) s.dtype = next(2);
    check_sizes(s);
  }
}

const uintptr_t FAKE = 0x7f0000000000ull;
void* P(uintptr_t off = 0) { return (void*)(FAKE + off); }

specfold_layer_weights weights() {
  specfold_layer_weights w{};
  w.rms1 = P(); w.w_qkv = P(); w.w_o = P(); w.rms2 = P(); w.w_gate_up = P(); w.w_down = P();
  return w;
}

// Entry points with arguments the host checks reject; each call must return `want`.
void reject_calls() {
  const specfold_shape s = base_shape();
  const size_t need = specfold_layer_workspace_bytes(&s);
  specfold_kv_view kv{P(), P(), 1024, 128};
  auto fwd = [&](specfold_status want, specfold_layer_weights w, const specfold_kv_view* pv,
                 void* hin, void* hout, const int32_t* fs, uint32_t flags,
                 specfold_fold_state* st, void* ws, size_t wsb, const char* what) {
    const specfold_status got = specfold_layer_forward(&s, &w, pv, hin, hout, fs, 0.05f, st,
                                                       flags, ws, wsb, nullptr);
    EXPECT(got == want, "%s: status %d, want %d (%s)", what, got, want, specfold_last_error());
    // the static variant takes no workspace: only the cases about other arguments apply
    if (ws == (void*)(FAKE + (1ull << 34)) && wsb == need) {
      const specfold_status got2 = specfold_layer_forward_static(&s, &w, pv, hin, hout, fs,
                                                                 0.05f, st, flags, nullptr);
      EXPECT(got2 == want, "%s (static): status %d", what, got2);
    }
  };
  const int32_t* fs = (const int32_t*)P(64);
  specfold_layer_weights w = weights();
  w.w_o = nullptr;
  fwd(SPECFOLD_ERR_INVALID_ARGUMENT, w, &kv, P(), P(1ull << 32), fs, 0, nullptr, P(1ull << 34),
      need, "missing weight");
  w = weights();
  w.w_down = P(8);
  fwd(SPECFOLD_ERR_INVALID_ARGUMENT, w, &kv, P(), P(1ull << 32), fs, 0, nullptr, P(1ull << 34),
      need, "misaligned weight");
  fwd(SPECFOLD_ERR_INVALID_ARGUMENT, weights(), &kv, P(), P(), fs, 0, nullptr, P(1ull << 34),
      need, "aliasing hidden buffers");
  fwd(SPECFOLD_ERR_INVALID_ARGUMENT, weights(), nullptr, P(), P(1ull << 32), fs, 0, nullptr,
      P(1ull << 34), need, "missing prefix");
  specfold_kv_view odd{P(), P(), 1001, 128};
  fwd(SPECFOLD_ERR_INVALID_ARGUMENT, weights(), &odd, P(), P(1ull << 32), fs, 0, nullptr,
      P(1ull << 34), need, "misaligned prefix stride");
  specfold_kv_view neg{P(), P(), -1024, 128};
  fwd(SPECFOLD_ERR_INVALID_ARGUMENT, weights(), &neg, P(), P(1ull << 32), fs, 0, nullptr,
      P(1ull << 34), need, "negative prefix stride");
  specfold_kv_view huge{P(), P(), 1ll << 40, 128};
  fwd(SPECFOLD_ERR_UNSUPPORTED, weights(), &huge, P(), P(1ull << 32), fs, 0, nullptr,
      P(1ull << 34), need, "token stride beyond the prefix kernels' reach");
  fwd(SPECFOLD_ERR_INVALID_ARGUMENT, weights(), &kv, P(), P(1ull << 32), nullptr, 0, nullptr,
      P(1ull << 34), need, "missing fold_src");
  fwd(SPECFOLD_ERR_INVALID_ARGUMENT, weights(), &kv, P(), P(1ull << 32), fs, 0x80, nullptr,
      P(1ull << 34), need, "unknown flag");
  specfold_fold_state partial{};
  partial.recompute = (uint8_t*)P();
  fwd(SPECFOLD_ERR_INVALID_ARGUMENT, weights(), &kv, P(), P(1ull << 32), fs,
      SPECFOLD_FLAG_FOLD_STATE_IN, &partial, P(1ull << 34), need, "partial fold state");
  fwd(SPECFOLD_ERR_WORKSPACE, weights(), &kv, P(), P(1ull << 32), fs, 0, nullptr, P(1ull << 34),
      need - 1, "short workspace");
  fwd(SPECFOLD_ERR_WORKSPACE, weights(), &kv, P(), P(1ull << 32), fs, 0, nullptr, nullptr, need,
      "no workspace");
  fwd(SPECFOLD_ERR_INVALID_ARGUMENT, weights(), &kv, P(), P(1ull << 32), fs, 0, nullptr,
      P((1ull << 34) + 16), need, "misaligned workspace");

  // stacks: per-layer checks name the layer
  specfold_layer_weights ws3[3] = {weights(), weights(), weights()};
  ws3[2].w_qkv = nullptr;
  specfold_kv_view kv3[3] = {kv, kv, kv};
  const size_t sneed = specfold_stack_workspace_bytes(&s);
  specfold_status st = specfold_stack_forward(&s, 3, ws3, kv3, P(), P(1ull << 32), fs, 0.05f,
                                              nullptr, 0, P(1ull << 34), sneed, nullptr);
  EXPECT(st == SPECFOLD_ERR_INVALID_ARGUMENT && strstr(specfold_last_error(), "layer 2"),
         "stack missing weight: %d %s", st, specfold_last_error());
  ws3[2] = weights();
  st = specfold_stack_forward(&s, 0, ws3, kv3, P(), P(1ull << 32), fs, 0.05f, nullptr, 0,
                              P(1ull << 34), sneed, nullptr);
  EXPECT(st == SPECFOLD_ERR_INVALID_ARGUMENT, "stack of 0 layers: %d", st);
  st = specfold_stack_forward(&s, 3, ws3, kv3, P(1ull << 34), P(1ull << 32), fs, 0.05f, nullptr,
                              0, P(1ull << 34), sneed, nullptr);
  EXPECT(st == SPECFOLD_ERR_INVALID_ARGUMENT, "stack input inside the workspace: %d", st);
  st = specfold_stack_forward(&s, 3, ws3, kv3, P(), P(1ull << 32), fs, 0.05f, nullptr, 0,
                              P(1ull << 34), sneed - 1, nullptr);
  EXPECT(st == SPECFOLD_ERR_WORKSPACE, "stack short workspace: %d", st);

  // fold steps
  EXPECT(specfold_gate(&s, P(), fs, 0.05f, nullptr, nullptr, nullptr) ==
             SPECFOLD_ERR_INVALID_ARGUMENT, "gate without recompute");
  EXPECT(specfold_gate(&s, P(4), fs, 0.05f, nullptr, (uint8_t*)P(), nullptr) ==
             SPECFOLD_ERR_INVALID_ARGUMENT, "gate misaligned hidden");
  EXPECT(specfold_resolve(&s, (const uint8_t*)P(), nullptr, (int32_t*)P(), nullptr) ==
             SPECFOLD_ERR_INVALID_ARGUMENT, "resolve without fold_src");
  EXPECT(specfold_pack(&s, (const uint8_t*)P(), (const int32_t*)P(), (int32_t*)P(), nullptr,
                       (int32_t*)P(), nullptr) == SPECFOLD_ERR_INVALID_ARGUMENT,
         "pack without slot_row");
  specfold_shape bad = s;
  bad.block = 0;
  EXPECT(specfold_pack(&bad, (const uint8_t*)P(), (const int32_t*)P(), (int32_t*)P(),
                       (int32_t*)P(), (int32_t*)P(), nullptr) == SPECFOLD_ERR_INVALID_ARGUMENT,
         "pack with block 0");
  EXPECT(specfold_gate(nullptr, P(), fs, 0.05f, nullptr, (uint8_t*)P(), nullptr) ==
             SPECFOLD_ERR_INVALID_ARGUMENT, "gate without shape");

  // LM head
  const int V = 152064;
  const size_t lw = specfold_lm_head_workspace_bytes(&s, V);
  void* a[9];
  for (int i = 0; i < 9; ++i) a[i] = P();
  for (int i = 0; i < 9; ++i) {
    if (i == 7) continue;   // row_logit is optional
    void* b[9];
    memcpy(b, a, sizeof a);
    b[i] = nullptr;
    st = specfold_lm_head_argmax(&s, V, b[0], b[1], b[2], (const int32_t*)b[3],
                                 (const int32_t*)b[4], (const int32_t*)b[5], (int32_t*)b[6],
                                 (float*)b[7], (int32_t*)b[8], P(1ull << 34), lw, nullptr);
    EXPECT(st == SPECFOLD_ERR_INVALID_ARGUMENT, "LM head pointer %d missing: %d", i, st);
  }
  st = specfold_lm_head_argmax(&s, INT_MAX, a[0], a[1], a[2], (const int32_t*)a[3],
                               (const int32_t*)a[4], (const int32_t*)a[5], (int32_t*)a[6],
                               (float*)a[7], (int32_t*)a[8], P(1ull << 34), lw, nullptr);
  EXPECT(st == SPECFOLD_ERR_INVALID_ARGUMENT, "LM head vocab INT_MAX: %d", st);
}

}  // namespace

int main() {
  fuzz_shapes();
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess) ndev = 0;
  (void)hipGetLastError();
  if (ndev > 0) {
    printf("a GPU is present: entry-point rejection calls skipped (they run on the CPU only)\n");
  } else {
    reject_calls();
  }
  printf("%s: %d failure(s)\n", g_failures ? "FAILED" : "OK", g_failures);
  return g_failures ? 1 : 0;
}
