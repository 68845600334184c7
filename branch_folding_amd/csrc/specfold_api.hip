// C ABI of the folded multi-branch verify layer: argument checks, workspace carving and
// the launch sequence.  Everything is enqueued on the caller's stream; nothing here
// synchronises or allocates device memory.  Global state: per-device caches of the
// compute-unit count and of the static workspace's device address, and the static
// workspace itself (specfold_layer_forward_static).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>

#include "../../include/specfold.h"
#include "common.h"
#include "kernels.h"

using namespace specfold;

// Workspace of specfold_layer_forward_static: a statically allocated device array, one
// copy per GPU, held until the process ends.  Host code never passes `specfold_scratch`
// itself to a kernel (its name stands for a host-side shadow, not a device address).
// It has external linkage on purpose: in a build without relocatable device code the
// device code object exports only externally linked variables in its dynamic symbol
// table, where hipGetSymbolAddress resolves names; a `static` array stays a local entry
// of .symtab that the runtime cannot find.  The library-specific name keeps its host
// shadow from colliding with another library's symbol.  `used` keeps the device
// compilation from dropping it, since no kernel names it.
static_assert(SPECFOLD_STATIC_WORKSPACE_BYTES % 256 == 0, "static workspace granularity");
__device__ __align__(256) __attribute__((used)) char specfold_scratch[SPECFOLD_STATIC_WORKSPACE_BYTES];
// Result of the draft-graph check (debug mode only): first offending node, its entry.
__device__ __align__(16) __attribute__((used)) int32_t specfold_debug_result[2];

namespace {

thread_local std::string g_last_error;

specfold_status fail(specfold_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

specfold_status ok() {
  g_last_error.clear();
  return SPECFOLD_OK;
}

#define HIP_CHECK(expr)                                                                  \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess)                                                                \
      return fail(SPECFOLD_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));      \
  } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_bytes(const specfold_shape* s) { return s->dtype == SPECFOLD_BF16 ? 2 : 4; }

// Largest supported model dimensions (well above today's largest open models).
constexpr int kMaxHidden = 32768;
constexpr int kMaxFfn = 131072;
constexpr int kMaxHeads = 256;
constexpr int kMaxPrefix = 1 << 24;
constexpr int kMaxVocab = 1 << 24;
constexpr int64_t kMaxTokStrideBytes = 1LL << 26;   // 64 MB per prefix token

specfold_status check_graph_shape(const specfold_shape* s) {
  if (!s) return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "shape is NULL");
  if (s->num_nodes < 1 || s->block < 1)
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "num_nodes and block must be >= 1 (got %d, %d)",
                s->num_nodes, s->block);
  if (s->block > 1024)
    return fail(SPECFOLD_ERR_UNSUPPORTED, "block %d > 1024 is not supported", s->block);
  if ((long)s->num_nodes * s->block > 16384)
    return fail(SPECFOLD_ERR_UNSUPPORTED, "num_nodes * block = %ld > 16384 is not supported",
                (long)s->num_nodes * s->block);
  return SPECFOLD_OK;
}

specfold_status check_shape(const specfold_shape* s, bool layer) {
  specfold_status st = check_graph_shape(s);
  if (st != SPECFOLD_OK) return st;
  if (s->dtype != SPECFOLD_F32 && s->dtype != SPECFOLD_BF16)
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "dtype %d is not a specfold_dtype", s->dtype);
  if (s->hidden < 128 || s->hidden % 128 != 0)
    return fail(SPECFOLD_ERR_UNSUPPORTED, "hidden %d must be a positive multiple of 128",
                s->hidden);
  // upper limits keep every size and index the kernels form in 32-bit range
  if (s->hidden > kMaxHidden)
    return fail(SPECFOLD_ERR_UNSUPPORTED, "hidden %d > %d is not supported", s->hidden,
                kMaxHidden);
  if (!(s->rms_eps >= 0.f) || s->rms_eps == __builtin_inff())
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "rms_eps must be finite and >= 0");
  if (!layer) return SPECFOLD_OK;
  if (s->ffn < 128 || s->ffn % 128 != 0)
    return fail(SPECFOLD_ERR_UNSUPPORTED, "ffn %d must be a positive multiple of 128", s->ffn);
  if (s->ffn > kMaxFfn)
    return fail(SPECFOLD_ERR_UNSUPPORTED, "ffn %d > %d is not supported", s->ffn, kMaxFfn);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(SPECFOLD_ERR_UNSUPPORTED, "head_dim %d must be 64 or 128", s->head_dim);
  if (s->n_q_heads < 1 || s->n_kv_heads < 1)
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "head counts must be >= 1");
  if (s->n_q_heads > kMaxHeads)
    return fail(SPECFOLD_ERR_UNSUPPORTED, "n_q_heads %d > %d is not supported", s->n_q_heads,
                kMaxHeads);
  if (s->n_q_heads % s->n_kv_heads != 0)
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "n_q_heads %d is not a multiple of n_kv_heads %d",
                s->n_q_heads, s->n_kv_heads);
  if (s->prefix_len < 0) return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "prefix_len < 0");
  if (s->prefix_len > kMaxPrefix)
    return fail(SPECFOLD_ERR_UNSUPPORTED, "prefix_len %d > %d is not supported", s->prefix_len,
                kMaxPrefix);
  if (!(s->rope_theta >= 0.f) || s->rope_theta == __builtin_inff())
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "rope_theta must be finite and >= 0");
  return SPECFOLD_OK;
}

// Compute units of the current device, cached per device (threads may race to fill an entry;
// they all store the same value).
int num_cus() {
  static std::atomic<int> cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kPlanCUs;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
      v = kPlanCUs;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Row stride (elements) of a workspace activation matrix with `cols` columns: one extra
// 128-byte cache line per row, so rows that many workgroups read at the same column do not
// all map to the same few L2 channels.
size_t padded_ld(size_t cols, size_t eb) { return cols + 128 / eb; }

// Workspace layout of one layer.
struct Layout {
  size_t ratio, rec, src, packed, slot_row, count;
  size_t qkv, part_o, part_lse, attn, h, a2, G, F, gpart, plan;
  size_t total;
  size_t ld_d, ld_qkv, ld_q, ld_ff;   // padded row strides (elements)
};

Layout layout_of(const specfold_shape* s) {
  const size_t S = (size_t)s->num_nodes * s->block;
  const size_t eb = elem_bytes(s);
  const size_t d = s->hidden, ff = s->ffn, dh = s->head_dim;
  const size_t qkvd = (size_t)(s->n_q_heads + 2 * s->n_kv_heads) * dh;
  const size_t qd = (size_t)s->n_q_heads * dh;
  const int g = s->n_q_heads / s->n_kv_heads;
  const size_t prow = attn_partial_rows((int)S, g, s->n_kv_heads, s->prefix_len, (int)dh, (int)eb);
  size_t gp = 0;
  const int ebi = (int)eb;
  gp = std::max(gp, gemm_partial_elems((int)S, (int)qkvd, (int)d, ebi));
  gp = std::max(gp, gemm_partial_elems((int)S, (int)d, (int)qd, ebi, true));
  gp = std::max(gp, gemm_partial_elems((int)S, (int)d, (int)ff, ebi));
  Layout L;
  L.ld_d = padded_ld(d, eb);
  L.ld_qkv = padded_ld(qkvd, eb);
  L.ld_q = padded_ld(qd, eb);
  L.ld_ff = padded_ld(ff, eb);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L.ratio = take(S * 4);
  L.rec = take(S);
  L.src = take(S * 4);
  L.packed = take(S * 4);
  L.slot_row = take(S * 4);
  L.count = take(256);
  L.plan = take(256);
  L.qkv = take(S * L.ld_qkv * eb);
  L.part_o = take(prow * qd * 4);
  L.part_lse = take(prow * (size_t)s->n_q_heads * 4);
  L.attn = take(S * L.ld_q * eb);
  L.h = take(S * d * eb);
  L.a2 = take(S * L.ld_d * eb);
  L.G = take(S * L.ld_ff * eb);
  L.F = take(S * d * eb);
  L.gpart = take(gp * 4);
  L.total = off;
  return L;
}

// The next layer's gate, run by this layer's combine (layer stacks): its RMSNorm gain,
// threshold and fold-state outputs.  Its normalised rows go to this workspace's A2 buffer,
// where the next layer's QKV GEMM reads them.
struct NextGate {
  const void* rms1;
  float tau;
  float* ratio;
  uint8_t* rec;
};

// Workspace of the LM head: normalised rows, then the argmax partials.
struct LmLayout {
  size_t an, val, idx, total, ld_an;
};
LmLayout lm_layout(const specfold_shape* s, int vocab) {
  const size_t S = (size_t)s->num_nodes * s->block, eb = elem_bytes(s);
  const size_t P = (size_t)gemm_argmax_partials(vocab);
  LmLayout L{};
  L.ld_an = padded_ld(s->hidden, eb);
  L.an = 0;
  L.val = align256(S * L.ld_an * eb);
  L.idx = align256(L.val + S * P * 4);
  L.total = align256(L.idx + S * P * 4);
  return L;
}

template <typename T>
specfold_status run_layer(const specfold_shape* s, const specfold_layer_weights* w,
                          const specfold_kv_view* prefix, const void* hin, void* hout,
                          const int32_t* fold_src, float tau, float* ratio, uint8_t* rec,
                          int32_t* src, int32_t* packed, int32_t* slot_row, int32_t* count,
                          bool state_in, char* ws, const Layout& L, hipStream_t st,
                          const specfold_probe* probe, bool gate_done, const NextGate* next,
                          bool reuse) {
  const int N = s->num_nodes, B = s->block, S = N * B, d = s->hidden, ff = s->ffn;
  const int dh = s->head_dim, nq = s->n_q_heads, nkv = s->n_kv_heads;
  const int qkvd = (nq + 2 * nkv) * dh, qd = nq * dh;
  const int cus = num_cus();
  // row tile of the packed GEMMs: with tau < 0 every slot is packed, so the row count is S.
  // (The O projection always has S rows; at 512 slots its 256-row tiles double the partial
  // planes its finish reads for no gain -- at the 7B layer -2 us in the GEMM, +2.5 us in
  // the finish -- so it takes them from kOprojTallFrom slots.)
  const bool exact = !state_in && tau < 0.f;
  // From kGemmTallExactFrom to kGemmTallFrom slots a folded call's packed row count can fall
  // on either side of kGemmTallAutoFrom, and only the device knows it: there the GEMMs pick
  // their row tile on the device (a call at tau = 0 packs nearly every slot).
  const int bm = (!exact && S >= kGemmTallExactFrom && S < kGemmTallFrom)
                     ? kGemmTileAuto : gemm_tile_m(S, exact);
  constexpr int kOprojTallFrom = 1024;
  // a failure left behind by some earlier, unrelated HIP call on this thread must not be
  // reported as a failure of these launches
  (void)hipGetLastError();
  auto mark = [&](int step, bool begin) -> hipError_t {
    if (!probe || probe->step != step) return hipSuccess;
    void* ev = begin ? probe->start : probe->stop;
    return ev ? hipEventRecord((hipEvent_t)ev, st) : hipSuccess;
  };
  // The gate pass also writes the RMS-normalised rows (QKV input) of the slots that compute
  // their own row into A1, which shares its buffer with the FFN input A2 (written only after
  // the QKV GEMM has consumed A1).  With a given fold state it writes no mask, and ratios
  // only into a caller's ratio buffer.
  // With gate_done the previous layer's combine already ran this gate.
  void* A2 = ws + L.a2;
  HIP_CHECK(mark(SPECFOLD_STEP_GATE, true));
  if (!gate_done)
    HIP_CHECK(launch_gate<T>(hin, fold_src, N, B, d, tau, ratio, state_in ? nullptr : rec,
                             state_in ? rec : nullptr, w->rms1, s->rms_eps, A2, (int)L.ld_d,
                             st));
  HIP_CHECK(mark(SPECFOLD_STEP_GATE, false));
  if (!state_in) {
    HIP_CHECK(mark(SPECFOLD_STEP_RESOLVE_PACK, true));
    HIP_CHECK(launch_resolve_pack(rec, fold_src, nullptr, N, B, kResolve | kPack, src, packed,
                                  slot_row, count, w->w_qkv, (size_t)qkvd * d * sizeof(T), cus,
                                  st));
    HIP_CHECK(mark(SPECFOLD_STEP_RESOLVE_PACK, false));
  }
  void* QKV = ws + L.qkv;
  void* ATT = ws + L.attn;
  void* Hh = ws + L.h;
  void* G = ws + L.G;
  void* F = ws + L.F;
  float* gpart = (float*)(ws + L.gpart);


  // packed rows of A1 are gathered by the GEMM's loads
  GemmParams gp{};
  gp.A = A2; gp.lda = L.ld_d; gp.a_rows = packed; gp.a_rows_cap = S; gp.W = w->w_qkv; gp.ldw = d; gp.C = QKV; gp.ldc = L.ld_qkv;
  gp.partial = gpart; gp.m_dev = count; gp.m_cap = S; gp.N = qkvd; gp.Kd = d; gp.bm = bm;
  // with a QKV bias or rotary embedding the split-K reduction also adds the bias and rotates
  // Q and K (one pass over the partial planes, one rounding to the model dtype)
  const bool qkv_epilogue = w->b_qkv || s->rope_theta > 0.f;
  gp.defer_reduce = qkv_epilogue ? 1 : 0;
  HIP_CHECK(mark(SPECFOLD_STEP_QKV, true));
  HIP_CHECK(launch_gemm<T>(gp, kEpiStore, cus, st));
  if (qkv_epilogue)
    HIP_CHECK(launch_qkv_reduce_rope_bias<T>(gp, packed, B, s->prefix_len, nq, nkv, dh,
                                             w->b_qkv, s->rope_theta, st));
  HIP_CHECK(mark(SPECFOLD_STEP_QKV, false));

  AttnParams ap{};
  ap.qkv = QKV; ap.ld_qkv = L.ld_qkv; ap.n_q = nq; ap.n_kv = nkv; ap.dh = dh;
  ap.count = count; ap.cap = S;
  ap.pk = prefix ? prefix->k : nullptr; ap.pv = prefix ? prefix->v : nullptr;
  ap.stride_tok = prefix ? prefix->stride_tok : 0; ap.stride_head = prefix ? prefix->stride_head : 0;
  ap.P = s->prefix_len;
  ap.scale_log2 = (float)(1.4426950408889634 / sqrt((double)dh));
  ap.part_o = ws + L.part_o; ap.part_lse = (float*)(ws + L.part_lse);
  ap.plan = (int32_t*)(ws + L.plan);
  ap.S = S; ap.slot_row = slot_row; ap.N = N; ap.B = B; ap.out = ATT; ap.ld_out = L.ld_q;
  ap.fused = attn_fused_prefix(s->prefix_len, N, B, nq, nkv, cus) ? 1 : 0;
  HIP_CHECK(mark(SPECFOLD_STEP_ATTN_PREFIX, true));
  HIP_CHECK(launch_attn_prefix<T>(ap, cus, st));
  HIP_CHECK(mark(SPECFOLD_STEP_ATTN_PREFIX, false));
  HIP_CHECK(mark(SPECFOLD_STEP_ATTN_BLOCK, true));
  HIP_CHECK(launch_attn_block<T>(ap, cus, st));
  HIP_CHECK(mark(SPECFOLD_STEP_ATTN_BLOCK, false));

  // O projection over every slot (with the REUSE variant: over the packed rows, gathered
  // by packed_slot, whose results every slot takes through slot_row): fp32 partials, then
  // one row pass adds the residual and computes the FFN's RMSNorm for the packed rows
  gp = GemmParams{};
  gp.A = ATT; gp.lda = L.ld_q; gp.W = w->w_o; gp.ldw = qd; gp.C = nullptr; gp.ldc = d;
  gp.partial = gpart; gp.m_dev = reuse ? count : nullptr; gp.m_cap = S; gp.N = d; gp.Kd = qd;
  // Without REUSE the O projection's row count is S on the host whatever tau decides, so
  // from kOprojTallFrom slots it takes the 256-row tiles (3B layer, 1024 slots: 29.0 us
  // against 34.6-38.0 us with 128-row tiles).
  gp.bm = reuse ? bm : (S >= kOprojTallFrom ? 256 : (bm == kGemmTileAuto ? 128 : bm));
  if (reuse) {
    gp.a_rows = packed;
    gp.a_rows_cap = S;
  }
  HIP_CHECK(mark(SPECFOLD_STEP_O_PROJ, true));
  HIP_CHECK(launch_gemm<T>(gp, kEpiPartial, cus, st));
  HIP_CHECK(mark(SPECFOLD_STEP_O_PROJ, false));
  HIP_CHECK(mark(SPECFOLD_STEP_RMSNORM2, true));
  HIP_CHECK(launch_oproj_finish<T>(gpart, gemm_host_split(S, d, qd, (int)sizeof(T), gp.bm), hin,
                                   Hh, S, d, slot_row, packed, count, w->rms2, s->rms_eps, A2,
                                   (int)L.ld_d, reuse, ceil_div(d, gemm_tile_n(d)),
                                   qd / (kGemmBKBytes / (int)sizeof(T)), gp.bm, st));
  HIP_CHECK(mark(SPECFOLD_STEP_RMSNORM2, false));

  gp = GemmParams{};
  gp.A = A2; gp.lda = L.ld_d; gp.W = w->w_gate_up; gp.ldw = d; gp.C = G; gp.ldc = L.ld_ff;
  gp.partial = gpart; gp.m_dev = count; gp.m_cap = S; gp.N = 2 * ff; gp.Kd = d; gp.ff = ff;
  gp.bm = bm;
  // the FFN weights are read once per call and nothing reads them ahead: streamed loads
  // (QKV and O weights are read ahead into the memory-side cache and keep the default)
  gp.w_stream = 1;
  // a probe of this step times the kernel itself when the step is one launch (its events
  // taken at the kernel's start and end, as a kernel trace does); else it brackets the launches
  KernelTimer kt{};
  const bool timed = probe && probe->step == SPECFOLD_STEP_FFN_GATE_UP && probe->start &&
                     probe->stop && swiglu_single_launch(gp);
  if (timed) kt = KernelTimer{(hipEvent_t)probe->start, (hipEvent_t)probe->stop};
  if (!timed) HIP_CHECK(mark(SPECFOLD_STEP_FFN_GATE_UP, true));
  HIP_CHECK(launch_gemm<T>(gp, kEpiSwiGLU, cus, st, timed ? &kt : nullptr));
  if (!timed) HIP_CHECK(mark(SPECFOLD_STEP_FFN_GATE_UP, false));

  gp = GemmParams{};
  gp.A = G; gp.lda = L.ld_ff; gp.W = w->w_down; gp.ldw = ff; gp.C = F; gp.ldc = d;
  gp.partial = gpart; gp.m_dev = count; gp.m_cap = S; gp.N = d; gp.Kd = ff; gp.bm = bm;
  gp.w_stream = 1;
  HIP_CHECK(mark(SPECFOLD_STEP_FFN_DOWN, true));
  HIP_CHECK(launch_gemm<T>(gp, kEpiStore, cus, st));
  HIP_CHECK(mark(SPECFOLD_STEP_FFN_DOWN, false));

  HIP_CHECK(mark(SPECFOLD_STEP_COMBINE, true));
  if (next)
    HIP_CHECK(launch_combine_gate<T>(Hh, F, slot_row, count, S, hout, fold_src, N, B, d,
                                     next->tau, next->ratio, next->rec, next->rms1, s->rms_eps,
                                     A2, (int)L.ld_d, st));
  else
    HIP_CHECK(launch_combine<T>(Hh, F, slot_row, count, S, S, d, hout, st));
  HIP_CHECK(mark(SPECFOLD_STEP_COMBINE, false));
  return ok();
}

specfold_status check_flags(uint32_t flags) {
  if (flags & ~(SPECFOLD_FLAG_FOLD_STATE_IN | SPECFOLD_FLAG_REUSE_ATTENTION))
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "unknown flag bits 0x%x", flags);
  return SPECFOLD_OK;
}

size_t hidden_bytes(const specfold_shape* s) {
  return (size_t)s->num_nodes * s->block * s->hidden * elem_bytes(s);
}

// Weights and prefix view of one layer (`layer` < 0: a single-layer call).
specfold_status check_layer_params(const specfold_shape* shape,
                                   const specfold_layer_weights* weights,
                                   const specfold_kv_view* prefix, int layer) {
  char at[32] = "";
  if (layer >= 0) snprintf(at, sizeof at, " (layer %d)", layer);
  if (!weights || !weights->rms1 || !weights->w_qkv || !weights->w_o || !weights->rms2 ||
      !weights->w_gate_up || !weights->w_down)
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "every layer weight pointer is required%s", at);
  const void* wp[7] = {weights->rms1, weights->w_qkv, weights->w_o, weights->rms2,
                       weights->w_gate_up, weights->w_down, weights->b_qkv};
  for (int i = 0; i < 7; ++i)
    if (!aligned16(wp[i]))
      return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "weight pointer %d is not 16-byte aligned%s", i,
                  at);
  const int64_t eb = elem_bytes(shape);
  if (shape->prefix_len > 0) {
    if (!prefix || !prefix->k || !prefix->v)
      return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "prefix_len > 0 needs a prefix view%s", at);
    if (!aligned16(prefix->k) || !aligned16(prefix->v) || prefix->stride_tok < 0 ||
        prefix->stride_head < 0 || (prefix->stride_tok * eb) % 16 != 0 ||
        (prefix->stride_head * eb) % 16 != 0)
      return fail(SPECFOLD_ERR_INVALID_ARGUMENT,
                  "prefix view pointers and strides must keep rows 16-byte aligned%s", at);
    // the prefix kernels hold a lane's offset inside a 64-key tile in 32 bits
    if (prefix->stride_tok * eb >= kMaxTokStrideBytes)
      return fail(SPECFOLD_ERR_UNSUPPORTED,
                  "prefix stride_tok of %lld elements is %lld bytes; token strides must stay "
                  "below %lld bytes%s", (long long)prefix->stride_tok,
                  (long long)(prefix->stride_tok * eb), (long long)kMaxTokStrideBytes, at);
  }
  return SPECFOLD_OK;
}

specfold_status check_hidden(const specfold_shape* shape, const void* hidden_in,
                             const void* hidden_out) {
  if (!hidden_in || !hidden_out)
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "hidden_in and hidden_out are required");
  if (!aligned16(hidden_in) || !aligned16(hidden_out))
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "hidden_in/hidden_out must be 16-byte aligned");
  const size_t hb = hidden_bytes(shape);
  const char* a = (const char*)hidden_in;
  const char* b = (const char*)hidden_out;
  if (a < b + hb && b < a + hb)
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "hidden_in and hidden_out overlap");
  return SPECFOLD_OK;
}

specfold_status check_state_in(const specfold_fold_state* state, int layer) {
  char at[32] = "";
  if (layer >= 0) snprintf(at, sizeof at, " (layer %d)", layer);
  if (!state || !state->recompute || !state->src_node || !state->packed_slot ||
      !state->slot_row || !state->packed_count)
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT,
                "SPECFOLD_FLAG_FOLD_STATE_IN needs every fold-state array except ratio%s", at);
  return SPECFOLD_OK;
}

specfold_status check_workspace(void* workspace, size_t workspace_bytes, size_t need) {
  if (!workspace || workspace_bytes < need)
    return fail(SPECFOLD_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required",
                workspace ? workspace_bytes : (size_t)0, need);
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  return SPECFOLD_OK;
}

// Fold-state buffers of one call (caller's where given, else the workspace's) and the
// launch sequence in the layer's dtype.
// `next_weights` / `next_state` (layer stacks, fold states made on the device): this layer's
// combine also runs the next layer's gate into the next layer's fold-state buffers;
// `gate_done`: the previous layer's combine ran this layer's gate.
specfold_status launch_layer(const specfold_shape* shape, const specfold_layer_weights* weights,
                             const specfold_kv_view* prefix, const void* hidden_in,
                             void* hidden_out, const int32_t* fold_src, float tau,
                             specfold_fold_state* state, bool state_in, char* ws,
                             const Layout& L, hipStream_t s, const specfold_probe* probe,
                             bool gate_done = false,
                             const specfold_layer_weights* next_weights = nullptr,
                             specfold_fold_state* next_state = nullptr, bool reuse = false) {
  auto pick = [&](auto* user, size_t off) {
    using P = decltype(user);
    return user ? user : (P)(ws + off);
  };
  NextGate ng{};
  if (next_weights) {
    ng.rms1 = next_weights->rms1;
    ng.tau = tau;
    ng.ratio = pick(next_state ? next_state->ratio : (float*)nullptr, L.ratio);
    ng.rec = pick(next_state ? next_state->recompute : (uint8_t*)nullptr, L.rec);
  }
  const NextGate* next = next_weights ? &ng : nullptr;
  float* ratio = pick(state ? state->ratio : (float*)nullptr, L.ratio);
  if (state_in && !(state && state->ratio && fold_src)) ratio = nullptr;
  uint8_t* rec = pick(state ? state->recompute : (uint8_t*)nullptr, L.rec);
  int32_t* src = pick(state ? state->src_node : (int32_t*)nullptr, L.src);
  int32_t* packed = pick(state ? state->packed_slot : (int32_t*)nullptr, L.packed);
  int32_t* slot_row = pick(state ? state->slot_row : (int32_t*)nullptr, L.slot_row);
  int32_t* count = pick(state ? state->packed_count : (int32_t*)nullptr, L.count);
  if (shape->dtype == SPECFOLD_BF16)
    return run_layer<bf16>(shape, weights, prefix, hidden_in, hidden_out, fold_src, tau, ratio,
                           rec, src, packed, slot_row, count, state_in, ws, L, s, probe,
                           gate_done, next, reuse);
  return run_layer<float>(shape, weights, prefix, hidden_in, hidden_out, fold_src, tau, ratio,
                          rec, src, packed, slot_row, count, state_in, ws, L, s, probe,
                          gate_done, next, reuse);
}

// Device address of the static workspace on each device, looked up once per device with
// that device current (hipGetSymbolAddress); host code passes only this address on.
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

specfold_status static_workspace(char** out) {
  int dev = -1;
  HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64)
    return fail(SPECFOLD_ERR_UNSUPPORTED, "device ordinal %d is beyond the 64 the static "
                "workspace tracks", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(specfold_scratch)));
    if (p == nullptr || ((uintptr_t)p & 255u) != 0)
      return fail(SPECFOLD_ERR_HIP, "static workspace of device %d has no usable address", dev);
    g_scratch_ptr[dev] = p;
  }
  *out = (char*)g_scratch_ptr[dev];
  return SPECFOLD_OK;
}

// Optional check of the draft graph before a call's kernels run (SPECFOLD_DEBUG set to
// anything but "" or "0" in the environment): a one-workgroup kernel looks for a node whose
// fold_src entry breaks the topological numbering and the call returns
// SPECFOLD_ERR_INVALID_ARGUMENT naming it.  Without the check, such entries are clamped on
// the device (wrong results, no out-of-range access).  The check waits for the caller's
// stream, so a call in debug mode cannot be captured into a graph.
bool debug_checks() {
  const char* e = getenv("SPECFOLD_DEBUG");   // read on every call: a process may toggle it
  return e && *e && strcmp(e, "0") != 0;
}

std::mutex g_debug_mu;

specfold_status debug_check_fold_src(const int32_t* fold_src, int N, hipStream_t s) {
  if (!debug_checks() || !fold_src) return SPECFOLD_OK;
  std::lock_guard<std::mutex> lock(g_debug_mu);
  (void)hipGetLastError();
  void* res = nullptr;
  HIP_CHECK(hipGetSymbolAddress(&res, HIP_SYMBOL(specfold_debug_result)));
  HIP_CHECK(launch_check_fold_src(fold_src, N, (int32_t*)res, s));
  int32_t host[2] = {0, 0};
  HIP_CHECK(hipMemcpyAsync(host, res, sizeof host, hipMemcpyDeviceToHost, s));
  HIP_CHECK(hipStreamSynchronize(s));
  if (host[0] >= 0)
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT,
                "fold_src[%d] = %d: the root needs -1 and node n a fold source in [0, n) "
                "(SPECFOLD_DEBUG check)", host[0], host[1]);
  return SPECFOLD_OK;
}

}  // namespace

extern "C" {

specfold_status specfold_gate(const specfold_shape* shape, const void* hidden,
                              const int32_t* fold_src, float tau, float* ratio,
                              uint8_t* recompute, void* stream) {
  specfold_status st = check_shape(shape, false);
  if (st != SPECFOLD_OK) return st;
  if (!hidden || !fold_src || !recompute)
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "hidden, fold_src and recompute are required");
  if (!aligned16(hidden)) return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "hidden is not 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const specfold_shape* sh = shape;
  (void)hipGetLastError();   // do not report an earlier, unrelated failure
  if ((st = debug_check_fold_src(fold_src, sh->num_nodes, s)) != SPECFOLD_OK) return st;
  if (sh->dtype == SPECFOLD_BF16) {
    HIP_CHECK(launch_gate<bf16>(hidden, fold_src, sh->num_nodes, sh->block, sh->hidden, tau,
                                ratio, recompute, nullptr, nullptr, 0.f, nullptr, 0, s));
  } else {
    HIP_CHECK(launch_gate<float>(hidden, fold_src, sh->num_nodes, sh->block, sh->hidden, tau,
                                 ratio, recompute, nullptr, nullptr, 0.f, nullptr, 0, s));
  }
  return ok();
}

specfold_status specfold_resolve(const specfold_shape* shape, const uint8_t* recompute,
                                 const int32_t* fold_src, int32_t* src_node, void* stream) {
  specfold_status st = check_graph_shape(shape);
  if (st != SPECFOLD_OK) return st;
  if (!recompute || !fold_src || !src_node)
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "recompute, fold_src and src_node are required");
  (void)hipGetLastError();
  st = debug_check_fold_src(fold_src, shape->num_nodes, (hipStream_t)stream);
  if (st != SPECFOLD_OK) return st;
  HIP_CHECK(launch_resolve_pack(recompute, fold_src, nullptr, shape->num_nodes, shape->block,
                                kResolve, src_node, nullptr, nullptr, nullptr, nullptr, 0, 0,
                                (hipStream_t)stream));
  return ok();
}

specfold_status specfold_pack(const specfold_shape* shape, const uint8_t* recompute,
                              const int32_t* src_node, int32_t* packed_slot,
                              int32_t* slot_row, int32_t* packed_count, void* stream) {
  specfold_status st = check_graph_shape(shape);
  if (st != SPECFOLD_OK) return st;
  if (!recompute || !src_node || !packed_slot || !slot_row || !packed_count)
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT,
                "recompute, src_node, packed_slot, slot_row and packed_count are required");
  (void)hipGetLastError();
  HIP_CHECK(launch_resolve_pack(recompute, nullptr, src_node, shape->num_nodes, shape->block,
                                kPack, nullptr, packed_slot, slot_row, packed_count, nullptr, 0,
                                0, (hipStream_t)stream));
  return ok();
}

size_t specfold_layer_workspace_bytes(const specfold_shape* shape) {
  if (check_shape(shape, true) != SPECFOLD_OK) return 0;
  g_last_error.clear();
  return layout_of(shape).total;
}

size_t specfold_workspace_offset(const specfold_shape* shape, int32_t which, int64_t* ld) {
  if (check_shape(shape, true) != SPECFOLD_OK) return SIZE_MAX;
  const Layout L = layout_of(shape);
  int64_t dummy;
  if (!ld) ld = &dummy;
  switch (which) {
    case SPECFOLD_T_QKV: *ld = (int64_t)L.ld_qkv; return L.qkv;
    case SPECFOLD_T_ATTN: *ld = (int64_t)L.ld_q; return L.attn;
    case SPECFOLD_T_H: *ld = shape->hidden; return L.h;
    case SPECFOLD_T_FFN: *ld = shape->hidden; return L.F;
    default:
      fail(SPECFOLD_ERR_INVALID_ARGUMENT, "unknown tensor id %d", which);
      return SIZE_MAX;
  }
}

specfold_status specfold_layer_forward(const specfold_shape* shape,
                                       const specfold_layer_weights* weights,
                                       const specfold_kv_view* prefix, const void* hidden_in,
                                       void* hidden_out, const int32_t* fold_src, float tau,
                                       specfold_fold_state* state, uint32_t flags,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  return specfold_layer_forward_probed(shape, weights, prefix, hidden_in, hidden_out, fold_src,
                                       tau, state, flags, workspace, workspace_bytes, stream,
                                       nullptr);
}

specfold_status specfold_layer_forward_probed(const specfold_shape* shape,
                                              const specfold_layer_weights* weights,
                                              const specfold_kv_view* prefix,
                                              const void* hidden_in, void* hidden_out,
                                              const int32_t* fold_src, float tau,
                                              specfold_fold_state* state, uint32_t flags,
                                              void* workspace, size_t workspace_bytes,
                                              void* stream, const specfold_probe* probe) {
  specfold_status st = check_shape(shape, true);
  if (st != SPECFOLD_OK) return st;
  if ((st = check_flags(flags)) != SPECFOLD_OK) return st;
  const bool state_in = (flags & SPECFOLD_FLAG_FOLD_STATE_IN) != 0;
  if ((st = check_layer_params(shape, weights, prefix, -1)) != SPECFOLD_OK) return st;
  if ((st = check_hidden(shape, hidden_in, hidden_out)) != SPECFOLD_OK) return st;
  if (!state_in && !fold_src)
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "fold_src is required unless the fold state is an input");
  if (state_in && (st = check_state_in(state, -1)) != SPECFOLD_OK) return st;
  const Layout L = layout_of(shape);
  if ((st = check_workspace(workspace, workspace_bytes, L.total)) != SPECFOLD_OK) return st;
  if ((st = debug_check_fold_src(fold_src, shape->num_nodes, (hipStream_t)stream)) != SPECFOLD_OK)
    return st;
  return launch_layer(shape, weights, prefix, hidden_in, hidden_out, fold_src, tau, state,
                      state_in, (char*)workspace, L, (hipStream_t)stream, probe, false, nullptr,
                      nullptr, (flags & SPECFOLD_FLAG_REUSE_ATTENTION) != 0);
}

specfold_status specfold_layer_forward_static(const specfold_shape* shape,
                                              const specfold_layer_weights* weights,
                                              const specfold_kv_view* prefix,
                                              const void* hidden_in, void* hidden_out,
                                              const int32_t* fold_src, float tau,
                                              specfold_fold_state* state, uint32_t flags,
                                              void* stream) {
  specfold_status st = check_shape(shape, true);
  if (st != SPECFOLD_OK) return st;
  if ((st = check_flags(flags)) != SPECFOLD_OK) return st;
  const bool state_in = (flags & SPECFOLD_FLAG_FOLD_STATE_IN) != 0;
  if ((st = check_layer_params(shape, weights, prefix, -1)) != SPECFOLD_OK) return st;
  if ((st = check_hidden(shape, hidden_in, hidden_out)) != SPECFOLD_OK) return st;
  if (!state_in && !fold_src)
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "fold_src is required unless the fold state is an input");
  if (state_in && (st = check_state_in(state, -1)) != SPECFOLD_OK) return st;
  const Layout L = layout_of(shape);
  if (L.total > (size_t)SPECFOLD_STATIC_WORKSPACE_BYTES)
    return fail(SPECFOLD_ERR_WORKSPACE,
                "this shape needs %zu bytes of workspace, more than the %zu-byte static "
                "workspace; call specfold_layer_forward with a caller workspace",
                L.total, (size_t)SPECFOLD_STATIC_WORKSPACE_BYTES);
  char* ws = nullptr;
  if ((st = static_workspace(&ws)) != SPECFOLD_OK) return st;
  if ((st = debug_check_fold_src(fold_src, shape->num_nodes, (hipStream_t)stream)) != SPECFOLD_OK)
    return st;
  // nothing in the workspace has to start at zero: every launch writes what a later
  // launch of the same call reads
  return launch_layer(shape, weights, prefix, hidden_in, hidden_out, fold_src, tau, state,
                      state_in, ws, L, (hipStream_t)stream, nullptr, false, nullptr, nullptr,
                      (flags & SPECFOLD_FLAG_REUSE_ATTENTION) != 0);
}

size_t specfold_stack_workspace_bytes(const specfold_shape* shape) {
  if (check_shape(shape, true) != SPECFOLD_OK) return 0;
  g_last_error.clear();
  return layout_of(shape).total + hidden_bytes(shape);
}

specfold_status specfold_stack_forward(const specfold_shape* shape, int32_t num_layers,
                                       const specfold_layer_weights* weights,
                                       const specfold_kv_view* prefix, const void* hidden_in,
                                       void* hidden_out, const int32_t* fold_src, float tau,
                                       specfold_fold_state* states, uint32_t flags,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  specfold_status st = check_shape(shape, true);
  if (st != SPECFOLD_OK) return st;
  if ((st = check_flags(flags)) != SPECFOLD_OK) return st;
  const bool state_in = (flags & SPECFOLD_FLAG_FOLD_STATE_IN) != 0;
  if (num_layers < 1) return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "num_layers must be >= 1");
  if (!weights) return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "weights array is NULL");
  if (shape->prefix_len > 0 && !prefix)
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "prefix_len > 0 needs an array of prefix views");
  for (int l = 0; l < num_layers; ++l) {
    if ((st = check_layer_params(shape, &weights[l], prefix ? &prefix[l] : nullptr, l)) !=
        SPECFOLD_OK)
      return st;
    if (state_in && (st = check_state_in(states ? &states[l] : nullptr, l)) != SPECFOLD_OK)
      return st;
  }
  if ((st = check_hidden(shape, hidden_in, hidden_out)) != SPECFOLD_OK) return st;
  if (!state_in && !fold_src)
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "fold_src is required unless the fold states are inputs");
  const Layout L = layout_of(shape);
  const size_t hb = hidden_bytes(shape);
  if ((st = check_workspace(workspace, workspace_bytes, L.total + hb)) != SPECFOLD_OK) return st;
  char* ws = (char*)workspace;
  char* pong = ws + L.total;
  {
    // the caller's activations must not live inside the workspace
    const char* w0 = ws;
    const char* w1 = ws + L.total + hb;
    const char* a = (const char*)hidden_in;
    const char* b = (const char*)hidden_out;
    if ((a < w1 && w0 < a + hb) || (b < w1 && w0 < b + hb))
      return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "hidden_in/hidden_out overlap the workspace");
  }
  // layer l writes hidden_out when (num_layers - 1 - l) is even, else the workspace's
  // spare hidden buffer, so consecutive layers never alias and the last writes hidden_out
  // With fold states made on the device, layer l's combine also runs layer l+1's gate on the
  // output it writes (same results, one launch and one pass over the hidden states fewer).
  if ((st = debug_check_fold_src(fold_src, shape->num_nodes, (hipStream_t)stream)) != SPECFOLD_OK)
    return st;
  const bool fuse = !state_in && combine_gate_fits(shape->hidden, (int)elem_bytes(shape));
  const void* x = hidden_in;
  for (int l = 0; l < num_layers; ++l) {
    void* y = ((num_layers - 1 - l) % 2 == 0) ? hidden_out : (void*)pong;
    const bool fuse_next = fuse && l + 1 < num_layers;
    st = launch_layer(shape, &weights[l], prefix ? &prefix[l] : nullptr, x, y, fold_src, tau,
                      states ? &states[l] : nullptr, state_in, ws, L, (hipStream_t)stream,
                      nullptr, fuse && l > 0, fuse_next ? &weights[l + 1] : nullptr,
                      fuse_next && states ? &states[l + 1] : nullptr,
                      (flags & SPECFOLD_FLAG_REUSE_ATTENTION) != 0);
    if (st != SPECFOLD_OK) return st;
    x = y;
  }
  return ok();
}

size_t specfold_lm_head_workspace_bytes(const specfold_shape* shape, int32_t vocab) {
  if (check_shape(shape, false) != SPECFOLD_OK) return 0;
  if (vocab < 1 || vocab > kMaxVocab) {
    fail(SPECFOLD_ERR_INVALID_ARGUMENT, "vocab must be in [1, %d]", kMaxVocab);
    return 0;
  }
  g_last_error.clear();
  return lm_layout(shape, vocab).total;
}

specfold_status specfold_lm_head_argmax(const specfold_shape* shape, int32_t vocab,
                                        const void* rms_final, const void* w_lm,
                                        const void* hidden, const int32_t* packed_slot,
                                        const int32_t* slot_row, const int32_t* packed_count,
                                        int32_t* row_token, float* row_logit, int32_t* token,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  specfold_status st = check_shape(shape, false);
  if (st != SPECFOLD_OK) return st;
  if (vocab < 1 || vocab > kMaxVocab)
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "vocab must be in [1, %d]", kMaxVocab);
  if (!rms_final || !w_lm || !hidden || !packed_slot || !slot_row || !packed_count ||
      !row_token || !token)
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT,
                "rms_final, w_lm, hidden, packed_slot, slot_row, packed_count, row_token and "
                "token are required");
  if (!aligned16(rms_final) || !aligned16(w_lm) || !aligned16(hidden))
    return fail(SPECFOLD_ERR_INVALID_ARGUMENT, "rms_final, w_lm and hidden must be 16-byte aligned");
  const LmLayout L = lm_layout(shape, vocab);
  if ((st = check_workspace(workspace, workspace_bytes, L.total)) != SPECFOLD_OK) return st;
  char* ws = (char*)workspace;
  LmHeadParams q{};
  q.hidden = hidden; q.rms = rms_final; q.w = w_lm; q.packed_slot = packed_slot;
  q.slot_row = slot_row; q.count = packed_count; q.N = shape->num_nodes; q.B = shape->block;
  q.d = shape->hidden; q.V = vocab; q.eps = shape->rms_eps; q.An = ws + L.an;
  q.ld_an = (int)L.ld_an; q.arg_val = (float*)(ws + L.val); q.arg_idx = (int32_t*)(ws + L.idx);
  q.row_token = row_token; q.row_logit = row_logit; q.token = token;
  (void)hipGetLastError();
  if (shape->dtype == SPECFOLD_BF16)
    HIP_CHECK(launch_lm_head<bf16>(q, num_cus(), (hipStream_t)stream));
  else
    HIP_CHECK(launch_lm_head<float>(q, num_cus(), (hipStream_t)stream));
  return ok();
}

const char* specfold_last_error(void) { return g_last_error.c_str(); }

int32_t specfold_version(void) { return 200; }

}  // extern "C"
