// Internal launchers of the folded verify-layer kernels (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace specfold {

// resolve_pack modes
constexpr int kResolve = 1;
constexpr int kPack = 2;

// Gate: writes ratio[slot] and recompute[slot] where those pointers are non-null, and with
// An the normalised row An[slot] = H[slot] * rstd * g (row stride ld_an) of every slot that
// computes its own row (as decided here, or as rec_given marks when it is non-null).
template <typename T>
hipError_t launch_gate(const void* H, const int32_t* fold_src, int N, int B, int d, float tau,
                       float* ratio, uint8_t* recompute, const uint8_t* rec_given,
                       const void* g, float eps, void* An, int ld_an, hipStream_t st);
// Combine of one layer fused with the next layer's gate: y = h + F[slot_row] (rounded to
// T), then the gate of y against its fold source's y with the next layer's tau and RMSNorm
// gain g, writing ratio / recompute (where non-null) and the normalised rows An of the slots
// that recompute.  Only for rows of at most 512 16-byte chunks (combine_gate_fits).
bool combine_gate_fits(int d, int elem_bytes);
template <typename T>
hipError_t launch_combine_gate(const void* h, const void* F, const int32_t* slot_row,
                               const int32_t* count, int cap, void* y, const int32_t* fold_src,
                               int N, int B, int d, float tau, float* ratio, uint8_t* recompute,
                               const void* g, float eps, void* An, int ld_an, hipStream_t st);
size_t resolve_pack_lds_bytes(int S);
// prefetch (may be nullptr): up to a fixed number of its bytes are read by otherwise idle
// workgroups of the same launch, so the following kernel finds them in the memory-side cache.
hipError_t launch_resolve_pack(const uint8_t* recompute, const int32_t* fold_src,
                               const int32_t* src_in, int N, int B, int mode, int32_t* src_out,
                               int32_t* packed_slot, int32_t* slot_row, int32_t* count,
                               const void* prefetch, size_t prefetch_bytes, int num_cu,
                               hipStream_t st);
template <typename T>
hipError_t launch_combine(const void* h, const void* F, const int32_t* slot_row,
                          const int32_t* count, int cap, int S, int d, void* y, hipStream_t st);
// Draft-graph check: out[0] = first node n with fold_src[n] outside its range ([0, n), -1
// for the root) or -1; out[1] = that entry.
hipError_t launch_check_fold_src(const int32_t* fold_src, int N, int32_t* out, hipStream_t st);

// ---------------------------------------------------------------------------------------
// GEMM  C[M, N] = A[M, Kd] . W[N, Kd]^T  (both operands K-contiguous), M read on the
// device.  Epilogues: plain store, + residual, SwiGLU (W = [gate; up], output [M, ff]).
// ---------------------------------------------------------------------------------------
// kEpiPartial: always write fp32 partial sums (plane s of p.partial), even without split-K;
// a row-wise finishing kernel applies the epilogue.
// kEpiArgmax: no C; for every row, the maximum over each wave's 64 columns and its first
// column index go to arg_val / arg_idx [row][arg_ld] (never split over K).
enum GemmEpi { kEpiStore = 0, kEpiResidual = 1, kEpiSwiGLU = 2, kEpiPartial = 3, kEpiArgmax = 4 };

struct GemmParams {
  const void* A;
  long lda;
  const void* W;
  long ldw;
  void* C;
  long ldc;
  const void* R;     // residual (kEpiResidual), [M, N] with leading dimension ldr
  long ldr;
  float* partial;    // split-K partial sums, [split][M][N] fp32
  const int32_t* m_dev;  // device row count (nullptr: m_cap rows)
  int m_cap;
  int N;             // logical output columns (2*ff for SwiGLU)
  int Kd;
  int ff;            // SwiGLU only
  // optional row gather: row m of the A operand is row a_rows[m] of `A` (clamped to
  // [0, a_rows_cap)); nullptr = row m
  const int32_t* a_rows;
  int a_rows_cap;
  // nonzero: the weight tiles are loaded with the nontemporal hint where each is read once
  // (one row tile); for weights read once per call and not read ahead into the memory-side
  // cache by an earlier kernel, the hint keeps them from displacing the activation tiles
  // every CU re-reads from L2.  Honoured by the SwiGLU and kEpiStore launches.  (Placed in
  // what would be padding, so the kernel argument block keeps its size.)
  int w_stream;
  // kEpiArgmax outputs: [m_cap][arg_ld] partial maxima and their column indices
  float* arg_val;
  int32_t* arg_idx;
  int arg_ld;
  // row tile: 128 or 256; 0 = gemm_tile_m(m_cap); kGemmTileAuto = chosen on the device from
  // the row count (gemm_bm_of)
  int bm;
  // nonzero: the caller runs the split-K reduction itself (the QKV projection of a layer
  // with a QKV bias or rotary embedding, launch_qkv_reduce_rope_bias); launch_gemm runs none
  int defer_reduce;
};

constexpr int kGemmBM = 128;      // row tile of the SwiGLU slabs
// Row tile of the split-K GEMM for calls of at most m_cap rows: with 2048+ rows possible,
// 256-row tiles (8 waves, two per SIMD): per flop a 256 x 128 tile loads 3/4 of the bytes
// of a 128 x 128 one, and the MFMA-bound GEMMs of big verify steps are held by the load
// rate per CU.  Every kernel that re-derives a GEMM's split uses this same function.
// A call whose row count is known to be m_cap (every slot packed) takes them from
// kGemmTallExactFrom rows on.
constexpr int kGemmTallFrom = 2048;
constexpr int kGemmTallExactFrom = 512;
__host__ __device__ inline int gemm_tile_m(int m_cap, bool exact = false) {
  return (m_cap >= kGemmTallFrom || (exact && m_cap >= kGemmTallExactFrom)) ? 256 : 128;
}
// A row tile left to the device: calls whose row count is known only there (a folded
// layer's packed rows) and may fall on either side of kGemmTallAutoFrom.  One launch of
// eight waves runs 256-row tiles with all of them from kGemmTallAutoFrom rows on, and
// 128-row tiles with four of them below (the other four only take part in the barriers).
constexpr int kGemmTileAuto = -1;
constexpr int kGemmTallAutoFrom = 512;
// A streamed-weight call (GemmParams::w_stream: the FFN down projection) takes the 256-row
// tiles from 129 rows: up to 256 rows one row tile then reads each weight tile once, with the
// nontemporal hint, and per flop the tile loads 3/4 of the bytes (28-layer stack, 220 rows:
// down 58.7 -> 53.0 us, the step 7.18 -> 7.02 ms).  The QKV projection keeps 128-row tiles up
// to 511 rows (3B layer, 307 rows: 27.6 us against 29.3 us with 256-row tiles).
constexpr int kGemmTallAutoStreamFrom = 129;
// the row tile a GEMM call with M rows (read on the device) runs with; every kernel that
// re-derives a GEMM's tiling or split uses this
__host__ __device__ inline int gemm_bm_of(int bm, int m_cap, int M, bool stream = false) {
  if (bm == kGemmTileAuto)
    return M >= (stream ? kGemmTallAutoStreamFrom : kGemmTallAutoFrom) ? 256 : 128;
  return bm ? bm : gemm_tile_m(m_cap);
}
__host__ __device__ inline int gemm_bm(const GemmParams& p, int M) {
  return gemm_bm_of(p.bm, p.m_cap, M, p.w_stream != 0);
}

constexpr int kGemmBKBytes = 128;
constexpr int kGemmTileN = 128;   // columns per tile of the split-K GEMM (gemm_tile_n)
constexpr int kGemmMaxSplit = 24;
// Split-K keeps units >= this many k-iterations long, so a unit's fp32 partial plane stays
// small next to the weight bytes it streams.
constexpr int kGemmMinUnitIters = 8;

// Split-K factor chosen on the device from the tile count (the packed row count is only
// known there); kiters = number of 128-byte k-iterations.  One CU pulls only a fraction of
// HBM bandwidth on its own, so the work is split until there is about one unit per CU
// (never more: a second round on some CUs costs as much as the whole first one).
__host__ __device__ inline int gemm_split(int tiles, int kiters) {
  if (tiles <= 0) return 1;
  int s = kPlanCUs / tiles;
  // Between half a round and a full round of tiles, one unit per tile leaves CUs idle; 3 or 4
  // splits finish in 2 of 3 or 3 of 4 unit-rounds (129..170 tiles: 3; 171..192: 4).  Only for
  // long k-loops, where the extra fp32 partial planes are small next to the work (the stress
  // layer's down projection, 224 k-iterations, gains 15%; an O projection of 48 k-iterations
  // over 1024 rows lost 10% to its four partial planes).
  if (s == 1 && kiters >= 128 && 3 * tiles <= 2 * kPlanCUs) s = 3;
  else if (s == 1 && kiters >= 128 && 4 * tiles <= 3 * kPlanCUs) s = 4;
  const int smax = kiters / kGemmMinUnitIters;
  if (s > smax) s = smax;
  if (s > kGemmMaxSplit) s = kGemmMaxSplit;
  return s < 1 ? 1 : s;
}

// Events that time one kernel launch from its start to its end (hipExtLaunchKernel records
// them on the launch's stream at the kernel's start and completion), for a timing probe of
// a step that is a single kernel.
struct KernelTimer {
  hipEvent_t start;
  hipEvent_t stop;
};
// Whether a SwiGLU GEMM call is one kernel launch (the column slabs or the device-chosen
// swiglu_auto8 launch); the 256-row tiles chosen on the host add a split reduction
inline bool swiglu_single_launch(const GemmParams& p) {
  return p.bm == kGemmTileAuto || gemm_bm_of(p.bm, p.m_cap, p.m_cap) == 128;
}
// `timer` (may be null): taken by a SwiGLU call that is one launch (swiglu_single_launch)
template <typename T>
hipError_t launch_gemm(const GemmParams& p, int epi, int num_cu, hipStream_t st,
                       const KernelTimer* timer = nullptr);
// The QKV projection's split-K reduction fused with its bias (bias may be nullptr) and
// rotary embedding (theta > 0).  gp is the QKV GEMM's parameters, launched with
// defer_reduce set: each of the K packed rows of the Q|K|V buffer gp.C gets the sum of the
// GEMM's split partials (the split it chose on the device from K; with one split, the
// GEMM's own output) plus the bias, then the Q and K heads are rotated; packed row k sits
// at block position packed_slot[k] % B, absolute position P + that.
template <typename T>
hipError_t launch_qkv_reduce_rope_bias(const GemmParams& gp, const int32_t* packed_slot, int B,
                                       int P, int n_q, int n_kv, int dh, const void* bias,
                                       float theta, hipStream_t st);
// the kEpiStore or kEpiArgmax GEMM kernel with streamed weights (gemm_stream.hip; no
// reduction pass)
template <typename T, int EPI>
void launch_gemm_stream(const GemmParams& p, int num_cu, hipStream_t st);
// split-K factor the GEMM uses when the row count M is known on the host
int gemm_host_split(int M, int N, int Kd, int elem_bytes, int bm);

// Finish of the O projection: h[s] = H[s] + sum of `split` partial planes (rounded to T),
// and for every packed slot s (packed_slot[slot_row[s]] == s) the FFN input
// A2[slot_row[s]] = h[s] / sqrt(mean(h[s]^2) + eps) * g.  One workgroup per slot.
// by_row: the partial planes hold the K packed rows (the GEMM's split re-derived on the
// device from its row-tile setting bm (gemm_bm_of with K rows), tiles_n column tiles and
// kiters k-iterations) and slot s adds row slot_row[s].
template <typename T>
hipError_t launch_oproj_finish(const float* partial, int split, const void* H, void* h, int S,
                               int d, const int32_t* slot_row, const int32_t* packed_slot,
                               const int32_t* count, const void* g, float eps, void* A2,
                               int ld_a2, bool by_row, int tiles_n, int kiters, int bm,
                               hipStream_t st);
// fp32 elements of split-K partial storage any GEMM with these bounds may use
// (always: the GEMM writes partial planes even without split-K, as kEpiPartial does)
size_t gemm_partial_elems(int m_cap, int N, int Kd, int elem_bytes, bool always = false);
// N-tile width used for a GEMM with N output columns (256 for wide, 128 otherwise)
int gemm_tile_n(int N);

// Partials per row of a kEpiArgmax GEMM with N columns (two waves along each 128-column
// tile).
inline int gemm_argmax_partials(int N) { return ceil_div(N, 128) * 2; }

// LM head + per-branch argmax over the final hidden states (see lm_head.hip).
struct LmHeadParams {
  const void* hidden;      // [S, d]
  const void* rms;         // [d]
  const void* w;           // [V, d]
  const int32_t* packed_slot;
  const int32_t* slot_row;
  const int32_t* count;
  int N, B, d, V;
  float eps;
  void* An;                // workspace: [S, ld_an] normalised rows
  int ld_an;
  float* arg_val;          // workspace: [S, P] partial maxima
  int32_t* arg_idx;        // workspace: [S, P]
  int32_t* row_token;      // [S] (first K used)
  float* row_logit;        // [S] or nullptr
  int32_t* token;          // [S]
};
template <typename T>
hipError_t launch_lm_head(const LmHeadParams& q, int num_cu, hipStream_t st);

// ---------------------------------------------------------------------------------------
// Attention.  Prefix phase: online-softmax partials of every packed row's queries over the
// prefix view (split over key ranges).  Block phase: every slot's query against its own
// branch's block keys, merged with the prefix partials of its packed row.
// ---------------------------------------------------------------------------------------
struct AttnParams {
  const void* qkv;     // packed [K, (n_q + 2 n_kv) dh]
  long ld_qkv;
  int n_q, n_kv, dh;
  const int32_t* count;  // K (device)
  int cap;               // max K (= S)
  const void* pk;
  const void* pv;
  long stride_tok, stride_head;
  int P;
  float scale_log2;
  void* part_o;          // [nsplit][K][n_q][dh] in the model dtype (K = device packed count)
  float* part_lse;       // [nsplit][K][n_q]
  int S;
  const int32_t* slot_row;
  int N, B;
  void* out;             // [S, n_q dh]
  long ld_out;
  // [2] workspace: the prefix splits and whether they are merged before the block phase, for
  // the packed count of this call.  The prefix phase writes it; the split merge and the block
  // phase load it next to the count instead of re-deriving both in every workgroup.
  int32_t* plan;
  // nonzero: no prefix phase; the block phase streams the prefix itself (attn_fused_prefix)
  int fused;
};

constexpr int kAttnMaxSplit = 32;
// Prefixes of at most kAttnFusedMaxPrefix keys are not run as a separate per-packed-row
// phase: every slot's query streams the prefix tiles (through the same zero-copy view) and
// then its branch's block tiles in the block-phase kernel.  That recomputes the prefix
// scores of a packed row once per slot that takes it, but the prefix stays L2-resident and
// no split partials are written, re-read per slot and merged.  7B layer (512-key prefix):
// 22.6 us for the fused pass against 12.5 + 16.0 us for the two phases (event probes).  A
// fused unit walks its key tiles one after another (~1.5-2 us each), so longer prefixes keep
// the split prefix phase, and so do calls whose units (64 query rows of one branch and KV
// head) would need more than one round over the CUs: at 1 + 63 branches of the 7B layer the
// fused pass (1024 units) made the layer 374 -> 404 us.
constexpr int kAttnFusedMaxPrefix = 512;
constexpr int kAttnSlotQRows = 64;
constexpr int kAttnBlockQRows = 128;   // query rows of a block-phase unit (bf16)
inline bool attn_fused_prefix(int P, int N, int B, int n_q, int n_kv, int num_cu) {
  const long units = (long)N * n_kv * ((B * (n_q / n_kv) + kAttnSlotQRows - 1) / kAttnSlotQRows);
  return P > 0 && P <= kAttnFusedMaxPrefix && units <= num_cu;
}
// Prefix-phase kernels: bf16 prefixes of at least kAttnTrMinPrefix keys run 256-query
// units, one workgroup per CU (direct-to-LDS K/V ring, transposed V reads); shorter bf16
// prefixes and fp32 run 64-query units, two workgroups per CU (K/V staged through
// registers), which spreads a short prefix over four times as many units.
constexpr int kAttnTrMinPrefix = 2048;
static_assert(kPlanCUs == 256, "attn_splits shifts by log2 of the slot count");
__host__ __device__ inline bool attn_use_tr(int elem_bytes, int P) {
  return elem_bytes == 2 && P >= kAttnTrMinPrefix;
}
struct AttnPlan {
  int qrows, slots;
};
__host__ __device__ inline AttnPlan attn_plan(int elem_bytes, int P) {
  return attn_use_tr(elem_bytes, P) ? AttnPlan{256, kPlanCUs} : AttnPlan{64, 2 * kPlanCUs};
}
// Prefix key splits per (KV head, query tile) unit.  A unit streams ceil(chunks / s) key
// tiles and the grid runs `slots` units at a time (a power of two), so the prefix phase
// takes about ceil(units * s / slots) rounds of that many tiles.  Each split also costs its
// partial rows: K*g*n_kv rows of dh+1 values written, merged and read again, about
// rows*(dh+1) / 2^18 quarter tiles at the measured tile time and partial traffic rate.  s
// minimises the sum (in quarter tiles) over a short candidate list: powers of two and the
// counts between them that can fill the last round (at 1+63 branches over a 16384-key prefix,
// 5 splits make 760 units, three full rounds of 256, where 8 make 4.75 rounds).  The prefix
// phase evaluates this in every workgroup, so it costs one 32-bit division per candidate.
__host__ __device__ inline int attn_splits(int K, int g, int n_kv, int P, int dh,
                                           int elem_bytes) {
  if (P <= 0 || K <= 0) return 0;
  constexpr int kCands[] = {1, 2, 3, 4, 5, 6, 8, 10, 12, 16, 20, 24, 32};
  static_assert(kCands[sizeof(kCands) / sizeof(kCands[0]) - 1] <= kAttnMaxSplit,
                "split candidates exceed the merge's lane count");
  const AttnPlan pl = attn_plan(elem_bytes, P);
  const int lslots = pl.slots == 2 * kPlanCUs ? 9 : 8;   // log2 of 512 / 256
  const int units = n_kv * ((K * g + pl.qrows - 1) / pl.qrows);
  const int chunks = (P + 63) >> 6;
  const long per_split = ((long)K * g * n_kv * (dh + 1)) >> 18;
  const int split_cost = per_split < 1 ? 1 : (int)per_split;
  int best = 1;
  long best_cost = -1;
  for (int c = 0; c < (int)(sizeof(kCands) / sizeof(kCands[0])); ++c) {
    const int s = kCands[c];
    if (s > 1 && s > chunks / 2) break;                  // every split keeps >= 2 tiles
    const long rounds = ((long)units * s + (1 << lslots) - 1) >> lslots;
    const long cost = rounds * ((chunks + s - 1) / s) * 4 + (long)s * split_cost;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = s;
    }
  }
  return best;
}
// Whether the prefix splits are merged once per (packed row, head) before the block phase.
// Without the pass every slot reads all ns partial planes of its packed row; with it the
// pass reads K * ns planes and writes K, and the slots read one.  The pass costs a launch
// (~4.5 us even when it finds nothing to do) plus its traffic, so it runs only when the
// partial bytes it saves exceed 32 MB; a shape for which no packed count gets there (the
// 7B layer with a 512-key prefix) never launches it.
__host__ __device__ inline bool attn_merge_on(int K, int g, int n_kv, int P, int S, int dh,
                                              int elem_bytes) {
  const int ns = attn_splits(K, g, n_kv, P, dh, elem_bytes);
  if (ns < 2) return false;
  const long saved_rows = (long)S * (ns - 1) - (long)K * (ns + 1);
  return saved_rows * g * n_kv * (dh + 1) * 4 >= (32L << 20);
}
// largest nsplit * K over K in [1, S] (rows of partial storage)
size_t attn_partial_rows(int S, int g, int n_kv, int P, int dh, int elem_bytes);

template <typename T>
hipError_t launch_attn_prefix(const AttnParams& p, int num_cu, hipStream_t st);
template <typename T>
hipError_t launch_attn_block(const AttnParams& p, int num_cu, hipStream_t st);

}  // namespace specfold
