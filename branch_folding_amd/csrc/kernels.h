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
size_t resolve_pack_lds_bytes(int S);
hipError_t launch_resolve_pack(const uint8_t* recompute, const int32_t* fold_src,
                               const int32_t* src_in, int N, int B, int mode, int32_t* src_out,
                               int32_t* packed_slot, int32_t* slot_row, int32_t* count,
                               hipStream_t st);
template <typename T>
hipError_t launch_combine(const void* h, const void* F, const int32_t* slot_row,
                          const int32_t* count, int cap, int S, int d, void* y, hipStream_t st);

// ---------------------------------------------------------------------------------------
// GEMM  C[M, N] = A[M, Kd] . W[N, Kd]^T  (both operands K-contiguous), M read on the
// device.  Epilogues: plain store, + residual, SwiGLU (W = [gate; up], output [M, ff]).
// ---------------------------------------------------------------------------------------
// kEpiPartial: always write fp32 partial sums (plane s of p.partial), even without split-K;
// a row-wise finishing kernel applies the epilogue.
enum GemmEpi { kEpiStore = 0, kEpiResidual = 1, kEpiSwiGLU = 2, kEpiPartial = 3 };

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
};

constexpr int kGemmBM = 128;
constexpr int kGemmBKBytes = 128;
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
  const int smax = kiters / kGemmMinUnitIters;
  if (s > smax) s = smax;
  if (s > kGemmMaxSplit) s = kGemmMaxSplit;
  return s < 1 ? 1 : s;
}

template <typename T>
hipError_t launch_gemm(const GemmParams& p, int epi, int num_cu, hipStream_t st);
// split-K factor the GEMM uses when the row count M is known on the host
int gemm_host_split(int M, int N, int Kd, int elem_bytes);

// Finish of the O projection: h[s] = H[s] + sum of `split` partial planes (rounded to T),
// and for every packed slot s (packed_slot[slot_row[s]] == s) the FFN input
// A2[slot_row[s]] = h[s] / sqrt(mean(h[s]^2) + eps) * g.  One workgroup per slot.
template <typename T>
hipError_t launch_oproj_finish(const float* partial, int split, const void* H, void* h, int S,
                               int d, const int32_t* slot_row, const int32_t* packed_slot,
                               const int32_t* count, const void* g, float eps, void* A2,
                               int ld_a2, hipStream_t st);
// fp32 elements of split-K partial storage any GEMM with these bounds may use
// (always: the GEMM writes partial planes even without split-K, as kEpiPartial does)
size_t gemm_partial_elems(int m_cap, int N, int Kd, int elem_bytes, bool always = false);
// N-tile width used for a GEMM with N output columns (256 for wide, 128 otherwise)
int gemm_tile_n(int N);

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
  float* part_o;         // [nsplit][K][n_q][dh]  (K = device packed count)
  float* part_lse;       // [nsplit][K][n_q]
  int S;
  const int32_t* slot_row;
  int N, B;
  void* out;             // [S, n_q dh]
  long ld_out;
};

constexpr int kAttnMaxSplit = 32;
__host__ __device__ inline int attn_splits(int K, int g, int n_kv, int P) {
  if (P <= 0 || K <= 0) return 0;
  const int qtiles = (K * g + 63) / 64;
  const int units = n_kv * qtiles;
  const int chunks = (P + 63) / 64;
  int s = (2 * kPlanCUs + units - 1) / units;
  int smax = chunks / 2;
  if (smax < 1) smax = 1;
  if (s > smax) s = smax;
  if (s > kAttnMaxSplit) s = kAttnMaxSplit;
  return s;
}
// Whether the prefix splits are merged once per (packed row, head) before the block phase:
// worth a pass when the slots' re-reads it saves, S * (ns - 1), dwarf its own K * (ns + 1).
__host__ __device__ inline bool attn_merge_on(int K, int g, int n_kv, int P, int S) {
  const int ns = attn_splits(K, g, n_kv, P);
  return ns >= 2 && (long)S * (ns - 1) >= 8L * K * (ns + 1);
}
// largest nsplit * K over K in [1, S] (rows of partial storage)
size_t attn_partial_rows(int S, int g, int n_kv, int P);

template <typename T>
hipError_t launch_attn_prefix(const AttnParams& p, int num_cu, hipStream_t st);
template <typename T>
hipError_t launch_attn_block(const AttnParams& p, int num_cu, hipStream_t st);

}  // namespace specfold
