// Packed-row GEMMs of the folded verify layer on MFMA (SpecFold explainer: the heavy
// projections and the FFN run once on the bundle of recompute rows).
//
//   C[M, N] = A[M, Kd] . W[N, Kd]^T     A = packed activations, W = [out, in] weights
//
// With few packed rows these GEMMs stream the weights from HBM while every tile's MFMA,
// LDS and load work competes inside one CU, so the main loop is built to let those three
// overlap instead of running in lock-step:
//   * A and W tiles go global -> LDS with direct-to-LDS loads (global_load_lds_dwordx4):
//     no VGPR staging, no ds_write instructions, nothing for the wave to wait on until the
//     stage is consumed;
//   * a ring of three LDS stages (separate arrays, so the compiler can see that the loads
//     into one stage never alias the reads of another) keeps two k-iterations in flight;
//     one s_waitcnt vmcnt + s_barrier per k-iteration publishes the oldest stage;
//   * each load instruction writes 8 rows x 128 bytes contiguously; the 16-byte chunks of
//     a row are XOR-swizzled by (row >> 1) & 7, so the loads stay fully coalesced (8 lanes
//     per 128-byte row segment) and the MFMA operand reads (16 rows at one k chunk) hit 16
//     distinct bank groups;
//   * M (the packed row count) is known only on the device, so the kernel is persistent: a
//     fixed grid reads M, derives the tile count and a split-K factor, and walks the work
//     units XCD-major, numbered so that an XCD's units share K-slices of the activation
//     operand and weight column tiles in its L2.
// Split-K partial sums (fp32) are reduced by a separate kernel in split order, so results
// are deterministic and no device-scope fences are needed.
// Wave tile 64 x 64 (4 x 4 MFMA 16x16 tiles); a k-iteration is 128 bytes of K.
#include <hip/hip_ext.h>

#include "gemm_units.h"

namespace specfold {

template <typename T, int EPI, int BN, int BM>
__global__ void __launch_bounds__(BM * BN / 64) gemm_kernel(GemmParams p) {
  constexpr int A_BYTES = BM * kGemmBKBytes;
  constexpr int W_BYTES = BN * kGemmBKBytes;
  __shared__ __attribute__((aligned(1024))) char As0[A_BYTES], As1[A_BYTES], As2[A_BYTES];
  __shared__ __attribute__((aligned(1024))) char Ws0[W_BYTES], Ws1[W_BYTES], Ws2[W_BYTES];
  const int M = p.m_dev ? imin(*p.m_dev, p.m_cap) : p.m_cap;
  if (M <= 0) return;
  gemm_units<T, EPI, BN, BM>(p, M, As0, As1, As2, Ws0, Ws1, Ws2);
  // no wave may end while its last (clamped) stage loads are still writing LDS
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

// Row tile chosen on the device (GemmParams::bm = kGemmTileAuto): eight waves, two per SIMD;
// 256 x BN tiles on all of them from kGemmTallAutoFrom rows on, 128 x BN tiles on four below
// (the other four take part in the barriers only).  A four-wave launch with 128 x 64 wave
// tiles for the 256-row mode ran it 15-20% slower (3B layer, 1024 packed rows: QKV 56.6
// against 47.2 us, down 77.3 against 67.7 us) and the 128-row mode no faster.
template <typename T, int EPI, int BN>
__global__ void __launch_bounds__(256 * BN / 64) gemm_auto_kernel(GemmParams p) {
  constexpr int A_BYTES = 256 * kGemmBKBytes;
  constexpr int W_BYTES = BN * kGemmBKBytes;
  __shared__ __attribute__((aligned(1024))) char As0[A_BYTES], As1[A_BYTES], As2[A_BYTES];
  __shared__ __attribute__((aligned(1024))) char Ws0[W_BYTES], Ws1[W_BYTES], Ws2[W_BYTES];
  const int M = p.m_dev ? imin(*p.m_dev, p.m_cap) : p.m_cap;
  if (M <= 0) return;
  if (gemm_bm(p, M) == 256)
    gemm_units<T, EPI, BN, 256>(p, M, As0, As1, As2, Ws0, Ws1, Ws2);
  else
    gemm_units<T, EPI, BN, 128, true, 64, 64, 4 * BN / 64>(p, M, As0, As1, As2, Ws0, Ws1, Ws2);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}


// ---------------------------------------------------------------------------------------
// SwiGLU gate/up GEMM in column slabs.  The ff/16 (gate, up) pairs of 16-column blocks are
// dealt out in contiguous ranges of P or P+1 pairs, one unit per CU, so every CU streams an
// equal share of the weights with no split-K partials: a fixed 256-column tiling leaves
// ~40% of the CUs idle at the 7B shape, and one CU cannot pull much more than ~30 GB/s
// from HBM on its own.  A unit has eight waves, two per SIMD; a pass covers 128 rows (R = 1,
// 16 per wave) or 256 (R = 2, 32 per wave), every wave on every block of the slab, so both
// halves of an output element land in the same lane, and waves 0-3 also load the weight
// chunk.  The main loop is a direct-to-LDS three-stage ring like gemm_kernel's, templated on
// P so that the per-wave load counts (and with them the s_waitcnt immediates) are
// compile-time constants.  Eight waves keep more loads in flight per CU than the earlier
// four (one per SIMD, 32 rows each): 7B layer gate/up 65.5-66.0 -> 63.9-64.4 us (probes,
// same box).  The loads are the untracked dma16: only some waves load weights, and with the
// tracked builtin the compiler drained the ring before every LDS read.
// ---------------------------------------------------------------------------------------
constexpr int kSlabMaxPairs = 5;
// calls of this many slots or more can reach the tiled SwiGLU path (swiglu_auto8_kernel)
constexpr int kSwigluTallAutoFrom = 769;
constexpr int kSlab8Threads = 512;

template <typename T, int P, int R, bool WNT>
__device__ __forceinline__ void slab8_unit(const GemmParams& p, int M, int m0, int pair0,
                                           char* As0, char* As1, char* As2, char* Bs0,
                                           char* Bs1, char* Bs2, char* Ws0, char* Ws1,
                                           char* Ws2) {
  using G = GemmTile<T>;
  static_assert(R == 1 || R == 2, "one or two row tiles per pass");
  constexpr int NB = 2 * P;                               // gate_0, up_0, gate_1, ...
  constexpr int AQ = kGemmBM * kGemmBKBytes / 1024 / 8;   // A loads per wave per row tile
  constexpr int WQ = NB * 16 * kGemmBKBytes / 1024 / 4;   // W loads of each of waves 0-3
  constexpr int LA = R * AQ, LW = LA + WQ;                // loads per k-iteration (4-7, 0-3)
  const int kiters = p.Kd / G::BK;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool wl = wave < 4;
  const int g4 = lane >> 4, l16 = lane & 15;
  const int lr = lane >> 3, lpc = lane & 7;
  // this wave's rows: R = 1, rows 16w.. of the tile; R = 2, rows 32(w%4).. of tile w/4
  const int tile = R == 2 ? wave >> 2 : 0;
  const int lb = R == 2 ? (wave & 3) * 32 : wave * 16;
  const char* Ab = (const char*)p.A;
  const char* Wb = (const char*)p.W;

  const char* a_src[R][AQ];
  const char* w_src[WQ];
#pragma unroll
  for (int rt = 0; rt < R; ++rt)
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
      const int r = (wave * AQ + q) * 8 + lr;
      const int c = lpc ^ ((r >> 1) & 7);
      a_src[rt][q] = Ab + (size_t)imin(m0 + rt * kGemmBM + r, M - 1) * p.lda * sizeof(T) + c * 16;
    }
  const int ww = wl ? wave : 0;
#pragma unroll
  for (int q = 0; q < WQ; ++q) {
    const int r = (ww * WQ + q) * 8 + lr;               // stage row: block r/16, row r%16
    const int c = lpc ^ ((r >> 1) & 7);
    const int b = r >> 4;
    const int j = (pair0 + (b >> 1)) * 16 + (r & 15);
    const int wr = (b & 1) ? p.ff + j : j;
    w_src[q] = Wb + (size_t)wr * p.ldw * sizeof(T) + c * 16;
  }
  // loads of k-iteration `it` into a stage: the weight chunk (waves 0-3) and the A tile(s)
  auto issue = [&](char* a0, char* a1, char* ws, int it) {
    const size_t off = (size_t)imin(it, kiters - 1) * kGemmBKBytes;
    if (wl) {
#pragma unroll
      for (int q = 0; q < WQ; ++q) {
        if (WNT) dma16_nt(w_src[q] + off, lds_addr(ws) + (wave * WQ + q) * 1024);
        else dma16(w_src[q] + off, lds_addr(ws) + (wave * WQ + q) * 1024);
      }
    }
#pragma unroll
    for (int rt = 0; rt < R; ++rt)
#pragma unroll
      for (int q = 0; q < AQ; ++q)
        dma16(a_src[rt][q] + off, lds_addr(rt == 0 ? a0 : a1) + (wave * AQ + q) * 1024);
  };

  f32x4 acc[R][NB];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool live = (m0 + tile * kGemmBM + lb) < M;
  auto compute = [&](const char* a0, const char* a1, const char* ws) {
    if (!live) return;
    constexpr int KS = kGemmBKBytes / 64;
    const char* as = tile == 0 ? a0 : a1;
    uint4 af[KS][R], bfr[KS][NB];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = ks * 4 + g4;
#pragma unroll
      for (int i = 0; i < R; ++i)
        af[ks][i] = *reinterpret_cast<const uint4*>(as + swz(lb + i * 16 + l16, c));
#pragma unroll
      for (int j = 0; j < NB; ++j)
        bfr[ks][j] = *reinterpret_cast<const uint4*>(ws + swz(j * 16 + l16, c));
    }
    __builtin_amdgcn_sched_barrier(0);   // keep every read ahead of the MFMAs
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int i = 0; i < R; ++i) acc[i][j] = mma_kstep(af[ks][i], bfr[ks][j], acc[i][j], T());
  };
  // three stages, two k-iterations in flight: once this wave's loads of i have landed (its
  // loads of i + 1 may still be pending) and every wave has passed the barrier, stage i is
  // read and the loads of i + 2 go into the stage i - 1 left
  auto body = [&](char* a0, char* a1, char* ws, char* n0, char* n1, char* nw, int i) {
    if (wl) __builtin_amdgcn_s_waitcnt(waitcnt_vm(LW));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(LA));
    __builtin_amdgcn_s_barrier();
    if (i < kiters) compute(a0, a1, ws);
    issue(n0, n1, nw, i + 2);
  };
  // every wave is done with the previous unit's stages and its loads have landed
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __builtin_amdgcn_s_barrier();
  issue(As0, Bs0, Ws0, 0);
  issue(As1, Bs1, Ws1, 1);
  for (int it = 0; it < kiters; it += kGemmStages) {
    body(As0, Bs0, Ws0, As2, Bs2, Ws2, it);
    body(As1, Bs1, Ws1, As0, Bs0, Ws0, it + 1);
    body(As2, Bs2, Ws2, As1, Bs1, Ws1, it + 2);
  }

  // epilogue: lane holds rows g4*4 + r of each 16-row block and column l16 of each block
  T* C = (T*)p.C;
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int pr = 0; pr < P; ++pr) {
      const int col = (pair0 + pr) * 16 + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + tile * kGemmBM + lb + i * 16 + g4 * 4 + r;
        if (row < M) {
          const float gv = acc[i][2 * pr][r], uv = acc[i][2 * pr + 1][r];
          C[(size_t)row * p.ldc + col] = from_f32<T>(silu_f(gv) * uv);
        }
      }
    }
}

// Every eight-wave slab unit of one SwiGLU call (rows M read on the device), walked
// persistently.  Stage s holds {As_s, Bs_s, Ws_s}.
template <typename T, bool WNT>
__device__ __forceinline__ void slab8_walk(const GemmParams& p, int M, int slabs, char* As0,
                                           char* As1, char* As2, char* Bs0, char* Bs1,
                                           char* Bs2, char* Ws0, char* Ws1, char* Ws2) {
  const int pairs = p.ff / 16;
  const int base = pairs / slabs, rem = pairs - base * slabs;
  const int mb = ceil_div(M, kGemmBM);
  const int R = mb > 1 ? 2 : 1;                 // pairs of row tiles share every weight chunk
  const int groups = ceil_div(mb, R);
  for (int u = blockIdx.x; u < groups * slabs; u += gridDim.x) {
    const int mg = u / slabs, sl = u - mg * slabs;
    const int np = base + (sl < rem ? 1 : 0);
    const int pair0 = sl * base + imin(sl, rem);
    const int m0 = mg * R * kGemmBM;
#define SLAB8_CASE(PP)                                                                      \
  case PP:                                                                                  \
    if (R == 1)                                                                             \
      slab8_unit<T, PP, 1, WNT>(p, M, m0, pair0, As0, As1, As2, Bs0, Bs1, Bs2, Ws0, Ws1, Ws2); \
    else                                                                                    \
      slab8_unit<T, PP, 2, WNT>(p, M, m0, pair0, As0, As1, As2, Bs0, Bs1, Bs2, Ws0, Ws1, Ws2); \
    break;
    switch (np) {
      SLAB8_CASE(1) SLAB8_CASE(2) SLAB8_CASE(3) SLAB8_CASE(4) SLAB8_CASE(5)
      default: break;          // the host never makes slabs wider than kSlabMaxPairs
    }
#undef SLAB8_CASE
  }
}

// Streamed weight loads when every slab streams its weights once (one group of row tiles,
// up to 256 rows); with more groups each group re-reads them and the default policy keeps
// them cached (3B layer, 307 rows: gate/up 60.5 us cached, 70.8 us streamed).
template <typename T>
__device__ __forceinline__ void slab8_units(const GemmParams& p, int M, int slabs, char* As0,
                                            char* As1, char* As2, char* Bs0, char* Bs1,
                                            char* Bs2, char* Ws0, char* Ws1, char* Ws2) {
  if (p.w_stream && M <= 2 * kGemmBM)
    slab8_walk<T, true>(p, M, slabs, As0, As1, As2, Bs0, Bs1, Bs2, Ws0, Ws1, Ws2);
  else
    slab8_walk<T, false>(p, M, slabs, As0, As1, As2, Bs0, Bs1, Bs2, Ws0, Ws1, Ws2);
}

template <typename T>
__global__ void __launch_bounds__(kSlab8Threads) swiglu_slab8_kernel(GemmParams p, int slabs) {
  constexpr int A_BYTES = kGemmBM * kGemmBKBytes;
  constexpr int W_BYTES = 2 * kSlabMaxPairs * 16 * kGemmBKBytes;
  // three stages of {A tile 0, A tile 1, W}: 3 x (16 + 16 + 20) KB = 156 KB
  __shared__ __attribute__((aligned(1024))) char As0[A_BYTES], As1[A_BYTES], As2[A_BYTES];
  __shared__ __attribute__((aligned(1024))) char Bs0[A_BYTES], Bs1[A_BYTES], Bs2[A_BYTES];
  __shared__ __attribute__((aligned(1024))) char Ws0[W_BYTES], Ws1[W_BYTES], Ws2[W_BYTES];
  const int M = p.m_dev ? imin(*p.m_dev, p.m_cap) : p.m_cap;
  if (M <= 0) return;
  slab8_units<T>(p, M, slabs, As0, As1, As2, Bs0, Bs1, Bs2, Ws0, Ws1, Ws2);
  // no wave may end while its last (clamped) stage loads are still writing LDS
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

// The device-chosen SwiGLU on eight waves: below kSwigluTallAutoFrom packed rows the
// eight-wave slabs, from there on 256 x 128 tiles of the split-K GEMM body with eight 64 x 64
// wave tiles and no split.  Each stage is one X array (the slabs' two 128-row A tiles, or the
// 256-row A tile) and one Y array (the slab's weight chunk, or the 128-row W tile).  The slab
// path's loads are untracked, so its two A tiles may share an array.
template <typename T>
__global__ void __launch_bounds__(kSlab8Threads) swiglu_auto8_kernel(GemmParams p, int slabs) {
  constexpr int X_BYTES = 2 * kGemmBM * kGemmBKBytes;
  constexpr int Y_BYTES = 2 * kSlabMaxPairs * 16 * kGemmBKBytes;
  static_assert(X_BYTES >= 256 * kGemmBKBytes && Y_BYTES >= 128 * kGemmBKBytes, "stage sizes");
  __shared__ __attribute__((aligned(1024))) char X0[X_BYTES], X1[X_BYTES], X2[X_BYTES];
  __shared__ __attribute__((aligned(1024))) char Y0[Y_BYTES], Y1[Y_BYTES], Y2[Y_BYTES];
  const int M = p.m_dev ? imin(*p.m_dev, p.m_cap) : p.m_cap;
  if (M <= 0) return;
  constexpr int H = kGemmBM * kGemmBKBytes;
  if (M >= kSwigluTallAutoFrom)
    gemm_units<T, kEpiSwiGLU, 128, 256, false>(p, M, X0, X1, X2, Y0, Y1, Y2);
  else
    slab8_units<T>(p, M, slabs, X0, X1, X2, X0 + H, X1 + H, X2 + H, Y0, Y1, Y2);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

// Slab count for an ff-wide SwiGLU GEMM: one per CU, unless that needs wider slabs.
static int swiglu_slabs(int ff, int num_cu) {
  const int pairs = ff / 16;
  int slabs = pairs < num_cu ? pairs : num_cu;
  if (ceil_div(pairs, slabs) > kSlabMaxPairs) slabs = ceil_div(pairs, kSlabMaxPairs);
  return slabs;
}

// Sums the split-K partials in split order and applies the epilogue (4 outputs / thread).
template <typename T, int EPI, int BN>
__global__ void __launch_bounds__(256) gemm_reduce_kernel(GemmParams p) {
  const int M = p.m_dev ? imin(*p.m_dev, p.m_cap) : p.m_cap;
  if (M <= 0) return;
  const int mb = ceil_div(M, gemm_bm(p, M)), nt = ceil_div(p.N, BN);
  const int kiters = p.Kd / (kGemmBKBytes / (int)sizeof(T));
  const int split = gemm_split(mb * nt, kiters);
  if (split == 1) return;
  const int Nout = (EPI == kEpiSwiGLU) ? p.ff : p.N;
  const int q4 = Nout / 4;                      // Nout is a multiple of 64
  const long total = (long)M * q4;
  const size_t plane = (size_t)M * p.N;
  T* C = (T*)p.C;
  for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (long)gridDim.x * blockDim.x) {
    const int row = (int)(idx / q4), col = (int)(idx - (long)row * q4) * 4;
    float v[4];
    if (EPI == kEpiSwiGLU) {
      // 4 consecutive outputs share a 16-column block: gate at lg, up at lg + 16
      const int t = col / (BN / 2), cc = col % (BN / 2);
      const int lg = t * BN + (cc / 16) * 32 + (cc % 16);
      float4 gs = make_float4(0.f, 0.f, 0.f, 0.f), us = gs;
      for (int s = 0; s < split; ++s) {
        const float* ps = p.partial + s * plane + (size_t)row * p.N;
        const float4 a = *reinterpret_cast<const float4*>(ps + lg);
        const float4 b = *reinterpret_cast<const float4*>(ps + lg + 16);
        gs.x += a.x; gs.y += a.y; gs.z += a.z; gs.w += a.w;
        us.x += b.x; us.y += b.y; us.z += b.z; us.w += b.w;
      }
      v[0] = silu_f(gs.x) * us.x; v[1] = silu_f(gs.y) * us.y;
      v[2] = silu_f(gs.z) * us.z; v[3] = silu_f(gs.w) * us.w;
    } else {
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int s = 0; s < split; ++s) {
        const float4 b = *reinterpret_cast<const float4*>(p.partial + s * plane +
                                                          (size_t)row * p.N + col);
        a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
      }
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      if (EPI == kEpiResidual) {
        const T* R = (const T*)p.R + (size_t)row * p.ldr + col;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += to_f32(R[e]);
      }
    }
    T* out = C + (size_t)row * p.ldc + col;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = from_f32<T>(v[e]);
  }
}

// 128-column tiles: at one unit per CU the split-K partial planes cost more HBM traffic
// than re-reading the (L2-resident) activation tile for twice as many column tiles.
int gemm_tile_n(int) { return kGemmTileN; }

int gemm_host_split(int M, int N, int Kd, int elem_bytes, int bm) {
  const int BN = gemm_tile_n(N);
  return gemm_split(ceil_div(M, gemm_bm_of(bm, M, M)) * ceil_div(N, BN),
                    Kd / (kGemmBKBytes / elem_bytes));
}

size_t gemm_partial_elems(int m_cap, int N, int Kd, int elem_bytes, bool always) {
  const int BN = gemm_tile_n(N);
  const int kiters = Kd / (kGemmBKBytes / elem_bytes);
  const int nt = ceil_div(N, BN);
  size_t best = 0;
  for (int BM = 128; BM <= 256; BM *= 2)            // either row tile may run
    for (int mb = 1; mb <= ceil_div(m_cap, BM); ++mb) {
      const int split = gemm_split(mb * nt, kiters);
      if (split > 1 || always) {
        const size_t e = (size_t)split * (size_t)(mb * BM < m_cap ? mb * BM : m_cap) * N;
        if (e > best) best = e;
      }
    }
  return best;
}

template <typename T, int EPI, int BN>
static hipError_t launch_gemm_bn(const GemmParams& p, int num_cu, hipStream_t st) {
  // plain stores and the argmax epilogue with streamed weights (the FFN down projection, the
  // LM head) run the kernels of gemm_stream.hip; compiled here, next to these kernels, they
  // made the compiler drain every load in flight before the LDS reads of these
  // (gemm_auto_kernel: QKV 21.4 -> 28.7 us at the 3B layer)
  if ((EPI == kEpiStore || EPI == kEpiArgmax) && BN == 128 && p.w_stream) {
    launch_gemm_stream<T, EPI>(p, num_cu, st);
  } else if (p.bm == kGemmTileAuto) {
    // the device-chosen tile serves the store, partial and argmax epilogues; a SwiGLU call
    // takes the slab or swiglu_auto8 launches, and nothing calls the residual epilogue here
    if constexpr (EPI == kEpiSwiGLU || EPI == kEpiResidual) return hipErrorInvalidValue;
    else gemm_auto_kernel<T, EPI, BN><<<num_cu, 256 * BN / 64, 0, st>>>(p);
  } else if (gemm_bm_of(p.bm, p.m_cap, p.m_cap) == 256) {
    gemm_kernel<T, EPI, BN, 256><<<num_cu, 256 * BN / 64, 0, st>>>(p);
  } else {
    gemm_kernel<T, EPI, BN, 128><<<num_cu, 128 * BN / 64, 0, st>>>(p);
  }
  // the reduction only runs when some row count could make the device choose split > 1
  if (EPI != kEpiPartial && EPI != kEpiArgmax && !p.defer_reduce &&
      gemm_split(ceil_div(p.N, BN), p.Kd / (kGemmBKBytes / (int)sizeof(T))) > 1) {
    const int Nout = (EPI == kEpiSwiGLU) ? p.ff : p.N;
    const long total = (long)p.m_cap * (Nout / 4);
    const int rgrid = (int)((total + 255) / 256 < 2048 ? (total + 255) / 256 : 2048);
    gemm_reduce_kernel<T, EPI, BN><<<rgrid, 256, 0, st>>>(p);
  }
  return hipGetLastError();
}

template <typename T, int EPI>
static hipError_t launch_gemm_epi(const GemmParams& p, int num_cu, hipStream_t st,
                                  const KernelTimer* timer) {
  // a single-kernel launch, through hipExtLaunchKernel when it is timed
  auto one = [&](auto kernel, int grid, int slabs) {
    if (timer)
      hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(kSlab8Threads), 0, st, timer->start,
                            timer->stop, 0, p, slabs);
    else
      kernel<<<grid, kSlab8Threads, 0, st>>>(p, slabs);
    return hipGetLastError();
  };
  if (EPI == kEpiSwiGLU && p.bm == kGemmTileAuto && p.m_cap >= kSwigluTallAutoFrom) {
    // slabs below kSwigluTallAutoFrom rows, unsplit 256-row tiles above: no reduction pass
    return one(swiglu_auto8_kernel<T>, num_cu, swiglu_slabs(p.ff, num_cu));
  }
  if (EPI == kEpiSwiGLU && swiglu_single_launch(p)) {
    // 128-row tiles, or too few slots for the tiled path: the slabs, whatever the row count
    const int slabs = swiglu_slabs(p.ff, num_cu);
    return one(swiglu_slab8_kernel<T>, slabs, slabs);
  }
  return launch_gemm_bn<T, EPI, 128>(p, num_cu, st);
}

template <typename T>
hipError_t launch_gemm(const GemmParams& p, int epi, int num_cu, hipStream_t st,
                       const KernelTimer* timer) {
  switch (epi) {
    case kEpiStore: return launch_gemm_epi<T, kEpiStore>(p, num_cu, st, nullptr);
    case kEpiResidual: return launch_gemm_epi<T, kEpiResidual>(p, num_cu, st, nullptr);
    case kEpiSwiGLU: return launch_gemm_epi<T, kEpiSwiGLU>(p, num_cu, st, timer);
    case kEpiPartial: return launch_gemm_epi<T, kEpiPartial>(p, num_cu, st, nullptr);
    case kEpiArgmax: return launch_gemm_epi<T, kEpiArgmax>(p, num_cu, st, nullptr);
    default: return hipErrorInvalidValue;
  }
}

template hipError_t launch_gemm<float>(const GemmParams&, int, int, hipStream_t,
                                       const KernelTimer*);
template hipError_t launch_gemm<bf16>(const GemmParams&, int, int, hipStream_t,
                                      const KernelTimer*);

}  // namespace specfold
