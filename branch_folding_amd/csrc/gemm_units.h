// The split-K GEMM body shared by the plain GEMM kernels (gemm.hip) and the streamed-weight
// store kernels (gemm_stream.hip); what it computes and how its main loop is built is
// described at the top of gemm.hip.
#pragma once
#include "common.h"
#include "kernels.h"

namespace specfold {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

template <typename T>
struct GemmTile {
  static constexpr int VE = 16 / sizeof(T);               // elements per 16 bytes
  static constexpr int BK = kGemmBKBytes / sizeof(T);     // elements per k-iteration
};

__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + expf(-x)); }

// W row feeding logical tile column c.  SwiGLU interleaves 16-column blocks of the gate
// and up projections so one lane ends up holding both halves of an output element.
template <int EPI, int BN>
__device__ __forceinline__ int w_row_of(int c, int N, int ff) {
  if (EPI == kEpiSwiGLU) {
    const int t = c / BN, cc = c % BN, blk = cc / 16;
    const int j = t * (BN / 2) + (blk / 2) * 16 + (cc % 16);
    return (blk & 1) ? ff + j : j;
  }
  return c < N ? c : N - 1;
}

// Byte offset of logical 16-byte chunk c of tile row r inside an LDS stage.
__device__ __forceinline__ int swz(int r, int c) {
  return r * kGemmBKBytes + ((c ^ ((r >> 1) & 7)) << 4);
}

// s_waitcnt immediate that waits until at most n vector-memory operations are pending
// (vmcnt split over bits 3:0 and 15:14; expcnt and lgkmcnt left at "no wait").
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

constexpr int kGemmStages = 3;
// cache-policy operand of the direct-to-LDS load builtin: the nontemporal hint
constexpr int kCpolNt = 2;

// Every unit of one GEMM call with BM x BN tiles, walked persistently by this workgroup.
// The tile's NW waves, one per WTM x WTN wave tile, load and compute; in a launch with
// more waves the others take part in the barriers only, so one launch can run either row
// tile.  Stage buffers: A stages of at least BM rows, W stages of at least BN rows.
// SPLIT = false keeps every unit on the whole K range (no partials, no reduction pass).
template <typename T, int EPI, int BN, int BM, bool SPLIT = true, int WTM = 64, int WTN = 64,
          int NWL = (BM / WTM) * (BN / WTN), bool WNT = false>
__device__ __forceinline__ void gemm_units(const GemmParams& p, int M, char* As0, char* As1,
                                           char* As2, char* Ws0, char* Ws1, char* Ws2) {
  using G = GemmTile<T>;
  constexpr int WN = BN / WTN;               // waves along N
  constexpr int NW = (BM / WTM) * WN;        // waves of the tile
  constexpr int TI = WTM / 16, TJ = WTN / 16;   // 16 x 16 MFMA tiles per wave
  static_assert(EPI != kEpiArgmax || WTN == 64, "argmax partials assume 64-column wave tiles");
  static_assert(EPI != kEpiSwiGLU || WTN % 32 == 0, "a wave holds whole gate/up pairs");
  constexpr int A_BYTES = BM * kGemmBKBytes;
  constexpr int W_BYTES = BN * kGemmBKBytes;
  constexpr int AQ = A_BYTES / 1024 / NW;    // A load instructions per wave per k-iteration
  constexpr int WQ = W_BYTES / 1024 / NW;    // W load instructions per wave per k-iteration
  constexpr int LPI = AQ + WQ;               // vector-memory ops per wave per k-iteration
  static_assert(AQ >= 1 && WQ >= 1 && A_BYTES % (1024 * NW) == 0, "tile/loader mismatch");

  const int mb = ceil_div(M, BM), nt = ceil_div(p.N, BN);
  const int kiters = p.Kd / G::BK;
  const int tiles = mb * nt;
  const int split = (EPI == kEpiArgmax || !SPLIT) ? 1 : gemm_split(tiles, kiters);
  const int units = tiles * split;
  const int per_xcd = ceil_div(units, 8);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // NWL = waves in the launch; when the tile has them all, nothing is predicated (a
  // predicated LDS DMA makes the compiler drain every load in flight before the LDS reads)
  static_assert(NWL >= NW, "launch narrower than the tile");
  const bool active = (NWL == NW) || wave < NW;
  const int wm = wave / WN, wn = wave % WN;
  const int g4 = lane >> 4, l16 = lane & 15;
  const char* Ab = (const char*)p.A;
  const char* Wb = (const char*)p.W;
  // loader geometry: instruction q of this wave fills rows 8*blk .. 8*blk+7 of a stage;
  // lane i carries row 8*blk + i/8, physical chunk i%8 (logical chunk swizzled back)
  const int lr = lane >> 3, lpc = lane & 7;

  for (int u = blockIdx.x; u < per_xcd * 8; u += gridDim.x) {
    const int v = (u & 7) * per_xcd + (u >> 3);       // XCD u%8 owns a contiguous range
    if (v >= units) continue;
    // K-slice slowest: an XCD's range covers one or two K-slices, so it pulls only those
    // slices of the shared activation operand into its L2.  Within a K-slice the tiles go in
    // bands of up to 8 row tiles, row tile fastest: the units an XCD runs side by side cover
    // a few column tiles of one band, so both operands of a round stay in its L2 (row tile
    // fastest over all rows would stream every activation row tile once per column tile).
    const int s = v / (mb * nt), vt = v - s * (mb * nt);
    const int band = vt / (8 * nt), bh = imin(8, mb - band * 8), vb = vt - band * 8 * nt;
    const int mt = band * 8 + vb % bh, ntile = vb / bh;
    const int m0 = mt * BM, n0 = ntile * BN;
    const int kb = (int)((long)s * kiters / split), ke = (int)((long)(s + 1) * kiters / split);

    const char* a_src[AQ];
    const char* w_src[WQ];
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
      const int r = (wave * AQ + q) * 8 + lr;
      const int c = lpc ^ ((r >> 1) & 7);
      int ar = imin(m0 + r, M - 1);
      if (p.a_rows) ar = imin(imax(p.a_rows[ar], 0), p.a_rows_cap - 1);
      a_src[q] = Ab + (size_t)ar * p.lda * sizeof(T) + c * 16;
    }
#pragma unroll
    for (int q = 0; q < WQ; ++q) {
      const int r = (wave * WQ + q) * 8 + lr;
      const int c = lpc ^ ((r >> 1) & 7);
      const int wr = w_row_of<EPI, BN>(n0 + r, p.N, p.ff);
      w_src[q] = Wb + (size_t)wr * p.ldw * sizeof(T) + c * 16;
    }
    // Stage loads of k-iteration `it` (clamped to the unit's last one: cache hits, unused):
    // the weight tile and the A tile.
    auto issue_w = [&](char* ws, int it) {
      if (!active) return;
      const size_t off = (size_t)imin(it, ke - 1) * kGemmBKBytes;
#pragma unroll
      for (int q = 0; q < WQ; ++q)
        __builtin_amdgcn_global_load_lds((glb_void_t*)(w_src[q] + off),
                                         (lds_void_t*)(ws + (wave * WQ + q) * 1024), 16, 0,
                                         WNT ? kCpolNt : 0);
    };
    auto issue_a = [&](char* as, int it) {
      if (!active) return;
      const size_t off = (size_t)imin(it, ke - 1) * kGemmBKBytes;
#pragma unroll
      for (int q = 0; q < AQ; ++q)
        __builtin_amdgcn_global_load_lds((glb_void_t*)(a_src[q] + off),
                                         (lds_void_t*)(as + (wave * AQ + q) * 1024), 16, 0, 0);
    };

    f32x4 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool rows_live = active && (m0 + wm * WTM) < M;

    // One wave per SIMD, so LDS latency is hidden inside the wave: all operand fragments of
    // the k-iteration are read at once (the second k-step's reads land while the first
    // k-step's MFMAs run), then its MFMAs.
    auto compute = [&](const char* as, const char* ws) {
      if (!rows_live) return;
      constexpr int KS = kGemmBKBytes / 64;
      uint4 af[KS][TI], bfr[KS][TJ];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c = ks * 4 + g4;
#pragma unroll
        for (int i = 0; i < TI; ++i)
          af[ks][i] = *reinterpret_cast<const uint4*>(as + swz(wm * WTM + i * 16 + l16, c));
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          bfr[ks][j] = *reinterpret_cast<const uint4*>(ws + swz(wn * WTN + j * 16 + l16, c));
      }
      __builtin_amdgcn_sched_barrier(0);   // keep every read ahead of the MFMAs
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[i][j] = mma_kstep(af[ks][i], bfr[ks][j], acc[i][j], T());
    };
    // k-iteration i on stage (as, ws): once this wave's loads of i have landed (only the
    // LPI loads of i + 1 may still be pending) and every wave has passed the barrier --
    // so all loads of i are visible and nobody still reads the stage that held i - 1 --
    // the loads of i + 2 go into that freed stage and the MFMAs run on stage i.  The
    // weight tile is issued before the MFMAs and the A tile after them, so a wave whose
    // CU has too many loads outstanding does not stall at the issue before its MFMAs.
    auto body = [&](char* as, char* ws, char* as2, char* ws2, int i) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPI));
      __builtin_amdgcn_s_barrier();
      issue_w(ws2, i + 2);
      if (i < ke) compute(as, ws);
      issue_a(as2, i + 2);
    };

    // every wave is done with the previous unit's stages and its loads have landed
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
    issue_w(Ws0, kb);
    issue_a(As0, kb);
    issue_w(Ws1, kb + 1);
    issue_a(As1, kb + 1);
    for (int it = kb; it < ke; it += kGemmStages) {
      body(As0, Ws0, As2, Ws2, it);
      body(As1, Ws1, As0, Ws0, it + 1);
      body(As2, Ws2, As1, Ws1, it + 2);
    }

    // epilogue: lane holds rows (g4*4 + r) and column l16 of every 16x16 tile
    if (!active) {
      // this wave holds no rows of the tile
    } else if (EPI == kEpiArgmax) {
      // per row: the largest of this wave's 64 columns and its first column index (columns
      // ascend with j within a lane; across the 16 lanes of a row ties go to the lower one)
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float bv = -__builtin_inff();
          int bi = 0x7fffffff;
#pragma unroll
          for (int j = 0; j < TJ; ++j) {
            const int col = n0 + wn * WTN + j * 16 + l16;
            const float v = acc[i][j][r];
            if (col < p.N && v > bv) {
              bv = v;
              bi = col;
            }
          }
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) {
            const float ov = __shfl_xor(bv, o, 16);
            const int oi = __shfl_xor(bi, o, 16);
            if (ov > bv || (ov == bv && oi < bi)) {
              bv = ov;
              bi = oi;
            }
          }
          const int row = m0 + wm * WTM + i * 16 + g4 * 4 + r;
          if (l16 == 0 && row < M) {
            const size_t at = (size_t)row * p.arg_ld + ntile * WN + wn;
            p.arg_val[at] = bv;
            p.arg_idx[at] = bi;
          }
        }
    } else if (split == 1 && EPI != kEpiPartial) {
      T* C = (T*)p.C;
      if (EPI == kEpiSwiGLU) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int jj = 0; jj < TJ / 2; ++jj) {
            const int col = ntile * (BN / 2) + (wn * (TJ / 2) + jj) * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = m0 + wm * WTM + i * 16 + g4 * 4 + r;
              if (row < M && col < p.ff) {
                const float gv = acc[i][2 * jj][r], uv = acc[i][2 * jj + 1][r];
                C[(size_t)row * p.ldc + col] = from_f32<T>(silu_f(gv) * uv);
              }
            }
          }
      } else {
        const T* R = (const T*)p.R;
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j) {
            const int col = n0 + wn * WTN + j * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = m0 + wm * WTM + i * 16 + g4 * 4 + r;
              if (row < M && col < p.N) {
                float x = acc[i][j][r];
                if (EPI == kEpiResidual) x += to_f32(R[(size_t)row * p.ldr + col]);
                C[(size_t)row * p.ldc + col] = from_f32<T>(x);
              }
            }
          }
      }
    } else {
      float* part = p.partial + (size_t)s * M * p.N;
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int col = n0 + wn * WTN + j * 16 + l16;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = m0 + wm * WTM + i * 16 + g4 * 4 + r;
            if (row < M && col < p.N) part[(size_t)row * p.N + col] = acc[i][j][r];
          }
        }
    }
  }
}

}  // namespace specfold
