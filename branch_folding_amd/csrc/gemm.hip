// Packed-row GEMMs of the folded verify layer on MFMA (SpecFold explainer: the heavy
// projections and the FFN run once on the bundle of recompute rows).
//
//   C[M, N] = A[M, Kd] . W[N, Kd]^T     A = packed activations, W = [out, in] weights
//
// With few packed rows these GEMMs stream the weights from HBM, so the kernel is shaped by
// how the CU memory pipeline behaves on MI355X:
//   * weight and activation tiles are fetched with fully coalesced 16-byte loads (8 lanes
//     cover one 128-byte row segment), staged through padded LDS and read back in MFMA
//     operand layout -- loading straight into operand layout (16 rows x 64 bytes per
//     instruction) measured ~20% slower for the same bytes;
//   * every workgroup re-reads the whole (small) activation tile from L2, and those hits
//     occupy the same L1 request slots as the weight misses, so wide-N GEMMs use 256-column
//     tiles (8 waves) to halve that traffic;
//   * M (the packed row count) is known only on the device, so the kernel is persistent: a
//     fixed grid reads M, derives the tile count and a split-K factor, and walks the work
//     units, XCD-major so the M tiles of one weight tile share an XCD's L2.
// Split-K partial sums (fp32) are reduced by a separate kernel in split order, so results
// are deterministic and no device-scope fences are needed.
// Wave tile 64 x 64 (4 x 4 MFMA 16x16 tiles); a k-iteration is 128 bytes of K; loads run
// two k-iterations ahead through a register ring, staged into double-buffered LDS.
#include "common.h"
#include "kernels.h"

namespace specfold {

template <typename T>
struct GemmTile {
  static constexpr int VE = 16 / sizeof(T);               // elements per 16 bytes
  static constexpr int BK = kGemmBKBytes / sizeof(T);     // elements per k-iteration
  // LDS row stride: 32 bytes of padding make the 16-byte operand reads of 16 rows x 2 lane
  // groups conflict-free on gfx950's LDS (16 bytes of padding measured ~2.9 conflict
  // cycles per LDS instruction).
  static constexpr int LDR = BK + 2 * VE;
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

// k-iterations in flight in registers per thread (ring slots).
template <int BN> struct GemmDepth { static constexpr int PD = 2; };

// NORMA: the A operand is gathered through p.a_rows and RMS-normalised on its way into LDS
// (row scale p.a_scale, column gain p.a_gain), which fuses the pre-attention RMSNorm.
template <typename T, int EPI, int BN, bool NORMA>
__global__ void __launch_bounds__(BN * 2) gemm_kernel(GemmParams p) {
  using G = GemmTile<T>;
  constexpr int VE = G::VE, LDR = G::LDR;
  constexpr int NT = BN * 2;                 // threads
  constexpr int WN = BN / 64;                // waves along N
  constexpr int AJ = kGemmBM * 8 / NT;       // 16-byte A chunks per thread per k-iteration
  constexpr int WJ = BN * 8 / NT;            // 16-byte W chunks per thread per k-iteration
  constexpr int RSTEP = NT / 8;              // rows covered by one pass of the loader
  __shared__ __attribute__((aligned(16))) T As[2][kGemmBM * LDR];
  __shared__ __attribute__((aligned(16))) T Ws[2][BN * LDR];

  const int M = p.m_dev ? imin(*p.m_dev, p.m_cap) : p.m_cap;
  if (M <= 0) return;
  const int mb = ceil_div(M, kGemmBM), nt = ceil_div(p.N, BN);
  const int kiters = p.Kd / G::BK;
  const int tiles = mb * nt;
  const int split = gemm_split(tiles, kiters);
  const int units = tiles * split;
  const int per_xcd = ceil_div(units, 8);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int g4 = lane >> 4, l16 = lane & 15;
  const char* Ab = (const char*)p.A;
  const char* Wb = (const char*)p.W;

  for (int u = blockIdx.x; u < per_xcd * 8; u += gridDim.x) {
    const int v = (u & 7) * per_xcd + (u >> 3);       // XCD u%8 owns a contiguous range
    if (v >= units) continue;
    const int tile = v / split, s = v - tile * split;
    const int mt = tile % mb, ntile = tile / mb;
    const int m0 = mt * kGemmBM, n0 = ntile * BN;
    const int kb = (int)((long)s * kiters / split), ke = (int)((long)(s + 1) * kiters / split);

    const int lrow = tid >> 3, lcol = tid & 7;
    const char* a_src[AJ];
    const char* w_src[WJ];
    float a_sc[AJ];
#pragma unroll
    for (int j = 0; j < AJ; ++j) {
      int ar = imin(m0 + lrow + RSTEP * j, M - 1);
      if (NORMA) {
        ar = imin(imax(p.a_rows[ar], 0), p.a_rows_cap - 1);
        a_sc[j] = p.a_scale[ar];
      }
      a_src[j] = Ab + ((size_t)ar * p.lda + (size_t)lcol * VE) * sizeof(T);
    }
    const char* g_src = NORMA ? (const char*)p.a_gain + (size_t)lcol * VE * sizeof(T) : nullptr;
#pragma unroll
    for (int j = 0; j < WJ; ++j) {
      const int wr = w_row_of<EPI, BN>(n0 + lrow + RSTEP * j, p.N, p.ff);
      w_src[j] = Wb + ((size_t)wr * p.ldw + (size_t)lcol * VE) * sizeof(T);
    }
    constexpr int PD = GemmDepth<BN>::PD;
    uint4 ra[PD][AJ], rw[PD][WJ], rg[PD];
    // loads past the unit's last k-iteration are clamped to it (cache hits, unused)
    auto gload = [&](int slot, int it) {
      const size_t off = (size_t)imin(it, ke - 1) * kGemmBKBytes;
#pragma unroll
      for (int j = 0; j < WJ; ++j) rw[slot][j] = ld16(w_src[j] + off);
#pragma unroll
      for (int j = 0; j < AJ; ++j) ra[slot][j] = ld16(a_src[j] + off);
      if (NORMA) rg[slot] = ld16(g_src + off);
    };
    auto lstore = [&](int buf, int slot) {
#pragma unroll
      for (int j = 0; j < AJ; ++j) {
        uint4 av = ra[slot][j];
        if (NORMA) {
          float x[VE], gv[VE];
          unpack16(av, x, T());
          unpack16(rg[slot], gv, T());
#pragma unroll
          for (int e = 0; e < VE; ++e) x[e] = x[e] * a_sc[j] * gv[e];
          av = pack16(x, T());
        }
        *reinterpret_cast<uint4*>(&As[buf][(lrow + RSTEP * j) * LDR + lcol * VE]) = av;
      }
#pragma unroll
      for (int j = 0; j < WJ; ++j)
        *reinterpret_cast<uint4*>(&Ws[buf][(lrow + RSTEP * j) * LDR + lcol * VE]) = rw[slot][j];
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool rows_live = (m0 + wm * 64) < M;

    auto compute = [&](int cur) {
      if (!rows_live) return;
      const T* as = As[cur];
      const T* ws = Ws[cur];
#pragma unroll
      for (int ks = 0; ks < kGemmBKBytes / 64; ++ks) {
        uint4 af[4], bfr[4];
        const int koff = ks * 4 * VE + g4 * VE;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          af[i] = *reinterpret_cast<const uint4*>(&as[(wm * 64 + i * 16 + l16) * LDR + koff]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bfr[j] = *reinterpret_cast<const uint4*>(&ws[(wn * 64 + j * 16 + l16) * LDR + koff]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mma_kstep(af[i], bfr[j], acc[i][j], T());
      }
    };
    // One k-iteration: refill the register slot whose data is already in LDS, run the
    // MFMAs, stage the next iteration into the other LDS buffer.  Whole ring turns run
    // without per-iteration conditions so the wait counts stay PD - 1 iterations deep.
    // LDS buffer parity is relative to the unit's first k-iteration (staged into buffer 0)
    auto step = [&](int q, int it) {
      gload(q, it + PD);
      compute((it - kb) & 1);
      lstore((it - kb + 1) & 1, (q + 1) % PD);
      __syncthreads();
    };
#pragma unroll
    for (int q = 0; q < PD; ++q) gload(q, kb + q);
    lstore(0, 0);
    __syncthreads();
    int it = kb;
    for (; it + PD <= ke; it += PD) {
#pragma unroll
      for (int q = 0; q < PD; ++q) step(q, it + q);
    }
#pragma unroll
    for (int q = 0; q < PD - 1; ++q)
      if (it + q < ke) step(q, it + q);

    // epilogue: lane holds rows (g4*4 + r) and column l16 of every 16x16 tile
    if (split == 1 && EPI != kEpiPartial) {
      T* C = (T*)p.C;
      if (EPI == kEpiSwiGLU) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int col = ntile * (BN / 2) + (wn * 2 + jj) * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = m0 + wm * 64 + i * 16 + g4 * 4 + r;
              if (row < M && col < p.ff) {
                const float gv = acc[i][2 * jj][r], uv = acc[i][2 * jj + 1][r];
                C[(size_t)row * p.ldc + col] = from_f32<T>(silu_f(gv) * uv);
              }
            }
          }
      } else {
        const T* R = (const T*)p.R;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int col = n0 + wn * 64 + j * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = m0 + wm * 64 + i * 16 + g4 * 4 + r;
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
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = n0 + wn * 64 + j * 16 + l16;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = m0 + wm * 64 + i * 16 + g4 * 4 + r;
            if (row < M && col < p.N) part[(size_t)row * p.N + col] = acc[i][j][r];
          }
        }
    }
  }
}

// Sums the split-K partials in split order and applies the epilogue (4 outputs / thread).
template <typename T, int EPI, int BN>
__global__ void __launch_bounds__(256) gemm_reduce_kernel(GemmParams p) {
  const int M = p.m_dev ? imin(*p.m_dev, p.m_cap) : p.m_cap;
  if (M <= 0) return;
  const int mb = ceil_div(M, kGemmBM), nt = ceil_div(p.N, BN);
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

int gemm_tile_n(int N) { return N >= 256 ? 256 : 128; }

int gemm_host_split(int M, int N, int Kd, int elem_bytes) {
  const int BN = gemm_tile_n(N);
  return gemm_split(ceil_div(M, kGemmBM) * ceil_div(N, BN), Kd / (kGemmBKBytes / elem_bytes));
}

size_t gemm_partial_elems(int m_cap, int N, int Kd, int elem_bytes, bool always) {
  const int BN = gemm_tile_n(N);
  const int kiters = Kd / (kGemmBKBytes / elem_bytes);
  const int nt = ceil_div(N, BN);
  size_t best = 0;
  for (int mb = 1; mb <= ceil_div(m_cap, kGemmBM); ++mb) {
    const int split = gemm_split(mb * nt, kiters);
    if (split > 1 || always) {
      const size_t e = (size_t)split * (size_t)(mb * kGemmBM < m_cap ? mb * kGemmBM : m_cap) * N;
      if (e > best) best = e;
    }
  }
  return best;
}

template <typename T, int EPI, int BN>
static hipError_t launch_gemm_bn(const GemmParams& p, int num_cu, hipStream_t st) {
  const int grid = (BN == 256 ? 1 : 2) * num_cu;
  if (p.a_rows)
    gemm_kernel<T, EPI, BN, true><<<grid, BN * 2, 0, st>>>(p);
  else
    gemm_kernel<T, EPI, BN, false><<<grid, BN * 2, 0, st>>>(p);
  // the reduction only runs when some row count could make the device choose split > 1
  if (EPI != kEpiPartial && ceil_div(p.N, BN) < kGemmMinTiles) {
    const int Nout = (EPI == kEpiSwiGLU) ? p.ff : p.N;
    const long total = (long)p.m_cap * (Nout / 4);
    const int rgrid = (int)((total + 255) / 256 < 2048 ? (total + 255) / 256 : 2048);
    gemm_reduce_kernel<T, EPI, BN><<<rgrid, 256, 0, st>>>(p);
  }
  return hipGetLastError();
}

template <typename T, int EPI>
static hipError_t launch_gemm_epi(const GemmParams& p, int num_cu, hipStream_t st) {
  return gemm_tile_n(p.N) == 256 ? launch_gemm_bn<T, EPI, 256>(p, num_cu, st)
                                 : launch_gemm_bn<T, EPI, 128>(p, num_cu, st);
}

template <typename T>
hipError_t launch_gemm(const GemmParams& p, int epi, int num_cu, hipStream_t st) {
  switch (epi) {
    case kEpiStore: return launch_gemm_epi<T, kEpiStore>(p, num_cu, st);
    case kEpiResidual: return launch_gemm_epi<T, kEpiResidual>(p, num_cu, st);
    case kEpiSwiGLU: return launch_gemm_epi<T, kEpiSwiGLU>(p, num_cu, st);
    case kEpiPartial: return launch_gemm_epi<T, kEpiPartial>(p, num_cu, st);
    default: return hipErrorInvalidValue;
  }
}

template hipError_t launch_gemm<float>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_gemm<bf16>(const GemmParams&, int, int, hipStream_t);

}  // namespace specfold
