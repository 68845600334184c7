// Packed-row GEMMs of the folded verify layer on MFMA (SpecFold explainer: the heavy
// projections and the FFN run once on the bundle of recompute rows).
//
//   C[M, N] = A[M, Kd] . W[N, Kd]^T     A = packed activations, W = [out, in] weights
//
// M (the packed row count) is known only on the device, so the kernel is persistent: a
// fixed grid reads M, derives the tile count and a split-K factor, and walks the work
// units.  Units are laid out so that each XCD owns a contiguous range (the M tiles of one
// weight tile run side by side on one XCD and share it through that XCD's L2).
// Workgroup tile 128 x 128 x 128 bytes of K, 4 waves (2 x 2), each wave 64 x 64 with
// 16x16 MFMA tiles; operands staged through double-buffered, padded LDS.
#include "common.h"
#include "kernels.h"

namespace specfold {

template <typename T>
struct GemmTile {
  static constexpr int VE = 16 / sizeof(T);               // elements per 16 bytes
  static constexpr int BK = kGemmBKBytes / sizeof(T);     // elements per k-iteration
  static constexpr int LDR = BK + VE;                     // LDS row stride (16-byte pad)
  static constexpr int kRowChunks = kGemmBKBytes / 16;    // 16-byte chunks per tile row
};

__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + expf(-x)); }

// W row feeding logical tile column c.  SwiGLU interleaves 16-column blocks of the gate
// and up projections so one lane ends up holding both halves of an output element.
template <int EPI>
__device__ __forceinline__ int w_row_of(int c, int N, int ff) {
  if (EPI == kEpiSwiGLU) {
    const int t = c / kGemmBN, cc = c % kGemmBN, blk = cc / 16;
    const int j = t * (kGemmBN / 2) + (blk / 2) * 16 + (cc % 16);
    return (blk & 1) ? ff + j : j;
  }
  return c < N ? c : N - 1;
}

template <typename T, int EPI>
__global__ void __launch_bounds__(256, 2) gemm_kernel(GemmParams p) {
  using G = GemmTile<T>;
  constexpr int VE = G::VE, BK = G::BK, LDR = G::LDR;
  __shared__ __attribute__((aligned(16))) T As[2][kGemmBM * LDR];
  __shared__ __attribute__((aligned(16))) T Ws[2][kGemmBN * LDR];

  const int M = p.m_dev ? imin(*p.m_dev, p.m_cap) : p.m_cap;
  if (M <= 0) return;
  const int mb = ceil_div(M, kGemmBM), nt = ceil_div(p.N, kGemmBN);
  const int kiters = p.Kd / BK;
  const int tiles = mb * nt;
  const int split = gemm_split(tiles, kiters);
  const int units = tiles * split;
  const int per_xcd = ceil_div(units, 8);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g4 = lane >> 4, l16 = lane & 15;
  const char* Ab = (const char*)p.A;
  const char* Wb = (const char*)p.W;

  for (int u = blockIdx.x; u < per_xcd * 8; u += gridDim.x) {
    const int v = (u & 7) * per_xcd + (u >> 3);       // XCD u%8 owns a contiguous range
    if (v >= units) continue;
    const int tile = v / split, s = v - tile * split;
    const int mt = tile % mb, ntile = tile / mb;
    const int m0 = mt * kGemmBM, n0 = ntile * kGemmBN;
    const int kb = (int)((long)s * kiters / split), ke = (int)((long)(s + 1) * kiters / split);

    // loader: thread handles 16-byte chunks (row = tid/8 + 32 j, chunk col = tid%8)
    const char* a_src[4];
    const char* w_src[4];
    const int lrow = tid >> 3, lcol = tid & 7;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = lrow + 32 * j;
      const int ar = imin(m0 + r, M - 1);
      a_src[j] = Ab + ((size_t)ar * p.lda + (size_t)lcol * VE) * sizeof(T);
      const int wr = w_row_of<EPI>(n0 + r, p.N, p.ff);
      w_src[j] = Wb + ((size_t)wr * p.ldw + (size_t)lcol * VE) * sizeof(T);
    }
    uint4 ra[4], rw[4];
    auto gload = [&](int it) {
      const size_t off = (size_t)it * kGemmBKBytes;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ra[j] = ld16(a_src[j] + off);
        rw[j] = ld16(w_src[j] + off);
      }
    };
    auto lstore = [&](int buf) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = lrow + 32 * j;
        *reinterpret_cast<uint4*>(&As[buf][r * LDR + lcol * VE]) = ra[j];
        *reinterpret_cast<uint4*>(&Ws[buf][r * LDR + lcol * VE]) = rw[j];
      }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    gload(kb);
    lstore(0);
    __syncthreads();
    for (int it = kb; it < ke; ++it) {
      const int cur = (it - kb) & 1;
      if (it + 1 < ke) gload(it + 1);
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
      if (it + 1 < ke) lstore(cur ^ 1);
      __syncthreads();
    }

    // epilogue: lane holds rows (g4*4 + r) and column l16 of every 16x16 tile
    if (split == 1) {
      T* C = (T*)p.C;
      if (EPI == kEpiSwiGLU) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int col = ntile * (kGemmBN / 2) + (wn * 2 + jj) * 16 + l16;
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
                float v = acc[i][j][r];
                if (EPI == kEpiResidual) v += to_f32(R[(size_t)row * p.ldr + col]);
                C[(size_t)row * p.ldc + col] = from_f32<T>(v);
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

// Sums the split-K partials in split order and applies the epilogue.
template <typename T, int EPI>
__global__ void __launch_bounds__(256) gemm_reduce_kernel(GemmParams p) {
  const int M = p.m_dev ? imin(*p.m_dev, p.m_cap) : p.m_cap;
  if (M <= 0) return;
  const int mb = ceil_div(M, kGemmBM), nt = ceil_div(p.N, kGemmBN);
  const int kiters = p.Kd / (kGemmBKBytes / (int)sizeof(T));
  const int split = gemm_split(mb * nt, kiters);
  if (split == 1) return;
  const int Nout = (EPI == kEpiSwiGLU) ? p.ff : p.N;
  const long total = (long)M * Nout;
  const size_t plane = (size_t)M * p.N;
  T* C = (T*)p.C;
  for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (long)gridDim.x * blockDim.x) {
    const int row = (int)(idx / Nout), col = (int)(idx - (long)row * Nout);
    float v;
    if (EPI == kEpiSwiGLU) {
      const int t = col / (kGemmBN / 2), cc = col % (kGemmBN / 2);
      const int lg = t * kGemmBN + (cc / 16) * 32 + (cc % 16);
      float gs = 0.f, us = 0.f;
      for (int s = 0; s < split; ++s) {
        gs += p.partial[s * plane + (size_t)row * p.N + lg];
        us += p.partial[s * plane + (size_t)row * p.N + lg + 16];
      }
      v = silu_f(gs) * us;
    } else {
      v = 0.f;
      for (int s = 0; s < split; ++s) v += p.partial[s * plane + (size_t)row * p.N + col];
      if (EPI == kEpiResidual) v += to_f32(((const T*)p.R)[(size_t)row * p.ldr + col]);
    }
    C[(size_t)row * p.ldc + col] = from_f32<T>(v);
  }
}

size_t gemm_partial_elems(int m_cap, int N, int Kd, int elem_bytes) {
  const int kiters = Kd / (kGemmBKBytes / elem_bytes);
  const int nt = ceil_div(N, kGemmBN);
  size_t best = 0;
  for (int mb = 1; mb <= ceil_div(m_cap, kGemmBM); ++mb) {
    const int split = gemm_split(mb * nt, kiters);
    if (split > 1) {
      const size_t e = (size_t)split * (size_t)(mb * kGemmBM < m_cap ? mb * kGemmBM : m_cap) * N;
      if (e > best) best = e;
    }
  }
  return best;
}

template <typename T>
hipError_t launch_gemm(const GemmParams& p, int epi, int num_cu, hipStream_t st) {
  const int grid = 2 * num_cu;
  const int Nout = (epi == kEpiSwiGLU) ? p.ff : p.N;
  const long total = (long)p.m_cap * Nout;
  const int rgrid = (int)((total + 255) / 256 < 8192 ? (total + 255) / 256 : 8192);
  switch (epi) {
    case kEpiStore:
      gemm_kernel<T, kEpiStore><<<grid, 256, 0, st>>>(p);
      gemm_reduce_kernel<T, kEpiStore><<<rgrid, 256, 0, st>>>(p);
      break;
    case kEpiResidual:
      gemm_kernel<T, kEpiResidual><<<grid, 256, 0, st>>>(p);
      gemm_reduce_kernel<T, kEpiResidual><<<rgrid, 256, 0, st>>>(p);
      break;
    case kEpiSwiGLU:
      gemm_kernel<T, kEpiSwiGLU><<<grid, 256, 0, st>>>(p);
      gemm_reduce_kernel<T, kEpiSwiGLU><<<rgrid, 256, 0, st>>>(p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template hipError_t launch_gemm<float>(const GemmParams&, int, int, hipStream_t);
template hipError_t launch_gemm<bf16>(const GemmParams&, int, int, hipStream_t);

}  // namespace specfold
