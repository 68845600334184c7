// GEMMs with streamed weights (GemmParams::w_stream): the FFN down projection (plain stores)
// and the LM head (argmax epilogue).  The kernels of gemm.hip's path for those epilogues,
// except that at one row tile -- each weight tile then read once -- the weight loads carry
// the nontemporal hint, so the weight stream does not push the activation operand, which
// every CU re-reads, out of L2 (7B layer, 122 packed rows: down 47.2 -> 44 us).  With more
// row tiles the weights are re-read and keep the default policy.
// A translation unit of its own: compiled beside the plain kernels these made the compiler
// drain every load in flight before the plain kernels' LDS reads.
#include "gemm_units.h"

namespace specfold {

// BM-row tiles chosen on the host
template <typename T, int EPI, int BN, int BM>
__global__ void __launch_bounds__(BM * BN / 64) gemm_nt_kernel(GemmParams p) {
  constexpr int A_BYTES = BM * kGemmBKBytes;
  constexpr int W_BYTES = BN * kGemmBKBytes;
  __shared__ __attribute__((aligned(1024))) char As0[A_BYTES], As1[A_BYTES], As2[A_BYTES];
  __shared__ __attribute__((aligned(1024))) char Ws0[W_BYTES], Ws1[W_BYTES], Ws2[W_BYTES];
  const int M = p.m_dev ? imin(*p.m_dev, p.m_cap) : p.m_cap;
  if (M <= 0) return;
  if (M <= BM)
    gemm_units<T, EPI, BN, BM, true, 64, 64, BM * BN / 4096, true>(p, M, As0, As1, As2, Ws0,
                                                                   Ws1, Ws2);
  else
    gemm_units<T, EPI, BN, BM>(p, M, As0, As1, As2, Ws0, Ws1, Ws2);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

// row tile chosen on the device (the nontemporal hint at one row tile only; GemmParams::bm =
// kGemmTileAuto with w_stream set)
template <typename T, int EPI, int BN>
__global__ void __launch_bounds__(256 * BN / 64) gemm_auto_nt_kernel(GemmParams p) {
  constexpr int A_BYTES = 256 * kGemmBKBytes;
  constexpr int W_BYTES = BN * kGemmBKBytes;
  __shared__ __attribute__((aligned(1024))) char As0[A_BYTES], As1[A_BYTES], As2[A_BYTES];
  __shared__ __attribute__((aligned(1024))) char Ws0[W_BYTES], Ws1[W_BYTES], Ws2[W_BYTES];
  const int M = p.m_dev ? imin(*p.m_dev, p.m_cap) : p.m_cap;
  if (M <= 0) return;
  // Streamed calls run 256-row tiles from kGemmTallAutoStreamFrom (129) rows, so the last
  // path (128-row tiles, default policy) is not taken with w_stream set.  It stays: without
  // it the compiler drained every load in flight before the LDS reads of the 256-row
  // streamed path (s_waitcnt vmcnt(0) ahead of its ds_reads; tests/test_gemm_asm.py checks
  // the assembly for that).
  if (gemm_bm(p, M) == 256 && M <= 256)
    gemm_units<T, EPI, BN, 256, true, 64, 64, 4 * BN / 64, true>(p, M, As0, As1, As2, Ws0, Ws1,
                                                                 Ws2);
  else if (gemm_bm(p, M) == 256)
    gemm_units<T, EPI, BN, 256>(p, M, As0, As1, As2, Ws0, Ws1, Ws2);
  else if (M <= 128)
    gemm_units<T, EPI, BN, 128, true, 64, 64, 4 * BN / 64, true>(p, M, As0, As1, As2, Ws0, Ws1,
                                                                 Ws2);
  else
    gemm_units<T, EPI, BN, 128, true, 64, 64, 4 * BN / 64>(p, M, As0, As1, As2, Ws0, Ws1, Ws2);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

template <typename T, int EPI>
void launch_gemm_stream(const GemmParams& p, int num_cu, hipStream_t st) {
  constexpr int BN = 128;
  if (p.bm == kGemmTileAuto)
    gemm_auto_nt_kernel<T, EPI, BN><<<num_cu, 256 * BN / 64, 0, st>>>(p);
  else if (gemm_bm_of(p.bm, p.m_cap, p.m_cap) == 256)
    gemm_nt_kernel<T, EPI, BN, 256><<<num_cu, 256 * BN / 64, 0, st>>>(p);
  else
    gemm_nt_kernel<T, EPI, BN, 128><<<num_cu, 128 * BN / 64, 0, st>>>(p);
}

template void launch_gemm_stream<float, kEpiStore>(const GemmParams&, int, hipStream_t);
template void launch_gemm_stream<bf16, kEpiStore>(const GemmParams&, int, hipStream_t);
template void launch_gemm_stream<float, kEpiArgmax>(const GemmParams&, int, hipStream_t);
template void launch_gemm_stream<bf16, kEpiArgmax>(const GemmParams&, int, hipStream_t);

}  // namespace specfold
