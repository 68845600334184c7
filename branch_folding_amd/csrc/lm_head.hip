// LM head after the last folded layer: the logits of the final layer's packed rows and
// every branch's predicted token at every position (the verify step compares the
// branches' predictions; a folded position takes its resolved source's prediction, as it
// takes the source's FFN output -- SpecFold explainer, the reuse path).
//
//   1. gate_kernel in its normalise-only mode: An[s] = RMSNorm(hidden[s]) * g for all slots;
//   2. gemm_kernel<kEpiArgmax>: logits of the packed rows (gathered from An through
//      packed_slot) against the [V, d] head, never stored: each wave keeps, per row, the
//      largest of its 64 columns and the first such column;
//   3. argmax_finish_kernel: one block per packed row reduces those partials (first index
//      of the maximum);
//   4. token_gather_kernel: token[s] = row_token[slot_row[s]].
#include "common.h"
#include "kernels.h"

namespace specfold {

// One 256-thread block per packed row: every thread scans P/256 partials (loads four at a
// time), then the wave and the block reduce (first index of the maximum on ties).
__device__ __forceinline__ void argmax_take(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

__global__ void __launch_bounds__(256) argmax_finish_kernel(const float* __restrict__ val,
                                                            const int32_t* __restrict__ idx,
                                                            int P, const int32_t* __restrict__ count,
                                                            int cap, int V,
                                                            int32_t* __restrict__ row_token,
                                                            float* __restrict__ row_logit) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int K = imin(*count, cap);
  for (int k = blockIdx.x; k < K; k += gridDim.x) {
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
    const float* v = val + (size_t)k * P;
    const int32_t* x = idx + (size_t)k * P;
    for (int j0 = t; j0 < P; j0 += 4 * 256) {
      float a[4];
      int b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = imin(j0 + u * 256, P - 1);
        a[u] = v[j];
        b[u] = x[j];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (j0 + u * 256 < P) argmax_take(bv, bi, a[u], b[u]);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      argmax_take(bv, bi, ov, oi);
    }
    if (lane == 0) {
      sv[wave] = bv;
      si[wave] = bi;
    }
    __syncthreads();
    if (t == 0) {
#pragma unroll
      for (int w = 1; w < 4; ++w) argmax_take(bv, bi, sv[w], si[w]);
      row_token[k] = (bi >= 0 && bi < V) ? bi : -1;   // -1: no logit above -inf (all NaN)
      if (row_logit) row_logit[k] = bv;
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(256) token_gather_kernel(const int32_t* __restrict__ row_token,
                                                           const int32_t* __restrict__ slot_row,
                                                           const int32_t* __restrict__ count,
                                                           int cap, int S,
                                                           int32_t* __restrict__ token) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= S) return;
  const int K = imin(*count, cap);
  token[s] = K > 0 ? row_token[imin(imax(slot_row[s], 0), K - 1)] : -1;
}

template <typename T>
hipError_t launch_lm_head(const LmHeadParams& q, int num_cu, hipStream_t st) {
  const int S = q.N * q.B;
  hipError_t e = launch_gate<T>(q.hidden, nullptr, q.N, q.B, q.d, 0.f, nullptr, nullptr, nullptr,
                                q.rms, q.eps, q.An, q.ld_an, st);
  if (e != hipSuccess) return e;
  GemmParams gp{};
  gp.A = q.An; gp.lda = q.ld_an; gp.a_rows = q.packed_slot; gp.a_rows_cap = S;
  gp.W = q.w; gp.ldw = q.d; gp.m_dev = q.count; gp.m_cap = S; gp.N = q.V; gp.Kd = q.d;
  gp.arg_val = q.arg_val; gp.arg_idx = q.arg_idx; gp.arg_ld = gemm_argmax_partials(q.V);
  gp.w_stream = 1;     // the head is read once per call: streamed weight loads
  if ((e = launch_gemm<T>(gp, kEpiArgmax, num_cu, st)) != hipSuccess) return e;
  const int fgrid = S < 4 * num_cu ? S : 4 * num_cu;
  argmax_finish_kernel<<<fgrid, 256, 0, st>>>(q.arg_val, q.arg_idx, gp.arg_ld, q.count, S, q.V,
                                               q.row_token, q.row_logit);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  token_gather_kernel<<<ceil_div(S, 256), 256, 0, st>>>(q.row_token, q.slot_row, q.count, S, S,
                                                        q.token);
  return hipGetLastError();
}

template hipError_t launch_lm_head<float>(const LmHeadParams&, int, hipStream_t);
template hipError_t launch_lm_head<bf16>(const LmHeadParams&, int, hipStream_t);

}  // namespace specfold
