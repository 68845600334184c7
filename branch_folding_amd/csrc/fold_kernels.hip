// Gate, provenance, packing, gathered RMSNorm and the final combine of the folded verify
// layer.  These steps move little data; they are written for coalesced 16-byte accesses
// and wave-level reductions, and leave the packed row count on the device.
#include "common.h"
#include "kernels.h"

namespace specfold {

// ------------------------------------------------------------------------------------
// Gate (SpecFold explainer, paragraph on measuring ||H_child - H_parent|| / ||H_parent||
// at the layer input).  One wave per slot; fp32 sums of squares; fold iff r <= tau.
// ratio and recompute are each optional (a caller-given fold state needs ratios only).
// ------------------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) gate_kernel(const T* __restrict__ H,
                                                   const int32_t* __restrict__ fold_src,
                                                   int N, int B, int d, float tau,
                                                   float* __restrict__ ratio,
                                                   uint8_t* __restrict__ recompute) {
  const int lane = threadIdx.x & 63;
  const int slot = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (slot >= N * B) return;
  const int n = slot / B, i = slot - n * B;
  int p = -1;
  if (n > 0 && fold_src) p = fold_src[n];
  const bool has_parent = (n > 0) && (p >= 0) && (p < n);
  const T* c = H + (size_t)slot * d;
  const T* q = has_parent ? H + ((size_t)p * B + i) * d : c;
  constexpr int VE = Pack16<T>::kElems;
  const int chunks = d / VE;
  float sd = 0.f, sp = 0.f;
  if (has_parent) {
    for (int ch = lane; ch < chunks; ch += 64) {
      float fc[VE], fp[VE];
      unpack16(ld16(c + ch * VE), fc, T());
      unpack16(ld16(q + ch * VE), fp, T());
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        const float df = fc[e] - fp[e];
        sd = fmaf(df, df, sd);
        sp = fmaf(fp[e], fp[e], sp);
      }
    }
    sd = wave_sum(sd);
    sp = wave_sum(sp);
  }
  if (lane == 0) {
    float r;
    bool rec;
    if (!has_parent) {
      r = __builtin_inff();
      rec = true;
    } else {
      const float num = sqrtf(sd), den = sqrtf(sp);
      r = (den == 0.f) ? (num == 0.f ? 0.f : __builtin_inff()) : num / den;
      rec = !(r <= tau);
    }
    if (ratio) ratio[slot] = r;
    if (recompute) recompute[slot] = rec ? 1 : 0;
  }
}

// ------------------------------------------------------------------------------------
// Provenance + packing in one workgroup (SpecFold explainer, implementation memo: the
// provenance kernel follows fold chains; the gate's packing compacts all branches'
// recompute positions).  Provenance runs one thread per position along the nodes in
// topological order; packing is a block-wide stable compaction (ballot + popcount +
// per-wave offsets) in ascending slot id.  Working arrays live in LDS.
// ------------------------------------------------------------------------------------
constexpr int kPackThreads = 1024;

__device__ __forceinline__ bool node_ok(const int32_t* fold_src, int n) {
  if (n == 0) return true;
  const int p = fold_src[n];
  return p >= 0 && p < n;
}

__global__ void __launch_bounds__(kPackThreads) resolve_pack_kernel(
    const uint8_t* __restrict__ recompute, const int32_t* __restrict__ fold_src,
    const int32_t* __restrict__ src_in, int N, int B, int mode,
    int32_t* __restrict__ src_out, int32_t* __restrict__ packed_slot,
    int32_t* __restrict__ slot_row, int32_t* __restrict__ packed_count) {
  extern __shared__ int32_t lds[];
  const int S = N * B;
  int32_t* src_l = lds;          // [S]
  int32_t* rank_l = lds + S;     // [S]
  __shared__ int32_t wave_cnt[kPackThreads / 64];
  __shared__ int32_t base_sh;
  const int t = threadIdx.x;
  const bool do_resolve = (mode & kResolve) != 0;
  const bool do_pack = (mode & kPack) != 0;

  // effective recompute flag of a slot: root rows and nodes with a malformed fold
  // source always compute their own rows.
  auto eff_rec = [&](int s) -> bool {
    const int n = s / B;
    return n == 0 || recompute[s] != 0 || (fold_src != nullptr && !node_ok(fold_src, n));
  };

  if (do_resolve) {
    for (int i = t; i < B; i += kPackThreads) {
      src_l[i] = 0;
      for (int n = 1; n < N; ++n) {
        const int s = n * B + i;
        if (eff_rec(s)) {
          src_l[s] = n;
        } else {
          src_l[s] = src_l[fold_src[n] * B + i];
        }
      }
    }
  } else {
    for (int s = t; s < S; s += kPackThreads) {
      int v = src_in[s];
      const int n = s / B;
      // a source must be an earlier-or-equal node; anything else is treated as the slot
      // itself (memory safety for malformed inputs)
      if (v < 0 || v > n) v = n;
      src_l[s] = v;
    }
  }
  __syncthreads();
  if (do_resolve && src_out) {
    for (int s = t; s < S; s += kPackThreads) src_out[s] = src_l[s];
  }
  if (!do_pack) return;

  // stable compaction of recompute slots
  const int lane = t & 63, wave = t >> 6;
  if (t == 0) base_sh = 0;
  __syncthreads();
  for (int c0 = 0; c0 < S; c0 += kPackThreads) {
    const int s = c0 + t;
    bool f = false;
    if (s < S) {
      const int n = s / B;
      // a slot is packed iff it computes its own row
      f = do_resolve ? (src_l[s] == n) : eff_rec(s);
    }
    const uint64_t bal = __ballot(f);
    const int before = __popcll(bal & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
    if (lane == 0) wave_cnt[wave] = __popcll(bal);
    __syncthreads();
    int off = base_sh;
    for (int w = 0; w < wave; ++w) off += wave_cnt[w];
    if (f) {
      const int k = off + before;
      packed_slot[k] = s;
      rank_l[s] = k;
    }
    __syncthreads();
    if (t == 0) {
      int tot = 0;
      for (int w = 0; w < kPackThreads / 64; ++w) tot += wave_cnt[w];
      base_sh += tot;
    }
    __syncthreads();
  }
  for (int s = t; s < S; s += kPackThreads) {
    const int i = s % B;
    int src = src_l[s];
    int target = src * B + i;
    // the source slot must be packed; fall back to the slot itself otherwise
    int k = -1;
    {
      const int n_src = src;
      bool packed = do_resolve ? (src_l[target] == n_src) : eff_rec(target);
      if (packed) k = rank_l[target];
    }
    if (k < 0) {
      const bool self_packed = do_resolve ? (src_l[s] == s / B) : eff_rec(s);
      k = self_packed ? rank_l[s] : 0;
    }
    slot_row[s] = k;
  }
  if (t == 0) packed_count[0] = base_sh;
}

// ------------------------------------------------------------------------------------
// Gathered RMSNorm: out[k] = X[rows[k]] / sqrt(mean(X^2) + eps) * g, for k < K (device).
// One wave per packed row.
// ------------------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) rmsnorm_gather_kernel(
    const T* __restrict__ X, const int32_t* __restrict__ rows, const int32_t* __restrict__ count,
    int cap, int S, int d, float eps, const T* __restrict__ g, T* __restrict__ out, int ld_out) {
  const int lane = threadIdx.x & 63;
  const int k = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int K = imin(*count, cap);
  if (k >= K) return;
  int r = rows[k];
  r = imin(imax(r, 0), S - 1);
  const T* x = X + (size_t)r * d;
  constexpr int VE = Pack16<T>::kElems;
  const int chunks = d / VE;
  float ss = 0.f;
  for (int ch = lane; ch < chunks; ch += 64) {
    float f[VE];
    unpack16(ld16(x + ch * VE), f, T());
#pragma unroll
    for (int e = 0; e < VE; ++e) ss = fmaf(f[e], f[e], ss);
  }
  ss = wave_sum(ss);
  const float rstd = 1.0f / sqrtf(ss / (float)d + eps);
  T* o = out + (size_t)k * ld_out;
  for (int ch = lane; ch < chunks; ch += 64) {
    float f[VE], w[VE];
    unpack16(ld16(x + ch * VE), f, T());
    unpack16(ld16(g + ch * VE), w, T());
#pragma unroll
    for (int e = 0; e < VE; ++e) f[e] = f[e] * rstd * w[e];
    st16(o + ch * VE, pack16(f, T()));
  }
}

// ------------------------------------------------------------------------------------
// O-projection finish: h = H + sum of the split-K partials, then the FFN's RMSNorm for the
// rows that are packed.  One wave per slot; pass 2 re-reads the row this lane just wrote.
// ------------------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) oproj_finish_kernel(
    const float* __restrict__ partial, int split, const T* __restrict__ H, T* __restrict__ h,
    int S, int d, const int32_t* __restrict__ slot_row, const int32_t* __restrict__ packed_slot,
    const int32_t* __restrict__ count, const T* __restrict__ g, float eps, T* __restrict__ A2,
    int ld_a2) {
  const int lane = threadIdx.x & 63;
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (s >= S) return;
  constexpr int VE = Pack16<T>::kElems;
  const int chunks = d / VE;
  const size_t plane = (size_t)S * d;
  float ss = 0.f;
  for (int ch = lane; ch < chunks; ch += 64) {
    float x[VE];
    unpack16(ld16(H + (size_t)s * d + ch * VE), x, T());
    for (int q = 0; q < split; ++q) {
      const float* pp = partial + q * plane + (size_t)s * d + ch * VE;
#pragma unroll
      for (int e = 0; e < VE; e += 4) {
        const float4 v = *reinterpret_cast<const float4*>(pp + e);
        x[e] += v.x; x[e + 1] += v.y; x[e + 2] += v.z; x[e + 3] += v.w;
      }
    }
    const uint4 hv = pack16(x, T());
    st16(h + (size_t)s * d + ch * VE, hv);
    float r[VE];
    unpack16(hv, r, T());                       // statistics of the rounded h
#pragma unroll
    for (int e = 0; e < VE; ++e) ss = fmaf(r[e], r[e], ss);
  }
  ss = wave_sum(ss);
  const int K = imin(*count, S);
  const int k = imin(imax(slot_row[s], 0), imax(K - 1, 0));
  if (K <= 0 || packed_slot[k] != s) return;     // not a packed row: no FFN input
  const float rstd = 1.0f / sqrtf(ss / (float)d + eps);
  for (int ch = lane; ch < chunks; ch += 64) {
    float x[VE], w[VE];
    unpack16(ld16(h + (size_t)s * d + ch * VE), x, T());
    unpack16(ld16(g + ch * VE), w, T());
#pragma unroll
    for (int e = 0; e < VE; ++e) x[e] = x[e] * rstd * w[e];
    st16(A2 + (size_t)k * ld_a2 + ch * VE, pack16(x, T()));
  }
}

// ------------------------------------------------------------------------------------
// Combine: y[s] = h[s] + F[slot_row[s]] (a folded slot keeps its own residual stream and
// adds its source's FFN output).
// ------------------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) combine_kernel(const T* __restrict__ h,
                                                      const T* __restrict__ F,
                                                      const int32_t* __restrict__ slot_row,
                                                      const int32_t* __restrict__ count,
                                                      int cap, int S, int d,
                                                      T* __restrict__ y) {
  constexpr int VE = Pack16<T>::kElems;
  const int chunks = d / VE;
  const long total = (long)S * chunks;
  const int K = imin(*count, cap);
  for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (long)gridDim.x * blockDim.x) {
    const int s = (int)(idx / chunks), ch = (int)(idx - (long)s * chunks);
    int k = slot_row[s];
    k = imin(imax(k, 0), imax(K - 1, 0));
    float a[VE], b[VE];
    unpack16(ld16(h + (size_t)s * d + ch * VE), a, T());
    unpack16(ld16(F + (size_t)k * d + ch * VE), b, T());
#pragma unroll
    for (int e = 0; e < VE; ++e) a[e] += b[e];
    st16(y + (size_t)s * d + ch * VE, pack16(a, T()));
  }
}

// ------------------------------------------------------------------------------------
// Host launchers.
// ------------------------------------------------------------------------------------
template <typename T>
hipError_t launch_gate(const void* H, const int32_t* fold_src, int N, int B, int d, float tau,
                       float* ratio, uint8_t* recompute, hipStream_t st) {
  const int S = N * B;
  gate_kernel<T><<<ceil_div(S, 4), 256, 0, st>>>((const T*)H, fold_src, N, B, d, tau, ratio,
                                                 recompute);
  return hipGetLastError();
}

size_t resolve_pack_lds_bytes(int S) { return (size_t)2 * S * sizeof(int32_t); }

hipError_t launch_resolve_pack(const uint8_t* recompute, const int32_t* fold_src,
                               const int32_t* src_in, int N, int B, int mode, int32_t* src_out,
                               int32_t* packed_slot, int32_t* slot_row, int32_t* count,
                               hipStream_t st) {
  const size_t lds = resolve_pack_lds_bytes(N * B);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)resolve_pack_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  resolve_pack_kernel<<<1, kPackThreads, lds, st>>>(recompute, fold_src, src_in, N, B, mode,
                                                     src_out, packed_slot, slot_row, count);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_rmsnorm_gather(const void* X, const int32_t* rows, const int32_t* count,
                                 int cap, int S, int d, float eps, const void* g, void* out,
                                 int ld_out, hipStream_t st) {
  rmsnorm_gather_kernel<T><<<ceil_div(cap, 4), 256, 0, st>>>(
      (const T*)X, rows, count, cap, S, d, eps, (const T*)g, (T*)out, ld_out);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_combine(const void* h, const void* F, const int32_t* slot_row,
                          const int32_t* count, int cap, int S, int d, void* y, hipStream_t st) {
  constexpr int VE = 16 / sizeof(T);
  const long total = (long)S * (d / VE);
  const int blocks = (int)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
  combine_kernel<T><<<blocks, 256, 0, st>>>((const T*)h, (const T*)F, slot_row, count, cap, S,
                                            d, (T*)y);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_oproj_finish(const float* partial, int split, const void* H, void* h, int S,
                               int d, const int32_t* slot_row, const int32_t* packed_slot,
                               const int32_t* count, const void* g, float eps, void* A2,
                               int ld_a2, hipStream_t st) {
  oproj_finish_kernel<T><<<ceil_div(S, 4), 256, 0, st>>>(partial, split, (const T*)H, (T*)h, S, d,
                                                          slot_row, packed_slot, count,
                                                          (const T*)g, eps, (T*)A2, ld_a2);
  return hipGetLastError();
}
template hipError_t launch_oproj_finish<float>(const float*, int, const void*, void*, int, int,
                                               const int32_t*, const int32_t*, const int32_t*,
                                               const void*, float, void*, int, hipStream_t);
template hipError_t launch_oproj_finish<bf16>(const float*, int, const void*, void*, int, int,
                                              const int32_t*, const int32_t*, const int32_t*,
                                              const void*, float, void*, int, hipStream_t);

template hipError_t launch_gate<float>(const void*, const int32_t*, int, int, int, float, float*,
                                       uint8_t*, hipStream_t);
template hipError_t launch_gate<bf16>(const void*, const int32_t*, int, int, int, float, float*,
                                      uint8_t*, hipStream_t);
template hipError_t launch_rmsnorm_gather<float>(const void*, const int32_t*, const int32_t*, int,
                                                 int, int, float, const void*, void*, int,
                                                 hipStream_t);
template hipError_t launch_rmsnorm_gather<bf16>(const void*, const int32_t*, const int32_t*, int,
                                                int, int, float, const void*, void*, int,
                                                hipStream_t);
template hipError_t launch_combine<float>(const void*, const void*, const int32_t*, const int32_t*,
                                          int, int, int, void*, hipStream_t);
template hipError_t launch_combine<bf16>(const void*, const void*, const int32_t*, const int32_t*,
                                         int, int, int, void*, hipStream_t);

}  // namespace specfold
