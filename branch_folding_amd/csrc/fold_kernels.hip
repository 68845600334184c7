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
// With `An` the same pass also writes the RMS-normalised row
// An[slot] = H[slot] / sqrt(mean(H[slot]^2) + eps) * g of every slot that computes its own
// row -- decided here, or marked in `rec_given` -- for the QKV GEMM to gather, so the layer
// input is read once for both.  A row of up to 512 16-byte chunks is fetched in a single
// round of loads and kept in registers for the normalisation.
// ------------------------------------------------------------------------------------
constexpr int kGateU = 8;                    // 16-byte chunks per lane held in registers
// Slots (one wave each) per workgroup of the gate passes: four, unless that leaves CUs
// without a workgroup (512 slots: 256 workgroups of two instead of 128 of four; the 7B
// layer's gate 8.2-8.5 -> 7.9-8.2 us, event probes).
static int gate_slots_per_block(int S) {
  return S >= 4 * kPlanCUs ? 4 : (S >= 2 * kPlanCUs ? 2 : 1);
}

// Everything of the gate after the rows are loaded: sums of squares over the chunks held in
// registers (and, for rows longer than 64*kGateU chunks, the rest through tail_c / tail_p),
// the fold decision, and the normalised row of a slot that computes its own row.
template <typename T, typename TailC, typename TailP>
__device__ __forceinline__ void gate_finish(int lane, int slot, int n, int d, bool fs_ok,
                                            bool has_parent, float tau, float* ratio,
                                            uint8_t* recompute, const uint8_t* rec_given,
                                            const T* g, float eps, T* An, int ld_an,
                                            const uint4 (&vc)[kGateU], const uint4 (&vp)[kGateU],
                                            const uint4 (&vg)[kGateU], TailC tail_c,
                                            TailP tail_p) {
  constexpr int VE = Pack16<T>::kElems;
  constexpr int U = kGateU;
  const int chunks = d / VE;
  float sd = 0.f, sp = 0.f, sc = 0.f;
  auto accum = [&](const uint4& xc, const uint4& xp) {
    float fc[VE], fp[VE];
    unpack16(xc, fc, T());
#pragma unroll
    for (int e = 0; e < VE; ++e) sc = fmaf(fc[e], fc[e], sc);
    if (has_parent) {
      unpack16(xp, fp, T());
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        const float df = fc[e] - fp[e];
        sd = fmaf(df, df, sd);
        sp = fmaf(fp[e], fp[e], sp);
      }
    }
  };
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (lane + 64 * u < chunks) accum(vc[u], vp[u]);
  // rows longer than 64*U chunks: the remaining chunks stream through in further rounds
  for (int c0 = lane + 64 * U; c0 < chunks; c0 += 64) {
    const uint4 xc = tail_c(c0);
    accum(xc, has_parent ? tail_p(c0) : xc);
  }
  // fold decision (root rows and malformed fold sources always compute their own row)
  bool rec = true;
  if (has_parent) {
    sd = wave_sum(sd);
    sp = wave_sum(sp);
    const float num = sqrtf(sd), den = sqrtf(sp);
    const float r = (den == 0.f) ? (num == 0.f ? 0.f : __builtin_inff()) : num / den;
    rec = !(r <= tau);
    if (lane == 0 && ratio) ratio[slot] = r;
  } else if (lane == 0 && ratio) {
    ratio[slot] = __builtin_inff();
  }
  if (lane == 0 && recompute) recompute[slot] = rec ? 1 : 0;
  if (!An) return;
  const bool own = rec_given ? (n == 0 || !fs_ok || rec_given[slot] != 0) : rec;
  if (!own) return;                          // folded: the QKV GEMM never reads this row
  const float rstd = 1.0f / sqrtf(wave_sum(sc) / (float)d + eps);
  T* o = An + (size_t)slot * ld_an;
  auto norm = [&](const uint4& xc, const uint4& xg, int ch) {
    float fc[VE], fg[VE];
    unpack16(xc, fc, T());
    unpack16(xg, fg, T());
#pragma unroll
    for (int e = 0; e < VE; ++e) fc[e] = fc[e] * rstd * fg[e];
    st16(o + ch * VE, pack16(fc, T()));
  };
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (lane + 64 * u < chunks) norm(vc[u], vg[u], lane + 64 * u);
  for (int c0 = lane + 64 * U; c0 < chunks; c0 += 64) norm(tail_c(c0), ld16(g + c0 * VE), c0);
}

template <typename T>
__global__ void __launch_bounds__(256) gate_kernel(const T* __restrict__ H,
                                                   const int32_t* __restrict__ fold_src,
                                                   int N, int B, int d, float tau,
                                                   float* __restrict__ ratio,
                                                   uint8_t* __restrict__ recompute,
                                                   const uint8_t* __restrict__ rec_given,
                                                   const T* __restrict__ g, float eps,
                                                   T* __restrict__ An, int ld_an) {
  const int lane = threadIdx.x & 63;
  // the slot is wave-uniform, so its fold source comes through a scalar load, which the
  // parent row's loads wait for without waiting for the child row's vector loads
  const int slot = blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (slot >= N * B) return;
  const int n = slot / B, i = slot - n * B;
  const bool decide = (ratio != nullptr) || (recompute != nullptr);
  constexpr int VE = Pack16<T>::kElems;
  constexpr int U = kGateU;
  const int chunks = d / VE;
  const T* c = H + (size_t)slot * d;
  // The child row's loads go out before the fold source is known, so its lookup and the
  // row fetch overlap; rows of up to 64*U chunks take one round of loads, and the
  // normalisation pass reuses the registers instead of re-reading the row.
  uint4 vc[U], vp[U], vg[U];
#pragma unroll
  for (int u = 0; u < U; ++u) vc[u] = ld16(c + imin(lane + 64 * u, chunks - 1) * VE);
  if (An) {
#pragma unroll
    for (int u = 0; u < U; ++u) vg[u] = ld16(g + imin(lane + 64 * u, chunks - 1) * VE);
  }
  int p = -1;
  if (n > 0 && fold_src) p = fold_src[n];
  const bool fs_ok = (n > 0) && (p >= 0) && (p < n);
  const bool has_parent = decide && fs_ok;
  const T* q = has_parent ? H + ((size_t)p * B + i) * d : c;
  if (has_parent) {
#pragma unroll
    for (int u = 0; u < U; ++u) vp[u] = ld16(q + imin(lane + 64 * u, chunks - 1) * VE);
  }
  gate_finish<T>(lane, slot, n, d, fs_ok, has_parent, tau, ratio, recompute, rec_given, g, eps,
                 An, ld_an, vc, vp, vg, [&](int ch) { return ld16(c + ch * VE); },
                 [&](int ch) { return ld16(q + ch * VE); });
}

// ------------------------------------------------------------------------------------
// Combine of layer l fused with the gate of layer l+1 (a stack of layers: the gate runs at
// every layer on the residual stream the previous layer hands over).  One wave per slot
// forms y = h + F[slot_row] for its slot and for the slot's fold source (recomputed, not
// read back: another wave writes it), rounds both to T as the stored output is rounded,
// writes its own y, and runs the next layer's gate on the two rows: ratio, mask and the
// RMS-normalised row for the next QKV GEMM.  Bit-identical to the combine followed by the
// gate; one launch and one read of y fewer.  Rows of at most 64*kGateU chunks.
// ------------------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) combine_gate_kernel(
    const T* __restrict__ h, const T* __restrict__ F, const int32_t* __restrict__ slot_row,
    const int32_t* __restrict__ count, int cap, T* __restrict__ y,
    const int32_t* __restrict__ fold_src, int N, int B, int d, float tau,
    float* __restrict__ ratio, uint8_t* __restrict__ recompute, const T* __restrict__ g,
    float eps, T* __restrict__ An, int ld_an) {
  const int lane = threadIdx.x & 63;
  // wave-uniform slot: the fold source, count and packed-row indices come through scalar loads
  const int slot = blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (slot >= N * B) return;
  const int n = slot / B, i = slot - n * B;
  constexpr int VE = Pack16<T>::kElems;
  constexpr int U = kGateU;
  const int chunks = d / VE;
  const int K = imin(*count, cap);
  auto row_of = [&](int s) { return imin(imax(slot_row[s], 0), imax(K - 1, 0)); };
  int p = -1;
  if (n > 0 && fold_src) p = fold_src[n];
  const bool fs_ok = (n > 0) && (p >= 0) && (p < n);
  const int ps = fs_ok ? p * B + i : slot;
  const T* hc = h + (size_t)slot * d;
  const T* fc = F + (size_t)row_of(slot) * d;
  const T* hp = h + (size_t)ps * d;
  const T* fp = F + (size_t)row_of(ps) * d;
  uint4 vc[U], vp[U], vg[U], xh[U], xf[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int ch = imin(lane + 64 * u, chunks - 1) * VE;
    xh[u] = ld16(hc + ch);
    xf[u] = ld16(fc + ch);
    vg[u] = ld16(g + ch);
  }
  auto add = [&](const uint4& a, const uint4& b) {
    float fa[VE], fb[VE];
    unpack16(a, fa, T());
    unpack16(b, fb, T());
#pragma unroll
    for (int e = 0; e < VE; ++e) fa[e] += fb[e];
    return pack16(fa, T());
  };
  T* yc = y + (size_t)slot * d;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    vc[u] = add(xh[u], xf[u]);
    if (lane + 64 * u < chunks) st16(yc + (lane + 64 * u) * VE, vc[u]);
  }
  if (fs_ok) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ch = imin(lane + 64 * u, chunks - 1) * VE;
      xh[u] = ld16(hp + ch);
      xf[u] = ld16(fp + ch);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) vp[u] = add(xh[u], xf[u]);
  }
  gate_finish<T>(lane, slot, n, d, fs_ok, fs_ok, tau, ratio, recompute, nullptr, g, eps, An,
                 ld_an, vc, vp, vg, [&](int) { return make_uint4(0, 0, 0, 0); },
                 [&](int) { return make_uint4(0, 0, 0, 0); });
}

// ------------------------------------------------------------------------------------
// Provenance + packing in one workgroup (SpecFold explainer, implementation memo: the
// provenance kernel follows fold chains; the gate's packing compacts all branches'
// recompute positions).  Provenance follows every slot's fold chain at once by pointer
// jumping (log2 of the chain length in rounds, not one step per node); packing is a
// block-wide stable compaction (ballot + popcount + per-wave offsets) in ascending slot id.
// Working arrays live in LDS.
// ------------------------------------------------------------------------------------
constexpr int kPackThreads = 1024;

__device__ __forceinline__ bool node_ok(const int32_t* fold_src, int n) {
  if (n == 0) return true;
  const int p = fold_src[n];
  return p >= 0 && p < n;
}

// Workgroups 1.. of the provenance + packing launch have nothing to pack: each reads one
// slice of the next GEMM's weights once and discards it, so those bytes sit in the
// memory-side cache when that GEMM starts (the packing itself occupies one CU).  16 MB is
// what the other CUs read in about the time the packing takes: at the 7B layer the QKV GEMM
// gets 1.6 us faster and the launch no longer; the whole 33 MB made the launch 4 us longer.
constexpr long kPackPrefetchBytes = 16L << 20;

__device__ __forceinline__ void prefetch_slice(const uint4* __restrict__ src, long n16,
                                               int part, int parts, int* sink) {
  const long per = (n16 + parts - 1) / parts;
  const long b = (long)part * per, e = b + per < n16 ? b + per : n16;
  uint32_t acc = 0;
  for (long i0 = b + threadIdx.x; i0 < e; i0 += 8L * kPackThreads) {
    uint4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const long i = i0 + (long)j * kPackThreads;
      v[j] = i < e ? src[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j].x ^ v[j].w;
  }
  if (sink != nullptr && acc == 0x9e3779b9u) *sink = (int)acc;   // keeps the loads (sink is null)
}

__global__ void __launch_bounds__(kPackThreads) resolve_pack_kernel(
    const uint8_t* __restrict__ recompute, const int32_t* __restrict__ fold_src,
    const int32_t* __restrict__ src_in, int N, int B, int mode,
    int32_t* __restrict__ src_out, int32_t* __restrict__ packed_slot,
    int32_t* __restrict__ slot_row, int32_t* __restrict__ packed_count,
    const uint4* __restrict__ pf, long pf_n16, int* pf_sink) {
  if (blockIdx.x > 0) {
    prefetch_slice(pf, pf_n16, blockIdx.x - 1, gridDim.x - 1, pf_sink);
    return;
  }
  extern __shared__ int32_t lds[];
  const int S = N * B;
  int32_t* src_l = lds;                               // [S] source node of each slot
  int32_t* rank_l = lds + S;                          // [S] parent slot, later packed row
  uint8_t* rec_l = reinterpret_cast<uint8_t*>(lds + 2 * S);   // [S] computes its own row
  __shared__ int32_t wave_cnt[kPackThreads / 64];
  __shared__ int32_t base_sh;
  const int t = threadIdx.x;
  const bool do_resolve = (mode & kResolve) != 0;
  const bool do_pack = (mode & kPack) != 0;

  // One parallel pass over global memory: a slot computes its own row if it is a root
  // row, marked for recompute, or its node has a malformed fold source; otherwise its
  // parent slot is (fold_src[n], i).
  for (int s = t; s < S; s += kPackThreads) {
    const int n = s / B;
    bool own = (n == 0) || recompute[s] != 0;
    int ps = s;
    if (fold_src != nullptr && n > 0) {
      const int f = fold_src[n];
      if (f < 0 || f >= n) own = true;
      else ps = f * B + (s - n * B);
    }
    rec_l[s] = own ? 1 : 0;
    if (do_resolve) rank_l[s] = own ? s : ps;          // an own-row slot ends its chain
    else {
      int v = src_in[s];
      // a source must be an earlier-or-equal node; anything else is treated as the slot
      // itself (memory safety for malformed inputs)
      if (v < 0 || v > n) v = n;
      src_l[s] = v;
    }
  }
  __syncthreads();
  if (do_resolve) {
    // Pointer jumping: each slot points at its parent slot, a slot computing its own row at
    // itself.  A parent has a smaller node id, so a chain has at most N-1 links; the first
    // pointers skip one link and each round doubles that, so after ceil(log2(N-1)) rounds
    // every pointer sits on the own-row slot its chain ends in.  The rounds ping-pong between
    // rank_l and src_l (every pointer stays a valid slot id throughout).
    int32_t* cur = rank_l;
    int32_t* nxt = src_l;
    for (int span = 1; span < N - 1; span <<= 1) {
      for (int s = t; s < S; s += kPackThreads) nxt[s] = cur[cur[s]];
      __syncthreads();
      int32_t* tmp = cur; cur = nxt; nxt = tmp;
    }
    for (int s = t; s < S; s += kPackThreads) src_l[s] = cur[s] / B;   // slot -> node
    __syncthreads();
    if (src_out)
      for (int s = t; s < S; s += kPackThreads) src_out[s] = src_l[s];
  }
  if (!do_pack) return;

  // a slot is packed iff it computes its own row
  auto packed_of = [&](int s) -> bool {
    return do_resolve ? (src_l[s] == s / B) : (rec_l[s] != 0);
  };
  // stable compaction of the packed slots (ballot + popcount + per-wave offsets)
  const int lane = t & 63, wave = t >> 6;
  if (t == 0) base_sh = 0;
  __syncthreads();
  for (int c0 = 0; c0 < S; c0 += kPackThreads) {
    const int s = c0 + t;
    const bool f = (s < S) && packed_of(s);
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
    const int target = src_l[s] * B + s % B;
    // the source slot must be packed; fall back to the slot itself otherwise
    int k = -1;
    if (packed_of(target)) k = rank_l[target];
    if (k < 0) k = packed_of(s) ? rank_l[s] : 0;
    slot_row[s] = k;
  }
  if (t == 0) packed_count[0] = base_sh;
}

// ------------------------------------------------------------------------------------
// O-projection finish: h = H + sum of the split-K partials, then the FFN's RMSNorm for the
// rows that are packed.  One 512-thread workgroup per slot (enough workgroups to spread the
// partial-plane reads over every CU, and at hidden <= 4096 one chunk per thread, so a CU keeps
// twice the loads in flight of 256 threads: stress layer 31.2-31.6 -> 29.5 us, 7B layer
// 9.7 -> 9.0 us, event probes); the row's sum of squares is reduced through LDS and pass 2
// re-reads the h chunks this thread just wrote.
// ------------------------------------------------------------------------------------
constexpr int kFinishThreads = 512;

template <typename T>
__global__ void __launch_bounds__(kFinishThreads) oproj_finish_kernel(
    const float* __restrict__ partial, int split, const T* __restrict__ H, T* __restrict__ h,
    int S, int d, const int32_t* __restrict__ slot_row, const int32_t* __restrict__ packed_slot,
    const int32_t* __restrict__ count, const T* __restrict__ g, float eps, T* __restrict__ A2,
    int ld_a2, bool by_row, int tiles_n, int kiters, int bm) {
  __shared__ float red[kFinishThreads / 64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int s = blockIdx.x;
  constexpr int VE = Pack16<T>::kElems;
  const int chunks = d / VE;
  const int K = imin(*count, S);
  // by_row (REUSE variant): the GEMM ran over the K packed rows with a split it chose on the
  // device; slot s adds the projection of its packed row slot_row[s]
  if (by_row && K <= 0) return;
  const int rows = by_row ? K : S;
  if (by_row) split = gemm_split(ceil_div(K, gemm_bm_of(bm, S, K)) * tiles_n, kiters);
  const size_t plane = (size_t)rows * d;
  const size_t row = (size_t)s * d;
  const size_t prow = by_row ? (size_t)imin(imax(slot_row[s], 0), K - 1) * d : row;
  float ss = 0.f;
  for (int ch = t; ch < chunks; ch += kFinishThreads) {
    float x[VE];
    unpack16(ld16(H + row + ch * VE), x, T());
    for (int q = 0; q < split; ++q) {
      const float* pp = partial + q * plane + prow + ch * VE;
#pragma unroll
      for (int e = 0; e < VE; e += 4) {
        const float4 v = *reinterpret_cast<const float4*>(pp + e);
        x[e] += v.x; x[e + 1] += v.y; x[e + 2] += v.z; x[e + 3] += v.w;
      }
    }
    const uint4 hv = pack16(x, T());
    st16(h + row + ch * VE, hv);
    float r[VE];
    unpack16(hv, r, T());                       // statistics of the rounded h
#pragma unroll
    for (int e = 0; e < VE; ++e) ss = fmaf(r[e], r[e], ss);
  }
  const int k = imin(imax(slot_row[s], 0), imax(K - 1, 0));
  if (K <= 0 || packed_slot[k] != s) return;     // not a packed row: no FFN input
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kFinishThreads / 64; ++w) tot += red[w];
  const float rstd = 1.0f / sqrtf(tot / (float)d + eps);
  for (int ch = t; ch < chunks; ch += kFinishThreads) {
    float x[VE], w[VE];
    unpack16(ld16(h + row + ch * VE), x, T());
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
// QKV bias and rotary embedding on the packed Q|K|V rows, in place (model families with
// both, e.g. Qwen / Llama style).  One thread per (packed row, head, pair j): the bias is
// added to elements j and j + dh/2 of every head; Q and K heads are then rotated by the
// angle pos * theta^(-2j/dh), pos = prefix length + the row's block position.  The angle and
// its sine and cosine are taken in double: at positions of ~17K an fp32 angle would be off
// by ~1e-3 rad.
// ------------------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) qkv_reduce_rope_bias_kernel(
    GemmParams p, const int32_t* __restrict__ packed_slot, int B, int P, int n_q, int n_kv,
    int dh, const T* __restrict__ bias, float theta) {
  const int K = p.m_dev ? imin(*p.m_dev, p.m_cap) : p.m_cap;
  if (K <= 0) return;
  // the split the GEMM ran with, derived as its own reduction derives it
  const int kiters = p.Kd / (kGemmBKBytes / (int)sizeof(T));
  const int split = gemm_split(ceil_div(K, gemm_bm(p, K)) * ceil_div(p.N, kGemmTileN), kiters);
  // one thread per (packed row, head, 4 consecutive j < dh/2): columns j..j+3 and their
  // rotation partners j+dh/2..j+dh/2+3
  const int half = dh / 2, q4 = half / 4, heads = n_q + 2 * n_kv;
  const long total = (long)K * heads * q4;
  const size_t plane = (size_t)K * p.N;
  T* C = (T*)p.C;
  for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (long)gridDim.x * blockDim.x) {
    const int k = (int)(idx / (heads * q4));
    const int rem = (int)(idx - (long)k * heads * q4);
    const int hd = rem / q4, j0 = (rem - hd * q4) * 4;
    const int c1 = hd * dh + j0, c2 = c1 + half;
    T* row = C + (size_t)k * p.ldc;
    float x1[4], x2[4];
    if (split > 1) {
      // the partial planes summed in split order, as the plain reduction sums them
      const float* pr = p.partial + (size_t)k * p.N;
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
      for (int sp = 0; sp < split; ++sp) {
        const float4 u = *reinterpret_cast<const float4*>(pr + (size_t)sp * plane + c1);
        const float4 v = *reinterpret_cast<const float4*>(pr + (size_t)sp * plane + c2);
        a.x += u.x; a.y += u.y; a.z += u.z; a.w += u.w;
        b.x += v.x; b.y += v.y; b.z += v.z; b.w += v.w;
      }
      x1[0] = a.x; x1[1] = a.y; x1[2] = a.z; x1[3] = a.w;
      x2[0] = b.x; x2[1] = b.y; x2[2] = b.z; x2[3] = b.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x1[e] = to_f32(row[c1 + e]);
        x2[e] = to_f32(row[c2 + e]);
      }
    }
    if (bias) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x1[e] += to_f32(bias[c1 + e]);
        x2[e] += to_f32(bias[c2 + e]);
      }
    }
    if (theta > 0.f && hd < n_q + n_kv) {
      const int ps = imin(imax(packed_slot[k], 0), p.m_cap - 1);
      const double pos = (double)(P + ps % B);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double ang = pos * pow((double)theta, -2.0 * (j0 + e) / dh);
        double sn, cs;
        sincos(ang, &sn, &cs);
        const float c = (float)cs, sv = (float)sn;
        const float y1 = x1[e] * c - x2[e] * sv, y2 = x2[e] * c + x1[e] * sv;
        x1[e] = y1;
        x2[e] = y2;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      row[c1 + e] = from_f32<T>(x1[e]);
      row[c2 + e] = from_f32<T>(x2[e]);
    }
  }
}

// ------------------------------------------------------------------------------------
// Draft-graph check (debug builds of a call): node 0 is the root (fold_src = -1) and every
// other node folds onto an earlier one (0 <= fold_src[n] < n), the topological numbering
// the provenance steps rely on.  One workgroup; out[0] = first offending node or -1,
// out[1] = its fold_src entry.
// ------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) check_fold_src_kernel(const int32_t* __restrict__ fs,
                                                              int N, int32_t* out) {
  __shared__ int first;
  if (threadIdx.x == 0) first = 0x7fffffff;
  __syncthreads();
  for (int n = threadIdx.x; n < N; n += blockDim.x) {
    const int v = fs[n];
    const bool bad = n == 0 ? v != -1 : (v < 0 || v >= n);
    if (bad) atomicMin(&first, n);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int f = first;
    out[0] = f == 0x7fffffff ? -1 : f;
    out[1] = f == 0x7fffffff ? 0 : fs[f];
  }
}

// ------------------------------------------------------------------------------------
// Host launchers.
// ------------------------------------------------------------------------------------
hipError_t launch_check_fold_src(const int32_t* fold_src, int N, int32_t* out, hipStream_t st) {
  check_fold_src_kernel<<<1, 256, 0, st>>>(fold_src, N, out);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_gate(const void* H, const int32_t* fold_src, int N, int B, int d, float tau,
                       float* ratio, uint8_t* recompute, const uint8_t* rec_given,
                       const void* g, float eps, void* An, int ld_an, hipStream_t st) {
  const int S = N * B;
  const int wpb = gate_slots_per_block(S);
  gate_kernel<T><<<ceil_div(S, wpb), 64 * wpb, 0, st>>>((const T*)H, fold_src, N, B, d, tau, ratio,
                                                 recompute, rec_given, (const T*)g, eps,
                                                 (T*)An, ld_an);
  return hipGetLastError();
}

bool combine_gate_fits(int d, int elem_bytes) { return d / (16 / elem_bytes) <= 64 * kGateU; }

template <typename T>
hipError_t launch_combine_gate(const void* h, const void* F, const int32_t* slot_row,
                               const int32_t* count, int cap, void* y, const int32_t* fold_src,
                               int N, int B, int d, float tau, float* ratio, uint8_t* recompute,
                               const void* g, float eps, void* An, int ld_an, hipStream_t st) {
  if (!combine_gate_fits(d, (int)sizeof(T))) return hipErrorInvalidValue;
  const int wpb = gate_slots_per_block(N * B);
  combine_gate_kernel<T><<<ceil_div(N * B, wpb), 64 * wpb, 0, st>>>(
      (const T*)h, (const T*)F, slot_row, count, cap, (T*)y, fold_src, N, B, d, tau, ratio,
      recompute, (const T*)g, eps, (T*)An, ld_an);
  return hipGetLastError();
}
template hipError_t launch_combine_gate<float>(const void*, const void*, const int32_t*,
                                               const int32_t*, int, void*, const int32_t*, int,
                                               int, int, float, float*, uint8_t*, const void*,
                                               float, void*, int, hipStream_t);
template hipError_t launch_combine_gate<bf16>(const void*, const void*, const int32_t*,
                                              const int32_t*, int, void*, const int32_t*, int,
                                              int, int, float, float*, uint8_t*, const void*,
                                              float, void*, int, hipStream_t);

size_t resolve_pack_lds_bytes(int S) {
  return (size_t)2 * S * sizeof(int32_t) + (((size_t)S + 3) & ~(size_t)3);
}

hipError_t launch_resolve_pack(const uint8_t* recompute, const int32_t* fold_src,
                               const int32_t* src_in, int N, int B, int mode, int32_t* src_out,
                               int32_t* packed_slot, int32_t* slot_row, int32_t* count,
                               const void* prefetch, size_t prefetch_bytes, int num_cu,
                               hipStream_t st) {
  const size_t lds = resolve_pack_lds_bytes(N * B);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)resolve_pack_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  long n16 = (long)((prefetch_bytes < (size_t)kPackPrefetchBytes ? prefetch_bytes
                                                               : (size_t)kPackPrefetchBytes) / 16);
  if (prefetch == nullptr || (((uintptr_t)prefetch) & 15u) != 0) n16 = 0;
  const int grid = n16 > 0 ? num_cu : 1;
  resolve_pack_kernel<<<grid, kPackThreads, lds, st>>>(recompute, fold_src, src_in, N, B, mode,
                                                        src_out, packed_slot, slot_row, count,
                                                        (const uint4*)prefetch, n16, nullptr);
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
hipError_t launch_qkv_reduce_rope_bias(const GemmParams& gp, const int32_t* packed_slot, int B,
                                       int P, int n_q, int n_kv, int dh, const void* bias,
                                       float theta, hipStream_t st) {
  const long total = (long)gp.m_cap * (n_q + 2 * n_kv) * (dh / 8);
  const long blocks = (total + 255) / 256;
  qkv_reduce_rope_bias_kernel<T><<<(int)(blocks < 4096 ? blocks : 4096), 256, 0, st>>>(
      gp, packed_slot, B, P, n_q, n_kv, dh, (const T*)bias, theta);
  return hipGetLastError();
}
template hipError_t launch_qkv_reduce_rope_bias<float>(const GemmParams&, const int32_t*, int,
                                                       int, int, int, int, const void*, float,
                                                       hipStream_t);
template hipError_t launch_qkv_reduce_rope_bias<bf16>(const GemmParams&, const int32_t*, int,
                                                      int, int, int, int, const void*, float,
                                                      hipStream_t);

template <typename T>
hipError_t launch_oproj_finish(const float* partial, int split, const void* H, void* h, int S,
                               int d, const int32_t* slot_row, const int32_t* packed_slot,
                               const int32_t* count, const void* g, float eps, void* A2,
                               int ld_a2, bool by_row, int tiles_n, int kiters, int bm,
                               hipStream_t st) {
  oproj_finish_kernel<T><<<S, kFinishThreads, 0, st>>>(partial, split, (const T*)H, (T*)h, S, d,
                                                          slot_row, packed_slot, count,
                                                          (const T*)g, eps, (T*)A2, ld_a2,
                                                          by_row, tiles_n, kiters, bm);
  return hipGetLastError();
}
template hipError_t launch_oproj_finish<float>(const float*, int, const void*, void*, int, int,
                                               const int32_t*, const int32_t*, const int32_t*,
                                               const void*, float, void*, int, bool, int, int,
                                               int, hipStream_t);
template hipError_t launch_oproj_finish<bf16>(const float*, int, const void*, void*, int, int,
                                              const int32_t*, const int32_t*, const int32_t*,
                                              const void*, float, void*, int, bool, int, int,
                                              int, hipStream_t);

template hipError_t launch_gate<float>(const void*, const int32_t*, int, int, int, float, float*,
                                       uint8_t*, const uint8_t*, const void*, float, void*, int,
                                       hipStream_t);
template hipError_t launch_gate<bf16>(const void*, const int32_t*, int, int, int, float, float*,
                                      uint8_t*, const uint8_t*, const void*, float, void*, int,
                                      hipStream_t);
template hipError_t launch_combine<float>(const void*, const void*, const int32_t*, const int32_t*,
                                          int, int, int, void*, hipStream_t);
template hipError_t launch_combine<bf16>(const void*, const void*, const int32_t*, const int32_t*,
                                         int, int, int, void*, hipStream_t);

}  // namespace specfold
