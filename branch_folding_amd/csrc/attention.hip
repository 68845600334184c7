// Streaming GQA attention of the folded verify layer (SpecFold explainer, implementation
// memo: FlashAttention-style streaming; folded positions' attention is corrected with
// their own branch's keys and values; the shared cache is a zero-copy strided view; GQA).
//
// Prefix phase: for every packed row k and query head h, online-softmax partials
//   (lse, normalised output) over a range of prefix keys.  The prefix is read through the
//   caller's strided view once per (KV head, 64-query tile) -- never copied per branch --
//   and all g query heads of a KV head share every K/V tile.
// Split merge: the prefix partials of each (packed row, head) are merged once.
// Block phase: for every slot (n, i) and head h, the query of its packed row slot_row[n,i]
//   attends to branch n's own block keys/values (rows slot_row[n, j]); the running state
//   starts from the merged prefix partial of that packed row, which is the correction step.
//
// MFMA formulation: scores are computed transposed, S^T = K Q^T (keys as the A operand from
// LDS, queries as the B operand in registers), so every lane ends up holding one query's
// scores for 16 keys; the output is accumulated transposed, O^T = V^T P^T, so the
// probabilities feed the B operand straight from registers and V is staged transposed.
#include "common.h"
#include "kernels.h"

namespace specfold {

constexpr int kKeys = 64;   // keys per LDS tile
constexpr int kQRows = 64;  // query rows per workgroup (16 per wave)

template <typename T, int DH>
struct AttnTile {
  static constexpr int VE = 16 / sizeof(T);
  static constexpr int LDK = DH + 2 * VE;    // K tile row stride (elements, 32 B padding)
  static constexpr int LDV = kKeys + VE;     // transposed V tile row stride
  static constexpr int KSTEPS_QK = DH * (int)sizeof(T) / 64;   // 64-byte k-steps over dh
  static constexpr int KSTEPS_PV = kKeys * (int)sizeof(T) / 64;  // over the 64 keys
  static constexpr int NT = DH / 16;         // 16-wide output column tiles
};

struct AttnState {
  float m, l;
};

// A 64-key K/V tile moves global -> registers -> LDS in two steps, so the next tile's
// loads can be in flight while the current tile is being attended.
//   K: thread t holds chunks c = t + 256*u (key c / CPR, 16-byte chunk c % CPR), stored in
//      natural layout (row stride LDK).
//   V: thread t holds KQ consecutive keys kq*KQ .. kq*KQ+KQ-1 of one 16-byte chunk db
//      (kq = t % (64/KQ), db = t / (64/KQ)); it transposes them in registers and writes
//      each of its VE dh rows of Vt as one KQ-element vector (row stride LDV).
template <typename T, int DH>
struct KVRegs {
  static constexpr int VE = 16 / sizeof(T);
  static constexpr int CPR = DH / VE;          // 16-byte chunks per row
  static constexpr int KC = kKeys * CPR / 256; // K chunks per thread
  static constexpr int KQ = kKeys * CPR / 256; // V keys per thread
  uint4 k[KC];
  uint4 v[KQ];
};

template <typename T, int DH, typename KF, typename VF>
__device__ __forceinline__ void load_kv(KVRegs<T, DH>& r, int nkeys, KF key_ptr, VF val_ptr) {
  using R = KVRegs<T, DH>;
  const int t = threadIdx.x;
#pragma unroll
  for (int u = 0; u < R::KC; ++u) {
    const int c = t + 256 * u, j = c / R::CPR, cc = c - j * R::CPR;
    r.k[u] = j < nkeys ? ld16(key_ptr(j) + cc * R::VE) : make_uint4(0, 0, 0, 0);
  }
  const int kq = t % (kKeys / R::KQ), db = t / (kKeys / R::KQ);
#pragma unroll
  for (int u = 0; u < R::KQ; ++u) {
    const int j = kq * R::KQ + u;
    r.v[u] = j < nkeys ? ld16(val_ptr(j) + db * R::VE) : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ uint32_t word_at(const uint4& x, int i) {
  return i == 0 ? x.x : (i == 1 ? x.y : (i == 2 ? x.z : x.w));
}
// 16-bit element e (of 8) of x, zero-extended
__device__ __forceinline__ uint32_t bf16_at(const uint4& x, int e) {
  return (word_at(x, e >> 1) >> (16 * (e & 1))) & 0xffffu;
}

template <typename T, int DH>
__device__ __forceinline__ void store_kv(T* Ks, T* Vt, const KVRegs<T, DH>& r) {
  using R = KVRegs<T, DH>;
  using A = AttnTile<T, DH>;
  const int t = threadIdx.x;
#pragma unroll
  for (int u = 0; u < R::KC; ++u) {
    const int c = t + 256 * u, j = c / R::CPR, cc = c - j * R::CPR;
    *reinterpret_cast<uint4*>(&Ks[j * A::LDK + cc * R::VE]) = r.k[u];
  }
  const int kq = t % (kKeys / R::KQ), db = t / (kKeys / R::KQ);
  constexpr int NWORD = R::KQ * (int)sizeof(T) / 4;     // 32-bit words per Vt row piece
#pragma unroll
  for (int e = 0; e < R::VE; ++e) {
    uint32_t w[NWORD];
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int u = 0; u < R::KQ; u += 2)
        w[u / 2] = bf16_at(r.v[u], e) | (bf16_at(r.v[u + 1], e) << 16);
    } else {
#pragma unroll
      for (int u = 0; u < R::KQ; ++u) w[u] = word_at(r.v[u], e);
    }
    T* dst = &Vt[(db * R::VE + e) * A::LDV + kq * R::KQ];
    if constexpr (NWORD == 1) {
      *reinterpret_cast<uint32_t*>(dst) = w[0];
    } else if constexpr (NWORD == 2) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
    } else {
#pragma unroll
      for (int q = 0; q < NWORD / 4; ++q)
        reinterpret_cast<uint4*>(dst)[q] =
            make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
    }
  }
}

// Process one staged key tile for the wave's 16 queries.
template <typename T, int DH>
__device__ __forceinline__ void attend_tile(const T* Ks, const T* Vt, int nkeys,
                                            const uint4 (&qf)[AttnTile<T, DH>::KSTEPS_QK],
                                            float scale_log2, AttnState& st,
                                            f32x4 (&o)[AttnTile<T, DH>::NT]) {
  using A = AttnTile<T, DH>;
  constexpr int VE = A::VE;
  const int lane = threadIdx.x & 63, g4 = lane >> 4, l16 = lane & 15;
  // scores: sc[t][r] = key t*16 + g4*4 + r, query l16
  f32x4 sc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < A::KSTEPS_QK; ++ks) {
      const uint4 kf =
          *reinterpret_cast<const uint4*>(&Ks[(t * 16 + l16) * A::LDK + ks * 4 * VE + g4 * VE]);
      sc[t] = mma_kstep(kf, qf[ks], sc[t], T());
    }
  }
  float mloc = -__builtin_inff();
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = t * 16 + g4 * 4 + r;
      float v = sc[t][r] * scale_log2;
      if (key >= nkeys) v = -__builtin_inff();
      sc[t][r] = v;
      mloc = fmaxf(mloc, v);
    }
  mloc = group4_max(mloc);
  const float m_new = fmaxf(st.m, mloc);
  const float alpha = exp2f(st.m - m_new);     // st.m = -inf -> 0
  float lsum = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pv = exp2f(sc[t][r] - m_new);
      sc[t][r] = pv;
      lsum += pv;
    }
  lsum = group4_sum(lsum);
  st.l = st.l * alpha + lsum;
  st.m = m_new;
#pragma unroll
  for (int nt = 0; nt < A::NT; ++nt) o[nt] *= alpha;

  // O^T[n][q] += sum_keys Vt[n][key] * P[q][key]
#pragma unroll
  for (int mu = 0; mu < A::KSTEPS_PV; ++mu) {
    uint4 pb;
    int koff0, koff1;   // key offsets of the two 8-byte halves (bf16) / one 16-byte (f32)
    if constexpr (sizeof(T) == 2) {
      float pf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pf[e] = sc[2 * mu][e];
        pf[4 + e] = sc[2 * mu + 1][e];
      }
      pb = pack16(pf, T());
      koff0 = 32 * mu + 4 * g4;
      koff1 = 32 * mu + 16 + 4 * g4;
    } else {
      float pf[4] = {sc[mu][0], sc[mu][1], sc[mu][2], sc[mu][3]};
      pb = pack16(pf, T());
      koff0 = 16 * mu + 4 * g4;
      koff1 = 0;
    }
#pragma unroll
    for (int nt = 0; nt < A::NT; ++nt) {
      const T* vrow = &Vt[(nt * 16 + l16) * A::LDV];
      uint4 vf;
      if constexpr (sizeof(T) == 2) {
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow + koff0);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + koff1);
        vf = make_uint4(lo.x, lo.y, hi.x, hi.y);
      } else {
        vf = *reinterpret_cast<const uint4*>(vrow + koff0);
      }
      o[nt] = mma_kstep(vf, pb, o[nt], T());
    }
  }
}

// ------------------------------------------------------------------------------------
// Prefix phase.
// ------------------------------------------------------------------------------------
template <typename T, int DH>
__global__ void __launch_bounds__(256, 2) attn_prefix_kernel(AttnParams p) {
  using A = AttnTile<T, DH>;
  constexpr int VE = A::VE;
  __shared__ __attribute__((aligned(16))) T Ks[kKeys * A::LDK];
  __shared__ __attribute__((aligned(16))) T Vt[DH * A::LDV];
  const int K = imin(*p.count, p.cap);
  const int g = p.n_q / p.n_kv;
  const int ns = attn_splits(K, g, p.n_kv, p.P);
  if (ns == 0) return;
  const int qtiles = ceil_div(K * g, kQRows);
  const int units = p.n_kv * qtiles * ns;
  const int chunks = ceil_div(p.P, kKeys);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g4 = lane >> 4, l16 = lane & 15;
  const T* qkv = (const T*)p.qkv;
  const T* pk = (const T*)p.pk;
  const T* pv = (const T*)p.pv;

  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    // split fastest: the splits of one query tile run on different XCDs concurrently
    const int s = u % ns, rest = u / ns;
    const int qt = rest % qtiles, kvh = rest / qtiles;
    const int r = qt * kQRows + wave * 16 + l16;
    const bool valid = r < K * g;
    const int rr = valid ? r : K * g - 1;
    const int k = rr / g, h = kvh * g + (rr - (rr / g) * g);
    const T* qp = qkv + (size_t)k * p.ld_qkv + (size_t)h * DH;
    uint4 qf[A::KSTEPS_QK];
#pragma unroll
    for (int ks = 0; ks < A::KSTEPS_QK; ++ks) qf[ks] = ld16(qp + ks * 4 * VE + g4 * VE);
    AttnState st{-__builtin_inff(), 0.f};
    f32x4 o[A::NT];
#pragma unroll
    for (int nt = 0; nt < A::NT; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int c0 = (int)((long)s * chunks / ns), c1 = (int)((long)(s + 1) * chunks / ns);
    auto kp = [&](int key0) {
      return [=](int j) { return pk + (size_t)(key0 + j) * p.stride_tok + (size_t)kvh * p.stride_head; };
    };
    auto vp = [&](int key0) {
      return [=](int j) { return pv + (size_t)(key0 + j) * p.stride_tok + (size_t)kvh * p.stride_head; };
    };
    // tile c is staged from registers while tile c + 1 is already being loaded
    KVRegs<T, DH> kv;
    if (c0 < c1) load_kv<T, DH>(kv, imin(kKeys, p.P - c0 * kKeys), kp(c0 * kKeys), vp(c0 * kKeys));
    for (int c = c0; c < c1; ++c) {
      const int key0 = c * kKeys;
      const int nkeys = imin(kKeys, p.P - key0);
      __syncthreads();
      store_kv<T, DH>(Ks, Vt, kv);
      __syncthreads();
      if (c + 1 < c1) {
        const int key1 = key0 + kKeys;
        load_kv<T, DH>(kv, imin(kKeys, p.P - key1), kp(key1), vp(key1));
      }
      attend_tile<T, DH>(Ks, Vt, nkeys, qf, p.scale_log2, st, o);
    }
    if (valid) {
      const float inv = st.l > 0.f ? 1.0f / st.l : 0.f;
      const float lse = st.l > 0.f ? st.m + log2f(st.l) : -__builtin_inff();
      float* po = p.part_o + (((size_t)s * K + k) * p.n_q + h) * DH;
#pragma unroll
      for (int nt = 0; nt < A::NT; ++nt) {
        float4 v = make_float4(o[nt][0] * inv, o[nt][1] * inv, o[nt][2] * inv, o[nt][3] * inv);
        *reinterpret_cast<float4*>(po + nt * 16 + g4 * 4) = v;
      }
      if (g4 == 0) p.part_lse[((size_t)s * K + k) * p.n_q + h] = lse;
    }
  }
}

// ------------------------------------------------------------------------------------
// Merge of the prefix splits: plane 0 of (lse, o) becomes the merge of all ns planes, once
// per (packed row, query head) instead of once per slot that reads it.  One wave per
// (k, h); every lane loads before any lane stores, so the merge runs in place.
// ------------------------------------------------------------------------------------
template <int DH>
__device__ __forceinline__ void merge_row(const AttnParams& p, int K, int ns, int row, int lane) {
  constexpr int E = DH / 64;                  // output elements per lane
  const size_t plane_l = (size_t)K * p.n_q;
  constexpr int SB = 8;                      // splits per batch of loads
  float m = -__builtin_inff();
  for (int s0 = 0; s0 < ns; s0 += SB) {
    float ls[SB];
#pragma unroll
    for (int b = 0; b < SB; ++b)
      ls[b] = (s0 + b < ns) ? p.part_lse[(size_t)(s0 + b) * plane_l + row] : -__builtin_inff();
#pragma unroll
    for (int b = 0; b < SB; ++b) m = fmaxf(m, ls[b]);
  }
  float l = 0.f, acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  if (m > -__builtin_inff()) {
    for (int s0 = 0; s0 < ns; s0 += SB) {
      float ls[SB], v[SB][E];
#pragma unroll
      for (int b = 0; b < SB; ++b) {
        const int sb = imin(s0 + b, ns - 1);
        ls[b] = (s0 + b < ns) ? p.part_lse[(size_t)sb * plane_l + row] : -__builtin_inff();
        const float* po = p.part_o + ((size_t)sb * plane_l + row) * DH + lane * E;
#pragma unroll
        for (int e = 0; e < E; ++e) v[b][e] = po[e];
      }
#pragma unroll
      for (int b = 0; b < SB; ++b) {
        const float w = exp2f(ls[b] - m);       // 0 for an absent or empty split
        l += w;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += w * v[b][e];
      }
    }
  }
  float* po = p.part_o + (size_t)row * DH + lane * E;
  const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) po[e] = acc[e] * inv;
  if (lane == 0) p.part_lse[row] = l > 0.f ? m + log2f(l) : -__builtin_inff();
}

template <int DH>
__global__ void __launch_bounds__(256) attn_merge_kernel(AttnParams p) {
  const int K = imin(*p.count, p.cap);
  const int g = p.n_q / p.n_kv;
  if (!attn_merge_on(K, g, p.n_kv, p.P, p.S)) return;
  const int ns = attn_splits(K, g, p.n_kv, p.P);
  const int lane = threadIdx.x & 63;
  for (int row = blockIdx.x * 4 + (threadIdx.x >> 6); row < K * p.n_q; row += gridDim.x * 4)
    merge_row<DH>(p, K, ns, row, lane);
}

// ------------------------------------------------------------------------------------
// Block phase + merge.
// ------------------------------------------------------------------------------------
template <typename T, int DH>
__global__ void __launch_bounds__(256, 2) attn_block_kernel(AttnParams p) {
  using A = AttnTile<T, DH>;
  constexpr int VE = A::VE;
  __shared__ __attribute__((aligned(16))) T Ks[kKeys * A::LDK];
  __shared__ __attribute__((aligned(16))) T Vt[DH * A::LDV];
  const int K = imin(*p.count, p.cap);
  if (K <= 0) return;
  const int g = p.n_q / p.n_kv;
  // plane 0 holds all prefix splits when attn_merge_kernel merged them
  const int ns = attn_merge_on(K, g, p.n_kv, p.P, p.S) ? 1 : attn_splits(K, g, p.n_kv, p.P);
  const int qtiles = ceil_div(p.B * g, kQRows);
  const int units = p.N * p.n_kv * qtiles;
  const int kchunks = ceil_div(p.B, kKeys);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g4 = lane >> 4, l16 = lane & 15;
  const T* qkv = (const T*)p.qkv;
  const long koff = (long)p.n_q * DH, voff = (long)(p.n_q + p.n_kv) * DH;
  auto row_of = [&](int slot) { return imin(imax(p.slot_row[slot], 0), K - 1); };

  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int qt = u % qtiles, rest = u / qtiles;
    const int kvh = rest % p.n_kv, n = rest / p.n_kv;
    const int r = qt * kQRows + wave * 16 + l16;
    const bool valid = r < p.B * g;
    const int rr = valid ? r : p.B * g - 1;
    const int i = rr / g, h = kvh * g + (rr - i * g);
    const int k = row_of(n * p.B + i);
    // branch n's own block rows are the keys; their packed rows come from slot_row
    auto kp = [&](int key0) {
      return [=](int j) { return qkv + (size_t)row_of(n * p.B + key0 + j) * p.ld_qkv + koff + (size_t)kvh * DH; };
    };
    auto vp = [&](int key0) {
      return [=](int j) { return qkv + (size_t)row_of(n * p.B + key0 + j) * p.ld_qkv + voff + (size_t)kvh * DH; };
    };
    KVRegs<T, DH> kv;
    load_kv<T, DH>(kv, imin(kKeys, p.B), kp(0), vp(0));
    const T* qp = qkv + (size_t)k * p.ld_qkv + (size_t)h * DH;
    uint4 qf[A::KSTEPS_QK];
#pragma unroll
    for (int ks = 0; ks < A::KSTEPS_QK; ++ks) qf[ks] = ld16(qp + ks * 4 * VE + g4 * VE);

    // start from the prefix partials of packed row k (merged a batch of splits at a time,
    // so all loads of a batch are in flight together)
    AttnState st{-__builtin_inff(), 0.f};
    f32x4 o[A::NT];
#pragma unroll
    for (int nt = 0; nt < A::NT; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int PB = 16 / A::NT;            // 2 (dh 128) or 4 (dh 64) splits per batch
    for (int s0 = 0; s0 < ns; s0 += PB) {
      float ls[PB];
      float4 po[PB][A::NT];
#pragma unroll
      for (int b = 0; b < PB; ++b) {
        const int sb = imin(s0 + b, ns - 1);
        const size_t prow = ((size_t)sb * K + k) * p.n_q + h;
        ls[b] = (s0 + b < ns) ? p.part_lse[prow] : -__builtin_inff();
        const float* pp = p.part_o + prow * DH;
#pragma unroll
        for (int nt = 0; nt < A::NT; ++nt)
          po[b][nt] = *reinterpret_cast<const float4*>(pp + nt * 16 + g4 * 4);
      }
      float mb = st.m;
#pragma unroll
      for (int b = 0; b < PB; ++b) mb = fmaxf(mb, ls[b]);
      if (mb > -__builtin_inff()) {
        const float alpha = exp2f(st.m - mb);
        st.l *= alpha;
#pragma unroll
        for (int nt = 0; nt < A::NT; ++nt) o[nt] *= alpha;
#pragma unroll
        for (int b = 0; b < PB; ++b) {
          const float w = exp2f(ls[b] - mb);       // 0 for an empty or absent split
          st.l += w;
#pragma unroll
          for (int nt = 0; nt < A::NT; ++nt) {
            o[nt][0] += w * po[b][nt].x;
            o[nt][1] += w * po[b][nt].y;
            o[nt][2] += w * po[b][nt].z;
            o[nt][3] += w * po[b][nt].w;
          }
        }
        st.m = mb;
      }
    }

    for (int c = 0; c < kchunks; ++c) {
      const int key0 = c * kKeys;
      const int nkeys = imin(kKeys, p.B - key0);
      __syncthreads();
      store_kv<T, DH>(Ks, Vt, kv);
      __syncthreads();
      if (c + 1 < kchunks) {
        const int key1 = key0 + kKeys;
        load_kv<T, DH>(kv, imin(kKeys, p.B - key1), kp(key1), vp(key1));
      }
      attend_tile<T, DH>(Ks, Vt, nkeys, qf, p.scale_log2, st, o);
    }
    if (valid) {
      const float inv = 1.0f / st.l;
      T* op = (T*)p.out + (size_t)(n * p.B + i) * p.ld_out + (size_t)h * DH;
#pragma unroll
      for (int nt = 0; nt < A::NT; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) op[nt * 16 + g4 * 4 + e] = from_f32<T>(o[nt][e] * inv);
    }
  }
}

size_t attn_partial_rows(int S, int g, int n_kv, int P) {
  size_t best = 0;
  for (int K = 1; K <= S; ++K) {
    const size_t v = (size_t)attn_splits(K, g, n_kv, P) * K;
    if (v > best) best = v;
  }
  return best;
}

template <typename T>
hipError_t launch_attn_prefix(const AttnParams& p, int num_cu, hipStream_t st) {
  if (p.P <= 0) return hipSuccess;
  const int grid = 2 * num_cu;
  const int mrows = ceil_div(p.cap * p.n_q, 4);
  const int mgrid = mrows < num_cu ? mrows : num_cu;   // persistent
  if (p.dh == 128) {
    attn_prefix_kernel<T, 128><<<grid, 256, 0, st>>>(p);
    attn_merge_kernel<128><<<mgrid, 256, 0, st>>>(p);
  } else if (p.dh == 64) {
    attn_prefix_kernel<T, 64><<<grid, 256, 0, st>>>(p);
    attn_merge_kernel<64><<<mgrid, 256, 0, st>>>(p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_attn_block(const AttnParams& p, int num_cu, hipStream_t st) {
  const int g = p.n_q / p.n_kv;
  const int units = p.N * p.n_kv * ceil_div(p.B * g, kQRows);
  const int grid = units < 2 * num_cu ? units : 2 * num_cu;
  if (p.dh == 128) attn_block_kernel<T, 128><<<grid, 256, 0, st>>>(p);
  else if (p.dh == 64) attn_block_kernel<T, 64><<<grid, 256, 0, st>>>(p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template hipError_t launch_attn_prefix<float>(const AttnParams&, int, hipStream_t);
template hipError_t launch_attn_prefix<bf16>(const AttnParams&, int, hipStream_t);
template hipError_t launch_attn_block<float>(const AttnParams&, int, hipStream_t);
template hipError_t launch_attn_block<bf16>(const AttnParams&, int, hipStream_t);

}  // namespace specfold
