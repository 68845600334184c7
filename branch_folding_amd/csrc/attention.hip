// Streaming GQA attention of the folded verify layer (SpecFold explainer, implementation
// memo: FlashAttention-style streaming; folded positions' attention is corrected with
// their own branch's keys and values; the shared cache is a zero-copy strided view; GQA).
//
// Prefix phase: for every packed row k and query head h, online-softmax partials
//   (lse, normalised output) over a range of prefix keys.  The prefix is read through the
//   caller's strided view once per (KV head, query tile) -- never copied per branch -- and
//   all g query heads of a KV head share every K/V tile.  Two kernels: 256-query tiles
//   with a direct-to-LDS K/V ring for bf16 prefixes of 2048+ keys, 64-query tiles with
//   K/V staged through registers otherwise (short prefixes spread over more units).
// Split merge: the prefix partials of each (packed row, head) are merged once, when that
//   saves enough partial traffic; otherwise the block phase merges them.
// Block phase: for every slot (n, i) and head h, the query of its packed row slot_row[n,i]
//   attends to branch n's own block keys/values (rows slot_row[n, j]); the running state
//   starts from the merged prefix partial of that packed row, which is the correction step.
//
// MFMA formulation: scores are computed transposed, S^T = K Q^T (keys as the A operand from
// LDS, queries as the B operand in registers), so every lane ends up holding one query's
// scores for 16 keys; the output is accumulated transposed, O^T = V^T P^T, so the
// probabilities feed the B operand straight from registers; the V^T operand comes from a
// transposed copy of V in LDS, or from V's natural layout through transposed LDS reads.
#include "common.h"
#include "kernels.h"

namespace specfold {

constexpr int kKeys = 64;   // keys per LDS tile
constexpr int kQRows = 64;  // query rows per workgroup (16 per wave)

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
// s_waitcnt immediates: at most n vector-memory operations pending (vmcnt split over bits
// 3:0 and 15:14; expcnt and lgkmcnt not waited for), and the same with every LDS
// operation of the wave returned
constexpr int tr_waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int tr_waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

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

// Raw v_exp_f32: 2^x for the softmax weights.  Its arguments are <= 0 here; results below
// the normal range flush towards 0, which only drops weights under 2^-126 of the maximum.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Prefix partial outputs (each split's normalised output rows) are stored in the model dtype:
// the block phase re-reads a packed row's partials once for every slot that takes that row,
// so bf16 layers halve those reads.  Four consecutive elements per access.
__device__ __forceinline__ void st_part4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void st_part4(bf16* p, float a, float b, float c, float d) {
  const bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ float4 ld_part4(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}
__device__ __forceinline__ float4 ld_part4(const bf16* p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
}

// Online-softmax update of one tile of KC x 16 keys (64 by default) for the lane's query:
// sc[t][r] holds the raw score of key t*16 + (lane/16)*4 + r and becomes its unnormalised
// weight 2^(score * scale_log2 - m).  Keys >= nkeys (a ragged last tile) get weight 0;
// nkeys >= 1.  The reference point m is the running maximum only up to a slack: a lane
// moves it only when the tile's maximum exceeds it by more than kSoftmaxSlack (log2
// units), so the weights stay below 2^kSoftmaxSlack, and the running output (m, l and o
// stay consistent, the normalised result is the same) is rescaled only when some lane
// moved it -- after the first tiles, rarely.
constexpr float kSoftmaxSlack = 8.0f;
template <int NT, int KC = 4>
__device__ __forceinline__ void softmax_tile(f32x4 (&sc)[KC], int nkeys, float scale_log2,
                                             AttnState& st, f32x4 (&o)[NT]) {
  if (nkeys < KC * 16) {   // uniform branch, ragged tiles only
    // key t*16 + g4*4 + r is past the end iff t*16 + r >= nkeys - g4*4
    const int th = nkeys - ((threadIdx.x & 63) >> 4) * 4;
#pragma unroll
    for (int t = 0; t < KC; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (t * 16 + r >= th) sc[t][r] = -__builtin_inff();
  }
  float mloc = sc[0][0];
#pragma unroll
  for (int t = 0; t < KC; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) mloc = fmaxf(mloc, sc[t][r]);
  mloc = group4_max(mloc);
  const float cand = mloc * scale_log2;                  // scale_log2 > 0
  const float m_new = cand > st.m + kSoftmaxSlack ? cand : st.m;   // st.m = -inf: cand
  const float alpha = fast_exp2(st.m - m_new);           // st.m = -inf -> 0
  float lsum = 0.f;
#pragma unroll
  for (int t = 0; t < KC; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pv = fast_exp2(fmaf(sc[t][r], scale_log2, -m_new));
      sc[t][r] = pv;
      lsum += pv;
    }
  lsum = group4_sum(lsum);
  st.l = st.l * alpha + lsum;
  st.m = m_new;
  if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[nt] *= alpha;
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
  softmax_tile<A::NT>(sc, nkeys, scale_log2, st, o);

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
// Order of the prefix units over the grid.  Workgroups are dispatched to the 8 XCDs round
// robin (workgroup b runs on XCD b % 8), and each XCD has its own L2.  The units are
// numbered (KV head, key split) major and query tile fastest, and XCD x takes the
// contiguous range [x * per, (x + 1) * per) of them: the query tiles that share one KV
// head's key range run side by side on one XCD and stream its K/V tiles through that
// XCD's L2 instead of each XCD fetching every key range from HBM.  A grid that is not a
// multiple of 8 walks the units in plain order.
struct PrefixWalk {
  int v, end, step;
  __device__ PrefixWalk(int units) {
    const int nx = (gridDim.x % 8 == 0) ? 8 : 1;
    const int per = (units + nx - 1) / nx;
    const int x = blockIdx.x % nx;
    v = x * per + blockIdx.x / nx;
    end = imin((x + 1) * per, units);
    step = gridDim.x / nx;
  }
};

// The prefix phase records its split count and the merge decision for this call's packed
// count (one thread of workgroup 0), so the later attention kernels need not evaluate the
// cost model again in every workgroup.  Without a prefix the phase is not launched and the
// readers use ns = 0.
__device__ __forceinline__ void write_plan(const AttnParams& p, int K, int g, int ns, int dh,
                                           int eb) {
  p.plan[0] = ns;
  p.plan[1] = attn_merge_on(K, g, p.n_kv, p.P, p.S, dh, eb) ? 1 : 0;
}

// fp32 and short bf16 prefixes: 64-query units, K/V tiles staged through registers (V
// transposed on the way into LDS), two workgroups per CU.
template <typename T, int DH>
__global__ void __launch_bounds__(256, 2) attn_prefix_kernel(AttnParams p) {
  using A = AttnTile<T, DH>;
  constexpr int VE = A::VE;
  __shared__ __attribute__((aligned(16))) T Ks[kKeys * A::LDK];
  __shared__ __attribute__((aligned(16))) T Vt[DH * A::LDV];
  const int K = imin(*p.count, p.cap);
  const int g = p.n_q / p.n_kv;
  const int ns = attn_splits(K, g, p.n_kv, p.P, DH, (int)sizeof(T));
  if (blockIdx.x == 0 && threadIdx.x == 0) write_plan(p, K, g, ns, DH, (int)sizeof(T));
  if (ns == 0) return;
  const int qtiles = ceil_div(K * g, kQRows);
  const int units = p.n_kv * qtiles * ns;
  const int chunks = ceil_div(p.P, kKeys);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g4 = lane >> 4, l16 = lane & 15;
  const T* qkv = (const T*)p.qkv;
  const T* pk = (const T*)p.pk;
  const T* pv = (const T*)p.pv;

  for (PrefixWalk w(units); w.v < w.end; w.v += w.step) {
    const int qt = w.v % qtiles, pair = w.v / qtiles;
    const int s = pair % ns, kvh = pair / ns;
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
      T* po = (T*)p.part_o + (((size_t)s * K + k) * p.n_q + h) * DH;
#pragma unroll
      for (int nt = 0; nt < A::NT; ++nt)
        st_part4(po + nt * 16 + g4 * 4, o[nt][0] * inv, o[nt][1] * inv, o[nt][2] * inv,
                 o[nt][3] * inv);
      if (g4 == 0) p.part_lse[((size_t)s * K + k) * p.n_q + h] = lse;
    }
  }
}

// ------------------------------------------------------------------------------------
// Prefix phase, bf16.  A unit is 256 query rows (8 waves x 2 blocks of 16) of one KV head
// against one key range, so every K/V tile staged in LDS serves 256 queries:
//   * K and V tiles go global -> LDS with direct-to-LDS loads into a ring of four stages
//     (separate arrays, so the compiler sees that loads into one stage never alias reads
//     of another), three tiles in flight while one is attended; one s_waitcnt + s_barrier
//     per tile;
//   * V stays in its natural [key][dh] layout: the V^T operand of O^T = V^T P^T is read
//     with ds_read_b64_tr_b16, which hands lane 4a+b of each 16-lane group element b of
//     the 8-byte rows that lanes a, a+4, a+8 and a+12 point at, i.e. four consecutive keys
//     of one dh column when the 16 lanes point at 4 keys x 4 column quads;
//   * every K fragment and V fragment read from LDS feeds the MFMAs of both query blocks.
// LDS rows are XOR-swizzled in 16-byte chunks (the loads pick their global chunk to
// match): the K fragment reads (16 rows at one chunk) and the transposed V reads (8 rows
// x 32 bytes per half wave) each touch distinct banks.
// ------------------------------------------------------------------------------------
constexpr int kTrWaves = 8;
constexpr int kTrQRows = kTrWaves * 32;   // query rows per unit
constexpr int kTrStages = 4;

template <int DH, int NWV = kTrWaves>
struct TrTile {
  static constexpr int ROWB = DH * 2;                   // bytes per K (or V) row
  static constexpr int TILEB = kKeys * ROWB;            // bytes per K (or V) tile
  static constexpr int RP = 256 / ROWB;                 // rows per 256 bytes (1 or 2)
  static constexpr int CPR = ROWB / 16;                 // 16-byte chunks per row
  static constexpr int QI = TILEB / 1024 / NWV;         // K (and V) loads per wave per tile
  static constexpr int LPI = 2 * QI;                    // vector-memory ops per wave per tile
  static constexpr int KSQ = DH / 32;                   // 64-byte k-steps over dh
  static constexpr int NT = DH / 16;                    // 16-wide dh tiles of the output
  static_assert(QI >= 1 && TILEB % (1024 * NWV) == 0, "tile/loader mismatch");
};
// physical 16-byte chunk = logical chunk ^ swizzle(row)
template <int DH>
__device__ __forceinline__ int tr_kswz(int r) {
  return (r / TrTile<DH>::RP) & (TrTile<DH>::CPR - 1);
}
template <int DH>
__device__ __forceinline__ int tr_vswz(int r) {
  return 2 * ((r / TrTile<DH>::RP) & (8 / TrTile<DH>::RP - 1));
}

typedef short tr_v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) tr_v4s lds_tr_v4s;

// KC x 16 keys starting at the stage rows Ks / Vs point at (a whole 64-key tile, or half of
// one with KC = 2); nkeys >= 1 of them are live.
template <int DH, int NB = 2, int KC = 4>
__device__ __forceinline__ void tr_attend(const char* Ks, const char* Vs, int nkeys,
                                          const uint4 (&qf)[NB][TrTile<DH>::KSQ],
                                          const int (&kofs)[TrTile<DH>::KSQ],
                                          const int (&vofs)[TrTile<DH>::NT], float scale_log2,
                                          AttnState (&st)[NB], f32x4 (&o)[NB][TrTile<DH>::NT]) {
  using Tt = TrTile<DH>;
  static_assert(KC == 2 || KC == 4, "whole or half tiles");
  // The two waves sharing a SIMD alternate between MFMA phases and the softmax; the MFMA
  // phases run at raised wave priority, so one wave's MFMAs issue ahead of the other's
  // softmax and the matrix pipe stays busy.
  __builtin_amdgcn_s_setprio(1);
  // S^T = K Q^T: sc[b][t][r] = key t*16 + g4*4 + r, query l16 of block b
  f32x4 sc[NB][KC];
#pragma unroll
  for (int t = 0; t < KC; ++t) {
#pragma unroll
    for (int b = 0; b < NB; ++b) sc[b][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < Tt::KSQ; ++ks) {
      const uint4 kf = *reinterpret_cast<const uint4*>(Ks + kofs[ks] + t * 16 * Tt::ROWB);
#pragma unroll
      for (int b = 0; b < NB; ++b) sc[b][t] = mma_kstep(kf, qf[b][ks], sc[b][t], bf16());
    }
  }
  __builtin_amdgcn_s_setprio(0);
#pragma unroll
  for (int b = 0; b < NB; ++b) softmax_tile<Tt::NT, KC>(sc[b], nkeys, scale_log2, st[b], o[b]);
  // P^T as the B operand: k-step mu covers keys 32mu + 4*g4 + 0..3 and 32mu + 16 + 4*g4 + 0..3
  constexpr int MU = KC / 2;
  uint4 pb[NB][MU];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int mu = 0; mu < MU; ++mu) {
      float pf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pf[e] = sc[b][2 * mu][e];
        pf[4 + e] = sc[b][2 * mu + 1][e];
      }
      pb[b][mu] = pack16(pf, bf16());
    }
  // O^T += V^T P^T with V^T fragments read transposed from the natural V tile: the same
  // two key quads per lane group as the P^T operand above
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int mu = 0; mu < MU; ++mu)
#pragma unroll
    for (int nt = 0; nt < Tt::NT; ++nt) {
      const tr_v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_tr_v4s*)(Vs + vofs[nt] + 32 * mu * Tt::ROWB));
      const tr_v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_tr_v4s*)(Vs + vofs[nt] + (32 * mu + 16) * Tt::ROWB));
      const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
      const uint4 vf = make_uint4(l2.x, l2.y, h2.x, h2.y);
#pragma unroll
      for (int b = 0; b < NB; ++b) o[b][nt] = mma_kstep(vf, pb[b][mu], o[b][nt], bf16());
    }
  __builtin_amdgcn_s_setprio(0);
}

template <int DH>
__global__ void __launch_bounds__(kTrWaves * 64, 1) attn_prefix_tr_kernel(AttnParams p) {
  using Tt = TrTile<DH>;
  constexpr int QI = Tt::QI, LPI = Tt::LPI, KSQ = Tt::KSQ, NT = Tt::NT;
  __shared__ __attribute__((aligned(1024))) char K0[Tt::TILEB], K1[Tt::TILEB], K2[Tt::TILEB],
      K3[Tt::TILEB];
  __shared__ __attribute__((aligned(1024))) char V0[Tt::TILEB], V1[Tt::TILEB], V2[Tt::TILEB],
      V3[Tt::TILEB];
  const int K = imin(*p.count, p.cap);
  const int g = p.n_q / p.n_kv;
  const int ns = attn_splits(K, g, p.n_kv, p.P, DH, 2);
  if (blockIdx.x == 0 && threadIdx.x == 0) write_plan(p, K, g, ns, DH, 2);
  if (ns == 0) return;
  const int rows = K * g;
  const int qtiles = ceil_div(rows, kTrQRows);
  const int units = p.n_kv * qtiles * ns;
  const int chunks = ceil_div(p.P, kKeys);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g4 = lane >> 4, l16 = lane & 15;
  const char* qkv = (const char*)p.qkv;
  const long st_tok = p.stride_tok * 2, st_head = p.stride_head * 2;   // bytes

  // LDS byte offsets of this lane's fragments: K rows t*16 + l16 at chunk 4ks + g4 (plus
  // t*16 rows); V^T quads at key 4*g4 + l16/4, dh 16nt + 4*(l16%4) (plus 32mu / +16 keys)
  int kofs[KSQ], vofs[NT];
#pragma unroll
  for (int ks = 0; ks < KSQ; ++ks)
    kofs[ks] = l16 * Tt::ROWB + (((4 * ks + g4) ^ tr_kswz<DH>(l16)) << 4);
  {
    const int vr = 4 * g4 + (l16 >> 2);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      vofs[nt] = vr * Tt::ROWB + (((2 * nt + ((l16 & 3) >> 1)) ^ tr_vswz<DH>(vr)) << 4) +
                 8 * (l16 & 1);
  }
  // loader geometry: load q of this wave fills LDS bytes (wave*QI + q)*1024 + 16*lane of a
  // stage, i.e. row r, physical chunk pc, and fetches the matching logical chunk; lko / lvo
  // are the byte offsets of that K / V chunk from the tile's first row (< 64 rows)
  uint32_t lko[QI], lvo[QI];
#pragma unroll
  for (int q = 0; q < QI; ++q) {
    const int byte = (wave * QI + q) * 1024 + 16 * lane;
    const int r = byte / Tt::ROWB, pc = (byte % Tt::ROWB) >> 4;
    lko[q] = (uint32_t)(r * st_tok) + ((pc ^ tr_kswz<DH>(r)) << 4);
    lvo[q] = (uint32_t)(r * st_tok) + ((pc ^ tr_vswz<DH>(r)) << 4);
  }
  const int wq = __builtin_amdgcn_readfirstlane(wave) * QI * 1024;   // wave's LDS slice

  for (PrefixWalk w(units); w.v < w.end; w.v += w.step) {
    const int qt = w.v % qtiles, pair = w.v / qtiles;
    const int s = pair % ns, kvh = pair / ns;
    uint4 qf[2][KSQ];
    bool valid[2];
    int krow[2], hq[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int r = qt * kTrQRows + wave * 32 + b * 16 + l16;
      valid[b] = r < rows;
      const int rr = valid[b] ? r : rows - 1;
      krow[b] = rr / g;
      hq[b] = kvh * g + (rr - krow[b] * g);
      const char* qp = qkv + ((size_t)krow[b] * p.ld_qkv + (size_t)hq[b] * DH) * 2;
#pragma unroll
      for (int ks = 0; ks < KSQ; ++ks) qf[b][ks] = ld16(qp + (4 * ks + g4) * 16);
    }
    AttnState st[2] = {{-__builtin_inff(), 0.f}, {-__builtin_inff(), 0.f}};
    f32x4 o[2][NT];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o[b][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int c0 = (int)((long)s * chunks / ns), c1 = (int)((long)(s + 1) * chunks / ns);
    const int n = c1 - c0;
    const char* kb = (const char*)p.pk + (size_t)kvh * st_head;
    const char* vb = (const char*)p.pv + (size_t)kvh * st_head;
    // Every tile slot issues its loads, so each wave has exactly two tiles in flight behind
    // the one it waits for and the wait count is a constant the compiler can track (with
    // conditional loads it drains the ring at the loop head).  Slots past the unit's last
    // tile load one shared cache line (the head's first row) into the stage just freed;
    // rows past the prefix (a ragged last tile) load the last key: finite values whose
    // weights the softmax sets to 0.
    auto issue = [&](char* Kd, char* Vd, int i) {
      const int key0 = (c0 + i) * kKeys;
      const uint32_t kl = lds_addr(Kd) + wq, vl = lds_addr(Vd) + wq;
      const char* ks[QI];
      const char* vs[QI];
      if (i >= n) {                       // past the unit's last tile
#pragma unroll
        for (int q = 0; q < QI; ++q) ks[q] = kb, vs[q] = vb;
      } else {
        const char* kt = kb + (size_t)key0 * st_tok;
        const char* vt = vb + (size_t)key0 * st_tok;
        if (key0 + kKeys <= p.P) {        // full tile
#pragma unroll
          for (int q = 0; q < QI; ++q) ks[q] = kt + lko[q], vs[q] = vt + lvo[q];
        } else {                          // ragged last tile: rows past the end reload row P-1
          const int last = p.P - 1 - key0;
#pragma unroll
          for (int q = 0; q < QI; ++q) {
            const int r = ((wave * QI + q) * 1024 + 16 * lane) / Tt::ROWB;
            const int cut = r > last ? r - last : 0;
            ks[q] = kt + lko[q] - (long)cut * st_tok;
            vs[q] = vt + lvo[q] - (long)cut * st_tok;
          }
        }
      }
#pragma unroll
      for (int q = 0; q < QI; ++q) {
        dma16(ks[q], kl + q * 1024);
        dma16(vs[q], vl + q * 1024);
      }
    };
    // tile i: once it has landed (tiles i + 1 and i + 2 may still be in flight) and every
    // wave has finished tile i - 1, tile i is attended and the loads of tile i + 3 go into
    // the stage of i - 1 (after the MFMAs: with two tiles in flight the CU's outstanding
    // loads are at their limit, and issuing first would stall the wave before its MFMAs)
    auto body = [&](const char* Kc, const char* Vc, char* Kn, char* Vn, int i) {
      if (i >= n) return;
      __builtin_amdgcn_s_waitcnt(tr_waitcnt_vm(2 * LPI));
      __builtin_amdgcn_s_barrier();
      const int nkeys = imin(kKeys, p.P - (c0 + i) * kKeys);
      tr_attend<DH>(Kc, Vc, nkeys, qf, kofs, vofs, p.scale_log2, st, o);
      issue(Kn, Vn, i + 3);
    };
    // the previous unit's loads, stores and LDS reads and this unit's query loads are done
    // before the ring is refilled (the scheduling fence keeps the query loads above the
    // wait, so no later wait has to drain the ring for them)
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(tr_waitcnt_vm_lgkm0(0));
    __builtin_amdgcn_s_barrier();
    issue(K0, V0, 0);
    issue(K1, V1, 1);
    issue(K2, V2, 2);
    for (int it = 0; it < n; it += kTrStages) {
      body(K0, V0, K3, V3, it);
      body(K1, V1, K0, V0, it + 1);
      body(K2, V2, K1, V1, it + 2);
      body(K3, V3, K2, V2, it + 3);
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if (!valid[b]) continue;
      const float inv = st[b].l > 0.f ? 1.0f / st[b].l : 0.f;
      const float lse = st[b].l > 0.f ? st[b].m + log2f(st[b].l) : -__builtin_inff();
      bf16* po = (bf16*)p.part_o + (((size_t)s * K + krow[b]) * p.n_q + hq[b]) * DH;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        st_part4(po + nt * 16 + g4 * 4, o[b][nt][0] * inv, o[b][nt][1] * inv,
                 o[b][nt][2] * inv, o[b][nt][3] * inv);
      if (g4 == 0) p.part_lse[((size_t)s * K + krow[b]) * p.n_q + hq[b]] = lse;
    }
  }
  __builtin_amdgcn_s_waitcnt(tr_waitcnt_vm_lgkm0(0));
}

// ------------------------------------------------------------------------------------
// Merge of the prefix splits: plane 0 of (lse, o) becomes the merge of all ns planes, once
// per (packed row, query head) instead of once per slot that reads it.  One wave per
// (k, h): lane s < ns loads split s's lse, the wave reduces the maximum and the weights,
// then every lane combines its DH/64 output elements over the splits, the loads of eight
// splits in flight at a time.  Every lane loads before any lane stores, so the merge runs
// in place.
// ------------------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

template <typename T, int DH>
__device__ __forceinline__ void merge_row(const AttnParams& p, int K, int ns, int row, int lane) {
  constexpr int E = DH / 64;                  // output elements per lane
  constexpr int SB = 8;                       // splits per batch of loads
  const size_t plane_l = (size_t)K * p.n_q;
  const float ls = lane < ns ? p.part_lse[(size_t)lane * plane_l + row] : -__builtin_inff();
  const float m = wave_max(ls);
  float l = 0.f, acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  if (m > -__builtin_inff()) {
    const float w = exp2f(ls - m);            // 0 for lanes past ns and for empty splits
    l = wave_sum(w);
    for (int s0 = 0; s0 < ns; s0 += SB) {
      float ws[SB], v[SB][E];
#pragma unroll
      for (int b = 0; b < SB; ++b) {
        const int sb = imin(s0 + b, ns - 1);
        ws[b] = s0 + b < ns ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), sb))
                            : 0.f;
        const T* po = (const T*)p.part_o + ((size_t)sb * plane_l + row) * DH + lane * E;
#pragma unroll
        for (int e = 0; e < E; ++e) v[b][e] = to_f32(po[e]);
      }
#pragma unroll
      for (int b = 0; b < SB; ++b)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += ws[b] * v[b][e];
    }
  }
  T* po = (T*)p.part_o + (size_t)row * DH + lane * E;
  const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) po[e] = from_f32<T>(acc[e] * inv);
  if (lane == 0) p.part_lse[row] = l > 0.f ? m + log2f(l) : -__builtin_inff();
}

template <typename T, int DH>
__global__ void __launch_bounds__(256) attn_merge_kernel(AttnParams p) {
  const int K = imin(*p.count, p.cap);
  if (p.P <= 0 || K <= 0 || p.plan[1] == 0) return;
  const int ns = p.plan[0];
  const int lane = threadIdx.x & 63;
  for (int row = blockIdx.x * 4 + (threadIdx.x >> 6); row < K * p.n_q; row += gridDim.x * 4)
    merge_row<T, DH>(p, K, ns, row, lane);
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
  // the plan is loaded with the count (without a prefix phase it is not written and not used)
  const int plan_ns = p.plan[0], plan_merged = p.plan[1];
  const int K = imin(*p.count, p.cap);
  if (K <= 0) return;
  const int g = p.n_q / p.n_kv;
  // a short prefix is streamed here, tile by tile, ahead of the block (no prefix phase ran)
  const bool fused = p.fused != 0;
  // plane 0 holds all prefix splits when attn_merge_kernel merged them
  const int ns = (p.P <= 0 || fused) ? 0 : (plan_merged ? 1 : plan_ns);
  const int qtiles = ceil_div(p.B * g, kQRows);
  const int units = p.N * p.n_kv * qtiles;
  const int pchunks = fused ? ceil_div(p.P, kKeys) : 0;
  const int tiles = pchunks + ceil_div(p.B, kKeys);
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
    // tile c < pchunks: prefix keys 64c.., through the caller's strided view; then the block
    const T* pkb = (const T*)p.pk + (size_t)kvh * p.stride_head;
    const T* pvb = (const T*)p.pv + (size_t)kvh * p.stride_head;
    auto tile_keys = [&](int c) {
      return c < pchunks ? imin(kKeys, p.P - c * kKeys) : imin(kKeys, p.B - (c - pchunks) * kKeys);
    };
    KVRegs<T, DH> kv;
    auto load_tile = [&](int c) {
      if (c < pchunks) {
        const size_t key0 = (size_t)c * kKeys;
        load_kv<T, DH>(kv, tile_keys(c),
                       [=](int j) { return pkb + (key0 + j) * p.stride_tok; },
                       [=](int j) { return pvb + (key0 + j) * p.stride_tok; });
      } else {
        const int key0 = (c - pchunks) * kKeys;
        load_kv<T, DH>(kv, tile_keys(c), kp(key0), vp(key0));
      }
    };
    load_tile(0);
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
        const T* pp = (const T*)p.part_o + prow * DH;
#pragma unroll
        for (int nt = 0; nt < A::NT; ++nt) po[b][nt] = ld_part4(pp + nt * 16 + g4 * 4);
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

    for (int c = 0; c < tiles; ++c) {
      const int nkeys = tile_keys(c);
      __syncthreads();
      store_kv<T, DH>(Ks, Vt, kv);
      __syncthreads();
      if (c + 1 < tiles) load_tile(c + 1);
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

// ------------------------------------------------------------------------------------
// Block phase with a short prefix streamed in, bf16 (AttnParams::fused): a unit is 64 query
// rows -- (position, head) pairs of one branch and KV head -- that attend to every prefix
// key, read through the caller's strided view, and then to the branch's own block keys,
// gathered from the packed K/V rows through slot_row.  The tiles stream through the same
// four-stage direct-to-LDS ring as the 256-query prefix kernel (three tiles in flight,
// transposed V reads).  Eight waves, two per SIMD: the waves w and w + 4 hold the same 16
// query rows and take the first and the second 32 keys of every tile, each with its own
// online-softmax state, so each SIMD runs two independent MFMA/softmax chains (with one
// wave per SIMD the chain's latency set the time).  The two states of a row are merged
// through LDS at the end, and the result is stored as the slot's attention output, with
// no partials in HBM.
// ------------------------------------------------------------------------------------
#ifndef SPECFOLD_SLOT_BLOCKS
#define SPECFOLD_SLOT_BLOCKS 1
#endif
constexpr int kSlotBlocks = SPECFOLD_SLOT_BLOCKS;   // 16-row query blocks per wave
constexpr int kSlotQRows = 64;
constexpr int kSlotGroups = kSlotQRows / (16 * kSlotBlocks);   // row groups of a unit
constexpr int kSlotWaves = 2 * kSlotGroups;                     // a wave pair per group
static_assert(kSlotQRows == kAttnSlotQRows, "unit size of the per-slot pass");
static_assert(kSlotBlocks == 1 || kSlotBlocks == 2, "one or two query blocks per wave");

template <int DH>
__global__ void __launch_bounds__(kSlotWaves * 64, 1) attn_slot_tr_kernel(AttnParams p) {
  using Tt = TrTile<DH, kSlotWaves>;
  constexpr int QI = Tt::QI, LPI = Tt::LPI, KSQ = Tt::KSQ, NT = Tt::NT;
  constexpr int NBQ = kSlotBlocks, RG = kSlotGroups;
  constexpr int HALF = kKeys / 2;                  // keys per wave per tile
  __shared__ __attribute__((aligned(1024))) char K0[Tt::TILEB], K1[Tt::TILEB], K2[Tt::TILEB],
      K3[Tt::TILEB];
  __shared__ __attribute__((aligned(1024))) char V0[Tt::TILEB], V1[Tt::TILEB], V2[Tt::TILEB],
      V3[Tt::TILEB];
  // after a unit's last tile, stage K<rg*NBQ + b> holds the second-half state of block b of
  // row group rg
  static_assert((NT * 4 + 2) * 64 * 4 <= Tt::TILEB, "merge slot of a query block");
  static_assert(RG * NBQ == 4, "four merge slots");
  const int K = imin(*p.count, p.cap);
  if (K <= 0) return;
  const int g = p.n_q / p.n_kv;
  const int rows = p.B * g;                       // query rows per (branch, KV head)
  const int qtiles = ceil_div(rows, kSlotQRows);
  const int units = p.N * p.n_kv * qtiles;
  const int pch = p.P > 0 ? ceil_div(p.P, kKeys) : 0;
  const int n = pch + ceil_div(p.B, kKeys);       // key tiles per unit
  const int lane = threadIdx.x & 63, g4 = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = wave % RG, half = wave / RG;     // row group; first or second 32 keys
  const char* qkv = (const char*)p.qkv;
  const long ldq = p.ld_qkv * 2, st_tok = p.stride_tok * 2, st_head = p.stride_head * 2;
  auto row_of = [&](int slot) { return imin(imax(p.slot_row[slot], 0), K - 1); };
  auto mslot_of = [&](int b) {
    const int m = rg * NBQ + b;
    return (float*)(m == 0 ? K0 : m == 1 ? K1 : m == 2 ? K2 : K3);
  };

  // LDS byte offsets of this lane's fragments (as in the prefix kernel)
  int kofs[KSQ], vofs[NT];
#pragma unroll
  for (int ks = 0; ks < KSQ; ++ks)
    kofs[ks] = l16 * Tt::ROWB + (((4 * ks + g4) ^ tr_kswz<DH>(l16)) << 4);
  {
    const int vr = 4 * g4 + (l16 >> 2);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      vofs[nt] = vr * Tt::ROWB + (((2 * nt + ((l16 & 3) >> 1)) ^ tr_vswz<DH>(vr)) << 4) +
                 8 * (l16 & 1);
  }
  // loader geometry: load q of this wave fills LDS bytes (wave*QI + q)*1024 + 16*lane of a
  // stage: key row lr[q] of the tile, physical chunk pc, fetching the matching logical chunk
  int lr[QI];
  uint32_t lkc[QI], lvc[QI];
#pragma unroll
  for (int q = 0; q < QI; ++q) {
    const int byte = (wave * QI + q) * 1024 + 16 * lane;
    const int r = byte / Tt::ROWB, pc = (byte % Tt::ROWB) >> 4;
    lr[q] = r;
    lkc[q] = (uint32_t)((pc ^ tr_kswz<DH>(r)) << 4);
    lvc[q] = (uint32_t)((pc ^ tr_vswz<DH>(r)) << 4);
  }
  const int wq = wave * QI * 1024;                  // this wave's LDS slice of a stage
  const int hofs = half * HALF * Tt::ROWB;          // this wave's keys inside a stage

  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int qt = u % qtiles, rest = u / qtiles;
    const int kvh = rest % p.n_kv, nb = rest / p.n_kv;
    bool valid[NBQ];
    int qi[NBQ], qh[NBQ];
    uint4 qf[NBQ][KSQ];
#pragma unroll
    for (int b = 0; b < NBQ; ++b) {
      const int r = qt * kSlotQRows + (rg * NBQ + b) * 16 + l16;
      valid[b] = r < rows;
      const int rr = valid[b] ? r : rows - 1;
      qi[b] = rr / g;
      qh[b] = kvh * g + (rr - (rr / g) * g);
      const char* qp = qkv + (size_t)row_of(nb * p.B + qi[b]) * ldq + (size_t)qh[b] * DH * 2;
#pragma unroll
      for (int ks = 0; ks < KSQ; ++ks) qf[b][ks] = ld16(qp + (4 * ks + g4) * 16);
    }
    // packed rows of the first block tile's keys, read with the queries: looked up inside
    // the ring, the index loads would make the wave wait for every tile in flight
    int brow[QI];
#pragma unroll
    for (int q = 0; q < QI; ++q) brow[q] = row_of(nb * p.B + imin(lr[q], p.B - 1));
    AttnState st[NBQ];
    f32x4 o[NBQ][NT];
#pragma unroll
    for (int b = 0; b < NBQ; ++b) {
      st[b] = AttnState{-__builtin_inff(), 0.f};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o[b][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const char* kpre = (const char*)p.pk + (size_t)kvh * st_head;
    const char* vpre = (const char*)p.pv + (size_t)kvh * st_head;
    const char* kblk = qkv + ((size_t)p.n_q + kvh) * DH * 2;           // K heads of a row
    const char* vblk = qkv + ((size_t)p.n_q + p.n_kv + kvh) * DH * 2;  // V heads of a row
    // Every tile slot issues its loads, so the wait count stays a constant: slots past the
    // unit's last tile load packed row 0's line; rows past the prefix (or the block) of a
    // ragged tile reload its last row (finite values the softmax weights with 0).
    auto issue = [&](char* Kd, char* Vd, int c) {
      const uint32_t kl = lds_addr(Kd) + wq, vl = lds_addr(Vd) + wq;
      const char* ks[QI];
      const char* vs[QI];
      if (c >= n) {
#pragma unroll
        for (int q = 0; q < QI; ++q) ks[q] = kblk, vs[q] = vblk;
      } else if (c < pch) {
        const int key0 = c * kKeys;
#pragma unroll
        for (int q = 0; q < QI; ++q) {
          const long key = imin(key0 + lr[q], p.P - 1);
          ks[q] = kpre + key * st_tok + lkc[q];
          vs[q] = vpre + key * st_tok + lvc[q];
        }
      } else if (c == pch) {
#pragma unroll
        for (int q = 0; q < QI; ++q) {
          ks[q] = kblk + (size_t)brow[q] * ldq + lkc[q];
          vs[q] = vblk + (size_t)brow[q] * ldq + lvc[q];
        }
      } else {
        const int j0 = (c - pch) * kKeys;
#pragma unroll
        for (int q = 0; q < QI; ++q) {
          const size_t prow = (size_t)row_of(nb * p.B + imin(j0 + lr[q], p.B - 1));
          ks[q] = kblk + prow * ldq + lkc[q];
          vs[q] = vblk + prow * ldq + lvc[q];
        }
      }
#pragma unroll
      for (int q = 0; q < QI; ++q) {
        dma16(ks[q], kl + q * 1024);
        dma16(vs[q], vl + q * 1024);
      }
    };
    auto body = [&](const char* Kc, const char* Vc, char* Kn, char* Vn, int c) {
      if (c >= n) return;
      __builtin_amdgcn_s_waitcnt(tr_waitcnt_vm(2 * LPI));
      __builtin_amdgcn_s_barrier();
      const int nkeys = c < pch ? imin(kKeys, p.P - c * kKeys)
                                : imin(kKeys, p.B - (c - pch) * kKeys);
      const int nk = nkeys - half * HALF;           // this wave's live keys (wave-uniform)
      if (nk > 0)
        tr_attend<DH, NBQ, 2>(Kc + hofs, Vc + hofs, nk, qf, kofs, vofs, p.scale_log2, st, o);
      issue(Kn, Vn, c + 3);
    };
    // the previous unit's loads and LDS reads and this unit's query loads are done before
    // the ring is refilled
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(tr_waitcnt_vm_lgkm0(0));
    __builtin_amdgcn_s_barrier();
    issue(K0, V0, 0);
    issue(K1, V1, 1);
    issue(K2, V2, 2);
    for (int it = 0; it < n; it += kTrStages) {
      body(K0, V0, K3, V3, it);
      body(K1, V1, K0, V0, it + 1);
      body(K2, V2, K1, V1, it + 2);
      body(K3, V3, K2, V2, it + 3);
    }
    // merge the wave pair's states: every wave's ring loads (the unused trailing ones too)
    // have landed and every tile has been read before the second halves are written
    __builtin_amdgcn_s_waitcnt(tr_waitcnt_vm_lgkm0(0));
    __syncthreads();
    if (half) {
#pragma unroll
      for (int b = 0; b < NBQ; ++b) {
        float* ms = mslot_of(b);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int e = 0; e < 4; ++e) ms[(nt * 4 + e) * 64 + lane] = o[b][nt][e];
        ms[NT * 4 * 64 + lane] = st[b].m;
        ms[(NT * 4 + 1) * 64 + lane] = st[b].l;
      }
    }
    __builtin_amdgcn_s_waitcnt(tr_waitcnt_vm_lgkm0(0));
    __syncthreads();
#pragma unroll
    for (int b = 0; b < NBQ; ++b) {
      if (half || !valid[b]) continue;
      // the first half always holds a live key, so its maximum is finite
      const float* ms = mslot_of(b);
      const float m1 = ms[NT * 4 * 64 + lane], l1 = ms[(NT * 4 + 1) * 64 + lane];
      const float m = fmaxf(st[b].m, m1);
      const float a0 = fast_exp2(st[b].m - m), a1 = fast_exp2(m1 - m);   // m1 = -inf -> 0
      const float inv = 1.0f / (st[b].l * a0 + l1 * a1);
      bf16* op = (bf16*)p.out + (size_t)(nb * p.B + qi[b]) * p.ld_out + (size_t)qh[b] * DH;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = (o[b][nt][e] * a0 + ms[(nt * 4 + e) * 64 + lane] * a1) * inv;
        st_part4(op + nt * 16 + g4 * 4, v[0], v[1], v[2], v[3]);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(tr_waitcnt_vm_lgkm0(0));
}

// ------------------------------------------------------------------------------------
// Block phase after a separate prefix phase, bf16: a unit is 128 query rows -- (position,
// head) pairs of one branch and KV head, 16 per wave -- whose state starts from the prefix
// partials of each row's packed row (one plane when the split merge ran, else every split's)
// and then attends the branch's own block keys, gathered from the packed K/V rows through
// slot_row.  The block tiles arrive by direct-to-LDS loads into a two-stage ring (V read
// transposed, as in the prefix kernel); at the usual block sizes there is one tile.  The
// normalised result is the slot's attention output.
// ------------------------------------------------------------------------------------
#ifndef SPECFOLD_BLOCK_TR
#define SPECFOLD_BLOCK_TR 1
#endif
constexpr bool kAttnBlockTr = SPECFOLD_BLOCK_TR != 0;
constexpr int kBlkWaves = 8;
constexpr int kBlkQRows = kBlkWaves * 16;
static_assert(kBlkQRows == kAttnBlockQRows, "unit size of the block phase");

template <int DH>
__global__ void __launch_bounds__(kBlkWaves * 64, 1) attn_block_tr_kernel(AttnParams p) {
  using Tt = TrTile<DH, kBlkWaves>;
  constexpr int QI = Tt::QI, LPI = Tt::LPI, KSQ = Tt::KSQ, NT = Tt::NT;
  __shared__ __attribute__((aligned(1024))) char K0[Tt::TILEB], K1[Tt::TILEB];
  __shared__ __attribute__((aligned(1024))) char V0[Tt::TILEB], V1[Tt::TILEB];
  // the plan is loaded with the count (without a prefix there are no partials)
  const int plan_ns = p.plan[0], plan_merged = p.plan[1];
  const int K = imin(*p.count, p.cap);
  if (K <= 0) return;
  const int ns = p.P <= 0 ? 0 : (plan_merged ? 1 : plan_ns);
  const int g = p.n_q / p.n_kv;
  const int rows = p.B * g;
  const int qtiles = ceil_div(rows, kBlkQRows);
  const int units = p.N * p.n_kv * qtiles;
  const int n = ceil_div(p.B, kKeys);             // block tiles per unit
  const int lane = threadIdx.x & 63, g4 = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const char* qkv = (const char*)p.qkv;
  const long ldq = p.ld_qkv * 2;
  auto row_of = [&](int slot) { return imin(imax(p.slot_row[slot], 0), K - 1); };

  int kofs[KSQ], vofs[NT];
#pragma unroll
  for (int ks = 0; ks < KSQ; ++ks)
    kofs[ks] = l16 * Tt::ROWB + (((4 * ks + g4) ^ tr_kswz<DH>(l16)) << 4);
  {
    const int vr = 4 * g4 + (l16 >> 2);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      vofs[nt] = vr * Tt::ROWB + (((2 * nt + ((l16 & 3) >> 1)) ^ tr_vswz<DH>(vr)) << 4) +
                 8 * (l16 & 1);
  }
  int lr[QI];
  uint32_t lkc[QI], lvc[QI];
#pragma unroll
  for (int q = 0; q < QI; ++q) {
    const int byte = (wave * QI + q) * 1024 + 16 * lane;
    const int r = byte / Tt::ROWB, pc = (byte % Tt::ROWB) >> 4;
    lr[q] = r;
    lkc[q] = (uint32_t)((pc ^ tr_kswz<DH>(r)) << 4);
    lvc[q] = (uint32_t)((pc ^ tr_vswz<DH>(r)) << 4);
  }
  const int wq = wave * QI * 1024;

  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int qt = u % qtiles, rest = u / qtiles;
    const int kvh = rest % p.n_kv, nb = rest / p.n_kv;
    const int r = qt * kBlkQRows + wave * 16 + l16;
    const bool valid = r < rows;
    const int rr = valid ? r : rows - 1;
    const int i = rr / g, h = kvh * g + (rr - (rr / g) * g);
    const int k = row_of(nb * p.B + i);
    // packed rows of the first block tile's keys, with the queries and the partials
    int brow[QI];
#pragma unroll
    for (int q = 0; q < QI; ++q) brow[q] = row_of(nb * p.B + imin(lr[q], p.B - 1));
    uint4 qf[1][KSQ];
    {
      const char* qp = qkv + (size_t)k * ldq + (size_t)h * DH * 2;
#pragma unroll
      for (int ks = 0; ks < KSQ; ++ks) qf[0][ks] = ld16(qp + (4 * ks + g4) * 16);
    }
    const char* kblk = qkv + ((size_t)p.n_q + kvh) * DH * 2;
    const char* vblk = qkv + ((size_t)p.n_q + p.n_kv + kvh) * DH * 2;
    // Every tile slot issues its loads (past the last tile: packed row 0's line), so the
    // wait count stays a constant; rows past the block reload its last row.
    auto issue = [&](char* Kd, char* Vd, int c) {
      const uint32_t kl = lds_addr(Kd) + wq, vl = lds_addr(Vd) + wq;
      const char* ks[QI];
      const char* vs[QI];
      if (c >= n) {
#pragma unroll
        for (int q = 0; q < QI; ++q) ks[q] = kblk, vs[q] = vblk;
      } else if (c == 0) {
#pragma unroll
        for (int q = 0; q < QI; ++q) {
          ks[q] = kblk + (size_t)brow[q] * ldq + lkc[q];
          vs[q] = vblk + (size_t)brow[q] * ldq + lvc[q];
        }
      } else {
        const int j0 = c * kKeys;
#pragma unroll
        for (int q = 0; q < QI; ++q) {
          const size_t prow = (size_t)row_of(nb * p.B + imin(j0 + lr[q], p.B - 1));
          ks[q] = kblk + prow * ldq + lkc[q];
          vs[q] = vblk + prow * ldq + lvc[q];
        }
      }
#pragma unroll
      for (int q = 0; q < QI; ++q) {
        dma16(ks[q], kl + q * 1024);
        dma16(vs[q], vl + q * 1024);
      }
    };
    // the previous unit's loads and LDS reads and this unit's query and index loads are
    // done before the ring is refilled
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(tr_waitcnt_vm_lgkm0(0));
    __builtin_amdgcn_s_barrier();
    issue(K0, V0, 0);

    // the state starts from the prefix partials of packed row k (while the tile loads fly)
    AttnState st[1] = {{-__builtin_inff(), 0.f}};
    f32x4 o[1][NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[0][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < ns; s0 += 2) {
      float ls[2];
      float4 po[2][NT];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int sb = imin(s0 + b, ns - 1);
        const size_t prow = ((size_t)sb * K + k) * p.n_q + h;
        ls[b] = (s0 + b < ns) ? p.part_lse[prow] : -__builtin_inff();
        const bf16* pp = (const bf16*)p.part_o + prow * DH;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) po[b][nt] = ld_part4(pp + nt * 16 + g4 * 4);
      }
      float mb = st[0].m;
#pragma unroll
      for (int b = 0; b < 2; ++b) mb = fmaxf(mb, ls[b]);
      if (mb > -__builtin_inff()) {
        const float alpha = fast_exp2(st[0].m - mb);   // st.m = -inf -> 0
        st[0].l *= alpha;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) o[0][nt] *= alpha;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const float w = fast_exp2(ls[b] - mb);       // 0 for an empty or absent split
          st[0].l += w;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            o[0][nt][0] += w * po[b][nt].x;
            o[0][nt][1] += w * po[b][nt].y;
            o[0][nt][2] += w * po[b][nt].z;
            o[0][nt][3] += w * po[b][nt].w;
          }
        }
        st[0].m = mb;
      }
    }

    // tile c: landed (c + 1 may be in flight) and every wave past tile c - 1, whose stage
    // takes the loads of c + 1 after the tile is attended
    auto body = [&](const char* Kc, const char* Vc, char* Kn, char* Vn, int c) {
      if (c >= n) return;
      __builtin_amdgcn_s_waitcnt(tr_waitcnt_vm(0));
      __builtin_amdgcn_s_barrier();
      issue(Kn, Vn, c + 1);
      tr_attend<DH, 1>(Kc, Vc, imin(kKeys, p.B - c * kKeys), qf, kofs, vofs, p.scale_log2, st,
                       o);
    };
    for (int it = 0; it < n; it += 2) {
      body(K0, V0, K1, V1, it);
      body(K1, V1, K0, V0, it + 1);
    }
    if (valid) {
      const float inv = 1.0f / st[0].l;
      bf16* op = (bf16*)p.out + (size_t)(nb * p.B + i) * p.ld_out + (size_t)h * DH;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        st_part4(op + nt * 16 + g4 * 4, o[0][nt][0] * inv, o[0][nt][1] * inv,
                 o[0][nt][2] * inv, o[0][nt][3] * inv);
    }
  }
  __builtin_amdgcn_s_waitcnt(tr_waitcnt_vm_lgkm0(0));
}

size_t attn_partial_rows(int S, int g, int n_kv, int P, int dh, int elem_bytes) {
  size_t best = 0;
  for (int K = 1; K <= S; ++K) {
    const size_t v = (size_t)attn_splits(K, g, n_kv, P, dh, elem_bytes) * K;
    if (v > best) best = v;
  }
  return best;
}

// Whether the split merge can run for some packed count K <= cap (otherwise its launch is
// skipped).  The last shape asked about is remembered: a stack asks with the same one for
// every layer.
static bool merge_possible(int cap, int g, int n_kv, int P, int S, int dh, int eb) {
  thread_local int key[7] = {-1, -1, -1, -1, -1, -1, -1};
  thread_local bool val = false;
  const int k[7] = {cap, g, n_kv, P, S, dh, eb};
  bool same = true;
  for (int i = 0; i < 7; ++i) same = same && key[i] == k[i];
  if (same) return val;
  bool v = false;
  for (int K = 1; K <= cap && !v; ++K) v = attn_merge_on(K, g, n_kv, P, S, dh, eb);
  for (int i = 0; i < 7; ++i) key[i] = k[i];
  val = v;
  return v;
}

template <typename T>
hipError_t launch_attn_prefix(const AttnParams& p, int num_cu, hipStream_t st) {
  // no prefix, or a short one that the block phase streams itself
  if (p.P <= 0 || p.fused) return hipSuccess;
  const int mrows = ceil_div(p.cap * p.n_q, 4);
  const int mgrid = mrows < 4 * num_cu ? mrows : 4 * num_cu;   // grid-stride over rows
  const bool tr = attn_use_tr((int)sizeof(T), p.P);
  const bool merge = merge_possible(p.cap, p.n_q / p.n_kv, p.n_kv, p.P, p.S, p.dh, (int)sizeof(T));
  if (p.dh == 128) {
    if (tr) attn_prefix_tr_kernel<128><<<num_cu, kTrWaves * 64, 0, st>>>(p);
    else attn_prefix_kernel<T, 128><<<2 * num_cu, 256, 0, st>>>(p);
    if (merge) attn_merge_kernel<T, 128><<<mgrid, 256, 0, st>>>(p);
  } else if (p.dh == 64) {
    if (tr) attn_prefix_tr_kernel<64><<<num_cu, kTrWaves * 64, 0, st>>>(p);
    else attn_prefix_kernel<T, 64><<<2 * num_cu, 256, 0, st>>>(p);
    if (merge) attn_merge_kernel<T, 64><<<mgrid, 256, 0, st>>>(p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_attn_block(const AttnParams& p, int num_cu, hipStream_t st) {
  const int g = p.n_q / p.n_kv;
  if (sizeof(T) == 2 && p.fused) {
    // bf16 with a short prefix: one pass per slot over the prefix and the block
    const int units = p.N * p.n_kv * ceil_div(p.B * g, kSlotQRows);
    const int grid = units < num_cu ? units : num_cu;
    if (p.dh == 128) attn_slot_tr_kernel<128><<<grid, kSlotWaves * 64, 0, st>>>(p);
    else if (p.dh == 64) attn_slot_tr_kernel<64><<<grid, kSlotWaves * 64, 0, st>>>(p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (sizeof(T) == 2 && kAttnBlockTr) {
    // bf16 after a separate prefix phase (or none): 128-query units, direct-to-LDS tiles
    const int units = p.N * p.n_kv * ceil_div(p.B * g, kBlkQRows);
    const int grid = units < num_cu ? units : num_cu;
    if (p.dh == 128) attn_block_tr_kernel<128><<<grid, kBlkWaves * 64, 0, st>>>(p);
    else if (p.dh == 64) attn_block_tr_kernel<64><<<grid, kBlkWaves * 64, 0, st>>>(p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
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
