// Fused softmax + linear attention of the STILL prefill, with the shared normaliser.
// (Page labels [P1]..[P4]: the pages listed at the top of include/still.h.)
//
// One workgroup per (chunk c, batch b, KV head h, head split, query split). The
// workgroup packs up to four query heads of the group (GQA): every staged key/value tile
// serves all of them. A wave handles one query head of the head split for QW = 32
// consecutive queries (a query slice). Where two workgroups fit in a CU, each takes one of
// the chunk's two slices and the pair hides each other's barriers; where one fills the
// CU's LDS (head_dim 128, fp32), it takes both slices with twice the waves.
//
// Key sets for query i = 64c + r ([P1] paragraph before "STILL三大创新", sections
// "Chunk-Wise并行+延迟选择" and NP-Map; [P2] excerpt):
//   chunks <= c-2  selected rows (compact cache) -> softmax; the rest are folded in the
//                  inclusive prefix state (S, z) of chunk c-2 -> linear;
//   chunk c-1      p > r + 64 - w or selected -> softmax, the rest -> linear;
//   chunk c        p <= r: p > r - w -> softmax, the rest -> linear.
//
// Phase 1 (linear attention): N = phi(q) S + sum phi(q).phi(k_j) v_j over the linear keys
// of chunks c-1 and c, D = phi(q) z + sum phi(q).phi(k_j). The whole linear branch then
// enters the online softmax as one entry of log-weight log2(D) and value N / D, so the
// shared-normaliser output  (sum_SA e^a v + N) / (sum_SA e^a + D)  needs no offset and
// cannot overflow whatever the magnitudes.
// Phase 2 (softmax): the two window tiles (masked), then the compact tiles, 64 keys per
// tile, in a four-stage LDS pipeline whose copies run straight from memory into LDS. Every
// score is the exact fp32 sum of bf16 products of the stored q and k; the logit scale
// log2(e)/sqrt(D) and the running max enter in fp32, in the fma that feeds the exp (a key
// pre-multiplied by the scale and rounded to bf16 would carry a logit error growing with
// the logit, 2^-9 of it per element). The
// running max is refreshed only when a tile's max exceeds it by more than kLazy = 32 (log2
// units): P and the accumulators keep fp32's exponent range (bf16 has it too), so terms up
// to 2^32 stay exact in relative terms and every sum stays finite. Before the compact
// tiles the max is set once, from the bound |q| max|k| of their logits (or, where that bound
// is far above every score so far, from their exact largest logit), so the compact loop
// itself has no max pass.
//
// Every tile the fixed part needs (phi(K) and V of chunk c-1, K and V of the window, the
// prefix state) is copied into its own LDS region at the start, together with the first
// compact tile, so the workgroup waits for memory once before computing.
//
// Everything is computed transposed (S^T = K Q^T, O^T += V^T P^T): a query is a lane's
// column, so its statistics need only the 4-lane-group reduction, and P leaves the
// softmax in the register layout the PV product consumes. The row sums of P ride along
// in the PV product as one extra 16-row block whose A operand is all ones. V tiles arrive
// transposed and key-permuted from the prep kernel, phi(K) rows feature-permuted, so
// every LDS operand fragment is a single 16-byte read.
#include <type_traits>

#include "still_launch.hpp"
#include "still_layout.hpp"
#include "still_route.hpp"

namespace still {

// lazy running max: rescale only when a score exceeds the running max by more than this
// (log2 units)
constexpr float kLazy = 32.f;
// how far (log2 units) the running max may be raised above every score seen so far to a
// bound of the compact logits, before the exact largest compact logit is taken instead
constexpr float kRaise = 64.f;

template <typename T> __device__ __forceinline__ typename Tr<T>::frag ones_frag() {
  typename Tr<T>::frag x;
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = Tr<T>::from_f(1.0f);
  return x;
}

// Scores of one 64-key tile for one wave: s[kb][qb] = S^T block (keys kb*16.., queries
// qb*16..) = K Q^T, K rows from the Swz<T, D> tile lk.
template <typename T, int D, int QB>
__device__ __forceinline__ void qk_tile(const T* lk, const typename Tr<T>::frag (&qf)[QB][D / 32], f32x4 (&s)[4][QB]) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const typename Tr<T>::frag ka = Swz<T, D>::load8(lk, kb * 16 + r16, ks * 32 + grp * 8);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) Tr<T>::mma(s[kb][qb], ka, qf[qb][ks]);
    }
  }
}

// Per-lane key masks. A lane holds keys p = kb*16 + 4*grp + i (kb, i in 0..3) of a
// 64-key tile; its "key word" has bit kb*4 + i set for the keys it keeps.
//
// Keys p with lo <= p <= hi (any integers; empty if lo > hi).
__device__ __forceinline__ uint32_t range_word(int lo, int hi) {
  const int g4 = 4 * ((threadIdx.x & 63) >> 4);
  uint32_t w = 0;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int base = kb * 16 + g4;  // key of element (kb, i = 0)
    const int nh = min(max(hi - base + 1, 0), 4);
    const int nl = min(max(lo - base, 0), 4);
    w |= (((1u << nh) - 1u) & ~((1u << nl) - 1u)) << (4 * kb);
  }
  return w;
}
// Keys whose bit is set in a 64-bit tile mask (bit p <-> key p).
__device__ __forceinline__ uint32_t bits_word(uint64_t m) {
  const uint64_t x = m >> (4 * ((threadIdx.x & 63) >> 4));
  return static_cast<uint32_t>((x & 0xFull) | ((x >> 12) & 0xF0ull) | ((x >> 24) & 0xF00ull) | ((x >> 36) & 0xF000ull));
}

// scores of keys not set in the lane's key word (one per query block) -> -inf
template <int QB>
__device__ __forceinline__ void mask_tile(f32x4 (&s)[4][QB], const uint32_t (&kw)[QB]) {
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!(kw[qb] & (1u << (kb * 4 + i)))) s[kb][qb][i] = -kInf;
}

// Running-max update for a tile: the max is refreshed only when the tile's max exceeds it
// by more than kLazy (log2 units); the accumulators (row-sum block included) are rescaled
// then, which is rare after the first tiles.
template <int D, int QB>
__device__ __forceinline__ void sm_max(const f32x4 (&s)[4][QB], f32x4 (&o)[D / 16 + 1][QB], float (&m_run)[QB],
                                       float c1) {
  bool need_any = false;
  float alpha[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float tm = fmaxf(fmaxf(fmaxf(s[0][qb][0], s[0][qb][1]), fmaxf(s[0][qb][2], s[0][qb][3])),
                     fmaxf(fmaxf(s[1][qb][0], s[1][qb][1]), fmaxf(s[1][qb][2], s[1][qb][3])));
    tm = fmaxf(tm, fmaxf(fmaxf(fmaxf(s[2][qb][0], s[2][qb][1]), fmaxf(s[2][qb][2], s[2][qb][3])),
                         fmaxf(fmaxf(s[3][qb][0], s[3][qb][1]), fmaxf(s[3][qb][2], s[3][qb][3]))));
    tm = xor_max_groups(tm) * c1;
    const bool need = tm > m_run[qb] + kLazy;
    alpha[qb] = need ? (m_run[qb] == -kInf ? 0.f : __builtin_amdgcn_exp2f(m_run[qb] - tm)) : 1.f;
    m_run[qb] = need ? tm : m_run[qb];
    need_any |= need;
  }
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(need_any) != 0, 0)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int db = 0; db <= D / 16; ++db) o[db][qb] *= alpha[qb];
  }
}

// P = 2^(s*c1 - m) (bf16 for bf16 inputs), then O^T += V^T P^T in two 32-key halves
// (V^T rows from the Swz<T, 64> tile lv); the all-ones block accumulates the row sums.
template <typename T, int D, int QB>
__device__ __forceinline__ void sm_exp_pv(const f32x4 (&s)[4][QB], const T* lv, f32x4 (&o)[D / 16 + 1][QB],
                                          const float (&m_run)[QB], float c1) {
  using TT = Tr<T>;
  using frag = typename TT::frag;
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
  float mq[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) mq[qb] = m_run[qb] == -kInf ? 0.f : m_run[qb];
  frag one;
#pragma unroll
  for (int e = 0; e < 8; ++e) one[e] = TT::from_f(1.0f);
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) {
    frag pf[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pf[qb][e] = TT::from_f(__builtin_amdgcn_exp2f(s[2 * hs + e / 4][qb][e % 4] * c1 - mq[qb]));
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const frag va = Swz<T, 64>::load8(lv, db * 16 + r16, hs * 32 + grp * 8);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) TT::mma(o[db][qb], va, pf[qb]);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) TT::mma(o[D / 16][qb], one, pf[qb]);
  }
}

// x + the sum of the 8 probabilities of a fragment (bf16: four dot2 with (1, 1); fp32: adds)
template <typename F> __device__ __forceinline__ float row_sum_add(const F& p, float x) {
  if constexpr (sizeof(p[0]) == 2) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
    const bf16x2_t one2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
    for (int j = 0; j < 4; ++j) x = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{p[2 * j], p[2 * j + 1]}, one2, x, false);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) x += p[j];
  }
  return x;
}

// Scores of one 64-key tile for HV query groups of a wave: every K fragment read from LDS
// feeds the products of all of them (qk_tile with HV groups).
template <typename T, int D, int QB, int HV>
__device__ __forceinline__ void qk_tile_hv(const T* lk, const typename Tr<T>::frag (&qf)[HV][QB][D / 32],
                                           f32x4 (&s)[HV][4][QB]) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int hv = 0; hv < HV; ++hv)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[hv][kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const typename Tr<T>::frag ka = Swz<T, D>::load8(lk, kb * 16 + r16, ks * 32 + grp * 8);
#pragma unroll
      for (int hv = 0; hv < HV; ++hv)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) Tr<T>::mma(s[hv][kb][qb], ka, qf[hv][qb][ks]);
    }
  }
}

// sm_exp_pv for HV query groups: every V^T fragment read from LDS feeds all of them. The
// row sums are not a ones block of the product here but per-lane partials lp (each lane
// adds the probabilities it holds, already rounded as the product uses them, by bf16 dot2;
// the four lane groups are summed once at the end), which frees that block's registers.
template <typename T, int D, int QB, int HV, int NO>
__device__ __forceinline__ void sm_exp_pv_hv(const f32x4 (&s)[HV][4][QB], const T* lv, f32x4 (&o)[HV][NO][QB],
                                             float (&lp)[HV][QB], const float (&m_run)[HV][QB], float c1) {
  using TT = Tr<T>;
  using frag = typename TT::frag;
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
  float mq[HV][QB];
#pragma unroll
  for (int hv = 0; hv < HV; ++hv)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mq[hv][qb] = m_run[hv][qb] == -kInf ? 0.f : m_run[hv][qb];
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) {
    frag pf[HV][QB];
#pragma unroll
    for (int hv = 0; hv < HV; ++hv)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pf[hv][qb][e] = TT::from_f(__builtin_amdgcn_exp2f(s[hv][2 * hs + e / 4][qb][e % 4] * c1 - mq[hv][qb]));
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const frag va = Swz<T, 64>::load8(lv, db * 16 + r16, hs * 32 + grp * 8);
#pragma unroll
      for (int hv = 0; hv < HV; ++hv)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) TT::mma(o[hv][db][qb], va, pf[hv][qb]);
    }
#pragma unroll
    for (int hv = 0; hv < HV; ++hv)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) lp[hv][qb] = row_sum_add(pf[hv][qb], lp[hv][qb]);
  }
}

// The largest compact logit of each query of a wave (log2 units: the fp32 score times c1),
// over the n_comp compact keys: K rows (D elements each, rsrc kr) straight from memory, no
// LDS and no barrier, so the other waves of the workgroup are not held up.
template <typename T, int D, int QB, int HV>
__device__ __forceinline__ void compact_max(__amdgpu_buffer_rsrc_t kr, int n_comp,
                                            const typename Tr<T>::frag (&qf)[HV][QB][D / 32], float (&mx)[HV][QB],
                                            float c1) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
  float m[HV][QB];
#pragma unroll
  for (int hv = 0; hv < HV; ++hv)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) m[hv][qb] = -kInf;
  for (int k0 = 0; k0 < n_comp; k0 += 16) {  // 16-key blocks: lane r16 loads key k0 + r16
    typename Tr<T>::frag ka[D / 32];
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      ka[ks] = Tr<T>::bload8(kr, ((k0 + r16) * D + ks * 32 + grp * 8) * static_cast<int>(sizeof(T)), 0);
#pragma unroll
    for (int hv = 0; hv < HV; ++hv)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        f32x4 sv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) Tr<T>::mma(sv, ka[ks], qf[hv][qb][ks]);
#pragma unroll
        for (int i = 0; i < 4; ++i)  // element i: key k0 + 4 grp + i
          if (k0 + 4 * grp + i < n_comp) m[hv][qb] = fmaxf(m[hv][qb], sv[i]);
      }
  }
#pragma unroll
  for (int hv = 0; hv < HV; ++hv)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mx[hv][qb] = xor_max_groups(m[hv][qb]) * c1;
}

// sm_exp_pv_hv with the row sums riding along in the product: an all-ones A block adds every
// probability of a query's column into every element of o[hv][D / 16][qb].
template <typename T, int D, int QB, int HV>
__device__ __forceinline__ void sm_exp_pv_ones_hv(const f32x4 (&s)[HV][4][QB], const T* lv,
                                                  f32x4 (&o)[HV][D / 16 + 1][QB], const float (&m_run)[HV][QB],
                                                  float c1) {
  using TT = Tr<T>;
  using frag = typename TT::frag;
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
  const frag one = ones_frag<T>();
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) {
    frag pf[HV][QB];
#pragma unroll
    for (int hv = 0; hv < HV; ++hv)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pf[hv][qb][e] = TT::from_f(__builtin_amdgcn_exp2f(s[hv][2 * hs + e / 4][qb][e % 4] * c1 - m_run[hv][qb]));
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const frag va = Swz<T, 64>::load8(lv, db * 16 + r16, hs * 32 + grp * 8);
#pragma unroll
      for (int hv = 0; hv < HV; ++hv)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) TT::mma(o[hv][db][qb], va, pf[hv][qb]);
    }
#pragma unroll
    for (int hv = 0; hv < HV; ++hv)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) TT::mma(o[hv][D / 16][qb], one, pf[hv][qb]);
  }
}

// Window tiles when the window equals the chunk (w = 64), for a wave whose queries start at
// QOFF within the chunk. Lane (r16, grp) holds keys kb*16 + 4 grp + i of query
// QOFF + qb*16 + r16, so a (key block, query block) pair is of one of three kinds, known at
// compile time: every key position below the query's (0), the diagonal (1: below where
// 4 grp + i < r16, equal where 4 grp + i = r16) or every key position above (2).
template <int QOFF>
__device__ constexpr int win_kind(int kb, int qb) {
  return 16 * (kb - qb) - QOFF < 0 ? 0 : (16 * (kb - qb) - QOFF == 0 ? 1 : 2);
}

// Chunk c: softmax keys p <= r (kinds 0 and 1; kind-2 blocks take no part).
// Chunk c-1 (if any): softmax keys p > r or selected, linear keys the rest. One P holds both:
// 2^(a c1 - m) for softmax keys, phi(q).phi(k) 2^-m for linear keys (the shared normaliser in
// the running frame), and the row-sum block adds both denominators. The largest linear
// weight is kept within the lazy-max bound too (2^-m times it <= 2^kLazy): only extreme inputs
// (every softmax score of a query far below its linear weights) reach that rescale.
template <typename T, int D, int DF, int QB, int QOFF>
__device__ __forceinline__ void window_fast(const T* lkc, const T* lvc, const T* lkp, const T* lfp, const T* lvp,
                                            bool has_prev, uint64_t selprev,
                                            const typename Tr<T>::frag (&qf)[QB][D / 32],
                                            const typename Tr<T>::frag (&pq)[QB][DF / 32],
                                            f32x4 (&o)[D / 16 + 1][QB], float (&m_run)[QB], float c1) {
  using TT = Tr<T>;
  using frag = typename TT::frag;
  constexpr int NB = D / 16;
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
  bool dmask[4];  // key position <= query position, on a diagonal block
#pragma unroll
  for (int i = 0; i < 4; ++i) dmask[i] = 4 * grp + i <= r16;
  frag one;
#pragma unroll
  for (int e = 0; e < 8; ++e) one[e] = TT::from_f(1.0f);

  // ---- chunk c
  {
    f32x4 s[4][QB];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      bool any = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) any |= win_kind<QOFF>(kb, qb) != 2;
      if (!any) continue;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const frag ka = Swz<T, D>::load8(lkc, kb * 16 + r16, ks * 32 + grp * 8);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          if (win_kind<QOFF>(kb, qb) != 2) TT::mma(s[kb][qb], ka, qf[qb][ks]);
      }
    }
    bool need_any = false;
    float alpha[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float tm = -kInf;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int kind = win_kind<QOFF>(kb, qb);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (kind == 1 && !dmask[i]) s[kb][qb][i] = -kInf;
          if (kind != 2) tm = fmaxf(tm, s[kb][qb][i]);
        }
      }
      tm = xor_max_groups(tm) * c1;  // finite: every query sees its own key
      const bool need = tm > m_run[qb] + kLazy;
      alpha[qb] = need ? (m_run[qb] == -kInf ? 0.f : __builtin_amdgcn_exp2f(m_run[qb] - tm)) : 1.f;
      m_run[qb] = need ? tm : m_run[qb];
      need_any |= need;
    }
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(need_any) != 0, 0)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int db = 0; db <= NB; ++db) o[db][qb] *= alpha[qb];
    }
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      bool live[QB], any = false;
      frag pf[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        live[qb] = win_kind<QOFF>(2 * hs, qb) != 2 || win_kind<QOFF>(2 * hs + 1, qb) != 2;
        any |= live[qb];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int kb = 2 * hs + e / 4;
          pf[qb][e] = win_kind<QOFF>(kb, qb) == 2
                          ? TT::from_f(0.f)
                          : TT::from_f(__builtin_amdgcn_exp2f(s[kb][qb][e % 4] * c1 - m_run[qb]));
        }
      }
      if (!any) continue;
#pragma unroll
      for (int db = 0; db < NB; ++db) {
        const frag va = Swz<T, 64>::load8(lvc, db * 16 + r16, hs * 32 + grp * 8);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          if (live[qb]) TT::mma(o[db][qb], va, pf[qb]);
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        if (live[qb]) TT::mma(o[NB][qb], one, pf[qb]);
    }
  }

  // ---- chunk c-1
  if (!has_prev) return;
  const uint32_t selw = bits_word(selprev);
  f32x4 s[4][QB], ls[4][QB];
  qk_tile<T, D, QB>(lkp, qf, s);  // every block: selected keys can be anywhere
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    bool any = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) any |= win_kind<QOFF>(kb, qb) != 2;
    if (!any) continue;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) ls[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int fs = 0; fs < DF / 32; ++fs) {
      const frag fa = Swz<T, DF>::load8(lfp, kb * 16 + r16, fs * 32 + grp * 8);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        if (win_kind<QOFF>(kb, qb) != 2) TT::mma(ls[kb][qb], fa, pq[qb][fs]);
    }
  }
  float lmax[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) lmax[qb] = 0.f;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool sel = (selw >> (kb * 4 + i)) & 1u;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int kind = win_kind<QOFF>(kb, qb);
        if (kind == 2) continue;  // all softmax keys
        const bool sa = sel || (kind == 1 && !dmask[i]);
        s[kb][qb][i] = sa ? s[kb][qb][i] : -kInf;
        ls[kb][qb][i] = sa ? 0.f : ls[kb][qb][i];
        lmax[qb] = fmaxf(lmax[qb], ls[kb][qb][i]);
      }
    }
  sm_max<D, QB>(s, o, m_run, c1);
  bool lfar = false;
  float lm[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    lm[qb] = xor_max_groups(lmax[qb]);
    lfar |= lm[qb] > __builtin_amdgcn_exp2f(m_run[qb] + kLazy);
  }
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(lfar) != 0, 0)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float ml = __log2f(lm[qb]);
      if (ml > m_run[qb] + kLazy) {
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - ml);
#pragma unroll
        for (int db = 0; db <= NB; ++db) o[db][qb] *= alpha;
        m_run[qb] = ml;
      }
    }
  }
  float sc2[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) sc2[qb] = __builtin_amdgcn_exp2f(-m_run[qb]);
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) {
    frag pf[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kb = 2 * hs + e / 4;
        const float ev = __builtin_amdgcn_exp2f(s[kb][qb][e % 4] * c1 - m_run[qb]);
        pf[qb][e] = TT::from_f(win_kind<QOFF>(kb, qb) == 2 ? ev : ls[kb][qb][e % 4] * sc2[qb] + ev);
      }
#pragma unroll
    for (int db = 0; db < NB; ++db) {
      const frag va = Swz<T, 64>::load8(lvp, db * 16 + r16, hs * 32 + grp * 8);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) TT::mma(o[db][qb], va, pf[qb]);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) TT::mma(o[NB][qb], one, pf[qb]);
  }
}

// One band chunk c-l (l >= 2, windows longer than a chunk) for 16-query blocks starting at
// qoff: key p of the chunk is in query r's window when p > r + lim (lim = 64 l - w); it is a
// softmax key when in the window or selected (bit p of sel), a linear key otherwise. As for
// chunk c-1 in window_fast, one P carries both kinds: 2^(a c1 - m) for softmax keys and
// phi(q).phi(k) 2^-m for linear keys, with the row-sum block adding both denominators. The
// masks are runtime values here. lk, lf, lv: K, phi(K) and V^T tiles of the chunk.
template <typename T, int D, int DF, int QB>
__device__ __forceinline__ void band_tile(const T* lk, const T* lf, const T* lv, int qoff, int lim, uint64_t sel,
                                          const typename Tr<T>::frag (&qf)[QB][D / 32],
                                          const typename Tr<T>::frag (&pq)[QB][DF / 32],
                                          f32x4 (&o)[D / 16 + 1][QB], float (&m_run)[QB], float c1) {
  using TT = Tr<T>;
  using frag = typename TT::frag;
  constexpr int NB = D / 16;
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
  f32x4 s[4][QB], ls[4][QB];
  qk_tile<T, D, QB>(lk, qf, s);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) ls[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int fs = 0; fs < DF / 32; ++fs) {
      const frag fa = Swz<T, DF>::load8(lf, kb * 16 + r16, fs * 32 + grp * 8);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) TT::mma(ls[kb][qb], fa, pq[qb][fs]);
    }
  }
  const uint32_t selw = bits_word(sel);
  float lmax[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const uint32_t kw = range_word(qoff + qb * 16 + r16 + lim + 1, 63) | selw;  // softmax keys
    lmax[qb] = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool sa = (kw >> (kb * 4 + i)) & 1u;
        s[kb][qb][i] = sa ? s[kb][qb][i] : -kInf;
        ls[kb][qb][i] = sa ? 0.f : ls[kb][qb][i];
        lmax[qb] = fmaxf(lmax[qb], ls[kb][qb][i]);
      }
  }
  sm_max<D, QB>(s, o, m_run, c1);
  bool lfar = false;
  float lm[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    lm[qb] = xor_max_groups(lmax[qb]);
    lfar |= lm[qb] > __builtin_amdgcn_exp2f(m_run[qb] + kLazy);
  }
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(lfar) != 0, 0)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float ml = __log2f(lm[qb]);
      if (ml > m_run[qb] + kLazy) {
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - ml);
#pragma unroll
        for (int db = 0; db <= NB; ++db) o[db][qb] *= alpha;
        m_run[qb] = ml;
      }
    }
  }
  float sc2[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) sc2[qb] = __builtin_amdgcn_exp2f(-m_run[qb]);
  frag one;
#pragma unroll
  for (int e = 0; e < 8; ++e) one[e] = TT::from_f(1.0f);
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) {
    frag pf[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kb = 2 * hs + e / 4;
        pf[qb][e] = TT::from_f(ls[kb][qb][e % 4] * sc2[qb] + __builtin_amdgcn_exp2f(s[kb][qb][e % 4] * c1 - m_run[qb]));
      }
#pragma unroll
    for (int db = 0; db < NB; ++db) {
      const frag va = Swz<T, 64>::load8(lv, db * 16 + r16, hs * 32 + grp * 8);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) TT::mma(o[db][qb], va, pf[qb]);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) TT::mma(o[NB][qb], one, pf[qb]);
  }
}

template <typename T, int D, int DF, int NH>
struct AttnCfg {
  static constexpr int QW = 32;                // queries per wave (one query slice)
  static constexpr int QB = QW / 16;           // 16-query blocks per wave
  static constexpr int KT = 64 * D, FT = 64 * DF, VT = D * 64;  // elements of a K, phi(K), V^T tile
  static constexpr int STAGE = KT + VT;        // one compact tile (K then V^T)
  // Sequential plan: the linear-attention tiles first, the window's K tiles then over the
  // phi(K) regions, W_h and the state read from memory, and the compact tiles in two stages
  // over the same regions. Taken where the usual plan (every fixed tile, the prefix state
  // and a compact stage resident at once) would pass the CU's 160 KiB (fp32 at head_dim
  // 128: six 32 KiB tiles and a 64 KiB state), and for bf16 at head_dim 128, where the usual
  // plan fills a CU with one workgroup (160 KiB) and this one lets two share it (64 KiB
  // each): their waits then overlap (Llama-3.1-8B-shaped layer: 7% less time at 8 x 4K
  // tokens, 22% less at 64K, for the shorter compact pipeline).
  static constexpr int ST_FULL = D * DF;
  static constexpr bool SEQ = (2 * FT + 2 * VT + 2 * KT + ST_FULL + STAGE) * static_cast<int>(sizeof(T)) > 160 * 1024 ||
                              (sizeof(T) == 2 && D == 128);
  // the prefix state (S^T [D][DF] in the layer's dtype) goes through LDS where it fits
  // beside the tiles: at D = d_f = 64 (two workgroups per CU) and at D = 128 (one, with
  // both query slices: 8 waves read one copy instead of 8)
  static constexpr bool STATE_LDS = !SEQ && ((D == 64 && DF == 64) || D == 128);
  static constexpr int ST = STATE_LDS ? D * DF : 0;
  // LDS regions of the fixed part (element offsets); compact stages 1 and 2 reuse them. In
  // the sequential plan the V^T tiles come first and K of chunks c and c-1 go over the
  // phi(K) regions once phase 1 is done with them (and past them where K is the wider).
  static constexpr int R_PHIP = SEQ ? 2 * VT : 0, R_PHIC = R_PHIP + FT;
  static constexpr int R_VP = SEQ ? 0 : 2 * FT, R_VC = R_VP + VT;
  static constexpr int R_KC = SEQ ? 2 * VT : 2 * FT + 2 * VT, R_KP = R_KC + KT;
  static constexpr int R_ST = SEQ ? 2 * FT + 2 * VT : R_KP + KT;
  // compact pipeline: 4 stages (2 in the sequential plan); stage 0 after the fixed regions,
  // stages 1..3 over them
  static constexpr int NSTAGE = SEQ ? 2 : 4;
  static constexpr int R_P0 = SEQ ? 0 : (R_ST + ST > 3 * STAGE ? R_ST + ST : 3 * STAGE);
  static constexpr int SEQ_FIXED = 2 * VT + (FT > KT ? 2 * FT : 2 * KT);
  static constexpr int LDS_ELEMS = SEQ ? (SEQ_FIXED > 2 * STAGE ? SEQ_FIXED : 2 * STAGE) : R_P0 + STAGE;
  static constexpr int LDS_BYTES = LDS_ELEMS * static_cast<int>(sizeof(T));
  // band chunks c-2 .. c-BL (windows longer than a chunk) staged one at a time once the
  // fixed part is done with its regions, before any compact tile but tile 0 is issued
  static constexpr int R_BV = 0, R_BK = VT, R_BF = VT + KT;
  static_assert(VT + KT + FT <= (SEQ ? LDS_ELEMS : R_ST), "band tiles stay inside the fixed regions");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS plan must fit a CU");
  static __device__ __forceinline__ int stage_off(int s) {
    if constexpr (SEQ) return s * STAGE;
    return s == 0 ? R_P0 : (s - 1) * STAGE;
  }
  // Query slices per workgroup. Where two workgroups fit in a CU's LDS (two 80 KiB
  // halves) each takes one slice, and the pair hides each other's waits. Where only one
  // fits (head_dim 128, or fp32) it takes both slices with twice the waves, so every SIMD
  // still runs two waves and every staged tile serves the whole chunk.
  // A workgroup of one query head (each query head selecting for itself, or one query head
  // per KV head) takes both slices too: the LDS per workgroup is the same, the waves double.
  static constexpr int QS = (LDS_BYTES > 80 * 1024 || NH == 1) ? 2 : 1;
  // Query halves per wave. At head_dim 64, where two workgroups share a CU, a wave takes
  // both 32-query halves of the chunk: every compact K and V^T fragment it reads from LDS
  // then feeds twice the MFMAs, and the step's fixed costs (copy issue and wait, barrier,
  // scalar control, LDS latency) are spread over twice the work.
  static constexpr int HV = (!SEQ && QS == 1 && D == 64) ? 2 : 1;
  static constexpr int QSPLIT = 64 / QW / QS / HV;  // workgroups per chunk
  static constexpr int NWAVE = NH * QS;        // wave w: head slot w % NH, query slice w / NH
  static constexpr int NTHR = 64 * NWAVE;
  // buffer->LDS instructions each wave issues per compact tile (1 KiB each)
  static constexpr int KINS = KT * static_cast<int>(sizeof(T)) / 1024, VINS = VT * static_cast<int>(sizeof(T)) / 1024;
  static_assert(KINS % NWAVE == 0 && VINS % NWAVE == 0, "tile copies must split evenly over the waves");
  static constexpr int NL = (KINS + VINS) / NWAVE;
};

// s_waitcnt immediate (gfx9 encoding) that waits for vector memory only, until at most n
// operations of this wave are outstanding (LDS and scalar counters untouched)
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Workgroup barrier with compiler-only fences around it: the hardware waits are the
// caller's (s_waitcnt before it), and no LDS access moves across it.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

template <typename T> __device__ __forceinline__ typename Tr<T>::frag frag_of(const f32x8& x) {
  typename Tr<T>::frag y;
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = Tr<T>::from_f(x[e]);
  return y;
}

// BAND: windows longer than a chunk (band chunks c-2 .. c-BL); a separate instantiation, so the
// kernels for windows up to a chunk keep their register plan
template <typename T, int D, int DF, int NH, bool BAND>
__global__ __launch_bounds__((AttnCfg<T, D, DF, NH>::NTHR), (3 - AttnCfg<T, D, DF, NH>::QS)) void attn_kernel(AttnArgs a) {
  using C = AttnCfg<T, D, DF, NH>;
  constexpr int QB = C::QB, QW = C::QW, NW = C::NWAVE;
  using SK = Swz<T, D>;    // K tile: 64 keys x D
  using SF = Swz<T, DF>;   // phi(K) tile: 64 keys x DF
  using SV = Swz<T, 64>;   // V^T tile: D rows x 64 keys
  constexpr int NB = D / 16;  // output blocks; block NB holds the row sums
  using TT = Tr<T>;
  using frag = typename TT::frag;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  T* L = reinterpret_cast<T*>(lds_raw);

  const Dims& d = a.d;
  const T* q = static_cast<const T*>(a.q);
  const T* kk = static_cast<const T*>(a.k);
  const T* w = static_cast<const T*>(a.w);
  const T* ksel = static_cast<const T*>(a.ksel);
  const T* vselT = static_cast<const T*>(a.vselT);
  const T* vT = static_cast<const T*>(a.vT);
  const T* phik = static_cast<const T*>(a.phik);

  // workgroup order: heaviest chunks first; within a chunk, consecutive workgroups take
  // consecutive (b, h, head split) so that, with 8 XCDs dispatched round-robin, one
  // XCD's L2 serves a fixed set of KV heads
  const int BHG = d.B * d.Hr * a.gsplit;
  const int P = BHG * C::QSPLIT;
  const int c = d.nC - 1 - static_cast<int>(blockIdx.x) / P;
  const int pi = static_cast<int>(blockIdx.x) % P;
  const int bhg = pi % BHG, qsb = pi / BHG;  // block of C::QS query slices
  const int gs = bhg % a.gsplit, bh = bhg / a.gsplit;
  // bh: the (b, routing head) record (compact rows, state, selection); bkv: the KV head's
  // (keys, values, phi(K), V^T tiles)
  const int b = bh / d.Hr, rh = bh % d.Hr, h = rh * d.Gr / d.G;
  const long long bkv = static_cast<long long>(b) * d.Hkv + h;
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: lets addresses stay scalar
  const int g = gs * NH + wave % NH;
  constexpr int HV = C::HV;
  const int qoff0 = (qsb * C::QS + wave / NH) * QW * HV;  // first query of this wave within the chunk
  const bool head_ok = g < d.Gr;
  const int hq = rh * d.Gr + (head_ok ? g : d.Gr - 1);
  const long long T_ = d.T;
  const long long t0 = static_cast<long long>(c) * kChunk;
  const int nvalid = static_cast<int>(T_ - t0 < kChunk ? T_ - t0 : kChunk);
  const float c1 = kLog2e / sqrtf(static_cast<float>(D));
  const int win = d.window;
  const bool has_prev = c >= 1;
  const bool la_cur = win < kChunk;  // chunk c holds linear keys (p <= r - w)
  // chunks c-BL .. c-1 are handled with per-query masks; the compact rows and the prefix
  // state cover chunks <= c-BL-1
  const int BL = BAND ? band_chunks(win) : 1;
  const int n_comp = c >= BL + 1 ? (c - BL) * d.topk : 0;  // compact rows of chunks <= c-BL-1
  const int nt_comp = (n_comp + 63) / 64;
  const T* kb_ptr = ksel + static_cast<long long>(bh) * a.ntiles_sel * 64 * D;
  const T* vb_ptr = vselT + static_cast<long long>(bh) * a.ntiles_sel * D * 64;
  // compact tile t -> LDS stage (asynchronous); K rows [64][D] and V^T rows [D][64] of a
  // tile are contiguous, so one resource per buffer covers the nt_comp tiles this chunk
  // reads (bounded by the sequence's own compact rows, so the 32-bit range holds whatever
  // the capacity of a decode cache the rows are written into)
  DmaTile<T, D, 64, NW> dk;
  DmaTile<T, 64, D, NW> dv;
  dk.init(D);
  dv.init(64);
  const auto krs = make_rsrc(kb_ptr, static_cast<uint32_t>(nt_comp) * C::KT * static_cast<int>(sizeof(T)));
  const auto vrs = make_rsrc(vb_ptr, static_cast<uint32_t>(nt_comp) * C::VT * static_cast<int>(sizeof(T)));
  auto issue = [&](int t, int stage) {
    T* st = L + C::stage_off(stage);
    dk.issue(st, krs, t * C::KT * static_cast<int>(sizeof(T)));
    dv.issue(st + C::KT, vrs, t * C::VT * static_cast<int>(sizeof(T)));
  };

  // ---- register operands, issued ahead of the tile copies. Vector loads complete in
  //      issue order, and every load up to phi(q) is unconditional (a range-checked
  //      buffer load reads zeros where a condition would skip it), so the number issued
  //      after the queries and W_h is the same on every path and phi(q) waits for those
  //      alone while the copies are in flight ---------------------------------------------
  // queries: B-operand fragments (SK over d); rows past the sequence end read as zeros
  frag qf[HV][QB][D / 32];  // [query half][16-query block][k slice]
#pragma unroll
  for (int hv = 0; hv < HV; ++hv) {
    const long long q0 = t0 + qoff0 + hv * QW;  // first query row of this half
    const int qrow = d.Hq * D;                   // elements from one position to the next
    const long long nq = T_ - q0 < QW ? T_ - q0 : QW;
    const auto qrs = make_rsrc(q + ((b * T_ + (nq > 0 ? q0 : 0)) * d.Hq + hq) * D,
                               nq > 0 ? static_cast<uint32_t>(((nq - 1) * qrow + D) * static_cast<int>(sizeof(T))) : 0u);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        qf[hv][qb][ks] = TT::bload8(qrs, ((qb * 16 + r16) * qrow + ks * 32 + grp * 8) * static_cast<int>(sizeof(T)), 0);
  }
  // W_h rows fb*16 + r16 (A operand of phi(q)): held in registers where they fit, else
  // copied once into compact stage 0 (free until the first compact tile) for all waves
  const T* Wh = w + static_cast<long long>(h) * DF * D;
  constexpr bool W_EARLY = D == 64 && DF == 64 && !C::SEQ;
  constexpr bool W_GLOBAL = C::SEQ;  // W_h fragments straight from memory (no LDS room)
  frag wq[W_EARLY ? DF / 16 : 1][D / 32];
  if constexpr (W_EARLY) {
#pragma unroll
    for (int fb = 0; fb < DF / 16; ++fb)
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) wq[fb][ks] = TT::load8(Wh + (fb * 16 + r16) * D + ks * 32 + grp * 8);
  }
  // z of the prefix state of chunks <= c-BL-1 (8 consecutive permuted features per lane
  // group): the A operand of the denominator, the same in every row
  const bool has_state = c >= BL + 1;
  const T* Sg = static_cast<const T*>(a.states) + (static_cast<long long>(bh) * d.nC + (has_state ? c - BL - 1 : 0)) * d.R;
  frag zf[DF / 32];
  {
    const auto zrs = make_rsrc(Sg + DF * D, has_state ? DF * static_cast<uint32_t>(sizeof(T)) : 0u);
#pragma unroll
    for (int fs = 0; fs < DF / 32; ++fs) zf[fs] = TT::bload8(zrs, (fs * 32 + grp * 8) * static_cast<int>(sizeof(T)), 0);
  }
  // the selection of chunk c-1 (0 if there is none); read out after the wait below
  const auto selv = __builtin_amdgcn_raw_buffer_load_b64(
      make_rsrc(a.selmask + static_cast<long long>(bh) * d.nC + (has_prev ? c - 1 : 0), has_prev ? 8u : 0u), 0, 0, 0);

  // ---- 0. every copy the fixed part needs, plus compact tile 0 (a copy that is not
  //      needed has no valid rows: it reads nothing and zero-fills its region) ----------
  {
    const int kvs = d.Hkv * D;  // row stride of k
    const long long tp = has_prev ? t0 - kChunk : t0;  // chunk c-1 (c itself if c = 0)
    const int cp = has_prev ? c - 1 : c;
    const T* kc = kk + ((b * T_ + t0) * d.Hkv + h) * D;
    const T* kp = kk + ((b * T_ + tp) * d.Hkv + h) * D;
    dma_tile<T, DF, 64, NW>(L + C::R_PHIP, phik + (bkv * T_ + tp) * DF, DF, has_prev ? 64 : 0);
    dma_tile<T, 64, D, NW>(L + C::R_VP, vT + (bkv * d.nC + cp) * D * 64, 64, has_prev ? D : 0);
    if constexpr (!C::SEQ) dma_tile<T, D, 64, NW>(L + C::R_KP, kp, kvs, has_prev && win >= 1 ? 64 : 0);
    dma_tile<T, DF, 64, NW>(L + C::R_PHIC, phik + (bkv * T_ + t0) * DF, DF, la_cur ? nvalid : 0);
    dma_tile<T, 64, D, NW>(L + C::R_VC, vT + (bkv * d.nC + c) * D * 64, 64, D);
    if constexpr (!C::SEQ) dma_tile<T, D, 64, NW>(L + C::R_KC, kc, kvs, win >= 1 ? nvalid : 0);
    if constexpr (C::STATE_LDS)
      dma_tile<T, DF, D, NW>(L + C::R_ST, Sg, DF, has_state ? D : 0);
    if constexpr (C::SEQ) {
      // the window's K tiles come after phase 1, over the phi(K) regions
    } else if constexpr (W_EARLY) {
      dk.issue(L + C::stage_off(0), make_rsrc(kb_ptr, nt_comp > 0 ? C::KT * static_cast<int>(sizeof(T)) : 0u), 0);
      dv.issue(L + C::stage_off(0) + C::KT, make_rsrc(vb_ptr, nt_comp > 0 ? C::VT * static_cast<int>(sizeof(T)) : 0u), 0);
    } else {
      static_assert(DF * D <= C::STAGE, "W_h must fit in one compact stage");
      dma_tile<T, D, DF, NW>(L + C::stage_off(0), Wh, D, DF);
    }
  }
  // key-norm bounds of compact tiles 0..255 (lane l of tb[j] holds tile 64 j + l; later
  // tiles, if any, are treated as unbounded)
  float tb[4];
  {
    const int ntb = nt_comp < 256 ? nt_comp : 256;
    const auto trs = make_rsrc(a.tilemax + static_cast<long long>(bh) * a.tm_stride, static_cast<uint32_t>(ntb) * 4u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(trs, (64 * j + lane) * 4, 0, 0));
      tb[j] = 64 * j + lane < nt_comp ? x : kInf;
    }
  }

  f32x4 o[HV][NB + 1][QB];
  float m_run[HV][QB];
  float qn[HV][QB];  // |q| c1: with |k| <= kmax, every logit of a tile is <= qn kmax
#pragma unroll
  for (int hv = 0; hv < HV; ++hv)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int db = 0; db <= NB; ++db) o[hv][db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // window = chunk takes a fast path for the masks and handles chunk c-1's linear keys
  // together with its window tile (head_dim 64; at 128 the extra live registers spill)
  const bool fast = D == 64 && win == kChunk && !C::SEQ;
  frag pq[HV][QB][DF / 32];  // phi(q): B-operand fragments (PK over f)
  uint64_t selprev;
  // =============================== phase 1: linear attention ===========================
  {
    // phi(q) = |q| m / |m|, m = elu(W_h q) + 1; wfrag(fb, ks) gives the W_h fragment
    auto phi_q = [&](int hv, auto wfrag) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      f32x4 pacc[DF / 16];
#pragma unroll
      for (int fb = 0; fb < DF / 16; ++fb) {
        pacc[fb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) TT::mma(pacc[fb], wfrag(fb, ks), qf[hv][qb][ks]);
      }
      float m2 = 0.f, x2 = 0.f;
#pragma unroll
      for (int fb = 0; fb < DF / 16; ++fb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float zv = pacc[fb][i];
          const float mv = zv > 0.f ? zv + 1.f : __builtin_amdgcn_exp2f(zv * kLog2e);
          pacc[fb][i] = mv;
          m2 += mv * mv;
        }
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xv = TT::to_f(qf[hv][qb][ks][e]);
          x2 += xv * xv;
        }
      m2 = xor_sum_groups(m2);
      x2 = xor_sum_groups(x2);
      qn[hv][qb] = __builtin_amdgcn_sqrtf(x2) * c1 * 1.001f;  // |q| in logit units, with slack for rounding
      const float sc = norm_ratio(x2, m2);
#pragma unroll
      for (int fs = 0; fs < DF / 32; ++fs)
#pragma unroll
        for (int e = 0; e < 8; ++e) pq[hv][qb][fs][e] = TT::from_f(pacc[2 * fs + e / 4][e % 4] * sc);
    }
    };
    if constexpr (W_EARLY) {
      // phi(q) before the wait (it overlaps the copies); keep the scheduler from moving it
      // past the wait
#pragma unroll
      for (int hv = 0; hv < HV; ++hv) phi_q(hv, [&](int fb, int ks) { return wq[fb][ks]; });
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();  // every region copied at the start has landed
    } else if constexpr (W_GLOBAL) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();  // the linear-attention tiles have landed
#pragma unroll
      for (int hv = 0; hv < HV; ++hv)
        phi_q(hv, [&](int fb, int ks) { return TT::load8(Wh + (fb * 16 + r16) * D + ks * 32 + grp * 8); });
    } else {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();  // every region copied at the start has landed, W_h among them
#pragma unroll
      for (int hv = 0; hv < HV; ++hv)
        phi_q(hv, [&](int fb, int ks) { return Swz<T, D>::load8(L + C::stage_off(0), fb * 16 + r16, ks * 32 + grp * 8); });
      __syncthreads();  // every wave is done with W_h: stage 0 takes compact tile 0
      dk.issue(L + C::stage_off(0), make_rsrc(kb_ptr, nt_comp > 0 ? C::KT * static_cast<int>(sizeof(T)) : 0u), 0);
      dv.issue(L + C::stage_off(0) + C::KT, make_rsrc(vb_ptr, nt_comp > 0 ? C::VT * static_cast<int>(sizeof(T)) : 0u), 0);
    }
    selprev = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(selv[1]))) << 32) |
              static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(selv[0]));

  }

  // ===================== per query half: phase 1 (linear attention), phase 2a (window) ==
  // Each half runs its prefix read-out, its linear keys and its window tiles before the
  // next one starts, so only one half's window scores are live at a time.
#pragma unroll
  for (int hv = 0; hv < HV; ++hv) {
  {
    // prefix state of chunks <= c-BL-1, stored as S^T[d][pk_pos(f)]: each A-operand fragment
    // (row d, the 8 features a lane group holds) is 8 consecutive elements
    if (has_state) {
#pragma unroll
      for (int fs = 0; fs < DF / 32; ++fs) {
#pragma unroll
        for (int db = 0; db < NB; ++db) {
          frag sa;
          if constexpr (C::STATE_LDS)
            sa = SF::load8(L + C::R_ST, db * 16 + r16, fs * 32 + grp * 8);
          else
            sa = TT::load8(Sg + (db * 16 + r16) * DF + fs * 32 + grp * 8);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) TT::mma(o[hv][db][qb], sa, pq[hv][qb][fs]);
        }
        // the denominator phi(q).z on the row-sum block: every row of its A operand is z,
        // so each of its entries ends up holding the whole dot product
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) TT::mma(o[hv][NB][qb], zf[fs], pq[hv][qb][fs]);
      }
    }
    // linear keys of chunk c-1 (p <= r + 64 - w, unselected) and of chunk c (p <= r - w);
    // the fast path takes chunk c-1's with its window tile (chunk c has none when w = 64)
    frag ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = TT::from_f(1.0f);
#pragma unroll
    for (int cur = 0; cur < 2; ++cur) {
      if (fast || (cur == 0 ? !has_prev : !la_cur)) continue;  // uniform
      const int qoff = qoff0 + hv * QW;
      const T* lk = L + (cur == 0 ? C::R_PHIP : C::R_PHIC);
      const T* lv = L + (cur == 0 ? C::R_VP : C::R_VC);
      f32x4 ls[4][QB];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) ls[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int fs = 0; fs < DF / 32; ++fs) {
          const frag fa = SF::load8(lk, kb * 16 + r16, fs * 32 + grp * 8);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) TT::mma(ls[kb][qb], fa, pq[hv][qb][fs]);
        }
      }
      const uint32_t selw = cur ? 0u : bits_word(selprev);
      frag pf[2][QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int r = qoff + qb * 16 + r16;
        const uint32_t lw = range_word(0, cur ? r - win : r + 64 - win) & ~selw;
        float pv[4][4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pv[kb][i] = (lw & (1u << (kb * 4 + i))) ? ls[kb][qb][i] : 0.f;
          }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[ks][qb][e] = TT::from_f(pv[2 * ks + e / 4][e % 4]);
      }
#pragma unroll
      for (int db = 0; db < NB; ++db)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const frag va = SV::load8(lv, db * 16 + r16, ks * 32 + grp * 8);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) TT::mma(o[hv][db][qb], va, pf[ks][qb]);
        }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) TT::mma(o[hv][NB][qb], ones, pf[ks][qb]);  // their denominator
    }
    // the linear branch becomes one online-softmax entry: log-weight log2(D), value N / D
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float dt = o[hv][NB][qb][0];
      const float inv = dt > 0.f ? __builtin_amdgcn_rcpf(dt) : 0.f;
#pragma unroll
      for (int db = 0; db < NB; ++db) o[hv][db][qb] *= inv;
      m_run[hv][qb] = dt > 0.f ? __log2f(dt) : -kInf;
      const float l0 = dt > 0.f ? 1.f : 0.f;
      o[hv][NB][qb] = f32x4{l0, l0, l0, l0};
    }
  }
  // =============================== phase 2: softmax tiles ==============================
  if constexpr (C::SEQ) {  // (one query half in this plan)  // K of chunks c and c-1 over the phi(K) regions phase 1 is done with
    __syncthreads();
    const int kvs = d.Hkv * D;
    const long long tp = has_prev ? t0 - kChunk : t0;
    dma_tile<T, D, 64, NW>(L + C::R_KP, kk + ((b * T_ + tp) * d.Hkv + h) * D, kvs, has_prev && win >= 1 ? 64 : 0);
    dma_tile<T, D, 64, NW>(L + C::R_KC, kk + ((b * T_ + t0) * d.Hkv + h) * D, kvs, win >= 1 ? nvalid : 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  // 2a. the window: chunk c (r - w < p <= r), chunk c-1 (p > r + 64 - w, or selected)
  {
  const int qoff = qoff0 + hv * QW;
  if (fast) {
    if (qoff == 0)
      window_fast<T, D, DF, QB, 0>(L + C::R_KC, L + C::R_VC, L + C::R_KP, L + C::R_PHIP, L + C::R_VP, has_prev, selprev,
                                   qf[hv], pq[hv], o[hv], m_run[hv], c1);
    else
      window_fast<T, D, DF, QB, QW>(L + C::R_KC, L + C::R_VC, L + C::R_KP, L + C::R_PHIP, L + C::R_VP, has_prev,
                                    selprev, qf[hv], pq[hv], o[hv], m_run[hv], c1);
  } else if (win >= 1) {
    f32x4 s[4][QB];
    uint32_t kw[QB];
    qk_tile<T, D, QB>(L + C::R_KC, qf[hv], s);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int r = qoff + qb * 16 + r16;
      kw[qb] = range_word(r - win + 1, r);
    }
    mask_tile<QB>(s, kw);
    sm_max<D, QB>(s, o[hv], m_run[hv], c1);
    sm_exp_pv<T, D, QB>(s, L + C::R_VC, o[hv], m_run[hv], c1);
    if (has_prev) {
      const uint32_t selw = bits_word(selprev);
      qk_tile<T, D, QB>(L + C::R_KP, qf[hv], s);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int r = qoff + qb * 16 + r16;
        kw[qb] = range_word(r + 65 - win, 63) | selw;
      }
      mask_tile<QB>(s, kw);
      sm_max<D, QB>(s, o[hv], m_run[hv], c1);
      sm_exp_pv<T, D, QB>(s, L + C::R_VP, o[hv], m_run[hv], c1);
    }
  }
  }

  }

  // 2c. band chunks c-2 .. c-BL (windows longer than a chunk): each staged into the fixed
  //     regions, then both kinds of keys for every query half
  if constexpr (BAND)
  for (int l = 2; l <= BL && l <= c; ++l) {  // uniform
    __syncthreads();  // every wave is done with the fixed regions (or the previous band chunk)
    const long long tb = t0 - static_cast<long long>(l) * kChunk;
    dma_tile<T, D, 64, NW>(L + C::R_BK, kk + ((b * T_ + tb) * d.Hkv + h) * D, d.Hkv * D, 64);
    dma_tile<T, DF, 64, NW>(L + C::R_BF, phik + (bkv * T_ + tb) * DF, DF, 64);
    dma_tile<T, 64, D, NW>(L + C::R_BV, vT + (bkv * d.nC + (c - l)) * D * 64, 64, D);
    const uint64_t sel = a.selmask[static_cast<long long>(bh) * d.nC + (c - l)];
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int hv = 0; hv < HV; ++hv)
      band_tile<T, D, DF, QB>(L + C::R_BK, L + C::R_BF, L + C::R_BV, qoff0 + hv * QW, l * kChunk - win, sel, qf[hv],
                              pq[hv], o[hv], m_run[hv], c1);
  }

  // 2b. the compact cache: selected rows of chunks <= c-BL-1, unmasked except a ragged end.
  //     Tile t lives in stage t % 4. Tile 0 was copied at the start; tiles 1..3 go into
  //     the fixed regions once every wave is done with them, and tile t+3 is issued in step
  //     t, two steps ahead of its first use. In step t each wave waits for its own copies of
  //     tile t+1 (those of tile t+2 may still be in flight), the barrier makes tile t+1
  //     visible and frees tile t-1's stage; the K Q^T product of tile t+1 (MFMA) then issues
  //     interleaved with the softmax of tile t (VALU). Rows past the last compact row of a
  //     ragged tile are copied too (they lie inside the buffer; their scores are masked and
  //     their V^T columns are zero or finite).
  if (nt_comp > 0) {
    // The running max is fixed for the whole compact loop, so its steps have no max pass
    // and no branch rewrites the accumulators. A compact logit of a query is at most
    // U = |q| max|k|, the largest key-norm bound of the chunk's compact tiles (prep and
    // scan). Where U - kLazy exceeds the running max by at most kRaise, the max is raised to
    // U - kLazy: what is accumulated so far keeps a weight of at least 2^-kRaise, and a
    // compact weight small enough to underflow (below 2^-126) is negligible next to it.
    // Otherwise (very large norms, or tiles past the bounds' reach) a pre-pass takes the
    // exact largest compact logit.
    {
      float tmax = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) tmax = fmaxf(tmax, 64 * j + lane < nt_comp ? tb[j] : 0.f);
      tmax = wave_max64(tmax);
      float m0[HV][QB];
      bool exact = nt_comp > 256;
#pragma unroll
      for (int hv = 0; hv < HV; ++hv)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          m0[hv][qb] = fmaxf(m_run[hv][qb], qn[hv][qb] * tmax - kLazy);
          exact |= m_run[hv][qb] == -kInf || m0[hv][qb] - m_run[hv][qb] > kRaise;
        }
      if (__builtin_amdgcn_ballot_w64(exact) != 0) {
        compact_max<T, D, QB, HV>(krs, n_comp, qf, m0, c1);
#pragma unroll
        for (int hv = 0; hv < HV; ++hv)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) m0[hv][qb] = fmaxf(m_run[hv][qb], m0[hv][qb]);
      }
      bool moved = false;
#pragma unroll
      for (int hv = 0; hv < HV; ++hv)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) moved |= m0[hv][qb] > m_run[hv][qb];
      if (__builtin_amdgcn_ballot_w64(moved) != 0) {
#pragma unroll
        for (int hv = 0; hv < HV; ++hv)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const float alpha = m_run[hv][qb] == -kInf ? 0.f : __builtin_amdgcn_exp2f(m_run[hv][qb] - m0[hv][qb]);
#pragma unroll
            for (int db = 0; db <= NB; ++db) o[hv][db][qb] *= alpha;
            m_run[hv][qb] = m0[hv][qb];
          }
      }
    }
    if constexpr (C::SEQ) {
      // two stages over the fixed regions: tile t in stage t % 2, tile t + 2 issued once
      // every wave is done with tile t
      __syncthreads();  // every wave is done with the window tiles
      issue(0, 0);
      if (nt_comp > 1) issue(1, 1);
      for (int t = 0; t < nt_comp; ++t) {
        if (t + 1 < nt_comp)
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::NL));
        else
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        lds_barrier();
        f32x4 sc[4][QB];
        qk_tile<T, D, QB>(L + C::stage_off(t & 1), qf[0], sc);
        const int nk = n_comp - t * 64;
        if (nk < 64) {
          uint32_t kw[QB];
          const uint32_t rw = range_word(0, nk - 1);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) kw[qb] = rw;
          mask_tile<QB>(sc, kw);
        }
        sm_exp_pv<T, D, QB>(sc, L + C::stage_off(t & 1) + C::KT, o[0], m_run[0], c1);
        __builtin_amdgcn_s_waitcnt(0);  // this wave's reads of the stage are done (and no copy is in flight)
        lds_barrier();
        if (t + 2 < nt_comp) issue(t + 2, t & 1);
      }
    } else if constexpr (HV == 2) {
      // Both query halves per step, each K and V^T fragment read once for both. Tile t in
      // stage t % 4; tile 0 landed with the fixed part, tiles 1 and 2 are issued once every
      // wave is done with the fixed regions, tile t + 3 in step t (into the stage of tile
      // t - 1, free after the step's barrier). Step t waits for its own copies of tile t
      // (those of tiles t + 1 and t + 2 may still be in flight).
      if constexpr (!W_EARLY) {  // tile 0 was copied after phi(q)
        __builtin_amdgcn_s_waitcnt(0);
      }
      __syncthreads();
      if (1 < nt_comp) issue(1, 1);
      if (2 < nt_comp) issue(2, 2);
      // the row sums as per-lane partials: lane group 0 starts from the whole sum so far
      float lp[HV][QB];
#pragma unroll
      for (int hv = 0; hv < HV; ++hv)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) lp[hv][qb] = grp == 0 ? o[hv][NB][qb][0] : 0.f;
      // One step; RAGGED: the last tile, keys past n_comp masked.
      auto step = [&](int t, auto ragged) {
        constexpr bool RAGGED = decltype(ragged)::value;
        if (t + 2 < nt_comp)
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * C::NL));
        else if (t + 1 < nt_comp)
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::NL));
        else
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        lds_barrier();
        if (t + 3 < nt_comp) issue(t + 3, (t + 3) & 3);
        f32x4 sc[HV][4][QB];
        qk_tile_hv<T, D, QB, HV>(L + C::stage_off(t & 3), qf, sc);
        if constexpr (RAGGED) {
          uint32_t kw[QB];
          const uint32_t rw = range_word(0, n_comp - t * 64 - 1);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) kw[qb] = rw;
#pragma unroll
          for (int hv = 0; hv < HV; ++hv) mask_tile<QB>(sc[hv], kw);
        }
        sm_exp_pv_hv<T, D, QB, HV>(sc, L + C::stage_off(t & 3) + C::KT, o, lp, m_run, c1);
      };
      const int nt_full = n_comp / 64;  // tiles of 64 keys; a ragged one, if any, follows
      for (int t = 0; t < nt_full; ++t) step(t, std::false_type{});
      if (nt_full < nt_comp) step(nt_full, std::true_type{});
#pragma unroll
      for (int hv = 0; hv < HV; ++hv)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float l = xor_sum_groups(lp[hv][qb]);
          o[hv][NB][qb] = f32x4{l, l, l, l};
        }
    } else {
    f32x4 sa[4][QB], sb[4][QB];
    if constexpr (!W_EARLY) {  // tile 0 was copied after phi(q)
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    qk_tile<T, D, QB>(L + C::stage_off(0), qf[0], sa);  // tile 0 has landed
    __syncthreads();
#pragma unroll
    for (int t = 1; t < 4; ++t)
      if (t < nt_comp) issue(t, t);
    auto step = [&](int t, f32x4 (&s_cur)[4][QB], f32x4 (&s_next)[4][QB]) {
      if (t + 2 < nt_comp)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::NL));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      lds_barrier();
      if (t >= 1 && t + 3 < nt_comp) issue(t + 3, (t + 3) & 3);
      const int nk = n_comp - t * 64;
      if (nk < 64) {
        uint32_t kw[QB];
        const uint32_t rw = range_word(0, nk - 1);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) kw[qb] = rw;
        mask_tile<QB>(s_cur, kw);
      }
      qk_tile<T, D, QB>(L + C::stage_off((t + 1) & 3), qf[0], s_next);  // after the last tile: unused
      sm_exp_pv<T, D, QB>(s_cur, L + C::stage_off(t & 3) + C::KT, o[0], m_run[0], c1);
    };
    for (int t = 0; t < nt_comp; t += 2) {
      step(t, sa, sb);
      if (t + 1 < nt_comp) step(t + 1, sb, sa);
    }
    }
  }

  // ---- epilogue: divide by the shared normaliser, write [B,T,Hq,D] ------------------
  T* out = static_cast<T*>(a.out);
#pragma unroll
  for (int hv = 0; hv < HV; ++hv)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = o[hv][NB][qb][0];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int r = qoff0 + hv * QW + qb * 16 + r16;
    if (head_ok && r < nvalid) {
      T* dst = out + ((b * T_ + t0 + r) * d.Hq + hq) * D + 4 * grp;
#pragma unroll
      for (int db = 0; db < NB; ++db) {
        typename TT::quad ov;
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = TT::from_f(o[hv][db][qb][i] * inv);
        *reinterpret_cast<typename TT::quad*>(dst + db * 16) = ov;
      }
    }
  }
}

// ======================================================================================
// Window = chunk at bf16 with head_dim = feat_dim = D in {64, 128} and four query heads per
// workgroup (the Llama-3.2-1B- and Llama-3.1-8B-shaped layers), under a softmax frame fixed
// up front.
//
// A wave takes one query head: at D = 64 all 64 queries of chunk c (two 32-query halves,
// HV = 2) in a four-wave workgroup; at D = 128 one 32-query half (HV = 1) in an eight-wave
// workgroup (wave w: head slot w % 4, half w / 4). Before any
// tile, each query's frame m0 (log2 units) is set so that no weight can pass 2^32 and
// nothing is ever rescaled: a softmax logit is at most |q| Kmax c1 and a linear weight
// phi(q).phi(k) at most |q| Kmax (the NP-Map preserves norms), where Kmax is the largest key
// norm of the window chunks (kall) and of the compact tiles (tilemax). So
//   m0 = max(a_ii c1, |q| Kmax c1 - kLazy, log2(|q| Kmax) - kLazy),
// with a_ii c1 the query's own logit, which is always a softmax term. Where m0 is more than
// kRaise above a_ii c1, the wave takes the exact largest log-weight over all of its terms
// instead (global loads only: no LDS, no barrier). Then, with no max pass anywhere:
//   1. per query half: phi(q) (W_h from LDS), the prefix read-out (one entry of weight
//      D 2^-m0 and value N / D), chunk c (causal) and chunk c-1 (softmax keys p > r, linear
//      keys p <= r, one P for both);
//   2. the compact tiles through a four-stage LDS ring (stage 0 of its own, stages 1..3 over
//      the window regions once the window is done), copies issued three tiles ahead. They
//      include chunk c-1's selected keys, which are softmax keys for every query of chunk c,
//      so chunk c-1's tile needs no per-key selection test: their V^T columns are zeroed in
//      LDS and its row sums use a not-selected vector;
//   3. the normalised output through LDS, so every position's four heads leave as one
//      contiguous row.
// Every P is 2^(a c1 - m0) or phi(q).phi(k) 2^-m0; the row sums ride along in the products
// as an extra all-ones (or not-selected) A block.
template <int D>
struct FF {
  static constexpr int QB = 2, NB = D / 16;
  static constexpr int HV = D == 64 ? 2 : 1;     // 32-query halves per wave
  static constexpr int NW = D == 64 ? 4 : 8;     // waves per workgroup: 4 head slots x 64 / (32 HV) halves
  static constexpr int NTHR = 64 * NW;
  static constexpr int KT = 64 * D, ST = D * D;  // a 64-row tile (K, V^T, phi(K)); the state S^T and W_h
  static constexpr int STAGE = 2 * KT;           // a compact stage (K, V^T)
  // window regions, then (D = 64) compact stage 0 and W_h, or (D = 128) W_h over compact
  // stage 0, which takes compact tile 0 once every wave has its phi(q)
  static constexpr bool W_IN_S0 = D == 128;
  static constexpr int R_PHIP = 0, R_VP = R_PHIP + KT, R_VC = R_VP + KT, R_KC = R_VC + KT, R_KP = R_KC + KT,
                       R_ST = R_KP + KT, R_S0 = R_ST + ST, R_W = W_IN_S0 ? R_S0 : R_S0 + STAGE,
                       LDS_ELEMS = W_IN_S0 ? R_S0 + STAGE : R_W + ST;
  static constexpr int LDS_BYTES = LDS_ELEMS * 2;
  static_assert(!W_IN_S0 || ST <= STAGE, "W_h fits in compact stage 0");
  static_assert(3 * STAGE <= R_S0, "compact stages 1..3 fit over the window regions");
  static_assert(LDS_BYTES <= (NW == 4 ? 80 : 160) * 1024, "two four-wave or one eight-wave workgroup per CU");
  // copy instructions per wave: one compact tile; the window tiles and the state; W_h
  static constexpr int NL = DmaTile<bf16, D, 64, NW>::PER_WAVE + DmaTile<bf16, 64, D, NW>::PER_WAVE;
  static constexpr int NWIN = 3 * DmaTile<bf16, D, 64, NW>::PER_WAVE + 2 * DmaTile<bf16, 64, D, NW>::PER_WAVE +
                              DmaTile<bf16, D, D, NW>::PER_WAVE;
  static constexpr int NWH = DmaTile<bf16, D, D, NW>::PER_WAVE;
  static __device__ __forceinline__ int stage_off(int s) { return s == 0 ? R_S0 : (s - 1) * STAGE; }
};

// acc + the dot product of two fragments (bf16: four dot2; fp32: fmas)
template <typename F> __device__ __forceinline__ float frag_dot(const F& x, const F& y, float acc) {
  if constexpr (sizeof(x[0]) == 2) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{x[2 * j], x[2 * j + 1]}, bf16x2_t{y[2 * j], y[2 * j + 1]}, acc, false);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += x[j] * y[j];
  }
  return acc;
}

// phi(q) = |q| m / |m|, m = elu(W_h q) + 1, for the 16-query blocks of qf (B-operand, SK
// over d); W_h fragments from wfrag(fb, ks). Leaves PK-ordered B fragments over f.
template <typename T, int D, int DF, int QB, typename WF>
__device__ __forceinline__ void phi_q_frags(const typename Tr<T>::frag (&qf)[QB][D / 32], WF wfrag,
                                            typename Tr<T>::frag (&pq)[QB][DF / 32]) {
  using TT = Tr<T>;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    f32x4 pacc[DF / 16];
#pragma unroll
    for (int fb = 0; fb < DF / 16; ++fb) {
      pacc[fb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) TT::mma(pacc[fb], wfrag(fb, ks), qf[qb][ks]);
    }
    float m2 = 0.f, x2 = 0.f;
#pragma unroll
    for (int fb = 0; fb < DF / 16; ++fb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float zv = pacc[fb][i];
        const float mv = zv > 0.f ? zv + 1.f : __builtin_amdgcn_exp2f(zv * kLog2e);
        pacc[fb][i] = mv;
        m2 += mv * mv;
      }
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) x2 = frag_dot(qf[qb][ks], qf[qb][ks], x2);
    const float sc = norm_ratio(xor_sum_groups(x2), xor_sum_groups(m2));
#pragma unroll
    for (int fs = 0; fs < DF / 32; ++fs)
#pragma unroll
      for (int e = 0; e < 8; ++e) pq[qb][fs][e] = TT::from_f(pacc[2 * fs + e / 4][e % 4] * sc);
  }
}

// The exact frame of a wave's queries (half0: its first 32-query half): the largest of the
// softmax logits (compact keys, chunk c up to the query, chunk c-1 past the query or
// selected; times c1) and of log2 of the whole linear weight (prefix state plus chunk c-1's
// other keys). Global loads only, so the other waves are not held up.
template <typename T, int D>
__device__ __forceinline__ void ff_exact_frame(const typename Tr<T>::frag (&qf)[FF<D>::HV][FF<D>::QB][D / 32],
                                               float (&m0)[FF<D>::HV][FF<D>::QB], int half0,
                                               __amdgpu_buffer_rsrc_t krs, int n_comp, __amdgpu_buffer_rsrc_t kc_rs,
                                               __amdgpu_buffer_rsrc_t kp_rs, int kst, __amdgpu_buffer_rsrc_t fp_rs,
                                               uint64_t selprev, const T* Wh, __amdgpu_buffer_rsrc_t z_rs,
                                               bool has_prev, float c1) {
  using TT = Tr<T>;
  using frag = typename TT::frag;
  constexpr int QB = FF<D>::QB, HV = FF<D>::HV, KS = D / 32;
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
  float cm[HV][QB];
  compact_max<T, D, QB, HV>(krs, n_comp, qf, cm, c1);
  const uint32_t selw = bits_word(selprev);
#pragma unroll
  for (int hv = 0; hv < HV; ++hv) {
    frag pq[QB][KS];
    phi_q_frags<T, D, D, QB>(qf[hv], [&](int fb, int ks) { return TT::load8(Wh + (fb * 16 + r16) * D + ks * 32 + grp * 8); },
                             pq);
    float smax[QB], lsum[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      smax[qb] = cm[hv][qb];
      lsum[qb] = 0.f;
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      frag ka[KS], kp[KS], fa[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        ka[ks] = TT::bload8(kc_rs, ((kb * 16 + r16) * kst + ks * 32 + grp * 8) * 2, 0);
        kp[ks] = TT::bload8(kp_rs, ((kb * 16 + r16) * kst + ks * 32 + grp * 8) * 2, 0);
        fa[ks] = TT::bload8(fp_rs, ((kb * 16 + r16) * D + ks * 32 + grp * 8) * 2, 0);
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        f32x4 sc = {0.f, 0.f, 0.f, 0.f}, sp = sc, ls = sc;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          TT::mma(sc, ka[ks], qf[hv][qb][ks]);
          TT::mma(sp, kp[ks], qf[hv][qb][ks]);
          TT::mma(ls, fa[ks], pq[qb][ks]);
        }
        const int r = (half0 + hv) * 32 + qb * 16 + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int p = kb * 16 + 4 * grp + i;
          const bool sel = (selw >> (kb * 4 + i)) & 1u;
          if (p <= r) smax[qb] = fmaxf(smax[qb], sc[i] * c1);
          if (has_prev && (p > r || sel)) smax[qb] = fmaxf(smax[qb], sp[i] * c1);
          if (has_prev && p <= r && !sel) lsum[qb] += ls[i];
        }
      }
    }
    // the prefix state's linear weight phi(q).z: every row of the A operand is z
    frag zf[KS];
#pragma unroll
    for (int fs = 0; fs < KS; ++fs) zf[fs] = TT::bload8(z_rs, (fs * 32 + grp * 8) * 2, 0);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      f32x4 dz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int fs = 0; fs < KS; ++fs) TT::mma(dz, zf[fs], pq[qb][fs]);
      const float la = xor_sum_groups(lsum[qb]) + dz[0];
      const float mx = xor_max_groups(smax[qb]);
      m0[hv][qb] = la > 0.f ? fmaxf(mx, __log2f(la)) : mx;
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(FF<D>::NTHR, (FF<D>::NW == 4 ? 2 : 1)) void attn_ff_kernel(AttnArgs a) {
  using C = FF<D>;
  constexpr int QB = C::QB, HV = C::HV, NW = C::NW, NB = C::NB, KT = C::KT, KS = D / 32;
  using TT = Tr<T>;
  using frag = typename TT::frag;
  using SK = Swz<T, D>;   // K, phi(K) (64 rows), the state S^T and W_h (D rows): rows of D
  using SV = Swz<T, 64>;  // V^T tiles: D rows of 64 keys
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  T* L = reinterpret_cast<T*>(lds_raw);

  const Dims& d = a.d;
  const T* q = static_cast<const T*>(a.q);
  const T* kk = static_cast<const T*>(a.k);
  const T* vT = static_cast<const T*>(a.vT);
  const T* phik = static_cast<const T*>(a.phik);
  // work item: heaviest chunks first; within a chunk consecutive (b, h, head split), so each
  // of the eight XCDs keeps a fixed set of KV heads in its L2
  const int BHG = d.B * d.Hr * a.gsplit;
  const int c = d.nC - 1 - static_cast<int>(blockIdx.x) / BHG;
  const int bhg = static_cast<int>(blockIdx.x) % BHG;
  const int gs = bhg % a.gsplit, bh = bhg / a.gsplit;
  const int b = bh / d.Hr, rh = bh % d.Hr, h = rh * d.Gr / d.G;
  const long long bkv = static_cast<long long>(b) * d.Hkv + h;
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = NW == 4 ? wave : wave & 3;    // head slot
  const int half0 = NW == 4 ? 0 : wave >> 2;     // first 32-query half of the wave
  const int hq = rh * d.Gr + gs * 4 + slot;      // every head of the split exists (Gr % 4 == 0)
  const long long T_ = d.T;
  const long long t0 = static_cast<long long>(c) * kChunk;
  const int nvalid = static_cast<int>(T_ - t0 < kChunk ? T_ - t0 : kChunk);
  const float c1 = kLog2e / sqrtf(static_cast<float>(D));
  const bool has_prev = c >= 1, has_state = c >= 2;
  // compact rows of chunks <= c-1: chunk c-1's selected keys are softmax keys for every query
  // of chunk c, so they join the compact tiles (their rows follow chunk c-2's)
  const int n_comp = c * d.topk;
  const int nt_comp = (n_comp + 63) / 64;
  const int kst = d.Hkv * D;  // row stride of k
  const long long tp = has_prev ? t0 - kChunk : t0;

  const T* kb_ptr = static_cast<const T*>(a.ksel) + static_cast<long long>(bh) * a.ntiles_sel * 64 * D;
  const T* vb_ptr = static_cast<const T*>(a.vselT) + static_cast<long long>(bh) * a.ntiles_sel * D * 64;
  DmaTile<T, D, 64, NW> dk;
  DmaTile<T, 64, D, NW> dv;
  dk.init(D);
  dv.init(64);
  const auto krs = make_rsrc(kb_ptr, static_cast<uint32_t>(nt_comp) * KT * 2u);
  const auto vrs = make_rsrc(vb_ptr, static_cast<uint32_t>(nt_comp) * KT * 2u);
  auto issue = [&](int t, int stage) {
    T* st = L + C::stage_off(stage);
    dk.issue(st, krs, t * KT * 2);
    dv.issue(st + KT, vrs, t * KT * 2);
  };

  // ---- 1. register operands: the queries and their own keys (B-operand layout), the tile
  //      and window key-norm bounds, the selection of chunk c-1 ------------------------------
  frag qf[HV][QB][KS], kd[HV][QB][KS];
#pragma unroll
  for (int hv = 0; hv < HV; ++hv) {
    const long long q0 = t0 + (half0 + hv) * 32;
    const long long nq = T_ - q0 < 32 ? T_ - q0 : 32;
    const int qrow = d.Hq * D;
    const auto qrs = make_rsrc(q + ((b * T_ + (nq > 0 ? q0 : 0)) * d.Hq + hq) * D,
                               nq > 0 ? static_cast<uint32_t>(((nq - 1) * qrow + D) * 2) : 0u);
    const auto krd = make_rsrc(kk + ((b * T_ + (nq > 0 ? q0 : 0)) * d.Hkv + h) * D,
                               nq > 0 ? static_cast<uint32_t>(((nq - 1) * kst + D) * 2) : 0u);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qf[hv][qb][ks] = TT::bload8(qrs, ((qb * 16 + r16) * qrow + ks * 32 + grp * 8) * 2, 0);
        kd[hv][qb][ks] = TT::bload8(krd, ((qb * 16 + r16) * kst + ks * 32 + grp * 8) * 2, 0);
      }
  }
  float tb[4];
  {
    const int ntb = nt_comp < 256 ? nt_comp : 256;
    const auto trs = make_rsrc(a.tilemax + static_cast<long long>(bh) * a.tm_stride, static_cast<uint32_t>(ntb) * 4u);
#pragma unroll
    for (int j = 0; j < 4; ++j) tb[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(trs, (64 * j + lane) * 4, 0, 0));
  }
  const auto selv = __builtin_amdgcn_raw_buffer_load_b64(
      make_rsrc(a.selmask + static_cast<long long>(bh) * d.nC + (has_prev ? c - 1 : 0), has_prev ? 8u : 0u), 0, 0, 0);
  const float kwin = fmaxf(a.kall[static_cast<long long>(bh) * d.nC + c],
                           has_prev ? a.kall[static_cast<long long>(bh) * d.nC + c - 1] : 0.f);

  // ---- 2. copies: the window tiles, the prefix state and W_h into their regions, then (W_h
  //      outside stage 0) compact tile 0 into stage 0 (zero-filled where absent) --------------
  const T* Sg = static_cast<const T*>(a.states) + (static_cast<long long>(bh) * d.nC + (has_state ? c - 2 : 0)) * d.R;
  const T* Wh = static_cast<const T*>(a.w) + static_cast<long long>(h) * D * D;
  dma_tile<T, D, 64, NW>(L + C::R_PHIP, phik + (bkv * T_ + tp) * D, D, has_prev ? 64 : 0);
  dma_tile<T, 64, D, NW>(L + C::R_VP, vT + (bkv * d.nC + (has_prev ? c - 1 : c)) * D * 64, 64, has_prev ? D : 0);
  dma_tile<T, 64, D, NW>(L + C::R_VC, vT + (bkv * d.nC + c) * D * 64, 64, D);
  dma_tile<T, D, 64, NW>(L + C::R_KC, kk + ((b * T_ + t0) * d.Hkv + h) * D, kst, nvalid);
  dma_tile<T, D, 64, NW>(L + C::R_KP, kk + ((b * T_ + tp) * d.Hkv + h) * D, kst, has_prev ? 64 : 0);
  dma_tile<T, D, D, NW>(L + C::R_ST, Sg, D, has_state ? D : 0);
  dma_tile<T, D, D, NW>(L + C::R_W, Wh, D, D);
  if constexpr (!C::W_IN_S0) issue(0, 0);
  constexpr int N_AFTER_WIN = C::W_IN_S0 ? 0 : C::NL;  // copies issued after the window ones
  // z of the prefix state (A operand of the denominator, the same in every row)
  frag zf[KS];
  {
    const auto zrs = make_rsrc(Sg + D * D, has_state ? static_cast<uint32_t>(D) * 2u : 0u);
#pragma unroll
    for (int fs = 0; fs < KS; ++fs) zf[fs] = TT::bload8(zrs, (fs * 32 + grp * 8) * 2, 0);
  }

  // ---- 3. the frame ---------------------------------------------------------------------
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::NWIN + C::NWH + N_AFTER_WIN + KS));  // the register operands
  const uint64_t selprev = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(selv[1]))) << 32) |
                           static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(selv[0]));
  float kmax = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) kmax = fmaxf(kmax, 64 * j + lane < nt_comp ? tb[j] : 0.f);
  kmax = fmaxf(wave_max64(kmax), kwin);
  float m0[HV][QB];
  bool exact = nt_comp > 256;  // tiles past 256 carry no bound here
#pragma unroll
  for (int hv = 0; hv < HV; ++hv)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float dq = 0.f, q2 = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        dq = frag_dot(qf[hv][qb][ks], kd[hv][qb][ks], dq);
        q2 = frag_dot(qf[hv][qb][ks], qf[hv][qb][ks], q2);
      }
      const float ref = xor_sum_groups(dq) * c1;                                      // the query's own logit
      const float ub = __builtin_amdgcn_sqrtf(xor_sum_groups(q2)) * 1.001f * kmax;  // >= |q| |k|, any key
      float m = fmaxf(ref, ub * c1 - kLazy);
      if (ub > 0.f) m = fmaxf(m, __log2f(ub) - kLazy);
      exact |= m - ref > kRaise;
      m0[hv][qb] = m;
    }
  if (__builtin_amdgcn_ballot_w64(exact) != 0)
    ff_exact_frame<T, D>(
        qf, m0, half0, krs, n_comp,
        make_rsrc(kk + ((b * T_ + t0) * d.Hkv + h) * D, static_cast<uint32_t>(((nvalid - 1) * kst + D) * 2)),
        make_rsrc(kk + ((b * T_ + tp) * d.Hkv + h) * D, has_prev ? static_cast<uint32_t>((63 * kst + D) * 2) : 0u), kst,
        make_rsrc(phik + (bkv * T_ + tp) * D, has_prev ? static_cast<uint32_t>(64 * D * 2) : 0u), selprev, Wh,
        make_rsrc(Sg + D * D, has_state ? static_cast<uint32_t>(D) * 2u : 0u), has_prev, c1);
  // o[hv][NB]: the row sums, riding along in the products (an all-ones A block)
  f32x4 o[HV][NB + 1][QB];
#pragma unroll
  for (int hv = 0; hv < HV; ++hv)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int db = 0; db <= NB; ++db) o[hv][db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const frag ones = ones_frag<T>();
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(N_AFTER_WIN));  // the window regions, the state and W_h
  lds_barrier();
  // chunk c-1's selected keys are taken with the compact tiles: zero their V^T columns here,
  // and count chunk c-1's row sums with a not-selected vector instead of ones
  if (has_prev && selprev != 0) {
    if (tid < D)
      for (uint64_t m = selprev; m != 0; m &= m - 1)
        L[C::R_VP + SV::off(tid, pk_pos(static_cast<int>(__builtin_ctzll(m))))] = TT::from_f(0.f);
    __syncthreads();
  }
  frag nsel[2];  // A operand: 1 for the keys of chunk c-1 that are not selected (PK order)
#pragma unroll
  for (int hs = 0; hs < 2; ++hs)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      nsel[hs][e] = TT::from_f(((selprev >> (hs * 32 + 16 * (e / 4) + 4 * grp + e % 4)) & 1ull) ? 0.f : 1.f);

  // ---- 4. per query half: phi(q), the prefix read-out, chunk c, chunk c-1 ----------------
  bool dmask[4];  // key position <= query position, on a diagonal block
#pragma unroll
  for (int i = 0; i < 4; ++i) dmask[i] = 4 * grp + i <= r16;
  frag pq[HV][QB][KS];  // phi(q): PK-ordered B fragments over f
#pragma unroll
  for (int hv = 0; hv < HV; ++hv)
    phi_q_frags<T, D, D, QB>(qf[hv], [&](int fb, int ks) { return SK::load8(L + C::R_W, fb * 16 + r16, ks * 32 + grp * 8); },
                             pq[hv]);
  if constexpr (C::W_IN_S0) {  // W_h's region becomes compact stage 0
    lds_barrier();
    issue(0, 0);
  }
#pragma unroll
  for (int hv = 0; hv < HV; ++hv) {
    const int qh = half0 + hv;  // this 32-query half of the chunk (wave-uniform)
    // prefix read-out: N = S^T phi(q) (state rows d, PK features) and D = phi(q).z
    if (has_state) {
      f32x4 la[NB][QB], dz[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        dz[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < NB; ++db) la[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int fs = 0; fs < KS; ++fs) {
#pragma unroll
        for (int db = 0; db < NB; ++db) {
          const frag sa = SK::load8(L + C::R_ST, db * 16 + r16, fs * 32 + grp * 8);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) TT::mma(la[db][qb], sa, pq[hv][qb][fs]);
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) TT::mma(dz[qb], zf[fs], pq[hv][qb][fs]);
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float dt = dz[qb][0];
        // weight D 2^-m0 taken in the log domain (D may be far outside 2^-m0's range)
        const float wgt = dt > 0.f ? __builtin_amdgcn_exp2f(__log2f(dt) - m0[hv][qb]) : 0.f;
        const float f = dt > 0.f ? wgt * __builtin_amdgcn_rcpf(dt) : 0.f;
#pragma unroll
        for (int db = 0; db < NB; ++db) o[hv][db][qb] += la[db][qb] * f;
        o[hv][NB][qb] += wgt;
      }
    }
    // chunk c: softmax keys p <= r
    {
      f32x4 s[4][QB];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const frag ka = SK::load8(L + C::R_KC, kb * 16 + r16, ks * 32 + grp * 8);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            if (kb <= 2 * qh + qb) TT::mma(s[kb][qb], ka, qf[hv][qb][ks]);
        }
      }
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        if (2 * hs > 2 * qh + 1) continue;  // every key of this half lies past every query
        frag pf[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int qblk = 2 * qh + qb;  // 16-query block of the chunk
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int kb = 2 * hs + e / 4, i = e % 4;
            float p = 0.f;
            if (kb < qblk || (kb == qblk && dmask[i]))
              p = __builtin_amdgcn_exp2f(s[kb][qb][i] * c1 - m0[hv][qb]);
            pf[qb][e] = TT::from_f(p);
          }
        }
#pragma unroll
        for (int db = 0; db < NB; ++db) {
          const frag va = SV::load8(L + C::R_VC, db * 16 + r16, hs * 32 + grp * 8);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            if (2 * hs <= 2 * qh + qb) TT::mma(o[hv][db][qb], va, pf[qb]);
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          if (2 * hs <= 2 * qh + qb) TT::mma(o[hv][NB][qb], ones, pf[qb]);
      }
    }
    // chunk c-1: softmax keys p > r, linear keys p <= r (one P for both); the selected keys
    // are in the compact tiles, and their columns here add nothing (zero V^T, zero in nsel)
    if (has_prev) {
      f32x4 s[4][QB], ls[4][QB];
      qk_tile<T, D, QB>(L + C::R_KP, qf[hv], s);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) ls[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int fs = 0; fs < KS; ++fs) {
          const frag fa = SK::load8(L + C::R_PHIP, kb * 16 + r16, fs * 32 + grp * 8);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            if (kb <= 2 * qh + qb) TT::mma(ls[kb][qb], fa, pq[hv][qb][fs]);
        }
      }
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        frag pf[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int qblk = 2 * qh + qb;
          const float sh = __builtin_amdgcn_exp2f(-0.5f * m0[hv][qb]);  // 2^-m0 as two factors
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int kb = 2 * hs + e / 4, i = e % 4;
            // key p vs query r: p > r on blocks past the query block, and past the diagonal
            // (qblk is a constant at D = 64, wave-uniform at D = 128: scalar branches)
            float pv;
            if (kb > qblk)
              pv = __builtin_amdgcn_exp2f(s[kb][qb][i] * c1 - m0[hv][qb]);
            else if (kb < qblk)
              pv = (ls[kb][qb][i] * sh) * sh;
            else
              pv = dmask[i] ? (ls[kb][qb][i] * sh) * sh : __builtin_amdgcn_exp2f(s[kb][qb][i] * c1 - m0[hv][qb]);
            pf[qb][e] = TT::from_f(pv);
          }
        }
#pragma unroll
        for (int db = 0; db < NB; ++db) {
          const frag va = SV::load8(L + C::R_VP, db * 16 + r16, hs * 32 + grp * 8);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) TT::mma(o[hv][db][qb], va, pf[qb]);
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) TT::mma(o[hv][NB][qb], nsel[hs], pf[qb]);
      }
    }
  }

  // ---- 5. the compact tiles: tile t in stage t % 4; tiles 1 and 2 are issued once every
  //      wave is done with the window regions, tile t + 3 in step t (into the stage of tile
  //      t - 1, free after the step's barrier). Step t waits for its own copies of tile t
  //      (those of tiles t + 1 and t + 2 may still be in flight). -------------------------
  if (nt_comp > 0) {
    lds_barrier();  // every wave is done with the window regions
    if (1 < nt_comp) issue(1, 1);
    if (2 < nt_comp) issue(2, 2);
    auto step = [&](int t, auto ragged) {
      constexpr bool RAGGED = decltype(ragged)::value;
      if (t + 2 < nt_comp)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * C::NL));
      else if (t + 1 < nt_comp)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::NL));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      lds_barrier();
      if (t + 3 < nt_comp) issue(t + 3, (t + 3) & 3);
      f32x4 sc[HV][4][QB];
      qk_tile_hv<T, D, QB, HV>(L + C::stage_off(t & 3), qf, sc);
      if constexpr (RAGGED) {
        uint32_t kw[QB];
        const uint32_t rw = range_word(0, n_comp - t * 64 - 1);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) kw[qb] = rw;
#pragma unroll
        for (int hv = 0; hv < HV; ++hv) mask_tile<QB>(sc[hv], kw);
      }
      sm_exp_pv_ones_hv<T, D, QB, HV>(sc, L + C::stage_off(t & 3) + KT, o, m0, c1);
    };
    const int nt_full = n_comp / 64;
    for (int t = 0; t < nt_full; ++t) step(t, std::false_type{});
    if (nt_full < nt_comp) step(nt_full, std::true_type{});
  }

  // ---- 6. normalise, stage in LDS as [position][4 heads x D], store whole rows -----------
  using SO = Swz<T, 4 * D>;
  __builtin_amdgcn_s_waitcnt(0);  // no copy into LDS is left in flight (an absent tile 0's included)
  lds_barrier();                  // every wave is done with the tiles
#pragma unroll
  for (int hv = 0; hv < HV; ++hv)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float lt = o[hv][NB][qb][0];
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const int r = (half0 + hv) * 32 + qb * 16 + r16;
#pragma unroll
      for (int db = 0; db < NB; ++db) {
        typename TT::quad ov;
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = TT::from_f(o[hv][db][qb][i] * inv);
        *reinterpret_cast<typename TT::quad*>(L + SO::off(r, slot * D + db * 16 + 4 * grp)) = ov;
      }
    }
  __syncthreads();
  T* out = static_cast<T*>(a.out) + ((b * T_ + t0) * d.Hq + rh * d.Gr + gs * 4) * D;
  constexpr int GPR = 4 * D / 8;  // 16-byte granules per output row
#pragma unroll
  for (int j = 0; j < 64 * GPR / C::NTHR; ++j) {
    const int idx = j * C::NTHR + tid, r = idx / GPR, col = (idx % GPR) * 8;
    if (r < nvalid) TT::store8(out + static_cast<long long>(r) * d.Hq * D + col, SO::load8(L, r, col));
  }
}

template <typename T, int D>
static hipError_t attn_ff(const AttnArgs& a, hipStream_t s) {
  using C = FF<D>;
  const dim3 grid(a.d.nC * a.d.B * a.d.Hr * a.gsplit);
  if (C::LDS_BYTES > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_ff_kernel<T, D>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  hipLaunchKernelGGL((attn_ff_kernel<T, D>), grid, dim3(C::NTHR), C::LDS_BYTES, s, a);
  return hipGetLastError();
}

template <typename T, int D, int DF, int NH, bool BAND>
static hipError_t attn_nhb(const AttnArgs& a, hipStream_t s) {
  using C = AttnCfg<T, D, DF, NH>;
  const int P = a.d.B * a.d.Hr * a.gsplit * C::QSPLIT;
  dim3 grid(a.d.nC * P);
  if (C::LDS_BYTES > 65536)  // opt in to more than 64 KiB of LDS (gfx950 has 160 KiB per CU)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_kernel<T, D, DF, NH, BAND>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  hipLaunchKernelGGL((attn_kernel<T, D, DF, NH, BAND>), grid, dim3(C::NTHR), C::LDS_BYTES, s, a);
  return hipGetLastError();
}

template <typename T, int D, int DF, int NH>
static hipError_t attn_nh(const AttnArgs& a, hipStream_t s) {
  return band_chunks(a.d.window) >= 2 ? attn_nhb<T, D, DF, NH, true>(a, s) : attn_nhb<T, D, DF, NH, false>(a, s);
}

template <typename T, int D, int DF>
static hipError_t attn_t(const AttnArgs& a, hipStream_t s) {
  // the fixed-frame kernel: bf16, head_dim = feat_dim, window = chunk, groups of four
  if constexpr (sizeof(T) == 2 && D == DF)
    if (a.nw == 4 && a.d.window == kChunk && a.d.Gr % 4 == 0) return attn_ff<T, D>(a, s);
  if (a.nw == 4) return attn_nh<T, D, DF, 4>(a, s);
  if (a.nw == 2) return attn_nh<T, D, DF, 2>(a, s);
  if (a.nw == 1) return attn_nh<T, D, DF, 1>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  const Dims& dd = a.d;
  if (dd.bf16) {
    if (dd.D == 64 && dd.DF == 64) return attn_t<bf16, 64, 64>(a, s);
    if (dd.D == 64 && dd.DF == 128) return attn_t<bf16, 64, 128>(a, s);
    if (dd.D == 128 && dd.DF == 64) return attn_t<bf16, 128, 64>(a, s);
    if (dd.D == 128 && dd.DF == 128) return attn_t<bf16, 128, 128>(a, s);
  } else {
    if (dd.D == 64 && dd.DF == 64) return attn_t<float, 64, 64>(a, s);
    if (dd.D == 64 && dd.DF == 128) return attn_t<float, 64, 128>(a, s);
    if (dd.D == 128 && dd.DF == 64) return attn_t<float, 128, 64>(a, s);
    if (dd.D == 128 && dd.DF == 128) return attn_t<float, 128, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace still
