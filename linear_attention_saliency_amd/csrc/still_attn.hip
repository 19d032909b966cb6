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
// tile, in a four-stage LDS pipeline whose copies run straight from memory into LDS. The
// running max is refreshed only when a tile's max exceeds it by more than kLazy = 32 (log2
// units): P and the accumulators keep fp32's exponent range (bf16 has it too), so terms up
// to 2^32 stay exact in relative terms and every sum stays finite. A per-tile bound
// |q| max|k| skips even the max pass when the max cannot move that far.
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
#include "still_launch.hpp"
#include "still_layout.hpp"
#include "still_route.hpp"

namespace still {

// lazy running max: rescale only when a score exceeds the running max by more than this
// (log2 units)
constexpr float kLazy = 32.f;

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

// Compact tiles: their K rows carry the factor log2(e)/sqrt(D), and the K Q^T product
// starts from the accumulator value -m (the running max of each query column), so the
// scores leave the MFMA as s = a_ij log2(e) - m and P = 2^s needs no VALU before the exp.
template <typename T, int D, int QB>
__device__ __forceinline__ void qk_tile_shifted(const T* lk, const typename Tr<T>::frag (&qf)[QB][D / 32],
                                                const f32x4 (&mneg)[QB], f32x4 (&s)[4][QB]) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mneg[qb];
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const typename Tr<T>::frag ka = Swz<T, D>::load8(lk, kb * 16 + r16, ks * 32 + grp * 8);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) Tr<T>::mma(s[kb][qb], ka, qf[qb][ks]);
    }
  }
}

// Running-max update for shifted scores: a column moves only if its tile max exceeds kLazy
// (2^kLazy is the largest P the accumulators then see); the accumulators are rescaled, the
// tile's scores and the column's -m re-based. Rare after the first tiles.
template <int D, int QB>
__device__ __forceinline__ void sm_max_shifted(f32x4 (&s)[4][QB], f32x4 (&o)[D / 16 + 1][QB], float (&m_run)[QB],
                                               f32x4 (&mneg)[QB]) {
  bool need_any = false;
  float dm[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float tm = -kInf;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) tm = fmaxf(tm, s[kb][qb][i]);
    tm = xor_max_groups(tm);
    const bool need = tm > kLazy;
    dm[qb] = need ? tm : 0.f;
    need_any |= need;
  }
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(need_any) != 0, 0)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float alpha = __builtin_amdgcn_exp2f(-dm[qb]);
      m_run[qb] += dm[qb];
      mneg[qb] -= dm[qb];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) s[kb][qb] -= dm[qb];
#pragma unroll
      for (int db = 0; db <= D / 16; ++db) o[db][qb] *= alpha;
    }
  }
}

// P = 2^s (shifted scores), then O^T += V^T P^T as in sm_exp_pv.
template <typename T, int D, int QB>
__device__ __forceinline__ void sm_exp_pv_shifted(const f32x4 (&s)[4][QB], const T* lv, f32x4 (&o)[D / 16 + 1][QB]) {
  using TT = Tr<T>;
  using frag = typename TT::frag;
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
  frag one;
#pragma unroll
  for (int e = 0; e < 8; ++e) one[e] = TT::from_f(1.0f);
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) {
    frag pf[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[qb][e] = TT::from_f(__builtin_amdgcn_exp2f(s[2 * hs + e / 4][qb][e % 4]));
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

template <typename T, int D, int DF, int NH>
struct AttnCfg {
  static constexpr int QW = 32;                // queries per wave (one query slice)
  static constexpr int QB = QW / 16;           // 16-query blocks per wave
  static constexpr int KT = 64 * D, FT = 64 * DF, VT = D * 64;  // elements of a K, phi(K), V^T tile
  static constexpr int STAGE = KT + VT;        // one compact tile (K then V^T)
  // the prefix state (S^T [D][DF] in the layer's dtype) goes through LDS where it fits
  // beside the tiles: at D = d_f = 64 (two workgroups per CU) and at D = 128 (one, with
  // both query slices: 8 waves read one copy instead of 8)
  static constexpr bool STATE_LDS = (D == 64 && DF == 64) || D == 128;
  static constexpr int ST = STATE_LDS ? D * DF : 0;
  // LDS regions of the fixed part (element offsets); compact stages 1 and 2 reuse them
  static constexpr int R_PHIP = 0, R_PHIC = FT, R_VP = 2 * FT, R_VC = 2 * FT + VT;
  static constexpr int R_KC = 2 * FT + 2 * VT, R_KP = R_KC + KT, R_ST = R_KP + KT;
  // compact pipeline: 4 stages; stage 0 after the fixed regions, stages 1..3 over them
  static constexpr int NSTAGE = 4;
  static constexpr int R_P0 = R_ST + ST > 3 * STAGE ? R_ST + ST : 3 * STAGE;
  static constexpr int LDS_BYTES = (R_P0 + STAGE) * static_cast<int>(sizeof(T));
  static __device__ __forceinline__ int stage_off(int s) { return s == 0 ? R_P0 : (s - 1) * STAGE; }
  // Query slices per workgroup. Where two workgroups fit in a CU's LDS (two 80 KiB
  // halves) each takes one slice, and the pair hides each other's waits. Where only one
  // fits (head_dim 128, or fp32) it takes both slices with twice the waves, so every SIMD
  // still runs two waves and every staged tile serves the whole chunk.
  static constexpr int QS = LDS_BYTES > 80 * 1024 ? 2 : 1;
  static constexpr int QSPLIT = 64 / QW / QS;  // workgroups per chunk
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

template <typename T, int D, int DF, int NH>
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
  const int BHG = d.B * d.Hkv * a.gsplit;
  const int P = BHG * C::QSPLIT;
  const int c = d.nC - 1 - static_cast<int>(blockIdx.x) / P;
  const int pi = static_cast<int>(blockIdx.x) % P;
  const int bhg = pi % BHG, qsb = pi / BHG;  // block of C::QS query slices
  const int gs = bhg % a.gsplit, bh = bhg / a.gsplit;
  const int b = bh / d.Hkv, h = bh % d.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: lets addresses stay scalar
  const int g = gs * NH + wave % NH;
  const int qoff = (qsb * C::QS + wave / NH) * QW;  // first query of this wave within the chunk
  const bool head_ok = g < d.G;
  const int hq = h * d.G + (head_ok ? g : d.G - 1);
  const long long T_ = d.T;
  const long long t0 = static_cast<long long>(c) * kChunk;
  const int nvalid = static_cast<int>(T_ - t0 < kChunk ? T_ - t0 : kChunk);
  const float c1 = kLog2e / sqrtf(static_cast<float>(D));
  const int win = d.window;
  const bool has_prev = c >= 1;
  const bool la_cur = win < kChunk;  // chunk c holds linear keys (p <= r - w)
  const int n_comp = c >= 2 ? (c - 1) * d.topk : 0;  // compact rows of chunks <= c-2
  const int nt_comp = (n_comp + 63) / 64;
  const T* kb_ptr = ksel + static_cast<long long>(bh) * a.ntiles_sel * 64 * D;
  const T* vb_ptr = vselT + static_cast<long long>(bh) * a.ntiles_sel * D * 64;
  // compact tile t -> LDS stage (asynchronous); K rows [64][D] and V^T rows [D][64] of a
  // tile are contiguous, so one resource per buffer covers every tile of this (b, h)
  DmaTile<T, D, 64, NW> dk;
  DmaTile<T, 64, D, NW> dv;
  dk.init(D);
  dv.init(64);
  const auto krs = make_rsrc(kb_ptr, static_cast<uint32_t>(a.ntiles_sel) * C::KT * static_cast<int>(sizeof(T)));
  const auto vrs = make_rsrc(vb_ptr, static_cast<uint32_t>(a.ntiles_sel) * C::VT * static_cast<int>(sizeof(T)));
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
  frag qf[QB][D / 32];
  {
    const long long q0 = t0 + qoff;  // first query row of this wave
    const int qrow = d.Hq * D;        // elements from one position to the next
    const long long nq = T_ - q0 < QW ? T_ - q0 : QW;
    const auto qrs = make_rsrc(q + ((b * T_ + (nq > 0 ? q0 : 0)) * d.Hq + hq) * D,
                               nq > 0 ? static_cast<uint32_t>(((nq - 1) * qrow + D) * static_cast<int>(sizeof(T))) : 0u);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        qf[qb][ks] = TT::bload8(qrs, ((qb * 16 + r16) * qrow + ks * 32 + grp * 8) * static_cast<int>(sizeof(T)), 0);
  }
  // W_h rows fb*16 + r16 (A operand of phi(q)): held in registers where they fit, else
  // copied once into compact stage 0 (free until the first compact tile) for all waves
  const T* Wh = w + static_cast<long long>(h) * DF * D;
  constexpr bool W_EARLY = D == 64 && DF == 64;
  frag wq[W_EARLY ? DF / 16 : 1][D / 32];
  if constexpr (W_EARLY) {
#pragma unroll
    for (int fb = 0; fb < DF / 16; ++fb)
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) wq[fb][ks] = TT::load8(Wh + (fb * 16 + r16) * D + ks * 32 + grp * 8);
  }
  // z of the prefix state of chunks <= c-2 (8 consecutive permuted features per lane group):
  // the A operand of the denominator, the same in every row
  const T* Sg = static_cast<const T*>(a.states) + (static_cast<long long>(bh) * d.nC + (c >= 2 ? c - 2 : 0)) * d.R;
  frag zf[DF / 32];
  {
    const auto zrs = make_rsrc(Sg + DF * D, c >= 2 ? DF * static_cast<uint32_t>(sizeof(T)) : 0u);
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
    dma_tile<T, DF, 64, NW>(L + C::R_PHIP, phik + (static_cast<long long>(bh) * T_ + tp) * DF, DF, has_prev ? 64 : 0);
    dma_tile<T, 64, D, NW>(L + C::R_VP, vT + (static_cast<long long>(bh) * d.nC + cp) * D * 64, 64, has_prev ? D : 0);
    dma_tile<T, D, 64, NW>(L + C::R_KP, kp, kvs, has_prev && win >= 1 ? 64 : 0);
    dma_tile<T, DF, 64, NW>(L + C::R_PHIC, phik + (static_cast<long long>(bh) * T_ + t0) * DF, DF, la_cur ? nvalid : 0);
    dma_tile<T, 64, D, NW>(L + C::R_VC, vT + (static_cast<long long>(bh) * d.nC + c) * D * 64, 64, D);
    dma_tile<T, D, 64, NW>(L + C::R_KC, kc, kvs, win >= 1 ? nvalid : 0);
    if constexpr (C::STATE_LDS)
      dma_tile<T, DF, D, NW>(L + C::R_ST, Sg, DF, c >= 2 ? D : 0);
    if constexpr (W_EARLY) {
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

  f32x4 o[NB + 1][QB];
  float m_run[QB];
  float qn[QB];  // |q| c1: with |k| <= kmax, every logit of a tile is <= qn kmax
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db <= NB; ++db) o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // window = chunk takes a fast path for the masks and handles chunk c-1's linear keys
  // together with its window tile (head_dim 64; at 128 the extra live registers spill)
  const bool fast = D == 64 && win == kChunk;
  frag pq[QB][DF / 32];  // phi(q): B-operand fragments (PK over f)
  uint64_t selprev;
  // =============================== phase 1: linear attention ===========================
  {
    // phi(q) = |q| m / |m|, m = elu(W_h q) + 1; wfrag(fb, ks) gives the W_h fragment
    auto phi_q = [&](auto wfrag) {
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
      for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xv = TT::to_f(qf[qb][ks][e]);
          x2 += xv * xv;
        }
      m2 = xor_sum_groups(m2);
      x2 = xor_sum_groups(x2);
      qn[qb] = __builtin_amdgcn_sqrtf(x2) * c1 * 1.001f;  // |q| in logit units, with slack for rounding
      const float sc = norm_ratio(x2, m2);
#pragma unroll
      for (int fs = 0; fs < DF / 32; ++fs)
#pragma unroll
        for (int e = 0; e < 8; ++e) pq[qb][fs][e] = TT::from_f(pacc[2 * fs + e / 4][e % 4] * sc);
    }
    };
    if constexpr (W_EARLY) {
      // phi(q) before the wait (it overlaps the copies); keep the scheduler from moving it
      // past the wait
      phi_q([&](int fb, int ks) { return wq[fb][ks]; });
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();  // every region copied at the start has landed
    } else {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();  // every region copied at the start has landed, W_h among them
      phi_q([&](int fb, int ks) { return Swz<T, D>::load8(L + C::stage_off(0), fb * 16 + r16, ks * 32 + grp * 8); });
      __syncthreads();  // every wave is done with W_h: stage 0 takes compact tile 0
      dk.issue(L + C::stage_off(0), make_rsrc(kb_ptr, nt_comp > 0 ? C::KT * static_cast<int>(sizeof(T)) : 0u), 0);
      dv.issue(L + C::stage_off(0) + C::KT, make_rsrc(vb_ptr, nt_comp > 0 ? C::VT * static_cast<int>(sizeof(T)) : 0u), 0);
    }
    selprev = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(selv[1]))) << 32) |
              static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(selv[0]));

    // prefix state of chunks <= c-2, stored as S^T[d][pk_pos(f)]: each A-operand fragment
    // (row d, the 8 features a lane group holds) is 8 consecutive elements
    if (c >= 2) {
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
          for (int qb = 0; qb < QB; ++qb) TT::mma(o[db][qb], sa, pq[qb][fs]);
        }
        // the denominator phi(q).z on the row-sum block: every row of its A operand is z,
        // so each of its entries ends up holding the whole dot product
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) TT::mma(o[NB][qb], zf[fs], pq[qb][fs]);
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
          for (int qb = 0; qb < QB; ++qb) TT::mma(ls[kb][qb], fa, pq[qb][fs]);
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
          for (int qb = 0; qb < QB; ++qb) TT::mma(o[db][qb], va, pf[ks][qb]);
        }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) TT::mma(o[NB][qb], ones, pf[ks][qb]);  // their denominator
    }
    // the linear branch becomes one online-softmax entry: log-weight log2(D), value N / D
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float dt = o[NB][qb][0];
      const float inv = dt > 0.f ? __builtin_amdgcn_rcpf(dt) : 0.f;
#pragma unroll
      for (int db = 0; db < NB; ++db) o[db][qb] *= inv;
      m_run[qb] = dt > 0.f ? __log2f(dt) : -kInf;
      const float l0 = dt > 0.f ? 1.f : 0.f;
      o[NB][qb] = f32x4{l0, l0, l0, l0};
    }
  }

  // =============================== phase 2: softmax tiles ==============================
  // 2a. the window: chunk c (r - w < p <= r), chunk c-1 (p > r + 64 - w, or selected)
  if (fast) {
    if (qoff == 0)
      window_fast<T, D, DF, QB, 0>(L + C::R_KC, L + C::R_VC, L + C::R_KP, L + C::R_PHIP, L + C::R_VP, has_prev, selprev,
                                   qf, pq, o, m_run, c1);
    else
      window_fast<T, D, DF, QB, QW>(L + C::R_KC, L + C::R_VC, L + C::R_KP, L + C::R_PHIP, L + C::R_VP, has_prev,
                                    selprev, qf, pq, o, m_run, c1);
  } else if (win >= 1) {
    f32x4 s[4][QB];
    uint32_t kw[QB];
    qk_tile<T, D, QB>(L + C::R_KC, qf, s);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int r = qoff + qb * 16 + r16;
      kw[qb] = range_word(r - win + 1, r);
    }
    mask_tile<QB>(s, kw);
    sm_max<D, QB>(s, o, m_run, c1);
    sm_exp_pv<T, D, QB>(s, L + C::R_VC, o, m_run, c1);
    if (has_prev) {
      const uint32_t selw = bits_word(selprev);
      qk_tile<T, D, QB>(L + C::R_KP, qf, s);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int r = qoff + qb * 16 + r16;
        kw[qb] = range_word(r + 65 - win, 63) | selw;
      }
      mask_tile<QB>(s, kw);
      sm_max<D, QB>(s, o, m_run, c1);
      sm_exp_pv<T, D, QB>(s, L + C::R_VP, o, m_run, c1);
    }
  }

  // 2b. the compact cache: selected rows of chunks <= c-2, unmasked except a ragged end.
  //     Tile t lives in stage t % 4. Tile 0 was copied at the start; tiles 1..3 go into
  //     the fixed regions once every wave is done with them, and tile t+3 is issued in step
  //     t, two steps ahead of its first use. In step t each wave waits for its own copies of
  //     tile t+1 (those of tile t+2 may still be in flight), the barrier makes tile t+1
  //     visible and frees tile t-1's stage; the K Q^T product of tile t+1 (MFMA) then issues
  //     interleaved with the softmax of tile t (VALU). Rows past the last compact row of a
  //     ragged tile are copied too (they lie inside the buffer; their scores are masked and
  //     their V^T columns are zero or finite).
  if (nt_comp > 0) {
    f32x4 mneg[QB];  // -m per query column, the starting accumulator of K Q^T
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mneg[qb] = f32x4{-m_run[qb], -m_run[qb], -m_run[qb], -m_run[qb]};
    // Tiles whose key-norm bound might move the running max, one bit each: the max can only
    // move if some query's |q| max|k| exceeds it by more than kLazy. Decided here for all
    // tiles at once, conservatively (the wave's largest |q| against its smallest running max,
    // which only grows), so a step tests one scalar bit; tiles from 256 on are always checked.
    uint64_t mayfar[4];
    {
      float qmax = qn[0], mmin = m_run[0];
#pragma unroll
      for (int qb = 1; qb < QB; ++qb) {
        qmax = fmaxf(qmax, qn[qb]);
        mmin = fminf(mmin, m_run[qb]);
      }
      qmax = wave_max64(qmax);
      mmin = -wave_max64(-mmin);
#pragma unroll
      for (int j = 0; j < 4; ++j) mayfar[j] = __builtin_amdgcn_ballot_w64(qmax * tb[j] > mmin + kLazy);
    }
    f32x4 sa[4][QB], sb[4][QB];
    if constexpr (!W_EARLY) {  // tile 0 was copied after phi(q)
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    qk_tile_shifted<T, D, QB>(L + C::stage_off(0), qf, mneg, sa);  // tile 0 has landed
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
      const int tj = t >> 6;
      const uint64_t fw = tj == 0 ? mayfar[0] : tj == 1 ? mayfar[1] : tj == 2 ? mayfar[2] : tj == 3 ? mayfar[3] : ~0ull;
      if ((fw >> (t & 63)) & 1ull) sm_max_shifted<D, QB>(s_cur, o, m_run, mneg);
      qk_tile_shifted<T, D, QB>(L + C::stage_off((t + 1) & 3), qf, mneg, s_next);  // after the last tile: unused
      sm_exp_pv_shifted<T, D, QB>(s_cur, L + C::stage_off(t & 3) + C::KT, o);
    };
    for (int t = 0; t < nt_comp; t += 2) {
      step(t, sa, sb);
      if (t + 1 < nt_comp) step(t + 1, sb, sa);
    }
  }

  // ---- epilogue: divide by the shared normaliser, write [B,T,Hq,D] ------------------
  T* out = static_cast<T*>(a.out);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = o[NB][qb][0];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int r = qoff + qb * 16 + r16;
    if (head_ok && r < nvalid) {
      T* dst = out + ((b * T_ + t0 + r) * d.Hq + hq) * D + 4 * grp;
#pragma unroll
      for (int db = 0; db < NB; ++db) {
        typename TT::quad ov;
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = TT::from_f(o[db][qb][i] * inv);
        *reinterpret_cast<typename TT::quad*>(dst + db * 16) = ov;
      }
    }
  }
}

template <typename T, int D, int DF, int NH>
static hipError_t attn_nh(const AttnArgs& a, hipStream_t s) {
  using C = AttnCfg<T, D, DF, NH>;
  const int P = a.d.B * a.d.Hkv * a.gsplit * C::QSPLIT;
  dim3 grid(a.d.nC * P);
  if (C::LDS_BYTES > 65536)  // opt in to more than 64 KiB of LDS (gfx950 has 160 KiB per CU)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_kernel<T, D, DF, NH>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  hipLaunchKernelGGL((attn_kernel<T, D, DF, NH>), grid, dim3(C::NTHR), C::LDS_BYTES, s, a);
  return hipGetLastError();
}

template <typename T, int D, int DF>
static hipError_t attn_t(const AttnArgs& a, hipStream_t s) {
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
  } else if (dd.D == 64 && dd.DF == 64) {
    return attn_t<float, 64, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace still
