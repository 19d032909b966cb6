// Fused softmax + linear attention of the STILL prefill, with the shared normaliser.
//
// One workgroup per (chunk c, batch b, KV head h, head split, query split). The
// workgroup packs up to four query heads of the group (GQA): every staged key/value tile
// serves all of them. Wave w handles query head w of the head split, for the QW
// consecutive queries of its query split (64 / QW query splits per chunk, so two
// independent workgroups can share a CU and hide each other's barriers).
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
// tile, with the next tile's global loads in flight while the current one is computed
// from a double-buffered LDS stage. The running max is refreshed only when a tile's max
// exceeds it by more than 8 (log2 units), so the rescale is rare.
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
// by more than 8 (log2 units); the accumulators (row-sum block included) are rescaled
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
    const bool need = tm > m_run[qb] + 8.f;
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

template <typename T, int D, int DF, int QW, int NH>
struct AttnCfg {
  static constexpr int QB = QW / 16;           // 16-query blocks per wave
  static constexpr int QSPLIT = 64 / QW;       // workgroups per chunk, one per query slice
  static constexpr int NTHR = 64 * NH;         // threads per workgroup: one wave per head
  static constexpr int KBUF = 64 * (D > DF ? D : DF);  // elements of one K / phi(K) stage
  static constexpr int VBUF = D * 64;                  // elements of one V^T stage
  static constexpr int NSTAGE = 3;
  static constexpr int LDS_BYTES = NSTAGE * (KBUF + VBUF) * static_cast<int>(sizeof(T));
};

template <typename T, int D, int DF, int QW, int NH>
__global__ __launch_bounds__(64 * NH, 2) void attn_kernel(AttnArgs a) {
  using C = AttnCfg<T, D, DF, QW, NH>;
  constexpr int QB = C::QB, NTHR = C::NTHR;
  using SK = Swz<T, D>;    // K tile: 64 keys x D
  using SF = Swz<T, DF>;   // phi(K) tile: 64 keys x DF; prefix state: D rows x DF
  using SV = Swz<T, 64>;   // V^T tile: D rows x 64 keys
  constexpr int NB = D / 16;  // output blocks; block NB holds the row sums
  using TT = Tr<T>;
  using frag = typename TT::frag;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  T* ldsK = reinterpret_cast<T*>(lds_raw);        // NSTAGE stages of KBUF
  T* ldsV = ldsK + C::NSTAGE * C::KBUF;            // NSTAGE stages of VBUF

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
  const int bhg = pi % BHG, qs = pi / BHG;
  const int gs = bhg % a.gsplit, bh = bhg / a.gsplit;
  const int b = bh / d.Hkv, h = bh % d.Hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
  const int g = gs * NH + wave;
  const int qoff = qs * QW;  // first query of this wave within the chunk
  const bool head_ok = g < d.G;
  const int hq = h * d.G + (head_ok ? g : d.G - 1);
  const long long T_ = d.T;
  const long long t0 = static_cast<long long>(c) * kChunk;
  const int nvalid = static_cast<int>(T_ - t0 < kChunk ? T_ - t0 : kChunk);
  const float c1 = kLog2e / sqrtf(static_cast<float>(D));
  const int win = d.window;

  // ---- queries: B-operand fragments (SK over d) -------------------------------------
  frag qf[QB][D / 32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const long long pos = t0 + qoff + qb * 16 + r16;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      qf[qb][ks] = pos < T_ ? TT::load8(q + ((b * T_ + pos) * d.Hq + hq) * D + ks * 32 + grp * 8) : TT::zero();
  }

  f32x4 o[NB + 1][QB];
  float m_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db <= NB; ++db) o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // =============================== phase 1: linear attention ===========================
  {
    // phi(q) = |q| m / |m|, m = elu(W_h q) + 1: B-operand fragments (PK over f)
    frag pq[QB][DF / 32];
    const T* Wh = w + static_cast<long long>(h) * DF * D;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      f32x4 pacc[DF / 16];
#pragma unroll
      for (int fb = 0; fb < DF / 16; ++fb) {
        pacc[fb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
          TT::mma(pacc[fb], TT::load8(Wh + (fb * 16 + r16) * D + ks * 32 + grp * 8), qf[qb][ks]);
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
      const float sc = m2 > 0.f ? sqrtf(x2) / sqrtf(m2) : 0.f;
#pragma unroll
      for (int fs = 0; fs < DF / 32; ++fs)
#pragma unroll
        for (int e = 0; e < 8; ++e) pq[qb][fs][e] = TT::from_f(pacc[2 * fs + e / 4][e % 4] * sc);
    }

    float den[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) den[qb] = 0.f;
    // prefix state of chunks <= c-2: staged in LDS as S^T[d][pk_pos(f)] (rounded to T)
    // and z[f] (fp32), with coalesced loads, then contracted on MFMA
    if (c >= 2) {
      const float* S = a.states + (static_cast<long long>(bh) * d.nC + (c - 2)) * d.R;
      T* st = ldsK;  // D rows of DF elements: fits in the two K stages (128 rows of >= DF)
      float* zs = reinterpret_cast<float*>(ldsV);
      for (int idx = tid; idx < DF * D / 4; idx += NTHR) {
        const int f = idx / (D / 4), d4 = (idx % (D / 4)) * 4;
        const f32x4 x = *reinterpret_cast<const f32x4*>(S + f * D + d4);
#pragma unroll
        for (int j = 0; j < 4; ++j) st[SF::off(d4 + j, pk_pos(f))] = TT::from_f(x[j]);
      }
      for (int idx = tid; idx < DF; idx += NTHR) zs[idx] = S[DF * D + idx];
      __syncthreads();
#pragma unroll
      for (int fs = 0; fs < DF / 32; ++fs) {
#pragma unroll
        for (int db = 0; db < NB; ++db) {
          const frag sa = SF::load8(st, db * 16 + r16, fs * 32 + grp * 8);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) TT::mma(o[db][qb], sa, pq[qb][fs]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float zf = zs[fs * 32 + 16 * (e / 4) + 4 * grp + (e % 4)];
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) den[qb] += TT::to_f(pq[qb][fs][e]) * zf;
        }
      }
      __syncthreads();  // the stages are reused below
    }
    // linear keys of chunk c-1 (p <= r + 64 - w, unselected) and of chunk c (p <= r - w)
    const uint64_t selprev = c >= 1 ? a.selmask[static_cast<long long>(bh) * d.nC + c - 1] : 0ull;
    const int cc_lo = c >= 1 ? c - 1 : c;
    const int cc_hi = win < kChunk ? c : c - 1;
    for (int cc = cc_lo; cc <= cc_hi; ++cc) {
      const int st = cc - cc_lo;  // LDS stage
      T* lk = ldsK + st * C::KBUF;
      T* lv = ldsV + st * C::VBUF;
      const int nk = cc == c ? nvalid : kChunk;
      for (int idx = tid; idx < 64 * (DF / 8); idx += NTHR) {
        const int p = idx / (DF / 8), c8 = idx % (DF / 8);
        frag fx = TT::zero();
        if (p < nk) fx = TT::load8(phik + (static_cast<long long>(bh) * T_ + static_cast<long long>(cc) * kChunk + p) * DF + c8 * 8);
        SF::store8(lk, p, c8 * 8, fx);
      }
      for (int idx = tid; idx < D * 8; idx += NTHR) {
        const int dd = idx / 8, c8 = idx % 8;
        SV::store8(lv, dd, c8 * 8, TT::load8(vT + ((static_cast<long long>(bh) * d.nC + cc) * D + dd) * 64 + c8 * 8));
      }
      __syncthreads();
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
      // linear keys: chunk c-1: p <= r + 64 - w and unselected; chunk c: p <= r - w
      const uint32_t selw = cc == c ? 0u : bits_word(selprev);
      frag pf[2][QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int r = qoff + qb * 16 + r16;
        const uint32_t lw = range_word(0, cc == c ? r - win : r + 64 - win) & ~selw;
        float pv[4][4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = (lw & (1u << (kb * 4 + i))) ? ls[kb][qb][i] : 0.f;
            pv[kb][i] = x;
            den[qb] += x;
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
    }
    // the linear branch becomes one online-softmax entry: log-weight log2(D), value N / D
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float dt = xor_sum_groups(den[qb]);
      const float inv = dt > 0.f ? 1.f / dt : 0.f;
#pragma unroll
      for (int db = 0; db < NB; ++db) o[db][qb] *= inv;
      m_run[qb] = dt > 0.f ? __log2f(dt) : -kInf;
      const float l0 = dt > 0.f ? 1.f : 0.f;
      o[NB][qb] = f32x4{l0, l0, l0, l0};
    }
    __syncthreads();  // LDS stages are reused by phase 2
  }

  // =============================== phase 2: softmax tiles ==============================
  const int n_comp = c >= 2 ? (c - 1) * d.topk : 0;  // compact rows of chunks <= c-2
  const int nt_comp = (n_comp + 63) / 64;
  constexpr int KLD = D / 8;                        // 8-element pieces per K row
  constexpr int NK16 = 64 * KLD;                    // pieces per K tile
  constexpr int NV16 = D * 8;                       // pieces per V^T tile
  constexpr int NPT = (NK16 + NV16 + NTHR - 1) / NTHR;
  // per-thread piece geometry, fixed across tiles: global offset within a tile, and the
  // tile row / column the piece lands on in LDS (K row = key, V^T row = d)
  long long goff[NPT];
  int prow[NPT], pcol[NPT];
  bool isk[NPT], live[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int idx = tid + i * NTHR;
    live[i] = idx < NK16 + NV16;
    isk[i] = idx < NK16;
    if (isk[i]) {
      const int p = idx / KLD, c8 = idx % KLD;
      goff[i] = static_cast<long long>(p) * D + c8 * 8;
      prow[i] = p;
      pcol[i] = c8 * 8;
    } else {
      const int j = idx - NK16, dd = j / 8, c8 = j % 8;
      goff[i] = static_cast<long long>(j) * 8;
      prow[i] = dd;
      pcol[i] = c8 * 8;
    }
  }
  const T* kb_ptr = ksel + static_cast<long long>(bh) * a.ntiles_sel * 64 * D;
  const T* vb_ptr = vselT + static_cast<long long>(bh) * a.ntiles_sel * D * 64;
  frag pre[NPT];  // a compact tile in flight (global -> registers -> LDS stage)
  auto issue = [&](int t) {
    const int rows = n_comp - t * 64;
    const T* kt = kb_ptr + static_cast<long long>(t) * 64 * D;
    const T* vt = vb_ptr + static_cast<long long>(t) * D * 64;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      frag x = TT::zero();
      if (live[i] && (isk[i] ? prow[i] < rows : true)) x = TT::load8((isk[i] ? kt : vt) + goff[i]);
      pre[i] = x;
    }
  };
  auto commit = [&](int stage) {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      if (!live[i]) continue;
      if (isk[i]) SK::store8(ldsK + stage * C::KBUF, prow[i], pcol[i], pre[i]);
      else SV::store8(ldsV + stage * C::VBUF, prow[i], pcol[i], pre[i]);
    }
  };

  // 2a. the window tiles: chunk c (causal) in stage 1, chunk c-1 (mixed) in stage 2.
  //     The first compact tile's loads are in flight meanwhile.
  if (win >= 1) {
    const int nct = c >= 1 ? 2 : 1;
    for (int ct = 0; ct < nct; ++ct) {
      T* lk = ldsK + (1 + ct) * C::KBUF;
      T* lv = ldsV + (1 + ct) * C::VBUF;
      const long long tb = ct == 0 ? t0 : t0 - 64;
      const int nk = ct == 0 ? nvalid : 64;
      for (int idx = tid; idx < 64 * (D / 8); idx += NTHR) {
        const int p = idx / (D / 8), c8 = idx % (D / 8);
        frag x = TT::zero();
        if (p < nk) x = TT::load8(kk + ((b * T_ + tb + p) * d.Hkv + h) * D + c8 * 8);
        SK::store8(lk, p, c8 * 8, x);
      }
      const T* src = vT + (static_cast<long long>(bh) * d.nC + (ct == 0 ? c : c - 1)) * D * 64;
      for (int idx = tid; idx < D * 8; idx += NTHR) {
        const int dd = idx / 8, c8 = idx % 8;
        SV::store8(lv, dd, c8 * 8, TT::load8(src + dd * 64 + c8 * 8));
      }
    }
  }
  if (nt_comp > 0) issue(0);
  __syncthreads();
  if (win >= 1) {
    f32x4 s[4][QB];
    uint32_t kw[QB];
    qk_tile<T, D, QB>(ldsK + C::KBUF, qf, s);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {  // chunk c: r - w < p <= r
      const int r = qoff + qb * 16 + r16;
      kw[qb] = range_word(r - win + 1, r);
    }
    mask_tile<QB>(s, kw);
    sm_max<D, QB>(s, o, m_run, c1);
    sm_exp_pv<T, D, QB>(s, ldsV + C::VBUF, o, m_run, c1);
    if (c >= 1) {
      const uint64_t selprev = a.selmask[static_cast<long long>(bh) * d.nC + c - 1];
      const uint32_t selw = bits_word(selprev);
      qk_tile<T, D, QB>(ldsK + 2 * C::KBUF, qf, s);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {  // chunk c-1: p > r + 64 - w, or selected
        const int r = qoff + qb * 16 + r16;
        kw[qb] = range_word(r + 65 - win, 63) | selw;
      }
      mask_tile<QB>(s, kw);
      sm_max<D, QB>(s, o, m_run, c1);
      sm_exp_pv<T, D, QB>(s, ldsV + 2 * C::VBUF, o, m_run, c1);
    }
  }

  // 2b. the compact cache: selected rows of chunks <= c-2, unmasked except a ragged end.
  //     Three LDS stages: while tile t's softmax runs, tile t+1 is already in LDS, so its
  //     K Q^T product (MFMA) is independent of the softmax (VALU) and issues interleaved
  //     with it; tile t+2 is in flight from global memory. One barrier per tile.
  if (nt_comp > 0) {
    commit(0);
    if (nt_comp > 1) issue(1);
    __syncthreads();
    f32x4 sa[4][QB], sb[4][QB];
    qk_tile<T, D, QB>(ldsK, qf, sa);
    auto step = [&](int t, f32x4 (&s_cur)[4][QB], f32x4 (&s_next)[4][QB]) {
      const int st = t % 3, stn = (t + 1) % 3;
      if (t + 1 < nt_comp) commit(stn);
      __syncthreads();
      if (t + 2 < nt_comp) issue(t + 2);
      const int nk = n_comp - t * 64;
      if (nk < 64) {
        uint32_t kw[QB];
        const uint32_t rw = range_word(0, nk - 1);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) kw[qb] = rw;
        mask_tile<QB>(s_cur, kw);
      }
      sm_max<D, QB>(s_cur, o, m_run, c1);
      qk_tile<T, D, QB>(ldsK + stn * C::KBUF, qf, s_next);  // the last tile reads a stale stage: unused
      sm_exp_pv<T, D, QB>(s_cur, ldsV + st * C::VBUF, o, m_run, c1);
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

template <typename T, int D, int DF, int QW, int NH>
static hipError_t attn_nh(const AttnArgs& a, hipStream_t s) {
  using C = AttnCfg<T, D, DF, QW, NH>;
  const int P = a.d.B * a.d.Hkv * a.gsplit * C::QSPLIT;
  dim3 grid(a.d.nC * P);
  if (C::LDS_BYTES > 65536)  // opt in to more than 64 KiB of LDS (gfx950 has 160 KiB per CU)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_kernel<T, D, DF, QW, NH>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  hipLaunchKernelGGL((attn_kernel<T, D, DF, QW, NH>), grid, dim3(C::NTHR), C::LDS_BYTES, s, a);
  return hipGetLastError();
}

template <typename T, int D, int DF, int QW>
static hipError_t attn_t(const AttnArgs& a, hipStream_t s) {
  if (a.nw == 4) return attn_nh<T, D, DF, QW, 4>(a, s);
  if (a.nw == 2) return attn_nh<T, D, DF, QW, 2>(a, s);
  if (a.nw == 1) return attn_nh<T, D, DF, QW, 1>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  const Dims& dd = a.d;
  if (dd.bf16) {
    if (dd.D == 64 && dd.DF == 64) return attn_t<bf16, 64, 64, 32>(a, s);
    if (dd.D == 64 && dd.DF == 128) return attn_t<bf16, 64, 128, 32>(a, s);
    if (dd.D == 128 && dd.DF == 64) return attn_t<bf16, 128, 64, 32>(a, s);
    if (dd.D == 128 && dd.DF == 128) return attn_t<bf16, 128, 128, 32>(a, s);
  } else if (dd.D == 64 && dd.DF == 64) {
    return attn_t<float, 64, 64, 32>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace still
