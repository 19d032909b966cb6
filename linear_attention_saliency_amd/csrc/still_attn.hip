// Fused softmax + linear attention of the STILL prefill, with the shared normaliser.
//
// One workgroup per (chunk c, batch b, KV head h, head split); wave w handles query head
// g = split*4 + w of the group for the chunk's 64 queries, so the 4 query heads share
// every staged key/value tile (GQA packing). For query i = 64c + r the key set splits as
// ([P1] paragraph before "STILL三大创新", sections "Chunk-Wise并行+延迟选择" and NP-Map;
// [P2] excerpt):
//   chunks <= c-2   selected rows (compact softmax cache, no mask) -> softmax;
//                   the others are folded in the prefix state (S, z) -> linear;
//   chunk c-1       p > r + 64 - w or selected -> softmax, the rest -> linear;
//   chunk c         p <= r: p > r - w -> softmax, the rest -> linear.
// Everything is computed transposed (S^T = K Q^T, O^T += V^T P^T) so that a query is a
// lane's column: row statistics need no cross-lane traffic beyond the 4 lane groups,
// and P leaves the softmax in exactly the register layout the PV product consumes.
// The running max starts at 0 (log2 units) and the linear-attention terms enter the
// same accumulators scaled by 2^-m, so out = (A + e^{-M} N_LA) / (Z + e^{-M} D_LA) with
// M = max(0, max logit) -- the shared-normaliser formula with an overflow-safe offset.
#include "still_launch.hpp"
#include "still_route.hpp"

namespace still {

template <typename T, int D, int DF>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  constexpr int LDK = pitch<T>(D);
  constexpr int LDV = pitch<T>(64);
  constexpr int LDF = pitch<T>(DF);
  constexpr int V8 = D / 8;
  constexpr int F8 = DF / 8;
  using TT = Tr<T>;
  using frag = typename TT::frag;

  __shared__ __attribute__((aligned(16))) T k_s[64 * LDK];
  __shared__ __attribute__((aligned(16))) T vt_s[D * LDV];
  __shared__ __attribute__((aligned(16))) T pk_s[64 * LDF];

  const Dims& d = a.d;
  const T* q = static_cast<const T*>(a.q);
  const T* kk = static_cast<const T*>(a.k);
  const T* vv = static_cast<const T*>(a.v);
  const T* w = static_cast<const T*>(a.w);
  const T* ksel = static_cast<const T*>(a.ksel);
  const T* vsel = static_cast<const T*>(a.vsel);
  const T* phik = static_cast<const T*>(a.phik);

  const int P = d.B * d.Hkv * a.gsplit;
  const int c = d.nC - 1 - static_cast<int>(blockIdx.x) / P;  // heaviest chunks first
  const int pi = static_cast<int>(blockIdx.x) % P;
  const int gs = pi % a.gsplit, bh = pi / a.gsplit;
  const int b = bh / d.Hkv, h = bh % d.Hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
  const int nthr = blockDim.x;
  const int g = gs * a.nw + wave;
  const bool head_ok = g < d.G;
  const int hq = h * d.G + (head_ok ? g : d.G - 1);
  const long long T_ = d.T;
  const long long t0 = static_cast<long long>(c) * kChunk;
  const int nvalid = static_cast<int>(T_ - t0 < kChunk ? T_ - t0 : kChunk);
  const float c1 = kLog2e / sqrtf(static_cast<float>(D));
  const int win = d.window;

  // ---- queries: B-operand fragments (SK over d) -------------------------------------
  frag qf[4][D / 32];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const long long pos = t0 + qb * 16 + r16;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      qf[qb][ks] = pos < T_ ? TT::load8(q + ((b * T_ + pos) * d.Hq + hq) * D + ks * 32 + grp * 8) : TT::zero();
  }

  // ---- phi(q): W_h Q^T on MFMA, elu+1, norm rescale; B-operand fragments (PK over f) --
  frag pq[4][DF / 32];
  {
    const T* Wh = w + static_cast<long long>(h) * DF * D;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
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
          const float mv = zv > 0.f ? zv + 1.f : expf(zv);
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
  }

  // ---- accumulators; linear attention over the prefix state of chunks <= c-2 ---------
  f32x4 o[D / 16][4];
  float m_run[4], l_run[4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    m_run[qb] = 0.f;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (c >= 2) {
    const float* S = a.states + (static_cast<long long>(bh) * d.nC + (c - 2)) * d.R;
    const float* z = S + DF * D;
#pragma unroll
    for (int fs = 0; fs < DF / 32; ++fs) {
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        frag sa;
#pragma unroll
        for (int e = 0; e < 8; ++e) sa[e] = TT::from_f(S[(fs * 32 + 16 * (e / 4) + 4 * grp + (e % 4)) * D + db * 16 + r16]);
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) TT::mma(o[db][qb], sa, pq[qb][fs]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float zf = z[fs * 32 + 16 * (e / 4) + 4 * grp + (e % 4)];
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) l_run[qb] += TT::to_f(pq[qb][fs][e]) * zf;
      }
    }
  }

  // ---- key tiles ----------------------------------------------------------------------
  const int n_comp = c >= 2 ? (c - 1) * d.topk : 0;
  const int nt_comp = (n_comp + 63) / 64;
  const int nt = nt_comp + (c >= 1 ? 1 : 0) + 1;
  const uint64_t selprev = c >= 1 ? a.selmask[static_cast<long long>(bh) * d.nC + c - 1] : 0ull;
  const long long sel_rows = static_cast<long long>(d.nCc) * d.topk;

  for (int tt = 0; tt < nt; ++tt) {
    const int type = tt < nt_comp ? 0 : ((tt == nt_comp && c >= 1) ? 1 : 2);
    const T* ksrc;
    const T* vsrc;
    long long kstride;
    int nkeys;
    long long tbase = 0;
    if (type == 0) {
      const long long off = (static_cast<long long>(bh) * sel_rows + static_cast<long long>(tt) * 64) * D;
      ksrc = ksel + off;
      vsrc = vsel + off;
      kstride = D;
      nkeys = n_comp - tt * 64 < 64 ? n_comp - tt * 64 : 64;
    } else {
      tbase = type == 1 ? t0 - 64 : t0;
      const long long off = ((b * T_ + tbase) * d.Hkv + h) * D;
      ksrc = kk + off;
      vsrc = vv + off;
      kstride = static_cast<long long>(d.Hkv) * D;
      nkeys = type == 1 ? 64 : nvalid;
    }
    const bool need_phi = type == 1 || (type == 2 && win < kChunk);

    __syncthreads();  // previous tile fully consumed
    for (int idx = tid; idx < 64 * V8; idx += nthr) {
      const int p = idx / V8, c8 = idx % V8;
      frag kx = TT::zero(), vx = TT::zero();
      if (p < nkeys) {
        kx = TT::load8(ksrc + p * kstride + c8 * 8);
        vx = TT::load8(vsrc + p * kstride + c8 * 8);
      }
      TT::store8(k_s + p * LDK + c8 * 8, kx);
#pragma unroll
      for (int e = 0; e < 8; ++e) vt_s[(c8 * 8 + e) * LDV + p] = vx[e];
    }
    if (need_phi) {
      for (int idx = tid; idx < 64 * F8; idx += nthr) {
        const int p = idx / F8, c8 = idx % F8;
        frag fx = TT::zero();
        if (p < nkeys) fx = TT::load8(phik + (static_cast<long long>(bh) * T_ + tbase + p) * DF + c8 * 8);
        TT::store8(pk_s + p * LDF + c8 * 8, fx);
      }
    }
    __syncthreads();

    // S^T = K Q^T
    f32x4 s[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const frag ka = TT::load8(k_s + (kb * 16 + r16) * LDK + ks * 32 + grp * 8);
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) TT::mma(s[kb][qb], ka, qf[qb][ks]);
      }
    }
    // phi(K) phi(Q)^T where some keys go to linear attention
    f32x4 ls[4][4];
    if (need_phi) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) ls[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int fs = 0; fs < DF / 32; ++fs) {
          const T* base = pk_s + (kb * 16 + r16) * LDF + fs * 32 + 4 * grp;
          const frag fa = TT::join(TT::load4(base), TT::load4(base + 16));
#pragma unroll
          for (int qb = 0; qb < 4; ++qb) TT::mma(ls[kb][qb], fa, pq[qb][fs]);
        }
      }
    }

    // online softmax + linear weights, per query column
    frag pf[2][4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const int r = qb * 16 + r16;
      float mx = m_run[qb];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int p = kb * 16 + 4 * grp + i;
          bool sa;
          if (type == 0) sa = p < nkeys;
          else if (type == 1) sa = (p > r + 64 - win) || ((selprev >> p) & 1ull);
          else sa = p <= r && p > r - win;
          if (sa) mx = fmaxf(mx, s[kb][qb][i] * c1);
        }
      mx = xor_max_groups(mx);
      const float alpha = exp2f(m_run[qb] - mx);
      m_run[qb] = mx;
      l_run[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) o[db][qb] *= alpha;
      const float la_scale = exp2f(-mx);
      float pv[4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int p = kb * 16 + 4 * grp + i;
          bool sa, la;
          if (type == 0) {
            sa = p < nkeys;
            la = false;
          } else if (type == 1) {
            sa = (p > r + 64 - win) || ((selprev >> p) & 1ull);
            la = !sa;
          } else {
            sa = p <= r && p > r - win;
            la = p <= r && !sa;
          }
          float x = 0.f;
          if (sa) x = exp2f(s[kb][qb][i] * c1 - mx);
          else if (la && need_phi) x = la_scale * ls[kb][qb][i];
          pv[kb][i] = x;
          l_run[qb] += x;
        }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[ks][qb][e] = TT::from_f(pv[2 * ks + e / 4][e % 4]);
    }

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const T* base = vt_s + (db * 16 + r16) * LDV + ks * 32 + 4 * grp;
        const frag va = TT::join(TT::load4(base), TT::load4(base + 16));
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) TT::mma(o[db][qb], va, pf[ks][qb]);
      }
  }

  // ---- epilogue: divide by the shared normaliser, write [B,T,Hq,D] ------------------
  T* out = static_cast<T*>(a.out);
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const float lt = xor_sum_groups(l_run[qb]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int r = qb * 16 + r16;
    if (head_ok && r < nvalid) {
      T* dst = out + ((b * T_ + t0 + r) * d.Hq + hq) * D + 4 * grp;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        typename TT::quad ov;
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = TT::from_f(o[db][qb][i] * inv);
        *reinterpret_cast<typename TT::quad*>(dst + db * 16) = ov;
      }
    }
  }
}

template <typename T, int D, int DF>
static hipError_t attn_t(const AttnArgs& a, hipStream_t s) {
  const int P = a.d.B * a.d.Hkv * a.gsplit;
  dim3 grid(a.d.nC * P);
  hipLaunchKernelGGL((attn_kernel<T, D, DF>), grid, dim3(64 * a.nw), 0, s, a);
  return hipGetLastError();
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
