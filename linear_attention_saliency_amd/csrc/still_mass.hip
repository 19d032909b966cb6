// Local-global consistency of the routing: the attention each key receives from far-future
// queries under full causal softmax, its per-chunk top-k, and the overlap of two selections.
// (Page labels [P1]..[P4]: the pages listed at the top of include/still.h. [P2] reports that
// the Self-Saliency Score, computed in a local window, predicts whether a token will still
// be attended once it is far history, with a measured overlap; [P1] section
// "Self-Saliency Score" claims selection accuracy close to that of global attention.)
//
// For KV head h and key j, F_j = sum over the group's query heads and over queries
// i >= j + window of p_ij = 2^{a_ij - L_i}, a_ij = q_i . k_j log2(e) / sqrt(D) and L_i the
// log2 of the full causal normaliser of row i.
//   mass_lse_kernel  per (chunk, query head, b): L_i over every key j <= i (the key tiles
//                    arrive by buffer -> LDS copies one tile ahead)
//   mass_col_kernel  per (key chunk, query slice, b * KV head): the column sums of p over
//                    the slice's queries, for the chunk's 64 keys; fp32 partials
//   mass_sum_kernel  F = the sum of the partials, in slice order
//   overlap_kernel   tokens two per-chunk selections share
#include "still_launch.hpp"
#include "still_tile.hpp"

namespace still {

namespace {
constexpr int MD = 64;  // head_dim of these kernels
}

template <typename T>
__global__ __launch_bounds__(256) void mass_lse_kernel(MassArgs a) {
  using TT = Tr<T>;
  using frag = typename TT::frag;
  using Dma = DmaTile<T, 64, 64, 4>;
  constexpr int ES = static_cast<int>(sizeof(T));
  __shared__ __attribute__((aligned(16))) T lds[2][64 * 64];
  const Dims& d = a.d;
  const int w = xcd_work(blockIdx.x, gridDim.x);
  const int c = __builtin_amdgcn_readfirstlane(w % d.nC);
  const int hq = __builtin_amdgcn_readfirstlane((w / d.nC) % d.Hq);
  const int b = __builtin_amdgcn_readfirstlane(w / (d.nC * d.Hq));
  const int h = hq / d.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r16 = lane & 15, grp = lane >> 4;
  const int qrow = wave * 16 + r16;
  const long long i = 64LL * c + qrow;
  const bool qvalid = i < d.T;
  const float scale2 = kLog2e * 0.125f;
  frag qf[2];
  const T* qp = static_cast<const T*>(a.q) + ((static_cast<long long>(b) * d.T + i) * d.Hq + hq) * MD;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) qf[ks] = qvalid ? TT::load8(qp + ks * 32 + grp * 8) : TT::zero();
  Dma dma;
  dma.init(d.Hkv * MD);
  const T* kb0 = static_cast<const T*>(a.k) + (static_cast<long long>(b) * d.T * d.Hkv + h) * MD;
  auto issue = [&](int t) {
    const int nv = min(64, d.T - 64 * t);
    const uint32_t bytes = static_cast<uint32_t>(((nv - 1) * d.Hkv * MD + MD) * ES);
    dma.issue(lds[t & 1], make_rsrc(kb0 + 64LL * t * d.Hkv * MD, bytes), 0);
  };
  float mx2 = -kInf, l = 0.f;
  issue(0);
  for (int t = 0; t <= c; ++t) {
    if (t + 1 <= c) {
      issue(t + 1);
      __builtin_amdgcn_s_waitcnt(vm_wait_imm(Dma::PER_WAVE));
    } else {
      __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
    }
    lds_sync();
    f32x4 s[4];
    rows_x_frag<T>(s, lds[t & 1], qf);  // s[kb][e] = q . k for key 64 t + 16 kb + 4 grp + e
    const bool diag = t == c;           // keys after the query are masked on the diagonal tile
    float tm = -kInf;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) tm = (!diag || kb * 16 + 4 * grp + e <= qrow) ? fmaxf(tm, s[kb][e]) : tm;
    tm = xor_max_groups(tm) * scale2;
    const float mn = fmaxf(mx2, tm);
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pe = __builtin_amdgcn_exp2f(fmaf(s[kb][e], scale2, -mn));
        ps += (!diag || kb * 16 + 4 * grp + e <= qrow) ? pe : 0.f;
      }
    ps = xor_sum_groups(ps);
    l = l * __builtin_amdgcn_exp2f(mx2 - mn) + ps;  // the first tile holds key 0 <= i, so mn is finite
    mx2 = mn;
    lds_sync();
  }
  if (grp == 0) a.lse[(static_cast<long long>(b) * d.Hq + hq) * d.nC * 64 + i] = qvalid ? mx2 + __log2f(l) : kInf;
}

// Column sums for the 64 keys of chunk c over the queries of chunks [max(c, s*per),
// min(nC, (s+1)*per)) of every query head of the group; the query rows and their L arrive
// one (chunk, head) step ahead.
template <typename T>
__global__ __launch_bounds__(256) void mass_col_kernel(MassArgs a) {
  using TT = Tr<T>;
  using frag = typename TT::frag;
  using Dma = DmaTile<T, 64, 64, 4>;
  constexpr int ES = static_cast<int>(sizeof(T));
  __shared__ __attribute__((aligned(16))) T lds[2][64 * 64];
  __shared__ __attribute__((aligned(16))) float s_l[2][64];
  const Dims& d = a.d;
  const int w = xcd_work(blockIdx.x, gridDim.x);
  const int c = __builtin_amdgcn_readfirstlane(w % d.nC);
  const int split = __builtin_amdgcn_readfirstlane((w / d.nC) % a.nsplit);
  const int bh = __builtin_amdgcn_readfirstlane(w / (d.nC * a.nsplit));
  const int b = bh / d.Hkv, h = bh % d.Hkv;
  const int cq0 = max(c, split * a.per), cq1 = min(d.nC, (split + 1) * a.per);
  if (cq1 <= cq0) return;  // this slice lies before the chunk: the sum skips it
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r16 = lane & 15, grp = lane >> 4;
  const int jr = wave * 16 + r16;
  const long long j = 64LL * c + jr;  // this lane column's key
  const bool kvalid = j < d.T;
  const float scale2 = kLog2e * 0.125f;
  frag kf[2];
  const T* kp = static_cast<const T*>(a.k) + ((static_cast<long long>(b) * d.T + j) * d.Hkv + h) * MD;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) kf[ks] = kvalid ? TT::load8(kp + ks * 32 + grp * 8) : TT::zero();
  Dma dmq;
  dmq.init(d.Hq * MD);
  const int nsteps = (cq1 - cq0) * d.G;
  auto step_of = [&](int st, int& cq, int& hq) {
    cq = cq0 + __builtin_amdgcn_readfirstlane(st / d.G);
    hq = h * d.G + __builtin_amdgcn_readfirstlane(st % d.G);
  };
  auto issue = [&](int st) {
    int cq, hq;
    step_of(st, cq, hq);
    const int nv = min(64, d.T - 64 * cq);
    const uint32_t bytes = static_cast<uint32_t>(((nv - 1) * d.Hq * MD + MD) * ES);
    const T* src = static_cast<const T*>(a.q) + ((static_cast<long long>(b) * d.T + 64LL * cq) * d.Hq + hq) * MD;
    dmq.issue(lds[st & 1], make_rsrc(src, bytes), 0);
  };
  auto l_of = [&](int st) {  // L of query row (tid & 63) of step st
    int cq, hq;
    step_of(st, cq, hq);
    return a.lse[(static_cast<long long>(b) * d.Hq + hq) * d.nC * 64 + 64LL * cq + (tid & 63)];
  };
  float msum = 0.f;
  float ln = l_of(0);
  issue(0);
  for (int st = 0; st < nsteps; ++st) {
    const float lc = ln;
    if (st + 1 < nsteps) {
      ln = l_of(st + 1);
      issue(st + 1);
      __builtin_amdgcn_s_waitcnt(vm_wait_imm(Dma::PER_WAVE + 1));
    } else {
      __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
    }
    if (tid < 64) s_l[st & 1][tid] = lc;
    __builtin_amdgcn_s_waitcnt(kLgkmWait0);
    lds_sync();
    int cq, hq;
    step_of(st, cq, hq);
    f32x4 s[4];
    rows_x_frag<T>(s, lds[st & 1], kf);  // s[qb][e] = q[16 qb + 4 grp + e] . k
    // every query of the tile is far enough from every key of the chunk: no mask
    const bool far = 64LL * cq >= 64LL * c + 63 + d.window;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const f32x4 lq = *reinterpret_cast<const f32x4*>(&s_l[st & 1][qb * 16 + 4 * grp]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const long long iq = 64LL * cq + qb * 16 + 4 * grp + e;
        const float p = __builtin_amdgcn_exp2f(fmaf(s[qb][e], scale2, -lq[e]));  // rows past T have L = inf
        msum += (far || iq - j >= d.window) ? p : 0.f;
      }
    }
    lds_sync();
  }
  msum = xor_sum_groups(msum);
  if (grp == 0 && kvalid) a.part[(static_cast<long long>(split) * d.B * d.Hkv + bh) * d.T + j] = msum;
}

__global__ __launch_bounds__(256) void mass_sum_kernel(const float* part, float* mass, int T, int per, int nsplit,
                                                       long long n) {
  const long long gid = blockIdx.x * 256LL + threadIdx.x;
  if (gid >= n) return;
  const int j = static_cast<int>(gid % T);
  const int s0 = (j / 64) / per;  // earlier slices hold no query of this key's chunk or later
  float acc = 0.f;
  for (int s = s0; s < nsplit; ++s) acc += part[static_cast<long long>(s) * n + gid];
  mass[gid] = acc;
}

__global__ __launch_bounds__(256) void overlap_kernel(const int32_t* sa, const int32_t* sb, int32_t* out, int k,
                                                      long long n) {
  const long long gid = blockIdx.x * 256LL + threadIdx.x;
  if (gid >= n) return;
  const int32_t* pa = sa + gid * k;
  const int32_t* pb = sb + gid * k;
  int common = 0;
  for (int x = 0; x < k; ++x)
    for (int y = 0; y < k; ++y) common += pa[x] == pb[y] ? 1 : 0;
  out[gid] = common;
}

template <typename T>
static hipError_t launch_mass_t(const MassArgs& a, hipStream_t s) {
  const Dims& d = a.d;
  hipLaunchKernelGGL(mass_lse_kernel<T>, dim3(d.nC * d.Hq * d.B), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mass_col_kernel<T>, dim3(d.nC * a.nsplit * d.B * d.Hkv), dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const long long n = static_cast<long long>(d.B) * d.Hkv * d.T;
  hipLaunchKernelGGL(mass_sum_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, a.part, a.mass,
                     d.T, a.per, a.nsplit, n);
  return hipGetLastError();
}

hipError_t launch_mass(const MassArgs& a, hipStream_t s) {
  return a.d.bf16 ? launch_mass_t<bf16>(a, s) : launch_mass_t<float>(a, s);
}

hipError_t launch_overlap(const Dims& d, const int32_t* sa, const int32_t* sb, int32_t* out, hipStream_t s) {
  const long long n = static_cast<long long>(d.B) * d.Hkv * d.nCc;
  if (n == 0 || d.topk == 0) return hipSuccess;
  hipLaunchKernelGGL(overlap_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, sa, sb, out, d.topk,
                     n);
  return hipGetLastError();
}

}  // namespace still
