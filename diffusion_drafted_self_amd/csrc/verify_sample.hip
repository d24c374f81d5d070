// Stochastic verification (temperature > 0) and sampling of the next drafts
// on gfx950.
//
// The final tokens are sampled autoregressively and match what sampling the
// AR model alone would give ("TiDAR：Nvidia 的擴散＋自回歸混合架構",
// engineer-news.pages.dev, section on what TiDAR does; "TiDAR : l'hybride de
// NVIDIA qui rédige par diffusion et parle de manière autorégressive",
// nodesdaily.com, paragraph on the reported numbers).  The rule is the
// speculative-sampling one: candidate i (token x, drawn from q_i) is kept
// when u_i * q_i(x) < p_i(x); at the first rejection a the next token is
// drawn from max(0, p_a - q_a), else (a = k) from p_k; the next drafts are
// drawn from the slots of group g = max(a, 1) - 1.  p = softmax(ar / T),
// q = softmax(q_logits / T).
//
// Draws are Gumbel-max: argmax_v (log2 w_v - log2(-log2 u_v)) is distributed
// as w / sum(w) (the ln 2 factors only scale and shift every score of a row).
// The uniforms come from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011)
// keyed by the caller's seed: counter (v / 4, row, b, step), word v % 4 for
// vocabulary entry v of draw row `row`; counter (i, 0xFFFFFFFF, b, step),
// word 0 for the keep test of candidate i.  u = ((x >> 9) + 0.5) * 2^-23 is
// exact in fp32.
//
//   sample_stats_kernel     (chunk, row) over the k AR rows and the k
//       proposal rows: max and sum of exp2 of z = logit * log2(e) / T.
//   sample_select_kernel    one workgroup per sequence, one wave per
//       candidate: the keep tests, then the first rejection by a ballot.
//   sample_partial_kernel   (chunk, row) over the k draw rows: row 0 the
//       residual of row a (or p_k), row m the draft slot m of group g; the
//       chunk's (score, lower index) maximum.
//   sample_finalize_kernel  one workgroup per sequence, one wave per row.
//
// A chunk is 4096 entries: thread t of 256 holds entries lo + 4t + 1024r + e
// (r, e < 4), so one Philox call gives the four words of one float4.
//
// Floating-point contraction is off in this file: z = logit * zscale is
// rounded before any use in every kernel, so the row maxima, the sums and
// the probabilities agree bit for bit wherever two rows hold the same logits
// (a fused multiply-subtract on one side and not the other would leave
// rounding-level residuals max(0, p - q) where p == q).
#include <algorithm>
#include <climits>

#include "check.h"
#include "common.h"
#include "launch.h"

#pragma clang fp contract(off)

namespace tidar {

namespace {

constexpr unsigned kPhiloxM0 = 0xD2511F53u, kPhiloxM1 = 0xCD9E8D57u;
constexpr unsigned kPhiloxW0 = 0x9E3779B9u, kPhiloxW1 = 0xBB67AE85u;
constexpr unsigned kAcceptPurpose = 0xFFFFFFFFu;
constexpr int kMaxRows = 16;   // k for the largest k
constexpr int kMaxWaves = 16;  // 1024 threads
constexpr int kPerThread = kSampleChunk / 256;
static_assert(kPerThread == 16, "a thread holds four float4 of its chunk");

struct U4 { unsigned x, y, z, w; };

// Ten rounds: words 0 and 2 are multiplied by the two multipliers, the
// products' halves become the next counter with the key folded into the
// high halves, and the key moves by the two Weyl constants between rounds.
__device__ __forceinline__ U4 philox4x32_10(U4 c, unsigned k0, unsigned k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    // one 32 x 32 -> 64-bit product per word (v_mad_u64_u32) gives both halves
    const unsigned long long p0 = (unsigned long long)kPhiloxM0 * c.x;
    const unsigned long long p1 = (unsigned long long)kPhiloxM1 * c.z;
    const unsigned lo0 = (unsigned)p0, hi0 = (unsigned)(p0 >> 32);
    const unsigned lo1 = (unsigned)p1, hi1 = (unsigned)(p1 >> 32);
    c = U4{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
  }
  return c;
}

// 23 random bits -> (0, 1), exact in fp32
__device__ __forceinline__ float to_uniform(unsigned x) {
  return ((float)(x >> 9) + 0.5f) * 1.1920928955078125e-7f;
}

// -log2(-log2(u)): the Gumbel shift in log2 units, up to a constant
__device__ __forceinline__ float gumbel2(unsigned x) {
  return -__builtin_amdgcn_logf(-__builtin_amdgcn_logf(to_uniform(x)));
}

// merge of (max, sum of exp2(z - max)) pairs; (-inf, 0) is the empty pair
__device__ __forceinline__ void stats_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * __builtin_amdgcn_exp2f(m - mn) + s2 * __builtin_amdgcn_exp2f(m2 - mn);
  m = mn;
}

__device__ __forceinline__ void wave_stats(float& m, float& s) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) stats_merge(m, s, __shfl_xor(m, o), __shfl_xor(s, o));
}

// entries v .. v+3 of a row; -inf past hi
// NT: nontemporal, for rows read once.  The statistics kernel reads every
// AR and proposal row once; the draw kernel reads the draft rows once, but
// the accepted position's AR and proposal rows (the residual) a second time.
template <bool NT>
__device__ __forceinline__ void load_row4(const float* src, int v, int hi, bool vec, float x[4]) {
  if (vec && v < hi) {
    const floatx4 f = NT ? __builtin_nontemporal_load((const floatx4*)(src + v)) : *(const floatx4*)(src + v);
    x[0] = f[0];
    x[1] = f[1];
    x[2] = f[2];
    x[3] = f[3];
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = v + e < hi ? (NT ? __builtin_nontemporal_load(src + v + e) : src[v + e]) : -INFINITY;
  }
}

// row r < B*k: AR row (b, i); else proposal row (b, i)
__global__ __launch_bounds__(256) void sample_stats_kernel(SampleArgs a) {
  __shared__ float sm[4], ss[4];
  const int chunk = blockIdx.x, row = blockIdx.y;
  const int nk = a.B * a.k;
  const float* src = row < nk ? a.ar_logits + ((size_t)(row / a.k) * (a.k + 1) + row % a.k) * a.V
                              : a.q_logits + (size_t)(row - nk) * a.V;
  const int lo = chunk * kSampleChunk, hi = min(a.V, lo + kSampleChunk);
  const bool vec = (a.V & 3) == 0;
  float x[kPerThread];
#pragma unroll
  for (int r = 0; r < 4; ++r) load_row4<true>(src, lo + 4 * (int)threadIdx.x + 1024 * r, hi, vec, x + 4 * r);
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    x[i] *= a.zscale;
    m = fmaxf(m, x[i]);
  }
  float s = 0.f;
  if (m != -INFINITY) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) s += __builtin_amdgcn_exp2f(x[i] - m);
  }
  wave_stats(m, s);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sm[wave] = m;
    ss[wave] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) stats_merge(m, s, sm[w], ss[w]);
    a.stats[(size_t)row * a.n_chunks + chunk] = make_float2(m, s);
  }
}

__device__ __forceinline__ float2 reduce_stats(const float2* part, int n_chunks) {
  float m = -INFINITY, s = 0.f;
  for (int c = threadIdx.x & 63; c < n_chunks; c += 64) stats_merge(m, s, part[c].x, part[c].y);
  wave_stats(m, s);
  return make_float2(m, s);
}

// block: min(k, kMaxWaves) waves over the k candidates of sequence blockIdx.x
__global__ __launch_bounds__(64 * kMaxWaves) void sample_select_kernel(SampleArgs a) {
  __shared__ int keep[kMaxRows];
  __shared__ float4 st[kMaxRows];  // (Mp, Zp, Mq, Zq) of candidate i's rows
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int i = wave; i < a.k; i += nw) {
    const float2 sp = reduce_stats(a.stats + ((size_t)b * a.k + i) * a.n_chunks, a.n_chunks);
    const float2 sq = reduce_stats(a.stats + ((size_t)a.B * a.k + (size_t)b * a.k + i) * a.n_chunks, a.n_chunks);
    if (lane == 0) {
      const int x = a.cand[(size_t)b * a.k + i];
      bool kept = false;  // a candidate outside the vocabulary is rejected
      if ((unsigned)x < (unsigned)a.V) {
        const float lp = a.ar_logits[((size_t)b * (a.k + 1) + i) * a.V + x];
        const float lq = a.q_logits[((size_t)b * a.k + i) * a.V + x];
        const U4 r = philox4x32_10(U4{(unsigned)i, kAcceptPurpose, (unsigned)b, a.step}, a.key0, a.key1);
        // u < p(x) / q(x) through d = log2 p(x) - log2 q(x), each term a
        // difference first: p(x) itself may lie below fp32's range at a low
        // temperature, and identical rows give d == 0 exactly.  d = NaN
        // (both logits -inf) rejects.
        const float d = (lp - lq) * a.zscale - (sp.x - sq.x) -
                        (__builtin_amdgcn_logf(sp.y) - __builtin_amdgcn_logf(sq.y));
        kept = d >= 0.f || to_uniform(r.x) < __builtin_amdgcn_exp2f(d);
      }
      keep[i] = kept;
      st[i] = make_float4(sp.x, sp.y, sq.x, sq.y);
    }
  }
  __syncthreads();
  if (wave == 0) {
    const bool reject = lane < a.k && !keep[lane];
    const unsigned long long mm = __ballot(reject || lane == a.k);
    const int acc = __ffsll((long long)mm) - 1;
    if (lane == 0) {
      a.accept_len[b] = acc;
      a.resid[b] = acc < a.k ? st[acc] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

// MODE 0: weights softmax(src) into (bv, bi).  MODE 1: weights max(0, p - q)
// of (src, qsrc) into (bv, bi), and the softmax(src) draw into (fv, fi) for a
// row whose residual weights are all 0 in fp32.
template <int MODE>
__device__ __forceinline__ void draw_chunk(const SampleArgs& a, const float* src, const float* qsrc, float4 rs,
                                           int b, int j, int lo, int hi, float& bv, int& bi, float& fv, int& fi) {
  const bool vec = (a.V & 3) == 0;
  const float inv_zp = MODE ? 1.f / rs.y : 0.f, inv_zq = MODE ? 1.f / rs.w : 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int v = lo + 4 * (int)threadIdx.x + 1024 * r;
    if (v >= hi) break;
    float x[4], y[4];
    load_row4<!MODE>(src, v, hi, vec, x);
    if (MODE) load_row4<false>(qsrc, v, hi, vec, y);
    const U4 rnd = philox4x32_10(U4{(unsigned)(v >> 2), (unsigned)j, (unsigned)b, a.step}, a.key0, a.key1);
    const unsigned w4[4] = {rnd.x, rnd.y, rnd.z, rnd.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (v + e >= hi) break;
      const float g = gumbel2(w4[e]);
      const float zp = x[e] * a.zscale;
      const float s0 = zp + g;
      if (MODE) {
        const float p = __builtin_amdgcn_exp2f(zp - rs.x) * inv_zp;
        const float q = __builtin_amdgcn_exp2f(y[e] * a.zscale - rs.z) * inv_zq;
        const float w = p - q;
        const float s = w > 0.f ? __builtin_amdgcn_logf(w) + g : -INFINITY;
        if (s > bv) {
          bv = s;
          bi = v + e;
        }
        if (s0 > fv) {
          fv = s0;
          fi = v + e;
        }
      } else if (s0 > bv) {
        bv = s0;
        bi = v + e;
      }
    }
  }
}

// (score, lower index) maximum over the workgroup; every thread returns it
__device__ __forceinline__ void block_argmax(float& bv, int& bi, float* sv, int* si) {
  argmax_wave(bv, bi);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  __syncthreads();
  for (int w = 0; w < 4; ++w)
    if (argmax_better(sv[w], si[w], bv, bi)) {
      bv = sv[w];
      bi = si[w];
    }
}

// row = b*k + j: j = 0 the token after the kept prefix, j >= 1 draft slot j
__global__ __launch_bounds__(256) void sample_partial_kernel(SampleArgs a) {
  __shared__ float sv[8];
  __shared__ int si[8];
  const int chunk = blockIdx.x, row = blockIdx.y;
  const int b = row / a.k, j = row % a.k;
  const int acc_read = a.accept_len[b];
  if (threadIdx.x == 0 && chunk == 0) (void)TIDAR_CHECK(acc_read >= 0 && acc_read <= a.k, TIDAR_CHECK_ACCEPT, acc_read);
  const int acc = min(max(acc_read, 0), a.k);  // written by sample_select_kernel; clamped regardless
  const int lo = chunk * kSampleChunk, hi = min(a.V, lo + kSampleChunk);
  float bv = -INFINITY, fv = -INFINITY;
  int bi = INT_MAX, fi = INT_MAX;
  if (j == 0 && acc < a.k) {
    const float* src = a.ar_logits + ((size_t)b * (a.k + 1) + acc) * a.V;
    const float* qsrc = a.q_logits + ((size_t)b * a.k + acc) * a.V;
    draw_chunk<1>(a, src, qsrc, a.resid[b], b, j, lo, hi, bv, bi, fv, fi);
    block_argmax(fv, fi, sv + 4, si + 4);
    if (threadIdx.x == 0) a.part_fb[(size_t)b * a.n_chunks + chunk] = make_float2(fv, __int_as_float(fi));
  } else {
    const int g = (acc > 0 ? acc : 1) - 1;
    const float* src = j == 0 ? a.ar_logits + ((size_t)b * (a.k + 1) + a.k) * a.V
                              : a.draft_logits + (((size_t)b * a.k + g) * a.k + j) * a.V;
    draw_chunk<0>(a, src, nullptr, make_float4(0.f, 0.f, 0.f, 0.f), b, j, lo, hi, bv, bi, fv, fi);
  }
  block_argmax(bv, bi, sv, si);
  if (threadIdx.x == 0) a.part[(size_t)row * a.n_chunks + chunk] = make_float2(bv, __int_as_float(bi));
}

__device__ __forceinline__ int reduce_draw(const float2* part, int n_chunks) {
  float bv = -INFINITY;
  int bi = INT_MAX;
  for (int c = threadIdx.x & 63; c < n_chunks; c += 64) {
    const float2 p = part[c];
    const int pi = __float_as_int(p.y);
    if (argmax_better(p.x, pi, bv, bi)) {
      bv = p.x;
      bi = pi;
    }
  }
  argmax_wave(bv, bi);
  return bi;
}

// block: min(k, kMaxWaves) waves over the k draw rows of sequence blockIdx.x
__global__ __launch_bounds__(64 * kMaxWaves) void sample_finalize_kernel(SampleArgs a) {
  const int b = blockIdx.x;
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int acc = min(max(a.accept_len[b], 0), a.k);
  for (int j = wave; j < a.k; j += nw) {
    int t = reduce_draw(a.part + ((size_t)b * a.k + j) * a.n_chunks, a.n_chunks);
    // a residual with no positive weight in fp32: the draw from p stands in
    if (j == 0 && acc < a.k && t == INT_MAX) t = reduce_draw(a.part_fb + (size_t)b * a.n_chunks, a.n_chunks);
    if ((threadIdx.x & 63) == 0) {
      (void)TIDAR_CHECK(t >= 0 && t < a.V, TIDAR_CHECK_TOKEN, t);
      a.next_cand[(size_t)b * a.k + j] = t;
    }
  }
}

}  // namespace

// Each launch is checked before the next: the draw kernels index rows by the
// accept length the selection writes.
hipError_t launch_verify_sample(const SampleArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  if (a.k > kMaxRows) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sample_stats_kernel, dim3(a.n_chunks, 2 * a.B * a.k), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sample_select_kernel, dim3(a.B), dim3(64 * std::min(a.k, kMaxWaves)), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sample_partial_kernel, dim3(a.n_chunks, a.B * a.k), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sample_finalize_kernel, dim3(a.B), dim3(64 * std::min(a.k, kMaxWaves)), 0, s, a);
  return hipGetLastError();
}

#if TIDAR_CHECKED
TIDAR_CHECK_RECORD_ACCESSOR(check_record_verify_sample)
#endif

}  // namespace tidar
