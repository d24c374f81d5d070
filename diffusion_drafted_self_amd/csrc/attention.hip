// Step attention of one TiDAR decode step on gfx950.
//
// Every query row of the step block (k candidates + n_groups*k draft slots,
// times the G query heads sharing a KV head) reads the whole settled prefix
// plus the step keys its zone lets it see ("TiDAR : l'hybride de NVIDIA qui
// rédige par diffusion et parle de manière autorégressive", nodesdaily.com,
// paragraphs on the three zones and on masking).  Because all R*G rows of a
// KV head read the same prefix, the prefix is streamed from HBM once per
// (sequence, KV head, key chunk) and the rows form a dense MFMA tile: the
// extra draft rows ride on otherwise idle matrix throughput (same page,
// paragraph on masking; abstract on fugumt.com).
//
// Kernels
//   attn_split_bf16_kernel<D, NW>  one workgroup = NW waves x 32 query rows
//       of one (b, kvh) against one key chunk.  Per 64-key tile: K and V^T
//       are staged in LDS, S^T = K.Q^T and O^T += V^T.P^T run on
//       v_mfma_f32_32x32x16_bf16, the online softmax runs in registers
//       (exp2 with the scale folded in), and the mask is evaluated from zone
//       indices only on tiles that hold step keys.  Writes the chunk's
//       unnormalised output, running max and sum.
//   attn_split_f32_kernel<D>  the f32 instance (VALU FMA; fp32 MFMA peak
//       equals VALU fp32 peak on this part), same partial format.
//   attn_merge_kernel<Out, D>  log-sum-exp merge of the chunks, one wave per
//       query row: normalised output (RNE to the output type) and the LSE.
#include "common.h"
#include "launch.h"

namespace tidar {

namespace {

constexpr int TK = 64;  // keys per tile

// S^T tile row i <-> key sigma(i) of the 32-key block.  With this order the
// 16 fp32 scores a lane holds after S^T = K.Q^T are, in register order, the
// keys 16h + 8*(lane/32) + 0..7 (h = 0, 1): exactly the B-operand layout of
// the P^T factor of O^T += V^T.P^T, so P needs no cross-lane shuffle.
__device__ __forceinline__ int sigma(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_split_bf16_kernel(AttnArgs a) {
  constexpr int KS = D + 8;   // K tile row stride (elements): 16 B pad per row
  constexpr int VS = TK + 8;  // V^T tile row stride (elements)
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(16))) bf16 Ks[TK * KS];
  __shared__ __attribute__((aligned(16))) bf16 Vt[D * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;

  int t = xcd_logical_block(blockIdx.x, gridDim.x);
  const int rb = t % a.n_rowblk;
  t /= a.n_rowblk;
  const int split = t % a.n_split;
  t /= a.n_split;
  const int kvh = t % a.Hkv;
  const int b = t / a.Hkv;

  const int L = a.lens[b];
  if (L < 0 || L > a.max_len) return;  // contract violation: merge writes NaN
  const int Ltot = L + a.R;
  const int kb = split * a.chunk;
  if (kb >= Ltot) return;
  const int ke = min(kb + a.chunk, Ltot);

  const int m = rb * (NW * 32) + wave * 32 + (lane & 31);  // this lane's query row
  const bool row_ok = m < a.M;
  const int r = row_ok ? m / a.G : 0;
  const int jh = row_ok ? m % a.G : 0;

  // Q^T operand: lane holds q[row m][16c + 8*half + 0..7] for each 16-wide d chunk c.
  bf16x8 qf[D / 16];
  {
    const bf16* qrow = (const bf16*)a.q + ((size_t)(b * a.R + r) * a.Hq + kvh * a.G + jh) * D;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      bf16x8 z = {};
      qf[c] = row_ok ? *(const bf16x8*)(qrow + 16 * c + 8 * half) : z;
    }
  }

  floatx16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[db][v] = 0.f;
  float m_run = kNoMax, l_run = 0.f;

  const int sig = sigma(lane & 31);
  const size_t pair = (size_t)b * a.Hkv + kvh;
  const bf16* kc_base = (const bf16*)a.k_cache + pair * a.S_max * D;
  const bf16* vc_base = (const bf16*)a.v_cache + pair * D * a.S_max;
  const size_t step_stride = (size_t)a.Hkv * D;  // elements between step rows
  const bf16* ks_base = (const bf16*)a.k_step + (size_t)b * a.R * step_stride + kvh * D;
  const bf16* vs_base = (const bf16*)a.v_step + (size_t)b * a.R * step_stride + kvh * D;

  for (int t0 = kb; t0 < ke; t0 += TK) {
    // ---- stage K tile [TK keys][D] (16 B per thread per iteration)
    for (int id = tid; id < TK * D / 8; id += NT) {
      const int key = id / (D / 8), dc = id % (D / 8);
      const int c = t0 + key;
      bf16x8 val = {};
      if (c < L) val = *(const bf16x8*)(kc_base + (size_t)c * D + 8 * dc);
      else if (c < Ltot) val = *(const bf16x8*)(ks_base + (size_t)(c - L) * step_stride + 8 * dc);
      *(bf16x8*)(Ks + key * KS + 8 * dc) = val;
    }
    // ---- stage V^T tile [D][TK keys]; the cache already holds values transposed
    for (int id = tid; id < D * TK / 8; id += NT) {
      const int d = id / (TK / 8), kc8 = id % (TK / 8);
      const int c0 = t0 + 8 * kc8;
      bf16x8 val = {};
      if (c0 + 8 <= L) {
        val = *(const bf16x8*)(vc_base + (size_t)d * a.S_max + c0);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = c0 + e;
          bf16 x = (bf16)0.f;
          if (c < L) x = vc_base[(size_t)d * a.S_max + c];
          else if (c < Ltot) x = vs_base[(size_t)(c - L) * step_stride + d];
          val[e] = x;
        }
      }
      *(bf16x8*)(Vt + d * VS + 8 * kc8) = val;
    }
    __syncthreads();

    // ---- S^T[key][row] = K . Q^T for two 32-key blocks
    floatx16 s[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb2][v] = 0.f;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const bf16x8 ka = *(const bf16x8*)(Ks + (32 * kb2 + sig) * KS + 16 * c + 8 * half);
        s[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[c], s[kb2], 0, 0, 0);
      }
    }

    // ---- zone mask (only tiles reaching past the settled prefix)
    if (t0 + TK > L) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int i = 8 * (v >> 2) + 4 * half + (v & 3);
          const int c = t0 + 32 * kb2 + sigma(i);
          const bool vis = c < ke && (c < L || step_visible(r, c - L, a.k));
          if (!vis) s[kb2][v] = -INFINITY;
        }
    }

    // ---- online softmax (log2 domain); lanes l and l^32 share a row
    float mx = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb2][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * a.scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;

    bf16x8 pk[4];
    float psum = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float p = __builtin_amdgcn_exp2f(s[kb2][8 * h + jj] * a.scale_log2 - m_new);
          psum += p;
          pk[2 * kb2 + h][jj] = (bf16)p;
        }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[db][v] *= alpha;

    // ---- O^T[d][row] += V^T . P^T, 16 keys per MFMA
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const bf16x8 va = *(const bf16x8*)(Vt + (32 * db + (lane & 31)) * VS + 16 * kc + 8 * half);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pk[kc], o[db], 0, 0, 0);
      }
    __syncthreads();  // the next tile overwrites Ks / Vt
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (row_ok) {
    const size_t base = (pair * a.n_split + split) * a.M + m;
    float* op = a.o_part + base * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        floatx4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = o[db][4 * g4 + e];
        *(floatx4*)(op + 32 * db + 8 * g4 + 4 * half) = w;
      }
    if (half == 0) a.ml_part[base] = make_float2(m_run, l_tot);
  }
}

// f32 instance: one wave per (b, kvh, chunk, query row).  Lanes first take
// keys (scores into LDS), then head-dim elements (P.V).  chunk <= 1024.
template <int D>
__global__ __launch_bounds__(64) void attn_split_f32_kernel(AttnArgs a) {
  __shared__ float qs[D];
  __shared__ float sc[1024];
  const int lane = threadIdx.x;
  int t = blockIdx.x;
  const int m = t % a.M;
  t /= a.M;
  const int split = t % a.n_split;
  t /= a.n_split;
  const int kvh = t % a.Hkv;
  const int b = t / a.Hkv;

  const int L = a.lens[b];
  if (L < 0 || L > a.max_len) return;
  const int Ltot = L + a.R;
  const int kb = split * a.chunk;
  if (kb >= Ltot) return;
  const int ke = min(kb + a.chunk, Ltot);
  const int r = m / a.G, jh = m % a.G;

  const float* qrow = (const float*)a.q + ((size_t)(b * a.R + r) * a.Hq + kvh * a.G + jh) * D;
  for (int d = lane; d < D; d += 64) qs[d] = qrow[d];
  __syncthreads();

  const size_t pair = (size_t)b * a.Hkv + kvh;
  const float* kc_base = (const float*)a.k_cache + pair * a.S_max * D;
  const float* vc_base = (const float*)a.v_cache + pair * D * a.S_max;
  const size_t step_stride = (size_t)a.Hkv * D;
  const float* ks_base = (const float*)a.k_step + (size_t)b * a.R * step_stride + kvh * D;
  const float* vs_base = (const float*)a.v_step + (size_t)b * a.R * step_stride + kvh * D;

  float mx = -INFINITY;
  for (int c = kb + lane; c < ke; c += 64) {
    const float* krow = c < L ? kc_base + (size_t)c * D : ks_base + (size_t)(c - L) * step_stride;
    float dot = 0.f;
    for (int d = 0; d < D; ++d) dot = fmaf(qs[d], krow[d], dot);
    const bool vis = c < L || step_visible(r, c - L, a.k);
    const float s2 = vis ? dot * a.scale_log2 : -INFINITY;
    sc[c - kb] = s2;
    mx = fmaxf(mx, s2);
  }
  mx = wave_max(mx);
  if (mx == -INFINITY) mx = kNoMax;
  float l = 0.f;
  for (int c = kb + lane; c < ke; c += 64) {
    const float p = exp2f(sc[c - kb] - mx);
    sc[c - kb] = p;
    l += p;
  }
  l = wave_sum(l);
  __syncthreads();

  const size_t base = (pair * a.n_split + split) * a.M + m;
  for (int d = lane; d < D; d += 64) {
    float acc = 0.f;
    for (int c = kb; c < ke; ++c) {
      const float p = sc[c - kb];
      const float v = c < L ? vc_base[(size_t)d * a.S_max + c] : vs_base[(size_t)(c - L) * step_stride + d];
      acc = fmaf(p, v, acc);
    }
    a.o_part[base * D + d] = acc;
  }
  if (lane == 0) a.ml_part[base] = make_float2(mx, l);
}

__device__ __forceinline__ void store_out(float* p, float x) { *p = x; }
__device__ __forceinline__ void store_out(bf16* p, float x) { *p = (bf16)x; }

// Log-sum-exp merge of the key chunks: one wave per (b, kvh, row m).
template <typename OutT, int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  constexpr int E = D / 64;  // elements per lane
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= a.B * a.Hkv * a.M) return;
  const int m = w % a.M;
  const int pr = w / a.M;  // b * Hkv + kvh
  const int kvh = pr % a.Hkv;
  const int b = pr / a.Hkv;
  const int r = m / a.G, h = kvh * a.G + m % a.G;
  OutT* orow = (OutT*)a.out + ((size_t)(b * a.R + r) * a.Hq + h) * D;
  float* lse = a.lse ? a.lse + ((size_t)b * a.Hq + h) * a.R + r : nullptr;

  const int L = a.lens[b];
  if (L < 0 || L > a.max_len) {
    for (int e = 0; e < E; ++e) store_out(orow + lane * E + e, NAN);
    if (lse && lane == 0) *lse = NAN;
    return;
  }
  const int n_valid = (L + a.R + a.chunk - 1) / a.chunk;
  const size_t base = (size_t)pr * a.n_split * a.M + m;

  float mx = -INFINITY;
  for (int s = 0; s < n_valid; ++s) mx = fmaxf(mx, a.ml_part[base + (size_t)s * a.M].x);
  float den = 0.f, acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int s = 0; s < n_valid; ++s) {
    const size_t idx = base + (size_t)s * a.M;
    const float2 ml = a.ml_part[idx];
    const float wgt = exp2f(ml.x - mx);
    den += wgt * ml.y;
    const float* op = a.o_part + idx * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(wgt, op[e], acc[e]);
  }
  const float inv = 1.f / den;
#pragma unroll
  for (int e = 0; e < E; ++e) store_out(orow + lane * E + e, acc[e] * inv);
  if (lse && lane == 0) *lse = (mx + log2f(den)) * kLn2;
}

template <int D, int NW>
hipError_t launch_bf16_split(const AttnArgs& a, hipStream_t s) {
  const int nblk = a.B * a.Hkv * a.n_split * a.n_rowblk;
  hipLaunchKernelGGL((attn_split_bf16_kernel<D, NW>), dim3(nblk), dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

template <typename OutT, int D>
hipError_t launch_merge(const AttnArgs& a, hipStream_t s) {
  const long rows = (long)a.B * a.Hkv * a.M;
  hipLaunchKernelGGL((attn_merge_kernel<OutT, D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  hipError_t e = hipErrorInvalidValue;
  if (a.D == 128) {
    switch (a.waves) {
      case 1: e = launch_bf16_split<128, 1>(a, s); break;
      case 2: e = launch_bf16_split<128, 2>(a, s); break;
      case 3: e = launch_bf16_split<128, 3>(a, s); break;
      case 4: e = launch_bf16_split<128, 4>(a, s); break;
    }
  } else if (a.D == 64) {
    switch (a.waves) {
      case 1: e = launch_bf16_split<64, 1>(a, s); break;
      case 2: e = launch_bf16_split<64, 2>(a, s); break;
      case 3: e = launch_bf16_split<64, 3>(a, s); break;
      case 4: e = launch_bf16_split<64, 4>(a, s); break;
    }
  }
  if (e != hipSuccess) return e;
  return a.D == 128 ? launch_merge<bf16, 128>(a, s) : launch_merge<bf16, 64>(a, s);
}

hipError_t launch_attention_f32(const AttnArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  const unsigned nblk = (unsigned)(a.B * a.Hkv * a.n_split * a.M);
  if (a.D == 128) hipLaunchKernelGGL((attn_split_f32_kernel<128>), dim3(nblk), dim3(64), 0, s, a);
  else hipLaunchKernelGGL((attn_split_f32_kernel<64>), dim3(nblk), dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return a.D == 128 ? launch_merge<float, 128>(a, s) : launch_merge<float, 64>(a, s);
}

}  // namespace tidar
