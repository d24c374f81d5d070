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
//       stream into two LDS stages by direct loads, S^T = K.Q^T and O^T += V^T.P^T run on
//       v_mfma_f32_32x32x16_bf16, the online softmax runs in registers
//       (exp2 with the scale folded in, lazy rescale), and the mask is
//       evaluated from zone indices only on tiles that hold step keys.
//       Single-chunk sequences are normalised and written directly; others
//       leave the chunk's unnormalised output, running max and sum.
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

// The value cache holds pages of VPAGE positions, each stored transposed
// ([S_max/VPAGE][D][VPAGE] per (b, kvh)), so one 64-key V^T tile is one
// contiguous 16 KB page, like the K tile.
constexpr int VPAGE = 64;
static_assert(TK == VPAGE, "a key tile is one value page");

__device__ __forceinline__ size_t vpos(int d, int c, int D) {  // element (d, position c) of a value cache
  return (size_t)(c / VPAGE) * D * VPAGE + (size_t)d * VPAGE + (c % VPAGE);
}

// LDS tile geometry.  K tile: TK rows of D bf16, row-major; V^T tile: D rows
// of TK bf16.  Both are filled 1 KB at a time by direct global->LDS loads
// (each lane moves 16 B; lane t lands at byte 16t of the 1 KB block), so a
// 16 B piece's position inside its row is permuted by an XOR swizzle chosen
// by the source address each lane reads: logical piece p of K row `row` sits
// at physical piece p ^ kswz(row), logical piece q of V^T row d at q ^ (d&7).
// With these, the 32 lanes reading one MFMA operand column hit distinct banks.
template <int D>
struct Tile {
  static constexpr int KROW = D * 2;        // bytes per K row
  static constexpr int KPPR = KROW / 16;    // 16 B pieces per K row
  static constexpr int K_BYTES = TK * KROW;
  static constexpr int VROW = TK * 2;       // bytes per V^T row (8 pieces)
  static constexpr int V_BYTES = D * VROW;
  static constexpr int NK = K_BYTES / 1024; // 1 KB load instructions per tile
  static constexpr int NV = V_BYTES / 1024;
  static constexpr int NI = NK + NV;
};

// V^T rows: 16 consecutive rows get distinct (row parity, piece) pairs and 8
// consecutive rows distinct pieces, so the read is conflict-free whether the
// LDS serves 8 or 16 lanes of a 16 B read per cycle.
__device__ __forceinline__ int vswz(int d) { return (d & 7) ^ ((d >> 3) & 1); }

template <int D>
__device__ __forceinline__ int kswz(int row) {
  if constexpr (Tile<D>::KPPR == 16) return sigma(row & 15);
  else return (row & 3) | ((row >> 1) & 4);
}

// LDS pointers stay in address space 3 end to end (no generic casts)
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0]+[15:14], expcnt[6:4], lgkmcnt[11:8])
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }

// Direct global->LDS load of 16 B per lane: lane t's bytes land at
// lds_dst + 16*t.  Issued as inline asm with a scalar base and a 32-bit
// per-lane offset, so the compiler neither rebuilds 64-bit addresses every
// tile nor treats the load as an LDS store it must order against unrelated
// LDS reads (its LDS-DMA alias tracking would serialise the pipeline); the
// kernel orders these loads itself with s_waitcnt vmcnt and barriers.  No
// output registers are involved.
__device__ __forceinline__ void dma_b128(const char* base, unsigned off, lds_char* lds_dst) {
  const unsigned long long b = (unsigned long long)base;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)b);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(b >> 32));
  const unsigned long long sb = ((unsigned long long)hi << 32) | lo;
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_dst);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(sb), "s"(m0) : "memory", "m0");
}

// Per-lane byte offsets of this wave's direct loads inside a tile: load
// i = wave + ii*NW of the tile (K loads first, then V^T loads), each moving
// one 1 KB block of the swizzled LDS layout.  Tile-invariant, so computed
// once per workgroup.
template <int D, int NW>
struct DmaPlan {
  static constexpr int N = (Tile<D>::NI + NW - 1) / NW;
  unsigned off[N];
};

template <int D, int NW>
__device__ __forceinline__ void dma_plan(DmaPlan<D, NW>& pl, int wave, int lane) {
  using T = Tile<D>;
#pragma unroll
  for (int ii = 0; ii < DmaPlan<D, NW>::N; ++ii) {
    const int i = wave + ii * NW;
    unsigned off = 0;
    if (i < T::NK) {
      const int row = i * (64 / T::KPPR) + lane / T::KPPR;
      const int p = (lane % T::KPPR) ^ kswz<D>(row);
      off = row * T::KROW + p * 16;
    } else if (i < T::NI) {
      const int d = (i - T::NK) * 8 + (lane >> 3);
      const int q = (lane & 7) ^ vswz(d);
      off = d * T::VROW + q * 16;
    }
    pl.off[ii] = off;
  }
}

// Issue this wave's share of the direct loads of one prefix tile (keys
// t0..t0+TK-1, all settled).  The K tile is 64 contiguous cache rows, the
// V^T tile one contiguous value page.
template <int D, int NW>
__device__ __forceinline__ void issue_tile(lds_char* sK, lds_char* sV, const bf16* kc_base, const bf16* vc_base,
                                           const DmaPlan<D, NW>& pl, int t0, int wave) {
  using T = Tile<D>;
  const char* kt = (const char*)(kc_base + (size_t)t0 * D);
  const char* vt = (const char*)(vc_base + (size_t)(t0 / VPAGE) * D * VPAGE);
#pragma unroll
  for (int ii = 0; ii < DmaPlan<D, NW>::N; ++ii) {
    const int i = wave + ii * NW;
    if (i < T::NK) dma_b128(kt, pl.off[ii], sK + i * 1024);
    else if (i < T::NI) dma_b128(vt, pl.off[ii], sV + (i - T::NK) * 1024);
  }
}

// Stage a tile that reaches past the settled prefix (the step block, or
// keys past the end) into the same swizzled layout.  Settled keys come from
// the caches in 16 B pieces; step rows are read 16 B at a time and their
// values scattered into V^T columns; everything else is zero.
template <int D, int NW>
__device__ __forceinline__ void stage_tail_tile(lds_char* sK, lds_char* sV, const bf16* kc_base, const bf16* vc_base,
                                                const bf16* ks_base, const bf16* vs_base, size_t step_stride,
                                                int t0, int L, int Ltot, int tid) {
  using T = Tile<D>;
  for (int id = tid; id < TK * T::KPPR; id += NW * 64) {
    const int row = id / T::KPPR, p = id % T::KPPR;
    const int c = t0 + row;
    bf16x8 val = {};
    if (c < L) val = *(const bf16x8*)(kc_base + (size_t)c * D + p * 8);
    else if (c < Ltot) val = *(const bf16x8*)(ks_base + (size_t)(c - L) * step_stride + p * 8);
    *(lds_bf16x8*)(sK + row * T::KROW + ((p ^ kswz<D>(row)) * 16)) = val;
  }
  // settled part of V^T (pieces of 8 positions), zero elsewhere
  for (int id = tid; id < D * 8; id += NW * 64) {
    const int d = id >> 3, q = id & 7;
    const int c0 = t0 + q * 8;
    bf16x8 val = {};
    if (c0 + 8 <= L) {
      val = *(const bf16x8*)(vc_base + vpos(d, c0, D));
    } else if (c0 < L) {
#pragma unroll
      for (int e = 0; e < 8; ++e) val[e] = c0 + e < L ? vc_base[vpos(d, c0 + e, D)] : (bf16)0.f;
    }
    *(lds_bf16x8*)(sV + d * T::VROW + ((q ^ vswz(d)) * 16)) = val;
  }
  wait_all();
  __builtin_amdgcn_s_barrier();
  // step rows: one 16 B load of 8 head-dim elements, scattered into 8 V^T rows
  const int j0 = max(t0, L), j1 = min(t0 + TK, Ltot);
  for (int id = tid; id < (j1 - j0) * (D / 8); id += NW * 64) {
    const int c = j0 + id / (D / 8), dc = id % (D / 8);
    const bf16x8 val = *(const bf16x8*)(vs_base + (size_t)(c - L) * step_stride + dc * 8);
    const int cl = c - t0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = dc * 8 + e;
      *(__attribute__((address_space(3))) bf16*)(sV + d * T::VROW + ((((cl >> 3) ^ vswz(d)) * 16)) + (cl & 7) * 2) = val[e];
    }
  }
}

// One 64-key tile: S^T = K.Q^T, mask (tail tiles only), online softmax,
// O^T += V^T.P^T.  LDS operand reads run a few MFMAs ahead of their use
// (a small ring of registers), so the LDS latency hides behind the MFMAs.
template <int D, bool MASK>
__device__ __forceinline__ void compute_tile(const lds_char* sK, const lds_char* sV, int t0, int L, int ke, int r, int k,
                                             float scale_log2, const bf16x8 (&qf)[D / 16], floatx16 (&o)[D / 32],
                                             float& m_run, float& l_run, int lane) {
  using T = Tile<D>;
  const int half = lane >> 5, l32 = lane & 31;
  // K operand of S^T item i (i = 2c + kb2): row 32*kb2 + sigma(l32), logical piece 2c + half
  const lds_char* kr0 = sK + sigma(l32) * T::KROW;
  const int ksw = kswz<D>(sigma(l32));  // same for rows +32
  auto kread = [&](int i) -> bf16x8 {
    const int kb2 = i & 1, c = i >> 1;
    return *(const lds_bf16x8*)(kr0 + kb2 * 32 * T::KROW + (((2 * c + half) ^ ksw) * 16));
  };
  // V operand of PV item j (j = 4*kc + db... for D/32 blocks): row 32*db + l32, logical piece 2*kc + half
  constexpr int NDB = D / 32;
  const lds_char* vr0 = sV + l32 * T::VROW;
  const int vsw = vswz(l32);  // rows 32*db + l32 share the low bits of l32
  auto vread = [&](int j) -> bf16x8 {
    const int db = j % NDB, kc = j / NDB;
    return *(const lds_bf16x8*)(vr0 + db * 32 * T::VROW + (((2 * kc + half) ^ vsw) * 16));
  };

  constexpr int NS = 2 * (D / 16);  // S^T MFMAs
  constexpr int RA = 3;             // read-ahead depth
  floatx16 s[2];
#pragma unroll
  for (int v = 0; v < 16; ++v) { s[0][v] = 0.f; s[1][v] = 0.f; }
  bf16x8 kbuf[RA + 1];
#pragma unroll
  for (int i = 0; i < RA; ++i) kbuf[i] = kread(i);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    if (i + RA < NS) kbuf[(i + RA) % (RA + 1)] = kread(i + RA);
    s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kbuf[i % (RA + 1)], qf[i >> 1], s[i & 1], 0, 0, 0);
  }
  // the first V operands load while the softmax runs
  constexpr int NPV = NDB * 4;
  constexpr int RV = 4;
  bf16x8 vbuf[RV];
#pragma unroll
  for (int j = 0; j < RV; ++j) vbuf[j] = vread(j);

  if (MASK) {
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = 8 * (v >> 2) + 4 * half + (v & 3);
        const int c = t0 + 32 * kb2 + sigma(i);
        const bool vis = c < ke && (c < L || step_visible(r, c - L, k));
        if (!vis) s[kb2][v] = -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb2][v]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  // The reference max only moves when a score exceeds it by more than 2^8:
  // in between, p = exp2(s - m_run) <= 256 stays far inside the fp32 and
  // bf16 ranges, and O, l keep one consistent scale, so most tiles skip the
  // rescale of O entirely.
  const float m_tile = mx * scale_log2;
  const bool grow = m_tile > m_run + 8.f;
  if (__any(grow)) {
    const float m_new = grow ? m_tile : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
  }
  bf16x8 pk[4];
  float psum = 0.f;
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const float p = __builtin_amdgcn_exp2f(s[kb2][8 * h + jj] * scale_log2 - m_run);
        psum += p;
        pk[2 * kb2 + h][jj] = (bf16)p;
      }
  l_run += psum;
#pragma unroll
  for (int j = 0; j < NPV; ++j) {
    const bf16x8 va = vbuf[j % RV];
    if (j + RV < NPV) vbuf[j % RV] = vread(j + RV);
    o[j % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pk[j / NDB], o[j % NDB], 0, 0, 0);
  }
}

// Step attention, bf16.  A sequence whose keys fit one chunk is normalised
// and written here; otherwise each chunk's partial goes to the workspace and
// attn_merge_kernel combines them (a kernel boundary is the cheap coherence
// point across XCDs; an in-kernel device-scope fence writes back and
// invalidates the whole L2 of the XCD).
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_split_bf16_kernel(AttnArgs a) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(1024))) char smK0[T::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char smV0[T::V_BYTES];
  __shared__ __attribute__((aligned(1024))) char smK1[T::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char smV1[T::V_BYTES];
  lds_char* sK0 = (lds_char*)smK0;
  lds_char* sV0 = (lds_char*)smV0;
  lds_char* sK1 = (lds_char*)smK1;
  lds_char* sV1 = (lds_char*)smV1;

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

  const int m = rb * (NW * 32) + wave * 32 + (lane & 31);  // this lane's query row
  const bool row_ok = m < a.M;
  const int r = row_ok ? m / a.G : 0;
  const int jh = row_ok ? m % a.G : 0;
  const int h = kvh * a.G + jh;
  bf16* orow = (bf16*)a.out + ((size_t)(b * a.R + r) * a.Hq + h) * D;

  const int L = a.lens[b];
  if (L < 0 || L > a.max_len) {  // contract violation: NaN rows, written once
    if (split == 0 && row_ok) {
      for (int e = half; e < D; e += 2) orow[e] = (bf16)NAN;
      if (a.lse && half == 0) a.lse[((size_t)b * a.Hq + h) * a.R + r] = NAN;
    }
    return;
  }
  const int Ltot = L + a.R;
  const int kb = split * a.chunk;
  if (kb >= Ltot) return;
  const int ke = min(kb + a.chunk, Ltot);
  const int n_valid = (Ltot + a.chunk - 1) / a.chunk;

  bf16x8 qf[D / 16];
  {
    const bf16* qrow = (const bf16*)a.q + ((size_t)(b * a.R + r) * a.Hq + h) * D;
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

  const size_t pair = (size_t)b * a.Hkv + kvh;
  const bf16* kc_base = (const bf16*)a.k_cache + pair * a.S_max * D;
  const bf16* vc_base = (const bf16*)a.v_cache + pair * D * a.S_max;
  const size_t step_stride = (size_t)a.Hkv * D;
  const bf16* ks_base = (const bf16*)a.k_step + (size_t)b * a.R * step_stride + kvh * D;
  const bf16* vs_base = (const bf16*)a.v_step + (size_t)b * a.R * step_stride + kvh * D;

  // Prefix tiles [kb, fast_end) stream through two LDS stages by direct
  // loads.  One barrier per tile: after it, every wave's loads of tile t have
  // landed and every wave is done with tile t-1, whose stage then receives
  // the loads of tile t+1 while tile t is computed.
  const int fast_end = min(ke, (L / TK) * TK);
  const int n_fast = fast_end > kb ? (fast_end - kb) / TK : 0;
  DmaPlan<D, NW> plan;
  dma_plan<D, NW>(plan, wave, lane);
  if (n_fast > 0) issue_tile<D, NW>(sK0, sV0, kc_base, vc_base, plan, kb, wave);
  for (int it = 0; it < n_fast; it += 2) {
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    if (it + 1 < n_fast) issue_tile<D, NW>(sK1, sV1, kc_base, vc_base, plan, kb + (it + 1) * TK, wave);
    compute_tile<D, false>(sK0, sV0, kb + it * TK, L, ke, r, a.k, a.scale_log2, qf, o, m_run, l_run, lane);
    if (it + 1 >= n_fast) break;
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    if (it + 2 < n_fast) issue_tile<D, NW>(sK0, sV0, kc_base, vc_base, plan, kb + (it + 2) * TK, wave);
    compute_tile<D, false>(sK1, sV1, kb + (it + 1) * TK, L, ke, r, a.k, a.scale_log2, qf, o, m_run, l_run, lane);
  }
  // tiles reaching past the prefix: staged through registers, masked by zone
  for (int t0 = max(kb, fast_end); t0 < ke; t0 += TK) {
    wait_all();
    __builtin_amdgcn_s_barrier();
    stage_tail_tile<D, NW>(sK0, sV0, kc_base, vc_base, ks_base, vs_base, step_stride, t0, L, Ltot, tid);
    wait_all();
    __builtin_amdgcn_s_barrier();
    compute_tile<D, true>(sK0, sV0, t0, L, ke, r, a.k, a.scale_log2, qf, o, m_run, l_run, lane);
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!row_ok) return;
  if (n_valid > 1) {  // one chunk of several: publish it for the merge kernel
    const size_t prow = (pair * a.n_split + split) * a.M + m;
    float* op = a.o_part + prow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        floatx4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = o[db][4 * g4 + e];
        *(floatx4*)(op + 32 * db + 8 * g4 + 4 * half) = w;
      }
    if (half == 0) a.ml_part[prow] = make_float2(m_run, l_tot);
    return;
  }
  const float inv = 1.f / l_tot;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (bf16)(o[db][4 * g4 + e] * inv);
      *(bf16x4*)(orow + 32 * db + 8 * g4 + 4 * half) = w;
    }
  if (a.lse && half == 0) a.lse[((size_t)b * a.Hq + h) * a.R + r] = (m_run + log2f(l_tot)) * kLn2;
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
      const float v = c < L ? vc_base[vpos(d, c, D)] : vs_base[(size_t)(c - L) * step_stride + d];
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
  if (n_valid == 1 && a.single_chunk_direct) return;  // the split kernel wrote it
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
  if (e != hipSuccess || a.n_split == 1) return e;
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
