// Step attention of one TiDAR decode step on gfx950: the two-waves-per-SIMD
// ("ping-pong") form of the bf16 kernel.
//
// The method's extra rows (k candidates + k*k draft slots per sequence,
// times the G query heads of a KV head) all read the same settled prefix,
// so they form a dense MFMA tile against each streamed key tile, and the
// extra blocks run on matrix throughput that a plain decode step leaves
// idle ("TiDAR : l'hybride de NVIDIA qui rédige par diffusion et parle de
// manière autorégressive", nodesdaily.com, paragraph on masking; abstract
// on fugumt.com).  Whether that throughput is really spent depends on
// keeping the matrix cores busy while the softmax runs, which is what this
// layout is for.
//
// Workgroup: eight waves, two per SIMD (wave w runs on SIMD w & 3; group
// w >> 2).  Each wave owns one tile of 16 query rows of one (sequence, KV
// head) for one key chunk; with NS = 1 a ninth tile is shared: group-0
// wave s scores its key block s (16 of each 64 keys) and publishes P
// through LDS, group-1 wave s accumulates O for head-dim blocks 2s, 2s+1.
// Every wave then carries 32 + 4 MFMAs per 64-key tile.
//
// Per 64-key tile j a wave runs two phases:
//   C(j)  MFMA cluster: S(j) = K(j).Q^T and O += V(j-1)^T.P(j-1)^T, with
//         K / V^T operands read from LDS;
//   M(j)  softmax of S(j) against the held row reference (exp2, sum, pack
//         to bf16) and this wave's share of the direct loads of K(j+3) and
//         V(j+2).
// The two groups run half a tile apart (group 1 passes one extra barrier
// first), so on every SIMD one wave's MFMA cluster overlaps the other
// wave's softmax and load issue: C and M of the two waves alternate at
// each workgroup barrier.
//
// Tiles that reach past the settled prefix (the step block) and, in a chunk
// without them, its first tile are processed before the loop with the
// exact softmax (true row maxima, rescale), which sets every row's
// reference; the loop keeps it and a tile sum above 2^64 sends the chunk to
// an exact recompute, as in the four-wave kernel.
#include <type_traits>

#include "attn_tile.h"
#include "common.h"
#include "launch.h"
#include "lds_dma.h"

namespace tidar {

namespace {

constexpr int PPW = 8;         // waves per workgroup, two per SIMD
constexpr int PPT = PPW * 64;  // threads per workgroup
constexpr int kPpDepth = 4;  // LDS operand reads in flight per wave in the MFMA phase

// s_waitcnt vmcnt(n) for a wave-uniform n that is not a compile-time
// constant (the load counts of the last ring steps).
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    default: wait_vmcnt<8>(); break;
  }
}

template <int D>
struct PpState {  // one wave's accumulators
  floatx4 o[D / 16];  // O^T of its tile: head-dim block db, rows in columns
  floatx4 os[2];      // group 1: O^T of the shared tile, head-dim blocks 2s, 2s+1
  floatx4 lv;         // its tile: row sums of the bf16 p of the pipelined tiles (every entry)
  float m, l;         // its tile: row reference (log2 units), this lane's part of the exact tiles' sum
  float ms, ls;       // shared tile: reference (same in every wave), group 0: its key block's sum
};

// The scores of one 64-key tile for the wave's own tile (S^T blocks kb4 =
// 0..3, key order of krow_of) and, for group 0 with a shared tile, of key
// block `simd` of the shared tile.
template <int D>
__device__ __forceinline__ void pp_scores(const lds_char* sK, const bf16x8 (&q)[D / 32], const bf16x8 (&qs)[D / 32],
                                          bool sh, floatx4 (&s)[4], floatx4& ss, int lane, int simd) {
  const floatx4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4)
      s[kb4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfrag<D>(sK, kb4, c, lane), q[c], c == 0 ? z : s[kb4], 0, 0, 0);
    if (sh) ss = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfrag<D>(sK, simd, c, lane), qs[c], c == 0 ? z : ss, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// O^T += V^T.P^T for the wave's own tile (all head-dim blocks) and, for
// group 1 with a shared tile, head-dim blocks 2s, 2s+1 of the shared tile
// with its P^T read from LDS.
template <int D>
__device__ __forceinline__ void pp_pv(const lds_char* sV, const bf16x8 (&p)[2], const bf16x8 (&ps)[2], bool sh,
                                      PpState<D>& st, int lane, int simd) {
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      st.o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vfrag<D>(sV, db, kc, lane), p[kc], st.o[db], 0, 0, 0);
    if (sh) {
#pragma unroll
      for (int e = 0; e < 2; ++e)
        st.os[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vfrag<D>(sV, 2 * simd + e, kc, lane), ps[kc], st.os[e], 0,
                                                          0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The C phase of the pipelined loop: S(j) from slot sK, then P.V of the
// previous tile from slot sV, as one fixed sequence of steps.  Each step
// reads one LDS operand and issues the MFMA that consumes it; the operand of
// the step DEPTH ahead is requested first, so DEPTH reads are in flight
// (what bounds the phase is the LDS reads' round trip, not their
// bandwidth).  The shared tile's MFMAs are steps of their own, with their
// own operand reads: after the four key blocks of each head-dim step, block
// `simd` again against the shared tile's Q (group 0); after the eight
// head-dim blocks of each key step, head-dim blocks 2s and 2s+1 again
// against the shared tile's P^T, read from LDS (group 1).
template <int D, int GRP, bool SH, bool DO_S, bool DO_PV, int DEPTH>
__device__ __forceinline__ void pp_c_phase(const lds_char* sK, const lds_char* sV, const lds_char* sP,
                                           const bf16x8 (&q)[D / 32], const bf16x8 (&qs)[D / 32], floatx4 (&s)[4],
                                           floatx4& ss, const bf16x8 (&p)[2], PpState<D>& st, int lane, int simd) {
  constexpr bool SH_S = SH && GRP == 0 && DO_S;
  constexpr bool SH_PV = SH && GRP == 1 && DO_PV;
  constexpr int SPC = 4 + (SH_S ? 1 : 0);        // score steps per head-dim step
  constexpr int PPK = D / 16 + (SH_PV ? 2 : 0);  // P.V steps per key step
  constexpr int NSS = DO_S ? (D / 32) * SPC : 0;
  constexpr int NPS = DO_PV ? 2 * PPK : 0;
  constexpr int NSTEP = NSS + NPS;
  const floatx4 z = {0.f, 0.f, 0.f, 0.f};
  auto frag = [&](int i) __attribute__((always_inline)) -> bf16x8 {
    if (i < NSS) {
      const int c = i / SPC, e = i % SPC;
      return kfrag<D>(sK, e < 4 ? e : simd, c, lane);
    }
    const int j = i - NSS, kc = j / PPK, e = j % PPK;
    return vfrag<D>(sV, e < D / 16 ? e : 2 * simd + (e - D / 16), kc, lane);
  };
  bf16x8 psh[SH_PV ? 2 : 1];
  if constexpr (SH_PV) {
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) psh[kc] = *(const lds_bf16x8*)(sP + (kc * 64 + lane) * 16);
  }
  bf16x8 fr[DEPTH + 1];
#pragma unroll
  for (int i = 0; i < DEPTH && i < NSTEP; ++i) fr[i] = frag(i);
  if constexpr (DO_PV) {
    // the row sums of P: an all-ones A operand against both key steps of
    // P^T (these need no operand read and cover the first read's latency)
    bf16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (bf16)1.f;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) st.lv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, p[kc], st.lv, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < NSTEP; ++i) {
    if (i + DEPTH < NSTEP) fr[(i + DEPTH) % (DEPTH + 1)] = frag(i + DEPTH);
    const bf16x8 f = fr[i % (DEPTH + 1)];
    if (i < NSS) {
      const int c = i / SPC, e = i % SPC;
      if (e < 4) s[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f, q[c], c == 0 ? z : s[e], 0, 0, 0);
      else ss = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f, qs[c], c == 0 ? z : ss, 0, 0, 0);
    } else {
      const int j = i - NSS, kc = j / PPK, e = j % PPK;
      if (e < D / 16) st.o[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f, p[kc], st.o[e], 0, 0, 0);
      else st.os[e - D / 16] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f, psh[kc], st.os[e - D / 16], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Softmax of one tile's scores against the held reference m: p =
// exp2(scale_log2 * s - m), P^T packed to bf16 in the B-operand layout of
// P.V.  SUM: also returns this lane's sum of p (the pipelined tiles take
// their sums on the matrix cores instead, from the packed p).
template <bool SUM = true>
__device__ __forceinline__ float pp_softmax(const floatx4 (&s)[4], float m, float sl2, bf16x8 (&p)[2]) {
  float sum = 0.f;
#pragma unroll
  for (int kb4 = 0; kb4 < 4; ++kb4) {
#pragma unroll
    for (int v = 0; v < 4; v += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb4][v], sl2, -m));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb4][v + 1], sl2, -m));
      if (SUM) sum += p0 + p1;
      p[kb4 >> 1][4 * (kb4 & 1) + v] = (bf16)p0;
      p[kb4 >> 1][4 * (kb4 & 1) + v + 1] = (bf16)p1;
    }
  }
  return sum;
}

// The shared tile's block: its four p values as bf16 into the LDS image of
// the P^T operand ([key step][lane][8 keys]); returns this lane's sum.
__device__ __forceinline__ float pp_softmax_shared(const floatx4& ss, float ms, float sl2, lds_char* sP, int lane,
                                                   int simd) {
  bf16x4 pk;
  float sum = 0.f;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float pv = __builtin_amdgcn_exp2f(fmaf(ss[v], sl2, -ms));
    sum += pv;
    pk[v] = (bf16)pv;
  }
  *(lds_bf16x4*)(sP + ((simd >> 1) * 64 + lane) * 16 + 8 * (simd & 1)) = pk;
  return sum;
}

template <int D, int NS, bool PAGED, bool TRAIN = false>
__global__ __launch_bounds__(PPT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_pp_kernel(AttnArgs a) {
  static_assert(D == 128, "the two-waves-per-SIMD layout is built for head dim 128");
  using T = Tile<D, PPW>;
  constexpr bool SH = NS > 0;
  __shared__ __attribute__((aligned(1024))) char smem[RING * (T::K_BYTES + T::V_BYTES)];
  __shared__ __attribute__((aligned(16))) char s_p[2][2 * 64 * 16];  // shared tile P^T, two buffers
  __shared__ float s_red[4][16];                                    // shared tile: per key block row values
  __shared__ int ovf_flag;
  lds_char* const sK0 = (lds_char*)smem;
  lds_char* const sV0 = sK0 + RING * T::K_BYTES;
  lds_char* const sP0 = (lds_char*)&s_p[0][0];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int simd = wave & 3, grp = wave >> 2;
  const int hi = lane >> 4;

  // (sequence, KV head, row block, key chunk) of this workgroup; decode
  // steps rank the units longest sequence first and deal each group of 8
  // ranks over the 8 XCDs in a snake (see the four-wave kernel)
  int rw, split, kvh, b;
  if (!TRAIN && a.B <= kMaxRankedB && (a.B * a.Hkv) % 8 == 0) {
    __shared__ int s_len[kMaxRankedB];
    __shared__ int s_pick;
    const int wpu = a.n_rowblk * a.n_split;
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int pos = j / wpu, within = j % wpu;
    const int rank = pos * 8 + ((pos & 1) ? 7 - x : x);
    const int rank_b = rank / a.Hkv;
    kvh = rank % a.Hkv;
    rw = within % a.n_rowblk;
    split = within / a.n_rowblk;
    for (int i = tid; i < a.B; i += PPT) s_len[i] = a.lens[i];
    __syncthreads();
    for (int i = tid; i < a.B; i += PPT) {
      const int li = s_len[i];
      int r = 0;
      for (int q2 = 0; q2 < a.B; ++q2) {
        const int lq = s_len[q2];
        r += (lq > li) | ((lq == li) & (q2 < i));
      }
      if (r == rank_b) s_pick = i;  // exactly one sequence has each rank
    }
    __syncthreads();
    b = s_pick;
  } else {
    int t = xcd_logical_block(blockIdx.x, gridDim.x);
    rw = t % a.n_rowblk;
    t /= a.n_rowblk;
    split = t % a.n_split;
    t /= a.n_split;
    kvh = t % a.Hkv;
    b = t / a.Hkv;
  }
  if (!TIDAR_CHECK(b >= 0 && b < a.B, TIDAR_CHECK_ROW, b)) b = 0;
  if (!TIDAR_CHECK(split < a.n_split, TIDAR_CHECK_CHUNK, split)) split = 0;

  // tiles [T0, T1) of this workgroup: wave w owns T0 + w; T0 + 8 is shared.
  // TRAIN: PPW + NS tiles per workgroup inside one half of the sequence, H
  // workgroups per half; workgroup ids alternate between the halves from
  // their last (heaviest) blocks down
  int T0, T1;
  if constexpr (TRAIN) {
    const int H = a.n_rowblk / 2, n16h = a.n16 / 2, tpw = PPW + NS;
    const int half = rw & 1, blk = H - 1 - (rw >> 1);
    T0 = half * n16h + blk * tpw;
    T1 = min(T0 + tpw, (half + 1) * n16h);
  } else {
    T0 = rw * a.n16 / a.n_rowblk;
    T1 = (rw + 1) * a.n16 / a.n_rowblk;
  }
  const int ti = T0 + wave;
  const int mrow = 16 * ti + (lane & 15);
  const bool ok = ti < T1 && mrow < a.M;
  const int mrow_s = 16 * (T0 + PPW) + (lane & 15);
  const bool ok_s = SH && T0 + PPW < T1 && mrow_s < a.M;
  const bool sh_s = SH && grp == 0;  // this wave scores a block of the shared tile
  auto out_row = [&](int m) __attribute__((always_inline)) {
    int r = m / a.G, h = kvh * a.G + m % a.G;
    if (!TIDAR_CHECK(r < a.R && h < a.Hq, TIDAR_CHECK_ROW, m)) r = h = 0;
    return (bf16*)a.out + ((size_t)(b * a.R + r) * a.Hq + h) * D;
  };
  auto lse_at = [&](int m) __attribute__((always_inline)) {
    int r = m / a.G, h = kvh * a.G + m % a.G;
    if (!TIDAR_CHECK(r < a.R && h < a.Hq, TIDAR_CHECK_ROW, m)) r = h = 0;
    return a.lse + ((size_t)b * a.Hq + h) * a.R + r;
  };

  const int L = TRAIN ? a.S_max : a.lens[b];  // TRAIN: every position's keys are in the buffers
  KvMap<D, PAGED> kv;
  const size_t pair = (size_t)b * a.Hkv + kvh;
  if constexpr (PAGED) {
    kv.k = (const bf16*)a.k_cache + (size_t)kvh * TK * D;
    kv.v = (const bf16*)a.v_cache + (size_t)kvh * D * TK;
    kv.tbl = a.block_table + (size_t)b * a.max_pages;
    kv.stride = (size_t)a.Hkv * TK * D;
  } else {
    kv.k = (const bf16*)a.k_cache + pair * a.S_max * D;
    kv.v = (const bf16*)a.v_cache + pair * D * a.S_max;
    kv.tbl = nullptr;
    kv.stride = (size_t)TK * D;
  }
  kv.n_tiles = PAGED ? a.max_pages : a.S_max / TK;
  kv.n_pages = a.n_pages;
  bool violated = !TRAIN && (L < 0 || L > a.max_len);
  if constexpr (PAGED) {  // every page holding a settled position must be in the pools
    bool bad = false;
    if (!violated)
      for (int pg = tid; pg < (L + TK - 1) / TK; pg += PPT) {
        const int32_t e = kv.tbl[pg];
        const bool eb = (unsigned)e >= (unsigned)a.n_pages;
        (void)TIDAR_CHECK(!eb, TIDAR_CHECK_PAGE, e);
        bad |= eb;
      }
    violated |= __syncthreads_or(bad) != 0;
  }
  if (violated) {  // contract violation: NaN rows, written once
    if (tid == 0) (void)TIDAR_CHECK(L >= 0 && L <= a.max_len, TIDAR_CHECK_LENS, L);
    if (split == 0) {
      auto nan_row = [&](int m) __attribute__((always_inline)) {
        bf16* orow = out_row(m);
        for (int db = 0; db < D / 16; ++db)
          for (int v = 0; v < 4; ++v) orow[16 * db + 4 * hi + v] = (bf16)NAN;
        if (a.lse && hi == 0) *lse_at(m) = NAN;
      };
      if (ok) nan_row(mrow);
      if (ok_s && wave == 0) nan_row(mrow_s);
    }
    return;
  }
  const int Ltot = TRAIN ? L : L + a.R;
  const int kb = split * a.chunk;
  if (kb >= Ltot) return;
  const int ke = min(kb + a.chunk, Ltot);
  const int n_valid = (Ltot + a.chunk - 1) / a.chunk;

  const size_t step_stride = (size_t)a.Hkv * D;
  const bf16* ks_base = TRAIN ? nullptr : (const bf16*)a.k_step + (size_t)b * a.R * step_stride + kvh * D;
  const bf16* vs_base = TRAIN ? nullptr : (const bf16*)a.v_step + (size_t)b * a.R * step_stride + kvh * D;

  // keys [kb, fast_end) through the rings; the tiles of [mA0, mA1) and
  // [mB0, mB1) masked.  Decode: [mA0, ke), the tiles reaching past the
  // prefix.  TRAIN: the key tiles every row of the workgroup sees in full
  // go through the ring; the few on its causal diagonal (clean half), or
  // at its blocks' prefix ends and on its own blocks (masked half), are
  // masked.
  int fast_end, mA0, mA1, mB0 = 0, mB1 = 0;
  if constexpr (TRAIN) {
    const int N = a.train_N, bs = a.train_bs;
    const int r_lo = 16 * T0 / a.G, r_hi = (min(16 * T1, a.M) - 1) / a.G;
    if (r_lo < N) {
      fast_end = (r_lo + 1) / TK * TK;
      mA1 = (r_hi + TK) / TK * TK;
    } else {
      const int lo_min = (r_lo - N) / bs * bs, lo_max = (r_hi - N) / bs * bs;
      fast_end = lo_min / TK * TK;
      mA1 = (lo_max + TK - 1) / TK * TK;
      mB0 = (N + lo_min) / TK * TK;
      mB1 = (N + min(lo_max + bs, N) + TK - 1) / TK * TK;
    }
    mA0 = fast_end;
  } else {
    fast_end = min(ke, (L / TK) * TK);
    mA0 = max(kb, fast_end);
    mA1 = ke;
  }
  const int n = fast_end > kb ? (fast_end - kb) / TK : 0;  // ring tiles
  const int tb = kb / TK;
  const int nA = (mA1 - mA0 + TK - 1) / TK, nB = (mB1 - mB0 + TK - 1) / TK;  // a range may end mid-tile
  const int n_tail = TRAIN ? nA + nB : nA;
  if (tid == 0) ovf_flag = 0;  // published by the first barrier below
  DmaPlan<D, PPW> plan;
  dma_plan<D, PPW>(plan, wave, lane);
  auto kslot = [&](int j) __attribute__((always_inline)) { return sK0 + (j & (RING - 1)) * T::K_BYTES; };
  auto vslot = [&](int j) __attribute__((always_inline)) { return sV0 + (j & (RING - 1)) * T::V_BYTES; };

  bf16x8 q[D / 32], qs[D / 32];
  auto load_q = [&](int m, bool ok_row, bf16x8 (&dst)[D / 32]) {
    int r = m / a.G, h = kvh * a.G + m % a.G;
    if (!TIDAR_CHECK(!ok_row || (r < a.R && h < a.Hq), TIDAR_CHECK_ROW, m)) r = h = 0;
    const bf16* qrow = (const bf16*)a.q + ((size_t)(b * a.R + r) * a.Hq + h) * D;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      bf16x8 zq = {};
      dst[c] = ok_row ? *(const bf16x8*)(qrow + 32 * c + 8 * hi) : zq;
    }
  };
  load_q(mrow, ok, q);
  if (sh_s) load_q(mrow_s, ok_s, qs);
  else {
#pragma unroll
    for (int c = 0; c < D / 32; ++c) qs[c] = (bf16x8){};
  }

  PpState<D> st;
  auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < D / 16; ++db) st.o[db] = (floatx4){0.f, 0.f, 0.f, 0.f};
    st.os[0] = st.os[1] = (floatx4){0.f, 0.f, 0.f, 0.f};
    st.m = st.ms = kNoMax;
    st.l = st.ls = 0.f;
    st.lv = (floatx4){0.f, 0.f, 0.f, 0.f};
  };
  reset();
  const float sl2 = a.scale_log2;
  floatx4 s[4], ss = {0.f, 0.f, 0.f, 0.f};
  bf16x8 p[2];

  // ---- exact path: one tile in slot RING-1, every wave together ----------
  // masked: the zone test applies (decode tiles past the prefix).  The row
  // reference moves to the true running max; O and the sums are rescaled.
  // The shared tile's four key blocks meet in LDS for their row maximum.
  lds_char* const sKx = kslot(RING - 1);
  lds_char* const sVx = vslot(RING - 1);
  // zone tests take step-row indices (decode) or positions (training)
  const int zoff = TRAIN ? 0 : L;
  auto zone = [&](int m) __attribute__((always_inline)) {
    return TRAIN ? train_zone(m / a.G, a.train_N, a.train_bs) : step_zone(m / a.G, a.k);
  };
  auto exact_tile = [&](int t0, bool masked) __attribute__((always_inline)) {
    pp_scores<D>(sKx, q, qs, sh_s, s, ss, lane, simd);
    if (masked) {
      const StepZone z = zone(mrow);
#pragma unroll
      for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int c = t0 + krow_of(kb4, 4 * hi + v);
          const bool vis = (c < ke) & z.sees(c - zoff);
          s[kb4][v] = vis ? s[kb4][v] : -INFINITY;
        }
      if (sh_s) {
        const StepZone zs = zone(mrow_s);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int c = t0 + krow_of(simd, 4 * hi + v);
          const bool vis = (c < ke) & zs.sees(c - zoff);
          ss[v] = vis ? ss[v] : -INFINITY;
        }
      }
    }
    // own tile: true row max over this tile, rescale, p
    float mx = -INFINITY;
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
      for (int v = 0; v < 4; ++v) mx = fmaxf(mx, s[kb4][v]);
    mx = row4_max(mx);
    {
      const float m_new = fmaxf(st.m, mx * sl2);
      const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
      st.m = m_new;
      st.l *= alpha;
      st.lv *= alpha;
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int v = 0; v < 4; ++v) st.o[db][v] *= alpha;
    }
    st.l += pp_softmax(s, st.m, sl2, p);
    if (SH) {
      // shared tile: each group-0 wave's block maximum, then the common one
      if (sh_s) {
        float bm = fmaxf(fmaxf(ss[0], ss[1]), fmaxf(ss[2], ss[3]));
        bm = row4_max(bm);
        if (hi == 0) s_red[simd][lane & 15] = bm;
      }
      wait_lgkmcnt0();
      barrier();
      const float bmx = fmaxf(fmaxf(s_red[0][lane & 15], s_red[1][lane & 15]),
                              fmaxf(s_red[2][lane & 15], s_red[3][lane & 15]));
      const float m_new = fmaxf(st.ms, bmx * sl2);
      const float alpha = __builtin_amdgcn_exp2f(st.ms - m_new);
      st.ms = m_new;
      if (sh_s) {
        st.ls *= alpha;
        st.ls += pp_softmax_shared(ss, st.ms, sl2, sP0, lane, simd);
      } else {
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int v = 0; v < 4; ++v) st.os[e][v] *= alpha;
      }
      wait_lgkmcnt0();
      barrier();  // P^T of the shared tile is in LDS; s_red is free again
    }
    bf16x8 ps[2];
    if (SH && !sh_s) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) ps[kc] = *(const lds_bf16x8*)(sP0 + (kc * 64 + lane) * 16);
    }
    pp_pv<D>(sVx, p, ps, SH && !sh_s, st, lane, simd);
    wait_lgkmcnt0();
  };

  // ---- masked tiles, staged through registers into slot RING-1 ----------
  StagedRows<D, PPT> staged;
  auto tail_t0 = [&](int i) __attribute__((always_inline)) {
    if constexpr (TRAIN) return i < nA ? mA0 + i * TK : mB0 + (i - nA) * TK;
    return mA0 + i * TK;
  };
  auto tail_issue = [&](int i) __attribute__((always_inline)) {
    const int t0 = tail_t0(i);
    stage_issue<D, PPT>(staged, t0 < L ? kv.ktile(t0 / TK) : nullptr, ks_base, vs_base, step_stride, t0, L, Ltot,
                        tid);
  };
  auto tail_stage = [&](int i) __attribute__((always_inline)) {
    const int t0 = tail_t0(i);
    barrier();  // every wave is done with the slot
    stage_commit<D, PPT>(staged, sKx, sVx, t0 < L ? kv.vtile(t0 / TK) : nullptr, t0, L, Ltot, tid,
                         [&] { wait_all(); });
    wait_all();
    barrier();
  };
  auto run_tails = [&]() __attribute__((always_inline)) {
    if (n_tail > 0) tail_issue(0);
    for (int i = 0; i < n_tail; ++i) {
      tail_stage(i);
      if (i + 1 < n_tail) tail_issue(i + 1);  // in flight while tile i computes
      exact_tile(tail_t0(i), true);
    }
  };
  // a ring tile through the exact path (direct loads into slot RING-1)
  auto exact_ring_tile = [&](int j) __attribute__((always_inline)) {
    barrier();  // every wave is done with the slot
    issue_k<D, PPW>(sKx, kv.ktile(tb + j), plan, wave);
    issue_v<D, PPW>(sVx, kv.vtile(tb + j), plan, wave);
    wait_vmcnt<0>();
    barrier();
    exact_tile(0, false);
  };

  run_tails();
  int j0 = 0;
  if (n > 0 && n_tail == 0) {  // no masked tile: the first ring tile sets the references
    exact_ring_tile(0);
    j0 = 1;
  }

  if (j0 < n) {
    // One workgroup barrier per key tile.  Between barriers B(j-1) and B(j)
    // group 0 runs C(j) then M(j) and group 1 runs M(j-1) then C(j), so the
    // two waves of a SIMD alternate between MFMA and softmax work without
    // a second rendezvous.  C(j): S(j) and P.V(j-1); M(i): softmax(i).
    // Direct loads: each tile's parts are spread over all eight waves; group
    // 0 issues K(i+3), V(i+2) in iteration i, group 1 K(i+2), V(i+1), into
    // ring slots whose last reader finished before B(i-1).  Before B(j) a
    // wave waits for its parts of K(j+1) and V(j), so C(j+1) reads complete
    // tiles.
    barrier();  // slots of the exact path are free
    auto kt_of = [&](int i) __attribute__((always_inline)) { return grp == 0 ? i + 3 : i + 2; };
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // LDS destinations in scalar registers
    auto issue_g = [&](int i) __attribute__((always_inline)) {
      const int tk = kt_of(i), tv = tk - 1;
      if (tk >= j0 && tk < n) issue_k<D, PPW>(kslot(tk), kv.ktile(tb + tk), plan, wave_s);
      if (tv >= j0 && tv < n) issue_v<D, PPW>(vslot(tv), kv.vtile(tb + tv), plan, wave_s);
    };
    // direct loads this wave issues in iteration i
    auto cnt = [&](int i) __attribute__((always_inline)) {
      const int tk = kt_of(i), tv = tk - 1;
      return T::NKW * (tk >= j0 && tk < n) + T::NVW * (tv >= j0 && tv < n);
    };
    // loads still allowed in flight before B(i): those issued after the
    // ones of K(i+1) and V(i)
    auto wait_parts = [&](int i) __attribute__((always_inline)) {
      wait_vmcnt_dyn(grp == 0 ? cnt(i - 1) + cnt(i) : cnt(i));
    };
    // ring prologue: the loads of iterations j0-3 .. j0-1
    issue_g(j0 - 3);
    issue_g(j0 - 2);
    issue_g(j0 - 1);
    wait_parts(j0 - 1);  // K(j0) has landed
    barrier();

    // the shared tile's P^T buffer of key tile i
    auto sPb = [&](int i) __attribute__((always_inline)) { return sP0 + (i & 1) * (2 * 64 * 16); };
    auto softmax = [&](auto grp_c, int i) __attribute__((always_inline)) {
      constexpr int G = decltype(grp_c)::value;
      pp_softmax<false>(s, st.m, sl2, p);
      if (G == 0 && SH) st.ls += pp_softmax_shared(ss, st.ms, sl2, sPb(i), lane, simd);
    };
    auto cphase = [&](auto grp_c, int j) __attribute__((always_inline)) {
      constexpr int G = decltype(grp_c)::value;
      __builtin_amdgcn_s_setprio(1);
      if (j > j0)
        pp_c_phase<D, G, SH, true, true, kPpDepth>(kslot(j), vslot(j - 1), sPb(j - 1), q, qs, s, ss, p, st, lane, simd);
      else
        pp_c_phase<D, G, SH, true, false, kPpDepth>(kslot(j), vslot(j), sPb(0), q, qs, s, ss, p, st, lane, simd);
      __builtin_amdgcn_s_setprio(0);
    };
    // one iteration; STEADY: every load of iterations j-1 and j exists
    // (j + 3 < n), so the loads go out unconditionally and the waits are
    // constants
    auto iter = [&](auto grp_c, auto steady_c, int j) __attribute__((always_inline)) {
      constexpr int G = decltype(grp_c)::value;
      constexpr bool STEADY = decltype(steady_c)::value;
      auto issue = [&]() __attribute__((always_inline)) {
        if (STEADY) {
          const int tk = G == 0 ? j + 3 : j + 2;
          issue_k<D, PPW>(kslot(tk), kv.ktile(tb + tk), plan, wave_s);
          issue_v<D, PPW>(vslot(tk - 1), kv.vtile(tb + tk - 1), plan, wave_s);
        } else {
          issue_g(j);
        }
      };
      if (G == 0) {
        cphase(grp_c, j);
        issue();  // before the softmax, which then runs while the loads are in flight
        softmax(grp_c, j);
      } else {
        if (j > j0) softmax(grp_c, j - 1);
        issue();
        cphase(grp_c, j);
      }
      if (STEADY) wait_vmcnt<(G == 0 ? 2 : 1) * (T::NKW + T::NVW)>();
      else wait_parts(j);
      wait_lgkmcnt0();
      barrier();
    };
    auto loop = [&](auto grp_c) __attribute__((always_inline)) {
      constexpr int G = decltype(grp_c)::value;
      int j = j0;
      for (; j + 3 < n; ++j) iter(grp_c, std::true_type{}, j);
      for (; j < n; ++j) iter(grp_c, std::false_type{}, j);
      // P.V(n-1)
      if (G == 1) softmax(grp_c, n - 1);
      __builtin_amdgcn_s_setprio(1);
      pp_c_phase<D, G, SH, false, true, kPpDepth>(kslot(n), vslot(n - 1), sPb(n - 1), q, qs, s, ss, p, st, lane, simd);
      __builtin_amdgcn_s_setprio(0);
    };
    if (grp == 0) loop(std::integral_constant<int, 0>{});
    else loop(std::integral_constant<int, 1>{});
    // A tile whose sum of p passed 2^64 leaves the row's total above it (the
    // sums only grow, and an infinite or NaN sum fails the test too): one
    // test after the loop.
    bool big = !(st.l <= kSumLimit) || !(st.lv[0] <= kSumLimit);
    if (SH && grp == 0) big |= !(st.ls <= kSumLimit);
    if (__any(big)) ovf_flag = 1;
    wait_all();
    barrier();
    if (ovf_flag) {  // a tile sum passed 2^64: the chunk again, exact tile by tile
      reset();
      for (int j = 0; j < n; ++j) exact_ring_tile(j);
      run_tails();
    }
  }

  // ---- output ----------------------------------------------------------
  auto emit = [&](int m, const floatx4* o, int db0, int ndb, float m_ref, float l_tot,
                  bool lse_lane) __attribute__((always_inline)) {
    if (n_valid > 1) {
      const size_t prow = (pair * a.n_split + split) * a.M + m;
      if (!TIDAR_CHECK(m < a.M, TIDAR_CHECK_ROW, m)) return;
      float* op = a.o_part + prow * D;
      for (int i = 0; i < ndb; ++i) *(floatx4*)(op + 16 * (db0 + i) + 4 * hi) = o[i];
      if (lse_lane) a.ml_part[prow] = make_float2(m_ref, l_tot);
      return;
    }
    bf16* orow = out_row(m);
    const float inv = 1.f / l_tot;
    for (int i = 0; i < ndb; ++i) {
      bf16x4 wv;
#pragma unroll
      for (int v = 0; v < 4; ++v) wv[v] = (bf16)(o[i][v] * inv);
      *(bf16x4*)(orow + 16 * (db0 + i) + 4 * hi) = wv;
    }
    if (a.lse && lse_lane) *lse_at(m) = (m_ref + log2f(l_tot)) * kLn2;
  };
  const float l_row = row4_sum(st.l) + st.lv[0];  // every lane takes part in the swaps
  if (ok) emit(mrow, st.o, 0, D / 16, st.m, l_row, hi == 0);
  if (SH) {
    wait_all();
    barrier();
    if (sh_s) {
      const float lt = row4_sum(st.ls);
      if (hi == 0) s_red[simd][lane & 15] = lt;
    }
    wait_lgkmcnt0();
    barrier();
    if (!sh_s && ok_s) {
      const float l_tot = s_red[0][lane & 15] + s_red[1][lane & 15] + s_red[2][lane & 15] + s_red[3][lane & 15];
      emit(mrow_s, st.os, 2 * simd, 2, st.ms, l_tot, simd == 0 && hi == 0);
    }
  }
}

template <int D, int NS>
hipError_t launch_pp(const AttnArgs& a, hipStream_t s) {
  const int nblk = a.B * a.Hkv * a.n_split * a.n_rowblk;
  if (a.block_table) hipLaunchKernelGGL((attn_pp_kernel<D, NS, true>), dim3(nblk), dim3(PPT), 0, s, a);
  else hipLaunchKernelGGL((attn_pp_kernel<D, NS, false>), dim3(nblk), dim3(PPT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_pp_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  if (a.D != 128) return hipErrorInvalidValue;
  return a.ns ? launch_pp<128, 1>(a, s) : launch_pp<128, 0>(a, s);
}

// Training-mask attention on the eight-wave kernel: 2 x H workgroups per
// (sequence, KV head), one row tile per wave (no shared tile).
hipError_t launch_train_attention_pp_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  if (a.D != 128 || a.n_split != 1 || a.ns != 0) return hipErrorInvalidValue;
  const int nblk = a.B * a.Hkv * a.n_rowblk;
  hipLaunchKernelGGL((attn_pp_kernel<128, 0, false, true>), dim3(nblk), dim3(PPT), 0, s, a);
  return hipGetLastError();
}

#if TIDAR_CHECKED
TIDAR_CHECK_RECORD_ACCESSOR(check_record_attention_pp)
#endif

}  // namespace tidar
