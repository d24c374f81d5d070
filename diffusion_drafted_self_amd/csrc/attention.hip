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
//   attn_pipe_bf16_kernel<D, NF, NS>  one workgroup per CU: four waves, one
//       per SIMD, each owning NF tiles of 16 query rows of one (b, kvh) and
//       one 16-key block of each of NS tiles they share, against one key
//       chunk.  Per 64-key tile, K and V^T arrive in LDS
//       rings by direct loads issued two and three tiles ahead; scores
//       S^T = K.Q^T and O^T += V^T.P^T run on v_mfma_f32_16x16x32_bf16, each
//       K / V^T operand read once from LDS and reused by the row tiles.
//       The loop body holds the softmax of tile t, the scores of tile t+1
//       and the P.V product of tile t-1, three independent streams in one
//       basic block, so the exp2 work of the VALU runs under the MFMAs.
//       Single-chunk sequences are normalised and written directly; others
//       leave the chunk's unnormalised output, reference max and sum.
//   attn_split_f32_kernel<D>  the f32 instance (VALU FMA; fp32 MFMA peak
//       equals VALU fp32 peak on this part), same partial format.
//   attn_merge_kernel<Out, D>  log-sum-exp merge of the chunks, one wave per
//       query row: normalised output (RNE to the output type) and the LSE.
#include "attn_tile.h"
#include "check.h"
#include "common.h"
#include "launch.h"
#include "lds_dma.h"

namespace tidar {

namespace {

constexpr int NWV = 4;  // waves per workgroup of the pipelined kernel, one per SIMD

// Row tiles of one wave.  A workgroup takes T tiles of 16 query rows of one
// (b, kvh): each of its four waves owns NF "full" tiles, and the remaining
// NS = T - 4*NF "shared" tiles are split by keys: wave w computes, for every
// 64-key tile, only score block w (16 keys) of each shared tile, keeps its
// own softmax state for that part, and the four parts are merged in LDS at
// the end.  Every wave then does the same work, NF + NS/4 tiles, whatever T
// is (T = 9: 2.25 tiles per wave instead of waves of 3 and 2 waiting for
// each other at every barrier).
//
// Running softmax state per tile (per part for a shared tile): the
// reference max m (log2 units, the same in the four lanes that hold a row)
// and this lane's part of the sum l.  Scores become p = exp2(scale_log2*s -
// m) against the current m without looking for the tile's max: while every
// p stays below 2^64 the fp32 sums and the bf16 P keep full relative
// precision (a reference below the true max only scales them), so a tile's
// sum of p decides.  Above 2^64 (always on the first tile, where m is
// kNoMax) the exact path runs: the true tile max across the four lanes of
// each row, rescale of O and l, p recomputed.

template <int D, int NF, int NS>
struct Acc {  // accumulators of one wave
  floatx4 o[at_least_1<NF>()][D / 16];
  floatx4 os[at_least_1<NS>()][D / 16];
  float m[at_least_1<NF>()], l[at_least_1<NF>()];
  float ms[at_least_1<NS>()], ls[at_least_1<NS>()];
};
template <int NF, int NS>
struct Scores {
  floatx4 s[at_least_1<NF>()][4];
  floatx4 ss[at_least_1<NS>()];  // block w of each shared tile
};
template <int NF, int NS>
struct Probs {
  bf16x8 p[at_least_1<NF>()][2];  // P^T operands of the two 32-key steps
  bf16x4 ps[at_least_1<NS>()];    // P^T operand of the 16 keys of block w
  float sum[at_least_1<NF>()], sums[at_least_1<NS>()];
};
template <int D, int NF, int NS>
struct QFrags {
  bf16x8 f[at_least_1<NF>()][D / 32];
  bf16x8 s[at_least_1<NS>()][D / 32];
};


template <int NF, int NS>
__device__ __forceinline__ void pair_to_p(Probs<NF, NS>& pr, bool shared, int t, int kb4, int v, float p0, float p1) {
  // convert here: the empty asm pins the packed pair to this point, so the
  // compiler cannot sink the conversion past the exact-path branch and keep
  // 32-bit p values alive instead
  unsigned u = __builtin_bit_cast(unsigned, (bf16x2){(bf16)p0, (bf16)p1});
  asm volatile("" : "+v"(u));
  const bf16x2 t2 = __builtin_bit_cast(bf16x2, u);
  if (!shared) {
    pr.p[t][kb4 >> 1][4 * (kb4 & 1) + v] = t2[0];
    pr.p[t][kb4 >> 1][4 * (kb4 & 1) + v + 1] = t2[1];
  } else {
    pr.ps[t][v] = t2[0];
    pr.ps[t][v + 1] = t2[1];
  }
}

// Softmax element pair e of a wave (full tiles' pairs first, then the
// shared parts'): p = exp2(scale_log2*s - m) against the held reference.
template <int NF, int NS>
__device__ __forceinline__ void sm_pair(int e, const Scores<NF, NS>& sc, Probs<NF, NS>& pr, const float* m,
                                        const float* ms, float sl2) {
  if (e < NF * 8) {
    const int t = e / 8, kb4 = (e / 2) % 4, v = 2 * (e % 2);
    const float p0 = __builtin_amdgcn_exp2f(fmaf(sc.s[t][kb4][v], sl2, -m[t]));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(sc.s[t][kb4][v + 1], sl2, -m[t]));
    pr.sum[t] += p0 + p1;
    pair_to_p(pr, false, t, kb4, v, p0, p1);
  } else {
    const int t = (e - NF * 8) / 2, v = 2 * ((e - NF * 8) % 2);
    const float p0 = __builtin_amdgcn_exp2f(fmaf(sc.ss[t][v], sl2, -ms[t]));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(sc.ss[t][v + 1], sl2, -ms[t]));
    pr.sums[t] += p0 + p1;
    pair_to_p(pr, true, t, 0, v, p0, p1);
  }
}

template <int NF, int NS>
__device__ __forceinline__ void sums_zero(Probs<NF, NS>& pr) {
#pragma unroll
  for (int t = 0; t < NF; ++t) pr.sum[t] = 0.f;
#pragma unroll
  for (int t = 0; t < NS; ++t) pr.sums[t] = 0.f;
}
template <int NF, int NS>
__device__ __forceinline__ bool sums_big(const Probs<NF, NS>& pr) {
  bool big = false;
#pragma unroll
  for (int t = 0; t < NF; ++t) big |= pr.sum[t] > kSumLimit;
#pragma unroll
  for (int t = 0; t < NS; ++t) big |= pr.sums[t] > kSumLimit;
  return big;
}
template <int D, int NF, int NS>
__device__ __forceinline__ void sums_commit(const Probs<NF, NS>& pr, Acc<D, NF, NS>& ac) {
#pragma unroll
  for (int t = 0; t < NF; ++t) ac.l[t] += pr.sum[t];
#pragma unroll
  for (int t = 0; t < NS; ++t) ac.ls[t] += pr.sums[t];
}

// Softmax of a whole tile against the held references (not pipelined).
template <int D, int NF, int NS>
__device__ __forceinline__ bool sm_tile(const Scores<NF, NS>& sc, Probs<NF, NS>& pr, const Acc<D, NF, NS>& ac,
                                        float sl2) {
  sums_zero(pr);
#pragma unroll
  for (int e = 0; e < NF * 8 + NS * 2; ++e) sm_pair<NF, NS>(e, sc, pr, ac.m, ac.ms, sl2);
  return sums_big(pr);
}

// Exact path for one row tile (or shared part): move each row's reference
// to the true running max, rescale O and l, recompute p.
template <int D, int NV>
__device__ __forceinline__ float exact_ref(const float* s, float& m, float& l, floatx4 (&o)[D / 16], float sl2) {
  float mx = -INFINITY;
#pragma unroll
  for (int v = 0; v < NV; ++v) mx = fmaxf(mx, s[v]);
  mx = row4_max(mx);
  const float m_new = fmaxf(m, mx * sl2);
  const float alpha = __builtin_amdgcn_exp2f(m - m_new);
  m = m_new;
  l *= alpha;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
#pragma unroll
    for (int v = 0; v < 4; ++v) o[db][v] *= alpha;
    __builtin_amdgcn_sched_barrier(0);
  }
  return m_new;
}

template <int D, int NF, int NS>
__device__ __forceinline__ void sm_exact(const Scores<NF, NS>& sc, Probs<NF, NS>& pr, Acc<D, NF, NS>& ac, float sl2) {
#pragma unroll
  for (int t = 0; t < NF; ++t) {
    float sv[16];
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
      for (int v = 0; v < 4; ++v) sv[4 * kb4 + v] = sc.s[t][kb4][v];
    exact_ref<D, 16>(sv, ac.m[t], ac.l[t], ac.o[t], sl2);
  }
#pragma unroll
  for (int t = 0; t < NS; ++t) {
    float sv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) sv[v] = sc.ss[t][v];
    exact_ref<D, 4>(sv, ac.ms[t], ac.ls[t], ac.os[t], sl2);
  }
  sm_tile<D, NF, NS>(sc, pr, ac, sl2);
  sums_commit(pr, ac);
}

template <int D, int NF, int NS>
__device__ __forceinline__ void softmax_commit(bool big, const Scores<NF, NS>& sc, Probs<NF, NS>& pr,
                                               Acc<D, NF, NS>& ac, float sl2) {
  if (__any(big)) sm_exact<D, NF, NS>(sc, pr, ac, sl2);
  else sums_commit(pr, ac);
}

template <int NT>
constexpr int operand_depth() { return NT <= 1 ? 8 : (NT == 2 ? 6 : 4); }

// One pipelined loop body: the scores of the next tile (S steps, one per
// (head-dim step, 16-key block)), the P.V product of the previous tile (PV
// steps, one per (32-key step, 16-row head-dim block)) and the softmax of
// the current tile, issued as a fixed sequence of steps.  Each step runs
// the full tiles' MFMAs on one LDS operand, reads the operand of the step
// DEPTH ahead and takes its slice of the softmax elements; the shared
// tiles' block-w MFMAs ride on the first steps of each kind (their
// operands are read at the start).  A scheduling fence after every step
// keeps the exp2 work spread under the MFMAs and bounds the operands in
// flight.  Returns true when some lane's softmax needs the exact path.
template <int D, int NF, int NS, bool DO_S, bool DO_PV>
__device__ __forceinline__ bool pipe_body(const lds_char* sKn, const lds_char* sVp, const QFrags<D, NF, NS>& q,
                                          Scores<NF, NS>& s_next, const Scores<NF, NS>& s_cur,
                                          Probs<NF, NS>& p_cur, const Probs<NF, NS>& p_prev,
                                          Acc<D, NF, NS>& ac, float sl2, int lane, int w) {
  using T = Tile<D>;
  constexpr int NSS = DO_S ? T::NDC * 4 : 0;
  constexpr int NPS = DO_PV ? 2 * T::NDB : 0;
  constexpr int NSTEP = NSS + NPS;
  constexpr int NE = NF * 8 + NS * 2;  // softmax element pairs of this lane
  constexpr int DEPTH = operand_depth<NF>();
  auto frag = [&](int i) -> bf16x8 {
    if (i < NSS) return kfrag<D>(sKn, i % 4, i / 4, lane);
    const int j = i - NSS;
    return vfrag<D>(sVp, j % T::NDB, j / T::NDB, lane);
  };
  const floatx4 z = {0.f, 0.f, 0.f, 0.f};
  bf16x8 ksh[T::NDC];   // shared tiles: K of block w, per head-dim step
  bf16x4 vsh[T::NDB];   // shared tiles: V^T of block w's keys, per head-dim block
  if (NS > 0) {
#pragma unroll
    for (int c = 0; c < T::NDC; ++c)
      if (DO_S) ksh[c] = kfrag<D>(sKn, w, c, lane);
#pragma unroll
    for (int db = 0; db < T::NDB; ++db)
      if (DO_PV) vsh[db] = vfrag16<D>(sVp, db, w, lane);
  }
  bf16x8 fr[DEPTH + 1];
  if (NF > 0) {
#pragma unroll
    for (int i = 0; i < DEPTH && i < NSTEP; ++i) fr[i] = frag(i);
  }
  sums_zero(p_cur);
#pragma unroll
  for (int i = 0; i < NSTEP; ++i) {
    if (NF > 0 && i + DEPTH < NSTEP) fr[(i + DEPTH) % (DEPTH + 1)] = frag(i + DEPTH);
    if (i < NSS) {
      const int c = i / 4, kb4 = i % 4;
#pragma unroll
      for (int t = 0; t < NF; ++t)
        s_next.s[t][kb4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[i % (DEPTH + 1)], q.f[t][c],
                                                                   c == 0 ? z : s_next.s[t][kb4], 0, 0, 0);
      if (kb4 == 0) {
#pragma unroll
        for (int t = 0; t < NS; ++t)
          s_next.ss[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ksh[c], q.s[t][c], c == 0 ? z : s_next.ss[t], 0, 0, 0);
      }
    } else {
      const int j = i - NSS, kc = j / T::NDB, db = j % T::NDB;
#pragma unroll
      for (int t = 0; t < NF; ++t)
        ac.o[t][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[i % (DEPTH + 1)], p_prev.p[t][kc], ac.o[t][db], 0, 0, 0);
      if (kc == 0) {
#pragma unroll
        for (int t = 0; t < NS; ++t)
          ac.os[t][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vsh[db], p_prev.ps[t], ac.os[t][db], 0, 0, 0);
      }
    }
#pragma unroll
    for (int e = i * NE / NSTEP; e < (i + 1) * NE / NSTEP; ++e) sm_pair<NF, NS>(e, s_cur, p_cur, ac.m, ac.ms, sl2);
    __builtin_amdgcn_sched_barrier(0);
  }
  return sums_big(p_cur);
}

// Scores of one tile alone, and P.V of one tile alone (ring prologue, tiles
// past the prefix, last tile, exact recompute).
template <int D, int NF, int NS>
__device__ __forceinline__ void s_tile(const lds_char* sK, const QFrags<D, NF, NS>& q, Scores<NF, NS>& s, int lane,
                                       int w) {
  using T = Tile<D>;
  const floatx4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < T::NDC; ++c) {
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4) {
      if (NF > 0) {
        const bf16x8 kf = kfrag<D>(sK, kb4, c, lane);
#pragma unroll
        for (int t = 0; t < NF; ++t)
          s.s[t][kb4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, q.f[t][c], c == 0 ? z : s.s[t][kb4], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (NS > 0) {
      const bf16x8 kf = kfrag<D>(sK, w, c, lane);
#pragma unroll
      for (int t = 0; t < NS; ++t)
        s.ss[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, q.s[t][c], c == 0 ? z : s.ss[t], 0, 0, 0);
    }
  }
}

template <int D, int NF, int NS>
__device__ __forceinline__ void pv_tile(const lds_char* sV, const Probs<NF, NS>& pr, Acc<D, NF, NS>& ac, int lane,
                                        int w) {
  using T = Tile<D>;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int db = 0; db < T::NDB; ++db) {
      if (NF > 0) {
        const bf16x8 vf = vfrag<D>(sV, db, kc, lane);
#pragma unroll
        for (int t = 0; t < NF; ++t)
          ac.o[t][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pr.p[t][kc], ac.o[t][db], 0, 0, 0);
      }
      if (NS > 0 && kc == 0) {
        const bf16x4 vf = vfrag16<D>(sV, db, w, lane);
#pragma unroll
        for (int t = 0; t < NS; ++t)
          ac.os[t][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, pr.ps[t], ac.os[t][db], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
}

// Step attention, bf16.  A sequence whose keys fit one chunk is normalised
// and written here; otherwise each chunk's partial goes to the workspace and
// attn_merge_kernel combines them (a kernel boundary is the cheap coherence
// point across XCDs; an in-kernel device-scope fence writes back and
// invalidates the whole L2 of the XCD).
//
// Prefix tiles j = 0..n-1 of the chunk flow through the LDS rings: K(j) is
// requested two loop iterations before the iteration that scores it (slot
// j%4), V(j) three before its P.V (slot j%4).  Iteration t waits for K(t+1) and V(t-1),
// passes one barrier (after which every wave is done with iteration t-1, so
// slots K(t-1) and V(t-2) are free), requests K(t+3) and V(t+2), then runs
// softmax(t) | scores(t+1) | P.V(t-1).  Tiles that reach past the settled
// prefix are staged through registers into the last slot first; the ring's
// prologue is requested once the last of them has landed.
//
// TRAIN: the duplicated training sequence (rows and keys are the T = 2N
// positions of one sequence, keys in the cache layouts with S_max = T).  A
// workgroup's rows lie in one half; the key tiles every row of it sees in
// full go through the ring, the few tiles on its causal diagonal, at its
// blocks' prefix ends and on its own blocks take the staged, masked path.
template <int D, int NF, int NS, bool PAGED, bool TRAIN = false>
__global__ __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_pipe_bf16_kernel(AttnArgs a) {
  using T = Tile<D>;
  constexpr int NSa = at_least_1<NS>();
  __shared__ __attribute__((aligned(1024))) char smem[RING * (T::K_BYTES + T::V_BYTES)];
  __shared__ int ovf_flag;
  lds_char* const sK0 = (lds_char*)smem;
  lds_char* const sV0 = sK0 + RING * T::K_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hi = lane >> 4;

  // The (sequence, KV head) unit this workgroup serves; a unit's n_rowblk
  // x n_split workgroups are consecutive and on one XCD (blocks are dealt
  // round-robin over the 8 XCDs, and each XCD starts its blocks in order).
  // Decode steps order the units longest sequence first (equal lengths in
  // sequence order) and deal each group of 8 ranks over the XCDs in a
  // snake, so every XCD gets a similar total and starts its longest units
  // first: with ragged lengths, consecutive sequences per XCD left some
  // XCDs with far more keys than others.  Each workgroup ranks the
  // lengths itself (B*B compares in LDS), so no pass before the kernel is
  // needed.  Other shapes keep the plain interleaved order.
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
    for (int i = tid; i < a.B; i += 64 * NWV) s_len[i] = a.lens[i];
    __syncthreads();
    for (int i = tid; i < a.B; i += 64 * NWV) {
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

  // this workgroup's tiles [T0, T1): wave w owns T0 + w*NF + f (f < NF);
  // the shared tiles T0 + 4*NF + s (s < NS) are split by key block
  int T0, T1;
  if constexpr (TRAIN) {
    // 4*NF + NS tiles per workgroup, H workgroups per half; workgroup ids
    // alternate between the halves from their last (heaviest) blocks down
    const int H = a.n_rowblk / 2, n16h = a.n16 / 2, tpw = 4 * NF + NS;
    const int half = rw & 1, blk = H - 1 - (rw >> 1);
    T0 = half * n16h + blk * tpw;
    T1 = min(T0 + tpw, (half + 1) * n16h);
  } else {
    T0 = rw * a.n16 / a.n_rowblk;
    T1 = (rw + 1) * a.n16 / a.n_rowblk;
  }
  int mrow[at_least_1<NF>()], mrow_s[NSa];
  bool ok[at_least_1<NF>()], ok_s[NSa];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int ti = T0 + wave * NF + f;
    mrow[f] = 16 * ti + (lane & 15);
    ok[f] = ti < T1 && mrow[f] < a.M;
  }
#pragma unroll
  for (int s2 = 0; s2 < NS; ++s2) {
    const int ti = T0 + 4 * NF + s2;
    mrow_s[s2] = 16 * ti + (lane & 15);
    ok_s[s2] = ti < T1 && mrow_s[s2] < a.M;
  }
  auto out_row = [&](int m) {
    int r = m / a.G, h = kvh * a.G + m % a.G;
    if (!TIDAR_CHECK(r < a.R && h < a.Hq, TIDAR_CHECK_ROW, m)) r = h = 0;
    return (bf16*)a.out + ((size_t)(b * a.R + r) * a.Hq + h) * D;
  };
  auto lse_at = [&](int m) {
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
      for (int pg = tid; pg < (L + TK - 1) / TK; pg += NWV * 64) {
        const int32_t e = kv.tbl[pg];
        const bool eb = (unsigned)e >= (unsigned)a.n_pages;
        (void)TIDAR_CHECK(!eb, TIDAR_CHECK_PAGE, e);
        bad |= eb;
      }
    violated |= __syncthreads_or(bad) != 0;
  }
  if (violated) {  // contract violation: NaN rows, written once
    if (tid == 0 && !TRAIN) (void)TIDAR_CHECK(L >= 0 && L <= a.max_len, TIDAR_CHECK_LENS, L);
    if (split == 0) {
      auto nan_row = [&](int m) {
        bf16* orow = out_row(m);
        for (int db = 0; db < D / 16; ++db)
          for (int v = 0; v < 4; ++v) orow[16 * db + 4 * hi + v] = (bf16)NAN;
        if (a.lse && hi == 0) *lse_at(m) = NAN;
      };
#pragma unroll
      for (int f = 0; f < NF; ++f)
        if (ok[f]) nan_row(mrow[f]);
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2)
        if (ok_s[s2] && wave == 0) nan_row(mrow_s[s2]);
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

  // keys [kb, fast_end) go through the rings unmasked; the tiles of
  // [mA0, mA1) and [mB0, mB1) take the staged path with the zone mask
  int fast_end, mA0, mA1, mB0 = 0, mB1 = 0;
  if constexpr (TRAIN) {
    const int N = a.train_N, bs = a.train_bs;
    const int r_lo = 16 * T0 / a.G, r_hi = (min(16 * T1, a.M) - 1) / a.G;
    if (r_lo < N) {  // clean rows: the causal diagonal
      fast_end = (r_lo + 1) / TK * TK;
      mA1 = (r_hi + TK) / TK * TK;
    } else {  // masked rows: their blocks' prefix ends, then their own blocks
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
  const int n = fast_end > kb ? (fast_end - kb) / TK : 0;  // tiles through the rings
  if (tid == 0) ovf_flag = 0;  // published by the first barrier below
  DmaPlan<D> plan;
  dma_plan<D>(plan, wave, lane);
  auto kslot = [&](int j) { return sK0 + (j & (RING - 1)) * T::K_BYTES; };
  auto vslot = [&](int j) { return sV0 + (j & (RING - 1)) * T::V_BYTES; };
  // ring prologue, as iterations -3..-1 would issue it: K(0); K(1), V(0); K(2), V(1)
  const int tb = kb / TK;  // the chunk's first tile
  // paged: the page of the last K tile requested; the V tile a ring step
  // requests is the K tile of the step before, so its page is known
  size_t pg_last_k = 0;
  // issued once the masked tiles below have staged their data (their waits
  // would otherwise include it), so it lands while they compute
  auto ring_prologue = [&]() {
    if (n > 0) issue_k<D>(kslot(0), kv.ktile(tb), plan, wave);
    if (n > 1) issue_k<D>(kslot(1), kv.ktile(tb + 1), plan, wave);
    if (n > 0) issue_v<D>(vslot(0), kv.vtile(tb), plan, wave);
    if (n > 2) {
      pg_last_k = kv.page(tb + 2);
      issue_k<D>(kslot(2), kv.k + pg_last_k * kv.stride, plan, wave);
    }
    if (n > 1) issue_v<D>(vslot(1), kv.vtile(tb + 1), plan, wave);
  };

  QFrags<D, NF, NS> q;
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
#pragma unroll
  for (int f = 0; f < NF; ++f) load_q(mrow[f], ok[f], q.f[f]);
#pragma unroll
  for (int s2 = 0; s2 < NS; ++s2) load_q(mrow_s[s2], ok_s[s2], q.s[s2]);

  Acc<D, NF, NS> ac;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    ac.m[f] = kNoMax;
    ac.l[f] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) ac.o[f][db] = (floatx4){0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int s2 = 0; s2 < NS; ++s2) {
    ac.ms[s2] = kNoMax;
    ac.ls[s2] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) ac.os[s2][db] = (floatx4){0.f, 0.f, 0.f, 0.f};
  }
  const float sl2 = a.scale_log2;
  Scores<NF, NS> sA, sB;
  Probs<NF, NS> pA, pB;

  // Masked tiles (decode: tiles reaching past the prefix): staged through
  // registers into the last slot (not used by the ring before its first
  // in-loop request), masked by zone, softmax against the held references
  // (the exact path when they overflow, so always for the first tile).
  const int zoff = TRAIN ? 0 : L;  // zone tests take step-row indices (decode) or positions (training)
  auto zone = [&](int m) { return TRAIN ? train_zone(m / a.G, a.train_N, a.train_bs) : step_zone(m / a.G, a.k); };
  const int nA = (mA1 - mA0 + TK - 1) / TK, nB = (mB1 - mB0 + TK - 1) / TK;  // a range may end mid-tile
  auto tail_t0 = [&](int i) { return i < nA ? mA0 + i * TK : mB0 + (i - nA) * TK; };
  // the two instances nearest the register limit stage one piece at a time
  constexpr bool kBatch = !(D == 128 && NF + NS >= 4);
  StagedRows<D> staged;
  auto tail_issue = [&](int i) {  // batched: masked tile i's loads, into registers
    if constexpr (kBatch) {
      const int t0 = tail_t0(i);
      const bool settled = t0 < L;  // the tile holds settled positions (its page is in the table)
      stage_issue<D>(staged, settled ? kv.ktile(t0 / TK) : nullptr, ks_base, vs_base, step_stride, t0, L, Ltot, tid);
    }
  };
  // The ring prologue goes out right after the last masked tile's loads
  // when that tile holds no settled position: its staging then issues no
  // load after them, so its waits can leave the prologue in flight (loads
  // complete in order) and the prologue lands during that tile's staging
  // and compute.  Otherwise (lean staging, or a settled part) it goes out
  // once that tile has landed, and lands while it computes.
  const int n_tail = nA + nB;
  const bool early = kBatch && n_tail > 0 && tail_t0(n_tail - 1) >= L;
  // the staged tile's loads (and LDS stores) are done; with the prologue
  // pending, its direct loads are the only ones that may still be in flight
  auto wait_staged = [&](bool prologue_pending) {
    if (!prologue_pending) {
      wait_all();
      return;
    }
    if (n > 2) wait_vmcnt<3 * T::NKW + 2 * T::NVW>();
    else if (n > 1) wait_vmcnt<2 * T::NKW + 2 * T::NVW>();
    else if (n > 0) wait_vmcnt<T::NKW + T::NVW>();
    else wait_vmcnt<0>();
    wait_lgkmcnt0();
  };
  auto tail_stage = [&](int i, bool prologue_pending) {  // masked tile i into the last slot
    const int t0 = tail_t0(i);
    barrier();
    const bool settled = t0 < L;
    if constexpr (kBatch)
      stage_commit<D>(staged, kslot(RING - 1), vslot(RING - 1), settled ? kv.vtile(t0 / TK) : nullptr, t0, L, Ltot,
                      tid, [&] { wait_staged(prologue_pending); });
    else
      stage_tail_tile_lean<D>(kslot(RING - 1), vslot(RING - 1), settled ? kv.ktile(t0 / TK) : nullptr,
                              settled ? kv.vtile(t0 / TK) : nullptr, ks_base, vs_base, step_stride, t0, L, Ltot, tid);
    wait_staged(prologue_pending);
    barrier();
  };
  // fresh: no reference is set yet (the kernel's first masked tile), so the
  // held-reference attempt, which would overflow, is skipped
  auto tail_compute = [&](int i, bool fresh) {
    const int t0 = tail_t0(i);
    lds_char* sK = kslot(RING - 1);
    lds_char* sV = vslot(RING - 1);
    s_tile<D, NF, NS>(sK, q, sA, lane, wave);
    // branch-free selects: no divergent control flow around the vector
    // element updates
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const StepZone z = zone(mrow[f]);
#pragma unroll
      for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int c = t0 + krow_of(kb4, 4 * hi + v);
          const bool vis = (c < ke) & z.sees(c - zoff);
          sA.s[f][kb4][v] = vis ? sA.s[f][kb4][v] : -INFINITY;
        }
    }
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) {
      const StepZone z = zone(mrow_s[s2]);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int c = t0 + krow_of(wave, 4 * hi + v);
        const bool vis = (c < ke) & z.sees(c - zoff);
        sA.ss[s2][v] = vis ? sA.ss[s2][v] : -INFINITY;
      }
    }
    // (the instances nearest the register limit always make the attempt)
    constexpr bool kSkipFresh = !(D == 128 && NF + NS >= 4);
    bool big = true;
    if (!(kSkipFresh && fresh)) big = sm_tile<D, NF, NS>(sA, pA, ac, sl2);
    softmax_commit<D, NF, NS>(big, sA, pA, ac, sl2);
    pv_tile<D, NF, NS>(sV, pA, ac, lane, wave);
    wait_lgkmcnt0();
  };
  // (the prologue's slots 0..RING-2 are not the masked tiles' slot)
  if (n_tail > 0) tail_issue(0);
  if (early && n_tail == 1) ring_prologue();
  for (int i = 0; i + 1 < n_tail; ++i) {
    tail_stage(i, false);
    tail_issue(i + 1);  // in flight while tile i computes
    if (early && i + 2 == n_tail) ring_prologue();
    tail_compute(i, i == 0);
  }
  if (n_tail > 0) {
    tail_stage(n_tail - 1, early);
    if (!early) ring_prologue();
    tail_compute(n_tail - 1, n_tail == 1);
  } else {
    ring_prologue();
  }

  if (n > 0) {
    // Tile 0 is scored against the held references, with the exact path
    // when they are unset (no masked tile in this chunk) or overflow, so
    // every row has a reference from an attained score before the
    // pipelined loop.  Inside the loop a reference is never moved: a tile
    // whose sum of p passes 2^64 (scores 64 above the reference, in log2
    // units) raises the workgroup's overflow flag, and the chunk is then
    // recomputed tile by tile with the exact path.
    if (n > 2) wait_vmcnt<2 * T::NKW + 2 * T::NVW>();
    else if (n > 1) wait_vmcnt<T::NKW + 2 * T::NVW>();
    else wait_vmcnt<T::NVW>();
    barrier();
    s_tile<D, NF, NS>(kslot(0), q, sA, lane, wave);
    {
      const bool big = sm_tile<D, NF, NS>(sA, pA, ac, sl2);
      softmax_commit<D, NF, NS>(big, sA, pA, ac, sl2);
    }

    // Iteration t: wait until only V(t), K(t+2), V(t+1) may be in flight.
    auto sync = [&](int it) {
      if (it + 2 < n) wait_vmcnt<T::NKW + 2 * T::NVW>();
      else if (it + 1 < n) wait_vmcnt<2 * T::NVW>();
      else wait_vmcnt<T::NVW>();
      wait_lgkmcnt0();
      barrier();
      if constexpr (PAGED) {
        const size_t pg_v = pg_last_k;  // tile it + 2, requested as K by the previous step (or the prologue)
        if (it + 3 < n) {
          pg_last_k = kv.page(tb + it + 3);
          issue_k<D>(kslot(it + 3), kv.k + pg_last_k * kv.stride, plan, wave);
        }
        if (it + 2 < n) issue_v<D>(vslot(it + 2), kv.v + pg_v * kv.stride, plan, wave);
      } else {
        if (it + 3 < n) issue_k<D>(kslot(it + 3), kv.ktile(tb + it + 3), plan, wave);
        if (it + 2 < n) issue_v<D>(vslot(it + 2), kv.vtile(tb + it + 2), plan, wave);
      }
    };
    bool overflow = false;
    auto commit_sum = [&](bool big, const Probs<NF, NS>& pr) {
      overflow |= __any(big);
      sums_commit(pr, ac);
    };
    if (n > 1) {  // t = 0: scores(1)
      sync(0);
      s_tile<D, NF, NS>(kslot(1), q, sB, lane, wave);
    }
    // iteration t: softmax(t) | scores(t+1) | P.V(t-1); the scores after
    // the last tile come from a stale slot and are never used
    int it = 1;
    for (; it + 1 < n; it += 2) {
      sync(it);
      commit_sum(pipe_body<D, NF, NS, true, true>(kslot(it + 1), vslot(it - 1), q, sA, sB, pB, pA, ac, sl2, lane, wave),
                 pB);
      sync(it + 1);
      commit_sum(pipe_body<D, NF, NS, true, true>(kslot(it + 2), vslot(it), q, sB, sA, pA, pB, ac, sl2, lane, wave),
                 pA);
    }
    if (it < n) {  // odd last tile: softmax(n-1) in sB
      sync(it);
      commit_sum(pipe_body<D, NF, NS, false, true>(kslot(it), vslot(it - 1), q, sA, sB, pB, pA, ac, sl2, lane, wave),
                 pB);
    }
    if (overflow) ovf_flag = 1;
    wait_all();
    barrier();
    pv_tile<D, NF, NS>(vslot(n - 1), ((n - 1) & 1) ? pB : pA, ac, lane, wave);

    if (ovf_flag) {  // the same for every wave after the barrier
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        ac.m[f] = kNoMax;
        ac.l[f] = 0.f;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) ac.o[f][db] = (floatx4){0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) {
        ac.ms[s2] = kNoMax;
        ac.ls[s2] = 0.f;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) ac.os[s2][db] = (floatx4){0.f, 0.f, 0.f, 0.f};
      }
      for (int j = 0; j < n; ++j) {
        barrier();
        issue_k<D>(kslot(0), kv.ktile(tb + j), plan, wave);
        issue_v<D>(vslot(0), kv.vtile(tb + j), plan, wave);
        wait_vmcnt<0>();
        barrier();
        s_tile<D, NF, NS>(kslot(0), q, sA, lane, wave);
        const bool big = sm_tile<D, NF, NS>(sA, pA, ac, sl2);
        softmax_commit<D, NF, NS>(big, sA, pA, ac, sl2);
        pv_tile<D, NF, NS>(vslot(0), pA, ac, lane, wave);
        wait_lgkmcnt0();
      }
      for (int i = 0; i < nA + nB; ++i) {
        tail_issue(i);
        tail_stage(i, false);  // nothing else is in flight here
        tail_compute(i, false);
      }
    }
  }

  // Output of a finished row tile: normalised bf16 rows and the LSE, or the
  // unnormalised partial of this chunk for the merge kernel.
  auto emit = [&](int m, bool ok_row, const floatx4 (&o)[D / 16], float m_ref, float l_tot) {
    if (!ok_row) return;
    if (n_valid > 1) {
      const size_t prow = (pair * a.n_split + split) * a.M + m;
      if (!TIDAR_CHECK(m < a.M, TIDAR_CHECK_ROW, m)) return;
      float* op = a.o_part + prow * D;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) *(floatx4*)(op + 16 * db + 4 * hi) = o[db];
      if (hi == 0) a.ml_part[prow] = make_float2(m_ref, l_tot);
      return;
    }
    bf16* orow = out_row(m);
    const float inv = 1.f / l_tot;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      typedef __bf16 bf16x4o __attribute__((ext_vector_type(4)));
      bf16x4o wv;
#pragma unroll
      for (int v = 0; v < 4; ++v) wv[v] = (bf16)(o[db][v] * inv);
      *(bf16x4o*)(orow + 16 * db + 4 * hi) = wv;
    }
    if (a.lse && hi == 0) *lse_at(m) = (m_ref + log2f(l_tot)) * kLn2;
  };

#pragma unroll
  for (int f = 0; f < NF; ++f) {
    float lt = ac.l[f];
    lt = row4_sum(lt);
    emit(mrow[f], ok[f], ac.o[f], ac.m[f], lt);
  }

  if (NS > 0) {
    // Merge the four key-block parts of each shared tile through LDS (the
    // ring is free now): part w of tile s is O (16 rows x D, this wave's
    // register layout), its reference and its sum.  Wave w then combines
    // head-dim blocks w, w+4, ... of every shared tile and writes them.
    float* mo = (float*)smem;                       // [NS][4 parts][D/16][64 lanes][4]
    float* mml = mo + NS * 4 * (D / 16) * 64 * 4;  // [NS][4 parts][16 rows][2]
    wait_all();
    barrier();
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) {
      float lt = ac.ls[s2];
      lt = row4_sum(lt);
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
        *(floatx4*)(mo + (((s2 * 4 + wave) * (D / 16) + db) * 64 + lane) * 4) = ac.os[s2][db];
      if (hi == 0) {
        mml[((s2 * 4 + wave) * 16 + (lane & 15)) * 2] = ac.ms[s2];
        mml[((s2 * 4 + wave) * 16 + (lane & 15)) * 2 + 1] = lt;
      }
    }
    wait_all();
    barrier();
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) {
      const int r16 = lane & 15;
      float mp[4], lp[4], mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        mp[w] = mml[((s2 * 4 + w) * 16 + r16) * 2];
        lp[w] = mml[((s2 * 4 + w) * 16 + r16) * 2 + 1];
        mx = fmaxf(mx, mp[w]);
      }
      float wt[4], l_tot = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        wt[w] = __builtin_amdgcn_exp2f(mp[w] - mx);
        l_tot += wt[w] * lp[w];
      }
      floatx4 om[D / 16];
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        om[db] = (floatx4){0.f, 0.f, 0.f, 0.f};
        if (db % 4 != wave) continue;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const floatx4 x = *(const floatx4*)(mo + (((s2 * 4 + w) * (D / 16) + db) * 64 + lane) * 4);
#pragma unroll
          for (int v = 0; v < 4; ++v) om[db][v] = fmaf(wt[w], x[v], om[db][v]);
        }
      }
      if (!ok_s[s2]) continue;
      const int m = mrow_s[s2];
      if (n_valid > 1) {
        const size_t prow = (pair * a.n_split + split) * a.M + m;
        if (!TIDAR_CHECK(m < a.M, TIDAR_CHECK_ROW, m)) continue;
        float* op = a.o_part + prow * D;
#pragma unroll
        for (int db = 0; db < D / 16; ++db)
          if (db % 4 == wave) *(floatx4*)(op + 16 * db + 4 * hi) = om[db];
        if (wave == 0 && hi == 0) a.ml_part[prow] = make_float2(mx, l_tot);
        continue;
      }
      bf16* orow = out_row(m);
      const float inv = 1.f / l_tot;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        if (db % 4 != wave) continue;
        typedef __bf16 bf16x4o __attribute__((ext_vector_type(4)));
        bf16x4o wv;
#pragma unroll
        for (int v = 0; v < 4; ++v) wv[v] = (bf16)(om[db][v] * inv);
        *(bf16x4o*)(orow + 16 * db + 4 * hi) = wv;
      }
      if (a.lse && wave == 0 && hi == 0) *lse_at(m) = (mx + log2f(l_tot)) * kLn2;
    }
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
  if (L < 0 || L > a.max_len) {
    if (lane == 0) (void)TIDAR_CHECK(false, TIDAR_CHECK_LENS, L);
    return;
  }
  const int Ltot = L + a.R;
  const int kb = split * a.chunk;
  if (kb >= Ltot) return;
  const int ke = min(kb + a.chunk, Ltot);
  const int r = m / a.G, jh = m % a.G;
  if (!TIDAR_CHECK(min(ke, L) <= a.S_max, TIDAR_CHECK_KEY_TILE, ke)) return;
  if (!TIDAR_CHECK(ke - kb <= 1024, TIDAR_CHECK_CHUNK, ke - kb)) return;

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

// Log-sum-exp merge of the key chunks: one wave per (b, kvh, row m).  Lane
// t takes chunk t (and t + 64, ...) for the reference max and the weights,
// and the chunk outputs are read eight chunks at a time, every load of a
// batch in flight together: the merge costs a few memory round trips
// whatever the number of chunks, not one per chunk.
template <typename OutT, int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  constexpr int E = D / 64;  // elements per lane
  constexpr int NB = 8;      // chunk outputs per batch of loads
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
  bool violated = L < 0 || L > a.max_len;
  if (a.block_table && !violated) {  // paged: the pages the split kernel checked
    bool bad = false;
    const int32_t* tbl = a.block_table + (size_t)b * a.max_pages;
    for (int pg = lane; pg < (L + VPAGE - 1) / VPAGE; pg += 64) bad |= (unsigned)tbl[pg] >= (unsigned)a.n_pages;
    violated = __any(bad);
  }
  if (violated) {  // (the split kernel recorded it)
    for (int e = 0; e < E; ++e) store_out(orow + lane * E + e, NAN);
    if (lse && lane == 0) *lse = NAN;
    return;
  }
  int n_valid = (L + a.R + a.chunk - 1) / a.chunk;
  if (!TIDAR_CHECK(n_valid <= a.n_split, TIDAR_CHECK_CHUNK, n_valid)) n_valid = a.n_split;
  if (n_valid == 1 && a.single_chunk_direct) return;  // the split kernel wrote it
  const size_t base = (size_t)pr * a.n_split * a.M + m;

  float mx = -INFINITY;
  for (int s = lane; s < n_valid; s += 64) mx = fmaxf(mx, a.ml_part[base + (size_t)s * a.M].x);
  mx = wave_max(mx);
  float den = 0.f, acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int g0 = 0; g0 < n_valid; g0 += 64) {
    // this lane's chunk g0 + lane: its weight (0 past the last chunk)
    float wl = 0.f;
    if (g0 + lane < n_valid) {
      const float2 ml = a.ml_part[base + (size_t)(g0 + lane) * a.M];
      wl = exp2f(ml.x - mx);
      den = fmaf(wl, ml.y, den);
    }
    const int ng = min(64, n_valid - g0);
    for (int u0 = 0; u0 < ng; u0 += NB) {
      float o[NB][E];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const float* op = a.o_part + (base + (size_t)(g0 + u0 + u) * a.M) * D + lane * E;
#pragma unroll
        for (int e = 0; e < E; ++e) o[u][e] = u0 + u < ng ? op[e] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const float wu = __shfl(wl, u0 + u);  // lanes past the last chunk hold 0
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = fmaf(wu, o[u][e], acc[e]);
      }
    }
  }
  den = wave_sum(den);
  const float inv = 1.f / den;
#pragma unroll
  for (int e = 0; e < E; ++e) store_out(orow + lane * E + e, acc[e] * inv);
  if (lse && lane == 0) *lse = (mx + log2f(den)) * kLn2;
}

template <int D, int NF, int NS>
hipError_t launch_bf16_pipe(const AttnArgs& a, hipStream_t s) {
  const int nblk = a.B * a.Hkv * a.n_split * a.n_rowblk;
  if (a.block_table) hipLaunchKernelGGL((attn_pipe_bf16_kernel<D, NF, NS, true>), dim3(nblk), dim3(NWV * 64), 0, s, a);
  else hipLaunchKernelGGL((attn_pipe_bf16_kernel<D, NF, NS, false>), dim3(nblk), dim3(NWV * 64), 0, s, a);
  return hipGetLastError();
}

template <int D, int NF>
hipError_t launch_bf16_train(const AttnArgs& a, hipStream_t s) {
  const int nblk = a.B * a.Hkv * a.n_rowblk;
  hipLaunchKernelGGL((attn_pipe_bf16_kernel<D, NF, 0, false, true>), dim3(nblk), dim3(NWV * 64), 0, s, a);
  return hipGetLastError();
}

// (full tiles per wave, shared tiles per workgroup) shapes that are built
template <int D>
hipError_t launch_bf16_shape(const AttnArgs& a, hipStream_t s) {
  switch (a.nf * 4 + a.ns) {
    case 1: return launch_bf16_pipe<D, 0, 1>(a, s);
    case 2: return launch_bf16_pipe<D, 0, 2>(a, s);
    case 3: return launch_bf16_pipe<D, 0, 3>(a, s);
    case 4: return launch_bf16_pipe<D, 1, 0>(a, s);
    case 5: return launch_bf16_pipe<D, 1, 1>(a, s);
    case 6: return launch_bf16_pipe<D, 1, 2>(a, s);
    case 7: return launch_bf16_pipe<D, 1, 3>(a, s);
    case 8: return launch_bf16_pipe<D, 2, 0>(a, s);
    case 9: return launch_bf16_pipe<D, 2, 1>(a, s);
    case 10: return launch_bf16_pipe<D, 2, 2>(a, s);
    case 12: return launch_bf16_pipe<D, 3, 0>(a, s);
    default: return hipErrorInvalidValue;
  }
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
  if (a.pp) e = launch_attention_pp_bf16(a, s);
  else if (a.D == 128) e = launch_bf16_shape<128>(a, s);
  else if (a.D == 64) e = launch_bf16_shape<64>(a, s);
  if (e != hipSuccess || a.n_split == 1) return e;
  return a.D == 128 ? launch_merge<bf16, 128>(a, s) : launch_merge<bf16, 64>(a, s);
}

hipError_t launch_train_attention_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  if (a.ns != 0) return hipErrorInvalidValue;
  if (a.D == 128) {
    if (a.nf == 1) return launch_bf16_train<128, 1>(a, s);
    if (a.nf == 2) return launch_bf16_train<128, 2>(a, s);
    if (a.nf == 3) return launch_bf16_train<128, 3>(a, s);
  } else if (a.D == 64) {
    if (a.nf == 1) return launch_bf16_train<64, 1>(a, s);
    if (a.nf == 2) return launch_bf16_train<64, 2>(a, s);
    if (a.nf == 3) return launch_bf16_train<64, 3>(a, s);
  }
  return hipErrorInvalidValue;
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

#if TIDAR_CHECKED
TIDAR_CHECK_RECORD_ACCESSOR(check_record_attention)
#endif

}  // namespace tidar
