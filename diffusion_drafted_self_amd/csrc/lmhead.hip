// LM head fused with the argmax of greedy verification, on gfx950.
//
// The single pass gives both the joint distribution that verifies and the
// marginals that draft ("TiDAR: Think in Diffusion, Talk in
// Autoregression", mauroscia.it, section "2. Single Forward Pass &
// Structured Attention Mask"); verification only needs each row's argmax
// ("TiDAR : l'hybride de NVIDIA qui rédige par diffusion et parle de manière
// autorégressive", nodesdaily.com, paragraphs on scoring left to right and
// on drafting for every outcome).  So the LM head's output never leaves the
// chip: a workgroup computes logits = h . W^T for every hidden row of the
// pass against 256 vocabulary rows of W, on v_mfma_f32_16x16x32_bf16, and
// keeps only each row's (max, lower index) over those 256 entries -- the
// chunk results the greedy selection and draft finalisation reduce.
//
// The product is bound by reading W (V x d bf16) once per pass: at most 144
// hidden rows share each W tile, under the bf16 ridge.  W and the hidden
// rows stream through a 3-stage LDS ring of 64-deep slices by direct
// global->LDS loads.  The hidden rows are reloaded for every vocabulary
// slice, so the wider the slice, the smaller their share of the loads.
// LDS rows are 128 B, their 16 B pieces XOR-swizzled by the row's low three
// bits, which makes the operand reads (16 consecutive rows, four pieces
// across the lane groups) free of bank conflicts.
#include <algorithm>
#include <climits>

#include "common.h"
#include "launch.h"
#include "lds_dma.h"

namespace tidar {

namespace {

constexpr int LK = 64;                    // hidden elements per stage
constexpr int ROWB = LK * 2;              // bytes per LDS row
constexpr int STAGES = 3;
constexpr int W_BYTES = kLmChunk * ROWB;  // 32 KB of W per stage
constexpr int W_LD = W_BYTES / 1024 / 4;  // direct loads per wave per stage: W
constexpr int CT = kLmChunk / 16 / 4;     // column tiles per wave
constexpr int KK = LK / 32;               // MFMA k-steps per stage

__device__ __forceinline__ int swz(int row) { return row & 7; }

// MT row tiles of 16 hidden rows per workgroup (the launch picks the fewest
// that hold its rows, so the loops below unroll completely and no stage
// loads hidden rows it does not use).
template <int MT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void lmhead_argmax_kernel(LmArgs a) {
  constexpr int ROWS = MT * 16;
  constexpr int H_BYTES = ROWS * ROWB;      // hidden rows per stage
  constexpr int STAGE_BYTES = W_BYTES + H_BYTES;
  constexpr int H_BLK = H_BYTES / 1024;     // 1 KB blocks of hidden rows (2 per row tile)
  constexpr int H_LD = (H_BLK + 3) / 4;     // ... per wave (the last block may be loaded twice)
  constexpr int LD = W_LD + H_LD;           // direct loads per wave per stage
  static_assert(STAGES == 3 && LD < 64, "vmcnt accounting below");
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE_BYTES];
  __shared__ float sv[4][ROWS];
  __shared__ int si[4][ROWS];
  lds_char* const ring = (lds_char*)smem;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = blockIdx.x;
  const int v0 = chunk * kLmChunk;
  const int r0 = blockIdx.y * ROWS;
  const int nrow = min(ROWS, a.rows - r0);

  // element offset of hidden row m of this pass
  auto hrow = [&](int m) -> size_t {
    if (!a.draft) return (size_t)m * a.d;
    const int b = m / (a.k - 1), s = 1 + m % (a.k - 1);
    const int g = min(max(a.group[b], 0), a.k - 1);  // written by the selection; clamped regardless
    return (((size_t)b * a.k + g) * a.k + s) * a.d;
  };
  // this wave's direct loads: lane t of a 1 KB block lands at row 8*blk + t/8,
  // physical piece t%8, so it fetches logical piece (t%8) ^ swz(row); rows
  // past V or past the pass's rows repeat the last valid one
  unsigned off[LD];
  unsigned dst[LD];  // byte offset inside a stage's slot
#pragma unroll
  for (int ii = 0; ii < W_LD; ++ii) {
    const int row = (wave * W_LD + ii) * 8 + lane / 8;
    const int p = (lane & 7) ^ swz(row);
    off[ii] = (unsigned)((size_t)min(v0 + row, a.V - 1) * a.d * 2 + p * 16);
    dst[ii] = (wave * W_LD + ii) * 1024;
  }
#pragma unroll
  for (int ii = 0; ii < H_LD; ++ii) {
    const int blk = min(wave + 4 * ii, H_BLK - 1);
    const int row = blk * 8 + lane / 8;
    const int p = (lane & 7) ^ swz(row);
    off[W_LD + ii] = (unsigned)(hrow(r0 + min(row, nrow - 1)) * 2 + p * 16);
    dst[W_LD + ii] = W_BYTES + blk * 1024;
  }
  // load q of this wave's share of stage st (W rows from a.w, hidden rows from a.h)
  auto issue_one = [&](int st, int q) {
    lds_char* slot = ring + (st % STAGES) * STAGE_BYTES;
    const unsigned dk = (unsigned)st * ROWB;
    // W is read once per pass (nontemporal); the hidden rows again for every slice
    if (q < W_LD) dma_b128<true>((const char*)a.w, off[q] + dk, slot + dst[q]);
    else dma_b128<false>((const char*)a.h, off[q] + dk, slot + dst[q]);
  };

  const int nst = a.d / LK;
#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st)
    if (st < nst) {
#pragma unroll
      for (int q = 0; q < LD; ++q) issue_one(st, q);
    }

  floatx4 acc[MT][CT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < CT; ++j) acc[i][j] = (floatx4){0.f, 0.f, 0.f, 0.f};

  for (int st = 0; st < nst; ++st) {
    // stage st has landed once at most the stage issued after it is in flight
    if (st + 1 < nst) wait_vmcnt<LD>();
    else wait_vmcnt<0>();
    wait_lgkmcnt0();  // this wave's reads of the slot refilled below are done
    barrier();        // ... and every wave's
    const bool refill = st + STAGES - 1 < nst;
    const lds_char* sw = ring + (st % STAGES) * STAGE_BYTES;
    const lds_char* sh = sw + W_BYTES;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int p = 4 * kk + (lane >> 4);
      bf16x8 bfr[CT], afr[MT];
#pragma unroll
      for (int j = 0; j < CT; ++j) {
        const int vr = 16 * (wave * CT + j) + (lane & 15);
        bfr[j] = *(const lds_bf16x8*)(sw + vr * ROWB + ((p ^ swz(vr)) * 16));
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int hr = 16 * i + (lane & 15);
        afr[i] = *(const lds_bf16x8*)(sh + hr * ROWB + ((p ^ swz(hr)) * 16));
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int j = 0; j < CT; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[i], bfr[j], acc[i][j], 0, 0, 0);
        // the next refill of the ring, dealt out between row tiles: the
        // address unit drains it while the MFMAs run, instead of the wave
        // stalling on all of it at once
        const int slot_i = kk * MT + i;
#pragma unroll
        for (int q = slot_i * LD / (KK * MT); q < (slot_i + 1) * LD / (KK * MT); ++q)
          if (refill) issue_one(st + STAGES - 1, q);
      }
    }
  }

  // lane l holds columns v0 + 16*(wave*CT + j) + (l & 15) of rows
  // 16i + 4*(l >> 4) + r: the best of its columns, then of the 16 lanes of
  // its row group, then of the four waves
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float bv = -INFINITY;
      int bi = INT_MAX;
#pragma unroll
      for (int j = 0; j < CT; ++j) {
        const int v = v0 + 16 * (wave * CT + j) + (lane & 15);
        if (v < a.V && acc[i][j][r] > bv) {
          bv = acc[i][j][r];
          bi = v;
        }
      }
      argmax_row16(bv, bi);
      if ((lane & 15) == 0) {
        sv[wave][16 * i + 4 * (lane >> 4) + r] = bv;
        si[wave][16 * i + 4 * (lane >> 4) + r] = bi;
      }
    }
  }
  __syncthreads();
  if (tid < nrow) {
    float bv = sv[0][tid];
    int bi = si[0][tid];
    for (int w = 1; w < 4; ++w)
      if (argmax_better(sv[w][tid], si[w][tid], bv, bi)) {
        bv = sv[w][tid];
        bi = si[w][tid];
      }
    a.part[(size_t)(r0 + tid) * a.n_chunks + chunk] = make_float2(bv, __int_as_float(bi));
  }
}

template <int MT>
hipError_t launch_mt(const LmArgs& a, hipStream_t s) {
  const dim3 grid(a.n_chunks, (a.rows + MT * 16 - 1) / (MT * 16));
  hipLaunchKernelGGL(lmhead_argmax_kernel<MT>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lmhead_argmax(const LmArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (a.d % LK != 0 || a.d < LK) return hipErrorInvalidValue;
  // the fewest row tiles that hold the pass's rows (at most kLmRows per workgroup)
  switch ((std::min(a.rows, kLmRows) + 15) / 16) {
    case 1: return launch_mt<1>(a, s);
    case 2: return launch_mt<2>(a, s);
    case 3: return launch_mt<3>(a, s);
    case 4: return launch_mt<4>(a, s);
    case 5: return launch_mt<5>(a, s);
    case 6: return launch_mt<6>(a, s);
    case 7: return launch_mt<7>(a, s);
    case 8: return launch_mt<8>(a, s);
    default: return launch_mt<9>(a, s);
  }
}

}  // namespace tidar
