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
//
// W comes in one of two layouts.  Row-major [V][d]: a stage reads 128 B
// from each of 256 rows 2*d bytes apart, and HBM serves such scattered
// short reads at about four fifths of its rate for long ones.  Packed
// (lmhead_pack_kernel, once, when the weights are loaded): each stage's
// tile is one contiguous 32 KB block already in the LDS image above, so a
// stage's W loads are a straight copy.
#include <algorithm>
#include <climits>

#include "check.h"
#include "common.h"
#include "launch.h"
#include "lds_dma.h"

namespace tidar {

namespace {

constexpr int LK = 64;                    // hidden elements per stage
constexpr int ROWB = LK * 2;              // bytes per LDS row
constexpr int STAGES = 3;
constexpr int NCW = 4;                    // compute waves (one per SIMD)
constexpr int NLW = 4;                    // load waves (one per SIMD)
constexpr int W_BYTES = kLmChunk * ROWB;  // 32 KB of W per stage
constexpr int W_LD = W_BYTES / 1024 / NLW;  // direct loads per load wave per stage: W
constexpr int CT = kLmChunk / 16 / NCW;   // column tiles per compute wave
constexpr int KK = LK / 32;               // MFMA k-steps per stage

__device__ __forceinline__ int swz(int row) { return row & 7; }

// MT row tiles of 16 hidden rows per workgroup (the launch picks the fewest
// that hold its rows, so the loops below unroll completely and no stage
// loads hidden rows it does not use).
//
// Eight waves, two per SIMD, in two roles.  Waves 0-3 compute: they read
// operands from LDS and run the MFMAs, and never issue a vector memory
// instruction.  Waves 4-7 load: after each stage's barrier they request the
// stage two ahead and wait for the next one to land.  A wave that issues a
// direct load stalls while the address unit drains the ones before it; with
// the loads on their own waves, those stalls no longer hold up the MFMAs of
// the same SIMD.  Both roles pass the same barriers: one per stage and one
// before the cross-wave merge.
template <int MT, bool PACKED>
__global__ __launch_bounds__(64 * (NCW + NLW)) __attribute__((amdgpu_waves_per_eu(2, 2)))
void lmhead_argmax_kernel(LmArgs a) {
  constexpr int ROWS = MT * 16;
  constexpr int H_BYTES = ROWS * ROWB;      // hidden rows per stage
  constexpr int STAGE_BYTES = W_BYTES + H_BYTES;
  constexpr int H_BLK = H_BYTES / 1024;     // 1 KB blocks of hidden rows (2 per row tile)
  constexpr int H_LD = (H_BLK + NLW - 1) / NLW;  // ... per load wave (the last block may be loaded twice)
  constexpr int LD = W_LD + H_LD;           // direct loads per load wave per stage
  static_assert(STAGES == 3 && LD < 64, "vmcnt accounting below");
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE_BYTES];
  __shared__ float sv[NCW][ROWS];
  __shared__ int si[NCW][ROWS];
  lds_char* const ring = (lds_char*)smem;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool loader = wave >= NCW;
  const int chunk = blockIdx.x;
  const int v0 = chunk * kLmChunk;
  const int r0 = blockIdx.y * ROWS;
  const int nrow = min(ROWS, a.rows - r0);
  const int nst = a.d / LK;

  if (loader) {
    const int lw = wave - NCW;
    // element offset of hidden row m of this pass
    auto hrow = [&](int m) -> size_t {
      if (!a.draft) return (size_t)m * a.d;
      const int b = m / (a.k - 1), s = 1 + m % (a.k - 1);
      const int g_read = a.group[b];
      (void)TIDAR_CHECK(g_read >= 0 && g_read < a.k, TIDAR_CHECK_GROUP, g_read);
      const int g = min(max(g_read, 0), a.k - 1);  // written by the selection; clamped (the draft finalisation flags it)
      return (((size_t)b * a.k + g) * a.k + s) * a.d;
    };
    // this wave's direct loads: lane t of a 1 KB block lands at row 8*blk + t/8,
    // physical piece t%8, so it fetches logical piece (t%8) ^ swz(row); rows
    // past V or past the pass's rows repeat the last valid one.  A packed W
    // holds that image already: the chunk's tiles follow one another.
    const char* wsrc = (const char*)a.w + (PACKED ? (size_t)chunk * nst * W_BYTES : 0);
    unsigned off[LD];
    unsigned dst[LD];  // byte offset inside a stage's slot
#pragma unroll
    for (int ii = 0; ii < W_LD; ++ii) {
      const int row = (lw * W_LD + ii) * 8 + lane / 8;
      const int p = (lane & 7) ^ swz(row);
      off[ii] = PACKED ? (unsigned)((lw * W_LD + ii) * 1024 + lane * 16)
                       : (unsigned)((size_t)min(v0 + row, a.V - 1) * a.d * 2 + p * 16);
      dst[ii] = (lw * W_LD + ii) * 1024;
    }
#pragma unroll
    for (int ii = 0; ii < H_LD; ++ii) {
      const int blk = min(lw + NLW * ii, H_BLK - 1);
      const int row = blk * 8 + lane / 8;
      const int p = (lane & 7) ^ swz(row);
      off[W_LD + ii] = (unsigned)(hrow(r0 + min(row, nrow - 1)) * 2 + p * 16);
      dst[W_LD + ii] = W_BYTES + blk * 1024;
    }
    // this wave's share of stage st (W rows from a.w, nontemporal: read once
    // per pass; hidden rows from a.h, read again for every slice)
    auto issue = [&](int st) {
      lds_char* slot = ring + (st % STAGES) * STAGE_BYTES;
      const unsigned dk = (unsigned)st * ROWB;
      const unsigned dw = PACKED ? (unsigned)st * W_BYTES : dk;
#pragma unroll
      for (int q = 0; q < W_LD; ++q) dma_b128<true>(wsrc, off[q] + dw, slot + dst[q]);
#pragma unroll
      for (int q = W_LD; q < LD; ++q) dma_b128<false>((const char*)a.h, off[q] + dk, slot + dst[q]);
    };
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
      if (st < nst) issue(st);
    for (int st = 0; st < nst; ++st) {
      // stage st has landed once at most the stage issued after it is in flight
      if (st + 1 < nst) wait_vmcnt<LD>();
      else wait_vmcnt<0>();
      barrier();  // ... and the compute waves are done with the slot refilled below
      if (st + STAGES - 1 < nst) issue(st + STAGES - 1);
    }
    __syncthreads();  // the compute waves' merge below
    return;
  }

  floatx4 acc[MT][CT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < CT; ++j) acc[i][j] = (floatx4){0.f, 0.f, 0.f, 0.f};

  for (int st = 0; st < nst; ++st) {
    wait_lgkmcnt0();  // this wave's reads of the slot refilled after the barrier are done
    barrier();        // stage st has landed
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
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < CT; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // lane l holds columns v0 + 16*(wave*CT + j) + (l & 15) of rows
  // 16i + 4*(l >> 4) + r: the best of its columns, then of the 16 lanes of
  // its row group, then of the compute waves
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
    for (int w = 1; w < NCW; ++w)
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
  if (a.packed) hipLaunchKernelGGL((lmhead_argmax_kernel<MT, true>), grid, dim3(64 * (NCW + NLW)), 0, s, a);
  else hipLaunchKernelGGL((lmhead_argmax_kernel<MT, false>), grid, dim3(64 * (NCW + NLW)), 0, s, a);
  return hipGetLastError();
}

// One 32 KB tile of the packed layout per workgroup: tile (chunk c, stage
// st) holds, at byte 128*r + 16*j, the 8 elements of W row kLmChunk*c + r
// starting at column LK*st + 8*(j ^ swz(r)); rows past V are zero.  Each
// thread copies 16 B pieces; 8 consecutive threads cover one 128 B run of a
// W row, and the writes are contiguous.
__global__ __launch_bounds__(256) void lmhead_pack_kernel(const bf16* w, bf16* wp, int V, int d) {
  const int nst = d / LK;
  const int c = blockIdx.x / nst, st = blockIdx.x % nst;
  char* tile = (char*)wp + (size_t)blockIdx.x * W_BYTES;
#pragma unroll
  for (int i = 0; i < W_BYTES / 16 / 256; ++i) {
    const int id = threadIdx.x + 256 * i;
    const int r = id / 8, j = id % 8;
    const int v = c * kLmChunk + r;
    uint4 x = {0u, 0u, 0u, 0u};
    if (v < V) x = *(const uint4*)(w + (size_t)v * d + st * LK + 8 * (j ^ swz(r)));
    *(uint4*)(tile + id * 16) = x;
  }
}

}  // namespace

size_t lmhead_packed_bytes(int V, int d) { return (size_t)((V + kLmChunk - 1) / kLmChunk) * kLmChunk * d * 2; }

hipError_t launch_lmhead_pack(const void* w, void* wp, int V, int d, hipStream_t s) {
  if (V == 0) return hipSuccess;
  if (d % LK != 0 || d < LK) return hipErrorInvalidValue;
  const long blocks = (long)((V + kLmChunk - 1) / kLmChunk) * (d / LK);
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lmhead_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const bf16*)w, (bf16*)wp, V, d);
  return hipGetLastError();
}

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

#if TIDAR_CHECKED
TIDAR_CHECK_RECORD_ACCESSOR(check_record_lmhead)
#endif

}  // namespace tidar
