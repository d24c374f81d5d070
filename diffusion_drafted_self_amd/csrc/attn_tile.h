// Tile geometry, LDS swizzles, direct-load plans and the staging of masked
// tiles, shared by the step-attention kernels (gfx950).  A 64-key tile of
// one (sequence, KV head) is a 16 KB block of keys and a 16 KB transposed
// value page; both reach LDS by direct global->LDS loads in 1 KB pieces.
#pragma once

#include "check.h"
#include "common.h"
#include "lds_dma.h"

namespace tidar {

namespace {

constexpr int TK = 64;    // keys per tile
constexpr int RING = 4;   // LDS slots for K tiles, and as many for V^T tiles
constexpr int kMaxRankedB = 256;  // batches up to this size run longest sequences first

// The value cache holds pages of VPAGE positions, each stored transposed
// ([S_max/VPAGE][D][VPAGE] per (b, kvh)), so one 64-key V^T tile is one
// contiguous 16 KB page, like the K tile.
constexpr int VPAGE = 64;
static_assert(TK == VPAGE, "a key tile is one value page");

__device__ __forceinline__ size_t vpos(int d, int c, int D) {  // element (d, position c) of a value cache
  return (size_t)(c / VPAGE) * D * VPAGE + (size_t)d * VPAGE + (c % VPAGE);
}

// Where tile t (settled positions 64t .. 64t+63) of one (sequence, KV head)
// lives: its 64 key rows start at ktile(t), its transposed value page at
// vtile(t).  Contiguous caches: tile t of the pair's own region.  Paged
// caches: page table[t] of the pools ([n_pages][Hkv][64][D] keys,
// [n_pages][Hkv][D][64] values), this KV head's slot at the same offset in
// every page.  Only tiles holding settled positions may be asked for.
//
// A table entry is read with a scalar load that waits inside its own asm
// block: a plain load would be a vector load (the compiler cannot prove the
// table unclobbered past the direct-to-LDS asm), and waiting for it would
// drain every tile load in flight at each ring step.
__device__ __forceinline__ int32_t scalar_load_i32(const int32_t* p) {
  const unsigned long long a = (unsigned long long)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  const unsigned long long sa = ((unsigned long long)hi << 32) | lo;
  int32_t v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(sa));
  return v;
}

template <int D, bool PAGED>
struct KvMap {
  const bf16* k;
  const bf16* v;
  const int32_t* tbl;  // this sequence's block-table row (paged)
  size_t stride;       // elements from one page to the next
  int n_tiles;         // checked build: tiles of the cache (S_max/64) or table slots (max_pages)
  int n_pages;         // checked build: pages in the pools
  __device__ __forceinline__ size_t page(int t) const {
    if (!TIDAR_CHECK(t >= 0 && t < n_tiles, TIDAR_CHECK_KEY_TILE, t)) t = 0;
    if constexpr (PAGED) {
      int32_t pg = scalar_load_i32(tbl + t);
      if (!TIDAR_CHECK((unsigned)pg < (unsigned)n_pages, TIDAR_CHECK_PAGE, pg)) pg = 0;
      return (size_t)pg;
    } else {
      return (size_t)t;
    }
  }
  __device__ __forceinline__ const bf16* ktile(int t) const { return k + page(t) * stride; }
  __device__ __forceinline__ const bf16* vtile(int t) const { return v + page(t) * stride; }
};

// LDS tile geometry.  K tile: TK rows of D bf16, row-major; V^T tile: D rows
// of TK bf16.  Both are filled 1 KB at a time by direct global->LDS loads
// (each lane moves 16 B; lane t lands at byte 16t of the 1 KB block), so a
// 16 B piece's position inside its row is permuted by an XOR swizzle chosen
// by the source address each lane reads: logical piece p of K row `row` sits
// at physical piece p ^ kswz(row), logical piece q of V^T row d at
// q ^ vswz(d).  With these the MFMA operand reads are free of bank
// conflicts.
template <int D, int NW = 4>
struct Tile {
  static constexpr int KROW = D * 2;        // bytes per K row
  static constexpr int KPPR = KROW / 16;    // 16 B pieces per K row
  static constexpr int K_BYTES = TK * KROW;
  static constexpr int VROW = TK * 2;       // bytes per V^T row (8 pieces)
  static constexpr int V_BYTES = D * VROW;
  static constexpr int NKW = K_BYTES / 1024 / NW;  // direct loads per wave per K tile (NW waves)
  static constexpr int NVW = V_BYTES / 1024 / NW;  // ... per V^T tile
  static constexpr int NDB = D / 16;  // 16-row head-dim blocks of O^T
  static constexpr int NDC = D / 32;  // 32-deep head-dim steps of S^T
};

// Score block kb4 (16 keys) of a tile: MFMA row i (= lane & 15 of the A
// operand) is tile key 32*(kb4>>1) + 8*(i>>2) + 4*(kb4&1) + (i&3).  With this
// order the 4 scores a lane holds from blocks 2c and 2c+1 are keys
// 32c + 8*(lane>>4) + 0..7: exactly the B-operand layout of P^T for the
// 32-key step c of O^T += V^T.P^T, so P needs no cross-lane movement.
__device__ __forceinline__ int krow_of(int kb4, int i) {
  return 32 * (kb4 >> 1) + 8 * (i >> 2) + 4 * (kb4 & 1) + (i & 3);
}

// Within one operand read the rows vary in bits 0, 1, 3 and 4; the swizzle
// maps those bits (with the row parity where a row is 128 B) to distinct
// 16 B slots.
template <int D>
__device__ __forceinline__ int kswz(int row) {
  if constexpr (Tile<D>::KPPR == 16) return (row & 3) | ((row >> 1) & 12);
  else return ((row >> 1) & 1) | ((row >> 2) & 2) | (((row ^ (row >> 4)) & 1) << 2);
}
// V^T rows: the piece index XOR the row's low three bits.  With the operand
// read of O^T += V^T.P^T (16 consecutive rows, four consecutive pieces per
// row across the four lane groups) this is free of bank conflicts on this
// part, measured with the LDS bank-conflict counter; the variant that also
// folded in bit 3 of the row conflicted on 40% of the active cycles.
__device__ __forceinline__ int vswz(int d) { return d & 7; }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));


// Per-lane byte offsets of this wave's direct loads inside a tile: wave w
// moves the 1 KB blocks w*NKW .. w*NKW+NKW-1 of the K tile and
// w*NVW .. w*NVW+NVW-1 of the V^T tile.  Tile-invariant.
template <int D, int NW = 4>
struct DmaPlan {
  unsigned k[Tile<D, NW>::NKW];
  unsigned v[Tile<D, NW>::NVW];
};

template <int D, int NW = 4>
__device__ __forceinline__ void dma_plan(DmaPlan<D, NW>& pl, int wave, int lane) {
  using T = Tile<D, NW>;
#pragma unroll
  for (int ii = 0; ii < T::NKW; ++ii) {
    const int row = (wave * T::NKW + ii) * (1024 / T::KROW) + lane / T::KPPR;
    const int p = (lane % T::KPPR) ^ kswz<D>(row);
    pl.k[ii] = row * T::KROW + p * 16;
  }
#pragma unroll
  for (int ii = 0; ii < T::NVW; ++ii) {
    const int d = (wave * T::NVW + ii) * 8 + (lane >> 3);
    const int q = (lane & 7) ^ vswz(d);
    pl.v[ii] = d * T::VROW + q * 16;
  }
}

// This wave's share of the direct loads of a K tile / V^T tile (a tile of
// 64 settled keys): 64 contiguous cache rows, one contiguous value page.
template <int D, int NW = 4>
__device__ __forceinline__ void issue_k(lds_char* sK, const bf16* ktile, const DmaPlan<D, NW>& pl, int wave) {
  using T = Tile<D, NW>;
  const char* kt = (const char*)ktile;
#pragma unroll
  for (int ii = 0; ii < T::NKW; ++ii) dma_b128(kt, pl.k[ii], sK + (wave * T::NKW + ii) * 1024);
}
template <int D, int NW = 4>
__device__ __forceinline__ void issue_v(lds_char* sV, const bf16* vtile, const DmaPlan<D, NW>& pl, int wave) {
  using T = Tile<D, NW>;
  const char* vt = (const char*)vtile;
#pragma unroll
  for (int ii = 0; ii < T::NVW; ++ii) dma_b128(vt, pl.v[ii], sV + (wave * T::NVW + ii) * 1024);
}

// Stage a tile that reaches past the settled prefix (the step block, or
// keys past the end) into the same swizzled layout.  Settled keys come from
// the tile's cache rows `kt` / value page `vt` (null when the tile holds no
// settled position) in 16 B pieces, one at a time; step rows are read 16 B at a time and
// their values scattered into V^T columns; everything else is zero.
//
// Kernels whose registers are not near the limit use the two-part form
// below instead (stage_issue / stage_commit), so a tile's loads can be in
// flight while the tile before it computes.
template <int D, int NT = 256>
__device__ __forceinline__ void stage_tail_tile_lean(lds_char* sK, lds_char* sV, const bf16* kt, const bf16* vt,
                                                     const bf16* ks_base, const bf16* vs_base, size_t step_stride,
                                                     int t0, int L, int Ltot, int tid) {
  using T = Tile<D>;
  for (int id = tid; id < TK * T::KPPR; id += NT) {
    const int row = id / T::KPPR, p = id % T::KPPR;
    const int c = t0 + row;
    bf16x8 val = {};
    if (c < L) val = *(const bf16x8*)(kt + (size_t)row * D + p * 8);
    else if (c < Ltot) val = *(const bf16x8*)(ks_base + (size_t)(c - L) * step_stride + p * 8);
    *(lds_bf16x8*)(sK + row * T::KROW + ((p ^ kswz<D>(row)) * 16)) = val;
  }
  for (int id = tid; id < D * 8; id += NT) {
    const int d = id >> 3, q = id & 7;
    const int c0 = t0 + q * 8;
    bf16x8 val = {};
    if (c0 + 8 <= L) {
      val = *(const bf16x8*)(vt + (size_t)d * VPAGE + q * 8);
    } else if (c0 < L) {
#pragma unroll
      for (int e = 0; e < 8; ++e) val[e] = c0 + e < L ? vt[(size_t)d * VPAGE + q * 8 + e] : (bf16)0.f;
    }
    *(lds_bf16x8*)(sV + d * T::VROW + ((q ^ vswz(d)) * 16)) = val;
  }
  wait_all();
  barrier();
  const int j0 = max(t0, L), j1 = min(t0 + TK, Ltot);
  for (int id = tid; id < TK * (D / 8); id += NT) {
    const int cl = id % TK, dc = id / TK;
    const int c = t0 + cl;
    if (c < j0 || c >= j1) continue;
    const bf16x8 val = *(const bf16x8*)(vs_base + (size_t)(c - L) * step_stride + dc * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = dc * 8 + e;
      *(__attribute__((address_space(3))) bf16*)(sV + d * T::VROW + ((((cl >> 3) ^ vswz(d)) * 16)) + (cl & 7) * 2) = val[e];
    }
  }
}

template <int D, int NT_ = 256>
struct StagedRows {  // a masked tile's K pieces and step-row values, in flight (NT_ threads)
  static constexpr int NT = NT_;
  static constexpr int NK = TK * Tile<D>::KPPR / NT;  // K pieces per thread
  static constexpr int NVS = D * 8 / NT;              // V^T pieces (8 positions) per thread
  static constexpr int NVR = TK * (D / 8) / NT;       // step-row value pieces per thread
  static_assert(NK * NT == TK * Tile<D>::KPPR && NVS * NT == D * 8 && NVR * NT == TK * (D / 8), "staging split");
  bf16x8 kp[NK], vr[NVR];
};

// The loads of a masked tile's K pieces and step rows' values, all issued at
// once (their latencies overlap); every masked tile has step rows or keys
// past the end.
template <int D, int NT = 256>
__device__ __forceinline__ void stage_issue(StagedRows<D, NT>& st, const bf16* kt, const bf16* ks_base,
                                            const bf16* vs_base, size_t step_stride, int t0, int L, int Ltot,
                                            int tid) {
  using S = StagedRows<D, NT>;
  using T = Tile<D>;
  const int j0 = max(t0, L), j1 = min(t0 + TK, Ltot);
#pragma unroll
  for (int i = 0; i < S::NK; ++i) {
    const int id = tid + i * S::NT, row = id / T::KPPR, p = id % T::KPPR;
    const int c = t0 + row;
    st.kp[i] = (bf16x8){};
    if (c < L) st.kp[i] = *(const bf16x8*)(kt + (size_t)row * D + p * 8);
    else if (c < Ltot) st.kp[i] = *(const bf16x8*)(ks_base + (size_t)(c - L) * step_stride + p * 8);
  }
#pragma unroll
  for (int i = 0; i < S::NVR; ++i) {  // step rows: 8 head-dim elements of one key
    const int id = tid + i * S::NT, cl = id % TK, dc = id / TK;
    const int c = t0 + cl;
    st.vr[i] = (bf16x8){};
    if (c >= j0 && c < j1) st.vr[i] = *(const bf16x8*)(vs_base + (size_t)(c - L) * step_stride + dc * 8);
  }
}

// The rest of staging a masked tile whose loads stage_issue made: the K
// pieces into their rows, the settled part of V^T (a second batch of loads,
// present only when the tile holds settled positions), then the step rows'
// values scattered into V^T columns.  wait_loads waits for this tile's
// loads and LDS stores (the caller knows what else is in flight).
template <int D, int NT, class Wait>
__device__ __forceinline__ void stage_commit(const StagedRows<D, NT>& st, lds_char* sK, lds_char* sV, const bf16* vt,
                                             int t0, int L, int Ltot, int tid, Wait&& wait_loads) {
  using S = StagedRows<D, NT>;
  using T = Tile<D>;
  const int j0 = max(t0, L), j1 = min(t0 + TK, Ltot);
#pragma unroll
  for (int i = 0; i < S::NK; ++i) {
    const int id = tid + i * S::NT, row = id / T::KPPR, p = id % T::KPPR;
    *(lds_bf16x8*)(sK + row * T::KROW + ((p ^ kswz<D>(row)) * 16)) = st.kp[i];
  }
  bf16x8 vp[S::NVS];
#pragma unroll
  for (int i = 0; i < S::NVS; ++i) {  // settled part of V^T, zero elsewhere
    const int id = tid + i * S::NT, d = id >> 3, q = id & 7;
    const int c0 = t0 + q * 8;
    vp[i] = (bf16x8){};
    if (c0 + 8 <= L) {
      vp[i] = *(const bf16x8*)(vt + (size_t)d * VPAGE + q * 8);
    } else if (c0 < L) {
#pragma unroll
      for (int e = 0; e < 8; ++e) vp[i][e] = c0 + e < L ? vt[(size_t)d * VPAGE + q * 8 + e] : (bf16)0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < S::NVS; ++i) {
    const int id = tid + i * S::NT, d = id >> 3, q = id & 7;
    *(lds_bf16x8*)(sV + d * T::VROW + ((q ^ vswz(d)) * 16)) = vp[i];
  }
  wait_loads();  // this tile's loads and stores are done
  barrier();     // the scatter below overwrites 2-byte parts of those pieces
  // step rows scattered into 8 V^T rows.  Consecutive lanes take
  // consecutive keys, so each 2-byte store of a wave fills one V^T row
  // across 64 columns (lanes on the same column would all hit one bank).
#pragma unroll
  for (int i = 0; i < S::NVR; ++i) {
    const int id = tid + i * S::NT, cl = id % TK, dc = id / TK;
    const int c = t0 + cl;
    if (c < j0 || c >= j1) continue;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = dc * 8 + e;
      *(__attribute__((address_space(3))) bf16*)(sV + d * T::VROW + ((((cl >> 3) ^ vswz(d)) * 16)) + (cl & 7) * 2) = st.vr[i][e];
    }
  }
}

// Operands of score block w and of the 16 keys of block w in P.V, read from
// LDS for the shared tiles (the full tiles read theirs inside the steps).
template <int D>
__device__ __forceinline__ bf16x8 kfrag(const lds_char* sK, int kb4, int c, int lane) {
  using T = Tile<D>;
  const int i16 = lane & 15, hi = lane >> 4;
  const int ksw = kswz<D>(krow_of(0, i16));  // the same for every block of the tile
  return *(const lds_bf16x8*)(sK + krow_of(kb4, i16) * T::KROW + (((4 * c + hi) ^ ksw) * 16));
}
template <int D>
__device__ __forceinline__ bf16x8 vfrag(const lds_char* sV, int db, int kc, int lane) {
  using T = Tile<D>;
  const int i16 = lane & 15, hi = lane >> 4;
  return *(const lds_bf16x8*)(sV + (16 * db + i16) * T::VROW + (((4 * kc + hi) ^ vswz(i16)) * 16));
}
// keys 32*(w>>1) + 8*(lane>>4) + 4*(w&1) + 0..3 of V^T row 16*db + (lane&15):
// with these the A operand of v_mfma_f32_16x16x16_bf16 holds, in its k order,
// the keys whose p this lane holds from score block w
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
template <int D>
__device__ __forceinline__ bf16x4 vfrag16(const lds_char* sV, int db, int w, int lane) {
  using T = Tile<D>;
  const int i16 = lane & 15, hi = lane >> 4;
  return *(const lds_bf16x4*)(sV + (16 * db + i16) * T::VROW + (((4 * (w >> 1) + hi) ^ vswz(i16)) * 16) + 8 * (w & 1));
}

// Above this tile sum of p (exp2 against a held reference) the fp32 sums
// and bf16 P could lose relative precision; the exact path then runs.
constexpr float kSumLimit = 18446744073709551616.0f;  // 2^64

template <int N>
constexpr int at_least_1() { return N > 0 ? N : 1; }

}  // namespace

}  // namespace tidar
