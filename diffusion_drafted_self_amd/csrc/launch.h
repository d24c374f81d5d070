// Host-side launch interface between the C ABI (capi.cpp) and the kernels.
#pragma once

#ifndef TIDAR_CHECKED
#define TIDAR_CHECKED 0  // 1 in the checked build (device-side bounds tests)
#endif

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tidar {

// Split plan and arguments of the step-attention kernels.  Query rows of
// one (sequence, KV head) are numbered m = r*G + j (step row r, head j of
// the group), M = R*G of them.  Keys are the [prefix ; step] sequence of
// L+R positions, cut into chunks of `chunk` positions.
struct AttnArgs {
  const void* q;
  const void* k_step;
  const void* v_step;
  const void* k_cache;
  const void* v_cache;
  const int32_t* lens;
  void* out;
  float* lse;
  float* o_part;   // [B][Hkv][n_split][M][D]  unnormalised partial outputs
  float2* ml_part; // [B][Hkv][n_split][M]     (running max in log2 units, sum)
  int B, Hq, Hkv, G, D, S_max, max_len, k, R, M;
  int chunk, n_split;
  int n16, nf, ns, n_rowblk;  // bf16 path: 16-row tiles of (b, kvh); per workgroup, full tiles per
                              // wave and tiles shared by key block; workgroups per (b, kvh)
  int pp;                     // bf16 path: the eight-wave (two per SIMD) kernel, one tile per wave
                              // plus ns (0 or 1) shared tile; nf is then 1
  float scale_log2;     // sm_scale * log2(e)
  int single_chunk_direct;  // the split kernel writes sequences that fit one chunk (bf16 path)
  // paged caches (bf16 path): k_cache / v_cache are pools of n_pages pages,
  // block_table [B][max_pages] maps tile t of sequence b to its page;
  // nullptr for per-sequence contiguous caches
  const int32_t* block_table;
  int max_pages, n_pages;
  // training sequence (train kernel only): N clean positions, masked blocks of train_bs
  int train_N, train_bs;
};

hipError_t launch_attention_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_attention_pp_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_train_attention_pp_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_attention_f32(const AttnArgs& a, hipStream_t s);
hipError_t launch_train_attention_bf16(const AttnArgs& a, hipStream_t s);

struct VerifyArgs {
  const float* ar_logits;
  const float* draft_logits;
  const int32_t* cand;
  int32_t* accept_len;
  int32_t* next_cand;
  float2* part_ar;     // [B*(k+1)][n_chunks] (value, index bits)
  float2* part_draft;  // [B*(k-1)][n_chunks]
  int32_t* group;      // [B]
  int B, k, V, chunk_elems, n_chunks;
};

hipError_t launch_verify(const VerifyArgs& a, hipStream_t s);

// One kernel launch: grid (gx, gy) of workgroups of `block` threads.  The
// launchers take their shapes from the functions below, which the C ABI
// also exports (tidar_launch_shapes), so every shape can be checked on the
// host: a block over 1024 threads does not launch at all.
struct LaunchShape {
  int gx, gy, block;
};
constexpr int kMaxLaunches = 4;
// greedy verification: AR argmax, selection, draft argmax, finalisation
// (the last two only for k > 1); returns the number of launches
int verify_launch_shapes(int B, int k, int V, LaunchShape* out);
int commit_launch_shapes(int B, int Hkv, int D, int k, int elem_bytes, LaunchShape* out);

// Greedy verification fused with the KV commit (or without it): three
// launches over per-row 64-bit argmax keys that every call leaves zeroed.
constexpr int kFusedKeyBytes = 128;  // one 64-bit argmax key per 128-byte line

struct FusedVerifyArgs {
  const float* ar_logits;     // [B][k+1][V]
  const float* draft_logits;  // [B][k][k][V]
  const int32_t* cand;        // [B][k]
  int32_t* accept_len;        // [B]
  int32_t* next_cand;         // [B][k]
  unsigned long long* key;    // [B*(k+1)] keys, kFusedKeyBytes apart         state
  unsigned long long* dkey;   // [B*n_draft_rows] keys, kFusedKeyBytes apart  state
  unsigned* arrive;           // [B] arrival counters, kFusedKeyBytes apart    state
  int B, k, V, n_draft_rows;  // n_draft_rows = max(k-1, 1)
  // commit (commit != 0)
  int commit;
  void* k_cache;
  void* v_cache;
  int32_t* lens;
  const void* k_step;
  const void* v_step;
  int32_t* err_flags;
  int Hkv, D, S_max, R, elem_bytes;
  const int32_t* block_table;  // paged pools (S_max = 64 * max_pages), or nullptr
  int max_pages, n_pages;
};

// Launch shapes of the fused path (the host checks them before launching).
struct FusedVerifyGeometry {
  int ar_grid_x, ar_grid_y;        // (chunks, AR rows)
  int draft_grid_x, draft_grid_y;  // (spans of kDraftSpan, sequences x draft rows)
  int draft_rows, block;
};
FusedVerifyGeometry fused_verify_geometry(int B, int k, int V);
int fused_launch_shapes(int B, int k, int V, LaunchShape* out);
hipError_t launch_fused_verify(const FusedVerifyArgs& a, hipStream_t s);

// The allocation-free entry point's state: a file-scope device array per
// GPU.  noalloc_scratch gives its device address on the current device
// (clearing it on stream s first when it is not known to be zero);
// noalloc_scratch_dirty marks it for clearing after a failed launch.
constexpr size_t kNoAllocScratchBytes = size_t(2) << 20;
hipError_t noalloc_scratch(hipStream_t s, void** out);
void noalloc_scratch_dirty();
hipError_t launch_verify_select(const VerifyArgs& a, hipStream_t s);
hipError_t launch_draft_finalize(const VerifyArgs& a, hipStream_t s);

// LM head fused with the argmax: chunk results of logits = h . W^T
constexpr int kLmChunk = 256;   // vocabulary entries per workgroup
constexpr int kLmRows = 144;    // hidden-state rows per workgroup (9 tiles of 16)

struct LmArgs {
  const void* h;        // pass 0: [B][k+1][d] AR rows; pass 1: [B][k][k][d] draft rows
  const void* w;        // [V][d] bf16, or packed (lmhead_pack_kernel)
  const int32_t* group; // [B] selected group (pass 1)
  float2* part;         // [rows][n_chunks] (value, index bits)
  int B, k, V, d, n_chunks, rows, draft, packed;
};

hipError_t launch_lmhead_argmax(const LmArgs& a, hipStream_t s);
size_t lmhead_packed_bytes(int V, int d);
hipError_t launch_lmhead_pack(const void* w, void* wp, int V, int d, hipStream_t s);
hipError_t launch_read_probe(const void* src, size_t bytes, unsigned* sink, hipStream_t s);

constexpr int kReadProbeBlocks = 16384;  // workgroups of the streaming-read probe
constexpr int kArgmaxChunk = 4096;  // logits per workgroup of the greedy argmax
constexpr int kDraftSpan = 2 * kArgmaxChunk;  // logits per workgroup of the fused path's draft pass
constexpr int kSampleChunk = 4096;  // vocabulary entries per workgroup of the sampling kernels

struct SampleArgs {
  const float* ar_logits;     // [B][k+1][V]
  const float* q_logits;      // [B][k][V]
  const float* draft_logits;  // [B][k][k][V]
  const int32_t* cand;        // [B][k]
  int32_t* accept_len;
  int32_t* next_cand;
  float2* stats;    // [2*B*k][n_chunks] (max, sum of exp2) of z = logit * zscale
  float4* resid;    // [B] (Mp, Zp, Mq, Zq) of the first rejected candidate's rows
  float2* part;     // [B*k][n_chunks] (score, index bits) of the draws
  float2* part_fb;  // [B][n_chunks]   the draw from p for the residual row
  int B, k, V, n_chunks;
  float zscale;     // log2(e) / T
  unsigned key0, key1, step;
};

hipError_t launch_verify_sample(const SampleArgs& a, hipStream_t s);

struct CommitArgs {
  void* k_cache;
  void* v_cache;
  int32_t* lens;
  const void* k_step;
  const void* v_step;
  const int32_t* accept_len;
  int32_t* err_flags;
  int B, Hkv, D, S_max, R, k, elem_bytes;
  const int32_t* block_table;  // paged pools (S_max = 64 * max_pages), or nullptr
  int max_pages, n_pages;
};

hipError_t launch_commit(const CommitArgs& a, hipStream_t s);

#if TIDAR_CHECKED
// Checked build: each kernel source file's record of its first failed
// bounds test on the current device, {code, workgroup, thread, value};
// `clear` zeroes it after the copy.  The device must be synchronised.
hipError_t check_record_attention(unsigned* rec, bool clear);
hipError_t check_record_attention_pp(unsigned* rec, bool clear);
hipError_t check_record_verify(unsigned* rec, bool clear);
hipError_t check_record_verify_fused(unsigned* rec, bool clear);
hipError_t check_record_verify_sample(unsigned* rec, bool clear);
hipError_t check_record_lmhead(unsigned* rec, bool clear);
hipError_t check_record_commit(unsigned* rec, bool clear);
#endif

}  // namespace tidar
