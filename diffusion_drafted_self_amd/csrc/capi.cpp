// C ABI of the TiDAR decode-step hot path: host-side validation, split
// planning, workspace carving and kernel launches.  No allocation, no
// synchronisation, no state kept between calls.
#include "tidar.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "launch.h"
#include "probe.h"

namespace {

constexpr int kMaxK = 16;
constexpr int kTileKeys = 64;           // keys per attention tile
constexpr int kValuePage = 64;          // positions per value-cache page
constexpr int kMaxChunkF32 = 1024;      // LDS score buffer of the f32 kernel
constexpr int kCUs = 256;               // compute units of the part

bool aligned(const void* p, uintptr_t a) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
long cdiv(long a, long b) { return (a + b - 1) / b; }

struct AttnPlan {
  int R, G, M, n16, nf, ns, n_rowblk, chunk, n_split, pp;
  size_t o_bytes, ml_bytes, total;
};

// Split plan of the step attention.
//
// bf16: the M = R*G query rows of one (b, kvh) form n16 tiles of 16 rows.  A
// workgroup (four waves, one per SIMD, one workgroup per CU) takes a
// contiguous share of T of them for one key chunk: each wave owns nf full
// tiles and the ns = T - 4*nf remaining tiles are shared by the four waves
// one 16-key block each, so every wave carries nf + ns/4 tiles; or all T
// tiles are full ones (ceil(T/4) per wave, the last waves partly idle).
// Built shapes: nf <= 3, ns <= 3, no shared tile next to three full ones or
// three shared next to two full ones (registers).  Candidates (row
// workgroups per (b, kvh), tile layout, key chunks) are scored in clocks:
// per 64-key tile a loop step costs body_clk(nf, ns) (fitted to whole-kernel
// timings on this part: ~700 of synchronisation and direct-load issue, ~400
// per full tile, ~300 per shared tile); per round of kCUs workgroups a fixed
// ~20k (prologue, tiles past the prefix, output);
// the HBM floor of the stream; and for several chunks the partial outputs
// (M*(D+2)*4 bytes per chunk, written and read back) plus the merge launch.
//
// f32: one wave per query row and chunk, chunks of at most kMaxChunkF32.
double body_clk(int nf, int ns) { return 700.0 + 400.0 * nf + 300.0 * ns; }

// The eight-wave kernel (two waves per SIMD, head dim 128): one tile per
// wave and at most one tile shared by the four SIMDs, so a workgroup takes
// at most nine tiles.  Per 64-key tile it costs the two waves' MFMA
// clusters of a SIMD (2 x 36 MFMAs of ~16 clocks) plus what of the softmax
// and load issue they do not hide.
double body_clk_pp(int ns) { return 1400.0 + 150.0 * ns; }

// Which step-attention kernel the planner may choose: both (default), or
// one of them when TIDAR_ATTN_KERNEL is "pp" (eight waves) or "pipe" (four
// waves), for measurements and tests of one against the other.  Read at
// every plan, so a process can switch between calls.
int kernel_choice() {
  const char* e = std::getenv("TIDAR_ATTN_KERNEL");
  if (!e) return 0;
  if (!std::strcmp(e, "pp")) return 1;
  if (!std::strcmp(e, "pipe")) return 2;
  return 0;
}

// The training mask's kernel (head dim 128): the eight-wave one unless
// TIDAR_ATTN_KERNEL asks for the four-wave one.  On the 8B training shape
// it took 1138 us against 1370 (sustained clock, one box).
bool train_kernel_is_pp() { return kernel_choice() != 2; }

bool shape_built(int nf, int ns) {
  if (nf < 0 || nf > 3 || ns < 0 || ns > 3 || nf + ns == 0) return false;
  return !(nf == 3 && ns > 0) && !(nf == 2 && ns == 3);
}

int plan_attention(int dtype, int B, int Hq, int Hkv, int D, int S_max, int max_len, int k,
                   int n_groups, int kv_chunk, AttnPlan* p) {
  if (dtype != TIDAR_BF16 && dtype != TIDAR_F32) return TIDAR_EUNSUPPORTED;
  if (D != 64 && D != 128) return TIDAR_EUNSUPPORTED;
  if (k > kMaxK) return TIDAR_EUNSUPPORTED;
  if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || k < 1) return TIDAR_EINVAL;
  if (n_groups != 0 && n_groups != k) return TIDAR_EINVAL;
  if (S_max < 1 || S_max % kValuePage != 0 || max_len < 0 || max_len > S_max) return TIDAR_EINVAL;
  if (kv_chunk < 0 || kv_chunk % kTileKeys != 0) return TIDAR_EINVAL;
  if (dtype == TIDAR_F32 && kv_chunk > kMaxChunkF32) return TIDAR_EINVAL;

  p->R = k + n_groups * k;
  p->G = Hq / Hkv;
  p->M = p->R * p->G;
  p->n16 = (int)cdiv(p->M, 16);
  const long keys = (long)max_len + p->R;
  const long pairs = std::max<long>(1, (long)B * Hkv);

  if (dtype == TIDAR_F32) {
    p->chunk = kv_chunk ? kv_chunk : (int)std::min<long>(kMaxChunkF32, (long)round_up(keys, kTileKeys));
    p->nf = 1;
    p->ns = 0;
    p->pp = 0;
    p->n_rowblk = 1;
  } else {
    const long n_key_tiles = cdiv(keys, kTileKeys);
    constexpr double kClkPerUs = 2000.0;  // shader clock under this kernel's load (GRBM_GUI_ACTIVE over the dispatch, 8B step)
    const double hbm_clk = (double)pairs * keys * D * 4 / 6.0e6 * kClkPerUs;  // K+V bytes at ~6 TB/s
    double best = 1e300;
    long best_chunk = 0;
    int best_wr = 1, best_nf = 1, best_ns = 0, best_pp = 0;
    long best_wgs = 0;
    const bool allow_pp = D == 128 && kernel_choice() != 2;
    const bool allow_pipe = !(allow_pp && kernel_choice() == 1);
    const long ns_max = kv_chunk ? 1 : std::min<long>(n_key_tiles, 64);
    for (long ns_try = 1; ns_try <= ns_max; ++ns_try) {
      const long chunk = kv_chunk ? kv_chunk : (long)round_up(cdiv(keys, ns_try), kTileKeys);
      const long ns = cdiv(keys, chunk);
      if (ns != ns_try && !kv_chunk) continue;  // the same chunk as a smaller count
      const long kt = cdiv(chunk, kTileKeys) + 1;  // + the step tile staged through registers
      for (int wr = 1; wr <= p->n16; ++wr) {
        const int t_max = (int)cdiv(p->n16, wr);
        // (full tiles per wave, shared tiles, eight-wave kernel)
        const int layouts[3][3] = {{t_max / 4, t_max % 4, 0}, {(int)cdiv(t_max, 4), 0, 0}, {1, t_max > 8, 1}};
        for (const auto& lay : layouts) {
          const int nf = lay[0], nsh = lay[1], pp = lay[2];
          if (pp ? (!allow_pp || t_max > 9) : (!allow_pipe || !shape_built(nf, nsh))) continue;
          const long wgs = pairs * wr * ns;
          const long rounds = cdiv(wgs, kCUs);
          const double body = pp ? body_clk_pp(nsh) : body_clk(nf, nsh);
          double cost = std::max((double)rounds * body * kt, hbm_clk) + 20000.0 * rounds;
          if (ns > 1) cost += (5.0 + (double)pairs * ns * p->M * (D * 4 + 8) * 2 / 5.0e6) * kClkPerUs;
          const bool better = cost < best * 0.999 || (cost <= best * 1.001 && wgs > best_wgs && wgs <= rounds * kCUs);
          if (better) {
            best = cost;
            best_chunk = chunk;
            best_wr = wr;
            best_nf = nf;
            best_ns = nsh;
            best_pp = pp;
            best_wgs = wgs;
          }
        }
      }
    }
    if (best_chunk == 0) return TIDAR_EUNSUPPORTED;  // no built layout fits
    p->chunk = (int)best_chunk;
    p->nf = best_nf;
    p->ns = best_ns;
    p->pp = best_pp;
    p->n_rowblk = best_wr;
  }
  p->n_split = (int)cdiv(keys, p->chunk);

  const long blocks = pairs * p->n_split * (dtype == TIDAR_F32 ? p->M : p->n_rowblk);
  if (blocks > 0x7fffffffL) return TIDAR_EUNSUPPORTED;
  if (dtype == TIDAR_BF16 && !p->pp && !shape_built(p->nf, p->ns)) return TIDAR_EUNSUPPORTED;
  if (p->pp && (p->ns > 1 || cdiv(p->n16, p->n_rowblk) > 8 + p->ns)) return TIDAR_EUNSUPPORTED;

  // workspace: [partial outputs][partial (max, sum)]; none is needed when
  // every sequence fits one chunk (bf16 path)
  const size_t parts = (dtype == TIDAR_F32 || p->n_split > 1) ? (size_t)B * Hkv * p->n_split * p->M : 0;
  p->o_bytes = round_up(parts * D * sizeof(float), 256);
  p->ml_bytes = round_up(parts * sizeof(float2), 256);
  p->total = p->o_bytes + p->ml_bytes;
  return TIDAR_OK;
}

struct VerifyPlan {
  int n_chunks;
  size_t ar_bytes, draft_bytes, group_bytes, total;
};

int plan_verify(int B, int k, int V, VerifyPlan* p) {
  if (k > kMaxK) return TIDAR_EUNSUPPORTED;
  if (B < 0 || k < 1 || V < 1) return TIDAR_EINVAL;
  if ((long)B * (k + 1) > 65535) return TIDAR_EUNSUPPORTED;  // grid y limit
  p->n_chunks = (int)cdiv(V, tidar::kArgmaxChunk);
  p->ar_bytes = round_up((size_t)B * (k + 1) * p->n_chunks * sizeof(float2), 256);
  p->draft_bytes = round_up((size_t)B * (k - 1) * p->n_chunks * sizeof(float2), 256);
  p->group_bytes = round_up((size_t)B * sizeof(int32_t), 256);
  p->total = p->ar_bytes + p->draft_bytes + p->group_bytes;
  return TIDAR_OK;
}

struct LmPlan {
  int n_chunks;
  size_t ar_bytes, draft_bytes, group_bytes, total;
};

int plan_lmhead(int B, int k, int V, int d, bool packed, LmPlan* p) {
  if (k > kMaxK) return TIDAR_EUNSUPPORTED;
  if (B < 0 || k < 1 || V < 1 || d < 64 || d % 64 != 0) return TIDAR_EINVAL;
  // direct loads address the hidden rows of either pass (B*(k+1) AR rows,
  // B*k*k draft rows), and a row-major W, with 32-bit byte offsets (a
  // packed W from the start of each chunk's tiles)
  if ((!packed && (double)V * d * 2 >= 4294967296.0) ||
      (double)B * std::max(k + 1, k * k) * d * 2 >= 4294967296.0)
    return TIDAR_EUNSUPPORTED;
  p->n_chunks = (int)cdiv(V, tidar::kLmChunk);
  if (cdiv((long)B * (k + 1), tidar::kLmRows) > 65535) return TIDAR_EUNSUPPORTED;
  p->ar_bytes = round_up((size_t)B * (k + 1) * p->n_chunks * sizeof(float2), 256);
  p->draft_bytes = round_up((size_t)B * (k - 1) * p->n_chunks * sizeof(float2), 256);
  p->group_bytes = round_up((size_t)B * sizeof(int32_t), 256);
  p->total = p->ar_bytes + p->draft_bytes + p->group_bytes;
  return TIDAR_OK;
}

struct SamplePlan {
  int n_chunks;
  size_t stats_bytes, resid_bytes, part_bytes, fb_bytes, total;
};

int plan_sample(int B, int k, int V, SamplePlan* p) {
  if (k > kMaxK) return TIDAR_EUNSUPPORTED;
  if (B < 0 || k < 1 || V < 1) return TIDAR_EINVAL;
  if ((long)2 * B * k > 65535) return TIDAR_EUNSUPPORTED;  // grid y limit
  p->n_chunks = (int)cdiv(V, tidar::kSampleChunk);
  p->stats_bytes = round_up((size_t)2 * B * k * p->n_chunks * sizeof(float2), 256);
  p->resid_bytes = round_up((size_t)B * 4 * sizeof(float), 256);
  p->part_bytes = round_up((size_t)B * k * p->n_chunks * sizeof(float2), 256);
  p->fb_bytes = round_up((size_t)B * p->n_chunks * sizeof(float2), 256);
  p->total = p->stats_bytes + p->resid_bytes + p->part_bytes + p->fb_bytes;
  return TIDAR_OK;
}

// Both cache forms: block_table == nullptr for per-sequence contiguous
// caches, else pools of n_pages pages with S_max = 64 * max_pages.
int step_attention_impl(int dtype, int B, int Hq, int Hkv, int D, int S_max, int max_len, int k, int n_groups,
                        float sm_scale, int kv_chunk, const void* q, const void* k_step, const void* v_step,
                        const void* k_cache, const void* v_cache, const int32_t* block_table, int max_pages,
                        int n_pages, const int32_t* lens, void* out, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream) {
  AttnPlan p;
  const int st = plan_attention(dtype, B, Hq, Hkv, D, S_max, max_len, k, n_groups, kv_chunk, &p);
  if (st != TIDAR_OK) return st;
  if (!(sm_scale > 0.f) || !(sm_scale < 3.0e38f)) return TIDAR_EINVAL;
  if (B == 0) return TIDAR_OK;
  if (!aligned(q, 16) || !aligned(k_step, 16) || !aligned(v_step, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(out, 16) || !aligned(lens, 4))
    return TIDAR_EINVAL;
  if (lse && !aligned(lse, 4)) return TIDAR_EINVAL;
  if (p.total > 0 && (!aligned(workspace, 256) || workspace_bytes < p.total)) return TIDAR_EWORKSPACE;

  tidar::AttnArgs a = {};
  a.q = q;
  a.k_step = k_step;
  a.v_step = v_step;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.lens = lens;
  a.out = out;
  a.lse = lse;
  char* ws = static_cast<char*>(workspace);
  a.o_part = reinterpret_cast<float*>(ws);
  a.ml_part = reinterpret_cast<float2*>(ws + p.o_bytes);
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = p.G;
  a.D = D;
  a.S_max = S_max;
  a.max_len = max_len;
  a.k = k;
  a.R = p.R;
  a.M = p.M;
  a.chunk = p.chunk;
  a.n_split = p.n_split;
  a.n16 = p.n16;
  a.nf = p.nf;
  a.ns = p.ns;
  a.n_rowblk = p.n_rowblk;
  a.pp = p.pp;
  a.scale_log2 = sm_scale * 1.44269504088896340736f;
  a.single_chunk_direct = dtype == TIDAR_BF16;
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.n_pages = n_pages;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = dtype == TIDAR_BF16 ? tidar::launch_attention_bf16(a, s) : tidar::launch_attention_f32(a, s);
  return e == hipSuccess ? TIDAR_OK : TIDAR_ELAUNCH;
}

int kv_commit_impl(int dtype, int B, int Hkv, int D, int S_max, int R, int k, void* k_cache, void* v_cache,
                   const int32_t* block_table, int max_pages, int n_pages, int32_t* lens, const void* k_step,
                   const void* v_step, const int32_t* accept_len, int32_t* err_flags, void* stream) {
  if (dtype != TIDAR_BF16 && dtype != TIDAR_F32) return TIDAR_EUNSUPPORTED;
  if (D != 64 && D != 128) return TIDAR_EUNSUPPORTED;
  // at most kMaxK (< 64) accepted rows: their positions span at most two
  // 64-position pages, the two the paged commit resolves
  if (k > kMaxK) return TIDAR_EUNSUPPORTED;
  if (B < 0 || Hkv < 1 || S_max < 1 || S_max % kValuePage != 0 || R < 1 || k < 1 || k > R) return TIDAR_EINVAL;
  if (B == 0) return TIDAR_OK;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(k_step, 16) || !aligned(v_step, 16) ||
      !aligned(lens, 4) || !aligned(accept_len, 4))
    return TIDAR_EINVAL;
  if (err_flags && !aligned(err_flags, 4)) return TIDAR_EINVAL;

  tidar::CommitArgs a;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.lens = lens;
  a.k_step = k_step;
  a.v_step = v_step;
  a.accept_len = accept_len;
  a.err_flags = err_flags;
  a.B = B;
  a.Hkv = Hkv;
  a.D = D;
  a.S_max = S_max;
  a.R = R;
  a.k = k;
  a.elem_bytes = dtype == TIDAR_BF16 ? 2 : 4;
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.n_pages = n_pages;
  const hipError_t e = tidar::launch_commit(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TIDAR_OK : TIDAR_ELAUNCH;
}

// State of the fused verify + commit: AR keys, then draft keys (one 8-byte
// key per 128-byte line), then one arrival counter per sequence (one per
// 128-byte line).
struct FusedPlan {
  size_t key_bytes, dkey_bytes, arrive_bytes, total;
};

int plan_fused(int B, int k, FusedPlan* p) {
  if (k > kMaxK) return TIDAR_EUNSUPPORTED;
  if (B < 0 || k < 1) return TIDAR_EINVAL;
  if ((long)B * (k + 1) > 65535) return TIDAR_EUNSUPPORTED;  // grid y limit
  p->key_bytes = round_up((size_t)B * (k + 1) * tidar::kFusedKeyBytes, 256);
  p->dkey_bytes = round_up((size_t)B * std::max(k - 1, 1) * tidar::kFusedKeyBytes, 256);
  p->arrive_bytes = round_up((size_t)B * tidar::kFusedKeyBytes, 256);
  p->total = p->key_bytes + p->dkey_bytes + p->arrive_bytes;
  return TIDAR_OK;
}

// The fused path's host checks (the verification's, then the commit's, then
// the state's); TIDAR_OK also for B == 0, where nothing is enqueued.
int verify_commit_checks(int dtype, int B, int Hkv, int D, int S_max, int R, int k, int V, const float* ar_logits,
                         const float* draft_logits, const int32_t* cand, const void* k_cache, const void* v_cache,
                         const int32_t* lens, const void* k_step, const void* v_step, const int32_t* accept_len,
                         const int32_t* next_cand, const int32_t* err_flags, const void* state, size_t state_bytes) {
  VerifyPlan vp;
  int st = plan_verify(B, k, V, &vp);
  if (st != TIDAR_OK) return st;
  FusedPlan fp;
  st = plan_fused(B, k, &fp);
  if (st != TIDAR_OK) return st;
  if (dtype != TIDAR_BF16 && dtype != TIDAR_F32) return TIDAR_EUNSUPPORTED;
  if (D != 64 && D != 128) return TIDAR_EUNSUPPORTED;
  if (Hkv < 1 || S_max < 1 || S_max % kValuePage != 0 || R < k) return TIDAR_EINVAL;
  if (B == 0) return TIDAR_OK;
  if (!aligned(ar_logits, 16) || !aligned(cand, 4) || !aligned(accept_len, 4) || !aligned(next_cand, 4))
    return TIDAR_EINVAL;
  if (k > 1 && !aligned(draft_logits, 16)) return TIDAR_EINVAL;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(k_step, 16) || !aligned(v_step, 16) ||
      !aligned(lens, 4))
    return TIDAR_EINVAL;
  if (err_flags && !aligned(err_flags, 4)) return TIDAR_EINVAL;
  if (!aligned(state, 8) || state_bytes < fp.total) return TIDAR_EWORKSPACE;
  return TIDAR_OK;
}

int verify_commit_impl(int dtype, int B, int Hkv, int D, int S_max, int R, int k, int V, const float* ar_logits,
                       const float* draft_logits, const int32_t* cand, void* k_cache, void* v_cache,
                       const int32_t* block_table, int max_pages, int n_pages, int32_t* lens, const void* k_step,
                       const void* v_step, int32_t* accept_len, int32_t* next_cand, int32_t* err_flags,
                       void* state, size_t state_bytes, void* stream) {
  const int st = verify_commit_checks(dtype, B, Hkv, D, S_max, R, k, V, ar_logits, draft_logits, cand, k_cache,
                                      v_cache, lens, k_step, v_step, accept_len, next_cand, err_flags, state,
                                      state_bytes);
  if (st != TIDAR_OK || B == 0) return st;
  FusedPlan fp;
  plan_fused(B, k, &fp);

  tidar::FusedVerifyArgs a = {};
  a.ar_logits = ar_logits;
  a.draft_logits = draft_logits;
  a.cand = cand;
  a.accept_len = accept_len;
  a.next_cand = next_cand;
  char* ws = static_cast<char*>(state);
  a.key = reinterpret_cast<unsigned long long*>(ws);
  a.dkey = reinterpret_cast<unsigned long long*>(ws + fp.key_bytes);
  a.arrive = reinterpret_cast<unsigned*>(ws + fp.key_bytes + fp.dkey_bytes);
  a.B = B;
  a.k = k;
  a.V = V;
  a.n_draft_rows = std::max(k - 1, 1);
  a.commit = 1;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.lens = lens;
  a.k_step = k_step;
  a.v_step = v_step;
  a.err_flags = err_flags;
  a.Hkv = Hkv;
  a.D = D;
  a.S_max = S_max;
  a.R = R;
  a.elem_bytes = dtype == TIDAR_BF16 ? 2 : 4;
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.n_pages = n_pages;
  const hipError_t e = tidar::launch_fused_verify(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TIDAR_OK : TIDAR_ELAUNCH;
}

}  // namespace

extern "C" {

const char* tidar_strerror(int status) {
  switch (status) {
    case TIDAR_OK: return "ok";
    case TIDAR_EINVAL: return "invalid argument (shape, pointer, alignment or value)";
    case TIDAR_EUNSUPPORTED: return "unsupported configuration (dtype, head dim, k or size)";
    case TIDAR_EWORKSPACE: return "workspace missing or too small";
    case TIDAR_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int tidar_abi_version(void) { return 1; }

int tidar_step_attention_workspace(int dtype, int B, int Hq, int Hkv, int D, int S_max, int max_len,
                                   int k, int n_groups, int kv_chunk, size_t* bytes) {
  if (!bytes) return TIDAR_EINVAL;
  AttnPlan p;
  const int st = plan_attention(dtype, B, Hq, Hkv, D, S_max, max_len, k, n_groups, kv_chunk, &p);
  if (st != TIDAR_OK) return st;
  *bytes = p.total;
  return TIDAR_OK;
}

int tidar_step_attention_plan(int dtype, int B, int Hq, int Hkv, int D, int S_max, int max_len,
                              int k, int n_groups, int kv_chunk, int* plan) {
  if (!plan) return TIDAR_EINVAL;
  AttnPlan p;
  const int st = plan_attention(dtype, B, Hq, Hkv, D, S_max, max_len, k, n_groups, kv_chunk, &p);
  if (st != TIDAR_OK) return st;
  plan[0] = dtype == TIDAR_F32 ? 2 : p.pp;
  plan[1] = p.nf;
  plan[2] = p.ns;
  plan[3] = p.n_rowblk;
  plan[4] = p.chunk;
  plan[5] = p.n_split;
  return TIDAR_OK;
}

int tidar_step_attention(int dtype, int B, int Hq, int Hkv, int D, int S_max, int max_len,
                         int k, int n_groups, float sm_scale, int kv_chunk,
                         const void* q, const void* k_step, const void* v_step,
                         const void* k_cache, const void* v_cache, const int32_t* lens,
                         void* out, float* lse, void* workspace, size_t workspace_bytes,
                         void* stream) {
  return step_attention_impl(dtype, B, Hq, Hkv, D, S_max, max_len, k, n_groups, sm_scale, kv_chunk, q, k_step,
                             v_step, k_cache, v_cache, nullptr, 0, 0, lens, out, lse, workspace, workspace_bytes,
                             stream);
}

int tidar_step_attention_paged(int dtype, int B, int Hq, int Hkv, int D, int max_pages, int n_pages, int max_len,
                               int k, int n_groups, float sm_scale, int kv_chunk,
                               const void* q, const void* k_step, const void* v_step,
                               const void* k_pool, const void* v_pool, const int32_t* block_table,
                               const int32_t* lens, void* out, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (dtype != TIDAR_BF16) return TIDAR_EUNSUPPORTED;  // paged pools: the bf16 kernels only
  if (max_pages < 1 || max_pages > (1 << 24) || n_pages < 1) return TIDAR_EINVAL;
  if (B > 0 && !aligned(block_table, 4)) return TIDAR_EINVAL;
  return step_attention_impl(dtype, B, Hq, Hkv, D, max_pages * kValuePage, max_len, k, n_groups, sm_scale,
                             kv_chunk, q, k_step, v_step, k_pool, v_pool, block_table, max_pages, n_pages, lens,
                             out, lse, workspace, workspace_bytes, stream);
}

int tidar_train_attention(int dtype, int B, int Hq, int Hkv, int D, int N, int block, float sm_scale,
                          const void* q, const void* k, const void* v, void* out, float* lse, void* stream) {
  if (dtype != TIDAR_BF16) return TIDAR_EUNSUPPORTED;
  if (D != 64 && D != 128) return TIDAR_EUNSUPPORTED;
  if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return TIDAR_EINVAL;
  if (N < kTileKeys || N % kTileKeys != 0 || N > (1 << 24) || block < 1 || block > N) return TIDAR_EINVAL;
  if (!(sm_scale > 0.f) || !(sm_scale < 3.0e38f)) return TIDAR_EINVAL;
  const int G = Hq / Hkv;
  const long T = 2L * N, M = T * G;
  if (M > 0x7fffffffL) return TIDAR_EUNSUPPORTED;
  if (B == 0) return TIDAR_OK;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return TIDAR_EINVAL;
  if (lse && !aligned(lse, 4)) return TIDAR_EINVAL;

  // row tiles of 16 per half.  Four-wave kernel: 4*nf tiles per workgroup,
  // as many as keep the chip fed at least four workgroups per CU.
  // Eight-wave kernel (head dim 128): eight tiles per workgroup, one per
  // wave (a ninth, shared tile measured 8% slower here: the workgroups are
  // many and the shared tile's extra MFMAs and LDS round trips are not).
  const long n16h = M / 32;
  const long pairs = (long)B * Hkv;
  const bool pp = D == 128 && train_kernel_is_pp();
  int nf = 1;
  if (!pp)
    for (int c = 3; c >= 2; --c)
      if (pairs * 2 * cdiv(n16h, 4 * c) >= 4L * kCUs) {
        nf = c;
        break;
      }
  const long H = pp ? cdiv(n16h, 8) : cdiv(n16h, 4 * nf);
  if (pairs * 2 * H > 0x7fffffffL) return TIDAR_EUNSUPPORTED;

  tidar::AttnArgs a = {};
  a.q = q;
  a.k_cache = k;
  a.v_cache = v;
  a.lens = nullptr;
  a.out = out;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = G;
  a.D = D;
  a.S_max = (int)T;
  a.max_len = (int)T;
  a.k = 1;
  a.R = (int)T;
  a.M = (int)M;
  a.chunk = (int)T;
  a.n_split = 1;
  a.n16 = (int)(M / 16);
  a.nf = nf;
  a.ns = 0;
  a.pp = pp ? 1 : 0;
  a.n_rowblk = (int)(2 * H);
  a.scale_log2 = sm_scale * 1.44269504088896340736f;
  a.single_chunk_direct = 1;
  a.block_table = nullptr;
  a.train_N = N;
  a.train_bs = block;
  const hipError_t e = pp ? tidar::launch_train_attention_pp_bf16(a, static_cast<hipStream_t>(stream))
                          : tidar::launch_train_attention_bf16(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TIDAR_OK : TIDAR_ELAUNCH;
}

int tidar_verify_workspace(int B, int k, int V, size_t* bytes) {
  if (!bytes) return TIDAR_EINVAL;
  VerifyPlan p;
  const int st = plan_verify(B, k, V, &p);
  if (st != TIDAR_OK) return st;
  *bytes = p.total;
  return TIDAR_OK;
}

int tidar_verify_greedy(int B, int k, int V, const float* ar_logits, const float* draft_logits,
                        const int32_t* cand, int32_t* accept_len, int32_t* next_cand,
                        void* workspace, size_t workspace_bytes, void* stream) {
  VerifyPlan p;
  const int st = plan_verify(B, k, V, &p);
  if (st != TIDAR_OK) return st;
  if (B == 0) return TIDAR_OK;
  if (!aligned(ar_logits, 16) || !aligned(cand, 4) || !aligned(accept_len, 4) || !aligned(next_cand, 4))
    return TIDAR_EINVAL;
  if (k > 1 && !aligned(draft_logits, 16)) return TIDAR_EINVAL;
  if (!aligned(workspace, 256) || workspace_bytes < p.total) return TIDAR_EWORKSPACE;

  tidar::VerifyArgs a;
  a.ar_logits = ar_logits;
  a.draft_logits = draft_logits;
  a.cand = cand;
  a.accept_len = accept_len;
  a.next_cand = next_cand;
  char* ws = static_cast<char*>(workspace);
  a.part_ar = reinterpret_cast<float2*>(ws);
  a.part_draft = reinterpret_cast<float2*>(ws + p.ar_bytes);
  a.group = reinterpret_cast<int32_t*>(ws + p.ar_bytes + p.draft_bytes);
  a.B = B;
  a.k = k;
  a.V = V;
  a.chunk_elems = tidar::kArgmaxChunk;
  a.n_chunks = p.n_chunks;
  const hipError_t e = tidar::launch_verify(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TIDAR_OK : TIDAR_ELAUNCH;
}

int tidar_lmhead_verify_workspace(int B, int k, int V, int d_model, size_t* bytes) {
  if (!bytes) return TIDAR_EINVAL;
  LmPlan p;
  const int st = plan_lmhead(B, k, V, d_model, true, &p);
  if (st != TIDAR_OK) return st;
  *bytes = p.total;
  return TIDAR_OK;
}

int tidar_lmhead_packed_bytes(int V, int d_model, size_t* bytes) {
  if (!bytes || V < 1 || d_model < 64 || d_model % 64 != 0) return TIDAR_EINVAL;
  *bytes = tidar::lmhead_packed_bytes(V, d_model);
  return TIDAR_OK;
}

int tidar_lmhead_pack(int V, int d_model, const void* w, void* w_packed, void* stream) {
  if (V < 1 || d_model < 64 || d_model % 64 != 0) return TIDAR_EINVAL;
  if (!aligned(w, 16) || !aligned(w_packed, 16)) return TIDAR_EINVAL;
  const hipError_t e = tidar::launch_lmhead_pack(w, w_packed, V, d_model, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TIDAR_OK : TIDAR_ELAUNCH;
}

// the two layouts of W share everything but the kernel's W addressing
static int lmhead_verify(bool packed, int B, int k, int V, int d_model, const void* h_ar, const void* h_draft,
                         const void* w, const int32_t* cand, int32_t* accept_len, int32_t* next_cand,
                         void* workspace, size_t workspace_bytes, void* stream) {
  LmPlan p;
  const int st = plan_lmhead(B, k, V, d_model, packed, &p);
  if (st != TIDAR_OK) return st;
  if (B == 0) return TIDAR_OK;
  if (!aligned(h_ar, 16) || !aligned(w, 16) || !aligned(cand, 4) || !aligned(accept_len, 4) ||
      !aligned(next_cand, 4))
    return TIDAR_EINVAL;
  if (k > 1 && !aligned(h_draft, 16)) return TIDAR_EINVAL;
  if (!aligned(workspace, 256) || workspace_bytes < p.total) return TIDAR_EWORKSPACE;

  char* ws = static_cast<char*>(workspace);
  tidar::VerifyArgs va = {};
  va.cand = cand;
  va.accept_len = accept_len;
  va.next_cand = next_cand;
  va.part_ar = reinterpret_cast<float2*>(ws);
  va.part_draft = reinterpret_cast<float2*>(ws + p.ar_bytes);
  va.group = reinterpret_cast<int32_t*>(ws + p.ar_bytes + p.draft_bytes);
  va.B = B;
  va.k = k;
  va.V = V;
  va.chunk_elems = tidar::kLmChunk;
  va.n_chunks = p.n_chunks;

  tidar::LmArgs la = {};
  la.w = w;
  la.B = B;
  la.k = k;
  la.V = V;
  la.d = d_model;
  la.n_chunks = p.n_chunks;
  la.packed = packed ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // AR rows -> chunk results -> accept length, bonus token, group
  la.h = h_ar;
  la.part = va.part_ar;
  la.rows = B * (k + 1);
  la.draft = 0;
  hipError_t e = tidar::launch_lmhead_argmax(la, s);
  if (e == hipSuccess) e = tidar::launch_verify_select(va, s);
  // the selected group's draft rows -> next drafts
  if (e == hipSuccess && k > 1) {
    la.h = h_draft;
    la.group = va.group;
    la.part = va.part_draft;
    la.rows = B * (k - 1);
    la.draft = 1;
    e = tidar::launch_lmhead_argmax(la, s);
    if (e == hipSuccess) e = tidar::launch_draft_finalize(va, s);
  }
  return e == hipSuccess ? TIDAR_OK : TIDAR_ELAUNCH;
}

int tidar_lmhead_verify_greedy(int B, int k, int V, int d_model, const void* h_ar, const void* h_draft,
                               const void* w, const int32_t* cand, int32_t* accept_len, int32_t* next_cand,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return lmhead_verify(false, B, k, V, d_model, h_ar, h_draft, w, cand, accept_len, next_cand, workspace,
                       workspace_bytes, stream);
}

int tidar_lmhead_verify_greedy_packed(int B, int k, int V, int d_model, const void* h_ar, const void* h_draft,
                                      const void* w_packed, const int32_t* cand, int32_t* accept_len,
                                      int32_t* next_cand, void* workspace, size_t workspace_bytes, void* stream) {
  return lmhead_verify(true, B, k, V, d_model, h_ar, h_draft, w_packed, cand, accept_len, next_cand, workspace,
                       workspace_bytes, stream);
}

int tidar_verify_sample_workspace(int B, int k, int V, size_t* bytes) {
  if (!bytes) return TIDAR_EINVAL;
  SamplePlan p;
  const int st = plan_sample(B, k, V, &p);
  if (st != TIDAR_OK) return st;
  *bytes = p.total;
  return TIDAR_OK;
}

int tidar_verify_sample(int B, int k, int V, float temperature, const float* ar_logits, const float* q_logits,
                        const float* draft_logits, const int32_t* cand, uint64_t seed, uint32_t step,
                        int32_t* accept_len, int32_t* next_cand, void* workspace, size_t workspace_bytes,
                        void* stream) {
  SamplePlan p;
  const int st = plan_sample(B, k, V, &p);
  if (st != TIDAR_OK) return st;
  if (!(temperature > 0.f) || !std::isfinite(temperature)) return TIDAR_EINVAL;
  if (B == 0) return TIDAR_OK;
  if (!aligned(ar_logits, 16) || !aligned(q_logits, 16) || !aligned(cand, 4) || !aligned(accept_len, 4) ||
      !aligned(next_cand, 4))
    return TIDAR_EINVAL;
  if (k > 1 && !aligned(draft_logits, 16)) return TIDAR_EINVAL;
  if (!aligned(workspace, 256) || workspace_bytes < p.total) return TIDAR_EWORKSPACE;

  tidar::SampleArgs a;
  a.ar_logits = ar_logits;
  a.q_logits = q_logits;
  a.draft_logits = draft_logits;
  a.cand = cand;
  a.accept_len = accept_len;
  a.next_cand = next_cand;
  char* ws = static_cast<char*>(workspace);
  a.stats = reinterpret_cast<float2*>(ws);
  a.resid = reinterpret_cast<float4*>(ws + p.stats_bytes);
  a.part = reinterpret_cast<float2*>(ws + p.stats_bytes + p.resid_bytes);
  a.part_fb = reinterpret_cast<float2*>(ws + p.stats_bytes + p.resid_bytes + p.part_bytes);
  a.B = B;
  a.k = k;
  a.V = V;
  a.n_chunks = p.n_chunks;
  a.zscale = (float)(1.4426950408889634074 / (double)temperature);
  a.key0 = (uint32_t)seed;
  a.key1 = (uint32_t)(seed >> 32);
  a.step = step;
  const hipError_t e = tidar::launch_verify_sample(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TIDAR_OK : TIDAR_ELAUNCH;
}

int tidar_kv_commit(int dtype, int B, int Hkv, int D, int S_max, int R, int k,
                    void* k_cache, void* v_cache, int32_t* lens,
                    const void* k_step, const void* v_step, const int32_t* accept_len,
                    int32_t* err_flags, void* stream) {
  return kv_commit_impl(dtype, B, Hkv, D, S_max, R, k, k_cache, v_cache, nullptr, 0, 0, lens, k_step, v_step,
                        accept_len, err_flags, stream);
}

int tidar_kv_commit_paged(int dtype, int B, int Hkv, int D, int max_pages, int n_pages, int R, int k,
                          void* k_pool, void* v_pool, const int32_t* block_table, int32_t* lens,
                          const void* k_step, const void* v_step, const int32_t* accept_len,
                          int32_t* err_flags, void* stream) {
  if (max_pages < 1 || max_pages > (1 << 24) || n_pages < 1) return TIDAR_EINVAL;
  if (B > 0 && !aligned(block_table, 4)) return TIDAR_EINVAL;
  return kv_commit_impl(dtype, B, Hkv, D, max_pages * kValuePage, R, k, k_pool, v_pool, block_table, max_pages,
                        n_pages, lens, k_step, v_step, accept_len, err_flags, stream);
}

int tidar_verify_commit_state_bytes(int B, int k, size_t* bytes) {
  if (!bytes) return TIDAR_EINVAL;
  FusedPlan p;
  const int st = plan_fused(B, k, &p);
  if (st != TIDAR_OK) return st;
  *bytes = p.total;
  return TIDAR_OK;
}

int tidar_verify_commit_greedy(int dtype, int B, int Hkv, int D, int S_max, int R, int k, int V,
                               const float* ar_logits, const float* draft_logits, const int32_t* cand,
                               void* k_cache, void* v_cache, int32_t* lens, const void* k_step, const void* v_step,
                               int32_t* accept_len, int32_t* next_cand, int32_t* err_flags, void* state,
                               size_t state_bytes, void* stream) {
  return verify_commit_impl(dtype, B, Hkv, D, S_max, R, k, V, ar_logits, draft_logits, cand, k_cache, v_cache,
                            nullptr, 0, 0, lens, k_step, v_step, accept_len, next_cand, err_flags, state,
                            state_bytes, stream);
}

int tidar_verify_commit_greedy_noalloc(int dtype, int B, int Hkv, int D, int S_max, int R, int k, int V,
                                       const float* ar_logits, const float* draft_logits, const int32_t* cand,
                                       void* k_cache, void* v_cache, int32_t* lens, const void* k_step,
                                       const void* v_step, int32_t* accept_len, int32_t* next_cand,
                                       int32_t* err_flags, void* stream) {
  FusedPlan fp;
  const int pst = plan_fused(B, k, &fp);
  if (pst != TIDAR_OK) return pst;
  if (fp.total > tidar::kNoAllocScratchBytes) return TIDAR_EWORKSPACE;
  // every check first (a stand-in for the array's address: aligned, large
  // enough), so a refused call enqueues nothing, not even the first clear
  const int cst = verify_commit_checks(dtype, B, Hkv, D, S_max, R, k, V, ar_logits, draft_logits, cand, k_cache,
                                       v_cache, lens, k_step, v_step, accept_len, next_cand, err_flags,
                                       reinterpret_cast<const void*>(uintptr_t(256)), tidar::kNoAllocScratchBytes);
  if (cst != TIDAR_OK || B == 0) return cst;
  void* state = nullptr;
  if (tidar::noalloc_scratch(static_cast<hipStream_t>(stream), &state) != hipSuccess) return TIDAR_ELAUNCH;
  const int st = verify_commit_impl(dtype, B, Hkv, D, S_max, R, k, V, ar_logits, draft_logits, cand, k_cache,
                                    v_cache, nullptr, 0, 0, lens, k_step, v_step, accept_len, next_cand, err_flags,
                                    state, tidar::kNoAllocScratchBytes, stream);
  if (st == TIDAR_ELAUNCH) tidar::noalloc_scratch_dirty();  // part of the state may be left set
  return st;
}

int tidar_verify_commit_greedy_paged(int dtype, int B, int Hkv, int D, int max_pages, int n_pages, int R, int k,
                                     int V, const float* ar_logits, const float* draft_logits,
                                     const int32_t* cand, void* k_pool, void* v_pool, const int32_t* block_table,
                                     int32_t* lens, const void* k_step, const void* v_step, int32_t* accept_len,
                                     int32_t* next_cand, int32_t* err_flags, void* state, size_t state_bytes,
                                     void* stream) {
  if (max_pages < 1 || max_pages > (1 << 24) || n_pages < 1) return TIDAR_EINVAL;
  if (B > 0 && !aligned(block_table, 4)) return TIDAR_EINVAL;
  return verify_commit_impl(dtype, B, Hkv, D, max_pages * kValuePage, R, k, V, ar_logits, draft_logits, cand, k_pool,
                            v_pool, block_table, max_pages, n_pages, lens, k_step, v_step, accept_len, next_cand,
                            err_flags, state, state_bytes, stream);
}

int tidar_launch_shapes(int path, int B, int k, int V, int Hkv, int D, int dtype, int* shapes) {
  if (!shapes) return TIDAR_EINVAL;
  tidar::LaunchShape sh[tidar::kMaxLaunches];
  int n = 0, st;
  if (path == 0 || path == 2) {  // the entry points' own checks first
    VerifyPlan vp;
    if ((st = plan_verify(B, k, V, &vp)) != TIDAR_OK) return st;
  }
  if (path == 1 || path == 2) {
    if (dtype != TIDAR_BF16 && dtype != TIDAR_F32) return TIDAR_EUNSUPPORTED;
    if (D != 64 && D != 128) return TIDAR_EUNSUPPORTED;
    if (k > kMaxK) return TIDAR_EUNSUPPORTED;
    if (B < 0 || Hkv < 1 || k < 1) return TIDAR_EINVAL;
  }
  if (path == 0) n = tidar::verify_launch_shapes(B, k, V, sh);
  else if (path == 1) n = tidar::commit_launch_shapes(B, Hkv, D, k, dtype == TIDAR_BF16 ? 2 : 4, sh);
  else if (path == 2) {
    FusedPlan fp;
    if ((st = plan_fused(B, k, &fp)) != TIDAR_OK) return st;
    n = tidar::fused_launch_shapes(B, k, V, sh);
  } else {
    return TIDAR_EINVAL;
  }
  for (int i = 0; i < n; ++i) {
    shapes[3 * i] = sh[i].gx;
    shapes[3 * i + 1] = sh[i].gy;
    shapes[3 * i + 2] = sh[i].block;
  }
  return n;
}

static_assert(TIDAR_READ_PROBE_BLOCKS == tidar::kReadProbeBlocks, "read probe sink size");

int tidar_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!aligned(src, 16) || !aligned(sink, 4) || bytes % 16 != 0) return TIDAR_EINVAL;
  if (bytes == 0) return TIDAR_OK;
  const hipError_t e = tidar::launch_read_probe(src, bytes, sink, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TIDAR_OK : TIDAR_ELAUNCH;
}

static_assert(TIDAR_MFMA_PROBE_BLOCKS == tidar::kMfmaProbeBlocks, "MFMA probe record count");

int tidar_mfma_probe(int waves_per_simd, int lds_reads, int iters, uint64_t* cycles, void* stream) {
  if (waves_per_simd != 1 && waves_per_simd != 2) return TIDAR_EINVAL;
  if (lds_reads != 0 && lds_reads != 1) return TIDAR_EINVAL;
  if (iters < 1 || iters > (1 << 20)) return TIDAR_EINVAL;
  if (!aligned(cycles, 8)) return TIDAR_EINVAL;
  const hipError_t e = tidar::launch_mfma_probe(waves_per_simd, lds_reads, iters,
                                                reinterpret_cast<unsigned long long*>(cycles),
                                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TIDAR_OK : TIDAR_ELAUNCH;
}

int tidar_check_enabled(void) { return TIDAR_CHECKED ? 1 : 0; }

int tidar_check_read(uint32_t* rec, int clear) {
  if (!rec) return TIDAR_EINVAL;
  rec[0] = rec[1] = rec[2] = rec[3] = 0;
#if TIDAR_CHECKED
  if (hipDeviceSynchronize() != hipSuccess) return TIDAR_ELAUNCH;
  hipError_t (*const files[])(unsigned*, bool) = {
      tidar::check_record_attention,    tidar::check_record_attention_pp, tidar::check_record_verify,
      tidar::check_record_verify_fused, tidar::check_record_verify_sample, tidar::check_record_lmhead,
      tidar::check_record_commit};
  for (auto read : files) {
    unsigned r[4];
    if (read(r, clear != 0) != hipSuccess) return TIDAR_ELAUNCH;
    if (rec[0] == 0 && r[0] != 0) std::memcpy(rec, r, sizeof(r));
  }
#else
  (void)clear;
#endif
  return TIDAR_OK;
}

}  // extern "C"
