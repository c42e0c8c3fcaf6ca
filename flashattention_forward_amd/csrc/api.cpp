// C-ABI front end of libfa.so: argument validation, launch planning (tiles,
// key-split counts, workspace carving) and kernel launch. Every check runs on
// the host before anything is enqueued.
//
// Planning follows two lessons of "CUDA: fix FA occupancy, optimize tile kernel"
// (llama.cpp, opening paragraph): launch enough workgroups to occupy every
// compute unit (the occupancy bug there launched too few), and size tiles to the
// chip (here 160 KiB of LDS and 256 CUs of MI355X).
#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "fa.h"
#include "fa_kernels.h"

using namespace fa;

namespace {

int env_int(const char* name, int dflt);

// Compute units the planner sizes grids for: those of the current device, read
// once per device with hipDeviceGetAttribute and cached (a racing first query
// stores the same value). FA_NUM_CUS overrides it; with no usable device (a
// host-only process asking for workspace sizes) the 256 of MI355X are assumed.
// Workspace sizes therefore hold for the device that is current when they are
// asked for, which must be the one the matching call runs on.
constexpr int kDefaultCus = 256;
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_cus[kMaxDevices];

int planner_cus() {
  const int forced = env_int("FA_NUM_CUS", 0);
  if (forced > 0) return forced;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();  // do not leave the failed query for a later launch check
    return kDefaultCus;
  }
  int cus = g_device_cus[dev].load(std::memory_order_relaxed);
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0) {
      (void)hipGetLastError();
      cus = kDefaultCus;
    }
    g_device_cus[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

int env_int(const char* name, int dflt) {
  const char* e = std::getenv(name);
  if (!e || !*e) return dflt;
  return std::atoi(e);
}

// FA_LOG=1 prints, per call, the plan it launches (one line on stderr). The
// variable is read once per process.
bool log_plans() {
  static const bool on = env_int("FA_LOG", 0) != 0;
  return on;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

constexpr int64_t kMaxGrid = 0x7fffffff;

// ---------------------------------------------------------------------------
// prefill planning
// ---------------------------------------------------------------------------
struct PrefillPlan {
  int waves = 4;
  int pack = 1;  // query heads per workgroup
  int n_qtiles = 0;
  int n_splits = 1;
  size_t ws_bytes = 0;
};

// Key splits for `base` workgroups of `waves` waves: two waves on every SIMD
// (two 4-wave or one 8-wave workgroup per CU) is the target; a split keeps at
// least 8 tiles (512 keys).
int prefill_splits(int64_t base, int max_tiles, int waves) {
  const int64_t target = (8 / waves) * (int64_t)planner_cus();
  int S = 1;
  while (base * S < target && S < 16 && max_tiles / (2 * S) >= 8) S *= 2;
  return S;
}

// out_bytes: bytes per element of the output type, which the split partials
// share (2 for bf16/fp16, 4 for fp32).
PrefillPlan plan_prefill(int B, int Hq, int Hkv, int Sq, int Skv, int D, bool allow_split,
                         int out_bytes) {
  PrefillPlan pl;
  const int max_tiles = ceil_div(Skv, PF_BN);
  // Head size 128 uses 8-wave workgroups when they (with splits) still give
  // every CU a workgroup; otherwise, and for head size 64, 4 waves.
  int waves = 4;
  if (D == 128) {
    const int64_t base8 = (int64_t)B * Hq * ceil_div(Sq, 256);
    const int S8 = allow_split ? prefill_splits(base8, max_tiles, 8) : 1;
    if (base8 * S8 >= planner_cus()) waves = 8;
  }
  const int forced_w = env_int("FA_PREFILL_WAVES", 0);
  if (D == 128 && (forced_w == 4 || forced_w == 8)) waves = forced_w;
  pl.waves = waves;
  // Head packs (the grouped-query packing of the same llama.cpp paragraph): a
  // workgroup takes PK query heads of one K/V head over 32 waves / PK rows, so
  // each K/V and mask tile it copies serves PK heads, and the causal diagonal
  // costs fewer masked tiles per workgroup. PK is the largest power of two
  // that divides the group size and the waves (workload 3 as 32 microbatches:
  // 2547 us unpacked, 2385 / 2412 us with packs of 2 / 4; with a distance-bias
  // mask 3259 / 2869 / 2801 us). FA_PREFILL_PACK forces a pack (1 = one head).
  const int G = Hq / Hkv;
  int pack = 1;
  for (int pk = waves; pk > 1; pk /= 2)
    if (G % pk == 0) {
      pack = pk;
      break;
    }
  const int forced_pk = env_int("FA_PREFILL_PACK", 0);
  if (forced_pk >= 1 && forced_pk <= waves && waves % forced_pk == 0 && G % forced_pk == 0)
    pack = forced_pk;
  if (waves == 8 && env_int("FA_PREFILL_PINGPONG", 0) != 0) pack = 1;  // one-head tiling only
  pl.pack = pack;
  pl.n_qtiles = ceil_div(Sq, 32 * waves / pack);
  // Splits are planned from the one-head tiling, so the workspace a shape needs
  // does not depend on the pack (nor on whether the call has a mask).
  const int64_t base = (int64_t)B * Hq * ceil_div(Sq, 32 * waves);
  int S = 1;
  if (allow_split && base > 0) {
    const int forced = env_int("FA_PREFILL_SPLITS", 0);
    S = forced > 0 ? std::min(forced, 64) : prefill_splits(base, max_tiles, waves);
    S = std::max(1, std::min(S, std::max(1, max_tiles)));
  }
  pl.n_splits = S;
  // Per split: the partial rows in the output type and an fp32 lse per row.
  if (S > 1)
    pl.ws_bytes = (size_t)S * B * Sq * Hq * ((size_t)D * out_bytes + sizeof(float));
  return pl;
}

// ---------------------------------------------------------------------------
// decode planning
// ---------------------------------------------------------------------------
struct DecodePlan {
  int n_splits = 1;
  int chunk = DEC_TILE;
  int n_hblk = 1;
  int heads_per_wg = 64;  // MLA only
  size_t ws_bytes = 0;
};

DecodePlan plan_decode(int B, int Hq, int Hkv, int D_v, int max_seq_len, fa_kv_layout layout,
                       int num_splits, bool allow_split, int Sq = 1) {
  DecodePlan pl;
  const int tiles = std::max(1, ceil_div(max_seq_len, DEC_TILE));
  int64_t units;
  int64_t target;
  int min_splits = 1;
  if (layout == FA_KV_MLA_SHARED) {
    // 32 heads per workgroup when there are at most 32 (no idle head group);
    // otherwise 64. (Two 32-head workgroups over one sequence's 64 heads read
    // its rows once from HBM, the second copy coming from L2, but each CU then
    // needs twice the bytes in flight for the same HBM rate: slower than
    // splitting the keys.)
    // Without a workspace a sequence longer than one 64-head split holds takes
    // 32-head workgroups, which need no split.
    int nh = env_int("FA_MLA_HEADS", 0);
    if (nh != 32 && nh != 64)
      nh = Hq * Sq <= 32 || (!allow_split && max_seq_len > MLA_MAX_CHUNK) ? 32 : 64;
    pl.heads_per_wg = nh;
    pl.n_hblk = ceil_div(Hq * Sq, nh);  // rows: new tokens x heads
    units = (int64_t)B * pl.n_hblk;   // one workgroup per unit
    target = planner_cus();           // one 8-wave workgroup per CU
    if (nh == 64) min_splits = ceil_div(std::max(1, max_seq_len), MLA_MAX_CHUNK);
  } else {
    pl.n_hblk = ceil_div((Hq / Hkv) * Sq, 16);  // rows: new tokens x heads of a group
    units = (int64_t)B * Hkv * pl.n_hblk;  // one wave per unit
    // 16 waves per CU, twice the 8 that are resident at a time (the kernel's
    // 168 VGPRs leave room for two waves per SIMD, one 8-wave workgroup per
    // CU): in a ragged batch the splits past a shorter sequence's end (about
    // half of them for lengths uniform up to max_seq_len) exit at once without
    // holding a slot, and a wave keeps one tile in flight, so shorter chains of
    // tiles pay. Measured on 4 sequences of 1.8K-23K tokens, 32/8 heads: 92
    // splits of 256 tokens take 50 us against 59 us for 62 of 384 (a grid
    // sized to the resident waves); with 8-wave workgroups 64 / 80 / 92 / 105
    // / 128 / 184 splits took 51.3 / 48.2 / 44.6 / 44.6 / 45.2 / 51.5 us.
    target = 16 * (int64_t)planner_cus();
  }
  int S = 1;
  int chunk_tiles = tiles;
  if (allow_split && units > 0) {
    int req = num_splits > 0 ? num_splits : env_int("FA_DECODE_SPLITS", 0);
    if (req > 0) {
      S = std::max(1, std::min(req, tiles));
      chunk_tiles = ceil_div(tiles, S);
    } else {
      // Split while the grid is short of the target, keeping >= 8 tiles
      // (256 tokens) per split; the chunk is rounded down, so the count may
      // come out one higher.
      const int64_t want = (target + units - 1) / units;
      S = (int)std::min<int64_t>(want, std::max(1, tiles / 8));
      chunk_tiles = std::max(1, tiles / S);
    }
  }
  if (S < min_splits) chunk_tiles = ceil_div(tiles, min_splits);
  pl.chunk = chunk_tiles * DEC_TILE;
  pl.n_splits = ceil_div(std::max(1, max_seq_len), pl.chunk);
  if (pl.n_splits < 1) pl.n_splits = 1;
  // Partial outputs in the 16-bit input type, fp32 lse.
  if (pl.n_splits > 1)
    pl.ws_bytes = (size_t)pl.n_splits * B * Sq * Hq * ((size_t)D_v * 2 + sizeof(float));
  return pl;
}

int check_prefill(const void* q, const void* k, const void* v, void* o, const float* lse, int B,
                  int Hq, int Hkv, int Sq, int Skv, int D, fa_dtype in_dtype,
                  fa_dtype out_dtype) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 0 || Skv < 0 || Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  if (in_dtype != FA_BF16 && in_dtype != FA_FP16) return FA_ERR_UNSUPPORTED;
  if (out_dtype != FA_BF16 && out_dtype != FA_FP16 && out_dtype != FA_FP32)
    return FA_ERR_UNSUPPORTED;
  if (Sq > 0 && (!q || !o)) return FA_ERR_NULL;
  if (Skv > 0 && (!k || !v)) return FA_ERR_NULL;
  if ((q && !aligned16(q)) || (k && !aligned16(k)) || (v && !aligned16(v)) ||
      (o && !aligned16(o)) || (lse && !aligned4(lse)))
    return FA_ERR_ALIGN;
  if ((int64_t)B * Hq * ceil_div(Sq, PF_BM_MIN) > kMaxGrid) return FA_ERR_SHAPE;
  return FA_OK;
}

}  // namespace

extern "C" {

const char* fa_version(void) { return "0.1.0"; }

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "a size is out of range or inconsistent";
    case FA_ERR_UNSUPPORTED: return "unsupported head size or dtype";
    case FA_ERR_ALIGN: return "a base pointer is not 16-byte aligned";
    case FA_ERR_WORKSPACE: return "workspace smaller than the plan needs";
    case FA_ERR_HIP: return "the HIP runtime reported an error at launch";
    case FA_ERR_SCRATCH:
      return "the split plan needs more than the library's static decode scratch (ask for "
             "fewer splits)";
    default: return "unknown status";
  }
}

size_t fa_prefill_workspace_size(int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                                 fa_dtype out_dtype) {
  (void)Hkv;
  (void)causal;
  if (B < 1 || Hq < 1 || Sq < 1 || Skv < 0 || (D != 64 && D != 128)) return 0;
  if (out_dtype != FA_BF16 && out_dtype != FA_FP16 && out_dtype != FA_FP32) return 0;
  if (Hkv < 1 || Hq % Hkv != 0) return 0;
  return plan_prefill(B, Hq, Hkv, Sq, Skv, D, true, out_dtype == FA_FP32 ? 4 : 2).ws_bytes;
}

static int prefill_impl(const void* q, const void* k, const void* v, const void* mask,
                        int64_t mask_stride, int64_t mask_bstride, void* o, float* lse, int B,
                        int Hq, int Hkv, int Sq, int Skv, int D, int causal, float scale,
                        fa_dtype in_dtype, fa_dtype out_dtype, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  int rc = check_prefill(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, D, in_dtype, out_dtype);
  if (rc != FA_OK) return rc;
  if (workspace && !aligned16(workspace)) return FA_ERR_ALIGN;
  if (Sq == 0) return FA_OK;
  const int out_bytes = out_dtype == FA_FP32 ? 4 : 2;
  const PrefillPlan pl =
      plan_prefill(B, Hq, Hkv, Sq, Skv, D, workspace != nullptr, out_bytes);
  if (pl.ws_bytes > 0 && workspace_bytes < pl.ws_bytes) return FA_ERR_WORKSPACE;
  if ((int64_t)B * (Hq / pl.pack) * pl.n_qtiles * pl.n_splits > kMaxGrid) return FA_ERR_SHAPE;
  if (pl.n_splits > 1 && (int64_t)B * Sq * Hq > INT_MAX) return FA_ERR_SHAPE;

  PrefillParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Sq = Sq;
  p.Skv = Skv;
  p.waves = pl.waves;
  p.pack = pl.pack;
  p.pingpong = env_int("FA_PREFILL_PINGPONG", 0) != 0;
  p.n_qtiles = pl.n_qtiles;
  p.n_splits = pl.n_splits;
  p.q_neg = scale < 0.f;
  p.scale = std::fabs(scale);
  // Exponent scale; zero is passed as the smallest positive value so that
  // masked scores (-inf) still give probability 0 (and exp2(s * 1e-30) == 1).
  p.scale_log2 = std::max(p.scale * 1.4426950408889634f, 1e-30f);
  p.mask = mask;
  p.mask_stride = mask_stride;
  p.mask_bstride = mask_bstride;
  const int64_t rows = (int64_t)B * Sq * Hq;
  if (pl.n_splits > 1) {
    p.part_o = workspace;
    p.part_lse = (float*)((char*)workspace + (size_t)pl.n_splits * rows * D * out_bytes);
  }
  const InType it = in_dtype == FA_BF16 ? InType::bf16 : InType::f16;
  const OutType ot = out_dtype == FA_BF16 ? OutType::bf16
                     : out_dtype == FA_FP16 ? OutType::f16
                                            : OutType::f32;
  if (log_plans())
    std::fprintf(stderr,
                 "fa_log prefill B=%d Hq=%d Hkv=%d Sq=%d Skv=%d D=%d causal=%d mask=%d "
                 "cus=%d waves=%d pack=%d qtiles=%d splits=%d workgroups=%lld ws_bytes=%zu\n",
                 B, Hq, Hkv, Sq, Skv, D, causal != 0, mask != nullptr, planner_cus(), pl.waves,
                 pl.pack, pl.n_qtiles, pl.n_splits,
                 (long long)B * (Hq / pl.pack) * pl.n_qtiles * pl.n_splits, pl.ws_bytes);
  if (launch_prefill(p, D, it, ot, causal != 0, stream) != hipSuccess) return FA_ERR_HIP;
  if (pl.n_splits > 1) {
    CombineParams c{};
    c.part_o = p.part_o;
    c.part16 = out_dtype != FA_FP32;
    c.part_lse = p.part_lse;
    c.o = o;
    c.lse = lse;
    c.rows = (int)rows;
    c.D = D;
    c.n_splits = pl.n_splits;
    c.Sq = Sq;
    c.Hq = Hq;
    if (launch_combine(c, ot, stream) != hipSuccess) return FA_ERR_HIP;
  }
  return FA_OK;
}

int fa_prefill_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                  int Hq, int Hkv, int Sq, int Skv, int D, int causal, float scale,
                  fa_dtype in_dtype, fa_dtype out_dtype, void* workspace,
                  size_t workspace_bytes, hipStream_t stream) {
  return prefill_impl(q, k, v, nullptr, 0, 0, o, lse, B, Hq, Hkv, Sq, Skv, D, causal, scale,
                      in_dtype, out_dtype, workspace, workspace_bytes, stream);
}

int fa_prefill_mask(const void* q, const void* k, const void* v, const void* mask,
                    int64_t mask_stride, int64_t mask_batch_stride, void* o, float* lse, int B,
                    int Hq, int Hkv, int Sq, int Skv, int D, int causal, float scale,
                    fa_dtype in_dtype, fa_dtype out_dtype, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  if (!mask) return FA_ERR_NULL;
  // The kernel copies the mask in 16-byte pieces (8 keys), with per-row byte
  // offsets of 32 bits.
  if ((reinterpret_cast<uintptr_t>(mask) & 15u) != 0 || mask_stride % 8 != 0 ||
      mask_batch_stride % 8 != 0)
    return FA_ERR_ALIGN;
  if (mask_stride < ((int64_t)Skv + 7) / 8 * 8 || mask_batch_stride < 0 ||
      (int64_t)Sq * mask_stride > (int64_t)1 << 30)
    return FA_ERR_SHAPE;
  return prefill_impl(q, k, v, mask, mask_stride, mask_batch_stride, o, lse, B, Hq, Hkv, Sq,
                      Skv, D, causal, scale, in_dtype, out_dtype, workspace, workspace_bytes,
                      stream);
}

int fa_prefill(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv,
               int Sq, int Skv, int D, int causal, float scale, hipStream_t stream) {
  return fa_prefill_ex(q, k, v, o, nullptr, B, Hq, Hkv, Sq, Skv, D, causal, scale, FA_BF16,
                       FA_BF16, nullptr, 0, stream);
}

static int check_decode(const void* q, const void* kv_pool, int num_pages,
                        const int32_t* page_table,
                        const int32_t* seq_lens, void* o, const float* lse, int B, int Hq,
                        int Hkv, int D_qk, int D_v, int page_size, int max_pages_per_seq,
                        int max_seq_len, fa_kv_layout layout, fa_dtype dtype) {
  if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || page_size < 1 || max_pages_per_seq < 1 ||
      max_seq_len < 0 || num_pages < 1)
    return FA_ERR_SHAPE;
  if ((int64_t)max_pages_per_seq * page_size < max_seq_len) return FA_ERR_SHAPE;
  if (layout == FA_KV_SPLIT) {
    if (D_qk != 128 || D_v != 128) return FA_ERR_UNSUPPORTED;
    // The kernel addresses a page's bytes (K and V blocks of every K/V head)
    // with 32-bit offsets.
    if ((int64_t)2 * Hkv * page_size * D_qk * 2 > INT32_MAX) return FA_ERR_SHAPE;
  } else if (layout == FA_KV_MLA_SHARED) {
    if (D_qk != 576 || D_v != 512) return FA_ERR_UNSUPPORTED;
    if (Hkv != 1) return FA_ERR_SHAPE;
  } else {
    return FA_ERR_UNSUPPORTED;
  }
  if (dtype != FA_BF16 && dtype != FA_FP16) return FA_ERR_UNSUPPORTED;
  if (B > 0 && (!q || !kv_pool || !page_table || !seq_lens || !o)) return FA_ERR_NULL;
  if ((q && !aligned16(q)) || (kv_pool && !aligned16(kv_pool)) || (o && !aligned16(o)) ||
      (page_table && !aligned4(page_table)) || (seq_lens && !aligned4(seq_lens)) ||
      (lse && !aligned4(lse)))
    return FA_ERR_ALIGN;
  return FA_OK;
}

size_t fa_decode_workspace_size(int B, int Hq, int Hkv, int D_qk, int D_v, int page_size,
                                int max_seq_len, fa_kv_layout layout, int num_splits) {
  (void)D_qk;
  (void)page_size;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_seq_len < 0 || D_v < 1) return 0;
  return plan_decode(B, Hq, Hkv, D_v, max_seq_len, layout, num_splits, true).ws_bytes;
}

int fa_decode_num_splits(int B, int Hq, int Hkv, int D_qk, int D_v, int page_size,
                         int max_seq_len, fa_kv_layout layout, int num_splits) {
  (void)D_qk;
  (void)page_size;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_seq_len < 0 || D_v < 1) return 1;
  return plan_decode(B, Hq, Hkv, D_v, max_seq_len, layout, num_splits, true).n_splits;
}

// Exponent scale |scale| log2(e). Zero is passed as the smallest positive
// value, as for prefill: a masked score (-inf) must still give probability 0,
// and exp2(s * 1e-30) == 1 in fp32 for every finite score.
static float decode_exp_scale(float abs_scale) {
  return std::max(abs_scale * 1.4426950408889634f, 1e-30f);
}

static int decode_impl(const void* q, const void* kv_pool, int num_pages,
                       const int32_t* page_table, const int32_t* seq_lens, void* o, float* lse,
                       int B, int Sq, int Hq, int Hkv, int D_qk, int D_v, int page_size,
                       int max_pages_per_seq, int max_seq_len, fa_kv_layout layout, float scale,
                       int num_splits, fa_dtype dtype, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  int rc = check_decode(q, kv_pool, num_pages, page_table, seq_lens, o, lse, B, Hq, Hkv, D_qk, D_v,
                        page_size, max_pages_per_seq, max_seq_len, layout, dtype);
  if (rc != FA_OK) return rc;
  if (Sq < 1 || Sq > 64) return FA_ERR_SHAPE;
  if (workspace && !aligned16(workspace)) return FA_ERR_ALIGN;
  if (B == 0) return FA_OK;
  const DecodePlan pl =
      plan_decode(B, Hq, Hkv, D_v, max_seq_len, layout, num_splits, workspace != nullptr, Sq);
  if (pl.ws_bytes > 0 && workspace_bytes < pl.ws_bytes) return FA_ERR_WORKSPACE;
  const int64_t rows = (int64_t)B * Sq * Hq;
  if (rows > INT_MAX) return FA_ERR_SHAPE;
  void* part_o = nullptr;
  float* part_lse = nullptr;
  if (pl.n_splits > 1) {
    part_o = workspace;
    part_lse = (float*)((char*)workspace + (size_t)pl.n_splits * rows * D_v * 2);
  }
  const InType it = dtype == FA_BF16 ? InType::bf16 : InType::f16;
  if (log_plans())
    std::fprintf(stderr,
                 "fa_log decode layout=%s B=%d Sq=%d Hq=%d Hkv=%d page_size=%d max_seq_len=%d "
                 "cus=%d splits=%d chunk=%d row_blocks=%d heads_per_wg=%d ws_bytes=%zu\n",
                 layout == FA_KV_MLA_SHARED ? "mla" : "split", B, Sq, Hq, Hkv, page_size,
                 max_seq_len, planner_cus(), pl.n_splits, pl.chunk, pl.n_hblk,
                 layout == FA_KV_MLA_SHARED ? pl.heads_per_wg : 0, pl.ws_bytes);
  hipError_t e;
  if (layout == FA_KV_MLA_SHARED) {
    DecodeMlaParams p{};
    p.q = q;
    p.pool = kv_pool;
    p.page_table = page_table;
    p.seq_lens = seq_lens;
    p.o = o;
    p.lse = lse;
    p.part_o = part_o;
    p.part_lse = part_lse;
    p.B = B;
    p.Sq = Sq;
    p.Hq = Hq;
    p.page_size = page_size;
    p.max_pages = max_pages_per_seq;
    p.num_pages = num_pages;
    p.max_seq_len = max_seq_len;
    p.heads_per_wg = pl.heads_per_wg;
    p.n_hblk = pl.n_hblk;
    p.chunk = pl.chunk;
    p.n_splits = pl.n_splits;
    p.q_neg = scale < 0.f;
    p.scale = std::fabs(scale);
    p.scale_log2 = decode_exp_scale(p.scale);
    if ((int64_t)B * p.n_hblk * p.n_splits > kMaxGrid) return FA_ERR_SHAPE;
    e = launch_decode_mla(p, it, stream);
  } else {
    DecodeSplitParams p{};
    p.q = q;
    p.pool = kv_pool;
    p.page_table = page_table;
    p.seq_lens = seq_lens;
    p.o = o;
    p.lse = lse;
    p.part_o = part_o;
    p.part_lse = part_lse;
    p.B = B;
    p.Sq = Sq;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.page_size = page_size;
    p.max_pages = max_pages_per_seq;
    p.num_pages = num_pages;
    p.max_seq_len = max_seq_len;
    p.n_hblk = pl.n_hblk;
    p.chunk = pl.chunk;
    p.n_splits = pl.n_splits;
    const int64_t units = (int64_t)B * Hkv * pl.n_hblk * pl.n_splits;
    if (units > kMaxGrid) return FA_ERR_SHAPE;
    p.n_units = (int)units;
    p.q_neg = scale < 0.f;
    p.scale = std::fabs(scale);
    p.scale_log2 = decode_exp_scale(p.scale);
    e = launch_decode_split(p, it, stream);
  }
  if (e != hipSuccess) return FA_ERR_HIP;
  if (pl.n_splits > 1) {
    CombineParams c{};
    c.part_o = part_o;
    c.part16 = 1;
    c.part_lse = part_lse;
    c.o = o;
    c.lse = lse;
    c.rows = (int)rows;
    c.D = D_v;
    c.n_splits = pl.n_splits;
    c.Sq = Sq;
    c.Hq = Hq;
    if (launch_combine(c, dtype == FA_BF16 ? OutType::bf16 : OutType::f16, stream) != hipSuccess)
      return FA_ERR_HIP;
  }
  return FA_OK;
}

int fa_decode_paged(const void* q, const void* kv_pool, const int32_t* page_table,
                    const int32_t* seq_lens, int num_pages, void* o, float* lse, int B, int Hq,
                    int Hkv, int D_qk, int D_v, int page_size, int max_pages_per_seq,
                    int max_seq_len, fa_kv_layout layout, float scale, int num_splits,
                    fa_dtype dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(q, kv_pool, num_pages, page_table, seq_lens, o, lse, B, 1, Hq, Hkv, D_qk,
                     D_v, page_size, max_pages_per_seq, max_seq_len, layout, scale, num_splits,
                     dtype, workspace, workspace_bytes, stream);
}

int fa_decode_paged_multi(const void* q, const void* kv_pool, const int32_t* page_table,
                          const int32_t* seq_lens, int num_pages, void* o, float* lse,
                          int B, int Sq, int Hq, int Hkv, int D_qk, int D_v, int page_size,
                          int max_pages_per_seq, int max_seq_len, fa_kv_layout layout,
                          float scale, int num_splits, fa_dtype dtype, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(q, kv_pool, num_pages, page_table, seq_lens, o, lse, B, Sq, Hq, Hkv, D_qk,
                     D_v, page_size, max_pages_per_seq, max_seq_len, layout, scale, num_splits,
                     dtype, workspace, workspace_bytes, stream);
}

int fa_decode_paged_noalloc(const void* q, const void* kv_pool, const int32_t* page_table,
                            const int32_t* seq_lens, int num_pages, void* o, float* lse, int B,
                            int Hq, int Hkv, int D_qk, int D_v, int page_size,
                            int max_pages_per_seq, int max_seq_len, fa_kv_layout layout,
                            float scale, int num_splits, fa_dtype dtype, hipStream_t stream) {
  // The plan (and so the result) is the one fa_decode_paged makes with a
  // workspace; its partials must fit the static scratch. Everything is
  // checked on the host before the scratch is looked up or anything enqueued.
  int rc = check_decode(q, kv_pool, num_pages, page_table, seq_lens, o, lse, B, Hq, Hkv, D_qk,
                        D_v, page_size, max_pages_per_seq, max_seq_len, layout, dtype);
  if (rc != FA_OK) return rc;
  if (B == 0) return FA_OK;
  const DecodePlan pl = plan_decode(B, Hq, Hkv, D_v, max_seq_len, layout, num_splits, true);
  if (pl.ws_bytes > NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
  // The scratch is passed even when the plan does not split, so that the
  // call plans exactly as above.
  void* ws = nullptr;
  if (device_scratch(&ws) != hipSuccess) {
    (void)hipGetLastError();
    return FA_ERR_HIP;
  }
  return decode_impl(q, kv_pool, num_pages, page_table, seq_lens, o, lse, B, 1, Hq, Hkv, D_qk,
                     D_v, page_size, max_pages_per_seq, max_seq_len, layout, scale, num_splits,
                     dtype, ws, NOALLOC_SCRATCH_BYTES, stream);
  static_assert(NOALLOC_SCRATCH_BYTES == FA_DECODE_NOALLOC_SCRATCH_BYTES, "scratch size");
}

size_t fa_decode_multi_workspace_size(int B, int Sq, int Hq, int Hkv, int D_qk, int D_v,
                                      int page_size, int max_seq_len, fa_kv_layout layout,
                                      int num_splits) {
  (void)D_qk;
  (void)page_size;
  if (B < 1 || Sq < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_seq_len < 0 || D_v < 1)
    return 0;
  return plan_decode(B, Hq, Hkv, D_v, max_seq_len, layout, num_splits, true, Sq).ws_bytes;
}

}  // extern "C"
